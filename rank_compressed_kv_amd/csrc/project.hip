// The projections on either side of the decode path (Palu digest, Method
// details): a token is cached as its latents h = x A (A_u, d_model x r, per
// unit), and the value up-projection is fused offline into the output
// projection, so the layer output is y = sum_j o_j (B^v_j W^o_j) with o_j the
// latent-space attention output of head j. Both are
//   C[M][N] = X[M][K] W^T[N][K]^T,   M = tokens in the batch (a few rows),
// with fp16 weights stored K-contiguous, fp32 X and C: a weight stream.
//
// One wave owns 16 columns over one K range: per 32-wide K step it loads its
// 16 weight rows (one 16-byte fragment per lane), and the 16x16x32 MFMA takes
// X as an fp16 hi + lo pair (x = hi + lo exactly to ~22 bits) against them.
// Four K steps are loaded before their MFMAs. The K ranges write partial sums
// [k_split][M][N]; a second kernel adds them in a fixed order (deterministic).
#include "common.h"

namespace lrkv {
namespace {

constexpr int kUnroll = 4;

__global__ __launch_bounds__(256) void skinny_partials(const float* __restrict__ X, const half_t* __restrict__ Wt,
                                                       float* __restrict__ part, int M, int N, int K, int kchunk) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int cb = blockIdx.x * 4 + w;           // 16-column block
    if (cb * 16 >= N) return;
    const int ks = blockIdx.y, mb = blockIdx.z;
    const int c = l & 15, g = l >> 4;
    const int k_begin = ks * kchunk, k_end = min(K, k_begin + kchunk);
    const int m = mb * 16 + c;                   // row of X this lane supplies
    const bool mrow = m < M;
    const float* xr = X + (long)(mrow ? m : 0) * K + 8 * g;
    const half_t* wr = Wt + (long)(cb * 16 + c) * K + 8 * g;
    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};

    auto step = [&](const half8& b, const float4& x0, const float4& x1) __attribute__((always_inline)) {
        const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        half8 ah, al;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = mrow ? xs[e] : 0.0f;
            ah[e] = (half_t)v;
            al[e] = (half_t)(v - (float)ah[e]);
        }
        acc = mfma16(ah, b, acc);
        acc = mfma16(al, b, acc);
    };
    int k0 = k_begin;
    for (; k0 + 32 * kUnroll <= k_end; k0 += 32 * kUnroll) {
        half8 b[kUnroll];
        float4 x0[kUnroll], x1[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            b[u] = *reinterpret_cast<const half8*>(wr + k0 + 32 * u);
            x0[u] = *reinterpret_cast<const float4*>(xr + k0 + 32 * u);
            x1[u] = *reinterpret_cast<const float4*>(xr + k0 + 32 * u + 4);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) step(b[u], x0[u], x1[u]);
    }
    for (; k0 < k_end; k0 += 32) {
        const half8 b = *reinterpret_cast<const half8*>(wr + k0);
        step(b, *reinterpret_cast<const float4*>(xr + k0), *reinterpret_cast<const float4*>(xr + k0 + 4));
    }
    // lane (c, g) holds C[16 mb + 4 g + i][16 cb + c]
    float* pp = part + ((long)ks * M) * N + cb * 16 + c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = mb * 16 + 4 * g + i;
        if (row < M) pp[(long)row * N] = acc[i];
    }
}

__global__ void skinny_reduce(const float* __restrict__ part, float* __restrict__ C, int MN, int k_split) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= MN) return;
    float s = 0.0f;
    for (int k = 0; k < k_split; ++k) s += part[(long)k * MN + e];
    C[e] = s;
}

}  // namespace

// K split that gives about 2048 waves (two per SIMD); K ranges are whole
// 32-wide steps.
SkinnyPlan skinny_plan(int M, int N, int K) {
    SkinnyPlan p;
    const int n_cb = N / 16, n_mb = (M + 15) / 16, steps = K / 32;
    int ks = (2048 + n_cb * n_mb - 1) / (n_cb * n_mb);
    if (ks > steps) ks = steps;
    if (ks < 1) ks = 1;
    const int per = (steps + ks - 1) / ks;
    p.kchunk = 32 * per;
    p.k_split = (steps + per - 1) / per;
    p.ws_bytes = align_up((size_t)p.k_split * M * N * sizeof(float), 256);
    return p;
}

int32_t launch_skinny(const float* X, const half_t* Wt, float* C, int M, int N, int K, void* ws,
                      const SkinnyPlan& p, hipStream_t st) {
    float* part = (float*)ws;
    hipLaunchKernelGGL(skinny_partials, dim3((N / 16 + 3) / 4, p.k_split, (M + 15) / 16), dim3(256), 0, st, X, Wt,
                       part, M, N, K, p.kchunk);
    const int MN = M * N;
    hipLaunchKernelGGL(skinny_reduce, dim3((MN + 255) / 256), dim3(256), 0, st, part, C, MN, p.k_split);
    return last_launch_status();
}

}  // namespace lrkv
