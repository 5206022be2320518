// Split-K merge of per-chunk softmax states (PuzzleKV section 3.3, step 4:
// partial results merged by online softmax; the same merge combines the
// sequence chunks of every decode mode).
#include "common.h"

#include <math.h>

namespace lrkv {
namespace {

// out[b][j][d] = sum_c 2^(m_c - M) acc_c[d] / sum_c 2^(m_c - M) l_c over the
// n_split chunks (at most 1024); empty chunks (m = -inf) contribute nothing.
// One wave per (sequence, head, 64 output dims): the chunk maxima and weights
// go through LDS, reductions are wave-wide shuffles. With `lens` non-null the
// first wave also adds `bump` to lens[0 .. B) (lrkv_decode_step: the step's
// appended tokens, once every kernel that reads lens before them has run).
__global__ __launch_bounds__(64) void merge_splits(const float* __restrict__ part,
                                                   float* __restrict__ out, int n_split, int D,
                                                   int32_t* __restrict__ lens, int B, int bump) {
    if (lens && blockIdx.x == 0 && blockIdx.y == 0)
        for (int b = threadIdx.x; b < B; b += 64) lens[b] += bump;
    constexpr int kPre = 32;                   // chunks whose outputs are requested up front
    __shared__ float wts[1024], lsum[1024];
    const long bj = blockIdx.x;
    const int lane = threadIdx.x, d = blockIdx.y * 64 + lane;
    const float* pp = part + bj * n_split * (D + 2);
    // one round trip for the common case: every chunk's (m, l) and the first kPre
    // chunks' outputs are requested before any of them is used
    float ov[kPre];
#pragma unroll
    for (int k = 0; k < kPre; ++k) ov[k] = (k < n_split && d < D) ? pp[(long)k * (D + 2) + 2 + d] : 0.0f;
    float mx = -INFINITY;
    for (int c = lane; c < n_split; c += 64) {
        const float m = pp[(long)c * (D + 2)];
        lsum[c] = pp[(long)c * (D + 2) + 1];
        wts[c] = m;
        mx = fmaxf(mx, m);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
    float den = 0.0f;
    for (int c = lane; c < n_split; c += 64) {
        const float m = wts[c];
        const float wgt = m == -INFINITY ? 0.0f : exp2f(m - mx);
        wts[c] = wgt;
        den = fmaf(wgt, lsum[c], den);
    }
    den = reduce_sum_width<64>(den);
    __syncthreads();
    if (d >= D) return;
    const float rden = 1.0f / den;
    float n0 = 0.0f, n1 = 0.0f, n2 = 0.0f, n3 = 0.0f;
#pragma unroll
    for (int k = 0; k < kPre; k += 4) {
        // chunks past n_split have ov = 0 (their weights are never read)
        if (k < n_split) n0 = fmaf(wts[k], ov[k], n0);
        if (k + 1 < n_split) n1 = fmaf(wts[k + 1], ov[k + 1], n1);
        if (k + 2 < n_split) n2 = fmaf(wts[k + 2], ov[k + 2], n2);
        if (k + 3 < n_split) n3 = fmaf(wts[k + 3], ov[k + 3], n3);
    }
    int c = kPre;
    for (; c + 4 <= n_split; c += 4) {
        n0 = fmaf(wts[c], pp[(long)c * (D + 2) + 2 + d], n0);
        n1 = fmaf(wts[c + 1], pp[(long)(c + 1) * (D + 2) + 2 + d], n1);
        n2 = fmaf(wts[c + 2], pp[(long)(c + 2) * (D + 2) + 2 + d], n2);
        n3 = fmaf(wts[c + 3], pp[(long)(c + 3) * (D + 2) + 2 + d], n3);
    }
    for (; c < n_split; ++c) n0 = fmaf(wts[c], pp[(long)c * (D + 2) + 2 + d], n0);
    out[bj * D + d] = ((n0 + n1) + (n2 + n3)) * rden;
}

// The same merge for many rows and at most 64 chunks (the prefill's key splits):
// four waves per workgroup, one (row, 64 output dims) per wave; lane c holds
// chunk c's (max, sum) in registers, the weights are broadcast by shuffles.
__global__ __launch_bounds__(256) void merge_rows(const float* __restrict__ part, float* __restrict__ out,
                                                  int n_split, int D, long n_items) {
    const long item = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= n_items) return;
    const int nd = (D + 63) / 64;
    const long bj = item / nd;
    const int lane = threadIdx.x & 63, d = (int)(item % nd) * 64 + lane;
    const float* pp = part + bj * n_split * (D + 2);
    const float m = lane < n_split ? pp[(long)lane * (D + 2)] : -INFINITY;
    const float l = lane < n_split ? pp[(long)lane * (D + 2) + 1] : 0.0f;
    float mx = m;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
    const float wgt = m == -INFINITY ? 0.0f : exp2f(m - mx);
    const float den = reduce_sum_width<64>(wgt * l);
    float num = 0.0f;
    for (int c = 0; c < n_split; ++c) {
        const float wc = __shfl(wgt, c, kWave);            // every lane takes part
        if (d < D) num = fmaf(wc, pp[(long)c * (D + 2) + 2 + d], num);
    }
    if (d < D) out[bj * D + d] = num / den;
}

}  // namespace

void launch_merge_rows(const float* part, float* out, int BH, int n_split, int D, hipStream_t st) {
    if (n_split > 64) {
        hipLaunchKernelGGL(merge_splits, dim3(BH, (D + 63) / 64), dim3(64), 0, st, part, out, n_split, D,
                           (int32_t*)nullptr, 0, 0);
        return;
    }
    const long n_items = (long)BH * ((D + 63) / 64);
    hipLaunchKernelGGL(merge_rows, dim3((unsigned)((n_items + 3) / 4)), dim3(256), 0, st, part, out, n_split, D,
                       n_items);
}

void launch_merge(const float* part, float* out, int BH, int n_split, int D, hipStream_t st) {
    hipLaunchKernelGGL(merge_splits, dim3(BH, (D + 63) / 64), dim3(64), 0, st, part, out, n_split, D,
                       (int32_t*)nullptr, 0, 0);
}

void launch_merge_bump(const float* part, float* out, int BH, int n_split, int D, hipStream_t st,
                       int32_t* lens, int B, int bump) {
    hipLaunchKernelGGL(merge_splits, dim3(BH, (D + 63) / 64), dim3(64), 0, st, part, out, n_split, D,
                       lens, B, bump);
}

}  // namespace lrkv
