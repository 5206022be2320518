// Query preparation for the reconstruct-with-RoPE decode (the query side of the
// Palu digest's RoPE path, Method details: RoPE is applied to q and to every
// rebuilt key at its position).
//
// For query head j with key slice B (r x d_h, columns of its KV head in the
// unit's B^k) and the rotate-half pair (i, i + d_h/2) at angle
// phi_i(t) = (t - q_pos) theta_i, theta_i = base^(-2i/d_h):
//     RoPE(q, q_pos) . RoPE(h_t B, t) = sum_i cos(phi_i) (h_t . u_i) + sin(phi_i) (h_t . w_i)
//     u_i = q_i B[:, i] + q_{i+h} B[:, i+h],   w_i = q_{i+h} B[:, i] - q_i B[:, i+h]
// This step writes Q' = [u_0, w_0, u_1, w_1, ...] (d_h rows of r values, fp16)
// for every head, and the cos/sin tables of the phi_i (fp64 angles, fp32 values).
// Q' is stored row-major per head, or (for the rank-256, d_h-128, 4-head units
// of the frequency-wave kernel) in MFMA-fragment order: for unit (b, u), row
// block w (rows 32 w .. 32 w + 31), head h and K step ks, one contiguous 1 KB
// block whose 16 bytes at 16 l are the A fragment of lane l (row 32 w + l%32,
// columns 16 ks + 8 (l/32) .. + 7).
#include "common.h"

#include <math.h>

namespace lrkv {
namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;

// Q'[f][k] scaled by sm_scale*log2(e)*2^e_i, one power of two per (unit,
// frequency) shared by the unit's heads, so that the largest |Q'| of the
// frequency lands in [2^14, 2^15) (fp16 range). 2^-e_i goes to qs.
// Grid: (B*U, DH/8); block: 4 frequencies; the 8 needed B columns of every
// head are staged in LDS with 8-byte loads first.
__device__ __forceinline__ size_t qp_index(bool frag, int bu, int NH, int h, int DH, int R, int row, int k) {
    if (!frag) return ((size_t)bu * NH + h) * DH * R + (size_t)row * R + k;
    const int w = row >> 5, ks = k >> 4, lane = (row & 31) + 32 * ((k >> 3) & 1);
    return ((((size_t)bu * (DH / 32) + w) * NH + h) * (R / 16) + ks) * 512 + lane * 8 + (k & 7);
}
__global__ __launch_bounds__(256) void rope_qprep(const float* __restrict__ q,
                                                  const half_t* __restrict__ bk,
                                                  half_t* __restrict__ qp, float* __restrict__ qs,
                                                  int U, int s, int gq, int DH, int R, float scale,
                                                  bool frag) {
    constexpr int MAXR = 256, MAXNH = 8;
    __shared__ __attribute__((aligned(8))) half_t Bs[MAXNH][2][MAXR][4];
    __shared__ float red[4][4];
    const int bu = blockIdx.x, u = bu % U, b = bu / U;
    const int NH = s * gq, Hq = U * NH, half = DH / 2, ldb = s * DH;
    const int i0 = blockIdx.y * 4;
    const half_t* Bu = bk + (size_t)u * R * ldb;
    // stage: item = (h, side, k) -> 4 consecutive columns (8 bytes)
    for (int item = threadIdx.x; item < NH * 2 * R; item += blockDim.x) {
        const int k = item % R, side = (item / R) & 1, h = item / (2 * R);
        const int w = ((u * NH + h) / gq) % s;
        *reinterpret_cast<uint2*>(&Bs[h][side][k][0]) =
            *reinterpret_cast<const uint2*>(Bu + (size_t)k * ldb + w * DH + side * half + i0);
    }
    __syncthreads();
    const int fi = threadIdx.x & 3, kl = threadIdx.x >> 2;    // 4 frequencies x 64 k-lanes
    const int i = i0 + fi;
    float mx = 0.0f;
    for (int h = 0; h < NH; ++h) {
        const int j = u * NH + h;
        const float qa = q[((size_t)b * Hq + j) * DH + i] * scale;
        const float qb = q[((size_t)b * Hq + j) * DH + i + half] * scale;
        for (int k = kl; k < R; k += 64) {
            const float b0 = (float)Bs[h][0][k][fi], b1 = (float)Bs[h][1][k][fi];
            mx = fmaxf(mx, fmaxf(fabsf(fmaf(qa, b0, qb * b1)), fabsf(fmaf(qb, b0, -qa * b1))));
        }
    }
#pragma unroll
    for (int o = 4; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
    if ((threadIdx.x & 63) < 4) red[fi][threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[fi][0], red[fi][1]), fmaxf(red[fi][2], red[fi][3]));
    const int ex = (mx > 0.0f && isfinite(mx)) ? 14 - ilogbf(mx) : 0;
    for (int h = 0; h < NH; ++h) {
        const int j = u * NH + h;
        const float qa = ldexpf(q[((size_t)b * Hq + j) * DH + i] * scale, ex);
        const float qb = ldexpf(q[((size_t)b * Hq + j) * DH + i + half] * scale, ex);
        for (int k = kl; k < R; k += 64) {
            const float b0 = (float)Bs[h][0][k][fi], b1 = (float)Bs[h][1][k][fi];
            qp[qp_index(frag, bu, NH, h, DH, R, 2 * i, k)] = (half_t)fmaf(qa, b0, qb * b1);
            qp[qp_index(frag, bu, NH, h, DH, R, 2 * i + 1, k)] = (half_t)fmaf(qb, b0, -qa * b1);
        }
    }
    if (kl == 0) qs[((size_t)b * U + u) * half + i] = ldexpf(1.0f, -ex);
}

// Angle tables: (cos, sin)(2 pi frac(n rho_f)), rho_f = theta_f / (2 pi), with the
// argument reduced in fp64 (exact for |n| < 2^31). One thread per entry:
//   rows [0, 1)           n = 32                     (one-tile rotation)
//   rows [1, 33)          n = t, t < 32              (offset inside a tile)
//   rows [33, 33 + B*S)   n = c * chunk - q_pos[b]   (chunk start)
__global__ __launch_bounds__(256) void rope_angles(float2* __restrict__ tab,
                                                   const int32_t* __restrict__ q_pos,
                                                   const int32_t* __restrict__ lens, int B,
                                                   int n_split, int chunk, int half, double theta) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    const int rows = 33 + B * n_split;
    if (e >= rows * half) return;
    const int row = e / half, f = e % half;
    long n;
    if (row == 0) {
        n = 32;
    } else if (row < 33) {
        n = row - 1;
    } else {
        const int b = (row - 33) / n_split, c = (row - 33) % n_split;
        const long qpos = q_pos ? q_pos[b] : (long)lens[b] - 1;
        n = (long)c * chunk - qpos;
    }
    const double rho = theta > 0.0 ? exp2(-2.0 * f / (2.0 * half) * log2(theta)) / kTwoPi : 0.0;
    double rev = (double)n * rho;
    rev -= rint(rev);
    double sd, cd;
    sincos(kTwoPi * rev, &sd, &cd);
    tab[e] = make_float2((float)cd, (float)sd);
}

// B^k of one-KV-head units (d_h = 128) in the 16x16x32 MFMA A-fragment order of
// the grouped-query kernel: bf[u][mt][ks][lane][e] = B^k[u][rank][dim] with
// dim = 16 mt + lane % 16 and rank = R/4 (lane / 16) + 8 ks + perm(e). For int4
// latents perm = (0, 4, 1, 5, 2, 6, 3, 7), the order in which that kernel unpacks
// a word of codes; identity for fp16.
__global__ __launch_bounds__(256) void gqa_bfrag(const half_t* __restrict__ bk, half_t* __restrict__ bf,
                                                 int U, int R, int int4) {
    const long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const int KS = R / 32;
    if (e >= (long)U * 128 * R) return;
    const int el = (int)(e & 7), lane = (int)((e >> 3) & 63);
    const long rest = e >> 9;
    const int ks = (int)(rest % KS), mt = (int)((rest / KS) % 8), u = (int)(rest / (KS * 8));
    const int pe = int4 ? ((el & 1) ? 4 + (el >> 1) : (el >> 1)) : el;
    const int rank = (R / 4) * (lane >> 4) + 8 * ks + pe, dim = 16 * mt + (lane & 15);
    bf[e] = bk[((long)u * R + rank) * 128 + dim];
}

// Queries of the grouped-query kernel: q x sm_scale x log2(e), fp32, same layout.
__global__ __launch_bounds__(256) void gqa_qscale(const float* __restrict__ q, float* __restrict__ qo, long n,
                                                  float scale) {
    const long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e < n) qo[e] = q[e] * scale;
}

}  // namespace

void launch_rope_prep(const float* q, const half_t* bk, const int32_t* q_pos, const int32_t* lens,
                      half_t* qp, float* qs, float2* angles, int B, int U, int s, int gq, int DH,
                      int R, int n_split, int chunk, double theta, float scale, int qmode,
                      bool int4, hipStream_t st) {
    if (qmode == kQpGqaFragments) {
        // B^k fragments, then the scaled queries right after them
        const long n = (long)U * 128 * R;
        hipLaunchKernelGGL(gqa_bfrag, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, bk, qp, U, R,
                           int4 ? 1 : 0);
        const long nq = (long)B * U * s * gq * DH;
        hipLaunchKernelGGL(gqa_qscale, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, st, q,
                           reinterpret_cast<float*>(qp + n), nq, scale);
    } else {
        hipLaunchKernelGGL(rope_qprep, dim3(B * U, DH / 8), dim3(256), 0, st, q, bk, qp, qs, U, s, gq,
                           DH, R, scale, qmode == kQpFragments);
    }
    const int n = (33 + B * n_split) * (DH / 2);
    hipLaunchKernelGGL(rope_angles, dim3((n + 255) / 256), dim3(256), 0, st, angles, q_pos, lens, B,
                       n_split, chunk, DH / 2, theta);
}

}  // namespace lrkv
