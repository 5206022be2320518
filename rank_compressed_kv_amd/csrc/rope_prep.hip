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
// One launch; its blocks take one of three roles: Q' (or, for the grouped-query
// kernel, B^k fragments and scaled queries), then the angle tables. For
// lrkv_decode_step a first block also appends the step's new fp16 latents
// without touching lens: `pending` tokens then count as cached (the merge of
// the same step adds them to lens once every reader of lens has finished).
// Q' is stored row-major per head, or (for the rank-256, d_h-128, 4-head units
// of the frequency-wave kernel) in MFMA-fragment order: for unit (b, u), row
// block w (rows 32 w .. 32 w + 31), head h and K step ks, one contiguous 1 KB
// block whose 16 bytes at 16 l are the A fragment of lane l (row 32 w + l%32,
// columns 16 ks + 8 (l/32) .. + 7).
#include "append_dev.h"
#include "tiles.h"

#include <math.h>

namespace lrkv {
namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;

struct PrepArgs {
    const float* q;          // [B][Hq][DH]
    const half_t* bk;        // [U][R][s DH]
    const int32_t* q_pos;
    const int32_t* lens;
    half_t* qp;
    float* qs;
    float2* ang;
    int B, U, s, gq, DH, R, n_split, chunk;
    double theta;
    float scale;
    int qmode, int4;
    int n_q, n_s;            // blocks of the Q' / B^k role and of the query-scaling role
    // fused append (lrkv_decode_step): n_app = 1 block writes the `pending` new
    // tokens (nk, nv [B][U][pending][R] fp32) into the cache (fp16 latents, or
    // int4 codes with their scales sk / sv)
    int n_app, pending, cap, app_int4;
    const float *nk, *nv;
    void *hk, *hv;
    half_t *sk, *sv;
};

__device__ __forceinline__ size_t qp_index(bool frag, int bu, int NH, int h, int DH, int R, int row, int k) {
    if (!frag) return ((size_t)bu * NH + h) * DH * R + (size_t)row * R + k;
    const int w = row >> 5, ks = k >> 4, lane = (row & 31) + 32 * ((k >> 3) & 1);
    return ((((size_t)bu * (DH / 32) + w) * NH + h) * (R / 16) + ks) * 512 + lane * 8 + (k & 7);
}

// Q'[2i][k] = qa B[k][i] + qb B[k][i + h], Q'[2i+1][k] = qb B[k][i] - qa B[k][i + h]
// (qa, qb = q[i], q[i + h] x scale), times 2^e_i, one power of two per (unit,
// frequency) shared by the unit's heads, so that the largest |Q'| of the
// frequency lands in [2^14, 2^15) (fp16 range); 2^-e_i goes to qs.
// Block = (sequence b, unit u, 8 frequencies). The 8 columns of B^k that each
// (KV head, rotate-half side) needs are staged in LDS with 16-byte loads; a
// thread = (8 ranks k8, 4 of the frequencies, head) keeps its 64 values in
// registers while the maxima are reduced, then writes 8 consecutive ranks (16
// bytes) per row. Scaling by 2^e is exact, so the written value is the fp16
// rounding of the scaled fused multiply-add.
constexpr int kPrepLds = 32768;      // staged B^k bytes: R * s * 2 sides * 16 B (r * s <= 1024)
constexpr int kPrepPad = kPrepLds / 8;   // one 16-byte pad after every 8 staged rows

// The power of two 2^e that brings a frequency's largest |Q'| m into [2^14, 2^15)
// (0 for an all-zero or non-finite m), clamped so that 2^e and 2^-e are normal
// fp32 numbers.
__device__ __forceinline__ int prep_exp(float m) {
    const int e = (m > 0.0f && isfinite(m)) ? 14 - ilogbf(m) : 0;
    return min(max(e, -126), 126);
}

// Staged row `x` = (KV head, side) * R + rank: 16 bytes, plus a 16-byte pad after
// every 8 rows, so that lanes 8 ranks apart read different LDS banks.
__device__ __forceinline__ int stage_off(int x) { return x * 8 + (x >> 3) * 8; }

__device__ void prep_qprime(const PrepArgs& a, int blk) {
    __shared__ unsigned smax[8];
    __shared__ __attribute__((aligned(16))) half_t Bs[(kPrepLds + kPrepPad) / 2];
    // consecutive blocks go to different XCDs: (b, u) varies fastest so that the
    // frequency groups of one unit, which share B^k's 64-byte lines, meet in one L2
    const int nbu = a.B * a.U;
    const int bu = blk % nbu, i0 = (blk / nbu) * 8;
    const int u = bu % a.U, b = bu / a.U;
    const int NH = a.s * a.gq, Hq = a.U * NH, half = a.DH / 2, ldb = a.s * a.DH;
    const int R8 = a.R / 8, per_head = R8 * 2;      // threads per head; per_head * NH <= 256
    const int t = threadIdx.x;
    const bool active = t < per_head * NH;
    const int k8 = t % R8, fq = (t / R8) & 1, h = t / per_head;
    const int i = i0 + 4 * fq;
    const bool frag = a.qmode == kQpFragments;
    if (t < 8) smax[t] = 0u;
    const int j = u * NH + h, w = (j / a.gq) % a.s;
    float qa4[4], qb4[4];
    if (active) {
        const float* qrow = a.q + ((size_t)b * Hq + j) * a.DH;
        const float4 qa = *reinterpret_cast<const float4*>(qrow + i);
        const float4 qb = *reinterpret_cast<const float4*>(qrow + i + half);
        qa4[0] = qa.x * a.scale; qa4[1] = qa.y * a.scale; qa4[2] = qa.z * a.scale; qa4[3] = qa.w * a.scale;
        qb4[0] = qb.x * a.scale; qb4[1] = qb.y * a.scale; qb4[2] = qb.z * a.scale; qb4[3] = qb.w * a.scale;
    }
    // stage: piece p = (rank, KV head w, side) -> Bs[(w, side)][rank][0..7];
    // loads in batches of 8 per thread, all in flight before the LDS stores
    const half_t* Bu = a.bk + (size_t)u * a.R * ldb;
    const int pieces = a.R * a.s * 2;
    for (int base = t; base < pieces; base += 8 * 256) {
        uint4 v[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int pc = min(base + 256 * m, pieces - 1);     // clamped: loads stay unconditional
            const int row = pc / (2 * a.s), sub = pc % (2 * a.s), ww = sub >> 1, side = sub & 1;
            v[m] = *reinterpret_cast<const uint4*>(Bu + (size_t)row * ldb + ww * a.DH + side * half + i0);
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int pc = base + 256 * m;
            if (pc < pieces) {
                const int row = pc / (2 * a.s), sub = pc % (2 * a.s);
                *reinterpret_cast<uint4*>(Bs + stage_off(sub * a.R + row)) = v[m];
            }
        }
    }
    __syncthreads();
    // Q' of ranks 8 k8 + e, frequencies i + f, rows (u, w) = (2i, 2i + 1)
    float v[8][4][2];
    if (active) {
        const half_t* s0 = Bs + stage_off(2 * w * a.R + 8 * k8) + 4 * fq;
        const half_t* s1 = Bs + stage_off((2 * w + 1) * a.R + 8 * k8) + 4 * fq;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const half4 b0 = *reinterpret_cast<const half4*>(s0 + 8 * e);
            const half4 b1 = *reinterpret_cast<const half4*>(s1 + 8 * e);
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const float x0 = (float)b0[f], x1 = (float)b1[f];
                v[e][f][0] = fmaf(qa4[f], x0, qb4[f] * x1);
                v[e][f][1] = fmaf(qb4[f], x0, -qa4[f] * x1);
            }
        }
        // per-frequency maximum: over this thread's ranks, then its 32-lane row, then LDS
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            float m = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fmaxf(fabsf(v[e][f][0]), fabsf(v[e][f][1])));
            if (R8 == 32) {
                m = half_max32(m);                 // the half-wave holds one (head, fq)
            } else {
                for (int o = 1; o < R8 && o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
            }
            if ((k8 & 31) == 0) atomicMax(&smax[4 * fq + f], __float_as_uint(m));
        }
    }
    __syncthreads();
    if (t < 8) {
        const int e = prep_exp(__uint_as_float(smax[t]));
        a.qs[((size_t)b * a.U + u) * half + i0 + t] = ldexpf(1.0f, -e);
    }
    if (!active) return;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const float sc = ldexpf(1.0f, prep_exp(__uint_as_float(smax[4 * fq + f])));   // exact
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
            half8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = (half_t)(v[e][f][r2] * sc);
            *reinterpret_cast<half8*>(a.qp + qp_index(frag, bu, NH, h, a.DH, a.R, 2 * (i + f) + r2, 8 * k8)) = o;
        }
    }
}

// B^k of one-KV-head units (d_h = 128) in the 16x16x32 MFMA A-fragment order of
// the grouped-query kernel: bf[u][mt][ks][lane][e] = B^k[u][rank][dim] with
// dim = 16 mt + lane % 16 and rank = R/4 (lane / 16) + 8 ks + perm(e). For int4
// latents perm = (0, 4, 1, 5, 2, 6, 3, 7), the order in which that kernel unpacks
// a word of codes; identity for fp16.
__device__ void prep_bfrag(const PrepArgs& a, int blk) {
    const long e = (long)blk * 256 + threadIdx.x;
    const int KS = a.R / 32;
    if (e >= (long)a.U * 128 * a.R) return;
    const int el = (int)(e & 7), lane = (int)((e >> 3) & 63);
    const long rest = e >> 9;
    const int ks = (int)(rest % KS), mt = (int)((rest / KS) % 8), u = (int)(rest / (KS * 8));
    const int pe = a.int4 ? ((el & 1) ? 4 + (el >> 1) : (el >> 1)) : el;
    const int rank = (a.R / 4) * (lane >> 4) + 8 * ks + pe, dim = 16 * mt + (lane & 15);
    a.qp[e] = a.bk[((long)u * a.R + rank) * 128 + dim];
}

// Queries of the grouped-query kernel: q x sm_scale x log2(e), fp32, same
// layout, right after the B^k fragments.
__device__ void prep_qscale(const PrepArgs& a, int blk) {
    const long e = (long)blk * 256 + threadIdx.x;
    const long n = (long)a.B * a.U * a.s * a.gq * a.DH;
    float* qo = reinterpret_cast<float*>(a.qp + (long)a.U * 128 * a.R);
    if (e < n) qo[e] = a.q[e] * a.scale;
}

// Angle tables: (cos, sin)(2 pi frac(n rho_f)), rho_f = theta_f / (2 pi), with the
// argument reduced in fp64 (exact for |n| < 2^31). One thread per entry:
//   rows [0, 1)           n = 32                     (one-tile rotation)
//   rows [1, 33)          n = t, t < 32              (offset inside a tile)
//   rows [33, 33 + B*S)   n = c * chunk - q_pos[b]   (chunk start)
__device__ void prep_angles(const PrepArgs& a, int blk) {
    const int half = a.DH / 2;
    const int e = blk * 256 + threadIdx.x;
    const int rows = 33 + a.B * a.n_split;
    if (e >= rows * half) return;
    const int row = e / half, f = e % half;
    long n;
    if (row == 0) {
        n = 32;
    } else if (row < 33) {
        n = row - 1;
    } else {
        const int b = (row - 33) / a.n_split, c = (row - 33) % a.n_split;
        const long qpos = a.q_pos ? a.q_pos[b] : (long)a.lens[b] + a.pending - 1;
        n = (long)c * a.chunk - qpos;
    }
    const double rho = a.theta > 0.0 ? exp2(-2.0 * f / (2.0 * half) * log2(a.theta)) / kTwoPi : 0.0;
    double rev = (double)n * rho;
    rev -= rint(rev);
    double sd, cd;
    sincos(kTwoPi * rev, &sd, &cd);
    a.ang[e] = make_float2((float)cd, (float)sd);
}

__global__ __launch_bounds__(256) void rope_prepare(const PrepArgs a) {
    if ((int)blockIdx.x < a.n_app) {
        if (!a.app_int4) {
            append_fp16_rows(a.nk, a.nv, (half_t*)a.hk, (half_t*)a.hv, a.lens, a.B, a.U, a.R, a.cap, a.pending,
                             threadIdx.x, 256);
        } else {
            // key groups and value pairs on different threads (independent items), so
            // that the two chains of loads and stores run side by side
            const long n_keys = (long)a.B * a.U * a.pending * (a.R / 32);
            const long n_vals = (long)a.B * a.U * (a.pending / 2 + 2) * (a.R / 32);
            for (long e = threadIdx.x; e < n_keys + n_vals; e += 256) {
                if (e < n_keys)
                    append_int4_key_group(a.nk, (uint8_t*)a.hk, a.sk, a.lens, a.B, a.U, a.R, a.cap, a.pending, e);
                else
                    append_int4_value_pair(a.nv, (uint8_t*)a.hv, a.sv, a.lens, a.B, a.U, a.R, a.cap, a.pending,
                                           e - n_keys);
            }
        }
        return;
    }
    const int blk = blockIdx.x - a.n_app;
    if (blk < a.n_q) {
        if (a.qmode == kQpGqaFragments) prep_bfrag(a, blk);
        else prep_qprime(a, blk);
    } else if (blk < a.n_q + a.n_s) {
        prep_qscale(a, blk - a.n_q);
    } else {
        prep_angles(a, blk - a.n_q - a.n_s);
    }
}

}  // namespace

void launch_rope_prep(const float* q, const half_t* bk, const int32_t* q_pos, const int32_t* lens,
                      half_t* qp, float* qs, float2* angles, int B, int U, int s, int gq, int DH,
                      int R, int n_split, int chunk, double theta, float scale, int qmode,
                      bool int4, hipStream_t st, int pending, const float* nk, const float* nv,
                      void* hk, void* hv, half_t* sk, half_t* sv, int cap) {
    PrepArgs a{q, bk, q_pos, lens, qp, qs, angles, B, U, s, gq, DH, R, n_split, chunk, theta, scale,
               qmode, int4 ? 1 : 0, 0, 0, nk ? 1 : 0, pending, cap, int4 ? 1 : 0, nk, nv, hk, hv, sk, sv};
    if (qmode == kQpGqaFragments) {
        a.n_q = (int)(((long)U * 128 * R + 255) / 256);
        a.n_s = (int)(((long)B * U * s * gq * DH + 255) / 256);
    } else {
        a.n_q = B * U * (DH / 16);
    }
    const int n_ang = ((33 + B * n_split) * (DH / 2) + 255) / 256;
    hipLaunchKernelGGL(rope_prepare, dim3(a.n_app + a.n_q + a.n_s + n_ang), dim3(256), 0, st, a);
}

}  // namespace lrkv
