// Batched page factorisation (PuzzleKV section 3.3, Eq. 2 and the Gram route).
//
// A P x d page X (P = 32 < d) is factored through its P x P Gram matrix
// G = X X^T: the top-r eigenvectors Q_r of G are the leading left singular
// vectors of X, so L = Q_r and R = Q_r^T X are the truncated-SVD factors
// (R = S_r W_r^T). Pages have one shape, so many are factored in one launch.
//
// One workgroup of four waves per page matrix (K or V of one page):
//   1. X (fp16) -> G on the 32x32x16 MFMA (A and B fragments are the same rows).
//   2. Cyclic Jacobi on G in LDS, fp32, round-robin (circle-method) ordering:
//      each round rotates 16 disjoint index pairs at once, applied as one pass
//      of 2x2 block updates (one block per thread; rows and columns together) plus the eigenvector
//      columns, written to the next round's positions in a second buffer. A
//      pair is skipped when |g_pq| <= 1e-6 trace(G); the sweeps stop when a
//      sweep skips every pair, when the off-diagonal Frobenius norm after a
//      sweep is at most 1e-4 trace(G) (the rank-r subspace error is second
//      order in it), or after max_sweeps.
//   3. Eigenvalues sorted descending (ties: lower index first); L = the first r
//      eigenvectors rounded to fp16, R = L^T X accumulated in fp32, stored fp16
//      (value pages transposed: L^T and R^T, the layout the decode reads). With
//      int4 factors (PuzzleKV, per-factor INT4) L is quantised in groups of 32
//      stored elements first and R = L_hat^T X is formed from the dequantised
//      L_hat, then quantised likewise (value R^T in rank quads).
// The page-table entries are switched to "factored" by a second kernel so that
// the K and V waves of one page never race on them.
#include "common.h"

#include <math.h>

namespace lrkv {
namespace {

struct FactorArgs {
    const half_t *dk, *dv, *src_k, *src_v;
    half_t *lk, *rk, *lv, *rv;
    half_t *lk_s, *rk_s, *lv_s, *rv_s;   // int4 factors: one scale per 32 stored elements
    int32_t* table;
    const int32_t* pages;
    int n_pages, B, H, P, sink, window, max_pages, rank_k, rank_v, src_len, max_sweeps;
    bool int4;
};

// Resolves a (b, h, page) triple: returns false when it must be skipped; sets the
// source pointer of the page's K (or V) otherwise. `dim_major`: the source is
// a dense slot's values, stored [d][P].
template <int D>
__device__ bool resolve(const FactorArgs& a, int idx, bool is_v, int& b, int& h, int& pg,
                        const half_t*& X, bool& dim_major) {
    dim_major = false;
    b = a.pages[3 * idx + 0];
    h = a.pages[3 * idx + 1];
    pg = a.pages[3 * idx + 2];
    if (b < 0 || b >= a.B || h < 0 || h >= a.H || pg < 0 || pg >= a.max_pages) return false;
    const long bh = (long)b * a.H + h;
    if (a.src_k) {
        if ((long)(pg + 1) * a.P > a.src_len) return false;
        X = (is_v ? a.src_v : a.src_k) + (bh * a.src_len + (long)pg * a.P) * D;
        return true;
    }
    const int entry = a.table[bh * a.max_pages + pg];
    if (entry >= 0 || entry == LRKV_PAGE_EMPTY) return false;
    const int slot = -1 - entry;
    if (slot >= a.sink + a.window) return false;
    X = (is_v ? a.dv : a.dk) + ((bh * (a.sink + a.window) + slot) * a.P) * D;
    dim_major = is_v;
    return true;
}

// Circle-method position map of the round-robin ordering: positions 2k and
// 2k+1 hold the pair rotated in a round; after the round, the element at
// position x moves to sigma(x). Position 0 stays; the other 31 positions form
// one cycle (top row 2 -> 4 -> ... -> 30, bottom row 31 -> 29 -> ... -> 1,
// 30 -> 31, 1 -> 2), so any two indices share a pair exactly once in 31
// rounds and the positions are the identity again after each sweep.
__device__ __forceinline__ int sigma(int x) {
    if (x == 0) return 0;
    if (x == 1) return 2;
    if (x & 1) return x - 2;
    return x == 30 ? 31 : x + 2;
}

template <int D>
__global__ __launch_bounds__(256) void factor_pages(const FactorArgs a) {
    constexpr int P = 32, LD = P + 1;
    __shared__ float Gb[2][P][LD];     // G, double-buffered across rounds
    __shared__ float Vb[2][P][LD];     // eigenvectors (columns), likewise
    __shared__ half_t Xs[P][D + 8];
    __shared__ float rot[16][2];
    __shared__ int order[P];
    __shared__ int stop;

    const int tid = threadIdx.x, l = tid & 63, wv = tid >> 6;
    const int m = blockIdx.x;
    if (m >= 2 * a.n_pages) return;
    const int idx = m >> 1;
    const bool is_v = m & 1;
    int b, h, pg;
    const half_t* X;
    bool dim_major;
    if (!resolve<D>(a, idx, is_v, b, h, pg, X, dim_major)) return;
    const int r = is_v ? a.rank_v : a.rank_k;

    // ---- Gram matrix on the MFMA (wave 0); X kept in LDS for R = L^T X
    if (dim_major) {
        // X^T [D][P] in global memory: transpose into Xs first
        for (int e = tid; e < D * P / 8; e += 256) {
            const int dd = e / (P / 8), t8 = e % (P / 8);
            const half8 x = *reinterpret_cast<const half8*>(X + (long)dd * P + 8 * t8);
#pragma unroll
            for (int j = 0; j < 8; ++j) Xs[8 * t8 + j][dd] = x[j];
        }
        __syncthreads();
    }
    if (wv == 0) {
        floatx16 acc = floatx16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            half8 x;
            if (dim_major) {
                x = *reinterpret_cast<const half8*>(&Xs[l & 31][16 * kk + 8 * (l >> 5)]);
            } else {
                x = *reinterpret_cast<const half8*>(X + (long)(l & 31) * D + 16 * kk + 8 * (l >> 5));
                *reinterpret_cast<half8*>(&Xs[l & 31][16 * kk + 8 * (l >> 5)]) = x;
            }
            acc = mfma32(x, x, acc);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) Gb[0][8 * (i / 4) + 4 * (l >> 5) + (i % 4)][l & 31] = acc[i];
    }
    for (int e = tid; e < P * P; e += 256) Vb[0][e / P][e % P] = (e / P == e % P) ? 1.0f : 0.0f;
    __syncthreads();
    // every wave forms the same trace
    float tr = l < P ? Gb[0][l][l] : 0.0f;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) tr += __shfl_xor(tr, o, kWave);
    const float thr = 1e-6f * tr;

    // ---- cyclic Jacobi. Round: threads k < 16 form the rotation of positions
    // (2k, 2k+1); then G <- J^T G J and V <- V J in one pass of 2x2 blocks, each
    // result written at its position for the next round (sigma) in the other
    // buffer. Thread t owns the block (pair t / 16) x (pair t % 16) and the
    // eigenvector rows t / 16 and t / 16 + 16 of pair t % 16: fixed addresses.
    const int pa = tid >> 4, pb = tid & 15, pv = tid & 15, vr = tid >> 4;
    const int ra0 = sigma(2 * pa), ra1 = sigma(2 * pa + 1);
    const int cb0 = sigma(2 * pb), cb1 = sigma(2 * pb + 1);
    int cur = 0;
    for (int sweep = 0; sweep < a.max_sweeps; ++sweep) {
        int rotated = 0;
        for (int rd = 0; rd < P - 1; ++rd) {
            float (*G)[LD] = Gb[cur];
            float (*Gn)[LD] = Gb[cur ^ 1];
            float (*V)[LD] = Vb[cur];
            float (*Vn)[LD] = Vb[cur ^ 1];
            if (tid < 16) {
                const float gpp = G[2 * tid][2 * tid], gqq = G[2 * tid + 1][2 * tid + 1];
                const float apq = G[2 * tid][2 * tid + 1];
                float c = 1.0f, s = 0.0f;
                if (fabsf(apq) > thr) {
                    const float tau = (gqq - gpp) * __builtin_amdgcn_rcpf(2.0f * apq);
                    const float t = copysignf(__builtin_amdgcn_rcpf(fabsf(tau) + __builtin_amdgcn_sqrtf(fmaf(tau, tau, 1.0f))), tau);
                    c = __builtin_amdgcn_rsqf(fmaf(t, t, 1.0f));
                    s = t * c;
                    rotated = 1;
                }
                rot[tid][0] = c;
                rot[tid][1] = s;
            }
            __syncthreads();
            {
                const float ca = rot[pa][0], sa = rot[pa][1], cb = rot[pb][0], sb = rot[pb][1];
                const float g00 = G[2 * pa][2 * pb], g01 = G[2 * pa][2 * pb + 1];
                const float g10 = G[2 * pa + 1][2 * pb], g11 = G[2 * pa + 1][2 * pb + 1];
                const float r00 = fmaf(ca, g00, -sa * g10), r01 = fmaf(ca, g01, -sa * g11);
                const float r10 = fmaf(sa, g00, ca * g10), r11 = fmaf(sa, g01, ca * g11);
                float n01 = fmaf(sb, r00, cb * r01), n10 = fmaf(cb, r10, -sb * r11);
                if (pa == pb && sa != 0.0f) n01 = n10 = 0.0f;   // the pair's own entry is annihilated
                Gn[ra0][cb0] = fmaf(cb, r00, -sb * r01);
                Gn[ra0][cb1] = n01;
                Gn[ra1][cb0] = n10;
                Gn[ra1][cb1] = fmaf(sb, r10, cb * r11);
                const float cv = cb, sv = sb;            // pv == pb
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int row = vr + 16 * i;
                    const float vp = V[row][2 * pv], vq = V[row][2 * pv + 1];
                    Vn[row][cb0] = fmaf(cv, vp, -sv * vq);
                    Vn[row][cb1] = fmaf(sv, vp, cv * vq);
                }
            }
            __syncthreads();
            cur ^= 1;
        }
        if (!__syncthreads_or(rotated)) break;
        // off-diagonal Frobenius norm of G after the sweep, against 1e-4 trace(G):
        // wave 0 sums it (lane l: row l / 2, columns of half l % 2) and decides
        if (wv == 0) {
            float off = 0.0f;
            float (*Gc)[LD] = Gb[cur];
            const int row = l >> 1, c0 = 16 * (l & 1);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float v = Gc[row][c0 + j];
                off = c0 + j == row ? off : fmaf(v, v, off);
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) off += __shfl_xor(off, o, kWave);
            if (l == 0) stop = off <= 1e-8f * tr * tr;
        }
        __syncthreads();
        if (stop) break;
    }
    float (*G)[LD] = Gb[cur];
    float (*V)[LD] = Vb[cur];
    float (*Ls)[LD] = Gb[cur ^ 1];     // free now: L^T [k][t] as rounded to fp16

    // ---- descending eigen-order, ties towards the lower index
    if (tid < P) {
        const float li = G[tid][tid];
        int rank = 0;
        for (int j = 0; j < P; ++j) {
            const float lj = G[j][j];
            rank += (lj > li) || (lj == li && j < tid);
        }
        order[rank] = tid;
    }
    __syncthreads();

    const long bh = (long)b * a.H + h;
    const long page = bh * a.max_pages + pg;
    if (!a.int4) {
        half_t* Lo = (is_v ? a.lv : a.lk) + page * P * r;
        half_t* Ro = (is_v ? a.rv : a.rk) + page * (long)r * D;
        // keys: L [P][r], R [r][D]; values transposed: L^T [r][P], R^T [D][r]
        for (int e = tid; e < P * r; e += 256) {
            const int t = e / r, k = e % r;
            const half_t v = (half_t)V[t][order[k]];
            Lo[is_v ? k * P + t : e] = v;
            Ls[k][t] = (float)v;
        }
        __syncthreads();
        // R[k][d] = sum_t fp16(L[t][k]) X[t][d]: thread d < D owns dim d
        if (tid < D) {
            float x0[P];
#pragma unroll
            for (int t = 0; t < P; ++t) x0[t] = (float)Xs[t][tid];
            for (int k = 0; k < r; ++k) {
                float s0 = 0.0f;
#pragma unroll
                for (int t = 0; t < P; ++t) s0 = fmaf(Ls[k][t], x0[t], s0);
                if (is_v) Ro[(long)tid * r + k] = (half_t)s0;
                else Ro[(long)k * D + tid] = (half_t)s0;
            }
        }
        return;
    }

    // ---- int4 factors (r <= 16): quantise L in groups of 32 consecutive stored
    // elements (one group per lane), then R = L_hat^T X from the dequantised L_hat,
    // then R likewise. Stored orders: keys L [P][r], R [r][D]; values L^T [r][P],
    // R^T in rank quads [r/4][D][4] (a decode lane's eight dims of one quad are
    // then one 16-byte run with one scale).
    uint8_t* Lc = (uint8_t*)(is_v ? a.lv : a.lk) + page * (P * r / 2);
    uint8_t* Rc = (uint8_t*)(is_v ? a.rv : a.rk) + page * (r * D / 2);
    half_t* Lsc = (is_v ? a.lv_s : a.lk_s) + page * (P * r / 32);
    half_t* Rsc = (is_v ? a.rv_s : a.rk_s) + page * (r * D / 32);
    auto store_group = [&](uint8_t* codes_out, half_t* scale_out, int j, const float* x, float* deq) {
        int c[32];
        half_t sc;
        quant_group(x, c, &sc);
        uint32_t wd[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t v = 0;
#pragma unroll
            for (int n = 0; n < 8; ++n) v |= ((uint32_t)c[8 * q + n] & 0xFu) << (4 * n);
            wd[q] = v;
        }
        *reinterpret_cast<uint4*>(codes_out + 16 * j) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        scale_out[j] = sc;
        if (deq) {
#pragma unroll
            for (int n = 0; n < 32; ++n) deq[n] = (float)c[n] * (float)sc;
        }
    };
    if (tid < P * r / 32) {
        float x[32], xd[32];
#pragma unroll
        for (int n = 0; n < 32; ++n) {
            const int e = 32 * tid + n;
            const int t = is_v ? e % P : e / r, k = is_v ? e / P : e % r;
            x[n] = V[t][order[k]];
        }
        store_group(Lc, Lsc, tid, x, xd);
#pragma unroll
        for (int n = 0; n < 32; ++n) {
            const int e = 32 * tid + n;
            const int t = is_v ? e % P : e / r, k = is_v ? e / P : e % r;
            Ls[k][t] = xd[n];
        }
    }
    __syncthreads();
    // R (fp32) [r][D] into the eigenvector buffers, which are free now
    float* Rs = &Vb[0][0][0];
    if (tid < D) {
        float x0[P];
#pragma unroll
        for (int t = 0; t < P; ++t) x0[t] = (float)Xs[t][tid];
        for (int k = 0; k < r; ++k) {
            float s0 = 0.0f;
#pragma unroll
            for (int t = 0; t < P; ++t) s0 = fmaf(Ls[k][t], x0[t], s0);
            Rs[k * D + tid] = s0;
        }
    }
    __syncthreads();
    if (tid < r * D / 32) {
        float x[32];
#pragma unroll
        for (int n = 0; n < 32; ++n) {
            const int e = 32 * tid + n;
            // keys R [r][D]; values in rank quads, [r/4][D][4]
            const int k = is_v ? 4 * (e / (4 * D)) + e % 4 : e / D, d = is_v ? (e / 4) % D : e % D;
            x[n] = Rs[k * D + d];
        }
        store_group(Rc, Rsc, tid, x, nullptr);
    }
}

__global__ void mark_factored(const FactorArgs a) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= a.n_pages) return;
    int b, h, pg;
    const half_t* X;
    bool dim_major;
    if (!resolve<128>(a, idx, false, b, h, pg, X, dim_major)) return;
    a.table[((long)b * a.H + h) * a.max_pages + pg] = pg;
}

}  // namespace

int32_t launch_factor_page(const lrkv_paged_cache* c, const int32_t* pages, int n_pages,
                           const half_t* src_k, const half_t* src_v, int src_len, int max_sweeps,
                           hipStream_t st) {
    if (n_pages == 0) return LRKV_OK;
    FactorArgs a{(const half_t*)c->dense_k, (const half_t*)c->dense_v, src_k, src_v,
                 (half_t*)c->lk, (half_t*)c->rk, (half_t*)c->lv, (half_t*)c->rv,
                 (half_t*)c->lk_s, (half_t*)c->rk_s, (half_t*)c->lv_s, (half_t*)c->rv_s, c->page_table,
                 pages, n_pages, c->batch, c->kv_heads, c->page_size, c->sink_pages,
                 c->window_pages, c->max_pages, c->rank_k, c->rank_v, src_len, max_sweeps,
                 c->factor_fmt == LRKV_FMT_INT4_G32};
    hipLaunchKernelGGL(factor_pages<128>, dim3(2 * n_pages), dim3(256), 0, st, a);
    hipLaunchKernelGGL(mark_factored, dim3((n_pages + 255) / 256), dim3(256), 0, st, a);
    return last_launch_status();
}

}  // namespace lrkv
