// Batched page factorisation (PuzzleKV section 3.3, Eq. 2 and the Gram route).
//
// A P x d page X (P = 32 < d) is factored through its P x P Gram matrix
// G = X X^T: the top-r eigenvectors Q_r of G are the leading left singular
// vectors of X, so L = Q_r and R = Q_r^T X are the truncated-SVD factors
// (R = S_r W_r^T). Pages have one shape, so many are factored in one launch.
//
// One wave per page matrix (K or V of one page):
//   1. X (fp16) -> G on the 32x32x16 MFMA (A and B fragments are the same rows).
//   2. Cyclic Jacobi on G in LDS, fp32, round-robin ordering: each round rotates
//      16 disjoint index pairs at once (rows, then columns, then the eigenvector
//      matrix). A pair is skipped when |g_pq| <= 1e-6 trace(G); the sweeps stop
//      when a sweep skips every pair or after max_sweeps.
//   3. Eigenvalues sorted descending (ties: lower index first); L = the first r
//      eigenvectors rounded to fp16, R = L^T X accumulated in fp32, stored fp16
//      (value pages transposed: L^T and R^T, the layout the decode reads).
// The page-table entries are switched to "factored" by a second kernel so that
// the K and V waves of one page never race on them.
#include "common.h"

#include <math.h>

namespace lrkv {
namespace {

struct FactorArgs {
    const half_t *dk, *dv, *src_k, *src_v;
    half_t *lk, *rk, *lv, *rv;
    int32_t* table;
    const int32_t* pages;
    int n_pages, B, H, P, sink, window, max_pages, rank_k, rank_v, src_len, max_sweeps;
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

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__global__ __launch_bounds__(256) void factor_pages(const FactorArgs a) {
    constexpr int P = 32;
    __shared__ float Gs[4][P][P + 1];
    __shared__ float Vs[4][P][P + 1];
    __shared__ half_t Xs[4][P][D + 8];
    __shared__ float rot[4][16][2];
    __shared__ int rpq[4][16][2];
    __shared__ int order[4][P];

    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int m = blockIdx.x * 4 + w;
    if (m >= 2 * a.n_pages) return;
    const int idx = m >> 1;
    const bool is_v = m & 1;
    int b, h, pg;
    const half_t* X;
    bool dim_major;
    if (!resolve<D>(a, idx, is_v, b, h, pg, X, dim_major)) return;
    const int r = is_v ? a.rank_v : a.rank_k;
    float (*G)[P + 1] = Gs[w];
    float (*V)[P + 1] = Vs[w];

    // ---- Gram matrix on the MFMA; X kept in LDS for R = L^T X
    floatx16 acc = floatx16{};
    if (dim_major) {
        // X^T [D][P] in global memory: transpose into Xs first
        for (int e = l; e < D * P / 8; e += 64) {
            const int dd = e / (P / 8), t8 = e % (P / 8);
            const half8 x = *reinterpret_cast<const half8*>(X + (long)dd * P + 8 * t8);
#pragma unroll
            for (int j = 0; j < 8; ++j) Xs[w][8 * t8 + j][dd] = x[j];
        }
        wave_sync_lds();
    }
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        half8 x;
        if (dim_major) {
            x = *reinterpret_cast<const half8*>(&Xs[w][l & 31][16 * kk + 8 * (l >> 5)]);
        } else {
            x = *reinterpret_cast<const half8*>(X + (long)(l & 31) * D + 16 * kk + 8 * (l >> 5));
            *reinterpret_cast<half8*>(&Xs[w][l & 31][16 * kk + 8 * (l >> 5)]) = x;
        }
        acc = mfma32(x, x, acc);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) G[8 * (i / 4) + 4 * (l >> 5) + (i % 4)][l & 31] = acc[i];
    for (int e = l; e < P * P; e += 64) V[e / P][e % P] = (e / P == e % P) ? 1.0f : 0.0f;
    wave_sync_lds();
    float tr = l < P ? G[l][l] : 0.0f;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) tr += __shfl_xor(tr, o, kWave);
    const float thr = 1e-6f * tr;

    // ---- cyclic Jacobi, round-robin pairs
    for (int sweep = 0; sweep < a.max_sweeps; ++sweep) {
        int rotated = 0;
        for (int rd = 0; rd < P - 1; ++rd) {
            if (l < 16) {
                int p = l == 0 ? P - 1 : (rd + l) % (P - 1);
                int q = l == 0 ? rd : (rd + (P - 1) - l) % (P - 1);
                if (p > q) { const int t = p; p = q; q = t; }
                const float apq = G[p][q];
                float c = 1.0f, s = 0.0f;
                if (fabsf(apq) > thr) {
                    const float tau = (G[q][q] - G[p][p]) / (2.0f * apq);
                    const float t = copysignf(1.0f, tau) / (fabsf(tau) + sqrtf(fmaf(tau, tau, 1.0f)));
                    c = 1.0f / sqrtf(fmaf(t, t, 1.0f));
                    s = t * c;
                    rotated = 1;
                }
                rot[w][l][0] = c;
                rot[w][l][1] = s;
                rpq[w][l][0] = p;
                rpq[w][l][1] = q;
            }
            wave_sync_lds();
            // rows: G <- J^T G
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int item = l + 64 * i, k = item >> 5, col = item & 31;
                const int p = rpq[w][k][0], q = rpq[w][k][1];
                const float c = rot[w][k][0], s = rot[w][k][1];
                const float gp = G[p][col], gq = G[q][col];
                G[p][col] = fmaf(c, gp, -s * gq);
                G[q][col] = fmaf(s, gp, c * gq);
            }
            wave_sync_lds();
            // columns: G <- G J, V <- V J
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int item = l + 64 * i, k = item >> 5, row = item & 31;
                const int p = rpq[w][k][0], q = rpq[w][k][1];
                const float c = rot[w][k][0], s = rot[w][k][1];
                const float gp = G[row][p], gq = G[row][q];
                G[row][p] = fmaf(c, gp, -s * gq);
                G[row][q] = fmaf(s, gp, c * gq);
                const float vp = V[row][p], vq = V[row][q];
                V[row][p] = fmaf(c, vp, -s * vq);
                V[row][q] = fmaf(s, vp, c * vq);
            }
            wave_sync_lds();
        }
        if (!__any(rotated)) break;
    }

    // ---- descending eigen-order, ties towards the lower index
    if (l < P) {
        const float li = G[l][l];
        int rank = 0;
        for (int j = 0; j < P; ++j) {
            const float lj = G[j][j];
            rank += (lj > li) || (lj == li && j < l);
        }
        order[w][rank] = l;
    }
    wave_sync_lds();

    const long bh = (long)b * a.H + h;
    half_t* Lo = (is_v ? a.lv : a.lk) + (bh * a.max_pages + pg) * P * r;
    half_t* Ro = (is_v ? a.rv : a.rk) + (bh * a.max_pages + pg) * (long)r * D;
    // keys: L [P][r], R [r][D]; values transposed: L^T [r][P], R^T [D][r]
    for (int e = l; e < P * r; e += 64) {
        const int t = e / r, k = e % r;
        Lo[is_v ? k * P + t : e] = (half_t)V[t][order[w][k]];
    }
    // R[k][d] = sum_t fp16(L[t][k]) X[t][d]
    for (int k = 0; k < r; ++k) {
        const int col = order[w][k];
        for (int d = l; d < D; d += 64) {
            float s = 0.0f;
#pragma unroll 8
            for (int t = 0; t < P; ++t) s = fmaf((float)(half_t)V[t][col], (float)Xs[w][t][d], s);
            Ro[is_v ? (long)d * r + k : (long)k * D + d] = (half_t)s;
        }
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
                 (half_t*)c->lk, (half_t*)c->rk, (half_t*)c->lv, (half_t*)c->rv, c->page_table,
                 pages, n_pages, c->batch, c->kv_heads, c->page_size, c->sink_pages,
                 c->window_pages, c->max_pages, c->rank_k, c->rank_v, src_len, max_sweeps};
    hipLaunchKernelGGL(factor_pages<128>, dim3((2 * n_pages + 3) / 4), dim3(256), 0, st, a);
    hipLaunchKernelGGL(mark_factored, dim3((n_pages + 255) / 256), dim3(256), 0, st, a);
    return last_launch_status();
}

}  // namespace lrkv
