// Hybrid paged decode attention (PuzzleKV section 3.3, step 4).
//
// Pages of one (sequence, KV head) are dense (sink page, local window) or
// factored (X_hat = L R, Eq. 2). A factored page is evaluated from its factors
// without forming X_hat: scores s = (q R_K^T) L_K^T / sqrt(d), values
// (a L_V) R_V (the value side follows by associativity; the page's text stops
// after the key-side formula). All partial results are merged by online softmax.
//
// Work split: one workgroup (4 waves) per (page range, KV head, sequence); the
// waves take pages round-robin and keep private (m, l, o) states that are merged
// in LDS at the end; chunks are merged by merge_splits. Lane l serves query head
// l/16 of the KV head and dims [8 (l%16), 8 (l%16) + 8); sums over a head's 16
// lanes use DPP row operations.
#include "common.h"

#include <math.h>

namespace lrkv {
namespace {

// DPP controls (gfx9): quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror, row_mirror.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    v += dpp<0x140>(v);
    return v;
}
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    return v;
}

__device__ __forceinline__ void load8(const half_t* p, float* o) {
    const half8 h = *reinterpret_cast<const half8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (float)h[e];
}

struct HybridArgs {
    const half_t *dk, *dv, *lk, *rk, *lv, *rv;
    const int32_t* table;
    const int32_t* lens;
    const float* q;       // [B][Hq][D]
    float* part;          // [B][Hq][n_split][D + 2]
    int H, G, P, sink, window, rkk, rvv, max_pages, n_split, pps;
    float qscale;         // sm_scale * log2(e)
};

template <int D>
__global__ __launch_bounds__(256, 2) void hybrid_decode(const HybridArgs a) {
    static_assert(D == 128, "head_dim 128");
    constexpr int P = 32;
    __shared__ float wst[4][4][D + 2];
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int hh = l >> 4, sub = l & 15;
    const bool head_ok = hh < a.G;
    const int Hq = a.H * a.G;
    const int len = min(a.lens[b], a.max_pages * 32);
    const int npg = (len + P - 1) / P;
    const int p_begin = split * a.pps;
    const int p_end = min(npg, p_begin + a.pps);
    const long bh = (long)b * a.H + h;
    const int j = h * a.G + (head_ok ? hh : 0);

    float qv[8];
    {
        const float* qp = a.q + ((long)b * Hq + j) * D + 8 * sub;
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = qp[e] * a.qscale;
    }
    float m_run = -INFINITY, l_run = 0.0f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.0f;

    for (int pg = p_begin + w; pg < p_end; pg += 4) {
        const int entry = a.table[bh * a.max_pages + pg];
        const int ntok = min(P, len - pg * P);
        // pages never written (or out of range) are skipped
        if (entry >= a.max_pages || (entry < 0 && -1 - (long)entry >= a.sink + a.window)) continue;
        float s2[2];                          // tokens sub and sub + 16
        float alpha, pv[2];
        if (entry >= 0) {
            // ---- factored page: u = q R_K^T (rank values), s = u L_K^T
            const half_t* Rk = a.rk + ((bh * a.max_pages + entry) * a.rkk) * D;
            const half_t* Lk = a.lk + ((bh * a.max_pages + entry) * P) * a.rkk;
            float s_a = 0.0f, s_b = 0.0f;
            for (int k = 0; k < a.rkk; ++k) {
                float r8[8];
                load8(Rk + (long)k * D + 8 * sub, r8);
                float uk = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) uk = fmaf(qv[e], r8[e], uk);
                uk = row_sum16(uk);
                s_a = fmaf(uk, (float)Lk[sub * a.rkk + k], s_a);
                s_b = fmaf(uk, (float)Lk[(sub + 16) * a.rkk + k], s_b);
            }
            s2[0] = sub < ntok ? s_a : -INFINITY;
            s2[1] = sub + 16 < ntok ? s_b : -INFINITY;
            const float mt = row_max16(fmaxf(s2[0], s2[1]));
            const float mn = fmaxf(m_run, mt);
            alpha = exp2f(m_run - mn);
            pv[0] = exp2f(s2[0] - mn);
            pv[1] = exp2f(s2[1] - mn);
            l_run = fmaf(l_run, alpha, row_sum16(pv[0] + pv[1]));
            m_run = mn;
            // ---- values: w = p L_V (rank values), o = o alpha + w R_V
            const half_t* Lv = a.lv + ((bh * a.max_pages + entry) * P) * a.rvv;
            const half_t* Rv = a.rv + ((bh * a.max_pages + entry) * a.rvv) * D;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] *= alpha;
            for (int k = 0; k < a.rvv; ++k) {
                float wk = pv[0] * (float)Lv[sub * a.rvv + k] + pv[1] * (float)Lv[(sub + 16) * a.rvv + k];
                wk = row_sum16(wk);
                float r8[8];
                load8(Rv + (long)k * D + 8 * sub, r8);
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = fmaf(wk, r8[e], o[e]);
            }
        } else {
            // ---- dense page: scores against K rows, then p V
            const int slot = -1 - entry;
            const half_t* Kp = a.dk + (bh * (a.sink + a.window) + slot) * P * D;
            const half_t* Vp = a.dv + (bh * (a.sink + a.window) + slot) * P * D;
            float my_s[2] = {-INFINITY, -INFINITY};
            for (int t = 0; t < ntok; ++t) {
                float k8[8];
                load8(Kp + (long)t * D + 8 * sub, k8);
                float st = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) st = fmaf(qv[e], k8[e], st);
                st = row_sum16(st);
                if (t == sub) my_s[0] = st;
                if (t == sub + 16) my_s[1] = st;
            }
            const float mt = row_max16(fmaxf(my_s[0], my_s[1]));
            const float mn = fmaxf(m_run, mt);
            alpha = exp2f(m_run - mn);
            pv[0] = exp2f(my_s[0] - mn);
            pv[1] = exp2f(my_s[1] - mn);
            l_run = fmaf(l_run, alpha, row_sum16(pv[0] + pv[1]));
            m_run = mn;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] *= alpha;
            for (int t = 0; t < ntok; ++t) {
                // p of token t lives in lane (t % 16) of this row, slot t / 16
                const float mine = t < 16 ? pv[0] : pv[1];
                const float pt = __shfl(mine, (l & ~15) | (t & 15), kWave);
                float v8[8];
                load8(Vp + (long)t * D + 8 * sub, v8);
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = fmaf(pt, v8[e], o[e]);
            }
        }
    }

    if (head_ok) {
        if (sub == 0) { wst[w][hh][0] = m_run; wst[w][hh][1] = l_run; }
#pragma unroll
        for (int e = 0; e < 8; ++e) wst[w][hh][2 + 8 * sub + e] = o[e];
    }
    __syncthreads();
    float* part = a.part + ((long)(b * Hq + h * a.G) * a.n_split + split) * (D + 2);
    const long hstride = (long)a.n_split * (D + 2);
    for (int e = tid; e < a.G * (D + 2); e += 256) {
        const int g = e / (D + 2), c = e % (D + 2);
        float mx = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) mx = fmaxf(mx, wst[ww][g][0]);
        float val = mx;
        if (c > 0) {
            val = 0.0f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                const float m = wst[ww][g][0];
                if (m != -INFINITY) val = fmaf(exp2f(m - mx), wst[ww][g][c], val);
            }
        }
        part[g * hstride + c] = val;
    }
}

}  // namespace

void launch_merge(const float* part, float* out, int BH, int n_split, int D, hipStream_t st);

int32_t launch_decode_hybrid(int phases, const lrkv_paged_cache* c, const float* q, float sm_scale,
                             float* out, void* ws, const PagedWorkspace& w, hipStream_t st) {
    float* part = (float*)((char*)ws + w.part_off);
    HybridArgs a{(const half_t*)c->dense_k, (const half_t*)c->dense_v, (const half_t*)c->lk,
                 (const half_t*)c->rk, (const half_t*)c->lv, (const half_t*)c->rv, c->page_table,
                 c->lens, q, part, c->kv_heads, c->q_per_kv, c->page_size, c->sink_pages,
                 c->window_pages, c->rank_k, c->rank_v, c->max_pages, w.n_split,
                 w.pages_per_split, sm_scale * kLog2e};
    if (phases & kPhasePartials)
        hipLaunchKernelGGL(hybrid_decode<128>, dim3(w.n_split, c->kv_heads, c->batch), dim3(256), 0, st, a);
    if (phases & kPhaseMerge)
        launch_merge(part, out, c->batch * c->kv_heads * c->q_per_kv, w.n_split, c->head_dim, st);
    return last_launch_status();
}

}  // namespace lrkv
