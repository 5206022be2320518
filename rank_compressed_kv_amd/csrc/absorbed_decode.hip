// Absorbed-query decode attention (no RoPE) over a Palu latent cache (gfx950).
//
// Palu digest, Method details (key fusion): without RoPE the key reconstruction
// is absorbed into the query, q' = q (B^k)^T, so scores are H^k q' and no key is
// ever rebuilt; values stay latent, o = p H^v. The path is a pure latent stream.
#include "tiles.h"

#include <math.h>

namespace lrkv {
namespace {

struct AbsorbArgs {
    const void* hk;
    const void* hv;
    const half_t* sk;
    const half_t* sv;
    const int32_t* lens;
    const float* q;       // [B][Hq][R]
    float* part;
    int U, cap, n_split, chunk;
    float qscale;         // sm_scale * log2(e)
};

// Every wave streams its own 32-token tiles (tile w, w+4, ...) with no barrier:
// scores on a 16x16x32 MFMA (A = key rows straight from memory, B = the absorbed
// queries, heads padded to 16), p x H^v on a second 16x16x32 MFMA whose token
// order follows the score layout, then the 4 wave states are merged in LDS.
template <int R, int NH, bool INT4>
__global__ __launch_bounds__(256, 2) void absorbed_decode(const AbsorbArgs p) {
    constexpr int KS = R / 32;
    constexpr int VM = R / 16;
    static_assert(NH <= 16, "at most 16 query heads per unit");
    __shared__ float wst[4][NH][R + 2];

    const int split = blockIdx.x, u = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int Hq = p.U * NH, j0 = u * NH;
    const int len = min(p.lens[b], p.cap);        // never read past the capacity
    const int t_begin = split * p.chunk;
    const int t_end = min(len, t_begin + p.chunk);
    const long bu = (long)b * p.U + u;
    float* part = p.part + ((long)(b * Hq + j0) * p.n_split + split) * (R + 2);
    const long hstride = (long)p.n_split * (R + 2);
    if (t_begin >= t_end) {
        for (int e = tid; e < NH * (R + 2); e += 256) {
            const int h = e / (R + 2), c = e % (R + 2);
            part[h * hstride + c] = c == 0 ? -INFINITY : 0.0f;
        }
        return;
    }

    // B fragments of the absorbed queries: head hn = l%16, dims 32kk + 8(l/16) + 0..7,
    // scaled by qscale * 2^e per head (max |q'| in [2^14, 2^15)).
    const int hn = l & 15, g = l >> 4;
    half8 qf[KS];
    float inv = 1.0f;
    {
        float qv[KS][8];
        float mx = 0.0f;
        // unconditional 16-byte loads (padding heads read head NH - 1, then zero)
        const float* qrow = p.q + ((long)b * Hq + j0 + (hn < NH ? hn : NH - 1)) * R + 8 * g;
        const float qs = hn < NH ? p.qscale : 0.0f;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const float4 x0 = *reinterpret_cast<const float4*>(qrow + 32 * kk);
            const float4 x1 = *reinterpret_cast<const float4*>(qrow + 32 * kk + 4);
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qv[kk][e] = xs[e] * qs;
                mx = fmaxf(mx, fabsf(qv[kk][e]));
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        const int ex = (mx > 0.0f && isfinite(mx)) ? 14 - ilogbf(mx) : 0;
        inv = ldexpf(1.0f, -ex);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[kk][e] = (half_t)ldexpf(qv[kk][e], ex);
    }

    float m_run = -INFINITY, l_run = 0.0f;
    floatx4 acc[VM];
#pragma unroll
    for (int v = 0; v < VM; ++v) acc[v] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int n_tiles = (t_end - t_begin + 31) / 32;
    for (int it = w; it < n_tiles; it += 4) {
        const int t0 = t_begin + 32 * it;
        const bool tail = t0 + 32 > t_end;
        const long blk_base = bu * (p.cap / kTile) + t0 / kTile;
        // every load of the tile is issued before the first MFMA: key rows
        // t0 + 16 mt + hn (clamped to the last valid token; their scores are
        // masked), value dims 16 v + hn at tokens {4g..4g+3, 16+4g..16+4g+3}
        half8 ka[2][KS], va[VM];
        uint32_t kcode[2][KS], vlo[VM], vhi[VM];
        half_t ksc[2][KS];
        half4 vslo[VM], vshi[VM];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const long row = bu * p.cap + min(t0 + 16 * mt + hn, t_end - 1);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                if constexpr (!INT4) {
                    ka[mt][kk] = *reinterpret_cast<const half8*>((const half_t*)p.hk + row * R + 32 * kk + 8 * g);
                } else {
                    kcode[mt][kk] = *reinterpret_cast<const uint32_t*>((const uint8_t*)p.hk + row * (R / 2) + 16 * kk + 4 * g);
                    ksc[mt][kk] = p.sk[row * (R / 32) + kk];
                }
            }
        }
#pragma unroll
        for (int v = 0; v < VM; ++v) {
            const int dim = 16 * v + hn;
            if constexpr (!INT4) {
                const half_t* src = (const half_t*)p.hv + (blk_base * R + dim) * kTile;
                const half4 lo = *reinterpret_cast<const half4*>(src + 4 * g);
                const half4 hi = *reinterpret_cast<const half4*>(src + 16 + 4 * g);
                va[v] = half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
                const uint8_t* src = (const uint8_t*)p.hv + (blk_base * R + dim) * (kTile / 2);
                vlo[v] = *reinterpret_cast<const uint16_t*>(src + 2 * g);
                vhi[v] = *reinterpret_cast<const uint16_t*>(src + 8 + 2 * g);
                const half_t* ss = p.sv + (blk_base * (R / 32) + dim / 32) * kTile;
                vslo[v] = *reinterpret_cast<const half4*>(ss + 4 * g);
                vshi[v] = *reinterpret_cast<const half4*>(ss + 16 + 4 * g);
            }
        }
        // scores: two 16-token M-tiles; lane holds tokens 16mt + 4g + e for head hn
        floatx4 sc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                half8 a;
                if constexpr (!INT4) {
                    a = ka[mt][kk];
                } else {
                    const float s = (float)ksc[mt][kk];
#pragma unroll
                    for (int e = 0; e < 8; ++e) a[e] = (half_t)((float)nibble(kcode[mt][kk], e) * s);
                }
                sc[mt] = mfma16(a, qf[kk], sc[mt]);
            }
        }
        float s8[8];
        float mt_loc = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = t0 + 16 * mt + 4 * g + e;
                const float v = t < t_end ? sc[mt][e] * inv : -INFINITY;
                s8[4 * mt + e] = v;
                mt_loc = fmaxf(mt_loc, v);
            }
        mt_loc = fmaxf(mt_loc, __shfl_xor(mt_loc, 16, kWave));
        mt_loc = fmaxf(mt_loc, __shfl_xor(mt_loc, 32, kWave));
        const float mn = fmaxf(m_run, mt_loc);
        const float alpha = exp2f(m_run - mn);
        half8 pf;
        float psum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pv = exp2f(s8[e] - mn);
            psum += pv;
            pf[e] = (half_t)pv;
        }
        psum += __shfl_xor(psum, 16, kWave);
        psum += __shfl_xor(psum, 32, kWave);
        l_run = fmaf(l_run, alpha, psum);
        m_run = mn;
        if (hn >= NH) pf = half8{};
        // values: A = V^T [16 dims][tokens {4g..4g+3, 16+4g..16+4g+3}]
        if constexpr (INT4) {
#pragma unroll
            for (int v = 0; v < VM; ++v)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    va[v][e] = (half_t)((float)nibble(vlo[v], e) * (float)vslo[v][e]);
                    va[v][4 + e] = (half_t)((float)nibble(vhi[v], e) * (float)vshi[v][e]);
                }
        }
        if (tail) {
            // tokens past t_end: zero (their p is zero; the memory may hold anything)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = t0 + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4);
                if (t >= t_end) {
#pragma unroll
                    for (int v = 0; v < VM; ++v) va[v][e] = (half_t)0.0f;
                }
            }
        }
#pragma unroll
        for (int v = 0; v < VM; ++v) {
            acc[v] *= alpha;
            acc[v] = mfma16(va[v], pf, acc[v]);
        }
    }

    // merge the 4 waves' states: lane (hn, g) holds dims 16v + 4g + e of head hn
    if (hn < NH) {
        if (g == 0) { wst[w][hn][0] = m_run; wst[w][hn][1] = l_run; }
#pragma unroll
        for (int v = 0; v < VM; ++v)
#pragma unroll
            for (int e = 0; e < 4; ++e) wst[w][hn][2 + 16 * v + 4 * g + e] = acc[v][e];
    }
    __syncthreads();
    for (int e = tid; e < NH * (R + 2); e += 256) {
        const int h = e / (R + 2), c = e % (R + 2);
        float mx = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) mx = fmaxf(mx, wst[ww][h][0]);
        float val;
        if (c == 0) {
            val = mx;
        } else {
            val = 0.0f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                const float m = wst[ww][h][0];
                if (m != -INFINITY) val = fmaf(exp2f(m - mx), wst[ww][h][c], val);
            }
        }
        part[h * hstride + c] = val;
    }
}

template <int R, int NH, bool INT4>
void launch_absorb(const AbsorbArgs& a, int B, hipStream_t st) {
    hipLaunchKernelGGL((absorbed_decode<R, NH, INT4>), dim3(a.n_split, a.U, B), dim3(256), 0, st, a);
}

}  // namespace

bool absorbed_shape_supported(int r, int nh) {
    return (r == 32 || r == 64 || r == 128 || r == 256) && (nh == 2 || nh == 4);
}

int32_t launch_absorbed_decode(const lrkv_latent_cache* c, const float* q, float* part, int n_split,
                               int chunk, float qscale, hipStream_t st) {
    const int nh = c->kv_per_unit * c->q_per_kv, r = c->rank;
    const bool int4 = c->fmt == LRKV_FMT_INT4_G32;
    AbsorbArgs a{c->hk, c->hv, (const half_t*)c->sk, (const half_t*)c->sv, c->lens, q, part,
                 c->units, c->capacity, n_split, chunk, qscale};
#define LRKV_ABS(R_, NH_)                                                                    \
    if (r == R_ && nh == NH_) {                                                              \
        if (int4) launch_absorb<R_, NH_, true>(a, c->batch, st);                             \
        else launch_absorb<R_, NH_, false>(a, c->batch, st);                                 \
        return LRKV_OK;                                                                      \
    }
    LRKV_ABS(32, 2) LRKV_ABS(64, 2) LRKV_ABS(128, 2) LRKV_ABS(256, 2)
    LRKV_ABS(32, 4) LRKV_ABS(64, 4) LRKV_ABS(128, 4) LRKV_ABS(256, 4)
#undef LRKV_ABS
    return LRKV_ERR_UNSUPPORTED;
}

}  // namespace lrkv
