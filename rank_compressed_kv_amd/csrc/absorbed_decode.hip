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
// queries, heads padded to 16), p x H^v on a second 16x16x32 MFMA, then the 4
// wave states are merged in LDS. Row m of score M-tile mt is token
// 8 (m / 4) + 4 mt + m % 4 of the tile, so lane group g ends up holding tokens
// 8 g .. 8 g + 7: the value fragments are then one contiguous run of the
// dimension-major value block (fp16: 16 bytes; int4: one 32-bit word).
// int4 keys: lane group g reads 16-byte chunks g + 4 q of a token's codes
// (rank 256: q = 0, 1), word w of chunk q serving K step 4 q + w; smaller ranks
// read one word per K step. Codes decode with the exponent-bias trick (element
// order 0, 4, 1, 5, 2, 6, 3, 7 of a word); the queries are loaded in the same
// rank order. int4 value scales are folded into p per 32-dim group.
template <int R>
struct KeyMap {
    static constexpr bool CHUNK = R >= 128;            // 16-byte chunks per lane group
    static constexpr int NQ = R / 128;                  // chunks per lane group
    // first rank of the 8 codes that lane group g feeds K step kk
    __host__ __device__ static constexpr int rank0(int kk, int g) {
        return CHUNK ? 32 * (g + 4 * (kk >> 2)) + 8 * (kk & 3) : 32 * kk + 8 * g;
    }
};

template <int R, int NH, bool INT4>
__global__ __launch_bounds__(256, 2) void absorbed_decode(const AbsorbArgs p) {
    constexpr int KS = R / 32;
    constexpr int VM = R / 16;
    constexpr int NG = R / 32;
    using KM = KeyMap<R>;
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

    // B fragments of the absorbed queries: head hn = l%16, the 8 ranks lane group
    // g feeds K step kk, scaled by qscale * 2^e per head (max |q'| in [2^14, 2^15)).
    const int hn = l & 15, g = l >> 4;
    half8 qf[KS];
    float inv = 1.0f;
    {
        float qv[KS][8];
        float mx = 0.0f;
        const float* qrow = p.q + ((long)b * Hq + j0 + (hn < NH ? hn : NH - 1)) * R;
        const float qs = hn < NH ? p.qscale : 0.0f;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const int r0 = INT4 ? KM::rank0(kk, g) : 32 * kk + 8 * g;
            const float4 x0 = *reinterpret_cast<const float4*>(qrow + r0);
            const float4 x1 = *reinterpret_cast<const float4*>(qrow + r0 + 4);
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qv[kk][e] = xs[INT4 ? code_pos_inv(e) : e] * qs;
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
    const uint32_t magic = 0x64006400u;
    // token of row hn of score M-tile mt
    const int trow = 8 * (hn >> 2) + (hn & 3);

    const int n_tiles = (t_end - t_begin + 31) / 32;
    // Tile data in registers, single-buffered but software-pipelined: the next
    // tile's key loads are issued as soon as this tile's score MFMAs have read
    // the key registers, its value loads once the value MFMAs have read theirs,
    // so each load's round trip overlaps the rest of the tile before it.
    half8 ka[2][KS], va[VM];
    uint32_t kw[2][KS], vc[VM];
    uint32_t ksc[2][KS];
    half8 vs[NG];
    // key rows (clamped to the last valid token; their scores are masked)
    auto load_keys = [&](int tile) __attribute__((always_inline)) {
        const int t0 = t_begin + 32 * tile;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const long row = bu * p.cap + min(t0 + trow + 4 * mt, t_end - 1);
            if constexpr (!INT4) {
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
                    ka[mt][kk] = *reinterpret_cast<const half8*>((const half_t*)p.hk + row * R + 32 * kk + 8 * g);
            } else if constexpr (KM::CHUNK) {
                const uint8_t* kr = (const uint8_t*)p.hk + row * (R / 2);
                const uint16_t* sr = reinterpret_cast<const uint16_t*>(p.sk) + row * (R / 32);
#pragma unroll
                for (int q = 0; q < KM::NQ; ++q) {
                    const uint4 c4 = *reinterpret_cast<const uint4*>(kr + 16 * (g + 4 * q));
                    kw[mt][4 * q + 0] = c4.x;
                    kw[mt][4 * q + 1] = c4.y;
                    kw[mt][4 * q + 2] = c4.z;
                    kw[mt][4 * q + 3] = c4.w;
                    const uint32_t sc = sr[g + 4 * q];
#pragma unroll
                    for (int wd = 0; wd < 4; ++wd) ksc[mt][4 * q + wd] = sc;
                }
            } else {
                const uint16_t* sr = reinterpret_cast<const uint16_t*>(p.sk) + row * (R / 32);
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    kw[mt][kk] = *reinterpret_cast<const uint32_t*>((const uint8_t*)p.hk + row * (R / 2) + 16 * kk + 4 * g);
                    ksc[mt][kk] = sr[kk];
                }
            }
        }
    };
    // value dims 16 v + hn at tokens 8 g .. 8 g + 7 (and int4 value scales)
    auto load_values = [&](int tile) __attribute__((always_inline)) {
        const long blk_base = bu * (p.cap / kTile) + (t_begin + 32 * tile) / kTile;
#pragma unroll
        for (int v = 0; v < VM; ++v) {
            const int dim = 16 * v + hn;
            if constexpr (!INT4)
                va[v] = *reinterpret_cast<const half8*>((const half_t*)p.hv + (blk_base * R + dim) * kTile + 8 * g);
            else
                vc[v] = *reinterpret_cast<const uint32_t*>((const uint8_t*)p.hv + (blk_base * R + dim) * (kTile / 2) + 4 * g);
        }
        if constexpr (INT4) {
#pragma unroll
            for (int gr = 0; gr < NG; ++gr)
                vs[gr] = *reinterpret_cast<const half8*>(p.sv + (blk_base * NG + gr) * kTile + 8 * g);
        }
    };
    // fp16 tiles at rank 256 fill the registers already: loaded at the top of
    // their own iteration instead
    constexpr bool PIPE = INT4 || R < 256;
    if (PIPE && w < n_tiles) {
        load_keys(w);
        load_values(w);
    }
    for (int it = w; it < n_tiles; it += 4) {
        const int t0 = t_begin + 32 * it;
        const bool tail = t0 + 32 > t_end;
        const bool next = PIPE && it + 4 < n_tiles;
        if (!PIPE) {
            load_keys(it);
            load_values(it);
        }
        // scores: lane holds head hn at tokens 8 g + 4 mt + e
        floatx4 sc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                half8 a;
                if constexpr (!INT4) a = ka[mt][kk];
                else a = dequant_keys(kw[mt][kk], ksc[mt][kk], magic);
                sc[mt] = mfma16(a, qf[kk], sc[mt]);
            }
        }
        if (next) load_keys(it + 4);
        float s8[8];
        float mt_loc = -INFINITY;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float v = t0 + 8 * g + k < t_end ? sc[k >> 2][k & 3] * inv : -INFINITY;
            s8[k] = v;
            mt_loc = fmaxf(mt_loc, v);
        }
        mt_loc = fmaxf(mt_loc, __shfl_xor(mt_loc, 16, kWave));
        mt_loc = fmaxf(mt_loc, __shfl_xor(mt_loc, 32, kWave));
        const float mn = fmaxf(m_run, mt_loc);
        // the accumulators are rescaled only when some head's running max moved
        const bool moved = __builtin_amdgcn_ballot_w64(mn > m_run) != 0;
        const float alpha = moved ? exp2f(m_run - mn) : 1.0f;
        float pr[8];
        float psum = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            pr[k] = hn < NH ? exp2f(s8[k] - mn) : 0.0f;
            psum += pr[k];
        }
        psum += __shfl_xor(psum, 16, kWave);
        psum += __shfl_xor(psum, 32, kWave);
        l_run = fmaf(l_run, alpha, psum);
        m_run = mn;
        if (moved) {
#pragma unroll
            for (int v = 0; v < VM; ++v) acc[v] *= alpha;
        }
        if constexpr (!INT4) {
            half8 pf;
#pragma unroll
            for (int k = 0; k < 8; ++k) pf[k] = (half_t)pr[k];
            if (tail) {
                // tokens past t_end: zero (their p is zero; the memory may hold anything)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (t0 + 8 * g + k >= t_end) {
#pragma unroll
                        for (int v = 0; v < VM; ++v) va[v][k] = (half_t)0.0f;
                    }
            }
#pragma unroll
            for (int v = 0; v < VM; ++v) acc[v] = mfma16(va[v], pf, acc[v]);
            if (next) load_values(it + 4);
        } else {
            // p in the code order (tokens 0, 4, 1, 5, 2, 6, 3, 7 of the group) times the
            // token's value scale of each 32-dim group; past t_end both are zeroed
            // (the scale there may hold anything)
            half2_t pk[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) pk[i] = pack2(pr[i], pr[4 + i]);
#pragma unroll
            for (int gr = 0; gr < NG; ++gr) {
                const uint4 sw = __builtin_bit_cast(uint4, vs[gr]);
                half2_t sp[4] = {__builtin_bit_cast(half2_t, __builtin_amdgcn_perm(sw.z, sw.x, 0x05040100u)),
                                 __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(sw.z, sw.x, 0x07060302u)),
                                 __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(sw.w, sw.y, 0x05040100u)),
                                 __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(sw.w, sw.y, 0x07060302u))};
                half2_t pp[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) pp[i] = pk[i] * sp[i];
                if (tail) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (t0 + 8 * g + i >= t_end) pp[i].x = (half_t)0.0f;
                        if (t0 + 8 * g + 4 + i >= t_end) pp[i].y = (half_t)0.0f;
                    }
                }
                const half8 pf = as_half8(pp);
#pragma unroll
                for (int v = 2 * gr; v < 2 * gr + 2; ++v) acc[v] = mfma16(value_codes(vc[v], magic), pf, acc[v]);
            }
            if (next) load_values(it + 4);
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
