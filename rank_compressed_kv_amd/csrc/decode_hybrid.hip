// Hybrid paged decode attention (PuzzleKV section 3.3, step 4).
//
// Pages of one (sequence, KV head) are dense (sink page, local window) or
// factored (X_hat = L R, Eq. 2). A factored page is evaluated from its factors
// without forming X_hat: scores s = (q R_K^T) L_K^T / sqrt(d), values
// (a L_V) R_V (the value side follows by associativity; the page's text stops
// after the key-side formula). All partial results are merged by online softmax.
//
// One wave streams the pages of one (page range, KV head, sequence); the
// range's chunk states are merged by merge_splits. Every product of a page is a
// 16x16 MFMA whose output fragment is already the next product's operand
// (lane l: column c = l % 16 = query head, lane group g = l / 16):
//   U^T [rank][head]  = R_K Q^T          16x16x32, A = R_K rows (rank c), K = 128 dims
//   S   [tok][head]   = L_K U^T          16x16x16, A = L_K rows (token c), K = ranks
//   online softmax: lane (c, g) holds head c at tokens 16 tb + 4 g + i
//   W^T [rank][head]  = L_V^T P^T        16x16x16, A = L_V^T rows (rank c), K = tokens
//   O^T [dim][head]  += R_V^T W^T        16x16x16, A = R_V^T rows (dim c), K = ranks
// so the value-side factors are stored dimension-major (L_V^T [r][P],
// R_V^T [d][r]), as are dense values (V^T [d][P]): every operand is a
// contiguous run of the contraction index. Heads c >= G are zero columns.
// Query and u = q R_K^T enter the MFMA as fp16 hi + lo pairs (u's magnitude
// grows with the factor scale; one fp16 rounding of it would cost ~1e-3 of the
// output), p and w once rounded to fp16. With int4 factors the key-side factors
// (R_K, L_K) also enter as exact hi + lo pairs of code x scale, since a rounded
// key factor moves the scores; the value-side factors are rounded once.
//
// Factored pages stream through three register buffers (two pages in flight
// while one is computed); dense pages (sink and window, a handful per
// sequence) follow them through two buffers (the next one's loads issued
// before the current one is computed) in the registers the factored pages
// have freed.
#include "tiles.h"

#include <math.h>

namespace lrkv {
namespace {

__device__ __forceinline__ floatx4 mfma16k16(half4 a, half4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rs(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// Offsets at or past the resource size read as zero: `kOff` marks a masked lane.
constexpr uint32_t kOff = 0x80000000u;
__device__ __forceinline__ half8 ld8(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ half4 ld4(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(half4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint4 ldw4(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t ldh(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// Four int4 codes (16 bits: code i at bits 4 i) times their fp16 scale, in the
// order 0, 2, 1, 3: the two bytes are spread to the two 16-bit halves, and the
// low / high nibbles masked into the mantissa of 1024.0 (exact integers).
__device__ __forceinline__ half4 decode4(uint32_t w16, uint32_t scale_bits) {
    const uint32_t x = (w16 ^ 0x8888u), y = __builtin_amdgcn_perm(0u, x, 0x0C010C00u);
    const uint32_t magic = 0x64006400u;
    const half2_t lo_off = {-1032.0f16, -1032.0f16};
    const half2_t hi_mul = {0.0625f16, 0.0625f16}, hi_off = {-72.0f16, -72.0f16};
    const half2_t s2 = __builtin_bit_cast(half2_t, scale_bits * 0x00010001u);
    const half2_t a = (__builtin_bit_cast(half2_t, and_or(y, 0x000F000Fu, magic)) + lo_off) * s2;
    const half2_t b = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, and_or(y, 0x00F000F0u, magic)), hi_mul, hi_off) * s2;
    return half4{a[0], a[1], b[0], b[1]};
}
// the order decode4 yields: element e is code pi4(e)
__host__ __device__ constexpr int pi4(int e) { return e == 1 ? 2 : e == 2 ? 1 : e; }

// Key-side factors as exact fp16 pairs: code x scale has at most 14 significant
// bits, so hi = fp16(code x scale) and lo = fma(code, scale, -hi) (one rounding of
// an exactly representable residual) give hi + lo = code x scale.
__device__ __forceinline__ void decode4_hl(uint32_t w16, uint32_t scale_bits, half4& hi, half4& lo) {
    const uint32_t x = (w16 ^ 0x8888u), y = __builtin_amdgcn_perm(0u, x, 0x0C010C00u);
    const uint32_t magic = 0x64006400u;
    const half2_t lo_off = {-1032.0f16, -1032.0f16};
    const half2_t hi_mul = {0.0625f16, 0.0625f16}, hi_off = {-72.0f16, -72.0f16};
    const half2_t s2 = __builtin_bit_cast(half2_t, scale_bits * 0x00010001u);
    const half2_t ca = __builtin_bit_cast(half2_t, and_or(y, 0x000F000Fu, magic)) + lo_off;
    const half2_t cb = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, and_or(y, 0x00F000F0u, magic)), hi_mul, hi_off);
    const half2_t ha = ca * s2, hb = cb * s2;
    const half2_t la = __builtin_elementwise_fma(ca, s2, -ha), lb = __builtin_elementwise_fma(cb, s2, -hb);
    hi = half4{ha[0], ha[1], hb[0], hb[1]};
    lo = half4{la[0], la[1], lb[0], lb[1]};
}
__device__ __forceinline__ void dequant_keys_hl(uint32_t w, uint32_t sc, uint32_t magic, half8& hi, half8& lo) {
    half2_t r[4], h[4], e[4];
    unpack_codes(w, magic, r);
    const half2_t s2 = __builtin_bit_cast(half2_t, sc * 0x00010001u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h[j] = r[j] * s2;
        e[j] = __builtin_elementwise_fma(r[j], s2, -h[j]);
    }
    hi = as_half8(h);
    lo = as_half8(e);
}

// max / sum over the four lane groups (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float xg_max(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
    v = fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
    r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
    return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float xg_sum(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
    v = __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
    r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
    return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

__device__ __forceinline__ half4 to_half4(floatx4 v) {
    return half4{(half_t)v[0], (half_t)v[1], (half_t)v[2], (half_t)v[3]};
}
// v = hi + lo with hi = fp16(v), lo = fp16(v - hi)
__device__ __forceinline__ void split4(floatx4 v, half4& hi, half4& lo) {
    hi = to_half4(v);
    lo = half4{(half_t)(v[0] - (float)hi[0]), (half_t)(v[1] - (float)hi[1]),
               (half_t)(v[2] - (float)hi[2]), (half_t)(v[3] - (float)hi[3])};
}

struct HybridArgs {
    const half_t *dk, *dv, *lk, *rk, *lv, *rv;
    const half_t *lks, *rks, *lvs, *rvs;   // int4 factor scales
    const int32_t* table;
    const int32_t* lens;
    const float* q;       // [B][Hq][128]
    float* part;          // [B][Hq][n_split][128 + 2]
    int B, H, G, sink, window, rkk, rvv, max_pages, n_split, pps, n_waves;
    float qscale;         // sm_scale * log2(e)
};

// Operands of one factored page for this lane (NK / NV: 16-rank blocks of the
// key / value factors).
template <int NK, int NV>
struct FPage {
    half8 rk[NK][4];      // R_K[16 rb + c][32 s + 8 g + 0..7]
    half4 lk[2][NK];      // L_K[16 tb + c][16 rb + 4 g + 0..3]
    half4 lv[2][NV];      // L_V^T[16 rb + c][16 tb + 4 g + 0..3]
    half4 rv[8][NV];      // R_V^T[16 mb + c][16 rb + 4 g + 0..3]
};

// int4 factors (ranks <= 16): the codes of one page for this lane, and their scales.
// R_K: the 16 bytes of dims [32 g, 32 g + 32) of rank row c (K step s takes dims
// 32 g + 8 s + ...; one scale); L_K: ranks 4 g .. 4 g + 3 of tokens c and 16 + c;
// L_V^T: tokens 16 tb + 4 g .. + 3 of rank row c (one scale); R_V^T (rank quads):
// the 16 bytes of quad g at dims 8 c .. 8 c + 7 (dim block mb takes dim 8 c + mb;
// one scale).
struct FPage4 {
    uint4 rk;
    uint32_t rks;
    uint32_t lk[2], lks[2];
    uint32_t lv[2], lvs;
    uint4 rv;
    uint32_t rvs;
};
template <bool I4, int NK, int NV> struct PageOf { using T = FPage<NK, NV>; };
template <int NK, int NV> struct PageOf<true, NK, NV> { using T = FPage4; };

template <int NK, int NV, bool I4>
__global__ __launch_bounds__(256, NK + NV == 2 ? 2 : 1) void hybrid_decode(const HybridArgs a) {
    constexpr int D = 128, P = 32;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), l = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + w;
    if (gw >= a.n_waves) return;
    const int split = gw % a.n_split, bh = gw / a.n_split, h = bh % a.H, b = bh / a.H;
    const int c = l & 15, g = l >> 4;
    const int Hq = a.H * a.G;
    const int len = min(a.lens[b], a.max_pages * P);
    const int npg = (len + P - 1) / P;
    const int p_begin = split * a.pps;
    const int p_end = min(npg, p_begin + a.pps);
    const int nd = a.sink + a.window;

    // this range's page-table entries, one per lane; factored / dense masks
    const int my_pg = p_begin + l;
    int entry = LRKV_PAGE_EMPTY;
    if (my_pg < p_end) entry = a.table[(long)bh * a.max_pages + my_pg];
    const bool fac = my_pg < p_end && entry >= 0 && entry < a.max_pages;
    const bool den = my_pg < p_end && entry < 0 && entry != LRKV_PAGE_EMPTY && -1 - entry < nd;
    uint64_t fmask = __builtin_amdgcn_ballot_w64(fac);
    uint64_t dmask = __builtin_amdgcn_ballot_w64(den);

    // queries of the KV head's G query heads (zero columns past G), hi + lo
    half8 qh[4], ql[4];
    {
        const float* qs = a.q + ((long)b * Hq + h * a.G + (c < a.G ? c : 0)) * D;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // int4 factors: K step s, lane group g takes dims 32 g + 8 s + (the code
                // unpack order 0, 4, 1, 5, 2, 6, 3, 7)
                const int dim = I4 ? 32 * g + 8 * s + code_pos_inv(j) : 32 * s + 8 * g + j;
                const float v = c < a.G ? qs[dim] * a.qscale : 0.0f;
                qh[s][j] = (half_t)v;
                ql[s][j] = (half_t)(v - (float)qh[s][j]);
            }
    }

    const int rk = a.rkk, rv = a.rvv;
    const long bhp = (long)bh * a.max_pages;
    const rsrc_t rs_rk = make_rs(a.rk + bhp * rk * D, (uint32_t)(a.max_pages * rk * D * 2));
    const rsrc_t rs_lk = make_rs(a.lk + bhp * P * rk, (uint32_t)(a.max_pages * P * rk * 2));
    const rsrc_t rs_lv = make_rs(a.lv + bhp * P * rv, (uint32_t)(a.max_pages * P * rv * 2));
    const rsrc_t rs_rv = make_rs(a.rv + bhp * rv * D, (uint32_t)(a.max_pages * rv * D * 2));

    // int4 factors: codes and scales of this (sequence, KV head); page strides in bytes
    const uint32_t s_rk = rk * D / 2, s_lk = P * rk / 2, s_lv = P * rv / 2, s_rv = rv * D / 2;
    rsrc_t q_rk, q_lk, q_lv, q_rv, q_rks, q_lks, q_lvs, q_rvs;
    uint32_t p_rk = kOff, p_lk0 = kOff, p_lk1 = kOff, p_lv0 = kOff, p_lv1 = kOff, p_rv = kOff;
    uint32_t p_rks = kOff, p_lks0 = kOff, p_lks1 = kOff, p_lvs = kOff, p_rvs = kOff;
    if constexpr (I4) {
        const uint32_t mp = (uint32_t)a.max_pages;
        q_rk = make_rs((const uint8_t*)a.rk + bhp * s_rk, mp * s_rk);
        q_lk = make_rs((const uint8_t*)a.lk + bhp * s_lk, mp * s_lk);
        q_lv = make_rs((const uint8_t*)a.lv + bhp * s_lv, mp * s_lv);
        q_rv = make_rs((const uint8_t*)a.rv + bhp * s_rv, mp * s_rv);
        q_rks = make_rs(a.rks + bhp * (s_rk / 16), mp * (s_rk / 8));
        q_lks = make_rs(a.lks + bhp * (s_lk / 16), mp * (s_lk / 8));
        q_lvs = make_rs(a.lvs + bhp * (s_lv / 16), mp * (s_lv / 8));
        q_rvs = make_rs(a.rvs + bhp * (s_rv / 16), mp * (s_rv / 8));
        // one scale per 32 stored elements (16 code bytes): scale byte = code byte / 8
        if (c < rk) {
            p_rk = c * 64 + 16 * g;                      // R_K[c][32 g .. 32 g + 31]
            p_rks = p_rk / 8;
        }
        if (4 * g < rk) {
            p_lk0 = (c * rk + 4 * g) / 2;                // L_K[c][4 g .. 4 g + 3]
            p_lk1 = ((16 + c) * rk + 4 * g) / 2;         // L_K[16 + c][4 g .. 4 g + 3]
            p_lks0 = p_lk0 / 16 * 2;
            p_lks1 = p_lk1 / 16 * 2;
        }
        if (c < rv) {
            p_lv0 = 16 * c + 2 * g;                      // L_V^T[c][4 g .. 4 g + 3]
            p_lv1 = 16 * c + 8 + 2 * g;                  // L_V^T[c][16 + 4 g .. 16 + 4 g + 3]
            p_lvs = 2 * c;
        }
        if (4 * g < rv) {
            p_rv = 256 * g + 16 * c;                     // quad g, dims 8 c .. 8 c + 7
            p_rvs = p_rv / 8;
        }
    }

    // per-lane offsets inside a page (kOff: masked lane), added to the page base
    uint32_t o_rk[NK], o_lk[NK], o_lv[NV], o_rv[NV];
#pragma unroll
    for (int rb = 0; rb < NK; ++rb) {
        o_rk[rb] = 16 * rb + c < rk ? ((16 * rb + c) * D + 8 * g) * 2 : kOff;
        o_lk[rb] = 16 * rb + 4 * g < rk ? (c * rk + 16 * rb + 4 * g) * 2 : kOff;
    }
#pragma unroll
    for (int rb = 0; rb < NV; ++rb) {
        o_lv[rb] = 16 * rb + c < rv ? ((16 * rb + c) * P + 4 * g) * 2 : kOff;
        o_rv[rb] = 16 * rb + 4 * g < rv ? (c * rv + 16 * rb + 4 * g) * 2 : kOff;
    }

    // Loads of the next factored page (its bit leaves `mask`); with none left,
    // every load reads past the buffers (zeros), so the load count per page is
    // fixed.
    using Page = typename PageOf<I4, NK, NV>::T;
    auto fetch = [&](Page& f, uint64_t& mask) __attribute__((always_inline)) {
        uint32_t slot = 0, none = kOff;
        if (mask) {
            const int bit = __builtin_ctzll(mask);
            mask &= mask - 1;
            slot = (uint32_t)__builtin_amdgcn_readlane(entry, bit);
            none = 0;
        }
        if constexpr (I4) {
            f.rk = ldw4(q_rk, none | (slot * s_rk + p_rk));
            f.rks = ldh(q_rks, none | (slot * (s_rk / 8) + p_rks));
            f.lk[0] = ldh(q_lk, none | (slot * s_lk + p_lk0));
            f.lk[1] = ldh(q_lk, none | (slot * s_lk + p_lk1));
            f.lks[0] = ldh(q_lks, none | (slot * (s_lk / 8) + p_lks0));
            f.lks[1] = ldh(q_lks, none | (slot * (s_lk / 8) + p_lks1));
            f.lv[0] = ldh(q_lv, none | (slot * s_lv + p_lv0));
            f.lv[1] = ldh(q_lv, none | (slot * s_lv + p_lv1));
            f.lvs = ldh(q_lvs, none | (slot * (s_lv / 8) + p_lvs));
            f.rv = ldw4(q_rv, none | (slot * s_rv + p_rv));
            f.rvs = ldh(q_rvs, none | (slot * (s_rv / 8) + p_rvs));
        } else {
#pragma unroll
        for (int rb = 0; rb < NK; ++rb) {
            const uint32_t base = none | (slot * rk * D * 2);
#pragma unroll
            for (int s = 0; s < 4; ++s) f.rk[rb][s] = ld8(rs_rk, (base + o_rk[rb] + 64 * s) | (o_rk[rb] & kOff));
            const uint32_t lbase = none | (slot * P * rk * 2);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) f.lk[tb][rb] = ld4(rs_lk, (lbase + o_lk[rb] + 32 * rk * tb) | (o_lk[rb] & kOff));
        }
#pragma unroll
        for (int rb = 0; rb < NV; ++rb) {
            const uint32_t lbase = none | (slot * P * rv * 2);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) f.lv[tb][rb] = ld4(rs_lv, (lbase + o_lv[rb] + 32 * tb) | (o_lv[rb] & kOff));
            const uint32_t base = none | (slot * rv * D * 2);
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) f.rv[mb][rb] = ld4(rs_rv, (base + o_rv[rb] + 32 * rv * mb) | (o_rv[rb] & kOff));
        }
        }
    };

    float m_run = -INFINITY, l_lane = 0.0f;
    floatx4 o[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) o[mb] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Online softmax of one page's scores (lane: head c, tokens 16 tb + 4 g + i;
    // tokens >= ntok masked); returns p as the next MFMA's B operand.
    // perm: pack p in the order pi4 (the token order of int4 L_V^T fragments)
    auto softmax = [&](const floatx4* S, int ntok, half4* pb, bool perm) __attribute__((always_inline)) {
        float sv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) sv[k] = S[k >> 2][k & 3];
        if (ntok < P) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (16 * (k >> 2) + 4 * g + (k & 3) >= ntok) sv[k] = -INFINITY;
        }
        float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
        mx = xg_max(mx);
        const float mn = fmaxf(m_run, mx);
        // rescale only when some head's running max moved (rare after the first pages)
        if (__builtin_amdgcn_ballot_w64(mn > m_run)) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
            l_lane *= alpha;
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) o[mb] *= alpha;
        }
        m_run = mn;
        float pr[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) pr[k] = __builtin_amdgcn_exp2f(sv[k] - mn);
        l_lane += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) pb[tb][i] = (half_t)pr[4 * tb + (perm ? pi4(i) : i)];
    };

    auto factored4 = [&](const FPage4& f, int ntok) __attribute__((always_inline)) {
        const uint32_t magic = 0x64006400u;
        const uint32_t rw[4] = {f.rk.x, f.rk.y, f.rk.z, f.rk.w};
        // u = (R_K hi + lo)(q hi + lo) without the lo x lo term
        floatx4 u = floatx4{0.f, 0.f, 0.f, 0.f}, u2 = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            half8 akh, akl;
            dequant_keys_hl(rw[s], f.rks, magic, akh, akl);
            u = mfma16(akh, qh[s], u);
            u2 = mfma16(akh, ql[s], u2);
            u2 = mfma16(akl, qh[s], u2);
        }
        u += u2;
        // lane (c, g) holds U^T[4 g + i][c]; L_K fragments decode in rank order pi4
        half4 uh, ul;
        split4(floatx4{u[0], u[2], u[1], u[3]}, uh, ul);
        floatx4 S[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            half4 lkh, lkl;
            decode4_hl(f.lk[tb], f.lks[tb], lkh, lkl);
            S[tb] = mfma16k16(lkh, uh, floatx4{0.f, 0.f, 0.f, 0.f});
            S[tb] = mfma16k16(lkh, ul, S[tb]);
            S[tb] = mfma16k16(lkl, uh, S[tb]);
        }
        half4 pb[2];
        softmax(S, ntok, pb, true);
        floatx4 wt = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) wt = mfma16k16(decode4(f.lv[tb], f.lvs), pb[tb], wt);
        const half4 wb = half4{(half_t)wt[0], (half_t)wt[2], (half_t)wt[1], (half_t)wt[3]};
        const uint32_t vw[4] = {f.rv.x, f.rv.y, f.rv.z, f.rv.w};
        // dim block mb: A row c is dim 8 c + mb (the 16-bit half mb of the lane's run)
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) o[mb] = mfma16k16(decode4(vw[mb >> 1] >> (16 * (mb & 1)), f.rvs), wb, o[mb]);
    };

    auto factored = [&](const Page& f, int ntok) __attribute__((always_inline)) {
        if constexpr (I4) {
            factored4(f, ntok);
            return;
        } else {
        half4 uh[NK], ul[NK];
#pragma unroll
        for (int rb = 0; rb < NK; ++rb) {
            floatx4 u = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                u = mfma16(f.rk[rb][s], qh[s], u);
                u = mfma16(f.rk[rb][s], ql[s], u);
            }
            split4(u, uh[rb], ul[rb]);
        }
        floatx4 S[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            S[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int rb = 0; rb < NK; ++rb) {
                S[tb] = mfma16k16(f.lk[tb][rb], uh[rb], S[tb]);
                S[tb] = mfma16k16(f.lk[tb][rb], ul[rb], S[tb]);
            }
        }
        half4 pb[2];
        softmax(S, ntok, pb, false);
#pragma unroll
        for (int rb = 0; rb < NV; ++rb) {
            floatx4 wt = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) wt = mfma16k16(f.lv[tb][rb], pb[tb], wt);
            const half4 wb = to_half4(wt);
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) o[mb] = mfma16k16(f.rv[mb][rb], wb, o[mb]);
        }
        }
    };

    // ---- factored pages, three register buffers
    {
        uint64_t fetch_mask = fmask, run_mask = fmask;
        auto next_ntok = [&]() __attribute__((always_inline)) {
            const int bit = __builtin_ctzll(run_mask);
            run_mask &= run_mask - 1;
            return min(P, len - (p_begin + bit) * P);
        };
        Page f0, f1, f2;
        fetch(f0, fetch_mask);
        fetch(f1, fetch_mask);
        while (run_mask) {
            fetch(f2, fetch_mask);
            factored(f0, next_ntok());
            if (!run_mask) break;
            fetch(f0, fetch_mask);
            factored(f1, next_ntok());
            if (!run_mask) break;
            fetch(f1, fetch_mask);
            factored(f2, next_ntok());
        }
    }

    // ---- dense pages: K [P][d], V^T [d][P] in their slots
    struct DPage {
        half8 kf[2][4];
        half4 vf[8][2];
    };
    auto load_dense = [&](DPage& d, int slot) __attribute__((always_inline)) {
        const long sb = (long)bh * nd + slot;
        const rsrc_t rs_k = make_rs(a.dk + sb * P * D, P * D * 2);
        const rsrc_t rs_v = make_rs(a.dv + sb * P * D, P * D * 2);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if constexpr (I4) {
                    // the queries' dim order: K step s, group g, element j = dim 32 g + 8 s + code_pos_inv(j)
                    const half8 raw = ld8(rs_k, ((16 * tb + c) * D + 32 * g + 8 * s) * 2);
#pragma unroll
                    for (int j = 0; j < 8; ++j) d.kf[tb][s][j] = raw[code_pos_inv(j)];
                } else {
                    d.kf[tb][s] = ld8(rs_k, ((16 * tb + c) * D + 32 * s + 8 * g) * 2);
                }
            }
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                // A row c of dim block mb: dim 16 mb + c, or 8 c + mb with int4 factors
                const int dim = I4 ? 8 * c + mb : 16 * mb + c;
                d.vf[mb][tb] = ld4(rs_v, (dim * P + 16 * tb + 4 * g) * 2);
            }
    };
    auto dense = [&](DPage& d, int ntok) __attribute__((always_inline)) {
        floatx4 S[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            S[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                S[tb] = mfma16(d.kf[tb][s], qh[s], S[tb]);
                S[tb] = mfma16(d.kf[tb][s], ql[s], S[tb]);
            }
        }
        half4 pb[2];
        softmax(S, ntok, pb, false);
        if (ntok < P) {
            // rows past the page's last token may hold anything; their p is zero
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (16 * tb + 4 * g + i >= ntok) d.vf[mb][tb][i] = (half_t)0.0f;
        }
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) o[mb] = mfma16k16(d.vf[mb][tb], pb[tb], o[mb]);
    };

    // this range's dense pages, two buffers (dmask is wave-uniform)
    if (dmask) {
        DPage d0, d1;
        int b0 = 0, b1 = 0;
        auto take = [&](int& bit) __attribute__((always_inline)) -> int {
            bit = __builtin_ctzll(dmask);
            dmask &= dmask - 1;
            return -1 - __builtin_amdgcn_readlane(entry, bit);
        };
        load_dense(d0, take(b0));
        while (true) {
            const bool h1 = dmask != 0;
            if (h1) load_dense(d1, take(b1));
            dense(d0, min(P, len - (p_begin + b0) * P));
            if (!h1) break;
            const bool h0 = dmask != 0;
            if (h0) load_dense(d0, take(b0));
            dense(d1, min(P, len - (p_begin + b1) * P));
            if (!h0) break;
        }
    }

    // ---- chunk state of the G heads: (m, l, unnormalised o)
    const float l_sum = xg_sum(l_lane);
    if (c < a.G) {
        float* ph = a.part + ((long)(b * Hq + h * a.G + c) * a.n_split + split) * (D + 2);
        if (g == 0) {
            ph[0] = m_run;
            ph[1] = l_sum;
        }
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) ph[2 + (I4 ? 8 * (4 * g + i) + mb : 16 * mb + 4 * g + i)] = o[mb][i];
    }
}

template <int NK, int NV, bool I4 = false>
void launch_hybrid(const HybridArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((hybrid_decode<NK, NV, I4>), dim3((a.n_waves + 3) / 4), dim3(256), 0, st, a);
}

}  // namespace

void launch_merge(const float* part, float* out, int BH, int n_split, int D, hipStream_t st);

int32_t launch_decode_hybrid(int phases, const lrkv_paged_cache* c, const float* q, float sm_scale,
                             float* out, void* ws, const PagedWorkspace& w, hipStream_t st) {
    float* part = (float*)((char*)ws + w.part_off);
    HybridArgs a{(const half_t*)c->dense_k, (const half_t*)c->dense_v, (const half_t*)c->lk,
                 (const half_t*)c->rk, (const half_t*)c->lv, (const half_t*)c->rv, (const half_t*)c->lk_s,
                 (const half_t*)c->rk_s, (const half_t*)c->lv_s, (const half_t*)c->rv_s, c->page_table,
                 c->lens, q, part, c->batch, c->kv_heads, c->q_per_kv, c->sink_pages,
                 c->window_pages, c->rank_k, c->rank_v, c->max_pages, w.n_split,
                 w.pages_per_split, c->batch * c->kv_heads * w.n_split, sm_scale * kLog2e};
    if (phases & kPhasePartials) {
        const bool k2 = c->rank_k > 16, v2 = c->rank_v > 16;
        // int4 factors: ranks <= 16 (checked with the cache description)
        if (c->factor_fmt == LRKV_FMT_INT4_G32) launch_hybrid<1, 1, true>(a, st);
        else if (!k2 && !v2) launch_hybrid<1, 1>(a, st);
        else if (!k2) launch_hybrid<1, 2>(a, st);
        else if (!v2) launch_hybrid<2, 1>(a, st);
        else launch_hybrid<2, 2>(a, st);
    }
    if (phases & kPhaseMerge)
        launch_merge(part, out, c->batch * c->kv_heads * c->q_per_kv, w.n_split, c->head_dim, st);
    return last_launch_status();
}

}  // namespace lrkv
