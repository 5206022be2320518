// Reconstruct-then-rotate decode attention for grouped-query units (gfx950):
// one KV head per unit whose latent is shared by NH query heads (GQA).
//
// Palu digest, Method details: keys are cached as latents and rebuilt on chip
// as K = H^k B^k; RoPE is applied at each token's position before the query
// attends, and the output stays in latent space (o = p H^v). The int4 latents
// follow the same digest: the Hadamard rotation folded into the factors as
// (A R)(R^T B) (Method details) and per-token groups of 32 elements with one
// scale each (Supplementary details); the symmetric [-7, 7] code range is the
// Shard post's (section 5, step 4), whose step 1 states the rotate-half RoPE.
//
// With several query heads per KV head, rebuilding K once per tile costs
// 2 r d_h FLOP per token, against 2 r d_h NH for scoring in a per-head rotated
// basis, so this kernel reconstructs K explicitly and rotates it:
//   score_h(t) = q_h^T R((t - q_pos) theta) K(t)
//              = (R(t0 - q_pos)^T q_h)^T (R(tau) K(t)),  t = t0 + tau, t0 = tile start,
// with R(tau) (tau < 32) a constant per-lane table and the per-tile rotation of
// the NH queries done once per tile by the whole wave (one frequency per lane)
// and passed to the score MFMA through LDS.
//
// Each wave streams one sequence chunk of one (sequence, unit) on its own and
// writes the chunk's (running max, running sum, unnormalised output) per head;
// merge.hip combines the chunks. Per 32-token tile (lane l: column c = l % 16,
// lane group g = l / 16; two 16-token N-blocks):
//   reconstruction  D[dim][tok] = B^k^T H^T   16x16x32 MFMA, A = B^k fragments held
//                   in registers for the whole chunk (prepared in fragment order),
//                   B = the lane's latents of token c: ranks [r/4 g, r/4 (g+1));
//   rotation        dims f and f + 64 sit in M-tiles mt and mt + 4 of the same
//                   lane, rotated as an fp16 pair by R(tau) (two packed ops);
//   scores          D2[tok][head] = K_rot Q~^T   16x16x32 MFMA (heads padded to 16);
//   softmax         lane (c, g) holds head c at tokens 4 g + i of both N-blocks:
//                   max and sum over the tile are 8 in-lane values plus two
//                   cross-row exchanges; log2 domain (queries carry log2 e);
//   values          D3[dim][head] += V^T P', P' = p x (the token's value scale of
//                   the M-tile's 32-dim group), transposed through LDS.
// int4 codes (two's complement nibbles) become fp16 with the offset-1024
// exponent trick: exact integers, then x scale (keys) rounded once to fp16.
// int4 super-tiles: with 4 query heads and 16 score columns, four consecutive
// tiles share one score accumulator, tile j in columns 4j..4j+3 (its queries are
// zero elsewhere); softmax and value scaling then run once per four tiles, and a
// tile's value product follows four tiles after its scores, with p passed by its
// own column group only. Each head's output is the sum of its four columns.
#include "tiles.h"

#include <math.h>

namespace lrkv {

struct GqaArgs {
    const void* hk;
    const void* hv;
    const half_t* sk;
    const half_t* sv;
    const int32_t* lens;
    const float* q;        // [B][Hq][128] un-rotated queries x sm_scale x log2(e), fp32
    const half_t* bfrag;   // [U][8][R/32][64][8] B^k in A-fragment order
    AngleTables ang;
    float* part;           // [B][Hq][n_split][R + 2]
    int B, U, cap, n_split, chunk, n_waves;
    int pending;           // tokens appended in this step whose lens update is still to come
};

namespace {

// (c ka - s kb, s ka + c kb) for kp = (ka, kb), cs = (c, s): a product with the
// swapped pair and (-s, s), then one fused multiply-add with (c, c).
__device__ __forceinline__ half2_t rot_pair(half2_t kp, half2_t cs) {
    half2_t t, r;
    asm("v_pk_mul_f16 %0, %1, %2 op_sel:[1,1] op_sel_hi:[0,1] neg_lo:[0,1]" : "=v"(t) : "v"(kp), "v"(cs));
    asm("v_pk_fma_f16 %0, %1, %2, %3 op_sel_hi:[1,0,1]" : "=v"(r) : "v"(kp), "v"(cs), "v"(t));
    return r;
}

// Position of token o (0..7) of an 8-token group in the order above.
__host__ __device__ constexpr int code_pos(int o) { return o < 4 ? 2 * o : 2 * (o - 4) + 1; }

// max / sum over the four lane groups (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float xrow_max(float v) {
    v = rowpair(v, true);
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
    return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float xrow_sum(float v) {
    v = rowpair(v, false);
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
    return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

// Orders this wave's LDS writes before its later LDS reads by other lanes (LDS
// executes one wave's operations in order; this stops compiler reordering).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// buf_dma16 for the lanes of `mask` only, with EXEC narrowed and restored
// inside the statement (no branch for the compiler; the caller is in uniform
// control flow).
__device__ __forceinline__ void buf_dma16_lanes(int32x4 rsrc, uint32_t voff, const void* lds, uint64_t mask) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    uint64_t save;
    // M0 (the LDS base) is an input bound to that register; the s_nop separates
    // the compiler's write of it from the load
    asm volatile("s_mov_b64 %0, exec\n\ts_and_b64 exec, exec, %4\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %1, %2, 0 offen lds\n\ts_mov_b64 exec, %0"
                 : "=&s"(save)
                 : "v"(voff), "s"(rsrc), "{m0}"(m), "s"(mask)
                 : "memory");
}

// v_permlane32_swap: upper 32 lanes of a <-> lower 32 lanes of b.
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
// v_permlane16_swap: odd 16-lane rows of a <-> even rows of b.
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
// p' of head c at tokens 16 nb + 4 g + (0..3), as packed fp16 pairs: x{nb}0 =
// tokens +0, +1 and x{nb}1 = tokens +2, +3. Returns head c's tokens 8 g + (0..7)
// (the value MFMA's B operand), in token order or in the int4 unpack order
// (0, 4, 1, 5, 2, 6, 3, 7). Row g needs N-block g / 2 of rows 2 (g % 2) and
// 2 (g % 2) + 1: a 32-lane swap between the N-blocks, then a 16-lane swap.
template <bool CODE_ORDER>
__device__ __forceinline__ half8 p_operand(uint32_t x00, uint32_t x01, uint32_t x10, uint32_t x11) {
    swap32(x00, x10);
    swap32(x01, x11);
    swap16(x00, x10);
    swap16(x01, x11);
    // row g: x00, x01 = tokens 8g + (0, 1), (2, 3); x10, x11 = tokens 8g + (4, 5), (6, 7)
    if constexpr (CODE_ORDER)
        return __builtin_bit_cast(half8, uint4{__builtin_amdgcn_perm(x10, x00, 0x05040100u),
                                               __builtin_amdgcn_perm(x10, x00, 0x07060302u),
                                               __builtin_amdgcn_perm(x11, x01, 0x05040100u),
                                               __builtin_amdgcn_perm(x11, x01, 0x07060302u)});
    else
        return __builtin_bit_cast(half8, uint4{x00, x01, x10, x11});
}

// One tile's raw data for this lane.
template <int R, bool INT4>
struct GqaTile;

// int4 tiles stream into LDS with direct buffer loads (no registers), several
// tiles ahead, into two rings: a key slot holds key codes [32 tok][R/2] | key
// scales [32 tok][R/32]; a value slot value codes [R dims][16] | value scales
// [R/32][32 tok]. At rank 64 a token's two 16-byte code chunks swap places in
// rows t with bit 2 of t set (the load picks its source chunk accordingly), so
// that the 16 rows one key read touches spread over all banks. Key slots are free once the tile is scored, value slots only
// after its value product, which runs a few tiles later.
template <int R>
struct GqaTile<R, true> {
    static constexpr int KS = R / 32, VM = R / 16, NG = R / 32;
    static constexpr int KB = 32 * R / 2, VB = R * 16, SB = 32 * NG * 2;
    static constexpr int KSLOT = KB + SB, VSLOT = VB + SB;
    uint32_t kc[2][KS];      // key codes of token 16 nb + c, ranks [R/4 g, R/4 (g+1))
    uint32_t ks0, ks1;       // key scale of those ranks (fp16 bits), N-blocks 0 and 1

    // Issue the loads of cache block `blk` of the unit (4 loads; a negative blk
    // reads past every buffer's end, i.e. zeros, so that every tile issues the
    // same number of loads).
    __device__ __forceinline__ static void issue(const int32x4* rs, int blk, const uint8_t* kslot,
                                                 const uint8_t* vslot, int l) {
        const uint32_t bad = 0x80000000u;
        const bool ok = blk >= 0;
        constexpr uint64_t all = ~0ull, ks_lanes = (1ull << (SB / 16)) - 1;
        buf_dma16_lanes(rs[0], ok ? (uint32_t)blk * KB + 16 * (KS == 2 ? l ^ ((l >> 3) & 1) : l) : bad, kslot,
                        KB / 16 >= 64 ? all : (1ull << (KB / 16)) - 1);
        buf_dma16_lanes(rs[1], ok ? (uint32_t)blk * VB + 16 * l : bad, vslot,
                        VB / 16 >= 64 ? all : (1ull << (VB / 16)) - 1);
        buf_dma16_lanes(rs[2], ok ? (uint32_t)blk * SB + 16 * l : bad, kslot + KB, ks_lanes);
        buf_dma16_lanes(rs[3], ok ? (uint32_t)blk * SB + 16 * l : bad, vslot + VB, ks_lanes);
    }
    // `valid`: tokens of the tile before the chunk's end. The key scales of the
    // others are zeroed (an unwritten scale may hold anything, and these keys
    // meet zero queries in other tiles' score columns, where inf x 0 would spread).
    __device__ __forceinline__ void read_keys(const uint8_t* kslot, int c, int g, int valid) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int t = 16 * nb + c;
            const uint8_t* src = KS == 2 ? kslot + 16 * (2 * t + ((g >> 1) ^ ((t >> 2) & 1))) + 8 * (g & 1)
                                         : kslot + t * (R / 2) + (R / 8) * g;
            if constexpr (KS == 2) {
                const uint2 v = *reinterpret_cast<const uint2*>(src);
                kc[nb][0] = v.x;
                kc[nb][1] = v.y;
            } else {
                kc[nb][0] = *reinterpret_cast<const uint32_t*>(src);
            }
        }
        const uint16_t* ksp = reinterpret_cast<const uint16_t*>(kslot + KB) + c * NG + (R / 4) * g / 32;
        // read unconditionally (the slot is always in the ring), then select: a
        // conditional LDS read compiles to a branch around a wait, which splits
        // the tile's instruction schedule
        const uint32_t r0 = ksp[0], r1 = ksp[16 * NG];
        ks0 = c < valid ? r0 : 0u;
        ks1 = 16 + c < valid ? r1 : 0u;
    }
    __device__ __forceinline__ half8 key_operand(int nb, int k, uint32_t magic) const {
        return dequant_keys(kc[nb][k], nb ? ks1 : ks0, magic);
    }
    // value codes of dim 16 mv + c, tokens 8g..8g+7
    __device__ __forceinline__ static uint32_t value_word(const uint8_t* vslot, int mv, int c, int g) {
        return *reinterpret_cast<const uint32_t*>(vslot + (16 * mv + c) * 16 + 4 * g);
    }
    // value scales (fp16) of tokens 16 nb + 4g + (0..3), 32-dim group gr
    __device__ __forceinline__ static uint2 value_scales(const uint8_t* vslot, int gr, int nb, int g) {
        return *reinterpret_cast<const uint2*>(vslot + VB + (gr * 32 + 16 * nb + 4 * g) * 2);
    }
};

template <int R>
struct GqaTile<R, false> {
    static constexpr int KS = R / 32, VM = R / 16, NG = 1;
    half8 kh[2][KS];         // key latents of token 16 nb + c, ranks R/4 g + 8 ks + (0..7)
    half8 vh[VM];            // value latents of dim 16 mv + c, tokens 8g..8g+7
    __device__ __forceinline__ void load(const GqaArgs& p, long bu, int t0, int c, int g) {
        const half_t* hk = (const half_t*)p.hk;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const half_t* src = hk + (bu * p.cap + t0 + 16 * nb + c) * R + (R / 4) * g;
#pragma unroll
            for (int k = 0; k < KS; ++k) kh[nb][k] = *reinterpret_cast<const half8*>(src + 8 * k);
        }
        const long blk = bu * (p.cap / kTile) + t0 / kTile;
        const half_t* hv = (const half_t*)p.hv;
#pragma unroll
        for (int mv = 0; mv < VM; ++mv)
            vh[mv] = *reinterpret_cast<const half8*>(hv + (blk * R + 16 * mv + c) * kTile + 8 * g);
    }
    __device__ __forceinline__ half8 key_operand(int nb, int k, uint32_t) const { return kh[nb][k]; }
    // tokens 8g..8g+7 in order
    __device__ __forceinline__ half8 value_operand(int mv, uint32_t) const { return vh[mv]; }
    __device__ __forceinline__ half2_t scale_pair(int, int, int, half2_t pp) const { return pp; }
};

template <bool B>
struct Flag {
    static constexpr bool value = B;
};

template <int R, int NH, bool INT4>
__global__ __launch_bounds__(256, 2) void rope_decode_gqa(const GqaArgs p) {
    constexpr int KS = R / 32;                 // reconstruction K steps (32 ranks each)
    constexpr int VM = R / 16;                 // value M-tiles
    constexpr int NG = INT4 ? R / 32 : 1;      // value scale groups
    static_assert(R == 32 || R == 64, "rank 32 or 64");
    static_assert(NH >= 1 && NH <= 16, "1..16 query heads per KV head");
    using Tile = GqaTile<R, INT4>;
    // int4 works in super-tiles of S = 16 / NH tiles whose NH heads fill the 16
    // score columns: column c = NH j + h is head h of the super-tile's tile j.
    constexpr int S = INT4 ? 16 / NH : 1;
    static_assert(!INT4 || NH == 4, "int4 super-tiles are laid out for 4 heads per KV head");
    // per wave, rotated queries, one u32 fp16 pair per (row, frequency): int4 one
    // buffer with row NH j + h for tile j of the super-tile, fp16 two buffers of
    // NH rows; then a zero row for the padding columns
    // rows 80 dwords apart, so that the distinct rows one read touches sit in
    // different banks
    constexpr int kQRows = NH * S + 1, kQBufs = INT4 ? 1 : 2, kZeroRow = NH * S, kQS = 80;
    __shared__ __attribute__((aligned(16))) uint32_t qt_s[4][kQBufs][kQRows * kQS];
    // int4: per-wave rings filled by direct loads kDepth tiles ahead; a tile's key
    // slot is free once it is scored, its value slot after its value product, S
    // tiles later (its value scales are read by the super-tile's softmax)
    constexpr int kDepth = 3, kKeySlots = kDepth + 1, kValSlots = kDepth + S + 1;
    constexpr int kKSlot = INT4 ? GqaTile<R, true>::KSLOT : 16, kVSlot = INT4 ? GqaTile<R, true>::VSLOT : 16;
    __shared__ __attribute__((aligned(16))) uint8_t kring_s[4][INT4 ? kKeySlots : 1][kKSlot];
    __shared__ __attribute__((aligned(16))) uint8_t vring_s[4][INT4 ? kValSlots : 1][kVSlot];

    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), l = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + w;
    if (gw >= p.n_waves) return;
    const int split = gw % p.n_split, bu = gw / p.n_split, u = bu % p.U, b = bu / p.U;
    const int len = min(p.lens[b] + p.pending, p.cap);
    const int t_begin = split * p.chunk, t_end = min(len, t_begin + p.chunk);
    const int Hq = p.U * NH, j0 = u * NH;
    float* part = p.part + ((long)(b * Hq + j0) * p.n_split + split) * (R + 2);
    const long hstride = (long)p.n_split * (R + 2);
    if (t_begin >= t_end) {
        for (int e = l; e < NH * (R + 2); e += 64) {
            const int h = e / (R + 2), col = e % (R + 2);
            part[h * hstride + col] = col == 0 ? -INFINITY : 0.0f;
        }
        return;
    }
    const int c = l & 15, g = l >> 4;
    const int hrow = c < NH ? c : NH;
#pragma unroll
    for (int qb = 0; qb < kQBufs; ++qb) qt_s[w][qb][kZeroRow * kQS + l] = 0u;
    const uint32_t magic = 0x64006400u;
    const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;
    const int t_last = t_begin + kTile * (n_tiles - 1);

    // int4: the first kDepth tiles start loading into the LDS ring before the
    // set-up loads. Every tile issues 4 loads (dummies past the chunk read
    // zeros), so before tile i is read, vmcnt(4 (kDepth - 1)) leaves exactly
    // tiles i+1..i+kDepth-1 in flight; the set-up loads are all waited for
    // before the loop, and no other vector-memory operation is issued in it.
    int32x4 rs[4];
    uint8_t* kring = &kring_s[w][0][0];
    uint8_t* vring = &vring_s[w][0][0];
    const int blk0 = t_begin / kTile;
    if constexpr (INT4) {
        const long nblk = p.cap / kTile;
        rs[0] = make_rsrc((const uint8_t*)p.hk + bu * nblk * Tile::KB, (uint32_t)(nblk * Tile::KB));
        rs[1] = make_rsrc((const uint8_t*)p.hv + bu * nblk * Tile::VB, (uint32_t)(nblk * Tile::VB));
        rs[2] = make_rsrc((const uint8_t*)p.sk + bu * nblk * Tile::SB, (uint32_t)(nblk * Tile::SB));
        rs[3] = make_rsrc((const uint8_t*)p.sv + bu * nblk * Tile::SB, (uint32_t)(nblk * Tile::SB));
#pragma unroll
        for (int i = 0; i < kDepth; ++i)
            Tile::issue(rs, i < n_tiles ? blk0 + i : -1, kring + i * kKSlot, vring + i * kVSlot, l);
    }

    // B^k fragments: A[dim 16 mt + c][ranks R/4 g + 8 ks + perm(0..7)]
    half8 af[8][KS];
    {
        const half8* bf = reinterpret_cast<const half8*>(p.bfrag) + (long)u * 8 * KS * 64 + l;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int k = 0; k < KS; ++k) af[mt][k] = bf[(mt * KS + k) * 64];
    }
    // R(tau) of the lane's (token 16 nb + c, frequency 16 mt + 4 g + i)
    half2_t rt[2][4][4];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float2 v = p.ang.tok[(16 * nb + c) * 64 + 16 * mt + 4 * g + i];
                rt[nb][mt][i] = pack2(v.x, v.y);
            }
    // queries of the unit (scaled), frequency l: (q[l], q[l + 64]), and the chunk's
    // start rotation (fp64-reduced) advanced by one tile per step
    float qa[NH], qb[NH];
    {
        const float* qs = p.q + ((long)b * Hq + j0) * 128;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            qa[h] = qs[h * 128 + l];
            qb[h] = qs[h * 128 + 64 + l];
        }
    }
    float2 ang = p.ang.start[((long)b * p.n_split + split) * 64 + l];
    const float2 stp = p.ang.step[l];
    // all set-up loads (and the ring's first tiles) complete; as a compiler
    // builtin the wait is known to the compiler's own wait-count tracking
    if constexpr (INT4) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

    float m_run = -INFINITY, l_run = 0.0f;
    floatx4 accv[VM];
#pragma unroll
    for (int mv = 0; mv < VM; ++mv) accv[mv] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Q~ = R(t0 - q_pos)^T q of the next tile for every head, (c qa + s qb,
    // c qb - s qa), into rows row0 .. row0 + NH - 1 of `qt`; the rotation then
    // advances a tile.
    auto rotate_queries = [&](uint32_t* qt, int row0) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const float ta = fmaf(ang.x, qa[h], ang.y * qb[h]);
            const float tb = fmaf(ang.x, qb[h], -ang.y * qa[h]);
            qt[(row0 + h) * kQS + l] = __builtin_bit_cast(uint32_t, pack2(ta, tb));
        }
        ang = cmul(ang, stp);
    };
    // Reconstruction, rotation by R(tau) and scores of one tile against query row
    // `row` of `qt` (the lane's column): sacc[nb][i] (+)= score of that row at token
    // 16 nb + 4 g + i. With `zero` the accumulators start from zero.
    auto scores = [&](const Tile& T, const uint32_t* qt, int row, floatx4* sacc, bool zero) __attribute__((always_inline)) {
        half8 bq[4];
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) bq[k2] = *reinterpret_cast<const half8*>(qt + row * kQS + 16 * k2 + 4 * g);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            floatx4 acc[8];
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const half8 hop = T.key_operand(nb, k, magic);
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) acc[mt] = mfma16(af[mt][k], hop, acc[mt]);
            }
            if (zero) sacc[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                half2_t a2[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) a2[i] = rot_pair(pack2(acc[mt][i], acc[mt + 4][i]), rt[nb][mt][i]);
                sacc[nb] = mfma16(as_half8(a2), bq[mt], sacc[nb]);
            }
        }
    };

    if constexpr (INT4) {
        // Sub-step i scores tile i (j = i % S of its super-tile) into the columns
        // of group j: the other columns read the zero query row, so they add
        // nothing. The value product of tile i - S runs in the same sub-step with
        // p' of its super-tile, whose softmax ran at the end of that super-tile.
        uint32_t* qt = qt_s[w][0];
        const int col_tile = c / NH;               // the lane's tile within a super-tile
        const int n_sub = (n_tiles + S - 1) / S * S;
        floatx4 sacc[2] = {};
        half8 bp[NG] = {};                         // p' (value B operand) of the lane's column
        // Online softmax over one super-tile (tiles ts..ts+S-1, starting at token
        // t0s): lane (c, g) holds head c % NH of tile c / NH at tokens 16 nb + 4 g + i.
        // p x the token's value scale becomes bp; the output is rescaled.
        auto softmax_super = [&](int ts) __attribute__((always_inline)) {
            const int tl = t_begin + kTile * (ts + col_tile);    // the lane's tile start
            float sv[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                sv[k] = sacc[k >> 2][k & 3];
                if (tl + 16 * (k >> 2) + 4 * g + (k & 3) >= t_end) sv[k] = -INFINITY;
            }
            float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
            mx = xrow_max(mx);
            mx = fmaxf(mx, dppf<0x124>(mx));       // row_ror:4 and :8, the head's other tiles
            mx = fmaxf(mx, dppf<0x128>(mx));
            const float mn = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
            float pr[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) pr[k] = __builtin_amdgcn_exp2f(sv[k] - mn);
            float ps = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
            ps = xrow_sum(ps);
            ps += dppf<0x124>(ps);
            ps += dppf<0x128>(ps);
            l_run = fmaf(l_run, alpha, ps);
            m_run = mn;
            const uint8_t* vsl = vring + ((ts + col_tile) % kValSlots) * kVSlot;
#pragma unroll
            for (int gr = 0; gr < NG; ++gr) {
                uint32_t x[2][2];
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const uint2 sc = Tile::value_scales(vsl, gr, nb, g);
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        half2_t q2 = pack2(pr[4 * nb + 2 * j], pr[4 * nb + 2 * j + 1]) *
                                     __builtin_bit_cast(half2_t, j ? sc.y : sc.x);
                        // an unwritten scale past t_end may hold anything; p there is 0
                        const int tk = tl + 16 * nb + 4 * g + 2 * j;
                        if (tk >= t_end) q2.x = (half_t)0.0f;
                        if (tk + 1 >= t_end) q2.y = (half_t)0.0f;
                        x[nb][j] = __builtin_bit_cast(uint32_t, q2);
                    }
                }
                bp[gr] = p_operand<true>(x[0][0], x[0][1], x[1][0], x[1][1]);
            }
#pragma unroll
            for (int mv = 0; mv < VM; ++mv) accv[mv] *= alpha;
        };
        // value product of tile t (position j in its super-tile): only the lanes of
        // column group j pass their p', the others zero
        auto values_sub = [&](int t, int j) __attribute__((always_inline)) {
            const uint8_t* vsl = vring + (t % kValSlots) * kVSlot;
            const bool mine = col_tile == j;
#pragma unroll
            for (int mv = 0; mv < VM; ++mv) {
                const half8 va = value_codes(Tile::value_word(vsl, mv, c, g), magic);
                const half8 pb = mine ? bp[mv / 2] : half8{};
                accv[mv] = mfma16(va, pb, accv[mv]);
            }
        };

        rotate_queries(qt, 0);
        wave_lds_sync();
        for (int i = 0; i < n_sub; ++i) {
            const int j = i % S;
            // tile i's loads are complete when at most the kDepth - 1 tiles after it
            // are in flight
            asm volatile("s_waitcnt vmcnt(%0)" :: "n"(4 * (kDepth - 1)) : "memory");
            Tile tk;
            tk.read_keys(kring + (i % kKeySlots) * kKSlot, c, g, t_end - (t_begin + kTile * i));
            Tile::issue(rs, i + kDepth < n_tiles ? blk0 + i + kDepth : -1, kring + ((i + kDepth) % kKeySlots) * kKSlot,
                        vring + ((i + kDepth) % kValSlots) * kVSlot, l);
            // the MFMA-heavy phase issues at raised priority, so that the other
            // wave on this SIMD fills its gaps with vector work
            __builtin_amdgcn_s_setprio(2);
            scores(tk, qt, col_tile == j ? c : kZeroRow, sacc, j == 0);
            __builtin_amdgcn_s_setprio(0);
            rotate_queries(qt, NH * ((i + 1) % S));
            if (i >= S) values_sub(i - S, j);
            if (j == S - 1) softmax_super(i - (S - 1));
            wave_lds_sync();
        }
#pragma unroll
        for (int j = 0; j < S; ++j) values_sub(n_sub - S + j, j);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // each head's output is spread over its S columns: sum them
#pragma unroll
        for (int mv = 0; mv < VM; ++mv)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = accv[mv][i];
                v += dppf<0x124>(v);
                v += dppf<0x128>(v);
                accv[mv][i] = v;
            }
    } else {
        rotate_queries(qt_s[w][0], 0);
        wave_lds_sync();
        // Online softmax of one tile's scores, p' = p x value scale (fp16), and
        // the value product. TAIL: the tile may end past t_end (masks on).
        auto softmax_values = [&](const Tile& T, const floatx4* sacc, int t0, auto tail_flag) __attribute__((always_inline)) {
            constexpr bool TAIL = decltype(tail_flag)::value;
            float sv[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) sv[k] = sacc[k >> 2][k & 3];
            if constexpr (TAIL) {
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (t0 + 16 * (k >> 2) + 4 * g + (k & 3) >= t_end) sv[k] = -INFINITY;
            }
            float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
            mx = xrow_max(mx);
            const float mn = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
            float pr[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) pr[k] = __builtin_amdgcn_exp2f(sv[k] - mn);
            const float ps = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
            l_run = fmaf(l_run, alpha, xrow_sum(ps));
            m_run = mn;
            half8 bp[NG];
#pragma unroll
            for (int gr = 0; gr < NG; ++gr) {
                uint32_t x[2][2];
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        half2_t q2 = T.scale_pair(gr, nb, j, pack2(pr[4 * nb + 2 * j], pr[4 * nb + 2 * j + 1]));
                        if constexpr (TAIL && INT4) {
                            // an unwritten scale past t_end may hold anything; p there is 0
                            const int tk = t0 + 16 * nb + 4 * g + 2 * j;
                            if (tk >= t_end) q2.x = (half_t)0.0f;
                            if (tk + 1 >= t_end) q2.y = (half_t)0.0f;
                        }
                        x[nb][j] = __builtin_bit_cast(uint32_t, q2);
                    }
                bp[gr] = p_operand<INT4>(x[0][0], x[0][1], x[1][0], x[1][1]);
            }
#pragma unroll
            for (int mv = 0; mv < VM; ++mv) {
                half8 va = T.value_operand(mv, magic);
                if constexpr (TAIL && !INT4) {
                    // fp16 values past t_end may hold anything (their p is zero)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (t0 + 8 * g + e >= t_end) va[e] = (half_t)0.0f;
                }
                accv[mv] *= alpha;
                accv[mv] = mfma16(va, bp[INT4 ? mv / 2 : 0], accv[mv]);
            }
        };

        // tiles in pairs through two register buffers (the next tile loads while
        // the current one is processed); the last tile runs with the masks on
        auto step = [&](const Tile& T, int t0, auto tail_flag) __attribute__((always_inline)) {
            floatx4 sacc[2];
            scores(T, qt_s[w][0], hrow, sacc, true);
            softmax_values(T, sacc, t0, tail_flag);
            rotate_queries(qt_s[w][0], 0);
            wave_lds_sync();
        };
        Tile ta, tb;
        ta.load(p, bu, t_begin, c, g);
        int t0 = t_begin;
        for (; t0 + kTile < t_last; t0 += 2 * kTile) {
            tb.load(p, bu, t0 + kTile, c, g);
            step(ta, t0, Flag<false>{});
            ta.load(p, bu, t0 + 2 * kTile, c, g);
            step(tb, t0 + kTile, Flag<false>{});
        }
        if (t0 < t_last) {
            tb.load(p, bu, t_last, c, g);
            step(ta, t0, Flag<false>{});
            step(tb, t_last, Flag<true>{});
        } else {
            step(ta, t0, Flag<true>{});
        }
    }

    if (c < NH) {
        float* ph = part + c * hstride;
        if (g == 0) {
            ph[0] = m_run;
            ph[1] = l_run;
        }
#pragma unroll
        for (int mv = 0; mv < VM; ++mv)
#pragma unroll
            for (int i = 0; i < 4; ++i) ph[2 + 16 * mv + 4 * g + i] = accv[mv][i];
    }
}

template <int R, int NH, bool INT4>
void launch_gqa(const GqaArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((rope_decode_gqa<R, NH, INT4>), dim3((a.n_waves + 3) / 4), dim3(256), 0, st, a);
}

}  // namespace

// Units of one 128-dim KV head shared by 4 query heads, rank 32 or 64, with byte
// offsets inside one unit's cache below 2^31.
bool use_gqa_kernel(const LatentGeom& g) {
    return g.s == 1 && g.gq == 4 && g.dh == 128 && (g.r == 32 || g.r == 64) &&
           (size_t)g.cap * g.r * 2 < ((size_t)1 << 31);
}

// `qbuf`: what the preparation wrote, B^k fragments [U][128][r] fp16 followed by
// the scaled queries [B][Hq][128] fp32.
int32_t launch_rope_gqa(const lrkv_latent_cache* c, const half_t* qbuf, const float2* angles, float* part,
                        int n_split, int chunk, hipStream_t st, int pending) {
    const LatentGeom g = latent_geom(c);
    const float* q = reinterpret_cast<const float*>(qbuf + (long)g.U * 128 * g.r);
    GqaArgs a{c->hk, c->hv, (const half_t*)c->sk, (const half_t*)c->sv, c->lens, q, qbuf,
              AngleTables{angles, angles + 64, angles + 33 * 64}, part, g.B, g.U, g.cap,
              n_split, chunk, g.B * g.U * n_split, pending};
    const bool int4 = g.fmt == LRKV_FMT_INT4_G32;
    if (g.r == 64) {
        if (int4) launch_gqa<64, 4, true>(a, st);
        else launch_gqa<64, 4, false>(a, st);
    } else {
        if (int4) launch_gqa<32, 4, true>(a, st);
        else launch_gqa<32, 4, false>(a, st);
    }
    return LRKV_OK;
}

}  // namespace lrkv
