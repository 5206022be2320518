// Reconstruct-with-RoPE decode attention over a Palu latent cache (gfx950).
//
// Palu digest, Method details: keys are cached as latents H^k and rebuilt on
// chip as K = H^k B^k, RoPE is applied at each token's position, the query
// attends, and the output stays in latent space, o = p H^v (B^v is folded into
// W^o offline). Palu digest, Supplementary details: the sequence is tiled along its length
// and each tile is reconstructed and scored on chip.
//
// Per 32-token tile and query head, the reconstruction GEMM H_tile B (r -> d_h)
// runs in the query-rotated basis Q' prepared by rope_prep (same MFMA work per
// token); RoPE is then one FMA per feature with the tile's cos/sin, which are
// shared by all heads of the unit. Scores feed an online softmax (log2 domain)
// and p (fp16) x H^v runs on a 16x16x32 MFMA from the dim-major value block.
// Each workgroup covers one sequence chunk of one unit and writes the chunk's
// (running max, running sum, unnormalised output) per head; merge.hip combines
// the chunks.
#include "tiles.h"

#include <math.h>

#include <type_traits>

namespace lrkv {

struct RopeArgs {
    const void* hk;
    const void* hv;
    const half_t* sk;
    const half_t* sv;
    const int32_t* lens;
    const half_t* qp;     // [B][Hq][DH][R] rotated-basis queries, scaled
    const float* qs;      // [B][U][DH/2] 2^-e scale of each frequency
    AngleTables ang;
    float* part;          // [B][Hq][n_split][R + 2]
    int B, U, NH, cap, n_split, chunk, n_groups;
    int pending;          // tokens appended in this step whose lens update is still to come
};

namespace {

// The lane's 8 frequencies in M-tile mt: feature f = 32 mt + 8 i + 4 (l/32) + e is
// the cos (e even) or sin (e odd) coefficient of frequency f / 2.
__device__ __forceinline__ int lane_freq(int k, int mt, int lane) {
    return 16 * mt + 4 * (k >> 1) + 2 * (lane >> 5) + (k & 1);
}

// Initial cos/sin (times the frequency's 2^-e) of the lane's token in the
// chunk's first tile, and the per-tile rotation.
__device__ __forceinline__ void init_angles(const RopeArgs& p, int b, int split, long bu, int mt,
                                            int lane, int DH, float* cs, float* sn, float* stc,
                                            float* sts) {
    const int half = DH / 2;
    const float2* start = p.ang.start + ((long)b * p.n_split + split) * half;
    const float2* tok = p.ang.tok + (lane & 31) * half;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int f = lane_freq(k, mt, lane);
        const float2 a = cmul(start[f], tok[f]);
        const float sc = p.qs[bu * half + f];
        cs[k] = a.x * sc;
        sn[k] = a.y * sc;
        const float2 st = p.ang.step[f];
        stc[k] = st.x;
        sts[k] = st.y;
    }
}

__device__ __forceinline__ void rotate_angles(float* cs, float* sn, const float* stc, const float* sts) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float c2 = fmaf(cs[k], stc[k], -sn[k] * sts[k]);
        const float s2 = fmaf(sn[k], stc[k], cs[k] * sts[k]);
        cs[k] = c2;
        sn[k] = s2;
    }
}

// Partial score of one head from a 32x32 score accumulator: sum over this lane's
// 16 features of cos/sin x accumulator, then over the two half-waves.
__device__ __forceinline__ float rope_combine(const floatx16& acc, const float* cs, const float* sn) {
    float ps = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
            ps = fmaf(cs[2 * i + e2], acc[4 * i + 2 * e2], ps);
            ps = fmaf(sn[2 * i + e2], acc[4 * i + 2 * e2 + 1], ps);
        }
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, ps), __builtin_bit_cast(int, ps),
                                                    false, false);
    return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

// Sum of the two half-waves' values (lane l gets v(l) + v(l ^ 32)).
__device__ __forceinline__ float add_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                                    false, false);
    return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

// Advance four cos/sin pairs by one tile: (c + i s) * st, written as in-place
// multiply / multiply-add steps so that the loop-carried values keep their
// registers.
__device__ __forceinline__ void rotate4(float* cs, float* sn, const float2* st) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float cy = cs[k] * st[k].y;
        cs[k] *= st[k].x;
        cs[k] = fmaf(-sn[k], st[k].y, cs[k]);
        sn[k] *= st[k].x;
        sn[k] += cy;
    }
}

__device__ void write_empty(float* part, long hstride, int nh, int R, int tid, int nthreads) {
    for (int e = tid; e < nh * (R + 2); e += nthreads) {
        const int h = e / (R + 2), c = e % (R + 2);
        part[h * hstride + c] = c == 0 ? -INFINITY : 0.0f;
    }
}

// ============================================================================ generic kernel
// One workgroup (4 waves): NHW query heads of one unit over one chunk. Wave w
// owns feature rows [32w, 32w+32) of each head's Q' (MFMA A fragments in
// registers); the key tile is staged in LDS; partial scores are summed across
// waves in LDS; every wave runs the same softmax; wave w owns latent dims
// [r/4 w, r/4 (w+1)) of the value product. The NH/NHW workgroups of a (chunk,
// unit) are dispatched 8 apart in block order, so they share an XCD's L2.
template <int R, int DH, int NHW, bool INT4>
__global__ __launch_bounds__(256, 2) void rope_decode(const RopeArgs p) {
    constexpr int KS = R / 16;                 // K steps of the score MFMA
    constexpr int MT = DH / 32;                // feature M-tiles per head (waves that score)
    constexpr int VM = R / 16;                 // 16-dim M-tiles of the value MFMA
    constexpr int VMW = (VM + 3) / 4;          // value M-tiles per wave
    constexpr int LDK = R + 8;
    static_assert(MT >= 1 && MT <= 4, "head_dim must be 32..128");
    __shared__ __attribute__((aligned(16))) half_t ktile[2][32][LDK];
    __shared__ float spart[4][32][NHW];
    __shared__ half_t pbuf[4][NHW][32];

    const int HG = p.NH / NHW;
    const int id = blockIdx.x, xcd = id & 7, kq = id >> 3;
    const int hg = kq % HG, g = (kq / HG) * 8 + xcd;
    if (g >= p.n_groups) return;
    const int split = g % p.n_split, u = (g / p.n_split) % p.U, b = g / (p.n_split * p.U);

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int Hq = p.U * p.NH, j0 = u * p.NH + hg * NHW;
    const int len = min(p.lens[b] + p.pending, p.cap);
    const int t_begin = split * p.chunk;
    const int t_end = min(len, t_begin + p.chunk);
    const long bu = (long)b * p.U + u;
    float* part = p.part + ((long)(b * Hq + j0) * p.n_split + split) * (R + 2);
    const long hstride = (long)p.n_split * (R + 2);
    if (t_begin >= t_end) {
        write_empty(part, hstride, NHW, R, tid, 256);
        return;
    }

    float cs[8], sn[8], stc[8], sts[8];
    if (w < MT) init_angles(p, b, split, bu, w, l, DH, cs, sn, stc, sts);

    half8 afrag[NHW][KS];
    if (w < MT) {
#pragma unroll
        for (int h = 0; h < NHW; ++h) {
            const half_t* src = p.qp + (((long)b * Hq + j0 + h) * DH + 32 * w + (l & 31)) * R + 8 * (l >> 5);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) afrag[h][kk] = *reinterpret_cast<const half8*>(src + 16 * kk);
        }
    }

    float m_run[NHW], l_run[NHW];
    floatx4 accv[VMW];
#pragma unroll
    for (int h = 0; h < NHW; ++h) { m_run[h] = -INFINITY; l_run[h] = 0.0f; }
#pragma unroll
    for (int v = 0; v < VMW; ++v) accv[v] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int n_tiles = (t_end - t_begin + 31) / 32;
    KStage<R, INT4> stage;
#pragma unroll
    for (int part_ = 0; part_ < 2; ++part_) {
        stage.load(p.hk, p.sk, bu * p.cap, t_begin, t_end, tid, part_);
        stage.template store<LDK>(ktile[0], tid, part_);
    }
    __syncthreads();

    for (int it = 0; it < n_tiles; ++it) {
        const int t0 = t_begin + 32 * it;
        const int buf = it & 1;
        const bool more = it + 1 < n_tiles;
        if (more) stage.load(p.hk, p.sk, bu * p.cap, t0 + 32, t_end, tid, 0);
        if (w < MT) {
            floatx16 acc[NHW];
#pragma unroll
            for (int h = 0; h < NHW; ++h) acc[h] = floatx16{};
            const half_t* brow = &ktile[buf][l & 31][8 * (l >> 5)];
            half8 bf = *reinterpret_cast<const half8*>(brow);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const half8 cur = bf;
                if (kk + 1 < KS) bf = *reinterpret_cast<const half8*>(brow + 16 * (kk + 1));
#pragma unroll
                for (int h = 0; h < NHW; ++h) acc[h] = mfma32(afrag[h][kk], cur, acc[h]);
            }
#pragma unroll
            for (int h = 0; h < NHW; ++h) {
                const float ps = rope_combine(acc[h], cs, sn);
                if (l < 32) spart[w][l][h] = ps;
            }
            rotate_angles(cs, sn, stc, sts);
        }
        half8 vfr[VMW];
        const long blk_base = bu * (p.cap / kTile) + t0 / kTile;
#pragma unroll
        for (int v = 0; v < VMW; ++v) {
            const int mv = w * VMW + v;
            if (mv < VM) vfr[v] = load_vfrag<R, INT4>(p.hv, p.sv, blk_base, mv, l, t0, t_end);
        }
        if (more) {
            stage.template store<LDK>(ktile[buf ^ 1], tid, 0);
            stage.load(p.hk, p.sk, bu * p.cap, t0 + 32, t_end, tid, 1);
        }
        __syncthreads();

        // online softmax (every wave, every head of the group; log2 domain)
        const int tok = l & 31;
        const bool valid = t0 + tok < t_end;
        float alpha[NHW];
#pragma unroll
        for (int h = 0; h < NHW; ++h) {
            float sc = 0.0f;
#pragma unroll
            for (int ww = 0; ww < MT; ++ww) sc += spart[ww][tok][h];
            sc = valid ? sc : -INFINITY;
            const float mn = fmaxf(m_run[h], half_max32(sc));
            alpha[h] = exp2f(m_run[h] - mn);
            const float pv = valid ? exp2f(sc - mn) : 0.0f;
            l_run[h] = fmaf(l_run[h], alpha[h], half_sum32(pv));
            m_run[h] = mn;
            if (l < 32) pbuf[w][h][tok] = (half_t)pv;
        }
        __builtin_amdgcn_wave_barrier();

        // values: acc[dim][head] += V^T p
        const int hn = l & 15;
        float a_hn = 1.0f;
#pragma unroll
        for (int h = 0; h < NHW; ++h) if (hn == h) a_hn = alpha[h];
        half8 pf = hn < NHW ? *reinterpret_cast<const half8*>(&pbuf[w][hn < NHW ? hn : 0][8 * (l >> 4)]) : half8{};
#pragma unroll
        for (int v = 0; v < VMW; ++v) {
            const int mv = w * VMW + v;
            if (mv < VM) {
                accv[v] *= a_hn;
                accv[v] = mfma16(vfr[v], pf, accv[v]);
            }
        }
        if (more) stage.template store<LDK>(ktile[buf ^ 1], tid, 1);
        __syncthreads();
    }

    if (tid < NHW) {
        part[tid * hstride + 0] = m_run[tid];
        part[tid * hstride + 1] = l_run[tid];
    }
    const int hn = l & 15;
    if (hn < NHW) {
#pragma unroll
        for (int v = 0; v < VMW; ++v) {
            const int mv = w * VMW + v;
            if (mv < VM) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    part[hn * hstride + 2 + 16 * mv + 4 * (l >> 4) + e] = accv[v][e];
            }
        }
    }
}

// ============================================================================ frequency-wave kernel
// fp16 latents, rank 256, head_dim 128, 4 query heads per unit. One workgroup
// of 4 waves per (chunk, unit). Wave w owns feature rows [32 w, 32 w + 32) of
// every head's Q' (frequencies 16 w .. 16 w + 15): 4 heads x 32 rows x 256 fp16
// = 256 registers per lane, resident in the accumulation registers and read
// there by the MFMAs. A lane's eight cos/sin pairs (its token, its
// frequencies) serve all four heads, so the per-tile angle rotation is shared.
// Iteration i of the tile loop is one instruction stream: tile i's 64 score
// MFMAs (4 heads x 16 K steps) in 16 slices, into the accumulators of tile
// parity i & 1, each slice carrying a share of the vector work:
//   * the RoPE combine of tile i-1 (the other parity's accumulators), one head
//     per slice, into per-wave partial scores, which go to LDS;
//   * the softmax of tile i-2 for head w
//     (sum of the four waves' partials; p and the rescale factor to LDS), the
//     angle rotation, and the value product of tile i-3 for all four heads on
//     16x16x32 MFMAs (wave w owns latent dims [64 w, 64 w + 64));
//   * the loads of tile i+3's keys and tile i+1's values.
// A scheduling barrier between slices keeps each share beside its MFMAs, and
// LDS reads sit at least one slice before their use. One workgroup barrier per
// tile; the stages that exchange data run one tile apart, so that barrier
// orders every exchange. Loads go buffer->LDS, keys three tiles ahead (four
// buffers) and values one tile ahead of tile i (five buffers: the value product
// lags three tiles); every wave issues exactly 8 loads per tile, so the waits
// count loads (the wait at the top of iteration i completes every wave's keys of
// tiles i and i+1, so the first fragments of tile i+1 are read at the end of
// iteration i):
//   keys   rows of 512 B with the 16-byte chunks of row t stored at
//          chunk ^ (t & 15), so that B-fragment reads (16 lanes = 16 rows, one
//          chunk) hit distinct banks; one 1 KB load writes two rows; the key
//          resource ends at the sequence's last token, so rows past it read as
//          zero (and are masked in the softmax);
//   values the dim-major 32-token block, with chunk (dim d, tokens 8c..8c+7) of
//          each 16-dim group stored at 4d + (c ^ s(d)), so that value
//          A-fragment reads (16 lanes = 16 dims, one token slot) are
//          conflict-free; tokens past the sequence end are zeroed in registers.
// The first iterations run the softmax and value product of tiles -2 and -1
// on prepared no-op data (scores -inf, p zero, rescale one, values zero).
template <int R>
__global__ __launch_bounds__(256, 1) void rope_decode_fw(const RopeArgs p) {
    constexpr int DH = 128, KS = R / 16, NH = 4, NBK = 4, NBV = 5, AH = 2;
    static_assert(R == 256, "frequency-wave kernel covers rank 256");
    __shared__ __attribute__((aligned(1024))) half_t ktile[NBK][32 * R];
    __shared__ __attribute__((aligned(1024))) half_t vtile[NBV][R * 32];
    __shared__ __attribute__((aligned(16))) float sbuf[2][NH][4][32];  // partial scores [tile parity][head][wave][token]
    __shared__ __attribute__((aligned(16))) half_t pbuf[2][16][32];    // p [tile parity][head][token]; rows 4.. zero
    __shared__ float abuf[2][16];                                      // rescale [tile parity][head]; entries 4.. one

    // unit-minor block order: blocks are dealt to the XCDs round-robin, so with 8
    // units each XCD runs every chunk of one unit and its L2 holds that unit's Q'
    const int g = blockIdx.x;
    if (g >= p.n_groups) return;
    const int u = g % p.U, split = (g / p.U) % p.n_split, b = g / (p.n_split * p.U);
    // the wave index in a scalar register, so that everything derived from it
    // (load addresses, LDS bases) is scalar arithmetic
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int Hq = p.U * NH;
    const int len = min(p.lens[b] + p.pending, p.cap);
    const int t_begin = split * p.chunk;
    const int t_end = min(len, t_begin + p.chunk);
    const long bu = (long)b * p.U + u;
    const long hstride = (long)p.n_split * (R + 2);
    float* part0 = p.part + ((long)(b * Hq + u * NH) * p.n_split + split) * (R + 2);   // head 0 of the unit
    if (t_begin >= t_end) {
        write_empty(part0 + w * hstride, 0, 1, R, l, kWave);
        return;
    }
    const int n_tiles = (t_end - t_begin + 31) / 32;
    const half_t* hk = (const half_t*)p.hk + bu * p.cap * R;
    const half_t* hv = (const half_t*)p.hv + bu * p.cap * R;      // [cap/32][R][32]

    // value chunk swizzle s(d) for dim d of a 16-dim group: distinct over any 8
    // (and any 16) consecutive dims of one token slot
    auto vswz = [](int d) { return (((d >> 1) ^ (d >> 3)) & 1) | (((d >> 2) & 1) << 1); };
    // lane offsets of the loads: key row 2n + l/32 of the wave's eight, chunk
    // (l%32) ^ (row & 15); value chunk l of a 1 KB block loads chunk l ^ s(l/4)
    const uint32_t kx = 512u * (l >> 5) + 16u * ((l & 31) ^ (l >> 5));
    const uint32_t vx = 16u * (l ^ vswz(l >> 2));
    // A tile at or past n_tiles gets empty resources: its loads fetch nothing
    // and write zeros into buffers no longer in use. Load n (0..3) of a tile's
    // keys or values; the loop spreads them over its slices.
    auto key_load = [&](int tile, int n, bool empty = false) {
        const bool real = tile < n_tiles && !empty;
        const int r0 = t_begin + 32 * min(tile, n_tiles - 1) + 8 * w;
        const int32x4 kr = make_rsrc(hk + (long)r0 * R, real ? (uint32_t)max(0, len - r0) * (R * 2) : 0u);
        buf_dma16(kr, (kx ^ (16u * (8 * (w & 1) + 2 * n))) + 1024u * n, ktile[tile % NBK] + (8 * w + 2 * n) * R);
    };
    auto value_load = [&](int tile, int n) {
        const bool real = tile < n_tiles;
        const int t0 = t_begin + 32 * min(tile, n_tiles - 1);
        const int32x4 vr = make_rsrc(hv + (long)(t0 / kTile) * R * kTile + 4 * w * 512, real ? 4096u : 0u);
        buf_dma16(vr, vx + 1024u * n, vtile[tile % NBV] + (4 * w + n) * 512);
    };
    auto issue_keys = [&](int tile, bool empty = false) {
#pragma unroll
        for (int n = 0; n < 4; ++n) key_load(tile, n, empty);
    };
    auto issue_values = [&](int tile) {
#pragma unroll
        for (int n = 0; n < 4; ++n) value_load(tile, n);
    };

    // Everything the loop starts from is requested at once: the first key and
    // value tiles, Q' and the angle tables (one wait below). Load order: keys 0,
    // values 0, keys 1, (empty), keys 2, (empty); then in iteration j (j = 0 in
    // the prologue) keys j+3 and values j+1. Keys of tile i are waited for at the
    // top of iteration i; the loads issued after them are values i-2 and the two
    // following iterations' loads, and the two empty key loads make that count
    // the same for i = 1 and 2, so every iteration waits with one count.
    issue_keys(0);
    issue_values(0);
    issue_keys(1);
    issue_keys(3, true);                       // empty: zeros into key buffer 3
    issue_keys(2);
    issue_keys(3, true);
    half8 qf[NH][KS];
    {
        // fragment-major Q': one contiguous 1 KB block per (row block, head, K step),
        // loaded into the accumulation registers (AGPRs), where the MFMAs read it
        // as their A operand
        const half_t* src = p.qp + ((bu * (DH / 32) + w) * NH * KS) * 512 + 8 * l;
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qf[h][ks] = *reinterpret_cast<const half8*>(src + (h * KS + ks) * 512);
    }
    // cos/sin (with the frequency's 2^-e) of the lane's token and eight
    // frequencies in the first tile, and the rotation by one tile
    float cs[8], sn[8];
    float2 stp[8];
    {
        float stc[8], sts[8];
        init_angles(p, b, split, bu, w, l, DH, cs, sn, stc, sts);
#pragma unroll
        for (int k = 0; k < 8; ++k) stp[k] = make_float2(stc[k], sts[k]);
    }
    // no-op data for tiles -2 and -1 (see above)
    for (int e = tid; e < NH * 4 * 32; e += 256) (&sbuf[1][0][0][0])[e] = -INFINITY;
    for (int e = tid; e < 2 * 16 * 32; e += 256) pbuf[e >> 9][(e >> 5) & 15][e & 31] = (half_t)0.0f;
    if (tid < 32) abuf[tid >> 4][tid & 15] = 1.0f;
    for (int e = tid; e < 2 * R * 32 / 8; e += 256)
        *reinterpret_cast<half8*>(&vtile[NBV - 2][8 * e]) = half8{};   // buffers NBV-2 and NBV-1
    // B fragment of K step ks: token row l%32, logical chunk 2 ks + l/32, stored at
    // chunk ^ (row & 15); with ks = 8 m + q that is 16 m + ((2 q + l/32) ^ (row & 15)).
    int koff[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) koff[q] = (l & 31) * R + 8 * ((2 * q + (l >> 5)) ^ (l & 15));
    auto kfrag = [&](const half_t* kt, int ks) -> half8 {
        return *reinterpret_cast<const half8*>(kt + koff[ks & 7] + 128 * (ks >> 3));
    };
    // value A fragment of a 16-dim group: dim l%16, token slot l/16
    const int vro = 8 * (4 * (l & 15) + ((l >> 4) ^ vswz(l & 15)));

    float m_run = -INFINITY, l_acc = 0.0f;
    floatx4 o[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) o[m] = floatx4{0.f, 0.f, 0.f, 0.f};
    // score accumulators by tile parity: tile i's MFMAs write acc[i & 1] while the
    // combine of tile i-1 reads acc[(i - 1) & 1]
    floatx16 acc[2][NH];
    half8 bq[AH];                              // the next tile's first key fragments

    // RoPE combine of head h of the tile with parity PAR (a compile-time constant,
    // so that the accumulators stay in registers): the lane's 16 features x cos/sin.
    auto combine = [&](auto PAR, int h) __attribute__((always_inline)) -> float {
        constexpr int par = decltype(PAR)::value;
        float x = 0.0f, y = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
            x = fmaf(cs[k], acc[par][h][2 * k], x);
            x = fmaf(sn[k], acc[par][h][2 * k + 1], x);
            y = fmaf(cs[k + 1], acc[par][h][2 * k + 2], y);
            y = fmaf(sn[k + 1], acc[par][h][2 * k + 3], y);
        }
        return x + y;
    };
    // Online-softmax update of head w from the tile's token scores (the sum of
    // the four waves' partials); p and the rescale factor go to LDS. A tile of
    // -inf scores (the no-op tiles) leaves the state as it is.
    auto softmax_update = [&](int tile, float s, float tmax) {
        const float mn = fmaxf(m_run, tmax);
        const float alpha = mn == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - mn);
        const float pv = s == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s - mn);
        m_run = mn;
        l_acc = fmaf(l_acc, alpha, pv);
        pbuf[tile & 1][w][l & 31] = (half_t)pv;
        abuf[tile & 1][w] = alpha;
    };
    auto read_scores = [&](int tile) -> float {
        const float* sp = &sbuf[tile & 1][w][0][l & 31];
        return (sp[0] + sp[32]) + (sp[64] + sp[96]);
    };
    // Value product of tile `tile` for all four heads, dims [64 w, 64 w + 64).
    auto value_product = [&](int tile, bool tail) {
        const half8 pf = *reinterpret_cast<const half8*>(&pbuf[tile & 1][l & 15][8 * (l >> 4)]);
        const float al = abuf[tile & 1][l & 15];
        const half_t* vt = vtile[(tile + NBV) % NBV] + 4 * w * 512 + vro;
        const int first = t_begin + 32 * tile + 8 * (l >> 4);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            half8 a = *reinterpret_cast<const half8*>(vt + 512 * m);
            if (tail) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (first + e >= len) a[e] = (half_t)0.0f;
            }
            o[m] = mfma16(a, pf, o[m] * al);
        }
    };
    // Partial scores of tile `tile` (this wave's frequencies) to LDS.
    auto write_partials = [&](int tile, const float* ps, bool tail) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            float v = add_halves(ps[h]);
            if (tail && t_begin + 32 * tile + (l & 31) >= len) v = -INFINITY;
            sbuf[tile & 1][h][w][l & 31] = v;
        }
    };
    auto score_mfma = [&](int tile) {
        const half_t* kt = ktile[tile % NBK];
#pragma unroll
        for (int a = 0; a < AH; ++a) bq[a] = kfrag(kt, a);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const half8 cur = bq[ks % AH];
            if (ks + AH < KS) bq[ks % AH] = kfrag(kt, ks + AH);
#pragma unroll
            for (int h = 0; h < NH; ++h) acc[0][h] = mfma32(qf[h][ks], cur, ks == 0 ? floatx16{} : acc[0][h]);
        }
    };

    // the one wait: a real s_waitcnt vmcnt(0), which the compiler's wait tracking
    // sees, so it adds no waits for these loads inside the loop. Q' is pinned to
    // the AGPRs only now: pinning a fragment right after its own load would
    // serialize the round trips.
    __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+a"(qf[h][ks]));
    __syncthreads();
    issue_keys(3);
    issue_values(1);
    score_mfma(0);
    // tile 1's keys came with the prologue (complete and visible since its barrier)
    if (n_tiles > 1) {
#pragma unroll
        for (int a = 0; a < AH; ++a) bq[a] = kfrag(ktile[1 % NBK], a);
    }
    // iteration i (parity PAR = i & 1 as a compile-time constant)
    auto iteration = [&](int i, auto PAR) __attribute__((always_inline)) {
        constexpr int cur_p = decltype(PAR)::value, prv_p = cur_p ^ 1;
        // every wave's keys of tiles i and i+1 are complete: the loads after the
        // keys of tile i+1 (issued two iterations ago) are at most 12
        asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
        __syncthreads();
        float ps[NH];
        const half_t* kt = ktile[i % NBK];
        float s = 0.0f, tmax = 0.0f;
        half8 pf = {}, va[2] = {};
        float al = 1.0f;
        const int st = i - 2, vt_tile = i - 3;   // softmax / value-product tiles (negative: no-op data)
        const half_t* vt = vtile[(vt_tile + NBV) % NBV] + 4 * w * 512 + vro;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const half8 cur = bq[ks % AH];
            if (ks + AH < KS) bq[ks % AH] = kfrag(kt, ks + AH);
#pragma unroll
            for (int h = 0; h < NH; ++h)
                acc[cur_p][h] = mfma32(qf[h][ks], cur, ks == 0 ? floatx16{} : acc[cur_p][h]);
            // combine of tile i-1, one head per slice, beside this tile's MFMAs
            if (ks < NH) {
                ps[ks] = combine(std::integral_constant<int, prv_p>{}, ks);
            } else if (ks == 4) {
                write_partials(i - 1, ps, false);
                s = read_scores(st);
            } else if (ks == 5) {
                tmax = fmaxf(s, dppf<0xB1>(s));
                tmax = fmaxf(tmax, dppf<0x4E>(tmax));
            } else if (ks == 6) {
                tmax = fmaxf(tmax, dppf<0x141>(tmax));
                tmax = fmaxf(tmax, dppf<0x140>(tmax));
                tmax = rowpair(tmax, true);
            } else if (ks == 7) {
                softmax_update(st, s, tmax);
            } else if (ks == 8 || ks == 9) {
                rotate4(cs + 4 * (ks - 8), sn + 4 * (ks - 8), stp + 4 * (ks - 8));
            }
            // value product of tile i-3
            if (ks == 10) {
                pf = *reinterpret_cast<const half8*>(&pbuf[vt_tile & 1][l & 15][8 * (l >> 4)]);
                al = abuf[vt_tile & 1][l & 15];
            }
            if (ks >= 10 && ks < 14) va[ks & 1] = *reinterpret_cast<const half8*>(vt + 512 * (ks - 10));
            if (ks >= 11 && ks < 15) {
                const int m = ks - 11;
                o[m] = mfma16(va[m & 1], pf, o[m] * al);
            }
            // keys of tile i+3 (their buffer was last read by tile i-1's MFMAs) and
            // values of tile i+1 (buffer last read by tile i-4's product), both
            // finished by every wave before this tile's barrier; one load every
            // other slice, so that no wave stalls long on a full memory queue
            // while its MFMAs wait behind the load
            if (ks < 8 && (ks & 1)) key_load(i + 3, ks >> 1);
            if (ks >= 8 && (ks & 1)) value_load(i + 1, (ks - 8) >> 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        // the next tile's first fragments (its keys are complete since this
        // iteration's barrier; their buffer is rewritten two iterations later)
        if (i + 1 < n_tiles) {
#pragma unroll
            for (int a = 0; a < AH; ++a) bq[a] = kfrag(ktile[(i + 1) % NBK], a);
        }
    };
    int it = 1;
    for (; it + 1 < n_tiles; it += 2) {
        iteration(it, std::integral_constant<int, 1>{});
        iteration(it + 1, std::integral_constant<int, 0>{});
    }
    if (it < n_tiles) iteration(it, std::integral_constant<int, 1>{});
    wait_vmem();                               // the loads past the last tile (empty)
    // drain: partials of the last tile; softmax of the last two tiles; value
    // products of the last three, each exchange separated by a barrier
    {
        float ps[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h)
            ps[h] = ((n_tiles - 1) & 1) ? combine(std::integral_constant<int, 1>{}, h)
                                        : combine(std::integral_constant<int, 0>{}, h);
        write_partials(n_tiles - 1, ps, true);
    }
    __syncthreads();
    {
        const float s = read_scores(n_tiles - 2);
        softmax_update(n_tiles - 2, s, half_max32(s));
    }
    value_product(n_tiles - 3, false);
    __syncthreads();
    {
        const float s = read_scores(n_tiles - 1);
        softmax_update(n_tiles - 1, s, half_max32(s));
    }
    __syncthreads();
    value_product(n_tiles - 2, false);
    value_product(n_tiles - 1, true);

    // lanes with head l%16 < 4 hold dims 16 (4 w + m) + 4 (l/16) + e of that head
    if ((l & 15) < NH) {
        float* ph = part0 + (l & 15) * hstride + 2 + 64 * w + 4 * (l >> 4);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) ph[16 * m + e] = o[m][e];
    }
    const float lsum = half_sum32(l_acc);
    if (l == 0) {
        part0[w * hstride + 0] = m_run;
        part0[w * hstride + 1] = lsum;
    }
}

template <int R, int DH, int NHW, bool INT4>
void launch_generic(RopeArgs a, hipStream_t st) {
    a.n_groups = a.n_split * a.U * a.B;
    const int slots = (a.n_groups + 7) / 8;
    hipLaunchKernelGGL((rope_decode<R, DH, NHW, INT4>), dim3(slots * 8 * (a.NH / NHW)), dim3(256), 0, st, a);
}

}  // namespace

// The frequency-wave kernel: fp16 rank-256 units of four 128-dim heads, with
// 32-bit byte offsets into one unit's cache. Its queries are prepared in
// fragment order.
static bool use_frequency_wave(const lrkv_latent_cache* c) {
    return c->rank == 256 && c->head_dim == 128 && c->kv_per_unit * c->q_per_kv == 4 &&
           c->fmt == LRKV_FMT_FP16 && (size_t)c->capacity * 256 * 2 < ((size_t)1 << 32);
}
bool rope_fragment_layout(const lrkv_latent_cache* c) { return use_frequency_wave(c); }

bool rope_shape_supported(int r, int dh, int nh) {
    return (r == 32 && dh == 64 && nh == 2) || (r == 64 && dh == 64 && nh == 2) ||
           (r == 256 && dh == 128 && nh == 4) || (r == 64 && dh == 128 && nh == 4) ||
           (r == 128 && dh == 128 && nh == 4);
}

int32_t launch_rope_decode(const lrkv_latent_cache* c, const half_t* qp, const float* qs,
                           const float2* angles, float* part, int n_split, int chunk, hipStream_t st, int pending) {
    const int nh = c->kv_per_unit * c->q_per_kv, r = c->rank, dh = c->head_dim;
    const bool int4 = c->fmt == LRKV_FMT_INT4_G32;
    RopeArgs a{c->hk, c->hv, (const half_t*)c->sk, (const half_t*)c->sv, c->lens, qp, qs,
               AngleTables{angles, angles + dh / 2, angles + 33 * (dh / 2)}, part, c->batch,
               c->units, nh, c->capacity, n_split, chunk, 0, pending};
    if (use_frequency_wave(c)) {
        a.n_groups = n_split * a.U * a.B;
        hipLaunchKernelGGL(rope_decode_fw<256>, dim3(a.n_groups), dim3(256), 0, st, a);
        return LRKV_OK;
    }
    // heads per workgroup of the generic kernel: two for the larger ranks
    // (register budget of two resident workgroups per CU)
#define LRKV_ROPE(R_, DH_, NH_, NHW16_, NHW4_)                                               \
    if (r == R_ && dh == DH_ && nh == NH_) {                                                \
        if (int4) launch_generic<R_, DH_, NHW4_, true>(a, st);                               \
        else launch_generic<R_, DH_, NHW16_, false>(a, st);                                  \
        return LRKV_OK;                                                                      \
    }
    LRKV_ROPE(32, 64, 2, 2, 2)
    LRKV_ROPE(64, 64, 2, 2, 2)
    LRKV_ROPE(256, 128, 4, 1, 1)
    LRKV_ROPE(64, 128, 4, 4, 4)
    LRKV_ROPE(128, 128, 4, 2, 2)
#undef LRKV_ROPE
    return LRKV_ERR_UNSUPPORTED;
}

}  // namespace lrkv
