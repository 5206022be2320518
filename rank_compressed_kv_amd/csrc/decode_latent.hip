// Decode attention over a Palu latent cache (gfx950).
//
// Palu digest, Method details: keys are cached as latents H^k and rebuilt on
// chip as K = H^k B^k; RoPE is applied at each token's position; the value
// reconstruction is folded into W^o, so the output is o = p H^v (latent space).
// Without RoPE the reconstruction is absorbed into the query: scores = H^k q'.
// Palu digest, Appendix: the sequence is tiled along its length and each tile
// is reconstructed and scored on chip.
//
// Reconstruct-with-RoPE path, as done here. For query head j with key slice
// B (r x d_h) and the rotate-half pair (i, i + d_h/2) at angle
// phi_i(t) = (t - q_pos) theta_i:
//     q_rot . k_rot(t) = sum_i cos(phi_i) (h_t . u_i) + sin(phi_i) (h_t . w_i)
//     u_i = q_i B[:, i] + q_{i+h} B[:, i+h],  w_i = q_{i+h} B[:, i] - q_i B[:, i+h]
// i.e. the tile's reconstruction GEMM H_tile B (r -> d_h columns) is done in the
// query-rotated basis Q' = [u_0, w_0, u_1, w_1, ...] (r x d_h): the same MFMA
// work per token, after which RoPE costs one FMA per feature and the cos/sin
// values are shared by every head of the unit.
//
// Work split (one workgroup = 4 waves per (sequence chunk, unit, batch)):
//   scores  wave w owns feature rows [32w, 32w+32) of every head's Q' (held in
//           registers as MFMA A fragments); the 32-token key tile is staged in
//           LDS and read as the B fragment; partial scores are summed across
//           waves through LDS.
//   softmax every wave keeps the same running (max, sum) per head (log2 domain).
//   values  wave w owns latent dims [r/4 w, r/4 (w+1)); p (fp16) x H^v on a
//           16x16x32 MFMA straight from the dim-major value block.
// The chunk's (m, l, acc) go to the workspace; a merge kernel combines chunks.
#include "common.h"

#include <math.h>

namespace lrkv {
namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;

struct RopeArgs {
    const void* hk;
    const void* hv;
    const half_t* sk;
    const half_t* sv;
    const int32_t* lens;
    const int32_t* q_pos;
    const half_t* qp;     // [B][Hq][DH][R] rotated-basis queries, scaled
    const float* qs;      // [B][U][DH/2] 2^-e of the scaling of each frequency
    float* part;          // [B][Hq][n_split][R + 2]
    int B, U, NH, cap, n_split, chunk, n_groups;
    double theta;
};

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

// ------------------------------------------------------------------------ query prep
// Rotated-basis queries Q'[f][k] (f < DH, k < R) of every head of a unit:
//   row 2i   = q_i B[:, i] + q_{i+h} B[:, i+h]     (cos coefficient of frequency i)
//   row 2i+1 = q_{i+h} B[:, i] - q_i B[:, i+h]     (sin coefficient)
// scaled by sm_scale*log2(e)*2^e_i, one power of two per (unit, frequency) shared
// by the unit's heads, chosen so that the largest |Q'| of that frequency lands in
// [2^14, 2^15) (fp16 range); the decode kernel folds 2^-e_i into its cos/sin.
// Grid: (B*U, DH/8); block: 4 frequencies x 64 k-lanes, looping over heads.
__global__ __launch_bounds__(256) void rope_qprep(const float* __restrict__ q,
                                                  const half_t* __restrict__ bk,
                                                  half_t* __restrict__ qp, float* __restrict__ qs,
                                                  int U, int s, int gq, int DH, int R, float scale) {
    constexpr int KPT = 4;                                   // k values per thread (R <= 256)
    const int bu = blockIdx.x, u = bu % U, b = bu / U;
    const int NH = s * gq, Hq = U * NH, half = DH / 2, ldb = s * DH;
    const int fi = threadIdx.x & 3, kl = threadIdx.x >> 2;   // 4 frequencies x 64 k-lanes
    const int i = blockIdx.y * 4 + fi;
    const half_t* Bu = bk + (size_t)u * R * ldb;
    __shared__ float red[4][64];
    float mx = 0.0f;
    for (int h = 0; h < NH; ++h) {
        const int j = u * NH + h, w = (j / gq) % s;
        const float qa = q[((size_t)b * Hq + j) * DH + i] * scale;
        const float qb = q[((size_t)b * Hq + j) * DH + i + half] * scale;
#pragma unroll
        for (int m = 0; m < KPT; ++m) {
            const int k = kl + 64 * m;
            if (k < R) {
                const float b0 = (float)Bu[(size_t)k * ldb + w * DH + i];
                const float b1 = (float)Bu[(size_t)k * ldb + w * DH + i + half];
                mx = fmaxf(mx, fmaxf(fabsf(fmaf(qa, b0, qb * b1)), fabsf(fmaf(qb, b0, -qa * b1))));
            }
        }
    }
    // max over the 64 k-lanes of each frequency: lanes fi, fi+4, ... of the block
#pragma unroll
    for (int o = 4; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
    if ((threadIdx.x & 63) < 4) red[fi][threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[fi][0], red[fi][1]), fmaxf(red[fi][2], red[fi][3]));
    const int ex = (mx > 0.0f && isfinite(mx)) ? 14 - ilogbf(mx) : 0;
    for (int h = 0; h < NH; ++h) {
        const int j = u * NH + h, w = (j / gq) % s;
        const float qa = ldexpf(q[((size_t)b * Hq + j) * DH + i] * scale, ex);
        const float qb = ldexpf(q[((size_t)b * Hq + j) * DH + i + half] * scale, ex);
        half_t* out = qp + ((size_t)b * Hq + j) * DH * R;
#pragma unroll
        for (int m = 0; m < KPT; ++m) {
            const int k = kl + 64 * m;
            if (k < R) {
                const float b0 = (float)Bu[(size_t)k * ldb + w * DH + i];
                const float b1 = (float)Bu[(size_t)k * ldb + w * DH + i + half];
                out[(size_t)(2 * i) * R + k] = (half_t)fmaf(qa, b0, qb * b1);
                out[(size_t)(2 * i + 1) * R + k] = (half_t)fmaf(qb, b0, -qa * b1);
            }
        }
    }
    if (kl == 0) qs[((size_t)b * U + u) * half + i] = ldexpf(1.0f, -ex);
}

// ------------------------------------------------------------------------ tile staging
// Key tile of 32 tokens as fp16 rows in LDS (int4 codes are dequantised here:
// code * scale rounded to fp16). Rows at or past t_end are zero.
template <int R, bool INT4>
struct KStage {
    static constexpr int NV = 32 * R / 8;                 // 8-dim items per tile
    static constexpr int PER = (NV + 255) / 256;
    static constexpr int HALF = (PER + 1) / 2;            // items staged per half
    uint4 v[HALF];

    // Loads items [HALF*part, HALF*part + HALF) of this thread (part 0 or 1).
    __device__ __forceinline__ void load(const void* hk, const half_t* sk, long row0, int t0,
                                         int t_end, int tid, int part) {
#pragma unroll
        for (int kk = 0; kk < HALF; ++kk) {
            const int k = HALF * part + kk;
            const int item = tid + 256 * k;
            const int row = item / (R / 8), c8 = item % (R / 8);
            v[kk] = make_uint4(0, 0, 0, 0);
            if (k < PER && item < NV && t0 + row < t_end) {
                const long tok = row0 + t0 + row;
                if constexpr (!INT4) {
                    v[kk] = *reinterpret_cast<const uint4*>((const half_t*)hk + tok * R + c8 * 8);
                } else {
                    const uint32_t code = *reinterpret_cast<const uint32_t*>((const uint8_t*)hk + tok * (R / 2) + c8 * 4);
                    const float sc = (float)sk[tok * (R / 32) + c8 / 4];
                    half8 h;
#pragma unroll
                    for (int e = 0; e < 8; ++e) h[e] = (half_t)((float)nibble(code, e) * sc);
                    v[kk] = *reinterpret_cast<uint4*>(&h);
                }
            }
        }
    }
    template <int LDK>
    __device__ __forceinline__ void store(half_t (*tile)[LDK], int tid, int part) const {
#pragma unroll
        for (int kk = 0; kk < HALF; ++kk) {
            const int k = HALF * part + kk;
            const int item = tid + 256 * k;
            if (k < PER && item < NV) {
                const int row = item / (R / 8), c8 = item % (R / 8);
                *reinterpret_cast<uint4*>(&tile[row][c8 * 8]) = v[kk];
            }
        }
    }
};

// A fragment of V^T for the 16x16x32 MFMA: dims [16*mv, 16*mv + 16) x the 8 tokens
// of lane group g = l/16 in the 32-token block `blk`, masked past t_end.
template <int R, bool INT4>
__device__ __forceinline__ half8 load_vfrag(const void* hv, const half_t* sv, long blk_base,
                                            int mv, int lane, int tok0, int t_end) {
    const int dim = 16 * mv + (lane & 15);
    const int g = lane >> 4;
    half8 a;
    if constexpr (!INT4) {
        a = *reinterpret_cast<const half8*>((const half_t*)hv + (blk_base * R + dim) * kTile + 8 * g);
    } else {
        const uint32_t code = *reinterpret_cast<const uint32_t*>((const uint8_t*)hv + (blk_base * R + dim) * (kTile / 2) + 4 * g);
        const half8 sc = *reinterpret_cast<const half8*>(sv + (blk_base * (R / 32) + dim / 32) * kTile + 8 * g);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = (half_t)((float)nibble(code, e) * (float)sc[e]);
    }
    const int first = tok0 + 8 * g;
    if (first + 8 > t_end) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (first + e >= t_end) a[e] = (half_t)0.0f;
    }
    return a;
}

// cos / sin of 2 pi * frac(dt * rho_k) for the 8 frequencies of this lane, exact
// to fp32 rounding: the angle is reduced in fp64 before the fp64 sincos. One
// frequency at a time into the lane's LDS slots (keeps the fp64 temporaries out
// of the register peak of the caller).
__device__ __forceinline__ double lane_rho(int k, int w, int lane, int dh, double log2_theta) {
    const int fr = 16 * w + 4 * (k >> 1) + 2 * (lane >> 5) + (k & 1);
    return log2_theta != 0.0 ? exp2(-2.0 * fr / dh * log2_theta) / kTwoPi : 0.0;
}
__device__ __forceinline__ void anchor_angles(float (*slot)[2], int w, int lane, int dh,
                                              double log2_theta, long dt0) {
#pragma unroll 1
    for (int k = 0; k < 8; ++k) {
        double rev = (double)dt0 * lane_rho(k, w, lane, dh, log2_theta);
        rev -= rint(rev);
        double sd, cd;
        sincos(kTwoPi * rev, &sd, &cd);
        slot[k][0] = (float)cd;
        slot[k][1] = (float)sd;
    }
}

// ------------------------------------------------------------------------ RoPE decode
// Sum over the 32 lanes of each half-wave (DPP within rows of 16, then a
// row-pair exchange).
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// v_permlane16_swap(v, v) returns {row 2k, row 2k+1} values in every lane of the
// row pair, so their sum / max is the row-pair result.
__device__ __forceinline__ float rowpair(float v, bool is_max) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                                    false, false);
    const float a = __builtin_bit_cast(float, (int)r[0]), b = __builtin_bit_cast(float, (int)r[1]);
    return is_max ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float half_sum32(float v) {
    v += dppf<0xB1>(v);
    v += dppf<0x4E>(v);
    v += dppf<0x141>(v);
    v += dppf<0x140>(v);
    return rowpair(v, false);
}
__device__ __forceinline__ float half_max32(float v) {
    v = fmaxf(v, dppf<0xB1>(v));
    v = fmaxf(v, dppf<0x4E>(v));
    v = fmaxf(v, dppf<0x141>(v));
    v = fmaxf(v, dppf<0x140>(v));
    return rowpair(v, true);
}

// Key tile of 32 tokens x 256 fp16 staged with direct global->LDS loads. A
// 64-lane load writes lane i at +16 i; issued by half a wave it writes one
// 512-byte row, so rows can be padded to 528 bytes (conflict-free B-fragment
// reads: consecutive rows start 4 banks apart). Rows at or past t_end are not
// loaded (their scores are masked).
template <int R>
struct KDma {
    static_assert(R == 256, "direct staging covers rank 256");
    static constexpr int LDK = R + 8;                        // padded row, in halves
    __device__ __forceinline__ static void issue(const half_t* hk, long row0, int t0, int t_end,
                                                 half_t* tile, int w, int l) {
        typedef __attribute__((address_space(3))) void lds_void;
        typedef __attribute__((address_space(1))) const void gbl_void;
        // One load per half-wave and row; the LDS address is built from wave-uniform
        // values only (the trip variable is uniform and the loop is not unrolled, so
        // the two halves never share one instruction with a per-lane address).
#pragma unroll 1
        for (int n = 0; n < 8; ++n) {
            const int half = n & 1;
            const int row = 8 * w + n;                         // rows 8w .. 8w + 7
            if ((l >> 5) == half && t0 + row < t_end) {
                const half_t* src = hk + (row0 + t0 + row) * R + (l & 31) * 8;
                __builtin_amdgcn_global_load_lds((gbl_void*)src, (lds_void*)(tile + row * LDK - half * 32 * 8),
                                                 16, 0, 0);
            }
        }
    }
};

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One workgroup: NHW query heads of one unit over one sequence chunk. The
// NH/NHW workgroups of a (chunk, unit) are dispatched 8 apart in block order, so
// they land on the same XCD at about the same time and share the latent tiles
// through its L2.
template <int R, int DH, int NHW, bool INT4>
__global__ __launch_bounds__(256, 2) void rope_decode(const RopeArgs p) {
    constexpr int KS = R / 16;                 // K steps of the score MFMA
    constexpr int MT = DH / 32;                // feature M-tiles per head (waves that score)
    constexpr int VM = R / 16;                 // 16-dim M-tiles of the value MFMA
    constexpr int VMW = (VM + 3) / 4;          // value M-tiles per wave
    constexpr bool DMA = !INT4 && R == 256;   // direct global->LDS key staging
    constexpr int LDK = R + 8;
    static_assert(MT >= 1 && MT <= 4, "head_dim must be 32..128");
    __shared__ __attribute__((aligned(16))) half_t ktile[2][32 * LDK];
    __shared__ float spart[4][32][NHW];
    __shared__ half_t pbuf[4][NHW][32];
    __shared__ float step[4][64][8][2];        // per-lane rotation by 32 positions
    __shared__ float anc[4][64][8][2];         // per-lane anchor angles

    // XCD-aware decode of the block index: group g (= chunk, unit, batch) on XCD g % 8
    const int HG = p.NH / NHW;
    const int id = blockIdx.x, xcd = id & 7, kq = id >> 3;
    const int hg = kq % HG, g = (kq / HG) * 8 + xcd;
    if (g >= p.n_groups) return;
    const int split = g % p.n_split, u = (g / p.n_split) % p.U, b = g / (p.n_split * p.U);

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int Hq = p.U * p.NH, j0 = u * p.NH + hg * NHW;
    const int len = min(p.lens[b], p.cap);        // never read past the capacity
    const int t_begin = split * p.chunk;
    const int t_end = min(len, t_begin + p.chunk);
    const long bu = (long)b * p.U + u;
    float* part = p.part + ((long)(b * Hq + j0) * p.n_split + split) * (R + 2);
    const long hstride = (long)p.n_split * (R + 2);

    if (t_begin >= t_end) {                    // empty chunk
        for (int e = tid; e < NHW * (R + 2); e += 256) {
            const int h = e / (R + 2), c = e % (R + 2);
            part[h * hstride + c] = c == 0 ? -INFINITY : 0.0f;
        }
        return;
    }

    // this lane's 8 frequencies: feature f = 32w + 8i + 4(l/32) + e has frequency
    // f/2 and is its cos (e even) or sin (e odd) coefficient. The cos/sin values
    // carry the frequency's 2^-e scale; the per-tile rotation table does not.
    float cs[8], sn[8];
    const int qpos = p.q_pos ? p.q_pos[b] : len - 1;
    const double l2t = p.theta > 0.0 ? log2(p.theta) : 0.0;
    anchor_angles(step[w][l], w, l, DH, l2t, 32);
    const float* fscale = p.qs + bu * (DH / 2) + 16 * w + 2 * (l >> 5);
    auto anchor = [&](long dt) {
        anchor_angles(anc[w][l], w, l, DH, l2t, dt);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float f = w < MT ? fscale[4 * (k >> 1) + (k & 1)] : 0.0f;
            cs[k] = anc[w][l][k][0] * f;
            sn[k] = anc[w][l][k][1] * f;
        }
    };
    anchor((long)t_begin + (l & 31) - qpos);

    // rotated-basis query fragments (MFMA A operands) for this wave's feature rows
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
    auto tile_rows = [&](int bsel) { return reinterpret_cast<half_t(*)[LDK]>(ktile[bsel]); };
    if constexpr (DMA) {
        KDma<R>::issue((const half_t*)p.hk, bu * p.cap, t_begin, t_end, ktile[0], w, l);
        wait_dma();
    } else {
#pragma unroll
        for (int part = 0; part < 2; ++part) {
            stage.load(p.hk, p.sk, bu * p.cap, t_begin, t_end, tid, part);
            stage.template store<LDK>(tile_rows(0), tid, part);
        }
    }
    __syncthreads();

    // The next key tile is staged in two halves (first half around the score
    // MFMAs, second half around the softmax) to halve the staging registers.
    for (int it = 0; it < n_tiles; ++it) {
        const int t0 = t_begin + 32 * it;
        const int buf = it & 1;
        const bool more = it + 1 < n_tiles;
        if constexpr (DMA) {
            if (more) KDma<R>::issue((const half_t*)p.hk, bu * p.cap, t0 + 32, t_end, ktile[buf ^ 1], w, l);
        } else {
            if (more) stage.load(p.hk, p.sk, bu * p.cap, t0 + 32, t_end, tid, 0);
        }

        // ---- scores in the rotated basis, then the RoPE combination
        if (w < MT) {
            floatx16 acc[NHW];
#pragma unroll
            for (int h = 0; h < NHW; ++h) acc[h] = floatx16{};
            // B fragments read one K step ahead of the MFMAs that use them
            const half_t* brow = &tile_rows(buf)[l & 31][8 * (l >> 5)];
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
                float ps = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e2 = 0; e2 < 2; ++e2) {
                        ps = fmaf(cs[2 * i + e2], acc[h][4 * i + 2 * e2], ps);
                        ps = fmaf(sn[2 * i + e2], acc[h][4 * i + 2 * e2 + 1], ps);
                    }
                ps += __shfl_xor(ps, 32, kWave);
                if (l < 32) spart[w][l][h] = ps;
            }
        }
        // value fragments of this tile, used after the softmax
        half8 vfr[VMW];
        const long blk_base = bu * (p.cap / kTile) + t0 / kTile;
#pragma unroll
        for (int v = 0; v < VMW; ++v) {
            const int mv = w * VMW + v;
            if (mv < VM) vfr[v] = load_vfrag<R, INT4>(p.hv, p.sv, blk_base, mv, l, t0, t_end);
        }
        if constexpr (!DMA) {
            if (more) {
                stage.template store<LDK>(tile_rows(buf ^ 1), tid, 0);
                stage.load(p.hk, p.sk, bu * p.cap, t0 + 32, t_end, tid, 1);
            }
        }
        // advance the angles by 32 positions (a chunk has at most kMaxRopeTiles
        // tiles, so the fp32 rotation drift stays below ~2e-5 rad)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float cst = step[w][l][k][0], snt = step[w][l][k][1];
            const float c2 = fmaf(cs[k], cst, -sn[k] * snt);
            const float s2 = fmaf(sn[k], cst, cs[k] * snt);
            cs[k] = c2;
            sn[k] = s2;
        }
        __syncthreads();

        // ---- online softmax (every wave, every head of the group; log2 domain)
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

        // ---- values: acc[dim][head] += V^T p
        const int hn = l & 15;
        float a_hn = 1.0f;
#pragma unroll
        for (int h = 0; h < NHW; ++h) if (hn == h) a_hn = alpha[h];
        half8 pf;
        if (hn < NHW) {
            pf = *reinterpret_cast<const half8*>(&pbuf[w][hn][8 * (l >> 4)]);
        } else {
            pf = half8{};
        }
#pragma unroll
        for (int v = 0; v < VMW; ++v) {
            const int mv = w * VMW + v;
            if (mv < VM) {
                accv[v] *= a_hn;
                accv[v] = mfma16(vfr[v], pf, accv[v]);
            }
        }
        if constexpr (DMA) {
            wait_dma();
        } else {
            if (more) stage.template store<LDK>(tile_rows(buf ^ 1), tid, 1);
        }
        __syncthreads();
    }

    // ---- chunk partials: (m, l) per head, then acc[dim] per head
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

// ------------------------------------------------------------------------ absorbed decode
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
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qv[kk][e] = hn < NH ? p.q[((long)b * Hq + j0 + hn) * R + 32 * kk + 8 * g + e] * p.qscale : 0.0f;
                mx = fmaxf(mx, fabsf(qv[kk][e]));
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
        // scores: two 16-token M-tiles; lane holds tokens 16mt + 4g + e for head hn
        floatx4 sc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
            const int row = t0 + 16 * mt + hn;
            const bool ok = row < t_end;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                half8 a;
                if constexpr (!INT4) {
                    a = ok ? *reinterpret_cast<const half8*>((const half_t*)p.hk + (bu * p.cap + row) * R + 32 * kk + 8 * g)
                           : half8{};
                } else {
                    a = half8{};
                    if (ok) {
                        const uint32_t code = *reinterpret_cast<const uint32_t*>((const uint8_t*)p.hk + (bu * p.cap + row) * (R / 2) + 16 * kk + 4 * g);
                        const float s = (float)p.sk[(bu * p.cap + row) * (R / 32) + kk];
#pragma unroll
                        for (int e = 0; e < 8; ++e) a[e] = (half_t)((float)nibble(code, e) * s);
                    }
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
        const long blk_base = bu * (p.cap / kTile) + t0 / kTile;
#pragma unroll
        for (int v = 0; v < VM; ++v) {
            const int dim = 16 * v + hn;
            half8 a;
            if constexpr (!INT4) {
                const half_t* src = (const half_t*)p.hv + (blk_base * R + dim) * kTile;
                const half4 lo = *reinterpret_cast<const half4*>(src + 4 * g);
                const half4 hi = *reinterpret_cast<const half4*>(src + 16 + 4 * g);
                a = half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
                const uint8_t* src = (const uint8_t*)p.hv + (blk_base * R + dim) * (kTile / 2);
                const uint32_t clo = *reinterpret_cast<const uint16_t*>(src + 2 * g);
                const uint32_t chi = *reinterpret_cast<const uint16_t*>(src + 8 + 2 * g);
                const half_t* ss = p.sv + (blk_base * (R / 32) + dim / 32) * kTile;
                const half4 slo = *reinterpret_cast<const half4*>(ss + 4 * g);
                const half4 shi = *reinterpret_cast<const half4*>(ss + 16 + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a[e] = (half_t)((float)nibble(clo, e) * (float)slo[e]);
                    a[4 + e] = (half_t)((float)nibble(chi, e) * (float)shi[e]);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = t0 + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4);
                if (t >= t_end) a[e] = (half_t)0.0f;
            }
            acc[v] *= alpha;
            acc[v] = mfma16(a, pf, acc[v]);
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

// ------------------------------------------------------------------------ split merge
// out[b][j][d] = sum_c 2^(m_c - M) acc_c[d] / sum_c 2^(m_c - M) l_c over the
// n_split chunks (at most 1024); empty chunks (m = -inf) contribute nothing.
// The chunk maxima and weights are loaded once into LDS by the whole block.
__global__ __launch_bounds__(256) void merge_splits(const float* __restrict__ part,
                                                    float* __restrict__ out, int n_split, int D) {
    __shared__ float wts[1024];
    __shared__ float red[256];
    const long bj = blockIdx.x;
    const float* pp = part + bj * n_split * (D + 2);
    float mx = -INFINITY;
    for (int c = threadIdx.x; c < n_split; c += blockDim.x) {
        const float m = pp[(long)c * (D + 2)];
        wts[c] = m;
        mx = fmaxf(mx, m);
    }
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
        __syncthreads();
    }
    mx = red[0];
    __syncthreads();
    float den = 0.0f;
    for (int c = threadIdx.x; c < n_split; c += blockDim.x) {
        const float m = wts[c];
        const float wgt = m == -INFINITY ? 0.0f : exp2f(m - mx);
        wts[c] = wgt;
        den = fmaf(wgt, pp[(long)c * (D + 2) + 1], den);
    }
    red[threadIdx.x] = den;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    const float rden = 1.0f / red[0];
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float n0 = 0.0f, n1 = 0.0f, n2 = 0.0f, n3 = 0.0f;
        int c = 0;
        for (; c + 4 <= n_split; c += 4) {
            n0 = fmaf(wts[c], pp[(long)c * (D + 2) + 2 + d], n0);
            n1 = fmaf(wts[c + 1], pp[(long)(c + 1) * (D + 2) + 2 + d], n1);
            n2 = fmaf(wts[c + 2], pp[(long)(c + 2) * (D + 2) + 2 + d], n2);
            n3 = fmaf(wts[c + 3], pp[(long)(c + 3) * (D + 2) + 2 + d], n3);
        }
        for (; c < n_split; ++c) n0 = fmaf(wts[c], pp[(long)c * (D + 2) + 2 + d], n0);
        out[bj * D + d] = ((n0 + n1) + (n2 + n3)) * rden;
    }
}

template <int R, int DH, int NHW, bool INT4>
void launch_rope(RopeArgs a, hipStream_t st) {
    a.n_groups = a.n_split * a.U * a.B;
    const int slots = (a.n_groups + 7) / 8;
    hipLaunchKernelGGL((rope_decode<R, DH, NHW, INT4>), dim3(slots * 8 * (a.NH / NHW)), dim3(256), 0, st, a);
}
template <int R, int NH, bool INT4>
void launch_absorb(const AbsorbArgs& a, int B, hipStream_t st) {
    hipLaunchKernelGGL((absorbed_decode<R, NH, INT4>), dim3(a.n_split, a.U, B), dim3(256), 0, st, a);
}

}  // namespace

void launch_merge(const float* part, float* out, int BH, int n_split, int D, hipStream_t st);

// Supported shapes: (rank, head_dim, heads per unit) instantiated below.
bool latent_shape_supported(int mode, const LatentGeom& g) {
    const int nh = g.s * g.gq;
    if (mode == LRKV_MODE_ROPE_RECON) {
        return (g.r == 32 && g.dh == 64 && nh == 2) || (g.r == 256 && g.dh == 128 && nh == 4) ||
               (g.r == 64 && g.dh == 128 && nh == 4) || (g.r == 64 && g.dh == 64 && nh == 2) ||
               (g.r == 128 && g.dh == 128 && nh == 4);
    }
    return (g.r == 32 || g.r == 64 || g.r == 128 || g.r == 256) && (nh == 2 || nh == 4);
}

int32_t launch_decode_latent(int mode, int phases, const lrkv_latent_cache* c, const float* q,
                             const half_t* bk, const int32_t* q_pos, float sm_scale, float* out,
                             void* ws, const LatentWorkspace& w, hipStream_t st) {
    const LatentGeom g = latent_geom(c);
    const int nh = g.s * g.gq;
    const bool int4 = g.fmt == LRKV_FMT_INT4_G32;
    char* base = (char*)ws;
    float* part = (float*)(base + w.part_off);
    if (mode == LRKV_MODE_ROPE_RECON && (phases & kPhasePrepare)) {
        half_t* qp = (half_t*)(base + w.qp_off);
        float* qs = (float*)(base + w.qs_off);
        hipLaunchKernelGGL(rope_qprep, dim3(g.B * g.U, g.dh / 8), dim3(256), 0, st, q, bk, qp, qs,
                           g.U, g.s, g.gq, g.dh, g.r, sm_scale * kLog2e);
    }
    if (mode == LRKV_MODE_ROPE_RECON && (phases & kPhasePartials)) {
        const half_t* qp = (const half_t*)(base + w.qp_off);
        const float* qs = (const float*)(base + w.qs_off);
        RopeArgs a{c->hk, c->hv, (const half_t*)c->sk, (const half_t*)c->sv, c->lens, q_pos, qp, qs,
                   part, g.B, g.U, nh, g.cap, w.n_split, w.chunk, 0, (double)g.theta};
        // heads per workgroup: two for rank 256 (register budget of two resident
        // workgroups per CU), all of the unit's heads otherwise
#define LRKV_ROPE(R_, DH_, NH_, NHW16_, NHW4_)                                               \
    if (g.r == R_ && g.dh == DH_ && nh == NH_) {                                            \
        if (int4) launch_rope<R_, DH_, NHW4_, true>(a, st);                                  \
        else launch_rope<R_, DH_, NHW16_, false>(a, st);                                     \
    } else
        LRKV_ROPE(32, 64, 2, 2, 2) LRKV_ROPE(64, 64, 2, 2, 2) LRKV_ROPE(256, 128, 4, 2, 1)
        LRKV_ROPE(64, 128, 4, 4, 4) LRKV_ROPE(128, 128, 4, 2, 2) { return LRKV_ERR_UNSUPPORTED; }
#undef LRKV_ROPE
    } else if (mode == LRKV_MODE_ABSORBED && (phases & kPhasePartials)) {
        AbsorbArgs a{c->hk, c->hv, (const half_t*)c->sk, (const half_t*)c->sv, c->lens, q, part,
                     g.U, g.cap, w.n_split, w.chunk, sm_scale * kLog2e};
#define LRKV_ABS(R_, NH_)                                                                    \
    if (g.r == R_ && nh == NH_) {                                                            \
        if (int4) launch_absorb<R_, NH_, true>(a, g.B, st);                                  \
        else launch_absorb<R_, NH_, false>(a, g.B, st);                                      \
    } else
        LRKV_ABS(32, 2) LRKV_ABS(64, 2) LRKV_ABS(128, 2) LRKV_ABS(256, 2) LRKV_ABS(32, 4)
        LRKV_ABS(64, 4) LRKV_ABS(128, 4) LRKV_ABS(256, 4) { return LRKV_ERR_UNSUPPORTED; }
#undef LRKV_ABS
    }
    if (phases & kPhaseMerge) launch_merge(part, out, g.B * g.Hq, w.n_split, g.r, st);
    return last_launch_status();
}

void launch_merge(const float* part, float* out, int BH, int n_split, int D, hipStream_t st) {
    hipLaunchKernelGGL(merge_splits, dim3(BH), dim3(256), 0, st, part, out, n_split, D);
}

}  // namespace lrkv
