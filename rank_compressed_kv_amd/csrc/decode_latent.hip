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
    const float* qs;      // [B][Hq] 2^-e of that scaling
    float* part;          // [B][Hq][n_split][R + 2]
    int U, cap, n_split, chunk;
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
// One block per (b, j): Q'[f][k] for f < DH, k < R, scaled by sm_scale*log2(e)*2^e
// with 2^e chosen so that max |Q'| lands in [2^14, 2^15) (fp16 range).
__global__ void rope_qprep(const float* __restrict__ q, const half_t* __restrict__ bk,
                           half_t* __restrict__ qp, float* __restrict__ qs, int Hq, int s, int gq,
                           int DH, int R, float scale) {
    const int j = blockIdx.x % Hq;
    const int b = blockIdx.x / Hq;
    const int kvh = j / gq, u = kvh / s, w = kvh % s;
    const int half = DH / 2;
    const int ldb = s * DH;
    const half_t* B = bk + (size_t)u * R * ldb + w * DH;
    const float* qv = q + ((size_t)b * Hq + j) * DH;
    __shared__ float red[256];
    float mx = 0.0f;
    const int n = DH * R;
    for (int e = threadIdx.x; e < n; e += blockDim.x) {
        const int f = e / R, k = e % R, i = f / 2;
        const float b0 = (float)B[(size_t)k * ldb + i], b1 = (float)B[(size_t)k * ldb + i + half];
        const float v = (f & 1) ? fmaf(qv[i + half], b0, -qv[i] * b1) : fmaf(qv[i], b0, qv[i + half] * b1);
        mx = fmaxf(mx, fabsf(v * scale));
    }
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int o = blockDim.x / 2; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
        __syncthreads();
    }
    mx = red[0];
    const int ex = (mx > 0.0f && isfinite(mx)) ? 14 - ilogbf(mx) : 0;
    const float mul = ldexpf(scale, ex);
    half_t* out = qp + ((size_t)b * Hq + j) * n;
    for (int e = threadIdx.x; e < n; e += blockDim.x) {
        const int f = e / R, k = e % R, i = f / 2;
        const float b0 = (float)B[(size_t)k * ldb + i], b1 = (float)B[(size_t)k * ldb + i + half];
        const float v = (f & 1) ? fmaf(qv[i + half], b0, -qv[i] * b1) : fmaf(qv[i], b0, qv[i + half] * b1);
        out[e] = (half_t)(v * mul);
    }
    if (threadIdx.x == 0) qs[(size_t)b * Hq + j] = ldexpf(1.0f, -ex);
}

// ------------------------------------------------------------------------ tile staging
// Key tile of 32 tokens as fp16 rows in LDS (int4 codes are dequantised here:
// code * scale rounded to fp16). Rows at or past t_end are zero.
template <int R, bool INT4>
struct KStage {
    static constexpr int NV = 32 * R / 8;                 // 8-dim items per tile
    static constexpr int PER = (NV + 255) / 256;
    uint4 v[PER];

    __device__ __forceinline__ void load(const void* hk, const half_t* sk, long row0, int t0,
                                         int t_end, int tid) {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int item = tid + 256 * k;
            const int row = item / (R / 8), c8 = item % (R / 8);
            v[k] = make_uint4(0, 0, 0, 0);
            if (item < NV && t0 + row < t_end) {
                const long tok = row0 + t0 + row;
                if constexpr (!INT4) {
                    v[k] = *reinterpret_cast<const uint4*>((const half_t*)hk + tok * R + c8 * 8);
                } else {
                    const uint32_t code = *reinterpret_cast<const uint32_t*>((const uint8_t*)hk + tok * (R / 2) + c8 * 4);
                    const float sc = (float)sk[tok * (R / 32) + c8 / 4];
                    half8 h;
#pragma unroll
                    for (int e = 0; e < 8; ++e) h[e] = (half_t)((float)nibble(code, e) * sc);
                    v[k] = *reinterpret_cast<uint4*>(&h);
                }
            }
        }
    }
    template <int LDK>
    __device__ __forceinline__ void store(half_t (*tile)[LDK], int tid) const {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int item = tid + 256 * k;
            if (item < NV) {
                const int row = item / (R / 8), c8 = item % (R / 8);
                *reinterpret_cast<uint4*>(&tile[row][c8 * 8]) = v[k];
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
// to fp32 rounding: the angle is reduced in fp64 before the fp64 sincos.
__device__ __forceinline__ double lane_rho(int k, int w, int lane, int dh, double log2_theta) {
    const int fr = 16 * w + 4 * (k >> 1) + 2 * (lane >> 5) + (k & 1);
    return log2_theta != 0.0 ? exp2(-2.0 * fr / dh * log2_theta) / kTwoPi : 0.0;
}
__device__ __noinline__ void anchor_angles(float* c, float* s, int w, int lane, int dh,
                                           double log2_theta, long dt0) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        double rev = (double)dt0 * lane_rho(k, w, lane, dh, log2_theta);
        rev -= rint(rev);
        double sd, cd;
        sincos(kTwoPi * rev, &sd, &cd);
        c[k] = (float)cd;
        s[k] = (float)sd;
    }
}

// ------------------------------------------------------------------------ RoPE decode
template <int R, int DH, int NH, bool INT4>
__global__ __launch_bounds__(256, 1) void rope_decode(const RopeArgs p) {
    constexpr int KS = R / 16;                 // K steps of the score MFMA
    constexpr int MT = DH / 32;                // feature M-tiles per head (waves that score)
    constexpr int VM = R / 16;                 // 16-dim M-tiles of the value MFMA
    constexpr int VMW = (VM + 3) / 4;          // value M-tiles per wave
    constexpr int LDK = R + 8;
    static_assert(MT >= 1 && MT <= 4, "head_dim must be 32..128");
    __shared__ half_t ktile[2][32][LDK];
    __shared__ float spart[4][32][NH];
    __shared__ half_t pbuf[4][NH][32];
    __shared__ float step[4][64][8][2];

    const int split = blockIdx.x, u = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int Hq = p.U * NH, j0 = u * NH;
    const int len = min(p.lens[b], p.cap);        // never read past the capacity
    const int t_begin = split * p.chunk;
    const int t_end = min(len, t_begin + p.chunk);
    const long bu = (long)b * p.U + u;
    float* part = p.part + ((long)(b * Hq + j0) * p.n_split + split) * (R + 2);
    const long hstride = (long)p.n_split * (R + 2);

    if (t_begin >= t_end) {                    // empty chunk
        for (int e = tid; e < NH * (R + 2); e += 256) {
            const int h = e / (R + 2), c = e % (R + 2);
            part[h * hstride + c] = c == 0 ? -INFINITY : 0.0f;
        }
        return;
    }

    // rotated-basis query fragments and per-head inverse scales
    half8 afrag[NH][KS];
    float inv[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        inv[h] = p.qs[(long)b * Hq + j0 + h];
        if (w < MT) {
            const half_t* src = p.qp + (((long)b * Hq + j0 + h) * DH + 32 * w + (l & 31)) * R + 8 * (l >> 5);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) afrag[h][kk] = *reinterpret_cast<const half8*>(src + 16 * kk);
        }
    }

    // this lane's 8 frequencies: feature f = 32w + 8i + 4(l/32) + e has frequency
    // f/2 and is its cos (e even) or sin (e odd) coefficient
    float cs[8], sn[8];
    const int qpos = p.q_pos ? p.q_pos[b] : len - 1;
    const double l2t = p.theta > 0.0 ? log2(p.theta) : 0.0;
    {
        float c32[8], s32[8];                  // rotation by 32 positions per tile
        anchor_angles(c32, s32, w, l, DH, l2t, 32);
        if (l < 64) {
#pragma unroll
            for (int k = 0; k < 8; ++k) { step[w][l][k][0] = c32[k]; step[w][l][k][1] = s32[k]; }
        }
    }
    anchor_angles(cs, sn, w, l, DH, l2t, (long)t_begin + (l & 31) - qpos);

    float m_run[NH], l_run[NH];
    floatx4 accv[VMW];
#pragma unroll
    for (int h = 0; h < NH; ++h) { m_run[h] = -INFINITY; l_run[h] = 0.0f; }
#pragma unroll
    for (int v = 0; v < VMW; ++v) accv[v] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int n_tiles = (t_end - t_begin + 31) / 32;
    KStage<R, INT4> stage;
    stage.load(p.hk, p.sk, bu * p.cap, t_begin, t_end, tid);
    stage.template store<LDK>(ktile[0], tid);
    __syncthreads();

    for (int it = 0; it < n_tiles; ++it) {
        const int t0 = t_begin + 32 * it;
        const int buf = it & 1;
        if (it + 1 < n_tiles) stage.load(p.hk, p.sk, bu * p.cap, t0 + 32, t_end, tid);
        // value fragments of this tile (used after the softmax)
        half8 vfr[VMW];
        const long blk_base = bu * (p.cap / kTile) + t0 / kTile;
#pragma unroll
        for (int v = 0; v < VMW; ++v) {
            const int mv = w * VMW + v;
            if (mv < VM) vfr[v] = load_vfrag<R, INT4>(p.hv, p.sv, blk_base, mv, l, t0, t_end);
        }

        // ---- scores in the rotated basis, then the RoPE combination
        if (w < MT) {
            floatx16 acc[NH];
#pragma unroll
            for (int h = 0; h < NH; ++h) acc[h] = floatx16{};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const half8 bf = *reinterpret_cast<const half8*>(&ktile[buf][l & 31][16 * kk + 8 * (l >> 5)]);
#pragma unroll
                for (int h = 0; h < NH; ++h) acc[h] = mfma32(afrag[h][kk], bf, acc[h]);
            }
#pragma unroll
            for (int h = 0; h < NH; ++h) {
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
        // advance the angles by 32 positions; re-anchor exactly every 64 tiles
        if ((it & 63) == 63) {
            anchor_angles(cs, sn, w, l, DH, l2t, (long)t0 + 32 + (l & 31) - qpos);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float cst = step[w][l][k][0], snt = step[w][l][k][1];
                const float c2 = fmaf(cs[k], cst, -sn[k] * snt);
                const float s2 = fmaf(sn[k], cst, cs[k] * snt);
                cs[k] = c2;
                sn[k] = s2;
            }
        }
        __syncthreads();

        // ---- online softmax (every wave, every head; log2 domain)
        const int tok = l & 31;
        const bool valid = t0 + tok < t_end;
        float alpha[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            float sc = 0.0f;
#pragma unroll
            for (int ww = 0; ww < MT; ++ww) sc += spart[ww][tok][h];
            sc = valid ? sc * inv[h] : -INFINITY;
            const float mt = reduce_max_width<32>(sc);
            const float mn = fmaxf(m_run[h], mt);
            alpha[h] = exp2f(m_run[h] - mn);
            const float pv = valid ? exp2f(sc - mn) : 0.0f;
            l_run[h] = fmaf(l_run[h], alpha[h], reduce_sum_width<32>(pv));
            m_run[h] = mn;
            if (l < 32) pbuf[w][h][tok] = (half_t)pv;
        }
        __builtin_amdgcn_wave_barrier();

        // ---- values: acc[dim][head] += V^T p
        const int hn = l & 15;
        float a_hn = 1.0f;
#pragma unroll
        for (int h = 0; h < NH; ++h) if (hn == h) a_hn = alpha[h];
        half8 pf;
        if (hn < NH) {
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
        if (it + 1 < n_tiles) stage.template store<LDK>(ktile[buf ^ 1], tid);
        __syncthreads();
    }

    // ---- chunk partials: (m, l) per head, then acc[dim] per head
    if (tid < NH) {
        part[tid * hstride + 0] = m_run[tid];
        part[tid * hstride + 1] = l_run[tid];
    }
    const int hn = l & 15;
    if (hn < NH) {
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
// n_split chunks; empty chunks (m = -inf) contribute nothing.
__global__ void merge_splits(const float* __restrict__ part, float* __restrict__ out, int n_split,
                             int D) {
    const long bj = blockIdx.x;
    const float* pp = part + bj * n_split * (D + 2);
    float mx = -INFINITY;
    for (int c = 0; c < n_split; ++c) mx = fmaxf(mx, pp[(long)c * (D + 2)]);
    float den = 0.0f;
    for (int c = 0; c < n_split; ++c) {
        const float m = pp[(long)c * (D + 2)];
        if (m != -INFINITY) den = fmaf(exp2f(m - mx), pp[(long)c * (D + 2) + 1], den);
    }
    const float rden = 1.0f / den;
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float num = 0.0f;
        for (int c = 0; c < n_split; ++c) {
            const float m = pp[(long)c * (D + 2)];
            if (m != -INFINITY) num = fmaf(exp2f(m - mx), pp[(long)c * (D + 2) + 2 + d], num);
        }
        out[bj * D + d] = num * rden;
    }
}

template <int R, int DH, int NH, bool INT4>
void launch_rope(const RopeArgs& a, int B, hipStream_t st) {
    hipLaunchKernelGGL((rope_decode<R, DH, NH, INT4>), dim3(a.n_split, a.U, B), dim3(256), 0, st, a);
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

int32_t launch_decode_latent(int mode, const lrkv_latent_cache* c, const float* q,
                             const half_t* bk, const int32_t* q_pos, float sm_scale, float* out,
                             void* ws, const LatentWorkspace& w, hipStream_t st) {
    const LatentGeom g = latent_geom(c);
    const int nh = g.s * g.gq;
    const bool int4 = g.fmt == LRKV_FMT_INT4_G32;
    char* base = (char*)ws;
    float* part = (float*)(base + w.part_off);
    if (mode == LRKV_MODE_ROPE_RECON) {
        half_t* qp = (half_t*)(base + w.qp_off);
        float* qs = (float*)(base + w.qs_off);
        hipLaunchKernelGGL(rope_qprep, dim3(g.B * g.Hq), dim3(256), 0, st, q, bk, qp, qs, g.Hq, g.s,
                           g.gq, g.dh, g.r, sm_scale * kLog2e);
        RopeArgs a{c->hk, c->hv, (const half_t*)c->sk, (const half_t*)c->sv, c->lens, q_pos, qp, qs,
                   part, g.U, g.cap, w.n_split, w.chunk, (double)g.theta};
#define LRKV_ROPE(R_, DH_, NH_)                                                              \
    if (g.r == R_ && g.dh == DH_ && nh == NH_) {                                            \
        if (int4) launch_rope<R_, DH_, NH_, true>(a, g.B, st);                               \
        else launch_rope<R_, DH_, NH_, false>(a, g.B, st);                                   \
    } else
        LRKV_ROPE(32, 64, 2) LRKV_ROPE(64, 64, 2) LRKV_ROPE(256, 128, 4) LRKV_ROPE(64, 128, 4)
        LRKV_ROPE(128, 128, 4) { return LRKV_ERR_UNSUPPORTED; }
#undef LRKV_ROPE
    } else {
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
    launch_merge(part, out, g.B * g.Hq, w.n_split, g.r, st);
    return last_launch_status();
}

void launch_merge(const float* part, float* out, int BH, int n_split, int D, hipStream_t st) {
    hipLaunchKernelGGL(merge_splits, dim3(BH), dim3(256), 0, st, part, out, n_split, D);
}

}  // namespace lrkv
