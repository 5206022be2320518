// Chunked-prefill attention over a Palu latent cache, reconstruct-with-RoPE path
// (Palu digest, Method details: K = H^k B^k rebuilt on chip, RoPE at each token's
// position, latent-space output o = p H^v). A chunk of M new tokens has been
// appended; query m of sequence b sits at position p0[b] + m and attends
// causally, to tokens 0 .. p0[b] + m.
//
// With many queries per token the reconstruction is shared by all of them, so
// it is done as a GEMM per 32-token key tile (no query-rotated basis): one
// workgroup of 4 waves per (sequence, unit, KV head of the unit, block of 128
// query rows, key split), a query row being one (token, query head) pair of that
// KV head; the splits' (max, sum, output) states are combined by the split-K
// merge of the decode path. Per key tile:
//   K^T [dim][token] = B^T H^T   32x32x16 MFMA, wave w owning dims
//                                16 w .. 16 w + 15 and their RoPE partners
//                                64 + 16 w .. (B^T fragments in registers), so a
//                                lane holds both halves of each rotated pair;
//   RoPE at each token's position in registers, (cos, sin) = tile start x
//   in-tile offset (both fp64-reduced by the prepare kernel); K written to LDS
//   in fp16 (queries too: the fp16 rounding of p for the value product already
//   bounds the output error, and splitting K and q into hi + lo pairs was
//   measured to change it by less than 15%);
//   S^T [token][row] = K Q^T     16x16x32 MFMA, wave w owning 32 query rows,
//                                rows of K permuted so that a lane's output is 8
//                                consecutive tokens of one query row;
//   causal mask, online softmax (log2 domain; queries pre-scaled);
//   O^T [dim][row] += V^T P^T    16x16x32 MFMA over the dim-major value block.
// Key and value tiles go buffer->LDS, one tile ahead; two barriers per tile.
#include "tiles.h"

#include <math.h>
#include <type_traits>

namespace lrkv {
namespace {

constexpr double kTwoPiP = 6.283185307179586476925286766559;

struct PrefillPrepArgs {
    const float* q;       // [B][M][Hq][DH]
    const int32_t* p0;
    const int32_t* lens;
    float* qr;            // [B][M][Hq][DH] rotated, scaled
    float2* ang;          // [n_tiles + 32][DH/2]
    int B, M, Hq, DH, n_tiles;
    double theta;
    float scale;
};

// (cos, sin)(n theta_f), theta_f = theta^(-2f/DH), with n theta_f / 2 pi reduced
// to [-1/2, 1/2] in fp64 before the fp64 sincos
__device__ float2 angle(long n, int f, int DH, double theta) {
    const double rho = theta > 0.0 ? exp2(-2.0 * f / DH * log2(theta)) / kTwoPiP : 0.0;
    double rev = (double)n * rho;
    rev -= rint(rev);
    double sd, cd;
    sincos(kTwoPiP * rev, &sd, &cd);
    return make_float2((float)cd, (float)sd);
}

// Query position of chunk token m, clamped to the sequence's tokens.
__device__ __forceinline__ int qpos(const int32_t* p0, const int32_t* lens, int b, int m) {
    return max(0, min(p0[b] + m, lens[b] - 1));
}

__global__ __launch_bounds__(256) void prefill_prep(const PrefillPrepArgs a) {
    const int half = a.DH / 2;
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    const long n_ang = (long)(a.n_tiles + 32) * half;
    if (e < n_ang) {
        const int row = (int)(e / half), f = (int)(e % half);
        a.ang[e] = angle(row < a.n_tiles ? 32L * row : (long)(row - a.n_tiles), f, a.DH, a.theta);
        return;
    }
    const long e2 = e - n_ang;
    if (e2 >= (long)a.B * a.M * a.Hq * half) return;
    const long bmj = e2 / half;
    const int f = (int)(e2 % half);
    const int b = (int)(bmj / ((long)a.M * a.Hq)), m = (int)((bmj / a.Hq) % a.M);
    const float2 cs = angle(qpos(a.p0, a.lens, b, m), f, a.DH, a.theta);
    const float x = a.q[bmj * a.DH + f], y = a.q[bmj * a.DH + f + half];
    a.qr[bmj * a.DH + f] = (x * cs.x - y * cs.y) * a.scale;
    a.qr[bmj * a.DH + f + half] = (y * cs.x + x * cs.y) * a.scale;
}

struct PrefillArgs {
    const half_t* hk;     // [B][U][cap][R]
    const half_t* hv;     // [B][U][cap/32][R][32]
    const half_t* bk;     // [U][R][s*DH]
    const int32_t* p0;
    const int32_t* lens;
    const float* qr;      // [B][M][Hq][DH] rotated, scaled
    const float2* ang;    // [n_tiles + 32][DH/2]
    float* part;          // [B][M][Hq][n_split][R + 2]: (max, sum, unnormalised output)
    int B, U, s, gq, M, cap, n_tiles, n_qb, n_split, tps;
};

__device__ __forceinline__ half8 lds8(const half_t* p) { return *reinterpret_cast<const half8*>(p); }

// max / sum over the four lane groups of a column
__device__ __forceinline__ float col_max(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
    v = fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
    r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
    return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float col_sum(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
    v = __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
    r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
    return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

// One workgroup per (sequence, unit, KV head of the unit, block of 128 query rows,
// key split): wave w owns rows 32 w .. 32 w + 31 as two 16-row blocks, which share
// every K and V fragment the wave reads; the key tiles of split sp are
// [sp tps, (sp + 1) tps) up to the block's causal end.
template <int R>
__global__ __launch_bounds__(256, 1) void prefill_attn(const PrefillArgs a) {
    constexpr int DH = 128, KS = R / 16, NDB = R / 16, NRB = 2;
    static_assert(R == 256, "prefill kernel covers rank 256");
    __shared__ __attribute__((aligned(1024))) half_t htile[2][32 * R];    // H^k [token][rank], chunks swizzled
    __shared__ __attribute__((aligned(1024))) half_t vtile[2][R * 32];    // H^v [rank][token], chunks swizzled
    __shared__ __attribute__((aligned(16))) half_t krot[32 * DH];         // K [token][dim], chunks swizzled
    __shared__ float2 tokb[DH / 2][32];                                   // (cos, sin)(tau theta_f), tau < 32

    const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int c = l & 15, g = l >> 4;
    int blk = blockIdx.x;
    const int sp = blk % a.n_split;
    blk /= a.n_split;
    const int qb = blk % a.n_qb;
    blk /= a.n_qb;
    const int w = blk % a.s;
    blk /= a.s;
    const int u = blk % a.U, b = blk / a.U;
    if (b >= a.B) return;
    const int Hq = a.U * a.s * a.gq;
    const int len = min(a.lens[b], a.cap);
    const int rows = a.M * a.gq;
    const int row0 = qb * 128;
    if (len <= 0 || row0 >= rows) return;

    // the lane's query rows (column c of the wave's two score blocks)
    int m_row[NRB], j_row[NRB], pos[NRB];
    bool row_ok[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        const int rho = row0 + 32 * wv + 16 * rb + c;
        row_ok[rb] = rho < rows;
        m_row[rb] = row_ok[rb] ? rho / a.gq : 0;
        j_row[rb] = (u * a.s + w) * a.gq + (row_ok[rb] ? rho % a.gq : 0);
        pos[rb] = row_ok[rb] ? qpos(a.p0, a.lens, b, m_row[rb]) : -1;
    }
    // the wave's smallest row position (-1 if it holds a row past the chunk): key
    // tiles ending at or before it are visible to all of the wave's rows
    int pos_min = min(pos[0], pos[1]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) pos_min = min(pos_min, __shfl_xor(pos_min, o, kWave));
    pos_min = __builtin_amdgcn_readfirstlane(pos_min);
    const int m_last = (min(rows, row0 + 128) - 1) / a.gq;
    const int n_t = min(a.n_tiles, qpos(a.p0, a.lens, b, m_last) / 32 + 1);
    const int t_beg = sp * a.tps, t_end = min(n_t, t_beg + a.tps);

    auto part_of = [&](int rb) {
        return a.part + (((long)(b * a.M + m_row[rb]) * Hq + j_row[rb]) * a.n_split + sp) * (R + 2);
    };
    if (t_beg >= t_end) {
        // an empty split: (max, sum, output) = (-inf, 0, 0) for every row
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
            if (row_ok[rb] && g == 0) {
                float* pp = part_of(rb);
                pp[0] = -INFINITY;
                pp[1] = 0.0f;
                for (int d = 0; d < R; ++d) pp[2 + d] = 0.0f;
            }
        return;
    }

    const long bu = (long)b * a.U + u;
    const half_t* hk = a.hk + bu * a.cap * R;
    const half_t* hv = a.hv + bu * a.cap * R;
    auto vswz = [](int d) { return (((d >> 1) ^ (d >> 3)) & 1) | (((d >> 2) & 1) << 1); };
    const uint32_t kx = 512u * (l >> 5) + 16u * ((l & 31) ^ (l >> 5));
    const uint32_t vx = 16u * (l ^ vswz(l >> 2));
    // wave wv loads key rows 8 wv .. 8 wv + 7 and value dims 64 wv .. 64 wv + 63 of tile t
    auto issue = [&](int t) {
        const int t0 = 32 * t;
        const int r0 = t0 + 8 * wv;
        const int32x4 kr = make_rsrc(hk + (long)r0 * R, (uint32_t)max(0, len - r0) * (R * 2));
        const int32x4 vr = make_rsrc(hv + (long)(t0 / 32) * R * 32 + 4 * wv * 512, 4096u);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            buf_dma16(kr, (kx ^ (16u * (8 * (wv & 1) + 2 * n))) + 1024u * n, htile[t & 1] + (8 * wv + 2 * n) * R);
            buf_dma16(vr, vx + 1024u * n, vtile[t & 1] + (4 * wv + n) * 512);
        }
    };
    issue(t_beg);

    // B^T fragments: A operand of K^T = B^T H^T. Row m of the wave's 32 dims is
    // dim 16 wv + m (m < 16) or 64 + 16 wv + m - 16; K step ks covers ranks
    // 16 ks + 8 (l / 32) .. + 7.
    half8 bf[KS];
    {
        const int m = l & 31;
        const int dim = m < 16 ? 16 * wv + m : 64 + 16 * wv + (m - 16);
        const half_t* col = a.bk + (long)u * R * (a.s * DH) + w * DH + dim;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) bf[ks][e] = col[(long)(16 * ks + 8 * (l >> 5) + e) * (a.s * DH)];
    }
    // queries of the lane's rows, dims 32 ks + 8 g + e, in fp16
    half8 qh[NRB][4];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        const float* qs = a.qr + ((long)(b * a.M + m_row[rb]) * Hq + j_row[rb]) * DH;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qh[rb][ks][e] = (half_t)(row_ok[rb] ? qs[32 * ks + 8 * g + e] : 0.0f);
            }
    }
    // in-tile offsets (cos, sin)(tau theta_f) to LDS, frequency-major (the 32 lanes
    // of a frequency read 32 consecutive entries); the lane's token is tau = l % 32
    // and its eight frequencies f_i = 16 wv + 8 (i / 4) + 4 (l / 32) + i % 4
    for (int e = tid; e < 32 * (DH / 2); e += 256)
        tokb[e % (DH / 2)][e / (DH / 2)] = a.ang[(long)a.n_tiles * (DH / 2) + e];
    auto freq = [&](int i) { return 16 * wv + 8 * (i >> 2) + 4 * (l >> 5) + (i & 3); };
    // key fragment of the reconstruction (B operand): token l % 32, ranks 16 ks + 8 (l/32)
    auto koff = [&](int ks) { return (l & 31) * R + 8 * ((2 * (ks & 7) + (l >> 5)) ^ (l & 15)) + 128 * (ks >> 3); };
    const int vro = 8 * (4 * (l & 15) + ((l >> 4) ^ vswz(l & 15)));

    float m_run[NRB], l_lane[NRB];
    floatx4 o[NRB][NDB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        m_run[rb] = -INFINITY;
        l_lane[rb] = 0.0f;
#pragma unroll
        for (int d = 0; d < NDB; ++d) o[rb][d] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    // (cos, sin) of the tile start for the lane's frequencies: loaded one tile ahead
    float2 st[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) st[i] = a.ang[(long)t_beg * (DH / 2) + freq(i)];
    // B^T fragments and queries stay in the AGPRs for the whole loop, where the
    // MFMAs read them in place (the accumulators and the vector work use the
    // arithmetic registers); pinned once every load above has been issued
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+a"(bf[ks]));
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+a"(qh[rb][ks]));
    for (int t = t_beg; t < t_end; ++t) {
        const int t0 = 32 * t;
        // vmcnt(0) as a builtin: the compiler sees it, so it inserts no later wait for
        // its own loads (which would also stall on the next tile's loads below)
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();                      // tile t in LDS; tile t-1 fully consumed
        if (t + 1 < t_end) issue(t + 1);

        // ---- K^T for the wave's 32 dims, RoPE, K to LDS
        {
            const half_t* ht = htile[t & 1];
            floatx16 acc = floatx16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc = mfma32(bf[ks], lds8(ht + koff(ks)), acc);
            const int tl = l & 31;
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
                half_t lh[4], hh[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * gi + e;
                    const float2 tk = tokb[freq(i)][tl];
                    const float cc = st[i].x * tk.x - st[i].y * tk.y;
                    const float ss = st[i].x * tk.y + st[i].y * tk.x;
                    const float lo = acc[i], hi = acc[i + 8];
                    const float lo2 = lo * cc - hi * ss, hi2 = hi * cc + lo * ss;
                    lh[e] = (half_t)lo2;
                    hh[e] = (half_t)hi2;
                }
                // dims 16 wv + 8 gi + 4 (l/32) + e (chunk 2 wv + gi) and their partners (+64)
                const int q_lo = (2 * wv + gi) ^ (tl & 15), q_hi = (8 + 2 * wv + gi) ^ (tl & 15);
                const int o_lo = tl * DH + 8 * q_lo + 4 * (l >> 5), o_hi = tl * DH + 8 * q_hi + 4 * (l >> 5);
                *reinterpret_cast<half4*>(&krot[o_lo]) = half4{lh[0], lh[1], lh[2], lh[3]};
                *reinterpret_cast<half4*>(&krot[o_hi]) = half4{hh[0], hh[1], hh[2], hh[3]};
            }
        }
        if (t + 1 < t_end) {
#pragma unroll
            for (int i = 0; i < 8; ++i) st[i] = a.ang[(long)(t + 1) * (DH / 2) + freq(i)];
        }
        __syncthreads();                      // K of tile t complete

        // ---- S^T [token][row] for both row blocks: block mb row m is token
        // 8 (m/4) + 4 mb + m % 4; four chains
        floatx4 S[NRB][2];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) S[rb][mb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            half8 kh[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const int tk = 8 * (c >> 2) + 4 * mb + (c & 3);
                kh[mb] = lds8(&krot[tk * DH + 8 * ((4 * ks + g) ^ (tk & 15))]);
            }
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) S[rb][mb] = mfma16(kh[mb], qh[rb][ks], S[rb][mb]);
        }

        // ---- causal mask and online softmax per row block; lane (c, g): row c at
        // tokens t0 + 8 g + jj, jj = 4 mb + i. A tile that every row of the wave
        // sees whole (FULL) needs no mask, and its maxima are finite, so the
        // guards against -inf - -inf drop out too (exp2(-inf) is 0).
        half8 pb[NRB];
        float alpha[NRB];
        bool moved[NRB];
        auto softmax = [&](auto full_c) __attribute__((always_inline)) {
            constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                float sv[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const float v = S[rb][jj >> 2][jj & 3];
                    sv[jj] = FULL || t0 + 8 * g + jj <= pos[rb] ? v : -INFINITY;
                }
                float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                                 fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
                mx = col_max(mx);
                const float mn = fmaxf(m_run[rb], mx);
                moved[rb] = __builtin_amdgcn_ballot_w64(mn > m_run[rb]) != 0;
                alpha[rb] = !moved[rb] ? 1.0f
                          : !FULL && m_run[rb] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run[rb] - mn);
                m_run[rb] = mn;
                float psum = 0.0f;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const float pv = !FULL && sv[jj] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sv[jj] - mn);
                    psum += pv;
                    pb[rb][jj] = (half_t)pv;
                }
                l_lane[rb] = fmaf(l_lane[rb], alpha[rb], psum);
            }
        };
        if (t0 + 31 <= pos_min) softmax(std::integral_constant<bool, true>{});
        else softmax(std::integral_constant<bool, false>{});
        // the accumulators' rescale, shared by both paths (only when some row's max moved)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
            if (moved[rb]) {
#pragma unroll
                for (int d = 0; d < NDB; ++d) o[rb][d] *= alpha[rb];
            }

        // ---- O^T [dim][row] += V^T P^T (tokens past the sequence end zeroed)
        {
            const half_t* vt = vtile[t & 1] + vro;
            const bool tail = t0 + 32 > len;
            const int first = t0 + 8 * (l >> 4);
#pragma unroll
            for (int d = 0; d < NDB; ++d) {
                half8 va = lds8(vt + 512 * d);
                if (tail) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (first + e >= len) va[e] = (half_t)0.0f;
                }
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) o[rb][d] = mfma16(va, pb[rb], o[rb][d]);
            }
        }
    }

    // the split's state per row: lane (c, g) holds dims 16 d + 4 g + i of row c
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        const float lsum = col_sum(l_lane[rb]);
        if (row_ok[rb]) {
            float* pp = part_of(rb);
            if (g == 0) {
                pp[0] = m_run[rb];
                pp[1] = lsum;
            }
#pragma unroll
            for (int d = 0; d < NDB; ++d)
#pragma unroll
                for (int i = 0; i < 4; ++i) pp[2 + 16 * d + 4 * g + i] = o[rb][d][i];
        }
    }
}

}  // namespace

// Key splits: enough workgroups for about one per compute unit, at least one tile each.
static int prefill_splits(int B, int U, int s, int n_qb, int n_tiles) {
    const long groups = (long)B * U * s * n_qb;
    long n = (256 + groups - 1) / groups;
    if (n > n_tiles) n = n_tiles;
    if (n > 256) n = 256;
    return n < 1 ? 1 : (int)n;
}

size_t prefill_workspace_bytes(int B, int U, int s, int gq, int M, int DH, int R, int n_tiles) {
    const int Hq = U * s * gq, n_qb = (M * gq + 127) / 128;
    const int n_split = prefill_splits(B, U, s, n_qb, n_tiles);
    return align_up((size_t)(n_tiles + 32) * (DH / 2) * sizeof(float2), 256) +
           align_up((size_t)B * M * Hq * DH * sizeof(float), 256) +
           align_up((size_t)B * M * Hq * n_split * (R + 2) * sizeof(float), 256);
}

void launch_merge(const float* part, float* out, int BH, int n_split, int D, hipStream_t st);

int32_t launch_prefill(const lrkv_latent_cache* c, const float* q, const half_t* bk, const int32_t* p0, int M,
                       int n_tiles, float sm_scale, float* out, void* ws, hipStream_t st) {
    const int Hq = c->units * c->kv_per_unit * c->q_per_kv, DH = c->head_dim, R = c->rank;
    const int n_qb = (M * c->q_per_kv + 127) / 128;
    const int n_split = prefill_splits(c->batch, c->units, c->kv_per_unit, n_qb, n_tiles);
    const int tps = (n_tiles + n_split - 1) / n_split;
    const size_t ang_bytes = align_up((size_t)(n_tiles + 32) * (DH / 2) * sizeof(float2), 256);
    const size_t q_bytes = align_up((size_t)c->batch * M * Hq * DH * sizeof(float), 256);
    float2* ang = (float2*)ws;
    float* qr = (float*)((char*)ws + ang_bytes);
    float* part = (float*)((char*)ws + ang_bytes + q_bytes);
    PrefillPrepArgs pa{q, p0, c->lens, qr, ang, c->batch, M, Hq, DH, n_tiles, (double)c->rope_theta,
                       sm_scale * kLog2e};
    const long n_prep = (long)(n_tiles + 32) * (DH / 2) + (long)c->batch * M * Hq * (DH / 2);
    hipLaunchKernelGGL(prefill_prep, dim3((unsigned)((n_prep + 255) / 256)), dim3(256), 0, st, pa);
    PrefillArgs a{(const half_t*)c->hk, (const half_t*)c->hv, bk, p0, c->lens, qr, ang, part,
                  c->batch, c->units, c->kv_per_unit, c->q_per_kv, M, c->capacity, n_tiles, n_qb, n_split, tps};
    const long blocks = (long)c->batch * c->units * c->kv_per_unit * n_qb * n_split;
    hipLaunchKernelGGL(prefill_attn<256>, dim3((unsigned)blocks), dim3(256), 0, st, a);
    launch_merge(part, out, c->batch * M * Hq, n_split, R, st);
    return last_launch_status();
}

}  // namespace lrkv
