// Chunked-prefill attention over a Palu latent cache, reconstruct-with-RoPE path
// (Palu digest, Method details: K = H^k B^k rebuilt on chip, RoPE at each token's
// position, latent-space output o = p H^v). A chunk of M new tokens has been
// appended; query m of sequence b sits at position p0[b] + m and attends
// causally, to tokens 0 .. p0[b] + m.
//
// With many queries per token the reconstruction is shared by all of them, so
// it is done as a GEMM per 32-token key tile (no query-rotated basis): one
// workgroup of 8 waves (four producers, four consumers, see prefill_attn) per
// (sequence, unit, KV head of the unit, block of 128 query rows, key split), a
// query row being one (token, query head) pair of that KV head; the splits'
// (max, sum, output) states are combined by a split-K merge. Per key tile:
//   K^T [dim][token] = B^T H^T   32x32x16 MFMA, producer p owning dims
//                                16 p .. 16 p + 15 and their RoPE partners
//                                64 + 16 p .. (B^T fragments in registers), so a
//                                lane holds both halves of each rotated pair;
//   RoPE at each token's position in registers, (cos, sin) = tile start x
//   in-tile offset (both fp64-reduced by the prepare kernel); K written to LDS
//   in fp16 (queries too: the fp16 rounding of p for the value product already
//   bounds the output error, and splitting K and q into hi + lo pairs was
//   measured to change it by less than 15%);
//   S^T [token][row] = K Q^T     16x16x32 MFMA, consumer w owning 32 query rows,
//                                rows of K permuted so that a lane's output is 8
//                                consecutive tokens of one query row;
//   causal mask, online softmax (log2 domain; queries pre-scaled);
//   O^T [dim][row] += V^T P^T    16x16x32 MFMA over the dim-major value block.
// Key tiles go buffer->LDS two tiles ahead of their reconstruction, value tiles
// one tile ahead of their product; one barrier per tile.
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

// One workgroup of 8 waves per (sequence, unit, KV head of the unit, block of 128
// query rows, key split); the key tiles of split sp are [sp tps, (sp + 1) tps) up
// to the block's causal end. Waves 4..7 (producers) load the latent tiles and
// rebuild the rotated keys of tile k into LDS while waves 0..3 (consumers) run
// scores, softmax and values of tile k - 1: one barrier per tile, and each SIMD
// holds one wave of each role, so one's MFMAs run under the other's vector work.
// Consumer wave w owns query rows 32 w .. 32 w + 31 as two 16-row blocks, which
// share every K and V fragment it reads; producer wave p owns dims
// 16 p .. 16 p + 15 and their RoPE partners 64 + 16 p .., loads key rows
// 8 p .. 8 p + 7 and value dims 64 p .. 64 p + 63 of each tile.
// LDS: keys three tiles deep (tile k read, k + 1 landed, k + 2 landing), values
// three deep (tile k - 1 read, k landed, k + 1 landing), rotated K two deep.
template <int R>
__global__ __launch_bounds__(512, 1) void prefill_attn(const PrefillArgs a) {
    constexpr int DH = 128, KS = R / 16, NDB = R / 16, NRB = 2;
    static_assert(R == 256, "prefill kernel covers rank 256");
    __shared__ __attribute__((aligned(1024))) half_t htile[3][32 * R];    // H^k [token][rank], chunks swizzled
    __shared__ __attribute__((aligned(1024))) half_t vtile[3][R * 32];    // H^v [rank][token], chunks swizzled
    __shared__ __attribute__((aligned(16))) half_t krot[2][32 * DH];      // K [token][dim], chunks swizzled
    __shared__ float2 tokb[DH / 2][32];                                   // (cos, sin)(tau theta_f), tau < 32

    const int tid = threadIdx.x, wid = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const bool producer = wid >= 4;
    const int wv = wid & 3;
    const int c = l & 15, g = l >> 4;
    // Logical block = (sequence, unit, split, KV head, row block), row block
    // fastest. Workgroups go to the 8 XCDs in turn, so consecutive logical blocks
    // are spread back onto one XCD: the s x n_qb workgroups that read the same
    // (unit, split) latents then share that XCD's L2 (one HBM read instead of one
    // per XCD they were spread over).
    int blk;
    {
        const int nb = gridDim.x, per = nb / 8, rem = nb % 8, x = blockIdx.x % 8, j = blockIdx.x / 8;
        blk = x < rem ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
    }
    const int qb = blk % a.n_qb;
    blk /= a.n_qb;
    const int w = blk % a.s;
    blk /= a.s;
    const int sp = blk % a.n_split;
    blk /= a.n_split;
    const int u = blk % a.U, b = blk / a.U;
    if (b >= a.B) return;
    const int Hq = a.U * a.s * a.gq;
    const int len = min(a.lens[b], a.cap);
    const int rows = a.M * a.gq;
    const int row0 = qb * 128;
    if (len <= 0 || row0 >= rows) return;
    const int m_last = (min(rows, row0 + 128) - 1) / a.gq;
    const int n_t = min(a.n_tiles, qpos(a.p0, a.lens, b, m_last) / 32 + 1);
    const int t_beg = sp * a.tps, t_end = min(n_t, t_beg + a.tps);

    // the consumer lane's query rows (column c of the wave's two score blocks)
    int m_row[NRB], j_row[NRB], pos[NRB];
    bool row_ok[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        const int rho = row0 + 32 * wv + 16 * rb + c;
        row_ok[rb] = !producer && rho < rows;
        m_row[rb] = row_ok[rb] ? rho / a.gq : 0;
        j_row[rb] = (u * a.s + w) * a.gq + (row_ok[rb] ? rho % a.gq : 0);
        pos[rb] = row_ok[rb] ? qpos(a.p0, a.lens, b, m_row[rb]) : -1;
    }
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

    // in-tile offsets (cos, sin)(tau theta_f) to LDS, frequency-major (the 32 lanes
    // of a frequency read 32 consecutive entries)
    for (int e = tid; e < 32 * (DH / 2); e += 512)
        tokb[e % (DH / 2)][e / (DH / 2)] = a.ang[(long)a.n_tiles * (DH / 2) + e];
    const int n = t_end - t_beg;

    if (producer) {
        const long bu = (long)b * a.U + u;
        const half_t* hk = a.hk + bu * a.cap * R;
        const half_t* hv = a.hv + bu * a.cap * R;
        auto vswz = [](int d) { return (((d >> 1) ^ (d >> 3)) & 1) | (((d >> 2) & 1) << 1); };
        const uint32_t kx = 512u * (l >> 5) + 16u * ((l & 31) ^ (l >> 5));
        const uint32_t vx = 16u * (l ^ vswz(l >> 2));
        // four loads each; past t_end the resource is empty (the loads read zero),
        // which keeps the count per iteration fixed at eight
        auto issue_keys = [&](int t, int buf) {
            const int r0 = 32 * t + 8 * wv;
            const uint32_t bytes = t < t_end ? (uint32_t)max(0, len - r0) * (R * 2) : 0u;
            const int32x4 kr = make_rsrc(hk + (long)min(r0, a.cap) * R, bytes);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                buf_dma16(kr, (kx ^ (16u * (8 * (wv & 1) + 2 * q))) + 1024u * q, htile[buf] + (8 * wv + 2 * q) * R);
        };
        auto issue_values = [&](int t, int buf) {
            const int32x4 vr = make_rsrc(hv + (long)min(t, a.cap / 32) * R * 32 + 4 * wv * 512,
                                         t < t_end ? 4096u : 0u);
#pragma unroll
            for (int q = 0; q < 4; ++q) buf_dma16(vr, vx + 1024u * q, vtile[buf] + (4 * wv + q) * 512);
        };
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
        // the lane's token is tau = l % 32 and its eight frequencies
        // f_i = 16 wv + 8 (i / 4) + 4 (l / 32) + i % 4
        auto freq = [&](int i) { return 16 * wv + 8 * (i >> 2) + 4 * (l >> 5) + (i & 3); };
        // key fragment of the reconstruction (B operand): token l % 32, ranks 16 ks + 8 (l/32)
        auto koff = [&](int ks) { return (l & 31) * R + 8 * ((2 * (ks & 7) + (l >> 5)) ^ (l & 15)) + 128 * (ks >> 3); };
        // (cos, sin) of the tile start for the lane's frequencies, loaded one tile ahead
        float2 st[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) st[i] = a.ang[(long)t_beg * (DH / 2) + freq(i)];

        issue_keys(t_beg, 0);
        issue_keys(t_beg + 1, 1);
        issue_values(t_beg, 0);
        // keys of t_beg complete: the eight loads issued after them may be in flight
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        __syncthreads();
        for (int k = 0; k <= n; ++k) {
            if (k < n) {
                // ---- K^T of tile t_beg + k for the wave's 32 dims, RoPE, K to LDS
                const half_t* ht = htile[k % 3];
                floatx16 acc = floatx16{};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) acc = mfma32(bf[ks], lds8(ht + koff(ks)), acc);
                const int tl = l & 31;
                half_t* kr = krot[k & 1];
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
                        lh[e] = (half_t)(lo * cc - hi * ss);
                        hh[e] = (half_t)(hi * cc + lo * ss);
                    }
                    // dims 16 wv + 8 gi + 4 (l/32) + e (chunk 2 wv + gi) and their partners (+64)
                    const int q_lo = (2 * wv + gi) ^ (tl & 15), q_hi = (8 + 2 * wv + gi) ^ (tl & 15);
                    *reinterpret_cast<half4*>(&kr[tl * DH + 8 * q_lo + 4 * (l >> 5)]) = half4{lh[0], lh[1], lh[2], lh[3]};
                    *reinterpret_cast<half4*>(&kr[tl * DH + 8 * q_hi + 4 * (l >> 5)]) = half4{hh[0], hh[1], hh[2], hh[3]};
                }
                if (k + 1 < n) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) st[i] = a.ang[(long)(t_beg + k + 1) * (DH / 2) + freq(i)];
                }
            }
            // every LDS read of this iteration done before the DMA may reuse a buffer
            // (the key buffer taken here was last read in iteration k - 1)
            issue_keys(t_beg + k + 2, (k + 2) % 3);
            issue_values(t_beg + k + 1, (k + 1) % 3);
            // what the next iteration reads (keys of tile k + 1, values of tile k) has
            // landed: only this iteration's eight loads may still be in flight
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            __syncthreads();
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }

    // ---- consumers
    // queries of the lane's rows, dims 32 ks + 8 g + e, in fp16
    half8 qh[NRB][4];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        const float* qs = a.qr + ((long)(b * a.M + m_row[rb]) * Hq + j_row[rb]) * DH;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) qh[rb][ks][e] = (half_t)(row_ok[rb] ? qs[32 * ks + 8 * g + e] : 0.0f);
    }
    // the wave's smallest row position (-1 if it holds a row past the chunk): key
    // tiles ending at or before it are visible to all of the wave's rows
    int pos_min = min(pos[0], pos[1]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) pos_min = min(pos_min, __shfl_xor(pos_min, o, kWave));
    pos_min = __builtin_amdgcn_readfirstlane(pos_min);
    auto vswz = [](int d) { return (((d >> 1) ^ (d >> 3)) & 1) | (((d >> 2) & 1) << 1); };
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
    __syncthreads();
    __syncthreads();                          // iteration 0: the producers rebuild the first tile
    for (int k = 1; k <= n; ++k) {
        const int t0 = 32 * (t_beg + k - 1);
        const half_t* kr = krot[(k - 1) & 1];

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
                kh[mb] = lds8(&kr[tk * DH + 8 * ((4 * ks + g) ^ (tk & 15))]);
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
            const half_t* vt = vtile[(k - 1) % 3] + vro;
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
        __syncthreads();
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

void launch_merge_rows(const float* part, float* out, int BH, int n_split, int D, hipStream_t st);

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
    hipLaunchKernelGGL(prefill_attn<256>, dim3((unsigned)blocks), dim3(512), 0, st, a);
    launch_merge_rows(part, out, c->batch * M * Hq, n_split, R, st);
    return last_launch_status();
}

}  // namespace lrkv
