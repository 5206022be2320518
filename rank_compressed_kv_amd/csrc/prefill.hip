// Chunked-prefill attention over a Palu latent cache, reconstruct-with-RoPE path
// (Palu digest, Method details: K = H^k B^k rebuilt on chip, RoPE at each token's
// position, latent-space output o = p H^v). A chunk of M new tokens has been
// appended; query m of sequence b sits at position p0[b] + m and attends
// causally, to tokens 0 .. p0[b] + m.
//
// With many queries per token the reconstruction is shared by all of them, so
// it is done as a GEMM per 32-token key tile (no query-rotated basis): one
// workgroup of 4 waves per (sequence, unit, KV head of the unit, block of 64
// query rows), a query row being one (token, query head) pair of that KV head.
// Per key tile:
//   K^T [dim][token] = B^T H^T   32x32x16 MFMA, wave w owning dims
//                                16 w .. 16 w + 15 and their RoPE partners
//                                64 + 16 w .. (B^T fragments in registers), so a
//                                lane holds both halves of each rotated pair;
//   RoPE at each token's position in registers, (cos, sin) = tile start x
//   in-tile offset (both fp64-reduced by the prepare kernel); K written to LDS
//   as fp16 hi + lo;
//   S^T [token][row] = K Q^T     16x16x32 MFMA, wave w owning 16 query rows,
//                                rows of K permuted so that a lane's output is 8
//                                consecutive tokens of one query row; hi x hi,
//                                hi x lo, lo x hi;
//   causal mask, online softmax (log2 domain; queries pre-scaled);
//   O^T [dim][row] += V^T P^T    16x16x32 MFMA over the dim-major value block.
// Key and value tiles go buffer->LDS, one tile ahead; two barriers per tile.
#include "tiles.h"

#include <math.h>

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
    float* out;           // [B][M][Hq][R]
    int B, U, s, gq, M, cap, n_tiles, n_qb;
};

__device__ __forceinline__ half8 lds8(const half_t* p) { return *reinterpret_cast<const half8*>(p); }

template <int R>
__global__ __launch_bounds__(256, 1) void prefill_attn(const PrefillArgs a) {
    constexpr int DH = 128, KS = R / 16, NDB = R / 16;
    static_assert(R == 256, "prefill kernel covers rank 256");
    __shared__ __attribute__((aligned(1024))) half_t htile[2][32 * R];    // H^k [token][rank], chunks swizzled
    __shared__ __attribute__((aligned(1024))) half_t vtile[2][R * 32];    // H^v [rank][token], chunks swizzled
    __shared__ __attribute__((aligned(16))) half_t krot[2][32 * DH];      // K hi, lo [token][dim], chunks swizzled

    const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int c = l & 15, g = l >> 4;
    int blk = blockIdx.x;
    const int qb = blk % a.n_qb;
    blk /= a.n_qb;
    const int w = blk % a.s;
    blk /= a.s;
    const int u = blk % a.U, b = blk / a.U;
    if (b >= a.B) return;
    const int Hq = a.U * a.s * a.gq;
    const int len = min(a.lens[b], a.cap);
    const int rows = a.M * a.gq;
    const int row0 = qb * 64;
    if (len <= 0 || row0 >= rows) return;

    // this lane's query row (column c of the wave's score tiles)
    const int rho = row0 + 16 * wv + c;
    const bool row_ok = rho < rows;
    const int m_row = row_ok ? rho / a.gq : 0;
    const int j_row = (u * a.s + w) * a.gq + (row_ok ? rho % a.gq : 0);
    const int pos = row_ok ? qpos(a.p0, a.lens, b, m_row) : -1;
    // the block's last position (rows ascend with the chunk token)
    const int m_last = (min(rows, row0 + 64) - 1) / a.gq;
    const int n_t = min(a.n_tiles, qpos(a.p0, a.lens, b, m_last) / 32 + 1);

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
    issue(0);

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
    // queries of the lane's row, dims 32 ks + 8 g + e, as fp16 hi + lo
    half8 qh[4], ql[4];
    {
        const float* qs = a.qr + ((long)(b * a.M + m_row) * Hq + j_row) * DH;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = row_ok ? qs[32 * ks + 8 * g + e] : 0.0f;
                qh[ks][e] = (half_t)v;
                ql[ks][e] = (half_t)(v - (float)qh[ks][e]);
            }
    }
    // in-tile offsets (cos, sin)(tau theta_f) of the lane's token tau = l % 32 and
    // its eight frequencies f_i = 16 wv + 8 (i / 4) + 4 (l / 32) + i % 4
    float2 tok[8];
    auto freq = [&](int i) { return 16 * wv + 8 * (i >> 2) + 4 * (l >> 5) + (i & 3); };
#pragma unroll
    for (int i = 0; i < 8; ++i) tok[i] = a.ang[(long)(a.n_tiles + (l & 31)) * (DH / 2) + freq(i)];

    // key fragment of the reconstruction (B operand): token l % 32, ranks 16 ks + 8 (l/32)
    int koff[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) koff[q] = (l & 31) * R + 8 * ((2 * q + (l >> 5)) ^ (l & 15));
    const int vro = 8 * (4 * (l & 15) + ((l >> 4) ^ vswz(l & 15)));

    float m_run = -INFINITY, l_lane = 0.0f;
    floatx4 o[NDB];
#pragma unroll
    for (int d = 0; d < NDB; ++d) o[d] = floatx4{0.f, 0.f, 0.f, 0.f};

    // (cos, sin) of the tile start for the lane's frequencies: loaded one tile ahead,
    // after the current tile's rotation, so the wait at the tile top covers them
    float2 st[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) st[i] = a.ang[freq(i)];
    for (int t = 0; t < n_t; ++t) {
        const int t0 = 32 * t;
        // vmcnt(0) as a builtin: the compiler sees it, so it inserts no later wait for
        // its own loads (which would also stall on the next tile's loads below)
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();                      // tile t in LDS; tile t-1 fully consumed
        if (t + 1 < n_t) issue(t + 1);

        // ---- K^T for the wave's 32 dims, RoPE, K hi / lo to LDS
        {
            const half_t* ht = htile[t & 1];
            floatx16 acc = floatx16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc = mfma32(bf[ks], lds8(ht + koff[ks & 7] + 128 * (ks >> 3)), acc);
            const int tl = l & 31;
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
                half_t lh[4], ll[4], hh[4], hl[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * gi + e;
                    const float cc = st[i].x * tok[i].x - st[i].y * tok[i].y;
                    const float ss = st[i].x * tok[i].y + st[i].y * tok[i].x;
                    const float lo = acc[i], hi = acc[i + 8];
                    const float lo2 = lo * cc - hi * ss, hi2 = hi * cc + lo * ss;
                    lh[e] = (half_t)lo2;
                    ll[e] = (half_t)(lo2 - (float)lh[e]);
                    hh[e] = (half_t)hi2;
                    hl[e] = (half_t)(hi2 - (float)hh[e]);
                }
                // dims 16 wv + 8 gi + 4 (l/32) + e (chunk 2 wv + gi) and their partners (+64)
                const int q_lo = (2 * wv + gi) ^ (tl & 15), q_hi = (8 + 2 * wv + gi) ^ (tl & 15);
                const int o_lo = tl * DH + 8 * q_lo + 4 * (l >> 5), o_hi = tl * DH + 8 * q_hi + 4 * (l >> 5);
                *reinterpret_cast<half4*>(&krot[0][o_lo]) = half4{lh[0], lh[1], lh[2], lh[3]};
                *reinterpret_cast<half4*>(&krot[1][o_lo]) = half4{ll[0], ll[1], ll[2], ll[3]};
                *reinterpret_cast<half4*>(&krot[0][o_hi]) = half4{hh[0], hh[1], hh[2], hh[3]};
                *reinterpret_cast<half4*>(&krot[1][o_hi]) = half4{hl[0], hl[1], hl[2], hl[3]};
            }
        }
        if (t + 1 < n_t) {
#pragma unroll
            for (int i = 0; i < 8; ++i) st[i] = a.ang[(long)(t + 1) * (DH / 2) + freq(i)];
        }
        __syncthreads();                      // K of tile t complete

        // ---- S^T [token][row]: block mb row m is token 8 (m/4) + 4 mb + m % 4
        // four independent accumulation chains: (hi x hi) and (hi x lo + lo x hi) per block
        floatx4 S[2], S2[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) S[mb] = S2[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            half8 kh[2], kl[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const int tk = 8 * (c >> 2) + 4 * mb + (c & 3);
                const int off = tk * DH + 8 * ((4 * ks + g) ^ (tk & 15));
                kh[mb] = lds8(&krot[0][off]);
                kl[mb] = lds8(&krot[1][off]);
            }
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) S[mb] = mfma16(kh[mb], qh[ks], S[mb]);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) S2[mb] = mfma16(kh[mb], ql[ks], S2[mb]);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) S2[mb] = mfma16(kl[mb], qh[ks], S2[mb]);
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) S[mb] += S2[mb];
        // lane (c, g): row c at tokens t0 + 8 g + j, j = 4 mb + i
        float sv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int tkn = t0 + 8 * g + jj;
            sv[jj] = tkn <= pos ? S[jj >> 2][jj & 3] : -INFINITY;
        }
        float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
        {
            auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, mx), __builtin_bit_cast(int, mx), false, false);
            mx = fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
            r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, mx), __builtin_bit_cast(int, mx), false, false);
            mx = fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
        }
        const float mn = fmaxf(m_run, mx);
        if (__builtin_amdgcn_ballot_w64(mn > m_run)) {
            const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - mn);
            l_lane *= alpha;
#pragma unroll
            for (int d = 0; d < NDB; ++d) o[d] *= alpha;
        }
        m_run = mn;
        half8 pb;
        float psum = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const float pv = sv[jj] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sv[jj] - mn);
            psum += pv;
            pb[jj] = (half_t)pv;
        }
        l_lane += psum;

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
                o[d] = mfma16(va, pb, o[d]);
            }
        }
    }

    // lane (c, g) holds dims 16 d + 4 g + i of row c
    float lsum = l_lane;
    {
        auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, lsum), __builtin_bit_cast(int, lsum), false, false);
        lsum = __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
        r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, lsum), __builtin_bit_cast(int, lsum), false, false);
        lsum = __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
    }
    if (row_ok) {
        const float inv = 1.0f / lsum;
        float* op = a.out + ((long)(b * a.M + m_row) * Hq + j_row) * R + 4 * g;
#pragma unroll
        for (int d = 0; d < NDB; ++d)
            *reinterpret_cast<float4*>(op + 16 * d) = make_float4(o[d][0] * inv, o[d][1] * inv, o[d][2] * inv, o[d][3] * inv);
    }
}

}  // namespace

size_t prefill_workspace_bytes(int B, int M, int Hq, int DH, int n_tiles) {
    return align_up((size_t)(n_tiles + 32) * (DH / 2) * sizeof(float2), 256) +
           align_up((size_t)B * M * Hq * DH * sizeof(float), 256);
}

int32_t launch_prefill(const lrkv_latent_cache* c, const float* q, const half_t* bk, const int32_t* p0, int M,
                       int n_tiles, float sm_scale, float* out, void* ws, hipStream_t st) {
    const int Hq = c->units * c->kv_per_unit * c->q_per_kv, DH = c->head_dim;
    float2* ang = (float2*)ws;
    float* qr = (float*)((char*)ws + align_up((size_t)(n_tiles + 32) * (DH / 2) * sizeof(float2), 256));
    PrefillPrepArgs pa{q, p0, c->lens, qr, ang, c->batch, M, Hq, DH, n_tiles, (double)c->rope_theta,
                       sm_scale * kLog2e};
    const long n_prep = (long)(n_tiles + 32) * (DH / 2) + (long)c->batch * M * Hq * (DH / 2);
    hipLaunchKernelGGL(prefill_prep, dim3((unsigned)((n_prep + 255) / 256)), dim3(256), 0, st, pa);
    const int n_qb = (M * c->q_per_kv + 63) / 64;
    PrefillArgs a{(const half_t*)c->hk, (const half_t*)c->hv, bk, p0, c->lens, qr, ang, out,
                  c->batch, c->units, c->kv_per_unit, c->q_per_kv, M, c->capacity, n_tiles, n_qb};
    const long blocks = (long)c->batch * c->units * c->kv_per_unit * n_qb;
    hipLaunchKernelGGL(prefill_attn<256>, dim3((unsigned)blocks), dim3(256), 0, st, a);
    return last_launch_status();
}

}  // namespace lrkv
