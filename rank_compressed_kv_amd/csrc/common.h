// Internal definitions shared by the lrkv HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lrkv.h"

namespace lrkv {

typedef _Float16 half_t;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kTile = 32;          // tokens per attention tile == cache block
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxSplit = 1024;    // sequence chunks merged per head (merge kernel's LDS)
// A decode-size append runs in one workgroup of 256 threads (and inside the query
// preparation of lrkv_decode_step) when it has at most this many items: fp16
// 8-element rows, or int4 key groups plus value token-pair groups.
constexpr int kSmallAppendRows = 1024;
constexpr int kMaxRopeTiles = 256; // tiles per RoPE chunk: bounds the angle-rotation drift

// ---------------------------------------------------------------- MFMA wrappers
// v_mfma_f32_32x32x16_f16. Lane l supplies A[l%32][8*(l/32) + 0..7] and
// B[8*(l/32) + 0..7][l%32]; accumulator element i of lane l is
// D[8*(i/4) + 4*(l/32) + i%4][l%32].
__device__ __forceinline__ floatx16 mfma32(half8 a, half8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x32_f16. Lane l supplies A[l%16][8*(l/16) + 0..7] and
// B[8*(l/16) + 0..7][l%16]; accumulator element i of lane l is
// D[4*(l/16) + i][l%16].
__device__ __forceinline__ floatx4 mfma16(half8 a, half8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- lane helpers
template <int W>
__device__ __forceinline__ float reduce_sum_width(float v) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Sign-extended 4-bit code in nibble `k` (0..7) of a 32-bit word.
__device__ __forceinline__ int nibble(uint32_t w, int k) {
    return ((int)(w << (28 - 4 * k))) >> 28;
}

// ---------------------------------------------------------------- int4 codec
// The symmetric int4 codec of one 32-element group (documented in lrkv.h): fp16
// scale and the 32 codes. Shared by the latent append and the page factors.
__device__ inline void quant_group(const float* __restrict__ x, int* codes, half_t* scale) {
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(x[k]));
    const float s32 = amax / 7.0f;                       // IEEE fp32 division
    half_t s16 = (half_t)s32;                            // round to nearest even
    if (__builtin_isinf((float)s16)) s16 = (half_t)65504.0f;
    const double den = (double)(float)s16;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
        int c = 0;
        if (den != 0.0) {
            double qd = rint((double)x[k] / den);        // fp64 quotient, half-even
            qd = fmin(7.0, fmax(-7.0, qd));
            c = (int)qd;
        }
        codes[k] = c;
    }
    *scale = s16;
}

// ---------------------------------------------------------------- launch plumbing
struct Status {
    static int32_t from_hip(hipError_t e) { return e == hipSuccess ? LRKV_OK : LRKV_ERR_HIP; }
};

inline int32_t last_launch_status() { return Status::from_hip(hipGetLastError()); }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- kernel entry points (host side)
struct LatentGeom {
    int B, U, s, gq, dh, r, cap, fmt, Hq;
    float theta;
};

LatentGeom latent_geom(const lrkv_latent_cache* c);

// Decode workspace for the Palu modes: partials [B][Hq][n_split][r + 2] float,
// then (RoPE mode) the rotated-basis queries [B][Hq][dh][r] half, their
// per-frequency scales [B][U][dh/2] float and the angle tables
// [33 + B * n_split][dh/2] float2.
struct LatentWorkspace {
    size_t part_off, qp_off, qs_off, ang_off, total;
    int n_split, chunk;
};
LatentWorkspace latent_workspace(int mode, const LatentGeom& g, int host_max_len, int n_split);

int32_t launch_append_latent(const lrkv_latent_cache* c, const float* nk, const float* nv,
                             int n_new, hipStream_t st);
int32_t launch_append_paged(const lrkv_paged_cache* c, const half_t* nk, const half_t* nv,
                            int n_new, hipStream_t st);
// Decode phases: query preparation, per-chunk partial states, split merge.
constexpr int kPhasePrepare = 1, kPhasePartials = 2, kPhaseMerge = 4, kPhaseAll = 7;
// What the RoPE preparation writes into the query buffer: Q' row-major, Q' in the
// frequency-wave kernel's fragment order, or B^k fragments of the grouped-query
// kernel (which rotates the raw queries itself).
constexpr int kQpRowMajor = 0, kQpFragments = 1, kQpGqaFragments = 2;
bool use_gqa_kernel(const LatentGeom& g);

// The new tokens of lrkv_decode_step when they are appended inside the decode's
// own launches (fp32 [B][U][n_new][R], like lrkv_append_latent's inputs).
struct FusedAppend {
    const float* nk;
    const float* nv;
    int n_new;
};
// Whether an append of n_new tokens fits the one-workgroup append role of the
// query preparation: fp16 rows of 8 elements, or int4 key groups plus value
// token-pair groups, at most kSmallAppendRows items.
inline bool fused_append_fits(const lrkv_latent_cache* c, int n_new) {
    const long bu = (long)c->batch * c->units;
    if (c->fmt == LRKV_FMT_FP16) return bu * n_new * (c->rank / 8) <= kSmallAppendRows;
    return bu * (n_new + n_new / 2 + 2) * (c->rank / 32) <= kSmallAppendRows;
}
// Validation and dispatch shared by every decode entry point (api.hip). With
// ws_need non-null it only validates and stores the workspace size needed.
int32_t decode_common(int32_t mode, int phases, const void* cache, const float* q, const void* bk,
                      const int32_t* q_pos, float sm_scale, float* out, void* workspace, size_t ws_bytes,
                      int32_t host_max_len, int32_t n_split, void* stream, size_t* ws_need = nullptr,
                      const FusedAppend* app = nullptr);

int32_t launch_decode_latent(int mode, int phases, const lrkv_latent_cache* c, const float* q,
                             const half_t* bk, const int32_t* q_pos, float sm_scale, float* out,
                             void* ws, const LatentWorkspace& w, hipStream_t st,
                             const FusedAppend* app = nullptr);

struct PagedWorkspace {
    size_t part_off, total;
    int n_split, pages_per_split;
};
PagedWorkspace paged_workspace(const lrkv_paged_cache* c, int host_max_len, int n_split);
int32_t launch_decode_hybrid(int phases, const lrkv_paged_cache* c, const float* q, float sm_scale,
                             float* out, void* ws, const PagedWorkspace& w, hipStream_t st);
// Weight-stream GEMM C[M][N] = X[M][K] W^T[N][K]^T (fp32 X and C, fp16 W):
// K split into k_split ranges of kchunk, partial sums in the workspace.
struct SkinnyPlan {
    int kchunk, k_split;
    size_t ws_bytes;
};
SkinnyPlan skinny_plan(int M, int N, int K);
int32_t launch_skinny(const float* X, const half_t* Wt, float* C, int M, int N, int K, void* ws,
                      const SkinnyPlan& p, hipStream_t st);
int32_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, int blocks, hipStream_t st);
size_t prefill_workspace_bytes(int B, int U, int s, int gq, int M, int DH, int R, int n_tiles);
int32_t launch_prefill(const lrkv_latent_cache* c, const float* q, const half_t* bk, const int32_t* p0, int M,
                       int n_tiles, float sm_scale, float* out, void* ws, hipStream_t st);
int32_t launch_factor_page(const lrkv_paged_cache* c, const int32_t* pages, int n_pages,
                           const half_t* src_k, const half_t* src_v, int src_len, int max_sweeps,
                           hipStream_t st);

}  // namespace lrkv
