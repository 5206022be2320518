// Device helpers shared by the latent-cache decode kernels: lane reductions,
// key-tile staging (registers or direct global->LDS), value fragments.
#pragma once

#include "common.h"

namespace lrkv {

// ---------------------------------------------------------------- reductions
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
// Sum / max over the 32 lanes of each half-wave: DPP within rows of 16
// (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror, row_mirror), then the row pair.
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

// ---------------------------------------------------------------- direct global->LDS loads
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Raw buffer resource over [base, base + bytes): loads at or past `bytes` read
// as zero. Word 3 is the gfx9 raw 32-bit data format. Built from wave-uniform
// values, held in scalar registers.
typedef int32_t int32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    int32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)((a >> 32) & 0xffffu));   // stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
    r[3] = 0x00020000;
    return r;
}
// buffer_load_dwordx4 ... lds as inline assembly (so the compiler adds no waits
// before LDS reads; the caller counts vmcnt): lane i loads 16 bytes at
// base + voff and writes them to LDS at lds + 16 i. `rsrc` and `lds` must be
// wave-uniform. No immediate or scalar offset (zero on this path).
__device__ __forceinline__ void buf_dma16(int32x4 rsrc, uint32_t voff, const void* lds) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    // M0 (the LDS base) is an input bound to that register, so the compiler sets
    // it and knows it in use; the s_nop separates that write from the load
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "{m0}"(m) : "memory");
}

// ---------------------------------------------------------------- key tile, register staging
// 32 tokens x R fp16 rows in LDS with rows padded to R + 8 halves; int4 codes are
// dequantised on the way (code * scale rounded to fp16). Rows at or past t_end
// are zero. Staged in two halves to halve the staging registers.
template <int R, bool INT4>
struct KStage {
    static constexpr int NV = 32 * R / 8;                 // 8-dim items per tile
    static constexpr int PER = (NV + 255) / 256;
    static constexpr int HALF = (PER + 1) / 2;            // items staged per half
    uint4 v[HALF];

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

// ---------------------------------------------------------------- value fragments
// A fragment of V^T for the 16x16x32 MFMA from the dim-major 32-token block in
// global memory: dims [16 mv, 16 mv + 16) x the 8 tokens of lane group l/16,
// masked past t_end.
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

// ---------------------------------------------------------------- int4 codes
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2_t pack2(float a, float b) { return half2_t{(half_t)a, (half_t)b}; }

__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(o));
    return r;
}

// The 8 two's complement nibbles of a word of codes (element k at bits 4k) as
// exact fp16 values, in the order k = 0, 4, 1, 5, 2, 6, 3, 7: after flipping
// the sign bits (code + 8 in 0..15), the nibble pair (k, k + 4) of each byte
// position is masked into the mantissas of 0x6400 = 1024 (k even: 1024 + c + 8;
// k odd, 4 bits up: 1024 + 16 (c + 8)); both are exact, as are the offsets.
__device__ __forceinline__ void unpack_codes(uint32_t w, uint32_t magic, half2_t* r) {
    const uint32_t x = w ^ 0x88888888u, y = x >> 8;
    const half2_t lo_off = {-1032.0f16, -1032.0f16};
    const half2_t hi_mul = {0.0625f16, 0.0625f16}, hi_off = {-72.0f16, -72.0f16};
    r[0] = __builtin_bit_cast(half2_t, and_or(x, 0x000F000Fu, magic)) + lo_off;
    r[1] = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, and_or(x, 0x00F000F0u, magic)), hi_mul, hi_off);
    r[2] = __builtin_bit_cast(half2_t, and_or(y, 0x000F000Fu, magic)) + lo_off;
    r[3] = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, and_or(y, 0x00F000F0u, magic)), hi_mul, hi_off);
}
// Source nibble of element e (0..7) of an unpacked word: 0, 4, 1, 5, 2, 6, 3, 7.
__host__ __device__ constexpr int code_pos_inv(int e) { return (e & 1) ? 4 + (e >> 1) : e >> 1; }
__device__ __forceinline__ half8 as_half8(const half2_t* r) {
    return __builtin_bit_cast(half8, uint4{__builtin_bit_cast(uint32_t, r[0]), __builtin_bit_cast(uint32_t, r[1]),
                                           __builtin_bit_cast(uint32_t, r[2]), __builtin_bit_cast(uint32_t, r[3])});
}
// Keys: codes x the token's fp16 scale (bits in the low half of sc; one
// rounding, as code * scale in fp16).
__device__ __forceinline__ half8 dequant_keys(uint32_t w, uint32_t sc, uint32_t magic) {
    half2_t r[4];
    unpack_codes(w, magic, r);
    const half2_t s2 = __builtin_bit_cast(half2_t, sc * 0x00010001u);
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] *= s2;
    return as_half8(r);
}
// Values: the codes alone (the per-token scale is folded into p).
__device__ __forceinline__ half8 value_codes(uint32_t w, uint32_t magic) {
    half2_t r[4];
    unpack_codes(w, magic, r);
    return as_half8(r);
}

// ---------------------------------------------------------------- RoPE angles
// Tables written by the query-preparation step (fp64 angles, fp32 values):
//   step[f]      = (cos, sin)(32 theta_f)                   rotation by one tile
//   tok[t][f]    = (cos, sin)(t theta_f), t < 32            offset inside a tile
//   start[b][c][f] = (cos, sin)((c * chunk - q_pos[b]) theta_f)   chunk start
// A lane starts at start (x) tok[l % 32] and advances by `step` per tile.
struct AngleTables {
    const float2* step;   // [DH/2]
    const float2* tok;    // [32][DH/2]
    const float2* start;  // [B][n_split][DH/2]
};
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}

}  // namespace lrkv
