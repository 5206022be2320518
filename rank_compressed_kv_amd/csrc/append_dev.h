// Device bodies of the latent appends (fp16 rows, int4 key groups, int4 value
// pairs), shared by the append kernels and by the query preparation of
// lrkv_decode_step (Palu digest, Method details: the cache holds per-token
// latents, values in their token's dim-major block; int4 with one fp16 scale per
// 32 elements, Supplementary details).
#pragma once

#include "common.h"

namespace lrkv {

// Threads tid, tid + nthreads, ... of one workgroup write the n_new new tokens of
// every (sequence, unit) at positions lens[b] + i (rounded to fp16): keys
// token-major, values into the dim-major 32-token block of their position.
// Positions at or past the capacity are skipped. lens is only read.
__device__ __forceinline__ void append_fp16_rows(const float* __restrict__ nk, const float* __restrict__ nv,
                                                 half_t* __restrict__ hk, half_t* __restrict__ hv,
                                                 const int32_t* __restrict__ lens, int B, int U, int r,
                                                 int cap, int n_new, int tid, int nthreads) {
    const int r8 = r / 8;
    const int total = B * U * n_new * r8;
    for (int e = tid; e < total; e += nthreads) {
        const int d8 = e % r8;
        int rest = e / r8;
        const int i = rest % n_new;
        rest /= n_new;
        const int u = rest % U;
        const int b = rest / U;
        const int pos = lens[b] + i;
        if (pos >= cap) continue;
        const long src = (((long)b * U + u) * n_new + i) * r + d8 * 8;
        const long bu = (long)b * U + u;
        half8 kh;
#pragma unroll
        for (int k = 0; k < 8; ++k) kh[k] = (half_t)nk[src + k];
        *reinterpret_cast<half8*>(hk + (bu * cap + pos) * r + d8 * 8) = kh;
        half_t* vblk = hv + ((bu * (cap / kTile) + pos / kTile) * r + d8 * 8) * kTile + pos % kTile;
#pragma unroll
        for (int k = 0; k < 8; ++k) vblk[k * kTile] = (half_t)nv[src + k];
    }
}

// int4 keys, item e of (b, u, i, group): the group's 32 codes (16 packed bytes)
// and its fp16 scale, at position lens[b] + i (skipped at or past the capacity).
__device__ __forceinline__ void append_int4_key_group(const float* __restrict__ nk, uint8_t* __restrict__ hk,
                                                      half_t* __restrict__ sk, const int32_t* __restrict__ lens,
                                                      int B, int U, int r, int cap, int n_new, long e) {
    const int G = r / 32;
    const int g = (int)(e % G);
    long rest = e / G;
    const int i = (int)(rest % n_new);
    rest /= n_new;
    const int u = (int)(rest % U);
    const int b = (int)(rest / U);
    const int pos = lens[b] + i;
    if (pos >= cap) return;
    const float* x = nk + ((((long)b * U + u) * n_new + i) * r + g * 32);
    int codes[32];
    half_t s16;
    quant_group(x, codes, &s16);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t acc = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc |= (uint32_t)(codes[q * 8 + k] & 0xF) << (4 * k);
        w[q] = acc;
    }
    const long bu = (long)b * U + u;
    *reinterpret_cast<uint4*>(hk + (bu * cap + pos) * (r / 2) + g * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    sk[(bu * cap + pos) * G + g] = s16;
}

// int4 values, item e of (b, u, token pair, group): the pair's byte column of the
// dim-major value block, so that no two items share a byte; a partner token
// outside [lens[b], lens[b] + n_new) keeps its nibble.
__device__ __forceinline__ void append_int4_value_pair(const float* __restrict__ nv, uint8_t* __restrict__ hv,
                                                       half_t* __restrict__ sv, const int32_t* __restrict__ lens,
                                                       int B, int U, int r, int cap, int n_new, long e) {
    const int G = r / 32;
    const int n_pairs = n_new / 2 + 2;       // pairs touched by [len, len + n_new)
    const int g = (int)(e % G);
    long rest = e / G;
    const int pi = (int)(rest % n_pairs);
    rest /= n_pairs;
    const int u = (int)(rest % U);
    const int b = (int)(rest / U);
    const int len = lens[b];
    const int pair = len / 2 + pi;           // covers tokens 2*pair, 2*pair + 1
    const long bu = (long)b * U + u;
    int codes[2][32];
    bool own[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int pos = 2 * pair + hh;
        own[hh] = pos >= len && pos < len + n_new && pos < cap;
        if (own[hh]) {
            half_t s16;
            quant_group(nv + ((bu * n_new + (pos - len)) * r + g * 32), codes[hh], &s16);
            sv[((bu * (cap / kTile) + pos / kTile) * G + g) * kTile + pos % kTile] = s16;
        }
    }
    if (!own[0] && !own[1]) return;
    const int pos0 = 2 * pair;
    uint8_t* base = hv + ((bu * (cap / kTile) + pos0 / kTile) * r + g * 32) * (kTile / 2) + (pos0 % kTile) / 2;
    // the partner token's nibbles: every byte read before any is written (one
    // round trip; the item owns these bytes, no other item touches them)
    uint32_t old[32];
    const bool keep = !(own[0] && own[1]);
#pragma unroll
    for (int k = 0; k < 32; ++k) old[k] = keep ? (uint32_t)base[k * (kTile / 2)] : 0u;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
        uint32_t byte = old[k];
        if (own[0]) byte = (byte & 0xF0u) | ((uint32_t)codes[0][k] & 0xFu);
        if (own[1]) byte = (byte & 0x0Fu) | (((uint32_t)codes[1][k] & 0xFu) << 4);
        base[k * (kTile / 2)] = (uint8_t)byte;
    }
}

}  // namespace lrkv
