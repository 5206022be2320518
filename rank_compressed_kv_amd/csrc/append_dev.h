// Device body of the decode-size fp16 latent append, shared by the append kernel
// and by the query preparation of lrkv_decode_step (Palu digest, Method details:
// the cache holds per-token latents; values in their token's dim-major block).
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

}  // namespace lrkv
