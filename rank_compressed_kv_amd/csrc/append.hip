// Cache append kernels: fp16 latents, int4 latents (group-32 symmetric codec) and
// dense tokens of the hybrid paged cache.
//
// Palu digest, Method details: the cache holds per-token latents h = x A
// instead of keys and values. PuzzleKV section 3.3, step 5: new key/value pairs
// go to the newest dense page. The int4 rule (Shard post, section 5, step 4:
// symmetric [-7, 7]; Palu digest, Supplementary details: per-token groups of
// 32) is documented in lrkv.h.
#include "append_dev.h"

namespace lrkv {
namespace {

__global__ void bump_lens(int32_t* lens, int B, int n_new) {
    int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) lens[b] += n_new;
}

// One thread per (b, u, i, 8 consecutive dims). Keys go token-major, values into
// the dim-major 32-token block of their position.
__global__ void append_fp16(const float* __restrict__ nk, const float* __restrict__ nv,
                            half_t* __restrict__ hk, half_t* __restrict__ hv,
                            const int32_t* __restrict__ lens, int B, int U, int r, int cap,
                            int n_new) {
    const int r8 = r / 8;
    const long total = (long)B * U * n_new * r8;
    long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= total) return;
    const int d8 = (int)(e % r8);
    long rest = e / r8;
    const int i = (int)(rest % n_new);
    rest /= n_new;
    const int u = (int)(rest % U);
    const int b = (int)(rest / U);
    const int pos = lens[b] + i;
    if (pos >= cap) return;                  // stale host bound: never write past the capacity
    const long src = (((long)b * U + u) * n_new + i) * r + d8 * 8;
    const float4 k0 = *reinterpret_cast<const float4*>(nk + src);
    const float4 k1 = *reinterpret_cast<const float4*>(nk + src + 4);
    const float4 v0 = *reinterpret_cast<const float4*>(nv + src);
    const float4 v1 = *reinterpret_cast<const float4*>(nv + src + 4);
    half8 kh;
    kh[0] = (half_t)k0.x; kh[1] = (half_t)k0.y; kh[2] = (half_t)k0.z; kh[3] = (half_t)k0.w;
    kh[4] = (half_t)k1.x; kh[5] = (half_t)k1.y; kh[6] = (half_t)k1.z; kh[7] = (half_t)k1.w;
    const long bu = (long)b * U + u;
    *reinterpret_cast<half8*>(hk + (bu * cap + pos) * r + d8 * 8) = kh;
    const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    half_t* vblk = hv + ((bu * (cap / kTile) + pos / kTile) * r + d8 * 8) * kTile + pos % kTile;
#pragma unroll
    for (int k = 0; k < 8; ++k) vblk[k * kTile] = (half_t)vv[k];
}

// Decode-size fp16 append in one workgroup: every thread reads lens before the
// workgroup barrier, so the same kernel can bump the lengths afterwards.
__global__ __launch_bounds__(256) void append_fp16_small(const float* __restrict__ nk,
                                                         const float* __restrict__ nv,
                                                         half_t* __restrict__ hk,
                                                         half_t* __restrict__ hv,
                                                         int32_t* __restrict__ lens, int B, int U,
                                                         int r, int cap, int n_new) {
    append_fp16_rows(nk, nv, hk, hv, lens, B, U, r, cap, n_new, threadIdx.x, blockDim.x);
    __syncthreads();
    for (int b = threadIdx.x; b < B; b += blockDim.x) lens[b] += n_new;
}

// Keys: one thread per (b, u, i, group). 16 packed bytes + one scale.
__global__ void append_int4_k(const float* __restrict__ nk, uint8_t* __restrict__ hk,
                              half_t* __restrict__ sk, const int32_t* __restrict__ lens, int B,
                              int U, int r, int cap, int n_new) {
    const long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e < (long)B * U * n_new * (r / 32)) append_int4_key_group(nk, hk, sk, lens, B, U, r, cap, n_new, e);
}

// Values: one thread per (b, u, token pair, group) so that no two threads share a
// byte; a partner token outside the appended range keeps its nibble.
__global__ void append_int4_v(const float* __restrict__ nv, uint8_t* __restrict__ hv,
                              half_t* __restrict__ sv, const int32_t* __restrict__ lens, int B,
                              int U, int r, int cap, int n_new) {
    const long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e < (long)B * U * (n_new / 2 + 2) * (r / 32))
        append_int4_value_pair(nv, hv, sv, lens, B, U, r, cap, n_new, e);
}

// Hybrid cache: one thread per (b, h, i, 8 dims) copying K and V into the dense
// slot of the token's page (values transposed), unless that page is already
// factored.
__global__ void append_paged(const half_t* __restrict__ nk, const half_t* __restrict__ nv,
                             half_t* __restrict__ dk, half_t* __restrict__ dv,
                             int32_t* __restrict__ table, const int32_t* __restrict__ lens, int B,
                             int H, int d, int P, int sink, int window, int max_pages, int n_new) {
    const int d8 = d / 8;
    const long total = (long)B * H * n_new * d8;
    long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= total) return;
    const int c8 = (int)(e % d8);
    long rest = e / d8;
    const int i = (int)(rest % n_new);
    rest /= n_new;
    const int h = (int)(rest % H);
    const int b = (int)(rest / H);
    const int pos = lens[b] + i;
    const int p = pos / P;
    if (p >= max_pages) return;              // stale host bound: never write past the table
    const long bh = (long)b * H + h;
    int32_t* entry = table + bh * max_pages + p;
    if (*entry >= 0) return;                 // factored already (prefill)
    const int slot = p < sink ? p : sink + (p - sink) % window;
    const long src = (bh * n_new + i) * d + c8 * 8;
    const long page = bh * (sink + window) + slot;
    // keys row-major [P][d], values dimension-major [d][P]
    *reinterpret_cast<half8*>(dk + (page * P + pos % P) * d + c8 * 8) = *reinterpret_cast<const half8*>(nk + src);
    const half8 v = *reinterpret_cast<const half8*>(nv + src);
#pragma unroll
    for (int e = 0; e < 8; ++e) dv[(page * d + c8 * 8 + e) * P + pos % P] = v[e];
    if (pos % P == 0 && c8 == 0) *entry = -1 - slot;
}

inline unsigned blocks_for(long n, int bs) { return (unsigned)((n + bs - 1) / bs); }

}  // namespace

int32_t launch_append_latent(const lrkv_latent_cache* c, const float* nk, const float* nv,
                             int n_new, hipStream_t st) {
    const int B = c->batch, U = c->units, r = c->rank, cap = c->capacity;
    if (c->fmt == LRKV_FMT_FP16 && (long)B * U * n_new * (r / 8) <= kSmallAppendRows) {
        hipLaunchKernelGGL(append_fp16_small, dim3(1), dim3(256), 0, st, nk, nv, (half_t*)c->hk,
                           (half_t*)c->hv, c->lens, B, U, r, cap, n_new);
        return last_launch_status();
    }
    if (c->fmt == LRKV_FMT_FP16) {
        const long n = (long)B * U * n_new * (r / 8);
        hipLaunchKernelGGL(append_fp16, dim3(blocks_for(n, 256)), dim3(256), 0, st, nk, nv,
                           (half_t*)c->hk, (half_t*)c->hv, c->lens, B, U, r, cap, n_new);
    } else {
        const long nk_threads = (long)B * U * n_new * (r / 32);
        hipLaunchKernelGGL(append_int4_k, dim3(blocks_for(nk_threads, 128)), dim3(128), 0, st, nk,
                           (uint8_t*)c->hk, (half_t*)c->sk, c->lens, B, U, r, cap, n_new);
        const long nv_threads = (long)B * U * (n_new / 2 + 2) * (r / 32);
        hipLaunchKernelGGL(append_int4_v, dim3(blocks_for(nv_threads, 128)), dim3(128), 0, st, nv,
                           (uint8_t*)c->hv, (half_t*)c->sv, c->lens, B, U, r, cap, n_new);
    }
    hipLaunchKernelGGL(bump_lens, dim3(blocks_for(B, 64)), dim3(64), 0, st, c->lens, B, n_new);
    return last_launch_status();
}

int32_t launch_append_paged(const lrkv_paged_cache* c, const half_t* nk, const half_t* nv,
                            int n_new, hipStream_t st) {
    const int B = c->batch, H = c->kv_heads, d = c->head_dim;
    const long n = (long)B * H * n_new * (d / 8);
    hipLaunchKernelGGL(append_paged, dim3(blocks_for(n, 256)), dim3(256), 0, st, nk, nv,
                       (half_t*)c->dense_k, (half_t*)c->dense_v, c->page_table, c->lens, B, H, d,
                       c->page_size, c->sink_pages, c->window_pages, c->max_pages, n_new);
    hipLaunchKernelGGL(bump_lens, dim3(blocks_for(B, 64)), dim3(64), 0, st, c->lens, B, n_new);
    return last_launch_status();
}

}  // namespace lrkv
