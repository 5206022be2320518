// lrkv_decode_attn_noalloc: the decode step with its workspace in a static
// device array, for callers that cannot allocate (graph capture, serving
// loops, harnesses that forbid hipMalloc).
//
// `scratch` below is a device symbol: in host code its name is only a host-side
// stand-in. Its device address is obtained once per device with
// hipGetSymbolAddress (with that device current) and kept in `g_scratch`; every
// kernel argument uses that address, never the symbol's name.
#include <mutex>

#include "common.h"

namespace lrkv {
namespace {

constexpr size_t kScratchBytes = LRKV_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

// One copy per device that loads the library; it keeps the last call's contents.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];

// The device address of `scratch` on the current device, looked up on the first
// call made with that device current.
int32_t device_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LRKV_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) return LRKV_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return LRKV_OK;
}

}  // namespace
}  // namespace lrkv

extern "C" int32_t lrkv_decode_attn_noalloc(int32_t mode, const void* cache, const float* q, const void* bk,
                                            const int32_t* q_pos, float sm_scale, float* out,
                                            int32_t host_max_len, int32_t n_split, void* stream) {
    using namespace lrkv;
    if (!q) return LRKV_ERR_INVALID_ARG;
    // every argument check of lrkv_decode_attn first, nothing enqueued
    size_t need = 0;
    const int32_t vrc = decode_common(mode, kPhaseAll, cache, q, bk, q_pos, sm_scale, out, nullptr, 0,
                                      host_max_len, n_split, stream, &need);
    if (vrc != LRKV_OK) return vrc;
    if (need > kScratchBytes) return LRKV_ERR_SCRATCH;
    void* ws = nullptr;
    const int32_t rc = device_scratch(&ws);
    if (rc != LRKV_OK) return rc;
    return decode_common(mode, kPhaseAll, cache, q, bk, q_pos, sm_scale, out, ws, kScratchBytes, host_max_len,
                         n_split, stream);
}
