// Streaming-read microkernel: the practical HBM read rate that the decode
// kernels are compared against (beside the nominal peak). Every byte of the
// buffer is read once with 16-byte loads, four in flight per lane, grid-stride;
// each workgroup folds what it read into one word, so nothing is elided.
#include "common.h"

namespace lrkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ src, size_t n16, uint32_t* out) {
    const size_t stride = (size_t)gridDim.x * 256 * 4;
    uint32_t acc = 0;
    size_t i = (size_t)blockIdx.x * 256 * 4 + threadIdx.x;
    for (; i + 3 * 256 < n16; i += stride) {
        u32x4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = __builtin_nontemporal_load(src + i + 256 * k);
#pragma unroll
        for (int k = 0; k < 4; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
    for (; i < n16; i += 256) {
        const u32x4 v = src[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    __shared__ uint32_t red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int k = 0; k < 256; ++k) s ^= red[k];
        out[blockIdx.x] = s;
    }
}

}  // namespace

int32_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, int blocks, hipStream_t st) {
    hipLaunchKernelGGL(stream_read, dim3(blocks), dim3(256), 0, st, (const u32x4*)buf, bytes / 16, out);
    return last_launch_status();
}

}  // namespace lrkv
