// Split-K merge of per-chunk softmax states (PuzzleKV section 3.3, step 4:
// partial results merged by online softmax; the same merge combines the
// sequence chunks of every decode mode).
#include "common.h"

#include <math.h>

namespace lrkv {
namespace {

// out[b][j][d] = sum_c 2^(m_c - M) acc_c[d] / sum_c 2^(m_c - M) l_c over the
// n_split chunks (at most 1024); empty chunks (m = -inf) contribute nothing.
// The chunk maxima and weights are loaded once into LDS by the whole block.
__global__ __launch_bounds__(256) void merge_splits(const float* __restrict__ part,
                                                    float* __restrict__ out, int n_split, int D) {
    __shared__ float wts[1024];
    __shared__ float red[256];
    const long bj = blockIdx.x;
    const float* pp = part + bj * n_split * (D + 2);
    float mx = -INFINITY;
    for (int c = threadIdx.x; c < n_split; c += blockDim.x) {
        const float m = pp[(long)c * (D + 2)];
        wts[c] = m;
        mx = fmaxf(mx, m);
    }
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
        __syncthreads();
    }
    mx = red[0];
    __syncthreads();
    float den = 0.0f;
    for (int c = threadIdx.x; c < n_split; c += blockDim.x) {
        const float m = wts[c];
        const float wgt = m == -INFINITY ? 0.0f : exp2f(m - mx);
        wts[c] = wgt;
        den = fmaf(wgt, pp[(long)c * (D + 2) + 1], den);
    }
    red[threadIdx.x] = den;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    const float rden = 1.0f / red[0];
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float n0 = 0.0f, n1 = 0.0f, n2 = 0.0f, n3 = 0.0f;
        int c = 0;
        for (; c + 4 <= n_split; c += 4) {
            n0 = fmaf(wts[c], pp[(long)c * (D + 2) + 2 + d], n0);
            n1 = fmaf(wts[c + 1], pp[(long)(c + 1) * (D + 2) + 2 + d], n1);
            n2 = fmaf(wts[c + 2], pp[(long)(c + 2) * (D + 2) + 2 + d], n2);
            n3 = fmaf(wts[c + 3], pp[(long)(c + 3) * (D + 2) + 2 + d], n3);
        }
        for (; c < n_split; ++c) n0 = fmaf(wts[c], pp[(long)c * (D + 2) + 2 + d], n0);
        out[bj * D + d] = ((n0 + n1) + (n2 + n3)) * rden;
    }
}

}  // namespace

void launch_merge(const float* part, float* out, int BH, int n_split, int D, hipStream_t st) {
    hipLaunchKernelGGL(merge_splits, dim3(BH), dim3(256), 0, st, part, out, n_split, D);
}

}  // namespace lrkv
