// sdm_round_bf16: float32 -> bfloat16 with the conversion every libsdm kernel
// uses when it stores a bfloat16 (the packed conversion of sdm_kernels.h, two
// values per instruction), exposed so that it can be checked on its own.

#include "sdm_kernels.h"

namespace sdm {

namespace {

// Thread i converts the pair (2i, 2i + 1), grid-stride; an odd last element is
// converted alone (paired with +0, whose half is dropped).
__global__ __launch_bounds__(256) void round_bf16_kernel(const float* __restrict__ in, uint16_t* __restrict__ out,
                                                         int64_t n) {
    const int64_t pairs = n / 2;
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < pairs; i += stride) {
        const float2 f = reinterpret_cast<const float2*>(in)[i];
        reinterpret_cast<uint32_t*>(out)[i] = to_bf16x2_rne(f.x, f.y);
    }
    if (n % 2 == 1 && blockIdx.x == 0 && threadIdx.x == 0) out[n - 1] = to_bf16_rne(in[n - 1]);
}

}  // namespace

hipError_t launch_round_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t stream) {
    int64_t blocks = (n / 2 + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(round_bf16_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, in, out, n);
    return hipGetLastError();
}

}  // namespace sdm
