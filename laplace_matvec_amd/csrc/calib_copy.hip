// A plain device copy of known size, the reference for the HBM traffic
// counters: every element is read once and written once with 4-byte
// accesses, consecutive lanes on consecutive words, as in the operator's
// streaming kernels.  Built into the input library, not the operator.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void lx_calib_copy(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                                                     int64_t words)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride) dst[i] = src[i];
}

}  // namespace

// Copies `words` 32-bit words from src to dst (device pointers, not
// overlapping) on `stream` in one dispatch.  Returns 0, 1 for bad
// arguments, 2 when the launch fails.
extern "C" int laplex_inputs_copy(const void* src, void* dst, int64_t words, void* stream)
{
    if (!src || !dst || words < 0) return 1;
    if (words == 0) return 0;
    int64_t blocks = (words + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    lx_calib_copy<<<(unsigned)blocks, 256, 0, (hipStream_t)stream>>>((const uint32_t*)src, (uint32_t*)dst, words);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
