// Device input generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC'11) with the conversions
// of laplace_matvec_amd/workloads.py, for inputs too large to draw on the
// host.  Not part of the operator library: it only makes test and benchmark
// inputs, and holds none of the operator's arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

struct U4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ U4 philox4x32_10(uint64_t block, uint32_t k0, uint32_t k1)
{
    uint32_t c0 = (uint32_t)block, c1 = (uint32_t)(block >> 32), c2 = 0, c3 = 0;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return U4{c0, c1, c2, c3};
}

__device__ __forceinline__ uint32_t word_of(const U4& u, int i)
{
    return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

// kind 0: normal (mean p, scale q); kind 1: uniform [p, q); kind 2: raw u32
__global__ __launch_bounds__(256) void lx_gen(void* out, int64_t n, int64_t offset, uint32_t k0, uint32_t k1,
                                             int kind, double p, double q)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const double two32 = 2.3283064365386963e-10;  // 2^-32
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int64_t e = offset + i;
        const U4 u = philox4x32_10((uint64_t)(e >> 2), k0, k1);
        const int w = (int)(e & 3);
        if (kind == 2) {
            ((uint32_t*)out)[i] = word_of(u, w);
        } else if (kind == 1) {
            const double f = (double)word_of(u, w) * two32;
            ((float*)out)[i] = (float)(p + (q - p) * f);
        } else {
            const int pair = w >> 1;
            const double a = (double)(pair ? u.z : u.x);
            const double b = (double)(pair ? u.w : u.y);
            const double r = sqrt(-2.0 * log((a + 1.0) * two32));
            const double t = 6.283185307179586 * (b * two32);
            const double z = (w & 1) ? r * sin(t) : r * cos(t);
            ((float*)out)[i] = (float)(p + q * z);
        }
    }
}

}  // namespace

extern "C" int laplex_inputs_generate(void* out, int64_t n, int64_t offset, uint32_t key0, uint32_t key1,
                                      int kind, double p, double q, void* stream)
{
    if (!out || n < 0 || offset < 0 || kind < 0 || kind > 2) return 1;
    if (n == 0) return 0;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipStream_t s = (hipStream_t)stream;
    lx_gen<<<(unsigned)blocks, 256, 0, s>>>(out, n, offset, key0, key1, kind, p, q);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
