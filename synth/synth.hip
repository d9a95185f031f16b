// synth.hip -- GPU generator of the seeded synthetic fp16 Linear weights.
//
// Input generation only (no arithmetic of the quantization method).  The
// definition is the one documented in synth/__init__.py: SplitMix64 counter
// bits, Box-Muller normals, a lognormal(0, 0.5) factor per output row and
// 0.1% outliers scaled by 20, all in fp64, rounded once to fp16.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t x)
{
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t bits(uint64_t key, uint64_t stream, uint64_t counter)
{
    return mix64(key ^ (stream << 56) ^ counter);
}

__device__ __forceinline__ double unit24(uint64_t a) { return ((double)a + 0.5) / 16777216.0; }

__device__ __forceinline__ double normal(uint64_t h)
{
    const double two_pi = 6.283185307179586;   // fp64 value of 2*pi (numpy's 2.0 * np.pi)
    double u1 = unit24(h >> 40);
    double u2 = unit24((h >> 16) & 0xFFFFFFull);
    return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

// fp64 -> fp16 bits, one round-to-nearest-even rounding
__device__ __forceinline__ uint16_t to_half_rne(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (isnan(a)) return (uint16_t)(sign | 0x7e00u);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u);
    if (a < 6.103515625e-05) {
        double m = rint(a * 16777216.0);
        return (uint16_t)(sign | (uint16_t)m);
    }
    int e;
    frexp(a, &e);
    double m = rint(ldexp(a, 11 - e));
    int biased = e - 1 + 15;
    if (m == 2048.0) { m = 1024.0; biased += 1; }
    if (biased >= 31) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)(biased << 10) | (uint16_t)((int)m - 1024));
}

__global__ void synth_fill_kernel(uint16_t *__restrict__ out, int64_t row0, int64_t nrows,
                                  int64_t cols, uint64_t key)
{
    const int64_t n = nrows * cols;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int64_t r = row0 + i / cols;
        const int64_t c = i % cols;
        const uint64_t idx = (uint64_t)(r * cols + c);
        const double f = exp(0.5 * normal(bits(key, 1, (uint64_t)r)));
        const double z = normal(bits(key, 0, idx));
        const double u = unit24(bits(key, 2, idx) >> 40);
        const double o = u < 0.001 ? 20.0 : 1.0;
        out[i] = to_half_rne(((0.02 * z) * f) * o);
    }
}

}  // namespace

// Fill out[nrows, cols] (fp16 bits, device memory) with rows row0 .. row0+nrows-1
// of the tensor identified by key.  Returns 0, or a negative HIP failure.
extern "C" int hqq_synth_fill(uint16_t *out, int64_t row0, int64_t nrows, int64_t cols,
                              uint64_t key, void *stream)
{
    if (!out || row0 < 0 || nrows < 0 || cols < 1) return -1;
    if (nrows == 0) return 0;
    const int64_t n = nrows * cols;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(synth_fill_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, out, row0, nrows, cols, key);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}
