// Device side of the seeded, counter-based input generator (see gen.py for the
// definition).  Random-number generation only: no attention, encoder or
// decoder arithmetic lives here.  Element i of a tensor gets
//   w   = splitmix64_mix(key + (idx0 + i + 1) * 0x9E3779B97F4A7C15)
//   v   = fp32(sum of the four 16-bit fields of w - 131070) * mult
// stored as fp32 or as bf16 (round to nearest even on the fp32 bits).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

__global__ void gen_normal_kernel(void *dst, int bf16, uint64_t n, uint64_t key, uint64_t idx0,
                                  float mult) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint64_t w = mix64(key + (idx0 + i + 1) * 0x9E3779B97F4A7C15ull);
    const int32_t s = (int32_t)((w & 0xFFFF) + ((w >> 16) & 0xFFFF) + ((w >> 32) & 0xFFFF) + (w >> 48)) - 131070;
    const float v = __fmul_rn((float)s, mult);
    if (bf16) {
      const uint32_t u = __float_as_uint(v);
      ((uint16_t *)dst)[i] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
    } else {
      ((float *)dst)[i] = v;
    }
  }
}

}  // namespace

extern "C" int llagen_normal(void *dst, int bf16, uint64_t n, uint64_t key, uint64_t idx0,
                             float mult, hipStream_t stream) {
  if (n == 0) return 0;
  if (!dst) return -1;
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(gen_normal_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dst, bf16, n,
                     key, idx0, mult);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
