// Split merge + V up-projection for decode / prefill attention (per-head LLA
// and LLA-2D, every storage type).
//
// A split of the context leaves, per (row, head), its running max m (base 2),
// its weight sum Z and its latent-space value sum acc[r_v] (partials layout
// [rows][H][splits][r_v + 2]).  The merge is the usual log-sum-exp combination
// in fixed split order (deterministic):
//   M = max_s m_s,   Z = sum_s 2^{m_s - M} Z_s,   a[r] = sum_s 2^{m_s - M} acc_s[r] / Z,
// followed by the one up-projection per (row, head) that linearity of the
// decoder allows (cc.laoqi.cc close reading, 方法 item 1, eq. (3)):
//   out[e] = mu_v,t[e] + sum_r a[r] W_up,v,t[e][r].
// It runs as its own launch after the attention kernel: the kernel boundary
// makes the partials visible, so the attention kernel needs no device-scope
// fences or completion counters (a device-scope fence writes back and
// invalidates an XCD's whole L2).
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {

// One wave per (row, head); 4 per workgroup.  IDENT: the partials already hold
// the output row (full-cache decode, r_v = d_head): no up-projection, no mu.
template <bool BF, bool IDENT = false>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a, int d_head, int r_v) {
  extern __shared__ float s_an[];  // [4][r_v]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long long rh = (long long)blockIdx.x * 4 + w;  // row * H + head
  if (rh >= (long long)a.rows * a.H) return;           // whole wave leaves together
  const int h = (int)(rh % a.H);
  const int S = a.splits;
  const float *pb = a.partials + rh * S * (r_v + 2);
  float *an = s_an + w * r_v;

  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, pb[(long long)s * (r_v + 2) + r_v]);
  M = max_in_wave(M);
  float Z = 0.f;
  for (int s = lane; s < S; s += 64) {
    const float m = pb[(long long)s * (r_v + 2) + r_v];
    Z += exp2f(m - M) * pb[(long long)s * (r_v + 2) + r_v + 1];  // NaN Z poisons the row
  }
  for (int o = 32; o >= 1; o >>= 1) Z += __shfl_xor(Z, o);
  for (int r = lane; r < r_v; r += 64) {
    float acc = 0.f;
    for (int s = 0; s < S; ++s) {
      const float m = pb[(long long)s * (r_v + 2) + r_v];
      acc = fmaf(exp2f(m - M), pb[(long long)s * (r_v + 2) + r], acc);
    }
    an[r] = acc / Z;
    if constexpr (IDENT) ((uint16_t *)a.out)[rh * d_head + r] = (uint16_t)f32_to_bf16(an[r]);
  }
  if constexpr (IDENT) return;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const int esz = BF ? 2 : 4;
  const char *wv = a.wup_v + (long long)h * a.wup_head_stride_v * esz;
  const char *mu = a.mu_v + (long long)h * a.mu_head_stride * esz;
  for (int e = lane; e < d_head; e += 64) {
    const char *we = wv + (long long)e * r_v * esz;
    float o;
    if constexpr (BF) {
      o = bf16_to_f32(((const uint16_t *)mu)[e]);
      for (int r8 = 0; r8 < r_v / 8; ++r8) {
        const u32x4 v = *(const u32x4 *)(we + r8 * 16);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          o = fmaf(bf16_lo(v[k]), an[8 * r8 + 2 * k], o);
          o = fmaf(bf16_hi(v[k]), an[8 * r8 + 2 * k + 1], o);
        }
      }
      ((uint16_t *)a.out)[rh * d_head + e] = (uint16_t)f32_to_bf16(o);
    } else {
      o = ((const float *)mu)[e];
      for (int r4 = 0; r4 < r_v / 4; ++r4) {
        const f32x4 v = *(const f32x4 *)(we + r4 * 16);
#pragma unroll
        for (int k = 0; k < 4; ++k) o = fmaf(v[k], an[4 * r4 + k], o);
      }
      ((float *)a.out)[rh * d_head + e] = o;
    }
  }
}

hipError_t launch_merge_ident(int d_head, const AttnArgs &a, hipStream_t stream) {
  const long long waves = (long long)a.rows * a.H;
  const long long blocks = (waves + 3) / 4;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((merge_kernel<true, true>), dim3((unsigned)blocks), dim3(256), sizeof(float) * 4 * d_head,
                     stream, a, d_head, d_head);
  return hipGetLastError();
}

hipError_t launch_merge(int dtype, int d_head, int r_v, const AttnArgs &a, hipStream_t stream) {
  if (r_v % 8) return hipErrorInvalidConfiguration;
  const long long waves = (long long)a.rows * a.H;
  const long long blocks = (waves + 3) / 4;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const size_t shmem = sizeof(float) * 4 * r_v;
  if (dtype == LLA_BF16)
    hipLaunchKernelGGL(merge_kernel<true>, dim3((unsigned)blocks), dim3(256), shmem, stream, a, d_head, r_v);
  else
    hipLaunchKernelGGL(merge_kernel<false>, dim3((unsigned)blocks), dim3(256), shmem, stream, a, d_head, r_v);
  return hipGetLastError();
}

}  // namespace lla
