// Encode + append, eq. (2) of the cc.laoqi.cc close reading (方法 item 1) and
// the gist.science "Kernmechanismus": c = (x - mu) W_down over the
// loop-concatenated pre-RoPE vector x = [x_1; ...; x_T], written to the paged
// latent pool at the slot of logical position pos0[b] + n.
//
// Computed as x W_down - (mu W_down): mu W_down is a per-(layer, head) constant
// (first kernel, fp32), the contraction accumulates exact bf16 x fp32 products
// in fp32, and the result is rounded once to the storage type.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {

template <bool BF>
__device__ __forceinline__ float ldx(const char *p, long long i) {
  if constexpr (BF) return bf16_to_f32(((const uint16_t *)p)[i]);
  else return ((const float *)p)[i];
}

// muw[li][grp][kv ? RK + r : r] = sum_i mu[i] W_down[i][r]
template <bool BF>
__global__ __launch_bounds__(256) void encode_muw_kernel(EncodeArgs a, int RK, int RV) {
  const int grp = blockIdx.x, li = blockIdx.y, kv = blockIdx.z;
  const int R = kv ? RV : RK;
  const int esz = BF ? 2 : 4;
  const long long gl = (long long)li * a.groups + grp;  // relative to layer0
  const char *mu = (kv ? a.mu_v : a.mu_k) + gl * a.width * esz;
  const char *wd = (kv ? a.wd_v : a.wd_k) + gl * a.width * (long long)R * esz;
  for (int r = threadIdx.x; r < R; r += blockDim.x) {
    float acc = 0.f;
    for (int i = 0; i < a.width; ++i) acc = fmaf(ldx<BF>(mu, i), ldx<BF>(wd, (long long)i * R + r), acc);
    a.muw[gl * (RK + RV) + (kv ? RK : 0) + r] = acc;
  }
}

// One workgroup per (16-token tile, group, layer*2 + kv).
template <bool BF>
__global__ __launch_bounds__(256) void encode_append_kernel(EncodeArgs a, int RK, int RV) {
  constexpr int TT = 16;
  const int grp = blockIdx.y, li = blockIdx.z >> 1, kv = blockIdx.z & 1;
  const int R = kv ? RV : RK;
  const int esz = BF ? 2 : 4;
  const long long tokens = (long long)a.batch * a.n_new;
  const long long tok0 = (long long)blockIdx.x * TT;
  const long long gl = (long long)li * a.groups + grp;
  const char *x = kv ? a.x_v : a.x_k;
  const char *wd = (kv ? a.wd_v : a.wd_k) + gl * a.width * (long long)R * esz;
  char *pool = (kv ? a.v_pool : a.k_pool) + (long long)li * (kv ? a.pool_layer_stride_v : a.pool_layer_stride_k) * esz;
  const long long pstride = kv ? a.pool_page_stride_v : a.pool_page_stride_k;
  const long long hstride = kv ? a.pool_head_stride_v : a.pool_head_stride_k;
  const float *muw = a.muw + gl * (RK + RV) + (kv ? RK : 0);
  for (int idx = threadIdx.x; idx < TT * R; idx += blockDim.x) {
    const long long tok = tok0 + idx / R;
    const int r = idx % R;
    if (tok >= tokens) continue;
    const int b = (int)(tok / a.n_new), n = (int)(tok % a.n_new);
    const long long pos = (long long)a.pos0[b] + n;
    if (pos < 0 || pos >= (long long)a.max_pages * kPage) {
      atomicOr(a.err, LLA_DEVERR_APPEND);
      continue;
    }
    const int page = a.page_table[(long long)b * a.max_pages + pos / kPage];
    if (page < 0 || page >= a.num_pages) {
      atomicOr(a.err, LLA_DEVERR_PAGE);
      continue;
    }
    const char *xr = x + ((((long long)li * a.batch + b) * a.n_new + n) * a.groups + grp) * a.width * esz;
    float acc = 0.f;
    for (int i = 0; i < a.width; ++i) acc = fmaf(ldx<BF>(xr, i), ldx<BF>(wd, (long long)i * R + r), acc);
    acc -= muw[r];
    const long long off = (long long)page * pstride + grp * hstride + (pos % kPage) * R + r;
    if constexpr (BF) ((uint16_t *)pool)[off] = (uint16_t)f32_to_bf16(acc);
    else ((float *)pool)[off] = acc;
  }
}

bool encode_supported(int dtype, int width, int r_k, int r_v) {
  return (dtype == LLA_BF16 || dtype == LLA_F32) && width > 0 && r_k > 0 && r_v > 0;
}

hipError_t launch_encode(int dtype, int r_k, int r_v, const EncodeArgs &a, hipStream_t stream) {
  const long long tokens = (long long)a.batch * a.n_new;
  if (tokens == 0 || a.n_layers == 0) return hipSuccess;
  const dim3 g1(a.groups, a.n_layers, 2);
  const dim3 g2((unsigned)((tokens + 15) / 16), a.groups, 2 * a.n_layers);
  if (dtype == LLA_BF16) {
    hipLaunchKernelGGL(encode_muw_kernel<true>, g1, dim3(256), 0, stream, a, r_k, r_v);
    hipLaunchKernelGGL(encode_append_kernel<true>, g2, dim3(256), 0, stream, a, r_k, r_v);
  } else {
    hipLaunchKernelGGL(encode_muw_kernel<false>, g1, dim3(256), 0, stream, a, r_k, r_v);
    hipLaunchKernelGGL(encode_append_kernel<false>, g2, dim3(256), 0, stream, a, r_k, r_v);
  }
  return hipGetLastError();
}

}  // namespace lla
