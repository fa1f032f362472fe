// Split merge + V up-projection for decode / prefill attention (per-head LLA
// and LLA-2D, every storage type).
//
// A split of the context leaves, per (row, head), its running max m (base 2),
// its weight sum Z and its latent-space value sum acc[r_v] (partials layout
// [rows][H][splits][r_v + 2]).  The merge is the usual log-sum-exp combination,
// reduced in a fixed order (deterministic):
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

// Work split: lanes run over splits (a row's splits are independent), so the
// cost per (row, head) is ceil(S / threads) partial rows per thread plus one
// cross-lane reduction per output column.  WPR waves share one (row, head):
// 4 (the whole workgroup) when a row has many splits (long contexts at small
// batch), else 1 (4 (row, head) pairs per workgroup).  IDENT: the partials
// already hold the output row (full-cache decode, r_v = d_head): no
// up-projection, no mu.
template <bool BF, bool IDENT, int WPR>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a, int d_head, int r_v) {
  extern __shared__ float s_an[];  // [4 / WPR][r_v]
  __shared__ float s_red[4][33];
  constexpr int G = 64 * WPR;      // threads per (row, head)
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int grp = threadIdx.x / G, u = threadIdx.x % G, wg = w % WPR;
  const long long rh = (long long)blockIdx.x * (4 / WPR) + grp;  // row * H + head
  const bool live = rh < (long long)a.rows * a.H;                // uniform per group
  const int h = live ? (int)(rh % a.H) : 0;
  const int S = a.splits, stride = r_v + 2;
  const float *pb = a.partials + (live ? rh : 0) * S * stride;
  float *an = s_an + grp * r_v;

  // group-wide max / sum: wave reduction, then (WPR = 4) across the 4 waves
  auto group_sum = [&](float x, int slot) -> float {
    x = sum_across_rows(sum_in_row(x));
    if constexpr (WPR == 1) return x;
    if (lane == 0) s_red[wg][slot] = x;
    __syncthreads();
    const float t = s_red[0][slot] + s_red[1][slot] + s_red[2][slot] + s_red[3][slot];
    __syncthreads();
    return t;
  };

  float M = -INFINITY;
  if (live)
    for (int s = u; s < S; s += G) M = fmaxf(M, pb[(long long)s * stride + r_v]);
  M = max_in_wave(M);
  if constexpr (WPR == 4) {
    if (lane == 0) s_red[wg][32] = M;
    __syncthreads();
    M = fmaxf(fmaxf(s_red[0][32], s_red[1][32]), fmaxf(s_red[2][32], s_red[3][32]));
    __syncthreads();
  }
  // A split that saw no token (m = -inf: its pages all lie past the row's
  // context) weighs 0; exp2(-inf - M) would be NaN when M is -inf as well.
  auto weight = [&](float m) -> float { return m == -INFINITY ? 0.f : exp2f(m - M); };
  float Z = 0.f;
  if (live)
    for (int s = u; s < S; s += G) {
      const float m = pb[(long long)s * stride + r_v];
      Z += weight(m) * pb[(long long)s * stride + r_v + 1];  // NaN Z poisons the row
    }
  Z = group_sum(Z, 32);

  // value sums, 32 columns at a time: each thread folds its splits' columns
  for (int c0 = 0; c0 < r_v; c0 += 32) {
    float acc[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) acc[k] = 0.f;
    if (live)
      for (int s = u; s < S; s += G) {
        const float *row = pb + (long long)s * stride;
        const float wgt = weight(row[r_v]);
#pragma unroll
        for (int k = 0; k < 32; k += 2) {
          if (c0 + k < r_v) {  // r_v is a multiple of 8: pairs stay whole
            const float2 v = *(const float2 *)(row + c0 + k);
            acc[k] = fmaf(wgt, v.x, acc[k]);
            acc[k + 1] = fmaf(wgt, v.y, acc[k + 1]);
          }
        }
      }
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const float t = sum_across_rows(sum_in_row(acc[k]));
      if constexpr (WPR == 1) {
        if (lane == k && c0 + k < r_v) an[c0 + k] = t / Z;
      } else {
        if (lane == 0) s_red[wg][k] = t;
      }
    }
    if constexpr (WPR == 4) {
      __syncthreads();
      if (threadIdx.x < 32 && c0 + (int)threadIdx.x < r_v) {
        const int k = threadIdx.x;
        an[c0 + k] = (s_red[0][k] + s_red[1][k] + s_red[2][k] + s_red[3][k]) / Z;
      }
      __syncthreads();
    }
  }
  __syncthreads();
  if (!live) return;  // after the last barrier

  if constexpr (IDENT) {
    for (int e = u; e < d_head; e += G) ((uint16_t *)a.out)[rh * d_head + e] = (uint16_t)f32_to_bf16(an[e]);
    return;
  }
  const int esz = BF ? 2 : 4;
  const char *wv = a.wup_v + (long long)h * a.wup_head_stride_v * esz;
  const char *mu = a.mu_v + (long long)h * a.mu_head_stride * esz;
  for (int e = u; e < d_head; e += G) {
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

// The same merge for few splits and narrow latents (S <= 64, r_v = RV in
// {32, 64}, d_head in {64, 128}), shaped for latency: one wave per (row,
// head); its decoder rows and mu are loaded first (they do not depend on the
// partials), lane s loads split s's whole partial row in one batch, and every
// lane ends with the merged latent vector in registers after one wave
// reduction per value.  Same reduction trees and fma order as merge_kernel,
// so the results are bitwise the same; the memory round trips per (row,
// head) drop from four dependent ones to one.
template <bool BF, int RV, int EPL>
__global__ __launch_bounds__(256) void merge_few_kernel(AttnArgs a) {
  constexpr int DH = 64 * EPL;
  constexpr int ES = BF ? 2 : 4;
  constexpr int WV = RV * ES / 16;  // 16-byte loads per decoder row
  const int lane = threadIdx.x & 63;
  const long long rh = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);  // row * H + head
  if (rh >= (long long)a.rows * a.H) return;  // a whole wave; no barrier follows
  const int h = (int)(rh % a.H), S = a.splits;
  const char *wv = a.wup_v + (long long)h * a.wup_head_stride_v * ES;
  const char *mu = a.mu_v + (long long)h * a.mu_head_stride * ES;
  u32x4 wr[EPL][WV];
  float mue[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
#pragma unroll
    for (int i = 0; i < WV; ++i) wr[j][i] = *(const u32x4 *)(wv + ((long long)e * RV * ES + 16 * i));
    mue[j] = BF ? bf16_to_f32(((const uint16_t *)mu)[e]) : ((const float *)mu)[e];
  }
  constexpr int STRIDE = RV + 2;
  const float *ps = a.partials + (rh * S + lane) * STRIDE;
  float v[STRIDE];
  const bool mine = lane < S;
#pragma unroll
  for (int k = 0; k < STRIDE; k += 2) {
    const float2 t = mine ? *(const float2 *)(ps + k) : float2{-INFINITY, 0.f};
    v[k] = t.x;
    v[k + 1] = t.y;
  }
  const float m = mine ? v[RV] : -INFINITY;
  const float M = max_in_wave(m);
  // a split that saw no token (m = -inf) weighs 0; a NaN Z poisons the row
  const float wgt = m == -INFINITY ? 0.f : exp2f(m - M);
  const float Z = sum_across_rows(sum_in_row(mine ? wgt * v[RV + 1] : 0.f));
  float an[RV];
#pragma unroll
  for (int k = 0; k < RV; ++k) an[k] = sum_across_rows(sum_in_row(fmaf(wgt, mine ? v[k] : 0.f, 0.f))) / Z;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    float o = mue[j];
    if constexpr (BF) {
#pragma unroll
      for (int i = 0; i < WV; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          o = fmaf(bf16_lo(wr[j][i][k]), an[8 * i + 2 * k], o);
          o = fmaf(bf16_hi(wr[j][i][k]), an[8 * i + 2 * k + 1], o);
        }
      ((uint16_t *)a.out)[rh * DH + e] = (uint16_t)f32_to_bf16(o);
    } else {
#pragma unroll
      for (int i = 0; i < WV; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) o = fmaf(__uint_as_float(wr[j][i][k]), an[4 * i + k], o);
      ((float *)a.out)[rh * DH + e] = o;
    }
  }
}

// The same for 64 < S <= 256: one workgroup per (row, head), thread s loads
// split s's partial row; wave reductions, then the four waves' results added
// in wave order through LDS (as merge_kernel with WPR = 4), with two barriers.
template <bool BF, int RV, int EPL>
__global__ __launch_bounds__(256) void merge_many_kernel(AttnArgs a) {
  constexpr int DH = 64 * EPL;
  constexpr int ES = BF ? 2 : 4;
  constexpr int WV = RV * ES / 16;
  constexpr int STRIDE = RV + 2;
  __shared__ float s_red[4][STRIDE];
  const int u = threadIdx.x, lane = u & 63, wg = u >> 6;
  const long long rh = blockIdx.x;  // row * H + head
  const int h = (int)(rh % a.H), S = a.splits;
  const char *wv = a.wup_v + (long long)h * a.wup_head_stride_v * ES;
  const char *mu = a.mu_v + (long long)h * a.mu_head_stride * ES;
  const bool has_e = u < DH;  // thread u writes output element u
  u32x4 wr[WV];
  float mue = 0.f;
  if (has_e) {
#pragma unroll
    for (int i = 0; i < WV; ++i) wr[i] = *(const u32x4 *)(wv + ((long long)u * RV * ES + 16 * i));
    mue = BF ? bf16_to_f32(((const uint16_t *)mu)[u]) : ((const float *)mu)[u];
  }
  const float *ps = a.partials + (rh * S + u) * STRIDE;
  float v[STRIDE];
  const bool mine = u < S;
#pragma unroll
  for (int k = 0; k < STRIDE; k += 2) {
    const float2 t = mine ? *(const float2 *)(ps + k) : float2{-INFINITY, 0.f};
    v[k] = t.x;
    v[k + 1] = t.y;
  }
  const float m = mine ? v[RV] : -INFINITY;
  const float mw = max_in_wave(m);
  if (lane == 0) s_red[wg][RV] = mw;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0][RV], s_red[1][RV]), fmaxf(s_red[2][RV], s_red[3][RV]));
  const float wgt = m == -INFINITY ? 0.f : exp2f(m - M);
  const float zw = sum_across_rows(sum_in_row(mine ? wgt * v[RV + 1] : 0.f));
  if (lane == 0) s_red[wg][RV + 1] = zw;
#pragma unroll
  for (int k = 0; k < RV; ++k) {
    const float t = sum_across_rows(sum_in_row(fmaf(wgt, mine ? v[k] : 0.f, 0.f)));
    if (lane == 0) s_red[wg][k] = t;
  }
  __syncthreads();
  if (!has_e) return;  // after the last barrier
  const float Z = s_red[0][RV + 1] + s_red[1][RV + 1] + s_red[2][RV + 1] + s_red[3][RV + 1];
  float o = mue;
#pragma unroll
  for (int i = 0; i < WV; ++i) {
    if constexpr (BF) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = 8 * i + 2 * k;
        o = fmaf(bf16_lo(wr[i][k]), (s_red[0][c] + s_red[1][c] + s_red[2][c] + s_red[3][c]) / Z, o);
        o = fmaf(bf16_hi(wr[i][k]), (s_red[0][c + 1] + s_red[1][c + 1] + s_red[2][c + 1] + s_red[3][c + 1]) / Z, o);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = 4 * i + k;
        o = fmaf(__uint_as_float(wr[i][k]), (s_red[0][c] + s_red[1][c] + s_red[2][c] + s_red[3][c]) / Z, o);
      }
    }
  }
  if constexpr (BF) ((uint16_t *)a.out)[rh * DH + u] = (uint16_t)f32_to_bf16(o);
  else ((float *)a.out)[rh * DH + u] = o;
}

namespace {
constexpr int kWholeGroupSplits = 64;  // more splits than this: 4 waves per (row, head)

template <bool BF>
bool go_merge_few(const AttnArgs &a, int d_head, int r_v, long long blocks, hipStream_t stream) {
  if (a.splits > 256) return false;
  const bool many = a.splits > 64;  // then blocks is the (row, head) count
#define LLA_MERGE_FEW(RV, EPL)                                                                      \
  if (r_v == RV && d_head == 64 * EPL) {                                                            \
    if (many)                                                                                       \
      hipLaunchKernelGGL((merge_many_kernel<BF, RV, EPL>), dim3((unsigned)blocks), dim3(256), 0, stream, a); \
    else                                                                                            \
      hipLaunchKernelGGL((merge_few_kernel<BF, RV, EPL>), dim3((unsigned)blocks), dim3(256), 0, stream, a); \
    return true;                                                                                    \
  }
  LLA_MERGE_FEW(32, 1) LLA_MERGE_FEW(32, 2) LLA_MERGE_FEW(64, 1) LLA_MERGE_FEW(64, 2)
#undef LLA_MERGE_FEW
  return false;
}

template <bool BF, bool IDENT>
hipError_t go_merge(const AttnArgs &a, int d_head, int r_v, hipStream_t stream) {
  if (r_v % 8) return hipErrorInvalidConfiguration;
  const long long pairs = (long long)a.rows * a.H;
  const bool whole = a.splits > kWholeGroupSplits;
  const long long blocks = whole ? pairs : (pairs + 3) / 4;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if constexpr (!IDENT) {
    if (go_merge_few<BF>(a, d_head, r_v, blocks, stream)) return hipGetLastError();
  }
  const size_t shmem = sizeof(float) * (whole ? 1 : 4) * r_v;
  if (whole)
    hipLaunchKernelGGL((merge_kernel<BF, IDENT, 4>), dim3((unsigned)blocks), dim3(256), shmem, stream, a, d_head, r_v);
  else
    hipLaunchKernelGGL((merge_kernel<BF, IDENT, 1>), dim3((unsigned)blocks), dim3(256), shmem, stream, a, d_head, r_v);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_merge_ident(int d_head, const AttnArgs &a, hipStream_t stream) {
  return go_merge<true, true>(a, d_head, d_head, stream);
}

hipError_t launch_merge(int dtype, int d_head, int r_v, const AttnArgs &a, hipStream_t stream) {
  return dtype == LLA_BF16 ? go_merge<true, false>(a, d_head, r_v, stream)
                           : go_merge<false, false>(a, d_head, r_v, stream);
}

}  // namespace lla
