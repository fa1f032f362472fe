// Encode + append, eq. (2) of the cc.laoqi.cc close reading (方法 item 1) and
// the gist.science "Kernmechanismus": c = (x - mu) W_down over the
// loop-concatenated pre-RoPE vector x = [x_1; ...; x_T], written to the paged
// latent pool at the slot of logical position pos0[b] + n.
//
// Computed as x W_down - (mu W_down): mu W_down is a per-(layer, group)
// constant (first kernel, fp32), the contraction accumulates exact products in
// fp32, and the result is rounded once to the storage type.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {

template <bool BF>
__device__ __forceinline__ float ldx(const char *p, long long i) {
  if constexpr (BF) return bf16_to_f32(((const uint16_t *)p)[i]);
  else return ((const float *)p)[i];
}

// muw[li][grp][kv ? RK + r : r] = sum_i mu[i] W_down[i][r], fp32: a constant of
// (layer, latent group), computed once per call and shared by every token tile.
// The rows of W_down are cut into muw_parts ranges of kMuwRows rows, summed by
// separate workgroups (one per (range, group), layer, K|V) into muw_part; a
// second launch adds the ranges in fixed order.  Within a range, wave w sums
// rows w, w + 4, ... (lanes over r, coalesced rows of W_down) and the 4 wave
// sums are added in fixed order.
constexpr int kMuwRows = 64;

int encode_muw_parts(int width) { return (width + kMuwRows - 1) / kMuwRows; }

template <bool BF>
__global__ __launch_bounds__(256) void encode_muw_kernel(EncodeArgs a, int RK, int RV) {
  __shared__ float part[4][256];
  const int grp = blockIdx.x % a.groups, pr = blockIdx.x / a.groups;
  const int li = blockIdx.y, kv = blockIdx.z;
  const int R = kv ? RV : RK;
  const int esz = BF ? 2 : 4;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long long gl = (long long)li * a.groups + grp;  // relative to layer0
  const char *mu = (kv ? a.mu_v : a.mu_k) + gl * a.width * esz;
  const char *wd = (kv ? a.wd_v : a.wd_k) + gl * a.width * (long long)R * esz;
  const int i0 = pr * kMuwRows, i1 = min(i0 + kMuwRows, a.width);
  float *dst = a.muw_part + ((long long)pr * a.n_layers * a.groups + gl) * (RK + RV) + (kv ? RK : 0);
  for (int r0 = 0; r0 < R; r0 += 256) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i = i0 + w; i < i1; i += 4) {
      const float m = ldx<BF>(mu, i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = r0 + lane + 64 * j;
        if (r < R) acc[j] = fmaf(m, ldx<BF>(wd, (long long)i * R + r), acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) part[w][lane + 64 * j] = acc[j];
    __syncthreads();
    const int r = r0 + threadIdx.x;
    if (r < R) dst[r] = ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) + part[3][threadIdx.x];
    __syncthreads();
  }
}

// muw = sum over the row ranges, in range order.  One thread per
// (layer, group, column).
__global__ __launch_bounds__(256) void encode_muw_reduce_kernel(EncodeArgs a) {
  const long long n = (long long)a.n_layers * a.groups * a.muw_stride;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  float s = 0.f;
  for (int pr = 0; pr < a.muw_parts; ++pr) s += a.muw_part[(long long)pr * n + idx];
  a.muw[idx] = s;
}

namespace {
template <bool BF>
hipError_t launch_muw(int r_k, int r_v, const EncodeArgs &a, hipStream_t stream) {
  const dim3 g1((unsigned)(a.groups * a.muw_parts), a.n_layers, 2);
  hipLaunchKernelGGL(encode_muw_kernel<BF>, g1, dim3(256), 0, stream, a, r_k, r_v);
  const long long n = (long long)a.n_layers * a.groups * a.muw_stride;
  hipLaunchKernelGGL(encode_muw_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}
}  // namespace

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

// ---------------------------------------------------------------- MFMA path (bf16)
//
// Per (layer, latent group, K|V) the encoder is a plain GEMM,
//   C[tokens x r] = X[tokens x width] W_down[width x r] - 1 (mu W_down),
// run on v_mfma_f32_16x16x32_bf16.  A workgroup (8 waves) takes 256 tokens
// (128 for r > 160); wave w owns two 16-row tiles (one) and all r columns, so
// every W_down operand read from LDS feeds two products.  W_down is streamed in
// chunks of 128 rows, transposed into LDS ([r][k], rows padded so the 16-byte
// B-operand reads of 16 consecutive r hit distinct banks) and shared by the 8
// waves; the chunks are software-pipelined: while chunk c multiplies out of
// one LDS buffer, the x rows and W_down rows of chunk c + 1 are in flight and
// land in the other buffer, one barrier per chunk.  K-slot e of K-step s in
// lane group g is chunk column 32 s + 8 g + e on both operands, so each x load
// instruction reads 64 contiguous bytes of every token's row.  mu W_down comes from encode_muw_kernel
// (once per call).  The result (minus mu W_down, rounded once to bf16) goes
// through LDS and leaves as 16-byte stores into the paged pool.
template <int R>
__global__ __launch_bounds__(512) void encode_mfma_kernel(EncodeArgs a, int kv) {
  constexpr int TPW = R <= 160 ? 2 : 1;  // 16-token row tiles per wave (registers bound it)
  constexpr int TOK = 128 * TPW;         // tokens per workgroup
  constexpr int KC = 128;         // W_down rows per chunk
  constexpr int LROW = KC + 8;    // padded LDS row (elements) of the transposed chunk
  constexpr int CT = R / 16;      // column tiles
  static_assert(R % 16 == 0 && R <= 256, "r");
  constexpr int WBUF = R * LROW;  // one transposed chunk
  __shared__ __attribute__((aligned(16))) uint16_t s_w[(2 * WBUF > TOK * R ? 2 * WBUF : TOK * R)];
  __shared__ long long s_off[TOK];  // element offset of each token's latent row, -1 = dropped

  // wave index as a scalar: branches on it must be uniform scalar branches,
  // never EXEC-masked MFMAs
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int grp = blockIdx.y, li = blockIdx.z;
  const long long tokens = (long long)a.batch * a.n_new;
  const long long tok0 = (long long)blockIdx.x * TOK;
  const long long gl = (long long)li * a.groups + grp;
  const char *x = kv ? a.x_v : a.x_k;
  const uint16_t *wd = (const uint16_t *)(kv ? a.wd_v : a.wd_k) + gl * a.width * (long long)R;
  uint16_t *pool = (uint16_t *)(kv ? a.v_pool : a.k_pool) +
                   (long long)li * (kv ? a.pool_layer_stride_v : a.pool_layer_stride_k);
  const long long pstride = kv ? a.pool_page_stride_v : a.pool_page_stride_k;
  const long long hstride = kv ? a.pool_head_stride_v : a.pool_head_stride_k;

  // destination slot of each token (placement is integer work, checked here)
  if (threadIdx.x < TOK) {
    const long long tok = tok0 + threadIdx.x;
    long long off = -1;
    if (tok < tokens) {
      const int b = (int)(tok / a.n_new), nn = (int)(tok % a.n_new);
      const long long pos = (long long)a.pos0[b] + nn;
      if (pos < 0 || pos >= (long long)a.max_pages * kPage) {
        atomicOr(a.err, LLA_DEVERR_APPEND);
      } else {
        const int page = a.page_table[(long long)b * a.max_pages + pos / kPage];
        if (page < 0 || page >= a.num_pages) atomicOr(a.err, LLA_DEVERR_PAGE);
        else off = (long long)page * pstride + grp * hstride + (pos % kPage) * R;
      }
    }
    s_off[threadIdx.x] = off;
  }

  // this lane's x rows: tokens tok0 + 16 (TPW w + tt) + n (clamped; dropped at the end)
  const uint16_t *xr[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    long long tk = tok0 + 16 * (TPW * w + tt) + n;
    if (tk >= tokens) tk = tokens - 1;
    xr[tt] = (const uint16_t *)x + ((li * tokens + tk) * a.groups + grp) * a.width;
  }

  f32x4 acc[TPW][CT];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[tt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = a.width / KC;
  // Software pipeline over 128-row chunks: while chunk c multiplies out of LDS
  // buffer c % 2, the x rows and W_down rows of chunk c + 1 are in flight in
  // registers; W_down goes into the other buffer after the products, then one
  // barrier per chunk.
  constexpr int WT = ((KC / 4) * (R / 8) + 511) / 512;  // transpose tasks per thread
  u32x4 xa[TPW][4], xn[TPW][4], wv[WT][4];
  auto load_x = [&](int c, u32x4 (&dst)[TPW][4]) {
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
      for (int s = 0; s < 4; ++s) dst[tt][s] = *(const u32x4 *)(xr[tt] + c * KC + 32 * s + 8 * g);
  };
  auto load_w = [&](int c) {
#pragma unroll
    for (int j = 0; j < WT; ++j) {
      const int task = min((int)threadIdx.x + 512 * j, (KC / 4) * (R / 8) - 1);
      const int k4 = task / (R / 8), r8 = task % (R / 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[j][i] = *(const u32x4 *)(wd + (long long)(c * KC + 4 * k4 + i) * R + 8 * r8);
    }
  };
  auto store_w = [&](uint16_t *buf) {
#pragma unroll
    for (int j = 0; j < WT; ++j) {
      const int task = (int)threadIdx.x + 512 * j;
      if (task < (KC / 4) * (R / 8)) {
        const int k4 = task / (R / 8), r8 = task % (R / 8);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int sh = (jj & 1) * 16;
          const uint32_t e0 = (wv[j][0][jj >> 1] >> sh) & 0xFFFFu, e1 = (wv[j][1][jj >> 1] >> sh) & 0xFFFFu;
          const uint32_t e2 = (wv[j][2][jj >> 1] >> sh) & 0xFFFFu, e3 = (wv[j][3][jj >> 1] >> sh) & 0xFFFFu;
          uint32_t *dst = (uint32_t *)(buf + (8 * r8 + jj) * LROW + 4 * k4);
          dst[0] = e0 | (e1 << 16);
          dst[1] = e2 | (e3 << 16);
        }
      }
    }
  };
  load_x(0, xa);
  load_w(0);
  store_w(s_w);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const bool more = c + 1 < nchunks;
    if (more) {
      load_x(c + 1, xn);
      load_w(c + 1);
    }
    const uint16_t *buf = s_w + (c & 1) * WBUF;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kk = 32 * s + 8 * g;  // K-step s: 64 contiguous bytes of each token's x row
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const u32x4 bw = *(const u32x4 *)(buf + (16 * ct + n) * LROW + kk);
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
          acc[tt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[tt][s]), as_bf16x8(bw), acc[tt][ct], 0, 0, 0);
      }
    }
    if (more) store_w(s_w + ((c + 1) & 1) * WBUF);
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
      for (int s = 0; s < 4; ++s) xa[tt][s] = xn[tt][s];
  }

  __syncthreads();  // s_w free for output staging
  uint16_t *s_out = s_w;  // [TOK][R] bf16
  const float *muw = a.muw + gl * (a.muw_stride) + (kv ? a.muw_v_off : 0);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int r = 16 * ct + n;
    const float mw = muw[r];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s_out[(16 * (TPW * w + tt) + 4 * g + e) * R + r] = (uint16_t)f32_to_bf16(acc[tt][ct][e] - mw);
  }
  __syncthreads();
  for (int q = threadIdx.x; q < TOK * (R / 8); q += blockDim.x) {
    const int tl = q / (R / 8), c8 = q % (R / 8);
    const long long off = s_off[tl];
    if (off >= 0) *(u32x4 *)(pool + off + 8 * c8) = *(const u32x4 *)(s_out + tl * R + 8 * c8);
  }
}

#define LLA_ENCODE_R(X) X(16) X(32) X(48) X(64) X(96) X(128) X(160) X(256)

bool encode_mfma_r(int r) {
#define X(RR) if (r == RR) return true;
  LLA_ENCODE_R(X)
#undef X
  return false;
}

hipError_t launch_encode_mfma(int r, int kv, const EncodeArgs &a, hipStream_t stream) {
  const long long tokens = (long long)a.batch * a.n_new;
#define X(RR)                                                                                     \
  if (r == RR) {                                                                                  \
    constexpr int tok = RR <= 160 ? 256 : 128;                                                    \
    const dim3 grid((unsigned)((tokens + tok - 1) / tok), a.groups, a.n_layers);                  \
    hipLaunchKernelGGL(encode_mfma_kernel<RR>, grid, dim3(512), 0, stream, a, kv);                \
    return hipGetLastError();                                                                     \
  }
  LLA_ENCODE_R(X)
#undef X
  return hipErrorInvalidConfiguration;
}

bool encode_supported(int dtype, int width, int r_k, int r_v) {
  return (dtype == LLA_BF16 || dtype == LLA_F32) && width > 0 && r_k > 0 && r_v > 0;
}

hipError_t launch_encode(int dtype, int r_k, int r_v, const EncodeArgs &a, hipStream_t stream) {
  const long long tokens = (long long)a.batch * a.n_new;
  if (tokens == 0 || a.n_layers == 0) return hipSuccess;
  // bf16 with whole 128-column chunks and an instantiated rank: matrix cores
  if (dtype == LLA_BF16 && a.width % 128 == 0 && encode_mfma_r(r_k) && encode_mfma_r(r_v) &&
      tokens <= 0x7FFFFFFFLL * 128) {
    hipError_t e = launch_muw<true>(r_k, r_v, a, stream);
    if (e != hipSuccess) return e;
    e = launch_encode_mfma(r_k, 0, a, stream);
    if (e != hipSuccess) return e;
    return launch_encode_mfma(r_v, 1, a, stream);
  }
  const dim3 g2((unsigned)((tokens + 15) / 16), a.groups, 2 * a.n_layers);
  if (dtype == LLA_BF16) {
    const hipError_t e = launch_muw<true>(r_k, r_v, a, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(encode_append_kernel<true>, g2, dim3(256), 0, stream, a, r_k, r_v);
  } else {
    const hipError_t e = launch_muw<false>(r_k, r_v, a, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(encode_append_kernel<false>, g2, dim3(256), 0, stream, a, r_k, r_v);
  }
  return hipGetLastError();
}

}  // namespace lla
