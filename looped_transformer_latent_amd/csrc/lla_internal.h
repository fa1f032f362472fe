// Host-side interfaces between the C ABI layer (lla_api.hip) and the kernel
// launchers.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "lla.h"

namespace lla {

constexpr int kPage = 16;          // tokens per cache page
#ifndef LLA_DECODE_LOOK
#define LLA_DECODE_LOOK 4          // decode: latent pages in flight per wave beyond the one computed
#endif
constexpr int kDecodeRing = LLA_DECODE_LOOK + 2;  // decode page-ring slots = pages per trip
constexpr int kHeaderBytes = 256;  // workspace header: int32 error word at byte 0
constexpr int kMaxPages2d = 1024;  // LLA-2D decode: page-table entries a workgroup stages in LDS

// Arguments of one attention launch (decode or prefill).  All pointers are
// device pointers; codec and pool pointers are already offset to (layer, loop).
struct AttnArgs {
  const void *q;
  void *out;
  const char *k_pool, *v_pool;          // pool base of the layer
  long long pool_page_stride_k;         // elements between physical pages
  long long pool_page_stride_v;
  long long pool_head_stride_k;         // elements between heads within a page (0 for LLA-2D)
  long long pool_head_stride_v;
  const char *mu_k, *mu_v;              // mu_t of head 0
  const char *wup_k, *wup_v;            // W_up,t of head 0
  long long mu_head_stride;             // elements between heads
  long long wup_head_stride_k, wup_head_stride_v;
  const int32_t *page_table;
  int max_pages, num_pages;
  const float *rope;                    // [rope_len][d/2][2]
  int rope_len;
  const int32_t *q_pos, *ctx_len, *p0;  // decode uses q_pos/ctx_len; prefill uses p0
  int n_q, prefill, rows, H, max_ctx;
  int splits, pages_per_split, head_groups, heads_per_wave, waves;
  int chunk_pages;                       // pages per LDS-staged RoPE chunk
  float qscale;                          // softmax scale * log2(e)
  int *err;
  float *partials;                       // [rows][H][splits][r_v + 2]
  int evict, n_sink, window;             // token eviction: retained [0, n_sink) and the last `window`
  const char *kr_pool;                   // decoupled RoPE: rotary keys of the layer
  long long kr_page_stride;              // elements between physical pages (16 d_rope)
};

// Decoupled RoPE: rotate and append rotary keys.
struct RopeAppendArgs {
  char *kr_pool;                         // layer0 base, [num_pages][16][d_rope] per layer
  long long layer_stride;                // elements between layers
  const char *kr_new;                    // [n_layers][batch][n_new][d_rope]
  const float *rope;                     // [rope_len][d_rope/2][2]
  int rope_len;
  const int32_t *page_table, *pos0;
  int max_pages, num_pages, batch, n_new, n_layers, d_rope;
  int *err;
};

struct EncodeArgs {
  const char *x_k, *x_v;       // [n_layers][B][n_new][groups][width]
  const char *mu_k, *mu_v;     // layer0 base, [D][groups][width]
  const char *wd_k, *wd_v;     // layer0 base, [D][groups][width][r]
  char *k_pool, *v_pool;       // layer0 base
  long long pool_layer_stride_k, pool_layer_stride_v;  // elements
  long long pool_page_stride_k, pool_page_stride_v;
  long long pool_head_stride_k, pool_head_stride_v;
  const int32_t *page_table, *pos0;
  int max_pages, num_pages, batch, n_new, n_layers, groups, width;
  float *muw;                  // workspace [n_layers][groups][r_k + r_v]: mu W_down, K then V
  int muw_stride, muw_v_off;   // r_k + r_v, r_k
  float *muw_part;             // workspace [muw_parts][n_layers][groups][r_k + r_v]: partial sums
  int muw_parts;               // row ranges of W_down summed independently
  int *err;
  float *kpart;                // split over the width: fp32 partial products [splits x tiles][tokens of a tile][r]
  size_t kpart_bytes;          // size of that region (0: no split)
};

// Pages of one sequence that a decode reads under token eviction (keep the
// first n_sink and the last `window` tokens of [0, ctx)).  The split plan runs
// over "virtual" pages: the sink pages [0, n_a), then the window pages
// [p_b, npages), so virtual page v is logical page v (v < n_a) or
// p_b + v - n_a.  Every virtual page holds at least one retained token, and
// no other page is read.  Without eviction every page is a sink page.
struct RetainedPages {
  int keep_lo, keep_hi;  // retained tokens: [0, keep_lo) and [keep_hi, ctx)
  int n_a, p_b, nvirt;
};
__host__ __device__ inline RetainedPages retained_pages(int ctx, int evict, int n_sink, int window) {
  RetainedPages r;
  const int npages = (ctx + kPage - 1) / kPage;
  r.keep_lo = ctx;
  r.keep_hi = ctx;
  if (evict) {
    r.keep_lo = n_sink < ctx ? n_sink : ctx;
    r.keep_hi = ctx - window > r.keep_lo ? ctx - window : r.keep_lo;
  }
  r.n_a = (r.keep_lo + kPage - 1) / kPage;
  // No window tokens (window 0, or the sink covers the context): no window
  // pages.  Otherwise the first window page holds token keep_hi.
  r.p_b = r.keep_hi >= ctx ? npages : (r.keep_hi / kPage > r.n_a ? r.keep_hi / kPage : r.n_a);
  r.nvirt = r.n_a + (npages - r.p_b);
  return r;
}

// Raise a kernel's dynamic-LDS limit to what a CU offers, once per device.
// Thread-safe: concurrent first calls serialise on a mutex, later calls see
// the device's bit set.
// One instantiation (and one set of flags) per kernel.
constexpr int kLdsLimit = 160 * 1024 - 1024;
template <auto kernel>
hipError_t raise_lds_limit() {
  static std::atomic<uint64_t> done{0};  // one bit per device ordinal < 64
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  std::lock_guard<std::mutex> lock(mu);
  if (bit && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
  e = hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsLimit);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Kernel dispatch: return hipSuccess, or hipErrorInvalidConfiguration when the
// shape has no instantiated kernel.
bool decode_supported(int dtype, int d_head, int r_k, int r_v, int heads_per_wave, int waves);
hipError_t launch_decode(int dtype, int d_head, int r_k, int r_v, const AttnArgs &a,
                         hipStream_t stream);
bool decode_g_supported(int d_head, int r_k, int r_v, int heads_per_wave, int waves);
hipError_t launch_decode_g(int d_head, int r_k, int r_v, const AttnArgs &a, hipStream_t stream);
bool decode2d_supported(int dtype, int d_head, int r_k, int r_v);
hipError_t launch_decode2d(int d_head, int r_k, int r_v, const AttnArgs &a, hipStream_t stream);
bool encode_supported(int dtype, int width, int r_k, int r_v);
hipError_t launch_encode(int dtype, int r_k, int r_v, const EncodeArgs &a, hipStream_t stream);
bool prefill_supported(int dtype, int variant, int d_head, int r_k, int r_v);
hipError_t launch_prefill(int d_head, int r_k, int r_v, const AttnArgs &a, hipStream_t stream);
hipError_t launch_merge(int dtype, int d_head, int r_v, const AttnArgs &a, hipStream_t stream);
hipError_t launch_merge_ident(int d_head, const AttnArgs &a, hipStream_t stream);
bool reconstruct_supported(int dtype, int variant, int d_head, int r_k, int r_v);
hipError_t launch_reconstruct(int d_head, int r_k, int r_v, const AttnArgs &a, void *k_full, void *v_full,
                              int batch, hipStream_t stream);
bool full_decode_supported(int dtype, int variant, int d_head);
hipError_t launch_full_decode(int d_head, const AttnArgs &a, hipStream_t stream);
bool absorbed_supported(int d_head, int r_k, int r_v, int d_rope, int heads_per_wave, int waves);
hipError_t launch_absorbed(int d_head, int r_k, int r_v, int d_rope, const AttnArgs &a, hipStream_t stream);
hipError_t launch_rope_key_append(const RopeAppendArgs &a, hipStream_t stream);
int encode_muw_parts(int width);
size_t encode_kpart_bytes(int width, int groups, int n_layers, int r_k, int r_v);
hipError_t launch_rope_table(int n_pos, int d_head, double base, float *table, hipStream_t s);

}  // namespace lla
