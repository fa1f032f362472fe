// C ABI of the LLA library: argument validation, workspace planning and
// kernel dispatch.  See include/lla.h for the contract of every entry point.
#include <math.h>
#include <stdio.h>

#include <string>

#include "lla_internal.h"

namespace lla {
namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const char *msg) {
  g_last_error = msg;
  return code;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kMaxPagesPerSplit = 2048;  // page-table entries a workgroup stages in LDS
constexpr long long kCUs = 256;          // compute units of an MI355X

bool dims_valid(const lla_dims *d) {
  return d && d->T > 0 && d->D > 0 && d->H > 0 && d->d_head > 0 && d->d_head % 2 == 0 &&
         d->r_k > 0 && d->r_v > 0 && (d->variant == LLA_PER_HEAD || d->variant == LLA_2D) &&
         (d->dtype == LLA_F32 || d->dtype == LLA_BF16) && d->page_size == kPage &&
         d->rope_base > 0.f;
}

size_t esize(const lla_dims *d) { return d->dtype == LLA_BF16 ? 2 : 4; }

// How an attention call is cut into workgroups.
struct AttnPlan {
  bool prefill;  // chunked prefill kernel (query blocks of 256, no partials)
  bool two_d;    // LLA-2D kernel (shared latent, 4 heads x 2 waves per workgroup)
  int hpw, waves, head_groups, splits, pages_per_split, chunk_pages;
  size_t partials_off, bytes;
};

void plan_workspace(const lla_dims *d, long long rows, AttnPlan *p) {
  p->partials_off = kHeaderBytes;
  p->bytes = p->splits > 1
                 ? align256(p->partials_off + sizeof(float) * (size_t)rows * d->H * p->splits * (d->r_v + 2))
                 : kHeaderBytes;
}

// LLA-2D: one workgroup per (row, 4 heads, split), 32-token blocks.  The
// kernel is bound by the matrix cores, so splits only need to fill the chip:
// about 4 workgroups per CU in total, none shorter than 8 pages.
bool plan_attn_2d(const lla_dims *d, long long rows, int max_ctx, AttnPlan *p) {
  if (d->variant != LLA_2D || d->H % 4 || !decode2d_supported(d->dtype, d->d_head, d->r_k, d->r_v))
    return false;
  p->two_d = true;
  p->hpw = 1;
  p->waves = 8;
  p->head_groups = d->H / 4;
  p->chunk_pages = 2;
  const int pages = (max_ctx + kPage - 1) / kPage;
  const long long base = rows * p->head_groups;
  long long s = (1024 + base - 1) / base;
  const long long smax = (pages + 7) / 8;
  if (s > smax) s = smax;
  const long long smin = (pages + kMaxPages2d - 1) / kMaxPages2d;
  if (s < smin) s = smin;
  if (s < 1) s = 1;
  int pps = (int)((pages + s - 1) / s);
  pps += pps & 1;  // whole 32-token blocks (kMaxPages2d is even)
  p->pages_per_split = pps;
  p->splits = (pages + pps - 1) / pps;
  if (p->splits < 1) p->splits = 1;
  plan_workspace(d, rows, p);
  return true;
}

void plan_decode_splits(const lla_dims *d, long long rows, int max_ctx, int hpw, int waves, AttnPlan *p);

bool plan_attn(const lla_dims *d, long long rows, int max_ctx, AttnPlan *p, bool prefill = false) {
  p->prefill = false;
  if (prefill && prefill_supported(d->dtype, d->variant, d->d_head, d->r_k, d->r_v)) {
    // A query chunk runs as a dense attention over rebuilt K tiles; otherwise
    // every query is one decode row.
    p->prefill = true;
    p->two_d = false;
    p->hpw = p->waves = p->head_groups = p->splits = p->pages_per_split = p->chunk_pages = 1;
    p->partials_off = kHeaderBytes;
    p->bytes = kHeaderBytes;
    return true;
  }
  if (plan_attn_2d(d, rows, max_ctx, p)) return true;
  p->two_d = false;
  // Workgroup shape: 8 waves of 2 heads (16 heads) where possible; otherwise
  // 8 waves of 1 head, or 2 waves for small head counts.
  const int H = d->H;
  int hpw = 0, waves = 0;
  const int cand[5][2] = {{2, 8}, {1, 8}, {1, 4}, {2, 2}, {1, 2}};
  for (const auto &c : cand) {
    if (H % (c[0] * c[1]) == 0 && decode_supported(d->dtype, d->d_head, d->r_k, d->r_v, c[0], c[1])) {
      hpw = c[0];
      waves = c[1];
      break;
    }
  }
  if (!hpw) return false;
  plan_decode_splits(d, rows, max_ctx, hpw, waves, p);
  return true;
}

// Decoupled-RoPE absorbed decode: the same grid and splits as the latent
// decode, with the workgroup shapes built for (d_head, r_k, r_v, d_rope).
bool plan_decoupled(const lla_dims *d, long long rows, int max_ctx, int d_rope, AttnPlan *p) {
  if (d->variant != LLA_PER_HEAD || d->dtype != LLA_BF16) return false;
  const int cand[3][2] = {{2, 8}, {1, 8}, {1, 4}};
  for (const auto &c : cand) {
    if (d->H % (c[0] * c[1]) == 0 && absorbed_supported(d->d_head, d->r_k, d->r_v, d_rope, c[0], c[1])) {
      p->prefill = false;
      p->two_d = false;
      plan_decode_splits(d, rows, max_ctx, c[0], c[1], p);
      return true;
    }
  }
  return false;
}

void plan_decode_splits(const lla_dims *d, long long rows, int max_ctx, int hpw, int waves, AttnPlan *p) {
  p->hpw = hpw;
  p->waves = waves;
  p->head_groups = d->H / (hpw * waves);
  p->chunk_pages = kDecodeRing;
  const int pages = (max_ctx + kPage - 1) / kPage;
  const long long base = rows * p->head_groups;
  // One round of workgroups over the chip: with fewer (row, head group)
  // workgroups than CUs, split each row's context until about one workgroup
  // per CU exists, and no further.  Each workgroup pays its start-up (page
  // table, folded query, pipeline fill) once, so the longest splits that still
  // occupy every CU win (measured at batch 1 x 262144 tokens, batch 32 x 4096
  // and batch 64 x 8192).  A split that is not a whole number of ring trips
  // masks the padding pages of its last trip.
  long long s = base >= kCUs ? 1 : (kCUs + base - 1) / base;
  const long long smax = pages / 4 > 1 ? pages / 4 : 1;  // at least 4 pages per split
  if (s > smax) s = smax;
  const long long smin = (pages + kMaxPagesPerSplit - 1) / kMaxPagesPerSplit;  // LDS staging bound
  if (s < smin) s = smin;
  if (s < 1) s = 1;
  const int pps = (int)((pages + s - 1) / s);
  p->pages_per_split = pps;
  p->splits = (pages + pps - 1) / pps;
  if (p->splits < 1) p->splits = 1;
  plan_workspace(d, rows, p);
}

// Full-cache decode: 4 heads per workgroup, split the context until about
// 1024 workgroups exist (HBM-bound like the latent decode).
bool plan_full(const lla_dims *d, long long rows, int max_ctx, AttnPlan *p) {
  if (!full_decode_supported(d->dtype, d->variant, d->d_head) || d->H % 4) return false;
  p->prefill = false;
  p->two_d = false;
  p->hpw = 1;
  p->waves = 4;
  p->head_groups = d->H / 4;
  p->chunk_pages = 1;
  const int pages = (max_ctx + kPage - 1) / kPage;
  const long long base = rows * p->head_groups;
  long long s = base >= 512 ? 1 : (1024 + base - 1) / base;
  const long long smax = pages / 2 > 1 ? pages / 2 : 1;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  p->pages_per_split = (int)((pages + s - 1) / s);
  p->splits = (pages + p->pages_per_split - 1) / p->pages_per_split;
  if (p->splits < 1) p->splits = 1;
  p->partials_off = kHeaderBytes;
  p->bytes = p->splits > 1
                 ? align256(kHeaderBytes + sizeof(float) * (size_t)rows * d->H * p->splits * (d->d_head + 2))
                 : kHeaderBytes;
  return true;
}

// Encode workspace: header, mu W_down [n_layers][groups][r_k + r_v], its
// per-range partial sums, and (for launches with few tiles over a wide input)
// the fp32 partial products of the split over the width.
size_t encode_ws_bytes(const lla_dims *d, int n_layers) {
  const int groups = d->variant == LLA_PER_HEAD ? d->H : 1;
  const int width = d->variant == LLA_PER_HEAD ? d->T * d->d_head : d->T * d->H * d->d_head;
  const size_t one = sizeof(float) * (size_t)n_layers * groups * (d->r_k + d->r_v);
  return align256(kHeaderBytes + one) + align256(one * encode_muw_parts(width)) +
         align256(encode_kpart_bytes(width, groups, n_layers, d->r_k, d->r_v));
}

int32_t check_launch(hipError_t e) {
  if (e == hipSuccess) return LLA_OK;
  if (e == hipErrorInvalidConfiguration) return fail(LLA_ERR_UNSUPPORTED, "no kernel for this shape");
  g_last_error = std::string("HIP launch failed: ") + hipGetErrorString(e);
  return LLA_ERR_LAUNCH;
}

void fill_layer(const lla_dims *d, const lla_codec *c, const lla_cache *k, int layer, int loop, AttnArgs *a);

// Common validation + argument filling for decode and prefill.
// Pages a token-eviction call can touch per row: the sink's, the window's and
// one partial page at each edge.
int window_plan_ctx(int max_ctx, int n_keep) {
  const long long t = (long long)kPage * ((n_keep + kPage - 1) / kPage + 2);
  return t < max_ctx ? (int)t : max_ctx;
}

// ---- scratch of the allocation-free decode (lla_decode_attn_noalloc) ----
// The split partials of that entry point live in this array, one copy per
// device, held until the process ends.  Host code never passes the array's
// name to a kernel (on the host it only stands in for the symbol): it uses the
// device address that hipGetSymbolAddress returns, looked up once per device
// on the first call made with that device current.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

hipError_t scratch_address(float **out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void *> addr[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = (float *)p;
  return hipSuccess;
}

// noalloc_err: non-null selects the allocation-free form: the error word is
// that device int32 and the split partials go to the per-device scratch array
// (ws and ws_bytes are ignored).
int32_t attn_call(const lla_dims *d, const lla_codec *c, const lla_cache *k, const float *rope,
                  int32_t rope_len, int32_t layer, int32_t loop, const void *q,
                  const int32_t *q_pos, const int32_t *ctx_len, const int32_t *p0, int32_t n_q,
                  int32_t prefill, int32_t max_ctx, float scale, void *out, void *ws,
                  size_t ws_bytes, hipStream_t stream, int evict = 0, int n_sink = 0, int window = 0,
                  int32_t *noalloc_err = nullptr) {
  if (!dims_valid(d)) return fail(LLA_ERR_INVALID_ARG, "invalid lla_dims");
  if (!c || !k) return fail(LLA_ERR_INVALID_ARG, "null codec or cache");
  if (!c->mu_k || !c->mu_v || !c->w_up_k || !c->w_up_v)
    return fail(LLA_ERR_INVALID_ARG, "null decoder parameter (mu or W_up)");
  if (!k->k_pool || !k->v_pool || !k->page_table) return fail(LLA_ERR_INVALID_ARG, "null pool or page table");
  if (k->batch < 0 || k->max_pages_per_seq < 1 || k->num_pages < 1)
    return fail(LLA_ERR_INVALID_ARG, "invalid cache sizes");
  if (layer < 0 || layer >= d->D) return fail(LLA_ERR_INVALID_ARG, "layer out of range");
  if (loop < 0 || loop >= d->T) return fail(LLA_ERR_INVALID_ARG, "loop out of range");
  if (!rope || rope_len < 1) return fail(LLA_ERR_INVALID_ARG, "null RoPE table");
  if (max_ctx < 1) return fail(LLA_ERR_INVALID_ARG, "max_ctx must be >= 1");
  if (max_ctx > rope_len) return fail(LLA_ERR_INVALID_ARG, "max_ctx exceeds the RoPE table");
  if ((long long)max_ctx > (long long)k->max_pages_per_seq * kPage)
    return fail(LLA_ERR_INVALID_ARG, "max_ctx exceeds the page table row");
  if (prefill ? (n_q < 0 || !p0) : (!q_pos || !ctx_len))
    return fail(LLA_ERR_INVALID_ARG, "null position array or bad n_q");
  if (!q || !out) return fail(LLA_ERR_INVALID_ARG, "null q or out");
  if (!(scale >= 0.f) || isinf(scale)) return fail(LLA_ERR_INVALID_ARG, "invalid scale");
  const long long rows = (long long)k->batch * (prefill ? n_q : 1);
  if (rows > (1LL << 30)) return fail(LLA_ERR_INVALID_ARG, "too many query rows");
  if (evict) {
    if (n_sink < 0 || window < 0 || (long long)n_sink + window < 1 || (long long)n_sink + window > (1LL << 30))
      return fail(LLA_ERR_INVALID_ARG, "need n_sink, window >= 0 and 1 <= n_sink + window <= 2^30");
    if (d->dtype != LLA_BF16 || d->variant != LLA_PER_HEAD)
      return fail(LLA_ERR_UNSUPPORTED, "token eviction is built for bf16 per-head LLA only");
  }
  AttnPlan p;
  if (!plan_attn(d, rows > 0 ? rows : 1, evict ? window_plan_ctx(max_ctx, n_sink + window) : max_ctx, &p,
                 prefill != 0))
    return fail(LLA_ERR_UNSUPPORTED, "no attention kernel built for this (dtype, d_head, r_k, r_v)");
  if (noalloc_err) {
    const size_t need = p.splits > 1 ? p.bytes - p.partials_off : 0;
    if (need > kNoAllocScratchBytes) {
      char msg[192];
      snprintf(msg, sizeof msg,
               "split partials of %zu bytes exceed the %zu-byte scratch of the allocation-free decode", need,
               kNoAllocScratchBytes);
      return fail(LLA_ERR_WORKSPACE, msg);
    }
  } else if (!ws || ws_bytes < p.bytes) {
    return fail(LLA_ERR_WORKSPACE, "workspace missing or too small");
  }
  if (rows == 0) return LLA_OK;

  AttnArgs a = {};
  a.q = q;
  a.out = out;
  fill_layer(d, c, k, layer, loop, &a);
  a.page_table = k->page_table;
  a.max_pages = k->max_pages_per_seq;
  a.num_pages = k->num_pages;
  a.rope = rope;
  a.rope_len = rope_len;
  a.q_pos = q_pos;
  a.ctx_len = ctx_len;
  a.p0 = p0;
  a.n_q = prefill ? n_q : 1;
  a.prefill = prefill;
  a.rows = (int)rows;
  a.H = d->H;
  a.max_ctx = max_ctx;
  a.splits = p.splits;
  a.pages_per_split = p.pages_per_split;
  a.head_groups = p.head_groups;
  a.heads_per_wave = p.hpw;
  a.waves = p.waves;
  a.chunk_pages = p.chunk_pages;
  a.evict = evict;
  a.n_sink = n_sink;
  a.window = window;
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)d->d_head);
  a.qscale = sc * 1.4426950408889634f;
  if (noalloc_err) {
    const hipError_t e = scratch_address(&a.partials);
    if (e != hipSuccess) {
      g_last_error = std::string("no scratch address on this device: ") + hipGetErrorString(e);
      return LLA_ERR_LAUNCH;
    }
    a.err = noalloc_err;
  } else {
    a.err = (int *)ws;
    a.partials = (float *)((char *)ws + p.partials_off);
  }
  if (p.prefill) return check_launch(launch_prefill(d->d_head, d->r_k, d->r_v, a, stream));
  const int32_t rc = check_launch(p.two_d ? launch_decode2d(d->d_head, d->r_k, d->r_v, a, stream)
                                          : launch_decode(d->dtype, d->d_head, d->r_k, d->r_v, a, stream));
  if (rc != LLA_OK || p.splits == 1) return rc;
  return check_launch(launch_merge(d->dtype, d->d_head, d->r_v, a, stream));
}

// Pool and codec pointers of (layer, loop), for both variants.
void fill_layer(const lla_dims *d, const lla_codec *c, const lla_cache *k, int layer, int loop, AttnArgs *ap) {
  AttnArgs &a = *ap;
  const size_t es = esize(d);
  const long long T = d->T, H = d->H, dh = d->d_head, rk = d->r_k, rv = d->r_v;
  const long long np = k->num_pages;
  if (d->variant == LLA_PER_HEAD) {
    a.k_pool = (const char *)k->k_pool + (size_t)layer * np * H * kPage * rk * es;
    a.v_pool = (const char *)k->v_pool + (size_t)layer * np * H * kPage * rv * es;
    a.pool_page_stride_k = H * kPage * rk;
    a.pool_page_stride_v = H * kPage * rv;
    a.pool_head_stride_k = kPage * rk;
    a.pool_head_stride_v = kPage * rv;
    const long long mu0 = ((long long)layer * H * T + loop) * dh;  // [D][H][T][d]
    a.mu_k = (const char *)c->mu_k + mu0 * es;
    a.mu_v = (const char *)c->mu_v + mu0 * es;
    a.wup_k = (const char *)c->w_up_k + mu0 * rk * es;              // [D][H][T][d][r]
    a.wup_v = (const char *)c->w_up_v + mu0 * rv * es;
    a.mu_head_stride = T * dh;
    a.wup_head_stride_k = T * dh * rk;
    a.wup_head_stride_v = T * dh * rv;
  } else {
    a.k_pool = (const char *)k->k_pool + (size_t)layer * np * kPage * rk * es;
    a.v_pool = (const char *)k->v_pool + (size_t)layer * np * kPage * rv * es;
    a.pool_page_stride_k = kPage * rk;
    a.pool_page_stride_v = kPage * rv;
    a.pool_head_stride_k = 0;
    a.pool_head_stride_v = 0;
    const long long mu0 = ((long long)layer * T + loop) * H * dh;   // [D][T][H][d]
    a.mu_k = (const char *)c->mu_k + mu0 * es;
    a.mu_v = (const char *)c->mu_v + mu0 * es;
    a.wup_k = (const char *)c->w_up_k + mu0 * rk * es;              // [D][T][H][d][r]
    a.wup_v = (const char *)c->w_up_v + mu0 * rv * es;
    a.mu_head_stride = dh;
    a.wup_head_stride_k = dh * rk;
    a.wup_head_stride_v = dh * rv;
  }
}

// The plan of an attention call of `op` for the arguments of
// lla_workspace_bytes; false where that returns 0.
bool plan_op(const lla_dims *d, int op, int batch, int max_ctx, int n, AttnPlan *p) {
  if (max_ctx < 1) return false;
  const long long b1 = batch > 0 ? batch : 1;
  switch (op) {
    case LLA_OP_DECOUPLED_DECODE: return plan_decoupled(d, b1, max_ctx, n, p);
    case LLA_OP_WINDOW_DECODE:
      return n >= 1 && d->dtype == LLA_BF16 && d->variant == LLA_PER_HEAD &&
             plan_attn(d, b1, window_plan_ctx(max_ctx, n), p);
    case LLA_OP_FULL_DECODE: return plan_full(d, b1, max_ctx, p);
    case LLA_OP_DECODE: return plan_attn(d, b1, max_ctx, p);
    case LLA_OP_PREFILL: {
      if (n < 0) return false;
      const long long rows = (long long)batch * n;
      return plan_attn(d, rows > 0 ? rows : 1, max_ctx, p, true);
    }
    default: return false;
  }
}

}  // namespace
}  // namespace lla

using namespace lla;

extern "C" {

int32_t lla_rope_table(const lla_dims *d, int32_t n_pos, float *table, hipStream_t stream) {
  if (!dims_valid(d)) return fail(LLA_ERR_INVALID_ARG, "invalid lla_dims");
  if (n_pos < 0 || (n_pos > 0 && !table)) return fail(LLA_ERR_INVALID_ARG, "bad RoPE table arguments");
  return check_launch(launch_rope_table(n_pos, d->d_head, (double)d->rope_base, table, stream));
}

size_t lla_workspace_bytes(const lla_dims *d, int32_t op, int32_t batch, int32_t max_ctx, int32_t n) {
  if (!dims_valid(d) || batch < 0) return 0;
  if (op == LLA_OP_ENCODE) return n >= 0 ? encode_ws_bytes(d, n) : 0;
  if (op == LLA_OP_RECONSTRUCT || op == LLA_OP_ROPE_KEY_APPEND) return kHeaderBytes;
  AttnPlan p;
  return plan_op(d, op, batch, max_ctx, n, &p) ? p.bytes : 0;
}

int32_t lla_attn_plan(const lla_dims *d, int32_t op, int32_t batch, int32_t max_ctx, int32_t n,
                      int32_t *splits, int32_t *pages_per_split) {
  if (!dims_valid(d) || batch < 0 || !splits || !pages_per_split)
    return fail(LLA_ERR_INVALID_ARG, "invalid arguments");
  AttnPlan p;
  if (!plan_op(d, op, batch, max_ctx, n, &p)) return fail(LLA_ERR_UNSUPPORTED, "no attention plan for these arguments");
  *splits = p.splits;
  *pages_per_split = p.pages_per_split;
  return LLA_OK;
}

int32_t lla_window_pages(int32_t ctx, int32_t n_sink, int32_t window, int32_t *sink_pages,
                         int32_t *first_window_page) {
  if (ctx < 0 || n_sink < 0 || window < 0 || (long long)n_sink + window < 1 || !sink_pages ||
      !first_window_page)
    return fail(LLA_ERR_INVALID_ARG, "need ctx, n_sink, window >= 0 and n_sink + window >= 1");
  const RetainedPages r = retained_pages(ctx, 1, n_sink, window);
  *sink_pages = r.n_a;
  *first_window_page = r.p_b;
  return LLA_OK;
}

int32_t lla_encode_append(const lla_dims *d, const lla_codec *c, const lla_cache *k,
                          const void *x_k, const void *x_v, const int32_t *pos0, int32_t n_new,
                          int32_t layer0, int32_t n_layers, void *ws, size_t ws_bytes,
                          hipStream_t stream) {
  if (!dims_valid(d)) return fail(LLA_ERR_INVALID_ARG, "invalid lla_dims");
  if (!c || !k) return fail(LLA_ERR_INVALID_ARG, "null codec or cache");
  if (!c->mu_k || !c->mu_v || !c->w_down_k || !c->w_down_v)
    return fail(LLA_ERR_INVALID_ARG, "null encoder parameter (mu or W_down)");
  if (!k->k_pool || !k->v_pool || !k->page_table) return fail(LLA_ERR_INVALID_ARG, "null pool or page table");
  if (k->batch < 0 || k->max_pages_per_seq < 1 || k->num_pages < 1)
    return fail(LLA_ERR_INVALID_ARG, "invalid cache sizes");
  if (n_new < 0 || n_layers < 0 || layer0 < 0 || layer0 + n_layers > d->D)
    return fail(LLA_ERR_INVALID_ARG, "layer range or n_new out of range");
  if ((!x_k || !x_v || !pos0) && n_new > 0 && n_layers > 0 && k->batch > 0)
    return fail(LLA_ERR_INVALID_ARG, "null x or pos0");
  const int groups = d->variant == LLA_PER_HEAD ? d->H : 1;
  const int width = d->variant == LLA_PER_HEAD ? d->T * d->d_head : d->T * d->H * d->d_head;
  if (!encode_supported(d->dtype, width, d->r_k, d->r_v))
    return fail(LLA_ERR_UNSUPPORTED, "no encode kernel for this shape");
  if (!ws || ws_bytes < encode_ws_bytes(d, n_layers)) return fail(LLA_ERR_WORKSPACE, "workspace missing or too small");
  if ((long long)k->batch * n_new == 0 || n_layers == 0) return LLA_OK;
  const size_t es = esize(d);
  const long long np = k->num_pages, rk = d->r_k, rv = d->r_v;
  EncodeArgs a = {};
  a.x_k = (const char *)x_k;
  a.x_v = (const char *)x_v;
  a.mu_k = (const char *)c->mu_k + (size_t)layer0 * groups * width * es;
  a.mu_v = (const char *)c->mu_v + (size_t)layer0 * groups * width * es;
  a.wd_k = (const char *)c->w_down_k + (size_t)layer0 * groups * width * rk * es;
  a.wd_v = (const char *)c->w_down_v + (size_t)layer0 * groups * width * rv * es;
  const long long hk = d->variant == LLA_PER_HEAD ? d->H : 1;
  a.pool_page_stride_k = hk * kPage * rk;
  a.pool_page_stride_v = hk * kPage * rv;
  a.pool_head_stride_k = d->variant == LLA_PER_HEAD ? kPage * rk : 0;
  a.pool_head_stride_v = d->variant == LLA_PER_HEAD ? kPage * rv : 0;
  a.pool_layer_stride_k = np * a.pool_page_stride_k;
  a.pool_layer_stride_v = np * a.pool_page_stride_v;
  a.k_pool = (char *)k->k_pool + (size_t)layer0 * a.pool_layer_stride_k * es;
  a.v_pool = (char *)k->v_pool + (size_t)layer0 * a.pool_layer_stride_v * es;
  a.page_table = k->page_table;
  a.pos0 = pos0;
  a.max_pages = k->max_pages_per_seq;
  a.num_pages = k->num_pages;
  a.batch = k->batch;
  a.n_new = n_new;
  a.n_layers = n_layers;
  a.groups = groups;
  a.width = width;
  a.err = (int *)ws;
  a.muw = (float *)((char *)ws + kHeaderBytes);
  a.muw_parts = encode_muw_parts(width);
  a.muw_part = (float *)((char *)ws + align256(kHeaderBytes + sizeof(float) * (size_t)n_layers * groups *
                                                                    (d->r_k + d->r_v)));
  a.muw_stride = d->r_k + d->r_v;
  a.muw_v_off = d->r_k;
  {
    const size_t one = sizeof(float) * (size_t)n_layers * groups * (d->r_k + d->r_v);
    a.kpart = (float *)((char *)ws + align256(kHeaderBytes + one) + align256(one * a.muw_parts));
    a.kpart_bytes = encode_kpart_bytes(width, groups, n_layers, d->r_k, d->r_v);
  }
  return check_launch(launch_encode(d->dtype, d->r_k, d->r_v, a, stream));
}

int32_t lla_decode_attn(const lla_dims *d, const lla_codec *c, const lla_cache *k,
                        const float *rope, int32_t rope_len, int32_t layer, int32_t loop,
                        const void *q, const int32_t *q_pos, const int32_t *ctx_len,
                        int32_t max_ctx, float scale, void *out, void *ws, size_t ws_bytes,
                        hipStream_t stream) {
  return attn_call(d, c, k, rope, rope_len, layer, loop, q, q_pos, ctx_len, nullptr, 1, 0,
                   max_ctx, scale, out, ws, ws_bytes, stream);
}

int32_t lla_decode_attn_noalloc(const lla_dims *d, const lla_codec *c, const lla_cache *k,
                                const float *rope, int32_t rope_len, int32_t layer, int32_t loop,
                                const void *q, const int32_t *q_pos, const int32_t *ctx_len,
                                int32_t max_ctx, float scale, void *out, int32_t *err, hipStream_t stream) {
  if (!err) return fail(LLA_ERR_INVALID_ARG, "null device error word");
  return attn_call(d, c, k, rope, rope_len, layer, loop, q, q_pos, ctx_len, nullptr, 1, 0, max_ctx, scale,
                   out, nullptr, 0, stream, 0, 0, 0, err);
}

int32_t lla_decode_window_attn(const lla_dims *d, const lla_codec *c, const lla_cache *k,
                               const float *rope, int32_t rope_len, int32_t layer, int32_t loop,
                               const void *q, const int32_t *q_pos, const int32_t *ctx_len, int32_t n_sink,
                               int32_t window, int32_t max_ctx, float scale, void *out, void *ws,
                               size_t ws_bytes, hipStream_t stream) {
  return attn_call(d, c, k, rope, rope_len, layer, loop, q, q_pos, ctx_len, nullptr, 1, 0, max_ctx, scale,
                   out, ws, ws_bytes, stream, 1, n_sink, window);
}

int32_t lla_prefill_attn(const lla_dims *d, const lla_codec *c, const lla_cache *k,
                         const float *rope, int32_t rope_len, int32_t layer, int32_t loop,
                         int32_t n_q, const void *q, const int32_t *p0, int32_t max_ctx,
                         float scale, void *out, void *ws, size_t ws_bytes, hipStream_t stream) {
  return attn_call(d, c, k, rope, rope_len, layer, loop, q, nullptr, nullptr, p0, n_q, 1,
                   max_ctx, scale, out, ws, ws_bytes, stream);
}

int32_t lla_reconstruct_kv(const lla_dims *d, const lla_codec *c, const lla_cache *k, const float *rope,
                           int32_t rope_len, int32_t layer, int32_t loop, const int32_t *ctx_len,
                           int32_t max_ctx, void *k_full, void *v_full, void *ws, size_t ws_bytes,
                           hipStream_t stream) {
  if (!dims_valid(d)) return fail(LLA_ERR_INVALID_ARG, "invalid lla_dims");
  if (!c || !k) return fail(LLA_ERR_INVALID_ARG, "null codec or cache");
  if (!c->mu_k || !c->mu_v || !c->w_up_k || !c->w_up_v)
    return fail(LLA_ERR_INVALID_ARG, "null decoder parameter (mu or W_up)");
  if (!k->k_pool || !k->v_pool || !k->page_table) return fail(LLA_ERR_INVALID_ARG, "null pool or page table");
  if (k->batch < 0 || k->max_pages_per_seq < 1 || k->num_pages < 1)
    return fail(LLA_ERR_INVALID_ARG, "invalid cache sizes");
  if (layer < 0 || layer >= d->D || loop < 0 || loop >= d->T)
    return fail(LLA_ERR_INVALID_ARG, "layer or loop out of range");
  if (!rope || rope_len < 1 || max_ctx < 1 || max_ctx > rope_len ||
      (long long)max_ctx > (long long)k->max_pages_per_seq * kPage)
    return fail(LLA_ERR_INVALID_ARG, "bad RoPE table or max_ctx");
  if (!ctx_len || !k_full || !v_full) return fail(LLA_ERR_INVALID_ARG, "null ctx_len or full cache");
  if (!reconstruct_supported(d->dtype, d->variant, d->d_head, d->r_k, d->r_v))
    return fail(LLA_ERR_UNSUPPORTED, "no reconstruct kernel for this (dtype, variant, d_head, r_k, r_v)");
  if (!ws || ws_bytes < kHeaderBytes) return fail(LLA_ERR_WORKSPACE, "workspace missing or too small");
  if (k->batch == 0) return LLA_OK;
  const long long T = d->T, H = d->H, dh = d->d_head, rk = d->r_k, rv = d->r_v, np = k->num_pages;
  AttnArgs a = {};
  a.k_pool = (const char *)k->k_pool + (size_t)layer * np * H * kPage * rk * 2;
  a.v_pool = (const char *)k->v_pool + (size_t)layer * np * H * kPage * rv * 2;
  a.pool_page_stride_k = H * kPage * rk;
  a.pool_page_stride_v = H * kPage * rv;
  a.pool_head_stride_k = kPage * rk;
  a.pool_head_stride_v = kPage * rv;
  const long long mu0 = ((long long)layer * H * T + loop) * dh;
  a.mu_k = (const char *)c->mu_k + mu0 * 2;
  a.mu_v = (const char *)c->mu_v + mu0 * 2;
  a.wup_k = (const char *)c->w_up_k + mu0 * rk * 2;
  a.wup_v = (const char *)c->w_up_v + mu0 * rv * 2;
  a.mu_head_stride = T * dh;
  a.wup_head_stride_k = T * dh * rk;
  a.wup_head_stride_v = T * dh * rv;
  a.page_table = k->page_table;
  a.max_pages = k->max_pages_per_seq;             // page-table row length
  a.pages_per_split = (max_ctx + kPage - 1) / kPage;  // pages a sequence can need (grid)
  a.num_pages = k->num_pages;
  a.rope = rope;
  a.rope_len = rope_len;
  a.ctx_len = ctx_len;
  a.H = d->H;
  a.max_ctx = max_ctx;
  a.err = (int *)ws;
  a.rows = k->batch;
  return check_launch(launch_reconstruct(d->d_head, d->r_k, d->r_v, a, k_full, v_full, k->batch, stream));
}

int32_t lla_full_decode_attn(const lla_dims *d, const lla_cache *k, const void *k_full, const void *v_full,
                             const float *rope, int32_t rope_len, const void *q, const int32_t *q_pos,
                             const int32_t *ctx_len, int32_t max_ctx, float scale, void *out, void *ws,
                             size_t ws_bytes, hipStream_t stream) {
  if (!dims_valid(d)) return fail(LLA_ERR_INVALID_ARG, "invalid lla_dims");
  if (!k || !k->page_table || !k_full || !v_full) return fail(LLA_ERR_INVALID_ARG, "null cache or full cache");
  if (k->batch < 0 || k->max_pages_per_seq < 1 || k->num_pages < 1)
    return fail(LLA_ERR_INVALID_ARG, "invalid cache sizes");
  if (!rope || rope_len < 1 || max_ctx < 1 || max_ctx > rope_len ||
      (long long)max_ctx > (long long)k->max_pages_per_seq * kPage)
    return fail(LLA_ERR_INVALID_ARG, "bad RoPE table or max_ctx");
  if (!q || !out || !q_pos || !ctx_len) return fail(LLA_ERR_INVALID_ARG, "null q, out or positions");
  if (!(scale >= 0.f) || isinf(scale)) return fail(LLA_ERR_INVALID_ARG, "invalid scale");
  AttnPlan p;
  const long long rows = k->batch;
  if (!plan_full(d, rows > 0 ? rows : 1, max_ctx, &p))
    return fail(LLA_ERR_UNSUPPORTED, "no full-cache decode kernel for this (dtype, variant, d_head, H)");
  if (!ws || ws_bytes < p.bytes) return fail(LLA_ERR_WORKSPACE, "workspace missing or too small");
  if (rows == 0) return LLA_OK;
  AttnArgs a = {};
  a.q = q;
  a.out = out;
  a.k_pool = (const char *)k_full;
  a.v_pool = (const char *)v_full;
  a.page_table = k->page_table;
  a.max_pages = k->max_pages_per_seq;
  a.num_pages = k->num_pages;
  a.rope = rope;
  a.rope_len = rope_len;
  a.q_pos = q_pos;
  a.ctx_len = ctx_len;
  a.n_q = 1;
  a.rows = (int)rows;
  a.H = d->H;
  a.max_ctx = max_ctx;
  a.splits = p.splits;
  a.pages_per_split = p.pages_per_split;
  a.head_groups = p.head_groups;
  a.heads_per_wave = 1;
  a.waves = 4;
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)d->d_head);
  a.qscale = sc * 1.4426950408889634f;
  a.err = (int *)ws;
  a.partials = (float *)((char *)ws + p.partials_off);
  const int32_t rc = check_launch(launch_full_decode(d->d_head, a, stream));
  if (rc != LLA_OK || p.splits == 1) return rc;
  return check_launch(launch_merge_ident(d->d_head, a, stream));
}

int32_t lla_rope_key_append(const lla_dims *d, const lla_cache *k, int32_t d_rope, void *kr_pool,
                            const float *rope_r, int32_t rope_r_len, const void *kr_new, const int32_t *pos0,
                            int32_t n_new, int32_t layer0, int32_t n_layers, void *ws, size_t ws_bytes,
                            hipStream_t stream) {
  if (!dims_valid(d)) return fail(LLA_ERR_INVALID_ARG, "invalid lla_dims");
  if (!k || !k->page_table || k->batch < 0 || k->max_pages_per_seq < 1 || k->num_pages < 1)
    return fail(LLA_ERR_INVALID_ARG, "null or invalid cache");
  if (d_rope < 2 || d_rope % 2 || d_rope > 1024) return fail(LLA_ERR_INVALID_ARG, "d_rope must be even, 2..1024");
  if (n_new < 0 || n_layers < 0 || layer0 < 0 || layer0 + n_layers > d->D)
    return fail(LLA_ERR_INVALID_ARG, "layer range or n_new out of range");
  if (!kr_pool || !rope_r || rope_r_len < 1) return fail(LLA_ERR_INVALID_ARG, "null rotary pool or table");
  if ((!kr_new || !pos0) && n_new > 0 && n_layers > 0 && k->batch > 0)
    return fail(LLA_ERR_INVALID_ARG, "null kr_new or pos0");
  if (d->dtype != LLA_BF16) return fail(LLA_ERR_UNSUPPORTED, "rotary keys are stored in bf16 only");
  if (!ws || ws_bytes < kHeaderBytes) return fail(LLA_ERR_WORKSPACE, "workspace missing or too small");
  RopeAppendArgs a = {};
  a.layer_stride = (long long)k->num_pages * kPage * d_rope;
  a.kr_pool = (char *)kr_pool + (size_t)layer0 * a.layer_stride * 2;
  a.kr_new = (const char *)kr_new;
  a.rope = rope_r;
  a.rope_len = rope_r_len;
  a.page_table = k->page_table;
  a.pos0 = pos0;
  a.max_pages = k->max_pages_per_seq;
  a.num_pages = k->num_pages;
  a.batch = k->batch;
  a.n_new = n_new;
  a.n_layers = n_layers;
  a.d_rope = d_rope;
  a.err = (int *)ws;
  return check_launch(launch_rope_key_append(a, stream));
}

int32_t lla_decoupled_decode_attn(const lla_dims *d, const lla_codec *c, const lla_cache *k, int32_t d_rope,
                                  const void *kr_pool, const float *rope_r, int32_t rope_r_len, int32_t layer,
                                  int32_t loop, const void *q, const int32_t *q_pos, const int32_t *ctx_len,
                                  int32_t max_ctx, float scale, void *out, void *ws, size_t ws_bytes,
                                  hipStream_t stream) {
  if (!dims_valid(d)) return fail(LLA_ERR_INVALID_ARG, "invalid lla_dims");
  if (!c || !k) return fail(LLA_ERR_INVALID_ARG, "null codec or cache");
  if (!c->mu_v || !c->w_up_k || !c->w_up_v) return fail(LLA_ERR_INVALID_ARG, "null decoder parameter");
  if (!k->k_pool || !k->v_pool || !k->page_table || !kr_pool)
    return fail(LLA_ERR_INVALID_ARG, "null pool, rotary pool or page table");
  if (k->batch < 0 || k->max_pages_per_seq < 1 || k->num_pages < 1)
    return fail(LLA_ERR_INVALID_ARG, "invalid cache sizes");
  if (layer < 0 || layer >= d->D || loop < 0 || loop >= d->T)
    return fail(LLA_ERR_INVALID_ARG, "layer or loop out of range");
  if (!rope_r || rope_r_len < 1) return fail(LLA_ERR_INVALID_ARG, "null rotary RoPE table");
  if (max_ctx < 1 || (long long)max_ctx > (long long)k->max_pages_per_seq * kPage)
    return fail(LLA_ERR_INVALID_ARG, "max_ctx out of range");
  if (!q || !out || !q_pos || !ctx_len) return fail(LLA_ERR_INVALID_ARG, "null q, out or positions");
  if (!(scale >= 0.f) || isinf(scale)) return fail(LLA_ERR_INVALID_ARG, "invalid scale");
  if (d_rope < 2 || d_rope % 2) return fail(LLA_ERR_INVALID_ARG, "d_rope must be even");
  const long long rows = k->batch;
  AttnPlan p;
  if (!plan_decoupled(d, rows > 0 ? rows : 1, max_ctx, d_rope, &p))
    return fail(LLA_ERR_UNSUPPORTED, "no decoupled-RoPE kernel for this (dtype, d_head, r_k, r_v, d_rope, H)");
  if (!ws || ws_bytes < p.bytes) return fail(LLA_ERR_WORKSPACE, "workspace missing or too small");
  if (rows == 0) return LLA_OK;
  AttnArgs a = {};
  a.q = q;
  a.out = out;
  fill_layer(d, c, k, layer, loop, &a);
  a.kr_pool = (const char *)kr_pool + (size_t)layer * k->num_pages * kPage * d_rope * 2;
  a.kr_page_stride = (long long)kPage * d_rope;
  a.page_table = k->page_table;
  a.max_pages = k->max_pages_per_seq;
  a.num_pages = k->num_pages;
  a.rope = rope_r;
  a.rope_len = rope_r_len;
  a.q_pos = q_pos;
  a.ctx_len = ctx_len;
  a.n_q = 1;
  a.rows = (int)rows;
  a.H = d->H;
  a.max_ctx = max_ctx;
  a.splits = p.splits;
  a.pages_per_split = p.pages_per_split;
  a.head_groups = p.head_groups;
  a.heads_per_wave = p.hpw;
  a.waves = p.waves;
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)(d->d_head + d_rope));
  a.qscale = sc * 1.4426950408889634f;
  a.err = (int *)ws;
  a.partials = (float *)((char *)ws + p.partials_off);
  const int32_t rc = check_launch(launch_absorbed(d->d_head, d->r_k, d->r_v, d_rope, a, stream));
  if (rc != LLA_OK || p.splits == 1) return rc;
  return check_launch(launch_merge(d->dtype, d->d_head, d->r_v, a, stream));
}

int32_t lla_cache_scalars(const lla_dims *d, int64_t *teacher, int64_t *latent) {
  if (!dims_valid(d) || !teacher || !latent) return fail(LLA_ERR_INVALID_ARG, "invalid arguments");
  *teacher = 2LL * d->T * d->H * d->d_head;
  *latent = d->variant == LLA_2D ? (int64_t)(d->r_k + d->r_v) : (int64_t)(d->r_k + d->r_v) * d->H;
  return LLA_OK;
}

int32_t lla_supported(const lla_dims *d, int32_t op) {
  if (!dims_valid(d)) return 0;
  if (op == LLA_OP_ENCODE) {
    const int width = d->variant == LLA_PER_HEAD ? d->T * d->d_head : d->T * d->H * d->d_head;
    return encode_supported(d->dtype, width, d->r_k, d->r_v) ? 1 : 0;
  }
  if (op == LLA_OP_DECODE || op == LLA_OP_PREFILL) {
    AttnPlan p;
    return plan_attn(d, 1, kPage, &p, op == LLA_OP_PREFILL) ? 1 : 0;
  }
  if (op == LLA_OP_RECONSTRUCT) return reconstruct_supported(d->dtype, d->variant, d->d_head, d->r_k, d->r_v);
  if (op == LLA_OP_ROPE_KEY_APPEND) return d->dtype == LLA_BF16 ? 1 : 0;
  if (op == LLA_OP_WINDOW_DECODE) {
    AttnPlan p;
    return d->dtype == LLA_BF16 && d->variant == LLA_PER_HEAD && plan_attn(d, 1, kPage, &p) ? 1 : 0;
  }
  if (op == LLA_OP_DECOUPLED_DECODE) {
    AttnPlan p;
    return plan_decoupled(d, 1, kPage, 64, &p) && plan_decoupled(d, 1, kPage, 32, &p) ? 1 : 0;
  }
  if (op == LLA_OP_FULL_DECODE) {
    AttnPlan p;
    return plan_full(d, 1, kPage, &p) ? 1 : 0;
  }
  return 0;
}

const char *lla_status_string(int32_t s) {
  switch (s) {
    case LLA_OK: return "ok";
    case LLA_ERR_INVALID_ARG: return "invalid argument";
    case LLA_ERR_UNSUPPORTED: return "unsupported shape or variant";
    case LLA_ERR_WORKSPACE: return "workspace missing or too small";
    case LLA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char *lla_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
