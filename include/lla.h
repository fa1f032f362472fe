/*
 * lla.h -- C ABI of the MI355X (gfx950) Looped Latent Attention (LLA) library.
 *
 * LLA is a post-training cache codec for looped, weight-tied Transformers: for
 * every cached token, layer and head it stores a K latent c_k (width r_k) and a
 * V latent c_v (width r_v) instead of T per-loop K/V vectors, and rebuilds the
 * loop-t K/V only when attention reads them.  Sources, cited by page title and
 * section:
 *   [CR] "Looped Latent Attention: 跨循环 KV 压缩精读" (cc.laoqi.cc close reading of
 *        arXiv 2607.15456v2), section 二:方法 items 1-3 and 6, section 四:结果 item 9
 *        (Table 5) and item 10 (appendix J: decoupled RoPE).
 *   [GS] gist.science summary of arXiv 2607.15456, "Technisches Resümee" /
 *        "Kernmechanismus" (text form of eq. (2)-(4)).
 *   encoder  eq. (2): c = (x - mu) W_down, x = [x_1; ...; x_T] (loop-major).
 *   decoder  eq. (3): x_hat_t = c W_up,t^T + mu_t.
 *   ratio    eq. (4): 2 T H d_head scalars per token and layer become
 *            (r_k + r_v) H (per-head) or r_k + r_v (LLA-2D).
 *   RoPE is applied to the rebuilt K at the token's position ([CR] 方法 item 3).
 *
 * Conventions shared by every entry point:
 *   - All tensor arguments are DEVICE pointers owned by the caller, row-major,
 *     dense, in the layouts given below.  The library never allocates, frees or
 *     synchronises; each call enqueues its kernels on `stream` and returns.
 *   - Floating-point storage is `dims->dtype`: LLA_F32 (IEEE fp32) or LLA_BF16
 *     (bfloat16 bit patterns).  It applies to latents, codec parameters, q, x
 *     and out.  Accumulation is fp32; bf16 results are rounded to nearest-even.
 *   - Indices: `layer` in [0, D); `loop` in [0, T) (loop t = loop + 1 in the
 *     pages' 1-based notation).  A cached token's RoPE position is its logical
 *     index j in its sequence; logical token j of sequence b lives in physical
 *     page page_table[b][j / page_size] at row j % page_size.
 *   - RoPE: pairs (i, i + d_head/2), angle p * rope_base^(-2i/d_head), rotation
 *     (a, b) -> (a cos - b sin, a sin + b cos).  The angles come from a caller-
 *     owned table filled once by lla_rope_table().
 *   - Return value: LLA_OK or a negative LLA_ERR_* code for errors the host can
 *     see (null pointers, bad sizes or indices, unsupported shapes, workspace
 *     too small, launch failure); lla_last_error() gives a thread-local message.
 *   - Errors only the device can see (a ctx_len, q_pos, p0 or pos0 out of range,
 *     a page-table entry outside [0, num_pages)) never cause out-of-bounds
 *     accesses: the affected output rows are written as NaN (decode, prefill) or
 *     the affected latents are not written (encode), and a bit is OR-ed into the
 *     int32 error word at byte 0 of the workspace (LLA_DEVERR_*).  That word is
 *     sticky: the library never clears it.
 *   - Workspace: size it with lla_workspace_bytes() and zero it once after
 *     allocation (the error word must start clear).  Beyond the 256-byte
 *     header it holds per-call scratch (split partials, encode's mu W_down),
 *     rewritten by every call.  One workspace must not be used by two calls
 *     that may run concurrently.
 */
#ifndef LLA_H
#define LLA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  LLA_OK = 0,
  LLA_ERR_INVALID_ARG = -1, /* null pointer, bad size, index out of range */
  LLA_ERR_UNSUPPORTED = -2, /* valid but not built: see lla_supported() */
  LLA_ERR_WORKSPACE = -3,   /* workspace null or smaller than lla_workspace_bytes() */
  LLA_ERR_LAUNCH = -4       /* the HIP runtime refused a launch */
};

enum { LLA_PER_HEAD = 0, LLA_2D = 1 }; /* [CR] 方法 item 6: LLA-2D folds heads into one latent */
enum { LLA_F32 = 0, LLA_BF16 = 1 };
enum {
  LLA_OP_ENCODE = 0,
  LLA_OP_DECODE = 1,
  LLA_OP_PREFILL = 2,
  LLA_OP_RECONSTRUCT = 3,
  LLA_OP_FULL_DECODE = 4,
  LLA_OP_ROPE_KEY_APPEND = 5,
  LLA_OP_DECOUPLED_DECODE = 6,
  LLA_OP_WINDOW_DECODE = 7
};

/* Device-side error bits (workspace byte 0). */
enum {
  LLA_DEVERR_CTX = 1,   /* ctx_len < 1 or > max_ctx, or q_pos / p0 outside the RoPE table */
  LLA_DEVERR_PAGE = 2,  /* page-table entry outside [0, num_pages) */
  LLA_DEVERR_APPEND = 4 /* pos0[b] + n_new beyond the sequence's page-table row */
};

/* Shapes, in the pages' notation ([CR] 方法 item 1 symbol table). */
typedef struct lla_dims {
  int32_t T;         /* loops (recurrence steps) */
  int32_t D;         /* shared layers */
  int32_t H;         /* attention heads */
  int32_t d_head;    /* head width */
  int32_t r_k, r_v;  /* K and V latent widths */
  int32_t variant;   /* LLA_PER_HEAD or LLA_2D */
  int32_t dtype;     /* LLA_F32 or LLA_BF16 */
  int32_t page_size; /* tokens per cache page; must be 16 */
  float rope_base;   /* RoPE base, e.g. 10000 */
} lla_dims;

/* Codec parameters, fixed and shared across tokens ([CR] 方法 item 1).
 * Per-head: an independent codec per (layer, head); mu_t and W_up,t per loop.
 *   mu_k, mu_v           [D][H][T][d_head]          (mu_t = mu[..][t][:])
 *   w_down_k / w_down_v  [D][H][T*d_head][r_k|r_v]
 *   w_up_k / w_up_v      [D][H][T][d_head][r_k|r_v] (W_up,t is d_head x r)
 * LLA-2D: one codec per layer over x ordered [t][h][d]:
 *   mu_k, mu_v           [D][T][H][d_head]
 *   w_down_k / w_down_v  [D][T*H*d_head][r_k|r_v]
 *   w_up_k / w_up_v      [D][T][H][d_head][r_k|r_v] (head h of loop t decodes with
 *                        its own d_head x r slice) */
typedef struct lla_codec {
  const void *mu_k, *mu_v;
  const void *w_down_k, *w_down_v;
  const void *w_up_k, *w_up_v;
} lla_codec;

/* Paged latent cache.  One page table serves every layer.
 *   per-head: k_pool [D][num_pages][H][page_size][r_k], v_pool [..][r_v]
 *   LLA-2D:   k_pool [D][num_pages][page_size][r_k],    v_pool [..][r_v]
 *   page_table [batch][max_pages_per_seq] int32 physical page indices. */
typedef struct lla_cache {
  void *k_pool, *v_pool;
  const int32_t *page_table;
  int32_t batch;
  int32_t max_pages_per_seq;
  int32_t num_pages;
} lla_cache;

/* Fill table[n_pos][d_head/2][2] (fp32 cos, sin of p * base^(-2i/d_head),
 * evaluated in fp64) for positions 0..n_pos-1.  The decode and prefill calls
 * read angles only from this table. */
int32_t lla_rope_table(const lla_dims *dims, int32_t n_pos, float *table, hipStream_t stream);

/* Bytes of workspace that `op` needs.  batch = sequences; max_ctx = the
 * host-known upper bound on every context the call may read (decode: on
 * ctx_len; prefill: on p0[b] + n); n = n_q for prefill, n_layers for encode,
 * d_rope for the decoupled decode, n_sink + window for the windowed decode,
 * ignored otherwise.  Returns 0 for invalid
 * arguments or shapes without a kernel. */
size_t lla_workspace_bytes(const lla_dims *dims, int32_t op, int32_t batch, int32_t max_ctx,
                           int32_t n);

/* Encode + append, eq. (2) ([CR] 方法 item 1; [GS] Kernmechanismus).
 * For layers layer0 .. layer0+n_layers-1, sequences b and new tokens n < n_new:
 *   c_k = (x_k - mu_k) W_down,k   and   c_v = (x_v - mu_v) W_down,v,
 * computed as x W_down - mu W_down with fp32 accumulation, rounded once to the
 * storage dtype, and written to the slot of logical token pos0[b] + n.  No
 * other slot is touched.
 *   x_k, x_v  per-head [n_layers][batch][n_new][H][T][d_head]
 *             LLA-2D   [n_layers][batch][n_new][T][H][d_head]   (pre-RoPE)
 *   pos0      device int32 [batch]: first logical position written per sequence.
 * The caller owns ctx_len and must append a token before attending to it. */
int32_t lla_encode_append(const lla_dims *dims, const lla_codec *codec, const lla_cache *cache,
                          const void *x_k, const void *x_v, const int32_t *pos0, int32_t n_new,
                          int32_t layer0, int32_t n_layers, void *workspace, size_t ws_bytes,
                          hipStream_t stream);

/* Decode attention of one query per sequence over its latent cache, for one
 * (layer, loop) ([CR] 方法 items 1-3; 四:结果 item 9 latent-store path):
 *   k_hat_j = mu_k,t + c_k,j W_up,k,t^T,  v_hat_j = mu_v,t + c_v,j W_up,v,t^T  (eq. (3))
 *   out = sum_j softmax_j(scale <R(q_pos) q, R(j) k_hat_j>) v_hat_j,  j in [0, ctx_len[b]).
 * The V side is summed in latent space and up-projected once (exact by the
 * linearity of eq. (3)); K is rebuilt per token.
 *   q         [batch][H][d_head] pre-RoPE;  out [batch][H][d_head]
 *   q_pos     device int32 [batch], in [0, rope_len)
 *   ctx_len   device int32 [batch], in [1, max_ctx]; max_ctx <= rope_len and
 *             max_ctx <= max_pages_per_seq * page_size
 *   scale     softmax scale; 0 selects 1/sqrt(d_head). */
int32_t lla_decode_attn(const lla_dims *dims, const lla_codec *codec, const lla_cache *cache,
                        const float *rope_table, int32_t rope_len, int32_t layer, int32_t loop,
                        const void *q, const int32_t *q_pos, const int32_t *ctx_len,
                        int32_t max_ctx, float scale, void *out, void *workspace,
                        size_t ws_bytes, hipStream_t stream);

/* lla_decode_attn without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same computation, kernels and arguments as
 * lla_decode_attn, except:
 *   err   device int32, caller-owned: the error word (LLA_DEVERR_* bits OR-ed
 *         in, sticky, never cleared by the library), as byte 0 of the
 *         workspace of lla_decode_attn.
 * The split partials live in a 16 MiB device array inside the library, one
 * per GPU, held until the process ends; every call on a GPU shares it, so
 * calls that may overlap on one GPU (other streams, other threads) race and
 * must be serialised by the caller.  A call whose partials would exceed
 * 16 MiB (lla_workspace_bytes(.., LLA_OP_DECODE, ..) - 256 bytes, when above
 * 256) returns LLA_ERR_WORKSPACE before anything is enqueued.  The call never
 * allocates or frees memory; the first call on a device looks up the array's
 * address once. */
int32_t lla_decode_attn_noalloc(const lla_dims *dims, const lla_codec *codec, const lla_cache *cache,
                                const float *rope_table, int32_t rope_len, int32_t layer, int32_t loop,
                                const void *q, const int32_t *q_pos, const int32_t *ctx_len,
                                int32_t max_ctx, float scale, void *out, int32_t *err, hipStream_t stream);

/* Decode attention with token eviction composed with LLA ([CR] 四:结果 item 10,
 * Table 9: a 4-token attention sink plus a 256-token window; item 9: 1024
 * retained tokens of the 21.3x cache take 36 KiB x 1024).  Of the ctx_len[b]
 * tokens of sequence b only logical tokens j < n_sink and j >= ctx_len[b] -
 * window take part, each at its own logical position j for RoPE; the softmax
 * runs over that set:
 *   out = sum_{j retained} softmax_j(scale <R(q_pos) q, R(j) k_hat_j>) v_hat_j.
 * Page-table entries of pages that hold no retained token are never read, so
 * the caller may release those pages (set their entries to anything).  A page
 * that holds a retained token must be valid (else LLA_DEVERR_PAGE, row NaN).
 *   n_sink, window  host ints, >= 0, 1 <= n_sink + window <= 2^30 (a budget at
 *                   or above a sequence's context keeps all of it)
 * Other arguments as for lla_decode_attn; workspace from lla_workspace_bytes(..,
 * LLA_OP_WINDOW_DECODE, batch, max_ctx, n_sink + window).  Supported: bf16
 * per-head shapes of lla_decode_attn. */
int32_t lla_decode_window_attn(const lla_dims *dims, const lla_codec *codec, const lla_cache *cache,
                               const float *rope_table, int32_t rope_len, int32_t layer, int32_t loop,
                               const void *q, const int32_t *q_pos, const int32_t *ctx_len, int32_t n_sink,
                               int32_t window, int32_t max_ctx, float scale, void *out, void *workspace,
                               size_t ws_bytes, hipStream_t stream);

/* Causal prefill attention over the latent cache ([CR] 方法 item 6: long
 * prefill reconstructs per layer).  Query i of sequence b sits at position
 * p0[b] + i and attends over logical tokens [0, p0[b] + i]; those tokens must
 * already be appended.
 *   q, out   [batch][n_q][H][d_head];  p0 device int32 [batch];
 *   max_ctx  >= p0[b] + n_q for every b (rows past it are written as NaN);
 *   other arguments as for lla_decode_attn.
 * bf16 per-head shapes with a chunk kernel (lla_supported(.., LLA_OP_PREFILL)
 * and d_head, r_k, r_v in (64,16,32), (128,16,32), (128,32,64), (128,96,160))
 * rebuild each 32-token K tile once per 256 queries and run a dense attention
 * on the matrix cores; other shapes run every query as one decode row.  Both
 * give the same result within the storage type's rounding. */
int32_t lla_prefill_attn(const lla_dims *dims, const lla_codec *codec, const lla_cache *cache,
                         const float *rope_table, int32_t rope_len, int32_t layer, int32_t loop,
                         int32_t n_q, const void *q, const int32_t *p0, int32_t max_ctx,
                         float scale, void *out, void *workspace, size_t ws_bytes,
                         hipStream_t stream);

/* Full ("teacher") K/V cache of one (layer, loop), the baseline the latent
 * cache is measured against ([CR] 四:结果 item 9: the full-memory fast path keeps
 * the complete reconstructed K/V; the capacity path rebuilds at read time).
 * Layout, bf16 per-head, same page table as the latent cache:
 *   k_full, v_full  [num_pages][H][page_size][d_head]
 * where the K row of logical token j is already rotated by RoPE at position j.
 *
 * lla_reconstruct_kv rebuilds the slots of logical tokens [0, ctx_len[b]) of
 * every sequence from the latent cache of (layer, loop), eq. (3) with RoPE
 * after reconstruction ([CR] 方法 items 1 and 3):
 *   k_j = R(j)(mu_k,t + c_k,j W_up,k,t^T),  v_j = mu_v,t + c_v,j W_up,v,t^T,
 * fp32 accumulation, rounded once to bf16.  Other slots are not touched.
 * ctx_len is device int32 [batch] (1 <= ctx_len <= max_ctx, else the row is
 * skipped and LLA_DEVERR_CTX set); pages with out-of-range table entries are
 * skipped and set LLA_DEVERR_PAGE.  Workspace: lla_workspace_bytes(..,
 * LLA_OP_RECONSTRUCT, ..) (the error word only).  Supported: bf16 per-head,
 * (d_head, r_k, r_v) in (64,16,32), (128,16,32), (128,32,64), (128,64,64),
 * (128,96,160). */
int32_t lla_reconstruct_kv(const lla_dims *dims, const lla_codec *codec, const lla_cache *cache,
                           const float *rope_table, int32_t rope_len, int32_t layer, int32_t loop,
                           const int32_t *ctx_len, int32_t max_ctx, void *k_full, void *v_full,
                           void *workspace, size_t ws_bytes, hipStream_t stream);

/* Decode attention over a full cache (textbook attention of R(q_pos) q over
 * the stored K/V): out = softmax(scale <R(q_pos) q, k_j>) V over j < ctx_len.
 * cache supplies the page table and sizes only (its pools are not read); q and
 * out [batch][H][d_head] bf16; other arguments as for lla_decode_attn; workspace
 * from lla_workspace_bytes(.., LLA_OP_FULL_DECODE, batch, max_ctx, 0).
 * Supported: bf16 per-head, d_head 64 or 128, H a multiple of 4. */
int32_t lla_full_decode_attn(const lla_dims *dims, const lla_cache *cache, const void *k_full,
                             const void *v_full, const float *rope_table, int32_t rope_len,
                             const void *q, const int32_t *q_pos, const int32_t *ctx_len,
                             int32_t max_ctx, float scale, void *out, void *workspace,
                             size_t ws_bytes, hipStream_t stream);

/* Decoupled RoPE ([CR] 四:结果 item 10, appendix J).  Full RoPE rotates each
 * rebuilt key by its own position, which keeps the K decoder out of the query;
 * the decoupled variant scores with a NoPE content path (the eq. (3) key, not
 * rotated) plus an explicit rotary branch of width d_rope:
 *   s_j = scale (<q_c, mu_k,t + c_k,j W_up,k,t^T> + <R_r(q_pos) q_r, kr_j>),
 *   out = sum_j softmax_j(s) v_hat_j   (v_hat_j as in lla_decode_attn),
 * where kr_j is one rotary key per (token, layer), shared by all heads and
 * loops and stored after rotation at its position, and R_r is RoPE over the
 * d_rope dims (pairs (i, i + d_rope/2), angle p * rope_base^(-2i/d_rope)).
 * The RoPE table for the branch is lla_rope_table() of a copy of dims with
 * d_head = d_rope: [rope_r_len][d_rope/2][2].
 *   kr_pool  bf16 [D][num_pages][page_size][d_rope], paged by cache->page_table.
 *
 * lla_rope_key_append writes the rotary keys of tokens pos0[b] + n
 * (n < n_new) for layers layer0 .. layer0 + n_layers - 1:
 *   kr_pool[layer][slot] = R_r(pos) kr_new[layer - layer0][b][n],  fp32, rounded once to bf16.
 *   kr_new  bf16 [n_layers][batch][n_new][d_rope] (before rotation).
 * A token whose position is outside the page table row is skipped with
 * LLA_DEVERR_APPEND, one past the table with LLA_DEVERR_CTX, one on an invalid
 * page with LLA_DEVERR_PAGE.  Workspace: the error word (LLA_OP_ROPE_KEY_APPEND).
 * bf16 only; d_rope even, 2..1024. */
int32_t lla_rope_key_append(const lla_dims *dims, const lla_cache *cache, int32_t d_rope, void *kr_pool,
                            const float *rope_r, int32_t rope_r_len, const void *kr_new, const int32_t *pos0,
                            int32_t n_new, int32_t layer0, int32_t n_layers, void *workspace,
                            size_t ws_bytes, hipStream_t stream);

/* Decode attention with the decoupled score above, one query per sequence,
 * for one (layer, loop).  The content path is absorbed into the query
 * (q~ = W_up,k,t^T q_c, r_k wide; the <q_c, mu_k,t> term is the same for every
 * token of a row and cancels in the softmax), so no key is rebuilt; V is
 * summed in latent space and up-projected once.
 *   q        bf16 [batch][H][d_head + d_rope]: content part, then rotary part
 *   out      bf16 [batch][H][d_head]
 *   q_pos    device int32 [batch], in [0, rope_r_len) (else LLA_DEVERR_CTX)
 *   ctx_len  device int32 [batch], in [1, max_ctx]; max_ctx <= max_pages_per_seq * page_size
 *   scale    0 selects 1/sqrt(d_head + d_rope)
 * codec->mu_k is not read.  Workspace: lla_workspace_bytes(.., LLA_OP_DECOUPLED_DECODE,
 * batch, max_ctx, d_rope).  Supported: bf16 per-head, (d_head, r_k, r_v) in
 * (128,16,32) with H a multiple of 16 and (128,96,160) with H a multiple of 4,
 * d_rope 32 or 64.  Device errors as lla_decode_attn. */
int32_t lla_decoupled_decode_attn(const lla_dims *dims, const lla_codec *codec, const lla_cache *cache,
                                  int32_t d_rope, const void *kr_pool, const float *rope_r, int32_t rope_r_len,
                                  int32_t layer, int32_t loop, const void *q, const int32_t *q_pos,
                                  const int32_t *ctx_len, int32_t max_ctx, float scale, void *out,
                                  void *workspace, size_t ws_bytes, hipStream_t stream);

/* Eq. (4): persistent cache scalars per token and layer, for the teacher
 * (2 T H d_head) and for the latent cache ((r_k + r_v) H, or r_k + r_v for
 * LLA-2D).  Host only.  ([CR] 方法 item 2; Table 5.) */
int32_t lla_cache_scalars(const lla_dims *dims, int64_t *teacher, int64_t *latent);

/* How an attention call is cut into workgroups (host only), for the same
 * arguments as lla_workspace_bytes with op = LLA_OP_DECODE, LLA_OP_PREFILL,
 * LLA_OP_WINDOW_DECODE, LLA_OP_DECOUPLED_DECODE or LLA_OP_FULL_DECODE:
 *   *splits           parts each row's context is cut into; with more than one,
 *                     each part leaves (max, weight sum, latent value sum)
 *                     partials in the workspace and a second launch merges them
 *                     in a fixed order;
 *   *pages_per_split  pages of a part (for the windowed decode: pages that
 *                     hold retained tokens, see lla_window_pages).
 * The chunked prefill kernel reports 1 and 1.  Returns LLA_OK, or
 * LLA_ERR_INVALID_ARG (null outputs, invalid dims) / LLA_ERR_UNSUPPORTED
 * where lla_workspace_bytes would return 0. */
int32_t lla_attn_plan(const lla_dims *dims, int32_t op, int32_t batch, int32_t max_ctx, int32_t n,
                      int32_t *splits, int32_t *pages_per_split);

/* Token eviction (lla_decode_window_attn): the pages of a sequence of ctx
 * tokens whose page-table entries the windowed decode reads (host only).  They
 * are pages [0, *sink_pages), which hold the sink tokens j < n_sink, and pages
 * [*first_window_page, ceil(ctx / page_size)), which hold the window tokens
 * j >= ctx - window; *first_window_page is ceil(ctx / page_size) when no token
 * lies in the window beyond the sink.  Each of these pages holds at least one
 * retained token; no other entry is read.  Returns LLA_OK or
 * LLA_ERR_INVALID_ARG (negative sizes, n_sink + window < 1, null outputs). */
int32_t lla_window_pages(int32_t ctx, int32_t n_sink, int32_t window, int32_t *sink_pages,
                         int32_t *first_window_page);

/* 1 if the library has kernels for (dims, op), else 0 (host only). */
int32_t lla_supported(const lla_dims *dims, int32_t op);

const char *lla_status_string(int32_t status);
const char *lla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LLA_H */
