/*
 * lla_oracle.c -- plain, slow, obviously-correct CPU oracle for Looped Latent
 * Attention (LLA).  TEST INFRASTRUCTURE ONLY: nothing on the product path may
 * include, link or call this file.  It shares no code, header, table or constant
 * generator with the HIP library; it is built on its own with gcc.
 *
 * Every arithmetic step runs in IEEE double.  Stored inputs (fp32 or bf16 bit
 * patterns) are decoded exactly into double before use.
 *
 * Sources (cited by page title and section, as the pages are numbered):
 *  [CR]  "Looped Latent Attention: 跨循环 KV 压缩精读" (cc.laoqi.cc close reading
 *        of arXiv 2607.15456v2): section 二:方法, item 1 (symbol table, eq. (2)-(3)),
 *        item 2 (eq. (4), exact cache-scalar ratio), item 3 (pre-RoPE compression,
 *        full RoPE applied after reconstruction), item 6 (LLA-2D, latent-store path);
 *        section 四:结果 item 9 (Table 5: latent attention checked against full
 *        reconstruction).
 *  [GS]  gist.science German summary of arXiv 2607.15456, "Technisches Resümee",
 *        "Kernmechanismus": encoder c = (x - mu) W_down, decoder
 *        x_hat_t = c W_up,t^T + mu_t, ratio rho = 2 T d_head / (r_k + r_v).
 *
 * What the oracle computes (the plain definition, nothing absorbed):
 *   encode (eq. (2)):  c = (x - mu) W_down, x = [x_1; ...; x_T] loop-major;
 *                      rounded once to the storage type (RNE for bf16).
 *   decode:            for each cached token j of sequence b, read its latents
 *                      through the page table, rebuild the FULL loop-t vectors
 *                      k_hat_j = mu_k,t + c_k,j W_up,k,t^T and
 *                      v_hat_j = mu_v,t + c_v,j W_up,v,t^T (eq. (3)), rotate q and
 *                      k_hat_j with RoPE at their positions ([CR] 方法 item 3),
 *                      then textbook softmax attention
 *                      o = sum_j softmax_j(scale <R(p_q) q, R(j) k_hat_j>) v_hat_j.
 *   LLA-2D ([CR] 方法 item 6): the concatenation also runs over heads, so one
 *                      latent per (token, layer) is shared by all heads; head h of
 *                      loop t decodes with its own slice mu_{t,h}, W_up,t,h.
 *
 * Readings taken where the pages are silent (each listed in the design doc):
 *   RoPE pairs are split-half (i, i + d/2), angle p * base^(-2i/d), rotation
 *   (a,b) -> (a cos - b sin, a sin + b cos); V is not rotated; a cached token's
 *   position is its logical index j; q arrives pre-RoPE with its position q_pos;
 *   decode attends over [0, ctx_len) with no mask (append happens first);
 *   prefill query i of sequence b sits at p0_b + i and attends over
 *   [0, p0_b + i]; LLA-2D vectors are ordered [t][h][d].
 *
 * Layouts (row-major, element offsets):
 *   per-head  mu [D][H][T][d]    W_down [D][H][T*d][r]   W_up [D][H][T][d][r]
 *             pool [D][num_pages][H][P][r]      x [n_layers][B][n_new][H][T][d]
 *   LLA-2D    mu [D][T][H][d]    W_down [D][T*H*d][r]    W_up [D][T][H][d][r]
 *             pool [D][num_pages][P][r]         x [n_layers][B][n_new][T][H][d]
 *   page_table [B][max_pages]; token j of sequence b lives in physical page
 *   page_table[b][j / P] at row j % P.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_F32 0
#define OR_BF16 1
#define OR_PER_HEAD 0
#define OR_2D 1

#define OR_OK 0
#define OR_BAD_ARG -1
#define OR_BAD_INDEX -2

/* ---------- storage decode / encode ---------- */

/* Exact value of element idx of a stored array (bf16 = top 16 bits of fp32). */
static double ld(const void *p, int dtype, size_t idx) {
  if (dtype == OR_F32) return (double)((const float *)p)[idx];
  uint32_t u = (uint32_t)((const uint16_t *)p)[idx] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a double to the nearest bfloat16, ties to even, directly from the
 * double (no intermediate rounding to fp32).  bf16 keeps fp32's exponent range
 * and 8 significant bits.  Returns the 16-bit pattern. */
uint16_t lla_oracle_bf16_rne(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return sign | 0x7F80;
  int e;
  frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  /* bf16 normal numbers have 8 significant bits: spacing 2^(e-8).  Below the
   * smallest normal (2^-126) the spacing is fixed at 2^-133. */
  int q = e - 8;
  if (q < -133) q = -133;
  double scaled = ldexp(a, -q); /* exact: only the exponent changes */
  double fl = floor(scaled);
  double frac = scaled - fl;
  double n = fl;
  if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) n = fl + 1.0;
  double r = ldexp(n, q);
  /* overflow: anything that rounds above the largest bf16 becomes inf */
  if (r > 3.3895313892515355e38) return sign | 0x7F80;
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

static void st(void *p, int dtype, size_t idx, double v) {
  if (dtype == OR_F32)
    ((float *)p)[idx] = (float)v; /* fp32 storage: C cast rounds to nearest */
  else
    ((uint16_t *)p)[idx] = lla_oracle_bf16_rne(v);
}

/* ---------- eq. (4): cache scalars per token and layer ---------- */

/* Teacher cache: 2*T*H*d scalars per token and layer; per-head LLA stores
 * (r_k + r_v)*H; LLA-2D stores r_k + r_v ([CR] 方法 items 2 and 6). */
void lla_oracle_cache_scalars(int T, int H, int d, int r_k, int r_v, int variant,
                              int64_t *teacher, int64_t *latent) {
  *teacher = 2LL * T * H * d;
  *latent = (variant == OR_2D) ? (int64_t)(r_k + r_v) : (int64_t)(r_k + r_v) * H;
}

/* ---------- paging ---------- */

/* Physical token slot of logical token j of sequence b, or -1 if the page
 * table entry is outside [0, num_pages) or j is outside the table. */
int64_t lla_oracle_slot(const int32_t *page_table, int max_pages, int num_pages, int P,
                        int b, int64_t j) {
  if (j < 0 || j / P >= max_pages) return -1;
  int32_t page = page_table[(size_t)b * max_pages + (size_t)(j / P)];
  if (page < 0 || page >= num_pages) return -1;
  return (int64_t)page * P + j % P;
}

/* ---------- RoPE ([CR] 方法 item 3) ---------- */

/* out = R(pos) x for a d-vector, pairs (i, i + d/2), angle pos * base^(-2i/d). */
void lla_oracle_rope(const double *x, int d, double pos, double base, double *out) {
  int h = d / 2;
  for (int i = 0; i < h; ++i) {
    double theta = pos * pow(base, -2.0 * (double)i / (double)d);
    double c = cos(theta), s = sin(theta);
    double a = x[i], b = x[i + h];
    out[i] = a * c - b * s;
    out[i + h] = a * s + b * c;
  }
}

/* ---------- shapes ---------- */

typedef struct {
  int T, D, H, d, r_k, r_v, variant, dtype, P;
  double base;
} odims;

static int dims_ok(const odims *m) {
  return m->T > 0 && m->D > 0 && m->H > 0 && m->d > 0 && (m->d % 2) == 0 && m->r_k > 0 &&
         m->r_v > 0 && m->P > 0 && (m->variant == OR_PER_HEAD || m->variant == OR_2D) &&
         (m->dtype == OR_F32 || m->dtype == OR_BF16);
}

/* Offsets of the decoder parameters of (layer l, head h, loop t). */
static size_t mu_off(const odims *m, int l, int h, int t) {
  if (m->variant == OR_PER_HEAD) return (((size_t)l * m->H + h) * m->T + t) * m->d;
  return (((size_t)l * m->T + t) * m->H + h) * m->d;
}
static size_t wup_off(const odims *m, int l, int h, int t, int r) {
  if (m->variant == OR_PER_HEAD) return ((((size_t)l * m->H + h) * m->T + t) * m->d) * r;
  return ((((size_t)l * m->T + t) * m->H + h) * m->d) * r;
}
/* Offset of the latent row of physical slot `slot` for (layer l, head h). */
static size_t pool_off(const odims *m, int num_pages, int l, int h, int64_t slot, int r) {
  int64_t page = slot / m->P, row = slot % m->P;
  if (m->variant == OR_PER_HEAD)
    return ((((size_t)l * num_pages + page) * m->H + h) * m->P + row) * r;
  return (((size_t)l * num_pages + page) * m->P + row) * r;
}

/* ---------- eq. (3): reconstruction of one loop-t vector ---------- */

/* xhat[e] = mu[e] + sum_r W_up[e][r] * c[r]  (row-vector c W_up,t^T + mu_t) */
static void reconstruct(const odims *m, const void *mu, const void *wup, size_t muo, size_t wo,
                        int r, const double *c, double *xhat) {
  for (int e = 0; e < m->d; ++e) {
    double acc = ld(mu, m->dtype, muo + e);
    for (int k = 0; k < r; ++k) acc += ld(wup, m->dtype, wo + (size_t)e * r + k) * c[k];
    xhat[e] = acc;
  }
}

/* ---------- encode + append (eq. (2)) ---------- */

int lla_oracle_encode(int T, int D, int H, int d, int r_k, int r_v, int variant, int dtype, int P,
                      const void *mu_k, const void *mu_v, const void *wdown_k,
                      const void *wdown_v, void *k_pool, void *v_pool,
                      const int32_t *page_table, int batch, int max_pages, int num_pages,
                      const void *x_k, const void *x_v, const int32_t *pos0, int n_new,
                      int layer0, int n_layers) {
  odims m = {T, D, H, d, r_k, r_v, variant, dtype, P, 10000.0};
  if (!dims_ok(&m) || n_new < 0 || layer0 < 0 || n_layers < 0 || layer0 + n_layers > D)
    return OR_BAD_ARG;
  const int width = (variant == OR_PER_HEAD) ? T * d : T * H * d; /* encoder input */
  const int groups = (variant == OR_PER_HEAD) ? H : 1;          /* latents per token */
  double *xv = (double *)malloc(sizeof(double) * width);
  int rc = OR_OK;
  for (int kv = 0; kv < 2; ++kv) {
    const void *x = kv ? x_v : x_k;
    const void *mu = kv ? mu_v : mu_k;
    const void *wd = kv ? wdown_v : wdown_k;
    void *pool = kv ? v_pool : k_pool;
    const int r = kv ? r_v : r_k;
    for (int li = 0; li < n_layers; ++li) {
      const int l = layer0 + li;
      for (int b = 0; b < batch; ++b) {
        for (int n = 0; n < n_new; ++n) {
          int64_t slot = lla_oracle_slot(page_table, max_pages, num_pages, P, b,
                                         (int64_t)pos0[b] + n);
          if (slot < 0) { rc = OR_BAD_INDEX; continue; }
          for (int g = 0; g < groups; ++g) {
            /* x = [x_1; ...; x_T] for this token (and head, per-head variant) */
            size_t xo = ((((size_t)li * batch + b) * n_new + n) * groups + g) * (size_t)width;
            size_t muo = ((size_t)l * groups + g) * (size_t)width;
            size_t wo = ((size_t)l * groups + g) * (size_t)width * r;
            for (int i = 0; i < width; ++i) xv[i] = ld(x, dtype, xo + i) - ld(mu, dtype, muo + i);
            size_t po = pool_off(&m, num_pages, l, g, slot, r);
            for (int k = 0; k < r; ++k) {
              double c = 0.0;
              for (int i = 0; i < width; ++i) c += xv[i] * ld(wd, dtype, wo + (size_t)i * r + k);
              st(pool, dtype, po + k, c);
            }
          }
        }
      }
    }
  }
  free(xv);
  return rc;
}

/* ---------- attention of one query over ctx cached tokens ---------- */

/* Textbook attention of query vector q (pre-RoPE, position qpos) of head h
 * over the retained logical tokens of [0, ctx) of sequence b, all in double:
 * token j takes part iff j < keep_lo or j >= keep_hi (keep_lo = keep_hi = ctx:
 * every token).  Tokens that do not take part are never looked up.  Writes
 * out[d]. */
static int attend_one(const odims *m, const void *mu_k, const void *mu_v, const void *wup_k,
                      const void *wup_v, const void *k_pool, const void *v_pool,
                      const int32_t *page_table, int max_pages, int num_pages, int layer,
                      int loop, int b, int h, const double *q, int64_t qpos, int64_t ctx,
                      int64_t keep_lo, int64_t keep_hi, double scale, double *out) {
  const int d = m->d;
  double *qr = (double *)malloc(sizeof(double) * d);
  double *ck = (double *)malloc(sizeof(double) * m->r_k);
  double *cv = (double *)malloc(sizeof(double) * m->r_v);
  double *kh = (double *)malloc(sizeof(double) * d);
  double *kr = (double *)malloc(sizeof(double) * d);
  double *vh = (double *)malloc(sizeof(double) * d * (size_t)ctx);
  double *s = (double *)malloc(sizeof(double) * (size_t)ctx);
  int rc = OR_OK;
  lla_oracle_rope(q, d, (double)qpos, m->base, qr);
  size_t muko = mu_off(m, layer, h, loop), muvo = mu_off(m, layer, h, loop);
  size_t wko = wup_off(m, layer, h, loop, m->r_k), wvo = wup_off(m, layer, h, loop, m->r_v);
  for (int64_t j = 0; j < ctx; ++j) {
    s[j] = -INFINITY; /* weight 0 unless the token takes part */
    if (j >= keep_lo && j < keep_hi) continue;
    int64_t slot = lla_oracle_slot(page_table, max_pages, num_pages, m->P, b, j);
    if (slot < 0) { rc = OR_BAD_INDEX; break; }
    size_t pk = pool_off(m, num_pages, layer, h, slot, m->r_k);
    size_t pv = pool_off(m, num_pages, layer, h, slot, m->r_v);
    for (int k = 0; k < m->r_k; ++k) ck[k] = ld(k_pool, m->dtype, pk + k);
    for (int k = 0; k < m->r_v; ++k) cv[k] = ld(v_pool, m->dtype, pv + k);
    reconstruct(m, mu_k, wup_k, muko, wko, m->r_k, ck, kh);               /* eq. (3), K */
    reconstruct(m, mu_v, wup_v, muvo, wvo, m->r_v, cv, vh + (size_t)j * d); /* eq. (3), V */
    lla_oracle_rope(kh, d, (double)j, m->base, kr); /* RoPE after reconstruction */
    double dot = 0.0;
    for (int e = 0; e < d; ++e) dot += qr[e] * kr[e];
    s[j] = scale * dot;
  }
  if (rc == OR_OK) {
    double mx = -INFINITY;
    for (int64_t j = 0; j < ctx; ++j) mx = s[j] > mx ? s[j] : mx;
    double z = 0.0;
    for (int64_t j = 0; j < ctx; ++j) { s[j] = exp(s[j] - mx); z += s[j]; }
    for (int e = 0; e < d; ++e) {
      double acc = 0.0;
      for (int64_t j = 0; j < ctx; ++j)
        if (s[j] != 0.0) acc += s[j] * vh[(size_t)j * d + e]; /* skipped tokens have no v_hat */
      out[e] = acc / z;
    }
  }
  free(qr); free(ck); free(cv); free(kh); free(kr); free(vh); free(s);
  return rc;
}

static void set_threads(int threads) {
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
}

/* ---------- decode: one query per sequence ---------- */

/* out[B][H][d] (double).  q [B][H][d] in the storage dtype.  loop is 0-based
 * (loop t = loop + 1 in the pages' 1-based notation).  Returns OR_OK, or an
 * error if an index is out of range (the affected rows are left NaN). */
int lla_oracle_decode(int T, int D, int H, int d, int r_k, int r_v, int variant, int dtype,
                      int P, double rope_base, const void *mu_k, const void *mu_v,
                      const void *wup_k, const void *wup_v, const void *k_pool,
                      const void *v_pool, const int32_t *page_table, int batch, int max_pages,
                      int num_pages, int layer, int loop, const void *q, const int32_t *q_pos,
                      const int32_t *ctx_len, double scale, double *out, int threads) {
  odims m = {T, D, H, d, r_k, r_v, variant, dtype, P, rope_base};
  if (!dims_ok(&m) || layer < 0 || layer >= D || loop < 0 || loop >= T) return OR_BAD_ARG;
  set_threads(threads);
  int rc = OR_OK;
#pragma omp parallel for schedule(dynamic) reduction(min : rc)
  for (int bh = 0; bh < batch * H; ++bh) {
    int b = bh / H, h = bh % H;
    double *o = out + (size_t)bh * d;
    for (int e = 0; e < d; ++e) o[e] = NAN;
    if (ctx_len[b] < 1 || (int64_t)ctx_len[b] > (int64_t)max_pages * P) { rc = OR_BAD_INDEX; continue; }
    double *qv = (double *)malloc(sizeof(double) * d);
    for (int e = 0; e < d; ++e) qv[e] = ld(q, dtype, (size_t)bh * d + e);
    int r1 = attend_one(&m, mu_k, mu_v, wup_k, wup_v, k_pool, v_pool, page_table, max_pages,
                        num_pages, layer, loop, b, h, qv, q_pos[b], ctx_len[b], ctx_len[b],
                        ctx_len[b], scale, o);
    if (r1 != OR_OK) { rc = r1 < rc ? r1 : rc; for (int e = 0; e < d; ++e) o[e] = NAN; }
    free(qv);
  }
  return rc;
}

/* ---------- decode over a sink + window retained set ([CR] 四:结果 item 10, Table 9) ---------- */

/* As lla_oracle_decode, but with token eviction: of the ctx_len[b] tokens of
 * sequence b only the first n_sink (the attention sink) and the last `window`
 * take part; the rest are evicted, never looked up (their page-table entries
 * may be invalid).  Retained tokens keep their logical positions for RoPE. */
int lla_oracle_decode_window(int T, int D, int H, int d, int r_k, int r_v, int variant, int dtype,
                             int P, double rope_base, const void *mu_k, const void *mu_v,
                             const void *wup_k, const void *wup_v, const void *k_pool,
                             const void *v_pool, const int32_t *page_table, int batch, int max_pages,
                             int num_pages, int layer, int loop, const void *q, const int32_t *q_pos,
                             const int32_t *ctx_len, int n_sink, int window, double scale,
                             double *out, int threads) {
  odims m = {T, D, H, d, r_k, r_v, variant, dtype, P, rope_base};
  if (!dims_ok(&m) || layer < 0 || layer >= D || loop < 0 || loop >= T || n_sink < 0 || window < 0 ||
      n_sink + window < 1)
    return OR_BAD_ARG;
  set_threads(threads);
  int rc = OR_OK;
#pragma omp parallel for schedule(dynamic) reduction(min : rc)
  for (int bh = 0; bh < batch * H; ++bh) {
    int b = bh / H, h = bh % H;
    double *o = out + (size_t)bh * d;
    for (int e = 0; e < d; ++e) o[e] = NAN;
    int64_t ctx = ctx_len[b];
    if (ctx < 1 || ctx > (int64_t)max_pages * P) { rc = OR_BAD_INDEX; continue; }
    int64_t lo = n_sink < ctx ? n_sink : ctx;           /* sink: [0, lo) */
    int64_t hi = ctx - window > lo ? ctx - window : lo;  /* window: [hi, ctx) */
    double *qv = (double *)malloc(sizeof(double) * d);
    for (int e = 0; e < d; ++e) qv[e] = ld(q, dtype, (size_t)bh * d + e);
    int r1 = attend_one(&m, mu_k, mu_v, wup_k, wup_v, k_pool, v_pool, page_table, max_pages,
                        num_pages, layer, loop, b, h, qv, q_pos[b], ctx, lo, hi, scale, o);
    if (r1 != OR_OK) { rc = r1 < rc ? r1 : rc; for (int e = 0; e < d; ++e) o[e] = NAN; }
    free(qv);
  }
  return rc;
}

/* ---------- prefill: n_q causal queries per sequence ---------- */

/* Query i of sequence b sits at position p0[b] + i and attends over logical
 * tokens [0, p0[b] + i].  q and out are [B][n_q][H][d]. */
int lla_oracle_prefill(int T, int D, int H, int d, int r_k, int r_v, int variant, int dtype,
                       int P, double rope_base, const void *mu_k, const void *mu_v,
                       const void *wup_k, const void *wup_v, const void *k_pool,
                       const void *v_pool, const int32_t *page_table, int batch, int max_pages,
                       int num_pages, int layer, int loop, int n_q, const void *q,
                       const int32_t *p0, double scale, double *out, int threads) {
  odims m = {T, D, H, d, r_k, r_v, variant, dtype, P, rope_base};
  if (!dims_ok(&m) || layer < 0 || layer >= D || loop < 0 || loop >= T || n_q < 0)
    return OR_BAD_ARG;
  set_threads(threads);
  int rc = OR_OK;
#pragma omp parallel for schedule(dynamic) reduction(min : rc)
  for (int row = 0; row < batch * n_q * H; ++row) {
    int h = row % H, i = (row / H) % n_q, b = row / (H * n_q);
    double *o = out + (size_t)row * d;
    int64_t pos = (int64_t)p0[b] + i;
    for (int e = 0; e < d; ++e) o[e] = NAN;
    if (p0[b] < 0 || pos + 1 > (int64_t)max_pages * P) { rc = OR_BAD_INDEX; continue; }
    double *qv = (double *)malloc(sizeof(double) * d);
    for (int e = 0; e < d; ++e) qv[e] = ld(q, dtype, (size_t)row * d + e);
    int r1 = attend_one(&m, mu_k, mu_v, wup_k, wup_v, k_pool, v_pool, page_table, max_pages,
                        num_pages, layer, loop, b, h, qv, pos, pos + 1, pos + 1, pos + 1, scale, o);
    if (r1 != OR_OK) { rc = r1 < rc ? r1 : rc; for (int e = 0; e < d; ++e) o[e] = NAN; }
    free(qv);
  }
  return rc;
}

/* ---------- decoupled RoPE: NoPE content path + explicit rotary branch ---------- */
/*
 * [CR] 四:结果 item 10 (appendix J): full RoPE depends on position and blocks
 * absorbing the K decoder into attention, so the absorbed variant scores with
 * a NoPE content path plus an explicit rotary branch of width d_rope (64 or
 * 32).  Readings (listed in the design doc): the content key of loop t is the eq. (3)
 * reconstruction, not rotated; the rotary key is one d_rope-vector per
 * (token, layer), shared by all heads and loops, stored after rotation at the
 * token's position with RoPE over d_rope dims (pairs (i, i + d_rope/2), angle
 * p * base^(-2i/d_rope)); a query row holds [q_content (d) ; q_rotary (d_rope)],
 * and q_rotary is rotated at q_pos; the score is
 *   s_j = scale (<q_content, k_hat_j> + <R(q_pos) q_rotary, kr_j>),
 * scale defaulting to 1/sqrt(d + d_rope); V is rebuilt by eq. (3) as in decode.
 * Layouts: kr_pool [D][num_pages][P][d_rope]; kr_new [n_layers][B][n_new][d_rope];
 * q [B][H][d + d_rope]; out [B][H][d].  Per-head LLA only.
 */

/* Rotate kr_new at position pos0[b] + n and store it (rounded once to the
 * storage type) in the slot of that logical token, for layers layer0 .. +n_layers-1.
 * Tokens whose slot is outside the page table (or whose entry is invalid) are
 * skipped and reported with OR_BAD_INDEX. */
int lla_oracle_rope_key_append(int D, int P, int d_rope, double rope_base, int dtype,
                               void *kr_pool, const int32_t *page_table, int batch,
                               int max_pages, int num_pages, const void *kr_new,
                               const int32_t *pos0, int n_new, int layer0, int n_layers) {
  if (D <= 0 || P <= 0 || d_rope <= 0 || d_rope % 2 || layer0 < 0 || n_layers < 0 ||
      layer0 + n_layers > D || n_new < 0 || (dtype != OR_F32 && dtype != OR_BF16))
    return OR_BAD_ARG;
  int rc = OR_OK;
  double *x = (double *)malloc(sizeof(double) * d_rope);
  double *y = (double *)malloc(sizeof(double) * d_rope);
  for (int l = 0; l < n_layers; ++l)
    for (int b = 0; b < batch; ++b)
      for (int n = 0; n < n_new; ++n) {
        int64_t pos = (int64_t)pos0[b] + n;
        int64_t slot = lla_oracle_slot(page_table, max_pages, num_pages, P, b, pos);
        if (slot < 0) { rc = OR_BAD_INDEX; continue; }
        size_t src = (((size_t)l * batch + b) * n_new + n) * d_rope;
        for (int e = 0; e < d_rope; ++e) x[e] = ld(kr_new, dtype, src + e);
        lla_oracle_rope(x, d_rope, (double)pos, rope_base, y);
        size_t dst = ((size_t)(layer0 + l) * num_pages * P + (size_t)slot) * d_rope;
        for (int e = 0; e < d_rope; ++e) st(kr_pool, dtype, dst + e, y[e]);
      }
  free(x); free(y);
  return rc;
}

/* Decode with the decoupled score above: one query row per sequence. */
int lla_oracle_decoupled_decode(int T, int D, int H, int d, int r_k, int r_v, int d_rope,
                                int dtype, int P, double rope_base, const void *mu_k,
                                const void *mu_v, const void *wup_k, const void *wup_v,
                                const void *k_pool, const void *v_pool, const void *kr_pool,
                                const int32_t *page_table, int batch, int max_pages,
                                int num_pages, int layer, int loop, const void *q,
                                const int32_t *q_pos, const int32_t *ctx_len, double scale,
                                double *out, int threads) {
  odims m = {T, D, H, d, r_k, r_v, OR_PER_HEAD, dtype, P, rope_base};
  if (!dims_ok(&m) || d_rope <= 0 || d_rope % 2 || layer < 0 || layer >= D || loop < 0 || loop >= T)
    return OR_BAD_ARG;
  set_threads(threads);
  const int dq = d + d_rope;
  int rc = OR_OK;
#pragma omp parallel for schedule(dynamic) reduction(min : rc)
  for (int bh = 0; bh < batch * H; ++bh) {
    int b = bh / H, h = bh % H;
    double *o = out + (size_t)bh * d;
    for (int e = 0; e < d; ++e) o[e] = NAN;
    int64_t ctx = ctx_len[b];
    if (ctx < 1 || ctx > (int64_t)max_pages * P) { rc = OR_BAD_INDEX; continue; }
    double *qc = (double *)malloc(sizeof(double) * d);
    double *qr = (double *)malloc(sizeof(double) * d_rope);
    double *qrr = (double *)malloc(sizeof(double) * d_rope);
    double *ck = (double *)malloc(sizeof(double) * r_k);
    double *cv = (double *)malloc(sizeof(double) * r_v);
    double *kh = (double *)malloc(sizeof(double) * d);
    double *vh = (double *)malloc(sizeof(double) * d * (size_t)ctx);
    double *s = (double *)malloc(sizeof(double) * (size_t)ctx);
    for (int e = 0; e < d; ++e) qc[e] = ld(q, dtype, (size_t)bh * dq + e);
    for (int e = 0; e < d_rope; ++e) qr[e] = ld(q, dtype, (size_t)bh * dq + d + e);
    lla_oracle_rope(qr, d_rope, (double)q_pos[b], rope_base, qrr); /* rotary branch of q */
    size_t muo = mu_off(&m, layer, h, loop);
    size_t wko = wup_off(&m, layer, h, loop, r_k), wvo = wup_off(&m, layer, h, loop, r_v);
    int r1 = OR_OK;
    for (int64_t j = 0; j < ctx; ++j) {
      int64_t slot = lla_oracle_slot(page_table, max_pages, num_pages, P, b, j);
      if (slot < 0) { r1 = OR_BAD_INDEX; break; }
      size_t pk = pool_off(&m, num_pages, layer, h, slot, r_k);
      size_t pv = pool_off(&m, num_pages, layer, h, slot, r_v);
      size_t pr = ((size_t)layer * num_pages * P + (size_t)slot) * d_rope;
      for (int k = 0; k < r_k; ++k) ck[k] = ld(k_pool, dtype, pk + k);
      for (int k = 0; k < r_v; ++k) cv[k] = ld(v_pool, dtype, pv + k);
      reconstruct(&m, mu_k, wup_k, muo, wko, r_k, ck, kh);                /* eq. (3), K, no RoPE */
      reconstruct(&m, mu_v, wup_v, muo, wvo, r_v, cv, vh + (size_t)j * d); /* eq. (3), V */
      double dot = 0.0;
      for (int e = 0; e < d; ++e) dot += qc[e] * kh[e];
      for (int e = 0; e < d_rope; ++e) dot += qrr[e] * ld(kr_pool, dtype, pr + e);
      s[j] = scale * dot;
    }
    if (r1 == OR_OK) {
      double mx = -INFINITY;
      for (int64_t j = 0; j < ctx; ++j) mx = s[j] > mx ? s[j] : mx;
      double z = 0.0;
      for (int64_t j = 0; j < ctx; ++j) { s[j] = exp(s[j] - mx); z += s[j]; }
      for (int e = 0; e < d; ++e) {
        double acc = 0.0;
        for (int64_t j = 0; j < ctx; ++j) acc += s[j] * vh[(size_t)j * d + e];
        o[e] = acc / z;
      }
    } else {
      rc = r1 < rc ? r1 : rc;
    }
    free(qc); free(qr); free(qrr); free(ck); free(cv); free(kh); free(vh); free(s);
  }
  return rc;
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int lla_oracle_max_threads(int threads) {
  set_threads(threads);
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
