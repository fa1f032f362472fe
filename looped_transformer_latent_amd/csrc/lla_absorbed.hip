// Decoupled-RoPE decode with the K decoder absorbed into the query, bf16
// per-head LLA (cc.laoqi.cc close reading, 四:结果 item 10, appendix J).
//
// Full RoPE rotates every reconstructed key by its own position, which keeps
// the K decoder out of any query-side absorption.  The decoupled variant
// scores with a NoPE content path plus an explicit rotary branch of width
// d_rope:
//   s_j = scale (<q_c, mu_k,t + c_k,j W_up,k,t^T> + <R(q_pos) q_r, kr_j>),
// kr_j being the token's rotary key, stored after rotation at its position
// (one d_rope-vector per token and layer, shared by heads and loops).  By
// linearity the content term is <q~, c_k,j> + <q_c, mu_k,t> with
// q~ = W_up,k,t^T q_c (r_k wide), and the second term is the same for every j
// of a row, so softmax drops it: per token and head what is left is an r_k dot
// product plus a d_rope one, instead of rebuilding a d_head key.  V is absorbed
// as in the latent decode: e^s-weighted sums of c_v, one up-projection per
// (row, head) at the end.
//
// Decomposition (as the latent decode): a workgroup is (row, head group,
// split); wave w owns HPW heads; lane (g, n) holds token n of each page, c_k
// columns 16 rt + 4 g .. + 3, c_v columns CV g .. + CV - 1 and rotary columns
// DR/4 g .. + DR/4 - 1.  Scores reduce across the four lane rows; pages stream
// through a ring of LOOK + 2 slots with LOOK in flight.  Bound by HBM:
// 2 (H (r_k + r_v) + d_rope) bytes per cached token and (layer, loop) call.
//
// The rotary keys are written by rope_key_append_kernel (below): x rotated by
// RoPE over d_rope dims at the token's position, from the caller's d_rope
// table, rounded once to bf16.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {

namespace {
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));
}

template <int DH, int RK, int RV, int DR, int HPW, int NW>
__global__ __launch_bounds__(64 * NW, 1) void absorbed_kernel(AttnArgs a) {
  constexpr int RT = RK / 16;  // 16-column tiles of c_k
  constexpr int CV = RV / 4;   // c_v columns per lane
  constexpr int KV = CV / 8;   // 16-byte c_v loads per lane and head
  constexpr int CR = DR / 4;   // rotary columns per lane
  constexpr int KR = CR / 8;   // 16-byte rotary loads per lane
  constexpr int HALF = DR / 2;
  constexpr int DQ = DH + DR;  // query row: [content; rotary]
  static_assert(RK % 16 == 0 && RV % 32 == 0 && DR % 32 == 0 && DH % 16 == 0, "shape");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;

  int bid = blockIdx.x;
  const int split = bid % a.splits;
  bid /= a.splits;
  const int hg = bid % a.head_groups;
  const int row = bid / a.head_groups;

  int qp = a.q_pos[row], ctx = a.ctx_len[row];
  int errbits = 0;
  if (ctx < 1 || ctx > a.max_ctx || qp < 0 || qp >= a.rope_len) {
    errbits |= LLA_DEVERR_CTX;
    ctx = 0;
    qp = 0;
  }
  const int npages = (ctx + kPage - 1) / kPage;
  const int lp0 = split * a.pages_per_split;
  const int lp1 = min(lp0 + a.pages_per_split, npages);
  const int h0 = (hg * a.waves + wave) * HPW;

  // ---- prologue: q~ = qscale W_up,k,t^T q_c and qscale R(q_pos) q_r ----
  // q~ column 16 rt + 4 g + e: lane n of row g sums d = n, n + 16, ..., then
  // the row's 16 lanes add up their parts.
  float qk[HPW][RT][4], qr[HPW][CR];
  {
    const float *rq = a.rope + (long long)qp * DR;  // [d_rope/2][2] (cos, sin)
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = h0 + hh;
      const uint16_t *qrow = (const uint16_t *)a.q + ((long long)row * a.H + h) * DQ;
      const uint16_t *w = (const uint16_t *)a.wup_k + (long long)h * a.wup_head_stride_k;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < DH / 16; ++i) {
          const int d = 16 * i + n;
          const float qd = bf16_to_f32(qrow[d]);
          const u32x2 wv = *(const u32x2 *)(w + (long long)d * RK + 16 * rt + 4 * g);
          p[0] = fmaf(qd, bf16_lo(wv[0]), p[0]);
          p[1] = fmaf(qd, bf16_hi(wv[0]), p[1]);
          p[2] = fmaf(qd, bf16_lo(wv[1]), p[2]);
          p[3] = fmaf(qd, bf16_hi(wv[1]), p[3]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) qk[hh][rt][e] = a.qscale * sum_in_row(p[e]);
      }
      // rotary columns CR g + k: pairs i0 + k, the first (g < 2) or second half
      const int i0 = CR * (g & 1);
      const bool upper = g >= 2;
      u32x4 xa8[CR / 8], xb8[CR / 8];
#pragma unroll
      for (int k8 = 0; k8 < CR / 8; ++k8) {
        xa8[k8] = *(const u32x4 *)(qrow + DH + i0 + 8 * k8);
        xb8[k8] = *(const u32x4 *)(qrow + DH + HALF + i0 + 8 * k8);
      }
#pragma unroll
      for (int k4 = 0; k4 < CR / 2; ++k4) {
        const f32x4 t = *(const f32x4 *)(rq + 2 * (i0 + 2 * k4));  // (cos, sin) of pairs i0 + 2 k4, + 1
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int k = 2 * k4 + e;
          const uint32_t wa = xa8[k / 8][(k % 8) / 2], wb = xb8[k / 8][(k % 8) / 2];
          const float xa = k & 1 ? bf16_hi(wa) : bf16_lo(wa), xb = k & 1 ? bf16_hi(wb) : bf16_lo(wb);
          const float cs = t[2 * e], sn = t[2 * e + 1];
          qr[hh][k] = a.qscale * (upper ? xa * sn + xb * cs : xa * cs - xb * sn);
        }
      }
    }
  }

  float m_run[HPW], z[HPW], acc[HPW][CV];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    m_run[hh] = -INFINITY;
    z[hh] = 0.f;
#pragma unroll
    for (int k = 0; k < CV; ++k) acc[hh][k] = 0.f;
  }

  // Rows past ctx_len (last page only) re-read the last valid row; their
  // scores are forced to -inf.  An invalid page-table entry reads page 0 and
  // masks the page.
  struct Page {
    u32x2 k[HPW][RT];
    u32x4 v[HPW][KV];
    u32x4 r[KR];
    int ok;
    int last;
  };
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int *s_pt = (int *)smem;
  {
    const int *pt_row = a.page_table + (long long)row * a.max_pages;
    for (int i = threadIdx.x; i < lp1 - lp0; i += blockDim.x) s_pt[i] = pt_row[lp0 + i];
    __syncthreads();
  }
  auto page_at = [&](int lp) -> int { return __builtin_amdgcn_readfirstlane(s_pt[lp - lp0]); };

  auto load_page = [&](int lp, int pp_raw, Page &pg) {
    pg.ok = (pp_raw >= 0 && pp_raw < a.num_pages);
    const long long pp = pg.ok ? pp_raw : 0;
    pg.last = min(kPage - 1, ctx - 1 - lp * kPage);
    const int row_n = min(n, pg.last);
    const char *kpage = a.k_pool + pp * a.pool_page_stride_k * 2;
    const char *vpage = a.v_pool + pp * a.pool_page_stride_v * 2;
    const char *rpage = a.kr_pool + pp * a.kr_page_stride * 2;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = h0 + hh;
      const uint32_t koff = (uint32_t)((h * a.pool_head_stride_k + row_n * RK + 4 * g) * 2);
      const uint32_t voff = (uint32_t)((h * a.pool_head_stride_v + row_n * RV + CV * g) * 2);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        pg.k[hh][rt] = __builtin_nontemporal_load((const u32x2 *)(kpage + koff + 32 * rt));
#pragma unroll
      for (int kv = 0; kv < KV; ++kv)
        pg.v[hh][kv] = __builtin_nontemporal_load((const u32x4 *)(vpage + voff + kv * 16));
    }
    const uint32_t roff = (uint32_t)((row_n * DR + CR * g) * 2);
#pragma unroll
    for (int k = 0; k < KR; ++k) pg.r[k] = *(const u32x4 *)(rpage + roff + k * 16);
  };

  auto compute_page = [&](const Page &cur, int lp) {
    errbits |= cur.ok ? 0 : LLA_DEVERR_PAGE;
    const bool valid = cur.ok && n <= cur.last && lp < lp1;  // lp >= lp1: ring padding
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      float sc = 0.f;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        sc = fmaf(bf16_lo(cur.k[hh][rt][0]), qk[hh][rt][0], sc);
        sc = fmaf(bf16_hi(cur.k[hh][rt][0]), qk[hh][rt][1], sc);
        sc = fmaf(bf16_lo(cur.k[hh][rt][1]), qk[hh][rt][2], sc);
        sc = fmaf(bf16_hi(cur.k[hh][rt][1]), qk[hh][rt][3], sc);
      }
#pragma unroll
      for (int k = 0; k < KR; ++k) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc = fmaf(bf16_lo(cur.r[k][e]), qr[hh][8 * k + 2 * e], sc);
          sc = fmaf(bf16_hi(cur.r[k][e]), qr[hh][8 * k + 2 * e + 1], sc);
        }
      }
      sc = sum_across_rows(sc);
      sc = valid ? sc : -INFINITY;
      const float mt = max_in_row(sc);
      if (mt > m_run[hh]) {  // wave-uniform
        const float corr = fast_exp2(m_run[hh] - mt);
        z[hh] *= corr;
#pragma unroll
        for (int k = 0; k < CV; ++k) acc[hh][k] *= corr;
        m_run[hh] = mt;
      }
      const float p = fast_exp2(sc - m_run[hh]);
      z[hh] += p;
#pragma unroll
      for (int kv = 0; kv < KV; ++kv) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[hh][8 * kv + 2 * e] = fmaf(p, bf16_lo(cur.v[hh][kv][e]), acc[hh][8 * kv + 2 * e]);
          acc[hh][8 * kv + 2 * e + 1] = fmaf(p, bf16_hi(cur.v[hh][kv][e]), acc[hh][8 * kv + 2 * e + 1]);
        }
      }
    }
  };

  // Ring of NBUF slots; every trip computes NBUF pages (pages past the split
  // are masked) and every load is issued (clamped to the split's last page),
  // so both ways into the loop head leave the same loads outstanding.
  constexpr int LOOK = LLA_DECODE_LOOK, NBUF = LOOK + 2;
  if (lp0 < lp1) {
    const int lp_end = lp0 + (lp1 - lp0 + NBUF - 1) / NBUF * NBUF;
    Page ring[NBUF];
#pragma unroll
    for (int u = 0; u < LOOK; ++u) {
      const int l = min(lp0 + u, lp1 - 1);
      load_page(l, page_at(l), ring[u]);
    }
    for (int lp = lp0; lp < lp_end; lp += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int l = min(lp + u + LOOK, lp1 - 1);
        load_page(l, page_at(l), ring[(u + LOOK) % NBUF]);
        compute_page(ring[u], lp + u);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- reduce over the 16 token lanes of each row ----
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    z[hh] = sum_in_row(z[hh]);
#pragma unroll
    for (int k = 0; k < CV; ++k) acc[hh][k] = sum_in_row(acc[hh][k]);
  }
  if (errbits && threadIdx.x == 0) atomicOr(a.err, errbits);
  const bool bad = __syncthreads_or(errbits != 0);

  float *sh = (float *)(s_pt + a.pages_per_split);  // [waves][HPW][RV + 2]
  float *mine = sh + (wave * HPW) * (RV + 2);
  if (a.splits > 1) {  // partials for the merge launch
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = h0 + hh;
      float *part = a.partials + (((long long)row * a.H + h) * a.splits + split) * (RV + 2);
      if (n == 0) {
#pragma unroll
        for (int k = 0; k < CV; ++k) part[CV * g + k] = acc[hh][k];
      }
      if (lane == 0) {
        part[RV] = m_run[hh];
        part[RV + 1] = bad ? __builtin_nanf("") : z[hh];
      }
    }
    return;
  }
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const float zz = bad ? __builtin_nanf("") : z[hh];
    if (n == 0) {
#pragma unroll
      for (int k = 0; k < CV; ++k) mine[hh * (RV + 2) + CV * g + k] = acc[hh][k] / zz;
    }
  }
  __syncthreads();

  // ---- V up-projection: out = mu_v,t + accn W_up,v,t^T ----
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int h = h0 + hh;
    const char *w = a.wup_v + (long long)h * a.wup_head_stride_v * 2;
    const uint16_t *mu = (const uint16_t *)a.mu_v + (long long)h * a.mu_head_stride;
    const float *an = mine + hh * (RV + 2);
    for (int e = lane; e < DH; e += 64) {
      float o = bf16_to_f32(mu[e]);
      const char *we = w + (long long)e * RV * 2;
#pragma unroll
      for (int r8 = 0; r8 < RV / 8; ++r8) {
        const u32x4 v = *(const u32x4 *)(we + r8 * 16);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          o = fmaf(bf16_lo(v[k]), an[8 * r8 + 2 * k], o);
          o = fmaf(bf16_hi(v[k]), an[8 * r8 + 2 * k + 1], o);
        }
      }
      ((uint16_t *)a.out)[((long long)row * a.H + h) * DH + e] = (uint16_t)f32_to_bf16(o);
    }
  }
}

// ---------------------------------------------------------------- rotary key append

// One thread per (layer, token, RoPE pair): kr[i], kr[i + d_rope/2] of the
// token's slot = the pair of x rotated by the table's angle at its position.
__global__ __launch_bounds__(256) void rope_key_append_kernel(RopeAppendArgs a) {
  const int h = a.d_rope / 2;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)a.n_layers * a.batch * a.n_new * h;
  if (idx >= total) return;
  const int i = (int)(idx % h);
  const long long tok = idx / h;  // (layer, b, n) flattened
  const int n = (int)(tok % a.n_new);
  const int b = (int)((tok / a.n_new) % a.batch);
  const int l = (int)(tok / ((long long)a.n_new * a.batch));
  const long long pos = (long long)a.pos0[b] + n;
  if (pos < 0 || pos >= (long long)a.max_pages * kPage) {
    if (i == 0) atomicOr(a.err, LLA_DEVERR_APPEND);
    return;
  }
  if (pos >= a.rope_len) {
    if (i == 0) atomicOr(a.err, LLA_DEVERR_CTX);
    return;
  }
  const int page = a.page_table[(long long)b * a.max_pages + pos / kPage];
  if (page < 0 || page >= a.num_pages) {
    if (i == 0) atomicOr(a.err, LLA_DEVERR_PAGE);
    return;
  }
  const uint16_t *x = (const uint16_t *)a.kr_new + tok * a.d_rope;
  const float xa = bf16_to_f32(x[i]), xb = bf16_to_f32(x[i + h]);
  const float cs = a.rope[pos * a.d_rope + 2 * i], sn = a.rope[pos * a.d_rope + 2 * i + 1];
  uint16_t *dst = (uint16_t *)a.kr_pool + (long long)l * a.layer_stride +
                  ((long long)page * kPage + pos % kPage) * a.d_rope;
  dst[i] = (uint16_t)f32_to_bf16(xa * cs - xb * sn);
  dst[i + h] = (uint16_t)f32_to_bf16(xa * sn + xb * cs);
}

// ---------------------------------------------------------------- dispatch

// (d_head, r_k, r_v, d_rope, heads per wave, waves per workgroup)
#define LLA_ABSORBED_SHAPES(X) \
  X(128, 16, 32, 64, 2, 8)     \
  X(128, 16, 32, 32, 2, 8)     \
  X(128, 96, 160, 64, 1, 4)    \
  X(128, 96, 160, 32, 1, 4)

bool absorbed_supported(int d_head, int r_k, int r_v, int d_rope, int hpw, int waves) {
#define X(DH, RK, RV, DR, HPW, NW) \
  if (d_head == DH && r_k == RK && r_v == RV && d_rope == DR && hpw == HPW && waves == NW) return true;
  LLA_ABSORBED_SHAPES(X)
#undef X
  return false;
}

hipError_t launch_absorbed(int d_head, int r_k, int r_v, int d_rope, const AttnArgs &a, hipStream_t stream) {
  const size_t shmem = sizeof(int) * a.pages_per_split + sizeof(float) * a.waves * a.heads_per_wave * (r_v + 2);
  const dim3 grid((unsigned)(a.rows * a.head_groups * a.splits));
#define X(DH, RK, RV, DR, HPW, NW)                                                                 \
  if (d_head == DH && r_k == RK && r_v == RV && d_rope == DR && a.heads_per_wave == HPW &&       \
      a.waves == NW) {                                                                             \
    hipLaunchKernelGGL((absorbed_kernel<DH, RK, RV, DR, HPW, NW>), grid, dim3(64 * NW), shmem, stream, a); \
    return hipGetLastError();                                                                      \
  }
  LLA_ABSORBED_SHAPES(X)
#undef X
  return hipErrorInvalidConfiguration;
}

hipError_t launch_rope_key_append(const RopeAppendArgs &a, hipStream_t stream) {
  const long long total = (long long)a.n_layers * a.batch * a.n_new * (a.d_rope / 2);
  if (total == 0) return hipSuccess;
  const long long blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(rope_key_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lla
