// Per-head LLA decode attention for fp32 storage (gfx950, wave64).
//
// What it computes (cc.laoqi.cc close reading, 方法 items 1-3; gist.science
// "Kernmechanismus"): for one (layer, loop t) and every query row,
//   k_hat_j = mu_k,t + c_k,j W_up,k,t^T   (eq. (3)), RoPE at position j,
//   s_j     = scale <R(q_pos) q, R(j) k_hat_j>,
//   out     = mu_v,t + (sum_j e^{s_j - m} c_v,j) W_up,v,t^T / sum_j e^{s_j - m}.
// The V side is exact by linearity of eq. (3): it is accumulated in latent
// space (r_v wide) and up-projected once per (row, head).
//
// fp32 storage is the exactness path (1e-4 relative); bf16 storage runs
// decode_g_kernel (lla_decode_g.hip).  How, per (row, head group, split)
// workgroup, one wave per HPW heads:
//  * Prologue -- fold the rotated query into the K decoder.  For RoPE pair i
//    (elements a = i, b = i + d/2) with q' = R(q_pos) q * scale * log2(e):
//      X_i(j) = q'_a k_hat_a + q'_b k_hat_b = alpha_i + sum_r A[i][r] c_r
//      Y_i(j) = q'_b k_hat_a - q'_a k_hat_b = beta_i  + sum_r B[i][r] c_r
//    with A[i][r] = q'_a W[a][r] + q'_b W[b][r], B[i][r] = q'_b W[a][r] - q'_a W[b][r],
//    alpha_i = q'_a mu_a + q'_b mu_b, beta_i = q'_b mu_a - q'_a mu_b, and then
//      s_j * log2(e) = sum_i cos(j w_i) X_i(j) + sin(j w_i) Y_i(j).
//    [A alpha; B beta] (d x (r_k + 1)) is held in registers as the A-operands of
//    v_mfma_f32_16x16x4f32 (exact fp32 products, alpha / beta in the last K-step).
//  * Per 16-token page -- one MFMA 16x16 tile gives X (or Y) for 16 pair
//    indices x 16 tokens; the latent tile [c_k, 1] is the B-operand, read
//    straight from the paged pool.  Each lane then needs cos/sin for its 16
//    pair indices and its token only: 2 FMAs per (i, token).
//  * Online softmax in base 2 with deferred rescaling; V accumulated as
//    sum_j p_j c_v,j in fp32 registers (lane = token x r_v/4 chunk).
//  * With one split the workgroup normalises and up-projects through W_up,v,t
//    itself; with several, each writes (m, Z, acc) partials and a separate
//    merge launch combines them in fixed split order (lla_merge.hip).
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {

template <int DH, int RK, int RV, int HPW, int NW>
__global__ __launch_bounds__(64 * NW) void decode_ph_kernel(AttnArgs a) {
  constexpr int NT = DH / 32;   // tile pairs: pair indices [16t, 16t + 16)
  constexpr int KS = RK / 4 + 1;  // K-steps of 4 latent columns, plus the constant column
  constexpr int CV = RV / 4;    // V latent elements per lane per token
  constexpr int HALF = DH / 2;
  static_assert(DH % 32 == 0 && RK % 16 == 0 && RV % 32 == 0, "shape");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NTH = 64 * NW;
  const int g = lane >> 4, n = lane & 15;

  int bid = blockIdx.x;
  const int split = bid % a.splits;
  bid /= a.splits;
  const int hg = bid % a.head_groups;
  const int row = bid / a.head_groups;
  const int b = row / a.n_q, qi = row - b * a.n_q;

  int qp, ctx;
  if (a.prefill) {
    qp = a.p0[b] + qi;
    ctx = qp + 1;
  } else {
    qp = a.q_pos[b];
    ctx = a.ctx_len[b];
  }
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

  // ---- prologue: query-folded K decoder as MFMA A-operands ----
  // Lane (g, n) holds row i = 16 t + n; K-step ks < RK/4 is latent column
  // (RK/4) g + ks, the last K-step carries alpha / beta in lane group g = 0.
  float A[HPW][NT][2][KS];
  {
    const float *rq = a.rope + (long long)qp * DH;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = h0 + hh;
      const float *qrow = (const float *)a.q + ((long long)row * a.H + h) * DH;
      const float *w = (const float *)a.wup_k + (long long)h * a.wup_head_stride_k;
      const float *mu = (const float *)a.mu_k + (long long)h * a.mu_head_stride;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int i = 16 * t + n;
        const float c = rq[2 * i], s = rq[2 * i + 1];
        const float qa = qrow[i], qb = qrow[i + HALF];
        const float pa = a.qscale * (qa * c - qb * s);
        const float pb = a.qscale * (qa * s + qb * c);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          float x = 0.f, y = 0.f;
          if (ks < RK / 4) {
            const int r = (RK / 4) * g + ks;
            const float wa = w[(long long)i * RK + r];
            const float wb = w[(long long)(i + HALF) * RK + r];
            x = pa * wa + pb * wb;
            y = pb * wa - pa * wb;
          } else if (g == 0) {
            const float ma = mu[i], mb = mu[i + HALF];
            x = pa * ma + pb * mb;
            y = pb * ma - pa * mb;
          }
          A[hh][t][0][ks] = x;
          A[hh][t][1][ks] = y;
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

  // Per page, lane (g, n) loads latent row n: per head its RK/4 K columns
  // (RK/4) g .. (RK/4) g + RK/4 - 1 and its CV V columns CV g ...  Tokens past
  // ctx_len (last page only) read the last valid row instead; their scores are
  // forced to -inf and their weights are exactly zero.
  constexpr int KV = CV / 4;   // 16-byte V loads per lane per head
  constexpr int KK = RK / 16;  // 16-byte K loads per lane per head
  struct Page {
    u32x4 k[HPW][KK];
    u32x4 v[HPW][KV];
    int ok;
    int last;  // last valid row of this page (15 unless the page is the last one)
  };
  // LDS: [RoPE rows: 2 chunk buffers][page-table entries of the split][epilogue]
  constexpr int SPR = DH / 4;                   // 16-byte slots per position row (fp32 pairs)
  constexpr int SWZ = SPR < 16 ? SPR - 1 : 15;  // XOR swizzle mask (row index low bits)
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int LOOK = LLA_DECODE_LOOK;  // pages in flight beyond the one computed
  constexpr int NBUF = LOOK + 2;        // page ring slots (see the main loop)
  constexpr int CH = NBUF;              // pages per RoPE chunk: one trip round the ring
  constexpr int TS = CH * kPage * SPR;  // 16-byte slots of one chunk
  constexpr int SLOTS = (TS + NTH - 1) / NTH;  // slots staged per thread
  constexpr int TSB = SLOTS * NTH;      // slots per chunk buffer (surplus = padding)
  char *s_trig = smem;
  int *s_pt = (int *)(smem + 2 * TSB * 16);
  {
    const int *pt_row = a.page_table + (long long)b * a.max_pages;
    for (int i = threadIdx.x; i < lp1 - lp0; i += blockDim.x) s_pt[i] = pt_row[lp0 + i];
    __syncthreads();
  }
  auto page_at = [&](int lp) -> int { return __builtin_amdgcn_readfirstlane(s_pt[lp - lp0]); };

  // RoPE staging.  Chunk c covers pages [lp0 + c*CH, lp0 + (c+1)*CH); row R of a
  // chunk buffer holds the table row of token position 16*(lp0 + c*CH) + R.
  // Within a row, 16-byte slot `ls` (pairs 2 ls, 2 ls + 1) is stored at
  // ls ^ (R % 16 & SWZ), so the 16 lanes of a row-group -- which read the same
  // slot of 16 consecutive positions -- hit different bank groups.  Loads are
  // unconditional (clamped slot) so the number in flight is the same on every path.
  const char *rope_b = (const char *)a.rope;
  f32x4 stg[SLOTS];
  auto stage_load = [&](int c) {
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      const int q = min((int)threadIdx.x + j * NTH, TS - 1);
      const int R = q / SPR, ps = q % SPR, rn = R % kPage;
      const int pos = min((lp0 + c * CH + R / kPage) * kPage + rn, ctx - 1);
      stg[j] = *(const f32x4 *)(rope_b + (long long)pos * (DH * 4) + (ps ^ (rn & SWZ)) * 16);
    }
  };
  auto stage_store = [&](int c) {
    char *dst = s_trig + (c & 1) * TSB * 16;
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      const int q = threadIdx.x + j * NTH;  // q >= TS lands in the buffer's padding
      *(f32x4 *)(dst + q * 16) = stg[j];
    }
  };

  auto load_page = [&](int lp, int pp_raw, Page &pg) {
    pg.ok = (pp_raw >= 0 && pp_raw < a.num_pages);
    const long long pp = pg.ok ? pp_raw : 0;
    pg.last = min(kPage - 1, ctx - 1 - lp * kPage);
    const int row_n = min(n, pg.last);
    // uniform page bases (scalar registers) + 32-bit per-lane offsets; latents
    // are read exactly once per call, so they are loaded non-temporally
    const char *kpage = a.k_pool + pp * a.pool_page_stride_k * 4;
    const char *vpage = a.v_pool + pp * a.pool_page_stride_v * 4;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = h0 + hh;
      const uint32_t koff = (uint32_t)((h * a.pool_head_stride_k + row_n * RK) * 4);
      const uint32_t voff = (uint32_t)((h * a.pool_head_stride_v + row_n * RV + CV * g) * 4);
#pragma unroll
      for (int k4 = 0; k4 < KK; ++k4)
        pg.k[hh][k4] = __builtin_nontemporal_load((const u32x4 *)(kpage + koff + ((RK / 4) * g + 4 * k4) * 4));
#pragma unroll
      for (int kv = 0; kv < KV; ++kv)
        pg.v[hh][kv] = __builtin_nontemporal_load((const u32x4 *)(vpage + voff + kv * 16));
    }
  };

  // An invalid page-table entry was replaced by page 0 at load time; its
  // tokens are masked out here (no branch, so every path waits the same way)
  // and the row is poisoned through the error bits.
  auto compute_page = [&](const Page &cur, int lp) {
    errbits |= cur.ok ? 0 : LLA_DEVERR_PAGE;
    const bool valid = cur.ok && n <= cur.last && lp < lp1;  // lp >= lp1: ring padding
    const int row_n = min(n, cur.last);
    const char *tb = s_trig + (((lp - lp0) / CH) & 1) * TSB * 16 +
                     (((lp - lp0) % CH) * kPage + row_n) * SPR * 16;
    // cos / sin of this lane's 16 pair indices 16 t + 4 g + e at its token
    float tc[NT][4], ts[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int ls = 8 * t + 2 * g;
      const f32x4 c0 = *(const f32x4 *)(tb + ((ls ^ (row_n & SWZ)) * 16));
      const f32x4 c1 = *(const f32x4 *)(tb + (((ls + 1) ^ (row_n & SWZ)) * 16));
      tc[t][0] = c0[0]; ts[t][0] = c0[1]; tc[t][1] = c0[2]; ts[t][1] = c0[3];
      tc[t][2] = c1[0]; ts[t][2] = c1[1]; tc[t][3] = c1[2]; ts[t][3] = c1[3];
    }
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      float bk[KS];
#pragma unroll
      for (int ks = 0; ks < RK / 4; ++ks) bk[ks] = __uint_as_float(cur.k[hh][ks / 4][ks % 4]);
      bk[RK / 4] = (g == 0) ? 1.f : 0.f;
      // X / Y tiles: rows = pair indices 16t + 4g + e, column = token n
      float sc0 = 0.f, sc1 = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4 X = {0.f, 0.f, 0.f, 0.f}, Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          X = __builtin_amdgcn_mfma_f32_16x16x4f32(A[hh][t][0][ks], bk[ks], X, 0, 0, 0);
          Y = __builtin_amdgcn_mfma_f32_16x16x4f32(A[hh][t][1][ks], bk[ks], Y, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc0 = fmaf(tc[t][e], X[e], sc0);
          sc1 = fmaf(ts[t][e], Y[e], sc1);
        }
      }
      float sc = sum_across_rows(sc0 + sc1);
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
        for (int e = 0; e < 4; ++e)
          acc[hh][4 * kv + e] = fmaf(p, __uint_as_float(cur.v[hh][kv][e]), acc[hh][4 * kv + e]);
      }
    }
  };

  // Ring of NBUF page slots: while page p is computed, pages p+1 .. p+LOOK are
  // in flight.  A slot is refilled LOOK steps after it was computed (NBUF =
  // LOOK + 2), so the old and new contents of a slot never overlap.  Every trip
  // computes exactly NBUF pages (pages past the split's end are masked) and
  // every load is issued unconditionally (clamped to the split's last page);
  // the next RoPE chunk is published at the end of the trip.
  if (lp0 < lp1) {
    const int lp_end = lp0 + (lp1 - lp0 + NBUF - 1) / NBUF * NBUF;
    Page ring[NBUF];
    stage_load(0);
#pragma unroll
    for (int u = 0; u < LOOK; ++u) {
      const int l = min(lp0 + u, lp1 - 1);
      load_page(l, page_at(l), ring[u]);
    }
    stage_store(0);
    __syncthreads();
    stage_load(1);
    for (int lp = lp0; lp < lp_end; lp += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int l = min(lp + u + LOOK, lp1 - 1);
        load_page(l, page_at(l), ring[(u + LOOK) % NBUF]);
        compute_page(ring[u], lp + u);
      }
      const int c = (lp - lp0) / CH;  // chunk just computed
      stage_store(c + 1);             // buffer of chunk c-1: every wave is past it
      __syncthreads();
      stage_load(c + 2);              // past the split's end: clamped rows, unused
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

  float *mine = (float *)(s_pt + a.pages_per_split) + (wave * HPW) * (RV + 2);  // [waves][HPW][RV + 2]
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
    const float *w = (const float *)a.wup_v + (long long)h * a.wup_head_stride_v;
    const float *mu = (const float *)a.mu_v + (long long)h * a.mu_head_stride;
    const float *an = mine + hh * (RV + 2);
    for (int e = lane; e < DH; e += 64) {
      float o = mu[e];
      const float *we = w + (long long)e * RV;
#pragma unroll
      for (int r4 = 0; r4 < RV / 4; ++r4) {
        const f32x4 v = *(const f32x4 *)(we + 4 * r4);
#pragma unroll
        for (int k = 0; k < 4; ++k) o = fmaf(v[k], an[4 * r4 + k], o);
      }
      ((float *)a.out)[((long long)row * a.H + h) * DH + e] = o;
    }
  }
}

// ---------------------------------------------------------------- dispatch

namespace {
template <int DH, int RK, int RV, int HPW, int NW>
hipError_t go(const AttnArgs &a, hipStream_t stream) {
  const hipError_t e = raise_lds_limit<decode_ph_kernel<DH, RK, RV, HPW, NW>>();  // more than the default 64 KiB
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(a.rows * a.head_groups * a.splits));
  const dim3 block((unsigned)(64 * NW));
  constexpr int TS = (LLA_DECODE_LOOK + 2) * kPage * (DH / 4);  // one chunk = ring
  constexpr int TSB = (TS + 64 * NW - 1) / (64 * NW) * (64 * NW);
  const size_t shmem = 2 * (size_t)TSB * 16 + sizeof(int) * a.pages_per_split +
                       sizeof(float) * NW * HPW * (RV + 2);
  hipLaunchKernelGGL((decode_ph_kernel<DH, RK, RV, HPW, NW>), grid, block, shmem, stream, a);
  return hipGetLastError();
}
}  // namespace

// fp32 storage: (d_head, r_k, r_v, heads per wave, waves per workgroup)
#define LLA_DECODE_F32_SHAPES(X) \
  X(64, 16, 32, 1, 2)            \
  X(64, 16, 32, 1, 8)            \
  X(128, 16, 32, 1, 2)           \
  X(128, 16, 32, 1, 8)           \
  X(128, 96, 160, 1, 8)

bool decode_supported(int dtype, int d_head, int r_k, int r_v, int hpw, int waves) {
  if (dtype == LLA_BF16) return decode_g_supported(d_head, r_k, r_v, hpw, waves);
#define X(DH, RK, RV, HPW, NW) \
  if (d_head == DH && r_k == RK && r_v == RV && hpw == HPW && waves == NW) return true;
  LLA_DECODE_F32_SHAPES(X)
#undef X
  return false;
}

hipError_t launch_decode(int dtype, int d_head, int r_k, int r_v, const AttnArgs &a,
                         hipStream_t stream) {
  if (dtype == LLA_BF16) return launch_decode_g(d_head, r_k, r_v, a, stream);
#define X(DH, RK, RV, HPW, NW)                                                                \
  if (d_head == DH && r_k == RK && r_v == RV && a.heads_per_wave == HPW && a.waves == NW) \
    return go<DH, RK, RV, HPW, NW>(a, stream);
  LLA_DECODE_F32_SHAPES(X)
#undef X
  return hipErrorInvalidConfiguration;
}

}  // namespace lla
