// Per-head LLA decode attention for bf16 storage, with the RoPE weighting on
// the matrix cores (gfx950, wave64).
//
// What it computes is the same as the fp32 kernel (cc.laoqi.cc close reading,
// 方法 items 1-3; gist.science "Kernmechanismus"): for layer l, loop t and
// every (row, head),
//   s_j = scale <R(q_pos) q, R(j) (mu_k,t + c_k,j W_up,k,t^T)>,
//   out = mu_v,t + (sum_j e^{s_j - m} c_v,j) W_up,v,t^T / sum_j e^{s_j - m}.
//
// How.  With q' = scale log2(e) R(q_pos) q and RoPE pair i = (a, b) = (i, i + d/2),
//   s_j log2(e) = sum_i cos_i(j) (alpha_i + A_i . c_j) + sin_i(j) (beta_i + B_i . c_j)
// where A_ir = q'_a W[a][r] + q'_b W[b][r], B_ir = q'_b W[a][r] - q'_a W[b][r],
// alpha_i = q'_a mu_a + q'_b mu_b and beta_i = q'_b mu_a - q'_a mu_b (exact algebra:
// RoPE is linear in the reconstructed key).  Regrouping by latent column,
//   s_j log2(e) = sum_r c_j[r] G[r][j] + G0[j],
//   G[r][j]  = sum_i cos_i(j) A_ir + sin_i(j) B_ir,   G0[j] = sum_i cos_i(j) alpha_i + sin_i(j) beta_i.
// G is a product of the folded decoder F (r_k x d, cos / sin slots interleaved)
// with the RoPE rows of the page's 16 tokens (d x 16): one chain of fp16 MFMAs
// (v_mfma_f32_16x16x32_f16) per 16 latent columns, K = d.  The RoPE rows are
// already in LDS as fp16 (cos, sin) pairs, which is exactly the B-operand
// layout, and are shared by all heads of the wave; G0 for the wave's heads is
// one more MFMA chain with alpha / beta in rows 0 .. HPW-1.  What is left on the
// vector ALUs per (token, head) is r_k / 4 FMAs per lane plus the softmax and
// the latent-space value sum.
//
// fp16 keeps the decoder and cos / sin to 11 bits (bf16 has 8); products are
// exact and accumulate in fp32.
//
// Work decomposition, latent streaming (ring of NBUF pages per wave, LOOK in
// flight) and RoPE staging in LDS are as in the fp32 kernel.  With one split a
// workgroup normalises and up-projects its heads itself; with several it
// writes (m, Z, acc) partials for the merge launch (lla_merge.hip).
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {

typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// LDS layout of decode_g_kernel: the RoPE chunk buffers [2][TSB] x 16 B at 0;
// the split's page-table entries and the epilogue's [NW][HPW][RV + 2] floats
// after them; the W_up,k stage [NW][HPW][DH][RK] bf16 that the prologue folds
// from (and that wide latents reuse for the per-page transposition).  For
// r_k <= 32 the stage is dead once the fold is done, so it shares its bytes
// with the RoPE buffers: a workgroup then takes under half of a CU's LDS (the
// register count decides how many run per CU).
template <int DH, int RK, int RV, int HPW, int NW>
struct GLayout {
  static constexpr int TS = (LLA_DECODE_LOOK + 2) * kPage * (DH / 8);
  static constexpr int TSB = (TS + 64 * NW - 1) / (64 * NW) * (64 * NW);
  static constexpr size_t trig_bytes = 2 * (size_t)TSB * 16;
  static constexpr size_t w_bytes = sizeof(uint16_t) * NW * HPW * DH * RK;
  static constexpr size_t epi_bytes = sizeof(float) * NW * HPW * (RV + 2);
  static constexpr bool alias = RK <= 32;
  static constexpr size_t pt_off = alias && w_bytes > trig_bytes ? w_bytes : trig_bytes;
  __host__ __device__ static constexpr size_t epi_off(int pps) { return pt_off + sizeof(int) * (size_t)pps; }
  __host__ __device__ static constexpr size_t w_off(int pps) {
    return alias ? 0 : (epi_off(pps) + epi_bytes + 15) / 16 * 16;
  }
  __host__ __device__ static constexpr size_t total(int pps) {
    return alias ? epi_off(pps) + epi_bytes : w_off(pps) + w_bytes;
  }
};

// NW = 4 runs one wave per SIMD (up to 512 registers): the shape with the
// widest latents (r_k = 96, r_v = 160) needs them for its decoder and page ring.
template <int DH, int RK, int RV, int HPW, int NW>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 1 : 2) void decode_g_kernel(AttnArgs a) {
  constexpr int KS = DH / 32;   // K-steps: 16 RoPE pairs (32 cos / sin slots) each
  constexpr int RT = RK / 16;   // 16-column tiles of the latent
  constexpr int CV = RV / 4;    // V elements per lane per token
  constexpr int KV = CV / 8;    // 16-byte V loads per lane per head
  constexpr int HALF = DH / 2;
  static_assert(DH % 32 == 0 && RK % 16 == 0 && RV % 32 == 0 && HPW <= 4, "shape");

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
  // Retained tokens: [0, keep_lo) and [keep_hi, ctx) (token eviction), or the
  // whole context.  Splits run over the pages that hold retained tokens
  // ("virtual" pages v: the sink pages [0, n_a), then the window pages from
  // page p_b on); the other pages' table entries are never read.
  const RetainedPages rp = retained_pages(ctx, a.evict, a.n_sink, a.window);
  const int keep_lo = rp.keep_lo, keep_hi = rp.keep_hi, n_a = rp.n_a, p_b = rp.p_b, nvirt = rp.nvirt;
  auto logical = [&](int v) -> int { return v < n_a ? v : p_b + (v - n_a); };
  const int lp0 = split * a.pages_per_split;
  const int lp1 = min(lp0 + a.pages_per_split, nvirt);
  const int h0 = (hg * a.waves + wave) * HPW;

  // ---- prologue: folded decoder as fp16 MFMA A-operands ----
  // F[hh][rt][s]: lane (g, n) = row r = 16 rt + n, K-slots 2p, 2p + 1 = (A_ir, B_ir)
  // of pair i = 16 s + 4 g + p.  Fa[s]: row hh (lanes n == hh) = (alpha_i, beta_i).
  // The wave's W_up,k,t (HPW x d x r_k bf16) is first copied into its own LDS
  // region with 16-byte loads: the fold reads it by (pair, column), which as
  // global loads would be one 2-byte load per element and lane.  The RoPE row
  // of q_pos, q and mu_k are read 4 pairs per load.
  //
  // Range.  fp16 overflows above 65504 and loses bits below 2^-14, while q, mu
  // and W_up may be any bf16 values.  Per head, F and (alpha, beta) are packed
  // scaled by a power of two 2^e chosen so that their largest possible
  // magnitude lies in [2^14, 2^15): by Cauchy-Schwarz on a pair,
  // |A_ir|, |B_ir| <= |(q'_a, q'_b)| |(W[a][r], W[b][r])| <= qscale max_i |(q_a, q_b)| sqrt(2) max |W|,
  // and the same with mu for (alpha_i, beta_i).  The scores are multiplied by
  // 2^-e after the products (inside the exponent's argument); scaling by a
  // power of two commutes with every rounding in normal range, so nothing
  // else changes.
  extern __shared__ __attribute__((aligned(16))) char smem[];
  u32x4 F[HPW][RT][KS];
  u32x4 Fa[KS];
  float unscale[HPW];  // 2^-e per head (wave-uniform)
  {
    uint16_t *s_w = (uint16_t *)(smem + GLayout<DH, RK, RV, HPW, NW>::w_off(a.pages_per_split)) +
                    wave * (HPW * DH * RK);
    // Every global load of the prologue goes out first (one round trip instead
    // of one per stage): the wave's W_up,k rows, its q and mu_k pairs, and the
    // RoPE row of q_pos.
    constexpr int WC = DH * RK / 8 / 64;  // 16-byte pieces of a head's W_up,k per lane
    u32x4 wv[HPW][WC];
    u32x2 qa4[HPW][KS], qb4[HPW][KS], ma4[HPW][KS], mb4[HPW][KS];
    f32x4 cs01[KS], cs23[KS];
    const float *rq = a.rope + (long long)qp * DH;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = h0 + hh;
      const u32x4 *src = (const u32x4 *)((const uint16_t *)a.wup_k + (long long)h * a.wup_head_stride_k);
#pragma unroll
      for (int c = 0; c < WC; ++c) wv[hh][c] = src[c * 64 + lane];
      const uint16_t *qrow = (const uint16_t *)a.q + ((long long)row * a.H + h) * DH;
      const uint16_t *mu = (const uint16_t *)a.mu_k + (long long)h * a.mu_head_stride;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int i0 = 16 * s + 4 * g;  // pairs i0 .. i0 + 3 of this lane
        qa4[hh][s] = *(const u32x2 *)(qrow + i0);
        qb4[hh][s] = *(const u32x2 *)(qrow + i0 + HALF);
        ma4[hh][s] = *(const u32x2 *)(mu + i0);
        mb4[hh][s] = *(const u32x2 *)(mu + i0 + HALF);
      }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int i0 = 16 * s + 4 * g;
      cs01[s] = *(const f32x4 *)(rq + 2 * i0);
      cs23[s] = *(const f32x4 *)(rq + 2 * i0 + 4);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads above together
    uint32_t mag[HPW];  // largest |bf16| bit pattern of W_up,k and mu_k (magnitude order = integer order)
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      u32x4 *dst = (u32x4 *)(s_w + hh * DH * RK);
      mag[hh] = 0;
#pragma unroll
      for (int c = 0; c < WC; ++c) {
        dst[c * 64 + lane] = wv[hh][c];
#pragma unroll
        for (int k = 0; k < 4; ++k) mag[hh] = max(mag[hh], max(wv[hh][c][k] & 0x7FFFu, (wv[hh][c][k] >> 16) & 0x7FFFu));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float qscale_h[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      float qn2 = 0.f;  // largest |(q_a, q_b)|^2 of the lane's pairs
#pragma unroll
      for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float qa = p & 1 ? bf16_hi(qa4[hh][s][p >> 1]) : bf16_lo(qa4[hh][s][p >> 1]);
          const float qb = p & 1 ? bf16_hi(qb4[hh][s][p >> 1]) : bf16_lo(qb4[hh][s][p >> 1]);
          qn2 = fmaxf(qn2, qa * qa + qb * qb);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k)
          mag[hh] = max(mag[hh], max(max(ma4[hh][s][k] & 0x7FFFu, (ma4[hh][s][k] >> 16) & 0x7FFFu),
                                     max(mb4[hh][s][k] & 0x7FFFu, (mb4[hh][s][k] >> 16) & 0x7FFFu)));
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        qn2 = fmaxf(qn2, __shfl_xor(qn2, o));
        mag[hh] = max(mag[hh], (uint32_t)__shfl_xor((int)mag[hh], o));
      }
      const float bound = a.qscale * sqrtf(qn2) * 1.41421356f * bf16_to_f32(mag[hh]);
      // bound = f 2^k with f in [1, 2): e = 14 - k, clamped to normal fp32 powers
      int e = 14 - ((int)((__float_as_uint(bound) >> 23) & 0xFFu) - 127);
      e = min(max(e, -100), 100);
      e = __builtin_amdgcn_readfirstlane(e);
      qscale_h[hh] = a.qscale * __uint_as_float((uint32_t)(127 + e) << 23);
      unscale[hh] = __uint_as_float((uint32_t)(127 - e) << 23);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) Fa[s] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int i0 = 16 * s + 4 * g;  // pairs i0 .. i0 + 3 of this lane
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const uint16_t *w = s_w + hh * DH * RK;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int i = i0 + p;
          const f32x4 &cq = p < 2 ? cs01[s] : cs23[s];
          const float c = cq[2 * (p & 1)], sn = cq[2 * (p & 1) + 1];
          const float qa = p & 1 ? bf16_hi(qa4[hh][s][p >> 1]) : bf16_lo(qa4[hh][s][p >> 1]);
          const float qb = p & 1 ? bf16_hi(qb4[hh][s][p >> 1]) : bf16_lo(qb4[hh][s][p >> 1]);
          const float pa = qscale_h[hh] * (qa * c - qb * sn);
          const float pb = qscale_h[hh] * (qa * sn + qb * c);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const int r = 16 * rt + n;
            const float wa = bf16_to_f32(w[i * RK + r]);
            const float wb = bf16_to_f32(w[(i + HALF) * RK + r]);
            F[hh][rt][s][p] = pack_f16(pa * wa + pb * wb, pb * wa - pa * wb);
          }
          const float ma = p & 1 ? bf16_hi(ma4[hh][s][p >> 1]) : bf16_lo(ma4[hh][s][p >> 1]);
          const float mb = p & 1 ? bf16_hi(mb4[hh][s][p >> 1]) : bf16_lo(mb4[hh][s][p >> 1]);
          const uint32_t ab = pack_f16(pa * ma + pb * mb, pb * ma - pa * mb);
          if (n == hh) Fa[s][p] = ab;
        }
      }
    }
  }

  // m_run: running maximum of the raw (2^e-scaled) scores; nmu = -m_run 2^-e,
  // so that a token's weight is exp2(fma(score, 2^-e, nmu)).
  float m_run[HPW], nmu[HPW], z[HPW], acc[HPW][CV];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    m_run[hh] = -INFINITY;
    nmu[hh] = 0.f;
    z[hh] = 0.f;
#pragma unroll
    for (int k = 0; k < CV; ++k) acc[hh][k] = 0.f;
  }

  // Per page and head, lane (g, n) computes with latent row n: c_k columns
  // 16 rt + 4 g .. + 3 (8 bytes per tile) and c_v columns CV g .. CV g + CV - 1.
  // Rows past ctx_len (last page only) use the last valid row; their scores
  // are forced to -inf.
  //
  // Narrow latents (r_k <= 32) are loaded in that layout directly: a load
  // instruction then covers 512 or 1024 contiguous bytes.  For wider rows the
  // same layout would spread each instruction over 16 rows (one 8- or 16-byte
  // piece per row) and the address unit, not HBM, sets the pace.  XP: the
  // (page, head) block is loaded in address order instead (lane l: bytes
  // 8 l of each 512-byte K piece, 16 l of each 1 KiB V piece), written to the
  // wave's own LDS region with padded rows, and read back in the compute
  // layout.  The region is the wave's W_up,k stage of the prologue, which is
  // no longer used by then.
  constexpr bool XP = RK > 32;
  constexpr int SKP = RK + 8, SVP = RV + 8;  // padded LDS rows (elements): conflict-free reads
  static_assert(!XP || (HPW == 1 && RK % 4 == 0 && RV % 8 == 0 && (kPage * RK) % 256 == 0 &&
                        (kPage * RV) % 512 == 0 && kPage * (SKP + SVP) <= DH * RK),
                "transposed page layout");
  struct Page {
    u32x2 k[HPW][RT];
    u32x4 v[HPW][KV];
    int ok;
    int last;  // last valid row of this page (15 unless the page is the last one)
  };
  // LDS: [RoPE rows: 2 chunk buffers][page-table entries of the split][epilogue]
  constexpr int SPR = DH / 8;                  // 16-byte slots per position row (fp16 pairs)
  constexpr int SWZ = SPR < 16 ? SPR - 1 : 15;  // XOR swizzle mask (row index low bits)
  constexpr int LOOK = LLA_DECODE_LOOK;  // pages in flight beyond the one computed
  constexpr int NBUF = LOOK + 2;        // page ring slots
  constexpr int CH = NBUF;              // pages per RoPE chunk: one trip round the ring
  constexpr int TS = CH * kPage * SPR;  // 16-byte slots of one chunk
  constexpr int SLOTS = (TS + NTH - 1) / NTH;
  constexpr int TSB = SLOTS * NTH;
  char *s_trig = smem;  // (aliases the prologue's W_up,k stage at narrow ranks)
  int *s_pt = (int *)(smem + GLayout<DH, RK, RV, HPW, NW>::pt_off);
  static_assert(GLayout<DH, RK, RV, HPW, NW>::TSB == TSB, "layout");
  {
    const int *pt_row = a.page_table + (long long)b * a.max_pages;
    for (int i = threadIdx.x; i < lp1 - lp0; i += blockDim.x) s_pt[i] = pt_row[logical(lp0 + i)];
    __syncthreads();
  }
  auto page_at = [&](int lp) -> int { return __builtin_amdgcn_readfirstlane(s_pt[lp - lp0]); };

  // RoPE staging: chunk c covers (virtual) pages [lp0 + c CH, lp0 + (c + 1) CH);
  // row R of a chunk buffer holds the fp16 (cos, sin) pairs of position
  // 16 logical(lp0 + c CH + R / 16) + R % 16.
  // Logical slot ls (pairs 4 ls .. 4 ls + 3) is stored at ls ^ (R % 16 & SWZ) so
  // that 16 lanes reading one slot of 16 consecutive positions use distinct banks.
  const char *rope_b = (const char *)a.rope;
  f32x4 stg[SLOTS][2];
  auto stage_load = [&](int c) {
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      const int q = min((int)threadIdx.x + j * NTH, TS - 1);
      const int R = q / SPR, ps = q % SPR, rn = R % kPage;
      const int pos = min(logical(lp0 + c * CH + R / kPage) * kPage + rn, ctx - 1);
      const char *src = rope_b + (long long)pos * (DH * 4) + (ps ^ (rn & SWZ)) * 32;
      stg[j][0] = *(const f32x4 *)(src);
      stg[j][1] = *(const f32x4 *)(src + 16);
    }
  };
  auto stage_store = [&](int c) {
    char *dst = s_trig + (c & 1) * TSB * 16;
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      const int q = threadIdx.x + j * NTH;  // q >= TS lands in the buffer's padding
      u32x4 hv;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        hv[e] = pack_f16(stg[j][e >> 1][(e & 1) * 2], stg[j][e >> 1][(e & 1) * 2 + 1]);
      *(u32x4 *)(dst + q * 16) = hv;
    }
  };

  // Per-head pools: [page][H][kPage][r] with the heads kPage r elements apart.
  const uint32_t kpb = (uint32_t)a.pool_page_stride_k * 2u, vpb = (uint32_t)a.pool_page_stride_v * 2u;
  constexpr int KHB = kPage * RK * 2, VHB = kPage * RV * 2;  // bytes per (page, head)
  const uint32_t kwave = (uint32_t)(h0 * KHB), vwave = (uint32_t)(h0 * VHB);
  auto load_page = [&](int lp, int pp_raw, Page &pg) {
    pg.ok = (uint32_t)pp_raw < (uint32_t)a.num_pages;
    const uint32_t pp = pg.ok ? (uint32_t)pp_raw : 0u;
    pg.last = min(kPage - 1, ctx - 1 - logical(lp) * kPage);
    const int row_n = min(n, pg.last);
    // uniform page bases + 32-bit lane offsets; latents are read exactly once
    const char *kpage = a.k_pool + (uint64_t)pp * kpb;
    const char *vpage = a.v_pool + (uint64_t)pp * vpb;
    if constexpr (XP) {  // whole (page, head) block in address order
      const uint32_t koff = kwave + 8 * lane;
      const uint32_t voff = vwave + 16 * lane;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        pg.k[0][rt] = __builtin_nontemporal_load((const u32x2 *)(kpage + koff + 512 * rt));
#pragma unroll
      for (int kv = 0; kv < KV; ++kv)
        pg.v[0][kv] = __builtin_nontemporal_load((const u32x4 *)(vpage + voff + 1024 * kv));
      return;
    }
    const uint32_t koff = kwave + (uint32_t)((row_n * RK + 4 * g) * 2);
    const uint32_t voff = vwave + (uint32_t)((row_n * RV + CV * g) * 2);
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        pg.k[hh][rt] = __builtin_nontemporal_load((const u32x2 *)(kpage + koff + hh * KHB + 32 * rt));
#pragma unroll
      for (int kv = 0; kv < KV; ++kv)
        pg.v[hh][kv] = __builtin_nontemporal_load((const u32x4 *)(vpage + voff + hh * VHB + kv * 16));
    }
  };

  // An invalid page-table entry was replaced by page 0 at load time; its
  // tokens are masked out here and the row is poisoned through the error bits.
  // th_off[s]: the lane's 16-byte slot (pairs 16 s + 4 g .. + 3, token row n)
  // within a page's rows of a RoPE chunk buffer.
  uint32_t th_off[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) th_off[s] = (uint32_t)((n * SPR + ((4 * s + g) ^ (n & SWZ))) * 16);
  auto compute_page = [&](Page &cur, int lp, const char *trip_rope, int u) {
    errbits |= cur.ok ? 0 : LLA_DEVERR_PAGE;
    // Lane token lo + n takes part iff it is retained and below ctx; a bad
    // page or ring padding (lp >= lp1) takes no token.  Written with bitwise
    // operators so that it stays a lane mask (no branches).
    const int lo = logical(lp) * kPage;
    const bool pg_in = cur.ok && lp < lp1;
    const int la = pg_in ? keep_lo - lo : 0, lb = keep_hi - lo, lc = pg_in ? ctx - lo : 0;
    const bool valid = (n < la) | ((n >= lb) & (n < lc));
    const int row_n = min(n, cur.last);
    if constexpr (XP) {  // address order -> compute layout, through the wave's LDS region
      uint16_t *xb = (uint16_t *)(smem + GLayout<DH, RK, RV, HPW, NW>::w_off(a.pages_per_split)) +
                     wave * (HPW * DH * RK);
      uint16_t *xv = xb + kPage * SKP;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int e = 256 * rt + 4 * lane, r = e / RK;
        *(u32x2 *)(xb + r * SKP + (e - r * RK)) = cur.k[0][rt];
      }
#pragma unroll
      for (int kv = 0; kv < KV; ++kv) {
        const int e = 512 * kv + 8 * lane, r = e / RV;
        *(u32x4 *)(xv + r * SVP + (e - r * RV)) = cur.v[0][kv];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) cur.k[0][rt] = *(const u32x2 *)(xb + row_n * SKP + 16 * rt + 4 * g);
#pragma unroll
      for (int kv = 0; kv < KV; ++kv) cur.v[0][kv] = *(const u32x4 *)(xv + row_n * SVP + CV * g + 8 * kv);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // B-operands: RoPE pairs 16 s + 4 g .. + 3 of token n, (cos, sin) fp16.
    // Rows past ctx hold the RoPE row of ctx - 1 (the staging clamps), so
    // they stay finite; their scores are masked.
    u32x4 th[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) th[s] = *(const u32x4 *)(trip_rope + th_off[s] + u * (kPage * SPR * 16));
    // G0 of the wave's heads: rows 0 .. HPW-1 (lane (0, n) element hh)
    f32x4 Ga = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      Ga = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(Fa[s]), as_f16x8(th[s]), Ga, 0, 0, 0);
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      // score partial of lane (g, n): latent columns 16 rt + 4 g + e of token n
      float sc = g == 0 ? Ga[hh] : 0.f;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4 G = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
          G = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(F[hh][rt][s]), as_f16x8(th[s]), G, 0, 0, 0);
        sc = fmaf(bf16_lo(cur.k[hh][rt][0]), G[0], sc);
        sc = fmaf(bf16_hi(cur.k[hh][rt][0]), G[1], sc);
        sc = fmaf(bf16_lo(cur.k[hh][rt][1]), G[2], sc);
        sc = fmaf(bf16_hi(cur.k[hh][rt][1]), G[3], sc);
      }
      sc = sum_across_rows(sc);
      sc = valid ? sc : -INFINITY;
      // Raise the running maximum only when a token of the page exceeds it
      // (after the first pages, rarely): same maxima as a max per page.
      if (__builtin_amdgcn_ballot_w64(sc > m_run[hh]) != 0) {  // wave-uniform
        const float mt = max_in_row(sc);  // all four rows hold the same 16 scores
        const float corr = fast_exp2((m_run[hh] - mt) * unscale[hh]);
        z[hh] *= corr;
#pragma unroll
        for (int k = 0; k < CV; ++k) acc[hh][k] *= corr;
        m_run[hh] = mt;
        nmu[hh] = -mt * unscale[hh];
      }
      // a masked token (-inf) weighs 0, also before the first valid token
      const float p = fast_exp2(fmaf(sc, unscale[hh], nmu[hh]));
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

  // Ring of NBUF page slots: while page p is computed, pages p+1 .. p+LOOK are
  // in flight.  A slot is refilled LOOK steps after it was computed (NBUF =
  // LOOK + 2), so the old and new contents of a slot never overlap and no
  // register copies (which would wait for the loads in flight) are needed.
  // Every trip computes exactly NBUF pages (pages past the split's end are
  // masked) and every load is issued unconditionally (clamped to the split's
  // last page); the next RoPE chunk is published at the end of the trip.  Both
  // ways into the loop head thus leave the same loads outstanding, so the
  // compiler's waits keep the ring's loads in flight.
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
      int pid[NBUF];  // the trip's page-table entries, read together (one LDS wait per trip)
#pragma unroll
      for (int u = 0; u < NBUF; ++u) pid[u] = s_pt[min(lp + u + LOOK, lp1 - 1) - lp0];
#pragma unroll
      for (int u = 0; u < NBUF; ++u) pid[u] = __builtin_amdgcn_readfirstlane(pid[u]);
      const char *trip_rope = s_trig + (((lp - lp0) / CH) & 1) * TSB * 16;
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int l = min(lp + u + LOOK, lp1 - 1);
        load_page(l, pid[u], ring[(u + LOOK) % NBUF]);
        compute_page(ring[u], lp + u, trip_rope, u);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
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

  float *sh = (float *)(smem + GLayout<DH, RK, RV, HPW, NW>::epi_off(a.pages_per_split));  // [waves][HPW][RV + 2]
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
        part[RV] = m_run[hh] * unscale[hh];
        part[RV + 1] = bad ? __builtin_nanf("") : z[hh];
      }
    }
    return;
  } else {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const float zz = bad ? __builtin_nanf("") : z[hh];
      if (n == 0) {
#pragma unroll
        for (int k = 0; k < CV; ++k) mine[hh * (RV + 2) + CV * g + k] = acc[hh][k] / zz;
      }
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

// ---------------------------------------------------------------- dispatch

namespace {
template <int DH, int RK, int RV, int HPW, int NW>
hipError_t go_g(const AttnArgs &a, hipStream_t stream) {
  const hipError_t e = raise_lds_limit<decode_g_kernel<DH, RK, RV, HPW, NW>>();  // more than the default 64 KiB
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(a.rows * a.head_groups * a.splits));
  const dim3 block((unsigned)(64 * NW));
  const size_t shmem = GLayout<DH, RK, RV, HPW, NW>::total(a.pages_per_split);
  hipLaunchKernelGGL((decode_g_kernel<DH, RK, RV, HPW, NW>), grid, block, shmem, stream, a);
  return hipGetLastError();
}
}  // namespace

// (d_head, r_k, r_v, heads per wave, waves per workgroup)
#define LLA_DECODE_G_SHAPES(X) \
  X(64, 16, 32, 1, 2)          \
  X(64, 16, 32, 2, 8)          \
  X(128, 16, 32, 1, 2)         \
  X(128, 16, 32, 2, 2)         \
  X(128, 16, 32, 1, 8)         \
  X(128, 16, 32, 2, 8)         \
  X(128, 32, 64, 1, 8)         \
  X(128, 96, 160, 1, 4)

bool decode_g_supported(int d_head, int r_k, int r_v, int hpw, int waves) {
#define X(DH, RK, RV, HPW, NW) \
  if (d_head == DH && r_k == RK && r_v == RV && hpw == HPW && waves == NW) return true;
  LLA_DECODE_G_SHAPES(X)
#undef X
  return false;
}

hipError_t launch_decode_g(int d_head, int r_k, int r_v, const AttnArgs &a, hipStream_t stream) {
#define X(DH, RK, RV, HPW, NW)                                                                \
  if (d_head == DH && r_k == RK && r_v == RV && a.heads_per_wave == HPW && a.waves == NW) \
    return go_g<DH, RK, RV, HPW, NW>(a, stream);
  LLA_DECODE_G_SHAPES(X)
#undef X
  return hipErrorInvalidConfiguration;
}

}  // namespace lla
