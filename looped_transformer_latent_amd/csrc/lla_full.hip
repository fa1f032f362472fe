// Full ("teacher") K/V cache for one (layer, loop), bf16 per-head: the baseline
// the latent path is measured against (cc.laoqi.cc close reading, 四:结果 item 9:
// the full-memory fast path keeps complete reconstructed K/V; the capacity
// path rebuilds from latents at read time).
//
//  * reconstruct_kernel: k_j = R(j)(mu_k,t + c_k,j W_up,k,t^T) and
//    v_j = mu_v,t + c_v,j W_up,v,t^T (eq. (3), RoPE after reconstruction) for
//    every cached token, written in bf16 to a paged full cache with the latent
//    cache's page table ([num_pages][H][16][d_head]).  One wave rebuilds 16
//    consecutive pages of one head, one page at a time on the matrix cores:
//    W_up rows are the A-operand (registers), the page's latent rows the
//    B-operand, so the accumulator holds 4 consecutive dims of one token and
//    both halves of each RoPE pair in one lane.  The bf16 page tile goes
//    through LDS and leaves in 1 KiB-contiguous stores (the write stream is
//    most of the traffic).
//  * full_decode_kernel: ordinary decode attention over the full cache,
//    s_j = scale <R(q_pos) q, k_j>, out = sum_j e^{s_j - m} v_j / sum_j e^{s_j - m}.
//    Bound by HBM (2 d_head bf16 per token and head).  One wave per (row,
//    head, split); every load instruction reads 1 KiB of a page contiguously
//    (lane l: bytes 16 l .. + 15), so a lane holds 8 dims of d_head / 16
//    tokens; scores reduce within the token's lanes (DPP), the value sum per
//    lane at the end.  Pages are loaded four ahead; online softmax in base 2
//    with the running max moved only when it grows by more than 8.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {

namespace {

typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));

__device__ __forceinline__ uint32_t cvt2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// dst rows d = 16 T + 4 g + i (i < 4), column t = lane & 15, of W_up[d][r] c[t][r]^T:
// RK / 32 steps of 16x16x32 plus one 16x16x16 step when RK % 32 == 16.
template <int RK>
struct WupTile {
  u32x4 a32[RK / 32 > 0 ? RK / 32 : 1];
  u32x2 a16;
};

template <int RK>
__device__ __forceinline__ void load_wup(WupTile<RK> &w, const uint16_t *row, int g) {
#pragma unroll
  for (int ks = 0; ks < RK / 32; ++ks) w.a32[ks] = *(const u32x4 *)(row + 32 * ks + 8 * g);
  if constexpr (RK % 32) w.a16 = *(const u32x2 *)(row + 32 * (RK / 32) + 4 * g);
}

// The B-operand: this lane's token row of the latent page, same K slots.
template <int RK>
using LatRow = WupTile<RK>;

template <int RK>
__device__ __forceinline__ f32x4 wup_times(const WupTile<RK> &w, const LatRow<RK> &b) {
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < RK / 32; ++ks)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w.a32[ks]), as_bf16x8(b.a32[ks]), acc, 0, 0, 0);
  if constexpr (RK % 32)
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, w.a16),
                                                     __builtin_bit_cast(bf16x4, b.a16), acc, 0, 0, 0);
  return acc;
}

// The same product with the W_up rows read from LDS (row stride R + 8
// elements): for ranks whose decoder does not fit in registers.
template <int RK>
__device__ __forceinline__ f32x4 wup_times_lds(const uint16_t *w_row, const LatRow<RK> &b, int g) {
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < RK / 32; ++ks)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(*(const u32x4 *)(w_row + 32 * ks + 8 * g)),
                                                  as_bf16x8(b.a32[ks]), acc, 0, 0, 0);
  if constexpr (RK % 32)
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
        __builtin_bit_cast(bf16x4, *(const u32x2 *)(w_row + 32 * (RK / 32) + 4 * g)),
        __builtin_bit_cast(bf16x4, b.a16), acc, 0, 0, 0);
  return acc;
}

}  // namespace

// ---------------------------------------------------------------- reconstruct

// Grid: x = batch * ceil(max pages / (NW * PPW)), y = H; NW waves, each PPW
// pages.  WLDS: W_up,k and W_up,v of the head are staged in LDS (shared by the
// workgroup's waves) instead of registers, for ranks whose decoder does not fit.
template <int DH, int RK, int RV, bool WLDS, int NW>
__global__ __launch_bounds__(64 * NW) void reconstruct_kernel(AttnArgs a, char *k_full, char *v_full, int ppw) {
  constexpr int NDT = DH / 16, HALF = DH / 2;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int groups = (a.pages_per_split + NW * ppw - 1) / (NW * ppw);  // pages_per_split: pages a row can need
  const int b = blockIdx.x / groups, grp = blockIdx.x - b * groups;
  const int h = blockIdx.y;
  int ctx = a.ctx_len[b];
  if (ctx < 1 || ctx > a.max_ctx) {
    if (grp == 0 && threadIdx.x == 0 && h == 0) atomicOr(a.err, LLA_DEVERR_CTX);
    return;
  }
  const int npg = (ctx + kPage - 1) / kPage;
  const int lp0 = (grp * NW + w) * ppw;

  // W_up,k rows 16 T + n (T < NDT), W_up,v rows likewise; mu per output row
  const uint16_t *wk = (const uint16_t *)a.wup_k + (long long)h * a.wup_head_stride_k;
  const uint16_t *wv = (const uint16_t *)a.wup_v + (long long)h * a.wup_head_stride_v;
  const uint16_t *mk = (const uint16_t *)a.mu_k + (long long)h * a.mu_head_stride;
  const uint16_t *mv = (const uint16_t *)a.mu_v + (long long)h * a.mu_head_stride;
  constexpr int WKR = RK + 8, WVR = RV + 8;  // LDS row strides of the staged decoder
  __shared__ __align__(16) uint16_t s_w[WLDS ? DH * (WKR + WVR) : 8];
  WupTile<RK> ak[WLDS ? 1 : NDT];
  WupTile<RV> av[WLDS ? 1 : NDT];
  if constexpr (WLDS) {
    for (int i = threadIdx.x; i < DH * RK / 8; i += 64 * NW)
      *(u32x4 *)(s_w + (i / (RK / 8)) * WKR + 8 * (i % (RK / 8))) = *(const u32x4 *)(wk + 8 * i);
    for (int i = threadIdx.x; i < DH * RV / 8; i += 64 * NW)
      *(u32x4 *)(s_w + DH * WKR + (i / (RV / 8)) * WVR + 8 * (i % (RV / 8))) = *(const u32x4 *)(wv + 8 * i);
    __syncthreads();
  } else {
#pragma unroll
    for (int T = 0; T < NDT; ++T) {
      load_wup<RK>(ak[T], wk + (16 * T + n) * RK, g);
      load_wup<RV>(av[T], wv + (16 * T + n) * RV, g);
    }
  }
  if (lp0 >= npg) return;  // whole wave, after the workgroup's only barrier
  // RoPE of token 16 lp + n by angle addition: the page's first position is
  // one table row shared by every lane (a broadcast read), the offset n is
  // fixed per lane (fp32 products of two table rotations)
  f32x4 rd[NDT / 2][2];
  {
    const float *r0 = a.rope + (long long)min(n, a.rope_len - 1) * DH;
#pragma unroll
    for (int T = 0; T < NDT / 2; ++T) {
      rd[T][0] = *(const f32x4 *)(r0 + 2 * (16 * T + 4 * g));
      rd[T][1] = *(const f32x4 *)(r0 + 2 * (16 * T + 4 * g) + 4);
    }
  }
  const long long ls = (long long)kPage * DH;  // elements per (page, head)
  // each wave's page tile of K and of V is staged in LDS, so that it leaves in
  // 1 KiB-contiguous stores (16-byte pad per row)
  constexpr int SROW = DH + 8;
  __shared__ __align__(16) uint16_t s_stage[NW][2][kPage * SROW];
  uint16_t *sk = s_stage[w][0], *sv = s_stage[w][1];
  int bad = 0;
  // latent rows of page lp (lane n: token n of the page), one page ahead
  const int lp_end = min(lp0 + ppw, npg);
  // mu_k, mu_v at this lane's output dims, read once (bf16 pairs)
  u32x2 mk2[NDT / 2][2], mv2[NDT];
#pragma unroll
  for (int T = 0; T < NDT / 2; ++T) {
    mk2[T][0] = *(const u32x2 *)(mk + 16 * T + 4 * g);
    mk2[T][1] = *(const u32x2 *)(mk + 16 * T + 4 * g + HALF);
  }
#pragma unroll
  for (int T = 0; T < NDT; ++T) mv2[T] = *(const u32x2 *)(mv + 16 * T + 4 * g);
  // the wave's page-table entries, one per lane, read once (lane i: page lp0 + i)
  const int pt_lane = lane < lp_end - lp0 ? a.page_table[(long long)b * a.max_pages + lp0 + lane] : 0;
  auto page_of = [&](int lp) { return __builtin_amdgcn_readlane(pt_lane, lp - lp0); };
  auto fetch = [&](int e, LatRow<RK> &rk, LatRow<RV> &rv) {
    const long long pe = e >= 0 && e < a.num_pages ? e : 0;
    load_wup<RK>(rk, (const uint16_t *)a.k_pool + pe * a.pool_page_stride_k + (long long)h * a.pool_head_stride_k + n * RK, g);
    load_wup<RV>(rv, (const uint16_t *)a.v_pool + pe * a.pool_page_stride_v + (long long)h * a.pool_head_stride_v + n * RV, g);
  };
  LatRow<RK> ck, ck_n;
  LatRow<RV> cv, cv_n;
  // RoPE of the page's first position for this lane's pairs, one page ahead
  f32x4 rb4[NDT / 2][2], rb4_n[NDT / 2][2];
  auto fetch_rope = [&](int lp, f32x4 (&dst)[NDT / 2][2]) {
    const float *rr = a.rope + (long long)(lp * kPage) * DH;
#pragma unroll
    for (int T = 0; T < NDT / 2; ++T) {
      dst[T][0] = *(const f32x4 *)(rr + 2 * (16 * T + 4 * g));
      dst[T][1] = *(const f32x4 *)(rr + 2 * (16 * T + 4 * g) + 4);
    }
  };
  int e = page_of(lp0);
  fetch(e, ck, cv);
  fetch_rope(lp0, rb4);
  for (int lp = lp0; lp < lp_end; ++lp) {
    const int e_n = lp + 1 < lp_end ? page_of(lp + 1) : e;
    if (lp + 1 < lp_end) {
      fetch(e_n, ck_n, cv_n);
      fetch_rope(lp + 1, rb4_n);
    }
    if (e < 0 || e >= a.num_pages) {  // uniform over the wave
      bad |= LLA_DEVERR_PAGE;
    } else {
      uint16_t *kd = (uint16_t *)k_full + ((long long)e * a.H + h) * ls;
      uint16_t *vd = (uint16_t *)v_full + ((long long)e * a.H + h) * ls;
#pragma unroll
      for (int T = 0; T < NDT / 2; ++T) {
        f32x4 x, y;
        if constexpr (WLDS) {
          x = wup_times_lds<RK>(s_w + (16 * T + n) * WKR, ck, g);
          y = wup_times_lds<RK>(s_w + (16 * (T + NDT / 2) + n) * WKR, ck, g);
        } else {
          x = wup_times<RK>(ak[T], ck);
          y = wup_times<RK>(ak[T + NDT / 2], ck);
        }
        const int d0 = 16 * T + 4 * g;  // RoPE pairs d0 .. d0 + 3
        const f32x4 c01 = rb4[T][0], c23 = rb4[T][1];
        float ra[4], rb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ka = x[i] + (i & 1 ? bf16_hi(mk2[T][0][i >> 1]) : bf16_lo(mk2[T][0][i >> 1]));
          const float kb = y[i] + (i & 1 ? bf16_hi(mk2[T][1][i >> 1]) : bf16_lo(mk2[T][1][i >> 1]));
          const f32x4 &cq = i < 2 ? c01 : c23;
          const float cb = cq[2 * (i & 1)], sb = cq[2 * (i & 1) + 1];
          const float cd = rd[T][i >> 1][2 * (i & 1)], sd = rd[T][i >> 1][2 * (i & 1) + 1];
          const float c = cb * cd - sb * sd, s = sb * cd + cb * sd;
          ra[i] = ka * c - kb * s;
          rb[i] = ka * s + kb * c;
        }
        *(u32x2 *)(sk + n * SROW + d0) = u32x2{cvt2(ra[0], ra[1]), cvt2(ra[2], ra[3])};
        *(u32x2 *)(sk + n * SROW + d0 + HALF) = u32x2{cvt2(rb[0], rb[1]), cvt2(rb[2], rb[3])};
      }
#pragma unroll
      for (int T = 0; T < NDT; ++T) {
        f32x4 x;
        if constexpr (WLDS) x = wup_times_lds<RV>(s_w + DH * WKR + (16 * T + n) * WVR, cv, g);
        else x = wup_times<RV>(av[T], cv);
        const int d0 = 16 * T + 4 * g;
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = x[i] + (i & 1 ? bf16_hi(mv2[T][i >> 1]) : bf16_lo(mv2[T][i >> 1]));
        *(u32x2 *)(sv + n * SROW + d0) = u32x2{cvt2(o[0], o[1]), cvt2(o[2], o[3])};
      }
      // store j, lane l: elements 512 j + 8 l .. + 7 of the tile, i.e. token
      // (512 j + 8 l) / DH; slots of tokens at or past ctx_len stay untouched
      // (the stage is wave-private and LDS accesses of one wave stay in order)
#pragma unroll
      for (int j = 0; j < kPage * DH / 512; ++j) {
        const int el = 512 * j + 8 * lane, t = el / DH, c = el % DH;
        const u32x4 kv = *(const u32x4 *)(sk + t * SROW + c);
        const u32x4 vv = *(const u32x4 *)(sv + t * SROW + c);
        if (lp * kPage + t < ctx) {
          __builtin_nontemporal_store(kv, (u32x4 *)(kd + el));
          __builtin_nontemporal_store(vv, (u32x4 *)(vd + el));
        }
      }
    }
    e = e_n;
    ck = ck_n;
    cv = cv_n;
#pragma unroll
    for (int T = 0; T < NDT / 2; ++T) {
      rb4[T][0] = rb4_n[T][0];
      rb4[T][1] = rb4_n[T][1];
    }
  }
  if (bad && lane == 0) atomicOr(a.err, bad);
}

// ---------------------------------------------------------------- full-cache decode

template <int DH>
__global__ __launch_bounds__(256, 2) void full_decode_kernel(AttnArgs a) {
  constexpr int NW = 4;              // heads per workgroup
  constexpr int LPR = DH / 8;        // lanes per token row (8 dims = 16 bytes each)
  constexpr int TPL = 16 * LPR / 64; // tokens per lane per page (one per 16-byte load)
  constexpr int RPW = 64 / LPR;      // token rows covered by one load instruction
  constexpr int HALF = DH / 2;
  constexpr int LOOK = 4, NB = LOOK + 1;  // pages in flight beyond the one computed
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // load j of a page reads bytes 1024 j + 16 lane: token RPW j + lane / LPR,
  // dims 8 (lane % LPR) .. + 7
  const int tr = lane / LPR, d0 = 8 * (lane % LPR);

  int bid = blockIdx.x;
  const int split = bid % a.splits;
  bid /= a.splits;
  const int hg = bid % a.head_groups;
  const int row = bid / a.head_groups;
  const int h = hg * NW + w;
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

  // q' = scale log2(e) R(q_pos) q for dims d0 .. d0 + 7
  float qr[8];
  {
    const uint16_t *qrow = (const uint16_t *)a.q + ((long long)row * a.H + h) * DH;
    const float *rq = a.rope + (long long)qp * DH;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = d0 + e;
      const int i = d < HALF ? d : d - HALF;  // RoPE pair
      const float qa = bf16_to_f32(qrow[i]), qb = bf16_to_f32(qrow[i + HALF]);
      const float c = rq[2 * i], s = rq[2 * i + 1];
      qr[e] = a.qscale * (d < HALF ? qa * c - qb * s : qa * s + qb * c);
    }
  }

  const int *pt_row = a.page_table + (long long)row * a.max_pages;
  const long long ls = (long long)kPage * DH;
  auto load = [&](int lp, u32x4 (&kq)[TPL], u32x4 (&vq)[TPL], int &ok) {
    const int e = pt_row[lp];
    ok = e >= 0 && e < a.num_pages;
    const long long off = ((long long)(ok ? e : 0) * a.H + h) * ls + 8 * lane;
    const uint16_t *kb = (const uint16_t *)a.k_pool + off;
    const uint16_t *vb = (const uint16_t *)a.v_pool + off;
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
      kq[j] = __builtin_nontemporal_load((const u32x4 *)(kb + 512 * j));
      vq[j] = __builtin_nontemporal_load((const u32x4 *)(vb + 512 * j));
    }
  };

  float m_ref = -INFINITY, z = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;

  // sum over the LPR lanes of a token row (LPR = 16: one DPP row; 8: half a row)
  auto row_sum = [&](float x) {
    x += dpp<kDppQuadSwap1>(x);
    x += dpp<kDppQuadSwap2>(x);
    x += dpp<kDppHalfMirror>(x);
    if constexpr (LPR == 16) x += dpp<kDppMirror>(x);
    return x;
  };

  auto compute = [&](int lp, const u32x4 (&kq)[TPL], const u32x4 (&vq)[TPL], int ok) {
    if (!ok) errbits |= LLA_DEVERR_PAGE;
    float s[TPL];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
      float x = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x = fmaf(qr[2 * e], bf16_lo(kq[j][e]), x);
        x = fmaf(qr[2 * e + 1], bf16_hi(kq[j][e]), x);
      }
      x = row_sum(x);
      // rows past ctx_len (last page) and rows of a bad page take no weight
      if (!ok || lp * kPage + RPW * j + tr >= ctx) x = -INFINITY;
      s[j] = x;
      mx = fmaxf(mx, x);
    }
    // the page's max: over this lane's tokens, then over the other token rows
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if constexpr (LPR == 8) mx = fmaxf(mx, __shfl_xor(mx, 8));
    if (mx > m_ref + 8.f) {  // uniform: mx is the wave's max
      const float al = m_ref == -INFINITY ? 0.f : fast_exp2(m_ref - mx);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= al;
      z *= al;
      m_ref = mx;
    }
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
      const float p = m_ref == -INFINITY ? 0.f : fast_exp2(s[j] - m_ref);
      z += p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(p, bf16_lo(vq[j][e]), acc[2 * e]);
        acc[2 * e + 1] = fmaf(p, bf16_hi(vq[j][e]), acc[2 * e + 1]);
      }
    }
  };

  u32x4 kb[NB][TPL], vb[NB][TPL];
  int okb[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) okb[u] = 1;
  const int n = lp1 - lp0;
#pragma unroll
  for (int u = 0; u < LOOK; ++u)
    if (u < n) load(lp0 + u, kb[u], vb[u], okb[u]);
  for (int i = 0; i < n; i += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if (i + u < n) {
        if (i + u + LOOK < n) load(lp0 + i + u + LOOK, kb[(u + LOOK) % NB], vb[(u + LOOK) % NB], okb[(u + LOOK) % NB]);
        compute(lp0 + i + u, kb[u], vb[u], okb[u]);
      }
    }
  }

  // z: every lane of a token row added that token's weight, so the wave sum
  // counts each token LPR times; acc sums over this lane's tokens only
  for (int o = 1; o < 64; o <<= 1) z += __shfl_xor(z, o);
  z *= 1.f / LPR;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    for (int o = LPR; o < 64; o <<= 1) acc[e] += __shfl_xor(acc[e], o);  // over the token rows
  if (errbits) atomicOr(a.err, errbits);
  const bool bad = __syncthreads_or(errbits != 0);
  if (a.splits > 1) {
    float *part_p = a.partials + (((long long)row * a.H + h) * a.splits + split) * (DH + 2);
    if (tr == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) part_p[d0 + e] = acc[e];
    }
    if (lane == 0) {
      part_p[DH] = m_ref;
      part_p[DH + 1] = bad ? __builtin_nanf("") : z;
    }
    return;
  }
  if (tr == 0) {
    const float inv = bad ? __builtin_nanf("") : 1.f / z;
    uint16_t *orow = (uint16_t *)a.out + ((long long)row * a.H + h) * DH + d0;
    *(u32x4 *)orow = u32x4{cvt2(acc[0] * inv, acc[1] * inv), cvt2(acc[2] * inv, acc[3] * inv),
                           cvt2(acc[4] * inv, acc[5] * inv), cvt2(acc[6] * inv, acc[7] * inv)};
  }
}

// ---------------------------------------------------------------- dispatch

// (d_head, r_k, r_v, decoder in LDS, waves per workgroup)
#define LLA_RECON_SHAPES(X)      \
  X(64, 16, 32, false, 4)        \
  X(128, 16, 32, false, 4)       \
  X(128, 32, 64, false, 4)       \
  X(128, 64, 64, false, 4)       \
  X(128, 96, 160, true, 8)

bool reconstruct_supported(int dtype, int variant, int d_head, int r_k, int r_v) {
  if (dtype != LLA_BF16 || variant != LLA_PER_HEAD) return false;
#define X(DH, RK, RV, WL, NW) \
  if (d_head == DH && r_k == RK && r_v == RV) return true;
  LLA_RECON_SHAPES(X)
#undef X
  return false;
}

hipError_t launch_reconstruct(int d_head, int r_k, int r_v, const AttnArgs &a, void *k_full, void *v_full,
                              int batch, hipStream_t stream) {
  const int ppw = 16;
#define X(DH, RK, RV, WL, NW)                                                                           \
  if (d_head == DH && r_k == RK && r_v == RV) {                                                         \
    const long long gx = (long long)batch * ((a.pages_per_split + NW * ppw - 1) / (NW * ppw));          \
    if (gx > 0x7FFFFFFF || a.H > 65535) return hipErrorInvalidConfiguration;                            \
    hipLaunchKernelGGL((reconstruct_kernel<DH, RK, RV, WL, NW>), dim3((unsigned)gx, (unsigned)a.H),     \
                       dim3(64 * NW), 0, stream, a, (char *)k_full, (char *)v_full, ppw);              \
    return hipGetLastError();                                                                           \
  }
  LLA_RECON_SHAPES(X)
#undef X
  return hipErrorInvalidConfiguration;
}

bool full_decode_supported(int dtype, int variant, int d_head) {
  return dtype == LLA_BF16 && variant == LLA_PER_HEAD && (d_head == 64 || d_head == 128);
}

hipError_t launch_full_decode(int d_head, const AttnArgs &a, hipStream_t stream) {
  if (a.H % 4 || a.head_groups * 4 != a.H) return hipErrorInvalidConfiguration;
  const long long grid = (long long)a.rows * a.head_groups * a.splits;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (d_head == 128)
    hipLaunchKernelGGL(full_decode_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else if (d_head == 64)
    hipLaunchKernelGGL(full_decode_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else
    return hipErrorInvalidConfiguration;
  return hipGetLastError();
}

}  // namespace lla
