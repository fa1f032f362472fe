// Causal prefill attention over the per-head latent cache, bf16 storage
// (gfx950, wave64): a query chunk at a time, on the matrix cores.
//
// What it computes (cc.laoqi.cc close reading, 方法 items 1, 3 and 6; gist.science
// "Technisches Resümee", eq. (3)): query i of sequence b sits at position
// p = p0[b] + i and attends over logical tokens j = 0..p of the cache,
//   k_hat_j = mu_k,t + c_k,j W_up,k,t^T, rotated by RoPE at position j,
//   s_ij    = scale <R(p) q_i, R(j) k_hat_j>,
//   out_i   = mu_v,t + (sum_j e^{s_ij - m_i} c_v,j) W_up,v,t^T / sum_j e^{s_ij - m_i}
// (V absorbed into latent space by linearity of eq. (3), as in decode).
//
// The decode kernels fold the query into the decoder, which costs d * r_k
// multiply-adds per token and query.  With a chunk of queries it is cheaper to
// rebuild each K tile once per workgroup (the close reading's long-prefill
// remark: rebuild per layer, keep nothing) and run a dense attention:
//  * A workgroup = 8 waves = 256 consecutive queries of one (sequence, head);
//    wave w owns 32 of them as two 16-query MFMA columns (two waves per SIMD).
//  * Keys go in 32-token tiles (two pages).  A tile's c_k and c_v rows are
//    copied global -> LDS with direct-to-LDS loads three tiles ahead, into one
//    of four slots (separate LDS objects, so that the compiler's waits stay
//    per slot; rows padded against bank conflicts).  Rows past the last needed
//    position, and rows of a page whose table entry is out of range, are
//    cleared to zero before use.  The page-table entries of the sequence are
//    staged in LDS, 1024 at a time.
//  * Rebuild, one tile ahead: every wave turns one 16-token x (16 + 16)-dim
//    block of the tile into rotated K (v_mfma_f32_16x16x32_bf16 with W_up,k rows
//    from LDS as the A-operand; mu and RoPE in fp32 on the accumulator, which
//    holds both halves of each RoPE pair in one lane) and stores it in bf16 to
//    a double-buffered LDS tile.
//  * S^T = K Q'^T per 16x16 block with Q' = scale log2(e) R(p) q in bf16
//    registers; each lane holds one query's column, so the online softmax
//    needs only two cross-row swaps for the max.  The running max is moved
//    only when a tile exceeds it by more than 8 (weights stay <= 2^8; the
//    result is the same), which skips most rescales of the accumulator.
//  * O^T[r][q] += C_v^T[r][t] P^T[t][q]: the bf16 weights come straight from
//    the score accumulator as the B-operand; the c_v tile is read transposed
//    with ds_read_b64_tr_b16 as the A-operand.
//  * One barrier per tile: each wave first waits for its own copies of the
//    tile the next step rebuilds, then all waves meet.
//  * Epilogue: O / Z in bf16 times W_up,v on the matrix cores, plus mu_v.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));

#define LLA_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// Two fp32 values to packed bf16 (hardware round to nearest even).
__device__ __forceinline__ uint32_t cvt2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float max_across_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const uint32_t v = __float_as_uint(y);
  const auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// Transposing LDS read: within each 16-lane group, lane i receives element i % 4
// of the 8-byte rows addressed by lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4.
__device__ __forceinline__ u32x2 lds_read_tr(const char *p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Workgroup barrier that leaves the newest VM loads of this wave in flight:
// wait until at most VM of them are outstanding and every LDS access is done,
// then meet.  The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
template <int VM>
__device__ __forceinline__ void barrier_vm() {
  static_assert(VM >= 0 && VM < 64, "vmcnt");
  // s_waitcnt: vmcnt bits [15:14] and [3:0], expcnt [6:4] (7 = no wait), lgkmcnt [11:8] = 0
  __builtin_amdgcn_s_waitcnt(((VM >> 4) << 14) | (VM & 15) | 0x70);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace

template <int DH, int RK, int RV>
__global__ __launch_bounds__(512, 1) void prefill_kernel(AttnArgs a) {
  constexpr int NW = 8, NTH = NW * 64, QB = NW * 32, KT = 32;  // queries per workgroup, tokens per tile
  constexpr int HALF = DH / 2, NDT = DH / 16, KSD = DH / 32;
  constexpr int NU = NDT;                          // rebuild units: 2 token halves x NDT / 2 tile pairs
  constexpr int KS32 = RK / 32;
  constexpr bool TAIL = (RK % 32) != 0;            // one extra 16-wide K-step
  constexpr int NRT = RV / 16, KSV = RV / 32;
  // LDS rows of a slot, in 16-byte chunks: RK / 8 (+1 pad) for c_k, RV / 8 (+2 pad) for c_v
  constexpr int CPK = RK / 8 + 1, CPV = RV / 8 + 2;
  constexpr int SK = 16 * CPK, SV = 16 * CPV, SKH = 2 * DH + 16;  // row strides, bytes
  constexpr int VOFF = KT * SK;
  constexpr int NPOS = (KT * (CPK + CPV) + 63) / 64 * 64;  // copied chunks per tile (pad included)
  constexpr int NCP = NPOS / 64;                            // wave-wide copies per tile
  constexpr int IPW = (NCP + NW - 1) / NW;                  // copies per wave (the last ones partial)
  constexpr int IPW_MIN = NCP / NW;                         // copies every wave issues
  constexpr int SLOT = NPOS * 16;
  static_assert(RK % 16 == 0 && RV % 32 == 0 && (DH == 64 || DH == 128), "shape");
  static_assert(NU <= NW && IPW <= 4, "tile split");

  __shared__ __attribute__((aligned(16))) char s_c0[SLOT], s_c1[SLOT], s_c2[SLOT], s_c3[SLOT];
  __shared__ __attribute__((aligned(16))) char s_kh0[KT * SKH], s_kh1[KT * SKH];  // rotated K, bf16
  __shared__ __attribute__((aligned(16))) char s_wk[DH * SK];                      // W_up,k,t rows
  __shared__ int s_pt[2][1024];  // page-table entries: chunk c (1024 logical pages) in s_pt[c % 2]

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;

  // ---- work item: (sequence, head, query block); the query blocks of one
  // (sequence, head) are dispatched to one XCD so that they share its L2 ----
  const int nq = a.n_q;
  const int nqb = (nq + QB - 1) / QB;
  const int batch = a.rows / nq;
  const long long nblk = (long long)batch * a.H * nqb;
  long long L = blockIdx.x;
  if ((nblk & 7) == 0) L = (L & 7) * (nblk >> 3) + (L >> 3);
  const int qb = (int)(L % nqb);
  const long long bh = L / nqb;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);

  // Valid rows are [lo, hi): position >= 0, context <= max_ctx, position inside
  // the RoPE table.  Other rows are written as NaN.
  const long long p0 = a.p0[b];
  const long long lo = p0 < 0 ? -p0 : 0;
  long long hi = nq;
  if (hi > (long long)a.max_ctx - p0) hi = (long long)a.max_ctx - p0;
  if (hi > (long long)a.rope_len - p0) hi = (long long)a.rope_len - p0;
  const int r0 = qb * QB, r1 = min(r0 + QB, nq);
  const int v0 = (int)max((long long)r0, lo), v1 = (int)min((long long)r1, hi);
  const bool any = v1 > v0;
  int errbits = (any ? v1 - v0 : 0) < r1 - r0 ? LLA_DEVERR_CTX : 0;
  const int kend = any ? (int)(p0 + v1) : 0;  // tokens [0, kend) are read
  const int nt = (kend + KT - 1) / KT;
  const int npg = (kend + kPage - 1) / kPage;

  const int w0 = r0 + 32 * w;
  const int wv0 = max(w0, v0);
  const int qmin = (int)(p0 + wv0);  // the wave's first query position

  // ---- prologue: Q' = scale log2(e) R(p) q as bf16 B-operands ----
  // qop[f][ks]: lane (n, g) = query w0 + 16 f + n, dims 32 ks + 8 g .. + 7.
  u32x4 qop[2][KSD];
  int qpos[2];
  bool qok[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int iq = w0 + 16 * f + n;
    qok[f] = iq >= v0 && iq < v1;
    qpos[f] = qok[f] ? (int)(p0 + iq) : 0;
    const uint16_t *qrow = (const uint16_t *)a.q + (((long long)b * nq + (qok[f] ? iq : v0)) * a.H + h) * DH;
    const float *rq = a.rope + (long long)qpos[f] * DH;
#pragma unroll
    for (int ks = 0; ks < KSD / 2; ++ks) {
      const int d0 = 32 * ks + 8 * g;
      u32x4 x = u32x4{0u, 0u, 0u, 0u}, y = x;
      if (qok[f]) {
        x = *(const u32x4 *)(qrow + d0);
        y = *(const u32x4 *)(qrow + d0 + HALF);
      }
      u32x4 pa, pb;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const f32x4 cs = *(const f32x4 *)(rq + 2 * (d0 + 2 * e2));  // (cos, sin) of pairs d0 + 2 e2, + 1
        const float qa0 = bf16_lo(x[e2]), qa1 = bf16_hi(x[e2]);
        const float qb0 = bf16_lo(y[e2]), qb1 = bf16_hi(y[e2]);
        pa[e2] = cvt2(a.qscale * (qa0 * cs[0] - qb0 * cs[1]), a.qscale * (qa1 * cs[2] - qb1 * cs[3]));
        pb[e2] = cvt2(a.qscale * (qa0 * cs[1] + qb0 * cs[0]), a.qscale * (qa1 * cs[3] + qb1 * cs[2]));
      }
      qop[f][ks] = pa;
      qop[f][ks + KSD / 2] = pb;
    }
  }

  // ---- W_up,k,t of the head in LDS (rows padded like the c_k rows), mu_k ----
  // Rebuild unit (tau, T) of wave w: tokens 16 tau .. + 15 of each tile, dims
  // 16 T + n and 16 T + n + d/2 (tile T and its RoPE partner tile).
  const int tau = w & 1, T = w >> 1;
  float muk[2][4];
  {
    const char *wkh = a.wup_k + (long long)h * a.wup_head_stride_k * 2;
    for (int c = tid; c < DH * RK / 8; c += NTH) {
      const int d = c / (RK / 8), k8 = c - d * (RK / 8);
      *(u32x4 *)(s_wk + d * SK + k8 * 16) = *(const u32x4 *)(wkh + ((long long)d * RK + 8 * k8) * 2);
    }
    const uint16_t *mkh = (const uint16_t *)a.mu_k + (long long)h * a.mu_head_stride;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) muk[j][i] = 0.f;
    if (w < NU) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) muk[j][i] = bf16_to_f32(mkh[16 * T + 4 * g + i + j * HALF]);
    }
  }

  // ---- page table, tile copies ----
  const int *pt_row = a.page_table + (long long)b * a.max_pages;
  const char *kpool = a.k_pool + (long long)h * a.pool_head_stride_k * 2;
  const char *vpool = a.v_pool + (long long)h * a.pool_head_stride_v * 2;
  const long long pstride_k = a.pool_page_stride_k * 2, pstride_v = a.pool_page_stride_v * 2;
  int bad_lp = 0x7FFFFFFF;  // first logical page with an out-of-range table entry

  auto fill_pt = [&](int c) {
    for (int i = tid; i < 1024; i += NTH) {
      const int lp = 1024 * c + i;
      s_pt[c & 1][i] = lp < npg ? pt_row[lp] : 0;
    }
  };

  // Copy it of this wave covers chunk positions 64 (it NW + w) .. + 63 of the
  // slot; lane position pos -> (c_v?, row, chunk) is the same for every tile.
  // Pad positions copy the row's first chunk (never read).
  int cp_off[IPW];   // byte offset within the page (from the K or V page base)
  int cp_row[IPW];   // tile row 0..31, or 32 for positions past the rows
  bool cp_v[IPW];
#pragma unroll
  for (int it = 0; it < IPW; ++it) {
    const int pos = 64 * (it * NW + w) + lane;
    int row = 32, off = 0;
    bool isv = false;
    if (pos < KT * CPK) {
      row = pos / CPK;
      const int c = pos - row * CPK;
      off = ((row & 15) * RK + 8 * (c < RK / 8 ? c : 0)) * 2;
    } else if (pos < KT * (CPK + CPV)) {
      isv = true;
      const int p2 = pos - KT * CPK;
      row = p2 / CPV;
      const int c = p2 - row * CPV;
      off = ((row & 15) * RV + 8 * (c < RV / 8 ? c : 0)) * 2;
    }
    cp_off[it] = off;
    cp_row[it] = row;
    cp_v[it] = isv;
  }
  // Direct-to-LDS copy of tile x (clamped to the last tile) into slot sb;
  // returns the page-validity bits (bit 0: first page, bit 1: second).
  auto copy_tile = [&](int x, char *sb) -> int {
    x = min(x, nt - 1);
    const int l0 = min(2 * x, npg - 1), l1 = min(2 * x + 1, npg - 1);
    const int e0 = __builtin_amdgcn_readfirstlane(s_pt[(l0 >> 10) & 1][l0 & 1023]);
    const int e1 = __builtin_amdgcn_readfirstlane(s_pt[(l1 >> 10) & 1][l1 & 1023]);
    const bool ok0 = e0 >= 0 && e0 < a.num_pages, ok1 = e1 >= 0 && e1 < a.num_pages;
    if (!ok0) bad_lp = min(bad_lp, l0);
    if (!ok1) bad_lp = min(bad_lp, l1);
    const long long pg0 = ok0 ? e0 : 0, pg1 = ok1 ? e1 : 0;
    const char *k0 = kpool + pg0 * pstride_k, *k1 = kpool + pg1 * pstride_k;
    const char *v0p = vpool + pg0 * pstride_v, *v1p = vpool + pg1 * pstride_v;
#pragma unroll
    for (int it = 0; it < IPW; ++it) {
      if (it < IPW_MIN || it * NW + w < NCP) {
        const bool p1 = cp_row[it] >= 16 && cp_row[it] < 32;
        const char *base = cp_v[it] ? (p1 ? v1p : v0p) : (p1 ? k1 : k0);
        __builtin_amdgcn_global_load_lds((const void *)(base + cp_off[it]), LLA_LDS(sb + 64 * 16 * (it * NW + w)), 16, 0, 0);
      }
    }
    return (ok0 ? 1 : 0) | (ok1 ? 2 : 0);
  };
  // Clear the rows of tile x (in slot sb, copies landed) that are past kend or
  // come from a bad page.
  auto clear_tile = [&](int x, char *sb, int okm) {
#pragma unroll
    for (int it = 0; it < IPW; ++it) {
      if (it < IPW_MIN || it * NW + w < NCP) {
        const int r = cp_row[it];
        if (r < 32 && (KT * x + r >= kend || !((okm >> (r >> 4)) & 1)))
          *(u32x4 *)(sb + 16 * (64 * (it * NW + w) + lane)) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  // RoPE rows of this wave's rebuild unit: pairs 16 T + 4 g .. + 3 at its token.
  f32x4 rp[2];
  auto load_rope = [&](int x) {
    const int pos = min(KT * min(x, nt - 1) + 16 * tau + n, kend - 1);
    const float *rr = a.rope + (long long)pos * DH + 2 * (16 * (w < NU ? T : 0) + 4 * g);
    rp[0] = *(const f32x4 *)rr;
    rp[1] = *(const f32x4 *)(rr + 4);
  };
  // Rotated K of the tile in slot sb into K buffer kb.
  auto rebuild = [&](const char *sb, char *kb) {
    if (w < NU) {
      const char *ck = sb + (16 * tau + n) * SK;
      const char *wa = s_wk + (16 * T + n) * SK, *wb = wa + HALF * SK;
      f32x4 k0 = f32x4{0.f, 0.f, 0.f, 0.f}, k1 = k0;
#pragma unroll
      for (int ks = 0; ks < KS32; ++ks) {
        const int off = (32 * ks + 8 * g) * 2;
        const u32x4 bop = *(const u32x4 *)(ck + off);
        k0 = mfma16(*(const u32x4 *)(wa + off), bop, k0);
        k1 = mfma16(*(const u32x4 *)(wb + off), bop, k1);
      }
      if constexpr (TAIL) {
        const int off = (32 * KS32 + 4 * g) * 2;
        const bf16x4 bt = __builtin_bit_cast(bf16x4, *(const u32x2 *)(ck + off));
        k0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, *(const u32x2 *)(wa + off)), bt, k0, 0, 0, 0);
        k1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, *(const u32x2 *)(wb + off)), bt, k1, 0, 0, 0);
      }
      float ra[4], rb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ka = k0[i] + muk[0][i], kb2 = k1[i] + muk[1][i];
        const float c = rp[i >> 1][2 * (i & 1)], s = rp[i >> 1][2 * (i & 1) + 1];
        ra[i] = ka * c - kb2 * s;
        rb[i] = ka * s + kb2 * c;
      }
      char *row = kb + (16 * tau + n) * SKH;
      *(u32x2 *)(row + (16 * T + 4 * g) * 2) = u32x2{cvt2(ra[0], ra[1]), cvt2(ra[2], ra[3])};
      *(u32x2 *)(row + (HALF + 16 * T + 4 * g) * 2) = u32x2{cvt2(rb[0], rb[1]), cvt2(rb[2], rb[3])};
    }
  };

  // ---- online softmax state and latent-space value sums ----
  f32x4 o[2][NRT];
  float m_ref[2], l_run[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    m_ref[f] = -INFINITY;
    l_run[f] = 0.f;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) o[f][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto attend = [&](int x, const char *sb, const char *kb) {
    f32x4 s[2][2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int f = 0; f < 2; ++f) s[t2][f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const u32x4 ak = *(const u32x4 *)(kb + (16 * t2 + n) * SKH + (32 * ks + 8 * g) * 2);
#pragma unroll
        for (int f = 0; f < 2; ++f) s[t2][f] = mfma16(ak, qop[f][ks], s[t2][f]);
      }
    }
    const bool masked = KT * x + KT - 1 > qmin;
    u32x4 pop[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      if (masked) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (KT * x + 16 * t2 + 4 * g + i > qpos[f]) s[t2][f][i] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(s[0][f][0], s[0][f][1]), fmaxf(s[0][f][2], s[0][f][3])),
                       fmaxf(fmaxf(s[1][f][0], s[1][f][1]), fmaxf(s[1][f][2], s[1][f][3])));
      mx = max_across_rows(mx);
      if (__builtin_amdgcn_ballot_w64(mx > m_ref[f] + 8.f)) {
        const float mn = fmaxf(m_ref[f], mx);
        const float al = mn == -INFINITY ? 1.f : fast_exp2(m_ref[f] - mn);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) o[f][rt] *= al;
        l_run[f] *= al;
        m_ref[f] = mn;
      }
      const float mu = m_ref[f] == -INFINITY ? 0.f : m_ref[f];
      float e[8];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int i = 0; i < 4; ++i) e[4 * t2 + i] = fast_exp2(s[t2][f][i] - mu);
      l_run[f] += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      pop[f] = u32x4{cvt2(e[0], e[1]), cvt2(e[2], e[3]), cvt2(e[4], e[5]), cvt2(e[6], e[7])};
    }
    // O^T += C_v^T P^T; K index 8 g + e <-> token 16 (e / 4) + 4 g + e % 4
    const char *vb = sb + VOFF + (4 * g + (n >> 2)) * SV + 8 * (n & 3);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const u32x2 lo2 = lds_read_tr(vb + 32 * rt);
      const u32x2 hi2 = lds_read_tr(vb + 16 * SV + 32 * rt);
      const u32x4 av = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
#pragma unroll
      for (int f = 0; f < 2; ++f) o[f][rt] = mfma16(av, pop[f], o[f][rt]);
    }
  };

  // ---- main loop ----
  // Step x: clear tile x + 1 if it needs it, load the RoPE rows for its
  // rebuild, copy tile x + 3 into its slot, attend tile x, rebuild tile x + 1,
  // barrier.  Tile y lives in slot y % 4 and K buffer y % 2; the copy of tile
  // y (issued in step y - 3) is complete in every wave after the barrier of
  // step y - 2 (each wave leaves only the copies of step y - 2 in flight).
  int okm0 = 3, okm1 = 3, okm2 = 3, okm3 = 3;
  if (nt > 0) {
    fill_pt(0);
    if (npg > 1024) fill_pt(1);
    __syncthreads();  // s_pt, s_wk
    okm0 = copy_tile(0, s_c0);
    if (nt > 1) okm1 = copy_tile(1, s_c1);
    if (nt > 2) okm2 = copy_tile(2, s_c2);
    load_rope(0);
    barrier_vm<0>();
    clear_tile(0, s_c0, okm0);
    if (nt > 1) clear_tile(1, s_c1, okm1);
    barrier_vm<0>();
    rebuild(s_c0, s_kh0);
    barrier_vm<0>();
  }
  auto step = [&](int x, char *sx, char *sx1, char *sx3, int okx1, int &okx3, char *kbx, char *kbx1) {
    if (x + 1 < nt && x >= 1 && (x + 1 == nt - 1 || okx1 != 3)) {  // tiles 0 and 1 were cleared above
      clear_tile(x + 1, sx1, okx1);
      barrier_vm<63>();
    }
    if (((2 * (x + 3)) & 1023) == 0 && 2 * (x + 3) + 1024 < npg) fill_pt(((2 * (x + 3)) >> 10) + 1);
    load_rope(x + 1);
    okx3 = copy_tile(x + 3, sx3);
    attend(x, sx, kbx);
    if (x + 1 < nt) rebuild(sx1, kbx1);
    barrier_vm<IPW_MIN>();
  };
  for (int x = 0; x < nt; x += 4) {
    step(x, s_c0, s_c1, s_c3, okm1, okm3, s_kh0, s_kh1);
    if (x + 1 < nt) step(x + 1, s_c1, s_c2, s_c0, okm2, okm0, s_kh1, s_kh0);
    if (x + 2 < nt) step(x + 2, s_c2, s_c3, s_c1, okm3, okm1, s_kh0, s_kh1);
    if (x + 3 < nt) step(x + 3, s_c3, s_c0, s_c2, okm0, okm2, s_kh1, s_kh0);
  }
  __syncthreads();  // no copy in flight past the loop

  // ---- epilogue: normalise, up-project with W_up,v, add mu_v ----
  if (bad_lp != 0x7FFFFFFF) errbits |= LLA_DEVERR_PAGE;
  if (errbits && tid == 0) atomicOr(a.err, errbits);

  u32x4 bup[2][KSV];  // B-operands: a[q][r] with K index 8 g + e <-> r = 32 ks + 16 (e / 4) + 4 g + e % 4
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const float z = sum_across_rows(l_run[f]);
    const bool bad = !qok[f] || (long long)qpos[f] >= (long long)kPage * bad_lp;
    const float inv = bad ? __builtin_nanf("") : 1.f / z;
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) {
      const f32x4 u0 = o[f][2 * ks] * inv, u1 = o[f][2 * ks + 1] * inv;
      bup[f][ks] = u32x4{cvt2(u0[0], u0[1]), cvt2(u0[2], u0[3]), cvt2(u1[0], u1[1]), cvt2(u1[2], u1[3])};
    }
  }
  const char *wvh = a.wup_v + (long long)h * a.wup_head_stride_v * 2;
  const uint16_t *mvh = (const uint16_t *)a.mu_v + (long long)h * a.mu_head_stride;
#pragma unroll 2
  for (int et = 0; et < NDT; ++et) {
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    const char *wr = wvh + ((long long)(16 * et + n) * RV + 4 * g) * 2;
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) {
      const u32x2 w0v = *(const u32x2 *)(wr + 64 * ks);
      const u32x2 w1v = *(const u32x2 *)(wr + 64 * ks + 32);
      const u32x4 av = u32x4{w0v[0], w0v[1], w1v[0], w1v[1]};
#pragma unroll
      for (int f = 0; f < 2; ++f) acc[f] = mfma16(av, bup[f][ks], acc[f]);
    }
    const u32x2 mu2 = *(const u32x2 *)(mvh + 16 * et + 4 * g);
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int iq = w0 + 16 * f + n;
      if (iq < r1) {
        uint16_t *orow = (uint16_t *)a.out + (((long long)b * nq + iq) * a.H + h) * DH + 16 * et + 4 * g;
        *(u32x2 *)orow = u32x2{cvt2(acc[f][0] + bf16_lo(mu2[0]), acc[f][1] + bf16_hi(mu2[0])),
                               cvt2(acc[f][2] + bf16_lo(mu2[1]), acc[f][3] + bf16_hi(mu2[1]))};
      }
    }
  }
}

// ---------------------------------------------------------------- dispatch

// (d_head, r_k, r_v)
#define LLA_PREFILL_SHAPES(X) \
  X(64, 16, 32)               \
  X(128, 16, 32)              \
  X(128, 32, 64)              \
  X(128, 96, 160)

bool prefill_supported(int dtype, int variant, int d_head, int r_k, int r_v) {
  if (dtype != LLA_BF16 || variant != LLA_PER_HEAD) return false;
#define X(DH, RK, RV) \
  if (d_head == DH && r_k == RK && r_v == RV) return true;
  LLA_PREFILL_SHAPES(X)
#undef X
  return false;
}

hipError_t launch_prefill(int d_head, int r_k, int r_v, const AttnArgs &a, hipStream_t stream) {
  if (a.n_q < 1 || a.rows % a.n_q) return hipErrorInvalidConfiguration;
  const long long nqb = (a.n_q + 255) / 256;
  const long long grid = (long long)(a.rows / a.n_q) * a.H * nqb;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
#define X(DH, RK, RV)                                                                                \
  if (d_head == DH && r_k == RK && r_v == RV) {                                                      \
    hipLaunchKernelGGL((prefill_kernel<DH, RK, RV>), dim3((unsigned)grid), dim3(512), 0, stream, a); \
    return hipGetLastError();                                                                        \
  }
  LLA_PREFILL_SHAPES(X)
#undef X
  return hipErrorInvalidConfiguration;
}

}  // namespace lla
