// LLA-2D decode attention (gfx950, wave64): heads folded into one latent.
//
// What it computes (cc.laoqi.cc close reading, 方法 item 6; gist.science
// "LLA-2D-Variante"): every cached token keeps ONE K latent c_k (r_k wide) and
// ONE V latent c_v (r_v wide) per layer, shared by all H heads; loop t and head
// h decode it with their own mu_t,h and W_up,t,h (d x r):
//   k_hat_j,h = mu_k,t,h + c_k,j W_up,k,t,h^T, RoPE at position j,
//   s_j,h     = scale <R(q_pos) q_h, R(j) k_hat_j,h>,
//   out_h     = mu_v,t,h + (sum_j e^{s_j,h - m} c_v,j) W_up,v,t,h^T / sum_j e^{s_j,h - m}.
//
// Per token this is d*r_k multiply-adds per head for the K side (2 MFLOP per
// token at H=32, d=128, r_k=256), so unlike per-head LLA the path is bound by
// the matrix cores, not by HBM.  Layout of the work:
//  * A workgroup = 8 waves = 4 heads of one query row and one split of the
//    context, two waves per head.  The waves of a head fold its rotated query
//    into the K decoder (the same exact algebra as the per-head kernel: for
//    RoPE pair i, X_i = alpha_i + A_i . c, Y_i = beta_i + B_i . c and
//    s * log2(e) = sum_i cos_i(j) X_i + sin_i(j) Y_i), each for half of the
//    RoPE pairs, and keep that half of the d x (r_k+1) result in registers as
//    the A-operands of v_mfma_f32_32x32x16_bf16 (alpha / beta as hi + lo bf16
//    in one extra K-step).
//  * Tokens go in blocks of 32 (two 16-token pages).  The block's c_k, c_v and
//    RoPE rows are copied global -> LDS with buffer loads straight into LDS (no
//    register staging; whole rows per instruction, one shared lane offset as
//    the only vector operand) into three buffers: the copy of block b+2 is in flight while the
//    K-side products of block b+1 share a barrier interval with the softmax of
//    block b, and the value sum of block b with the cos / sin weighting of
//    block b+1 (two barriers per block).
//    The tile is shared by the 4 waves, so each latent is fetched from L2 once
//    per workgroup.  Workgroups of the same (row, split) but different head
//    groups are dispatched to the same XCD so that they share its L2.
//  * K side: 2 x 17 MFMAs per wave per block give X / Y for its 32 pairs x 32
//    tokens; each lane weights its values by cos / sin (fp32), one permlane32
//    swap completes the wave's half-score, and the two halves of a head meet
//    in LDS (added in the same order by both).  Online softmax in base 2.
//  * V side, exact by linearity: sum_j p_j,h c_v,j for the 4 heads is one more
//    MFMA product, P[tokens x 4 heads] (bf16 weights via LDS) times the c_v
//    tile; wave w owns r_v/8 of the columns for all 4 heads.
//  * With one split the workgroup up-projects once per head; with several it
//    writes (m, Z, acc) partials for the merge launch (lla_merge.hip).
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {

typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

#define LLA_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// Word 3 of a raw buffer descriptor on gfx9-family parts: 32-bit data format,
// no swizzle, no index stride (untyped loads by byte offset).
constexpr int kBufferWord3 = 0x00020000;

// 16 bytes per active lane from base + soff + voff into LDS at lds + 16 lane,
// as a buffer load of the `bytes`-long range at base (reads past it give zeros).
// base, bytes and soff are uniform; only voff is per lane.
__device__ __forceinline__ void buffer_to_lds16(const char *base, uint32_t bytes, void *lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)bytes, kBufferWord3), LLA_LDS(lds), 16, voff,
      soff, 0, 0);
}

// Barrier that first waits for this wave's LDS writes and for all but its VM
// most recent vector-memory operations (direct-to-LDS copies still in flight).
template <int VM>
__device__ __forceinline__ void barrier_vm() {
  static_assert(VM >= 0 && VM < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(((VM >> 4) << 14) | (VM & 15) | 0x70);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 32-token block in LDS.  c_k and the RoPE rows keep their memory layout,
// one token per row, with each row padded by 16 bytes: a copy instruction
// then reads one whole row (512 contiguous bytes), and the operand reads (16
// lanes of consecutive tokens at one 16-byte piece) hit 16 distinct bank
// groups at immediate offsets.
template <int DH, int RK, int RV>
struct Tile2d {
  u32x4 ck[32][RK / 8 + 1];    // [token][r chunk of 8], padded row
  u32x4 cv[32 * RV / 8];       // [token 32][r_v]: row-major latent rows
  f32x4 trig[32][DH / 4 + 1];  // [token][pair chunk of 2]: (cos, sin) x 2, fp32, padded row
};

template <int DH, int RK, int RV>
__global__ __launch_bounds__(512) void decode_2d_kernel(AttnArgs a) {
  constexpr int NW = 8;          // waves per workgroup: 4 heads x 2 halves of the RoPE pairs
  constexpr int NH = 4;          // heads per workgroup
  constexpr int HALF = DH / 2;   // RoPE pairs of a head
  constexpr int PW = HALF / 2;   // pairs per wave
  constexpr int RTW = PW / 16;   // 32-row tiles per wave (X and Y rows of 16 pairs each)
  constexpr int KS = RK / 16;    // K-steps of 16 (8 per lane half)
  constexpr int CVQ = RV / 16;   // 1 KiB direct loads per tile: c_v
  constexpr int VR = RV / NW;    // V columns per wave (all 4 heads)
  constexpr int VT = VR / 16;    // V MFMA tiles per wave (16x16x32)
  static_assert(PW % 16 == 0 && RK % 128 == 0 && VR == 32 && VT == 2 && KS >= 5, "shape");
  static_assert(CVQ % NW == 0 && 32 % NW == 0 && RK / 8 <= 64 && DH / 4 <= 64 && RV == 256, "tile split");

  __shared__ Tile2d<DH, RK, RV> tile0, tile1, tile2;
  __shared__ __attribute__((aligned(16))) uint16_t s_p[16][32];  // bf16 weights; rows >= 4 stay 0
  __shared__ float s_alpha[16];                                   // rescale per head; >= 4 stay 1
  __shared__ float s_part[NH][2][32];                             // half-scores per head
  __shared__ int s_pt[kMaxPages2d + 2];
  __shared__ float s_red[NH][RV + 2];  // epilogue: normalised latent sums per head
  __shared__ float s_z[NH];

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = w >> 1, rh = w & 1;         // head within the group, half of the pairs
  const int t = lane & 31, kh = lane >> 5;   // 32x32 operand column (token) and K half
  const int g16 = lane >> 4, n16 = lane & 15;  // 16x16 operand layout

  // ---- XCD-aware placement: the head groups of one (row, split) share an XCD ----
  const int units = a.rows * a.splits;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, u = bid >> 3;
  const int hg = u % a.head_groups;
  const int unit = (u / a.head_groups) * 8 + xcd;
  if (unit >= units) return;  // grid padding, uniform over the workgroup
  const int row = unit / a.splits, split = unit - row * a.splits;
  const int b = row / a.n_q, qi = row - b * a.n_q;
  const int h = hg * NH + hl;

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
  const int j_lo = lp0 * kPage, j_hi = min(lp1 * kPage, ctx);
  const int nblk = j_hi > j_lo ? (j_hi - j_lo + 31) / 32 : 0;

  for (int i = threadIdx.x; i < 16 * 32; i += blockDim.x) (&s_p[0][0])[i] = 0;
  if (threadIdx.x < 16) s_alpha[threadIdx.x] = 1.f;
  {
    const int *pt_row = a.page_table + (long long)b * a.max_pages;
    for (int i = threadIdx.x; i < lp1 - lp0; i += blockDim.x) {
      const int p = pt_row[lp0 + i];
      const bool ok = p >= 0 && p < a.num_pages;
      if (!ok) errbits |= LLA_DEVERR_PAGE;
      s_pt[i] = ok ? p : 0;
    }
  }

  // ---- prologue: the rotated query folded into W_up,k,t,h as MFMA A-operands ----
  // Row m of this wave's row tile rt (global tile gt = RTW rh + rt) is RoPE pair
  //   i = 16 gt + 8 ((m / 4) % 2) + 2 (m / 8) + (m % 4) / 2, an X row if m is even,
  // which makes lane (t, kh)'s accumulator element j of tile rt the X (j even)
  // or Y (j odd) value of pair 16 gt + 8 kh + 2 (j / 4) + (j % 4) / 2 at token t.
  // K-slot e of K-step s in lane half kh is latent column 8 (kh KS + s) + e.
  bf16x8 A[RTW][KS];
  uint32_t A1[RTW];  // extra K-step, slot pair (0, 1): alpha or beta as bf16 hi + lo
  {
    const float *rq = a.rope + (long long)qp * DH;
    const uint16_t *qrow = (const uint16_t *)a.q + ((long long)row * a.H + h) * DH;
    const char *wk = a.wup_k + (long long)h * a.wup_head_stride_k * 2;
    const uint16_t *mu = (const uint16_t *)a.mu_k + (long long)h * a.mu_head_stride;
    const int m = t;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int gt = RTW * rh + rt;
      const int i = 16 * gt + 8 * ((m >> 2) & 1) + 2 * (m >> 3) + ((m & 3) >> 1);
      const float c = rq[2 * i], s = rq[2 * i + 1];
      const float qa = bf16_to_f32(qrow[i]), qb = bf16_to_f32(qrow[i + HALF]);
      const float pa = a.qscale * (qa * c - qb * s);
      const float pb = a.qscale * (qa * s + qb * c);
      // X = pa k_a + pb k_b ; Y = pb k_a - pa k_b
      const float ca = (m & 1) ? pb : pa, cb = (m & 1) ? -pa : pb;
#pragma unroll
      for (int s8 = 0; s8 < KS; ++s8) {
        const int r0 = 8 * (kh * KS + s8);
        const u32x4 wa = *(const u32x4 *)(wk + ((long long)i * RK + r0) * 2);
        const u32x4 wb = *(const u32x4 *)(wk + ((long long)(i + HALF) * RK + r0) * 2);
        u32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[e] = pack_bf16(ca * bf16_lo(wa[e]) + cb * bf16_lo(wb[e]),
                           ca * bf16_hi(wa[e]) + cb * bf16_hi(wb[e]));
        // materialise now (otherwise the packing sinks to the loop and the raw
        // W_up rows stay live, twice the registers of the result)
        asm volatile("" : "+v"(x));
        A[rt][s8] = as_bf16x8(x);
      }
      const float v = ca * bf16_to_f32(mu[i]) + cb * bf16_to_f32(mu[i + HALF]);
      const uint32_t hi = f32_to_bf16(v);
      const uint32_t lo = f32_to_bf16(v - bf16_to_f32(hi));
      A1[rt] = kh == 0 ? (hi | (lo << 16)) : 0u;
    }
  }
  // constant B-operand of the extra K-step: bf16 (1, 1) in slots 0, 1 of half 0
  const bf16x8 bone = as_bf16x8(u32x4{kh == 0 ? 0x3F803F80u : 0u, 0u, 0u, 0u});
  __syncthreads();  // s_pt, s_p, s_alpha

  // ---- direct-to-LDS loads of one 32-token block ----
  const char *rope_b = (const char *)a.rope;
  // Every copy instruction reads whole rows as a buffer load into LDS: a
  // descriptor for the page (or the block's RoPE rows) in scalar registers, the
  // row offset as a scalar, and 16 bytes per lane as the only vector operand.
  // Offsets past a descriptor's size read zeros.  Waves 0 .. NW/2 - 1 copy
  // the block's first page, the others its second.
  const int lane16 = 16 * lane;
  // s_pt index of the page this wave copies for block blk
  auto page_idx = [&](int blk) -> int {
    return min((j_lo + 32 * blk) / kPage + (w >= NW / 2 ? 1 : 0), lp1 - 1) - lp0;
  };
  // pg: that page (read from s_pt a step earlier, so no LDS wait sits here)
  // The copies of one block in five parts of two instructions each (c_k rows,
  // c_v, RoPE rows), so that they can be issued between K-side products: a
  // wave that issued them all at once waited on the copy queue.
  auto issue_part = [&](int blk, long long pg, Tile2d<DH, RK, RV> &T, int part) {
    const int j0 = j_lo + 32 * blk;
    if (part < 2) {  // c_k: one row (token) per half-wave instruction
      constexpr int CPT = RK / 8;  // 16-byte pieces per c_k row
      const char *kpg = a.k_pool + pg * a.pool_page_stride_k * 2;
#pragma unroll
      for (int i = 2 * part; i < 2 * part + 2; ++i) {
        const int tok = w * (32 / NW) + i;
        if (lane < CPT)
          buffer_to_lds16(kpg, kPage * RK * 2, &T.ck[tok][0], lane16, (tok & 15) * RK * 2);
      }
    } else if (part == 2) {  // c_v: two rows per instruction
      const char *vpg = a.v_pool + pg * a.pool_page_stride_v * 2;
#pragma unroll
      for (int i = 0; i < CVQ / NW; ++i) {
        const int q = w * (CVQ / NW) + i;
        buffer_to_lds16(vpg, kPage * RV * 2, &T.cv[q * 64], lane16, ((2 * q) & 15) * RV * 2);
      }
    } else {  // RoPE rows of the block's positions: one row per half-wave
              // instruction; rows past the table read zeros (their tokens lie
              // past the context)
      constexpr int TPT = DH / 4;  // 16-byte pieces per RoPE row
      const int jr = min(j0, a.rope_len - 1);
      const char *rrow = rope_b + (long long)jr * (DH * 4);
      const uint32_t rbytes = (uint32_t)(a.rope_len - jr) * (DH * 4);
#pragma unroll
      for (int i = 2 * (part - 3); i < 2 * (part - 3) + 2; ++i) {
        const int tok = w * (32 / NW) + i;
        if (lane < TPT)
          buffer_to_lds16(rrow, rbytes, &T.trig[tok][0], lane16, (j0 - jr + tok) * (DH * 4));
      }
    }
  };
  auto issue = [&](int blk, long long pg, Tile2d<DH, RK, RV> &T) {
#pragma unroll
    for (int part = 0; part < 5; ++part) issue_part(blk, pg, T, part);
  };

  float m_run = -INFINITY, z_run = 0.f;
  f32x4 accv[VT];
#pragma unroll
  for (int v = 0; v < VT; ++v) accv[v] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The block loop is software-pipelined over three tile buffers so that the
  // K-side products of block b + 1 sit in the same barrier interval as the
  // softmax of block b (the matrix cores run while the vector units reduce):
  //   interval A(b): issue copies of block b + 2; softmax(b); K side(b + 1)
  //   interval B(b): value sum(b); cos / sin weighting(b + 1) -> s_part
  // A(b) ends with a barrier that leaves this wave's copies of block b + 2 in
  // flight; B(b) ends with a barrier after all copies have landed.
  // between(s8) runs after the products of K-step s8
  auto kside = [&](Tile2d<DH, RK, RV> &T, f32x16 (&acc)[RTW], auto &&between) {
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) acc[rt] = f32x16{};
    // B-operand pieces PF K-steps ahead; the scheduling fence keeps each read
    // above the products it feeds (the compiler would otherwise sink it to its use)
    constexpr int PF = 4;
    u32x4 bk[PF + 1];
    auto piece = [&](int c) { return T.ck[t][c]; };  // r chunk c of token t
#pragma unroll
    for (int p = 0; p < PF; ++p) bk[p] = piece(kh * KS + p);
#pragma unroll
    for (int s8 = 0; s8 < KS; ++s8) {
      if (s8 + PF < KS) bk[(s8 + PF) % (PF + 1)] = piece(kh * KS + s8 + PF);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt)
        acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[rt][s8], as_bf16x8(bk[s8 % (PF + 1)]), acc[rt], 0, 0, 0);
      between(s8);
    }
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
      acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u32x4{A1[rt], 0u, 0u, 0u}), bone,
                                                         acc[rt], 0, 0, 0);
  };
  auto weigh = [&](Tile2d<DH, RK, RV> &T, const f32x16 (&acc)[RTW]) {
    float sp = 0.f;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int gt = RTW * rh + rt;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 tr = T.trig[t][8 * gt + 4 * kh + q];
        sp = fmaf(tr[0], acc[rt][4 * q + 0], sp);
        sp = fmaf(tr[1], acc[rt][4 * q + 1], sp);
        sp = fmaf(tr[2], acc[rt][4 * q + 2], sp);
        sp = fmaf(tr[3], acc[rt][4 * q + 3], sp);
      }
    }
    const uint32_t us = __float_as_uint(sp);
    const auto sw = __builtin_amdgcn_permlane32_swap(us, us, false, false);
    sp = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (kh == 0) s_part[hl][rh][t] = sp;
  };
  auto softmax = [&](int blk) {
    const int j0 = j_lo + 32 * blk;
    const int nvalid = min(32, j_hi - j0);
    // both halves of a head add the two half-scores in the same order
    const float sfull = s_part[hl][0][t] + s_part[hl][1][t];
    const float s = t < nvalid ? sfull : -INFINITY;
    float bm = max_in_row(s);
    {
      const uint32_t ub = __float_as_uint(bm);
      const auto sw = __builtin_amdgcn_permlane16_swap(ub, ub, false, false);
      bm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float m_new = fmaxf(m_run, bm);  // finite: block has >= 1 valid token
    const float alpha = fast_exp2(m_run - m_new);
    const uint32_t pbits = f32_to_bf16(fast_exp2(s - m_new));
    float ps = sum_in_row(bf16_to_f32(pbits));
    {
      const uint32_t up = __float_as_uint(ps);
      const auto sw = __builtin_amdgcn_permlane16_swap(up, up, false, false);
      ps = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    z_run = fmaf(z_run, alpha, ps);
    m_run = m_new;
    if (rh == 0 && kh == 0) s_p[hl][t] = (uint16_t)pbits;
    if (rh == 0 && lane == 0) s_alpha[hl] = alpha;
  };
  auto vside = [&](int blk, Tile2d<DH, RK, RV> &T) {
    const int j0 = j_lo + 32 * blk;
    const int nvalid = min(32, j_hi - j0);
    // accv[head n][r] = accv * alpha_n + sum_t p[n][t] c_v[t][r]
    const float al = s_alpha[n16];
    const u32x4 pv = *(const u32x4 *)&s_p[n16][8 * g16];
    const int rb = w * VR + 2 * n16;  // lane's 2 columns: rb, rb + 1 (one per tile)
    uint32_t cvr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tok = 8 * g16 + e;
      cvr[e] = *(const uint32_t *)((const char *)T.cv + (tok * RV + rb) * 2);
      if (nvalid < 32 && tok >= nvalid) cvr[e] = 0u;
    }
#pragma unroll
    for (int v = 0; v < VT; ++v) {
      // tile v holds column rb + v for tokens 8 g16 + e: select bf16 half v of each dword
      u32x4 av;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        av[d] = v ? __builtin_amdgcn_perm(cvr[2 * d + 1], cvr[2 * d], 0x07060302u)
                  : __builtin_amdgcn_perm(cvr[2 * d + 1], cvr[2 * d], 0x05040100u);
      accv[v] = accv[v] * al;
      accv[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(pv), accv[v], 0, 0, 0);
    }
  };
  // this wave's copy instructions per block (all of them count on vmcnt)
  constexpr int NCOPY = 2 * (32 / NW) + CVQ / NW;
  int pgv = 0;  // s_pt entry of the next copy, loaded one step ahead
  auto step = [&](int blk, Tile2d<DH, RK, RV> &Tb, Tile2d<DH, RK, RV> &Tn, Tile2d<DH, RK, RV> &Tnn) {
    const long long pg = __builtin_amdgcn_readfirstlane(pgv);
    pgv = s_pt[page_idx(min(blk + 3, nblk - 1))];
    const int cb = min(blk + 2, nblk - 1);  // past the end: a harmless re-copy of the last block
    f32x16 acc[RTW];
    kside(Tn, acc, [&](int s8) {  // block b + 1 (past the end: ignored)
#pragma unroll
      for (int part = 0; part < 5; ++part)  // every part once: K-steps 0, KS/5, .. (distinct for KS >= 5)
        if (s8 == part * KS / 5) issue_part(cb, pg, Tnn, part);
    });
    softmax(blk);
    barrier_vm<NCOPY>();
    weigh(Tn, acc);
    vside(blk, Tb);
    barrier_vm<0>();
  };

  if (nblk > 0) {
    issue(0, __builtin_amdgcn_readfirstlane(s_pt[page_idx(0)]), tile0);
    issue(min(1, nblk - 1), __builtin_amdgcn_readfirstlane(s_pt[page_idx(min(1, nblk - 1))]), tile1);
    pgv = s_pt[page_idx(min(2, nblk - 1))];
    barrier_vm<0>();
    f32x16 acc0[RTW];
    kside(tile0, acc0, [](int) {});
    weigh(tile0, acc0);
    barrier_vm<0>();
    int blk = 0;
    for (; blk + 3 <= nblk; blk += 3) {
      step(blk, tile0, tile1, tile2);
      step(blk + 1, tile1, tile2, tile0);
      step(blk + 2, tile2, tile0, tile1);
    }
    if (blk < nblk) step(blk, tile0, tile1, tile2);
    if (blk + 1 < nblk) step(blk + 1, tile1, tile2, tile0);
  }

  // ---- epilogue ----
  if (errbits) atomicOr(a.err, errbits);
  const bool bad = __syncthreads_or(errbits != 0);
  // accv[v][e] = latent sum of head n16 at column w VR + 2 (4 g16 + e) + v
  auto col = [&](int v, int e) { return w * VR + 2 * (4 * g16 + e) + v; };

  if (a.splits > 1) {
    if (n16 < NH) {
      float *part = a.partials + (((long long)row * a.H + hg * NH + n16) * a.splits + split) * (RV + 2);
#pragma unroll
      for (int v = 0; v < VT; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) part[col(v, e)] = accv[v][e];
    }
    if (rh == 0 && lane == 0) {
      float *part = a.partials + (((long long)row * a.H + h) * a.splits + split) * (RV + 2);
      part[RV] = m_run;
      part[RV + 1] = bad ? __builtin_nanf("") : z_run;
    }
    return;  // the merge launch combines the splits
  } else {
    if (rh == 0 && lane == 0) s_z[hl] = bad ? __builtin_nanf("") : z_run;
    __syncthreads();
    if (n16 < NH) {
      const float zz = s_z[n16];
#pragma unroll
      for (int v = 0; v < VT; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) s_red[n16][col(v, e)] = accv[v][e] / zz;
    }
  }
  __syncthreads();

  // ---- V up-projection of head h, outputs rh * d/2 ... : out = mu_v + accn W_up,v^T ----
  {
    const char *wv = a.wup_v + (long long)h * a.wup_head_stride_v * 2;
    const uint16_t *mu = (const uint16_t *)a.mu_v + (long long)h * a.mu_head_stride;
    const float *an = s_red[hl];
    for (int e = rh * HALF + lane; e < (rh + 1) * HALF; e += 64) {
      float o = bf16_to_f32(mu[e]);
      const char *we = wv + (long long)e * RV * 2;
#pragma unroll 4
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

// (d_head, r_k, r_v); r_v = 256 gives each lane 2 adjacent V columns (one per tile)
#define LLA_DECODE2D_SHAPES(X) \
  X(128, 256, 256)             \
  X(64, 128, 256)

bool decode2d_supported(int dtype, int d_head, int r_k, int r_v) {
  if (dtype != LLA_BF16) return false;
#define X(DH, RK, RV) \
  if (d_head == DH && r_k == RK && r_v == RV) return true;
  LLA_DECODE2D_SHAPES(X)
#undef X
  return false;
}

hipError_t launch_decode2d(int d_head, int r_k, int r_v, const AttnArgs &a, hipStream_t stream) {
  if (a.waves != 8 || a.heads_per_wave != 1) return hipErrorInvalidConfiguration;
  if (a.pages_per_split > kMaxPages2d || a.pages_per_split % 2) return hipErrorInvalidConfiguration;
  const long long units = (long long)a.rows * a.splits;
  const long long grid = (units + 7) / 8 * 8 * a.head_groups;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
#define X(DH, RK, RV)                                                                        \
  if (d_head == DH && r_k == RK && r_v == RV) {                                              \
    hipLaunchKernelGGL((decode_2d_kernel<DH, RK, RV>), dim3((unsigned)grid), dim3(512), 0,   \
                       stream, a);                                                           \
    return hipGetLastError();                                                                \
  }
  LLA_DECODE2D_SHAPES(X)
#undef X
  return hipErrorInvalidConfiguration;
}

}  // namespace lla
