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
//  * A workgroup = 256 consecutive queries of one (sequence, head): 8 waves of
//    32 queries at d = 128 (two waves per SIMD), 4 waves of 64 at d = 64.
//  * Keys go in 32-token tiles (two pages).  A tile's c_k and c_v rows and the
//    RoPE row of its first position are copied global -> LDS with direct-to-LDS
//    loads five tiles ahead, into one of six slots.  The copies are issued in
//    inline asm and waited for explicitly (each step's barrier leaves the
//    newest copies in flight), so that the compiler adds no waits of its own
//    on them.  c_k rows are padded and c_v rows sized so that the transposing
//    reads avoid bank conflicts.  Rows past the last needed position, and rows
//    of a page whose table entry is out of range, are cleared to zero before
//    use.  The page-table entries of the sequence are staged in LDS.
//  * Rebuild, one tile ahead: each wave turns a 16-dim block and its RoPE
//    partner block of the tile into rotated K (v_mfma_f32_16x16x32_bf16 with
//    the W_up,k rows staged once in LDS as the A-operand; mu as the initial
//    accumulator; RoPE in fp32 by angle addition from the copied row of the
//    tile's first position and per-lane constants of the row offset) and stores
//    it in bf16 to a double-buffered LDS tile.
//  * S^T = K Q'^T with v_mfma_f32_32x32x16_bf16 and Q' = scale log2(e) R(p) q
//    in bf16 registers: each lane holds one query's column for 16 tokens.
//  * Softmax with one fixed reference per query (the max of its first tile):
//    no rescaling of the accumulators.  If a score exceeds the reference by
//    more than 64 or the sum of weights is not finite, the block runs again
//    with the exact max as the reference.  The sums of weights are taken of the
//    bf16 weights the value sums use.
//  * O^T[r][q] += C_v^T[r][t] P^T[t][q]: the bf16 weights come straight from
//    the score accumulator as the B-operand; the c_v tile is read transposed
//    with ds_read_b64_tr_b16 as the A-operand.
//  * The LDS operands of each matrix phase are loaded in a batch ahead of it.
//  * Epilogue: O / Z in bf16 times W_up,v on the matrix cores, plus mu_v.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

#define LLA_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// Byte address in LDS of byte off of the LDS object at base (wave-uniform).
__device__ __forceinline__ uint32_t lds_addr(const char *base, int off) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)base + off);
}

// Direct global -> LDS copies: lane l's 16 (4) bytes at g land at LDS byte
// lds + 16 l (4 l).  They are issued here rather than through the compiler's
// builtin so that the compiler adds no waits of its own for them: the tile
// pipeline waits for its copies itself (vmcnt at each step's barrier), and the
// compiler's tracking of such copies made every access to another LDS buffer
// wait for all copies in flight.  No register is written by them.
__device__ __forceinline__ void dma_lds16(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma_lds4(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

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

// Max and sum of a value over lanes l and l ^ 32 (v_permlane32_swap hands each
// lane both its own value and its partner's).
__device__ __forceinline__ float max_across_halves(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
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

template <int DH, int RK, int RV, int NW>
__global__ __launch_bounds__(NW * 64, 1) void prefill_kernel(AttnArgs a) {
  constexpr int NTH = NW * 64, QB = 256, QW = QB / NW, QF = QW / 32, KT = 32;  // queries per workgroup / wave, tokens per tile
  constexpr int HALF = DH / 2, KSQ = DH / 16;      // score K-steps of 16 dims
  constexpr int NDB = DH / 32;                     // 16-dim blocks in each RoPE half
  constexpr int NTW = 2 * NDB / NW;               // 16-token halves of a tile each wave rebuilds
  constexpr int KS32 = RK / 32;
  constexpr bool TAIL = (RK % 32) != 0;            // one extra 16-wide rebuild K-step
  constexpr int KSW = KS32 > 0 ? KS32 : 1;
  constexpr int NRB = RV / 32, KSV = RV / 16;      // 32-row blocks of O^T, up-projection K-steps
  // LDS rows of a slot, in 16-byte chunks: RK / 8 (+1 pad) for c_k; for c_v the
  // first count >= RV / 8 that is 4 or 12 mod 16, so that the four rows a
  // 16-lane group of a transposing read touches fall in four disjoint 16-bank
  // quarters (64 banks of 4 bytes)
  constexpr int CPK = RK / 8 + 1;
  constexpr int CPV = (RV / 8) % 16 <= 4 ? RV / 8 + (4 - (RV / 8) % 16) : (RV / 8) % 16 <= 12 ? RV / 8 + (12 - (RV / 8) % 16) : RV / 8 + (20 - (RV / 8) % 16);
  constexpr int SK = 16 * CPK, SV = 16 * CPV, SKH = 2 * DH + 16;  // row strides, bytes
  constexpr int VOFF = KT * SK;
  constexpr int NPOS = (KT * (CPK + CPV) + 63) / 64 * 64;  // copied chunks per tile (pad included)
  constexpr int NCP = NPOS / 64;                            // wave-wide copies per tile
  constexpr int NROPE = DH / 64;                            // 256-byte copies of the RoPE row
  constexpr int NJOB = NCP + NROPE;
  // Copies per wave and tile, the same for every wave (the last jobs repeat
  // latent copies), so that the compiler's count of outstanding copies is exact.
  constexpr int CPW = (NJOB + NW - 1) / NW;
  constexpr int ROPE_OFF = NPOS * 16;                       // (cos, sin) row of the tile's first position
  constexpr int SLOT = ROPE_OFF + 4 * DH;
  // Tile y is copied in step y - 5 into slot y % 6, rebuilt in step y - 1 and
  // attended in step y.  At the end of step x a wave may still have in flight
  // the copies of steps x - 2 .. x.
  constexpr int NSLOT = 6, DIST = NSLOT - 1;
  constexpr int VM_KEEP = 3 * CPW;
  constexpr int PTC = 512;  // page-table entries staged per chunk
  static_assert(RK % 16 == 0 && RV % 32 == 0 && (DH == 64 || DH == 128), "shape");
  static_assert(QF * 32 * NW == QB && NTW >= 1 && NTW * NW == 2 * NDB, "wave split");
  static_assert(CPW <= 8 && VM_KEEP < 64 && NW * CPW - NJOB <= NCP && (CPW - 1) * NW <= NCP, "copy split");

  __shared__ __attribute__((aligned(16))) char s_c0[SLOT], s_c1[SLOT], s_c2[SLOT], s_c3[SLOT], s_c4[SLOT], s_c5[SLOT];
  __shared__ __attribute__((aligned(16))) char s_k0[KT * SKH], s_k1[KT * SKH];  // rotated K, bf16
  __shared__ __attribute__((aligned(16))) char s_wk[NDB * 32 * SK];               // W_up,k,t rows of each dim block and its partner
  __shared__ int s_pt[2][PTC];  // page-table entries: chunk c (PTC logical pages) in s_pt[c % 2]

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g16 = lane >> 4;  // lane coordinates of the 16x16 products
  const int n32 = lane & 31, g32 = lane >> 5;  // lane coordinates of the 32x32 products

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

  const int w0 = r0 + QW * w;
  const int qmin = (int)(p0 + max(w0, v0));  // the wave's first query position

  // ---- prologue: Q' = scale log2(e) R(p) q as bf16 B-operands ----
  // qop[f][ks]: lane (n32, g32) = query w0 + 32 f + n32, dims 16 ks + 8 g32 .. + 7.
  u32x4 qop[QF][KSQ];
  int qpos[QF];
  bool qok[QF];
#pragma unroll
  for (int f = 0; f < QF; ++f) {
    const int iq = w0 + 32 * f + n32;
    qok[f] = iq >= v0 && iq < v1;
    qpos[f] = qok[f] ? (int)(p0 + iq) : 0;
    const uint16_t *qrow = (const uint16_t *)a.q + (((long long)b * nq + (qok[f] ? iq : v0)) * a.H + h) * DH;
    const float *rq = a.rope + (long long)qpos[f] * DH;
#pragma unroll
    for (int ks = 0; ks < KSQ / 2; ++ks) {
      const int d0 = 16 * ks + 8 * g32;
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
      qop[f][ks + KSQ / 2] = pb;
    }
  }

  // ---- this wave's share of the K rebuild: W_up,k,t rows in LDS, mu_k in registers ----
  // Wave w rebuilds dims dlo .. + 15 and their RoPE partners dlo + d/2 .. + 15
  // (block 1) at tokens 16 tau .. + 15 of each tile, tau = tau0 .. tau0 + NTW - 1.
  const int dlo = 16 * (w % (HALF / 16));
  const int tau0 = NTW * (w / (HALF / 16));
  f32x4 muk[2];
  char *const wk_lds = s_wk + 32 * (dlo / 16) * SK;  // this wave's rows: block j at 16 j
  {
    const char *wkh = a.wup_k + (long long)h * a.wup_head_stride_k * 2;
    const uint16_t *mkh = (const uint16_t *)a.mu_k + (long long)h * a.mu_head_stride;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int dblk = dlo + j * HALF;
      const char *wrow = wkh + (long long)(dblk + n16) * RK * 2;
      if (w < NDB)  // the first wave of each dim block stores its rows (read after the next barrier)
        for (int c = g16; c < RK / 8; c += 4)
          *(u32x4 *)(wk_lds + (16 * j + n16) * SK + 16 * c) = *(const u32x4 *)(wrow + 16 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) muk[j][i] = bf16_to_f32(mkh[dblk + 4 * g16 + i]);
    }
  }

  // ---- page table, tile copies ----
  const int *pt_row = a.page_table + (long long)b * a.max_pages;
  const char *kpool = a.k_pool + (long long)h * a.pool_head_stride_k * 2;
  const char *vpool = a.v_pool + (long long)h * a.pool_head_stride_v * 2;
  const long long pstride_k = a.pool_page_stride_k * 2, pstride_v = a.pool_page_stride_v * 2;
  int bad_lp = 0x7FFFFFFF;  // first logical page with an out-of-range table entry

  auto fill_pt = [&](int c) {
    for (int i = tid; i < PTC; i += NTH) {
      const int lp = PTC * c + i;
      s_pt[c & 1][i] = lp < npg ? pt_row[lp] : 0;
    }
  };

  // Job J = it NW + w of a tile: J < NCP copies chunk positions 64 J .. + 63 of
  // the slot (lane position pos -> (c_v?, row, chunk) is the same for every
  // tile; pad positions copy the row's first chunk, never read); NCP <= J < NJOB
  // copies part J - NCP of the RoPE row; J >= NJOB repeats latent job J - NJOB.
  // cp[it] packs the byte offset within the page (from the K or V page base,
  // bits 0..15), the tile row (0..31, or 32 past the rows; bits 16..21) and
  // whether the chunk is c_v (bit 22).
  auto job_pos = [&](int it) {
    const int J = it * NW + w;
    return J < NCP ? J : (J >= NJOB ? J - NJOB : -1);
  };
  int cp[CPW];
#pragma unroll
  for (int it = 0; it < CPW; ++it) {
    const int pos = 64 * max(job_pos(it), 0) + lane;
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
    cp[it] = off | (row << 16) | (isv ? 1 << 22 : 0);
  }
  auto cp_row = [&](int it) { return (cp[it] >> 16) & 63; };
  // Direct-to-LDS copy of tile x (clamped to the last tile) into slot sb, in
  // three parts: the tile's two page-table entries (an LDS read, issued a step
  // before they are needed), the page bases, and the CPW copy instructions,
  // which the main loop spreads over its step (a wave that issued them back to
  // back waited on the copy queue).
  auto tile_pages = [&](int x, int &e0, int &e1) {
    x = min(x, nt - 1);
    const int l0 = min(2 * x, npg - 1), l1 = min(2 * x + 1, npg - 1);
    e0 = s_pt[(l0 / PTC) & 1][l0 % PTC];
    e1 = s_pt[(l1 / PTC) & 1][l1 % PTC];
  };
  struct CopyBase {
    uint64_t k0, k1, v0, v1;
    int okm;  // page-validity bits (bit 0: first page, bit 1: second)
  };
  auto copy_base = [&](int x, int e0v, int e1v) -> CopyBase {
    x = min(x, nt - 1);
    const int l0 = min(2 * x, npg - 1), l1 = min(2 * x + 1, npg - 1);
    const int e0 = __builtin_amdgcn_readfirstlane(e0v), e1 = __builtin_amdgcn_readfirstlane(e1v);
    const bool ok0 = e0 >= 0 && e0 < a.num_pages, ok1 = e1 >= 0 && e1 < a.num_pages;
    if (!ok0) bad_lp = min(bad_lp, l0);
    if (!ok1) bad_lp = min(bad_lp, l1);
    const long long pg0 = ok0 ? e0 : 0, pg1 = ok1 ? e1 : 0;
    uint64_t k0 = (uint64_t)(kpool + pg0 * pstride_k), k1 = (uint64_t)(kpool + pg1 * pstride_k);
    uint64_t v0 = (uint64_t)(vpool + pg0 * pstride_v), v1 = (uint64_t)(vpool + pg1 * pstride_v);
    // (opaque, so that each lane selects one of the four page addresses and adds
    // its offset, rather than the compiler multiplying a selected page number)
    asm volatile("" : "+s"(k0), "+s"(k1), "+s"(v0), "+s"(v1));
    return CopyBase{k0, k1, v0, v1, (ok0 ? 1 : 0) | (ok1 ? 2 : 0)};
  };
  auto copy_job = [&](int x, char *sb, const CopyBase &cb, int it) {
    x = min(x, nt - 1);
    const int J = it * NW + w;
    const bool rope_job = it + 1 == CPW && J >= NCP && J < NJOB;
    if (!rope_job) {
      const int jp = J < NCP ? J : J - NJOB;
      const bool p1 = ((cp[it] >> 20) & 3) == 1;  // rows 16..31
      const bool isv = (cp[it] >> 22) != 0;
      const uint64_t pa = isv ? cb.v0 : cb.k0, pb = isv ? cb.v1 : cb.k1;
      dma_lds16((const char *)((p1 ? pb : pa) + (uint32_t)(cp[it] & 0xFFFF)), lds_addr(sb, 1024 * jp));
    } else {
      const int k = J - NCP;
      dma_lds4(a.rope + (long long)KT * x * DH + 64 * k + lane, lds_addr(sb, ROPE_OFF + 256 * k));
    }
  };
  // copy jobs it with it * 3 / CPW == point: three insertion points per step
  auto copy_jobs_at = [&](int x, char *sb, const CopyBase &cb, int point) {
#pragma unroll
    for (int it = 0; it < CPW; ++it)
      if (it * 3 / CPW == point) copy_job(x, sb, cb, it);
  };
  auto copy_tile = [&](int x, char *sb) -> int {
    int e0, e1;
    tile_pages(x, e0, e1);
    const CopyBase cb = copy_base(x, e0, e1);
#pragma unroll
    for (int it = 0; it < CPW; ++it) copy_job(x, sb, cb, it);
    return cb.okm;
  };
  // Clear the rows of tile x (in slot sb, copies landed) that are past kend or
  // come from a bad page.
  auto clear_tile = [&](int x, char *sb, int okm) {
#pragma unroll
    for (int it = 0; it < CPW; ++it) {
      if (it * NW + w < NCP) {
        const int r = cp_row(it);
        if (r < 32 && (KT * x + r >= kend || !((okm >> (r >> 4)) & 1)))
          *(u32x4 *)(sb + 16 * (64 * (it * NW + w) + lane)) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto needs_clear = [&](int y, int okm) { return y < nt && (okm != 3 || (y == nt - 1 && kend % KT != 0)); };

  // RoPE of this wave's rebuild share: the angle of position 32 y + r is the
  // sum of the angle of 32 y (a row copied with the tile) and that of r, the
  // lane's row in the tile (held here: (cos, sin) of pairs dlo + 4 g16 + i at
  // r = 16 tau + n16, tau = tau0 + t; rows past the table only serve tokens
  // past the context, which are masked).  No global loads in the main loop
  // besides the tile copies, so that the compiler's waits stay on them.
  float ro_c[NTW][4], ro_s[NTW][4];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int r = min(16 * (tau0 + t) + n16, a.rope_len - 1);
    const float *rr = a.rope + (long long)r * DH + 2 * (dlo + 4 * g16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ro_c[t][i] = rr[2 * i];
      ro_s[t][i] = rr[2 * i + 1];
    }
  }
  // K^T blocks (16 dims x 16 tokens) of the tile in slot sb, plus mu: kacc[2 t + j]
  // gives lane (n16, g16) dims dlo + j d/2 + 4 g16 .. + 3 at token 16 (tau0 + t) + n16.
  const int ck_lane = (16 * tau0 + n16) * SK + 16 * g16;
  const int wa_lane = 32 * (dlo / 16) * SK + n16 * SK + 16 * g16;
  auto rebuild_mfma = [&](const char *sb, f32x4 (&kacc)[2 * NTW]) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      u32x4 bop[KSW];
#pragma unroll
      for (int ks = 0; ks < KS32; ++ks) bop[ks] = *(const u32x4 *)(sb + (ck_lane + 16 * t * SK + 64 * ks));
#pragma unroll
      for (int j = 0; j < 2; ++j) kacc[2 * t + j] = muk[j];
#pragma unroll
      for (int ks = 0; ks < KS32; ++ks)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          kacc[2 * t + j] = mfma16(*(const u32x4 *)(s_wk + (wa_lane + 16 * j * SK + 64 * ks)), bop[ks], kacc[2 * t + j]);
      if constexpr (TAIL) {
        const bf16x4 bt = __builtin_bit_cast(bf16x4, *(const u32x2 *)(sb + (ck_lane + 16 * t * SK + 64 * KS32 - 8 * g16)));
#pragma unroll
        for (int j = 0; j < 2; ++j)
          kacc[2 * t + j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              __builtin_bit_cast(bf16x4, *(const u32x2 *)(s_wk + (wa_lane + 16 * j * SK + 64 * KS32 - 8 * g16))), bt,
              kacc[2 * t + j], 0, 0, 0);
      }
    }
  };
  // RoPE on the rebuilt blocks, bf16 rows of K buffer kb.
  const int kw_lane = (16 * tau0 + n16) * SKH + (dlo + 4 * g16) * 2;
  const int rb_lane = ROPE_OFF + 8 * (dlo + 4 * g16);
  auto rebuild_store = [&](const f32x4 (&kacc)[2 * NTW], const char *sb, char *kb) {
    const f32x4 b01 = *(const f32x4 *)(sb + rb_lane), b23 = *(const f32x4 *)(sb + (rb_lane + 16));
    const float bc[4] = {b01[0], b01[2], b23[0], b23[2]}, bs[4] = {b01[1], b01[3], b23[1], b23[3]};
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      float ra[4], rb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float c = bc[i] * ro_c[t][i] - bs[i] * ro_s[t][i];
        const float s = bs[i] * ro_c[t][i] + bc[i] * ro_s[t][i];
        const float ka = kacc[2 * t][i], kb2 = kacc[2 * t + 1][i];
        ra[i] = ka * c - kb2 * s;
        rb[i] = ka * s + kb2 * c;
      }
      *(u32x2 *)(kb + (kw_lane + 16 * t * SKH)) = u32x2{cvt2(ra[0], ra[1]), cvt2(ra[2], ra[3])};
      *(u32x2 *)(kb + (kw_lane + 16 * t * SKH + HALF * 2)) = u32x2{cvt2(rb[0], rb[1]), cvt2(rb[2], rb[3])};
    }
  };
  // S^T = K Q'^T of the tile in K buffer kb: lane (n32, g32) gets query 32 f + n32
  // at tokens 8 (e / 4) + 4 g32 + e % 4 (element e).
  const int kr_lane = n32 * SKH + 16 * g32;

  // ---- softmax state and latent-space value sums ----
  // The weights of a query use one fixed reference m_ref: the max of its scores
  // in the first tile (first pass), so the accumulators are never rescaled.  A
  // weight is 2^(s - m_ref); should any score exceed m_ref by more than 64 or
  // the sum of weights not be finite, the block runs again with m_ref = the
  // exact max of each query's scores (second pass), where every weight is <= 1.
  // The shift cancels in the normalised result.
  f32x16 o[QF][NRB];
  float m_ref[QF] = {}, l_run[QF], m_run[QF];
  // Causal mask of tile x's scores and the running max of this lane's scores.
  auto softmax_max = [&](int x, f32x16 (&s)[QF]) {
    if (KT * x + KT - 1 > qmin) {
#pragma unroll
      for (int f = 0; f < QF; ++f)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (KT * x + 8 * (e >> 2) + 4 * g32 + (e & 3) > qpos[f]) s[f][e] = -INFINITY;
    }
#pragma unroll
    for (int f = 0; f < QF; ++f) {
      float m = fmaxf(fmaxf(s[f][0], s[f][1]), s[f][2]);
#pragma unroll
      for (int e = 3; e < 15; e += 2) m = fmaxf(fmaxf(m, s[f][e]), s[f][e + 1]);
      m_run[f] = fmaxf(fmaxf(m, s[f][15]), m_run[f]);
    }
  };
  // Weights of tile x and the latent-space value sums, one 16-token K-step at a
  // time.  The weights of K-step k are bf16 B-operands holding accumulator
  // elements 8 k .. + 7, i.e. K index 8 g32 + e <-> token 16 k + 8 (e / 4) +
  // 4 g32 + e % 4; the sums of weights are taken of the bf16 values.
  // O^T[r][q] += C_v^T[r][t] P^T[t][q] reads the c_v rows of the tile (slot sb)
  // transposed: lane (m, g32) of K-step k gets rows 16 k + 8 h + 4 g32 + 0..3.
  // (Each LDS address is one integer offset from its slot: the compiler loses
  // the LDS alias scopes on long address chains.)
  const int vb_lane = VOFF + (4 * g32 + ((lane & 15) >> 2)) * SV + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
  auto weights = [&](const f32x16 (&s)[QF], int k, u32x4 (&pop)[QF]) {
    const uint32_t one2 = 0x3F803F80u;  // (1, 1) in bf16
#pragma unroll
    for (int f = 0; f < QF; ++f) {
      const float mu = m_ref[f];
      float lsum = l_run[f];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t pe = cvt2(fast_exp2(s[f][8 * k + 2 * e] - mu), fast_exp2(s[f][8 * k + 2 * e + 1] - mu));
        pop[f][e] = pe;
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pe), __builtin_bit_cast(bf16x2, one2), lsum, false);
      }
      l_run[f] = lsum;
    }
  };
  auto cv_operands = [&](const char *sb, int k, u32x4 (&av)[NRB]) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const u32x2 lo2 = lds_read_tr(sb + (vb_lane + 16 * k * SV + 64 * rb));
      const u32x2 hi2 = lds_read_tr(sb + (vb_lane + (16 * k + 8) * SV + 64 * rb));
      av[rb] = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
    }
  };
  auto value_sums = [&](const u32x4 (&av)[NRB], const u32x4 (&pop)[QF]) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int f = 0; f < QF; ++f) o[f][rb] = mfma32(av[rb], pop[f], o[f][rb]);
  };

  // ---- main loop ----
  // Step x: clear tile x + 1 if it needs it, copy tile x + 5, scores of tile x,
  // mask and max, weights and latent-space value sums of tile x, rebuild of
  // tile x + 1, barrier.  Tile y lives in slot y % 6 and K buffer y % 2.  The
  // LDS operands of each matrix phase are loaded in a batch ahead of it
  // (scheduling fences keep the compiler from pairing each load with its
  // product, which would expose the LDS latency at every product).
  // Every load the compiler sees lands before the first tile copy: its own waits
  // count only those loads, so none of them may be left for the main loop.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt (7) and lgkmcnt (15) not waited
  int okm0 = 3, okm1 = 3, okm2 = 3, okm3 = 3, okm4 = 3, okm5 = 3;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
  for (int f = 0; f < QF; ++f) {
    l_run[f] = 0.f;
    m_run[f] = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) o[f][rb] = f32x16{};
  }
  if (nt > 0) {
    fill_pt(0);
    if (npg > PTC) fill_pt(1);
    __syncthreads();  // s_pt
    okm0 = copy_tile(0, s_c0);
    okm1 = copy_tile(1, s_c1);
    okm2 = copy_tile(2, s_c2);
    okm3 = copy_tile(3, s_c3);
    okm4 = copy_tile(4, s_c4);
    barrier_vm<4 * CPW>();  // tile 0
    if (needs_clear(0, okm0)) clear_tile(0, s_c0, okm0);
    barrier_vm<4 * CPW>();
    f32x4 kacc[2 * NTW];
    rebuild_mfma(s_c0, kacc);
    rebuild_store(kacc, s_c0, s_k0);
    barrier_vm<3 * CPW>();  // tile 1, K of tile 0
  }
  int pe0 = 0, pe1 = 0;  // page-table entries of the next step's copy (read a step ahead)
  tile_pages(DIST, pe0, pe1);
  auto step = [&](int x, const char *sx, char *sx1, char *sxd, int okx1, int &okxd, const char *kb0, char *kb1) {
    if (needs_clear(x + 1, okx1)) {
      clear_tile(x + 1, sx1, okx1);
      barrier_vm<63>();
    }
    if ((2 * (x + DIST)) % PTC == 0 && 2 * (x + DIST) + PTC < npg) fill_pt(2 * (x + DIST) / PTC + 1);
    const CopyBase cbx = copy_base(x + DIST, pe0, pe1);
    okxd = cbx.okm;
    tile_pages(x + DIST + 1, pe0, pe1);
    if (x >= nt) {  // past the last tile: the copies only
#pragma unroll
      for (int point = 0; point < 3; ++point) copy_jobs_at(x + DIST, sxd, cbx, point);
    }
    if (x < nt) {
      u32x4 ak[KSQ];
#pragma unroll
      for (int ks = 0; ks < KSQ; ++ks) ak[ks] = *(const u32x4 *)(kb0 + (kr_lane + 32 * ks));
      __builtin_amdgcn_sched_barrier(0);
      f32x16 sc[QF];
#pragma unroll
      for (int ks = 0; ks < KSQ; ++ks)
#pragma unroll
        for (int f = 0; f < QF; ++f) sc[f] = mfma32(ak[ks], qop[f][ks], ks == 0 ? f32x16{} : sc[f]);
      copy_jobs_at(x + DIST, sxd, cbx, 0);
      u32x4 av0[NRB];
      cv_operands(sx, 0, av0);
      __builtin_amdgcn_sched_barrier(0);
      softmax_max(x, sc);
      if (pass == 0 && x == 0) {
#pragma unroll
        for (int f = 0; f < QF; ++f) m_ref[f] = max_across_halves(m_run[f]);
      }
      u32x4 pop0[QF], pop1[QF], av1[NRB];
      weights(sc, 0, pop0);
      cv_operands(sx, 1, av1);
      __builtin_amdgcn_sched_barrier(0);
      copy_jobs_at(x + DIST, sxd, cbx, 1);
      value_sums(av0, pop0);
      weights(sc, 1, pop1);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 kacc[2 * NTW];
      value_sums(av1, pop1);
      copy_jobs_at(x + DIST, sxd, cbx, 2);
      rebuild_mfma(sx1, kacc);
      __builtin_amdgcn_sched_barrier(0);
      rebuild_store(kacc, sx1, kb1);
    }
    barrier_vm<VM_KEEP>();
  };
  // Whole groups of six steps; the steps past the last tile only copy (clamped
  // tiles) and meet.  Every path through a group issues the same copies, so
  // that the compiler's count of outstanding copies stays exact and its waits
  // stay on them.
  for (int x = 0; x < nt; x += 6) {
    step(x, s_c0, s_c1, s_c5, okm1, okm5, s_k0, s_k1);
    step(x + 1, s_c1, s_c2, s_c0, okm2, okm0, s_k1, s_k0);
    step(x + 2, s_c2, s_c3, s_c1, okm3, okm1, s_k0, s_k1);
    step(x + 3, s_c3, s_c4, s_c2, okm4, okm2, s_k1, s_k0);
    step(x + 4, s_c4, s_c5, s_c3, okm5, okm3, s_k0, s_k1);
    step(x + 5, s_c5, s_c0, s_c4, okm0, okm4, s_k1, s_k0);
  }
  barrier_vm<0>();  // no copy in flight past the loop
  // Second pass if a weight could have left the safe range (a workgroup-wide decision).
  if (pass == 1) break;
  bool redo = false;
#pragma unroll
  for (int f = 0; f < QF; ++f) {
    const float z = sum_across_halves(l_run[f]);
    redo |= m_run[f] > m_ref[f] + 64.f || !(fabsf(z) <= 3.0e38f);
  }
  if (tid == 0) s_pt[0][0] = 0;
  __syncthreads();
  if (__builtin_amdgcn_ballot_w64(redo) && lane == 0) s_pt[0][0] = 1;
  __syncthreads();
  if (!__builtin_amdgcn_readfirstlane(s_pt[0][0])) break;
  __syncthreads();
#pragma unroll
  for (int f = 0; f < QF; ++f) m_ref[f] = max_across_halves(m_run[f]);
  }

  // ---- epilogue: normalise, up-project with W_up,v, add mu_v ----
  if (bad_lp != 0x7FFFFFFF) errbits |= LLA_DEVERR_PAGE;
  if (errbits && tid == 0) atomicOr(a.err, errbits);

  // B-operands: K-step k holds r = 16 k + 8 (e / 4) + 4 g32 + e % 4 (elements 8 (k % 2) .. + 7 of block k / 2)
  u32x4 bup[QF][KSV];
#pragma unroll
  for (int f = 0; f < QF; ++f) {
    const float z = sum_across_halves(l_run[f]);
    const bool bad = !qok[f] || (long long)qpos[f] >= (long long)kPage * bad_lp;
    const float inv = bad ? __builtin_nanf("") : 1.f / z;
#pragma unroll
    for (int k = 0; k < KSV; ++k) {
      const f32x16 &u = o[f][k >> 1];
      const int e0 = 8 * (k & 1);
      bup[f][k] = u32x4{cvt2(u[e0] * inv, u[e0 + 1] * inv), cvt2(u[e0 + 2] * inv, u[e0 + 3] * inv),
                        cvt2(u[e0 + 4] * inv, u[e0 + 5] * inv), cvt2(u[e0 + 6] * inv, u[e0 + 7] * inv)};
    }
  }
  const char *wvh = a.wup_v + (long long)h * a.wup_head_stride_v * 2;
  const uint16_t *mvh = (const uint16_t *)a.mu_v + (long long)h * a.mu_head_stride;
#pragma unroll 1
  for (int db = 0; db < DH / 32; ++db) {
    f32x16 acc[QF];
#pragma unroll
    for (int f = 0; f < QF; ++f) acc[f] = f32x16{};
    const char *wr = wvh + ((long long)(32 * db + n32) * RV + 4 * g32) * 2;
#pragma unroll
    for (int k = 0; k < KSV; ++k) {
      const u32x2 wlo = *(const u32x2 *)(wr + 32 * k);
      const u32x2 whi = *(const u32x2 *)(wr + 32 * k + 16);
      const u32x4 av = u32x4{wlo[0], wlo[1], whi[0], whi[1]};
#pragma unroll
      for (int f = 0; f < QF; ++f) acc[f] = mfma32(av, bup[f][k], acc[f]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * db + 8 * j + 4 * g32;
      const u32x2 mu2 = *(const u32x2 *)(mvh + d);
#pragma unroll
      for (int f = 0; f < QF; ++f) {
        const int iq = w0 + 32 * f + n32;
        if (iq < r1) {
          uint16_t *orow = (uint16_t *)a.out + (((long long)b * nq + iq) * a.H + h) * DH + d;
          *(u32x2 *)orow = u32x2{cvt2(acc[f][4 * j] + bf16_lo(mu2[0]), acc[f][4 * j + 1] + bf16_hi(mu2[0])),
                                 cvt2(acc[f][4 * j + 2] + bf16_lo(mu2[1]), acc[f][4 * j + 3] + bf16_hi(mu2[1]))};
        }
      }
    }
  }
}

// ---------------------------------------------------------------- dispatch

// Waves per workgroup (256 queries): two per SIMD at d = 128, one at d = 64.
#ifndef PREFILL_WAVES128
#define PREFILL_WAVES128 8
#endif
#define PREFILL_WAVES(DH) ((DH) == 128 ? PREFILL_WAVES128 : 4)

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
    hipLaunchKernelGGL((prefill_kernel<DH, RK, RV, PREFILL_WAVES(DH)>), dim3((unsigned)grid),              \
                       dim3(64 * PREFILL_WAVES(DH)), 0, stream, a);                                            \
    return hipGetLastError();                                                                        \
  }
  LLA_PREFILL_SHAPES(X)
#undef X
  return hipErrorInvalidConfiguration;
}

}  // namespace lla
