// Encode + append, eq. (2) of the cc.laoqi.cc close reading (方法 item 1) and
// the gist.science "Kernmechanismus": c = (x - mu) W_down over the
// loop-concatenated pre-RoPE vector x = [x_1; ...; x_T], written to the paged
// latent pool at the slot of logical position pos0[b] + n.
//
// Computed as x W_down - (mu W_down): mu W_down is a per-(layer, group)
// constant (first kernel, fp32), the contraction accumulates exact products in
// fp32, and the result is rounded once to the storage type.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {

template <bool BF>
__device__ __forceinline__ float ldx(const char *p, long long i) {
  if constexpr (BF) return bf16_to_f32(((const uint16_t *)p)[i]);
  else return ((const float *)p)[i];
}

// muw[li][grp][kv ? RK + r : r] = sum_i mu[i] W_down[i][r], fp32: a constant of
// (layer, latent group), computed once per call and shared by every token tile.
// The rows of W_down are cut into muw_parts ranges of kMuwRows rows, summed by
// separate workgroups (one per (range, group), layer, K|V) into muw_part; a
// second launch adds the ranges in fixed order.  Within a range, wave w sums
// rows w, w + 4, ... (lanes over r, coalesced rows of W_down) and the 4 wave
// sums are added in fixed order.
constexpr int kMuwRows = 64;

int encode_muw_parts(int width) { return (width + kMuwRows - 1) / kMuwRows; }

template <bool BF>
__global__ __launch_bounds__(256) void encode_muw_kernel(EncodeArgs a, int RK, int RV) {
  __shared__ float part[4][256];
  const int grp = blockIdx.x % a.groups, pr = blockIdx.x / a.groups;
  const int li = blockIdx.y, kv = blockIdx.z;
  const int R = kv ? RV : RK;
  const int esz = BF ? 2 : 4;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long long gl = (long long)li * a.groups + grp;  // relative to layer0
  const char *mu = (kv ? a.mu_v : a.mu_k) + gl * a.width * esz;
  const char *wd = (kv ? a.wd_v : a.wd_k) + gl * a.width * (long long)R * esz;
  const int i0 = pr * kMuwRows, i1 = min(i0 + kMuwRows, a.width);
  float *dst = a.muw_part + ((long long)pr * a.n_layers * a.groups + gl) * (RK + RV) + (kv ? RK : 0);
  for (int r0 = 0; r0 < R; r0 += 256) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i = i0 + w; i < i1; i += 4) {
      const float m = ldx<BF>(mu, i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = r0 + lane + 64 * j;
        if (r < R) acc[j] = fmaf(m, ldx<BF>(wd, (long long)i * R + r), acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) part[w][lane + 64 * j] = acc[j];
    __syncthreads();
    const int r = r0 + threadIdx.x;
    if (r < R) dst[r] = ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) + part[3][threadIdx.x];
    __syncthreads();
  }
}

// muw = sum over the row ranges, in range order.  One thread per
// (layer, group, column).
__global__ __launch_bounds__(256) void encode_muw_reduce_kernel(EncodeArgs a) {
  const long long n = (long long)a.n_layers * a.groups * a.muw_stride;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  float s = 0.f;
  // unrolled so that the loads of 16 ranges are in flight together; the sum
  // keeps range order
#pragma unroll 16
  for (int pr = 0; pr < a.muw_parts; ++pr) s += a.muw_part[(long long)pr * n + idx];
  a.muw[idx] = s;
}

namespace {
template <bool BF>
hipError_t launch_muw(int r_k, int r_v, const EncodeArgs &a, hipStream_t stream) {
  const dim3 g1((unsigned)(a.groups * a.muw_parts), a.n_layers, 2);
  hipLaunchKernelGGL(encode_muw_kernel<BF>, g1, dim3(256), 0, stream, a, r_k, r_v);
  const long long n = (long long)a.n_layers * a.groups * a.muw_stride;
  hipLaunchKernelGGL(encode_muw_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}
}  // namespace

// One workgroup per (16-token tile, group, layer*2 + kv).
template <bool BF>
__global__ __launch_bounds__(256) void encode_append_kernel(EncodeArgs a, int RK, int RV) {
  constexpr int TT = 16;
  const int grp = blockIdx.y, li = blockIdx.z >> 1, kv = blockIdx.z & 1;
  const int R = kv ? RV : RK;
  const int esz = BF ? 2 : 4;
  const long long tokens = (long long)a.batch * a.n_new;
  const long long tok0 = (long long)blockIdx.x * TT;
  const long long gl = (long long)li * a.groups + grp;
  const char *x = kv ? a.x_v : a.x_k;
  const char *wd = (kv ? a.wd_v : a.wd_k) + gl * a.width * (long long)R * esz;
  char *pool = (kv ? a.v_pool : a.k_pool) + (long long)li * (kv ? a.pool_layer_stride_v : a.pool_layer_stride_k) * esz;
  const long long pstride = kv ? a.pool_page_stride_v : a.pool_page_stride_k;
  const long long hstride = kv ? a.pool_head_stride_v : a.pool_head_stride_k;
  const float *muw = a.muw + gl * (RK + RV) + (kv ? RK : 0);
  for (int idx = threadIdx.x; idx < TT * R; idx += blockDim.x) {
    const long long tok = tok0 + idx / R;
    const int r = idx % R;
    if (tok >= tokens) continue;
    const int b = (int)(tok / a.n_new), n = (int)(tok % a.n_new);
    const long long pos = (long long)a.pos0[b] + n;
    if (pos < 0 || pos >= (long long)a.max_pages * kPage) {
      atomicOr(a.err, LLA_DEVERR_APPEND);
      continue;
    }
    const int page = a.page_table[(long long)b * a.max_pages + pos / kPage];
    if (page < 0 || page >= a.num_pages) {
      atomicOr(a.err, LLA_DEVERR_PAGE);
      continue;
    }
    const char *xr = x + ((((long long)li * a.batch + b) * a.n_new + n) * a.groups + grp) * a.width * esz;
    float acc = 0.f;
    for (int i = 0; i < a.width; ++i) acc = fmaf(ldx<BF>(xr, i), ldx<BF>(wd, (long long)i * R + r), acc);
    acc -= muw[r];
    const long long off = (long long)page * pstride + grp * hstride + (pos % kPage) * R + r;
    if constexpr (BF) ((uint16_t *)pool)[off] = (uint16_t)f32_to_bf16(acc);
    else ((float *)pool)[off] = acc;
  }
}

// ---------------------------------------------------------------- MFMA path (bf16)
//
// Per (layer, latent group, K|V) the encoder is a plain GEMM,
//   C[tokens x r] = X[tokens x width] W_down[width x r] - 1 (mu W_down),
// on v_mfma_f32_16x16x32_bf16.  A workgroup (8 waves) takes 256 tokens (128
// for r > 160); wave w owns two 16-row tiles (one) and all r columns.  The
// contraction runs over chunks of 64 rows of W_down (32 for r > 160):
//  * x: each wave loads its rows x chunk bytes in address order (for 64-row
//    chunks one load instruction covers 8 whole 128-byte row pieces), two
//    chunks ahead in registers, and passes them through its own LDS region
//    (16-byte slots XOR-swizzled by row) into the A-operand layout;
//  * W_down: the chunk's rows are copied as stored (r contiguous; rows padded
//    so that the transposing reads below hit distinct banks) straight into
//    LDS by the 8 waves together (global_load_lds_dwordx4), two chunks ahead
//    in three buffers, one barrier per chunk;
//  * B-operands come from ds_read_b64_tr_b16, which hands lane (g, n) column n
//    of four consecutive rows: K-slot 8 g + 4 h + e of K-step s is chunk row
//    32 s + 16 h + 4 g + e, on both operands.
// mu W_down comes from encode_muw_kernel (once per call).  The result (minus
// mu W_down, rounded once to bf16) goes through LDS and leaves as 16-byte
// stores into the paged pool.  Workgroups are persistent (at most one per CU)
// and walk (token tile, group, layer) tiles; a tile's output stores drain
// while the next tile's first two chunks load.
namespace {
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

// Transposing LDS read: within each 16-lane group, lane i receives element i % 4
// of the 8-byte rows addressed by lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4.
__device__ __forceinline__ u32x2 lds_read_tr(const char *p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
  return __builtin_bit_cast(u32x2, v);
}

// 16 bytes per lane from global memory straight into LDS at byte address
// lds + 16 x lane (global_load_lds_dwordx4).  Written as assembly on purpose:
// the compiler does not see that it writes LDS, so it does not hold every
// later LDS access of the wave until all copies in flight have landed (which
// undoes any prefetch); callers order the copies with explicit vmcnt waits
// and barriers instead.  No register is written; M0 is set inside the block
// (the kernels of this file keep nothing else in M0, which the build checks in
// their assembly; hence the silenced warning about clobbering a reserved
// register).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const void *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src) : "memory", "m0");
}
#pragma clang diagnostic pop
// Wave-uniform LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(__attribute__((address_space(3))) const char *)p);
}

// Wait until at most VM vector-memory operations of this wave are outstanding,
// then meet the other waves.
template <int VM>
__device__ __forceinline__ void barrier_vm() {
  static_assert(VM >= 0 && VM < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(((VM >> 4) << 14) | (VM & 15) | 0x70);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
}  // namespace

// 16-row tiles per wave (registers bound it), tokens per workgroup and W_down
// rows per chunk
__host__ __device__ constexpr int enc_tpw(int r) { return r <= 160 ? 2 : 1; }
__host__ __device__ constexpr int enc_tok(int r) { return 128 * enc_tpw(r); }
__host__ __device__ constexpr int enc_kc(int r) { return r <= 160 ? 64 : 32; }

template <int R>
__global__ __launch_bounds__(512) void encode_mfma_kernel(EncodeArgs a, int kv) {
  constexpr int TPW = enc_tpw(R), TOK = enc_tok(R), KC = enc_kc(R);
  constexpr int XP = KC / 8;                               // 16-byte pieces of a token's chunk row
  constexpr int NXI = 16 * TPW * XP / 64;                  // x load instructions per wave and chunk
  constexpr int CT = R / 16;                               // column tiles
  constexpr int PW = R / 8 + ((R / 8) % 4 == 0 ? 2 : 0);   // 16-byte pieces per LDS row of W_down
  constexpr int NWI = (KC * PW + 511) / 512;               // W_down copy instructions per wave and chunk
  constexpr int WBUF = NWI * 512 * 16;                     // bytes of one W_down buffer
  constexpr int XW = 16 * TPW * KC * 2;                    // bytes of a wave's x region
  static_assert(R % 16 == 0 && R <= 256 && KC % 32 == 0 && (16 * TPW * XP) % 64 == 0, "r");
  // The x slots double as the output staging area at the end of a tile.
  __shared__ __attribute__((aligned(16))) char s_xo[8 * XW > TOK * R * 2 ? 8 * XW : TOK * R * 2];
  __shared__ __attribute__((aligned(16))) char s_w0[WBUF], s_w1[WBUF], s_w2[WBUF];
  __shared__ long long s_off[2][TOK];  // per tile parity: element offset of each token's latent row, -1 = dropped

  // wave index as a scalar: branches on it must be uniform scalar branches,
  // never EXEC-masked MFMAs
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, n = lane & 15;
  const long long tokens = (long long)a.batch * a.n_new;
  const long long ntt = (tokens + TOK - 1) / TOK;  // token tiles per (layer, group)
  const long long ntiles = ntt * a.groups * a.n_layers;
  const char *x = kv ? a.x_v : a.x_k;
  const uint16_t *wd_all = (const uint16_t *)(kv ? a.wd_v : a.wd_k);
  uint16_t *pool_all = (uint16_t *)(kv ? a.v_pool : a.k_pool);
  const long long lstride = kv ? a.pool_layer_stride_v : a.pool_layer_stride_k;
  const long long pstride = kv ? a.pool_page_stride_v : a.pool_page_stride_k;
  const long long hstride = kv ? a.pool_head_stride_v : a.pool_head_stride_k;

  // Tiles t = blockIdx.x, + gridDim.x, ...: token tile fastest, then group,
  // then layer, so that the workgroups running together share W_down in L2.
  struct Tile {
    long long tok0;
    int grp, li;
  };
  auto tile_of = [&](long long t) {
    Tile v;
    v.tok0 = (t % ntt) * TOK;
    const long long r = t / ntt;
    v.grp = (int)(r % a.groups);
    v.li = (int)(r / a.groups);
    return v;
  };
  // destination slot of each token of tile v (placement is integer work, checked here)
  auto place = [&](const Tile &v, long long *dst) {
    if (threadIdx.x < TOK) {
      const long long tok = v.tok0 + threadIdx.x;
      long long off = -1;
      if (tok < tokens) {
        const int b = (int)(tok / a.n_new), nn = (int)(tok % a.n_new);
        const long long pos = (long long)a.pos0[b] + nn;
        if (pos < 0 || pos >= (long long)a.max_pages * kPage) {
          atomicOr(a.err, LLA_DEVERR_APPEND);
        } else {
          const int page = a.page_table[(long long)b * a.max_pages + pos / kPage];
          if (page < 0 || page >= a.num_pages) atomicOr(a.err, LLA_DEVERR_PAGE);
          else off = (long long)page * pstride + v.grp * hstride + (pos % kPage) * R;
        }
      }
      dst[threadIdx.x] = off;
    }
  };

  // this wave's x slots: row tl, piece p at tl XP + (p ^ (tl / 2 % XP))
  char *s_x = s_xo + w * XW;

  // x loads: instruction i, lane l -> local row (64 i + l) / XP (token
  // 16 TPW w + that, clamped; dropped at the end), piece l % XP of the chunk
  const char *xsrc[NXI];
  int xslot[NXI];
  const uint16_t *wd;
  auto sources = [&](const Tile &v) {
    wd = wd_all + ((long long)v.li * a.groups + v.grp) * a.width * (long long)R;
#pragma unroll
    for (int i = 0; i < NXI; ++i) {
      const int tl = (64 * i + lane) / XP, p = lane % XP;
      long long tk = v.tok0 + 16 * TPW * w + tl;
      if (tk >= tokens) tk = tokens - 1;
      xsrc[i] = x + ((((long long)v.li * tokens + tk) * a.groups + v.grp) * a.width) * 2 + 16 * p;
    }
  };
#pragma unroll
  for (int i = 0; i < NXI; ++i) {
    const int tl = (64 * i + lane) / XP, p = lane % XP;
    xslot[i] = (tl * XP + (p ^ ((tl >> 1) & (XP - 1)))) * 16;
  }
  auto load_x = [&](int c, u32x4 (&d)[NXI]) {
#pragma unroll
    for (int i = 0; i < NXI; ++i) d[i] = __builtin_nontemporal_load((const u32x4 *)(xsrc[i] + c * (KC * 2)));
  };
  auto put_x = [&](const u32x4 (&d)[NXI]) {
#pragma unroll
    for (int i = 0; i < NXI; ++i) *(u32x4 *)(s_x + xslot[i]) = d[i];
  };
  // W_down rows c KC .. c KC + KC - 1 into buffer buf; pad and surplus slots
  // copy the chunk's first piece (never read)
  auto copy_w = [&](int c, char *dst) {
#pragma unroll
    for (int i = 0; i < NWI; ++i) {
      const int slot = (i * 8 + w) * 64 + lane;
      const int k = slot / PW, pc = slot - k * PW;
      const bool ok = k < KC && pc < R / 8;
      const uint16_t *src = wd + (long long)(c * KC + (ok ? k : 0)) * R + (ok ? 8 * pc : 0);
      copy16_to_lds(src, lds_addr(dst + (i * 8 + w) * 1024));
    }
  };

  f32x4 acc[TPW][CT];
  auto compute = [&](const char *wb) {
#pragma unroll
    for (int s = 0; s < KC / 32; ++s) {
      u32x4 av[TPW];
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        const char *xr = s_x + (16 * tt + n) * (XP * 16) + 8 * (g & 1);
        const u32x2 lo = *(const u32x2 *)(xr + ((4 * s + (g >> 1)) ^ ((n >> 1) & (XP - 1))) * 16);
        const u32x2 hi = *(const u32x2 *)(xr + ((4 * s + 2 + (g >> 1)) ^ ((n >> 1) & (XP - 1))) * 16);
        av[tt] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
      const char *wr = wb + (32 * s + 4 * g + (n >> 2)) * (PW * 16) + 8 * (n & 3);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const u32x2 lo = lds_read_tr(wr + 32 * ct);
        const u32x2 hi = lds_read_tr(wr + 16 * (PW * 16) + 32 * ct);
        const u32x4 bw = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
          acc[tt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[tt]), as_bf16x8(bw), acc[tt][ct], 0, 0, 0);
      }
    }
  };

  // Chunk c (W_down buffer c % 3): its x rows, in registers since two chunks
  // ago, go to the wave's slots.  The W_down copies of chunk c were issued
  // just before those x loads, so once only the copies and loads of chunk
  // c + 1 may be outstanding (older stores of the previous tile's output
  // complete first: vector-memory operations count down in issue order),
  // this wave's part of chunk c is in LDS; all waves meet, which also frees
  // buffer (c + 2) % 3; then the copies and x loads of chunk c + 2 are issued
  // and chunk c is multiplied.
  const int nch = a.width / KC;
  auto step = [&](int c, const char *buf, char *buf2, u32x4 (&cur)[NXI], u32x4 (&nx2)[NXI]) {
    put_x(cur);
    if (c + 1 < nch) barrier_vm<NWI + NXI>();
    else barrier_vm<0>();
    if (c + 2 < nch) {
      copy_w(c + 2, buf2);
      load_x(c + 2, nx2);
    }
    compute(buf);
  };
  u32x4 xa[NXI], xb[NXI], xc[NXI];
  // the first two chunks of a tile
  auto start = [&]() {
    copy_w(0, s_w0);
    load_x(0, xa);
    if (nch > 1) {
      copy_w(1, s_w1);
      load_x(1, xb);
    }
  };

  long long t = blockIdx.x;
  if (t >= ntiles) return;
  Tile cur = tile_of(t);
  place(cur, s_off[0]);
  sources(cur);
  start();
  for (int par = 0;; par ^= 1) {
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[tt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    int c = 0;
    for (; c + 3 <= nch; c += 3) {
      step(c, s_w0, s_w2, xa, xc);
      step(c + 1, s_w1, s_w0, xb, xa);
      step(c + 2, s_w2, s_w1, xc, xb);
    }
    if (c < nch) step(c, s_w0, s_w2, xa, xc);
    if (c + 1 < nch) step(c + 1, s_w1, s_w0, xb, xa);

    // every wave is past its last products: the x slots (output staging) and
    // the W_down buffers are free
    barrier_vm<63>();
    uint16_t *s_out = (uint16_t *)s_xo;  // [TOK][R] bf16
    const float *muw = a.muw + ((long long)cur.li * a.groups + cur.grp) * a.muw_stride + (kv ? a.muw_v_off : 0);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int r = 16 * ct + n;
      const float mw = muw[r];
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s_out[(16 * (TPW * w + tt) + 4 * g + e) * R + r] = (uint16_t)f32_to_bf16(acc[tt][ct][e] - mw);
    }
    // the next tile's slots, while nothing else is in flight (its loads are waited for)
    const long long tn = t + gridDim.x;
    const Tile nxt = tile_of(tn < ntiles ? tn : t);
    if (tn < ntiles) place(nxt, s_off[par ^ 1]);
    barrier_vm<63>();
    uint16_t *pool = pool_all + (long long)cur.li * lstride;
    for (int q = threadIdx.x; q < TOK * (R / 8); q += blockDim.x) {
      const int tl = q / (R / 8), c8 = q % (R / 8);
      const long long off = s_off[par][tl];
      if (off >= 0) *(u32x4 *)(pool + off + 8 * c8) = *(const u32x4 *)(s_out + tl * R + 8 * c8);
    }
    if (tn >= ntiles) break;
    // the next tile's first chunks load while this tile's output drains
    t = tn;
    cur = nxt;
    sources(cur);
    start();
    barrier_vm<63>();  // the staged output has been read before the slots take x rows again
  }
}

// Persistent grid: one workgroup per CU (LDS and registers allow no more).
constexpr long long kEncWorkgroups = 256;

#define LLA_ENCODE_R(X) X(16) X(32) X(48) X(64) X(96) X(128) X(160) X(256)

bool encode_mfma_r(int r) {
#define X(RR) if (r == RR) return true;
  LLA_ENCODE_R(X)
#undef X
  return false;
}

hipError_t launch_encode_mfma(int r, int kv, const EncodeArgs &a, hipStream_t stream) {
  const long long tokens = (long long)a.batch * a.n_new;
#define X(RR)                                                                                     \
  if (r == RR) {                                                                                  \
    const long long tiles = (tokens + enc_tok(RR) - 1) / enc_tok(RR) * a.groups * a.n_layers;      \
    hipLaunchKernelGGL(encode_mfma_kernel<RR>, dim3((unsigned)(tiles < kEncWorkgroups ? tiles : kEncWorkgroups)), \
                       dim3(512), 0, stream, a, kv);                                             \
    return hipGetLastError();                                                                     \
  }
  LLA_ENCODE_R(X)
#undef X
  return hipErrorInvalidConfiguration;
}

bool encode_supported(int dtype, int width, int r_k, int r_v) {
  return (dtype == LLA_BF16 || dtype == LLA_F32) && width > 0 && r_k > 0 && r_v > 0;
}

hipError_t launch_encode(int dtype, int r_k, int r_v, const EncodeArgs &a, hipStream_t stream) {
  const long long tokens = (long long)a.batch * a.n_new;
  if (tokens == 0 || a.n_layers == 0) return hipSuccess;
  // bf16 with whole 64-row chunks of W_down and an instantiated rank: matrix cores
  if (dtype == LLA_BF16 && a.width % 64 == 0 && encode_mfma_r(r_k) && encode_mfma_r(r_v) &&
      tokens <= 0x7FFFFFFFLL * 128) {
    hipError_t e = launch_muw<true>(r_k, r_v, a, stream);
    if (e != hipSuccess) return e;
    e = launch_encode_mfma(r_k, 0, a, stream);
    if (e != hipSuccess) return e;
    return launch_encode_mfma(r_v, 1, a, stream);
  }
  const dim3 g2((unsigned)((tokens + 15) / 16), a.groups, 2 * a.n_layers);
  if (dtype == LLA_BF16) {
    const hipError_t e = launch_muw<true>(r_k, r_v, a, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(encode_append_kernel<true>, g2, dim3(256), 0, stream, a, r_k, r_v);
  } else {
    const hipError_t e = launch_muw<false>(r_k, r_v, a, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(encode_append_kernel<false>, g2, dim3(256), 0, stream, a, r_k, r_v);
  }
  return hipGetLastError();
}

}  // namespace lla
