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
// The rows of W_down are cut into at most 64 ranges of a multiple of 64 rows,
// summed by separate workgroups (one per (range, group), layer, K|V) into
// muw_part; a second launch adds the ranges in fixed order.  Within a range,
// lane l of wave w reads 8 columns (16 bytes) of row w RPI + l / P8 and then
// every 4 RPI rows (P8 = R / 8 lanes per row, RPI = 64 / P8 rows per load
// instruction); the lanes' sums of a column are added in fixed order.
constexpr int kMuwRows = 64;
constexpr int kMuwMaxParts = 64;

__host__ __device__ int encode_muw_rows(int width) {
  const int blocks = (width + kMuwRows - 1) / kMuwRows;  // 64-row blocks
  return kMuwRows * ((blocks + kMuwMaxParts - 1) / kMuwMaxParts);
}
int encode_muw_parts(int width) { return (width + encode_muw_rows(width) - 1) / encode_muw_rows(width); }

template <bool BF>
__global__ __launch_bounds__(256) void encode_muw_kernel(EncodeArgs a, int RK, int RV) {
  __shared__ float part[4][64][8];  // [wave][lane][8 columns]
  const int grp = blockIdx.x % a.groups, pr = blockIdx.x / a.groups;
  const int li = blockIdx.y, kv = blockIdx.z;
  const int R = kv ? RV : RK;
  const int esz = BF ? 2 : 4;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long long gl = (long long)li * a.groups + grp;  // relative to layer0
  const char *mu = (kv ? a.mu_v : a.mu_k) + gl * a.width * esz;
  const char *wd = (kv ? a.wd_v : a.wd_k) + gl * a.width * (long long)R * esz;
  const int rows = encode_muw_rows(a.width);
  const int i0 = pr * rows, i1 = min(i0 + rows, a.width);
  float *dst = a.muw_part + ((long long)pr * a.n_layers * a.groups + gl) * (RK + RV) + (kv ? RK : 0);
  if (R % 8 || R > 512) {  // other widths: lanes over columns, wave w sums rows w, w + 4, ...
    __shared__ float part1[4][256];
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
      for (int j = 0; j < 4; ++j) part1[w][lane + 64 * j] = acc[j];
      __syncthreads();
      const int r = r0 + threadIdx.x;
      if (r < R) dst[r] = ((part1[0][threadIdx.x] + part1[1][threadIdx.x]) + part1[2][threadIdx.x]) + part1[3][threadIdx.x];
      __syncthreads();
    }
    return;
  }
  const int P8 = R / 8, RPI = 64 / P8;
  const int ro = lane / P8, p = lane % P8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (ro < RPI) {
#pragma unroll 8
    for (int i = i0 + w * RPI + ro; i < i1; i += 4 * RPI) {
      const float m = ldx<BF>(mu, i);
      const char *src = wd + ((long long)i * R + 8 * p) * esz;
      if constexpr (BF) {
        const u32x4 v = *(const u32x4 *)src;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[2 * k] = fmaf(m, bf16_lo(v[k]), acc[2 * k]);
          acc[2 * k + 1] = fmaf(m, bf16_hi(v[k]), acc[2 * k + 1]);
        }
      } else {
        const f32x4 lo = *(const f32x4 *)src, hi = *(const f32x4 *)(src + 16);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[k] = fmaf(m, lo[k], acc[k]);
          acc[4 + k] = fmaf(m, hi[k], acc[4 + k]);
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) part[w][lane][k] = acc[k];
  __syncthreads();
  // column r: lanes q P8 + r / 8 of every wave, added in (wave, q) order
  for (int r = threadIdx.x; r < R; r += blockDim.x) {
    float s = 0.f;
    for (int ww = 0; ww < 4; ++ww)
      for (int q = 0; q < RPI; ++q) s += part[ww][q * P8 + r / 8][r % 8];
    dst[r] = s;
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
// on v_mfma_f32_16x16x32_bf16, computed transposed (W_down^T as the A
// operand, x^T as the B operand) so that each lane ends with four consecutive
// latent columns of one token.  A workgroup (8 waves) takes 256 tokens (128
// for r > 160); wave w owns two 16-token tiles (one) and all r columns.  The
// contraction runs over chunks of 64 rows of W_down (32 for r > 160):
//  * x: each wave loads its rows x chunk bytes in address order (for 64-row
//    chunks one load instruction covers 8 whole 128-byte row pieces) with
//    buffer loads, two chunks ahead in registers, and passes them through its
//    own LDS region (16-byte slots XOR-swizzled by row) into operand layout;
//  * W_down: the chunk's rows are copied as stored (r contiguous; rows padded
//    so that the transposing reads below hit distinct banks) straight into
//    LDS by the 8 waves together (global_load_lds_dwordx4), two chunks ahead
//    in three buffers, one barrier per chunk;
//  * W_down operands come from ds_read_b64_tr_b16, which hands lane (g, n)
//    column n of four consecutive rows: K-slot 8 g + 4 h + e of K-step s is
//    chunk row 32 s + 16 h + 4 g + e, on both operands.
// mu W_down comes from encode_muw_kernel (once per call) and is copied into
// LDS with the tile's first chunk.  The result (minus mu W_down, rounded once
// to bf16) is staged in LDS with 8-byte stores (16-byte pieces swizzled per
// row across the banks) and leaves as 16-byte stores into the paged pool.  Workgroups are persistent (at most one per CU) and
// walk (group, token tile, layer) tiles, group fastest; the next tile's first
// two chunks load while a tile's output is staged and drains.
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
// Raw buffer descriptor word 3 on gfx9-family parts (32-bit data format, no
// swizzle, no index stride: untyped loads by byte offset), and the buffer
// load's cache-policy bit for data read once (nt).
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNonTemporal = 2;

// The same from the wave-uniform address base + off (off: this lane's 32-bit
// byte offset), in the instruction's scalar-base form.
__device__ __forceinline__ void copy16_to_lds_at(const void *base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base) : "memory", "m0");
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

// SPLIT: the width is cut into ksplit ranges (a separate instantiation, so
// that the unsplit kernel carries none of its state).
template <int R, bool SPLIT>
__global__ __launch_bounds__(512) void encode_mfma_kernel(EncodeArgs a, int kv, int ksplit_arg) {
  const int ksplit = SPLIT ? ksplit_arg : 1;
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
  __shared__ __attribute__((aligned(16))) float s_muw[2][SPLIT ? 4 : R];  // mu W_down per tile parity

  // wave index as a scalar: branches on it must be uniform scalar branches,
  // never EXEC-masked MFMAs
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, n = lane & 15;
  const long long tokens = (long long)a.batch * a.n_new;
  const long long ntt = (tokens + TOK - 1) / TOK;  // token tiles per (layer, group)
  const long long ntiles = ntt * a.groups * a.n_layers;
  // Work item t: tile t % ntiles over chunk range t / ntiles of the width (one
  // range unless the width is split: then the item's fp32 products go to
  // a.kpart and encode_splitk_reduce_kernel finishes the tile).
  const long long nwork = ntiles * ksplit;
  const char *x = kv ? a.x_v : a.x_k;
  const uint16_t *wd_all = (const uint16_t *)(kv ? a.wd_v : a.wd_k);
  uint16_t *pool_all = (uint16_t *)(kv ? a.v_pool : a.k_pool);
  const long long lstride = kv ? a.pool_layer_stride_v : a.pool_layer_stride_k;
  const long long pstride = kv ? a.pool_page_stride_v : a.pool_page_stride_k;
  const long long hstride = kv ? a.pool_head_stride_v : a.pool_head_stride_k;

  // Tiles t = blockIdx.x, + gridDim.x, ...: group fastest, then token tile,
  // then layer.  x is [layer][token][group][width], so the workgroups running
  // together read neighbouring pieces of the same token rows (DRAM pages stay
  // open: in a read-only test of this access pattern, reads at 6.0 TB/s with
  // token tile fastest and 6.8 TB/s with group fastest); the workgroups of one
  // XCD (blockIdx.x mod 8) still share a few groups' W_down in L2.
  struct Tile {
    long long tok0;
    int grp, li;
  };
  auto tile_of = [&](long long t) {
    Tile v;
    t %= ntiles;
    v.grp = (int)(t % a.groups);
    const long long r = t / a.groups;
    v.tok0 = (r % ntt) * TOK;
    v.li = (int)(r / ntt);
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
  // 16 TPW w + that, clamped; dropped at the end), piece l % XP of the chunk.
  // They are buffer loads over the wave's rows (a uniform descriptor from its
  // first row, clamped) with a 32-bit byte offset per lane and the chunk's
  // offset in a scalar; W_down copies take the tile's W_down as a uniform base
  // plus a fixed per-lane offset.  So few registers stay live for addresses.
  __amdgpu_buffer_rsrc_t xrs;
  uint32_t xoff[NXI];
  int xslot[NXI];
  const char *wbase;
  auto sources = [&](const Tile &v) {
    wbase = (const char *)(wd_all + ((long long)v.li * a.groups + v.grp) * a.width * (long long)R);
    const long long row0 = min(v.tok0 + 16 * TPW * w, tokens - 1);
    const char *xbase = x + ((((long long)v.li * tokens + row0) * a.groups + v.grp) * a.width) * 2;
    const long long xbytes = (long long)16 * TPW * a.groups * a.width * 2;  // covers every row the wave reads
    xrs = __builtin_amdgcn_make_buffer_rsrc((void *)xbase, (short)0, (int)min(xbytes, 0x7FFFFFFFll), kBufferWord3);
#pragma unroll
    for (int i = 0; i < NXI; ++i) {
      const int tl = (64 * i + lane) / XP, p = lane % XP;
      const long long tk = min(v.tok0 + 16 * TPW * w + tl, tokens - 1);
      xoff[i] = (uint32_t)((tk - row0) * a.groups * a.width * 2 + 16 * p);
    }
  };
  uint32_t woff[NWI];
#pragma unroll
  for (int i = 0; i < NWI; ++i) {
    const int slot = (i * 8 + w) * 64 + lane;
    const int k = slot / PW, pc = slot - k * PW;
    const bool ok = k < KC && pc < R / 8;
    woff[i] = (uint32_t)(((ok ? k : 0) * R + (ok ? 8 * pc : 0)) * 2);
  }
#pragma unroll
  for (int i = 0; i < NXI; ++i) {
    const int tl = (64 * i + lane) / XP, p = lane % XP;
    xslot[i] = (tl * XP + (p ^ ((tl >> 1) & (XP - 1)))) * 16;
  }
  auto load_x = [&](int c, u32x4 (&d)[NXI]) {
#pragma unroll
    for (int i = 0; i < NXI; ++i)
      d[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff[i], c * (KC * 2), kNonTemporal));
  };
  auto put_x = [&](const u32x4 (&d)[NXI]) {
#pragma unroll
    for (int i = 0; i < NXI; ++i) *(u32x4 *)(s_x + xslot[i]) = d[i];
  };
  // W_down rows c KC .. c KC + KC - 1 into buffer buf; pad and surplus slots
  // copy the chunk's first piece (never read)
  auto copy_w = [&](int c, char *dst) {
#pragma unroll
    for (int i = 0; i < NWI; ++i)
      copy16_to_lds_at(wbase + (long long)c * (KC * R * 2), woff[i], lds_addr(dst + (i * 8 + w) * 1024));
  };

  // Staged output rows: 16-byte piece c of row tl sits at c ^ out_swz(tl).
  // Rows P apart start on the same LDS bank (P = 64 / gcd(64, R / 2) for 64
  // banks of 4 bytes), so the swizzle takes row / P; it flips at most the low
  // bits that keep a piece inside its row (SWM + 1 divides R / 8).
  constexpr int RD = R / 2, GCD = RD % 64 == 0 ? 64 : RD % 32 == 0 ? 32 : RD % 16 == 0 ? 16 : RD % 8 == 0 ? 8 : 4;
  constexpr int SWP = 64 / GCD;
  constexpr int P8 = R / 8, SWM = P8 % 16 == 0 ? 15 : P8 % 8 == 0 ? 7 : P8 % 4 == 0 ? 3 : P8 % 2 == 0 ? 1 : 0;
  auto out_swz = [](int tl) { return (tl / SWP) & SWM; };

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
          acc[tt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(bw), as_bf16x8(av[tt]), acc[tt][ct], 0, 0, 0);
      }
    }
  };

  // Chunk c (W_down buffer c % 3): its x rows, in registers since two chunks
  // ago, go to the wave's slots.  The W_down copies of chunk c were issued
  // just before those x loads, so once at most NWI + NXI vector-memory
  // operations are outstanding (they count down in issue order), this wave's
  // part of chunk c is in LDS; all waves meet, which also frees buffer
  // (c + 2) % 3; then the copies and x loads of chunk c + 2 are issued and
  // chunk c is multiplied.  At a tile's first chunk the previous tile's
  // output stores are the most recent operations, so that wait also covers
  // chunk 1 and some of the stores: conservative, never short.
  const int nch_all = a.width / KC;
  const int per = (nch_all + ksplit - 1) / ksplit;  // chunks of one range
  int c_lo = 0, nch = nch_all;                     // the current item's range
  auto range_of = [&](long long t) {
    if constexpr (SPLIT) {
      c_lo = (int)(t / ntiles) * per;
      nch = min(per, nch_all - c_lo);
    }
  };
  auto step = [&](int c, const char *buf, char *buf2, u32x4 (&cur)[NXI], u32x4 (&nx2)[NXI]) {
    put_x(cur);
    if (c + 1 < nch) barrier_vm<NWI + NXI>();
    else barrier_vm<0>();
    if (c + 2 < nch) {
      copy_w(c_lo + c + 2, buf2);
      load_x(c_lo + c + 2, nx2);
    }
    compute(buf);
  };
  u32x4 xa[NXI], xb[NXI], xc[NXI];
  // the first two chunks of an item
  auto start = [&](const Tile &v, int par) {
    if constexpr (!SPLIT) {
      // mu W_down of the item's (layer, group): R/4 lanes of wave 0, older than
      // the first chunk's copies, so the first chunk's wait covers it
      if (w == 0) {
        const float *muw = a.muw + ((long long)v.li * a.groups + v.grp) * a.muw_stride + (kv ? a.muw_v_off : 0);
        if (lane < R / 4) copy16_to_lds(muw + 4 * lane, lds_addr(s_muw[par]));
      }
    }
    copy_w(c_lo, s_w0);
    load_x(c_lo, xa);
    if (nch > 1) {
      copy_w(c_lo + 1, s_w1);
      load_x(c_lo + 1, xb);
    }
  };

  long long t = blockIdx.x;
  if (t >= nwork) return;
  Tile cur = tile_of(t);
  range_of(t);
  if (!SPLIT) place(cur, s_off[0]);
  sources(cur);
  start(cur, 0);
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
    if constexpr (SPLIT) {  // fp32 products of this range, [item][token of the tile][r]
      float *dst = a.kpart + t * TOK * R;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) *(f32x4 *)(dst + (16 * (TPW * w + tt) + n) * R + 16 * ct + 4 * g) = acc[tt][ct];
      const long long tn = t + gridDim.x;
      if (tn >= nwork) break;
      t = tn;
      cur = tile_of(t);
      range_of(t);
      sources(cur);
      start(cur, 0);
      continue;
    }
    // The next tile's first two chunks load from here on, while this tile's
    // output is staged and drains (W_down buffers and x registers are free).
    const long long tn = t + gridDim.x;
    const Tile nxt = tile_of(tn < ntiles ? tn : t);
    if (tn < ntiles) {
      sources(nxt);
      start(nxt, par ^ 1);
    }
    // lane (g, n) holds columns 16 ct + 4 g .. + 3 of token 16 (TPW w + tt) + n
    uint16_t *s_out = (uint16_t *)s_xo;  // [TOK][R] bf16, 16-byte pieces swizzled per row
    const int tl0 = 16 * TPW * w + n;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const f32x4 mw = *(const f32x4 *)(s_muw[par] + 16 * ct + 4 * g);
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        const int tl = tl0 + 16 * tt;
        *(u32x2 *)(s_out + tl * R + 8 * ((2 * ct + (g >> 1)) ^ out_swz(tl)) + 4 * (g & 1)) =
            u32x2{pack_bf16(acc[tt][ct][0] - mw[0], acc[tt][ct][1] - mw[1]),
                  pack_bf16(acc[tt][ct][2] - mw[2], acc[tt][ct][3] - mw[3])};
      }
    }
    if (tn < ntiles) place(nxt, s_off[par ^ 1]);
    barrier_vm<63>();
    uint16_t *pool = pool_all + (long long)cur.li * lstride;
    constexpr int NQ = TOK * (R / 8);  // 16-byte pieces of the tile's output
#pragma unroll 5  // five pieces per thread in flight fit the register budget of every instance
    for (int q0 = 0; q0 < NQ; q0 += 512) {
      const int q = q0 + (int)threadIdx.x;
      if (NQ % 512 == 0 || q < NQ) {
        const int tl = q / (R / 8), c8 = q % (R / 8);
        const long long off = s_off[par][tl];
        if (off >= 0) *(u32x4 *)(pool + off + 8 * c8) = *(const u32x4 *)(s_out + tl * R + 8 * (c8 ^ out_swz(tl)));
      }
    }
    if (tn >= ntiles) break;
    t = tn;
    cur = nxt;
    barrier_vm<63>();  // the staged output has been read before the slots take x rows again
  }
}

// Finishes the tiles of a split width: adds the ranges' fp32 products in
// range order, subtracts mu W_down, rounds once to bf16 and stores each
// token's latent row in its slot.  One thread per (tile, token, 8 columns).
template <int R>
__global__ __launch_bounds__(256) void encode_splitk_reduce_kernel(EncodeArgs a, int kv, int ksplit) {
  constexpr int TOK = enc_tok(R), C8 = R / 8;
  const long long tokens = (long long)a.batch * a.n_new;
  const long long ntt = (tokens + TOK - 1) / TOK;
  const long long ntiles = ntt * a.groups * a.n_layers;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= ntiles * TOK * C8) return;
  const long long ti = idx / (TOK * C8);
  const int tl = (int)(idx / C8 % TOK), c8 = (int)(idx % C8);
  const long long tok = ti % ntt * TOK + tl;
  if (tok >= tokens) return;
  const long long rest = ti / ntt;
  const int grp = (int)(rest % a.groups), li = (int)(rest / a.groups);
  float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // unrolled so that the loads of 16 ranges are in flight together; the sum
  // keeps range order
#pragma unroll 16
  for (int sp = 0; sp < ksplit; ++sp) {
    const float *src = a.kpart + ((sp * ntiles + ti) * TOK + tl) * R + 8 * c8;
    const f32x4 lo = *(const f32x4 *)src, hi = *(const f32x4 *)(src + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sum[j] += lo[j];
      sum[4 + j] += hi[j];
    }
  }
  const int b = (int)(tok / a.n_new), nn = (int)(tok % a.n_new);
  const long long pos = (long long)a.pos0[b] + nn;
  if (pos < 0 || pos >= (long long)a.max_pages * kPage) {
    if (c8 == 0) atomicOr(a.err, LLA_DEVERR_APPEND);
    return;
  }
  const int page = a.page_table[(long long)b * a.max_pages + pos / kPage];
  if (page < 0 || page >= a.num_pages) {
    if (c8 == 0) atomicOr(a.err, LLA_DEVERR_PAGE);
    return;
  }
  const float *muw = a.muw + ((long long)li * a.groups + grp) * a.muw_stride + (kv ? a.muw_v_off : 0) + 8 * c8;
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16(sum[2 * j] - muw[2 * j], sum[2 * j + 1] - muw[2 * j + 1]);
  const long long lstride = kv ? a.pool_layer_stride_v : a.pool_layer_stride_k;
  const long long off = (long long)page * (kv ? a.pool_page_stride_v : a.pool_page_stride_k) +
                        grp * (kv ? a.pool_head_stride_v : a.pool_head_stride_k) + (pos % kPage) * R + 8 * c8;
  uint16_t *pool = (uint16_t *)(kv ? a.v_pool : a.k_pool) + (long long)li * lstride;
  *(u32x4 *)(pool + off) = o;
}

// Persistent grid: one workgroup per CU (LDS and registers allow no more).
constexpr long long kEncWorkgroups = 256;
// Split of the width: only for launches with fewer tiles than half the
// workgroups and at least kSplitMinChunks chunks of W_down; at most
// kSplitMaxItems (tile, range) items, which bounds the fp32 products region.
constexpr int kSplitMinChunks = 16;
constexpr long long kSplitMaxItems = kEncWorkgroups + kEncWorkgroups / 2;

#define LLA_ENCODE_R(X) X(16) X(32) X(48) X(64) X(96) X(128) X(160) X(256)

bool encode_mfma_r(int r) {
#define X(RR) if (r == RR) return true;
  LLA_ENCODE_R(X)
#undef X
  return false;
}

size_t encode_kpart_bytes(int width, int groups, int n_layers, int r_k, int r_v) {
  if (width % 64 || !encode_mfma_r(r_k) || !encode_mfma_r(r_v) || (long long)groups * n_layers >= kEncWorkgroups / 2)
    return 0;
  size_t bytes = 0;
  for (const int r : {r_k, r_v})
    if (width / enc_kc(r) >= kSplitMinChunks) {
      const size_t b = sizeof(float) * kSplitMaxItems * enc_tok(r) * r;
      if (b > bytes) bytes = b;
    }
  return bytes;
}

// Ranges the width is split into for a launch of ntiles tiles (1: no split).
int encode_ksplit(long long ntiles, int nch, size_t region, size_t tile_bytes) {
  if (ntiles >= kEncWorkgroups / 2 || nch < kSplitMinChunks || region == 0) return 1;
  int ks = (int)((kEncWorkgroups + ntiles - 1) / ntiles);
  if (ks > nch / 4) ks = nch / 4;  // at least 4 chunks per range
  const int per = (nch + ks - 1) / ks;
  ks = (nch + per - 1) / per;      // no empty range
  if (ks < 2 || (size_t)(ntiles * ks) * tile_bytes > region) return 1;
  return ks;
}

hipError_t launch_encode_mfma(int r, int kv, const EncodeArgs &a, hipStream_t stream) {
  const long long tokens = (long long)a.batch * a.n_new;
#define X(RR)                                                                                          \
  if (r == RR) {                                                                                       \
    const long long tiles = (tokens + enc_tok(RR) - 1) / enc_tok(RR) * a.groups * a.n_layers;           \
    const int ks = encode_ksplit(tiles, a.width / enc_kc(RR), a.kpart_bytes, sizeof(float) * enc_tok(RR) * RR); \
    const long long items = tiles * ks;                                                                \
    const dim3 grid((unsigned)(items < kEncWorkgroups ? items : kEncWorkgroups));                       \
    if (ks > 1)                                                                                        \
      hipLaunchKernelGGL((encode_mfma_kernel<RR, true>), grid, dim3(512), 0, stream, a, kv, ks);       \
    else                                                                                               \
      hipLaunchKernelGGL((encode_mfma_kernel<RR, false>), grid, dim3(512), 0, stream, a, kv, 1);       \
    if (ks > 1) {                                                                                      \
      const long long threads = tiles * enc_tok(RR) * (RR / 8);                                        \
      hipLaunchKernelGGL(encode_splitk_reduce_kernel<RR>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, \
                         stream, a, kv, ks);                                                          \
    }                                                                                                  \
    return hipGetLastError();                                                                          \
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
