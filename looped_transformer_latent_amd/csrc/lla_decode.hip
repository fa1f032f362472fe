// Fused split-K latent-cache decode attention for LLA (gfx950, wave64).
//
// What it computes (cc.laoqi.cc close reading, 方法 items 1-3; gist.science
// "Kernmechanismus"): for one (layer, loop t) and every query row,
//   k_hat_j = mu_k,t + c_k,j W_up,k,t^T   (eq. (3)), RoPE at position j,
//   s_j     = scale <R(q_pos) q, R(j) k_hat_j>,
//   out     = mu_v,t + (sum_j e^{s_j - m} c_v,j) W_up,v,t^T / sum_j e^{s_j - m}.
// The V side is exact by linearity of eq. (3): it is accumulated in latent
// space (r_v wide) and up-projected once per (row, head).
//
// How, per (row, head group, split) workgroup; one wave per HPW heads:
//  * Prologue -- fold the rotated query into the K decoder.  For RoPE pair i
//    (elements a = i, b = i + d/2) with q' = R(q_pos) q * scale * log2(e):
//      X_i(j) = q'_a k_hat_a + q'_b k_hat_b = alpha_i + sum_r A[i][r] c_r
//      Y_i(j) = q'_b k_hat_a - q'_a k_hat_b = beta_i  + sum_r B[i][r] c_r
//    with A[i][r] = q'_a W[a][r] + q'_b W[b][r], B[i][r] = q'_b W[a][r] - q'_a W[b][r],
//    alpha_i = q'_a mu_a + q'_b mu_b, beta_i = q'_b mu_a - q'_a mu_b, and then
//      s_j * log2(e) = sum_i cos(j w_i) X_i(j) + sin(j w_i) Y_i(j).
//    [A alpha; B beta] (d x (r_k + 1)) is held in registers as MFMA A-operands
//    (bf16: alpha/beta split into hi + lo bf16 parts; fp32: exact).
//  * Per 16-token page -- one MFMA 16x16 tile gives X (or Y) for 16 pair
//    indices x 16 tokens; the latent tile [c_k, 1, 1] is the B-operand, read
//    straight from the paged pool with 16-byte loads.  Each lane then needs
//    cos/sin for its 16 pair indices and its token only: 2 FMAs per (i, token).
//  * Online softmax in base 2 with deferred rescaling; V accumulated as
//    sum_j p_j c_v,j in fp32 registers (lane = token x r_v/4 chunk).
//  * Splits write (m, Z, acc) partials; the last workgroup of a row (atomic
//    counter, reset by that workgroup) merges them in fixed split order --
//    deterministic -- and up-projects through W_up,v,t.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {

template <bool BF>
struct St;
template <>
struct St<true> {
  using Opnd = bf16x8;
  static constexpr int esz = 2;
  __device__ static f32x4 mma(Opnd a, Opnd b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static float ld(const char *p, long long i) {
    return bf16_to_f32(((const uint16_t *)p)[i]);
  }
};
template <>
struct St<false> {
  using Opnd = float;
  static constexpr int esz = 4;
  __device__ static f32x4 mma(Opnd a, Opnd b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static float ld(const char *p, long long i) { return ((const float *)p)[i]; }
};

// Number of MFMA K-steps for r_k latent columns plus the constant column(s).
template <bool BF, int RK>
constexpr int ksteps() {
  return BF ? (RK + 2 + 31) / 32 : RK / 4 + 1;
}

template <bool BF, int DH, int RK, int RV, int HPW>
__global__ __launch_bounds__(512) void decode_ph_kernel(AttnArgs a) {
  using S = St<BF>;
  using Op = typename S::Opnd;
  constexpr int NT = DH / 32;         // tile pairs: pair indices [16t, 16t + 16)
  constexpr int KS = ksteps<BF, RK>();
  constexpr int CV = RV / 4;          // V latent elements per lane per token
  constexpr int HALF = DH / 2;
  static_assert(DH % 32 == 0 && RK % 16 == 0 && RV % 32 == 0, "shape");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
  Op A[HPW][NT][2][KS];
  {
    const float *rq = a.rope + (long long)qp * DH;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = h0 + hh;
      const char *qrow = (const char *)a.q + ((long long)row * a.H + h) * DH * S::esz;
      const char *w = a.wup_k + (long long)h * a.wup_head_stride_k * S::esz;
      const char *mu = a.mu_k + (long long)h * a.mu_head_stride * S::esz;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int i = 16 * t + n;
        const float c = rq[2 * i], s = rq[2 * i + 1];
        const float qa = S::ld(qrow, i), qb = S::ld(qrow, i + HALF);
        const float pa = a.qscale * (qa * c - qb * s);
        const float pb = a.qscale * (qa * s + qb * c);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if constexpr (BF) {
            const int r0 = 32 * ks + 8 * g;
            u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
            if (r0 + 8 <= RK) {
              const u32x4 wa = *(const u32x4 *)(w + ((long long)i * RK + r0) * 2);
              const u32x4 wb = *(const u32x4 *)(w + ((long long)(i + HALF) * RK + r0) * 2);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float a0 = bf16_lo(wa[e]), a1 = bf16_hi(wa[e]);
                const float b0 = bf16_lo(wb[e]), b1 = bf16_hi(wb[e]);
                x[e] = pack_bf16(pa * a0 + pb * b0, pa * a1 + pb * b1);
                y[e] = pack_bf16(pb * a0 - pa * b0, pb * a1 - pa * b1);
              }
            } else if (r0 == RK) {
              const float ma = S::ld(mu, i), mb = S::ld(mu, i + HALF);
              const float al = pa * ma + pb * mb, be = pb * ma - pa * mb;
              const uint32_t ah = f32_to_bf16(al), bh = f32_to_bf16(be);
              const uint32_t alo = f32_to_bf16(al - bf16_to_f32(ah));
              const uint32_t blo = f32_to_bf16(be - bf16_to_f32(bh));
              x[0] = ah | (alo << 16);
              y[0] = bh | (blo << 16);
            }
            A[hh][t][0][ks] = as_bf16x8(x);
            A[hh][t][1][ks] = as_bf16x8(y);
          } else {
            float x = 0.f, y = 0.f;
            if (ks < RK / 4) {
              const int r = (RK / 4) * g + ks;
              const float wa = S::ld(w, (long long)i * RK + r);
              const float wb = S::ld(w, (long long)(i + HALF) * RK + r);
              x = pa * wa + pb * wb;
              y = pb * wa - pa * wb;
            } else if (g == 0) {
              const float ma = S::ld(mu, i), mb = S::ld(mu, i + HALF);
              x = pa * ma + pb * mb;
              y = pb * ma - pa * mb;
            }
            A[hh][t][0][ks] = x;
            A[hh][t][1][ks] = y;
          }
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

  // ---- main loop over this split's pages ----
  for (int lp = lp0; lp < lp1; ++lp) {
    const int pp = a.page_table[(long long)b * a.max_pages + lp];
    if (pp < 0 || pp >= a.num_pages) {
      errbits |= LLA_DEVERR_PAGE;
      continue;
    }
    const int pos = lp * kPage + n;
    const bool valid = pos < ctx;
    const int tpos = valid ? pos : ctx - 1;  // keep table reads in range on a ragged page
    float cs[NT][8];
    {
      const float *rt = a.rope + (long long)tpos * DH + 8 * g;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const f32x4 u = *(const f32x4 *)(rt + 32 * t);
        const f32x4 v = *(const f32x4 *)(rt + 32 * t + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          cs[t][e] = u[e];
          cs[t][4 + e] = v[e];
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = h0 + hh;
      const char *kp = a.k_pool + ((long long)pp * a.pool_page_stride_k +
                                   (long long)h * a.pool_head_stride_k + (long long)n * RK) * S::esz;
      const char *vp = a.v_pool + ((long long)pp * a.pool_page_stride_v +
                                   (long long)h * a.pool_head_stride_v + (long long)n * RV + CV * g) * S::esz;
      Op bk[KS];
      float cv[CV];
      if constexpr (BF) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int r0 = 32 * ks + 8 * g;
          u32x4 v = {0, 0, 0, 0};
          if (r0 + 8 <= RK) v = *(const u32x4 *)(kp + r0 * 2);
          else if (r0 == RK) v[0] = 0x3F803F80u;  // bf16 (1, 1) multiplies alpha hi, lo
          bk[ks] = as_bf16x8(v);
        }
#pragma unroll
        for (int k8 = 0; k8 < CV / 8; ++k8) {
          const u32x4 v = *(const u32x4 *)(vp + k8 * 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            cv[8 * k8 + 2 * e] = bf16_lo(v[e]);
            cv[8 * k8 + 2 * e + 1] = bf16_hi(v[e]);
          }
        }
      } else {
        float kr[RK / 4];
#pragma unroll
        for (int k4 = 0; k4 < RK / 16; ++k4) {
          const f32x4 v = *(const f32x4 *)(kp + ((RK / 4) * g + 4 * k4) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) kr[4 * k4 + e] = v[e];
        }
#pragma unroll
        for (int ks = 0; ks < RK / 4; ++ks) bk[ks] = kr[ks];
        bk[RK / 4] = (g == 0) ? 1.f : 0.f;
#pragma unroll
        for (int k4 = 0; k4 < CV / 4; ++k4) {
          const f32x4 v = *(const f32x4 *)(vp + k4 * 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) cv[4 * k4 + e] = v[e];
        }
      }
      // X / Y tiles: rows = pair indices 16t + 4g + e, column = token n
      float sc = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4 X = {0.f, 0.f, 0.f, 0.f}, Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          X = S::mma(A[hh][t][0][ks], bk[ks], X);
          Y = S::mma(A[hh][t][1][ks], bk[ks], Y);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc = fmaf(cs[t][2 * e], X[e], sc);
          sc = fmaf(cs[t][2 * e + 1], Y[e], sc);
        }
      }
      sc = sum_across_rows(sc);
      sc = valid ? sc : -INFINITY;
      const float mt = max_in_row(sc);
      if (mt > m_run[hh]) {  // wave-uniform
        const float corr = exp2f(m_run[hh] - mt);
        z[hh] *= corr;
#pragma unroll
        for (int k = 0; k < CV; ++k) acc[hh][k] *= corr;
        m_run[hh] = mt;
      }
      const float p = exp2f(sc - m_run[hh]);
      z[hh] += p;
#pragma unroll
      for (int k = 0; k < CV; ++k) acc[hh][k] = fmaf(p, valid ? cv[k] : 0.f, acc[hh][k]);
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
  const bool bad = errbits != 0;

  extern __shared__ float sh[];  // [waves][HPW][RV + 2]
  __shared__ int s_last;
  float *mine = sh + (wave * HPW) * (RV + 2);

  if (a.splits > 1) {
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
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const int prev = atomicAdd(&a.counters[row * a.head_groups + hg], 1);
      s_last = (prev == a.splits - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (threadIdx.x == 0) a.counters[row * a.head_groups + hg] = 0;
    // merge the splits in fixed order
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = h0 + hh;
      const float *pb = a.partials + ((long long)row * a.H + h) * a.splits * (RV + 2);
      float M = -INFINITY;
      for (int s = 0; s < a.splits; ++s) M = fmaxf(M, pb[s * (RV + 2) + RV]);
      float Z = 0.f;
      for (int s = 0; s < a.splits; ++s)
        Z = fmaf(exp2f(pb[s * (RV + 2) + RV] - M), pb[s * (RV + 2) + RV + 1], Z);
      for (int r = lane; r < RV; r += 64) {
        float s_acc = 0.f;
        for (int s = 0; s < a.splits; ++s)
          s_acc = fmaf(exp2f(pb[s * (RV + 2) + RV] - M), pb[s * (RV + 2) + r], s_acc);
        mine[hh * (RV + 2) + r] = s_acc / Z;
      }
    }
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
    const char *w = a.wup_v + (long long)h * a.wup_head_stride_v * S::esz;
    const char *mu = a.mu_v + (long long)h * a.mu_head_stride * S::esz;
    const float *an = mine + hh * (RV + 2);
    for (int e = lane; e < DH; e += 64) {
      float o = S::ld(mu, e);
      const char *we = w + (long long)e * RV * S::esz;
      if constexpr (BF) {
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
      } else {
#pragma unroll
        for (int r4 = 0; r4 < RV / 4; ++r4) {
          const f32x4 v = *(const f32x4 *)(we + r4 * 16);
#pragma unroll
          for (int k = 0; k < 4; ++k) o = fmaf(v[k], an[4 * r4 + k], o);
        }
        ((float *)a.out)[((long long)row * a.H + h) * DH + e] = o;
      }
    }
  }
}

// ---------------------------------------------------------------- dispatch

namespace {
struct Shape {
  int bf, dh, rk, rv, hpw;
};
template <bool BF, int DH, int RK, int RV, int HPW>
hipError_t go(const AttnArgs &a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.rows * a.head_groups * a.splits));
  const dim3 block((unsigned)(64 * a.waves));
  const size_t shmem = sizeof(float) * a.waves * HPW * (RV + 2);
  hipLaunchKernelGGL((decode_ph_kernel<BF, DH, RK, RV, HPW>), grid, block, shmem, stream, a);
  return hipGetLastError();
}
}  // namespace

#define LLA_DECODE_SHAPES(X)   \
  X(false, 64, 16, 32, 1)      \
  X(false, 64, 16, 32, 2)      \
  X(false, 128, 16, 32, 1)     \
  X(false, 128, 16, 32, 2)     \
  X(true, 64, 16, 32, 1)       \
  X(true, 64, 16, 32, 2)       \
  X(true, 128, 16, 32, 1)      \
  X(true, 128, 16, 32, 2)      \
  X(true, 128, 32, 64, 1)      \
  X(true, 128, 96, 160, 1)     \
  X(false, 128, 96, 160, 1)

bool decode_supported(int dtype, int d_head, int r_k, int r_v, int hpw) {
  const bool bf = dtype == LLA_BF16;
#define X(BF, DH, RK, RV, HPW) \
  if (bf == BF && d_head == DH && r_k == RK && r_v == RV && hpw == HPW) return true;
  LLA_DECODE_SHAPES(X)
#undef X
  return false;
}

hipError_t launch_decode(int dtype, int d_head, int r_k, int r_v, const AttnArgs &a,
                         hipStream_t stream) {
  const bool bf = dtype == LLA_BF16;
#define X(BF, DH, RK, RV, HPW)                                                  \
  if (bf == BF && d_head == DH && r_k == RK && r_v == RV && a.heads_per_wave == HPW) \
    return go<BF, DH, RK, RV, HPW>(a, stream);
  LLA_DECODE_SHAPES(X)
#undef X
  return hipErrorInvalidConfiguration;
}

}  // namespace lla
