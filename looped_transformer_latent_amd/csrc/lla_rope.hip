// RoPE angle table: table[p][i] = (cos, sin)(p * base^(-2i/d)), evaluated in
// fp64 and rounded to fp32.  Split-half pairs (i, i + d/2); the rotation is
// applied to the rebuilt K at the token's position and to q at q_pos (cc.laoqi.cc
// close reading, 方法 item 3: full-dimension RoPE after reconstruction).
#include "lla_internal.h"

namespace lla {

__global__ void rope_table_kernel(int n_pos, int half, int d, double base, float *table) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)n_pos * half) return;
  const int p = (int)(idx / half), i = (int)(idx % half);
  const double theta = (double)p * pow(base, -2.0 * (double)i / (double)d);
  double s, c;
  sincos(theta, &s, &c);
  table[2 * idx] = (float)c;
  table[2 * idx + 1] = (float)s;
}

hipError_t launch_rope_table(int n_pos, int d_head, double base, float *table, hipStream_t s) {
  const long long total = (long long)n_pos * (d_head / 2);
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, s, n_pos, d_head / 2, d_head,
                     base, table);
  return hipGetLastError();
}

}  // namespace lla
