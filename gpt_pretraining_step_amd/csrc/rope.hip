// Rotary position embedding of the modern variant ("Reproduce GPT-2 124M":
// x cos + rotate_half(x) sin on q and k, base 10000), head dimension 64:
// the angle table and the backward rotation.  The forward rotation is a
// GEMM epilogue (GPT2_EPI_ROPE).
#include "common.h"

namespace g2 {

// tab[t][i] = (cos, sin)(t base^(-2i/64)), i < 32, angles in double precision.
__global__ __launch_bounds__(256) void rope_table_kernel(float2* __restrict__ tab, int T, double base) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= T * 32) return;
  const int t = k >> 5, i = k & 31;
  const double ang = (double)t * pow(base, -(2.0 * i) / 64.0);
  double s, c;
  sincos(ang, &s, &c);
  tab[k] = make_float2((float)c, (float)s);
}

// In place on the q and k column blocks of dqkv ([rows][ld] bf16, heads of 64
// at columns 64 h of each block, cols = 2 C columns in all): the transpose of
// the forward rotation, z1' = z1 c + z2 s, z2' = z2 c - z1 s, position
// t = row % period.  One thread per 4 consecutive pair indices of one head.
__global__ __launch_bounds__(256) void rope_bwd_kernel(bf16* __restrict__ dqkv, int rows, int64_t ld, int cols,
                                                       int period, const float2* __restrict__ tab) {
  const int per_row = cols / 8;  // (cols / 64 heads) x 8 groups of 4
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= (int64_t)rows * per_row) return;
  const int row = (int)(k / per_row), w = (int)(k % per_row);
  const int head = w >> 3, d = (w & 7) * 4;
  bf16* p = dqkv + (int64_t)row * ld + 64 * head + d;
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 32);
  const float2* cs = tab + (int64_t)(row % period) * 32 + d;
  bf16x4 oa, ob;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float c = cs[e].x, s = cs[e].y, z1 = bf2f(a[e]), z2 = bf2f(b[e]);
    oa[e] = f2bf(z1 * c + z2 * s);
    ob[e] = f2bf(z2 * c - z1 * s);
  }
  *reinterpret_cast<bf16x4*>(p) = oa;
  *reinterpret_cast<bf16x4*>(p + 32) = ob;
}

hipError_t launch_rope_table(const Launch& L, float2* tab, int T, double base) {
  prof_begin(L);
  rope_table_kernel<<<(T * 32 + 255) / 256, 256, 0, L.stream>>>(tab, T, base);
  prof_end(L);
  return hipGetLastError();
}

hipError_t launch_rope_bwd(const Launch& L, bf16* dqkv, int rows, int64_t ld, int cols, int period,
                           const float2* tab) {
  const int64_t n = (int64_t)rows * (cols / 8);
  prof_begin(L);
  rope_bwd_kernel<<<(unsigned)((n + 255) / 256), 256, 0, L.stream>>>(dqkv, rows, ld, cols, period, tab);
  prof_end(L);
  return hipGetLastError();
}

}  // namespace g2
