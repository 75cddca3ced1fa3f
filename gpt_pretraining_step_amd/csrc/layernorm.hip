// LayerNorm forward and backward ("How I trained my own GPT-2 124M on
// FineWeb-Edu" 2.3/2.5/2.8: nn.LayerNorm(n_embd) -- eps 1e-5, biased variance).
//
// One wave (64 lanes) per row; the row lives in registers, statistics in
// float32.  HBM-bound: the forward reads x (4 B) and writes y (2 or 4 B) per
// element; the backward reads dy, x (8 B), read-modify-writes dx (8 B) and
// writes its bf16 copy (2 B).
#include "common.h"

namespace g2 {

constexpr int LN_MAXV = 16;  // supports C <= 1024
constexpr float LN_EPS = 1e-5f;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <typename YT>
__global__ __launch_bounds__(256) void ln_fwd_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                                     const float* __restrict__ b, YT* __restrict__ y,
                                                     float* __restrict__ mean, float* __restrict__ rstd, int rows,
                                                     int C) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* xr = x + (int64_t)row * C;
  float v[LN_MAXV];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < LN_MAXV; ++j) {
    const int c = lane + 64 * j;
    v[j] = (c < C) ? xr[c] : 0.f;
    s += v[j];
  }
  const float mu = wave_sum(s) / C;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < LN_MAXV; ++j) {
    const int c = lane + 64 * j;
    const float d = (c < C) ? v[j] - mu : 0.f;
    q += d * d;
  }
  const float rs = rsqrtf(wave_sum(q) / C + LN_EPS);
  YT* yr = y + (int64_t)row * C;
#pragma unroll
  for (int j = 0; j < LN_MAXV; ++j) {
    const int c = lane + 64 * j;
    if (c < C) yr[c] = from_f<YT>((v[j] - mu) * rs * w[c] + b[c]);
  }
  if (lane == 0) {
    mean[row] = mu;
    rstd[row] = rs;
  }
}

// dx = rstd (g - mean(g) - xhat mean(g xhat)), g = dy w; dx is added into
// dR; optionally dRb = bf16(dR) for the bf16 products that consume it.  The
// weight and bias gradients are summed over the block's rows in registers,
// then added with one atomic per column per block.
template <int ROWS_PER_WAVE>
__global__ __launch_bounds__(256) void ln_bwd_kernel(const float* __restrict__ dy, const float* __restrict__ x,
                                                     const float* __restrict__ mean, const float* __restrict__ rstd,
                                                     const float* __restrict__ w, float* __restrict__ dR,
                                                     bf16* __restrict__ dRb, float* __restrict__ dw,
                                                     float* __restrict__ db, int rows, int C) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float gw[LN_MAXV], gb[LN_MAXV], wr[LN_MAXV];
#pragma unroll
  for (int j = 0; j < LN_MAXV; ++j) {
    const int c = lane + 64 * j;
    gw[j] = 0.f;
    gb[j] = 0.f;
    wr[j] = (c < C) ? w[c] : 0.f;
  }
  const int row0 = (blockIdx.x * 4 + wave) * ROWS_PER_WAVE;
  for (int rr = 0; rr < ROWS_PER_WAVE; ++rr) {
    const int row = row0 + rr;
    if (row >= rows) break;
    const float mu = mean[row], rs = rstd[row];
    const float* xr = x + (int64_t)row * C;
    const float* dyr = dy + (int64_t)row * C;
    float xh[LN_MAXV], g[LN_MAXV];
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int j = 0; j < LN_MAXV; ++j) {
      const int c = lane + 64 * j;
      float d = 0.f, xv = 0.f;
      if (c < C) {
        d = dyr[c];
        xv = (xr[c] - mu) * rs;
      }
      xh[j] = xv;
      g[j] = d * wr[j];
      gw[j] += d * xv;
      gb[j] += d;
      sg += g[j];
      sgx += g[j] * xv;
    }
    sg = wave_sum(sg) / C;
    sgx = wave_sum(sgx) / C;
    float* dr = dR + (int64_t)row * C;
#pragma unroll
    for (int j = 0; j < LN_MAXV; ++j) {
      const int c = lane + 64 * j;
      if (c < C) {
        const float nv = dr[c] + rs * (g[j] - sg - xh[j] * sgx);
        dr[c] = nv;
        if (dRb) dRb[(int64_t)row * C + c] = f2bf(nv);
      }
    }
  }
  __shared__ float red[4][2][64 * 4];
  // reduce the 4 waves' column partials through LDS in slices of 256 columns
#pragma unroll
  for (int j0 = 0; j0 < LN_MAXV; j0 += 4) {
    if (64 * j0 >= C) break;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      red[wave][0][lane + 64 * jj] = gw[j0 + jj];
      red[wave][1][lane + 64 * jj] = gb[j0 + jj];
    }
    __syncthreads();
    const int t = threadIdx.x;  // 256 threads: one column of this slice each
    const int c = 64 * j0 + t;
    if (c < C) {
      float sw = red[0][0][t] + red[1][0][t] + red[2][0][t] + red[3][0][t];
      float sb = red[0][1][t] + red[1][1][t] + red[2][1][t] + red[3][1][t];
      unsafeAtomicAdd(dw + c, sw);
      unsafeAtomicAdd(db + c, sb);
    }
    __syncthreads();
  }
}

hipError_t launch_layernorm_fwd(const Launch& L, const float* x, const float* w, const float* b, void* y, int y_bf16,
                                float* mean, float* rstd, int rows, int C) {
  dim3 grid((rows + 3) / 4), block(256);
  prof_begin(L);
  if (y_bf16)
    ln_fwd_kernel<bf16><<<grid, block, 0, L.stream>>>(x, w, b, static_cast<bf16*>(y), mean, rstd, rows, C);
  else
    ln_fwd_kernel<float><<<grid, block, 0, L.stream>>>(x, w, b, static_cast<float*>(y), mean, rstd, rows, C);
  prof_end(L);
  return hipGetLastError();
}

hipError_t launch_layernorm_bwd_b(const Launch& L, const float* dy, const float* x, const float* mean,
                                  const float* rstd, const float* w, float* dx, bf16* dxb, float* dw, float* db,
                                  int rows, int C) {
  constexpr int RPW = 16;
  dim3 grid((rows + 4 * RPW - 1) / (4 * RPW)), block(256);
  prof_begin(L);
  ln_bwd_kernel<RPW><<<grid, block, 0, L.stream>>>(dy, x, mean, rstd, w, dx, dxb, dw, db, rows, C);
  prof_end(L);
  return hipGetLastError();
}

}  // namespace g2
