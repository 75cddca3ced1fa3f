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
//
// VEC: C is a multiple of 256 and each lane owns float4 groups of columns
// (lane*4 + 256*j); otherwise one column per lane (c = lane + 64*j).
template <bool VEC, int ROWS_PER_WAVE>
__global__ __launch_bounds__(256) void ln_bwd_kernel(const float* __restrict__ dy, const float* __restrict__ x,
                                                     const float* __restrict__ mean, const float* __restrict__ rstd,
                                                     const float* __restrict__ w, float* __restrict__ dR,
                                                     bf16* __restrict__ dRb, float* __restrict__ dw,
                                                     float* __restrict__ db, int rows, int C) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int NV = LN_MAXV;  // values per lane
  float gw[NV], gb[NV], wr[NV];
  auto col = [&](int j) { return VEC ? (4 * lane + 256 * (j >> 2) + (j & 3)) : (lane + 64 * j); };
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = col(j);
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
    float xh[NV], g[NV], d[NV];
    if constexpr (VEC) {
#pragma unroll
      for (int q = 0; q < NV / 4; ++q) {
        const int c = 4 * lane + 256 * q;
        float4 dv = make_float4(0.f, 0.f, 0.f, 0.f), xv = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c < C) {
          dv = *reinterpret_cast<const float4*>(dyr + c);
          xv = *reinterpret_cast<const float4*>(xr + c);
        }
        d[4 * q] = dv.x; d[4 * q + 1] = dv.y; d[4 * q + 2] = dv.z; d[4 * q + 3] = dv.w;
        xh[4 * q] = xv.x; xh[4 * q + 1] = xv.y; xh[4 * q + 2] = xv.z; xh[4 * q + 3] = xv.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int c = col(j);
        d[j] = (c < C) ? dyr[c] : 0.f;
        xh[j] = (c < C) ? xr[c] : 0.f;
      }
    }
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const bool in = col(j) < C;
      const float xv = in ? (xh[j] - mu) * rs : 0.f;
      xh[j] = xv;
      g[j] = d[j] * wr[j];
      gw[j] += d[j] * xv;
      gb[j] += d[j];
      sg += g[j];
      sgx += g[j] * xv;
    }
    sg = wave_sum(sg) / C;
    sgx = wave_sum(sgx) / C;
    float* dr = dR + (int64_t)row * C;
    if constexpr (VEC) {
#pragma unroll
      for (int q = 0; q < NV / 4; ++q) {
        const int c = 4 * lane + 256 * q;
        if (c < C) {
          float4 o = *reinterpret_cast<float4*>(dr + c);
          o.x += rs * (g[4 * q] - sg - xh[4 * q] * sgx);
          o.y += rs * (g[4 * q + 1] - sg - xh[4 * q + 1] * sgx);
          o.z += rs * (g[4 * q + 2] - sg - xh[4 * q + 2] * sgx);
          o.w += rs * (g[4 * q + 3] - sg - xh[4 * q + 3] * sgx);
          *reinterpret_cast<float4*>(dr + c) = o;
          if (dRb) {
            bf16x4 ob;
            ob[0] = f2bf(o.x); ob[1] = f2bf(o.y); ob[2] = f2bf(o.z); ob[3] = f2bf(o.w);
            *reinterpret_cast<bf16x4*>(dRb + (int64_t)row * C + c) = ob;
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int c = col(j);
        if (c < C) {
          const float nv = dr[c] + rs * (g[j] - sg - xh[j] * sgx);
          dr[c] = nv;
          if (dRb) dRb[(int64_t)row * C + c] = f2bf(nv);
        }
      }
    }
  }
  // reduce the 4 waves' column partials through LDS, 256 columns at a time
  __shared__ float red[4][2][256];
#pragma unroll
  for (int j0 = 0; j0 < NV; j0 += 4) {
    if (64 * j0 >= C) break;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      // position of value j0+jj within this 256-column slice
      const int pos = VEC ? (4 * lane + jj) : (lane + 64 * jj);
      red[wave][0][pos] = gw[j0 + jj];
      red[wave][1][pos] = gb[j0 + jj];
    }
    __syncthreads();
    const int t = threadIdx.x;
    const int c = 64 * j0 + t;
    if (c < C) {
      const float sw = red[0][0][t] + red[1][0][t] + red[2][0][t] + red[3][0][t];
      const float sb = red[0][1][t] + red[1][1][t] + red[2][1][t] + red[3][1][t];
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
  constexpr int RPW = 4;
  dim3 grid((rows + 4 * RPW - 1) / (4 * RPW)), block(256);
  prof_begin(L);
  if (C % 256 == 0)
    ln_bwd_kernel<true, RPW><<<grid, block, 0, L.stream>>>(dy, x, mean, rstd, w, dx, dxb, dw, db, rows, C);
  else
    ln_bwd_kernel<false, RPW><<<grid, block, 0, L.stream>>>(dy, x, mean, rstd, w, dx, dxb, dw, db, rows, C);
  prof_end(L);
  return hipGetLastError();
}

}  // namespace g2
