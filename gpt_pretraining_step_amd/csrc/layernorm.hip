// LayerNorm forward and backward ("How I trained my own GPT-2 124M on
// FineWeb-Edu" 2.3/2.5/2.8: nn.LayerNorm(n_embd) -- eps 1e-5, biased variance).
//
// One wave (64 lanes) per row; the row lives in registers, statistics in
// float32.  HBM-bound: the forward reads x (4 B) and writes y (2 or 4 B) per
// element; the backward reads dy (2 or 4 B) and x (4 B), read-modify-writes
// dx (8 B) and writes its bf16 copy (2 B).
#include "common.h"

namespace g2 {

constexpr int LN_MAXV = 16;  // supports C <= 1024
constexpr float LN_EPS = 1e-5f;
constexpr float RMS_EPS = 1.1920928955078125e-07f;  // float32 machine epsilon, 2^-23

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
// dR (acc = 1) or written there without reading it (acc = 0); optionally
// dRb = bf16(dR) for the bf16 products that consume it.  The
// weight and bias gradients are summed over the block's rows in registers,
// then added with one atomic per column per block.  Any C <= 1024: one
// column per lane (c = lane + 64 j); dy is float32 or bf16.
template <typename DYT, int ROWS_PER_WAVE>
__global__ __launch_bounds__(256) void ln_bwd_kernel(const DYT* __restrict__ dy, const float* __restrict__ x,
                                                     const float* __restrict__ mean, const float* __restrict__ rstd,
                                                     const float* __restrict__ w, float* __restrict__ dR,
                                                     bf16* __restrict__ dRb, float* __restrict__ dw,
                                                     float* __restrict__ db, int rows, int C, int acc) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int NV = LN_MAXV;  // values per lane
  float gw[NV], gb[NV], wr[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
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
    const DYT* dyr = dy + (int64_t)row * C;
    float xh[NV], g[NV], d[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int c = lane + 64 * j;
      d[j] = (c < C) ? to_f<DYT>(dyr[c]) : 0.f;
      xh[j] = (c < C) ? xr[c] : 0.f;
    }
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const bool in = lane + 64 * j < C;
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
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int c = lane + 64 * j;
      if (c < C) {
        const float nv = (acc ? dr[c] : 0.f) + rs * (g[j] - sg - xh[j] * sgx);
        dr[c] = nv;
        if (dRb) dRb[(int64_t)row * C + c] = f2bf(nv);
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
      red[wave][0][lane + 64 * jj] = gw[j0 + jj];
      red[wave][1][lane + 64 * jj] = gb[j0 + jj];
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

// ------------------------------------------------ vector kernels, C % 256 == 0
//
// Lane l owns the float4 column groups 4l + 256q (q < NQ = C/256), so every
// load and store is 16 bytes (8 for bf16) per lane and a wave's access to a
// row is contiguous.

// RMS: the RMSNorm of the rotary variant ("Reproduce GPT-2 124M", nn.RMSNorm
// with its defaults): no centring, no bias, eps = float32 machine epsilon;
// mean is not written.
template <int NQ, bool RMS>
__global__ __launch_bounds__(256) void ln_fwd_vec_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                                         const float* __restrict__ b, bf16* __restrict__ y,
                                                         float* __restrict__ mean, float* __restrict__ rstd,
                                                         int rows, int C) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* xr = x + (int64_t)row * C + 4 * lane;
  float4 v[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) v[q] = *reinterpret_cast<const float4*>(xr + 256 * q);
  float mu = 0.f;
  if constexpr (!RMS) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) s += (v[q].x + v[q].y) + (v[q].z + v[q].w);
    mu = wave_sum(s) / C;
  }
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const float a = v[q].x - mu, bb = v[q].y - mu, c = v[q].z - mu, d = v[q].w - mu;
    ss += (a * a + bb * bb) + (c * c + d * d);
  }
  const float rs = rsqrtf(wave_sum(ss) / C + (RMS ? RMS_EPS : LN_EPS));
  bf16* yr = y + (int64_t)row * C + 4 * lane;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int c = 4 * lane + 256 * q;
    const float4 ww = *reinterpret_cast<const float4*>(w + c);
    const float4 bv = RMS ? make_float4(0.f, 0.f, 0.f, 0.f) : *reinterpret_cast<const float4*>(b + c);
    bf16x4 o;
    o[0] = f2bf((v[q].x - mu) * rs * ww.x + bv.x);
    o[1] = f2bf((v[q].y - mu) * rs * ww.y + bv.y);
    o[2] = f2bf((v[q].z - mu) * rs * ww.z + bv.z);
    o[3] = f2bf((v[q].w - mu) * rs * ww.w + bv.w);
    *reinterpret_cast<bf16x4*>(yr + 256 * q) = o;
  }
  if (lane == 0) {
    if constexpr (!RMS) mean[row] = mu;
    rstd[row] = rs;
  }
}

template <typename T>
__device__ __forceinline__ float4 load4(const T* p);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
template <>
__device__ __forceinline__ float4 load4<bf16>(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return make_float4(bf2f(v[0]), bf2f(v[1]), bf2f(v[2]), bf2f(v[3]));
}

// Backward over RPW consecutive rows per wave, WPB waves per block; the
// next row's dy, x and dR are loaded before the current row is reduced, so
// each wave keeps two rows of loads in flight (dR only with acc = 1: with
// acc = 0 the branch is written to dR, not added).  dy is float32 or bf16.
// RMS: the RMSNorm backward, dx = rstd (g - xhat mean(g xhat)) (no
// centring term), no db.
template <typename DYT, int NQ, int RPW, int WPB, bool RMS>
__global__ __launch_bounds__(64 * WPB) void ln_bwd_vec_kernel(const DYT* __restrict__ dy, const float* __restrict__ x,
                                                         const float* __restrict__ mean,
                                                         const float* __restrict__ rstd,
                                                         const float* __restrict__ w, float* __restrict__ dR,
                                                         bf16* __restrict__ dRb, float* __restrict__ dw,
                                                         float* __restrict__ db, float* __restrict__ part, int rows,
                                                         int C, int acc) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float4 wr[NQ], gw[NQ], gb[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    wr[q] = *reinterpret_cast<const float4*>(w + 4 * lane + 256 * q);
    gw[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    gb[q] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int row0 = (blockIdx.x * WPB + wave) * RPW;
  const int nrows = min(RPW, rows - row0);
  float4 d[NQ], xv[NQ], r[NQ];
  float mu = 0.f, rs = 0.f;
  auto load = [&](int row, float4 (&d_)[NQ], float4 (&x_)[NQ], float4 (&r_)[NQ], float& mu_, float& rs_) {
    const int64_t o = (int64_t)row * C + 4 * lane;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      d_[q] = load4<DYT>(dy + o + 256 * q);
      x_[q] = *reinterpret_cast<const float4*>(x + o + 256 * q);
      r_[q] = acc ? *reinterpret_cast<const float4*>(dR + o + 256 * q) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    mu_ = RMS ? 0.f : mean[row];
    rs_ = rstd[row];
  };
  if (nrows > 0) load(row0, d, xv, r, mu, rs);
#pragma unroll 1
  for (int rr = 0; rr < nrows; ++rr) {
    const int row = row0 + rr;
    float4 nd[NQ], nx[NQ], nr[NQ];
    float nmu = 0.f, nrs = 0.f;
    if (rr + 1 < nrows) load(row + 1, nd, nx, nr, nmu, nrs);
    float sg = 0.f, sgx = 0.f;
    float4 g[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      xv[q] = make_float4((xv[q].x - mu) * rs, (xv[q].y - mu) * rs, (xv[q].z - mu) * rs, (xv[q].w - mu) * rs);
      g[q] = make_float4(d[q].x * wr[q].x, d[q].y * wr[q].y, d[q].z * wr[q].z, d[q].w * wr[q].w);
      gw[q].x += d[q].x * xv[q].x; gw[q].y += d[q].y * xv[q].y;
      gw[q].z += d[q].z * xv[q].z; gw[q].w += d[q].w * xv[q].w;
      gb[q].x += d[q].x; gb[q].y += d[q].y; gb[q].z += d[q].z; gb[q].w += d[q].w;
      sg += (g[q].x + g[q].y) + (g[q].z + g[q].w);
      sgx += (g[q].x * xv[q].x + g[q].y * xv[q].y) + (g[q].z * xv[q].z + g[q].w * xv[q].w);
    }
    sg = RMS ? 0.f : wave_sum(sg) / C;
    sgx = wave_sum(sgx) / C;
    const int64_t o = (int64_t)row * C + 4 * lane;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float4 v = r[q];
      v.x += rs * (g[q].x - sg - xv[q].x * sgx);
      v.y += rs * (g[q].y - sg - xv[q].y * sgx);
      v.z += rs * (g[q].z - sg - xv[q].z * sgx);
      v.w += rs * (g[q].w - sg - xv[q].w * sgx);
      *reinterpret_cast<float4*>(dR + o + 256 * q) = v;
      if (dRb) {
        bf16x4 ob;
        ob[0] = f2bf(v.x); ob[1] = f2bf(v.y); ob[2] = f2bf(v.z); ob[3] = f2bf(v.w);
        *reinterpret_cast<bf16x4*>(dRb + o + 256 * q) = ob;
      }
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      d[q] = nd[q];
      xv[q] = nx[q];
      r[q] = nr[q];
    }
    mu = nmu;
    rs = nrs;
  }
  // the waves' column partials through LDS, then per column and block
  // either one atomic (consecutive threads, consecutive columns; threads
  // 0-255 sum dw, 256-511 db: the fewer blocks, the less the atomics
  // contend) or, with `part`, a plain store of the block's row of partials
  // (dw in columns [0, C), db in [C, 2C)) that ln_param_grad_kernel sums
  static_assert(WPB % 4 == 0 && WPB >= 8, "two groups of 256 threads");
  __shared__ float red[2][WPB][256 * NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    *reinterpret_cast<float4*>(&red[0][wave][4 * lane + 256 * q]) = gw[q];
    *reinterpret_cast<float4*>(&red[1][wave][4 * lane + 256 * q]) = gb[q];
  }
  __syncthreads();
  const int which = threadIdx.x >> 8;
  if (which > 1 || (RMS && which == 1)) return;
  const float (*rw)[256 * NQ] = red[which];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int c = (threadIdx.x & 255) + 256 * q;
    float t[WPB / 4];
#pragma unroll
    for (int k = 0; k < WPB / 4; ++k) t[k] = (rw[4 * k][c] + rw[4 * k + 1][c]) + (rw[4 * k + 2][c] + rw[4 * k + 3][c]);
#pragma unroll
    for (int h = 1; h < WPB / 4; h *= 2)
#pragma unroll
      for (int k = 0; k + h < WPB / 4; k += 2 * h) t[k] += t[k + h];
    if (part) part[(int64_t)blockIdx.x * 2 * C + which * C + c] = t[0];
    else unsafeAtomicAdd((which ? db : dw) + c, t[0]);
  }
}

hipError_t launch_layernorm_fwd(const Launch& L, const float* x, const float* w, const float* b, void* y, int y_bf16,
                                float* mean, float* rstd, int rows, int C) {
  dim3 grid((rows + 3) / 4), block(256);
  prof_begin(L);
  bf16* yb = static_cast<bf16*>(y);
  if (y_bf16 && C % 256 == 0) {
    switch (C / 256) {
      case 1: ln_fwd_vec_kernel<1, false><<<grid, block, 0, L.stream>>>(x, w, b, yb, mean, rstd, rows, C); break;
      case 2: ln_fwd_vec_kernel<2, false><<<grid, block, 0, L.stream>>>(x, w, b, yb, mean, rstd, rows, C); break;
      case 3: ln_fwd_vec_kernel<3, false><<<grid, block, 0, L.stream>>>(x, w, b, yb, mean, rstd, rows, C); break;
      default: ln_fwd_vec_kernel<4, false><<<grid, block, 0, L.stream>>>(x, w, b, yb, mean, rstd, rows, C); break;
    }
  } else if (y_bf16) {
    ln_fwd_kernel<bf16><<<grid, block, 0, L.stream>>>(x, w, b, yb, mean, rstd, rows, C);
  } else {
    ln_fwd_kernel<float><<<grid, block, 0, L.stream>>>(x, w, b, static_cast<float*>(y), mean, rstd, rows, C);
  }
  prof_end(L);
  return hipGetLastError();
}

// Rows per block of the vector backward (8 waves of 8 rows): its blocks
// each leave one row of column partials when the caller asks for them.
constexpr int kLnBwdRows = 64;
int ln_bwd_part_blocks(int rows, int C) {
  return C % 256 == 0 && C <= 1024 ? (rows + kLnBwdRows - 1) / kLnBwdRows : 0;
}

template <typename DYT, bool RMS>
static void ln_bwd_dispatch(hipStream_t st, const DYT* dy, const float* x, const float* mean, const float* rstd,
                            const float* w, float* dx, bf16* dxb, float* dw, float* db, float* part, int rows,
                            int C, int acc) {
  if (C % 256 == 0) {
    // 8 rows per wave, 8 waves per block (one block per compute unit at
    // 16,384 rows): the next row's loads in flight keep HBM busy, and the
    // column atomics (one per column and block) are few.  Per GPT-2 step on
    // one box: 4-wave blocks 34.5 ms (their atomics alone 5.1 ms), 8-wave
    // 30.8 ms, 16-wave blocks of 4 rows per wave 52.9 ms; 16 rows per wave
    // in 4-wave blocks was slower than 8
    constexpr int RPW = 8, WPB = 8;
    static_assert(RPW * WPB == kLnBwdRows, "rows per block");
    const dim3 grid((rows + WPB * RPW - 1) / (WPB * RPW));
    switch (C / 256) {
      case 1: ln_bwd_vec_kernel<DYT, 1, RPW, WPB, RMS><<<grid, 64 * WPB, 0, st>>>(dy, x, mean, rstd, w, dx, dxb, dw, db, part, rows, C, acc); break;
      case 2: ln_bwd_vec_kernel<DYT, 2, RPW, WPB, RMS><<<grid, 64 * WPB, 0, st>>>(dy, x, mean, rstd, w, dx, dxb, dw, db, part, rows, C, acc); break;
      case 3: ln_bwd_vec_kernel<DYT, 3, RPW, WPB, RMS><<<grid, 64 * WPB, 0, st>>>(dy, x, mean, rstd, w, dx, dxb, dw, db, part, rows, C, acc); break;
      default: ln_bwd_vec_kernel<DYT, 4, RPW, WPB, RMS><<<grid, 64 * WPB, 0, st>>>(dy, x, mean, rstd, w, dx, dxb, dw, db, part, rows, C, acc); break;
    }
  } else if constexpr (!RMS) {
    constexpr int RPW = 4;
    const dim3 grid((rows + 4 * RPW - 1) / (4 * RPW));
    ln_bwd_kernel<DYT, RPW><<<grid, 256, 0, st>>>(dy, x, mean, rstd, w, dx, dxb, dw, db, rows, C, acc);
  }
}

hipError_t launch_layernorm_bwd_b(const Launch& L, const void* dy, int dy_bf16, const float* x, const float* mean,
                                  const float* rstd, const float* w, float* dx, bf16* dxb, float* dw, float* db,
                                  int rows, int C, float* part, int accumulate) {
  if (part && ln_bwd_part_blocks(rows, C) == 0) return hipErrorInvalidValue;
  prof_begin(L);
  if (dy_bf16)
    ln_bwd_dispatch<bf16, false>(L.stream, static_cast<const bf16*>(dy), x, mean, rstd, w, dx, dxb, dw, db, part,
                                 rows, C, accumulate);
  else
    ln_bwd_dispatch<float, false>(L.stream, static_cast<const float*>(dy), x, mean, rstd, w, dx, dxb, dw, db, part,
                                  rows, C, accumulate);
  prof_end(L);
  return hipGetLastError();
}

// RMSNorm (C % 256 == 0): y bf16, rstd float32 per row.
hipError_t launch_rmsnorm_fwd(const Launch& L, const float* x, const float* w, bf16* y, float* rstd, int rows, int C) {
  if (C % 256 != 0 || C > 1024) return hipErrorInvalidValue;
  dim3 grid((rows + 3) / 4), block(256);
  prof_begin(L);
  switch (C / 256) {
    case 1: ln_fwd_vec_kernel<1, true><<<grid, block, 0, L.stream>>>(x, w, nullptr, y, nullptr, rstd, rows, C); break;
    case 2: ln_fwd_vec_kernel<2, true><<<grid, block, 0, L.stream>>>(x, w, nullptr, y, nullptr, rstd, rows, C); break;
    case 3: ln_fwd_vec_kernel<3, true><<<grid, block, 0, L.stream>>>(x, w, nullptr, y, nullptr, rstd, rows, C); break;
    default: ln_fwd_vec_kernel<4, true><<<grid, block, 0, L.stream>>>(x, w, nullptr, y, nullptr, rstd, rows, C); break;
  }
  prof_end(L);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const Launch& L, const void* dy, int dy_bf16, const float* x, const float* rstd,
                              const float* w, float* dx, bf16* dxb, float* dw, int rows, int C, float* part,
                              int accumulate) {
  if (C % 256 != 0 || C > 1024) return hipErrorInvalidValue;
  prof_begin(L);
  if (dy_bf16)
    ln_bwd_dispatch<bf16, true>(L.stream, static_cast<const bf16*>(dy), x, nullptr, rstd, w, dx, dxb, dw, nullptr,
                                part, rows, C, accumulate);
  else
    ln_bwd_dispatch<float, true>(L.stream, static_cast<const float*>(dy), x, nullptr, rstd, w, dx, dxb, dw, nullptr,
                                 part, rows, C, accumulate);
  prof_end(L);
  return hipGetLastError();
}

// dw[s][c] += sum over blocks b of part[s][b][c] (and db from columns C + c
// where db[s] is non-null), for every norm site s of one backward: the
// blocks' partial rows are summed in block order, so the result does not
// depend on scheduling.  A 1,024-thread block covers 64 columns of one site:
// its 16 row groups each sum every 16th partial row, then the groups are
// added in order.
__global__ __launch_bounds__(1024) void ln_param_grad_kernel(const float* __restrict__ part, int nblk, int C,
                                                             LnGradSites sites) {
  const int col = blockIdx.x * 64 + (threadIdx.x & 63), grp = threadIdx.x >> 6, s = blockIdx.y;
  const float* ps = part + (int64_t)s * nblk * 2 * C;
  __shared__ float red[2][16][64];
  for (int h = 0; h < 2; ++h) {
    if (h == 1 && !sites.db[s]) break;  // (no bias: its columns were never written)
    float acc = 0.f;
    if (col < C) {
      // eight loads in flight, then added in row order
      const float* pc = ps + h * C + col;
      int b = grp;
      for (; b + 7 * 16 < nblk; b += 8 * 16) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = pc[(int64_t)(b + 16 * u) * 2 * C];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
      }
      for (; b < nblk; b += 16) acc += pc[(int64_t)b * 2 * C];
    }
    red[h][grp][threadIdx.x & 63] = acc;
  }
  __syncthreads();
  if (threadIdx.x < 128 && col < C) {
    const int h = threadIdx.x >> 6, cc = threadIdx.x & 63;
    float* dst = h ? sites.db[s] : sites.dw[s];
    if (dst) {
      float t = 0.f;
      for (int k = 0; k < 16; ++k) t += red[h][k][cc];
      dst[blockIdx.x * 64 + cc] += t;
    }
  }
}

hipError_t launch_ln_param_grad(const Launch& L, const float* part, int rows, int C, const LnGradSites& sites,
                                int nsites) {
  const int nblk = ln_bwd_part_blocks(rows, C);
  if (nblk == 0 || nsites < 1 || nsites > kLnGradSites) return hipErrorInvalidValue;
  prof_begin(L);
  ln_param_grad_kernel<<<dim3((C + 63) / 64, nsites), 1024, 0, L.stream>>>(part, nblk, C, sites);
  prof_end(L);
  return hipGetLastError();
}

}  // namespace g2
