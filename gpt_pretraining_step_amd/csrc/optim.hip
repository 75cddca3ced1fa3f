// Optimizer step, zeroing and initialisation.
//
// clip + AdamW: "Reproduce GPT-2 124M 复盘" (clip_grad_norm_(params, 1.0),
// fused AdamW with weight decay) and "How I trained my own GPT-2 124M on
// FineWeb-Edu" section 6 (AdamW, betas (0.9, 0.95), eps 1e-8, decay only on
// tensors of dim >= 2).  The update is the documented decoupled-decay AdamW
// with bias correction; the clip coefficient is min(1, max_norm/(norm+1e-6)).
// Two passes over the gradients: per-block partial sums of squares, then one
// fused pass that updates p, m, v and the bf16 shadow.  Between them one
// block reduces the partials in a fixed order to the norm and, when it is
// finite, advances the step counter (kept on the device, so a skipped step
// leaves it unchanged) and writes the clip coefficient and the two bias
// corrections for the update pass.  HBM traffic: 4 B/param for the norm, 30
// B/param for the update.
//
// Init ("How I trained my own GPT-2 124M on FineWeb-Edu" section 7): normals
// from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011) through the
// Box-Muller transform, evaluated in double precision.
#include "common.h"

namespace g2 {

__global__ __launch_bounds__(256) void sumsq_kernel(const float* __restrict__ g, size_t n, float* __restrict__ partials) {
  float s = 0.f;
  const size_t n4 = n / 4;
  const float4* g4 = reinterpret_cast<const float4*>(g);
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const float4 v = g4[i];
    s += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  for (size_t i = 4 * n4 + (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) s += g[i] * g[i];
  __shared__ float red[256];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) partials[blockIdx.x] = red[0];
}

__device__ __forceinline__ void adamw_elem(float& p, float g, float& m, float& v, float coef, float lr, float b1,
                                           float b2, float eps, float decay, float bc1, float bc2_sqrt) {
  g *= coef;
  p *= decay;
  m = b1 * m + (1.f - b1) * g;
  v = b2 * v + (1.f - b2) * g * g;
  const float denom = sqrtf(v) / bc2_sqrt + eps;
  p -= (lr / bc1) * m / denom;
}

// One block: norm = sqrt(sum of the partials), reduced in a fixed order.
// Finite: t = ++step[0]; sc = (clip coefficient, 1 - b1^t, sqrt(1 - b2^t),
// 1).  Not finite: GPT2_ERR_NONFINITE is raised and sc[3] = 0, so the update
// pass changes nothing and the step counter stays.
__global__ __launch_bounds__(256) void adamw_prep_kernel(const float* __restrict__ partials, int nparts, float b1,
                                                         float b2, float max_norm, int64_t* __restrict__ step,
                                                         float* __restrict__ sc, float* __restrict__ norm_out,
                                                         int* flag) {
  __shared__ float red[256];
  float s = 0.f;
  for (int i = threadIdx.x; i < nparts; i += 256) s += partials[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
  const float norm = sqrtf(red[0]);
  norm_out[0] = norm;
  if (!isfinite(norm)) {
    raise_flag(flag, GPT2_ERR_NONFINITE);
    sc[3] = 0.f;
    return;
  }
  const int64_t t = step[0] + 1;
  step[0] = t;
  sc[0] = fminf(1.f, max_norm / (norm + 1e-6f));
  sc[1] = (float)(1.0 - pow((double)b1, (double)t));
  sc[2] = sqrtf((float)(1.0 - pow((double)b2, (double)t)));
  sc[3] = 1.f;
}

__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    bf16* __restrict__ shadow, size_t n, size_t decay_end,
                                                    const float* __restrict__ sc, float lr, float b1, float b2,
                                                    float eps, float wd) {
  if (sc[3] == 0.f) return;
  const float coef = sc[0], bc1 = sc[1], bc2s = sc[2];
  const float dec = 1.f - lr * wd;
  const size_t n4 = n / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    float4 pp = reinterpret_cast<float4*>(p)[i];
    const float4 gg = reinterpret_cast<const float4*>(g)[i];
    float4 mm = reinterpret_cast<float4*>(m)[i];
    float4 vv = reinterpret_cast<float4*>(v)[i];
    const float d = (4 * i < decay_end) ? dec : 1.f;  // decay_end is a multiple of 4
    adamw_elem(pp.x, gg.x, mm.x, vv.x, coef, lr, b1, b2, eps, d, bc1, bc2s);
    adamw_elem(pp.y, gg.y, mm.y, vv.y, coef, lr, b1, b2, eps, d, bc1, bc2s);
    adamw_elem(pp.z, gg.z, mm.z, vv.z, coef, lr, b1, b2, eps, d, bc1, bc2s);
    adamw_elem(pp.w, gg.w, mm.w, vv.w, coef, lr, b1, b2, eps, d, bc1, bc2s);
    reinterpret_cast<float4*>(p)[i] = pp;
    reinterpret_cast<float4*>(m)[i] = mm;
    reinterpret_cast<float4*>(v)[i] = vv;
    if (shadow) {
      bf16x4 sh;
      sh[0] = f2bf(pp.x);
      sh[1] = f2bf(pp.y);
      sh[2] = f2bf(pp.z);
      sh[3] = f2bf(pp.w);
      reinterpret_cast<bf16x4*>(shadow)[i] = sh;
    }
  }
  for (size_t i = 4 * n4 + (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    float pp = p[i], mm = m[i], vv = v[i];
    adamw_elem(pp, g[i], mm, vv, coef, lr, b1, b2, eps, i < decay_end ? dec : 1.f, bc1, bc2s);
    p[i] = pp;
    m[i] = mm;
    v[i] = vv;
    if (shadow) shadow[i] = f2bf(pp);
  }
}

__global__ void fill_f32_kernel(float* p, size_t n, float value) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = value;
}
__global__ void fill_i32_kernel(int* p, size_t n, int value) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = value;
}
__global__ void to_bf16_kernel(const float* __restrict__ s, bf16* __restrict__ d, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    d[i] = f2bf(s[i]);
}

// ---------------------------------------------------------------- Philox

__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += W0;
      k1 += W1;
    }
    const uint32_t hi0 = __umulhi(M0, c[0]), lo0 = M0 * c[0];
    const uint32_t hi1 = __umulhi(M1, c[2]), lo1 = M1 * c[2];
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

__global__ __launch_bounds__(256) void init_normal_kernel(float* __restrict__ dst, size_t n, uint32_t tensor_index,
                                                          uint64_t seed, float stdv) {
  const size_t calls = (n + 3) / 4;
  for (size_t c = (size_t)blockIdx.x * 256 + threadIdx.x; c < calls; c += (size_t)gridDim.x * 256) {
    uint32_t w[4] = {(uint32_t)(c & 0xFFFFFFFFu), (uint32_t)(c >> 32), tensor_index, 0x6770u};
    philox4x32_10(w, (uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32));
    const double inv = 1.0 / 4294967296.0;
    const double u0 = ((double)w[0] + 0.5) * inv, u1 = ((double)w[1] + 0.5) * inv;
    const double u2 = ((double)w[2] + 0.5) * inv, u3 = ((double)w[3] + 0.5) * inv;
    const double ra = sqrt(-2.0 * log(u0)), rb = sqrt(-2.0 * log(u2));
    const double two_pi = 6.283185307179586;
    double z[4];
    z[0] = ra * cos(two_pi * u1);
    z[1] = ra * sin(two_pi * u1);
    z[2] = rb * cos(two_pi * u3);
    z[3] = rb * sin(two_pi * u3);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const size_t j = 4 * c + e;
      if (j < n) dst[j] = (float)((double)stdv * z[e]);
    }
  }
}

static unsigned grid_for(size_t n, unsigned per_block, unsigned cap) {
  size_t g = (n + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (unsigned)(g > cap ? cap : g);
}

hipError_t launch_sumsq_partials(const Launch& L, const float* g, size_t n, float* partials, int nparts) {
  prof_begin(L);
  sumsq_kernel<<<nparts, 256, 0, L.stream>>>(g, n, partials);
  prof_end(L);
  return hipGetLastError();
}

hipError_t launch_adamw(const Launch& L, const Launch& Lprep, float* p, const float* g, float* m, float* v,
                        bf16* shadow, size_t n, size_t decay_end, const float* partials, int nparts, float lr,
                        float b1, float b2, float eps, float wd, float max_norm, int64_t* step, float* sc,
                        float* norm_out, int* flag) {
  prof_begin(Lprep);
  adamw_prep_kernel<<<1, 256, 0, Lprep.stream>>>(partials, nparts, b1, b2, max_norm, step, sc, norm_out, flag);
  prof_end(Lprep);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_begin(L);
  adamw_kernel<<<grid_for(n / 4, 256, 2048), 256, 0, L.stream>>>(p, g, m, v, shadow, n, decay_end, sc, lr, b1, b2, eps,
                                                                  wd);
  prof_end(L);
  return hipGetLastError();
}

hipError_t launch_fill_f32(const Launch& L, float* p, size_t n, float value) {
  if (n == 0) return hipSuccess;
  prof_begin(L);
  fill_f32_kernel<<<grid_for(n, 256, 4096), 256, 0, L.stream>>>(p, n, value);
  prof_end(L);
  return hipGetLastError();
}

hipError_t launch_fill_i32(const Launch& L, int* p, size_t n, int value) {
  if (n == 0) return hipSuccess;
  prof_begin(L);
  fill_i32_kernel<<<grid_for(n, 256, 4096), 256, 0, L.stream>>>(p, n, value);
  prof_end(L);
  return hipGetLastError();
}

hipError_t launch_to_bf16(const Launch& L, const float* src, bf16* dst, size_t n) {
  if (n == 0) return hipSuccess;
  prof_begin(L);
  to_bf16_kernel<<<grid_for(n, 256, 4096), 256, 0, L.stream>>>(src, dst, n);
  prof_end(L);
  return hipGetLastError();
}

hipError_t launch_init_normal(const Launch& L, float* dst, size_t n, uint32_t tensor_index, uint64_t seed, float stdv) {
  if (n == 0) return hipSuccess;
  prof_begin(L);
  init_normal_kernel<<<grid_for((n + 3) / 4, 256, 4096), 256, 0, L.stream>>>(dst, n, tensor_index, seed, stdv);
  prof_end(L);
  return hipGetLastError();
}

}  // namespace g2
