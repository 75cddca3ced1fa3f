// Cross-entropy over the tied lm_head's logits, one row chunk at a time
// ("How I trained my own GPT-2 124M on FineWeb-Edu" section 4: softmax, pick
// the target's probability, -log, mean over positions).  Rows whose target
// equals ignore_index (the library cross-entropy's argument; the training
// step passes -1) are ignored and the mean divides by the valid count
// ("Multi-GPU calculation of gradients for accelerated training",
// "Cross-entropy averages within one micro-batch").  The softmax runs over
// every padded column.
#include "common.h"

namespace g2 {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bool target_valid(int t, int V, int ig) { return t != ig && t >= 0 && t < V; }

// count[0] = number of targets in [0, V) other than ignore_index; ids outside
// [0, V) other than ignore_index raise GPT2_ERR_BAD_ID (and are then treated
// as ignored).  One block.
__global__ __launch_bounds__(1024) void count_targets_kernel(const int32_t* __restrict__ tgt, int n, int V, int ig,
                                                             int* __restrict__ count, int* flag) {
  __shared__ int red[1024];
  int c = 0, bad = 0;
  // 16 loads per thread in flight at a time
  for (int i0 = threadIdx.x; i0 < n; i0 += 16 * blockDim.x) {
    int tv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) tv[u] = i0 + u * (int)blockDim.x < n ? tgt[i0 + u * blockDim.x] : ig;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      c += target_valid(tv[u], V, ig);
      bad |= (tv[u] != ig && (tv[u] < 0 || tv[u] >= V));
    }
  }
  red[threadIdx.x] = c;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) count[0] = red[0];
  if (bad) raise_flag(flag, GPT2_ERR_BAD_ID);
}

// One block per row: online (max, sum of exp) over the row, then
// loss_row = lse - z[target], dlogits = scale / count * (softmax - onehot).
// VEC: V % 4 == 0 and float32 logits, read as float4.
template <typename LT, typename DT, bool VEC>
__global__ __launch_bounds__(256) void ce_rows_kernel(const LT* __restrict__ logits, int64_t ld_l, DT* __restrict__ dl,
                                                      int64_t ld_d, const int32_t* __restrict__ tgt, int V,
                                                      int ig, const int* __restrict__ count, float scale,
                                                      float* __restrict__ row_loss) {
  const int r = blockIdx.x;
  const LT* z = logits + (int64_t)r * ld_l;
  float m = -INFINITY, s = 0.f;
  auto upd = [&](float x) {
    x *= LOG2E;
    if (x > m) {
      s = s * exp2f(m - x) + 1.f;
      m = x;
    } else {
      s += exp2f(x - m);
    }
  };
  if constexpr (VEC) {
    const float4* z4 = reinterpret_cast<const float4*>(z);
    for (int v = threadIdx.x; v < V / 4; v += 256) {
      const float4 q = z4[v];
      // one max per group of four, then the four exponentials
      const float mx = fmaxf(fmaxf(q.x, q.y), fmaxf(q.z, q.w)) * LOG2E;
      if (mx > m) {
        s *= exp2f(m - mx);
        m = mx;
      }
      s += exp2f(q.x * LOG2E - m) + exp2f(q.y * LOG2E - m) + exp2f(q.z * LOG2E - m) + exp2f(q.w * LOG2E - m);
    }
  } else {
    for (int v = threadIdx.x; v < V; v += 256) upd(to_f<LT>(z[v]));
  }
  __shared__ float sm[256], ss[256];
  sm[threadIdx.x] = m;
  ss[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) {
      const float m1 = sm[threadIdx.x], m2 = sm[threadIdx.x + k];
      const float mm = fmaxf(m1, m2);
      const float s1 = ss[threadIdx.x] * (m1 == -INFINITY ? 0.f : exp2f(m1 - mm));
      const float s2 = ss[threadIdx.x + k] * (m2 == -INFINITY ? 0.f : exp2f(m2 - mm));
      sm[threadIdx.x] = mm;
      ss[threadIdx.x] = s1 + s2;
    }
    __syncthreads();
  }
  const float lse2 = sm[0] + log2f(ss[0]);  // log2-domain log-sum-exp
  const int t = tgt[r];
  const bool valid = target_valid(t, V, ig);
  const int n = count[0];
  if (threadIdx.x == 0) row_loss[r] = valid ? (lse2 * LN2 - to_f<LT>(z[t])) : 0.f;
  const float coef = (valid && n > 0) ? scale / (float)n : 0.f;
  DT* d = dl + (int64_t)r * ld_d;
  if constexpr (VEC) {
    const float4* z4 = reinterpret_cast<const float4*>(z);
    for (int v = threadIdx.x; v < V / 4; v += 256) {
      const float4 q = z4[v];
      float o[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = coef * (exp2f(o[e] * LOG2E - lse2) - (4 * v + e == t ? 1.f : 0.f));
      if constexpr (sizeof(DT) == 2) {
        bf16x4 ob;
#pragma unroll
        for (int e = 0; e < 4; ++e) ob[e] = f2bf(o[e]);
        *reinterpret_cast<bf16x4*>(d + 4 * v) = ob;
      } else {
        *reinterpret_cast<float4*>(d + 4 * v) = make_float4(o[0], o[1], o[2], o[3]);
      }
    }
  } else {
    for (int v = threadIdx.x; v < V; v += 256) {
      const float p = exp2f(to_f<LT>(z[v]) * LOG2E - lse2);
      d[v] = from_f<DT>(coef * (p - (v == t ? 1.f : 0.f)));
    }
  }
}

// loss = sum(row_loss) / count, or NaN with GPT2_WARN_NO_TARGETS if count = 0.
__global__ __launch_bounds__(1024) void ce_finish_kernel(const float* __restrict__ row_loss, int n,
                                                         const int* __restrict__ count, float* __restrict__ loss,
                                                         int* flag) {
  __shared__ float red[1024];
  float s = 0.f;
  // this thread's rows i, i + blockDim, ... in increasing order, 16 loads in
  // flight at a time
  for (int i0 = threadIdx.x; i0 < n; i0 += 16 * blockDim.x) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = i0 + u * (int)blockDim.x < n ? row_loss[i0 + u * blockDim.x] : 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (i0 + u * (int)blockDim.x < n) s += v[u];
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int k = 512; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int c = count[0];
    if (c > 0) {
      loss[0] = red[0] / (float)c;
    } else {
      loss[0] = __builtin_nanf("");
      raise_flag(flag, GPT2_WARN_NO_TARGETS);
    }
  }
}

// One block per row of the fused path.  From the per-tile statistics
// (mx_t, s_t) of row r: lse = max_t mx_t + log(sum_t s_t exp(mx_t - max)).
// The target logit is recomputed in float32 as hidden[r] . wte[target], and
// loss_r = lse - z_target.  Then y[r][n] = z - mx_t(n) is overwritten with
// dlogits = scale / count * (exp(z - lse) - [n == target]), the target entry
// from the float32 logit.  Rows with an ignored target get zeros.
__global__ __launch_bounds__(256) void ce_apply_kernel(bf16* __restrict__ y, const float2* __restrict__ stats,
                                                       int tiles, const bf16* __restrict__ hidden,
                                                       const bf16* __restrict__ wte, const int32_t* __restrict__ tgt,
                                                       int V, int C, int ig, const int* __restrict__ count,
                                                       float scale, float* __restrict__ row_loss) {
  extern __shared__ float shift[];  // [tiles]: mx_t - lse, then scratch
  __shared__ float red[256 / 64];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float2* st = stats + (int64_t)r * tiles;
  auto block_max = [&](float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    if (lane == 0) red[wave] = v;
    __syncthreads();
    v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return v;
  };
  auto block_sum = [&](float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) red[wave] = v;
    __syncthreads();
    v = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return v;
  };
  float mx = -INFINITY;
  for (int t = tid; t < tiles; t += 256) mx = fmaxf(mx, st[t].x);
  mx = block_max(mx);
  float sm = 0.f;
  for (int t = tid; t < tiles; t += 256) {
    const float2 s2 = st[t];
    sm += s2.y * exp2f((s2.x - mx) * LOG2E);
  }
  sm = block_sum(sm);
  const float lse = mx + log2f(sm) * LN2;
  for (int t = tid; t < tiles; t += 256) shift[t] = (st[t].x - lse) * LOG2E;
  const int t = tgt[r];
  const bool valid = target_valid(t, V, ig);
  float zt = 0.f;
  if (valid) {
    const bf16* h = hidden + (int64_t)r * C;
    const bf16* w = wte + (int64_t)t * C;
    for (int c = tid; c < C; c += 256) zt = fmaf(bf2f(h[c]), bf2f(w[c]), zt);
  }
  zt = block_sum(zt);  // also orders the shift[] writes before their reads
  const int n = count[0];
  const float coef = (valid && n > 0) ? scale / (float)n : 0.f;
  if (tid == 0) row_loss[r] = valid ? lse - zt : 0.f;
  const float dt = coef * (exp2f((zt - lse) * LOG2E) - 1.f);
  bf16* yr = y + (int64_t)r * V;
  auto apply = [&](int c8, bf16x8 v) {
    const int n0 = 8 * c8;
    const float sh = shift[n0 / kCeTile];
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = coef * __builtin_amdgcn_exp2f(fmaf(bf2f(v[e]), LOG2E, sh));
    if (valid && t >= n0 && t < n0 + 8) o[t - n0] = dt;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2v pr = __builtin_convertvector((f32x2v){o[e], o[e + 1]}, bf16x2v);
      v[e] = pr[0];
      v[e + 1] = pr[1];
    }
    *reinterpret_cast<bf16x8*>(yr + n0) = v;
  };
  // eight 16-byte loads in flight per lane before the first store (the
  // stores go to the same row, so the compiler would not hoist the next
  // load above them): four were worth 1.5% of this kernel's time against
  // one, eight another 1% (21.43 -> 21.22 ms per GPT-2 step, same box)
  constexpr int U = 8;
  const int nc = V / 8;
  int c8 = tid;
  for (; c8 + 256 * (U - 1) < nc; c8 += 256 * U) {
    bf16x8 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const bf16x8*>(yr + 8 * (c8 + 256 * u));
#pragma unroll
    for (int u = 0; u < U; ++u) apply(c8 + 256 * u, v[u]);
  }
  for (; c8 < nc; c8 += 256) apply(c8, *reinterpret_cast<const bf16x8*>(yr + 8 * c8));
}

hipError_t launch_ce_apply(const Launch& L, bf16* y, const float2* stats, const bf16* hidden, const bf16* wte,
                           const int32_t* tgt, int rows, int V, int C, int ignore_index, const int* count,
                           float scale, float* row_loss) {
  const int tiles = ce_stat_tiles(V);
  prof_begin(L);
  ce_apply_kernel<<<rows, 256, tiles * sizeof(float), L.stream>>>(y, stats, tiles, hidden, wte, tgt, V, C,
                                                                   ignore_index, count, scale, row_loss);
  prof_end(L);
  return hipGetLastError();
}

hipError_t launch_count_targets(const Launch& L, const int32_t* tgt, int n, int V, int ignore_index, int* count,
                                int* flag) {
  prof_begin(L);
  count_targets_kernel<<<1, 1024, 0, L.stream>>>(tgt, n, V, ignore_index, count, flag);
  prof_end(L);
  return hipGetLastError();
}

template <typename LT, typename DT>
hipError_t launch_ce_rows(const Launch& L, const LT* logits, int64_t ld_logits, DT* dlogits, int64_t ld_d,
                          const int32_t* tgt, int rows, int V, const int* count, float scale, float* /*loss_sum*/,
                          float* row_loss) {
  prof_begin(L);
  const bool vec = sizeof(LT) == 4 && V % 4 == 0 && ld_logits % 4 == 0 && ld_d % 4 == 0;
  if (vec)
    ce_rows_kernel<LT, DT, true><<<rows, 256, 0, L.stream>>>(logits, ld_logits, dlogits, ld_d, tgt, V, -1, count,
                                                             scale, row_loss);
  else
    ce_rows_kernel<LT, DT, false><<<rows, 256, 0, L.stream>>>(logits, ld_logits, dlogits, ld_d, tgt, V, -1, count,
                                                              scale, row_loss);
  prof_end(L);
  return hipGetLastError();
}
template hipError_t launch_ce_rows<float, float>(const Launch&, const float*, int64_t, float*, int64_t, const int32_t*,
                                                int, int, const int*, float, float*, float*);

hipError_t launch_ce_finish_n(const Launch& L, const float* row_loss, int n, const int* count, float* loss, int* flag) {
  prof_begin(L);
  ce_finish_kernel<<<1, 1024, 0, L.stream>>>(row_loss, n, count, loss, flag);
  prof_end(L);
  return hipGetLastError();
}

}  // namespace g2
