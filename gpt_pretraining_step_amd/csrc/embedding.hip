// Token + position embedding ("How I trained my own GPT-2 124M on
// FineWeb-Edu" 2.2 and 2.10: x = wte[idx] + wpe[0..T-1]) and its backward.
// The tied wte also receives the lm_head gradient elsewhere (section 4).
// Without a position table (wpe == NULL: the rotary variant of "Reproduce
// GPT-2 124M", whose model holds no wpe) x = wte[idx].
#include "common.h"

namespace g2 {

// out[b,t,:] = wte[tok[b,t],:] + wpe[t,:] (float32).  Out-of-range ids raise
// GPT2_ERR_BAD_ID and are clamped to 0 so the gather stays in bounds.
__global__ __launch_bounds__(256) void embed_fwd_kernel(const int32_t* __restrict__ tok, const float* __restrict__ wte,
                                                        const float* __restrict__ wpe, float* __restrict__ out, int BT,
                                                        int T, int C, int V, int* flag) {
  const int row = blockIdx.x;
  if (row >= BT) return;
  int id = tok[row];
  if (id < 0 || id >= V) {
    if (threadIdx.x == 0) raise_flag(flag, GPT2_ERR_BAD_ID);
    id = 0;
  }
  const int t = row % T;
  const float* a = wte + (int64_t)id * C;
  float* o = out + (int64_t)row * C;
  if (!wpe) {
    for (int c = threadIdx.x; c < C; c += blockDim.x) o[c] = a[c];
    return;
  }
  const float* p = wpe + (int64_t)t * C;
  if ((C & 3) == 0) {
    for (int c = 4 * threadIdx.x; c < C; c += 4 * blockDim.x) {
      float4 x = *reinterpret_cast<const float4*>(a + c);
      float4 y = *reinterpret_cast<const float4*>(p + c);
      *reinterpret_cast<float4*>(o + c) = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
    }
  } else {
    for (int c = threadIdx.x; c < C; c += blockDim.x) o[c] = a[c] + p[c];
  }
}

// dwte[tok[b,t], :] += dR[b,t,:]  (atomics: repeated ids share rows)
__global__ __launch_bounds__(256) void embed_bwd_wte_kernel(const int32_t* __restrict__ tok,
                                                            const float* __restrict__ dr, float* __restrict__ dwte,
                                                            int BT, int C, int V) {
  const int row = blockIdx.x;
  if (row >= BT) return;
  int id = tok[row];
  if (id < 0 || id >= V) id = 0;
  const float* g = dr + (int64_t)row * C;
  float* d = dwte + (int64_t)id * C;
  for (int c = threadIdx.x; c < C; c += blockDim.x) unsafeAtomicAdd(d + c, g[c]);
}

// dwpe[t, :] += sum_b dR[b,t,:]  (one thread per (t, c); no atomics)
__global__ __launch_bounds__(256) void embed_bwd_wpe_kernel(const float* __restrict__ dr, float* __restrict__ dwpe,
                                                            int B, int T, int C) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * C) return;
  const int t = (int)(i / C), c = (int)(i % C);
  float s = 0.f;
  for (int b = 0; b < B; ++b) s += dr[((int64_t)b * T + t) * C + c];
  dwpe[i] += s;
}

hipError_t launch_embed_fwd(const Launch& L, const int32_t* tok, const float* wte, const float* wpe, float* out, int B,
                            int T, int C, int V, int* flag) {
  prof_begin(L);
  embed_fwd_kernel<<<B * T, 256, 0, L.stream>>>(tok, wte, wpe, out, B * T, T, C, V, flag);
  prof_end(L);
  return hipGetLastError();
}

hipError_t launch_embed_bwd(const Launch& L, const int32_t* tok, const float* dr, float* dwte, float* dwpe, int B,
                            int T, int C, int V) {
  prof_begin(L);
  embed_bwd_wte_kernel<<<B * T, 256, 0, L.stream>>>(tok, dr, dwte, B * T, C, V);
  const int64_t n = (int64_t)T * C;
  if (dwpe) embed_bwd_wpe_kernel<<<(unsigned)((n + 255) / 256), 256, 0, L.stream>>>(dr, dwpe, B, T, C);
  prof_end(L);
  return hipGetLastError();
}

}  // namespace g2
