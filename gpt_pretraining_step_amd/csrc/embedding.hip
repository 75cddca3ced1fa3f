// Token + position embedding ("How I trained my own GPT-2 124M on
// FineWeb-Edu" 2.2 and 2.10: x = wte[idx] + wpe[0..T-1]) and its backward.
// The tied wte also receives the lm_head gradient elsewhere (section 4).
// Without a position table (wpe == NULL: the rotary variant of "Reproduce
// GPT-2 124M", whose model holds no wpe) x = wte[idx].
//
// Packed windows with a document mask ("GPT" chapter of Zero to Frontier,
// "Document boundaries, packing and masking"): a document begins at its EOT
// token, and position ids restart there, x = wte[idx] + wpe[t - seg[t]], with
// seg the document starts computed here from the tokens.
#include "common.h"

namespace g2 {

// seg[b, t] = max{ s <= t : tok[b, s] == eot } (0 if none): an inclusive
// max-scan of (tok == eot ? t : 0) along the row.  One block per row, 256
// positions per pass, the running maximum carried between passes.
__global__ __launch_bounds__(256) void segment_start_kernel(const int32_t* __restrict__ tok, int32_t* __restrict__ seg,
                                                            int T, int eot) {
  __shared__ int wave_max[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t* tr = tok + (int64_t)blockIdx.x * T;
  int32_t* sr = seg + (int64_t)blockIdx.x * T;
  int carry = 0;
  for (int t0 = 0; t0 < T; t0 += 256) {
    const int t = t0 + threadIdx.x;
    int v = (t < T && tr[t] == eot) ? t : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(v, d);
      if (lane >= d) v = max(v, u);
    }
    if (lane == 63) wave_max[wave] = v;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wave; ++w) before = max(before, wave_max[w]);
    if (t < T) sr[t] = max(v, before);
    carry = max(max(carry, wave_max[0]), max(wave_max[1], max(wave_max[2], wave_max[3])));
    __syncthreads();  // wave_max is rewritten by the next pass
  }
}

// out[b,t,:] = wte[tok[b,t],:] + wpe[t,:] (float32).  Out-of-range ids raise
// GPT2_ERR_BAD_ID and are clamped to 0 so the gather stays in bounds.
__global__ __launch_bounds__(256) void embed_fwd_kernel(const int32_t* __restrict__ tok, const float* __restrict__ wte,
                                                        const float* __restrict__ wpe, float* __restrict__ out, int BT,
                                                        int T, int C, int V, int* flag,
                                                        const int32_t* __restrict__ seg) {
  const int row = blockIdx.x;
  if (row >= BT) return;
  int id = tok[row];
  if (id < 0 || id >= V) {
    if (threadIdx.x == 0) raise_flag(flag, GPT2_ERR_BAD_ID);
    id = 0;
  }
  const int t = seg ? row % T - seg[row] : row % T;
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

// dwte[tok[b,t], :] += dR[b,t,:]  (atomics: repeated ids share rows); with
// restarted positions also dwpe[t - seg[b,t], :] += dR[b,t,:]
__global__ __launch_bounds__(256) void embed_bwd_wte_kernel(const int32_t* __restrict__ tok,
                                                            const float* __restrict__ dr, float* __restrict__ dwte,
                                                            int BT, int T, int C, int V,
                                                            const int32_t* __restrict__ seg,
                                                            float* __restrict__ dwpe) {
  const int row = blockIdx.x;
  if (row >= BT) return;
  int id = tok[row];
  if (id < 0 || id >= V) id = 0;
  const float* g = dr + (int64_t)row * C;
  float* d = dwte + (int64_t)id * C;
  for (int c = threadIdx.x; c < C; c += blockDim.x) unsafeAtomicAdd(d + c, g[c]);
  if (seg && dwpe) {
    float* dp = dwpe + (int64_t)(row % T - seg[row]) * C;
    for (int c = threadIdx.x; c < C; c += blockDim.x) unsafeAtomicAdd(dp + c, g[c]);
  }
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

hipError_t launch_segment_starts(const Launch& L, const int32_t* tok, int B, int T, int eot, int32_t* seg) {
  prof_begin(L);
  segment_start_kernel<<<B, 256, 0, L.stream>>>(tok, seg, T, eot);
  prof_end(L);
  return hipGetLastError();
}

hipError_t launch_embed_fwd(const Launch& L, const int32_t* tok, const float* wte, const float* wpe, float* out, int B,
                            int T, int C, int V, int* flag, const int32_t* seg) {
  prof_begin(L);
  embed_fwd_kernel<<<B * T, 256, 0, L.stream>>>(tok, wte, wpe, out, B * T, T, C, V, flag, seg);
  prof_end(L);
  return hipGetLastError();
}

hipError_t launch_embed_bwd(const Launch& L, const int32_t* tok, const float* dr, float* dwte, float* dwpe, int B,
                            int T, int C, int V, const int32_t* seg) {
  prof_begin(L);
  embed_bwd_wte_kernel<<<B * T, 256, 0, L.stream>>>(tok, dr, dwte, B * T, T, C, V, seg, dwpe);
  const int64_t n = (int64_t)T * C;
  if (dwpe && !seg) embed_bwd_wpe_kernel<<<(unsigned)((n + 255) / 256), 256, 0, L.stream>>>(dr, dwpe, B, T, C);
  prof_end(L);
  return hipGetLastError();
}

}  // namespace g2
