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
#include <algorithm>
#include <utility>

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

// ---- deterministic scatter-add: dst[key[i], :] += src[i, :] for rows i of
// [N, C], each destination row summing its source rows in increasing i, so
// the result does not depend on scheduling (float addition is not
// associative; atomics would make the gradient vary from run to run).
//  1. a stable LSD radix sort (8-bit digits) of (key, row) pairs: rows come
//     out grouped by key and, within a key, in increasing row order;
//  2. the sorted list in tiles of 32 positions: each tile sums every run of
//     one key that falls inside it, in order; a run that is the key's whole
//     run is added to dst there, otherwise its sum goes to part[first
//     position of the run in the tile];
//  3. per tile, the key whose run starts in it and continues past its end
//     adds the partials of its tiles, in tile order, to dst.
// Every destination row has exactly one writer, in a fixed order.
constexpr int kScatTile = 32;

__global__ __launch_bounds__(256) void scat_keys_tok_kernel(const int32_t* __restrict__ tok, int N, int V,
                                                            int32_t* __restrict__ key, int32_t* __restrict__ val) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  const int id = tok[i];
  key[i] = (id < 0 || id >= V) ? 0 : id;  // the forward flagged it and read row 0
  val[i] = i;
}
__global__ __launch_bounds__(256) void scat_keys_pos_kernel(const int32_t* __restrict__ seg, int N, int T,
                                                            int32_t* __restrict__ key, int32_t* __restrict__ val) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  key[i] = min(max(i % T - seg[i], 0), T - 1);  // (starts from segment_start_kernel are in range)
  val[i] = i;
}

// Exclusive scan of n ints in place by one block of 1024 threads: chunks of
// 4096 staged through LDS (coalesced), four consecutive elements per
// thread, wave scans by shuffles, the 16 wave totals scanned by one wave,
// a running carry between chunks.
__global__ __launch_bounds__(1024) void scat_scan_kernel(int* __restrict__ a, int n) {
  __shared__ int buf[4096];
  __shared__ int wtot[16];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int carry = 0;
  for (int base = 0; base < n; base += 4096) {
    const int m = min(4096, n - base);
    for (int i = t; i < m; i += 1024) buf[i] = a[base + i];
    __syncthreads();
    int x[4], s = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      x[u] = 4 * t + u < m ? buf[4 * t + u] : 0;
      s += x[u];
    }
    int inc = s;  // inclusive scan of the thread totals within the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(inc, d);
      if (lane >= d) inc += v;
    }
    if (lane == 63) wtot[wave] = inc;
    __syncthreads();
    if (wave == 0) {
      int w = lane < 16 ? wtot[lane] : 0;
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) {
        const int v = __shfl_up(w, d);
        if (lane >= d) w += v;
      }
      if (lane < 16) wtot[lane] = w;  // inclusive over the waves
    }
    __syncthreads();
    int run = carry + (wave ? wtot[wave - 1] : 0) + inc - s;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (4 * t + u < m) buf[4 * t + u] = run;
      run += x[u];
    }
    carry += wtot[15];
    __syncthreads();
    for (int i = t; i < m; i += 1024) a[base + i] = buf[i];
    __syncthreads();
  }
}

// Radix pass, digit (key >> shift) & 255; nb blocks of 256 elements.
// hist[d * nb + block] = how many of the block's elements have digit d.
__global__ __launch_bounds__(256) void radix_hist_kernel(const int32_t* __restrict__ key, int N, int shift,
                                                         int* __restrict__ hist) {
  __shared__ int h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < N) atomicAdd(&h[(key[i] >> shift) & 255], 1);
  __syncthreads();
  hist[threadIdx.x * gridDim.x + blockIdx.x] = h[threadIdx.x];
}
// Stable scatter: an element's place among the block's elements of its digit
// is the count of those before it (lanes below it in its wave, found with
// ballots on the digit's 8 bits, plus the earlier waves' counts).
__global__ __launch_bounds__(256) void radix_scatter_kernel(const int32_t* __restrict__ key,
                                                            const int32_t* __restrict__ val, int N, int shift,
                                                            const int* __restrict__ off, int32_t* __restrict__ key2,
                                                            int32_t* __restrict__ val2) {
  __shared__ int wc[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int j = threadIdx.x; j < 4 * 256; j += 256) (&wc[0][0])[j] = 0;
  __syncthreads();
  const int i = blockIdx.x * 256 + threadIdx.x;
  const bool ok = i < N;
  const int k = ok ? key[i] : 0;
  const int d = (k >> shift) & 255;
  uint64_t same = __ballot(ok);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint64_t m = __ballot((d >> b) & 1);
    same &= ((d >> b) & 1) ? m : ~m;
  }
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  const int rank = __popcll(same & below);
  if (ok && rank == 0) wc[wave][d] = __popcll(same);
  __syncthreads();
  if (!ok) return;
  int pos = off[d * gridDim.x + blockIdx.x] + rank;
  for (int w = 0; w < wave; ++w) pos += wc[w][d];
  key2[pos] = k;
  val2[pos] = val[i];
}

// Step 2 over the sorted (key, row) list.  A thread owns columns c, c + 256,
// ...; it loads the tile's 32 source values of a column first (independent
// loads in flight together), then sums the runs in order.
__global__ __launch_bounds__(256) void scat_tile_kernel(const int32_t* __restrict__ skey,
                                                        const int32_t* __restrict__ srow, int N,
                                                        const float* __restrict__ src, int C,
                                                        float* __restrict__ dst, float* __restrict__ part) {
  __shared__ int key[kScatTile + 2], row[kScatTile];
  const int p0 = blockIdx.x * kScatTile, n = min(N - p0, kScatTile);
  if (threadIdx.x < n) {
    key[threadIdx.x + 1] = skey[p0 + threadIdx.x];
    row[threadIdx.x] = srow[p0 + threadIdx.x];
  }
  if (threadIdx.x == 0) {
    key[0] = p0 > 0 ? skey[p0 - 1] : -1;      // the key before the tile
    key[n + 1] = p0 + n < N ? skey[p0 + n] : -1;  // and after it
  }
  __syncthreads();
  // run structure (the same for every column): end[j] = a run ends at j;
  // whole[j] = and it is its key's whole run, added to dst here; otherwise
  // its sum goes to part at the run's first position head[j]
  __shared__ bool end[kScatTile], whole[kScatTile];
  __shared__ int head[kScatTile];
  if (threadIdx.x == 0) {
    int a = 0;
    for (int j = 0; j < kScatTile; ++j) {
      end[j] = j < n && (key[j + 2] != key[j + 1] || j + 1 == n);
      if (end[j]) {
        const int k = key[j + 1];
        whole[j] = !(a == 0 && key[0] == k) && !(j + 1 == n && key[n + 1] == k);
        head[j] = a;
        a = j + 1;
      }
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    float v[kScatTile], d[kScatTile];
#pragma unroll
    for (int j = 0; j < kScatTile; ++j) v[j] = j < n ? src[(int64_t)row[j] * C + c] : 0.f;
    // the dst rows the tile adds to, loaded together
#pragma unroll
    for (int j = 0; j < kScatTile; ++j) d[j] = end[j] && whole[j] ? dst[(int64_t)key[j + 1] * C + c] : 0.f;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kScatTile; ++j) {
      acc += v[j];
      if (end[j]) {
        if (whole[j]) dst[(int64_t)key[j + 1] * C + c] = d[j] + acc;
        else part[(int64_t)(p0 + head[j]) * C + c] = acc;
        acc = 0.f;
      }
    }
  }
}
// Step 3: block t joins the key whose run starts in tile t and continues
// past its end (at most one per tile).  The tile's keys and every tile's
// first key are staged in LDS, so finding the run's extent takes no
// dependent global loads.
constexpr int kScatMaxTiles = 4096;  // tile-start keys held in LDS: N <= 131,072
__global__ __launch_bounds__(1024) void scat_join_kernel(const int32_t* __restrict__ skey, int N, int C,
                                                        const float* __restrict__ part, float* __restrict__ dst) {
  __shared__ int tk[kScatTile], first[kScatMaxTiles];
  __shared__ int s_a, s_m;
  const int t = blockIdx.x, ntiles = (N + kScatTile - 1) / kScatTile;
  const int p0 = t * kScatTile, p1 = min(N, p0 + kScatTile);
  if (p1 >= N) return;  // the last tile's runs end inside it
  if (threadIdx.x < p1 - p0) tk[threadIdx.x] = skey[p0 + threadIdx.x];
  for (int i = t + 1 + threadIdx.x; i < ntiles; i += blockDim.x) first[i] = skey[i * kScatTile];
  __syncthreads();
  if (threadIdx.x == 0) {
    const int k = tk[p1 - p0 - 1];
    int a = p1 - p0 - 1, m = 0;
    if (first[t + 1] == k) {  // the tile's last run continues past its end
      while (a > 0 && tk[a - 1] == k) --a;
      if (!(a == 0 && p0 > 0 && skey[p0 - 1] == k)) {  // and began in this tile
        m = 1;
        while (t + 1 + m < ntiles && first[t + 1 + m] == k) ++m;  // tiles t+1 .. t+m hold the rest
      }
    }
    s_a = p0 + a;
    s_m = m;
  }
  __syncthreads();
  const int m = s_m, a = s_a;
  if (m == 0) return;
  const int k = tk[p1 - p0 - 1];
  // partials at a, then at the starts of tiles t+1 .. t+m; loaded 8 at a time,
  // added in that order
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    float acc = part[(int64_t)a * C + c];
    for (int i = 1; i <= m; i += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = i + u <= m ? part[(int64_t)(p0 + (i + u) * kScatTile) * C + c] : 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (i + u <= m) acc += v[u];
    }
    dst[(int64_t)k * C + c] += acc;
  }
}

size_t det_scatter_scratch(int N) {
  const size_t nb = (size_t)(N + 255) / 256;
  return (4 * (size_t)N + 256 * nb) * sizeof(int) + 256;
}

// keys in [0, nkeys); part: [N, C] float32 scratch; ws: det_scatter_scratch(N) bytes.
static hipError_t det_scatter_add(const Launch& L, bool by_token, const int32_t* ids, int N, int nkeys, int T,
                                  const float* src, int C, float* dst, float* part, void* ws) {
  if ((N + kScatTile - 1) / kScatTile > kScatMaxTiles) return hipErrorInvalidValue;
  const int nb = (N + 255) / 256;
  int32_t* k0 = static_cast<int32_t*>(ws);
  int32_t* v0 = k0 + N;
  int32_t* k1 = v0 + N;
  int32_t* v1 = k1 + N;
  int* hist = v1 + N;
  if (by_token) scat_keys_tok_kernel<<<nb, 256, 0, L.stream>>>(ids, N, nkeys, k0, v0);
  else scat_keys_pos_kernel<<<nb, 256, 0, L.stream>>>(ids, N, T, k0, v0);
  for (int shift = 0; (nkeys - 1) >> shift; shift += 8) {
    radix_hist_kernel<<<nb, 256, 0, L.stream>>>(k0, N, shift, hist);
    scat_scan_kernel<<<1, 1024, 0, L.stream>>>(hist, 256 * nb);
    radix_scatter_kernel<<<nb, 256, 0, L.stream>>>(k0, v0, N, shift, hist, k1, v1);
    std::swap(k0, k1);
    std::swap(v0, v1);
  }
  // the join: one thread per column (up to 1024; more columns loop); the
  // tiles: 256 threads, so that several blocks share a compute unit
  const int ntiles = (N + kScatTile - 1) / kScatTile, nt = std::min(1024, std::max(64, (C + 63) / 64 * 64));
  scat_tile_kernel<<<ntiles, 256, 0, L.stream>>>(k0, v0, N, src, C, dst, part);
  scat_join_kernel<<<ntiles, nt, 0, L.stream>>>(k0, N, C, part, dst);
  return hipGetLastError();
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

size_t embed_bwd_scratch(int rows) { return det_scatter_scratch(rows); }
int embed_bwd_max_rows() { return kScatMaxTiles * kScatTile; }

hipError_t launch_embed_bwd(const Launch& L, const int32_t* tok, const float* dr, float* dwte, float* dwpe, int B,
                            int T, int C, int V, const int32_t* seg, float* part, void* ws) {
  prof_begin(L);
  const int N = B * T;
  hipError_t e = det_scatter_add(L, true, tok, N, V, T, dr, C, dwte, part, ws);
  if (e == hipSuccess && dwpe) {
    if (seg) {  // restarted positions: another scatter
      e = det_scatter_add(L, false, seg, N, T, T, dr, C, dwpe, part, ws);
    } else {
      const int64_t n = (int64_t)T * C;
      embed_bwd_wpe_kernel<<<(unsigned)((n + 255) / 256), 256, 0, L.stream>>>(dr, dwpe, B, T, C);
      e = hipGetLastError();
    }
  }
  prof_end(L);
  return e;
}

}  // namespace g2
