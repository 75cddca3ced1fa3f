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
//  1. a stable sort of (key, row) pairs by key (LSD radix passes of 8-bit
//     digits over the grid): rows come out grouped by key and, within a
//     key, in increasing row order;
//  2. the sorted list in tiles of 32 positions: each tile sums every run of
//     one key that falls inside it, in order; a run that is the key's whole
//     run is added to dst there, otherwise its sum goes to part[first
//     position of the run in the tile];
//  3. per tile, the key whose run starts in it and continues past its end
//     adds the partials of its tiles, in tile order, to dst.
// Every destination row has exactly one writer, in a fixed order.
constexpr int kScatTile = 32;
constexpr int kScatMaxTiles = 4096;  // rows one call sorts: at most 131,072

template <int VW>
struct FVec;
template <>
struct FVec<1> {
  using T = float;
  static __device__ __forceinline__ T zero() { return 0.f; }
  static __device__ __forceinline__ T add(T a, T b) { return a + b; }
};
template <>
struct FVec<2> {
  using T = float2;
  static __device__ __forceinline__ T zero() { return make_float2(0.f, 0.f); }
  static __device__ __forceinline__ T add(T a, T b) { return make_float2(a.x + b.x, a.y + b.y); }
};
template <>
struct FVec<4> {
  using T = float4;
  static __device__ __forceinline__ T zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  static __device__ __forceinline__ T add(T a, T b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }
};

// Step 1: LSD radix passes over 8-bit digits of the key, 1,024 elements per
// block (one per thread), two launches per pass.
//  count: block b's digit histogram -> hist[d * nb + b] (the first pass
//         also forms the keys and the row indices, in row order);
//  place: block b finds, for every digit d, its first position: the count
//         of smaller digits overall plus the count of d in blocks before b;
//         each wave ranks its 64 elements among the lanes of equal digit
//         (ballots on the digit's 8 bits), the waves' counts are prefixed in
//         wave order, and every element goes to first[d] + (earlier waves'
//         count of d) + rank.
// Each pass is stable, so the result is sorted by (key, row).
constexpr int kRadixBlock = 1024;
__device__ __forceinline__ int scat_key(const int32_t* __restrict__ ids, int i, int nkeys, int T, bool by_token) {
  if (by_token) {
    const int id = ids[i];
    return (id < 0 || id >= nkeys) ? 0 : id;  // the forward flagged it and read row 0
  }
  return min(max(i % T - ids[i], 0), T - 1);  // (starts from segment_start_kernel are in range)
}

// dwpe[t, :] += sum_b dR[b,t,:], b in increasing order (no atomics): thread
// e owns VW columns of one position, its B loads in flight 16 at a time.
template <int VW>
__device__ __forceinline__ void wpe_sum(const float* __restrict__ dr, float* __restrict__ dwpe, int B, int T, int C,
                                        int64_t e) {
  using F = FVec<VW>;
  using VT = typename F::T;
  const int64_t i = e * VW;
  const int64_t TC = (int64_t)T * C;
  if (i >= TC) return;
  VT s = *reinterpret_cast<const VT*>(dr + i);
  for (int b0 = 1; b0 < B; b0 += 16) {
    VT v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = *reinterpret_cast<const VT*>(dr + (b0 + u < B ? b0 + u : 0) * TC + i);
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (b0 + u < B) s = F::add(s, v[u]);
  }
  VT* o = reinterpret_cast<VT*>(dwpe + i);
  *o = F::add(*o, s);
}

// Blocks [0, nb) count; with WVW > 0 the blocks after them sum the position
// table's gradient (wpe_sum, VW = WVW), independent work that fills the
// compute units the sort leaves idle.
template <bool FIRST, int WVW>
__global__ __launch_bounds__(kRadixBlock) void radix_count_kernel(const int32_t* __restrict__ ids, int N, int nb,
                                                                  int nkeys, int T, int by_token, int shift,
                                                                  int32_t* __restrict__ key,
                                                                  int32_t* __restrict__ val, int* __restrict__ hist,
                                                                  const float* __restrict__ wsrc,
                                                                  float* __restrict__ wdst, int B, int C) {
  if constexpr (WVW > 0) {
    if ((int)blockIdx.x >= nb) {
      wpe_sum<WVW>(wsrc, wdst, B, T, C, (int64_t)(blockIdx.x - nb) * kRadixBlock + threadIdx.x);
      return;
    }
  }
  __shared__ int h[256];
  if (threadIdx.x < 256) h[threadIdx.x] = 0;
  __syncthreads();
  const int i = blockIdx.x * kRadixBlock + threadIdx.x;
  if (i < N) {
    int k;
    if constexpr (FIRST) {
      k = scat_key(ids, i, nkeys, T, by_token != 0);
      key[i] = k;
      val[i] = i;
    } else {
      k = key[i];
    }
    atomicAdd(&h[(k >> shift) & 255], 1);
  }
  __syncthreads();
  if (threadIdx.x < 256) hist[threadIdx.x * nb + blockIdx.x] = h[threadIdx.x];
}

__global__ __launch_bounds__(kRadixBlock) void radix_place_kernel(const int32_t* __restrict__ key,
                                                                  const int32_t* __restrict__ val, int N, int shift,
                                                                  const int* __restrict__ hist,
                                                                  int32_t* __restrict__ key2,
                                                                  int32_t* __restrict__ val2) {
  __shared__ int first[256];
  __shared__ int wc[kRadixBlock / 64][256];
  __shared__ int wsum[4];
  const int nb = gridDim.x, blk = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // per digit (threads 0..255): its elements in earlier blocks, and in all
  int before = 0, total = 0;
  if (tid < 256) {
    const int* hd = hist + tid * nb;
    for (int j0 = 0; j0 < nb; j0 += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = j0 + u < nb ? hd[j0 + u] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        total += c[u];
        before += j0 + u < blk ? c[u] : 0;
      }
    }
  }
  int inc = total;  // inclusive scan of the totals within each wave of digits
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(inc, d);
    if (lane >= d) inc += v;
  }
  if (tid < 256 && lane == 63) wsum[wave] = inc;
  for (int d = lane; d < 256; d += 64) wc[wave][d] = 0;
  // this wave's 64 elements: rank among the lanes of equal digit
  const int i = blk * kRadixBlock + tid;
  const bool ok = i < N;
  const int k = ok ? key[i] : 0;
  const int dg = (k >> shift) & 255;
  uint64_t same = __ballot(ok);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const uint64_t m = __ballot((dg >> bit) & 1);
    same &= ((dg >> bit) & 1) ? m : ~m;
  }
  const int rank = __popcll(same & ((1ull << lane) - 1));
  __syncthreads();  // wsum and the zeroed wc rows are complete
  if (ok && rank == 0) wc[wave][dg] = __popcll(same);
  if (tid < 256) {
    int off = inc - total + before;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    first[tid] = off;
  }
  __syncthreads();
  if (tid < 256) {  // per digit: the waves' counts -> counts of earlier waves
    int run = 0;
    for (int w = 0; w < kRadixBlock / 64; ++w) {
      const int c = wc[w][tid];
      wc[w][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  if (ok) {
    const int pos = first[dg] + wc[wave][dg] + rank;
    key2[pos] = k;
    val2[pos] = val[i];
  }
}

// Step 2 over the sorted (key, row) list, one block per tile.  Wave 0 finds
// the tile's runs with ballots: for each position j, whether a run ends there
// (end), whether that run is its key's whole run (whole: it neither began
// before the tile nor continues after it) and the run's first position in
// the tile (head).  Every thread then owns VW adjacent columns: it loads the
// tile's 32 source rows and the destination rows of its whole runs (all
// independent loads in flight together), sums the runs in order, and writes
// dst (whole runs) or part[p0 + head] (the others).
template <int VW>
__global__ __launch_bounds__(512) void scat_tile_kernel(const int32_t* __restrict__ skey,
                                                        const int32_t* __restrict__ srow, int N,
                                                        const float* __restrict__ src, int C,
                                                        float* __restrict__ dst, float* __restrict__ part) {
  using F = FVec<VW>;
  using VT = typename F::T;
  // per position j, as element offsets (N C and V C stay below 2^31,
  // checked by the host): the source row; the dst row read for a whole run
  // ending at j (else the tile's first key's, read and not written); where
  // a run ending at j goes (kind 1: dst, 2: part, 0: no run ends at j)
  __shared__ int s_src[kScatTile], s_ld[kScatTile], s_st[kScatTile], s_kind[kScatTile];
  const int p0 = blockIdx.x * kScatTile, n = min(N - p0, kScatTile);
  if (threadIdx.x < 64) {
    const int l = threadIdx.x;
    const bool in = l < n;
    const int k = in ? skey[p0 + l] : -1;
    const int kprev = p0 > 0 ? skey[p0 - 1] : -1;   // the key before the tile
    const int knext = p0 + n < N ? skey[p0 + n] : -1;  // and after it
    const int kl = __shfl(k, l > 0 ? l - 1 : 0), kr = __shfl(k, l + 1 < 64 ? l + 1 : 63);
    const uint64_t heads = __ballot(in && (l == 0 || kl != k));
    const int head = 63 - __clzll(heads & ((2ull << l) - 1));
    const bool end = in && (l == n - 1 || kr != k);
    const bool whole = end && !(head == 0 && kprev == k) && !(l == n - 1 && knext == k);
    const int k0 = __shfl(k, 0), r0 = srow[p0];
    if (l < kScatTile) {
      s_src[l] = (in ? srow[p0 + l] : r0) * C;
      s_ld[l] = (whole ? k : k0) * C;
      s_st[l] = whole ? k * C : (p0 + head) * C;
      s_kind[l] = whole ? 1 : end ? 2 : 0;
    }
  }
  __syncthreads();
  for (int c = VW * threadIdx.x; c < C; c += VW * blockDim.x) {
    // the tile in two halves of 16 positions (fewer registers, so that two
    // blocks share a compute unit); the run sum carries across
    VT acc = F::zero();
#pragma unroll
    for (int h = 0; h < kScatTile; h += kScatTile / 2) {
      VT v[kScatTile / 2], d[kScatTile / 2];
#pragma unroll
      for (int j = 0; j < kScatTile / 2; ++j) v[j] = *reinterpret_cast<const VT*>(src + (uint32_t)(s_src[h + j] + c));
#pragma unroll
      for (int j = 0; j < kScatTile / 2; ++j) d[j] = *reinterpret_cast<const VT*>(dst + (uint32_t)(s_ld[h + j] + c));
#pragma unroll
      for (int j = 0; j < kScatTile / 2; ++j) {
        acc = F::add(acc, v[j]);
        const int kind = s_kind[h + j];
        if (kind == 1) *reinterpret_cast<VT*>(dst + (uint32_t)(s_st[h + j] + c)) = F::add(d[j], acc);
        else if (kind == 2) *reinterpret_cast<VT*>(part + (uint32_t)(s_st[h + j] + c)) = acc;
        if (kind) acc = F::zero();
      }
    }
  }
}
// Step 3: block t joins the key whose run starts in tile t and continues
// past its end (at most one per tile): its partials are the one at the
// run's first position a and those at the first positions of tiles t+1 ..
// t+m.  The block's threads form G groups of one thread per VW columns;
// group g sums the g-th contiguous share of the partials in order, and the
// G group sums are then added in group order (a fixed order for a given m).
template <int VW>
__global__ __launch_bounds__(1024) void scat_join_kernel(const int32_t* __restrict__ skey, int N, int C,
                                                        const float* __restrict__ part, float* __restrict__ dst) {
  using F = FVec<VW>;
  using VT = typename F::T;
  __shared__ int s_a, s_k, s_own;
  __shared__ VT gsum[1024];
  const int t = blockIdx.x, ntiles = (N + kScatTile - 1) / kScatTile;
  const int p0 = t * kScatTile, p1 = min(N, p0 + kScatTile);
  if (p1 >= N) return;  // the last tile's runs end inside it
  if (threadIdx.x < 64) {
    // the tile's keys and its two neighbours in one round of loads
    const int l = threadIdx.x;
    const int kl = p0 + l < p1 ? skey[p0 + l] : -1;
    const int kafter = skey[p1], kbefore = p0 > 0 ? skey[p0 - 1] : -1;
    const int k = __shfl(kl, p1 - p0 - 1);  // the tile's last key
    const uint64_t eq = __ballot(kl == k);  // a suffix of the tile
    const int a = p0 + __ffsll((long long)eq) - 1;
    if (l == 0) {
      s_k = k;
      s_a = a;
      // the run continues past the tile and began in it
      s_own = kafter == k && (a > p0 || kbefore != k);
    }
  }
  __syncthreads();
  if (!s_own) return;
  const int a = s_a, k = s_k;
  // tiles after t whose first key is k: consecutive, since the keys are sorted
  __shared__ int s_m;
  if (threadIdx.x == 0) s_m = 0;
  __syncthreads();
  int cm = 0;
  for (int i = t + 1 + (int)threadIdx.x; i < ntiles; i += blockDim.x) cm += skey[i * kScatTile] == k;
  if (cm) atomicAdd(&s_m, cm);
  __syncthreads();
  const int np = s_m + 1;  // partials: at a, then at p0 + 32 i for i = 1 .. m
  const int cw = (C + VW - 1) / VW;                     // threads per row of columns
  const int gw = (cw + 63) / 64 * 64;                   // a group: whole waves
  const int G = gw <= (int)blockDim.x ? (int)blockDim.x / gw : 1;
  const int g = G > 1 ? (int)threadIdx.x / gw : 0;
  const int ct = G > 1 ? (int)threadIdx.x % gw : (int)threadIdx.x;
  const int cstride = G > 1 ? gw : (int)blockDim.x;
  const int lo = g * np / G, hi = (g + 1) * np / G;
  auto pos = [&](int i) { return i == 0 ? a : p0 + i * kScatTile; };
  // (G > 1) group 0 reads the destination row together with its partials
  VT old = F::zero();
  if (G > 1 && g == 0 && VW * ct < C) old = *reinterpret_cast<const VT*>(dst + (int64_t)k * C + VW * ct);
  for (int c = VW * ct; c < C; c += VW * cstride) {
    VT acc = F::zero();
    if (g < G && lo < hi) {
      acc = *reinterpret_cast<const VT*>(part + (int64_t)pos(lo) * C + c);
      for (int i = lo + 1; i < hi; i += 16) {
        VT v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          v[u] = *reinterpret_cast<const VT*>(part + (int64_t)pos(i + u < hi ? i + u : lo) * C + c);
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (i + u < hi) acc = F::add(acc, v[u]);
      }
    }
    if (G == 1) {
      VT* o = reinterpret_cast<VT*>(dst + (int64_t)k * C + c);
      *o = F::add(*o, acc);
    } else {
      gsum[threadIdx.x] = acc;
    }
  }
  if (G == 1) return;
  __syncthreads();
  if (g == 0 && VW * ct < C) {
    VT tot = gsum[ct];
    for (int h = 1; h < G; ++h)
      if (h * np / G < (h + 1) * np / G) tot = F::add(tot, gsum[h * gw + ct]);
    *reinterpret_cast<VT*>(dst + (int64_t)k * C + VW * ct) = F::add(old, tot);
  }
}

size_t det_scatter_scratch(int N) {
  const size_t nb = (size_t)(N + kRadixBlock - 1) / kRadixBlock;
  return (4 * (size_t)N + 256 * nb) * sizeof(int) + 256;
}

// keys in [0, nkeys); part: [N, C] float32 scratch; ws: det_scatter_scratch(N) bytes.
// With wpe != NULL (and B * T == N) the first launch also runs wpe_sum of src
// into wpe.
static hipError_t det_scatter_add(const Launch& L, bool by_token, const int32_t* ids, int N, int nkeys, int T,
                                  const float* src, int C, float* dst, float* part, void* ws, float* wpe = nullptr,
                                  int B = 0) {
  if ((N + kScatTile - 1) / kScatTile > kScatMaxTiles) return hipErrorInvalidValue;
  // the tile pass addresses rows with 32-bit element offsets
  if ((int64_t)N * C >= ((int64_t)1 << 31) || (int64_t)nkeys * C >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int nb = (N + kRadixBlock - 1) / kRadixBlock;
  int32_t* k0 = static_cast<int32_t*>(ws);
  int32_t* v0 = k0 + N;
  int32_t* k1 = v0 + N;
  int32_t* v1 = k1 + N;
  int* hist = v1 + N;
  const int64_t TC = (int64_t)T * C;
  const bool wvec = (C % 4) == 0 && ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(wpe)) & 15) == 0;
  const int nw = wpe ? (int)((TC / (wvec ? 4 : 1) + kRadixBlock - 1) / kRadixBlock) : 0;
  for (int shift = 0; shift == 0 || ((nkeys - 1) >> shift); shift += 8) {
    const int bt = by_token ? 1 : 0;
    if (shift == 0 && !wpe)
      radix_count_kernel<true, 0><<<nb, kRadixBlock, 0, L.stream>>>(ids, N, nb, nkeys, T, bt, shift, k0, v0, hist,
                                                                    nullptr, nullptr, 0, C);
    else if (shift == 0 && wvec)
      radix_count_kernel<true, 4><<<nb + nw, kRadixBlock, 0, L.stream>>>(ids, N, nb, nkeys, T, bt, shift, k0, v0,
                                                                         hist, src, wpe, B, C);
    else if (shift == 0)
      radix_count_kernel<true, 1><<<nb + nw, kRadixBlock, 0, L.stream>>>(ids, N, nb, nkeys, T, bt, shift, k0, v0,
                                                                         hist, src, wpe, B, C);
    else
      radix_count_kernel<false, 0><<<nb, kRadixBlock, 0, L.stream>>>(nullptr, N, nb, nkeys, T, 0, shift, k0, v0, hist,
                                                                     nullptr, nullptr, 0, C);
    if (nkeys > 1) {
      radix_place_kernel<<<nb, kRadixBlock, 0, L.stream>>>(k0, v0, N, shift, hist, k1, v1);
      std::swap(k0, k1);
      std::swap(v0, v1);
    }
  }
  // tiles: one thread per VW columns; the join: up to 1024 threads in
  // groups of one row of columns
  const int ntiles = (N + kScatTile - 1) / kScatTile;
  const bool vec = (C % 4) == 0 && ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) |
                                     reinterpret_cast<uintptr_t>(part)) & 15) == 0;
  auto threads = [](int cols) { return std::min(512, std::max(64, (cols + 63) / 64 * 64)); };
  if (vec) {
    scat_tile_kernel<2><<<ntiles, threads(C / 2), 0, L.stream>>>(k0, v0, N, src, C, dst, part);
    scat_join_kernel<4><<<ntiles, 1024, 0, L.stream>>>(k0, N, C, part, dst);
  } else {
    scat_tile_kernel<1><<<ntiles, threads(C), 0, L.stream>>>(k0, v0, N, src, C, dst, part);
    scat_join_kernel<1><<<ntiles, 1024, 0, L.stream>>>(k0, N, C, part, dst);
  }
  return hipGetLastError();
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
  // without a document mask the position table's gradient is summed by
  // extra blocks of the sort's first launch; with one, positions restart,
  // and a second sorted scatter adds it
  hipError_t e = det_scatter_add(L, true, tok, N, V, T, dr, C, dwte, part, ws, seg ? nullptr : dwpe, B);
  if (e == hipSuccess && dwpe && seg) e = det_scatter_add(L, false, seg, N, T, T, dr, C, dwpe, part, ws);
  prof_end(L);
  return e;
}

}  // namespace g2
