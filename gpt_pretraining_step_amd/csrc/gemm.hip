// Matrix products of the training step.
//
// bf16: the multi-stage MFMA kernel of gemm_kernel.h on 256x256 tiles.
// float32 (FP32 precision mode, small models): a float32-MFMA kernel on
// 64x64 tiles with the same operand layouts and epilogues.
//
// The epilogues fuse what follows each product in the step: bias, the
// residual add of the block ("How I trained my own GPT-2 124M on
// FineWeb-Edu" 2.11/2.13, the += additions), the tanh GELU of the MLP
// (2.13), its derivative in the backward, and accumulation into float32
// gradients (section 8.1: grads add up over micro-steps).  Weight-gradient
// products can also sum the rows of their first operand, which is the bias
// gradient of the same Linear.
#include "gemm_kernel.h"

#include <algorithm>
#include <cstring>
#include <functional>
#include <mutex>
#include <vector>

namespace g2 {

// ------------------------------------------------------- float32 MFMA GEMM
//
// FP32 precision mode: v_mfma_f32_32x32x2_f32 on 64x64 block tiles (4 waves,
// each one 32x32 MFMA tile), K step 16 staged through LDS as [k][row] for
// either operand layout (ragged edges read as zeros), float32 accumulation;
// the same epilogues as the bf16 kernel, element by element.  The MFMA takes
// A[row = lane % 32][k = lane / 32] and B[k = lane / 32][col = lane % 32]
// and leaves D[8 (r / 4) + 4 (lane / 32) + r % 4][lane % 32] in register r.

template <bool A_K, bool B_K, int EPI, bool ATOMIC>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmP p) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 1];
  __shared__ float Bs[BK][BN + 1];
  const int tm = blockIdx.x % p.tiles_m;
  const int rest = blockIdx.x / p.tiles_m;
  const int tn = rest % p.tiles_n;
  const int split = rest / p.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = split * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const int lr = lane & 31, lg = lane >> 5;
  const float* A = static_cast<const float*>(p.A);
  const float* B = static_cast<const float*>(p.B);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    for (int e = threadIdx.x; e < BM * BK; e += 256) {
      int mm, kk;
      if (A_K) { mm = e / BK; kk = e % BK; } else { kk = e / BM; mm = e % BM; }
      const int gm = m0 + mm, gk = k0 + kk;
      float v = 0.f;
      if (gm < p.M && gk < kend) v = A_K ? A[(int64_t)gm * p.lda + gk] : A[(int64_t)gk * p.lda + gm];
      As[kk][mm] = v;
    }
    for (int e = threadIdx.x; e < BN * BK; e += 256) {
      int nn, kk;
      if (B_K) { nn = e / BK; kk = e % BK; } else { kk = e / BN; nn = e % BN; }
      const int gn = n0 + nn, gk = k0 + kk;
      float v = 0.f;
      if (gn < p.N && gk < kend) v = B_K ? B[(int64_t)gn * p.ldb + gk] : B[(int64_t)gk * p.ldb + gn];
      Bs[kk][nn] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 2)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[kk + lg][wm + lr], Bs[kk + lg][wn + lr], acc, 0, 0, 0);
    __syncthreads();
  }
  const int n = n0 + wn + lr;
  if (n >= p.N) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + wm + 8 * (r >> 2) + 4 * lg + (r & 3);
    if (m < p.M) epi_store<EPI, false, ATOMIC>(p, m, n, acc[r]);
  }
}

// ------------------------------------------------------------- dispatching

static GemmP make_params(const gpt2_gemm_args& a) {
  GemmP p{};
  p.M = a.M; p.N = a.N; p.K = a.K;
  p.lda = a.lda; p.ldb = a.ldb; p.ldc = a.ldc;
  p.A = a.A; p.B = a.B; p.C = a.C; p.C2 = a.C2; p.R = a.R; p.U = a.U; p.bias = a.bias;
  p.alpha = a.alpha;
  p.rope = static_cast<const float2*>(a.rope);
  p.rope_period = a.rope_period;
  p.rope_cols = a.rope_cols;
  p.ld2 = a.ld2;
  p.splits = 1;
  p.k_per_split = a.K;
  return p;
}

// Launch one instantiation of the bf16 kernel (its LDS stages are static).
template <int BM, int BN, int BK, int WGM, int WGN, int ST, bool A_K, bool B_K, int EPI, bool OB, bool AT, bool SW = false>
static hipError_t launch_v2(const Launch& L, const GemmP& p) {
  auto kern = gemm2_kernel<BM, BN, BK, WGM, WGN, ST, A_K, B_K, EPI, OB, AT, SW>;
  dim3 grid(p.tiles_m * p.tiles_n * p.splits), block(64 * WGM * WGN);
  kern<<<grid, block, 0, L.stream>>>(p);
  return hipGetLastError();
}

// bf16 products: 256 x BN block tiles (BN = 256: 8 waves of 128x64; BN =
// 192: 12 waves of 64x64, three per SIMD, which hide the fragment reads
// better than 8 waves of 64x96 did), K step 64, two LDS stages fed by DMA.  Most
// epilogues keep 32 consecutive columns of a row per instruction (coalesced
// scalar loads, stores and atomics: the fewest row segments per
// instruction); the residual of a long-K product (K >= 2048) measured faster
// with 4 consecutive columns per lane (16-byte loads of R and stores).
template <int BN, int WGM, int WGN, bool A_K, bool B_K>
static hipError_t dispatch_tile(const Launch& L, GemmP p, int epi, bool ob) {
  constexpr int BM = 256, BK = 64, ST = 2;
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  const bool at = p.splits > 1;
  hipError_t e;
  prof_begin(L);
  switch (epi) {
    case GPT2_EPI_STORE:
      e = ob ? launch_v2<BM, BN, BK, WGM, WGN, ST, A_K, B_K, GPT2_EPI_STORE, true, false>(L, p)
             : launch_v2<BM, BN, BK, WGM, WGN, ST, A_K, B_K, GPT2_EPI_STORE, false, false>(L, p);
      break;
    case GPT2_EPI_RESIDUAL:
      e = p.K >= 2048 ? launch_v2<BM, BN, BK, WGM, WGN, ST, A_K, B_K, GPT2_EPI_RESIDUAL, false, false, true>(L, p)
                      : launch_v2<BM, BN, BK, WGM, WGN, ST, A_K, B_K, GPT2_EPI_RESIDUAL, false, false, false>(L, p);
      break;
    case GPT2_EPI_GELU:
      e = launch_v2<BM, BN, BK, WGM, WGN, ST, A_K, B_K, GPT2_EPI_GELU, true, false>(L, p);
      break;
    case GPT2_EPI_DGELU:
      e = launch_v2<BM, BN, BK, WGM, WGN, ST, A_K, B_K, GPT2_EPI_DGELU, true, false, false>(L, p);
      break;
    case GPT2_EPI_GELU_GRAD:
      e = launch_v2<BM, BN, BK, WGM, WGN, ST, A_K, B_K, GPT2_EPI_GELU_GRAD, true, false>(L, p);
      break;
    case GPT2_EPI_MUL:
      e = launch_v2<BM, BN, BK, WGM, WGN, ST, A_K, B_K, GPT2_EPI_MUL, true, false, false>(L, p);
      break;
    case GPT2_EPI_ROPE:
    case GPT2_EPI_SWIGLU:
      // paired columns in one lane: 64 columns per wave (256-wide tiles), forward layout
      if constexpr (BN == 256 && A_K && B_K) {
        // (RoPE measured alike in both layouts; SwiGLU faster unswapped)
        e = epi == GPT2_EPI_ROPE ? launch_v2<BM, BN, BK, WGM, WGN, ST, true, true, GPT2_EPI_ROPE, true, false, true>(L, p)
                                 : launch_v2<BM, BN, BK, WGM, WGN, ST, true, true, GPT2_EPI_SWIGLU, true, false, false>(L, p);
      } else {
        e = hipErrorInvalidValue;
      }
      break;
    case GPT2_EPI_SWIGLU_BWD:
      if constexpr (A_K && !B_K) e = launch_v2<BM, BN, BK, WGM, WGN, ST, true, false, GPT2_EPI_SWIGLU_BWD, true, false, false>(L, p);
      else e = hipErrorInvalidValue;
      break;
    default:
      e = at ? launch_v2<BM, BN, BK, WGM, WGN, ST, A_K, B_K, GPT2_EPI_ACCUMULATE, false, true>(L, p)
             : launch_v2<BM, BN, BK, WGM, WGN, ST, A_K, B_K, GPT2_EPI_ACCUMULATE, false, false>(L, p);
      break;
  }
  prof_end(L);
  return e;
}

constexpr int kUnits = 256;  // compute units: one block each per round

// Split-K count for an accumulating product (each split adds its partial
// sums atomically): the count that minimises the rounds of blocks over the
// compute units per unit of work, keeping at least 16 K steps per split; a
// larger count must save at least 3%.
static int choose_splits(long tiles, int K, int BK) {
  int best = 1;
  double best_cost = (double)((tiles + kUnits - 1) / kUnits);
  for (int s = 2; s <= 32 && K / s >= 16 * BK; ++s) {
    const double cost = (double)((tiles * s + kUnits - 1) / kUnits) / s;
    if (cost < 0.97 * best_cost) {
      best = s;
      best_cost = cost;
    }
  }
  return best;
}

// Relative time of a product under 256 x bn block tiles: rounds of blocks
// per split times the tile width.
static double tiling_cost(int M, int N, int K, int bn, bool accumulate, int* splits) {
  const long tiles = (long)((M + 255) / 256) * ((N + bn - 1) / bn);
  *splits = accumulate ? choose_splits(tiles, K, 64) : 1;
  return (double)((tiles * *splits + kUnits - 1) / kUnits) / *splits * bn;
}

template <bool A_K, bool B_K>
static hipError_t dispatch_bf16(const Launch& L, GemmP p, int epi, bool ob) {
  const bool acc = epi == GPT2_EPI_ACCUMULATE;
  int s256 = 1, s192 = 1;
  const double c256 = tiling_cost(p.M, p.N, p.K, 256, acc, &s256);
  const double c192 = tiling_cost(p.M, p.N, p.K, 192, acc, &s192);
  // the narrower tile re-reads A more often: take it only for a clear gain;
  // the paired epilogues need 64 columns per wave
  const bool narrow = c192 < 0.9 * c256 && epi != GPT2_EPI_ROPE && epi != GPT2_EPI_SWIGLU;
  const int splits = narrow ? s192 : s256;
  p.k_per_split = (p.K + splits * 64 - 1) / (splits * 64) * 64;
  p.splits = (p.K + p.k_per_split - 1) / p.k_per_split;
  if (narrow) return dispatch_tile<192, 4, 3, A_K, B_K>(L, p, epi, ob);
  // 256 x 256: 8 waves of 128 x 64, except the GELU_GRAD product with both
  // operands K-major (the GPT-2 fc), 16 waves of 64 x 64 (41.2 -> 40.0 ms
  // per step, same box).  Measured slower at 16 waves: the residual
  // (rotary attn_proj 12.2 -> 14.4 ms per step), the paired rotary /
  // SwiGLU epilogues (30.8 -> 32.5 ms), and with a K-slow operand the
  // mlp_proj_dx product (39.1 -> 44.4 ms).
  if constexpr (A_K && B_K) {
    if (epi == GPT2_EPI_GELU_GRAD) return dispatch_tile<256, 4, 4, A_K, B_K>(L, p, epi, ob);
  }
  return dispatch_tile<256, 2, 4, A_K, B_K>(L, p, epi, ob);
}

template <bool A_K, bool B_K>
static hipError_t dispatch_f32(const Launch& L, GemmP p, int epi) {
  p.tiles_m = (p.M + 63) / 64;
  p.tiles_n = (p.N + 63) / 64;
  dim3 grid(p.tiles_m * p.tiles_n * p.splits), block(256);
  const bool atomic = p.splits > 1;
  prof_begin(L);
  switch (epi) {
    case GPT2_EPI_STORE: gemm_f32_kernel<A_K, B_K, GPT2_EPI_STORE, false><<<grid, block, 0, L.stream>>>(p); break;
    case GPT2_EPI_RESIDUAL: gemm_f32_kernel<A_K, B_K, GPT2_EPI_RESIDUAL, false><<<grid, block, 0, L.stream>>>(p); break;
    case GPT2_EPI_GELU: gemm_f32_kernel<A_K, B_K, GPT2_EPI_GELU, false><<<grid, block, 0, L.stream>>>(p); break;
    case GPT2_EPI_DGELU: gemm_f32_kernel<A_K, B_K, GPT2_EPI_DGELU, false><<<grid, block, 0, L.stream>>>(p); break;
    case GPT2_EPI_GELU_GRAD: gemm_f32_kernel<A_K, B_K, GPT2_EPI_GELU_GRAD, false><<<grid, block, 0, L.stream>>>(p); break;
    case GPT2_EPI_MUL: gemm_f32_kernel<A_K, B_K, GPT2_EPI_MUL, false><<<grid, block, 0, L.stream>>>(p); break;
    default:
      if (atomic) gemm_f32_kernel<A_K, B_K, GPT2_EPI_ACCUMULATE, true><<<grid, block, 0, L.stream>>>(p);
      else gemm_f32_kernel<A_K, B_K, GPT2_EPI_ACCUMULATE, false><<<grid, block, 0, L.stream>>>(p);
      break;
  }
  prof_end(L);
  return hipGetLastError();
}

// Number of K splits for accumulate-into products whose output has few tiles
// (the weight gradients: small outputs, K = tokens).  Partial products are
// added with float32 atomics, whose cost grows with the split count, so the
// grid is filled to about one block per CU and no further.
hipError_t launch_gemm_ce_stats(const Launch& L, const bf16* hidden, const bf16* wte, bf16* y, float2* stats, int M,
                                int V, int C) {
  constexpr int BM = 256, BN = kCeTile, BK = 64, WGM = 2, WGN = 4, ST = 2;
  GemmP p{};
  p.M = M; p.N = V; p.K = C;
  p.lda = C; p.ldb = C; p.ldc = V;
  p.A = hidden; p.B = wte; p.C = y;
  p.stats = stats;
  p.alpha = 1.f;
  p.splits = 1;
  p.k_per_split = C;
  p.tiles_m = (M + BM - 1) / BM;
  p.tiles_n = (V + BN - 1) / BN;
  prof_begin(L);
  const hipError_t e = launch_v2<BM, BN, BK, WGM, WGN, ST, true, true, EPI_CE_STATS, true, false, true>(L, p);
  prof_end(L);
  return e;
}

hipError_t launch_gemm(const Launch& L, const gpt2_gemm_args& a, float* row_sum) {
  GemmP p = make_params(a);
  p.row_sum = row_sum;
  const bool ak = a.a_kmajor != 0, bk = a.b_kmajor != 0;
  if (a.dtype == GPT2_PRECISION_FP32) {
    if (a.epilogue == GPT2_EPI_ACCUMULATE) {
      const int tiles = ((a.M + 63) / 64) * ((a.N + 63) / 64);
      p.splits = 1;
      while (tiles * p.splits * 2 <= 2 * kUnits && a.K / (p.splits * 2) >= 64) p.splits *= 2;
      p.k_per_split = ((a.K + p.splits * 16 - 1) / (p.splits * 16)) * 16;
      p.splits = (a.K + p.k_per_split - 1) / p.k_per_split;
    }
    if (ak && bk) return dispatch_f32<true, true>(L, p, a.epilogue);
    if (ak && !bk) return dispatch_f32<true, false>(L, p, a.epilogue);
    if (!ak && bk) return dispatch_f32<false, true>(L, p, a.epilogue);
    return dispatch_f32<false, false>(L, p, a.epilogue);
  }
  const bool ob = a.out_bf16 != 0;
  if (ak && bk) return dispatch_bf16<true, true>(L, p, a.epilogue, ob);
  if (ak && !bk) return dispatch_bf16<true, false>(L, p, a.epilogue, ob);
  if (!ak && bk) return dispatch_bf16<false, true>(L, p, a.epilogue, ob);
  return dispatch_bf16<false, false>(L, p, a.epilogue, ob);
}

// ------------------------------------------------------- grouped products
//
// One block per 256x256 output tile, whole K, so the launch runs in rounds of
// kUnits equal blocks.  A partial last round would leave CUs idle for a whole
// tile's time: the products at the end of the list that cover the tiles past
// the last full round are split in K into kTailSplit pieces (each adds its
// partial sums atomically), or into two where K is too short for that, when
// a list-scheduling estimate of the launch says the span gets shorter.  The
// pieces then fill the CUs that the last whole tiles leave idle.  Units are
// placed in block order: the whole tiles XCD-aware (each XCD a contiguous run
// of them, sharing panels in its L2), then the pieces, which the round-robin
// hands to every XCD alike.  GPT-2 124M at 16,384 tokens (1,296 tiles, a
// 16-tile tail), same box: pieces of a half 79.6 ms per step, of a quarter
// 76.4, an eighth 76.4, a sixteenth 76.2.

namespace {
constexpr int kGroupTile = 256;
constexpr int kTailSplit = 4;
size_t align256(size_t b) { return (b + 255) / 256 * 256; }
int group_tiles(const gpt2_gemm_args& a) {
  return ((a.M + kGroupTile - 1) / kGroupTile) * ((a.N + kGroupTile - 1) / kGroupTile);
}
// In-order list scheduling over kUnits CUs: u0 units of cost c0, then u1 of
// cost c1, each starting on the CU that frees up first; returns the span.
double list_span(int64_t u0, double c0, int64_t u1, double c1) {
  std::vector<double> load(kUnits, 0.0);  // a min-heap of CU finish times
  std::make_heap(load.begin(), load.end(), std::greater<double>());
  for (int64_t i = 0; i < u0 + u1; ++i) {
    std::pop_heap(load.begin(), load.end(), std::greater<double>());
    load.back() += i < u0 ? c0 : c1;
    std::push_heap(load.begin(), load.end(), std::greater<double>());
  }
  return *std::max_element(load.begin(), load.end());
}
// K splits of each product (1, 2 or kTailSplit); returns the unit count
int64_t group_plan(const gpt2_gemm_args* a, int n, std::vector<int>& splits) {
  splits.assign(n, 1);
  int64_t tiles = 0;
  for (int i = 0; i < n; ++i) tiles += group_tiles(a[i]);
  const int64_t tail = tiles % kUnits;
  if (tiles > kUnits && tail > 0) {
    for (int s = kTailSplit; s >= 2; s /= 2) {
      std::vector<int> sp(n, 1);
      int64_t covered = 0;
      int kmin = a[n - 1].K;
      for (int i = n - 1; i >= 0 && covered < tail; --i) {
        if (a[i].K < s * 16 * 64) break;  // pieces keep at least 16 K steps
        sp[i] = s;
        covered += group_tiles(a[i]);
        kmin = std::min(kmin, a[i].K);
      }
      // a table holds at most two units per tile
      if (covered < tail || covered * (s - 1) > tiles) continue;
      // costs in K steps; a tile's float32 read-modify-write epilogue as in
      // the pair plan below (an atomic one 8 times as much)
      const double k = (kmin + 63) / 64, whole = k + 4.0, piece = (k + s - 1) / s + 32.0;
      if (list_span(tiles - covered, whole, covered * s, piece) < 0.99 * list_span(tiles, whole, 0, 0.0)) {
        splits = sp;
        break;
      }
    }
  }
  int64_t units = 0;
  for (int i = 0; i < n; ++i) units += (int64_t)group_tiles(a[i]) * splits[i];
  return units;
}
}  // namespace

int gemm_grouped_units(const gpt2_gemm_args* a, int n) {
  std::vector<int> splits;
  const int64_t u = group_plan(a, n, splits);
  int64_t largest = 0;
  for (int i = 0; i < n; ++i) largest = std::max<int64_t>(largest, (int64_t)group_tiles(a[i]) * splits[i]);
  return u < (1 << 30) && largest <= 0xffff && n <= 0x7fff ? (int)u : -1;
}

size_t gemm_grouped_table_bytes(int n, int units) {
  return align256(n * sizeof(GemmP)) + align256((size_t)units * sizeof(int));
}

// Host image of the table: parameters of every product, then the (product,
// unit) of every block (no pointers into itself: it can be copied anywhere).
void gemm_grouped_table(const gpt2_gemm_args* a, float* const* row_sums, int n, int units, void* host) {
  char* h = static_cast<char*>(host);
  memset(h, 0, gemm_grouped_table_bytes(n, units));
  GemmP* ps = reinterpret_cast<GemmP*>(h);
  int* unit_map = reinterpret_cast<int*>(h + align256(n * sizeof(GemmP)));
  std::vector<int> splits;
  group_plan(a, n, splits);
  std::vector<int> whole, pieces;  // (product << 16) | unit, in product order
  for (int i = 0; i < n; ++i) {
    GemmP p = make_params(a[i]);
    p.row_sum = row_sums ? row_sums[i] : nullptr;
    p.tiles_m = (a[i].M + kGroupTile - 1) / kGroupTile;
    p.tiles_n = (a[i].N + kGroupTile - 1) / kGroupTile;
    if (splits[i] > 1) {
      p.k_per_split = (a[i].K + splits[i] * 64 - 1) / (splits[i] * 64) * 64;
      p.splits = (a[i].K + p.k_per_split - 1) / p.k_per_split;
    }
    ps[i] = p;
    const int nu = p.tiles_m * p.tiles_n * p.splits;
    for (int k = 0; k < nu; ++k) (p.splits > 1 ? pieces : whole).push_back((i << 16) | k);
  }
  // whole tiles: block b of the first 8 * floor(W / 8) takes the unit that
  // gives XCD b % 8 a contiguous run
  const int W = (int)whole.size(), W8 = W / 8 * 8;
  for (int b = 0; b < W; ++b) unit_map[b] = whole[b < W8 ? xcd_remap_host(b, W8) : b];
  for (size_t k = 0; k < pieces.size(); ++k) unit_map[W + k] = pieces[k];
}

hipError_t launch_gemm_grouped(const Launch& L, const void* d_table, int n, int units, int K_all) {
  const char* d = static_cast<const char*>(d_table);
  GemmGroups t;
  t.p = reinterpret_cast<const GemmP*>(d);
  t.unit_map = reinterpret_cast<const int*>(d + align256(n * sizeof(GemmP)));
  prof_begin(L);
  // 16 waves of 64 x 64 (four per SIMD): the weight gradients' transposing
  // fragment reads and MFMAs hide better behind four waves than behind the
  // two of the 8-wave 128 x 64 layout (the grouped launch 83.9 -> 79.6 ms per
  // GPT-2 step, same box); both operands K-slow keep that within 128
  // registers, the K-major layouts would spill
  gemm2_grouped_kernel<kGroupTile, kGroupTile, 64, 4, 4, 2, false, false, GPT2_EPI_ACCUMULATE, false, false, false>
      <<<units, 1024, 0, L.stream>>>(t, K_all);
  prof_end(L);
  return hipGetLastError();
}

// ------------------------------------------------------------ product pairs
//
// Two accumulating products of the lm_head backward for one row chunk, in
// one launch: dZ += dlogits W (A K-major, B K-slow; few output tiles, K = V)
// and dW += dlogits^T Z (both K-slow; many tiles, K = the chunk's rows).  The
// split counts come from a list-scheduling estimate of the launch: units
// are handed in block order to the earliest-free of the 256 CUs, a unit
// costing its K steps plus an epilogue (much longer when it adds
// atomically), and the plan with the shortest estimated span wins.

namespace {
constexpr int kPairTile = 256;
struct PairPlan {
  int s0 = 1, s1 = 1;
  double span = 0.0;
};
PairPlan plan_pair_uncached(int64_t t0, int k0, int64_t t1, int k1) {
  // epilogue of a 256x256 float32 read-modify-write, in K steps; an atomic
  // one is charged 8 times as much (measured: with 2 times, the plan split
  // the lm_head's dZ 7 ways and the launch took 78.4 ms per GPT-2 step; with
  // 8 times it splits 2 ways, 73.1 ms, on the same box)
  constexpr double EPI = 4.0, EPI_ATOMIC = 8 * EPI;
  PairPlan best;
  best.span = 1e300;
  for (int s0 = 1; s0 <= 64 && (s0 == 1 || k0 / s0 >= 8); ++s0)
    for (int s1 = 1; s1 <= 4 && (s1 == 1 || k1 / s1 >= 8); ++s1) {
      const double c0 = (k0 + s0 - 1) / s0 + (s0 > 1 ? EPI_ATOMIC : EPI);
      const double c1 = (k1 + s1 - 1) / s1 + (s1 > 1 ? EPI_ATOMIC : EPI);
      const double span = list_span(t0 * s0, c0, t1 * s1, c1);
      if (span < 0.99 * best.span) {
        best.s0 = s0;
        best.s1 = s1;
        best.span = span;
      }
    }
  return best;
}
// The search above costs milliseconds of host time; a training step asks
// for the same few shapes every micro-step, so plans are kept.
PairPlan plan_pair(const gpt2_gemm_args& a0, const gpt2_gemm_args& a1) {
  const int64_t t0 = (int64_t)((a0.M + kPairTile - 1) / kPairTile) * ((a0.N + kPairTile - 1) / kPairTile);
  const int64_t t1 = (int64_t)((a1.M + kPairTile - 1) / kPairTile) * ((a1.N + kPairTile - 1) / kPairTile);
  const int k0 = (a0.K + 63) / 64, k1 = (a1.K + 63) / 64;
  struct Entry {
    int64_t t0, t1;
    int k0, k1;
    PairPlan plan;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  {
    std::lock_guard<std::mutex> lk(mu);
    for (const Entry& e : cache)
      if (e.t0 == t0 && e.t1 == t1 && e.k0 == k0 && e.k1 == k1) return e.plan;
  }
  const PairPlan pl = plan_pair_uncached(t0, k0, t1, k1);
  std::lock_guard<std::mutex> lk(mu);
  if (cache.size() >= 256) cache.erase(cache.begin());
  cache.push_back(Entry{t0, t1, k0, k1, pl});
  return pl;
}
GemmP pair_params(const gpt2_gemm_args& a, int splits) {
  GemmP p = make_params(a);
  p.tiles_m = (a.M + kPairTile - 1) / kPairTile;
  p.tiles_n = (a.N + kPairTile - 1) / kPairTile;
  p.k_per_split = (a.K + splits * 64 - 1) / (splits * 64) * 64;
  p.splits = (a.K + p.k_per_split - 1) / p.k_per_split;
  return p;
}
}  // namespace

hipError_t launch_gemm_pair(const Launch& L, const gpt2_gemm_args& a0, const gpt2_gemm_args& a1) {
  if (!a0.a_kmajor || a0.b_kmajor || a1.a_kmajor || a1.b_kmajor) return hipErrorInvalidValue;
  const PairPlan pl = plan_pair(a0, a1);
  const GemmP p0 = pair_params(a0, pl.s0), p1 = pair_params(a1, pl.s1);
  const int units0 = p0.tiles_m * p0.tiles_n * p0.splits;
  const int units1 = p1.tiles_m * p1.tiles_n * p1.splits;
  prof_begin(L);
  // 16 waves of 64 x 64, as the grouped weight gradients (lm_head backward
  // 74.3 -> 72.6 ms per GPT-2 step, same box)
  gemm2_pair_kernel<kPairTile, kPairTile, 64, 4, 4, true, false, false, false>
      <<<units0 + units1, 1024, 0, L.stream>>>(p0, p1, units0);
  prof_end(L);
  return hipGetLastError();
}

// ------------------------------------------------------------ column sums

template <typename T>
__global__ __launch_bounds__(256) void colsum_kernel(const T* __restrict__ y, int M, int N, int64_t ld,
                                                     float* __restrict__ db, int rows_per_block) {
  __shared__ float red[4][64];
  const int c = blockIdx.x * 64 + (threadIdx.x & 63);
  const int g = threadIdx.x >> 6;
  const int r0 = blockIdx.y * rows_per_block;
  const int r1 = min(M, r0 + rows_per_block);
  float s = 0.f;
  if (c < N)
    for (int r = r0 + g; r < r1; r += 4) s += to_f<T>(y[(int64_t)r * ld + c]);
  red[g][threadIdx.x & 63] = s;
  __syncthreads();
  if (g == 0 && c < N) {
    s = red[0][threadIdx.x] + red[1][threadIdx.x] + red[2][threadIdx.x] + red[3][threadIdx.x];
    unsafeAtomicAdd(db + c, s);
  }
}

hipError_t launch_colsum(const Launch& L, const void* y, int y_bf16, int M, int N, int64_t ld, float* db) {
  const int rpb = 256;
  dim3 grid((N + 63) / 64, (M + rpb - 1) / rpb), block(256);
  prof_begin(L);
  if (y_bf16) colsum_kernel<bf16><<<grid, block, 0, L.stream>>>(static_cast<const bf16*>(y), M, N, ld, db, rpb);
  else colsum_kernel<float><<<grid, block, 0, L.stream>>>(static_cast<const float*>(y), M, N, ld, db, rpb);
  prof_end(L);
  return hipGetLastError();
}

}  // namespace g2
