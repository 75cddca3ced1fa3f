// Matrix products of the training step.
//
// bf16 path: MFMA (v_mfma_f32_32x32x16_bf16) tiles with float32 accumulation,
// global -> register -> LDS staging with two LDS buffers (one barrier per K
// step, the next tile's global loads in flight while the current one is
// multiplied).  Operands whose reduction index is the slow one in memory
// (the "transposed" cases of the backward: dX = dY W and dW = dY^T X) are
// transposed in registers 8x8 at a time on their way into LDS, so that every
// LDS read feeding the MFMA is a 16-byte vector along K.
//
// float32 path (FP32 precision mode, small models): a plain LDS-tiled SIMT
// kernel with the same operand layouts and epilogues.
//
// The epilogues fuse what follows each product in the step: bias, the
// residual add of the block ("How I trained my own GPT-2 124M on
// FineWeb-Edu" 2.11/2.13, the += additions), the tanh GELU of the MLP
// (2.13), its derivative in the backward, and accumulation into float32
// gradients (section 8.1: grads add up over micro-steps).
#include "common.h"

namespace g2 {

struct GemmP {
  int M, N, K;
  int64_t lda, ldb, ldc;
  const void* A;
  const void* B;
  void* C;
  void* C2;
  const float* R;
  const void* U;
  const float* bias;
  float alpha;
  int tiles_m, tiles_n, splits, k_per_split;
};

// ------------------------------------------------------------------ epilogue

template <int EPI, bool OUT_BF16, bool ATOMIC>
__device__ __forceinline__ void epi_store(const GemmP& p, int m, int n, float acc) {
  float v = p.alpha * acc;
  if (p.bias) v += p.bias[n];
  const int64_t idx = (int64_t)m * p.ldc + n;
  if constexpr (EPI == GPT2_EPI_STORE) {
    if constexpr (OUT_BF16) static_cast<bf16*>(p.C)[idx] = f2bf(v);
    else static_cast<float*>(p.C)[idx] = v;
  } else if constexpr (EPI == GPT2_EPI_RESIDUAL) {
    static_cast<float*>(p.C)[idx] = p.R[idx] + v;
  } else if constexpr (EPI == GPT2_EPI_GELU) {
    if constexpr (OUT_BF16) {
      bf16 u = f2bf(v);
      static_cast<bf16*>(p.C)[idx] = u;
      static_cast<bf16*>(p.C2)[idx] = f2bf(gelu_tanh(bf2f(u)));
    } else {
      static_cast<float*>(p.C)[idx] = v;
      static_cast<float*>(p.C2)[idx] = gelu_tanh(v);
    }
  } else if constexpr (EPI == GPT2_EPI_DGELU) {
    if constexpr (OUT_BF16) {
      float u = bf2f(static_cast<const bf16*>(p.U)[idx]);
      static_cast<bf16*>(p.C)[idx] = f2bf(v * gelu_tanh_grad(u));
    } else {
      float u = static_cast<const float*>(p.U)[idx];
      static_cast<float*>(p.C)[idx] = v * gelu_tanh_grad(u);
    }
  } else {  // ACCUMULATE
    float* c = static_cast<float*>(p.C) + idx;
    if constexpr (ATOMIC) unsafeAtomicAdd(c, v);
    else *c += v;
  }
}

// ---------------------------------------------------------- bf16 MFMA GEMM

// Tile -> block mapping.  Blocks are handed to the 8 XCDs round-robin; the
// remap makes consecutive logical tiles run on one XCD (sharing its L2), and
// the grouped order walks GROUP_M row tiles per column panel.
__device__ __forceinline__ void tile_of_block(const GemmP& p, int& tm, int& tn, int& split) {
  int bid = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int per_split = p.tiles_m * p.tiles_n;
  split = bid / per_split;
  int t = bid - split * per_split;
  const int GROUP_M = 8;
  const int in_group = GROUP_M * p.tiles_n;
  const int group = t / in_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(p.tiles_m - first_m, GROUP_M);
  const int r = t - group * in_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

union V8 {
  uint4 u;
  bf16x8 v;
  uint32_t w[4];
};

template <int ROWS, int BK, bool KMAJOR>
struct TileLoader {
  // KMAJOR: source stored [rows][ld] with K contiguous; chunk = 8 K-values of one row.
  // !KMAJOR: source stored [K][ld] with rows contiguous; sub-block = 8 K x 8 rows.
  static constexpr int CHUNKS = KMAJOR ? (ROWS * BK / 8) : (ROWS * BK / 64);
  static constexpr int PER_THREAD = (CHUNKS + 255) / 256;
  static constexpr int REGS = KMAJOR ? PER_THREAD : PER_THREAD * 8;
  V8 r[REGS];

  __device__ __forceinline__ void load(const bf16* __restrict__ src, int64_t ld, int row0, int nrows, int k0,
                                       int K) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int id = t + 256 * i;
      if constexpr (KMAJOR) {
        const int row = id / (BK / 8), c8 = id % (BK / 8);
        const int gr = row0 + row, gk = k0 + 8 * c8;
        if (id < CHUNKS && gr < nrows && gk < K)
          r[i].u = *reinterpret_cast<const uint4*>(src + (int64_t)gr * ld + gk);
        else
          r[i].u = make_uint4(0, 0, 0, 0);
      } else {
        const int kb = id / (ROWS / 8), rb = id % (ROWS / 8);
        const int gr = row0 + 8 * rb;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int gk = k0 + 8 * kb + j;
          if (id < CHUNKS && gr < nrows && gk < K)
            r[8 * i + j].u = *reinterpret_cast<const uint4*>(src + (int64_t)gk * ld + gr);
          else
            r[8 * i + j].u = make_uint4(0, 0, 0, 0);
        }
      }
    }
  }

  template <int PITCH>
  __device__ __forceinline__ void store(bf16* lds) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int id = t + 256 * i;
      if (id >= CHUNKS) break;
      if constexpr (KMAJOR) {
        const int row = id / (BK / 8), c8 = id % (BK / 8);
        *reinterpret_cast<uint4*>(lds + row * PITCH + 8 * c8) = r[i].u;
      } else {
        const int kb = id / (ROWS / 8), rb = id % (ROWS / 8);
        // r[8i + j] holds 8 rows (2 per dword) at k = 8kb + j; emit, for each
        // row, the 8 k-values as one 16-byte vector.
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const int word = rr >> 1;
          const bool hi = rr & 1;
          V8 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t a = r[8 * i + 2 * q].w[word];
            uint32_t b = r[8 * i + 2 * q + 1].w[word];
            o.w[q] = hi ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
          }
          *reinterpret_cast<uint4*>(lds + (8 * rb + rr) * PITCH + 8 * kb) = o.u;
        }
      }
    }
  }
};

template <int BM, int BN, int BK, bool A_K, bool B_K, int EPI, bool OUT_BF16, bool ATOMIC>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmP p) {
  constexpr int PITCH = BK + 8;  // 16-byte pad keeps the 32-row MFMA reads conflict-free
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * PITCH];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][BN * PITCH];

  int tm, tn, split;
  tile_of_block(p, tm, tn, split);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = split * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int nk = (kend - kbeg + BK - 1) / BK;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
  const int lr = lane & 31, lg = lane >> 5;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  TileLoader<BM, BK, A_K> la;
  TileLoader<BN, BK, B_K> lb;
  const bf16* Ag = static_cast<const bf16*>(p.A);
  const bf16* Bg = static_cast<const bf16*>(p.B);

  if (nk > 0) {
    la.load(Ag, p.lda, m0, p.M, kbeg, kend);
    lb.load(Bg, p.ldb, n0, p.N, kbeg, kend);
    la.template store<PITCH>(As[0]);
    lb.template store<PITCH>(Bs[0]);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(Ag, p.lda, m0, p.M, kbeg + (kt + 1) * BK, kend);
      lb.load(Bg, p.ldb, n0, p.N, kbeg + (kt + 1) * BK, kend);
    }
    const bf16* as = As[cur];
    const bf16* bs = Bs[cur];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(as + (wm0 + 32 * i + lr) * PITCH + 16 * kk + 8 * lg);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(bs + (wn0 + 32 * j + lr) * PITCH + 16 * kk + 8 * lg);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      la.template store<PITCH>(As[cur ^ 1]);
      lb.template store<PITCH>(Bs[cur ^ 1]);
    }
    __syncthreads();
  }

  // accumulator element r of tile (i, j): row 8*(r/4) + 4*lg + r%4, column lr
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn0 + 32 * j + lr;
      if (n >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm0 + 32 * i + 8 * (r >> 2) + 4 * lg + (r & 3);
        if (m < p.M) epi_store<EPI, OUT_BF16, ATOMIC>(p, m, n, acc[i][j][r]);
      }
    }
}

// ------------------------------------------------------- float32 SIMT GEMM

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
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const float* A = static_cast<const float*>(p.A);
  const float* B = static_cast<const float*>(p.B);
  float acc[4][4] = {};
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
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty + 16 * i, n = n0 + tx + 16 * j;
      if (m < p.M && n < p.N) epi_store<EPI, false, ATOMIC>(p, m, n, acc[i][j]);
    }
}

// ------------------------------------------------------------- dispatching

static GemmP make_params(const gpt2_gemm_args& a) {
  GemmP p;
  p.M = a.M; p.N = a.N; p.K = a.K;
  p.lda = a.lda; p.ldb = a.ldb; p.ldc = a.ldc;
  p.A = a.A; p.B = a.B; p.C = a.C; p.C2 = a.C2; p.R = a.R; p.U = a.U; p.bias = a.bias;
  p.alpha = a.alpha;
  p.splits = 1;
  p.k_per_split = a.K;
  return p;
}

template <int BM, int BN, int BK, bool A_K, bool B_K>
static hipError_t dispatch_epi(const Launch& L, GemmP p, int epi, bool out_bf16) {
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  dim3 grid(p.tiles_m * p.tiles_n * p.splits), block(256);
  const bool atomic = p.splits > 1;
  prof_begin(L);
  switch (epi) {
    case GPT2_EPI_STORE:
      if (out_bf16) gemm_bf16_kernel<BM, BN, BK, A_K, B_K, GPT2_EPI_STORE, true, false><<<grid, block, 0, L.stream>>>(p);
      else gemm_bf16_kernel<BM, BN, BK, A_K, B_K, GPT2_EPI_STORE, false, false><<<grid, block, 0, L.stream>>>(p);
      break;
    case GPT2_EPI_RESIDUAL:
      gemm_bf16_kernel<BM, BN, BK, A_K, B_K, GPT2_EPI_RESIDUAL, false, false><<<grid, block, 0, L.stream>>>(p);
      break;
    case GPT2_EPI_GELU:
      gemm_bf16_kernel<BM, BN, BK, A_K, B_K, GPT2_EPI_GELU, true, false><<<grid, block, 0, L.stream>>>(p);
      break;
    case GPT2_EPI_DGELU:
      gemm_bf16_kernel<BM, BN, BK, A_K, B_K, GPT2_EPI_DGELU, true, false><<<grid, block, 0, L.stream>>>(p);
      break;
    default:
      if (atomic) gemm_bf16_kernel<BM, BN, BK, A_K, B_K, GPT2_EPI_ACCUMULATE, false, true><<<grid, block, 0, L.stream>>>(p);
      else gemm_bf16_kernel<BM, BN, BK, A_K, B_K, GPT2_EPI_ACCUMULATE, false, false><<<grid, block, 0, L.stream>>>(p);
      break;
  }
  prof_end(L);
  return hipGetLastError();
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
    default:
      if (atomic) gemm_f32_kernel<A_K, B_K, GPT2_EPI_ACCUMULATE, true><<<grid, block, 0, L.stream>>>(p);
      else gemm_f32_kernel<A_K, B_K, GPT2_EPI_ACCUMULATE, false><<<grid, block, 0, L.stream>>>(p);
      break;
  }
  prof_end(L);
  return hipGetLastError();
}

// Number of K splits for accumulate-into products whose output has too few
// tiles to fill 256 CUs (the weight gradients: few output tiles, K = tokens).
static int choose_splits(int tiles, int K, int BK) {
  int splits = 1;
  while (tiles * splits < 512 && K / (splits * 2) >= 4 * BK) splits *= 2;
  return splits;
}

hipError_t launch_gemm(const Launch& L, const gpt2_gemm_args& a, int* /*flag*/) {
  GemmP p = make_params(a);
  const bool ak = a.a_kmajor != 0, bk = a.b_kmajor != 0;
  if (a.dtype == GPT2_PRECISION_FP32) {
    if (a.epilogue == GPT2_EPI_ACCUMULATE) {
      const int tiles = ((a.M + 63) / 64) * ((a.N + 63) / 64);
      p.splits = choose_splits(tiles, a.K, 16);
      p.k_per_split = ((a.K + p.splits * 16 - 1) / (p.splits * 16)) * 16;
      p.splits = (a.K + p.k_per_split - 1) / p.k_per_split;
    }
    if (ak && bk) return dispatch_f32<true, true>(L, p, a.epilogue);
    if (ak && !bk) return dispatch_f32<true, false>(L, p, a.epilogue);
    if (!ak && bk) return dispatch_f32<false, true>(L, p, a.epilogue);
    return dispatch_f32<false, false>(L, p, a.epilogue);
  }
  // bf16: 256x128 tiles for tall products with many tiles, 128x128 otherwise.
  constexpr int BK = 64;
  const bool big = (int64_t)((a.M + 255) / 256) * ((a.N + 127) / 128) >= 1024;
  if (a.epilogue == GPT2_EPI_ACCUMULATE) {
    const int tiles = big ? ((a.M + 255) / 256) * ((a.N + 127) / 128) : ((a.M + 127) / 128) * ((a.N + 127) / 128);
    p.splits = choose_splits(tiles, a.K, BK);
    p.k_per_split = ((a.K + p.splits * BK - 1) / (p.splits * BK)) * BK;
    p.splits = (a.K + p.k_per_split - 1) / p.k_per_split;
  }
  const bool ob = a.out_bf16 != 0;
  if (big) {
    if (ak && bk) return dispatch_epi<256, 128, BK, true, true>(L, p, a.epilogue, ob);
    if (ak && !bk) return dispatch_epi<256, 128, BK, true, false>(L, p, a.epilogue, ob);
    if (!ak && bk) return dispatch_epi<256, 128, BK, false, true>(L, p, a.epilogue, ob);
    return dispatch_epi<256, 128, BK, false, false>(L, p, a.epilogue, ob);
  }
  if (ak && bk) return dispatch_epi<128, 128, BK, true, true>(L, p, a.epilogue, ob);
  if (ak && !bk) return dispatch_epi<128, 128, BK, true, false>(L, p, a.epilogue, ob);
  if (!ak && bk) return dispatch_epi<128, 128, BK, false, true>(L, p, a.epilogue, ob);
  return dispatch_epi<128, 128, BK, false, false>(L, p, a.epilogue, ob);
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
