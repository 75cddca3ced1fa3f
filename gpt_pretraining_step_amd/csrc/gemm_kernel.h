// bf16 MFMA GEMM kernel template (dispatch in gemm.hip).
//
// C[m][n] = alpha * sum_k A(m,k) B(n,k), then a fused epilogue.  Block tile
// BM x BN, K step BK, WGM x WGN waves, each wave owning a (BM/WGM) x (BN/WGN)
// sub-tile of 32x32 MFMA tiles (v_mfma_f32_32x32x16_bf16, float32
// accumulators).  STAGES LDS buffers form a pipeline: every operand tile is
// copied from global memory straight into LDS by DMA (global_load_lds_dwordx4),
// so the loads of later K steps are in flight while the current one is
// multiplied.  Operands stored with K contiguous ("K-major") are kept as
// [rows][BK] and fetched with 16-byte LDS reads; operands whose K index is the
// slow one in memory (the backward products) are kept in their memory layout,
// [BK][rows], and fetched with the transposing LDS read (ds_read_b64_tr_b16).
// Tiles carry no padding: 16-byte chunks are XOR-swizzled per row, which keeps
// the DMA writes (1 KB of consecutive bytes per wave instruction) and the
// operand reads free of bank conflicts.
#pragma once

#include "tile_io.h"

#include <type_traits>

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
  float* row_sum;  // optional: row_sum[m] += sum over this product's K of A(m, k) (one column-tile adds it)
  float2* stats;   // EPI_CE_STATS: per (row, column tile) softmax statistics, [M][tiles_n]
  const float2* rope;  // ROPE: (cos, sin) [rope_period][32]
  int rope_period, rope_cols;
  int64_t ld2;  // SWIGLU: row pitch of C2; SWIGLU_BWD: row pitch of U
  float alpha;
  int tiles_m, tiles_n, splits, k_per_split;
  int group_m;  // row tiles walked per column panel (0: 8)
};

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
  } else if constexpr (EPI == GPT2_EPI_GELU_GRAD) {
    float g, dg;
    if constexpr (OUT_BF16) {
      gelu_tanh_and_grad(bf2f(f2bf(v)), g, dg);
      static_cast<bf16*>(p.C)[idx] = f2bf(g);
      static_cast<bf16*>(p.C2)[idx] = f2bf(dg);
    } else {
      gelu_tanh_and_grad(v, g, dg);
      static_cast<float*>(p.C)[idx] = g;
      static_cast<float*>(p.C2)[idx] = dg;
    }
  } else if constexpr (EPI == GPT2_EPI_MUL) {
    if constexpr (OUT_BF16) static_cast<bf16*>(p.C)[idx] = f2bf(v * bf2f(static_cast<const bf16*>(p.U)[idx]));
    else static_cast<float*>(p.C)[idx] = v * static_cast<const float*>(p.U)[idx];
  } else {  // ACCUMULATE
    float* c = static_cast<float*>(p.C) + idx;
    if constexpr (ATOMIC) unsafeAtomicAdd(c, v);
    else *c += v;
  }
}


typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x2 f2bf2(float a, float b) { return __builtin_convertvector((f32x2){a, b}, bf16x2); }

// Epilogue of a tile that lies wholly inside C (no bounds checks): this lane
// holds column ncol + 32 j of rows
// mrow + 32 i + 8 (q / 4) + q % 4.  Rows q and q + 1 are converted to bf16
// together (one packed conversion for two rows).
template <int EPI, bool OUT_BF16, bool ATOMIC, int TM, int TN>
__device__ __forceinline__ void epi_tile(const GemmP& p, int mrow, int ncol, const f32x16 (&acc)[TM][TN]) {
  float bj[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) bj[j] = p.bias ? p.bias[ncol + 32 * j] : 0.f;
  const int ldc = (int)p.ldc;
  const int64_t base = (int64_t)mrow * p.ldc + ncol;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int q = 0; q < 16; q += 2) {
      const int64_t r0 = base + (int64_t)((32 * i + 8 * (q >> 2) + (q & 3)) * ldc);
      const int64_t r1 = r0 + ldc;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t i0 = r0 + 32 * j, i1 = r1 + 32 * j;
        const float v0 = fmaf(p.alpha, acc[i][j][q], bj[j]);
        const float v1 = fmaf(p.alpha, acc[i][j][q + 1], bj[j]);
        if constexpr (EPI == GPT2_EPI_STORE) {
          if constexpr (OUT_BF16) {
            const bf16x2 o = f2bf2(v0, v1);
            static_cast<bf16*>(p.C)[i0] = o[0];
            static_cast<bf16*>(p.C)[i1] = o[1];
          } else {
            static_cast<float*>(p.C)[i0] = v0;
            static_cast<float*>(p.C)[i1] = v1;
          }
        } else if constexpr (EPI == GPT2_EPI_GELU) {
          if constexpr (OUT_BF16) {
            const bf16x2 u = f2bf2(v0, v1);
            const float u0 = bf2f(u[0]), u1 = bf2f(u[1]);
            const bf16x2 g = f2bf2(gelu_tanh(u0), gelu_tanh(u1));
            static_cast<bf16*>(p.C)[i0] = u[0];
            static_cast<bf16*>(p.C)[i1] = u[1];
            static_cast<bf16*>(p.C2)[i0] = g[0];
            static_cast<bf16*>(p.C2)[i1] = g[1];
          } else {
            static_cast<float*>(p.C)[i0] = v0;
            static_cast<float*>(p.C)[i1] = v1;
            static_cast<float*>(p.C2)[i0] = gelu_tanh(v0);
            static_cast<float*>(p.C2)[i1] = gelu_tanh(v1);
          }
        } else if constexpr (EPI == GPT2_EPI_GELU_GRAD) {
          float g0, g1, d0, d1;
          if constexpr (OUT_BF16) {
            const bf16x2 u = f2bf2(v0, v1);
            gelu_tanh_and_grad(bf2f(u[0]), g0, d0);
            gelu_tanh_and_grad(bf2f(u[1]), g1, d1);
            const bf16x2 g = f2bf2(g0, g1), d = f2bf2(d0, d1);
            static_cast<bf16*>(p.C)[i0] = g[0];
            static_cast<bf16*>(p.C)[i1] = g[1];
            static_cast<bf16*>(p.C2)[i0] = d[0];
            static_cast<bf16*>(p.C2)[i1] = d[1];
          } else {
            gelu_tanh_and_grad(v0, g0, d0);
            gelu_tanh_and_grad(v1, g1, d1);
            static_cast<float*>(p.C)[i0] = g0;
            static_cast<float*>(p.C)[i1] = g1;
            static_cast<float*>(p.C2)[i0] = d0;
            static_cast<float*>(p.C2)[i1] = d1;
          }
        } else if constexpr (EPI == GPT2_EPI_MUL) {
          if constexpr (OUT_BF16) {
            const bf16* U = static_cast<const bf16*>(p.U);
            const bf16x2 o = f2bf2(v0 * bf2f(U[i0]), v1 * bf2f(U[i1]));
            static_cast<bf16*>(p.C)[i0] = o[0];
            static_cast<bf16*>(p.C)[i1] = o[1];
          } else {
            static_cast<float*>(p.C)[i0] = v0 * static_cast<const float*>(p.U)[i0];
            static_cast<float*>(p.C)[i1] = v1 * static_cast<const float*>(p.U)[i1];
          }
        } else if constexpr (EPI == GPT2_EPI_RESIDUAL) {
          static_cast<float*>(p.C)[i0] = p.R[i0] + v0;
          static_cast<float*>(p.C)[i1] = p.R[i1] + v1;
        } else if constexpr (EPI == GPT2_EPI_DGELU) {
          if constexpr (OUT_BF16) {
            const float u0 = bf2f(static_cast<const bf16*>(p.U)[i0]);
            const float u1 = bf2f(static_cast<const bf16*>(p.U)[i1]);
            const bf16x2 o = f2bf2(v0 * gelu_tanh_grad(u0), v1 * gelu_tanh_grad(u1));
            static_cast<bf16*>(p.C)[i0] = o[0];
            static_cast<bf16*>(p.C)[i1] = o[1];
          } else {
            static_cast<float*>(p.C)[i0] = v0 * gelu_tanh_grad(static_cast<const float*>(p.U)[i0]);
            static_cast<float*>(p.C)[i1] = v1 * gelu_tanh_grad(static_cast<const float*>(p.U)[i1]);
          }
        } else {  // ACCUMULATE
          float* c = static_cast<float*>(p.C);
          if constexpr (ATOMIC) {
            unsafeAtomicAdd(c + i0, v0);
            unsafeAtomicAdd(c + i1, v1);
          } else {
            c[i0] += v0;
            c[i1] += v1;
          }
        }
      }
    }
}

// Unswapped layout, interior tile, epilogues that read an operand of C's
// shape (RESIDUAL: R float32; MUL, DGELU: U in the output dtype).  A lane
// holds column ncol + 32 j of rows mrow + 32 i + 8 (r / 4) + r % 4, so the 32
// lanes of a row read and write 128 (float32) or 64 (bf16) contiguous bytes.
// The operands of row group i + 1 are loaded before row group i is stored:
// the compiler must assume that C may alias them, so a load issued after a
// store would wait out the full memory latency.
template <int EPI, bool OUT_BF16, int TM, int TN>
__device__ __forceinline__ void epi_tile_gathered(const GemmP& p, int mrow, int ncol, const f32x16 (&acc)[TM][TN]) {
  static_assert(EPI == GPT2_EPI_RESIDUAL || EPI == GPT2_EPI_MUL || EPI == GPT2_EPI_DGELU, "operand epilogues");
  using Op = std::conditional_t<EPI == GPT2_EPI_RESIDUAL || !OUT_BF16, float, bf16>;
  const Op* src = EPI == GPT2_EPI_RESIDUAL ? reinterpret_cast<const Op*>(p.R) : static_cast<const Op*>(p.U);
  float bj[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) bj[j] = p.bias ? p.bias[ncol + 32 * j] : 0.f;
  const int64_t ldc = p.ldc;
  const int64_t base = (int64_t)mrow * ldc + ncol;
  auto idx = [&](int i, int j, int r) { return base + (int64_t)(32 * i + 8 * (r >> 2) + (r & 3)) * ldc + 32 * j; };
  Op op[2][TN][16];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) op[0][j][r] = src[idx(0, j, r)];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if (i + 1 < TM) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) op[(i + 1) & 1][j][r] = src[idx(i + 1, j, r)];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float v0 = fmaf(p.alpha, acc[i][j][r], bj[j]), v1 = fmaf(p.alpha, acc[i][j][r + 1], bj[j]);
        const float u0 = to_f(op[i & 1][j][r]), u1 = to_f(op[i & 1][j][r + 1]);
        const int64_t i0 = idx(i, j, r), i1 = idx(i, j, r + 1);
        if constexpr (EPI == GPT2_EPI_RESIDUAL) {
          static_cast<float*>(p.C)[i0] = u0 + v0;
          static_cast<float*>(p.C)[i1] = u1 + v1;
        } else {
          const float o0 = EPI == GPT2_EPI_MUL ? v0 * u0 : v0 * gelu_tanh_grad(u0);
          const float o1 = EPI == GPT2_EPI_MUL ? v1 * u1 : v1 * gelu_tanh_grad(u1);
          if constexpr (OUT_BF16) {
            const bf16x2 o = f2bf2(o0, o1);
            static_cast<bf16*>(p.C)[i0] = o[0];
            static_cast<bf16*>(p.C)[i1] = o[1];
          } else {
            static_cast<float*>(p.C)[i0] = o0;
            static_cast<float*>(p.C)[i1] = o1;
          }
        }
      }
  }
}

// Stores 4 consecutive outputs C[idx .. idx+3] whose values v already carry
// alpha and the bias (idx % 4 == 0); the epilogues of the swapped layout
// (bf16 output for dGELU and the product).
template <int EPI>
__device__ __forceinline__ void epi_put4(const GemmP& p, int64_t idx, const float* v) {
  static_assert(EPI == GPT2_EPI_RESIDUAL || EPI == GPT2_EPI_DGELU || EPI == GPT2_EPI_MUL,
                "swapped layout: residual, dGELU or product");
  if constexpr (EPI == GPT2_EPI_MUL) {
    const bf16x4 u = *reinterpret_cast<const bf16x4*>(static_cast<const bf16*>(p.U) + idx);
    const bf16x2 o0 = f2bf2(v[0] * bf2f(u[0]), v[1] * bf2f(u[1]));
    const bf16x2 o1 = f2bf2(v[2] * bf2f(u[2]), v[3] * bf2f(u[3]));
    *reinterpret_cast<bf16x4*>(static_cast<bf16*>(p.C) + idx) = bf16x4{o0[0], o0[1], o1[0], o1[1]};
  } else if constexpr (EPI == GPT2_EPI_RESIDUAL) {
    const float4 r = *reinterpret_cast<const float4*>(p.R + idx);
    *reinterpret_cast<float4*>(static_cast<float*>(p.C) + idx) =
        make_float4(r.x + v[0], r.y + v[1], r.z + v[2], r.w + v[3]);
  } else {
    const bf16x4 u = *reinterpret_cast<const bf16x4*>(static_cast<const bf16*>(p.U) + idx);
    const bf16x2 o0 = f2bf2(v[0] * gelu_tanh_grad(bf2f(u[0])), v[1] * gelu_tanh_grad(bf2f(u[1])));
    const bf16x2 o1 = f2bf2(v[2] * gelu_tanh_grad(bf2f(u[2])), v[3] * gelu_tanh_grad(bf2f(u[3])));
    *reinterpret_cast<bf16x4*>(static_cast<bf16*>(p.C) + idx) = bf16x4{o0[0], o0[1], o1[0], o1[1]};
  }
}

// Swapped layout (the MFMA takes B's fragment first): this lane holds row
// mrow + 32 i, columns ncol + 32 j + 8 q .. +3 (ncol includes 4 * (lane / 32)),
// so the epilogue reads and writes 16-byte vectors.  With CHECK, rows at or
// past M and columns at or past N are skipped (a group of 4 that straddles N
// is stored element by element).
//
// Interior tiles gather a row group's operands (bias, and R or U) into
// registers before the first store: the compiler must assume that C may
// alias them, so loads interleaved with stores would each wait out the full
// memory latency in turn.  Every lane reads only the elements it writes, so
// R == C (in place) stays correct.
template <int EPI, int TN>
__device__ __forceinline__ void epi_row_gathered(const GemmP& p, int64_t rb, int ncol, int i,
                                                 const f32x16 (&acc)[TN]) {
  using Op = std::conditional_t<EPI == GPT2_EPI_RESIDUAL, float4, bf16x4>;
  Op op[TN][4];
  float4 bias[TN][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int co = 32 * j + 8 * q;
      bias[j][q] = p.bias ? *reinterpret_cast<const float4*>(p.bias + ncol + co) : make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (EPI == GPT2_EPI_RESIDUAL) op[j][q] = *reinterpret_cast<const float4*>(p.R + rb + co);
      else op[j][q] = *reinterpret_cast<const bf16x4*>(static_cast<const bf16*>(p.U) + rb + co);
    }
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int co = 32 * j + 8 * q;
      const float4 b = bias[j][q];
      const float v0 = fmaf(p.alpha, acc[j][4 * q + 0], b.x), v1 = fmaf(p.alpha, acc[j][4 * q + 1], b.y);
      const float v2 = fmaf(p.alpha, acc[j][4 * q + 2], b.z), v3 = fmaf(p.alpha, acc[j][4 * q + 3], b.w);
      if constexpr (EPI == GPT2_EPI_RESIDUAL) {
        const float4 r = op[j][q];
        *reinterpret_cast<float4*>(static_cast<float*>(p.C) + rb + co) =
            make_float4(r.x + v0, r.y + v1, r.z + v2, r.w + v3);
      } else {
        const bf16x4 u = op[j][q];
        float f0 = bf2f(u[0]), f1 = bf2f(u[1]), f2 = bf2f(u[2]), f3 = bf2f(u[3]);
        if constexpr (EPI == GPT2_EPI_DGELU) {
          f0 = gelu_tanh_grad(f0); f1 = gelu_tanh_grad(f1); f2 = gelu_tanh_grad(f2); f3 = gelu_tanh_grad(f3);
        }
        const bf16x2 o0 = f2bf2(v0 * f0, v1 * f1), o1 = f2bf2(v2 * f2, v3 * f3);
        *reinterpret_cast<bf16x4*>(static_cast<bf16*>(p.C) + rb + co) = bf16x4{o0[0], o0[1], o1[0], o1[1]};
      }
    }
}

template <int EPI, bool OUT_BF16, int TM, int TN, bool CHECK>
__device__ __forceinline__ void epi_tile_swap(const GemmP& p, int mrow, int ncol, const f32x16 (&acc)[TM][TN]) {
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = mrow + 32 * i;
    if (CHECK && m >= p.M) continue;
    const int64_t rb = (int64_t)m * p.ldc + ncol;
    if constexpr (!CHECK) {
      epi_row_gathered<EPI, TN>(p, rb, ncol, i, acc[i]);
      continue;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int co = 32 * j + 8 * q;
        if (CHECK && ncol + co >= p.N) continue;
        if (CHECK && ncol + co + 4 > p.N) {
          for (int e = 0; ncol + co + e < p.N; ++e) epi_store<EPI, OUT_BF16, false>(p, m, ncol + co + e, acc[i][j][4 * q + e]);
          continue;
        }
        float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
        if (p.bias) b = *reinterpret_cast<const float4*>(p.bias + ncol + co);
        const float v[4] = {fmaf(p.alpha, acc[i][j][4 * q + 0], b.x), fmaf(p.alpha, acc[i][j][4 * q + 1], b.y),
                            fmaf(p.alpha, acc[i][j][4 * q + 2], b.z), fmaf(p.alpha, acc[i][j][4 * q + 3], b.w)};
        epi_put4<EPI>(p, rb + co, v);
      }
  }
}

// MUL epilogue of an interior tile, swapped layout.  The factors of row
// group 0 arrive in registers from the first K step (upre); the loop then
// loads row group i + 1's factors before storing row group i, so one row
// group of loads is always in flight behind the stores.
template <int TM, int TN, int TMP>
__device__ __forceinline__ void epi_tile_mul_pre(const GemmP& p, int mrow, int ncol, const f32x16 (&acc)[TM][TN],
                                                 const bf16x4 (&upre)[TMP][TN][4]) {
  static_assert(TMP == 1, "row group 0 prefetched");
  float4 bias[TN][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      bias[j][q] = p.bias ? *reinterpret_cast<const float4*>(p.bias + ncol + 32 * j + 8 * q)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
  bf16x4 cur[TN][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) cur[j][q] = upre[0][j][q];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t rb = (int64_t)(mrow + 32 * i) * p.ldc + ncol;
    bf16x4 nxt[TN][4];
    if (i + 1 < TM) {
      const bf16* un = static_cast<const bf16*>(p.U) + rb + 32 * p.ldc;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) nxt[j][q] = *reinterpret_cast<const bf16x4*>(un + 32 * j + 8 * q);
    }
    bf16* crow = static_cast<bf16*>(p.C) + rb;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int co = 32 * j + 8 * q;
        const float4 b = bias[j][q];
        const bf16x4 u = cur[j][q];
        const f32x16& a = acc[i][j];
        const bf16x2 o0 = f2bf2(fmaf(p.alpha, a[4 * q], b.x) * bf2f(u[0]), fmaf(p.alpha, a[4 * q + 1], b.y) * bf2f(u[1]));
        const bf16x2 o1 =
            f2bf2(fmaf(p.alpha, a[4 * q + 2], b.z) * bf2f(u[2]), fmaf(p.alpha, a[4 * q + 3], b.w) * bf2f(u[3]));
        *reinterpret_cast<bf16x4*>(crow + co) = bf16x4{o0[0], o0[1], o1[0], o1[1]};
      }
    if (i + 1 < TM) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) cur[j][q] = nxt[j][q];
    }
  }
}

// ------------------------------------------------ rotary and SwiGLU epilogues
//
// Swapped layout with 64 columns per wave (TN == 2): in accumulator j = 0 a
// lane holds columns g + 8q + 4 lg + e of the wave's 64-column group g, in
// j = 1 the columns 32 further on, so the two elements that a rotation or
// the SwiGLU gate combine sit in the same lane and register.

// sigmoid(x) = 1 / (1 + 2^(-x log2 e))
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

// ROPE: rotary embedding of q and k ("Reproduce GPT-2 124M", x cos +
// rotate_half(x) sin, dimension i of a 64-wide head paired with i + 32) on
// the bf16 output of the qkv product.  Column groups g < rope_cols are
// rotated with the angle table of position m % rope_period; the others
// (v) are stored as they are.
// SWIGLU: the product's columns are the interleaved rows of [W_gate; W_up]
// (group g holds gate rows g/2 .. g/2+31 in j = 0 and the matching up rows
// in j = 1): act = silu(gate) up goes to C at column g/2 + d, the bf16 gate
// and up to C2 at columns g/2 + d and F + g/2 + d (F = N / 2).
template <int EPI, int TM, bool CHECK>
__device__ __forceinline__ void epi_tile_pair(const GemmP& p, int mrow, int gcol, int lg, const f32x16 (&acc)[TM][2]) {
  if (CHECK && gcol >= p.N) return;  // N % 64 == 0: a group is wholly in or out
  const bool rot = EPI == GPT2_EPI_ROPE && gcol < p.rope_cols;
  const int F = p.N >> 1;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = mrow + 32 * i;
    if (CHECK && m >= p.M) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 8 * q + 4 * lg;
      float v0[4], v1[4];
      float4 b0 = make_float4(0.f, 0.f, 0.f, 0.f), b1 = b0;
      if (EPI == GPT2_EPI_ROPE && p.bias) {
        b0 = *reinterpret_cast<const float4*>(p.bias + gcol + d);
        b1 = *reinterpret_cast<const float4*>(p.bias + gcol + 32 + d);
      }
      const float bb0[4] = {b0.x, b0.y, b0.z, b0.w}, bb1[4] = {b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v0[e] = fmaf(p.alpha, acc[i][0][4 * q + e], bb0[e]);
        v1[e] = fmaf(p.alpha, acc[i][1][4 * q + e], bb1[e]);
      }
      if constexpr (EPI == GPT2_EPI_ROPE) {
        bf16* crow = static_cast<bf16*>(p.C) + (int64_t)m * p.ldc + gcol;
        float o0[4], o1[4];
        if (rot) {
          const float2* tab = p.rope + (int64_t)(m % p.rope_period) * 32 + d;
          const float4 cs01 = *reinterpret_cast<const float4*>(tab);
          const float4 cs23 = *reinterpret_cast<const float4*>(tab + 2);
          const float cc[4] = {cs01.x, cs01.z, cs23.x, cs23.z}, sn[4] = {cs01.y, cs01.w, cs23.y, cs23.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o0[e] = v0[e] * cc[e] - v1[e] * sn[e];
            o1[e] = v1[e] * cc[e] + v0[e] * sn[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o0[e] = v0[e];
            o1[e] = v1[e];
          }
        }
        const bf16x2 a01 = f2bf2(o0[0], o0[1]), a23 = f2bf2(o0[2], o0[3]);
        const bf16x2 c01 = f2bf2(o1[0], o1[1]), c23 = f2bf2(o1[2], o1[3]);
        *reinterpret_cast<bf16x4*>(crow + d) = bf16x4{a01[0], a01[1], a23[0], a23[1]};
        *reinterpret_cast<bf16x4*>(crow + 32 + d) = bf16x4{c01[0], c01[1], c23[0], c23[1]};
      } else {  // SWIGLU
        const int f = (gcol >> 1) + d;
        const bf16x2 g01 = f2bf2(v0[0], v0[1]), g23 = f2bf2(v0[2], v0[3]);
        const bf16x2 u01 = f2bf2(v1[0], v1[1]), u23 = f2bf2(v1[2], v1[3]);
        const bf16x4 g = bf16x4{g01[0], g01[1], g23[0], g23[1]}, u = bf16x4{u01[0], u01[1], u23[0], u23[1]};
        float a[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gf = bf2f(g[e]);
          a[e] = gf * sigmoid_fast(gf) * bf2f(u[e]);
        }
        const bf16x2 a01 = f2bf2(a[0], a[1]), a23 = f2bf2(a[2], a[3]);
        *reinterpret_cast<bf16x4*>(static_cast<bf16*>(p.C) + (int64_t)m * p.ldc + f) =
            bf16x4{a01[0], a01[1], a23[0], a23[1]};
        bf16* c2 = static_cast<bf16*>(p.C2) + (int64_t)m * p.ld2 + f;
        *reinterpret_cast<bf16x4*>(c2) = g;
        *reinterpret_cast<bf16x4*>(c2 + F) = u;
      }
    }
  }
}

// ROPE and SWIGLU in the unswapped layout (64 columns per wave): this lane
// holds columns gcol + d (j = 0) and gcol + 32 + d (j = 1), d = lane % 32, of
// rows mrow + 32 i + 8 (r / 4) + r % 4, so the pair a rotation or the gate
// combines is again in one lane, and the 32 lanes of a row write 64-byte runs.
template <int EPI, int TM, bool CHECK>
__device__ __forceinline__ void epi_tile_pair_rows(const GemmP& p, int mrow, int gcol, int d,
                                                   const f32x16 (&acc)[TM][2]) {
  if (CHECK && gcol >= p.N) return;  // N % 64 == 0: a group is wholly in or out
  const bool rot = EPI == GPT2_EPI_ROPE && gcol < p.rope_cols;
  const int F = p.N >> 1;
  float b0 = 0.f, b1 = 0.f;
  if (EPI == GPT2_EPI_ROPE && p.bias) {
    b0 = p.bias[gcol + d];
    b1 = p.bias[gcol + 32 + d];
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const int m[2] = {mrow + 32 * i + 8 * (r >> 2) + (r & 3), mrow + 32 * i + 8 * (r >> 2) + (r & 3) + 1};
      float o0[2], o1[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float v0 = fmaf(p.alpha, acc[i][0][r + t], b0), v1 = fmaf(p.alpha, acc[i][1][r + t], b1);
        if constexpr (EPI == GPT2_EPI_ROPE) {
          if (rot) {
            const float2 cs = p.rope[(int64_t)(m[t] % p.rope_period) * 32 + d];
            o0[t] = v0 * cs.x - v1 * cs.y;
            o1[t] = v1 * cs.x + v0 * cs.y;
          } else {
            o0[t] = v0;
            o1[t] = v1;
          }
        } else {
          o0[t] = v0;  // gate
          o1[t] = v1;  // up
        }
      }
      const bf16x2 a = f2bf2(o0[0], o0[1]), c = f2bf2(o1[0], o1[1]);
      if constexpr (EPI == GPT2_EPI_ROPE) {
        bf16* C = static_cast<bf16*>(p.C);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if (CHECK && m[t] >= p.M) continue;
          C[(int64_t)m[t] * p.ldc + gcol + d] = a[t];
          C[(int64_t)m[t] * p.ldc + gcol + 32 + d] = c[t];
        }
      } else {
        const int f = (gcol >> 1) + d;
        float act[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float gf = bf2f(a[t]);
          act[t] = gf * sigmoid_fast(gf) * bf2f(c[t]);
        }
        const bf16x2 ab = f2bf2(act[0], act[1]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if (CHECK && m[t] >= p.M) continue;
          static_cast<bf16*>(p.C)[(int64_t)m[t] * p.ldc + f] = ab[t];
          bf16* c2 = static_cast<bf16*>(p.C2) + (int64_t)m[t] * p.ld2 + f;
          c2[0] = a[t];
          c2[F] = c[t];
        }
      }
    }
}

// SWIGLU_BWD: the product is d(act) [M, F] (F = N); with gate g = U[m][f]
// and up u = U[m][F + f] (row pitch ld2), C[m][f] = d(act) u silu'(g) and
// C[m][F + f] = d(act) silu(g), silu'(g) = s (1 + g (1 - s)), s = sigmoid(g).
// Swapped layout, any tile width; N % 4 == 0.
template <int TN>
__device__ __forceinline__ void swiglu_bwd_store(const GemmP& p, bf16* crow, int ncol, int F, const bf16x4 (&g)[TN][4],
                                                 const bf16x4 (&u)[TN][4], const f32x16 (&acc)[TN], bool check) {
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int f = ncol + 32 * j + 8 * q;
      if (check && f >= p.N) continue;
      float dg[4], du[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = p.alpha * acc[j][4 * q + e];
        const float gf = bf2f(g[j][q][e]), sg = sigmoid_fast(gf);
        du[e] = v * gf * sg;
        dg[e] = v * bf2f(u[j][q][e]) * sg * fmaf(gf, 1.f - sg, 1.f);
      }
      const bf16x2 g01 = f2bf2(dg[0], dg[1]), g23 = f2bf2(dg[2], dg[3]);
      const bf16x2 u01 = f2bf2(du[0], du[1]), u23 = f2bf2(du[2], du[3]);
      *reinterpret_cast<bf16x4*>(crow + f) = bf16x4{g01[0], g01[1], g23[0], g23[1]};
      *reinterpret_cast<bf16x4*>(crow + F + f) = bf16x4{u01[0], u01[1], u23[0], u23[1]};
    }
}

template <int TN>
__device__ __forceinline__ void swiglu_bwd_load(const GemmP& p, const bf16* urow, int ncol, int F, bf16x4 (&g)[TN][4],
                                                bf16x4 (&u)[TN][4], bool check) {
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int f = ncol + 32 * j + 8 * q;
      if (check && f >= p.N) continue;
      g[j][q] = *reinterpret_cast<const bf16x4*>(urow + f);
      u[j][q] = *reinterpret_cast<const bf16x4*>(urow + F + f);
    }
}

// Rows are visited in order; the gate and up values of row group i + 1 are
// loaded before row group i is stored (interior tiles), or just before it
// (edge tiles, whose row groups may be absent).
template <int TM, int TN, bool CHECK>
__device__ __forceinline__ void epi_tile_swiglu_bwd(const GemmP& p, int mrow, int ncol, const f32x16 (&acc)[TM][TN]) {
  const int F = p.N;
  const bf16* U = static_cast<const bf16*>(p.U);
  bf16* C = static_cast<bf16*>(p.C);
  if constexpr (CHECK) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = mrow + 32 * i;
      if (m >= p.M) continue;
      bf16x4 g[TN][4], u[TN][4];
      swiglu_bwd_load<TN>(p, U + (int64_t)m * p.ld2, ncol, F, g, u, true);
      swiglu_bwd_store<TN>(p, C + (int64_t)m * p.ldc, ncol, F, g, u, acc[i], true);
    }
  } else {
    bf16x4 g[2][TN][4], u[2][TN][4];
    swiglu_bwd_load<TN>(p, U + (int64_t)mrow * p.ld2, ncol, F, g[0], u[0], false);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = mrow + 32 * i;
      if (i + 1 < TM)
        swiglu_bwd_load<TN>(p, U + (int64_t)(m + 32) * p.ld2, ncol, F, g[(i + 1) & 1], u[(i + 1) & 1], false);
      swiglu_bwd_store<TN>(p, C + (int64_t)m * p.ldc, ncol, F, g[i & 1], u[i & 1], acc[i], false);
    }
  }
}

// SWIGLU_BWD in the unswapped layout: this lane holds column f = ncol + 32 j
// of rows mrow + 32 i + 8 (r / 4) + r % 4, so the 32 lanes of a row read gate
// and up and write dgate and dup in 64-byte runs.  The row group is taken in
// halves of 8 registers; gate and up of the next half are loaded before the
// current half is stored (loads after a store would each wait out the full
// latency: the compiler must assume C may alias U).
template <int TM, int TN, bool CHECK>
__device__ __forceinline__ void epi_tile_swiglu_bwd_rows(const GemmP& p, int mrow, int ncol,
                                                         const f32x16 (&acc)[TM][TN]) {
  const int F = p.N;
  const bf16* U = static_cast<const bf16*>(p.U);
  bf16* Cp = static_cast<bf16*>(p.C);
  constexpr int NCH = 2 * TM;  // halves of row groups
  auto row_of = [&](int ch, int e) { return mrow + 32 * (ch >> 1) + 8 * ((8 * (ch & 1) + e) >> 2) + (e & 3); };
  bf16 g[2][TN][8], u[2][TN][8];
  auto load = [&](int ch, int b) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int m = row_of(ch, e), f = ncol + 32 * j;
        if (CHECK && (m >= p.M || f >= F)) continue;
        const bf16* ur = U + (int64_t)m * p.ld2 + f;
        g[b][j][e] = ur[0];
        u[b][j][e] = ur[F];
      }
  };
  load(0, 0);
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    if (ch + 1 < NCH) load(ch + 1, (ch + 1) & 1);
    const int b = ch & 1;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int m0 = row_of(ch, e), m1 = row_of(ch, e + 1), f = ncol + 32 * j;
        float dg[2], du[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float v = p.alpha * acc[ch >> 1][j][8 * (ch & 1) + e + t];
          const float gf = bf2f(g[b][j][e + t]), sg = sigmoid_fast(gf);
          du[t] = v * gf * sg;
          dg[t] = v * bf2f(u[b][j][e + t]) * sg * fmaf(gf, 1.f - sg, 1.f);
        }
        const bf16x2 dgb = f2bf2(dg[0], dg[1]), dub = f2bf2(du[0], du[1]);
        if (!CHECK || (m0 < p.M && f < F)) {
          Cp[(int64_t)m0 * p.ldc + f] = dgb[0];
          Cp[(int64_t)m0 * p.ldc + F + f] = dub[0];
        }
        if (!CHECK || (m1 < p.M && f < F)) {
          Cp[(int64_t)m1 * p.ldc + f] = dgb[1];
          Cp[(int64_t)m1 * p.ldc + F + f] = dub[1];
        }
      }
  }
}

// Internal epilogue of the lm_head product (logits = hidden wte^T), swapped
// layout only.  For every row m and column tile tn it stores the tile's
// softmax statistics stats[m][tn] = (mx, sum over the tile's columns n < N of
// exp(z[m][n] - mx)) with mx the tile's largest logit, all from the float32
// accumulators, and writes C[m][n] = bf16(z[m][n] - mx) (staged through LDS
// so each row goes out in 512-byte pieces).  Entries near the row's
// maximum, the ones that carry the softmax, keep nearly full precision.
constexpr int EPI_CE_STATS = 16;

template <int BM, int BN, int WGN, int TM, int TN, bool EDGE>
__device__ __forceinline__ void epi_ce_stats(const GemmP& p, int m0, int n0, int tn, int wm0, int wn0, int wave,
                                             int lr, int lg, const f32x16 (&acc)[TM][TN], float* red, char* st0,
                                             char* st1) {
  // the output tile is staged in the two operand stages: rows below BM / 2
  // in the first, the others in the second
  auto srow = [&](int row) { return row < BM / 2 ? st0 + row * (BN * 2) : st1 + (row - BM / 2) * (BN * 2); };
  constexpr float L2E = 1.4426950408889634f;
  constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
  const int wn = wave % WGN;
  // per row: this wave's 64 columns (32 in each lane half) -> (max, sum of exp)
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int col = n0 + wn0 + 32 * j + 8 * (e >> 2) + 4 * lg + (e & 3);
        if (!EDGE || col < p.N) mx = fmaxf(mx, acc[i][j][e]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float sm = 0.f;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int col = n0 + wn0 + 32 * j + 8 * (e >> 2) + 4 * lg + (e & 3);
        if (!EDGE || col < p.N) sm += __builtin_amdgcn_exp2f((acc[i][j][e] - mx) * L2E);
      }
    sm += __shfl_xor(sm, 32);
    const int row = wm0 + 32 * i + lr;
    if (lg == 0) {
      red[2 * (wn * BM + row)] = mx;
      red[2 * (wn * BM + row) + 1] = sm;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // the tile's row maxima and sums; the offsets z - max go to LDS as bf16,
  // row-major with 16-byte chunk c of row r at c ^ (r % 32)
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = wm0 + 32 * i + lr;
    const int m = m0 + row;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < WGN; ++w) mx = fmaxf(mx, red[2 * (w * BM + row)]);
    float sm = 0.f;
#pragma unroll
    for (int w = 0; w < WGN; ++w) {
      const float mw = red[2 * (w * BM + row)];
      if (mw != -INFINITY) sm += red[2 * (w * BM + row) + 1] * __builtin_amdgcn_exp2f((mw - mx) * L2E);
    }
    if (wn == 0 && lg == 0 && m < p.M) p.stats[(int64_t)m * p.tiles_n + tn] = make_float2(mx, sm);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = wn0 + 32 * j + 8 * q + 4 * lg;  // within the tile
        const bf16x2 lo = f2bf2(acc[i][j][4 * q] - mx, acc[i][j][4 * q + 1] - mx);
        const bf16x2 hi = f2bf2(acc[i][j][4 * q + 2] - mx, acc[i][j][4 * q + 3] - mx);
        const int addr = (((col >> 3) ^ (row & (CPR - 1))) << 4) + ((col >> 2) & 1) * 8;
        *reinterpret_cast<bf16x4*>(srow(row) + addr) = bf16x4{lo[0], lo[1], hi[0], hi[1]};
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // copy out: each lane 16 bytes, 32 lanes a 512-byte row
  bf16* C = static_cast<bf16*>(p.C);
  constexpr int NT = 64 * (BM / (TM * 32)) * WGN;
#pragma unroll 4
  for (int idx = threadIdx.x; idx < BM * CPR; idx += NT) {
    const int row = idx / CPR, c = idx % CPR;
    const int m = m0 + row, n = n0 + 8 * c;
    if (m >= p.M || (EDGE && n >= p.N)) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(srow(row) + ((c ^ (row & (CPR - 1))) << 4));
    bf16* d = C + (int64_t)m * p.ldc + n;
    if (!EDGE || n + 8 <= p.N) {
      *reinterpret_cast<uint4*>(d) = v;
    } else {
      const bf16* vv = reinterpret_cast<const bf16*>(&v);
      for (int e = 0; n + e < p.N; ++e) d[e] = vv[e];
    }
  }
}

// Tile -> block mapping.  Blocks are handed to the 8 XCDs round-robin; the
// remap makes consecutive logical units (tiles, or tiles of a group) run on
// one XCD (sharing its L2).
__host__ __device__ __forceinline__ int xcd_remap(int bid, int nb) {
  return (nb & 7) == 0 ? (bid & 7) * (nb >> 3) + (bid >> 3) : bid;
}
inline int xcd_remap_host(int bid, int nb) { return xcd_remap(bid, nb); }

// Unit -> (row tile, column tile, K split) of one product: the grouped order
// walks GROUP_M row tiles per column panel.
__device__ __forceinline__ void tile_of_unit(const GemmP& p, int bid, int& tm, int& tn, int& split) {
  const int per_split = p.tiles_m * p.tiles_n;
  split = bid / per_split;
  int t = bid - split * per_split;
  const int GROUP_M = p.group_m > 0 ? p.group_m : 8;
  const int in_group = GROUP_M * p.tiles_n;
  const int group = t / in_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(p.tiles_m - first_m, GROUP_M);
  const int r = t - group * in_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

union GV8 {
  uint4 u;
  bf16x8 v;
  uint32_t w[4];
};

// Instruction order of one K step (sched_group_barrier masks: 0x008 MFMA,
// 0x100 LDS read): NR reads of the first slice, then for every slice but the
// last its NM MFMAs with the NR reads of the next slice spread among them,
// then the last slice's MFMAs.
template <int NR, int NM, int M>
__device__ __forceinline__ void sched_pair() {
  if constexpr (M < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int per = (NR + NM - 1) / NM;
    constexpr int left = NR - M * per;
    if constexpr (left > 0) __builtin_amdgcn_sched_group_barrier(0x100, left < per ? left : per, 0);
    sched_pair<NR, NM, M + 1>();
  }
}
template <int NR, int NM, int S>
__device__ __forceinline__ void sched_slices() {
  if constexpr (S > 0) {
    sched_pair<NR, NM, 0>();
    sched_slices<NR, NM, S - 1>();
  }
}
template <int NR, int NM, int SLICES>
__device__ __forceinline__ void sched_kstep() {
  __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
  sched_slices<NR, NM, SLICES - 1>();
  __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
}

// One block's unit of a product: its output tile (and K split), main loop
// and epilogue.
// The two LDS stages of a block: (BM + BN) * BK bf16 elements each.  They are
// two distinct LDS objects, declared by the kernel and passed down (a kernel
// that runs units of several operand layouts shares them among those), and
// the K loop is unrolled by two, so every copy and every read names its stage
// statically.  The compiler then sees that a copy into one stage cannot
// alias reads of the other and adds no wait for it; with one object (or a
// stage picked at run time) it must assume the transposing reads alias every
// copy in flight and drains the next step's copy (s_waitcnt vmcnt(0)) before
// computing the current step.
#define G2_STAGES(BM, BN, BK)                                      \
  __shared__ __attribute__((aligned(16))) bf16 lds0[((BM) + (BN)) * (BK)]; \
  __shared__ __attribute__((aligned(16))) bf16 lds1[((BM) + (BN)) * (BK)]

template <int BM, int BN, int BK, int WGM, int WGN, int STAGES, bool A_K, bool B_K, int EPI, bool OUT_BF16,
          bool ATOMIC, bool SWAP>
__device__ __forceinline__ void gemm2_unit(const GemmP& p, int unit, bf16* lds0, bf16* lds1) {
  constexpr int NW = WGM * WGN;
  constexpr int NT = 64 * NW;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int STAGE = (BM + BN) * BK;  // elements per stage
  static_assert(TM >= 1 && TN >= 1, "wave tile must hold at least one 32x32 MFMA tile");
  static_assert(STAGES == 2, "two LDS stages");

  int tm, tn, split;
  tile_of_unit(p, unit, tm, tn, split);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = split * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int nk = (kend - kbeg + BK - 1) / BK;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm0 = (wave / WGN) * WM, wn0 = (wave % WGN) * WN;
  const int lr = lane & 31, lg = lane >> 5;
  const bool do_rowsum = p.row_sum != nullptr && tn == 0;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  float rsum = 0.f;

  const bf16* Ag = static_cast<const bf16*>(p.A);
  const bf16* Bg = static_cast<const bf16*>(p.B);

  // Every operand tile is copied into LDS by DMA: K-major ones as [rows][BK]
  // (row-swizzled), K-slow ones in their memory layout as [BK][rows].
  // full K steps: per-lane offsets fixed for the tile (tile_io.h); a ragged
  // last step: the bounds-checked, zero-filling copy
  std::conditional_t<A_K, RowsDma<BM, BK, NW>, KrDma<BM, BK, NW>> dma_a;
  std::conditional_t<B_K, RowsDma<BN, BK, NW>, KrDma<BN, BK, NW>> dma_b;
  // SWIGLU reads B's rows interleaved (64-column group g: gate rows g/2 ..
  // g/2+31, then the up rows F + g/2 ..), from absolute row offsets
  constexpr bool MAP_B = EPI == GPT2_EPI_SWIGLU;
  static_assert(!MAP_B || (B_K && WN == 64), "SwiGLU: K-major B, 64 columns per wave");
  const int b_row0 = MAP_B ? 0 : n0;
  dma_a.init(p.lda, m0, p.M);
  if constexpr (MAP_B) dma_b.init_swiglu(p.ldb, n0, p.N);
  else dma_b.init(p.ldb, n0, p.N);
  auto issue = [&](bf16* as, int kstep) {
    bf16* bs = as + BM * BK;
    const int k0 = kbeg + kstep * BK;
    // (copies through inline asm: the compiler adds no waits for them; the
    // top of each K step waits and meets the other waves)
    if (MAP_B || k0 + BK <= kend) {  // SWIGLU: K % BK == 0, checked by the host
      dma_a.issue(as, Ag, p.lda, m0, k0);
      dma_b.issue(bs, Bg, p.ldb, b_row0, k0);
    } else {
      if constexpr (A_K) dma_rows<BM, BK, NW, true>(as, Ag, p.lda, m0, p.M, k0, kend);
      else dma_kr<BM, BK, NW, true>(as, Ag, p.lda, m0, p.M, k0, kend);
      if constexpr (B_K) dma_rows<BN, BK, NW, true>(bs, Bg, p.ldb, n0, p.N, k0, kend);
      else dma_kr<BN, BK, NW, true>(bs, Bg, p.ldb, n0, p.N, k0, kend);
    }
  };
  const bool interior = m0 + BM <= p.M && n0 + BN <= p.N;
  // MUL epilogue (swapped layout) of an interior tile: the factors this lane
  // multiplies by are loaded during the first K step (64 registers), so
  // their latency hides behind the main loop
  constexpr bool PRE_U = SWAP && EPI == GPT2_EPI_MUL;
  constexpr int TMP = 1;  // accumulator rows whose factors are prefetched (register budget)
  bf16x4 upre[PRE_U ? TMP : 1][PRE_U ? TN : 1][PRE_U ? 4 : 1];

  // One K step: wait for this wave's copy of step kt, meet the other waves
  // (so every wave's copy has landed), start the copy of step kt + 1 into
  // the other stage, then multiply.  The asm is also a compiler memory
  // barrier: no LDS access moves across it.
  auto kstep = [&](const bf16* as, bf16* next, int kt) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if constexpr (PRE_U) {
      // issued before the next step's copy, so the next wait covers them
      if (kt == 0 && interior) {
        const bf16* U = static_cast<const bf16*>(p.U) + (int64_t)(m0 + wm0 + lr) * p.ldc + n0 + wn0 + 4 * lg;
#pragma unroll
        for (int i = 0; i < TMP; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              upre[i][j][q] = *reinterpret_cast<const bf16x4*>(U + (int64_t)(32 * i) * p.ldc + 32 * j + 8 * q);
      }
    }
    if (kt + 1 < nk) issue(next, kt + 1);
    const bf16* bs = as + BM * BK;
    // Fragments of the next 16-wide K slice are read from LDS while the
    // current slice's MFMAs issue.  Without SWAP a lane's accumulator holds
    // one output column of 4 consecutive rows per register group, and the 32
    // lanes of a row cover 32 consecutive columns (coalesced stores and
    // atomics); with SWAP the MFMA takes B's fragment first and a lane holds
    // 4 consecutive columns of one row (16-byte reads of the residual or the
    // GELU input).
    bf16x8 a[2][TM], b[2][TN];
    // 16-wave blocks with a K-major operand: the slice's chunk index is
    // recomputed for every read from an opaque lane value, so that the
    // compiler keeps no per-slice address registers
    constexpr bool LEAN = NW >= 16 && (A_K || B_K);
    auto frag = [&](int kk, bf16x8* fa, bf16x8* fb) {
      int lgv = lg;
      if constexpr (LEAN) asm volatile("" : "+v"(lgv));
      const int c = 2 * kk + lgv;
      const int h = (lane >> 4) & 1;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if constexpr (A_K) {
          const int row = wm0 + 32 * i + lr;
          fa[i] = *reinterpret_cast<const bf16x8*>(as + row * BK + 8 * swz_chunk<BK>(row, c));
        } else {
          const bf16x4 lo = tr_read4_kr<BM>(as, 16 * kk + 8 * lg, wm0 + 32 * i + 16 * h);
          const bf16x4 hi = tr_read4_kr<BM>(as, 16 * kk + 8 * lg + 4, wm0 + 32 * i + 16 * h);
          fa[i] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (B_K) {
          const int row = wn0 + 32 * j + lr;
          fb[j] = *reinterpret_cast<const bf16x8*>(bs + row * BK + 8 * swz_chunk<BK>(row, c));
        } else {
          const bf16x4 lo = tr_read4_kr<BN>(bs, 16 * kk + 8 * lg, wn0 + 32 * j + 16 * h);
          const bf16x4 hi = tr_read4_kr<BN>(bs, 16 * kk + 8 * lg + 4, wn0 + 32 * j + 16 * h);
          fb[j] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
    };
    if constexpr (!LEAN) {
    frag(0, a[0], b[0]);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int cb = kk & 1;
      if (kk + 1 < BK / 16) frag(kk + 1, a[cb ^ 1], b[cb ^ 1]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = SWAP ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[cb][j], a[cb][i], acc[i][j], 0, 0, 0)
                           : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cb][i], b[cb][j], acc[i][j], 0, 0, 0);
    }
    // Left to itself the compiler issues each slice's fragment reads just
    // before that slice's MFMAs and waits for them there; this order keeps
    // the next slice's reads in flight behind the current slice's MFMAs.
    sched_kstep<TM * (A_K ? 1 : 2) + TN * (B_K ? 1 : 2), TM * TN, BK / 16>();
    } else {
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      frag(kk, a[0], b[0]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = SWAP ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[0][j], a[0][i], acc[i][j], 0, 0, 0)
                           : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][i], b[0][j], acc[i][j], 0, 0, 0);
    }
    }
    if (do_rowsum && threadIdx.x < BM) {
      // row sums of this block's A tile (K values past kend read as zeros)
      const int t = threadIdx.x;
      if constexpr (A_K) {
        const bf16* row = as + t * BK;
#pragma unroll
        for (int c = 0; c < BK / 8; ++c) {
          const bf16x8 v = *reinterpret_cast<const bf16x8*>(row + 8 * c);
#pragma unroll
          for (int e = 0; e < 8; ++e) rsum += bf2f(v[e]);
        }
      } else {
#pragma unroll 8
        for (int k = 0; k < BK; ++k) rsum += bf2f(as[k * BM + 8 * kr_chunk<BM>(k, t >> 3) + (t & 7)]);
      }
    }
  };

  if (nk > 0) issue(lds0, 0);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    kstep(lds0, lds1, kt);
    kstep(lds1, lds0, kt + 1);
  }
  if (kt < nk) kstep(lds0, lds1, kt);
  if (do_rowsum && threadIdx.x < BM && m0 + (int)threadIdx.x < p.M)
    unsafeAtomicAdd(p.row_sum + m0 + threadIdx.x, p.alpha * rsum);

  if constexpr (EPI == EPI_CE_STATS) {
    static_assert(SWAP && WN == 64, "statistics epilogue: swapped layout, 64 columns per wave");
    // every wave is done with the operand stages: reuse them for the
    // cross-wave reduction
    static_assert(BM / 2 * BN * 2 <= STAGE * 2, "half the output tile fits in one operand stage");
    __shared__ float red[2 * WGN * BM];
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (n0 + BN <= p.N)
      epi_ce_stats<BM, BN, WGN, TM, TN, false>(p, m0, n0, tn, wm0, wn0, wave, lr, lg, acc, red,
                                               reinterpret_cast<char*>(lds0), reinterpret_cast<char*>(lds1));
    else
      epi_ce_stats<BM, BN, WGN, TM, TN, true>(p, m0, n0, tn, wm0, wn0, wave, lr, lg, acc, red,
                                              reinterpret_cast<char*>(lds0), reinterpret_cast<char*>(lds1));
  } else if constexpr (EPI == GPT2_EPI_ROPE || EPI == GPT2_EPI_SWIGLU) {
    static_assert(WN == 64, "paired epilogues: 64 columns per wave");
    if constexpr (SWAP) {
      if (interior) epi_tile_pair<EPI, TM, false>(p, m0 + wm0 + lr, n0 + wn0, lg, acc);
      else epi_tile_pair<EPI, TM, true>(p, m0 + wm0 + lr, n0 + wn0, lg, acc);
    } else {
      if (interior) epi_tile_pair_rows<EPI, TM, false>(p, m0 + wm0 + 4 * lg, n0 + wn0, lr, acc);
      else epi_tile_pair_rows<EPI, TM, true>(p, m0 + wm0 + 4 * lg, n0 + wn0, lr, acc);
    }
  } else if constexpr (EPI == GPT2_EPI_SWIGLU_BWD) {
    if constexpr (SWAP) {
      if (interior) epi_tile_swiglu_bwd<TM, TN, false>(p, m0 + wm0 + lr, n0 + wn0 + 4 * lg, acc);
      else epi_tile_swiglu_bwd<TM, TN, true>(p, m0 + wm0 + lr, n0 + wn0 + 4 * lg, acc);
    } else {
      if (interior) epi_tile_swiglu_bwd_rows<TM, TN, false>(p, m0 + wm0 + 4 * lg, n0 + wn0 + lr, acc);
      else epi_tile_swiglu_bwd_rows<TM, TN, true>(p, m0 + wm0 + 4 * lg, n0 + wn0 + lr, acc);
    }
  } else {
    if constexpr (PRE_U) {
      if (interior) epi_tile_mul_pre<TM, TN, TMP>(p, m0 + wm0 + lr, n0 + wn0 + 4 * lg, acc, upre);
      else epi_tile_swap<EPI, OUT_BF16, TM, TN, true>(p, m0 + wm0 + lr, n0 + wn0 + 4 * lg, acc);
    } else if constexpr (SWAP) {
      if (interior) epi_tile_swap<EPI, OUT_BF16, TM, TN, false>(p, m0 + wm0 + lr, n0 + wn0 + 4 * lg, acc);
      else epi_tile_swap<EPI, OUT_BF16, TM, TN, true>(p, m0 + wm0 + lr, n0 + wn0 + 4 * lg, acc);
    } else if (interior) {
      if constexpr (!ATOMIC && (EPI == GPT2_EPI_RESIDUAL || EPI == GPT2_EPI_MUL || EPI == GPT2_EPI_DGELU))
        epi_tile_gathered<EPI, OUT_BF16, TM, TN>(p, m0 + wm0 + 4 * lg, n0 + wn0 + lr, acc);
      else
        if (EPI == GPT2_EPI_ACCUMULATE && !ATOMIC && p.splits > 1)  // a grouped launch's split products
          epi_tile<EPI, OUT_BF16, true, TM, TN>(p, m0 + wm0 + 4 * lg, n0 + wn0 + lr, acc);
        else
          epi_tile<EPI, OUT_BF16, ATOMIC, TM, TN>(p, m0 + wm0 + 4 * lg, n0 + wn0 + lr, acc);
    } else {
      // accumulator (i, j), register r: row 8*(r/4) + 4*lg + r%4, column lr
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = n0 + wn0 + 32 * j + lr;
          if (n >= p.N) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + wm0 + 32 * i + 8 * (r >> 2) + 4 * lg + (r & 3);
            if (m >= p.M) continue;
            if (EPI == GPT2_EPI_ACCUMULATE && !ATOMIC && p.splits > 1) epi_store<EPI, OUT_BF16, true>(p, m, n, acc[i][j][r]);
            else epi_store<EPI, OUT_BF16, ATOMIC>(p, m, n, acc[i][j][r]);
          }
        }
    }
  }
}

template <int BM, int BN, int BK, int WGM, int WGN, int STAGES, bool A_K, bool B_K, int EPI, bool OUT_BF16,
          bool ATOMIC, bool SWAP>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm2_kernel(GemmP p) {
  G2_STAGES(BM, BN, BK);
  gemm2_unit<BM, BN, BK, WGM, WGN, STAGES, A_K, B_K, EPI, OUT_BF16, ATOMIC, SWAP>(p, xcd_remap(blockIdx.x, gridDim.x),
                                                                               lds0, lds1);
}

// Several independent products in one launch.  Block b runs unit
// unit_map[b] & 0xffff of product unit_map[b] >> 16 (the host orders the
// units: blocks go to the XCDs round-robin in index order).  A product with
// splits > 1 adds its partial sums atomically (ACCUMULATE).  K_all > 0
// replaces every product's K (all products of one launch reduce over the
// same tokens), so one table serves every token count: a product split S
// ways takes pieces of ceil(K_all / (64 S)) * 64.
struct GemmGroups {
  const GemmP* __restrict__ p;
  const int* __restrict__ unit_map;
};

template <int BM, int BN, int BK, int WGM, int WGN, int STAGES, bool A_K, bool B_K, int EPI, bool OUT_BF16,
          bool ATOMIC, bool SWAP>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm2_grouped_kernel(GemmGroups t, int K_all) {
  G2_STAGES(BM, BN, BK);
  const int e = t.unit_map[blockIdx.x];
  GemmP p = t.p[e >> 16];
  if (K_all > 0) {
    p.K = K_all;
    p.k_per_split = p.splits > 1 ? (K_all + p.splits * BK - 1) / (p.splits * BK) * BK : K_all;
  }
  gemm2_unit<BM, BN, BK, WGM, WGN, STAGES, A_K, B_K, EPI, OUT_BF16, ATOMIC, SWAP>(p, e & 0xffff, lds0, lds1);
}

// Two accumulating products of different operand layouts in one launch,
// their parameters passed by value: blocks [0, units0) run product 0 (layout
// A_K0, B_K0), the others product 1 (A_K1, B_K1).  Within each product the
// units are spread XCD-aware (when both unit counts are multiples of 8, each
// XCD takes a contiguous run of each product).  A product with splits > 1
// adds its partial sums atomically.
template <int BM, int BN, int BK, int WGM, int WGN, bool A_K0, bool B_K0, bool A_K1, bool B_K1>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm2_pair_kernel(GemmP p0, GemmP p1, int units0) {
  G2_STAGES(BM, BN, BK);
  const int b = blockIdx.x;
  if (b < units0) {
    gemm2_unit<BM, BN, BK, WGM, WGN, 2, A_K0, B_K0, GPT2_EPI_ACCUMULATE, false, false, false>(
        p0, xcd_remap(b, units0), lds0, lds1);
  } else {
    const int n1 = (int)gridDim.x - units0;
    const int u = b - units0;
    gemm2_unit<BM, BN, BK, WGM, WGN, 2, A_K1, B_K1, GPT2_EPI_ACCUMULATE, false, false, false>(
        p1, (units0 & 7) == 0 ? xcd_remap(u, n1) : u, lds0, lds1);
  }
}

}  // namespace g2
