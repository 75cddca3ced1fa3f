// Internal declarations shared by the HIP kernels and the host runtime of
// libgpt2hip.so.  Not part of the public C-ABI (see include/gpt2.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/gpt2.h"

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace g2 {

// Device error flag values (the most severe wins: lower is more severe).
__host__ __device__ inline int flag_rank(int s) {
  return s == GPT2_OK ? 0 : (s == GPT2_WARN_NO_TARGETS ? 1 : (s == GPT2_ERR_BAD_ID ? 2 : 3));
}

// Raise the device flag to `code` unless it already holds something more
// severe.  Uses a vector-memory atomic.
__device__ inline void raise_flag(int* flag, int code) {
  if (!flag) return;
  int old = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while (flag_rank(code) > flag_rank(old)) {
    int prev = atomicCAS(flag, old, code);
    if (prev == old) break;
    old = prev;
  }
}

__device__ __forceinline__ float bf2f(bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ bf16 f2bf(float x) { return static_cast<bf16>(x); }

// Element type helpers for kernels templated on float / bf16 storage.
template <typename T> __device__ __forceinline__ float to_f(T x);
template <> __device__ __forceinline__ float to_f<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f<bf16>(bf16 x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return static_cast<bf16>(x); }

// GELU, tanh form ("How I trained my own GPT-2 124M on FineWeb-Edu" 2.13):
// 0.5 u (1 + tanh(z/2)) with z = 2 sqrt(2/pi) (u + 0.044715 u^3), which is
// u * sigmoid(z) since 1 + tanh(z/2) = 2 sigmoid(z).  sigmoid(z) is
// 1 / (1 + 2^(-z log2 e)), evaluated with the hardware exp2 and reciprocal
// (v_exp_f32, v_rcp_f32; a result that would be denormal flushes to zero,
// which only moves sigmoid by less than 2^-126).  The derivative is
// sigmoid(z) + u sigmoid(z) (1 - sigmoid(z)) dz/du with
// dz/du = 2 sqrt(2/pi) (1 + 3 * 0.044715 u^2).
namespace gelu_k {
constexpr float K2 = 1.5957691216057308f;            // 2 sqrt(2/pi)
constexpr float C1 = -K2 * 1.4426950408889634f;      // -z / u at u = 0, in log2 units
constexpr float C3 = C1 * 0.044715f;                 // cubic term of the same
constexpr float D0 = K2, D2 = K2 * 3.0f * 0.044715f;  // dz/du = D0 + D2 u^2
}  // namespace gelu_k
// sigmoid(z(u)), given u and u^2
__device__ __forceinline__ float gelu_sig(float u, float u2) {
  const float a = u * fmaf(gelu_k::C3, u2, gelu_k::C1);  // -z log2 e
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a));
}
__device__ __forceinline__ float gelu_tanh(float u) { return u * gelu_sig(u, u * u); }
// gelu(u) and gelu'(u) from one sigmoid evaluation
__device__ __forceinline__ void gelu_tanh_and_grad(float u, float& g, float& dg) {
  const float u2 = u * u;
  const float s = gelu_sig(u, u2);
  g = u * s;
  dg = fmaf(u * fmaf(-s, s, s), fmaf(gelu_k::D2, u2, gelu_k::D0), s);
}
__device__ __forceinline__ float gelu_tanh_grad(float u) {
  const float u2 = u * u;
  const float s = gelu_sig(u, u2);
  const float dz = fmaf(gelu_k::D2, u2, gelu_k::D0);
  return fmaf(u * fmaf(-s, s, s), dz, s);
}

// Kernel launch bookkeeping: the runtime passes a Launch to every launcher,
// which records HIP events around the kernel when profiling is on.
struct Prof;
struct Launch {
  hipStream_t stream;
  Prof* prof;      // may be null
  const char* site;
};
void prof_begin(const Launch& L);
void prof_end(const Launch& L);

// ---------------------------------------------------------------- launchers
// Each returns a hipError_t from the launch (hipSuccess when fine) after
// host-side shape checks done by the caller.

// row_sum (optional): row_sum[m] += alpha * sum_k A(m, k) -- the bias gradient of
// a weight-gradient product (bf16 only).
hipError_t launch_gemm(const Launch& L, const gpt2_gemm_args& a, float* row_sum = nullptr);
// Grouped weight-gradient products (bf16, both operands K-slow, ACCUMULATE
// into float32, optional bias row sums): n products in one launch, one
// 256x256 output tile per block and no K split, so no atomics on C.  The
// group table lives in device memory (gemm_grouped_table_bytes); its image
// is built on the host by gemm_grouped_table and copied there by the caller.
int gemm_grouped_units(const gpt2_gemm_args* a, int n);
size_t gemm_grouped_table_bytes(int n, int units);
void gemm_grouped_table(const gpt2_gemm_args* a, float* const* row_sums, int n, int units, void* host);
// K_all > 0: every product reduces over K_all (the table's own K values and
// splits are kept otherwise).
hipError_t launch_gemm_grouped(const Launch& L, const void* d_table, int n, int units, int K_all = 0);
// Two bf16 ACCUMULATE products in one launch: a0 with A K-major and B
// K-slow, a1 with both K-slow (the lm_head's dZ and dW products of one row
// chunk); each may be split in K (atomic adds), as a plan of the launch's
// span decides.
hipError_t launch_gemm_pair(const Launch& L, const gpt2_gemm_args& a0, const gpt2_gemm_args& a1);
hipError_t launch_colsum(const Launch& L, const void* y, int y_bf16, int M, int N, int64_t ld, float* db);

hipError_t launch_layernorm_fwd(const Launch& L, const float* x, const float* w, const float* b, void* y,
                                int y_bf16, float* mean, float* rstd, int rows, int C);
// dx is added into `dx` (accumulate = 0: written, `dx` not read); when dxb is
// non-null it also receives bf16(dx_new).
// dw / db are added into with atomics, or, when `part` is non-null, each of
// ln_bwd_part_blocks(rows, C) blocks stores its row of 2C column partials
// there (dw then db) for launch_ln_param_grad to sum; 0 blocks: no such mode.
int ln_bwd_part_blocks(int rows, int C);
hipError_t launch_layernorm_bwd_b(const Launch& L, const void* dy, int dy_bf16, const float* x, const float* mean,
                                  const float* rstd, const float* w, float* dx, bf16* dxb, float* dw, float* db,
                                  int rows, int C, float* part = nullptr, int accumulate = 1);
// The weight (and bias) gradients of up to kLnGradSites norm sites from their
// partial rows: site s's rows start at part + s * blocks * 2C; db[s] may be
// null (RMSNorm).
constexpr int kLnGradSites = 64;
struct LnGradSites {
  float* dw[kLnGradSites];
  float* db[kLnGradSites];
};
hipError_t launch_ln_param_grad(const Launch& L, const float* part, int rows, int C, const LnGradSites& sites,
                                int nsites);
// Rotary embedding, head dimension 64: the (cos, sin) table [T][32] and the
// backward rotation of the q and k blocks of dqkv in place.
hipError_t launch_rope_table(const Launch& L, float2* tab, int T, double base);
hipError_t launch_rope_bwd(const Launch& L, bf16* dqkv, int rows, int64_t ld, int cols, int period,
                           const float2* tab);
// RMSNorm of the rotary variant (C % 256 == 0, C <= 1024).
hipError_t launch_rmsnorm_fwd(const Launch& L, const float* x, const float* w, bf16* y, float* rstd, int rows, int C);
hipError_t launch_rmsnorm_bwd(const Launch& L, const void* dy, int dy_bf16, const float* x, const float* rstd,
                              const float* w, float* dx, bf16* dxb, float* dw, int rows, int C,
                              float* part = nullptr, int accumulate = 1);

// seg: [B, T] document starts of packed windows (nullptr: plain causal).
// Hkv key/value heads (H % Hkv == 0); qkv rows [H q | Hkv k | Hkv v] heads.
hipError_t launch_attention_fwd(const Launch& L, int dtype, int B, int T, int H, int Hkv, int hd, const void* qkv,
                                void* y, float* lse, const int32_t* seg);
// rope (nullable, bf16 only): [T][32] (cos, sin) table; dq and dk are
// rotated back with it before they are written.
hipError_t launch_attention_bwd(const Launch& L, int dtype, int B, int T, int H, int Hkv, int hd, const void* qkv,
                                const void* y, const void* dy, const float* lse, void* dqkv, void* scratch,
                                const int32_t* seg, const float2* rope);
size_t attention_bwd_scratch(int B, int T, int H);

// seg[b, t] = last position s <= t of row b with tok[b, s] == eot (0 if none).
hipError_t launch_segment_starts(const Launch& L, const int32_t* tok, int B, int T, int eot, int32_t* seg);
// seg (nullable): positions restart at each document start, t - seg[b, t].
hipError_t launch_embed_fwd(const Launch& L, const int32_t* tok, const float* wte, const float* wpe, float* out,
                            int B, int T, int C, int V, int* flag, const int32_t* seg);
// Deterministic: every gradient row sums its token's (position's) rows in a
// fixed order.  part: [B*T, C] float32 scratch; ws: embed_bwd_scratch bytes.
size_t embed_bwd_scratch(int rows);
int embed_bwd_max_rows();  // rows (B * T) one backward call can take: 131,072
hipError_t launch_embed_bwd(const Launch& L, const int32_t* tok, const float* dr, float* dwte, float* dwpe, int B,
                            int T, int C, int V, const int32_t* seg, float* part, void* ws);

// Cross-entropy helpers for the chunked lm_head.
// count = number of targets in [0, V) other than ignore_index (the fp32 row
// pass ignores -1).
hipError_t launch_count_targets(const Launch& L, const int32_t* tgt, int n, int V, int ignore_index, int* count,
                                int* flag);
template <typename LT, typename DT>
hipError_t launch_ce_rows(const Launch& L, const LT* logits, int64_t ld_logits, DT* dlogits, int64_t ld_d,
                          const int32_t* tgt, int rows, int V, const int* count, float scale, float* loss_sum,
                          float* token_loss);
hipError_t launch_ce_finish_n(const Launch& L, const float* row_loss, int n, const int* count, float* loss,
                              int* flag);

// Fused lm_head + cross-entropy (bf16): the logits product writes per-tile
// softmax statistics and bf16 logits offset by their tile maximum (ld = V),
// then one pass per row turns them into dlogits in place.
constexpr int kCeTile = 256;  // columns per statistics tile
inline int ce_stat_tiles(int V) { return (V + kCeTile - 1) / kCeTile; }
hipError_t launch_gemm_ce_stats(const Launch& L, const bf16* hidden, const bf16* wte, bf16* y, float2* stats, int M,
                                int V, int C);
hipError_t launch_ce_apply(const Launch& L, bf16* y, const float2* stats, const bf16* hidden, const bf16* wte,
                           const int32_t* tgt, int rows, int V, int C, int ignore_index, const int* count,
                           float scale, float* row_loss);

// Optimizer.
hipError_t launch_sumsq_partials(const Launch& L, const float* g, size_t n, float* partials, int nparts);
// The norm of the partials and, when it is finite, ++step[0] and the update
// scalars sc[4] (one block, on Lprep), then the update pass (on L).
hipError_t launch_adamw(const Launch& L, const Launch& Lprep, float* p, const float* g, float* m, float* v,
                        bf16* shadow, size_t n, size_t decay_end, const float* partials, int nparts, float lr,
                        float b1, float b2, float eps, float wd, float max_norm, int64_t* step, float* sc,
                        float* norm_out, int* flag);
hipError_t launch_fill_f32(const Launch& L, float* p, size_t n, float value);
hipError_t launch_fill_i32(const Launch& L, int* p, size_t n, int value);
hipError_t launch_to_bf16(const Launch& L, const float* src, bf16* dst, size_t n);
hipError_t launch_init_normal(const Launch& L, float* dst, size_t n, uint32_t tensor_index, uint64_t seed,
                              float std);

}  // namespace g2
