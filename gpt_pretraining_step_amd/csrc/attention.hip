// Causal multi-head self-attention, forward and backward ("How I trained my
// own GPT-2 124M on FineWeb-Edu" 2.12 and 5: S = q k^T / sqrt(hd), keys after
// the query masked, softmax over keys, o = P v; section 5 replaces the
// materialised form with a tiled flash kernel that never stores S).
//
// bf16, head_dim 64: MFMA 32x32x16 tiles.  The forward and the dQ pass work
// in the transposed orientation, S^T = K Q^T and O^T = V^T P^T, so that every
// lane owns one query: softmax statistics are per-lane scalars (plus one
// exchange with the partner lane 32 away) and the S^T accumulator feeds the
// next product directly as its B operand.  The dK/dV pass works in the
// direct orientation S = Q K^T so that each lane owns one key.  Operands whose
// contraction index is the slow one in memory are transposed once per tile
// in LDS (8x8 blocks through registers).  The MFMA k-slots of an accumulator
// used as an operand follow the accumulator's row order (row 8*(r/4) + 4*g +
// r%4 of register r in lane group g); the matching operand is read in that
// same order.
//
// Backward (derived from the forward by the chain rule): D = rowsum(dO o O),
// P recomputed from the saved row log-sum-exp, dV = P^T dO,
// dS = P o (dO V^T - D), dQ = dS K / sqrt(hd), dK = dS^T Q / sqrt(hd).
//
// float32 (FP32 precision mode, small heads): one thread per query (or key),
// plain loops.
#include "common.h"

namespace g2 {

constexpr float kLOG2E = 1.4426950408889634f;
constexpr float kLN2 = 0.6931471805599453f;

// ========================================================= float32 kernels

__global__ void attn_fwd_f32_kernel(const float* __restrict__ qkv, float* __restrict__ y, float* __restrict__ lse,
                                    int B, int T, int H, int hd, float scale) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * H * T) return;
  const int t = i % T, bh = i / T, h = bh % H, b = bh / H;
  const int C = H * hd, C3 = 3 * C;
  const float* q = qkv + ((int64_t)b * T + t) * C3 + h * hd;
  float acc[64];
  for (int d = 0; d < hd; ++d) acc[d] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int s = 0; s <= t; ++s) {
    const float* k = qkv + ((int64_t)b * T + s) * C3 + C + h * hd;
    const float* v = k + C;
    float sc = 0.f;
    for (int d = 0; d < hd; ++d) sc += q[d] * k[d];
    sc *= scale;
    const float mn = fmaxf(m, sc);
    const float a = expf(m - mn), p = expf(sc - mn);
    l = l * a + p;
    for (int d = 0; d < hd; ++d) acc[d] = acc[d] * a + p * v[d];
    m = mn;
  }
  float* o = y + ((int64_t)b * T + t) * C + h * hd;
  for (int d = 0; d < hd; ++d) o[d] = acc[d] / l;
  lse[i] = m + logf(l);
}

__global__ void attn_bwd_dq_f32_kernel(const float* __restrict__ qkv, const float* __restrict__ y,
                                       const float* __restrict__ dy, const float* __restrict__ lse,
                                       float* __restrict__ dqkv, float* __restrict__ Dbuf, int B, int T, int H, int hd,
                                       float scale) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * H * T) return;
  const int t = i % T, bh = i / T, h = bh % H, b = bh / H;
  const int C = H * hd, C3 = 3 * C;
  const float* q = qkv + ((int64_t)b * T + t) * C3 + h * hd;
  const float* o = y + ((int64_t)b * T + t) * C + h * hd;
  const float* dO = dy + ((int64_t)b * T + t) * C + h * hd;
  float D = 0.f;
  for (int d = 0; d < hd; ++d) D += dO[d] * o[d];
  Dbuf[i] = D;
  float acc[64];
  for (int d = 0; d < hd; ++d) acc[d] = 0.f;
  const float L = lse[i];
  for (int s = 0; s <= t; ++s) {
    const float* k = qkv + ((int64_t)b * T + s) * C3 + C + h * hd;
    const float* v = k + C;
    float sc = 0.f, dp = 0.f;
    for (int d = 0; d < hd; ++d) {
      sc += q[d] * k[d];
      dp += dO[d] * v[d];
    }
    const float p = expf(sc * scale - L);
    const float ds = p * (dp - D);
    for (int d = 0; d < hd; ++d) acc[d] += ds * k[d];
  }
  float* dq = dqkv + ((int64_t)b * T + t) * C3 + h * hd;
  for (int d = 0; d < hd; ++d) dq[d] = acc[d] * scale;
}

__global__ void attn_bwd_dkdv_f32_kernel(const float* __restrict__ qkv, const float* __restrict__ dy,
                                         const float* __restrict__ lse, const float* __restrict__ Dbuf,
                                         float* __restrict__ dqkv, int B, int T, int H, int hd, float scale) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * H * T) return;
  const int s = i % T, bh = i / T, h = bh % H, b = bh / H;
  const int C = H * hd, C3 = 3 * C;
  const float* k = qkv + ((int64_t)b * T + s) * C3 + C + h * hd;
  const float* v = k + C;
  float dk[64], dv[64];
  for (int d = 0; d < hd; ++d) dk[d] = dv[d] = 0.f;
  for (int t = s; t < T; ++t) {
    const float* q = qkv + ((int64_t)b * T + t) * C3 + h * hd;
    const float* dO = dy + ((int64_t)b * T + t) * C + h * hd;
    float sc = 0.f, dp = 0.f;
    for (int d = 0; d < hd; ++d) {
      sc += q[d] * k[d];
      dp += dO[d] * v[d];
    }
    const float p = expf(sc * scale - lse[bh * T + t]);
    const float ds = p * (dp - Dbuf[bh * T + t]);
    for (int d = 0; d < hd; ++d) {
      dv[d] += p * dO[d];
      dk[d] += ds * q[d];
    }
  }
  float* o = dqkv + ((int64_t)b * T + s) * C3 + C + h * hd;
  for (int d = 0; d < hd; ++d) {
    o[d] = dk[d] * scale;
    o[C + d] = dv[d];
  }
}

// ============================================================ bf16 kernels

constexpr int HD = 64;
constexpr int RP = HD + 8;  // pitch of [row][d] tiles (elements)
constexpr int TP = 64 + 8;  // pitch of [d][row] tiles (elements)

union V8 {
  uint4 u;
  bf16x8 v;
  uint32_t w[4];
};
union V4 {
  uint2 u;
  bf16x4 v;
};

// rows row0..row0+63 of a [*, ld] bf16 matrix (columns 0..63 from g) -> LDS
// [64][RP]; rows >= nrows are zero.
__device__ __forceinline__ void load_rows64(bf16* lds, const bf16* __restrict__ g, int64_t ld, int row0, int nrows) {
  for (int c = threadIdx.x; c < 64 * 8; c += 256) {
    const int r = c >> 3, c8 = c & 7;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row0 + r < nrows) v = *reinterpret_cast<const uint4*>(g + (int64_t)(row0 + r) * ld + 8 * c8);
    *reinterpret_cast<uint4*>(lds + r * RP + 8 * c8) = v;
  }
}

// dst[d][r] = src[r][d] for a 64x64 tile; 64 threads, one 8x8 block each.
__device__ __forceinline__ void transpose64(bf16* dst, const bf16* src, int tid) {
  if (tid < 0 || tid >= 64) return;
  const int rb = tid >> 3, db = tid & 7;
  V8 in[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) in[j].u = *reinterpret_cast<const uint4*>(src + (8 * rb + j) * RP + 8 * db);
#pragma unroll
  for (int dd = 0; dd < 8; ++dd) {
    const int word = dd >> 1;
    const bool hi = dd & 1;
    V8 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a = in[2 * q].w[word], b = in[2 * q + 1].w[word];
      o.w[q] = hi ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
    }
    *reinterpret_cast<uint4*>(dst + (8 * db + dd) * TP + 8 * rb) = o.u;
  }
}

// MFMA operand holding row (base + lane%32), k-slots 16kk + 8g .. +7 of a
// [row][d] tile.
__device__ __forceinline__ bf16x8 row_frag(const bf16* t, int base, int kk, int lr, int lg) {
  return *reinterpret_cast<const bf16x8*>(t + (base + lr) * RP + 16 * kk + 8 * lg);
}
// MFMA operand from a [d][row] tile: row d, k-slots mapped to rows
// kbase + 8*(e/4) + 4g + e%4 (the accumulator row order).
__device__ __forceinline__ bf16x8 tr_frag(const bf16* t, int d, int kbase, int lg) {
  V4 a, b;
  a.u = *reinterpret_cast<const uint2*>(t + d * TP + kbase + 4 * lg);
  b.u = *reinterpret_cast<const uint2*>(t + d * TP + kbase + 8 + 4 * lg);
  bf16x8 r;
  r[0] = a.v[0]; r[1] = a.v[1]; r[2] = a.v[2]; r[3] = a.v[3];
  r[4] = b.v[0]; r[5] = b.v[1]; r[6] = b.v[2]; r[7] = b.v[3];
  return r;
}
// registers 8s..8s+7 of an accumulator, as a bf16 operand
__device__ __forceinline__ bf16x8 acc_frag(const f32x16& a, int s) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = f2bf(a[8 * s + e]);
  return r;
}
__device__ __forceinline__ bf16x8 load8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = f2bf(0.f);
  return z;
}
__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.f;
  return z;
}
#define MFMA(a, b, c) __builtin_amdgcn_mfma_f32_32x32x16_bf16((a), (b), (c), 0, 0, 0)

// Forward: block = 4 waves x 32 queries; loop over 64-key blocks.
__global__ __launch_bounds__(256) void attn_fwd_bf16_kernel(const bf16* __restrict__ qkv, bf16* __restrict__ y,
                                                            float* __restrict__ lse, int T, int H, float sl2) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[64 * RP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[64 * RP];
  __shared__ __attribute__((aligned(16))) bf16 Vt[64 * TP];
  const int nqb = (T + 127) / 128;
  const int qb = nqb - 1 - blockIdx.x;  // longest rows first
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int C = H * HD, C3 = 3 * C;
  const bf16* Qg = qkv + (int64_t)b * T * C3 + h * HD;
  const bf16* Kg = Qg + C;
  const bf16* Vg = Qg + 2 * C;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const int q0 = qb * 128 + wave * 32;
  const int qi = q0 + lr;

  bf16x8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qf[kk] = (qi < T) ? load8(Qg + (int64_t)qi * C3 + 16 * kk + 8 * lg) : zero8();
  f32x16 oT[2] = {zero16(), zero16()};
  float m = -1e30f, l = 0.f;
  const int kv_end = min(T, qb * 128 + 128);
  for (int kb = 0; kb < kv_end; kb += 64) {
    __syncthreads();
    load_rows64(Ks, Kg, C3, kb, T);
    load_rows64(Vs, Vg, C3, kb, T);
    __syncthreads();
    transpose64(Vt, Vs, threadIdx.x);
    __syncthreads();
    if (q0 >= T || kb > q0 + 31) continue;
    f32x16 sT[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      sT[c] = zero16();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) sT[c] = MFMA(row_frag(Ks, 32 * c, kk, lr, lg), qf[kk], sT[c]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb + 32 * c + 8 * (r >> 2) + 4 * lg + (r & 3);
        float v = sT[c][r] * sl2;
        if (key > qi || key >= T) v = -INFINITY;
        sT[c][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    const float alpha = exp2f(m - mn);
    m = mn;
    float ls = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(sT[c][r] - mn);
        sT[c][r] = p;
        ls += p;
      }
    l = l * alpha + ls;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oT[dt][r] *= alpha;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 pb = acc_frag(sT[c], s);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) oT[dt] = MFMA(tr_frag(Vt, 32 * dt + lr, 32 * c + 16 * s, lg), pb, oT[dt]);
      }
  }
  l += __shfl_xor(l, 32);
  if (qi < T) {
    const float inv = 1.f / l;
    bf16* yo = y + ((int64_t)b * T + qi) * C + h * HD;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = f2bf(oT[dt][4 * a + e] * inv);
        *reinterpret_cast<bf16x4*>(yo + 32 * dt + 8 * a + 4 * lg) = o4;
      }
    if (lg == 0) lse[(int64_t)bh * T + qi] = (m + log2f(l)) * kLN2;
  }
}

// Backward, pass 1: D = rowsum(dO o O) and dQ.  Same tiling as the forward.
__global__ __launch_bounds__(256) void attn_bwd_dq_bf16_kernel(const bf16* __restrict__ qkv,
                                                               const bf16* __restrict__ y, const bf16* __restrict__ dy,
                                                               const float* __restrict__ lse, bf16* __restrict__ dqkv,
                                                               float* __restrict__ Dbuf, int T, int H, float scale,
                                                               float sl2) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[64 * RP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[64 * RP];
  __shared__ __attribute__((aligned(16))) bf16 Kt[64 * TP];
  const int nqb = (T + 127) / 128;
  const int qb = nqb - 1 - blockIdx.x;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int C = H * HD, C3 = 3 * C;
  const bf16* Qg = qkv + (int64_t)b * T * C3 + h * HD;
  const bf16* Kg = Qg + C;
  const bf16* Vg = Qg + 2 * C;
  const bf16* Og = y + (int64_t)b * T * C + h * HD;
  const bf16* dOg = dy + (int64_t)b * T * C + h * HD;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const int q0 = qb * 128 + wave * 32;
  const int qi = q0 + lr;
  const bool qv = qi < T;

  bf16x8 qf[4], dof[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    qf[kk] = qv ? load8(Qg + (int64_t)qi * C3 + 16 * kk + 8 * lg) : zero8();
    dof[kk] = qv ? load8(dOg + (int64_t)qi * C + 16 * kk + 8 * lg) : zero8();
  }
  float Dp = 0.f;
  if (qv) {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const bf16x8 o8 = load8(Og + (int64_t)qi * C + 32 * lg + 8 * cc);
      const bf16x8 d8 = load8(dOg + (int64_t)qi * C + 32 * lg + 8 * cc);
#pragma unroll
      for (int e = 0; e < 8; ++e) Dp += bf2f(o8[e]) * bf2f(d8[e]);
    }
  }
  const float D = Dp + __shfl_xor(Dp, 32);
  if (qv && lg == 0) Dbuf[(int64_t)bh * T + qi] = D;
  const float lse2 = qv ? lse[(int64_t)bh * T + qi] * kLOG2E : 0.f;

  f32x16 dqT[2] = {zero16(), zero16()};
  const int kv_end = min(T, qb * 128 + 128);
  for (int kb = 0; kb < kv_end; kb += 64) {
    __syncthreads();
    load_rows64(Ks, Kg, C3, kb, T);
    load_rows64(Vs, Vg, C3, kb, T);
    __syncthreads();
    transpose64(Kt, Ks, threadIdx.x);
    __syncthreads();
    if (q0 >= T || kb > q0 + 31) continue;
    f32x16 sT[2], dpT[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      sT[c] = zero16();
      dpT[c] = zero16();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        sT[c] = MFMA(row_frag(Ks, 32 * c, kk, lr, lg), qf[kk], sT[c]);
        dpT[c] = MFMA(row_frag(Vs, 32 * c, kk, lr, lg), dof[kk], dpT[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb + 32 * c + 8 * (r >> 2) + 4 * lg + (r & 3);
        const float p = (key <= qi && key < T) ? exp2f(sT[c][r] * sl2 - lse2) : 0.f;
        sT[c][r] = p * (dpT[c][r] - D);
      }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 db = acc_frag(sT[c], s);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) dqT[dt] = MFMA(tr_frag(Kt, 32 * dt + lr, 32 * c + 16 * s, lg), db, dqT[dt]);
      }
  }
  if (qv) {
    bf16* o = dqkv + ((int64_t)b * T + qi) * C3 + h * HD;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = f2bf(dqT[dt][4 * a + e] * scale);
        *reinterpret_cast<bf16x4*>(o + 32 * dt + 8 * a + 4 * lg) = o4;
      }
  }
}

// Backward, pass 2: dK and dV.  Block = 4 waves x 32 keys; loop over 64-query
// blocks from the block's diagonal to T.
__global__ __launch_bounds__(256) void attn_bwd_dkdv_bf16_kernel(const bf16* __restrict__ qkv,
                                                                 const bf16* __restrict__ dy,
                                                                 const float* __restrict__ lse,
                                                                 const float* __restrict__ Dbuf,
                                                                 bf16* __restrict__ dqkv, int T, int H, float scale,
                                                                 float sl2) {
  __shared__ __attribute__((aligned(16))) bf16 Qs[64 * RP];
  __shared__ __attribute__((aligned(16))) bf16 dOs[64 * RP];
  __shared__ __attribute__((aligned(16))) bf16 Qt[64 * TP];
  __shared__ __attribute__((aligned(16))) bf16 dOt[64 * TP];
  __shared__ __attribute__((aligned(16))) float lse_s[64];
  __shared__ __attribute__((aligned(16))) float D_s[64];
  const int kblk = blockIdx.x;  // smallest keys (most queries) first
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int C = H * HD, C3 = 3 * C;
  const bf16* Qg = qkv + (int64_t)b * T * C3 + h * HD;
  const bf16* Kg = Qg + C;
  const bf16* Vg = Qg + 2 * C;
  const bf16* dOg = dy + (int64_t)b * T * C + h * HD;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const int k0 = kblk * 128 + wave * 32;
  const int kj = k0 + lr;
  const bool kvld = kj < T;

  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    kf[kk] = kvld ? load8(Kg + (int64_t)kj * C3 + 16 * kk + 8 * lg) : zero8();
    vf[kk] = kvld ? load8(Vg + (int64_t)kj * C3 + 16 * kk + 8 * lg) : zero8();
  }
  f32x16 dvT[2] = {zero16(), zero16()}, dkT[2] = {zero16(), zero16()};
  for (int qs = kblk * 128; qs < T; qs += 64) {
    __syncthreads();
    load_rows64(Qs, Qg, C3, qs, T);
    load_rows64(dOs, dOg, C, qs, T);
    if (threadIdx.x < 64) {
      const int q = qs + threadIdx.x;
      lse_s[threadIdx.x] = (q < T) ? lse[(int64_t)bh * T + q] * kLOG2E : INFINITY;
      D_s[threadIdx.x] = (q < T) ? Dbuf[(int64_t)bh * T + q] : 0.f;
    }
    __syncthreads();
    transpose64(Qt, Qs, threadIdx.x);
    transpose64(dOt, dOs, threadIdx.x - 64);
    __syncthreads();
    if (k0 >= T) continue;
    if (qs + 63 < k0) continue;
    f32x16 sc[2], dp[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      sc[c] = zero16();
      dp[c] = zero16();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        sc[c] = MFMA(row_frag(Qs, 32 * c, kk, lr, lg), kf[kk], sc[c]);
        dp[c] = MFMA(row_frag(dOs, 32 * c, kk, lr, lg), vf[kk], dp[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int ql = 32 * c + 8 * a + 4 * lg;
        const float4 L4 = *reinterpret_cast<const float4*>(lse_s + ql);
        const float4 D4 = *reinterpret_cast<const float4*>(D_s + ql);
        const float Ls[4] = {L4.x, L4.y, L4.z, L4.w};
        const float Ds[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * a + e;
          const int q = qs + ql + e;
          const float p = (kj <= q && q < T) ? exp2f(sc[c][r] * sl2 - Ls[e]) : 0.f;
          sc[c][r] = p;
          dp[c][r] = p * (dp[c][r] - Ds[e]);
        }
      }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 pb = acc_frag(sc[c], s);
        const bf16x8 db = acc_frag(dp[c], s);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          dvT[dt] = MFMA(tr_frag(dOt, 32 * dt + lr, 32 * c + 16 * s, lg), pb, dvT[dt]);
          dkT[dt] = MFMA(tr_frag(Qt, 32 * dt + lr, 32 * c + 16 * s, lg), db, dkT[dt]);
        }
      }
  }
  if (kvld) {
    bf16* ok = dqkv + ((int64_t)b * T + kj) * C3 + C + h * HD;
    bf16* ov = ok + C;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 k4, v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k4[e] = f2bf(dkT[dt][4 * a + e] * scale);
          v4[e] = f2bf(dvT[dt][4 * a + e]);
        }
        *reinterpret_cast<bf16x4*>(ok + 32 * dt + 8 * a + 4 * lg) = k4;
        *reinterpret_cast<bf16x4*>(ov + 32 * dt + 8 * a + 4 * lg) = v4;
      }
  }
}

// =============================================================== launchers

hipError_t launch_attention_fwd(const Launch& L, int dtype, int B, int T, int H, int hd, const void* qkv, void* y,
                                float* lse) {
  const float scale = 1.f / sqrtf((float)hd);
  prof_begin(L);
  if (dtype == GPT2_PRECISION_BF16) {
    dim3 grid((T + 127) / 128, B * H);
    attn_fwd_bf16_kernel<<<grid, 256, 0, L.stream>>>(static_cast<const bf16*>(qkv), static_cast<bf16*>(y), lse, T, H,
                                                     scale * kLOG2E);
  } else {
    const int n = B * H * T;
    attn_fwd_f32_kernel<<<(n + 127) / 128, 128, 0, L.stream>>>(static_cast<const float*>(qkv), static_cast<float*>(y),
                                                              lse, B, T, H, hd, scale);
  }
  prof_end(L);
  return hipGetLastError();
}

size_t attention_bwd_scratch(int B, int T, int H) { return (size_t)B * T * H * sizeof(float); }

hipError_t launch_attention_bwd(const Launch& L, int dtype, int B, int T, int H, int hd, const void* qkv,
                                const void* y, const void* dy, const float* lse, void* dqkv, void* scratch) {
  const float scale = 1.f / sqrtf((float)hd);
  float* Dbuf = static_cast<float*>(scratch);
  prof_begin(L);
  if (dtype == GPT2_PRECISION_BF16) {
    dim3 grid((T + 127) / 128, B * H);
    attn_bwd_dq_bf16_kernel<<<grid, 256, 0, L.stream>>>(static_cast<const bf16*>(qkv), static_cast<const bf16*>(y),
                                                        static_cast<const bf16*>(dy), lse, static_cast<bf16*>(dqkv),
                                                        Dbuf, T, H, scale, scale * kLOG2E);
    attn_bwd_dkdv_bf16_kernel<<<grid, 256, 0, L.stream>>>(static_cast<const bf16*>(qkv), static_cast<const bf16*>(dy),
                                                          lse, Dbuf, static_cast<bf16*>(dqkv), T, H, scale,
                                                          scale * kLOG2E);
  } else {
    const int n = B * H * T;
    attn_bwd_dq_f32_kernel<<<(n + 127) / 128, 128, 0, L.stream>>>(
        static_cast<const float*>(qkv), static_cast<const float*>(y), static_cast<const float*>(dy), lse,
        static_cast<float*>(dqkv), Dbuf, B, T, H, hd, scale);
    attn_bwd_dkdv_f32_kernel<<<(n + 127) / 128, 128, 0, L.stream>>>(static_cast<const float*>(qkv),
                                                                   static_cast<const float*>(dy), lse, Dbuf,
                                                                   static_cast<float*>(dqkv), B, T, H, hd, scale);
  }
  prof_end(L);
  return hipGetLastError();
}

}  // namespace g2
