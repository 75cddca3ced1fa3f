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
// contraction index is the slow one in memory are read from LDS with the
// transposing read.  The MFMA k-slots of an accumulator
// used as an operand follow the accumulator's row order (row 8*(r/4) + 4*g +
// r%4 of register r in lane group g); the matching operand is read in that
// same order.
//
// Backward (derived from the forward by the chain rule): D = rowsum(dO o O),
// P recomputed from the saved row log-sum-exp, dV = P^T dO,
// dS = P o (dO V^T - D), dQ = dS K / sqrt(hd), dK = dS^T Q / sqrt(hd).
//
// Packed windows ("GPT" chapter of Zero to Frontier, "Document boundaries,
// packing and masking"): with a document mask, query t of a row sees only
// the keys s with start[t] <= s <= t, start[t] being the first position of
// t's document (seg, [B, T] int32, non-decreasing along a row with
// start[t] <= t).  Whole key tiles before the block's first document start
// are not copied at all, each wave computes only from its own first
// document start, and the remaining tiles are masked per element where they
// reach below some query's start.  seg == nullptr is the plain causal mask.
//
// Within a block every wave takes part in the copies and barriers of all
// tiles but runs the products only on the tiles it can see (the causal
// diagonal leaves the last forward tile of the first two waves, and the
// first dK/dV tile of the last two, wholly masked).
//
// Grouped-query attention ("Build an LLM From Scratch: Making Training Fast
// on One GPU", step 2, the textbook form repeats each key/value head for
// n_head / n_kv_head consecutive query heads): qkv rows hold H query heads,
// then Hkv key heads, then Hkv value heads; query head h reads key/value
// head h / (H / Hkv), and the dK/dV pass runs once per key/value head, its
// loop covering the query heads of the group one after the other, so the
// shared head's gradient is summed in registers.
//
// Rotary variant ("Reproduce GPT-2 124M": q and k rotated after c_attn):
// given the (cos, sin) table of the positions, the bf16 backward applies the
// transpose of the rotation to dQ and dK in registers before their one bf16
// rounding (dims i and i + 32 of a head sit in the same lane), so no
// separate pass over dQKV is needed.
//
// float32 (FP32 precision mode, small heads): one thread per query (or key),
// plain loops.
#include "tile_io.h"

namespace g2 {

constexpr float kLOG2E = 1.4426950408889634f;
constexpr float kLN2 = 0.6931471805599453f;

// ========================================================= float32 kernels

__global__ void attn_fwd_f32_kernel(const float* __restrict__ qkv, float* __restrict__ y, float* __restrict__ lse,
                                    const int32_t* __restrict__ seg, int B, int T, int H, int Hkv, int hd,
                                    float scale) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * H * T) return;
  const int t = i % T, bh = i / T, h = bh % H, b = bh / H;
  const int C = H * hd, Ckv = Hkv * hd, C3 = C + 2 * Ckv, kvo = C + (h / (H / Hkv)) * hd;
  const float* q = qkv + ((int64_t)b * T + t) * C3 + h * hd;
  float acc[64];
  for (int d = 0; d < hd; ++d) acc[d] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int s = seg ? max(seg[(int64_t)b * T + t], 0) : 0; s <= t; ++s) {
    const float* k = qkv + ((int64_t)b * T + s) * C3 + kvo;
    const float* v = k + Ckv;
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
                                       float* __restrict__ dqkv, float* __restrict__ Dbuf,
                                       const int32_t* __restrict__ seg, int B, int T, int H, int Hkv, int hd,
                                       float scale) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * H * T) return;
  const int t = i % T, bh = i / T, h = bh % H, b = bh / H;
  const int C = H * hd, Ckv = Hkv * hd, C3 = C + 2 * Ckv, kvo = C + (h / (H / Hkv)) * hd;
  const float* q = qkv + ((int64_t)b * T + t) * C3 + h * hd;
  const float* o = y + ((int64_t)b * T + t) * C + h * hd;
  const float* dO = dy + ((int64_t)b * T + t) * C + h * hd;
  float D = 0.f;
  for (int d = 0; d < hd; ++d) D += dO[d] * o[d];
  Dbuf[i] = D;
  float acc[64];
  for (int d = 0; d < hd; ++d) acc[d] = 0.f;
  const float L = lse[i];
  for (int s = seg ? max(seg[(int64_t)b * T + t], 0) : 0; s <= t; ++s) {
    const float* k = qkv + ((int64_t)b * T + s) * C3 + kvo;
    const float* v = k + Ckv;
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
                                         float* __restrict__ dqkv, const int32_t* __restrict__ seg, int B, int T,
                                         int H, int Hkv, int hd, float scale) {
  // one thread per (batch, key/value head, key)
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * Hkv * T) return;
  const int s = i % T, bj = i / T, j = bj % Hkv, b = bj / Hkv, grp = H / Hkv;
  const int C = H * hd, Ckv = Hkv * hd, C3 = C + 2 * Ckv;
  const float* k = qkv + ((int64_t)b * T + s) * C3 + C + j * hd;
  const float* v = k + Ckv;
  float dk[64], dv[64];
  for (int d = 0; d < hd; ++d) dk[d] = dv[d] = 0.f;
  for (int h = j * grp; h < (j + 1) * grp; ++h) {
    const int bh = b * H + h;
    for (int t = s; t < T; ++t) {
      if (seg && seg[(int64_t)b * T + t] > s) break;  // t's document starts after key s, as do all later ones
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
  }
  float* o = dqkv + ((int64_t)b * T + s) * C3 + C + j * hd;
  for (int d = 0; d < hd; ++d) {
    o[d] = dk[d] * scale;
    o[Ckv + d] = dv[d];
  }
}

// ============================================================ bf16 kernels
//
// Tiles of 64 rows x 64 head dims (128-byte rows) are copied from HBM into
// LDS by DMA, double-buffered: the next tile's copy is in flight while the
// current one is multiplied, one barrier per tile.  The copies are issued
// through inline asm (tile_io.h): the compiler would otherwise drain them
// before every transposing read; the explicit wait at the top of each tile
// orders them.  Rows are stored with
// their 16-byte chunks swizzled (tile_io.h).  Operands read along a row
// (K, V, Q, dO rows) use 16-byte LDS reads; operands read along a column
// (V^T, K^T, Q^T, dO^T) use the transposing LDS read, so no tile is ever
// transposed in memory.

constexpr int HD = 64;

union V8 {
  uint4 u;
  bf16x8 v;
  uint32_t w[4];
};

// MFMA operand: row `row` of a swizzled tile, k-slots 16kk + 8lg .. +7.
__device__ __forceinline__ bf16x8 rowfrag(const bf16* t, int row, int kk, int lg) {
  return *reinterpret_cast<const bf16x8*>(t + row * HD + 8 * swz_chunk<64>(row, 2 * kk + lg));
}
// MFMA operand: column d = d0 + lane%32 of a swizzled tile, with k-slots in
// the accumulator row order: slots 0..3 <-> rows r0 + 4lg + 0..3, slots
// 4..7 <-> rows r0 + 8 + 4lg + 0..3.
__device__ __forceinline__ bf16x8 colfrag(const bf16* t, int r0, int d0, int lg) {
  const int h = (threadIdx.x >> 4) & 1;
  const bf16x4 a = tr_read4(t, r0 + 4 * lg, d0 + 16 * h);
  const bf16x4 b = tr_read4(t, r0 + 8 + 4 * lg, d0 + 16 * h);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
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

// dS = P o (dP - D) without a subtraction per score: -D is split into two
// bf16 values hi = bf16(-D), lo = bf16(-D - hi) (together exact to about
// 2^-17 |D|), which ride as two extra contraction slots of the dP product
// against two ones on the other side.  An MFMA operand's lane holds
// contraction slots 8 lg .. 8 lg + 7, so lanes with lg = 0 carry the pair in
// slots 0 and 1 and all other slots are zero.
__device__ __forceinline__ uint32_t neg_d_pair(float D) {
  const bf16 hi = f2bf(-D);
  const bf16 lo = f2bf(-D - bf2f(hi));
  return (uint32_t)__builtin_bit_cast(uint16_t, hi) | ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16);
}
__device__ __forceinline__ bf16x8 slot01(uint32_t pair, int lg) {
  V8 r;
  r.u = make_uint4(lg ? 0u : pair, 0u, 0u, 0u);
  return r.v;
}
constexpr uint32_t kOnePair = 0x3F803F80u;  // bf16 1.0 in slots 0 and 1

// Write a head's 64 gradient values held as the transposed accumulators g[0]
// (dims 0..31) and g[1] (dims 32..63): register 4a + e of g[dt] is dim
// 32 dt + 8a + 4 lg + e.  With a rotary table (rope != nullptr: row `pos`
// of [T][32] (cos, sin) pairs) the pair (i, i + 32) is first rotated back:
// z_i' = z_i c + z_{i+32} s, z_{i+32}' = z_{i+32} c - z_i s.
__device__ __forceinline__ void store_head_grad(bf16* out, const f32x16 (&g)[2], float scale,
                                                const float2* __restrict__ rope, int pos, int lg) {
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    float lo[4], hi[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = g[0][4 * a + e] * scale;
      hi[e] = g[1][4 * a + e] * scale;
    }
    if (rope) {
      const float4* cs = reinterpret_cast<const float4*>(rope + (int64_t)pos * 32 + 8 * a + 4 * lg);
      const float4 c01 = cs[0], c23 = cs[1];
      const float cv[4] = {c01.x, c01.z, c23.x, c23.z}, sv[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float z1 = lo[e], z2 = hi[e];
        lo[e] = z1 * cv[e] + z2 * sv[e];
        hi[e] = z2 * cv[e] - z1 * sv[e];
      }
    }
    bf16x4 l4, h4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      l4[e] = f2bf(lo[e]);
      h4[e] = f2bf(hi[e]);
    }
    *reinterpret_cast<bf16x4*>(out + 8 * a + 4 * lg) = l4;
    *reinterpret_cast<bf16x4*>(out + 32 + 8 * a + 4 * lg) = h4;
  }
}

// Wait for this wave's outstanding DMA and LDS writes, then meet the other
// waves (no fence: later tiles' copies are not in flight at this point).
__device__ __forceinline__ void tile_barrier() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Forward.  Block = NW waves x 32 queries; loop over 64-key tiles.  Each lane
// owns one query (S^T = K Q^T, O^T = V^T P^T), so the online-softmax state is
// per lane, shared with the partner lane 32 away.
template <int NW, int ST, bool DOC>
__global__ __launch_bounds__(64 * NW) void attn_fwd_bf16_kernel(const bf16* __restrict__ qkv, bf16* __restrict__ y,
                                                                float* __restrict__ lse,
                                                                const int32_t* __restrict__ seg, int T, int H,
                                                                int Hkv, float sl2) {
  constexpr int BQ = 32 * NW;
  constexpr int DMA_TILE = 2 * 64 * HD / 512 / NW;  // DMA instructions per wave per K/V tile
  __shared__ __attribute__((aligned(16))) bf16 sm[ST][2][64 * HD];  // [stage][K, V]
  const int nqb = (T + BQ - 1) / BQ;
  // blocks are dispatched x-fastest: every head's longest (last) query
  // block first, then the next longest, ... (longest work first balances the
  // causal triangle over the compute units)
  const int qb = nqb - 1 - blockIdx.y;
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int C = H * HD, Ckv = Hkv * HD, C3 = C + 2 * Ckv;
  const bf16* Qg = qkv + (int64_t)b * T * C3 + h * HD;
  const bf16* Kg = qkv + (int64_t)b * T * C3 + C + (h / (H / Hkv)) * HD;
  const bf16* Vg = Kg + Ckv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const int q0 = qb * BQ + wave * 32;
  const int qi = q0 + lr;

  bf16x8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qf[kk] = (qi < T) ? load8(Qg + (int64_t)qi * C3 + 16 * kk + 8 * lg) : zero8();
  f32x16 oT[2] = {zero16(), zero16()};
  float m = -1e30f, l = 0.f;
  const int kv_end = min(T, qb * BQ + BQ);
  const int ntiles = (kv_end + 63) / 64;
  // document mask: the key tiles before the block's first query's document
  // start are skipped (that query has the smallest start of the block);
  // seg_lo is this lane's query's start, seg_hi the wave's largest
  int jt0 = 0, seg_lo = 0, seg_hi = 0;
  if constexpr (DOC) {
    const int32_t* sr = seg + (int64_t)b * T;
    jt0 = min(max(sr[qb * BQ] / 64, 0), ntiles - 1);
    seg_lo = sr[min(qi, T - 1)];
    seg_hi = sr[min(q0 + 31, T - 1)];
  }
  auto issue = [&](int st, int tile) {
    dma_rows<64, 64, NW, true>(sm[st][0], Kg, C3, tile * 64, T, 0, HD);
    dma_rows<64, 64, NW, true>(sm[st][1], Vg, C3, tile * 64, T, 0, HD);
  };
  // ST-stage ring: tiles jt+1 .. jt+ST-2 stay in flight while tile jt is
  // used; tile jt+ST-1 goes into the buffer of tile jt-1 once every wave has
  // passed this iteration's barrier.  Tile jt lives in stage (jt - jt0) % ST.
#pragma unroll
  for (int t = 0; t < ST - 1; ++t)
    if (jt0 + t < ntiles) issue(t, jt0 + t);
  drain_vector_loads();
  // wait for tile jt, meet the other waves, start the copy of tile jt+ST-1;
  // returns the stage of tile jt
  auto sync = [&](int jt) {
    if (jt + ST - 2 < ntiles) {
      if constexpr (ST == 2) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      else if constexpr (ST == 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DMA_TILE) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * DMA_TILE) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int stg = (jt - jt0) % ST;
    if (jt + ST - 1 < ntiles) issue((stg + ST - 1) % ST, jt + ST - 1);
    return stg;
  };
  // The tiles this wave can see are jw0 .. jw1 (wave-uniform): the ones
  // after its last query, and in a packed window the ones before its first
  // query's document start, hold only masked keys.  The wave takes part in
  // the copies and barriers of every tile of the block but computes only
  // its own range (three loops, so that no branch sits in the computing one).
  const int qw = __builtin_amdgcn_readfirstlane(q0);
  const int jw1 = min(ntiles - 1, min(qw + 31, T - 1) / 64);
  int jw0 = jt0;
  if constexpr (DOC) jw0 = min(max(jt0, __builtin_amdgcn_readfirstlane(seg[(int64_t)b * T + min(qw, T - 1)]) / 64), jw1);
  int jt = jt0;
  for (; jt < jw0; ++jt) sync(jt);
  for (; jt <= jw1; ++jt) {
    const int stg = sync(jt);
    const int kb = jt * 64;
    const bf16* Ks = sm[stg][0];
    const bf16* Vs = sm[stg][1];
    f32x16 sT[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      sT[c] = zero16();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) sT[c] = MFMA(rowfrag(Ks, 32 * c + lr, kk, lg), qf[kk], sT[c]);
    }
    // keys after the query (and past T) only occur in the diagonal and
    // ragged tiles, keys before its document start only in tiles below the
    // wave's largest start; the branch is uniform over the wave (the empty
    // asm keeps the compiler from turning it into selects on every tile).
    // Element r of block c is key kb + 32 c + 4 lg + (8 (r / 4) + r % 4).
    if ((kb + 63 > q0) || (kb + 63 >= T) || (DOC && kb < seg_hi)) {
      asm volatile("");
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int lim = min(qi, T - 1) - kb - 32 * c - 4 * lg;
        const int lo = seg_lo - kb - 32 * c - 4 * lg;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = 8 * (r >> 2) + (r & 3);
          sT[c][r] = (o > lim || (DOC && o < lo)) ? -INFINITY : sT[c][r];
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sT[c][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;  // log2 units (sl2 > 0)
    // The running maximum m moves only when some query of the wave sees a
    // score more than 2^8 above it; otherwise p = 2^(s - m) <= 256 and O, l
    // keep their scale.  The normalisation O / l is exact either way.
    if (__any(mx > m + 8.f)) {
      const float mn = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oT[dt][r] *= alpha;
    }
    float ls = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sT[c][r], sl2, -m));
        sT[c][r] = p;
        ls += p;
      }
    l += ls;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 pb = acc_frag(sT[c], s);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) oT[dt] = MFMA(colfrag(Vs, 32 * c + 16 * s, 32 * dt, lg), pb, oT[dt]);
      }
  }
  for (; jt < ntiles; ++jt) sync(jt);
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
    if (lg == 0) lse[(int64_t)bh * T + qi] = (m + __log2f(l)) * kLN2;
  }
}

// Backward, pass 1: D = rowsum(dO o O) and dQ.  Same tiling as the forward.
// For the dK/dV pass it leaves, per query, -D as a bf16 pair (neg_d_pair) in
// Dpk and the log-sum-exp in log2 units in L2buf.
template <int NW, int ST, bool DOC>
__global__ __launch_bounds__(64 * NW) void attn_bwd_dq_bf16_kernel(const bf16* __restrict__ qkv,
                                                                   const bf16* __restrict__ y,
                                                                   const bf16* __restrict__ dy,
                                                                   const float* __restrict__ lse,
                                                                   bf16* __restrict__ dqkv, uint32_t* __restrict__ Dpk,
                                                                   float* __restrict__ L2buf,
                                                                   const int32_t* __restrict__ seg,
                                                                   const float2* __restrict__ rope, int T, int H,
                                                                   int Hkv, float scale, float sl2) {
  constexpr int BQ = 32 * NW;
  constexpr int DMA_TILE = 2 * 64 * HD / 512 / NW;  // DMA instructions per wave per K/V tile
  __shared__ __attribute__((aligned(16))) bf16 sm[ST][2][64 * HD];  // [stage][K, V]
  const int nqb = (T + BQ - 1) / BQ;
  const int qb = nqb - 1 - blockIdx.y;  // longest work first, over all heads
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int C = H * HD, Ckv = Hkv * HD, C3 = C + 2 * Ckv;
  const bf16* Qg = qkv + (int64_t)b * T * C3 + h * HD;
  const bf16* Kg = qkv + (int64_t)b * T * C3 + C + (h / (H / Hkv)) * HD;
  const bf16* Vg = Kg + Ckv;
  const bf16* Og = y + (int64_t)b * T * C + h * HD;
  const bf16* dOg = dy + (int64_t)b * T * C + h * HD;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const int q0 = qb * BQ + wave * 32;
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
  const uint32_t dpair = neg_d_pair(D);
  const float lse2 = qv ? lse[(int64_t)bh * T + qi] * kLOG2E : 0.f;
  if (qv && lg == 0) {
    Dpk[(int64_t)bh * T + qi] = dpair;
    L2buf[(int64_t)bh * T + qi] = lse2;
  }
  // the extra contraction step of dP^T = V dO^T: ones on the key side, this
  // lane's query's -D pair on the query side
  const bf16x8 ones = slot01(kOnePair, lg), negd = slot01(dpair, lg);

  f32x16 dqT[2] = {zero16(), zero16()};
  const int kv_end = min(T, qb * BQ + BQ);
  const int ntiles = (kv_end + 63) / 64;
  // document mask: as in the forward
  int jt0 = 0, seg_lo = 0, seg_hi = 0;
  if constexpr (DOC) {
    const int32_t* sr = seg + (int64_t)b * T;
    jt0 = min(max(sr[qb * BQ] / 64, 0), ntiles - 1);
    seg_lo = sr[min(qi, T - 1)];
    seg_hi = sr[min(q0 + 31, T - 1)];
  }
  auto issue = [&](int st, int tile) {
    dma_rows<64, 64, NW, true>(sm[st][0], Kg, C3, tile * 64, T, 0, HD);
    dma_rows<64, 64, NW, true>(sm[st][1], Vg, C3, tile * 64, T, 0, HD);
  };
  // ST-stage ring: tiles jt+1 .. jt+ST-2 stay in flight while tile jt is
  // used; tile jt+ST-1 goes into the buffer of tile jt-1 once every wave has
  // passed this iteration's barrier.  Tile jt lives in stage (jt - jt0) % ST.
#pragma unroll
  for (int t = 0; t < ST - 1; ++t)
    if (jt0 + t < ntiles) issue(t, jt0 + t);
  drain_vector_loads();
  // wait for tile jt, meet the other waves, start the copy of tile jt+ST-1;
  // returns the stage of tile jt
  auto sync = [&](int jt) {
    if (jt + ST - 2 < ntiles) {
      if constexpr (ST == 2) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      else if constexpr (ST == 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DMA_TILE) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * DMA_TILE) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int stg = (jt - jt0) % ST;
    if (jt + ST - 1 < ntiles) issue((stg + ST - 1) % ST, jt + ST - 1);
    return stg;
  };
  // The tiles this wave can see are jw0 .. jw1 (wave-uniform): the ones
  // after its last query, and in a packed window the ones before its first
  // query's document start, hold only masked keys.  The wave takes part in
  // the copies and barriers of every tile of the block but computes only
  // its own range (three loops, so that no branch sits in the computing one).
  const int qw = __builtin_amdgcn_readfirstlane(q0);
  const int jw1 = min(ntiles - 1, min(qw + 31, T - 1) / 64);
  int jw0 = jt0;
  if constexpr (DOC) jw0 = min(max(jt0, __builtin_amdgcn_readfirstlane(seg[(int64_t)b * T + min(qw, T - 1)]) / 64), jw1);
  int jt = jt0;
  for (; jt < jw0; ++jt) sync(jt);
  for (; jt <= jw1; ++jt) {
    const int stg = sync(jt);
    const int kb = jt * 64;
    const bf16* Ks = sm[stg][0];
    const bf16* Vs = sm[stg][1];
    const bool edge = (kb + 63 > q0) || (kb + 63 >= T) || (DOC && kb < seg_hi);  // uniform over the wave
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f32x16 sT = zero16(), dpT = zero16();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        sT = MFMA(rowfrag(Ks, 32 * c + lr, kk, lg), qf[kk], sT);
        dpT = MFMA(rowfrag(Vs, 32 * c + lr, kk, lg), dof[kk], dpT);
      }
      dpT = MFMA(ones, negd, dpT);  // dP - D
      if (edge) {
        asm volatile("");
        const int lim = min(qi, T - 1) - kb - 32 * c - 4 * lg;
        const int lo = seg_lo - kb - 32 * c - 4 * lg;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = 8 * (r >> 2) + (r & 3);
          sT[r] = (o > lim || (DOC && o < lo)) ? -INFINITY : sT[r];
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sT[r] = __builtin_amdgcn_exp2f(fmaf(sT[r], sl2, -lse2)) * dpT[r];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 db = acc_frag(sT, s);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) dqT[dt] = MFMA(colfrag(Ks, 32 * c + 16 * s, 32 * dt, lg), db, dqT[dt]);
      }
    }
  }
  for (; jt < ntiles; ++jt) sync(jt);
  if (qv) store_head_grad(dqkv + ((int64_t)b * T + qi) * C3 + h * HD, dqT, scale, rope, qi, lg);
}

// Backward, pass 2: dK and dV.  Block = NW waves x 32 keys of one key/value
// head; loop over the query heads of its group and, for each, over 64-query
// tiles from the block's diagonal to T (in a packed window: to the end of the
// document of the block's last key).  Each lane owns one key (S = Q K^T).
template <int NW, bool DOC>
__global__ __launch_bounds__(64 * NW, 2) void attn_bwd_dkdv_bf16_kernel(const bf16* __restrict__ qkv,
                                                                     const bf16* __restrict__ dy,
                                                                     const float* __restrict__ L2buf,
                                                                     const uint32_t* __restrict__ Dpk,
                                                                     bf16* __restrict__ dqkv,
                                                                     const int32_t* __restrict__ seg,
                                                                     const float2* __restrict__ rope, int T, int H,
                                                                     int Hkv, float scale, float sl2) {
  constexpr int BK = 32 * NW;
  constexpr int NR = DOC ? 3 : 2;
  __shared__ __attribute__((aligned(16))) bf16 sm[2][2][64 * HD];  // [stage][Q, dO]
  // [stage][log2 lse, -D pair (u32), document start (int)]
  __shared__ __attribute__((aligned(16))) float rowst[2][NR][64];
  const int kblk = blockIdx.y;  // smallest keys (most queries) first, over all heads
  const int bj = blockIdx.x, b = bj / Hkv, j = bj % Hkv, grp = H / Hkv;
  const int C = H * HD, Ckv = Hkv * HD, C3 = C + 2 * Ckv;
  const bf16* Kg = qkv + (int64_t)b * T * C3 + C + j * HD;
  const bf16* Vg = Kg + Ckv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const int k0 = kblk * BK + wave * 32;
  const int kj = k0 + lr;
  const bool kvld = kj < T;

  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    kf[kk] = kvld ? load8(Kg + (int64_t)kj * C3 + 16 * kk + 8 * lg) : zero8();
    vf[kk] = kvld ? load8(Vg + (int64_t)kj * C3 + 16 * kk + 8 * lg) : zero8();
  }
  f32x16 dvT[2] = {zero16(), zero16()}, dkT[2] = {zero16(), zero16()};
  const int qstart = kblk * BK;
  int qend = T;
  const int32_t* sr = DOC ? seg + (int64_t)b * T : nullptr;
  if constexpr (DOC) {
    // the queries that see a key of this block are those before the first
    // document start past the block's last key (starts never decrease)
    const int kmax = min(qstart + BK - 1, T - 1);
    int lo = qstart, hi = T;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sr[mid] > kmax) hi = mid;
      else lo = mid + 1;
    }
    qend = max(lo, qstart + 1);
  }
  const int ntiles = (qend - qstart + 63) / 64;
  // Q and dO tiles of query head h, and the tile's 64 lse and -D values, by
  // DMA (those two from wave 0; rows past T read zeros, and their scores are
  // masked)
  const bool w0 = __builtin_amdgcn_readfirstlane(wave) == 0;
  const bf16x8 ones = slot01(kOnePair, lg);  // key side of the -D contraction step
  auto issue = [&](int st, int h, int tile) {
    const int q0t = qstart + tile * 64;
    const float* lseg = L2buf + ((int64_t)b * H + h) * T;
    const uint32_t* Dg = Dpk + ((int64_t)b * H + h) * T;
    dma_rows<64, 64, NW, true>(sm[st][0], qkv + (int64_t)b * T * C3 + h * HD, C3, q0t, T, 0, HD);
    dma_rows<64, 64, NW, true>(sm[st][1], dy + (int64_t)b * T * C + h * HD, C, q0t, T, 0, HD);
    if (w0) {
      const int q = q0t + lane;
      dma4_ptr(q < T ? static_cast<const void*>(lseg + q) : static_cast<const void*>(g2_zero16),
               lds_addr(&rowst[st][0][0]));
      dma4_ptr(q < T ? static_cast<const void*>(Dg + q) : static_cast<const void*>(g2_zero16),
               lds_addr(&rowst[st][1][0]));
      if constexpr (DOC)
        dma4_ptr(q < T ? static_cast<const void*>(sr + q) : static_cast<const void*>(g2_zero16),
                 lds_addr(&rowst[st][NR - 1][0]));
    }
  };
  issue(0, j * grp, 0);
  drain_vector_loads();
  // Iteration it covers query head j * grp + it / ntiles, tile it % ntiles.
  // sync: wait for this iteration's tile, meet the other waves, start the
  // copy of the next iteration's tile (head hg, tile jt now).
  const int niter = grp * ntiles;
  auto sync = [&](int it, int hg, int jt) {
    tile_barrier();
    if (it + 1 < niter) {
      if (jt + 1 < ntiles) issue((it + 1) & 1, j * grp + hg, jt + 1);
      else issue((it + 1) & 1, j * grp + hg + 1, 0);
    }
  };
  // The query tiles this wave can see start at jw0 (wave-uniform): tiles
  // that end before its first key are all masked.  The wave joins the
  // copies and barriers of every tile but computes from jw0 on (two loops
  // per head, no branch in the computing one).  (In a packed window a
  // per-wave end, found by a second search over the starts, cost more than
  // the tiles it saved.)
  const int kw = __builtin_amdgcn_readfirstlane(k0);
  const int jw0 = min(max((kw - qstart) / 64, 0), ntiles - 1);
  int it = 0;
  for (int hg = 0; hg < grp; ++hg) {
  int jt = 0;
  for (; jt < jw0; ++jt, ++it) sync(it, hg, jt);
  for (; jt < ntiles; ++jt, ++it) {
    sync(it, hg, jt);
    const int qs = qstart + jt * 64;
    const bf16* Qs = sm[it & 1][0];
    const bf16* dOs = sm[it & 1][1];
    const float* Ls = rowst[it & 1][0];
    const uint32_t* Ds = reinterpret_cast<const uint32_t*>(rowst[it & 1][1]);
    const int* Ss = reinterpret_cast<const int*>(rowst[it & 1][NR - 1]);
    // in a packed window: some query of the tile starts its document after
    // this wave's first key (the tile's last query has the largest start)
    const bool edge = (qs < k0 + 31) || (qs + 63 >= T) || (DOC && Ss[min(63, T - 1 - qs)] > k0);
    // the two 32-query halves of the tile one after the other (fewer live
    // accumulators and operand fragments)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      // no instruction moves between the halves (keeps one half's scores
      // and gradients live at a time)
      __builtin_amdgcn_sched_barrier(0);
      f32x16 sc = zero16(), dp = zero16();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        sc = MFMA(rowfrag(Qs, 32 * c + lr, kk, lg), kf[kk], sc);
        dp = MFMA(rowfrag(dOs, 32 * c + lr, kk, lg), vf[kk], dp);
      }
      dp = MFMA(slot01(Ds[32 * c + lr], lg), ones, dp);  // dP - D
      if (edge) {
        // element r is query qs + 32 c + 4 lg + (8 (r / 4) + r % 4): keep
        // lo <= 8 (r / 4) + r % 4 <= hi (query >= key, query < T)
        asm volatile("");
        const int base = qs + 32 * c + 4 * lg;
        const int lo = kj - base, hi = T - 1 - base;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = 8 * (r >> 2) + (r & 3);
          sc[r] = (o < lo || o > hi) ? -INFINITY : sc[r];
        }
        if constexpr (DOC) {
          // and queries whose document starts after this lane's key
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int4 S4 = *reinterpret_cast<const int4*>(Ss + 32 * c + 8 * a + 4 * lg);
            const int Sv[4] = {S4.x, S4.y, S4.z, S4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) sc[4 * a + e] = Sv[e] > kj ? -INFINITY : sc[4 * a + e];
          }
        }
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float4 L4 = *reinterpret_cast<const float4*>(Ls + 32 * c + 8 * a + 4 * lg);
        const float Lv[4] = {L4.x, L4.y, L4.z, L4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * a + e;
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[r], sl2, -Lv[e]));
          sc[r] = p;
          dp[r] = p * dp[r];
        }
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 pb = acc_frag(sc, s);
        const bf16x8 db = acc_frag(dp, s);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          dvT[dt] = MFMA(colfrag(dOs, 32 * c + 16 * s, 32 * dt, lg), pb, dvT[dt]);
          dkT[dt] = MFMA(colfrag(Qs, 32 * c + 16 * s, 32 * dt, lg), db, dkT[dt]);
        }
      }
    }
  }
  }
  if (kvld) {
    bf16* ok = dqkv + ((int64_t)b * T + kj) * C3 + C + j * HD;
    store_head_grad(ok, dkT, scale, rope, kj, lg);
    store_head_grad(ok + Ckv, dvT, 1.f, nullptr, kj, lg);
  }
}

// =============================================================== launchers

hipError_t launch_attention_fwd(const Launch& L, int dtype, int B, int T, int H, int Hkv, int hd, const void* qkv,
                                void* y, float* lse, const int32_t* seg) {
  const float scale = 1.f / sqrtf((float)hd);
  prof_begin(L);
  if (dtype == GPT2_PRECISION_BF16) {
    constexpr int NW = 4, ST = 2;
    dim3 grid(B * H, (T + 32 * NW - 1) / (32 * NW));
    const bf16* q = static_cast<const bf16*>(qkv);
    bf16* o = static_cast<bf16*>(y);
    if (seg)
      attn_fwd_bf16_kernel<NW, ST, true><<<grid, 64 * NW, 0, L.stream>>>(q, o, lse, seg, T, H, Hkv, scale * kLOG2E);
    else
      attn_fwd_bf16_kernel<NW, ST, false><<<grid, 64 * NW, 0, L.stream>>>(q, o, lse, nullptr, T, H, Hkv, scale * kLOG2E);
  } else {
    const int n = B * H * T;
    attn_fwd_f32_kernel<<<(n + 127) / 128, 128, 0, L.stream>>>(static_cast<const float*>(qkv), static_cast<float*>(y),
                                                              lse, seg, B, T, H, Hkv, hd, scale);
  }
  prof_end(L);
  return hipGetLastError();
}

// bf16: [-D pairs (u32) | lse in log2 units (fp32)], B * H * T each; fp32: D.
size_t attention_bwd_scratch(int B, int T, int H) { return 2 * (size_t)B * T * H * sizeof(float); }

hipError_t launch_attention_bwd(const Launch& L, int dtype, int B, int T, int H, int Hkv, int hd, const void* qkv,
                                const void* y, const void* dy, const float* lse, void* dqkv, void* scratch,
                                const int32_t* seg, const float2* rope) {
  const float scale = 1.f / sqrtf((float)hd);
  float* Dbuf = static_cast<float*>(scratch);
  prof_begin(L);
  if (dtype == GPT2_PRECISION_BF16) {
    constexpr int NW = 4;
    const int nb = (T + 32 * NW - 1) / (32 * NW);
    dim3 grid(B * H, nb), grid_kv(B * Hkv, nb);
    const bf16* q = static_cast<const bf16*>(qkv);
    const bf16* o = static_cast<const bf16*>(y);
    const bf16* dO = static_cast<const bf16*>(dy);
    bf16* dq = static_cast<bf16*>(dqkv);
    const float sl2 = scale * kLOG2E;
    uint32_t* Dpk = static_cast<uint32_t*>(scratch);
    float* L2buf = Dbuf + (size_t)B * H * T;
    if (seg) {
      attn_bwd_dq_bf16_kernel<NW, 2, true><<<grid, 64 * NW, 0, L.stream>>>(q, o, dO, lse, dq, Dpk, L2buf, seg, rope,
                                                                           T, H, Hkv, scale, sl2);
      attn_bwd_dkdv_bf16_kernel<NW, true><<<grid_kv, 64 * NW, 0, L.stream>>>(q, dO, L2buf, Dpk, dq, seg, rope, T, H,
                                                                             Hkv, scale, sl2);
    } else {
      attn_bwd_dq_bf16_kernel<NW, 2, false><<<grid, 64 * NW, 0, L.stream>>>(q, o, dO, lse, dq, Dpk, L2buf, nullptr,
                                                                            rope, T, H, Hkv, scale, sl2);
      attn_bwd_dkdv_bf16_kernel<NW, false><<<grid_kv, 64 * NW, 0, L.stream>>>(q, dO, L2buf, Dpk, dq, nullptr, rope, T,
                                                                              H, Hkv, scale, sl2);
    }
  } else {
    const int n = B * H * T;
    attn_bwd_dq_f32_kernel<<<(n + 127) / 128, 128, 0, L.stream>>>(
        static_cast<const float*>(qkv), static_cast<const float*>(y), static_cast<const float*>(dy), lse,
        static_cast<float*>(dqkv), Dbuf, seg, B, T, H, Hkv, hd, scale);
    const int nkv = B * Hkv * T;
    attn_bwd_dkdv_f32_kernel<<<(nkv + 127) / 128, 128, 0, L.stream>>>(static_cast<const float*>(qkv),
                                                                     static_cast<const float*>(dy), lse, Dbuf,
                                                                     static_cast<float*>(dqkv), seg, B, T, H, Hkv, hd,
                                                                     scale);
  }
  prof_end(L);
  return hipGetLastError();
}

}  // namespace g2
