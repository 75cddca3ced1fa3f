// Host runtime of libgpt2hip.so: configuration checks, the parameter table,
// the activation/scratch layout, the launch sequence of one micro-step and
// of the optimizer step, and the C-ABI of include/gpt2.h.
//
// The micro-step follows "How I trained my own GPT-2 124M on FineWeb-Edu":
// embedding (2.2, 2.10), n_layer pre-LN blocks x + attn(ln_1(x)),
// x + mlp(ln_2(x)) (2.3-2.13; the residual reading of the page's garbled
// Block.forward), ln_f (2.8), the tied lm_head and mean cross-entropy (4), and
// the backward pass (8.1: the gradient of loss / grad_accum_steps is added to
// the gradients).  Everything is enqueued on the context's stream.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "common.h"

namespace g2 {

// ------------------------------------------------------------- profiling

struct Prof {
  bool on = false;
  bool mark = false;  // launch site_marker_kernel before each timed launch
  std::string only;  // when non-empty, only launches from this site are timed
  std::vector<std::string> names;
  std::vector<int64_t> counts;
  std::vector<double> ms;
  struct Pending {
    int site;
    hipEvent_t a, b;
  };
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  hipEvent_t cur = nullptr;

  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  int site(const char* n) {
    for (size_t i = 0; i < names.size(); ++i)
      if (names[i] == n) return (int)i;
    names.emplace_back(n);
    counts.push_back(0);
    ms.push_back(0.0);
    return (int)names.size() - 1;
  }
  void resolve() {
    for (auto& p : pending) {
      float t = 0.f;
      if (hipEventElapsedTime(&t, p.a, p.b) == hipSuccess) {
        counts[p.site] += 1;
        ms[p.site] += t;
      }
      pool.push_back(p.a);
      pool.push_back(p.b);
    }
    pending.clear();
  }
  ~Prof() {
    for (auto& p : pending) {
      (void)hipEventDestroy(p.a);
      (void)hipEventDestroy(p.b);
    }
    for (auto e : pool) (void)hipEventDestroy(e);
  }
};

// An empty kernel: in a per-dispatch counter trace, the dispatch that follows
// it belongs to the marked launch site.
__global__ void site_marker_kernel() {}

void prof_begin(const Launch& L) {
  if (!L.prof || !L.prof->on) return;
  if (!L.prof->only.empty() && L.prof->only != L.site) return;
  if (L.prof->mark) site_marker_kernel<<<1, 64, 0, L.stream>>>();
  L.prof->cur = L.prof->get();
  if (L.prof->cur) (void)hipEventRecord(L.prof->cur, L.stream);
}
void prof_end(const Launch& L) {
  if (!L.prof || !L.prof->on || !L.prof->cur) return;
  hipEvent_t b = L.prof->get();
  if (!b) return;
  (void)hipEventRecord(b, L.stream);
  L.prof->pending.push_back({L.prof->site(L.site), L.prof->cur, b});
  L.prof->cur = nullptr;
}

}  // namespace g2

using namespace g2;

// ------------------------------------------------------------ param table

namespace {

constexpr size_t kAlignElems = 64;  // 256 B for float32 tensors
constexpr int kNormParts = 1024;
constexpr int kCeChunk = 4096;  // rows per lm_head chunk, float32 mode
// Rows per lm_head chunk in bf16 mode: the bf16 logit buffer holds one chunk
// (8192 x 50304 x 2 B = 824 MB for GPT-2), never the whole micro-batch.
#ifndef GPT2_CE_CHUNK_ROWS
#define GPT2_CE_CHUNK_ROWS 8192
#endif
constexpr int kCeChunkBf16 = GPT2_CE_CHUNK_ROWS;

struct Desc {
  std::string name;
  int ndim;
  int shape[2];
  int hf_index;  // position in the page's named_parameters order
  int decayed;
  size_t offset;
  size_t numel() const { return (size_t)shape[0] * (ndim == 2 ? (size_t)shape[1] : 1); }
};

// Kinds of per-layer tensors, for lookups.
enum Kind { LN1_W, LN1_B, QKV_W, QKV_B, PROJ_W, PROJ_B, LN2_W, LN2_B, FC_W, FC_B, MLP_W, MLP_B, N_KINDS };

struct Table {
  std::vector<Desc> d;
  size_t n_elems = 0, n_params = 0, decay_end = 0;
  int n_decayed = 0;
  int wte = -1, wpe = -1, lnf_w = -1, lnf_b = -1;
  std::vector<int> layer;  // [n_layer * N_KINDS] -> index into d
};

// key/value heads of the attention (n_kv_head, 0 meaning n_head)
int kv_heads(const gpt2_config& c) { return c.n_kv_head ? c.n_kv_head : c.n_head; }

bool check_config(const gpt2_config* c) {
  if (!c) return false;
  if (c->n_kv_head < 0 || c->n_head < 1 || c->n_head % kv_heads(*c)) return false;
  if (c->arch == GPT2_ARCH_GPT2 && kv_heads(*c) != c->n_head) return false;
  if (c->vocab_size < 1 || c->block_size < 1 || c->n_layer < 1 || c->n_head < 1 || c->n_embd < 1 ||
      c->mlp_hidden < 1 || c->max_batch < 1)
    return false;
  if (c->precision != GPT2_PRECISION_FP32 && c->precision != GPT2_PRECISION_BF16) return false;
  if (c->n_embd % c->n_head) return false;
  const int hd = c->n_embd / c->n_head;
  if (c->n_embd > 1024) return false;  // LayerNorm keeps a row in one wave's registers
  if (c->precision == GPT2_PRECISION_BF16) {
    if (hd != 64) return false;
    if (c->vocab_size % 8 || c->n_embd % 8 || c->mlp_hidden % 8) return false;
  } else {
    if (hd > 64) return false;
  }
  if ((int64_t)c->max_batch * c->block_size > (1 << 30) / 4) return false;
  // the rows one embedding backward sorts, and the 32-bit element offsets
  // of its tile pass (rows C and V C)
  if ((int64_t)c->max_batch * c->block_size > (int64_t)embed_bwd_max_rows()) return false;
  if ((int64_t)c->vocab_size * c->n_embd >= ((int64_t)1 << 31)) return false;
  if (c->arch != GPT2_ARCH_GPT2 && c->arch != GPT2_ARCH_ROTARY) return false;
  if (c->arch == GPT2_ARCH_ROTARY) {
    // bf16 kernels only: vector RMSNorm (C % 256), paired rotary / SwiGLU
    // epilogues (heads of 64, hidden width % 32)
    if (c->precision != GPT2_PRECISION_BF16 || c->n_embd % 256 || c->mlp_hidden % 32) return false;
  }
  return true;
}

Table build_table(const gpt2_config& c) {
  const int V = c.vocab_size, T = c.block_size, C = c.n_embd, F = c.mlp_hidden, L = c.n_layer;
  const int NQKV = C + 2 * kv_heads(c) * (C / c.n_head);  // q, k and v columns
  std::vector<Desc> hf;
  auto add = [&](const std::string& n, int nd, int s0, int s1) {
    Desc x;
    x.name = n;
    x.ndim = nd;
    x.shape[0] = s0;
    x.shape[1] = s1;
    x.hf_index = (int)hf.size();
    x.decayed = nd >= 2;
    x.offset = 0;
    hf.push_back(x);
  };
  const bool rotary = c.arch == GPT2_ARCH_ROTARY;
  add("transformer.wte.weight", 2, V, C);
  if (rotary) {
    for (int l = 0; l < L; ++l) {
      const std::string p = "transformer.h." + std::to_string(l) + ".";
      add(p + "ln_1.weight", 1, C, 1);
      add(p + "attn.c_attn.weight", 2, NQKV, C);
      add(p + "attn.c_proj.weight", 2, C, C);
      add(p + "ln_2.weight", 1, C, 1);
      add(p + "mlp.c_fc.weight", 2, 2 * F, C);
      add(p + "mlp.c_proj.weight", 2, C, F);
    }
    add("transformer.ln_f.weight", 1, C, 1);
  }
  if (!rotary) add("transformer.wpe.weight", 2, T, C);
  for (int l = 0; !rotary && l < L; ++l) {
    const std::string p = "transformer.h." + std::to_string(l) + ".";
    add(p + "ln_1.weight", 1, C, 1);
    add(p + "ln_1.bias", 1, C, 1);
    add(p + "attn.c_attn.weight", 2, NQKV, C);
    add(p + "attn.c_attn.bias", 1, NQKV, 1);
    add(p + "attn.c_proj.weight", 2, C, C);
    add(p + "attn.c_proj.bias", 1, C, 1);
    add(p + "ln_2.weight", 1, C, 1);
    add(p + "ln_2.bias", 1, C, 1);
    add(p + "mlp.c_fc.weight", 2, F, C);
    add(p + "mlp.c_fc.bias", 1, F, 1);
    add(p + "mlp.c_proj.weight", 2, C, F);
    add(p + "mlp.c_proj.bias", 1, C, 1);
  }
  if (!rotary) {
    add("transformer.ln_f.weight", 1, C, 1);
    add("transformer.ln_f.bias", 1, C, 1);
  }

  Table t;
  // decayed (dim >= 2) tensors first, each group in the page's order
  for (auto& x : hf)
    if (x.decayed) t.d.push_back(x);
  t.n_decayed = (int)t.d.size();
  for (auto& x : hf)
    if (!x.decayed) t.d.push_back(x);
  size_t off = 0;
  for (size_t i = 0; i < t.d.size(); ++i) {
    t.d[i].offset = off;
    off += (t.d[i].numel() + kAlignElems - 1) / kAlignElems * kAlignElems;
    t.n_params += t.d[i].numel();
    if ((int)i == t.n_decayed - 1) t.decay_end = off;
  }
  t.n_elems = off;
  t.layer.assign((size_t)L * N_KINDS, -1);
  for (size_t i = 0; i < t.d.size(); ++i) {
    const std::string& n = t.d[i].name;
    if (n == "transformer.wte.weight") t.wte = (int)i;
    else if (n == "transformer.wpe.weight") t.wpe = (int)i;
    else if (n == "transformer.ln_f.weight") t.lnf_w = (int)i;
    else if (n == "transformer.ln_f.bias") t.lnf_b = (int)i;
    else {
      int l = 0;
      char rest[64];
      if (sscanf(n.c_str(), "transformer.h.%d.%63s", &l, rest) == 2) {
        static const char* kinds[N_KINDS] = {"ln_1.weight",       "ln_1.bias",       "attn.c_attn.weight",
                                             "attn.c_attn.bias",  "attn.c_proj.weight", "attn.c_proj.bias",
                                             "ln_2.weight",       "ln_2.bias",       "mlp.c_fc.weight",
                                             "mlp.c_fc.bias",     "mlp.c_proj.weight", "mlp.c_proj.bias"};
        for (int k = 0; k < N_KINDS; ++k)
          if (strcmp(rest, kinds[k]) == 0) t.layer[(size_t)l * N_KINDS + k] = (int)i;
      }
    }
  }
  return t;
}

// ---------------------------------------------------------------- layout

struct Layout {
  int rows = 0, chunk = 0;
  size_t es = 4;  // bytes of an "activation" element (bf16 or float32)
  // activations
  std::vector<size_t> Rin, Rmid, A1, mean1, rstd1, QKV, Y, LSE, A2, mean2, rstd2, U, G;
  size_t Z = 0, meanf = 0, rstdf = 0, act_bytes = 0;
  // scratch
  size_t dR = 0, dA = 0, dQKV = 0, dY = 0, dU = 0, attnD = 0, logits = 0, dlogits = 0, rowloss = 0;
  size_t ce_stats = 0, rope = 0, seg = 0, embws = 0;
  // the norm backward's column partials, one region per norm site (0: the
  // sites add their weight gradients with atomics instead)
  size_t lnpart = 0;
  size_t count = 0, flag = 0, parts = 0, loss = 0, norm = 0, step = 0, adam_sc = 0, scratch_bytes = 0;
  // bf16: the first operands of the weight-gradient products, kept per layer
  // until the products run together at the end of the backward: dRbS[2l+1]
  // the residual gradient entering layer l's MLP branch, dRbS[2l] its
  // attention branch; dUL[l], dQKVL[l] the gradients of the fc and qkv
  // outputs; dw_table the group table of that launch
  std::vector<size_t> dRbS, dUL, dQKVL;
  // two copies of that table: [0] without K splits (fewer than 4096
  // tokens), [1] with the split tail (see run_dw)
  size_t dw_table[2] = {0, 0}, dw_table_bytes = 0;
};

struct Bump {
  size_t off = 0;
  size_t take(size_t bytes) {
    off = (off + 255) / 256 * 256;
    size_t r = off;
    off += bytes;
    return r;
  }
};

Layout build_layout(const gpt2_config& c) {
  Layout y;
  const size_t rows = (size_t)c.max_batch * c.block_size;
  const size_t C = c.n_embd, F = c.mlp_hidden, H = c.n_head, V = c.vocab_size;
  const size_t NQKV = C + 2 * (size_t)kv_heads(c) * (C / H);  // q, k and v columns
  const int L = c.n_layer;
  // U / dU: gelu'(u) [rows, F] for GPT-2; [gate | up] [rows, 2F] for the
  // rotary variant (G then holds silu(gate) up)
  const size_t FU = c.arch == GPT2_ARCH_ROTARY ? 2 * F : F;
  y.rows = (int)rows;
  y.es = c.precision == GPT2_PRECISION_BF16 ? 2 : 4;
  y.chunk = (int)std::min<size_t>(rows, kCeChunk);
  Bump a;
  for (int l = 0; l <= L; ++l) y.Rin.push_back(a.take(rows * C * 4));
  for (int l = 0; l < L; ++l) {
    y.Rmid.push_back(a.take(rows * C * 4));
    y.A1.push_back(a.take(rows * C * y.es));
    y.mean1.push_back(a.take(rows * 4));
    y.rstd1.push_back(a.take(rows * 4));
    y.QKV.push_back(a.take(rows * NQKV * y.es));
    y.Y.push_back(a.take(rows * C * y.es));
    y.LSE.push_back(a.take(rows * H * 4));
    y.A2.push_back(a.take(rows * C * y.es));
    y.mean2.push_back(a.take(rows * 4));
    y.rstd2.push_back(a.take(rows * 4));
    y.U.push_back(a.take(rows * FU * y.es));
    y.G.push_back(a.take(rows * F * y.es));
  }
  y.Z = a.take(rows * C * y.es);
  y.meanf = a.take(rows * 4);
  y.rstdf = a.take(rows * 4);
  y.act_bytes = (a.off + 255) / 256 * 256;

  Bump s;
  y.flag = s.take(256);
  y.count = s.take(256);
  y.loss = s.take(256);
  y.norm = s.take(256);
  y.step = s.take(256);     // the optimizer step counter (int64)
  y.adam_sc = s.take(256);  // clip coefficient and bias corrections of the step
  y.parts = s.take(kNormParts * 4);
  y.dR = s.take(rows * C * 4);
  y.dA = s.take(rows * C * 4);
  y.dY = s.take(rows * C * y.es);
  if (c.precision != GPT2_PRECISION_BF16) {  // bf16 mode keeps these per layer (below)
    y.dQKV = s.take(rows * NQKV * y.es);
    y.dU = s.take(rows * FU * y.es);
  }
  y.attnD = s.take(attention_bwd_scratch(1, (int)rows, H));
  y.seg = s.take(rows * 4);  // document starts of packed windows
  y.embws = s.take(embed_bwd_scratch((int)rows));  // sort of the embedding gradient
  if (ln_bwd_part_blocks((int)rows, (int)C) > 0 && 2 * L + 1 <= kLnGradSites)
    y.lnpart = s.take((size_t)(2 * L + 1) * ln_bwd_part_blocks((int)rows, (int)C) * 2 * C * 4);
  if (c.arch == GPT2_ARCH_ROTARY) y.rope = s.take((size_t)c.block_size * 32 * sizeof(float2));
  if (c.precision == GPT2_PRECISION_BF16) {
    for (int l = 0; l < 2 * L; ++l) y.dRbS.push_back(s.take(rows * C * 2));
    for (int l = 0; l < L; ++l) {
      y.dUL.push_back(s.take(rows * FU * 2));
      y.dQKVL.push_back(s.take(rows * NQKV * 2));
    }
    // the products of that launch: four per layer; a table holds at most
    // two units per output tile (every product split in two)
    int tiles = 0;
    for (int l = 0; l < L; ++l) {
      const int mn[4][2] = {{(int)C, (int)F}, {(int)FU, (int)C}, {(int)C, (int)C}, {(int)NQKV, (int)C}};
      for (int k = 0; k < 4; ++k) tiles += ((mn[k][0] + 255) / 256) * ((mn[k][1] + 255) / 256);
    }
    y.dw_table_bytes = gemm_grouped_table_bytes(4 * L, 2 * tiles);
    y.dw_table[0] = s.take(y.dw_table_bytes);
    y.dw_table[1] = s.take(y.dw_table_bytes);
  }
  if (c.precision == GPT2_PRECISION_BF16) {
    // fused lm_head + cross-entropy, one row chunk at a time: the chunk's
    // bf16 logits (then dlogits, in place) and per-tile softmax statistics
    y.chunk = (int)std::min<size_t>(rows, kCeChunkBf16);
    y.dlogits = s.take((size_t)y.chunk * V * 2);
    y.ce_stats = s.take((size_t)y.chunk * ce_stat_tiles((int)V) * sizeof(float2));
  } else {
    y.logits = s.take((size_t)y.chunk * V * 4);
    y.dlogits = s.take((size_t)y.chunk * V * y.es);
  }
  y.rowloss = s.take(rows * 4);
  y.scratch_bytes = (s.off + 255) / 256 * 256;
  return y;
}

}  // namespace

struct gpt2_ctx {
  gpt2_config cfg;
  Table tab;
  Layout lay;
  gpt2_buffers buf;
  hipStream_t stream;
  Prof prof;
  // the weight-gradient launch's two table images (see run_dw), kept for
  // the context's life: their device copies are made from them
  // asynchronously, once
  std::vector<char> dw_image[2];
  std::vector<gpt2_gemm_args> dw_sig;  // the products they describe
  int dw_units[2] = {0, 0};
  hipStream_t cap = nullptr;    // capture stream of gpt2_graph_capture
  hipGraphExec_t graph = nullptr;
  int doc_eot = -1;  // >= 0: packed windows under the document mask of this EOT id

  bool bf() const { return cfg.precision == GPT2_PRECISION_BF16; }
  Launch at(const char* site) { return Launch{stream, &prof, site}; }
  float* P(int i) const { return static_cast<float*>(buf.params) + tab.d[i].offset; }
  float* Gr(int i) const { return static_cast<float*>(buf.grads) + tab.d[i].offset; }
  // GEMM operand view of a weight: the bf16 shadow in BF16 mode, else float32.
  const void* W(int i) const {
    if (bf()) return static_cast<const bf16*>(buf.shadow) + tab.d[i].offset;
    return static_cast<const float*>(buf.params) + tab.d[i].offset;
  }
  int L(int l, int k) const { return tab.layer[(size_t)l * N_KINDS + k]; }
  template <typename T = void>
  T* act(size_t off) const { return reinterpret_cast<T*>(static_cast<char*>(buf.activations) + off); }
  template <typename T = void>
  T* scr(size_t off) const { return reinterpret_cast<T*>(static_cast<char*>(buf.scratch) + off); }
  int* flag() const { return scr<int>(lay.flag); }
  int64_t* step() const { return scr<int64_t>(lay.step); }
};

// step counter <- t (two 32-bit halves, little-endian), on the stream
static hipError_t set_step_dev(gpt2_ctx* c, int64_t t) {
  int* w = reinterpret_cast<int*>(c->step());
  hipError_t e = launch_fill_i32(c->at("fill"), w, 1, (int)(uint32_t)((uint64_t)t & 0xffffffffu));
  if (e == hipSuccess) e = launch_fill_i32(c->at("fill"), w + 1, 1, (int)(uint32_t)((uint64_t)t >> 32));
  return e;
}

// --------------------------------------------------------------- helpers

#define HIP_TRY(...)                            \
  do {                                          \
    hipError_t e__ = (__VA_ARGS__);             \
    if (e__ != hipSuccess) return GPT2_ERR_HIP; \
  } while (0)

static gpt2_gemm_args gemm_base(int dtype) {
  gpt2_gemm_args a;
  memset(&a, 0, sizeof(a));
  a.dtype = dtype;
  a.alpha = 1.f;
  return a;
}

// y[M,N] = x[M,K] W[N,K]^T (+bias) with the given epilogue: a forward Linear.
static hipError_t linear_fwd(gpt2_ctx* c, const char* site, const void* x, int M, int K, int wi, int N, int bi,
                             int epi, void* out, void* out2, const float* resid) {
  gpt2_gemm_args a = gemm_base(c->cfg.precision);
  a.M = M; a.N = N; a.K = K;
  a.a_kmajor = 1; a.b_kmajor = 1;
  a.lda = K; a.ldb = K; a.ldc = N;
  a.A = x; a.B = c->W(wi); a.C = out; a.C2 = out2; a.R = resid;
  a.bias = bi >= 0 ? c->P(bi) : nullptr;
  a.epilogue = epi;
  a.out_bf16 = c->bf() && (epi == GPT2_EPI_STORE || epi == GPT2_EPI_GELU || epi == GPT2_EPI_GELU_GRAD);
  return launch_gemm(c->at(site), a);
}

// dx[M,K] = dy[M,N] W[N,K] (a Linear's input gradient), epilogue STORE or DGELU.
static hipError_t linear_dx(gpt2_ctx* c, const char* site, const void* dy, int M, int N, int wi, int K, int epi,
                            bool out_act, void* out, const void* u) {
  gpt2_gemm_args a = gemm_base(c->cfg.precision);
  a.M = M; a.N = K; a.K = N;
  a.a_kmajor = 1; a.b_kmajor = 0;
  a.lda = N; a.ldb = K; a.ldc = K;
  a.A = dy; a.B = c->W(wi); a.C = out; a.U = u;
  a.epilogue = epi;
  a.out_bf16 = c->bf() && out_act;
  return launch_gemm(c->at(site), a);
}

// dW[N,K] += dy[M,N]^T x[M,K] (a Linear's weight gradient, reduced over
// tokens) and db[N] += sum over tokens of dy.  In bf16 mode the bias gradient
// is summed inside the product from its first operand; in float32 mode by a
// column-sum kernel over dy_f32.
static hipError_t linear_dw(gpt2_ctx* c, const char* site, const void* dy, int M, int N, const void* x, int K,
                            int wi, int bi, const float* dy_f32) {
  gpt2_gemm_args a = gemm_base(c->cfg.precision);
  a.M = N; a.N = K; a.K = M;
  a.a_kmajor = 0; a.b_kmajor = 0;
  a.lda = N; a.ldb = K; a.ldc = K;
  a.A = dy; a.B = x; a.C = c->Gr(wi);
  a.epilogue = GPT2_EPI_ACCUMULATE;
  if (c->bf()) return launch_gemm(c->at(site), a, bi >= 0 ? c->Gr(bi) : nullptr);
  hipError_t e = launch_gemm(c->at(site), a);
  if (e != hipSuccess || bi < 0) return e;
  return launch_colsum(c->at("colsum"), dy_f32, 0, M, N, N, c->Gr(bi));
}

// Weight-gradient products of the bf16 backward, queued per layer and run
// as one grouped launch once every layer's input gradients exist: with all
// layers' output tiles in one grid there are enough tiles to fill the chip
// without splitting K, so no partial sums are added atomically.
struct DwQueue {
  std::vector<gpt2_gemm_args> a;
  std::vector<float*> row_sum;
};

static void queue_dw(gpt2_ctx* c, DwQueue& q, const void* dy, int M, int N, const void* x, int K, int wi, int bi) {
  gpt2_gemm_args a = gemm_base(GPT2_PRECISION_BF16);
  a.M = N; a.N = K; a.K = M;
  a.a_kmajor = 0; a.b_kmajor = 0;
  a.lda = N; a.ldb = K; a.ldc = K;
  a.A = dy; a.B = x; a.C = c->Gr(wi);
  a.epilogue = GPT2_EPI_ACCUMULATE;
  q.a.push_back(a);
  q.row_sum.push_back(bi >= 0 ? c->Gr(bi) : nullptr);
}

// The grouped launch reads its products from a table in device memory.  All
// products reduce over the micro-step's tokens, and the kernel takes that
// count (K) as an argument, so the table depends on the token count only
// through the split plan: without splits below 4096 tokens, with the split
// tail (pieces of at least 16 K steps) from 4096 on.  Both tables are built from the first queue and copied
// once, asynchronously on the stream (their host images live as long as
// the context); later calls only check that the queue is the same.
static hipError_t run_dw(gpt2_ctx* c, DwQueue& q, int tokens) {
  const int n = (int)q.a.size();
  std::vector<gpt2_gemm_args> sig = q.a;
  for (auto& a : sig) a.K = 0;
  if (c->dw_sig.empty()) {
    // not while the stream is being captured into a graph (the copies
    // would be recorded with it): the capturing call fails instead
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(c->stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
      return hipErrorStreamCaptureUnsupported;
    for (int pl = 0; pl < 2; ++pl) {
      std::vector<gpt2_gemm_args> a = q.a;
      for (auto& x : a) x.K = pl ? (1 << 20) : 1;  // no split below 4096 tokens; the split tail above
      const int units = gemm_grouped_units(a.data(), n);
      const size_t bytes = gemm_grouped_table_bytes(n, units);
      if (units < 1 || bytes > c->lay.dw_table_bytes) return hipErrorInvalidValue;
      c->dw_image[pl].assign(bytes, 0);
      gemm_grouped_table(a.data(), q.row_sum.data(), n, units, c->dw_image[pl].data());
      c->dw_units[pl] = units;
      hipError_t e = hipMemcpyAsync(c->scr(c->lay.dw_table[pl]), c->dw_image[pl].data(), bytes,
                                    hipMemcpyHostToDevice, c->stream);
      if (e != hipSuccess) return e;
    }
    c->dw_sig = sig;
  } else {
    // the buffers behind the products never change
    auto same = [](const gpt2_gemm_args& a, const gpt2_gemm_args& b) {
      return a.A == b.A && a.B == b.B && a.C == b.C && a.M == b.M && a.N == b.N && a.lda == b.lda &&
             a.ldb == b.ldb && a.ldc == b.ldc && a.alpha == b.alpha;
    };
    if (sig.size() != c->dw_sig.size()) return hipErrorInvalidValue;
    for (size_t i = 0; i < sig.size(); ++i)
      if (!same(sig[i], c->dw_sig[i])) return hipErrorInvalidValue;
  }
  const int pl = tokens >= 4096 ? 1 : 0;
  return launch_gemm_grouped(c->at("gemm.dw"), c->scr(c->lay.dw_table[pl]), n, c->dw_units[pl], tokens);
}

// Tied lm_head + cross-entropy, bf16, one chunk of rows at a time, so the
// logits are never held for the whole batch: per chunk the statistics
// product (bf16 logit offsets + per-tile softmax statistics), the row pass
// that turns them into the row losses and the chunk's dlogits in place,
// then dZ += dlogits wte and dW += dlogits^T Z in one launch, before the
// chunk buffer is reused.  count holds the number of valid targets of all M
// rows; dZ (float32 [M, C]) must hold zeros.
static hipError_t lmhead_ce_chunked(Prof* prof, hipStream_t st, const bf16* Z, const bf16* W, const int32_t* tgt,
                                    int M, int C, int V, int ig, const int* count, float scale, float* rowloss,
                                    float* dZ, float* dW, bf16* dlog, float2* stats, int chunk) {
  for (int r0 = 0; r0 < M; r0 += chunk) {
    const int rows = std::min(chunk, M - r0);
    const bf16* Zc = Z + (size_t)r0 * C;
    hipError_t e = launch_gemm_ce_stats(Launch{st, prof, "gemm.lm_head"}, Zc, W, dlog, stats, rows, V, C);
    if (e != hipSuccess) return e;
    e = launch_ce_apply(Launch{st, prof, "ce.rows"}, dlog, stats, Zc, W, tgt + r0, rows, V, C, ig, count, scale,
                        rowloss + r0);
    if (e != hipSuccess) return e;
    gpt2_gemm_args dz = gemm_base(GPT2_PRECISION_BF16);  // dZ_c += dlogits_c wte
    dz.M = rows; dz.N = C; dz.K = V;
    dz.a_kmajor = 1; dz.b_kmajor = 0;
    dz.lda = V; dz.ldb = C; dz.ldc = C;
    dz.A = dlog; dz.B = W; dz.C = dZ + (size_t)r0 * C;
    dz.epilogue = GPT2_EPI_ACCUMULATE;
    gpt2_gemm_args dw = gemm_base(GPT2_PRECISION_BF16);  // dW += dlogits_c^T Z_c
    dw.M = V; dw.N = C; dw.K = rows;
    dw.a_kmajor = 0; dw.b_kmajor = 0;
    dw.lda = V; dw.ldb = C; dw.ldc = C;
    dw.A = dlog; dw.B = Zc; dw.C = dW;
    dw.epilogue = GPT2_EPI_ACCUMULATE;
    e = launch_gemm_pair(Launch{st, prof, "gemm.lm_head_bwd"}, dz, dw);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static hipError_t lmhead_ce_bf16(gpt2_ctx* c, const int32_t* tgt, int M, const int* count, float scale,
                                 float* rowloss, float* dZ) {
  const Layout& y = c->lay;
  return lmhead_ce_chunked(&c->prof, c->stream, c->act<bf16>(y.Z), static_cast<const bf16*>(c->W(c->tab.wte)), tgt,
                           M, c->cfg.n_embd, c->cfg.vocab_size, -1, count, scale, rowloss, dZ, c->Gr(c->tab.wte),
                           c->scr<bf16>(y.dlogits), c->scr<float2>(y.ce_stats), y.chunk);
}

// ------------------------------------------------------------- the step

static int fwd_bwd_impl(gpt2_ctx* c, const int32_t* tok, const int32_t* tgt, int B, int T, float scale, float* loss,
                        float* token_loss) {
  const gpt2_config& g = c->cfg;
  const Layout& y = c->lay;
  const int M = B * T, C = g.n_embd, F = g.mlp_hidden, V = g.vocab_size, H = g.n_head, hd = C / H;
  const int dt = g.precision;
  const bool bf = c->bf();
  int* flag = c->flag();
  int* count = c->scr<int>(y.count);
  float* rowloss = token_loss ? token_loss : c->scr<float>(y.rowloss);

  HIP_TRY(launch_count_targets(c->at("ce.count"), tgt, M, V, -1, count, flag));
  const int32_t* seg = nullptr;
  if (c->doc_eot >= 0) {
    seg = c->scr<int32_t>(y.seg);
    HIP_TRY(launch_segment_starts(c->at("embed.seg"), tok, B, T, c->doc_eot, c->scr<int32_t>(y.seg)));
  }
  HIP_TRY(launch_embed_fwd(c->at("embed.fwd"), tok, c->P(c->tab.wte), c->P(c->tab.wpe), c->act<float>(y.Rin[0]), B,
                           T, C, V, flag, seg));
  // ---- forward
  for (int l = 0; l < g.n_layer; ++l) {
    float* rin = c->act<float>(y.Rin[l]);
    float* rmid = c->act<float>(y.Rmid[l]);
    HIP_TRY(launch_layernorm_fwd(c->at("ln.fwd"), rin, c->P(c->L(l, LN1_W)), c->P(c->L(l, LN1_B)), c->act(y.A1[l]),
                                 bf, c->act<float>(y.mean1[l]), c->act<float>(y.rstd1[l]), M, C));
    HIP_TRY(linear_fwd(c, "gemm.qkv", c->act(y.A1[l]), M, C, c->L(l, QKV_W), 3 * C, c->L(l, QKV_B), GPT2_EPI_STORE,
                       c->act(y.QKV[l]), nullptr, nullptr));
    HIP_TRY(launch_attention_fwd(c->at("attn.fwd"), dt, B, T, H, H, hd, c->act(y.QKV[l]), c->act(y.Y[l]),
                                 c->act<float>(y.LSE[l]), seg));
    HIP_TRY(linear_fwd(c, "gemm.attn_proj", c->act(y.Y[l]), M, C, c->L(l, PROJ_W), C, c->L(l, PROJ_B),
                       GPT2_EPI_RESIDUAL, rmid, nullptr, rin));
    HIP_TRY(launch_layernorm_fwd(c->at("ln.fwd"), rmid, c->P(c->L(l, LN2_W)), c->P(c->L(l, LN2_B)), c->act(y.A2[l]),
                                 bf, c->act<float>(y.mean2[l]), c->act<float>(y.rstd2[l]), M, C));
    // G = gelu(u) for the next product, U = gelu'(u) for the backward
    HIP_TRY(linear_fwd(c, "gemm.fc", c->act(y.A2[l]), M, C, c->L(l, FC_W), F, c->L(l, FC_B), GPT2_EPI_GELU_GRAD,
                       c->act(y.G[l]), c->act(y.U[l]), nullptr));
    HIP_TRY(linear_fwd(c, "gemm.mlp_proj", c->act(y.G[l]), M, F, c->L(l, MLP_W), C, c->L(l, MLP_B),
                       GPT2_EPI_RESIDUAL, c->act<float>(y.Rin[l + 1]), nullptr, rmid));
  }
  float* rlast = c->act<float>(y.Rin[g.n_layer]);
  HIP_TRY(launch_layernorm_fwd(c->at("ln.fwd"), rlast, c->P(c->tab.lnf_w), c->P(c->tab.lnf_b), c->act(y.Z), bf,
                               c->act<float>(y.meanf), c->act<float>(y.rstdf), M, C));

  // ---- tied lm_head + cross-entropy
  float* dZ = c->scr<float>(y.dA);
  HIP_TRY(launch_fill_f32(c->at("fill"), dZ, (size_t)M * C, 0.f));
  const size_t es = y.es;
  DwQueue q;  // bf16: weight-gradient products, run together after the backward
  if (bf) HIP_TRY(lmhead_ce_bf16(c, tgt, M, count, scale, rowloss, dZ));
  for (int r0 = 0; !bf && r0 < M; r0 += y.chunk) {
    const int rows = std::min(y.chunk, M - r0);
    const char* z_c = c->act<char>(y.Z) + (size_t)r0 * C * es;
    float* logits = c->scr<float>(y.logits);
    void* dlog = c->scr(y.dlogits);
    {
      gpt2_gemm_args a = gemm_base(dt);
      a.M = rows; a.N = V; a.K = C;
      a.a_kmajor = 1; a.b_kmajor = 1;
      a.lda = C; a.ldb = C; a.ldc = V;
      a.A = z_c; a.B = c->W(c->tab.wte); a.C = logits;
      a.epilogue = GPT2_EPI_STORE; a.out_bf16 = 0;
      HIP_TRY(launch_gemm(c->at("gemm.lm_head"), a));
    }
    HIP_TRY(launch_ce_rows<float, float>(c->at("ce.rows"), logits, V, static_cast<float*>(dlog), V, tgt + r0, rows, V,
                                         count, scale, nullptr, rowloss + r0));
    {  // dZ_c += dlogits_c wte
      gpt2_gemm_args a = gemm_base(dt);
      a.M = rows; a.N = C; a.K = V;
      a.a_kmajor = 1; a.b_kmajor = 0;
      a.lda = V; a.ldb = C; a.ldc = C;
      a.A = dlog; a.B = c->W(c->tab.wte); a.C = dZ + (size_t)r0 * C;
      a.epilogue = GPT2_EPI_ACCUMULATE;
      HIP_TRY(launch_gemm(c->at("gemm.lm_head_dx"), a));
    }
    {  // dwte += dlogits_c^T Z_c
      gpt2_gemm_args a = gemm_base(dt);
      a.M = V; a.N = C; a.K = rows;
      a.a_kmajor = 0; a.b_kmajor = 0;
      a.lda = V; a.ldb = C; a.ldc = C;
      a.A = dlog; a.B = z_c; a.C = c->Gr(c->tab.wte);
      a.epilogue = GPT2_EPI_ACCUMULATE;
      HIP_TRY(launch_gemm(c->at("gemm.lm_head_dw"), a));
    }
  }
  HIP_TRY(launch_ce_finish_n(c->at("ce.finish"), rowloss, M, count, loss, flag));

  // ---- backward through the blocks
  float* dR = c->scr<float>(y.dR);
  // bf16 copies of the residual gradient, one slot per (layer, branch) (the
  // weight-gradient products read them after the loop); float32 mode reads
  // dR itself
  auto dRb_slot = [&](int s) -> bf16* { return bf && s >= 0 ? c->scr<bf16>(y.dRbS[s]) : nullptr; };
  // gradient of an LN output: bf16 in BF16 mode (the products' output type,
  // as under autocast), float32 otherwise; dZ (float32) lives here first and
  // the final LN backward consumes it before the buffer is reused
  void* dA = c->scr(y.dA);
  // dW += dy^T x (+ bias row sums): queued in bf16 mode, run now in float32
  auto dw = [&](const char* site, const void* dy, int N, const void* x, int K, int wi, int bi,
                const float* dy_f32) -> hipError_t {
    if (bf) {
      queue_dw(c, q, dy, M, N, x, K, wi, bi);
      return hipSuccess;
    }
    return linear_dw(c, site, dy, M, N, x, K, wi, bi, dy_f32);
  };
  // the norm sites' weight gradients: each backward leaves its blocks'
  // column partials (site 2L: the final norm, 2l + 1 / 2l: layer l's second
  // / first), summed in block order after the loop, so they do not depend on
  // scheduling (no partial buffer: atomics)
  const int lnb = y.lnpart ? ln_bwd_part_blocks(M, C) : 0;
  LnGradSites lns{};
  auto lnp = [&](int site, float* dw, float* db) -> float* {
    if (!lnb) return nullptr;
    lns.dw[site] = dw;
    lns.db[site] = db;
    return c->scr<float>(y.lnpart) + (size_t)site * lnb * 2 * C;
  };
  // the final norm's backward writes dR (its first value) rather than adding to it
  HIP_TRY(launch_layernorm_bwd_b(c->at("ln.bwd"), dZ, 0, rlast, c->act<float>(y.meanf), c->act<float>(y.rstdf),
                                 c->P(c->tab.lnf_w), dR, dRb_slot(2 * g.n_layer - 1), c->Gr(c->tab.lnf_w),
                                 c->Gr(c->tab.lnf_b), M, C,
                                 lnp(2 * g.n_layer, c->Gr(c->tab.lnf_w), c->Gr(c->tab.lnf_b)), 0));
  void* dY = c->scr(y.dY);
  for (int l = g.n_layer - 1; l >= 0; --l) {
    const void* dRm = bf ? static_cast<const void*>(dRb_slot(2 * l + 1)) : static_cast<const void*>(dR);
    const void* dRa = bf ? static_cast<const void*>(dRb_slot(2 * l)) : static_cast<const void*>(dR);
    void* dU = c->scr(bf ? y.dUL[l] : y.dU);
    void* dQKV = c->scr(bf ? y.dQKVL[l] : y.dQKV);
    // MLP branch: R_{l+1} = Rmid + G Wmp^T + b
    HIP_TRY(dw("gemm.mlp_proj_dw", dRm, C, c->act(y.G[l]), F, c->L(l, MLP_W), c->L(l, MLP_B), dR));
    // dU = (dR W_mp) * gelu'(u), gelu'(u) kept by the forward
    HIP_TRY(linear_dx(c, "gemm.mlp_proj_dx", dRm, M, C, c->L(l, MLP_W), F, GPT2_EPI_MUL, true, dU, c->act(y.U[l])));
    HIP_TRY(dw("gemm.fc_dw", dU, F, c->act(y.A2[l]), C, c->L(l, FC_W), c->L(l, FC_B), static_cast<const float*>(dU)));
    HIP_TRY(linear_dx(c, "gemm.fc_dx", dU, M, F, c->L(l, FC_W), C, GPT2_EPI_STORE, true, dA, nullptr));
    HIP_TRY(launch_layernorm_bwd_b(c->at("ln.bwd"), dA, bf, c->act<float>(y.Rmid[l]), c->act<float>(y.mean2[l]),
                                   c->act<float>(y.rstd2[l]), c->P(c->L(l, LN2_W)), dR, dRb_slot(2 * l),
                                   c->Gr(c->L(l, LN2_W)), c->Gr(c->L(l, LN2_B)), M, C,
                                   lnp(2 * l + 1, c->Gr(c->L(l, LN2_W)), c->Gr(c->L(l, LN2_B)))));
    // attention branch: Rmid = R_l + Y Wo^T + b
    HIP_TRY(dw("gemm.attn_proj_dw", dRa, C, c->act(y.Y[l]), C, c->L(l, PROJ_W), c->L(l, PROJ_B), dR));
    HIP_TRY(linear_dx(c, "gemm.attn_proj_dx", dRa, M, C, c->L(l, PROJ_W), C, GPT2_EPI_STORE, true, dY, nullptr));
    HIP_TRY(launch_attention_bwd(c->at("attn.bwd"), dt, B, T, H, H, hd, c->act(y.QKV[l]), c->act(y.Y[l]), dY,
                                 c->act<float>(y.LSE[l]), dQKV, c->scr(y.attnD), seg, nullptr));
    HIP_TRY(dw("gemm.qkv_dw", dQKV, 3 * C, c->act(y.A1[l]), C, c->L(l, QKV_W), c->L(l, QKV_B),
               static_cast<const float*>(dQKV)));
    HIP_TRY(linear_dx(c, "gemm.qkv_dx", dQKV, M, 3 * C, c->L(l, QKV_W), C, GPT2_EPI_STORE, true, dA, nullptr));
    HIP_TRY(launch_layernorm_bwd_b(c->at("ln.bwd"), dA, bf, c->act<float>(y.Rin[l]), c->act<float>(y.mean1[l]),
                                   c->act<float>(y.rstd1[l]), c->P(c->L(l, LN1_W)), dR, dRb_slot(2 * l - 1),
                                   c->Gr(c->L(l, LN1_W)), c->Gr(c->L(l, LN1_B)), M, C,
                                   lnp(2 * l, c->Gr(c->L(l, LN1_W)), c->Gr(c->L(l, LN1_B)))));
  }
  if (lnb) HIP_TRY(launch_ln_param_grad(c->at("ln.bwd"), c->scr<float>(y.lnpart), M, C, lns, 2 * g.n_layer + 1));
  if (bf) HIP_TRY(run_dw(c, q, M));
  // (dA, free after the last block, holds the scatter's partial sums)
  HIP_TRY(launch_embed_bwd(c->at("embed.bwd"), tok, dR, c->Gr(c->tab.wte), c->Gr(c->tab.wpe), B, T, C, V, seg,
                           static_cast<float*>(dA), c->scr(y.embws)));
  return GPT2_OK;
}

// The rotary variant ("Reproduce GPT-2 124M 复盘": RMSNorm, rotary q/k,
// SwiGLU, no position table, no biases), bf16.
static int fwd_bwd_rotary(gpt2_ctx* c, const int32_t* tok, const int32_t* tgt, int B, int T, float scale, float* loss,
                          float* token_loss) {
  const gpt2_config& g = c->cfg;
  const Layout& y = c->lay;
  const int M = B * T, C = g.n_embd, F = g.mlp_hidden, V = g.vocab_size, H = g.n_head, hd = C / H;
  const int Hkv = kv_heads(g), Ckv = Hkv * hd, NQKV = C + 2 * Ckv;  // grouped-query attention when Hkv < H
  const int dt = g.precision;
  int* flag = c->flag();
  int* count = c->scr<int>(y.count);
  float* rowloss = token_loss ? token_loss : c->scr<float>(y.rowloss);
  float2* rope = c->scr<float2>(y.rope);

  HIP_TRY(launch_rope_table(c->at("rope.table"), rope, T, 10000.0));
  HIP_TRY(launch_count_targets(c->at("ce.count"), tgt, M, V, -1, count, flag));
  // packed windows: the mask only.  q and k keep the rotation of position t
  // (not of t's place in its document): a rotation by t - start of both
  // differs from one by t by the same angle for every pair of tokens of a
  // document, and the mask hides every other pair, so the scores are those
  // of restarted positions
  const int32_t* seg = nullptr;
  if (c->doc_eot >= 0) {
    seg = c->scr<int32_t>(y.seg);
    HIP_TRY(launch_segment_starts(c->at("embed.seg"), tok, B, T, c->doc_eot, c->scr<int32_t>(y.seg)));
  }
  HIP_TRY(launch_embed_fwd(c->at("embed.fwd"), tok, c->P(c->tab.wte), nullptr, c->act<float>(y.Rin[0]), B, T, C, V,
                           flag, seg));
  for (int l = 0; l < g.n_layer; ++l) {
    float* rin = c->act<float>(y.Rin[l]);
    float* rmid = c->act<float>(y.Rmid[l]);
    HIP_TRY(launch_rmsnorm_fwd(c->at("norm.fwd"), rin, c->P(c->L(l, LN1_W)), c->act<bf16>(y.A1[l]),
                               c->act<float>(y.rstd1[l]), M, C));
    {  // qkv = a1 Wqkv^T, q and k rotated in the epilogue
      gpt2_gemm_args a = gemm_base(dt);
      a.M = M; a.N = NQKV; a.K = C;
      a.a_kmajor = 1; a.b_kmajor = 1;
      a.lda = C; a.ldb = C; a.ldc = NQKV;
      a.A = c->act(y.A1[l]); a.B = c->W(c->L(l, QKV_W)); a.C = c->act(y.QKV[l]);
      a.epilogue = GPT2_EPI_ROPE; a.out_bf16 = 1;
      a.rope = rope; a.rope_period = T; a.rope_cols = C + Ckv;
      HIP_TRY(launch_gemm(c->at("gemm.qkv"), a));
    }
    HIP_TRY(launch_attention_fwd(c->at("attn.fwd"), dt, B, T, H, Hkv, hd, c->act(y.QKV[l]), c->act(y.Y[l]),
                                 c->act<float>(y.LSE[l]), seg));
    HIP_TRY(linear_fwd(c, "gemm.attn_proj", c->act(y.Y[l]), M, C, c->L(l, PROJ_W), C, -1, GPT2_EPI_RESIDUAL, rmid,
                       nullptr, rin));
    HIP_TRY(launch_rmsnorm_fwd(c->at("norm.fwd"), rmid, c->P(c->L(l, LN2_W)), c->act<bf16>(y.A2[l]),
                               c->act<float>(y.rstd2[l]), M, C));
    {  // act = silu(a2 Wg^T) (a2 Wu^T); gate | up kept for the backward
      gpt2_gemm_args a = gemm_base(dt);
      a.M = M; a.N = 2 * F; a.K = C;
      a.a_kmajor = 1; a.b_kmajor = 1;
      a.lda = C; a.ldb = C; a.ldc = F; a.ld2 = 2 * F;
      a.A = c->act(y.A2[l]); a.B = c->W(c->L(l, FC_W)); a.C = c->act(y.G[l]); a.C2 = c->act(y.U[l]);
      a.epilogue = GPT2_EPI_SWIGLU; a.out_bf16 = 1;
      HIP_TRY(launch_gemm(c->at("gemm.fc"), a));
    }
    HIP_TRY(linear_fwd(c, "gemm.mlp_proj", c->act(y.G[l]), M, F, c->L(l, MLP_W), C, -1, GPT2_EPI_RESIDUAL,
                       c->act<float>(y.Rin[l + 1]), nullptr, rmid));
  }
  float* rlast = c->act<float>(y.Rin[g.n_layer]);
  HIP_TRY(launch_rmsnorm_fwd(c->at("norm.fwd"), rlast, c->P(c->tab.lnf_w), c->act<bf16>(y.Z),
                             c->act<float>(y.rstdf), M, C));

  float* dZ = c->scr<float>(y.dA);
  HIP_TRY(launch_fill_f32(c->at("fill"), dZ, (size_t)M * C, 0.f));
  DwQueue q;  // weight-gradient products, run together after the backward
  HIP_TRY(lmhead_ce_bf16(c, tgt, M, count, scale, rowloss, dZ));
  HIP_TRY(launch_ce_finish_n(c->at("ce.finish"), rowloss, M, count, loss, flag));

  // ---- backward
  float* dR = c->scr<float>(y.dR);
  // bf16 copies of the residual gradient, one slot per (layer, branch), and
  // per-layer fc / qkv output gradients: the weight-gradient products read
  // them in one grouped launch after the loop
  auto dRb_slot = [&](int s) -> bf16* { return s >= 0 ? c->scr<bf16>(y.dRbS[s]) : nullptr; };
  void* dA = c->scr(y.dA);  // dZ (float32) first, then bf16 norm-output gradients
  void* dY = c->scr(y.dY);
  // the norm sites' weight gradients: each backward leaves its blocks'
  // column partials (site 2L: the final norm, 2l + 1 / 2l: layer l's second
  // / first), summed in block order after the loop, so they do not depend on
  // scheduling (no partial buffer: atomics)
  const int lnb = y.lnpart ? ln_bwd_part_blocks(M, C) : 0;
  LnGradSites lns{};
  auto lnp = [&](int site, float* dw, float* db) -> float* {
    if (!lnb) return nullptr;
    lns.dw[site] = dw;
    lns.db[site] = db;
    return c->scr<float>(y.lnpart) + (size_t)site * lnb * 2 * C;
  };
  // the final norm's backward writes dR (its first value) rather than adding to it
  HIP_TRY(launch_rmsnorm_bwd(c->at("norm.bwd"), dZ, 0, rlast, c->act<float>(y.rstdf), c->P(c->tab.lnf_w), dR,
                             dRb_slot(2 * g.n_layer - 1), c->Gr(c->tab.lnf_w), M, C,
                             lnp(2 * g.n_layer, c->Gr(c->tab.lnf_w), nullptr), 0));
  for (int l = g.n_layer - 1; l >= 0; --l) {
    bf16* dRm = dRb_slot(2 * l + 1);
    bf16* dRa = dRb_slot(2 * l);
    void* dGU = c->scr(y.dUL[l]);
    bf16* dQKV = c->scr<bf16>(y.dQKVL[l]);
    // feed-forward: R_{l+1} = Rmid + act Wd^T
    queue_dw(c, q, dRm, M, C, c->act(y.G[l]), F, c->L(l, MLP_W), -1);
    {  // d(act) = dR Wd; dgate, dup through the SwiGLU gate
      gpt2_gemm_args a = gemm_base(dt);
      a.M = M; a.N = F; a.K = C;
      a.a_kmajor = 1; a.b_kmajor = 0;
      a.lda = C; a.ldb = F; a.ldc = 2 * F; a.ld2 = 2 * F;
      a.A = dRm; a.B = c->W(c->L(l, MLP_W)); a.C = dGU; a.U = c->act(y.U[l]);
      a.epilogue = GPT2_EPI_SWIGLU_BWD; a.out_bf16 = 1;
      HIP_TRY(launch_gemm(c->at("gemm.mlp_proj_dx"), a));
    }
    queue_dw(c, q, dGU, M, 2 * F, c->act(y.A2[l]), C, c->L(l, FC_W), -1);
    HIP_TRY(linear_dx(c, "gemm.fc_dx", dGU, M, 2 * F, c->L(l, FC_W), C, GPT2_EPI_STORE, true, dA, nullptr));
    HIP_TRY(launch_rmsnorm_bwd(c->at("norm.bwd"), dA, 1, c->act<float>(y.Rmid[l]), c->act<float>(y.rstd2[l]),
                               c->P(c->L(l, LN2_W)), dR, dRa, c->Gr(c->L(l, LN2_W)), M, C,
                               lnp(2 * l + 1, c->Gr(c->L(l, LN2_W)), nullptr)));
    // attention: Rmid = R_l + Y Wo^T
    queue_dw(c, q, dRa, M, C, c->act(y.Y[l]), C, c->L(l, PROJ_W), -1);
    HIP_TRY(linear_dx(c, "gemm.attn_proj_dx", dRa, M, C, c->L(l, PROJ_W), C, GPT2_EPI_STORE, true, dY, nullptr));
    HIP_TRY(launch_attention_bwd(c->at("attn.bwd"), dt, B, T, H, Hkv, hd, c->act(y.QKV[l]), c->act(y.Y[l]), dY,
                                 c->act<float>(y.LSE[l]), dQKV, c->scr(y.attnD), seg, rope));
    queue_dw(c, q, dQKV, M, NQKV, c->act(y.A1[l]), C, c->L(l, QKV_W), -1);
    HIP_TRY(linear_dx(c, "gemm.qkv_dx", dQKV, M, NQKV, c->L(l, QKV_W), C, GPT2_EPI_STORE, true, dA, nullptr));
    HIP_TRY(launch_rmsnorm_bwd(c->at("norm.bwd"), dA, 1, c->act<float>(y.Rin[l]), c->act<float>(y.rstd1[l]),
                               c->P(c->L(l, LN1_W)), dR, dRb_slot(2 * l - 1), c->Gr(c->L(l, LN1_W)), M, C,
                               lnp(2 * l, c->Gr(c->L(l, LN1_W)), nullptr)));
  }
  if (lnb) HIP_TRY(launch_ln_param_grad(c->at("norm.bwd"), c->scr<float>(y.lnpart), M, C, lns, 2 * g.n_layer + 1));
  HIP_TRY(run_dw(c, q, M));
  HIP_TRY(launch_embed_bwd(c->at("embed.bwd"), tok, dR, c->Gr(c->tab.wte), nullptr, B, T, C, V, seg,
                           static_cast<float*>(dA), c->scr(y.embws)));
  return GPT2_OK;
}

// ================================================================== C-ABI

extern "C" {

double gpt2_lr_at(int64_t step, double max_lr, double min_lr, int64_t warmup, int64_t max_steps) {
  if (warmup < 1 || max_steps <= warmup || step < 0) return NAN;
  if (step < warmup) return max_lr * (double)(step + 1) / (double)warmup;
  if (step > max_steps) return min_lr;
  const double r = (double)(step - warmup) / (double)(max_steps - warmup);
  return min_lr + (max_lr - min_lr) * 0.5 * (1.0 + cos(M_PI * r));
}

int gpt2_query_sizes(const gpt2_config* cfg, gpt2_sizes* out) {
  if (!cfg || !out) return GPT2_ERR_ARG;
  if (!check_config(cfg)) return GPT2_ERR_SHAPE;
  Table t = build_table(*cfg);
  Layout y = build_layout(*cfg);
  out->n_params = t.n_params;
  out->n_elems = t.n_elems;
  out->n_tensors = (int32_t)t.d.size();
  out->n_decayed = t.n_decayed;
  out->params_bytes = t.n_elems * 4;
  out->grads_bytes = t.n_elems * 4;
  out->adam_m_bytes = t.n_elems * 4;
  out->adam_v_bytes = t.n_elems * 4;
  out->shadow_bytes = cfg->precision == GPT2_PRECISION_BF16 ? t.n_elems * 2 : 0;
  out->activations_bytes = y.act_bytes;
  out->scratch_bytes = y.scratch_bytes;
  return GPT2_OK;
}

int gpt2_param_info(const gpt2_config* cfg, int idx, gpt2_param_desc* out) {
  if (!cfg || !out) return GPT2_ERR_ARG;
  if (!check_config(cfg)) return GPT2_ERR_SHAPE;
  Table t = build_table(*cfg);
  if (idx < 0 || idx >= (int)t.d.size()) return GPT2_ERR_ARG;
  const Desc& d = t.d[idx];
  memset(out, 0, sizeof(*out));
  snprintf(out->name, sizeof(out->name), "%s", d.name.c_str());
  out->offset = d.offset;
  out->ndim = d.ndim;
  out->shape[0] = d.shape[0];
  out->shape[1] = d.ndim == 2 ? d.shape[1] : 0;
  out->decayed = d.decayed;
  return GPT2_OK;
}

int gpt2_create(const gpt2_config* cfg, const gpt2_buffers* bufs, void* stream, gpt2_ctx** out) {
  if (!cfg || !bufs || !out) return GPT2_ERR_ARG;
  if (!check_config(cfg)) return GPT2_ERR_SHAPE;
  if (!bufs->params || !bufs->grads || !bufs->adam_m || !bufs->adam_v || !bufs->activations || !bufs->scratch)
    return GPT2_ERR_UNBOUND;
  if (cfg->precision == GPT2_PRECISION_BF16 && !bufs->shadow) return GPT2_ERR_UNBOUND;
  gpt2_ctx* c = new gpt2_ctx();
  c->cfg = *cfg;
  c->tab = build_table(*cfg);
  c->lay = build_layout(*cfg);
  c->buf = *bufs;
  c->stream = static_cast<hipStream_t>(stream);
  if (launch_fill_i32(c->at("fill"), c->flag(), 1, GPT2_OK) != hipSuccess || set_step_dev(c, 0) != hipSuccess) {
    delete c;
    return GPT2_ERR_HIP;
  }
  *out = c;
  return GPT2_OK;
}

int gpt2_destroy(gpt2_ctx* c) {
  if (!c) return GPT2_ERR_ARG;
  (void)hipStreamSynchronize(c->stream);
  if (c->graph) (void)hipGraphExecDestroy(c->graph);
  if (c->cap) (void)hipStreamDestroy(c->cap);
  delete c;
  return GPT2_OK;
}

int gpt2_set_stream(gpt2_ctx* c, void* stream) {
  if (!c) return GPT2_ERR_ARG;
  c->stream = static_cast<hipStream_t>(stream);
  return GPT2_OK;
}

int gpt2_set_doc_mask(gpt2_ctx* c, int eot) {
  if (!c) return GPT2_ERR_ARG;
  if (eot < -1 || eot >= c->cfg.vocab_size) return GPT2_ERR_ARG;
  if (eot != c->doc_eot && c->graph) {  // a captured micro-step keeps the mask it was captured with
    (void)hipStreamSynchronize(c->stream);
    (void)hipGraphExecDestroy(c->graph);
    c->graph = nullptr;
  }
  c->doc_eot = eot;
  return GPT2_OK;
}

int gpt2_sync_shadow(gpt2_ctx* c) {
  if (!c) return GPT2_ERR_ARG;
  if (!c->bf()) return GPT2_OK;
  HIP_TRY(launch_to_bf16(c->at("shadow"), static_cast<const float*>(c->buf.params), static_cast<bf16*>(c->buf.shadow),
                         c->tab.n_elems));
  return GPT2_OK;
}

int gpt2_init_params(gpt2_ctx* c, uint64_t seed) {
  if (!c) return GPT2_ERR_ARG;
  const size_t n = c->tab.n_elems;
  HIP_TRY(launch_fill_f32(c->at("fill"), static_cast<float*>(c->buf.params), n, 0.f));
  const double resid_std = 0.02 / sqrt(2.0 * c->cfg.n_layer);
  for (size_t i = 0; i < c->tab.d.size(); ++i) {
    const Desc& d = c->tab.d[i];
    float* p = c->P((int)i);
    if (d.ndim == 2) {
      const bool resid = d.name.size() > 13 && d.name.compare(d.name.size() - 13, 13, "c_proj.weight") == 0;
      HIP_TRY(launch_init_normal(c->at("init"), p, d.numel(), (uint32_t)d.hf_index, seed,
                                 (float)(resid ? resid_std : 0.02)));
    } else {
      const bool ln_w = d.name.find("ln_") != std::string::npos && d.name.compare(d.name.size() - 6, 6, "weight") == 0;
      HIP_TRY(launch_fill_f32(c->at("fill"), p, d.numel(), ln_w ? 1.f : 0.f));
    }
  }
  HIP_TRY(launch_fill_f32(c->at("fill"), static_cast<float*>(c->buf.grads), n, 0.f));
  HIP_TRY(launch_fill_f32(c->at("fill"), static_cast<float*>(c->buf.adam_m), n, 0.f));
  HIP_TRY(launch_fill_f32(c->at("fill"), static_cast<float*>(c->buf.adam_v), n, 0.f));
  HIP_TRY(set_step_dev(c, 0));
  return gpt2_sync_shadow(c);
}

int gpt2_zero_grad(gpt2_ctx* c) {
  if (!c) return GPT2_ERR_ARG;
  HIP_TRY(launch_fill_f32(c->at("zero_grad"), static_cast<float*>(c->buf.grads), c->tab.n_elems, 0.f));
  return GPT2_OK;
}

int gpt2_fwd_bwd(gpt2_ctx* c, const int32_t* d_tokens, const int32_t* d_targets, int B, int T, float loss_scale,
                 float* d_loss, float* d_token_loss) {
  if (!c || !d_tokens || !d_targets || !d_loss) return GPT2_ERR_ARG;
  if (B < 1 || B > c->cfg.max_batch || T < 1 || T > c->cfg.block_size) return GPT2_ERR_SHAPE;
  if (!isfinite(loss_scale)) return GPT2_ERR_ARG;
  if (c->cfg.arch == GPT2_ARCH_ROTARY)
    return fwd_bwd_rotary(c, d_tokens, d_targets, B, T, loss_scale, d_loss, d_token_loss);
  return fwd_bwd_impl(c, d_tokens, d_targets, B, T, loss_scale, d_loss, d_token_loss);
}

int gpt2_graph_capture(gpt2_ctx* c, const int32_t* d_tokens, const int32_t* d_targets, int B, int T,
                       float loss_scale, float* d_loss) {
  if (!c || !d_tokens || !d_targets || !d_loss) return GPT2_ERR_ARG;
  if (B < 1 || B > c->cfg.max_batch || T < 1 || T > c->cfg.block_size) return GPT2_ERR_SHAPE;
  if (!isfinite(loss_scale) || c->prof.on) return GPT2_ERR_ARG;
  if (!c->cap) HIP_TRY(hipStreamCreateWithFlags(&c->cap, hipStreamNonBlocking));
  // the capture stream starts after everything issued so far
  HIP_TRY(hipStreamSynchronize(c->stream));
  const hipStream_t user = c->stream;
  c->stream = c->cap;
  hipGraph_t g = nullptr;
  int rc = GPT2_ERR_HIP;
  if (hipStreamBeginCapture(c->cap, hipStreamCaptureModeThreadLocal) == hipSuccess) {
    rc = gpt2_fwd_bwd(c, d_tokens, d_targets, B, T, loss_scale, d_loss, nullptr);
    if (hipStreamEndCapture(c->cap, &g) != hipSuccess) rc = GPT2_ERR_HIP;
  }
  c->stream = user;
  if (rc != GPT2_OK) {
    if (g) (void)hipGraphDestroy(g);
    return rc;
  }
  hipGraphExec_t exec = nullptr;
  const hipError_t e = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (e != hipSuccess) return GPT2_ERR_HIP;
  if (c->graph) (void)hipGraphExecDestroy(c->graph);
  c->graph = exec;
  return GPT2_OK;
}

int gpt2_graph_launch(gpt2_ctx* c) {
  if (!c) return GPT2_ERR_ARG;
  if (!c->graph) return GPT2_ERR_UNBOUND;
  HIP_TRY(hipGraphLaunch(c->graph, c->stream));
  return GPT2_OK;
}

int gpt2_clip_adamw_step(gpt2_ctx* c, const gpt2_adamw* hp, float* d_grad_norm) {
  if (!c || !hp) return GPT2_ERR_ARG;
  if (!(hp->lr >= 0.f) || !(hp->beta1 >= 0.f && hp->beta1 < 1.f) || !(hp->beta2 >= 0.f && hp->beta2 < 1.f) ||
      !(hp->eps > 0.f) || !(hp->max_norm > 0.f) || !isfinite(hp->weight_decay))
    return GPT2_ERR_ARG;
  const Layout& y = c->lay;
  float* parts = c->scr<float>(y.parts);
  float* norm = d_grad_norm ? d_grad_norm : c->scr<float>(y.norm);
  HIP_TRY(launch_sumsq_partials(c->at("opt.sumsq"), static_cast<const float*>(c->buf.grads), c->tab.n_elems, parts,
                                kNormParts));
  HIP_TRY(launch_adamw(c->at("opt.adamw"), c->at("opt.prep"), static_cast<float*>(c->buf.params),
                       static_cast<const float*>(c->buf.grads), static_cast<float*>(c->buf.adam_m),
                       static_cast<float*>(c->buf.adam_v), c->bf() ? static_cast<bf16*>(c->buf.shadow) : nullptr,
                       c->tab.n_elems, c->tab.decay_end, parts, kNormParts, hp->lr, hp->beta1, hp->beta2, hp->eps,
                       hp->weight_decay, hp->max_norm, c->step(), c->scr<float>(y.adam_sc), norm, c->flag()));
  return GPT2_OK;
}

int gpt2_get_step(gpt2_ctx* c, int64_t* t) {
  if (!c || !t) return GPT2_ERR_ARG;
  if (hipStreamSynchronize(c->stream) != hipSuccess) return GPT2_ERR_HIP;
  if (hipMemcpy(t, c->step(), sizeof(int64_t), hipMemcpyDeviceToHost) != hipSuccess) return GPT2_ERR_HIP;
  return GPT2_OK;
}

int gpt2_set_step(gpt2_ctx* c, int64_t t) {
  if (!c || t < 0) return GPT2_ERR_ARG;
  HIP_TRY(set_step_dev(c, t));
  return GPT2_OK;
}

int gpt2_get_status(gpt2_ctx* c) {
  if (!c) return GPT2_ERR_ARG;
  if (hipStreamSynchronize(c->stream) != hipSuccess) return GPT2_ERR_HIP;
  int f = 0;
  if (hipMemcpy(&f, c->flag(), sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return GPT2_ERR_HIP;
  c->prof.resolve();
  if (f != GPT2_OK) {
    if (launch_fill_i32(c->at("fill"), c->flag(), 1, GPT2_OK) != hipSuccess) return GPT2_ERR_HIP;
    if (hipStreamSynchronize(c->stream) != hipSuccess) return GPT2_ERR_HIP;
    c->prof.resolve();
  }
  return f;
}

const char* gpt2_strerror(int s) {
  switch (s) {
    case GPT2_OK: return "ok";
    case GPT2_WARN_NO_TARGETS: return "no valid target in the micro-batch (loss is NaN, no gradient added)";
    case GPT2_ERR_ARG: return "invalid argument";
    case GPT2_ERR_SHAPE: return "unsupported shape or configuration";
    case GPT2_ERR_HIP: return "HIP runtime error";
    case GPT2_ERR_UNBOUND: return "required buffer not bound";
    case GPT2_ERR_BAD_ID: return "token or target id out of range";
    case GPT2_ERR_NONFINITE: return "non-finite gradient norm: update skipped";
    default: return "unknown status";
  }
}

// ---------------------------------------------------- isolated lm_head + CE

// scratch of gpt2_lmhead_ce: count, row losses, one chunk's bf16 logits and
// tile statistics, dHidden in float32
static size_t lmhead_scratch(int M, int C, int V, size_t* off) {
  const int chunk = std::min(M, kCeChunkBf16);
  Bump s;
  off[0] = s.take(256);                                               // count
  off[1] = s.take((size_t)M * 4);                                     // row losses
  off[2] = s.take((size_t)chunk * V * 2);                             // a chunk's logits, then dlogits
  off[3] = s.take((size_t)chunk * ce_stat_tiles(V) * sizeof(float2));  // its per-tile softmax statistics
  off[4] = s.take((size_t)M * C * 4);                                 // dhidden (float32 accumulation)
  return (s.off + 255) / 256 * 256;
}

size_t gpt2_lmhead_ce_scratch_bytes(int M, int C, int V) {
  if (M < 1 || C < 1 || V < 1) return 0;
  size_t off[5];
  return lmhead_scratch(M, C, V, off);
}

int gpt2_lmhead_ce(void* stream, const void* d_hidden, const void* d_weight, const int32_t* d_targets, int M, int C,
                   int V, int ignore_index, float* d_loss, void* d_dhidden, float* d_dweight, void* d_scratch,
                   int32_t* d_flag) {
  if (!d_hidden || !d_weight || !d_targets || !d_loss || !d_dhidden || !d_dweight || !d_scratch) return GPT2_ERR_ARG;
  if (M < 1 || C < 8 || V < 8 || C % 8 || V % 8) return GPT2_ERR_SHAPE;
  if (((uintptr_t)d_hidden | (uintptr_t)d_weight | (uintptr_t)d_dhidden | (uintptr_t)d_dweight |
       (uintptr_t)d_scratch) & 15)
    return GPT2_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Launch L{st, nullptr, ""};
  size_t off[5];
  lmhead_scratch(M, C, V, off);
  char* base = static_cast<char*>(d_scratch);
  int* count = reinterpret_cast<int*>(base + off[0]);
  float* rowloss = reinterpret_cast<float*>(base + off[1]);
  bf16* dlog = reinterpret_cast<bf16*>(base + off[2]);
  float2* stats = reinterpret_cast<float2*>(base + off[3]);
  float* dh32 = reinterpret_cast<float*>(base + off[4]);
  int* flag = reinterpret_cast<int*>(d_flag);
  HIP_TRY(launch_count_targets(L, d_targets, M, V, ignore_index, count, flag));
  HIP_TRY(launch_fill_f32(L, dh32, (size_t)M * C, 0.f));
  HIP_TRY(lmhead_ce_chunked(nullptr, st, static_cast<const bf16*>(d_hidden), static_cast<const bf16*>(d_weight),
                            d_targets, M, C, V, ignore_index, count, 1.f, rowloss, dh32, d_dweight, dlog, stats,
                            std::min(M, kCeChunkBf16)));
  HIP_TRY(launch_ce_finish_n(L, rowloss, M, count, d_loss, flag));
  HIP_TRY(launch_to_bf16(L, dh32, static_cast<bf16*>(d_dhidden), (size_t)M * C));
  return GPT2_OK;
}

// ------------------------------------------------------------ single ops

static bool gemm_args_ok(const gpt2_gemm_args* a) {
  if (!a || !a->A || !a->B || !a->C) return false;
  if (a->M < 1 || a->N < 1 || a->K < 1) return false;
  if (a->dtype != GPT2_PRECISION_BF16 && a->dtype != GPT2_PRECISION_FP32) return false;
  if (a->epilogue < GPT2_EPI_STORE || a->epilogue > GPT2_EPI_SWIGLU_BWD) return false;
  const bool rotary_family = a->epilogue >= GPT2_EPI_ROPE;
  if (rotary_family) {
    if (a->dtype != GPT2_PRECISION_BF16 || !a->out_bf16) return false;
    if (a->epilogue == GPT2_EPI_ROPE) {
      if (!a->a_kmajor || !a->b_kmajor || a->N % 64 || a->rope_cols % 64 || a->rope_cols < 0 ||
          (a->rope_cols > 0 && (!a->rope || a->rope_period < 1)))
        return false;
      if ((uintptr_t)a->rope & 15) return false;
    } else if (a->epilogue == GPT2_EPI_SWIGLU) {
      if (!a->a_kmajor || !a->b_kmajor || a->N % 64 || a->K % 64 || !a->C2 || a->bias) return false;
      if (a->ld2 < a->N || a->ld2 % 8 || a->ldc < a->N / 2) return false;
      if ((int64_t)a->N * a->ldb * 2 >= ((int64_t)1 << 32)) return false;  // 32-bit row offsets of B
    } else {  // SWIGLU_BWD
      if (!a->a_kmajor || a->b_kmajor || a->N % 8 || !a->U || a->bias) return false;
      if (a->ld2 < 2 * (int64_t)a->N || a->ld2 % 8 || a->ldc < 2 * (int64_t)a->N) return false;
    }
  }
  if (a->epilogue == GPT2_EPI_GELU_GRAD && !a->C2) return false;
  if (a->epilogue == GPT2_EPI_MUL && !a->U) return false;
  if (a->epilogue == GPT2_EPI_RESIDUAL && !a->R) return false;
  if (a->epilogue == GPT2_EPI_GELU && !a->C2) return false;
  if (a->epilogue == GPT2_EPI_DGELU && !a->U) return false;
  if (a->epilogue == GPT2_EPI_ACCUMULATE && a->bias) return false;
  const int64_t need_a = a->a_kmajor ? a->K : a->M;
  const int64_t need_b = a->b_kmajor ? a->K : a->N;
  const int64_t need_c = a->epilogue == GPT2_EPI_SWIGLU ? a->N / 2 : (a->epilogue == GPT2_EPI_SWIGLU_BWD ? 2 * (int64_t)a->N : a->N);
  if (a->lda < need_a || a->ldb < need_b || a->ldc < need_c) return false;
  if (a->dtype == GPT2_PRECISION_BF16) {
    if (a->M % 8 && !a->a_kmajor) return false;
    if (a->N % 8 && !a->b_kmajor) return false;
    if ((a->a_kmajor && a->K % 8) || (a->b_kmajor && a->K % 8)) return false;
    if (a->lda % 8 || a->ldb % 8 || a->ldc % 8) return false;
    if (((uintptr_t)a->A | (uintptr_t)a->B | (uintptr_t)a->C | (uintptr_t)a->C2 | (uintptr_t)a->R |
         (uintptr_t)a->U | (uintptr_t)a->bias) & 15)
      return false;
    // the output dtype each epilogue writes in bf16 mode
    const bool bf_out = a->epilogue == GPT2_EPI_GELU || a->epilogue == GPT2_EPI_DGELU ||
                        a->epilogue == GPT2_EPI_GELU_GRAD || a->epilogue == GPT2_EPI_MUL || rotary_family;
    const bool f32_out = a->epilogue == GPT2_EPI_RESIDUAL || a->epilogue == GPT2_EPI_ACCUMULATE;
    if ((bf_out && !a->out_bf16) || (f32_out && a->out_bf16)) return false;
  }
  return true;
}

int gpt2_op_gemm(void* stream, const gpt2_gemm_args* a) {
  if (!gemm_args_ok(a)) return GPT2_ERR_ARG;
  HIP_TRY(launch_gemm(Launch{static_cast<hipStream_t>(stream), nullptr, ""}, *a));
  return GPT2_OK;
}

static bool grouped_args_ok(const gpt2_gemm_args* a, int n) {
  if (!a || n < 1) return false;
  for (int i = 0; i < n; ++i) {
    if (!gemm_args_ok(a + i)) return false;
    if (a[i].dtype != GPT2_PRECISION_BF16 || a[i].a_kmajor || a[i].b_kmajor ||
        a[i].epilogue != GPT2_EPI_ACCUMULATE)
      return false;
  }
  return gemm_grouped_units(a, n) > 0;
}

size_t gpt2_gemm_grouped_workspace_bytes(const gpt2_gemm_args* args, int n) {
  if (!grouped_args_ok(args, n)) return 0;
  return gemm_grouped_table_bytes(n, gemm_grouped_units(args, n));
}

int gpt2_op_gemm_grouped(void* stream, const gpt2_gemm_args* args, int n, float* const* d_row_sums,
                         void* d_workspace) {
  if (!grouped_args_ok(args, n) || !d_workspace || ((uintptr_t)d_workspace & 15)) return GPT2_ERR_ARG;
  if (d_row_sums)
    for (int i = 0; i < n; ++i)
      if ((uintptr_t)d_row_sums[i] & 3) return GPT2_ERR_ARG;
  const int units = gemm_grouped_units(args, n);
  std::vector<char> host(gemm_grouped_table_bytes(n, units));
  gemm_grouped_table(args, d_row_sums, n, units, host.data());
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIP_TRY(hipMemcpyAsync(d_workspace, host.data(), host.size(), hipMemcpyHostToDevice, s));
  HIP_TRY(hipStreamSynchronize(s));
  HIP_TRY(launch_gemm_grouped(Launch{s, nullptr, ""}, d_workspace, n, units));
  return GPT2_OK;
}

int gpt2_op_colsum(void* stream, const void* d_y, int y_bf16, int M, int N, int64_t ld, float* d_db) {
  if (!d_y || !d_db || M < 1 || N < 1 || ld < N) return GPT2_ERR_ARG;
  HIP_TRY(launch_colsum(Launch{static_cast<hipStream_t>(stream), nullptr, ""}, d_y, y_bf16, M, N, ld, d_db));
  return GPT2_OK;
}

int gpt2_op_layernorm_fwd(void* stream, const float* d_x, const float* d_w, const float* d_b, void* d_y, int y_bf16,
                          float* d_mean, float* d_rstd, int rows, int C) {
  if (!d_x || !d_w || !d_b || !d_y || !d_mean || !d_rstd) return GPT2_ERR_ARG;
  if (rows < 1 || C < 1 || C > 1024) return GPT2_ERR_SHAPE;
  if (y_bf16 && C % 256 == 0 && (((uintptr_t)d_x | (uintptr_t)d_w | (uintptr_t)d_b | (uintptr_t)d_y) & 15))
    return GPT2_ERR_ARG;
  HIP_TRY(launch_layernorm_fwd(Launch{static_cast<hipStream_t>(stream), nullptr, ""}, d_x, d_w, d_b, d_y, y_bf16,
                               d_mean, d_rstd, rows, C));
  return GPT2_OK;
}

int gpt2_op_layernorm_bwd(void* stream, const void* d_dy, int dy_bf16, const float* d_x, const float* d_mean,
                          const float* d_rstd, const float* d_w, float* d_dx, void* d_dx_bf16, float* d_dw, float* d_db,
                          int rows, int C) {
  if (!d_dy || !d_x || !d_mean || !d_rstd || !d_w || !d_dx || !d_dw || !d_db) return GPT2_ERR_ARG;
  if (rows < 1 || C < 1 || C > 1024) return GPT2_ERR_SHAPE;
  // the vector kernels (C a multiple of 256) move 16 bytes per lane
  if (C % 256 == 0 && (((uintptr_t)d_dy | (uintptr_t)d_x | (uintptr_t)d_w | (uintptr_t)d_dx |
                        (uintptr_t)d_dx_bf16 | (uintptr_t)d_dw | (uintptr_t)d_db) & 15))
    return GPT2_ERR_ARG;
  HIP_TRY(launch_layernorm_bwd_b(Launch{static_cast<hipStream_t>(stream), nullptr, ""}, d_dy, dy_bf16 != 0, d_x,
                                 d_mean, d_rstd, d_w, d_dx, static_cast<bf16*>(d_dx_bf16), d_dw, d_db, rows, C));
  return GPT2_OK;
}

int gpt2_op_rmsnorm_fwd(void* stream, const float* d_x, const float* d_w, void* d_y, float* d_rstd, int rows, int C) {
  if (!d_x || !d_w || !d_y || !d_rstd) return GPT2_ERR_ARG;
  if (rows < 1 || C < 256 || C > 1024 || C % 256) return GPT2_ERR_SHAPE;
  if (((uintptr_t)d_x | (uintptr_t)d_w | (uintptr_t)d_y) & 15) return GPT2_ERR_ARG;
  HIP_TRY(launch_rmsnorm_fwd(Launch{static_cast<hipStream_t>(stream), nullptr, ""}, d_x, d_w, static_cast<bf16*>(d_y),
                             d_rstd, rows, C));
  return GPT2_OK;
}

int gpt2_op_rmsnorm_bwd(void* stream, const void* d_dy, int dy_bf16, const float* d_x, const float* d_rstd,
                        const float* d_w, float* d_dx, void* d_dx_bf16, float* d_dw, int rows, int C) {
  if (!d_dy || !d_x || !d_rstd || !d_w || !d_dx || !d_dw) return GPT2_ERR_ARG;
  if (rows < 1 || C < 256 || C > 1024 || C % 256) return GPT2_ERR_SHAPE;
  if (((uintptr_t)d_dy | (uintptr_t)d_x | (uintptr_t)d_w | (uintptr_t)d_dx | (uintptr_t)d_dx_bf16 |
       (uintptr_t)d_dw) & 15)
    return GPT2_ERR_ARG;
  HIP_TRY(launch_rmsnorm_bwd(Launch{static_cast<hipStream_t>(stream), nullptr, ""}, d_dy, dy_bf16 != 0, d_x, d_rstd,
                             d_w, d_dx, static_cast<bf16*>(d_dx_bf16), d_dw, rows, C));
  return GPT2_OK;
}

int gpt2_op_rope_table(void* stream, int T, double base, float* d_table) {
  if (!d_table || !(base > 0.0)) return GPT2_ERR_ARG;
  if (T < 1) return GPT2_ERR_SHAPE;
  HIP_TRY(launch_rope_table(Launch{static_cast<hipStream_t>(stream), nullptr, ""}, reinterpret_cast<float2*>(d_table),
                            T, base));
  return GPT2_OK;
}

int gpt2_op_rope_bwd(void* stream, void* d_dqkv, int rows, int64_t ld, int cols, int T, const float* d_table) {
  if (!d_dqkv || !d_table) return GPT2_ERR_ARG;
  if (rows < 1 || T < 1 || cols < 64 || cols % 64 || ld < cols || ld % 4) return GPT2_ERR_SHAPE;
  if (((uintptr_t)d_dqkv & 7) || ((uintptr_t)d_table & 7)) return GPT2_ERR_ARG;
  HIP_TRY(launch_rope_bwd(Launch{static_cast<hipStream_t>(stream), nullptr, ""}, static_cast<bf16*>(d_dqkv), rows, ld,
                          cols, T, reinterpret_cast<const float2*>(d_table)));
  return GPT2_OK;
}

static bool attn_shape_ok(int dtype, int B, int T, int H, int Hkv, int hd) {
  if (B < 1 || T < 1 || H < 1 || Hkv < 1 || H % Hkv) return false;
  if (dtype == GPT2_PRECISION_BF16) return hd == 64;
  if (dtype == GPT2_PRECISION_FP32) return hd >= 1 && hd <= 64;
  return false;
}

int gpt2_op_attention_fwd(void* stream, int dtype, int B, int T, int H, int Hkv, int hd, const void* d_qkv,
                          void* d_y, float* d_lse, const int32_t* d_seg) {
  if (!d_qkv || !d_y || !d_lse) return GPT2_ERR_ARG;
  if (!attn_shape_ok(dtype, B, T, H, Hkv, hd)) return GPT2_ERR_SHAPE;
  HIP_TRY(launch_attention_fwd(Launch{static_cast<hipStream_t>(stream), nullptr, ""}, dtype, B, T, H, Hkv, hd, d_qkv,
                               d_y, d_lse, d_seg));
  return GPT2_OK;
}

size_t gpt2_attention_bwd_scratch_bytes(int B, int T, int H) { return attention_bwd_scratch(B, T, H); }

int gpt2_op_attention_bwd(void* stream, int dtype, int B, int T, int H, int Hkv, int hd, const void* d_qkv,
                          const void* d_y, const void* d_dy, const float* d_lse, void* d_dqkv, void* d_scratch,
                          const int32_t* d_seg, const float* d_rope) {
  if (!d_qkv || !d_y || !d_dy || !d_lse || !d_dqkv || !d_scratch) return GPT2_ERR_ARG;
  if (!attn_shape_ok(dtype, B, T, H, Hkv, hd)) return GPT2_ERR_SHAPE;
  if (d_rope && (dtype != GPT2_PRECISION_BF16 || ((uintptr_t)d_rope & 15))) return GPT2_ERR_ARG;
  HIP_TRY(launch_attention_bwd(Launch{static_cast<hipStream_t>(stream), nullptr, ""}, dtype, B, T, H, Hkv, hd, d_qkv,
                               d_y, d_dy, d_lse, d_dqkv, d_scratch, d_seg, reinterpret_cast<const float2*>(d_rope)));
  return GPT2_OK;
}

size_t gpt2_embedding_bwd_scratch_bytes(int rows, int C) {
  if (rows < 1 || C < 1) return 0;
  return ((size_t)rows * C * 4 + 255) / 256 * 256 + embed_bwd_scratch(rows);
}

int gpt2_op_embedding_bwd(void* stream, const int32_t* d_tokens, const float* d_dres, float* d_dwte, float* d_dwpe,
                          int B, int T, int C, int V, const int32_t* d_seg, void* d_scratch) {
  if (!d_tokens || !d_dres || !d_dwte || !d_scratch) return GPT2_ERR_ARG;
  if (B < 1 || T < 1 || C < 1 || V < 1) return GPT2_ERR_SHAPE;
  const int64_t rows = (int64_t)B * T;
  if (rows > embed_bwd_max_rows() || rows * C >= ((int64_t)1 << 31) || (int64_t)V * C >= ((int64_t)1 << 31))
    return GPT2_ERR_SHAPE;
  if ((uintptr_t)d_scratch & 255) return GPT2_ERR_ARG;
  float* part = static_cast<float*>(d_scratch);
  void* ws = static_cast<char*>(d_scratch) + ((size_t)rows * C * 4 + 255) / 256 * 256;
  HIP_TRY(launch_embed_bwd(Launch{static_cast<hipStream_t>(stream), nullptr, ""}, d_tokens, d_dres, d_dwte, d_dwpe, B,
                           T, C, V, d_seg, part, ws));
  return GPT2_OK;
}

int gpt2_op_segment_starts(void* stream, const int32_t* d_tokens, int B, int T, int eot, int32_t* d_seg) {
  if (!d_tokens || !d_seg) return GPT2_ERR_ARG;
  if (B < 1 || T < 1) return GPT2_ERR_SHAPE;
  HIP_TRY(launch_segment_starts(Launch{static_cast<hipStream_t>(stream), nullptr, ""}, d_tokens, B, T, eot, d_seg));
  return GPT2_OK;
}

// ------------------------------------------------------------ profiling

int gpt2_profile_enable(gpt2_ctx* c, int on) {
  if (!c) return GPT2_ERR_ARG;
  c->prof.on = on != 0;
  return GPT2_OK;
}

int gpt2_profile_only(gpt2_ctx* c, const char* site) {
  if (!c) return GPT2_ERR_ARG;
  c->prof.only = site ? site : "";
  return GPT2_OK;
}

int gpt2_profile_mark(gpt2_ctx* c, int on) {
  if (!c) return GPT2_ERR_ARG;
  c->prof.mark = on != 0;
  return GPT2_OK;
}

int gpt2_op_marker(void* stream) {
  site_marker_kernel<<<1, 64, 0, static_cast<hipStream_t>(stream)>>>();
  return hipGetLastError() == hipSuccess ? GPT2_OK : GPT2_ERR_HIP;
}

int gpt2_profile_reset(gpt2_ctx* c) {
  if (!c) return GPT2_ERR_ARG;
  (void)hipStreamSynchronize(c->stream);
  c->prof.resolve();
  std::fill(c->prof.counts.begin(), c->prof.counts.end(), 0);
  std::fill(c->prof.ms.begin(), c->prof.ms.end(), 0.0);
  return GPT2_OK;
}

int gpt2_profile_count(gpt2_ctx* c) {
  if (!c) return GPT2_ERR_ARG;
  return (int)c->prof.names.size();
}

int gpt2_profile_entry(gpt2_ctx* c, int i, const char** name, int64_t* launches, double* total_ms) {
  if (!c || i < 0 || i >= (int)c->prof.names.size()) return GPT2_ERR_ARG;
  if (name) *name = c->prof.names[i].c_str();
  if (launches) *launches = c->prof.counts[i];
  if (total_ms) *total_ms = c->prof.ms[i];
  return GPT2_OK;
}

}  // extern "C"
