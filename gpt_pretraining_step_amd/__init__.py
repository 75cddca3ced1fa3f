"""One GPT-2 training micro-step and optimizer step on an MI355X (gfx950).

A thin Python layer over libgpt2hip.so (include/gpt2.h).  PyTorch provides the
device buffers and the stream; every step of the computation runs in the
library's HIP kernels.  The calls mirror the training loop of "How I trained
my own GPT-2 124M on FineWeb-Edu" (sections 8.1 and 9):

    m = GPT2(GPT2_124M)                      # buffers sized for B <= max_batch
    m.init_params(seed=42)
    m.zero_grad()
    for k in range(grad_accum_steps):
        m.fwd_bwd(x_k, y_k, loss_scale=1 / grad_accum_steps)
    norm = m.clip_adamw_step(lr=6e-4)
"""

from __future__ import annotations

import ctypes as ct
from dataclasses import dataclass

from . import _ffi
from ._ffi import (GPT2Error, check, lib, PRECISION_BF16, PRECISION_FP32,  # noqa: F401
                   EPI_STORE, EPI_RESIDUAL, EPI_GELU, EPI_DGELU, EPI_ACCUMULATE, EPI_GELU_GRAD, EPI_MUL,
                   EPI_ROPE, EPI_SWIGLU, EPI_SWIGLU_BWD, ARCH_GPT2, ARCH_ROTARY, GPT2_ERR_ARG)

__all__ = ["ModelConfig", "GPT2", "TINY_CHAR_FP32", "GPT2_124M", "GPT2Error", "lmhead_ce", "op_gemm", "op_gemm_grouped",
           "op_attention_fwd", "op_attention_bwd", "op_attention_bwd_noalloc", "op_embedding_bwd", "op_segment_starts", "op_layernorm_fwd", "op_layernorm_bwd", "op_colsum", "op_marker",
           "op_rope_table", "op_rope_bwd", "op_rmsnorm_fwd", "op_rmsnorm_bwd", "query_sizes", "param_table",
           "GPT2_ROTARY_124M"]


@dataclass(frozen=True)
class ModelConfig:
    vocab_size: int
    block_size: int
    n_layer: int
    n_head: int
    n_embd: int
    mlp_hidden: int
    max_batch: int
    precision: int  # PRECISION_FP32 or PRECISION_BF16
    arch: int = ARCH_GPT2  # ARCH_GPT2 or ARCH_ROTARY
    n_kv_head: int = 0  # key/value heads (grouped-query attention, rotary variant); 0: n_head

    def c(self) -> _ffi.Config:
        return _ffi.Config(self.vocab_size, self.block_size, self.n_layer, self.n_head, self.n_embd,
                           self.mlp_hidden, self.max_batch, self.precision, self.arch, self.n_kv_head)


# The tiny character-level GPT in float32 (vocab 66, 2 layers, 64 wide, 4 heads, MLP 256, T 64, B 4).
TINY_CHAR_FP32 = ModelConfig(66, 64, 2, 4, 64, 256, 4, PRECISION_FP32)
# GPT-2 124M with the padded vocabulary, bf16 compute with float32 master weights, micro-batch 16.
GPT2_124M = ModelConfig(50304, 1024, 12, 12, 768, 3072, 16, PRECISION_BF16)
# The rotary variant ("Reproduce GPT-2 124M": RMSNorm, RoPE, SwiGLU 2048, no
# position table, no biases), bf16, micro-batch 64.
GPT2_ROTARY_124M = ModelConfig(50304, 1024, 12, 12, 768, 2048, 64, PRECISION_BF16, ARCH_ROTARY)


def query_sizes(cfg: ModelConfig) -> _ffi.Sizes:
    s = _ffi.Sizes()
    c = cfg.c()
    check(lib().gpt2_query_sizes(ct.byref(c), ct.byref(s)), "gpt2_query_sizes")
    return s


def param_table(cfg: ModelConfig):
    """[(name, offset, shape, decayed)] in table order (host only)."""
    s = query_sizes(cfg)
    c = cfg.c()
    out = []
    for i in range(s.n_tensors):
        d = _ffi.ParamDesc()
        check(lib().gpt2_param_info(ct.byref(c), i, ct.byref(d)), "gpt2_param_info")
        shape = (d.shape[0], d.shape[1]) if d.ndim == 2 else (d.shape[0],)
        out.append((d.name.decode(), int(d.offset), shape, bool(d.decayed)))
    return out


def _stream_ptr(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


class GPT2:
    """A model instance: caller-owned (torch) device buffers bound to a
    library context."""

    def __init__(self, cfg: ModelConfig, device: str = "cuda", stream=None):
        import torch
        self.cfg = cfg
        self.device = torch.device(device)
        self.sizes = query_sizes(cfg)
        s = self.sizes
        n = s.n_elems

        def buf(nbytes, dtype=torch.uint8):
            return torch.zeros(max(nbytes, 1), dtype=dtype, device=self.device)

        self.params = torch.zeros(n, dtype=torch.float32, device=self.device)
        self.grads = torch.zeros(n, dtype=torch.float32, device=self.device)
        self.adam_m = torch.zeros(n, dtype=torch.float32, device=self.device)
        self.adam_v = torch.zeros(n, dtype=torch.float32, device=self.device)
        self.shadow = torch.zeros(n, dtype=torch.bfloat16, device=self.device) if s.shadow_bytes else None
        self.activations = buf(s.activations_bytes)
        self.scratch = buf(s.scratch_bytes)
        self.loss = torch.zeros(1, dtype=torch.float32, device=self.device)
        self.grad_norm = torch.zeros(1, dtype=torch.float32, device=self.device)
        b = _ffi.Buffers(self.params.data_ptr(), self.grads.data_ptr(), self.adam_m.data_ptr(),
                         self.adam_v.data_ptr(), _ptr(self.shadow), self.activations.data_ptr(),
                         self.scratch.data_ptr())
        c = cfg.c()
        h = ct.c_void_p()
        torch.cuda.synchronize(self.device)
        check(lib().gpt2_create(ct.byref(c), ct.byref(b), _stream_ptr(stream), ct.byref(h)), "gpt2_create")
        self._h = h
        self.table = param_table(cfg)
        self.index = {name: (off, shape, dec) for name, off, shape, dec in self.table}

    # -- parameter views ---------------------------------------------------
    def view(self, flat, name: str):
        off, shape, _ = self.index[name]
        n = 1
        for d in shape:
            n *= d
        return flat[off:off + n].view(*shape)

    def param(self, name):
        return self.view(self.params, name)

    def grad(self, name):
        return self.view(self.grads, name)

    # -- the training step ---------------------------------------------------
    def init_params(self, seed: int = 42):
        check(lib().gpt2_init_params(self._h, seed), "gpt2_init_params")

    def sync_shadow(self):
        check(lib().gpt2_sync_shadow(self._h), "gpt2_sync_shadow")

    def set_doc_mask(self, eot):
        """Packed windows under the document mask of ``eot`` (None: plain
        causal rows)."""
        check(lib().gpt2_set_doc_mask(self._h, -1 if eot is None else int(eot)), "gpt2_set_doc_mask")

    def zero_grad(self):
        check(lib().gpt2_zero_grad(self._h), "gpt2_zero_grad")

    def fwd_bwd(self, tokens, targets, loss_scale: float = 1.0, token_loss=None, loss_out=None):
        """tokens, targets: int32 device tensors [B, T].  Returns the device
        loss tensor (unscaled micro-batch mean)."""
        import torch
        assert tokens.dtype == torch.int32 and targets.dtype == torch.int32
        assert tokens.is_contiguous() and targets.is_contiguous() and tokens.shape == targets.shape
        B, T = tokens.shape
        out = self.loss if loss_out is None else loss_out
        check(lib().gpt2_fwd_bwd(self._h, tokens.data_ptr(), targets.data_ptr(), B, T, float(loss_scale),
                                 out.data_ptr(), _ptr(token_loss)), "gpt2_fwd_bwd")
        return out

    def graph_capture(self, tokens, targets, loss_scale: float = 1.0, loss_out=None):
        """Capture one micro-step over these token / target buffers into a HIP
        graph (see gpt2_graph_capture); replay it with graph_launch()."""
        import torch
        assert tokens.dtype == torch.int32 and targets.dtype == torch.int32
        assert tokens.is_contiguous() and targets.is_contiguous() and tokens.shape == targets.shape
        B, T = tokens.shape
        out = self.loss if loss_out is None else loss_out
        check(lib().gpt2_graph_capture(self._h, tokens.data_ptr(), targets.data_ptr(), B, T, float(loss_scale),
                                       out.data_ptr()), "gpt2_graph_capture")
        return out

    def graph_launch(self):
        check(lib().gpt2_graph_launch(self._h), "gpt2_graph_launch")

    def clip_adamw_step(self, lr: float, beta1: float = 0.9, beta2: float = 0.95, eps: float = 1e-8,
                        weight_decay: float = 0.1, max_norm: float = 1.0, norm_out=None):
        hp = _ffi.AdamW(lr, beta1, beta2, eps, weight_decay, max_norm)
        out = self.grad_norm if norm_out is None else norm_out
        check(lib().gpt2_clip_adamw_step(self._h, ct.byref(hp), out.data_ptr()), "gpt2_clip_adamw_step")
        return out

    @property
    def step(self) -> int:
        t = ct.c_int64()
        check(lib().gpt2_get_step(self._h, ct.byref(t)), "gpt2_get_step")
        return t.value

    @step.setter
    def step(self, t: int):
        check(lib().gpt2_set_step(self._h, t), "gpt2_set_step")

    def status(self) -> int:
        """Synchronise and return (and clear) the device flag."""
        return lib().gpt2_get_status(self._h)

    # -- measurement ---------------------------------------------------------
    def profile(self, on: bool = True):
        check(lib().gpt2_profile_enable(self._h, 1 if on else 0), "gpt2_profile_enable")

    def profile_only(self, site=None):
        """Time only launches from `site` (None: every site)."""
        check(lib().gpt2_profile_only(self._h, site.encode() if site else None), "gpt2_profile_only")

    def profile_mark(self, on: bool = True):
        """Precede every timed launch with the empty marker kernel."""
        check(lib().gpt2_profile_mark(self._h, 1 if on else 0), "gpt2_profile_mark")

    def profile_reset(self):
        check(lib().gpt2_profile_reset(self._h), "gpt2_profile_reset")

    def profile_entries(self):
        n = lib().gpt2_profile_count(self._h)
        out = {}
        for i in range(n):
            name = ct.c_char_p()
            cnt = ct.c_int64()
            ms = ct.c_double()
            check(lib().gpt2_profile_entry(self._h, i, ct.byref(name), ct.byref(cnt), ct.byref(ms)), "profile")
            out[name.value.decode()] = (cnt.value, ms.value)
        return out

    def close(self):
        if getattr(self, "_h", None):
            lib().gpt2_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------ single ops

def lmhead_ce(hidden, weight, targets, dweight, stream=None, flag=None, ignore_index=-1, scratch=None, loss=None,
              dhidden=None):
    """Isolated tied lm_head + mean cross-entropy (bf16 hidden [M, C], bf16
    weight [V, C], int32 targets [M]; targets equal to ignore_index are
    ignored); dweight (float32 [V, C]) is added to.  scratch, loss and
    dhidden may be passed in (reused across calls).  Returns (loss [1]
    float32, dhidden bf16 [M, C])."""
    import torch
    M, C = hidden.shape
    V = weight.shape[0]
    if scratch is None:
        scratch = torch.empty(lib().gpt2_lmhead_ce_scratch_bytes(M, C, V), dtype=torch.uint8, device=hidden.device)
    loss = torch.empty(1, dtype=torch.float32, device=hidden.device) if loss is None else loss
    dh = torch.empty_like(hidden) if dhidden is None else dhidden
    check(lib().gpt2_lmhead_ce(_stream_ptr(stream), hidden.data_ptr(), weight.data_ptr(), targets.data_ptr(), M, C, V,
                               int(ignore_index), loss.data_ptr(), dh.data_ptr(), dweight.data_ptr(),
                               scratch.data_ptr(), _ptr(flag)),
          "gpt2_lmhead_ce")
    return loss, dh


def op_gemm(A, B, C, M, N, K, a_kmajor=True, b_kmajor=True, lda=None, ldb=None, ldc=None, epilogue=EPI_STORE,
            C2=None, R=None, U=None, bias=None, alpha=1.0, rope=None, rope_period=0, rope_cols=0, ld2=None,
            stream=None):
    import torch
    dtype = PRECISION_BF16 if A.dtype == torch.bfloat16 else PRECISION_FP32
    a = _ffi.GemmArgs()
    a.M, a.N, a.K, a.dtype = M, N, K, dtype
    a.a_kmajor, a.b_kmajor = int(a_kmajor), int(b_kmajor)
    a.lda = lda if lda is not None else (K if a_kmajor else M)
    a.ldb = ldb if ldb is not None else (K if b_kmajor else N)
    default_ldc = {EPI_SWIGLU: N // 2, EPI_SWIGLU_BWD: 2 * N}.get(epilogue, N)
    a.ldc = ldc if ldc is not None else default_ldc
    a.A, a.B, a.C = A.data_ptr(), B.data_ptr(), C.data_ptr()
    a.C2, a.R, a.U, a.bias = _ptr(C2), _ptr(R), _ptr(U), _ptr(bias)
    a.alpha = alpha
    a.epilogue = epilogue
    a.out_bf16 = int(C.dtype == torch.bfloat16)
    a.rope, a.rope_period, a.rope_cols = _ptr(rope), rope_period, rope_cols
    a.ld2 = ld2 if ld2 is not None else {EPI_SWIGLU: N, EPI_SWIGLU_BWD: 2 * N}.get(epilogue, 0)
    check(lib().gpt2_op_gemm(_stream_ptr(stream), ct.byref(a)), "gpt2_op_gemm")


def op_gemm_grouped(products, stream=None):
    """Weight-gradient products in one launch: each item (A, B, C, M, N, K,
    row_sum, alpha) computes C[M, N] += alpha * A^T B over K (A bf16 stored
    [K][M], B bf16 stored [K][N], C float32 [M][N]) and, when row_sum is a
    tensor, row_sum[m] += alpha * sum_k A[k][m]."""
    import torch
    n = len(products)
    arr = (_ffi.GemmArgs * n)()
    rs = (ct.c_void_p * n)()
    for i, (A, B, C, M, N, K, row_sum, alpha) in enumerate(products):
        a = arr[i]
        a.M, a.N, a.K, a.dtype = M, N, K, PRECISION_BF16
        a.a_kmajor, a.b_kmajor = 0, 0
        a.lda, a.ldb, a.ldc = M, N, N
        a.A, a.B, a.C = A.data_ptr(), B.data_ptr(), C.data_ptr()
        a.alpha = alpha
        a.epilogue = EPI_ACCUMULATE
        a.out_bf16 = 0
        rs[i] = row_sum.data_ptr() if row_sum is not None else None
    nbytes = lib().gpt2_gemm_grouped_workspace_bytes(arr, n)
    if nbytes == 0:
        raise GPT2Error(GPT2_ERR_ARG, "gpt2_gemm_grouped_workspace_bytes")
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    check(lib().gpt2_op_gemm_grouped(_stream_ptr(stream), arr, n, rs, ws.data_ptr()), "gpt2_op_gemm_grouped")
    return ws


def op_rope_table(T, base=10000.0, stream=None):
    """(cos, sin) of the rotary angles for head dimension 64: float32 [T, 32, 2]."""
    import torch
    tab = torch.empty((T, 32, 2), dtype=torch.float32, device="cuda")
    check(lib().gpt2_op_rope_table(_stream_ptr(stream), T, float(base), tab.data_ptr()), "gpt2_op_rope_table")
    return tab


def op_rope_bwd(dqkv, T, n_embd, tab, stream=None):
    """Backward rotation, in place, of the q and k blocks of dqkv [rows, 3 C] (bf16)."""
    rows = dqkv.shape[0]
    check(lib().gpt2_op_rope_bwd(_stream_ptr(stream), dqkv.data_ptr(), rows, dqkv.stride(0), 2 * n_embd, T,
                                 tab.data_ptr()), "gpt2_op_rope_bwd")


def op_rmsnorm_fwd(x, w, y, rstd, stream=None):
    rows, C = x.shape
    check(lib().gpt2_op_rmsnorm_fwd(_stream_ptr(stream), x.data_ptr(), w.data_ptr(), y.data_ptr(), rstd.data_ptr(),
                                    rows, C), "gpt2_op_rmsnorm_fwd")


def op_rmsnorm_bwd(dy, x, rstd, w, dx, dw, dx_bf16=None, stream=None):
    import torch
    rows, C = x.shape
    check(lib().gpt2_op_rmsnorm_bwd(_stream_ptr(stream), dy.data_ptr(), int(dy.dtype == torch.bfloat16), x.data_ptr(),
                                    rstd.data_ptr(), w.data_ptr(), dx.data_ptr(), _ptr(dx_bf16), dw.data_ptr(),
                                    rows, C), "gpt2_op_rmsnorm_bwd")


def op_marker(stream=None):
    """One launch of the library's empty marker kernel (delimits work in a
    per-dispatch counter trace)."""
    check(lib().gpt2_op_marker(_stream_ptr(stream)), "gpt2_op_marker")


def op_colsum(Y, db, stream=None):
    import torch
    M, N = Y.shape
    check(lib().gpt2_op_colsum(_stream_ptr(stream), Y.data_ptr(), int(Y.dtype == torch.bfloat16), M, N, Y.stride(0),
                               db.data_ptr()), "gpt2_op_colsum")


def op_layernorm_fwd(x, w, b, y, mean, rstd, stream=None):
    import torch
    rows, C = x.shape
    check(lib().gpt2_op_layernorm_fwd(_stream_ptr(stream), x.data_ptr(), w.data_ptr(), b.data_ptr(), y.data_ptr(),
                                      int(y.dtype == torch.bfloat16), mean.data_ptr(), rstd.data_ptr(), rows, C),
          "gpt2_op_layernorm_fwd")


def op_layernorm_bwd(dy, x, mean, rstd, w, dx, dw, db, dx_bf16=None, stream=None):
    """dy float32 or bf16; dx (float32) += the input gradient; dx_bf16 (optional)
    receives bf16 of the updated dx."""
    import torch
    rows, C = x.shape
    check(lib().gpt2_op_layernorm_bwd(_stream_ptr(stream), dy.data_ptr(), int(dy.dtype == torch.bfloat16),
                                      x.data_ptr(), mean.data_ptr(), rstd.data_ptr(), w.data_ptr(), dx.data_ptr(),
                                      _ptr(dx_bf16), dw.data_ptr(), db.data_ptr(), rows, C),
          "gpt2_op_layernorm_bwd")


def op_attention_fwd(qkv, y, lse, B, T, H, hd, stream=None, seg=None, n_kv_head=None):
    """seg: optional int32 device tensor [B, T] of document starts
    (op_segment_starts) for packed windows; n_kv_head: key/value heads
    (grouped-query attention; default H)."""
    import torch
    dtype = PRECISION_BF16 if qkv.dtype == torch.bfloat16 else PRECISION_FP32
    _check_seg(seg, B, T)
    Hkv = H if n_kv_head is None else n_kv_head
    check(lib().gpt2_op_attention_fwd(_stream_ptr(stream), dtype, B, T, H, Hkv, hd, qkv.data_ptr(), y.data_ptr(),
                                      lse.data_ptr(), _ptr(seg)), "gpt2_op_attention_fwd")


def op_attention_bwd(qkv, y, dy, lse, dqkv, B, T, H, hd, stream=None, seg=None, n_kv_head=None, rope=None):
    """rope: optional [T][32] (cos, sin) table (op_rope_table): dq and dk are
    rotated back before they are written."""
    import torch
    dtype = PRECISION_BF16 if qkv.dtype == torch.bfloat16 else PRECISION_FP32
    _check_seg(seg, B, T)
    Hkv = H if n_kv_head is None else n_kv_head
    nbytes = lib().gpt2_attention_bwd_scratch_bytes(B, T, H)
    scratch = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=qkv.device)
    check(lib().gpt2_op_attention_bwd(_stream_ptr(stream), dtype, B, T, H, Hkv, hd, qkv.data_ptr(), y.data_ptr(),
                                      dy.data_ptr(), lse.data_ptr(), dqkv.data_ptr(), scratch.data_ptr(), _ptr(seg),
                                      _ptr(rope)),
          "gpt2_op_attention_bwd")


def op_attention_bwd_noalloc(qkv, y, dy, lse, dqkv, B, T, H, hd, stream=None, seg=None, n_kv_head=None, rope=None):
    """op_attention_bwd without a workspace: the library's static per-GPU
    array holds its two floats per row (B * H * T <= 1,048,576); calls
    overlapping on one GPU race on it."""
    import torch
    dtype = PRECISION_BF16 if qkv.dtype == torch.bfloat16 else PRECISION_FP32
    _check_seg(seg, B, T)
    Hkv = H if n_kv_head is None else n_kv_head
    check(lib().gpt2_op_attention_bwd_noalloc(_stream_ptr(stream), dtype, B, T, H, Hkv, hd, qkv.data_ptr(),
                                              y.data_ptr(), dy.data_ptr(), lse.data_ptr(), dqkv.data_ptr(),
                                              _ptr(seg), _ptr(rope)),
          "gpt2_op_attention_bwd_noalloc")


def _check_seg(seg, B, T):
    import torch
    if seg is not None:
        assert seg.dtype == torch.int32 and seg.is_contiguous() and seg.numel() == B * T


def op_embedding_bwd(tokens, dres, dwte, dwpe=None, seg=None, stream=None):
    """dwte[tokens[i]] += dres[i] and dwpe[t(i)] += dres[i] (float32, accumulated
    in place; t(i) restarts at document starts when seg is given), each
    gradient row summing its rows in increasing i."""
    import torch
    assert tokens.dtype == torch.int32 and tokens.is_contiguous() and tokens.dim() == 2
    B, T = tokens.shape
    V, C = dwte.shape
    assert dres.dtype == torch.float32 and dres.is_contiguous() and dres.numel() == B * T * C
    assert dwte.dtype == torch.float32 and dwte.is_contiguous()
    if dwpe is not None:
        assert dwpe.dtype == torch.float32 and dwpe.is_contiguous() and dwpe.shape == (T, C)
    _check_seg(seg, B, T)
    nbytes = lib().gpt2_embedding_bwd_scratch_bytes(B * T, C)
    scratch = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dres.device)
    check(lib().gpt2_op_embedding_bwd(_stream_ptr(stream), tokens.data_ptr(), dres.data_ptr(), dwte.data_ptr(),
                                      _ptr(dwpe), B, T, C, V, _ptr(seg), scratch.data_ptr()),
          "gpt2_op_embedding_bwd")


def op_segment_starts(tokens, eot: int, stream=None):
    """Document starts of packed rows: int32 [B, T], entry t = the last
    position <= t holding ``eot`` (0 if none)."""
    import torch
    assert tokens.dtype == torch.int32 and tokens.is_contiguous() and tokens.dim() == 2
    B, T = tokens.shape
    seg = torch.empty_like(tokens)
    check(lib().gpt2_op_segment_starts(_stream_ptr(stream), tokens.data_ptr(), B, T, int(eot), seg.data_ptr()),
          "gpt2_op_segment_starts")
    return seg
from . import train  # noqa: E402,F401  (the training loop)
