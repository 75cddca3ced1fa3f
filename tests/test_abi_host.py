"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every entry point include/gpt2.h declares, and its host logic (config
validation, buffer sizes, the parameter table) is right."""

import ctypes as ct
import os
import re

import numpy as np
import pytest

from oracle import model as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gpt2.h")


def _lib():
    from gpt_pretraining_step_amd import _ffi
    if not os.path.exists(_ffi.LIB_PATH):
        pytest.fail("libgpt2hip.so is not built (python -m gpt_pretraining_step_amd.build)")
    return _ffi.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gpt2_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_core_calls():
    names = declared_functions()
    for core in ("gpt2_init_params", "gpt2_fwd_bwd", "gpt2_clip_adamw_step", "gpt2_zero_grad"):
        assert core in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing
    from gpt_pretraining_step_amd import _ffi
    assert set(declared_functions()) == set(_ffi.SIGNATURES), "binding and header disagree"


def test_struct_layouts_match_header_sizes():
    from gpt_pretraining_step_amd import _ffi
    assert ct.sizeof(_ffi.Config) == 10 * 4
    assert ct.sizeof(_ffi.AdamW) == 6 * 4
    assert ct.sizeof(_ffi.Buffers) == 7 * 8
    assert ct.sizeof(_ffi.ParamDesc) == 64 + 8 + 4 + 8 + 4


def test_rotary_param_table_matches_oracle_specs():
    """The rotary variant's table: the oracle's names and shapes, decayed 2-D
    tensors first, 123,587,328 parameters at the full size; configurations
    the kernels do not cover are rejected."""
    _lib()
    import gpt_pretraining_step_amd as g
    from oracle import modern as MM
    for cfg in (g.GPT2_ROTARY_124M,
                g.ModelConfig(1024, 256, 2, 4, 256, 160, 3, g.PRECISION_BF16, g.ARCH_ROTARY),
                g.ModelConfig(1024, 256, 2, 4, 256, 160, 3, g.PRECISION_BF16, g.ARCH_ROTARY, n_kv_head=2),
                g.ModelConfig(50304, 1024, 12, 12, 768, 2048, 8, g.PRECISION_BF16, g.ARCH_ROTARY, n_kv_head=4)):
        oc = MM.ModernConfig(cfg.vocab_size, cfg.block_size, cfg.n_layer, cfg.n_head, cfg.n_embd, cfg.mlp_hidden,
                             n_kv_head=cfg.n_kv_head)
        table = g.param_table(cfg)
        assert {n: tuple(s) for n, _, s, _ in table} == dict(MM.param_specs(oc))
        decayed = [d for _, _, _, d in table]
        assert decayed == sorted(decayed, reverse=True)
        assert all(d == (len(s) == 2) for _, _, s, d in table)
        assert g.query_sizes(cfg).n_params == MM.n_params(oc)
    assert g.query_sizes(g.GPT2_ROTARY_124M).n_params == 123_587_328
    for bad in (g.ModelConfig(1024, 256, 2, 4, 256, 160, 3, g.PRECISION_FP32, g.ARCH_ROTARY),  # bf16 only
                g.ModelConfig(1024, 256, 2, 2, 128, 160, 3, g.PRECISION_BF16, g.ARCH_ROTARY),   # C % 256
                g.ModelConfig(1024, 256, 2, 4, 256, 150, 3, g.PRECISION_BF16, g.ARCH_ROTARY),   # F % 32
                g.ModelConfig(1024, 256, 2, 4, 256, 160, 3, g.PRECISION_BF16, 7),
                g.ModelConfig(1024, 256, 2, 4, 256, 160, 3, g.PRECISION_BF16, g.ARCH_ROTARY, n_kv_head=3),  # 4 % 3
                g.ModelConfig(1024, 256, 2, 4, 256, 160, 3, g.PRECISION_BF16, g.ARCH_ROTARY, n_kv_head=-1),
                g.ModelConfig(1024, 256, 2, 4, 256, 1024, 3, g.PRECISION_BF16, n_kv_head=2),  # GPT-2: MHA only
                g.ModelConfig(1024, 1024, 2, 2, 128, 512, 129, g.PRECISION_BF16)):  # > 131,072 rows
        with pytest.raises(g.GPT2Error):
            g.query_sizes(bad)
    g.query_sizes(g.ModelConfig(1024, 1024, 2, 2, 128, 512, 128, g.PRECISION_BF16))  # 131,072 rows


def _cfgs():
    import gpt_pretraining_step_amd as g
    return g.GPT2_124M, g.TINY_CHAR_FP32


def _oracle_cfg(c):
    return M.Config(c.vocab_size, c.block_size, c.n_layer, c.n_head, c.n_embd, c.mlp_hidden)


@pytest.mark.parametrize("which", [0, 1])
def test_param_table_matches_oracle_specs(which):
    _lib()
    import gpt_pretraining_step_amd as g
    cfg = _cfgs()[which]
    sizes = g.query_sizes(cfg)
    table = g.param_table(cfg)
    ocfg = _oracle_cfg(cfg)
    specs = dict(M.param_specs(ocfg))
    assert len(table) == len(specs) == sizes.n_tensors
    assert sizes.n_params == M.n_params(ocfg)
    names = [t[0] for t in table]
    assert set(names) == set(specs)
    # decayed (dim >= 2) entries first
    dec = [t[3] for t in table]
    assert dec == sorted(dec, reverse=True)
    assert sum(dec) == sizes.n_decayed
    spans = []
    for name, off, shape, decayed in table:
        assert tuple(shape) == tuple(specs[name])
        assert decayed == M.is_decayed(specs[name])
        assert off % 64 == 0
        spans.append((off, off + int(np.prod(shape))))
    spans.sort()
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert spans[-1][1] <= sizes.n_elems
    assert sizes.params_bytes == 4 * sizes.n_elems
    if cfg.precision == g.PRECISION_BF16:
        assert sizes.shadow_bytes == 2 * sizes.n_elems
        assert sizes.n_params == 124_475_904 and sizes.n_tensors == 148 and sizes.n_decayed == 50
    else:
        assert sizes.shadow_bytes == 0 and sizes.n_params == 108_416


def test_bad_configs_are_rejected():
    _lib()
    import gpt_pretraining_step_amd as g
    from gpt_pretraining_step_amd import _ffi
    good = g.GPT2_124M
    bad = [
        good.__class__(**{**good.__dict__, "n_head": 7}),           # 768 % 7 != 0
        good.__class__(**{**good.__dict__, "n_head": 6}),           # head dim 128 in bf16
        good.__class__(**{**good.__dict__, "vocab_size": 50257}),   # not a multiple of 8 in bf16
        good.__class__(**{**good.__dict__, "max_batch": 0}),
        good.__class__(**{**good.__dict__, "precision": 7}),
        good.__class__(**{**good.__dict__, "n_embd": 2048, "n_head": 32}),
    ]
    for c in bad:
        with pytest.raises(_ffi.GPT2Error) as e:
            g.query_sizes(c)
        assert e.value.status == _ffi.GPT2_ERR_SHAPE
    # unpadded vocabulary is fine in float32 mode
    ok = good.__class__(**{**good.__dict__, "vocab_size": 50257, "precision": 0})
    assert g.query_sizes(ok).n_params == 124_439_808


def test_null_arguments_are_rejected():
    L = _lib()
    from gpt_pretraining_step_amd import _ffi
    assert L.gpt2_query_sizes(None, None) == _ffi.GPT2_ERR_ARG
    assert L.gpt2_fwd_bwd(None, None, None, 1, 1, 1.0, None, None) == _ffi.GPT2_ERR_ARG
    assert L.gpt2_zero_grad(None) == _ffi.GPT2_ERR_ARG
    assert L.gpt2_get_status(None) == _ffi.GPT2_ERR_ARG
    assert L.gpt2_strerror(_ffi.GPT2_ERR_BAD_ID).decode().startswith("token or target")
    c = _ffi.Config(66, 64, 2, 4, 64, 256, 4, 0)
    b = _ffi.Buffers()
    h = ct.c_void_p()
    assert L.gpt2_create(ct.byref(c), ct.byref(b), None, ct.byref(h)) == _ffi.GPT2_ERR_UNBOUND
    d = _ffi.ParamDesc()
    assert L.gpt2_param_info(ct.byref(c), 10_000, ct.byref(d)) == _ffi.GPT2_ERR_ARG


def test_grouped_products_validate_on_the_host():
    """The grouped weight-gradient call accepts only bf16 products with both
    operands K-slow that accumulate into float32, and says so before any
    device work (fake, aligned pointers: nothing is dereferenced)."""
    L = _lib()
    from gpt_pretraining_step_amd import _ffi
    arr = (_ffi.GemmArgs * 2)()
    for i, (M, N) in enumerate([(768, 3072), (264, 136)]):
        a = arr[i]
        a.M, a.N, a.K, a.dtype = M, N, 1024, _ffi.PRECISION_BF16
        a.lda, a.ldb, a.ldc = M, N, N
        a.A, a.B, a.C = 0x10000, 0x20000, 0x30000
        a.alpha, a.epilogue = 1.0, _ffi.EPI_ACCUMULATE
    # 3 x 12 + 2 x 1 tiles of 256 x 256: the table holds both products' parameters and the unit map
    nbytes = L.gpt2_gemm_grouped_workspace_bytes(arr, 2)
    assert nbytes >= 38 * 4
    assert L.gpt2_gemm_grouped_workspace_bytes(arr, 0) == 0
    assert L.gpt2_op_gemm_grouped(None, arr, 0, None, ct.c_void_p(0x40000)) == _ffi.GPT2_ERR_ARG
    assert L.gpt2_op_gemm_grouped(None, arr, 2, None, None) == _ffi.GPT2_ERR_ARG
    for field, bad in [("a_kmajor", 1), ("b_kmajor", 1), ("epilogue", _ffi.EPI_STORE), ("dtype", _ffi.PRECISION_FP32),
                       ("out_bf16", 1), ("lda", 100)]:
        old = getattr(arr[1], field)
        setattr(arr[1], field, bad)
        assert L.gpt2_gemm_grouped_workspace_bytes(arr, 2) == 0, field
        assert L.gpt2_op_gemm_grouped(None, arr, 2, None, ct.c_void_p(0x40000)) == _ffi.GPT2_ERR_ARG, field
        setattr(arr[1], field, old)
    assert L.gpt2_gemm_grouped_workspace_bytes(arr, 2) == nbytes


def test_grouped_split_plan_for_the_gpt2_step():
    """The weight-gradient products of one GPT-2 124M micro-step (per layer
    mlp_proj, fc, attn_proj, qkv: 36 + 36 + 9 + 27 tiles of 256 x 256, 1,296
    in all, 16 past five full rounds of 256 blocks): from 4,096 tokens the
    last product (27 tiles) runs as quarters of K (27 x 3 more units in the
    table), below that whole."""
    L = _lib()
    from gpt_pretraining_step_amd import _ffi
    n = 48
    arr = (_ffi.GemmArgs * n)()
    shapes = [(768, 3072), (3072, 768), (768, 768), (2304, 768)] * 12
    def table_bytes(K):
        for i, (M, N) in enumerate(shapes):
            a = arr[i]
            a.M, a.N, a.K, a.dtype = M, N, K, _ffi.PRECISION_BF16
            a.lda, a.ldb, a.ldc = M, N, N
            a.A, a.B, a.C = 0x10000, 0x20000, 0x30000
            a.alpha, a.epilogue = 1.0, _ffi.EPI_ACCUMULATE
        return L.gpt2_gemm_grouped_workspace_bytes(arr, n)
    a256 = lambda b: (b + 255) // 256 * 256
    params = table_bytes(1024) - a256(1296 * 4)  # whole tiles only
    assert params > 0 and params % 256 == 0
    assert table_bytes(16384) == params + a256((1296 + 27 * 3) * 4)
    assert table_bytes(4096) == params + a256((1296 + 27 * 3) * 4)
    assert table_bytes(2048) == params + a256(1296 * 4)


def _declarations():
    """name -> number of parameters, from the header's prototypes."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(gpt2_[a-z0-9_]+)\s*\(([^;{]*?)\)\s*;", text, flags=re.S):
        args = m.group(2).strip()
        out[m.group(1)] = 0 if args in ("", "void") else args.count(",") + 1
    return out


def test_binding_argument_counts_match_the_header():
    from gpt_pretraining_step_amd import _ffi
    decl = _declarations()
    assert set(decl) == set(_ffi.SIGNATURES)
    wrong = {n: (k, len(_ffi.SIGNATURES[n][1])) for n, k in decl.items() if k != len(_ffi.SIGNATURES[n][1])}
    assert not wrong, wrong


def test_logits_are_never_sized_for_the_whole_batch():
    """The lm_head runs in row chunks: neither the training step's scratch
    nor the isolated lm_head's grows with rows x vocabulary beyond one chunk
    of 8192 rows."""
    _lib()
    import gpt_pretraining_step_amd as g
    from gpt_pretraining_step_amd import _ffi
    L = _ffi.lib()
    V, C = 50304, 768
    chunk_bytes = 8192 * V * 2 + 8192 * ((V + 255) // 256) * 8
    for M in (8192, 16384, 65536):
        got = L.gpt2_lmhead_ce_scratch_bytes(M, C, V)
        assert got <= M * (C + 1) * 4 + chunk_bytes + 5 * 256, M
        if M > 8192:
            assert got < M * V * 2  # less than the whole logit matrix in bf16
    # the training step at B=16 (16,384 rows): 256 more vocabulary columns
    # cost one chunk's worth of logits (8192 rows) and statistics, not 16,384
    sa = g.query_sizes(g.GPT2_124M).scratch_bytes
    sb = g.query_sizes(g.ModelConfig(50304 + 256, 1024, 12, 12, 768, 3072, 16, g.PRECISION_BF16)).scratch_bytes
    assert 8192 * 256 * 2 <= sb - sa <= 8192 * 256 * 2 + 8192 * 8 + 1024, sb - sa


def test_embedding_backward_validates_on_the_host():
    """gpt2_op_embedding_bwd rejects bad shapes, null pointers and a
    misaligned workspace before it launches anything."""
    L = _lib()
    from gpt_pretraining_step_amd import _ffi
    p = ct.c_void_p(0x40000)
    call = lambda B, T, C, V, tok=p, scr=p: L.gpt2_op_embedding_bwd(None, tok, p, p, None, B, T, C, V, None, scr)
    assert call(0, 4, 4, 4) == _ffi.GPT2_ERR_SHAPE
    assert call(129, 1024, 4, 4) == _ffi.GPT2_ERR_SHAPE       # more than 131,072 rows
    assert call(1, 4, 1 << 20, 4096) == _ffi.GPT2_ERR_SHAPE   # V * C >= 2^31
    assert call(1, 4, 4, 4, tok=None) == _ffi.GPT2_ERR_ARG
    assert call(1, 4, 4, 4, scr=ct.c_void_p(0x40010)) == _ffi.GPT2_ERR_ARG
    n = L.gpt2_embedding_bwd_scratch_bytes(16384, 768)
    assert n >= 16384 * 768 * 4 + 2 * 16384 * 4
    assert L.gpt2_embedding_bwd_scratch_bytes(0, 768) == 0
