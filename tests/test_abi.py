"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments on the host before any launch (no GPU needed: no call here reaches a
kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


@pytest.fixture(scope="module")
def B():
    from indexer_top_sparse_relu_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from indexer_top_sparse_relu_amd import build
        build.build()
    return binding


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:sa_status|size_t|const char \*|int32_t)\s*\*?\s*(\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("sparse_indexer_scores", "sparse_topk", "sparse_topk_workspace_size", "sparse_gated_attn_fwd",
              "sparse_gated_attn_workspace_size", "sa_status_string", "sa_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(B):
    L = B.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(B.EXPORTS) == set(declared_functions())
    assert L.sa_abi_version() == 1


def test_status_strings(B):
    for st in (0, -1, -2, -3, -4, 7):
        s = B.status_string(st)
        assert isinstance(s, str) and s


FAKE = 1 << 20   # an aligned non-null address: validation rejects before anything dereferences it


def batch(B, **kw):
    f = dict(num_seqs=1, total_q=4, max_q=4, max_ctx=100, page_size=64, max_pages=2,
             q_start=FAKE, ctx_len=FAKE, page_table=FAKE)
    f.update(kw)
    return B.SaBatch(f["num_seqs"], f["total_q"], f["max_q"], f["max_ctx"], f["page_size"], f["max_pages"],
                     f["q_start"], f["ctx_len"], f["page_table"])


def idx_call(B, bt, dtype=1, H=16, D=64, q=FAKE, qs=None, w=FAKE, k=FAKE, ks=None, sc=FAKE, ld=128):
    return B.lib().sparse_indexer_scores(ctypes.byref(bt), dtype, q, H, D, qs, w, k, ks, sc, ld, None)


def test_indexer_argument_errors(B):
    ok = batch(B)
    assert B.lib().sparse_indexer_scores(None, 1, FAKE, 16, 64, None, FAKE, FAKE, None, FAKE, 128, None) == B.SA_EINVAL
    assert idx_call(B, batch(B, page_size=48)) == B.SA_EINVAL          # not a power of two
    assert idx_call(B, batch(B, page_size=8)) == B.SA_EINVAL           # below 16
    assert idx_call(B, batch(B, max_pages=1)) == B.SA_EINVAL           # table too short for max_ctx
    assert idx_call(B, batch(B, total_q=0)) == B.SA_EINVAL            # T = 0 needs max_q = 0
    assert idx_call(B, batch(B, total_q=-1)) == B.SA_EINVAL
    assert idx_call(B, batch(B, max_q=0)) == B.SA_EINVAL              # T > 0 needs max_q >= 1
    assert idx_call(B, batch(B, q_start=None)) == B.SA_EINVAL
    assert idx_call(B, ok, ld=64) == B.SA_EINVAL                       # ld < max_ctx
    assert idx_call(B, ok, ld=130) == B.SA_EINVAL                      # ld not a multiple of 4
    assert idx_call(B, ok, q=None) == B.SA_EINVAL
    assert idx_call(B, ok, q=FAKE + 4) == B.SA_EINVAL                  # misaligned
    assert idx_call(B, ok, dtype=2) == B.SA_EINVAL                     # fp8 without scales
    assert idx_call(B, ok, dtype=5) == B.SA_EINVAL
    assert idx_call(B, ok, H=12) == B.SA_EUNSUPPORTED
    assert idx_call(B, ok, D=48) == B.SA_EUNSUPPORTED
    assert idx_call(B, ok, dtype=2, D=64, qs=FAKE, ks=FAKE) == B.SA_EUNSUPPORTED


def test_topk_argument_errors_and_workspace(B):
    L = B.lib()
    ok = batch(B)
    call = lambda bt, k=32, ld=128, ws=None, wsb=0, sc=FAKE, out=FAKE: L.sparse_topk(
        ctypes.byref(bt), sc, ld, k, out, ws, wsb, None)
    assert call(ok, k=0) == B.SA_EINVAL
    assert call(ok, k=5000) == B.SA_EUNSUPPORTED
    assert call(ok, sc=None) == B.SA_EINVAL
    assert call(ok, out=None) == B.SA_EINVAL
    assert call(ok, ld=96) == B.SA_EINVAL
    # few rows over a long context need a workspace (chunked selection)
    long = batch(B, num_seqs=16, total_q=16, max_q=1, max_ctx=1 << 20, max_pages=(1 << 20) // 64)
    need = L.sparse_topk_workspace_size(ctypes.byref(long), 2048)
    assert need > 0
    assert call(long, k=2048, ld=1 << 20) == B.SA_EWORKSPACE
    assert call(long, k=2048, ld=1 << 20, ws=FAKE, wsb=need - 1) == B.SA_EWORKSPACE
    # many rows: no workspace
    assert L.sparse_topk_workspace_size(ctypes.byref(batch(B, total_q=4096, max_q=4096, max_ctx=8192,
                                                           max_pages=128)), 2048) == 0


def test_attention_argument_errors(B):
    L = B.lib()
    ok = batch(B)

    def call(bt=ok, dtype=1, H=32, dqk=128, kc=FAKE, vc=FAKE + (1 << 16), dv=128, rs=128, idx=FAKE, k=32,
             gate=FAKE, scale=0.1, out=FAKE, ws=None, wsb=0):
        return L.sparse_gated_attn_fwd(ctypes.byref(bt), dtype, FAKE, H, dqk, kc, vc, dv, rs, idx, k, gate, 1,
                                       ctypes.c_float(scale), out, None, ws, wsb, None)

    assert call(dtype=2) == B.SA_EINVAL
    assert call(k=0) == B.SA_EINVAL
    assert call(idx=None) == B.SA_EINVAL
    assert call(gate=None) == B.SA_EINVAL
    assert call(rs=100) == B.SA_EINVAL                     # row stride below d_qk
    assert call(rs=132) == B.SA_EINVAL                     # row not 16-byte aligned
    assert call(scale=float("nan")) == B.SA_EINVAL
    assert call(H=24) == B.SA_EUNSUPPORTED                 # bf16 needs heads in multiples of 16
    assert call(dqk=96, dv=96, rs=96) == B.SA_EUNSUPPORTED
    assert call(kc=FAKE, vc=FAKE, dqk=512, dv=576, rs=576) == B.SA_EINVAL   # aliased V wider than K
    dec = batch(B, num_seqs=16, total_q=16, max_q=1)
    need = L.sparse_gated_attn_workspace_size(ctypes.byref(dec), 128, 512, 2048)
    assert need > 0
    assert call(bt=dec, H=128, dqk=576, dv=512, rs=576, kc=FAKE, vc=FAKE, k=2048) == B.SA_EWORKSPACE


def test_empty_batch_is_a_no_op(B):
    """T = 0 passes validation and returns SA_OK without touching a pointer or the GPU."""
    L = B.lib()
    e = ctypes.byref(batch(B, total_q=0, max_q=0))
    f = ctypes.c_float(0.1)
    assert L.sparse_indexer_scores(e, 2, None, 64, 128, None, None, None, None, None, 0, None) == B.SA_OK
    assert L.sparse_topk_workspace_size(e, 2048) == 0
    assert L.sparse_topk(e, None, 0, 2048, None, None, 0, None) == B.SA_OK
    assert L.sparse_gated_attn_workspace_size(e, 128, 512, 2048) == 0
    assert L.sparse_gated_attn_fwd(e, 1, None, 128, 576, None, None, 512, 576, None, 2048, None, 1, f, None, None,
                                   None, 0, None) == B.SA_OK
    assert L.sparse_block_scores_workspace_size(e, 128) == 0
    assert L.sparse_block_scores(e, 1, None, 16, 128, None, None, 0, None, 0, None) == B.SA_OK
    assert L.sparse_block_topk_workspace_size(e, 16) == 0
    assert L.sparse_block_topk(e, None, 0, 16, None, None, 0, None) == B.SA_OK
    assert L.sparse_block_expand(e, None, 16, None, None) == B.SA_OK
    assert L.sparse_gated_attn_bwd(e, 1, None, 16, 128, None, None, 128, 128, None, 64, None, 1, f, None, None,
                                   None, None, None, None, None, None, 0, None) == B.SA_OK
    assert L.sparse_gated_attn_bwd_workspace_size(e, 16, 128, 128, 64) == 0
    assert L.sparse_window_indices(e, 64, None, None) == B.SA_OK
    assert L.sparse_cache_append(e, 1, None, 128, None, 128, None, None, 128, 1, None, 128, 2, None, None,
                                 None) == B.SA_OK
    assert L.sparse_branch_fuse(1, 0, 128, None, None, None, 1, None, None) == B.SA_OK
    assert L.sparse_quantize_fp8_rows(1, None, 0, 128, None, None, None) == B.SA_OK
    # pooling depends on the cached pages only: it still validates its arguments
    assert L.sparse_block_pool(e, 1, None, 128, 128, None, None) == B.SA_EINVAL


def test_binding_fails_loudly_without_library(B, monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        B.lib()


def test_noalloc_attention_rejects_batches_beyond_its_scratch(B):
    """The no-allocation entry point checks its static scratch limit on the host: a decode batch
    whose split partials need more than SA_NOALLOC_SCRATCH_BYTES returns SA_EWORKSPACE before any
    HIP call, and argument errors are those of sparse_gated_attn_fwd."""
    L = B.lib()
    f = ctypes.c_float(1.0 / 24)

    def call(bt, H=128, dqk=576, dv=512, k=2048, gate=FAKE):
        return L.sparse_gated_attn_fwd_noalloc(ctypes.byref(bt), 1, FAKE, H, dqk, FAKE, FAKE, dv, dqk, FAKE, k,
                                               gate, 1, f, FAKE, None, None)

    big = batch(B, num_seqs=200, total_q=200, max_q=1)
    need = L.sparse_gated_attn_workspace_size(ctypes.byref(big), 128, 512, 2048)
    assert need > (128 << 20)
    assert call(big) == B.SA_EWORKSPACE
    assert call(batch(B), gate=None) == B.SA_EINVAL
    assert call(batch(B), H=24) == B.SA_EUNSUPPORTED
    e = batch(B, total_q=0, max_q=0)
    assert L.sparse_gated_attn_fwd_noalloc(ctypes.byref(e), 1, None, 128, 576, None, None, 512, 576, None, 2048, None,
                                           1, f, None, None, None) == B.SA_OK


def test_fused_mix_entry_point_checks_the_other_branch(B):
    """sparse_attn_fuse_fwd: the other branch's output is required, 16-byte aligned and not the
    output itself; the rest of its checks are those of sparse_gated_attn_fwd."""
    L = B.lib()
    f = ctypes.c_float(1.0 / 24)
    OUT = ctypes.c_void_p(0x20000)

    def call(other, out=OUT, H=128, gate=FAKE):
        return L.sparse_attn_fuse_fwd(ctypes.byref(batch(B)), 1, FAKE, H, 576, FAKE, FAKE, 512, 576, FAKE, 2048,
                                      gate, 1, f, other, out, None, FAKE, 1 << 30, None)

    assert call(None) == B.SA_EINVAL
    assert call(OUT) == B.SA_EINVAL
    assert call(ctypes.c_void_p(0x30008)) == B.SA_EINVAL
    assert call(ctypes.c_void_p(0x30000), gate=None) == B.SA_EINVAL
    assert call(ctypes.c_void_p(0x30000), H=24) == B.SA_EUNSUPPORTED


def test_backward_checks_shapes_layout_and_workspace(B):
    """sparse_gated_attn_bwd: supported shapes, the latent layout's shared cache, and its workspace
    (size, 256-byte alignment) are checked on the host before anything is launched."""
    L = B.lib()
    f = ctypes.c_float(1.0 / 12)
    bt = batch(B)
    OTHER = 0x40000

    def call(H=32, dqk=128, dv=128, vc=FAKE, dk=FAKE, dvc=FAKE, ws=FAKE, wsb=1 << 40):
        return L.sparse_gated_attn_bwd(ctypes.byref(bt), 1, FAKE, H, dqk, FAKE, vc, dv, dqk, FAKE, 64, FAKE, 1, f,
                                       FAKE, FAKE, FAKE, FAKE, dk, dvc, FAKE, ws, wsb, None)

    need = L.sparse_gated_attn_bwd_workspace_size(ctypes.byref(bt), 32, 128, 128, 64)
    assert need > 0
    assert call(H=24) == B.SA_EUNSUPPORTED                     # heads not a multiple of 16
    assert call(H=272) == B.SA_EUNSUPPORTED                    # above 256 heads
    assert call(dqk=96, dv=96) == B.SA_EUNSUPPORTED
    assert call(dqk=576, dv=512, vc=OTHER, dvc=OTHER) == B.SA_EUNSUPPORTED   # latent rows need one cache
    assert call(vc=OTHER) == B.SA_EINVAL                       # separate caches, one gradient array
    assert call(wsb=need - 1) == B.SA_EWORKSPACE
    assert call(ws=None, wsb=need) == B.SA_EWORKSPACE
    assert call(ws=FAKE + 16, wsb=need) == B.SA_EINVAL         # not 256-byte aligned
    assert L.sparse_gated_attn_bwd_workspace_size(ctypes.byref(bt), 32, 128, 128, 64) == need
