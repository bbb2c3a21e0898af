"""GPU parity of branch fusion with a sliding-window local branch.

The sparse branch runs over the GPU's own Top-K indices (as the other parity
tests do), the local branch over the window positions (checked bit-exact
against the oracle's), both ungated through a per-head gate of +inf; the fused
output is compared with the oracle's double-precision fusion of its own branch
outputs on the same index sets.  Both forms of the fusion are checked: the
separate mix pass over the two branch outputs, and the local branch's attention
with the mix in its epilogue (the sparse branch's output read there, the local
branch's never rounded).
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import parity as P
from indexer_top_sparse_relu_amd import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from indexer_top_sparse_relu_amd import binding as B  # noqa: E402

DEV = "cuda"


def run_fused(wl, w):
    s = wl.spec
    pl = B.Pipeline(wl)
    pl.indexer()
    pl.topk()
    bt = pl.batch
    inf = torch.full((s.T, s.Hq), float("inf"), device=DEV).to(wl.q.dtype)
    win = torch.full((s.T, w), -7, dtype=torch.int32, device=DEV)
    B.sparse_window_indices(bt, w, win)
    outs = []
    for idx in (pl.indices, win):
        o = torch.full((s.T, s.Hq, s.d_v), float("nan"), device=DEV).to(wl.q.dtype)
        aw = B.sparse_gated_attn_workspace_size(bt, s.Hq, s.d_v, idx.shape[1])
        aws = torch.empty(aw, dtype=torch.uint8, device=DEV) if aw else None
        B.sparse_gated_attn_fwd(bt, wl.q, wl.k_cache, wl.v_cache, s.d_v, idx, inf, o,
                                softmax_scale=s.softmax_scale, workspace=aws)
        outs.append(o)
    y = torch.full_like(outs[0], float("nan"))
    B.sparse_branch_fuse(outs[0], outs[1], wl.gate, y)
    y2 = torch.full_like(outs[0], float("nan"))
    lse2 = torch.full((s.T, s.Hq), float("nan"), device=DEV)
    aw = B.sparse_gated_attn_workspace_size(bt, s.Hq, s.d_v, w)
    aws = torch.empty(aw, dtype=torch.uint8, device=DEV) if aw else None
    B.sparse_attn_fuse_fwd(bt, wl.q, wl.k_cache, wl.v_cache, s.d_v, win, wl.gate, outs[0], y2,
                           softmax_scale=s.softmax_scale, lse=lse2, workspace=aws)
    torch.cuda.synchronize()
    return pl.indices.cpu().numpy(), win.cpu().numpy(), outs, y, y2, lse2.cpu().numpy()


def check_fused(spec, w, tag, rows=None):
    P.say(f"[{tag}] {spec.name} T={spec.T} B={spec.B} window={w}")
    wl = W.generate(spec, DEV)
    idx, win, (o_s, o_l), y, y2, lse2 = run_fused(wl, w)
    inp = O.Inputs.from_workload(wl)
    rows = np.arange(spec.T) if rows is None else np.asarray(rows)
    assert np.array_equal(win, O.window_indices(inp, w)), "window positions"
    u = O.ungated(inp)
    a = O.sparse_attn(u, idx[rows], rows, spec.softmax_scale)
    b, b_lse = O.sparse_attn(u, win[rows], rows, spec.softmax_scale, with_lse=True)
    tol = P.RTOL[spec.attn_dtype]
    fa = P.attn_floor(u, idx[rows], rows, spec.softmax_scale)
    fb = P.attn_floor(u, win[rows], rows, spec.softmax_scale)
    P.check_attn(o_s.float().cpu().numpy()[rows], a, tol, fa, "sparse branch")
    P.check_attn(o_l.float().cpu().numpy()[rows], b, tol, fb, "local branch")
    ref = O.branch_fuse(inp, a, b, rows)
    # the fusion's floor: both branches' floors plus their rounding to the output type
    a_abs = P.attn_abs(u, idx[rows], rows, spec.softmax_scale)
    b_abs = P.attn_abs(u, win[rows], rows, spec.softmax_scale)
    ff = P.fused_floor(inp, fa, fb, a_abs, b_abs, rows)
    worst = P.check_attn(y.float().cpu().numpy()[rows], ref, tol, ff, "fused output")
    # the epilogue mix rounds one branch fewer, so the same floor bounds it
    worst2 = P.check_attn(y2.float().cpu().numpy()[rows], ref, tol, ff, "fused in the epilogue")
    assert P.close(lse2[rows], b_lse, tol).all(), "local branch lse"
    P.say(f"[{tag}] ok: worst {worst:.2f} (mix pass), {worst2:.2f} (epilogue mix) of the bound")


def test_fusion_latent_prefill_per_channel_gate():
    spec = W.chunked_prefill_mla(cached=3000, T=333)
    check_fused(spec, 256, "fuse-mla", rows=P.sample_tokens(333, 24, seed=10))


def test_fusion_paged_decode_per_head_gate():
    spec = W.decode_bf16(B=10, lo=100, hi=6000).replace(K=512, gate_per_channel=False, seed=43)
    check_fused(spec, 300, "fuse-decode")


def test_fusion_fp32_window_longer_than_rows():
    spec = W.tiny_prefill_fp32().replace(seed=44)
    check_fused(spec, 100, "fuse-f32")
