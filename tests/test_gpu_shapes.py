"""GPU parity of every shape the C ABI accepts.

The library accepts a fixed set of (dtype, heads, head_dim) shapes for the
indexer and of (dtype, d_qk, d_v, layout, query heads) for the attention, each
served by a template instance of a kernel.  Every accepted shape runs here, in
both launch forms (prefill: the tile kernel / one workgroup per index list;
decode: the token kernel / split index lists with the combine), at small sizes
that the oracle checks on every row.  Shapes outside the set are rejected on
the host (tests/test_abi.py).
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

INDEXER_SHAPES = [(dt, h, d) for dt, d in (("f32", 32), ("bf16", 64), ("bf16", 128), ("fp8", 128))
                  for h in (4, 8, 16, 32, 64)]


def _base(mode, seed):
    """Prefill: two sequences with cached prefixes (tile kernels); decode: five sequences
    with one new token each (token kernels, split index lists)."""
    spec = W.prefill_bf16().replace(K=96, seed=seed)
    if mode == "prefill":
        return spec.replace(q_lens=(70, 45), ctx_lens=(700, 45), paged_random=True)
    return spec.replace(q_lens=(1,) * 5, ctx_lens=(90, 1500, 3100, 640, 2200), paged_random=True)


@pytest.mark.parametrize("mode", ["prefill", "decode"])
@pytest.mark.parametrize("dt,h,d", INDEXER_SHAPES, ids=[f"{a}-h{b}-d{c}" for a, b, c in INDEXER_SHAPES])
def test_indexer_shape(dt, h, d, mode):
    spec = _base(mode, seed=100 + h + d).replace(idx_dtype=dt, H_I=h, d_I=d, name=f"indexer-{dt}-{h}x{d}")
    P.say(f"[indexer {dt} {h}x{d} {mode}] T={spec.T} max_ctx={spec.max_ctx}")
    wl = W.generate(spec, DEV)
    pl = B.Pipeline(wl)
    pl.scores.fill_(float("nan"))
    pl.indices.fill_(-7)
    pl.indexer()
    pl.topk()
    torch.cuda.synchronize()
    inp = O.Inputs.from_workload(wl)
    n = P.token_geometry(spec)[2]
    sc = pl.scores.cpu().numpy()
    ref = O.indexer(inp, ld=pl.ld)
    w1 = P.check_scores(sc, ref, n, P.RTOL[dt])
    for r in range(spec.T):
        assert np.all(np.isnan(sc[r, n[r]:])), f"row {r} written past n"
    idx = pl.indices.cpu().numpy()
    P.check_idx_invariants(idx, n, spec.K)
    P.check_topk_exact(idx, sc, n, spec.K)
    rec = P.check_selection(idx, ref, n, spec.K)
    P.say(f"[indexer {dt} {h}x{d} {mode}] ok: worst score rel {w1:.2e}, recall {rec:.4f}")


# page sizes other than 64 on each indexer path: the fp8 linear-term tile kernel, the
# bf16 and fp32 tile kernels, and the decode kernels
PAGE_CASES = [(dt, h, d, ps) for dt, h, d in (("fp8", 64, 128), ("bf16", 16, 64), ("f32", 4, 32)) for ps in (16, 256)]


@pytest.mark.parametrize("mode", ["prefill", "decode"])
@pytest.mark.parametrize("dt,h,d,ps", PAGE_CASES, ids=[f"{a}-h{b}-d{c}-p{e}" for a, b, c, e in PAGE_CASES])
def test_indexer_page_size(dt, h, d, ps, mode):
    spec = _base(mode, seed=400 + h + ps).replace(idx_dtype=dt, H_I=h, d_I=d, page_size=ps,
                                                  name=f"indexer-{dt}-{h}x{d}-p{ps}")
    P.say(f"[indexer page {ps} {dt} {h}x{d} {mode}] T={spec.T} max_ctx={spec.max_ctx}")
    wl = W.generate(spec, DEV)
    pl = B.Pipeline(wl)
    pl.scores.fill_(float("nan"))
    pl.indexer()
    pl.topk()
    torch.cuda.synchronize()
    inp = O.Inputs.from_workload(wl)
    n = P.token_geometry(spec)[2]
    sc = pl.scores.cpu().numpy()
    w1 = P.check_scores(sc, O.indexer(inp, ld=pl.ld), n, P.RTOL[dt])
    for r in range(spec.T):
        assert np.all(np.isnan(sc[r, n[r]:])), f"row {r} written past n"
    idx = pl.indices.cpu().numpy()
    P.check_idx_invariants(idx, n, spec.K)
    P.check_topk_exact(idx, sc, n, spec.K)
    P.say(f"[indexer page {ps} {dt} {h}x{d} {mode}] ok: worst score rel {w1:.2e}")


# (dtype, d_qk, d_v, shared K/V row, query heads): every kernel instance the library
# dispatches to -- fp32 per head; bf16 MQA rows of 128 with 1, 2, 4 or 8 waves of 16
# heads, separate or shared; the 576/512 latent row on the general kernel (heads not a
# multiple of 128) and on the latent kernel (multiples of 128)
ATTN_SHAPES = [
    ("f32", 32, 32, False, 3), ("f32", 64, 64, False, 1), ("f32", 128, 128, False, 5), ("f32", 64, 64, True, 2),
    ("bf16", 128, 128, False, 16), ("bf16", 128, 128, False, 48), ("bf16", 128, 128, False, 64),
    ("bf16", 128, 128, False, 128), ("bf16", 128, 128, True, 32),
    ("bf16", 576, 512, True, 16), ("bf16", 576, 512, True, 64), ("bf16", 576, 512, True, 256),
]


@pytest.mark.parametrize("mode", ["prefill", "decode"])
@pytest.mark.parametrize("dt,dqk,dv,mla,hq", ATTN_SHAPES,
                         ids=[f"{a}-{b}x{c}-{'shared' if d else 'sep'}-h{e}" for a, b, c, d, e in ATTN_SHAPES])
def test_attention_shape(dt, dqk, dv, mla, hq, mode):
    spec = _base(mode, seed=200 + hq + dqk).replace(attn_dtype=dt, d_qk=dqk, d_v=dv, mla=mla, Hq=hq,
                                                  gate_per_channel=(hq % 2 == 0), name=f"attn-{dt}-{dqk}")
    P.say(f"[attn {dt} {dqk}/{dv} {'shared' if mla else 'separate'} h{hq} {mode}] T={spec.T}")
    wl = W.generate(spec, DEV)
    pl = B.Pipeline(wl)
    pl.out.fill_(float("nan"))
    pl.indexer()
    pl.topk()
    pl.attn()
    torch.cuda.synchronize()
    inp = O.Inputs.from_workload(wl)
    idx = pl.indices.cpu().numpy()
    ref, ref_lse = O.sparse_attn(inp, idx, None, spec.softmax_scale, with_lse=True)
    w = P.check_attn(pl.out.float().cpu().numpy(), ref, P.RTOL[dt], P.attn_floor(inp, idx, None, spec.softmax_scale))
    assert P.close(pl.lse.cpu().numpy(), ref_lse, P.RTOL[dt]).all(), "lse"
    P.say(f"[attn {dt} {dqk}/{dv} h{hq} {mode}] ok: worst {w:.2f} of the bound")


# one instance of each attention kernel: MQA rows (one wave per 32 heads), the general
# kernel, the latent kernel, fp32
HOLE_SHAPES = [("bf16", 128, 128, False, 32), ("bf16", 128, 128, True, 64), ("bf16", 128, 128, False, 16),
               ("bf16", 576, 512, True, 128), ("f32", 64, 64, False, 4)]


@pytest.mark.parametrize("mode", ["prefill", "decode"])
@pytest.mark.parametrize("dt,dqk,dv,mla,hq", HOLE_SHAPES,
                         ids=[f"{a}-{b}x{c}-{'shared' if d else 'sep'}-h{e}" for a, b, c, d, e in HOLE_SHAPES])
def test_attention_index_holes(dt, dqk, dv, mla, hq, mode):
    """Padding (-1) anywhere in a list, not only at its end: rows with no valid entry (out = 0,
    lse = -inf), rows with a hole every third slot from slot 1 (the first tile already has a
    missing key), and rows whose first 40 slots are padding."""
    spec = _base(mode, seed=300 + hq + dqk).replace(attn_dtype=dt, d_qk=dqk, d_v=dv, mla=mla, Hq=hq,
                                                  gate_per_channel=(hq % 2 == 0), name=f"holes-{dt}-{dqk}")
    P.say(f"[holes {dt} {dqk}/{dv} {'shared' if mla else 'separate'} h{hq} {mode}] T={spec.T}")
    wl = W.generate(spec, DEV)
    pl = B.Pipeline(wl)
    pl.out.fill_(float("nan"))
    pl.indexer()
    pl.topk()
    v = pl.indices.clone()
    T = v.shape[0]
    a, b = min(2, T), min(8, T)
    v[0:a, :] = -1
    v[a:b, 1::3] = -1
    v[b:min(b + 4, T), :40] = -1
    pl.indices.copy_(v)
    pl.attn()
    torch.cuda.synchronize()
    inp = O.Inputs.from_workload(wl)
    idx = pl.indices.cpu().numpy()
    ref, ref_lse = O.sparse_attn(inp, idx, None, spec.softmax_scale, with_lse=True)
    w = P.check_attn(pl.out.float().cpu().numpy(), ref, P.RTOL[dt], P.attn_floor(inp, idx, None, spec.softmax_scale))
    lse = pl.lse.cpu().numpy()
    dead = ~np.isfinite(ref_lse)
    assert np.all(lse[dead] == -np.inf), "lse of heads with no valid entry"
    assert P.close(lse[~dead], ref_lse[~dead], P.RTOL[dt]).all(), "lse"
    P.say(f"[holes {dt} {dqk}/{dv} h{hq} {mode}] ok: worst {w:.2f} of the bound")


ATTN_PAGE_CASES = [(*shape, ps) for shape in HOLE_SHAPES for ps in (16, 256)]


@pytest.mark.parametrize("mode", ["prefill", "decode"])
@pytest.mark.parametrize("dt,dqk,dv,mla,hq,ps", ATTN_PAGE_CASES,
                         ids=[f"{a}-{b}x{c}-{'shared' if d else 'sep'}-h{e}-p{f}" for a, b, c, d, e, f in ATTN_PAGE_CASES])
def test_attention_page_size(dt, dqk, dv, mla, hq, ps, mode):
    """Page sizes other than 64 on each attention kernel (the gather resolves every slot
    through the page table)."""
    spec = _base(mode, seed=500 + hq + ps).replace(attn_dtype=dt, d_qk=dqk, d_v=dv, mla=mla, Hq=hq, page_size=ps,
                                                  gate_per_channel=(hq % 2 == 0), name=f"page-{dt}-{dqk}")
    P.say(f"[attn page {ps} {dt} {dqk}/{dv} h{hq} {mode}] T={spec.T}")
    wl = W.generate(spec, DEV)
    pl = B.Pipeline(wl)
    pl.out.fill_(float("nan"))
    pl.run()
    torch.cuda.synchronize()
    inp = O.Inputs.from_workload(wl)
    idx = pl.indices.cpu().numpy()
    ref = O.sparse_attn(inp, idx, None, spec.softmax_scale)
    w = P.check_attn(pl.out.float().cpu().numpy(), ref, P.RTOL[dt], P.attn_floor(inp, idx, None, spec.softmax_scale))
    P.say(f"[attn page {ps} {dt} {dqk}/{dv} h{hq} {mode}] ok: worst {w:.2f} of the bound")


@pytest.mark.parametrize("mode", ["prefill", "decode"])
@pytest.mark.parametrize("dt,dqk,dv,mla,hq", ATTN_SHAPES,
                         ids=[f"{a}-{b}x{c}-{'shared' if d else 'sep'}-h{e}" for a, b, c, d, e in ATTN_SHAPES])
def test_epilogue_mix_shape(dt, dqk, dv, mla, hq, mode):
    """The branch mix formed in the attention epilogue, for every kernel instance: the
    attention kernel itself mixes when the list is whole, the combine kernel when it is
    split.  The other branch's output is random data of the output type."""
    spec = _base(mode, seed=400 + hq + dqk).replace(attn_dtype=dt, d_qk=dqk, d_v=dv, mla=mla, Hq=hq,
                                                  gate_per_channel=(hq % 2 == 1), name=f"mix-{dt}-{dqk}")
    P.say(f"[mix {dt} {dqk}/{dv} {'shared' if mla else 'separate'} h{hq} {mode}] T={spec.T}")
    wl = W.generate(spec, DEV)
    pl = B.Pipeline(wl)
    pl.indexer()
    pl.topk()
    g = torch.Generator(device=DEV).manual_seed(spec.seed)
    other = (torch.randn((spec.T, hq, dv), device=DEV, generator=g) * 0.05).to(wl.q.dtype)
    y = torch.full_like(other, float("nan"))
    lse = torch.full((spec.T, hq), float("nan"), device=DEV)
    B.sparse_attn_fuse_fwd(pl.batch, wl.q, wl.k_cache, wl.v_cache, dv, pl.indices, wl.gate, other, y,
                           softmax_scale=spec.softmax_scale, lse=lse, workspace=pl.attn_ws)
    torch.cuda.synchronize()
    inp = O.Inputs.from_workload(wl)
    idx = pl.indices.cpu().numpy()
    u = O.ungated(inp)
    o, o_lse = O.sparse_attn(u, idx, None, spec.softmax_scale, with_lse=True)
    a = other.float().cpu().numpy()
    ref = O.branch_fuse(inp, a, o)
    fb = P.attn_floor(u, idx, None, spec.softmax_scale)
    floor = P.epilogue_mix_floor(inp, fb, a, P.attn_abs(u, idx, None, spec.softmax_scale))
    w = P.check_attn(y.float().cpu().numpy(), ref, P.RTOL[dt], floor, "epilogue mix")
    assert P.close(lse.cpu().numpy(), o_lse, P.RTOL[dt]).all(), "lse"
    P.say(f"[mix {dt} {dqk}/{dv} h{hq} {mode}] ok: worst {w:.2f} of the bound")


@pytest.mark.parametrize("mode", ["prefill", "decode"])
@pytest.mark.parametrize("h", [8, 64])
def test_fp8_indexer_weight_range(h, mode):
    """Weights far from 1: per-token factors from 1e-9 to 1e9 and, within a token, heads
    spread over 2^20.  The fp8 epilogue multiplies in fp16 (8 heads at prefill, every head
    count at decode): its per-token power-of-two weight scaling keeps every score within
    the tolerance, with no overflow and no subnormal weights."""
    spec = _base(mode, seed=300 + h).replace(idx_dtype="fp8", H_I=h, d_I=128, name=f"indexer-fp8-wrange-{h}")
    P.say(f"[indexer fp8 weight range h{h} {mode}] T={spec.T}")
    wl = W.generate(spec, DEV)
    g = torch.Generator(device=DEV).manual_seed(17)
    tok = 10.0 ** (torch.rand(spec.T, device=DEV, generator=g) * 18.0 - 9.0)
    head = 2.0 ** (torch.rand(spec.T, h, device=DEV, generator=g) * 20.0 - 10.0)
    wl.w.mul_(tok[:, None] * head)
    pl = B.Pipeline(wl)
    pl.scores.fill_(float("nan"))
    pl.indexer()
    pl.topk()
    torch.cuda.synchronize()
    inp = O.Inputs.from_workload(wl)
    n = P.token_geometry(spec)[2]
    sc = pl.scores.cpu().numpy()
    assert np.all(np.isfinite(np.concatenate([sc[r, :n[r]] for r in range(spec.T)])))
    ref = O.indexer(inp, ld=pl.ld)
    w1 = P.check_scores(sc, ref, n, P.RTOL["fp8"])
    idx = pl.indices.cpu().numpy()
    P.check_topk_exact(idx, sc, n, spec.K)
    P.check_selection(idx, ref, n, spec.K)
    P.say(f"[indexer fp8 weight range h{h} {mode}] ok: worst score rel {w1:.2e}")
