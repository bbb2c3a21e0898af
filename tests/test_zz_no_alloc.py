"""GPU check of the no-allocation attention entry point against the workspace one.

sparse_gated_attn_fwd_noalloc runs the same kernels as sparse_gated_attn_fwd,
with its split partials in the library's static per-GPU scratch instead of a
caller workspace.  Both are called through the C ABI on the same inputs and
must agree bit for bit (outputs and log-sum-exp), on two calls in a row, the
second with a smaller batch than the first (the scratch keeps the first
call's contents), and on a batch without split lists (no scratch used).
"""
import numpy as np
import pytest
import torch

from tests import parity as P
from indexer_top_sparse_relu_amd import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from indexer_top_sparse_relu_amd import binding as B  # noqa: E402

DEV = "cuda"


def _both(spec):
    wl = W.generate(spec, DEV)
    pl = B.Pipeline(wl)
    pl.indexer()
    pl.topk()
    pl.attn(with_lse=True)
    out = torch.full_like(pl.out, float("nan"))
    lse = torch.full_like(pl.lse, float("nan"))
    B.sparse_gated_attn_fwd_noalloc(pl.batch, wl.q, wl.k_cache, wl.v_cache, spec.d_v, pl.indices, wl.gate, out,
                                    spec.softmax_scale, lse)
    torch.cuda.synchronize()
    need = B.sparse_gated_attn_workspace_size(pl.batch, spec.Hq, spec.d_v, spec.K)
    return pl, out, lse, need


def _same(pl, out, lse, tag):
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                       pl.out.view(torch.int16) if pl.out.dtype == torch.bfloat16 else pl.out.view(torch.int32)), \
        f"{tag}: outputs differ"
    assert torch.equal(lse.view(torch.int32), pl.lse.view(torch.int32)), f"{tag}: lse differs"


def test_noalloc_matches_workspace_entry_point_twice_then_smaller():
    big = W.long_decode_mla(B=16, lo=5000, hi=40000)
    small = W.decode_bf16(B=10, lo=300, hi=6000).replace(K=512, seed=71)
    sizes = []
    for tag, spec in (("first", big), ("second, smaller", small)):
        P.say(f"[noalloc {tag}] {spec.name} T={spec.T} Hq={spec.Hq} K={spec.K}")
        pl, out, lse, need = _both(spec)
        assert need > 0, "the batch must use split partials"
        sizes.append(need)
        _same(pl, out, lse, tag)
        assert np.isfinite(out.float().cpu().numpy()).all()
    assert sizes[1] < sizes[0]
    P.say(f"[noalloc] ok: scratch bytes {sizes[0]} then {sizes[1]}")


def test_noalloc_without_split_lists():
    spec = W.chunked_prefill_mla(cached=3000, T=600)       # 600 workgroups: no split lists
    pl, out, lse, need = _both(spec)
    assert need == 0
    _same(pl, out, lse, "prefill")


def test_noalloc_rejects_batches_beyond_its_scratch():
    spec = W.long_decode_mla(B=200, lo=100, hi=200, short_len=50, short_at=0)
    wl = W.generate(spec, DEV)
    pl = B.Pipeline(wl)
    assert B.sparse_gated_attn_workspace_size(pl.batch, spec.Hq, spec.d_v, spec.K) > (128 << 20)
    with pytest.raises(B.SparseAttnError) as e:
        B.sparse_gated_attn_fwd_noalloc(pl.batch, wl.q, wl.k_cache, wl.v_cache, spec.d_v, pl.indices, wl.gate,
                                        pl.out, spec.softmax_scale)
    assert e.value.status == B.SA_EWORKSPACE
