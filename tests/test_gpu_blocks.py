"""GPU parity of block-level selection against the oracle.

Each stage is checked on its own inputs, so that a mismatch names the stage:
pooled keys and block scores within fp32 tolerance of the oracle's doubles;
the block Top-K bit-exact against brute force on the GPU's own block scores
and, against the oracle's scores, identical wherever the gap rule decides;
the expansion bit-exact; the attention over the expanded positions within
the bf16 tolerance.
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
RTOL_BLOCK = 1e-4        # fp32 sums of bf16 values against the oracle's doubles


def run_blocks(wl, kb):
    s = wl.spec
    bt = B.batch_of(wl)
    n_pages = wl.k_cache.shape[0]
    kbar = torch.full((n_pages, s.d_qk), float("nan"), device=DEV)
    max_blocks = (s.max_ctx + s.page_size - 1) // s.page_size
    ld = (max_blocks + 3) // 4 * 4
    scores = torch.full((s.T, ld), float("nan"), device=DEV)
    ws = torch.empty(B.sparse_block_scores_workspace_size(bt, s.d_qk), dtype=torch.uint8, device=DEV)
    blk = torch.full((s.T, kb), -7, dtype=torch.int32, device=DEV)
    tws = B.sparse_block_topk_workspace_size(bt, kb)
    tws = torch.empty(tws, dtype=torch.uint8, device=DEV) if tws else None
    idx = torch.full((s.T, kb * s.page_size), -7, dtype=torch.int32, device=DEV)
    out = torch.full((s.T, s.Hq, s.d_v), float("nan"), device=DEV).to(wl.q.dtype)
    P.say(f"  [{s.name}] block pool / scores / topk / expand / attention, kb={kb}")
    B.sparse_block_pool(bt, wl.k_cache, s.d_qk, kbar)
    B.sparse_block_scores(bt, wl.q, kbar, scores, ws)
    B.sparse_block_topk(bt, scores, kb, blk, tws)
    B.sparse_block_expand(bt, blk, idx)
    aws = B.sparse_gated_attn_workspace_size(bt, s.Hq, s.d_v, kb * s.page_size)
    aws = torch.empty(aws, dtype=torch.uint8, device=DEV) if aws else None
    B.sparse_gated_attn_fwd(bt, wl.q, wl.k_cache, wl.v_cache, s.d_v, idx, wl.gate, out,
                            softmax_scale=s.softmax_scale, workspace=aws)
    torch.cuda.synchronize()
    return kbar, scores, blk, idx, out


def check_blocks(spec, kb, tag, attn_rows=None):
    P.say(f"[{tag}] {spec.name} T={spec.T} B={spec.B} max_ctx={spec.max_ctx} kb={kb}")
    wl = W.generate(spec, DEV)
    kbar, scores, blk, idx, out = run_blocks(wl, kb)
    inp = O.Inputs.from_workload(wl)
    # pooled keys: the pages some sequence uses
    ref_kbar = O.block_pool(inp)
    used = ~np.isnan(ref_kbar[:, 0])
    got_kbar = kbar.cpu().numpy()
    assert np.allclose(got_kbar[used], ref_kbar[used], rtol=RTOL_BLOCK, atol=1e-6), "pooled keys"
    # block scores
    nb = O.block_row_lengths(inp)
    ref_sc = O.block_scores(inp, ref_kbar, ld=scores.shape[1])
    sc = scores.cpu().numpy()
    w1 = P.check_scores(sc, ref_sc, nb, RTOL_BLOCK, "block scores")
    for r in range(spec.T):
        assert np.all(np.isnan(sc[r, nb[r]:])), f"row {r} written past its candidate blocks"
    # block Top-K: exact on the GPU's own scores, the gap rule against the oracle's
    b_idx = blk.cpu().numpy()
    P.check_idx_invariants(b_idx, nb, kb)
    P.check_topk_exact(b_idx, sc, nb, kb)
    P.check_selection(b_idx, ref_sc, nb, kb)
    # expansion of the GPU's blocks
    e_idx = idx.cpu().numpy()
    assert np.array_equal(e_idx, O.block_expand(inp, b_idx)), "expanded positions"
    # attention over the GPU's expanded positions
    rows = np.arange(spec.T) if attn_rows is None else np.asarray(attn_rows)
    ref_out = O.sparse_attn(inp, e_idx[rows], rows, spec.softmax_scale)
    w2 = P.check_attn(out.float().cpu().numpy()[rows], ref_out, P.RTOL[spec.attn_dtype],
                      P.attn_floor(inp, e_idx[rows], rows, spec.softmax_scale))
    P.say(f"[{tag}] ok: worst block-score rel {w1:.2e}, worst attn {w2:.2f} of the bound")


def test_block_selection_latent_prefill():
    spec = W.chunked_prefill_mla(cached=3000, T=333)
    check_blocks(spec, kb=8, tag="blocks-mla", attn_rows=P.sample_tokens(333, 24, seed=9))


def test_block_selection_paged_decode_with_short_rows():
    """Decode over separate bf16 K/V caches: rows with fewer candidate blocks than kb are padded."""
    spec = W.decode_bf16(B=12, lo=100, hi=6000).replace(K=256, seed=41)
    check_blocks(spec, kb=16, tag="blocks-decode")


def test_block_selection_ragged_prefill_fp32():
    spec = W.tiny_prefill_fp32().replace(q_lens=(40, 70), ctx_lens=(300, 70), page_size=16, paged_random=True,
                                         seed=42)
    check_blocks(spec, kb=4, tag="blocks-f32")


def test_block_selection_long_context():
    """More than 128 candidate blocks per token: the scoring spans several column groups of workgroups."""
    spec = W.chunked_prefill_mla(cached=20000, T=70).replace(seed=43)
    check_blocks(spec, kb=8, tag="blocks-long", attn_rows=P.sample_tokens(70, 8, seed=10))


def test_block_selection_large_pages_two_sequences():
    """256-position blocks over a random page permutation, two ragged bf16 sequences with separate K/V caches."""
    spec = W.prefill_bf16(T=100).replace(q_lens=(37, 63), ctx_lens=(1500, 700), page_size=256, paged_random=True,
                                         seed=44)
    check_blocks(spec, kb=3, tag="blocks-p256")
