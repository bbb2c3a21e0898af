"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small workloads are compared element by element on every row; the full-size
workloads (the shapes the benchmark times) on sampled rows that the oracle
computes one by one, plus properties that hold at any size.
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


def run(wl, stages=("indexer", "topk", "attn"), canary=True):
    pl = B.Pipeline(wl)
    if canary:
        pl.scores.fill_(float("nan"))
        pl.indices.fill_(-7)
        pl.out.fill_(float("nan"))
    for st in stages:
        P.say(f"  [{wl.spec.name}] launch {st}")
        getattr(pl, st)()
        torch.cuda.synchronize()
    return pl


def full_check(spec, tag, attn_rows=None):
    """Every row: scores, Top-K exactness, selection rule, invariants, attention, lse."""
    P.say(f"[{tag}] {spec.name} T={spec.T} B={spec.B} K={spec.K} max_ctx={spec.max_ctx}")
    wl = W.generate(spec, DEV)
    pl = run(wl)
    inp = O.Inputs.from_workload(wl)
    seq, pos, n = P.token_geometry(spec)
    sc_gpu = pl.scores.cpu().numpy()
    sc_ref = O.indexer(inp, ld=pl.ld)
    w1 = P.check_scores(sc_gpu, sc_ref, n, P.RTOL[spec.idx_dtype])
    # nothing written beyond each row's causal length
    for r in range(spec.T):
        assert np.all(np.isnan(sc_gpu[r, n[r]:])), f"row {r} written past n"
    idx = pl.indices.cpu().numpy()
    P.check_idx_invariants(idx, n, spec.K)
    P.check_topk_exact(idx, sc_gpu, n, spec.K)
    rec = P.check_selection(idx, sc_ref, n, spec.K)
    rows = np.arange(spec.T) if attn_rows is None else np.asarray(attn_rows)
    ref_out, ref_lse = O.sparse_attn(inp, idx[rows], rows, spec.softmax_scale, with_lse=True)
    out = pl.out.float().cpu().numpy()[rows]
    w2 = P.check_attn(out, ref_out, P.RTOL[spec.attn_dtype], P.attn_floor(inp, idx[rows], rows, spec.softmax_scale))
    lse = pl.lse.cpu().numpy()[rows]
    assert P.close(lse, ref_lse, P.RTOL[spec.attn_dtype]).all()
    P.say(f"[{tag}] ok: worst score rel {w1:.2e}, worst attn {w2:.2f} of the bound, recall {rec:.4f}")
    return wl, pl


# ------------------------------------------------------------------ tiny fp32

def test_tiny_prefill_fp32():
    full_check(W.tiny_prefill_fp32(), "tiny")


def test_tiny_prefill_fp32_sharp_softmax_and_per_head_gate():
    spec = W.tiny_prefill_fp32().replace(q_gain=4.0 * 8.0, gate_per_channel=False, seed=11)
    full_check(spec, "tiny-sharp")


def test_k_covering_context_equals_dense_control():
    """K >= every row's length: the path must equal dense causal gated attention."""
    spec = W.tiny_prefill_fp32().replace(K=256, seed=12)
    wl = W.generate(spec, DEV)
    pl = run(wl)
    inp = O.Inputs.from_workload(wl)
    dense = O.dense_attn(inp, scale=spec.softmax_scale)
    n = P.token_geometry(spec)[2]
    every = np.where(np.arange(spec.K)[None, :] < n[:, None], np.arange(spec.K)[None, :], -1)
    fl = P.attn_floor(inp, every, None, spec.softmax_scale)
    P.check_attn(pl.out.cpu().numpy(), dense, P.RTOL["f32"], fl, "dense control")


# ------------------------------------------------------------ prefill bf16

def test_prefill_bf16_ragged():
    spec = W.prefill_bf16(T=1000).replace(K=256)       # ragged against every tile size
    full_check(spec, "prefill-ragged")


def test_prefill_bf16_multi_sequence_per_head_gate():
    """Packed prefill of three sequences with cached prefixes (multi-turn concatenation)."""
    spec = W.prefill_bf16().replace(q_lens=(300, 17, 450), ctx_lens=(700, 17, 1200), K=128,
                                    gate_per_channel=False, paged_random=True, seed=21)
    full_check(spec, "prefill-multi")


def test_sequences_without_new_tokens():
    """Sequences with a cached context but no new tokens, first, between and last in the batch."""
    spec = W.prefill_bf16().replace(q_lens=(0, 90, 0, 41, 0), ctx_lens=(500, 90, 300, 700, 64), K=128,
                                    paged_random=True, seed=22)
    full_check(spec, "prefill-empty-seqs")


def test_decode_with_sequences_without_new_tokens():
    spec = W.decode_bf16(B=6, lo=100, hi=3000).replace(q_lens=(0, 1, 1, 0, 1, 0), K=512, seed=24)
    full_check(spec, "decode-empty-seqs")


def test_fp8_latent_with_sequences_without_new_tokens():
    spec = W.chunked_prefill_mla(cached=3000, T=333).replace(q_lens=(0, 200, 0, 133),
                                                            ctx_lens=(900, 3200, 64, 1500), seed=23)
    full_check(spec, "mla-empty-seqs", attn_rows=P.sample_tokens(333, 24, seed=23))


def test_prefill_bf16_full_size_sampled():
    spec = W.prefill_bf16()
    P.say(f"[prefill-full] {spec.name} T={spec.T}")
    wl = W.generate(spec, DEV)
    pl = run(wl, canary=False)
    seq, pos, n = P.token_geometry(spec)
    idx = pl.indices.cpu().numpy()
    sc_gpu = pl.scores.cpu().numpy()
    P.check_idx_invariants(idx, n, spec.K)
    rows = P.sample_tokens(spec.T, 256, seed=1, edge=64)
    P.check_topk_exact(idx[rows], sc_gpu[rows], n[rows], spec.K)
    srows = P.sample_tokens(spec.T, 24, seed=2)
    inp = P.indexer_inputs(wl, srows)
    ref = O.indexer(inp, ld=pl.ld)
    P.check_scores(sc_gpu[srows], ref, n[srows], P.RTOL["bf16"])
    P.check_selection(idx[srows], ref, n[srows], spec.K)
    arows = P.sample_tokens(spec.T, 16, seed=3)
    ainp, aidx = P.attn_inputs(wl, arows, idx[arows])
    ref_out = O.sparse_attn(ainp, aidx, None, spec.softmax_scale)
    P.check_attn(pl.out.float().cpu().numpy()[arows], ref_out, P.RTOL["bf16"],
                 P.attn_floor(ainp, aidx, None, spec.softmax_scale))


# ------------------------------------------------------------- decode bf16

def test_decode_bf16_full_size():
    full_check(W.decode_bf16(), "decode")


def test_decode_bf16_short_contexts():
    """Decode rows shorter than K (all positions taken, -1 padded) next to long ones."""
    spec = W.decode_bf16(B=8, lo=100, hi=5000).replace(K=1024, seed=31)
    full_check(spec, "decode-short")


# -------------------------------------------------------- MLA + fp8 indexer

def test_chunked_prefill_mla_reduced():
    spec = W.chunked_prefill_mla(cached=3000, T=333)
    full_check(spec, "mla-prefill-reduced", attn_rows=P.sample_tokens(333, 48, seed=4))


@pytest.mark.parametrize("h_i", [8, 16, 32])
def test_chunked_prefill_mla_fp8_indexer_head_counts(h_i):
    """fp8 indexer at other head counts: 8 (packed-fp16 epilogue), 16 (four tokens per
    wave, 32-row linear-term tile), 32 (two tokens per wave, 16-row linear-term tile)."""
    spec = W.chunked_prefill_mla(cached=3000, T=333).replace(H_I=h_i, seed=40 + h_i)
    full_check(spec, f"mla-prefill-h{h_i}", attn_rows=P.sample_tokens(333, 16, seed=8))


def test_chunked_prefill_mla_full_size_sampled():
    """The benchmark's own launch at full size: Top-K bit-exact on 512 rows (the first and
    last 64 among them), scores and the selection rule on 128 rows (first and last 16),
    attention element by element on 64 rows (first and last 16)."""
    spec = W.chunked_prefill_mla()
    P.say(f"[mla-prefill-full] T={spec.T} ctx={spec.max_ctx}")
    wl = W.generate(spec, DEV)
    pl = run(wl, canary=False)
    seq, pos, n = P.token_geometry(spec)
    idx = pl.indices.cpu().numpy()
    P.check_idx_invariants(idx, n, spec.K)
    rows = P.sample_tokens(spec.T, 512, seed=5, edge=64)
    for part in np.array_split(np.asarray(rows), 8):
        sc_rows = pl.scores[torch.as_tensor(part, device=DEV)].cpu().numpy()
        P.check_topk_exact(idx[part], sc_rows, n[part], spec.K)
    P.say(f"[mla-prefill-full] Top-K exact on {len(rows)} rows")
    inp = O.Inputs.from_workload(wl)
    srows = np.asarray(P.sample_tokens(spec.T, 128, seed=6, edge=16))
    ref = O.indexer(inp, rows=srows, ld=pl.ld)
    sc = pl.scores[torch.as_tensor(srows, device=DEV)].cpu().numpy()
    w1 = P.check_scores(sc, ref, n[srows], P.RTOL["fp8"])
    rec = P.check_selection(idx[srows], ref, n[srows], spec.K)
    P.say(f"[mla-prefill-full] scores and selection on {len(srows)} rows: worst rel {w1:.2e}, recall {rec:.4f}")
    arows = np.asarray(P.sample_tokens(spec.T, 64, seed=7, edge=16))
    ref_out = O.sparse_attn(inp, idx[arows], arows, spec.softmax_scale)
    w2 = P.check_attn(pl.out[torch.as_tensor(arows, device=DEV)].float().cpu().numpy(), ref_out, P.RTOL["bf16"],
                      P.attn_floor(inp, idx[arows], arows, spec.softmax_scale))
    P.say(f"[mla-prefill-full] ok: attention on {len(arows)} rows, worst {w2:.2f} of the bound")


@pytest.mark.parametrize("page_size", [64, 16])
def test_chunked_prefill_two_sequences_balanced_chunks(page_size):
    """Prefill key chunks sized on the mean causal limit, the last one open to each token's
    limit (long contexts: no rotation), in a batch whose longest query run and longest
    context belong to different sequences: scores, Top-K exactness and the selection rule
    on sampled rows of both."""
    spec = W.chunked_prefill_mla(cached=0, T=0).replace(q_lens=(48, 400), ctx_lens=(40000, 22000),
                                                        page_size=page_size, seed=90 + page_size)
    P.say(f"[mla-prefill-2seq-p{page_size}] T={spec.T} ctx={spec.ctx_lens}")
    wl = W.generate(spec, DEV)
    pl = run(wl, stages=("indexer", "topk"))
    seq, pos, n = P.token_geometry(spec)
    idx = pl.indices.cpu().numpy()
    P.check_idx_invariants(idx, n, spec.K)
    rows = np.asarray(sorted(set(P.sample_tokens(48, 12, seed=1, edge=3)) |
                             {48 + r for r in P.sample_tokens(400, 20, seed=2, edge=4)}))
    sc = pl.scores[torch.as_tensor(rows, device=DEV)].cpu().numpy()
    for i, r in enumerate(rows):
        assert np.all(np.isnan(sc[i, n[r]:])), f"row {r} written past n"
    P.check_topk_exact(idx[rows], sc, n[rows], spec.K)
    inp = O.Inputs.from_workload(wl)
    ref = O.indexer(inp, rows=rows, ld=pl.ld)
    w1 = P.check_scores(sc, ref, n[rows], P.RTOL["fp8"])
    rec = P.check_selection(idx[rows], ref, n[rows], spec.K)
    P.say(f"[mla-prefill-2seq-p{page_size}] ok on {len(rows)} rows: worst rel {w1:.2e}, recall {rec:.4f}")


def test_long_decode_mla_reduced_with_ties():
    spec = W.long_decode_mla(lo=5000, hi=40000)
    full_check(spec, "long-decode-reduced")


def test_ties_straddling_the_boundary():
    """Copies of the oracle's K-th ranked key row planted at 4 positions below and 4 above
    it: exact score ties across the selection boundary; lowest positions must win."""
    spec = W.long_decode_mla(B=4, lo=6000, hi=9000, short_at=1).replace(dup_frac=0.0, seed=41)
    wl = W.generate(spec, DEV)
    seq, pos, n = P.token_geometry(spec)
    inp = O.Inputs.from_workload(wl)
    ref = O.indexer(inp)
    kflat = wl.k_idx.view(-1, spec.d_I).view(torch.uint8)
    ksf = wl.k_scale.view(-1)
    for t in range(spec.T):
        if n[t] <= spec.K + 8:
            continue
        order = np.lexsort((np.arange(n[t]), -ref[t, :n[t]]))
        s_k = int(order[spec.K - 1])
        rows = P.logical_rows(wl, int(seq[t]), int(n[t]))
        for d in (-4, -3, -2, -1, 1, 2, 3, 4):
            s2 = min(max(s_k + d, 0), int(n[t]) - 1)
            kflat[rows[s2]] = kflat[rows[s_k]]
            ksf[rows[s2]] = ksf[rows[s_k]]
    pl = run(wl)
    inp = O.Inputs.from_workload(wl)
    ref = O.indexer(inp, ld=pl.ld)
    sc = pl.scores.cpu().numpy()
    idx = pl.indices.cpu().numpy()
    P.check_scores(sc, ref, n, P.RTOL["fp8"])
    P.check_topk_exact(idx, sc, n, spec.K)
    P.check_selection(idx, ref, n, spec.K)


def test_long_decode_mla_full_size_sampled():
    spec = W.long_decode_mla()
    P.say(f"[long-decode-full] B={spec.B} max_ctx={spec.max_ctx}")
    wl = W.generate(spec, DEV)
    pl = run(wl, canary=False)
    seq, pos, n = P.token_geometry(spec)
    idx = pl.indices.cpu().numpy()
    sc = pl.scores.cpu().numpy()
    P.check_idx_invariants(idx, n, spec.K)
    P.check_topk_exact(idx, sc, n, spec.K)
    short = int(np.argmin(n))
    longs = [int(t) for t in np.argsort(n) if n[t] > spec.K]
    srows = sorted({short, longs[0]})
    inp = P.indexer_inputs(wl, srows)
    ref = O.indexer(inp, ld=pl.ld)
    P.check_scores(sc[srows], ref, n[srows], P.RTOL["fp8"])
    P.check_selection(idx[srows], ref, n[srows], spec.K)
    arows = list(range(spec.T))
    ainp, aidx = P.attn_inputs(wl, arows, idx)
    ref_out = O.sparse_attn(ainp, aidx, None, spec.softmax_scale)
    w2 = P.check_attn(pl.out.float().cpu().numpy(), ref_out, P.RTOL["bf16"],
                      P.attn_floor(ainp, aidx, None, spec.softmax_scale))
    P.say(f"[long-decode-full] ok: worst attn {w2:.2f} of the bound")


# --------------------------------------------------------------- properties

def test_runs_are_bitwise_deterministic():
    spec = W.decode_bf16(B=16).replace(seed=51)
    wl = W.generate(spec, DEV)
    a = run(wl)
    b = run(wl)
    assert torch.equal(a.indices, b.indices)
    assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16))
    n = P.token_geometry(spec)[2]
    sa, sb = a.scores.cpu().numpy(), b.scores.cpu().numpy()
    for r in range(spec.T):
        assert np.array_equal(sa[r, :n[r]], sb[r, :n[r]])


# ------------------------------------------------- softmax reference bound

def _sharpen_to_last_selected(wl, pl, gain):
    """Point each query head at the key row of its highest selected position, scaled so
    that logit rises far (tens of nats) above those of the earlier keys."""
    spec = wl.spec
    idx = pl.indices.cpu().numpy()
    seq, pos, n = P.token_geometry(spec)
    kc = wl.k_cache.view(-1, wl.kv_row_stride)
    for t in range(spec.T):
        valid = idx[t][idx[t] >= 0]
        s_last = int(valid.max())
        row = P.logical_rows(wl, int(seq[t]), s_last + 1)[s_last]
        kv = kc[row, :spec.d_qk].float()
        q = kv / kv.norm() * gain
        wl.q[t] = q.to(wl.q.dtype).unsqueeze(0).expand(spec.Hq, -1)


@pytest.mark.parametrize("mode", ["prefill", "decode-split", "mqa-prefill", "mqa-shared-prefill"])
def test_latent_attention_logit_far_above_first_keys(mode):
    """A logit ~70 nats above the first tile's: the latent kernel (and the MQA kernel, with
    separate or shared K/V rows) must rerun with the exact maximum as its reference and still
    match the oracle."""
    if mode == "prefill":
        spec = W.chunked_prefill_mla(cached=3000, T=64).replace(seed=61)
    elif mode == "decode-split":
        spec = W.long_decode_mla(B=4, lo=5000, hi=9000, short_at=1).replace(seed=62)
    else:
        # 600 tokens x 32 heads: one wave per token, no split lists
        spec = W.prefill_bf16().replace(q_lens=(600,), ctx_lens=(3000,), K=256, paged_random=True,
                                        mla=(mode == "mqa-shared-prefill"), seed=63)
    P.say(f"[rerun-{mode}] T={spec.T} max_ctx={spec.max_ctx}")
    wl = W.generate(spec, DEV)
    pl = run(wl, stages=("indexer", "topk"))
    _sharpen_to_last_selected(wl, pl, gain=24.0 * 70.0)
    # the data must break the kernel's bound: some logit (log2 units) exceeds the
    # maximum over the first 32 selected keys by more than 64
    idx_t = pl.indices.long()
    seq, pos, n = P.token_geometry(spec)
    jump = 0.0
    for t in range(spec.T):
        sel = idx_t[t][idx_t[t] >= 0]
        rows = P.logical_rows(wl, int(seq[t]), int(n[t]))[sel]
        k = wl.k_cache.view(-1, wl.kv_row_stride)[rows, :spec.d_qk].float()
        z = (k @ wl.q[t, 0].float()) * spec.softmax_scale * 1.4426950408889634
        jump = max(jump, float(z.max() - z[:32].max()))
    assert jump > 64.0, jump
    pl.attn()
    torch.cuda.synchronize()
    rows = list(range(spec.T))
    idx = pl.indices.cpu().numpy()
    ainp, aidx = P.attn_inputs(wl, rows, idx)
    ref_out, ref_lse = O.sparse_attn(ainp, aidx, None, spec.softmax_scale, with_lse=True)
    out = pl.out.float().cpu().numpy()
    assert np.isfinite(out).all()
    w = P.check_attn(out, ref_out, P.RTOL["bf16"], P.attn_floor(ainp, aidx, None, spec.softmax_scale))
    assert P.close(pl.lse.cpu().numpy(), ref_lse, P.RTOL["bf16"]).all()
    P.say(f"[rerun-{mode}] ok: worst attn {w:.2f} of the bound")
