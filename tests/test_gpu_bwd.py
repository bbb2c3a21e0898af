"""GPU parity of the backward over fixed indices against the oracle.

The forward runs on the GPU (its output and log-sum-exp feed the backward),
except for the head dimension the bf16 forward does not take (64), where the
oracle's forward, rounded to the types the forward would write, stands in.  The
oracle recomputes everything from the raw inputs in double.  Tolerance: the GPU
rounds P, dS and do to bf16 for the MFMAs and takes D from the bf16 forward
output, so gradients are compared as 2-norms per (token, head) row (d_q,
per-channel d_gate) or per cache row (d_k, d_v) against the bf16 tolerance,
with a floor of 1% of the largest reference row norm for rows that are nearly
zero; the per-head d_gate elementwise by the same rule.

The cases cover both ways the rows are merged: key-major (d = 64 or 128 with
16, 32 or 64 heads) and per-slot (the latent 576/512 layout, other head
counts), index lists longer than one pass of resolved rows, positions repeated
inside a row (counted once per slot, as in the forward), and the prefill
benchmark shape with the rows whose every selecting token the oracle can run.
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
TOL = P.RTOL["bf16"]


def rows_close(got, ref, tol, what, floor_rows=None):
    got = got.reshape(got.shape[0], -1).astype(np.float64)
    ref = ref.reshape(ref.shape[0], -1)
    rn = np.linalg.norm(ref, axis=1)
    err = np.linalg.norm(got - ref, axis=1)
    floor = 0.01 * rn.max() if rn.size else 0.0
    if floor_rows is not None:
        floor = np.maximum(floor, floor_rows)
    rel = err / np.maximum(rn, floor)
    assert np.all(rel <= tol), f"{what}: worst rel {rel.max():.3g} at row {int(rel.argmax())}"
    return float(rel.max()) if rel.size else 0.0


def forward(spec, mutate=None, oracle_fwd=False):
    """Workload, pipeline (indices on the GPU), forward output and lse, and a seeded upstream gradient."""
    wl = W.generate(spec, DEV)
    pl = B.Pipeline(wl)
    pl.indexer()
    pl.topk()
    if mutate is not None:
        mutate(pl.indices)
    if oracle_fwd:
        inp = O.Inputs.from_workload(wl)
        o, l = O.sparse_attn(inp, pl.indices.cpu().numpy(), None, spec.softmax_scale, with_lse=True)
        out = torch.from_numpy(o.astype(np.float32)).to(DEV).to(torch.bfloat16)
        lse = torch.from_numpy(l.astype(np.float32)).to(DEV)
    else:
        pl.attn(with_lse=True)
        out, lse = pl.out, pl.lse
    g = torch.Generator(device=DEV).manual_seed(spec.seed + 100)
    dy = torch.randn(out.shape, device=DEV, generator=g).to(torch.bfloat16)
    return wl, pl, out, lse, dy


def backward(spec, wl, pl, out, lse, dy):
    shared = wl.v_cache.data_ptr() == wl.k_cache.data_ptr()
    dk = torch.zeros((wl.k_cache.shape[0], wl.k_cache.shape[1], wl.kv_row_stride), device=DEV)
    dv = dk if shared else torch.zeros_like(dk)
    dq = torch.full(wl.q.shape, float("nan"), device=DEV)
    dg = torch.full(wl.gate.shape, float("nan"), device=DEV)
    B.sparse_gated_attn_bwd(pl.batch, wl.q, wl.k_cache, wl.v_cache, spec.d_v, pl.indices, wl.gate, out, lse,
                            dy, dq, dk, dv, dg, softmax_scale=spec.softmax_scale)
    torch.cuda.synchronize()
    rows = wl.k_cache.shape[0] * wl.k_cache.shape[1]
    return (dq.cpu().numpy(), dk.cpu().numpy().reshape(rows, -1), None if shared else dv.cpu().numpy().reshape(rows, -1),
            dg.cpu().numpy())


def dq_model(spec, wl, out, dy, toks):
    """d_q error model: D = d_out . out comes from the bf16 forward output, so dS_j = P_j (dP_j - D)
    carries an error of up to 2^-8 * P_j * sum_c |d_out_c out_c|, and d_q = scale * sum_j dS_j K_j one
    of up to 2^-8 * scale * sum_c |d_out_c out_c| * max_s |K_s| (P sums to 1).  A row whose exact
    gradient cancels to near zero (a token with a single key has d_q = 0) is held to that bound."""
    y32 = out.float().cpu().numpy()[toks].reshape(-1, spec.d_v)
    dy32 = dy.float().cpu().numpy()[toks].reshape(-1, spec.d_v)
    kmax = float(np.linalg.norm(wl.k_cache.float().cpu().numpy().reshape(-1, wl.kv_row_stride)[:, :spec.d_qk],
                                axis=1).max())
    return 2.0 ** -8 * spec.softmax_scale * np.abs(dy32 * y32).sum(axis=1) * kmax / TOL, y32, dy32


def check_gate(spec, wl, gg, rg, y32, dy32, toks):
    if spec.gate_per_channel:
        return rows_close(gg.reshape(-1, spec.d_v), rg.reshape(-1, spec.d_v), TOL, "d_gate")
    # per head, d_gate = (1 - g) * sum_c d_out_c out_c cancels like D: the bf16 forward output bounds its
    # error by 2^-8 * (1 - g) * sum_c |d_out_c out_c|
    rgf = rg.reshape(-1)
    gl = wl.gate.float().cpu().numpy()[toks].reshape(-1)
    model = 2.0 ** -8 * (1.0 - 1.0 / (1.0 + np.exp(-gl))) * np.abs(dy32 * y32).sum(axis=1) / TOL
    floor = np.maximum(0.01 * np.abs(rgf).max(), model)
    rel = np.abs(gg.reshape(-1) - rgf) / np.maximum(np.abs(rgf), floor)
    assert np.all(rel <= TOL), f"d_gate: worst rel {rel.max():.3g}"
    return float(rel.max())


def check_bwd(spec, tag, mutate=None, oracle_fwd=False):
    P.say(f"[{tag}] {spec.name} T={spec.T} B={spec.B} Hq={spec.Hq} d={spec.d_qk}/{spec.d_v} K={spec.K} "
          f"{'shared' if spec.mla else 'separate'} cache, {'per-channel' if spec.gate_per_channel else 'per-head'} gate")
    wl, pl, out, lse, dy = forward(spec, mutate, oracle_fwd)
    gq, gk, gv, gg = backward(spec, wl, pl, out, lse, dy)
    inp = O.Inputs.from_workload(wl)
    idx = pl.indices.cpu().numpy()
    rq, rk, rv, rg = O.sparse_attn_bwd(inp, idx, P.to_np(dy), scale=spec.softmax_scale)
    toks = np.arange(spec.T)
    model, y32, dy32 = dq_model(spec, wl, out, dy, toks)
    w_q = rows_close(gq.reshape(-1, spec.d_qk), rq.reshape(-1, spec.d_qk), TOL, "d_q", model)
    touched = np.nonzero((rk != 0).any(axis=1) | (rv != 0).any(axis=1))[0]
    w_k = rows_close(gk[touched], rk[touched], TOL, "d_k")
    untouched = np.setdiff1d(np.arange(gk.shape[0]), touched)
    assert np.all(gk[untouched] == 0), "rows no token selected were written"
    w_v = w_k if gv is None else rows_close(gv[touched], rv[touched], TOL, "d_v")
    w_g = check_gate(spec, wl, gg, rg, y32, dy32, toks)
    P.say(f"[{tag}] ok: worst rel d_q {w_q:.2e}, d_k {w_k:.2e}, d_v {w_v:.2e}, d_gate {w_g:.2e}")


def test_bwd_prefill_separate_caches_per_channel_gate():
    spec = W.prefill_bf16(T=200).replace(q_lens=(120, 80), ctx_lens=(400, 80), K=256, paged_random=True, seed=61)
    check_bwd(spec, "bwd-prefill")


def test_bwd_decode_per_head_gate_16_heads():
    spec = W.decode_bf16(B=6, lo=300, hi=3000).replace(K=512, Hq=16, gate_per_channel=False, seed=62)
    check_bwd(spec, "bwd-decode")


def test_bwd_shared_cache_64_heads():
    spec = W.prefill_bf16(T=96).replace(K=64, Hq=64, mla=True, seed=63)
    check_bwd(spec, "bwd-shared")


def test_bwd_48_heads_merged_per_slot():
    """48 heads: not a key-major shape, so every slot's dK, dV goes through the per-slot merge."""
    spec = W.prefill_bf16(T=90).replace(q_lens=(50, 40), ctx_lens=(700, 300), K=128, Hq=48, paged_random=True,
                                        seed=64)
    check_bwd(spec, "bwd-48")


@pytest.mark.parametrize("hq,mla", [(32, False), (16, True)])
def test_bwd_head_dim_64(hq, mla):
    """d = 64 (the oracle's forward stands in for the bf16 forward, which takes 128 and 576/512)."""
    spec = W.prefill_bf16(T=70).replace(q_lens=(70,), ctx_lens=(900,), d_qk=64, d_v=64, Hq=hq, mla=mla, K=160,
                                        paged_random=True, gate_per_channel=not mla, seed=65 + hq)
    check_bwd(spec, f"bwd-d64-h{hq}", oracle_fwd=True)


@pytest.mark.parametrize("hq", [16, 128])
def test_bwd_latent_layout(hq):
    """576/512 latent rows (V inside the K row), per-slot merge, 16 heads (one wave per group) and
    128 (two groups of 64)."""
    spec = W.chunked_prefill_mla(cached=700, T=24).replace(K=256, Hq=hq, gate_per_channel=(hq == 128),
                                                           seed=70 + hq)
    check_bwd(spec, f"bwd-latent-h{hq}")


def test_bwd_index_list_longer_than_one_pass():
    """k = 1500 > 1024 slots resolved per pass."""
    spec = W.prefill_bf16(T=40).replace(q_lens=(40,), ctx_lens=(3000,), K=1500, paged_random=True, seed=72)
    check_bwd(spec, "bwd-long-list")


def test_bwd_index_list_beyond_the_one_wave_dq_kernel():
    """32 heads x 128 with K = 2500: longer than the lists the one-wave-per-32-heads d_q kernel takes
    (2048), so d_q and the flagged repeats go through the query-major kernel in several passes."""
    spec = W.prefill_bf16(T=24).replace(q_lens=(24,), ctx_lens=(4000,), K=2500, paged_random=True, seed=74)
    check_bwd(spec, "bwd-long-list")


def test_bwd_rows_without_valid_slots_and_holes():
    """Rows whose list is all -1 (no key: lse = -inf, no gradient) and rows with -1 holes in the middle
    of the list (masked slots inside full tiles), on the one-wave-per-32-heads d_q kernel."""
    def mutate(idx):
        v = idx.clone()
        v[0:3, :] = -1
        v[3:9, 1::3] = -1
        idx.copy_(v)

    spec = W.prefill_bf16(T=72).replace(q_lens=(72,), ctx_lens=(900,), K=192, paged_random=True, seed=75)
    check_bwd(spec, "bwd-holes", mutate=mutate)


def test_bwd_repeated_positions():
    """Positions repeated inside a row: slot 1 repeats slot 0 on every row, slots 2 and 3 repeat slot 5
    on even rows.  The forward attends over every slot, so the backward counts each repeat once more:
    the key-major merge takes a position once and the flagged repeats go through the per-slot merge."""
    def mutate(idx):
        v = idx.clone()
        v[:, 1] = v[:, 0]
        v[0::2, 2] = v[0::2, 5]
        v[0::2, 3] = v[0::2, 5]
        idx.copy_(v)

    spec = W.prefill_bf16(T=100).replace(q_lens=(60, 40), ctx_lens=(500, 200), K=128, paged_random=True, seed=73)
    check_bwd(spec, "bwd-repeats", mutate=mutate)


def test_bwd_prefill_benchmark_shape_sampled():
    """The benchmark's backward shape (8192 tokens of one sequence, 32 heads x 128, K = 2048) at full
    size.  Causal lists mean a row at position p is selected only by tokens at p or later: the oracle
    runs the last 512 tokens, which covers every selector of the 512 rows at positions >= 7680 (four
    key blocks, two token chunks of the key-major kernel), and the first 64 tokens for d_q."""
    spec = W.prefill_bf16()
    P.say(f"[bwd-full] {spec.name} T={spec.T} Hq={spec.Hq} K={spec.K}")
    wl, pl, out, lse, dy = forward(spec)
    gq, gk, gv, gg = backward(spec, wl, pl, out, lse, dy)
    inp = O.Inputs.from_workload(wl)
    idx = pl.indices.cpu().numpy()
    dyr = P.to_np(dy)
    T, tail = spec.T, 512
    for first, n in ((T - tail, tail), (0, 64)):
        toks = np.arange(first, first + n)
        sub = P.sub_inputs(inp, 0, first, n)
        rq, rk, rv, rg = O.sparse_attn_bwd(sub, idx[toks], dyr[toks], scale=spec.softmax_scale)
        model, y32, dy32 = dq_model(spec, wl, out, dy, toks)
        w_q = rows_close(gq[toks].reshape(-1, spec.d_qk), rq.reshape(-1, spec.d_qk), TOL, "d_q", model)
        w_g = check_gate(spec, wl, gg[toks], rg, y32, dy32, toks)
        msg = f"tokens {first}..{first + n - 1}: d_q {w_q:.2e}, d_gate {w_g:.2e}"
        if first == T - tail:
            ps = inp.page_size
            pos = np.arange(T - tail, T)
            rows = inp.page_table[0, pos // ps].astype(np.int64) * ps + pos % ps
            w_k = rows_close(gk[rows], rk[rows], TOL, "d_k")
            w_v = rows_close(gv[rows], rv[rows], TOL, "d_v")
            msg += f", d_k {w_k:.2e}, d_v {w_v:.2e} on positions {T - tail}..{T - 1}"
        P.say(f"[bwd-full] ok: {msg}")
