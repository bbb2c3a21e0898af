"""GPU parity of the backward over fixed indices against the oracle.

The forward runs on the GPU (its output and log-sum-exp feed the backward);
the oracle recomputes everything from the raw inputs in double.  Tolerance:
the GPU rounds P, dS and do to bf16 for the MFMAs and takes D from the bf16
forward output, so gradients are compared as 2-norms per (token, head) row
(d_q, per-channel d_gate) or per cache row (d_k, d_v) against the bf16
tolerance, with a floor of 1% of the largest reference row norm for rows
that are nearly zero; the per-head d_gate elementwise by the same rule.
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


def check_bwd(spec, tag):
    P.say(f"[{tag}] {spec.name} T={spec.T} B={spec.B} Hq={spec.Hq} d={spec.d_qk} K={spec.K} "
          f"{'shared' if spec.mla else 'separate'} cache, {'per-channel' if spec.gate_per_channel else 'per-head'} gate")
    wl = W.generate(spec, DEV)
    pl = B.Pipeline(wl)
    pl.indexer()
    pl.topk()
    pl.attn(with_lse=True)
    g = torch.Generator(device=DEV).manual_seed(spec.seed + 100)
    dy = torch.randn(pl.out.shape, device=DEV, generator=g).to(torch.bfloat16)
    shared = wl.v_cache.data_ptr() == wl.k_cache.data_ptr()
    rows = wl.k_cache.shape[0] * wl.k_cache.shape[1]
    dk = torch.zeros((wl.k_cache.shape[0], wl.k_cache.shape[1], wl.kv_row_stride), device=DEV)
    dv = dk if shared else torch.zeros_like(dk)
    dq = torch.full(wl.q.shape, float("nan"), device=DEV)
    dg = torch.full(wl.gate.shape, float("nan"), device=DEV)
    B.sparse_gated_attn_bwd(pl.batch, wl.q, wl.k_cache, wl.v_cache, spec.d_v, pl.indices, wl.gate, pl.out, pl.lse,
                            dy, dq, dk, dv, dg, softmax_scale=spec.softmax_scale)
    torch.cuda.synchronize()
    inp = O.Inputs.from_workload(wl)
    idx = pl.indices.cpu().numpy()
    rq, rk, rv, rg = O.sparse_attn_bwd(inp, idx, P.to_np(dy), scale=spec.softmax_scale)
    # d_q error model: D = d_out . out comes from the bf16 forward output, so dS_j = P_j (dP_j - D) carries an
    # error of up to 2^-8 * P_j * sum_c |d_out_c out_c|, and d_q = scale * sum_j dS_j K_j one of up to
    # 2^-8 * scale * sum_c |d_out_c out_c| * max_s |K_s| (P sums to 1).  A row whose exact gradient cancels
    # to near zero (a token with a single key has d_q = 0) is held to that absolute bound.
    y32 = pl.out.float().cpu().numpy().reshape(-1, spec.d_v)
    dy32 = dy.float().cpu().numpy().reshape(-1, spec.d_v)
    kmax = float(np.linalg.norm(wl.k_cache.float().cpu().numpy().reshape(-1, wl.kv_row_stride)[:, :spec.d_qk],
                                axis=1).max())
    model = 2.0 ** -8 * spec.softmax_scale * np.abs(dy32 * y32).sum(axis=1) * kmax / TOL
    w_q = rows_close(dq.cpu().numpy().reshape(-1, spec.d_qk), rq.reshape(-1, spec.d_qk), TOL, "d_q", model)
    touched = np.nonzero((rk != 0).any(axis=1) | (rv != 0).any(axis=1))[0]
    gk = dk.cpu().numpy().reshape(rows, -1)
    w_k = rows_close(gk[touched], rk[touched], TOL, "d_k")
    untouched = np.setdiff1d(np.arange(rows), touched)
    assert np.all(gk[untouched] == 0), "rows no token selected were written"
    if not shared:
        w_v = rows_close(dv.cpu().numpy().reshape(rows, -1)[touched], rv[touched], TOL, "d_v")
    else:
        w_v = w_k
    gg = dg.cpu().numpy()
    if spec.gate_per_channel:
        w_g = rows_close(gg.reshape(-1, spec.d_v), rg.reshape(-1, spec.d_v), TOL, "d_gate")
    else:
        # per head, d_gate = (1 - g) * sum_c d_out_c out_c cancels like D: the bf16 forward output bounds its
        # error by 2^-8 * (1 - g) * sum_c |d_out_c out_c|
        rgf = rg.reshape(-1)
        gl = wl.gate.float().cpu().numpy().reshape(-1)
        model = 2.0 ** -8 * (1.0 - 1.0 / (1.0 + np.exp(-gl))) * np.abs(dy32 * y32).sum(axis=1) / TOL
        floor = np.maximum(0.01 * np.abs(rgf).max(), model)
        rel = np.abs(gg.reshape(-1) - rgf) / np.maximum(np.abs(rgf), floor)
        assert np.all(rel <= TOL), f"d_gate: worst rel {rel.max():.3g}"
        w_g = float(rel.max())
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
