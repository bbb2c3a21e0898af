"""GPU Top-K on crafted score rows, bit-exact against the oracle's brute force.

The rows kernel and the chunked kernels try a single pass whose threshold comes
from a sample of 64 (128 on rows of 32K slots or more) runs of 64 consecutive
slots; when the kept count misses [K, capacity] they fall back to the general
selection.  Few long rows (k <= 2048) take a per-row threshold from 512 runs
instead, compact every chunk against it and finish per row, falling back to
the single-workgroup selection of the row.  These rows drive every branch:
plain random rows, constant rows and coarse alphabets (massive ties), ramps,
rows whose large values sit exactly on (or exactly off) the sampled runs of
either sample, and signed zeros.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from indexer_top_sparse_relu_amd import binding as B  # noqa: E402

DEV = "cuda"


def sample_runs(n):
    """Runs of 64 slots the single-pass sample reads: 64 runs, or 128 on rows of
    at least 32768 slots."""
    return 128 if n >= 32768 else 64


def sampled_mask(n, runs=None):
    """Slots a sample reads: run r starts at r*(n-64)//(runs-1) (the single pass's runs by default)."""
    runs = runs or sample_runs(n)
    m = np.zeros(n, bool)
    for r in range(runs):
        j = (r * (n - 64)) // (runs - 1)
        m[j:j + 64] = True
    return m


def pattern_row(kind, n, rng):
    if kind == "normal":
        return rng.standard_normal(n).astype(np.float32)
    if kind == "constant":
        return np.full(n, 1.25, np.float32)
    if kind == "alphabet":
        return rng.choice(np.array([-1.0, 0.0, 0.5, 2.0, 3.0], np.float32), n)
    if kind == "ramp":
        return (1.0 + np.arange(n) * 1e-6).astype(np.float32)
    if kind == "on_sample":
        v = rng.uniform(0.0, 1.0, n).astype(np.float32)
        m = sampled_mask(n)
        v[m] = rng.uniform(10.0, 11.0, int(m.sum())).astype(np.float32)
        return v
    if kind == "off_sample":
        v = rng.uniform(10.0, 11.0, n).astype(np.float32)
        m = sampled_mask(n)
        v[m] = rng.uniform(0.0, 1.0, int(m.sum())).astype(np.float32)
        return v
    if kind in ("on_sample512", "off_sample512"):
        hi, lo = (10.0, 0.0) if kind == "on_sample512" else (0.0, 10.0)
        v = rng.uniform(lo, lo + 1.0, n).astype(np.float32)
        m = sampled_mask(n, 512)
        v[m] = rng.uniform(hi, hi + 1.0, int(m.sum())).astype(np.float32)
        return v
    if kind == "signed_zero":
        v = rng.standard_normal(n).astype(np.float32)
        z = rng.random(n) < 0.5
        v[z] = np.where(rng.random(int(z.sum())) < 0.5, np.float32(0.0), np.float32(-0.0))
        v[v > 0] *= -1.0                       # the top K are all zeros of either sign
        return v
    if kind == "rounded":
        return np.round(rng.standard_normal(n), 2).astype(np.float32)
    raise ValueError(kind)


KINDS = ["normal", "constant", "alphabet", "ramp", "on_sample", "off_sample", "signed_zero", "rounded"]


def run_rows(lengths, kinds, K, seed):
    rng = np.random.default_rng(seed)
    Bn = len(lengths)
    n = np.asarray(lengths, np.int64)
    ld = int((n.max() + 63) // 64 * 64)
    sc = np.full((Bn, ld), np.nan, np.float32)
    for r in range(Bn):
        sc[r, :n[r]] = pattern_row(kinds[r % len(kinds)], int(n[r]), rng)
    # one query token per sequence: row r has n[r] causal candidates
    q_start = torch.arange(Bn + 1, dtype=torch.int32, device=DEV)
    ctx = torch.as_tensor(n.astype(np.int32), device=DEV)
    ps = 64
    max_pages = (ld + ps - 1) // ps
    pt = torch.zeros((Bn, max_pages), dtype=torch.int32, device=DEV)
    bt = B.make_batch(q_start, ctx, pt, total_q=Bn, max_q=1, max_ctx=int(n.max()), page_size=ps)
    scores = torch.as_tensor(sc, device=DEV)
    idx = torch.full((Bn, K), -7, dtype=torch.int32, device=DEV)
    wsb = B.sparse_topk_workspace_size(bt, K)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=DEV) if wsb else None
    B.sparse_topk(bt, scores, K, idx, ws)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    ref = O.topk(sc.astype(np.float64), n, K)
    for r in range(Bn):
        assert np.array_equal(got[r], ref[r]), f"row {r} ({kinds[r % len(kinds)]}, n={n[r]}) differs"
    P.check_idx_invariants(got, n, K)
    return wsb


def test_topk_rows_kernel_crafted_rows():
    """256 rows (the per-row kernel), lengths 9K-40K, every pattern."""
    rng = np.random.default_rng(7)
    lengths = rng.integers(9000, 40000, 256).tolist()
    P.say("[topk-rows] 256 rows, K=2048")
    wsb = run_rows(lengths, KINDS, 2048, seed=8)
    assert wsb == 0                       # 256 rows: no chunking


def test_topk_few_rows_crafted():
    """Fewer than 256 rows of 9K-40K (one launch: the single pass, and the general path in the same
    workgroup for the rows it cannot finish), every pattern."""
    rng = np.random.default_rng(17)
    lengths = rng.integers(9000, 40000, 96).tolist()
    P.say("[topk-few] 96 rows, K=2048")
    assert run_rows(lengths, KINDS, 2048, seed=18) == 0


def test_topk_chunked_crafted_rows():
    """Few long rows (sampled threshold, chunk compaction, per-row finish), every pattern."""
    lengths = [300000, 150001, 70000, 40960, 262144, 100000, 65537, 200000]
    P.say("[topk-chunked] 8 rows up to 300K, K=2048")
    wsb = run_rows(lengths, KINDS, 2048, seed=9)
    assert wsb > 0


@pytest.mark.parametrize("K", [1, 2048, 4096])
def test_topk_register_rows_crafted(K):
    """Rows of up to 8192 slots, one workgroup each with the row in registers (16 slots per
    thread): every pattern, rows shorter than K included; and 64 rows of up to 32768 (the single
    pass and the general path)."""
    rng = np.random.default_rng(20 + K)
    for hi, nrows in ((8192, 300), (32768, 64)):
        lengths = rng.integers(1, hi + 1, nrows).tolist()
        lengths[0], lengths[1] = hi, max(1, K - 1)
        P.say(f"[topk-reg] {nrows} rows up to {hi}, K={K}")
        assert run_rows(lengths, KINDS, K, seed=30 + K + hi) == 0


@pytest.mark.parametrize("K", [64, 4096])
def test_topk_chunked_long_rows_k(K):
    """Rows past 131072 slots (sampled from 512 runs), including rows made to fool that sample;
    k = 4096 takes the per-chunk selection and merge instead."""
    lengths = [1000003, 524288, 131072, 140000, 400000, 1000]
    kinds = ["normal", "on_sample512", "off_sample512", "rounded", "alphabet", "normal"]
    P.say(f"[topk-long] 6 rows up to 1M, K={K}")
    wsb = run_rows(lengths, kinds, K, seed=12 + K)
    assert wsb > 0


def test_topk_small_k_and_large_k():
    rng = np.random.default_rng(10)
    lengths = rng.integers(8192, 30000, 256).tolist()
    for K in (1, 64, 4096):
        P.say(f"[topk-k] K={K}")
        run_rows(lengths, KINDS, K, seed=11 + K)
