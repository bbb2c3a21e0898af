"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test ties one oracle function to a library routine, a closed form, an
invariant, a brute force on tiny inputs, or a printed code table, so that a
plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, a missed mask) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers

def mk(*, q_idx, w, k_idx, q_lens, ctx_lens, idx_dtype="f32", attn_dtype="f32", q=None, k_cache=None,
       v_cache=None, gate=None, q_scale=None, k_scale=None, page_size=4, page_table=None, Hq=1,
       d_qk=None, d_v=None, gate_per_channel=True):
    """Inputs over an identity (or given) page table; rows of caches are physical rows."""
    q_lens, ctx_lens = list(q_lens), list(ctx_lens)
    B = len(q_lens)
    q_start = np.zeros(B + 1, np.int32)
    q_start[1:] = np.cumsum(q_lens)
    if page_table is None:
        npg = [(L + page_size - 1) // page_size for L in ctx_lens]
        mp = max(npg)
        page_table = np.zeros((B, mp), np.int32)
        off = 0
        for b, n in enumerate(npg):
            page_table[b, :n] = np.arange(off, off + n)
            off += n
    T = int(q_start[-1])
    H_I, d_I = q_idx.shape[1], q_idx.shape[2]
    if q is None:
        d_qk = d_qk or 4
        d_v = d_v or 4
        rows = k_idx.shape[0]
        q = np.zeros((T, Hq, d_qk), np.float32)
        k_cache = np.zeros((rows, d_qk), np.float32)
        v_cache = np.zeros((rows, d_v), np.float32)
        gate = np.zeros((T, Hq, d_v), np.float32)
    return O.Inputs(q_start=q_start, ctx_len=np.array(ctx_lens, np.int32), page_table=page_table,
                    page_size=page_size, idx_dtype=idx_dtype, attn_dtype=attn_dtype, q_idx=q_idx,
                    q_scale=q_scale, w=w, k_idx=k_idx, k_scale=k_scale, q=q, k_cache=k_cache,
                    v_cache=v_cache, gate=gate, H_I=H_I, d_I=d_I, Hq=q.shape[1], d_qk=q.shape[2],
                    d_v=v_cache.shape[-1], row_stride=k_cache.shape[-1], gate_per_channel=gate_per_channel)


def attn_inputs(rng, T, L, Hq, d, dv, page_size=8, mla=False, dtype="f32", q_gain=1.0, per_channel=True,
                q_lens=None, ctx_lens=None):
    q_lens = q_lens or [T]
    ctx_lens = ctx_lens or [L]
    Ttot = sum(q_lens)
    rows = sum((c + page_size - 1) // page_size for c in ctx_lens) * page_size
    q = (rng.standard_normal((Ttot, Hq, d)) * q_gain / math.sqrt(d)).astype(np.float32)
    kc = (rng.standard_normal((rows, d)) / math.sqrt(d)).astype(np.float32)
    # K and V caches share one row stride (d); V occupies the first dv elements of its row
    vfull = kc if mla else (rng.standard_normal((rows, d)) / math.sqrt(dv)).astype(np.float32)
    vc = vfull[:, :dv]
    g = rng.standard_normal((Ttot, Hq, dv) if per_channel else (Ttot, Hq)).astype(np.float32)
    qi = np.zeros((Ttot, 1, 4), np.float32)
    ki = np.zeros((rows, 4), np.float32)
    inp = mk(q_idx=qi, w=np.ones((Ttot, 1), np.float32), k_idx=ki, q_lens=q_lens, ctx_lens=ctx_lens,
             q=q, k_cache=kc, v_cache=vfull, gate=g, page_size=page_size, gate_per_channel=per_channel)
    inp.d_v = dv
    return inp, q, kc, vc, g


def sdpa_gated(q, k, v, pos, gate, scale, per_channel=True):
    """torch SDPA (float64, CPU) over positions s <= pos[i], then * sigmoid(gate)."""
    qt = torch.from_numpy(q.astype(np.float64)).transpose(0, 1)          # [H, T, d]
    H = qt.shape[0]
    kt = torch.from_numpy(k.astype(np.float64))[None].expand(H, -1, -1)
    vt = torch.from_numpy(v.astype(np.float64))[None].expand(H, -1, -1)
    L = kt.shape[1]
    mask = torch.arange(L)[None, :] <= torch.from_numpy(np.asarray(pos))[:, None]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask[None], scale=scale)
    o = o.transpose(0, 1)                                                  # [T, H, dv]
    g = torch.sigmoid(torch.from_numpy(gate.astype(np.float64)))
    if not per_channel:
        g = g[..., None]
    return (o * g).numpy()


# ------------------------------------------------------------ decoding pins

def test_fp8_codes_match_ocp_table():
    tab = O.fp8_table()
    for line in open(os.path.join(GOLDEN, "e4m3fn_codes.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = tab[int(code, 16)]
        want = float(val)
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)


def test_fp8_table_matches_torch_decoding():
    tab = O.fp8_table()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(tab))
    assert np.array_equal(ref[~nan], tab[~nan])


def test_bf16_decoding_matches_torch_all_codes():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([O.bf16_value(int(b)) for b in bits[::97]])
    r = ref[::97]
    nan = np.isnan(r)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(r[~nan], got[~nan])


# -------------------------------------------------------------- indexer pins

def test_indexer_identity_relu_is_matmul():
    """H_I=1, w=1, positive entries: every dot is > 0, so ReLU is the identity
    and the causal score block equals the numpy product q k^T."""
    rng = np.random.default_rng(0)
    T, D = 13, 8
    q = rng.uniform(0.1, 1.0, (T, 1, D)).astype(np.float32)
    k = rng.uniform(0.1, 1.0, (16, D)).astype(np.float32)   # 4 pages of 4
    inp = mk(q_idx=q, w=np.ones((T, 1), np.float32), k_idx=k, q_lens=[T], ctx_lens=[T])
    sc = O.indexer(inp)
    ref = q[:, 0, :].astype(np.float64) @ k[:T].astype(np.float64).T
    tri = np.tril(np.ones((T, T), bool))
    assert np.allclose(sc[tri], ref[tri], rtol=1e-14, atol=0)
    assert np.all(np.isnan(sc[~tri]))          # nothing written past the causal boundary


def test_indexer_head_weights_reduce_to_weighted_query():
    """All dots positive: sum_h w[i,h] (q_h . k) = (sum_h w[i,h] q_h) . k (numpy einsum + matmul).
    T != H so a transposed w index cannot pass."""
    rng = np.random.default_rng(1)
    T, H, D = 7, 3, 5
    q = rng.uniform(0.1, 1.0, (T, H, D)).astype(np.float32)
    w = rng.uniform(0.0, 1.0, (T, H)).astype(np.float32)
    k = rng.uniform(0.1, 1.0, (8, D)).astype(np.float32)
    inp = mk(q_idx=q, w=w, k_idx=k, q_lens=[T], ctx_lens=[T])
    sc = O.indexer(inp)
    qbar = np.einsum("th,thd->td", w.astype(np.float64), q.astype(np.float64))
    ref = qbar @ k[:T].astype(np.float64).T
    tri = np.tril(np.ones((T, T), bool))
    assert np.allclose(sc[tri], ref[tri], rtol=1e-13, atol=0)


def test_indexer_relu_drops_negative_heads():
    """Head 1 is the negation of head 0, so its dot is -(dot of head 0) < 0 and
    contributes nothing: score = w0 * (q0 . k)."""
    rng = np.random.default_rng(2)
    T, D = 6, 4
    u = rng.uniform(0.1, 1.0, (T, D)).astype(np.float32)
    q = np.stack([u, -u], axis=1)
    w = rng.uniform(0.5, 1.0, (T, 2)).astype(np.float32)
    k = rng.uniform(0.1, 1.0, (8, D)).astype(np.float32)
    inp = mk(q_idx=q, w=w, k_idx=k, q_lens=[T], ctx_lens=[T])
    sc = O.indexer(inp)
    ref = w[:, :1].astype(np.float64) * (u.astype(np.float64) @ k[:T].astype(np.float64).T)
    tri = np.tril(np.ones((T, T), bool))
    assert np.allclose(sc[tri], ref[tri], rtol=1e-13, atol=0)


def test_indexer_weight_outside_relu():
    """A negative weight multiplies the rectified dot (w * ReLU(x) <= 0), it is not
    rectified itself (ReLU(w x) >= 0 would give 0 here)."""
    T, D = 3, 2
    q = np.ones((T, 1, D), np.float32)
    k = np.ones((4, D), np.float32)
    inp = mk(q_idx=q, w=-np.ones((T, 1), np.float32), k_idx=k, q_lens=[T], ctx_lens=[T])
    sc = O.indexer(inp)
    tri = np.tril(np.ones((T, T), bool))
    assert np.all(sc[tri] == -2.0)


def test_indexer_one_hot_by_inspection():
    """One-hot query heads and keys: dot(q_h, k_s) = [a_h == b_s]; the score is the sum of
    the weights of the heads whose one-hot position matches the key's."""
    D, H = 4, 3
    a = [0, 2, 2]               # head h points at dim a[h]
    w = np.array([[1.0, 10.0, 100.0]], np.float32)
    q = np.zeros((1, H, D), np.float32)
    for h in range(H):
        q[0, h, a[h]] = 1.0
    k = np.zeros((4, D), np.float32)
    for s, b in enumerate([2, 0, 3, 1]):
        k[s, b] = 1.0
    inp = mk(q_idx=q, w=w, k_idx=k, q_lens=[1], ctx_lens=[4])
    sc = O.indexer(inp)[0]
    assert list(sc) == [110.0, 1.0, 0.0, 0.0]


def test_indexer_homogeneity_and_sign():
    rng = np.random.default_rng(3)
    T, H, D = 9, 4, 6
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    w = rng.uniform(0, 1, (T, H)).astype(np.float32)
    k = rng.standard_normal((12, D)).astype(np.float32)
    base = O.indexer(mk(q_idx=q, w=w, k_idx=k, q_lens=[T], ctx_lens=[T]))
    tri = np.tril(np.ones((T, T), bool))
    assert np.all(base[tri] >= 0.0)                     # w >= 0 gives nonnegative scores
    w2 = O.indexer(mk(q_idx=q, w=w * 4, k_idx=k, q_lens=[T], ctx_lens=[T]))
    q2 = O.indexer(mk(q_idx=q * 2, w=w, k_idx=k, q_lens=[T], ctx_lens=[T]))
    assert np.allclose(w2[tri], 4 * base[tri], rtol=1e-12)
    assert np.allclose(q2[tri], 2 * base[tri], rtol=1e-12)


def test_indexer_fp8_scales_apply_to_the_dot():
    """fp8 codes with per-token scales: with positive codes, H=1 and w=1 the score is
    q_scale[i] * k_scale[s] * (decoded q . decoded k) (torch decoding + numpy matmul)."""
    rng = np.random.default_rng(4)
    T, D = 5, 16
    qc = rng.integers(0x08, 0x50, (T, 1, D)).astype(np.uint8)   # positive normal codes
    kc = rng.integers(0x08, 0x50, (8, D)).astype(np.uint8)
    qs = rng.uniform(0.5, 2.0, T).astype(np.float32)
    ks = rng.uniform(0.5, 2.0, 8).astype(np.float32)
    inp = mk(q_idx=qc, w=np.ones((T, 1), np.float32), k_idx=kc, q_lens=[T], ctx_lens=[T], idx_dtype="fp8",
             q_scale=qs, k_scale=ks)
    sc = O.indexer(inp)
    dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = (dec(qc)[:, 0, :] @ dec(kc[:T]).T) * qs[:, None].astype(np.float64) * ks[None, :T].astype(np.float64)
    tri = np.tril(np.ones((T, T), bool))
    assert np.allclose(sc[tri], ref[tri], rtol=1e-14)


def test_indexer_paging_and_ragged_positions():
    """Scores depend only on logical positions: the same logical keys behind a random page
    table give the same rows.  Sequence b's last query sees all ctx_len[b] positions; a
    prefill's first query sees one."""
    rng = np.random.default_rng(5)
    ps, D, H = 4, 3, 2
    q_lens, ctx_lens = [3, 1, 5], [7, 10, 5]
    T = sum(q_lens)
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    w = rng.uniform(0, 1, (T, H)).astype(np.float32)
    logical = [rng.standard_normal((L, D)).astype(np.float32) for L in ctx_lens]
    npg = [(L + ps - 1) // ps for L in ctx_lens]
    total = sum(npg)

    def lay(perm):
        kc = np.zeros((total * ps, D), np.float32)
        table = np.zeros((3, max(npg)), np.int32)
        off = 0
        for b, L in enumerate(ctx_lens):
            pages = perm[off:off + npg[b]]
            table[b, :npg[b]] = pages
            for s in range(L):
                kc[pages[s // ps] * ps + s % ps] = logical[b][s]
            off += npg[b]
        return mk(q_idx=q, w=w, k_idx=kc, q_lens=q_lens, ctx_lens=ctx_lens, page_size=ps, page_table=table)

    a = O.indexer(lay(np.arange(total)))
    b = O.indexer(lay(rng.permutation(total)))
    assert np.array_equal(np.isnan(a), np.isnan(b))
    assert np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])
    n = O.row_lengths(lay(np.arange(total)))
    q_start = np.concatenate([[0], np.cumsum(q_lens)])
    for bi in range(3):
        assert n[q_start[bi + 1] - 1] == ctx_lens[bi]
    assert n[q_start[2]] == 1                         # fresh prefill sequence: first query sees itself
    assert np.all(np.diff(n[q_start[0]:q_start[1]]) == 1)


def test_indexer_row_subset_equals_full_rows():
    rng = np.random.default_rng(6)
    T, H, D = 11, 2, 4
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    w = rng.uniform(0, 1, (T, H)).astype(np.float32)
    k = rng.standard_normal((12, D)).astype(np.float32)
    inp = mk(q_idx=q, w=w, k_idx=k, q_lens=[T], ctx_lens=[T])
    full = O.indexer(inp)
    rows = [10, 3, 0]
    sub = O.indexer(inp, rows)
    assert np.array_equal(np.nan_to_num(sub, nan=-7), np.nan_to_num(full[rows], nan=-7))


# ----------------------------------------------------------------- Top-K pins

def lexsort_topk(row, n, K):
    s = row[:n]
    order = np.lexsort((np.arange(n), -s))      # primary: score desc, secondary: position asc
    sel = np.sort(order[:min(K, n)])
    return np.concatenate([sel, -np.ones(K - sel.size, np.int64)])


@pytest.mark.parametrize("alphabet", [None, 5, 2])
def test_topk_matches_lexsort(alphabet):
    rng = np.random.default_rng(7)
    R, L, K = 40, 64, 9
    if alphabet is None:
        sc = rng.standard_normal((R, L))
    else:
        sc = rng.integers(0, alphabet, (R, L)).astype(np.float64) * 0.25 - 0.5
    n = rng.integers(1, L + 1, R)
    got = O.topk(sc, n, K)
    for r in range(R):
        assert np.array_equal(got[r], lexsort_topk(sc[r], n[r], K)), r


def test_topk_invariants_and_ties():
    rng = np.random.default_rng(8)
    R, L, K = 25, 200, 31
    sc = np.round(rng.standard_normal((R, L)), 1)          # heavy ties
    n = rng.integers(1, L + 1, R)
    idx = O.topk(sc, n, K)
    for r in range(R):
        v = idx[r][idx[r] >= 0]
        assert v.size == min(K, n[r])
        assert np.all(idx[r][v.size:] == -1)
        assert np.all(np.diff(v) > 0) and v.min() >= 0 and v.max() < n[r]
        unsel = np.setdiff1d(np.arange(n[r]), v)
        if unsel.size:
            thr = sc[r][v].min()
            assert sc[r][unsel].max() <= thr
            ties_out = unsel[sc[r][unsel] == thr]
            ties_in = v[sc[r][v] == thr]
            if ties_out.size:
                assert ties_in.max() < ties_out.min()      # lowest positions win ties


def test_topk_short_rows_take_everything_and_needle():
    sc = np.zeros((3, 50))
    sc[1, 37] = 1e9
    n = np.array([5, 50, 32])
    idx = O.topk(sc, n, 32)
    assert list(idx[0][:5]) == [0, 1, 2, 3, 4] and np.all(idx[0][5:] == -1)
    assert 37 in idx[1]
    assert list(idx[2]) == list(range(32))
    # all-equal row: the K lowest positions
    assert list(idx[1][idx[1] != 37]) == list(range(31))


def test_topk_signed_zero_ties_by_position():
    row = np.array([[0.0, -0.0, 0.0, -0.0, -1.0]])
    idx = O.topk(row, np.array([5]), 2)
    assert list(idx[0]) == [0, 1]


# ------------------------------------------------------------- attention pins

def test_sparse_attention_with_all_positions_equals_sdpa_and_dense():
    """K >= n: the sparse path over every causal position equals torch SDPA (float64, causal
    mask) times sigmoid(gate), and the separately written dense control oracle."""
    rng = np.random.default_rng(9)
    T, Hq, d, dv = 10, 3, 8, 6
    inp, q, kc, vc, g = attn_inputs(rng, T, T, Hq, d, dv, page_size=4)
    K = 16
    idx = np.full((T, K), -1, np.int32)
    for i in range(T):
        idx[i, :i + 1] = np.arange(i + 1)
    out = O.sparse_attn(inp, idx)
    dense = O.dense_attn(inp)
    ref = sdpa_gated(q, kc[:T], vc[:T], np.arange(T), g, 1 / math.sqrt(d))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-15)
    assert np.allclose(dense, ref, rtol=1e-12, atol=1e-15)


def test_mla_latent_row_serves_k_and_v():
    rng = np.random.default_rng(10)
    T, Hq, d, dv = 6, 2, 12, 8
    inp, q, kc, vc, g = attn_inputs(rng, T, T, Hq, d, dv, page_size=4, mla=True)
    idx = np.tile(np.arange(T, dtype=np.int32), (T, 1))
    for i in range(T):
        idx[i, i + 1:] = -1
    out = O.sparse_attn(inp, idx)
    ref = sdpa_gated(q, kc[:T], kc[:T, :dv], np.arange(T), g, 1 / math.sqrt(d))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-15)


def test_single_index_gives_gated_value_row():
    rng = np.random.default_rng(11)
    inp, q, kc, vc, g = attn_inputs(rng, 4, 8, 2, 8, 8, page_size=4, ctx_lens=[8], q_lens=[4])
    idx = np.array([[3], [0], [6], [7]], np.int32)
    out, lse = O.sparse_attn(inp, idx, with_lse=True)
    sig = torch.sigmoid(torch.from_numpy(g.astype(np.float64))).numpy()
    for i in range(4):
        s = idx[i, 0]
        assert np.allclose(out[i], vc[s].astype(np.float64)[None, :] * sig[i], rtol=1e-15, atol=0)
        z = (q[i].astype(np.float64) @ kc[s].astype(np.float64)) / math.sqrt(8)
        assert np.allclose(lse[i], z, rtol=1e-14)


def test_zero_query_is_mean_of_selected_rows_and_padding_is_ignored():
    rng = np.random.default_rng(12)
    inp, q, kc, vc, g = attn_inputs(rng, 2, 16, 2, 8, 4, page_size=4, ctx_lens=[16], q_lens=[2])
    inp.q[:] = 0.0
    idx = np.array([[1, 5, 9, -1, -1], [0, 14, -1, 2, -1]], np.int32)
    out, lse = O.sparse_attn(inp, idx, with_lse=True)
    sig = torch.sigmoid(torch.from_numpy(g.astype(np.float64))).numpy()
    for i in range(2):
        s = idx[i][idx[i] >= 0]
        assert np.allclose(out[i], vc[s].astype(np.float64).mean(0)[None] * sig[i], rtol=1e-14)
        assert np.allclose(lse[i], math.log(s.size), rtol=1e-14)


def test_index_order_does_not_matter():
    rng = np.random.default_rng(13)
    inp, *_ = attn_inputs(rng, 3, 40, 2, 8, 8, page_size=8, ctx_lens=[40], q_lens=[3], q_gain=6.0)
    idx = np.stack([rng.choice(38 + i, 12, replace=False) for i in range(3)]).astype(np.int32)
    a = O.sparse_attn(inp, idx)
    b = O.sparse_attn(inp, idx[:, ::-1].copy())
    assert np.allclose(a, b, rtol=1e-13, atol=1e-16)


def test_gate_limits():
    """G = 100: sigmoid rounds to 1 in double, so y is the ungated output; G = 0 halves it."""
    rng = np.random.default_rng(14)
    inp, q, kc, vc, g = attn_inputs(rng, 3, 12, 2, 8, 8, page_size=4, ctx_lens=[12], q_lens=[3])
    idx = np.array([[0, 3, 9], [1, 2, 10], [4, 5, 11]], np.int32)
    inp.gate[:] = 100.0
    ungated = O.sparse_attn(inp, idx)
    ref = np.zeros_like(ungated)
    for i in range(3):
        ref[i] = sdpa_gated(q[i:i + 1], kc[idx[i]], vc[idx[i]], [len(idx[i]) - 1],
                            np.full((1, 2, 8), 100.0, np.float32), 1 / math.sqrt(8))[0]
    assert np.allclose(ungated, ref, rtol=1e-13)
    inp.gate[:] = 0.0
    half = O.sparse_attn(inp, idx)
    assert np.array_equal(half, ungated * 0.5)


def test_per_head_gate_is_broadcast_per_channel_gate():
    rng = np.random.default_rng(15)
    a, q, kc, vc, gh = attn_inputs(rng, 3, 9, 2, 8, 8, page_size=4, ctx_lens=[9], q_lens=[3], per_channel=False)
    idx = np.array([[0, 1, 6], [2, 3, 7], [4, 5, 8]], np.int32)
    out_h = O.sparse_attn(a, idx)
    a.gate = np.ascontiguousarray(np.repeat(gh[:, :, None], 8, axis=2))
    a.gate_per_channel = True
    out_c = O.sparse_attn(a, idx)
    assert np.array_equal(out_h, out_c)


def test_sharp_softmax_matches_sdpa():
    """Large logits (q x 40): exercises the max subtraction."""
    rng = np.random.default_rng(16)
    T = 8
    inp, q, kc, vc, g = attn_inputs(rng, T, T, 2, 16, 8, page_size=4, q_gain=40.0)
    idx = np.full((T, T), -1, np.int32)
    for i in range(T):
        idx[i, :i + 1] = np.arange(i + 1)
    out = O.sparse_attn(inp, idx)
    ref = sdpa_gated(q, kc[:T], vc[:T], np.arange(T), g, 1 / math.sqrt(16))
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-15)


# -------------------------------------------------------------- end to end

def test_pipeline_with_k_at_least_context_is_dense_gated_attention():
    """Tiny causal prefill with K = T: selection keeps every causal position, so the pipeline
    equals dense causal gated attention (torch SDPA)."""
    import indexer_top_sparse_relu_amd.workloads as W
    spec = W.tiny_prefill_fp32().replace(q_lens=(64,), ctx_lens=(64,), K=64)
    wl = W.generate(spec, "cpu")
    inp = O.Inputs.from_workload(wl)
    sc, idx, out = O.pipeline(inp, spec.K)
    n = O.row_lengths(inp)
    for i in range(spec.T):
        assert np.array_equal(idx[i][:n[i]], np.arange(n[i])) and np.all(idx[i][n[i]:] == -1)
    kc = inp.k_cache.reshape(-1, spec.d_qk)
    vc = inp.v_cache.reshape(-1, spec.d_v)
    ref = sdpa_gated(inp.q, kc[:spec.T], vc[:spec.T], np.arange(spec.T), inp.gate, spec.softmax_scale)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-15)


def test_small_k_pipeline_selects_planted_needle():
    """A key row planted equal to a query's indexer heads scores highest and is selected."""
    import indexer_top_sparse_relu_amd.workloads as W
    spec = W.tiny_prefill_fp32().replace(q_lens=(48,), ctx_lens=(48,), K=8)
    wl = W.generate(spec, "cpu")
    inp = O.Inputs.from_workload(wl)
    i, s = 40, 3
    inp.k_idx.reshape(-1, spec.d_I)[s] = 10.0 * inp.q_idx[i].sum(0)
    sc, idx, _ = O.pipeline(inp, spec.K, rows=[i])
    assert s in idx[0]


# ------------------------------------------------ cache append + fp8 quantisation

def _fp8_finite_codes():
    tab = O.fp8_table()
    return [c for c in range(256) if not math.isnan(tab[c])], tab


def test_fp8_encode_round_trips_every_finite_code():
    codes, tab = _fp8_finite_codes()
    got = O.fp8_encode(np.array([tab[c] for c in codes], np.float32))
    # -0 keeps its sign bit; every other finite value encodes back to its own code
    assert list(got) == codes


def test_fp8_encode_midpoints_round_to_the_even_code():
    codes, tab = _fp8_finite_codes()
    pos = sorted(c for c in codes if c < 0x80)            # 0x00 .. 0x7E, ascending values
    for lo, hi in zip(pos[:-1], pos[1:]):
        mid = np.float32((tab[lo] + tab[hi]) / 2)          # exact: one bit more than e4m3 has
        assert float(mid) == (tab[lo] + tab[hi]) / 2
        even = lo if (lo & 1) == 0 else hi
        above = np.nextafter(mid, np.float32(np.inf))
        below = np.nextafter(mid, np.float32(0))
        got = O.fp8_encode([mid, above, below, -mid])
        assert list(got) == [even, hi, lo, even | 0x80], (lo, hi, float(mid))


def test_fp8_encode_matches_torch_in_range_and_saturates():
    rng = np.random.default_rng(7)
    y = np.concatenate([rng.uniform(-448, 448, 4000), rng.standard_normal(4000) * 0.01,
                        rng.standard_normal(2000) * 2.0 ** rng.integers(-12, 8, 2000)]).astype(np.float32)
    y = y[np.abs(y) <= 448]
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.fp8_encode(y), want)
    big = O.fp8_encode([448.0, 449.0, 463.9, 464.0, 1e30, -1e30, -500.0])
    assert list(big) == [0x7E] * 5 + [0xFE] * 2
    assert O.fp8_encode([np.nan])[0] == 0x7F


def test_quantize_rows_scale_and_codes_closed_forms():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((6, 64)).astype(np.float32)
    x[0] = 0.0                                          # zero row: scale 0, codes 0
    x[1, 5] = -448.0                                    # amax 448: scale exactly 1, codes = e4m3fn(x)
    x[1] = np.clip(x[1], -448, 448)
    codes, scales = O.quantize_rows(x, "f32")
    assert scales[0] == 0 and not codes[0].any()
    assert scales[1] == 1.0 and np.array_equal(codes[1], O.fp8_encode(x[1]))
    amax = np.abs(x).max(axis=1)
    assert np.array_equal(scales[2:], (amax[2:] / np.float32(448)).astype(np.float32))
    # every row reaches +-448 at its largest element
    tab = O.fp8_table()
    for r in range(2, 6):
        j = int(np.argmax(np.abs(x[r])))
        assert abs(tab[codes[r, j]]) == 448.0


def test_quantize_rows_power_of_two_invariance_and_error_bound():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((4, 128)) * 3).astype(np.float32)
    c0, s0 = O.quantize_rows(x, "f32")
    for k in (-20, -3, 5, 40):
        ck, sk = O.quantize_rows((x * np.float32(2.0 ** k)).astype(np.float32), "f32")
        assert np.array_equal(ck, c0) and np.array_equal(sk, (s0 * np.float32(2.0 ** k)).astype(np.float32))
    tab = O.fp8_table()
    deq = tab[c0] * s0[:, None]
    y = x / s0[:, None]
    normal = np.abs(y) >= 2.0 ** -6
    # half a step: 2^-4 relative in the normal range, 2^-10 * s below it
    assert np.all(np.abs(deq - x)[normal] <= (2.0 ** -4) * np.abs(x)[normal] * (1 + 1e-6))
    assert np.all(np.abs(deq - x)[~normal] <= (2.0 ** -10) * np.broadcast_to(s0[:, None], x.shape)[~normal] * 1.0001)


def test_quantize_rows_bf16_input_equals_f32_of_the_same_values():
    rng = np.random.default_rng(10)
    bits = (rng.integers(0, 2 ** 16, (3, 32)) & 0xFF7F | 0x3C00).astype(np.uint16)   # finite, moderate
    vals = np.array([[O.bf16_value(int(b)) for b in row] for row in bits], np.float32)
    cb, sb = O.quantize_rows(bits, "bf16")
    cf, sf = O.quantize_rows(vals, "f32")
    assert np.array_equal(cb, cf) and np.array_equal(sb, sf)


def test_cache_append_writes_the_rows_the_position_rule_names():
    # two sequences over 4-row pages with a shuffled page table:
    #   seq 0: ctx 6, 2 new tokens -> positions 4, 5; its pages are [3, 0] -> rows 0, 1
    #   seq 1: ctx 3, 3 new tokens -> positions 0, 1, 2; its page is [2]    -> rows 8, 9, 10
    q_start = np.array([0, 2, 5], np.int32)
    ctx_len = np.array([6, 3], np.int32)
    page_table = np.array([[3, 0], [2, 1]], np.int32)
    rows_expected = [0, 1, 8, 9, 10]
    R, dqk, dv, di = 16, 8, 4, 16
    rng = np.random.default_rng(11)
    k_new = rng.integers(0, 2 ** 16, (5, dqk)).astype(np.uint16)
    v_new = rng.integers(0, 2 ** 16, (5, dv)).astype(np.uint16)
    kidx = (rng.standard_normal((5, di)) * 2).astype(np.float32)
    k_cache = np.full((R, dqk), 7, np.uint16)
    v_cache = np.full((R, dqk), 9, np.uint16)
    kic = np.full((R, di), 5, np.uint8)
    ksc = np.full(R, -1.0, np.float32)
    O.cache_append(q_start=q_start, ctx_len=ctx_len, page_table=page_table, page_size=4, kv_dtype="bf16",
                   k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, src_dtype="f32",
                   k_idx_new=kidx, idx_dtype="fp8", k_idx_cache=kic, k_scale_cache=ksc)
    codes, scales = O.quantize_rows(kidx, "f32")
    for i, r in enumerate(rows_expected):
        assert np.array_equal(k_cache[r], k_new[i])
        assert np.array_equal(v_cache[r, :dv], v_new[i]) and np.all(v_cache[r, dv:] == 9)
        assert np.array_equal(kic[r], codes[i]) and ksc[r] == scales[i]
    others = [r for r in range(R) if r not in rows_expected]
    assert np.all(k_cache[others] == 7) and np.all(v_cache[others] == 9)
    assert np.all(kic[others] == 5) and np.all(ksc[others] == -1.0)


def test_cache_append_copies_same_dtype_keys_and_skips_v_for_latent_rows():
    q_start = np.array([0, 1], np.int32)
    ctx_len = np.array([5], np.int32)
    page_table = np.array([[0, 1]], np.int32)         # identity: position 4 -> row 4
    k_cache = np.zeros((8, 6), np.float32)
    kic = np.zeros((8, 4), np.uint16)
    k_new = np.arange(6, dtype=np.float32)[None] + 1
    kidx = np.array([[1, 2, 3, 4]], np.uint16)
    O.cache_append(q_start=q_start, ctx_len=ctx_len, page_table=page_table, page_size=4, kv_dtype="f32",
                   k_new=k_new, v_new=None, k_cache=k_cache, v_cache=k_cache, src_dtype="bf16",
                   k_idx_new=kidx, idx_dtype="bf16", k_idx_cache=kic)
    assert np.array_equal(k_cache[4], k_new[0]) and not np.delete(k_cache, 4, axis=0).any()
    assert np.array_equal(kic[4], kidx[0]) and not np.delete(kic, 4, axis=0).any()


# ------------------------------------------------------ block-level selection

def _paged_attn_inputs(rng, q_lens, ctx_lens, ps, Hq=3, d=8, dv=8, shuffle=True):
    """f32 attention inputs over a shuffled page table (rows of the caches are physical rows)."""
    B_ = len(q_lens)
    npg = [(L + ps - 1) // ps for L in ctx_lens]
    perm = rng.permutation(sum(npg)) if shuffle else np.arange(sum(npg))
    pt = np.zeros((B_, max(npg)), np.int32)
    off = 0
    for b, n in enumerate(npg):
        pt[b, :n] = perm[off:off + n]
        off += n
    inp, q, kc, vc, g = attn_inputs(rng, 0, 0, Hq, d, dv, page_size=ps, q_lens=list(q_lens),
                                    ctx_lens=list(ctx_lens))
    inp.page_table = np.ascontiguousarray(pt)
    inp._bt = O._Batch(inp.B, ps, int(pt.shape[1]), 0, inp.q_start.ctypes.data, inp.ctx_len.ctypes.data,
                       inp.page_table.ctypes.data)
    return inp


def test_block_pool_is_the_mean_of_the_blocks_valid_rows():
    rng = np.random.default_rng(40)
    inp = _paged_attn_inputs(rng, [3, 2], [13, 6], ps=4)
    kc = inp.k_cache.reshape(-1, inp.row_stride)
    kbar = O.block_pool(inp)
    for b, L in enumerate(inp.ctx_len):
        for j in range((L + 3) // 4):
            page = inp.page_table[b, j]
            n = min(4, L - 4 * j)
            want = kc[page * 4: page * 4 + n, :inp.d_qk].astype(np.float64).mean(axis=0)
            assert np.allclose(kbar[page], want, rtol=1e-14, atol=1e-15), (b, j)
    # rows past a sequence's end do not enter its last block
    page = inp.page_table[0, 3]                 # positions 12..15 of seq 0; only 12 is valid
    kc[page * 4 + 1: page * 4 + 4] = 1e30
    assert np.allclose(O.block_pool(inp)[page], kc[page * 4, :inp.d_qk])


def test_block_scores_sum_of_head_dots_over_candidate_blocks():
    rng = np.random.default_rng(41)
    inp = _paged_attn_inputs(rng, [5, 1], [11, 9], ps=4, Hq=3)
    kbar = O.block_pool(inp)
    sc = O.block_scores(inp, kbar, ld=8)
    nb = O.block_row_lengths(inp)
    pos = O.row_lengths(inp) - 1
    assert list(nb) == [p // 4 + 1 for p in pos]
    qbar = inp.q.astype(np.float64).sum(axis=1)                     # [T, d]
    for i in range(inp.T):
        b = 0 if i < 5 else 1
        pages = inp.page_table[b, :nb[i]]
        want = kbar[pages] @ qbar[i]                                 # numpy matmul of the same operands
        assert np.allclose(sc[i, :nb[i]], want, rtol=1e-12, atol=1e-14)
        assert np.all(np.isnan(sc[i, nb[i]:]))


def test_block_expand_hand_example():
    rng = np.random.default_rng(42)
    inp = _paged_attn_inputs(rng, [1], [10], ps=4)                   # pos = 9: blocks 0, 1, 2 (2 is partial)
    blk = np.array([[0, 2, -1]], np.int32)
    got = O.block_expand(inp, blk)
    assert list(got[0]) == [0, 1, 2, 3, 8, 9] + [-1] * 6


def test_block_pipeline_with_every_block_is_dense_gated_attention():
    """kb >= the number of blocks keeps every causal position: block-sparse attention equals dense causal
    gated attention (written separately in the oracle) and torch SDPA."""
    rng = np.random.default_rng(43)
    inp = _paged_attn_inputs(rng, [6, 3], [23, 10], ps=4, Hq=2, d=8, dv=8)
    sc, blk, idx, out = O.block_pipeline(inp, kb=8, scale=0.3)
    dense = O.dense_attn(inp, scale=0.3)
    assert np.allclose(out, dense, rtol=1e-12, atol=1e-15)
    n = O.row_lengths(inp)
    for i in range(inp.T):
        assert sorted(idx[i][idx[i] >= 0]) == list(range(n[i]))


def test_block_pipeline_selects_the_planted_block():
    """One block's keys point along every query's head sum: with kb = 1 it is always chosen, and the
    attention runs over exactly its causal positions."""
    rng = np.random.default_rng(44)
    ps = 4
    inp = _paged_attn_inputs(rng, [4], [40], ps=ps, Hq=2, d=8, dv=8, shuffle=True)
    qbar = inp.q.sum(axis=1)
    u = qbar.mean(axis=0)
    kc = inp.k_cache.reshape(-1, inp.row_stride)
    page = inp.page_table[0, 5]                                      # block 5: positions 20..23
    kc[page * ps: page * ps + ps, :inp.d_qk] = 50.0 * u / np.linalg.norm(u)
    assert np.all(qbar @ u > 0)
    sc, blk, idx, out = O.block_pipeline(inp, kb=1, scale=0.3)
    assert np.all(blk[:, 0] == 5)
    assert np.all(idx[:, :ps] == np.arange(20, 24)) and np.all(idx[:, ps:] == -1)
    ref = O.sparse_attn(inp, np.tile(np.arange(20, 24, dtype=np.int32), (inp.T, 1)), scale=0.3)
    assert np.allclose(out, ref, rtol=0, atol=0)


# ------------------------------------------ branch fusion with a local branch

def test_window_indices_hand_example():
    rng = np.random.default_rng(50)
    inp = _paged_attn_inputs(rng, [3], [10], ps=4)          # positions 7, 8, 9
    got = O.window_indices(inp, 4)
    assert got.tolist() == [[4, 5, 6, 7], [5, 6, 7, 8], [6, 7, 8, 9]]
    inp2 = _paged_attn_inputs(rng, [2], [2], ps=4)          # positions 0, 1
    assert O.window_indices(inp2, 4).tolist() == [[0, -1, -1, -1], [0, 1, -1, -1]]


def test_window_attention_is_banded_causal_sdpa():
    """The local branch against torch SDPA with a banded causal mask (f32 inputs, float64 math)."""
    rng = np.random.default_rng(51)
    T, L, Hq, d, w = 12, 30, 2, 8, 5
    inp, q, kc, vc, g = attn_inputs(rng, T, L, Hq, d, d, page_size=8)
    u = O.ungated(inp)
    out = O.sparse_attn(u, O.window_indices(inp, w), scale=0.4)
    pos = np.arange(L - T, L)
    qt = torch.from_numpy(q.astype(np.float64)).transpose(0, 1)
    kt = torch.from_numpy(kc[:L].astype(np.float64))[None].expand(Hq, -1, -1)
    vt = torch.from_numpy(vc[:L].astype(np.float64))[None].expand(Hq, -1, -1)
    s = torch.arange(L)[None, :]
    p = torch.from_numpy(pos)[:, None]
    mask = (s <= p) & (s >= p - w + 1)
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask[None], scale=0.4).transpose(0, 1).numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_branch_fuse_limits_and_midpoint():
    rng = np.random.default_rng(52)
    inp, q, kc, vc, g = attn_inputs(rng, 4, 9, 2, 8, 8, page_size=4)
    a = rng.standard_normal((4, 2, 8))
    b = rng.standard_normal((4, 2, 8))
    for G, want in ((80.0, a), (-80.0, b), (0.0, (a + b) / 2)):
        inp.gate = np.full_like(inp.gate, G)
        assert np.allclose(O.branch_fuse(inp, a, b), want, rtol=1e-15, atol=1e-30), G
    # per-head gate broadcasts over channels
    inp.gate = rng.standard_normal((4, 2)).astype(np.float32)
    inp.gate_per_channel = False
    gg = 1.0 / (1.0 + np.exp(-inp.gate.astype(np.float64)))[..., None]
    assert np.allclose(O.branch_fuse(inp, a, b), gg * a + (1 - gg) * b, rtol=1e-14)


def test_fused_pipeline_with_full_branches_is_dense_attention():
    """K >= n and w >= n: both branches see every causal position, so any gate mix is dense attention."""
    import indexer_top_sparse_relu_amd.workloads as W
    spec = W.tiny_prefill_fp32().replace(q_lens=(48,), ctx_lens=(48,), K=48)
    inp = O.Inputs.from_workload(W.generate(spec, "cpu"))
    idx, a, b, y = O.fused_pipeline(inp, spec.K, 48, scale=spec.softmax_scale)
    dense = O.dense_attn(O.ungated(inp), scale=spec.softmax_scale)
    assert np.allclose(a, dense, rtol=1e-12, atol=1e-15) and np.allclose(b, dense, rtol=1e-12, atol=1e-15)
    assert np.allclose(y, dense, rtol=1e-12, atol=1e-15)


# ------------------------------------------------- backward over fixed indices

def _torch_gated_attn_grads(q, kc, vc, idx, gate, dy, scale, per_channel, same):
    """torch float64 autograd of y = softmax(scale q K_sel^T) V_sel * sigmoid(G), loss = sum(y * dy)."""
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(kc, dtype=torch.float64, requires_grad=True)
    vt = kt if same else torch.tensor(vc, dtype=torch.float64, requires_grad=True)
    gt = torch.tensor(gate, dtype=torch.float64, requires_grad=True)
    dv = dy.shape[-1]
    loss = 0.0
    for i in range(q.shape[0]):
        sel = torch.from_numpy(idx[i][idx[i] >= 0].astype(np.int64))
        if sel.numel() == 0:
            continue
        K_ = kt.index_select(0, sel)[:, :q.shape[2]]
        V_ = vt.index_select(0, sel)[:, :dv]
        p = torch.softmax(scale * qt[i] @ K_.T, dim=-1)               # [H, n]
        o = p @ V_                                                      # [H, dv]
        g = torch.sigmoid(gt[i] if per_channel else gt[i][:, None])
        loss = loss + (o * g * torch.from_numpy(dy[i].astype(np.float64))).sum()
    loss.backward()
    dk = kt.grad.numpy()
    return qt.grad.numpy(), dk, (dk if same else vt.grad.numpy()), gt.grad.numpy()


@pytest.mark.parametrize("per_channel,mla", [(True, False), (False, False), (True, True)])
def test_backward_matches_torch_autograd(per_channel, mla):
    rng = np.random.default_rng(60)
    T, Hq, d, dv = 5, 3, 8, 8 if not mla else 6
    inp, q, kc, vc, g = attn_inputs(rng, T, 20, Hq, d, dv, page_size=4, mla=mla, per_channel=per_channel)
    K = 7
    idx = np.full((T, K), -1, np.int32)
    n = O.row_lengths(inp)
    for i in range(T):
        m = min(K - 1, n[i])                               # leave at least one padding slot
        idx[i, :m] = np.sort(rng.choice(n[i], size=m, replace=False))
    dy = rng.standard_normal((T, Hq, dv)).astype(np.float32)
    dq, dk, dvv, dg = O.sparse_attn_bwd(inp, idx, dy, scale=0.35)
    kfull = inp.k_cache.reshape(-1, inp.row_stride)
    vfull = inp.v_cache.reshape(-1, inp.row_stride)
    tq, tk, tv, tg = _torch_gated_attn_grads(q, kfull, vfull, idx, inp.gate, dy, 0.35, per_channel, mla)
    assert np.allclose(dq, tq, rtol=1e-10, atol=1e-13)
    assert np.allclose(dk, tk, rtol=1e-10, atol=1e-13)
    assert np.allclose(dvv, tv, rtol=1e-10, atol=1e-13)
    assert np.allclose(dg, tg, rtol=1e-10, atol=1e-13)


def test_backward_of_a_single_index_is_the_gated_row():
    """K = 1: y = V[s] * sigmoid(G), so dq = 0, dK = 0, dV[s] = sum over tokens of dy * g."""
    rng = np.random.default_rng(61)
    T, Hq, d = 3, 2, 8
    inp, q, kc, vc, g = attn_inputs(rng, T, 10, Hq, d, d, page_size=4)
    idx = np.array([[4], [4], [6]], np.int32)
    dy = rng.standard_normal((T, Hq, d)).astype(np.float32)
    dq, dk, dvv, dg = O.sparse_attn_bwd(inp, idx, dy)
    sg = 1 / (1 + np.exp(-inp.gate.astype(np.float64)))
    assert np.allclose(dq, 0, atol=1e-15) and np.allclose(dk, 0, atol=1e-15)
    assert np.allclose(dvv[4, :d], (dy[0] * sg[0]).sum(0) + (dy[1] * sg[1]).sum(0), rtol=1e-12)
    assert np.allclose(dvv[6, :d], (dy[2] * sg[2]).sum(0), rtol=1e-12)
