"""Comparison rules and host marshalling shared by the GPU parity tests.

Scores: |x - r| <= rtol * max(|r|, 0.01 * max_row |r|) on every entry of a
token's row, rtol 1e-5 (fp32) or 2e-2 (bf16/fp8).
Attention outputs, element by element: |y_c - r_c| <= rtol * |r_c| + E_c with
rtol 1e-5 (fp32) or 2e-2 (bf16), where E_c is the forward error bound of the
kernels' arithmetic (see attn_floor); and, as a second check, the relative
error of each (token, head) output vector in the 2-norm is at most rtol.
Top-K: bit-exact against the oracle's brute force on the GPU's own fp32
scores; against the oracle's double scores, the set must match wherever the
K-th/(K+1)-th gap exceeds 1e-3 relative, else every selected score must be at
least s_K - 1e-3 |s_K|.
"""
from __future__ import annotations

import copy
import sys

import numpy as np
import torch

from oracle import oracle as O

RTOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------------ rules

def close(x, r, rtol, floor=0.01):
    """Boolean mask of the tolerance rule along the last axis."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    rowmax = np.max(np.abs(r), axis=-1, keepdims=True)
    den = np.maximum(np.abs(r), floor * rowmax)
    return np.abs(x - r) <= rtol * den + 1e-300


def check_scores(gpu, ref, n, rtol, what="scores"):
    """gpu [R, >=max n] fp32, ref [R, >=max n] double; compare entries [0, n_r) of each row."""
    bad = 0
    worst = 0.0
    for r in range(len(n)):
        x, y = gpu[r, :n[r]], ref[r, :n[r]]
        ok = close(x, y, rtol)
        if not ok.all():
            bad += int((~ok).sum())
        rowmax = np.abs(y).max()
        worst = max(worst, float((np.abs(x - y) / np.maximum(np.abs(y), 0.01 * rowmax)).max()))
    assert bad == 0, f"{what}: {bad} entries outside rtol {rtol} (worst rel {worst:.3g})"
    return worst


def check_idx_invariants(idx, n, K):
    idx = np.asarray(idx)
    for r in range(idx.shape[0]):
        v = idx[r]
        c = min(K, int(n[r]))
        assert np.all(v[:c] >= 0) and np.all(v[c:] == -1), f"row {r}: padding layout"
        s = v[:c]
        assert np.all(np.diff(s) > 0), f"row {r}: not ascending/unique"
        assert s.size == 0 or (s[0] >= 0 and s[-1] < n[r]), f"row {r}: out of causal range"


def check_topk_exact(gpu_idx, gpu_scores, n, K):
    """Bit-exact Top-K of the GPU's own fp32 scores (oracle brute force on the same values)."""
    ref = O.topk(np.asarray(gpu_scores, np.float64), np.asarray(n, np.int64), K)
    diff = np.nonzero((ref != np.asarray(gpu_idx)).any(axis=1))[0]
    assert diff.size == 0, f"Top-K differs from brute force on rows {diff[:10].tolist()}"


def check_selection(gpu_idx, ref_scores, n, K, tol=1e-3):
    """The spec rule against the oracle's double scores; returns mean recall@K."""
    recalls = []
    for r in range(len(n)):
        nr = int(n[r])
        sel = np.asarray(gpu_idx[r][:min(K, nr)])
        if nr <= K:
            assert np.array_equal(sel, np.arange(nr))
            recalls.append(1.0)
            continue
        row = ref_scores[r, :nr]
        order = np.lexsort((np.arange(nr), -row))
        sK, sK1 = row[order[K - 1]], row[order[K]]
        ref_set = np.sort(order[:K])
        recalls.append(np.intersect1d(sel, ref_set).size / K)
        if sK - sK1 > tol * abs(sK):
            assert np.array_equal(sel, ref_set), f"row {r}: selection differs with a clear gap"
        else:
            assert np.all(row[sel] >= sK - tol * abs(sK)), f"row {r}: selected score below threshold"
    return float(np.mean(recalls))


U_BF16 = 2.0 ** -8      # unit roundoff of bf16 (8-bit significand, round to nearest even)
U_F32 = 2.0 ** -24      # unit roundoff of fp32


def _decode(raw, dtype):
    """Raw input elements (bf16 bits or fp32) to float64."""
    raw = np.asarray(raw)
    if dtype == "bf16":
        return (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return raw.astype(np.float64)


def _max_row_norm(raw, dtype, row_stride, d, chunk=1 << 18):
    """Largest 2-norm over the cache rows' first d elements (in chunks of rows)."""
    raw = np.asarray(raw).reshape(-1, row_stride)
    best = 0.0
    for r0 in range(0, raw.shape[0], chunk):
        k = _decode(raw[r0:r0 + chunk, :d], dtype)
        best = max(best, float(np.sqrt((k * k).sum(axis=1)).max()))
    return best


def attn_abs(inp, idx, rows=None, scale=None):
    """A [len(rows), Hq, d_v]: A_c = sum_j p_j |V[s_j, c]| * sigmoid(G_c), the oracle's own
    gated attention with every V element replaced by its magnitude (K is unchanged, so the
    weights p_j are the exact ones).  |o_c * sigmoid(G_c)| <= A_c."""
    rows = np.arange(inp.T) if rows is None else np.asarray(rows)
    scale = float(scale if scale is not None else 1.0 / np.sqrt(inp.d_qk))
    absv = copy.copy(inp)
    v = np.asarray(inp.v_cache)
    absv.v_cache = np.ascontiguousarray(v & np.uint16(0x7FFF) if inp.attn_dtype == "bf16" else np.abs(v))
    return O.sparse_attn(absv, np.asarray(idx), rows, scale)


def attn_floor(inp, idx, rows=None, scale=None):
    """Absolute part E [len(rows), Hq, d_v] of the attention tolerance: a first-order
    bound on the error of the kernels' arithmetic for every output element.

    With p_j the exact softmax weights over the valid entries s_j of a row (n of them)
    and A_c from attn_abs:
      * the bf16 kernels round every p_j to bf16 before the P.V product: relative
        error u_p = 2^-8 per weight (0 for the fp32 kernel);
      * the logit z_j = scale * q.K_j is an fp32 dot of d_qk products, then scaled and
        offset by the softmax reference: absolute error eps_z <= (d_qk + 8) u32 Z +
        4 u32 with Z = scale |q| max_s |K_s| (Cauchy-Schwarz), which perturbs each
        p_j by a relative eps_z;
      * the weighted sum and the normaliser l = sum_j p_j are fp32 sums of n terms:
        relative (n + 2) u32 each.
    A relative error of at most d on every weight moves o = sum_j p_j V_j / l by at most
    d A_c through the numerator and d |o_c| <= d A_c through l, so
        E_c = (u_p + 2 eps_z + 2 (n + 2) u32) A_c.
    The gate's fp32 sigmoid and the final rounding of y to the output type are relative
    to |y_c| and sit inside rtol * |r_c|.  Near zero, where components of o cancel, E_c
    is what remains of the tolerance."""
    rows = np.arange(inp.T) if rows is None else np.asarray(rows)
    idx = np.asarray(idx)
    scale = float(scale if scale is not None else 1.0 / np.sqrt(inp.d_qk))
    A = attn_abs(inp, idx, rows, scale)
    q = _decode(inp.q, inp.attn_dtype).reshape(inp.T, inp.Hq, inp.d_qk)[rows]
    kmax = _max_row_norm(inp.k_cache, inp.attn_dtype, inp.row_stride, inp.d_qk)
    zmax = scale * np.linalg.norm(q, axis=-1) * kmax
    n = (idx >= 0).sum(axis=1).astype(np.float64)[:, None]
    u_p = U_BF16 if inp.attn_dtype == "bf16" else 0.0
    eps_z = (inp.d_qk + 8) * U_F32 * zmax + 4 * U_F32
    coef = u_p + 2.0 * eps_z + 2.0 * (n + 2.0) * U_F32
    return coef[..., None] * A


def check_attn(gpu_out, ref_out, rtol, floor, what="attention"):
    """Element by element |y - r| <= rtol |r| + floor (floor from attn_floor), and the
    relative error of every (token, head) output vector in the 2-norm <= rtol.
    Returns the worst elementwise ratio |y - r| / (rtol |r| + floor)."""
    x = np.asarray(gpu_out, np.float64)
    r = np.asarray(ref_out, np.float64)
    f = np.broadcast_to(np.asarray(floor, np.float64), r.shape)
    err = np.abs(x - r)
    bound = rtol * np.abs(r) + f
    ratio = err / np.maximum(bound, 1e-300)
    bad = ~(err <= bound)
    if bad.any():
        w = np.unravel_index(int(np.argmax(np.where(np.isnan(ratio), np.inf, ratio))), r.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements outside rtol {rtol} + error floor "
                             f"(worst at {tuple(int(a) for a in w)}: got {x[w]:.6g}, want {r[w]:.6g}, "
                             f"bound {bound[w]:.3g})")
    num = np.linalg.norm(x - r, axis=-1)
    den = np.linalg.norm(r, axis=-1)
    rel = num / np.maximum(den, 1e-300)
    badv = rel > rtol
    assert not badv.any(), (f"{what}: {int(badv.sum())} of {badv.size} vectors above rtol {rtol} in the 2-norm "
                            f"(worst {rel.max():.3g})")
    return float(ratio.max()) if ratio.size else 0.0


def fused_floor(inp, fa, fb, a_abs, b_abs, rows=None):
    """Error floor of y = g a + (1 - g) b computed from the two ungated branch outputs as
    stored (rounded to the output type, unit roundoff u_o): each branch carries its own
    floor (fa, fb) plus u_o times its A (a_abs, b_abs bound |a|, |b|), mixed by the same
    gate weights g and 1 - g, both in [0, 1]."""
    u_o = U_BF16 if inp.attn_dtype == "bf16" else U_F32
    return O.branch_fuse(inp, fa + u_o * a_abs, fb + u_o * b_abs, rows)


def epilogue_mix_floor(inp, fb, a, b_abs, rows=None):
    """Error floor of y = g a + (1 - g) o with the mix formed where the attention output
    is: `a` is an input (exact), o the unrounded attention (floor fb, |o| <= b_abs).  The
    attention's floor enters with weight 1 - g; the fp32 mix adds the sigmoid's error (its
    exponential's argument G log2(e) is rounded once, the rest a few ulps: (|G| + 4) u32
    relative) times |a - o|, and the subtraction and fused multiply-add, a few u32 of
    |a| + |o| more.  The rounding of y itself sits inside rtol |r|."""
    rows = np.arange(inp.T) if rows is None else np.asarray(rows)
    shape = (inp.T, inp.Hq, inp.d_v if inp.gate_per_channel else 1)
    gl = np.abs(_decode(inp.gate, inp.attn_dtype).reshape(shape)[rows])
    fmix = (gl + 8.0) * U_F32 * (np.abs(a) + b_abs)
    return O.branch_fuse(inp, np.zeros_like(fb), fb, rows) + fmix


def sub_inputs(inp, b, first, n):
    """Inputs holding only tokens first .. first+n-1 (global indices, all of sequence b) at their own
    positions: the sub-batch's context ends at the last of them."""
    q0, q1 = int(inp.q_start[b]), int(inp.q_start[b + 1])
    assert q0 <= first and first + n <= q1
    pos0 = int(inp.ctx_len[b]) - (q1 - q0) + (first - q0)
    rows = np.arange(first, first + n)
    return O.Inputs(q_start=np.array([0, n], np.int32), ctx_len=np.array([pos0 + n], np.int32),
                    page_table=inp.page_table[b:b + 1], page_size=inp.page_size, idx_dtype=inp.idx_dtype,
                    attn_dtype=inp.attn_dtype, q_idx=inp.q_idx[rows], q_scale=None if inp.q_scale is None
                    else inp.q_scale[rows], w=inp.w[rows], k_idx=inp.k_idx, k_scale=inp.k_scale, q=inp.q[rows],
                    k_cache=inp.k_cache, v_cache=inp.v_cache, gate=inp.gate[rows], H_I=inp.H_I, d_I=inp.d_I,
                    Hq=inp.Hq, d_qk=inp.d_qk, d_v=inp.d_v, row_stride=inp.row_stride,
                    gate_per_channel=inp.gate_per_channel)


# --------------------------------------------------------- host marshalling

def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def token_geometry(spec):
    """(sequence, position, n) of every token, from the layout convention."""
    seq, pos = [], []
    for b, (nq, L) in enumerate(zip(spec.q_lens, spec.ctx_lens)):
        for j in range(nq):
            seq.append(b)
            pos.append(L - nq + j)
    pos = np.array(pos, np.int64)
    return np.array(seq, np.int64), pos, pos + 1


def logical_rows(wl, b: int, n: int) -> torch.Tensor:
    """Physical cache rows of positions 0..n-1 of sequence b (device tensor)."""
    ps = wl.spec.page_size
    s = torch.arange(n, device=wl.page_table.device)
    return wl.page_table[b, s // ps].long() * ps + s % ps


def indexer_inputs(wl, toks):
    """Oracle inputs holding only what the indexer needs for the listed tokens: one
    sequence per token with that token as its last query, its logical key rows packed
    behind an identity page table.  Row r of the result is token toks[r]."""
    spec = wl.spec
    seq, pos, n = token_geometry(spec)
    ps = spec.page_size
    kr, ksr, ctx = [], [], []
    for t in toks:
        rows = logical_rows(wl, int(seq[t]), int(n[t]))
        pad = (-int(n[t])) % ps
        rows = torch.cat([rows, rows[:1].expand(pad)]) if pad else rows
        kr.append(wl.k_idx.view(-1, spec.d_I)[rows])
        if wl.k_scale is not None:
            ksr.append(wl.k_scale.view(-1)[rows])
        ctx.append(int(n[t]))
    toks_t = torch.as_tensor(np.asarray(toks), device=wl.q_idx.device)
    npg = [(c + ps - 1) // ps for c in ctx]
    table = np.zeros((len(toks), max(npg)), np.int32)
    off = 0
    for r, m in enumerate(npg):
        table[r, :m] = np.arange(off, off + m)
        off += m
    B = len(toks)
    z = np.zeros((B, 1, 16), np.float32)
    return O.Inputs(q_start=np.arange(B + 1, dtype=np.int32), ctx_len=np.array(ctx, np.int32), page_table=table,
                    page_size=ps, idx_dtype=spec.idx_dtype, attn_dtype="f32", q_idx=to_np(wl.q_idx[toks_t]),
                    q_scale=to_np(wl.q_scale[toks_t]) if wl.q_scale is not None else None,
                    w=to_np(wl.w[toks_t]), k_idx=to_np(torch.cat(kr)),
                    k_scale=to_np(torch.cat(ksr)) if ksr else None, q=z, k_cache=np.zeros((off * ps, 16), np.float32),
                    v_cache=np.zeros((off * ps, 16), np.float32), gate=np.zeros((B, 1, 16), np.float32),
                    H_I=spec.H_I, d_I=spec.d_I, Hq=1, d_qk=16, d_v=16, row_stride=16, gate_per_channel=True)


def attn_inputs(wl, toks, idx_rows):
    """Oracle inputs for attention of the listed tokens over their GPU index rows: the
    selected cache rows are packed per token (in index order) and the indices rewritten
    to those packed positions; padding (-1) stays padding."""
    spec = wl.spec
    seq, pos, n = token_geometry(spec)
    K = idx_rows.shape[1]
    ps = spec.page_size
    width = (K + ps - 1) // ps * ps
    kc_rows, new_idx = [], np.full((len(toks), K), -1, np.int32)
    rs = wl.kv_row_stride
    kflat = wl.k_cache.view(-1, rs)
    vflat = wl.v_cache.view(-1, rs)
    same = wl.v_cache.data_ptr() == wl.k_cache.data_ptr()
    vk_rows = []
    for r, t in enumerate(toks):
        sel = idx_rows[r]
        valid = sel[sel >= 0]
        rows = logical_rows(wl, int(seq[t]), int(n[t]))[torch.as_tensor(valid, device=wl.page_table.device).long()]
        pad = width - rows.numel()
        rows = torch.cat([rows, rows.new_zeros(pad)])
        kc_rows.append(kflat[rows])
        vk_rows.append(vflat[rows])
        new_idx[r, :valid.size] = np.arange(valid.size)
    toks_t = torch.as_tensor(np.asarray(toks), device=wl.q.device)
    B = len(toks)
    table = np.arange(B * (width // ps), dtype=np.int32).reshape(B, width // ps)
    kc = to_np(torch.cat(kc_rows))
    vc = kc if same else to_np(torch.cat(vk_rows))
    inp = O.Inputs(q_start=np.arange(B + 1, dtype=np.int32), ctx_len=np.full(B, width, np.int32), page_table=table,
                   page_size=ps, idx_dtype="f32", attn_dtype=spec.attn_dtype,
                   q_idx=np.zeros((B, 1, 16), np.float32), q_scale=None, w=np.zeros((B, 1), np.float32),
                   k_idx=np.zeros((B * width, 16), np.float32), k_scale=None, q=to_np(wl.q[toks_t]), k_cache=kc,
                   v_cache=vc, gate=to_np(wl.gate[toks_t]), H_I=1, d_I=16, Hq=spec.Hq, d_qk=spec.d_qk,
                   d_v=spec.d_v, row_stride=rs, gate_per_channel=spec.gate_per_channel)
    return inp, new_idx


def sample_tokens(T, k, seed=0, edge=4):
    """First/last `edge` tokens plus random ones, sorted, unique."""
    rng = np.random.default_rng(seed)
    base = set(range(min(edge, T))) | set(range(max(0, T - edge), T))
    rest = [t for t in range(T) if t not in base]
    extra = rng.choice(rest, size=min(len(rest), max(0, k - len(base))), replace=False) if rest else []
    return sorted(base | set(int(x) for x in extra))
