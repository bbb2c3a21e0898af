"""The attention comparison rule itself, on the CPU.

The GPU parity tests hold every attention output element to
|y - r| <= rtol |r| + E with E from an error model of the kernels' arithmetic
(tests/parity.py: attn_floor).  Here that rule is checked against an emulation
of the same arithmetic in numpy (fp32 logits and sums, weights rounded to bf16
before the weighted sum, output rounded to bf16): the emulation must pass, and
a single element moved by a few percent must fail even where the per-vector
2-norm rule alone would let it through.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import parity as P


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def _bf16_round(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def _case(seed, T=6, Hq=4, d=512, rows=300, K=64, q_gain=1.0):
    rng = np.random.default_rng(seed)
    q = _bf16_round(rng.standard_normal((T, Hq, d)) / np.sqrt(d) * q_gain)
    k = _bf16_round(rng.standard_normal((rows, d)) / np.sqrt(d))
    v = _bf16_round(rng.standard_normal((rows, d)) / np.sqrt(d))
    g = _bf16_round(rng.standard_normal((T, Hq, d)))
    idx = np.stack([np.sort(rng.choice(rows, size=K, replace=False)) for _ in range(T)]).astype(np.int32)
    idx[0, K - 5:] = -1                                 # a padded row
    ps = 64
    npg = (rows + ps - 1) // ps
    kc = np.zeros((npg * ps, d), np.float32)
    vc = np.zeros((npg * ps, d), np.float32)
    kc[:rows], vc[:rows] = k, v
    table = np.tile(np.arange(npg, dtype=np.int32), (T, 1))
    inp = O.Inputs(q_start=np.arange(T + 1, dtype=np.int32), ctx_len=np.full(T, rows, np.int32), page_table=table,
                   page_size=ps, idx_dtype="f32", attn_dtype="bf16", q_idx=np.zeros((T, 1, 16), np.float32),
                   q_scale=None, w=np.zeros((T, 1), np.float32), k_idx=np.zeros((npg * ps, 16), np.float32),
                   k_scale=None, q=_bf16_bits(q), k_cache=_bf16_bits(kc), v_cache=_bf16_bits(vc), gate=_bf16_bits(g),
                   H_I=1, d_I=16, Hq=Hq, d_qk=d, d_v=d, row_stride=d, gate_per_channel=True)
    return inp, q, kc, vc, g, idx


def _emulate(q, kc, vc, g, idx, scale):
    """The bf16 kernels' arithmetic in numpy: fp32 logits, fp32 weights rounded to bf16 for
    the weighted sum, fp32 normaliser of the unrounded weights, fp32 gate, bf16 output."""
    T, Hq, d = q.shape
    y = np.zeros((T, Hq, d), np.float32)
    for t in range(T):
        sel = idx[t][idx[t] >= 0]
        K = kc[sel].astype(np.float32)
        V = vc[sel].astype(np.float32)
        for h in range(Hq):
            z = (K @ q[t, h].astype(np.float32)).astype(np.float32) * np.float32(scale)
            p = np.exp(z - z.max()).astype(np.float32)
            l = np.float32(p.sum(dtype=np.float32))
            o = (_bf16_round(p) @ V).astype(np.float32) / l
            y[t, h] = o * (np.float32(1.0) / (np.float32(1.0) + np.exp(-g[t, h].astype(np.float32))))
    return _bf16_round(y)


@pytest.mark.parametrize("seed,q_gain", [(1, 1.0), (2, 16.0), (3, 64.0)])
def test_emulated_bf16_kernel_arithmetic_meets_the_rule(seed, q_gain):
    inp, q, kc, vc, g, idx = _case(seed, q_gain=q_gain)
    scale = 1.0 / np.sqrt(inp.d_qk)
    ref = O.sparse_attn(inp, idx, None, scale)
    floor = P.attn_floor(inp, idx, None, scale)
    y = _emulate(q, kc, vc, g, idx, scale)
    worst = P.check_attn(y, ref, P.RTOL["bf16"], floor)
    assert worst < 1.0
    # the floor is the bf16 weight term plus fp32 terms that stay within a few percent
    # of it at these logit sizes (up to |z| ~ 3)
    A = P.attn_abs(inp, idx, None, scale)
    ratio = floor / np.maximum(A, 1e-300)
    assert np.all(ratio >= P.U_BF16) and np.all(ratio <= 1.1 * P.U_BF16)


def test_one_element_off_fails_the_elementwise_rule_but_not_the_norm():
    inp, q, kc, vc, g, idx = _case(4)
    scale = 1.0 / np.sqrt(inp.d_qk)
    ref = O.sparse_attn(inp, idx, None, scale)
    floor = P.attn_floor(inp, idx, None, scale)
    y = _emulate(q, kc, vc, g, idx, scale).astype(np.float64)
    t, h = 1, 2
    c = int(np.argmin(np.abs(ref[t, h])))               # a component that nearly cancels
    y[t, h, c] = ref[t, h, c] + 0.3 * np.abs(ref[t, h]).mean()
    rel = np.linalg.norm(y[t, h] - ref[t, h]) / np.linalg.norm(ref[t, h])
    assert rel < P.RTOL["bf16"]                          # the per-vector 2-norm alone would pass it
    with pytest.raises(AssertionError, match="elements outside"):
        P.check_attn(y, ref, P.RTOL["bf16"], floor)


def test_fused_floor_mixes_the_branch_floors_by_the_gate():
    inp, *_ = _case(5, T=3, Hq=2, d=64, rows=100, K=16)
    rng = np.random.default_rng(0)
    fa, fb = rng.random((3, 2, 64)), rng.random((3, 2, 64))
    a_abs, b_abs = rng.random((3, 2, 64)), rng.random((3, 2, 64))
    got = P.fused_floor(inp, fa, fb, a_abs, b_abs)
    gl = P._decode(inp.gate, "bf16").reshape(3, 2, 64)
    s = 1.0 / (1.0 + np.exp(-gl))
    want = s * (fa + P.U_BF16 * a_abs) + (1 - s) * (fb + P.U_BF16 * b_abs)
    np.testing.assert_allclose(got, want, rtol=1e-12)
