"""GPU parity of the cache append and the fp8 row quantiser against the oracle.

Codes, scales and every cache byte are compared exactly: the codes are
integers decided by fp32 arithmetic on both sides, and everything else is a
copy.  Untouched cache rows must keep their contents.
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


def raw(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy().copy()
    return t.numpy().copy()


def bf16_all_in_range() -> torch.Tensor:
    """Every finite bf16 value with |v| <= 448, as float32."""
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    bits = bits[torch.isfinite(bits) & (bits.abs() <= 448)]
    return bits


def check_quantize(x: torch.Tensor, tag: str):
    rows, cols = x.shape
    codes = torch.full((rows, cols), 0x55, dtype=torch.uint8, device=DEV)
    scales = torch.full((rows,), -1.0, dtype=torch.float32, device=DEV)
    P.say(f"[{tag}] quantize rows={rows} cols={cols} {x.dtype}")
    B.sparse_quantize_fp8_rows(x, codes, scales)
    torch.cuda.synchronize()
    want_c, want_s = O.quantize_rows(raw(x), "bf16" if x.dtype == torch.bfloat16 else "f32")
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:3].tolist()}: " \
        f"{[(int(got_c[r, c]), int(want_c[r, c])) for r, c in bad[:3]]}"
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32))


def test_quantize_every_bf16_value_with_unit_scale():
    """Rows that hold 448 have scale exactly 1, so each code is e4m3fn of the bf16 value
    itself: every representable bf16 in [-448, 448] (all ties included) once."""
    v = bf16_all_in_range()
    cols = 1024
    n = (v.numel() + cols - 2) // (cols - 1)
    pad = torch.zeros(n * (cols - 1) - v.numel())
    body = torch.cat([v, pad]).reshape(n, cols - 1)
    x = torch.cat([torch.full((n, 1), 448.0), body], dim=1).to(torch.bfloat16).to(DEV)
    check_quantize(x, "bf16-all")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_random_rows_of_many_magnitudes(dtype):
    g = torch.Generator().manual_seed(21)
    rows, cols = 96, 64 * 128
    x = torch.randn(rows, cols, generator=g)
    x *= torch.pow(2.0, torch.randint(-40, 40, (rows, 1), generator=g).float())
    x[0] = 0.0                                          # zero row
    x[1, :] = 0.0
    x[1, 7] = -3.0                                      # one nonzero element
    x[2] = torch.randn(cols, generator=g) * 1e-39      # subnormal magnitudes
    x = x.to(dtype).to(DEV)
    check_quantize(x, f"rand-{dtype}")


def make_batch(q_lens, ctx_lens, page_size, n_pages, seed):
    rng = np.random.default_rng(seed)
    B_ = len(q_lens)
    max_pages = max((L + page_size - 1) // page_size for L in ctx_lens)
    perm = rng.permutation(n_pages).astype(np.int32)
    page_table = np.zeros((B_, max_pages), np.int32)
    off = 0
    for b, L in enumerate(ctx_lens):
        npg = (L + page_size - 1) // page_size
        page_table[b, :npg] = perm[off:off + npg]
        off += npg
    assert off <= n_pages
    q_start = np.zeros(B_ + 1, np.int32)
    q_start[1:] = np.cumsum(q_lens)
    host = dict(q_start=q_start, ctx_len=np.array(ctx_lens, np.int32), page_table=page_table,
                page_size=page_size)
    dev = {k: torch.from_numpy(v).to(DEV) for k, v in host.items() if k != "page_size"}
    bt = B.make_batch(dev["q_start"], dev["ctx_len"], dev["page_table"], total_q=int(q_start[-1]),
                      max_q=max(q_lens), max_ctx=max(ctx_lens), page_size=page_size)
    return host, dev, bt


@pytest.mark.parametrize("case", ["latent-fp8-bf16src", "separate-bf16-copy", "f32-fp8-f32src"])
def test_cache_append_matches_oracle(case):
    g = torch.Generator().manual_seed({"latent-fp8-bf16src": 31, "separate-bf16-copy": 32, "f32-fp8-f32src": 33}[case])
    if case == "latent-fp8-bf16src":
        q_lens, ctx_lens, ps = [300, 1, 1, 57], [3300, 40000, 1000, 57], 64
        kv_dt, d_qk, d_v, stride, latent, src_dt, d_i, idx_dt = torch.bfloat16, 576, 512, 576, True, \
            torch.bfloat16, 128, torch.float8_e4m3fn
    elif case == "separate-bf16-copy":
        q_lens, ctx_lens, ps = [1] * 8 + [200], [8000 + 997 * i for i in range(8)] + [700], 16
        kv_dt, d_qk, d_v, stride, latent, src_dt, d_i, idx_dt = torch.bfloat16, 128, 128, 128, False, \
            torch.bfloat16, 64, torch.bfloat16
    else:
        q_lens, ctx_lens, ps = [33, 5], [100, 5], 16
        kv_dt, d_qk, d_v, stride, latent, src_dt, d_i, idx_dt = torch.float32, 64, 64, 64, False, \
            torch.float32, 128, torch.float8_e4m3fn
    n_pages = sum((L + ps - 1) // ps for L in ctx_lens) + 5
    host, dev, bt = make_batch(q_lens, ctx_lens, ps, n_pages, seed=len(case))
    T = sum(q_lens)
    P.say(f"[append {case}] T={T} pages={n_pages} page_size={ps}")
    rows = n_pages * ps
    k_cache = torch.randn(n_pages, ps, stride, generator=g).to(kv_dt).to(DEV)
    v_cache = k_cache if latent else torch.randn(n_pages, ps, stride, generator=g).to(kv_dt).to(DEV)
    if idx_dt == torch.float8_e4m3fn:
        kic = torch.randint(0, 126, (n_pages, ps, d_i), generator=g, dtype=torch.uint8).view(
            torch.float8_e4m3fn).to(DEV)
        ksc = torch.rand(n_pages, ps, generator=g).to(DEV)
    else:
        kic = torch.randn(n_pages, ps, d_i, generator=g).to(idx_dt).to(DEV)
        ksc = None
    k_new = torch.randn(T, d_qk, generator=g).to(kv_dt).to(DEV)
    v_new = None if latent else torch.randn(T, d_v, generator=g).to(kv_dt).to(DEV)
    kidx_new = (torch.randn(T, d_i, generator=g) * torch.pow(2.0, torch.randint(-8, 8, (T, 1), generator=g).float()))
    kidx_new[0] = 0.0
    kidx_new = kidx_new.to(src_dt).to(DEV)

    want = dict(k=raw(k_cache).reshape(rows, stride), v=None if latent else raw(v_cache).reshape(rows, stride),
                ki=raw(kic).reshape(rows, d_i), ks=None if ksc is None else raw(ksc).reshape(rows))
    dname = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8"}
    O.cache_append(q_start=host["q_start"], ctx_len=host["ctx_len"], page_table=host["page_table"],
                   page_size=ps, kv_dtype=dname[kv_dt], k_new=raw(k_new), v_new=None if latent else raw(v_new),
                   k_cache=want["k"], v_cache=want["k"] if latent else want["v"], src_dtype=dname[src_dt],
                   k_idx_new=raw(kidx_new), idx_dtype=dname[idx_dt], k_idx_cache=want["ki"],
                   k_scale_cache=want["ks"])

    B.sparse_cache_append(bt, k_new, k_cache, kidx_new, kic, v_new=v_new, v_cache=None if latent else v_cache,
                          k_scale_cache=ksc)
    torch.cuda.synchronize()
    assert np.array_equal(raw(k_cache).reshape(rows, stride), want["k"])
    if not latent:
        assert np.array_equal(raw(v_cache).reshape(rows, stride), want["v"])
    got_ki = raw(kic).reshape(rows, d_i)
    bad = np.argwhere(got_ki != want["ki"])
    assert bad.size == 0, f"{len(bad)} key bytes differ, first {bad[:3].tolist()}"
    if ksc is not None:
        assert np.array_equal(raw(ksc).reshape(rows).view(np.uint32), want["ks"].view(np.uint32))


def test_cache_append_rejects_bad_arguments():
    host, dev, bt = make_batch([1], [10], 16, 2, seed=1)
    k = torch.zeros(1, 576, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(2, 16, 576, dtype=torch.bfloat16, device=DEV)
    ki = torch.zeros(1, 127, dtype=torch.bfloat16, device=DEV)      # odd d_i
    kic = torch.zeros(2, 16, 127, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(B.SparseAttnError) as e:
        B.sparse_cache_append(bt, k, kc, ki, kic)
    assert e.value.status == B.SA_EINVAL
    x = torch.zeros(4, 12, dtype=torch.bfloat16, device=DEV)           # cols not a multiple of 8
    with pytest.raises(B.SparseAttnError):
        B.sparse_quantize_fp8_rows(x, torch.zeros(4, 12, dtype=torch.uint8, device=DEV),
                                   torch.zeros(4, device=DEV))
