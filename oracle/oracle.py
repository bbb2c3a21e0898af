"""ctypes wrapper of the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It imports nothing
from the HIP package; inputs arrive as plain numpy arrays (raw element bits for
bf16 and fp8) or as any object with the workload's attribute names.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

DT = {"f32": 0, "bf16": 1, "fp8": 2}


def build(force: bool = False, sanitize: bool = False, out: Optional[str] = None) -> str:
    """Compile the oracle with gcc (fp contraction off, no fast-math)."""
    out = out or LIB
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(SRC):
        return out
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
           "-std=c11", "-Wall", "-Wextra", "-Wno-unused-parameter", SRC, "-o", out + ".tmp", "-lm"]
    if sanitize:
        cmd[1:1] = ["-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class _Batch(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("pad_", ctypes.c_int32),
        ("q_start", ctypes.c_void_p),
        ("ctx_len", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        # ORACLE_LIB names a prebuilt copy (the sanitizer run of the pins builds one)
        path = os.environ.get("ORACLE_LIB") or build()
        L = ctypes.CDLL(path)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.orc_fp8_e4m3fn.restype = dbl
        L.orc_fp8_e4m3fn.argtypes = [ctypes.c_uint8]
        L.orc_bf16.restype = dbl
        L.orc_bf16.argtypes = [ctypes.c_uint16]
        L.orc_fp8_table.argtypes = [vp]
        L.orc_set_threads.restype = ctypes.c_int
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_row_lengths.argtypes = [vp, vp, i64, vp]
        L.orc_indexer.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, i64, vp, i64]
        L.orc_topk.argtypes = [vp, i64, vp, i64, ctypes.c_int, vp]
        L.orc_sparse_attn.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_int, i64,
                                      vp, ctypes.c_int, vp, ctypes.c_int, dbl, vp, i64, vp, vp]
        L.orc_dense_attn.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_int, i64,
                                     vp, ctypes.c_int, dbl, vp, i64, vp]
        L.orc_block_pool.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, i64, vp]
        L.orc_block_scores.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, vp, vp, i64, vp, i64]
        L.orc_block_expand.argtypes = [vp, vp, ctypes.c_int, vp, i64, vp]
        L.orc_window_indices.argtypes = [vp, ctypes.c_int, vp, i64, vp]
        L.orc_branch_fuse.argtypes = [ctypes.c_int, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, i64,
                                      vp]
        L.orc_sparse_attn_bwd.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_int,
                                          i64, vp, ctypes.c_int, vp, ctypes.c_int, dbl, vp, i64, vp, vp, vp, vp]
        L.orc_fp8_encode.restype = ctypes.c_uint8
        L.orc_fp8_encode.argtypes = [ctypes.c_float]
        L.orc_quantize_rows.argtypes = [ctypes.c_int, vp, i64, i64, vp, vp]
        L.orc_cache_append.argtypes = [vp, i64, ctypes.c_int, vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, i64,
                                       ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, vp, vp]
        _lib = L
    return _lib


def set_threads(n: int = 0) -> int:
    """Set (n > 0) and return the number of OpenMP threads the oracle uses."""
    return int(lib().orc_set_threads(n))


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if dtype is not None and a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def fp8_table() -> np.ndarray:
    out = np.zeros(256, dtype=np.float64)
    lib().orc_fp8_table(out.ctypes.data)
    return out


def bf16_value(bits: int) -> float:
    return float(lib().orc_bf16(bits))


class Inputs:
    """Host-side raw arrays of one workload, as the oracle reads them."""

    def __init__(self, *, q_start, ctx_len, page_table, page_size, idx_dtype, attn_dtype,
                 q_idx, q_scale, w, k_idx, k_scale, q, k_cache, v_cache, gate,
                 H_I, d_I, Hq, d_qk, d_v, row_stride, gate_per_channel):
        self.q_start = _c(q_start, np.int32)
        self.ctx_len = _c(ctx_len, np.int32)
        self.page_table = _c(page_table, np.int32)
        self.page_size = int(page_size)
        self.idx_dtype, self.attn_dtype = idx_dtype, attn_dtype
        self.q_idx, self.q_scale, self.w = _c(q_idx), _c(q_scale, np.float32), _c(w, np.float32)
        self.k_idx, self.k_scale = _c(k_idx), _c(k_scale, np.float32)
        self.q, self.k_cache, self.v_cache, self.gate = _c(q), _c(k_cache), _c(v_cache), _c(gate)
        self.H_I, self.d_I, self.Hq, self.d_qk, self.d_v = int(H_I), int(d_I), int(Hq), int(d_qk), int(d_v)
        self.row_stride = int(row_stride)
        self.gate_per_channel = bool(gate_per_channel)
        self.B = int(self.ctx_len.shape[0])
        self._bt = _Batch(self.B, self.page_size, int(self.page_table.shape[1]), 0,
                          self.q_start.ctypes.data, self.ctx_len.ctypes.data, self.page_table.ctypes.data)

    @property
    def T(self) -> int:
        return int(self.q_start[-1])

    @classmethod
    def from_workload(cls, wl) -> "Inputs":
        """Copy a workload's tensors (any device) to host raw arrays."""
        import torch

        def raw(t):
            if t is None:
                return None
            t = t.detach().contiguous().cpu()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16)
            if t.dtype == torch.float8_e4m3fn:
                return t.view(torch.uint8).numpy()
            return t.numpy()

        s = wl.spec
        same = wl.v_cache.data_ptr() == wl.k_cache.data_ptr()
        kc = raw(wl.k_cache)
        return cls(q_start=raw(wl.q_start), ctx_len=raw(wl.ctx_len), page_table=raw(wl.page_table),
                   page_size=s.page_size, idx_dtype=s.idx_dtype, attn_dtype=s.attn_dtype,
                   q_idx=raw(wl.q_idx), q_scale=raw(wl.q_scale), w=raw(wl.w), k_idx=raw(wl.k_idx),
                   k_scale=raw(wl.k_scale), q=raw(wl.q), k_cache=kc, v_cache=kc if same else raw(wl.v_cache),
                   gate=raw(wl.gate), H_I=s.H_I, d_I=s.d_I, Hq=s.Hq, d_qk=s.d_qk, d_v=s.d_v,
                   row_stride=wl.kv_row_stride, gate_per_channel=s.gate_per_channel)


def _rows(inp: Inputs, rows) -> np.ndarray:
    if rows is None:
        rows = np.arange(inp.T)
    return np.ascontiguousarray(np.asarray(rows, dtype=np.int64))


def row_lengths(inp: Inputs, rows=None) -> np.ndarray:
    rows = _rows(inp, rows)
    n = np.zeros(rows.shape[0], dtype=np.int64)
    lib().orc_row_lengths(ctypes.byref(inp._bt), rows.ctypes.data, rows.shape[0], n.ctypes.data)
    return n


def indexer(inp: Inputs, rows=None, ld: Optional[int] = None) -> np.ndarray:
    """Indexer scores in double, [len(rows), ld]; entries at or beyond n are NaN."""
    rows = _rows(inp, rows)
    ld = int(ld or int(inp.ctx_len.max()))
    out = np.full((rows.shape[0], ld), np.nan, dtype=np.float64)
    lib().orc_indexer(ctypes.byref(inp._bt), DT[inp.idx_dtype], _p(inp.q_idx), inp.H_I, inp.d_I,
                      _p(inp.q_scale), _p(inp.w), _p(inp.k_idx), _p(inp.k_scale),
                      rows.ctypes.data, rows.shape[0], out.ctypes.data, ld)
    return out


def topk(scores: np.ndarray, n: np.ndarray, K: int) -> np.ndarray:
    """Brute-force Top-K of each row's first n entries: ascending positions, then -1."""
    scores = np.ascontiguousarray(scores, dtype=np.float64)
    n = np.ascontiguousarray(n, dtype=np.int64)
    if scores.ndim != 2 or n.shape[0] != scores.shape[0] or (n.size and n.max() > scores.shape[1]):
        raise ValueError("bad topk shapes")
    out = np.zeros((scores.shape[0], K), dtype=np.int32)
    lib().orc_topk(scores.ctypes.data, scores.shape[1], n.ctypes.data, scores.shape[0], int(K), out.ctypes.data)
    return out


def sparse_attn(inp: Inputs, idx: np.ndarray, rows=None, scale: Optional[float] = None, with_lse: bool = False):
    """Gated attention of the listed tokens over their index rows (idx[r] belongs to rows[r])."""
    rows = _rows(inp, rows)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    if idx.shape[0] != rows.shape[0]:
        raise ValueError("idx needs one row per listed token")
    K = idx.shape[1]
    scale = float(scale if scale is not None else 1.0 / np.sqrt(inp.d_qk))
    out = np.zeros((rows.shape[0], inp.Hq, inp.d_v), dtype=np.float64)
    lse = np.zeros((rows.shape[0], inp.Hq), dtype=np.float64) if with_lse else None
    lib().orc_sparse_attn(ctypes.byref(inp._bt), DT[inp.attn_dtype], _p(inp.q), inp.Hq, inp.d_qk,
                          _p(inp.k_cache), _p(inp.v_cache), inp.d_v, inp.row_stride, idx.ctypes.data, K,
                          _p(inp.gate), int(inp.gate_per_channel), scale, rows.ctypes.data, rows.shape[0],
                          out.ctypes.data, _p(lse))
    return (out, lse) if with_lse else out


def dense_attn(inp: Inputs, rows=None, scale: Optional[float] = None) -> np.ndarray:
    """Causal gated full attention (the control branch), no index set."""
    rows = _rows(inp, rows)
    scale = float(scale if scale is not None else 1.0 / np.sqrt(inp.d_qk))
    out = np.zeros((rows.shape[0], inp.Hq, inp.d_v), dtype=np.float64)
    lib().orc_dense_attn(ctypes.byref(inp._bt), DT[inp.attn_dtype], _p(inp.q), inp.Hq, inp.d_qk,
                         _p(inp.k_cache), _p(inp.v_cache), inp.d_v, inp.row_stride, _p(inp.gate),
                         int(inp.gate_per_channel), scale, rows.ctypes.data, rows.shape[0], out.ctypes.data)
    return out


def pipeline(inp: Inputs, K: int, rows=None, scale: Optional[float] = None):
    """Indexer -> Top-K -> gated sparse attention for the listed tokens, all in the oracle."""
    rows = _rows(inp, rows)
    sc = indexer(inp, rows)
    n = row_lengths(inp, rows)
    idx = topk(sc, n, K)
    out = sparse_attn(inp, idx, rows, scale)
    return sc, idx, out


# ------------------------------------------------ cache append + fp8 quantisation

def fp8_encode(y) -> np.ndarray:
    """e4m3fn codes of float32 values: nearest, ties to even, saturating at +-448."""
    y = np.ascontiguousarray(y, dtype=np.float32).ravel()
    return np.array([lib().orc_fp8_encode(float(v)) for v in y], dtype=np.uint8)


def quantize_rows(x: np.ndarray, src_dtype: str):
    """Per-row fp8 quantisation of x [rows, cols] (f32 values, or raw bf16 bits as uint16):
    returns (codes uint8 [rows, cols], scales float32 [rows]) with scale = max|x| / 448."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    codes = np.zeros((rows, cols), np.uint8)
    scales = np.zeros(rows, np.float32)
    lib().orc_quantize_rows(DT[src_dtype], x.ctypes.data, rows, cols, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def cache_append(*, q_start, ctx_len, page_table, page_size, kv_dtype, k_new, v_new, k_cache, v_cache,
                 src_dtype, k_idx_new, idx_dtype, k_idx_cache, k_scale_cache=None):
    """Apply the cache append in place to host raw arrays.  Caches are indexed by physical row:
    k_cache / v_cache [rows, row_stride], k_idx_cache [rows, d_i], k_scale_cache [rows]."""
    q_start = _c(q_start, np.int32)
    ctx_len = _c(ctx_len, np.int32)
    page_table = _c(page_table, np.int32)
    bt = _Batch(int(ctx_len.shape[0]), int(page_size), int(page_table.shape[1]), 0,
                q_start.ctypes.data, ctx_len.ctypes.data, page_table.ctypes.data)
    for a in (k_cache, v_cache, k_idx_cache, k_scale_cache):
        if a is not None and not a.flags.c_contiguous:
            raise ValueError("caches must be contiguous (they are written in place)")
    k_new, v_new, k_idx_new = _c(k_new), _c(v_new), _c(k_idx_new)
    T = int(q_start[-1])
    lib().orc_cache_append(ctypes.byref(bt), T, DT[kv_dtype], _p(k_new), int(k_new.shape[-1]), _p(v_new),
                           0 if v_new is None else int(v_new.shape[-1]), _p(k_cache), _p(v_cache),
                           int(k_cache.shape[-1]), DT[src_dtype], _p(k_idx_new), int(k_idx_new.shape[-1]),
                           DT[idx_dtype], _p(k_idx_cache), _p(k_scale_cache))


# ------------------------------------------------------ block-level selection

def block_pool(inp: Inputs) -> np.ndarray:
    """Mean K row (first d_qk elements) of every block a sequence uses, [num_pages, d_qk] float64,
    indexed by physical page (a block is one page); pages no sequence uses stay NaN."""
    rows = inp.k_cache.reshape(-1, inp.row_stride).shape[0]
    kbar = np.full((rows // inp.page_size, inp.d_qk), np.nan, dtype=np.float64)
    lib().orc_block_pool(ctypes.byref(inp._bt), DT[inp.attn_dtype], _p(inp.k_cache), inp.d_qk, inp.row_stride,
                         kbar.ctypes.data)
    return kbar


def block_row_lengths(inp: Inputs, rows=None) -> np.ndarray:
    """Candidate blocks of each token: those whose first position is <= pos."""
    return (row_lengths(inp, rows) - 1) // inp.page_size + 1


def block_scores(inp: Inputs, kbar: np.ndarray, rows=None, ld: Optional[int] = None) -> np.ndarray:
    """S[i, j] = sum_h q[i,h,:] . kbar[page of block j], [len(rows), ld]; NaN beyond the candidates."""
    rows = _rows(inp, rows)
    ld = int(ld or int(inp.page_table.shape[1]))
    kbar = np.ascontiguousarray(kbar, dtype=np.float64)
    out = np.full((rows.shape[0], ld), np.nan, dtype=np.float64)
    lib().orc_block_scores(ctypes.byref(inp._bt), DT[inp.attn_dtype], _p(inp.q), inp.Hq, inp.d_qk,
                           kbar.ctypes.data, rows.ctypes.data, rows.shape[0], out.ctypes.data, ld)
    return out


def block_expand(inp: Inputs, blk: np.ndarray, rows=None) -> np.ndarray:
    """Positions (<= pos) of the listed blocks, in block order, then -1: [len(rows), kb * page_size]."""
    rows = _rows(inp, rows)
    blk = np.ascontiguousarray(blk, dtype=np.int32)
    kb = blk.shape[1]
    out = np.zeros((rows.shape[0], kb * inp.page_size), dtype=np.int32)
    lib().orc_block_expand(ctypes.byref(inp._bt), blk.ctypes.data, kb, rows.ctypes.data, rows.shape[0],
                           out.ctypes.data)
    return out


def block_pipeline(inp: Inputs, kb: int, rows=None, scale: Optional[float] = None):
    """Pool -> block scores -> top-kb blocks -> expansion -> gated sparse attention, all in the oracle."""
    rows = _rows(inp, rows)
    kbar = block_pool(inp)
    sc = block_scores(inp, kbar, rows)
    nb = block_row_lengths(inp, rows)
    blk = topk(sc, nb, kb)
    idx = block_expand(inp, blk, rows)
    out = sparse_attn(inp, idx, rows, scale)
    return sc, blk, idx, out


# ------------------------------------------ branch fusion with a local branch

def window_indices(inp: Inputs, w: int, rows=None) -> np.ndarray:
    """Positions max(0, pos - w + 1) .. pos of each token, ascending, then -1: [len(rows), w]."""
    rows = _rows(inp, rows)
    out = np.zeros((rows.shape[0], int(w)), dtype=np.int32)
    lib().orc_window_indices(ctypes.byref(inp._bt), int(w), rows.ctypes.data, rows.shape[0], out.ctypes.data)
    return out


def ungated(inp: Inputs) -> Inputs:
    """The same inputs with a per-head gate of +inf (sigmoid = 1): attention without its output gate."""
    import copy
    u = copy.copy(inp)
    inf = np.full((inp.T, inp.Hq), np.inf, dtype=np.float32)
    if inp.attn_dtype == "bf16":
        inf = (inf.view(np.uint32) >> 16).astype(np.uint16)
    u.gate = np.ascontiguousarray(inf)
    u.gate_per_channel = False
    return u


def branch_fuse(inp: Inputs, a: np.ndarray, b: np.ndarray, rows=None) -> np.ndarray:
    """g * a + (1 - g) * b with g = sigmoid(G) of the inputs' gate, [len(rows), Hq, d_v]."""
    rows = _rows(inp, rows)
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    y = np.zeros_like(a)
    lib().orc_branch_fuse(DT[inp.attn_dtype], a.ctypes.data, b.ctypes.data, _p(inp.gate), int(inp.gate_per_channel),
                          inp.Hq, inp.d_v, rows.ctypes.data, rows.shape[0], y.ctypes.data)
    return y


def fused_pipeline(inp: Inputs, K: int, w: int, rows=None, scale: Optional[float] = None):
    """Indexer -> Top-K -> ungated sparse attention, ungated window attention, then the gated fusion."""
    rows = _rows(inp, rows)
    sc, idx, _ = pipeline(inp, K, rows, scale)
    u = ungated(inp)
    a = sparse_attn(u, idx, rows, scale)
    b = sparse_attn(u, window_indices(inp, w, rows), rows, scale)
    return idx, a, b, branch_fuse(inp, a, b, rows)


# ------------------------------------------------- backward over fixed indices

def sparse_attn_bwd(inp: Inputs, idx: np.ndarray, dy: np.ndarray, scale: Optional[float] = None):
    """Gradients of the gated sparse attention of every token over idx [T, K], for the upstream
    gradient dy [T, Hq, d_v] (raw bits for bf16): returns (dq [T, Hq, d_qk], dk [rows, row_stride],
    dv [rows, row_stride], dgate like the gate), all float64; dk/dv are indexed by physical cache row
    and are the same array for the latent layout (V inside the K row)."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    dy = np.ascontiguousarray(dy)
    T = inp.T
    if idx.shape[0] != T:
        raise ValueError("idx needs one row per token")
    scale = float(scale if scale is not None else 1.0 / np.sqrt(inp.d_qk))
    rows = inp.k_cache.reshape(-1, inp.row_stride).shape[0]
    same = inp.v_cache is inp.k_cache or (inp.v_cache.ctypes.data == inp.k_cache.ctypes.data)
    dq = np.zeros((T, inp.Hq, inp.d_qk), dtype=np.float64)
    dk = np.zeros((rows, inp.row_stride), dtype=np.float64)
    dv = dk if same else np.zeros((rows, inp.row_stride), dtype=np.float64)
    dg = np.zeros((T, inp.Hq, inp.d_v) if inp.gate_per_channel else (T, inp.Hq), dtype=np.float64)
    lib().orc_sparse_attn_bwd(ctypes.byref(inp._bt), DT[inp.attn_dtype], _p(inp.q), inp.Hq, inp.d_qk,
                              _p(inp.k_cache), _p(inp.v_cache), inp.d_v, inp.row_stride, idx.ctypes.data,
                              idx.shape[1], _p(inp.gate), int(inp.gate_per_channel), scale, dy.ctypes.data, T,
                              dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, dg.ctypes.data)
    return dq, dk, dv, dg
