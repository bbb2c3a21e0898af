"""Thin ctypes binding of libsparse_attn.so (argument marshalling only).

Each function has the name of the C entry point it calls and passes torch
tensors' device pointers and the current HIP stream straight through; every
step of the path runs in the library's kernels.  Loading fails loudly when the
library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparse_attn.so")

SA_F32, SA_BF16, SA_FP8_E4M3 = 0, 1, 2
SA_OK, SA_EINVAL, SA_EUNSUPPORTED, SA_EWORKSPACE, SA_ELAUNCH = 0, -1, -2, -3, -4

EXPORTS = ("sparse_indexer_scores", "sparse_topk_workspace_size", "sparse_topk",
           "sparse_gated_attn_workspace_size", "sparse_gated_attn_fwd", "sparse_gated_attn_fwd_noalloc",
           "sparse_block_pool",
           "sparse_block_scores_workspace_size", "sparse_block_scores", "sparse_block_topk_workspace_size",
           "sparse_block_topk", "sparse_block_expand", "sparse_gated_attn_bwd_workspace_size",
           "sparse_gated_attn_bwd", "sparse_window_indices",
           "sparse_branch_fuse", "sparse_attn_fuse_fwd",
           "sparse_cache_append",
           "sparse_quantize_fp8_rows", "sa_status_string", "sa_abi_version")

_DT = {torch.float32: SA_F32, torch.bfloat16: SA_BF16, torch.float8_e4m3fn: SA_FP8_E4M3}


class SaBatch(ctypes.Structure):
    """Mirror of ``sa_batch`` (include/sparse_attn.h)."""

    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("max_q", ctypes.c_int32),
        ("max_ctx", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("q_start", ctypes.c_void_p),
        ("ctx_len", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
    ]


class SparseAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status} ({status_string(status)})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library; raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run indexer_top_sparse_relu_amd/build.py "
                               "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        bp = ctypes.POINTER(SaBatch)
        L.sparse_indexer_scores.restype = ctypes.c_int
        L.sparse_indexer_scores.argtypes = [bp, ctypes.c_int, vp, i32, i32, vp, vp, vp, vp, vp, i64, vp]
        L.sparse_topk_workspace_size.restype = sz
        L.sparse_topk_workspace_size.argtypes = [bp, i32]
        L.sparse_topk.restype = ctypes.c_int
        L.sparse_topk.argtypes = [bp, vp, i64, i32, vp, vp, sz, vp]
        L.sparse_gated_attn_workspace_size.restype = sz
        L.sparse_gated_attn_workspace_size.argtypes = [bp, i32, i32, i32]
        L.sparse_gated_attn_fwd.restype = ctypes.c_int
        L.sparse_gated_attn_fwd.argtypes = [bp, ctypes.c_int, vp, i32, i32, vp, vp, i32, i64, vp, i32, vp, i32,
                                            ctypes.c_float, vp, vp, vp, sz, vp]
        L.sparse_attn_fuse_fwd.restype = ctypes.c_int
        L.sparse_attn_fuse_fwd.argtypes = [bp, ctypes.c_int, vp, i32, i32, vp, vp, i32, i64, vp, i32, vp, i32,
                                           ctypes.c_float, vp, vp, vp, vp, sz, vp]
        L.sparse_gated_attn_fwd_noalloc.restype = ctypes.c_int
        L.sparse_gated_attn_fwd_noalloc.argtypes = [bp, ctypes.c_int, vp, i32, i32, vp, vp, i32, i64, vp, i32, vp,
                                                    i32, ctypes.c_float, vp, vp, vp]
        L.sparse_block_pool.restype = ctypes.c_int
        L.sparse_block_pool.argtypes = [bp, ctypes.c_int, vp, i32, i64, vp, vp]
        L.sparse_block_scores_workspace_size.restype = sz
        L.sparse_block_scores_workspace_size.argtypes = [bp, i32]
        L.sparse_block_scores.restype = ctypes.c_int
        L.sparse_block_scores.argtypes = [bp, ctypes.c_int, vp, i32, i32, vp, vp, i64, vp, sz, vp]
        L.sparse_block_topk_workspace_size.restype = sz
        L.sparse_block_topk_workspace_size.argtypes = [bp, i32]
        L.sparse_block_topk.restype = ctypes.c_int
        L.sparse_block_topk.argtypes = [bp, vp, i64, i32, vp, vp, sz, vp]
        L.sparse_block_expand.restype = ctypes.c_int
        L.sparse_block_expand.argtypes = [bp, vp, i32, vp, vp]
        L.sparse_gated_attn_bwd_workspace_size.restype = sz
        L.sparse_gated_attn_bwd_workspace_size.argtypes = [bp, i32, i32, i32, i32]
        L.sparse_gated_attn_bwd.restype = ctypes.c_int
        L.sparse_gated_attn_bwd.argtypes = [bp, ctypes.c_int, vp, i32, i32, vp, vp, i32, i64, vp, i32, vp, i32,
                                            ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.sparse_window_indices.restype = ctypes.c_int
        L.sparse_window_indices.argtypes = [bp, i32, vp, vp]
        L.sparse_branch_fuse.restype = ctypes.c_int
        L.sparse_branch_fuse.argtypes = [ctypes.c_int, i64, i32, vp, vp, vp, i32, vp, vp]
        L.sparse_cache_append.restype = ctypes.c_int
        L.sparse_cache_append.argtypes = [bp, ctypes.c_int, vp, i32, vp, i32, vp, vp, i64, ctypes.c_int, vp, i32,
                                          ctypes.c_int, vp, vp, vp]
        L.sparse_quantize_fp8_rows.restype = ctypes.c_int
        L.sparse_quantize_fp8_rows.argtypes = [ctypes.c_int, vp, i64, i32, vp, vp, vp]
        L.sa_status_string.restype = ctypes.c_char_p
        L.sa_status_string.argtypes = [ctypes.c_int]
        L.sa_abi_version.restype = i32
        L.sa_abi_version.argtypes = []
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().sa_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(fn: str, status: int) -> None:
    if status != SA_OK:
        raise SparseAttnError(fn, status)


def make_batch(q_start: torch.Tensor, ctx_len: torch.Tensor, page_table: torch.Tensor, *, total_q: int,
               max_q: int, max_ctx: int, page_size: int) -> SaBatch:
    """Describe a ragged batch (host sizes + device arrays); the tensors must outlive its use."""
    for t in (q_start, ctx_len, page_table):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError("q_start, ctx_len and page_table must be contiguous int32")
    return SaBatch(int(ctx_len.shape[0]), int(total_q), int(max_q), int(max_ctx), int(page_size),
                   int(page_table.shape[1]), q_start.data_ptr(), ctx_len.data_ptr(), page_table.data_ptr())


def batch_of(wl) -> SaBatch:
    """Batch description of a generated workload (host values from its spec)."""
    s = wl.spec
    return SaBatch(s.B, s.T, s.max_q, s.max_ctx, s.page_size, wl.max_pages,
                   wl.q_start.data_ptr(), wl.ctx_len.data_ptr(), wl.page_table.data_ptr())


def sparse_indexer_scores(batch: SaBatch, q_idx: torch.Tensor, weights: torch.Tensor, k_idx: torch.Tensor,
                          scores: torch.Tensor, q_scale: Optional[torch.Tensor] = None,
                          k_scale: Optional[torch.Tensor] = None, stream=None) -> None:
    """Indexer scores into `scores` [T, ld] (row i: entries [0, n_i))."""
    T, H, D = q_idx.shape
    st = lib().sparse_indexer_scores(ctypes.byref(batch), _DT[q_idx.dtype], _ptr(q_idx), H, D, _ptr(q_scale),
                                     _ptr(weights), _ptr(k_idx), _ptr(k_scale), _ptr(scores), scores.stride(0),
                                     _stream(stream))
    _check("sparse_indexer_scores", st)


def sparse_topk_workspace_size(batch: SaBatch, k: int) -> int:
    return int(lib().sparse_topk_workspace_size(ctypes.byref(batch), int(k)))


def sparse_topk(batch: SaBatch, scores: torch.Tensor, k: int, indices: torch.Tensor,
                workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Top-k positions of each score row into `indices` [T, k] (ascending, then -1)."""
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().sparse_topk(ctypes.byref(batch), _ptr(scores), scores.stride(0), int(k), _ptr(indices),
                           _ptr(workspace), wsb, _stream(stream))
    _check("sparse_topk", st)


def sparse_gated_attn_workspace_size(batch: SaBatch, n_q_heads: int, d_v: int, k: int) -> int:
    return int(lib().sparse_gated_attn_workspace_size(ctypes.byref(batch), int(n_q_heads), int(d_v), int(k)))


def sparse_gated_attn_fwd(batch: SaBatch, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, d_v: int,
                          indices: torch.Tensor, gate: torch.Tensor, out: torch.Tensor,
                          softmax_scale: Optional[float] = None, lse: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Gated sparse attention of q over the indexed cache rows into `out` [T, Hq, d_v]."""
    T, Hq, dqk = q.shape
    per_channel = 1 if gate.dim() == 3 else 0
    scale = float(softmax_scale if softmax_scale is not None else dqk ** -0.5)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().sparse_gated_attn_fwd(ctypes.byref(batch), _DT[q.dtype], _ptr(q), Hq, dqk, _ptr(k_cache),
                                     _ptr(v_cache), int(d_v), k_cache.stride(-2), _ptr(indices), indices.shape[1],
                                     _ptr(gate), per_channel, ctypes.c_float(scale), _ptr(out), _ptr(lse),
                                     _ptr(workspace), wsb, _stream(stream))
    _check("sparse_gated_attn_fwd", st)


def sparse_attn_fuse_fwd(batch: SaBatch, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, d_v: int,
                         indices: torch.Tensor, gate: torch.Tensor, other: torch.Tensor, out: torch.Tensor,
                         softmax_scale: Optional[float] = None, lse: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Attention over `indices` mixed with another branch's output in the epilogue:
    out = sigmoid(G) * other + (1 - sigmoid(G)) * attention."""
    T, Hq, dqk = q.shape
    per_channel = 1 if gate.dim() == 3 else 0
    scale = float(softmax_scale if softmax_scale is not None else dqk ** -0.5)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().sparse_attn_fuse_fwd(ctypes.byref(batch), _DT[q.dtype], _ptr(q), Hq, dqk, _ptr(k_cache),
                                    _ptr(v_cache), int(d_v), k_cache.stride(-2), _ptr(indices), indices.shape[1],
                                    _ptr(gate), per_channel, ctypes.c_float(scale), _ptr(other), _ptr(out),
                                    _ptr(lse), _ptr(workspace), wsb, _stream(stream))
    _check("sparse_attn_fuse_fwd", st)


def sparse_gated_attn_fwd_noalloc(batch: SaBatch, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                  d_v: int, indices: torch.Tensor, gate: torch.Tensor, out: torch.Tensor,
                                  softmax_scale: Optional[float] = None, lse: Optional[torch.Tensor] = None,
                                  stream=None) -> None:
    """sparse_gated_attn_fwd with the library's static per-GPU scratch instead of a workspace."""
    T, Hq, dqk = q.shape
    per_channel = 1 if gate.dim() == 3 else 0
    scale = float(softmax_scale if softmax_scale is not None else dqk ** -0.5)
    st = lib().sparse_gated_attn_fwd_noalloc(ctypes.byref(batch), _DT[q.dtype], _ptr(q), Hq, dqk, _ptr(k_cache),
                                             _ptr(v_cache), int(d_v), k_cache.stride(-2), _ptr(indices),
                                             indices.shape[1], _ptr(gate), per_channel, ctypes.c_float(scale),
                                             _ptr(out), _ptr(lse), _stream(stream))
    _check("sparse_gated_attn_fwd_noalloc", st)


def sparse_block_pool(batch: SaBatch, k_cache: torch.Tensor, d_qk: int, k_blocks: torch.Tensor, stream=None) -> None:
    """Mean K row of every block (page) a sequence uses, into k_blocks [num_pages, d_qk] fp32."""
    st = lib().sparse_block_pool(ctypes.byref(batch), _DT[k_cache.dtype], _ptr(k_cache), int(d_qk),
                                 k_cache.stride(-2), _ptr(k_blocks), _stream(stream))
    _check("sparse_block_pool", st)


def sparse_block_scores_workspace_size(batch: SaBatch, d_qk: int) -> int:
    return int(lib().sparse_block_scores_workspace_size(ctypes.byref(batch), int(d_qk)))


def sparse_block_scores(batch: SaBatch, q: torch.Tensor, k_blocks: torch.Tensor, scores: torch.Tensor,
                        workspace: torch.Tensor, stream=None) -> None:
    """Block scores (sum of the query heads' dots with each candidate block's pooled key) into scores [T, ld]."""
    T, Hq, dqk = q.shape
    wsb = workspace.numel() * workspace.element_size()
    st = lib().sparse_block_scores(ctypes.byref(batch), _DT[q.dtype], _ptr(q), Hq, dqk, _ptr(k_blocks),
                                   _ptr(scores), scores.stride(0), _ptr(workspace), wsb, _stream(stream))
    _check("sparse_block_scores", st)


def sparse_block_topk_workspace_size(batch: SaBatch, kb: int) -> int:
    return int(lib().sparse_block_topk_workspace_size(ctypes.byref(batch), int(kb)))


def sparse_block_topk(batch: SaBatch, scores: torch.Tensor, kb: int, block_idx: torch.Tensor,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Top-kb candidate blocks of each token (ascending block ids, then -1) into block_idx [T, kb]."""
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().sparse_block_topk(ctypes.byref(batch), _ptr(scores), scores.stride(0), int(kb), _ptr(block_idx),
                                 _ptr(workspace), wsb, _stream(stream))
    _check("sparse_block_topk", st)


def sparse_block_expand(batch: SaBatch, block_idx: torch.Tensor, indices: torch.Tensor, stream=None) -> None:
    """Causal positions of the selected blocks into indices [T, kb * page_size] (ascending, then -1)."""
    st = lib().sparse_block_expand(ctypes.byref(batch), _ptr(block_idx), block_idx.shape[1], _ptr(indices),
                                   _stream(stream))
    _check("sparse_block_expand", st)


def sparse_gated_attn_bwd(batch: SaBatch, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, d_v: int,
                          indices: torch.Tensor, gate: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                          d_out: torch.Tensor, d_q: torch.Tensor, d_k_cache: torch.Tensor, d_v_cache: torch.Tensor,
                          d_gate: torch.Tensor, softmax_scale: Optional[float] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Gradients of the gated sparse attention over fixed indices: d_q and d_gate written, d_k_cache and
    d_v_cache (fp32, zeroed by the caller, the same tensor for a shared cache) added to.  `workspace`
    (uint8, sparse_gated_attn_bwd_workspace_size bytes, 256-byte aligned) is allocated when not given."""
    T, Hq, dqk = q.shape
    per_channel = 1 if gate.dim() == 3 else 0
    scale = float(softmax_scale if softmax_scale is not None else dqk ** -0.5)
    K = indices.shape[1]
    if workspace is None:
        n = sparse_gated_attn_bwd_workspace_size(batch, Hq, dqk, int(d_v), K)
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().sparse_gated_attn_bwd(ctypes.byref(batch), _DT[q.dtype], _ptr(q), Hq, dqk, _ptr(k_cache),
                                     _ptr(v_cache), int(d_v), k_cache.stride(-2), _ptr(indices), K,
                                     _ptr(gate), per_channel, ctypes.c_float(scale), _ptr(out), _ptr(lse),
                                     _ptr(d_out), _ptr(d_q), _ptr(d_k_cache), _ptr(d_v_cache), _ptr(d_gate),
                                     _ptr(workspace), wsb, _stream(stream))
    _check("sparse_gated_attn_bwd", st)


def sparse_gated_attn_bwd_workspace_size(batch: SaBatch, n_q_heads: int, d_qk: int, d_v: int, k: int) -> int:
    return int(lib().sparse_gated_attn_bwd_workspace_size(ctypes.byref(batch), int(n_q_heads), int(d_qk), int(d_v),
                                                          int(k)))


def sparse_window_indices(batch: SaBatch, window: int, indices: torch.Tensor, stream=None) -> None:
    """The last `window` positions of each token (ascending, then -1) into indices [T, window]."""
    st = lib().sparse_window_indices(ctypes.byref(batch), int(window), _ptr(indices), _stream(stream))
    _check("sparse_window_indices", st)


def sparse_branch_fuse(o_sparse: torch.Tensor, o_local: torch.Tensor, gate: torch.Tensor, out: torch.Tensor,
                       stream=None) -> None:
    """out = g * o_sparse + (1 - g) * o_local, g = sigmoid(gate); outputs [T, Hq, d_v], gate [T, Hq(, d_v)]."""
    T, Hq, dv = o_sparse.shape
    per_channel = 1 if gate.dim() == 3 else 0
    st = lib().sparse_branch_fuse(_DT[o_sparse.dtype], T * Hq, dv, _ptr(o_sparse), _ptr(o_local), _ptr(gate),
                                  per_channel, _ptr(out), _stream(stream))
    _check("sparse_branch_fuse", st)


def sparse_cache_append(batch: SaBatch, k_new: torch.Tensor, k_cache: torch.Tensor, k_idx_new: torch.Tensor,
                        k_idx_cache: torch.Tensor, v_new: Optional[torch.Tensor] = None,
                        v_cache: Optional[torch.Tensor] = None, k_scale_cache: Optional[torch.Tensor] = None,
                        stream=None) -> None:
    """Write the new tokens' K (and V) rows and indexer keys at their positions' cache rows.

    k_cache / v_cache [pages, page_size, row_stride]; k_idx_cache [pages, page_size, d_i] whose dtype picks
    copy (same as k_idx_new) or fp8 quantisation (float8_e4m3fn, scales into k_scale_cache)."""
    v_cache = k_cache if v_cache is None else v_cache
    st = lib().sparse_cache_append(ctypes.byref(batch), _DT[k_new.dtype], _ptr(k_new), k_new.shape[-1],
                                   _ptr(v_new), 0 if v_new is None else v_new.shape[-1], _ptr(k_cache),
                                   _ptr(v_cache), k_cache.stride(-2), _DT[k_idx_new.dtype], _ptr(k_idx_new),
                                   k_idx_new.shape[-1], _DT[k_idx_cache.dtype], _ptr(k_idx_cache),
                                   _ptr(k_scale_cache), _stream(stream))
    _check("sparse_cache_append", st)


def sparse_quantize_fp8_rows(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, stream=None) -> None:
    """Per-row fp8 quantisation of x [rows, cols] into codes (uint8 or float8_e4m3fn) and scales [rows]."""
    rows, cols = x.reshape(x.shape[0], -1).shape
    st = lib().sparse_quantize_fp8_rows(_DT[x.dtype], _ptr(x), rows, cols, _ptr(codes), _ptr(scales),
                                        _stream(stream))
    _check("sparse_quantize_fp8_rows", st)


class Pipeline:
    """Preallocated outputs and workspaces for indexer -> Top-K -> gated attention on one workload."""

    def __init__(self, wl, ld: Optional[int] = None):
        s = wl.spec
        dev = wl.q.device
        self.wl = wl
        self.batch = batch_of(wl)
        self.ld = int(ld or ((s.max_ctx + 63) // 64 * 64))
        self.scores = torch.empty((s.T, self.ld), device=dev, dtype=torch.float32)
        self.indices = torch.empty((s.T, s.K), device=dev, dtype=torch.int32)
        self.out = torch.empty((s.T, s.Hq, s.d_v), device=dev, dtype=wl.q.dtype)
        self.lse = torch.empty((s.T, s.Hq), device=dev, dtype=torch.float32)
        tw = sparse_topk_workspace_size(self.batch, s.K)
        aw = sparse_gated_attn_workspace_size(self.batch, s.Hq, s.d_v, s.K)
        self.topk_ws = torch.empty(max(tw, 1), device=dev, dtype=torch.uint8) if tw else None
        self.attn_ws = torch.empty(max(aw, 1), device=dev, dtype=torch.uint8) if aw else None

    def indexer(self, stream=None):
        wl = self.wl
        sparse_indexer_scores(self.batch, wl.q_idx, wl.w, wl.k_idx, self.scores, wl.q_scale, wl.k_scale, stream)

    def topk(self, stream=None):
        sparse_topk(self.batch, self.scores, self.wl.spec.K, self.indices, self.topk_ws, stream)

    def attn(self, stream=None, with_lse: bool = True):
        wl = self.wl
        sparse_gated_attn_fwd(self.batch, wl.q, wl.k_cache, wl.v_cache, wl.spec.d_v, self.indices, wl.gate,
                              self.out, wl.spec.softmax_scale, self.lse if with_lse else None, self.attn_ws,
                              stream)

    def run(self, stream=None):
        self.indexer(stream)
        self.topk(stream)
        self.attn(stream)
