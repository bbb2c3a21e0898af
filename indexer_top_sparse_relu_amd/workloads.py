"""Seeded synthetic workloads for the gated sparse attention hot path.

This module draws random inputs and lays them out in the memory layout the
C-ABI expects.  It performs none of the method's arithmetic (no scoring, no
selection, no attention): both the HIP path and the CPU oracle consume what it
produces, and neither is imported here.

Recipe (shared by every workload):

* structural randomness (ragged lengths, page permutation, duplicated indexer
  key rows) comes from ``numpy.random.Generator(PCG64(seed))``;
* tensor values come from ``torch.Generator(device).manual_seed(seed)``:
  Gaussian draws scaled by ``1/sqrt(d)`` (``d`` = the tensor's last dim) for
  ``q``, ``k``, ``v``, ``q^I`` and ``k^I``; ``w ~ U(0, 1)``; gate logits
  ``~ N(0, 1)``;
* bf16 tensors are the fp32 draws rounded to nearest-even by torch;
* fp8 tensors use OCP e4m3fn (``torch.float8_e4m3fn``) with one fp32 scale
  per token: ``scale = max|x| / 448`` over the token's vector (over all heads
  and dims for ``q^I``), stored value ``fp8(x / scale)``, and the represented
  value is ``fp8 * scale``;
* caches are paged: ``[num_pages, page_size, row]``; a sequence's logical
  position ``s`` lives at physical row ``page_table[b, s // page_size] *
  page_size + s % page_size``.  Prefill workloads use an identity table;
  decode and chunked-prefill workloads deal a random permutation of exactly
  ``sum_b ceil(L_b / page_size)`` pages to the sequences in order.

The pages describe the paged cache and the ragged batches this layout serves:
[From Full Attention to Sparsity..., "Engineering Considerations" item 1] names
variable-length Top-K, gathering and paged cache management; [Hybrid Attention
Architectures: Engineering Trade-offs..., §5 item 4] names per-sample lengths
that need padding and masking.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

DTYPES = ("f32", "bf16", "fp8")

_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


@dataclass(frozen=True)
class Spec:
    """Shape and dtype description of one workload."""

    name: str
    seed: int
    q_lens: tuple            # new query tokens per sequence
    ctx_lens: tuple          # L_b: cache length after the new tokens were appended
    H_I: int                 # indexer heads
    d_I: int                 # indexer head dim
    idx_dtype: str           # "f32" | "bf16" | "fp8"
    Hq: int                  # attention query heads (all share one KV head)
    d_qk: int                # key / query dim
    d_v: int                 # value dim
    attn_dtype: str          # "f32" | "bf16"
    K: int                   # Top-K
    mla: bool = False        # V is the first d_v dims of the K row (one latent row)
    page_size: int = 64
    paged_random: bool = False
    gate_per_channel: bool = True
    dup_frac: float = 0.0    # fraction of indexer key rows per sequence copied from another row
    q_gain: float = 1.0      # extra factor on attention q (sharp-softmax parity variant)

    @property
    def B(self) -> int:
        return len(self.q_lens)

    @property
    def T(self) -> int:
        return int(sum(self.q_lens))

    @property
    def max_ctx(self) -> int:
        return int(max(self.ctx_lens))

    @property
    def max_q(self) -> int:
        return int(max(self.q_lens))

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


def _lengths(seed: int, n: int, lo: int, hi: int) -> List[int]:
    rng = np.random.Generator(np.random.PCG64(seed))
    return [int(x) for x in rng.integers(lo, hi + 1, size=n)]


def tiny_prefill_fp32(seed: int = 1) -> Spec:
    """Tiny causal prefill in fp32: T=256, indexer 4x32, 4 q heads x 64, K=32."""
    return Spec("tiny_prefill_fp32", seed, (256,), (256,), 4, 32, "f32", 4, 64, 64, "f32", 32)


def prefill_bf16(seed: int = 2, T: int = 8192) -> Spec:
    """Prefill bf16: one sequence of T tokens, indexer 16x64, MQA 32x128, K=2048."""
    return Spec("prefill_bf16_8k", seed, (T,), (T,), 16, 64, "bf16", 32, 128, 128, "bf16", 2048)


def decode_bf16(seed: int = 3, B: int = 64, lo: int = 8192, hi: int = 32768) -> Spec:
    """Batched paged decode bf16: B sequences, L_b ~ U{lo..hi}, one query each."""
    L = _lengths(seed, B, lo, hi)
    return Spec("decode_bf16_paged", seed, tuple([1] * B), tuple(L), 16, 64, "bf16", 32, 128, 128,
                "bf16", 2048, paged_random=True)


def chunked_prefill_mla(seed: int = 4, cached: int = 131072, T: int = 4096) -> Spec:
    """Chunked prefill, MLA-like latent KV: T new tokens on `cached` cached positions."""
    return Spec("chunked_prefill_mla_128k", seed, (T,), (cached + T,), 64, 128, "fp8", 128, 576, 512,
                "bf16", 2048, mla=True, paged_random=True)


def long_decode_mla(seed: int = 5, B: int = 16, lo: int = 262144, hi: int = 1048576,
                    short_len: int = 1000, short_at: int = 5) -> Spec:
    """Long-context decode: B-1 sequences with L ~ U{lo..hi} plus one of `short_len` (< K)."""
    L = _lengths(seed, B - 1, lo, hi)
    L.insert(short_at, short_len)
    return Spec("long_decode_mla", seed, tuple([1] * B), tuple(L), 64, 128, "fp8", 128, 576, 512,
                "bf16", 2048, mla=True, paged_random=True, dup_frac=0.01)


CONFIGS = {
    "tiny_prefill_fp32": tiny_prefill_fp32,
    "prefill_bf16_8k": prefill_bf16,
    "decode_bf16_paged": decode_bf16,
    "chunked_prefill_mla_128k": chunked_prefill_mla,
    "long_decode_mla": long_decode_mla,
}


@dataclass
class Workload:
    """Tensors of one workload, all on one device, in the C-ABI layout."""

    spec: Spec
    q_start: torch.Tensor        # [B+1] int32
    ctx_len: torch.Tensor        # [B] int32
    page_table: torch.Tensor     # [B, max_pages] int32
    num_pages: int
    max_pages: int
    q_idx: torch.Tensor          # [T, H_I, d_I] idx dtype (fp8 as float8_e4m3fn)
    q_scale: Optional[torch.Tensor]   # [T] f32 (fp8 only)
    w: torch.Tensor              # [T, H_I] f32
    k_idx: torch.Tensor          # [num_pages, page_size, d_I]
    k_scale: Optional[torch.Tensor]   # [num_pages, page_size] f32 (fp8 only)
    q: torch.Tensor              # [T, Hq, d_qk] attn dtype
    k_cache: torch.Tensor        # [num_pages, page_size, d_qk]
    v_cache: torch.Tensor        # [num_pages, page_size, d_v] view, or the same storage as k_cache (mla)
    gate: torch.Tensor           # [T, Hq, d_v] or [T, Hq]
    extra: dict = field(default_factory=dict)

    @property
    def kv_row_stride(self) -> int:
        """Elements between consecutive token rows of both K and V caches."""
        return int(self.k_cache.shape[-1])

    def to(self, device) -> "Workload":
        kw = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            kw[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        return Workload(**kw)


def _page_layout(spec: Spec):
    ps = spec.page_size
    npg = [(L + ps - 1) // ps for L in spec.ctx_lens]
    total = int(sum(npg))
    max_pages = int(max(npg))
    table = np.zeros((spec.B, max_pages), dtype=np.int32)
    if spec.paged_random:
        rng = np.random.Generator(np.random.PCG64(spec.seed + 1000))
        perm = rng.permutation(total).astype(np.int32)
    else:
        perm = np.arange(total, dtype=np.int32)
    off = 0
    for b, n in enumerate(npg):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, total, max_pages


def _fill_normal(out: torch.Tensor, gen: torch.Generator, d: int, gain: float = 1.0,
                 chunk_rows: int = 1 << 16) -> None:
    """Fill ``out`` (any float dtype, last dim d) with N(0,1)/sqrt(d)*gain, chunked over rows."""
    flat = out.view(-1, out.shape[-1])
    s = gain / math.sqrt(d)
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        x = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=out.device, dtype=torch.float32)
        flat[r0:r1] = (x * s).to(out.dtype)


def _quant_fp8_rows(x32: torch.Tensor):
    """Per-row (last dim) fp8 e4m3fn quantisation with scale = max|x| / 448."""
    amax = x32.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
    scale = amax / 448.0
    q8 = (x32 / scale).to(torch.float8_e4m3fn)
    return q8, scale.squeeze(-1)


def generate(spec: Spec, device="cpu") -> Workload:
    """Draw every input tensor of `spec` on `device` (deterministic for a given device)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(spec.seed)
    T, B, ps = spec.T, spec.B, spec.page_size
    for ql, L in zip(spec.q_lens, spec.ctx_lens):
        if ql > L:
            raise ValueError("a sequence has more new tokens than cache positions")
    table, num_pages, max_pages = _page_layout(spec)
    q_start = np.zeros(B + 1, dtype=np.int32)
    q_start[1:] = np.cumsum(spec.q_lens)

    # indexer query and weights
    if spec.idx_dtype == "fp8":
        x = torch.empty((T, spec.H_I * spec.d_I), device=device, dtype=torch.float32)
        _fill_normal(x, gen, spec.d_I)
        q8, qs = _quant_fp8_rows(x)
        q_idx = q8.view(T, spec.H_I, spec.d_I)
        q_scale = qs.contiguous()
        del x
    else:
        q_idx = torch.empty((T, spec.H_I, spec.d_I), device=device, dtype=_TORCH[spec.idx_dtype])
        _fill_normal(q_idx, gen, spec.d_I)
        q_scale = None
    w = torch.rand((T, spec.H_I), generator=gen, device=device, dtype=torch.float32)

    # indexer key cache
    rows = num_pages * ps
    if spec.idx_dtype == "fp8":
        k8 = torch.empty((rows, spec.d_I), device=device, dtype=torch.float8_e4m3fn)
        k_scale = torch.empty((rows,), device=device, dtype=torch.float32)
        chunk = 1 << 16
        for r0 in range(0, rows, chunk):
            r1 = min(rows, r0 + chunk)
            x = torch.randn((r1 - r0, spec.d_I), generator=gen, device=device, dtype=torch.float32)
            x *= 1.0 / math.sqrt(spec.d_I)
            a, s = _quant_fp8_rows(x)
            k8[r0:r1] = a
            k_scale[r0:r1] = s
        k_idx = k8.view(num_pages, ps, spec.d_I)
        k_scale = k_scale.view(num_pages, ps)
    else:
        k_idx = torch.empty((num_pages, ps, spec.d_I), device=device, dtype=_TORCH[spec.idx_dtype])
        _fill_normal(k_idx, gen, spec.d_I)
        k_scale = None

    # attention query, KV cache, gate logits
    adt = _TORCH[spec.attn_dtype]
    q = torch.empty((T, spec.Hq, spec.d_qk), device=device, dtype=adt)
    _fill_normal(q, gen, spec.d_qk, gain=spec.q_gain)
    if spec.mla:
        if spec.d_v > spec.d_qk:
            raise ValueError("mla layout needs d_v <= d_qk")
        k_cache = torch.empty((num_pages, ps, spec.d_qk), device=device, dtype=adt)
        _fill_normal(k_cache, gen, spec.d_qk)
        v_cache = k_cache  # V = first d_v dims of the same latent row
    else:
        k_cache = torch.empty((num_pages, ps, spec.d_qk), device=device, dtype=adt)
        _fill_normal(k_cache, gen, spec.d_qk)
        if spec.d_v != spec.d_qk:
            raise ValueError("separate K/V caches share one row stride: d_v must equal d_qk")
        v_cache = torch.empty((num_pages, ps, spec.d_v), device=device, dtype=adt)
        _fill_normal(v_cache, gen, spec.d_v)
    gshape = (T, spec.Hq, spec.d_v) if spec.gate_per_channel else (T, spec.Hq)
    gate = torch.randn(gshape, generator=gen, device=device, dtype=torch.float32).to(adt)

    # duplicated indexer-key rows (exact score ties), within each sequence
    if spec.dup_frac > 0.0:
        rng = np.random.Generator(np.random.PCG64(spec.seed + 2000))
        dst_all, src_all = [], []
        for b, L in enumerate(spec.ctx_lens):
            m = int(round(spec.dup_frac * L))
            if m == 0 or L < 2:
                continue
            dst = rng.choice(L, size=m, replace=False)
            src = rng.integers(0, L, size=m)
            phys = lambda s: table[b, s // ps].astype(np.int64) * ps + (s % ps)
            dst_all.append(phys(dst))
            src_all.append(phys(src))
        if dst_all:
            dst_t = torch.from_numpy(np.concatenate(dst_all)).to(device)
            src_t = torch.from_numpy(np.concatenate(src_all)).to(device)
            kf = k_idx.view(rows, spec.d_I)
            if kf.dtype == torch.float8_e4m3fn:
                kb = kf.view(torch.uint8)
                kb[dst_t] = kb[src_t].clone()
            else:
                kf[dst_t] = kf[src_t].clone()
            if k_scale is not None:
                ksf = k_scale.view(rows)
                ksf[dst_t] = ksf[src_t].clone()

    return Workload(
        spec=spec,
        q_start=torch.from_numpy(q_start).to(device),
        ctx_len=torch.tensor(spec.ctx_lens, dtype=torch.int32, device=device),
        page_table=torch.from_numpy(table).to(device),
        num_pages=num_pages,
        max_pages=max_pages,
        q_idx=q_idx, q_scale=q_scale, w=w, k_idx=k_idx, k_scale=k_scale,
        q=q, k_cache=k_cache, v_cache=v_cache, gate=gate,
    )
