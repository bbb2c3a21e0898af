"""Benchmark: query tokens/s of indexer + Top-K + gated sparse attention on one MI355X.

Workload (default): chunked prefill with an MLA-like latent cache — 4096 new
query tokens on a 131072-token cached context (ctx 135168), fp8 e4m3 indexer
(64 heads x 128) with per-token scales, 128 query heads over 576-dim latent
rows (V = first 512 dims), bf16 attention, K = 2048, paged cache (64-token
pages, random page table).  One step = the three C-ABI calls over the whole
batch; inputs are resident in HBM before the timed region.

Prints one JSON line.  Per-stage durations come from HIP events recorded on
the stream the kernels run on; the dominant stage's roofline uses algorithmic
work only (flops of the contraction, or bytes the method must move).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK = {"hbm_GBs": 8000.0, "fp8_TFLOPs": 5000.0, "bf16_TFLOPs": 2500.0, "fp32_TFLOPs": 157.3}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_ELEMS = 1 << 28          # calibration copy: 2^28 fp32 = 1 GiB read + 1 GiB written
FLUSH_BYTES = 512 << 20       # written between timed steps: twice the 256 MB MALL


def calibration_copy():
    """A plain streaming kernel of known traffic for scaling HBM counters: y = -x over
    COPY_ELEMS fp32 (reads and writes 4 * COPY_ELEMS bytes), run three times."""
    import torch

    x = torch.ones(COPY_ELEMS, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    del x, y


def causal_lengths(spec):
    """n = pos + 1 of every query token (new tokens are the last positions of each sequence)."""
    out = []
    for nq, L in zip(spec.q_lens, spec.ctx_lens):
        out.extend(L - nq + j + 1 for j in range(nq))
    return out


METRIC = "query tokens/s (indexer+TopK+sparse attn) at 128K ctx, K=2048; % HBM/MFMA peak"


def algorithmic_work(spec, n_valid, n_unique_rows):
    """Per-step algorithmic work of each stage: flops of the contractions, and the bytes the
    method must move (inputs read once, outputs written once).  The attention reads each cache
    row it touches once (n_unique_rows distinct rows over the whole step), not once per query
    token that selects it: at prefill a row shared by many tokens is one HBM read."""
    pairs = int(sum(causal_lengths(spec)))
    esz = {"fp8": 1, "bf16": 2, "f32": 4}
    ie, ae = esz[spec.idx_dtype], esz[spec.attn_dtype]
    scale_b = 4 if spec.idx_dtype == "fp8" else 0
    keys = int(sum(spec.ctx_lens))
    kv_row = spec.d_qk * ae + (0 if spec.mla else spec.d_v * ae)
    gate_elems = spec.Hq * (spec.d_v if spec.gate_per_channel else 1)
    return {
        "indexer": {"flops": 2.0 * spec.H_I * spec.d_I * pairs,
                    "bytes": spec.T * (spec.H_I * spec.d_I * ie + scale_b + spec.H_I * 4)
                    + keys * (spec.d_I * ie + scale_b) + pairs * 4},
        "topk": {"bytes": pairs * 4 + spec.T * spec.K * 4},
        "attn": {"flops": 2.0 * spec.Hq * n_valid * (spec.d_qk + spec.d_v),
                 "bytes": n_unique_rows * kv_row
                 + spec.T * (spec.Hq * spec.d_qk + gate_elems + spec.Hq * spec.d_v) * ae + spec.T * spec.K * 4,
                 "gathered_bytes": n_valid * kv_row},
    }


def unique_rows(wl, indices):
    """Distinct physical cache rows the step's index lists touch (outside the timed region)."""
    import torch

    s = wl.spec
    seq = torch.repeat_interleave(torch.arange(s.B, device=indices.device),
                                  torch.tensor(s.q_lens, device=indices.device))
    acc = torch.empty(0, dtype=torch.long, device=indices.device)
    for t0 in range(0, s.T, 512):
        idx = indices[t0:t0 + 512].long()
        b = seq[t0:t0 + 512, None].expand_as(idx)
        ok = idx >= 0
        rows = wl.page_table[b[ok], idx[ok] // s.page_size].long() * s.page_size + idx[ok] % s.page_size
        acc = torch.unique(torch.cat([acc, rows]))
    return int(acc.numel())


def stats_ms(vals):
    import statistics

    return {"mean": sum(vals) / len(vals), "median": statistics.median(vals), "min": min(vals), "max": max(vals)}


def graph_step(pl, steps, flush_bytes):
    """The step (indexer, Top-K, attention) captured once in a HIP graph and replayed, as a serving
    loop would run it: the graph submits the launches together, so the gaps between kernels shrink.
    Between replays the outputs get a canary and the cache flush runs (eager work); every replay
    must reproduce the eager step's indices and output bit for bit."""
    import torch

    stream = torch.cuda.current_stream()
    ref_idx, ref_out = pl.indices.clone(), pl.out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s = torch.cuda.current_stream()
        pl.indexer(s)
        pl.topk(s)
        pl.attn(s, with_lse=False)
    flush = torch.empty(flush_bytes // 4, device="cuda") if flush_bytes else None
    clean = torch.zeros(flush_bytes // 4, device="cuda") if flush_bytes else None
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    same = True
    for i in range(steps):
        pl.indices.fill_(-7)
        if flush is not None:
            flush.fill_(float(i))
            clean.amax()
        ev[i][0].record(stream)
        g.replay()
        ev[i][1].record(stream)
        same = same and torch.equal(pl.indices, ref_idx) and torch.equal(pl.out.view(torch.int16),
                                                                         ref_out.view(torch.int16))
    torch.cuda.synchronize()
    del g, flush, clean
    st = stats_ms([e[0].elapsed_time(e[1]) for e in ev])
    assert same, "a graph replay differs from the eager step"
    return {"ms_per_step": st["median"], "ms_per_step_stats": st,
            "query_tokens_per_s": pl.wl.spec.T / (st["median"] * 1e-3), "replays_match_eager": same}


def machine_info():
    """GPU, ROCm and host facts for the record."""
    import glob
    import platform

    import torch

    info = {}
    try:
        p = torch.cuda.get_device_properties(0)
        info["gpu"] = p.name
        info["gpu_arch"] = getattr(p, "gcnArchName", None)
        info["gpu_cus"] = p.multi_processor_count
        info["gpu_mem_GB"] = round(p.total_memory / 1e9, 1)
    except Exception as e:  # noqa: BLE001
        info["gpu"] = f"unknown ({e})"
    info["hip"] = torch.version.hip
    info["torch"] = torch.__version__
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    clocks = {}
    for card in sorted(glob.glob("/sys/class/drm/card*/device")):
        for name in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
            try:
                with open(os.path.join(card, name)) as f:
                    levels = [l.strip() for l in f if l.strip()]
            except OSError:
                continue
            cur = [l for l in levels if l.endswith("*")]
            clocks[name[7:]] = {"levels": levels, "current": cur[0] if cur else None}
        if clocks:
            break
    info["clocks"] = clocks or None
    info.update(machine_info_cpu())
    info["host_cpus"] = os.cpu_count()
    try:
        info["host_cpus_usable"] = len(os.sched_getaffinity(0))
    except AttributeError:
        info["host_cpus_usable"] = None
    return info


def machine_info_cpu():
    """The host CPU: its model name and identification fields."""
    import platform

    cpu, ids = None, {}
    try:
        # the first processor's entry: a virtualised host may give only the brand as its
        # model name, so the family, model number and stepping (the generation) go with it
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "model name":
                    cpu = val
                elif key in ("vendor_id", "cpu family", "model", "stepping", "cpu MHz"):
                    ids[key.replace(" ", "_")] = val
                elif key == "flags":
                    ids["avx512f"] = "avx512f" in val.split()
    except OSError:
        pass
    return {"cpu": cpu or platform.processor(), "cpu_id": ids or None}


def measured_ceilings(stream):
    """Ceilings measured on this GPU with library kernels (not the path's): a 1 GiB streaming copy
    (bytes read + written per second), a bf16 GEMM and an fp8 GEMM (8192^3, hipBLASLt through
    torch).  Reported beside the published peaks; the roofline fractions use the published ones."""
    import torch

    out = {}

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e-3

    x = torch.empty(1 << 28, device="cuda")
    y = torch.empty_like(x)
    t = timed(lambda: y.copy_(x), 10)
    out["hbm_copy_GBs"] = 2 * x.numel() * 4 / t / 1e9
    del x, y
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    t = timed(lambda: torch.matmul(a, b), 10)
    out["bf16_gemm_TFLOPs"] = 2.0 * n ** 3 / t / 1e12
    try:
        a8 = a.to(torch.float8_e4m3fn)
        b8 = b.t().contiguous().to(torch.float8_e4m3fn).t()
        one = torch.ones((), device="cuda")
        t = timed(lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one, out_dtype=torch.bfloat16), 10)
        out["fp8_gemm_TFLOPs"] = 2.0 * n ** 3 / t / 1e12
    except Exception as e:  # noqa: BLE001
        out["fp8_gemm_TFLOPs"] = None
        out["fp8_gemm_error"] = str(e)[:120]
    del a, b
    torch.cuda.empty_cache()
    return out


def to_np(t):
    import numpy as np
    import torch

    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def cpu_baseline(wl, gpu_indices, sample_tokens: int):
    """The oracle (as it stands) on the last `sample_tokens` query tokens of the workload, and the
    recall@K of the GPU's selection against the oracle's on those tokens (the share of the
    oracle's K positions the GPU also selected, averaged over the rows)."""
    import numpy as np

    from oracle import oracle as O

    s = wl.spec
    S = min(sample_tokens, s.T)
    sl = slice(s.T - S, s.T)
    same = wl.v_cache.data_ptr() == wl.k_cache.data_ptr()
    kc = to_np(wl.k_cache)
    inp = O.Inputs(q_start=np.array([0, S], np.int32), ctx_len=np.array(s.ctx_lens[-1:], np.int32),
                   page_table=to_np(wl.page_table[-1:]), page_size=s.page_size, idx_dtype=s.idx_dtype,
                   attn_dtype=s.attn_dtype, q_idx=to_np(wl.q_idx[sl]),
                   q_scale=to_np(wl.q_scale[sl]) if wl.q_scale is not None else None, w=to_np(wl.w[sl]),
                   k_idx=to_np(wl.k_idx), k_scale=to_np(wl.k_scale) if wl.k_scale is not None else None,
                   q=to_np(wl.q[sl]), k_cache=kc, v_cache=kc if same else to_np(wl.v_cache), gate=to_np(wl.gate[sl]),
                   H_I=s.H_I, d_I=s.d_I, Hq=s.Hq, d_qk=s.d_qk, d_v=s.d_v, row_stride=wl.kv_row_stride,
                   gate_per_channel=s.gate_per_channel)
    threads = O.set_threads(0)
    t0 = time.perf_counter()
    _, ref_idx, _ = O.pipeline(inp, s.K, scale=s.softmax_scale)
    dt = time.perf_counter() - t0
    gpu = to_np(gpu_indices[sl])
    rec = []
    for r in range(S):
        want = ref_idx[r][ref_idx[r] >= 0]
        got = gpu[r][gpu[r] >= 0]
        rec.append(np.intersect1d(want, got).size / max(1, want.size))
    return {"value": S / dt, "unit": "query_tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"last {S} of {s.T} query tokens (positions {s.ctx_lens[-1] - S}..{s.ctx_lens[-1] - 1}), "
                      f"full indexer + Top-K + gated attention in fp64, {dt:.1f} s",
            "recall_at_K": float(np.mean(rec)), "recall_min": float(np.min(rec)), "recall_rows": S,
            "cpu": {k: machine_info_cpu()[k] for k in ("cpu", "cpu_id")}}


def before_path(wl, steps: int, stream):
    """The step before the path, timed apart (not part of the step above): the cache append
    of the batch's new tokens (latent K rows in bf16 and fp8 indexer keys quantised from bf16,
    into copies of the caches) and the fp8 quantisation of the indexer queries from bf16.
    Algorithmic bytes: every input read once and every output written once."""
    import torch

    from indexer_top_sparse_relu_amd import binding as B

    s = wl.spec
    if s.idx_dtype != "fp8":
        return None
    g = torch.Generator(device="cuda").manual_seed(5)
    k_cache, k_idx = wl.k_cache.clone(), wl.k_idx.clone()
    k_scale = wl.k_scale.clone()
    ae = 2 if s.attn_dtype == "bf16" else 4
    k_new = torch.randn(s.T, s.d_qk, device="cuda", generator=g).to(wl.k_cache.dtype)
    v_new = None if s.mla else torch.randn(s.T, s.d_v, device="cuda", generator=g).to(wl.k_cache.dtype)
    v_cache = None if s.mla else wl.v_cache.clone()
    kidx_new = torch.randn(s.T, s.d_I, device="cuda", generator=g).to(torch.bfloat16)
    q_bf16 = torch.randn(s.T, s.H_I * s.d_I, device="cuda", generator=g).to(torch.bfloat16)
    codes = torch.empty(s.T, s.H_I * s.d_I, device="cuda", dtype=torch.uint8)
    scales = torch.empty(s.T, device="cuda", dtype=torch.float32)
    bt = B.batch_of(wl)

    def append():
        B.sparse_cache_append(bt, k_new, k_cache, kidx_new, k_idx, v_new=v_new, v_cache=v_cache,
                              k_scale_cache=k_scale, stream=stream)

    def quant():
        B.sparse_quantize_fp8_rows(q_bf16, codes, scales, stream=stream)

    kv_bytes = s.d_qk * ae + (0 if s.mla else s.d_v * ae)
    work = {"cache_append": (append, s.T * (2 * kv_bytes + 2 * s.d_I + s.d_I + 4)),
            "quantize_q": (quant, s.T * (2 * s.H_I * s.d_I + s.H_I * s.d_I + 4))}
    out = {}
    for name, (fn, nbytes) in work.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        ach = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"bound": "hbm", "achieved": ach, "peak": PEAK["hbm_GBs"], "unit": "GB/s",
                     "frac": ach / PEAK["hbm_GBs"], "ms": ms, "bytes": nbytes}
    return out


def block_variant(wl, steps: int, stream, kb: int):
    """The pages' block-level variant on the same workload, timed apart from the step above:
    pooled block keys, block scores, top-kb blocks, their expansion to positions, and the same
    gated attention over kb * page_size positions.  Stage rooflines use algorithmic work:
    pooling reads every cache row once; scoring is 2 * d_qk flops per (token, candidate block)
    on fp32 MFMA plus one read of q; the attention counts its selected positions as the step does."""
    import torch

    from indexer_top_sparse_relu_amd import binding as B

    s = wl.spec
    bt = B.batch_of(wl)
    ps = s.page_size
    n_pages = wl.k_cache.shape[0]
    max_blocks = (s.max_ctx + ps - 1) // ps
    ld = (max_blocks + 3) // 4 * 4
    kbar = torch.empty((n_pages, s.d_qk), device="cuda")
    scores = torch.empty((s.T, ld), device="cuda")
    ws = torch.empty(B.sparse_block_scores_workspace_size(bt, s.d_qk), dtype=torch.uint8, device="cuda")
    blk = torch.empty((s.T, kb), dtype=torch.int32, device="cuda")
    tw = B.sparse_block_topk_workspace_size(bt, kb)
    tws = torch.empty(tw, dtype=torch.uint8, device="cuda") if tw else None
    idx = torch.empty((s.T, kb * ps), dtype=torch.int32, device="cuda")
    out = torch.empty((s.T, s.Hq, s.d_v), device="cuda", dtype=wl.q.dtype)
    aw = B.sparse_gated_attn_workspace_size(bt, s.Hq, s.d_v, kb * ps)
    aws = torch.empty(aw, dtype=torch.uint8, device="cuda") if aw else None
    stages = {
        "pool": lambda: B.sparse_block_pool(bt, wl.k_cache, s.d_qk, kbar, stream=stream),
        "scores": lambda: B.sparse_block_scores(bt, wl.q, kbar, scores, ws, stream=stream),
        "topk": lambda: B.sparse_block_topk(bt, scores, kb, blk, tws, stream=stream),
        "expand": lambda: B.sparse_block_expand(bt, blk, idx, stream=stream),
        "attn": lambda: B.sparse_gated_attn_fwd(bt, wl.q, wl.k_cache, wl.v_cache, s.d_v, idx, wl.gate, out,
                                                softmax_scale=s.softmax_scale, workspace=aws, stream=stream),
    }
    for fn in stages.values():
        fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        for k, fn in enumerate(stages.values()):
            fn()
            ev[i][k + 1].record(stream)
    torch.cuda.synchronize()
    ms = {name: sum(e[k].elapsed_time(e[k + 1]) for e in ev) / steps for k, name in enumerate(stages)}
    step_ms = sum(e[0].elapsed_time(e[-1]) for e in ev) / steps
    ae = 2 if s.attn_dtype == "bf16" else 4
    nb = [((L - nq + j) // ps) + 1 for nq, L in zip(s.q_lens, s.ctx_lens) for j in range(nq)]
    n_valid = int((idx >= 0).sum().item())
    cache_rows = sum(s.ctx_lens)
    work = {
        "pool": ("hbm", cache_rows * s.d_qk * ae + sum((L + ps - 1) // ps for L in s.ctx_lens) * s.d_qk * 4),
        "scores": ("mfma_fp32", 2.0 * s.d_qk * sum(nb)),
        "topk": ("hbm", sum(nb) * 4 + s.T * kb * 4),
        "expand": ("hbm", s.T * kb * 4 + s.T * kb * ps * 4),
        "attn": ("mfma", 2.0 * s.Hq * n_valid * (s.d_qk + s.d_v)),
    }
    rl = {}
    for name, (kind, w) in work.items():
        t = ms[name] * 1e-3
        if kind == "hbm":
            ach = w / t / 1e9
            rl[name] = {"bound": "hbm", "achieved": ach, "peak": PEAK["hbm_GBs"], "unit": "GB/s"}
        else:
            peak = PEAK["fp32_TFLOPs"] if kind == "mfma_fp32" or s.attn_dtype != "bf16" else PEAK["bf16_TFLOPs"]
            ach = w / t / 1e12
            rl[name] = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s"}
        rl[name]["frac"] = rl[name]["achieved"] / rl[name]["peak"]
        rl[name]["ms"] = ms[name]
    return {"kb": kb, "block": ps, "positions": kb * ps, "ms_per_step": step_ms,
            "query_tokens_per_s": s.T / (step_ms * 1e-3), "stages": rl}


def branch_fusion(wl, pl, steps: int, stream, window: int):
    """Branch fusion with a sliding-window local branch on the same workload, timed apart from the
    step: the sparse branch (the step's attention over its Top-K indices, ungated), the window
    list, and the local branch (the same attention over the last `window` positions) with the
    fusion y = g * sparse + (1 - g) * local formed in its epilogue.  The separate form (an
    ungated local branch written out, then a mix pass over both outputs) is timed beside it.
    The indexer and Top-K are the step's and are not repeated here."""
    import torch

    from indexer_top_sparse_relu_amd import binding as B

    s = wl.spec
    bt = pl.batch
    inf = torch.full((s.T, s.Hq), float("inf"), device="cuda").to(wl.q.dtype)
    win = torch.empty((s.T, window), dtype=torch.int32, device="cuda")
    o_s = torch.empty((s.T, s.Hq, s.d_v), device="cuda", dtype=wl.q.dtype)
    o_l = torch.empty_like(o_s)
    y = torch.empty_like(o_s)
    y2 = torch.empty_like(o_s)
    ws = {}
    for k in (s.K, window):
        n = B.sparse_gated_attn_workspace_size(bt, s.Hq, s.d_v, k)
        ws[k] = torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
    stages = {
        "sparse_branch": lambda: B.sparse_gated_attn_fwd(bt, wl.q, wl.k_cache, wl.v_cache, s.d_v, pl.indices, inf,
                                                         o_s, softmax_scale=s.softmax_scale, workspace=ws[s.K],
                                                         stream=stream),
        "window": lambda: B.sparse_window_indices(bt, window, win, stream=stream),
        "local_branch": lambda: B.sparse_gated_attn_fwd(bt, wl.q, wl.k_cache, wl.v_cache, s.d_v, win, inf, o_l,
                                                        softmax_scale=s.softmax_scale, workspace=ws[window],
                                                        stream=stream),
        "fuse": lambda: B.sparse_branch_fuse(o_s, o_l, wl.gate, y, stream=stream),
        "local_branch_fused": lambda: B.sparse_attn_fuse_fwd(bt, wl.q, wl.k_cache, wl.v_cache, s.d_v, win, wl.gate,
                                                             o_s, y2, softmax_scale=s.softmax_scale,
                                                             workspace=ws[window], stream=stream),
    }
    for fn in stages.values():
        fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        for k, fn in enumerate(stages.values()):
            fn()
            ev[i][k + 1].record(stream)
    torch.cuda.synchronize()
    ms = {name: sum(e[k].elapsed_time(e[k + 1]) for e in ev) / steps for k, name in enumerate(stages)}
    ae = 2 if s.attn_dtype == "bf16" else 4
    n_sparse = int((pl.indices >= 0).sum().item())
    n_local = int((win >= 0).sum().item())
    gate_elems = s.Hq * (s.d_v if s.gate_per_channel else 1)
    peak_mma = PEAK["bf16_TFLOPs"] if s.attn_dtype == "bf16" else PEAK["fp32_TFLOPs"]
    work = {
        "sparse_branch": ("mfma", 2.0 * s.Hq * n_sparse * (s.d_qk + s.d_v)),
        "window": ("hbm", s.T * window * 4),
        "local_branch": ("mfma", 2.0 * s.Hq * n_local * (s.d_qk + s.d_v)),
        "fuse": ("hbm", s.T * (3 * s.Hq * s.d_v * ae + gate_elems * ae)),
        "local_branch_fused": ("mfma", 2.0 * s.Hq * n_local * (s.d_qk + s.d_v)),
    }
    rl = {}
    for name, (kind, w) in work.items():
        t = ms[name] * 1e-3
        if kind == "hbm":
            rl[name] = {"bound": "hbm", "achieved": w / t / 1e9, "peak": PEAK["hbm_GBs"], "unit": "GB/s"}
        else:
            rl[name] = {"bound": "mfma", "achieved": w / t / 1e12, "peak": peak_mma, "unit": "TFLOP/s"}
        rl[name]["frac"] = rl[name]["achieved"] / rl[name]["peak"]
        rl[name]["ms"] = ms[name]
    fused = ms["sparse_branch"] + ms["window"] + ms["local_branch_fused"]
    separate = ms["sparse_branch"] + ms["window"] + ms["local_branch"] + ms["fuse"]
    return {"window": window, "ms_attention_and_fusion": fused, "ms_separate_mix_pass": separate, "stages": rl}


def backward_pass(steps: int, stream):
    """The backward over fixed indices on the bf16 prefill workload (8192 tokens, 32 query heads of
    128 dims, K = 2048), timed apart from the step: the forward (indexer, Top-K, attention with its
    log-sum-exp) runs once to produce the indices, the output and lse, then sparse_gated_attn_bwd is
    timed.  Algorithmic work: 2 * H_q * (3 d_qk + 2 d_v) flops per (token, selected position) for
    the S, dq and dK contractions over d_qk and the dP and dV ones over d_v (S is recomputed),
    against the bf16 peak."""
    import torch

    from indexer_top_sparse_relu_amd import binding as B
    from indexer_top_sparse_relu_amd import workloads as W

    spec = W.CONFIGS["prefill_bf16_8k"]()
    wl = W.generate(spec, "cuda")
    pl = B.Pipeline(wl)
    pl.run(stream)
    torch.cuda.synchronize()
    g = torch.Generator(device="cuda").manual_seed(7)
    dy = torch.randn(pl.out.shape, device="cuda", generator=g).to(torch.bfloat16)
    shared = wl.v_cache.data_ptr() == wl.k_cache.data_ptr()
    dk = torch.zeros((wl.k_cache.shape[0], wl.k_cache.shape[1], wl.kv_row_stride), device="cuda")
    dv = dk if shared else torch.zeros_like(dk)
    dq = torch.empty(wl.q.shape, device="cuda")
    dg = torch.empty(wl.gate.shape, device="cuda")
    nws = B.sparse_gated_attn_bwd_workspace_size(pl.batch, spec.Hq, spec.d_qk, spec.d_v, spec.K)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")

    def bwd():
        B.sparse_gated_attn_bwd(pl.batch, wl.q, wl.k_cache, wl.v_cache, spec.d_v, pl.indices, wl.gate, pl.out,
                                pl.lse, dy, dq, dk, dv, dg, softmax_scale=spec.softmax_scale, workspace=ws,
                                stream=stream)

    bwd()
    torch.cuda.synchronize()
    n = max(1, min(steps, 10))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        bwd()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    n_valid = int((pl.indices >= 0).sum().item())
    flops = 2.0 * spec.Hq * n_valid * (3 * spec.d_qk + 2 * spec.d_v)     # S, dq, dK over d_qk; dP, dV over d_v
    ach = flops / (ms * 1e-3) / 1e12
    return {"workload": spec.name, "ms": ms, "query_tokens_per_s": spec.T / (ms * 1e-3),
            "workspace_bytes": nws,
            "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK["bf16_TFLOPs"], "unit": "TFLOP/s",
                         "frac": ach / PEAK["bf16_TFLOPs"]}}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="chunked_prefill_mla_128k")
    ap.add_argument("--cpu-sample", type=int, default=192, help="query tokens the oracle baseline runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="time only the step (no cache append, block variant or branch fusion runs), so that "
                         "a profile of this process holds the step's kernels alone")
    ap.add_argument("--no-flush", action="store_true", help="do not evict the caches between timed steps")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a copy kernel of known size (for HBM counter calibration)")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    from indexer_top_sparse_relu_amd import binding as B
    from indexer_top_sparse_relu_amd import workloads as W

    from indexer_top_sparse_relu_amd.profiling import source_hash

    if args.calibrate_copy:
        calibration_copy()
    spec = W.CONFIGS[args.workload]()
    wl = W.generate(spec, "cuda")
    pl = B.Pipeline(wl)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        pl.run(stream)
    torch.cuda.synchronize()

    # Between timed steps, on the same stream and outside the event pairs, a 512 MiB buffer is
    # written and then another 512 MiB buffer read, so that no step finds its inputs in L2 or the
    # 256 MB MALL. The read replaces the written (dirty) lines with clean ones: after a write alone,
    # the next step's reads would first have to write up to 256 MB of those lines back to HBM, a
    # cost of the flush, not of the step. The write-only protocol is timed as well and reported.
    def timed_steps(modes):
        """args.steps timed steps per flush mode, the modes alternating step by step (so that
        neither gets the warmer clock); per mode, per stage statistics and the wall time."""
        wbuf = torch.empty(FLUSH_BYTES // 4, device="cuda") if modes != ["none"] else None
        rbuf = torch.zeros(FLUSH_BYTES // 4, device="cuda") if "write+read" in modes else None
        ev = {m: [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
              for m in modes}
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            for m in modes:
                if m != "none":
                    wbuf.fill_(float(i))
                if m == "write+read":
                    rbuf.amax()
                e = ev[m][i]
                e[0].record(stream)
                pl.indexer(stream)
                e[1].record(stream)
                pl.topk(stream)
                e[2].record(stream)
                pl.attn(stream, with_lse=False)
                e[3].record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / len(modes)
        del wbuf, rbuf
        res = {}
        for m in modes:
            per = {"indexer": [e[0].elapsed_time(e[1]) for e in ev[m]],
                   "topk": [e[1].elapsed_time(e[2]) for e in ev[m]],
                   "attn": [e[2].elapsed_time(e[3]) for e in ev[m]],
                   "step": [e[0].elapsed_time(e[3]) for e in ev[m]]}
            res[m] = {k: stats_ms(v) for k, v in per.items()}
        return res, wall

    res, wall = timed_steps(["none"] if args.no_flush else ["write+read", "write"])
    st_ms = res["none"] if args.no_flush else res["write+read"]
    st_write = None if args.no_flush else res["write"]
    stage_ms = {k: st_ms[k]["mean"] for k in ("indexer", "topk", "attn")}
    step_ms = st_ms["step"]["median"]
    wall_ms = wall * 1e3 / args.steps
    n_valid = int((pl.indices >= 0).sum().item())
    n_unique = unique_rows(wl, pl.indices)
    assert torch.isfinite(pl.out.float()).all().item(), "non-finite output"

    work = algorithmic_work(spec, n_valid, n_unique)
    dom = max(stage_ms, key=stage_ms.get)
    rl = {}
    for st, ms in stage_ms.items():
        w = work[st]
        peak = None
        if st == "indexer":
            peak = PEAK["fp8_TFLOPs"] if spec.idx_dtype == "fp8" else PEAK["bf16_TFLOPs"] if spec.idx_dtype == "bf16" \
                else PEAK["fp32_TFLOPs"]
        elif st == "attn":
            peak = PEAK["bf16_TFLOPs"] if spec.attn_dtype == "bf16" else PEAK["fp32_TFLOPs"]
        # a contraction whose flops per algorithmic byte fall below the ridge point (peak flops over
        # peak bandwidth) is bound by HBM: decode, where every key row is used by one query token
        if peak is not None and w["flops"] / w["bytes"] >= peak * 1e12 / (PEAK["hbm_GBs"] * 1e9):
            ach = w["flops"] / (ms * 1e-3) / 1e12
            rl[st] = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s", "frac": ach / peak}
        else:
            ach = w["bytes"] / (ms * 1e-3) / 1e9
            rl[st] = {"bound": "hbm", "achieved": ach, "peak": PEAK["hbm_GBs"], "unit": "GB/s",
                      "frac": ach / PEAK["hbm_GBs"]}
        rl[st]["ms"] = ms
        rl[st]["ms_median"] = st_ms[st]["median"]
        rl[st]["ms_min"] = st_ms[st]["min"]
        rl[st]["ms_max"] = st_ms[st]["max"]
        rl[st]["algorithmic_bytes"] = w["bytes"]
        if "flops" in w:
            rl[st]["algorithmic_flops"] = w["flops"]
    rl["attn"]["gathered_rows_GBs"] = work["attn"]["gathered_bytes"] / (stage_ms["attn"] * 1e-3) / 1e9
    rl["attn"]["unique_rows"] = n_unique
    rl["attn"]["selected_slots"] = n_valid
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        ent = tr.get(spec.name, {}).get(dom)
        if ent and ent.get("source_hash") == source_hash(dom):
            traffic = ent["bytes_per_launch"]
    roof = {k: rl[dom][k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    roof["kernel"] = dom
    roof["traffic"] = traffic

    tokens = spec.T
    line = {
        "metric": METRIC if spec.name == "chunked_prefill_mla_128k" else
        f"query tokens/s (indexer+TopK+sparse attn), {spec.name}, K={spec.K}; % HBM/MFMA peak",
        "value": tokens / (step_ms * 1e-3),
        "unit": "query_tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "ms_per_step_stats": st_ms["step"],
        "wall_ms_per_step": wall_ms,
        "timing": ("HIP events on the kernels' stream around each stage; value and ms_per_step from the median "
                   "step" + ("" if args.no_flush else f"; between steps, outside the events, a {FLUSH_BYTES >> 20} "
                                                       f"MiB buffer is written and another {FLUSH_BYTES >> 20} MiB "
                                                       "read, which evicts L2 and the MALL and leaves them clean")
                   + "; roofline achieved from the dominant stage's mean duration"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{spec.idx_dtype}+{spec.attn_dtype}",
        "data": "synthetic",
        "config": {"workload": spec.name, "new_tokens": spec.T, "ctx": spec.max_ctx, "K": spec.K,
                   "indexer": f"{spec.H_I}x{spec.d_I} {spec.idx_dtype}", "q_heads": spec.Hq,
                   "d_qk": spec.d_qk, "d_v": spec.d_v, "kv": "latent (V = first d_v of K row)" if spec.mla else "MQA",
                   "page_size": spec.page_size, "gate": "per-channel" if spec.gate_per_channel else "per-head"},
        "roofline": roof,
        "stages": rl,
    }
    if st_write is not None:
        # the same steps after a write-only flush: the step then also pays for writing the flush's
        # dirty lines back to HBM
        line["write_only_flush"] = {"ms_per_step": st_write["step"]["median"],
                                    "query_tokens_per_s": tokens / (st_write["step"]["median"] * 1e-3),
                                    "stage_ms_mean": {k: st_write[k]["mean"] for k in ("indexer", "topk", "attn")}}
    line["graph_step"] = graph_step(pl, args.steps, 0 if args.no_flush else FLUSH_BYTES)
    line["machine"] = machine_info()
    if not args.step_only:
        line["measured_ceilings"] = measured_ceilings(stream)
        c = line["measured_ceilings"]
        for st, r in rl.items():
            if r["bound"] == "hbm" and c.get("hbm_copy_GBs"):
                r["frac_of_measured"] = r["achieved"] / c["hbm_copy_GBs"]
            elif r["bound"] == "mfma":
                key = "fp8_gemm_TFLOPs" if (st == "indexer" and spec.idx_dtype == "fp8") else "bf16_gemm_TFLOPs"
                if c.get(key) and (st == "attn" or spec.idx_dtype != "f32"):
                    r["frac_of_measured"] = r["achieved"] / c[key]
        line["before_path"] = before_path(wl, args.steps, stream)
        line["block_variant"] = block_variant(wl, args.steps, stream, kb=max(1, spec.K // spec.page_size))
        line["branch_fusion"] = branch_fusion(wl, pl, args.steps, stream, window=512)
        line["backward"] = backward_pass(args.steps, stream)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, pl.indices, args.cpu_sample)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
