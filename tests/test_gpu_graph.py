"""The path captured in a HIP graph and replayed.

A serving loop captures the step once (no call of the path allocates, sets
memory or synchronises) and replays it.  Each workload here reaches different
kernels: the decode indexer and the single-launch Top-K with split attention,
the sampled-threshold Top-K of few long rows, the prefill tile indexer with the
two-launch Top-K and the latent attention kernel, and the register-resident
Top-K with the MQA kernel.  Every replay runs after eager work that overwrites
the outputs with canaries, and must give the eager step's scores, indices and
output bit for bit (the eager step itself is held to the oracle by the parity
tests).
"""
import pytest
import torch

from indexer_top_sparse_relu_amd import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from indexer_top_sparse_relu_amd import binding as B  # noqa: E402

REPLAYS = 4


def _valid_scores(pl):
    """Score rows up to each token's causal length (the rest of a row is never written)."""
    n = P.token_geometry(pl.wl.spec)[2]
    return [pl.scores[r, :int(n[r])].clone() for r in range(pl.wl.spec.T)]


@pytest.mark.parametrize("name", ["decode", "long-decode", "mla-prefill", "mqa-prefill"])
def test_graph_replays_match_eager(name):
    spec = {
        "decode": lambda: W.decode_bf16(B=16, lo=3000, hi=9000).replace(seed=81),
        "long-decode": lambda: W.long_decode_mla(B=4, lo=140000, hi=300000, short_len=700, short_at=1).replace(seed=82),
        "mla-prefill": lambda: W.chunked_prefill_mla(cached=3000, T=333).replace(seed=83),
        "mqa-prefill": lambda: W.prefill_bf16(T=1536).replace(K=512, seed=84),
    }[name]()
    P.say(f"[graph-{name}] {spec.name} T={spec.T} B={spec.B} K={spec.K} max_ctx={spec.max_ctx}")
    wl = W.generate(spec, "cuda")
    pl = B.Pipeline(wl)
    stream = torch.cuda.current_stream()
    pl.run(stream)
    torch.cuda.synchronize()
    ref_scores, ref_idx, ref_out = _valid_scores(pl), pl.indices.clone(), pl.out.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s = torch.cuda.current_stream()
        pl.indexer(s)
        pl.topk(s)
        pl.attn(s, with_lse=False)
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        pl.scores.fill_(float("nan"))
        pl.indices.fill_(-7)
        pl.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _valid_scores(pl)
        assert all(torch.equal(a.view(torch.int32), b.view(torch.int32)) for a, b in zip(got, ref_scores)), \
            f"replay {i}: scores"
        assert torch.equal(pl.indices, ref_idx), f"replay {i}: indices"
        assert torch.equal(pl.out.view(torch.int16), ref_out.view(torch.int16)), f"replay {i}: output"
        P.say(f"[graph-{name}] replay {i} matches the eager step")
    del g
