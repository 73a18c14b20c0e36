"""The codec's calls under HIP graph capture: a captured step replays bit for bit like eager calls.

bench.py times the step as replays of one captured graph.  Here a step (the
encode of one worker and the decode of W payloads, in each download
variant) is captured once; then it is replayed three times, with the
program's own eager work and synchronisations between the replays, and
after every replay its momentum, payload and parameters (or sign words) must
equal, bit for bit, those of the same step run eagerly on copies of the same
state.  The library enqueues kernels only (no memset or copy nodes), which
this checks on every variant bench.py captures.
"""
import numpy as np
import pytest
import torch

import demo_inputs as DI
from communication_compressed_optimizer_demo_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()
    return torch.device("cuda:0")


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint8)


@pytest.mark.parametrize("variant", ["apply", "chunk128", "signs", "wire", "signs128", "wire128", "aggregated",
                                     "muon"])
def test_graph_replay_matches_eager(dev, variant):
    chunk = 128 if "128" in variant else 64
    shapes = [(192, 320), (300,), (130, 70)]
    W, k = 3, 16
    w = DI.WORKLOADS["tiny_256"].replace(name=f"graph_{variant}", shapes=tuple(shapes), k=k, workers=W)
    codec = B.Codec(shapes, k, w.beta, w.alpha, chunk=chunk, aggregated=variant == "aggregated")
    ne = codec.n_entries
    G = [torch.from_numpy(DI.gradient(w, 0, 0, i)).cuda() for i in range(len(shapes))]
    # two identical copies of the state: a = graph replays, b = eager calls
    st = {}
    for tag in "ab":
        vals, idx = codec.alloc_payload(W)
        for wk in range(1, W):  # the other workers' payloads, the same in both copies
            gf = [torch.from_numpy(DI.gradient(w, wk, 0, i)).cuda() for i in range(len(shapes))]
            codec.encode(gf, [torch.zeros(s, device="cuda") for s in shapes], vals[wk * ne:(wk + 1) * ne],
                         idx[wk * ne:(wk + 1) * ne])
        st[tag] = dict(M=[torch.zeros(s, device="cuda") for s in shapes],
                       X=[torch.from_numpy(DI.initial_params(w, i)).cuda() for i in range(len(shapes))],
                       vals=vals, idx=idx,
                       signs=codec.alloc_signs() if variant.startswith("signs") else None,
                       wire=codec.alloc_wire(W) if variant.startswith("wire") else None,
                       ws=codec.alloc_muon_workspace() if variant == "muon" else None)
    torch.cuda.synchronize()

    def step(s, stream):
        codec.encode(G, s["M"], s["vals"][:ne], s["idx"][:ne], stream=stream)
        if variant.startswith("signs"):
            codec.decode_signs(W, s["vals"], s["idx"], s["signs"], stream=stream)
            codec.apply_signs(s["X"], s["signs"], w.eta, w.lam, stream=stream)
        elif variant.startswith("wire"):
            wv, wi = s["wire"]
            codec.pack_wire(W, s["vals"], s["idx"], wv, wi, stream=stream)
            codec.decode_apply_wire(s["X"], W, wv, wi, B.DEMO_PHI_SIGN, w.eta, w.lam, stream=stream)
        elif variant == "aggregated":
            codec.decode_apply_subtract(s["X"], s["M"], W, s["vals"], s["idx"], B.DEMO_PHI_SIGN, w.eta, w.lam,
                                        stream=stream)
        elif variant == "muon":
            codec.decode_apply_muon(s["X"], W, s["vals"], s["idx"], s["ws"], eta=0.01, lam=w.lam, eps=1e-10,
                                    iters=12, stream=stream)
        else:
            codec.decode_apply(s["X"], W, s["vals"], s["idx"], B.DEMO_PHI_SIGN, w.eta, w.lam, stream=stream)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(st["a"], torch.cuda.current_stream())
    torch.cuda.synchronize()
    other = torch.randn(1 << 20, device="cuda")
    for r in range(3):
        g.replay()
        step(st["b"], torch.cuda.current_stream())
        other.mul_(1.0001).add_(0.5)  # the program's own eager work between replays
        torch.cuda.synchronize()
        a, b = st["a"], st["b"]
        for name in ("M", "X"):
            for i, (ta, tb) in enumerate(zip(a[name], b[name])):
                assert np.array_equal(_bits(ta), _bits(tb)), f"replay {r}: {name}[{i}] differs from the eager call"
        assert np.array_equal(_bits(a["vals"][:ne]), _bits(b["vals"][:ne])), f"replay {r}: payload values differ"
        assert np.array_equal(_bits(a["idx"][:ne]), _bits(b["idx"][:ne])), f"replay {r}: payload indices differ"
        if variant.startswith("signs"):
            assert np.array_equal(_bits(a["signs"]), _bits(b["signs"])), f"replay {r}: sign words differ"
        if variant.startswith("wire"):
            for ta, tb in zip(a["wire"], b["wire"]):
                assert np.array_equal(_bits(ta), _bits(tb)), f"replay {r}: wire arrays differ"
        assert any(bool((x != 0).any()) for x in a["M"]), "the momentum never moved"
    codec.close()
