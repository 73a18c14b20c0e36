"""The Muon decode on the library's static scratch against the same decode on a caller workspace.

demo_decode_apply_muon_noalloc runs the kernels of demo_decode_apply_muon
with the workspace taken from a static device array; the two must give
bitwise the same parameters.  Two calls in a row on one scratch, the second
with a smaller list (the scratch keeps the first call's contents).  The
caller workspace is filled with NaN bit patterns first, so neither path may
read workspace memory it has not written.  A list whose workspace exceeds the
scratch is refused before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import demo_inputs as DI
import parity as PR
from communication_compressed_optimizer_demo_amd import binding as B

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()
    return torch.device("cuda:0")


def _payload(shapes, k, W, seed):
    lay = [(n, keff, 4096 if len(sh) == 2 else 64) for (n, keff, _), sh in zip(PR.layout(shapes, k), shapes)]
    vals, idx = DI.synthetic_payload(lay, W, seed=seed, scale=1.0)
    return torch.from_numpy(vals).cuda(), torch.from_numpy(idx.view(np.int16)).cuda()


@pytest.mark.parametrize("avg", [B.DEMO_AVG_CONTRIBUTORS, B.DEMO_AVG_WORKERS])
def test_noalloc_muon_matches_workspace_muon(dev, avg):
    w = DI.WORKLOADS["tiny_256"]
    cases = [([(256, 384), (300,), (130, 70), (384, 256)], 16, 3, 1e-2),
             ([(64, 96), (50,)], 8, 2, 1e-3)]   # second call: a smaller list
    for call, (shapes, k, W, eps) in enumerate(cases):
        say(f"  no-alloc Muon call {call}: shapes {shapes}, k={k}, W={W}, "
            f"workspace {B.demo_muon_workspace(shapes)} bytes of {B.DEMO_MUON_SCRATCH_BYTES}")
        assert B.demo_muon_workspace(shapes) <= B.DEMO_MUON_SCRATCH_BYTES
        codec = B.Codec(shapes, k, w.beta, w.alpha)
        vals, idx = _payload(shapes, k, W, seed=60 + call)
        X0 = [torch.from_numpy(DI.initial_params(w.replace(shapes=tuple(shapes)), i)).cuda()
              for i in range(len(shapes))]
        Xa = [x.clone() for x in X0]
        Xb = [x.clone() for x in X0]
        ws = codec.alloc_muon_workspace()
        ws.fill_(0xFF)  # NaN bit patterns
        codec.decode_apply_muon(Xa, W, vals, idx, ws, eta=0.05, lam=0.01, eps=eps, iters=20, avg=avg)
        codec.decode_apply_muon_noalloc(Xb, W, vals, idx, eta=0.05, lam=0.01, eps=eps, iters=20, avg=avg)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(Xa, Xb)):
            an, bn = a.cpu().numpy(), b.cpu().numpy()
            assert np.isfinite(an).all(), f"call {call} tensor {i}: non-finite parameters"
            assert not np.array_equal(an, X0[i].cpu().numpy()), f"call {call} tensor {i}: parameters unchanged"
            assert np.array_equal(an.view(np.uint32), bn.view(np.uint32)), \
                f"call {call} tensor {i}: static-scratch decode differs from the workspace decode"
        codec.close()


def test_noalloc_refuses_a_list_beyond_the_scratch(dev):
    shapes = [(2048, 2048)]
    need = B.demo_muon_workspace(shapes)
    assert need > B.DEMO_MUON_SCRATCH_BYTES
    codec = B.Codec(shapes, 8)
    vals, idx = codec.alloc_payload(1)
    X = [torch.zeros(shapes[0], device="cuda")]
    with pytest.raises(B.DemoError) as e:
        codec.decode_apply_muon_noalloc(X, 1, vals, idx)
    assert e.value.status == 3 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert not X[0].any(), "a refused call touched the parameters"
    codec.close()
