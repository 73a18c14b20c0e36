"""Seeded synthetic inputs for the DeMo momentum codec.

This module is shared by the CPU oracle side (tests, cpu baseline) and the
HIP side (tests, bench, smoke).  It holds no step of the codec itself: only
the workload descriptions (tensor shapes and hyper-parameters) and the
seeded random draws that stand in for gradients, initial parameters and the
Gaussian matrices of the random-projection variant.

Workloads stand in for the pages' OLMo-300M / OLMo-1B training runs on
Dolma ("DeMo: Decoupled Momentum Optimization", §5 Experimental Analysis,
Evaluation Methodology): no dataset or trained weight is used; gradients are
i.i.d. Gaussian draws of the stated spread, every tensor of a set is drawn
from its own stream.

Seeding: every array comes from PCG64 seeded with
``SeedSequence([config_id, role, worker, step, tensor])`` where role 0 is a
gradient, role 1 the initial parameters, role 2 a projection draw and role 3
a synthetic payload.
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence, Tuple

import numpy as np

ROLE_GRAD = 0
ROLE_PARAM = 1
ROLE_BASIS = 2
ROLE_PAYLOAD = 3

PHI_SIGN = "sign"
PHI_IDENTITY = "identity"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One workload: a tensor list plus the codec hyper-parameters."""

    name: str
    config_id: int
    shapes: Tuple[Tuple[int, ...], ...]
    grad_std: float
    grad_bf16: bool
    beta: float
    alpha: float
    k: int
    workers: int
    phi: str
    eta: float
    lam: float
    steps: int
    param_std: float = 0.02
    random_basis: bool = False

    @property
    def n_params(self) -> int:
        return int(sum(int(np.prod(s)) for s in self.shapes))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _olmo_block(d: int) -> List[Tuple[int, ...]]:
    # QKV, attention out, MLP up, MLP down, two norm vectors
    return [(d, 3 * d), (d, d), (d, 4 * d), (4 * d, d), (d,), (d,)]


def _olmo_set(d: int, blocks: int) -> Tuple[Tuple[int, ...], ...]:
    out: List[Tuple[int, ...]] = []
    for _ in range(blocks):
        out.extend(_olmo_block(d))
    return tuple(out)


WORKLOADS = {
    # one 256x256 fp32 weight, 16 chunks
    "tiny_256": Workload("tiny_256", 1, ((256, 256),), 1e-3, False,
                         0.999, 0.2, 8, 2, PHI_SIGN, 1e-3, 0.01, 10),
    # one 4096x4096 weight, gradients drawn then rounded to bf16
    "single_4096": Workload("single_4096", 2, ((4096, 4096),), 1e-2, True,
                            0.999, 0.2, 8, 4, PHI_SIGN, 1e-3, 0.01, 20),
    # OLMo-300M-shaped set: 24 blocks at d=1024 (302,039,040 parameters)
    "olmo_300m": Workload("olmo_300m", 3, _olmo_set(1024, 24), 1e-3, False,
                          0.999, 0.2, 8, 8, PHI_SIGN, 1e-3, 0.01, 3),
    # OLMo-1B-shaped set: 16 blocks at d=2048 (805,371,904 parameters)
    "olmo_1b": Workload("olmo_1b", 4, _olmo_set(2048, 16), 1e-3, False,
                        0.999, 0.5, 32, 16, PHI_IDENTITY, 1e-3, 0.01, 3),
    # padded chunks, 1-D vectors of awkward lengths, extreme k
    "edge_mix": Workload("edge_mix", 5, ((1000, 777), (3, 5000), (777,), (1000,), (64,), (1,)),
                         1e-3, False, 0.999, 0.2, 1, 4, PHI_SIGN, 1e-3, 0.01, 3),
    # rows of 2^23 and 2^22 floats: 64 rows of the first (128 of the second) span 2^31 bytes, past what the
    # kernels' 32-bit buffer offsets cover, so their full chunks take the 64-bit-address path
    "wide_rows": Workload("wide_rows", 6, ((64, 1 << 23), (128, 1 << 22)), 1e-3, False,
                          0.999, 0.2, 8, 2, PHI_SIGN, 1e-3, 0.01, 2),
}


def rng(config_id: int, role: int, worker: int, step: int, tensor: int) -> np.random.Generator:
    ss = np.random.SeedSequence([int(config_id), int(role), int(worker), int(step), int(tensor)])
    return np.random.Generator(np.random.PCG64(ss))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    b = (b + 0x7FFF + lsb) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def gradient(w: Workload, worker: int, step: int, tensor: int) -> np.ndarray:
    """Worker ``worker``'s gradient of tensor ``tensor`` at ``step`` (float32)."""
    shape = w.shapes[tensor]
    g = rng(w.config_id, ROLE_GRAD, worker, step, tensor).standard_normal(shape, dtype=np.float32)
    g *= np.float32(w.grad_std)
    if w.grad_bf16:
        g = round_to_bf16(g)
    return g


def initial_params(w: Workload, tensor: int) -> np.ndarray:
    shape = w.shapes[tensor]
    x = rng(w.config_id, ROLE_PARAM, 0, 0, tensor).standard_normal(shape, dtype=np.float32)
    return x * np.float32(w.param_std)


def gaussian_matrix(w: Workload, step: int, which: int, s: int = 64) -> np.ndarray:
    """Fresh N(0, 1) s x s draw for the random-projection variant (float64).

    The same draw is used by every worker at a step; ``which`` is 0 for the
    dimension-0 matrix and 1 for the dimension-1 matrix.
    """
    return rng(w.config_id, ROLE_BASIS, which, step, 0).standard_normal((s, s))


def synthetic_payload(chunks: Sequence[Tuple[int, int, int]], workers: int, seed: int, scale: float = 1e-5,
                      specials: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Payloads of ``workers`` workers in the codec's layout, drawn directly.

    ``chunks`` lists, per tensor, (chunk count, entries per chunk, index
    range per chunk).  Every chunk gets distinct indices in ascending order
    and N(0, scale^2) values.  With ``specials`` about one value in four is
    replaced by a bit pattern that exercises float32 -> bfloat16 rounding:
    exact halfway cases, one ulp either side of them, signed zeros,
    subnormals, the largest finite float and the float32 maximum rounded.
    Returns float32 values and uint16 indices, worker-major.
    """
    vals, idx = [], []
    for wk in range(workers):
        r = rng(seed, ROLE_PAYLOAD, wk, 0, 0)
        for n, keff, numel in chunks:
            for _ in range(n):
                idx.append(np.sort(r.permutation(numel)[:keff]).astype(np.uint16))
                vals.append((r.standard_normal(keff) * scale).astype(np.float32))
    v = np.concatenate(vals) if vals else np.zeros(0, np.float32)
    i = np.concatenate(idx) if idx else np.zeros(0, np.uint16)
    if specials and v.size:
        r = rng(seed, ROLE_PAYLOAD, workers, 1, 0)
        pick = r.random(v.size) < 0.25
        hi = r.integers(0, 0x7F7F, v.size, dtype=np.uint32) | (r.integers(0, 2, v.size, dtype=np.uint32) << 15)
        low = r.choice(np.array([0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF], np.uint32), v.size)
        bits = (hi << 16) | low
        fixed = np.array([0x00000000, 0x80000000, 0x00000001, 0x807FFFFF, 0x7F7FFFFF, 0xFF7F7FFF,
                          0x3F808000, 0x3F818000, 0x00008000, 0x80018000], np.uint32)
        bits[:min(fixed.size, v.size)] = fixed[:min(fixed.size, v.size)]
        pick[:min(fixed.size, v.size)] = True
        v = np.where(pick, bits.view(np.float32), v).astype(np.float32)
    return v, i


# ---------------------------------------------------------------------------
# device-side draws for full-size lists
# ---------------------------------------------------------------------------
#
# Host PCG64 draws of the OLMo-shaped lists (hundreds of millions of values
# per worker and step) would take minutes, so full-size runs draw on the
# device with torch's seeded generator instead.  The values are inputs, not
# codec results: a test copies the chunks it samples back to the host and
# hands exactly those float32 values to the oracle.

def device_seed(config_id: int, role: int, worker: int, step: int, tensor: int) -> int:
    """A 63-bit seed for torch's generator, derived from the same key as ``rng``."""
    ss = np.random.SeedSequence([int(config_id), int(role), int(worker), int(step), int(tensor)])
    return int(ss.generate_state(2, dtype=np.uint32).view(np.uint64)[0] >> np.uint64(1))


def device_normal(shape, std: float, seed: int, device, bf16: bool = False):
    """float32 (or bf16-rounded, returned as bf16) N(0, std^2) draw on ``device``."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    t = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    t.mul_(float(std))
    return t.to(torch.bfloat16) if bf16 else t


def device_gradient(w: Workload, worker: int, step: int, tensor: int, device):
    return device_normal(w.shapes[tensor], w.grad_std, device_seed(w.config_id, ROLE_GRAD, worker, step, tensor),
                         device, w.grad_bf16)


def device_initial_params(w: Workload, tensor: int, device):
    return device_normal(w.shapes[tensor], w.param_std, device_seed(w.config_id, ROLE_PARAM, 0, 0, tensor), device)
