"""Parity of the HIP codec with the CPU oracle, through the C ABI.

Every case runs W simulated workers: each worker encodes its own seeded
gradients on the GPU and in the oracle, both free-running from the same
initial state; then all W payloads are decoded and applied on the GPU and
in the oracle.  Comparison rules (tolerances, near-tie and sign exemptions)
are in parity.py.
"""
import numpy as np
import pytest
import torch

import demo_inputs as DI
import parity as PR
from communication_compressed_optimizer_demo_amd import binding as B
from oracle import demo_oracle as O

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()
    return torch.device("cuda:0")


class Sim:
    """W workers of one workload, GPU next to the oracle.

    After every step's decode the same payloads are decoded once more into a
    zero tensor with eta = 1, lambda = 0 and phi = identity, which leaves
    exactly -M* there: M* itself is compared with the oracle's element by
    element (parity.compare_mstar), not only through the parameters.
    """

    def __init__(self, w: DI.Workload, *, plain=False, avg="count", inputs=None, identity=False, aggregated=False,
                 signs=False, chunk=64, wire=False, noise=None, mstar=True):
        self.w = w
        self.s = chunk
        self.noise = noise if noise is not None else (PR.NOISE_DENSE if w.random_basis else PR.NOISE)
        self.mstar = mstar
        self.wire = wire  # payloads go through the compact wire format: pack, then decode_apply_wire
        assert not (wire and (signs or aggregated))
        self.signs = signs  # one-bit download: decode_signs, then apply_signs (phi = sign)
        assert not (signs and (aggregated or w.phi != "sign"))
        self.plain = plain
        self.identity = identity
        self.aggregated = aggregated
        self.avg = avg
        self.inputs = inputs  # optional callable (worker, step, tensor) -> float32 gradient
        self.shapes = [tuple(s) for s in w.shapes]
        self.codec = B.Codec(self.shapes, w.k, w.beta, w.alpha, plain, identity=identity, aggregated=aggregated,
                             chunk=chunk)
        self.lay = PR.layout(self.shapes, w.k, chunk)
        nc, ne, eb = B.demo_plan(self.shapes, w.k, chunk)
        assert ne == sum(n * k for n, k, _ in self.lay)
        assert eb[:-1] == [e for _, _, e in self.lay]
        W = w.workers
        self.M_gpu = [[torch.zeros(s, dtype=torch.float32, device="cuda") for s in self.shapes] for _ in range(W)]
        self.M_or = [[np.zeros(s, dtype=np.float32) for s in self.shapes] for _ in range(W)]
        X0 = [DI.initial_params(w, i) for i in range(len(self.shapes))]
        self.X_gpu = [torch.from_numpy(x.copy()).cuda() for x in X0]
        self.X_or = [x.copy() for x in X0]
        self.vals, self.idx = self.codec.alloc_payload(W)
        self.probe = [torch.zeros(sh, dtype=torch.float32, device="cuda") for sh in self.shapes]
        self.sign_words = self.codec.alloc_signs() if signs else None
        if wire:
            self.wv, self.wi = self.codec.alloc_wire(W)
            self.wire_bytes = B.demo_wire_size(self.codec.n_entries, chunk)[1]
            self.xdiv = [np.zeros(n, dtype=bool) for n, _, _ in self.lay]  # chunks whose X follows other codes
        self.cdiv = [[np.zeros(n, dtype=bool) for n, _, _ in self.lay] for _ in range(W)]
        self.ediv = [None for _ in self.shapes]
        self.report = PR.EncodeReport()

    def grad(self, worker, step, i):
        if self.inputs is not None:
            return self.inputs(worker, step, i)
        return DI.gradient(self.w, worker, step, i)

    def basis(self, step):
        if self.identity:
            eye = np.eye(64)
            return eye, eye, None, None
        if not self.w.random_basis:
            return None, None, None, None
        P0 = O.orthonormal_rows(DI.gaussian_matrix(self.w, step, 0)).astype(np.float32)
        P1 = O.orthonormal_rows(DI.gaussian_matrix(self.w, step, 1)).astype(np.float32)
        return P0, P1, torch.from_numpy(P0).cuda(), torch.from_numpy(P1).cuda()

    def step(self, t):
        w = self.w
        W = w.workers
        P0, P1, P0d, P1d = self.basis(t)
        ne = self.codec.n_entries
        phi_c = B.DEMO_PHI_SIGN if w.phi == "sign" else B.DEMO_PHI_IDENTITY
        avg_c = B.DEMO_AVG_CONTRIBUTORS if self.avg == "count" else B.DEMO_AVG_WORKERS
        or_vals = [[None] * W for _ in self.shapes]
        or_idx = [[None] * W for _ in self.shapes]
        or_q = [[None] * W for _ in self.shapes]
        for wk in range(W):
            G = [self.grad(wk, t, i) for i in range(len(self.shapes))]
            gd = [torch.from_numpy(g).cuda() for g in G]
            if w.grad_bf16:
                gd = [g.to(torch.bfloat16) for g in gd]
            say(f"  [{w.name}] step {t} worker {wk}: GPU encode")
            self.codec.encode(gd, self.M_gpu[wk], self.vals[wk * ne:(wk + 1) * ne],
                              self.idx[wk * ne:(wk + 1) * ne], P0d, P1d)
            torch.cuda.synchronize()
            gv = self.vals[wk * ne:(wk + 1) * ne].cpu().numpy()
            gi = self.idx[wk * ne:(wk + 1) * ne].cpu().numpy().view(np.uint16)
            for i, shp in enumerate(self.shapes):
                n, keff, e0 = self.lay[i]
                out = O.encode(self.M_or[wk][i], G[i], beta=w.beta, alpha=w.alpha, k=w.k, plain=self.plain,
                               P0=P0, P1=P1, s=self.s, subtract="aggregated" if self.aggregated else "local")
                gM = self.M_gpu[wk][i].cpu().numpy()
                self.cdiv[wk][i] = PR.compare_encode(
                    out, shp, keff, 0.0 if self.aggregated else w.alpha,
                    O.dct_basis(self.s) if P0 is None else P0, O.dct_basis(self.s) if P1 is None else P1, gM,
                    gv[e0:e0 + n * keff].reshape(n, keff), gi[e0:e0 + n * keff].reshape(n, keff),
                    self.cdiv[wk][i], self.report, where=f"{w.name} step {t} worker {wk} tensor {i} {shp}", s=self.s,
                    noise=self.noise)
                self.M_or[wk][i] = out["M"]
                or_vals[i][wk] = out["values"]
                or_idx[i][wk] = out["idx"]
                or_q[i][wk] = out["terms_chunks"]
        if self.wire:
            return self.step_wire(t, or_vals, or_idx, or_q, phi_c, avg_c, P0, P1, P0d, P1d)
        say(f"  [{w.name}] step {t}: GPU decode/apply over {W} payloads")
        if self.aggregated:
            # worker 0 updates the parameters and its momentum in one pass, the others their momentum only
            self.codec.decode_apply_subtract(self.X_gpu, self.M_gpu[0], W, self.vals, self.idx, phi_c, w.eta, w.lam,
                                             avg_c, P0d, P1d)
            for wk in range(1, W):
                self.codec.decode_apply_subtract(None, self.M_gpu[wk], W, self.vals, self.idx, phi_c, w.eta, w.lam,
                                                 avg_c, P0d, P1d)
        elif self.signs:
            self.sign_words.fill_(-1)  # every word must be rewritten, padding bits included
            self.codec.decode_signs(W, self.vals, self.idx, self.sign_words, avg_c, P0d, P1d)
            torch.cuda.synchronize()
            words = self.sign_words.cpu().numpy().view(np.uint64)
            self.codec.apply_signs(self.X_gpu, self.sign_words, w.eta, w.lam)
        else:
            self.codec.decode_apply(self.X_gpu, W, self.vals, self.idx, phi_c, w.eta, w.lam, avg_c, P0d, P1d)
        torch.cuda.synchronize()
        probe = self.probe_mstar(avg_c, P0d, P1d)
        for i, shp in enumerate(self.shapes):
            dec = O.decode_apply(self.X_or[i], np.stack(or_vals[i]), np.stack(or_idx[i]), phi=w.phi, eta=w.eta,
                                 lam=w.lam, mode=self.avg, P0=P0, P1=P1, s=self.s)
            cd = np.zeros_like(self.cdiv[0][i])
            for wk in range(W):
                cd |= self.cdiv[wk][i]
            if probe is not None:
                PR.compare_mstar(dec["Qabs"], dec["Mstar"], -probe[i], shp, cd, noise=self.noise,
                                 where=f"{w.name} step {t} tensor {i} {shp} (M*)", s=self.s)
            if self.signs:
                wb = self.codec.sign_word_begin
                PR.compare_signs(dec["Mstar"], shp, words[wb[i]:wb[i + 1]], cd,
                                 where=f"{w.name} step {t} tensor {i} {shp} (signs)", s=self.s)
                dec = {"X": O.apply_signs(self.X_or[i], O.pack_signs(dec["Mstar"], self.s), eta=w.eta, lam=w.lam,
                                          s=self.s),
                       "Mstar": dec["Mstar"]}
            self.ediv[i] = PR.compare_decode(dec, shp, w.phi, w.eta, self.X_gpu[i].cpu().numpy(), cd, self.ediv[i],
                                             where=f"{w.name} step {t} tensor {i} {shp}", s=self.s)
            self.X_or[i] = dec["X"]
            if self.aggregated:
                for wk in range(W):
                    self.M_or[wk][i] = O.subtract_aggregated(self.M_or[wk][i], dec["Mstar"], w.alpha)
                    PR.compare_momentum(self.M_or[wk][i], self.M_gpu[wk][i].cpu().numpy(), shp, cd,
                                        where=f"{w.name} step {t} worker {wk} tensor {i} {shp} (aggregated)", s=self.s,
                                        scale=O.hp(w.alpha) * dec["Mstar"], noise=self.noise)
                    self.cdiv[wk][i] = self.cdiv[wk][i] | cd

    def probe_mstar(self, avg_c, P0d, P1d, wire=False):
        """-M* of this step's payloads (host arrays per tensor), or None when disabled."""
        if not self.mstar:
            return None
        for t in self.probe:
            t.zero_()
        if wire:
            self.codec.decode_apply_wire(self.probe, self.w.workers, self.wv, self.wi, B.DEMO_PHI_IDENTITY, 1.0, 0.0,
                                         avg_c, P0d, P1d)
        else:
            self.codec.decode_apply(self.probe, self.w.workers, self.vals, self.idx, B.DEMO_PHI_IDENTITY, 1.0, 0.0,
                                    avg_c, P0d, P1d)
        torch.cuda.synchronize()
        return [t.cpu().numpy() for t in self.probe]

    def step_wire(self, t, or_vals, or_idx, or_q, phi_c, avg_c, P0, P1, P0d, P1d):
        """Pack all W payloads into the wire format, check it, decode from it."""
        w = self.w
        W = w.workers
        ne = self.codec.n_entries
        say(f"  [{w.name}] step {t}: GPU wire pack + decode/apply over {W} payloads")
        self.wv.fill_(-1)
        self.wi.fill_(255)  # padding bytes must be rewritten as zero
        self.codec.pack_wire(W, self.vals, self.idx, self.wv, self.wi)
        torch.cuda.synchronize()
        wv = self.wv.cpu().numpy().view(np.uint16)
        wi = self.wi.cpu().numpy()
        self.codec.decode_apply_wire(self.X_gpu, W, self.wv, self.wi, phi_c, w.eta, w.lam, avg_c, P0d, P1d)
        torch.cuda.synchronize()
        probe = self.probe_mstar(avg_c, P0d, P1d, wire=True)
        wb = self.wire_bytes
        nbits = ne * O.wire_index_bits(self.s)
        used = (nbits + 7) // 8
        codes, gidx = [], []
        for wk in range(W):
            blk = wi[wk * wb:(wk + 1) * wb]
            assert not blk[used:].any(), f"{w.name} step {t} worker {wk}: wire padding not zero"
            if nbits % 8:
                assert blk[used - 1] >> (nbits % 8) == 0, f"{w.name} step {t} worker {wk}: wire padding bits set"
            codes.append(wv[wk * ne:(wk + 1) * ne])
            gidx.append(O.unpack_wire(wv[wk * ne:(wk + 1) * ne], blk, ne, self.s)[1])
        for i, shp in enumerate(self.shapes):
            n, keff, e0 = self.lay[i]
            cd = self.xdiv[i].copy()
            for wk in range(W):
                cd |= self.cdiv[wk][i]
            for wk in range(W):
                sl = slice(e0, e0 + n * keff)
                self.xdiv[i] |= PR.compare_wire(or_vals[i][wk], or_idx[i][wk], or_q[i][wk],
                                                codes[wk][sl].reshape(n, keff), gidx[wk][sl].reshape(n, keff), cd,
                                                where=f"{w.name} step {t} worker {wk} tensor {i} {shp} (wire)",
                                                noise=self.noise)
            cd |= self.xdiv[i]
            # the oracle decodes its own payload as the wire carries it: values rounded to bfloat16
            vr = [O.unpack_wire(*O.pack_wire(or_vals[i][wk], or_idx[i][wk], self.s), n * keff, self.s)[0]
                  .reshape(n, keff) for wk in range(W)]
            dec = O.decode_apply(self.X_or[i], np.stack(vr), np.stack(or_idx[i]), phi=w.phi, eta=w.eta, lam=w.lam,
                                 mode=self.avg, P0=P0, P1=P1, s=self.s)
            if probe is not None:
                PR.compare_mstar(dec["Qabs"], dec["Mstar"], -probe[i], shp, cd, noise=self.noise,
                                 where=f"{w.name} step {t} tensor {i} {shp} (wire M*)", s=self.s)
            self.ediv[i] = PR.compare_decode(dec, shp, w.phi, w.eta, self.X_gpu[i].cpu().numpy(), cd, self.ediv[i],
                                             where=f"{w.name} step {t} tensor {i} {shp} (wire)", s=self.s)
            self.X_or[i] = dec["X"]

    def run(self, steps, max_tie_fraction=0.02):
        for t in range(steps):
            self.step(t)
        r = self.report
        say(f"  [{self.w.name}] chunks checked {r.chunks}: exact {r.exact}, near-tie {r.ties}, skipped {r.skipped}")
        assert r.ties + r.skipped <= max(2, max_tie_fraction * r.chunks), "too many near-tie divergences"
        return r


def test_single_chunk_one_worker(dev):
    w = DI.WORKLOADS["tiny_256"].replace(shapes=((64, 64),), workers=1, steps=2)
    Sim(w).run(2)


def test_tiny_256_ten_steps(dev):
    w = DI.WORKLOADS["tiny_256"]
    Sim(w).run(w.steps)


@pytest.mark.parametrize("k,alpha,rand", [(1, 0.2, False), (4096, 1.0, False), (4096, 0.2, False),
                                           (4, 0.2, True), (4096, 1.0, True), (37, 0.5, False)])
def test_edge_mix(dev, k, alpha, rand):
    w = DI.WORKLOADS["edge_mix"].replace(k=k, alpha=alpha, random_basis=rand)
    Sim(w).run(w.steps)


def test_single_4096_bf16_gradients(dev):
    w = DI.WORKLOADS["single_4096"]
    Sim(w).run(2)


def test_bf16_gradients_random_basis(dev):
    """bfloat16 gradients with a caller basis: the matrix-core transform behind the bfloat16 loads."""
    w = DI.WORKLOADS["single_4096"].replace(name="bf16_random", shapes=((256, 320), (130,)), random_basis=True)
    Sim(w).run(2)


@pytest.mark.parametrize("k", [1, 8, 64, 4096])
def test_tiny_and_ragged_shapes(dev, k):
    w = DI.WORKLOADS["tiny_256"].replace(
        name=f"ragged_k{k}", shapes=((1, 1), (1, 64), (64, 1), (2, 3), (65, 65), (1,), (63,), (65,), (130,)),
        k=k, workers=2)
    Sim(w).run(2)


@pytest.mark.parametrize("plain,avg,phi", [(True, "count", "sign"), (False, "workers", "sign"),
                                           (False, "count", "identity"), (True, "workers", "identity")])
def test_momentum_form_average_and_phi(dev, plain, avg, phi):
    w = DI.WORKLOADS["tiny_256"].replace(name=f"modes_{plain}_{avg}_{phi}", shapes=((256, 192), (300,)),
                                         phi=phi, workers=3)
    Sim(w, plain=plain, avg=avg).run(3)


def test_unit_scale_inputs(dev):
    """Unit-scale momenta exercise the relative tolerance, not the 1e-7 floor."""
    w = DI.WORKLOADS["tiny_256"].replace(name="unit_scale", shapes=((192, 320), (129,)), grad_std=1.0,
                                         param_std=1.0, beta=0.9, k=16, workers=3, eta=0.01)
    Sim(w, plain=True).run(3)


UNIT_CASES = {
    # name: (Sim keyword arguments, workload overrides)
    "s64_damped": (dict(), dict()),
    "s64_damped_k100_w20": (dict(), dict(k=100, workers=20)),
    "s128_damped": (dict(chunk=128), dict(shapes=((256, 300), (130,)))),
    "s128_plain_workers": (dict(chunk=128, plain=True, avg="workers"), dict(shapes=((300, 256), (257,)), phi="identity")),
    "s128_k100": (dict(chunk=128), dict(shapes=((256, 256), (300,)), k=100, workers=5)),
    "identity": (dict(identity=True), dict()),
    "identity_workers": (dict(identity=True, avg="workers"), dict(phi="identity")),
    "caller_basis": (dict(), dict(random_basis=True)),
    "caller_basis_plain": (dict(plain=True), dict(random_basis=True, phi="identity")),
    "aggregated": (dict(aggregated=True), dict()),
    "aggregated_s128": (dict(aggregated=True, chunk=128), dict(shapes=((256, 128), (200,)))),
    "aggregated_caller_basis": (dict(aggregated=True), dict(random_basis=True, k=4)),
}


@pytest.mark.parametrize("case", sorted(UNIT_CASES))
def test_unit_scale_variants(dev, case):
    """Unit-scale gradients and parameters (std 1) through every variant: the encode's payload and
    momentum, M* and the parameters all at a scale where the relative tolerance decides."""
    kw, over = UNIT_CASES[case]
    base = dict(name=f"unit_{case}", shapes=((192, 320), (129,)), grad_std=1.0, param_std=1.0, k=16, workers=3,
                eta=0.01)
    base.update(over)
    w = DI.WORKLOADS["tiny_256"].replace(**base)
    Sim(w, **kw).run(3)


def test_long_run_drift(dev):
    """The 256x256 workload free-running for 700 steps (the pages' momentum half-life at beta = 0.999 is
    about 693 steps), GPU and oracle each from their own state.  The momentum's rounding differences
    accumulate over the momentum's memory; the floor each step needs (per unit of chunk norm) must stay
    under parity.NOISE, the same floor as the short runs, and every chunk must stay on the oracle's top-k
    sets or within a tie window."""
    w = DI.WORKLOADS["tiny_256"].replace(name="long_run", steps=700)
    sim = Sim(w)
    curve, worst = [], {}
    for t in range(w.steps):
        sim.step(t)
        for kind in list(PR.STATS):
            worst[kind] = max(worst.get(kind, 0.0), PR.STATS[kind])
        curve.append(PR.STATS.get("momentum", 0.0))
        PR.STATS.clear()
        if t + 1 in (1, 10, 50, 100, 200, 300, 400, 500, 600, 700):
            say(f"  [long_run] step {t + 1}: momentum floor needed this step {curve[-1]:.3e} "
                f"(2^{np.log2(max(curve[-1], 1e-300)):.1f}), largest so far {max(curve):.3e}")
    PR.STATS.update(worst)
    r = sim.report
    say(f"  [long_run] chunks checked {r.chunks}: exact {r.exact} ({r.exact / r.chunks:.4f}), near-tie {r.ties}, "
        f"skipped {r.skipped}")
    assert max(curve) <= PR.NOISE
    assert r.ties + r.skipped <= 0.02 * r.chunks


def _sum_order_payloads(s, keff, c, split):
    """Payloads of 4 workers for one s x s chunk (keff entries each, ascending indices) where
    coefficient c is at entry position >= 64 for worker 0 and < 64 for workers 1 and 2; worker 3
    lacks it.  split: the three values at c."""
    numel = s * s
    below = list(range(0, 30))
    above_hi = list(range(c + 1, c + 1 + (keff - 31)))
    assert above_hi[-1] < numel
    w0 = sorted(set(range(c - (keff - 1), c)) | {c})  # c last: position keff - 1 >= 64
    w12 = sorted(set(below) | {c} | set(above_hi))     # c at position 30 < 64
    w3 = sorted(set(range(c - keff, c)))
    vals, idx = [], []
    for wk, ix in enumerate([w0, w12, w12, w3]):
        assert len(ix) == keff
        v = np.zeros(keff, np.float32)
        if wk < 3:
            v[ix.index(c)] = split[wk]
        vals.append(v)
        idx.append(np.array(ix, np.uint16))
    return np.concatenate(vals), np.concatenate(idx)


@pytest.mark.parametrize("chunk,c", [(64, 4000), (128, 16000)])
def test_summation_follows_worker_order(dev, chunk, c):
    """Coefficients are summed in worker order 0..W-1 also when one worker holds the coefficient in its
    second 64-entry block and later workers in their first (keff = 100).  With values 1, 2^-24, 2^-24 the
    float32 sum in worker order is 1, the same as a payload that sends 1, 0, 0: M* must be bitwise equal
    for the two.  Summed block by block (workers 1 and 2 first) it would be 1 + 2^-23.  Repeated calls are
    bitwise equal too, also with 20 workers."""
    keff = 100
    shapes = ((chunk, chunk),)
    codec = B.Codec(shapes, keff, chunk=chunk)
    outs = []
    for split in ([1.0, 2.0 ** -24, 2.0 ** -24], [1.0, 0.0, 0.0]):
        v, ix = _sum_order_payloads(chunk, keff, c, split)
        X = [torch.zeros(shapes[0], device="cuda")]
        codec.decode_apply(X, 4, torch.from_numpy(v).cuda(), torch.from_numpy(ix.view(np.int16)).cuda(),
                           B.DEMO_PHI_IDENTITY, 1.0, 0.0, B.DEMO_AVG_WORKERS)
        torch.cuda.synchronize()
        outs.append(X[0].cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), "coefficients not summed in worker order"
    # determinism with W = 20 workers, keff = 100 (several register batches and entry blocks)
    lay = [(n, k, chunk * chunk if len(sh) == 2 else chunk) for (n, k, _), sh in
           zip(PR.layout(((chunk, 2 * chunk), (300,)), keff, chunk), ((chunk, 2 * chunk), (300,)))]
    codec.close()
    codec = B.Codec(((chunk, 2 * chunk), (300,)), keff, chunk=chunk)
    v, ix = DI.synthetic_payload(lay, 20, seed=91, scale=1.0)
    vd, idd = torch.from_numpy(v).cuda(), torch.from_numpy(ix.view(np.int16)).cuda()
    res = []
    for _ in range(2):
        X = [torch.zeros((chunk, 2 * chunk), device="cuda"), torch.zeros((300,), device="cuda")]
        codec.decode_apply(X, 20, vd, idd, B.DEMO_PHI_IDENTITY, 1.0, 0.0)
        torch.cuda.synchronize()
        res.append([x.cpu().numpy() for x in X])
    for a, b in zip(*res):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    codec.close()


def test_degenerate_chunks(dev):
    """All-zero, constant and single-basis-function gradients (exact ties in the top-k)."""
    P = O.dct_basis()
    w = DI.WORKLOADS["tiny_256"].replace(name="degenerate", shapes=((64, 64), (64, 128), (64, 64), (200,)),
                                         k=8, workers=2)

    def inputs(worker, step, i):
        if i == 0:
            return np.zeros((64, 64), np.float32)
        if i == 1:
            return np.full((64, 128), 1e-3 * (worker + 1), np.float32)
        if i == 2:
            return (1e-3 * np.outer(P[3], P[7])).astype(np.float32)
        return np.full((200,), -2e-3, np.float32)

    # constant and single-frequency chunks tie exactly at zero: every such chunk may take the window path
    r = Sim(w, inputs=inputs).run(2, max_tie_fraction=1.0)
    assert r.exact >= 4


def test_deterministic_repeat(dev):
    w = DI.WORKLOADS["tiny_256"].replace(name="repeat", shapes=((256, 256), (100,)), workers=3)
    results = []
    for _ in range(2):
        codec = B.Codec(w.shapes, w.k, w.beta, w.alpha)
        M = [[torch.zeros(s, device="cuda") for s in w.shapes] for _ in range(3)]
        X = [torch.from_numpy(DI.initial_params(w, i)).cuda() for i in range(2)]
        v, ix = codec.alloc_payload(3)
        ne = codec.n_entries
        for t in range(3):
            for wk in range(3):
                g = [torch.from_numpy(DI.gradient(w, wk, t, i)).cuda() for i in range(2)]
                codec.encode(g, M[wk], v[wk * ne:(wk + 1) * ne], ix[wk * ne:(wk + 1) * ne])
            codec.decode_apply(X, 3, v, ix, B.DEMO_PHI_SIGN, w.eta, w.lam)
        torch.cuda.synchronize()
        results.append([t.cpu().numpy() for t in [v, ix] + X + M[0] + M[1] + M[2]])
    for a, b in zip(*results):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_list_longer_than_one_launch(dev):
    """More tensors than one launch's table holds: the call splits into launches, vectors first in each."""
    shapes = []
    for i in range(B.DEMO_MAX_TENSORS_PER_LAUNCH + 7):
        shapes.append([(64, 64), (100,), (65, 3), (1,), (70, 130)][i % 5])
    w = DI.WORKLOADS["tiny_256"].replace(name="long_list", shapes=tuple(shapes), workers=2, k=5)
    Sim(w).run(2)


@pytest.mark.parametrize("k,alpha", [(8, 0.2), (1, 1.0), (4096, 0.5)])
def test_identity_basis(dev, k, alpha):
    """P0 = P1 = I: top-k and subtraction act on the momentum itself (padded chunks and vectors included)."""
    w = DI.WORKLOADS["edge_mix"].replace(name=f"identity_k{k}", k=k, alpha=alpha)
    Sim(w, identity=True).run(w.steps)


@pytest.mark.parametrize("name,k,alpha,rand", [("tiny_256", 8, 0.2, False), ("edge_mix", 4, 0.5, False),
                                                ("edge_mix", 4096, 1.0, True)])
def test_aggregated_subtraction(dev, name, k, alpha, rand):
    """The summary page's reading of the momentum subtraction: every worker removes alpha * M*."""
    w = DI.WORKLOADS[name].replace(name=f"aggregated_{name}_k{k}", k=k, alpha=alpha, random_basis=rand, workers=3)
    Sim(w, aggregated=True).run(3)


@pytest.mark.parametrize("avg", ["count", "workers"])
def test_more_workers_than_one_batch(dev, avg):
    """W = 20 (> 16 payloads per register batch): the decode's general averaging path."""
    w = DI.WORKLOADS["tiny_256"].replace(name=f"w20_{avg}", shapes=((128, 192), (130,)), workers=20, k=16)
    Sim(w, avg=avg).run(2)


@pytest.mark.parametrize("k,chunk", [(4096, 64), (8, 64), (16384, 128), (8, 128)])
def test_maximum_workers(dev, k, chunk):
    """W = 255, the most the 8-bit contributor counts allow: at lossless k every coefficient is sent by
    all 255 workers (count 255 everywhere); at k = 8 the counts vary per coefficient."""
    w = DI.WORKLOADS["tiny_256"].replace(name=f"w255_k{k}_s{chunk}", shapes=((chunk, 2 * chunk), (100,)),
                                         workers=255, k=k)
    Sim(w, chunk=chunk).run(2)


@pytest.mark.parametrize("name,k,avg,rand", [("tiny_256", 8, "count", False), ("edge_mix", 4, "workers", False),
                                              ("edge_mix", 37, "count", True)])
def test_one_bit_sign_download(dev, name, k, avg, rand):
    """Server packs sign(M*) into bits, workers apply them: bits against the oracle's packing,
    parameters against the oracle's apply (padded chunks, vectors and a random basis included)."""
    w = DI.WORKLOADS[name].replace(name=f"signs_{name}_k{k}", k=k, random_basis=rand, workers=3, phi="sign")
    Sim(w, avg=avg, signs=True).run(3)


@pytest.mark.parametrize("shapes,k,avg,W", [
    (((256, 384), (1000,)), 16, "count", 3),
    (((128, 128), (300, 77), (129,)), 4, "workers", 2),
    (((128, 256), (300,)), 200, "count", 20),      # keff > 64, several worker batches
    (((256, 128),), 16384, "count", 2),            # lossless
])
def test_one_bit_sign_download_chunk128(dev, shapes, k, avg, W):
    """The one-bit download at chunk edge 128: 256 words per matrix chunk (two per chunk row), two per
    vector chunk; bits against the oracle's packing, parameters against the oracle's apply."""
    w = DI.WORKLOADS["tiny_256"].replace(name=f"signs128_k{k}_W{W}", shapes=shapes, k=k, workers=W, phi="sign")
    Sim(w, avg=avg, signs=True, chunk=128).run(3)


@pytest.mark.parametrize("chunk", [64, 128])
def test_one_bit_sign_download_ragged_and_zero(dev, chunk):
    """Tiny and ragged shapes plus an all-zero tensor (M* = 0 reads as +1 on both sides).

    A 1x1 tensor is a single element in its chunk, so Q[u][v] = x P[u][0] P[v][0] = Q[v][u]: every
    off-diagonal magnitude ties exactly with its transpose, and float32 rounding breaks each tie either
    way on either side.  Those chunks take the tie window (every GPU set is checked to be a valid top-k
    set), so this test allows a tenth of its 64-68 chunks to do so."""
    s = chunk
    w = DI.WORKLOADS["tiny_256"].replace(
        name=f"signs_ragged_s{s}", shapes=((1, 1), (2, 3), (s + 1, s + 1), (s, s), (1,), (s - 1,), (2 * s + 2,),
                                           (3 * s + 70,)), k=5, workers=2)

    def inputs(worker, step, i):
        if i == 3:
            return np.zeros((s, s), np.float32)
        return DI.gradient(w, worker, step, i)

    Sim(w, inputs=inputs, signs=True, chunk=chunk).run(2, max_tie_fraction=0.1)


def test_sign_download_on_zero_momentum_differs_from_signum_as_documented(dev):
    """An all-zero tensor (M* = 0 everywhere): the Signum decode applies sign(0) = 0, X(1 - eta lambda);
    the one-bit download cannot carry 0 and applies +1, X - eta (1 + lambda X).  Both against the oracle."""
    shapes = ((64, 128), (100,))
    w = DI.WORKLOADS["tiny_256"].replace(name="signs_zero", shapes=shapes, workers=2, k=8)
    codec = B.Codec(shapes, w.k, w.beta, w.alpha)
    v, ix = codec.alloc_payload(2)
    ne = codec.n_entries
    for wk in range(2):
        codec.encode([torch.zeros(sh, device="cuda") for sh in shapes], [torch.zeros(sh, device="cuda") for sh in shapes],
                      v[wk * ne:(wk + 1) * ne], ix[wk * ne:(wk + 1) * ne])
    X0 = [DI.initial_params(w, i) for i in range(len(shapes))]
    Xs = [torch.from_numpy(x.copy()).cuda() for x in X0]
    Xb = [torch.from_numpy(x.copy()).cuda() for x in X0]
    codec.decode_apply(Xs, 2, v, ix, B.DEMO_PHI_SIGN, w.eta, w.lam)
    words = codec.alloc_signs()
    codec.decode_signs(2, v, ix, words)
    codec.apply_signs(Xb, words, w.eta, w.lam)
    torch.cuda.synchronize()
    assert not words.any(), "zero momentum must give all-clear sign words"
    for i, sh in enumerate(shapes):
        z = np.zeros(sh)
        nch = O.split_chunks(z).shape[0]
        # the payload of an all-zero chunk: indices 0..7 (ties to the lower index), values 0
        signum = O.decode_apply(X0[i], np.zeros((2, nch, 8), np.float32),
                                np.tile(np.arange(8, dtype=np.uint16), (2, nch, 1)), phi="sign", eta=w.eta, lam=w.lam)
        np.testing.assert_array_equal(signum["Mstar"], z)
        onebit = O.apply_signs(X0[i], O.pack_signs(z), eta=w.eta, lam=w.lam)
        gs, gb = Xs[i].cpu().numpy(), Xb[i].cpu().numpy()
        PR.compare_decode(signum, sh, "sign", w.eta, gs, np.zeros(nch, bool), None,
                          where=f"signum decode on zero momentum, tensor {i}")
        PR.compare_decode({"X": onebit, "Mstar": z + 1.0}, sh, "identity", w.eta, gb, np.zeros(nch, bool), None,
                          where=f"one-bit apply, tensor {i}")
        assert np.all(np.abs(gs - gb) > 0.5 * w.eta), "the two paths must differ by about eta everywhere"
    codec.close()


@pytest.mark.parametrize("chunk", [64, 128])
def test_sign_download_matches_signum_decode(dev, chunk):
    """apply_signs(decode_signs(payloads)) equals decode_apply with phi = sign wherever M* != 0."""
    shapes = ((192, 256), (300,)) if chunk == 64 else ((384, 300), (1000,))
    w = DI.WORKLOADS["tiny_256"].replace(name="signs_vs_signum", shapes=shapes, workers=3, k=12)
    codec = B.Codec(w.shapes, w.k, w.beta, w.alpha, chunk=chunk)
    v, ix = codec.alloc_payload(w.workers)
    ne = codec.n_entries
    for wk in range(w.workers):
        g = [torch.from_numpy(DI.gradient(w, wk, 0, i)).cuda() for i in range(len(w.shapes))]
        codec.encode(g, [torch.zeros(s, device="cuda") for s in w.shapes], v[wk * ne:(wk + 1) * ne],
                     ix[wk * ne:(wk + 1) * ne])
    X0 = [torch.from_numpy(DI.initial_params(w, i)).cuda() for i in range(len(w.shapes))]
    Xa = [x.clone() for x in X0]
    Xb = [x.clone() for x in X0]
    codec.decode_apply(Xa, w.workers, v, ix, B.DEMO_PHI_SIGN, w.eta, w.lam)
    words = codec.alloc_signs()
    codec.decode_signs(w.workers, v, ix, words)
    codec.apply_signs(Xb, words, w.eta, w.lam)
    torch.cuda.synchronize()
    for a, b in zip(Xa, Xb):
        assert torch.equal(a, b)


# --------------------------------------------------------------------------- chunk edge 128

@pytest.mark.parametrize("k", [1, 8, 32, 64])
def test_chunk128_single_chunk(dev, k):
    """One 128x128 chunk, two workers: the fast top-k path (keff <= 64)."""
    w = DI.WORKLOADS["tiny_256"].replace(name=f"s128_one_k{k}", shapes=((128, 128),), k=k, workers=2)
    Sim(w, chunk=128).run(2)


@pytest.mark.parametrize("k", [65, 500, 16384])
def test_chunk128_large_k(dev, k):
    """keff > 64 (workgroup-wide bitwise search) and the lossless k = 16384."""
    w = DI.WORKLOADS["tiny_256"].replace(name=f"s128_bigk{k}", shapes=((128, 256), (300,)), k=k, workers=2)
    Sim(w, chunk=128).run(2)


@pytest.mark.parametrize("k", [1, 4, 37])
def test_chunk128_ragged_and_vectors(dev, k):
    """Padded chunks, tiny matrices and vectors of awkward lengths at s = 128."""
    w = DI.WORKLOADS["tiny_256"].replace(
        name=f"s128_ragged_k{k}",
        shapes=((1, 1), (2, 3), (129, 130), (300, 77), (1,), (127,), (129,), (5000,)), k=k, workers=3)
    Sim(w, chunk=128).run(2)


@pytest.mark.parametrize("plain,avg,phi", [(False, "count", "sign"), (True, "workers", "identity")])
def test_chunk128_modes(dev, plain, avg, phi):
    w = DI.WORKLOADS["tiny_256"].replace(name=f"s128_modes_{plain}_{avg}_{phi}", shapes=((256, 384), (1000,)),
                                         phi=phi, workers=3, k=16)
    Sim(w, chunk=128, plain=plain, avg=avg).run(3)


def test_chunk128_aggregated_and_many_workers(dev):
    w = DI.WORKLOADS["tiny_256"].replace(name="s128_agg", shapes=((256, 128), (200,)), workers=3, k=8)
    Sim(w, chunk=128, aggregated=True).run(3)
    w = DI.WORKLOADS["tiny_256"].replace(name="s128_w20", shapes=((128, 256), (130,)), workers=20, k=16)
    Sim(w, chunk=128).run(2)


def test_chunk128_degenerate(dev):
    """All-zero and constant gradients: exact ties in the workgroup-wide top-k."""
    w = DI.WORKLOADS["tiny_256"].replace(name="s128_degenerate", shapes=((128, 128), (128, 256), (300,)), k=8,
                                         workers=2)

    def inputs(worker, step, i):
        if i == 0:
            return np.zeros((128, 128), np.float32)
        if i == 1:
            return np.full((128, 256), 1e-3 * (worker + 1), np.float32)
        return np.full((300,), -2e-3, np.float32)

    Sim(w, inputs=inputs, chunk=128).run(2, max_tie_fraction=1.0)


# --------------------------------------------------------------------------- compact wire format

@pytest.mark.parametrize("case", ["tiny", "ragged_k3", "k100_w20", "unit_identity_workers", "user_basis",
                                  "s128_tiny", "s128_ragged", "s128_k200_w20", "s128_unit_workers"])
def test_wire_end_to_end(dev, case):
    """Encode, pack into the wire format, decode from it; the oracle decodes its own payload rounded the same way.
    At chunk edge 128 the positions take 14 bits."""
    base = DI.WORKLOADS["tiny_256"]
    kw = {}
    if case.startswith("s128"):
        kw["chunk"] = 128
        if case == "s128_tiny":
            w = base.replace(name="wire128_tiny", shapes=((256, 384), (300,)), workers=3, k=16)
        elif case == "s128_ragged":
            w = base.replace(name="wire128_ragged", shapes=((1, 1), (129, 130), (300, 77), (127,), (5000,)), k=5,
                             workers=3)
        elif case == "s128_k200_w20":  # keff > 64 and more than one worker batch
            w = base.replace(name="wire128_k200_w20", shapes=((128, 256), (300,)), k=200, workers=20)
        else:
            w = base.replace(name="wire128_unit", shapes=((256, 300), (257,)), grad_std=1.0, param_std=1.0, beta=0.9,
                             k=16, workers=3, eta=0.01, phi="identity")
            kw.update(plain=True, avg="workers")
        Sim(w, wire=True, **kw).run(3)
        return
    if case == "tiny":
        w = base.replace(name="wire_tiny", workers=3)
    elif case == "ragged_k3":
        w = DI.WORKLOADS["edge_mix"].replace(name="wire_ragged", k=3)
    elif case == "k100_w20":  # more than one worker batch and one entry block per chunk
        w = base.replace(name="wire_k100_w20", shapes=((128, 192), (300,)), k=100, workers=20)
    elif case == "unit_identity_workers":
        w = base.replace(name="wire_unit", shapes=((192, 320), (129,)), grad_std=1.0, param_std=1.0, beta=0.9,
                         k=16, workers=3, eta=0.01, phi="identity")
        kw = dict(plain=True, avg="workers")
    else:
        w = base.replace(name="wire_user_basis", shapes=((128, 200), (65,)), k=4, workers=2, random_basis=True)
    Sim(w, wire=True, **kw).run(3)


def _lay_chunks(shapes, k, s=64):
    return [(n, keff, s * s if len(sh) == 2 else s) for (n, keff, _), sh in zip(PR.layout(shapes, k, s), shapes)]


@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("shapes,k,workers", [
    (((256, 256),), 8, 2),
    (((1000, 777), (3, 5000), (777,), (1,)), 3, 5),   # odd entry counts, vectors, ragged chunks
    (((64, 64),), 1, 1),                               # one entry
    (((130, 70), (63,)), 37, 17),
    (((256, 128),), 15, 3),                            # entry counts that are not whole groups at either width
])
def test_wire_pack_bit_exact(dev, shapes, k, workers, chunk):
    """The pack kernel against the oracle's format on drawn payloads full of rounding edge cases: 12-bit
    positions at chunk edge 64, 14-bit at 128 (indices drawn over the whole 128x128 chunk)."""
    codec = B.Codec(shapes, k, chunk=chunk)
    ne = codec.n_entries
    vals, idx = DI.synthetic_payload(_lay_chunks(shapes, k, chunk), workers, seed=40 + k, specials=True)
    assert vals.size == workers * ne
    wv, wi = codec.alloc_wire(workers)
    wv.fill_(-1)
    wi.fill_(255)
    say(f"  wire pack {shapes} k={k} W={workers}: {ne} entries per worker")
    codec.pack_wire(workers, torch.from_numpy(vals).cuda(), torch.from_numpy(idx.view(np.int16)).cuda(), wv, wi)
    torch.cuda.synchronize()
    gv = wv.cpu().numpy().view(np.uint16)
    gb = wi.cpu().numpy()
    ib = B.demo_wire_size(ne, chunk)[1]
    for wk in range(workers):
        ov, ob = O.pack_wire(vals[wk * ne:(wk + 1) * ne], idx[wk * ne:(wk + 1) * ne], chunk)
        assert np.array_equal(gv[wk * ne:(wk + 1) * ne], ov), f"worker {wk}: value codes differ"
        blk = gb[wk * ib:(wk + 1) * ib]
        assert np.array_equal(blk[:ob.size], ob), f"worker {wk}: index bytes differ"
        assert not blk[ob.size:].any(), f"worker {wk}: padding not zero"
    codec.close()


@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("phi,avg", [("sign", "count"), ("identity", "workers")])
def test_wire_decode_synthetic(dev, phi, avg, chunk):
    """decode_apply_wire on drawn payloads against the oracle's decode of the same wire; and bit-equal to
    decode_apply given the same values rounded to bfloat16 (same arithmetic, same order)."""
    shapes = ((200, 130), (1000,), (64, 64), (5,)) if chunk == 64 else ((300, 260), (1000,), (128, 128), (5,))
    k, W = 12, 6
    w = DI.WORKLOADS["tiny_256"].replace(name="wire_synth", shapes=shapes, k=k, workers=W, phi=phi)
    codec = B.Codec(shapes, k, chunk=chunk)
    ne = codec.n_entries
    vals, idx = DI.synthetic_payload(_lay_chunks(shapes, k, chunk), W, seed=77)
    vd, idd = torch.from_numpy(vals).cuda(), torch.from_numpy(idx.view(np.int16)).cuda()
    wv, wi = codec.alloc_wire(W)
    codec.pack_wire(W, vd, idd, wv, wi)
    X0 = [DI.initial_params(w, i) for i in range(len(shapes))]
    Xw = [torch.from_numpy(x.copy()).cuda() for x in X0]
    Xf = [torch.from_numpy(x.copy()).cuda() for x in X0]
    phi_c = B.DEMO_PHI_SIGN if phi == "sign" else B.DEMO_PHI_IDENTITY
    avg_c = B.DEMO_AVG_CONTRIBUTORS if avg == "count" else B.DEMO_AVG_WORKERS
    codec.decode_apply_wire(Xw, W, wv, wi, phi_c, w.eta, w.lam, avg_c)
    vr = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float32).cuda()  # torch's own round-to-nearest-even
    codec.decode_apply(Xf, W, vr, idd, phi_c, w.eta, w.lam, avg_c)
    torch.cuda.synchronize()
    lay = PR.layout(shapes, k, chunk)
    for i, shp in enumerate(shapes):
        n, keff, e0 = lay[i]
        ov, oi = [], []
        for wk in range(W):
            sl = slice(wk * ne + e0, wk * ne + e0 + n * keff)
            v_, i_ = O.unpack_wire(*O.pack_wire(vals[sl], idx[sl], chunk), n * keff, chunk)
            ov.append(v_.reshape(n, keff))
            oi.append(i_.reshape(n, keff))
        dec = O.decode_apply(X0[i], np.stack(ov), np.stack(oi), phi=phi, eta=w.eta, lam=w.lam, mode=avg, s=chunk)
        gx = Xw[i].cpu().numpy()
        PR.compare_decode(dec, shp, phi, w.eta, gx, np.zeros(n, bool), None, where=f"wire synthetic tensor {i} {shp}",
                          s=chunk)
        assert np.array_equal(gx, Xf[i].cpu().numpy()), f"tensor {i}: wire decode differs from the float32 decode"
    codec.close()
