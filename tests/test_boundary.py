"""C-ABI boundary checks that need no GPU.

The library must load on a machine without a GPU, export every function the
public header declares, plan payloads exactly as the oracle counts them, and
reject every malformed argument before touching a device (a NULL context is
only reported once all other arguments passed).
"""
import ctypes
import glob
import os
import re

import pytest

import demo_inputs as DI
from communication_compressed_optimizer_demo_amd import binding as B
from oracle import demo_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from communication_compressed_optimizer_demo_amd import build
        build.build()
    return B.load_library()


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*[A-Za-z_][\w \*]*?\b(demo_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("demo_encode", "demo_decode_apply", "demo_plan", "demo_ctx_create", "demo_ctx_destroy",
                     "demo_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


@pytest.mark.parametrize("name", sorted(DI.WORKLOADS))
def test_plan_matches_oracle_payload_count(lib, name):
    w = DI.WORKLOADS[name]
    for k in (1, w.k, 64, 4096, 5000):
        n_chunks, n_entries, begin = B.demo_plan(w.shapes, k)
        assert n_entries == O.payload_entries(w.shapes, k)
        assert n_chunks == sum(int(__import__("numpy").prod(O.chunk_grid(s))) for s in w.shapes)
        acc = 0
        for i, s in enumerate(w.shapes):
            assert begin[i] == acc
            numel = 64 if len(s) == 1 else 4096
            acc += int(__import__("numpy").prod(O.chunk_grid(s))) * O.k_effective(k, numel)
        assert begin[len(w.shapes)] == acc == n_entries


def test_plan_olmo_sizes(lib):
    # chunk and entry counts counted from the shapes: an OLMo-1B block has 32x96 + 32x32 + 32x128 + 128x32
    # chunks of 64x64 and two 2048-vectors of 32 chunks, 16 blocks, keff 32; OLMo-300M: 24 blocks at d = 1024,
    # keff 8
    assert B.demo_plan(DI.WORKLOADS["olmo_1b"].shapes, 32)[:2] == (197632, 6324224)
    assert B.demo_plan(DI.WORKLOADS["olmo_300m"].shapes, 8)[:2] == (74496, 595968)
    assert DI.WORKLOADS["olmo_1b"].n_params == 805371904
    assert DI.WORKLOADS["olmo_300m"].n_params == 302039040


def _call_encode(lib, shapes, k=8, chunk=64, grad_dtype=0, beta=0.9, alpha=0.2, form=0, basis=0,
                 P0=None, P1=None, entries=None, grads=0x1000, moms=0x2000, vals=0x3000, idx=0x4000, subtraction=0):
    cfg = B.demo_codec_cfg(chunk, k, beta, alpha, form, basis, P0, P1, subtraction)
    n = len(shapes)
    sh = B._shapes(shapes)
    if entries is None:
        entries = O.payload_entries(shapes, max(k, 1), chunk) if k >= 1 and chunk in (64, 128) else 0
    gp = B._ptrs([grads] * n)
    mp = B._ptrs([moms] * n)
    return lib.demo_encode(None, n, sh, gp, grad_dtype, mp, ctypes.byref(cfg), vals, idx, entries, None)


def _call_decode(lib, shapes, k=8, workers=2, phi=0, avg=0, eta=1e-3, lam=0.0, entries=None, params=0x1000,
                 vals=0x3000, idx=0x4000, basis=0, P0=None, P1=None):
    cfg = B.demo_codec_cfg(64, k, 0.9, 0.2, 0, basis, P0, P1)
    n = len(shapes)
    if entries is None:
        entries = O.payload_entries(shapes, k)
    return lib.demo_decode_apply(None, n, B._shapes(shapes), B._ptrs([params] * n), ctypes.byref(cfg), workers,
                                 vals, idx, entries, phi, eta, lam, avg, None)


def _call_decode_subtract(lib, shapes, params=0x1000, moms=0x2000, alpha=0.2, k=8, workers=2, vals=0x3000,
                          idx=0x4000, bad_index=None):
    cfg = B.demo_codec_cfg(64, k, 0.9, alpha, 0, 0, None, None, 1)
    n = len(shapes)
    pl = None if params is None else B._ptrs([params] * n)
    ml = None if moms is None else B._ptrs([moms] * n)
    if bad_index is not None:
        ml[bad_index] = None
    return lib.demo_decode_apply_subtract(None, n, B._shapes(shapes), pl, ml, ctypes.byref(cfg), workers, vals, idx,
                                          O.payload_entries(shapes, k), 0, 1e-3, 0.0, 0, None)


def _msg(lib):
    return lib.demo_last_error().decode()


def test_valid_arguments_reach_the_context_check(lib):
    assert _call_encode(lib, [(128, 64), (100,)]) == 1 and "context" in _msg(lib)
    assert _call_decode(lib, [(128, 64), (100,)]) == 1 and "context" in _msg(lib)


@pytest.mark.parametrize("kw,status", [
    (dict(shapes=[(0, 5)]), 2),
    (dict(shapes=[(5, 0)]), 2),
    (dict(shapes=[(3, 4, 5)]), 2),
    (dict(shapes=[(2 ** 31, 4)]), 2),
    (dict(k=0), 3),
    (dict(k=-3), 3),
    (dict(chunk=96), 3),
    (dict(chunk=128, basis=2), 3),
    (dict(chunk=128, basis=1, P0=0x5000, P1=0x6000), 3),
    (dict(chunk=128, entries=O.payload_entries([(128, 64), (100,)], 8)), 4),
    (dict(grad_dtype=7), 1),
    (dict(form=2), 1),
    (dict(beta=float("nan")), 1),
    (dict(alpha=float("inf")), 1),
    (dict(entries=5), 4),
    (dict(grads=0), 1),
    (dict(moms=0), 1),
    (dict(vals=0), 1),
    (dict(grads=0x1002), 7),
    (dict(grads=0x1002, grad_dtype=1), 1 + 0 * 7),  # bf16 needs 2-byte alignment only: reaches ctx check
    (dict(moms=0x2001), 7),
    (dict(vals=0x3002), 7),
    (dict(idx=0x4001), 7),
    (dict(basis=5), 1),
    (dict(basis=1), 1),
    (dict(basis=1, P0=0x5000), 1),
    (dict(basis=1, P0=0x5002, P1=0x6000), 7),
    (dict(basis=1, P0=0x5000, P1=0x6004), 7),  # the basis is read 16 bytes at a time
    (dict(basis=3), 1),
    (dict(subtraction=2), 1),
    (dict(subtraction=-1), 1),
])
def test_encode_rejects_bad_arguments(lib, kw, status):
    shapes = kw.pop("shapes", [(128, 64), (100,)])
    assert _call_encode(lib, shapes, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(workers=0), 3),
    (dict(workers=256), 3),
    (dict(phi=2), 1),
    (dict(avg=2), 1),
    (dict(eta=float("nan")), 1),
    (dict(lam=float("inf")), 1),
    (dict(entries=1), 4),
    (dict(params=0), 1),
    (dict(params=0x1001), 7),
    (dict(vals=0), 1),
    (dict(idx=0x4001), 7),
    (dict(k=0), 3),
])
def test_decode_rejects_bad_arguments(lib, kw, status):
    assert _call_decode(lib, [(128, 64), (100,)], **kw) == status


@pytest.mark.parametrize("kw", [dict(subtraction=1), dict(basis=2), dict(basis=2, subtraction=1, k=4096)])
def test_identity_basis_and_aggregated_subtraction_are_valid(lib, kw):
    assert _call_encode(lib, [(128, 64), (100,)], **kw) == 1 and "context" in _msg(lib)


@pytest.mark.parametrize("kw,status,text", [
    (dict(), 1, "context"),
    (dict(params=None), 1, "context"),
    (dict(moms=None), 1, "context"),
    (dict(params=None, moms=None), 1, "neither"),
    (dict(moms=0x2002), 7, "misaligned"),
    (dict(bad_index=1), 1, "NULL"),
    (dict(alpha=float("nan")), 1, "alpha"),
    (dict(workers=0), 3, "workers"),
])
def test_decode_apply_subtract_arguments(lib, kw, status, text):
    assert _call_decode_subtract(lib, [(128, 64), (100,)], **kw) == status
    assert text in _msg(lib)


def test_vectors_only_user_basis_needs_no_p1(lib):
    # 1-D tensors use P0 only: valid arguments reach the context check
    assert _call_encode(lib, [(100,)], basis=1, P0=0x5000) == 1 and "context" in _msg(lib)


def test_empty_tensor_list_is_valid(lib):
    assert _call_encode(lib, [], entries=0) == 1 and "context" in _msg(lib)
    nc, ne, begin = B.demo_plan([], 8)
    assert (nc, ne, begin) == (0, 0, [0])


def test_ctx_create_without_gpu_fails_cleanly(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(B.DemoError):
        B.demo_ctx_create(0)


# --------------------------------------------------------------------------- one-bit sign download

@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("name", sorted(DI.WORKLOADS))
def test_plan_signs_matches_oracle_word_count(lib, name, chunk):
    import numpy as np
    w = DI.WORKLOADS[name]
    n_words, begin = B.demo_plan_signs(w.shapes, chunk)
    assert n_words == O.sign_words(w.shapes, chunk)
    acc = 0
    for i, s in enumerate(w.shapes):
        assert begin[i] == acc
        acc += O.sign_words([s], chunk)
    assert begin[len(w.shapes)] == acc == n_words
    if name == "olmo_1b":
        assert n_words * 64 == w.n_params  # no padding in the OLMo shapes: exactly one bit per parameter
        assert np.isclose(n_words * 8 / (4 * w.n_params), 1 / 32)


def _call_decode_signs(lib, shapes, k=8, workers=2, avg=0, vals=0x3000, idx=0x4000, signs=0x5000, words=None,
                       entries=None, chunk=64):
    cfg = B.demo_codec_cfg(chunk, k, 0.9, 0.2, 0, 0, None, None, 0)
    n = len(shapes)
    if words is None:
        words = O.sign_words(shapes, chunk)
    if entries is None:
        entries = O.payload_entries(shapes, k, chunk)
    return lib.demo_decode_signs(None, n, B._shapes(shapes), ctypes.byref(cfg), workers, vals, idx, entries, avg,
                                 signs, words, None)


def _call_apply_signs(lib, shapes, params=0x1000, signs=0x5000, words=None, eta=1e-3, lam=0.0, chunk=64,
                      null_list=False):
    n = len(shapes)
    if words is None:
        words = O.sign_words(shapes, chunk if chunk in (64, 128) else 64)
    pl = None if null_list else B._ptrs([params] * n)
    return lib.demo_apply_signs(None, n, B._shapes(shapes), pl, chunk, signs, words, eta, lam, None)


@pytest.mark.parametrize("kw,status,text", [
    (dict(), 1, "context"),
    (dict(words=3), 4, "sign buffer"),
    (dict(signs=0), 1, "sign buffer is NULL"),
    (dict(signs=0x5004), 7, "misaligned"),
    (dict(entries=2), 4, "payload"),
    (dict(workers=0), 3, "workers"),
    (dict(avg=5), 1, "average"),
    (dict(chunk=32), 3, "chunk"),
    (dict(chunk=128), 1, "context"),
    (dict(chunk=128, words=3), 4, "sign buffer"),
    (dict(vals=0), 1, "payload is NULL"),
])
def test_decode_signs_arguments(lib, kw, status, text):
    assert _call_decode_signs(lib, [(128, 64), (100,)], **kw) == status
    assert text in _msg(lib)


@pytest.mark.parametrize("kw,status,text", [
    (dict(), 1, "context"),
    (dict(words=129), 4, "sign buffer"),
    (dict(signs=0), 1, "sign buffer is NULL"),
    (dict(signs=0x5002), 7, "misaligned"),
    (dict(params=0), 1, "NULL device pointer"),
    (dict(params=0x1002), 7, "misaligned"),
    (dict(null_list=True), 1, "pointer list"),
    (dict(eta=float("nan")), 1, "eta"),
    (dict(chunk=32), 3, "chunk"),
    (dict(chunk=128), 1, "context"),
])
def test_apply_signs_arguments(lib, kw, status, text):
    assert _call_apply_signs(lib, [(128, 64), (100,)], **kw) == status
    assert text in _msg(lib)


@pytest.mark.parametrize("name", sorted(DI.WORKLOADS))
def test_plan_chunk128_matches_oracle(lib, name):
    import numpy as np
    w = DI.WORKLOADS[name]
    for k in (1, w.k, 64, 128, 16384, 20000):
        n_chunks, n_entries, begin = B.demo_plan(w.shapes, k, 128)
        assert n_entries == O.payload_entries(w.shapes, k, 128)
        assert n_chunks == sum(int(np.prod(O.chunk_grid(s, 128))) for s in w.shapes)
        assert begin[-1] == n_entries


def test_chunk128_valid_arguments_reach_the_context_check(lib):
    assert _call_encode(lib, [(300, 200), (1000,)], chunk=128, k=16) == 1 and "context" in _msg(lib)
    assert _call_encode(lib, [(300, 200)], chunk=128, k=16, subtraction=1) == 1 and "context" in _msg(lib)
    cfg = B.demo_codec_cfg(128, 16, 0.9, 0.2, 0, 0, None, None, 0)
    sh = [(300, 200), (1000,)]
    e = O.payload_entries(sh, 16, 128)
    assert lib.demo_decode_apply(None, 2, B._shapes(sh), B._ptrs([0x1000] * 2), ctypes.byref(cfg), 3, 0x3000,
                                 0x4000, e, 0, 1e-3, 0.0, 0, None) == 1 and "context" in _msg(lib)
    # the one-bit download: 2 words per 128-element row of a padded matrix chunk, 2 per vector chunk
    nw = ctypes.c_int64()
    assert lib.demo_plan_signs(B._shapes(sh), 2, 128, ctypes.byref(nw), None) == 0
    assert nw.value == 3 * 2 * 256 + 8 * 2 == O.sign_words(sh, 128)
    assert lib.demo_decode_signs(None, 2, B._shapes(sh), ctypes.byref(cfg), 3, 0x3000, 0x4000, e, 0, 0x5000,
                                 nw.value, None) == 1 and "context" in _msg(lib)
    assert lib.demo_plan_signs(B._shapes(sh), 2, 96, ctypes.byref(nw), None) == 3


# --------------------------------------------------------------------------- phi = Muon

def test_muon_workspace_size(lib):
    # M* of every tensor (64-float rounded), then one slot per matrix (at most 8): six n_max^2 matrices
    # (64-float rounded), 256 doubles, 64 floats
    shapes = [(70, 90), (100,), (130, 200)]
    mstar = (6336 + 128 + 26048)
    slot = (6 * 130 * 130 + 63) // 64 * 64 + 512 + 64
    assert B.demo_muon_workspace(shapes) == (mstar + 2 * slot) * 4
    many = [(64, 96)] * 11 + [(10,)]
    assert B.demo_muon_workspace(many) == (11 * 6144 + 64 + 8 * (6 * 64 * 64 + 576)) * 4


def test_muon_params_checked_before_any_work(lib):
    # a NULL parameter pointer is refused before the decode of M* could be enqueued: with every other
    # argument valid and no context, the status names the tensor, not the context
    assert _call_muon(lib, [(70, 90), (100,)], params=0) == 1
    assert "NULL device pointer" in _msg(lib)


def _call_muon(lib, shapes, k=8, workers=2, eps=1e-6, iters=24, ws=0x7000, ws_bytes=None, chunk=64, params=0x1000,
               eta=1e-3):
    cfg = B.demo_codec_cfg(chunk, k, 0.9, 0.2, 0, 0, None, None, 0)
    n = len(shapes)
    if ws_bytes is None:
        ws_bytes = B.demo_muon_workspace(shapes)
    return lib.demo_decode_apply_muon(None, n, B._shapes(shapes), B._ptrs([params] * n), ctypes.byref(cfg), workers,
                                      0x3000, 0x4000, O.payload_entries(shapes, k), eta, 0.0, eps, iters, 0, ws,
                                      ws_bytes, None)


@pytest.mark.parametrize("kw,status,text", [
    (dict(), 1, "context"),
    (dict(eps=-1.0), 1, "eps"),
    (dict(eps=float("nan")), 1, "eps"),
    (dict(iters=0), 3, "iters"),
    (dict(iters=65), 3, "iters"),
    (dict(ws_bytes=16), 3, "workspace"),
    (dict(ws=0), 1, "workspace is NULL"),
    (dict(ws=0x7004), 7, "misaligned"),
    (dict(chunk=128), 3, "chunk 64"),
    (dict(workers=0), 3, "workers"),
])
def test_muon_arguments(lib, kw, status, text):
    assert _call_muon(lib, [(70, 90), (100,)], **kw) == status
    assert text in _msg(lib)


# --------------------------------------------------------------------------- compact wire format

@pytest.mark.parametrize("entries", [0, 1, 7, 8, 9, 15, 16, 17, 1000, 6_291_456])
def test_wire_size(lib, entries):
    vb, ib = B.demo_wire_size(entries)
    assert vb == 2 * entries
    # whole 8-entry groups of 12 bytes, which hold the oracle's 12-bit string
    assert ib == 12 * ((entries + 7) // 8)
    vb, ib14 = B.demo_wire_size(entries, 128)
    assert vb == 2 * entries
    # whole 16-entry groups of 28 bytes (7 words), which hold the oracle's 14-bit string
    assert ib14 == 28 * ((entries + 15) // 16)
    if entries < 2000:
        assert O.pack_wire([0.0] * entries, [0] * entries)[1].size <= ib
        assert O.pack_wire([0.0] * entries, [0] * entries, s=128)[1].size <= ib14
        assert ib - O.pack_wire([0.0] * entries, [0] * entries)[1].size < 12
        assert ib14 - O.pack_wire([0.0] * entries, [0] * entries, s=128)[1].size < 28


def test_wire_size_rejects_other_chunks(lib):
    assert lib.demo_wire_size(96, 10, None, None) == 3 and "chunk" in _msg(lib)


def _call_wire_decode(lib, k=8, workers=2, chunk=64, wv=0x3000, wi=0x4000, entries=None, phi=0):
    shapes = [(70, 90), (100,)]
    cfg = B.demo_codec_cfg(chunk, k, 0.9, 0.2, 0, 0, None, None, 0)
    e = O.payload_entries(shapes, k) if entries is None else entries
    return lib.demo_decode_apply_wire(None, 2, B._shapes(shapes), B._ptrs([0x1000] * 2), ctypes.byref(cfg), workers,
                                      wv, wi, e, phi, 1e-3, 0.0, 0, None)


@pytest.mark.parametrize("kw,status,text", [
    (dict(), 1, "context"),
    (dict(chunk=128), 4, "entries"),
    (dict(chunk=128, entries=O.payload_entries([(70, 90), (100,)], 8, 128)), 1, "context"),
    (dict(chunk=32), 3, "chunk"),
    (dict(workers=0), 3, "workers"),
    (dict(workers=256), 3, "workers"),
    (dict(entries=5), 4, "entries"),
    (dict(wv=0), 1, "wire payload is NULL"),
    (dict(wi=0), 1, "wire payload is NULL"),
    (dict(wv=0x3001), 7, "misaligned"),
    (dict(wi=0x4002), 7, "misaligned"),
    (dict(phi=9), 1, "phi"),
])
def test_wire_decode_arguments(lib, kw, status, text):
    assert _call_wire_decode(lib, **kw) == status
    assert text in _msg(lib)


@pytest.mark.parametrize("args,status,text", [
    ((64, 2, 0x3000, 0x4000, 100, 0x5000, 0x6000), 1, "context"),
    ((128, 2, 0x3000, 0x4000, 100, 0x5000, 0x6000), 1, "context"),
    ((32, 2, 0x3000, 0x4000, 100, 0x5000, 0x6000), 3, "chunk"),
    ((64, 0, 0x3000, 0x4000, 100, 0x5000, 0x6000), 3, "workers"),
    ((64, 2, 0x3000, 0x4000, -1, 0x5000, 0x6000), 3, "entry count"),
    ((64, 2, 0, 0x4000, 100, 0x5000, 0x6000), 1, "NULL"),
    ((64, 2, 0x3000, 0x4000, 100, 0, 0x6000), 1, "NULL"),
    ((64, 2, 0x3002, 0x4000, 100, 0x5000, 0x6000), 7, "misaligned"),
    ((64, 2, 0x3000, 0x4000, 100, 0x5000, 0x6001), 7, "misaligned"),
])
def test_pack_wire_arguments(lib, args, status, text):
    assert lib.demo_pack_wire(None, *args, None) == status
    assert text in _msg(lib)


# --------------------------------------------------------------------------- Muon decode without allocation

def _call_muon_noalloc(lib, shapes, k=8, workers=2, eps=1e-6, iters=24, chunk=64, params=0x1000):
    cfg = B.demo_codec_cfg(chunk, k, 0.9, 0.2, 0, 0, None, None, 0)
    n = len(shapes)
    return lib.demo_decode_apply_muon_noalloc(None, n, B._shapes(shapes), B._ptrs([params] * n), ctypes.byref(cfg),
                                              workers, 0x3000, 0x4000, O.payload_entries(shapes, k), 1e-3, 0.0, eps,
                                              iters, 0, None)


def test_muon_noalloc_scratch_size_matches_header(lib):
    text = open(os.path.join(ROOT, "include", "demo_codec.h")).read()
    m = re.search(r"#define DEMO_MUON_SCRATCH_BYTES \((\d+)ll << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.DEMO_MUON_SCRATCH_BYTES


@pytest.mark.parametrize("shapes,status,text", [
    ([(70, 90), (100,)], 1, "context"),            # fits: every other check passes, then the context is NULL
    ([(2048, 2048)], 3, "static scratch"),          # 112 MB of workspace: refused before anything else
    ([(1024, 1024), (1024, 1024), (1024, 1024)], 3, "static scratch"),
])
def test_muon_noalloc_arguments(lib, shapes, status, text):
    assert _call_muon_noalloc(lib, shapes) == status
    assert text in _msg(lib)
    fits = B.demo_muon_workspace(shapes) <= B.DEMO_MUON_SCRATCH_BYTES
    assert fits == (status != 3)


@pytest.mark.parametrize("kw,status,text", [
    (dict(eps=-1.0), 1, "eps"),
    (dict(iters=0), 3, "iters"),
    (dict(chunk=128), 3, "chunk 64"),
    (dict(workers=0), 3, "workers"),
    (dict(params=0), 1, "NULL device pointer"),
])
def test_muon_noalloc_checks_the_rest_before_the_context(lib, kw, status, text):
    assert _call_muon_noalloc(lib, [(70, 90), (100,)], **kw) == status
    assert text in _msg(lib)
