"""ctypes binding of libdemo_codec.so, one Python function per C entry point.

Argument marshalling only: tensors are passed as device pointers and every
step of the codec runs in the library's HIP kernels.  There is no fallback:
if the library is missing, or no gfx950 device is present, the calls raise.
PyTorch tensors are accepted as buffers (it supplies device memory and
streams); torch is imported lazily so the library can be inspected without it.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdemo_codec.so")

DEMO_CHUNK = 64
DEMO_CHUNK_LARGE = 128  # the other chunk edge built (DCT basis, no one-bit download)
DEMO_MAX_WORKERS = 255
DEMO_MAX_TENSORS_PER_LAUNCH = 96  # one kernel launch per this many tensors of a call

# demo_status
DEMO_OK = 0
STATUS_NAMES = {0: "DEMO_OK", 1: "DEMO_ERR_INVALID", 2: "DEMO_ERR_SHAPE", 3: "DEMO_ERR_RANGE",
                4: "DEMO_ERR_PAYLOAD", 5: "DEMO_ERR_DEVICE", 6: "DEMO_ERR_HIP", 7: "DEMO_ERR_ALIGN"}
# enums
DEMO_F32, DEMO_BF16 = 0, 1
DEMO_MOMENTUM_DAMPED, DEMO_MOMENTUM_PLAIN = 0, 1
DEMO_BASIS_DCT, DEMO_BASIS_USER, DEMO_BASIS_IDENTITY = 0, 1, 2
DEMO_PHI_SIGN, DEMO_PHI_IDENTITY = 0, 1
DEMO_AVG_CONTRIBUTORS, DEMO_AVG_WORKERS = 0, 1
DEMO_SUBTRACT_LOCAL, DEMO_SUBTRACT_AGGREGATED = 0, 1


class DemoError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class demo_shape(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int32), ("dims", ctypes.c_int64 * 2)]


class demo_codec_cfg(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int32), ("k", ctypes.c_int32), ("beta", ctypes.c_float),
                ("alpha", ctypes.c_float), ("momentum_form", ctypes.c_int32), ("basis", ctypes.c_int32),
                ("P0", ctypes.c_void_p), ("P1", ctypes.c_void_p), ("subtraction", ctypes.c_int32)]


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m communication_compressed_optimizer_demo_amd.build`")
    lib = ctypes.CDLL(path)
    i32, i64, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    P = ctypes.POINTER
    lib.demo_last_error.restype = ctypes.c_char_p
    lib.demo_last_error.argtypes = []
    lib.demo_ctx_create.restype = i32
    lib.demo_ctx_create.argtypes = [i32, P(vp)]
    lib.demo_ctx_destroy.restype = None
    lib.demo_ctx_destroy.argtypes = [vp]
    lib.demo_plan.restype = i32
    lib.demo_plan.argtypes = [P(demo_shape), i32, i32, i32, P(i64), P(i64), P(i64)]
    lib.demo_encode.restype = i32
    lib.demo_encode.argtypes = [vp, i32, P(demo_shape), P(vp), i32, P(vp), P(demo_codec_cfg),
                                vp, vp, i64, vp]
    lib.demo_decode_apply.restype = i32
    lib.demo_decode_apply.argtypes = [vp, i32, P(demo_shape), P(vp), P(demo_codec_cfg), i32,
                                      vp, vp, i64, i32, f32, f32, i32, vp]
    lib.demo_decode_apply_subtract.restype = i32
    lib.demo_decode_apply_subtract.argtypes = [vp, i32, P(demo_shape), P(vp), P(vp), P(demo_codec_cfg), i32,
                                               vp, vp, i64, i32, f32, f32, i32, vp]
    lib.demo_plan_signs.restype = i32
    lib.demo_plan_signs.argtypes = [P(demo_shape), i32, i32, P(i64), P(i64)]
    lib.demo_decode_signs.restype = i32
    lib.demo_decode_signs.argtypes = [vp, i32, P(demo_shape), P(demo_codec_cfg), i32, vp, vp, i64, i32, vp, i64,
                                      vp]
    lib.demo_apply_signs.restype = i32
    lib.demo_apply_signs.argtypes = [vp, i32, P(demo_shape), P(vp), i32, vp, i64, f32, f32, vp]
    lib.demo_muon_workspace.restype = i32
    lib.demo_muon_workspace.argtypes = [P(demo_shape), i32, P(i64)]
    lib.demo_decode_apply_muon.restype = i32
    lib.demo_decode_apply_muon.argtypes = [vp, i32, P(demo_shape), P(vp), P(demo_codec_cfg), i32, vp, vp, i64, f32,
                                           f32, f32, i32, i32, vp, i64, vp]
    lib.demo_decode_apply_muon_noalloc.restype = i32
    lib.demo_decode_apply_muon_noalloc.argtypes = [vp, i32, P(demo_shape), P(vp), P(demo_codec_cfg), i32, vp, vp,
                                                   i64, f32, f32, f32, i32, i32, vp]
    lib.demo_wire_size.restype = i32
    lib.demo_wire_size.argtypes = [i32, i64, P(i64), P(i64)]
    lib.demo_pack_wire.restype = i32
    lib.demo_pack_wire.argtypes = [vp, i32, i32, vp, vp, i64, vp, vp, vp]
    lib.demo_decode_apply_wire.restype = i32
    lib.demo_decode_apply_wire.argtypes = [vp, i32, P(demo_shape), P(vp), P(demo_codec_cfg), i32,
                                           vp, vp, i64, i32, f32, f32, i32, vp]
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != DEMO_OK:
        raise DemoError(status, load_library().demo_last_error().decode())


def _shapes(shapes: Sequence[Sequence[int]]):
    arr = (demo_shape * max(1, len(shapes)))()
    for i, s in enumerate(shapes):
        arr[i].ndim = len(s)
        arr[i].dims[0] = int(s[0]) if len(s) > 0 else 0
        arr[i].dims[1] = int(s[1]) if len(s) > 1 else 0
    return arr


def _ptrs(values: Sequence[int]):
    arr = (ctypes.c_void_p * max(1, len(values)))()
    for i, v in enumerate(values):
        arr[i] = v
    return arr


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_cfg(k: int, beta: float = 0.999, alpha: float = 0.2, plain: bool = False,
             P0=None, P1=None, chunk: int = DEMO_CHUNK, identity: bool = False,
             aggregated: bool = False) -> demo_codec_cfg:
    """Codec configuration; P0/P1 (device float32 64x64 tensors) select the user basis,
    ``identity`` the identity basis (top-k in the parameter domain), ``aggregated``
    the subtraction of the averaged coefficients on the decode side."""
    cfg = demo_codec_cfg()
    cfg.chunk = chunk
    cfg.k = int(k)
    cfg.beta = float(beta)
    cfg.alpha = float(alpha)
    cfg.momentum_form = DEMO_MOMENTUM_PLAIN if plain else DEMO_MOMENTUM_DAMPED
    cfg.subtraction = DEMO_SUBTRACT_AGGREGATED if aggregated else DEMO_SUBTRACT_LOCAL
    if identity:
        if P0 is not None:
            raise ValueError("the identity basis takes no P0/P1")
        cfg.basis = DEMO_BASIS_IDENTITY
        cfg.P0 = cfg.P1 = None
    elif P0 is None:
        cfg.basis = DEMO_BASIS_DCT
        cfg.P0 = cfg.P1 = None
    else:
        cfg.basis = DEMO_BASIS_USER
        cfg.P0 = _device_ptr(P0, 4)
        cfg.P1 = _device_ptr(P1 if P1 is not None else P0, 4)
    return cfg


def _device_ptr(t, elem_size: int) -> int:
    if not t.is_cuda:
        raise ValueError("tensor must live in device memory")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if t.element_size() != elem_size:
        raise ValueError(f"tensor element size {t.element_size()} != {elem_size}")
    return t.data_ptr()


# ----------------------------------------------------------------------------- entry points

def demo_plan(shapes: Sequence[Sequence[int]], k: int, chunk: int = DEMO_CHUNK) -> Tuple[int, int, List[int]]:
    """(n_chunks, n_entries, entry_begin[n+1]) of a tensor list; host-only."""
    lib = load_library()
    n = len(shapes)
    sh = _shapes(shapes)
    nc, ne = ctypes.c_int64(), ctypes.c_int64()
    eb = (ctypes.c_int64 * (n + 1))()
    _check(lib.demo_plan(sh, n, chunk, int(k), ctypes.byref(nc), ctypes.byref(ne), eb))
    return nc.value, ne.value, list(eb)


def demo_ctx_create(device: int = 0) -> int:
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.demo_ctx_create(int(device), ctypes.byref(h)))
    return h.value


def demo_ctx_destroy(ctx: int) -> None:
    load_library().demo_ctx_destroy(ctx)


def demo_encode(ctx: int, grads, moms, cfg: demo_codec_cfg, pay_values, pay_idx, stream=None) -> None:
    """Encode one worker's tensors: moms updated in place, payload written."""
    lib = load_library()
    import torch
    n = len(grads)
    if len(moms) != n:
        raise ValueError("grads and moms differ in length")
    shapes = []
    for g, m in zip(grads, moms):
        if tuple(g.shape) != tuple(m.shape):
            raise ValueError("gradient and momentum shapes differ")
        if m.dtype != torch.float32:
            raise ValueError("momentum must be float32")
        shapes.append(tuple(m.shape))
    gdt = grads[0].dtype if n else torch.float32
    if any(g.dtype != gdt for g in grads):
        raise ValueError("all gradients must share one dtype")
    if gdt == torch.float32:
        code, gsz = DEMO_F32, 4
    elif gdt == torch.bfloat16:
        code, gsz = DEMO_BF16, 2
    else:
        raise ValueError("gradients must be float32 or bfloat16")
    _check(lib.demo_encode(ctx, n, _shapes(shapes), _ptrs([_device_ptr(g, gsz) for g in grads]), code,
                           _ptrs([_device_ptr(m, 4) for m in moms]), ctypes.byref(cfg),
                           _device_ptr(pay_values, 4), _device_ptr(pay_idx, 2), pay_values.numel(),
                           _stream_handle(stream)))


def demo_decode_apply(ctx: int, params, cfg: demo_codec_cfg, workers: int, pay_values, pay_idx,
                      phi: int = DEMO_PHI_SIGN, eta: float = 1e-3, lam: float = 0.0,
                      avg: int = DEMO_AVG_CONTRIBUTORS, stream=None) -> None:
    """Average ``workers`` payloads (worker-major rows) and update params in place."""
    lib = load_library()
    import torch
    n = len(params)
    for x in params:
        if x.dtype != torch.float32:
            raise ValueError("parameters must be float32")
    if pay_values.numel() % workers or pay_idx.numel() != pay_values.numel():
        raise ValueError("payload arrays must hold workers x entries elements")
    per = pay_values.numel() // workers
    _check(lib.demo_decode_apply(ctx, n, _shapes([tuple(x.shape) for x in params]),
                                 _ptrs([_device_ptr(x, 4) for x in params]), ctypes.byref(cfg), int(workers),
                                 _device_ptr(pay_values, 4), _device_ptr(pay_idx, 2), per, int(phi),
                                 float(eta), float(lam), int(avg), _stream_handle(stream)))


def demo_decode_apply_subtract(ctx: int, params, moms, cfg: demo_codec_cfg, workers: int, pay_values, pay_idx,
                               phi: int = DEMO_PHI_SIGN, eta: float = 1e-3, lam: float = 0.0,
                               avg: int = DEMO_AVG_CONTRIBUTORS, stream=None) -> None:
    """Aggregated-subtraction decode: params (or None) get the update, moms (or None) M - alpha M*."""
    lib = load_library()
    import torch
    lists = [t for t in (params, moms) if t is not None]
    if not lists:
        raise ValueError("give params, moms or both")
    ref = lists[0]
    for lst in lists:
        if len(lst) != len(ref) or any(tuple(a.shape) != tuple(b.shape) for a, b in zip(lst, ref)):
            raise ValueError("params and moms must match in count and shape")
        if any(t.dtype != torch.float32 for t in lst):
            raise ValueError("parameters and momenta must be float32")
    if pay_values.numel() % workers or pay_idx.numel() != pay_values.numel():
        raise ValueError("payload arrays must hold workers x entries elements")
    per = pay_values.numel() // workers
    pp = None if params is None else _ptrs([_device_ptr(x, 4) for x in params])
    mp = None if moms is None else _ptrs([_device_ptr(m, 4) for m in moms])
    _check(lib.demo_decode_apply_subtract(ctx, len(ref), _shapes([tuple(x.shape) for x in ref]), pp, mp,
                                          ctypes.byref(cfg), int(workers), _device_ptr(pay_values, 4),
                                          _device_ptr(pay_idx, 2), per, int(phi), float(eta), float(lam), int(avg),
                                          _stream_handle(stream)))


def demo_plan_signs(shapes: Sequence[Sequence[int]], chunk: int = DEMO_CHUNK) -> Tuple[int, List[int]]:
    """(n_words, word_begin[n+1]) of the packed one-bit sign of a tensor list; host-only."""
    lib = load_library()
    n = len(shapes)
    nw = ctypes.c_int64()
    wb = (ctypes.c_int64 * (n + 1))()
    _check(lib.demo_plan_signs(_shapes(shapes), n, chunk, ctypes.byref(nw), wb))
    return nw.value, list(wb)


def demo_decode_signs(ctx: int, shapes: Sequence[Sequence[int]], cfg: demo_codec_cfg, workers: int, pay_values,
                      pay_idx, signs, avg: int = DEMO_AVG_CONTRIBUTORS, stream=None) -> None:
    """Average ``workers`` payloads and pack sign(M*) into ``signs`` (64-bit words, int64 storage)."""
    lib = load_library()
    if pay_values.numel() % workers or pay_idx.numel() != pay_values.numel():
        raise ValueError("payload arrays must hold workers x entries elements")
    per = pay_values.numel() // workers
    _check(lib.demo_decode_signs(ctx, len(shapes), _shapes(shapes), ctypes.byref(cfg), int(workers),
                                 _device_ptr(pay_values, 4), _device_ptr(pay_idx, 2), per, int(avg),
                                 _device_ptr(signs, 8), signs.numel(), _stream_handle(stream)))


def demo_apply_signs(ctx: int, params, signs, eta: float = 1e-3, lam: float = 0.0, chunk: int = DEMO_CHUNK,
                     stream=None) -> None:
    """X <- X - eta * (s + lam * X) with s = -1 where the packed bit is set, else +1."""
    lib = load_library()
    import torch
    for x in params:
        if x.dtype != torch.float32:
            raise ValueError("parameters must be float32")
    _check(lib.demo_apply_signs(ctx, len(params), _shapes([tuple(x.shape) for x in params]),
                                _ptrs([_device_ptr(x, 4) for x in params]), int(chunk), _device_ptr(signs, 8),
                                signs.numel(), float(eta), float(lam), _stream_handle(stream)))


def demo_muon_workspace(shapes: Sequence[Sequence[int]]) -> int:
    """Bytes of device workspace demo_decode_apply_muon needs for a tensor list; host-only."""
    lib = load_library()
    out = ctypes.c_int64()
    _check(lib.demo_muon_workspace(_shapes(shapes), len(shapes), ctypes.byref(out)))
    return out.value


def demo_decode_apply_muon(ctx: int, params, cfg: demo_codec_cfg, workers: int, pay_values, pay_idx, workspace,
                           eta: float = 1e-3, lam: float = 0.0, eps: float = 1e-8, iters: int = 24,
                           avg: int = DEMO_AVG_CONTRIBUTORS, stream=None) -> None:
    """decode_apply with phi = Muon; ``workspace`` is a device buffer of demo_muon_workspace bytes."""
    lib = load_library()
    import torch
    for x in params:
        if x.dtype != torch.float32:
            raise ValueError("parameters must be float32")
    if pay_values.numel() % workers or pay_idx.numel() != pay_values.numel():
        raise ValueError("payload arrays must hold workers x entries elements")
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    per = pay_values.numel() // workers
    _check(lib.demo_decode_apply_muon(ctx, len(params), _shapes([tuple(x.shape) for x in params]),
                                      _ptrs([_device_ptr(x, 4) for x in params]), ctypes.byref(cfg), int(workers),
                                      _device_ptr(pay_values, 4), _device_ptr(pay_idx, 2), per, float(eta),
                                      float(lam), float(eps), int(iters), int(avg), workspace.data_ptr(),
                                      workspace.numel() * workspace.element_size(), _stream_handle(stream)))


DEMO_MUON_SCRATCH_BYTES = 64 << 20


def demo_decode_apply_muon_noalloc(ctx: int, params, cfg: demo_codec_cfg, workers: int, pay_values, pay_idx,
                                   eta: float = 1e-3, lam: float = 0.0, eps: float = 1e-8, iters: int = 24,
                                   avg: int = DEMO_AVG_CONTRIBUTORS, stream=None) -> None:
    """demo_decode_apply_muon on the library's static scratch (no workspace, nothing allocated)."""
    lib = load_library()
    import torch
    for x in params:
        if x.dtype != torch.float32:
            raise ValueError("parameters must be float32")
    if pay_values.numel() % workers or pay_idx.numel() != pay_values.numel():
        raise ValueError("payload arrays must hold workers x entries elements")
    per = pay_values.numel() // workers
    _check(lib.demo_decode_apply_muon_noalloc(ctx, len(params), _shapes([tuple(x.shape) for x in params]),
                                              _ptrs([_device_ptr(x, 4) for x in params]), ctypes.byref(cfg),
                                              int(workers), _device_ptr(pay_values, 4), _device_ptr(pay_idx, 2), per,
                                              float(eta), float(lam), float(eps), int(iters), int(avg),
                                              _stream_handle(stream)))


def demo_wire_size(n_entries: int, chunk: int = DEMO_CHUNK) -> Tuple[int, int]:
    """(value bytes, index bytes) of one worker's wire payload of n_entries entries; host-only."""
    lib = load_library()
    vb, ib = ctypes.c_int64(), ctypes.c_int64()
    _check(lib.demo_wire_size(int(chunk), int(n_entries), ctypes.byref(vb), ctypes.byref(ib)))
    return vb.value, ib.value


def demo_pack_wire(ctx: int, workers: int, pay_values, pay_idx, wire_values, wire_idx, stream=None,
                   chunk: int = DEMO_CHUNK) -> None:
    """``workers`` payloads (worker-major) -> wire values (int16 storage) and wire index bytes (uint8)."""
    lib = load_library()
    if pay_values.numel() % workers or pay_idx.numel() != pay_values.numel():
        raise ValueError("payload arrays must hold workers x entries elements")
    per = pay_values.numel() // workers
    vb, ib = demo_wire_size(per, chunk)
    if wire_values.numel() * wire_values.element_size() != workers * vb:
        raise ValueError("wire value buffer must hold workers x entries 16-bit values")
    if wire_idx.numel() * wire_idx.element_size() != workers * ib:
        raise ValueError("wire index buffer must hold workers x demo_wire_size index bytes")
    _check(lib.demo_pack_wire(ctx, int(chunk), int(workers), _device_ptr(pay_values, 4), _device_ptr(pay_idx, 2), per,
                              _device_ptr(wire_values, 2), _device_ptr(wire_idx, wire_idx.element_size()), _stream_handle(stream)))


def demo_decode_apply_wire(ctx: int, params, cfg: demo_codec_cfg, workers: int, wire_values, wire_idx,
                           phi: int = DEMO_PHI_SIGN, eta: float = 1e-3, lam: float = 0.0,
                           avg: int = DEMO_AVG_CONTRIBUTORS, stream=None) -> None:
    """demo_decode_apply reading ``workers`` wire payloads (worker-major)."""
    lib = load_library()
    import torch
    for x in params:
        if x.dtype != torch.float32:
            raise ValueError("parameters must be float32")
    if wire_values.element_size() != 2 or wire_values.numel() % workers:
        raise ValueError("wire values must hold workers x entries 16-bit values")
    per = wire_values.numel() // workers
    _, ib = demo_wire_size(per, cfg.chunk)
    if wire_idx.numel() * wire_idx.element_size() != workers * ib:
        raise ValueError("wire index buffer must hold workers x demo_wire_size index bytes")
    _check(lib.demo_decode_apply_wire(ctx, len(params), _shapes([tuple(x.shape) for x in params]),
                                      _ptrs([_device_ptr(x, 4) for x in params]), ctypes.byref(cfg), int(workers),
                                      _device_ptr(wire_values, 2), _device_ptr(wire_idx, wire_idx.element_size()), per, int(phi),
                                      float(eta), float(lam), int(avg), _stream_handle(stream)))


class Codec:
    """A context bound to one device plus the codec configuration of a tensor list."""

    def __init__(self, shapes: Sequence[Sequence[int]], k: int, beta: float = 0.999, alpha: float = 0.2,
                 plain: bool = False, device: int = 0, identity: bool = False, aggregated: bool = False,
                 chunk: int = DEMO_CHUNK):
        self.shapes = [tuple(int(d) for d in s) for s in shapes]
        self.chunk = int(chunk)
        self.k = int(k)
        self.beta = float(beta)
        self.alpha = float(alpha)
        self.plain = bool(plain)
        self.identity = bool(identity)
        self.aggregated = bool(aggregated)
        self.n_chunks, self.n_entries, self.entry_begin = demo_plan(self.shapes, self.k, self.chunk)
        self.n_sign_words, self.sign_word_begin = demo_plan_signs(self.shapes, self.chunk)
        self.ctx = demo_ctx_create(device)

    def close(self) -> None:
        if self.ctx:
            demo_ctx_destroy(self.ctx)
            self.ctx = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def cfg(self, P0=None, P1=None) -> demo_codec_cfg:
        return make_cfg(self.k, self.beta, self.alpha, self.plain, P0, P1, chunk=self.chunk,
                        identity=self.identity, aggregated=self.aggregated)

    def alloc_payload(self, workers: int = 1, device="cuda"):
        """Empty payload buffers: float32 values and 16-bit indices (int16 storage of uint16)."""
        import torch
        v = torch.empty(workers * self.n_entries, dtype=torch.float32, device=device)
        i = torch.empty(workers * self.n_entries, dtype=torch.int16, device=device)
        return v, i

    def encode(self, grads, moms, pay_values, pay_idx, P0=None, P1=None, stream=None) -> None:
        demo_encode(self.ctx, grads, moms, self.cfg(P0, P1), pay_values, pay_idx, stream)

    def decode_apply(self, params, workers, pay_values, pay_idx, phi=DEMO_PHI_SIGN, eta=1e-3, lam=0.0,
                     avg=DEMO_AVG_CONTRIBUTORS, P0=None, P1=None, stream=None) -> None:
        demo_decode_apply(self.ctx, params, self.cfg(P0, P1), workers, pay_values, pay_idx, phi, eta, lam,
                          avg, stream)

    def decode_apply_subtract(self, params, moms, workers, pay_values, pay_idx, phi=DEMO_PHI_SIGN, eta=1e-3,
                              lam=0.0, avg=DEMO_AVG_CONTRIBUTORS, P0=None, P1=None, stream=None) -> None:
        demo_decode_apply_subtract(self.ctx, params, moms, self.cfg(P0, P1), workers, pay_values, pay_idx, phi,
                                   eta, lam, avg, stream)

    def alloc_signs(self, device="cuda"):
        """Empty packed-sign buffer: one 64-bit word per 64 elements of every chunk (int64 storage)."""
        import torch
        return torch.empty(self.n_sign_words, dtype=torch.int64, device=device)

    def decode_signs(self, workers, pay_values, pay_idx, signs, avg=DEMO_AVG_CONTRIBUTORS, P0=None, P1=None,
                     stream=None) -> None:
        demo_decode_signs(self.ctx, self.shapes, self.cfg(P0, P1), workers, pay_values, pay_idx, signs, avg,
                          stream)

    def apply_signs(self, params, signs, eta=1e-3, lam=0.0, stream=None) -> None:
        demo_apply_signs(self.ctx, params, signs, eta, lam, chunk=self.chunk, stream=stream)

    def alloc_wire(self, workers: int = 1, device="cuda"):
        """Empty wire buffers: bfloat16 bits (int16 storage) and packed 12- or 14-bit positions (uint8)."""
        import torch
        vb, ib = demo_wire_size(self.n_entries, self.chunk)
        v = torch.empty(workers * vb // 2, dtype=torch.int16, device=device)
        i = torch.empty(workers * ib, dtype=torch.uint8, device=device)
        return v, i

    def pack_wire(self, workers, pay_values, pay_idx, wire_values, wire_idx, stream=None) -> None:
        demo_pack_wire(self.ctx, workers, pay_values, pay_idx, wire_values, wire_idx, stream, chunk=self.chunk)

    def decode_apply_wire(self, params, workers, wire_values, wire_idx, phi=DEMO_PHI_SIGN, eta=1e-3, lam=0.0,
                          avg=DEMO_AVG_CONTRIBUTORS, P0=None, P1=None, stream=None) -> None:
        demo_decode_apply_wire(self.ctx, params, self.cfg(P0, P1), workers, wire_values, wire_idx, phi, eta, lam,
                               avg, stream)

    def alloc_muon_workspace(self, device="cuda"):
        """Device workspace of the Muon decode for this list (uint8 storage)."""
        import torch
        return torch.empty(demo_muon_workspace(self.shapes), dtype=torch.uint8, device=device)

    def decode_apply_muon_noalloc(self, params, workers, pay_values, pay_idx, eta=1e-3, lam=0.0, eps=1e-8,
                                  iters=24, avg=DEMO_AVG_CONTRIBUTORS, P0=None, P1=None, stream=None) -> None:
        demo_decode_apply_muon_noalloc(self.ctx, params, self.cfg(P0, P1), workers, pay_values, pay_idx, eta, lam,
                                       eps, iters, avg, stream)

    def decode_apply_muon(self, params, workers, pay_values, pay_idx, workspace, eta=1e-3, lam=0.0, eps=1e-8,
                          iters=24, avg=DEMO_AVG_CONTRIBUTORS, P0=None, P1=None, stream=None) -> None:
        demo_decode_apply_muon(self.ctx, params, self.cfg(P0, P1), workers, pay_values, pay_idx, workspace, eta, lam,
                               eps, iters, avg, stream)
