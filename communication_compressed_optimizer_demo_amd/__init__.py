"""DeMo per-step momentum codec for AMD MI355X (gfx950).

The codec runs in hand-written HIP kernels behind the C ABI declared in
``include/demo_codec.h``; this package holds their sources (``csrc/``), the
in-tree build (``build.py``) and a thin ctypes binding (``binding.py``).
"""
from .binding import (  # noqa: F401
    DEMO_AVG_CONTRIBUTORS, DEMO_AVG_WORKERS, DEMO_BASIS_DCT, DEMO_BASIS_IDENTITY, DEMO_BASIS_USER, DEMO_BF16,
    DEMO_CHUNK, DEMO_CHUNK_LARGE, DEMO_F32, DEMO_MAX_TENSORS_PER_LAUNCH, DEMO_MAX_WORKERS, DEMO_MOMENTUM_DAMPED, DEMO_MOMENTUM_PLAIN,
    DEMO_PHI_IDENTITY, DEMO_PHI_SIGN, DEMO_SUBTRACT_AGGREGATED, DEMO_SUBTRACT_LOCAL, Codec, DemoError, LIB_PATH,
    demo_apply_signs, demo_ctx_create, demo_ctx_destroy, demo_decode_apply, demo_decode_apply_subtract,
    demo_decode_apply_muon, demo_decode_apply_wire, demo_decode_signs, demo_encode, demo_muon_workspace,
    demo_pack_wire, demo_plan, demo_plan_signs, demo_wire_size, load_library, make_cfg,
)
