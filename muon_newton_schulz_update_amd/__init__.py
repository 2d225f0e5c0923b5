"""Python binding of libmuon, the MI355X (gfx950) Muon / Aurora-Muon step.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libmuon.so, reached through its C ABI (include/libmuon.h) with
ctypes. PyTorch supplies device memory and the current stream.

    import torch, muon_newton_schulz_update_amd as mu
    mu.muon_update(grads, moms, weights, update_out=outs)
    U = mu.ns_polar([G])[0]
    U = mu.aurora_orthogonalize([G])[0]

The entry points take lists of 2-D CUDA tensors with unit column stride
(row stride = ld). Grads, weights and outputs may be float32 or bfloat16;
momentum is float32. Calls are asynchronous on torch's current stream.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Iterable, Sequence

import torch  # loaded first so libmuon binds to the HIP runtime torch already mapped

__all__ = [
    "MuonConfig", "MuonProfile", "LibMuonError", "Handle", "load_library",
    "library_path", "default_config", "classic_config", "momentum_warmup", "make_config", "ns_polar",
    "aurora_orthogonalize", "muon_update", "check_update_args",
    "check_polar_args", "get_handle", "STATUS", "muon_update_static", "MUON_FLAG_SGD_MOMENTUM", "MUON_FLAG_WIDE_ROWS",
    "MUON_FLAG_FP8_GRAM", "MUON_FLAG_CHECK_FINITE", "debug_check_plan",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmuon.so"

MUON_F32, MUON_BF16 = 0, 1
# muon_config.flags bits (include/libmuon.h)
MUON_FLAG_SGD_MOMENTUM = 0x1    # classic recipe's SGD momentum (buf = mu buf + G)
MUON_FLAG_WIDE_ROWS = 0x2       # Aurora on a wide matrix's own rows
MUON_FLAG_FP8_GRAM = 0x4        # fp8 operands for the first Gram of each pass (research option)
MUON_FLAG_CHECK_FINITE = 0x8    # refuse (MUON_ERR_NONFINITE, nothing written) inputs with a NaN or Inf
STATUS = {
    0: "MUON_OK", -1: "MUON_ERR_INVALID_ARG", -2: "MUON_ERR_UNSUPPORTED_DTYPE",
    -3: "MUON_ERR_SHAPE_MISMATCH", -4: "MUON_ERR_ALLOC", -5: "MUON_ERR_HIP",
    -6: "MUON_ERR_NO_DEVICE", -7: "MUON_ERR_TOO_LARGE", -8: "MUON_ERR_NONFINITE",
}


class MuonMatrix(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("ld", ctypes.c_int64),
                ("dtype", ctypes.c_int32)]


class MuonConfig(ctypes.Structure):
    _fields_ = [("ns_steps", ctypes.c_int32), ("ns_a", ctypes.c_float),
                ("ns_b", ctypes.c_float), ("ns_c", ctypes.c_float),
                ("ns_eps", ctypes.c_float), ("pp_iterations", ctypes.c_int32),
                ("pp_beta", ctypes.c_float), ("pp_eps", ctypes.c_float),
                ("mu", ctypes.c_float), ("nesterov", ctypes.c_int32),
                ("power_steps", ctypes.c_int32), ("contra", ctypes.c_float),
                ("target_uw", ctypes.c_float), ("lr", ctypes.c_float),
                ("flags", ctypes.c_uint32)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class MuonProfile(ctypes.Structure):
    _fields_ = [("gemm_launches", ctypes.c_int64), ("gemm_ms", ctypes.c_double),
                ("gemm_counted_flop", ctypes.c_double),
                ("gemm_executed_flop", ctypes.c_double),
                ("gemm_algorithmic_flop", ctypes.c_double),
                ("stream_launches", ctypes.c_int64), ("stream_ms", ctypes.c_double),
                ("stream_bytes", ctypes.c_double), ("aux_launches", ctypes.c_int64),
                ("aux_ms", ctypes.c_double), ("aux_bytes", ctypes.c_double)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class LibMuonError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {message}")


_lib = None
_lib_lock = threading.Lock()


def library_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def load_library() -> ctypes.CDLL:
    """Load libmuon.so from the package directory (raises if it is not built)."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m muon_newton_schulz_update_amd.build`")
        lib = ctypes.CDLL(path)
        P = ctypes.POINTER
        sig = {
            "muon_config_default": (None, [P(MuonConfig)]),
            "muon_config_classic": (None, [P(MuonConfig)]),
            "muon_momentum_warmup": (ctypes.c_float, [ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                                                      ctypes.c_int64]),
            "muon_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "muon_version": (ctypes.c_char_p, []),
            "muon_create": (ctypes.c_int, [P(ctypes.c_void_p), ctypes.c_void_p]),
            "muon_destroy": (ctypes.c_int, [ctypes.c_void_p]),
            "muon_set_stream": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p]),
            "muon_last_error": (ctypes.c_char_p, [ctypes.c_void_p]),
            "muon_check_update_args": (ctypes.c_int, [ctypes.c_int, P(MuonMatrix), P(MuonMatrix),
                                                      P(MuonMatrix), P(MuonMatrix), P(MuonConfig),
                                                      ctypes.c_char_p, ctypes.c_int]),
            "muon_check_polar_args": (ctypes.c_int, [ctypes.c_int, P(MuonMatrix), P(MuonMatrix),
                                                     P(MuonConfig), ctypes.c_char_p, ctypes.c_int]),
            "muon_reserve": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, P(MuonMatrix)]),
            "muon_debug_check_plan": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, P(MuonMatrix), P(MuonConfig),
                                                     ctypes.c_char_p, ctypes.c_int]),
            "ns_polar": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, P(MuonMatrix),
                                        P(MuonMatrix), P(MuonConfig)]),
            "aurora_orthogonalize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, P(MuonMatrix),
                                                    P(MuonMatrix), P(MuonConfig)]),
            "muon_update": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, P(MuonMatrix),
                                           P(MuonMatrix), P(MuonMatrix), P(MuonMatrix),
                                           P(MuonConfig)]),
            "muon_update_static": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, P(MuonMatrix),
                                                  P(MuonMatrix), P(MuonMatrix), P(MuonMatrix),
                                                  P(MuonConfig)]),
            "muon_profile_enable": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int]),
            "muon_profile_reset": (ctypes.c_int, [ctypes.c_void_p]),
            "muon_profile_read": (ctypes.c_int, [ctypes.c_void_p, P(MuonProfile)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def default_config() -> MuonConfig:
    cfg = MuonConfig()
    load_library().muon_config_default(ctypes.byref(cfg))
    return cfg


def classic_config() -> MuonConfig:
    """The classic five-step Muon recipe (muon_config_classic)."""
    cfg = MuonConfig()
    load_library().muon_config_classic(ctypes.byref(cfg))
    return cfg


def momentum_warmup(step: int, mu_start: float = 0.85, mu_end: float = 0.95, warmup_steps: int = 500) -> float:
    """Host-side momentum warm-up of the classic recipe (muon_momentum_warmup)."""
    return float(load_library().muon_momentum_warmup(int(step), float(mu_start), float(mu_end),
                                                     int(warmup_steps)))


def make_config(recipe: str = "aurora", **overrides) -> MuonConfig:
    """A recipe's values ("aurora": the page's locked values, the default;
    "classic": the five-step Muon recipe) with keyword overrides."""
    if recipe == "aurora":
        cfg = default_config()
    elif recipe == "classic":
        cfg = classic_config()
    else:
        raise ValueError(f"unknown recipe {recipe!r}")
    for k, v in overrides.items():
        if k not in dict(MuonConfig._fields_):
            raise KeyError(f"unknown config field {k!r}")
        setattr(cfg, k, int(v) if isinstance(v, bool) else v)
    return cfg


# ---------------------------------------------------------------------------
# descriptors
# ---------------------------------------------------------------------------
_DT = {torch.float32: MUON_F32, torch.bfloat16: MUON_BF16}


def _desc(t: torch.Tensor | None, what: str) -> MuonMatrix:
    if t is None:
        return MuonMatrix(None, 0, 0, 0, MUON_F32)
    if t.dim() != 2:
        raise ValueError(f"{what}: expected a 2-D tensor, got shape {tuple(t.shape)}")
    if t.dtype not in _DT:
        raise TypeError(f"{what}: dtype {t.dtype} is not float32 or bfloat16")
    rows, cols = t.shape
    if rows and cols:
        if not t.is_cuda:
            raise ValueError(f"{what}: tensor must live on a GPU")
        if t.stride(1) != 1 and cols > 1:
            raise ValueError(f"{what}: columns must be contiguous (stride(1) == 1)")
    return MuonMatrix(t.data_ptr() if rows and cols else None, rows, cols, row_stride(t), _DT[t.dtype])


def row_stride(t: torch.Tensor) -> int:
    """The descriptor's ld for a 2-D tensor: its row stride as it is, so that a
    view whose rows overlap (stride(0) < cols, e.g. an expanded tensor) is
    rejected by the library (MUON_ERR_SHAPE_MISMATCH) instead of being given
    rows it does not own. A single row has no stride to speak of."""
    rows, cols = t.shape
    return t.stride(0) if rows > 1 else max(cols, 1)


def _array(descs: Sequence[MuonMatrix]):
    arr = (MuonMatrix * max(1, len(descs)))()
    for i, d in enumerate(descs):
        arr[i] = d
    return arr


# ---------------------------------------------------------------------------
# handles (one per device and thread)
# ---------------------------------------------------------------------------
class Handle:
    def __init__(self, device: int | None = None):
        self._lib = load_library()
        self.device = torch.cuda.current_device() if device is None else int(device)
        h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            stream = torch.cuda.current_stream(self.device).cuda_stream
            rc = self._lib.muon_create(ctypes.byref(h), ctypes.c_void_p(stream))
        if rc != 0:
            raise LibMuonError(rc, "muon_create failed (is a gfx950 GPU present?)")
        self._h = h
        self._stream = stream

    def _bind_stream(self) -> None:
        stream = torch.cuda.current_stream(self.device).cuda_stream
        if stream != self._stream:
            self._check(self._lib.muon_set_stream(self._h, ctypes.c_void_p(stream)))
            self._stream = stream

    def _check(self, rc: int) -> None:
        if rc != 0:
            msg = self._lib.muon_last_error(self._h)
            raise LibMuonError(rc, msg.decode() if msg else "")

    @property
    def ptr(self) -> ctypes.c_void_p:
        return self._h

    def reserve(self, shapes: Iterable[tuple[int, int, torch.dtype]]) -> None:
        descs = [MuonMatrix(None, r, c, c, _DT[dt]) for r, c, dt in shapes]
        self._check(self._lib.muon_reserve(self._h, len(descs), _array(descs)))

    def profile_enable(self, on: bool = True) -> None:
        self._check(self._lib.muon_profile_enable(self._h, 1 if on else 0))

    def profile_reset(self) -> None:
        self._check(self._lib.muon_profile_reset(self._h))

    def profile_read(self) -> dict:
        p = MuonProfile()
        self._check(self._lib.muon_profile_read(self._h, ctypes.byref(p)))
        return p.as_dict()

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.muon_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_handles: dict = {}


def get_handle(device: int | None = None) -> Handle:
    dev = torch.cuda.current_device() if device is None else int(device)
    key = (dev, threading.get_ident())
    h = _handles.get(key)
    if h is None:
        h = Handle(dev)
        _handles[key] = h
    return h


def _device_of(tensors: Sequence[torch.Tensor]) -> int | None:
    for t in tensors:
        if t is not None and t.is_cuda:
            return t.device.index
    return None


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def ns_polar(inputs: Sequence[torch.Tensor], outputs: Sequence[torch.Tensor] | None = None,
             cfg: MuonConfig | None = None, handle: Handle | None = None) -> list[torch.Tensor]:
    """out_i = Newton-Schulz polar factor of in_i (libmuon `ns_polar`)."""
    return _polar("ns_polar", inputs, outputs, cfg, handle)


def aurora_orthogonalize(inputs: Sequence[torch.Tensor], outputs: Sequence[torch.Tensor] | None = None,
                         cfg: MuonConfig | None = None, handle: Handle | None = None) -> list[torch.Tensor]:
    """Leverage-equilibrated polar (libmuon `aurora_orthogonalize`)."""
    return _polar("aurora_orthogonalize", inputs, outputs, cfg, handle)


def _polar(name, inputs, outputs, cfg, handle):
    inputs = list(inputs)
    if outputs is None:
        outputs = [torch.empty_like(t) for t in inputs]
    outputs = list(outputs)
    if len(outputs) != len(inputs):
        raise ValueError("inputs and outputs differ in length")
    h = handle or get_handle(_device_of(inputs))
    h._bind_stream()
    ins = _array([_desc(t, "in") for t in inputs])
    outs = _array([_desc(t, "out") for t in outputs])
    fn = getattr(h._lib, name)
    h._check(fn(h.ptr, len(inputs), ins, outs, ctypes.byref(cfg) if cfg is not None else None))
    return outputs


def muon_update(grads: Sequence[torch.Tensor], momenta: Sequence[torch.Tensor],
                weights: Sequence[torch.Tensor | None] | None = None,
                cfg: MuonConfig | None = None,
                update_out: Sequence[torch.Tensor | None] | None = None,
                handle: Handle | None = None) -> None:
    """One Aurora + Contra-Muon + u/w-floor step (libmuon `muon_update`).

    Momenta and weights are updated in place; update_out[i], when given,
    receives the update after the floor and before the learning rate.
    """
    _update("muon_update", grads, momenta, weights, cfg, update_out, handle)


def _update(name, grads, momenta, weights, cfg, update_out, handle):
    grads = list(grads)
    momenta = list(momenta)
    n = len(grads)
    if len(momenta) != n:
        raise ValueError("grads and momenta differ in length")
    if weights is not None and len(weights) != n:
        raise ValueError("weights has the wrong length")
    if update_out is not None and len(update_out) != n:
        raise ValueError("update_out has the wrong length")
    h = handle or get_handle(_device_of(grads))
    h._bind_stream()
    g = _array([_desc(t, "grad") for t in grads])
    m = _array([_desc(t, "momentum") for t in momenta])
    w = _array([_desc(t, "weight") for t in weights]) if weights is not None else None
    u = _array([_desc(t, "update_out") for t in update_out]) if update_out is not None else None
    fn = getattr(h._lib, name)
    h._check(fn(h.ptr, n, g, m, w, u, ctypes.byref(cfg) if cfg is not None else None))


def muon_update_static(grads: Sequence[torch.Tensor], momenta: Sequence[torch.Tensor],
                       weights: Sequence[torch.Tensor | None] | None = None,
                       cfg: MuonConfig | None = None,
                       update_out: Sequence[torch.Tensor | None] | None = None,
                       handle: Handle | None = None) -> None:
    """`muon_update` through libmuon's `muon_update_static`: the call itself
    allocates no device memory (its workspace is the library's static
    per-device scratch, 64 MiB), for batches that fit it."""
    _update("muon_update_static", grads, momenta, weights, cfg, update_out, handle)


def check_update_args(grads, momenta, weights=None, update_out=None, cfg=None) -> tuple[int, str]:
    """Host-only validation (no device needed). Descriptors may be MuonMatrix objects."""
    lib = load_library()
    conv = lambda xs: _array(list(xs)) if xs is not None else None
    buf = ctypes.create_string_buffer(256)
    rc = lib.muon_check_update_args(len(grads), conv(grads), conv(momenta), conv(weights),
                                    conv(update_out), ctypes.byref(cfg) if cfg is not None else None,
                                    buf, 256)
    return rc, buf.value.decode()


def debug_check_plan(kind: str, shapes, cfg=None) -> tuple[int, str]:
    """Host-only check of the launch plan for a batch (libmuon
    `muon_debug_check_plan`; no device needed). kind: "update", "polar" or
    "aurora"; shapes: (rows, cols, torch dtype) triples."""
    lib = load_library()
    descs = [MuonMatrix(None, r, c, c, MUON_BF16 if dt == torch.bfloat16 else MUON_F32) for r, c, dt in shapes]
    buf = ctypes.create_string_buffer(512)
    rc = lib.muon_debug_check_plan({"update": 0, "polar": 1, "aurora": 2}[kind], len(descs),
                                   _array(descs) if descs else None,
                                   ctypes.byref(cfg) if cfg is not None else None, buf, 512)
    return rc, buf.value.decode()


def check_polar_args(inputs, outputs, cfg=None) -> tuple[int, str]:
    lib = load_library()
    buf = ctypes.create_string_buffer(256)
    rc = lib.muon_check_polar_args(len(inputs), _array(list(inputs)), _array(list(outputs)),
                                   ctypes.byref(cfg) if cfg is not None else None, buf, 256)
    return rc, buf.value.decode()
