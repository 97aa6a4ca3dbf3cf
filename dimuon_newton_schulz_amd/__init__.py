"""Python binding of libmuon_mi355x.so (the MI355X Muon / Dimuon step).

Argument marshalling only: tensors are turned into device pointers and
shapes, and every step of the method runs in the library's HIP kernels.  The
library must be built (``python -m dimuon_newton_schulz_amd.build``); there
is no fallback.

Entry points mirror the C ABI in ``include/muon_mi355x.h``:
``muon_step``, ``dimuon_step``, ``muon_workspace_bytes``,
``muon_status_string``.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import torch  # loads the HIP runtime the library then shares

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmuon_mi355x.so")

MUON_F32, MUON_BF16 = 0, 1
_DT_CODE = {torch.float32: MUON_F32, torch.bfloat16: MUON_BF16}
_DT_NAME = {"f32": MUON_F32, "bf16": MUON_BF16}

STATUS_NAMES = {0: "MUON_OK", 1: "MUON_ERR_INVALID_ARG", 2: "MUON_ERR_DTYPE",
                3: "MUON_ERR_WORKSPACE", 4: "MUON_ERR_ALIAS", 5: "MUON_ERR_HIP",
                6: "MUON_ERR_UNSUPPORTED"}

EXPORTED_SYMBOLS = ("muon_config_default", "muon_workspace_bytes", "muon_step", "dimuon_step", "muon_step_noalloc",
                    "muon_set_launch_events", "muon_plan_create", "muon_plan_step", "muon_plan_set_lr",
                    "muon_plan_reset", "muon_plan_set_graph", "muon_plan_destroy", "muon_status_string", "muon_last_error", "muon_abi_version")

LAUNCH_KINDS = {-1: "start", 0: "thin_b", 1: "momentum", 2: "condition", 3: "prescale", 4: "norm",
                5: "gram", 6: "poly", 7: "combine", 8: "postnorm", 9: "update", 10: "thin_energy",
                11: "thin_a", 12: "momentum_prescale", 13: "energy"}


class MuonMatrix(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("g", ctypes.c_void_p), ("mom", ctypes.c_void_p),
                ("o_out", ctypes.c_void_p), ("energy_out", ctypes.c_void_p),
                ("m", ctypes.c_int64), ("n", ctypes.c_int64),
                ("update_scale", ctypes.c_float), ("reserved0", ctypes.c_float)]


class MuonConfig(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("momentum", ctypes.c_float), ("ns_steps", ctypes.c_int32),
                ("a", ctypes.c_float), ("b", ctypes.c_float), ("c", ctypes.c_float),
                ("coeff_schedule", ctypes.POINTER(ctypes.c_float)),
                ("w_dtype", ctypes.c_int32), ("g_dtype", ctypes.c_int32),
                ("mom_dtype", ctypes.c_int32), ("ns_dtype", ctypes.c_int32),
                ("dimuon_eps", ctypes.c_float), ("nesterov", ctypes.c_int32),
                ("weight_decay", ctypes.c_float), ("reserved", ctypes.c_int32 * 4)]


class MuonError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m dimuon_newton_schulz_amd.build`")
    lib = ctypes.CDLL(path)
    lib.muon_config_default.argtypes = [ctypes.POINTER(MuonConfig)]
    lib.muon_config_default.restype = None
    lib.muon_workspace_bytes.argtypes = [ctypes.POINTER(MuonMatrix), ctypes.c_int64,
                                         ctypes.POINTER(MuonConfig), ctypes.POINTER(ctypes.c_size_t)]
    lib.muon_workspace_bytes.restype = ctypes.c_int
    for name in ("muon_step", "dimuon_step"):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.POINTER(MuonMatrix), ctypes.c_int64, ctypes.POINTER(MuonConfig),
                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    lib.muon_step_noalloc.argtypes = [ctypes.POINTER(MuonMatrix), ctypes.c_int64, ctypes.POINTER(MuonConfig),
                                      ctypes.c_int32, ctypes.c_void_p]
    lib.muon_step_noalloc.restype = ctypes.c_int
    lib.muon_set_launch_events.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32]
    lib.muon_set_launch_events.restype = ctypes.c_int32
    lib.muon_plan_create.argtypes = [ctypes.POINTER(MuonMatrix), ctypes.c_int64, ctypes.POINTER(MuonConfig),
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                     ctypes.POINTER(ctypes.c_void_p)]
    lib.muon_plan_create.restype = ctypes.c_int
    lib.muon_plan_step.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.muon_plan_step.restype = ctypes.c_int
    lib.muon_plan_set_lr.argtypes = [ctypes.c_void_p, ctypes.c_float]
    lib.muon_plan_set_lr.restype = ctypes.c_int
    lib.muon_plan_reset.argtypes = [ctypes.c_void_p]
    lib.muon_plan_reset.restype = ctypes.c_int
    lib.muon_plan_set_graph.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    lib.muon_plan_set_graph.restype = ctypes.c_int
    lib.muon_plan_destroy.argtypes = [ctypes.c_void_p]
    lib.muon_plan_destroy.restype = None
    lib.muon_status_string.argtypes = [ctypes.c_int]
    lib.muon_status_string.restype = ctypes.c_char_p
    lib.muon_last_error.argtypes = []
    lib.muon_last_error.restype = ctypes.c_char_p
    lib.muon_abi_version.argtypes = []
    lib.muon_abi_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def muon_status_string(status: int) -> str:
    return load_library().muon_status_string(status).decode()


def _check(status: int):
    if status != 0:
        lib = load_library()
        raise MuonError(status, lib.muon_last_error().decode() or lib.muon_status_string(status).decode())


@dataclass
class StepConfig:
    """Mirror of muon_config_t with the library's defaults."""
    lr: float = 0.02
    momentum: float = 0.95
    ns_steps: int = 5
    a: float = 3.4445
    b: float = -4.7750
    c: float = 2.0315
    coeff_schedule: Optional[Sequence[Sequence[float]]] = None
    w_dtype: str = "bf16"
    g_dtype: str = "bf16"
    mom_dtype: str = "bf16"
    ns_dtype: str = "bf16"
    dimuon_eps: float = 1e-4
    nesterov: bool = False
    weight_decay: float = 0.0

    def to_c(self):
        cfg = MuonConfig()
        cfg.lr, cfg.momentum, cfg.ns_steps = self.lr, self.momentum, self.ns_steps
        cfg.a, cfg.b, cfg.c = self.a, self.b, self.c
        keep = None
        if self.coeff_schedule is not None:
            flat = [float(v) for row in self.coeff_schedule for v in row]
            keep = (ctypes.c_float * len(flat))(*flat)
            cfg.coeff_schedule = ctypes.cast(keep, ctypes.POINTER(ctypes.c_float))
        cfg.w_dtype = _DT_NAME[self.w_dtype]
        cfg.g_dtype = _DT_NAME[self.g_dtype]
        cfg.mom_dtype = _DT_NAME[self.mom_dtype]
        cfg.ns_dtype = _DT_NAME[self.ns_dtype]
        cfg.dimuon_eps = self.dimuon_eps
        cfg.nesterov = 1 if self.nesterov else 0
        cfg.weight_decay = self.weight_decay
        return cfg, keep


@dataclass
class Param:
    """One matrix of a batch: weight, gradient and momentum tensors."""
    w: torch.Tensor
    g: torch.Tensor
    mom: torch.Tensor
    o_out: Optional[torch.Tensor] = None
    energy_out: Optional[torch.Tensor] = None
    update_scale: float = 1.0


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _marshal(params: Sequence[Param]):
    arr = (MuonMatrix * len(params))()
    for i, p in enumerate(params):
        if p.w.dim() != 2:
            raise ValueError(f"matrix {i}: expected a 2-D weight, got {tuple(p.w.shape)}")
        for name in ("w", "g", "mom", "o_out", "energy_out"):
            t = getattr(p, name)
            if t is not None and not t.is_contiguous():
                raise ValueError(f"matrix {i}: {name} must be contiguous")
        m, n = p.w.shape
        if tuple(p.g.shape) != (m, n) or tuple(p.mom.shape) != (m, n):
            raise ValueError(f"matrix {i}: w, g and mom shapes differ")
        if p.o_out is not None and (tuple(p.o_out.shape) != (m, n) or p.o_out.dtype != torch.float32):
            raise ValueError(f"matrix {i}: o_out must be float32 {m}x{n}")
        if p.energy_out is not None and (p.energy_out.numel() != m + n or p.energy_out.dtype != torch.float32):
            raise ValueError(f"matrix {i}: energy_out must be float32 with m+n elements")
        arr[i].w, arr[i].g, arr[i].mom = _ptr(p.w), _ptr(p.g), _ptr(p.mom)
        arr[i].o_out, arr[i].energy_out = _ptr(p.o_out), _ptr(p.energy_out)
        arr[i].m, arr[i].n = m, n
        arr[i].update_scale = float(p.update_scale)
    return arr


def config_for(params: Sequence[Param], ns_dtype: str = "bf16", **kw) -> StepConfig:
    """StepConfig whose w/g/mom dtypes are those of the first matrix."""
    p = params[0]
    name = {torch.float32: "f32", torch.bfloat16: "bf16"}
    return StepConfig(w_dtype=name[p.w.dtype], g_dtype=name[p.g.dtype], mom_dtype=name[p.mom.dtype],
                      ns_dtype=ns_dtype, **kw)


def _check_dtypes(params: Sequence[Param], cfg: StepConfig):
    want = {"w": _DT_NAME[cfg.w_dtype], "g": _DT_NAME[cfg.g_dtype], "mom": _DT_NAME[cfg.mom_dtype]}
    for i, p in enumerate(params):
        for name, code in want.items():
            t = getattr(p, name)
            if _DT_CODE.get(t.dtype) != code:
                raise ValueError(f"matrix {i}: {name} is {t.dtype}, config says {getattr(cfg, name + '_dtype')}")


def muon_workspace_bytes(params: Sequence[Param], cfg: StepConfig) -> int:
    lib = load_library()
    arr = _marshal(params)
    c, _keep = cfg.to_c()
    out = ctypes.c_size_t(0)
    _check(lib.muon_workspace_bytes(arr, len(params), ctypes.byref(c), ctypes.byref(out)))
    return int(out.value)


def workspace_for(params: Sequence[Param], cfg: StepConfig, device=None) -> torch.Tensor:
    nbytes = muon_workspace_bytes(params, cfg)
    dev = device if device is not None else params[0].w.device
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)


def _torch_stream(stream, device):
    """The launch stream as a torch stream object (None: the current stream)."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if hasattr(stream, "cuda_stream"):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _step(fn_name: str, params: Sequence[Param], cfg: StepConfig, workspace: Optional[torch.Tensor],
          stream=None):
    lib = load_library()
    _check_dtypes(params, cfg)
    arr = _marshal(params)
    c, _keep = cfg.to_c()
    device = params[0].w.device
    ts = _torch_stream(stream, device)
    if workspace is None:
        workspace = workspace_for(params, cfg)
        # Allocated on the current stream; if the kernels run on another one,
        # the caching allocator must not hand the block out again before they
        # finish.
        if ts != torch.cuda.current_stream(device):
            workspace.record_stream(ts)
    fn = getattr(lib, fn_name)
    with torch.cuda.device(device):
        _check(fn(arr, len(params), ctypes.byref(c), ctypes.c_void_p(workspace.data_ptr()),
                  ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(ts.cuda_stream)))
    return workspace


def muon_step(params: Sequence[Param], cfg: StepConfig, workspace: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """One Muon step over the batch (asynchronous on ``stream``).  Returns the workspace."""
    return _step("muon_step", params, cfg, workspace, stream)


def dimuon_step(params: Sequence[Param], cfg: StepConfig, workspace: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """One Dimuon step over the batch (asynchronous on ``stream``).  Returns the workspace."""
    return _step("dimuon_step", params, cfg, workspace, stream)


NOALLOC_MAX_BYTES = 64 << 20   # MUON_NOALLOC_MAX_BYTES


def muon_step_noalloc(params: Sequence[Param], cfg: StepConfig, dimuon: bool, stream=None) -> None:
    """One Muon (dimuon False) or Dimuon step without a workspace argument:
    the library's static device scratch serves (muon_step_noalloc).  Nothing
    is allocated; calls on one GPU must be ordered (they share the scratch)."""
    lib = load_library()
    _check_dtypes(params, cfg)
    arr = _marshal(params)
    c, _keep = cfg.to_c()
    device = params[0].w.device
    ts = _torch_stream(stream, device)
    with torch.cuda.device(device):
        _check(lib.muon_step_noalloc(arr, len(params), ctypes.byref(c), 1 if dimuon else 0,
                                     ctypes.c_void_p(ts.cuda_stream)))


class LaunchTimer:
    """Per-launch HIP events for one step at a time (timing only).

    ``with LaunchTimer(capacity) as t: step(...); ...; t.durations()`` returns
    [(kind, ms)] for the launches of the last step, measured on its stream."""

    def __init__(self, capacity: int = 256):
        self.capacity = capacity
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]
        # torch.cuda.Event creates the HIP event lazily; record once to create it.
        for e in self.events:
            e.record()
        self.handles = (ctypes.c_void_p * capacity)(*[e.cuda_event for e in self.events])
        self.kinds = (ctypes.c_int32 * capacity)()

    def __enter__(self):
        load_library().muon_set_launch_events(self.handles, self.kinds, self.capacity)
        return self

    def __exit__(self, *exc):
        load_library().muon_set_launch_events(None, None, 0)

    def durations(self, count: int):
        """(kind name, ms) of launches 1..count-1 of the last step (after synchronising)."""
        out = []
        for i in range(1, count):
            out.append((LAUNCH_KINDS[self.kinds[i]], self.events[i - 1].elapsed_time(self.events[i])))
        return out

    def recorded(self) -> int:
        lib = load_library()
        n = lib.muon_set_launch_events(self.handles, self.kinds, self.capacity)
        return n


def _stream_handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class Plan:
    """A prepared batch (muon_plan_t): validated and uploaded once, then
    stepped repeatedly.  Keeps the tensors and the workspace alive."""

    def __init__(self, params: Sequence[Param], cfg: StepConfig, dimuon: bool,
                 workspace: Optional[torch.Tensor] = None, stream=None):
        lib = load_library()
        _check_dtypes(params, cfg)
        self.params = list(params)
        self.cfg = cfg
        self.device = params[0].w.device
        self.workspace = workspace if workspace is not None else workspace_for(params, cfg)
        arr = _marshal(params)
        c, keep = cfg.to_c()
        handle = ctypes.c_void_p(0)
        with torch.cuda.device(self.device):
            _check(lib.muon_plan_create(arr, len(params), ctypes.byref(c), 1 if dimuon else 0,
                                        ctypes.c_void_p(self.workspace.data_ptr()),
                                        ctypes.c_size_t(self.workspace.numel()),
                                        ctypes.c_void_p(_stream_handle(stream, self.device)),
                                        ctypes.byref(handle)))
        self._handle = handle
        self._lib = lib

    def step(self, stream=None):
        _check(self._lib.muon_plan_step(self._handle, ctypes.c_void_p(_stream_handle(stream, self.device))))

    def set_lr(self, lr: float):
        _check(self._lib.muon_plan_set_lr(self._handle, lr))

    def reset(self):
        """Call after writing to the momentum buffers outside the plan."""
        _check(self._lib.muon_plan_reset(self._handle))

    def set_graph(self, enable: bool = True):
        """Replay the launch sequence as a HIP graph (muon_plan_set_graph)."""
        _check(self._lib.muon_plan_set_graph(self._handle, 1 if enable else 0))

    def close(self):
        if self._handle:
            self._lib.muon_plan_destroy(self._handle)
            self._handle = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


__all__ = ["MuonMatrix", "MuonConfig", "MuonError", "StepConfig", "Param", "load_library",
           "muon_step", "dimuon_step", "muon_step_noalloc", "muon_workspace_bytes", "muon_status_string",
           "Plan", "workspace_for", "config_for", "EXPORTED_SYMBOLS", "LaunchTimer",
           "LAUNCH_KINDS"]
