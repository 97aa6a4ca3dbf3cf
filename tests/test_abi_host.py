"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and rejects invalid calls before touching the GPU (validation precedes any
HIP call, so these run without a device)."""

import ctypes
import os
import re

import pytest

import dimuon_newton_schulz_amd as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon_mi355x.h")

pytestmark = pytest.mark.skipif(not os.path.exists(D.LIB_PATH), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_]+)\s*\(", text)) - {"sizeof"})


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("muon_step", "dimuon_step", "muon_workspace_bytes", "muon_status_string"):
        assert want in names
    assert set(names) == set(D.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = D.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.muon_abi_version() == 1


def _mats(shapes, base=0x100000000):
    arr = (D.MuonMatrix * len(shapes))()
    for i, (m, n) in enumerate(shapes):
        stride = 0x10000000
        arr[i].w = base + 3 * i * stride
        arr[i].g = base + (3 * i + 1) * stride
        arr[i].mom = base + (3 * i + 2) * stride
        arr[i].m, arr[i].n = m, n
        arr[i].update_scale = 1.0
    return arr


def _cfg(**kw):
    c, keep = D.StepConfig(**kw).to_c()
    return c, keep


def _ws_bytes(arr, n, cfg):
    out = ctypes.c_size_t(0)
    st = D.load_library().muon_workspace_bytes(arr, n, ctypes.byref(cfg), ctypes.byref(out))
    return st, out.value


def test_config_default_matches_pages():
    lib = D.load_library()
    c = D.MuonConfig()
    lib.muon_config_default(ctypes.byref(c))
    assert (round(c.a, 4), round(c.b, 4), round(c.c, 4)) == (3.4445, -4.775, 2.0315)
    assert c.ns_steps == 5 and abs(c.momentum - 0.95) < 1e-7 and abs(c.dimuon_eps - 1e-4) < 1e-10


def test_workspace_sizes():
    c, _ = _cfg()
    st, thin = _ws_bytes(_mats([(8, 4096), (4096, 8)]), 2, c)
    assert st == 0 and thin < 1 << 20          # the thin path: table, energy caches, Gram partials
    st, big = _ws_bytes(_mats([(4096, 4096)]), 1, c)
    assert st == 0
    # two X buffers (the bf16 combine reads X itself), A, B and Z, all bf16,
    # of 4096^2 at least, and no X^T copies
    assert 4096 * 4096 * 2 * (2 + 2 + 1) <= big < 4096 * 4096 * 2 * (4 + 2 + 1)
    c32, _ = _cfg(ns_dtype="f32")
    st, big32 = _ws_bytes(_mats([(4096, 4096)]), 1, c32)
    # fp32: four X buffers (X and X^T, ping and pong), A, B and Z
    assert st == 0 and big32 >= 4096 * 4096 * 4 * (4 + 2 + 1)
    st, ragged = _ws_bytes(_mats([(300, 700)]), 1, c)
    assert st == 0 and ragged >= 384 * 768 * 2 * 4
    # A Gram side of 1408 (an odd multiple of 128) stays 1408: X twice, A,
    # B and Z, and nothing padded to 1536.
    st, moe = _ws_bytes(_mats([(1408, 2048)]), 1, c)
    assert st == 0 and 2 * (2 * 1408 * 2048 + 2 * 1408 * 1408 + 1408 * 2048) <= moe < \
        2 * (2 * 1536 * 2048 + 2 * 1536 * 1536 + 1536 * 2048)


@pytest.mark.parametrize("kind", ["null_mats", "count0", "zero_dim", "too_big", "steps", "dtype", "eps",
                                  "nan_lr", "null_w", "misaligned", "alias", "ws_null", "ws_small",
                                  "ws_misaligned", "ws_alias"])
def test_invalid_calls_rejected_before_launch(kind):
    lib = D.load_library()
    shapes = [(64, 256), (256, 64)]
    arr = _mats(shapes)
    c, keep = _cfg()
    ws, ws_bytes, count = ctypes.c_void_p(0x700000000000), 1 << 40, 2
    want = 1
    if kind == "null_mats":
        arr = None
    elif kind == "count0":
        count = 0
    elif kind == "zero_dim":
        arr[1].n = 0
    elif kind == "too_big":
        arr[0].m = 70000
        want = 6
    elif kind == "steps":
        c.ns_steps = 33
    elif kind == "dtype":
        c.ns_dtype = 7
        want = 2
    elif kind == "eps":
        c.dimuon_eps = -1.0
    elif kind == "nan_lr":
        c.lr = float("nan")
    elif kind == "null_w":
        arr[0].w = None
    elif kind == "misaligned":
        arr[1].g = arr[1].g + 4
    elif kind == "alias":
        arr[1].mom = arr[0].w + 64
        want = 4
    elif kind == "ws_null":
        ws = None
        want = 3
    elif kind == "ws_small":
        ws_bytes = 1024
        want = 3
    elif kind == "ws_misaligned":
        ws = ctypes.c_void_p(0x700000000010)
        want = 3
    elif kind == "ws_alias":
        ws = ctypes.c_void_p(arr[0].w)
        want = 4
    for fn in (lib.muon_step, lib.dimuon_step):
        st = fn(arr, count, ctypes.byref(c), ws, ws_bytes, None)
        assert st == want, (kind, st, lib.muon_last_error())
        assert lib.muon_last_error()


def test_read_only_gradients_may_share_memory():
    # Two matrices reading the same gradient buffer is allowed; the workspace
    # check then fails (NULL), which proves validation got past aliasing.
    lib = D.load_library()
    arr = _mats([(64, 256), (64, 256)])
    arr[1].g = arr[0].g
    c, _ = _cfg()
    assert lib.muon_step(arr, 2, ctypes.byref(c), None, 0, None) == 3


def test_status_strings():
    for code in range(7):
        assert D.muon_status_string(code)
    assert D.muon_status_string(99) == "unknown status"


def test_plan_create_rejects_invalid_batches():
    lib = D.load_library()
    arr = _mats([(64, 256), (256, 64)])
    c, _ = _cfg()
    out = ctypes.c_void_p(123)
    assert lib.muon_plan_create(arr, 2, ctypes.byref(c), 1, None, 0, None, ctypes.byref(out)) == 3
    assert out.value is None
    arr[1].w = arr[0].w
    assert lib.muon_plan_create(arr, 2, ctypes.byref(c), 0, ctypes.c_void_p(0x700000000000), 1 << 40, None,
                                ctypes.byref(out)) == 4
    assert lib.muon_plan_step(None, None) == 1
    assert lib.muon_plan_set_lr(None, 0.1) == 1
    lib.muon_plan_destroy(None)


def test_binding_records_workspace_on_launch_stream(monkeypatch):
    # A workspace the binding allocates on the current stream is recorded on
    # the launch stream when the two differ, and not otherwise (CPU: the
    # library, the allocation and the streams are stand-ins).
    import torch

    class FakeStream:
        def __init__(self, h):
            self.cuda_stream = h

        def __eq__(self, other):
            return isinstance(other, FakeStream) and other.cuda_stream == self.cuda_stream

        def __ne__(self, other):
            return not self == other

    class FakeWorkspace:
        def __init__(self):
            self.recorded = []

        def record_stream(self, s):
            self.recorded.append(s)

        def data_ptr(self):
            return 0x1000

        def numel(self):
            return 256

    class FakeLib:
        def __init__(self):
            self.calls = []

        def muon_step(self, arr, n, cfg, ws, ws_bytes, stream):
            self.calls.append(stream.value or 0)
            return 0

    lib = FakeLib()
    current = FakeStream(0)
    made = []

    def fake_ws(params, cfg, device=None):
        made.append(FakeWorkspace())
        return made[-1]

    monkeypatch.setattr(D, "load_library", lambda *a, **k: lib)
    monkeypatch.setattr(D, "workspace_for", fake_ws)
    monkeypatch.setattr(torch.cuda, "current_stream", lambda device=None: current)
    monkeypatch.setattr(torch.cuda, "device", lambda d: __import__("contextlib").nullcontext())
    t = torch.zeros(8, 64, dtype=torch.bfloat16)
    p = D.Param(w=t, g=t.clone(), mom=t.clone())
    D.muon_step([p], D.StepConfig())
    assert made[-1].recorded == [] and lib.calls[-1] == 0
    side = FakeStream(77)
    D.muon_step([p], D.StepConfig(), stream=side)
    assert made[-1].recorded == [side] and lib.calls[-1] == 77


def test_noalloc_rejects_oversized_batch_before_any_hip_call():
    # 4096 x 4096 in bf16 needs far more than the 64 MiB static scratch; the
    # check runs on the host before the scratch is looked up.
    lib = D.load_library()
    arr = _mats([(4096, 4096)])
    cfg, _keep = _cfg()
    st, need = _ws_bytes(arr, 1, cfg)
    assert st == 0 and need > D.NOALLOC_MAX_BYTES
    st = lib.muon_step_noalloc(arr, 1, ctypes.byref(cfg), 0, None)
    assert st == 3, st
    assert b"static scratch" in lib.muon_last_error()
