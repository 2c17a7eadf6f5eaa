"""CPU-side checks of the C ABI: the library loads, exports every function
``include/moe.h`` declares, and refuses bad arguments on the host before any
launch (no GPU is touched by these calls)."""
import ctypes
import os
import re

import pytest

import sparse_moe_layer_wg_amd as moe
from sparse_moe_layer_wg_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = moe.library()
    names = declared_functions()
    assert set(names) >= {"moe_gate", "moe_dispatch", "moe_expert_ffn", "moe_combine",
                          "moe_layer_forward", "moe_capacity", "moe_workspace_bytes",
                          "moe_status_string"}
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_config_struct_matches_header_layout():
    # int32 x6, double, int32, uint32 -> 40 bytes with the double at offset 24
    assert ctypes.sizeof(moe.MoeConfig) == 40
    assert moe.MoeConfig.capacity_factor.offset == 24
    assert moe.MoeConfig.act_dtype.offset == 32


def test_capacity_formula():
    for (S, E, k, cf, C) in [(256, 8, 2, 1.25, 80), (16384, 128, 2, 2.0, 512),
                             (16384, 128, 2, 1.0, 256), (65536, 64, 2, 1.25, 2560),
                             (8192, 256, 8, 1.5, 384), (10, 3, 1, 1.0, 4), (0, 4, 2, 1.0, 0)]:
        assert moe.capacity(moe.config(S, 64, 64, E, k, cf)) == C
    assert moe.capacity(moe.config(100, 64, 64, 8, 2, 1.0, capacity=7)) == 7


def test_dropless_rows_and_workspace():
    # padded: E*C rows; dropless: S*k compact rows whatever capacity_factor says
    pad = moe.config(1000, 256, 512, 16, 2, 1.0)
    assert moe.dispatch_rows(pad) == 16 * 125
    for cf in (0.0, 1.0, 7.5):
        free = moe.config(1000, 256, 512, 16, 2, cf, dropless=True)
        assert free.dropless and moe.dispatch_rows(free) == 2000
        assert moe.capacity(free) == 1000      # no expert can receive more than S
    # the dropless workspace is sized by S*k, not by E*S
    many = moe.config(4096, 256, 512, 256, 2, dropless=True)
    assert moe.workspace_bytes(many) < 2 * 4096 * 2 * (256 + 512) * 2
    assert moe.workspace_bytes(many) >= 4096 * 2 * (256 + 512) * 2
    # the size limit applies to the compact rows: E*S*h would overflow 2^31,
    # S*k*h does not
    big = moe.config(65536, 1024, 4096, 256, 2, dropless=True)
    assert moe.workspace_bytes(big) > 0
    assert moe.dispatch_rows(big) == 131072


def _status(fn, *args):
    return fn(*args)


def test_invalid_configs_rejected_on_host():
    lib = moe.library()
    n = ctypes.c_size_t(0)
    bad = [
        moe.config(-1, 64, 64, 8, 2),          # negative S
        moe.config(10, 0, 64, 8, 2),           # d = 0
        moe.config(10, 64, 64, 0, 1),          # E = 0
        moe.config(10, 64, 64, 4, 5),          # k > E
        moe.config(10, 64, 64, 4, 0),          # k = 0
        moe.config(10, 64, 64, 4, 2, capacity_factor=0.0),
        moe.config(10, 64, 64, 4, 2, capacity=-3),
    ]
    c = moe.config(10, 64, 64, 4, 2)
    c.act_dtype = 7
    bad.append(c)
    c = moe.config(10, 64, 64, 4, 2)
    c.flags = 4                            # unknown config flag
    bad.append(c)
    bad.append(moe.config(10, 64, 64, 4, 2, capacity=3, dropless=True))
    bad.append(moe.config(10, 64, 64, 4, 2, dropless=True, reroute=True))
    for cfg in bad:
        assert lib.moe_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)) == 1
        assert lib.moe_capacity(ctypes.byref(cfg)) == -1
        assert lib.moe_dispatch_rows(ctypes.byref(cfg)) == -1
    assert lib.moe_workspace_bytes(None, ctypes.byref(n)) == 1


def test_unsupported_shapes_rejected_on_host():
    lib = moe.library()
    n = ctypes.c_size_t(0)
    for cfg in [moe.config(10, 96, 128, 4, 2, dtype="bf16"),    # d not a multiple of 64
                moe.config(10, 64, 100, 4, 2, dtype="bf16"),    # h not a multiple of 64
                moe.config(10, 66, 64, 4, 2, dtype="f32"),      # d not a multiple of 4
                moe.config(10, 64, 64, 4096, 2),                # E > 2048
                moe.config(10, 64, 64, 16, 9),                  # k > 8
                # one expert matrix of 4 GiB or more: its byte offsets are 32-bit
                moe.config(1, 65536, 32768, 1, 1, capacity=1, dtype="bf16"),
                moe.config(1, 32768, 32768, 1, 1, capacity=1, dtype="f32")]:
        assert lib.moe_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)) == 2
    # just under the limit: supported
    ok = moe.config(1, 65536, 32704, 1, 1, capacity=1, dtype="bf16")
    assert lib.moe_workspace_bytes(ctypes.byref(ok), ctypes.byref(n)) == 0


def test_workspace_size_and_errors_before_launch():
    lib = moe.library()
    cfg = moe.config(1000, 256, 512, 16, 2, 1.0)
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)) == 0
    C = moe.capacity(cfg)
    assert C == 125
    # at least H [E,C,h] + one [E,C,d] buffer in bf16
    assert n.value >= 16 * C * (512 + 256) * 2
    assert lib.moe_workspace_bytes(ctypes.byref(cfg), None) == 1
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation
    vp = lambda: fake
    # required pointer missing -> INVALID_ARG
    st = lib.moe_layer_forward(ctypes.byref(cfg), None, vp(), None, vp(), None, vp(), None, vp(),
                               None, None, None, None, None, None, None, None, None, vp(),
                               n.value, None, None)
    assert st == 1
    # workspace too small -> WORKSPACE
    st = lib.moe_layer_forward(ctypes.byref(cfg), vp(), vp(), None, vp(), None, vp(), None, vp(),
                               None, None, None, None, None, None, None, None, None, vp(),
                               n.value - 1, None, None)
    assert st == 3
    # misaligned activation pointer -> INVALID_ARG
    st = lib.moe_dispatch(ctypes.byref(cfg), ctypes.c_void_p((1 << 20) + 2), vp(), vp(), vp(),
                          None)
    assert st == 1
    # router weight not 16-byte aligned -> INVALID_ARG (gate and whole layer)
    odd = ctypes.c_void_p((1 << 20) + 4)
    st = lib.moe_gate(ctypes.byref(cfg), vp(), odd, None, None, vp(), vp(), vp(), vp(), vp(),
                      0, vp(), n.value, None)
    assert st == 1
    st = lib.moe_layer_forward(ctypes.byref(cfg), vp(), odd, None, vp(), None, vp(), None, vp(),
                               None, None, None, None, None, None, None, None, None, vp(),
                               n.value, None, None)
    assert st == 1
    # unknown gate flag -> INVALID_ARG
    st = lib.moe_gate(ctypes.byref(cfg), vp(), vp(), None, None, vp(), vp(), vp(), vp(), vp(),
                      2, vp(), n.value, None)
    assert st == 1
    for s in range(5):
        assert lib.moe_status_string(s).startswith(b"MOE_")


def test_binding_rejects_host_tensors():
    import torch
    cfg = moe.config(4, 64, 64, 2, 1, 1.0, dtype="f32")
    x = torch.zeros(4, 64)
    with pytest.raises(ValueError):
        moe.dispatch(cfg, x, torch.zeros(4, 1, dtype=torch.int32),
                     torch.zeros(4, 1, dtype=torch.int32), torch.zeros(2, 2, 64))
    assert _lib.MOE_NUM_STAGE_EVENTS == 9


def test_backward_validation_on_host():
    lib = moe.library()
    n = ctypes.c_size_t(0)
    # bf16 only; fp32 activations are valid but not supported by the backward
    f32 = moe.config(100, 64, 64, 4, 2, dtype="f32")
    assert lib.moe_backward_workspace_bytes(ctypes.byref(f32), ctypes.byref(n)) == 2
    cfg = moe.config(1000, 256, 512, 16, 2, 1.0)
    assert lib.moe_backward_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)) == 0
    # at least H [R,h] and one [R,d] buffer in bf16 with R = E*C rows
    assert n.value >= 16 * 125 * (512 + 256) * 2
    need = n.value
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation
    f = ctypes.c_float

    def call(ws_bytes=need, g_aux=0.0, drop=None, dw_gate=fake, w_gate=fake):
        args = [fake] * 13
        args[1] = w_gate
        args[11] = None                                  # hidden: optional
        if drop is not None:
            args[drop] = None
        return lib.moe_layer_backward(ctypes.byref(cfg), *args, f(g_aux), f(0.0), fake, dw_gate,
                                      None, fake, None, fake, None, fake, ws_bytes, None, None)
    assert call(ws_bytes=need - 1) == 3                 # workspace too small
    assert call(dw_gate=ctypes.c_void_p((1 << 20) + 4)) == 1   # dw_gate not 16-byte aligned
    assert call(w_gate=ctypes.c_void_p((1 << 20) + 4)) == 1    # w_gate not 16-byte aligned
    assert call(drop=12) == 1                           # dy missing
    assert call(drop=10) == 1                           # forward expert outputs missing
    assert call(g_aux=float("nan")) == 1                # loss weight not finite
    assert moe.backward_workspace_bytes(moe.config(2000, 128, 256, 8, 2, dropless=True)) > 0


def test_stale_library_is_rebuilt(tmp_path, monkeypatch):
    """library() builds again when the sources differ from those the loaded
    library was built from (the digest stored beside it), and loads it
    without a build when they match."""
    import shutil
    from sparse_moe_layer_wg_amd import _build
    src = tmp_path / "csrc"
    inc = tmp_path / "include"
    shutil.copytree(_build.CSRC, src)
    shutil.copytree(_build.INCLUDE, inc)
    lib = tmp_path / "libmoe.so"
    lib.write_bytes(b"")
    stamp = tmp_path / "libmoe.so.srcsha"
    paths = _build.sources(str(src), str(inc))
    stamp.write_text(_build.source_digest(paths) + "\n")
    assert _build.is_current(str(lib), str(stamp), paths)
    # the digest covers every source file, headers included
    one = src / "permute.hip"
    one.write_text(one.read_text() + "\n// edited\n")
    assert not _build.is_current(str(lib), str(stamp), paths)
    (inc / "moe.h").write_text((inc / "moe.h").read_text())   # unchanged content
    stamp.write_text(_build.source_digest(paths) + "\n")
    assert _build.is_current(str(lib), str(stamp), paths)
    (inc / "moe.h").write_text((inc / "moe.h").read_text() + " ")
    assert not _build.is_current(str(lib), str(stamp), paths)
    assert not _build.is_current(str(tmp_path / "missing.so"), str(stamp), paths)

    # library() itself: a stale stamp triggers exactly one build
    calls = []
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_build, "is_current",
                        lambda *a, **k: len(calls) > 0)
    monkeypatch.setattr(_build, "build", lambda *a, **k: calls.append(1))
    monkeypatch.setattr(_lib.ctypes, "CDLL", lambda path: (_ for _ in ()).throw(
        RuntimeError("loaded")))
    with pytest.raises(RuntimeError, match="loaded"):
        _lib.library()
    assert calls == [1]


def test_noalloc_gate_refuses_shapes_beyond_the_static_scratch():
    """moe_gate_noalloc refuses, on the host and before anything is enqueued,
    a valid shape whose router scratch exceeds MOE_STATIC_SCRATCH_BYTES
    (here 64 MiB of logits alone); bad arguments fail as in moe_gate."""
    lib = moe.library()
    fake = ctypes.c_void_p(1 << 20)     # never dereferenced
    big = moe.config(262144, 64, 64, 64, 2, 1.0, dtype="bf16")
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_bytes(ctypes.byref(big), ctypes.byref(n)) == 0
    assert n.value > moe.MOE_STATIC_SCRATCH_BYTES
    for logits in (None, fake):
        st = lib.moe_gate_noalloc(ctypes.byref(big), fake, fake, None, logits, fake, fake, fake,
                                  fake, fake, 0, None)
        assert st == 5
    assert b"SCRATCH_LIMIT" in lib.moe_status_string(5)
    # argument checks come first, as in moe_gate
    small = moe.config(100, 64, 64, 8, 2, 1.0, dtype="bf16")
    assert lib.moe_gate_noalloc(ctypes.byref(small), fake, fake, None, None, fake, fake, fake,
                                None, fake, 0, None) == 1        # counts missing
    assert lib.moe_gate_noalloc(ctypes.byref(small), fake, fake, None, None, fake, fake, fake,
                                fake, fake, 8, None) == 1        # unknown flag
