"""The C ABI without a GPU: the library loads, exports every function that
include/fsq.h declares, and rejects invalid arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import fsq_latent_decode_amd as fsq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fsq.h")

needs_lib = pytest.mark.skipif(not os.path.exists(fsq.library_path()),
                               reason="libfsq.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fsq_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(fsq.EXPORTS)


def test_header_compiles_as_c(tmp_path):
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "t.c"
    src.write_text('#include "fsq.h"\nint main(void){return FSQ_OK;}\n')
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), "-c",
                        str(src), "-o", str(tmp_path / "t.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@needs_lib
def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(fsq.library_path())
    for name in declared_functions():
        assert hasattr(L, name), name


@needs_lib
def test_status_strings():
    assert fsq.status_string(0) == "FSQ_OK"
    assert fsq.status_string(fsq.FSQ_ERR_WORKSPACE) == "FSQ_ERR_WORKSPACE"
    assert fsq.status_string(99) == "FSQ_UNKNOWN"


@needs_lib
def test_workspace_bytes_host_logic():
    L = fsq.lib()
    assert L.fsq_decode_workspace_bytes(0, 32, 256, 10) == 0
    assert L.fsq_decode_workspace_bytes(1, 65, 256, 10) == 0
    assert L.fsq_decode_workspace_bytes(1, 32, 257, 10) == 0
    assert L.fsq_decode_workspace_bytes(1, 32, 256, -1) == 0
    small = L.fsq_decode_workspace_bytes(1, 32, 256, 1024)
    big = L.fsq_decode_workspace_bytes(1, 32, 256, 32768)
    assert 0 < small <= big
    # holds at least the absorbed queries (fp16) and one split of partials (fp32)
    assert small >= 32 * 256 * 2 + 32 * 256 * 4 + 32 * 2 * 4
    assert L.fsq_decode_workspace_bytes(1, 32, 84, 0) > 0
    assert L.fsq_decode_workspace_bytes(1, 32, 84, 1 << 20) % 256 == 0


@needs_lib
@pytest.mark.parametrize("args,status", [
    # (q, codes, W, lens, out, batch, n_q, n_kv, d_h, G, cap, ws, ws_bytes)
    ((1, 1, 1, 1, 1, 0, 32, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_SHAPE),
    ((1, 1, 1, 1, 1, 1, 32, 6, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_SHAPE),
    ((1, 1, 1, 1, 1, 1, 32, 8, 128, 256, -1, 256, 1 << 20), fsq.FSQ_ERR_SHAPE),
    ((1, 1, 1, 1, 1, 1, 32, 8, 512, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_UNSUPPORTED),
    ((1, 1, 1, 1, 1, 1, 32, 8, 128, 300, 16, 256, 1 << 20), fsq.FSQ_ERR_UNSUPPORTED),
    ((1, 1, 1, 1, 1, 1, 128, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_UNSUPPORTED),
    ((0, 256, 256, 256, 256, 1, 32, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_NULL),
    ((256, 0, 256, 256, 256, 1, 32, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_NULL),
    ((256, 8, 256, 256, 256, 1, 32, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_UNSUPPORTED),
    ((256, 256, 256, 256, 256, 1, 32, 8, 128, 256, 16, 0, 1 << 20), fsq.FSQ_ERR_WORKSPACE),
    ((256, 256, 256, 256, 256, 1, 32, 8, 128, 256, 16, 256, 64), fsq.FSQ_ERR_WORKSPACE),
    ((256, 256, 256, 256, 256, 1, 32, 8, 128, 256, 16, 128, 1 << 20), fsq.FSQ_ERR_WORKSPACE),
])
def test_decode_validation_before_any_hip_call(args, status):
    # pointer values are never dereferenced: every case fails validation first
    (q, c, w, l, o, B, nq, nkv, dh, G, cap, ws, wsb) = args
    rc = fsq.lib().fsq_decode_attn(q, c, w, l, o, B, nq, nkv, dh, G, cap, ws, wsb, None)
    assert rc == status


@needs_lib
@pytest.mark.parametrize("args,status", [
    ((256, 256, 256, -1, 64, 8), fsq.FSQ_ERR_SHAPE),
    ((256, 256, 256, 4, 0, 8), fsq.FSQ_ERR_SHAPE),
    ((256, 256, 256, 4, 64, 0), fsq.FSQ_ERR_SHAPE),
    ((256, 256, 256, 4, 60, 8), fsq.FSQ_ERR_UNSUPPORTED),
    ((256, 256, 256, 4, 64, 257), fsq.FSQ_ERR_UNSUPPORTED),
    ((0, 256, 256, 4, 64, 8), fsq.FSQ_ERR_NULL),
    ((256, 256, 0, 4, 64, 8), fsq.FSQ_ERR_NULL),
    ((264, 256, 256, 4, 64, 8), fsq.FSQ_ERR_UNSUPPORTED),
    ((0, 0, 0, 0, 64, 8), fsq.FSQ_OK),
])
def test_append_validation_before_any_hip_call(args, status):
    x, E, c, n, C, G = args
    assert fsq.lib().fsq_append(x, E, c, n, C, G, None) == status


@needs_lib
@pytest.mark.parametrize("args,status", [
    # (x_new, E, q, codes, W, lens, out, batch, C, n_q, n_kv, d_h, G, cap, ws, ws_bytes)
    ((256, 256, 256, 256, 256, 256, 256, 1, 0, 32, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_SHAPE),
    ((256, 256, 256, 256, 256, 256, 256, 1, 60, 32, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_UNSUPPORTED),
    ((0, 256, 256, 256, 256, 256, 256, 1, 64, 32, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_NULL),
    ((256, 0, 256, 256, 256, 256, 256, 1, 64, 32, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_NULL),
    ((264, 256, 256, 256, 256, 256, 256, 1, 64, 32, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_UNSUPPORTED),
    ((256, 264, 256, 256, 256, 256, 256, 1, 64, 32, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_UNSUPPORTED),
    # the decode checks apply as well
    ((256, 256, 256, 256, 256, 256, 256, 0, 64, 32, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_SHAPE),
    ((256, 256, 256, 256, 256, 256, 256, 1, 64, 32, 6, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_SHAPE),
    ((256, 256, 256, 256, 256, 256, 256, 1, 64, 32, 8, 128, 300, 16, 256, 1 << 20), fsq.FSQ_ERR_UNSUPPORTED),
    ((256, 256, 256, 0, 256, 256, 256, 1, 64, 32, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_NULL),
    ((256, 256, 256, 8, 256, 256, 256, 1, 64, 32, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_UNSUPPORTED),
    ((256, 256, 256, 256, 256, 256, 256, 1, 64, 32, 8, 128, 256, 16, 256, 64), fsq.FSQ_ERR_WORKSPACE),
    ((256, 256, 256, 256, 256, 256, 256, 1, 64, 32, 8, 128, 256, 16, 0, 1 << 20), fsq.FSQ_ERR_WORKSPACE),
])
def test_decode_step_validation_before_any_hip_call(args, status):
    (x, E, q, c, w, l, o, B, C, nq, nkv, dh, G, cap, ws, wsb) = args
    rc = fsq.lib().fsq_decode_step(x, E, q, c, w, l, o, B, C, nq, nkv, dh, G, cap, ws, wsb, None)
    assert rc == status


@needs_lib
@pytest.mark.parametrize("levels,C,G,status", [
    (8, 64, 256, "FSQ_ERR_UNSUPPORTED"),    # not 4, 16 or 256 levels
    (3, 64, 84, "FSQ_ERR_UNSUPPORTED"),
    (4, 60, 84, "FSQ_ERR_UNSUPPORTED"),     # C % 8 != 0, as for the 4-bit step
    (256, 0, 42, "FSQ_ERR_SHAPE"),
    (4, 64, 300, "FSQ_ERR_UNSUPPORTED"),    # G > FSQ_MAX_G
])
def test_decode_step_levels_validation_before_any_hip_call(levels, C, G, status):
    rc = fsq.lib().fsq_decode_step_levels(256, 256, 256, 256, 256, 256, 256, 1, C, 32, 8, 128, G, levels,
                                          16, 256, 1 << 20, None)
    assert rc == getattr(fsq, status)


@needs_lib
@pytest.mark.parametrize("args,status", [
    # (q, codes, W, lens, out, batch, n_q, n_kv, d_h, G, cap, ws, ws_bytes)
    ((256, 256, 256, 256, 256, 0, 32, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_SHAPE),
    ((256, 256, 256, 256, 256, 1, 32, 6, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_SHAPE),
    ((256, 256, 256, 256, 256, 1, 32, 8, 80, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_UNSUPPORTED),   # d_h % 32
    ((256, 256, 256, 256, 256, 1, 32, 8, 256, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_UNSUPPORTED),  # d_h > 128
    ((256, 256, 256, 256, 256, 1, 64, 1, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_UNSUPPORTED),  # 64 heads per kv head
    ((256, 256, 256, 256, 256, 1, 32, 8, 128, 300, 16, 256, 1 << 20), fsq.FSQ_ERR_UNSUPPORTED),
    ((0, 256, 256, 256, 256, 1, 32, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_NULL),
    ((256, 8, 256, 256, 256, 1, 32, 8, 128, 256, 16, 256, 1 << 20), fsq.FSQ_ERR_UNSUPPORTED),
    ((256, 256, 256, 256, 256, 1, 32, 8, 128, 256, 16, 256, 64), fsq.FSQ_ERR_WORKSPACE),
    ((256, 256, 256, 256, 256, 1, 32, 8, 128, 256, 16, 0, 1 << 20), fsq.FSQ_ERR_WORKSPACE),
])
def test_decode_recon_validation_before_any_hip_call(args, status):
    (q, c, w, l, o, B, nq, nkv, dh, G, cap, ws, wsb) = args
    rc = fsq.lib().fsq_decode_attn_recon(q, c, w, l, o, B, nq, nkv, dh, G, cap, ws, wsb, None)
    assert rc == status


@needs_lib
@pytest.mark.parametrize("args,status", [
    # (q, codes, W, k_norm, lens, out, batch, n_q, n_kv, d_h, G, cap, theta, eps, ws, ws_bytes)
    ((256, 256, 256, 256, 256, 256, 1, 32, 8, 96, 256, 16, 1e6, 1e-6, 256, 1 << 20), fsq.FSQ_ERR_UNSUPPORTED),
    ((256, 256, 256, 256, 256, 256, 1, 32, 8, 32, 256, 16, 1e6, 1e-6, 256, 1 << 20), fsq.FSQ_ERR_UNSUPPORTED),
    ((256, 256, 256, 0, 256, 256, 1, 32, 8, 128, 256, 16, 1e6, 1e-6, 256, 1 << 20), fsq.FSQ_ERR_NULL),
    ((256, 256, 256, 256, 256, 256, 1, 32, 8, 128, 256, 16, 0.5, 1e-6, 256, 1 << 20), fsq.FSQ_ERR_SHAPE),
    ((256, 256, 256, 256, 256, 256, 1, 32, 8, 128, 256, 16, 1e6, -1.0, 256, 1 << 20), fsq.FSQ_ERR_SHAPE),
    ((256, 256, 256, 256, 256, 256, 1, 32, 8, 128, 256, 16, float("nan"), 1e-6, 256, 1 << 20), fsq.FSQ_ERR_SHAPE),
    ((256, 256, 256, 256, 256, 256, 0, 32, 8, 128, 256, 16, 1e6, 1e-6, 256, 1 << 20), fsq.FSQ_ERR_SHAPE),
    ((256, 256, 256, 256, 256, 256, 1, 32, 8, 128, 256, 16, 1e6, 1e-6, 256, 64), fsq.FSQ_ERR_WORKSPACE),
])
def test_decode_rope_validation_before_any_hip_call(args, status):
    (q, c, w, k, l, o, B, nq, nkv, dh, G, cap, th, ep, ws, wsb) = args
    rc = fsq.lib().fsq_decode_attn_rope(q, c, w, k, l, o, B, nq, nkv, dh, G, cap, th, ep, ws, wsb, None)
    assert rc == status


@needs_lib
@pytest.mark.parametrize("levels,status", [(8, fsq.FSQ_ERR_UNSUPPORTED), (2, fsq.FSQ_ERR_UNSUPPORTED),
                                           (0, fsq.FSQ_ERR_UNSUPPORTED)])
def test_levels_validation_before_any_hip_call(levels, status):
    assert fsq.lib().fsq_append_levels(256, 256, 256, 4, 64, 8, levels, None) == status
    rc = fsq.lib().fsq_decode_attn_levels(256, 256, 256, 256, 256, 1, 32, 8, 128, 256, levels, 16, 256,
                                          1 << 20, None)
    assert rc == status


@needs_lib
def test_timed_entry_points_need_both_events():
    # the event-timed forms reject a NULL event before any HIP call
    for ev in [(None, 256), (256, None)]:
        assert fsq.lib().fsq_decode_attn_timed(256, 256, 256, 256, 256, 1, 32, 8, 128, 256, 16, 256,
                                               1 << 20, None, *ev) == fsq.FSQ_ERR_NULL
        assert fsq.lib().fsq_decode_attn_levels_timed(256, 256, 256, 256, 256, 1, 32, 8, 128, 256, 4, 16,
                                                      256, 1 << 20, None, *ev) == fsq.FSQ_ERR_NULL
    # and otherwise validate as the untimed forms
    assert fsq.lib().fsq_decode_attn_levels_timed(256, 256, 256, 256, 256, 1, 32, 8, 128, 256, 5, 16,
                                                  256, 1 << 20, None, 256, 256) == fsq.FSQ_ERR_UNSUPPORTED


@needs_lib
def test_levels_workspace_is_the_default_one():
    # the 2- and 8-bit decode needs no more workspace than fsq_decode_workspace_bytes
    ok = fsq.lib().fsq_decode_attn_levels(256, 256, 256, 256, 256, 1, 32, 8, 128, 84, 4, 1 << 20, 256,
                                          64, None)
    assert ok == fsq.FSQ_ERR_WORKSPACE


@needs_lib
def test_decode_plan_host_logic():
    # short caches: the round-synchronous split kernel; long ones: the streaming kernel
    assert fsq.decode_plan(1, 32, 256, 32768)["kernel"] == "decode_split_kernel"
    assert fsq.decode_plan(1, 32, 84, 131072)["kernel"] == "decode_split_kernel"
    assert fsq.decode_plan(1, 32, 84, 1 << 20)["kernel"] == "decode_stream_kernel"
    assert fsq.decode_plan(16, 16, 256, 65536)["kernel"] == "decode_stream_kernel"
    for args in [(1, 32, 256, 1), (1, 32, 84, 1 << 20), (16, 16, 256, 65536), (3, 12, 37, 5000),
                 (65, 16, 256, 65536)]:
        p = fsq.decode_plan(*args)
        if p["device_split"]:   # the chunk is also >= sum of lengths / CTAs: at most that many items
            ncta = 256 if (args[2] + 31) // 32 * 32 < 128 else 512
            assert p["splits"] == min(-(-args[3] // p["chunk"]), ncta)
        else:
            assert p["splits"] * p["chunk"] >= args[3] > (p["splits"] - 1) * p["chunk"]
        assert p["splits"] <= 1024 and p["chunk"] % 128 == 0
    # streaming calls of up to 64 sequences split on the device from the actual
    # lengths: the plan then gives the smallest chunk (4 rounds of the CTA's
    # waves x 32 tokens: 4 waves at width 256, 8 below 128; and at least
    # seq_cap / 1024) and the largest split count (at most one per CTA)
    p = fsq.decode_plan(16, 16, 256, 65536)
    assert p["device_split"] and p["chunk"] == 512 and p["splits"] == 128
    p = fsq.decode_plan(1, 32, 84, 1 << 20)
    assert p["device_split"] and p["chunk"] == 1024 and p["splits"] == 256
    assert not fsq.decode_plan(65, 16, 256, 65536)["device_split"]
    assert fsq.decode_plan(65, 16, 256, 65536)["kernel"] == "decode_stream_kernel"
    assert not fsq.decode_plan(1, 32, 256, 32768)["device_split"]
    # widths 64 and 96: 8-wave split CTAs (256-token rounds, about 256 CTAs)
    # once the work reaches 2 x 256 x 256 tokens, 4-wave CTAs (about 512) below
    p = fsq.decode_plan(1, 32, 84, 131072)
    assert p["kernel"] == "decode_split_kernel" and p["chunk"] == 512 and p["splits"] == 256
    p = fsq.decode_plan(1, 32, 84, 65536)
    assert p["chunk"] == 128 and p["splits"] == 512
    p = fsq.decode_plan(1, 32, 32, 131072)
    assert p["chunk"] == 256 and p["splits"] == 512
    p = fsq.decode_plan(1, 32, 256, 32768)
    assert p["chunk"] == 256 and p["splits"] == 128
    assert fsq.decode_plan(1, 32, 256, 0)["splits"] == 0
    with pytest.raises(fsq.FsqError):
        fsq.decode_plan(0, 32, 256, 10)


def test_binding_raises_without_library(monkeypatch):
    monkeypatch.setattr(fsq, "_lib", None)
    monkeypatch.setattr(fsq, "_LIB_PATH", "/nonexistent/libfsq.so")
    with pytest.raises(RuntimeError, match="missing"):
        fsq.lib()
