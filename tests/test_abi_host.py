"""Host-side checks of the C ABI: the library loads, exports every symbol
include/tts.h declares, and validates configs without touching a GPU."""
import ctypes
import os
import re

import pytest

from autoregressive_tts_decode_amd import config, tts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tts.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tts_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = tts.load_library()
    names = declared_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(tts.EXPORTED)


def test_nm_shows_c_linkage():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", tts.LIB_PATH], capture_output=True, text=True).stdout
    for n in declared_functions():
        assert re.search(rf"\bT {n}$", out, re.M), n


def _cfg(**over):
    c = tts.config_struct(config.M17B, 1, 320, 240)
    for k, v in over.items():
        setattr(c, k, v)
    return c


def test_workspace_bytes_for_the_workloads():
    for name, wl in config.WORKLOADS.items():
        n = tts.workspace_bytes(wl.model, wl.batch, wl.prefill_len + wl.frames, wl.frames)
        assert n > 0
    # KV cache dominates at long context: 28 layers x 2 x 8 heads x 2256 x 128 x 2 B
    long_wl = config.WORKLOADS["1.7b-long"]
    n = tts.workspace_bytes(long_wl.model, 1, 2256, 2000)
    assert n >= 28 * 2 * 8 * 2256 * 128 * 2


@pytest.mark.parametrize("field,value", [
    ("n_acoustic", 14), ("max_batch", 0), ("max_batch", 65), ("max_cache_steps", 1), ("max_frames", 0),
    ("weight_dtype", 7), ("rms_eps", 0.0), ("rope_theta", 1.0), ("text_vocab", 0),
])
def test_workspace_bytes_rejects_bad_configs(field, value):
    lib = tts.load_library()
    c = _cfg(**{field: value})
    n = ctypes.c_size_t(0)
    assert lib.tts_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == tts.TTS_E_SHAPE


def test_workspace_bytes_fp8_needs_1024_multiples():
    """E4M3 matrices are read 16 per 16-byte lane load, so every contraction width must be a
    multiple of 1024 (64 lanes x 16): the 1.7B shapes pass, the tiny model's 256 does not."""
    lib = tts.load_library()
    n = ctypes.c_size_t(0)
    ok = tts.config_struct(config.MODELS["1.7b-fp8"], 1, 512, 64)
    assert lib.tts_workspace_bytes(ctypes.byref(ok), ctypes.byref(n)) == tts.TTS_OK and n.value > 0
    tiny = config.ModelCfg(name="tiny-fp8", talker=config.TINY.talker, codepred=config.TINY.codepred,
                           text_vocab=config.TINY.text_vocab, weight_dtype="fp8")
    bad = tts.config_struct(tiny, 1, 64, 8)
    assert lib.tts_workspace_bytes(ctypes.byref(bad), ctypes.byref(n)) == tts.TTS_E_SHAPE


def test_workspace_bytes_rejects_unsupported_stack_shapes():
    lib = tts.load_library()
    n = ctypes.c_size_t(0)
    for sub, field, value in [("talker", "head_dim", 96), ("codepred", "n_kv_heads", 3), ("talker", "hidden", 1000),
                              ("codepred", "ffn", 5 * 512), ("talker", "n_q_heads", 48)]:
        c = _cfg()
        setattr(getattr(c, sub), field, value)
        assert lib.tts_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == tts.TTS_E_SHAPE, (sub, field)


def test_null_arguments():
    lib = tts.load_library()
    n = ctypes.c_size_t(0)
    assert lib.tts_workspace_bytes(None, ctypes.byref(n)) == tts.TTS_E_ARG
    c = _cfg()
    assert lib.tts_workspace_bytes(ctypes.byref(c), None) == tts.TTS_E_ARG
    out = ctypes.c_void_p()
    assert lib.tts_create(ctypes.byref(c), None, None, 0, ctypes.byref(out)) == tts.TTS_E_ARG
    assert out.value is None
    assert lib.tts_create(ctypes.byref(c), None, ctypes.c_void_p(256), 0, None) == tts.TTS_E_ARG
    assert lib.tts_last_error(None) == b"context is NULL"
    lib.tts_destroy(None)
    for fn in ("tts_reset",):
        assert getattr(lib, fn)(None) == tts.TTS_E_ARG
    assert lib.tts_prefill(None, None, 1, 1, None) == tts.TTS_E_ARG
    assert lib.tts_talker_step(None, None, None) == tts.TTS_E_ARG
    assert lib.tts_run_frames(None, 1, None, None, None, None) == tts.TTS_E_ARG
    assert lib.tts_get_progress(None, None, None) == tts.TTS_E_ARG


def test_create_rejects_small_or_misaligned_workspace_before_touching_the_device():
    lib = tts.load_library()
    c = _cfg()
    out = ctypes.c_void_p()
    need = tts.workspace_bytes(config.M17B, 1, 320, 240)
    # misaligned pointer -> TTS_E_ARG; too small -> TTS_E_CAPACITY (no device access happens first)
    assert lib.tts_create(ctypes.byref(c), None, ctypes.c_void_p(4096 + 8), need, ctypes.byref(out)) == tts.TTS_E_ARG
    assert lib.tts_create(ctypes.byref(c), None, ctypes.c_void_p(4096), need - 1, ctypes.byref(out)) == tts.TTS_E_CAPACITY
    assert out.value is None


def test_measured_traffic_record_follows_the_kernel_sources(tmp_path, monkeypatch):
    """The bench's HBM traffic comes from a committed counter record and is dropped (None) as soon
    as the kernel's sources no longer hash to the recorded value."""
    from autoregressive_tts_decode_amd import roofline
    h = roofline.kernel_source_sha256()
    assert len(h) == 64 and int(h, 16) >= 0
    monkeypatch.setattr(roofline, "_PROFILES", str(tmp_path))
    assert roofline.measured_traffic("absent.md") is None
    (tmp_path / "ok.md").write_text(f"text\n    kernel_source_sha256: {h}\n    traffic_bytes_per_launch: 12345\n")
    assert roofline.measured_traffic("ok.md") == 12345
    (tmp_path / "stale.md").write_text("    kernel_source_sha256: " + "0" * 64 + "\n    traffic_bytes_per_launch: 12345\n")
    assert roofline.measured_traffic("stale.md") is None


@pytest.mark.parametrize("arch,cus,xccs,cp,tk,want", [
    ("gfx950:sramecc+:xnack-", 256, 8, 1, 1, tts.PERSISTENT_CODEPRED | tts.PERSISTENT_TALKER),
    ("gfx950", 256, 8, 1, 0, tts.PERSISTENT_CODEPRED),
    ("gfx950", 256, 8, 0, 2, tts.PERSISTENT_TALKER),
    ("gfx950", 256, 8, 0, 0, 0),
    ("gfx950:sramecc+", 128, 4, 1, 1, 0),      # a partition of the device: fewer CUs and XCDs
    ("gfx950", 256, 1, 1, 1, 0),               # one XCD reported
    ("gfx950", 304, 8, 1, 1, 0),               # another CU count
    ("gfx942:sramecc+:xnack-", 256, 8, 1, 1, 0),
    ("gfx9500", 256, 8, 1, 1, 0),
    ("", 256, 8, 1, 1, 0),
])
def test_persistent_kernels_are_gated_on_the_device(arch, cus, xccs, cp, tk, want):
    """The persistent kernels run only where all 256 of their workgroups can be resident at once,
    32 on each of 8 XCDs of a gfx950, with room for one of their workgroups per CU."""
    assert tts.persistent_allowed(arch, cus, xccs, cp, tk) == want


def test_persistent_gate_rejects_null():
    assert tts.load_library().tts_persistent_allowed(None) == 0


def test_bf16_kv_cache_is_refused():
    """The KV caches stay fp32 (a bf16 cache alone puts the 1.7B acoustic logits over the 1e-2 bar)."""
    lib = tts.load_library()
    n = ctypes.c_size_t(0)
    c = _cfg(kv_dtype=tts.DTYPE_BF16)
    assert lib.tts_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == tts.TTS_E_SHAPE
    c = _cfg(kv_dtype=tts.DTYPE_F32)
    assert lib.tts_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == tts.TTS_OK
