"""Thin ctypes binding of libtts.so (the C ABI of include/tts.h).

Argument marshalling only: every step of the decode runs in the library's HIP
kernels. PyTorch provides device memory (weights, workspace, inputs and
outputs) and the stream; pointers are passed through as integers.

The library must be built first (``python -m autoregressive_tts_decode_amd.build``);
loading fails loudly when it is missing -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

from .config import ModelCfg, SamplingCfg, StackCfg, N_ACOUSTIC, tensor_specs, scale_specs

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtts.so")

TTS_OK = 0
TTS_E_ARG = -1
TTS_E_SHAPE = -2
TTS_E_CAPACITY = -3
TTS_E_STATE = -4
TTS_E_HIP = -5
TTS_E_UNSUPPORTED = -6
TTS_E_DEVICE = -7
STATUS_NAMES = {0: "TTS_OK", -1: "TTS_E_ARG", -2: "TTS_E_SHAPE", -3: "TTS_E_CAPACITY", -4: "TTS_E_STATE",
                -5: "TTS_E_HIP", -6: "TTS_E_UNSUPPORTED", -7: "TTS_E_DEVICE"}
DTYPE_F32, DTYPE_BF16, DTYPE_FP8_E4M3 = 0, 1, 2
_WEIGHT_DTYPE = {"fp32": DTYPE_F32, "bf16": DTYPE_BF16, "fp8": DTYPE_FP8_E4M3}

EXPORTED = ["tts_workspace_bytes", "tts_create", "tts_load_weights", "tts_prefill", "tts_talker_step",
            "tts_talker_step_text", "tts_set_text_stream", "tts_prefill_ragged", "tts_set_stop", "tts_codepred_frame", "tts_sample", "tts_run_frames", "tts_run_frames_noalloc", "tts_set_exec_mode", "tts_get_exec_mode", "tts_set_prefill_mode", "tts_get_prefill_mode",
            "tts_device_status", "tts_persistent_allowed", "tts_get_progress", "tts_reset", "tts_last_error",
            "tts_destroy"]
EXEC_KERNELS, EXEC_PERSISTENT = 0, 1
PERSISTENT_CODEPRED, PERSISTENT_TALKER = 1, 2  # bits of exec_mode()[1]
PREFILL_STEPS, PREFILL_GEMM = 0, 1


class StackCfgC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "vocab")]


class ConfigC(ctypes.Structure):
    _fields_ = [("talker", StackCfgC), ("codepred", StackCfgC), ("text_vocab", ctypes.c_int32),
                ("n_acoustic", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("weight_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_cache_steps", ctypes.c_int32), ("max_frames", ctypes.c_int32)]


class DeviceDescC(ctypes.Structure):
    _fields_ = [("arch", ctypes.c_char * 64), ("compute_units", ctypes.c_int32), ("xccs", ctypes.c_int32),
                ("codepred_wg_per_cu", ctypes.c_int32), ("talker_wg_per_cu", ctypes.c_int32)]


class SamplingC(ctypes.Structure):
    _fields_ = [("do_sample", ctypes.c_int32), ("top_k", ctypes.c_int32), ("top_p", ctypes.c_float),
                ("temperature", ctypes.c_float), ("repetition_penalty", ctypes.c_float)]


class TTSError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libtts.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libtts.so not found at {path}; build it with "
                           "`python -m autoregressive_tts_decode_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.tts_workspace_bytes.argtypes = [ctypes.POINTER(ConfigC), ctypes.POINTER(SZ)]
    lib.tts_create.argtypes = [ctypes.POINTER(ConfigC), P, P, SZ, ctypes.POINTER(P)]
    lib.tts_load_weights.argtypes = [P, I32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(P),
                                     ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(I32), ctypes.POINTER(I32)]
    lib.tts_prefill.argtypes = [P, P, I32, I32, P]
    lib.tts_talker_step.argtypes = [P, P, P]
    lib.tts_talker_step_text.argtypes = [P, P, P, P]
    lib.tts_set_text_stream.argtypes = [P, P, I32, I32]
    lib.tts_prefill_ragged.argtypes = [P, P, ctypes.POINTER(I32), I32, I32, P]
    lib.tts_set_stop.argtypes = [P, I32, P]
    lib.tts_codepred_frame.argtypes = [P, P, ctypes.POINTER(SamplingC), P, P, P, P]
    lib.tts_sample.argtypes = [P, P, I32, I32, ctypes.POINTER(SamplingC), P, P, P]
    lib.tts_run_frames.argtypes = [P, I32, ctypes.POINTER(SamplingC), ctypes.POINTER(SamplingC), P, P]
    lib.tts_run_frames_noalloc.argtypes = [P, I32, ctypes.POINTER(SamplingC), ctypes.POINTER(SamplingC), P, P]
    lib.tts_get_progress.argtypes = [P, ctypes.POINTER(I32), ctypes.POINTER(I32)]
    lib.tts_set_exec_mode.argtypes = [P, I32]
    lib.tts_set_prefill_mode.argtypes = [P, I32]
    lib.tts_get_prefill_mode.argtypes = [P, ctypes.POINTER(I32)]
    lib.tts_get_exec_mode.argtypes = [P, ctypes.POINTER(I32), ctypes.POINTER(I32)]
    lib.tts_device_status.argtypes = [P, ctypes.POINTER(I32)]
    lib.tts_persistent_allowed.argtypes = [ctypes.POINTER(DeviceDescC)]
    lib.tts_reset.argtypes = [P]
    lib.tts_last_error.argtypes = [P]
    lib.tts_last_error.restype = ctypes.c_char_p
    lib.tts_destroy.argtypes = [P]
    lib.tts_destroy.restype = None
    for name in EXPORTED:
        if name not in ("tts_last_error", "tts_destroy"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def persistent_allowed(arch: str, compute_units: int, xccs: int, codepred_wg_per_cu: int, talker_wg_per_cu: int) -> int:
    """tts_persistent_allowed on a device description: the PERSISTENT_* bits of the kernels allowed."""
    d = DeviceDescC(arch.encode(), compute_units, xccs, codepred_wg_per_cu, talker_wg_per_cu)
    return int(load_library().tts_persistent_allowed(ctypes.byref(d)))


def config_struct(model: ModelCfg, max_batch: int, max_cache_steps: int, max_frames: int,
                  kv_dtype: str = "fp32") -> ConfigC:
    def sc(s: StackCfg) -> StackCfgC:
        return StackCfgC(s.n_layers, s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn, s.vocab)

    return ConfigC(sc(model.talker), sc(model.codepred), model.text_vocab, model.n_acoustic, model.rms_eps,
                   model.rope_theta, _WEIGHT_DTYPE[model.weight_dtype],
                   DTYPE_BF16 if kv_dtype == "bf16" else DTYPE_F32, max_batch, max_cache_steps, max_frames)


def sampling_struct(s: SamplingCfg | dict) -> SamplingC:
    d = s if isinstance(s, dict) else s.as_dict()
    return SamplingC(int(bool(d["do_sample"])), int(d["top_k"]), float(d["top_p"]), float(d["temperature"]),
                     float(d["repetition_penalty"]))


def workspace_bytes(model: ModelCfg, max_batch: int, max_cache_steps: int, max_frames: int,
                    kv_dtype: str = "fp32") -> int:
    lib = load_library()
    cfg = config_struct(model, max_batch, max_cache_steps, max_frames, kv_dtype)
    n = ctypes.c_size_t(0)
    rc = lib.tts_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n))
    if rc != TTS_OK:
        raise TTSError(rc, "tts_workspace_bytes rejected the config")
    return n.value


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


class TTSDecoder:
    """One decode context on the current device: workspace, weights, streams.

    All tensors passed in are torch CUDA tensors (int32 ids/codes, fp32
    logits/uniforms); they are used in place by the library's kernels.
    """

    def __init__(self, model: ModelCfg, max_batch: int, max_cache_steps: int, max_frames: int,
                 stream=None, device: str = "cuda", kv_dtype: str = "fp32"):
        import torch
        self.torch = torch
        self.lib = load_library()
        self.model = model
        self.max_batch, self.max_cache_steps, self.max_frames = max_batch, max_cache_steps, max_frames
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        self.kv_dtype = kv_dtype
        self.cfg = config_struct(model, max_batch, max_cache_steps, max_frames, kv_dtype)
        nbytes = workspace_bytes(model, max_batch, max_cache_steps, max_frames, kv_dtype)
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        base = self.workspace.data_ptr()
        self._ws_ptr = (base + 255) // 256 * 256
        self.ctx = ctypes.c_void_p()
        rc = self.lib.tts_create(ctypes.byref(self.cfg), ctypes.c_void_p(self.stream.cuda_stream),
                                 ctypes.c_void_p(self._ws_ptr), nbytes, ctypes.byref(self.ctx))
        if rc != TTS_OK:
            raise TTSError(rc, "tts_create failed")
        self._weights = None

    # -------------------------------------------------------------- plumbing
    def _check(self, rc: int, what: str):
        if rc != TTS_OK:
            raise TTSError(rc, f"{what}: {self.lib.tts_last_error(self.ctx).decode()}")

    def close(self):
        if getattr(self, "ctx", None) and self.ctx.value:
            self.lib.tts_destroy(self.ctx)
            self.ctx = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -------------------------------------------------------------- API
    def load_weights(self, weights: dict):
        """weights: name -> torch CUDA tensor (float32, or bfloat16 for bf16 models)."""
        torch = self.torch
        names = list(weights.keys())
        n = len(names)
        c_names = (ctypes.c_char_p * n)(*[k.encode() for k in names])
        ptrs = (ctypes.c_void_p * n)(*[weights[k].data_ptr() for k in names])
        shapes = (ctypes.c_int64 * (4 * n))()
        ranks = (ctypes.c_int32 * n)()
        dtypes = (ctypes.c_int32 * n)()
        for i, k in enumerate(names):
            t = weights[k]
            if not t.is_contiguous():
                raise ValueError(f"{k} must be contiguous")
            ranks[i] = t.dim()
            for j, s in enumerate(t.shape):
                shapes[4 * i + j] = s
            dtypes[i] = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32, torch.uint8: DTYPE_FP8_E4M3}.get(t.dtype, 99)
        self._check(self.lib.tts_load_weights(self.ctx, n, c_names, ptrs, shapes, ranks, dtypes), "tts_load_weights")
        self._weights = weights

    def prefill(self, ids, sem_logits=None):
        B, n = ids.shape
        self._check(self.lib.tts_prefill(self.ctx, _ptr(ids), B, n, _ptr(sem_logits)), "tts_prefill")

    def prefill_ragged(self, ids, lengths, sem_logits=None):
        """Prefill of prompts of different lengths: ids [B, n] (stream b's prompt is its first
        lengths[b] ids), lengths a host sequence of B ints in [1, n]."""
        B, n = ids.shape
        arr = (ctypes.c_int32 * B)(*[int(x) for x in lengths])
        self._check(self.lib.tts_prefill_ragged(self.ctx, _ptr(ids), arr, B, n, _ptr(sem_logits)), "tts_prefill_ragged")

    def set_stop(self, eos_id: int, stop_frames=None):
        """Per-stream stop on semantic id eos_id (-1: off); stop_frames: int32 device tensor of
        max_batch entries receiving each stream's stop frame (-1 while it runs)."""
        self._check(self.lib.tts_set_stop(self.ctx, int(eos_id), _ptr(stop_frames)), "tts_set_stop")

    def talker_step(self, prev_codes, sem_logits=None, text_ids=None):
        """One Talker step on the previous frame's codes [B, 16]; text_ids [B] (int32, -1 = none)
        adds the streaming text row of each stream."""
        if text_ids is None:
            self._check(self.lib.tts_talker_step(self.ctx, _ptr(prev_codes), _ptr(sem_logits)), "tts_talker_step")
        else:
            self._check(self.lib.tts_talker_step_text(self.ctx, _ptr(prev_codes), _ptr(text_ids), _ptr(sem_logits)),
                        "tts_talker_step_text")

    def set_text_stream(self, text_ids, next_index: int = 0):
        """Streaming text for run_frames: text_ids [B, n_text] (int32 device tensor, kept alive by
        the caller) or None; the step on frame t's codes adds id [b][next_index + t]."""
        if text_ids is None:
            self._check(self.lib.tts_set_text_stream(self.ctx, None, 0, 0), "tts_set_text_stream")
        else:
            self._check(self.lib.tts_set_text_stream(self.ctx, _ptr(text_ids), int(text_ids.shape[1]), int(next_index)),
                        "tts_set_text_stream")

    def codepred_frame(self, semantic, sampling, u, codes, forced=None, logits=None):
        s = sampling_struct(sampling)
        self._check(self.lib.tts_codepred_frame(self.ctx, _ptr(semantic), ctypes.byref(s), _ptr(u), _ptr(forced),
                                                _ptr(codes), _ptr(logits)), "tts_codepred_frame")

    def sample(self, logits, sampling, u, out, history=None):
        B, V = logits.shape
        s = sampling_struct(sampling)
        self._check(self.lib.tts_sample(self.ctx, _ptr(logits), B, V, ctypes.byref(s), _ptr(u), _ptr(history),
                                        _ptr(out)), "tts_sample")

    def run_frames(self, n, sem, ac, u, codes):
        s1, s2 = sampling_struct(sem), sampling_struct(ac)
        self._check(self.lib.tts_run_frames(self.ctx, n, ctypes.byref(s1), ctypes.byref(s2), _ptr(u), _ptr(codes)),
                    "tts_run_frames")

    def run_frames_noalloc(self, n, sem, ac, u, codes):
        s1, s2 = sampling_struct(sem), sampling_struct(ac)
        self._check(self.lib.tts_run_frames_noalloc(self.ctx, n, ctypes.byref(s1), ctypes.byref(s2), _ptr(u), _ptr(codes)),
                    "tts_run_frames_noalloc")

    def progress(self) -> tuple[int, int]:
        p, f = ctypes.c_int32(), ctypes.c_int32()
        self._check(self.lib.tts_get_progress(self.ctx, ctypes.byref(p), ctypes.byref(f)), "tts_get_progress")
        return p.value, f.value

    def reset(self):
        self._check(self.lib.tts_reset(self.ctx), "tts_reset")

    def set_exec_mode(self, mode: int):
        self._check(self.lib.tts_set_exec_mode(self.ctx, mode), "tts_set_exec_mode")

    def exec_mode(self) -> tuple[int, int]:
        """(mode, bits of the persistent kernels this config allows: PERSISTENT_CODEPRED | PERSISTENT_TALKER)."""
        m, sup = ctypes.c_int32(), ctypes.c_int32()
        self._check(self.lib.tts_get_exec_mode(self.ctx, ctypes.byref(m), ctypes.byref(sup)), "tts_get_exec_mode")
        return m.value, sup.value

    def set_prefill_mode(self, mode: int):
        self._check(self.lib.tts_set_prefill_mode(self.ctx, mode), "tts_set_prefill_mode")

    def prefill_mode(self) -> int:
        m = ctypes.c_int32()
        self._check(self.lib.tts_get_prefill_mode(self.ctx, ctypes.byref(m)), "tts_get_prefill_mode")
        return m.value

    def device_status(self) -> int:
        st = ctypes.c_int32()
        self._check(self.lib.tts_device_status(self.ctx, ctypes.byref(st)), "tts_device_status")
        return st.value


def weights_to_device(weights: dict, model: ModelCfg, device="cuda") -> dict:
    """Upload generator arrays as torch tensors: fp32 arrays as float32, uint16 bf16 bit patterns
    as bfloat16, uint8 E4M3 codes as uint8 (fp8 models; their '<name>.scale' arrays as float32)."""
    import torch
    out = {}
    names = [n for n, _, _ in tensor_specs(model)] + [n for n, _ in scale_specs(model)]
    for name in names:
        a = np.ascontiguousarray(weights[name])
        if a.dtype == np.uint16:
            t = torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        elif a.dtype == np.uint8:
            t = torch.from_numpy(a).to(device)
        else:
            t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
        out[name] = t
    return out
