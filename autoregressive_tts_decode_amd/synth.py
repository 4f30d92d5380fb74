"""Seeded synthetic inputs: weights, text ids and sampling uniforms.

This module is shared by the oracle side (tests, CPU baseline) and the HIP
side (tests, bench). It holds no arithmetic of the decode method: only random
draws, the bf16 storage rounding of the drawn weights, and array plumbing.

Recipe (the pages name no dataset; real Qwen3-TTS weights and tokenizer are
not available, so seeded random tensors of the same shapes stand in):
  * tensor k of the canonical order (config.tensor_specs) is drawn from
    numpy Generator(PCG64([seed, k])): projections/embeddings are
    0.02 * standard_normal(float32), norm gains 1 + 0.01 * standard_normal;
  * bf16 configs store round-to-nearest-even bf16 of those fp32 draws
    (returned as uint16 bit patterns);
  * fp8 configs start from the same bf16 values; each projection matrix
    (config.is_quantized) is then stored per output row as scale = max|w| / 448
    (fp32; 1 for an all-zero row) and E4M3 codes of w / scale, rounded to
    nearest even by torch's float8_e4m3fn cast (uint8 codes; the scale goes
    under '<name>.scale'). This is weight preparation, done once offline;
    the decode then reads only codes and scales.
  * text ids are uniform integers in [0, text_vocab) from PCG64([ids_seed]);
  * uniforms are fp32 in [0, 1) from PCG64([uniform_seed]), laid out
    [batch, frame, 16]: index 0 drives the semantic draw, j the acoustic j.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .config import ModelCfg, Workload, tensor_specs, is_quantized, CODES_PER_FRAME


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _draw(seed: int, k: int, shape: tuple[int, ...], kind: str, bf16: bool) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64([seed, k]))
    a = g.standard_normal(shape, dtype=np.float32)
    if kind == "w":
        a *= np.float32(0.02)
    else:
        a *= np.float32(0.01)
        a += np.float32(1.0)
    return f32_to_bf16_bits(a) if bf16 else a


E4M3_MAX = 448.0  # largest finite E4M3 magnitude


def quantize_rows_e4m3(bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """bf16 bit patterns [..., K] -> (uint8 E4M3 codes [..., K], fp32 row scales [...])."""
    import torch
    w = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    amax = np.abs(w).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = np.clip(w / scale[..., None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(q)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def _draw_stored(cfg: ModelCfg, seed: int, k: int, name: str, shape: tuple[int, ...], kind: str) -> dict:
    if cfg.weight_dtype != "fp8":
        return {name: _draw(seed, k, shape, kind, cfg.weight_dtype == "bf16")}
    a = _draw(seed, k, shape, kind, True)
    if not is_quantized(cfg, name):
        return {name: a}
    codes, scale = quantize_rows_e4m3(a)
    return {name: codes, name + ".scale": scale}


def make_weights(cfg: ModelCfg, seed: int = 0, threads: int | None = None,
                 only: set[str] | None = None) -> dict[str, np.ndarray]:
    """All model tensors. fp32 configs: float32 arrays; bf16 configs: uint16 bf16 bits;
    fp8 configs: uint8 E4M3 codes + float32 '<name>.scale' for the matrices, bf16 bits otherwise."""
    specs = tensor_specs(cfg)
    jobs = [(k, name, shape, kind) for k, (name, shape, kind) in enumerate(specs)
            if only is None or name in only]
    threads = threads or min(8, len(os.sched_getaffinity(0)))
    out: dict[str, np.ndarray] = {}
    with ThreadPoolExecutor(max_workers=threads) as ex:
        futs = [ex.submit(_draw_stored, cfg, seed, k, name, shape, kind) for k, name, shape, kind in jobs]
        for f in futs:
            out.update(f.result())
    return out


def make_text_ids(wl: Workload) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64([wl.ids_seed]))
    return g.integers(0, wl.model.text_vocab, size=(wl.batch, wl.prefill_len), dtype=np.int64).astype(np.int32)


def make_uniforms(wl: Workload, frames: int | None = None) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64([wl.uniform_seed]))
    fr = wl.frames if frames is None else frames
    return g.random((wl.batch, fr, CODES_PER_FRAME), dtype=np.float32)


def random_ids(n: int, high: int, seed: int, batch: int = 1) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64([seed]))
    return g.integers(0, high, size=(batch, n), dtype=np.int64).astype(np.int32)


def random_logits(shape: tuple[int, ...], scale: float, seed: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64([seed]))
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def random_uniforms(shape: tuple[int, ...], seed: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64([seed]))
    return g.random(shape, dtype=np.float32)
