"""Bytes-per-frame and bandwidth-bound arithmetic for the frame decode.

The pages' own cost model ("Running Qwen3-TTS on an AMD R9700", section
"Running Qwen3-TTS"): if the decode is bound by memory bandwidth, the time
per frame is the bytes read per frame -- one Talker pass plus 15
CodePredictor passes -- divided by the bandwidth; with fp16 sizes 3.483 GB
and 0.350 GB that is 8.733 GB per frame, i.e. 73.3 frames/s at 640 GB/s.

``pages_crude_bytes_per_frame`` is that formula. ``algorithmic_bytes`` is the
refined count used for the roofline fraction: only the weights a frame
actually streams (all Talker layers + the semantic head; per CodePredictor
step all its layers, one acoustic head and the input projection; the gathered
embedding rows) plus the KV-cache bytes attention reads. Embedding tables are
not streamed whole and the 14 idle heads of a step are not read.
"""
from __future__ import annotations

import hashlib
import os
import re

from .config import ModelCfg, StackCfg, FRAME_RATE_HZ

HBM_PEAK_BYTES_PER_S = 8.0e12  # MI355X published HBM3E bandwidth


def pages_crude_bytes_per_frame(talker_bytes: float, cp_bytes: float, cp_passes: int = 15) -> float:
    return talker_bytes + cp_passes * cp_bytes


def bound_fps(bytes_per_frame: float, bandwidth_bytes_per_s: float) -> float:
    return bandwidth_bytes_per_s / bytes_per_frame


def rtf_from_fps(fps: float) -> float:
    """Real-time factor = compute time / audio time = 12.5 / fps."""
    return FRAME_RATE_HZ / fps


def _mbytes(cfg: ModelCfg) -> int:
    """Bytes per projection-matrix element (E4M3 codes: 1)."""
    return {"fp32": 4, "bf16": 2, "fp8": 1}[cfg.weight_dtype]


def _tbytes(cfg: ModelCfg) -> int:
    """Bytes per gain / embedding element (bf16 next to E4M3 matrices)."""
    return 4 if cfg.weight_dtype == "fp32" else 2


def _matrix_bytes(cfg: ModelCfg, rows: int, cols: int) -> int:
    """A projection matrix as stored: its elements, plus one fp32 scale per row for E4M3."""
    return rows * cols * _mbytes(cfg) + (4 * rows if cfg.weight_dtype == "fp8" else 0)


def layer_weight_elems(s: StackCfg) -> int:
    qd, kd = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim
    proj = s.hidden * (qd + 2 * kd) + qd * s.hidden + 3 * s.hidden * s.ffn
    norms = 2 * s.hidden + 2 * s.head_dim
    return proj + norms


def layer_weight_bytes(cfg: ModelCfg, s: StackCfg) -> int:
    """Stored bytes of one decoder layer: the seven projections and the four gains."""
    qd, kd = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim
    mats = (_matrix_bytes(cfg, qd + 2 * kd, s.hidden) + _matrix_bytes(cfg, s.hidden, qd)
            + _matrix_bytes(cfg, 2 * s.ffn, s.hidden) + _matrix_bytes(cfg, s.hidden, s.ffn))
    return mats + (2 * s.hidden + 2 * s.head_dim) * _tbytes(cfg)


def kv_bytes_per_position(s: StackCfg, kv_elem_bytes: int) -> int:
    """K and V bytes of one position in one layer."""
    return 2 * s.n_kv_heads * s.head_dim * kv_elem_bytes


def algorithmic_bytes(cfg: ModelCfg, talker_positions_read: float, batch: int = 1, kv_elem_bytes: int | None = None) -> dict:
    """Algorithmic bytes of one frame (per stream batch of ``batch`` lockstep streams).

    talker_positions_read: number of cached positions the Talker's attention
    reads in this frame (p + 1 at Talker position p). Weights are shared by
    the batch; embeddings, KV reads scale with it.
    """
    t, c = cfg.talker, cfg.codepred
    tb = _tbytes(cfg)
    kvb = tb if kv_elem_bytes is None else kv_elem_bytes
    talker_w = t.n_layers * layer_weight_bytes(cfg, t) + t.hidden * tb + _matrix_bytes(cfg, t.vocab, t.hidden)
    emb_rows = batch * (1 + cfg.n_acoustic) * t.hidden * tb
    cp_step_w = c.n_layers * layer_weight_bytes(cfg, c) + c.hidden * tb + _matrix_bytes(cfg, c.vocab, c.hidden)
    if t.hidden != c.hidden:
        cp_step_w += _matrix_bytes(cfg, c.hidden, t.hidden)
    cp_rows = batch * (1 + cfg.n_acoustic) * t.hidden * tb  # E_sem row + 14 acoustic rows (+h_T) fed to the CodePredictor
    kv_t = batch * t.n_layers * kv_bytes_per_position(t, kvb) * talker_positions_read
    # CodePredictor attention over positions 0..j for its 16 positions (0..15).
    cp_positions = sum(j + 1 for j in range(cfg.n_acoustic + 1))
    kv_c = batch * c.n_layers * kv_bytes_per_position(c, kvb) * cp_positions
    weights = talker_w + cfg.n_acoustic * cp_step_w
    total = weights + emb_rows + cp_rows + kv_t + kv_c
    return {"talker_weights": talker_w, "cp_step_weights": cp_step_w, "weights": weights,
            "embedding_rows": emb_rows + cp_rows, "kv_talker": kv_t, "kv_cp": kv_c, "total": total,
            # the CodePredictor part of the frame alone (its 15 steps)
            "cp_frame": cfg.n_acoustic * cp_step_w + cp_rows + kv_c}


def frame_bytes_for_run(cfg: ModelCfg, prefill_len: int, first_frame: int, n_frames: int, batch: int = 1,
                        kv_elem_bytes: int | None = None) -> float:
    """Total algorithmic bytes of frames [first_frame, first_frame + n_frames).

    Frame t (t >= 0) samples its semantic token from the pending Talker
    output, runs the 15 CodePredictor steps and then the Talker step that
    consumes its codes at position prefill_len + t (reading prefill_len + t + 1
    cached positions).
    """
    tot = 0.0
    for t in range(first_frame, first_frame + n_frames):
        tot += algorithmic_bytes(cfg, prefill_len + t + 1, batch, kv_elem_bytes)["total"]
    return tot


# ---------------------------------------------------------------------------- measured traffic

_CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
_PROFILES = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")


def kernel_source_sha256(files=("tts_xcp.h", "tts_xtp.h", "tts_device.h")) -> str:
    """SHA-256 over the sources a persistent kernel is built from (in the given order)."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(_CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(record: str, files=("tts_xcp.h", "tts_xtp.h", "tts_device.h")) -> int | None:
    """HBM bytes per launch from a committed counter record, or None when there is none or the
    kernel's sources changed since the counters were taken.

    The record (a text file under profiles/) holds the lines
    ``kernel_source_sha256: <hex>`` and ``traffic_bytes_per_launch: <int>``.
    """
    path = os.path.join(_PROFILES, record)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            m = re.match(r"^\s*(kernel_source_sha256|traffic_bytes_per_launch):\s*(\S+)\s*$", line)
            if m:
                fields[m.group(1)] = m.group(2)
    if fields.get("kernel_source_sha256") != kernel_source_sha256(files):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None
