"""Shared helpers of the GPU parity tests (imported by tests only)."""
from __future__ import annotations

import numpy as np

from oracle.sampler import sample_token

MARGIN = 0.05  # greedy steps whose oracle top-2 margin is at most this are exempt


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def rowwise_rel_err(got, ref) -> np.ndarray:
    """max|got - ref| / max|ref| per row of the last axis."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.max(np.abs(got - ref), axis=-1) / np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)


def top2_margin(logits) -> np.ndarray:
    s = np.sort(np.asarray(logits, dtype=np.float64), axis=-1)
    return s[..., -1] - s[..., -2]


def greedy_agreement(gpu_tokens, ref_logits):
    """Return (n_checked, n_exempt, mismatches) for greedy tokens vs oracle argmax."""
    ref_logits = np.asarray(ref_logits)
    ref_tok = np.argmax(ref_logits, axis=-1)
    ok = top2_margin(ref_logits) > MARGIN
    gpu_tokens = np.asarray(gpu_tokens)
    bad = np.nonzero(ok & (gpu_tokens != ref_tok))
    return int(ok.sum()), int((~ok).sum()), list(zip(*bad))


def sample_exempt(logits_row, cfg: dict, u: float, history=None, rel: float = 1e-4) -> bool:
    """A sampled step is exempt when the draw sits within rel of a boundary:
    |u*sum(w) - running sum| < rel*sum(w), or the top-k cut falls between
    logits closer than rel*max|logit| after penalty and temperature.
    rel is the relative logit error the compared path may carry."""
    if not cfg["do_sample"]:
        return bool(top2_margin(logits_row) <= MARGIN)
    tok, det = sample_token(np.asarray(logits_row, np.float32), cfg, u, history, dtype=np.float32, return_detail=True)
    cum, target = det["cum"].astype(np.float64), float(det["target"])
    if np.min(np.abs(cum - target)) < rel * cum[-1]:
        return True
    scaled = np.sort(det["scaled_all"].astype(np.float64))[::-1]
    k = len(det["keep"])
    if k < len(scaled) and (scaled[k - 1] - scaled[k]) < rel * np.max(np.abs(scaled)):
        return True
    return False
