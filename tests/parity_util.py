"""Shared helpers of the GPU parity tests (imported by tests only)."""
from __future__ import annotations

import numpy as np

from oracle.sampler import sample_token

MARGIN = 0.05  # greedy steps whose oracle top-2 margin is at most this are exempt
# Sampled-draw tests compare at least this fraction of their draws (the rest are exempt, see
# sample_exempt): dense top-k sets of small synthetic logits hold near ties in their order.
MIN_CHECKED = 0.8


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


def greedy_agreement(gpu_tokens, ref_logits, rel=None):
    """Return (n_checked, n_exempt, mismatches) for greedy tokens vs oracle argmax. A step is
    exempt when the oracle's top-2 margin is at most MARGIN, or, with rel (the fp32 model's
    relative logit bar), at most 2 rel max|logit|: the most two logits within the bar can move
    against each other."""
    ref_logits = np.asarray(ref_logits)
    ref_tok = np.argmax(ref_logits, axis=-1)
    thr = MARGIN if rel is None else 2.0 * rel * np.max(np.abs(ref_logits), axis=-1)
    ok = top2_margin(ref_logits) > thr
    gpu_tokens = np.asarray(gpu_tokens)
    bad = np.nonzero(ok & (gpu_tokens != ref_tok))
    return int(ok.sum()), int((~ok).sum()), list(zip(*bad))


def sample_exempt(logits_row, cfg: dict, u: float, history=None, rel: float = 1e-4) -> bool:
    """A sampled step is exempt when the draw sits within rel of a boundary:
    |u*sum(w) - running sum| < rel*sum(w); or the top-k cut falls between
    logits closer than rel*max|logit| after penalty and temperature; or the
    drawn id's logit is that close to a neighbour's in the kept order (two ids
    that near a tie may trade places, and the draw's interval then belongs to
    either: the order of equal keys is not unique).
    rel is the relative logit error the compared path may carry."""
    if not cfg["do_sample"]:
        return bool(top2_margin(logits_row) <= MARGIN)
    tok, det = sample_token(np.asarray(logits_row, np.float32), cfg, u, history, dtype=np.float32, return_detail=True)
    cum, target = det["cum"].astype(np.float64), float(det["target"])
    if np.min(np.abs(cum - target)) < rel * cum[-1]:
        return True
    scaled = np.sort(det["scaled_all"].astype(np.float64))[::-1]
    band = rel * np.max(np.abs(scaled))
    k = len(det["keep"])
    if k < len(scaled) and (scaled[k - 1] - scaled[k]) < band:
        return True
    lk, pos = det["scaled"].astype(np.float64), det["pos"]
    if (pos > 0 and lk[pos - 1] - lk[pos] < band) or (pos + 1 < len(lk) and lk[pos] - lk[pos + 1] < band):
        return True
    return False


def check_free_running(orc, ids, got, frames, sampling, tag, rel=None, min_frac=0.5, upto=None, **gen_kw):
    """A free-running GPU run checked step by step: the oracle is run teacher-forced along the
    GPU's own codes got [B, frames, 16], and at every step the oracle does not find near a tie
    (see greedy_agreement) the GPU's code must be the oracle's argmax. upto [B] (or None): the
    number of codes of each stream that count (a stopped stream's later codes are masked).
    At least min_frac of the counted codes must be checked. Returns (checked, exempt)."""
    got = np.asarray(got)
    B = got.shape[0]
    fref = orc.generate(ids, frames, sampling, sampling, np.zeros((B, frames, 16), np.float32),
                        teacher=np.maximum(got, 0), **gen_kw)
    thr_s = MARGIN if rel is None else 2.0 * rel * np.max(np.abs(fref["sem_logits"]), axis=-1)
    thr_a = MARGIN if rel is None else 2.0 * rel * np.max(np.abs(fref["ac_logits"]), axis=-1)
    tok = np.empty((B, frames, 16), np.int64)
    tok[:, :, 0] = np.argmax(fref["sem_logits"], axis=-1)
    tok[:, :, 1:] = np.argmax(fref["ac_logits"], axis=-1)
    ok = np.empty((B, frames, 16), bool)
    ok[:, :, 0] = top2_margin(fref["sem_logits"]) > thr_s
    ok[:, :, 1:] = top2_margin(fref["ac_logits"]) > thr_a
    counted = np.ones((B, frames * 16), bool)
    if upto is not None:
        for b in range(B):
            counted[b, int(upto[b]):] = False
    counted = counted.reshape(B, frames, 16)
    bad = np.nonzero(counted & ok & (got != tok))
    assert bad[0].size == 0, f"{tag}: {bad[0].size} codes differ from the oracle's argmax at non-exempt steps, first at " \
                             f"stream {bad[0][0]} frame {bad[1][0]} code {bad[2][0]}"
    n, ex = int((counted & ok).sum()), int((counted & ~ok).sum())
    assert n >= min_frac * counted.sum(), f"{tag}: only {n} of {int(counted.sum())} codes checked ({ex} near ties)"
    return n, ex


def check_stop_masking(got, stop_got, eos, tag):
    """The reported codes of a frame-graph run with the stop id eos: stream b's stop frame is the
    first frame whose drawn semantic token is eos (-1 if there is none), that frame's 15 acoustic
    codes and every later code read -1, and stop_got[b] names that frame. Returns upto [B], the
    number of each stream's codes before the masking (the stop frame's semantic token included)."""
    got = np.asarray(got)
    B, F = got.shape[:2]
    upto = np.full(B, F * 16)
    for b in range(B):
        hits = np.nonzero(got[b, :, 0] == eos)[0]
        ts = int(hits[0]) if hits.size else -1
        assert int(stop_got[b]) == ts, f"{tag}: stream {b} reports stop frame {int(stop_got[b])}, its codes say {ts}"
        if ts >= 0:
            assert (got[b, ts, 1:] == -1).all() and (got[b, ts + 1:] == -1).all(), f"{tag}: stream {b} codes after the stop"
            upto[b] = ts * 16 + 1
        else:
            assert (got[b] >= 0).all(), f"{tag}: stream {b} has masked codes without a stop"
    return upto
