"""Oracle token sampler.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The controls are the ones the "qwen3-tts-hip" README lists in section
"Library Usage": do_sample, top_k, top_p, temperature and repetition_penalty
for the semantic token, and the same set without a repetition penalty for the
acoustic ("subtalker") tokens; a fixed seed makes sampling reproducible, here
by passing pre-drawn uniforms in [0, 1).

Readings where the pages are silent (listed in the design notes):
  * greedy (do_sample false) = argmax of the raw logits, lowest id on ties;
  * order: repetition penalty -> temperature -> top-k -> top-p -> softmax ->
    inverse CDF;
  * repetition penalty on the set of previously emitted ids: a positive logit
    is divided by r, a non-positive one multiplied by r;
  * top-k keeps exactly k ids ordered by (logit descending, id ascending);
    top_k <= 0 keeps all;
  * top-p keeps the shortest prefix of that order whose probability mass
    reaches top_p; top_p >= 1 keeps everything;
  * inverse CDF: with w_i = exp(l_i - l_max) in that order, return the first
    id whose running sum exceeds u * sum(w); the last kept id otherwise.

``dtype`` sets the precision of the decision: float64 for the pins, float32
to take the decision in the same precision as a float32 kernel.
"""
from __future__ import annotations

import numpy as np


def _cfg(c) -> dict:
    return c if isinstance(c, dict) else c.as_dict()


def sample_token(logits_row: np.ndarray, cfg, u: float, history: np.ndarray | None = None,
                 dtype=np.float64, return_detail: bool = False):
    """Draw one id from a logit row [V]. history: bool mask [V] of emitted ids or None."""
    cfg = _cfg(cfg)
    dt = np.dtype(dtype)
    l = np.array(logits_row, dtype=dt, copy=True)
    V = l.shape[0]
    if not cfg["do_sample"]:
        tok = int(np.argmax(l))
        return (tok, None) if return_detail else tok
    r = dt.type(cfg["repetition_penalty"])
    if history is not None and cfg["repetition_penalty"] != 1.0:
        idx = np.nonzero(history)[0]
        vals = l[idx]
        l[idx] = np.where(vals > 0, vals / r, vals * r)
    l = l / dt.type(cfg["temperature"])
    order = np.lexsort((np.arange(V), -l))  # primary: logit descending; secondary: id ascending
    k = V if cfg["top_k"] <= 0 else min(int(cfg["top_k"]), V)
    keep = order[:k]
    lk = l[keep]
    if cfg["top_p"] < 1.0:
        e = np.exp(lk - lk[0])
        cum = np.cumsum(e / np.sum(e))
        m = int(np.searchsorted(cum, dt.type(cfg["top_p"]), side="left"))
        keep, lk = keep[: m + 1], lk[: m + 1]
    w = np.exp(lk - lk[0])
    cum = np.cumsum(w)
    target = dt.type(u) * cum[-1]
    hit = np.nonzero(cum > target)[0]
    pos = int(hit[0]) if hit.size else len(keep) - 1
    tok = int(keep[pos])
    if return_detail:
        return tok, {"keep": keep, "scaled": lk, "cum": cum, "target": target, "pos": pos, "scaled_all": l}
    return tok


def sample_rows(logits: np.ndarray, cfg, u: np.ndarray, history: np.ndarray | None = None,
                dtype=np.float64) -> np.ndarray:
    """Row-wise sample_token over [B, V] logits with per-row uniforms u [B]."""
    B = logits.shape[0]
    out = np.empty(B, dtype=np.int32)
    for b in range(B):
        out[b] = sample_token(logits[b], cfg, float(u[b]), None if history is None else history[b], dtype)
    return out
