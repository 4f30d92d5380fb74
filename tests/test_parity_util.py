"""The exemption rule the sampled-draw parity tests use (tests/parity_util.py), pinned on hand-built
logit rows: a draw is exempt only where the compared path's logit error could change it."""
import numpy as np

from oracle.sampler import sample_token
from parity_util import sample_exempt

CFG = {"do_sample": True, "top_k": 50, "top_p": 1.0, "temperature": 0.9, "repetition_penalty": 1.0}


def _row(tie: bool) -> np.ndarray:
    """Logits falling by 0.05 per id (id order = sorted order); with tie, id 11 sits 1e-6 below id 10."""
    lg = (-0.05 * np.arange(100)).astype(np.float32)
    if tie:
        lg[11] = lg[10] - np.float32(1e-6)
    return lg


def _cum(lg: np.ndarray) -> np.ndarray:
    _, det = sample_token(lg, CFG, 0.5, None, dtype=np.float32, return_detail=True)
    return det["cum"].astype(np.float64)


def test_a_draw_far_from_every_boundary_is_compared():
    lg = _row(False)
    cum = _cum(lg)
    u = float((cum[9] + cum[10]) / 2 / cum[-1])  # the middle of id 10's interval
    assert sample_token(lg, CFG, u, None, dtype=np.float32) == 10
    assert sample_exempt(lg, CFG, u, rel=1e-4) is False


def test_a_draw_at_a_cdf_step_is_exempt():
    lg = _row(False)
    cum = _cum(lg)
    assert sample_exempt(lg, CFG, float(cum[10] / cum[-1]), rel=1e-4) is True


def test_a_near_tie_at_the_drawn_position_is_exempt():
    # ids 10 and 11 within the band: either may hold position 10 of the order, so the draw is not unique
    lg = _row(True)
    cum = _cum(lg)
    u = float((cum[9] + cum[10]) / 2 / cum[-1])
    assert sample_token(lg, CFG, u, None, dtype=np.float32) == 10
    assert sample_exempt(lg, CFG, u, rel=1e-4) is True
    # a draw two positions away from the tie is still compared
    u2 = float((cum[12] + cum[13]) / 2 / cum[-1])
    assert sample_token(lg, CFG, u2, None, dtype=np.float32) == 13
    assert sample_exempt(lg, CFG, u2, rel=1e-4) is False


def test_a_top_k_cut_inside_a_tie_is_exempt():
    lg = _row(False)
    lg[50] = lg[49] - np.float32(1e-6)  # ids 49 and 50 straddle the cut of top-k 50
    cum = _cum(lg)
    u = float((cum[9] + cum[10]) / 2 / cum[-1])
    assert sample_exempt(lg, CFG, u, rel=1e-4) is True
