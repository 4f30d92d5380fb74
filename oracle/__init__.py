"""Oracle: a plain, slow CPU reference of the per-frame Talker + CodePredictor decode.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The product path (``autoregressive_tts_decode_amd`` and its HIP
library) never imports it, and this package imports nothing from the product:
the two sides share only the seeded input arrays.

The oracle is NumPy, written step by step in the order the method runs
(an autoregressive recurrence has no cheaper closed form), parameterised by a
working dtype (float64 for pins, float32 for parity and timing). Library
primitives used as steps: matrix products (``@``), ``np.exp``, ``np.sort``.

Sources, by page title and section:
  * "Running Qwen3-TTS on an AMD R9700", section "Running Qwen3-TTS": a frame
    is [semantic, acoustic 1..15]; the Talker emits the semantic token, the
    CodePredictor the 15 acoustic tokens; the per-frame cost model is one
    Talker pass plus 15 CodePredictor passes.
  * "qwen3-tts-hip" README, section "Library Usage": sampling controls
    (do_sample, top_k, top_p, temperature, repetition_penalty for the
    semantic token; the subtalker set without a repetition penalty);
    section "Python Parity Fixtures": CodePredictor token and embedding-sum
    parity as a checked stage.
  * Block internals (pre-norm Qwen3 decoder: per-head q/k RMSNorm before
    rotate-half RoPE, grouped-query attention, SwiGLU) are a reading, not on
    the pages; every such reading is listed in the module docstrings below.

Parity pins live in ``tests/test_oracle_*.py``. Parity unpinned: fidelity to
the real Qwen3-TTS checkpoints (not available) is not pinned; internal
consistency and the closed forms are.
"""
from .decoder import (  # noqa: F401
    OracleModel,
    rms_norm,
    rope_cos_sin,
    apply_rope,
    softmax,
    attend,
    linear,
    swiglu,
    silu,
    bf16_bits_to_float,
)
from .sampler import sample_token, sample_rows  # noqa: F401
