"""MI355X-native per-frame Talker + CodePredictor decode (Qwen3-style TTS).

The compute path is the HIP library ``libtts.so`` behind the C ABI declared in
``include/tts.h``; :mod:`autoregressive_tts_decode_amd.tts` is its thin ctypes
binding. Importing the package does not load the library.
"""
from .config import WORKLOADS, MODELS, ModelCfg, StackCfg, SamplingCfg, Workload  # noqa: F401
