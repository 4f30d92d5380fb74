"""Model and workload shapes for the per-frame Talker + CodePredictor decode.

Pure data: no arithmetic of the method lives here.

A frame is 16 codebook tokens [semantic, acoustic 1..15] covering 80 ms of
audio at 24 kHz (1920 samples), so real time is 12.5 frames/s
["Running Qwen3-TTS on an AMD R9700", section "Running Qwen3-TTS"].
The Talker emits the semantic token once per frame and the CodePredictor
fills in the 15 acoustic tokens in 15 sequential steps (same section).
The block shapes below are synthetic Qwen3-style decoders at the 0.6B and
1.7B sizes the pages name; the 1.7B CodePredictor reproduces the 0.350 GB
fp16 size the same section gives (15 Talker-width acoustic tables plus a
2048->1024 input projection).
"""
from __future__ import annotations

from dataclasses import dataclass, field, asdict

FRAME_RATE_HZ = 24000 / 1920  # 12.5 frames per second of audio
N_ACOUSTIC = 15
CODES_PER_FRAME = 1 + N_ACOUSTIC


@dataclass(frozen=True)
class StackCfg:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int  # semantic vocab (Talker) or per-codebook acoustic vocab (CodePredictor)


@dataclass(frozen=True)
class ModelCfg:
    name: str
    talker: StackCfg
    codepred: StackCfg
    text_vocab: int
    weight_dtype: str  # "fp32", "bf16" or "fp8" (E4M3 projection matrices, bf16 gains/embeddings)
    n_acoustic: int = N_ACOUSTIC
    rms_eps: float = 1e-6
    rope_theta: float = 1e6

    def as_dict(self) -> dict:
        return asdict(self)


@dataclass(frozen=True)
class SamplingCfg:
    do_sample: bool = False
    top_k: int = 50
    top_p: float = 1.0
    temperature: float = 1.0
    repetition_penalty: float = 1.0

    def as_dict(self) -> dict:
        return asdict(self)


GREEDY = SamplingCfg(do_sample=False)
# Semantic sampling defaults: top_k 50, top_p 1.0, temperature 0.9, repetition
# penalty 1.05; the acoustic ("subtalker") controls list no repetition penalty
# ["qwen3-tts-hip" README, section "Library Usage"].
SEMANTIC_SAMPLED = SamplingCfg(do_sample=True, top_k=50, top_p=1.0, temperature=0.9, repetition_penalty=1.05)
ACOUSTIC_SAMPLED = SamplingCfg(do_sample=True, top_k=50, top_p=1.0, temperature=0.9, repetition_penalty=1.0)


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelCfg
    batch: int
    prefill_len: int
    frames: int
    semantic: SamplingCfg = field(default=GREEDY)
    acoustic: SamplingCfg = field(default=GREEDY)
    weight_seed: int = 0
    ids_seed: int = 1
    uniform_seed: int = 2


TINY = ModelCfg(
    name="tiny-fp32",
    talker=StackCfg(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=768, vocab=512),
    codepred=StackCfg(n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=768, vocab=512),
    text_vocab=1024,
    weight_dtype="fp32",
)

M06B = ModelCfg(
    name="0.6b-class-bf16",
    talker=StackCfg(n_layers=28, hidden=1024, n_q_heads=16, n_kv_heads=8, head_dim=128, ffn=3072, vocab=3072),
    codepred=StackCfg(n_layers=5, hidden=1024, n_q_heads=16, n_kv_heads=8, head_dim=128, ffn=3072, vocab=2048),
    text_vocab=151936,
    weight_dtype="bf16",
)

M17B = ModelCfg(
    name="1.7b-class-bf16",
    talker=StackCfg(n_layers=28, hidden=2048, n_q_heads=16, n_kv_heads=8, head_dim=128, ffn=6144, vocab=3072),
    codepred=StackCfg(n_layers=5, hidden=1024, n_q_heads=16, n_kv_heads=8, head_dim=128, ffn=3072, vocab=2048),
    text_vocab=151936,
    weight_dtype="bf16",
)

# Weight-only FP8 variants: the same drawn (bf16-rounded) weights, with every projection matrix
# stored as E4M3 codes and one fp32 scale per output row.
M06B_FP8 = ModelCfg(name="0.6b-class-fp8", talker=M06B.talker, codepred=M06B.codepred, text_vocab=M06B.text_vocab,
                    weight_dtype="fp8")
M17B_FP8 = ModelCfg(name="1.7b-class-fp8", talker=M17B.talker, codepred=M17B.codepred, text_vocab=M17B.text_vocab,
                    weight_dtype="fp8")

WORKLOADS = {
    "tiny": Workload("tiny", TINY, batch=1, prefill_len=32, frames=16),
    "0.6b": Workload("0.6b", M06B, batch=1, prefill_len=64, frames=240),
    "1.7b": Workload("1.7b", M17B, batch=1, prefill_len=64, frames=240),
    "1.7b-long": Workload("1.7b-long", M17B, batch=1, prefill_len=256, frames=2000),
    # the 1.7B batch-1 decode with the pages' default sampling of both token kinds
    "1.7b-sampled": Workload("1.7b-sampled", M17B, batch=1, prefill_len=64, frames=240,
                             semantic=SEMANTIC_SAMPLED, acoustic=ACOUSTIC_SAMPLED),
    "1.7b-x32": Workload("1.7b-x32", M17B, batch=32, prefill_len=64, frames=240,
                         semantic=SEMANTIC_SAMPLED, acoustic=ACOUSTIC_SAMPLED),
    "0.6b-fp8": Workload("0.6b-fp8", M06B_FP8, batch=1, prefill_len=64, frames=240),
    "1.7b-fp8": Workload("1.7b-fp8", M17B_FP8, batch=1, prefill_len=64, frames=240),
}

MODELS = {"tiny": TINY, "0.6b": M06B, "1.7b": M17B, "0.6b-fp8": M06B_FP8, "1.7b-fp8": M17B_FP8}

# Projection matrices (stored as E4M3 codes plus per-row scales in fp8 models).
QUANT_SUFFIXES = (".wq", ".wk", ".wv", ".wo", ".wg", ".wu", ".wd")
QUANT_NAMES = ("talker.lm_head", "cp.proj", "cp.heads")


def is_quantized(cfg: ModelCfg, name: str) -> bool:
    """True for the tensors an fp8 model stores as E4M3 codes with a '<name>.scale' companion."""
    return cfg.weight_dtype == "fp8" and (name in QUANT_NAMES or name.endswith(QUANT_SUFFIXES))


def scale_specs(cfg: ModelCfg) -> list[tuple[str, tuple[int, ...]]]:
    """The fp32 per-row scale tensors of an fp8 model (none for other dtypes)."""
    return [(name + ".scale", shape[:-1]) for name, shape, _ in tensor_specs(cfg) if is_quantized(cfg, name)]


def tensor_specs(cfg: ModelCfg) -> list[tuple[str, tuple[int, ...], str]]:
    """Canonical tensor list (name, shape, kind) in generation order.

    kind is "w" for a projection/embedding drawn N(0, 0.02) or "gain" for a
    norm gain drawn 1 + N(0, 0.01). All projections are [out, in] row-major.
    """
    specs: list[tuple[str, tuple[int, ...], str]] = []
    t, c = cfg.talker, cfg.codepred
    specs.append(("talker.embed_text", (cfg.text_vocab, t.hidden), "w"))
    specs.append(("talker.embed_sem", (t.vocab, t.hidden), "w"))

    def stack(prefix: str, s: StackCfg) -> None:
        qd, kd = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim
        for i in range(s.n_layers):
            p = f"{prefix}.layers.{i}."
            specs.extend([
                (p + "attn_norm", (s.hidden,), "gain"),
                (p + "wq", (qd, s.hidden), "w"),
                (p + "wk", (kd, s.hidden), "w"),
                (p + "wv", (kd, s.hidden), "w"),
                (p + "q_norm", (s.head_dim,), "gain"),
                (p + "k_norm", (s.head_dim,), "gain"),
                (p + "wo", (s.hidden, qd), "w"),
                (p + "mlp_norm", (s.hidden,), "gain"),
                (p + "wg", (s.ffn, s.hidden), "w"),
                (p + "wu", (s.ffn, s.hidden), "w"),
                (p + "wd", (s.hidden, s.ffn), "w"),
            ])
        specs.append((f"{prefix}.final_norm", (s.hidden,), "gain"))

    stack("talker", t)
    specs.append(("talker.lm_head", (t.vocab, t.hidden), "w"))
    if t.hidden != c.hidden:
        specs.append(("cp.proj", (c.hidden, t.hidden), "w"))
    specs.append(("cp.embed_ac", (cfg.n_acoustic, c.vocab, t.hidden), "w"))
    stack("cp", c)
    specs.append(("cp.heads", (cfg.n_acoustic, c.vocab, c.hidden), "w"))
    return specs


def param_count(cfg: ModelCfg, part: str) -> int:
    """Parameter count of "talker" or "cp" (the CodePredictor incl. its tables)."""
    n = 0
    for name, shape, _ in tensor_specs(cfg):
        if name.startswith(part + "."):
            k = 1
            for s in shape:
                k *= s
            n += k
    return n
