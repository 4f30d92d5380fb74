"""Oracle decoder: Talker and CodePredictor stacks, prefill and the frame loop.

TEST INFRASTRUCTURE ONLY (see the package docstring). Plain NumPy in a chosen
working dtype; no blocking, fusion or reordering beyond the definitions.

What the pages fix ("Running Qwen3-TTS on an AMD R9700", section "Running
Qwen3-TTS"): each acoustic frame holds 16 tokens [semantic, acoustic 1..15];
the Talker emits the semantic token once per frame; the CodePredictor then
fills in the 15 acoustic tokens of the same frame, one after another.
"qwen3-tts-hip" README, section "Python Parity Fixtures", names the
embedding-sum as a checked stage of the CodePredictor.

Readings where the pages are silent (each is listed in the design notes):
  * Block: pre-norm Qwen3 decoder layer without biases: RMSNorm, q/k/v
    projections, per-head RMSNorm of q and k over head_dim, rotate-half RoPE,
    causal grouped-query attention scaled by 1/sqrt(head_dim), output
    projection + residual, RMSNorm, SwiGLU MLP + residual; final RMSNorm.
  * RoPE: pairs (i, i + d/2), inverse frequency theta^(-2i/d); the angle
    p * inv_i is formed in float64 and cos/sin are rounded to the working dtype.
  * GQA grouping: query head h reads KV head h // (n_q_heads / n_kv_heads).
  * Talker input for frame t >= 1 is the sum of the 16 codebook embeddings of
    frame t-1: E_sem[s] + sum_j E_ac[j][a_j], at Talker position n + t - 1.
  * Streaming text conditioning ("Running Qwen3-TTS on an AMD R9700": the
    streaming mode feeds the model one text token at a time; "qwen3-tts-hip"
    README, section "Library Usage": text_lookahead_tokens sets the text of the
    streaming prefill): with lookahead L the prefill covers ids[:, :L] only,
    and the Talker step of frame t >= 1 adds the text row E_text[ids[:, L+t-1]]
    to the frame's embedding sum while L+t-1 < n; once the text is used up
    nothing is added. With L = n this is the non-streaming decode.
  * Ragged batches and the per-stream stop (the method's next steps; the pages
    name no scheme, and leave the stop unfinished): streams with prompts of
    different lengths decode exactly as if each ran alone, from position 0;
    with a designated semantic id eos, a stream whose drawn semantic token of
    frame t is eos stops there: stop[b] = t, the frame's 15 acoustic codes are
    reported as -1 and every later frame as 16 x -1. The drawn codes are what
    the stream's own next steps consume either way (a stopped stream's later
    output is discarded, so what it computes does not matter).
  * CodePredictor conditioning: positions restart at 0 every frame with an
    empty cache; position 0 holds P·h_T (h_T = the Talker's post-final-norm
    hidden of this frame), position 1 holds P·E_sem[s]; acoustic token j is
    drawn from head j applied to the final-normed output at position j; for
    j >= 2 position j holds P·E_ac[j-1][a_{j-1}]. P is the CodePredictor's
    input projection, the identity when both widths are equal.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .sampler import sample_rows


# ----------------------------------------------------------------------------- primitives

def bf16_bits_to_float(bits: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) exactly: they are the top half of an fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(dtype)


def e4m3_to_float(codes: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Decode OCP E4M3 bytes by the format's definition: bit 7 sign, bits 6..3
    exponent e (bias 7), bits 2..0 mantissa m. e = 0 is subnormal, (m / 8) * 2^-6;
    otherwise (1 + m / 8) * 2^(e - 7); e = 15 with m = 7 is NaN (the format has no
    infinities). Every finite code is exact in float32 and float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return (sign * mag).astype(dtype)


def dequant_rows(codes: np.ndarray, scale: np.ndarray, dtype=np.float64) -> np.ndarray:
    """The matrix an FP8 weight stands for: element [.., r, k] = scale[.., r] * decode(code[.., r, k])
    ("Benchmarking a TTS Model on Your Own GPU": eight-bit weights are widened on the fly; the
    per-row scale is the reading of how the 8-bit range is fitted to each row)."""
    return (e4m3_to_float(codes, np.float64) * np.asarray(scale, dtype=np.float64)[..., None]).astype(dtype)


def rms_norm(v: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: v * g / sqrt(mean(v^2) + eps)."""
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v * g / np.sqrt(ms + v.dtype.type(eps))


def rope_cos_sin(positions, head_dim: int, theta: float, dtype) -> tuple[np.ndarray, np.ndarray]:
    """cos/sin tables [len(positions), head_dim/2]; angles formed in float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = np.power(np.float64(theta), -2.0 * i / head_dim)
    ang = np.asarray(positions, dtype=np.float64).reshape(-1, 1) * inv[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def apply_rope(v: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE on the last axis: pair (i, i + d/2) is rotated by angle_i."""
    h = v.shape[-1] // 2
    a, b = v[..., :h], v[..., h:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (z.dtype.type(1) + np.exp(-z))


def linear(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Bias-free projection with W stored [out, in]: y[..., i] = sum_j W[i, j] x[..., j]."""
    return x @ W.T


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """SwiGLU gating: silu applied to the gate branch, times the up branch."""
    return silu(gate) * up


def attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray) -> np.ndarray:
    """Decode attention of one new position over cached positions 0..p.

    q: [B, nq, d]; keys, vals: [B, nkv, p+1, d]. Query head h reads KV head
    h // (nq / nkv); scores are q.k / sqrt(d); softmax over positions.
    Returns [B, nq, d].
    """
    B, nq, d = q.shape
    group = nq // keys.shape[1]
    scale = q.dtype.type(1.0 / np.sqrt(d))
    o = np.empty_like(q)
    for h in range(nq):
        g = h // group
        scores = np.einsum("btd,bd->bt", keys[:, g], q[:, h]) * scale
        o[:, h] = np.einsum("bt,btd->bd", softmax(scores), vals[:, g])
    return o


# ----------------------------------------------------------------------------- weights

@dataclass
class _Stack:
    n_layers: int
    hidden: int
    nq: int
    nkv: int
    d: int
    ffn: int
    vocab: int
    layers: list = field(default_factory=list)
    final_norm: np.ndarray | None = None


@dataclass
class OracleState:
    """Per-utterance decode state for B lockstep streams."""
    talker_k: list
    talker_v: list
    pos: int = 0            # next Talker position to be written
    h_T: np.ndarray | None = None


class OracleModel:
    """Talker + CodePredictor in a working dtype (np.float64 or np.float32).

    ``weights`` maps the canonical tensor names to arrays: float32 for fp32
    models, uint16 bf16 bit patterns for bf16 models; fp8 models give the
    projection matrices as uint8 E4M3 codes with a float32 '<name>.scale' per
    output row (everything else bf16), and the oracle runs on the matrices
    they stand for (``dequant_rows``). ``cfg`` is a plain dict
    with keys talker / codepred (n_layers, hidden, n_q_heads, n_kv_heads,
    head_dim, ffn, vocab), text_vocab, n_acoustic, rms_eps, rope_theta,
    weight_dtype.
    """

    def __init__(self, weights: dict, cfg: dict, dtype=np.float64):
        self.dtype = np.dtype(dtype)
        self.eps = float(cfg["rms_eps"])
        self.theta = float(cfg["rope_theta"])
        self.n_ac = int(cfg["n_acoustic"])
        wd = cfg["weight_dtype"]

        def cvt(name):
            a = weights[name]
            if wd == "fp8" and name + ".scale" in weights:
                return dequant_rows(a, weights[name + ".scale"], self.dtype)
            if np.asarray(a).dtype == np.uint8:
                raise KeyError(f"{name}: E4M3 codes without '{name}.scale'")
            return bf16_bits_to_float(a, self.dtype) if wd in ("bf16", "fp8") else np.asarray(a, dtype=self.dtype)

        def stack(prefix, s):
            st = _Stack(s["n_layers"], s["hidden"], s["n_q_heads"], s["n_kv_heads"], s["head_dim"], s["ffn"], s["vocab"])
            for i in range(st.n_layers):
                p = f"{prefix}.layers.{i}."
                st.layers.append({k: cvt(p + k) for k in
                                  ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "mlp_norm", "wg", "wu", "wd")})
            st.final_norm = cvt(prefix + ".final_norm")
            return st

        self.talker = stack("talker", cfg["talker"])
        self.cp = stack("cp", cfg["codepred"])
        self.embed_text = cvt("talker.embed_text")
        self.embed_sem = cvt("talker.embed_sem")
        self.lm_head = cvt("talker.lm_head")
        self.proj = cvt("cp.proj") if "cp.proj" in weights else None
        self.embed_ac = cvt("cp.embed_ac")
        self.heads = cvt("cp.heads")

    # ------------------------------------------------------------------ one block, one position

    def _block_step(self, s: _Stack, L: dict, x: np.ndarray, p: int, kc: np.ndarray, vc: np.ndarray) -> np.ndarray:
        """One decoder layer at position p for B streams; appends k, v at p."""
        B = x.shape[0]
        xn = rms_norm(x, L["attn_norm"], self.eps)
        q = linear(xn, L["wq"]).reshape(B, s.nq, s.d)
        k = linear(xn, L["wk"]).reshape(B, s.nkv, s.d)
        v = linear(xn, L["wv"]).reshape(B, s.nkv, s.d)
        q = rms_norm(q, L["q_norm"], self.eps)
        k = rms_norm(k, L["k_norm"], self.eps)
        cos, sin = rope_cos_sin([p], s.d, self.theta, self.dtype)
        q = apply_rope(q, cos, sin)
        k = apply_rope(k, cos, sin)
        kc[:, :, p, :] = k
        vc[:, :, p, :] = v
        o = attend(q, kc[:, :, : p + 1, :], vc[:, :, : p + 1, :])
        x = x + linear(o.reshape(B, s.nq * s.d), L["wo"])
        xn2 = rms_norm(x, L["mlp_norm"], self.eps)
        x = x + linear(swiglu(linear(xn2, L["wg"]), linear(xn2, L["wu"])), L["wd"])
        return x

    def _stack_step(self, s: _Stack, x: np.ndarray, p: int, kcs: list, vcs: list) -> np.ndarray:
        for L, kc, vc in zip(s.layers, kcs, vcs):
            x = self._block_step(s, L, x, p, kc, vc)
        return rms_norm(x, s.final_norm, self.eps)

    def _cache(self, s: _Stack, B: int, cap: int):
        ks = [np.zeros((B, s.nkv, cap, s.d), dtype=self.dtype) for _ in range(s.n_layers)]
        vs = [np.zeros((B, s.nkv, cap, s.d), dtype=self.dtype) for _ in range(s.n_layers)]
        return ks, vs

    # ------------------------------------------------------------------ the method's calls

    def new_state(self, batch: int, capacity: int) -> OracleState:
        ks, vs = self._cache(self.talker, batch, capacity)
        return OracleState(ks, vs)

    def embed_sum(self, codes: np.ndarray) -> np.ndarray:
        """Talker input from one frame's codes [B, 16]: E_sem[s] + sum_j E_ac[j][a_j]."""
        x = self.embed_sem[codes[:, 0]].copy()
        for j in range(1, self.n_ac + 1):
            x = x + self.embed_ac[j - 1][codes[:, j]]
        return x

    def prefill(self, st: OracleState, ids: np.ndarray) -> np.ndarray:
        """Run the Talker over text ids [B, n] at positions 0..n-1; return frame-0 logits."""
        ids = np.asarray(ids)
        h = None
        for p in range(ids.shape[1]):
            h = self._stack_step(self.talker, self.embed_text[ids[:, p]], p, st.talker_k, st.talker_v)
        st.pos = ids.shape[1]
        st.h_T = h
        return linear(h, self.lm_head)

    def text_rows(self, text_ids: np.ndarray) -> np.ndarray:
        """Streaming text term per stream: E_text[id], or zeros where id < 0 (no text left)."""
        text_ids = np.asarray(text_ids)
        rows = self.embed_text[np.maximum(text_ids, 0)].copy()
        rows[text_ids < 0] = 0
        return rows

    def talker_step(self, st: OracleState, prev_codes: np.ndarray, text_ids: np.ndarray | None = None) -> np.ndarray:
        """One Talker step fed with the previous frame's 16 codes (plus, when text_ids [B] is
        given, the streaming text row E_text[id] of each stream with id >= 0); returns semantic
        logits."""
        x = self.embed_sum(np.asarray(prev_codes))
        if text_ids is not None:
            x = x + self.text_rows(text_ids)
        h = self._stack_step(self.talker, x, st.pos, st.talker_k, st.talker_v)
        st.pos += 1
        st.h_T = h
        return linear(h, self.lm_head)

    def _cp_in(self, v: np.ndarray) -> np.ndarray:
        return v if self.proj is None else linear(v, self.proj)

    def codepred_frame(self, st: OracleState, semantic: np.ndarray, sampling: dict, u: np.ndarray,
                       forced: np.ndarray | None = None, sampler_dtype=np.float64):
        """15 CodePredictor steps for one frame. u: [B, 15]; forced: [B, 15] or None.

        forced[:, j-1] replaces the drawn a_j as the input of step j+1; the
        drawn tokens and all logits are still returned.
        """
        semantic = np.asarray(semantic)
        B = semantic.shape[0]
        ks, vs = self._cache(self.cp, B, self.n_ac + 1)
        self._stack_step(self.cp, self._cp_in(st.h_T), 0, ks, vs)
        out = self._stack_step(self.cp, self._cp_in(self.embed_sem[semantic]), 1, ks, vs)
        codes = np.zeros((B, self.n_ac), dtype=np.int32)
        logits = np.zeros((B, self.n_ac, self.cp.vocab), dtype=self.dtype)
        for j in range(1, self.n_ac + 1):
            if j >= 2:
                prev = forced[:, j - 2] if forced is not None else codes[:, j - 2]
                out = self._stack_step(self.cp, self._cp_in(self.embed_ac[j - 2][prev]), j, ks, vs)
            lg = linear(out, self.heads[j - 1])
            logits[:, j - 1] = lg
            codes[:, j - 1] = sample_rows(lg, sampling, u[:, j - 1], None, dtype=sampler_dtype)
        return codes, logits

    def stream_text_ids(self, ids: np.ndarray, lookahead: int, t: int) -> np.ndarray:
        """Text ids [B] the Talker step of frame t >= 1 adds in streaming mode (-1: none)."""
        ids = np.asarray(ids)
        j = lookahead + t - 1
        return ids[:, j] if j < ids.shape[1] else np.full(ids.shape[0], -1, dtype=ids.dtype)

    def generate(self, ids: np.ndarray, frames: int, sem_sampling: dict, ac_sampling: dict,
                 uniforms: np.ndarray, teacher: np.ndarray | None = None, keep_logits: bool = True,
                 keep_hidden: bool = False, sampler_dtype=np.float64, text_lookahead: int | None = None,
                 lengths=None, eos_id: int | None = None) -> dict:
        """Prefill then ``frames`` frames. uniforms: [B, >=frames, 16].

        teacher: [B, frames, 16] codes to feed forward instead of the drawn ones
        (teacher forcing); drawn tokens and logits are still reported.
        text_lookahead: streaming mode with that many text ids in the prefill, the rest
        fed one per frame (see the module docstring); None = all ids in the prefill.
        lengths: per-stream prompt lengths (stream b's prompt is ids[b, :lengths[b]]); each
        stream then runs on its own. eos_id: the per-stream stop (see the module docstring);
        out["stop"] [B] holds each stream's stop frame or -1.
        """
        ids = np.asarray(ids)
        B = ids.shape[0]
        if lengths is not None:
            if text_lookahead is not None:
                raise ValueError("lengths and text_lookahead do not combine")
            parts = [self.generate(ids[b:b + 1, :int(lengths[b])], frames, sem_sampling, ac_sampling, uniforms[b:b + 1],
                                   None if teacher is None else teacher[b:b + 1], keep_logits, keep_hidden, sampler_dtype,
                                   eos_id=eos_id) for b in range(B)]
            return {k: np.concatenate([q[k] for q in parts], axis=0) for k in parts[0]}
        L = ids.shape[1] if text_lookahead is None else int(text_lookahead)
        if not 1 <= L <= ids.shape[1]:
            raise ValueError("text_lookahead must lie in [1, n]")
        st = self.new_state(B, L + frames)
        logits = self.prefill(st, ids[:, :L])
        history = np.zeros((B, self.talker.vocab), dtype=bool)
        codes = np.zeros((B, frames, 1 + self.n_ac), dtype=np.int32)  # as drawn
        stop = np.full(B, -1, dtype=np.int64)
        out = {"codes": codes}
        if keep_logits:
            out["sem_logits"] = np.zeros((B, frames, self.talker.vocab), dtype=self.dtype)
            out["ac_logits"] = np.zeros((B, frames, self.n_ac, self.cp.vocab), dtype=self.dtype)
        if keep_hidden:
            out["h_T"] = np.zeros((B, frames, self.talker.hidden), dtype=self.dtype)
        rows = np.arange(B)
        for t in range(frames):
            if t > 0:
                prev = teacher[:, t - 1] if teacher is not None else codes[:, t - 1]
                text = self.stream_text_ids(ids, L, t) if L < ids.shape[1] else None
                logits = self.talker_step(st, prev, text)
            if keep_logits:
                out["sem_logits"][:, t] = logits
            if keep_hidden:
                out["h_T"][:, t] = st.h_T
            s = sample_rows(logits, sem_sampling, uniforms[:, t, 0], history, dtype=sampler_dtype)
            codes[:, t, 0] = s
            s_in = teacher[:, t, 0] if teacher is not None else s
            history[rows, s_in] = True
            forced = teacher[:, t, 1:] if teacher is not None else None
            a, lg = self.codepred_frame(st, s_in, ac_sampling, uniforms[:, t, 1:], forced, sampler_dtype)
            codes[:, t, 1:] = a
            if keep_logits:
                out["ac_logits"][:, t] = lg
            if eos_id is not None:
                for b in range(B):
                    if stop[b] < 0 and codes[b, t, 0] == eos_id:
                        stop[b] = t
        if eos_id is not None:
            shown = codes.copy()
            for b in range(B):
                if stop[b] >= 0:
                    shown[b, stop[b], 1:] = -1
                    shown[b, stop[b] + 1:] = -1
            out["codes"] = shown
            out["stop"] = stop
        return out

    # ------------------------------------------------------------------ brute force (no cache)

    def full_forward(self, which: str, X: np.ndarray) -> np.ndarray:
        """Whole-sequence causal forward of a stack without any KV cache.

        X: [B, S, H] inputs at positions 0..S-1. Returns the final-normed
        outputs [B, S, H]. Written independently of the cached path: all
        positions at once, explicit causal mask, KV heads expanded by repeat.
        """
        s = self.talker if which == "talker" else self.cp
        B, S, _ = X.shape
        cos, sin = rope_cos_sin(np.arange(S), s.d, self.theta, self.dtype)
        cos, sin = cos[None, :, None, :], sin[None, :, None, :]
        causal = np.tril(np.ones((S, S), dtype=bool))
        rep = s.nq // s.nkv
        x = np.asarray(X, dtype=self.dtype)
        for L in s.layers:
            xn = rms_norm(x, L["attn_norm"], self.eps)
            Q = rms_norm(linear(xn, L["wq"]).reshape(B, S, s.nq, s.d), L["q_norm"], self.eps)
            K = rms_norm(linear(xn, L["wk"]).reshape(B, S, s.nkv, s.d), L["k_norm"], self.eps)
            V = linear(xn, L["wv"]).reshape(B, S, s.nkv, s.d)
            Q = apply_rope(Q, cos, sin).transpose(0, 2, 1, 3)                       # [B, nq, S, d]
            K = np.repeat(apply_rope(K, cos, sin), rep, axis=2).transpose(0, 2, 3, 1)  # [B, nq, d, S]
            V = np.repeat(V, rep, axis=2).transpose(0, 2, 1, 3)                       # [B, nq, S, d]
            scores = np.matmul(Q, K) / self.dtype.type(np.sqrt(s.d))
            scores = np.where(causal[None, None], scores, -np.inf)
            O = np.matmul(softmax(scores), V).transpose(0, 2, 1, 3).reshape(B, S, s.nq * s.d)
            x = x + linear(O, L["wo"])
            xn2 = rms_norm(x, L["mlp_norm"], self.eps)
            x = x + linear(swiglu(linear(xn2, L["wg"]), linear(xn2, L["wu"])), L["wd"])
        return rms_norm(x, s.final_norm, self.eps)
