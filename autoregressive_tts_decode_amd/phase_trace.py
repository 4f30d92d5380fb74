"""Per-phase timeline of the two persistent kernels of one frame.

    python -m autoregressive_tts_decode_amd.phase_trace [--workload 1.7b] [--frames-before 4] [--save FILE.npy]

Loads libtts_trace.so (the library built with TTS_PHASE_TRACE: thread 0 of every workgroup
stamps (label, 100 MHz wall clock) at each phase boundary), decodes a few frames to warm up,
records one frame, and prints for each kernel the time between consecutive stamps, averaged over
the 256 workgroups and summed over the layers, largest first. "skew" is the spread of the later
stamp across the workgroups. The stamps cost time of their own (a traced frame runs roughly a
fifth slower), so the table apportions the frame; the untraced kernel times come from the bench.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys
from collections import defaultdict

import numpy as np

from . import config, synth, tts
from .build import TRACE_LIB

TRACE_WG, TRACE_PER = 256, 4096
CP_BASE, TALKER_BASE = 0, 2048

# labels as the kernels stamp them
CP_LABELS = {
    1: "start", 2: "constants+tiles issued", 3: "end",
    40: "step", 41: "step input", 10: "layer", 11: "q/k/v published", 13: "q/k/v gathered", 14: "attention",
    15: "gate/up published", 16: "SwiGLU gathered", 20: "reduce published", 21: "after-publish issue",
    22: "reduce-scatter got", 23: "all-gather published", 24: "all-gather got", 42: "head dot", 43: "token",
    44: "logits gathered", 45: "top-k bound found", 46: "kept keys placed",
}
TALKER_LABELS = {
    49: "start", 50: "layer", 51: "q/k/v dots", 52: "q/k/v gathered", 53: "q/k prepared", 54: "attention chunk",
    55: "partial published", 56: "partials combined", 57: "outputs gathered", 58: "out-proj dot",
    59: "out-proj reduced", 60: "gate/up LDS dot", 61: "gate/up register dots", 62: "SwiGLU gathered",
    63: "down dot", 64: "layers done", 65: "head",
}


def phase_table(buf: np.ndarray, lo: int, hi: int, labels: dict) -> list[str]:
    """Rows 'from -> to: total us, share, count, average us, skew us' for stamps [lo, hi)."""
    lab, ts = [], []
    for b in range(TRACE_WG):
        row = buf[b, lo:hi]
        row = row[row != 0]
        lab.append((row >> 48).astype(int))
        ts.append((row & ((1 << 48) - 1)).astype(np.int64))
    n = min(len(x) for x in lab)
    if n < 2:
        return ["(no stamps)"]
    L = lab[0][:n]
    if not all((x[:n] == L).all() for x in lab):
        return ["(workgroups stamped different sequences)"]
    T = np.stack([t[:n] for t in ts]) * 0.01  # 100 MHz ticks -> us
    acc, skew = defaultdict(list), defaultdict(list)
    for i in range(1, n):
        acc[(L[i - 1], L[i])].append(float((T[:, i] - T[:, i - 1]).mean()))
        skew[L[i]].append(float(T[:, i].max() - T[:, i].min()))
    tot = sum(sum(v) for v in acc.values())
    out = [f"{n} stamps, span {float(np.mean(T[:, -1] - T[:, 0])):.1f} us",
           f"{'from':>24} -> {'to':<24} {'total us':>9} {'share':>6} {'n':>4} {'avg us':>7} {'skew us':>7}"]
    for k in sorted(acc, key=lambda k: -sum(acc[k])):
        v = acc[k]
        out.append(f"{labels.get(k[0], k[0]):>24} -> {labels.get(k[1], k[1]):<24} {sum(v):9.1f} {100 * sum(v) / tot:5.1f}% "
                   f"{len(v):4d} {np.mean(v):7.3f} {np.mean(skew[k[1]]):7.2f}")
    return out


def main(argv=None) -> int:
    import torch

    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="1.7b")
    ap.add_argument("--frames-before", type=int, default=4)
    ap.add_argument("--save", default="")
    ap.add_argument("--lib", default=TRACE_LIB, help="a library built with TTS_PHASE_TRACE")
    args = ap.parse_args(argv)
    if not os.path.exists(args.lib):
        raise RuntimeError(f"{args.lib} not built: python -m autoregressive_tts_decode_amd.build")
    lib = tts.load_library(args.lib)
    lib.tts_trace_ctl.argtypes = [ctypes.c_int, ctypes.c_void_p]
    wl = config.WORKLOADS[args.workload]
    d = torch.device("cuda:0")
    w = synth.make_weights(wl.model, wl.weight_seed)
    F = args.frames_before + 1
    dec = tts.TTSDecoder(wl.model, 1, wl.prefill_len + F + 2, F)
    dec.load_weights(tts.weights_to_device(w, wl.model, d))
    ids = torch.from_numpy(synth.make_text_ids(wl)).to(d)
    u = torch.from_numpy(synth.make_uniforms(wl, frames=F)).to(d)
    codes = torch.zeros((1, F, 16), dtype=torch.int32, device=d)
    dec.prefill(ids)
    dec.run_frames(args.frames_before, wl.semantic, wl.acoustic, u, codes)
    torch.cuda.synchronize()
    if lib.tts_trace_ctl(1, None) != 0:
        raise RuntimeError("tts_trace_ctl failed")
    dec.run_frames(1, wl.semantic, wl.acoustic, u, codes)
    torch.cuda.synchronize()
    buf = np.zeros((TRACE_WG, TRACE_PER), np.int64)
    if lib.tts_trace_ctl(0, buf.ctypes.data) != 0:
        raise RuntimeError("tts_trace_ctl failed")
    if dec.device_status() != 0:
        raise RuntimeError("a persistent kernel reported an exchange time-out")
    dec.close()
    if args.save:
        np.save(args.save, buf)
    print(f"{wl.model.name}: frame {args.frames_before} after a {wl.prefill_len}-id prefill (traced build)")
    print("\n== CodePredictor frame kernel (15 steps)")
    print("\n".join(phase_table(buf, CP_BASE, TALKER_BASE, CP_LABELS)))
    print("\n== Talker step kernel")
    print("\n".join(phase_table(buf, TALKER_BASE, TRACE_PER, TALKER_LABELS)))
    return 0


if __name__ == "__main__":
    sys.exit(main())
