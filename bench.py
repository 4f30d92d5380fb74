"""Frame-decode benchmark: acoustic frames/s and RTF at batch 1 (1.7B-class).

A step is one acoustic frame: draw the semantic token, 15 CodePredictor
steps, and the Talker step that consumes the frame's codes -- one replay of
the captured frame graph. The workload follows the 1.7B-class config: seeded
bf16 weights, prefill of 64 random text ids, greedy frames at batch 1.

    python bench.py [--steps K] [--warmup W] [--workload 1.7b] [--reps R] [--extra LIST]

Protocol: one full run (prefill + W + K frames) is discarded; then R runs,
each a prefill, W untimed frames and K frames timed with HIP events on the
decoder's stream. ``value`` is the median frames/s; the slowest run (the p90
at 5 runs) is reported beside it, with the GPU clock and temperature read
after every run. The other configs named in --extra run the same protocol on
their own workloads (W = 16, K = the rest of their frames) and are reported
under ``extra``. Prints one JSON line. The oracle (plain NumPy) is timed on a
bounded sample of the same workload on the host cores as ``cpu_baseline``. Each roofline fraction
is also given against the box's measured device-copy bandwidth (``copy_bandwidth``,
``frac_of_copy``).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

METRIC = "acoustic frames/sec (RTF) at batch 1, 1.7B-class; % of HBM roofline"
EXTRA_WARMUP = 16


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=224, help="timed frames per run")
    p.add_argument("--warmup", type=int, default=16, help="untimed frames before the timed ones")
    p.add_argument("--reps", type=int, default=5, help="timed runs (prefill + warmup + timed); median and max reported")
    p.add_argument("--workload", default="1.7b")
    p.add_argument("--extra", default="0.6b,1.7b-sampled,1.7b-x32,1.7b-long",
                   help="comma-separated workloads also timed, each on its own frame count ('' for none)")
    p.add_argument("--cpu-frames", type=int, default=200, help="frames of the oracle CPU baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--ragged", action="store_true",
                   help="prompt lengths drawn per stream (seed 7) from [prefill/4, prefill], prefilled ragged")
    p.add_argument("--exec", default="auto", choices=["auto", "kernels"],
                   help="auto: the persistent step kernels where the config allows them; kernels: per-op kernels only")
    p.add_argument("--kernel-iters", type=int, default=40,
                   help="back-to-back launches of the dominant kernel timed for the roofline")
    return p.parse_args()


# ---------------------------------------------------------------------------- host / device facts

def cpu_facts() -> dict:
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0))}


class Smi:
    """GPU clock and temperature through the amdsmi library (read-only queries); None when the
    library or a query is unavailable."""

    def __init__(self):
        self.h = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            hs = amdsmi.amdsmi_get_processor_handles()
            self.smi, self.h = amdsmi, (hs[0] if hs else None)
        except Exception as e:  # noqa: BLE001 - reported, never fatal
            self.err = f"{type(e).__name__}: {e}"

    def sample(self) -> dict:
        if self.h is None:
            return {"error": getattr(self, "err", "no device handle")}
        out = {}
        s = self.smi
        for key, fn in (("gfx_clock_mhz", lambda: s.amdsmi_get_clock_info(self.h, s.AmdSmiClkType.GFX)),
                        ("mem_clock_mhz", lambda: s.amdsmi_get_clock_info(self.h, s.AmdSmiClkType.MEM))):
            try:
                info = fn()
                out[key] = info.get("clk", info.get("cur_clk")) if isinstance(info, dict) else info
            except Exception as e:  # noqa: BLE001
                out[key] = None
                out.setdefault("errors", []).append(f"{key}: {type(e).__name__}")
        for key, typ in (("temp_hotspot_c", "HOTSPOT"), ("temp_mem_c", "VRAM"), ("temp_edge_c", "EDGE")):
            try:
                out[key] = s.amdsmi_get_temp_metric(self.h, getattr(s.AmdSmiTemperatureType, typ),
                                                    s.AmdSmiTemperatureMetric.CURRENT)
            except Exception as e:  # noqa: BLE001
                out[key] = None
        return out

    def close(self):
        if self.h is not None:
            try:
                self.smi.amdsmi_shut_down()
            except Exception:  # noqa: BLE001
                pass


# ---------------------------------------------------------------------------- CPU baseline

def cpu_baseline(wl, weights, frames: int) -> dict:
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import OracleModel
    from autoregressive_tts_decode_amd import synth

    cores = len(os.sched_getaffinity(0))
    model = wl.model
    with threadpool_limits(limits=cores):
        orc = OracleModel(weights, model.as_dict(), np.float32)
        ids = synth.make_text_ids(wl)[:1, :8]
        greedy = {"do_sample": False, "top_k": 0, "top_p": 1.0, "temperature": 1.0, "repetition_penalty": 1.0}
        st = orc.new_state(1, 8 + frames + 1)
        lg = orc.prefill(st, ids)
        t0 = time.perf_counter()
        for _ in range(frames):
            s = int(np.argmax(lg[0]))
            a, _ = orc.codepred_frame(st, np.array([s], np.int32), greedy, np.zeros((1, 15), np.float32))
            lg = orc.talker_step(st, np.concatenate([[[s]], a], axis=1).astype(np.int32))
        dt = time.perf_counter() - t0
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(frames / dt, 4), "unit": "frames/s", "cores": int(threads), "kind": "oracle",
            "rtf": round(12.5 / (frames / dt), 3),
            "sample": f"{model.name}, batch 1, prefill 8 ids, {frames} greedy frames timed (NumPy fp32, "
                      f"weights pre-upcast from the same bf16 values, BLAS threads = {cores} affinity cores), "
                      f"{dt:.1f} s"}


# ---------------------------------------------------------------------------- GPU runs

def copy_bandwidth(mib: int = 1024, reps: int = 10) -> dict:
    """The box's device-to-device copy rate, the practical HBM ceiling beside the 8 TB/s peak: one
    buffer of `mib` MiB copied `reps` times by torch's copy kernel, HIP events around the copies on
    the current stream; bytes moved = bytes read + bytes written."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"gbs": round(2 * n * 4 / t / 1e9, 1), "bytes_per_copy": 2 * n * 4, "reps": reps,
            "note": "torch device copy; read + written bytes over HIP-event time"}


def time_workload(name: str, K: int, W: int, reps: int, smi: Smi, args, weights=None, dominant: bool = False) -> dict:
    """The protocol on one workload: a discarded full run, then `reps` timed runs."""
    import torch
    from autoregressive_tts_decode_amd import config, synth, tts, roofline

    wl = config.WORKLOADS[name]
    model, B = wl.model, wl.batch
    cap = wl.prefill_len + W + K + 1
    d = torch.device("cuda:0")
    if weights is None:
        weights = synth.make_weights(model, wl.weight_seed)
    dw = tts.weights_to_device(weights, model, d)
    dec = tts.TTSDecoder(model, B, cap, W + K)
    dec.load_weights(dw)
    if args.exec == "kernels":
        dec.set_exec_mode(tts.EXEC_KERNELS)
    ids = torch.from_numpy(synth.make_text_ids(wl)).to(d)
    u = torch.from_numpy(synth.make_uniforms(wl, frames=W + K)).to(d)
    codes = torch.zeros((B, W + K, 16), dtype=torch.int32, device=d)
    stream = dec.stream
    lengths = None
    if args.ragged and dominant:
        lengths = np.random.default_rng(7).integers(max(1, wl.prefill_len // 4), wl.prefill_len + 1, B).tolist()

    def one_run(timed: bool):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if lengths is None:
            dec.prefill(ids)
        else:
            dec.prefill_ragged(ids, lengths)
        torch.cuda.synchronize()
        pre = (time.perf_counter() - t0) * 1e3
        if W:
            dec.run_frames(W, wl.semantic, wl.acoustic, u, codes)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dec.run_frames(K, wl.semantic, wl.acoustic, u, codes)
        e1.record(stream)
        torch.cuda.synchronize()
        if dec.device_status() != 0:
            raise RuntimeError(f"{name}: a persistent kernel reported an exchange time-out")
        return e0.elapsed_time(e1) / 1e3, pre

    one_run(False)  # full warm-up run, discarded
    runs = []
    for _ in range(reps):
        t, pre = one_run(True)
        runs.append({"s": t, "prefill_ms": pre, "smi": smi.sample()})
    times = [r["s"] for r in runs]
    t_med, t_max = statistics.median(times), max(times)
    res = {
        "workload": name, "batch": B, "prefill_len": wl.prefill_len, "frames": W + K, "timed_frames": K, "warmup": W,
        "reps": reps,
        "value": round(B * K / t_med, 3), "unit": "frames/s" if B == 1 else "stream-frames/s",
        "ms_per_step": round(t_med / K * 1e3, 4), "ms_per_step_max": round(t_max / K * 1e3, 4),
        "value_at_max": round(B * K / t_max, 3),
        "rtf": round(roofline.rtf_from_fps(K / t_med), 6),
        "prefill_ms": round(statistics.median(r["prefill_ms"] for r in runs), 2),
        "runs": [{"ms_per_step": round(r["s"] / K * 1e3, 4), "prefill_ms": round(r["prefill_ms"], 2), **r["smi"]} for r in runs],
    }
    mode, _ = dec.exec_mode()
    res["exec"] = "persistent" if mode == tts.EXEC_PERSISTENT else "per-op kernels"
    bytes_avg = roofline.frame_bytes_for_run(model, wl.prefill_len, W, K, batch=B, kv_elem_bytes=4) / K
    achieved = bytes_avg * K / t_med / 1e9
    peak = roofline.HBM_PEAK_BYTES_PER_S / 1e9
    res["frame_roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": peak, "unit": "GB/s",
                             "frac": round(achieved / peak, 4),
                             "unit_of_work": "one frame graph replay (all kernels of a frame)",
                             "algorithmic_bytes_per_frame": int(bytes_avg)}
    if lengths is not None:
        res["prompt_lengths"] = {"ragged": True, "min": min(lengths), "max": max(lengths),
                                 "mean": round(sum(lengths) / len(lengths), 1)}
    if dominant:
        tt = model.talker
        res["prefill"] = {"mode": "gemm" if dec.prefill_mode() == tts.PREFILL_GEMM else "steps", "positions": wl.prefill_len,
                          "streams": B,
                          "tflops": round(2.0 * B * wl.prefill_len * tt.n_layers * roofline.layer_weight_elems(tt)
                                          / (res["prefill_ms"] * 1e-3) / 1e12, 2),
                          "note": "algorithmic FLOPs (2 per weight per row) of the Talker prompt pass; wall time includes the head"}
        res["dom"] = None
        if mode == tts.EXEC_PERSISTENT and B == 1:
            # Dominant kernel: the persistent CodePredictor frame kernel (about half of a frame),
            # timed alone with HIP events on the decoder's stream over back-to-back launches.
            sem = torch.zeros((1,), dtype=torch.int32, device=d)
            acodes = torch.zeros((1, 15), dtype=torch.int32, device=d)
            greedy = config.GREEDY.as_dict()
            dec.prefill(ids)
            for _ in range(3):
                dec.codepred_frame(sem, greedy, None, acodes)
            torch.cuda.synchronize()
            k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            k0.record(stream)
            for _ in range(args.kernel_iters):
                dec.codepred_frame(sem, greedy, None, acodes)
            k1.record(stream)
            torch.cuda.synchronize()
            if dec.device_status() != 0:
                raise RuntimeError("persistent CodePredictor kernel reported an exchange time-out")
            dom_s = k0.elapsed_time(k1) / 1e3 / args.kernel_iters
            res["dom"] = (dom_s, roofline.algorithmic_bytes(model, wl.prefill_len + 1, B, 4)["cp_frame"])
        res["peak_memory"] = {"allocated_bytes": int(torch.cuda.max_memory_allocated(d)),
                              "reserved_bytes": int(torch.cuda.max_memory_reserved(d))}
    dec.close()
    del dec, dw
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "the library decodes on one GPU: a batch-1 frame does not shard usefully and "
                                   "independent streams are data parallel with no exchange; run with --gpus 1"}))
        sys.exit(2)

    import torch
    from autoregressive_tts_decode_amd import config, synth, tts, roofline

    tts.load_library()  # fails loudly when the HIP library is missing
    wl = config.WORKLOADS[args.workload]
    model, B = wl.model, wl.batch
    K, W = args.steps, args.warmup
    smi = Smi()
    weights = synth.make_weights(model, wl.weight_seed)
    head = time_workload(args.workload, K, W, args.reps, smi, args, weights=weights, dominant=True)
    peak = roofline.HBM_PEAK_BYTES_PER_S / 1e9
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8_e4m3 weights, f32 arithmetic", "fp32": "f32"}[model.weight_dtype],
        "data": "synthetic",
        "config": {"workload": f"{model.name}: Talker 28x2048 (16q/8kv heads, d128, FFN 6144, Vs 3072) + "
                               f"CodePredictor 5x1024 (FFN 3072, 15 heads x 2048); batch {B}, prefill "
                               f"{wl.prefill_len} ids, {W + K} frames ({'sampled' if wl.semantic.do_sample else 'greedy'})"
                   if args.workload.startswith("1.7b") else f"{model.name}; batch {B}, prefill {wl.prefill_len}, {W + K} frames",
                   "batch": B, "prefill_len": wl.prefill_len, "frames": W + K, "timed_frames": K,
                   "exec": head["exec"], "kv_cache": "fp32"},
        "rtf": head["rtf"],
        "reps": args.reps,
        "ms_per_step_max": head["ms_per_step_max"],
        "value_at_max": head["value_at_max"],
        "runs": head["runs"],
        "prefill_ms": head["prefill_ms"],
        "prefill": head["prefill"],
        "frame_roofline": head["frame_roofline"],
        "peak_memory": head["peak_memory"],
        "host": cpu_facts(),
    }
    if "prompt_lengths" in head:
        out["config"]["prompt_lengths"] = head["prompt_lengths"]
    cbw = copy_bandwidth()
    out["copy_bandwidth"] = cbw
    out["frame_roofline"]["frac_of_copy"] = round(out["frame_roofline"]["achieved"] / cbw["gbs"], 4)
    if head["dom"] is not None:
        dom_s, dom_bytes = head["dom"]
        a_gbs = dom_bytes / dom_s / 1e9
        # HBM bytes per launch from the committed counter record (null once the kernel changed)
        traffic = roofline.measured_traffic("k_cp_frame_1.7b_b1_hbm_traffic.md") if args.workload == "1.7b" else None
        out["roofline"] = {"bound": "hbm", "achieved": round(a_gbs, 1), "peak": peak, "unit": "GB/s",
                           "frac": round(a_gbs / peak, 4), "traffic": traffic,
                           "kernel": "k_cp_frame (persistent CodePredictor frame: 15 steps)",
                           "avg_launch_us": round(dom_s * 1e6, 2), "algorithmic_bytes_per_launch": int(dom_bytes),
                           "frac_of_copy": round(a_gbs / cbw["gbs"], 4)}
    else:
        out["roofline"] = dict(head["frame_roofline"], traffic=None)
    extra = {}
    for name in [x for x in args.extra.split(",") if x and x != args.workload]:
        ewl = config.WORKLOADS[name]
        ew = weights if ewl.model is model and ewl.weight_seed == wl.weight_seed else None
        r = time_workload(name, ewl.frames - EXTRA_WARMUP, EXTRA_WARMUP, args.reps, smi, args, weights=ew)
        extra[name] = {k: r[k] for k in ("value", "unit", "value_at_max", "ms_per_step", "ms_per_step_max", "rtf",
                                         "batch", "prefill_len", "frames", "timed_frames", "reps", "exec",
                                         "prefill_ms", "frame_roofline", "runs")}
    if extra:
        out["extra"] = extra
    smi.close()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, weights, args.cpu_frames)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
