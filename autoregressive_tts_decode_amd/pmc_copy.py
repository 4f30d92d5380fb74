"""A plain device-to-device copy of known size, the calibration run for HBM byte counters.

    rocprofv3 --pmc FETCH_SIZE -- python3 -m autoregressive_tts_decode_amd.pmc_copy --mib 512

reads and writes exactly --mib MiB once (torch's copy kernel, no library code involved), so the
FETCH_SIZE / WRITE_SIZE a counter run reports for that dispatch, against the known byte count,
gives the factor that turns the same counter's reading for another kernel into HBM bytes.
"""
from __future__ import annotations

import argparse

import torch


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=512)
    a = ap.parse_args()
    n = a.mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    assert torch.equal(dst[-4:], src[-4:])
    print(f"copied {a.mib} MiB ({n * 4} bytes read, {n * 4} bytes written)", flush=True)


if __name__ == "__main__":
    main()
