"""Benchmark of the SplitZip BF16 codec on one MI355X.

One step = the whole hot path over one tensor already resident in HBM:
exponent histogram -> top-16 codebook -> pack (encode), then unpack ->
escape scatter (decode).  Every pass is bracketed by HIP events on the
stream the kernels run on, so each kernel's average duration is measured
inside the timed region.  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload llama3_8b_kv_8k]

Throughput is uncompressed bytes (2 per BF16 word) per second.  The
roofline object describes the kernel with the longest average duration:
algorithmic bytes per launch / average launch time, against the MI355X's
8 TB/s HBM peak.  ``traffic`` (HBM bytes per launch from rocprofv3 FETCH_SIZE
and WRITE_SIZE, scaled by what the same counters read for a copy of known
size) comes from profiles/traffic.json and is reported only while the kernel
sources still hash to the value recorded there.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCES = ["lossless_bf16_kv_split_amd/csrc/encode.hip",
                  "lossless_bf16_kv_split_amd/csrc/decode.hip",
                  "lossless_bf16_kv_split_amd/csrc/sz_internal.h"]
PASSES = ["histogram", "codebook", "pack", "unpack", "scatter"]
KERNEL_NAMES = {"histogram": "k_histogram", "codebook": "k_merge_rows+k_select",
                "pack": "k_pack", "unpack": "k_unpack", "scatter": "k_scatter"}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(n: int, e: int) -> dict:
    """Bytes each pass must move (per launch), from the container layout:
    nibbles ceil(n/2), sign|mantissa n, escapes 5e, header+codebook 176."""
    nib, sm, esc, pre = (n + 1) // 2, n, 5 * e, 176
    return {
        "histogram": 2 * n,                        # read every word once
        "codebook": 0,                             # O(chunks) metadata only
        "pack": 2 * n + nib + sm + esc + pre,      # read words, write container
        "unpack": pre + nib + sm + 2 * n,          # read codes + sm, write words
        "scatter": esc + 3 * e,                    # read records; sm read + word write per escape
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(words, repeats: int) -> dict:
    """The CPU oracle as it stands (single-threaded C), on the same input."""
    import numpy as np
    import oracle
    n = words.size
    dst = np.empty(oracle.max_compressed_size(n), dtype=np.uint8)
    out = np.empty(n, dtype=np.uint16)
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        size = oracle.encode_into(words, dst)
        t1 = time.perf_counter()
        st, _ = oracle.decode_status(dst[:size], n, out)
        t2 = time.perf_counter()
        assert st == 0
        times.append((t1 - t0, t2 - t1))
    enc = statistics.median(t[0] for t in times)
    dec = statistics.median(t[1] for t in times)
    return {
        "value": round(2 * n / (enc + dec) / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"whole workload ({n} words), encode+decode, median of {repeats}; "
                  f"{cpu_model()}, 1 of {os.cpu_count()} host threads",
        "encode_GBps": round(2 * n / enc / 1e9, 4),
        "decode_GBps": round(2 * n / dec / 1e9, 4),
    }


def load_traffic(kernel: str, workload: str) -> float | None:
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash() or t.get("workload") != workload:
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b_kv_8k")
    ap.add_argument("--cpu-repeats", type=int, default=2,
                    help="oracle runs for the CPU baseline (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run one device copy of known size (for PMC scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the codec runs on a single MI355X and this "
              "build has no multi-GPU path (use --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import kvgen
    import lossless_bf16_kv_split_amd as sz

    w = kvgen.resolve(args.workload)
    torch.cuda.set_device(0)
    words = kvgen.generate(w.name)
    n = words.size
    x = torch.from_numpy(words.view(np.int16)).cuda()
    cap = sz.sz_max_compressed_size(n)
    ws_bytes = sz.sz_workspace_size(n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(cap, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    # container size is known after one encode; decode needs it on the host
    sz.sz_encode(x, n, dst, cap, size, stream)
    total = int(size.item())
    container = dst[:total]
    e = int.from_bytes(container[16:24].cpu().numpy().tobytes(), "little")

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        sz.sz_encode_histogram(x, n, ws, ws_bytes, stream)
        if ev:
            ev[1].record(stream)
        sz.sz_encode_codebook(n, ws, ws_bytes, dst, cap, size, stream)
        if ev:
            ev[2].record(stream)
        sz.sz_encode_pack(x, n, ws, ws_bytes, dst, cap, stream)
        if ev:
            ev[3].record(stream)
        sz.sz_decode_unpack(container, total, out, n, status, stream)
        if ev:
            ev[4].record(stream)
        sz.sz_decode_scatter(container, total, out, n, status, stream)
        if ev:
            ev[5].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        step(events[k])
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(stop)

    per = {p: [] for p in PASSES}
    for ev in events:
        for i, p in enumerate(PASSES):
            per[p].append(ev[i].elapsed_time(ev[i + 1]))
    avg_ms = {p: sum(v) / len(v) for p, v in per.items()}

    # the timed work is correct: same container, exact round trip
    ok = bool(torch.equal(out, x)) and int(status.item()) == 0 and int(size.item()) == total

    alg = algorithmic_bytes(n, e)
    kernels = {}
    for p in PASSES:
        ms = avg_ms[p]
        gbps = alg[p] / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
        kernels[p] = {"kernel": KERNEL_NAMES[p], "avg_ms": round(ms, 5),
                      "alg_bytes": alg[p], "GBps": round(gbps, 1),
                      "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4)}
    enc_ms = avg_ms["histogram"] + avg_ms["codebook"] + avg_ms["pack"]
    dec_ms = avg_ms["unpack"] + avg_ms["scatter"]
    enc_alg = alg["histogram"] + alg["pack"]
    dec_alg = alg["unpack"] + (5 * e)
    ms_per_step = total_ms / args.steps

    dominant = max(["histogram", "pack", "unpack", "scatter"], key=lambda p: avg_ms[p])
    ach = kernels[dominant]["GBps"]
    traffic = load_traffic(KERNEL_NAMES[dominant], w.name)

    copy_ms = None
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        b.copy_(a)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_ms = c0.elapsed_time(c1)
        del a, b

    line = {
        "metric": "encode/decode GB/s (uncompressed) + compression ratio; % of HBM peak, 1 GPU",
        "value": round(2 * n / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16",
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "n_elements": n,
                   "input_bytes": 2 * n, "seed": w.seed},
        "encode_GBps": round(2 * n / (enc_ms * 1e-3) / 1e9, 2),
        "decode_GBps": round(2 * n / (dec_ms * 1e-3) / 1e9, 2),
        "encode_frac_hbm": round(enc_alg / (enc_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "decode_frac_hbm": round(dec_alg / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "ratio": round(2 * n / total, 5),
        "escapes": e,
        "container_bytes": total,
        "round_trip_ok": ok,
        "kernels": kernels,
        "roofline": {"bound": "hbm", "kernel": KERNEL_NAMES[dominant], "achieved": ach,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": traffic},
        "kernel_source_hash": kernel_source_hash(),
        "wall_s_timed": round(t_wall, 4),
        "context": {"pages_compress_GBps": 613, "pages_decompress_GBps": 2181,
                    "pages_hardware": "not stated"},
    }
    if copy_ms is not None:
        line["copy_1GiB_ms"] = round(copy_ms, 4)
        line["copy_GBps_rw"] = round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9, 1)
    if args.cpu_repeats > 0:
        line["cpu_baseline"] = cpu_baseline(words, args.cpu_repeats)
    print(json.dumps(line), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
