"""Streaming ceilings of the HBM for the fused Adam update's access shape
(tests/hw/stream_probe.hip): read-only, write-only, copy, and the update's
own stream mixes (4 fp32 reads and 3 writes for fp32 p, m, v, g; 4 and 4),
each without and with the update's limit of 7 resident workgroups per
compute unit.  Prints one JSON line per probe; rates count the algorithmic
bytes (every stream element read or written once).

    python tests/hw/stream_probe.py [--n N] [--launches L]
    python tests/hw/stream_probe.py --summarize-trace DIR --log LOG
        (writes profiles/stream_probe_ceilings.txt from a rocprofv3
        kernel trace of the first form and its printed lines)
"""
import argparse
import ctypes
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIBRARY = os.path.join(HERE, "libstream_probe.so")
HBM_PEAK_GBPS = 8000.0
# (reads, writes): read-only, write-only, copy, 2:2, the fp32 update's 4:3, 4:4
CONFIGS = ((1, 0), (0, 1), (1, 1), (2, 2), (4, 3), (4, 4))
LIMITS = (0, 7)
COMMANDS = {
    "trace": "cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace_probe -o run -- "
             "python3 <repo>/tests/hw/stream_probe.py > <out>/trace_probe.log",
    "summary": "python tests/hw/stream_probe.py --summarize-trace <out>/trace_probe --log <out>/trace_probe.log",
}


def run(n: int, launches: int) -> None:
    import torch

    if not torch.cuda.is_available():
        sys.exit("stream_probe.py needs a GPU")
    lib = ctypes.CDLL(LIBRARY)
    lib.stream_probe_run.restype = ctypes.c_int
    lib.stream_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_void_p),
                                     ctypes.POINTER(ctypes.c_void_p), ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
    max_r = max(r for r, _ in CONFIGS)
    max_w = max(max(w for _, w in CONFIGS), 1)
    ins = [torch.zeros(n, dtype=torch.float32, device="cuda") for _ in range(max_r)]
    outs = [torch.zeros(n, dtype=torch.float32, device="cuda") for _ in range(max_w)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    in_arr = (ctypes.c_void_p * max_r)(*[t.data_ptr() for t in ins])
    out_arr = (ctypes.c_void_p * max_w)(*[t.data_ptr() for t in outs])
    print(f"[probe] {n:,} floats per stream, {launches} launches per probe", file=sys.stderr, flush=True)
    for r, w in CONFIGS:
        for limit in LIMITS:
            ms = ctypes.c_float(0.0)
            for count in (1, launches):  # one warm-up launch, then the timed ones
                rc = lib.stream_probe_run(r, w, in_arr, out_arr, n, limit, count, 0, ctypes.c_void_p(stream),
                                          ctypes.byref(ms))
                if rc != 0:
                    sys.exit(f"stream_probe_run({r}, {w}) failed: {rc}")
            nbytes = n * 4 * (r + w)
            print(json.dumps({"reads": r, "writes": w, "wg_per_cu": limit, "launches": launches,
                              "ms": round(ms.value, 4), "bytes_per_launch": nbytes,
                              "gbps": round(nbytes / (ms.value * 1e-3) / 1e9, 1)}), flush=True)


def summarize(trace_dir: str, log: str) -> None:
    """Matches the trace's stream_probe dispatches, in launch order, to the
    probes the log lists (one warm-up launch, then `launches` timed ones)."""
    import csv

    lines = [json.loads(x) for x in open(log) if x.startswith("{")]
    disp = []
    for row in csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))):
        if "stream_probe" in row["Kernel_Name"]:
            disp.append((int(row["Start_Timestamp"]), int(row["End_Timestamp"]), row["Kernel_Name"]))
    disp.sort()
    want = sum(1 + x["launches"] for x in lines)
    assert len(disp) == want, f"{len(disp)} probe dispatches in the trace, {want} expected"
    out = [f"Streaming ceilings of MI355X's HBM for the fused Adam update's access shape "
           f"(tests/hw/stream_probe.hip): fp32 streams, 16 B per lane and stream, 128-thread "
           f"workgroups, one 512-element tile each, XCD runs of 32768 elements, non-temporal "
           f"accesses; {lines[0]['bytes_per_launch'] // 4 // (lines[0]['reads'] + lines[0]['writes']):,} "
           f"elements per stream.",
           f"command: {COMMANDS['trace']}", f"summary: {COMMANDS['summary']}", "",
           f"{'reads':>5s} {'writes':>6s} {'WG/CU':>6s} {'events ms':>10s} {'trace ms':>9s} "
           f"{'GB/s (trace)':>13s} {'% of 8 TB/s':>12s}"]
    i = 0
    for x in lines:
        i += 1  # the warm-up launch
        durs = [(e - s) / 1e6 for s, e, _ in disp[i:i + x["launches"]]]
        i += x["launches"]
        tr = statistics.mean(durs)
        gbps = x["bytes_per_launch"] / (tr * 1e-3) / 1e9
        limit = str(x["wg_per_cu"]) if x["wg_per_cu"] else "none"
        out.append(f"{x['reads']:5d} {x['writes']:6d} {limit:>6s} {x['ms']:10.3f} {tr:9.3f} "
                   f"{gbps:13.1f} {100 * gbps / HBM_PEAK_GBPS:12.1f}")
    out += ["", "WG/CU: resident workgroups per compute unit (none: no limit; 7: the limit the fp32-moment "
                "update launches with).", "GB/s counts each stream element read or written once."]
    path = os.path.join(ROOT, "profiles", "stream_probe_ceilings.txt")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--n", type=int, default=201 * 320 * 65536, help="floats per stream (multiple of 512)")
    ap.add_argument("--launches", type=int, default=5)
    ap.add_argument("--summarize-trace")
    ap.add_argument("--log")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize(args.summarize_trace, args.log)
    else:
        run(args.n, args.launches)
    return 0


if __name__ == "__main__":
    sys.exit(main())
