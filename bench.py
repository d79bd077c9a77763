"""Benchmark of the fused multi-tensor AdamW step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload bench201] [--no-extra]

Default workload: 201 fp32 tensors of 320*65536 = 20,971,520 elements
(4,215,275,520 elements; p, g, m, v fp32), AdamW, lr 1.6e-3, betas
(0.9, 0.95), eps 1e-8, weight decay 0.1: the shape of the benchmark script in
TransformerEngine issue "[Performance] FusedAdam capturable kernel is ~1.9x
slower than regular Adam on GB300".  Inputs are synthetic (p ~ N(0,1),
g ~ N(0,1)*1e-3, m = v = 0), drawn on the GPU and resident in HBM before the
timed region.

One step is one call of the library's non-capturable ``adam_step`` over the
whole list (one launch of the update kernel).  The timed region is exactly K
steps between two device synchronisations.  ``value`` is effective HBM GB/s
counting algorithmic bytes (every state word read and written once, the
gradient read once: 28 B/element here).  The same K steps are also timed for
the capturable call (device lr/step/grad scale/noop) and for a HIP-graph
replay of the capturable call; per-launch kernel durations come from HIP
events recorded on the launch stream around each launch.  Where a second
set of p, m, v fits in HBM, the same K steps are timed once more on a
two-buffer handle (``two_buffer_state``: each step reads one buffer set and
writes the other); ``value`` and ``roofline`` stay the in-place step.

In the same process, three interleaved rounds of K update steps and K
launches of an in-place streaming probe over the same buffers (the same
streams read and written once each, in the update's tile map, with no
arithmetic: ``tests/hw/stream_probe.hip``) give the ceiling this machine's HBM
reaches for the workload's own stream mix (``ceiling``).  With the default
workload the other configurations follow, one at a time, each with its
ceiling, its 85%-of-8-TB/s target and a short oracle sample
(``workloads``): the 30B-class shard (non-capturable, two groups), the ZeRO
shard (capturable), the remainder list, 16-bit state and scaled 16-bit
state.

The CPU baseline is the oracle (plain scalar C) on a bounded sample of the
same workload, run on every core of the process's affinity mask (one thread
per core, each on a contiguous slice).

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused AdamW step effective HBM GB/s (% of MI355X peak) and elements/s"
HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCE = os.path.join(ROOT, "adamw_optimizer_step_tensor_amd", "csrc", "adam.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash() -> str:
    """sha256 (first 16 hex digits) of the kernel source's code: comments and
    whitespace are dropped first, so a change to the comments alone does not
    invalidate the recorded counter figures."""
    import re

    with open(KERNEL_SOURCE) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    code = " ".join(text.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def measured_traffic(workload: str, key: str = "bytes_per_launch"):
    """HBM bytes per launch from the committed counter summary (`key`:
    "bytes_per_launch" for the in-place update, "two_buffer_bytes_per_launch"
    for the two-buffer one), or None when there is none for this workload or
    the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_hash():
        return None
    return rec.get(key)


# The commands behind profiles/: <repo> is the repository root, <out> any
# writable directory the rocprofv3 CSV output goes to.
PROFILE_COMMANDS = {
    "trace": "cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace_{w} "
             "-o run -- python3 <repo>/bench.py --workload {w} --no-extra --no-ceiling > <out>/trace_{w}.log",
    "fetch": "cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/pmc_fetch_{w} "
             "-o run -- python3 <repo>/bench.py --workload {w} --no-extra --no-ceiling --steps 3 --warmup 1 --no-cpu --no-capturable "
             "> <out>/pmc_fetch_{w}.log",
    "write": "cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/pmc_write_{w} "
             "-o run -- python3 <repo>/bench.py --workload {w} --no-extra --no-ceiling --steps 3 --warmup 1 --no-cpu --no-capturable "
             "> <out>/pmc_write_{w}.log",
    "summary": "python bench.py --summarize-profiles --workload {w} --trace-dir <out>/trace_{w} "
               "--trace-log <out>/trace_{w}.log --fetch-dir <out>/pmc_fetch_{w} --write-dir <out>/pmc_write_{w} "
               "--fetch-log <out>/pmc_fetch_{w}.log --write-log <out>/pmc_write_{w}.log",
    "valu": "cd /tmp && rocprofv3 --pmc SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_WAVES GRBM_GUI_ACTIVE "
            "--output-format csv -d <out>/pmc_valu_{w} -o run -- python3 <repo>/bench.py "
            "--workload {w} --no-extra --no-ceiling --steps 3 --warmup 1 --no-cpu --no-capturable --no-two-buffer",
    "valu_summary": "python bench.py --summarize-valu --workload {w} --valu-dir <out>/pmc_valu_{w}",
    "occupancy": "cd /tmp && rocprofv3 --pmc MeanOccupancyPerCU OccupancyPercent --output-format csv "
                 "-d <out>/pmc_occ_{w} -o run -- python3 <repo>/bench.py --workload {w} --no-extra --no-ceiling "
                 "--steps 3 --warmup 1 --no-cpu --no-capturable --no-two-buffer",
    "occupancy_summary": "python bench.py --summarize-occupancy --workload {w} --occupancy-dir <out>/pmc_occ_{w}",
    "dram_req": "cd /tmp && rocprofv3 --pmc TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_128B_sum TCC_EA0_WRREQ_sum "
                "TCC_EA0_WRREQ_64B_sum --output-format csv -d <out>/pmc_dreq_{w} -o run -- "
                "python3 <repo>/bench.py --workload {w} --no-extra --no-ceiling --steps 3 --warmup 1 --no-cpu --no-capturable "
                "--no-two-buffer",
    "dram_stall": "cd /tmp && rocprofv3 --pmc TCC_EA0_RDREQ_LEVEL_sum TCC_EA0_WRREQ_LEVEL_sum "
                  "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum GRBM_GUI_ACTIVE "
                  "--output-format csv -d <out>/pmc_dstall_{w} -o run -- python3 <repo>/bench.py "
                  "--workload {w} --no-extra --no-ceiling --steps 3 --warmup 1 --no-cpu --no-capturable --no-two-buffer",
    "dram_summary": "python bench.py --summarize-dram --workload {w} --dram-req-dir <out>/pmc_dreq_{w} "
                    "--dram-stall-dir <out>/pmc_dstall_{w}",
    "memunit": "cd /tmp && rocprofv3 --pmc TA_TA_BUSY_sum GRBM_GUI_ACTIVE MemUnitStalled --output-format csv "
               "-d <out>/pmc_mem_{w} -o run -- python3 <repo>/bench.py --workload {w} --no-extra --no-ceiling --steps 3 --warmup 1 "
               "--no-cpu --no-capturable --no-two-buffer",
    "memunit_summary": "python bench.py --summarize-memunit --workload {w} --memunit-dir <out>/pmc_mem_{w}",
}

# the kernels that stream the elements: the update, and the scaled-state
# maxima and store passes
MAIN_KERNELS = ("adam_update", "adam_scaled_maxima", "adam_scaled_pass", "adam_scaled_one")
# the kernels of one scaled-state step, once per piece (one pass: the
# persistent kernel, its follow-up pass and the per-tensor scales)
SCALED_STEP_KERNELS = ("adam_scaled_maxima", "adam_scaled_fold", "adam_scaled_pass", "adam_scaled_finish")
ONE_PASS_STEP_KERNELS = ("adam_scaled_one",)  # adam_scaled_one, _one_redo, _one_finish


def is_main(name: str) -> bool:
    """A kernel that streams the elements (not the per-tensor scales one)."""
    return name.startswith(MAIN_KERNELS) and not name.startswith("adam_scaled_one_finish")

CU_NUM = 256
XCD_NUM = 8


def _plan_pieces(w) -> int:
    """Pieces a scaled-state step of the workload's first group runs in, from
    a host-only plan of its tensor list (addresses are never dereferenced)."""
    import adamw_optimizer_step_tensor_amd as A

    base, stride = 1 << 44, 1 << 38
    tensors = [dict(p=base + (8 * i) * stride, m=base + (8 * i + 1) * stride, v=base + (8 * i + 2) * stride,
                    g=base + (8 * i + 3) * stride, scales=base + (8 * i + 4) * stride,
                    p_out=base + (8 * i + 5) * stride if w.p_out else None, numel=n)
               for i, n in enumerate(w.sizes)]
    p_out = ("bf16" if w.p_out is True else w.p_out) or None
    return A.adam_tl_plan(tensors, A.make_desc(g=w.g_dtype, p=w.p_kind, p_out=p_out,
                                               scaled_passes=w.scaled_passes))["pieces"]


def _main_dispatches(names_grids, scaled):
    """The (kernel, dispatch) keys of the step's main kernels: for scaled
    state every piece's (each has its own grid), else the largest grid."""
    if scaled:
        return {k for k in names_grids if is_main(k[0])}
    big = max(g for (n, _), g in names_grids.items() if is_main(n))
    return {k for k, g in names_grids.items() if g == big and is_main(k[0])}


def summarize_valu(w, valu_dir: str) -> None:
    """Writes profiles/<kernel>_<workload>_valu.txt: VALU instructions per
    element and VALU activity of the main group's kernels, from one rocprofv3
    --pmc pass (SQ_INSTS_VALU, SQ_ACTIVE_INST_VALU, SQ_WAVES, GRBM_GUI_ACTIVE;
    the CSV sums each over shader engines and XCDs).  "VALU busy" is
    rocprofv3's VALUBusy expression, 100 * SQ_ACTIVE_INST_VALU / CUs /
    GRBM_GUI_ACTIVE of one XCD (the summed value / 8)."""
    import csv

    cmds = {k: v.format(w=w.name) for k, v in PROFILE_COMMANDS.items()}
    n0 = sum(w.sizes)
    scaled = w.p_kind.endswith("_scaled")
    prefix = "adam_scaled" if scaled else "adam_update"
    vals = {}  # (kernel, dispatch) -> {counter: value}
    grids = {}
    for r in csv.DictReader(open(os.path.join(valu_dir, "run_counter_collection.csv"))):
        name = _short(r["Kernel_Name"])
        key = (name, r["Dispatch_Id"])
        vals.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
        grids[key] = int(r["Grid_Size"]) // int(r["Workgroup_Size"])
    main = _main_dispatches(grids, scaled)
    per = {}
    for key, c in vals.items():
        if key in main:
            per.setdefault(key[0], []).append(c)
    pieces = _plan_pieces(w) if scaled else 1
    lines = [f"rocprofv3 VALU counters: workload {w.name}, main group ({n0:,} elements"
             + (f", {pieces} piece(s) per step)" if scaled else ")"),
             f"command: {cmds['valu']}", f"summary: {cmds['valu_summary']}", "",
             f"{'kernel':40s} {'n':>3s} {'VALU insts/elem':>16s} {'VALU busy %':>12s} {'waves':>12s}"]
    for name, cs in sorted(per.items()):
        insts = sum(c["SQ_INSTS_VALU"] for c in cs) / (len(cs) / pieces)  # per step
        active = statistics.mean(c["SQ_ACTIVE_INST_VALU"] for c in cs)
        gui = statistics.mean(c["GRBM_GUI_ACTIVE"] for c in cs) / XCD_NUM  # per-XCD cycles
        waves = statistics.mean(c["SQ_WAVES"] for c in cs)
        busy = 100.0 * active / CU_NUM / gui
        lines.append(f"{name:40s} {len(cs):3d} {insts * 64 / n0:16.1f} {busy:12.1f} {waves:12.0f}")
    lines += ["", "VALU insts/elem = SQ_INSTS_VALU (wave-level instructions) x 64 lanes / elements.",
              "VALU busy is rocprofv3's VALUBusy expression; on this part it is not capped at 100%",
              "(its quad-cycle normalisation), so compare kernels with each other: the same",
              "expression for a memory-bound kernel and an ALU-bound one differs by ~3x."]
    path = os.path.join(ROOT, "profiles", f"{prefix}_{w.name}_valu.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_occupancy(w, occ_dir: str) -> None:
    """Writes profiles/<kernel>_<workload>_occupancy.txt: the mean resident
    waves per CU of the main group's kernels and that as a percentage of the
    32-wave maximum, from rocprofv3's derived metrics MeanOccupancyPerCU
    (accumulated SQ_LEVEL_WAVES / GRBM_GUI_ACTIVE / CUs) and OccupancyPercent
    (SQ_WAVE_CYCLES based), one --pmc pass."""
    import csv

    cmds = {k: v.format(w=w.name) for k, v in PROFILE_COMMANDS.items()}
    n0 = sum(w.sizes)
    prefix = "adam_scaled" if w.p_kind.endswith("_scaled") else "adam_update"
    vals, grids, regs = {}, {}, {}
    for r in csv.DictReader(open(os.path.join(occ_dir, "run_counter_collection.csv"))):
        name = _short(r["Kernel_Name"])
        key = (name, r["Dispatch_Id"])
        vals.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
        grids[key] = int(r["Grid_Size"]) // int(r["Workgroup_Size"])
        regs[name] = (int(r["Workgroup_Size"]), int(r["VGPR_Count"]), int(r["SGPR_Count"]), int(r["LDS_Block_Size"]))
    scaled = w.p_kind.endswith("_scaled")
    main = _main_dispatches(grids, scaled)
    big = max(grids[k] for k in main)
    per = {}
    for key, c in vals.items():
        if key in main:
            per.setdefault(key[0], []).append(c)
    lines = [f"rocprofv3 occupancy: workload {w.name}, main group ({n0:,} elements, "
             + ("every piece of the step)" if scaled else f"{big:,} workgroups)"),
             f"command: {cmds['occupancy']}", f"summary: {cmds['occupancy_summary']}", "",
             f"{'kernel':40s} {'n':>3s} {'waves/CU':>9s} {'% of 32':>8s} {'wg size':>8s} {'VGPRs':>6s} {'SGPRs':>6s} {'LDS':>6s}"]
    for name, cs in sorted(per.items()):
        occ = statistics.mean(c["MeanOccupancyPerCU"] for c in cs)
        pct = statistics.mean(c["OccupancyPercent"] for c in cs)
        wg, vg, sg, lds = regs[name]
        lines.append(f"{name:40s} {len(cs):3d} {occ:9.2f} {pct:8.1f} {wg:8d} {vg:6d} {sg:6d} {lds:6d}")
    lines += ["", "waves/CU: mean resident waves per compute unit over the kernel (4 SIMDs, at most",
              "8 waves each); VGPRs as rocprofv3 reports them for the code object."]
    path = os.path.join(ROOT, "profiles", f"{prefix}_{w.name}_occupancy.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


XCDS = 8            # GRBM_GUI_ACTIVE adds up the busy cycles of every XCD
CUS = 256           # one texture-address unit per compute unit


def summarize_memunit(w, mem_dir: str) -> None:
    """Writes profiles/<kernel>_<workload>_memunit.txt: how busy the vector
    memory path of the main group's kernels is, from one rocprofv3 --pmc
    pass: TA_TA_BUSY_sum (busy cycles of the 256 texture-address units, the
    first stage of every vector memory instruction) over GRBM_GUI_ACTIVE
    (GPU busy cycles summed over the 8 XCDs) and rocprofv3's derived
    MemUnitStalled (% of time the memory unit is stalled).  The clock implied
    by GRBM_GUI_ACTIVE / 8 over the dispatch's duration checks that
    normalisation."""
    import csv

    cmds = {k: v.format(w=w.name) for k, v in PROFILE_COMMANDS.items()}
    n0 = sum(w.sizes)
    prefix = "adam_scaled" if w.p_kind.endswith("_scaled") else "adam_update"
    vals, grids, times = {}, {}, {}
    for r in csv.DictReader(open(os.path.join(mem_dir, "run_counter_collection.csv"))):
        key = (_short(r["Kernel_Name"]), r["Dispatch_Id"])
        vals.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
        grids[key] = int(r["Grid_Size"]) // int(r["Workgroup_Size"])
        times[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    scaled = w.p_kind.endswith("_scaled")
    main = _main_dispatches(grids, scaled)
    big = max(grids[k] for k in main)
    per = {}
    for key, c in vals.items():
        if key in main:
            per.setdefault(key[0], []).append((c, times[key]))
    lines = [f"rocprofv3 memory-unit counters: workload {w.name}, main group ({n0:,} elements, "
             + ("every piece of the step)" if scaled else f"{big:,} workgroups)"),
             f"command: {cmds['memunit']}", f"summary: {cmds['memunit_summary']}", "",
             f"{'kernel':40s} {'n':>3s} {'TA busy %':>10s} {'MemUnitStalled %':>17s} {'implied GHz':>12s}"]
    for name, cs in sorted(per.items()):
        busy = statistics.mean(c["TA_TA_BUSY_sum"] / (CUS * c["GRBM_GUI_ACTIVE"] / XCDS) for c, _ in cs)
        stall = statistics.mean(c["MemUnitStalled"] for c, _ in cs)
        ghz = statistics.mean(c["GRBM_GUI_ACTIVE"] / XCDS / t / 1e9 for c, t in cs if t > 0)
        lines.append(f"{name:40s} {len(cs):3d} {100 * busy:10.1f} {stall:17.2f} {ghz:12.2f}")
    lines += ["", "TA busy: TA_TA_BUSY_sum / (256 units x GRBM_GUI_ACTIVE / 8 XCDs): the share of cycles",
              "the address units are working; MemUnitStalled: rocprofv3's derived stall percentage."]
    path = os.path.join(ROOT, "profiles", f"{prefix}_{w.name}_memunit.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


TCC_CHANNELS = 128  # L2 channels over the 8 XCDs


def summarize_dram(w, req_dir: str, stall_dir: str) -> None:
    """Writes profiles/<kernel>_<workload>_dram.txt: the main kernel's memory
    requests as the L2 sends them to the fabric, from two rocprofv3 --pmc
    passes: request counts by size (TCC_EA0_RDREQ / _128B, TCC_EA0_WRREQ /
    _64B, summed over the L2 channels), and occupancy of the request queues
    (TCC_EA0_RDREQ_LEVEL / WRREQ_LEVEL: outstanding requests summed per
    cycle) with the cycles a request waited for a DRAM credit
    (TCC_EA0_*_DRAM_CREDIT_STALL), against GRBM_GUI_ACTIVE."""
    import csv

    cmds = {k: v.format(w=w.name) for k, v in PROFILE_COMMANDS.items()}
    n0 = sum(w.sizes)
    prefix = "adam_scaled" if w.p_kind.endswith("_scaled") else "adam_update"

    def load(d):
        vals, grids = {}, {}
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            key = (_short(r["Kernel_Name"]), r["Dispatch_Id"])
            vals.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
            grids[key] = int(r["Grid_Size"]) // int(r["Workgroup_Size"])
        # the kernel that streams the elements (the one-pass follow-up pass,
        # which has nothing to store unless a wait ran out, is not it)
        def streams(n):
            return is_main(n) and not n.startswith("adam_scaled_one_redo")
        big = max(g for (n, _), g in grids.items() if streams(n))
        per = {}
        for key, c in vals.items():
            if grids[key] == big and streams(key[0]):
                per.setdefault(key[0], []).append(c)
        return per

    req, stall = load(req_dir), load(stall_dir)
    lines = [f"rocprofv3 memory requests: workload {w.name}, main group ({n0:,} elements, "
             f"{w.bytes_per_elem} B/elem algorithmic)",
             f"command (requests): {cmds['dram_req']}", f"command (queues): {cmds['dram_stall']}",
             f"summary: {cmds['dram_summary']}", ""]
    for name in sorted(req):
        rq = {k: statistics.mean(c[k] for c in req[name]) for k in req[name][0]}
        st = {k: statistics.mean(c[k] for c in stall[name]) for k in stall[name][0]}
        rd, rd128 = rq["TCC_EA0_RDREQ_sum"], rq["TCC_EA0_RDREQ_128B_sum"]
        wr, wr64 = rq["TCC_EA0_WRREQ_sum"], rq["TCC_EA0_WRREQ_64B_sum"]
        cycles = st["GRBM_GUI_ACTIVE"] / XCD_NUM  # per-XCD cycles of the dispatch
        lines += [f"{name}:",
                  f"  read requests {rd:,.0f}, of them 128-byte {rd128:,.0f} ({100 * rd128 / rd:.2f}%)",
                  f"  write requests {wr:,.0f}, of them 64-byte {wr64:,.0f} ({100 * wr64 / wr:.2f}%)",
                  f"  bytes per element implied (128 B reads + 64 B writes, the rest 64 / 32 B): "
                  f"{(128 * rd128 + 64 * (rd - rd128) + 64 * wr64 + 32 * (wr - wr64)) / n0:.3f}",
                  f"  mean outstanding requests over the GPU: reads {st['TCC_EA0_RDREQ_LEVEL_sum'] / cycles:,.0f}, "
                  f"writes {st['TCC_EA0_WRREQ_LEVEL_sum'] / cycles:,.0f}",
                  f"  mean read request lifetime (Little): {st['TCC_EA0_RDREQ_LEVEL_sum'] / rd:,.0f} cycles; "
                  f"write: {st['TCC_EA0_WRREQ_LEVEL_sum'] / wr:,.0f} cycles",
                  f"  DRAM credit stalls, % of channel-cycles: reads "
                  f"{100 * st['TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum'] / (cycles * TCC_CHANNELS):.1f}, "
                  f"writes {100 * st['TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum'] / (cycles * TCC_CHANNELS):.1f}",
                  ""]
    lines += ["Counters are summed over the L2 channels (128); GRBM_GUI_ACTIVE is summed over the",
              "8 XCDs and divided by 8 here.  A request's lifetime is its time in the L2-to-fabric",
              "queue until the data returns (reads) or the write is acknowledged."]
    path = os.path.join(ROOT, "profiles", f"{prefix}_{w.name}_dram.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _short(name: str) -> str:
    """A readable kernel name: the update kernel with its configuration, other
    kernels without template arguments (plus the functor they apply)."""
    import re

    n = name.replace("(anonymous namespace)::", "")
    for kernel, cfg_name in (("adam_update", "Config<"), ("adam_scaled_maxima", "ScaledConfig<"),
                             ("adam_scaled_pass", "ScaledConfig<"), ("adam_scaled_one_redo", "ScaledConfig<"),
                             ("adam_scaled_one", "ScaledConfig<")):
        if kernel in n and cfg_name in n:
            i = n.index(cfg_name) + len(cfg_name)
            return f"{kernel}<{n[i:n.index('>', i)]}>"
    base = re.split(r"[<(]", n.replace("void ", ""), maxsplit=1)[0]
    m = re.search(r"(\w+Functor)<", n)
    return base + (f"[{m.group(1)}]" if m else "")


def _bench_line(path):
    """The last bench line (JSON) a profiled bench command printed, or None."""
    if not path:
        return None
    line = None
    for text in open(path):
        if text.startswith("{"):
            line = json.loads(text)
    return line


def _two_buffer_launches(line) -> int:
    """Launches of the main group's two-buffer step in a bench run (its last
    non-capturable update launches), 0 when it did not run."""
    tb = (line or {}).get("two_buffer_state")
    return line["warmup"] + line["steps"] if isinstance(tb, dict) and "ms_per_step" in tb else 0


TWO_BUFFER_TAG = " [two-buffer]"


def summarize_profiles(w, trace_dir: str, fetch_dir: str, write_dir: str, trace_log: str = None,
                       fetch_log: str = None, write_log: str = None) -> None:
    """Writes profiles/<kernel>_<workload>_{kernel_trace,pmc}.txt (kernel
    adam_update, or adam_scaled for scaled state) and updates
    profiles/traffic.json from rocprofv3 CSV output.

    Durations of the update kernel come from the per-dispatch trace, grouped
    by kernel configuration and grid size (the largest grid is the workload's
    main group).  HBM traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of
    the main group's update dispatches, each scaled by the factor that makes
    the same counter agree with the known bytes of a plain elementwise kernel
    in the same run: torch's in-place multiply that scales the gradient while
    the inputs are drawn, which reads and writes every element of an fp32
    buffer of the workload's size once.

    With `trace_log` (the bench line the traced command printed), the
    launch durations bench.py measured with HIP events in that same process
    are set beside the trace's averages for the same dispatches.  When a
    run also timed the two-buffer step (the bench line says so), its update
    launches are that run's last non-capturable ones of the main group; they
    are reported apart from the in-place ones (`fetch_log` and `write_log`
    are the counter runs' bench lines).  The bench line's roofline and
    profiles/traffic.json describe the in-place kernel."""
    import csv

    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    cmds = {k: v.format(w=w.name) for k, v in PROFILE_COMMANDS.items()}
    n0 = sum(w.sizes)
    algo = n0 * w.bytes_per_elem
    scaled = w.p_kind.endswith("_scaled")
    prefix = "adam_scaled" if scaled else "adam_update"

    def main_kernel(name):
        return is_main(name)

    # kernel trace: all kernels (stats), then the update kernel per dispatch
    rows = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv"))))
    lines = [f"rocprofv3 kernel trace: workload {w.name} ({w.numel:,} elements; main group "
             f"{n0:,} elements x {w.bytes_per_elem} B/elem algorithmic = {algo / 1e9:.3f} GB per launch)",
             f"command: {cmds['trace']}", f"summary: {cmds['summary']}", "",
             "all kernels (rocprofv3 --stats):",
             f"{'kernel':62s} {'calls':>5s} {'avg ms':>9s} {'min ms':>9s} {'max ms':>9s}"]
    for r in rows:
        lines.append(f"{_short(r['Name']):62s} {int(r['Calls']):5d} {float(r['AverageNs']) / 1e6:9.3f} "
                     f"{float(r['MinNs']) / 1e6:9.3f} {float(r['MaxNs']) / 1e6:9.3f}")
    per = {}
    for r in csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))):
        name = _short(r["Kernel_Name"])
        if main_kernel(name):
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
            per.setdefault((name, int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])), []).append(
                (int(r["Start_Timestamp"]), dur))
    big = max(g for _, g in per)
    bench_line = _bench_line(trace_log)
    n_tb = 0 if scaled else _two_buffer_launches(bench_line)
    for (name, grid) in list(per):
        if n_tb and grid == big and name.endswith("false>"):
            d = sorted(per.pop((name, grid)))
            per[(name, grid)], per[(name + TWO_BUFFER_TAG, grid)] = d[:-n_tb], d[-n_tb:]
    per = {k: [dur for _, dur in v] for k, v in per.items()}
    pieces = int(((bench_line or {}).get("config") or {}).get("pieces", 1))
    spans = []
    if scaled:
        # a scaled step is 4 kernels per piece, the pieces pipelined over two
        # streams; its time is its first dispatch's start to its last's end
        disp = []
        step_kernels = ONE_PASS_STEP_KERNELS if w.scaled_passes == 1 else SCALED_STEP_KERNELS
        for r in csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))):
            if _short(r["Kernel_Name"]).startswith(step_kernels):
                disp.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
        disp.sort()
        k = 3 if w.scaled_passes == 1 else 4 * pieces
        spans = [(max(e for _, e in disp[i:i + k]) - disp[i][0]) / 1e6 for i in range(0, len(disp) - k + 1, k)]
    lines += ["", ("scaled-state passes" if scaled else "update kernel") +
              (f" per dispatch ({pieces} piece(s) per step, each its own grid):" if scaled else
               " per dispatch (main group = the largest grid):"),
              f"{'kernel':46s} {'workgroups':>13s} {'calls':>5s} {'avg ms':>9s} {'min ms':>9s} "
              f"{'max ms':>9s} {'GB/s(avg)':>10s}"]
    for (name, grid), durs in sorted(per.items()):
        avg = statistics.mean(durs)
        gbps = f"{algo / (avg * 1e-3) / 1e9:10.1f}" if grid == big and not scaled else ""
        lines.append(f"{name:46s} {grid:13d} {len(durs):5d} {avg:9.3f} {min(durs):9.3f} "
                     f"{max(durs):9.3f} {gbps}")
    if scaled and spans:
        # kernel time per step: every piece's maxima and store pass
        kern = sum(sum(d) for d in per.values()) / len(spans)
        step = statistics.mean(spans)
        lines.append(f"one step: {step:.3f} ms from its first dispatch to its last (mean of {len(spans)} steps), "
                     f"{kern:.3f} ms of maxima and store pass time summed over its pieces; algorithmic bytes "
                     f"per step {algo / 1e9:.3f} GB -> {algo / (step * 1e-3) / 1e9:.1f} GB/s")
    if trace_log:
        assert bench_line is not None, f"no bench line in {trace_log}"
        lines += ["", "bench.py in the same traced process (HIP events on the launch stream) vs the "
                      "trace's average over the same main-group dispatches:"]
        if scaled:
            nw = bench_line["warmup"] + bench_line["steps"]
            pairs = [("scaled step, regular (all pieces)", bench_line["roofline"]["launch_ms_mean"],
                      statistics.mean(spans[:nw]))]
            if "capturable" in bench_line and len(spans) >= 2 * nw:
                pairs.append(("scaled step, capturable", bench_line["capturable"]["launch_ms_mean"],
                              statistics.mean(spans[nw:2 * nw])))
        else:
            def trace_avg(capt):
                d = [x for (n, g), v in per.items() if g == big and n.endswith(f"{capt}>") for x in v]
                return statistics.mean(d) if d else float("nan")
            pairs = [("update, regular", bench_line["roofline"]["launch_ms_mean"], trace_avg("false"))]
            if "capturable" in bench_line:
                pairs.append(("update, capturable", bench_line["capturable"]["launch_ms_mean"], trace_avg("true")))
            if n_tb:
                d = [x for (nm, g), v in per.items() if g == big and nm.endswith(TWO_BUFFER_TAG) for x in v]
                pairs.append(("update, two-buffer state", bench_line["two_buffer_state"]["launch_ms_mean"],
                              statistics.mean(d)))
        for what, ev, tr in pairs:
            lines.append(f"  {what:42s} events {ev:9.3f} ms   trace {tr:9.3f} ms   events / trace {ev / tr:.4f}")
        lines.append(f"  bench line of the traced run: value {bench_line['value']} {bench_line['unit']}, "
                     f"ms/step {bench_line['ms_per_step']}, roofline.achieved {bench_line['roofline']['achieved']}")
    trace_path = os.path.join(ROOT, "profiles", f"{prefix}_{w.name}_kernel_trace.txt")
    with open(trace_path, "w") as f:
        f.write("\n".join(lines) + "\n")

    # counters
    def per_kernel(path, log):
        """Counter value per dispatch, by kernel, in dispatch order; the main
        group's last two-buffer launches (if the run made them) apart."""
        rows = list(csv.DictReader(open(os.path.join(path, "run_counter_collection.csv"))))
        if rows and "Dispatch_Id" in rows[0]:
            rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        agg = {}
        for r in rows:
            name = _short(r["Kernel_Name"])
            if not scaled and main_kernel(name) and int(r["Grid_Size"]) // int(r["Workgroup_Size"]) != big:
                name += " (small group)"
            agg.setdefault(name, []).append(float(r["Counter_Value"]))
        n = 0 if scaled else _two_buffer_launches(_bench_line(log))
        if n:
            main = [k for k in agg if main_kernel(k) and not k.endswith("(small group)")]
            assert len(main) == 1, main
            vals = agg.pop(main[0])
            agg[main[0]], agg[main[0] + TWO_BUFFER_TAG] = vals[:-n], vals[-n:]
        return agg

    fetch, write = per_kernel(fetch_dir, fetch_log), per_kernel(write_dir, write_log)
    cal = [k for k in fetch if "AUnaryFunctor" in k]
    assert cal, "calibration kernel (elementwise multiply) not found"
    # fp32 temporaries of all elements, read once and written once: the
    # gradient's, and for scaled fp16 state also the param's
    from workloads import scaled_p_scale

    draws = 2 if scaled and scaled_p_scale(w.p_kind) != 1.0 else 1
    known_kib = draws * w.numel * 4 / 1024
    f_factor = known_kib / sum(fetch[cal[0]])
    w_factor = known_kib / sum(write[cal[0]])
    upd = [k for k in fetch if main_kernel(k) and not k.endswith("(small group)") and
           not k.endswith(TWO_BUFFER_TAG)]
    assert len(upd) == (2 if scaled else 1), upd
    tb_key = [k for k in fetch if k.endswith(TWO_BUFFER_TAG)]
    tb_traffic = None
    if tb_key and tb_key[0] in write:
        tb_traffic = (statistics.mean(fetch[tb_key[0]]) * f_factor + statistics.mean(write[tb_key[0]]) * w_factor) * 1024
    if scaled:
        # every piece's dispatches of both passes, per step
        line_f = _bench_line(fetch_log)
        steps_run = line_f["warmup"] + line_f["steps"] if line_f else len(fetch[upd[0]])
        fetch_kib = sum(sum(fetch[k]) for k in upd) / steps_run
        write_kib = sum(sum(write[k]) for k in upd) / steps_run
    else:
        fetch_kib = sum(statistics.mean(fetch[k]) for k in upd)
        write_kib = sum(statistics.mean(write[k]) for k in upd)
    k = " + ".join(upd)
    traffic = (fetch_kib * f_factor + write_kib * w_factor) * 1024
    lines = [f"rocprofv3 counters: workload {w.name}, kernel {k} (main group, {n0:,} elements)",
             f"command (read): {cmds['fetch']}", f"command (write): {cmds['write']}",
             f"summary: {cmds['summary']}", "",
             "per-kernel mean counter value per dispatch (KiB), raw:",
             f"{'kernel':62s} {'n':>3s} {'FETCH_SIZE':>14s} {'WRITE_SIZE':>14s}"]
    for name in fetch:
        lines.append(f"{name:62s} {len(fetch[name]):3d} {statistics.mean(fetch[name]):14.1f} "
                     f"{statistics.mean(write.get(name, [0])):14.1f}")
    lines += ["",
              f"calibration: {cal[0]} reads and writes {known_kib:,.0f} KiB in total",
              f"  (scaling the drawn fp32 temporaries: the gradient's, and the param's for scaled fp16 state);",
              f"  counters summed over its dispatches give",
              f"  FETCH factor {f_factor:.4f}, WRITE factor {w_factor:.4f}",
              f"{('one-pass kernels per step' if w.scaled_passes == 1 else 'both passes per step') if scaled else 'update kernel per launch'}: "
              f"read {fetch_kib * f_factor * 1024 / 1e9:.3f} GB, "
              f"write {write_kib * w_factor * 1024 / 1e9:.3f} GB, total {traffic / 1e9:.3f} GB",
              f"algorithmic bytes per launch: {algo / 1e9:.3f} GB ({n0:,} elements x {w.bytes_per_elem} B); "
              f"measured / algorithmic = {traffic / algo:.4f}"]
    if tb_traffic is not None:
        lines.append(f"two-buffer state (the runs' last {len(fetch[tb_key[0]])} update launches): "
                     f"{tb_traffic / 1e9:.3f} GB per launch; measured / algorithmic = {tb_traffic / algo:.4f}")
    lines.append(f"kernel source sha256[:16] = {source_hash()}")
    if scaled and w.scaled_passes == 1:
        lines.append("one pass: each of p, m, v and g is read once (a tile is stored from registers "
                     "and local memory once its tensor's scales are published)")
    elif scaled:
        lines.append("scaled state reads p, m, v and g twice (the maxima pass, then the store pass "
                     "recomputes the update): the second read is counted whether the Infinity Cache "
                     "or HBM serves it")
    pmc_path = os.path.join(ROOT, "profiles", f"{prefix}_{w.name}_pmc.txt")
    with open(pmc_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    try:
        with open(TRAFFIC_FILE) as f:
            allrec = json.load(f)
    except (OSError, ValueError):
        allrec = {}
    allrec[w.name] = {"bytes_per_launch": round(traffic), "algorithmic_bytes_per_launch": algo,
                      "ratio": round(traffic / algo, 5), "fetch_factor": round(f_factor, 5),
                      "write_factor": round(w_factor, 5), "kernel": k,
                      "source_sha256_16": source_hash()}
    if tb_traffic is not None:
        allrec[w.name]["two_buffer_bytes_per_launch"] = round(tb_traffic)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(allrec, f, indent=1, sort_keys=True)
    print("\n".join(open(trace_path).read().splitlines() + [""] + open(pmc_path).read().splitlines()))


def cpu_baseline(w, sample_elems: int, sample_steps: int, target_s: float = 10.0) -> dict:
    """The oracle on whole tensors from the start of the workload's list (at
    least `sample_elems` elements, with the workload's dtypes) for
    `sample_steps` steps (0: as many as fill about `target_s` seconds of
    wall time, judged from the second step), on the host's cores: one thread
    per core, each on a contiguous slice of the concatenated sample."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    from workloads import host_tensors

    o = oracle.default()
    cores = max(1, len(os.sched_getaffinity(0)))  # every core the process may run on
    if w.p_kind.endswith("_scaled"):
        sample_elems //= 8  # the scaled-state oracle is ~8x slower per element
    sizes = []
    for n in w.sizes:
        sizes.append(n)
        if sum(sizes) >= sample_elems:
            break
    host = host_tensors(sizes, g_dtype=w.g_dtype, p_kind=w.p_kind, p_out=w.p_out, seed=w.seed,
                        g_multiplier=w.grad_multiplier)
    hp = oracle.HParams(w.beta1, w.beta2, w.eps, w.weight_decay, w.mode, 1)
    if host[0].scales is not None:
        # scaled state: each tensor's new scales need all of it, so the
        # threads take whole tensors
        ts = [oracle.OracleTensor(h.p, h.m, h.v, h.g, h.p_out, None, h.scales) for h in host]
        n = sum(t.numel for t in ts)
        jobs = [lambda bc1, bc2, t=t: o.update_tensor(t, hp, w.lr, bc1, bc2, w.grad_scale) for t in ts]
    else:
        cat = lambda role: (None if getattr(host[0], role) is None
                            else np.concatenate([getattr(h, role) for h in host]))
        t = oracle.OracleTensor(cat("p"), cat("m"), cat("v"), cat("g"), cat("p_out"), cat("rem"))
        n = t.numel
        bounds = [(i * n // cores, (i + 1) * n // cores) for i in range(cores)]
        jobs = [lambda bc1, bc2, b=b: o.update_tensor(t, hp, w.lr, bc1, bc2, w.grad_scale, b[0], b[1])
                for b in bounds]
    del host
    cores = min(cores, len(jobs))  # the threads that get work
    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        step = 0
        while True:
            step += 1
            bc1, bc2 = o.bias_corrections(w.beta1, w.beta2, step, 1)
            list(ex.map(lambda job: job(bc1, bc2), jobs))
            if step == 1 and sample_steps <= 0:
                t1 = time.perf_counter()
            if step == 2 and sample_steps <= 0:
                # the second step: the first also pays for first-touch page faults
                per = time.perf_counter() - t1
                sample_steps = max(2, min(1000, int((target_s - (t1 - t0)) / max(per, 1e-6)) + 1))
            if sample_steps > 0 and step >= sample_steps:
                break
    dt = time.perf_counter() - t0
    gbps = n * sample_steps * w.bytes_per_elem / dt / 1e9
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "affinity_cores": len(os.sched_getaffinity(0)),
            "sample": f"first {len(sizes)} of {len(w.sizes)} tensors ({n:,} elements, workload dtypes) x "
                      f"{sample_steps} steps: {n * sample_steps:,} element updates in {dt:.2f} s wall "
                      f"({dt * cores:.0f} thread-seconds)",
            "elements_per_s": round(n * sample_steps / dt, 1), "cpu_model": cpu_model()}


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it: model name, family, model and
    stepping of the first processor, and whether it runs under a hypervisor."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break  # the first processor's block
                key, _, val = line.partition(":")
                info.setdefault(key.strip(), val.strip())
    except OSError:
        return ""
    text = info.get("model name", "")
    ids = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
    extra = ids + (["virtualised (hypervisor flag)"] if "hypervisor" in info.get("flags", "").split() else [])
    return f"{text} ({', '.join(extra)})" if extra else text


def build_run(w, args, A, torch):
    """Draws a workload's inputs on the GPU and builds one handle per group
    (views into flat buffers); returns the buffers, handles and step
    helpers."""
    from types import SimpleNamespace

    from workloads import device_flat, scaled_p_scale, split_views

    groups = [(w.sizes, w.weight_decay)] + list(w.extra_groups)
    total = w.numel
    t0 = time.perf_counter()
    bufs = device_flat(total, g_dtype=w.g_dtype, p_kind=w.p_kind, p_out=w.p_out, seed=w.seed,
                       g_multiplier=w.grad_multiplier)
    torch.cuda.synchronize()
    log(f"{w.name}: inputs drawn on the GPU in {time.perf_counter() - t0:.1f} s")

    # one handle per group, views into the flat buffers
    scaled = w.p_kind.endswith("_scaled")
    mv_desc = "scaled 16-bit" if scaled else w.p_kind if w.p_kind in ("bf16", "f16") else "f32"
    p_out = ("bf16" if w.p_out is True else w.p_out) or None
    handles = []
    scale_bufs = []
    off = 0
    for sizes, wd in groups:
        n = sum(sizes)
        views = {k: split_views(v[off:off + n], sizes) for k, v in bufs.items()}
        tensors = [{k: views[k][i] for k in views} for i in range(len(sizes))]
        if scaled:
            # per-tensor scales of p, m, v: the drawn p's power-of-two scale;
            # zero moments carry scale 0 (a fresh optimizer)
            sc = torch.zeros((len(sizes), 3), dtype=torch.float32, device="cuda")
            sc[:, 0] = scaled_p_scale(w.p_kind)
            scale_bufs.append(sc)
            for i, t in enumerate(tensors):
                t["scales"] = sc[i]
        desc = A.make_desc(g=w.g_dtype, p=w.p_kind, p_out=p_out, chunk_elems=args.chunk_elems,
                           scaled_passes=w.scaled_passes)
        tl = A.adam_tl_build(tensors, desc)
        hp = A.AdamHParams(w.beta1, w.beta2, w.eps, wd, w.mode, 1)
        # each group keeps its own counter, host and device
        handles.append((tl, hp, n, A.HostStep(0), torch.zeros(1, dtype=torch.int32, device="cuda")))
        off += n
    info = handles[0][0].info()
    log(f"{w.name}: work table: {info['chunks']} records of {info['chunk_elems']} elements; "
        f"{info['grid_blocks']} workgroups of {info['block_threads']} threads, "
        f"{info['tile_elems']} elements each, {info['dispatches']} dispatch(es)")

    step_fn = {"bf16_rem": A.adam_step_remainders, "bf16_scaled": A.adam_step_scaled,
               "f16_scaled": A.adam_step_scaled}.get(w.p_kind, A.adam_step)
    cap_fn = {"bf16_rem": A.adam_step_remainders_capturable, "bf16_scaled": A.adam_step_scaled_capturable,
              "f16_scaled": A.adam_step_scaled_capturable}.get(w.p_kind, A.adam_step_capturable)
    stream = torch.cuda.current_stream()
    d_scale = torch.tensor([w.grad_scale], dtype=torch.float32, device="cuda")
    d_lr = torch.tensor([w.lr], dtype=torch.float32, device="cuda")
    d_noop = torch.zeros(1, dtype=torch.int32, device="cuda")

    def launch_timed(ev, launch):
        """Runs launch(); when ev is a list, brackets it with HIP events on the
        launch stream and appends the pair."""
        if ev is None:
            launch()
            return
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch()
        e1.record(stream)
        ev.append((e0, e1))

    def one_step_noncap(ev=None):
        """One step: every group once; events bracket the first (largest)
        group's launch."""
        for i, (tl, hp, _, host_step, _) in enumerate(handles):
            launch_timed(ev if i == 0 else None,
                         lambda: step_fn(tl, hp, w.lr, host_step, 1.0, d_scale, stream))

    def one_step_cap(ev=None, s=stream):
        """One capturable step of every group (device lr, counter, grad scale
        and noop flag); events bracket the first group's call."""
        for i, (tl, hp, _, _, d_step) in enumerate(handles):
            launch_timed(ev if i == 0 else None,
                         lambda: cap_fn(tl, hp, d_lr, d_step, d_scale, d_noop, s))

    def timed(step_once, k, events=True):
        """Runs k steps between two synchronisations; returns (wall ms per
        step, per-launch event ms of the first group's launches)."""
        ev = [] if events else None
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for _ in range(k):
            step_once(ev)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t_start) * 1e3 / k
        per = [a.elapsed_time(b) for a, b in (ev or [])]
        return wall, per

    def destroy():
        for h in handles:
            h[0].destroy()

    return SimpleNamespace(w=w, groups=groups, total=total, bufs=bufs, handles=handles, scale_bufs=scale_bufs,
                           info=info, scaled=scaled, mv_desc=mv_desc, p_out=p_out, step_fn=step_fn, cap_fn=cap_fn,
                           stream=stream, d_scale=d_scale, d_lr=d_lr, d_noop=d_noop, launch_timed=launch_timed,
                           one_step_noncap=one_step_noncap, one_step_cap=one_step_cap, timed=timed, destroy=destroy)


# ---------------------------------------------------------------------------
# The streaming ceiling of a workload's own stream mix, in the same process
# ---------------------------------------------------------------------------

PROBE_LIBRARY = os.path.join(ROOT, "tests", "hw", "libstream_probe.so")
# The update launches fp32-moment lists with at most this many workgroups per
# compute unit (the library's occupancy limit); the probe copies it.
FP32_MOMENT_WG_PER_CU = 7


def probe_library():
    """The in-place streaming probe (tests/hw/stream_probe.hip), or None if it
    has not been built."""
    import ctypes

    if not os.path.exists(PROBE_LIBRARY):
        return None
    lib = ctypes.CDLL(PROBE_LIBRARY)
    vp = ctypes.c_void_p
    lib.stream_probe_mix_run.restype = ctypes.c_int
    lib.stream_probe_mix_run.argtypes = [ctypes.c_int] * 5 + [vp] * 6 + [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                                        vp, ctypes.POINTER(ctypes.c_float)]
    return lib


def probe_mix(w):
    """(p, m/v, g, p_out bytes per element, remainders) of a workload's streams,
    and the probe's resident-workgroup limit (the update's)."""
    state16 = w.p_kind in ("bf16", "f16") or w.p_kind.endswith("_scaled")
    rem = w.p_kind == "bf16_rem"
    pb = 2 if state16 or rem else 4
    mb = 2 if state16 else 4
    gb = 4 if w.g_dtype == "f32" else 2
    out = ("bf16" if w.p_out is True else w.p_out) or None
    ob = {None: 0, "f32": 4}.get(out, 2)
    limit = FP32_MOMENT_WG_PER_CU if mb == 4 else 0
    return (pb, mb, gb, ob, 1 if rem else 0), limit


def probe_ms(lib, r, launches: int) -> float:
    """Mean launch time of the in-place probe over the workload's own flat
    buffers (p, m, v and remainders read and written back unchanged, g read,
    p_out written), `launches` launches on the run's stream."""
    import ctypes

    mix, limit = probe_mix(r.w)
    b = r.bufs
    ptr = lambda k: ctypes.c_void_p(b[k].data_ptr()) if k in b else None
    ms = ctypes.c_float(0.0)
    rc = lib.stream_probe_mix_run(*mix, ptr("p"), ptr("rem"), ptr("m"), ptr("v"), ptr("g"), ptr("p_out"),
                                  r.total - r.total % 4, limit, launches, ctypes.c_void_p(r.stream.cuda_stream),
                                  ctypes.byref(ms))
    if rc != 0:
        raise RuntimeError(f"stream_probe_mix_run failed: {rc}")
    return ms.value


def interleaved_rounds(r, lib, step_once, k: int, rounds: int) -> dict:
    """`rounds` rounds of: k steps of the update (wall time per step between
    two synchronisations, and HIP-event time of the first group's launch),
    then k launches of the probe of the same stream mix over the same
    buffers; medians over the rounds."""
    upd, upd_launch, probe = [], [], []
    for _ in range(rounds):
        wall, per = r.timed(step_once, k)
        upd.append(wall)
        upd_launch.append(statistics.mean(per))
        probe_ms(lib, r, 1)  # the probe's first launch in a round is not timed
        probe.append(probe_ms(lib, r, k))
    bytes_step = r.total * r.w.bytes_per_elem
    u, ul, c = statistics.median(upd), statistics.median(upd_launch), statistics.median(probe)
    (pb, mb, gb, ob, rem), limit = probe_mix(r.w)
    return {
        "what": f"in-place probe of the same streams (p {pb} B, m/v {mb} B, g {gb} B, p_out {ob} B, "
                f"remainders {'2 B' if rem else 'none'} per element; read and written once, no arithmetic; "
                f"the update's tile map{', ' + str(limit) + ' workgroups per CU' if limit else ''}), "
                f"interleaved with the update, medians of {rounds} rounds of {k}",
        "gbps": round(bytes_step / (c * 1e-3) / 1e9, 1),
        "frac": round(bytes_step / (c * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "probe_ms": round(c, 4),
        "update_ms_per_step": round(u, 4),
        "update_launch_ms": round(ul, 4),
        "update_gbps": round(bytes_step / (u * 1e-3) / 1e9, 1),
        "update_over_ceiling": round(c / u, 4),
        "rounds_update_ms": [round(x, 4) for x in upd],
        "rounds_probe_ms": [round(x, 4) for x in probe],
    }


# The configurations timed beside the main workload, each with the step call
# its configuration names ("capturable": device scalars, noop flag 0).
EXTRA_WORKLOADS = ("shard30b", "zero1e9", "rem5e8", "state16_1e9", "scaled1e9", "scaled1e9_one")
CAPTURABLE_WORKLOADS = ("zero1e9",)
TARGET_FRAC = 0.85


def measure_extra(name, args, A, torch, lib) -> dict:
    """Draws one more workload, times its step (and the probe of its stream
    mix) in interleaved rounds, and times the oracle on a short sample."""
    from workloads import workloads

    w = workloads()[name]
    r = build_run(w, args, A, torch)
    capt = name in CAPTURABLE_WORKLOADS
    step_once = r.one_step_cap if capt else r.one_step_noncap
    for _ in range(args.warmup):
        step_once()
    torch.cuda.synchronize()
    bytes_step = r.total * w.bytes_per_elem
    out = {"config": f"{len(w.sizes) + sum(len(s) for s, _ in w.extra_groups)} tensors, {r.total:,} elements, "
                     f"p {w.p_kind}, g {w.g_dtype}, m/v {r.mv_desc}, p_out {r.p_out or 'none'}, "
                     f"{w.bytes_per_elem} B/elem",
           "call": (r.cap_fn if capt else r.step_fn).__name__,
           "pieces": r.info["pieces"], "dispatches": r.info["dispatches"]}
    if lib is not None:
        rounds = interleaved_rounds(r, lib, step_once, args.steps, args.rounds)
        ms = rounds["update_ms_per_step"]
        out["ceiling"] = {k: rounds[k] for k in ("what", "gbps", "frac", "probe_ms", "update_over_ceiling",
                                                 "rounds_update_ms", "rounds_probe_ms")}
        launch = rounds["update_launch_ms"]
    else:
        ms, per = r.timed(step_once, args.steps)
        launch = statistics.mean(per)
        out["ceiling"] = None
    gbps = bytes_step / (ms * 1e-3) / 1e9
    target_ms = bytes_step / (TARGET_FRAC * HBM_PEAK_GBPS * 1e9) * 1e3
    out.update({
        "ms_per_step": round(ms, 4),
        "gbps": round(gbps, 1),
        "frac": round(gbps / HBM_PEAK_GBPS, 4),
        "elements_per_s": round(r.total / (ms * 1e-3), 1),
        "first_group_launch_ms": round(launch, 4),
        "target_ms_at_85pct": round(target_ms, 3),
        "meets_target": ms <= target_ms,
        "traffic": measured_traffic(name),
    })
    log(f"{name}: {ms:.3f} ms/step, {gbps:.0f} GB/s ({100 * gbps / HBM_PEAK_GBPS:.1f}%), ceiling "
        f"{(out['ceiling'] or {}).get('gbps')} GB/s")
    r.destroy()
    del r
    torch.cuda.empty_cache()
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_elements // 4, 0, target_s=args.extra_cpu_seconds)
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="bench201")
    ap.add_argument("--chunk-elems", type=int, default=0)
    ap.add_argument("--cpu-elements", type=int, default=200_000_000)
    ap.add_argument("--cpu-steps", type=int, default=0,
                    help="oracle steps for the CPU baseline (0: about 10 s of wall time)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-capturable", action="store_true")
    ap.add_argument("--no-two-buffer", action="store_true",
                    help="skip the two-buffer-state measurement")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the in-place streaming probe of the same stream mix")
    ap.add_argument("--rounds", type=int, default=3,
                    help="interleaved rounds of update and probe for the ceilings")
    ap.add_argument("--no-extra", action="store_true",
                    help="time the main workload only (no per-configuration map)")
    ap.add_argument("--extra", default=",".join(EXTRA_WORKLOADS),
                    help="configurations timed after the default workload (comma separated)")
    ap.add_argument("--extra-cpu-seconds", type=float, default=2.0,
                    help="wall seconds of oracle time per extra configuration")
    ap.add_argument("--summarize-profiles", action="store_true",
                    help="write profiles/ summaries from rocprofv3 CSV directories (no GPU)")
    ap.add_argument("--trace-dir")
    ap.add_argument("--trace-log", help="stdout of the traced bench command (its bench line)")
    ap.add_argument("--fetch-log", help="stdout of the FETCH_SIZE run (its bench line)")
    ap.add_argument("--write-log", help="stdout of the WRITE_SIZE run (its bench line)")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--summarize-valu", action="store_true",
                    help="write profiles/ VALU summary from a rocprofv3 counter directory (no GPU)")
    ap.add_argument("--valu-dir")
    ap.add_argument("--summarize-occupancy", action="store_true",
                    help="write profiles/ occupancy summary from a rocprofv3 counter directory (no GPU)")
    ap.add_argument("--occupancy-dir")
    ap.add_argument("--summarize-dram", action="store_true",
                    help="write profiles/ memory-request summary from two rocprofv3 counter directories (no GPU)")
    ap.add_argument("--summarize-memunit", action="store_true",
                    help="write profiles/ memory-unit summary from a rocprofv3 counter directory (no GPU)")
    ap.add_argument("--memunit-dir")
    ap.add_argument("--dram-req-dir")
    ap.add_argument("--dram-stall-dir")
    args = ap.parse_args()

    if args.summarize_profiles:
        from workloads import workloads

        summarize_profiles(workloads()[args.workload], args.trace_dir, args.fetch_dir, args.write_dir,
                           args.trace_log, args.fetch_log, args.write_log)
        return 0
    if args.summarize_valu:
        from workloads import workloads

        summarize_valu(workloads()[args.workload], args.valu_dir)
        return 0
    if args.summarize_occupancy:
        from workloads import workloads

        summarize_occupancy(workloads()[args.workload], args.occupancy_dir)
        return 0
    if args.summarize_memunit:
        from workloads import workloads

        summarize_memunit(workloads()[args.workload], args.memunit_dir)
        return 0
    if args.summarize_dram:
        from workloads import workloads

        summarize_dram(workloads()[args.workload], args.dram_req_dir, args.dram_stall_dir)
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import adamw_optimizer_step_tensor_amd as A
    from workloads import split_views, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    A.lib()
    w = workloads()[args.workload]
    groups = [(w.sizes, w.weight_decay)] + list(w.extra_groups)
    total = w.numel
    log(f"workload {w.name}: {total:,} elements in {sum(len(s) for s, _ in groups)} tensors, "
        f"{w.bytes_per_elem} B/elem, {total * w.bytes_per_elem / 1e9:.2f} GB per step")

    r = build_run(w, args, A, torch)
    bufs, handles, scale_bufs, info = r.bufs, r.handles, r.scale_bufs, r.info
    scaled, mv_desc, p_out = r.scaled, r.mv_desc, r.p_out
    step_fn, stream, d_scale = r.step_fn, r.stream, r.d_scale
    launch_timed, one_step_noncap, timed = r.launch_timed, r.one_step_noncap, r.timed

    # --- non-capturable -----------------------------------------------------
    for _ in range(args.warmup):
        one_step_noncap()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")
    wall_ms, per_ms = timed(one_step_noncap, args.steps)
    log(f"non-capturable: {wall_ms:.3f} ms/step wall, event median {statistics.median(per_ms):.3f} ms")
    bytes_step = total * w.bytes_per_elem
    gbps = bytes_step / (wall_ms * 1e-3) / 1e9
    launch_ms = statistics.mean(per_ms)
    launch_bytes = handles[0][2] * w.bytes_per_elem
    achieved = launch_bytes / (launch_ms * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (p~N(0,1), g~N(0,1)*1e-3, m=v=0; drawn on the GPU)",
        "config": {
            "workload": f"{w.name}: {len(w.sizes)} tensors, {total:,} elements, "
                        f"p {w.p_kind}, g {w.g_dtype}, m/v {mv_desc}, "
                        f"p_out {p_out or 'none'}, "
                        f"{'AdamW' if w.mode else 'L2'}, lr {w.lr}, betas ({w.beta1}, {w.beta2}), "
                        f"eps {w.eps}, wd {w.weight_decay}",
            "path": f"{step_fn.__name__} (non-capturable), "
                    + (("one pass: a persistent kernel, a follow-up pass and the per-tensor scales"
                        if w.scaled_passes == 1 else
                        "four launches per piece (maxima pass, per-tensor fold, store pass, scales)")
                       if scaled else "one launch per group per step"),
            "bytes_per_elem": w.bytes_per_elem,
            "chunk_elems": info["chunk_elems"],
            "grid_blocks": info["grid_blocks"],
            "block_threads": info["block_threads"],
            "tile_elems": info["tile_elems"],
            "pieces": info["pieces"],
        },
        "elements_per_s": round(total / (wall_ms * 1e-3), 1),
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": (f"adam_scaled_one + follow-up + scales (the whole one-pass scaled step; p {w.p_kind}, "
                       f"g {w.g_dtype}, p_out {p_out or 'none'})" if scaled and w.scaled_passes == 1 else
                       f"adam_scaled_maxima + fold + adam_scaled_pass + scales (the whole scaled step of the main group; "
                       f"p {w.p_kind}, g {w.g_dtype}, p_out {p_out or 'none'})" if scaled else
                       f"adam_update (p {w.p_kind}, g {w.g_dtype}, m/v {mv_desc}, p_out "
                       f"{p_out or 'none'}, {'AdamW' if w.mode else 'L2'}, non-capturable)"),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(w.name),
            "launch_ms_mean": round(launch_ms, 4),
            "algorithmic_bytes_per_launch": launch_bytes,
        },
    }

    # --- the streaming ceiling of the same stream mix, interleaved -----------
    probe = None if args.no_ceiling else probe_library()
    if args.no_ceiling:
        result["ceiling"] = None
    elif probe is None:
        result["ceiling"] = {"skipped": f"{PROBE_LIBRARY} is not built"}
    else:
        result["ceiling"] = interleaved_rounds(r, probe, one_step_noncap, args.steps, args.rounds)
        log(f"ceiling: probe {result['ceiling']['gbps']} GB/s, update {result['ceiling']['update_gbps']} GB/s "
            f"(update / ceiling {result['ceiling']['update_over_ceiling']})")

    # --- capturable, eager and graph -----------------------------------------
    cap_fn, d_lr, d_noop, one_step_cap = r.cap_fn, r.d_lr, r.d_noop, r.one_step_cap
    if not args.no_capturable and cap_fn is not None:
        for _ in range(args.warmup):
            one_step_cap()
        cap_wall, cap_per = timed(one_step_cap, args.steps)
        log(f"capturable: {cap_wall:.3f} ms/step wall")
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            one_step_cap(None, side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            one_step_cap(None, side)
        torch.cuda.synchronize()
        g_wall, _ = timed(lambda ev: graph.replay(), args.steps, events=False)
        log(f"graph replay: {g_wall:.3f} ms/step wall")
        result["capturable"] = {
            "ms_per_step": round(cap_wall, 4),
            "value": round(bytes_step / (cap_wall * 1e-3) / 1e9, 2),
            "launch_ms_mean": round(statistics.mean(cap_per), 4),
            "vs_noncapturable": round(cap_wall / wall_ms, 4),
        }
        result["graph_replay"] = {
            "ms_per_step": round(g_wall, 4),
            "value": round(bytes_step / (g_wall * 1e-3) / 1e9, 2),
            "vs_noncapturable": round(g_wall / wall_ms, 4),
        }

        # The whole capturable optimizer step: reset the grad scale, gradient
        # sum of squares over every group, clip / found-inf, capturable update
        # of every group; eager, then as one graph.
        d_sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
        d_norm = torch.zeros(1, dtype=torch.float32, device="cuda")
        d_full_scale = torch.ones(1, dtype=torch.float32, device="cuda")
        max_norm = 1.0

        def one_full_step(ev=None, s=stream):
            d_full_scale.fill_(w.grad_scale)
            for i, (tl, _, _, _, _) in enumerate(handles):
                launch_timed(ev if i == 0 else None,
                             lambda: A.adam_grad_sumsq(tl, d_sumsq, i > 0, s))
            A.adam_clip_grad_scale(d_sumsq, d_full_scale, max_norm, d_norm, d_noop, s)
            for tl, hp, _, _, d_step in handles:
                cap_fn(tl, hp, d_lr, d_step, d_full_scale, d_noop, s)

        for _ in range(args.warmup):
            one_full_step()
        full_wall, sumsq_per = timed(one_full_step, args.steps)
        log(f"full capturable step (sum of squares, clip, update): {full_wall:.3f} ms/step wall")
        graph2 = torch.cuda.CUDAGraph()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            one_full_step(None, side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph2, stream=side):
            one_full_step(None, side)
        torch.cuda.synchronize()
        full_g_wall, _ = timed(lambda ev: graph2.replay(), args.steps, events=False)
        log(f"full capturable step as one graph: {full_g_wall:.3f} ms/step wall")
        g_bytes = handles[0][2] * (4 if w.g_dtype == "f32" else 2)
        sumsq_ms = statistics.mean(sumsq_per)
        result["full_capturable_step"] = {
            "what": "grad-scale reset + gradient sum of squares (all groups) + clip/found-inf "
                    "+ capturable update (all groups)",
            "ms_per_step": round(full_wall, 4),
            "graph_ms_per_step": round(full_g_wall, 4),
            "graph_vs_update_only": round(full_g_wall / wall_ms, 4),
            "grad_sumsq_launch_ms": round(sumsq_ms, 4),
            "grad_sumsq_gbps": round(g_bytes / (sumsq_ms * 1e-3) / 1e9, 1),
        }

    # --- two-buffer state: the same step reading one buffer set of p, m, v
    # (and remainders) and writing a second one (adam_tl_build_two_buffer) ---
    if not scaled and not args.no_two_buffer:
        keys = [k for k in ("p", "rem", "m", "v") if k in bufs]
        extra = sum(bufs[k].numel() * bufs[k].element_size() for k in keys)
        free, _ = torch.cuda.mem_get_info()
        if extra * 1.02 + (2 << 30) > free:
            result["two_buffer_state"] = {
                "skipped": f"a second set of p, m, v ({extra / 1e9:.1f} GB) does not fit beside the first "
                           f"({free / 1e9:.1f} GB free)"}
        else:
            alt_bufs = {k: torch.empty_like(bufs[k]) for k in keys}
            tb_handles = []
            off = 0
            for (sizes, wd), (_, hp, n, _, _) in zip(groups, handles):
                views = {k: split_views(v[off:off + n], sizes) for k, v in bufs.items()}
                aviews = {k: split_views(v[off:off + n], sizes) for k, v in alt_bufs.items()}
                tensors = [{k: views[k][i] for k in views} for i in range(len(sizes))]
                alts = [{k: aviews[k][i] for k in aviews} for i in range(len(sizes))]
                desc = A.make_desc(g=w.g_dtype, p=w.p_kind, p_out=p_out, chunk_elems=args.chunk_elems)
                tb_handles.append((A.adam_tl_build(tensors, desc, alternates=alts), hp, A.HostStep(0)))
                off += n

            def one_step_tb(ev=None):
                for i, (tl, hp, host_step) in enumerate(tb_handles):
                    launch_timed(ev if i == 0 else None,
                                 lambda: step_fn(tl, hp, w.lr, host_step, 1.0, d_scale, stream))

            for _ in range(args.warmup):
                one_step_tb()
            tb_wall, tb_per = timed(one_step_tb, args.steps)
            tb_launch = statistics.mean(tb_per)
            tb_achieved = launch_bytes / (tb_launch * 1e-3) / 1e9
            log(f"two-buffer state: {tb_wall:.3f} ms/step wall, {bytes_step / (tb_wall * 1e-3) / 1e9:.1f} GB/s")
            result["two_buffer_state"] = {
                "what": "the same non-capturable step with p, m, v (and remainders) read from one buffer set "
                        "and written to a second (adam_tl_build_two_buffer); same algorithmic bytes",
                "ms_per_step": round(tb_wall, 4),
                "value": round(bytes_step / (tb_wall * 1e-3) / 1e9, 2),
                "pct_of_hbm_peak": round(100 * bytes_step / (tb_wall * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                "launch_ms_mean": round(tb_launch, 4),
                "achieved": round(tb_achieved, 2),
                "frac": round(tb_achieved / HBM_PEAK_GBPS, 4),
                "vs_in_place": round(tb_wall / wall_ms, 4),
                "traffic": measured_traffic(w.name, "two_buffer_bytes_per_launch"),
                "extra_device_bytes": extra,
            }
            for h in tb_handles:
                h[0].destroy()
            del alt_bufs

    r.destroy()
    del bufs, scale_bufs, r
    torch.cuda.empty_cache()

    # --- the other configurations, each with its own ceiling -----------------
    extra = [] if args.no_extra or args.workload != "bench201" else \
        [x for x in args.extra.split(",") if x and x != w.name]
    if extra:
        if probe is None and not args.no_ceiling:
            probe = probe_library()
        result["workloads"] = {}
        for name in extra:
            result["workloads"][name] = measure_extra(name, args, A, torch, None if args.no_ceiling else probe)
            print(f"[bench] {name}: " + json.dumps({k: v for k, v in result['workloads'][name].items()
                                                    if k not in ('cpu_baseline', 'ceiling')}),
                  file=sys.stderr, flush=True)

    if not args.no_cpu:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_elements, args.cpu_steps)
        log(f"cpu baseline: {result['cpu_baseline']['value']} GB/s on {result['cpu_baseline']['cores']} cores")
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
