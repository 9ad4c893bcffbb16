#!/usr/bin/env python
"""Benchmark of the gated delta-rule forward on one MI355X.

One step = one kda_fwd_chunked call (two launches: the chunk-parallel prep/WY
kernel, then the sequential state-and-output kernel) over one batch of
synthetic inputs already resident in HBM.
The default workload is the scalar-gated DK = DV = 128 case
(B8 T4096 H16, chunk 64, initial state); the printed JSON line also carries the
per-channel-gated DK = DV = 128 case and the single-token decode as extra
measurements, the roofline of the chunked kernel (HIP-event kernel time,
algorithmic bytes) and the fp64 CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --write-traffic FETCH_DIR WRITE_DIR   (profiles/traffic.json
        from two rocprofv3 --pmc runs of this script with --calibrate-copy)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunked fwd tokens/s + MFMA util (DK=DV=128); decode state GB/s vs HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_F16 = 2.5e15         # MI355X dense fp16/bf16 MFMA, flop/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
SIMDS = 256 * 4                # MI355X: 256 CUs of 4 SIMDs
KERNEL_SOURCES = ["chunked_impl.h", "chunked_layout.h", "common.h"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gated_delta_rule_fwd_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def act_bytes(w) -> int:
    return 4 if w.dtype == "f32" else 2


def chunked_bytes(w) -> int:
    """Algorithmic HBM bytes of one chunked call: every input read once, o and
    the final state written once."""
    a = act_bytes(w)
    tok = w.B * w.T * w.H
    per_tok = (2 * w.DK + w.DV + 1) * a + w.DV * 4
    if w.decay_kind == 1:
        per_tok += a
    elif w.decay_kind == 2:
        per_tok += w.DK * a
    state = w.B * w.H * w.DK * w.DV * 4
    return tok * per_tok + state * (2 if w.init_state else 1)


def chunked_flops(w) -> float:
    """Algorithmic flops of the chunked WY form, dense C x C tiles: per
    token-head 3 C DK + 2 C DV + 3 DK DV + C^2 / 6 multiply-adds."""
    C = w.chunk
    macs = 3 * C * w.DK + 2 * C * w.DV + 3 * w.DK * w.DV + C * C / 6
    return 2.0 * macs * w.B * w.T * w.H


def decode_bytes(w) -> int:
    a = act_bytes(w)
    bh = w.B * w.H
    per = 2 * w.DK * w.DV * 4 + (2 * w.DK + w.DV + 1) * a + w.DV * 4
    if w.decay_kind == 1:
        per += a
    elif w.decay_kind == 2:
        per += w.DK * a
    return bh * per


def to_dev(inp, dev):
    return {k: (None if v is None else v.to(dev)) for k, v in inp.items()}


WARM_SECONDS = 0.5


def warm_up(call, warmup):
    """The untimed warm-up: at least `warmup` calls, and more until the GPU
    has been busy for WARM_SECONDS (its clocks ramp up over the first few
    hundred milliseconds of work; without this a short run times the ramp)."""
    import torch
    n, t0 = 0, time.perf_counter()
    while n < warmup or time.perf_counter() - t0 < WARM_SECONDS:
        for _ in range(8):
            call()
        n += 8
        torch.cuda.synchronize()


def time_chunked(w, steps, warmup, dev, raw=False):
    """raw: the raw gate and raw beta of make_transform_inputs, transformed in
    the kernels (gate floor -5, beta sigmoid)."""
    import torch
    from gated_delta_rule_fwd_amd import fwd_chunked
    from gated_delta_rule_fwd_amd.inputs import make_inputs, make_transform_inputs
    o = torch.empty((w.B, w.T, w.hv, w.DV), device=dev, dtype=torch.float32)
    fs = torch.empty((w.B, w.hv, w.DK, w.DV), device=dev, dtype=torch.float32)
    if raw:
        d = to_dev(make_transform_inputs(w), dev)
        args = (d["q"], d["k"], d["v"], d["beta_logits"], d["gate"], d["initial_state"])
        tkw = dict(use_gate_in_kernel=True, A_log=d["A_log"], dt_bias=d["dt_bias"],
                   lower_bound=-5.0, use_beta_sigmoid_in_kernel=True)
    else:
        d = to_dev(make_inputs(w), dev)
        args = (d["q"], d["k"], d["v"], d["beta"], d["decay"], d["initial_state"])
        tkw = {}
    # the caller-owned workspace, allocated once outside the timed calls
    from gated_delta_rule_fwd_amd import chunked_workspace_bytes
    ws = torch.empty(chunked_workspace_bytes(w.B, w.T, w.H, w.hv, w.DK, w.DV, args[0].dtype,
                                             w.decay_kind, w.chunk), dtype=torch.uint8, device=dev)
    call = lambda: fwd_chunked(*args, chunk_size=w.chunk, out=o, final_state=fs, workspace=ws,
                               **tkw)
    warm_up(call, warmup)
    # Events on torch's current stream, which is the stream the library launches on.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for s, e in evs:
        s.record()
        call()
        e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [s.elapsed_time(e) for s, e in evs]
    return wall / steps * 1e3, sum(kern_ms) / len(kern_ms), min(kern_ms)


def backward_bytes(w) -> int:
    """Algorithmic HBM bytes of one backward call: q, k, v, beta, the decay
    and do read once, dq, dk, dv, dbeta and the decay gradient written once
    (fp32), the initial state and the final-state gradient read and the
    initial-state gradient written (the workspace's records are not
    counted)."""
    a = act_bytes(w)
    gate = {0: 0, 1: 1, 2: w.DK}[w.decay_kind]
    qk = w.B * w.T * w.H * 2 * w.DK * (a + 4)                       # q, k read; dq, dk written
    per_tok = (w.DV + 1 + gate) * a + w.DV * 4 + (w.DV + 1 + gate) * 4   # v beta decay do; dv dbeta ddecay
    state = w.DK * w.DV * 4 * (3 if w.init_state else 2)
    return qk + w.B * w.T * w.hv * per_tok + w.B * w.hv * state


BWD_CHUNK = 32                  # tokens per chunk of the chunked backward
MFMA_PEAK_F32 = 157.3e12        # MI355X dense fp32 MFMA, flop/s


def backward_flops(w) -> int:
    """Algorithmic flops of one chunked backward call, its contractions as
    dense tiles (chunks of C = 32): per token-head 2 (11 DK DV + 6 C DK +
    2 C DV).  The state walks: K S and the state update (2 DK DV), K dS and
    the dS update with q and k (3 DK DV); per chunk: K S0, Q S0, K dS1 and
    dO S0^T, D dS1^T, dY S0^T (6 DK DV); K K^T and Q K^T in the prep, K K^T
    again and Z K, dG K, Z^T Q at the end (6 C DK); dT and dP (2 C DV)."""
    C = BWD_CHUNK
    return 2 * (11 * w.DK * w.DV + 6 * C * w.DK + 2 * C * w.DV) * w.B * w.T * w.hv


def time_backward(w, steps, warmup, dev):
    """Per-call time (HIP events on the launch stream) of kda_bwd on workload
    w, from do and a final-state gradient; the workspace is allocated once."""
    import torch
    from gated_delta_rule_fwd_amd import bwd
    from gated_delta_rule_fwd_amd.inputs import make_inputs
    d = to_dev(make_inputs(w), dev)
    g = torch.Generator(device=dev).manual_seed(7)
    do = torch.randn((w.B, w.T, w.hv, w.DV), device=dev, generator=g)
    dST = torch.randn((w.B, w.hv, w.DK, w.DV), device=dev, generator=g)
    import gated_delta_rule_fwd_amd.kda as K
    ws = torch.empty(max(1, K.lib().kda_bwd_workspace_bytes(w.B, w.T, w.hv, w.DK, w.DV)),
                     dtype=torch.uint8, device=dev)
    call = lambda: bwd(d["q"], d["k"], d["v"], d["beta"], d["decay"], d["initial_state"], do, dST,
                       workspace=ws)
    call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for s_, e in evs:
        s_.record()
        call()
        e.record()
    torch.cuda.synchronize()
    return sum(s_.elapsed_time(e) for s_, e in evs) / steps


VARLEN_SEQS = 16


def varlen_lengths(total, n, seed=2024):
    """n sequence lengths summing to total, from a seeded gamma(2) mix (a
    spread of short and long prompts, none empty)."""
    import numpy as np
    x = np.random.default_rng(seed).gamma(2.0, size=n)
    lens = np.maximum(1, np.floor(x / x.sum() * total)).astype(np.int64)
    lens[-1] += total - lens.sum()
    return [int(v) for v in lens]


def time_chunked_varlen(w, steps, warmup, dev):
    """The workload's B*T tokens per head packed as VARLEN_SEQS sequences of
    mixed lengths (one launch pair over all of them), a state per sequence."""
    import torch
    from gated_delta_rule_fwd_amd import fwd_chunked_varlen
    from gated_delta_rule_fwd_amd.inputs import make_inputs
    d = to_dev(make_inputs(w), dev)
    tot = w.B * w.T
    pack = lambda x: None if x is None else x.reshape((1, tot) + tuple(x.shape[2:])).contiguous()
    q, k, v, be, de = (pack(d[n]) for n in ("q", "k", "v", "beta", "decay"))
    lens = varlen_lengths(tot, VARLEN_SEQS)
    cu = torch.tensor([0] + list(torch.tensor(lens).cumsum(0).tolist()), dtype=torch.int32)
    g = torch.Generator().manual_seed(7)
    s0 = (0.1 * torch.randn((VARLEN_SEQS, w.H, w.DK, w.DV), generator=g)).to(dev)
    o = torch.empty((1, tot, w.H, w.DV), device=dev, dtype=torch.float32)
    fs = torch.empty((VARLEN_SEQS, w.H, w.DK, w.DV), device=dev, dtype=torch.float32)
    cu_dev = cu.to(dev)
    from gated_delta_rule_fwd_amd.kda import chunked_varlen_workspace_bytes
    nws = chunked_varlen_workspace_bytes(cu, w.H, w.hv, w.DK, w.DV, q.dtype, w.decay_kind, w.chunk)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    call = lambda: fwd_chunked_varlen(q, k, v, be, cu_dev, decay=de, initial_state=s0,
                                      chunk_size=w.chunk, out=o, final_state=fs, workspace=ws)
    warm_up(call, warmup)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for s, e in evs:
        s.record()
        call()
        e.record()
    torch.cuda.synchronize()
    kern_ms = [s.elapsed_time(e) for s, e in evs]
    state = VARLEN_SEQS * w.H * w.DK * w.DV * 4
    byts = chunked_bytes(w) - w.B * w.H * w.DK * w.DV * 4 * (2 if w.init_state else 1) + 2 * state
    return sum(kern_ms) / len(kern_ms), byts, lens


def time_decode(w, steps, warmup, dev, state_v_first=False):
    """state_v_first: value-major states [B, H, DV, DK] (the same bytes)."""
    import torch
    from gated_delta_rule_fwd_amd import decode_step
    from gated_delta_rule_fwd_amd.inputs import make_inputs
    inp = make_inputs(w)
    d = to_dev(inp, dev)
    # two state buffers used alternately so consecutive calls stream different memory
    s0 = d["initial_state"]
    if state_v_first:
        s0 = s0.transpose(-1, -2).contiguous()
    states = [s0, s0.clone()]
    o = torch.empty((w.B, w.H, w.DV), device=dev, dtype=torch.float32)
    args = (d["q"], d["k"], d["v"], d["beta"], d["decay"])
    it = iter(range(1 << 30))
    kw = dict(out=o, state_v_first=state_v_first)
    warm_up(lambda: decode_step(*args, states[next(it) % 2], **kw), warmup)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i, (s, e) in enumerate(evs):
        s.record()
        decode_step(*args, states[i % 2], **kw)
        e.record()
    torch.cuda.synchronize()
    ms = [s.elapsed_time(e) for s, e in evs]
    return sum(ms) / len(ms)


CPU_SECONDS = 10.0


def cpu_baseline(w):
    """The fp64 oracle, as it is, on whole sequences (all heads, full length)
    of the workload, one after another until CPU_SECONDS have passed or all
    are done; scaled to tokens/s of the same head count."""
    import numpy as np
    from gated_delta_rule_fwd_amd.inputs import make_inputs
    from oracle import kda_scan
    inp = make_inputs(w)
    nb, t0, c0 = 0, time.perf_counter(), time.process_time()
    while nb < w.B and (nb == 0 or time.perf_counter() - t0 < CPU_SECONDS):
        sl = slice(nb, nb + 1)
        kda_scan(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["beta"][sl],
                 None if inp["decay"] is None else inp["decay"][sl],
                 None if inp["initial_state"] is None else inp["initial_state"][sl])
        nb += 1
    dt = time.perf_counter() - t0
    # threads actually used: the process's CPU time over the wall time
    used = max(1, round((time.process_time() - c0) / dt))
    return {"value": nb * w.T / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "seconds": round(dt, 2), "host_cores": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model(),
            "sample": f"{w.name}: {nb} of {w.B} sequences x {w.H} heads x {w.T} tokens, "
                      f"NumPy fp64 sequential scan (numpy {np.__version__}); "
                      f"cores = threads used (process CPU time / wall time), "
                      f"host_cores = cores this process may run on"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def stored_traffic(name):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    ent = t.get(name)
    if not ent or ent.get("kernel_hash") != kernel_hash():
        return None   # counters were taken on another version of the kernels
    return ent.get("bytes_per_call")


def stored_counters(name):
    """The MFMA figures of one call of workload `name` from profiles/counters.json
    (None if the counters were taken on other kernel sources): the matrix
    units' busy fraction over the call (busy SIMD-cycles of its kernels over
    their cycles x 1024 SIMDs; GRBM_GUI_ACTIVE is summed over the 8 XCDs)
    and the MFMA flops executed."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    ent = c.get(name)
    if not ent or c.get("kernel_hash") != kernel_hash():
        return None
    busy = sum(k.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) for k in ent.values())
    cycles = sum(k.get("GRBM_GUI_ACTIVE", 0) / 8 for k in ent.values())
    flops = sum(k.get("mfma_flops", 0) for k in ent.values())
    if not cycles:
        return None
    return {"mfma_busy_frac": round(busy / (cycles * SIMDS), 4), "mfma_flops_executed": flops}


# kernel-name fragments of one call of each workload, as rocprofv3 prints them
TRAFFIC_KERNELS = {
    "gdn_d128": ["prep_kernel<128, 64, kda::bf16_t, 1, false>", "state_kernel<128, 64, 64, kda::bf16_t, 1>"],
    "kda_d128": ["prep_kernel<128, 64, kda::bf16_t, 2, false>", "state_kernel<128, 32, 64, kda::bf16_t, 2>"],
    "deltanet_d64": ["prep_kernel<64, 64, kda::bf16_t, 0, false>", "state_kernel<64, 16, 64, kda::bf16_t, 0>"],
    "decode_d128": ["decode_kernel<128, 128, kda::bf16_t>"],
}
# Later workloads of the same run reuse some of these kernels (the grouped-head
# and packed gdn calls, the raw-gate kda call): a workload's dispatches are
# those before the first dispatch of the kernel named here.
TRAFFIC_WINDOW_END = {
    "gdn_d128": "prep_kernel<128, 64, kda::bf16_t, 2,",
    "kda_d128": "prep_kernel<128, 64, kda::bf16_t, 2, true>",
    "deltanet_d64": None,
    "decode_d128": None,
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30   # the --calibrate-copy copies: 1 GiB read and 1 GiB written


def write_traffic(fetch_dir, write_dir):
    """profiles/traffic.json from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs
    (KiB per dispatch): each counter is scaled by what it read for a plain
    1 GiB device copy, then averaged over dispatches of each kernel and summed
    over the kernels of one call."""
    import csv
    import glob

    def per_kernel(d, counter):
        """[(dispatch id, kernel name, bytes)] in dispatch order"""
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r["Counter_Name"] == counter:
                        rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"],
                                     float(r["Counter_Value"]) * 1024))
        return sorted(rows)

    out = {"_comment": "HBM bytes per call from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE "
                       "(KiB per dispatch), each scaled by the ratio of a plain 1 GiB device "
                       "copy's true bytes to what the same counter read for it, summed over the "
                       "kernels of one call; kernel_hash names the chunked kernel sources",
           "kernel_hash": kernel_hash()}
    scale = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        v = per_kernel(d, counter)
        copies = [x for _, k, x in v if COPY_KERNEL in k and x > COPY_BYTES / 2]
        if not copies:
            raise SystemExit(f"no 1 GiB calibration copy found under {d}")
        scale[counter] = COPY_BYTES / (sum(copies) / len(copies))
        out[counter.lower() + "_scale"] = round(scale[counter], 4)
        for name, frags in TRAFFIC_KERNELS.items():
            ent = out.setdefault(name, {"kernels": frags})
            end = TRAFFIC_WINDOW_END[name]
            last = min([i for i, k, _ in v if end and end in k], default=None)
            total = 0.0
            for fr in frags:
                xs = [x for i, k, x in v if fr in k and (last is None or i < last)]
                if not xs:
                    raise SystemExit(f"{counter}: no dispatch of {fr} under {d}")
                total += sum(xs) / len(xs) * scale[counter]
            ent[counter.lower() + "_bytes"] = int(total)
    for name in TRAFFIC_KERNELS:
        ent = out[name]
        ent["bytes_per_call"] = ent["fetch_size_bytes"] + ent["write_size_bytes"]
        ent["kernel_hash"] = None if name.startswith("decode") else out["kernel_hash"]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def write_counters(dirs, out=COUNTERS_FILE):
    """profiles/counters.json from rocprofv3 --pmc runs of this script (any
    number of passes): per workload and kernel the mean of every counter
    over that kernel's dispatches in the workload's window (as for the HBM
    traffic), and the MFMA figures derived from them: utilisation =
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs) and executed MFMA
    flops = 512 x the MOPS counters."""
    import csv
    import glob
    passes = []   # per pass directory: [(dispatch, kernel, counter, value)]
    for d in dirs:
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], r["Counter_Name"],
                                 float(r["Counter_Value"])))
        passes.append(rows)
    res = {"_comment": "mean per dispatch of each rocprofv3 --pmc counter over the dispatches of "
                       "each kernel of one call of the workload (dispatches before the first "
                       "one of the next workload that reuses the kernel); mfma_util = "
                       "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 1024 SIMDs), "
                       "mfma_flops = 512 x (MOPS_F16 + MOPS_BF16 + MOPS_F32)",
           "kernel_hash": kernel_hash()}
    for name, frags in TRAFFIC_KERNELS.items():
        end = TRAFFIC_WINDOW_END[name]
        ent = {}
        for fr in frags:
            sums, counts = {}, {}
            for rows in passes:
                last = min([i for i, k, _, _ in rows if end and end in k], default=None)
                for i, k, c, v in rows:
                    if fr in k and (last is None or i < last):
                        sums[c] = sums.get(c, 0.0) + v
                        counts[c] = counts.get(c, 0) + 1
            if not sums:
                continue
            kc = {c: sums[c] / counts[c] for c in sums}
            if "SQ_VALU_MFMA_BUSY_CYCLES" in kc and "GRBM_GUI_ACTIVE" in kc:
                kc["mfma_util"] = kc["SQ_VALU_MFMA_BUSY_CYCLES"] / (kc["GRBM_GUI_ACTIVE"] * SIMDS)
            mops = [kc.get(c) for c in ("SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                                        "SQ_INSTS_VALU_MFMA_MOPS_F32")]
            if all(m is not None for m in mops):
                kc["mfma_flops"] = 512.0 * sum(mops)
            ent[fr] = {c: round(v, 4) if abs(v) < 1e6 else round(v) for c, v in sorted(kc.items())}
        res[name] = ent
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res, indent=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gdn_d128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--write-counters", nargs="+", metavar="PMC_DIR",
                    help="write profiles/counters.json from rocprofv3 --pmc runs and exit")
    ap.add_argument("--counters-out", default=COUNTERS_FILE)
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.write_counters:
        write_counters(args.write_counters, args.counters_out)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); each (batch, head) is independent, so a "
              f"multi-GPU run would be this single-GPU kernel on each GPU's share.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_fwd_amd.inputs import WORKLOADS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    w = WORKLOADS[args.workload]
    if w.decode:
        print("--workload must be a chunked workload", file=sys.stderr)
        sys.exit(2)

    ms_step, kern_ms, kern_min = time_chunked(w, args.steps, args.warmup, dev)
    tokens = w.B * w.T
    byts = chunked_bytes(w)
    flops = chunked_flops(w)
    achieved = byts / (kern_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": stored_traffic(w.name),
            "kernel": "prep_kernel + state_kernel (one chunked call)", "kernel_ms_mean": round(kern_ms, 4),
            "kernel_ms_min": round(kern_min, 4), "algorithmic_bytes": byts,
            "mfma_frac_dense_count": round(flops / (kern_ms * 1e-3) / MFMA_PEAK_F16, 4),
            "mfma_counters": stored_counters(w.name)}
    line = {
        "metric": METRIC,
        "value": round(tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16+bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "DK": w.DK, "DV": w.DV,
                   "chunk": w.chunk, "decay": w.decay, "initial_state": w.init_state,
                   "activations": w.dtype, "mfma": "f16 x f16 and bf16 x bf16 -> f32", "state": "f32",
                   "output": "f32"},
        "roofline": roof,
    }
    if not args.no_extra:
        extra = {}
        w4 = WORKLOADS["kda_d128"]
        if w4.name != w.name:
            m4, k4, _ = time_chunked(w4, max(3, args.steps // 2), args.warmup, dev)
            extra[w4.name] = {"tokens_per_s": round(w4.B * w4.T / (m4 * 1e-3), 1),
                              "kernel_ms_mean": round(k4, 4),
                              "hbm_frac": round(chunked_bytes(w4) / (k4 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "mfma_frac_dense_count": round(chunked_flops(w4) / (k4 * 1e-3) / MFMA_PEAK_F16, 4)}
            # the same shape from the raw gate and raw beta, transformed in the prep kernel
            _, k4r, _ = time_chunked(w4, max(3, args.steps // 2), args.warmup, dev, raw=True)
            extra[w4.name + "_raw_gate"] = {
                "tokens_per_s": round(w4.B * w4.T / (k4r * 1e-3), 1), "kernel_ms_mean": round(k4r, 4),
                "hbm_frac": round(chunked_bytes(w4) / (k4r * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "transforms": "gate -exp(A_log) softplus(gate + dt_bias) floored at -5, beta sigmoid"}
        # the ungated D64 workload (B4 T2048 H16; its 85 MB fit in the 256 MB
        # last-level cache, so the figure is cache-warm)
        w2 = WORKLOADS["deltanet_d64"]
        if w2.name != w.name:
            _, k2, _ = time_chunked(w2, max(3, args.steps // 2), args.warmup, dev)
            extra[w2.name] = {"tokens_per_s": round(w2.B * w2.T / (k2 * 1e-3), 1),
                              "kernel_ms_mean": round(k2, 4),
                              "algorithmic_bytes": chunked_bytes(w2),
                              "hbm_frac": round(chunked_bytes(w2) / (k2 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "mfma_frac_dense_count": round(chunked_flops(w2) / (k2 * 1e-3) / MFMA_PEAK_F16, 4)}
        # the same shape with grouped value heads: 4 q/k heads, 16 value heads
        wg = w.scaled(H=4, HV=w.H)
        _, kg, _ = time_chunked(wg, max(3, args.steps // 2), args.warmup, dev)
        extra[w.name + "_gva4"] = {"H": wg.H, "HV": wg.hv, "tokens_per_s": round(wg.B * wg.T / (kg * 1e-3), 1),
                                   "kernel_ms_mean": round(kg, 4)}
        # the same tokens as packed sequences of mixed lengths
        vk, vb, lens = time_chunked_varlen(w, max(3, args.steps // 2), args.warmup, dev)
        extra[w.name + "_varlen"] = {
            "sequences": VARLEN_SEQS, "tokens": w.B * w.T, "min_len": min(lens), "max_len": max(lens),
            "tokens_per_s": round(w.B * w.T / (vk * 1e-3), 1), "kernel_ms_mean": round(vk, 4),
            "hbm_frac": round(vb / (vk * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        # the backward (kda_bwd) at the headline shape and at the per-channel
        # one: the chunked form, fp32 MFMA contractions
        for wb in (w, WORKLOADS["kda_d128"]):
            b_ms = time_backward(wb, max(3, args.steps // 20), args.warmup, dev)
            extra[wb.name + "_backward"] = {
                "kernel_ms_mean": round(b_ms, 3), "tokens_per_s": round(wb.B * wb.T / (b_ms * 1e-3), 1),
                "algorithmic_flops": backward_flops(wb),
                "mfma_f32_frac": round(backward_flops(wb) / (b_ms * 1e-3) / MFMA_PEAK_F32, 4),
                "algorithmic_bytes": backward_bytes(wb),
                "hbm_frac": round(backward_bytes(wb) / (b_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
                "form": "chunked WY (C = 32), fp32 MFMA contractions"}
        w5 = WORKLOADS["decode_d128"]
        d_ms = time_decode(w5, max(5, args.steps), args.warmup, dev)
        gbs = decode_bytes(w5) / (d_ms * 1e-3) / 1e9
        extra[w5.name] = {"kernel_ms_mean": round(d_ms, 4), "GB_per_s": round(gbs, 1),
                          "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                          "bytes_per_call": decode_bytes(w5)}
        d_vm = time_decode(w5, max(5, args.steps), args.warmup, dev, state_v_first=True)
        gbs_vm = decode_bytes(w5) / (d_vm * 1e-3) / 1e9
        extra[w5.name + "_value_major"] = {"kernel_ms_mean": round(d_vm, 4),
                                           "GB_per_s": round(gbs_vm, 1),
                                           "hbm_frac": round(gbs_vm / HBM_PEAK_GBS, 4)}
        line["extra"] = extra
        torch.cuda.empty_cache()
    if args.calibrate_copy:
        a = torch.empty(1 << 28, device=dev, dtype=torch.float32)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
