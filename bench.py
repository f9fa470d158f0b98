"""Benchmark of the KDA state layer on one MI355X.

Prints ONE JSON line.  The timed step is one chunked prefill over the KDA
batch B=2, H=32, T=32768, dk=dv=128 (bf16 q/k/v, fp32 per-channel log_a
clipped to [-8, 0], fp32 state); `value` is prefill tokens/s (each token
counted once across heads).  The decode leg (256 sequences x 32 heads,
dk=dv=128, 100 chained steps, fp32 state streamed once per step) is timed in
the same run and reported under "decode" in state GB/s.  All inputs are seeded
synthetic tensors, resident on the GPU before timing starts.  The same
prefill batch is also timed with state snapshots every 1024 tokens, with the
decay-first ordering, and from raw inputs through the input prologue (against
torch transforming them first), and the decode leg with the decay-first
ordering ("variants", "decode.decay_first").  The gradient of the same prefill
(kda_chunk_bwd, for seeded upstream derivatives) is timed as "backward".  Two
more prefill workloads get their own timing, roofline and parity under "legs":
Gated DeltaNet (scalar decay, 16 heads x 4096 tokens) and 64 packed sequences
of 512 to 16384 tokens x 32 heads.  The headline batch's every output and final
state is checked against the fp64 oracle ("parity"), whose run is also the CPU
baseline.

Timing uses HIP events recorded on the stream the kernels are launched on
(torch's current stream, which the library receives).  The fp64 CPU oracle is
timed afterwards on a bounded sample of the same prefill workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-variants] [--no-backward] [--no-legs]
                    [--only prefill|decode|gdn|varlen]
    python bench.py --copy-calibration   # plain device copy of known size, for counters
    python bench.py --record-traffic FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR
        # writes profiles/traffic_counters.json from four rocprofv3 --pmc output
        # folders (FETCH_SIZE and WRITE_SIZE of a bench run, then of --copy-calibration)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s (MFMA %peak) + decode-step state GB/s, 1 MI355X"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = {
    # the two-pass prefill that the bench runs: operator pass (dk = 128) and state pass
    "prefill": ["kda_recurrent_state_amd/csrc/kda_prep2.hip", "kda_recurrent_state_amd/csrc/kda_scan.hip",
                "kda_recurrent_state_amd/csrc/kda_ws.hpp", "kda_recurrent_state_amd/csrc/kda_chunk_common.hpp",
                "kda_recurrent_state_amd/csrc/kda_device.hpp", "kda_recurrent_state_amd/csrc/kda_api.cpp"],
    "decode": ["kda_recurrent_state_amd/csrc/kda_decode.hip", "kda_recurrent_state_amd/csrc/kda_device.hpp"],
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(kind):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def prefill_algorithmic(w, chunk_alg=64, tokens=None):
    """Algorithmic bytes and flops of one prefill pass (what the method must move
    and compute, not what the kernel executes).  Bytes per token-head: q, k, v
    in bf16, log_a fp32 per channel (GDN: one fp32 per token-head), beta fp32,
    o bf16; plus S0 read (when the workload has one) and S_T written once per
    (sequence, head).  Flops per chunk of C tokens per head:
      KDA: 10 C^2 dk + 6 C^2 dv + 8 C dk dv + (2/3) C^3 (four C x C Gram products,
           W, U, E, O, the two state products, the triangular solve);
      GDN: 6 C^2 dk + 4 C^2 dv + 6 C dk dv + (2/3) C^3 (two Gram products with a
           scalar decay mask, and one state-side product fewer).
    `tokens`: total tokens when the lengths vary (default n_seqs * seqlen)."""
    T = tokens if tokens is not None else w.n_seqs * w.seqlen
    th = T * w.heads
    la_bytes = 4 if w.scalar_decay else 4 * w.dk
    per_th = 2 * (2 * w.dk + w.dv) + la_bytes + 4 + 2 * w.dv
    states = w.n_seqs * w.heads * (2 if w.s0_std > 0 else 1) * 4 * w.dk * w.dv
    C, dk, dv = chunk_alg, w.dk, w.dv
    if w.scalar_decay:
        per_chunk = 6 * C * C * dk + 4 * C * C * dv + 6 * C * dk * dv + (2.0 / 3.0) * C ** 3
    else:
        per_chunk = 10 * C * C * dk + 6 * C * C * dv + 8 * C * dk * dv + (2.0 / 3.0) * C ** 3
    return th * per_th + states, th * per_chunk / C


def backward_algorithmic(w, chunk_alg=64):
    """Algorithmic bytes and flops of one gradient call.  Bytes per token-head:
    q, k, v and dO read in bf16, log_a and beta read in fp32; dq, dk, dv written
    in bf16, dlog_a and dbeta in fp32; per (sequence, head) S0 and dS_T read and
    dS0 written (fp32).  Flops: twice the prefill's (reverse mode runs two
    products of the same size for every product of the chunk form), plus once
    the prefill's for recovering the forward states."""
    th = w.n_seqs * w.seqlen * w.heads
    per_th = 2 * (2 * w.dk + 2 * w.dv) + 4 * w.dk + 4 + 2 * (2 * w.dk + w.dv) + 4 * w.dk + 4
    states = w.n_seqs * w.heads * 3 * 4 * w.dk * w.dv
    _, F = prefill_algorithmic(w, chunk_alg)
    return th * per_th + states, 3.0 * F


def decode_algorithmic(w):
    """Bytes of one decode step: the fp32 state read and written once, plus the
    token's q, k, v (bf16), log_a (fp32 per channel), beta and o."""
    per = 2 * 4 * w.dk * w.dv + 2 * (2 * w.dk + w.dv) + 4 * w.dk + 4 + 2 * w.dv
    return w.n_seqs * w.heads * per


def stored_traffic(kind, launch_bytes):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except OSError:
        return None
    ent = data.get(kind)
    if not ent or ent.get("source_hash") != source_hash(kind):
        return None
    return ent.get("hbm_bytes_per_launch")


def max_rel(x, r):
    """max |x - r| / max |r| over one whole output tensor (GPU tensor x, fp64 numpy r),
    computed in slices so that host memory stays bounded."""
    import numpy as np
    num = den = 0.0
    flat_x = x.reshape(x.shape[0], -1)
    flat_r = r.reshape(r.shape[0], -1)
    step = max(1, (1 << 26) // max(1, flat_r.shape[1]))
    for a in range(0, flat_r.shape[0], step):
        xs = flat_x[a:a + step].double().cpu().numpy()
        rs = flat_r[a:a + step]
        num = max(num, float(np.abs(xs - rs).max()))
        den = max(den, float(np.abs(rs).max()))
    return num / den if den > 0 else num


def host_info(threads):
    """The host the CPU baseline ran on: CPUs visible, CPUs this process may use,
    the CPU model, and the oracle's thread count (at most 16: the host CPU share
    that goes with one GPU on a shared machine)."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = None
    return {"nproc": os.cpu_count(), "affinity_cpus": aff, "cpu_model": model, "oracle_threads": threads}


def time_events(fn, iters, stream):
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / 1e3  # seconds


def copy_calibration(steps):
    """A plain device-to-device copy of 1 GiB, `steps` times: the reference
    against which the FETCH_SIZE / WRITE_SIZE counters are scaled."""
    import torch
    n = 1 << 28  # 1 GiB of fp32
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": steps}))


# kernels whose per-dispatch counters add up to one call of each measured entry point
KERNEL_SYMBOLS = {"prefill": ["kda_prep2_kernel", "kda_prep2_exact_kernel", "kda_scan_kernel"],
                  "decode": ["kda_decode_kernel"]}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _counter_means(folder, counter):
    """Mean counter value (KiB per dispatch) per kernel name in a rocprofv3 csv folder."""
    import csv
    import glob
    paths = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    acc = {}
    for p in paths:
        with open(p) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def record_traffic(fetch_dir, write_dir, cfetch_dir, cwrite_dir):
    """HBM bytes per launch of each kernel: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) scaled by what the same counters read for a plain 1 GiB copy."""
    fetch, write = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")
    cfetch, cwrite = _counter_means(cfetch_dir, "FETCH_SIZE"), _counter_means(cwrite_dir, "WRITE_SIZE")
    copy_kib = (1 << 30) / 1024.0
    fr = copy_kib / cfetch[COPY_KERNEL]
    wr = copy_kib / cwrite[COPY_KERNEL]
    out = {"copy_calibration": {"kernel": COPY_KERNEL, "bytes_each_way": 1 << 30,
                                "fetch_kib": cfetch[COPY_KERNEL], "write_kib": cwrite[COPY_KERNEL],
                                "fetch_scale": fr, "write_scale": wr}}
    for kind, syms in KERNEL_SYMBOLS.items():
        per = {}
        for sym in syms:
            f = [v for k, v in fetch.items() if sym in k]
            w = [v for k, v in write.items() if sym in k]
            if len(f) != 1 or len(w) != 1:
                break
            per[sym] = {"fetch_kib_raw": f[0], "write_kib_raw": w[0],
                        "hbm_read_bytes": f[0] * fr * 1024.0, "hbm_write_bytes": w[0] * wr * 1024.0}
        if len(per) != len(syms):
            continue
        rb = sum(v["hbm_read_bytes"] for v in per.values())
        wb = sum(v["hbm_write_bytes"] for v in per.values())
        out[kind] = {"kernels": per, "source_hash": source_hash(kind), "hbm_read_bytes": rb,
                     "hbm_write_bytes": wb, "hbm_bytes_per_launch": rb + wb}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def prefill_leg(leg, args, kda, dev, stream):
    """One more prefill workload, timed like the headline one (HIP events on the
    launch stream, inputs resident, default method and workspace):
      gdn    -- Gated DeltaNet (scalar log a per token and head), 1 x 16 heads x 4096
                tokens, d = 128, bf16, S0 = 0: whole batch checked against the oracle;
      varlen -- KDA, 64 packed sequences of U[512, 16384] tokens x 32 heads, d = 128,
                per-sequence S0: two sequences (all heads) checked against the oracle
                (every unit is checked by the GPU test suite)."""
    import numpy as np
    import torch
    from kda_recurrent_state_amd.workloads import WORKLOADS, generate
    from oracle import kda_oracle
    name = {"gdn": "gdn_h16_t4096_d128_bf16", "varlen": "kda_varlen_64seq_h32_d128"}[leg]
    w = WORKLOADS[name]
    log(f"leg {leg}: generating {name}")
    x = generate(w, seed=2 if leg == "gdn" else 5, device=dev)
    T = int(x["q"].shape[0])
    lens = np.asarray(x["lengths"], dtype=np.int64)
    maxlen = int(lens.max())
    o = torch.empty((T, w.heads, w.dv), dtype=w.dtype, device=dev)
    ST = torch.empty((w.n_seqs, w.heads, w.dk, w.dv), dtype=torch.float32, device=dev)
    wsb = kda.chunk_workspace_size(x["q"], x["v"], num_seqs=w.n_seqs, scalar_decay=w.scalar_decay,
                                   max_seqlen=maxlen)
    if args.workspace_mib and wsb:
        wsb = max(kda.chunk_workspace_size(x["q"], x["v"], num_seqs=w.n_seqs, scalar_decay=w.scalar_decay,
                                           max_seqlen=maxlen, minimum=True), args.workspace_mib << 20)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None

    def step():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["log_a"], x["beta"], S0=x["S0"], cu_seqlens=x["cu_seqlens"],
                      out=o, final_state=ST, workspace=ws, max_seqlen=maxlen)
    for _ in range(max(args.warmup, 3)):
        step()
    torch.cuda.synchronize()
    t = time_events(step, args.steps, stream) / args.steps
    m_run, chunk_run, split_run = kda.chunk_plan(x["q"], x["v"], num_seqs=w.n_seqs, packed=True, workspace_bytes=wsb,
                                                 scalar_decay=w.scalar_decay, max_seqlen=maxlen)
    B, F64 = prefill_algorithmic(w, 64, tokens=T)
    _, F32 = prefill_algorithmic(w, chunk_run, tokens=T)
    gbs = B / t / 1e9
    res = {"workload": name, "tokens": T, "ms_per_step": t * 1e3, "tokens_per_s": T / t,
           "method": "two-pass" if m_run == kda.METHOD_TWO_PASS else "single", "chunk": chunk_run,
           "dv_split": split_run, "workspace_MiB": round(wsb / 2**20, 1),
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": gbs / PEAK_HBM_GBS, "traffic": None, "algorithmic_bytes_per_launch": B,
                        "avg_launch_ms": t * 1e3},
           "mfma": {"algorithmic_tflop_at_C64": F64 / 1e12, "pct_peak": 100.0 * F64 / t / 1e12 / PEAK_BF16_TFLOPS,
                    "pct_peak_at_run_chunk": 100.0 * F32 / t / 1e12 / PEAK_BF16_TFLOPS}}
    if leg == "gdn":
        res["note"] = ("the workload names C = 64; at d = 128 the kernels run C = 32: a 64-token operator block "
                       "(65 KB in the decay-first form a scalar decay runs) leaves room for two slots of the state "
                       "pass's LDS ring, which needs three to keep its copies ahead of the walk")
        seqs = list(range(w.n_seqs))
    else:
        seqs = [int(np.argmax(lens)), int(np.argmin(lens))]
    # parity on the timed output
    cu = x["cu_seqlens"].cpu().numpy().astype(np.int64)
    eo = es = 0.0
    for n in seqs:
        a, b = int(cu[n]), int(cu[n + 1])
        h = {k_: x[k_][a:b].cpu() for k_ in ("q", "k", "v", "log_a", "beta")}
        S0 = None if x["S0"] is None else x["S0"][n:n + 1].cpu()
        ro, rS = kda_oracle(h["q"], h["k"], h["v"], h["log_a"], h["beta"], S0=S0)
        eo = max(eo, max_rel(o[a:b], ro))
        es = max(es, max_rel(ST[n:n + 1], rS))
    res["parity"] = {"o_max_rel_err": eo, "S_T_max_rel_err": es, "tol": 2e-2,
                     "checked": "whole batch" if leg == "gdn" else
                                f"sequences {seqs} (longest, shortest), all heads"}
    log(f"leg {leg}: {t*1e3:.3f} ms/step, {T/t/1e6:.2f} Mtok/s, {gbs:.0f} GB/s ({100*gbs/PEAK_HBM_GBS:.1f}%), "
        f"parity o {eo:.2e} S {es:.2e}")
    del x, o, ST, ws
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip the snapshot and decay-first legs")
    ap.add_argument("--no-backward", action="store_true", help="skip the gradient leg")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "gdn", "varlen"], default=None)
    ap.add_argument("--no-legs", action="store_true", help="skip the Gated DeltaNet and varlen prefill legs")
    ap.add_argument("--method", choices=["auto", "single", "two-pass"], default="auto")
    ap.add_argument("--workspace-mib", type=int, default=0, help="two-pass workspace size (default: preferred)")
    ap.add_argument("--record-traffic", nargs=4, metavar="DIR", default=None)
    args = ap.parse_args()

    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return

    if args.gpus != 1:
        print("bench.py measures one GPU only: the layer shards over (sequence, head) with no "
              "exchange, so run it once per GPU; --gpus above 1 is not supported.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.steps)
        return

    import numpy as np
    import torch

    import kda_recurrent_state_amd as kda
    from kda_recurrent_state_amd.workloads import WORKLOADS, generate

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    out = {"metric": METRIC}

    # ---------------- prefill: KDA B=2, H=32, T=32768 ----------------
    wp = WORKLOADS["kda_b2_h32_t32768_d128_bf16"]
    if args.only in (None, "prefill"):
        log("generating prefill inputs")
        x = generate(wp, seed=3, device=dev)
        o = torch.empty((x["q"].shape[0], wp.heads, wp.dv), dtype=wp.dtype, device=dev)
        ST = torch.empty((wp.n_seqs, wp.heads, wp.dk, wp.dv), dtype=torch.float32, device=dev)
        method = {"auto": kda.METHOD_AUTO, "single": kda.METHOD_SINGLE, "two-pass": kda.METHOD_TWO_PASS}[args.method]
        wsb = kda.chunk_workspace_size(x["q"], x["v"], num_seqs=wp.n_seqs, method=method, max_seqlen=wp.seqlen)
        if args.workspace_mib:
            wsb = max(wsb and kda.chunk_workspace_size(x["q"], x["v"], num_seqs=wp.n_seqs, method=method,
                                                       max_seqlen=wp.seqlen, minimum=True),
                      args.workspace_mib << 20)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
        # the configuration the library runs for this call (kda_chunk_plan)
        m_run, chunk_run, split_run = kda.chunk_plan(x["q"], x["v"], num_seqs=wp.n_seqs, packed=False,
                                                     workspace_bytes=wsb, method=method, max_seqlen=wp.seqlen)
        used = "two-pass" if m_run == kda.METHOD_TWO_PASS else "single"
        log(f"prefill method {used}, chunk {chunk_run}, dv split {split_run}, workspace {wsb / 2**20:.1f} MiB")

        def step():
            kda.chunk_fwd(x["q"], x["k"], x["v"], x["log_a"], x["beta"], S0=x["S0"],
                          cu_seqlens=x["cu_seqlens"], out=o, final_state=ST, method=method, workspace=ws,
                          max_seqlen=wp.seqlen)

        log("prefill warmup")
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        log("prefill timed")
        t = time_events(step, args.steps, stream)
        torch.cuda.synchronize()
        per = t / args.steps
        tokens = wp.n_seqs * wp.seqlen
        B, F = prefill_algorithmic(wp)
        gbs = B / per / 1e9
        tflops = F / per / 1e12
        out.update({
            "value": tokens / per, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": per * 1e3, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic: seeded tensors with the layer's shapes and value distributions (no dataset)",
            "config": {"workload": wp.name, "batch": wp.n_seqs, "heads": wp.heads, "seq_len": wp.seqlen,
                       "dk": wp.dk, "dv": wp.dv, "state": "fp32", "chunk": chunk_run, "dv_split": split_run,
                       "method": used, "workspace_MiB": round(wsb / 2**20, 1)},
        })
        # One prefill call is the unit: with the two-pass method it is one launch of the
        # operator pass and one of the state pass (a single segment at the preferred
        # workspace); the bytes are the method's algorithmic bytes, not the workspace's.
        kernels = ("kda_prep2_kernel + kda_prep2_exact_kernel + kda_scan_kernel" if used == "two-pass"
                   else "kda_chunk_kernel")
        out["roofline"] = {
            "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS,
            "traffic": stored_traffic("prefill", B) if used == "two-pass" else None,
            "kernel": kernels, "algorithmic_bytes_per_launch": B,
            "avg_launch_ms": per * 1e3,
        }
        _, F_run = prefill_algorithmic(wp, chunk_run)
        out["mfma"] = {"algorithmic_tflop_per_launch": F / 1e12, "achieved_tflops": tflops,
                       "peak_tflops": PEAK_BF16_TFLOPS, "pct_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
                       "pct_peak_at_run_chunk": 100.0 * F_run / per / 1e12 / PEAK_BF16_TFLOPS,
                       "algorithmic_tflop_at_run_chunk": F_run / 1e12, "run_chunk": chunk_run,
                       "note": f"pct_peak counts the algorithmic flops at C=64 (the chunk the workload names); "
                               f"pct_peak_at_run_chunk at the C={chunk_run} the kernels run; bf16 dense peak"}
        # parity of the whole timed batch (o and S_T of every (sequence, head)) against the
        # fp64 oracle, whose run is also the CPU baseline below
        from oracle import default_threads, kda_oracle
        ncpu = default_threads()
        log(f"oracle on the whole prefill batch, {ncpu} threads")
        hx = {k_: x[k_].cpu() for k_ in ("q", "k", "v", "log_a", "beta", "S0")}
        t0 = time.perf_counter()
        ro, rS = kda_oracle(hx["q"], hx["k"], hx["v"], hx["log_a"], hx["beta"], S0=hx["S0"],
                            cu_seqlens=x["cu_seqlens"].cpu().numpy(), threads=ncpu)
        dt_oracle = time.perf_counter() - t0
        del hx
        perr = max_rel(o, ro)
        serr = max_rel(ST, rS)
        del ro, rS
        out["parity"] = {"prefill_o_max_rel_err": perr, "prefill_S_T_max_rel_err": serr, "tol": 2e-2,
                         "checked": f"every output and final state of the timed batch "
                                    f"({wp.n_seqs} x {wp.seqlen} tokens x {wp.heads} heads)"}
        log(f"prefill: {per*1e3:.3f} ms/step, {tokens/per/1e6:.2f} Mtok/s, {gbs:.0f} GB/s, "
            f"{tflops:.1f} TFLOP/s, parity o {perr:.2e} S_T {serr:.2e}")

        if not args.no_variants:
            # the same batch through the two other prefill entries: state snapshots every
            # 1024 tokens (written into a preallocated buffer), and the decay-first order
            vsteps = args.steps
            every = 1024
            rows = kda.snapshot_rows(None, every, total_tokens=tokens, num_seqs=wp.n_seqs)
            snaps = torch.empty((rows, wp.heads, wp.dk, wp.dv), dtype=torch.float32, device=dev)

            def snap_step():
                kda.chunk_fwd_snapshots(x["q"], x["k"], x["v"], x["log_a"], x["beta"], S0=x["S0"],
                                        cu_seqlens=x["cu_seqlens"], snapshot_every=every, snapshots=snaps,
                                        out=o, final_state=ST, method=method, workspace=ws,
                                        max_seqlen=wp.seqlen)
            # each leg warms up like the main one: the clocks drop during the host-side
            # parity check before it
            for _ in range(max(args.warmup, 3)):
                snap_step()
            torch.cuda.synchronize()
            ts = time_events(snap_step, vsteps, stream) / vsteps
            del snaps
            wsb1 = kda.chunk_workspace_size(x["q"], x["v"], num_seqs=wp.n_seqs, method=method,
                                            max_seqlen=wp.seqlen, order=kda.ORDER_DECAY_FIRST)
            ws1 = torch.empty(wsb1, dtype=torch.uint8, device=dev) if wsb1 else None

            def d1_step():
                kda.chunk_fwd(x["q"], x["k"], x["v"], x["log_a"], x["beta"], S0=x["S0"],
                              cu_seqlens=x["cu_seqlens"], out=o, final_state=ST, method=method, workspace=ws1,
                              max_seqlen=wp.seqlen, order=kda.ORDER_DECAY_FIRST)
            for _ in range(max(args.warmup, 3)):
                d1_step()
            torch.cuda.synchronize()
            t1 = time_events(d1_step, vsteps, stream) / vsteps
            sl = lambda t: t[:2048, 0:1].cpu()
            ro1, _ = kda_oracle(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["log_a"]), sl(x["beta"]),
                                S0=x["S0"][0:1, 0:1].cpu(), order=1)
            perr1 = float(np.abs(o[:2048, 0].double().cpu().numpy() - ro1[:, 0]).max() / np.abs(ro1).max())
            del ws1
            # input prologue: raw keys, beta logits and log-decay pre-activations of the same
            # shapes, transformed in the operator pass, against torch transforming them first
            from kda_recurrent_state_amd.workloads import generate_raw
            xr = generate_raw(wp, seed=3, device=dev)
            pro = dict(normalize_k=True, beta_logits=True, log_a_raw=True, log_a_min=wp.la_clip)

            def pro_step():
                kda.chunk_fwd(x["q"], xr["k"], x["v"], xr["log_a"], xr["beta"], S0=x["S0"],
                              cu_seqlens=x["cu_seqlens"], out=o, final_state=ST, method=method, workspace=ws,
                              max_seqlen=wp.seqlen, prologue=pro)

            def torch_step():
                kf = xr["k"].float()
                kn = (kf * torch.rsqrt((kf * kf).sum(-1, keepdim=True) + 1e-6)).to(wp.dtype)
                la = (-torch.nn.functional.softplus(xr["log_a"])).clamp_(min=wp.la_clip)
                kda.chunk_fwd(x["q"], kn, x["v"], la, torch.sigmoid(xr["beta"]), S0=x["S0"],
                              cu_seqlens=x["cu_seqlens"], out=o, final_state=ST, method=method, workspace=ws,
                              max_seqlen=wp.seqlen)
            for _ in range(max(args.warmup, 3)):
                pro_step()
            torch.cuda.synchronize()
            tp = time_events(pro_step, vsteps, stream) / vsteps
            for _ in range(max(args.warmup, 3)):
                torch_step()
            torch.cuda.synchronize()
            tt = time_events(torch_step, vsteps, stream) / vsteps
            del xr
            out["variants"] = {
                "snapshots": {"snapshot_every": every, "rows": rows, "ms_per_step": ts * 1e3,
                              "tokens_per_s": tokens / ts, "overhead_vs_plain": ts / per - 1.0,
                              "snapshot_bytes": rows * wp.heads * wp.dk * wp.dv * 4},
                "prologue": {"ms_per_step": tp * 1e3, "tokens_per_s": tokens / tp,
                             "overhead_vs_plain": tp / per - 1.0, "torch_prologue_then_plain_ms": tt * 1e3,
                             "note": "raw k, beta logits, log-decay pre-activations transformed in the operator "
                                     "pass vs by torch before the plain call"},
                "decay_first": {"ms_per_step": t1 * 1e3, "tokens_per_s": tokens / t1,
                                "algorithmic_GBps": B / t1 / 1e9, "frac_hbm": B / t1 / 1e9 / PEAK_HBM_GBS,
                                "workspace_MiB": round(wsb1 / 2**20, 1),
                                "parity_o_max_rel_err": perr1, "tol": 2e-2},
            }
            log(f"prefill with snapshots every {every}: {ts*1e3:.3f} ms; decay-first: {t1*1e3:.3f} ms, "
                f"parity {perr1:.2e}; prologue fused {tp*1e3:.3f} ms vs torch first {tt*1e3:.3f} ms")

        if not args.no_backward:
            # gradient of the same prefill for seeded upstream derivatives dO, dS_T
            g = torch.Generator(device=dev)
            g.manual_seed(5)
            dO = torch.randn(o.shape, generator=g, device=dev).to(wp.dtype)
            dST = torch.randn(ST.shape, generator=g, device=dev)
            wsbb = kda.chunk_bwd_workspace_size(x["q"], x["v"], num_seqs=wp.n_seqs, method=method,
                                                max_seqlen=wp.seqlen)
            wsB = torch.empty(wsbb, dtype=torch.uint8, device=dev)

            def bwd_step():
                return kda.chunk_bwd(x["q"], x["k"], x["v"], x["log_a"], x["beta"], dO, S0=x["S0"],
                                     cu_seqlens=x["cu_seqlens"], dS_T=dST, method=method, workspace=wsB,
                                     max_seqlen=wp.seqlen)
            for _ in range(max(args.warmup, 3)):
                bwd_step()
            torch.cuda.synchronize()
            log("backward timed")
            tb = time_events(bwd_step, args.steps, stream) / args.steps
            # the prefill rerun alone (states kept every 64 tokens), to split the call
            snaps64 = torch.empty((tokens // 64, wp.heads, wp.dk, wp.dv), dtype=torch.float32, device=dev)

            def rerun_step():
                kda.chunk_fwd_snapshots(x["q"], x["k"], x["v"], x["log_a"], x["beta"], S0=x["S0"],
                                        cu_seqlens=x["cu_seqlens"], snapshot_every=64, snapshots=snaps64,
                                        out=o, final_state=False, method=method, workspace=ws,
                                        max_seqlen=wp.seqlen)
            for _ in range(max(args.warmup, 3)):
                rerun_step()
            torch.cuda.synchronize()
            tr = time_events(rerun_step, args.steps, stream) / args.steps
            # the same gradient from the forward's kept states (kda_chunk_bwd_saved):
            # a training step whose forward kept them runs no rerun
            rerun_grads = {n_: t_.clone() for n_, t_ in bwd_step().items() if t_ is not None}
            del wsB
            wssb = kda.chunk_bwd_workspace_size(x["q"], x["v"], num_seqs=wp.n_seqs, method=method,
                                                max_seqlen=wp.seqlen, saved=True)
            wsS = torch.empty(wssb, dtype=torch.uint8, device=dev)

            def saved_step():
                return kda.chunk_bwd(x["q"], x["k"], x["v"], x["log_a"], x["beta"], dO, S0=x["S0"],
                                     cu_seqlens=x["cu_seqlens"], dS_T=dST, workspace=wsS, max_seqlen=wp.seqlen,
                                     states=snaps64)
            same = all(torch.equal(t_, rerun_grads[n_]) for n_, t_ in saved_step().items() if t_ is not None)
            del rerun_grads
            for _ in range(max(args.warmup, 3)):
                saved_step()
            torch.cuda.synchronize()
            tsv = time_events(saved_step, args.steps, stream) / args.steps
            # the decay-first order's gradient from that order's kept states
            kda.chunk_fwd_snapshots(x["q"], x["k"], x["v"], x["log_a"], x["beta"], S0=x["S0"],
                                    cu_seqlens=x["cu_seqlens"], snapshot_every=64, snapshots=snaps64, out=o,
                                    final_state=False, method=method, workspace=ws, max_seqlen=wp.seqlen,
                                    order=kda.ORDER_DECAY_FIRST)

            def saved_step_df():
                return kda.chunk_bwd(x["q"], x["k"], x["v"], x["log_a"], x["beta"], dO, S0=x["S0"],
                                     cu_seqlens=x["cu_seqlens"], dS_T=dST, workspace=wsS, max_seqlen=wp.seqlen,
                                     states=snaps64, order=kda.ORDER_DECAY_FIRST)
            for _ in range(max(args.warmup, 3)):
                saved_step_df()
            torch.cuda.synchronize()
            tdf = time_events(saved_step_df, args.steps, stream) / args.steps
            del snaps64, wsS
            Bb, Fb = backward_algorithmic(wp)
            out["backward"] = {
                "ms_per_step": tb * 1e3, "tokens_per_s": tokens / tb,
                "prefill_rerun_ms": tr * 1e3, "gradient_kernels_ms": (tb - tr) * 1e3,
                "algorithmic_bytes": Bb, "algorithmic_GBps": Bb / tb / 1e9, "frac_hbm": Bb / tb / 1e9 / PEAK_HBM_GBS,
                "algorithmic_tflop": Fb / 1e12, "achieved_tflops": Fb / tb / 1e12,
                "pct_bf16_peak": 100.0 * Fb / tb / 1e12 / PEAK_BF16_TFLOPS,
                "workspace_MiB": round(wsbb / 2**20, 1),
                "kernels": "prefill rerun (kda_prep2_kernel + kda_scan_kernel, states every 64 tokens) + "
                           "kda_bwd_ops_kernel + kda_bwd_walk_kernel (bf16; kda_bwd_scan_kernel for fp32) + kda_bwd_grad_kernel",
                "saved_states": {
                    "ms_per_step": tsv * 1e3, "tokens_per_s": tokens / tsv,
                    "algorithmic_GBps": Bb / tsv / 1e9, "frac_hbm": Bb / tsv / 1e9 / PEAK_HBM_GBS,
                    "pct_bf16_peak": 100.0 * Fb / tsv / 1e12 / PEAK_BF16_TFLOPS,
                    "workspace_MiB": round(wssb / 2**20, 1),
                    "bit_identical_to_rerun": same,
                    "forward_keeping_states_ms": tr * 1e3,
                    "training_step_ms": (tr + tsv) * 1e3,
                    "training_step_with_rerun_ms": (per + tb) * 1e3,
                    "note": "kda_chunk_bwd_saved with the states a forward call kept every 64 tokens; a training "
                            "step is that forward plus this call, against the plain forward plus kda_chunk_bwd",
                },
                "decay_first_saved_states": {"ms_per_step": tdf * 1e3, "tokens_per_s": tokens / tdf,
                                             "frac_hbm": Bb / tdf / 1e9 / PEAK_HBM_GBS},
            }
            log(f"backward: {tb*1e3:.3f} ms/step ({tokens/tb/1e6:.2f} Mtok/s), prefill rerun {tr*1e3:.3f} ms, "
                f"gradient kernels {(tb-tr)*1e3:.3f} ms; from saved states {tsv*1e3:.3f} ms (identical: {same})")

        if not args.no_cpu_baseline:
            dt = dt_oracle
            out["cpu_baseline"] = {
                "value": tokens / dt, "unit": "tokens/s", "cores": ncpu, "kind": "oracle",
                "sample": f"the whole timed prefill batch ({wp.n_seqs} x {wp.seqlen} tokens x "
                          f"{wp.heads} heads), fp64 token-by-token, one pass, {dt:.1f} s",
                "gpu_speedup": (tokens / per) / (tokens / dt),
                "host": host_info(ncpu),
            }
            log(f"cpu oracle: {tokens/dt:.0f} tokens/s ({dt:.1f} s)")
            if not args.no_backward:
                # the oracle's gradient on a bounded sample: the first 2048 tokens of both
                # sequences, all heads, and the GPU gradient of the same sample beside it
                from oracle import kda_oracle_bwd
                ns = 2048
                idx = torch.cat([torch.arange(n * wp.seqlen, n * wp.seqlen + ns) for n in range(wp.n_seqs)]).to(dev)
                cus = torch.arange(0, (wp.n_seqs + 1) * ns, ns, dtype=torch.int32, device=dev)
                sx = {k: x[k].index_select(0, idx).contiguous() for k in ("q", "k", "v", "log_a", "beta")}
                sdO = dO.index_select(0, idx).contiguous()
                hs = {k: v_.cpu() for k, v_ in sx.items()}
                t0 = time.perf_counter()
                ref = kda_oracle_bwd(hs["q"], hs["k"], hs["v"], hs["log_a"], hs["beta"], S0=x["S0"].cpu(),
                                     cu_seqlens=cus.cpu().numpy(), dO=sdO.cpu(), dST=dST.cpu(), threads=ncpu)
                dtb = time.perf_counter() - t0
                gg = kda.chunk_bwd(sx["q"], sx["k"], sx["v"], sx["log_a"], sx["beta"], sdO, S0=x["S0"],
                                   cu_seqlens=cus, dS_T=dST, max_seqlen=ns)
                torch.cuda.synchronize()
                berr = {n_: float(np.abs(gg[n_].double().cpu().numpy() - ref[n_]).max() / np.abs(ref[n_]).max())
                        for n_ in ref}
                out["backward"]["parity"] = {"max_rel_err": berr, "tol": 2e-2,
                                             "sample": f"first {ns} tokens of each sequence, all heads"}
                out["backward"]["cpu_baseline"] = {
                    "value": wp.n_seqs * ns / dtb, "unit": "tokens/s", "cores": ncpu, "kind": "oracle",
                    "sample": f"gradient of the first {ns} tokens of each sequence, all {wp.heads} heads, "
                              f"fp64 token-by-token with replay, {dtb:.1f} s",
                    "gpu_speedup": (tokens / tb) / (wp.n_seqs * ns / dtb)}
                log(f"cpu oracle gradient: {wp.n_seqs * ns / dtb:.0f} tokens/s ({dtb:.1f} s); "
                    f"gpu sample parity {max(berr.values()):.2e}")
                del dO, dST
        del x, o, ST
        torch.cuda.empty_cache()

    # ---------------- other prefill workloads: each its own timing, roofline and parity ----------------
    legs = [] if args.no_legs or args.only not in (None, "gdn", "varlen") else ["gdn", "varlen"]
    if args.only in ("gdn", "varlen"):
        legs = [args.only]
    for leg in legs:
        out.setdefault("legs", {})[leg] = prefill_leg(leg, args, kda, dev, stream)


    # ---------------- decode: 256 sequences x 32 heads, 100 chained steps ----------------
    if args.only in (None, "decode"):
        wd = WORKLOADS["kda_decode_b256_h32_d128"]
        steps = args.decode_steps
        from kda_recurrent_state_amd.workloads import scaled
        wds = scaled(wd, steps=steps)
        log("generating decode inputs")
        y = generate(wds, seed=4, device=dev)
        S = y["S"].clone()
        od = torch.empty((wd.n_seqs, wd.heads, wd.dv), dtype=wd.dtype, device=dev)
        ctr = [0]

        def dstep():
            i = ctr[0] % steps
            ctr[0] += 1
            kda.decode_step(y["q"][i], y["k"][i], y["v"][i], y["log_a"][i], y["beta"][i], S, out=od)

        for _ in range(min(args.warmup, steps)):
            dstep()
        torch.cuda.synchronize()
        ctr[0] = 0
        log("decode timed")
        t = time_events(dstep, steps, stream)
        per = t / steps
        Bd = decode_algorithmic(wd)
        gbs = Bd / per / 1e9
        state_gbs = 2 * 4 * wd.n_seqs * wd.heads * wd.dk * wd.dv / per / 1e9
        out.setdefault("value", None)
        out["decode"] = {
            "workload": wd.name, "value": gbs, "unit": "GB/s", "us_per_step": per * 1e6,
            "steps": steps, "state_only_GBps": state_gbs, "tokens_per_s": wd.n_seqs / per,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "traffic": stored_traffic("decode", Bd),
                         "kernel": "kda_decode_kernel", "algorithmic_bytes_per_launch": Bd,
                         "avg_launch_us": per * 1e6},
        }
        log(f"decode: {per*1e6:.1f} us/step, {gbs:.0f} GB/s ({100*gbs/PEAK_HBM_GBS:.1f}% of HBM peak)")
        if not args.no_variants:
            def d1step():
                i = ctr[0] % steps
                ctr[0] += 1
                kda.decode_step(y["q"][i], y["k"][i], y["v"][i], y["log_a"][i], y["beta"][i], S, out=od,
                                order=kda.ORDER_DECAY_FIRST)
            ctr[0] = 0
            for _ in range(min(max(args.warmup, 3), steps)):
                d1step()
            torch.cuda.synchronize()
            ctr[0] = 0
            t1 = time_events(d1step, steps, stream) / steps
            out["decode"]["decay_first"] = {"us_per_step": t1 * 1e6, "GBps": Bd / t1 / 1e9,
                                            "frac_hbm": Bd / t1 / 1e9 / PEAK_HBM_GBS}
            log(f"decode decay-first: {t1*1e6:.1f} us/step")

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
