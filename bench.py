"""Benchmark of the fused cascaded-reduction hot path on one MI355X.

One step = one pass of every kernel of the path over one batch of synthetic,
seeded input already resident in HBM:
  prefill attention, bf16, B=4 H=32 L=2048 d=128, non-causal and causal;
  split-KV decode, bf16 KV cache, B=8 Hq=32 Hkv=8 Lk=32768 d=128, S segments,
    partial states + merge;
  MoE routing, 16384 x 256 fp32 logits, softmax -> top-8 (renormalised);
  FP8 per-token quantise + GEMM, M=N=4096, K=7168.
After the timed steps, further rows are timed on their own: the one-pass
running-scale FP8 GEMM, split-KV decode over a shared latent cache (B=32
sequences, 16 heads, 8192 latent rows of 576 bf16 values), and safe softmax, variance and moment of inertia over
rows of 1K..8K fp32 values at each fusion level of the reduction tree
(unfused, thread, wave, block).
Routing logits rotate over 20 buffers, the FP8 A operand over 5 and the
multi-latent cache over 2, so those inputs (which would otherwise fit, or
partly fit, the 256 MB last-level cache) come from HBM.

Prints ONE JSON line. ``value`` is the mean of two fractions of MI355X peak:
prefill (non-causal) TFLOP/s over the 2.5 PFLOP/s dense bf16 MFMA peak, and
split-KV decode GB/s over the 8 TB/s HBM peak (best of the timed segment
counts). Kernel times come from HIP events on the stream the kernels run on.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0

PREFILL = dict(B=4, H=32, L=2048, d=128)
DECODE = dict(B=8, Hq=32, Hkv=8, Lk=32768, d=128)
ROUTING = dict(T=16384, E=256, k=8)
FP8 = dict(M=4096, N=4096, K=7168)
MLA = dict(B=32, H=16, Lk=8192, dqk=576, dv=512)
MLA_SEGMENTS = (8, 16, 32)
SOFTMAX_VALUES = 1 << 26
ROW_ROTATE = 3  # input copies per row length, so no launch re-reads the last one from cache


def rotated(t, n=ROW_ROTATE):
    """n device copies of t with rows rolled by 0, 7, 14, ...: the same rows at
    other addresses (row results are unchanged, only their order)."""
    return [t] + [t.roll(7 * r, dims=0).contiguous() for r in range(1, n)]
SOFTMAX_E = (1024, 2048, 4096, 8192)
DECODE_SEGMENTS = (1, 4, 8, 16, 64)
ROUTING_ROTATE = 20
FP8_ROTATE = 5


def prefill_flops(causal):
    B, H, L, d = PREFILL["B"], PREFILL["H"], PREFILL["L"], PREFILL["d"]
    pairs = L * (L + 1) // 2 if causal else L * L
    return 4.0 * B * H * pairs * d


def decode_bytes():
    B, Hq, Hkv, Lk, d = (DECODE[x] for x in ("B", "Hq", "Hkv", "Lk", "d"))
    return 2 * B * Hkv * Lk * d * 2 + 2 * B * Hq * d * 2   # K + V read, q read + O written


def routing_bytes():
    T, E, k = ROUTING["T"], ROUTING["E"], ROUTING["k"]
    return T * E * 4 + T * k * 8


def quant_bytes():
    M, K = FP8["M"], FP8["K"]
    return M * K * 2 + M * K + M * 4


def gemm_flops():
    return 2.0 * FP8["M"] * FP8["N"] * FP8["K"]


def read_traffic():
    """Measured HBM traffic per launch from profiles/traffic.txt, kept only while
    the kernel source it was measured on, and the device header every kernel
    includes, are unchanged (matching hash of the two files' bytes)."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "traffic.txt")
    out = {}
    if not os.path.exists(path):
        return out
    for line in open(path):
        parts = line.split()
        if len(parts) != 4 or line.startswith("#"):
            continue
        kernel, src, digest, nbytes = parts
        src_path = os.path.join(ROOT, src)
        if not os.path.exists(src_path):
            continue
        header = os.path.join(ROOT, "online_softmax_attention_cascaded_amd", "csrc", "rf_device.hpp")
        now = hashlib.sha256(open(src_path, "rb").read() + open(header, "rb").read()).hexdigest()[:16]
        if now == digest:
            out[kernel] = float(nbytes)
    return out


def _cpu_worker(args):
    """One pool worker: the oracle on its own (batch, head) prefill slice, then on
    its own query rows of the S=16 decode, each for half the budget, with BLAS
    held to one thread."""
    wid, budget_s = args
    import threadpoolctl

    import oracle
    from online_softmax_attention_cascaded_amd import inputs

    with threadpoolctl.threadpool_limits(limits=1):
        P = PREFILL
        q, k, v = inputs.attention_inputs(1 + wid, 1, 1, 1, P["L"], P["L"], P["d"])
        scale = 1 / math.sqrt(P["d"])
        oracle.attention(q, k, v, scale)            # untimed: first-touch of the work arrays
        n_heads, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < budget_s / 2 or n_heads == 0:
            oracle.attention(q, k, v, scale)
            n_heads += 1
        t_pre = time.perf_counter() - t0
        Dc = DECODE
        qd, kd, vd = inputs.decode_inputs(2 + wid, 1, 4, 1, Dc["Lk"], Dc["d"])
        oracle.decode_partials(qd, kd, vd, scale, 16)
        n_rows, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < budget_s / 2 or n_rows == 0:
            m, l, acc = oracle.decode_partials(qd, kd, vd, scale, 16)
            oracle.merge_states(m, l, acc)
            n_rows += qd.shape[1]
        t_dec = time.perf_counter() - t0
    return n_heads, t_pre, n_rows, t_dec


def _host_description():
    import platform

    import numpy as np
    import threadpoolctl

    model = platform.processor() or "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpoolctl.threadpool_info()
            if i.get("user_api") == "blas"]
    return model, np.__version__, ", ".join(blas) or "none found"


def cpu_baseline(budget_s=12.0):
    """The oracle as it stands, timed on this host on a bounded sample of the same
    workloads: a pool of one process per usable core (at most 16), BLAS held to
    one thread in each, every worker running whole (batch, head) slices of the
    non-causal prefill and then whole query rows of the S=16 decode for half the
    budget each (after one untimed call of each). Throughputs are the sums over the workers. Called before this
    process touches the GPU, so the forked workers inherit no device state."""
    import multiprocessing as mp

    workers = max(1, min(os.cpu_count() or 1, len(os.sched_getaffinity(0)), 16))
    with mp.get_context("fork").Pool(workers) as pool:
        res = pool.map(_cpu_worker, [(w, budget_s) for w in range(workers)])
    P, Dc = PREFILL, DECODE
    n_heads = sum(r[0] for r in res)
    n_rows = sum(r[2] for r in res)
    pre_tflops = sum(r[0] * 4.0 * P["L"] * P["L"] * P["d"] / r[1] for r in res) / 1e12
    # Bytes of the full workload per query row: its share of K/V (one GQA group of 4
    # rows reads one K/V head) plus q and O.
    bytes_per_row = (2 * Dc["Lk"] * Dc["d"] * 2) / (Dc["Hq"] // Dc["Hkv"]) + 2 * Dc["d"] * 2
    dec_gbs = sum(r[2] * bytes_per_row / r[3] for r in res) / 1e9
    model, np_version, blas = _host_description()
    value = 0.5 * (pre_tflops / PEAK_BF16_TFLOPS + dec_gbs / PEAK_HBM_GBS) * 100
    return {
        "value": value,
        "unit": "% of MI355X peak (mean of prefill/bf16-MFMA and decode/HBM fractions)",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle in {workers} processes, one BLAS thread each, about "
                   f"{budget_s:.0f} s: {n_heads} (batch, head) slices of the non-causal prefill "
                   f"(L=2048, d=128) and {n_rows} query rows of the S=16 decode (Lk=32768)"),
        "host": {"cpu": model, "numpy": np_version, "blas": blas},
        "prefill_tflops": pre_tflops,
        "decode_gbs": dec_gbs,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps; the GPU clocks need tens of milliseconds of work to settle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one elementwise copy of 512 MiB first (reference kernel of known "
                         "traffic for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU variant "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import online_softmax_attention_cascaded_amd as rf
    from online_softmax_attention_cascaded_amd import inputs
    from online_softmax_attention_cascaded_amd.build import LIB_PATH

    if not os.path.exists(LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()

    def progress(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        progress("timing the oracle on the host (before the GPU is touched)")
        cpu = cpu_baseline()
        progress(f"oracle on {cpu['cores']} host cores: {cpu['value']:.5f} % of peak")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
        progress("copy calibration kernel done (reads 512 MiB, writes 512 MiB)")

    # ---------------- inputs (seeded, generated on the host, copied to HBM once)
    progress("generating inputs")
    P, Dc, R, F = PREFILL, DECODE, ROUTING, FP8
    q, k, v = (t.to(dev) for t in inputs.attention_inputs(1, P["B"], P["H"], P["H"], P["L"], P["L"], P["d"]))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    scale = 1 / math.sqrt(P["d"])

    qd, kd, vd = (t.to(dev) for t in inputs.decode_inputs(2, Dc["B"], Dc["Hq"], Dc["Hkv"], Dc["Lk"], Dc["d"]))
    dec_bufs = {}
    for S in DECODE_SEGMENTS:
        dec_bufs[S] = (torch.empty((Dc["B"], Dc["Hq"], S), device=dev),
                       torch.empty((Dc["B"], Dc["Hq"], S), device=dev),
                       torch.empty((Dc["B"], Dc["Hq"], S, Dc["d"]), device=dev))
    od = torch.empty((Dc["B"], Dc["Hq"], Dc["d"]), dtype=torch.bfloat16, device=dev)
    lsed = torch.empty((Dc["B"], Dc["Hq"]), device=dev)

    logits0 = inputs.routing_inputs(3, R["T"], R["E"]).to(dev)
    logits = [logits0] + [logits0.clone() for _ in range(ROUTING_ROTATE - 1)]
    rw = torch.empty((R["T"], R["k"]), device=dev)
    ri = torch.empty((R["T"], R["k"]), dtype=torch.int32, device=dev)

    a0, bsrc = inputs.quant_inputs(4, F["M"], F["N"], F["K"])
    a_bufs = [a0.to(dev)] + [a0.to(dev) for _ in range(FP8_ROTATE - 1)]
    bq, bs = rf.absmax_quant_fp8(bsrc.to(dev))
    aq = torch.empty((F["M"], F["K"]), dtype=torch.uint8, device=dev)
    sa = torch.empty(F["M"], device=dev)
    c = torch.empty((F["M"], F["N"]), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    # ---------------- one step of the path, each kernel bracketed by events
    names = ["prefill", "prefill_causal"] + [f"decode_s{S}" for S in DECODE_SEGMENTS] + ["routing", "fp8"]
    times = {n: 0.0 for n in names}

    def step(i, record):
        ev = []

        def mark():
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                ev.append(e)

        mark()
        rf.rf_attn_fwd(q, k, v, o, lse, scale, False)
        mark()
        rf.rf_attn_fwd(q, k, v, o, lse, scale, True)
        mark()
        for S in DECODE_SEGMENTS:
            pm, pl, pa = dec_bufs[S]
            rf.rf_attn_decode_split(qd, kd, vd, pm, pl, pa, scale)
            rf.rf_merge_states(pm, pl, pa, od, lsed)
            mark()
        rf.rf_softmax_topk(logits[i % ROUTING_ROTATE], R["k"], True, rw, ri)
        mark()
        rf.rf_absmax_quant_gemm_fp8(a_bufs[i % FP8_ROTATE], bq, bs, aq, sa, c)
        mark()
        return ev

    progress("warmup")
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    events = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        events.append(step(i, True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    samples = {n: [] for n in names}
    for ev in events:
        for n, a, b in zip(names, ev[:-1], ev[1:]):
            dt = a.elapsed_time(b) / 1e3  # seconds
            times[n] += dt
            samples[n].append(dt)
    per = {n: times[n] / args.steps for n in names}  # seconds per launch group

    # Routing on its own: inside the step a 7 us launch sits between two event
    # records, whose overhead is then part of its time. Here a spin kernel holds
    # the queue while 40 launches over the rotating logits are submitted, so
    # they run back to back between one event pair (kernel time plus the gap
    # between consecutive dispatches).
    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(2_000_000)
    r0.record()
    for i in range(2 * ROUTING_ROTATE):
        rf.rf_softmax_topk(logits[i % ROUTING_ROTATE], R["k"], True, rw, ri)
    r1.record()
    torch.cuda.synchronize()
    t_rout_b2b = r0.elapsed_time(r1) / 1e3 / (2 * ROUTING_ROTATE)

    pre_tflops = prefill_flops(False) / per["prefill"] / 1e12
    pre_c_tflops = prefill_flops(True) / per["prefill_causal"] / 1e12
    dec = {S: decode_bytes() / per[f"decode_s{S}"] / 1e9 for S in DECODE_SEGMENTS}
    best_S = max(dec, key=dec.get)
    dec_gbs = dec[best_S]
    rout_gbs = routing_bytes() / t_rout_b2b / 1e9
    pre_frac = pre_tflops / PEAK_BF16_TFLOPS
    dec_frac = dec_gbs / PEAK_HBM_GBS
    value = 0.5 * (pre_frac + dec_frac) * 100

    traffic = read_traffic()
    step_ms = wall / args.steps * 1e3
    result = {
        "metric": "prefill attn TFLOP/s + split-KV decode GB/s, as % of MI355X peak",
        "value": round(value, 3),
        "unit": "% of peak (mean of prefill bf16-MFMA fraction and decode HBM fraction)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1); routing spikes and FP8 outliers as configured)",
        "config": {
            "workload": "prefill attention B4 H32 L2048 d128 bf16 (non-causal and causal) + "
                        "split-KV decode B8 Hq32 Hkv8 Lk32768 d128 bf16 + routing 16384x256 top-8 + "
                        "FP8 quant+GEMM 4096x4096x7168",
            "prefill": PREFILL, "decode": dict(DECODE, segments=list(DECODE_SEGMENTS)),
            "routing": ROUTING, "fp8": FP8, "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd_bf16 (non-causal prefill)",
            "achieved": round(pre_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pre_frac, 4),
            "traffic": traffic.get("attn_fwd_bf16"),
        },
        "rooflines": {
            "prefill_causal": {"bound": "mfma", "achieved": round(pre_c_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                               "unit": "TFLOP/s", "frac": round(pre_c_tflops / PEAK_BF16_TFLOPS, 4)},
            "decode": {"bound": "hbm", "segments": best_S, "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS,
                       "unit": "GB/s", "frac": round(dec_frac, 4),
                       "by_segments": {str(S): round(x, 1) for S, x in dec.items()},
                       "traffic": traffic.get("decode_split")},
            "routing": {"bound": "hbm", "achieved": round(rout_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(rout_gbs / PEAK_HBM_GBS, 4), "traffic": traffic.get("softmax_topk"),
                        "us_per_launch": round(t_rout_b2b * 1e6, 2),
                        "note": "40 launches back to back over 20 rotating logit buffers; the in-step "
                                "time (us_per_launch.routing) adds the event records around it"},
            "fp8_quant_gemm": {"bound": "mfma", "achieved": round(gemm_flops() / per["fp8"] / 1e12, 2),
                               "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(gemm_flops() / per["fp8"] / 1e12 / PEAK_FP8_TFLOPS, 4),
                               "note": "quantiser + GEMM time, GEMM flops only",
                               "traffic": (traffic["absmax_quant"] + traffic["gemm_fp8"]
                                           if "absmax_quant" in traffic and "gemm_fp8" in traffic else None)},
        },
        "us_per_launch": {n: round(per[n] * 1e6, 2) for n in names},
        "us_spread": {n: {"min": round(min(v) * 1e6, 2), "median": round(sorted(v)[len(v) // 2] * 1e6, 2),
                          "max": round(max(v) * 1e6, 2)} for n, v in samples.items()},
        "tokens_per_s": {
            "prefill": PREFILL["B"] * PREFILL["L"] / per["prefill"],
            "decode": DECODE["B"] / per[f"decode_s{best_S}"],
            "routing": ROUTING["T"] / per["routing"],
            "fp8": FP8["M"] / per["fp8"],
        },
    }
    progress(f"timed {args.steps} steps in {wall:.2f} s")

    # The one-pass running-scale FP8 GEMM (quantises A inside the K loop) is
    # an alternative to the step's quantise + GEMM, timed on its own.
    sr = torch.empty(F["M"], device=dev)
    for i in range(10):
        rf.rf_absmax_quant_gemm_fp8_running(a_bufs[i % FP8_ROTATE], bq, bs, sr, c)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        rf.rf_absmax_quant_gemm_fp8_running(a_bufs[i % FP8_ROTATE], bq, bs, sr, c)
    e1.record()
    torch.cuda.synchronize()
    t_run = e0.elapsed_time(e1) / 1e3 / args.steps
    result["us_per_launch"]["fp8_running"] = round(t_run * 1e6, 2)
    result["rooflines"]["fp8_running_scale_one_pass"] = {
        "bound": "mfma", "achieved": round(gemm_flops() / t_run / 1e12, 2), "peak": PEAK_FP8_TFLOPS,
        "unit": "TFLOP/s", "frac": round(gemm_flops() / t_run / 1e12 / PEAK_FP8_TFLOPS, 4),
        "note": "single kernel: running per-row scale, A quantised inside the K loop"}
    # Split-KV decode over a shared latent cache (multi-latent attention),
    # partial states + merge, at each segment count, as two launches and as
    # one (the last workgroup of each group merges). Algorithmic bytes: the
    # latent rows once (B * Lk * 576 * 2) plus q and O.
    Mq, Mkv = (t.to(dev) for t in inputs.mla_inputs(7, MLA["B"], MLA["H"], MLA["Lk"]))
    # two copies of the 302 MB latent cache, used in turn, so no launch finds
    # the previous one's rows in the 256 MB last-level cache
    Mkvs = [Mkv, Mkv.clone()]
    mla_bytes = (MLA["B"] * MLA["Lk"] * MLA["dqk"] * 2 + MLA["B"] * MLA["H"] * MLA["dqk"] * 2
                 + MLA["B"] * MLA["H"] * MLA["dv"] * 2)
    mo = torch.empty((MLA["B"], MLA["H"], MLA["dv"]), dtype=torch.bfloat16, device=dev)
    mlse = torch.empty((MLA["B"], MLA["H"]), device=dev)
    counters = torch.zeros(MLA["B"] * MLA["H"] // 16, dtype=torch.int32, device=dev)
    mla_t, mla_one = {}, {}
    for S in MLA_SEGMENTS:
        pm = torch.empty((MLA["B"], MLA["H"], S), device=dev)
        pl = torch.empty_like(pm)
        pa = torch.empty((MLA["B"], MLA["H"], S, MLA["dv"]), device=dev)

        def mla_two_launches(kv):
            rf.rf_mla_decode_split(Mq, kv, pm, pl, pa, 1 / math.sqrt(MLA["dqk"]))
            rf.rf_merge_states(pm, pl, pa, mo, mlse)

        def mla_fused(kv):
            rf.rf_mla_decode(Mq, kv, pm, pl, pa, counters, mo, mlse, 1 / math.sqrt(MLA["dqk"]))
        for fn, store in ((mla_two_launches, mla_t), (mla_fused, mla_one)):
            for i in range(10):
                fn(Mkvs[i % 2])
            e0.record()
            for i in range(args.steps):
                fn(Mkvs[i % 2])
            e1.record()
            torch.cuda.synchronize()
            store[S] = e0.elapsed_time(e1) / 1e3 / args.steps
    best_mla = min(mla_t, key=mla_t.get)
    result["us_per_launch"].update({f"mla_decode_s{S}": round(t * 1e6, 2) for S, t in mla_t.items()})
    result["us_per_launch"].update({f"mla_decode_one_launch_s{S}": round(t * 1e6, 2)
                                    for S, t in mla_one.items()})
    result["rooflines"]["mla_decode"] = {
        "bound": "hbm", "segments": best_mla, "achieved": round(mla_bytes / mla_t[best_mla] / 1e9, 1),
        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(mla_bytes / mla_t[best_mla] / 1e9 / PEAK_HBM_GBS, 4),
        "by_segments": {str(S): round(mla_bytes / t / 1e9, 1) for S, t in mla_t.items()},
        "one_launch_by_segments": {str(S): round(mla_bytes / t / 1e9, 1) for S, t in mla_one.items()},
        "note": ("latent rows read once (launches alternate between two copies of the cache, so they "
                 "come from HBM, not the last-level cache); split + merge as two launches. One launch (rf_mla_decode, "
                 "last workgroup merges) is slower here: each workgroup's agent-scope release is an "
                 "L2 write-back, and one workgroup folds all S states of its group"),
        "traffic": traffic.get("mla_decode_split"),
        "traffic_one_launch": traffic.get("mla_decode_one_launch"),
        "traffic_note": ("split-only kernel, mean over the timed segment counts (the merge reads the partials "
                         "again); traffic_one_launch: the single-launch form, whose merging workgroups also "
                         "read their group's partial states")}
    del Mq, Mkv
    progress("multi-latent decode timed")

    # The other widths and dtypes the boundary takes, on the decode and prefill
    # shapes: split-KV decode (split + merge) with fp32 K/V at head size 128
    # and 64 and with bf16 K/V at head size 64, and bf16 prefill at head size 64.
    def timed(fn):
        for _ in range(5):
            fn()
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / args.steps

    variants = {}
    for name, d_, dt_ in (("decode_f32_d128", 128, torch.float32), ("decode_f32_d64", 64, torch.float32),
                          ("decode_bf16_d64", 64, torch.bfloat16)):
        vq, vk, vv = (t.to(dev) for t in inputs.decode_inputs(2, Dc["B"], Dc["Hq"], Dc["Hkv"], Dc["Lk"], d_,
                                                                dtype=dt_))
        es = 4 if dt_ == torch.float32 else 2
        nbytes = 2 * Dc["B"] * Dc["Hkv"] * Dc["Lk"] * d_ * es + 2 * Dc["B"] * Dc["Hq"] * d_ * es
        vo = torch.empty((Dc["B"], Dc["Hq"], d_), dtype=dt_, device=dev)
        vl = torch.empty((Dc["B"], Dc["Hq"]), device=dev)
        by = {}
        for S in (4, 8, 16):
            pm = torch.empty((Dc["B"], Dc["Hq"], S), device=dev)
            pl = torch.empty_like(pm)
            pa = torch.empty((Dc["B"], Dc["Hq"], S, d_), device=dev)

            def dec():
                rf.rf_attn_decode_split(vq, vk, vv, pm, pl, pa, 1 / math.sqrt(d_))
                rf.rf_merge_states(pm, pl, pa, vo, vl)
            by[str(S)] = round(nbytes / timed(dec) / 1e9, 1)
        best = max(by, key=by.get)
        variants[name] = {"bound": "hbm", "segments": int(best), "achieved": by[best], "peak": PEAK_HBM_GBS,
                          "unit": "GB/s", "frac": round(by[best] / PEAK_HBM_GBS, 4), "by_segments": by}
        del vq, vk, vv
    pq, pk, pv = (t.to(dev) for t in inputs.attention_inputs(1, P["B"], P["H"], P["H"], P["L"], P["L"], 64))
    po = torch.empty_like(pq)
    pls = torch.empty(pq.shape[:3], dtype=torch.float32, device=dev)
    for causal in (False, True):
        t = timed(lambda: rf.rf_attn_fwd(pq, pk, pv, po, pls, 0.125, causal))
        pairs = P["L"] * (P["L"] + 1) // 2 if causal else P["L"] * P["L"]
        fl = 4.0 * P["B"] * P["H"] * pairs * 64
        variants["prefill_d64" + ("_causal" if causal else "")] = {
            "bound": "mfma", "achieved": round(fl / t / 1e12, 1), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(fl / t / 1e12 / PEAK_BF16_TFLOPS, 4), "us_per_launch": round(t * 1e6, 2)}
    del pq, pk, pv, po
    result["other_widths"] = variants
    progress("other head sizes and fp32 decode timed")

    # Safe softmax alone at each fusion level of the reduction tree, rows of
    # 1K .. 8K fp32 values, 2^26 values per launch (launches rotate over three
    # copies of the input, 268 MB each). The rate is counted with the
    # fused form's algorithmic bytes (x read once, y written once: 8 B/value)
    # for every level, so the rates compare like for like; the unfused cascade
    # moves 16 B/value (three reads of x, one write).
    levels = {"unfused": rf.RF_FUSE_NONE, "thread": rf.RF_FUSE_THREAD, "wave": rf.RF_FUSE_WAVE,
              "block": rf.RF_FUSE_BLOCK}
    sm_rates = {}
    for E in SOFTMAX_E:
        T = SOFTMAX_VALUES // E
        xs = rotated(inputs.softmax_inputs(6, T, E).to(dev))
        ys = torch.empty_like(xs[0])
        work = torch.empty(2 * T, device=dev)
        for lname, lv in levels.items():
            for i in range(10):
                rf.rf_softmax(xs[i % ROW_ROTATE], lv, work, ys)
            e0.record()
            for i in range(args.steps):
                rf.rf_softmax(xs[i % ROW_ROTATE], lv, work, ys)
            e1.record()
            torch.cuda.synchronize()
            t_sm = e0.elapsed_time(e1) / 1e3 / args.steps
            sm_rates[(E, lname)] = (t_sm, 8.0 * T * E / t_sm / 1e9)
        del xs, ys, work
    result["softmax_fusion_levels"] = {
        "values_per_launch": SOFTMAX_VALUES,
        "unit": "GB/s at 8 B/value (x read once, y written once)",
        "us_per_launch": {f"E{E}": {ln: round(sm_rates[(E, ln)][0] * 1e6, 2) for ln in levels}
                          for E in SOFTMAX_E},
        "GBs": {f"E{E}": {ln: round(sm_rates[(E, ln)][1], 1) for ln in levels} for E in SOFTMAX_E},
    }
    best_sm = max(sm_rates[(E, "block")][1] for E in SOFTMAX_E)
    result["rooflines"]["softmax_block_level"] = {
        "bound": "hbm", "achieved": round(best_sm, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "frac": round(best_sm / PEAK_HBM_GBS, 4), "note": "best row length of the block-level form"}
    progress("softmax fusion levels timed")

    # Variance and moment of inertia (centre, then centred second moment) at
    # each fusion level, rows of 1K .. 8K values, 2^26 values per launch
    # (rotating over three copies of the input).
    # Algorithmic bytes: 4 B/value (x) for the variance, 8 B/value (x and the
    # masses) for the moment of inertia; the unfused cascade reads them twice.
    mom = {}
    for E in SOFTMAX_E:
        T = SOFTMAX_VALUES // E
        xm0, wm0 = (t.to(dev) for t in inputs.moment_inputs(8, T, E))
        sets = list(zip(rotated(xm0), rotated(wm0)))
        del xm0, wm0
        oc = torch.empty(T, device=dev)
        oi = torch.empty(T, device=dev)
        for kind, per_value in (("variance", 4), ("inertia", 8)):
            for lname, lv in levels.items():
                def call(i):
                    xm, wm = sets[i % ROW_ROTATE]
                    if kind == "variance":
                        rf.rf_row_variance(xm, lv, oc, oi)
                    else:
                        rf.rf_row_inertia(xm, wm, lv, oc, oi)
                for i in range(10):
                    call(i)
                e0.record()
                for i in range(args.steps):
                    call(i)
                e1.record()
                torch.cuda.synchronize()
                t_m = e0.elapsed_time(e1) / 1e3 / args.steps
                mom[(kind, E, lname)] = (t_m, per_value * T * E / t_m / 1e9)
        del sets, oc, oi
    result["moment_fusion_levels"] = {
        kind: {
            "unit": f"GB/s at {per_value} B/value",
            "us_per_launch": {f"E{E}": {ln: round(mom[(kind, E, ln)][0] * 1e6, 2) for ln in levels}
                              for E in SOFTMAX_E},
            "GBs": {f"E{E}": {ln: round(mom[(kind, E, ln)][1], 1) for ln in levels} for E in SOFTMAX_E},
        }
        for kind, per_value in (("variance", 4), ("inertia", 8))
    }
    for kind in ("variance", "inertia"):
        best = max(mom[(kind, E, ln)][1] for E in SOFTMAX_E for ln in levels if ln != "unfused")
        result["rooflines"][f"{kind}_fused_best"] = {
            "bound": "hbm", "achieved": round(best, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(best / PEAK_HBM_GBS, 4)}
    progress("variance and moment-of-inertia fusion levels timed")

    # Context for the bf16 MFMA roofline: the rate the vendor's bf16 GEMM
    # (hipBLASLt through torch.matmul, 8192^3) sustains on this GPU with N(0,1)
    # operands. With such data the matrix cores run below their peak clock,
    # so this is the practical ceiling of a bf16 contraction here; it is shown
    # beside the published peak, which stays the roofline's `peak`.
    gen = torch.Generator(device=dev).manual_seed(11)
    ga = torch.randn(8192, 8192, device=dev, generator=gen).to(torch.bfloat16)
    gb = torch.randn(8192, 8192, device=dev, generator=gen).to(torch.bfloat16)
    for _ in range(5):
        gc = ga @ gb
    e0.record()
    for _ in range(20):
        gc = ga @ gb
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2.0 * 8192 ** 3 / (e0.elapsed_time(e1) / 1e3 / 20) / 1e12
    del ga, gb, gc
    result["roofline"]["context"] = {
        "kind": "vendor bf16 GEMM 8192x8192x8192 (hipBLASLt via torch.matmul), N(0,1) operands",
        "achieved": round(gemm_tflops, 1), "unit": "TFLOP/s",
        "prefill_frac_of_it": round(pre_tflops / gemm_tflops, 4)}
    progress("vendor bf16 GEMM timed for context")

    # The vendor's attention on the same prefill inputs: torch's
    # scaled_dot_product_attention restricted to its flash backend (on ROCm,
    # AOTriton kernels), which raises instead of falling back to the unfused
    # math path. Reported beside the roofline; null if the backend is missing.
    from torch.nn.attention import SDPBackend, sdpa_kernel

    vendor_attn = {}
    for causal in (False, True):
        try:
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                for _ in range(3):
                    torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
                e0.record()
                for _ in range(10):
                    torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
                e1.record()
                torch.cuda.synchronize()
            vendor_attn[causal] = prefill_flops(causal) / (e0.elapsed_time(e1) / 1e3 / 10) / 1e12
        except RuntimeError as ex:
            progress(f"torch flash attention unavailable: {ex}")
            vendor_attn[causal] = None
    va = vendor_attn[False]
    result["roofline"]["vendor_attention"] = {
        "kind": "torch scaled_dot_product_attention, flash backend only, same inputs",
        "achieved": None if va is None else round(va, 1), "unit": "TFLOP/s",
        "speedup": None if va is None else round(pre_tflops / va, 3)}
    vc = vendor_attn[True]
    result["rooflines"]["prefill_causal"]["vendor_attention"] = {
        "achieved": None if vc is None else round(vc, 1), "unit": "TFLOP/s",
        "speedup": None if vc is None else round(pre_c_tflops / vc, 3)}
    progress("vendor attention timed for context")

    # Measured ceilings beside the published peaks: the MFMA loops of
    # rf_peak_mfma on operand data like the workloads' (512 workgroups, two
    # waves per SIMD), with the shader clock they ran at; for HBM, a 2 GiB read
    # stream (rf_peak_read) and a 1 GiB device copy (read + write bytes).
    khz = rf.rf_wall_clock_khz()
    blocks = 512
    measured = {}
    for kind, name, iters, per_mfma in ((rf.RF_PEAK_BF16, "bf16", 8192, 32768),
                                        (rf.RF_PEAK_FP8, "fp8", 4096, 131072)):
        if kind == rf.RF_PEAK_BF16:
            vals = torch.randn((blocks * 256, 128), device=dev, generator=gen).to(torch.bfloat16)
        else:
            vals = (torch.randn((blocks * 256, 256), device=dev, generator=gen) * 100).clamp(
                -448, 448).to(torch.float8_e4m3fn)
        src = vals.view(torch.uint8).reshape(blocks * 256, 256)
        pout = torch.empty(blocks * 4, device=dev)
        clk = torch.zeros((blocks, 2), dtype=torch.int64, device=dev)
        for _ in range(2):
            rf.rf_peak_mfma(kind, src, iters, pout, clk)
        e0.record()
        for _ in range(5):
            rf.rf_peak_mfma(kind, src, iters, pout, clk)
        e1.record()
        torch.cuda.synchronize()
        t_pk = e0.elapsed_time(e1) / 1e3 / 5
        ck = clk.cpu().double()
        ghz = float((ck[:, 0] / ck[:, 1]).median()) * khz / 1e6
        measured[name] = (blocks * 4 * iters * 8 * per_mfma / t_pk / 1e12, ghz)
        del vals, src, pout, clk
    cp_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cp_dst = torch.empty_like(cp_src)
    for _ in range(3):
        cp_dst.copy_(cp_src)
    e0.record()
    for _ in range(10):
        cp_dst.copy_(cp_src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * (1 << 30) / (e0.elapsed_time(e1) / 1e3 / 10) / 1e9
    del cp_dst
    rd_src = torch.cat([cp_src, cp_src])   # 2 GiB, well past the 256 MB last-level cache
    del cp_src
    # 2048 workgroups, each streaming its own contiguous 1 MiB
    rd_out = torch.empty(2048, dtype=torch.int32, device=dev)
    for _ in range(3):
        rf.rf_peak_read(rd_src, 2048, rd_out)
    e0.record()
    for _ in range(10):
        rf.rf_peak_read(rd_src, 2048, rd_out)
    e1.record()
    torch.cuda.synchronize()
    read_gbs = 2.0 * (1 << 30) / (e0.elapsed_time(e1) / 1e3 / 10) / 1e9
    del rd_src, rd_out
    bf_tf, bf_ghz = measured["bf16"]
    f8_tf, f8_ghz = measured["fp8"]
    mfma_kind = "MFMA loop (rf_peak_mfma) on N(0,1)-like operands, 2 waves per SIMD"
    result["roofline"]["measured_peak"] = {
        "kind": "bf16 " + mfma_kind, "achieved": round(bf_tf, 1), "unit": "TFLOP/s",
        "clock_ghz": round(bf_ghz, 3), "frac": round(pre_tflops / bf_tf, 4)}
    result["rooflines"]["prefill_causal"]["measured_peak_frac"] = round(pre_c_tflops / bf_tf, 4)
    fp8_tf = gemm_flops() / per["fp8"] / 1e12
    result["rooflines"]["fp8_quant_gemm"]["measured_peak"] = {
        "kind": "fp8 e4m3 " + mfma_kind, "achieved": round(f8_tf, 1), "unit": "TFLOP/s",
        "clock_ghz": round(f8_ghz, 3), "frac": round(fp8_tf / f8_tf, 4)}
    result["rooflines"]["decode"]["measured_peak"] = {
        "kind": "HBM read stream of 2 GiB (rf_peak_read, 2048 workgroups of contiguous 1 MiB)",
        "achieved": round(read_gbs, 1), "unit": "GB/s", "frac": round(dec_gbs / read_gbs, 4),
        "copy_1GiB": {"achieved": round(copy_gbs, 1), "unit": "GB/s (read + write bytes, torch copy)"}}
    progress("measured MFMA and copy ceilings timed")

    # The vendor libraries on the same inputs, row by row (torch's own kernels;
    # none of them is part of the path). Short launches run back to back behind
    # a spin kernel, as for the routing roofline.
    def vendor_time(fn, n, warm=3):
        for _ in range(warm):
            fn(0)
        torch.cuda.synchronize()
        torch.cuda._sleep(2_000_000)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / n

    def torch_routing(i):
        p = torch.softmax(logits[i % ROUTING_ROTATE], dim=-1)
        wv, iv = torch.topk(p, R["k"], dim=-1)
        return wv / wv.sum(dim=-1, keepdim=True), iv

    t_vr = vendor_time(torch_routing, 2 * ROUTING_ROTATE)
    vendor = {"routing": {"kind": "torch softmax, topk, renormalise", "us_per_launch": round(t_vr * 1e6, 2),
                          "speedup": round(t_vr / t_rout_b2b, 3)}}
    sm_v, var_v = {}, {}
    for E in SOFTMAX_E:
        T = SOFTMAX_VALUES // E
        xs = rotated(inputs.softmax_inputs(6, T, E).to(dev))
        t_v = vendor_time(lambda i: torch.softmax(xs[i % ROW_ROTATE], dim=-1), 10)
        sm_v[f"E{E}"] = {"GBs": round(8.0 * T * E / t_v / 1e9, 1),
                         "speedup": round(t_v / sm_rates[(E, "block")][0], 3)}
        xm = rotated(inputs.moment_inputs(8, T, E)[0].to(dev))
        t_v = vendor_time(lambda i: torch.var_mean(xm[i % ROW_ROTATE], dim=-1, unbiased=False), 10)
        best = min(mom[("variance", E, ln)][0] for ln in levels if ln != "unfused")
        var_v[f"E{E}"] = {"GBs": round(4.0 * T * E / t_v / 1e9, 1), "speedup": round(t_v / best, 3)}
        del xs, xm
    vendor["softmax_rows"] = {"kind": "torch.softmax over the same rows; speedup of the block-level form",
                              "by_row_length": sm_v}
    vendor["variance"] = {"kind": "torch.var_mean(unbiased=False); speedup of the best fused form",
                          "by_row_length": var_v}
    try:
        a8 = aq.view(torch.float8_e4m3fn)
        b8 = bq.view(torch.float8_e4m3fn)
        rf.rf_absmax_quant_fp8(a_bufs[0], aq, sa)
        sa2, sb2 = sa.view(-1, 1), bs.view(1, -1)
        t_vg = vendor_time(lambda i: torch._scaled_mm(a8, b8.t(), scale_a=sa2, scale_b=sb2,
                                                      out_dtype=torch.bfloat16), 10)
        vendor["fp8_gemm"] = {"kind": "torch._scaled_mm with row and column scales (GEMM only) on this "
                                      "path's quantised operands",
                              "us_per_launch": round(t_vg * 1e6, 2),
                              "tflops": round(gemm_flops() / t_vg / 1e12, 1),
                              "this_path_quant_plus_gemm_us": round(per["fp8"] * 1e6, 2)}
    except RuntimeError as ex:
        progress(f"torch scaled FP8 GEMM unavailable: {ex}")
        vendor["fp8_gemm"] = None
    result["vendor"] = vendor
    progress("vendor kernels timed for context")
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result))


if __name__ == "__main__":
    main()
