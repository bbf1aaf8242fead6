"""Benchmark of the join-agg einsum executor on one MI355X.

One step = one pass of the whole hot path over the LLaMA-7B-shaped block
(4 x 2048 tokens, hidden 4096, 32 heads x 128, SwiGLU 11008, bf16 weights):
every operator is a join-agg spec (join enumeration, MFMA block contraction,
streaming map / SUM-MAX reduce) and the head-major relayouts around the
causal attention are repartitions.  Inputs are seeded synthetic tensors
already resident in HBM when the timed region starts.

Prints one JSON line: value = algorithmic TFLOP/s of the step (contraction
FLOPs, causal attention counted element-wise) with the chain recorded once
as a HIP graph and replayed per step (the eager per-call timing is reported
beside it and feeds the per-spec breakdown), a roofline entry for the
dominant kernel (the bf16 MFMA contraction of the projection / FFN specs),
the repartition GB/s of the 8192^2, 4-D and packed-sequence (interval)
reblocking workloads, the other measured workloads (256^3 matmul, the
attention chain and its fused, grouped-query and packed-sequence forms, the
multi-index fp32 contraction) with per-spec rates, and the CPU oracle timed
on a bounded sample of the block's specs.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from tensor_relational_einsum_amd import inputs as I  # noqa: E402
from tensor_relational_einsum_amd import jagg  # noqa: E402
from tensor_relational_einsum_amd.runner import ChainRunner  # noqa: E402

METRIC = "join-agg einsum TFLOP/s (% bf16 MFMA peak) + repartition GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def spec_flops(st: I.Step, ext: dict) -> float:
    """Algorithmic FLOPs of a contraction spec: 2 per multiply-add over the
    unpadded index space; under a causal pair only t <= s is counted.  Fused
    attention counts its two products (scores and P V), as the unfused chain
    does; softmax arithmetic is not counted."""
    ins = st.spec.split("->")[0].split(",")
    if st.g == "attention":
        q, k, v = ins
        groups = [set(q) | set(k), set(v) | set(st.spec.split("->")[1])]
    elif st.g == "mul" and st.agg == "sum" and len(st.ins) == 2:
        groups = [set("".join(ins))]
    else:
        return 0.0
    total = 0.0
    for letters in groups:
        n = 1.0
        for c in letters:
            n *= ext[c]
        if st.segment:
            # (s, t) pairs inside each segment only (t <= s under a causal pair)
            s, t = st.segment
            b = st.blockings[s]
            if isinstance(b, list):
                lens = [y - x for x, y in zip(b, b[1:])]
            else:
                e = -(-ext[s] // b)
                lens = [min(e, ext[s] - q * e) for q in range(b)]
            pairs = sum(L * (L + 1) / 2 if st.causal else L * L for L in lens)
            n = n / (ext[s] * ext[t]) * pairs
        elif st.causal:
            s, t = st.causal
            S = ext[s]
            n = n / (ext[s] * ext[t]) * (S * (S + 1) / 2)
        total += 2.0 * n
    return total


def spec_bytes(run: ChainRunner, st, ext: dict) -> float:
    """Algorithmic bytes of a spec or relayout: every valid element of each
    input read once and of the output written once."""
    def rel_bytes(name):
        r = run.rel[name]
        return math.prod(r.extents) * jagg.ESZ[r.dtype]
    if isinstance(st, I.Relayout):
        return 2.0 * rel_bytes(st.src)
    b = rel_bytes(st.out) + sum(rel_bytes(n) for n in st.ins)
    if st.causal:
        # score-shaped operands only hold t <= s
        s, t = st.causal
        frac = (ext[s] + 1) / (2 * ext[s])
        b = 0.0
        for n in list(st.ins) + [st.out]:
            r = run.rel[n]
            full = math.prod(r.extents) * jagg.ESZ[r.dtype]
            b += full * frac if (s in r.letters and t in r.letters) else full
    return b


def counter_traffic() -> float | None:
    """HBM bytes per launch of the bf16 contraction kernel, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, if the kernel source is still
    the one the counters were taken on."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "llama_block_fused_attention_hbm_counters.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", " ")):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if "traffic_bytes_per_launch" not in vals or "kernel_source_sha256_16" not in vals:
        return None
    h = hashlib.sha256()
    for rel in ("tensor_relational_einsum_amd/csrc/contract_impl.h", "tensor_relational_einsum_amd/csrc/contract_dma.h",
                "tensor_relational_einsum_amd/csrc/contract_bf16.hip"):
        h.update(open(os.path.join(ROOT, rel), "rb").read())
    if h.hexdigest()[:16] != vals["kernel_source_sha256_16"]:
        return None
    return float(vals["traffic_bytes_per_launch"])


def timed_graph(run: ChainRunner, steps: int, warmup: int) -> float:
    """Mean ms per step when the whole chain is recorded once as a HIP graph
    (jagg_capture_begin / jagg_capture_end) and replayed once per step: the
    same launches as the eager chain, joins included, without per-call host
    work in between."""
    g = run.capture()
    for _ in range(max(warmup, 1)):
        g.launch()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(run.ctx.stream)
    for _ in range(steps):
        g.launch()
    b.record(run.ctx.stream)
    torch.cuda.synchronize()
    g.close()
    return a.elapsed_time(b) / steps


def timed_chain(run: ChainRunner, steps: int, warmup: int):
    stream = run.ctx.stream
    n = len(run.calls)
    for _ in range(warmup):
        run.run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        ev[k][0].record(stream)
        for i in range(n):
            run.run_step(i)
            ev[k][i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = np.zeros((steps, n))
    step_ms = np.zeros(steps)
    for k in range(steps):
        for i in range(n):
            per_call[k, i] = ev[k][i].elapsed_time(ev[k][i + 1])
        step_ms[k] = ev[k][0].elapsed_time(ev[k][n])
    return step_ms, per_call, wall


def flush_caches(buf):
    # A 512 MiB read evicts L2 and the 256 MB Infinity Cache.  It must not
    # write: dirty lines left by the flush would be written back while the
    # timed kernel runs (a plain 128 MiB copy drops from 5.1-5.4 to 4.0 TB/s).
    return buf.sum()


def repartition_rate(ctx, w: I.Workload, reps: int, scratch) -> dict:
    dense = I.generate(w)
    run = ChainRunner(ctx, w, dense)
    st = w.chain[0]
    src, dst = run.rel[st.src], run.rel[st.out]
    # algorithmic bytes: every element read once, every destination slot
    # (padding of interval blocks included) written once
    nbytes = float(math.prod(src.extents) * jagg.ESZ[src.dtype] + dst.nbytes)
    for _ in range(3):
        jagg.repartition(ctx, src, dst)
    times = []
    for _ in range(reps):
        flush_caches(scratch)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(ctx.stream)
        jagg.repartition(ctx, src, dst)
        b.record(ctx.stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    med = float(np.median(times))
    gbps = nbytes / (med * 1e-3) / 1e9
    return {"workload": w.name, "bytes": nbytes, "ms_median": med, "ms_min": float(np.min(times)),
            "GB/s": gbps, "frac_hbm": gbps / PEAK_HBM_GBPS}


def other_config(ctx, w: I.Workload, steps: int = 5, warmup: int = 2) -> dict:
    """One of the other measured workloads: the step time both as one ABI
    call per spec and as the chain recorded as a HIP graph and replayed
    (events on the context stream around the timed steps, as for the main
    workload), the rate and fraction of the bounding peak from the faster of
    the two (a graph replay carries a fixed launch cost that a chain of one
    or two kernels does not recover), and per-spec rates from the eager
    calls (events around every call, joins included)."""
    dense = I.generate(w)
    run = ChainRunner(ctx, w, dense)
    step_ms, per_call, _ = timed_chain(run, steps, warmup)
    eager_ms = float(np.mean(step_ms))
    graph_ms = timed_graph(run, steps, warmup)
    ms = min(eager_ms, graph_ms)
    call_ms = per_call.mean(axis=0)
    flops = sum(spec_flops(st, w.extents) if isinstance(st, I.Step) else 0.0 for st in w.chain)
    big = max((st for st in w.chain if isinstance(st, I.Step)), key=lambda st: spec_flops(st, w.extents))
    in_dtype = run.rel[big.ins[0]].dtype
    peak = PEAK_F32_TFLOPS if in_dtype == "f32" else PEAK_BF16_TFLOPS
    specs = []
    for i, st in enumerate(w.chain):
        by = spec_bytes(run, st, w.extents)
        f = spec_flops(st, w.extents) if isinstance(st, I.Step) else 0.0
        e = {"name": st.out, "op": st.spec if isinstance(st, I.Step) else f"relayout->{st.letters}",
             "ms": round(float(call_ms[i]), 4), "GB/s": round(by / (call_ms[i] * 1e-3) / 1e9, 1),
             "frac_hbm": round(by / (call_ms[i] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 3)}
        if f:
            e["TFLOP/s"] = round(f / (call_ms[i] * 1e-3) / 1e12, 2)
        specs.append(e)
    tf = flops / (ms * 1e-3) / 1e12
    out = {"workload": w.name, "ms_per_step": round(ms, 4), "TFLOP/s": round(tf, 3), "dtype": in_dtype,
           "frac_mfma_peak": round(tf / peak, 4), "peak_TFLOP/s": peak,
           "execution": "graph replay" if graph_ms <= eager_ms else "one ABI call per spec",
           "eager_ms_per_step": round(eager_ms, 4), "graph_ms_per_step": round(graph_ms, 4), "specs": specs}
    del run, dense
    torch.cuda.synchronize()
    return out


def cpu_baseline(w: I.Workload, dense: dict, target_s: float = 12.0) -> dict:
    """The oracle, as it stands, on a bounded sample of the block's
    contraction specs: sampled outputs of each projection / FFN spec, scaled
    to TFLOP/s from the sampled multiply-adds."""
    from oracle import oracle as O

    vals = {k: v.to(torch.float64).numpy() for k, v in dense.items() if v.dim() > 0}
    # the projection specs read r1 / r2 (bf16); a stand-in with the same
    # shape and distribution is enough to time the oracle's loops
    gen = I.streams(4242, 2)
    vals["r1"] = I.draw(gen[0], [w.extents[c] for c in "bsh"], "normal", "bf16").to(torch.float64).numpy()
    vals["r2"] = vals["r1"]
    vals["O"] = I.draw(gen[1], [w.extents[c] for c in "bsqd"], "normal", "bf16").to(torch.float64).numpy()
    # (r1, r2 and O are outputs of earlier steps: stand-ins of the same shape)
    specs = [st for st in w.chain if isinstance(st, I.Step) and spec_flops(st, w.extents) > 0 and not st.causal
             and all(n in vals for n in st.ins)]
    rng = np.random.default_rng(0)
    # calibrate on a small sample, then size the run to about target_s
    st = specs[0]
    out_shape = [w.extents[c] for c in st.spec.split("->")[1]]
    t0 = time.perf_counter()
    O.dense(st.spec, [vals[n] for n in st.ins], w.extents, sample=rng.integers(0, math.prod(out_shape), 2000))
    per_flop = (time.perf_counter() - t0) / (2000 * spec_flops(st, w.extents) / math.prod(out_shape))
    budget = target_s / len(specs)
    flops = 0.0
    t_total = 0.0
    samples = 0
    for st in specs:
        out_shape = [w.extents[c] for c in st.spec.split("->")[1]]
        per_out = spec_flops(st, w.extents) / math.prod(out_shape)
        k = max(1000, int(budget / (per_flop * per_out)))
        idx = rng.integers(0, math.prod(out_shape), k)
        t0 = time.perf_counter()
        O.dense(st.spec, [vals[n] for n in st.ins], w.extents, sample=idx)
        t_total += time.perf_counter() - t0
        flops += k * per_out
        samples += k
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{samples} sampled outputs of the {len(specs)} projection/FFN contraction specs "
                      f"(fp64 nested loops, {t_total:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama",
                    choices=["llama", "llama_chain", "attention", "attention_chain", "attention_gqa",
                             "attention_packed", "multi_index", "matmul"],
                    help="llama / attention: fused attention; *_chain: the five-spec attention chain")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-repartition", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip timing the other workloads (matmul, attention chain and fused forms, multi-index)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this executor has no multi-GPU path "
              "(the sharding design is described, not built); rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    # a stream of its own (default priority): graph capture cannot record the null stream
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    ctx = jagg.Context(0, stream)
    w = {"llama": lambda: I.llama_block(fused_attention=True), "llama_chain": I.llama_block,
         "attention": lambda: I.attention_chain(fused=True), "attention_chain": I.attention_chain,
         "attention_gqa": I.attention_gqa, "attention_packed": I.attention_packed,
         "multi_index": I.multi_index, "matmul": I.matmul_256}[args.workload]()
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    dense = I.generate(w)
    run = ChainRunner(ctx, w, dense)
    print(f"[bench] timing {args.steps} steps after {args.warmup} warm-up", file=sys.stderr, flush=True)
    # eager: one ABI call per spec, events around every call (the breakdown);
    # the step that `value` reports is the chain replayed as a recorded graph
    step_ms, per_call, wall = timed_chain(run, args.steps, args.warmup)
    eager_ms = float(np.mean(step_ms))
    ms = timed_graph(run, args.steps, args.warmup)
    steps = [st for st in w.chain]
    flops = sum(spec_flops(st, w.extents) if isinstance(st, I.Step) else 0.0 for st in steps)
    value = flops / (ms * 1e-3) / 1e12
    call_ms = per_call.mean(axis=0)
    breakdown = []
    dom_flops = dom_ms = dom_bytes = 0.0
    dom_launches = 0
    for i, st in enumerate(steps):
        f = spec_flops(st, w.extents) if isinstance(st, I.Step) else 0.0
        by = spec_bytes(run, st, w.extents)
        ent = {"name": st.out, "op": st.spec if isinstance(st, I.Step) else f"relayout->{st.letters}",
               "ms": round(float(call_ms[i]), 4)}
        if f:
            ent["TFLOP/s"] = round(f / (call_ms[i] * 1e-3) / 1e12, 2)
        ent["GB/s"] = round(by / (call_ms[i] * 1e-3) / 1e9, 1)
        breakdown.append(ent)
        if (isinstance(st, I.Step) and f and not st.causal and st.g == "mul"
                and run.rel[st.ins[0]].dtype == "bf16"):
            dom_flops += f
            dom_ms += float(call_ms[i])
            dom_bytes += by
            dom_launches += 1
    # the arithmetic type of the dominant kernel: the inputs of the largest contraction
    big = max((st for st in steps if isinstance(st, I.Step)), key=lambda st: spec_flops(st, w.extents))
    in_dtype = run.rel[big.ins[0]].dtype
    if dom_launches:
        achieved = dom_flops / (dom_ms * 1e-3) / 1e12
        tr = counter_traffic() if args.workload == "llama" else None
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": tr,
                "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-calibrated)",
                "algorithmic_bytes_per_launch": round(dom_bytes / dom_launches),
                "kernel": "contract_dma_kernel<bf16> (projection / FFN specs, 256x256 tiles)",
                "launches_per_step": dom_launches,
                "avg_launch_ms": round(dom_ms / dom_launches, 4)}
    else:
        peak = PEAK_F32_TFLOPS if in_dtype == "f32" else PEAK_BF16_TFLOPS
        achieved = value
        kname = "attention_kernel<bf16>" if big.g == "attention" else f"contract_kernel<{in_dtype}>"
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None, "kernel": kname}
    rep = {}
    if not args.no_repartition:
        del run
        torch.cuda.empty_cache()
        scratch = torch.zeros(512 << 20 >> 2, dtype=torch.float32, device="cuda")
        rep = {"8192x8192": repartition_rate(ctx, I.repartition_2d(), 15, scratch),
               "32x128x64x64": repartition_rate(ctx, I.repartition_4d(), 15, scratch),
               "packed_to_uniform": repartition_rate(ctx, I.repartition_packed(), 15, scratch),
               "uniform_to_packed": repartition_rate(ctx, I.repartition_packed(to_packed=True), 15, scratch)}
        del scratch
    others = {}
    if not args.no_other_configs and args.workload == "llama":
        print("[bench] timing the other workloads", file=sys.stderr, flush=True)
        for name, mk in (("matmul_256_fp32", I.matmul_256), ("attention_chain", I.attention_chain),
                         ("attention_fused", lambda: I.attention_chain(fused=True)),
                         ("attention_gqa_causal", I.attention_gqa), ("attention_packed_causal", I.attention_packed),
                         ("multi_index_fp32", I.multi_index)):
            others[name] = other_config(ctx, mk())
            torch.cuda.empty_cache()
    if args.copy_calibration:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    cpu = None
    if not args.no_cpu_baseline and args.workload in ("llama", "llama_chain"):
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, dense)
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": in_dtype, "data": "synthetic (seeded; random-init weights)",
        "config": {"workload": w.name, "extents": w.extents, "step_flops": flops, "wall_s": round(wall, 3),
                   "execution": "the chain recorded once as a HIP graph (jagg_capture_begin/end), replayed per step"},
        "roofline": roof, "cpu_baseline": cpu, "repartition": rep, "other_configs": others,
        "eager": {"ms_per_step": round(eager_ms, 4), "value": round(flops / (eager_ms * 1e-3) / 1e12, 3),
                  "note": "the same chain as one ABI call per spec from Python; the breakdown times these calls"},
        "breakdown": breakdown,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
