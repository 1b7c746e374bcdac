"""Benchmark of the decoder block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode]
    python bench.py --steps 3 --warmup 1 --no-cpu-baseline --copy-calibration   (under rocprofv3 --pmc)
    python bench.py --ingest-pmc FETCH_DIR WRITE_DIR                          (no GPU: writes profiles/)

A step is one pass of the whole block over one batch of seeded synthetic
input (random-init weights, no checkpoints):

  * headline: Llama-3-8B-shaped block prefill, B=1, L=4096, bf16 weights /
    float32 accumulation (a self-contained prefill, mojolearn forward with no
    state): whole-block tokens/s and the share of the bf16 MFMA peak (the
    prefill captured in a HIP graph and replayed; the eagerly launched time is
    reported beside it);
  * decode: the same block shape, 64 rows one token each, KV cache of 8192
    slots pre-filled to per-row positions drawn from [1024, 8192): step time
    (the step captured in a HIP graph and replayed; the eagerly launched time
    is reported beside it) and achieved HBM bandwidth.

HBM traffic of the dominant kernel: two rocprofv3 --pmc runs (FETCH_SIZE,
then WRITE_SIZE) of this script with --copy-calibration, which adds a plain
1 GiB device copy; --ingest-pmc scales each counter by what it read for that
copy and stores bytes per launch under profiles/ together with a hash of the
kernel sources.  A normal run reports that figure as roofline.traffic while
the hash still matches, else null.

Inputs are resident in HBM before timing starts.  The timed region is K
steps bracketed by device synchronisation; per-kernel durations come from
HIP events recorded around each launch on the launch stream during the same
region.  Prints ONE JSON line on stdout; details go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block prefill tokens/s (%MFMA peak) + decode step µs (%HBM BW), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (published)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def mlp_matrices(cfg):
    """Weight matrices of the MLP: gate, up, down (ungated MLPs have no gate)."""
    return 2 if cfg.get("mlp", "swiglu") in ("gelu", "gelu_tanh") else 3


def prefill_flops(cfg, B, L):
    """Algorithmic flops of one block prefill: GEMMs plus unmasked attention pairs."""
    d, H, KV, hd, IT = cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["intermediate"]
    QW, KW = H * hd, KV * hd
    T = B * L
    gemm = 2 * T * (d * (QW + 2 * KW) + QW * d + mlp_matrices(cfg) * d * IT)
    W = cfg.get("window", 0)
    pairs = 0
    for t in range(L):
        pairs += min(t + 1, W) if W else t + 1
    attn = 4 * H * hd * B * pairs
    return gemm, attn


def decode_bytes(cfg, lengths, elem=2):
    d, KV, hd, IT, H = cfg["d_model"], cfg["n_kv_heads"], cfg["head_dim"], cfg["intermediate"], cfg["n_heads"]
    QW, KW = H * hd, KV * hd
    B = len(lengths)
    weights = (d * (QW + 2 * KW) + QW * d + mlp_matrices(cfg) * d * IT) * elem
    W = cfg.get("window", 0)
    keys = sum(min(int(p) + 1, W) if W else int(p) + 1 for p in lengths)
    kv_read = keys * KV * hd * 2 * elem          # every attended key and value once (incl. the new one)
    append = B * KV * hd * 2 * elem
    io = 2 * B * d * 4
    return weights, kv_read, append, io


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_gate_up_llama3_8b_prefill_4k_traffic.json")
# What defines the prefill gate/up GEMM launch: its kernel source, the device
# helpers, the GemmArgs struct and the host's tile planning.
GEMM_SOURCES = [("gqa_causal_attention_amd/csrc/kernels/gemm_dma.hip", None, None),
                ("gqa_causal_attention_amd/csrc/kernels/common.h", None, None),
                ("gqa_causal_attention_amd/csrc/kernels/launch.h", "struct GemmArgs {", "};"),
                ("gqa_causal_attention_amd/csrc/host/block.cpp", "int big_tile() {", "struct WsLayout {")]
COPY_BYTES = 1 << 30          # the calibration copy: 1 GiB read + 1 GiB written


def sources_hash(parts):
    """Hash of the listed files (or of the text between two markers in them)."""
    import hashlib
    h = hashlib.sha256()
    for path, begin, end in parts:
        with open(os.path.join(ROOT, path), "rb") as f:
            data = f.read()
        if begin is not None:
            i = data.index(begin.encode())
            data = data[i:data.index(end.encode(), i)]
        h.update(data)
    return h.hexdigest()[:16]


def stored_traffic():
    """HBM bytes per launch of the prefill gate/up GEMM from the committed
    counter runs, or None when the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_hash") != sources_hash(GEMM_SOURCES):
        return None
    return rec


def ingest_pmc(fetch_dir, write_dir):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)
    of `bench.py --copy-calibration` into bytes per gate/up launch, each counter
    scaled by its reading for the 1 GiB calibration copy."""
    import csv
    import glob
    import re

    def rows(d, counter):
        out = []
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(fn) as f:
                for r in csv.DictReader(f):
                    if r["Counter_Name"] == counter:
                        out.append((r["Kernel_Name"], float(r["Counter_Value"]), int(r["Grid_Size"])))
        if not out:
            raise SystemExit(f"no {counter} records under {d}")
        return out

    gu = re.compile(r"gemm_dma_kernel<256, 256, 64, 2, 2, 4, 16, 1, 1, 2, 0>")
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rr = rows(d, counter)
        g = [v for n, v, _ in rr if gu.search(n)]
        c = [v for n, v, grid in rr if "copyBuffer" in n and grid >= 65536]
        if not g or not c:
            raise SystemExit(f"{counter}: gate/up dispatches {len(g)}, copy dispatches {len(c)}")
        copy_kib = max(c)
        scale = COPY_BYTES / (copy_kib * 1024.0)
        res[counter] = {"kernel_kib_avg": sum(g) / len(g), "dispatches": len(g), "copy_kib": copy_kib,
                        "scale": scale, "bytes": sum(g) / len(g) * 1024.0 * scale}
    rec = {"kernel": "gemm_gate_up", "workload": "llama3_8b_prefill_4k",
           "sources_hash": sources_hash(GEMM_SOURCES),
           "fetch_bytes": round(res["FETCH_SIZE"]["bytes"]), "write_bytes": round(res["WRITE_SIZE"]["bytes"]),
           "traffic_bytes": round(res["FETCH_SIZE"]["bytes"] + res["WRITE_SIZE"]["bytes"]),
           "counters": res}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def copy_calibration(torch):
    """A plain device copy of known size for the counter runs to scale by."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[calibration] copied {COPY_BYTES} bytes 3 times")


def bench_prefill(args, torch):
    from gqa_causal_attention_amd import Block
    from gqa_causal_attention_amd.workloads import make_workload
    t0 = time.time()
    wl = make_workload("llama3_8b_prefill_4k")
    wl["cfg"] = cfg = dict(wl["cfg"], **VARIANTS[args.variant])
    wl["weights"] = variant_weights(wl, cfg)
    B, L = wl["batch"], wl["seq_len"]
    blk = Block(cfg, wl["weights"])
    x = torch.from_numpy(wl["x"]).cuda()
    y = torch.empty_like(x)
    log(f"[prefill] inputs ready in {time.time() - t0:.1f}s")
    for _ in range(args.warmup):
        blk.forward(x, out=y)
    torch.cuda.synchronize()
    blk.set_timing(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        blk.forward(x, out=y)
    torch.cuda.synchronize()
    el = time.perf_counter() - t1
    times = blk.kernel_times()
    blk.set_timing(False)
    ms_eager = el * 1e3 / args.steps
    # The same prefill captured once in a HIP graph and replayed: the step
    # without per-launch host overhead (workspace already allocated above).
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        blk.forward(x, out=y)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t1) * 1e3 / args.steps
    log(f"[prefill] step {ms:.4f} ms replayed from a HIP graph, {ms_eager:.4f} ms launched eagerly")
    gemm_f, attn_f = prefill_flops(cfg, B, L)
    d, IT = cfg["d_model"], cfg["intermediate"]
    T = B * L
    gated = mlp_matrices(cfg) == 3
    mlp_in = "gemm_gate_up" if gated else "gemm_up"
    per_kernel_flops = {
        "gemm_qkv": 2 * T * d * (cfg["n_heads"] + 2 * cfg["n_kv_heads"]) * cfg["head_dim"],
        "gemm_o": 2 * T * cfg["n_heads"] * cfg["head_dim"] * d,
        mlp_in: 2 * T * d * (2 if gated else 1) * IT,
        "gemm_down": 2 * T * IT * d,
        "attn_prefill": attn_f,
    }
    breakdown = {}
    for name, (tot, cnt) in times.items():
        avg = tot / max(cnt, 1)
        f = per_kernel_flops.get(name)
        breakdown[name] = {"avg_ms": round(avg, 4), "launches": cnt,
                           "tflops": round(f / (avg * 1e-3) / 1e12, 1) if f else None}
    log("[prefill] per-kernel (HIP events over the timed region):")
    for k, v in breakdown.items():
        log(f"   {k:16s} {v}")
    gu = breakdown[mlp_in]
    achieved = per_kernel_flops[mlp_in] / (gu["avg_ms"] * 1e-3) / 1e12
    # the stored counter record is the plain block's gate/up launch
    tr = stored_traffic() if args.variant == "plain" else None
    roofline = {"bound": "mfma", "kernel": mlp_in, "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": tr["traffic_bytes"] if tr else None,
                "algorithmic_bytes": 2 * (T * d + (2 if gated else 1) * IT * d + T * IT),
                "flops_per_launch": per_kernel_flops[mlp_in]}
    total_f = gemm_f + attn_f
    step_tflops = total_f / (ms * 1e-3) / 1e12
    return dict(cfg=cfg, B=B, L=L, ms=ms, ms_eager=ms_eager, tokens_per_s=T / (ms * 1e-3), roofline=roofline,
                step={"tflops": round(step_tflops, 1), "frac_of_peak": round(step_tflops / PEAK_BF16_TFLOPS, 4),
                      "algorithmic_tflop": round(total_f / 1e12, 4)},
                breakdown=breakdown, wl=wl)


def bench_backward(args, torch, wl):
    """Gradients of a zero-state prefill on the prefill workload (x, and a seeded
    N(0, 1) grad_output): the forward recompute plus the backward, timed over
    eager launches (synchronised), with per-kernel HIP events in a second pass."""
    from gqa_causal_attention_amd import Block
    cfg, B, L = wl["cfg"], wl["batch"], wl["seq_len"]
    blk = Block(cfg, wl["weights"])
    x = torch.from_numpy(wl["x"]).cuda()
    dy = torch.from_numpy(np.random.default_rng(7).standard_normal(wl["x"].shape, dtype=np.float32)).cuda()
    grads = blk.backward(x, dy)
    for _ in range(args.warmup):
        blk.backward(x, dy, grads=grads)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        blk.backward(x, dy, grads=grads)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t1) * 1e3 / args.steps
    blk.set_timing(True)
    for _ in range(3):
        blk.backward(x, dy, grads=grads)
    torch.cuda.synchronize()
    times = blk.kernel_times()
    blk.set_timing(False)
    gemm_f, attn_f = prefill_flops(cfg, B, L)
    # recompute (gemm_f + attn_f), the dX and dW products (2 gemm_f), the
    # attention backward (S again, dP, dV, dQ, dK: 2.5 attn_f)
    flops = 3 * gemm_f + 3.5 * attn_f
    per = {k: round(v[0] / max(v[1], 1), 4) for k, v in times.items()}
    log(f"[backward] step {ms:.3f} ms, {flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s algorithmic")
    for k, v in sorted(per.items(), key=lambda kv: -kv[1] * times[kv[0]][1]):
        log(f"   {k:20s} avg {v:.4f} ms x {times[k][1] // 3} per step")
    del grads
    return {"workload": "llama3-8b-shaped block backward of a zero-state prefill, B=1 L=4096 (x and nine weight "
                        "gradients; forward recomputed)",
            "step_ms": round(ms, 3), "algorithmic_tflop": round(flops / 1e12, 4),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_of_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "attention_ms": round(per.get("bwd_attention", 0.0), 3)}


def bench_decode(args, torch):
    from gqa_causal_attention_amd import Block
    from gqa_causal_attention_amd.workloads import make_workload
    t0 = time.time()
    wl = make_workload("llama3_8b_decode_b64")
    wl["cfg"] = cfg = dict(wl["cfg"], **VARIANTS[args.variant])
    wl["weights"] = variant_weights(wl, cfg)
    B, cap = wl["batch"], wl["capacity"]
    lengths = wl["lengths"]
    blk = Block(cfg, wl["weights"])
    st = blk.allocate_state(B, cap)
    st.k.copy_(torch.from_numpy(wl.pop("k_fill")).cuda().to(torch.bfloat16))
    st.v.copy_(torch.from_numpy(wl.pop("v_fill")).cuda().to(torch.bfloat16))
    x = torch.from_numpy(wl["x"]).cuda()
    y = torch.empty_like(x)
    log(f"[decode] inputs ready in {time.time() - t0:.1f}s")
    for _ in range(args.warmup):
        st.set_lengths(lengths)
        blk.step(x, st, out=y)
    torch.cuda.synchronize()
    blk.set_timing(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        st.set_lengths(lengths)       # every step decodes at the same positions
        blk.step(x, st, out=y)
    torch.cuda.synchronize()
    el = time.perf_counter() - t1
    times = blk.kernel_times()
    blk.set_timing(False)
    us_eager = el * 1e6 / args.steps
    # The same step captured once in a HIP graph (positions restored on the
    # device inside the graph) and replayed: no per-launch host overhead.
    lengths_dev = torch.from_numpy(lengths.astype(np.int32)).cuda()
    st.set_lengths(lengths)
    blk.step(x, st, out=y)                  # workspace and code paths warm
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.lengths.copy_(lengths_dev)
        blk.step(x, st, out=y)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t1) * 1e6 / args.steps
    st.set_lengths(lengths)                 # host mirror back in step with the device
    log(f"[decode] step {us:.1f} us replayed from a HIP graph, {us_eager:.1f} us launched eagerly")
    wb, kvb, apb, iob = decode_bytes(cfg, lengths)
    total = wb + kvb + apb + iob
    breakdown = {k: {"avg_us": round(t / max(c, 1) * 1e3, 2), "launches": c} for k, (t, c) in times.items()}
    log("[decode] per-kernel (HIP events over the eager timed region):")
    for k, v in breakdown.items():
        log(f"   {k:22s} {v}")
    att = breakdown.get("attn_decode")
    kv_bytes_launch = kvb
    achieved = kv_bytes_launch / (att["avg_us"] * 1e-6) / 1e9 if att else None
    roofline = {"bound": "hbm", "kernel": "attn_decode", "achieved": round(achieved, 1) if achieved else None,
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4) if achieved else None, "traffic": None,
                "bytes_per_launch": kv_bytes_launch}
    gbs = total / (us * 1e-6) / 1e9
    return dict(us=us, us_eager=us_eager, tokens_per_s=B / (us * 1e-6), bytes=total, gbs=gbs,
                frac=gbs / PEAK_HBM_GBS, roofline=roofline, breakdown=breakdown, B=B)


def cpu_baseline(pre, budget_s=20.0):
    """The CPU oracle (float32 numpy, as it stands) on the first 512 positions of
    the same prefill workload (a causal prefix: those rows' outputs are exactly
    the full run's), repeated until ~budget_s of work; reported in tokens/s."""
    from threadpoolctl import threadpool_info

    from oracle import block_forward
    wl = pre["wl"]
    cfg, W, x = wl["cfg"], wl["weights"], wl["x"][:, :512]
    n, t0 = 0, time.perf_counter()
    while True:
        block_forward(cfg, W, x)
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": round(n * x.shape[1] / el, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} x prefill of the first 512 of 4096 positions (causal prefix), float32 numpy, "
                      f"{el:.1f}s wall"}


# Options of the block on the same 8B shapes (the default is the plain
# block): Llama 3.1's RoPE ramp (factor 8 over an original 8192-token context)
# changes only the table; half rotary (64 of 128 dimensions) splits each head's
# RoPE lanes into rotated and pass-through ones; Gemma-style sandwich norms add
# two output norms ((1 + w) RMSNorm, tanh GeGLU); LayerNorm with every bias;
# an ungated exact-GELU MLP (no gate_proj: two thirds of the MLP weights).
VARIANTS = {
    "plain": {},
    "llama31": {"rope_scaling": {"type": "llama3", "factor": 8.0, "low_freq_factor": 1.0,
                                 "high_freq_factor": 4.0, "original_max_position_embeddings": 8192}},
    "half_rotary": {"rope_dim": 64},
    "gemma_sandwich": {"norm": "rmsnorm_offset", "mlp": "geglu_tanh", "sandwich_norms": True},
    "layernorm_biases": {"norm": "layernorm", "norm_bias": True, "qkv_bias": True, "o_bias": True,
                         "mlp_bias": True},
    "ungated_gelu": {"mlp": "gelu"},
}


def variant_weights(wl, cfg):
    """The workload's weights for a variant config: the same draws for the
    tensors both have, the variant's extra tensors drawn after them."""
    from gqa_causal_attention_amd.workloads import draw_weights, weight_shapes
    W = wl["weights"]
    shapes = weight_shapes(cfg)
    if set(shapes) == set(W):
        return W
    extra = draw_weights(cfg, np.random.default_rng(12345))
    return {k: (W[k] if k in W else extra[k]) for k in shapes}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variant", choices=list(VARIANTS), default="plain",
                    help="block options on the same shapes (default: the plain Llama-shaped block)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="decode line only (profiling); no JSON headline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (scale for the --pmc byte counters)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs into the stored gate/up traffic record (no GPU)")
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(*args.ingest_pmc)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the block runs on a single device); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.no_prefill:
        dec = bench_decode(args, torch)
        log(json.dumps({"decode_step_us": round(dec["us"], 2), "achieved_gbs": round(dec["gbs"], 1)}))
        return
    pre = bench_prefill(args, torch)
    if args.copy_calibration:
        copy_calibration(torch)
    dec = None if args.no_decode else bench_decode(args, torch)
    bwd = None if (args.no_backward or args.variant != "plain") else bench_backward(args, torch, pre["wl"])
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(pre)
        log(f"[cpu] {cpu}")
    out = {
        "metric": METRIC,
        "value": round(pre["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms"], 4),
        "ms_per_step_eager": round(pre["ms_eager"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3-8b-shaped block prefill (d=4096, 32/8 heads, hd=128, IT=14336)",
                   "batch": pre["B"], "seq_len": pre["L"], "parallelism": "none",
                   **({"variant": args.variant} if args.variant != "plain" else {})},
        "prefill_mfma": pre["step"],
        "roofline": pre["roofline"],
        "cpu_baseline": cpu,
    }
    if dec:
        out["decode"] = {"workload": "llama3-8b-shaped block decode, 64 rows, cache 8192, positions U[1024, 8192)",
                         "step_us": round(dec["us"], 2), "step_us_eager": round(dec["us_eager"], 2),
                         "tokens_per_s": round(dec["tokens_per_s"], 1),
                         "algorithmic_bytes": dec["bytes"], "achieved_gbs": round(dec["gbs"], 1),
                         "frac_of_hbm_peak": round(dec["frac"], 4), "roofline": dec["roofline"]}
    if bwd:
        out["backward"] = bwd
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
