"""Benchmark of the decoder block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs c2,c3,c4,c5p,c5d,bwd] [--no-cpu-baseline]
    python bench.py --counters c3 --seq-out DIR/sequence.json     (under rocprofv3 --pmc, one leg per run)
    python bench.py --ingest-counters c3 NAME DIR [DIR ...]       (no GPU: writes profiles/NAME.json/.md)

A step is one pass of the whole block over one batch of seeded synthetic
input (random-init weights drawn by gqa_causal_attention_amd.workloads, no
checkpoints).  The headline is the Llama-3-8B-shaped prefill (B=1, L=4096,
bf16 weights / float32 accumulation) into a fresh state (mojolearn
``forward(x, state)`` on an empty cache of 4096 slots, so the cache write is
timed with it): whole-block tokens/s and the share of the bf16 MFMA peak.
Beside it, each as its own JSON object:

  * decode: the same block, 64 rows one token each, a cache of 8192 slots
    pre-filled to per-row positions drawn from [1024, 8192);
  * the Gemma2-style sliding-window prefill (B=2, L=8192, W=4096, hd=256,
    softcap 50), the Qwen-style 32k prefill (q/k/v biases, qk-norm) and its
    decode at 16 rows x 32768 cached positions;
  * the backward of the 8B-shaped prefill (gradients of a zero-state prefill);
  * a measured device copy (the achievable streaming ceiling beside the
    8 TB/s specification);
  * the CPU oracle (float32 numpy, as it stands) on the host's cores for the
    same units of work: the whole 4096-token prefill and one 64-row decode step.

Step times are HIP-graph replays of the step (K back to back between device
synchronisations), plus the same replays each preceded by a 512 MiB read +
write of an unrelated buffer (so the 256 MB Infinity Cache holds none of the
step's weights or cache: the "flushed" figures), plus the eagerly launched
step.  Per-kernel durations come from HIP events the library records around
each launch on the launch stream over the eager timed steps.

HBM traffic per kernel: rocprofv3 --pmc runs of ``--counters LEG`` (FETCH_SIZE,
then WRITE_SIZE; each run also makes a plain 1 GiB device copy), turned into
bytes per launch by ``--ingest-counters``, which scales each counter by what it
read for that copy and stores the result under profiles/ with a hash of the
kernel sources; a normal run reports those bytes as ``roofline.traffic`` while
the hash still matches, else null.

Inputs are resident in HBM before timing starts.  Prints ONE JSON line on
stdout; details go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block prefill tokens/s (%MFMA peak) + decode step µs (%HBM BW), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (published)
FLUSH_BYTES = 512 << 20        # > the 256 MB Infinity Cache
COPY_BYTES = 1 << 30           # the calibration / ceiling copy: 1 GiB read + 1 GiB written

# Legs: key -> (workload, kind).  c2/c3 are the 8B-shaped prefill/decode.
LEGS = {
    "c2": ("llama3_8b_prefill_4k", "prefill"),
    "c3": ("llama3_8b_decode_b64", "decode"),
    "c4": ("gemma2_window_prefill_8k", "prefill"),
    "c5p": ("qwen_long_prefill_32k", "prefill"),
    "c5d": ("qwen_long_decode_b16", "decode"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def mlp_matrices(cfg):
    """Weight matrices of the MLP: gate, up, down (ungated MLPs have no gate)."""
    return 2 if cfg.get("mlp", "swiglu") in ("gelu", "gelu_tanh") else 3


def attn_pairs(L, W):
    """Unmasked (query, key) pairs of one causal row of L tokens (window W)."""
    if not W or W >= L:
        return L * (L + 1) // 2
    return W * (W + 1) // 2 + (L - W) * W


def prefill_flops(cfg, B, L):
    """Algorithmic flops of one block prefill: GEMMs plus unmasked attention pairs."""
    d, H, KV, hd, IT = cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["intermediate"]
    QW, KW = H * hd, KV * hd
    T = B * L
    gemm = 2 * T * (d * (QW + 2 * KW) + QW * d + mlp_matrices(cfg) * d * IT)
    attn = 4 * H * hd * B * attn_pairs(L, cfg.get("window", 0))
    return gemm, attn


def prefill_kernel_flops(cfg, B, L):
    """Algorithmic flops per launch of the prefill's matrix kernels."""
    d, H, KV, hd, IT = cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["intermediate"]
    T = B * L
    gated = mlp_matrices(cfg) == 3
    return {"gemm_qkv": 2 * T * d * (H + 2 * KV) * hd, "gemm_o": 2 * T * H * hd * d,
            ("gemm_gate_up" if gated else "gemm_up"): 2 * T * d * (2 if gated else 1) * IT,
            "gemm_down": 2 * T * IT * d, "attn_prefill": prefill_flops(cfg, B, L)[1]}


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


def decode_kernel_bytes(cfg, lengths, elem=2):
    """Algorithmic bytes per launch of the decode step's streaming kernels."""
    d, KV, hd, IT, H = cfg["d_model"], cfg["n_kv_heads"], cfg["head_dim"], cfg["intermediate"], cfg["n_heads"]
    QW, KW = H * hd, KV * hd
    gated = mlp_matrices(cfg) == 3
    return {"gemm_qkv": d * (QW + 2 * KW) * elem, "gemm_o": QW * d * elem,
            ("gemm_gate_up" if gated else "gemm_up"): (2 if gated else 1) * IT * d * elem,
            "gemm_down": IT * d * elem, "attn_decode": decode_bytes(cfg, lengths, elem)[1]}


# ---- counter records (profiles/counters_<workload>.json) ----

# What defines each kernel family's launches: its source, the shared device
# helpers and launch structs, and the host's planning and launch sequence.
KERNEL_SOURCES = {
    "gemm_dma": ["csrc/kernels/gemm_dma.hip"],
    "gemm_skinny": ["csrc/kernels/gemm_skinny.hip"],
    "attn_prefill": ["csrc/kernels/attn_prefill.hip", "csrc/kernels/attn_tile.h"],
    "attn_decode": ["csrc/kernels/attn_decode.hip"],
    "norm": ["csrc/kernels/norm.hip"],
    "rope_append": ["csrc/kernels/rope_append.hip"],
    "splitk_reduce": ["csrc/kernels/gemm_bf16.hip"],
}
# (file, first marker, end marker): the forward's argument structs and
# launchers, and the host's kernel and tile planning.
SHARED_SOURCES = [("csrc/kernels/common.h", None, None),
                  ("csrc/kernels/launch.h", "struct GemmArgs {", "// Backward of a zero-state prefill"),
                  ("csrc/host/block.cpp", "int big_tile() {", "struct WsLayout {")]


def family_of(role):
    if role.startswith("attn_decode") or role == "attn_combine":
        return "attn_decode"
    if role.startswith("attn_prefill"):
        return "attn_prefill"
    if role.endswith("_reduce"):
        return "splitk_reduce"
    if "norm" in role:
        return "norm"
    if role.startswith("rope") or role == "kv_append":
        return "rope_append"
    return None  # GEMMs: resolved by kind


def sources_hash(files):
    """Hash of the code (comments and whitespace removed, so a reworded comment
    keeps the stored counters) of the files and shared regions."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f, begin, end in [(f, None, None) for f in files] + SHARED_SOURCES:
        with open(os.path.join(ROOT, "gqa_causal_attention_amd", f), encoding="utf-8") as fh:
            data = fh.read()
        if begin is not None:
            i = data.index(begin)
            data = data[i:data.index(end, i)]
        data = re.sub(r"/\*.*?\*/", " ", data, flags=re.S)
        data = re.sub(r"//[^\n]*", " ", data)
        h.update(" ".join(data.split()).encode())
    return h.hexdigest()[:16]


def role_sources(role, kind):
    fam = family_of(role)
    if fam is None:
        fam = "gemm_dma" if kind == "prefill" else "gemm_skinny"
    return KERNEL_SOURCES[fam]


def counters_file(workload):
    return os.path.join(ROOT, "profiles", f"counters_{workload}.json")


def stored_counters(workload, role, kind):
    """The stored counter record of one kernel role, or None when its sources
    changed since the counters were taken."""
    try:
        with open(counters_file(workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    r = rec.get("kernels", {}).get(role)
    if not r or r.get("sources_hash") != sources_hash(role_sources(role, kind)):
        return None
    return r


def stored_traffic(workload, role, kind):
    r = stored_counters(workload, role, kind)
    if not r or "fetch_bytes" not in r or "write_bytes" not in r:
        return None
    return int(r["fetch_bytes"] + r["write_bytes"])


def _not_block_kernel(name):
    return any(s in name for s in ("at::native", "rocclr", "__amd", "elementwise", "fillBuffer", "copyBuffer",
                                   "nonfinite_kernel"))


def _role_matches(role, kernel):
    """Loose check that a dispatch is the launch the recorded order says."""
    if role.endswith("_reduce"):
        return "reduce" in kernel
    if "norm" in role:
        return "norm" in kernel
    return role.split("_")[0] in kernel


def ingest_counters(leg, name, dirs):
    """rocprofv3 --pmc runs of `bench.py --counters LEG` -> profiles/NAME.json/.md.

    The block's dispatches (every kernel that is not a torch or runtime copy /
    fill) come in the launch order the bench recorded (sequence.json in each
    run directory), one role per launch; counters are averaged per role over
    the run's calls.  FETCH_SIZE / WRITE_SIZE (KiB per dispatch) are scaled by
    what the same counter read for the run's 1 GiB device copy."""
    import csv
    import glob
    workload, kind = LEGS[leg]
    per_role, cmds, calib = {}, [], {}
    for d in dirs:
        with open(os.path.join(d, "sequence.json")) as f:
            seq = json.load(f)["sequence"]
        disp = {}
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(fn) as f:
                for r in csv.DictReader(f):
                    did = int(r["Dispatch_Id"])
                    e = disp.setdefault(did, {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"]), "c": {}})
                    e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if not disp:
            raise SystemExit(f"no counter records under {d}")
        order = [disp[k] for k in sorted(disp)]
        counters = sorted({c for e in order for c in e["c"]})
        copies = [e for e in order if "copyBuffer" in e["name"] and e["grid"] >= 65536]
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if c in counters:
                if not copies:
                    raise SystemExit(f"{d}: {c} without a calibration copy")
                kib = max(e["c"][c] for e in copies)
                calib[c] = {"copy_kib": kib, "scale": COPY_BYTES / (kib * 1024.0)}
        blk = [e for e in order if not _not_block_kernel(e["name"])]
        if len(blk) % len(seq) != 0:
            raise SystemExit(f"{d}: {len(blk)} block dispatches, not a multiple of the {len(seq)}-launch step")
        for i, e in enumerate(blk):
            role = seq[i % len(seq)]
            if not _role_matches(role, e["name"]):
                raise SystemExit(f"{d}: dispatch {i} is {e['name']!r}, expected the {role} launch")
            rr = per_role.setdefault(role, {"kernel": e["name"], "grid": e["grid"], "vals": {}})
            for c, v in e["c"].items():
                rr["vals"].setdefault(c, []).append(v)
        cmds.append(f"timeout -s KILL 150 rocprofv3 --pmc {' '.join(counters)} -f csv -d {d} -o run -- "
                    f"python -u bench.py --counters {leg} --seq-out {d}/sequence.json")
    out = {"workload": workload, "leg": leg, "calibration": calib, "commands": cmds, "kernels": {}}
    for role, rr in per_role.items():
        k = {"kernel": rr["kernel"], "dispatches": len(next(iter(rr["vals"].values()))),
             "sources_hash": sources_hash(role_sources(role, kind)),
             "avg": {c: sum(v) / len(v) for c, v in rr["vals"].items()}}
        if "FETCH_SIZE" in k["avg"]:
            k["fetch_bytes"] = round(k["avg"]["FETCH_SIZE"] * 1024.0 * calib["FETCH_SIZE"]["scale"])
        if "WRITE_SIZE" in k["avg"]:
            k["write_bytes"] = round(k["avg"]["WRITE_SIZE"] * 1024.0 * calib["WRITE_SIZE"]["scale"])
        out["kernels"][role] = k
    # merge with an existing record (other counter groups of the same leg)
    path = os.path.join(ROOT, "profiles", name + ".json")
    try:
        with open(path) as f:
            old = json.load(f)
        if old.get("leg") == leg:
            kept = False  # does any value of the old record survive (then its commands stay listed)?
            for role, k in old.get("kernels", {}).items():
                if role in out["kernels"] and k.get("sources_hash") == out["kernels"][role]["sources_hash"]:
                    merged = dict(k)
                    kept = kept or any(c not in out["kernels"][role]["avg"] for c in k.get("avg", {}))
                    merged["avg"] = dict(k.get("avg", {}), **out["kernels"][role]["avg"])
                    merged.update({kk: vv for kk, vv in out["kernels"][role].items() if kk != "avg"})
                    out["kernels"][role] = merged
                elif role not in out["kernels"]:
                    out["kernels"][role] = k
                    kept = True
            if kept:
                out["commands"] = sorted(set(old.get("commands", [])) | set(cmds))
                out["calibration"] = dict(old.get("calibration", {}), **calib)
    except (OSError, ValueError):
        pass
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    write_counters_md(out, os.path.join(ROOT, "profiles", name + ".md"))
    log(f"wrote {path}")


def write_counters_md(rec, path):
    """Human-readable summary of a counter record: bytes against the
    algorithmic bytes, and the matrix-core / cache / LDS derived figures."""
    from gqa_causal_attention_amd.workloads import make_workload
    workload, kind = LEGS[rec["leg"]]
    wl = make_workload(workload, fill_kv=False)
    cfg = wl["cfg"]
    lines = [f"# Counters: {workload} ({kind}, one MI355X)", "",
             "Commands (repo root; one counter group per run), then the ingest step (no GPU):", ""]
    lines += ["    " + c for c in rec["commands"]]
    lines += ["    python bench.py --ingest-counters " + rec["leg"] + " " + os.path.basename(path)[:-3] + " DIR ...", ""]
    for c, v in rec.get("calibration", {}).items():
        lines.append(f"Calibration: a plain 1 GiB device copy reads {c} = {v['copy_kib']:.0f} KiB "
                     f"(scale {v['scale']:.3f}).")
    lines.append("")
    if kind == "prefill":
        algo = prefill_kernel_flops(cfg, wl["batch"], wl["seq_len"])
    else:
        algo = decode_kernel_bytes(cfg, wl["lengths"])
    lines += ["| role | kernel | dispatches | HBM read MB | HBM write MB | algorithmic | MFMA busy | "
              "TCC busy | L2 hit | LDS bank conflicts |", "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for role, k in rec["kernels"].items():
        a = k["avg"]
        fetch = f"{k['fetch_bytes'] / 1e6:.1f}" if "fetch_bytes" in k else ""
        write = f"{k['write_bytes'] / 1e6:.1f}" if "write_bytes" in k else ""
        al = algo.get(role)
        al_s = "" if al is None else (f"{al / 1e9:.1f} GF" if kind == "prefill" else f"{al / 1e6:.1f} MB")
        mf = ""
        if "SQ_VALU_MFMA_BUSY_CYCLES" in a and "SQ_BUSY_CU_CYCLES" in a and a["SQ_BUSY_CU_CYCLES"] > 0:
            # per SIMD (4 per CU) over per-CU busy cycles
            mf = f"{100.0 * a['SQ_VALU_MFMA_BUSY_CYCLES'] / (4.0 * a['SQ_BUSY_CU_CYCLES']):.0f} %"
        tb = ""
        if "TCC_BUSY_sum" in a and "GRBM_GUI_ACTIVE" in a and a["GRBM_GUI_ACTIVE"] > 0:
            tb = f"{100.0 * a['TCC_BUSY_sum'] / (16.0 * a['GRBM_GUI_ACTIVE']):.0f} %"
        hit = ""
        if "TCC_HIT_sum" in a and "TCC_MISS_sum" in a and a["TCC_HIT_sum"] + a["TCC_MISS_sum"] > 0:
            hit = f"{100.0 * a['TCC_HIT_sum'] / (a['TCC_HIT_sum'] + a['TCC_MISS_sum']):.0f} %"
        bc = f"{a['SQ_LDS_BANK_CONFLICT']:.3g}" if "SQ_LDS_BANK_CONFLICT" in a else ""
        kname = k["kernel"] if len(k["kernel"]) < 70 else k["kernel"][:67] + "..."
        lines.append(f"| {role} | `{kname}` | {k['dispatches']} | {fetch} | {write} | {al_s} | {mf} | {tb} | "
                     f"{hit} | {bc} |")
    lines += ["", "Derived columns: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x SQ_BUSY_CU_CYCLES); "
              "TCC busy = TCC_BUSY_sum / (16 channels x GRBM_GUI_ACTIVE), GRBM_GUI_ACTIVE being summed over the "
              "8 XCDs (so this is the per-channel share over 128 channels); L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS).",
              "", "Raw averages per dispatch:", "", "```"]
    for role, k in rec["kernels"].items():
        lines.append(f"{role}: " + ", ".join(f"{c}={v:.4g}" for c, v in sorted(k["avg"].items())))
    lines += ["```", ""]
    with open(path, "w") as f:
        f.write("\n".join(lines))


# ---- timing helpers ----

class Flusher:
    """A 512 MiB buffer read and written before a timed replay, so the 256 MB
    Infinity Cache holds none of the step's own data."""

    def __init__(self, torch):
        self.buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")

    def __call__(self):
        self.buf.add_(1.0)


def replay_times(torch, graph, steps, flusher=None):
    """Per-replay durations (ms) from torch events on the current stream (the
    replay's stream), each replay optionally preceded by a cache flush."""
    ev = []
    for _ in range(steps):
        if flusher is not None:
            flusher()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def timed_replays(torch, graph, steps):
    """K back-to-back replays between device synchronisations: ms per step."""
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t1) * 1e3 / steps


def merge_tails(times):
    """A tail-split GEMM's launches (name, name_tail, name_tail_reduce) as one
    entry: its whole time against its whole work."""
    out = {}
    for name, (tot, cnt) in times.items():
        base = name[:-len("_tail_reduce")] if name.endswith("_tail_reduce") else (
            name[:-len("_tail")] if name.endswith("_tail") else name)
        if base != name and base in times:
            t, c = out.get(base, (0.0, 0))
            out[base] = (t + tot, c)
        else:
            t, c = out.get(name, (0.0, 0))
            out[name] = (t + tot, c + cnt)
    return out


def breakdown_of(times, work, unit):
    out = {}
    times = merge_tails(times)
    for name, (tot, cnt) in times.items():
        avg_ms = tot / max(cnt, 1)
        e = {"avg_us": round(avg_ms * 1e3, 2), "launches": cnt}
        w = work.get(name)
        if w:
            if unit == "flop":
                e["tflops"] = round(w / (avg_ms * 1e-3) / 1e12, 1)
            else:
                e["gbs"] = round(w / (avg_ms * 1e-3) / 1e9, 1)
        out[name] = e
    return out


# ---- legs ----

def leg_prefill(args, torch, leg, flusher, variant="plain", steps=None):
    """Prefill into a fresh state: the graph zeroes the rows' lengths (a fill
    kernel) and runs forward(x, state)."""
    from gqa_causal_attention_amd import Block
    from gqa_causal_attention_amd.workloads import make_workload
    steps = steps or args.steps
    t0 = time.time()
    wl = make_workload(LEGS[leg][0])
    wl["cfg"] = cfg = dict(wl["cfg"], **VARIANTS[variant])
    wl["weights"] = variant_weights(wl, cfg)
    B, L = wl["batch"], wl["seq_len"]
    blk = Block(cfg, wl["weights"])
    st = blk.allocate_state(B, wl["capacity"])
    zeros = np.zeros(B, dtype=np.int32)
    x = torch.from_numpy(wl["x"]).cuda()
    y = torch.empty_like(x)
    log(f"[{leg}] inputs ready in {time.time() - t0:.1f}s")

    def eager():
        st.set_lengths(zeros)
        blk.forward(x, st, out=y)

    for _ in range(args.warmup):
        eager()
    torch.cuda.synchronize()
    blk.set_timing(True)
    t1 = time.perf_counter()
    for _ in range(steps):
        eager()
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t1) * 1e3 / steps
    times = blk.kernel_times()
    blk.set_timing(False)
    st.set_lengths(zeros)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.lengths.zero_()
        blk.forward(x, st, out=y)
    st.set_lengths(zeros)            # the host mirror: capture advanced it
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    ms = timed_replays(torch, graph, steps)
    fl = replay_times(torch, graph, steps, flusher)
    ms_flushed = statistics.median(fl)
    gemm_f, attn_f = prefill_flops(cfg, B, L)
    total_f = gemm_f + attn_f
    kf = prefill_kernel_flops(cfg, B, L)
    bd = breakdown_of(times, kf, "flop")
    log(f"[{leg}] step {ms:.4f} ms replayed ({ms_flushed:.4f} ms median with the cache flushed), "
        f"{ms_eager:.4f} ms eager")
    for k, v in bd.items():
        log(f"   {k:16s} {v}")
    attn_ms = bd.get("attn_prefill", {}).get("avg_us", 0.0) / 1e3
    res = dict(cfg=cfg, B=B, L=L, wl=wl, ms=ms, ms_flushed=ms_flushed, ms_eager=ms_eager, breakdown=bd,
               tokens_per_s=B * L / (ms * 1e-3), total_f=total_f, gemm_f=gemm_f, attn_f=attn_f, kf=kf,
               tflops=total_f / (ms * 1e-3) / 1e12)
    res["summary"] = {
        "workload": f"{LEGS[leg][0]} (d={cfg['d_model']}, {cfg['n_heads']}/{cfg['n_kv_heads']} heads, "
                    f"hd={cfg['head_dim']}, IT={cfg['intermediate']}"
                    + (f", window {cfg['window']}" if cfg.get("window") else "")
                    + (f", softcap {cfg['attn_softcap']:g}" if cfg.get("attn_softcap") else "")
                    + (", qkv bias, qk_norm" if cfg.get("qkv_bias") else "") + f"), B={B}, L={L}, fresh state",
        "ms_per_step": round(ms, 4), "ms_per_step_flushed": round(ms_flushed, 4),
        "ms_per_step_eager": round(ms_eager, 4), "tokens_per_s": round(B * L / (ms * 1e-3), 1),
        "algorithmic_tflop": round(total_f / 1e12, 4), "tflops": round(res["tflops"], 1),
        "frac_of_peak": round(res["tflops"] / PEAK_BF16_TFLOPS, 4),
        "attention": {"tflop": round(attn_f / 1e12, 4), "avg_ms": round(attn_ms, 4),
                      "tflops": round(attn_f / (attn_ms * 1e-3) / 1e12, 1) if attn_ms else None,
                      "share_of_step": round(attn_ms / ms, 3) if attn_ms else None},
        "steps": steps,
    }
    del blk, st, x, y, graph
    torch.cuda.empty_cache()
    return res


def leg_decode(args, torch, leg, flusher, variant="plain", steps=None, keep_fill=False):
    """One decode step of B rows at their own cached positions; every replay
    restores the rows' positions (a device copy inside the graph) so each step
    decodes at the same positions."""
    from gqa_causal_attention_amd import Block
    from gqa_causal_attention_amd.workloads import make_workload
    steps = steps or args.steps
    t0 = time.time()
    wl = make_workload(LEGS[leg][0])
    wl["cfg"] = cfg = dict(wl["cfg"], **VARIANTS[variant])
    wl["weights"] = variant_weights(wl, cfg)
    B, cap = wl["batch"], wl["capacity"]
    lengths = wl["lengths"]
    blk = Block(cfg, wl["weights"])
    st = blk.allocate_state(B, cap)
    st.k.copy_(torch.from_numpy(wl["k_fill"]).cuda().to(torch.bfloat16))
    st.v.copy_(torch.from_numpy(wl["v_fill"]).cuda().to(torch.bfloat16))
    if not keep_fill:
        del wl["k_fill"], wl["v_fill"]
    x = torch.from_numpy(wl["x"]).cuda()
    y = torch.empty_like(x)
    log(f"[{leg}] inputs ready in {time.time() - t0:.1f}s")
    for _ in range(args.warmup):
        st.set_lengths(lengths)
        blk.step(x, st, out=y)
    torch.cuda.synchronize()
    blk.set_timing(True)
    t1 = time.perf_counter()
    for _ in range(steps):
        st.set_lengths(lengths)
        blk.step(x, st, out=y)
    torch.cuda.synchronize()
    us_eager = (time.perf_counter() - t1) * 1e6 / steps
    times = blk.kernel_times()
    blk.set_timing(False)
    lengths_dev = torch.from_numpy(lengths.astype(np.int32)).cuda()
    st.set_lengths(lengths)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.lengths.copy_(lengths_dev)
        blk.step(x, st, out=y)
    st.set_lengths(lengths)                 # host mirror back in step with the device
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    us = timed_replays(torch, graph, steps) * 1e3
    us_flushed = statistics.median(replay_times(torch, graph, steps, flusher)) * 1e3
    wb, kvb, apb, iob = decode_bytes(cfg, lengths)
    total = wb + kvb + apb + iob
    kb = decode_kernel_bytes(cfg, lengths)
    bd = breakdown_of(times, kb, "byte")
    log(f"[{leg}] step {us:.1f} us replayed ({us_flushed:.1f} us median with the cache flushed), "
        f"{us_eager:.1f} us eager")
    for k, v in bd.items():
        log(f"   {k:22s} {v}")
    gbs = total / (us * 1e-6) / 1e9
    res = dict(cfg=cfg, wl=wl, B=B, us=us, us_flushed=us_flushed, breakdown=bd, bytes=total, kb=kb)
    res["summary"] = {
        "workload": f"{LEGS[leg][0]} (d={cfg['d_model']}, {cfg['n_heads']}/{cfg['n_kv_heads']} heads, "
                    f"hd={cfg['head_dim']}, IT={cfg['intermediate']}), {B} rows one token each, cache {cap} slots, "
                    f"positions {int(lengths.min())}..{int(lengths.max())}",
        "step_us": round(us, 2), "step_us_flushed": round(us_flushed, 2), "step_us_eager": round(us_eager, 2),
        "tokens_per_s": round(B / (us * 1e-6), 1), "algorithmic_bytes": total,
        "achieved_gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "achieved_gbs_flushed": round(total / (us_flushed * 1e-6) / 1e9, 1),
        "frac_of_hbm_peak_flushed": round(total / (us_flushed * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "steps": steps,
    }
    del blk, st, x, y, graph
    torch.cuda.empty_cache()
    return res


def leg_ragged(args, torch, steps=None):
    """A ragged batch of the 8B-shaped block (mojolearn forward with
    ``lengths``): 4 rows padded to 4096 tokens, real lengths drawn from
    [256, 4096] (seeded), run packed (only the real tokens through the norms,
    GEMMs and attention); beside it the same batch run unragged, so the time
    can be set against the share of real tokens."""
    from gqa_causal_attention_amd import Block
    from gqa_causal_attention_amd.workloads import make_workload
    steps = steps or args.steps
    wl = make_workload("llama3_8b_prefill_4k", batch=4)
    cfg = wl["cfg"]
    B, L = wl["batch"], wl["seq_len"]
    lens = [int(v) for v in np.random.default_rng(21).integers(256, L + 1, size=B)]
    blk = Block(cfg, wl["weights"])
    x = torch.from_numpy(wl["x"]).cuda()
    y = torch.empty_like(x)
    res, per = {}, {}
    for name, kw in (("ragged", {"lengths": lens}), ("padded", {})):
        for _ in range(args.warmup):
            blk.forward(x, out=y, **kw)
        torch.cuda.synchronize()
        blk.set_timing(True)
        for _ in range(3):
            blk.forward(x, out=y, **kw)
        torch.cuda.synchronize()
        per[name] = {k: round(v[0] / max(v[1], 1), 4) for k, v in merge_tails(blk.kernel_times()).items()}
        blk.set_timing(False)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            blk.forward(x, out=y, **kw)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        res[name] = timed_replays(torch, graph, steps)
        del graph
    real = sum(lens)
    log(f"[c2r] lengths {lens}: ragged {res['ragged']:.4f} ms, padded batch {res['padded']:.4f} ms "
        f"(real tokens {real} of {B * L})")
    for k in per["padded"]:
        log(f"   {k:16s} ragged {per['ragged'].get(k, 0.0):.4f} ms  padded {per['padded'][k]:.4f} ms")
    for k in set(per["ragged"]) - set(per["padded"]):
        log(f"   {k:16s} ragged {per['ragged'][k]:.4f} ms")
    del blk, x, y
    torch.cuda.empty_cache()
    return {"workload": f"llama3_8b_prefill_4k ragged: B={B} rows padded to L={L}, lengths {lens} (seeded U[256, 4096])",
            "ms_per_step": round(res["ragged"], 4), "ms_per_step_padded_batch": round(res["padded"], 4),
            "real_tokens": real, "padded_tokens": B * L, "real_token_share": round(real / (B * L), 4),
            "time_share": round(res["ragged"] / res["padded"], 4),
            "real_tokens_per_s": round(real / (res["ragged"] * 1e-3), 1), "steps": steps}


def leg_backward(args, torch, wl):
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
    log(f"[bwd] step {ms:.3f} ms, {flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s algorithmic")
    for k, v in sorted(per.items(), key=lambda kv: -kv[1] * times[kv[0]][1]):
        log(f"   {k:20s} avg {v:.4f} ms x {times[k][1] // 3} per step")
    del grads, blk
    torch.cuda.empty_cache()
    return {"workload": "llama3-8b-shaped block backward of a zero-state prefill, B=1 L=4096 (x and nine weight "
                        "gradients; forward recomputed)",
            "step_ms": round(ms, 3), "algorithmic_tflop": round(flops / 1e12, 4),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_of_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "attention_ms": round(per.get("bwd_attention", 0.0), 3)}


def copy_ceiling(torch, reps=10):
    """A plain 1 GiB device-to-device copy (torch): (read + write bytes) / time,
    best of `reps` (the achievable streaming rate beside the 8 TB/s spec)."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ev = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    best = min(a.elapsed_time(b) for a, b in ev)
    del src, dst
    torch.cuda.empty_cache()
    return {"gbs": round(2 * COPY_BYTES / (best * 1e-3) / 1e9, 1), "bytes_moved": 2 * COPY_BYTES,
            "best_ms": round(best, 4), "kind": "torch device copy, 1 GiB read + 1 GiB written, best of 10"}


def cpu_threads():
    return len(os.sched_getaffinity(0))


def cpu_prefill(wl, runs=3):
    """The float32 numpy oracle (as it stands) on the whole prefill: median of
    `runs` after one warm-up, BLAS threads pinned to the process's cores."""
    from threadpoolctl import threadpool_limits

    from oracle import block_forward
    cores = cpu_threads()
    cfg, W, x = wl["cfg"], wl["weights"], wl["x"]
    with threadpool_limits(limits=cores):
        ts = []
        for i in range(runs + 1):
            t0 = time.perf_counter()
            block_forward(cfg, W, x)
            if i:
                ts.append(time.perf_counter() - t0)
    med = statistics.median(ts)
    T = x.shape[0] * x.shape[1]
    return {"value": round(T / med, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole prefill (B={x.shape[0]}, L={x.shape[1]}), float32 numpy oracle, median of {runs} "
                      f"after 1 warm-up: {med:.2f} s per prefill ({', '.join(f'{t:.2f}' for t in ts)})"}


def cpu_decode(wl, runs=3):
    """The float32 numpy oracle on one decode step of all rows (the state's
    lengths restored before each run): median of `runs` after one warm-up."""
    from threadpoolctl import threadpool_limits

    from oracle import OracleState, block_step
    cores = cpu_threads()
    cfg, W = wl["cfg"], wl["weights"]
    st = OracleState.from_fill(cfg, wl["k_fill"], wl["v_fill"], wl["lengths"])
    del wl["k_fill"], wl["v_fill"]
    L0 = st.lengths.copy()
    with threadpool_limits(limits=cores):
        ts = []
        for i in range(runs + 1):
            st.lengths[:] = L0
            t0 = time.perf_counter()
            block_step(cfg, W, wl["x"], st)
            if i:
                ts.append(time.perf_counter() - t0)
    med = statistics.median(ts)
    return {"value": round(med * 1e6, 1), "unit": "µs/step", "cores": cores, "kind": "oracle",
            "sample": f"one decode step of all {wl['batch']} rows at the same positions, float32 numpy oracle, "
                      f"median of {runs} after 1 warm-up ({', '.join(f'{t:.2f}' for t in ts)} s)"}


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


def run_counters(args, torch):
    """One leg launched eagerly for rocprofv3 --pmc: one call with the
    library's timing on (its launch order -> --seq-out), then warm-up and
    `steps` calls, then a plain 1 GiB device copy (the counters' scale)."""
    from gqa_causal_attention_amd import Block
    from gqa_causal_attention_amd.workloads import make_workload
    workload, kind = LEGS[args.counters]
    wl = make_workload(workload)
    cfg = wl["cfg"]
    blk = Block(cfg, wl["weights"])
    B = wl["batch"]
    st = blk.allocate_state(B, wl["capacity"])
    x = torch.from_numpy(wl["x"]).cuda()
    y = torch.empty_like(x)
    if kind == "decode":
        st.k.copy_(torch.from_numpy(wl.pop("k_fill")).cuda().to(torch.bfloat16))
        st.v.copy_(torch.from_numpy(wl.pop("v_fill")).cuda().to(torch.bfloat16))
        lens = wl["lengths"]
    else:
        lens = np.zeros(B, dtype=np.int32)

    def call():
        st.set_lengths(lens)
        if kind == "decode":
            blk.step(x, st, out=y)
        else:
            blk.forward(x, st, out=y)

    blk.set_timing(True)
    call()
    torch.cuda.synchronize()
    times = blk.kernel_times()
    blk.set_timing(False)
    seq = list(times)
    if any(c != 1 for _, c in times.values()):
        raise SystemExit(f"a launch name repeats within one call: {times}")
    if args.seq_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.seq_out)), exist_ok=True)
        with open(args.seq_out, "w") as f:
            json.dump({"leg": args.counters, "workload": workload, "sequence": seq}, f)
    for _ in range(args.warmup):
        call()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[counters] {args.counters}: {1 + args.warmup + args.steps} calls of {seq}, then a 1 GiB copy")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs", default="c2,c3,bwd,c2r,c4,c5p,c5d",
                    help="comma list of legs: c2 (headline, always run), c3, bwd, c2r, c4, c5p, c5d")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variant", choices=list(VARIANTS), default="plain",
                    help="block options on the 8B shapes (default: the plain Llama-shaped block)")
    ap.add_argument("--counters", choices=list(LEGS), help="one leg, eager launches only (under rocprofv3 --pmc)")
    ap.add_argument("--seq-out", help="with --counters: where to write the block's launch order")
    ap.add_argument("--ingest-counters", nargs="+", metavar="ARG",
                    help="LEG NAME DIR [DIR ...]: rocprofv3 --pmc runs -> profiles/NAME.json and .md (no GPU)")
    args = ap.parse_args()
    if args.ingest_counters:
        if len(args.ingest_counters) < 3:
            ap.error("--ingest-counters LEG NAME DIR [DIR ...]")
        ingest_counters(args.ingest_counters[0], args.ingest_counters[1], args.ingest_counters[2:])
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
    if args.counters:
        run_counters(args, torch)
        return
    legs = [s.strip() for s in args.legs.split(",") if s.strip()]
    flusher = Flusher(torch)
    pre = leg_prefill(args, torch, "c2", flusher, args.variant)
    kf = pre["kf"]
    mlp_in = "gemm_gate_up" if mlp_matrices(pre["cfg"]) == 3 else "gemm_up"
    gu_us = pre["breakdown"][mlp_in]["avg_us"]
    achieved = kf[mlp_in] / (gu_us * 1e-6) / 1e12
    d, IT, T = pre["cfg"]["d_model"], pre["cfg"]["intermediate"], pre["B"] * pre["L"]
    gated = mlp_in == "gemm_gate_up"
    roofline = {"bound": "mfma", "kernel": mlp_in, "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": stored_traffic(LEGS["c2"][0], mlp_in, "prefill") if args.variant == "plain" else None,
                "algorithmic_bytes": 2 * (T * d + (2 if gated else 1) * IT * d + T * IT),
                "flops_per_launch": kf[mlp_in], "avg_us": gu_us}
    out = {
        "metric": METRIC,
        "value": round(pre["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms"], 4),
        "ms_per_step_flushed": round(pre["ms_flushed"], 4),
        "ms_per_step_eager": round(pre["ms_eager"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3-8b-shaped block prefill into a fresh state (d=4096, 32/8 heads, hd=128, "
                               "IT=14336)",
                   "batch": pre["B"], "seq_len": pre["L"], "parallelism": "none",
                   **({"variant": args.variant} if args.variant != "plain" else {})},
        "prefill_mfma": {k: pre["summary"][k] for k in ("tflops", "frac_of_peak", "algorithmic_tflop")},
        "prefill_attention": pre["summary"]["attention"],
        "roofline": roofline,
        "cpu_baseline": None,
    }
    dec = None
    if "c3" in legs:
        dec = leg_decode(args, torch, "c3", flusher, args.variant, keep_fill=not args.no_cpu_baseline)
        att_us = dec["breakdown"]["attn_decode"]["avg_us"]
        kvb = dec["kb"]["attn_decode"]
        ach = kvb / (att_us * 1e-6) / 1e9
        dec["summary"]["roofline"] = {
            "bound": "hbm", "kernel": "attn_decode", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
            "traffic": stored_traffic(LEGS["c3"][0], "attn_decode", "decode") if args.variant == "plain" else None,
            "bytes_per_launch": kvb, "avg_us": att_us}
        dec["summary"]["per_kernel"] = dec["breakdown"]
        out["decode"] = dec["summary"]
    if "bwd" in legs and args.variant == "plain":
        out["backward"] = leg_backward(args, torch, pre["wl"])
    if "c2r" in legs and args.variant == "plain":
        out["ragged_prefill"] = leg_ragged(args, torch, steps=min(args.steps, 10))
    for leg in ("c4", "c5p"):
        if leg in legs:
            r = leg_prefill(args, torch, leg, flusher, steps=min(args.steps, 10))
            r["summary"]["per_kernel"] = r["breakdown"]
            out[LEGS[leg][0]] = r["summary"]
    if "c5d" in legs:
        r = leg_decode(args, torch, "c5d", flusher, steps=args.steps)
        r["summary"]["per_kernel"] = r["breakdown"]
        out[LEGS["c5d"][0]] = r["summary"]
    del flusher
    torch.cuda.empty_cache()
    out["copy_ceiling"] = copy_ceiling(torch)
    log(f"[copy] {out['copy_ceiling']}")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_prefill(pre["wl"])
        log(f"[cpu] prefill {out['cpu_baseline']}")
        if dec is not None and "k_fill" in dec["wl"]:
            out["decode"]["cpu_baseline"] = cpu_decode(dec["wl"])
            log(f"[cpu] decode {out['decode']['cpu_baseline']}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
