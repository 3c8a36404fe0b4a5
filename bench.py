"""Benchmark of the ViT encoder forward pass on one MI355X.

One step = vit_forward + vit_descriptor over one batch (patch embedding, every
encoder block, final LayerNorm, L2-normalised CLS descriptor), inputs already in
HBM.  Prints ONE JSON line: images/s on ViT-S/16 @336 batch 32 (the headline
workload), its fraction of the bf16 MFMA peak, the same for ViT-L/16 @1024
batch 1, the roofline of the dominant kernel (timed with HIP events on the
launch stream), and the CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--no-cpu] [--no-large]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
PEAK_INT8_TOPS = 5000.0    # MI355X dense int8 MFMA (TOP/s)
PEAK_HBM_GBS = 8000.0
METRIC = "images/s and % of bf16 MFMA peak, ViT-S/16@336 b32 and ViT-L/16@1024 b1"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flops_per_image(cfg: dict) -> dict:
    """Algorithmic FLOPs (2 per multiply-add) of one image, by operation."""
    p, D, Hm = cfg["patch"], cfg["dim"], cfg["mlp_hidden"]
    gh, gw = cfg["img_h"] // p, cfg["img_w"] // p
    P = gh * gw
    N = P + 1 + cfg["registers"]
    L = cfg["depth"] + cfg.get("extra_blocks", 0)
    f = {
        "patch_embed": 2 * P * 3 * p * p * D,
        "qkv": L * 2 * N * D * 3 * D,
        "attention": L * 4 * N * N * D,
        "out_proj": L * 2 * N * D * D,
        "fc1": L * 2 * N * D * Hm,
        "fc2": L * 2 * N * Hm * D,
    }
    f["total"] = sum(f.values())
    return f


def time_gpu(fn, steps, warmup):
    """`warmup` untimed calls, then exactly `steps` calls between a device
    synchronisation on either side, each bracketed by its own pair of HIP events
    on the current stream (the stream the library launches on).  Returns the
    per-call times in ms (median, p10, p90, mean) and the host wall time per
    call."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    return dict(median=float(np.median(ms)), p10=float(np.percentile(ms, 10)), p90=float(np.percentile(ms, 90)),
                mean=float(ms.mean()), wall=wall)


def time_loop(fn, steps, warmup):
    """Average duration in ms of one call among `steps` back-to-back calls, from
    one pair of HIP events around them on the current stream.  Used for single
    kernels of a few microseconds, whose launches run back to back the way they
    do inside a forward: an event pair around every launch would add its own
    gaps (2-6 us per launch measured) to each one."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def bench_workload(name, batch, steps, warmup):
    import torch
    import synth
    import vision_transformer_encoder_block_amd as vit
    cfg = synth.preset(name)
    P = synth.make_params(cfg)
    enc = vit.Encoder(cfg, P, max_batch=batch)
    x = torch.from_numpy(synth.make_images(cfg, batch)).cuda()
    tok = torch.empty((batch, enc.tokens, cfg["dim"]), dtype=torch.float32, device="cuda")
    desc = torch.empty((batch, cfg["dim"]), dtype=torch.float32, device="cuda")

    def step():
        enc.forward(x, tokens_out=tok)
        enc.descriptor(tok, desc_out=desc)

    # eager: one launch per kernel from Python
    eager = time_gpu(step, steps, warmup)
    # the same step recorded once as a HIP graph and replayed (the serving path)
    graph = vit.EncoderGraph(enc, x, tok, desc_out=desc)
    t = time_gpu(graph.replay, steps, warmup)
    torch.cuda.synchronize()
    assert torch.isfinite(desc).all().item(), "non-finite descriptor"
    fl = flops_per_image(cfg)
    ms = t["median"]
    tflops = fl["total"] * batch / (ms * 1e-3) / 1e12
    res = dict(images_per_s=batch / (ms * 1e-3), ms_per_step=ms, ms_per_step_p10=t["p10"], ms_per_step_p90=t["p90"],
               ms_per_step_mean=t["mean"], wall_ms_per_step=t["wall"], tflops=tflops,
               frac_bf16_peak=tflops / PEAK_BF16_TFLOPS, gflop_per_image=fl["total"] / 1e9,
               eager_images_per_s=batch / (eager["median"] * 1e-3), eager_ms_per_step=eager["median"])
    del graph
    return cfg, enc, res


def bench_preprocess(batch=32, src=(720, 1280), dst=(336, 336), steps=50, warmup=10):
    """Frame preprocessing (8-bit BGR HWC -> normalised CHW) at the live-camera
    frame size of the model card into the ViT-S/16 @336 input, HBM-bound:
    algorithmic bytes = frames read once + fp32 images written."""
    import torch
    import vision_transformer_encoder_block_amd as vit
    g = torch.Generator(device="cuda").manual_seed(5000)
    frames = torch.randint(0, 256, (batch,) + src + (3,), dtype=torch.uint8, device="cuda", generator=g)
    out = torch.empty((batch, 3) + dst, dtype=torch.float32, device="cuda")
    ms = time_loop(lambda: vit.vit_op_preprocess(frames, batch, src[0], src[1], True, out, dst[0], dst[1]),
                   steps, warmup)
    nbytes = batch * (src[0] * src[1] * 3 + 3 * dst[0] * dst[1] * 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"{batch} BGR frames {src[1]}x{src[0]} -> {dst[1]}x{dst[0]} ImageNet-normalised",
            "frames_per_s": batch / (ms * 1e-3), "us_per_batch": ms * 1e3, "bytes_per_batch": nbytes,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS}}


def kernel_breakdown(cfg, batch, steps=20, warmup=5):
    """Average duration of each block kernel at the workload's shapes (HIP events
    on the launch stream), through the per-op C ABI entry points."""
    import torch
    import vision_transformer_encoder_block_amd as vit
    D, Hm, H = cfg["dim"], cfg["mlp_hidden"], cfg["heads"]
    p = cfg["patch"]
    N = (cfg["img_h"] // p) * (cfg["img_w"] // p) + 1 + cfg["registers"]
    M = batch * N
    L = cfg["depth"] + cfg.get("extra_blocks", 0)
    nv = (N + 63) // 64 * 64
    g = torch.Generator(device="cuda").manual_seed(7)
    bf = torch.bfloat16

    def rnd(*shape, dtype=bf, scale=0.05):
        return (torch.randn(*shape, generator=g, device="cuda") * scale).to(dtype)

    x = rnd(M, D, dtype=torch.float32, scale=1.0)
    gam, bet = torch.ones(D, device="cuda"), torch.zeros(D, device="cuda")
    h = rnd(M, D, scale=1.0)
    wqkv, bqkv = rnd(3 * D, D), rnd(3 * D, dtype=torch.float32)
    q = torch.empty((batch, H, N, 64), dtype=bf, device="cuda")
    k = torch.empty_like(q)
    vt = torch.zeros((batch, H, 64, nv), dtype=bf, device="cuda")
    o = torch.empty((M, D), dtype=bf, device="cuda")
    wo, bo, ls = rnd(D, D), rnd(D, dtype=torch.float32), torch.full((D,), 1e-5, device="cuda")
    w1, b1 = rnd(Hm, D), rnd(Hm, dtype=torch.float32)
    w2, b2 = rnd(D, Hm), rnd(D, dtype=torch.float32)
    f = torch.empty((M, Hm), dtype=bf, device="cuda")
    vit.vit_op_qkv(h, wqkv, bqkv, batch, N, H, q, k, vt)
    # D = 384: the residual GEMMs also apply the LayerNorm after them (as the
    # forward does), leaving the first block's LN1 and the final norm standalone
    fused = D == 384
    ops = {
        "layernorm": (lambda: vit.vit_op_layernorm(x, M, D, gam, bet, 1e-6, h, 0), 2 if fused else 2 * L, 0.0,
                      M * D * (4 + 2) + 8 * D, "hbm"),
        "qkv": (lambda: vit.vit_op_qkv(h, wqkv, bqkv, batch, N, H, q, k, vt), L, 2.0 * M * D * 3 * D,
                M * D * 2 + 3 * D * D * 2 + 3 * M * D * 2, "mfma"),
        "attention": (lambda: vit.vit_op_attention(q, k, vt, batch, N, H, o), L, 4.0 * batch * N * N * D,
                      4 * M * D * 2, "mfma"),
        "out_proj": ((lambda: vit.vit_op_linear_residual_ln(o, wo, bo, ls, M, D, D, x, gam, bet, 1e-6, h)) if fused
                     else (lambda: vit.vit_op_linear(o, wo, bo, M, D, D, vit.EPI_RESIDUAL, ls, x)), L,
                     2.0 * M * D * D, M * D * 2 + D * D * 2 + 2 * M * D * 4 + (M * D * 2 if fused else 0), "mfma"),
        "fc1": (lambda: vit.vit_op_linear(h, w1, b1, M, Hm, D, vit.EPI_GELU_BF16, None, f), L,
                2.0 * M * D * Hm, M * D * 2 + Hm * D * 2 + M * Hm * 2, "mfma"),
        "fc2": ((lambda: vit.vit_op_linear_residual_ln(f, w2, b2, ls, M, D, Hm, x, gam, bet, 1e-6, h)) if fused
                else (lambda: vit.vit_op_linear(f, w2, b2, M, D, Hm, vit.EPI_RESIDUAL, ls, x)), L,
                2.0 * M * Hm * D, M * Hm * 2 + D * Hm * 2 + 2 * M * D * 4 + (M * D * 2 if fused else 0), "mfma"),
    }
    out = {}
    for name, (fn, per_step, flops, nbytes, bound) in ops.items():
        ms = time_loop(fn, steps, warmup)
        out[name] = dict(ms=ms, launches_per_step=per_step, ms_per_step=ms * per_step, flops=flops,
                         bytes=nbytes, bound=bound, tflops=flops / (ms * 1e-3) / 1e12,
                         gbs=nbytes / (ms * 1e-3) / 1e9)
    return out


def breakdown_table(bd):
    """Per-op summary for the JSON line: time per launch and per step, TFLOP/s
    and algorithmic HBM GB/s (bytes the op must move at least, per launch)."""
    return {n: {"us_per_launch": round(b["ms"] * 1e3, 2), "launches_per_step": b["launches_per_step"],
                "ms_per_step": round(b["ms_per_step"], 4), "tflops": round(b["tflops"], 1),
                "hbm_gbs": round(b["gbs"], 1)} for n, b in bd.items()}


def roofline(breakdown, kernel_names, workload):
    name = max(breakdown, key=lambda n: breakdown[n]["ms_per_step"])
    b = breakdown[name]
    if b["bound"] == "mfma":
        achieved = b["flops"] / (b["ms"] * 1e-3) / 1e12
        rl = dict(bound="mfma", achieved=achieved, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                  frac=achieved / PEAK_BF16_TFLOPS)
    else:
        achieved = b["bytes"] / (b["ms"] * 1e-3) / 1e9
        rl = dict(bound="hbm", achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s", frac=achieved / PEAK_HBM_GBS)
    rl["kernel"] = kernel_names.get(name, name)
    rl["avg_launch_us"] = b["ms"] * 1e3
    rl["traffic"] = traffic_for(workload, name)
    return name, rl


def _strip_comments(text: str) -> str:
    """Source text without // and /* */ comments or blank lines (a comment edit
    does not change a kernel, so it must not invalidate counter data)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def _source_digest():
    """Digest of the device-code sources (comments stripped) and the build flags."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "vision_transformer_encoder_block_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        if fn.endswith((".hip", ".h")):
            h.update(_strip_comments(open(os.path.join(csrc, fn)).read()).encode())
    # compile flags change the kernels too
    h.update(open(os.path.join(ROOT, "vision_transformer_encoder_block_amd", "build.py"), "rb").read())
    return h.hexdigest()[:16]


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def traffic_for(workload, op):
    """HBM bytes per launch of `op` at `workload` from the committed rocprofv3
    counter summary, if it was taken on the current kernel sources (else null)."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    try:
        t = json.load(open(TRAFFIC_JSON))
    except ValueError:
        return None
    w = t.get("workloads", {}).get(workload)
    if w is None or w.get("source_digest") != _source_digest():
        return None
    entry = w.get("ops", {}).get(op)
    return None if entry is None else entry.get("bytes_per_launch")


def _cpu_threads():
    """Threads NumPy's BLAS actually uses (the oracle's matrix products)."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_baseline(budget_s=15.0, max_images=128):
    """The oracle (float64 NumPy), untuned, on ViT-S/16 @336 images until the budget is spent."""
    import synth
    from oracle import vit_oracle as O
    cores = _cpu_threads()
    cfg = synth.preset("vits16_336")
    P = synth.make_params(cfg)
    x = synth.make_images(cfg, max_images)
    done, t0 = 0, time.perf_counter()
    chunk = 2
    while done < max_images and (time.perf_counter() - t0) < budget_s:
        O.forward(x[done:done + chunk], P, cfg)
        done += chunk
    dt = time.perf_counter() - t0
    return dict(value=done / dt, unit="images/s", cores=cores, kind="oracle",
                sample=f"{done} ViT-S/16@336 images (float64 NumPy oracle, batches of {chunk}), {dt:.1f} s")


def copy_calibration(mib=256, reps=3):
    """A plain device copy of known size, so HBM counters can be scaled."""
    import torch
    src = torch.ones(mib * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return mib


# Per workload: op -> predicate on the kernel name selecting its dispatches in a
# counter run of that workload's per-op loops (bench.py --breakdown-only).
# Residual GEMMs that share one kernel (out-proj and fc2) are told apart by
# FETCH_SIZE: fc2 reads an A operand 4x longer.
def _has(*subs, without=()):
    return lambda k: all(x in k for x in subs) and not any(x in k for x in without)


PMC_OPS = {
    "vits16_336_b32": {"fc1": _has("EpiGeluBf16"), "attention": _has("attention_kernel"),
                       "layernorm": _has("layernorm_kernel"), "qkv": _has("EpiQKV"),
                       "out_proj|fc2": _has("EpiResidualLN")},
    "vitl16_1024_b1": {"fc1": _has("EpiGeluBf16"), "attention": _has("attention_kernel"),
                       "layernorm": _has("layernorm_kernel"), "qkv": _has("EpiQKV"),
                       "out_proj|fc2": _has("EpiResidual", without=("EpiResidualLN",))},
    # counter run of `bench.py --head-only --copy-calibration`: the Bottleneck
    # 3x3 ConvX launches, six per head forward and the ones timed alone
    "semantic_head_b8": {"convx": _has("EpiChanLN<128>", "AMapConv3")},
}

WORKLOADS = {"vits16_336_b32": ("vits16_336", 32), "vitl16_1024_b1": ("vitl16_1024", 1)}


def summarize_pmc(fetch_csv, write_csv, workload, copy_mib=256):
    """Per-dispatch HBM bytes of one workload's block kernels from two rocprofv3
    --pmc runs (FETCH_SIZE, WRITE_SIZE in KiB) of `bench.py --breakdown-only
    WORKLOAD --copy-calibration`, scaled by the same counters on a plain copy of
    known size; stored under the workload in profiles/hbm_traffic.json with the
    kernel source digest."""
    import csv

    def load(path, counter):
        rows = {}
        for r in csv.DictReader(open(path)):
            if r.get("Counter_Name") != counter:
                continue
            rows.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return rows

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")

    def vals(table, pred):
        return [v for k, vs in table.items() if pred(k) for v in vs]

    def avg(xs):
        return sum(xs) / len(xs) if xs else None

    def copy_avg(table):
        xs = sorted(vals(table, lambda k: "copy" in k.lower() or "elementwise" in k.lower()))[-3:]
        return avg(xs)  # the three large calibration copies

    expect_kib = copy_mib * 1024.0
    cf, cw = copy_avg(fetch), copy_avg(write)
    if not cf or not cw:
        raise SystemExit("no calibration copy in the counter runs (run with --copy-calibration)")
    scale_f, scale_w = expect_kib / cf, expect_kib / cw
    ops = {}
    for op, pred in PMC_OPS[workload].items():
        f, w = vals(fetch, pred), vals(write, pred)
        if not f or not w:
            continue
        if op == "out_proj|fc2":
            mid = (min(f) + max(f)) / 2
            groups = (("out_proj", [v for v in f if v < mid]), ("fc2", [v for v in f if v >= mid]))
            kname = "FETCH cluster"
        else:
            groups = ((op, f),)
            kname = None
        for name, grp in groups:
            if not grp:
                continue
            fk, wk = avg(grp), avg(w)
            ops[name] = {"dispatches": len(grp), "fetch_kib": fk, "write_kib": wk,
                         "bytes_per_launch": (fk * scale_f + wk * scale_w) * 1024.0}
            if kname:
                ops[name]["note"] = kname
    doc = json.load(open(TRAFFIC_JSON)) if os.path.exists(TRAFFIC_JSON) else {}
    doc = {"workloads": doc.get("workloads", {})}
    doc["workloads"][workload] = {"source_digest": _source_digest(), "copy_mib": copy_mib, "copy_fetch_kib": cf,
                                  "copy_write_kib": cw, "scale_fetch": scale_f, "scale_write": scale_w, "ops": ops}
    json.dump(doc, open(TRAFFIC_JSON, "w"), indent=1)
    print(json.dumps(doc["workloads"][workload], indent=1))


def summarize_mfma(csv_path, workload, simds=1024, clock_ghz=2.4):
    """Matrix-core utilisation of one workload's block kernels from one
    rocprofv3 --pmc run (SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16,
    SQ_INSTS_MFMA, SQ_INSTS_VALU_TRANS_F32) of `bench.py --breakdown-only
    WORKLOAD`.  Kernels shared by two ops (out-proj and fc2) are told apart by
    their hardware FLOP count (MOPS x 512), taking the dispatch cluster nearest
    each op's algorithmic FLOPs.  A busy cycle is one SIMD's full-rate MFMA
    cycle (1024 bf16 FLOPs), so utilisation = busy SIMD-cycles / (SIMDs x
    dispatch duration x clock), the duration from the dispatch's own
    timestamps and the clock the one the dense peak is quoted at.  Prints a
    markdown table."""
    import csv
    import math
    import synth
    per = {}
    for r in csv.DictReader(open(csv_path)):
        c = per.setdefault((r["Kernel_Name"], r["Dispatch_Id"]), {})
        c["dur_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    name, B = WORKLOADS[workload]
    cfg = synth.preset(name)
    D, Hm = cfg["dim"], cfg["mlp_hidden"]
    N = synth.tokens(cfg)
    M = B * N
    pm = PMC_OPS[workload]
    ops = [("qkv", pm["qkv"], 2.0 * M * D * 3 * D), ("attention", pm["attention"], 4.0 * B * N * N * D),
           ("out_proj", pm["out_proj|fc2"], 2.0 * M * D * D), ("fc1", pm["fc1"], 2.0 * M * D * Hm),
           ("fc2", pm["out_proj|fc2"], 2.0 * M * Hm * D)]
    print("| Op | dispatches | dispatch us | hardware GFLOP (MOPS x 512) | algorithmic GFLOP | MFMA instr. | "
          "MFMA busy % | transcendental instr. |")
    print("|---|---|---|---|---|---|---|---|")
    for op, pred, fl in ops:
        groups = {}
        for (kname, _), c in per.items():
            if pred(kname) and "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:
                groups.setdefault(round(c["SQ_INSTS_VALU_MFMA_MOPS_BF16"]), []).append(c)
        if not groups:
            continue
        mops = min(groups, key=lambda m: abs(math.log(max(m, 1) * 512.0 / fl)))
        sel = groups[mops]
        av = {k: sum(c.get(k, 0.0) for c in sel) / len(sel) for k in sel[0]}
        util = av["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * av["dur_us"] * clock_ghz * 1e3)
        print(f"| {op} | {len(sel)} | {av['dur_us']:.1f} | {mops * 512 / 1e9:.2f} | {fl / 1e9:.2f} | "
              f"{av.get('SQ_INSTS_MFMA', 0):.0f} | {100 * util:.1f} | {av.get('SQ_INSTS_VALU_TRANS_F32', 0):.0f} |")


KERNEL_NAMES = {
    "vits16_336_b32": {
        "qkv": "gemm_bf16_kernel<EpiQKV>",
        "attention": "attention_kernel",
        "out_proj": "gemm_bf16_kernel<EpiResidualLN> (out-proj + LN2)",
        "fc1": "gemm_bf16_kernel<EpiGeluBf16>",
        "fc2": "gemm_bf16_kernel<EpiResidualLN> (fc2 + next LN1)",
        "layernorm": "layernorm_kernel (block 1 LN1, final norm)",
    },
    "vitl16_1024_b1": {
        "qkv": "gemm_bf16_kernel<EpiQKV>",
        "attention": "attention_kernel",
        "out_proj": "gemm_bf16_kernel<EpiResidual> (out-proj)",
        "fc1": "gemm_bf16_kernel<EpiGeluBf16>",
        "fc2": "gemm_bf16_kernel<EpiResidual> (fc2)",
        "layernorm": "layernorm_kernel (LN1, LN2)",
    },
}


def head_flops(hcfg, batch: int) -> float:
    """Algorithmic FLOP of the semantic head (2 per multiply-add over its convs)."""
    M = batch * hcfg.grid_h * hcfg.grid_w
    W, H2, T, C = hcfg.width, hcfg.width // 2, hcfg.taps * hcfg.dim, hcfg.classes
    macs = T * W + 6 * 9 * H2 * H2 + 5 * H2 * W + W * W + 9 * W * W + W * C
    return 2.0 * M * macs


def bench_head(steps=30, warmup=5):
    """DINOv2-S/14 @518 batch 8: the encoder with its four taps, then the LibreYOLO
    DINOv2 semantic head (projector P4 + task head, logits resized to 518 x 518)."""
    import torch
    import synth
    import vision_transformer_encoder_block_amd as vit
    cfg = synth.preset("vits14_518")
    B = 8
    enc = vit.Encoder(cfg, synth.make_params(cfg), max_batch=B)
    hcfg = vit.head_config_preset()
    head = vit.SemanticHead(hcfg, synth.make_head_params(cfg))
    x = torch.from_numpy(synth.make_images(cfg, B)).cuda()
    tok = torch.empty((B, enc.tokens, cfg["dim"]), dtype=torch.float32, device="cuda")
    taps = torch.empty((B, 4, cfg["dim"], 37, 37), dtype=torch.float32, device="cuda")
    logits = torch.empty((B, hcfg.classes, hcfg.out_h, hcfg.out_w), dtype=torch.float32, device="cuda")

    def both():
        enc.forward(x, with_taps=True, tokens_out=tok, taps_out=taps)
        head.forward(taps, logits_out=logits)

    ms_all = time_gpu(both, steps, warmup)["median"]
    ms_head = time_loop(lambda: head.forward(taps, logits_out=logits), steps, warmup)
    torch.cuda.synchronize()
    assert torch.isfinite(logits).all().item(), "non-finite logits"
    fl = head_flops(hcfg, B)
    tf = fl / (ms_head * 1e-3) / 1e12
    head.close()
    enc.close()
    # the head's dominant kernel: a Bottleneck ConvX (3x3 conv as an implicit
    # GEMM, channel LayerNorm and SiLU in its epilogue; six per forward), alone
    M, H2 = B * 37 * 37, hcfg.width // 2
    xin = torch.randn(M, 5 * H2, device="cuda").to(torch.bfloat16)
    wk = (torch.randn(H2, 9 * H2, device="cuda") * 0.05).to(torch.bfloat16)
    lg, lb = torch.ones(H2, device="cuda"), torch.zeros(H2, device="cuda")
    cout = torch.empty(M, 5 * H2, dtype=torch.bfloat16, device="cuda")
    ms_conv = time_loop(lambda: vit.vit_op_convx(xin, 5 * H2, H2, H2, B, 37, 37, 3, wk, H2, lg, lb, None, None, 1e-6,
                                                 cout, 5 * H2, 2 * H2), steps, warmup)
    conv_tf = 2.0 * M * H2 * 9 * H2 / (ms_conv * 1e-3) / 1e12
    return {"workload": "DINOv2-S/14 @518 b8, taps 3/6/9/12 -> semantic head -> 19 x 518 x 518 logits",
            "images_per_s": B / (ms_all * 1e-3), "ms_per_step": ms_all, "head_ms": ms_head,
            "head_gflop": fl / 1e9, "head_tflops": tf, "head_pct_bf16_peak": 100 * tf / PEAK_BF16_TFLOPS,
            "roofline": {"bound": "mfma", "kernel": "gemm_bf16_kernel<32, 128, ..., EpiChanLN<128>, AMapConv3> "
                         "(Bottleneck ConvX: 3x3 conv + channel LN + SiLU, M = 10952, N = 128, K = 1152)",
                         "achieved": conv_tf,
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": conv_tf / PEAK_BF16_TFLOPS,
                         "avg_launch_us": ms_conv * 1e3, "traffic": traffic_for("semantic_head_b8", "convx")}}


def bench_fp8(steps=30, warmup=5):
    """The fp8 (E4M3) and int8 linear layers against the bf16 one on the same
    shapes: the encoder's fc1 / fc2 (ViT-S/16 @336 b32, ViT-L/16 @1024 b1) and
    a square 8192^3 product; TFLOP/s against the fp8 dense peak (5.0 PF) and
    TOP/s against the int8 dense peak (5.0 POP/s)."""
    import torch
    import vision_transformer_encoder_block_amd as vit
    g = torch.Generator(device="cuda").manual_seed(8)
    res = {}
    for name, M, N, K in [("vits_fc1", 14272, 1536, 384), ("vits_fc2", 14272, 384, 1536),
                          ("vitl_fc1", 4101, 4096, 1024), ("square_8192", 8192, 8192, 8192)]:
        qa = torch.randint(0, 0x7F, (M, K), dtype=torch.uint8, device="cuda", generator=g)
        qw = torch.randint(0, 0x7F, (N, K), dtype=torch.uint8, device="cuda", generator=g)
        bias = torch.zeros(N, device="cuda")
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ms8 = time_loop(lambda: vit.vit_op_linear_fp8(qa, qw, M, N, K, 1.0, bias, out), steps, warmup)
        ia = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
        iw = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
        msi = time_loop(lambda: vit.vit_op_linear_int8(ia, iw, M, N, K, 1.0 / 16384, bias, out), steps, warmup)
        a = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        w = torch.randn(N, K, device="cuda", generator=g).to(torch.bfloat16)
        ms16 = time_loop(lambda: vit.vit_op_linear(a, w, bias, M, N, K, vit.EPI_BIAS_BF16, None, out), steps,
                         warmup)
        fl = 2.0 * M * N * K
        res[name] = {"shape": [M, N, K], "fp8_us": ms8 * 1e3, "fp8_tflops": fl / (ms8 * 1e-3) / 1e12,
                     "fp8_frac_peak": fl / (ms8 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
                     "int8_us": msi * 1e3, "int8_tops": fl / (msi * 1e-3) / 1e12,
                     "int8_frac_peak": fl / (msi * 1e-3) / 1e12 / PEAK_INT8_TOPS,
                     "bf16_us": ms16 * 1e3, "bf16_tflops": fl / (ms16 * 1e-3) / 1e12, "speedup": ms16 / ms8}
        del qa, qw, ia, iw, a, w, out
    return res


def gemm_vs_library(steps=30, warmup=5):
    """The library's GEMM (bias epilogue, bf16 out) against hipBLASLt, reached
    through torch.nn.functional.linear in bf16 with the same bias, on the
    encoder's Linear shapes (ViT-L/16 @1024 b1, ViT-S/16 @336 b32); the same
    process and inputs, back-to-back launches timed as a loop average."""
    import torch
    import vision_transformer_encoder_block_amd as vit
    g = torch.Generator(device="cuda").manual_seed(11)
    shapes = [("ViT-L b1 qkv", 4101, 3072, 1024), ("ViT-L b1 out-proj", 4101, 1024, 1024),
              ("ViT-L b1 fc1", 4101, 4096, 1024), ("ViT-L b1 fc2", 4101, 1024, 4096),
              ("ViT-S b32 qkv", 14272, 1152, 384), ("ViT-S b32 out-proj", 14272, 384, 384),
              ("ViT-S b32 fc1", 14272, 1536, 384), ("ViT-S b32 fc2", 14272, 384, 1536)]
    rows = []
    for name, M, N, K in shapes:
        a = (torch.randn(M, K, generator=g, device="cuda") * 0.5).to(torch.bfloat16)
        w = (torch.randn(N, K, generator=g, device="cuda") * 0.05).to(torch.bfloat16)
        bias = torch.randn(N, generator=g, device="cuda") * 0.1
        bias16 = bias.to(torch.bfloat16)
        out = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        ours = time_loop(lambda: vit.vit_op_linear(a, w, bias, M, N, K, vit.EPI_BIAS_BF16, None, out), steps, warmup)
        lib = time_loop(lambda: torch.nn.functional.linear(a, w, bias16), steps, warmup)
        fl = 2.0 * M * N * K
        rows.append({"op": name, "shape": [M, N, K], "ours_us": round(ours * 1e3, 2), "hipblaslt_us": round(lib * 1e3, 2),
                     "ours_tflops": round(fl / (ours * 1e-3) / 1e12, 1),
                     "hipblaslt_tflops": round(fl / (lib * 1e-3) / 1e12, 1)})
        log(json.dumps(rows[-1]))
        del a, w, out
    return rows


def head_cpu_baseline(images=8):
    """The head's oracle (float64 NumPy), untuned, on DINOv2-S/14 @518 stand-in taps."""
    import synth
    from oracle import head_oracle as H
    cfg = synth.preset("vits14_518")
    Ph = synth.make_head_params(cfg)
    taps = synth.make_taps(cfg, images)
    t0 = time.perf_counter()
    for b in range(images):
        H.semantic_head(taps[b], Ph, 518, 518)
    dt = time.perf_counter() - t0
    return {"value": images / dt, "unit": "images/s", "cores": _cpu_threads(), "kind": "oracle",
            "sample": f"{images} images of 4 x 384 x 37 x 37 taps through the float64 head oracle, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-large", action="store_true", help="skip the ViT-L/16 @1024 b1 line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device copy (for scaling HBM counters)")
    ap.add_argument("--head-only", action="store_true",
                    help="run only the semantic-head leg (DINOv2-S/14 @518 b8 + head) and print its JSON")
    ap.add_argument("--fp8-only", action="store_true", help="run only the fp8 linear leg and print its JSON")
    ap.add_argument("--gemm-vs-library", action="store_true",
                    help="run only the comparison of the library's GEMM with hipBLASLt (through torch) and print it")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "WORKLOAD"),
                    help="host only: turn two rocprofv3 --pmc CSVs of --breakdown-only WORKLOAD (or of "
                         "--head-only for semantic_head_b8) into profiles/hbm_traffic.json")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("CSV", "WORKLOAD"),
                    help="host only: matrix-core utilisation table from a rocprofv3 --pmc CSV of "
                         "--breakdown-only WORKLOAD")
    ap.add_argument("--forward-only", choices=sorted(WORKLOADS),
                    help="run only the whole-forward timing of one workload (eager, then graph replays) and print "
                         "its JSON (for kernel traces of the forward as it runs in the graph)")
    ap.add_argument("--breakdown-only", choices=sorted(WORKLOADS),
                    help="run only the per-op timing loops of one workload and print their JSON (for counter runs)")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the encoder path is single-GPU (images are independent, "
              "so several GPUs would each run their own batch); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"

    if args.copy_calibration:
        copy_calibration()
    if args.head_only:
        print(json.dumps(bench_head(args.steps, args.warmup)), flush=True)
        return
    if args.fp8_only:
        print(json.dumps(bench_fp8(args.steps, args.warmup)), flush=True)
        return
    if args.gemm_vs_library:
        print(json.dumps(gemm_vs_library(args.steps, args.warmup)), flush=True)
        return
    if args.forward_only:
        name, batch = WORKLOADS[args.forward_only]
        _, enc, res = bench_workload(name, batch, args.steps, args.warmup)
        enc.close()
        print(json.dumps(res), flush=True)
        return
    if args.breakdown_only:
        name, batch = WORKLOADS[args.breakdown_only]
        import synth
        bd = kernel_breakdown(synth.preset(name), batch, args.steps, args.warmup)
        print(json.dumps(breakdown_table(bd)), flush=True)
        return
    log("ViT-S/16 @336 b32 ...")
    cfg, enc, small = bench_workload("vits16_336", 32, args.steps, args.warmup)
    enc.close()
    log(json.dumps(small))
    large = None
    if not args.no_large:
        log("ViT-L/16 @1024 b1 ...")
        cfg_l, enc_l, large = bench_workload("vitl16_1024", 1, args.steps, args.warmup)
        enc_l.close()
        log(json.dumps(large))
    log("frame preprocessing ...")
    pre = bench_preprocess()
    log(json.dumps(pre))
    log("semantic head ...")
    hd = bench_head()
    log(json.dumps(hd))
    log("fp8 linear ...")
    f8 = bench_fp8()
    log(json.dumps(f8))
    log("kernel breakdown ...")
    bd = kernel_breakdown(cfg, 32)
    for n, b in bd.items():
        log(f"  {n:10s} {b['ms'] * 1e3:9.1f} us/launch  x{b['launches_per_step']:3d} = {b['ms_per_step']:.3f} ms/step"
            f"  {b['tflops']:7.1f} TFLOP/s  {b['gbs']:7.1f} GB/s")
    dom, rl = roofline(bd, KERNEL_NAMES["vits16_336_b32"], "vits16_336_b32")
    bd_l = rl_l = None
    if large:
        log("kernel breakdown, ViT-L/16 @1024 b1 ...")
        bd_l = kernel_breakdown(cfg_l, 1)
        for n, b in bd_l.items():
            log(f"  {n:10s} {b['ms'] * 1e3:9.1f} us/launch  x{b['launches_per_step']:3d} = "
                f"{b['ms_per_step']:.3f} ms/step  {b['tflops']:7.1f} TFLOP/s  {b['gbs']:7.1f} GB/s")
        _, rl_l = roofline(bd_l, KERNEL_NAMES["vitl16_1024_b1"], "vitl16_1024_b1")
    out = {
        "metric": METRIC,
        "value": small["images_per_s"],
        "unit": "images/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": small["ms_per_step"],
        "ms_per_step_p10": small["ms_per_step_p10"],
        "ms_per_step_p90": small["ms_per_step_p90"],
        "ms_per_step_mean": small["ms_per_step_mean"],
        "timing": "median of per-step HIP event pairs (p10/p90 and mean beside it); images/s from the median",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) images, N(0,0.02) random-init weights)",
        "config": {"workload": "ViT-S/16@336 b32 (DINOv3-style, 446 tokens, 4 registers, attention sink)",
                   "global_batch": 32, "tokens": 446, "dim": 384, "depth": 12, "heads": 6,
                   "launch": "forward + descriptor replayed as one HIP graph"},
        "eager_images_per_s": small["eager_images_per_s"],
        "tflops": small["tflops"],
        "pct_bf16_peak": 100 * small["frac_bf16_peak"],
        "roofline": rl,
        "kernels": breakdown_table(bd),
    }
    if large:
        out["vitl16_1024_b1"] = {"images_per_s": large["images_per_s"], "ms_per_step": large["ms_per_step"],
                                 "ms_per_step_p10": large["ms_per_step_p10"],
                                 "ms_per_step_p90": large["ms_per_step_p90"],
                                 "ms_per_step_mean": large["ms_per_step_mean"],
                                 "eager_images_per_s": large["eager_images_per_s"],
                                 "tflops": large["tflops"], "pct_bf16_peak": 100 * large["frac_bf16_peak"],
                                 "roofline": rl_l, "kernels": breakdown_table(bd_l)}
    out["preprocess"] = pre
    if not args.no_cpu:
        hd["cpu_baseline"] = head_cpu_baseline()
    out["semantic_head"] = hd
    out["fp8_linear"] = f8
    if not args.no_cpu:
        log("CPU oracle baseline ...")
        out["cpu_baseline"] = cpu_baseline()
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
