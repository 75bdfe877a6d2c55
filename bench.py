"""Throughput of the MI355X encoder hot path (one GPU).

One step = one vit_encode_varlen call over the whole batch: patch embedding,
every block (RMSNorm, wqkv, rotary, attention, out-projection, RMSNorm, SwiGLU
gate/up, down) and the final norm, plus the aligner when the workload has one.
Inputs and weights are resident in HBM before the timed region.

Prints one JSON line (metric, value in patches/s, roofline of the dominant
kernel measured with HIP events inside the timed region, cpu_baseline of the
oracle on a bounded sample on the host cores).
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

METRIC = "patches/sec through ViT stack + aligner (bf16), % of MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "ragged_varlen_4img"

# kernel class -> sources of its kernels (for the counter-traffic freshness check)
_GEMM_SRC = ("common.h", "gemm_bf16.hip", "gemm_mfma.h", "gemm_mfma.hip")
KERNEL_SOURCE = {"qkv": _GEMM_SRC, "outproj": _GEMM_SRC, "gateup": _GEMM_SRC, "down": _GEMM_SRC,
                 "embed": _GEMM_SRC, "aligner": _GEMM_SRC, "attn": ("common.h", "attention.hip"),
                 "rmsnorm": ("common.h", "elementwise.hip"), "rope": ("common.h", "elementwise.hip"),
                 "gather": ("common.h", "elementwise.hip"), "merge": ("common.h", "merge.hip"),
                 "proj1": _GEMM_SRC, "attn72": ("common.h", "attention.hip")}


def class_flops(cfg):
    """Algorithmic FLOPs per launch of each MFMA-bound kernel class."""
    P, d, h = cfg.total_patches, cfg.vision_dim, cfg.mlp_hidden
    f = {"qkv": 6.0 * P * d * d, "outproj": 2.0 * P * d * d, "gateup": 4.0 * P * d * h,
         "down": 2.0 * P * d * h, "attn": sum(4.0 * d * p * p for p in cfg.seqlens),
         "embed": 2.0 * P * cfg.patch_dim * d}
    if cfg.aligner:
        f["aligner"] = 2.0 * P * d * cfg.llm_dim
    return f


def class_bytes(cfg):
    """Algorithmic HBM bytes per launch of the bandwidth-bound classes (bf16 activations).
    With head_dim 72 the rotary class is one pass that rotates q and k in place and
    writes V transposed: q, k read and written, V read, V^T written (each image's keys
    padded to a multiple of 64), the table read."""
    P, d, D, H = cfg.total_patches, cfg.vision_dim, cfg.head_dim, cfg.n_heads
    rope = 2 * (2 * P * H * D * 2) + P * (D // 2) * 8
    if D == 72 and cfg.dtype == "bf16":
        kv = sum((p + 63) // 64 * 64 for p in cfg.seqlens)
        rope += P * d * 2 + kv * d * 2
    return {"rmsnorm": P * d * 4 + P * d * 2 + d * 4,        # fp32 residual in, bf16 out, scale
            "rope": rope,
            "gather": 2 * P * d * 2}


def source_sha(kernel_class):
    h = hashlib.sha256()
    for f in KERNEL_SOURCE[kernel_class]:
        h.update(open(os.path.join(ROOT, "vision_transformer_encoder_image_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def counter_traffic(kernel_class, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_class}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != source_sha(kernel_class):
        return None  # the kernel changed since the counters were taken
    return rec.get("hbm_bytes_per_launch")


# kernel-name patterns of each class in rocprofv3 output (SwiGLU is the only
# dual-B GEMM instantiation, i.e. the template argument list ends in "true>")
KERNEL_NAME_PATTERN = {"gateup": ("gemm_", ", true>("), "attn": ("attn_vt_kernel", ""),
                       "attn72": ("attn_bf16_kernel<72", ""), "rope": ("tpack_kernel<72, true>", ""),
                       "rmsnorm": ("rmsnorm_", ""), "merge": ("merge_copy_kernel", ""),
                       "proj1": ("gemm_mfma_kernel", ", 5, false>(")}


def _pmc_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    return rows


def pmc_summary(fetch_dir, write_dir, kernel, workload, copy_mb, out_path=None):
    """HBM bytes per launch of `kernel` from FETCH_SIZE / WRITE_SIZE runs, each scaled
    by the bytes the same counter reports for a plain copy of known size."""
    import statistics

    pat, tail = KERNEL_NAME_PATTERN[kernel]
    out = {"kernel": kernel, "workload": workload, "source_sha256": source_sha(kernel)}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _pmc_rows(d) if r["Counter_Name"] == counter]
        # one call of a class may launch several kernels (a column-split GEMM: a
        # large-tile launch and a tail launch): per call, the sum over the distinct
        # matching kernels of each one's median
        by_name = {}
        for r in rows:
            if pat in r["Kernel_Name"] and tail in r["Kernel_Name"]:
                by_name.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        copy = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]
                or "copy_kernel" in r["Kernel_Name"] or "elementwise" in r["Kernel_Name"]]
        known_kib = copy_mb * 1024.0
        scale = known_kib / max(copy) if copy else 1.0
        kib = sum(statistics.median(v) for v in by_name.values()) if by_name else float("nan")
        out[counter.lower() + "_kib_raw"] = kib
        out[counter.lower() + "_copy_kib_raw"] = max(copy) if copy else None
        out[counter.lower() + "_scale"] = scale
        out[counter.lower() + "_bytes_per_launch"] = kib * scale * 1024.0
        out[counter.lower() + "_launches"] = sum(len(v) for v in by_name.values())
        out[counter.lower() + "_kernels_per_call"] = len(by_name)
    out["hbm_bytes_per_launch"] = out["fetch_size_bytes_per_launch"] + out["write_size_bytes_per_launch"]
    try:
        from vision_transformer_encoder_image_amd import configs
        alg = class_bytes(configs.get(workload)).get(kernel)
    except (KeyError, ValueError):
        alg = None
    if alg:
        out["algorithmic_bytes_per_launch"] = alg
        out["ratio_hbm_to_algorithmic"] = out["hbm_bytes_per_launch"] / alg
    path = out_path or os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def trace_summary(trace_dir, out_path, title, command, per_call=0):
    """Per-kernel table (calls, average / min / max duration, share of GPU time) from a
    rocprofv3 --kernel-trace --stats run's kernel_stats.csv.  With per_call = the number
    of calls of the entry point in the trace, the table gives each kernel's time per call
    of the entry point instead, and their sum."""
    import csv
    import glob
    import shlex

    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    cmds = command if not per_call else (
        command + "\npython3 bench.py --trace-summary " + " ".join(
            shlex.quote(a) for a in (trace_dir, out_path, title, command)) + f" --per-call {per_call}")
    lines = [f"# rocprofv3 kernel statistics — {title}", "",
             "Command (repo root, MI355X, `export TMPDIR=/tmp`):", "", "```", cmds, "```", ""]
    if per_call:
        lines += [f"({per_call} calls of the entry point in the trace)", "",
                  "| Kernel | Calls | Avg (us) | Per call of the entry point (us) |",
                  "|---|---|---|---|"]
    else:
        lines += ["| Kernel | Calls | Avg (us) | Min (us) | Max (us) | Share of GPU time |",
                  "|---|---|---|---|---|---|"]
    total = 0.0
    for r in rows:
        n = r["Name"].replace("void (anonymous namespace)::", "").replace("(anonymous namespace)::", "")
        avg = float(r["AverageNs"]) / 1e3
        if per_call:
            each = int(r["Calls"]) * avg / per_call
            total += each
            lines.append(f"| `{n[:100]}` | {r['Calls']} | {avg:.2f} | {each:.1f} |")
        else:
            lines.append(f"| `{n[:100]}` | {r['Calls']} | {avg:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['Percentage']):.1f}% |")
    if per_call:
        lines += ["", f"Kernel time per call of the entry point: {total / 1e3:.3f} ms."]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def mfma_util_summary(pmc_dir, out_path):
    """Per kernel, the median over its dispatches of MFMA busy cycles over the SIMD
    cycles of the dispatch (SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE
    / 8 XCDs)), from one rocprofv3 --pmc run of SQ_VALU_MFMA_BUSY_CYCLES and
    GRBM_GUI_ACTIVE."""
    import statistics

    per = {}
    for r in _pmc_rows(pmc_dir):
        key = (r["Kernel_Name"], r.get("Dispatch_Id", ""))
        per.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    util = {}
    for (name, _), c in per.items():
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in c or not c.get("GRBM_GUI_ACTIVE"):
            continue
        u = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024.0 * c["GRBM_GUI_ACTIVE"] / 8.0)
        util.setdefault(name, []).append(u)
    rows = sorted(util.items(), key=lambda kv: -statistics.median(kv[1]))
    lines = ["| Kernel | Dispatches | MFMA busy / SIMD cycles (median) |", "|---|---|---|"]
    for name, v in rows:
        n = name.replace("void (anonymous namespace)::", "").replace("(anonymous namespace)::", "")
        lines.append(f"| `{n[:95]}` | {len(v)} | {statistics.median(v):.3f} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def timed_then_profiled(fn, steps, roofline_class, classes):
    """K timed calls with the library's HIP events around the roofline class's
    launches only (few events: each record costs the GPU a few microseconds), then
    K more with events on every class of the breakdown; returns (elapsed seconds
    of the timed calls, {class: (ms, launches)}), the roofline class's figures
    from the timed calls."""
    from vision_transformer_encoder_image_amd import api
    import torch

    api.profile_enable(roofline_class, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per = {roofline_class: api.profile_read(roofline_class)}
    api.profile_enable(roofline_class, False)
    others = [k for k in classes if k != roofline_class]
    for k in others:
        api.profile_enable(k, True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    for k in others:
        per[k] = api.profile_read(k)
        api.profile_enable(k, False)
    return elapsed, per


def cpu_baseline(cfg, inp, budget_s=30.0):
    """Time the oracle (as is, in single precision: the workload's fp32 oracle reading) on
    a bounded sample of the workload on the host cores: the median of 3 passes with every
    BLAS thread, and the median of 3 passes with one BLAS thread."""
    import statistics

    import numpy as np
    import threadpoolctl

    import oracle

    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    # sample: whole images, in order, up to ~4096 patches (the ragged 4-image batch
    # runs whole)
    grids = list(cfg.grids)
    take = []
    for g in grids:
        take.append(g)
        if sum(a * b for a, b in take) >= 4096:
            break
    P = sum(a * b for a, b in take)

    def run(patches, gs):
        t0 = time.perf_counter()
        oracle.encode_varlen(patches, gs, inp["weights"], cfg.n_heads, cfg.rms_eps,
                             cfg.rope_theta, with_aligner=cfg.aligner, dtype=np.float32)
        return time.perf_counter() - t0

    times = [run(inp["patches"][:P], take) for _ in range(3)]
    dt = statistics.median(times)
    # one BLAS thread: the same sample when three passes fit the budget, otherwise
    # the smallest image of it
    one = take
    if 3 * dt * cores > budget_s:
        one = [min(take, key=lambda g: g[0] * g[1])]
    off = 0
    for g in take:
        if g == one[0]:
            break
        off += g[0] * g[1]
    P1 = sum(a * b for a, b in one)
    with threadpoolctl.threadpool_limits(limits=1, user_api="blas"):
        times1 = [run(inp["patches"][off:off + P1], one) for _ in range(3)]
    dt1 = statistics.median(times1)
    blas = sorted({i.get("internal_api", "?") for i in info if i.get("user_api") == "blas"})
    cpu_model = "?"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    desc1 = ("the same sample" if one == take else f"the {one[0][0]}x{one[0][1]} image")
    return {"value": P / dt, "unit": "patches/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(take)} of {len(grids)} images ({P} patches, {cfg.n_blocks} blocks, "
                      f"float32 numpy oracle, median of 3 passes: "
                      f"{', '.join(f'{t:.2f}' for t in times)} s)",
            "value_1_thread": P1 / dt1,
            "sample_1_thread": f"{desc1}, one BLAS thread, median of 3 passes: "
                               f"{', '.join(f'{t:.2f}' for t in times1)} s",
            "cpu_model": cpu_model, "cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)), "blas": blas}


def copy_calibration(mb, dev):
    """A plain device copy of known size, whose counter readings scale FETCH_SIZE /
    WRITE_SIZE of the measured kernels to bytes."""
    import torch

    n = mb * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


MERGE_METRIC = "GB/s, image tokens + sentinels merged into the LLM embedding stream (bf16)"


def bench_merge(args):
    """vit_merge_image_embeddings on the throughput batch's aligner output: 16 images
    of 48x48 patches -> 24x24 merged tokens each, in newline layout (602 positions
    per image), each image after 256 text positions; LLM width 4096, bf16.  One step
    is one merge call over the whole stream (group counts, scan, row copies)."""
    import numpy as np
    import torch

    from vision_transformer_encoder_image_amd import api

    dev = "cuda:0"
    n_img, (gh, gw), text, L = 16, (48, 48), 256, 4096
    _, nl_type, _ = api.aligner_layout(gh, gw, device=dev)
    span = torch.cat([torch.full((text,), -1, dtype=torch.int32, device=dev), nl_type])
    types = span.repeat(n_img).contiguous()
    positions = types.numel()
    n_tok = n_img * (gh // 2) * (gw // 2)
    g = torch.Generator(device="cpu").manual_seed(5)
    tokens = torch.randn((n_tok, L), generator=g).to(dev, torch.bfloat16)
    sent = torch.randn((3, L), generator=g).to(dev, torch.bfloat16)
    embeds = torch.randn((positions, L), generator=g).to(dev, torch.bfloat16)
    ws = torch.empty(api.merge_workspace_bytes(positions), dtype=torch.uint8, device=dev)
    n_image = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(max(args.warmup, 1)):
        api.merge_image_embeddings_(embeds, types, tokens, sent, ws=ws, n_image=n_image)
    torch.cuda.synchronize()
    assert int(n_image.item()) == n_tok
    replaced = int((types >= 0).sum().item())  # codes 0..3 are all replaced
    row_bytes = L * 2
    alg_bytes = replaced * row_bytes * 2 + positions * 4  # rows read + written, types read

    api.profile_enable("merge", True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        api.merge_image_embeddings_(embeds, types, tokens, sent, ws=ws, n_image=n_image)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms, n = api.profile_read("merge")
    api.profile_enable("merge", False)
    copy_s = ms / 1e3 / max(n, 1)
    achieved = alg_bytes / copy_s / 1e9
    result = {
        "metric": MERGE_METRIC,
        "value": round(alg_bytes * args.steps / elapsed / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "merge_16x48x48_nlayout", "positions": positions,
                   "replaced_rows": replaced, "image_tokens": n_tok, "hidden": L,
                   "algorithmic_bytes": alg_bytes},
        "roofline": {"kernel": "merge_copy", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic("merge", "merge_16x48x48_nlayout"),
                     "avg_launch_us": round(copy_s * 1e6, 3), "launches": n,
                     "bytes_per_launch": alg_bytes},
    }
    if args.copy_calibration_mb:
        copy_calibration(args.copy_calibration_mb, dev)
    if not args.no_cpu_baseline:
        import oracle

        ty, tk, st, em = (types.cpu().numpy(), tokens.float().cpu().numpy(),
                          sent.float().cpu().numpy(), embeds.float().cpu().numpy())
        runs, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0:
            oracle.merge_image_embeddings(em, ty, tk, st)
            runs += 1
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(alg_bytes * runs / dt / 1e9, 3), "unit": "GB/s",
                                  "cores": 1, "kind": "oracle",
                                  "sample": f"the whole stream, {runs} oracle passes in {dt:.1f} s "
                                            "(float32 rows, one Python thread)"}
    print(json.dumps(result), flush=True)


PROJ_METRIC = "TFLOP/s through the PatchMerger projector (bf16)"


def bench_projector(args):
    """vit_patch_merger on the high-res workload's tower output: one 64x64 grid of
    1152-dim patches (synthetic bf16 stand-in for the encoder output) -> LayerNorm
    and 2x2 merge -> 1024 x 4608 -> Linear 4608 -> GELU -> Linear 4096 (the
    projector shape of the NVFP4 model page).  One step is one projector call."""
    import torch

    from vision_transformer_encoder_image_amd import api, synth

    dev = "cuda:0"
    gh = gw = 64
    dim, hidden, out = 1152, 4608, 4096
    grids = [(gh, gw)]
    P = gh * gw
    T = P // 4
    x_host = synth.random_array((P, dim), 60, bf16=True)
    w_host = synth.make_merger_weights(dim, hidden, out, seed=61)
    x = torch.from_numpy(x_host).to(dev, torch.bfloat16)
    mw = api.MergerWeights(w_host, device=dev)
    y = torch.empty((T, out), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(api.merger_workspace_bytes(mw, grids), dtype=torch.uint8, device=dev)
    flops = {"proj1": 2.0 * T * 4 * dim * hidden, "proj2": 2.0 * T * hidden * out}
    total = sum(flops.values())
    for _ in range(max(args.warmup, 1)):
        api.patch_merger(x, grids, mw, out=y, ws=ws)
    torch.cuda.synchronize()
    for k in ("lngather", "proj1", "proj2"):
        api.profile_enable(k, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        api.patch_merger(x, grids, mw, out=y, ws=ws)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per = {}
    for k in ("lngather", "proj1", "proj2"):
        ms, n = api.profile_read(k)
        api.profile_enable(k, False)
        per[k] = ms * 1e3 / max(n, 1)
    avg = per["proj1"] * 1e-6
    achieved = flops["proj1"] / avg / 1e12
    peak = PEAK_TFLOPS["bf16"]
    ln_bytes = P * dim * 2 * 2 + 2 * dim * 4  # rows read and written (bf16), weight and bias
    result = {
        "metric": PROJ_METRIC,
        "value": round(total * args.steps / elapsed / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "projector_64x64_1152", "patches": P, "tokens": T, "dim": dim,
                   "hidden": hidden, "out": out, "flops_per_step": total},
        "roofline": {"kernel": "proj1", "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": counter_traffic("proj1", "projector_64x64_1152"),
                     "avg_launch_us": round(per["proj1"], 3), "flops_per_launch": flops["proj1"]},
        "breakdown": {"lngather": {"avg_us": round(per["lngather"], 2),
                                   "gbs": round(ln_bytes / (per["lngather"] * 1e-6) / 1e9, 1)},
                      "proj1": {"avg_us": round(per["proj1"], 2),
                                "tflops": round(flops["proj1"] / (per["proj1"] * 1e-6) / 1e12, 1)},
                      "proj2": {"avg_us": round(per["proj2"], 2),
                                "tflops": round(flops["proj2"] / (per["proj2"] * 1e-6) / 1e12, 1)}},
    }
    if args.copy_calibration_mb:
        copy_calibration(args.copy_calibration_mb, dev)
    if not args.no_cpu_baseline:
        import threadpoolctl

        import oracle

        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
        rows, runs, t0 = 2, 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0:  # the top two patch rows: 32 merged tokens
            oracle.patch_merger(x_host[:rows * gw], rows, gw, w_host)
            runs += 1
        dt = time.perf_counter() - t0
        sample_flops = total * (rows * gw) / P
        result["cpu_baseline"] = {"value": round(sample_flops * runs / dt / 1e12, 4),
                                  "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
                                  "sample": f"the top {rows} patch rows ({rows * gw // 4} merged "
                                            f"tokens), {runs} float64 oracle passes in {dt:.1f} s"}
    print(json.dumps(result), flush=True)


BWD_METRIC = "TFLOP/s through the backward of a block's MLP half (bf16 GEMMs)"


def bench_mlp_backward(args):
    """vit_mlp_backward at the ragged 4-image batch's shape: 3,562 rows, vision_dim
    1024, MLP hidden 2816 (synthetic fp32 x / dy, bf16 weights).  One step is one
    backward call: the SwiGLU pre-activations recomputed, da, dn and the three
    weight gradients (GEMMs), plus norm, cast, transpose and SwiGLU-gradient passes."""
    import numpy as np
    import torch

    from vision_transformer_encoder_image_amd import api, synth

    dev = "cuda:0"
    P, d, h = 3562, 1024, 2816
    Pp = (P + 63) // 64 * 64
    host = [synth.random_array((P, d), 100), np.float32(1.0) + synth.random_array((d,), 101, std=0.02),
            synth.random_array((h, d), 102, std=0.02, bf16=True),
            synth.random_array((h, d), 103, std=0.02, bf16=True),
            synth.random_array((d, h), 104, std=0.02, bf16=True), synth.random_array((P, d), 105)]
    f = lambda a: torch.from_numpy(a).to(dev)
    b = lambda a: torch.from_numpy(a).to(dev, torch.bfloat16)
    x, w, wg, wu, wd, dy = f(host[0]), f(host[1]), b(host[2]), b(host[3]), b(host[4]), f(host[5])
    ws = torch.empty(api._lib.load().vit_mlp_backward_workspace_bytes(P, d, h), dtype=torch.uint8,
                     device=dev)
    flops = {"recompute": 4.0 * P * h * d, "da": 2.0 * P * d * h, "dn": 4.0 * P * h * d,
             "wgrad": 6.0 * d * h * Pp}
    total = sum(flops.values())
    for _ in range(max(args.warmup, 1)):
        api.mlp_backward(x, w, wg, wu, wd, dy, ws=ws)
    torch.cuda.synchronize()
    elapsed, per = timed_then_profiled(lambda: api.mlp_backward(x, w, wg, wu, wd, dy, ws=ws),
                                       args.steps, "bwd_dn", ("bwd_gemm", "bwd_dn", "bwd_pass"))
    dn_us = per["bwd_dn"][0] * 1e3 / max(per["bwd_dn"][1], 1)
    peak = PEAK_TFLOPS["bf16"]
    achieved = flops["dn"] / (dn_us * 1e-6) / 1e12
    result = {
        "metric": BWD_METRIC,
        "value": round(total * args.steps / elapsed / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mlp_backward_ragged_varlen_4img", "rows": P, "dim": d, "hidden": h,
                   "flops_per_step": total},
        "roofline": {"kernel": "bwd_dn", "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": None, "avg_launch_us": round(dn_us, 3),
                     "flops_per_launch": flops["dn"]},
        "breakdown": {"gemms_us_per_step": round(per["bwd_gemm"][0] * 1e3 / args.steps, 1),
                      "gemm_tflops": round(total / (per["bwd_gemm"][0] * 1e-3 / args.steps) / 1e12, 1),
                      "passes_us_per_step": round(per["bwd_pass"][0] * 1e3 / args.steps, 1)},
    }
    if not args.no_cpu_baseline:
        import threadpoolctl

        import oracle

        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
        rows, runs, t0 = 512, 0, time.perf_counter()
        sample = [host[0][:rows], host[1], host[2], host[3], host[4], host[5][:rows]]
        while time.perf_counter() - t0 < 10.0:
            oracle.mlp_half_backward(*sample)
            runs += 1
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(total * rows / P * runs / dt / 1e12, 4),
                                  "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
                                  "sample": f"{rows} of {P} rows, {runs} float64 oracle passes "
                                            f"in {dt:.1f} s"}
    print(json.dumps(result), flush=True)


ATTN_BWD_METRIC = "TFLOP/s through the backward of a block's attention half (bf16)"


def bench_attn_backward(args):
    """vit_attn_backward on the ragged 4-image batch (27x37, 37x27, 10x78, 112x7;
    vision_dim 1024, 16 heads x 64; synthetic fp32 x / dy, bf16 weights).  One step
    is one backward call: the forward recomputation (norm, wqkv, rotary, attention
    with log-sum-exp), dO, the attention gradient, the wqkv / out-projection
    gradients and the norm gradient."""
    import numpy as np
    import torch

    from vision_transformer_encoder_image_amd import api, configs, synth

    dev = "cuda:0"
    cfg = configs.get("ragged_varlen_4img")
    grids = list(cfg.grids)
    P, d, H = cfg.total_patches, cfg.vision_dim, cfg.n_heads
    Pp = (P + 63) // 64 * 64
    sq = sum((h * w) ** 2 for h, w in grids)
    host = [synth.random_array((P, d), 140), np.float32(1.0) + synth.random_array((d,), 141, std=0.02),
            synth.random_array((3 * d, d), 142, std=0.02, bf16=True),
            synth.random_array((d, d), 143, std=0.02, bf16=True), synth.random_array((P, d), 144)]
    f = lambda a: torch.from_numpy(a).to(dev)
    b = lambda a: torch.from_numpy(a).to(dev, torch.bfloat16)
    x, w, wqkv, wo, dy = f(host[0]), f(host[1]), b(host[2]), b(host[3]), f(host[4])
    flops = {"recompute": 6.0 * P * d * d + 4.0 * d * sq, "do": 2.0 * P * d * d,
             "attn": 10.0 * d * sq, "dn": 6.0 * P * d * d, "wgrad": 8.0 * d * d * Pp}
    total = sum(flops.values())
    for _ in range(max(args.warmup, 1)):
        api.attn_backward(x, w, wqkv, wo, dy, grids, H)
    torch.cuda.synchronize()
    elapsed, per = timed_then_profiled(lambda: api.attn_backward(x, w, wqkv, wo, dy, grids, H),
                                       args.steps, "bwd_attn", ("bwd_attn", "bwd_gemm"))
    attn_us = per["bwd_attn"][0] * 1e3 / max(per["bwd_attn"][1], 1)
    peak = PEAK_TFLOPS["bf16"]
    achieved = flops["attn"] / (attn_us * 1e-6) / 1e12
    result = {
        "metric": ATTN_BWD_METRIC,
        "value": round(total * args.steps / elapsed / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "attn_backward_ragged_varlen_4img", "grids": [list(g) for g in grids],
                   "patches": P, "dim": d, "heads": H, "head_dim": 64, "flops_per_step": total},
        "roofline": {"kernel": "bwd_attn", "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": None, "avg_launch_us": round(attn_us, 3),
                     "flops_per_launch": flops["attn"],
                     "note": "the dQ and dK/dV kernels together; algorithmic FLOPs 10 d sum(P_i^2) "
                             "(S recomputed once); the kernels execute 14 d sum(P_i^2)"},
        "breakdown": {"gemms_us_per_step": round(per["bwd_gemm"][0] * 1e3 / args.steps, 1)},
    }
    if not args.no_cpu_baseline:
        import threadpoolctl

        import oracle

        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
        gh, gw = grids[2]  # the 10x78 image: 780 patches
        off = grids[0][0] * grids[0][1] + grids[1][0] * grids[1][1]
        cos, sin = oracle.rope_table(gh, gw, 64, 10000.0)
        Pi = gh * gw
        runs, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0:
            oracle.attn_half_backward(host[0][off:off + Pi], host[1], host[2], host[3], cos, sin, H,
                                      host[4][off:off + Pi])
            runs += 1
        dt = time.perf_counter() - t0
        sample = 6.0 * Pi * d * d + 4.0 * d * Pi * Pi + 2.0 * Pi * d * d + 10.0 * d * Pi * Pi + \
            6.0 * Pi * d * d + 8.0 * d * d * Pi
        result["cpu_baseline"] = {"value": round(sample * runs / dt / 1e12, 4), "unit": "TFLOP/s",
                                  "cores": int(cores), "kind": "oracle",
                                  "sample": f"the 10x78 image ({Pi} patches), {runs} float64 "
                                            f"oracle passes in {dt:.1f} s"}
    print(json.dumps(result), flush=True)


TOWER_BWD_METRIC = "TFLOP/s through the backward of the whole tower (bf16)"


def tower_backward_flops(cfg, grids):
    """Algorithmic FLOPs of one tower backward: the forward once (patch embedding,
    blocks), every block GEMM's data and weight gradients (2x its forward FLOPs),
    the attention gradient 8 d sum(P_i^2) per block (dV, dP, dQ, dK; no recomputed
    S) and the patch embedding's weight gradient."""
    P, d, h = sum(a * b for a, b in grids), cfg.vision_dim, cfg.mlp_hidden
    sq = sum((a * b) ** 2 for a, b in grids)
    gemm = 8.0 * P * d * d + 6.0 * P * d * h
    fwd = cfg.n_blocks * (gemm + 4.0 * d * sq) + 2.0 * P * cfg.patch_dim * d
    return fwd + cfg.n_blocks * (2.0 * gemm + 8.0 * d * sq) + 2.0 * P * cfg.patch_dim * d


def bench_tower_backward(args):
    """vit_tower_backward on the ragged 4-image batch (27x37, 37x27, 10x78, 112x7;
    vision_dim 1024, 16 heads x 64, hidden 2816, 4 blocks), or with --workload on
    another workload's grids and widths (the 64x64 tower: 1152, 16 heads x 72,
    hidden 4304, 32 blocks); synthetic bf16 patches and weights, fp32 dy.  One step
    is one call: the forward with residual checkpoints, the final norm's gradient,
    every block's halves in reverse and the patch embedding's gradient."""
    import torch

    from vision_transformer_encoder_image_amd import api, configs, synth

    dev = "cuda:0"
    cfg = configs.get(args.workload)
    grids = list(cfg.grids)
    P, d, h, L = cfg.total_patches, cfg.vision_dim, cfg.mlp_hidden, cfg.n_blocks
    Pp = (P + 63) // 64 * 64
    hp = (h + 63) // 64 * 64  # the MLP backward's padded hidden width
    inp = synth.make_inputs(cfg, seed=2)
    w = api.DeviceWeights(cfg, inp["weights"], device=dev)
    x = torch.from_numpy(inp["patches"]).to(dev, torch.bfloat16)
    dy = torch.from_numpy(synth.random_array((P, d), 180)).to(dev)
    ws = torch.empty(api.tower_backward_workspace_bytes(cfg, grids), dtype=torch.uint8, device=dev)
    total = tower_backward_flops(cfg, grids)
    # FLOPs the backward GEMM class executes per call (with the halves' recomputed
    # forward GEMMs and the weight gradients' row padding)
    gemm_exec = L * (6.0 * P * d * d + 2.0 * P * d * d + 6.0 * P * d * d + 8.0 * d * d * Pp +
                     4.0 * P * d * h + 2.0 * P * d * h + 4.0 * P * d * hp + 6.0 * d * h * Pp)
    for _ in range(max(args.warmup, 1)):
        api.tower_backward(x, grids, w, dy, ws=ws)
    torch.cuda.synchronize()
    classes = ("bwd_gemm", "bwd_attn", "bwd_pass")
    elapsed, per = timed_then_profiled(lambda: api.tower_backward(x, grids, w, dy, ws=ws),
                                       args.steps, "bwd_gemm", classes)
    gemm_us = per["bwd_gemm"][0] * 1e3 / args.steps
    peak = PEAK_TFLOPS["bf16"]
    achieved = gemm_exec / (gemm_us * 1e-6) / 1e12
    result = {
        "metric": TOWER_BWD_METRIC,
        "value": round(total * args.steps / elapsed / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"tower_backward_{cfg.name}", "grids": [list(g) for g in grids],
                   "patches": P, "dim": d, "heads": cfg.n_heads, "mlp_hidden": h, "blocks": L,
                   "flops_per_step": total},
        "roofline": {"kernel": "bwd_gemm", "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": None, "avg_launch_us": round(gemm_us, 3),
                     "flops_per_launch": gemm_exec,
                     "note": "every GEMM of the blocks' backward halves per call (the halves' "
                             "recomputed forward GEMMs included), timed as one class"},
        "breakdown": {k + "_us_per_step": round(per[k][0] * 1e3 / args.steps, 1) for k in classes},
    }
    if not args.no_cpu_baseline:
        import threadpoolctl

        import oracle

        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
        wts = inp["weights"]
        if cfg.name == "ragged_varlen_4img":
            sub = [grids[2]]  # the 10x78 image: 780 patches, all four blocks
            off = grids[0][0] * grids[0][1] + grids[1][0] * grids[1][1]
            scfg, what = cfg, f"the 10x78 image (780 patches, {L} blocks)"
        else:
            # the first 16x16 patches of the first image (rows of its top 16 x 16
            # corner are not contiguous, so the sample is a 16x16 grid of the image's
            # first 256 patches) through the first two blocks
            sub, off = [(16, 16)], 0
            scfg = configs.VitConfig(cfg.name, tuple(sub), d, cfg.n_heads, h, min(L, 2), 0,
                                     cfg.dtype)
            wts = dict(wts, blocks=wts["blocks"][:scfg.n_blocks])
            what = f"a 16x16 grid of the first 256 patches, the first {scfg.n_blocks} blocks"
        Pi = sub[0][0] * sub[0][1]
        pt = inp["patches"][off:off + Pi]
        dyh = synth.random_array((P, d), 180)[off:off + Pi]
        runs, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0:
            oracle.tower_backward(pt, sub, wts, cfg.n_heads, dyh, cfg.rms_eps, cfg.rope_theta)
            runs += 1
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(tower_backward_flops(scfg, sub) * runs / dt / 1e12, 4),
                                  "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
                                  "sample": f"{what}, {runs} float64 oracle passes in {dt:.1f} s"}
    print(json.dumps(result), flush=True)


GEMM_LIB_METRIC = "TFLOP/s of the encoder's GEMM shapes, library kernel vs vendor BLAS (bf16)"


def bench_gemm_library(args):
    """The block GEMM shapes of a workload (wqkv, out-projection, gate and up side
    by side, down) plus a large square one, each timed as C = A B^T with a plain
    bf16 store: through vit_gemm (the library's MFMA kernel and tile choice) and
    through torch.nn.functional.linear (the vendor BLAS, hipBLASLt), same inputs
    and stream.  Median of per-call HIP events; the outputs are compared.  The
    BLAS leg is a reference point for the hand-written kernel, not part of the
    encoder."""
    import statistics

    import torch

    from vision_transformer_encoder_image_amd import _lib, api, configs

    dev = "cuda:0"
    cfg = configs.get(args.workload)
    P, d, h = cfg.total_patches, cfg.vision_dim, cfg.mlp_hidden
    shapes = [("wqkv", P, 3 * d, d), ("outproj", P, d, d), ("gateup", P, 2 * h, d),
              ("down", P, d, h), ("square8192", 8192, 8192, 8192)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)

    def med_us(fn):
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(args.steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        return statistics.median(ts)

    rows = []
    for name, M, N, K in shapes:
        A = (torch.rand(M, K, device=dev, generator=gen) * 2 - 1).bfloat16()
        B = (torch.randn(N, K, device=dev, generator=gen) * 0.02).bfloat16()
        C = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
        t_lib = med_us(lambda: api.gemm(A, B, _lib.VIT_EPI_STORE, C=C))
        ref = torch.nn.functional.linear(A, B)
        t_blas = med_us(lambda: torch.nn.functional.linear(A, B))
        diff = float((C.float() - ref.float()).abs().max() / ref.float().abs().max())
        fl = 2.0 * M * N * K
        rows.append({"gemm": name, "M": M, "N": N, "K": K,
                     "library_us": round(t_lib, 2), "library_tflops": round(fl / t_lib / 1e6, 1),
                     "blas_us": round(t_blas, 2), "blas_tflops": round(fl / t_blas / 1e6, 1),
                     "max_rel_diff": float(f"{diff:.3e}")})
        del A, B, C, ref
    enc = [r for r in rows if r["gemm"] != "square8192"]
    fl_enc = sum(2.0 * r["M"] * r["N"] * r["K"] for r in enc)
    t_enc = sum(r["library_us"] for r in enc)
    result = {
        "metric": GEMM_LIB_METRIC,
        "value": round(fl_enc / t_enc / 1e6, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "higher_is_better": True,
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"gemm_library_{cfg.name}", "shapes": rows,
                   "blas_tflops_encoder_shapes": round(
                       fl_enc / sum(r["blas_us"] for r in enc) / 1e6, 1)},
        "note": "value: the library kernel over the encoder shapes (plain bf16 store, no fused "
                "epilogue); per-call events include the launch; blas = torch.nn.functional.linear",
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--stage", choices=("encode", "merge", "projector", "mlp_backward",
                                        "attn_backward", "tower_backward", "gemm_library"),
                    default="encode",
                    help="encode: the encoder step; merge: image tokens into the LLM stream; "
                         "projector: the PatchMerger projector; mlp_backward / attn_backward: "
                         "the backward of a block's MLP / attention half; tower_backward: the "
                         "backward of the whole tower; gemm_library: the library GEMM against "
                         "the vendor BLAS on the workload's GEMM shapes")
    ap.add_argument("--pixels", action="store_true",
                    help="encode stage: pixel images in (the library cuts the patches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mfma-probe", action="store_true",
                    help="skip the dense-MFMA probe (e.g. under a counter run)")
    ap.add_argument("--breakdown", action="store_true", help="also time every kernel class")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="after the timed steps, run a plain device copy of this many MiB "
                         "(the reference kernel for HBM byte counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "script into profiles/traffic_<kernel>_<workload>.json and exit")
    ap.add_argument("--kernel", default="gateup", help="kernel class for --pmc-summary")
    ap.add_argument("--mfma-summary", nargs=2, metavar=("PMC_DIR", "OUT"),
                    help="summarise a rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE run "
                         "of this script into a per-kernel MFMA-utilisation table and exit")
    ap.add_argument("--pmc-out", default=None, help="output path for --pmc-summary")
    ap.add_argument("--trace-summary", nargs=4, metavar=("TRACE_DIR", "OUT", "TITLE", "COMMAND"),
                    help="summarise a rocprofv3 --kernel-trace --stats run into a markdown table "
                         "and exit")
    ap.add_argument("--per-call", type=int, default=0,
                    help="with --trace-summary: calls of the entry point in the trace (the table "
                         "then gives each kernel's time per call)")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(*args.trace_summary, per_call=args.per_call)
        return
    if args.mfma_summary:
        mfma_util_summary(args.mfma_summary[0], args.mfma_summary[1])
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.kernel, args.workload,
                    args.copy_calibration_mb, args.pmc_out)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the encoder shards "
              "by image across GPUs with no exchange, so run one process per GPU instead.",
              file=sys.stderr)
        sys.exit(2)

    if args.stage == "merge":
        bench_merge(args)
        return
    if args.stage == "projector":
        bench_projector(args)
        return
    if args.stage == "mlp_backward":
        bench_mlp_backward(args)
        return
    if args.stage == "attn_backward":
        bench_attn_backward(args)
        return
    if args.stage == "tower_backward":
        bench_tower_backward(args)
        return
    if args.stage == "gemm_library":
        bench_gemm_library(args)
        return

    import torch

    from vision_transformer_encoder_image_amd import api, configs, synth

    cfg = configs.get(args.workload)
    idx = [c.name for c in configs.CONFIGS].index(cfg.name)
    inp = synth.make_inputs(cfg, seed=idx)
    dev = "cuda:0"
    w = api.DeviceWeights(cfg, inp["weights"], device=dev)
    # with --pixels the same synthetic values are read as the images' pixels
    # ([3, 14 gh, 14 gw] each, back to back) and the library cuts the patches
    x = torch.from_numpy(inp["patches"]).to(dev, torch.bfloat16 if cfg.dtype == "bf16" else torch.float32)
    if args.pixels:
        x = x.reshape(-1)
    enc = api.Encoder(cfg, w, cfg.grids, aligner=cfg.aligner, device=dev, pixels=args.pixels)
    out = torch.empty(enc.out_shape, dtype=x.dtype, device=dev)

    flops = class_flops(cfg)
    for _ in range(max(args.warmup, 1)):
        enc(x, out)
    torch.cuda.synchronize()

    # which kernel dominates: one profiled step per class (not part of the timing)
    per_class = {}
    for k in list(flops) + ["rmsnorm"]:
        api.profile_enable(k, True)
    enc(x, out)
    torch.cuda.synchronize()
    for k in list(flops) + ["rmsnorm"]:
        ms, n = api.profile_read(k)
        api.profile_enable(k, False)
        per_class[k] = ms
    outside_ms = per_class.pop("embed", 0.0) + per_class.pop("rmsnorm", 0.0)
    if cfg.aligner:
        outside_ms += per_class.pop("aligner", 0.0)
    dominant = max(per_class, key=per_class.get)

    # timed region: K steps bracketed by synchronisations, with a HIP event pair around
    # every call on the call's stream (created beforehand; no library events inside)
    import statistics

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        enc(x, out)
        e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    call_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    med_ms = statistics.median(call_ms)
    # then the same number of calls with the library's HIP events around every launch
    # of the dominant class (its average launch duration for the roofline)
    api.profile_enable(dominant, True)
    for _ in range(args.steps):
        enc(x, out)
    torch.cuda.synchronize()
    dom_ms, dom_n = api.profile_read(dominant)
    api.profile_enable(dominant, False)

    P = cfg.total_patches
    ms_per_step = med_ms
    value = P / (med_ms / 1e3)
    peak = PEAK_TFLOPS[cfg.dtype]
    avg_launch_s = dom_ms / 1e3 / max(dom_n, 1)
    achieved = flops[dominant] / avg_launch_s / 1e12
    traffic = counter_traffic(dominant, cfg.name)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "patches/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "timing": {"value_from": "median of per-call HIP event times",
                   "call_ms_min": round(min(call_ms), 4), "call_ms_max": round(max(call_ms), 4),
                   "wall_ms_per_step": round(elapsed * 1e3 / args.steps, 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "grids": [list(g) for g in cfg.grids], "patches": P,
                   "vision_dim": cfg.vision_dim, "heads": cfg.n_heads, "head_dim": cfg.head_dim,
                   "mlp_hidden": cfg.mlp_hidden, "blocks": cfg.n_blocks,
                   "aligner": cfg.llm_dim if cfg.aligner else None,
                   "input": "pixels" if args.pixels else "patches"},
        "mfma_frac_step": round(cfg.total_flops() / (ms_per_step / 1e3) / (peak * 1e12), 4),
        # the block stack alone (norm1 .. down + residual of every block): the step's
        # time less the patch embedding, the final norm and the aligner, timed with
        # HIP events in one profiled step before the timed region
        "mfma_frac_blocks": round(cfg.n_blocks * cfg.block_flops() /
                                  ((ms_per_step - outside_ms) / 1e3) / (peak * 1e12), 4),
        "roofline": {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic, "avg_launch_us": round(avg_launch_s * 1e6, 3),
                     "launches": dom_n, "flops_per_launch": flops[dominant]},
    }
    # the dense-MFMA probe: what the chip sustains, beside the published peak
    measured = None if args.no_mfma_probe else api.mfma_peak_tflops(device=dev)
    if measured:
        result["mfma_peak_measured"] = {
            "tflops": round(measured, 1), "kernel": "mfma_peak_kernel",
            "roofline_frac_of_measured": round(achieved / measured, 4),
            "blocks_frac_of_measured": round(result["mfma_frac_blocks"] * peak / measured, 4),
            "note": "back-to-back v_mfma_f32_32x32x16_bf16 on register operands, one 8-wave "
                    "workgroup per CU, no memory traffic; best of 5 calls"}
    if args.breakdown:
        bd = {}
        for k in list(flops) + ["rmsnorm", "rope", "gather"]:
            if k == "gather" and not cfg.aligner:
                continue
            api.profile_enable(k, True)
        for _ in range(5):
            enc(x, out)
        torch.cuda.synchronize()
        byts = class_bytes(cfg)
        for k in list(flops) + ["rmsnorm", "rope", "gather"]:
            if k == "gather" and not cfg.aligner:
                continue
            ms, n = api.profile_read(k)
            api.profile_enable(k, False)
            if n == 0:
                continue
            us = ms * 1e3 / n
            e = {"avg_us": round(us, 2), "launches_per_step": n // 5}
            if k in flops:
                e["tflops"] = round(flops[k] / (us * 1e-6) / 1e12, 1)
                e["mfma_frac"] = round(flops[k] / (us * 1e-6) / 1e12 / peak, 4)
            else:
                e["gbs"] = round(byts[k] / (us * 1e-6) / 1e9, 1)
                e["hbm_frac"] = round(byts[k] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
            bd[k] = e
        result["breakdown"] = bd
    if args.copy_calibration_mb:
        copy_calibration(args.copy_calibration_mb, dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, inp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
