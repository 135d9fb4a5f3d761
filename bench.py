"""Benchmark of the SparseSAM encoder-block hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input: Sobel importance,
stripe-sort permutation and keep-set, then one SparseSAM block (gathered LayerNorm,
QKV, block-sparse attention, projection with residual scatter, routed MLP), on the
SAM ViT-B global-attention workload (64 x 64 tokens, C 768, 12 heads x 64, MLP
3072, batch 1, attention and MLP density 0.4). Inputs are resident in HBM before
timing starts.

Prints ONE JSON line (rank 0). Extra fields report the attention and MLP kernels'
TFLOP/s on the computed work (the kept tiles and routed tokens only), the same at
density 0.3, the dense comparators (this library at density 1.0 and a PyTorch eager
bf16 dense block) and the CPU oracle timed on this host on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--profile-only]
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0
METRIC = "SparseSAM block tokens/s + attn/MLP TFLOP/s (% bf16 peak) at density 0.4/0.3"


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


ATTN_SOURCE = os.path.join(ROOT, "structured_sparse_vit_amd", "csrc", "k_attention.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_mfma64_c2_traffic.txt")


def _source_hash(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per attention launch from the committed counter summary, or None.

    The summary records FETCH_SIZE and WRITE_SIZE of the attention dispatch and of a
    plain copy of known size (the scale factor), and the hash of the kernel source
    they were taken with; a different source hash means the numbers are stale.
    """
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    vals = {}
    with open(TRAFFIC_PROFILE) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    try:
        if vals.get("source_sha256_16") != _source_hash(ATTN_SOURCE):
            return None
        return float(vals["scaled_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def attention_flops(plan):
    """4 * B^2 * D per kept tile per head (2 for Q K^T, 2 for P V), per segment."""
    info = plan.info
    return 4.0 * info["pairs_kept"] * plan.desc.head_dim * plan.desc.heads


def mlp_flops(plan, batch):
    return 4.0 * plan.desc.channels * plan.desc.mlp_hidden * plan.info["routed_per_image"] * batch


def block_flops(plan, batch):
    C = plan.desc.channels
    tokens = plan.info["seq_len"] * plan.info["segments_per_image"] * batch
    segs = plan.info["segments_per_image"] * batch
    return 8.0 * C * C * tokens + attention_flops(plan) * segs + mlp_flops(plan, batch)


class Workload:
    """Device-resident inputs, weights, outputs and workspace of one config."""

    def __init__(self, cfg, dev, seed=0, rel_pos=False):
        import numpy as np
        import torch

        import structured_sparse_vit_amd as ss
        from synth import block_weights, synthetic_images, token_features
        from synth.generate import rel_pos_tables

        self.cfg = cfg
        self.ss = ss
        self.plan = ss.Plan.from_config(cfg, rel_pos=rel_pos)
        self.img = torch.from_numpy(synthetic_images(cfg, seed)).to(dev)
        self.x0 = torch.from_numpy(token_features(cfg, seed)).to(dev)
        self.x = self.x0.clone()
        w = block_weights(cfg, seed)
        if rel_pos:
            w["rel_h"], w["rel_w"] = rel_pos_tables(cfg, seed)
        self.w = ss.weights_to_device(w, self.plan)
        info = self.plan.info
        b = cfg.batch
        self.imp = torch.empty(b, cfg.grid * cfg.grid, dtype=torch.float32, device=dev)
        self.perm = torch.empty(b * info["segments_per_image"], info["seq_len"], dtype=torch.int32, device=dev)
        self.inv = torch.empty_like(self.perm)
        self.routed = torch.empty(b * info["routed_per_image"], dtype=torch.int32, device=dev)
        self.ws = torch.empty(info["block_workspace_bytes"], dtype=torch.uint8, device=dev)
        self.mlp_ws = torch.empty(info["mlp_workspace_bytes"], dtype=torch.uint8, device=dev)
        self.attn_ws = torch.empty(max(1, info["attn_workspace_bytes"]), dtype=torch.uint8, device=dev)
        self.relpos_ws = (torch.empty(max(1, info["relpos_workspace_bytes"]), dtype=torch.uint8, device=dev)
                          if rel_pos else None)
        self.np = np

    def step(self):
        """Importance, permutation and block: one sparsesam_forward call."""
        self.ss.forward(self.plan, self.w, self.img, self.x, self.cfg.patch,
                        out=(self.imp, self.perm, self.inv, self.routed), workspace=self.ws)

    def attn_operands(self, seed=1):
        """Random q, k, vt and an output buffer in the layout sparsesam_attn takes."""
        import torch
        p = self.plan
        info = p.info
        segs = self.cfg.batch * info["segments_per_image"]
        n, H, D = info["seq_len"], p.desc.heads, p.desc.head_dim
        n_pad = (n + 7) // 8 * 8
        g = torch.Generator(device=self.x.device).manual_seed(seed)
        dt = p.torch_dtype
        q = torch.randn(segs, H, n, D, generator=g, device=self.x.device).to(dt)
        k = torch.randn(segs, H, n, D, generator=g, device=self.x.device).to(dt)
        vt = torch.randn(segs, H, D, n_pad, generator=g, device=self.x.device).to(dt)
        o = torch.empty(segs, n, H * D, dtype=dt, device=self.x.device)
        return q, k, vt, o


def time_region(fn, iters, warmup):
    """Average milliseconds of fn() measured with HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(iters):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters


def torch_dense_block_ms(cfg, dev, iters=20):
    """PyTorch eager bf16 dense block (SDPA + F.linear) on the same shapes, in ms."""
    import torch
    import torch.nn.functional as F
    from synth import block_weights, token_features

    w = {k: torch.from_numpy(v).to(dev) for k, v in block_weights(cfg).items()}
    for k in ("w_qkv", "w_proj", "w1", "w2", "b_qkv", "b_proj", "b1", "b2"):
        w[k] = w[k].to(torch.bfloat16)
    x = torch.from_numpy(token_features(cfg)).to(dev).view(cfg.batch, -1, cfg.channels)
    H, D, C = cfg.heads, cfg.head_dim, cfg.channels

    def run():
        h = F.layer_norm(x, (C,), w["ln1_g"], w["ln1_b"], eps=1e-6).to(torch.bfloat16)
        qkv = F.linear(h, w["w_qkv"], w["b_qkv"])
        q, k, v = qkv.view(cfg.batch, -1, 3, H, D).permute(2, 0, 3, 1, 4).contiguous().unbind(0)
        o = F.scaled_dot_product_attention(q, k, v).transpose(1, 2).reshape(cfg.batch, -1, C)
        x1 = x + F.linear(o, w["w_proj"], w["b_proj"]).float()
        h2 = F.layer_norm(x1, (C,), w["ln2_g"], w["ln2_b"], eps=1e-6).to(torch.bfloat16)
        return x1 + F.linear(F.gelu(F.linear(h2, w["w1"], w["b1"])), w["w2"], w["b2"]).float()

    with torch.no_grad():
        return time_region(run, iters, 3)


def encoder_run(key, dev, density=None, passes=3, rel_pos=False, sorted_stream=False):
    """One pass of a whole encoder config (c4: ViT-L 24 blocks, c5: ViT-H 32 blocks) through
    sparsesam_encoder (or, sorted_stream, sparsesam_encoder_permuted: the residual stream
    kept in stripe-sorted order between blocks): importance and both permutations once
    per pass, then every block. Timing only: one random-init layer's weights serve every
    layer (the work per layer is the same). Returns tokens/s and ms per pass."""
    import torch

    import structured_sparse_vit_amd as ss
    from synth import block_weights, encoder_global_layers, get_config, synthetic_images, token_features
    from synth.configs import global_variant, window_variant
    base = get_config(key)
    if density is not None:
        base = base.with_(attn_density=density, mlp_density=density)
    cg, cw = global_variant(base).with_(batch=base.batch), window_variant(base).with_(batch=base.batch)
    pg, pw = ss.Plan.from_config(cg, rel_pos=rel_pos), ss.Plan.from_config(cw, rel_pos=rel_pos)
    wd = ss.weights_to_device(block_weights(cg, 0), pg)
    gl = set(encoder_global_layers(base.layers))
    kinds = [1 if l in gl else 0 for l in range(base.layers)]
    if rel_pos:  # each block type has tables of its own segment shape
        from synth.generate import rel_pos_tables
        wg = dict(wd)
        wg["rel_pos_h"], wg["rel_pos_w"] = (torch.from_numpy(t).to(dev) for t in rel_pos_tables(cg, 0))
        ww = dict(wd)
        ww["rel_pos_h"], ww["rel_pos_w"] = (torch.from_numpy(t).to(dev) for t in rel_pos_tables(cw, 0))
        layers = [wg if k else ww for k in kinds]
    else:
        layers = [wd] * base.layers
    img = torch.from_numpy(synthetic_images(base, 0)).to(dev)
    x0 = torch.from_numpy(token_features(base, 0)).to(dev)
    x = x0.clone()
    ws = torch.empty(max(pg.info["block_workspace_bytes"], pw.info["block_workspace_bytes"]), dtype=torch.uint8,
                     device=dev)

    if sorted_stream:
        need = ctypes.c_size_t()
        lib = ss._lib.load()
        ss.check(lib.sparsesam_encoder_permuted_workspace(pg.handle, pw.handle, base.batch, ctypes.byref(need)),
                 "sparsesam_encoder_permuted_workspace")
        del ws
        ws = torch.empty(need.value, dtype=torch.uint8, device=dev)

    def one_pass():
        x.copy_(x0)  # every pass starts from the same features
        imp = ss.importance(img, base.patch)
        perm_g, inv_g, routed_g = ss.permute(pg, imp)
        perm_w, inv_w, routed_w = ss.permute(pw, imp)
        if sorted_stream:
            ss.encoder(pg, pw, layers, kinds, x, (perm_g, inv_g), (perm_w, inv_w), workspace=ws, sorted_stream=True)
        else:
            ss.encoder(pg, pw, layers, kinds, x, (perm_g, routed_g), (perm_w, routed_w), workspace=ws)

    ms = time_region(one_pass, passes, 1)
    tokens = base.batch * base.grid * base.grid
    del x, ws
    return {"batch": base.batch, "blocks": base.layers, "global_blocks": sorted(gl),
            "attn_density": base.attn_density, "mlp_density": base.mlp_density,
            "ms_per_pass": round(ms, 3), "tokens_per_s": round(tokens / (ms * 1e-3), 1), "rel_pos": rel_pos,
            "sorted_stream": sorted_stream,
            "weights": "one random-init layer reused by every layer (timing only)"}


def window_block_run(dev):
    """The c3 windowed block (ViT-B, 25 windows of 14 x 14 per image, batch 4): step and
    block times, attention and routed-MLP rates, and the same step at density 1."""
    from synth import get_config
    cfg = get_config("c3")
    wl = Workload(cfg, dev)
    wl.step()
    ss, plan = wl.ss, wl.plan
    blk = time_region(lambda: ss.block(plan, wl.w, wl.x, wl.perm, wl.routed, workspace=wl.ws), 20, 3)
    step = time_region(wl.step, 20, 3)
    tokens = cfg.batch * cfg.grid * cfg.grid
    segs = cfg.batch * plan.info["segments_per_image"]
    q, k, vt, o = wl.attn_operands()
    attn_ms = time_region(lambda: ss.attn(plan, q, k, vt, out=o, workspace=wl.attn_ws), 30, 5)
    attn_tf = attention_flops(plan) * segs / (attn_ms * 1e-3) / 1e12
    xr = wl.x.view(-1, cfg.channels)
    mlp_ms = time_region(lambda: ss.mlp(plan, xr, wl.routed, wl.w["ln2_g"], wl.w["ln2_b"], wl.w["w1"], wl.w["b1"],
                                        wl.w["w2"], wl.w["b2"], workspace=wl.mlp_ws), 30, 5)
    mlp_tf = mlp_flops(plan, cfg.batch) / (mlp_ms * 1e-3) / 1e12
    del wl, q, k, vt, o
    wld = Workload(cfg.with_(attn_density=1.0, mlp_density=1.0), dev)
    wld.step()
    dense = time_region(wld.step, 20, 3)
    dense_blk = time_region(lambda: ss.block(wld.plan, wld.w, wld.x, wld.perm, wld.routed, workspace=wld.ws), 20, 3)
    del wld
    return {"batch": cfg.batch, "block_ms": round(blk, 5), "step_ms": round(step, 5),
            "tokens_per_s": round(tokens / (step * 1e-3), 1),
            "realised_attn_density": plan.info["realised_density"],
            "attn_ms": round(attn_ms, 5), "attn_tflops": round(attn_tf, 2),
            "attn_pct_peak": round(100 * attn_tf / PEAK_BF16_TFLOPS, 2),
            "mlp_ms": round(mlp_ms, 5), "mlp_tflops": round(mlp_tf, 2),
            "mlp_pct_peak": round(100 * mlp_tf / PEAK_BF16_TFLOPS, 2),
            "density_1_step_ms": round(dense, 5), "speedup_vs_density_1": round(dense / step, 3),
            "density_1_block_ms": round(dense_blk, 5), "speedup_vs_density_1_block": round(dense_blk / step, 3),
            "note": "attention TFLOP/s counts kept token pairs only (4 D per pair per head); "
                    "speedup_vs_density_1_block: the sparse step against the block alone at density 1"}


def tiny_block_run(dev):
    """The c1 fp32 block (16 x 16 tokens, C 64, one head): step time and the same step at
    density 1. fp32 runs on the SIMT kernels; the rates are against the fp32 vector peak."""
    from synth import get_config
    cfg = get_config("c1")
    wl = Workload(cfg, dev)
    wl.step()
    step = time_region(wl.step, 50, 5)
    flops = block_flops(wl.plan, cfg.batch)
    wld = Workload(cfg.with_(attn_density=1.0, mlp_density=1.0), dev)
    wld.step()
    dense = time_region(wld.step, 50, 5)
    ss = wld.ss
    dense_blk = time_region(lambda: ss.block(wld.plan, wld.w, wld.x, wld.perm, wld.routed, workspace=wld.ws), 50, 5)
    tokens = cfg.batch * cfg.grid * cfg.grid
    return {"batch": cfg.batch, "step_ms": round(step, 5), "tokens_per_s": round(tokens / (step * 1e-3), 1),
            "realised_attn_density": wl.plan.info["realised_density"],
            "block_tflops": round(flops / (step * 1e-3) / 1e12, 4),
            "density_1_step_ms": round(dense, 5), "speedup_vs_density_1": round(dense / step, 3),
            "density_1_block_ms": round(dense_blk, 5), "speedup_vs_density_1_block": round(dense_blk / step, 3),
            "note": "launch-bound: 256 tokens of 64 channels"}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_step_s(cfg, threads, budget_s, max_runs=3):
    """Seconds per oracle step (importance + permutation + one block) with `threads` BLAS
    threads (None: the library's default, all cores); (seconds, runs)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from synth import block_weights, synthetic_images, token_features
    imgs = synthetic_images(cfg)
    x = token_features(cfg)
    w = block_weights(cfg)
    done, t0 = 0, time.perf_counter()
    with threadpool_limits(threads):
        while True:
            imp = np.stack([oracle.importance(im, cfg.patch) for im in imgs])
            oracle.block_forward(x, imp, w, cfg)
            done += 1
            if time.perf_counter() - t0 > budget_s or done >= max_runs:
                break
    return (time.perf_counter() - t0) / done, done


def cpu_baseline(cfg, budget_s=8.0):
    """The oracle, as it stands, on a bounded sample of the same workload on this host:
    the headline figure (all cores) plus the c1 block, one c2 block and one image's c3
    windowed block (25 windows), each at 1 thread and at all threads."""
    from threadpoolctl import threadpool_info

    from synth import get_config
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    dt, done = _oracle_step_s(cfg, None, budget_s)
    tokens = cfg.batch * cfg.grid * cfg.grid
    by_cfg = {}
    for key, over in (("c1", {}), ("c2", {}), ("c3", {"batch": 1})):
        c = get_config(key).with_(**over)
        tk = c.batch * c.grid * c.grid
        row = {"batch": c.batch, "tokens": tk}
        for th, label in ((1, "1_thread"), (None, "all_threads")):
            if key == cfg_key(cfg) and th is None:
                s, n = dt, done
            else:
                s, n = _oracle_step_s(c, th, budget_s / 2, max_runs=3 if key != "c1" else 20)
            row[label] = {"s_per_step": round(s, 4), "tokens_per_s": round(tk / s, 1), "runs": n}
        by_cfg[key] = row
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": "%d full step(s) of the same workload (importance + permutation + one block, dense "
                      "attention with an explicit mask, fp64 numpy), %.2f s each" % (done, dt),
            "nproc": os.cpu_count(), "cpu_model": _cpu_model(),
            "by_config": by_cfg,
            "note": "the oracle computes every one of the N^2 attention scores (explicit mask) and the MLP on the "
                    "keep-set rows only; c3 is one image of 25 windows; c4 / c5 are not timed end to end"}


def cfg_key(cfg):
    """The config table key of a workload (c1 .. c5), or '' for derived ones."""
    from synth.configs import CONFIGS
    for k, v in CONFIGS.items():
        if v == cfg:
            return k
    return ""


def _prof(out, counters, cfg="c2", extra="", steps=5, warmup=2):
    mode = "--kernel-trace --stats" if counters is None else "--pmc " + counters
    return ("rocprofv3 %s --output-format csv -d gpurun_out/%s -o p -- python3 bench.py --profile-only --config %s "
            "--steps %d --warmup %d%s" % (mode, out, cfg, steps, warmup, extra))


# rocprofv3 runs behind the summaries in profiles/ (one counter group per run; run each from
# the repository root, e.g. under `timeout -s KILL 150`), then
# `python bench.py --summarize-profiles gpurun_out`.
PROFILE_COMMANDS = {
    "trace": _prof("trace_c2", None, steps=20, warmup=5),
    "trace_relpos": _prof("trace_relpos", None, extra=" --rel-pos", steps=20, warmup=5),
    "trace_c3": _prof("trace_c3", None, cfg="c3", steps=20, warmup=5),
    "mfma": _prof("pmc_mfma_c2", "MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16"),
    "fetch": _prof("pmc_fetch_c2", "FETCH_SIZE"),
    "write": _prof("pmc_write_c2", "WRITE_SIZE"),
    "mfma_c3": _prof("pmc_mfma_c3", "MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16", cfg="c3"),
    "fetch_c3": _prof("pmc_fetch_c3", "FETCH_SIZE", cfg="c3"),
    "write_c3": _prof("pmc_write_c3", "WRITE_SIZE", cfg="c3"),
    "trace_c4": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/trace_c4 -o p -- "
                "python3 bench.py --profile-encoder c4 --passes 2",
    "trace_c5": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/trace_c5 -o p -- "
                "python3 bench.py --profile-encoder c5 --passes 2",
    "copy_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch_copy -o p -- "
                  "python3 bench.py --copy-calibration",
    "copy_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write_copy -o p -- "
                  "python3 bench.py --copy-calibration",
}
ATTN_KERNELS = ("attn_mfma64_kernel", "attn_combine_kernel")
COPY_BYTES = 256 << 20


def _csv_rows(folder, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(folder, "**", "*" + suffix), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit("no %s under %s" % (suffix, folder))
    return rows


_DEMANGLED = {}


def _demangle(name):
    """Itanium-demangled kernel name (binutils' c++filt, with the bf16 / fp16 builtin types
    spelled as vendor types it knows); the name itself when that fails."""
    if not name.startswith("_Z"):
        return name
    if name not in _DEMANGLED:
        import subprocess
        try:
            r = subprocess.run(["c++filt"], input=name.replace("DF16b", "u6__bf16").replace("DF16_", "u8_Float16"),
                               capture_output=True, text=True, timeout=10)
            _DEMANGLED[name] = r.stdout.strip() or name
        except (OSError, subprocess.SubprocessError):
            _DEMANGLED[name] = name
    return _DEMANGLED[name]


def _label(name):
    """Short kernel label: no return type, namespace or argument list."""
    import re
    n = _demangle(name).replace("void ", "").replace("sparsesam::", "")
    depth, out = 0, []
    for ch in n:  # cut the argument list (the first '(' at template depth 0)
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            break
        out.append(ch)
    return re.sub(r"\s+", " ", "".join(out)).strip()


def _counter_kib(folder, counter, match):
    """Average of `counter` (KiB per dispatch) over the dispatches whose kernel name contains match."""
    vals = [float(r["Counter_Value"]) for r in _csv_rows(folder, "counter_collection.csv")
            if r["Counter_Name"] == counter and match in r["Kernel_Name"]]
    if not vals:
        raise SystemExit("no %s dispatches of %s in %s" % (counter, match, folder))
    return sum(vals) / len(vals), len(vals)


def _per_kernel(folder, suffix, value):
    """{label: [values]} over the dispatches of a CSV (value(row) -> float or None)."""
    out = {}
    for r in _csv_rows(folder, suffix):
        v = value(r)
        if v is not None:
            out.setdefault(_label(r["Kernel_Name"]), []).append(v)
    return out


def _avg(v):
    return sum(v) / len(v)


def _write_trace(src, sub, name, what, key):
    durs = _per_kernel(os.path.join(src, sub), "kernel_trace.csv",
                       lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in durs.values())
    lines = ["# Kernel-trace statistics of %s." % what,
             "# command (from the repository root):",
             "#   " + PROFILE_COMMANDS[key],
             "# Durations in microseconds (per dispatch, from the kernel trace).",
             "%-78s %6s %10s %10s %10s %7s" % ("kernel", "calls", "avg_us", "min_us", "max_us", "pct")]
    for k, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        lines.append("%-78s %6d %10.2f %10.2f %10.2f %7.2f" % (k[:78], len(v), _avg(v), min(v), max(v),
                                                                100 * sum(v) / total))
    with open(os.path.join(ROOT, "profiles", name), "w") as f:
        f.write("\n".join(lines) + "\n")
    return durs


def _write_counters(src, cfgname, trace_sub, mfma_sub, fetch_sub, write_sub, keys, name, what, f_scale, w_scale):
    durs = _per_kernel(os.path.join(src, trace_sub), "kernel_trace.csv",
                       lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    def counter(sub, cname):
        return _per_kernel(os.path.join(src, sub), "counter_collection.csv",
                           lambda r: float(r["Counter_Value"]) if r["Counter_Name"] == cname else None)
    util = counter(mfma_sub, "MfmaUtil")
    mops = counter(mfma_sub, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    fetch = counter(fetch_sub, "FETCH_SIZE")
    write = counter(write_sub, "WRITE_SIZE")
    lines = ["# Hardware counters per kernel of %s." % what,
             "# commands (from the repository root):"]
    lines += ["#   " + PROFILE_COMMANDS[k] for k in keys + ("copy_fetch", "copy_write")]
    lines += ["# avg_us: kernel trace; mfma_util_pct: rocprofv3's MfmaUtil (MFMA-busy cycles over active",
              "# cycles of all SIMDs); mfma_tflops: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 FLOP / avg_us (executed",
              "# matrix-core work, bf16); hbm_mb: FETCH_SIZE x %.3f + WRITE_SIZE x %.3f (KiB per dispatch, each" % (
                  f_scale, w_scale),
              "# scaled by what it reads for a plain 256 MiB copy); gbs: hbm_mb / avg_us; pct_hbm: of 8 TB/s.",
              "%-70s %8s %8s %9s %9s %8s %7s" % ("kernel", "avg_us", "mfma%", "mfma_TF/s", "hbm_MB", "GB/s",
                                                "%hbm")]
    for k, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        us = _avg(v)
        u = _avg(util[k]) if k in util else float("nan")
        tf = _avg(mops[k]) * 512 / (us * 1e-6) / 1e12 if k in mops else float("nan")
        mb = ((_avg(fetch[k]) * f_scale if k in fetch else 0.0) + (_avg(write[k]) * w_scale if k in write else 0.0)) \
            * 1024 / 1e6
        gbs = mb * 1e6 / (us * 1e3)
        lines.append("%-70s %8.2f %8.1f %9.1f %9.2f %8.0f %7.1f" % (k[:70], us, u, tf, mb, gbs, 100 * gbs / 8000))
    with open(os.path.join(ROOT, "profiles", name), "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_profiles(src):
    """Turn the rocprofv3 output of PROFILE_COMMANDS (under src) into the text summaries in profiles/."""
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    c2 = ("the c2 step (SAM ViT-B global block, 64 x 64 tokens, C 768, 12 heads x 64, MLP 3072, density 0.4, "
          "batch 1: Sobel importance, permutation and keep-set, one SparseSAM block)")
    c3 = ("the c3 step (SAM ViT-B windowed block, 25 windows of 14 x 14 per image, batch 4, density 0.4: "
          "importance, permutation, one SparseSAM block)")
    _write_trace(src, "trace_c2", "c2_step_kernel_trace.txt", c2 + ", 20 timed + 5 warm-up steps", "trace")
    if os.path.isdir(os.path.join(src, "trace_relpos")):
        _write_trace(src, "trace_relpos", "c2_relpos_step_kernel_trace.txt",
                     c2 + " with the decomposed relative-position bias", "trace_relpos")
    if os.path.isdir(os.path.join(src, "trace_c3")):
        _write_trace(src, "trace_c3", "c3_step_kernel_trace.txt", c3, "trace_c3")
    if os.path.isdir(os.path.join(src, "trace_c4")):
        _write_trace(src, "trace_c4", "c4_encoder_kernel_trace.txt",
                     "the c4 encoder (SAM ViT-L shape, 24 blocks: 4 global on 64 x 64 tokens, 20 on 25 windows of "
                     "14 x 14 per image; C 1024, 16 heads x 64, MLP 4096, density 0.3, batch 8), 3 passes "
                     "(one untimed), one random-init layer's weights in every block", "trace_c4")
    if os.path.isdir(os.path.join(src, "trace_c5")):
        _write_trace(src, "trace_c5", "c5_encoder_kernel_trace.txt",
                     "the c5 encoder (SAM ViT-H shape, 32 blocks: 4 global on 64 x 64 tokens, 28 on 25 windows of "
                     "14 x 14 per image; C 1280, 16 heads x 80, MLP 5120, density 0.3, batch 16), 3 passes "
                     "(one untimed), one random-init layer's weights in every block", "trace_c5")
    # HBM byte counters are scaled by what they read for a plain copy of known size
    cf, _ = _counter_kib(os.path.join(src, "pmc_fetch_copy"), "FETCH_SIZE", "copyBuffer")
    cw, _ = _counter_kib(os.path.join(src, "pmc_write_copy"), "WRITE_SIZE", "copyBuffer")
    f_scale, w_scale = (COPY_BYTES / 1024) / cf, (COPY_BYTES / 1024) / cw
    if os.path.isdir(os.path.join(src, "pmc_mfma_c2")):
        _write_counters(src, "c2", "trace_c2", "pmc_mfma_c2", "pmc_fetch_c2", "pmc_write_c2",
                        ("trace", "mfma", "fetch", "write"), "c2_step_counters.txt", c2, f_scale, w_scale)
    if os.path.isdir(os.path.join(src, "pmc_mfma_c3")):
        _write_counters(src, "c3", "trace_c3", "pmc_mfma_c3", "pmc_fetch_c3", "pmc_write_c3",
                        ("trace_c3", "mfma_c3", "fetch_c3", "write_c3"), "c3_step_counters.txt", c3, f_scale,
                        w_scale)
    lines = ["# HBM traffic of one sparsesam_attn launch on the c2 workload (attention kernel, and the",
             "# combine of split rows when there are any), from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch,",
             "# separate passes), each scaled by the same counter on a plain 256 MiB device copy.",
             "# commands (from the repository root):"]
    lines += ["#   " + PROFILE_COMMANDS[k] for k in ("fetch", "write", "copy_fetch", "copy_write")]
    lines += ["copy_fetch_kib = %.1f" % cf, "copy_write_kib = %.1f" % cw,
              "fetch_scale = %.5f" % f_scale, "write_scale = %.5f" % w_scale]
    total = 0.0
    for kname in ATTN_KERNELS:
        try:
            fk, nf = _counter_kib(os.path.join(src, "pmc_fetch_c2"), "FETCH_SIZE", kname)
            wk, nw = _counter_kib(os.path.join(src, "pmc_write_c2"), "WRITE_SIZE", kname)
        except SystemExit:  # not launched at this workload (the combine runs only for split rows)
            lines.append("%s: no dispatches" % kname)
            continue
        b = (fk * f_scale + wk * w_scale) * 1024
        total += b
        lines += ["%s_fetch_kib = %.1f  # average of %d dispatches" % (kname, fk, nf),
                  "%s_write_kib = %.1f  # average of %d dispatches" % (kname, wk, nw),
                  "%s_scaled_bytes = %.0f" % (kname, b)]
    lines += ["scaled_bytes_per_launch = %.0f" % total,
              "source_sha256_16 = %s" % _source_hash(ATTN_SOURCE)]
    with open(TRAFFIC_PROFILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote the summaries under", out_dir)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-encoders", action="store_true", help="skip the c3 windowed block and c4 / c5 encoder runs")
    ap.add_argument("--profile-only", action="store_true", help="run the steps only (for rocprofv3)")
    ap.add_argument("--profile-encoder", metavar="KEY",
                    help="run passes of encoder KEY (c4 or c5) only (for rocprofv3)")
    ap.add_argument("--passes", type=int, default=2, help="timed passes of --profile-encoder")
    ap.add_argument("--rel-pos", action="store_true",
                    help="with --profile-only: steps of a plan with the relative-position bias")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 256 MiB device copy 5 times (scale factor for HBM byte counters)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/ summaries from the rocprofv3 output of the profiling commands in DIR")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (the data-parallel "
              "split is by image, with no communication; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from synth import get_config
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile_encoder:
        r = encoder_run(args.profile_encoder, dev, passes=args.passes)
        _log("%s encoder: %.3f ms per pass" % (args.profile_encoder, r["ms_per_pass"]))
        return
    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        _log("copied 256 MiB x 5")
        return
    cfg = get_config(args.config)
    _log("workload", cfg)
    if args.rel_pos and not args.profile_only:
        sys.exit("--rel-pos applies to --profile-only runs; the full run reports the bias under 'relpos'")
    wl = Workload(cfg, dev, rel_pos=args.rel_pos)

    # timed region: K full steps
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        wl.step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    _log("step %.4f ms (events), wall %.4f ms" % (ms, wall * 1e3 / args.steps))
    if args.profile_only:
        return

    # cold caches: 512 MiB written between steps (more than the L2s and the 256 MB
    # Infinity Cache hold), each step timed alone
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(max(5, args.steps // 2)):
        flush.zero_()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        wl.step()
        b.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del flush
    cold_ms = sorted(cold)[len(cold) // 2]
    _log("cold-cache step %.4f ms (median of %d)" % (cold_ms, len(cold)))

    ss = wl.ss
    plan = wl.plan
    tokens = cfg.batch * cfg.grid * cfg.grid
    # per-kernel: attention (dominant kernel) and routed MLP, same launch configuration as in the block
    q, k, vt, o = wl.attn_operands()
    segs = cfg.batch * plan.info["segments_per_image"]
    attn_ms = time_region(lambda: ss.attn(plan, q, k, vt, out=o, workspace=wl.attn_ws), 50, 5)
    attn_tf = attention_flops(plan) * segs / (attn_ms * 1e-3) / 1e12
    xr = wl.x.view(-1, cfg.channels)
    mlp_ms = time_region(lambda: ss.mlp(plan, xr, wl.routed, wl.w["ln2_g"], wl.w["ln2_b"], wl.w["w1"], wl.w["b1"],
                                        wl.w["w2"], wl.w["b2"], workspace=wl.mlp_ws), 50, 5)
    mlp_tf = mlp_flops(plan, cfg.batch) / (mlp_ms * 1e-3) / 1e12
    imp_ms = time_region(lambda: ss.importance(wl.img, cfg.patch, out=wl.imp), 50, 5)
    perm_ms = time_region(lambda: ss.permute(plan, wl.imp, out=(wl.perm, wl.inv, wl.routed)), 50, 5)
    block_ms = time_region(lambda: ss.block(plan, wl.w, wl.x, wl.perm, wl.routed, workspace=wl.ws), 50, 5)
    _log("attn %.4f ms (%.1f TFLOP/s), mlp %.4f ms (%.1f TFLOP/s), importance %.4f ms, permute %.4f ms, block %.4f ms"
         % (attn_ms, attn_tf, mlp_ms, mlp_tf, imp_ms, perm_ms, block_ms))

    extra = {}
    # the same workload at density 0.3
    cfg3 = cfg.with_(attn_density=0.3, mlp_density=0.3)
    wl3 = Workload(cfg3, dev)
    wl3.step()
    q3, k3, vt3, o3 = wl3.attn_operands()
    a3 = time_region(lambda: ss.attn(wl3.plan, q3, k3, vt3, out=o3, workspace=wl3.attn_ws), 50, 5)
    xr3 = wl3.x.view(-1, cfg.channels)
    m3 = time_region(lambda: ss.mlp(wl3.plan, xr3, wl3.routed, wl3.w["ln2_g"], wl3.w["ln2_b"], wl3.w["w1"],
                                    wl3.w["b1"], wl3.w["w2"], wl3.w["b2"], workspace=wl3.mlp_ws), 50, 5)
    s3 = time_region(wl3.step, 30, 5)
    extra["density_0.3"] = {
        "step_ms": round(s3, 5), "tokens_per_s": round(tokens / (s3 * 1e-3), 1),
        "realised_attn_density": wl3.plan.info["realised_density"],
        "attn_ms": round(a3, 5), "attn_tflops": round(attention_flops(wl3.plan) * segs / (a3 * 1e-3) / 1e12, 2),
        "mlp_ms": round(m3, 5), "mlp_tflops": round(mlp_flops(wl3.plan, cfg.batch) / (m3 * 1e-3) / 1e12, 2),
    }
    extra["density_0.3"]["attn_pct_peak"] = round(100 * extra["density_0.3"]["attn_tflops"] / PEAK_BF16_TFLOPS, 2)
    extra["density_0.3"]["mlp_pct_peak"] = round(100 * extra["density_0.3"]["mlp_tflops"] / PEAK_BF16_TFLOPS, 2)
    del wl3

    # the other token orders of the pages (Z-order, Hilbert curve, seeded random) ahead of the
    # same stripe-sort: the whole step and the permutation alone
    extra["orderings"] = {}
    for ordering in ("zorder", "hilbert", "random"):
        wlo = Workload(cfg.with_(ordering=ordering, order_seed=12345), dev)
        wlo.step()
        so = time_region(wlo.step, 30, 5)
        po = time_region(lambda: ss.permute(wlo.plan, wlo.imp, out=(wlo.perm, wlo.inv, wlo.routed)), 50, 5)
        extra["orderings"][ordering] = {"step_ms": round(so, 5), "tokens_per_s": round(tokens / (so * 1e-3), 1),
                                        "permute_ms": round(po, 5)}
        del wlo

    # SAM's decomposed relative-position bias: the step with a rel_pos plan, and the
    # attention with the bias (table kernel + attention) on the operands timed above
    wlr = Workload(cfg, dev, rel_pos=True)
    wlr.step()
    sr = time_region(wlr.step, 30, 5)
    ar = time_region(lambda: ss.attn_relpos(wlr.plan, q, k, vt, wlr.perm, wlr.w["rel_pos_h"], wlr.w["rel_pos_w"],
                                            out=o, workspace=wlr.relpos_ws), 50, 5)
    ar_tf = attention_flops(plan) * segs / (ar * 1e-3) / 1e12
    extra["relpos"] = {"step_ms": round(sr, 5), "tokens_per_s": round(tokens / (sr * 1e-3), 1),
                       "attn_ms": round(ar, 5), "attn_tflops": round(ar_tf, 2),
                       "attn_pct_peak": round(100 * ar_tf / PEAK_BF16_TFLOPS, 2),
                       "note": "attn_ms includes the bias-table kernel; TFLOP/s counts QK^T and PV only"}
    del wlr
    if not args.no_encoders:
        # the windowed block (c3, four images) with the bias
        cw = get_config("c3")
        wlw = Workload(cw, dev, rel_pos=True)
        wlw.step()
        bw = time_region(lambda: ss.block(wlw.plan, wlw.w, wlw.x, wlw.perm, wlw.routed, workspace=wlw.ws), 30, 5)
        extra["relpos"]["c3_window_block_ms"] = round(bw, 5)
        extra["relpos"]["c3_window_tokens_per_s"] = round(cw.batch * cw.grid * cw.grid / (bw * 1e-3), 1)
        del wlw
    _log("relative-position bias", extra["relpos"])

    if not args.no_dense:
        cfgd = cfg.with_(attn_density=1.0, mlp_density=1.0)
        wld = Workload(cfgd, dev)
        dense_lib = time_region(wld.step, 30, 5)
        # the block alone at density 1 (no importance and no permutation kernels): the
        # plain dense block that the sparse step replaces
        dense_block = time_region(
            lambda: ss.block(wld.plan, wld.w, wld.x, wld.perm, wld.routed, workspace=wld.ws), 30, 5)
        qd, kd, vtd, od = wld.attn_operands()
        dense_attn = time_region(lambda: ss.attn(wld.plan, qd, kd, vtd, out=od, workspace=wld.attn_ws), 30, 5)
        del wld
        dense_torch = torch_dense_block_ms(cfg, dev)
        best = min(dense_block, dense_torch)
        extra["dense"] = {"library_block_ms": round(dense_block, 5), "library_step_ms": round(dense_lib, 5),
                          "library_attn_ms": round(dense_attn, 5), "torch_eager_block_ms": round(dense_torch, 5),
                          "speedup_vs_faster_dense": round(best / ms, 3),
                          "speedup_vs_library_step": round(dense_lib / ms, 3),
                          "note": "speedup_vs_faster_dense: the sparse step (importance, permutation and "
                                  "block) against the faster dense block with no importance or permutation; "
                                  "speedup_vs_library_step: against the same three calls at density 1"}

    if not args.no_encoders:
        extra["c3_window_block"] = window_block_run(dev)
        _log("c3 windowed block", extra["c3_window_block"])
        extra["c1_block"] = tiny_block_run(dev)
        _log("c1 block", extra["c1_block"])
        enc = {}
        for key in ("c4", "c5"):
            enc[key] = {"sparse": encoder_run(key, dev), "density_1.0": encoder_run(key, dev, density=1.0),
                        "sparse_rel_pos": encoder_run(key, dev, rel_pos=True),
                        "sparse_sorted_stream": encoder_run(key, dev, sorted_stream=True)}
            if key == "c5":  # the ViT-H sweep's middle point
                enc[key]["density_0.4"] = encoder_run(key, dev, density=0.4)
                enc[key]["speedup_0.4_vs_density_1"] = round(enc[key]["density_1.0"]["ms_per_pass"] /
                                                             enc[key]["density_0.4"]["ms_per_pass"], 3)
            enc[key]["speedup_vs_density_1"] = round(enc[key]["density_1.0"]["ms_per_pass"] /
                                                     enc[key]["sparse"]["ms_per_pass"], 3)
            enc[key]["sorted_stream_vs_raster"] = round(enc[key]["sparse"]["ms_per_pass"] /
                                                        enc[key]["sparse_sorted_stream"]["ms_per_pass"], 3)
            _log("encoder", key, enc[key])
            torch.cuda.empty_cache()
        extra["encoders"] = enc

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg)
        _log("cpu baseline", cpu)

    line = {
        "metric": METRIC,
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "grid": cfg.grid, "channels": cfg.channels, "heads": cfg.heads,
                   "head_dim": cfg.head_dim, "mlp_hidden": cfg.mlp_hidden, "batch": cfg.batch,
                   "attn_density": cfg.attn_density, "mlp_density": cfg.mlp_density,
                   "realised_attn_density": plan.info["realised_density"],
                   "routed_tokens": plan.info["routed_per_image"] * cfg.batch},
        "roofline": {"bound": "mfma", "kernel": "sparsesam_attn (attn_mfma64_kernel)", "achieved": round(attn_tf, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(attn_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(), "launch_ms": round(attn_ms, 5),
                     "algorithmic_flop": attention_flops(plan) * segs},
        "cpu_baseline": cpu,
        "timing": {"warm_ms_per_step": round(ms, 5),
                   "cold_ms_per_step": round(cold_ms, 5),
                   "note": "warm: steps back to back (the ~30 MB working set stays in the L2s and the Infinity "
                           "Cache); cold: 512 MiB written before each step, median step"},
        "attn_tflops": round(attn_tf, 2),
        "attn_pct_peak": round(100 * attn_tf / PEAK_BF16_TFLOPS, 2),
        "mlp_tflops": round(mlp_tf, 2),
        "mlp_pct_peak": round(100 * mlp_tf / PEAK_BF16_TFLOPS, 2),
        "block_tflops": round(block_flops(plan, cfg.batch) / (block_ms * 1e-3) / 1e12, 2),
        "kernel_ms": {"importance": round(imp_ms, 5), "permute": round(perm_ms, 5), "block": round(block_ms, 5),
                      "attention": round(attn_ms, 5), "mlp": round(mlp_ms, 5)},
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
