#!/usr/bin/env python3
"""Benchmark of the video-DiT block hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input at the
75,600-token workload (21x45x80 latent grid, 40 heads x 128, bf16, batch 1):

  1. per-token AdaLN modulation of x [75600, 5120]   (vx_adaln_modulate)
  2. 3D RoPE on K (and on Q unless it is fused)      (vx_rope3d_apply)
  3. full non-causal flash attention                 (vx_flash_attn_fwd)

Inputs are generated on the host, copied to HBM once, and stay resident;
the timed region holds only the three launches per step.  The reported
value is attention TFLOP/s (4 N^2 d H per step) over the whole step time.
The dominant kernel (attention) is also timed alone with HIP events on the
stream it is launched on, and compared with the bf16 dense MFMA peak.

The CPU baseline times the fp64 oracle on a bounded sample of the same
workload (a few query rows, every head, every key) on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
MALL_BYTES = 256 * 2**20       # MI355X memory-side (Infinity) cache
METRIC = "flash-attn TFLOP/s + % bf16 MFMA peak at 75,600 tokens, 40 heads × d128"


# AdaLN variants: (x dtype, table dtype, per-sample tables); y is bf16.
ADALN_MODES = {
    "token": ("bf16", "bf16", False),          # Wan2.2: a table row per token
    "sample": ("bf16", "bf16", True),          # Wan2.1: a table row per sample
    "f32-residual": ("f32", "bf16", False),    # residual stream kept in fp32
    "f32-tables": ("bf16", "f32", False),      # modulation tables kept in fp32
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="large")
    p.add_argument("--dtype", choices=["workload", "f32"], default="workload",
                   help="workload: the workload's own storage type (bf16 except tiny); f32: the "
                        "same shapes with Q, K, V, x and the tables in fp32 (fp32 MFMA "
                        "attention, rated against the fp32 MFMA peak)")
    p.add_argument("--rope", choices=["fused", "separate"], default="fused",
                   help="fused: K rotated by vx_rope3d_apply, Q inside the attention load")
    p.add_argument("--adaln", choices=list(ADALN_MODES), default="token",
                   help="AdaLN variant in the step: table layout and storage types")
    p.add_argument("--pairing", type=int, choices=[0, 1, 2], default=None,
                   help="RoPE pairing override (0 adjacent, 1 head halves, 2 band halves)")
    p.add_argument("--kv-split", type=int, default=0,
                   help="run attention as two key parts [0, S) and [S, N) merged through their "
                        "LSEs (vx_flash_attn_fwd_kv twice + vx_attn_merge2); 0 = one call")
    p.add_argument("--cpu-rows", type=int, default=8192,
                   help="query rows of the oracle CPU baseline (0 = skip it)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB elementwise copy (HBM counter calibration)")
    return p.parse_args()


def attention_kernel_name(wl):
    if wl.dtype != "bf16":
        return f"fa_fwd_f32_mfma_kernel<{wl.head_dim}, false>"
    return f"fa_fwd_bf16_dma_kernel<{wl.head_dim}, false, false>"


def measured_traffic(wl, args, pairing):
    """HBM bytes per attention launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE record (scaled by the copy calibration), or None when the record
    is for another workload or launch (it was taken with one attention call, Q
    rotated on load, adjacent RoPE pairs) or the kernel source has changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attention_large_traffic.json")
    if (wl.name != "large" or wl.dtype != "bf16" or args.kv_split or args.rope != "fused"
            or pairing != 0 or not os.path.exists(path)):
        return None
    with open(path) as f:
        rec = json.load(f)
    with open(os.path.join(ROOT, rec["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
            return None
    return rec["bytes_per_launch"]


# Inputs of the CPU baseline, set before its worker processes are forked so
# that they inherit them (copy on write) instead of receiving copies.
_CPU_JOB = {}


def _oracle_head(h, rows=None):
    """Worker: the oracle on head h, every sampled query row (or `rows`)."""
    import threadpoolctl
    import oracle
    j = _CPU_JOB
    wl = j["wl"]
    rows = j["rows"] if rows is None else rows
    with threadpoolctl.threadpool_limits(1):
        oracle.attention_rope(j["q"][:, h:h + 1], j["k"][:, h:h + 1], j["v"][:, h:h + 1], wl.grid,
                              wl.split, wl.theta, wl.n_prefix, rows=rows,
                              pairing=j["pairing"])
    return rows.size


def _warm_worker(_):
    """Untimed: head 0 on the first 512 sampled rows (the oracle's row block,
    so every buffer size it allocates) in a fresh worker, which pays the page
    faults of its first calls; then wait until every worker holds one of these
    tasks, so that each worker takes exactly one."""
    _oracle_head(0, _CPU_JOB["rows"][:512])
    _CPU_JOB["barrier"].wait(timeout=600)
    return 0


def cpu_workers():
    """Host processes the CPU baseline uses: the thread budget the host sets for
    this job (OMP_NUM_THREADS) if any, else every core the OS reports."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    n = int(env) if env.isdigit() and int(env) > 0 else (os.cpu_count() or 1)
    return max(1, min(n, os.cpu_count() or 1))


def cpu_baseline(wl, q, k, v, rows_count, pairing=0):
    """The oracle, as it stands, on `rows_count` query rows x all heads x all keys.

    Heads are spread over a pool of forked worker processes, one per core of
    the host's budget, each with one BLAS thread; the oracle itself is
    unchanged.  Each worker first runs one head untimed (process start-up and
    first-touch page faults are not the oracle's rate).  Call it before this
    process initialises the GPU: the workers are forked from it."""
    import concurrent.futures as cf
    import multiprocessing as mp
    from spatiotemporal_attention_vx_amd import inputs
    rows = inputs.sample_rows(wl, count=rows_count)
    _CPU_JOB.update(q=inputs.values(q[0]), k=inputs.values(k[0]), v=inputs.values(v[0]), wl=wl,
                    rows=rows, pairing=pairing)
    workers = min(cpu_workers(), wl.heads)
    ctx = mp.get_context("fork")
    _CPU_JOB["barrier"] = ctx.Barrier(workers)
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        list(ex.map(_warm_worker, range(workers)))
        t0 = time.perf_counter()
        done = sum(ex.map(_oracle_head, range(wl.heads)))
        dt = time.perf_counter() - t0
    _CPU_JOB.clear()
    assert done == rows.size * wl.heads
    flops = 4.0 * rows.size * wl.n_tokens * wl.head_dim * wl.heads
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": workers,
            "kind": "oracle",
            "sample": (f"fp64 oracle, RoPE on Q and K then attention, {rows.size} seeded query "
                       f"rows x {wl.heads} heads x all {wl.n_tokens} keys of the same workload, "
                       f"heads spread over {workers} worker processes of one BLAS thread each; "
                       f"{dt:.1f} s wall, {flops / 1e9:.1f} GFLOP"),
            "seconds": dt,
            # the same oracle over every query row, extrapolated linearly in rows
            "full_workload_seconds_extrapolated": round(dt * wl.n_tokens / rows.size, 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(the path would shard heads across GPUs; no multi-GPU run is built)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from spatiotemporal_attention_vx_amd import binding, configs, inputs

    # device_count() does not initialise the GPU; the CPU baseline's workers are
    # forked below, before anything touches it
    if torch.cuda.device_count() < 1:
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = configs.get(args.workload)
    if args.dtype == "f32" and wl.dtype != "f32":
        import dataclasses
        wl = dataclasses.replace(wl, dtype="f32")
    pairing = wl.pairing if args.pairing is None else args.pairing

    # ---- inputs: host generation (seeded)
    t0 = time.perf_counter()
    q, k, v = inputs.attention_inputs(wl)
    x, sh, sc = inputs.adaln_inputs(wl) if args.adaln == "token" else (None, None, None)
    gen_s = time.perf_counter() - t0
    cpu = cpu_baseline(wl, q, k, v, args.cpu_rows, pairing) if args.cpu_rows > 0 else None

    # ---- the GPU from here on; inputs are copied to HBM once
    binding.load()
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    t0 = time.perf_counter()

    def up(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    def up_any(a):
        return up(a) if a.dtype == np.uint16 else torch.from_numpy(a).to(dev)

    tq, tk, tv = up_any(q), up_any(k), up_any(v)
    x_dt, m_dt, per_sample = ADALN_MODES[args.adaln]
    if args.adaln == "token":
        tx, tsh, tsc = up_any(x), up_any(sh), up_any(sc)
        ty = torch.empty_like(tx)
    else:
        x, sh, sc = inputs.adaln_inputs_ex(wl, x_dt, m_dt, per_sample)
        tx, tsh, tsc = up_any(x), up_any(sh), up_any(sc)
        ty = torch.empty(tx.shape, dtype=torch.bfloat16, device=dev)
    adaln_bytes = sum(t.numel() * t.element_size() for t in (tx, tsh, tsc, ty))
    to = torch.empty_like(tq)
    gen_s += time.perf_counter() - t0
    desc = binding.RopeDesc.of(wl.grid, wl.split, wl.theta, wl.n_prefix, pairing)
    fused = args.rope == "fused"
    stream = torch.cuda.current_stream()

    ev = {name: [] for name in ("adaln", "rope", "attn", "merge")}
    split = args.kv_split
    if split:
        if not 0 < split < wl.n_tokens or wl.batch != 1:
            raise SystemExit(f"--kv-split needs 0 < S < {wl.n_tokens} and batch 1")
        parts = [(torch.empty_like(tq), torch.empty((1, wl.heads, wl.n_tokens), device=dev))
                 for _ in range(2)]
        keys = [(tk[:, :split], tv[:, :split]), (tk[:, split:], tv[:, split:])]

    def attention():
        if not split:
            binding.flash_attn_fwd(tq, tk, tv, to, None, 0.0, desc if fused else None,
                                   stream=stream)
            return
        for (o_p, l_p), (k_p, v_p) in zip(parts, keys):
            binding.flash_attn_fwd_kv(tq, k_p, v_p, o_p, l_p, 0.0, desc if fused else None,
                                      stream=stream)

    def step(record):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if record else None
        if record:
            marks[0].record(stream)
        if args.adaln == "token":
            binding.adaln_modulate(tx, tsh, tsc, ty, wl.eps, stream=stream)
        else:
            binding.adaln_modulate_ex(tx, tsh, tsc, ty, wl.eps, stream=stream)
        if record:
            marks[1].record(stream)
        binding.rope3d_apply(None if fused else tq, tk, desc, stream=stream)
        if record:
            marks[2].record(stream)
        attention()
        if record:
            marks[3].record(stream)
        if split:
            (oa, la), (ob, lb) = parts
            binding.attn_merge2(oa, la, ob, lb, to, None, stream=stream)
        if record:
            marks[4].record(stream)
            ev["adaln"].append((marks[0], marks[1]))
            ev["rope"].append((marks[1], marks[2]))
            ev["attn"].append((marks[2], marks[3]))
            ev["merge"].append((marks[3], marks[4]))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # AdaLN and RoPE alone, 100 back-to-back launches each after 3 warm-ups,
    # each launch bracketed by HIP events on the same stream (RoPE rotates K
    # again on every launch: harmless for timing)
    def reps(fn, n=100):
        for _ in range(3):
            fn()
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(n)]
        for a_, b_ in pairs:
            a_.record(stream)
            fn()
            b_.record(stream)
        torch.cuda.synchronize()
        t = np.array([a_.elapsed_time(b_) for a_, b_ in pairs])
        return {"reps": n, "median_ms": round(float(np.median(t)), 4),
                "mean_ms": round(float(t.mean()), 4)}

    adaln_call = ((lambda: binding.adaln_modulate(tx, tsh, tsc, ty, wl.eps, stream=stream))
                  if args.adaln == "token" else
                  (lambda: binding.adaln_modulate_ex(tx, tsh, tsc, ty, wl.eps, stream=stream)))
    rep_adaln = reps(adaln_call)
    rep_rope = reps(lambda: binding.rope3d_apply(None if fused else tq, tk, desc, stream=stream))
    # Reference for AdaLN's access pattern on this GPU: torch's own elementwise
    # kernel streaming the same four tensors (three read, one written), timed
    # the same way.  Not part of the step.
    rep_stream = (reps(lambda: torch.addcmul(tsh, tx, tsc, out=ty))
                  if args.adaln == "token" else None)
    # and for RoPE's (K read and written in place; a multiply by one keeps the
    # bits), when only K is rotated in the step
    rep_rope_stream = reps(lambda: tk.mul_(1)) if fused else None

    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).normal_()
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)          # 1 GiB read + 1 GiB written, one elementwise kernel
        torch.cuda.synchronize()
        del src, dst

    ms = {kname: float(np.mean([a.elapsed_time(b) for a, b in pairs]))
          for kname, pairs in ev.items() if pairs}
    ms_step = wall * 1e3 / args.steps
    flops = wl.attn_flops()
    value = flops / (ms_step * 1e-3) / 1e12
    attn_tflops = flops / (ms["attn"] * 1e-3) / 1e12
    rope_bytes = wl.rope_bytes() / (1 if not fused else 2)     # fused: K only
    attn_all = [a_.elapsed_time(b_) for a_, b_ in ev["attn"]]
    kernels = {
        "attn_ms": round(ms["attn"], 4),
        "attn_ms_median": round(float(np.median(attn_all)), 4),
        "attn_tflops": round(attn_tflops, 2),
        "attn_exps": float(wl.n_tokens) ** 2 * wl.heads,
        "adaln_ms": round(ms["adaln"], 4),
        "adaln_mode": args.adaln,
        "adaln_bytes": adaln_bytes,
        "adaln_gbs": round(adaln_bytes / (ms["adaln"] * 1e-3) / 1e9, 1),
        "adaln_hbm_frac": round(adaln_bytes / (ms["adaln"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "rope_ms": round(ms["rope"], 4),
        "rope_tensors": "K" if fused else "Q,K",
        "rope_gbs": round(rope_bytes / (ms["rope"] * 1e-3) / 1e9, 1),
        "rope_hbm_frac": round(rope_bytes / (ms["rope"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
    }
    if adaln_bytes + rope_bytes < MALL_BYTES:
        kernels["note"] = ("AdaLN and RoPE tensors fit in the 256 MB memory-side cache together: "
                           "their GB/s is cache bandwidth, not HBM")
    kernels["adaln_100"] = dict(rep_adaln, hbm_frac=round(
        adaln_bytes / (rep_adaln["median_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
    if rep_stream is not None:
        kernels["adaln_pattern_reference"] = dict(
            rep_stream, hbm_frac=round(
                adaln_bytes / (rep_stream["median_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            what="torch.addcmul over the same x, shift, scale and y (3 reads + 1 write, bf16), "
                 "100 launches: plain elementwise streaming of AdaLN's bytes on this GPU")
    if rep_rope_stream is not None:
        k_bytes = 2 * tk.numel() * tk.element_size()       # all of K, read and written
        kernels["rope_pattern_reference"] = dict(
            rep_rope_stream, hbm_frac=round(
                k_bytes / (rep_rope_stream["median_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            what="torch.mul_(1) on K in place (1 read + 1 write, bf16), 100 launches: plain "
                 "elementwise streaming of RoPE's bytes on this GPU")
    kernels["rope_100"] = dict(rep_rope, hbm_frac=round(
        rope_bytes / (rep_rope["median_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
    if split:
        # o_a, o_b and both LSEs read, o written
        o_bytes = to.numel() * to.element_size()
        merge_bytes = 3 * o_bytes + 2 * parts[0][1].numel() * 4
        kernels.update({
            "kv_split": split,
            "merge_ms": round(ms["merge"], 4),
            "merge_gbs": round(merge_bytes / (ms["merge"] * 1e-3) / 1e9, 1),
            "merge_hbm_frac": round(merge_bytes / (ms["merge"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        })
    peak = PEAK_F32_TFLOPS if wl.dtype == "f32" else PEAK_BF16_TFLOPS
    record = {
        "metric": METRIC if wl.name == configs.BENCH_WORKLOAD and wl.dtype == "bf16" else
        (f"flash-attn TFLOP/s + % {'fp32' if wl.dtype == 'f32' else 'bf16'} MFMA peak at "
         f"{wl.n_tokens:,} tokens, "
         f"{wl.heads} heads × d{wl.head_dim}"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": (f"{wl.name}: {wl.grid[0]}x{wl.grid[1]}x{wl.grid[2]} latent grid"
                         + (f" + {wl.n_prefix} text tokens" if wl.n_prefix else "")
                         + f", {wl.n_tokens} tokens, {wl.heads} heads x {wl.head_dim}, "
                         f"{wl.dtype}, batch {wl.batch}"),
            "tokens": wl.n_tokens, "heads": wl.heads, "head_dim": wl.head_dim,
            "batch": wl.batch, "rope": args.rope, "rope_pairing": pairing,
            "step": (f"adaln [{wl.adaln_rows}, {wl.adaln_hidden}] + rope3d + flash attention fwd"
                     + (f"; one GPU's share of sequence parallelism over {wl.sp} GPUs "
                        f"(token shard for adaln, {wl.heads} of {wl.sp * wl.heads} heads "
                        f"for attention; all-to-alls not included)" if wl.sp > 1 else "")),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / peak, 4),
            "traffic": measured_traffic(wl, args, pairing),
            "kernel": attention_kernel_name(wl),
        },
        "kernels": kernels,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "gcn_arch": getattr(props, "gcnArchName", "")},
        "input_setup_s": round(gen_s, 2),
    }
    if cpu is not None:
        record["cpu_baseline"] = cpu
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
