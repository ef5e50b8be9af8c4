"""Benchmark: causal self-attention forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--no-cpu-baseline]

Workload (the one the headline metric is quoted on): B=2, H=32, S=32768, d=128,
bf16, causal, one attn_fwd_partial call (balanced schedule) and one attn_bwd
call per step.  A step is one forward + backward pass over one batch.
Throughput counts 4*S*S*d per (b, h) for the forward, halved for causal, and
2.5x that for the backward: 61.572 TFLOP per step.

Prints one JSON line.  Besides the contract fields it carries:
  roofline      the backward call (the dominant cost): algorithmic FLOPs per call
                over its average duration, timed with HIP events on the stream it
                runs on, against the 2.5 PFLOP/s dense bf16 MFMA peak;
  peak_on_device  the bf16 MFMA peak recomputed from rocminfo (compute units x 4096
                FLOP/clk x maximum shader clock), beside the published 2.5 PFLOP/s
                that the fractions use;
  kernels       per-call timings (forward call, backward call);
  device_state  socket power and shader clocks (amd-smi samples) over a window of
                the same steps after the timed ones, with that window's
                throughput: the MFMA kernels run at the chip's power limit, so
                their speed follows the clock it holds, which varies by box;
  secondary     the other workloads: the 128K sequence shard forward over 32
                chunks, its backward, split-KV GQA decode (GB/s of K/V, also
                as a fraction of a plain 1 GiB device copy's bandwidth), the
                fp32 workload, the packed variable-length batch and tree
                decode; each timed as the median of its calls (HIP events,
                at least 10 timed calls after 3 warm-up ones; 20 for decode,
                100 for the fp32 workload);
  cpu_baseline  the fp64 oracle, unmodified, on bounded samples of each workload
                on the host's cores (value: one full (batch, head) of the
                causal 32K workload, forward + backward), with the host's
                core count, CPU model and BLAS, and per-workload times with
                labelled linear extrapolations to the full sizes.
Inputs are seeded synthetic N(0,1) values generated on the device and rounded
to bf16; they are resident in HBM before timing starts.
"""

from __future__ import annotations

import argparse
import itertools
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
# HBM bytes per backward call of the causal 32K workload, from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE
# runs of its kernels (statistics + dK/dV + dQ), FETCH_SIZE scaled by 2 and WRITE_SIZE by 1 as a plain 1 GiB
# copy calibrates them (profiles/causal_fwdbwd_32k_hbm_traffic.md): 14.20 GB read + 2.79 GB written.  Set to
# None whenever these kernels change, until they are measured again.
BWD_CALL_HBM_BYTES = 16987541152
HBM_PEAK_GBS = 8000.0


def causal_flops(b, h, s, d):
    return 4.0 * s * s * d * b * h / 2.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["main", "shard_fwd", "shard_bwd", "decode", "fp32_small", "varlen", "tree", "copy"], default=None,
                    help="run a single workload (for profiling); 'copy' runs a plain 1 GiB device copy that "
                         "calibrates the HBM traffic counters")
    ap.add_argument("--schedule", choices=["balanced", "heaviest"], default="balanced",
                    help="work order of the headline workload's timed steps with --only main (for profiling the "
                         "causal work order; the default run always times the balanced order)")
    return ap.parse_args()


def randn_bf16(shape, gen):
    import torch

    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def time_calls(fns, steps, warmup, stream, stat="mean"):
    """Run each step's calls in order; returns per-call ms (the mean over the steps, or the median with
    stat="median") and the wall ms per step."""
    import torch

    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
          for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        for i, f in enumerate(fns):
            ev[s][i][0].record(stream)
            f()
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    times = [sorted(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)) for i in range(len(fns))]
    if stat == "median":
        per = [t[(steps - 1) // 2] if steps % 2 else 0.5 * (t[steps // 2 - 1] + t[steps // 2]) for t in times]
    else:
        per = [sum(t) / steps for t in times]
    return per, wall


def bench_main(args, stream):
    import torch

    from exact_blockwise_attention_attn_amd import shard

    B, H, S, D = 2, 32, 32768, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    q, k, v, do = (randn_bf16((B, S, H, D), g) for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dq_acc = torch.empty((B, S, H, D), dtype=torch.float32, device="cuda")
    ws = shard.bwd_workspace(B, H, S, "cuda")
    # The headline is the balanced order; --only main --schedule heaviest times the other order (profiling).
    bal = args.only is None or args.schedule == "balanced"

    def fwd():
        shard.causal_attention_forward(q, k, v, balanced=bal, o=o, lse=lse, stream=stream)

    def bwd():
        shard.causal_attention_backward(q, k, v, o, do, lse, balanced=bal, stream=stream, dq=dq, dk=dk, dv=dv,
                                        dq_acc=dq_acc, workspace=ws)

    (t_f, t_b), wall = time_calls([fwd, bwd], args.steps, args.warmup, stream)
    f_fwd = causal_flops(B, H, S, D)
    f_bwd = 2.5 * f_fwd
    res = {
        "B": B, "H": H, "S": S, "D": D, "schedule": "balanced" if bal else "heaviest_first", "fwd_ms": t_f, "bwd_ms": t_b, "step_ms": wall, "event_ms": t_f + t_b,
        "flops_step": f_fwd + f_bwd, "fwd_tflops": f_fwd / t_f / 1e9, "bwd_tflops": f_bwd / t_b / 1e9,
        "tflops": (f_fwd + f_bwd) / wall / 1e9,
    }
    if args.only is None:
        # The same calls without the balanced pairing (heaviest tiles first), timed after the
        # headline steps: the effect of balancing causal work across workgroups.
        def fwd_u():
            shard.causal_attention_forward(q, k, v, balanced=False, o=o, lse=lse, stream=stream)

        def bwd_u():
            shard.causal_attention_backward(q, k, v, o, do, lse, balanced=False, stream=stream, dq=dq, dk=dk, dv=dv,
                                            dq_acc=dq_acc, workspace=ws)

        (t_fu, t_bu), _ = time_calls([fwd_u, bwd_u], max(2, args.steps // 3), 1, stream)
        res["unbalanced"] = {"fwd_ms": t_fu, "bwd_ms": t_bu}
        # The chip's socket power and shader clocks under the same steps, in a window of their own
        # after the timed ones: the MFMA rates follow the clock the chip holds at its power limit,
        # which differs from box to box.
        res["device_state"] = sustained_device_state([fwd, bwd], f_fwd + f_bwd, stream)
    return res


def parse_smi_metric_csv(text):
    """(socket power W, [shader clock MHz of each XCD]) of every data row of `amd-smi metric -p -c --csv`."""
    rows, header = [], None
    for line in text.splitlines():
        cells = [c.strip() for c in line.split(",")]
        if not line.strip():
            continue
        if cells[0] == "gpu":
            header = cells
            continue
        if header is None or len(cells) != len(header):
            continue
        rec = dict(zip(header, cells))
        try:
            power = float(rec["socket_power"])
        except (KeyError, ValueError):
            continue
        clocks = []
        for name, val in rec.items():
            parts = name.split("_")
            if len(parts) == 3 and parts[0] == "gfx" and parts[2] == "clk":
                try:
                    clocks.append(float(val))
                except ValueError:
                    pass
        rows.append((power, clocks))
    return rows


def sustained_device_state(fns, flops_step, stream, seconds=4.0):
    """Repeat the step for `seconds` while `amd-smi` samples socket power and shader clocks
    (None if amd-smi is not available); also the throughput over the same window."""
    import shutil
    import subprocess
    import threading

    import torch

    smi = shutil.which("amd-smi")
    if smi is None:
        return None
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                out = subprocess.run([smi, "metric", "-p", "-c", "--csv"], capture_output=True, text=True,
                                     timeout=10).stdout
            except (OSError, subprocess.SubprocessError):
                return
            samples.extend(parse_smi_metric_csv(out))
            stop.wait(0.25)

    th = threading.Thread(target=sampler, daemon=True)
    torch.cuda.synchronize()
    th.start()
    t0, steps = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for f in fns:
            f()
        torch.cuda.synchronize()
        steps += 1
    elapsed = time.perf_counter() - t0
    stop.set()
    th.join(timeout=15)
    # The first sample can predate the load; keep those taken under it (above half the busiest power).
    busy = [x for x in samples if samples and x[0] > 0.5 * max(p for p, _ in samples)]
    if not busy:
        return None
    power = sorted(p for p, _ in busy)
    clocks = sorted(c for _, cs in busy for c in cs)

    def stats(v):
        return {"min": v[0], "median": v[len(v) // 2], "max": v[-1]}

    return {"samples": len(busy), "window_s": round(elapsed, 2), "steps": steps,
            "tflops": round(flops_step * steps / elapsed / 1e12, 1), "socket_power_w": stats(power),
            "shader_clock_mhz": stats(clocks) if clocks else None}


def bench_shard(args, stream, do_bwd):
    import torch

    from exact_blockwise_attention_attn_amd import binding, shard

    H, D, SQ, SK, CH, QP = 32, 128, 4096, 131072, 4096, 65536
    g = torch.Generator(device="cuda")
    g.manual_seed(2)
    q = randn_bf16((1, SQ, H, D), g)
    k = randn_bf16((1, SK, H, D), g)
    v = randn_bf16((1, SK, H, D), g)
    o_run = torch.empty((1, SQ, H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, H, SQ), dtype=torch.float32, device="cuda")
    o = torch.empty((1, SQ, H, D), dtype=torch.bfloat16, device="cuda")

    def fwd():
        shard.shard_forward(q, k, v, CH, q_pos0=QP, causal=True, stream=stream, o_run=o_run, lse=lse, o_out=o)

    def fwd_fused():
        shard.shard_forward_fused(q, k, v, CH, q_pos0=QP, causal=True, stream=stream, lse=lse, o_out=o)

    # The partials-then-merge form: 17 live chunks into stacked fp32 partials, then one merge call.
    live = [(a, a + CH) for a in range(0, SK, CH) if a <= QP + SQ - 1]
    o_parts = torch.empty((len(live), 1, SQ, H, D), dtype=torch.float32, device="cuda")
    lse_parts = torch.empty((len(live), 1, H, SQ), dtype=torch.float32, device="cuda")

    def partials():
        for i, (a, e) in enumerate(live):
            binding.attn_fwd_partial(q, k[:, a:e], v[:, a:e], o_parts[i], lse_parts[i], q_pos0=QP, k_pos0=a,
                                     causal=True, stream=stream)

    def merge():
        binding.attn_merge_lse(o_parts, lse_parts, o, lse, stream=stream)

    f_fwd = 4.0 * SQ * SK * D * H / 2.0  # the stated convention: halved for causal
    if not do_bwd:
        (t, tf, tp, tm), _ = time_calls([fwd, fwd_fused, partials, merge], max(10, args.steps), 3, stream,
                                        stat="median")
        # The headline figure is the chunk loop as one call over the chunk table (attn_fwd_chunks); the
        # chained per-chunk calls and the partials-then-merge form are reported beside it.
        return {"workload": "shard_fwd_128k", "method": "attn_fwd_chunks over the 32-chunk table", "ms": tf,
                "tflops": f_fwd / tf / 1e9, "frac_mfma": f_fwd / tf / 1e9 / MFMA_BF16_PEAK_TFLOPS, "chunks": 32,
                "live_chunks": len(live),
                "chained_accumulate": {"ms": t, "tflops": f_fwd / t / 1e9,
                                       "frac_mfma": f_fwd / t / 1e9 / MFMA_BF16_PEAK_TFLOPS},
                "partials_then_merge": {"partials_ms": tp, "merge_ms": tm, "merge_gbs":
                                        (len(live) + 0.5) * SQ * H * D * 4 / tm / 1e6}}
    fwd()
    do = randn_bf16((1, SQ, H, D), g)
    dq = torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    dq_acc = torch.empty((1, SQ, H, D), dtype=torch.float32, device="cuda")
    ws = shard.bwd_workspace(1, H, SQ, "cuda")

    def bwd():
        shard.shard_backward(q, k, v, o, do, lse, CH, q_pos0=QP, causal=True, stream=stream, dq=dq, dk=dk, dv=dv,
                             dq_acc=dq_acc, workspace=ws)

    def bwd_fused():
        shard.shard_backward_fused(q, k, v, o, do, lse, CH, q_pos0=QP, causal=True, stream=stream, dq=dq, dk=dk,
                                   dv=dv, dq_acc=dq_acc, workspace=ws)

    (t, tf), _ = time_calls([bwd, bwd_fused], max(10, args.steps), 3, stream, stat="median")
    f_bwd = 2.5 * f_fwd
    return {"workload": "shard_bwd_128k", "method": "attn_bwd_chunks over the 32-chunk table", "ms": tf,
            "tflops": f_bwd / tf / 1e9, "frac_mfma": f_bwd / tf / 1e9 / MFMA_BF16_PEAK_TFLOPS,
            "chained_calls": {"ms": t, "tflops": f_bwd / t / 1e9,
                              "frac_mfma": f_bwd / t / 1e9 / MFMA_BF16_PEAK_TFLOPS}}


def bench_fp32_small(args, stream):
    """The fp32 workload (Q, K, V [256, 64], four chunks of 64, non-causal): latency of the chunk loops."""
    import torch

    from exact_blockwise_attention_attn_amd import shard

    S, D, CH = 256, 64, 64
    g = torch.Generator(device="cuda")
    g.manual_seed(6)
    q, k, v, do = (torch.randn((1, S, 1, D), generator=g, device="cuda", dtype=torch.float32) for _ in range(4))
    o = torch.empty_like(q)  # the fp32 running result is the output
    lse = torch.empty((1, 1, S), dtype=torch.float32, device="cuda")

    def fwd():
        shard.shard_forward(q, k, v, CH, stream=stream, o_run=o, lse=lse)

    fwd()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dq_acc = torch.empty((1, S, 1, D), dtype=torch.float32, device="cuda")
    ws = shard.bwd_workspace(1, 1, S, "cuda")

    def bwd():
        shard.shard_backward(q, k, v, o, do, lse, CH, stream=stream, dq=dq, dk=dk, dv=dv, dq_acc=dq_acc, workspace=ws)

    (tf, tb), _ = time_calls([fwd, bwd], 100, 10, stream, stat="median")
    return {"workload": "fp32_s256_4chunks", "fwd_us": tf * 1e3, "bwd_us": tb * 1e3,
            "note": "4 chained chunk calls each way; latency-bound, no roofline"}


def bench_varlen(args, stream):
    """Packed variable-length batch: 16 causal sequences of 512 k tokens (k = 1..16), H = 32, d = 128, bf16."""
    import torch

    from exact_blockwise_attention_attn_amd import binding
    from seeded_inputs import VARLEN_PACKED as W

    H, D = W["H"], W["D"]
    lens = [W["unit"] * k for k in W["k"]]
    cu = torch.tensor([0] + list(itertools.accumulate(lens)), dtype=torch.int32, device="cuda")
    T, mx = sum(lens), max(lens)
    g = torch.Generator(device="cuda")
    g.manual_seed(8)
    q, k, v, do = (randn_bf16((T, H, D), g) for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dq_acc = torch.empty((T, H, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(binding.attn_bwd_workspace_size(len(lens), H, mx), dtype=torch.uint8, device="cuda")

    def fwd():
        binding.attn_fwd_varlen(q, k, v, o, lse, cu, cu, mx, mx, causal=True, balanced=True, stream=stream)

    def bwd():
        binding.attn_bwd_varlen(q, k, v, o, do, lse, ws, dq_acc, dk, dv, cu, cu, mx, mx, dq=dq, causal=True,
                                compute_delta=True, dq_overwrite=True, finalize_dq=True, balanced=True, stream=stream)

    (tf, tb), _ = time_calls([fwd, bwd], max(10, args.steps), 3, stream, stat="median")
    f_fwd = sum(causal_flops(1, H, L, D) for L in lens)
    f_bwd = 2.5 * f_fwd
    return {"workload": "varlen_packed_70k", "sequences": len(lens), "tokens": T, "fwd_ms": tf, "bwd_ms": tb,
            "tflops": (f_fwd + f_bwd) / (tf + tb) / 1e9,
            "frac_mfma": (f_fwd + f_bwd) / (tf + tb) / 1e9 / MFMA_BF16_PEAK_TFLOPS,
            "fwd_tflops": f_fwd / tf / 1e9, "bwd_tflops": f_bwd / tb / 1e9}


def bench_tree_decode(args, stream):
    """Tree-structured decode (64 queries under one 32K-token root, 8 children of 4K, 8 leaves of 512 each)
    against split-KV decode of the same queries over their materialised per-query caches."""
    import torch

    from exact_blockwise_attention_attn_amd import binding
    from seeded_inputs import TREE_DECODE as T
    from seeded_inputs import tree_nodes

    nodes = tree_nodes(T)
    nq = T["children"] * T["leaves"]
    L = T["root"] + T["children"] * (T["child_len"] + T["leaves"] * T["leaf_len"])
    Hq, Hkv, D = T["H_q"], T["H_kv"], T["D"]
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    q = randn_bf16((nq, Hq, D), g)
    kc, vc = randn_bf16((L, Hkv, D), g), randn_bf16((L, Hkv, D), g)
    ks, kl, qb, qe = zip(*nodes)
    o = torch.empty((nq, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((nq, Hq), dtype=torch.float32, device="cuda")
    need = binding.attn_decode_tree_workspace_size(q, kc, kv_start=ks, kv_len=kl, q_begin=qb, q_end=qe)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def tree():
        binding.attn_decode_tree(q, kc, vc, o, lse, ws, kv_start=ks, kv_len=kl, q_begin=qb, q_end=qe, stream=stream)

    # The same queries over materialised caches: each query's path keys copied out (not timed).
    path = T["root"] + T["child_len"] + T["leaf_len"]
    rows = []
    for i in range(nq):
        rows.append(torch.cat([torch.arange(s, s + n) for s, n, b, e in nodes if b <= i < e]))
    idx = torch.stack(rows).cuda()
    kp, vp = kc[idx], vc[idx]  # [nq, path, Hkv, D]
    o2, l2 = torch.empty_like(o), torch.empty_like(lse)
    ns = 16
    ws2 = torch.empty(binding.attn_decode_workspace_size(nq, Hq, D, ns), dtype=torch.uint8, device="cuda")

    def flat():
        binding.attn_decode_splitkv(q, kp, vp, o2, l2, ws2, n_splits=ns, stream=stream)

    (tt, tf), _ = time_calls([tree, flat], max(20, args.steps), 3, stream, stat="median")
    uniq = 2.0 * L * Hkv * D * 2
    flat_bytes = 2.0 * nq * path * Hkv * D * 2
    return {"workload": "tree_decode_64q", "queries": nq, "nodes": len(nodes), "tree_ms": tt,
            "unique_kv_bytes": uniq, "unique_gbs": uniq / tt / 1e6, "frac_hbm_unique": uniq / tt / 1e6 / HBM_PEAK_GBS,
            "flat_splitkv_ms": tf, "flat_kv_bytes": flat_bytes, "speedup_vs_flat": tf / tt}


def bench_decode(args, stream):
    import torch

    from exact_blockwise_attention_attn_amd import binding

    B, HQ, HKV, L, D, NS = 16, 32, 8, 131072, 128, 64
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    q = randn_bf16((B, HQ, D), g)
    kc = randn_bf16((B, L, HKV, D), g)
    vc = randn_bf16((B, L, HKV, D), g)
    o = torch.empty((B, HQ, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, HQ), dtype=torch.float32, device="cuda")
    ws = torch.empty(binding.attn_decode_workspace_size(B, HQ, D, NS), dtype=torch.uint8, device="cuda")

    def dec():
        binding.attn_decode_splitkv(q, kc, vc, o, lse, ws, n_splits=NS, stream=stream)

    # The same cache with uneven lengths (8K k tokens for k = 1..16, shuffled): whether fixed splits
    # per sequence keep the HBM rate when the work per sequence differs 16-fold.
    lens = [8192 * k for k in (5, 12, 1, 16, 9, 3, 14, 7, 11, 2, 15, 6, 10, 4, 13, 8)]
    seqlens = torch.tensor(lens, dtype=torch.int32, device="cuda")

    def dec_uneven():
        binding.attn_decode_splitkv(q, kc, vc, o, lse, ws, n_splits=NS, seqlens=seqlens, stream=stream)

    (t, tu), _ = time_calls([dec, dec_uneven], max(20, args.steps), 3, stream, stat="median")
    kv_bytes = 2.0 * B * L * HKV * D * 2
    gbs = kv_bytes / t / 1e6
    u_bytes = 2.0 * sum(lens) * HKV * D * 2
    # The achievable bandwidth beside the 8 TB/s specification: a plain 1 GiB device-to-device
    # copy (the runtime's copy kernel), counting the bytes read and written.
    src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    (tc,), _ = time_calls([lambda: dst.copy_(src)], 10, 3, stream)
    copy_gbs = 2.0 * src.numel() * 2 / tc / 1e6
    del src, dst
    return {"workload": "decode_gqa_128k", "ms": t, "kv_bytes": kv_bytes, "gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
            "copy_gbs": copy_gbs, "frac_of_copy": gbs / copy_gbs,
            "uneven_lengths": {"ms": tu, "kv_bytes": u_bytes, "gbs": u_bytes / tu / 1e6,
                               "frac_hbm": u_bytes / tu / 1e6 / HBM_PEAK_GBS,
                               "frac_of_copy": u_bytes / tu / 1e6 / copy_gbs}}


def _device_peak():
    """The bf16 MFMA peak recomputed from the device: compute units x 4096 FLOP/clk x the maximum
    shader clock, both read from rocminfo (None when it is not available)."""
    import re
    import subprocess

    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for agent in out.split("Agent ")[1:]:
        if "gfx950" not in agent:
            continue
        cu = re.search(r"Compute Unit:\s+(\d+)", agent)
        mhz = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", agent)
        if cu and mhz:
            cus, clk = int(cu.group(1)), int(mhz.group(1))
            return {"compute_units": cus, "max_sclk_mhz": clk, "mfma_bf16_tflops": cus * 4096 * clk / 1e6}
    return None


def _host_facts():
    facts = {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": None, "blas": []}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    facts["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info

        facts["blas"] = [{"api": i.get("internal_api"), "version": i.get("version"), "threads": i.get("num_threads")}
                         for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:  # noqa: BLE001
        pass
    return facts


def cpu_baseline():
    """The fp64 oracle, as it stands, timed on bounded samples of each workload on the host's cores.

    Inputs are seeded N(0,1) rounded to bf16 (fp32 for the fp32 workload), the
    shapes and positions of each workload's sample; generation is not timed.
    Full-size times are linear extrapolations from the sample (per head, per
    sampled row, or per (batch, key/value head)) and are labelled as such.
    """
    import numpy as np

    import oracle
    from seeded_inputs import bf16_bits_to_f32, normal_f32
    from seeded_inputs.gen import normal_bf16_bits

    facts = _host_facts()
    threads = max([b["threads"] or 0 for b in facts["blas"]] or [0]) or facts["affinity_cores"]
    gen = lambda wid, t, s, d: bf16_bits_to_f32(normal_bf16_bits(wid, t, 0, (s, 1, d))[:, 0]).astype(np.float64)  # noqa: E731
    configs = {}

    def timed(f):
        t0 = time.perf_counter()
        r = f()
        return r, time.perf_counter() - t0

    # Causal self-attention, 32K (the headline workload): one (batch, head) in full, fwd + bwd.
    S, D = 32768, 128
    q, k, v, do = (gen(5, t, S, D) for t in range(4))
    c = 1 / math.sqrt(D)
    (O, L), tf = timed(lambda: oracle.attention_head(q, k, v, c, True))
    _, tb = timed(lambda: oracle.attention_backward_head(q, k, v, O, do, L, c, True))
    per_head = 3.5 * causal_flops(1, 1, S, D)
    configs["causal_fwdbwd_32k"] = {
        "sample": "one (batch, head) of 64, S=32768, forward + backward", "fwd_s": round(tf, 2), "bwd_s": round(tb, 2),
        "tflops": per_head / (tf + tb) / 1e12, "full_s_extrapolated": round(64 * (tf + tb), 1)}
    del q, k, v, do, O, L

    # 128K shard forward: 256 sampled query rows of one head (rows 0-127 and 3968-4095 at positions
    # 65536 + i) against the keys up to the shard's last position; backward: one head in full.
    SQ, QP = 4096, 65536
    last = QP + SQ
    q, do = gen(2, 0, SQ, D), gen(2, 3, SQ, D)
    k, v = gen(2, 1, last, D), gen(2, 2, last, D)
    rows = np.r_[0:128, SQ - 128:SQ]
    t_rows = 0.0
    for a in (0, SQ - 128):
        _, t = timed(lambda: oracle.attention_head(q[a:a + 128], k, v, c, True, QP + a, 0))
        t_rows += t
    shard_flops = 4.0 * SQ * 131072 * D * 32 / 2
    full_fwd = t_rows / len(rows) * SQ * 32
    configs["shard_fwd_128k"] = {"sample": "256 query rows of one head of 32", "sample_s": round(t_rows, 2),
                                 "full_s_extrapolated": round(full_fwd, 1),
                                 "tflops_extrapolated": shard_flops / full_fwd / 1e12}
    (O, L), _ = timed(lambda: oracle.attention_head(q, k, v, c, True, QP, 0))
    _, tb = timed(lambda: oracle.attention_backward_head(q, k, v, O, do, L, c, True, QP, 0))
    configs["shard_bwd_128k"] = {"sample": "one head of 32 in full (backward from the saved O and LSE)",
                                 "sample_s": round(tb, 2), "full_s_extrapolated": round(32 * tb, 1),
                                 "tflops_extrapolated": 2.5 * shard_flops / (32 * tb) / 1e12}
    del q, k, v, do, O, L

    # Split-KV decode with GQA: one (sequence, key/value head) slice: 4 query heads over 131072 keys.
    L4 = 131072
    qd = bf16_bits_to_f32(normal_bf16_bits(4, 0, 0, (1, 4, D))).astype(np.float64)
    kd, vd = gen(4, 1, L4, D)[None, :, None], gen(4, 2, L4, D)[None, :, None]
    _, t = timed(lambda: oracle.decode(qd, kd, vd, c))
    kv_bytes = 2.0 * 16 * L4 * 8 * D * 2
    configs["decode_gqa_128k"] = {"sample": "one (sequence, key/value head) of 16 x 8", "sample_s": round(t, 3),
                                  "full_s_extrapolated": round(128 * t, 2),
                                  "gbs_extrapolated": kv_bytes / (128 * t) / 1e9}

    # fp32 workload in full: 4 chunk partials merged, then the backward per chunk from the merged result.
    S1, D1 = 256, 64
    x = [normal_f32(1, t, 0, (S1, 1, D1))[:, 0].astype(np.float64) for t in range(4)]
    c1 = 1 / math.sqrt(D1)

    def fp32_all():
        parts = [oracle.attention_head(x[0], x[1][a:a + 64], x[2][a:a + 64], c1, False) for a in range(0, S1, 64)]
        Om, Lm = oracle.merge(parts)
        for a in range(0, S1, 64):
            oracle.attention_backward_head(x[0], x[1][a:a + 64], x[2][a:a + 64], Om, x[3], Lm, c1, False)

    _, t = timed(fp32_all)
    configs["fp32_s256_4chunks"] = {"sample": "the whole workload", "s": round(t, 4)}

    head = configs["causal_fwdbwd_32k"]
    return {"value": head["tflops"], "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one (batch, head) of the causal 32K workload (S=32768, d=128), forward + backward, fp64 NumPy: "
                      f"{head['fwd_s'] + head['bwd_s']:.1f} s for {per_head / 1e12:.3f} TFLOP (same FLOP convention); "
                      f"the full 64 (batch, head) pairs would take {head['full_s_extrapolated']:.0f} s (linear "
                      f"extrapolation)",
            "host": facts, "configs": configs}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch

    from exact_blockwise_attention_attn_amd import binding

    binding.load(build_if_missing=False)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    if args.only == "shard_fwd":
        print(json.dumps(bench_shard(args, stream, False)), flush=True)
        return
    if args.only == "shard_bwd":
        print(json.dumps(bench_shard(args, stream, True)), flush=True)
        return
    if args.only == "decode":
        print(json.dumps(bench_decode(args, stream)), flush=True)
        return
    if args.only == "fp32_small":
        print(json.dumps(bench_fp32_small(args, stream)), flush=True)
        return
    if args.only == "varlen":
        print(json.dumps(bench_varlen(args, stream)), flush=True)
        return
    if args.only == "tree":
        print(json.dumps(bench_tree_decode(args, stream)), flush=True)
        return
    if args.only == "copy":
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 2, "copies": 3}), flush=True)
        return

    m = bench_main(args, stream)
    print(f"# main: fwd {m['fwd_ms']:.2f} ms ({m['fwd_tflops']:.0f} TF/s), bwd {m['bwd_ms']:.2f} ms "
          f"({m['bwd_tflops']:.0f} TF/s)", file=sys.stderr, flush=True)
    secondary = {}
    if not args.no_secondary and args.only is None:
        torch.cuda.empty_cache()
        secondary["shard_fwd_128k"] = bench_shard(args, stream, False)
        torch.cuda.empty_cache()
        secondary["shard_bwd_128k"] = bench_shard(args, stream, True)
        torch.cuda.empty_cache()
        secondary["decode_gqa_128k"] = bench_decode(args, stream)
        torch.cuda.empty_cache()
        secondary["fp32_s256_4chunks"] = bench_fp32_small(args, stream)
        secondary["varlen_packed_70k"] = bench_varlen(args, stream)
        torch.cuda.empty_cache()
        secondary["tree_decode_64q"] = bench_tree_decode(args, stream)
        torch.cuda.empty_cache()
    cpu = None if (args.no_cpu_baseline or args.only) else cpu_baseline()
    bwd_achieved = m["bwd_tflops"]
    line = {
        "metric": "attention TFLOP/s fwd+bwd (causal, d=128, bf16)",
        "value": round(m["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["step_ms"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal_fwdbwd_32k", "batch": m["B"], "heads": m["H"], "seq_len": m["S"],
                   "head_dim": m["D"], "causal": True, "schedule": m["schedule"], "parallelism": "single GPU"},
        "frac_of_mfma_peak": round(m["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
        "peak_on_device": _device_peak(),
        "roofline": {"bound": "mfma", "kernel": "attn_bwd call (statistics + dK/dV + dQ kernels)",
                     "achieved": round(bwd_achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(bwd_achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": BWD_CALL_HBM_BYTES},
        "device_state": m.get("device_state"),
        "kernels": {"fwd_call_ms": round(m["fwd_ms"], 3), "bwd_call_ms": round(m["bwd_ms"], 3),
                    "fwd_tflops": round(m["fwd_tflops"], 2), "bwd_tflops": round(m["bwd_tflops"], 2),
                    "event_ms_per_step": round(m["event_ms"], 3),
                    **({"unbalanced_fwd_call_ms": round(m["unbalanced"]["fwd_ms"], 3),
                        "unbalanced_bwd_call_ms": round(m["unbalanced"]["bwd_ms"], 3)} if "unbalanced" in m else {})},
        "secondary": secondary,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
