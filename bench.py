#!/usr/bin/env python3
"""Benchmark of the deterministic GQA attention path on one MI355X.

Timed workload (one "step"): fused causal prefill, B=4, S=4096, Hq=32, Hkv=8,
D=128, 128-key blocks, bf16 output, inputs resident in HBM.  `value` is prefill
TFLOP/s with the algorithmic flop count 4*D*Hq*B*S*(S+1)/2 (QK^T and PV over
unmasked pairs only).  The same JSON line also reports:

* roofline: the prefill kernel's average launch duration from HIP events on
  the stream it runs on, against the dense bf16 MFMA peak;
* decode: paged-KV decode over 64 sequences (lengths U[512, 16384], page 16,
  1M-slot pool) as KV-read GB/s against the HBM peak, with the last-level
  caches flushed between repetitions;
* invariance: max abs drift of a sequence alone vs in the batch and of a
  CP=2 emit+merge (reversed arrival) vs the fused result (must be 0.0);
* cpu_baseline: the FP64 CPU oracle timed on a bounded sample of the same
  workload on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from deterministic_gqa_attention_amd import inputs as gen  # noqa: E402

METRIC = "prefill TFLOP/s & paged-decode KV GB/s (% of peak) at 0.0 invariance drift"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(q, k, v, cfg, seconds):
    """Time the FP64 oracle on a seeded sample of query rows (all heads)."""
    import oracle

    rng = np.random.Generator(np.random.PCG64(1000 * cfg.cfg_id + 99))
    S = cfg.S

    def flops(rows):
        return float(sum(4.0 * cfg.D * cfg.Hq * ((int(r) % S) + 1) for r in rows))

    probe = rng.integers(0, cfg.B * S, 16)
    t0 = time.perf_counter()
    oracle.attention(q, k, v, scale=cfg.softmax_scale, rows=probe)
    rate = flops(probe) / max(time.perf_counter() - t0, 1e-6)
    mean_row = 4.0 * cfg.D * cfg.Hq * (S + 1) / 2.0
    n = int(max(16, min(cfg.B * S, seconds * rate / mean_row)))
    rows = rng.integers(0, cfg.B * S, n)
    t0 = time.perf_counter()
    oracle.attention(q, k, v, scale=cfg.softmax_scale, rows=rows)
    dt = time.perf_counter() - t0
    return {"value": flops(rows) / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.oracle_threads(), "kind": "oracle",
            "sample": f"{n} seeded query rows x all {cfg.Hq} heads of the B={cfg.B} S={S} causal prefill "
                      f"({flops(rows):.3e} flop, {dt:.1f} s, FP64)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=10)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only", choices=["prefill", "decode", "copy"], default=None,
                    help="run one leg only (for profiler and counter runs)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} (WORLD_SIZE={world}) is not supported: "
              "the attention path runs on a single device and nothing is sharded across GPUs.", file=sys.stderr)
        sys.exit(2)

    if args.only == "copy":
        copy_calibration(args)
        return
    if args.only == "decode":
        args.no_cpu_baseline = True

    cfg = gen.CFG2
    log("generating prefill inputs")
    q, k, v = gen.prefill_inputs(cfg)
    dcfg = gen.CFG4
    d = None
    if not args.no_decode and args.only != "prefill":
        log("generating paged-decode inputs")
        d = gen.decode_inputs(dcfg)

    base = None
    if not args.no_cpu_baseline and args.only is None:
        log(f"timing the CPU oracle for ~{args.cpu_seconds:.0f} s")
        base = cpu_baseline(q, k, v, cfg, args.cpu_seconds)
        log(f"cpu baseline {base['value'] * 1e3:.2f} GFLOP/s on {base['cores']} threads")

    import torch

    from deterministic_gqa_attention_amd import api

    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    qd, kd, vd = up(q), up(k), up(v)
    stream = torch.cuda.current_stream(dev)
    flops = cfg.flops()

    if args.only == "decode":
        args.steps = 0
    log("prefill warmup")
    for _ in range(args.warmup if args.steps else 0):
        api.prefill(qd, kd, vd, block=cfg.block)
    torch.cuda.synchronize()

    # timed region: K back-to-back steps, events per launch on the launch stream
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    out = None
    torch.cuda.synchronize()
    t_begin.record(stream)
    for i in range(args.steps):
        starts[i].record(stream)
        out = api.prefill(qd, kd, vd, block=cfg.block)
        ends[i].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    if args.steps:
        total_ms = t_begin.elapsed_time(t_end)
        launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
        ms_per_step = total_ms / args.steps
        kern_ms = float(np.mean(launch_ms))
        tflops = flops / (ms_per_step * 1e-3) / 1e12
        achieved = flops / (kern_ms * 1e-3) / 1e12
        log(f"prefill {ms_per_step:.3f} ms/step, kernel {kern_ms:.3f} ms, {tflops:.1f} TFLOP/s")
    else:
        total_ms = ms_per_step = kern_ms = tflops = achieved = float("nan")
    if args.only == "prefill":
        print(json.dumps({"only": "prefill", "ms_per_step": ms_per_step, "kernel_ms": kern_ms, "tflops": tflops}))
        return

    drift_batch = drift_cp = None
    if args.only is None:
        drift_batch, drift_cp = invariance_probe(api, cfg, qd, kd, vd, out, dev)
        log(f"invariance drift: batch {drift_batch}, CP=2 reversed {drift_cp}")
    del qd, kd, vd, out
    torch.cuda.empty_cache()
    decode = decode_leg(args, api, d, dcfg, up, dev, stream) if d is not None else None
    if args.only == "decode":
        print(json.dumps({"only": "decode", "decode": decode}))
        return

    line = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "fused causal prefill B=4 S=4096 Hq=32 Hkv=8 D=128, 128-key blocks, bf16 in/out, "
                               "fp32 accumulate", "global_batch": cfg.B, "seq_len": cfg.S, "parallelism": "none",
                   "flop_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel_ms": round(kern_ms, 4)},
        "decode": decode,
        "invariance": {"batch_alone_vs_batch": drift_batch, "cp2_reversed_arrival": drift_cp},
        "cpu_baseline": base,
    }
    print(json.dumps(line), flush=True)


def invariance_probe(api, cfg, qd, kd, vd, out, dev):
    """Untimed: a sequence alone vs in the batch, and CP=2 emit+merge with
    reversed arrival on the last 512 query rows; returns the max abs drifts."""
    import torch

    fo, fl = out
    so, sl = api.prefill(qd[1:2].contiguous(), kd[1:2].contiguous(), vd[1:2].contiguous(), block=cfg.block)
    drift_batch = max((so[0].float() - fo[1].float()).abs().max().item(),
                      (sl[0] - fl[1]).abs().max().item())
    q0, qn = cfg.S - 512, 512
    arrival = list(range(cfg.n_blocks))[::-1]
    po = torch.empty((cfg.n_blocks, cfg.B * qn, cfg.Hq, cfg.D), dtype=torch.float32, device=dev)
    pl = torch.empty((cfg.n_blocks, cfg.B * qn, cfg.Hq), dtype=torch.float32, device=dev)
    for shard in cfg.shards:
        lo = arrival.index(max(shard))
        api.emit_partials(qd, kd, vd, sorted(shard, reverse=True), block=cfg.block, q_begin=q0, q_count=qn,
                          part_out=po[lo:lo + len(shard)], part_lse=pl[lo:lo + len(shard)])
    mo, ml = api.merge_states(po, pl, arrival)
    mo = mo.view(cfg.B, qn, cfg.Hq, cfg.D)
    ml = ml.view(cfg.B, qn, cfg.Hq)
    drift_cp = max((mo.float() - fo[:, q0:].float()).abs().max().item(), (ml - fl[:, q0:]).abs().max().item())
    del po, pl
    torch.cuda.empty_cache()
    return drift_batch, drift_cp


def decode_leg(args, api, d, dcfg, up, dev, stream):
    """Paged decode over the 64-sequence workload; caches flushed before each
    timed repetition.  Returns the decode record of the JSON line."""
    import torch

    log("decode setup")
    kp, vp = up(d["k_pool"]), up(d["v_pool"])
    qq = up(d["q"])
    table = torch.from_numpy(d["page_table"]).to(dev)
    lens = torch.from_numpy(d["ctx_lens"]).to(dev)
    host_lens = d["ctx_lens"]
    max_ctx = dcfg.len_hi
    ws = torch.empty((api.decode_workspace_bytes(dcfg.Hq, dcfg.Hkv, dcfg.batch, max_ctx, block=dcfg.block),),
                     dtype=torch.uint8, device=dev)
    flush = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)  # > 256 MB last-level cache
    kv_bytes = gen.decode_kv_bytes(host_lens, dcfg.Hkv, dcfg.D)
    used_pages = int((-(-host_lens.astype(np.int64) // dcfg.page_size)).sum())
    other = dcfg.batch * dcfg.Hq * dcfg.D * 2 * 2 + dcfg.batch * dcfg.Hq * 4 + used_pages * 4 + dcfg.batch * 4
    alg_bytes = kv_bytes + other
    for _ in range(2):
        api.decode_paged(qq, kp, vp, table, lens, block=dcfg.block, max_context_len=max_ctx,
                         host_ctx_lens=host_lens, workspace=ws)
    times = []
    for _ in range(args.decode_steps):
        flush.fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        api.decode_paged(qq, kp, vp, table, lens, block=dcfg.block, max_context_len=max_ctx,
                         host_ctx_lens=host_lens, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    dms = float(np.median(times))
    gbs = kv_bytes / (dms * 1e-3) / 1e9
    ach = alg_bytes / (dms * 1e-3) / 1e9
    decode = {"value": round(gbs, 1), "unit": "GB/s", "ms": round(dms, 4), "kv_bytes": kv_bytes,
              "workload": "paged decode, 64 seqs, len U[512,16384] (sum %d), Hq=32 Hkv=8 D=128, page 16, "
                          "1M-slot pool, 128-key blocks, bf16 out" % int(host_lens.sum()),
              "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None}}
    log(f"decode {dms:.3f} ms, {gbs:.0f} GB/s KV")
    return decode


def copy_calibration(args):
    """A plain device copy of known size (1 GiB read + 1 GiB written per
    dispatch), used to scale the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = 1 << 30
    src = torch.ones((n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(max(1, args.warmup)):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(max(1, args.steps)):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / max(1, args.steps)
    print(json.dumps({"only": "copy", "bytes_read": n, "bytes_written": n, "ms": ms,
                      "GBps": 2 * n / (ms * 1e-3) / 1e9}))


if __name__ == "__main__":
    main()
