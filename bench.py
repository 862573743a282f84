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
import csv
import glob
import hashlib
import json
import os
import re
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


PROFILES = os.path.join(ROOT, "profiles")
PREFILL_PROFILE = os.path.join(PROFILES, "prefill_kernel_b4_s4096.md")
DECODE_PROFILE = os.path.join(PROFILES, "decode_paged_64seq.md")
BACKWARD_PROFILE = os.path.join(PROFILES, "backward_b4_s4096.md")
LM_HEAD_PROFILE = os.path.join(PROFILES, "lm_head_logprobs_t64_v151936.md")
TIMED_STEPS = 20  # --steps of the prefill profiling commands below
BACKWARD_TIMED_STEPS = 10  # --steps of the backward trace command
LM_HEAD_TIMED_REPS = 5  # timed calls of the lm_head leg
TRACE_CMD = {
    "lm_head": "rocprofv3 --kernel-trace --stats -d rocprof_out/prof_lm_head -o run --output-format csv -- "
               "python3 bench.py --only lm_head",
    "backward": "rocprofv3 --kernel-trace --stats -d rocprof_out/prof_backward -o run --output-format csv -- "
                "python3 bench.py --only backward --steps 10",
    "prefill": "rocprofv3 --kernel-trace --stats -d rocprof_out/prof_prefill -o run --output-format csv -- "
               "python3 bench.py --only prefill --steps 20",
    "decode": "rocprofv3 --kernel-trace --stats -d rocprof_out/prof_decode -o run --output-format csv -- "
              "python3 bench.py --only decode --decode-steps 10 --decode-write-only-ref 0",
}
PMC_CMD = ("rocprofv3 --pmc {c} -d rocprof_out/pmc_{c}_{m} -o run --output-format csv -- "
           "python3 bench.py --only {m} --steps 2 --warmup 1 --decode-steps 2 --decode-write-only-ref 0")
PMC_CMD_LM_HEAD = ("rocprofv3 --pmc {c} -d rocprof_out/pmc_{c}_lm_head -o run --output-format csv -- "
                   "python3 bench.py --only lm_head")
PMC_CMD_MFMA = ("rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA "
                "SQ_WAVE_CYCLES -d rocprof_out/pmc_mfma_prefill -o run --output-format csv -- "
                "python3 bench.py --only prefill --steps 20")
PMC_CMD_BACKWARD = ("rocprofv3 --pmc {c} -d rocprof_out/pmc_{c}_backward -o run --output-format csv -- "
                    "python3 bench.py --only backward --steps 2")


SETTLE_MS = 100.0  # untimed dense work before a reported leg's timing


def settle(fn, ms=SETTLE_MS, cap=4096):
    """Run fn, untimed, until about `ms` milliseconds of wall time have passed
    (at least once).  After an idle spell the GPU comes back at a high clock,
    overshoots its power budget and is throttled for the next few tens of
    milliseconds of dense work before it settles; timing that starts at once
    measures the transient (prefill B=4 S=4096: 0.675 ms per launch for the
    20 launches after 3 warm-ups, 0.565-0.59 ms from about the 50th launch on,
    0.69 ms again after 2 s idle)."""
    import torch

    t0 = time.perf_counter()
    for n in range(cap):
        fn()
        if n % 4 == 3 or n == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= ms * 1e-3:
                break
    torch.cuda.synchronize()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """SHA-256 over the HIP sources: counter-derived traffic is used only while
    the kernels are the ones the counters were taken on."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "deterministic_gqa_attention_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def sha256_of(a) -> str:
    """SHA-256 of a generated buffer's bytes (numpy stream stability across
    versions is not guaranteed, so the record names exactly what was used)."""
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def git_commit():
    """The commit of this tree when it is a git checkout (a copy without .git
    gives None)."""
    try:
        import subprocess
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        return r.stdout.strip() or None if r.returncode == 0 else None
    except Exception:
        return None


def shard_manifest(cfg):
    """The logical blocks of the emulated context-parallel shards of a prefill
    workload: per logical CP rank, each owned global_block_index with its key
    range, and the SHA-256 of that manifest (the block metadata hash of a
    drift report)."""
    ranks = []
    for r, blocks in enumerate(cfg.shards):
        ranks.append({"cp_rank": r, "blocks": [[int(b), int(b) * cfg.block, min(cfg.S, (int(b) + 1) * cfg.block)]
                                               for b in blocks]})
    text = json.dumps({"block": cfg.block, "S": cfg.S, "ranks": ranks}, sort_keys=True)
    return {"kv_block_size": cfg.block, "n_blocks": cfg.n_blocks,
            "ranks": [{"cp_rank": r["cp_rank"], "n_blocks": len(r["blocks"]),
                       "key_ranges": _ranges([b[0] for b in r["blocks"]], cfg.block, cfg.S)} for r in ranks],
            "sha256": hashlib.sha256(text.encode()).hexdigest()}


def _ranges(blocks, block, S):
    """Contiguous key ranges [lo, hi) covered by a sorted block list."""
    out = []
    for b in sorted(blocks):
        lo, hi = b * block, min(S, (b + 1) * block)
        if out and out[-1][1] == lo:
            out[-1][1] = hi
        else:
            out.append([lo, hi])
    return out


def profile_traffic(path):
    """HBM bytes per launch recorded in a profile summary, if it was taken on
    the current kernel sources; else None."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel source sha256: `([0-9a-f]+)`", text)
    m_bytes = re.search(r"traffic bytes per launch: `([0-9]+)`", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return int(m_bytes.group(1))


def cpu_baseline(q, k, v, cfg, seconds):
    """Time the FP64 oracle on a seeded sample of query rows (all heads) of a
    causal prefill workload."""
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


def decode_cpu_baseline(d, dcfg):
    """Time the FP64 oracle on the whole paged-decode workload (every sequence
    and head; its 8.9e9 flop take seconds), as KV bytes scanned per second."""
    import oracle
    lens = d["ctx_lens"]
    kv = gen.decode_kv_bytes(lens, dcfg.Hkv, dcfg.D)
    t0 = time.perf_counter()
    oracle.decode_paged(d["q"], d["k_pool"], d["v_pool"], d["page_table"], lens, scale=dcfg.softmax_scale)
    dt = time.perf_counter() - t0
    return {"value": round(kv / dt / 1e9, 3), "unit": "GB/s", "cores": oracle.oracle_threads(), "kind": "oracle",
            "sample": f"all {lens.size} sequences x {dcfg.Hq} heads of the paged-decode workload "
                      f"({kv:.3e} KV bytes, {dt:.2f} s, FP64)"}


def reported_legs(api, up, stream, cpu_seconds=None):
    """Reported (not the headline value): the long-context prefill (B=1,
    S=32768, Q and K drawn x4) and the chunked-prefill replay of 8192 tokens
    in chunks of 2048, 512 and 1.  TFLOP/s from the algorithmic flops of a
    whole prefill / replay over the wall time of the launches (events on the
    launch stream)."""
    import torch

    def timed(fn, reps):
        settle(fn)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    res = {}
    cfg5 = gen.CFG5
    log("long-context prefill (S=32768)")
    q, k, v = gen.prefill_inputs(cfg5)
    qd, kd, vd = up(q), up(k), up(v)
    sha = {"q": sha256_of(q), "k": sha256_of(k), "v": sha256_of(v)}
    cpu5 = None
    if cpu_seconds:
        log(f"timing the CPU oracle on the S=32768 workload for ~{cpu_seconds:.0f} s")
        cpu5 = cpu_baseline(q, k, v, cfg5, cpu_seconds)
    del q, k, v
    ms = timed(lambda: api.prefill(qd, kd, vd, block=cfg5.block), 3)
    res["long_prefill_b1_s32768"] = {"tflops": round(cfg5.flops() / (ms * 1e-3) / 1e12, 2), "ms": round(ms, 4),
                                     "frac_of_peak": round(cfg5.flops() / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                     "input_sha256": sha, "cp_shards": shard_manifest(cfg5),
                                     "cpu_baseline": cpu5}
    del qd, kd, vd
    torch.cuda.empty_cache()
    cfg3 = gen.CFG3
    q, k, v = gen.prefill_inputs(cfg3)
    qd, kd, vd = up(q), up(k), up(v)
    del q, k, v
    # one workspace for the chunk-of-one route, sized for the longest call
    ws1 = api.alloc_workspace(api.decode_workspace_bytes(cfg3.Hq, cfg3.Hkv, cfg3.B, cfg3.S, block=cfg3.block),
                              qd.device)
    for chunk in (2048, 512, 1):
        log(f"chunked replay, chunk {chunk}")
        parts = [(qd[:, c0:c0 + chunk].contiguous(), c0) for c0 in range(0, cfg3.S, chunk)]

        def replay():
            for qc, c0 in parts:
                api.prefill_chunked(qc, kd, vd, cache_len=c0, block=cfg3.block, workspace=ws1)

        ms = timed(replay, 1 if chunk == 1 else 3)
        res[f"chunked_replay_s8192_c{chunk}"] = {"tflops": round(cfg3.flops() / (ms * 1e-3) / 1e12, 2),
                                                 "ms": round(ms, 4), "calls": len(parts)}
        if chunk == 1:
            # launch-bound (two launches per call): the same replay captured once
            # into a HIP graph, its last outputs checked against the eager ones
            log("chunked replay, chunk 1, as one HIP graph")
            ref = api.prefill_chunked(parts[-1][0], kd, vd, cache_len=parts[-1][1], block=cfg3.block, workspace=ws1)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                outs = [api.prefill_chunked(qc, kd, vd, cache_len=c0, block=cfg3.block, workspace=ws1)
                        for qc, c0 in parts]
            msg = timed(graph.replay, 3)
            same = bool(torch.equal(outs[-1][0].view(torch.int16), ref[0].view(torch.int16)) and
                        torch.equal(outs[-1][1].view(torch.int32), ref[1].view(torch.int32)))
            res["chunked_replay_s8192_c1_graph"] = {"tflops": round(cfg3.flops() / (msg * 1e-3) / 1e12, 2),
                                                    "ms": round(msg, 4), "calls": len(parts),
                                                    "bitwise_equal_to_eager": same}
            del graph, outs, ref
        del parts
    # the same replay (chunks of 2048) with the keys in a paged pool of 16-key pages
    P = 16
    npp = cfg3.S // P
    perm = np.random.Generator(np.random.PCG64(1000 * cfg3.cfg_id + 5)).permutation(npp)
    table = torch.from_numpy(perm.astype(np.int32).reshape(1, npp)).to(qd.device)
    inv = torch.from_numpy(np.argsort(perm)).to(qd.device)  # pool slot p holds logical page inv[p]
    kp = kd[0].reshape(npp, P, cfg3.Hkv, cfg3.D).transpose(1, 2)[inv].contiguous()
    vp = vd[0].reshape(npp, P, cfg3.Hkv, cfg3.D).transpose(1, 2)[inv].contiguous()
    parts = [(qd[:, c0:c0 + 2048].contiguous(), c0) for c0 in range(0, cfg3.S, 2048)]

    def paged_replay():
        for qc, c0 in parts:
            api.prefill_paged(qc, kp, vp, table, cache_len=c0, block=cfg3.block)

    log("paged chunked replay, chunk 2048")
    ms = timed(paged_replay, 3)
    res["paged_replay_s8192_c2048_p16"] = {"tflops": round(cfg3.flops() / (ms * 1e-3) / 1e12, 2), "ms": round(ms, 4),
                                            "calls": len(parts)}
    del parts, kp, vp, qd, kd, vd, ws1
    torch.cuda.empty_cache()
    return res


def backward_leg(api, cfg, qd, kd, vd, up, stream, steps, cpu_q=None):
    """Backward (dQ, dK, dV) of the same causal prefill: the dQ and dK/dV
    launches timed together with events on the launch stream.  Algorithmic
    flops: the five products QK^T, dOut V^T, P^T dOut, dS^T Q, dS K over the
    unmasked pairs, 2.5x the forward's."""
    import torch
    do = up(gen.dout_inputs(cfg))
    out, lse = api.prefill(qd, kd, vd, block=cfg.block)
    dq = torch.empty(qd.shape, dtype=torch.float32, device=qd.device)
    dk = torch.zeros(kd.shape, dtype=torch.float32, device=qd.device)
    dv = torch.zeros(kd.shape, dtype=torch.float32, device=qd.device)

    ws = api.alloc_workspace(api.backward_workspace_bytes(cfg.Hq, cfg.Hkv, cfg.B, cfg.S), qd.device)

    def call():
        api.backward(qd, kd, vd, out, lse, do, scale=cfg.softmax_scale, dq=dq, dk=dk, dv=dv, workspace=ws)

    settle(call)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 2.5 * cfg.flops()
    del do, out, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    res = {"tflops": round(flops / (ms * 1e-3) / 1e12, 2), "ms": round(ms, 4),
           "frac_of_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "flop_per_step": flops,
           "workload": "backward of causal prefill B=4 S=4096 Hq=32 Hkv=8 D=128, bf16 in, fp32 dQ/dK/dV"}
    if cpu_q is not None:
        res["cpu_baseline"] = backward_cpu_baseline(cfg, *cpu_q)
    return res


def backward_cpu_baseline(cfg, q, k, v, do, seconds=10.0, probe_rows=48):
    """The FP64 oracle's backward on a seeded sample of query rows of the same
    workload (their complete dQ and their dK/dV terms), in algorithmic flops:
    10*D per visible (row, key) pair and q head.  A 48-row probe sizes the
    timed sample to about `seconds` of host work."""
    import oracle

    def sample(n):
        rng = np.random.Generator(np.random.PCG64(77))
        return np.unique(rng.integers(0, cfg.B * cfg.S, n))

    t0 = time.perf_counter()
    oracle.attention_backward(q, k, v, do, scale=cfg.softmax_scale, rows=sample(probe_rows))
    per_row = (time.perf_counter() - t0) / probe_rows
    rows = sample(int(min(cfg.B * cfg.S, max(probe_rows, seconds / max(per_row, 1e-6)))))
    t = rows % cfg.S
    flops = float(np.sum(10.0 * cfg.D * cfg.Hq * (t + 1)))
    t0 = time.perf_counter()
    oracle.attention_backward(q, k, v, do, scale=cfg.softmax_scale, rows=rows)
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.oracle_threads(),
            "kind": "oracle", "sample": f"{rows.size} seeded query rows x all {cfg.Hq} heads of the B=4 S=4096 "
                                        f"backward ({flops:.3e} flop, {dt:.1f} s, FP64)"}


PEAK_FP32_TFLOPS = 157.3   # MI355X dense fp32 MFMA (published)


def lm_head_leg(api, up, stream, reps=5, cpu=False):
    """Selected log-probs of 64 active tokens (one per decode sequence, the
    attention output of all 32 heads: H = 4096) through a synthetic FP32
    lm_head over Qwen3-8B's 151936-token vocabulary: one pass over W (2.49 GB)
    with 2*T*V*H flops of FP32 MFMA work."""
    import torch
    T, H, V = 64, 4096, gen.LM_VOCAB
    log("generating the synthetic lm_head (151936 x 4096 fp32)")
    w_host = gen.lm_head_weights(V, H)
    w = torch.from_numpy(w_host).to(stream.device)
    x = up(gen.draw_bf16(1000 * 4 + 11, (T, H)))
    tok = torch.from_numpy(gen.lm_tokens(T, V)).to(stream.device)
    ws = api.alloc_workspace(api.lm_head_workspace_bytes(T, V), stream.device)
    settle(lambda: api.lm_head_logprobs(x, w, tok, workspace=ws))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        api.lm_head_logprobs(x, w, tok, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 2.0 * T * V * H
    wbytes = V * H * 4
    del w, tok, ws
    torch.cuda.empty_cache()
    res = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
           "frac_of_fp32_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4),
           "w_gbs": round(wbytes / (ms * 1e-3) / 1e9, 1),
           "workload": "selected log-probs, 64 tokens x H=4096 bf16 through an fp32 lm_head of 151936 rows"}
    if cpu:
        import oracle
        n = T  # every token: about 3 s of host work
        xs = x[:n].view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        oracle.lm_head_logprobs(xs, w_host, gen.lm_tokens(T, V)[:n])
        dt = time.perf_counter() - t0
        f = 2.0 * n * V * H
        res["cpu_baseline"] = {"value": round(f / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.oracle_threads(),
                               "kind": "oracle", "sample": f"all {n} tokens over the full vocabulary "
                                                           f"({f:.3e} flop, {dt:.1f} s, FP64)"}
    del x
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed prefill launches first (~60 ms: the clock settles after idle)")
    ap.add_argument("--decode-steps", type=int, default=25)
    ap.add_argument("--decode-write-only-ref", type=int, default=1,
                    help="also time each decode rep after a write-only flush (0: skip, for profiling)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-reported", action="store_true", help="skip the long-context and chunked-replay legs")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--only", choices=["prefill", "decode", "copy", "backward", "lm_head"], default=None,
                    help="run one leg only (for profiler and counter runs)")
    ap.add_argument("--summarize", metavar="DIR", default=None,
                    help="write profiles/*.md from the rocprofv3 CSVs under DIR (no GPU work)")
    ap.add_argument("--profile-commands", action="store_true",
                    help="print the rocprofv3 commands whose output --summarize reads, one per line")
    args = ap.parse_args()
    if args.profile_commands:
        print("\n".join(profile_commands()))
        return
    if args.summarize:
        summarize_profiles(args.summarize)
        return
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
    if not args.no_decode and args.only in (None, "decode"):
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

    if args.only == "lm_head":
        print(json.dumps({"only": "lm_head", "lm_head": lm_head_leg(api, up, stream)}))
        return
    if args.only == "backward":
        log("backward")
        print(json.dumps({"only": "backward", "backward": backward_leg(api, cfg, qd, kd, vd, up, stream,
                                                                       max(args.steps, 1))}))
        return
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
    backward = None
    if args.only is None:
        log("backward")
        backward = backward_leg(api, cfg, qd, kd, vd, up, stream, 10,
                                cpu_q=None if args.no_cpu_baseline else (q, k, v, gen.dout_inputs(cfg)))
        log(f"backward {backward['ms']:.3f} ms, {backward['tflops']:.1f} TFLOP/s")
    del qd, kd, vd, out
    torch.cuda.empty_cache()
    decode = decode_leg(args, api, d, dcfg, up, dev, stream) if d is not None else None
    if decode is not None and not args.no_cpu_baseline and args.only is None:
        log("timing the CPU oracle on the paged-decode workload")
        decode["cpu_baseline"] = decode_cpu_baseline(d, dcfg)
        decode["input_sha256"] = {name: sha256_of(d[name]) for name in ("q", "k_pool", "v_pool", "page_table",
                                                                         "ctx_lens")}
    if args.only == "decode":
        print(json.dumps({"only": "decode", "decode": decode}))
        return
    reported = None if args.no_reported else reported_legs(
        api, up, stream, cpu_seconds=None if args.no_cpu_baseline else min(args.cpu_seconds, 15.0))
    lm_head = None
    if not args.no_reported:
        lm_head = lm_head_leg(api, up, stream, cpu=not args.no_cpu_baseline)
        log(f"lm_head {lm_head['ms']:.3f} ms, {lm_head['tflops']:.1f} TFLOP/s fp32")

    line = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "fused causal prefill B=4 S=4096 Hq=32 Hkv=8 D=128, 128-key blocks, bf16 in/out, "
                               "fp32 accumulate", "global_batch": cfg.B, "seq_len": cfg.S, "parallelism": "none",
                   "flop_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": profile_traffic(PREFILL_PROFILE),
                     "kernel_ms": round(kern_ms, 4)},
        "decode": decode,
        "backward": backward,
        "lm_head_logprobs": lm_head,
        "invariance": {"batch_alone_vs_batch": drift_batch, "cp2_reversed_arrival": drift_cp,
                       "max_abs_drift": None if drift_batch is None else max(drift_batch, drift_cp)},
        "provenance": {
            "core_id": api.core_id(), "commit": git_commit(), "kernel_source_sha256": kernel_source_hash(),
            "merge_order": "global_block_index", "downcast_at": "final_write", "acc_dtype": "fp32",
            "split_kv": "fixed 128-key blocks counted from position 0; no data-dependent split (decode: fixed "
                        "4-block units, per-block states folded in ascending block index)",
            "fallback": False,
            "input_sha256": {"q": sha256_of(q), "k": sha256_of(k), "v": sha256_of(v)},
            "cp_shards": shard_manifest(cfg),
            "tolerances": {"bf16_out": "|g-o| <= 2e-2 + 1e-2*|o|", "fp32_out_abs": 1e-4, "lse_abs": 1e-4,
                           "invariance_max_abs": 0.0},
        },
        "reported": reported,
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
    # Cache flush before each timed call: 1 GiB written, then 1 GiB read, both
    # far above the 256 MB last-level cache, so no KV byte of the previous call
    # is served from cache.  The read also drains the dirty lines the write
    # leaves behind; after a write alone their write-back to HBM lands inside
    # the timed call (measured: write only 521 us, write + read 458 us, read
    # only 459 us, no flush 483 us per call), which is traffic the decode does
    # not make.  The write-only figure is reported beside the main one.
    flush_w = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
    flush_r = torch.ones((1 << 28,), dtype=torch.float32, device=dev)
    kv_bytes = gen.decode_kv_bytes(host_lens, dcfg.Hkv, dcfg.D)
    used_pages = int((-(-host_lens.astype(np.int64) // dcfg.page_size)).sum())
    other = dcfg.batch * dcfg.Hq * dcfg.D * 2 * 2 + dcfg.batch * dcfg.Hq * 4 + used_pages * 4 + dcfg.batch * 4
    alg_bytes = kv_bytes + other
    for _ in range(2):
        api.decode_paged(qq, kp, vp, table, lens, block=dcfg.block, max_context_len=max_ctx,
                         host_ctx_lens=host_lens, workspace=ws)
    def timed_call(read_after_write):
        flush_w.fill_(1)
        if read_after_write:
            flush_r.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        api.decode_paged(qq, kp, vp, table, lens, block=dcfg.block, max_context_len=max_ctx,
                         host_ctx_lens=host_lens, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    times, times_w = [], []
    for _ in range(args.decode_steps):
        times.append(timed_call(True))
        if args.decode_write_only_ref:
            times_w.append(timed_call(False))
    dms = float(np.median(times))
    dms_w = float(np.median(times_w)) if times_w else None
    gbs = kv_bytes / (dms * 1e-3) / 1e9
    ach = alg_bytes / (dms * 1e-3) / 1e9
    decode = {"value": round(gbs, 1), "unit": "GB/s", "ms": round(dms, 4), "kv_bytes": kv_bytes,
              "workload": "paged decode, 64 seqs, len U[512,16384] (sum %d), Hq=32 Hkv=8 D=128, page 16, "
                          "1M-slot pool, 128-key blocks, bf16 out" % int(host_lens.sum()),
              "flush": "1 GiB written then 1 GiB read before each timed call (median of %d)" % len(times),
              "ms_after_write_only_flush": round(dms_w, 4) if dms_w else None,
              "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": profile_traffic(DECODE_PROFILE)}}
    log(f"decode {dms:.3f} ms, {gbs:.0f} GB/s KV" + (f" (after a write-only flush {dms_w:.3f} ms)" if dms_w else ""))
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


def _read_csv(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def profile_commands():
    """Every rocprofv3 command the profiles/*.md summaries quote, in run order
    (kernel traces first, then one counter per run)."""
    cmds = [TRACE_CMD[m] for m in ("prefill", "decode", "backward", "lm_head")]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cmds += [PMC_CMD.format(c=c, m=m) for m in ("prefill", "decode", "copy")]
        cmds += [PMC_CMD_LM_HEAD.format(c=c), PMC_CMD_BACKWARD.format(c=c)]
    return cmds + [PMC_CMD_MFMA]


def _last_dispatches(d, mode, parts, n):
    """(name, n, avg us, min us, max us) per kernel over its last n dispatches
    in the kernel trace under d/prof_<mode>: the timed launches, after the
    untimed warm-up ones."""
    trace = sorted(_read_csv(os.path.join(d, f"prof_{mode}", "run_kernel_trace.csv")),
                   key=lambda r: int(r["Start_Timestamp"]))
    per = {}
    for r in trace:
        if any(p in r["Kernel_Name"] for p in parts):
            per.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return [(k, len(v[-n:]), float(np.mean(v[-n:])), min(v[-n:]), max(v[-n:])) for k, v in per.items()]


def _pmc_mean(d, counter, mode, name_part):
    """Mean counter value (KiB per dispatch) of the kernels whose name contains name_part."""
    path = os.path.join(d, f"pmc_{counter}_{mode}", "run_counter_collection.csv")
    vals = [float(r["Counter_Value"]) for r in _read_csv(path) if name_part in r["Kernel_Name"]]
    return sum(vals) / len(vals), len(vals)


def summarize_profiles(d):
    """Turn the kernel-trace stats and the FETCH_SIZE / WRITE_SIZE counter runs
    under d into profiles/prefill_kernel_b4_s4096.md and profiles/decode_paged_64seq.md.
    Counter KiB are scaled by what the same counter reads for a plain 1 GiB
    device copy (the runtime's copy kernel): bytes = KiB * 1024 * factor."""
    copy_f, _ = _pmc_mean(d, "FETCH_SIZE", "copy", "copyBuffer")
    copy_w, _ = _pmc_mean(d, "WRITE_SIZE", "copy", "copyBuffer")
    f_fetch = (1 << 30) / (copy_f * 1024.0)
    f_write = (1 << 30) / (copy_w * 1024.0)
    src = kernel_source_hash()
    cfg, dcfg = gen.CFG2, gen.CFG4
    lens = gen.decode_lengths(dcfg)
    kv = gen.decode_kv_bytes(lens, dcfg.Hkv, dcfg.D)
    pages = int((-(-lens.astype(np.int64) // dcfg.page_size)).sum())
    dec_alg = kv + dcfg.batch * dcfg.Hq * dcfg.D * 2 * 2 + dcfg.batch * dcfg.Hq * 4 + pages * 4 + dcfg.batch * 4
    pre_alg = (cfg.B * cfg.S * (cfg.Hq + 2 * cfg.Hkv) * cfg.D * 2 + cfg.B * cfg.S * cfg.Hq * cfg.D * 2
               + cfg.B * cfg.S * cfg.Hq * 4)

    def stats_rows(mode, parts):
        rows = _read_csv(os.path.join(d, f"prof_{mode}", "run_kernel_stats.csv"))
        out = []
        for r in rows:
            if any(p in r["Name"] for p in parts):
                out.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                            float(r["MaxNs"]) / 1e3))
        return out

    def counters(mode, part):
        fk, n1 = _pmc_mean(d, "FETCH_SIZE", mode, part)
        wk, n2 = _pmc_mean(d, "WRITE_SIZE", mode, part)
        return fk, wk, int(round(fk * 1024 * f_fetch)), int(round(wk * 1024 * f_write)), min(n1, n2)

    header = ("Counter scaling: a plain 1 GiB device copy (`python3 bench.py --only copy`) reads "
              f"FETCH_SIZE = {copy_f:.1f} KiB and WRITE_SIZE = {copy_w:.1f} KiB per dispatch, so "
              f"fetch bytes = KiB x 1024 x {f_fetch:.4f} and write bytes = KiB x 1024 x {f_write:.4f}.\n")
    cmds = "\n".join("    " + PMC_CMD.format(c=c, m=m) for c in ("FETCH_SIZE", "WRITE_SIZE")
                     for m in ("prefill", "decode", "copy"))

    # prefill
    st = stats_rows("prefill", ["prefill_pp_kernel"])
    fk, wk, fb, wb, n = counters("prefill", "prefill_pp_kernel")
    name, calls, avg, mn, mx = st[0]
    trace = _read_csv(os.path.join(d, "prof_prefill", "run_kernel_trace.csv"))
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            for r in sorted(trace, key=lambda r: int(r["Start_Timestamp"])) if "prefill_pp_kernel" in r["Kernel_Name"]]
    timed = durs[-TIMED_STEPS:]
    t_avg = float(np.mean(timed))
    flops = cfg.flops()

    def row(label, c, a, lo, hi):
        return (f"| {label} | {c} | {a:.1f} | {lo:.1f} | {hi:.1f} | {flops / (a * 1e-6) / 1e12:.1f} | "
                f"{flops / (a * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.4f} |")

    lines = [
        "# Prefill kernel, causal B=4 S=4096 Hq=32 Hkv=8 D=128, 128-key blocks, bf16 out",
        "",
        f"Kernel trace (100 untimed warm-up launches, then the {TIMED_STEPS} timed ones):",
        "",
        "    " + TRACE_CMD["prefill"],
        "",
        "| dispatches | calls | avg us | min us | max us | TFLOP/s at avg | frac of 2500 |",
        "|---|---|---|---|---|---|---|",
        row(f"`{name}`, the {TIMED_STEPS} timed", len(timed), t_avg, min(timed), max(timed)),
        row("all, warm-up included (the --stats summary)", calls, avg, mn, mx),
        "",
        f"Algorithmic work per launch: {flops:.6e} flop (4·D·Hq·B·S(S+1)/2); algorithmic HBM bytes "
        f"{pre_alg} (Q, K, V in; Out bf16, LSE out).",
        "",
        "HBM counters, one run per counter:",
        "",
        cmds,
        "",
        header,
        f"| counter | KiB per dispatch (mean of {n}) | bytes |",
        "|---|---|---|",
        f"| FETCH_SIZE | {fk:.1f} | {fb} |",
        f"| WRITE_SIZE | {wk:.1f} | {wb} |",
        "",
        f"traffic bytes per launch: `{fb + wb}` ({(fb + wb) / pre_alg:.2f} x algorithmic)",
        "",
        f"kernel source sha256: `{src}`",
        "",
    ]
    with open(PREFILL_PROFILE, "w") as f:
        f.write("\n".join(lines))

    # decode
    st = stats_rows("decode", ["decode_items_kernel", "fold_kernel"])
    ci = counters("decode", "decode_items_kernel")
    cf = counters("decode", "fold_kernel")
    total_us = sum(r[2] for r in st)
    lines = [
        "# Paged decode, 64 sequences, lengths U[512,16384], page 16, 128-key blocks, bf16 out",
        "",
        f"Drawn lengths sum to {int(lens.sum())} tokens; K+V bytes read {kv}; algorithmic bytes per decode call "
        f"{dec_alg} (KV, Q, Out, LSE, used page-table entries, lengths).",
        "",
        "Kernel trace (decode = items kernel + fold kernel; before each timed call 1 GiB is written, then 1 GiB read,",
        "so no KV byte is cache-served and no dirty line of the flush is written back inside the call; the first",
        "two calls are unflushed warm-ups):",
        "",
        "    " + TRACE_CMD["decode"],
        "",
        "| kernel | calls | avg us | min us | max us |",
        "|---|---|---|---|---|",
    ] + [f"| `{r[0]}` | {r[1]} | {r[2]:.1f} | {r[3]:.1f} | {r[4]:.1f} |" for r in st] + [
        "",
        f"Sum of averages {total_us:.1f} us -> {dec_alg / (total_us * 1e-6) / 1e9:.1f} GB/s algorithmic "
        f"({dec_alg / (total_us * 1e-6) / 1e9 / PEAK_HBM_GBS:.4f} of 8000 GB/s).",
        "",
        "HBM counters, one run per counter:",
        "",
        cmds,
        "",
        header,
        "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | fetch bytes | write bytes |",
        "|---|---|---|---|---|",
        f"| decode_items_kernel | {ci[0]:.1f} | {ci[1]:.1f} | {ci[2]} | {ci[3]} |",
        f"| fold_kernel | {cf[0]:.1f} | {cf[1]:.1f} | {cf[2]} | {cf[3]} |",
        "",
        f"traffic bytes per launch: `{ci[2] + ci[3] + cf[2] + cf[3]}` (both kernels; "
        f"{(ci[2] + ci[3] + cf[2] + cf[3]) / dec_alg:.3f} x algorithmic; the per-block partial states "
        "written by the items kernel and read back by the fold are the excess)",
        "",
        f"kernel source sha256: `{src}`",
        "",
    ]
    with open(DECODE_PROFILE, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {PREFILL_PROFILE} and {DECODE_PROFILE}")
    if os.path.isdir(os.path.join(d, "prof_backward")):
        summarize_backward(d, f_fetch, f_write, header, src)
    if os.path.isdir(os.path.join(d, "prof_lm_head")):
        summarize_lm_head(d, f_fetch, f_write, header, src)
    if os.path.isdir(os.path.join(d, "pmc_mfma_prefill")):
        summarize_mfma(d, src)


def summarize_mfma(d, src):
    """profiles/prefill_mfma_counters_b4_s4096.md: clock, MFMA and VALU activity
    of the bf16 prefill kernel from one counter run (per-XCD GRBM counters are
    summed by rocprofv3, so the busy cycles of one XCD are the sum / 8)."""
    rows = _read_csv(os.path.join(d, "pmc_mfma_prefill", "run_counter_collection.csv"))
    per = {}
    for r in rows:
        if "prefill_pp_kernel" not in r["Kernel_Name"]:
            continue
        e = per.setdefault(r["Dispatch_Id"], {"_ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    runs = [per[k] for k in sorted(per, key=int)][-TIMED_STEPS:]  # the timed launches, after the warm-up
    mean = {k: float(np.mean([x[k] for x in runs])) for k in runs[0]}
    cfg = gen.CFG2
    n_xcd, n_simd = 8, 1024
    clk = mean["GRBM_GUI_ACTIVE"] / n_xcd / mean["_ns"]  # GHz
    busy = mean["GRBM_GUI_ACTIVE"] / n_xcd
    mfma_flop = mean["SQ_INSTS_MFMA"] * 32 * 32 * 16 * 2
    lines = [
        "# Prefill kernel MFMA and VALU counters, causal B=4 S=4096 Hq=32 Hkv=8 D=128, bf16 out",
        "",
        "    " + PMC_CMD_MFMA,
        "",
        f"Mean over the last {len(runs)} dispatches of `prefill_pp_kernel<128, 0>` (the timed launches; the "
        "100 before them are the warm-up):",
        "",
        "| counter | value per dispatch |",
        "|---|---|",
    ] + [f"| {k} | {v:.0f} |" for k, v in sorted(mean.items()) if not k.startswith("_")] + [
        f"| duration (ns) | {mean['_ns']:.0f} |",
        "",
        f"* Clock: GRBM_GUI_ACTIVE / 8 XCDs / duration = {clk:.2f} GHz.",
        f"* MFMA instructions (v_mfma_f32_32x32x16_bf16, 32768 flop each): {mean['SQ_INSTS_MFMA']:.0f} = "
        f"{mfma_flop:.4e} flop executed, {mfma_flop / cfg.flops():.3f} x the algorithmic {cfg.flops():.4e} "
        "(the masked halves of diagonal blocks).",
        f"* Matrix-core busy: SQ_VALU_MFMA_BUSY_CYCLES / (busy cycles x {n_simd} SIMDs) = "
        f"{mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (busy * n_simd):.3f}.",
        f"* VALU instructions (MFMAs included): {mean['SQ_INSTS_VALU']:.0f}, "
        f"{mean['SQ_INSTS_VALU'] * 4 / (busy * n_simd):.3f} of the SIMDs' cycles at 4 cycles per wave64 instruction.",
        "",
        f"kernel source sha256: `{src}`",
        "",
    ]
    path = os.path.join(PROFILES, "prefill_mfma_counters_b4_s4096.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {path}")


def summarize_lm_head(d, f_fetch, f_write, header, src):
    """profiles/lm_head_logprobs_t64_v151936.md from the lm_head trace and counters."""
    T, H, V = 64, 4096, gen.LM_VOCAB
    flops = 2.0 * T * V * H
    alg_bytes = V * H * 4 + T * H * 2 + T * 4 * 3
    kern = _last_dispatches(d, "lm_head", ["lmh_"], LM_HEAD_TIMED_REPS)
    kern.sort(key=lambda r: 0 if "partial" in r[0] else 1)
    total_us = sum(r[2] for r in kern)

    def counter(c, part):
        vals = [float(r["Counter_Value"]) for r in
                _read_csv(os.path.join(d, f"pmc_{c}_lm_head", "run_counter_collection.csv"))
                if part in r["Kernel_Name"] and r["Counter_Name"] == c]
        return sum(vals) / max(len(vals), 1)

    lines = [
        "# Selected log-probs through the FP32 lm_head: 64 tokens, H = 4096 (bf16 x), V = 151936",
        "",
        "Kernel trace (two launches per call: logits with per-block log-sum-exp partials, then the ordered fold; "
        f"the figures are over the {LM_HEAD_TIMED_REPS} timed calls, after about 100 ms of untimed warm-up calls):",
        "",
        "    " + TRACE_CMD["lm_head"],
        "",
        "| kernel | calls | avg us | min us | max us |",
        "|---|---|---|---|---|",
    ] + [f"| `{r[0]}` | {r[1]} | {r[2]:.1f} | {r[3]:.1f} | {r[4]:.1f} |" for r in kern] + [
        "",
        f"Sum of averages {total_us:.1f} us.  Algorithmic work {flops:.4e} flop (2·T·V·H FP32 MFMA) -> "
        f"{flops / (total_us * 1e-6) / 1e12:.1f} TFLOP/s ({flops / (total_us * 1e-6) / 1e12 / PEAK_FP32_TFLOPS:.4f} of "
        f"the 157.3 TFLOP/s dense fp32 peak); algorithmic bytes {alg_bytes} (W once, x, tokens, logp, logZ) -> "
        f"{alg_bytes / (total_us * 1e-6) / 1e9:.1f} GB/s.",
        "",
        "HBM counters, one run per counter:",
        "",
    ] + ["    " + PMC_CMD_LM_HEAD.format(c=c) for c in ("FETCH_SIZE", "WRITE_SIZE")] + [
        "",
        header,
        "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | fetch bytes | write bytes |",
        "|---|---|---|---|---|",
    ]
    tot = 0
    for part in ("lmh_partial", "lmh_fold"):
        fk, wk = counter("FETCH_SIZE", part), counter("WRITE_SIZE", part)
        fb, wb = int(round(fk * 1024 * f_fetch)), int(round(wk * 1024 * f_write))
        tot += fb + wb
        lines.append(f"| {part} | {fk:.1f} | {wk:.1f} | {fb} | {wb} |")
    lines += ["", f"traffic bytes per call: `{tot}` ({tot / alg_bytes:.2f} x algorithmic)", "",
              f"kernel source sha256: `{src}`", ""]
    with open(LM_HEAD_PROFILE, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {LM_HEAD_PROFILE}")


def summarize_backward(d, f_fetch, f_write, header, src):
    """profiles/backward_b4_s4096.md from the backward kernel trace and counters."""
    cfg = gen.CFG2
    kern = _last_dispatches(d, "backward", ["bwd_"], BACKWARD_TIMED_STEPS)
    order = {"bwd_dq": 0, "bwd_dkdv": 1}
    kern.sort(key=lambda r: min(v for k, v in order.items() if k in r[0]))
    fwd = cfg.flops()
    alg = 2.5 * fwd
    executed = {"bwd_dq": 1.5 * fwd, "bwd_dkdv": 2.0 * fwd}
    B, S, Hq, Hkv, D = cfg.B, cfg.S, cfg.Hq, cfg.Hkv, cfg.D
    alg_bytes = B * S * (3 * Hq + 2 * Hkv) * D * 2 + B * S * Hq * 4 + B * S * (Hq + 2 * Hkv) * D * 4
    total_us = sum(r[2] for r in kern)

    def counter(c, part):
        vals = []
        for r in _read_csv(os.path.join(d, f"pmc_{c}_backward", "run_counter_collection.csv")):
            if part in r["Kernel_Name"] and r["Counter_Name"] == c:
                vals.append(float(r["Counter_Value"]))
        return sum(vals) / max(len(vals), 1), len(vals)

    lines = [
        "# Backward (dQ, dK, dV), causal B=4 S=4096 Hq=32 Hkv=8 D=128, bf16 in, fp32 gradients",
        "",
        "Kernel trace (two launches per backward call: dQ, which also writes Delta per row, then dK/dV; the "
        f"figures are over the {BACKWARD_TIMED_STEPS} timed calls, after about 100 ms of untimed warm-up calls):",
        "",
        "    " + TRACE_CMD["backward"],
        "",
        "| kernel | calls | avg us | min us | max us | MFMA work executed (flop) | TFLOP/s executed at avg |",
        "|---|---|---|---|---|---|---|",
    ]
    for name, calls, avg, mn, mx in kern:
        ex = next(v for k, v in executed.items() if k in name)
        rate = f"{ex / (avg * 1e-6) / 1e12:.1f}" if ex else "-"
        lines.append(f"| `{name}` | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {ex:.4e} | {rate} |")
    lines += [
        "",
        f"Sum of averages {total_us:.1f} us.  Algorithmic work of one backward: {alg:.6e} flop (the five products "
        "QK^T, dOut V^T, P^T dOut, dS^T Q, dS K over the unmasked pairs, 2.5x the forward's "
        f"{fwd:.6e}) -> {alg / (total_us * 1e-6) / 1e12:.1f} TFLOP/s "
        f"({alg / (total_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.4f} of 2500).  The dQ kernel recomputes QK^T and "
        "dOut V^T (no atomics, no dS in HBM), so the MFMA work executed is 3.5x the forward's.",
        "",
        f"Algorithmic HBM bytes: {alg_bytes} (Q, K, V, Out, dOut bf16 and LSE in; dQ, dK, dV fp32 out).",
        "",
        "HBM counters, one run per counter:",
        "",
    ] + ["    " + PMC_CMD_BACKWARD.format(c=c) for c in ("FETCH_SIZE", "WRITE_SIZE")] + [
        "",
        header,
        "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | fetch bytes | write bytes |",
        "|---|---|---|---|---|",
    ]
    tot = 0
    for part in ("bwd_dq", "bwd_dkdv"):
        fk, _ = counter("FETCH_SIZE", part)
        wk, _ = counter("WRITE_SIZE", part)
        fb, wb = int(round(fk * 1024 * f_fetch)), int(round(wk * 1024 * f_write))
        tot += fb + wb
        lines.append(f"| {part} | {fk:.1f} | {wk:.1f} | {fb} | {wb} |")
    lines += [
        "",
        f"traffic bytes per backward: `{tot}` ({tot / alg_bytes:.2f} x algorithmic; the dK/dV walk re-reads the "
        "Q and dOut tiles of its kv head once per 128-key block, and the dQ walk the K/V blocks once per "
        "64-row tile)",
        "",
        f"kernel source sha256: `{src}`",
        "",
    ]
    with open(BACKWARD_PROFILE, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {BACKWARD_PROFILE}")


if __name__ == "__main__":
    main()
