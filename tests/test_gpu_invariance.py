"""Bitwise invariances of the GPU path (max abs 0.0 on Out and LSE):
a row's independence of every other query row, batch composition, chunk size, context-parallel split (contiguous and zigzag),
fused vs emit+merge, arrival order of partial states, repeat runs.  Plus a
parity check of the chunked path against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from deterministic_gqa_attention_amd import api
from deterministic_gqa_attention_amd import inputs as gen
from tests.gpu_util import assert_bitwise, check_parity, dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu


def _rand(seed, shape, scale=1.0):
    return gen.f64_to_bf16_bits(gen.normals(seed, shape) * scale)


def _emit_and_merge(qd, kd, vd, shards, *, block, out_dtype, order, cache_len=None, q_begin=0, q_count=None):
    """Emit every shard's per-block states into one buffer in `order` (a
    permutation of all owned blocks = arrival order) and merge them."""
    B, S, Hq, D = qd.shape
    q_count = S - q_begin if q_count is None else q_count
    blocks = [b for sh in shards for b in sh]
    arrival = [blocks[i] for i in order]
    n = len(arrival)
    part_out = torch.empty((n, B * q_count, Hq, D), dtype=torch.float32, device=qd.device)
    part_lse = torch.empty((n, B * q_count, Hq), dtype=torch.float32, device=qd.device)
    # each shard writes its own blocks where they sit in the arrival order
    for sh in shards:
        pos = [arrival.index(b) for b in sh]
        lo, hi = min(pos), max(pos) + 1
        if pos == list(range(lo, hi)):
            api.emit_partials(qd, kd, vd, sh, block=block, out_dtype=out_dtype, q_begin=q_begin, q_count=q_count,
                              cache_len=cache_len, part_out=part_out[lo:hi], part_lse=part_lse[lo:hi])
        else:
            for b, p in zip(sh, pos):
                api.emit_partials(qd, kd, vd, [b], block=block, out_dtype=out_dtype, q_begin=q_begin,
                                  q_count=q_count, cache_len=cache_len, part_out=part_out[p:p + 1],
                                  part_lse=part_lse[p:p + 1])
    out, lse = api.merge_states(part_out, part_lse, arrival, out_dtype=out_dtype)
    return out.view(B, q_count, Hq, D), lse.view(B, q_count, Hq), (part_out, part_lse, arrival)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_tiny_cp2_split_and_arrival(out_dtype):
    """TP=2 local shard, S=256, 64-key blocks, CP=2 split at key 128: fused ==
    CP=1 emit+merge == CP=2 emit+merge, for sorted, reversed and shuffled arrival."""
    cfg = gen.CFG1
    q, k, v = gen.prefill_inputs(cfg)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    say(f"[invariance] tiny CP=2 {out_dtype}")
    fo, fl = api.prefill(qd, kd, vd, block=cfg.block, out_dtype=out_dtype)
    nb = cfg.n_blocks
    for shards in (((0, 1, 2, 3),), cfg.shards):
        for name, order in (("sorted", list(range(nb))), ("reversed", list(range(nb))[::-1]),
                            ("shuffled", list(gen.arrival_shuffle(cfg.cfg_id, nb)))):
            mo, ml, _ = _emit_and_merge(qd, kd, vd, shards, block=cfg.block, out_dtype=out_dtype, order=order)
            assert_bitwise(mo, fo, f"CP={len(shards)} {name} Out")
            assert_bitwise(ml, fl, f"CP={len(shards)} {name} LSE")


def test_tiny_partials_match_oracle_block_states():
    """Each emitted per-block state (out_i, lse_i) matches the oracle's
    block-restricted attention (fp32 output mode)."""
    cfg = gen.CFG1
    q, k, v = gen.prefill_inputs(cfg)
    say("[invariance] per-block states vs oracle")
    po, pl = api.emit_partials(dev_bf16(q), dev_bf16(k), dev_bf16(v), list(range(cfg.n_blocks)), block=cfg.block,
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.block_states(q, k, v, scale=cfg.softmax_scale, block=cfg.block, blocks=range(cfg.n_blocks))
    check_parity(host_f64(po), host_f64(pl), ro, rl, f32_out=True, what="block states")


def test_arrival_order_diagnostic_vs_sorted():
    """The merge-order probe: folding partial states in their arrival order
    drifts from the fused result (floating-point addition is not associative),
    while the merge sorted by global block index is bitwise equal to it for
    every arrival order.  16 blocks of 64 keys, fp32 output."""
    q, k, v = _rand(41, (1, 1024, 8, 128)), _rand(42, (1, 1024, 2, 128)), _rand(43, (1, 1024, 2, 128))
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    say("[invariance] arrival-order diagnostic")
    fo, fl = api.prefill(qd, kd, vd, block=64, out_dtype=torch.float32)
    nb = 16
    po, pl = api.emit_partials(qd, kd, vd, list(range(nb)), block=64, out_dtype=torch.float32)
    drifts = []
    for name, order in (("reversed", list(range(nb))[::-1]), ("shuffled", list(gen.arrival_shuffle(2, nb))),
                        ("shuffled2", list(gen.arrival_shuffle(5, nb)))):
        idx = torch.tensor(order, device=po.device)
        po_a, pl_a = po[idx].contiguous(), pl[idx].contiguous()
        so, sl = api.merge_states(po_a, pl_a, order, out_dtype=torch.float32)
        assert_bitwise(so.view_as(fo), fo, f"sorted merge of {name} arrival Out")
        assert_bitwise(sl.view_as(fl), fl, f"sorted merge of {name} arrival LSE")
        ao, al = api.merge_states(po_a, pl_a, order, out_dtype=torch.float32, order="arrival")
        d_out = (ao.view_as(fo) - fo).abs().max().item()
        d_lse = (al.view_as(fl) - fl).abs().max().item()
        say(f"    {name}: arrival-order drift Out {d_out:.3e} LSE {d_lse:.3e}; sorted 0.0")
        # a fold in another order is still the same merge up to fp32 rounding
        assert d_out <= 1e-4 and d_lse <= 1e-4
        drifts.append(max(d_out, d_lse))
    assert max(drifts) > 0.0, "arrival order showed no drift: the probe shows nothing"


def test_batch_composition():
    """A sequence alone (B=1) gives the same bits as inside a batch of 4."""
    q, k, v = _rand(21, (4, 520, 8, 128)), _rand(22, (4, 520, 2, 128)), _rand(23, (4, 520, 2, 128))
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    say("[invariance] batch composition")
    bo, bl = api.prefill(qd, kd, vd, block=128)
    for b in (0, 2, 3):
        so, sl = api.prefill(qd[b:b + 1].contiguous(), kd[b:b + 1].contiguous(), vd[b:b + 1].contiguous(), block=128)
        assert_bitwise(so[0], bo[b], f"seq {b} alone vs batch Out")
        assert_bitwise(sl[0], bl[b], f"seq {b} alone vs batch LSE")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_row_independent_of_other_rows(out_dtype):
    """A row's bits depend on its own query and the keys it sees only: every
    other query row and every other q head (its MFMA tile neighbours, the
    other rows of its workgroup and the other heads of its kv group) redrawn,
    the kept rows give the same Out and LSE.  Kept rows sit at tile edges and
    inside tiles, on and off the causal diagonal, and in the ragged tail."""
    B, S, Hq, Hkv = 1, 300, 8, 2
    q, k, v = _rand(71, (B, S, Hq, 128)), _rand(72, (B, S, Hkv, 128)), _rand(73, (B, S, Hkv, 128))
    keep = [0, 1, 31, 32, 63, 64, 127, 128, 150, 255, 256, 299]
    head = 5
    q2 = _rand(74, (B, S, Hq, 128), scale=3.0)
    q2[:, keep, head] = q[:, keep, head]
    kd, vd = dev_bf16(k), dev_bf16(v)
    say(f"[invariance] row independence out={out_dtype}")
    for block in (64, 128):
        o1, l1 = api.prefill(dev_bf16(q), kd, vd, block=block, out_dtype=out_dtype)
        o2, l2 = api.prefill(dev_bf16(q2), kd, vd, block=block, out_dtype=out_dtype)
        assert_bitwise(o2[:, keep, head], o1[:, keep, head], f"block {block} kept rows Out")
        assert_bitwise(l2[:, keep, head], l1[:, keep, head], f"block {block} kept rows LSE")
        assert not torch.equal(o2[:, 2, head], o1[:, 2, head]), "a redrawn row should change"


def _replay(qd, kd, vd, chunk, *, block, out_dtype=torch.bfloat16):
    """Chunked-prefill replay: write each chunk's K/V into an empty cache, then
    run the chunk against everything cached so far."""
    B, S, Hq, D = qd.shape
    kc = torch.zeros_like(kd)
    vc = torch.zeros_like(vd)
    outs, lses = [], []
    for c0 in range(0, S, chunk):
        c1 = min(S, c0 + chunk)
        kc[:, c0:c1] = kd[:, c0:c1]
        vc[:, c0:c1] = vd[:, c0:c1]
        o, l = api.prefill_chunked(qd[:, c0:c1].contiguous(), kc, vc, cache_len=c0, block=block, out_dtype=out_dtype)
        outs.append(o)
        lses.append(l)
    return torch.cat(outs, dim=1), torch.cat(lses, dim=1)


@pytest.mark.parametrize("chunk", [1, 7, 64, 100, 512])
def test_chunked_equals_one_shot_small(chunk):
    q, k, v = _rand(31, (2, 700, 8, 128)), _rand(32, (2, 700, 2, 128)), _rand(33, (2, 700, 2, 128))
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    say(f"[invariance] chunked replay chunk={chunk}")
    fo, fl = api.prefill(qd, kd, vd, block=128)
    co, cl = _replay(qd, kd, vd, chunk, block=128)
    assert_bitwise(co, fo, f"chunk {chunk} Out")
    assert_bitwise(cl, fl, f"chunk {chunk} LSE")


def test_chunked_parity_with_oracle():
    q, k, v = _rand(34, (1, 300, 8, 128)), _rand(35, (1, 300, 2, 128)), _rand(36, (1, 300, 2, 128))
    say("[invariance] chunk vs oracle")
    c0, C = 129, 100
    kd, vd = dev_bf16(k), dev_bf16(v)
    o, l = api.prefill_chunked(dev_bf16(q[:, c0:c0 + C]), kd, vd, cache_len=c0, block=64, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q[:, c0:c0 + C], k, v, scale=1 / np.sqrt(128), pos0=c0, kv_len=c0 + C)
    check_parity(host_f64(o).reshape(C, 8, 128), host_f64(l).reshape(C, 8), ro, rl, f32_out=True, what="chunk")


@pytest.mark.slow
def test_chunked_replay_8192_all_chunk_sizes():
    """Chunked-prefill replay of 8192 tokens (Hq=32, Hkv=8) in chunks of 1, 512
    and 2048: the one-shot prefill matches the oracle on every row, and every
    replay is bitwise equal to it."""
    cfg = gen.CFG3
    q, k, v = gen.prefill_inputs(cfg)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    say("[invariance] 8192-token one-shot vs oracle (every row)")
    fo, fl = api.prefill(qd, kd, vd, block=cfg.block)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, scale=cfg.softmax_scale)
    stats = check_parity(host_f64(fo).reshape(ro.shape), host_f64(fl).reshape(rl.shape), ro, rl, f32_out=False,
                         what="8192-token one-shot")
    say(f"    parity {stats}")
    del ro, rl
    for chunk in gen.CFG3_CHUNKS:
        say(f"[invariance] 8192-token replay chunk={chunk}")
        co, cl = _replay(qd, kd, vd, chunk, block=cfg.block)
        assert_bitwise(co, fo, f"chunk {chunk} Out")
        assert_bitwise(cl, fl, f"chunk {chunk} LSE")


@pytest.mark.slow
def test_full_prefill_cp_and_batch():
    """B=4, S=4096: fused == CP=1 emit+merge == CP=2 (contiguous halves)
    emit+merge with reversed arrival; one sequence alone == in the batch."""
    cfg = gen.CFG2
    q, k, v = gen.prefill_inputs(cfg)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    say("[invariance] B=4 S=4096 fused")
    fo, fl = api.prefill(qd, kd, vd, block=cfg.block)
    nb = cfg.n_blocks
    for shards, order, name in ((((tuple(range(nb))),), list(range(nb)), "CP=1"),
                                (cfg.shards, list(range(nb))[::-1], "CP=2 reversed")):
        say(f"[invariance] B=4 S=4096 {name}")
        mo, ml, parts = _emit_and_merge(qd, kd, vd, shards, block=cfg.block, out_dtype=torch.bfloat16, order=order)
        assert_bitwise(mo, fo, f"{name} Out")
        assert_bitwise(ml, fl, f"{name} LSE")
        del parts, mo, ml
        torch.cuda.empty_cache()
    say("[invariance] B=4 S=4096 batch composition")
    so, sl = api.prefill(qd[1:2].contiguous(), kd[1:2].contiguous(), vd[1:2].contiguous(), block=cfg.block)
    assert_bitwise(so[0], fo[1], "seq alone Out")
    assert_bitwise(sl[0], fl[1], "seq alone LSE")


@pytest.mark.slow
def test_long_context_zigzag_cp2_shuffled():
    """S=32768, Q/K x4: zigzag CP=2 (chunks 0+3 / 1+2 of 4), partial states in
    query slabs of 4096 rows, shuffled arrival: bitwise equal to fused."""
    cfg = gen.CFG5
    q, k, v = gen.prefill_inputs(cfg)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    say("[invariance] S=32768 fused")
    fo, fl = api.prefill(qd, kd, vd, block=cfg.block)
    nb = cfg.n_blocks
    order = list(gen.arrival_shuffle(cfg.cfg_id, nb))
    slab = 4096
    for s0 in range(0, cfg.S, slab):
        say(f"[invariance] S=32768 zigzag slab {s0}")
        mo, ml, parts = _emit_and_merge(qd, kd, vd, cfg.shards, block=cfg.block, out_dtype=torch.bfloat16,
                                        order=order, q_begin=s0, q_count=slab)
        assert_bitwise(mo, fo[:, s0:s0 + slab], f"slab {s0} Out")
        assert_bitwise(ml, fl[:, s0:s0 + slab], f"slab {s0} LSE")
        del parts, mo, ml
        torch.cuda.empty_cache()
