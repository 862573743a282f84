"""GPU paged-KV decode: parity with the FP64 oracle, and bitwise invariance to
batch composition (a sequence alone vs in the batch) and to page placement
(pages relocated in the pool).  Also: decode equals the last row of a prefill
over the same tokens, bit for bit, because both run the same per-block core.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from deterministic_gqa_attention_amd import api
from deterministic_gqa_attention_amd import inputs as gen
from tests.gpu_util import assert_bitwise, check_parity, dev_bf16, dev_i32, host_f64, say

pytestmark = pytest.mark.gpu

SMALL = gen.DecodeConfig(41, "small paged decode", batch=7, Hq=8, Hkv=2, D=128, page_size=16, num_pages=512,
                         len_lo=1, len_hi=700, block=128)
SMALL_LENS = np.array([1, 16, 127, 128, 129, 300, 700], np.int32)


def _decode(d, cfg, *, block, out_dtype=torch.bfloat16, max_ctx=None, seqs=None, host_lens=True):
    """Run decode on the inputs in d (numpy); the pools are uploaded once and
    cached in d under "_dev"."""
    if "_dev" not in d:
        d["_dev"] = (dev_bf16(d["k_pool"]), dev_bf16(d["v_pool"]))
    kp, vp = d["_dev"]
    lens = d["ctx_lens"] if seqs is None else d["ctx_lens"][seqs]
    table = d["page_table"] if seqs is None else d["page_table"][seqs]
    q = d["q"] if seqs is None else d["q"][seqs]
    max_ctx = int(cfg.len_hi) if max_ctx is None else max_ctx
    return api.decode_paged(dev_bf16(q), kp, vp, dev_i32(table), dev_i32(lens), block=block,
                            max_context_len=max_ctx, host_ctx_lens=lens if host_lens else None,
                            out_dtype=out_dtype)


@pytest.mark.parametrize("block", [64, 128])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_small_decode_parity(block, out_dtype):
    d = gen.decode_inputs(SMALL, lengths=SMALL_LENS)
    say(f"[decode] small parity block={block} out={out_dtype}")
    out, lse = _decode(d, SMALL, block=block, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged(d["q"], d["k_pool"], d["v_pool"], d["page_table"], d["ctx_lens"],
                                 scale=SMALL.softmax_scale)
    stats = check_parity(host_f64(out), host_f64(lse), ro, rl, f32_out=out_dtype == torch.float32,
                         what="small decode")
    say(f"    parity {stats}")


def test_small_decode_batch_and_relocation():
    d = gen.decode_inputs(SMALL, lengths=SMALL_LENS)
    say("[decode] small batch/relocation invariance")
    bo, bl = _decode(d, SMALL, block=128)
    for s in (0, 3, 6):
        so, sl = _decode(d, SMALL, block=128, seqs=[s])
        assert_bitwise(so[0], bo[s], f"seq {s} alone Out")
        assert_bitwise(sl[0], bl[s], f"seq {s} alone LSE")
    r = gen.relocate({k: d[k] for k in ("q", "k_pool", "v_pool", "page_table", "ctx_lens")},
                     gen.relocation(SMALL, SMALL.num_pages))
    ro, rl = _decode(r, SMALL, block=128)
    assert_bitwise(ro, bo, "relocated Out")
    assert_bitwise(rl, bl, "relocated LSE")


@pytest.mark.parametrize("block", [64, 128])
def test_small_decode_without_host_lengths(block):
    """Without host-side lengths the launch covers every possible unit and idle
    ones exit; results are bitwise those of the compact launch."""
    d = gen.decode_inputs(SMALL, lengths=SMALL_LENS)
    say(f"[decode] no host lengths block={block}")
    a_o, a_l = _decode(d, SMALL, block=block)
    b_o, b_l = _decode(d, SMALL, block=block, host_lens=False)
    assert_bitwise(b_o, a_o, "Out without host lengths")
    assert_bitwise(b_l, a_l, "LSE without host lengths")


def test_decode_equals_prefill_last_row():
    """Same per-(row, block) arithmetic: decode over a cache of L tokens equals
    row L-1 of causal prefill over the same tokens, bitwise."""
    d = gen.decode_inputs(SMALL, lengths=SMALL_LENS)
    say("[decode] decode == prefill last row")
    do, dl = _decode(d, SMALL, block=128, out_dtype=torch.float32)
    P = SMALL.page_size
    for s in (2, 4, 6):
        L = int(SMALL_LENS[s])
        pages = d["page_table"][s, : -(-L // P)]
        k = d["k_pool"][pages].transpose(0, 2, 1, 3).reshape(-1, SMALL.Hkv, 128)[:L][None]
        v = d["v_pool"][pages].transpose(0, 2, 1, 3).reshape(-1, SMALL.Hkv, 128)[:L][None]
        q = np.zeros((1, L, SMALL.Hq, 128), np.uint16)
        q[0, L - 1] = d["q"][s]
        po, pl = api.prefill(dev_bf16(q), dev_bf16(k), dev_bf16(v), block=128, out_dtype=torch.float32)
        assert_bitwise(do[s], po[0, L - 1], f"seq {s} Out")
        assert_bitwise(dl[s], pl[0, L - 1], f"seq {s} LSE")


# Lengths around the boundaries of the decode workgroup units.  A sequence's
# head unit folds its first blocks in registers: 64 of them (8192 keys at
# 128-key blocks, 4096 at 64) when the batch has at least 512 (sequence, kv
# head) pairs, fewer for smaller batches, down to 4.  The rest goes to tail
# units of 4 blocks (512 / 256 keys), whose last one then holds 1, 2, 3 or 4
# blocks, with or without a block two ahead to prefetch.  Short lengths end
# inside the head unit (odd and even block counts, a lone block).  The batch
# is padded with one-key sequences to 256 sequences x 2 kv heads = 512 pairs,
# so its heads are 64 blocks long; the same sequences alone get 4-block heads.
UNIT_LENS = np.array([255, 256, 257, 511, 512, 513, 640, 769, 1023, 1024, 1025, 1537, 2049, 2303,
                      4095, 4096, 4097, 4351, 4352, 4353, 4609,
                      8191, 8192, 8193, 8703, 8704, 8705, 8833, 9217], np.int32)
UNIT_BATCH = np.concatenate([UNIT_LENS, np.ones(256 - UNIT_LENS.size, np.int32)])
UNITS = gen.DecodeConfig(43, "decode unit boundaries", batch=UNIT_BATCH.size, Hq=8, Hkv=2, D=128, page_size=16,
                         num_pages=8192, len_lo=1, len_hi=9300, block=128)


@pytest.mark.parametrize("block", [64, 128])
def test_unit_boundaries_parity_and_prefill_identity(block):
    """Decode at lengths around the unit boundaries matches the oracle, and
    every sequence's Out/LSE equal the last row of a causal prefill over the
    same tokens, bitwise."""
    cfg = dataclasses.replace(UNITS, block=block)
    d = gen.decode_inputs(cfg, lengths=UNIT_BATCH)
    say(f"[decode] unit boundaries block={block}")
    do, dl = _decode(d, cfg, block=block, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged(d["q"], d["k_pool"], d["v_pool"], d["page_table"], d["ctx_lens"],
                                 scale=cfg.softmax_scale)
    stats = check_parity(host_f64(do), host_f64(dl), ro, rl, f32_out=True, what="unit-boundary decode")
    say(f"    parity {stats}")
    eo, el = _decode(d, cfg, block=block, out_dtype=torch.float32, host_lens=False)
    assert_bitwise(eo, do, "Out with device lengths")
    assert_bitwise(el, dl, "LSE with device lengths")
    # the boundary sequences alone: 58 pairs, so 4-block heads and all else in tails
    n = UNIT_LENS.size
    so, sl = _decode(d, cfg, block=block, out_dtype=torch.float32, seqs=np.arange(n))
    assert_bitwise(so, do[:n], "Out with short heads")
    assert_bitwise(sl, dl[:n], "LSE with short heads")
    P = cfg.page_size
    for s, L in enumerate(UNIT_LENS.tolist()):
        pages = d["page_table"][s, : -(-L // P)]
        k = d["k_pool"][pages].transpose(0, 2, 1, 3).reshape(-1, cfg.Hkv, 128)[:L][None]
        v = d["v_pool"][pages].transpose(0, 2, 1, 3).reshape(-1, cfg.Hkv, 128)[:L][None]
        q = np.zeros((1, L, cfg.Hq, 128), np.uint16)
        q[0, L - 1] = d["q"][s]
        po, pl = api.prefill(dev_bf16(q), dev_bf16(k), dev_bf16(v), block=block, out_dtype=torch.float32)
        assert_bitwise(do[s], po[0, L - 1], f"len {L} Out")
        assert_bitwise(dl[s], pl[0, L - 1], f"len {L} LSE")


@pytest.mark.parametrize("block,pages", [(128, (1, 2, 4, 8, 32, 64, 128)), (64, (1, 8, 32, 64))])
def test_page_sizes_bitwise(block, pages):
    """The page size only changes where keys live: every page size that
    divides the block gives the bits of page size 16 (1 = one key per page,
    where a block spans 128 pages; = block, one page per block)."""
    d16 = gen.decode_inputs(SMALL, lengths=SMALL_LENS)
    ref_o, ref_l = _decode(d16, SMALL, block=block, out_dtype=torch.float32)
    for P in pages:
        need = int((-(-SMALL_LENS.astype(np.int64) // P)).sum())
        cfg = dataclasses.replace(SMALL, page_size=P, num_pages=need + 8)
        say(f"[decode] page size {P} block={block}")
        d = gen.decode_inputs(cfg, lengths=SMALL_LENS)
        o, l = _decode(d, cfg, block=block, out_dtype=torch.float32)
        assert_bitwise(o, ref_o, f"page size {P} Out")
        assert_bitwise(l, ref_l, f"page size {P} LSE")


@pytest.mark.parametrize("block", [64, 128])
def test_out_of_range_page_ids_are_clamped(block):
    """Ids below 0 read page 0 and ids at or past num_pages read the last
    page: the same bits as the table with those ids clamped."""
    d = gen.decode_inputs(SMALL, lengths=SMALL_LENS)
    n_pages = d["k_pool"].shape[0]
    bad, clamped = d["page_table"].copy(), d["page_table"].copy()
    # sequence 6 (700 keys, 44 pages) and sequence 4 (129 keys)
    for (s, i), (b_id, c_id) in zip([(6, 0), (6, 9), (6, 43), (4, 8)],
                                    [(-1, 0), (n_pages, n_pages - 1), (1 << 30, n_pages - 1), (-(1 << 30), 0)]):
        bad[s, i] = b_id
        clamped[s, i] = c_id
    say(f"[decode] out-of-range page ids block={block}")
    ro, rl = _decode(dict(d, page_table=clamped), SMALL, block=block, out_dtype=torch.float32)
    o, l = _decode(dict(d, page_table=bad), SMALL, block=block, out_dtype=torch.float32)
    assert_bitwise(o, ro, "Out with out-of-range ids")
    assert_bitwise(l, rl, "LSE with out-of-range ids")


def test_device_lengths_above_max_context_are_clamped():
    """A device context length above max_context_len attends only the first
    max_context_len keys (the bits of the same call with the lengths clamped);
    host lengths above it are rejected before any launch."""
    d = gen.decode_inputs(SMALL, lengths=SMALL_LENS)
    cap = 300  # SMALL_LENS holds 700 and lengths on both sides of it
    say(f"[decode] device lengths above max_context_len={cap}")
    o, l = _decode(d, SMALL, block=128, out_dtype=torch.float32, max_ctx=cap, host_lens=False)
    dc = dict(d, ctx_lens=np.minimum(d["ctx_lens"], cap).astype(np.int32))
    ro, rl = _decode(dc, SMALL, block=128, out_dtype=torch.float32, max_ctx=cap, host_lens=False)
    assert_bitwise(o, ro, "Out with lengths above max_context_len")
    assert_bitwise(l, rl, "LSE with lengths above max_context_len")
    with pytest.raises(Exception, match="outside"):
        _decode(d, SMALL, block=128, out_dtype=torch.float32, max_ctx=cap, host_lens=True)


def test_empty_context():
    d = gen.decode_inputs(SMALL, lengths=np.array([0, 5, 0], np.int32))
    say("[decode] zero-length contexts")
    out, lse = _decode(d, SMALL, block=128, out_dtype=torch.float32)
    assert torch.all(out[0] == 0) and torch.all(out[2] == 0)
    assert torch.all(torch.isneginf(lse[0])) and torch.all(torch.isneginf(lse[2]))
    assert torch.isfinite(lse[1]).all()


@pytest.mark.slow
def test_paged_decode_64_seqs_full():
    """64 sequences, lengths U[512, 16384], page size 16, 1M-slot pool, random
    page table: parity for every sequence; one sequence alone == in the batch;
    relocated pages give identical bits."""
    cfg = gen.CFG4
    d = gen.decode_inputs(cfg)
    say("[decode] 64 seqs full")
    out, lse = _decode(d, cfg, block=cfg.block)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged(d["q"], d["k_pool"], d["v_pool"], d["page_table"], d["ctx_lens"],
                                 scale=cfg.softmax_scale)
    stats = check_parity(host_f64(out), host_f64(lse), ro, rl, f32_out=False, what="64-seq decode")
    say(f"    parity {stats}")
    for s in (0, 17, 63):
        so, sl = _decode(d, cfg, block=cfg.block, seqs=[s])
        assert_bitwise(so[0], out[s], f"seq {s} alone Out")
        assert_bitwise(sl[0], lse[s], f"seq {s} alone LSE")
    say("[decode] 64 seqs relocated")
    r = gen.relocate({k: d[k] for k in ("q", "k_pool", "v_pool", "page_table", "ctx_lens")},
                     gen.relocation(cfg, cfg.num_pages))
    del d
    torch.cuda.empty_cache()
    o2, l2 = _decode(r, cfg, block=cfg.block)
    assert_bitwise(o2, out, "relocated Out")
    assert_bitwise(l2, lse, "relocated LSE")


# Empty sequences at the start, in the middle and at the end of the batch.
EMPTY_LENS = np.array([0, 5, 0, 0, 700, 129, 0], np.int32)


@pytest.mark.parametrize("block", [64, 128])
def test_length_sources_and_empty_sequences(block):
    """The lengths reach the kernels either with the launch (host lengths, up
    to 256 sequences) or from device memory; both give the same bits, and an
    empty sequence gives Out = 0 and LSE = -inf."""
    d = gen.decode_inputs(SMALL, lengths=EMPTY_LENS)
    say(f"[decode] length sources, empty sequences, block={block}")
    a_o, a_l = _decode(d, SMALL, block=block, out_dtype=torch.float32)
    b_o, b_l = _decode(d, SMALL, block=block, out_dtype=torch.float32, host_lens=False)
    assert_bitwise(b_o, a_o, "Out, device lengths")
    assert_bitwise(b_l, a_l, "LSE, device lengths")
    empty = torch.from_numpy(EMPTY_LENS == 0).to(a_o.device)
    assert not a_o[empty].any(), "empty sequence Out not zero"
    assert bool(torch.isneginf(a_l[empty]).all()), "empty sequence LSE not -inf"
    ro, rl = oracle.decode_paged(d["q"], d["k_pool"], d["v_pool"], d["page_table"], d["ctx_lens"],
                                 scale=SMALL.softmax_scale)
    live = EMPTY_LENS > 0
    check_parity(host_f64(a_o)[live], host_f64(a_l)[live], ro[live], rl[live], f32_out=True,
                 what="decode with empty sequences")


def test_more_sequences_than_the_launch_table():
    """300 sequences (above the 256 whose lengths travel with the launch):
    with host lengths the kernels read the device lengths; every sequence's
    bits equal those of a batch small enough for the launch table."""
    lens = (np.arange(300, dtype=np.int32) * 37) % 400 + 1
    cfg = gen.DecodeConfig(47, "decode, 300 sequences", batch=300, Hq=8, Hkv=2, D=128, page_size=16,
                           num_pages=8192, len_lo=1, len_hi=400, block=128)
    d = gen.decode_inputs(cfg, lengths=lens)
    say("[decode] 300 sequences")
    big_o, big_l = _decode(d, cfg, block=128)
    for seqs in (np.arange(0, 150), np.arange(150, 300)):
        o, l = _decode(d, cfg, block=128, seqs=seqs)
        assert_bitwise(o, big_o[seqs[0]:seqs[-1] + 1], f"Out of sequences {seqs[0]}..{seqs[-1]}")
        assert_bitwise(l, big_l[seqs[0]:seqs[-1] + 1], f"LSE of sequences {seqs[0]}..{seqs[-1]}")


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 4), (16, 2)], ids=["G1", "G2", "G8"])
def test_group_sizes_parity_and_prefill_identity(Hq, Hkv):
    """GQA groups of 1, 2 and 8 q heads per kv head (the decode kernel's MFMA
    columns, staged tail items and head-unit fold per q head): parity with the
    oracle and the last prefill row, bitwise, on lengths that end in the head
    unit, in a full tail unit and in a partial one."""
    lens = np.array([1, 200, 640, 1100, 1537], np.int32)
    cfg = gen.DecodeConfig(48, "decode group sizes", batch=lens.size, Hq=Hq, Hkv=Hkv, D=128, page_size=16,
                           num_pages=512, len_lo=1, len_hi=1600, block=128)
    d = gen.decode_inputs(cfg, lengths=lens)
    say(f"[decode] group size {Hq // Hkv}")
    do, dl = _decode(d, cfg, block=128, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged(d["q"], d["k_pool"], d["v_pool"], d["page_table"], d["ctx_lens"],
                                 scale=cfg.softmax_scale)
    check_parity(host_f64(do), host_f64(dl), ro, rl, f32_out=True, what=f"decode G={Hq // Hkv}")
    P = cfg.page_size
    for s, L in enumerate(lens.tolist()):
        pages = d["page_table"][s, : -(-L // P)]
        k = d["k_pool"][pages].transpose(0, 2, 1, 3).reshape(-1, Hkv, 128)[:L][None]
        v = d["v_pool"][pages].transpose(0, 2, 1, 3).reshape(-1, Hkv, 128)[:L][None]
        q = np.zeros((1, L, Hq, 128), np.uint16)
        q[0, L - 1] = d["q"][s]
        po, pl = api.prefill(dev_bf16(q), dev_bf16(k), dev_bf16(v), block=128, out_dtype=torch.float32)
        assert_bitwise(do[s], po[0, L - 1], f"G={Hq // Hkv} len {L} Out")
        assert_bitwise(dl[s], pl[0, L - 1], f"G={Hq // Hkv} len {L} LSE")
