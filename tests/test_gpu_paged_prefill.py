"""GPU paged chunked prefill: the keys of the chunk's queries gathered through
a page table.  Bit for bit equal to chunked prefill over the same keys in a
contiguous cache, for every page size, page placement, output mode and block
size; the padding slots of the last page hold NaN, which must never reach a
result (their V rows are cleared, their scores masked).  Also a direct parity
check against the FP64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from deterministic_gqa_attention_amd import api
from deterministic_gqa_attention_amd import inputs as gen
from tests.gpu_util import assert_bitwise, check_parity, dev_bf16, dev_i32, host_f64, say

pytestmark = pytest.mark.gpu

BF16_NAN = 0x7FC0


def _rand(seed, shape, scale=1.0):
    return gen.f64_to_bf16_bits(gen.normals(seed, shape) * scale)


def _paged(cache, P, seed):
    """Scatter a contiguous cache [B, S, Hkv, D] into a pool [pages, Hkv, P, D]
    through a seeded page permutation; slots past S hold NaN."""
    B, S, Hkv, D = cache.shape
    npp = -(-S // P)
    n_pages = B * npp + 3
    perm = np.random.Generator(np.random.PCG64(seed)).permutation(n_pages)
    pool = np.full((n_pages, Hkv, P, D), BF16_NAN, np.uint16)
    table = np.full((B, npp + 2), -1, np.int32)
    for b in range(B):
        for i in range(npp):
            page = perm[b * npp + i]
            table[b, i] = page
            rows = cache[b, i * P:(i + 1) * P]  # [<=P, Hkv, D]
            pool[page, :, :rows.shape[0]] = rows.transpose(1, 0, 2)
    return pool, table


CASES = [(0, 300), (130, 200), (513, 77), (640, 1), (128, 128)]  # the last ends on a block boundary


@pytest.mark.parametrize("block,pages", [(128, (4, 16, 64, 128)), (64, (4, 8, 16, 32, 64))])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_paged_equals_contiguous(block, pages, out_dtype):
    B, S, Hq, Hkv = 2, 720, 8, 2
    q, k, v = _rand(51, (B, S, Hq, 128)), _rand(52, (B, S, Hkv, 128)), _rand(53, (B, S, Hkv, 128))
    kd, vd = dev_bf16(k), dev_bf16(v)
    for c0, C in CASES:
        # the cache holds exactly the keys up to the chunk's end; the rest is NaN in both layouts
        kc, vc = k.copy(), v.copy()
        kc[:, c0 + C:] = BF16_NAN
        vc[:, c0 + C:] = BF16_NAN
        qc = dev_bf16(q[:, c0:c0 + C])
        say(f"[paged] block={block} out={out_dtype} cache={c0} chunk={C} contiguous")
        ro, rl = api.prefill_chunked(qc, dev_bf16(kc), dev_bf16(vc), cache_len=c0, block=block, out_dtype=out_dtype)
        assert torch.isfinite(ro.float()).all() and torch.isfinite(rl).all()
        for P in pages:
            kp, table = _paged(kc[:, :c0 + C], P, 1000 + P)
            vp, _ = _paged(vc[:, :c0 + C], P, 1000 + P)
            say(f"[paged]   page size {P}")
            o, l = api.prefill_paged(qc, dev_bf16(kp), dev_bf16(vp), dev_i32(table), cache_len=c0, block=block,
                                     out_dtype=out_dtype)
            assert_bitwise(o, ro, f"P={P} cache={c0} chunk={C} Out")
            assert_bitwise(l, rl, f"P={P} cache={c0} chunk={C} LSE")
    del kd, vd


def test_paged_relocation_and_batch():
    """Another page placement gives the same bits; so does a sequence alone."""
    B, S, Hq, Hkv = 3, 500, 8, 2
    q, k, v = _rand(54, (B, S, Hq, 128)), _rand(55, (B, S, Hkv, 128)), _rand(56, (B, S, Hkv, 128))
    c0, C = 200, 300
    qc = dev_bf16(q[:, c0:])
    outs = []
    for seed in (7, 8):
        kp, table = _paged(k, 16, seed)
        vp, _ = _paged(v, 16, seed)
        say(f"[paged] placement seed {seed}")
        outs.append(api.prefill_paged(qc, dev_bf16(kp), dev_bf16(vp), dev_i32(table), cache_len=c0, block=128))
        if seed == 7:
            o1, l1 = api.prefill_paged(qc[1:2].contiguous(), dev_bf16(kp), dev_bf16(vp), dev_i32(table[1:2]),
                                       cache_len=c0, block=128)
    assert_bitwise(outs[1][0], outs[0][0], "relocated Out")
    assert_bitwise(outs[1][1], outs[0][1], "relocated LSE")
    assert_bitwise(o1[0], outs[0][0][1], "sequence alone Out")
    assert_bitwise(l1[0], outs[0][1][1], "sequence alone LSE")


def test_paged_parity_with_oracle():
    q, k, v = _rand(57, (1, 400, 8, 128)), _rand(58, (1, 400, 2, 128)), _rand(59, (1, 400, 2, 128))
    c0, C = 257, 143
    kp, table = _paged(k, 32, 11)
    vp, _ = _paged(v, 32, 11)
    say("[paged] parity with the oracle")
    o, l = api.prefill_paged(dev_bf16(q[:, c0:]), dev_bf16(kp), dev_bf16(vp), dev_i32(table), cache_len=c0,
                             block=128, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q[:, c0:], k, v, scale=1 / np.sqrt(128), pos0=c0, kv_len=c0 + C)
    check_parity(host_f64(o).reshape(C, 8, 128), host_f64(l).reshape(C, 8), ro, rl, f32_out=True, what="paged")


@pytest.mark.parametrize("P,block,out_dtype", [(16, 128, torch.bfloat16), (32, 128, torch.bfloat16),
                                               (16, 64, torch.float32)], ids=["p16-bf16", "p32-bf16", "p16-fp32"])
def test_out_of_range_page_ids_are_clamped(P, block, out_dtype):
    """Ids below 0 read page 0 and ids at or past num_pages read the last
    page: the same bits as the table with those ids clamped."""
    B, S, Hq, Hkv = 1, 400, 8, 2
    q, k, v = _rand(60, (B, S, Hq, 128)), _rand(61, (B, S, Hkv, 128)), _rand(62, (B, S, Hkv, 128))
    kp, table = _paged(k, P, 2000 + P)
    vp, _ = _paged(v, P, 2000 + P)
    # finite values in the unused pages, which a clamped id may land on
    kp = np.where(kp == BF16_NAN, np.uint16(0x3F80), kp)
    vp = np.where(vp == BF16_NAN, np.uint16(0x3F80), vp)
    n_pages = kp.shape[0]
    bad, clamped = table.copy(), table.copy()
    for i, (b_id, c_id) in enumerate([(-3, 0), (n_pages + 10, n_pages - 1), (-(1 << 30), 0),
                                      (1 << 30, n_pages - 1)]):
        bad[0, 2 + 3 * i] = b_id
        clamped[0, 2 + 3 * i] = c_id
    qc = dev_bf16(q[:, 100:])
    say(f"[paged] out-of-range page ids P={P} block={block} out={out_dtype}")
    ro, rl = api.prefill_paged(qc, dev_bf16(kp), dev_bf16(vp), dev_i32(clamped), cache_len=100, block=block,
                               out_dtype=out_dtype)
    o, l = api.prefill_paged(qc, dev_bf16(kp), dev_bf16(vp), dev_i32(bad), cache_len=100, block=block,
                             out_dtype=out_dtype)
    assert_bitwise(o, ro, "Out with out-of-range ids")
    assert_bitwise(l, rl, "LSE with out-of-range ids")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_non_causal_chunk_parity_and_paged(out_dtype):
    """A non-causal chunk (every query sees all cache_len + chunk_len keys,
    also those of later chunk positions): parity of the contiguous chunked
    path with the oracle, and the paged path (16- and 32-key pages) equal to
    it bit for bit."""
    B, S, Hq, Hkv = 2, 330, 8, 2
    c0, C = 200, 130
    q, k, v = _rand(63, (B, S, Hq, 128)), _rand(64, (B, S, Hkv, 128)), _rand(65, (B, S, Hkv, 128))
    qc = dev_bf16(q[:, c0:c0 + C])
    say(f"[paged] non-causal chunk cache={c0} chunk={C} out={out_dtype}")
    ro, rl = api.prefill_chunked(qc, dev_bf16(k), dev_bf16(v), cache_len=c0, block=128, out_dtype=out_dtype,
                                 causal=False)
    torch.cuda.synchronize()
    eo, el = oracle.attention(q[:, c0:c0 + C], k, v, scale=1 / np.sqrt(128), pos0=c0, kv_len=c0 + C, causal=False)
    check_parity(host_f64(ro).reshape(B * C, Hq, 128), host_f64(rl).reshape(B * C, Hq), eo, el,
                 f32_out=out_dtype == torch.float32, what="non-causal chunk")
    for P in (16, 32):
        kp, table = _paged(k, P, 3000 + P)
        vp, _ = _paged(v, P, 3000 + P)
        o, l = api.prefill_paged(qc, dev_bf16(kp), dev_bf16(vp), dev_i32(table), cache_len=c0, block=128,
                                 out_dtype=out_dtype, causal=False)
        assert_bitwise(o, ro, f"P={P} non-causal Out")
        assert_bitwise(l, rl, f"P={P} non-causal LSE")
