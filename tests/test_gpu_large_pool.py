"""Page pools larger than 4 GiB (GPU).

A page's byte offset in the pool, page_id * Hkv * page_size * 256, passes
2^32 once the pool holds more than 4 GiB, so it must be formed in 64-bit
arithmetic.  Here the pages of a few sequences are moved to the top of a
5.5 GiB pool, one of them starting exactly at the 4 GiB offset and one just
below it; decode and paged prefill must give the same bits as with the pages
in a small pool (decode) or as the contiguous chunked path (prefill).
"""
import numpy as np
import pytest
import torch

from deterministic_gqa_attention_amd import api
from deterministic_gqa_attention_amd import inputs as gen
from tests.gpu_util import assert_bitwise, dev_bf16, dev_i32, say

pytestmark = pytest.mark.gpu

HQ, HKV, D = 8, 2, 128
POOL_BYTES = 11 << 29  # 5.5 GiB per pool


def _high_ids(n, page_bytes):
    """n distinct page ids: the page at byte offset 2^32, the one below it,
    then the top of the pool downwards."""
    big = POOL_BYTES // page_bytes
    at4g = (1 << 32) // page_bytes
    ids = [at4g, at4g - 1] + [big - 1 - i for i in range(max(n - 2, 0))]
    assert len(set(ids)) == len(ids) and max(ids) < big
    return np.array(ids[:n], np.int64), big


def _relocate(table, kp, vp, page_bytes):
    """Copy the pages the table uses into fresh pools of POOL_BYTES, at the
    ids of _high_ids; returns the new table and pools (device)."""
    used = [int(p) for p in table.ravel() if p >= 0]
    new, big = _high_ids(len(used), page_bytes)
    remap = dict(zip(used, new.tolist()))
    t2 = np.where(table >= 0, np.vectorize(lambda p: remap.get(int(p), -1))(table), -1).astype(np.int32)
    shape = (big,) + tuple(kp.shape[1:])
    bk = torch.empty(shape, dtype=torch.bfloat16, device=kp.device)
    bv = torch.empty(shape, dtype=torch.bfloat16, device=kp.device)
    src = torch.tensor(used, dtype=torch.long, device=kp.device)
    dst = torch.from_numpy(new).to(kp.device)
    bk[dst] = kp[src]
    bv[dst] = vp[src]
    return t2, bk, bv


def test_decode_pool_beyond_4gib():
    P = 16
    lens = np.array([1, 200, 1500, 4100], np.int32)
    need = int((-(-lens.astype(np.int64) // P)).sum())
    cfg = gen.DecodeConfig(51, "decode, pool beyond 4 GiB", batch=lens.size, Hq=HQ, Hkv=HKV, D=D, page_size=P,
                           num_pages=need + 8, len_lo=1, len_hi=4100, block=128)
    d = gen.decode_inputs(cfg, lengths=lens)
    kp, vp = dev_bf16(d["k_pool"]), dev_bf16(d["v_pool"])
    q, ctx = dev_bf16(d["q"]), dev_i32(d["ctx_lens"])
    say("[large pool] decode, small pool")
    ro, rl = api.decode_paged(q, kp, vp, dev_i32(d["page_table"]), ctx, block=128, max_context_len=4100,
                              host_ctx_lens=lens)
    t2, bk, bv = _relocate(d["page_table"], kp, vp, HKV * P * D * 2)
    say(f"[large pool] decode, {bk.shape[0]}-page pool, pages from id {int(t2[t2 >= 0].min())}")
    for host in (lens, None):  # host length table, then lengths read on the device
        o, l = api.decode_paged(q, bk, bv, dev_i32(t2), ctx, block=128, max_context_len=4100, host_ctx_lens=host)
        assert_bitwise(o, ro, "decode Out, pages past 4 GiB")
        assert_bitwise(l, rl, "decode LSE, pages past 4 GiB")
    del bk, bv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("P", [16, 32])
def test_paged_prefill_pool_beyond_4gib(P):
    S, c0 = 1500, 1200
    q = gen.f64_to_bf16_bits(gen.normals(5101, (1, S, HQ, D)))
    k = gen.f64_to_bf16_bits(gen.normals(5102, (1, S, HKV, D)))
    v = gen.f64_to_bf16_bits(gen.normals(5103, (1, S, HKV, D)))
    qc = dev_bf16(q[:, c0:])
    say(f"[large pool] paged prefill P={P}, contiguous reference")
    ro, rl = api.prefill_chunked(qc, dev_bf16(k), dev_bf16(v), cache_len=c0, block=128)
    npp = -(-S // P)
    pad = np.zeros((npp * P - S, HKV, D), np.uint16)
    kpages = np.concatenate([k[0], pad]).reshape(npp, P, HKV, D).transpose(0, 2, 1, 3)
    vpages = np.concatenate([v[0], pad]).reshape(npp, P, HKV, D).transpose(0, 2, 1, 3)
    table = np.arange(npp, dtype=np.int32).reshape(1, npp)
    t2, bk, bv = _relocate(table, dev_bf16(np.ascontiguousarray(kpages)), dev_bf16(np.ascontiguousarray(vpages)),
                           HKV * P * D * 2)
    say(f"[large pool] paged prefill P={P}, {bk.shape[0]}-page pool")
    o, l = api.prefill_paged(qc, bk, bv, dev_i32(t2), cache_len=c0, block=128)
    assert_bitwise(o, ro, f"paged prefill Out, P={P}, pages past 4 GiB")
    assert_bitwise(l, rl, f"paged prefill LSE, P={P}, pages past 4 GiB")
    del bk, bv
    torch.cuda.empty_cache()
