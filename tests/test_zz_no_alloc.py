"""rla_attn_decode_paged_static (block items in the library's fixed device
array, no workspace): the same bits as rla_attn_decode_paged, on two calls in
a row through the C ABI, the second with a smaller input (the array keeps the
first call's items, which must not leak into the second)."""
import numpy as np
import pytest
import torch

from deterministic_gqa_attention_amd import api
from deterministic_gqa_attention_amd import inputs as gen
from tests.gpu_util import assert_bitwise, dev_bf16, dev_i32, say

pytestmark = pytest.mark.gpu

SMALL = gen.DecodeConfig(43, "small paged decode", batch=5, Hq=8, Hkv=2, D=128, page_size=16, num_pages=256,
                         len_lo=1, len_hi=600, block=128)


def _both(d, cfg, *, out_dtype):
    kp, vp = dev_bf16(d["k_pool"]), dev_bf16(d["v_pool"])
    q, table, lens = dev_bf16(d["q"]), dev_i32(d["page_table"]), dev_i32(d["ctx_lens"])
    kw = dict(block=cfg.block, max_context_len=int(cfg.len_hi), host_ctx_lens=d["ctx_lens"], out_dtype=out_dtype)
    ref = api.decode_paged(q, kp, vp, table, lens, **kw)
    got = api.decode_paged_static(q, kp, vp, table, lens, **kw)
    torch.cuda.synchronize()
    return ref, got


def test_static_decode_equals_workspace_decode_two_calls():
    cfg = gen.CFG4
    say("[no-alloc] call 1: 64 sequences, lengths U[512, 16384], bf16 Out")
    d = gen.decode_inputs(cfg)
    (ro, rl), (go, gl) = _both(d, cfg, out_dtype=torch.bfloat16)
    assert_bitwise(go, ro, "static vs workspace decode Out (64 sequences)")
    assert_bitwise(gl, rl, "static vs workspace decode LSE (64 sequences)")
    del d
    torch.cuda.empty_cache()
    for out_dtype in (torch.float32, torch.bfloat16):
        say(f"[no-alloc] smaller call: 5 sequences, lengths 1..600, {out_dtype}")
        d = gen.decode_inputs(SMALL, lengths=np.array([1, 129, 600, 256, 64], np.int32))
        (ro, rl), (go, gl) = _both(d, SMALL, out_dtype=out_dtype)
        assert_bitwise(go, ro, "static vs workspace decode Out (5 sequences)")
        assert_bitwise(gl, rl, "static vs workspace decode LSE (5 sequences)")
