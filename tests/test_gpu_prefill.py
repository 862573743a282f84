"""GPU prefill parity against the FP64 oracle (through the C ABI).

Every case checks every row of Out and LSE except the S=32768 workload, which
checks rows stratified over every 32-row tile plus the first and last blocks.
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


def _run_and_check(q, k, v, *, block, out_dtype, scale=None, causal=True, rows=None, what=""):
    B, S, Hq, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    say(f"[prefill] {what} B={B} S={S} Hq={Hq} Hkv={k.shape[2]} block={block} out={out_dtype} causal={causal}")
    out, lse = api.prefill(dev_bf16(q), dev_bf16(k), dev_bf16(v), block=block, out_dtype=out_dtype,
                           causal=causal, scale=scale)
    torch.cuda.synchronize()
    flat_rows = None if rows is None else rows
    o_ref, l_ref = oracle.attention(q, k, v, scale=scale, causal=causal, rows=flat_rows)
    og = host_f64(out).reshape(B * S, Hq, D)
    lg = host_f64(lse).reshape(B * S, Hq)
    if rows is not None:
        og, lg = og[rows], lg[rows]
    stats = check_parity(og, lg, o_ref, l_ref, f32_out=out_dtype == torch.float32, what=what)
    say(f"    parity {stats}")
    return out, lse


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_tiny_causal_prefill_tp2_shard(out_dtype):
    """Qwen3-8B TP=2 local shard (Hq=16, Hkv=4), S=256, NeoX RoPE on Q/K, 64-key
    blocks: every row against the oracle, both output modes."""
    cfg = gen.CFG1
    q, k, v = gen.prefill_inputs(cfg)
    out, lse = _run_and_check(q, k, v, block=cfg.block, out_dtype=out_dtype, what="tiny TP=2 shard")
    # single-key row: row 0 sees only key 0.  Its weight is 2^e with e the
    # rounding error of dot*c (below 2^-23), so bf16 Out is V row 0 exactly and
    # fp32 Out is V row 0 to within 2 ulp.
    v0 = torch.from_numpy(gen.bf16_bits_to_f32(v[0, 0])).cuda()        # [Hkv, D]
    g = cfg.Hq // cfg.Hkv
    for h in range(cfg.Hq):
        got = out[0, 0, h].float()
        want = v0[h // g]
        if out_dtype == torch.bfloat16:
            assert torch.equal(got, want), f"row 0 head {h} is not V row 0"
        else:
            assert torch.all((got - want).abs() <= 2.4e-7 * want.abs()), f"row 0 head {h} differs from V row 0"


@pytest.mark.parametrize("block", [64, 128])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_ragged_multi_tile(block, out_dtype):
    """Several position tiles and KV blocks with a ragged tail (S=300), B=2."""
    q, k, v = _rand(1, (2, 300, 8, 128)), _rand(2, (2, 300, 2, 128)), _rand(3, (2, 300, 2, 128))
    _run_and_check(q, k, v, block=block, out_dtype=out_dtype, what="ragged multi-tile")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (16, 2)], ids=["mha", "gqa2", "gqa8"])
def test_group_sizes(Hq, Hkv, out_dtype):
    """GQA groups other than 4 (MHA, 2, 8) map heads to kv heads correctly (the
    workgroup then holds 8 position groups of one head, 4 of two heads, or one
    of eight heads)."""
    q, k, v = _rand(4, (1, 200, Hq, 128)), _rand(5, (1, 200, Hkv, 128)), _rand(6, (1, 200, Hkv, 128))
    _run_and_check(q, k, v, block=128, out_dtype=out_dtype, what=f"group Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_grouped_tile_order_ragged(out_dtype):
    """B*Hkv = 16 takes the grouped tile order (each XCD's (b, kv head) pairs
    two at a time); with 5 position tiles of which the last is ragged, every
    row still matches the oracle."""
    q, k, v = _rand(16, (2, 300, 32, 128)), _rand(17, (2, 300, 8, 128)), _rand(18, (2, 300, 8, 128))
    _run_and_check(q, k, v, block=128, out_dtype=out_dtype, what="grouped tile order, ragged")


@pytest.mark.parametrize("block", [64, 128])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_non_causal(block, out_dtype):
    q, k, v = _rand(7, (1, 150, 8, 128)), _rand(8, (1, 150, 2, 128)), _rand(9, (1, 150, 2, 128))
    _run_and_check(q, k, v, block=block, out_dtype=out_dtype, causal=False, what="non-causal")


def test_peaky_scores():
    """Q and K scaled by 4 (peaky softmax, score std ~16)."""
    q, k, v = _rand(10, (1, 640, 8, 128), 4.0), _rand(11, (1, 640, 2, 128), 4.0), _rand(12, (1, 640, 2, 128))
    _run_and_check(q, k, v, block=128, out_dtype=torch.bfloat16, what="peaky x4")
    _run_and_check(q, k, v, block=128, out_dtype=torch.float32, what="peaky x4")


def test_single_token():
    q, k, v = _rand(13, (3, 1, 32, 128)), _rand(14, (3, 1, 8, 128)), _rand(15, (3, 1, 8, 128))
    out, lse = _run_and_check(q, k, v, block=128, out_dtype=torch.bfloat16, what="S=1")
    vv = torch.from_numpy(gen.bf16_bits_to_f32(v)).cuda()
    assert torch.equal(out[:, 0].float(), vv[:, 0].repeat_interleave(4, dim=1))


def test_repeat_run_bitwise():
    q, k, v = _rand(16, (2, 257, 8, 128)), _rand(17, (2, 257, 2, 128)), _rand(18, (2, 257, 2, 128))
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    say("[prefill] repeat-run bitwise")
    a = api.prefill(qd, kd, vd, block=128)
    b = api.prefill(qd, kd, vd, block=128)
    assert_bitwise(a[0], b[0], "repeat Out")
    assert_bitwise(a[1], b[1], "repeat LSE")


@pytest.mark.slow
def test_full_prefill_b4_s4096_all_rows():
    """Full causal prefill B=4, S=4096, Hq=32, Hkv=8, 128-key blocks, bf16 Out
    (the timed workload and launch): every row of Out and LSE against the
    oracle."""
    cfg = gen.CFG2
    q, k, v = gen.prefill_inputs(cfg)
    _run_and_check(q, k, v, block=cfg.block, out_dtype=torch.bfloat16, what="B=4 S=4096 all rows")


def stratified_rows(S: int, tile: int = 32, block: int = 128) -> np.ndarray:
    """Rows of a long sequence covering every tile of `tile` rows (two rows per
    tile, so every offset within a tile occurs S / tile / 16 times), plus every
    row of the first and the last KV block."""
    t = np.arange(S // tile, dtype=np.int64)
    rows = np.concatenate([t * tile + t % tile, t * tile + (t * 7 + 13) % tile,
                           np.arange(block), np.arange(S - block, S)])
    return np.unique(rows)


@pytest.mark.slow
def test_long_context_s32768_stratified():
    """S=32768, Q/K scaled by 4, 128-key blocks, bf16 Out + LSE: 2048 rows that
    cover every 32-row tile and every offset within a tile, plus the first and
    last 128-key blocks in full, against the oracle."""
    cfg = gen.CFG5
    q, k, v = gen.prefill_inputs(cfg)
    rows = stratified_rows(cfg.S)
    assert len(rows) >= 2048
    _run_and_check(q, k, v, block=cfg.block, out_dtype=torch.bfloat16, rows=rows, what="S=32768 x4 stratified")
