"""GPU backward (dQ, dK, dV) against the FP64 oracle, and its bitwise
invariances, through the C ABI.

Parity bar.  The oracle reports with each gradient element mag, the sum of
the absolute values of its terms, each widened by the part of dS an error in
Delta can move (p * sum_j p_j |dP_j|).  Each term carries at most one bf16
rounding in the kernels (unit roundoff 2^-8): P as the dV operand, scale*dS as
the dQ and dK operand.  Delta comes from the bf16 forward output, whose
rounding moves it by at most 2^-8 * sum_d |dOut_d||Out_d| <= 2^-8 *
sum_j p_j |dP_j|, inside the widening.  FP32 accumulation adds at most about
n * 2^-24 relative over n <= 2^14 terms (2^-10).  So |gpu - oracle| <=
(2^-8 + 2^-10) * mag, and the test requires 2^-7 * mag.  tests/test_grad_bar.py
shows on the CPU that a model of these roundings stays well inside this bar
while plausible mistakes (Delta from the wrong row, a dropped scale, ...)
exceed it several times over.
"""
import numpy as np
import pytest
import torch

import oracle
from deterministic_gqa_attention_amd import api
from deterministic_gqa_attention_amd import inputs as gen
from tests.gpu_util import assert_bitwise, dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu

GRAD_FACTOR = 2.0 ** -7
GRAD_FLOOR = 1e-12


def _rand(seed, shape, scale=1.0):
    return gen.f64_to_bf16_bits(gen.normals(seed, shape) * scale)


def _inputs(seed, B, Sq, Skv, Hq, Hkv, qk_scale=1.0):
    q = _rand(seed, (B, Sq, Hq, 128), qk_scale)
    k = _rand(seed + 1, (B, Skv, Hkv, 128), qk_scale)
    v = _rand(seed + 2, (B, Skv, Hkv, 128))
    do = _rand(seed + 3, (B, Sq, Hq, 128))
    return q, k, v, do


def _forward(qd, kd, vd, *, cache_len, causal, out_dtype, scale):
    if cache_len == 0 and qd.shape[1] == kd.shape[1]:
        return api.prefill(qd, kd, vd, block=128, out_dtype=out_dtype, causal=causal, scale=scale)
    return api.prefill_chunked(qd, kd, vd, cache_len=cache_len, block=128, out_dtype=out_dtype, causal=causal,
                               scale=scale)


def _check(got, ref, mag, what):
    g = host_f64(got).reshape(ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    err = np.abs(g - ref)
    bound = GRAD_FACTOR * mag + GRAD_FLOOR
    bad = err > bound
    ratio = float((err / np.maximum(bound, 1e-30)).max(initial=0.0))
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements exceed 2^-7 * mag; max abs err "
                           f"{err.max():.3e}, worst err/bound {ratio:.3f}")
    return float(err.max(initial=0.0)), ratio


def _parity_case(seed, B, Sq, Hq, Hkv, *, cache_len=0, s_max=None, causal=True, out_dtype=torch.bfloat16,
                 qk_scale=1.0, what=""):
    kv_len = cache_len + Sq
    s_max = kv_len if s_max is None else s_max
    q, k, v, do = _inputs(seed, B, Sq, s_max, Hq, Hkv, qk_scale)
    scale = 1.0 / np.sqrt(128.0)
    say(f"[backward] {what}: B={B} Sq={Sq} cache={cache_len} s_max={s_max} Hq={Hq} Hkv={Hkv} causal={causal} "
        f"out={out_dtype}")
    qd, kd, vd, dod = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
    out, lse = _forward(qd, kd, vd, cache_len=cache_len, causal=causal, out_dtype=out_dtype, scale=scale)
    dq, dk, dv = api.backward(qd, kd, vd, out, lse, dod, cache_len=cache_len, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv, mq, mk, mv = oracle.attention_backward(q, k, v, do, scale=scale, causal=causal, pos0=cache_len,
                                                       kv_len=kv_len, mags=True)
    stats = [_check(dq, rq, mq, f"{what} dQ"), _check(dk, rk, mk, f"{what} dK"), _check(dv, rv, mv, f"{what} dV")]
    say(f"    max abs err / worst err-to-bound: dQ {stats[0]}, dK {stats[1]}, dV {stats[2]}")
    # keys past kv_len are not touched
    if s_max > kv_len:
        assert not dk[:, kv_len:].any() and not dv[:, kv_len:].any(), f"{what}: keys past kv_len written"
    return (q, k, v, do), (out, lse), (dq, dk, dv)


def test_backward_parity_gqa4_causal_ragged():
    """Qwen3-8B grouping (G=4), causal, 200 rows: three full 64-row tiles and a
    ragged one; two batch rows."""
    _parity_case(11, 2, 200, 8, 2, what="G4 causal ragged")


def test_backward_parity_grouped_tile_order():
    """B*Hkv = 16: the dQ walk takes the grouped tile order; 4 row tiles, the
    last ragged."""
    _parity_case(12, 2, 200, 32, 8, what="grouped tile order")


def test_backward_parity_tp2_shard_fp32_out_noncausal():
    """The TP=2 local head shard (Hq=16, Hkv=4), non-causal, forward Out in fp32."""
    _parity_case(21, 1, 160, 16, 4, causal=False, out_dtype=torch.float32, what="TP2 non-causal fp32 Out")


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (16, 2)], ids=["G1", "G2", "G8"])
def test_backward_parity_groupings(Hq, Hkv):
    """Other GQA groupings: the dQ kernel's head subgroups and idle waves, the
    dK/dV walk over G heads per tile."""
    _parity_case(31 + Hq, 1, 130, Hq, Hkv, what=f"Hq={Hq} Hkv={Hkv}")


def test_backward_parity_chunk_after_cache():
    """A chunk of 72 queries after 128 cached keys, in a cache of 256 slots
    (keys past the chunk must stay untouched)."""
    _parity_case(41, 2, 72, 8, 2, cache_len=128, s_max=256, what="chunk after cache")


def test_backward_parity_noncausal_chunk():
    """A non-causal chunk of 72 queries after 64 cached keys (every query sees
    all 136 keys) in a cache of 200 slots."""
    _parity_case(43, 2, 72, 8, 2, cache_len=64, s_max=200, causal=False, what="non-causal chunk")


def test_backward_noncausal_replay_bitwise():
    """Non-causal replay: rows [0,128) then [128,200), each chunk seeing all
    200 keys, accumulate into dK/dV and give the single call's bits."""
    B, S, Hq, Hkv = 1, 200, 8, 2
    q, k, v, do = _inputs(44, B, S, S, Hq, Hkv)
    scale = 1.0 / np.sqrt(128.0)
    qd, kd, vd, dod = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
    out, lse = api.prefill(qd, kd, vd, block=128, causal=False, scale=scale)
    ref = api.backward(qd, kd, vd, out, lse, dod, causal=False, scale=scale)
    dk = torch.zeros_like(ref[1])
    dv = torch.zeros_like(ref[2])
    dqs = []
    for c0, c1 in ((0, 128), (128, 200)):
        # a chunk sees the keys [0, cache_len + rows): with cache_len = S - rows
        # that is all S keys, as in the single call (without a causal mask the
        # rows' positions do not matter)
        n = c1 - c0
        dq_c, _, _ = api.backward(qd[:, c0:c1].contiguous(), kd, vd, out[:, c0:c1].contiguous(),
                                  lse[:, c0:c1].contiguous(), dod[:, c0:c1].contiguous(), cache_len=S - n,
                                  causal=False, scale=scale, dk=dk, dv=dv, accumulate=True)
        dqs.append(dq_c)
    assert_bitwise(torch.cat(dqs, dim=1), ref[0], "non-causal replay dQ")
    assert_bitwise(dk, ref[1], "non-causal replay dK")
    assert_bitwise(dv, ref[2], "non-causal replay dV")


def test_backward_bf16_gradients_are_rounded_fp32():
    """bf16 gradient output is the round-to-nearest-even of the fp32 result,
    element for element (the downcast is the final write and nothing else)."""
    B, S, Hq, Hkv = 2, 200, 8, 2
    q, k, v, do = _inputs(45, B, S, S, Hq, Hkv)
    qd, kd, vd, dod = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
    out, lse = api.prefill(qd, kd, vd, block=128)
    g32 = api.backward(qd, kd, vd, out, lse, dod)
    g16 = api.backward(qd, kd, vd, out, lse, dod, grad_dtype=torch.bfloat16)
    for a32, a16, n in zip(g32, g16, "qkv"):
        assert a16.dtype == torch.bfloat16
        assert_bitwise(a16, a32.to(torch.bfloat16), f"bf16 d{n}")


def test_backward_parity_peaky_scores():
    """Large scores (Q and K scaled by 4): probabilities near 0 and 1, where dS
    is most sensitive to the rounding of P."""
    _parity_case(51, 1, 192, 8, 2, qk_scale=4.0, what="peaky")


@pytest.mark.parametrize("S", [1, 63, 64, 65])
def test_backward_parity_edge_lengths(S):
    """Single row, one row short of a tile, exactly one tile, one row over."""
    _parity_case(61 + S, 1, S, 8, 2, what=f"S={S}")


def test_backward_bitwise_invariances():
    """Run-to-run, batch makeup, TP head shard and chunked replay (accumulate
    mode, chunk boundaries on 64-row tiles) all give bit-identical dQ/dK/dV."""
    B, S, Hq, Hkv = 3, 600, 32, 8
    q, k, v, do = _inputs(71, B, S, S, Hq, Hkv)
    scale = 1.0 / np.sqrt(128.0)
    qd, kd, vd, dod = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
    say(f"[backward] invariances B={B} S={S} Hq={Hq} Hkv={Hkv}")
    out, lse = api.prefill(qd, kd, vd, block=128, scale=scale)
    ref = api.backward(qd, kd, vd, out, lse, dod, scale=scale)
    again = api.backward(qd, kd, vd, out, lse, dod, scale=scale)
    for a, b_, n in zip(ref, again, "qkv"):
        assert_bitwise(a, b_, f"run-to-run d{n}")
    # batch makeup: each sequence alone
    for b in range(B):
        one = api.backward(qd[b:b + 1].contiguous(), kd[b:b + 1].contiguous(), vd[b:b + 1].contiguous(),
                           out[b:b + 1].contiguous(), lse[b:b + 1].contiguous(), dod[b:b + 1].contiguous(),
                           scale=scale)
        for a, b_, n in zip(one, ref, "qkv"):
            assert_bitwise(a, b_[b:b + 1], f"batch row {b} alone d{n}")
    # TP=2 head shard: the first half of the heads alone
    h2, k2 = Hq // 2, Hkv // 2
    shard = api.backward(qd[:, :, :h2].contiguous(), kd[:, :, :k2].contiguous(), vd[:, :, :k2].contiguous(),
                         out[:, :, :h2].contiguous(), lse[:, :, :h2].contiguous(), dod[:, :, :h2].contiguous(),
                         scale=scale)
    assert_bitwise(shard[0], ref[0][:, :, :h2].contiguous(), "TP shard dQ")
    assert_bitwise(shard[1], ref[1][:, :, :k2].contiguous(), "TP shard dK")
    assert_bitwise(shard[2], ref[2][:, :, :k2].contiguous(), "TP shard dV")
    # chunked replay with accumulation
    dk = torch.zeros_like(ref[1])
    dv = torch.zeros_like(ref[2])
    dqs = []
    for c0, c1 in ((0, 192), (192, 448), (448, 600)):
        say(f"    replay chunk [{c0}, {c1})")
        dq_c, _, _ = api.backward(qd[:, c0:c1].contiguous(), kd, vd, out[:, c0:c1].contiguous(),
                                  lse[:, c0:c1].contiguous(), dod[:, c0:c1].contiguous(), cache_len=c0,
                                  scale=scale, dk=dk, dv=dv, accumulate=True)
        dqs.append(dq_c)
    assert_bitwise(torch.cat(dqs, dim=1), ref[0], "replay dQ")
    assert_bitwise(dk, ref[1], "replay dK")
    assert_bitwise(dv, ref[2], "replay dV")


@pytest.mark.slow
def test_backward_full_size_sampled():
    """The benchmarked workload (B=4, S=4096, Hq=32, Hkv=8, causal): dQ of
    sampled rows against the oracle; dV against the identity
    sum_j dV_j = sum_i dOut_i (each probability row sums to 1), within the
    bf16 rounding of P; chunked replay in 2048-row chunks bitwise equal."""
    cfg = gen.CFG2
    q, k, v = gen.prefill_inputs(cfg)
    do = gen.dout_inputs(cfg)
    scale = cfg.softmax_scale
    say(f"[backward] full size B={cfg.B} S={cfg.S}")
    qd, kd, vd, dod = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
    out, lse = api.prefill(qd, kd, vd, block=cfg.block, scale=scale)
    dq, dk, dv = api.backward(qd, kd, vd, out, lse, dod, scale=scale)
    torch.cuda.synchronize()
    S = cfg.S
    rows_t = np.array([0, 1, 63, 64, 65, 127, 128, 2047, 2048, 2049, 4030, 4095], np.int64)
    rows = np.concatenate([b * S + rows_t for b in (0, 3)])
    rq, _, _, mq, _, _ = oracle.attention_backward(q, k, v, do, scale=scale, rows=rows, mags=True)
    flat = lambda a: a.reshape(cfg.B * S, cfg.Hq, 128)[rows]
    _check(flat(dq), flat(rq), flat(mq), "full-size dQ rows")
    g = cfg.Hq // cfg.Hkv
    dof = gen.bf16_bits_to_f32(do).astype(np.float64).reshape(cfg.B, S, cfg.Hkv, g, 128)
    want = dof.sum(axis=(1, 3))
    bound = 2.0 ** -7 * np.abs(dof).sum(axis=(1, 3)) + 1e-6
    got = host_f64(dv).sum(axis=1)
    assert (np.abs(got - want) <= bound).all(), \
        f"sum of dV deviates from sum of dOut: {np.abs(got - want).max():.3e}"
    dk2 = torch.zeros_like(dk)
    dv2 = torch.zeros_like(dv)
    dqs = []
    for c0 in (0, 2048):
        dq_c, _, _ = api.backward(qd[:, c0:c0 + 2048].contiguous(), kd, vd, out[:, c0:c0 + 2048].contiguous(),
                                  lse[:, c0:c0 + 2048].contiguous(), dod[:, c0:c0 + 2048].contiguous(),
                                  cache_len=c0, scale=scale, dk=dk2, dv=dv2, accumulate=True)
        dqs.append(dq_c)
    assert_bitwise(torch.cat(dqs, dim=1), dq, "full-size replay dQ")
    assert_bitwise(dk2, dk, "full-size replay dK")
    assert_bitwise(dv2, dv, "full-size replay dV")


@pytest.mark.slow
def test_backward_long_context_zigzag_replay():
    """The long-context workload (B=1, S=32768, Q and K drawn x4, causal):
    dQ of sampled rows against the oracle, the dV row-sum identity, and a
    replay of the query rows in the zigzag CP=2 ownership order (shard 0 owns
    quarters 0 and 3, shard 1 quarters 1 and 2; dK/dV handed on in ascending
    row order) bitwise equal to one call."""
    cfg = gen.CFG5
    q, k, v = gen.prefill_inputs(cfg)
    do = gen.dout_inputs(cfg)
    scale = cfg.softmax_scale
    S = cfg.S
    say(f"[backward] long context S={S}")
    qd, kd, vd, dod = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
    out, lse = api.prefill(qd, kd, vd, block=cfg.block, scale=scale)
    dq, dk, dv = api.backward(qd, kd, vd, out, lse, dod, scale=scale)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 8191, 8192, 16383, 16384, 24575, 24576, 32766, 32767], np.int64)
    rq, _, _, mq, _, _ = oracle.attention_backward(q, k, v, do, scale=scale, rows=rows, mags=True)
    _check(dq.reshape(S, cfg.Hq, 128)[rows], rq.reshape(S, cfg.Hq, 128)[rows],
           mq.reshape(S, cfg.Hq, 128)[rows], "long-context dQ rows")
    g = cfg.Hq // cfg.Hkv
    dof = gen.bf16_bits_to_f32(do).astype(np.float64).reshape(1, S, cfg.Hkv, g, 128)
    got = host_f64(dv).sum(axis=1)
    assert (np.abs(got - dof.sum(axis=(1, 3))) <= 2.0 ** -7 * np.abs(dof).sum(axis=(1, 3)) + 1e-6).all()
    quarter = S // 4
    dk2 = torch.zeros_like(dk)
    dv2 = torch.zeros_like(dv)
    dq2 = torch.empty_like(dq)
    for owner, c in ((0, 0), (1, 1), (1, 2), (0, 3)):  # ascending rows, alternating owners
        c0, c1 = c * quarter, (c + 1) * quarter
        say(f"    shard {owner} rows [{c0}, {c1})")
        part, _, _ = api.backward(qd[:, c0:c1].contiguous(), kd, vd, out[:, c0:c1].contiguous(),
                                  lse[:, c0:c1].contiguous(), dod[:, c0:c1].contiguous(), cache_len=c0, scale=scale,
                                  dk=dk2, dv=dv2, accumulate=True)
        dq2[:, c0:c1] = part
    assert_bitwise(dq2, dq, "zigzag replay dQ")
    assert_bitwise(dk2, dk, "zigzag replay dK")
    assert_bitwise(dv2, dv, "zigzag replay dV")
