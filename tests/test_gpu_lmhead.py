"""GPU selected log-probabilities through the FP32 lm_head against the FP64
oracle, and the decode/prefill dlogp identity, through the C ABI.

Parity bar.  Each logit is an FP32 accumulation of H exact-product terms, so
|dz_v| <= H 2^-24 sum_h |x_h||W_vh| <= H 2^-24 mag (mag from the oracle: the
largest such sum over the vocabulary); log-sum-exp is 1-Lipschitz in every
logit, and its own FP32 evaluation (exponentials, block sums, fold, log) adds
well under 1e-5 (1 + |logZ|).  The test requires
|gpu - oracle| <= 2 H 2^-24 mag + 1e-5 (1 + |logZ|) for logp and logZ.
"""
import numpy as np
import pytest
import torch

import oracle
from deterministic_gqa_attention_amd import api
from deterministic_gqa_attention_amd import inputs as gen
from tests.gpu_util import assert_bitwise, dev_bf16, dev_i32, say

pytestmark = pytest.mark.gpu


def _bound(H, mag, logz):
    return 2.0 * H * 2.0 ** -24 * mag + 1e-5 * (1.0 + np.abs(logz))


def _case(T, H, V, *, xf32=False, seed=0, what=""):
    rng = np.random.Generator(np.random.PCG64(900 + seed))
    x = gen.f64_to_bf16_bits(rng.standard_normal((T, H)))
    w = gen.lm_head_weights(V, H, seed=910 + seed)
    tok = rng.integers(0, V, T).astype(np.int32)
    tok[0] = 0
    tok[-1] = V - 1
    say(f"[lm_head] {what}: T={T} H={H} V={V} x={'fp32' if xf32 else 'bf16'}")
    if xf32:
        xh = gen.bf16_bits_to_f32(x)
        xd = torch.from_numpy(xh).cuda()
    else:
        xh = x
        xd = dev_bf16(x)
    lp, lz = api.lm_head_logprobs(xd, torch.from_numpy(w).cuda(), dev_i32(tok))
    torch.cuda.synchronize()
    rp, rz, mag = oracle.lm_head_logprobs(xh, w, tok, mags=True)
    b = _bound(H, mag, rz)
    for got, ref, n in ((lp, rp, "logp"), (lz, rz, "logZ")):
        g = got.cpu().numpy().astype(np.float64)
        assert np.isfinite(g).all(), f"{what}: non-finite {n}"
        err = np.abs(g - ref)
        assert (err <= b).all(), f"{what}: {n} max err {err.max():.3e}, worst err/bound {(err / b).max():.3f}"
    say(f"    max abs err logp {np.abs(lp.cpu().numpy() - rp).max():.3e}")
    return xd, w, tok, lp


@pytest.mark.parametrize("xf32", [False, True], ids=["bf16_x", "fp32_x"])
def test_lm_head_parity_ragged(xf32):
    """37 tokens (one full 32-column tile, a ragged one), V = 5003 (ragged last
    64-row block), H = 1024; first and last token ids of the vocabulary."""
    _case(37, 1024, 5003, xf32=xf32, seed=1, what="ragged")


@pytest.mark.parametrize("T,H,V", [(1, 8, 1), (2, 16, 33), (70, 4096, 700)])
def test_lm_head_parity_edges(T, H, V):
    """One vocabulary row (logp = 0), a vocabulary of 33, the attention-output
    width H = 32 * 128 with more than one token group."""
    _case(T, H, V, seed=2 + T, what="edge")


def test_lm_head_token_alone_and_bad_id():
    """A token's result does not depend on the other tokens (bitwise); an id
    outside the vocabulary gives NaN for that token only."""
    xd, w, tok, lp = _case(37, 1024, 5003, seed=3, what="batch")
    wd = torch.from_numpy(w).cuda()
    for t in (0, 5, 31, 32, 36):
        one, _ = api.lm_head_logprobs(xd[t:t + 1].contiguous(), wd, dev_i32(tok[t:t + 1]))
        assert_bitwise(one, lp[t:t + 1], f"token {t} alone")
    bad = tok.copy()
    bad[4] = 5003
    lpb, _ = api.lm_head_logprobs(xd, wd, dev_i32(bad))
    assert torch.isnan(lpb[4]) and not torch.isnan(lpb[torch.arange(37) != 4]).any()


def test_dlogp_decode_equals_prefill():
    """The pages' strict decode/prefill dlogp: the Out of decode over a paged
    cache and the last row of causal prefill over the same tokens give
    bit-identical attention outputs, so their selected log-probs through the
    same FP32 lm_head are bitwise equal (dlogp max abs 0.0)."""
    Hq, Hkv, D, P = 32, 8, 128, 16
    lens = [200, 333, 77]
    Lmax = max(lens)
    rng = np.random.Generator(np.random.PCG64(950))
    q = gen.f64_to_bf16_bits(rng.standard_normal((len(lens), Lmax, Hq, D)))
    k = gen.f64_to_bf16_bits(rng.standard_normal((len(lens), Lmax, Hkv, D)))
    v = gen.f64_to_bf16_bits(rng.standard_normal((len(lens), Lmax, Hkv, D)))
    w = torch.from_numpy(gen.lm_head_weights(4099, Hq * D, seed=951)).cuda()
    tok = dev_i32(gen.lm_tokens(len(lens), 4099, seed=952))
    say(f"[lm_head] dlogp decode vs prefill, lens {lens}")
    # prefill: last row of each sequence
    pre = []
    for s, L in enumerate(lens):
        o, _ = api.prefill(dev_bf16(q[s:s + 1, :L]), dev_bf16(k[s:s + 1, :L]), dev_bf16(v[s:s + 1, :L]), block=128)
        pre.append(o[0, L - 1])
    x_pre = torch.stack(pre).contiguous()
    # decode over a paged pool holding the same keys
    n = [-(-L // P) for L in lens]
    num_pages = sum(n) + 5
    perm = np.random.Generator(np.random.PCG64(953)).permutation(num_pages)
    table = np.zeros((len(lens), max(n)), np.int32)
    kp = np.zeros((num_pages, Hkv, P, D), np.uint16)
    vp = np.zeros_like(kp)
    c = 0
    for s, L in enumerate(lens):
        for i in range(n[s]):
            pg = perm[c]
            c += 1
            table[s, i] = pg
            seg = slice(i * P, min(L, (i + 1) * P))
            kp[pg, :, : seg.stop - seg.start] = k[s, seg].transpose(1, 0, 2)
            vp[pg, :, : seg.stop - seg.start] = v[s, seg].transpose(1, 0, 2)
    qd = dev_bf16(np.stack([q[s, L - 1] for s, L in enumerate(lens)]))
    x_dec, _ = api.decode_paged(qd, dev_bf16(kp), dev_bf16(vp), dev_i32(table), dev_i32(np.array(lens, np.int32)),
                                block=128, max_context_len=Lmax)
    assert_bitwise(x_dec, x_pre, "decode Out vs prefill last row")
    lp_pre, _ = api.lm_head_logprobs(x_pre, w, tok)
    lp_dec, _ = api.lm_head_logprobs(x_dec.contiguous(), w, tok)
    assert_bitwise(lp_dec, lp_pre, "dlogp decode vs prefill")


@pytest.mark.slow
def test_lm_head_full_vocabulary():
    """Qwen3-8B's vocabulary (151936 rows) over H = 4096, eight tokens."""
    _case(8, 4096, gen.LM_VOCAB, seed=4, what="full vocabulary")
