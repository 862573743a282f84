"""Why the GPU backward's parity bar is 2^-7 * mag (CPU only).

The GPU gradient tests accept an element when |gpu - oracle| <= 2^-7 * mag,
where mag is the sum of the absolute values of the element's terms that the
FP64 oracle reports with the gradient.  This file shows, with the oracle's own
values, that the bar separates the arithmetic the kernels are allowed from
plausible mistakes:

* an FP64 model of the kernels' arithmetic, with every rounding they make on
  purpose (P and scale*dS rounded to bf16 as MFMA operands, Delta taken from
  the bf16 forward output), stays well inside the bar;
* the same model with one planted mistake (Delta from the neighbouring row,
  Delta dropped, the softmax scale dropped from dS, P from the neighbouring
  row's LSE, the causal mask shifted by one key, dV accumulated from dS, dP
  taken against K instead of V, P left unnormalised) exceeds it on every
  gradient the mistake touches.

The model is written here from the definition of the attention backward,
independently of the oracle (which supplies the reference values and mag).
"""
import numpy as np
import pytest

import oracle
from deterministic_gqa_attention_amd import inputs as gen

BAR = 2.0 ** -7  # the factor the GPU tests use
FLOOR = 1e-12

B, S, HQ, HKV, D = 1, 96, 4, 2, 128
SCALE = 1.0 / np.sqrt(D)


def _bf16(x):
    return gen.bf16_bits_to_f32(gen.f64_to_bf16_bits(np.asarray(x, np.float64))).astype(np.float64)


def _inputs():
    q = gen.f64_to_bf16_bits(gen.normals(901, (B, S, HQ, D)))
    k = gen.f64_to_bf16_bits(gen.normals(902, (B, S, HKV, D)))
    v = gen.f64_to_bf16_bits(gen.normals(903, (B, S, HKV, D)))
    do = gen.f64_to_bf16_bits(gen.normals(904, (B, S, HQ, D)))
    return q, k, v, do


def _model(q, k, v, do, mistake=None):
    """Gradients of causal attention (pos0 = 0) computed the way the kernels
    do, optionally with one planted mistake.  Returns (dq, dk, dv) in FP64."""
    f = lambda a: gen.bf16_bits_to_f32(a).astype(np.float64)
    Q, K, V, G = f(q), f(k), f(v), f(do)
    grp = HQ // HKV
    dq = np.zeros_like(Q)
    dk = np.zeros_like(K)
    dv = np.zeros_like(V)
    t = np.arange(S)
    shift = 1 if mistake == "causal_off_by_one" else 0
    visible = t[None, :] <= t[:, None] - shift  # key j visible to row i
    for b in range(B):
        for h in range(HQ):
            hk = h // grp
            s = SCALE * (Q[b, :, h] @ K[b, :, hk].T)
            s = np.where(visible, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)  # a row with no visible key (only under the shifted mask)
            L = m + np.log(np.maximum(np.exp(s - m).sum(axis=1, keepdims=True), np.finfo(np.float64).tiny))
            if mistake == "lse_wrong_row":
                L = np.roll(L, 1, axis=0)
            P = np.where(visible, np.exp(s - (m if mistake == "p_unnormalised" else L)), 0.0)
            out = _bf16(P @ V[b, :, hk])  # the forward's bf16 output
            Gh = G[b, :, h]
            dP = Gh @ (K[b, :, hk] if mistake == "dp_against_k" else V[b, :, hk]).T
            delta = (Gh * out).sum(axis=1, keepdims=True)
            if mistake == "delta_wrong_row":
                delta = np.roll(delta, 1, axis=0)
            if mistake == "delta_dropped":
                delta = np.zeros_like(delta)
            dS = P * (dP - delta)
            dSs = _bf16(dS if mistake == "scale_dropped" else SCALE * dS)
            Pb = _bf16(P)
            dq[b, :, h] = dSs @ K[b, :, hk]
            dk[b, :, hk] += dSs.T @ Q[b, :, h]
            dv[b, :, hk] += (dSs if mistake == "dv_uses_ds" else Pb).T @ Gh
    return dq, dk, dv


@pytest.fixture(scope="module")
def reference():
    q, k, v, do = _inputs()
    rq, rk, rv, mq, mk, mv = oracle.attention_backward(q, k, v, do, scale=SCALE, causal=True, mags=True)
    return (q, k, v, do), (rq, rk, rv), (mq, mk, mv)


def _ratios(got, ref, mag):
    return [float((np.abs(g - r) / (BAR * m + FLOOR)).max()) for g, r, m in zip(got, ref, mag)]


def test_kernel_rounding_model_is_inside_the_bar(reference):
    """The intended roundings use at most half of the bar on every gradient
    (the bound derived for them is 2^-8 + 2^-10 of mag, about 0.62 of it)."""
    x, ref, mag = reference
    worst = _ratios(_model(*x), ref, mag)
    assert max(worst) < 0.5, f"kernel rounding model uses {worst} of the bar (dQ, dK, dV)"


# mistake -> the gradients it must push past the bar
MISTAKES = {
    "delta_wrong_row": "qk",
    "delta_dropped": "qk",
    "scale_dropped": "qk",
    "lse_wrong_row": "qkv",
    "causal_off_by_one": "qkv",
    "dv_uses_ds": "v",
    "dp_against_k": "qk",
    "p_unnormalised": "qkv",
}


@pytest.mark.parametrize("mistake", sorted(MISTAKES))
def test_planted_mistake_exceeds_the_bar(reference, mistake):
    x, ref, mag = reference
    ratios = dict(zip("qkv", _ratios(_model(*x, mistake=mistake), ref, mag)))
    for g in MISTAKES[mistake]:
        assert ratios[g] > 4.0, f"{mistake}: d{g.upper()} deviates only {ratios[g]:.3f} x the bar"
