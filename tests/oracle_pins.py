"""Pins for the FP64 oracle: checks against facts that do not come from the
oracle itself (a separately written numpy brute force, closed forms, exact
special cases and invariants that the mathematics fixes).

Each ``pin_*`` function raises AssertionError when the oracle library at
``lib_path`` violates it.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutations.py`` runs them on copies of the oracle with planted
mistakes and requires that every mistake is caught by at least one pin.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
from oracle import brute
from deterministic_gqa_attention_amd import inputs as gen

TOL = 1e-12


def _rand(seed, shape, scale=1.0):
    return gen.f64_to_bf16_bits(np.random.Generator(np.random.PCG64(seed)).standard_normal(shape) * scale)


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    diff = np.where(same_inf, 0.0, np.abs(a - b))
    assert not np.isnan(diff).any(), f"{what}: NaN"
    m = float(diff.max(initial=0.0))
    assert m <= tol, f"{what}: max abs diff {m:.3e} > {tol:.1e}"


def _bits_equal(a, b, what=""):
    assert np.array_equal(np.asarray(a).view(np.uint64), np.asarray(b).view(np.uint64)), \
        f"{what}: not bitwise identical"


# --------------------------------------------------------------------------- pins


def pin_brute_force(lib_path=None):
    """C oracle == numpy brute force (raw exp, no max subtraction) on tiny shapes,
    across GQA groupings, causal and non-causal, position offsets, short kv_len."""
    cases = [
        # B, Sq, Skv, Hq, Hkv, D, causal, pos0, kv_len
        (2, 13, 13, 4, 2, 8, True, 0, 13),
        (1, 9, 9, 6, 3, 4, True, 0, 9),
        (2, 5, 11, 4, 1, 8, True, 6, 11),     # chunk of 5 queries after 6 cached keys
        (1, 7, 16, 2, 2, 6, False, 0, 12),    # non-causal, kv_len < Skv
        (3, 4, 10, 8, 2, 8, True, 3, 7),      # causal with kv_len cutting keys
    ]
    for n, (B, Sq, Skv, Hq, Hkv, D, causal, pos0, kv_len) in enumerate(cases):
        q = _rand(100 + n, (B, Sq, Hq, D))
        k = _rand(200 + n, (B, Skv, Hkv, D))
        v = _rand(300 + n, (B, Skv, Hkv, D))
        scale = 1.0 / math.sqrt(D)
        o, l = oracle.attention(q, k, v, scale=scale, causal=causal, pos0=pos0, kv_len=kv_len,
                                lib_path=lib_path)
        bo, bl = brute.attention(q, k, v, scale=scale, causal=causal, pos0=pos0, kv_len=kv_len)
        _close(o.reshape(B, Sq, Hq, D), bo, what=f"brute out case {n}")
        _close(l.reshape(B, Sq, Hq), bl, what=f"brute lse case {n}")


def pin_single_key_row(lib_path=None):
    """Causal row 0 sees only key 0: LSE = scale * q0.k0 and Out = v0 exactly."""
    B, S, Hq, Hkv, D = 2, 6, 4, 2, 16
    q, k, v = _rand(11, (B, S, Hq, D)), _rand(12, (B, S, Hkv, D)), _rand(13, (B, S, Hkv, D))
    scale = 0.25
    o, l = oracle.attention(q, k, v, scale=scale, causal=True, lib_path=lib_path)
    o = o.reshape(B, S, Hq, D)
    l = l.reshape(B, S, Hq)
    Q, K, V = (brute.bf16_bits_to_f64(x) for x in (q, k, v))
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            s00 = scale * float(np.dot(Q[b, 0, h], K[b, 0, hk]))
            assert abs(l[b, 0, h] - s00) <= 1e-14 * max(1.0, abs(s00)), "row-0 LSE"
            assert np.array_equal(o[b, 0, h], V[b, 0, hk]), "row-0 Out must equal v0 exactly"


def pin_uniform_scores(lib_path=None):
    """All keys equal -> every score equal: Out = mean of the visible V rows,
    LSE = s + ln(n_visible).  Q = 0 gives s = 0 and LSE = ln(n_visible)."""
    B, S, Hq, Hkv, D = 1, 12, 4, 2, 8
    q = _rand(21, (B, S, Hq, D))
    krow = _rand(22, (1, 1, Hkv, D))
    k = np.broadcast_to(krow, (B, S, Hkv, D)).copy()
    v = _rand(23, (B, S, Hkv, D))
    scale = 0.5
    o, l = oracle.attention(q, k, v, scale=scale, causal=True, lib_path=lib_path)
    o, l = o.reshape(B, S, Hq, D), l.reshape(B, S, Hq)
    Q, K, V = (brute.bf16_bits_to_f64(x) for x in (q, k, v))
    for t in range(S):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            s = scale * float(np.dot(Q[0, t, h], K[0, 0, hk]))
            _close(l[0, t, h], s + math.log(t + 1), 1e-13, "uniform LSE")
            _close(o[0, t, h], V[0, : t + 1, hk].mean(axis=0), 1e-13, "uniform Out")
    qz = np.zeros_like(q)
    _, lz = oracle.attention(qz, _rand(24, (B, S, Hkv, D)), v, scale=scale, causal=True,
                             lib_path=lib_path)
    expect = np.log(np.arange(1, S + 1, dtype=np.float64))[:, None]
    _close(lz.reshape(S, Hq), np.broadcast_to(expect, (S, Hq)), 1e-14, "Q=0 LSE")


def pin_constant_v(lib_path=None):
    """Out is a convex combination of V rows: constant V gives that constant."""
    B, S, Hq, Hkv, D = 1, 20, 4, 1, 8
    q, k = _rand(31, (B, S, Hq, D), 3.0), _rand(32, (B, S, Hkv, D), 3.0)
    c = gen.f64_to_bf16_bits(np.full((B, S, Hkv, D), -1.71875))
    o, _ = oracle.attention(q, k, c, scale=1.0, causal=True, lib_path=lib_path)
    _close(o, np.full_like(o, -1.71875), 1e-12, "constant V")


def pin_two_key_closed_form(lib_path=None):
    """Hand-derived two-token example, every value exactly representable in bf16.

    q0=(1,0), q1=(0.5,1), k0=(2,0), k1=(1,-1), v0=(1,2), v1=(-3,0.5), scale 0.5.
    Row 0 sees key 0 only: s=1, so LSE=1 and Out=v0.
    Row 1: s0=0.5*(0.5*2)=0.5, s1=0.5*(0.5-1)=-0.25, LSE=ln(e^0.5+e^-0.25),
    weights w0=1/(1+e^-0.75), w1=1/(1+e^0.75), Out=w0*v0+w1*v1.
    """
    q = gen.f64_to_bf16_bits(np.array([1, 0, 0.5, 1], np.float64).reshape(1, 2, 1, 2))
    k = gen.f64_to_bf16_bits(np.array([2, 0, 1, -1], np.float64).reshape(1, 2, 1, 2))
    v = gen.f64_to_bf16_bits(np.array([1, 2, -3, 0.5], np.float64).reshape(1, 2, 1, 2))
    o, l = oracle.attention(q, k, v, scale=0.5, causal=True, lib_path=lib_path)
    w0 = 1.0 / (1.0 + math.exp(-0.75))
    w1 = 1.0 / (1.0 + math.exp(0.75))
    lse = [1.0, math.log(math.exp(0.5) + math.exp(-0.25))]
    out = [[1.0, 2.0], [w0 * 1.0 + w1 * -3.0, w0 * 2.0 + w1 * 0.5]]
    _close(l.reshape(2), np.array(lse), 1e-14, "two-key lse")
    _close(o.reshape(2, 2), np.array(out), 1e-14, "two-key out")


def pin_merge_identity(lib_path=None):
    """Merging the single-block states of every block equals unsplit attention;
    merging one state is the identity; empty (-inf) states change nothing."""
    B, S, Hq, Hkv, D, Bk = 2, 23, 4, 2, 8, 4
    q, k, v = _rand(41, (B, S, Hq, D)), _rand(42, (B, S, Hkv, D)), _rand(43, (B, S, Hkv, D))
    scale = 0.4
    nb = -(-S // Bk)
    po, pl = oracle.block_states(q, k, v, scale=scale, block=Bk, blocks=range(nb), causal=True,
                                 lib_path=lib_path)
    mo, ml = oracle.merge(po, pl, np.arange(nb), lib_path=lib_path)
    fo, fl = oracle.attention(q, k, v, scale=scale, causal=True, lib_path=lib_path)
    _close(mo, fo, 1e-12, "merge identity out")
    _close(ml, fl, 1e-12, "merge identity lse")
    # a block partial equals the brute force restricted to its key range
    bo, bl = brute.attention(q[:, 4:9], k[:, 4:8], v[:, 4:8], scale=scale, causal=True, pos0=0)
    _close(po[1].reshape(B, S, Hq, D)[:, 4:9], np.where(np.isinf(bl)[..., None], 0.0, bo), 1e-12,
           "block 1 state (first rows see only part of it)")
    # single state
    so, sl = oracle.merge(fo[None], fl[None], [5], lib_path=lib_path)
    _close(so, fo, 1e-15, "merge of one state")
    _close(sl, fl, 1e-15, "merge of one state lse")
    # empty states
    eo = np.zeros_like(fo)
    el = np.full_like(fl, -np.inf)
    xo, xl = oracle.merge(np.stack([eo, fo, eo]), np.stack([el, fl, el]), [0, 1, 2],
                          lib_path=lib_path)
    _close(xo, fo, 1e-15, "empty states out")
    _close(xl, fl, 1e-15, "empty states lse")
    ao, al = oracle.merge(np.stack([eo, eo]), np.stack([el, el]), [3, 4], lib_path=lib_path)
    assert np.all(ao == 0.0) and np.all(np.isneginf(al)), "all-empty merge must be (0, -inf)"


def pin_merge_permutation(lib_path=None):
    """The merge sorts by global_block_index: any arrival order gives bitwise the
    same result, and a repeated index is rejected."""
    B, S, Hq, Hkv, D, Bk = 1, 40, 4, 2, 8, 8
    q, k, v = _rand(51, (B, S, Hq, D), 2.0), _rand(52, (B, S, Hkv, D), 2.0), _rand(53, (B, S, Hkv, D))
    nb = S // Bk
    po, pl = oracle.block_states(q, k, v, scale=0.3, block=Bk, blocks=range(nb), lib_path=lib_path)
    ref_o, ref_l = oracle.merge(po, pl, np.arange(nb), lib_path=lib_path)
    for perm in (np.arange(nb)[::-1], np.array([2, 0, 4, 1, 3])):
        o, l = oracle.merge(po[perm], pl[perm], perm, lib_path=lib_path)
        _bits_equal(o, ref_o, "merge out under permutation")
        _bits_equal(l, ref_l, "merge lse under permutation")
    # a merge that trusted arrival order would pair the wrong indices with the wrong data
    try:
        oracle.merge(po[:2], pl[:2], [3, 3], lib_path=lib_path)
    except ValueError:
        pass
    else:
        raise AssertionError("duplicate global_block_index must be rejected")


def pin_causality(lib_path=None):
    """Changing K/V rows after position t leaves row t bitwise unchanged."""
    B, S, Hq, Hkv, D = 1, 16, 4, 2, 8
    q, k, v = _rand(61, (B, S, Hq, D)), _rand(62, (B, S, Hkv, D)), _rand(63, (B, S, Hkv, D))
    o1, l1 = oracle.attention(q, k, v, scale=0.3, lib_path=lib_path)
    t = 9
    k2, v2 = k.copy(), v.copy()
    k2[:, t + 1:] = _rand(64, k2[:, t + 1:].shape, 5.0)
    v2[:, t + 1:] = _rand(65, v2[:, t + 1:].shape, 5.0)
    o2, l2 = oracle.attention(q, k2, v2, scale=0.3, lib_path=lib_path)
    _bits_equal(o1[: t + 1], o2[: t + 1], "causality out")
    _bits_equal(l1[: t + 1], l2[: t + 1], "causality lse")
    assert not np.array_equal(o1[t + 1:], o2[t + 1:]), "later rows must see the change"


def pin_gqa_replication(lib_path=None):
    """GQA with contiguous groups equals MHA on K/V heads replicated per group."""
    B, S, Hq, Hkv, D = 2, 10, 8, 2, 8
    q, k, v = _rand(71, (B, S, Hq, D)), _rand(72, (B, S, Hkv, D)), _rand(73, (B, S, Hkv, D))
    g = Hq // Hkv
    o1, l1 = oracle.attention(q, k, v, scale=0.35, lib_path=lib_path)
    km, vm = np.repeat(k, g, axis=2), np.repeat(v, g, axis=2)
    o2, l2 = oracle.attention(q, km, vm, scale=0.35, lib_path=lib_path)
    _bits_equal(o1, o2, "GQA out")
    _bits_equal(l1, l2, "GQA lse")


def pin_chunk_equals_full(lib_path=None):
    """A chunk of queries at positions [c, c+C) over the cached keys [0, c+C) is
    the same definition as rows c..c+C-1 of full prefill (bitwise)."""
    B, S, Hq, Hkv, D = 1, 24, 4, 2, 8
    q, k, v = _rand(81, (B, S, Hq, D)), _rand(82, (B, S, Hkv, D)), _rand(83, (B, S, Hkv, D))
    fo, fl = oracle.attention(q, k, v, scale=0.3, lib_path=lib_path)
    for c, C in ((0, 5), (5, 1), (6, 11), (17, 7)):
        co, cl = oracle.attention(q[:, c:c + C], k, v, scale=0.3, pos0=c, kv_len=c + C,
                                  lib_path=lib_path)
        _bits_equal(co, fo[c:c + C], f"chunk {c}+{C} out")
        _bits_equal(cl, fl[c:c + C], f"chunk {c}+{C} lse")


def _paged_from_contiguous(k, v, P, rng_seed, num_pages):
    """Scatter contiguous K/V [Bd, L, Hkv, D] into a pool with random page placement."""
    Bd, L, Hkv, D = k.shape
    n = -(-L // P)
    perm = np.random.Generator(np.random.PCG64(rng_seed)).permutation(num_pages)
    table = perm[: Bd * n].reshape(Bd, n).astype(np.int32)
    kp = np.zeros((num_pages, Hkv, P, D), np.uint16)
    vp = np.zeros_like(kp)
    for s in range(Bd):
        for i in range(n):
            seg = slice(i * P, min(L, (i + 1) * P))
            w = seg.stop - seg.start
            kp[table[s, i], :, :w] = k[s, seg].transpose(1, 0, 2)
            vp[table[s, i], :, :w] = v[s, seg].transpose(1, 0, 2)
    return kp, vp, table


def pin_decode_equals_prefill_last_row(lib_path=None):
    """Decode over a paged cache of length L equals the last row of causal
    prefill over the same L tokens; relocating pages changes nothing."""
    Bd, L, Hq, Hkv, D, P = 3, 37, 4, 2, 8, 4
    q = _rand(91, (Bd, L, Hq, D))
    k, v = _rand(92, (Bd, L, Hkv, D)), _rand(93, (Bd, L, Hkv, D))
    lens = np.array([37, 20, 1], np.int32)
    kp, vp, table = _paged_from_contiguous(k, v, P, 94, 64)
    qd = np.stack([q[s, lens[s] - 1] for s in range(Bd)])
    do, dl = oracle.decode_paged(qd, kp, vp, table, lens, scale=0.3, lib_path=lib_path)
    for s in range(Bd):
        Ls = int(lens[s])
        fo, fl = oracle.attention(q[s:s + 1, :Ls], k[s:s + 1, :Ls], v[s:s + 1, :Ls], scale=0.3,
                                  rows=[Ls - 1], lib_path=lib_path)
        _bits_equal(do[s], fo[0], f"decode seq {s} out")
        _bits_equal(dl[s], fl[0], f"decode seq {s} lse")
    kp2, vp2, table2 = _paged_from_contiguous(k, v, P, 95, 64)
    do2, dl2 = oracle.decode_paged(qd, kp2, vp2, table2, lens, scale=0.3, lib_path=lib_path)
    _bits_equal(do, do2, "relocated out")
    _bits_equal(dl, dl2, "relocated lse")


# ------------------------------------------------------------------ backward pins


def pin_backward_finite_differences(lib_path=None):
    """The oracle's dQ/dK/dV equal central differences of the separately written
    numpy forward (``brute.attention_f64``) of  sum(Out * dOut),  element by
    element: causal GQA, a chunk after cached keys, and non-causal with a short
    kv_len."""
    cases = [
        # B, Sq, Skv, Hq, Hkv, D, causal, pos0, kv_len
        (1, 6, 6, 4, 2, 4, True, 0, 6),
        (2, 3, 7, 2, 1, 4, True, 4, 7),
        (1, 4, 6, 2, 2, 3, False, 0, 5),
    ]
    h = 1e-6
    for n, (B, Sq, Skv, Hq, Hkv, D, causal, pos0, kv_len) in enumerate(cases):
        q, k = _rand(400 + n, (B, Sq, Hq, D)), _rand(410 + n, (B, Skv, Hkv, D))
        v, do = _rand(420 + n, (B, Skv, Hkv, D)), _rand(430 + n, (B, Sq, Hq, D))
        scale = 0.45
        grads = oracle.attention_backward(q, k, v, do, scale=scale, causal=causal, pos0=pos0,
                                          kv_len=kv_len, lib_path=lib_path)
        xs = [brute.bf16_bits_to_f64(a) for a in (q, k, v)]
        G = brute.bf16_bits_to_f64(do)

        def loss(a):
            o, _ = brute.attention_f64(*a, scale=scale, causal=causal, pos0=pos0, kv_len=kv_len)
            return float((o * G).sum())

        for w, name in enumerate("qkv"):
            num = np.zeros_like(xs[w])
            for idx in np.ndindex(xs[w].shape):
                a = list(xs)
                a[w] = xs[w].copy()
                a[w][idx] += h
                lp = loss(a)
                a[w][idx] -= 2 * h
                num[idx] = (lp - loss(a)) / (2 * h)
            _close(grads[w], num, tol=1e-7, what=f"d{name} vs finite differences, case {n}")


def pin_backward_shift_invariances(lib_path=None):
    """Softmax ignores a common shift of a row's scores, so adding one vector to
    every key changes nothing: sum_j dK_j = 0.  Every probability row sums to 1,
    so sum_j dV_j is the sum of dOut over the rows (and group heads) that see at
    least one key."""
    B, S, Hq, Hkv, D = 2, 9, 4, 2, 8
    q, k = _rand(441, (B, S, Hq, D)), _rand(442, (B, S, Hkv, D), 2.0)
    v, do = _rand(443, (B, S, Hkv, D)), _rand(444, (B, S, Hq, D))
    for causal, pos0, kv_len, Sq in ((True, 0, S, S), (True, 5, S, 4), (False, 0, 6, S)):
        qq, dd = q[:, :Sq], do[:, :Sq]
        dq, dk, dv = oracle.attention_backward(qq, k, v, dd, scale=0.4, causal=causal, pos0=pos0,
                                               kv_len=kv_len, lib_path=lib_path)
        _close(dk.sum(axis=1), 0.0, tol=1e-12, what="sum of dK")
        G = brute.bf16_bits_to_f64(dd).reshape(B, Sq, Hkv, Hq // Hkv, D).sum(axis=(1, 3))
        _close(dv.sum(axis=1), G, tol=1e-12, what="sum of dV")
        assert np.abs(dk).max() > 1e-3, "dK must not vanish"


def pin_backward_single_key(lib_path=None):
    """A row that sees exactly one key has P = 1 and dS = 0, so its dQ is exactly
    0; with a single token, dK = 0 and dV_0 is the sum of dOut over the group."""
    B, Hq, Hkv, D = 2, 6, 3, 8
    q, k = _rand(451, (B, 1, Hq, D)), _rand(452, (B, 1, Hkv, D))
    v, do = _rand(453, (B, 1, Hkv, D)), _rand(454, (B, 1, Hq, D))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale=0.3, lib_path=lib_path)
    assert np.array_equal(dq, np.zeros_like(dq)), "single-key dQ must be exactly 0"
    assert np.array_equal(dk, np.zeros_like(dk)), "single-key dK must be exactly 0"
    G = brute.bf16_bits_to_f64(do).reshape(B, 1, Hkv, Hq // Hkv, D).sum(axis=3)
    _close(dv, G, tol=1e-15, what="single-key dV")
    # rows of a longer causal sequence: row 0 sees one key
    q, k = _rand(455, (B, 5, Hq, D)), _rand(456, (B, 5, Hkv, D))
    v, do = _rand(457, (B, 5, Hkv, D)), _rand(458, (B, 5, Hq, D))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale=0.3, lib_path=lib_path)
    assert np.array_equal(dq[:, 0], np.zeros_like(dq[:, 0])), "row 0 dQ must be exactly 0"
    assert np.abs(dq[:, 1:]).max() > 1e-3, "later rows must have a gradient"


def pin_backward_gqa_and_chunks(lib_path=None):
    """GQA gradients equal MHA gradients on replicated K/V heads with dK/dV summed
    over each group; a chunk's dQ rows equal the full call's rows (bitwise: the
    same operations), and the chunks' dK/dV add up to the full dK/dV."""
    B, S, Hq, Hkv, D = 1, 12, 8, 2, 8
    g = Hq // Hkv
    q, k = _rand(461, (B, S, Hq, D)), _rand(462, (B, S, Hkv, D))
    v, do = _rand(463, (B, S, Hkv, D)), _rand(464, (B, S, Hq, D))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale=0.35, lib_path=lib_path)
    mq, mk, mv = oracle.attention_backward(q, np.repeat(k, g, axis=2), np.repeat(v, g, axis=2), do,
                                           scale=0.35, lib_path=lib_path)
    _close(dq, mq, tol=1e-13, what="GQA dQ")
    _close(dk, mk.reshape(B, S, Hkv, g, D).sum(axis=3), tol=1e-13, what="GQA dK")
    _close(dv, mv.reshape(B, S, Hkv, g, D).sum(axis=3), tol=1e-13, what="GQA dV")
    sk, sv = np.zeros_like(dk), np.zeros_like(dv)
    for c, C in ((0, 5), (5, 1), (6, 6)):
        cq, ck, cv = oracle.attention_backward(q[:, c:c + C], k, v, do[:, c:c + C], scale=0.35,
                                               pos0=c, kv_len=c + C, lib_path=lib_path)
        _bits_equal(cq, dq[:, c:c + C], f"chunk {c}+{C} dQ")
        sk += ck
        sv += cv
    _close(sk, dk, tol=1e-13, what="chunked dK sum")
    _close(sv, dv, tol=1e-13, what="chunked dV sum")


def pin_backward_row_subset(lib_path=None):
    """dQ of a listed row subset equals those rows of the full call (bitwise);
    dK/dV of a partition of the rows add up to the full dK/dV."""
    B, S, Hq, Hkv, D = 2, 7, 4, 2, 8
    q, k = _rand(481, (B, S, Hq, D)), _rand(482, (B, S, Hkv, D))
    v, do = _rand(483, (B, S, Hkv, D)), _rand(484, (B, S, Hq, D))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale=0.3, lib_path=lib_path)
    part = [0, 3, 4, 9, 13]
    rest = [r for r in range(B * S) if r not in part]
    aq, ak, av = oracle.attention_backward(q, k, v, do, scale=0.3, rows=part, lib_path=lib_path)
    bq, bk, bv = oracle.attention_backward(q, k, v, do, scale=0.3, rows=rest, lib_path=lib_path)
    flat = dq.reshape(B * S, Hq, D)
    _bits_equal(aq.reshape(B * S, Hq, D)[part], flat[part], "subset dQ rows")
    assert not aq.reshape(B * S, Hq, D)[rest].any(), "unlisted dQ rows must stay 0"
    _close(ak + bk, dk, tol=1e-13, what="partitioned dK")
    _close(av + bv, dv, tol=1e-13, what="partitioned dV")


def pin_backward_magnitudes(lib_path=None):
    """The error-bound magnitudes dominate the gradients they bound (triangle
    inequality), and vanish exactly where the gradient has no term."""
    B, S, Hq, Hkv, D = 1, 7, 4, 2, 8
    q, k = _rand(471, (B, S, Hq, D)), _rand(472, (B, S, Hkv, D))
    v, do = _rand(473, (B, S, Hkv, D)), _rand(474, (B, S, Hq, D))
    dq, dk, dv, mq, mk, mv = oracle.attention_backward(q, k, v, do, scale=0.3, kv_len=5,
                                                       causal=False, mags=True, lib_path=lib_path)
    for grad, mag, name in ((dq, mq, "dQ"), (dk, mk, "dK"), (dv, mv, "dV")):
        assert (mag >= np.abs(grad) * (1 - 1e-12)).all(), f"{name} magnitude below |gradient|"
    assert not mk[:, 5:].any() and not mv[:, 5:].any(), "keys past kv_len carry no magnitude"
    assert mq.min() > 0


# -------------------------------------------------------------- lm_head pins


def _lm_inputs(seed, T, H, V, xscale=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = gen.f64_to_bf16_bits(rng.standard_normal((T, H)) * xscale)
    w = (rng.standard_normal((V, H)) / np.sqrt(H)).astype(np.float32)
    tok = rng.integers(0, V, T).astype(np.int32)
    return x, w, tok


def pin_lm_head_brute_force(lib_path=None):
    """Selected log-probs equal a numpy brute force (float64 matmul, plain
    exp-sum without max subtraction) for bf16 and fp32 inputs."""
    for n, (T, H, V) in enumerate(((5, 16, 7), (3, 24, 40), (1, 8, 1))):
        x, w, tok = _lm_inputs(500 + n, T, H, V)
        for xin in (x, brute.bf16_bits_to_f64(x).astype(np.float32)):
            lp, lz = oracle.lm_head_logprobs(xin, w, tok, lib_path=lib_path)
            z = brute.bf16_bits_to_f64(x) @ w.astype(np.float64).T
            blz = np.log(np.exp(z).sum(axis=1))
            _close(lz, blz, tol=1e-12, what=f"lm_head logZ case {n}")
            _close(lp, z[np.arange(T), tok] - blz, tol=1e-12, what=f"lm_head logp case {n}")


def pin_lm_head_closed_forms(lib_path=None):
    """W = 0 gives logp = -ln V exactly; a common vector added to every row of W
    changes nothing; the probabilities of all tokens sum to 1; V = 2 is a
    log-sigmoid of the logit difference."""
    T, H, V = 4, 32, 9
    x, w, tok = _lm_inputs(511, T, H, V)
    lp, _ = oracle.lm_head_logprobs(x, np.zeros_like(w), tok, lib_path=lib_path)
    assert np.array_equal(lp, np.full(T, -np.log(V))), "W = 0 must give -ln V"
    # rows and shift on a 2^-8 grid, so the shifted rows are exact in fp32
    rng = np.random.Generator(np.random.PCG64(512))
    wg = (np.round(rng.standard_normal((V, H)) * 64) / 256).astype(np.float32)
    shift = (np.round(rng.standard_normal(H) * 64) / 256).astype(np.float32)
    lp1, _ = oracle.lm_head_logprobs(x, wg, tok, lib_path=lib_path)
    lp2, _ = oracle.lm_head_logprobs(x, wg + shift, tok, lib_path=lib_path)
    _close(lp1, lp2, tol=1e-12, what="row shift")
    total = np.zeros(T)
    for v in range(V):
        p, _ = oracle.lm_head_logprobs(x, w, np.full(T, v, np.int32), lib_path=lib_path)
        total += np.exp(p)
    _close(total, 1.0, tol=1e-12, what="probabilities sum to 1")
    w2 = w[:2].copy()
    lpa, _ = oracle.lm_head_logprobs(x, w2, np.zeros(T, np.int32), lib_path=lib_path)
    xd = brute.bf16_bits_to_f64(x)
    dz = xd @ (w2[1].astype(np.float64) - w2[0].astype(np.float64))
    _close(lpa, -np.log1p(np.exp(dz)), tol=1e-12, what="V=2 log-sigmoid")


def pin_lm_head_magnitude(lib_path=None):
    """The magnitude dominates every |logit| of its token."""
    T, H, V = 3, 16, 11
    x, w, tok = _lm_inputs(521, T, H, V)
    lp, lz, mag = oracle.lm_head_logprobs(x, w, tok, mags=True, lib_path=lib_path)
    z = brute.bf16_bits_to_f64(x) @ w.astype(np.float64).T
    assert (mag >= np.abs(z).max(axis=1) * (1 - 1e-12)).all()


ALL_PINS = [pin_brute_force, pin_single_key_row, pin_uniform_scores, pin_constant_v,
            pin_two_key_closed_form, pin_merge_identity, pin_merge_permutation, pin_causality,
            pin_gqa_replication, pin_chunk_equals_full, pin_decode_equals_prefill_last_row,
            pin_backward_finite_differences, pin_backward_shift_invariances,
            pin_backward_single_key, pin_backward_gqa_and_chunks, pin_backward_row_subset,
            pin_backward_magnitudes, pin_lm_head_brute_force, pin_lm_head_closed_forms,
            pin_lm_head_magnitude]
