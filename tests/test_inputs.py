"""The seeded generator (CPU only): bf16 rounding, determinism, RoPE, shard
layouts and the paged layout."""
import numpy as np
import torch

from deterministic_gqa_attention_amd import inputs as gen


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.Generator(np.random.PCG64(5))
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-6, 6, 100000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 3.0e38, -3.0e38]])
    f32 = x.astype(np.float32)
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gen.f64_to_bf16_bits(x), ref)
    assert np.array_equal(gen.f64_to_bf16_bits_reference(x), ref)
    nan = np.array([np.nan, -np.nan])
    assert (gen.f64_to_bf16_bits_reference(nan) & 0x7FC0 == 0x7FC0).all()
    assert (gen.f64_to_bf16_bits(nan) & 0x7F80 == 0x7F80).all() and (gen.f64_to_bf16_bits(nan) & 0x7F).any()
    # ties round to even: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7
    assert gen.f64_to_bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    assert gen.f64_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82


def test_bf16_widening_roundtrip():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f = gen.bf16_bits_to_f32(bits)
    finite = np.isfinite(f)
    assert np.array_equal(gen.f64_to_bf16_bits(f[finite].astype(np.float64)), bits[finite])


def test_seeded_draws_are_reproducible():
    a = gen.prefill_inputs(gen.CFG1)
    b = gen.prefill_inputs(gen.CFG1)
    for x, y in zip(a, b):
        assert gen.sha256(x) == gen.sha256(y)
    q, k, v = a
    assert q.shape == (1, 256, 16, 128) and k.shape == (1, 256, 4, 128) and v.shape == k.shape
    assert gen.sha256(q) != gen.sha256(gen.prefill_inputs(gen.CFG2, B=1, S=256)[0])


def test_neox_rope_is_a_rotation():
    x = np.random.Generator(np.random.PCG64(1)).standard_normal((1, 8, 2, 16))
    y = gen.neox_rope(x, np.arange(8), 1.0e6)
    assert np.allclose(y[:, 0], x[:, 0], atol=0, rtol=0)  # position 0 is the identity
    half = 8
    nx = x[..., :half] ** 2 + x[..., half:] ** 2
    ny = y[..., :half] ** 2 + y[..., half:] ** 2
    assert np.allclose(nx, ny, rtol=1e-12)
    # frequency 0 pair (i=0, inv_freq=1) rotates by exactly the position angle
    p = 3
    c, s = np.cos(p), np.sin(p)
    assert np.isclose(y[0, p, 0, 0], x[0, p, 0, 0] * c - x[0, p, 0, half] * s)


def test_shard_layouts():
    assert gen.CFG1.shards == ((0, 1), (2, 3))
    assert gen.CFG2.shards == (tuple(range(16)), tuple(range(16, 32)))
    s0, s1 = gen.CFG5.shards
    assert s0 == tuple(range(0, 64)) + tuple(range(192, 256))
    assert s1 == tuple(range(64, 192))
    assert sorted(s0 + s1) == list(range(256))


def test_paged_layout_small():
    cfg = gen.DecodeConfig(9, "small", batch=5, Hq=4, Hkv=2, D=8, page_size=4, num_pages=64,
                           len_lo=3, len_hi=30, block=16)
    lens = gen.decode_lengths(cfg)
    d = gen.decode_inputs(cfg)
    assert np.array_equal(d["ctx_lens"], lens)
    table = d["page_table"]
    used = []
    for s in range(cfg.batch):
        n = -(-int(lens[s]) // cfg.page_size)
        assert (table[s, :n] >= 0).all() and (table[s, n:] == -1).all()
        used.extend(table[s, :n].tolist())
    assert len(used) == len(set(used)), "pages must not be shared"
    # content is independent of placement: gather logical rows back
    for s in range(cfg.batch):
        L = int(lens[s])
        ks = gen.draw_bf16([1000 * cfg.cfg_id + gen.TID_K, s], (L, cfg.Hkv, cfg.D))
        for j in range(L):
            page = table[s, j // cfg.page_size]
            assert np.array_equal(d["k_pool"][page, :, j % cfg.page_size], ks[j])
    r = gen.relocate(d, gen.relocation(cfg, cfg.num_pages))
    for s in range(cfg.batch):
        for j in range(int(lens[s])):
            a = d["v_pool"][table[s, j // 4], :, j % 4]
            b = r["v_pool"][r["page_table"][s, j // 4], :, j % 4]
            assert np.array_equal(a, b)


def test_cfg4_lengths_and_bytes():
    lens = gen.decode_lengths(gen.CFG4)
    assert lens.shape == (64,) and lens.min() >= 512 and lens.max() <= 16384
    assert -(-lens.astype(np.int64) // 16).sum() <= gen.CFG4.num_pages
    assert gen.decode_kv_bytes(lens, 8, 128) == int(lens.sum()) * 8 * 128 * 4
