"""Seeded synthetic inputs for the attention path.

This module only *draws* inputs: random normals, the bf16 rounding of those
samples, the NeoX rotary embedding that is applied before attention (the pages
specify that attention consumes post-RoPE Q/K), page tables, context lengths and
the block ownership of emulated context-parallel shards.  It holds none of the
attention arithmetic, so both the HIP path and the FP64 oracle may use it.

Recipe (stated once here and in the design notes):

* every tensor has its own ``numpy.random.Generator(PCG64(seed))`` with
  ``seed = 1000 * config_id + tensor_id`` (Q=1, K=2, V=3, lengths=4,
  page permutation=5, relocation permutation=6, arrival shuffle=7); paged K/V
  content is drawn per sequence with seed ``[1000 * config_id + tensor_id, seq]``
  in logical token order, so it does not depend on page placement;
* samples are ``standard_normal`` in FP64, optionally scaled, optionally rotated
  (NeoX rotate-half RoPE in FP64), then rounded to bf16: FP64 -> FP32
  round-to-nearest-even, then FP32 -> bf16 round-to-nearest-even;
* tensors are token-major: Q ``[B, S, Hq, D]``, K/V ``[B, S, Hkv, D]``;
  the paged pool is ``[num_pages, Hkv, page_size, D]``.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

TID_Q, TID_K, TID_V, TID_LENS, TID_PAGES, TID_RELOC, TID_ARRIVAL, TID_DOUT, TID_LMW, TID_TOK = (
    1, 2, 3, 4, 5, 6, 7, 8, 9, 10)


# --------------------------------------------------------------------------- bf16


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """FP64 -> FP32 (RNE) -> bf16 (RNE) bit patterns as uint16.  NaN stays NaN.

    Both roundings are done by torch's CPU conversions (IEEE round-to-nearest-
    even, vectorised and multithreaded); ``f64_to_bf16_bits_reference`` is the
    same rounding written out in numpy, and the tests check the two agree."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    return t.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f64_to_bf16_bits_reference(x: np.ndarray) -> np.ndarray:
    """Numpy statement of the same rounding: FP64 -> FP32 by the hardware cast,
    then add 0x7FFF plus the lowest kept bit and truncate (uint32 cannot wrap
    for a non-NaN input); NaN -> 0x7FC0."""
    f = np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    out = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


# --------------------------------------------------------------------------- draws


def normals(seed, shape) -> np.ndarray:
    """FP64 standard normals from a PCG64 generator seeded with ``seed``."""
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def neox_rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """NeoX (rotate-half) rotary embedding in FP64.

    x [B, S, H, D]; positions [S].  inv_freq_i = theta^(-2i/D) for i < D/2; the
    first and second halves of the head dimension form the rotated pairs.
    """
    D = x.shape[-1]
    half = D // 2
    inv_freq = theta ** (-(np.arange(half, dtype=np.float64) * 2.0) / D)
    ang = positions.astype(np.float64)[:, None] * inv_freq[None, :]  # [S, half]
    cos = np.cos(ang)[None, :, None, :]
    sin = np.sin(ang)[None, :, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def draw_bf16(seed, shape, *, scale=1.0, rope_theta=None, pos0=0) -> np.ndarray:
    x = normals(seed, shape)
    if scale != 1.0:
        x = x * scale
    if rope_theta is not None:
        x = neox_rope(x, pos0 + np.arange(shape[1]), rope_theta)
    return f64_to_bf16_bits(x)


# --------------------------------------------------------------------------- configs


@dataclass(frozen=True)
class PrefillConfig:
    """A prefill workload (full causal prefill over B sequences of S tokens)."""
    cfg_id: int
    name: str
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    block: int
    qk_scale: float = 1.0          # multiplier on the Q and K samples (peaky softmax)
    rope_theta: float | None = None  # NeoX RoPE applied to Q and K, or None
    shards: tuple = field(default_factory=tuple)  # emulated CP shards: tuples of block ids

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    @property
    def n_blocks(self) -> int:
        return -(-self.S // self.block)

    def flops(self) -> float:
        """Algorithmic flops of causal prefill: QK^T and PV over unmasked pairs."""
        return 4.0 * self.D * self.Hq * self.B * self.S * (self.S + 1) / 2.0


def contiguous_shards(n_blocks: int, cp: int):
    per = -(-n_blocks // cp)
    return tuple(tuple(range(r * per, min(n_blocks, (r + 1) * per))) for r in range(cp))


def zigzag_shards(n_blocks: int, cp: int):
    """Load-balanced causal split: cut the blocks into 2*cp equal chunks; shard r
    owns chunks r and 2*cp-1-r."""
    n_chunks = 2 * cp
    per = n_blocks // n_chunks
    if per * n_chunks != n_blocks:
        raise ValueError("zigzag split needs n_blocks divisible by 2*cp")
    out = []
    for r in range(cp):
        a = list(range(r * per, (r + 1) * per))
        c = n_chunks - 1 - r
        b = list(range(c * per, (c + 1) * per))
        out.append(tuple(a + b))
    return tuple(out)


CFG1 = PrefillConfig(1, "tiny causal prefill, TP=2 local shard", B=1, S=256, Hq=16, Hkv=4, D=128,
                     block=64, rope_theta=1.0e6, shards=((0, 1), (2, 3)))
CFG2 = PrefillConfig(2, "full causal prefill", B=4, S=4096, Hq=32, Hkv=8, D=128, block=128,
                     shards=contiguous_shards(32, 2))
CFG3 = PrefillConfig(3, "chunked-prefill replay", B=1, S=8192, Hq=32, Hkv=8, D=128, block=128)
CFG5 = PrefillConfig(5, "long-context prefill stress", B=1, S=32768, Hq=32, Hkv=8, D=128,
                     block=128, qk_scale=4.0, shards=zigzag_shards(256, 2))
CFG3_CHUNKS = (1, 512, 2048)


def prefill_inputs(cfg: PrefillConfig, *, B=None, S=None, seed_cfg=None):
    """Q, K, V bf16 bit patterns for a prefill config (optionally with a smaller
    B or S, drawn from the same seeds so shapes can be scaled down for tests)."""
    B = cfg.B if B is None else B
    S = cfg.S if S is None else S
    c = cfg.cfg_id if seed_cfg is None else seed_cfg
    q = draw_bf16(1000 * c + TID_Q, (B, S, cfg.Hq, cfg.D), scale=cfg.qk_scale,
                  rope_theta=cfg.rope_theta)
    k = draw_bf16(1000 * c + TID_K, (B, S, cfg.Hkv, cfg.D), scale=cfg.qk_scale,
                  rope_theta=cfg.rope_theta)
    v = draw_bf16(1000 * c + TID_V, (B, S, cfg.Hkv, cfg.D))
    return q, k, v


def dout_inputs(cfg: PrefillConfig, *, B=None, S=None, seed_cfg=None):
    """Upstream gradient dOut [B, S, Hq, D] (bf16 bit patterns) for the backward
    of a prefill config: standard normals, like the other activations."""
    B = cfg.B if B is None else B
    S = cfg.S if S is None else S
    c = cfg.cfg_id if seed_cfg is None else seed_cfg
    return draw_bf16(1000 * c + TID_DOUT, (B, S, cfg.Hq, cfg.D))


# Synthetic lm_head: Qwen3-8B's vocabulary over the attention output of all q
# heads (H = Hq * D = 4096), W ~ N(0, 1/H) in fp32 so logits are O(|x|).
LM_VOCAB = 151936


def lm_head_weights(V: int, H: int, seed: int = 1000 * 4 + TID_LMW) -> np.ndarray:
    """FP32 lm_head [V, H]: PCG64 standard normals drawn directly in float32,
    scaled by 1/sqrt(H) (rounded once to fp32)."""
    w = np.random.Generator(np.random.PCG64(seed)).standard_normal((V, H), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(H))
    return w


def lm_tokens(T: int, V: int, seed: int = 1000 * 4 + TID_TOK) -> np.ndarray:
    """Active token ids [T], integer-uniform on [0, V)."""
    return np.random.Generator(np.random.PCG64(seed)).integers(0, V, T).astype(np.int32)


def arrival_shuffle(cfg_id: int, n: int) -> np.ndarray:
    """Seeded arrival order (a permutation of range(n))."""
    return np.random.Generator(np.random.PCG64(1000 * cfg_id + TID_ARRIVAL)).permutation(n)


# --------------------------------------------------------------------------- paged decode


@dataclass(frozen=True)
class DecodeConfig:
    cfg_id: int
    name: str
    batch: int
    Hq: int
    Hkv: int
    D: int
    page_size: int
    num_pages: int
    len_lo: int
    len_hi: int
    block: int

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    @property
    def max_pages_per_seq(self) -> int:
        return -(-self.len_hi // self.page_size)


CFG4 = DecodeConfig(4, "paged-KV decode", batch=64, Hq=32, Hkv=8, D=128, page_size=16,
                    num_pages=65536, len_lo=512, len_hi=16384, block=128)


def decode_lengths(cfg: DecodeConfig, batch=None) -> np.ndarray:
    batch = cfg.batch if batch is None else batch
    rng = np.random.Generator(np.random.PCG64(1000 * cfg.cfg_id + TID_LENS))
    return rng.integers(cfg.len_lo, cfg.len_hi, size=batch, endpoint=True).astype(np.int32)


def decode_inputs(cfg: DecodeConfig, *, lengths=None, num_pages=None):
    """Paged decode inputs.

    Returns dict with q [Bd, Hq, D] uint16, k_pool / v_pool
    [num_pages, Hkv, P, D] uint16, page_table [Bd, max_pages] int32 (unused
    entries -1), ctx_lens [Bd] int32.  Sequence s takes the next ceil(len/P)
    entries of a seeded permutation of the page ids.
    """
    lens = decode_lengths(cfg) if lengths is None else np.asarray(lengths, np.int32)
    Bd = lens.size
    P, Hkv, D = cfg.page_size, cfg.Hkv, cfg.D
    num_pages = cfg.num_pages if num_pages is None else num_pages
    max_pages = -(-int(max(cfg.len_hi, lens.max(initial=0))) // P)
    need = -(-lens.astype(np.int64) // P)
    if need.sum() > num_pages:
        raise ValueError("pool too small for the drawn lengths")
    perm = np.random.Generator(np.random.PCG64(1000 * cfg.cfg_id + TID_PAGES)).permutation(num_pages)
    table = np.full((Bd, max_pages), -1, np.int32)
    k_pool = np.zeros((num_pages, Hkv, P, D), np.uint16)
    v_pool = np.zeros((num_pages, Hkv, P, D), np.uint16)
    # one reusable FP64 buffer (fresh per-sequence allocations dominate the cost otherwise)
    buf = np.empty((int(need.max(initial=0)) * P, Hkv, D), np.float64)
    cursor = 0
    for s in range(Bd):
        n = int(need[s])
        pages = perm[cursor:cursor + n]
        cursor += n
        table[s, :n] = pages
        L = int(lens[s])
        for seed_tid, pool in ((TID_K, k_pool), (TID_V, v_pool)):
            x = buf[: n * P]
            np.random.Generator(np.random.PCG64([1000 * cfg.cfg_id + seed_tid, s])).standard_normal(out=x[:L])
            x[L:] = 0.0
            # [n*P, Hkv, D] -> [n, P, Hkv, D] -> [n, Hkv, P, D]
            pool[pages] = f64_to_bf16_bits(x).reshape(n, P, Hkv, D).transpose(0, 2, 1, 3)
    q = draw_bf16(1000 * cfg.cfg_id + TID_Q, (Bd, cfg.Hq, D))
    return {"q": q, "k_pool": k_pool, "v_pool": v_pool, "page_table": table, "ctx_lens": lens}


def relocation(cfg: DecodeConfig, num_pages: int) -> np.ndarray:
    """Seeded page relocation: page p moves to slot perm[p]."""
    return np.random.Generator(np.random.PCG64(1000 * cfg.cfg_id + TID_RELOC)).permutation(num_pages)


def relocate(inputs: dict, perm: np.ndarray) -> dict:
    """Move every page to a new slot (pool[perm[p]] = old_pool[p]) and rewrite
    the page table accordingly.  Logical content is unchanged."""
    k_new = np.empty_like(inputs["k_pool"])
    v_new = np.empty_like(inputs["v_pool"])
    k_new[perm] = inputs["k_pool"]
    v_new[perm] = inputs["v_pool"]
    table = inputs["page_table"]
    new_table = np.where(table >= 0, perm[np.maximum(table, 0)], -1).astype(np.int32)
    out = dict(inputs)
    out.update(k_pool=k_new, v_pool=v_new, page_table=new_table)
    return out


def decode_kv_bytes(lens, Hkv, D, elem_bytes=2) -> int:
    """K and V bytes a decode pass must read: every cached key once per kv head."""
    return int(np.asarray(lens, np.int64).sum()) * Hkv * D * elem_bytes * 2
