"""Shape checks of the torch binding, as pure functions of shapes.

The C ABI takes raw device pointers, so a tensor whose shape disagrees with
what the kernels index would be read or written out of bounds.  Every wrapper
in ``api.py`` passes its tensors' shapes through the matching function here
before anything is launched; each raises ValueError naming the first mismatch.
They take plain tuples, so the CPU tests exercise them without a GPU.
"""
from __future__ import annotations

HEAD_DIM = 128


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _rank(name, shape, n):
    _need(len(shape) == n, f"{name} must have {n} dims, got {tuple(shape)}")


def _heads(Hq, Hkv):
    _need(Hq >= 1 and Hkv >= 1 and Hq % Hkv == 0, f"Hq={Hq} must be a positive multiple of Hkv={Hkv}")


def prefill(q, k, v):
    """q [B,S,Hq,128]; k, v [B,S,Hkv,128] (same B and S).  Returns (B, S, Hq, Hkv)."""
    _rank("q", q, 4); _rank("k", k, 4); _rank("v", v, 4)
    B, S, Hq, D = q
    _need(D == HEAD_DIM, f"head dim must be {HEAD_DIM}, got {D}")
    _need(tuple(k[:2]) == (B, S) and k[3] == D, f"k {tuple(k)} does not match q {tuple(q)}")
    _need(tuple(v) == tuple(k), f"v {tuple(v)} must equal k {tuple(k)}")
    _heads(Hq, k[2])
    return B, S, Hq, k[2]


def chunked(q_chunk, k_cache, v_cache, cache_len):
    """q_chunk [B,C,Hq,128]; caches [B,S_max,Hkv,128] with cache_len + C <= S_max.
    Returns (B, C, Hq, Hkv, S_max)."""
    _rank("q_chunk", q_chunk, 4); _rank("k_cache", k_cache, 4); _rank("v_cache", v_cache, 4)
    B, C, Hq, D = q_chunk
    _need(D == HEAD_DIM, f"head dim must be {HEAD_DIM}, got {D}")
    _need(k_cache[0] == B and k_cache[3] == D, f"k_cache {tuple(k_cache)} does not match q_chunk {tuple(q_chunk)}")
    _need(tuple(v_cache) == tuple(k_cache), f"v_cache {tuple(v_cache)} must equal k_cache {tuple(k_cache)}")
    S_max, Hkv = k_cache[1], k_cache[2]
    _heads(Hq, Hkv)
    _need(0 <= cache_len and cache_len + C <= S_max, f"cache_len {cache_len} + chunk {C} exceeds the cache ({S_max})")
    return B, C, Hq, Hkv, S_max


def paged(q_chunk, k_pool, v_pool, page_table, cache_len):
    """q_chunk [B,C,Hq,128]; pools [num_pages,Hkv,P,128]; page_table [B,max_pages]
    covering cache_len + C keys.  Returns (B, C, Hq, Hkv, num_pages, P, max_pages)."""
    _rank("q_chunk", q_chunk, 4); _rank("k_pool", k_pool, 4); _rank("v_pool", v_pool, 4)
    _rank("page_table", page_table, 2)
    B, C, Hq, D = q_chunk
    num_pages, Hkv, P, Dk = k_pool
    _need(D == HEAD_DIM and Dk == D, f"head dim must be {HEAD_DIM}: q {tuple(q_chunk)}, k_pool {tuple(k_pool)}")
    _need(tuple(v_pool) == tuple(k_pool), f"v_pool {tuple(v_pool)} must equal k_pool {tuple(k_pool)}")
    _heads(Hq, Hkv)
    _need(page_table[0] == B, f"page_table has {page_table[0]} rows for batch {B}")
    _need(cache_len >= 0 and page_table[1] * P >= cache_len + C,
          f"page_table rows of {page_table[1]} pages of {P} do not cover cache_len + chunk = {cache_len + C}")
    return B, C, Hq, Hkv, num_pages, P, page_table[1]


def decode(q, k_pool, v_pool, page_table, ctx_lens, host_ctx_lens=None):
    """q [Bd,Hq,128]; pools [num_pages,Hkv,P,128]; page_table [Bd,max_pages];
    ctx_lens [Bd]; host lengths (if given) of length Bd.
    Returns (Bd, Hq, Hkv, num_pages, P, max_pages)."""
    _rank("q", q, 3); _rank("k_pool", k_pool, 4); _rank("v_pool", v_pool, 4); _rank("page_table", page_table, 2)
    _rank("ctx_lens", ctx_lens, 1)
    Bd, Hq, D = q
    num_pages, Hkv, P, Dk = k_pool
    _need(D == HEAD_DIM and Dk == D, f"head dim must be {HEAD_DIM}: q {tuple(q)}, k_pool {tuple(k_pool)}")
    _need(tuple(v_pool) == tuple(k_pool), f"v_pool {tuple(v_pool)} must equal k_pool {tuple(k_pool)}")
    _heads(Hq, Hkv)
    _need(page_table[0] == Bd, f"page_table has {page_table[0]} rows for {Bd} sequences")
    _need(ctx_lens[0] == Bd, f"ctx_lens has {ctx_lens[0]} entries for {Bd} sequences")
    if host_ctx_lens is not None:
        _need(len(host_ctx_lens) == Bd, f"host_ctx_lens has {len(host_ctx_lens)} entries for {Bd} sequences")
    return Bd, Hq, Hkv, num_pages, P, page_table[1]


def backward(q, k, v, out, lse, dout, cache_len, dq=None, dk=None, dv=None):
    """q, out, dout, dq [B,C,Hq,128]; lse [B,C,Hq]; k, v, dk, dv [B,S_max,Hkv,128]
    with cache_len + C <= S_max.  Returns (B, C, Hq, Hkv, S_max)."""
    B, C, Hq, Hkv, S_max = chunked(q, k, v, cache_len)
    _need(tuple(out) == tuple(q), f"out {tuple(out)} must equal q {tuple(q)}")
    _need(tuple(dout) == tuple(q), f"dout {tuple(dout)} must equal q {tuple(q)}")
    _need(tuple(lse) == (B, C, Hq), f"lse {tuple(lse)} must be {(B, C, Hq)}")
    if dq is not None:
        _need(tuple(dq) == tuple(q), f"dq {tuple(dq)} must equal q {tuple(q)}")
    for name, g in (("dk", dk), ("dv", dv)):
        if g is not None:
            _need(tuple(g) == tuple(k), f"{name} {tuple(g)} must equal k {tuple(k)}")
    return B, C, Hq, Hkv, S_max


def partials(part_out, part_lse, n_parts, rows, Hq):
    """part_out [>=n_parts, rows, Hq, 128] fp32; part_lse [>=n_parts, rows, Hq] (the
    first n_parts parts are used)."""
    _rank("part_out", part_out, 4)
    _need(part_out[0] >= n_parts and tuple(part_out[1:]) == (rows, Hq, HEAD_DIM),
          f"part_out {tuple(part_out)} cannot hold {n_parts} parts of [{rows}, {Hq}, {HEAD_DIM}]")
    _need(len(part_lse) in (2, 3), f"part_lse must have 2 or 3 dims, got {tuple(part_lse)}")
    if len(part_lse) == 3:
        _need(part_lse[0] >= n_parts and tuple(part_lse[1:]) == (rows, Hq),
              f"part_lse {tuple(part_lse)} cannot hold {n_parts} parts of [{rows}, {Hq}]")
    else:
        _need(part_lse[0] >= n_parts and part_lse[1] == rows * Hq,
              f"part_lse {tuple(part_lse)} cannot hold {n_parts} parts of {rows * Hq} values")


def lm_head(x_tokens, x_width, w, tokens):
    """x flattened to [T, H]; w [V, H]; tokens [T].  Returns (T, H, V)."""
    _rank("w", w, 2); _rank("tokens", tokens, 1)
    V, H = w
    _need(x_width == H, f"x has {x_width} values per token, w has {H}")
    _need(tokens[0] == x_tokens, f"tokens has {tokens[0]} entries for {x_tokens} rows of x")
    return x_tokens, H, V
