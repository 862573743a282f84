"""Torch-facing wrappers over the C ABI (``include/rla_attn.h``).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs are allocated with torch, and the raw device pointers plus
torch's current HIP stream are handed to librla_attn.so.  Every arithmetic step
runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _checks, _lib
from ._lib import RLAError, RlaParams, RlaPartials, RlaShard

__all__ = ["RLAError", "core_id", "prefill", "prefill_chunked", "prefill_paged", "emit_partials",
           "merge_states", "decode_paged", "decode_workspace_bytes", "backward", "lm_head_logprobs", "params",
           "alloc_workspace", "decode_paged_static", "backward_workspace_bytes", "lm_head_workspace_bytes"]

_OUT_DT = {torch.bfloat16: _lib.RLA_DT_BF16, torch.float32: _lib.RLA_DT_FP32}
_ORDER = {"global_block_index": _lib.RLA_ORDER_GLOBAL_BLOCK_INDEX, "arrival": _lib.RLA_ORDER_ARRIVAL}


def core_id() -> str:
    return _lib.load().rla_core_id().decode()


def params(Hq, Hkv, *, block, out_dtype=torch.bfloat16, causal=True, scale=None, head_dim=128,
           merge_order="global_block_index", acc_dtype=torch.float32) -> RlaParams:
    p = RlaParams()
    p.num_q_heads, p.num_kv_heads, p.head_dim, p.kv_block_size = Hq, Hkv, head_dim, block
    p.softmax_scale = (1.0 / math.sqrt(head_dim)) if scale is None else float(scale)
    p.causal = int(bool(causal))
    p.merge_order = _ORDER[merge_order]
    p.acc_dtype = _lib.RLA_DT_FP32 if acc_dtype == torch.float32 else _lib.RLA_DT_BF16
    if out_dtype not in _OUT_DT:
        raise ValueError(f"out_dtype must be bfloat16 or float32, got {out_dtype}")
    p.out_dtype = _OUT_DT[out_dtype]
    return p


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _same_device(*tensors) -> None:
    devs = {t.device for t in tensors if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors live on different devices: {sorted(str(d) for d in devs)}")


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """Device scratch of at least ``nbytes`` for an entry point's workspace argument."""
    return torch.empty((max(int(nbytes), 1),), dtype=torch.uint8, device=device)


def _ws(buf, need: int, device):
    """(pointer, bytes) of a caller-given or freshly allocated workspace."""
    if need <= 0 and buf is None:
        return None, 0
    if buf is None:
        buf = alloc_workspace(need, device)
    _dev(buf, "workspace")
    return buf, buf.numel() * buf.element_size()


def _i64_array(values):
    vals = [int(x) for x in values]
    return (ctypes.c_int64 * len(vals))(*vals), len(vals)


def _shard_struct(kv_blocks, q_begin, q_count, part_out, part_lse, rows):
    arr, n = _i64_array(kv_blocks)
    parts = RlaPartials(out=part_out.data_ptr(), lse=part_lse.data_ptr(), global_block_index=arr,
                        n_parts=n, rows=rows)
    shard = RlaShard(kv_blocks=arr, n_kv_blocks=n, q_begin=q_begin, q_count=q_count,
                     partials=ctypes.pointer(parts))
    return shard, (arr, parts)  # keep the ctypes objects alive across the call


def prefill(q, k, v, *, block, out_dtype=torch.bfloat16, causal=True, scale=None):
    """Fused causal prefill.  q [B,S,Hq,128], k/v [B,S,Hkv,128] bf16 ->
    (out [B,S,Hq,128] out_dtype, lse [B,S,Hq] fp32)."""
    B, S, Hq, Hkv = _checks.prefill(q.shape, k.shape, v.shape)
    _same_device(q, k, v)
    D = q.shape[3]
    p = params(Hq, Hkv, block=block, out_dtype=out_dtype, causal=causal, scale=scale, head_dim=D)
    out = torch.empty((B, S, Hq, D), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, S, Hq), dtype=torch.float32, device=q.device)
    lib = _lib.load()
    _lib.check(lib.rla_attn_prefill(ctypes.byref(p), _dev(q, "q", torch.bfloat16, 4), _dev(k, "k", torch.bfloat16, 4),
                                    _dev(v, "v", torch.bfloat16, 4), B, S, None, out.data_ptr(), lse.data_ptr(),
                                    _stream(q.device)))
    return out, lse


def prefill_chunked(q_chunk, k_cache, v_cache, *, cache_len, block, out_dtype=torch.bfloat16, causal=True,
                    scale=None, workspace=None):
    """One chunked-prefill replay step.  q_chunk [B,C,Hq,128]; caches
    [B,S_max,Hkv,128] already holding the chunk's K/V -> (out, lse).  A chunk of
    one query uses a device workspace (allocated here unless given)."""
    B, C, Hq, Hkv, S_max = _checks.chunked(q_chunk.shape, k_cache.shape, v_cache.shape, int(cache_len))
    _same_device(q_chunk, k_cache, v_cache, workspace)
    D = q_chunk.shape[3]
    p = params(Hq, Hkv, block=block, out_dtype=out_dtype, causal=causal, scale=scale, head_dim=D)
    out = torch.empty((B, C, Hq, D), dtype=out_dtype, device=q_chunk.device)
    lse = torch.empty((B, C, Hq), dtype=torch.float32, device=q_chunk.device)
    lib = _lib.load()
    need = int(lib.rla_chunked_workspace_bytes(ctypes.byref(p), B, C, int(cache_len), S_max))
    ws, ws_bytes = _ws(workspace, need, q_chunk.device)
    _lib.check(lib.rla_attn_prefill_chunked(
        ctypes.byref(p), _dev(q_chunk, "q_chunk", torch.bfloat16, 4), _dev(k_cache, "k_cache", torch.bfloat16, 4),
        _dev(v_cache, "v_cache", torch.bfloat16, 4), B, C, int(cache_len), S_max, None,
        None if ws is None else ws.data_ptr(), ws_bytes, out.data_ptr(), lse.data_ptr(), _stream(q_chunk.device)))
    return out, lse


def prefill_paged(q_chunk, k_pool, v_pool, page_table, *, cache_len, block, out_dtype=torch.bfloat16, causal=True,
                  scale=None):
    """Chunked prefill over paged pools.  q_chunk [B,C,Hq,128]; pools
    [num_pages,Hkv,P,128] bf16 already holding the chunk's K/V; page_table
    [B,max_pages] int32 -> (out, lse)."""
    B, C, Hq, Hkv, num_pages, P, _ = _checks.paged(q_chunk.shape, k_pool.shape, v_pool.shape, page_table.shape,
                                                   int(cache_len))
    _same_device(q_chunk, k_pool, v_pool, page_table)
    D = q_chunk.shape[3]
    p = params(Hq, Hkv, block=block, out_dtype=out_dtype, causal=causal, scale=scale, head_dim=D)
    out = torch.empty((B, C, Hq, D), dtype=out_dtype, device=q_chunk.device)
    lse = torch.empty((B, C, Hq), dtype=torch.float32, device=q_chunk.device)
    lib = _lib.load()
    _lib.check(lib.rla_attn_prefill_paged(
        ctypes.byref(p), _dev(q_chunk, "q_chunk", torch.bfloat16, 4), _dev(k_pool, "k_pool", torch.bfloat16, 4),
        _dev(v_pool, "v_pool", torch.bfloat16, 4), num_pages, P, _dev(page_table, "page_table", torch.int32, 2),
        page_table.shape[1], B, C, int(cache_len), out.data_ptr(), lse.data_ptr(), _stream(q_chunk.device)))
    return out, lse


def backward(q, k, v, out, lse, dout, *, cache_len=0, causal=True, scale=None, dq=None, dk=None, dv=None,
             accumulate=False, grad_dtype=torch.float32, workspace=None):
    """dQ, dK, dV of Out for (chunked) prefill.

    q, dout [B,C,Hq,128] bf16; k, v [B,S_max,Hkv,128] bf16 (keys [0, cache_len+C)
    used); out [B,C,Hq,128] (bf16 or fp32, the forward output); lse [B,C,Hq] fp32.
    Returns (dq [B,C,Hq,128], dk, dv [B,S_max,Hkv,128]) in grad_dtype (fp32, or
    bf16 rounded once from the fp32 result); dk/dv rows past cache_len+C are left
    as given (zeros when allocated here).  With ``accumulate`` (fp32 only) the
    call adds to the given dk/dv.  The per-row scratch is ``workspace`` (allocated
    here unless given)."""
    B, C, Hq, Hkv, S_max = _checks.backward(q.shape, k.shape, v.shape, out.shape, lse.shape, dout.shape,
                                            int(cache_len), None if dq is None else dq.shape,
                                            None if dk is None else dk.shape, None if dv is None else dv.shape)
    _same_device(q, k, v, out, lse, dout, dq, dk, dv, workspace)
    D = q.shape[3]
    if out.dtype not in _OUT_DT:
        raise ValueError(f"out must be bf16 or fp32, got {out.dtype}")
    p = params(Hq, Hkv, block=128, out_dtype=out.dtype, causal=causal, scale=scale, head_dim=D)
    if grad_dtype not in _OUT_DT:
        raise ValueError(f"grad_dtype must be bfloat16 or float32, got {grad_dtype}")
    dq = torch.empty((B, C, Hq, D), dtype=grad_dtype, device=q.device) if dq is None else dq
    if dk is None:
        dk = torch.zeros((B, S_max, Hkv, D), dtype=grad_dtype, device=q.device)
    if dv is None:
        dv = torch.zeros((B, S_max, Hkv, D), dtype=grad_dtype, device=q.device)
    lib = _lib.load()
    ws, ws_bytes = _ws(workspace, int(lib.rla_backward_workspace_bytes(ctypes.byref(p), B, C)), q.device)
    _lib.check(lib.rla_attn_backward(
        ctypes.byref(p), _dev(q, "q", torch.bfloat16, 4), _dev(k, "k", torch.bfloat16, 4),
        _dev(v, "v", torch.bfloat16, 4), _dev(out, "out", out.dtype, 4), _dev(lse, "lse", torch.float32, 3),
        _dev(dout, "dout", torch.bfloat16, 4), B, C, int(cache_len), S_max, int(bool(accumulate)),
        _OUT_DT[grad_dtype], _dev(dq, "dq", grad_dtype, 4), _dev(dk, "dk", grad_dtype, 4),
        _dev(dv, "dv", grad_dtype, 4), ws.data_ptr(), ws_bytes, _stream(q.device)))
    return dq, dk, dv


def lm_head_logprobs(x, w, tokens, *, workspace=None):
    """Selected log-probabilities through an FP32 lm_head.  x [T, H] (or any
    [T, ...] contiguous tensor, flattened per token) bf16 or fp32; w [V, H]
    fp32; tokens [T] int32.  Returns (logp [T], logz [T]) fp32.  Scratch comes
    from ``workspace`` (allocated here unless given)."""
    T = x.shape[0]
    xf = x.reshape(T, -1)
    T, H, V = _checks.lm_head(T, xf.shape[1], w.shape, tokens.shape)
    _same_device(x, w, tokens, workspace)
    if x.dtype not in _OUT_DT:
        raise ValueError(f"x must be bf16 or fp32, got {x.dtype}")
    logp = torch.empty(T, dtype=torch.float32, device=x.device)
    logz = torch.empty(T, dtype=torch.float32, device=x.device)
    lib = _lib.load()
    ws, ws_bytes = _ws(workspace, int(lib.rla_lm_head_workspace_bytes(T, V)), x.device)
    _lib.check(lib.rla_lm_head_logprobs(
        _dev(xf, "x", x.dtype, 2), _OUT_DT[x.dtype], _dev(w, "w", torch.float32, 2),
        _dev(tokens, "tokens", torch.int32, 1), T, H, V, logp.data_ptr(), logz.data_ptr(), ws.data_ptr(), ws_bytes,
        _stream(x.device)))
    return logp, logz


def emit_partials(q, k, v, kv_blocks, *, block, out_dtype=torch.bfloat16, causal=True, scale=None, q_begin=0,
                  q_count=None, cache_len=None, part_out=None, part_lse=None):
    """Per-block partial states of the owned ``kv_blocks`` (emulated CP shard).

    Full prefill (cache_len None) or chunked (q is the chunk, k/v the caches).
    Returns (part_out [n,B*q_count,Hq,128] fp32, part_lse [n,B*q_count,Hq])."""
    if cache_len is None:
        B, S, Hq, Hkv = _checks.prefill(q.shape, k.shape, v.shape)
    else:
        B, S, Hq, Hkv, _ = _checks.chunked(q.shape, k.shape, v.shape, int(cache_len))
    _same_device(q, k, v, part_out, part_lse)
    D = q.shape[3]
    q_count = S - q_begin if q_count is None else q_count
    n = len(kv_blocks)
    rows = B * q_count
    if part_out is None:
        part_out = torch.empty((n, rows, Hq, D), dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty((n, rows, Hq), dtype=torch.float32, device=q.device)
    _dev(part_out, "part_out", torch.float32)
    _dev(part_lse, "part_lse", torch.float32)
    _checks.partials(part_out.shape, part_lse.shape, n, rows, Hq)
    p = params(Hq, Hkv, block=block, out_dtype=out_dtype, causal=causal, scale=scale, head_dim=D)
    shard, keep = _shard_struct(kv_blocks, q_begin, q_count, part_out, part_lse, rows)
    lib = _lib.load()
    qp, kp, vp = _dev(q, "q", torch.bfloat16, 4), _dev(k, "k", torch.bfloat16, 4), _dev(v, "v", torch.bfloat16, 4)
    if cache_len is None:
        st = lib.rla_attn_prefill(ctypes.byref(p), qp, kp, vp, B, S, ctypes.byref(shard), None, None,
                                  _stream(q.device))
    else:
        st = lib.rla_attn_prefill_chunked(ctypes.byref(p), qp, kp, vp, B, S, int(cache_len), k.shape[1],
                                          ctypes.byref(shard), None, 0, None, None, _stream(q.device))
    del keep
    _lib.check(st)
    return part_out, part_lse


def merge_states(part_out, part_lse, global_block_index, *, Hq=None, out_dtype=torch.bfloat16,
                 order="global_block_index", n_parts=None):
    """Fold partial states (part_out [n,rows,Hq,128] fp32, part_lse [n,rows,Hq])
    whose global block indices are given in arrival order -> (out [rows,Hq,128], lse [rows,Hq])."""
    n, rows, Hq_, D = part_out.shape
    Hq = Hq_ if Hq is None else Hq
    n = n if n_parts is None else n_parts
    _checks.partials(part_out.shape, part_lse.shape, n, rows, Hq)
    _same_device(part_out, part_lse)
    p = params(Hq, Hq, block=128, out_dtype=out_dtype, head_dim=D, merge_order=order)
    arr, m = _i64_array(global_block_index)
    if m != n:
        raise ValueError(f"{m} block indices for {n} parts")
    parts = RlaPartials(out=_dev(part_out, "part_out", torch.float32, 4), lse=_dev(part_lse, "part_lse", torch.float32),
                        global_block_index=arr, n_parts=n, rows=rows)
    out = torch.empty((rows, Hq, D), dtype=out_dtype, device=part_out.device)
    lse = torch.empty((rows, Hq), dtype=torch.float32, device=part_out.device)
    lib = _lib.load()
    _lib.check(lib.rla_merge_states(ctypes.byref(p), ctypes.byref(parts), out.data_ptr(), lse.data_ptr(),
                                    _stream(part_out.device)))
    return out, lse


def backward_workspace_bytes(Hq, Hkv, batch, q_rows) -> int:
    p = params(Hq, Hkv, block=128)
    return int(_lib.load().rla_backward_workspace_bytes(ctypes.byref(p), batch, q_rows))


def lm_head_workspace_bytes(T, V) -> int:
    return int(_lib.load().rla_lm_head_workspace_bytes(T, V))


def decode_workspace_bytes(Hq, Hkv, batch, max_context_len, *, block, out_dtype=torch.bfloat16) -> int:
    p = params(Hq, Hkv, block=block, out_dtype=out_dtype)
    return int(_lib.load().rla_decode_workspace_bytes(ctypes.byref(p), batch, max_context_len))


def decode_paged(q, k_pool, v_pool, page_table, ctx_lens, *, block, max_context_len, host_ctx_lens=None,
                 out_dtype=torch.bfloat16, scale=None, workspace=None):
    """Paged-KV decode.  q [Bd,Hq,128] bf16; pools [num_pages,Hkv,P,128] bf16;
    page_table [Bd,max_pages] int32; ctx_lens [Bd] int32 (device) ->
    (out [Bd,Hq,128], lse [Bd,Hq])."""
    Bd, Hq, Hkv, num_pages, P, _ = _checks.decode(q.shape, k_pool.shape, v_pool.shape, page_table.shape,
                                                  ctx_lens.shape, host_ctx_lens)
    _same_device(q, k_pool, v_pool, page_table, ctx_lens, workspace)
    D = q.shape[2]
    p = params(Hq, Hkv, block=block, out_dtype=out_dtype, scale=scale, head_dim=D)
    lib = _lib.load()
    need = int(lib.rla_decode_workspace_bytes(ctypes.byref(p), Bd, int(max_context_len)))
    if workspace is None:
        workspace = alloc_workspace(need, q.device)
    host = None
    if host_ctx_lens is not None:
        host = (ctypes.c_int32 * Bd)(*[int(x) for x in host_ctx_lens])
    out = torch.empty((Bd, Hq, D), dtype=out_dtype, device=q.device)
    lse = torch.empty((Bd, Hq), dtype=torch.float32, device=q.device)
    _lib.check(lib.rla_attn_decode_paged(
        ctypes.byref(p), _dev(q, "q", torch.bfloat16, 3), _dev(k_pool, "k_pool", torch.bfloat16, 4),
        _dev(v_pool, "v_pool", torch.bfloat16, 4), num_pages, P, _dev(page_table, "page_table", torch.int32, 2),
        page_table.shape[1], _dev(ctx_lens, "ctx_lens", torch.int32, 1), host, Bd, int(max_context_len),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), out.data_ptr(),
        lse.data_ptr(), _stream(q.device)))
    return out, lse


def decode_paged_static(q, k_pool, v_pool, page_table, ctx_lens, *, block, max_context_len, host_ctx_lens=None,
                        out_dtype=torch.bfloat16, scale=None):
    """Paged-KV decode through rla_attn_decode_paged_static: the block items go
    to the library's fixed device array instead of a workspace (no allocation
    besides the outputs here; calls overlapping on one GPU race).  Same
    arguments and bits as ``decode_paged``."""
    Bd, Hq, Hkv, num_pages, P, _ = _checks.decode(q.shape, k_pool.shape, v_pool.shape, page_table.shape,
                                                  ctx_lens.shape, host_ctx_lens)
    _same_device(q, k_pool, v_pool, page_table, ctx_lens)
    D = q.shape[2]
    p = params(Hq, Hkv, block=block, out_dtype=out_dtype, scale=scale, head_dim=D)
    lib = _lib.load()
    host = None
    if host_ctx_lens is not None:
        host = (ctypes.c_int32 * Bd)(*[int(x) for x in host_ctx_lens])
    out = torch.empty((Bd, Hq, D), dtype=out_dtype, device=q.device)
    lse = torch.empty((Bd, Hq), dtype=torch.float32, device=q.device)
    _lib.check(lib.rla_attn_decode_paged_static(
        ctypes.byref(p), _dev(q, "q", torch.bfloat16, 3), _dev(k_pool, "k_pool", torch.bfloat16, 4),
        _dev(v_pool, "v_pool", torch.bfloat16, 4), num_pages, P, _dev(page_table, "page_table", torch.int32, 2),
        page_table.shape[1], _dev(ctx_lens, "ctx_lens", torch.int32, 1), host, Bd, int(max_context_len),
        out.data_ptr(), lse.data_ptr(), _stream(q.device)))
    return out, lse
