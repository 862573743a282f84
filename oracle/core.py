"""ctypes wrapper around the FP64 C oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: see the package docstring.

Inputs are bf16 bit patterns held in ``numpy.uint16`` arrays (token-major
``[B, S, H, D]``); outputs are ``float64``.  Definitions and page citations are
in ``oracle.c`` next to each C function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(_HERE, "oracle.c")
ORACLE_LIB = os.path.join(_HERE, "liboracle.so")

_libs = {}


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (FP64, OpenMP, no fast-math)."""
    if force or not os.path.exists(ORACLE_LIB):
        tmp = ORACLE_LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-shared", "-fPIC",
                               ORACLE_SRC, "-o", tmp, "-lm"])
        os.replace(tmp, ORACLE_LIB)
    return ORACLE_LIB


def _load(path=None):
    """Load (once) the oracle library at ``path`` (default: the built liboracle.so)."""
    path = ORACLE_LIB if path is None else path
    if path in _libs:
        return _libs[path]
    if path == ORACLE_LIB and not os.path.exists(ORACLE_LIB):
        build(force=True)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.orc_attention.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, i64, i32, i64, f64,
                                  i64, i64, P, i64, P, P]
    lib.orc_attention.restype = i32
    lib.orc_merge.argtypes = [P, P, P, i32, i64, i32, i32, P, P]
    lib.orc_merge.restype = i32
    lib.orc_decode_paged.argtypes = [P, P, P, i64, i32, P, i32, P, i32, i32, i32, i32, f64,
                                     P, i64, P, P]
    lib.orc_decode_paged.restype = i32
    lib.orc_attention_backward.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, i64, i32, i64,
                                           f64, P, i64, P, P, P, P, P, P]
    lib.orc_attention_backward.restype = i32
    lib.orc_lm_head_logprobs.argtypes = [P, P, P, P, i32, i32, i32, P, P, P]
    lib.orc_lm_head_logprobs.restype = i32
    _libs[path] = lib
    return lib


def oracle_threads() -> int:
    """Threads OpenMP will use for the oracle (OMP_NUM_THREADS, else all host cores)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.strip().isdigit() and int(env) > 0:
        return int(env)
    return os.cpu_count() or 1


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _u16(a, name):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"{name} must hold bf16 bit patterns as uint16, got {a.dtype}")
    return a


def attention(q, k, v, *, scale, causal=True, pos0=0, kv_len=None, key_lo=0, key_hi=None,
              rows=None, lib_path=None):
    """Plain FP64 attention (see ``orc_attention`` in oracle.c).

    q: uint16 [B, Sq, Hq, D]; k, v: uint16 [B, Skv, Hkv, D].
    Query t of each batch row sits at absolute position ``pos0 + t``.
    Keys used: ``key_lo <= j < min(key_hi, kv_len)`` and, if causal, ``j <= pos``.
    rows: optional flat indices ``b * Sq + t`` to evaluate.
    Returns (out [n_rows, Hq, D] float64, lse [n_rows, Hq] float64).
    """
    q, k, v = _u16(q, "q"), _u16(k, "k"), _u16(v, "v")
    B, Sq, Hq, D = q.shape
    Bk_, Skv, Hkv, Dk = k.shape
    if Bk_ != B or Dk != D or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k and v")
    kv_len = Skv if kv_len is None else int(kv_len)
    key_hi = kv_len if key_hi is None else int(key_hi)
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n_rows = B * Sq if rows_arr is None else rows_arr.size
    out = np.empty((n_rows, Hq, D), np.float64)
    lse = np.empty((n_rows, Hq), np.float64)
    rc = _load(lib_path).orc_attention(_ptr(q), _ptr(k), _ptr(v), B, Sq, Skv, Hq, Hkv, D, int(pos0),
                               int(bool(causal)), kv_len, float(scale), int(key_lo), key_hi,
                               _ptr(rows_arr), n_rows, _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"orc_attention rejected its arguments (rc={rc})")
    return out, lse


def block_states(q, k, v, *, scale, block, blocks, causal=True, pos0=0, kv_len=None, rows=None,
                 lib_path=None):
    """Per-block partial states: for each global block index i in ``blocks`` the
    attention restricted to keys ``[i*block, (i+1)*block)``.

    Returns (out [n_parts, n_rows, Hq, D], lse [n_parts, n_rows, Hq]).
    """
    outs, lses = [], []
    for i in blocks:
        o, l = attention(q, k, v, scale=scale, causal=causal, pos0=pos0, kv_len=kv_len,
                         key_lo=int(i) * block, key_hi=(int(i) + 1) * block, rows=rows,
                         lib_path=lib_path)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def merge(out_parts, lse_parts, gbi, *, lib_path=None):
    """Fixed-order log-sum-exp merge (see ``orc_merge``).

    out_parts float64 [n_parts, rows, Hq, D]; lse_parts [n_parts, rows, Hq];
    gbi: global block indices in arrival order.  Raises on a duplicate index.
    """
    out_parts = np.ascontiguousarray(out_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    gbi = np.ascontiguousarray(gbi, dtype=np.int64)
    n_parts, rows, Hq, D = out_parts.shape
    if lse_parts.shape != (n_parts, rows, Hq) or gbi.shape != (n_parts,):
        raise ValueError("partial-state shapes disagree")
    out = np.empty((rows, Hq, D), np.float64)
    lse = np.empty((rows, Hq), np.float64)
    rc = _load(lib_path).orc_merge(_ptr(out_parts), _ptr(lse_parts), _ptr(gbi), n_parts, rows, Hq, D,
                           _ptr(out), _ptr(lse))
    if rc == -2:
        raise ValueError("duplicate global_block_index")
    if rc != 0:
        raise ValueError(f"orc_merge rejected its arguments (rc={rc})")
    return out, lse


def decode_paged(q, k_pool, v_pool, page_table, ctx_lens, *, scale, seqs=None, lib_path=None):
    """Paged-KV decode (see ``orc_decode_paged``).

    q uint16 [Bd, Hq, D]; pools uint16 [num_pages, Hkv, P, D];
    page_table int32 [Bd, max_pages]; ctx_lens int32 [Bd].
    Returns (out [n_seq, Hq, D], lse [n_seq, Hq]) in float64.
    """
    q = _u16(q, "q")
    k_pool, v_pool = _u16(k_pool, "k_pool"), _u16(v_pool, "v_pool")
    page_table = np.ascontiguousarray(page_table, dtype=np.int32)
    ctx_lens = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    Bd, Hq, D = q.shape
    num_pages, Hkv, P, Dk = k_pool.shape
    if Dk != D or v_pool.shape != k_pool.shape or page_table.shape[0] != Bd:
        raise ValueError("shape mismatch")
    seqs_arr = None if seqs is None else np.ascontiguousarray(seqs, dtype=np.int64)
    n_seq = Bd if seqs_arr is None else seqs_arr.size
    out = np.empty((n_seq, Hq, D), np.float64)
    lse = np.empty((n_seq, Hq), np.float64)
    rc = _load(lib_path).orc_decode_paged(_ptr(q), _ptr(k_pool), _ptr(v_pool), num_pages, P,
                                  _ptr(page_table), page_table.shape[1], _ptr(ctx_lens), Bd, Hq,
                                  Hkv, D, float(scale), _ptr(seqs_arr), n_seq, _ptr(out),
                                  _ptr(lse))
    if rc != 0:
        raise ValueError(f"orc_decode_paged rejected its arguments (rc={rc})")
    return out, lse


def attention_backward(q, k, v, dout, *, scale, causal=True, pos0=0, kv_len=None, mags=False,
                       rows=None, lib_path=None):
    """Exact FP64 gradient of attention's Out (see ``orc_attention_backward``).

    q, dout: uint16 [B, Sq, Hq, D]; k, v: uint16 [B, Skv, Hkv, D].
    Returns (dq [B, Sq, Hq, D], dk [B, Skv, Hkv, D], dv [B, Skv, Hkv, D]) in float64,
    followed by (mag_dq, mag_dk, mag_dv) of the same shapes when ``mags`` is set.
    rows: optional ascending flat indices ``b * Sq + t``; only those rows are
    taken (their dQ is complete, dK/dV hold only their terms, other dQ rows are 0).
    """
    q, k, v, dout = _u16(q, "q"), _u16(k, "k"), _u16(v, "v"), _u16(dout, "dout")
    B, Sq, Hq, D = q.shape
    Bk_, Skv, Hkv, Dk = k.shape
    if Bk_ != B or Dk != D or v.shape != k.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v and dout")
    kv_len = Skv if kv_len is None else int(kv_len)
    dq = np.empty(q.shape, np.float64)
    dk = np.empty(k.shape, np.float64)
    dv = np.empty(k.shape, np.float64)
    m = [np.empty(q.shape, np.float64), np.empty(k.shape, np.float64),
         np.empty(k.shape, np.float64)] if mags else [None, None, None]
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n_rows = 0 if rows_arr is None else rows_arr.size
    rc = _load(lib_path).orc_attention_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, Sq, Skv, Hq, Hkv, D, int(pos0), int(bool(causal)),
        kv_len, float(scale), _ptr(rows_arr), n_rows, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(m[0]),
        _ptr(m[1]), _ptr(m[2]))
    if rc != 0:
        raise ValueError(f"orc_attention_backward rejected its arguments (rc={rc})")
    return (dq, dk, dv, *m) if mags else (dq, dk, dv)


def lm_head_logprobs(x, w, tokens, *, mags=False, lib_path=None):
    """Selected log-probabilities through an FP32 lm_head (see ``orc_lm_head_logprobs``).

    x: [T, H] as uint16 bf16 bits or float32; w: float32 [V, H]; tokens: int32 [T].
    Returns (logp [T], logZ [T]) in float64, plus mag [T] when ``mags`` is set.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        xb, xf = x, None
    elif x.dtype == np.float32:
        xb, xf = None, x
    else:
        raise TypeError("x must be bf16 bits (uint16) or float32")
    T, H = x.shape
    V, Hw = w.shape
    if Hw != H or tokens.shape != (T,):
        raise ValueError("shape mismatch between x, w and tokens")
    logp = np.empty(T, np.float64)
    logz = np.empty(T, np.float64)
    mag = np.empty(T, np.float64) if mags else None
    rc = _load(lib_path).orc_lm_head_logprobs(_ptr(xb), _ptr(xf), _ptr(w), _ptr(tokens), T, H, V, _ptr(logp),
                                              _ptr(logz), _ptr(mag))
    if rc != 0:
        raise ValueError(f"orc_lm_head_logprobs rejected its arguments (rc={rc})")
    return (logp, logz, mag) if mags else (logp, logz)
