"""The C-ABI library loads, exports every function include/rla_attn.h declares,
and rejects bad arguments on the host before anything reaches the GPU (CPU
only: every call here fails validation, so no HIP work is ever enqueued)."""
import ctypes
import os
import re
import subprocess

import pytest

from deterministic_gqa_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rla_attn.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:rla_status|size_t|const char\*)\s+(rla_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("librla_attn.so not built (run __graft_entry__.build())")
    return _lib.load()


def test_header_matches_binding_list():
    assert _declared() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s(rla_\w+)$", out, re.M))
    for name in _declared():
        assert name in exported, f"{name} declared but not exported with C linkage"
        assert hasattr(lib, name)


def test_core_id(lib):
    assert lib.rla_core_id().decode() == "rla.attention.core.v1"


def _params(**kw):
    p = _lib.RlaParams(num_q_heads=32, num_kv_heads=8, head_dim=128, kv_block_size=128, softmax_scale=0.0884,
                       causal=1, merge_order=0, acc_dtype=_lib.RLA_DT_FP32, out_dtype=_lib.RLA_DT_BF16)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), 3), (dict(kv_block_size=96), 3), (dict(acc_dtype=_lib.RLA_DT_BF16), 3),
    (dict(num_kv_heads=5), 2), (dict(num_q_heads=48, num_kv_heads=3), 3), (dict(out_dtype=7), 3),
    (dict(merge_order=_lib.RLA_ORDER_ARRIVAL), 3), (dict(softmax_scale=float("nan")), 2),
    (dict(softmax_scale=-1.0), 2), (dict(causal=2), 2), (dict(num_q_heads=0), 2),
])
def test_prefill_rejects_bad_params(lib, kw, status):
    p = _params(**kw)
    st = lib.rla_attn_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, 1, 16, None, FAKE, FAKE, None)
    assert st == status, lib.rla_last_error()
    assert lib.rla_last_error().decode()


def test_prefill_rejects_null_and_shapes(lib):
    p = _params()
    assert lib.rla_attn_prefill(None, FAKE, FAKE, FAKE, 1, 16, None, FAKE, FAKE, None) == 1
    assert lib.rla_attn_prefill(ctypes.byref(p), None, FAKE, FAKE, 1, 16, None, FAKE, FAKE, None) == 1
    assert lib.rla_attn_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, 1, 16, None, None, FAKE, None) == 1
    assert lib.rla_attn_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, 0, 16, None, FAKE, FAKE, None) == 2
    assert lib.rla_attn_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, 1, 0, None, FAKE, FAKE, None) == 2


def test_chunked_rejects_overflowing_cache(lib):
    p = _params()
    st = lib.rla_attn_prefill_chunked(ctypes.byref(p), FAKE, FAKE, FAKE, 1, 64, 4000, 4032, None, None, 0, FAKE,
                                      FAKE, None)
    assert st == 2 and "s_max" in lib.rla_last_error().decode()
    st = lib.rla_attn_prefill_chunked(ctypes.byref(p), FAKE, FAKE, FAKE, 1, 0, 0, 4032, None, None, 0, FAKE, FAKE,
                                      None)
    assert st == 2


def test_chunk_of_one_needs_its_workspace(lib):
    """A single-query chunk runs as a decode step over the cache and takes its
    block items from the caller's workspace; nothing is allocated inside."""
    p = _params()
    need = lib.rla_chunked_workspace_bytes(ctypes.byref(p), 2, 1, 4095, 8192)
    assert need == lib.rla_decode_workspace_bytes(ctypes.byref(p), 2, 4096) > 0
    assert lib.rla_chunked_workspace_bytes(ctypes.byref(p), 2, 64, 4032, 8192) == 0   # prefill route
    assert lib.rla_chunked_workspace_bytes(ctypes.byref(_params(head_dim=64)), 2, 1, 4095, 8192) == 0
    call = lambda ws, nbytes: lib.rla_attn_prefill_chunked(ctypes.byref(p), FAKE, FAKE, FAKE, 2, 1, 4095, 8192, None,
                                                           ws, nbytes, FAKE, FAKE, None)
    assert call(None, need) == 1
    assert call(FAKE, need - 1) == 5 and "workspace" in lib.rla_last_error().decode()


def test_prefill_rejects_rows_beyond_32bit_offsets(lib):
    """One head's Q or K/V rows must span < 2 GiB (32-bit buffer offsets)."""
    p = _params()  # Hq=32: 2^18 query rows of one head span 2 GiB
    st = lib.rla_attn_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, 1, (1 << 18) + 1, None, FAKE, FAKE, None)
    assert st == 3 and "2 GiB" in lib.rla_last_error().decode()
    st = lib.rla_attn_prefill_chunked(ctypes.byref(p), FAKE, FAKE, FAKE, 1, 16, (1 << 20), (1 << 20) + 16, None,
                                      None, 0, FAKE, FAKE, None)  # Hkv=8: 2^20 keys span 2 GiB
    assert st == 3 and "2 GiB" in lib.rla_last_error().decode()


def test_paged_prefill_rejects_bad_args(lib):
    p = _params()
    # (num_pages, page_size, max_pages, batch, chunk, cache) -> status
    call = lambda np_, ps, mp, b, c, cl, q=FAKE: lib.rla_attn_prefill_paged(
        ctypes.byref(p), q, FAKE, FAKE, np_, ps, FAKE, mp, b, c, cl, FAKE, FAKE, None)
    assert call(64, 16, 8, 1, 16, 0, q=None) == 1            # NULL q
    assert call(64, 2, 64, 1, 16, 0) == 3                    # page size below 4
    assert call(64, 24, 8, 1, 16, 0) == 3                    # not a power of two
    assert call(64, 256, 1, 1, 16, 0) == 3                   # larger than the block
    assert call(64, 16, 4, 1, 16, 60) == 2                   # table covers 64 keys, chunk ends at 76
    assert "max_pages_per_seq" in lib.rla_last_error().decode()
    assert call(64, 16, 8, 1, 0, 0) == 2                     # empty chunk
    assert call(0, 16, 8, 1, 16, 0) == 2                     # empty pool
    assert call(64, 16, 1 << 27, 1, 16, (1 << 30) - 8) == 2  # cache_len + chunk_len past 2^30
    assert "2^30" in lib.rla_last_error().decode()


def _shard(blocks, q_begin=0, q_count=16, n_parts=None, rows=16):
    arr = (ctypes.c_int64 * len(blocks))(*blocks)
    parts = _lib.RlaPartials(out=FAKE.value, lse=FAKE.value, global_block_index=arr,
                             n_parts=len(blocks) if n_parts is None else n_parts, rows=rows)
    shard = _lib.RlaShard(kv_blocks=arr, n_kv_blocks=len(blocks), q_begin=q_begin, q_count=q_count,
                          partials=ctypes.pointer(parts))
    return shard, (arr, parts)


@pytest.mark.parametrize("blocks,kw,status", [
    ([0, 1, 1], {}, 4),                       # duplicate owned block
    ([0, 2], {}, 2),                          # block 2 does not exist for 256 keys at Bk=128
    ([-1], {}, 2),
    ([0], dict(q_begin=250, q_count=16), 2),  # slab past the end
    ([0, 1], dict(n_parts=1), 2),             # partial buffer too small
    ([0], dict(rows=8), 2),                   # rows disagree with batch * q_count
])
def test_emit_rejects_bad_shards(lib, blocks, kw, status):
    p = _params()
    shard, keep = _shard(blocks, **kw)
    st = lib.rla_attn_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, 1, 256, ctypes.byref(shard), None, None, None)
    assert st == status, lib.rla_last_error()


def test_merge_rejects_duplicates_and_sizes(lib):
    p = _params()
    arr = (ctypes.c_int64 * 3)(4, 7, 4)
    parts = _lib.RlaPartials(out=FAKE.value, lse=FAKE.value, global_block_index=arr, n_parts=3, rows=10)
    assert lib.rla_merge_states(ctypes.byref(p), ctypes.byref(parts), FAKE, FAKE, None) == 4
    parts.n_parts = 0
    assert lib.rla_merge_states(ctypes.byref(p), ctypes.byref(parts), FAKE, FAKE, None) == 2
    parts.n_parts = _lib.RLA_MAX_PARTS + 1
    assert lib.rla_merge_states(ctypes.byref(p), ctypes.byref(parts), FAKE, FAKE, None) == 2
    parts.n_parts = 2
    assert lib.rla_merge_states(ctypes.byref(p), ctypes.byref(parts), None, FAKE, None) == 1


def test_decode_validation_and_workspace(lib):
    p = _params()
    need64 = lib.rla_decode_workspace_bytes(ctypes.byref(p), 64, 16384)
    items = 64 * 128 * 32
    assert need64 == -(-items * 128 * 4 // 256) * 256 + items * 4
    assert lib.rla_decode_workspace_bytes(ctypes.byref(_params(head_dim=64)), 64, 16384) == 0
    need = lib.rla_decode_workspace_bytes(ctypes.byref(p), 2, 16384)
    host = (ctypes.c_int32 * 2)(100, 20000)
    # every call below must fail validation: the pointers are fake
    args = [ctypes.byref(p), FAKE, FAKE, FAKE, 4096, 16, FAKE, 1024, FAKE, host, 2, 16384, FAKE, need - 1, FAKE,
            FAKE, None]
    assert lib.rla_attn_decode_paged(*args) == 2          # length beyond max_context_len
    host[1] = 200
    assert lib.rla_attn_decode_paged(*args) == 5          # workspace one byte short
    args[5] = 48                                          # page size not dividing the block
    assert lib.rla_attn_decode_paged(*args) == 3
    args[5] = 16
    args[14] = None
    assert lib.rla_attn_decode_paged(*args) == 1


def test_backward_rejects_bad_args(lib):
    """The backward entry validates pointers, shapes, the accumulate flag and
    the parameter contract before anything is enqueued."""
    call = lambda p, b, rows, cache, smax, acc=0, q=FAKE, dq=FAKE, gdt=_lib.RLA_DT_FP32, ws=FAKE, wsb=1 << 40: \
        lib.rla_attn_backward(ctypes.byref(p), q, FAKE, FAKE, FAKE, FAKE, FAKE, b, rows, cache, smax, acc, gdt, dq,
                              FAKE, FAKE, ws, wsb, None)
    p = _params()
    need = lib.rla_backward_workspace_bytes(ctypes.byref(p), 2, 100)
    assert need == 2 * 32 * 2 * 128 * 4                     # 8 bytes per row and head, rows padded to 64
    assert lib.rla_backward_workspace_bytes(ctypes.byref(p), 2, 0) == 0
    assert call(p, 2, 100, 0, 100, ws=None) == 1
    assert call(p, 2, 100, 0, 100, wsb=need - 1) == 5
    assert call(p, 1, 16, 0, 16, q=None) == 1
    assert call(p, 1, 16, 0, 16, dq=None) == 1
    assert call(p, 0, 16, 0, 16) == 2
    assert call(p, 1, 0, 0, 16) == 2
    assert call(p, 1, 16, 8, 16) == 2          # cache_len + q_rows > s_max
    assert call(p, 1, 16, -1, 16) == 2
    assert call(p, 1, 16, 0, 16, acc=2) == 2
    assert call(p, 1, 16, 0, 16, gdt=7) == 3
    assert call(p, 1, 16, 0, 16, acc=1, gdt=_lib.RLA_DT_BF16) == 3   # running sums must be fp32
    assert call(_params(head_dim=64), 1, 16, 0, 16) == 3
    assert call(_params(num_kv_heads=5), 1, 16, 0, 16) == 2
    # one head's query rows spanning 2 GiB (Hq=32: 2^18 rows)
    assert call(p, 1, (1 << 18) + 1, 0, (1 << 18) + 1) == 3
    assert "2 GiB" in lib.rla_last_error().decode()


def test_lm_head_rejects_bad_args(lib):
    """Pointers, dtype and shapes are checked before anything is enqueued."""
    call = lambda x, dt, T, H, V, w=FAKE, lp=FAKE, ws=FAKE, wsb=1 << 40: lib.rla_lm_head_logprobs(
        x, dt, w, FAKE, T, H, V, lp, None, ws, wsb, None)
    need = lib.rla_lm_head_workspace_bytes(64, 151936)
    assert need == (-(-151936 // 32) * 64 * 2 + 64) * 4
    assert lib.rla_lm_head_workspace_bytes(0, 10) == 0
    assert call(FAKE, 0, 64, 4096, 151936, ws=None) == 1
    assert call(FAKE, 0, 64, 4096, 151936, wsb=need - 1) == 5
    assert call(None, 0, 4, 64, 10) == 1
    assert call(FAKE, 0, 4, 64, 10, w=None) == 1
    assert call(FAKE, 0, 4, 64, 10, lp=None) == 1
    assert call(FAKE, 7, 4, 64, 10) == 3
    assert call(FAKE, 0, 0, 64, 10) == 2
    assert call(FAKE, 0, 4, 12, 10) == 2      # H not a multiple of 8
    assert call(FAKE, 0, 4, 64, 0) == 2


def test_static_decode_rejects_oversize_before_touching_the_device(lib):
    """rla_attn_decode_paged_static validates like rla_attn_decode_paged and
    rejects a call whose block items exceed its fixed scratch before anything
    reaches the device (this runs without a GPU)."""
    p = _params()
    cap = _lib.RLA_DECODE_STATIC_SCRATCH_BYTES
    assert lib.rla_decode_workspace_bytes(ctypes.byref(p), 64, 16384) <= cap      # the paged-decode workload fits
    assert lib.rla_decode_workspace_bytes(ctypes.byref(p), 70, 16384) > cap
    host = (ctypes.c_int32 * 70)(*([100] * 70))
    call = lambda b, mcl, ps=16, out=FAKE: lib.rla_attn_decode_paged_static(
        ctypes.byref(p), FAKE, FAKE, FAKE, 1 << 16, ps, FAKE, 1024, FAKE, host, b, mcl, out, FAKE, None)
    assert call(70, 16384) == 5 and "static scratch" in lib.rla_last_error().decode()
    assert call(2, 16384, out=None) == 1
    assert call(2, 16384, ps=48) == 3
    host[0] = 20000
    assert call(2, 16384) == 2
