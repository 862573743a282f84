"""The torch binding's shape checks (pure functions of shapes, CPU only): every
mismatch between tensors that the kernels would index out of bounds is
rejected with ValueError before anything is launched."""
import pytest

from deterministic_gqa_attention_amd import _checks as ck


def test_prefill_shapes():
    assert ck.prefill((2, 64, 32, 128), (2, 64, 8, 128), (2, 64, 8, 128)) == (2, 64, 32, 8)
    for q, k, v in [((2, 64, 32, 128), (1, 64, 8, 128), (1, 64, 8, 128)),   # batch
                    ((2, 64, 32, 128), (2, 32, 8, 128), (2, 32, 8, 128)),   # sequence length
                    ((2, 64, 32, 128), (2, 64, 8, 128), (2, 64, 4, 128)),   # v heads differ from k
                    ((2, 64, 32, 128), (2, 64, 5, 128), (2, 64, 5, 128)),   # Hq not a multiple of Hkv
                    ((2, 64, 32, 64), (2, 64, 8, 64), (2, 64, 8, 64)),      # head dim
                    ((64, 32, 128), (2, 64, 8, 128), (2, 64, 8, 128))]:     # rank
        with pytest.raises(ValueError):
            ck.prefill(q, k, v)


def test_chunked_shapes():
    assert ck.chunked((1, 512, 32, 128), (1, 8192, 8, 128), (1, 8192, 8, 128), 7680) == (1, 512, 32, 8, 8192)
    with pytest.raises(ValueError):
        ck.chunked((1, 512, 32, 128), (1, 8192, 8, 128), (1, 8192, 8, 128), 7681)   # past the cache
    with pytest.raises(ValueError):
        ck.chunked((2, 512, 32, 128), (1, 8192, 8, 128), (1, 8192, 8, 128), 0)      # batch
    with pytest.raises(ValueError):
        ck.chunked((1, 512, 32, 128), (1, 8192, 8, 128), (1, 4096, 8, 128), 0)      # v cache shorter


def test_paged_and_decode_shapes():
    assert ck.paged((2, 16, 32, 128), (64, 8, 16, 128), (64, 8, 16, 128), (2, 4), 48)[:2] == (2, 16)
    with pytest.raises(ValueError):
        ck.paged((2, 16, 32, 128), (64, 8, 16, 128), (64, 8, 16, 128), (2, 4), 49)   # table too short
    with pytest.raises(ValueError):
        ck.paged((2, 16, 32, 128), (64, 8, 16, 128), (64, 8, 16, 128), (3, 4), 0)    # table rows
    assert ck.decode((64, 32, 128), (65536, 8, 16, 128), (65536, 8, 16, 128), (64, 1024), (64,), [1] * 64)[0] == 64
    bad = [((64, 32, 128), (65536, 8, 16, 128), (65536, 8, 16, 128), (63, 1024), (64,), None),   # table rows
           ((64, 32, 128), (65536, 8, 16, 128), (65536, 8, 16, 128), (64, 1024), (63,), None),   # lengths
           ((64, 32, 128), (65536, 8, 16, 128), (65536, 8, 16, 128), (64, 1024), (64,), [1] * 63),  # host lengths
           ((64, 32, 128), (65536, 8, 16, 128), (65535, 8, 16, 128), (64, 1024), (64,), None)]   # pools differ
    for args in bad:
        with pytest.raises(ValueError):
            ck.decode(*args)


def test_backward_shapes():
    q, k = (2, 100, 32, 128), (2, 256, 8, 128)
    assert ck.backward(q, k, k, q, (2, 100, 32), q, 156, q, k, k) == (2, 100, 32, 8, 256)
    with pytest.raises(ValueError):
        ck.backward(q, k, k, q, (2, 100, 32), q, 157)                      # cache overflow
    with pytest.raises(ValueError):
        ck.backward(q, k, k, q, (2, 100, 16), q, 0)                        # lse heads
    with pytest.raises(ValueError):
        ck.backward(q, k, k, (2, 99, 32, 128), (2, 100, 32), q, 0)         # out rows
    with pytest.raises(ValueError):
        ck.backward(q, k, k, q, (2, 100, 32), q, 0, dk=(2, 255, 8, 128))   # dk smaller than k


def test_partials_and_lm_head_shapes():
    ck.partials((4, 256, 16, 128), (4, 256, 16), 4, 256, 16)
    ck.partials((4, 256, 16, 128), (4, 4096), 3, 256, 16)
    with pytest.raises(ValueError):
        ck.partials((4, 256, 16, 128), (4, 256, 16), 5, 256, 16)           # fewer parts than used
    with pytest.raises(ValueError):
        ck.partials((4, 256, 16, 128), (4, 255, 16), 4, 256, 16)           # lse rows
    assert ck.lm_head(64, 4096, (151936, 4096), (64,)) == (64, 4096, 151936)
    with pytest.raises(ValueError):
        ck.lm_head(64, 4096, (151936, 4096), (63,))                        # token count
    with pytest.raises(ValueError):
        ck.lm_head(64, 4096, (151936, 2048), (64,))                        # hidden width
