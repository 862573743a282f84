"""FP64 CPU oracle for deterministic grouped-query attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and never consumes anything the GPU produced.

Two independent implementations live here:

* ``oracle.c`` (loaded through ctypes): the plain definition in C, FP64, OpenMP
  over (row, head).  Used at every size.
* ``brute.py``: a numpy FP64 brute force for tiny shapes that exponentiates raw
  scores without any max subtraction.  It exists only to pin the C oracle.
"""
from .core import (ORACLE_LIB, attention, attention_backward, block_states, build, decode_paged,
                   lm_head_logprobs, merge, oracle_threads)

__all__ = ["ORACLE_LIB", "attention", "attention_backward", "block_states", "build",
           "decode_paged", "lm_head_logprobs", "merge", "oracle_threads"]
