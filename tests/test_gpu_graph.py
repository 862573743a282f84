"""The entry points under HIP graph capture (GPU).

No call allocates device memory or records a memset, so a sequence of calls
can be captured once into a graph and replayed: the launch-bound single-query
chunk replay is the case that gains.  Each replay here is separated by eager
work and a synchronization, and every replay's outputs must equal the eager
results bit for bit.
"""
import numpy as np
import pytest
import torch

from deterministic_gqa_attention_amd import api
from deterministic_gqa_attention_amd import inputs as gen
from tests.gpu_util import assert_bitwise, dev_bf16, dev_i32, say

pytestmark = pytest.mark.gpu


def test_graph_replay_of_decode_and_single_query_chunks():
    cfg = gen.DecodeConfig(49, "graph decode", batch=5, Hq=8, Hkv=2, D=128, page_size=16, num_pages=512,
                           len_lo=1, len_hi=1500, block=128)
    lens = np.array([3, 130, 700, 1100, 1499], np.int32)
    d = gen.decode_inputs(cfg, lengths=lens)
    qd, kp, vp = dev_bf16(d["q"]), dev_bf16(d["k_pool"]), dev_bf16(d["v_pool"])
    table, ctx = dev_i32(d["page_table"]), dev_i32(d["ctx_lens"])
    ws = api.alloc_workspace(api.decode_workspace_bytes(cfg.Hq, cfg.Hkv, cfg.batch, int(cfg.len_hi), block=128),
                             qd.device)
    # a contiguous cache and single-query chunks at three positions
    S = 640
    q = dev_bf16(gen.f64_to_bf16_bits(gen.normals(491, (1, S, 8, 128))))
    k = dev_bf16(gen.f64_to_bf16_bits(gen.normals(492, (1, S, 2, 128))))
    v = dev_bf16(gen.f64_to_bf16_bits(gen.normals(493, (1, S, 2, 128))))
    pos = (0, 300, S - 1)
    ws1 = api.alloc_workspace(api.decode_workspace_bytes(8, 2, 1, S, block=128), qd.device)
    chunks = [q[:, c:c + 1].contiguous() for c in pos]

    def calls():
        res = [api.decode_paged(qd, kp, vp, table, ctx, block=128, max_context_len=int(cfg.len_hi),
                                host_ctx_lens=lens, workspace=ws)]
        res += [api.prefill_chunked(qc, k, v, cache_len=c, block=128, workspace=ws1) for qc, c in zip(chunks, pos)]
        return res

    eager = calls()
    torch.cuda.synchronize()
    eager = [(o.clone(), l.clone()) for o, l in eager]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = calls()
    for rep in range(3):
        say(f"[graph] replay {rep}")
        # eager work between replays: the same calls on the default stream
        calls()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, ((eo, el), (co, cl)) in enumerate(zip(eager, captured)):
            assert_bitwise(co, eo, f"replay {rep} call {i} Out")
            assert_bitwise(cl, el, f"replay {rep} call {i} LSE")
