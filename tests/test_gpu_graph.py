"""Decode and build captured in a HIP graph (torch.cuda.graph) replay to the eager result.

The library enqueues only kernel launches on the caller's stream (no memset, no allocation,
no host synchronisation), so a captured step can be replayed. Each replay is checked
against the eager result, with eager work and synchronisations between replays.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import to_dev_bf16
    ctx = [4096, 2500]
    G, H, seg, K_s = 2, 8, 1024, 64
    K, V, _ = synth.kv(61, 2, G, np.array(ctx), seg)
    q, _ = synth.queries(62, 3, 2, H, G, np.array(ctx), K)
    Kd, Vd = to_dev_bf16(K), to_dev_bf16(V)
    qd = [to_dev_bf16(q[s]) for s in range(3)]
    ix_e = rsa.wave_index_build(Kd, Vd, G, ctx, seg, K_s, 3, 5)
    o_e, ids_e, lse_e = rsa.wave_attn_decode(ix_e, qd[0], 4, 64, 0.1)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ix_e.arrays.items()}
    o_ref, ids_ref, lse_ref = o_e.clone(), ids_e.clone(), lse_e.clone()

    ix, z = rsa.WaveIndex.allocate(G, ctx, seg, K_s)
    bws = torch.empty(int(z["build_ws_bytes"]), dtype=torch.uint8, device="cuda")
    k_max, dwsb = rsa.wave_attn_decode_plan(ix, H, 4, 64, 0.1)
    dws = torch.empty(dwsb, dtype=torch.uint8, device="cuda")
    out = torch.empty((2, H, 128), dtype=torch.float32, device="cuda")
    ids = torch.empty((2, H, k_max), dtype=torch.int32, device="cuda")
    lse = torch.empty((2, H), dtype=torch.float32, device="cuda")
    qbuf = qd[0].clone()
    # warm up eagerly on the same buffers, then capture
    rsa.wave_index_build(Kd, Vd, G, ctx, seg, K_s, 3, 5, index=ix, ws=bws)
    rsa.wave_attn_decode(ix, qbuf, 4, 64, 0.1, ws=dws, out=out, sel_ids=ids, lse=lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rsa.wave_index_build(Kd, Vd, G, ctx, seg, K_s, 3, 5, index=ix, ws=bws)
        rsa.wave_attn_decode(ix, qbuf, 4, 64, 0.1, ws=dws, out=out, sel_ids=ids, lse=lse)
    for rep in range(4):
        # scribble over the outputs eagerly between replays
        out.fill_(float("nan"))
        ids.fill_(-7)
        ix.assign.fill_(-1)
        ix.vsum.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref), rep
        assert torch.equal(ids, ids_ref), rep
        assert torch.equal(lse, lse_ref), rep
        for k, v in ref.items():
            assert torch.equal(ix.arrays[k], v), (rep, k)
    # a replay after changing the query buffer follows the new query
    qbuf.copy_(qd[1])
    g.replay()
    o2, ids2, _ = rsa.wave_attn_decode(ix_e, qd[1], 4, 64, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(ids, ids2)
