"""Concurrent decodes over one shared index from two host threads (GPU).

The C ABI promises that an index is read only after its build and may be shared by
decode calls on different streams from different host threads, each with its own
workspace and outputs (the query-dependent phase touches nothing else; Vortex technical
summary, section 2.A, separates the pre-processed cache from the per-query indexer).
Both threads' results must equal the serial run bit for bit (the decode is deterministic).
"""
import threading

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def test_two_threads_two_streams_one_index():
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import DEV, say, to_dev_bf16, upload_index
    ctx = np.array([40000, 23000], np.int64)
    G, H, seg, K_s, ns, nl, frac = 2, 8, 4096, 256, 4, 64, 0.03
    K, V, _ = synth.kv(71, len(ctx), G, ctx, seg)
    idx = oracle.build(K, V, G, ctx, seg, K_s, 2, 5)
    ixd = upload_index(idx)
    q, _ = synth.queries(72, 6, len(ctx), H, G, ctx, K)
    qd = [to_dev_bf16(q[s]) for s in range(q.shape[0])]
    say("serial reference")
    serial = []
    for s in range(len(qd)):
        o, i, l = rsa.wave_attn_decode(ixd, qd[s], ns, nl, frac)
        serial.append((o.clone(), i.clone(), l.clone()))
    torch.cuda.synchronize()
    serial = [tuple(t.cpu().numpy() for t in r) for r in serial]

    k_max, wsb = rsa.wave_attn_decode_plan(ixd, H, ns, nl, frac)
    results = {}
    errors = []

    def worker(tid, steps):
        try:
            torch.cuda.set_device(DEV)
            st = torch.cuda.Stream(device=DEV)
            ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
            outs = []
            with torch.cuda.stream(st):
                for rep in range(20):
                    for s in steps:
                        o, i, l = rsa.wave_attn_decode(ixd, qd[s], ns, nl, frac, ws=ws)
                        outs.append((s, o, i, l))
            st.synchronize()
            results[tid] = [(s, o.cpu().numpy(), i.cpu().numpy(), l.cpu().numpy()) for s, o, i, l in outs]
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    say("two threads")
    th = [threading.Thread(target=worker, args=(0, [0, 1, 2])), threading.Thread(target=worker, args=(1, [3, 4, 5]))]
    for t in th:
        t.start()
    for t in th:
        t.join(timeout=120)
    assert not errors, errors
    assert sorted(results) == [0, 1]
    for tid in (0, 1):
        assert len(results[tid]) == 60
        for s, o, i, l in results[tid]:
            so, si, sl = serial[s]
            assert np.array_equal(o, so) and np.array_equal(i, si) and np.array_equal(l, sl), (tid, s)
    # and the serial results are the oracle's
    o_ref, lse_ref, ids_ref, _ = oracle.decode(idx, K, V, q[0], ns, nl, frac)
    assert np.array_equal(serial[0][1], ids_ref)
    assert np.abs(serial[0][0] - o_ref).max() <= 2e-3
