"""wave_attn_decode_static (no workspace, static device scratch) against wave_attn_decode (GPU).

The static entry point runs the same kernels on the library's static scratch array, so
its ids, outputs and lse must equal the workspace entry point's bit for bit. Two calls in
a row, the second on a smaller input: the scratch keeps the first call's contents, which
the second must not depend on. A call whose workspace would exceed the scratch is refused.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def _case(seed, ctx, G, H, seg, K_s):
    from gpu_util import to_dev_bf16, upload_index
    ctx = np.array(ctx, np.int64)
    K, V, _ = synth.kv(seed, len(ctx), G, ctx, seg)
    idx = oracle.build(K, V, G, ctx, seg, K_s, 2, seed)
    q, _ = synth.queries(seed + 1, 1, len(ctx), H, G, ctx, K)
    return idx, K, V, q[0], upload_index(idx), to_dev_bf16(q[0])


def test_static_scratch_equals_workspace_entry_point():
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import say
    big = _case(81, [60000, 41000], 4, 16, 4096, 256)
    small = _case(83, [9000], 2, 8, 2048, 128)
    for name, (idx, K, V, q, ixd, qd), (ns, nl, frac) in [("big", big, (4, 64, 0.05)),
                                                         ("small", small, (2, 16, 0.1))]:
        say("static scratch decode: %s" % name)
        k_max, wsb = rsa.wave_attn_decode_plan(ixd, qd.shape[1], ns, nl, frac)
        assert wsb <= rsa.STATIC_SCRATCH_BYTES
        o1, i1, l1 = rsa.wave_attn_decode_static(ixd, qd, ns, nl, frac)
        o2, i2, l2 = rsa.wave_attn_decode(ixd, qd, ns, nl, frac)
        torch.cuda.synchronize()
        assert torch.equal(i1, i2) and torch.equal(o1, o2) and torch.equal(l1, l2), name
        o_ref, _, ids_ref, _ = oracle.decode(idx, K, V, q, ns, nl, frac)
        assert np.array_equal(i1.cpu().numpy(), ids_ref)
        assert np.abs(o1.cpu().numpy() - o_ref).max() <= 2e-3


def test_static_scratch_refuses_a_larger_workspace():
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import DEV
    # a 2M-token sequence of 8 kv heads: its decode workspace is far above the scratch
    arrs = {k: torch.empty(16, dtype=torch.uint8, device=DEV) for k in
            ("k_sorted", "v_sorted", "perm", "inv_perm", "assign", "offsets", "sizes", "centroids",
             "centroids_bf16", "vsum")}
    ix = rsa.WaveIndex(8, [1 << 21], 16384, 1024, arrs)
    _, wsb = rsa.wave_attn_decode_plan(ix, 32, 4, 512, 0.02)
    assert wsb > rsa.STATIC_SCRATCH_BYTES
    q = torch.zeros((1, 32, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(rsa.WaveError, match="static scratch"):
        rsa.wave_attn_decode_static(ix, q, 4, 512, 0.02)
