"""GPU parity of the block top-k baseline (Vortex technical summary, section A: block
summaries built once, blocks scored, the top-k attended) against the oracle.

The block index (wave_index_build_blocks) must equal the oracle's layout over its block
clustering bit-exactly; the decode without the estimation zone (wave_attn_decode_topk)
must select the same ids and match the oracle's masked attention to the decode tolerances
(out 2e-3 max-abs, lse 1e-3), over the block index and over a k-means index.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3
LSE_TOL = 1e-3


def _gpu_blocks(K, V, G, ctx, seg, K_s):
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import index_to_host, to_dev_bf16
    ix = rsa.wave_index_build_blocks(to_dev_bf16(K), to_dev_bf16(V), G, [int(n) for n in ctx], seg, K_s)
    torch.cuda.synchronize()
    return ix, index_to_host(ix)


@pytest.mark.parametrize("ctx,G,seg,K_s", [([3000, 1700], 2, 1024, 64), ([2500, 999, 1], 3, 1000, 37),
                                           ([4096], 1, 2048, 1024), ([45000], 1, 20000, 64)])
def test_block_build_bit_exact(ctx, G, seg, K_s):
    from gpu_util import say
    say("block build ctx=%s G=%d seg=%d K_s=%d" % (ctx, G, seg, K_s))
    ctx = np.array(ctx, np.int64)
    K, V, _ = synth.kv(51, len(ctx), G, ctx, seg)
    _, got = _gpu_blocks(K, V, G, ctx, seg, K_s)
    ref = oracle.build_blocks(K, V, G, ctx, seg, K_s)
    for f in oracle.Index.FIELDS:
        assert np.array_equal(got[f], getattr(ref, f)), "%s differs" % f


def _compare_topk(idx, K, V, q, ixd, ns, nl, frac, tag):
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import say, to_dev_bf16
    say("top-k decode %s frac=%g sink=%d local=%d" % (tag, frac, ns, nl))
    out, ids, lse = rsa.wave_attn_decode_topk(ixd, to_dev_bf16(q), ns, nl, frac)
    torch.cuda.synchronize()
    o, ids, lse = out.cpu().numpy(), ids.cpu().numpy(), lse.cpu().numpy()
    o_ref, lse_ref, ids_ref, _ = oracle.decode_topk(idx, K, V, q, ns, nl, frac)
    assert np.array_equal(ids, ids_ref), "ids differ at %s" % (np.argwhere(ids != ids_ref)[:5],)
    assert np.abs(o - o_ref).max() <= OUT_TOL
    assert np.abs(lse - lse_ref).max() <= LSE_TOL


@pytest.mark.parametrize("frac,ns,nl", [(0.05, 4, 64), (0.3, 16, 100), (1.0, 0, 0), (0.02, 0, 1), (0.1, 1500, 1500)])
def test_topk_decode_small(frac, ns, nl):
    from gpu_util import upload_index
    ctx = np.array([3000, 1700], np.int64)
    G, H = 2, 8
    K, V, _ = synth.kv(21, 2, G, ctx, 1024)
    q, _ = synth.queries(22, 2, 2, H, G, ctx, K)
    kidx = oracle.build(K, V, G, ctx, 1024, 64, 3, 1234)
    bidx = oracle.build_blocks(K, V, G, ctx, 1024, 64)
    for name, idx in (("k-means", kidx), ("blocks", bidx)):
        ixd = upload_index(idx)
        for s in range(q.shape[0]):
            _compare_topk(idx, K, V, q[s], ixd, ns, nl, frac, "%s step %d" % (name, s))


def test_topk_decode_128k_blocks():
    # the block baseline at the 128K layer's shape: GPU block build, oracle decode on its index
    from gpu_util import say
    ctx = np.array([131072], np.int64)
    G, H, seg, K_s = 8, 32, 8192, 512
    say("generating 128K")
    K, V, _ = synth.kv(2, 1, G, ctx, seg)
    ixd, host = _gpu_blocks(K, V, G, ctx, seg, K_s)
    idx = oracle.build_blocks(K, V, G, ctx, seg, K_s)
    for f in ("assign", "sizes", "offsets"):
        assert np.array_equal(host[f], getattr(idx, f)), f
    q, _ = synth.queries(102, 2, 1, H, G, ctx, K)
    for s in range(2):
        _compare_topk(idx, K, V, q[s], ixd, 4, 64, 0.02, "128K blocks step %d" % s)
