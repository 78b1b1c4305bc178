"""GPU parity of the stochastic radix top-k variant (wave_attn_decode_stochastic) against
the oracle's ref_decode_stochastic (Vortex page, section 2.C: the top-k terminates early and
samples the rest from a threshold bin).

The selection is a deterministic function of the rank keys (bit-exact on both sides), the
seed and (b, h), so the bar is the decode's: ids bit-exact (ascending order, -1 padded), out
within 2e-3, lse within 1e-3. Recall of the exact ids is printed, not asserted: the variant is
inexact by design.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3
LSE_TOL = 1e-3


def _compare(idx, K, V, q, ixd, ns, nl, frac, passes, seed, tag):
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import say, to_dev_bf16
    o, ids, lse = rsa.wave_attn_decode_stochastic(ixd, to_dev_bf16(q), ns, nl, frac, passes, seed)
    torch.cuda.synchronize()
    o_ref, lse_ref, ids_ref, kc = oracle.decode_stochastic(idx, K, V, q, ns, nl, frac, passes, seed)
    ids = ids.cpu().numpy()
    assert np.array_equal(ids, ids_ref), "ids differ at %s" % (np.argwhere(ids != ids_ref)[:5],)
    err = np.abs(o.cpu().numpy() - o_ref).max()
    assert err <= OUT_TOL, err
    assert np.abs(lse.cpu().numpy() - lse_ref).max() <= LSE_TOL
    _, _, ex, kx = oracle.decode(idx, K, V, q, ns, nl, frac)
    hit = sum(len(set(ids[b, h, :kc[b, h]].tolist()) & set(ex[b, h, :kx[b, h]].tolist()))
              for b in range(ids.shape[0]) for h in range(ids.shape[1]))
    say("stochastic top-k %s passes=%d seed=%d: recall %.4f, out err %.2e"
        % (tag, passes, seed, hit / max(int(kx.sum()), 1), err))


@pytest.fixture(scope="module")
def small():
    from gpu_util import upload_index
    ctx = np.array([3000, 1700], np.int64)
    G, H = 2, 8
    K, V, _ = synth.kv(51, 2, G, ctx, 1024)
    idx = oracle.build(K, V, G, ctx, 1024, 64, 3, 1234)
    q, _ = synth.queries(52, 2, 2, H, G, ctx, K)
    return idx, K, V, q, upload_index(idx)


@pytest.mark.parametrize("passes", [1, 2, 3, 4])
@pytest.mark.parametrize("frac,ns,nl", [(0.05, 4, 64), (0.3, 0, 0), (1.0, 0, 17), (0.0, 4, 4)])
def test_small_ragged(small, passes, frac, ns, nl):
    idx, K, V, q, ixd = small
    for s in range(2):
        _compare(idx, K, V, q[s], ixd, ns, nl, frac, passes, 1000 + s, "small step %d" % s)


def _prescribed(ctx, G, seg, K_s, data_seed):
    from test_gpu_decode import _label_assign
    ctxa = np.array([ctx], np.int64)
    K, V, comp = synth.kv(data_seed, 1, G, ctxa, seg, comp=True)
    idx = oracle.index_from_assign(K, V, G, ctxa, seg, K_s, 7, _label_assign(comp, ctxa, G, seg, K_s))
    return K, V, ctxa, idx


@pytest.mark.parametrize("ctx,G,H,seg,K_s,frac,nl", [
    (131072, 8, 32, 8192, 512, 0.02, 64),       # the 128K layer: 8192 clusters, 8 keys a thread
    (1048576, 8, 32, 16384, 1024, 0.018, 512),  # the 1M layer: 65,536 clusters, 64 keys a thread
    (524288, 2, 8, 1024, 256, 0.02, 64),        # 131,072 clusters: keys re-read from memory
])
def test_full_size(ctx, G, H, seg, K_s, frac, nl):
    from gpu_util import say, upload_index
    say("generating %d tokens, %d clusters per kv head" % (ctx, ctx // seg * K_s))
    K, V, ctxa, idx = _prescribed(ctx, G, seg, K_s, 53)
    q, _ = synth.queries(54, 1, 1, H, G, ctxa, K)
    ixd = upload_index(idx)
    for passes in (1, 2):
        _compare(idx, K, V, q[0], ixd, 4, nl, frac, passes, 99, "%d tokens" % ctx)
