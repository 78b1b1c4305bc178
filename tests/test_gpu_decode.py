"""GPU parity of the decode path (k_score, k_topk, k_attend, k_merge) against the oracle.

The index comes from the oracle (built by its k-means, or over a prescribed clustering at
full size) and is uploaded unchanged, so these tests check the decode kernels alone.
Bar: selected ids bit-exact (including the -1 padding), out within 2e-3 max-abs,
lse within 1e-3 (fp32 accumulation of bf16 inputs; measured errors are ~1e-6).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3
LSE_TOL = 1e-3


def _run(ix_dev, q, ns, nl, frac):
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import to_dev_bf16
    out, ids, lse = rsa.wave_attn_decode(ix_dev, to_dev_bf16(q), ns, nl, frac)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy(), lse.cpu().numpy()


def _compare(idx, K, V, q, ix_dev, ns, nl, frac, tag=""):
    from gpu_util import say
    say("decode parity %s frac=%g sink=%d local=%d" % (tag, frac, ns, nl))
    o, ids, lse = _run(ix_dev, q, ns, nl, frac)
    o_ref, lse_ref, ids_ref, _ = oracle.decode(idx, K, V, q, ns, nl, frac)
    assert ids.shape == ids_ref.shape
    assert np.array_equal(ids, ids_ref), "ids differ at %s" % (np.argwhere(ids != ids_ref)[:5],)
    err = np.abs(o - o_ref).max()
    assert err <= OUT_TOL, err
    assert np.abs(lse - lse_ref).max() <= LSE_TOL
    return err


@pytest.fixture(scope="module")
def small():
    from gpu_util import upload_index
    ctx = np.array([3000, 1700], np.int64)
    G, H = 2, 8
    K, V, _ = synth.kv(21, 2, G, ctx, 1024)
    idx = oracle.build(K, V, G, ctx, 1024, 64, 3, 1234)
    q, _ = synth.queries(22, 3, 2, H, G, ctx, K)
    return idx, K, V, q, upload_index(idx)


@pytest.mark.parametrize("frac,ns,nl", [(0.05, 4, 64), (0.3, 16, 100), (1.0, 0, 0), (0.0, 0, 0), (0.0, 4, 64),
                                        (0.02, 0, 1), (0.5, 1000, 0), (0.1, 1500, 1500)])
def test_small_ragged(small, frac, ns, nl):
    idx, K, V, q, ixd = small
    for s in range(q.shape[0]):
        _compare(idx, K, V, q[s], ixd, ns, nl, frac, "small step %d" % s)


def test_zero_query_picks_lowest_ids(small):
    idx, K, V, q, ixd = small
    q0 = np.zeros_like(q[0])
    _compare(idx, K, V, q0, ixd, 4, 64, 0.1, "q=0")


def test_deterministic(small):
    idx, K, V, q, ixd = small
    a = _run(ixd, q[0], 4, 64, 0.05)
    b = _run(ixd, q[0], 4, 64, 0.05)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("G,H", [(1, 1), (2, 2), (1, 8), (4, 12), (2, 14)])
def test_group_sizes(G, H):
    from gpu_util import upload_index
    ctx = np.array([2100], np.int64)
    K, V, _ = synth.kv(31, 1, G, ctx, 512)
    idx = oracle.build(K, V, G, ctx, 512, 40, 2, 5)
    q, _ = synth.queries(32, 1, 1, H, G, ctx, K)
    _compare(idx, K, V, q[0], upload_index(idx), 4, 64, 0.1, "G=%d H=%d" % (G, H))


def test_singleton_clusters_equal_full_attention():
    from gpu_util import upload_index
    ctx = np.array([700, 300], np.int64)
    G, H = 2, 4
    K, V, _ = synth.kv(41, 2, G, ctx, 256)
    idx = oracle.build(K, V, G, ctx, 256, 256, 2, 9)
    q, _ = synth.queries(42, 1, 2, H, G, ctx, K)
    ixd = upload_index(idx)
    of, _ = oracle.full_attention(K, V, q[0], G, ctx)
    for frac, ns, nl in [(0.0, 0, 0), (0.05, 4, 64), (0.3, 0, 17)]:
        o, _, _ = _run(ixd, q[0], ns, nl, frac)
        assert np.abs(o - of).max() <= OUT_TOL


def test_global_sort_path():
    # k > 8192 selected clusters: the rank order is sorted in global memory
    from gpu_util import upload_index
    ctx = np.array([40000], np.int64)
    G, H = 1, 2
    K, V, comp = synth.kv(51, 1, G, ctx, 1024, comp=True)
    idx = oracle.index_from_assign(K, V, G, ctx, 1024, 256, 3, _label_assign(comp, ctx, G, 1024, 256))
    q, _ = synth.queries(52, 1, 1, H, G, ctx, K)
    _compare(idx, K, V, q[0], upload_index(idx), 4, 64, 1.0, "global sort")
    _compare(idx, K, V, q[0], upload_index(idx), 4, 64, 0.9, "global sort 0.9")


def test_cfg1_oracle_index():
    # 16K context, 8 q / 2 kv heads, segments of 8192 with 512 clusters, 10 rounds, top 5%, 4 + 64 steady
    from gpu_util import upload_index
    ctx = np.array([16384], np.int64)
    K, V, _ = synth.kv(1, 1, 2, ctx, 8192)
    idx = oracle.build(K, V, 2, ctx, 8192, 512, 10, 1234)
    q, _ = synth.queries(101, 4, 1, 8, 2, ctx, K)
    ixd = upload_index(idx)
    for s in range(4):
        _compare(idx, K, V, q[s], ixd, 4, 64, 0.05, "cfg1 step %d" % s)


def _label_assign(comp, ctx, G, seg, K_s):
    """A prescribed clustering: label = mixture component mod K(s), per segment."""
    a = np.empty_like(comp)
    row = 0
    for N in ctx:
        for g in range(G):
            t = np.arange(N)
            s = t // seg
            L = np.minimum(seg, N - s * seg)
            kc = np.where(L >= seg, K_s, (L * K_s + seg - 1) // seg)
            a[row:row + N] = s * K_s + comp[row:row + N] % kc
            row += N
    return a


@pytest.mark.parametrize("name,ctx,G,H,seg,K_s,frac,ns,nl", [
    ("128K", [131072], 8, 32, 8192, 512, 0.02, 4, 64),
    ("1M", [1048576], 8, 32, 16384, 1024, 0.018, 4, 512),
    ("ragged16", None, 8, 32, 8192, 512, 0.02, 4, 64),
])
def test_full_size_prescribed_clustering(name, ctx, G, H, seg, K_s, frac, ns, nl):
    # the benchmark shapes: an index over a prescribed clustering (built by the oracle from
    # the generator's component labels), all heads compared
    from gpu_util import say, upload_index
    if ctx is None:
        ctx = synth.ctx_lengths(4, 16, 65536, 131072)
    ctx = np.array(ctx, np.int64)
    say("generating %s" % name)
    K, V, comp = synth.kv(3, len(ctx), G, ctx, seg, comp=True)
    idx = oracle.index_from_assign(K, V, G, ctx, seg, K_s, 1234, _label_assign(comp, ctx, G, seg, K_s))
    q, _ = synth.queries(103, 2, len(ctx), H, G, ctx, K)
    ixd = upload_index(idx)
    for s in range(2):
        _compare(idx, K, V, q[s], ixd, ns, nl, frac, "%s step %d" % (name, s))


def _tie_at_kth(idx, K, V, q, b, h, ns, nl, frac, width=3):
    """Give the clusters ranked k-1-width .. k-1+width for q head h (in the oracle's order) the centroid of the
    k-th ranked one, so that equal nonzero rank keys straddle the k-th place; returns the cluster ids."""
    _, _, order, kc = oracle.decode(idx, K, V, q, ns, nl, 1.0)  # every eligible cluster in rank order
    order = order[b, h, :kc[b, h]]
    k = oracle.k_from_frac(frac, int(idx.C[b]))
    assert width < k <= len(order) - width - 1
    g = h * idx.G // q.shape[1]
    base = int(idx.G * idx.C[:b].sum() + g * idx.C[b])
    donor = int(order[k - 1])
    tied = [int(j) for j in order[k - 1 - width:k + width]]
    for j in tied:
        idx.centroids_bf16[base + j] = idx.centroids_bf16[base + donor]
    return tied


# Cluster counts per (sequence, kv head) that select each register width of the top-k (keys
# per lane of 16 waves x 64 lanes: 1 up to 1024 clusters, then 2, 4, 8, 16, 32 per doubling;
# 0 = keys beyond registers: the chunk-top threshold path). 4 tokens per cluster; top 2%:
# k = 21 .. 1311, the fast path (k <= 1024, up to 16 keys a lane), the general path at 32.
@pytest.mark.parametrize("ctx", [4096, 8192, 16384, 32768, 65536, 131072, 262144])
def test_topk_register_widths_with_ties_at_the_kth_place(ctx):
    from gpu_util import upload_index
    G, H, seg, K_s, frac, ns, nl = 2, 8, 1024, 256, 0.02, 4, 64
    ctxa = np.array([ctx], np.int64)
    K, V, comp = synth.kv(61, 1, G, ctxa, seg, comp=True)
    idx = oracle.index_from_assign(K, V, G, ctxa, seg, K_s, 7, _label_assign(comp, ctxa, G, seg, K_s))
    q, _ = synth.queries(62, 2, 1, H, G, ctxa, K)
    # ties at the k-th place of q head 1 (kv head 0) and q head 6 (kv head 1), step 0
    t0 = _tie_at_kth(idx, K, V, q[0], 0, 1, ns, nl, frac)
    t1 = _tie_at_kth(idx, K, V, q[0], 0, 6, ns, nl, frac)
    assert len(set(t0)) == len(t0) and len(set(t1)) == len(t1)
    ixd = upload_index(idx)
    for s in range(2):
        _compare(idx, K, V, q[s], ixd, ns, nl, frac, "C=%d step %d" % (ctx // 4, s))


def test_full_size_gpu_built_index_128k():
    # the 128K layer end to end: the GPU builds the index (10 rounds), the GPU decodes against
    # it, and the oracle decodes against the same index copied back to the host
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import index_to_host, say, to_dev_bf16
    ctx = np.array([131072], np.int64)
    G, H, seg, K_s = 8, 32, 8192, 512
    say("generating 128K")
    K, V, _ = synth.kv(2, 1, G, ctx, seg)
    q, _ = synth.queries(102, 3, 1, H, G, ctx, K)
    say("GPU build 128K")
    ixd = rsa.wave_index_build(to_dev_bf16(K), to_dev_bf16(V), G, ctx.tolist(), seg, K_s, 10, 1234)
    torch.cuda.synchronize()
    host = index_to_host(ixd)
    idx = oracle.Index(G, ctx, seg, K_s)
    for f in oracle.Index.FIELDS:
        getattr(idx, f)[...] = host[f]
    for s in range(3):
        _compare(idx, K, V, q[s], ixd, 4, 64, 0.02, "GPU-built 128K step %d" % s)
