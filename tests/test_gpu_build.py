"""GPU parity of the index build (k_init .. k_layout) against the oracle.

Bar: every integer array (assignments of every round, perm, inv_perm, offsets, sizes) and,
since the assignments then agree, every float array (fp32 centroids, ordered fp32 value sums,
bf16 centroids, sorted K/V) bit-exact. The GPU takes each nearest-centroid decision that its
fp32 MFMA scores cannot settle in the oracle's binary64 arithmetic, so assignments are exact.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def _gpu_build(K, V, G, ctx, seg, K_s, iters, seed, trace=True):
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import index_to_host, to_dev_bf16
    Kd, Vd = to_dev_bf16(K), to_dev_bf16(V)
    r = rsa.wave_index_build(Kd, Vd, G, [int(n) for n in ctx], seg, K_s, iters, seed, assign_trace=trace)
    torch.cuda.synchronize()
    if trace:
        ix, tr = r
        return index_to_host(ix), tr.cpu().numpy()
    return index_to_host(r), None


def _check_all(name, K, V, G, ctx, seg, K_s, iters, seed):
    from gpu_util import say
    say("build parity %s" % name)
    ctx = np.array(ctx, np.int64)
    got, tr = _gpu_build(K, V, G, ctx, seg, K_s, iters, seed)
    ref, tr_ref = oracle.build(K, V, G, ctx, seg, K_s, iters, seed, trace=True)
    for it in range(iters):
        d = np.nonzero(tr[it] != tr_ref[it])[0]
        assert len(d) == 0, "round %d: %d assignments differ, first rows %s" % (it, len(d), d[:5])
    for f in oracle.Index.FIELDS:
        assert np.array_equal(got[f], getattr(ref, f)), "%s differs" % f


def test_small_ragged():
    ctx = [3000, 1700]
    K, V, _ = synth.kv(21, 2, 2, np.array(ctx), 1024)
    _check_all("small ragged", K, V, 2, ctx, 1024, 64, 3, 1234)


def test_partial_segments_odd_cluster_counts():
    ctx = [2500, 999, 1]
    K, V, _ = synth.kv(22, 3, 3, np.array(ctx), 1000)
    _check_all("odd counts", K, V, 3, ctx, 1000, 37, 4, 77)


def test_more_than_512_clusters_per_segment():
    ctx = [4096]
    K, V, _ = synth.kv(23, 1, 1, np.array(ctx), 2048)
    _check_all("K_s=1024", K, V, 1, ctx, 2048, 1024, 2, 5)


def test_long_segments_general_sort():
    # segments longer than 16384 tokens take the ballot counting sort instead of the LDS radix sort
    ctx = [45000]
    K, V, _ = synth.kv(16, 1, 1, np.array(ctx), 20000)
    _check_all("seg=20000", K, V, 1, ctx, 20000, 64, 2, 13)


def test_large_cluster_list_overflow():
    # 16 segments of 65536 tokens with 512 clusters each (128 members on average): more than
    # the 256 large clusters a sorting workgroup stages (up to ~350 of 64 or more members in a
    # segment) and more than the 4096 entries of the update's list (over 5000 in all), so some
    # large clusters run in the plain order; every array of both rounds bit-exact
    ctx = [262144]
    K, V, _ = synth.kv(28, 1, 4, np.array(ctx), 65536)
    _check_all("large-cluster list overflow", K, V, 4, ctx, 65536, 512, 2, 29)


def test_duplicate_keys_and_ties():
    # many identical keys: exact distance ties go to the lowest id (binary64 decision path)
    ctx = [2048]
    K, V, _ = synth.kv(24, 1, 2, np.array(ctx), 1024)
    K = K.copy()
    K[100:600] = K[50]
    K[1500:1900] = K[1400]
    _check_all("duplicates", K, V, 2, ctx, 1024, 64, 3, 9)


@pytest.mark.parametrize("scale_log2", [60, 63])
def test_huge_keys_take_the_exact_decision(scale_log2):
    # keys scaled by 2^60 (x.c near the top of the fp32 range: the margin test sends every
    # token to the exact binary64 decision) and 2^63 (|x|^2 and |c|^2 overflow fp32: the
    # MFMA values are inf/NaN, and every centroid is a candidate of the exact decision)
    ctx = [2048]
    K, V, _ = synth.kv(26, 1, 1, np.array(ctx), 1024)
    Kf = oracle.bf16_to_f32(K).astype(np.float64) * 2.0 ** scale_log2
    Kh = oracle.f32_to_bf16(Kf.astype(np.float32))
    assert np.isfinite(oracle.bf16_to_f32(Kh)).all()
    _check_all("keys x 2^%d" % scale_log2, Kh, V, 1, ctx, 1024, 64, 2, 31)


def test_singleton_clusters():
    ctx = [700, 300]
    K, V, _ = synth.kv(25, 2, 2, np.array(ctx), 256)
    _check_all("singletons", K, V, 2, ctx, 256, 256, 2, 9)


def test_cfg1():
    ctx = [16384]
    K, V, _ = synth.kv(1, 1, 2, np.array(ctx), 8192)
    _check_all("cfg1 16K", K, V, 2, ctx, 8192, 512, 10, 1234)


def test_heavy_tailed_keys():
    ctx = [16384]
    K, V, _ = synth.kv(5, 1, 2, np.array(ctx), 8192, heavy=True)
    _check_all("student-t", K, V, 2, ctx, 8192, 512, 10, 1234)


def test_deterministic():
    ctx = np.array([5000], np.int64)
    K, V, _ = synth.kv(26, 1, 2, ctx, 2048)
    a, ta = _gpu_build(K, V, 2, ctx, 2048, 128, 3, 3)
    b, tb = _gpu_build(K, V, 2, ctx, 2048, 128, 3, 3)
    assert np.array_equal(ta, tb)
    for f in a:
        assert np.array_equal(a[f], b[f]), f


def _sampled_units(name, K, V, G, ctx, seg, K_s, iters, seed, sample):
    """Full-size GPU build; chosen units (independent k-means problems) against the oracle."""
    from gpu_util import say
    say("full-size build %s" % name)
    got, _ = _gpu_build(K, V, G, ctx, seg, K_s, iters, seed, trace=False)
    C = [oracle.num_clusters(int(n), seg, K_s) for n in ctx]
    # layout invariants on every block
    row = clu = 0
    for b, N in enumerate(ctx):
        for g in range(G):
            perm = got["perm"][row:row + N]
            assert np.array_equal(got["inv_perm"][row:row + N][perm], np.arange(N))
            a = got["assign"][row:row + N]
            assert np.all(np.diff(a[perm].astype(np.int64) * (N + 1) + perm) > 0)
            assert np.array_equal(got["sizes"][clu:clu + C[b]], np.bincount(a, minlength=C[b]))
            row += N
            clu += C[b]
    # the whole layout of the final assignment, every cluster: the oracle's layout and update
    # of the GPU's assignments (the last update pass took every cluster exactly once, in
    # whatever order it started them); an empty cluster keeps its centroid, not compared
    lay = oracle.index_from_assign(K, V, G, ctx, seg, K_s, seed, got["assign"])
    for f in ("perm", "inv_perm", "offsets", "sizes", "k_sorted", "v_sorted"):
        assert np.array_equal(got[f], getattr(lay, f)), "%s differs from the oracle's layout" % f
    nz = lay.sizes > 0
    for f in ("centroids", "centroids_bf16", "vsum"):
        assert np.array_equal(got[f][nz], getattr(lay, f)[nz]), "%s of a non-empty cluster differs" % f
    # sampled units bit-exact
    nseg = [-(-int(n) // seg) for n in ctx]
    units = []
    for b in range(len(ctx)):
        for g in range(G):
            for s in range(nseg[b]):
                units.append((b, g, s))
    rb = np.concatenate([[0], np.cumsum(G * np.array(ctx))])
    cb = np.concatenate([[0], np.cumsum(G * np.array(C))])
    from concurrent.futures import ThreadPoolExecutor

    def ref_unit(u):
        b, g, s = units[u]
        N = int(ctx[b])
        r0 = rb[b] + g * N + s * seg
        L = min(seg, N - s * seg)
        return oracle.kmeans_segment(K[r0:r0 + L], oracle.segment_clusters(L, seg, K_s), iters, seed, key=oracle.seed_key(b, g, s))

    with ThreadPoolExecutor(len(sample)) as ex:  # the oracle releases the GIL
        refs = dict(zip(sample, ex.map(ref_unit, sample)))
    for u in sample:
        b, g, s = units[u]
        N = int(ctx[b])
        r0 = rb[b] + g * N + s * seg
        L = min(seg, N - s * seg)
        kc = oracle.segment_clusters(L, seg, K_s)
        say("  unit %d (b=%d g=%d s=%d)" % (u, b, g, s))
        a, c, _, _ = refs[u]
        assert np.array_equal(got["assign"][r0:r0 + L], a + s * K_s)
        c0 = cb[b] + g * C[b] + s * K_s
        assert np.array_equal(got["centroids"][c0:c0 + kc], c)


def test_full_size_128k():
    ctx = np.array([131072], np.int64)
    K, V, _ = synth.kv(2, 1, 8, ctx, 8192)
    _sampled_units("128K", K, V, 8, ctx, 8192, 512, 10, 1234, sample=[0, 37, 127])


def test_full_size_heavy_tailed_1m_keys():
    ctx = np.array([1048576], np.int64)
    K, _, _ = synth.kv(5, 1, 8, ctx, 8192, heavy=True, values=False)
    _sampled_units("1M x 8 student-t", K, K, 8, ctx, 8192, 512, 10, 1234, sample=[0, 511, 1023])


def test_segments_of_16384_with_1024_clusters():
    # the 1M layer's segment shape: the LDS radix sort at its 14-bit position limit and
    # k_assign with more than 512 clusters per segment, 4096 tokens per workgroup; every
    # array bit-exact (two kv heads, a full and a partial segment each)
    ctx = [20000]
    K, V, _ = synth.kv(27, 1, 2, np.array(ctx), 16384)
    _check_all("seg=16384 K_s=1024", K, V, 2, ctx, 16384, 1024, 3, 41)


def test_full_size_1m_layer_build():
    # the 1M-token layer's build: 8 kv heads x 64 segments of 16384 tokens, 1024 clusters
    # each, 10 rounds; layout invariants on every block, sampled units bit-exact
    ctx = np.array([1048576], np.int64)
    K, _, _ = synth.kv(3, 1, 8, ctx, 16384, values=False)
    _sampled_units("1M layer", K, K, 8, ctx, 16384, 1024, 10, 1234, sample=[0, 262, 511])
