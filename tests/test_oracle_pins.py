"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test fixes one part of the oracle with something other than the oracle itself:
format definitions and hand-worked rounding cases, published generator outputs,
brute force on tiny inputs, library routines (scipy, scikit-learn, torch's bf16
conversion), closed forms and invariants.  The method is RetroInfer's wave index
(gist.science summary page, section 2.A: steady, retrieval and estimation zones over
a segmented-clustered KV cache).
"""
import itertools
import math

import numpy as np
import pytest
import scipy.cluster.vq
import scipy.special
import torch

import oracle
import synth

D = 128


def _bits(x):
    return np.array([x], dtype=np.float32).view(np.uint32)[0]


def _f(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


# ------------------------------------------------------------------------- bf16
@pytest.mark.parametrize("src,dst", [
    (0x3F808000, 0x3F80),  # 1 + 2^-8: halfway between 0x3F80 and 0x3F81, tie to even -> 0x3F80
    (0x3F818000, 0x3F82),  # halfway between 0x3F81 and 0x3F82, tie to even -> 0x3F82
    (0x3F80C000, 0x3F81),  # above halfway -> up
    (0x3F804000, 0x3F80),  # below halfway -> down
    (0xBF808000, 0xBF80),  # negative tie, magnitude rounds to even
    (0x7F7FFFFF, 0x7F80),  # largest float rounds past the largest bf16 to infinity
    (0x00000000, 0x0000),
    (0x80000000, 0x8000),  # -0 stays -0
])
def test_bf16_rne_hand_cases(src, dst):
    assert oracle.f32_to_bf16(np.array([_f(src)]))[0] == dst


def test_bf16_roundtrip_and_library_conversion():
    # every non-NaN bf16 value is exactly representable: widening then rounding returns it
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(h)
    ok = ~np.isnan(f)
    assert np.array_equal(oracle.f32_to_bf16(f[ok]), h[ok])
    # NaN stays NaN
    assert np.isnan(oracle.bf16_to_f32(oracle.f32_to_bf16(np.array([np.nan], np.float32))))[0]
    # random floats: same as torch's round-to-nearest-even float32 -> bfloat16 conversion
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16(x), ref)


# ------------------------------------------------------------------- SplitMix64
def test_splitmix64_published_outputs():
    # Reference outputs of SplitMix64 (Steele, Lea and Flood 2014; public-domain
    # reference implementation): state 0 and state 1234567.
    assert [int(v) for v in oracle.splitmix64_stream(0, 3)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert [int(v) for v in oracle.splitmix64_stream(1234567, 5)] == [
        6457827717110365317, 3203168211198807973, 9817491932198370423, 4593380528125082431,
        16408922859458223821]


def test_seed_key_closed_form():
    # stream key of (b, g, s): b*2^56 + g*2^40 + s*2^16 modulo 2^64
    assert oracle.seed_key(0, 0, 0) == 0
    assert oracle.seed_key(0, 0, 1) == 1 << 16
    assert oracle.seed_key(0, 1, 0) == 1 << 40
    assert oracle.seed_key(1, 0, 0) == 1 << 56
    assert oracle.seed_key(3, 7, 11) == (3 << 56) + (7 << 40) + (11 << 16)
    assert oracle.seed_key(255, (1 << 16) - 1, (1 << 24) - 1) == (1 << 64) - (1 << 16)


def _fisher_yates(L, K, state):
    # the partial shuffle written out from its definition over the pinned SplitMix64 stream
    a = list(range(L))
    for i, r in enumerate(oracle.splitmix64_stream(state, K).tolist()):
        j = i + r % (L - i)
        a[i], a[j] = a[j], a[i]
    return a[:K]


def test_init_indices_are_the_seeded_partial_shuffle():
    # segment with stream key k: SplitMix64 from state seed + gamma*(k+1), one draw per swap
    gamma = 0x9E3779B97F4A7C15
    for L, K, seed, key in [(37, 3, 5, 0), (100, 100, 1234, oracle.seed_key(1, 2, 3)), (8192, 64, 99, 1 << 16),
                            (5, 5, (1 << 64) - 1, oracle.seed_key(255, 3, 0))]:
        st = (seed + gamma * (key + 1)) % (1 << 64)
        assert oracle.init_indices(L, K, seed, key).tolist() == _fisher_yates(L, K, st), (L, K, key)


def test_init_indices_distinct_in_range():
    for L, K in [(8192, 512), (100, 100), (37, 3), (1, 1)]:
        for s in range(5):
            idx = oracle.init_indices(L, K, 1234, oracle.seed_key(0, 0, s))
            assert len(set(idx.tolist())) == K
            assert idx.min() >= 0 and idx.max() < L
    # K = L: the shuffle is a full permutation
    assert sorted(oracle.init_indices(64, 64, 7, 3).tolist()) == list(range(64))
    # deterministic, and different keys differ
    k0, k1 = oracle.seed_key(0, 0, 0), oracle.seed_key(0, 1, 0)
    assert np.array_equal(oracle.init_indices(8192, 512, 1, k0), oracle.init_indices(8192, 512, 1, k0))
    assert not np.array_equal(oracle.init_indices(8192, 512, 1, k0), oracle.init_indices(8192, 512, 1, k1))


def test_init_shuffle_is_uniform():
    # Fisher-Yates draws every permutation with equal probability; the classic
    # "j = next() mod L" mistake does not (chi-square over the 24 orders of 4 items).
    counts = {}
    n = 48000
    for s in range(n):
        p = tuple(oracle.init_indices(4, 4, 99, oracle.seed_key(0, 0, s)).tolist())
        counts[p] = counts.get(p, 0) + 1
    assert len(counts) == 24
    exp = n / 24
    chi2 = sum((c - exp) ** 2 / exp for c in counts.values())
    assert chi2 < 60.0  # 23 dof: p ~ 5e-5 at 60


# ------------------------------------------------------------- segments and k
def test_segment_cluster_counts():
    assert oracle.num_clusters(16384, 8192, 512) == 1024
    assert oracle.num_clusters(131072, 8192, 512) == 8192
    assert oracle.num_clusters(1048576, 16384, 1024) == 65536
    assert oracle.num_clusters(1048576, 8192, 512) == 65536
    # partial last segment of 1000 tokens: ceil(1000 * 512 / 8192) = ceil(62.5) = 63
    assert oracle.segment_clusters(1000, 8192, 512) == 63
    assert oracle.num_clusters(8 * 8192 + 1000, 8192, 512) == 8 * 512 + 63
    assert oracle.segment_clusters(1, 8192, 512) == 1
    assert oracle.num_clusters(5, 8192, 512) == 1


@pytest.mark.parametrize("frac,C,k", [(0.05, 1024, 52), (0.02, 8192, 164), (0.018, 65536, 1180),
                                      (0.0, 8192, 0), (1.0, 8192, 8192), (1e-9, 10, 1)])
def test_k_from_frac(frac, C, k):
    assert oracle.k_from_frac(frac, C) == k


# ---------------------------------------------------------------------- k-means
def _tiny_data(seed, L, spread=3.0):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((L, D)) * 0.3
    X[:, :4] += rng.integers(0, 4, (L, 1)) * spread  # a few separated groups along the first dims
    return oracle.f32_to_bf16(X.astype(np.float32))


def test_assign_point_matches_scipy_vq():
    rng = np.random.default_rng(1)
    X = oracle.f32_to_bf16(rng.standard_normal((300, D)).astype(np.float32))
    Cb = oracle.f32_to_bf16(rng.standard_normal((17, D)).astype(np.float32))
    codes, _ = scipy.cluster.vq.vq(oracle.bf16_to_f32(X).astype(np.float64), oracle.bf16_to_f32(Cb).astype(np.float64))
    ours = np.array([oracle.assign_point(x, Cb) for x in X])
    assert np.array_equal(ours, codes)


def test_assign_ties_go_to_lowest_id():
    rng = np.random.default_rng(2)
    c = oracle.f32_to_bf16(rng.standard_normal((1, D)).astype(np.float32))
    other = oracle.f32_to_bf16(rng.standard_normal((1, D)).astype(np.float32) + 5)
    chat = np.concatenate([other, c, c, c])  # ids 1, 2, 3 identical
    assert oracle.assign_point(c[0], chat) == 1


def test_kmeans_hand_example_two_groups():
    # Six points on the first axis, two groups {-2,-1.5,-1} and {1,1.5,2}; whatever two
    # tokens the seeded init picks, Lloyd's rounds reach the two groups with means -1.5
    # and 1.5 (exact in fp32: -4.5/3 and 4.5/3).
    vals = [-2.0, -1.5, -1.0, 1.0, 1.5, 2.0]
    X = np.zeros((6, D), np.float32)
    X[:, 0] = vals
    Xb = oracle.f32_to_bf16(X)
    for seed in range(20):
        a, c, _, _ = oracle.kmeans_segment(Xb, 2, 6, seed)
        assert a[0] == a[1] == a[2] and a[3] == a[4] == a[5] and a[0] != a[3]
        assert c[a[0], 0] == -1.5 and c[a[3], 0] == 1.5
        assert np.all(c[:, 1:] == 0.0)


def test_kmeans_exact_mode_matches_sklearn_lloyd():
    from sklearn.cluster import KMeans
    for seed in range(3):
        Xb = _tiny_data(seed, 64)
        K, iters = 6, 30
        a, c, tr, obj = oracle.kmeans_segment(Xb, K, iters, 1000 + seed, exact=True)
        init = oracle.bf16_to_f32(Xb[oracle.init_indices(64, K, 1000 + seed, 0)]).astype(np.float64)
        km = KMeans(n_clusters=K, init=init, n_init=1, max_iter=iters, tol=0.0, algorithm="lloyd")
        km.fit(oracle.bf16_to_f32(Xb).astype(np.float64))
        assert np.array_equal(a, km.labels_)
        np.testing.assert_allclose(c, km.cluster_centers_.astype(np.float32), rtol=1e-6, atol=1e-6)


def test_kmeans_exact_mode_objective_monotone():
    K, _, _ = synth.kv(11, 1, 1, np.array([2048]), 2048)
    for s in range(3):
        _, _, _, obj = oracle.kmeans_segment(K, 128, 10, 5, key=oracle.seed_key(0, 0, s), exact=True)
        assert np.all(obj[1:] <= obj[:-1] * (1 + 1e-12)), obj
    # spec mode (bf16 centroids in the assignment) stays monotone to 1e-3
    _, _, _, obj = oracle.kmeans_segment(K, 128, 10, 5, key=0, exact=False)
    assert np.all(obj[1:] <= obj[:-1] * (1 + 1e-3)), obj


def test_kmeans_update_is_ordered_fp32_mean():
    # one round: centroids are the ordered fp32 sums of the first assignment's members
    # divided by n (numpy's sequential float32 cumsum and IEEE float32 division);
    # empty clusters keep the initial token.
    Xb = _tiny_data(5, 300)
    K = 40
    a, c, tr, _ = oracle.kmeans_segment(Xb, K, 1, 77, key=2)
    X = oracle.bf16_to_f32(Xb)
    init = oracle.init_indices(300, K, 77, 2)
    for j in range(K):
        mem = np.nonzero(tr[0] == j)[0]
        if len(mem) == 0:
            assert np.array_equal(c[j], X[init[j]])
            continue
        S = np.cumsum(X[mem], axis=0, dtype=np.float32)[-1]
        assert np.array_equal(c[j], S / np.float32(len(mem)))


def test_kmeans_brute_force_tiny():
    # tiny segments: every assignment is the brute-force argmin over all centroids
    # computed independently (float64 distances through numpy), with the centroids
    # the oracle used in that round (bf16 of the previous round's fp32 centroids).
    Xb = _tiny_data(9, 48)
    K, iters = 5, 4
    X = oracle.bf16_to_f32(Xb).astype(np.float64)
    init = oracle.init_indices(48, K, 3, 0)
    cent = X[init].astype(np.float32)
    _, _, tr, _ = oracle.kmeans_segment(Xb, K, iters, 3)
    for it in range(iters):
        chat = oracle.bf16_to_f32(oracle.f32_to_bf16(cent)).astype(np.float64)
        d = ((X[:, None, :] - chat[None, :, :]) ** 2).sum(-1)
        assert np.array_equal(tr[it], d.argmin(1))
        for j in range(K):
            mem = np.nonzero(tr[it] == j)[0]
            if len(mem):
                cent[j] = np.cumsum(X[mem].astype(np.float32), axis=0, dtype=np.float32)[-1] / np.float32(len(mem))


# ------------------------------------------------------------------ index layout
def _small_build(seed=3, ctx=(3000, 1700), G=2, seg=1024, K_s=64, iters=3):
    ctx = np.array(ctx, np.int64)
    K, V, _ = synth.kv(seed, len(ctx), G, ctx, seg)
    idx = oracle.build(K, V, G, ctx, seg, K_s, iters, 1234)
    return K, V, ctx, idx


def test_layout_invariants():
    K, V, ctx, idx = _small_build()
    G = idx.G
    row = clu = off = 0
    for b, N in enumerate(ctx):
        C = oracle.num_clusters(int(N), idx.seg_len, idx.K_s)
        for g in range(G):
            sl = slice(row, row + N)
            perm, inv, a = idx.perm[sl], idx.inv_perm[sl], idx.assign[sl]
            assert np.array_equal(np.sort(perm), np.arange(N))
            assert np.array_equal(inv[perm], np.arange(N))
            assert np.array_equal(idx.k_sorted[sl], K[sl][perm])
            assert np.array_equal(idx.v_sorted[sl], V[sl][perm])
            # sorted by (cluster, position)
            key = a[perm].astype(np.int64) * (N + 1) + perm
            assert np.all(np.diff(key) > 0)
            sizes = idx.sizes[clu:clu + C]
            offs = idx.offsets[off:off + C + 1]
            assert np.array_equal(sizes, np.bincount(a, minlength=C))
            assert offs[0] == 0 and np.array_equal(np.diff(offs), sizes)
            # segments: ids of segment s own exactly its tokens; offsets at segment bases
            nseg = -(-N // idx.seg_len)
            for s in range(nseg):
                t0, t1 = s * idx.seg_len, min((s + 1) * idx.seg_len, N)
                kc = oracle.segment_clusters(t1 - t0, idx.seg_len, idx.K_s)
                assert a[t0:t1].min() >= s * idx.K_s and a[t0:t1].max() < s * idx.K_s + kc
                assert offs[s * idx.K_s] == t0
            Vf = oracle.bf16_to_f32(V[sl]).astype(np.float64)
            for j in range(C):
                mem = np.nonzero(a == j)[0]
                vs = idx.vsum[clu + j]
                if len(mem) == 0:
                    assert np.all(vs == 0)
                    continue
                # ordered fp32 sum, and within 1e-6 of the exact sum
                assert np.array_equal(vs, np.cumsum(oracle.bf16_to_f32(V[sl][mem]), axis=0, dtype=np.float32)[-1])
                ex = Vf[mem].sum(0)
                assert np.all(np.abs(vs - ex) <= 1e-6 * np.abs(Vf[mem]).sum(0) + 1e-30)
            # chat = RNE bf16 of the fp32 centroids (torch's conversion)
            cc = idx.centroids[clu:clu + C]
            ref = torch.from_numpy(cc).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(idx.centroids_bf16[clu:clu + C], ref)
            row += N
            clu += C
            off += C + 1


def test_build_equals_per_segment_kmeans():
    # every (b, g, s) problem of a build is the segment's own k-means seeded by seed_key(b, g, s)
    K, V, ctx, idx = _small_build(ctx=(2500, 1100), G=2, iters=4)
    row = clu = 0
    for b, N in enumerate(ctx):
        C = oracle.num_clusters(int(N), 1024, 64)
        for g in range(2):
            for s in range(-(-int(N) // 1024)):
                t0, t1 = s * 1024, min((s + 1) * 1024, int(N))
                kc = oracle.segment_clusters(t1 - t0, 1024, 64)
                a, c, _, _ = oracle.kmeans_segment(K[row + t0:row + t1], kc, 4, 1234, key=oracle.seed_key(b, g, s))
                assert np.array_equal(idx.assign[row + t0:row + t1], a + s * 64), (b, g, s)
                assert np.array_equal(idx.centroids[clu + s * 64:clu + s * 64 + kc], c), (b, g, s)
            row += int(N)
            clu += C


def _block(idx, ctx, b, g):
    """(rows, clusters, offsets) slices of block (b, g) of an oracle index."""
    row = clu = off = 0
    for bb in range(b):
        C = oracle.num_clusters(int(ctx[bb]), idx.seg_len, idx.K_s)
        row, clu, off = row + idx.G * int(ctx[bb]), clu + idx.G * C, off + idx.G * (C + 1)
    N, C = int(ctx[b]), oracle.num_clusters(int(ctx[b]), idx.seg_len, idx.K_s)
    return (slice(row + g * N, row + (g + 1) * N), slice(clu + g * C, clu + (g + 1) * C),
            slice(off + g * (C + 1), off + (g + 1) * (C + 1)))


def test_build_of_a_longer_context_keeps_the_full_segments():
    # Segments are clustered independently and seeded by their own coordinates, so the index
    # of a longer context (same leading tokens) repeats every segment that was already full:
    # labels, centroids and value sums of its clusters, its sorted rows and offsets. Only
    # the segments from the first one that was partial on are new.
    seg, K_s, G = 512, 32, 3
    long = np.array([2300, 1600], np.int64)
    Kf, Vf, _ = synth.kv(21, 2, G, long, seg)
    full = oracle.build(Kf, Vf, G, long, seg, K_s, 3, 77)
    for short in ([1024, 1537], [2047, 512], [1, 1600]):
        short = np.array(short, np.int64)
        rows = np.concatenate([np.arange(sum(G * long[:b]) + g * long[b], sum(G * long[:b]) + g * long[b] + short[b])
                               for b in range(2) for g in range(G)])
        part = oracle.build(Kf[rows], Vf[rows], G, short, seg, K_s, 3, 77)
        for b in range(2):
            keep = int(short[b]) // seg  # segments full in the shorter context
            nk, ck = keep * seg, keep * K_s
            for g in range(G):
                (rs, cs, os_), (rl, cl, ol) = _block(part, short, b, g), _block(full, long, b, g)
                for name in ("assign", "perm", "inv_perm", "k_sorted", "v_sorted"):
                    assert np.array_equal(getattr(part, name)[rs][:nk], getattr(full, name)[rl][:nk]), (name, b, g)
                for name in ("sizes", "centroids", "centroids_bf16", "vsum"):
                    assert np.array_equal(getattr(part, name)[cs][:ck], getattr(full, name)[cl][:ck]), (name, b, g)
                assert np.array_equal(part.offsets[os_][:ck + 1], full.offsets[ol][:ck + 1]), (b, g)


# ---------------------------------------------------------------------- rank key
def _bf(vals):
    return oracle.f32_to_bf16(np.asarray(vals, np.float32))


def test_rank_key_error_bound():
    rng = np.random.default_rng(4)
    for _ in range(200):
        q = _bf(rng.standard_normal(D) * rng.uniform(0.1, 10))
        c = _bf(rng.standard_normal(D) * rng.uniform(0.1, 10))
        p = oracle.bf16_to_f32(q).astype(np.float64) * oracle.bf16_to_f32(c).astype(np.float64)
        r = oracle.rank_key(q, c)
        assert abs(r - p.sum()) <= 128 * 2.0 ** -24 * np.abs(p).sum()


def test_rank_key_tree_order_worked_cases():
    ones = np.ones(D, np.float32)
    # (1) inside a lane the 8 products are added left to right from +0:
    #     dims 0,1,2 = 2^24, 1, 1 -> ((2^24 + 1) + 1): 2^24 + 1 is a tie between 2^24 and
    #     2^24 + 2 and rounds to the even 2^24, twice -> 2^24 (any order adding the two
    #     ones first would give 2^24 + 2 exactly).
    c = np.zeros(D, np.float32)
    c[0], c[1], c[2] = 2.0 ** 24, 1.0, 1.0
    assert oracle.rank_key(_bf(ones), _bf(c)) == 2.0 ** 24
    # (2) lanes hold consecutive 8-dim blocks: dims 0 and 8 (lanes 0 and 1) with the
    #     same values do not share a lane sum; butterfly s=8: lanes 0+8, 1+9 -> u0 = 2^24,
    #     u1 = 1; ... s=1: 2^24 + 1 -> 2^24. Check with dims 0 = 2^24 and 8 = 1, 16 = 1:
    #     lanes 0, 1, 2 -> s=8,4 leave them; s=2: u0+u2 = 2^24+1 -> 2^24, u1+u3 = 1;
    #     s=1: 2^24 + 1 -> 2^24.
    c = np.zeros(D, np.float32)
    c[0], c[8], c[16] = 2.0 ** 24, 1.0, 1.0
    assert oracle.rank_key(_bf(ones), _bf(c)) == 2.0 ** 24
    # (3) butterfly order s = 8, 4, 2, 1: lane 0 = 2^24, lane 8 = 1, lane 12 = 1.
    #     s=8: u0 = 2^24 + 1 -> 2^24, u4 = u4 + u12 = 1; s=4: u0 = 2^24 + 1 -> 2^24 -> 2^24.
    #     (Order s = 4 first would give u8 + u12 = 2 and then 2^24 + 2 exactly.)
    c = np.zeros(D, np.float32)
    c[0], c[64], c[96] = 2.0 ** 24, 1.0, 1.0
    assert oracle.rank_key(_bf(ones), _bf(c)) == 2.0 ** 24
    # (4) q = 0 gives +0 (sign bit clear)
    r = oracle.rank_key(_bf(np.zeros(D)), _bf(-np.ones(D)))
    assert r == 0.0 and not math.copysign(1.0, r) < 0
    # (5) a unit query picks one coordinate exactly
    e = np.zeros(D, np.float32)
    e[37] = 1.0
    c = np.random.default_rng(5).standard_normal(D).astype(np.float32)
    assert oracle.rank_key(_bf(e), _bf(c)) == oracle.bf16_to_f32(_bf(c))[37]


def test_select_brute_force_with_ties():
    rng = np.random.default_rng(6)
    for trial in range(50):
        n = int(rng.integers(1, 300))
        keys = rng.choice(np.array([-1.5, -0.0, 0.0, 0.25, 3.0, 7.5], np.float32), n)
        ids = rng.permutation(1000)[:n].astype(np.int32)
        k = int(rng.integers(0, n + 1))
        got = oracle.select(keys, ids, k)
        want = [i for _, i in sorted(zip(keys.tolist(), ids.tolist()), key=lambda t: (-t[0], t[1]))][:k]
        assert got.tolist() == want


# ------------------------------------------------------------------------ decode
def _softmax_attention(K, V, q, G, ctx):
    """Dense attention through scipy.special.softmax, float64."""
    B, H = q.shape[:2]
    out = np.zeros((B, H, D))
    row = 0
    for b, N in enumerate(ctx):
        for h in range(H):
            g = h * G // H
            Kf = oracle.bf16_to_f32(K[row + g * N: row + (g + 1) * N]).astype(np.float64)
            Vf = oracle.bf16_to_f32(V[row + g * N: row + (g + 1) * N]).astype(np.float64)
            qf = oracle.bf16_to_f32(q[b, h]).astype(np.float64)
            w = scipy.special.softmax(Kf @ qf / math.sqrt(D))
            out[b, h] = w @ Vf
        row += G * N
    return out


def _setup_decode(seed=21, ctx=(3000, 1700), G=2, H=4, seg=1024, K_s=64, iters=3):
    K, V, ctx, idx = _small_build(seed, ctx, G, seg, K_s, iters)
    q, _ = synth.queries(seed + 1, 1, len(ctx), H, G, ctx, K)
    return K, V, ctx, idx, q[0]


def test_full_attention_matches_scipy_softmax():
    K, V, ctx, idx, q = _setup_decode()
    of, _ = oracle.full_attention(K, V, q, idx.G, ctx)
    np.testing.assert_allclose(of, _softmax_attention(K, V, q, idx.G, ctx), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n_sink,n_local", [(0, 0), (4, 64), (100, 0), (0, 333)])
def test_decode_topk_all_equals_full_attention(n_sink, n_local):
    # topk_frac = 1 retrieves every eligible cluster: the three zones together are
    # exactly dense attention, whatever the clustering.
    K, V, ctx, idx, q = _setup_decode()
    o, lse, ids, kc = oracle.decode(idx, K, V, q, n_sink, n_local, 1.0)
    of, lf = oracle.full_attention(K, V, q, idx.G, ctx)
    np.testing.assert_allclose(o, of, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lf, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("frac,n_sink,n_local", [(0.0, 0, 0), (0.05, 4, 64), (0.3, 0, 17), (0.0, 50, 50)])
def test_decode_singleton_clusters_equal_full_attention(frac, n_sink, n_local):
    # clusters_per_seg = seg_len: every token is its own cluster, its centroid is the
    # key itself, so the estimation zone is exact and any split of the zones gives
    # dense attention.
    ctx = np.array([700, 300], np.int64)
    G, H, seg = 2, 4, 256
    K, V, _ = synth.kv(31, 2, G, ctx, seg)
    idx = oracle.build(K, V, G, ctx, seg, seg, 2, 9)
    q, _ = synth.queries(32, 1, 2, H, G, ctx, K)
    o, lse, _, _ = oracle.decode(idx, K, V, q[0], n_sink, n_local, frac)
    of, lf = oracle.full_attention(K, V, q[0], G, ctx)
    np.testing.assert_allclose(o, of, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(lse, lf, rtol=1e-10, atol=1e-10)


def test_decode_zero_query_closed_forms():
    # q = 0: every score is 0, every rank key +0, so the ids are the k lowest eligible
    # ids in ascending order, and every token weighs the same: o = mean of all V
    # (up to the fp32 rounding of the stored value sums, <= 1e-8 here).
    K, V, ctx, idx, q = _setup_decode()
    q0 = np.zeros_like(q)
    for frac, ns, nl in [(0.05, 4, 64), (0.2, 0, 0), (0.0, 10, 10)]:
        o, lse, ids, kc = oracle.decode(idx, K, V, q0, ns, nl, frac)
        row = 0
        for b, N in enumerate(ctx):
            C = int(idx.C[b])
            for h in range(q.shape[1]):
                g = h * idx.G // q.shape[1]
                sl = slice(row + g * N, row + (g + 1) * N)
                Vf = oracle.bf16_to_f32(V[sl]).astype(np.float64)
                np.testing.assert_allclose(o[b, h], Vf.mean(0), rtol=0, atol=1e-8)
                assert abs(lse[b, h] - math.log(N)) < 1e-12
                t = np.arange(N)
                nonsteady = ~((t < ns) | (t >= N - nl))
                elig = np.unique(idx.assign[sl][nonsteady])
                k = min(oracle.k_from_frac(frac, C), len(elig))
                assert kc[b, h] == k
                assert ids[b, h, :k].tolist() == elig[:k].tolist()
                assert np.all(ids[b, h, k:] == -1)
            row += idx.G * N


def test_decode_constant_values():
    K, V, ctx, idx, q = _setup_decode()
    v = np.random.default_rng(3).standard_normal(D).astype(np.float32)
    Vc = np.tile(oracle.f32_to_bf16(v), (V.shape[0], 1))
    idx2 = oracle.build(K, Vc, idx.G, ctx, idx.seg_len, idx.K_s, 3, 1234)
    o, _, _, _ = oracle.decode(idx2, K, Vc, q, 4, 64, 0.05)
    want = oracle.bf16_to_f32(oracle.f32_to_bf16(v)).astype(np.float64)
    np.testing.assert_allclose(o, np.broadcast_to(want, o.shape), rtol=1e-6, atol=1e-6)


def test_decode_all_steady():
    K, V, ctx, idx, q = _setup_decode()
    o, lse, ids, kc = oracle.decode(idx, K, V, q, 1500, 1500, 0.05)  # covers N_b = 3000 and 1700
    of, lf = oracle.full_attention(K, V, q, idx.G, ctx)
    np.testing.assert_allclose(o, of, rtol=1e-12, atol=1e-12)
    assert np.all(ids == -1) and np.all(kc == 0)


def test_decode_estimation_only_closed_form():
    # topk_frac = 0 and no steady tokens: o = sum_j e^{s_j} Vsum_j / sum_j e^{s_j} n_j
    K, V, ctx, idx, q = _setup_decode()
    o, lse, _, _ = oracle.decode(idx, K, V, q, 0, 0, 0.0)
    clu = 0
    for b, N in enumerate(ctx):
        C = int(idx.C[b])
        for h in range(q.shape[1]):
            g = h * idx.G // q.shape[1]
            cs = slice(clu + g * C, clu + (g + 1) * C)
            n = idx.sizes[cs].astype(np.float64)
            chat = oracle.bf16_to_f32(idx.centroids_bf16[cs]).astype(np.float64)
            s = chat @ oracle.bf16_to_f32(q[b, h]).astype(np.float64) / math.sqrt(D)
            s = np.where(n > 0, s, -np.inf)
            w = np.exp(s - s.max())
            want = (w[:, None] * idx.vsum[cs].astype(np.float64)).sum(0) / (w * n).sum()
            np.testing.assert_allclose(o[b, h], want, rtol=1e-10, atol=1e-10)
        clu += idx.G * C


def test_decode_selection_brute_force():
    # ids are the brute-force top-k of the rank keys over eligible clusters
    K, V, ctx, idx, q = _setup_decode()
    ns, nl, frac = 4, 64, 0.1
    _, _, ids, kc = oracle.decode(idx, K, V, q, ns, nl, frac)
    row = clu = 0
    for b, N in enumerate(ctx):
        C = int(idx.C[b])
        for h in range(q.shape[1]):
            g = h * idx.G // q.shape[1]
            a = idx.assign[row + g * N: row + (g + 1) * N]
            t = np.arange(N)
            elig = np.unique(a[~((t < ns) | (t >= N - nl))])
            keys = [oracle.rank_key(q[b, h], idx.centroids_bf16[clu + g * C + j]) for j in elig]
            k = min(oracle.k_from_frac(frac, C), len(elig))
            want = [j for _, j in sorted(zip(keys, elig.tolist()), key=lambda u: (-u[0], u[1]))][:k]
            assert ids[b, h, :k].tolist() == want
        row += idx.G * N
        clu += idx.G * C


# ------------------------------------------------------------- block baseline
def test_block_assign_closed_form():
    # token i of a segment of L tokens with K(s) blocks is in block floor(i K(s) / L):
    # contiguous, ascending, block j holds ceil((j+1) L / K) - ceil(j L / K) tokens
    G, seg, K_s = 2, 1000, 64
    ctx = np.array([2500, 999, 1], np.int64)
    a = oracle.block_assign(G, ctx, seg, K_s)
    row = 0
    for N in ctx:
        for g in range(G):
            blk = a[row: row + N]
            for s0 in range(0, N, seg):
                L = min(seg, N - s0)
                Kc = oracle.segment_clusters(L, seg, K_s)
                loc = blk[s0: s0 + L] - (s0 // seg) * K_s
                assert np.all(np.diff(loc) >= 0) and loc[0] == 0 and loc[-1] == Kc - 1
                cnt = np.bincount(loc, minlength=Kc)
                want = [-(-(j + 1) * L // Kc) - -(-j * L // Kc) for j in range(Kc)]
                assert cnt.tolist() == want
            row += N


def test_block_index_is_identity_layout_with_block_means():
    ctx = np.array([1500, 700], np.int64)
    G, seg, K_s = 2, 512, 32
    K, V, _ = synth.kv(41, 2, G, ctx, seg)
    idx = oracle.build_blocks(K, V, G, ctx, seg, K_s)
    assert np.array_equal(idx.perm, np.concatenate([np.arange(N) for N in ctx for _ in range(G)]))
    assert np.array_equal(idx.k_sorted, K) and np.array_equal(idx.v_sorted, V)
    # centroid = ordered fp32 mean of the block's keys (numpy float32 cumulative sum in order)
    a = oracle.block_assign(G, ctx, seg, K_s)
    row = clu = 0
    for N in ctx:
        C = oracle.num_clusters(int(N), seg, K_s)
        for g in range(G):
            for j in (0, 7, C - 1):
                m = np.nonzero(a[row: row + N] == j)[0]
                x = oracle.bf16_to_f32(K[row + m]).astype(np.float32)
                acc = np.zeros(D, np.float32)
                for r in x:
                    acc = (acc + r).astype(np.float32)
                assert np.array_equal(idx.centroids[clu + j], (acc / np.float32(len(m))).astype(np.float32))
            row += N
            clu += C


def _masked_attention(K, V, q, G, ctx, keep):
    """Softmax attention of every (b, h) over the rows keep[b][h] (boolean per token), float64."""
    B, H = q.shape[:2]
    out = np.zeros((B, H, D))
    row = 0
    for b, N in enumerate(ctx):
        for h in range(H):
            g = h * G // H
            sl = slice(row + g * N, row + (g + 1) * N)
            Kf = oracle.bf16_to_f32(K[sl]).astype(np.float64)[keep[b][h]]
            Vf = oracle.bf16_to_f32(V[sl]).astype(np.float64)[keep[b][h]]
            w = scipy.special.softmax(Kf @ oracle.bf16_to_f32(q[b, h]).astype(np.float64) / math.sqrt(D))
            out[b, h] = w @ Vf
        row += G * N
    return out


@pytest.mark.parametrize("blocks", [False, True])
def test_decode_topk_only_is_masked_attention(blocks):
    # without the estimation zone the output is softmax attention restricted to the steady
    # tokens and the members of the selected clusters (brute force with scipy's softmax)
    K, V, ctx, idx, q = _setup_decode()
    if blocks:
        idx = oracle.build_blocks(K, V, idx.G, ctx, idx.seg_len, idx.K_s)
    ns, nl, frac = 4, 64, 0.1
    o, lse, ids, kc = oracle.decode_topk(idx, K, V, q, ns, nl, frac)
    _, _, ids_w, kc_w = oracle.decode(idx, K, V, q, ns, nl, frac)
    assert np.array_equal(ids, ids_w) and np.array_equal(kc, kc_w)  # same selection as the wave decode
    keep, row = [], 0
    for b, N in enumerate(ctx):
        keep.append([])
        for h in range(q.shape[1]):
            g = h * idx.G // q.shape[1]
            a = idx.assign[row + g * N: row + (g + 1) * N]
            t = np.arange(N)
            keep[b].append(((t < ns) | (t >= N - nl)) | np.isin(a, ids[b, h, :kc[b, h]]))
        row += idx.G * N
    np.testing.assert_allclose(o, _masked_attention(K, V, q, idx.G, ctx, keep), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("n_sink,n_local", [(0, 0), (4, 64)])
def test_decode_topk_only_all_selected_equals_full_attention(n_sink, n_local):
    K, V, ctx, idx, q = _setup_decode()
    idxb = oracle.build_blocks(K, V, idx.G, ctx, idx.seg_len, idx.K_s)
    of, lf = oracle.full_attention(K, V, q, idx.G, ctx)
    for ix in (idx, idxb):
        o, lse, _, _ = oracle.decode_topk(ix, K, V, q, n_sink, n_local, 1.0)
        np.testing.assert_allclose(o, of, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, lf, rtol=1e-12, atol=1e-12)


# -------------------------------------------------- selection shared by a kv head
def test_decode_shared_one_q_head_per_kv_head_is_decode():
    # with one q head per kv head the group key is that head's rank key
    K, V, ctx, idx, q = _setup_decode(H=2, G=2)
    for frac, ns, nl in [(0.05, 4, 64), (0.2, 0, 0), (0.5, 7, 0)]:
        a = oracle.decode(idx, K, V, q, ns, nl, frac)
        s = oracle.decode(idx, K, V, q, ns, nl, frac, shared=True)
        for x, y in zip(a, s):
            assert np.array_equal(x, y)


def test_decode_shared_equal_q_heads_is_decode():
    # two equal q heads per kv head: the group key is 2 r (exact), which orders the
    # clusters as r does, so the selection and every output equal the per-head decode
    K, V, ctx, idx, q = _setup_decode(H=4, G=2)
    q2 = q.copy()
    q2[:, 1] = q2[:, 0]
    q2[:, 3] = q2[:, 2]
    for frac, ns, nl in [(0.05, 4, 64), (0.3, 0, 17)]:
        a = oracle.decode(idx, K, V, q2, ns, nl, frac)
        s = oracle.decode(idx, K, V, q2, ns, nl, frac, shared=True)
        for x, y in zip(a, s):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("n_sink,n_local", [(0, 0), (4, 64)])
def test_decode_shared_all_and_none(n_sink, n_local):
    # everything or nothing retrieved: the selection no longer matters
    K, V, ctx, idx, q = _setup_decode()
    o, lse, _, _ = oracle.decode(idx, K, V, q, n_sink, n_local, 1.0, shared=True)
    of, lf = oracle.full_attention(K, V, q, idx.G, ctx)
    np.testing.assert_allclose(o, of, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lf, rtol=1e-12, atol=1e-12)
    a = oracle.decode(idx, K, V, q, n_sink, n_local, 0.0)
    s = oracle.decode(idx, K, V, q, n_sink, n_local, 0.0, shared=True)
    for x, y in zip(a, s):
        assert np.array_equal(x, y)


def test_decode_shared_selection_is_top_k_of_summed_queries():
    # the group key equals (sum of the group's q) . chat_j up to the fp32 rounding of the
    # rank keys and of their sum (below 2^-20 of sum_h |q_h| |chat_j| here); so the selected
    # clusters' binary64 group scores are, up to that bound, the k largest over E, in
    # descending order, and every q head of a kv head has the same ids
    K, V, ctx, idx, q = _setup_decode(H=8, G=2)
    ns, nl, frac = 4, 64, 0.1
    _, _, ids, kc = oracle.decode(idx, K, V, q, ns, nl, frac, shared=True)
    H = q.shape[1]
    GS = H // idx.G
    row = clu = 0
    for b, N in enumerate(ctx):
        C = int(idx.C[b])
        for g in range(idx.G):
            hs = list(range(g * GS, (g + 1) * GS))
            for h in hs[1:]:
                assert ids[b, h].tolist() == ids[b, hs[0]].tolist() and kc[b, h] == kc[b, hs[0]]
            a = idx.assign[row + g * N: row + (g + 1) * N]
            t = np.arange(N)
            elig = np.unique(a[~((t < ns) | (t >= N - nl))])
            qf = oracle.bf16_to_f32(q[b, hs]).astype(np.float64)
            ch = oracle.bf16_to_f32(idx.centroids_bf16[clu + g * C: clu + (g + 1) * C]).astype(np.float64)
            score = ch[elig] @ qf.sum(0)
            bound = 2.0 ** -20 * (np.abs(ch[elig]) @ np.abs(qf).sum(0))
            k = min(oracle.k_from_frac(frac, C), len(elig))
            assert kc[b, hs[0]] == k
            sel = ids[b, hs[0], :k]
            pos = {j: i for i, j in enumerate(elig.tolist())}
            si = np.array([pos[j] for j in sel.tolist()])
            rest = np.setdiff1d(np.arange(len(elig)), si)
            assert len(set(sel.tolist())) == k
            if len(rest):
                assert np.all(score[si] + bound[si] >= score[rest].max() - bound[rest].max())
            assert np.all(score[si][:-1] + bound[si][:-1] >= score[si][1:] - bound[si][1:])
        row += idx.G * N
        clu += idx.G * C


# ------------------------------------------- tokens appended after the index was built
def _split_tail(Kf, Vf, ctx_full, tail, G, cap):
    """Split [b][g][t] rows of ctx_full into the first ctx_full - tail tokens of every (b, g)
    (index input) and the rest as tails [B][G][cap][128] (zero padded)."""
    B = len(ctx_full)
    ctx_idx = np.array([n - t for n, t in zip(ctx_full, tail)], np.int64)
    Ki, Vi, Kt, Vt = [], [], np.zeros((B, G, cap, D), np.uint16), np.zeros((B, G, cap, D), np.uint16)
    row = 0
    for b, (N, T) in enumerate(zip(ctx_full, tail)):
        for g in range(G):
            r = row + g * N
            Ki.append(Kf[r:r + N - T])
            Vi.append(Vf[r:r + N - T])
            Kt[b, g, :T] = Kf[r + N - T:r + N]
            Vt[b, g, :T] = Vf[r + N - T:r + N]
        row += G * N
    return np.concatenate(Ki), np.concatenate(Vi), ctx_idx, Kt, Vt


def _tail_setup(tail=(40, 0), cap=64, seed=41):
    G, H, seg, K_s = 2, 4, 1024, 64
    ctx_full = np.array([3000 + tail[0], 1700 + tail[1]], np.int64)
    Kf, Vf, _ = synth.kv(seed, 2, G, ctx_full, seg)
    Ki, Vi, ctx, Kt, Vt = _split_tail(Kf, Vf, ctx_full, tail, G, cap)
    idx = oracle.build(Ki, Vi, G, ctx, seg, K_s, 3, 1234)
    q, _ = synth.queries(seed + 1, 1, 2, H, G, ctx_full, Kf)
    return Kf, Vf, ctx_full, Ki, Vi, ctx, Kt, Vt, idx, q[0]


def test_decode_tail_empty_is_decode():
    Kf, Vf, cf, Ki, Vi, ctx, Kt, Vt, idx, q = _tail_setup()
    a = oracle.decode(idx, Ki, Vi, q, 4, 64, 0.05)
    t = oracle.decode_tail(idx, Ki, Vi, q, 4, 64, 0.05, Kt, Vt, [0, 0])
    for x, y in zip(a, t):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("frac,ns,nl", [(1.0, 4, 64), (1.0, 0, 0), (0.05, 1500, 1500)])
def test_decode_tail_everything_exact_is_full_attention(frac, ns, nl):
    # every indexed token exact (all clusters retrieved, or all steady) and the tail exact:
    # dense attention over the indexed tokens followed by the appended ones
    Kf, Vf, cf, Ki, Vi, ctx, Kt, Vt, idx, q = _tail_setup(tail=(40, 7))
    o, lse, _, _ = oracle.decode_tail(idx, Ki, Vi, q, ns, nl, frac, Kt, Vt, [40, 7])
    of, lf = oracle.full_attention(Kf, Vf, q, idx.G, cf)
    np.testing.assert_allclose(o, of, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lf, rtol=1e-12, atol=1e-12)


def test_decode_tail_estimation_only_closed_form():
    # topk_frac = 0, no steady tokens: the centroid terms of every cluster plus the exact tail
    Kf, Vf, cf, Ki, Vi, ctx, Kt, Vt, idx, q = _tail_setup(tail=(33, 64))
    tl = [33, 64]
    o, lse, _, _ = oracle.decode_tail(idx, Ki, Vi, q, 0, 0, 0.0, Kt, Vt, tl)
    clu = 0
    for b, N in enumerate(ctx):
        C = int(idx.C[b])
        for h in range(q.shape[1]):
            g = h * idx.G // q.shape[1]
            cs = slice(clu + g * C, clu + (g + 1) * C)
            n = idx.sizes[cs].astype(np.float64)
            qf = oracle.bf16_to_f32(q[b, h]).astype(np.float64)
            chat = oracle.bf16_to_f32(idx.centroids_bf16[cs]).astype(np.float64)
            s = np.where(n > 0, chat @ qf / math.sqrt(D), -np.inf)
            kt = oracle.bf16_to_f32(Kt[b, g, :tl[b]]).astype(np.float64)
            vt = oracle.bf16_to_f32(Vt[b, g, :tl[b]]).astype(np.float64)
            st = kt @ qf / math.sqrt(D)
            m = max(s.max(), st.max())
            w, wt = np.exp(s - m), np.exp(st - m)
            num = (w[:, None] * idx.vsum[cs].astype(np.float64)).sum(0) + wt @ vt
            den = (w * n).sum() + wt.sum()
            np.testing.assert_allclose(o[b, h], num / den, rtol=1e-10, atol=1e-10)
            assert abs(lse[b, h] - (m + math.log(den))) < 1e-10
        clu += idx.G * C


def test_decode_tail_rejects_lengths_beyond_capacity():
    Kf, Vf, cf, Ki, Vi, ctx, Kt, Vt, idx, q = _tail_setup()
    with pytest.raises(ValueError):
        oracle.decode_tail(idx, Ki, Vi, q, 4, 64, 0.05, Kt, Vt, [65, 0])


# ------------------------------------------------------------ bf16 value sums
def test_value_sums_bf16_is_rne_of_the_fp32_sums():
    # the reading: bf16 sums are the round-to-nearest-even of the ordered fp32 sums (torch's
    # float32 -> bfloat16 conversion is an independent implementation of that rounding)
    K, V, ctx, idx, q = _setup_decode()
    ref = torch.from_numpy(idx.vsum).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.value_sums_bf16(idx), ref)


def test_decode_bf16_sums_estimation_only_closed_form():
    # topk_frac = 0 and no steady tokens: o = sum_j e^{s_j} bf16(Vsum_j) / sum_j e^{s_j} n_j
    K, V, ctx, idx, q = _setup_decode()
    o, lse, _, _ = oracle.decode(idx, K, V, q, 0, 0, 0.0, vsum_bf16=True)
    vb = torch.from_numpy(idx.vsum).to(torch.bfloat16).to(torch.float64).numpy()
    clu = 0
    for b, N in enumerate(ctx):
        C = int(idx.C[b])
        for h in range(q.shape[1]):
            g = h * idx.G // q.shape[1]
            cs = slice(clu + g * C, clu + (g + 1) * C)
            n = idx.sizes[cs].astype(np.float64)
            chat = oracle.bf16_to_f32(idx.centroids_bf16[cs]).astype(np.float64)
            s = chat @ oracle.bf16_to_f32(q[b, h]).astype(np.float64) / math.sqrt(D)
            s = np.where(n > 0, s, -np.inf)
            w = np.exp(s - s.max())
            want = (w[:, None] * vb[cs]).sum(0) / (w * n).sum()
            np.testing.assert_allclose(o[b, h], want, rtol=1e-10, atol=1e-10)
        clu += idx.G * C


@pytest.mark.parametrize("frac,ns,nl", [(0.05, 4, 64), (0.0, 0, 0), (0.3, 16, 16)])
def test_decode_bf16_sums_bound(frac, ns, nl):
    # Only the estimation zone's value sums change, each by at most 2^-8 of itself (bf16 has
    # 8 significant bits): |o_bf16 - o_fp32| <= 2^-8 sum_E w_j |Vsum_j| / Z <= 2^-8 max_t |v_t|
    # per dim; the selection and the lse do not change (they do not read the values).
    K, V, ctx, idx, q = _setup_decode()
    o1, l1, i1, _ = oracle.decode(idx, K, V, q, ns, nl, frac)
    o2, l2, i2, _ = oracle.decode(idx, K, V, q, ns, nl, frac, vsum_bf16=True)
    assert np.array_equal(i1, i2) and np.array_equal(l1, l2)
    vmax = np.abs(oracle.bf16_to_f32(V).astype(np.float64)).max(0)
    assert np.all(np.abs(o2 - o1) <= 2.0 ** -8 * vmax[None, None, :] + 1e-12)
    if frac < 1.0 and not (ns == 0 and nl == 0 and frac == 0.0):
        assert np.abs(o2 - o1).max() > 0  # the rounding is visible


def test_decode_bf16_sums_exact_when_sums_are_representable():
    # values in {-1, 0, 1} and clusters of at most 256 members: every value sum is an integer
    # of magnitude <= 256, exact in bf16, so both decodes agree bit for bit
    K, V, ctx, idx, q = _setup_decode()
    rng = np.random.default_rng(5)
    Vi = oracle.f32_to_bf16(rng.integers(-1, 2, V.shape).astype(np.float32))
    idx2 = oracle.build(K, Vi, idx.G, ctx, idx.seg_len, idx.K_s, 3, 1234)
    assert idx2.sizes.max() <= 256
    for frac, ns, nl in [(0.05, 4, 64), (0.0, 0, 0)]:
        o1, l1, i1, _ = oracle.decode(idx2, K, Vi, q, ns, nl, frac)
        o2, l2, i2, _ = oracle.decode(idx2, K, Vi, q, ns, nl, frac, vsum_bf16=True)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2) and np.array_equal(i1, i2)


# ------------------------------------------------------- stochastic radix top-k
def test_sortable_key_order_and_zero():
    # an order-preserving map of floats to 32-bit keys: +0 and -0 equal, 0 never produced
    assert oracle.sortable(0.0) == oracle.sortable(-0.0) == 0x80000000
    assert oracle.sortable(1.0) == 0xBF800000 and oracle.sortable(-1.0) == 0x407FFFFF
    fmax = float(np.finfo(np.float32).max)
    assert oracle.sortable(-fmax) == 0x00800000 and oracle.sortable(fmax) == 0xFF7FFFFF
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(3000) * np.exp(rng.uniform(-80, 80, 3000))).astype(np.float32)
    x = np.concatenate([x, np.float32([1e-45, -1e-45, 0.0, 3.0, -3.0])])
    u = np.array([oracle.sortable(v) for v in x], np.uint64)
    i, j = rng.integers(0, len(x), (2, 20000))
    assert np.all((x[i] < x[j]) == (u[i] < u[j]))
    assert np.all((x[i] == x[j]) == (u[i] == u[j]))


def _exact_top(keys, k):
    return set(np.lexsort((np.arange(len(keys)), -keys.astype(np.float64)))[:k].tolist())


@pytest.mark.parametrize("passes", [1, 2, 3, 4])
def test_select_stochastic_invariants(passes):
    # exactly k distinct eligible ids in ascending order; every key whose first 8*passes bits
    # exceed those of the k-th largest key is taken, none below them is
    rng = np.random.default_rng(passes)
    for n, k in [(1000, 50), (300, 1), (64, 64), (5000, 1180), (10, 0)]:
        keys = (rng.standard_normal(n) * rng.choice([0.01, 1.0, 100.0])).astype(np.float32)
        ids = np.arange(n, dtype=np.int32) * 3
        s = oracle.select_stochastic(keys, ids, k, passes, 77 + n)
        assert len(s) == k and len(set(s.tolist())) == k and np.all(np.diff(s) > 0)
        if k == 0:
            continue
        u = np.array([oracle.sortable(v) for v in keys], np.uint64)
        sh = 32 - 8 * passes
        pk = np.sort(u)[::-1][k - 1] >> sh
        pre = u >> sh
        chosen = np.isin(ids, s)
        assert np.all(chosen[pre > pk]) and not np.any(chosen[pre < pk])


def test_select_stochastic_full_resolution_is_the_exact_top_k():
    # four passes resolve every bit: with distinct keys the set is the exact top-k
    rng = np.random.default_rng(9)
    keys = rng.standard_normal(4000).astype(np.float32)
    keys = np.unique(keys)
    rng.shuffle(keys)
    ids = np.arange(len(keys), dtype=np.int32)
    for k in (1, 37, 500, len(keys)):
        assert set(oracle.select_stochastic(keys, ids, k, 4, 5).tolist()) == _exact_top(keys, k)


def test_select_stochastic_whole_threshold_bin_is_exact():
    # the k-th and (k+1)-th keys differ in their first byte: the first pass takes its
    # threshold bin whole, and the result is the exact top-k whatever the phase
    keys = np.float32([3.0, 2.5, -1.0, -1.5, 0.25, 0.3])  # 2.5 (0xC0..) vs 0.3 (0xBE..)
    ids = np.arange(6, dtype=np.int32)
    for ph in range(20):
        assert oracle.select_stochastic(keys, ids, 2, 1, ph).tolist() == [0, 1]


def test_select_stochastic_sampling_is_uniform_over_the_bin():
    # systematic sampling with a random phase: each member of the threshold bin is taken
    # with probability m / n (here 3 of 10 members of one bin, nothing above it)
    keys = np.float32(1.0) + np.arange(10, dtype=np.float32) * np.float32(2 ** -20)  # one first-2-byte bin
    ids = np.arange(10, dtype=np.int32)
    cnt = np.zeros(10)
    T = 6000
    for t in range(T):
        s = oracle.select_stochastic(keys, ids, 3, 2, oracle.stochastic_phase_state(t, 0, 0))
        assert len(s) == 3
        cnt[s] += 1
    np.testing.assert_allclose(cnt / T, 0.3, atol=0.03)


def test_decode_stochastic_special_cases():
    K, V, ctx, idx, q = _setup_decode()
    # every eligible cluster selected: dense attention, ids ascending
    o, lse, ids, kc = oracle.decode_stochastic(idx, K, V, q, 4, 64, 1.0, 1, 3)
    of, lf = oracle.full_attention(K, V, q, idx.G, ctx)
    np.testing.assert_allclose(o, of, rtol=1e-12, atol=1e-12)
    for b in range(len(ctx)):
        for h in range(q.shape[1]):
            v = ids[b, h, :kc[b, h]]
            assert np.all(np.diff(v) > 0)
    # four passes on distinct rank keys: the exact selection's set, hence the exact output
    o1, l1, i1, k1 = oracle.decode(idx, K, V, q, 4, 64, 0.05)
    o2, l2, i2, k2 = oracle.decode_stochastic(idx, K, V, q, 4, 64, 0.05, 4, 11)
    assert np.array_equal(k1, k2)
    for b in range(len(ctx)):
        for h in range(q.shape[1]):
            assert np.array_equal(np.sort(i1[b, h, :k1[b, h]]), i2[b, h, :k2[b, h]])
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
