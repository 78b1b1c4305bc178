"""GPU parity of the in-place index append (wave_index_append) against the oracle's build
over the longer context.

RetroInfer page, section 2.A: segments are clustered independently, so the index of a
longer context differs from the shorter one's only from the segment that held the old end
on; IceCache page: tokens produced while decoding join the indexed cache as they
accumulate. With the build's seed and rounds, an index grown by appends must equal, array
by array and bit for bit, the oracle's build over the whole longer context (the oracle
seeds each segment by its (sequence, kv head, segment) key, so the earlier segments are
the same in both). Decode over the grown index must equal decode over that oracle index.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def _prefix_rows(ctx_full, ctx, G):
    """Rows of the leading ctx[b] tokens of every block of a ragged layout over ctx_full."""
    base = np.concatenate([[0], np.cumsum(G * np.asarray(ctx_full, np.int64))])
    return np.concatenate([np.arange(base[b] + g * ctx_full[b], base[b] + g * ctx_full[b] + ctx[b])
                           for b in range(len(ctx)) for g in range(G)]).astype(np.int64)


def _span_rows(ctx_full, lo, hi, G):
    """Rows of tokens [lo[b], hi[b]) of every block (ragged over the appended counts)."""
    base = np.concatenate([[0], np.cumsum(G * np.asarray(ctx_full, np.int64))])
    parts = [np.arange(base[b] + g * ctx_full[b] + lo[b], base[b] + g * ctx_full[b] + hi[b])
             for b in range(len(lo)) for g in range(G)]
    return np.concatenate(parts).astype(np.int64) if parts else np.zeros(0, np.int64)


def _check_index(ix, K, V, G, ctx_full, ctx, seg, K_s, iters, seed, cap, tag):
    from gpu_util import dense_from_capacity, index_to_host, say
    say("append parity %s ctx=%s" % (tag, list(ctx)))
    torch.cuda.synchronize()
    got = dense_from_capacity(index_to_host(ix), G, ctx, seg, K_s, cap)
    rows = _prefix_rows(ctx_full, ctx, G)
    ref = oracle.build(K[rows], V[rows], G, np.asarray(ctx, np.int64), seg, K_s, iters, seed)
    for f in oracle.Index.FIELDS:
        a, r = got[f], getattr(ref, f)
        assert a.shape == r.shape and np.array_equal(a, r), "%s: %s differs" % (tag, f)
    return ref


def _grow(G, ctx_steps, seg, K_s, iters, seed, cap, data_seed, decode_check=False):
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import to_dev_bf16, say
    ctx_full = np.asarray(ctx_steps[-1], np.int64)
    K, V, _ = synth.kv(data_seed, len(ctx_full), G, ctx_full, seg)
    c0 = [int(n) for n in ctx_steps[0]]
    rows = _prefix_rows(ctx_full, c0, G)
    ix = rsa.wave_index_build(to_dev_bf16(K[rows]), to_dev_bf16(V[rows]), G, c0, seg, K_s, iters, seed, cap_segs=cap)
    ref = _check_index(ix, K, V, G, ctx_full, c0, seg, K_s, iters, seed, cap, "build")
    prev = c0
    for step, c in enumerate(ctx_steps[1:]):
        c = [int(n) for n in c]
        ar = _span_rows(ctx_full, prev, c, G)
        kn, vn = to_dev_bf16(K[ar]), to_dev_bf16(V[ar])
        rsa.wave_index_append(ix, kn, vn, c, iters, seed)
        ref = _check_index(ix, K, V, G, ctx_full, c, seg, K_s, iters, seed, cap, "step %d" % step)
        assert ix.ctx == c
        prev = c
        if decode_check:
            from gpu_util import upload_index
            H = 4 * G
            q, _ = synth.queries(data_seed + 1 + step, 1, len(c), H, G, np.asarray(c, np.int64), K[_prefix_rows(ctx_full, c, G)])
            qd = to_dev_bf16(q[0])
            say("  decode over the grown index and over the oracle's")
            o1, i1, l1 = rsa.wave_attn_decode(ix, qd, 4, 64, 0.05)
            o2, i2, l2 = rsa.wave_attn_decode(upload_index(ref), qd, 4, 64, 0.05)
            torch.cuda.synchronize()
            assert torch.equal(i1, i2) and torch.equal(o1, o2) and torch.equal(l1, l2)
            rows_c = _prefix_rows(ctx_full, c, G)
            o_ref, lse_ref, ids_ref, _ = oracle.decode(ref, K[rows_c], V[rows_c], q[0], 4, 64, 0.05)
            assert np.array_equal(i1.cpu().numpy(), ids_ref)
            assert np.abs(o1.cpu().numpy() - o_ref).max() <= 2e-3
            assert np.abs(l1.cpu().numpy() - lse_ref).max() <= 1e-3
    return ix


def test_capacity_build_equals_dense_build():
    # the capacity layout only moves each block; a build into it equals the dense one
    _grow(2, [[2500, 1700]], 1024, 64, 3, 1234, 3, 31)


def test_append_ragged_partial_and_full_segments():
    # b0: partial -> partial, exactly full, then +1 segment; b1: full -> new partial, ...;
    # b2: untouched, then one token, then several segments at once
    steps = [[2500, 1024, 3000], [3000, 2100, 3000], [3072, 2100, 3001], [4096, 3500, 5000]]
    _grow(2, steps, 1024, 64, 3, 1234, 5, 32, decode_check=True)


def test_append_one_token_at_a_time_across_a_boundary():
    steps = [[1022], [1023], [1024], [1025], [1026]]
    _grow(3, steps, 1024, 37, 2, 7, 2, 33)


def test_append_more_than_512_clusters_per_segment():
    # K_s > 512: the assignment takes the centroids in groups (running bests in LDS)
    _grow(1, [[3000], [5000], [6144]], 2048, 1024, 2, 5, 3, 34)


def test_append_long_segments_counting_sort():
    # segments above 16384 tokens take the counting sort with its per-row rank workspace
    _grow(1, [[25000], [41000]], 20000, 100, 2, 9, 3, 35)


def test_append_of_nothing_keeps_the_index():
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import index_to_host, to_dev_bf16
    K, V, _ = synth.kv(36, 1, 2, np.array([1500]), 1024)
    ix = rsa.wave_index_build(to_dev_bf16(K), to_dev_bf16(V), 2, [1500], 1024, 64, 2, 3, cap_segs=2)
    before = index_to_host(ix)
    e = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    rsa.wave_index_append(ix, e, e, [1500], 2, 3)
    after = index_to_host(ix)
    for f in before:
        assert np.array_equal(before[f], after[f]), f


def test_append_rejects_beyond_capacity_and_shrinking():
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import to_dev_bf16
    K, V, _ = synth.kv(37, 1, 1, np.array([1500]), 1024)
    ix = rsa.wave_index_build(to_dev_bf16(K), to_dev_bf16(V), 1, [1500], 1024, 64, 2, 3, cap_segs=2)
    kn = torch.zeros((600, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rsa.WaveError, match="capacity"):
        rsa.wave_index_append(ix, kn, kn, [2100], 2, 3)
    with pytest.raises(ValueError, match="shorter"):
        rsa.wave_index_append(ix, kn[:0], kn[:0], [1400], 2, 3)
    assert ix.ctx == [1500]


def test_append_128k_one_segment():
    # the 128K layer (8 kv heads, 16 segments of 8192 tokens, 512 clusters each) grows by one
    # segment: the 8 new units equal the oracle's k-means of their segments under their keys,
    # the earlier segments stay bit-identical, and the layout of every block is whole
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import dense_from_capacity, index_to_host, say, to_dev_bf16
    G, seg, K_s, iters, seed, cap = 8, 8192, 512, 10, 1234, 17
    N0, N1 = 131072, 131072 + 8192
    say("generating 128K + one segment")
    K, V, _ = synth.kv(3, 1, G, np.array([N1]), seg)
    rows0 = _prefix_rows([N1], [N0], G)
    ix = rsa.wave_index_build(to_dev_bf16(K[rows0]), to_dev_bf16(V[rows0]), G, [N0], seg, K_s, iters, seed,
                              cap_segs=cap)
    torch.cuda.synchronize()
    before = dense_from_capacity(index_to_host(ix), G, [N0], seg, K_s, cap)
    ar = _span_rows([N1], [N0], [N1], G)
    rsa.wave_index_append(ix, to_dev_bf16(K[ar]), to_dev_bf16(V[ar]), [N1], iters, seed)
    torch.cuda.synchronize()
    got = dense_from_capacity(index_to_host(ix), G, [N1], seg, K_s, cap)
    C0, C1 = N0 // seg * K_s, N1 // seg * K_s
    for g in range(G):
        say("  kv head %d" % g)
        r0, r1 = g * N1, g * N1 + N0
        o0, o1 = g * N0, (g + 1) * N0
        for f in ("assign", "perm", "inv_perm", "k_sorted", "v_sorted"):
            assert np.array_equal(got[f][r0:r1], before[f][o0:o1]), (f, g)
        for f in ("sizes", "centroids", "centroids_bf16", "vsum"):
            assert np.array_equal(got[f][g * C1:g * C1 + C0], before[f][g * C0:(g + 1) * C0]), (f, g)
        offs = got["offsets"][g * (C1 + 1):(g + 1) * (C1 + 1)]
        assert np.array_equal(offs[:C0 + 1], before["offsets"][g * (C0 + 1):(g + 1) * (C0 + 1)])
        a = got["assign"][g * N1:(g + 1) * N1]
        assert np.array_equal(np.diff(offs), got["sizes"][g * C1:(g + 1) * C1]) and offs[-1] == N1
        assert np.array_equal(np.sort(got["perm"][g * N1 + N0:(g + 1) * N1]), np.arange(N0, N1))
    # two of the new units against the oracle's k-means of their segment
    for g in (0, G - 1):
        say("  new unit of kv head %d against the oracle" % g)
        r = g * N1 + N0
        a_ref, c_ref, _, _ = oracle.kmeans_segment(K[r:r + seg], K_s, iters, seed, key=oracle.seed_key(0, g, N0 // seg))
        assert np.array_equal(got["assign"][r:r + seg], a_ref + C0)
        assert np.array_equal(got["centroids"][g * C1 + C0:(g + 1) * C1], c_ref)
