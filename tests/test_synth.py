"""The seeded input generator: deterministic, right shapes and the stated distributions."""
import numpy as np

import synth


def test_deterministic_and_ragged_layout():
    ctx = np.array([300, 129], np.int64)
    K1, V1, c1 = synth.kv(5, 2, 3, ctx, 64, comp=True)
    K2, V2, c2 = synth.kv(5, 2, 3, ctx, 64, comp=True)
    assert K1.shape == (3 * 429, 128) and V1.shape == K1.shape and c1.shape == (3 * 429,)
    assert np.array_equal(K1, K2) and np.array_equal(V1, V2) and np.array_equal(c1, c2)
    K3, _, _ = synth.kv(6, 2, 3, ctx, 64)
    assert not np.array_equal(K1, K3)
    # per-block streams: a longer context leaves the shared prefix of block (0, 0) unchanged
    K4, _, _ = synth.kv(5, 1, 1, np.array([500]), 64)
    assert np.array_equal(K4[:300], K1[:300])


def test_distributions():
    z = synth.normals(1, 400000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    t = synth.student4(1, 400000)
    assert abs(t.mean()) < 0.02 and abs(t.var() - 2.0) < 0.15  # Student-t(4): variance 4/(4-2)
    ctx = np.array([8192], np.int64)
    K, V, comp = synth.kv(2, 1, 1, ctx, 8192, comp=True)
    Kf, Vf = synth.bf16_bits_to_f32(K), synth.bf16_bits_to_f32(V)
    # centres N(0,1) plus noise sd 0.3: per-dim variance ~1.09; tokens of one component
    # lie within sd ~0.3 of each other
    assert abs(Kf.var() - 1.09) < 0.1 and abs(Vf.var() - 1.09) < 0.1
    m = np.bincount(comp).argmax()
    grp = Kf[comp == m]
    assert abs(grp.std(0).mean() - 0.3) < 0.05
    assert comp.min() >= 0 and comp.max() < 1024


def test_queries_near_a_key():
    ctx = np.array([1000, 2000], np.int64)
    K, _, _ = synth.kv(3, 2, 2, ctx, 512, values=False)
    q, ts = synth.queries(7, 3, 2, 8, 2, ctx, K)
    assert q.shape == (3, 2, 8, 128) and ts.shape == (3, 2, 8)
    row0 = [0, 2 * 1000]
    for st in range(3):
        for b in range(2):
            for h in range(8):
                g = h * 2 // 8
                t = ts[st, b, h]
                assert 0 <= t < ctx[b]
                k = synth.bf16_bits_to_f32(K[row0[b] + g * ctx[b] + t])
                d = synth.bf16_bits_to_f32(q[st, b, h]) - k
                assert 0.3 < d.std() < 0.7  # noise sd 0.5


def test_ctx_lengths_range():
    n = synth.ctx_lengths(4, 1000, 65536, 131072)
    assert n.min() >= 65536 and n.max() <= 131072 and n.std() > 10000
