"""GPU parity of the bf16 value sums (variant): the build and the append write the
round-to-nearest-even bf16 of the ordered fp32 sums, bit-exact against the oracle, and the
estimation zone reads them (RetroInfer page, section 2.A: value sums per cluster stand in
for the unselected clusters; Vortex page: byte-lean index variants).

Decode bar as for the fp32 sums against the oracle's decode with the same bf16 sums: ids
bit-exact, out within 2e-3, lse within 1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3
LSE_TOL = 1e-3


def _decode_compare(idx, K, V, q, ixd, ns, nl, frac, tag):
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import say, to_dev_bf16
    say("bf16-sum decode parity %s frac=%g sink=%d local=%d" % (tag, frac, ns, nl))
    o, ids, lse = rsa.wave_attn_decode(ixd, to_dev_bf16(q), ns, nl, frac)
    torch.cuda.synchronize()
    o_ref, lse_ref, ids_ref, _ = oracle.decode(idx, K, V, q, ns, nl, frac, vsum_bf16=True)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(o.cpu().numpy() - o_ref).max() <= OUT_TOL
    assert np.abs(lse.cpu().numpy() - lse_ref).max() <= LSE_TOL
    return o


def test_build_writes_rounded_sums():
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import index_to_host, say, to_dev_bf16
    ctx = [3000, 1700]
    K, V, _ = synth.kv(41, 2, 2, np.array(ctx), 1024)
    ref = oracle.build(K, V, 2, np.array(ctx), 1024, 64, 3, 1234)
    for vs in ("both", "bf16"):
        say("build with value_sums=%s" % vs)
        ix = rsa.wave_index_build(to_dev_bf16(K), to_dev_bf16(V), 2, ctx, 1024, 64, 3, 1234, value_sums=vs)
        h = index_to_host(ix)
        assert np.array_equal(h["vsum_bf16"], oracle.value_sums_bf16(ref))
        if vs == "both":
            assert np.array_equal(h["vsum"], ref.vsum)
        else:
            assert "vsum" not in h and ix.c.vsum is None


def test_decode_small_ragged():
    from gpu_util import upload_index
    ctx = np.array([3000, 1700], np.int64)
    G, H = 2, 8
    K, V, _ = synth.kv(42, 2, G, ctx, 1024)
    idx = oracle.build(K, V, G, ctx, 1024, 64, 3, 1234)
    q, _ = synth.queries(43, 2, 2, H, G, ctx, K)
    ixb = upload_index(idx, "bf16")
    ixf = upload_index(idx, "f32")
    for frac, ns, nl in [(0.05, 4, 64), (0.0, 0, 0), (0.3, 0, 17), (1.0, 0, 0)]:
        for s in range(2):
            ob = _decode_compare(idx, K, V, q[s], ixb, ns, nl, frac, "small step %d" % s)
            # the same index with fp32 sums: only the estimation term moves, by <= 2^-8 max|v|
            import retrieval_sparse_attention_amd as rsa
            from gpu_util import to_dev_bf16
            of, _, _ = rsa.wave_attn_decode(ixf, to_dev_bf16(q[s]), ns, nl, frac)
            vmax = np.abs(oracle.bf16_to_f32(V)).max(0)
            d = np.abs(ob.cpu().numpy() - of.cpu().numpy())
            assert np.all(d <= 2.0 ** -8 * vmax[None, None, :] + 1e-5)


def test_append_writes_rounded_sums():
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import dense_from_capacity, index_to_host, to_dev_bf16
    G, seg, K_s, iters, seed, cap = 2, 1024, 64, 3, 5, 4
    K, V, _ = synth.kv(44, 1, G, np.array([3500]), seg)
    r0 = np.concatenate([np.arange(g * 3500, g * 3500 + 2500) for g in range(G)])
    r1 = np.concatenate([np.arange(g * 3500 + 2500, g * 3500 + 3500) for g in range(G)])
    ix = rsa.wave_index_build(to_dev_bf16(K[r0]), to_dev_bf16(V[r0]), G, [2500], seg, K_s, iters, seed,
                              cap_segs=cap, value_sums="bf16")
    rsa.wave_index_append(ix, to_dev_bf16(K[r1]), to_dev_bf16(V[r1]), [3500], iters, seed)
    torch.cuda.synchronize()
    h = index_to_host(ix)
    h["vsum"] = np.zeros(h["centroids"].shape, np.float32)  # not stored by this index
    got = dense_from_capacity(h, G, [3500], seg, K_s, cap)
    ref = oracle.build(K, V, G, np.array([3500]), seg, K_s, iters, seed)
    R, Cs = cap * seg, cap * K_s
    vb = np.concatenate([h["vsum_bf16"][g * Cs:g * Cs + int(ref.C[0])] for g in range(G)])
    assert np.array_equal(vb, oracle.value_sums_bf16(ref))
    assert np.array_equal(got["assign"], ref.assign)


def test_decode_1m_prescribed_clustering():
    # the 1M layer (8 kv heads, 65,536 clusters each, top 1.8%) with bf16 value sums
    from gpu_util import say, upload_index
    from test_gpu_decode import _label_assign
    G, H, seg, K_s, frac, ns, nl = 8, 32, 16384, 1024, 0.018, 4, 512
    ctx = np.array([1048576], np.int64)
    say("generating 1M")
    K, V, comp = synth.kv(3, 1, G, ctx, seg, comp=True)
    idx = oracle.index_from_assign(K, V, G, ctx, seg, K_s, 1234, _label_assign(comp, ctx, G, seg, K_s))
    q, _ = synth.queries(103, 1, 1, H, G, ctx, K)
    _decode_compare(idx, K, V, q[0], upload_index(idx, "bf16"), ns, nl, frac, "1M")


def test_tail_and_shared_read_the_rounded_sums():
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import to_dev_bf16, upload_index
    from test_oracle_pins import _split_tail
    G, H, seg, K_s = 2, 8, 1024, 64
    tail = (300, 17)
    ctx_full = np.array([3000 + tail[0], 1700 + tail[1]], np.int64)
    Kf, Vf, _ = synth.kv(45, 2, G, ctx_full, seg)
    Ki, Vi, ctx, Kt, Vt = _split_tail(Kf, Vf, ctx_full, tail, G, 300)
    idx = oracle.build(Ki, Vi, G, ctx, seg, K_s, 3, 1234)
    q, _ = synth.queries(46, 1, 2, H, G, ctx_full, Kf)
    ixb = upload_index(idx, "bf16")
    kt = to_dev_bf16(Kt)
    vt = to_dev_bf16(Vt)
    tl = torch.tensor(list(tail), dtype=torch.int32, device="cuda")
    o, ids, lse = rsa.wave_attn_decode_tail(ixb, to_dev_bf16(q[0]), 4, 64, 0.05, kt, vt, tl)
    torch.cuda.synchronize()
    o_ref, lse_ref, ids_ref, _ = oracle.decode_tail(idx, Ki, Vi, q[0], 4, 64, 0.05, Kt, Vt, tail, vsum_bf16=True)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(o.cpu().numpy() - o_ref).max() <= OUT_TOL
    o, ids, lse = rsa.wave_attn_decode_shared(ixb, to_dev_bf16(q[0]), 4, 64, 0.05)
    torch.cuda.synchronize()
    o_ref, lse_ref, ids_ref, _ = oracle.decode(idx, Ki, Vi, q[0], 4, 64, 0.05, shared=True, vsum_bf16=True)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(o.cpu().numpy() - o_ref).max() <= OUT_TOL
