"""GPU parity of the decode over an index plus the tokens appended after its build
(wave_attn_decode_tail) against the oracle's ref_decode_tail.

Bar as for the decode: selected ids bit-exact, out within 2e-3 max-abs, lse within 1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from test_oracle_pins import _split_tail

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3
LSE_TOL = 1e-3


def _run(ixd, q, ns, nl, frac, Kt, Vt, tl):
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import to_dev_bf16
    kt = torch.from_numpy(Kt.view(np.int16)).cuda().view(torch.bfloat16)
    vt = torch.from_numpy(Vt.view(np.int16)).cuda().view(torch.bfloat16)
    tld = torch.tensor(np.asarray(tl, np.int32), device="cuda")
    o, ids, lse = rsa.wave_attn_decode_tail(ixd, to_dev_bf16(q), ns, nl, frac, kt, vt, tld)
    torch.cuda.synchronize()
    return o.cpu().numpy(), ids.cpu().numpy(), lse.cpu().numpy()


def _compare(idx, Ki, Vi, q, ixd, ns, nl, frac, Kt, Vt, tl, tag, tl_dev=None):
    from gpu_util import say
    say("tail decode parity %s frac=%g sink=%d local=%d tails=%s" % (tag, frac, ns, nl, list(tl)))
    o, ids, lse = _run(ixd, q, ns, nl, frac, Kt, Vt, tl if tl_dev is None else tl_dev)
    o_ref, lse_ref, ids_ref, _ = oracle.decode_tail(idx, Ki, Vi, q, ns, nl, frac, Kt, Vt, tl)
    assert np.array_equal(ids, ids_ref), "ids differ at %s" % (np.argwhere(ids != ids_ref)[:5],)
    err = np.abs(o - o_ref).max()
    assert err <= OUT_TOL, err
    assert np.abs(lse - lse_ref).max() <= LSE_TOL


@pytest.fixture(scope="module")
def small():
    from gpu_util import upload_index
    G, H, seg, K_s, cap = 2, 8, 1024, 64, 300
    tail = (300, 17)
    ctx_full = np.array([3000 + tail[0], 1700 + tail[1]], np.int64)
    Kf, Vf, _ = synth.kv(71, 2, G, ctx_full, seg)
    Ki, Vi, ctx, Kt, Vt = _split_tail(Kf, Vf, ctx_full, tail, G, cap)
    idx = oracle.build(Ki, Vi, G, ctx, seg, K_s, 3, 1234)
    q, _ = synth.queries(72, 2, 2, H, G, ctx_full, Kf)
    return idx, Ki, Vi, Kt, Vt, q, upload_index(idx)


@pytest.mark.parametrize("frac,ns,nl,tl", [(0.05, 4, 64, (300, 17)), (0.05, 4, 64, (0, 0)), (0.3, 0, 0, (1, 300)),
                                           (1.0, 0, 0, (300, 17)), (0.0, 4, 64, (123, 0)),
                                           (0.1, 1500, 1500, (300, 17))])
def test_tail_small_ragged(small, frac, ns, nl, tl):
    idx, Ki, Vi, Kt, Vt, q, ixd = small
    for s in range(q.shape[0]):
        _compare(idx, Ki, Vi, q[s], ixd, ns, nl, frac, Kt, Vt, tl, "small step %d" % s)


def test_tail_lengths_are_clamped(small):
    # device lengths outside [0, cap] read as 0 and cap
    idx, Ki, Vi, Kt, Vt, q, ixd = small
    _compare(idx, Ki, Vi, q[0], ixd, 4, 64, 0.05, Kt, Vt, (300, 0), "clamped", tl_dev=(1000, -5))


def test_tail_128k():
    # the 128K layer (prescribed clustering) with half a segment of decoded tokens
    from gpu_util import say, upload_index
    from test_gpu_decode import _label_assign
    G, H, seg, K_s, T = 8, 32, 8192, 512, 4096
    ctx_full = np.array([131072 + T], np.int64)
    say("generating 128K + tail")
    Kf, Vf, comp = synth.kv(3, 1, G, ctx_full, seg, comp=True)
    Ki, Vi, ctx, Kt, Vt = _split_tail(Kf, Vf, ctx_full, (T,), G, T)
    ci = np.concatenate([comp[g * int(ctx_full[0]): g * int(ctx_full[0]) + int(ctx[0])] for g in range(G)])
    idx = oracle.index_from_assign(Ki, Vi, G, ctx, seg, K_s, 1234, _label_assign(ci, ctx, G, seg, K_s))
    q, _ = synth.queries(103, 1, 1, H, G, ctx_full, Kf)
    _compare(idx, Ki, Vi, q[0], upload_index(idx), 4, 64, 0.02, Kt, Vt, (T,), "128K")


def test_decode_loop_with_growing_context():
    # A decode loop on the GPU: tokens join the tail after the index; when the tail holds
    # a full segment, that segment is appended to the index in place (wave_index_append:
    # segments are clustered independently) and the tail starts again. Every step is
    # checked against the oracle's decode over its build of the indexed prefix.
    import retrieval_sparse_attention_amd as rsa
    from gpu_util import say, to_dev_bf16
    G, H, seg, K_s, iters, seed = 2, 8, 1024, 64, 3, 99
    N0, cap, total = 2048, 1024, 2048 + 2 * 1024 + 300
    Kf, Vf, _ = synth.kv(81, 1, G, np.array([total], np.int64), seg)
    q, _ = synth.queries(82, 1, 1, H, G, np.array([total], np.int64), Kf)

    def rows_of(lo, hi):
        return np.concatenate([np.arange(g * total + lo, g * total + hi) for g in range(G)])

    ixd = rsa.wave_index_build(to_dev_bf16(Kf[rows_of(0, N0)]), to_dev_bf16(Vf[rows_of(0, N0)]), G, [N0], seg, K_s,
                               iters, seed, cap_segs=total // seg + 1)
    n_idx = N0
    for n_now in (N0, N0 + 1, N0 + 517, N0 + cap, N0 + cap + 1, N0 + 2 * cap, N0 + 2 * cap + 300):
        if n_now - n_idx >= cap:  # a full segment waits: append it to the index
            r = rows_of(n_idx, n_idx + cap)
            rsa.wave_index_append(ixd, to_dev_bf16(Kf[r]), to_dev_bf16(Vf[r]), [n_idx + cap], iters, seed)
            n_idx += cap
        say("growing context: %d tokens, %d indexed" % (n_now, n_idx))
        Kn, Vn = Kf[rows_of(0, n_now)], Vf[rows_of(0, n_now)]
        Ki, Vi, ctx, Kt, Vt = _split_tail(Kn, Vn, np.array([n_now], np.int64), (n_now - n_idx,), G, cap)
        idx = oracle.build(Ki, Vi, G, ctx, seg, K_s, iters, seed)
        _compare(idx, Ki, Vi, q[0], ixd, 4, 64, 0.05, Kt, Vt, (n_now - n_idx,), "growing %d" % n_now)
