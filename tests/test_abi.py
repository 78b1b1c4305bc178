"""The C ABI on the CPU: the library loads, exports every declared entry point, sizes its
arrays, and rejects bad arguments before touching a device (no GPU needed)."""
import ctypes
import math
import os
import re

import pytest

import oracle
import retrieval_sparse_attention_amd as rsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, ARG, SHAPE, UNSUP, WS, ALIGN, HIP = 0, -1, -2, -3, -4, -5, -6


def _declared():
    text = open(os.path.join(ROOT, "include", "wave_attn.h")).read()
    return sorted(set(re.findall(r"^(?:wave_status|const char\*|int32_t)\s+(wave_\w+)\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert {"wave_index_plan", "wave_index_build", "wave_attn_decode_plan", "wave_attn_decode",
            "wave_last_error", "wave_attn_decode_shared", "wave_attn_decode_tail"} <= set(names)
    L = rsa.lib()
    for n in names:
        assert hasattr(L, n), n


def _shape(G, ctx, head_dim=128):
    arr = (ctypes.c_int64 * len(ctx))(*ctx)
    return rsa._Shape(len(ctx), G, head_dim, 0, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64))), arr


def _plan(G, ctx, L, K, head_dim=128):
    sh, keep = _shape(G, ctx, head_dim)
    z = rsa._Sizes()
    return rsa.lib().wave_index_plan(ctypes.byref(sh), L, K, ctypes.byref(z)), z


def test_index_plan_sizes():
    for G, ctx, L, K in [(8, [131072], 8192, 512), (8, [1048576], 16384, 1024), (2, [16384], 8192, 512),
                         (3, [70000, 8192 * 2 + 5, 1], 8192, 512)]:
        st, z = _plan(G, ctx, L, K)
        assert st == OK
        C = [oracle.num_clusters(n, L, K) for n in ctx]
        assert z.rows == G * sum(ctx)
        assert z.clusters == G * sum(C)
        assert z.offsets_len == G * sum(c + 1 for c in C)
        assert z.units == G * sum(-(-n // L) for n in ctx)
        assert z.max_clusters == max(C)
        assert z.build_ws_bytes >= 4 * (z.clusters + z.rows)  # squared norms, sort ranks


@pytest.mark.parametrize("args,status", [
    ((8, [1000], 256, 16, 64), UNSUP),     # head_dim 64
    ((8, [1000], 256, 300), SHAPE),        # K_s > L_s
    ((8, [1000], 0, 1), SHAPE),
    ((8, [1000], 256, 0), SHAPE),
    ((0, [1000], 256, 16), SHAPE),
    ((8, [0], 256, 16), SHAPE),
    ((8, [1000], 65537, 16), UNSUP),
    ((8, [1000], 4096, 4096), UNSUP),     # K_s above the per-segment limit
    ((8, [1 << 31], 4096, 16), UNSUP),
])
def test_index_plan_rejects(args, status):
    st, _ = _plan(*args)
    assert st == status
    assert rsa.lib().wave_last_error().decode() != ""


def test_index_plan_batch_limits():
    st, _ = _plan(1, [10] * 257, 8, 2)
    assert st == UNSUP
    sh = rsa._Shape(1, 1, 128, 0, None)
    z = rsa._Sizes()
    assert rsa.lib().wave_index_plan(ctypes.byref(sh), 8, 2, ctypes.byref(z)) == ARG


def _fake_index(G, ctx, L, K):
    sh, keep = _shape(G, ctx)
    ix = rsa._Index()
    ix.shape = sh
    ix.seg_len, ix.clusters_per_seg = L, K
    for i, f in enumerate(("k_sorted", "v_sorted", "perm", "inv_perm", "assign", "offsets", "sizes",
                           "centroids", "centroids_bf16", "vsum")):
        setattr(ix, f, 0x10000 * (i + 1))  # aligned, never dereferenced on the CPU
    return ix, keep


def _dplan(ix, H, ns, nl, frac):
    k = ctypes.c_int32()
    w = ctypes.c_size_t()
    st = rsa.lib().wave_attn_decode_plan(ctypes.byref(ix), H, ns, nl, frac, ctypes.byref(k), ctypes.byref(w))
    return st, k.value, w.value


@pytest.mark.parametrize("G,H,N,L,K,frac,kmax", [(2, 8, 16384, 8192, 512, 0.05, 52), (8, 32, 131072, 8192, 512, 0.02, 164),
                                              (8, 32, 1048576, 16384, 1024, 0.018, 1180),
                                              (8, 32, 131072, 8192, 512, 0.0, 0), (8, 32, 131072, 8192, 512, 1.0, 8192)])
def test_decode_plan_k_max(G, H, N, L, K, frac, kmax):
    ix, keep = _fake_index(G, [N], L, K)
    st, k, w = _dplan(ix, H, 4, 64, frac)
    assert st == OK and k == kmax and k == oracle.k_from_frac(frac, oracle.num_clusters(N, L, K))
    assert w > 4 * H * oracle.num_clusters(N, L, K)


@pytest.mark.parametrize("H,ns,nl,frac,status", [
    (30, 4, 64, 0.02, SHAPE),        # 30 % 8
    (0, 4, 64, 0.02, SHAPE),
    (80, 4, 64, 0.02, UNSUP),        # 10 q heads per kv head
    (32, -1, 64, 0.02, ARG),
    (32, 4, -5, 0.02, ARG),
    (32, 4, 64, float("nan"), ARG),
    (32, 4, 64, 1.5, ARG),
    (32, 4, 64, -0.1, ARG),
    (32, 3000, 3000, 0.02, UNSUP),   # 6000 steady tokens, not the whole sequence
])
def test_decode_plan_rejects(H, ns, nl, frac, status):
    ix, keep = _fake_index(8, [131072], 8192, 512)
    st, _, _ = _dplan(ix, H, ns, nl, frac)
    assert st == status


def test_decode_plan_all_steady_is_supported():
    ix, keep = _fake_index(8, [5000], 1024, 64)
    st, k, w = _dplan(ix, 32, 2500, 2500, 0.1)
    assert st == OK


def test_calls_fail_cleanly_without_device():
    if os.path.exists("/dev/kfd"):
        pytest.skip("a GPU is present")
    L = rsa.lib()
    sh, keep = _shape(2, [4096])
    ix, keep2 = _fake_index(2, [4096], 1024, 64)
    st, z = _plan(2, [4096], 1024, 64)
    args = [ctypes.byref(sh), ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), 1024, 64, 2, ctypes.c_uint64(1),
            ctypes.byref(ix), ctypes.c_void_p(0x3000), z.build_ws_bytes, None, None]
    assert L.wave_index_build(*args) == HIP
    # argument errors win over the missing device and nothing is touched
    bad = list(args)
    bad[1] = None
    assert L.wave_index_build(*bad) == ARG
    bad = list(args)
    bad[1] = ctypes.c_void_p(0x1001)
    assert L.wave_index_build(*bad) == ALIGN
    bad = list(args)
    bad[9] = z.build_ws_bytes - 1
    assert L.wave_index_build(*bad) == WS
    bad = list(args)
    bad[5] = 0
    assert L.wave_index_build(*bad) == SHAPE
    st, k, w = _dplan(ix, 8, 4, 64, 0.05)
    dargs = [ctypes.byref(ix), ctypes.c_void_p(0x4000), 8, 4, 64, 0.05, ctypes.c_void_p(0x5000),
             ctypes.c_void_p(0x6000), None, ctypes.c_void_p(0x7000), w, None]
    assert L.wave_attn_decode(*dargs) == HIP
    bad = list(dargs)
    bad[10] = w - 1
    assert L.wave_attn_decode(*bad) == WS
    bad = list(dargs)
    bad[7] = None
    assert L.wave_attn_decode(*bad) == ARG
    bad = list(dargs)
    bad[1] = ctypes.c_void_p(0x4008)
    assert L.wave_attn_decode(*bad) == ALIGN
    # the block baseline's entry points check the same way
    bargs = [ctypes.byref(sh), ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), 1024, 64, ctypes.byref(ix),
             ctypes.c_void_p(0x3000), z.build_ws_bytes, None]
    assert L.wave_index_build_blocks(*bargs) == HIP
    bad = list(bargs)
    bad[2] = None
    assert L.wave_index_build_blocks(*bad) == ARG
    bad = list(bargs)
    bad[6] = ctypes.c_void_p(0x3004)
    assert L.wave_index_build_blocks(*bad) == ALIGN
    bad = list(bargs)
    bad[7] = z.build_ws_bytes - 1
    assert L.wave_index_build_blocks(*bad) == WS
    bad = list(bargs)
    bad[4] = 2048
    assert L.wave_index_build_blocks(*bad) == SHAPE
    assert L.wave_attn_decode_topk(*dargs) == HIP
    bad = list(dargs)
    bad[10] = w - 1
    assert L.wave_attn_decode_topk(*bad) == WS
    bad = list(dargs)
    bad[6] = None
    assert L.wave_attn_decode_topk(*bad) == ARG
    k2 = ctypes.c_int32()
    w2 = ctypes.c_size_t()
    assert L.wave_attn_decode_tail_plan(ctypes.byref(ix), 8, 4, 64, 0.05, 512, ctypes.byref(k2), ctypes.byref(w2)) == OK
    assert k2.value == k and w2.value >= w  # the tail's rows may take more row workgroups
    assert L.wave_attn_decode_tail_plan(ctypes.byref(ix), 8, 4, 64, 0.05, 0, ctypes.byref(k2), ctypes.byref(w2)) == ARG
    targs = [ctypes.byref(ix), ctypes.c_void_p(0x4000), 8, 4, 64, 0.05, ctypes.c_void_p(0x8000),
             ctypes.c_void_p(0x9000), 512, ctypes.c_void_p(0xA000), ctypes.c_void_p(0x5000), ctypes.c_void_p(0x6000),
             None, ctypes.c_void_p(0x7000), w2.value, None]
    assert L.wave_attn_decode_tail(*targs) == HIP
    bad = list(targs)
    bad[6] = None
    assert L.wave_attn_decode_tail(*bad) == ARG
    bad = list(targs)
    bad[7] = ctypes.c_void_p(0x9004)
    assert L.wave_attn_decode_tail(*bad) == ALIGN
    bad = list(targs)
    bad[8] = 65537
    assert L.wave_attn_decode_tail(*bad) == ARG
    bad = list(targs)
    bad[14] = w2.value - 1
    assert L.wave_attn_decode_tail(*bad) == WS
    assert L.wave_attn_decode_shared(*dargs) == HIP
    bad = list(dargs)
    bad[10] = w - 1
    assert L.wave_attn_decode_shared(*bad) == WS
    bad = list(dargs)
    bad[2] = 7  # not a multiple of the 2 kv heads
    assert L.wave_attn_decode_shared(*bad) == SHAPE


def _plan_cap(G, ctx, L, K, cap):
    sh, keep = _shape(G, ctx)
    z = rsa._Sizes()
    return rsa.lib().wave_index_plan_cap(ctypes.byref(sh), L, K, cap, ctypes.byref(z)), z


def test_capacity_plan_sizes():
    # every (b, g) block holds cap segments of room; the build reads the dense K and V
    for G, ctx, L, K, cap in [(8, [131072], 8192, 512, 17), (3, [70000, 16389, 1], 8192, 512, 9), (2, [5], 4, 3, 2)]:
        st, z = _plan_cap(G, ctx, L, K, cap)
        assert st == OK
        B = len(ctx)
        assert z.rows == B * G * cap * L
        assert z.clusters == B * G * cap * K
        assert z.offsets_len == B * G * (cap * K + 1)
        assert z.kv_rows == G * sum(ctx)
        assert z.cap_segs == cap
        assert z.units == G * sum(-(-n // L) for n in ctx)
        assert z.build_ws_bytes >= 4 * z.clusters + 8 * z.kv_rows
        st0, z0 = _plan_cap(G, ctx, L, K, 0)  # cap 0: the dense plan
        st1, z1 = _plan(G, ctx, L, K)
        assert st0 == st1 == OK and (z0.rows, z0.clusters, z0.kv_rows) == (z1.rows, z1.clusters, z1.rows)


@pytest.mark.parametrize("cap,status", [(-1, ARG), (1, SHAPE), (1 << 20, UNSUP)])
def test_capacity_plan_rejects(cap, status):
    st, _ = _plan_cap(2, [3000], 2048, 64, cap)
    assert st == status


def _append_plan(ix, new_ctx):
    arr = (ctypes.c_int64 * len(new_ctx))(*new_ctx)
    n = ctypes.c_size_t()
    return rsa.lib().wave_index_append_plan(ctypes.byref(ix), arr, ctypes.byref(n)), n.value


def test_append_plan_sizes_and_rejects():
    ix, keep = _fake_index(2, [2500, 1024], 1024, 64)
    assert _append_plan(ix, [2600, 1024])[0] == ARG  # a dense index cannot grow
    ix.cap_segs = 4
    st, w = _append_plan(ix, [3000, 2100])
    assert st == OK
    # input rows: b0 from token 2048 (segment 2 held the old end), b1 from 1024, both kv heads
    rows = 2 * (3000 - 2048) + 2 * (2100 - 1024)
    assert w >= 4 * 2 * 2 * 4 * 64 + 8 * rows + 2 * 2 * 128 * rows
    assert _append_plan(ix, [2400, 1024])[0] == SHAPE   # shorter
    assert _append_plan(ix, [4097, 1024])[0] == SHAPE   # beyond 4 segments of 1024
    st, w0 = _append_plan(ix, [2500, 1024])              # nothing appended
    assert st == OK


def test_append_fails_cleanly_without_device():
    if os.path.exists("/dev/kfd"):
        pytest.skip("a GPU is present")
    L = rsa.lib()
    ix, keep = _fake_index(2, [2500], 1024, 64)
    ix.cap_segs = 4
    new = (ctypes.c_int64 * 1)(3000)
    st, w = _append_plan(ix, [3000])
    args = [ctypes.byref(ix), new, ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), 2, ctypes.c_uint64(1),
            ctypes.c_void_p(0x3000), w, None]
    assert L.wave_index_append(*args) == HIP
    assert ix.shape.ctx[0] == 2500  # unchanged on an error
    bad = list(args)
    bad[2] = None
    assert L.wave_index_append(*bad) == ARG
    bad = list(args)
    bad[3] = ctypes.c_void_p(0x2008)
    assert L.wave_index_append(*bad) == ALIGN
    bad = list(args)
    bad[7] = w - 1
    assert L.wave_index_append(*bad) == WS
    bad = list(args)
    bad[4] = 0
    assert L.wave_index_append(*bad) == ARG
    # nothing appended: no device work, the index takes the new (equal) contexts
    same = (ctypes.c_int64 * 1)(2500)
    assert L.wave_index_append(ctypes.byref(ix), same, None, None, 2, ctypes.c_uint64(1), None, 0, None) == OK
    assert ctypes.addressof(ix.shape.ctx.contents) == ctypes.addressof(same)


def test_struct_layout_matches_the_header(tmp_path):
    # the binding's ctypes mirrors have the C structs' sizes and field offsets
    src = tmp_path / "layout.c"
    fields = {"wave_shape": rsa._Shape, "wave_index_sizes": rsa._Sizes, "wave_index": rsa._Index}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "wave_attn.h"', "int main(void) {"]
    for cname, py in fields.items():
        lines.append('printf("%s %%zu\\n", sizeof(%s));' % (cname, cname))
        for f, _ in py._fields_:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (cname, f, cname, f))
    lines.append("return 0; }")
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    import subprocess
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = dict(l.split() for l in subprocess.check_output([str(exe)]).decode().split("\n") if l)
    for cname, py in fields.items():
        assert int(got[cname]) == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert int(got["%s.%s" % (cname, f)]) == getattr(py, f).offset, (cname, f)
