"""CPU oracle of wave-index sparse decode attention (ctypes front of liboracle.so).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline
leg use it.  The GPU library never imports it, and the two share no code.

The arithmetic lives in oracle.c (plain C, binary64 except the steps defined in
fp32/bf16).  This module only marshals numpy arrays.  Method: RetroInfer page,
section 2.A (steady, retrieval and estimation zones over a segmented-clustered
KV cache).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
D = 128


def compile_lib():
    """Compile liboracle.so (gcc, OpenMP over independent units, no fused or fast math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-ffp-contract=off",
           "-fno-fast-math", "-o", _LIB_PATH, os.path.join(_HERE, "oracle.c"), "-lm"]
    subprocess.check_call(cmd)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            compile_lib()
        lib = ctypes.CDLL(_LIB_PATH)
        P, i32, i64, u64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
        lib.ref_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.ref_bf16_to_f32.restype = ctypes.c_float
        lib.ref_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.ref_f32_to_bf16.restype = ctypes.c_uint16
        lib.ref_f32_to_bf16_array.argtypes = [P, i64, P]
        lib.ref_splitmix64_stream.argtypes = [u64, i64, P]
        lib.ref_seed_key.argtypes = [i32, i32, i64]
        lib.ref_seed_key.restype = u64
        lib.ref_init_indices.argtypes = [i32, i32, u64, u64, P]
        lib.ref_segment_clusters.argtypes = [i64, i32, i32]
        lib.ref_segment_clusters.restype = i64
        lib.ref_num_clusters.argtypes = [i64, i32, i32]
        lib.ref_num_clusters.restype = i64
        lib.ref_k_from_frac.argtypes = [f64, i64]
        lib.ref_k_from_frac.restype = i64
        lib.ref_sq_dist.argtypes = [P, P]
        lib.ref_sq_dist.restype = f64
        lib.ref_assign_point.argtypes = [P, P, i32]
        lib.ref_assign_point.restype = i32
        lib.ref_kmeans_segment.argtypes = [P, i32, i32, i32, u64, u64, i32, P, P, P, P]
        lib.ref_build.argtypes = [i32, i32, P, P, P, i32, i32, i32, u64] + [P] * 11
        lib.ref_build.restype = ctypes.c_int
        lib.ref_index_from_assign.argtypes = [i32, i32, P, P, P, i32, i32, u64, P] + [P] * 10
        lib.ref_index_from_assign.restype = ctypes.c_int
        lib.ref_sortable.argtypes = [ctypes.c_float]
        lib.ref_sortable.restype = ctypes.c_uint32
        lib.ref_select_stochastic.argtypes = [P, P, i32, i32, i32, u64, P]
        lib.ref_decode_stochastic.argtypes = [i32, i32, i32, P, i32, i32, P, P, P, P, P, P, i32, i32, f64, i32, u64,
                                              i32, P, P, P, P]
        lib.ref_decode_stochastic.restype = ctypes.c_int
        lib.ref_rank_key.argtypes = [P, P]
        lib.ref_rank_key.restype = ctypes.c_float
        lib.ref_select.argtypes = [P, P, i32, i32, P]
        lib.ref_decode.argtypes = [i32, i32, i32, P, i32, i32, P, P, P, P, P, P, i32, i32, f64, i32, P, P, P, P]
        lib.ref_decode.restype = ctypes.c_int
        lib.ref_decode_shared.argtypes = lib.ref_decode.argtypes
        lib.ref_decode_tail.argtypes = [i32, i32, i32, P, i32, i32, P, P, P, P, P, P, i32, i32, f64, P, P, i32, P,
                                        i32, P, P, P, P]
        lib.ref_decode_tail.restype = ctypes.c_int
        lib.ref_decode_shared.restype = ctypes.c_int
        lib.ref_decode_topk.argtypes = [i32, i32, i32, P, i32, i32, P, P, P, P, P, i32, i32, f64, i32, P, P, P, P]
        lib.ref_decode_topk.restype = ctypes.c_int
        lib.ref_block_assign.argtypes = [i32, i32, P, i32, i32, P]
        lib.ref_full_attention.argtypes = [i32, i32, i32, P, P, P, P, P, P]
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ---------------------------------------------------------------- format / rng
def f32_to_bf16(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().ref_f32_to_bf16_array(_p(x), x.size, _p(out))
    return out


def bf16_to_f32(h):
    return (_c(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def splitmix64_stream(state, n):
    out = np.empty(n, dtype=np.uint64)
    _load().ref_splitmix64_stream(state, n, _p(out))
    return out


def seed_key(b, g, s):
    """Stream key of the k-means problem of (sequence b, kv head g, segment s)."""
    return _load().ref_seed_key(b, g, s)


def init_indices(L, K, seed, key):
    out = np.empty(K, dtype=np.int32)
    _load().ref_init_indices(L, K, seed, key, _p(out))
    return out


# ---------------------------------------------------------------- segments / k
def segment_clusters(L, seg_len, K_s):
    return _load().ref_segment_clusters(L, seg_len, K_s)


def num_clusters(N, seg_len, K_s):
    return _load().ref_num_clusters(N, seg_len, K_s)


def k_from_frac(frac, C):
    return _load().ref_k_from_frac(frac, C)


# ---------------------------------------------------------------- k-means
def sq_dist(x, c):
    return _load().ref_sq_dist(_p(_c(x, np.uint16)), _p(_c(c, np.uint16)))


def assign_point(x, chat):
    chat = _c(chat, np.uint16)
    return _load().ref_assign_point(_p(_c(x, np.uint16)), _p(chat), chat.shape[0])


def kmeans_segment(X, K, iters, seed, key=0, exact=False):
    """Lloyd's k-means of one segment seeded by stream key `key` (seed_key(b, g, s) inside a build).
    Returns (assign, centroids fp32, trace [iters][L], objective [iters])."""
    X = _c(X, np.uint16)
    L = X.shape[0]
    a = np.empty(L, dtype=np.int32)
    c = np.empty((K, D), dtype=np.float32)
    tr = np.empty((iters, L), dtype=np.int32)
    obj = np.empty(iters, dtype=np.float64)
    _load().ref_kmeans_segment(_p(X), L, K, iters, seed, key, 1 if exact else 0, _p(a), _p(c), _p(tr), _p(obj))
    return a, c, tr, obj


class Index:
    """Host copy of every index array (same layout as the GPU library's)."""

    FIELDS = ("k_sorted", "v_sorted", "perm", "inv_perm", "assign", "offsets", "sizes", "centroids",
              "centroids_bf16", "vsum")

    def __init__(self, n_kv_heads, ctx, seg_len, clusters_per_seg):
        self.G = int(n_kv_heads)
        self.ctx = _c(ctx, np.int64)
        self.seg_len = int(seg_len)
        self.K_s = int(clusters_per_seg)
        C = [num_clusters(int(n), seg_len, clusters_per_seg) for n in self.ctx]
        self.C = np.array(C, dtype=np.int64)
        rows = int(self.G * self.ctx.sum())
        ncl = int(self.G * self.C.sum())
        noff = int(self.G * (self.C + 1).sum())
        self.k_sorted = np.empty((rows, D), np.uint16)
        self.v_sorted = np.empty((rows, D), np.uint16)
        self.perm = np.empty(rows, np.int32)
        self.inv_perm = np.empty(rows, np.int32)
        self.assign = np.empty(rows, np.int32)
        self.offsets = np.empty(noff, np.int32)
        self.sizes = np.empty(ncl, np.int32)
        self.centroids = np.empty((ncl, D), np.float32)
        self.centroids_bf16 = np.empty((ncl, D), np.uint16)
        self.vsum = np.empty((ncl, D), np.float32)

    def _outs(self):
        return [_p(getattr(self, f)) for f in self.FIELDS]


def build(K, V, n_kv_heads, ctx, seg_len, clusters_per_seg, iters, seed, trace=False):
    """Whole index build (segmented k-means + layout). Returns Index (and the trace if asked)."""
    idx = Index(n_kv_heads, ctx, seg_len, clusters_per_seg)
    K, V = _c(K, np.uint16), _c(V, np.uint16)
    tr = np.empty((iters, K.shape[0]), np.int32) if trace else None
    rc = _load().ref_build(len(idx.ctx), idx.G, _p(idx.ctx), _p(K), _p(V), seg_len, clusters_per_seg, iters, seed,
                           *idx._outs(), _p(tr))
    if rc != 0:
        raise ValueError("ref_build rejected its arguments")
    return (idx, tr) if trace else idx


def index_from_assign(K, V, n_kv_heads, ctx, seg_len, clusters_per_seg, seed, assign):
    """Index over a prescribed clustering: one update from the seeded init with the given labels, then layout."""
    idx = Index(n_kv_heads, ctx, seg_len, clusters_per_seg)
    K, V = _c(K, np.uint16), _c(V, np.uint16)
    rc = _load().ref_index_from_assign(len(idx.ctx), idx.G, _p(idx.ctx), _p(K), _p(V), seg_len, clusters_per_seg,
                                       seed, _p(_c(assign, np.int32)), *idx._outs())
    if rc != 0:
        raise ValueError("ref_index_from_assign rejected its arguments")
    return idx


def block_assign(n_kv_heads, ctx, seg_len, clusters_per_seg):
    """Block ids of every row for the block baseline: token i of a segment of L tokens with K(s) blocks is in
    block floor(i K(s) / L) (Vortex technical summary, section A)."""
    ctx = _c(ctx, np.int64)
    a = np.empty(int(n_kv_heads * ctx.sum()), np.int32)
    _load().ref_block_assign(len(ctx), n_kv_heads, _p(ctx), seg_len, clusters_per_seg, _p(a))
    return a


def build_blocks(K, V, n_kv_heads, ctx, seg_len, clusters_per_seg):
    """Index of the block baseline: the layout, means and value sums over the block clustering."""
    return index_from_assign(K, V, n_kv_heads, ctx, seg_len, clusters_per_seg, 0,
                             block_assign(n_kv_heads, ctx, seg_len, clusters_per_seg))


# ---------------------------------------------------------------- decode
def rank_key(q, c):
    return _load().ref_rank_key(_p(_c(q, np.uint16)), _p(_c(c, np.uint16)))


def select(keys, ids, k):
    keys, ids = _c(keys, np.float32), _c(ids, np.int32)
    out = np.empty(k, np.int32)
    _load().ref_select(_p(keys), _p(ids), len(keys), k, _p(out))
    return out


def sortable(f):
    """Order-preserving 32-bit key of a float (-0 ranks with +0; 0 is never produced)."""
    return _load().ref_sortable(float(np.float32(f)))


def select_stochastic(keys, ids, k, passes, phase_state):
    """Stochastic radix top-k of eligible (keys, ids) (ids ascending): ids in ascending order."""
    keys, ids = _c(keys, np.float32), _c(ids, np.int32)
    out = np.empty(max(k, 1), np.int32)
    _load().ref_select_stochastic(_p(keys), _p(ids), len(keys), k, passes, ctypes.c_uint64(phase_state), _p(out))
    return out[:k]


def stochastic_phase_state(seed, b, h):
    """State whose first SplitMix64 output gives the sampling phase of (b, h)."""
    return (int(seed) + 0x9E3779B97F4A7C15 * (((int(b) << 32) | int(h)) + 1)) % (1 << 64)


def decode_stochastic(index, K, V, q, n_sink, n_local, topk_frac, passes, seed, k_max=None):
    """Wave-index decode with the stochastic radix top-k (ids ascending). Returns as decode()."""
    q = _c(q, np.uint16)
    B, H = q.shape[0], q.shape[1]
    if k_max is None:
        k_max = decode_k_max(index.C, topk_frac)
    out = np.empty((B, H, D), np.float64)
    lse = np.empty((B, H), np.float64)
    ids = np.empty((B, H, max(k_max, 1)), np.int32)
    kc = np.empty((B, H), np.int32)
    rc = _load().ref_decode_stochastic(B, H, index.G, _p(index.ctx), index.seg_len, index.K_s, _p(_c(K, np.uint16)),
                                       _p(_c(V, np.uint16)), _p(index.assign), _p(index.centroids_bf16),
                                       _p(index.vsum), _p(q), n_sink, n_local, topk_frac, passes,
                                       ctypes.c_uint64(seed), k_max, _p(out), _p(lse), _p(ids), _p(kc))
    if rc != 0:
        raise ValueError("ref_decode_stochastic rejected its arguments (rc=%d)" % rc)
    return out, lse, ids[:, :, :k_max], kc


def decode_k_max(C_list, topk_frac):
    return max([k_from_frac(topk_frac, int(C)) for C in C_list] + [0])


def value_sums_bf16(index):
    """The bf16 value sums of an index: round-to-nearest-even of the ordered fp32 sums (the
    estimation zone's per-cluster value sums, RetroInfer page section 2.A, stored at half the
    bytes, as the Vortex page's byte-lean variants do)."""
    return f32_to_bf16(index.vsum)


def _vsum(index, vsum_bf16):
    return bf16_to_f32(value_sums_bf16(index)).astype(np.float32) if vsum_bf16 else index.vsum


def decode(index, K, V, q, n_sink, n_local, topk_frac, k_max=None, shared=False, vsum_bf16=False):
    """Wave-index decode for q [B][H][128] against `index`. Returns (out [B,H,128] f64, lse [B,H], ids, k [B,H]).
    shared: one retrieval set per kv head, chosen by the group key (ref_decode_shared).
    vsum_bf16: the estimation zone reads the bf16 value sums (value_sums_bf16) widened exactly."""
    q = _c(q, np.uint16)
    B, H = q.shape[0], q.shape[1]
    if k_max is None:
        k_max = decode_k_max(index.C, topk_frac)
    out = np.empty((B, H, D), np.float64)
    lse = np.empty((B, H), np.float64)
    ids = np.empty((B, H, max(k_max, 1)), np.int32)
    kc = np.empty((B, H), np.int32)
    fn = _load().ref_decode_shared if shared else _load().ref_decode
    rc = fn(B, H, index.G, _p(index.ctx), index.seg_len, index.K_s, _p(_c(K, np.uint16)),
            _p(_c(V, np.uint16)), _p(index.assign), _p(index.centroids_bf16), _p(_c(_vsum(index, vsum_bf16), np.float32)),
            _p(q), n_sink, n_local, topk_frac, k_max, _p(out), _p(lse), _p(ids), _p(kc))
    if rc != 0:
        raise ValueError("ref_decode rejected its arguments (rc=%d)" % rc)
    return out, lse, ids[:, :, :k_max], kc


def decode_tail(index, K, V, q, n_sink, n_local, topk_frac, Kt, Vt, tail_len, k_max=None, vsum_bf16=False):
    """Wave-index decode plus the tokens appended after the build (exact): Kt, Vt [B][G][cap][128] bf16 bits,
    tail_len [B] <= cap. Returns as decode()."""
    q = _c(q, np.uint16)
    B, H = q.shape[0], q.shape[1]
    Kt = _c(Kt, np.uint16)
    Vt = _c(Vt, np.uint16)
    cap = Kt.shape[2]
    tl = _c(np.asarray(tail_len), np.int32)
    if k_max is None:
        k_max = decode_k_max(index.C, topk_frac)
    out = np.empty((B, H, D), np.float64)
    lse = np.empty((B, H), np.float64)
    ids = np.empty((B, H, max(k_max, 1)), np.int32)
    kc = np.empty((B, H), np.int32)
    rc = _load().ref_decode_tail(B, H, index.G, _p(index.ctx), index.seg_len, index.K_s, _p(_c(K, np.uint16)),
                                 _p(_c(V, np.uint16)), _p(index.assign), _p(index.centroids_bf16),
                                 _p(_c(_vsum(index, vsum_bf16), np.float32)),
                                 _p(q), n_sink, n_local, topk_frac, _p(Kt), _p(Vt), cap, _p(tl), k_max, _p(out),
                                 _p(lse), _p(ids), _p(kc))
    if rc != 0:
        raise ValueError("ref_decode_tail rejected its arguments (rc=%d)" % rc)
    return out, lse, ids[:, :, :k_max], kc


def decode_topk(index, K, V, q, n_sink, n_local, topk_frac, k_max=None):
    """Top-k retrieval without the estimation zone (steady zone + the selected clusters' tokens, exact)."""
    q = _c(q, np.uint16)
    B, H = q.shape[0], q.shape[1]
    if k_max is None:
        k_max = decode_k_max(index.C, topk_frac)
    out = np.empty((B, H, D), np.float64)
    lse = np.empty((B, H), np.float64)
    ids = np.empty((B, H, max(k_max, 1)), np.int32)
    kc = np.empty((B, H), np.int32)
    rc = _load().ref_decode_topk(B, H, index.G, _p(index.ctx), index.seg_len, index.K_s, _p(_c(K, np.uint16)),
                                 _p(_c(V, np.uint16)), _p(index.assign), _p(index.centroids_bf16), _p(q),
                                 n_sink, n_local, topk_frac, k_max, _p(out), _p(lse), _p(ids), _p(kc))
    if rc != 0:
        raise ValueError("ref_decode_topk rejected its arguments (rc=%d)" % rc)
    return out, lse, ids[:, :, :k_max], kc


def full_attention(K, V, q, n_kv_heads, ctx):
    q = _c(q, np.uint16)
    B, H = q.shape[0], q.shape[1]
    ctx = _c(ctx, np.int64)
    out = np.empty((B, H, D), np.float64)
    lse = np.empty((B, H), np.float64)
    _load().ref_full_attention(B, H, n_kv_heads, _p(ctx), _p(_c(K, np.uint16)), _p(_c(V, np.uint16)), _p(q),
                               _p(out), _p(lse))
    return out, lse
