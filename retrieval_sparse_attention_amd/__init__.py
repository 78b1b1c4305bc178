"""Wave-index sparse decode attention on AMD MI355X (gfx950): Python binding.

A thin ctypes layer over the C ABI of ``include/wave_attn.h`` (libwaveattn.so, built
in this directory).  It only marshals torch tensors' device pointers, sizes and the
current HIP stream into the C calls; every step of the method runs in the library's
HIP kernels.  PyTorch provides device memory and streams.

Method: RetroInfer (gist.science summary page, section 2.A): a segment-clustered KV
cache; per decode query a steady zone (sink + recent tokens), a retrieval zone (the
clusters whose centroids score highest) and an estimation zone (centroids stand in
for the remaining clusters).
"""
import ctypes
import os

import torch  # loads the HIP runtime the library binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwaveattn.so")
HEAD_DIM = 128

WAVE_OK = 0
_STATUS = {0: "OK", -1: "ARG", -2: "SHAPE", -3: "UNSUPPORTED", -4: "WORKSPACE", -5: "ALIGN", -6: "HIP"}


class WaveError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("wave status %s (%d): %s" % (_STATUS.get(status, "?"), status, msg))
        self.status = status


class _Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("ctx", ctypes.POINTER(ctypes.c_int64))]


class _Sizes(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("clusters", ctypes.c_int64), ("offsets_len", ctypes.c_int64),
                ("units", ctypes.c_int64), ("max_clusters", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("build_ws_bytes", ctypes.c_size_t)]


class _Index(ctypes.Structure):
    _fields_ = [("shape", _Shape), ("seg_len", ctypes.c_int32), ("clusters_per_seg", ctypes.c_int32),
                ("k_sorted", ctypes.c_void_p), ("v_sorted", ctypes.c_void_p), ("perm", ctypes.c_void_p),
                ("inv_perm", ctypes.c_void_p), ("assign", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("sizes", ctypes.c_void_p), ("centroids", ctypes.c_void_p), ("centroids_bf16", ctypes.c_void_p),
                ("vsum", ctypes.c_void_p)]


_lib = None


def lib():
    """The loaded libwaveattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libwaveattn.so is not built (run __graft_entry__.build() or "
                               "python -m retrieval_sparse_attention_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
        L.wave_index_plan.argtypes = [ctypes.POINTER(_Shape), i32, i32, ctypes.POINTER(_Sizes)]
        L.wave_index_build.argtypes = [ctypes.POINTER(_Shape), P, P, i32, i32, i32, u64, ctypes.POINTER(_Index), P,
                                       sz, P, P]
        L.wave_attn_decode_plan.argtypes = [ctypes.POINTER(_Index), i32, i32, i32, ctypes.c_double,
                                            ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_size_t)]
        L.wave_attn_decode.argtypes = [ctypes.POINTER(_Index), P, i32, i32, i32, ctypes.c_double, P, P, P, P, sz, P]
        L.wave_attn_decode_topk.argtypes = L.wave_attn_decode.argtypes
        L.wave_attn_decode_shared.argtypes = L.wave_attn_decode.argtypes
        L.wave_attn_decode_tail_plan.argtypes = [ctypes.POINTER(_Index), i32, i32, i32, ctypes.c_double, i32,
                                                 ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_size_t)]
        L.wave_attn_decode_tail.argtypes = [ctypes.POINTER(_Index), P, i32, i32, i32, ctypes.c_double, P, P, i32, P,
                                            P, P, P, P, sz, P]
        L.wave_index_build_blocks.argtypes = [ctypes.POINTER(_Shape), P, P, i32, i32, ctypes.POINTER(_Index), P, sz,
                                              P]
        L.wave_last_error.restype = ctypes.c_char_p
        L.wave_profiler_enable.argtypes = [i32]
        L.wave_profiler_read.argtypes = [ctypes.c_char_p, P, P, i32]
        L.wave_profiler_read.restype = i32
        for f in ("wave_index_plan", "wave_index_build", "wave_attn_decode_plan", "wave_attn_decode",
                  "wave_profiler_enable", "wave_index_build_blocks", "wave_attn_decode_topk",
                  "wave_attn_decode_shared", "wave_attn_decode_tail_plan", "wave_attn_decode_tail"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(st):
    if st != WAVE_OK:
        raise WaveError(st, lib().wave_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _shape(n_kv_heads, ctx):
    ctx_arr = (ctypes.c_int64 * len(ctx))(*[int(n) for n in ctx])
    sh = _Shape(len(ctx), int(n_kv_heads), HEAD_DIM, 0, ctypes.cast(ctx_arr, ctypes.POINTER(ctypes.c_int64)))
    return sh, ctx_arr


def wave_index_plan(n_kv_heads, ctx, seg_len, clusters_per_seg):
    """Sizes of the index arrays and of the build workspace (dict)."""
    sh, _keep = _shape(n_kv_heads, ctx)
    z = _Sizes()
    _check(lib().wave_index_plan(ctypes.byref(sh), int(seg_len), int(clusters_per_seg), ctypes.byref(z)))
    return {f: getattr(z, f) for f, _ in _Sizes._fields_}


class WaveIndex:
    """Device arrays of one index (torch tensors) and the C struct pointing at them."""

    def __init__(self, n_kv_heads, ctx, seg_len, clusters_per_seg, arrays):
        self.n_kv_heads = int(n_kv_heads)
        self.ctx = [int(n) for n in ctx]
        self.seg_len = int(seg_len)
        self.clusters_per_seg = int(clusters_per_seg)
        self.arrays = arrays
        for k, v in arrays.items():
            setattr(self, k, v)
        sh, self._ctx_arr = _shape(n_kv_heads, self.ctx)
        self.c = _Index()
        self.c.shape = sh
        self.c.seg_len = self.seg_len
        self.c.clusters_per_seg = self.clusters_per_seg
        for k in ("k_sorted", "v_sorted", "perm", "inv_perm", "assign", "offsets", "sizes", "centroids",
                  "centroids_bf16", "vsum"):
            setattr(self.c, k, arrays[k].data_ptr())

    @staticmethod
    def allocate(n_kv_heads, ctx, seg_len, clusters_per_seg, device="cuda"):
        z = wave_index_plan(n_kv_heads, ctx, seg_len, clusters_per_seg)
        R, Cn, O = z["rows"], z["clusters"], z["offsets_len"]
        e = dict(device=device)
        arrays = {
            "k_sorted": torch.empty((R, HEAD_DIM), dtype=torch.bfloat16, **e),
            "v_sorted": torch.empty((R, HEAD_DIM), dtype=torch.bfloat16, **e),
            "perm": torch.empty(R, dtype=torch.int32, **e),
            "inv_perm": torch.empty(R, dtype=torch.int32, **e),
            "assign": torch.empty(R, dtype=torch.int32, **e),
            "offsets": torch.empty(O, dtype=torch.int32, **e),
            "sizes": torch.empty(Cn, dtype=torch.int32, **e),
            "centroids": torch.empty((Cn, HEAD_DIM), dtype=torch.float32, **e),
            "centroids_bf16": torch.empty((Cn, HEAD_DIM), dtype=torch.bfloat16, **e),
            "vsum": torch.empty((Cn, HEAD_DIM), dtype=torch.float32, **e),
        }
        return WaveIndex(n_kv_heads, ctx, seg_len, clusters_per_seg, arrays), z


def wave_index_build(K, V, n_kv_heads, ctx, seg_len, clusters_per_seg, iters, seed, assign_trace=False,
                     stream=None, index=None, ws=None):
    """Build the index of K, V (bf16 [sum_b G*N_b, 128] device tensors) on the current stream.

    Returns the WaveIndex (and the [iters, rows] int32 assignment trace if asked).  `index`
    and `ws` may be passed to reuse existing allocations.
    """
    if index is None:
        index, z = WaveIndex.allocate(n_kv_heads, ctx, seg_len, clusters_per_seg, device=K.device)
    else:
        z = wave_index_plan(n_kv_heads, ctx, seg_len, clusters_per_seg)
    if ws is None:
        ws = torch.empty(max(int(z["build_ws_bytes"]), 16), dtype=torch.uint8, device=K.device)
    tr = torch.empty((iters, z["rows"]), dtype=torch.int32, device=K.device) if assign_trace else None
    sh = _Shape()
    ctypes.pointer(sh)[0] = index.c.shape  # a copy whose ctx points at the index's own array
    _check(lib().wave_index_build(ctypes.byref(sh), _ptr(K), _ptr(V), int(seg_len), int(clusters_per_seg), int(iters),
                                  ctypes.c_uint64(seed), ctypes.byref(index.c), _ptr(ws), ws.numel(), _ptr(tr),
                                  _stream(stream)))
    return (index, tr) if assign_trace else index


def wave_index_build_blocks(K, V, n_kv_heads, ctx, seg_len, clusters_per_seg, stream=None, index=None, ws=None):
    """Index of the block top-k baseline: contiguous blocks in place of the k-means clusters."""
    if index is None:
        index, z = WaveIndex.allocate(n_kv_heads, ctx, seg_len, clusters_per_seg, device=K.device)
    else:
        z = wave_index_plan(n_kv_heads, ctx, seg_len, clusters_per_seg)
    if ws is None:
        ws = torch.empty(max(int(z["build_ws_bytes"]), 16), dtype=torch.uint8, device=K.device)
    sh = _Shape()
    ctypes.pointer(sh)[0] = index.c.shape
    _check(lib().wave_index_build_blocks(ctypes.byref(sh), _ptr(K), _ptr(V), int(seg_len), int(clusters_per_seg),
                                         ctypes.byref(index.c), _ptr(ws), ws.numel(), _stream(stream)))
    return index


def wave_attn_decode_plan(index, n_q_heads, n_sink, n_local, topk_frac):
    """(k_max, workspace bytes) of a decode call."""
    k = ctypes.c_int32()
    w = ctypes.c_size_t()
    _check(lib().wave_attn_decode_plan(ctypes.byref(index.c), int(n_q_heads), int(n_sink), int(n_local),
                                       float(topk_frac), ctypes.byref(k), ctypes.byref(w)))
    return k.value, w.value


def wave_attn_decode(index, q, n_sink, n_local, topk_frac, ws=None, out=None, sel_ids=None, lse=None,
                     stream=None, estimate=True, shared=False):
    """One decode query per (sequence, q head): q bf16 [B, H, 128] on the device.

    Returns (out fp32 [B, H, 128], sel_ids int32 [B, H, k_max], lse fp32 [B, H]).
    estimate=False: top-k retrieval only (wave_attn_decode_topk); shared=True: one
    selection per kv head (wave_attn_decode_shared).
    """
    B, H = q.shape[0], q.shape[1]
    k_max, wsb = wave_attn_decode_plan(index, H, n_sink, n_local, topk_frac)
    dev = q.device
    if ws is None:
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((B, H, HEAD_DIM), dtype=torch.float32, device=dev)
    if sel_ids is None:
        sel_ids = torch.empty((B, H, max(k_max, 1)), dtype=torch.int32, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    if shared and not estimate:
        raise ValueError("the shared selection is a variant of wave attention (estimate=True)")
    fn = lib().wave_attn_decode_shared if shared else (lib().wave_attn_decode if estimate else lib().wave_attn_decode_topk)
    _check(fn(ctypes.byref(index.c), _ptr(q), H, int(n_sink), int(n_local), float(topk_frac), _ptr(out), _ptr(sel_ids),
              _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))
    return out, sel_ids[:, :, :k_max], lse


def wave_attn_decode_topk(index, q, n_sink, n_local, topk_frac, ws=None, out=None, sel_ids=None, lse=None,
                          stream=None):
    """Top-k retrieval without the estimation zone (the block baseline's decode); as wave_attn_decode."""
    return wave_attn_decode(index, q, n_sink, n_local, topk_frac, ws, out, sel_ids, lse, stream, estimate=False)


def wave_attn_decode_tail_plan(index, n_q_heads, n_sink, n_local, topk_frac, tail_cap):
    """(k_max, workspace bytes) of a decode call with up to tail_cap appended tokens."""
    k = ctypes.c_int32()
    w = ctypes.c_size_t()
    _check(lib().wave_attn_decode_tail_plan(ctypes.byref(index.c), int(n_q_heads), int(n_sink), int(n_local),
                                            float(topk_frac), int(tail_cap), ctypes.byref(k), ctypes.byref(w)))
    return k.value, w.value


def wave_attn_decode_tail(index, q, n_sink, n_local, topk_frac, k_tail, v_tail, tail_len, ws=None, out=None,
                          sel_ids=None, lse=None, stream=None):
    """Wave attention plus the tokens appended after the build: k_tail, v_tail bf16 [B, G, cap, 128] and
    tail_len int32 [B] on the device. Returns as wave_attn_decode."""
    B, H = q.shape[0], q.shape[1]
    cap = int(k_tail.shape[2])
    if tuple(v_tail.shape) != tuple(k_tail.shape) or tuple(k_tail.shape[:2]) != (B, index.n_kv_heads) or k_tail.shape[3] != 128:
        raise ValueError("k_tail and v_tail must be [B, G, cap, 128]")
    if tail_len.dtype != torch.int32 or tail_len.numel() != B:
        raise ValueError("tail_len must be int32 [B]")
    k_max, wsb = wave_attn_decode_tail_plan(index, H, n_sink, n_local, topk_frac, cap)
    dev = q.device
    if ws is None:
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((B, H, HEAD_DIM), dtype=torch.float32, device=dev)
    if sel_ids is None:
        sel_ids = torch.empty((B, H, max(k_max, 1)), dtype=torch.int32, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _check(lib().wave_attn_decode_tail(ctypes.byref(index.c), _ptr(q), H, int(n_sink), int(n_local), float(topk_frac),
                                       _ptr(k_tail), _ptr(v_tail), cap, _ptr(tail_len), _ptr(out), _ptr(sel_ids),
                                       _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))
    return out, sel_ids[:, :, :k_max], lse


def wave_attn_decode_shared(index, q, n_sink, n_local, topk_frac, ws=None, out=None, sel_ids=None, lse=None,
                            stream=None):
    """Wave attention with one retrieval set per kv head (group key); as wave_attn_decode."""
    return wave_attn_decode(index, q, n_sink, n_local, topk_frac, ws, out, sel_ids, lse, stream, shared=True)


def wave_profiler_enable(on=True):
    _check(lib().wave_profiler_enable(1 if on else 0))


def wave_profiler_read(n_max=64):
    """{kernel name: (launches, total ms)} of the launches recorded since wave_profiler_enable(True)."""
    names = ctypes.create_string_buffer(64 * n_max)
    launches = (ctypes.c_int64 * n_max)()
    ms = (ctypes.c_double * n_max)()
    n = lib().wave_profiler_read(names, ctypes.cast(launches, ctypes.c_void_p), ctypes.cast(ms, ctypes.c_void_p),
                                 n_max)
    if n < 0:
        _check(n)
    return {names.raw[64 * i:64 * i + 64].split(b"\0", 1)[0].decode(): (launches[i], ms[i]) for i in range(n)}
