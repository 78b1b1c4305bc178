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
                ("units", ctypes.c_int64), ("max_clusters", ctypes.c_int32), ("cap_segs", ctypes.c_int32),
                ("build_ws_bytes", ctypes.c_size_t), ("kv_rows", ctypes.c_int64)]


class _Index(ctypes.Structure):
    _fields_ = [("shape", _Shape), ("seg_len", ctypes.c_int32), ("clusters_per_seg", ctypes.c_int32),
                ("cap_segs", ctypes.c_int32), ("reserved", ctypes.c_int32), ("k_sorted", ctypes.c_void_p), ("v_sorted", ctypes.c_void_p), ("perm", ctypes.c_void_p),
                ("inv_perm", ctypes.c_void_p), ("assign", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("sizes", ctypes.c_void_p), ("centroids", ctypes.c_void_p), ("centroids_bf16", ctypes.c_void_p),
                ("vsum", ctypes.c_void_p), ("vsum_bf16", ctypes.c_void_p)]


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
        L.wave_index_plan_cap.argtypes = [ctypes.POINTER(_Shape), i32, i32, i32, ctypes.POINTER(_Sizes)]
        L.wave_index_append_plan.argtypes = [ctypes.POINTER(_Index), ctypes.POINTER(ctypes.c_int64),
                                             ctypes.POINTER(ctypes.c_size_t)]
        L.wave_index_append.argtypes = [ctypes.POINTER(_Index), ctypes.POINTER(ctypes.c_int64), P, P, i32, u64, P,
                                        sz, P]
        L.wave_index_build.argtypes = [ctypes.POINTER(_Shape), P, P, i32, i32, i32, u64, ctypes.POINTER(_Index), P,
                                       sz, P, P]
        L.wave_attn_decode_plan.argtypes = [ctypes.POINTER(_Index), i32, i32, i32, ctypes.c_double,
                                            ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_size_t)]
        L.wave_attn_decode.argtypes = [ctypes.POINTER(_Index), P, i32, i32, i32, ctypes.c_double, P, P, P, P, sz, P]
        L.wave_attn_decode_topk.argtypes = L.wave_attn_decode.argtypes
        L.wave_attn_decode_static.argtypes = [ctypes.POINTER(_Index), P, i32, i32, i32, ctypes.c_double, P, P, P, P]
        L.wave_attn_decode_shared.argtypes = L.wave_attn_decode.argtypes
        L.wave_attn_decode_stochastic.argtypes = [ctypes.POINTER(_Index), P, i32, i32, i32, ctypes.c_double, i32, u64,
                                                  P, P, P, P, sz, P]
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
                  "wave_attn_decode_shared", "wave_attn_decode_tail_plan", "wave_attn_decode_tail",
                  "wave_attn_decode_static", "wave_index_plan_cap", "wave_index_append_plan", "wave_index_append",
                  "wave_attn_decode_stochastic"):
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


def _check_tensor(t, name, dtype, shape):
    """Raise ValueError unless t is a contiguous `dtype` tensor of `shape`."""
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_devices(device, **tensors):
    """Every tensor on the GPU `device` (the library reads and writes device memory only)."""
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("%s must be on the GPU, got %s" % (name, t.device))
        if t.device != device:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _check_reuse(index, n_kv_heads, ctx, seg_len, clusters_per_seg, cap_segs=0):
    """An index passed for reuse must have been planned for exactly this shape."""
    if index.cap_segs != int(cap_segs):
        raise ValueError("index was allocated with cap_segs=%d, not %d" % (index.cap_segs, int(cap_segs)))
    if index.cap_segs > 0:
        # a capacity index takes any contexts of its batch size that fit (the plan checks them)
        if (index.n_kv_heads != int(n_kv_heads) or len(index.ctx) != len(ctx) or index.seg_len != int(seg_len)
                or index.clusters_per_seg != int(clusters_per_seg)):
            raise ValueError("index was allocated for n_kv_heads=%d batch=%d seg_len=%d clusters_per_seg=%d"
                             % (index.n_kv_heads, len(index.ctx), index.seg_len, index.clusters_per_seg))
        return
    if (index.n_kv_heads != int(n_kv_heads) or index.ctx != [int(n) for n in ctx]
            or index.seg_len != int(seg_len) or index.clusters_per_seg != int(clusters_per_seg)):
        raise ValueError("index was allocated for n_kv_heads=%d ctx=%s seg_len=%d clusters_per_seg=%d, not for "
                         "n_kv_heads=%d ctx=%s seg_len=%d clusters_per_seg=%d"
                         % (index.n_kv_heads, index.ctx, index.seg_len, index.clusters_per_seg, int(n_kv_heads),
                            [int(n) for n in ctx], int(seg_len), int(clusters_per_seg)))


def _check_build_io(K, V, index, ws, z):
    _check_tensor(K, "K", torch.bfloat16, (z["kv_rows"], HEAD_DIM))
    _check_tensor(V, "V", torch.bfloat16, (z["kv_rows"], HEAD_DIM))
    if ws is not None:
        _check_tensor(ws, "ws", torch.uint8, (ws.numel(),))
        if ws.numel() < z["build_ws_bytes"]:
            raise ValueError("workspace has %d bytes, the build needs %d" % (ws.numel(), z["build_ws_bytes"]))
    _check_devices(index.device if index is not None else K.device, K=K, V=V, ws=ws)


def _check_decode_io(index, q, out, sel_ids, lse, ws, k_max, wsb, **more):
    """q bf16 [B, H, 128] and the outputs of a decode call; then every tensor on the index's device."""
    B, H = int(q.shape[0]), int(q.shape[1])
    if B != len(index.ctx):
        raise ValueError("q holds %d sequences, the index %d" % (B, len(index.ctx)))
    _check_tensor(q, "q", torch.bfloat16, (B, H, HEAD_DIM))
    if out is not None:
        _check_tensor(out, "out", torch.float32, (B, H, HEAD_DIM))
    if sel_ids is not None:
        _check_tensor(sel_ids, "sel_ids", torch.int32, (B, H, max(k_max, 1)))
    if lse is not None:
        _check_tensor(lse, "lse", torch.float32, (B, H))
    if ws is not None:
        _check_tensor(ws, "ws", torch.uint8, (ws.numel(),))
        if ws.numel() < wsb:
            raise ValueError("workspace has %d bytes, the call needs %d" % (ws.numel(), wsb))
    _check_devices(index.device, q=q, out=out, sel_ids=sel_ids, lse=lse, ws=ws, **more)


def wave_index_plan(n_kv_heads, ctx, seg_len, clusters_per_seg, cap_segs=0):
    """Sizes of the index arrays and of the build workspace (dict); cap_segs > 0: every
    (sequence, kv head) block has room for that many segments (wave_index_append)."""
    sh, _keep = _shape(n_kv_heads, ctx)
    z = _Sizes()
    _check(lib().wave_index_plan_cap(ctypes.byref(sh), int(seg_len), int(clusters_per_seg), int(cap_segs),
                                     ctypes.byref(z)))
    return {f: getattr(z, f) for f, _ in _Sizes._fields_}


class WaveIndex:
    """Device arrays of one index (torch tensors) and the C struct pointing at them."""

    def __init__(self, n_kv_heads, ctx, seg_len, clusters_per_seg, arrays, cap_segs=0):
        self.n_kv_heads = int(n_kv_heads)
        self.ctx = [int(n) for n in ctx]
        self.seg_len = int(seg_len)
        self.clusters_per_seg = int(clusters_per_seg)
        self.cap_segs = int(cap_segs)
        self.arrays = arrays
        for k, v in arrays.items():
            setattr(self, k, v)
        self.device = arrays["k_sorted"].device
        sh, self._ctx_arr = _shape(n_kv_heads, self.ctx)
        self.c = _Index()
        self.c.shape = sh
        self.c.seg_len = self.seg_len
        self.c.clusters_per_seg = self.clusters_per_seg
        self.c.cap_segs = self.cap_segs
        for k in ("k_sorted", "v_sorted", "perm", "inv_perm", "assign", "offsets", "sizes", "centroids",
                  "centroids_bf16", "vsum", "vsum_bf16"):
            if k in arrays:
                setattr(self.c, k, arrays[k].data_ptr())
        self.value_sums = "both" if ("vsum" in arrays and "vsum_bf16" in arrays) else (
            "bf16" if "vsum_bf16" in arrays else "f32")

    def set_ctx(self, ctx):
        """Point the index at new contexts (host array kept alive here)."""
        self.ctx = [int(n) for n in ctx]
        self._ctx_arr = (ctypes.c_int64 * len(self.ctx))(*self.ctx)
        self.c.shape.ctx = ctypes.cast(self._ctx_arr, ctypes.POINTER(ctypes.c_int64))

    @staticmethod
    def allocate(n_kv_heads, ctx, seg_len, clusters_per_seg, device="cuda", cap_segs=0, value_sums="f32"):
        """Device arrays of an index. value_sums: "f32" (ordered fp32 sums), "bf16" (their
        round-to-nearest-even bf16, which the estimation zone then reads) or "both"."""
        if value_sums not in ("f32", "bf16", "both"):
            raise ValueError("value_sums must be 'f32', 'bf16' or 'both', got %r" % (value_sums,))
        z = wave_index_plan(n_kv_heads, ctx, seg_len, clusters_per_seg, cap_segs)
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
        }
        if value_sums in ("f32", "both"):
            arrays["vsum"] = torch.empty((Cn, HEAD_DIM), dtype=torch.float32, **e)
        if value_sums in ("bf16", "both"):
            arrays["vsum_bf16"] = torch.empty((Cn, HEAD_DIM), dtype=torch.bfloat16, **e)
        return WaveIndex(n_kv_heads, ctx, seg_len, clusters_per_seg, arrays, cap_segs), z


def _build_prep(K, V, n_kv_heads, ctx, seg_len, clusters_per_seg, cap_segs, index, ws, value_sums="f32"):
    """Checks, and the index and workspace of a build (allocated unless passed)."""
    if index is not None:
        cap_segs = index.cap_segs
    z = wave_index_plan(n_kv_heads, ctx, seg_len, clusters_per_seg, cap_segs)
    if index is not None:
        _check_reuse(index, n_kv_heads, ctx, seg_len, clusters_per_seg, cap_segs)
    _check_build_io(K, V, index, ws, z)
    if index is None:
        index, z = WaveIndex.allocate(n_kv_heads, ctx, seg_len, clusters_per_seg, device=K.device, cap_segs=cap_segs,
                                      value_sums=value_sums)
    else:
        index.set_ctx(ctx)
    if ws is None:
        ws = torch.empty(max(int(z["build_ws_bytes"]), 16), dtype=torch.uint8, device=K.device)
    return index, ws, z


def wave_index_build(K, V, n_kv_heads, ctx, seg_len, clusters_per_seg, iters, seed, assign_trace=False,
                     stream=None, index=None, ws=None, cap_segs=0, value_sums="f32"):
    """Build the index of K, V (bf16 [sum_b G*N_b, 128] device tensors) on the current stream.

    Returns the WaveIndex (and the [iters, rows] int32 assignment trace if asked).  `index`
    and `ws` may be passed to reuse existing allocations; cap_segs > 0 lays the index out
    with room for that many segments per (sequence, kv head) block, for wave_index_append;
    value_sums picks the value sums a new index stores (WaveIndex.allocate).
    """
    index, ws, z = _build_prep(K, V, n_kv_heads, ctx, seg_len, clusters_per_seg, cap_segs, index, ws, value_sums)
    tr = torch.empty((iters, z["rows"]), dtype=torch.int32, device=K.device) if assign_trace else None
    sh = _Shape()
    ctypes.pointer(sh)[0] = index.c.shape  # a copy whose ctx points at the index's own array
    _check(lib().wave_index_build(ctypes.byref(sh), _ptr(K), _ptr(V), int(seg_len), int(clusters_per_seg), int(iters),
                                  ctypes.c_uint64(seed), ctypes.byref(index.c), _ptr(ws), ws.numel(), _ptr(tr),
                                  _stream(stream)))
    return (index, tr) if assign_trace else index


def wave_index_build_blocks(K, V, n_kv_heads, ctx, seg_len, clusters_per_seg, stream=None, index=None, ws=None,
                            cap_segs=0, value_sums="f32"):
    """Index of the block top-k baseline: contiguous blocks in place of the k-means clusters."""
    index, ws, z = _build_prep(K, V, n_kv_heads, ctx, seg_len, clusters_per_seg, cap_segs, index, ws, value_sums)
    sh = _Shape()
    ctypes.pointer(sh)[0] = index.c.shape
    _check(lib().wave_index_build_blocks(ctypes.byref(sh), _ptr(K), _ptr(V), int(seg_len), int(clusters_per_seg),
                                         ctypes.byref(index.c), _ptr(ws), ws.numel(), _stream(stream)))
    return index


def wave_index_append_plan(index, new_ctx):
    """Workspace bytes of wave_index_append(index, ..., new_ctx)."""
    arr = (ctypes.c_int64 * len(new_ctx))(*[int(n) for n in new_ctx])
    n = ctypes.c_size_t()
    _check(lib().wave_index_append_plan(ctypes.byref(index.c), arr, ctypes.byref(n)))
    return n.value


def wave_index_append(index, K_new, V_new, new_ctx, iters, seed, ws=None, stream=None):
    """Grow a capacity index in place to new_ctx: K_new, V_new are bf16 device tensors of the
    appended tokens, [sum_b G*(new_ctx[b] - ctx[b]), 128] ragged over the appended counts.
    Only the segments from the one that held the old end on are clustered again; with the
    build's iters and seed the index equals a build over the longer context."""
    if index.cap_segs < 1:
        raise ValueError("the index has no capacity (built with cap_segs=0)")
    if len(new_ctx) != len(index.ctx):
        raise ValueError("new_ctx has %d sequences, the index %d" % (len(new_ctx), len(index.ctx)))
    new_ctx = [int(n) for n in new_ctx]
    A = [n - o for n, o in zip(new_ctx, index.ctx)]
    if min(A) < 0:
        raise ValueError("new_ctx %s is shorter than the index's ctx %s" % (new_ctx, index.ctx))
    rows = index.n_kv_heads * sum(A)
    _check_tensor(K_new, "K_new", torch.bfloat16, (rows, HEAD_DIM))
    _check_tensor(V_new, "V_new", torch.bfloat16, (rows, HEAD_DIM))
    wsb = wave_index_append_plan(index, new_ctx)
    if ws is not None:
        _check_tensor(ws, "ws", torch.uint8, (ws.numel(),))
        if ws.numel() < wsb:
            raise ValueError("workspace has %d bytes, the append needs %d" % (ws.numel(), wsb))
    _check_devices(index.device, K_new=K_new, V_new=V_new, ws=ws)
    if ws is None:
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=index.device)
    arr = (ctypes.c_int64 * len(new_ctx))(*new_ctx)
    _check(lib().wave_index_append(ctypes.byref(index.c), arr, _ptr(K_new) if rows else None,
                                   _ptr(V_new) if rows else None, int(iters), ctypes.c_uint64(seed), _ptr(ws),
                                   ws.numel(), _stream(stream)))
    index.ctx = new_ctx
    index._ctx_arr = arr  # the C struct now points at it
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
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a [B, H, 128] tensor")
    B, H = q.shape[0], q.shape[1]
    k_max, wsb = wave_attn_decode_plan(index, H, n_sink, n_local, topk_frac)
    _check_decode_io(index, q, out, sel_ids, lse, ws, k_max, wsb)
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


STATIC_SCRATCH_BYTES = 16 << 20  # WAVE_STATIC_SCRATCH_BYTES


def wave_attn_decode_static(index, q, n_sink, n_local, topk_frac, out=None, sel_ids=None, lse=None, stream=None):
    """wave_attn_decode on the library's static device scratch (no workspace; calls on one GPU must not overlap).

    The outputs are allocated here unless given; pass preallocated ones where nothing may allocate."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a [B, H, 128] tensor")
    B, H = q.shape[0], q.shape[1]
    k_max, wsb = wave_attn_decode_plan(index, H, n_sink, n_local, topk_frac)
    _check_decode_io(index, q, out, sel_ids, lse, None, k_max, wsb)
    dev = q.device
    if out is None:
        out = torch.empty((B, H, HEAD_DIM), dtype=torch.float32, device=dev)
    if sel_ids is None:
        sel_ids = torch.empty((B, H, max(k_max, 1)), dtype=torch.int32, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _check(lib().wave_attn_decode_static(ctypes.byref(index.c), _ptr(q), H, int(n_sink), int(n_local),
                                         float(topk_frac), _ptr(out), _ptr(sel_ids), _ptr(lse), _stream(stream)))
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
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a [B, H, 128] tensor")
    B, H = q.shape[0], q.shape[1]
    if not isinstance(k_tail, torch.Tensor) or k_tail.dim() != 4:
        raise ValueError("k_tail must be a [B, G, cap, 128] tensor")
    cap = int(k_tail.shape[2])
    _check_tensor(k_tail, "k_tail", torch.bfloat16, (B, index.n_kv_heads, cap, HEAD_DIM))
    _check_tensor(v_tail, "v_tail", torch.bfloat16, (B, index.n_kv_heads, cap, HEAD_DIM))
    _check_tensor(tail_len, "tail_len", torch.int32, (B,))
    k_max, wsb = wave_attn_decode_tail_plan(index, H, n_sink, n_local, topk_frac, cap)
    _check_decode_io(index, q, out, sel_ids, lse, ws, k_max, wsb, k_tail=k_tail, v_tail=v_tail, tail_len=tail_len)
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


def wave_attn_decode_stochastic(index, q, n_sink, n_local, topk_frac, passes, seed, ws=None, out=None, sel_ids=None,
                                lse=None, stream=None):
    """Wave attention with the stochastic radix top-k (an inexact variant of the selection; ids in
    ascending order). passes: 8-bit radix passes before the threshold bin is sampled (1..4)."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a [B, H, 128] tensor")
    B, H = int(q.shape[0]), int(q.shape[1])
    k_max, wsb = wave_attn_decode_plan(index, H, n_sink, n_local, topk_frac)
    _check_decode_io(index, q, out, sel_ids, lse, ws, k_max, wsb)
    dev = index.device
    if ws is None:
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((B, H, HEAD_DIM), dtype=torch.float32, device=dev)
    if sel_ids is None:
        sel_ids = torch.empty((B, H, max(k_max, 1)), dtype=torch.int32, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _check(lib().wave_attn_decode_stochastic(ctypes.byref(index.c), _ptr(q), H, int(n_sink), int(n_local),
                                             float(topk_frac), int(passes), ctypes.c_uint64(seed), _ptr(out),
                                             _ptr(sel_ids), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))
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
