// wave_attn.hip -- the C ABI of include/wave_attn.h: argument checks, sizes,
// workspace carving and kernel sequencing on the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "internal.h"

namespace {

thread_local char g_err[512] = "";

wave_status fail(wave_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

wave_status ok() {
  g_err[0] = '\0';
  return WAVE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// the value sums: each given array 16-byte aligned; at least one when `need`
wave_status check_vsums(const wave_index* ix, bool need) {
  if (need && ix->vsum == nullptr && ix->vsum_bf16 == nullptr)
    return fail(WAVE_ERR_ARG, "vsum and vsum_bf16 are both NULL");
  if ((ix->vsum && !aligned16(ix->vsum)) || (ix->vsum_bf16 && !aligned16(ix->vsum_bf16)))
    return fail(WAVE_ERR_ALIGN, "index arrays must be 16-byte aligned");
  return WAVE_OK;
}

// ------------------------------------------------------------------ shape checks
wave_status check_shape(const wave_shape* s) {
  if (s == nullptr) return fail(WAVE_ERR_ARG, "shape is NULL");
  if (s->head_dim != WAVE_HEAD_DIM) return fail(WAVE_ERR_UNSUPPORTED, "head_dim %d != 128", s->head_dim);
  if (s->batch < 1) return fail(WAVE_ERR_SHAPE, "batch %d < 1", s->batch);
  if (s->batch > WAVE_MAX_BATCH) return fail(WAVE_ERR_UNSUPPORTED, "batch %d > %d", s->batch, WAVE_MAX_BATCH);
  if (s->n_kv_heads < 1) return fail(WAVE_ERR_SHAPE, "n_kv_heads %d < 1", s->n_kv_heads);
  if (s->ctx == nullptr) return fail(WAVE_ERR_ARG, "shape.ctx is NULL");
  for (int b = 0; b < s->batch; ++b) {
    if (s->ctx[b] < 1) return fail(WAVE_ERR_SHAPE, "ctx[%d] = %lld < 1", b, (long long)s->ctx[b]);
    if (s->ctx[b] >= ((int64_t)1 << 31)) return fail(WAVE_ERR_UNSUPPORTED, "ctx[%d] >= 2^31", b);
  }
  return WAVE_OK;
}

wave_status check_seg(int32_t seg_len, int32_t K_s) {
  if (seg_len < 1) return fail(WAVE_ERR_SHAPE, "seg_len %d < 1", seg_len);
  if (K_s < 1) return fail(WAVE_ERR_SHAPE, "clusters_per_seg %d < 1", K_s);
  if (K_s > seg_len) return fail(WAVE_ERR_SHAPE, "clusters_per_seg %d > seg_len %d", K_s, seg_len);
  if (seg_len > WAVE_MAX_SEG_LEN) return fail(WAVE_ERR_UNSUPPORTED, "seg_len %d > %d", seg_len, WAVE_MAX_SEG_LEN);
  if (K_s > WAVE_MAX_CLUSTERS_PER_SEG)
    return fail(WAVE_ERR_UNSUPPORTED, "clusters_per_seg %d > %d", K_s, WAVE_MAX_CLUSTERS_PER_SEG);
  return WAVE_OK;
}

// capacity of cap segments per block (0: dense) for the contexts of s
wave_status check_cap(const wave_shape* s, int32_t seg_len, int32_t cap) {
  if (cap < 0) return fail(WAVE_ERR_ARG, "cap_segs %d < 0", cap);
  if (cap == 0) return WAVE_OK;
  if ((int64_t)cap * seg_len >= ((int64_t)1 << 31))
    return fail(WAVE_ERR_UNSUPPORTED, "cap_segs * seg_len = %lld >= 2^31", (long long)cap * seg_len);
  for (int b = 0; b < s->batch; ++b)
    if (s->ctx[b] > (int64_t)cap * seg_len)
      return fail(WAVE_ERR_SHAPE, "ctx[%d] = %lld exceeds the capacity of %lld tokens", b, (long long)s->ctx[b],
                  (long long)cap * seg_len);
  return WAVE_OK;
}

wave::SeqArgs make_seq(const wave_shape* s, int32_t seg_len, int32_t K_s, int32_t cap = 0) {
  wave::SeqArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.B = s->batch;
  sa.G = s->n_kv_heads;
  sa.seg_len = seg_len;
  sa.K_s = K_s;
  sa.cap = cap;
  for (int b = 0; b < s->batch; ++b) {
    sa.N[b] = (int32_t)s->ctx[b];
    sa.C[b] = (int32_t)wave::num_clusters(s->ctx[b], seg_len, K_s);
  }
  return sa;
}

void index_sizes(const wave::SeqArgs& sa, wave_index_sizes* o) {
  memset(o, 0, sizeof(*o));
  o->cap_segs = sa.cap;
  for (int b = 0; b < sa.B; ++b) {
    const int64_t R = sa.cap ? (int64_t)sa.cap * sa.seg_len : sa.N[b];
    const int64_t Cs = sa.cap ? (int64_t)sa.cap * sa.K_s : sa.C[b];
    o->rows += (int64_t)sa.G * R;
    o->clusters += (int64_t)sa.G * Cs;
    o->offsets_len += (int64_t)sa.G * (Cs + 1);
    o->kv_rows += (int64_t)sa.G * sa.N[b];
    o->units += (int64_t)sa.G * ((sa.N[b] + sa.seg_len - 1) / sa.seg_len);
    if (sa.C[b] > o->max_clusters) o->max_clusters = sa.C[b];
  }
}

// Build and append workspaces: the norms per index cluster; per input row the sort's
// ranks and the keys' squared norms; an append also stages its input rows (K and V).
struct BuildLayout {
  size_t norm, rank, xn2, big, stage_k, stage_v, total;
};

BuildLayout build_layout(int64_t clusters, int64_t in_rows, bool stage) {
  BuildLayout L;
  size_t o = 0;
  L.norm = o;  o += align256(sizeof(float) * (size_t)clusters);
  L.rank = o;  o += align256(sizeof(int32_t) * (size_t)in_rows);
  L.xn2 = o;   o += align256(sizeof(float) * (size_t)in_rows);
  L.big = o;   o += align256(sizeof(int32_t) * (size_t)wave::BUILD_BIG_WORDS + (size_t)clusters);
  L.stage_k = L.stage_v = o;
  if (stage) {
    L.stage_k = o;  o += align256(2 * (size_t)WAVE_HEAD_DIM * (size_t)in_rows);
    L.stage_v = o;  o += align256(2 * (size_t)WAVE_HEAD_DIM * (size_t)in_rows);
  }
  L.total = o;
  return L;
}

wave_status hip_device_ok() {
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n < 1) return fail(WAVE_ERR_HIP, "no HIP device (%s)", hipGetErrorString(e));
  return WAVE_OK;
}

// ------------------------------------------------------------------ decode sizes
struct DecodePlan {
  wave::DecodeArgs da;
  size_t keys, key32, span, selpre, selw, corr, counts, part, ctop, sortg, total;
};

wave_status decode_plan(const wave_index* ix, int32_t H, int32_t n_sink, int32_t n_local, double frac,
                        DecodePlan* P, int32_t tail_cap = 0) {
  if (ix == nullptr) return fail(WAVE_ERR_ARG, "index is NULL");
  wave_status st = check_shape(&ix->shape);
  if (st != WAVE_OK) return st;
  st = check_seg(ix->seg_len, ix->clusters_per_seg);
  if (st != WAVE_OK) return st;
  const int G = ix->shape.n_kv_heads;
  if (H < 1 || H % G != 0) return fail(WAVE_ERR_SHAPE, "n_q_heads %d is not a positive multiple of n_kv_heads %d", H, G);
  if (H / G > WAVE_MAX_GROUP) return fail(WAVE_ERR_UNSUPPORTED, "%d q heads per kv head > %d", H / G, WAVE_MAX_GROUP);
  if (n_sink < 0 || n_local < 0) return fail(WAVE_ERR_ARG, "n_sink %d / n_local %d negative", n_sink, n_local);
  if (!(frac >= 0.0 && frac <= 1.0)) return fail(WAVE_ERR_ARG, "topk_frac %g outside [0, 1]", frac);
  st = check_cap(&ix->shape, ix->seg_len, ix->cap_segs);
  if (st != WAVE_OK) return st;
  const wave::SeqArgs sa = make_seq(&ix->shape, ix->seg_len, ix->clusters_per_seg, ix->cap_segs);
  wave::DecodeArgs& da = P->da;
  memset(&da, 0, sizeof(da));
  da.H = H;
  da.GS = H / G;
  da.n_sink = n_sink;
  da.n_local = n_local;
  da.tau = (float)(1.0 / sqrt((double)WAVE_HEAD_DIM));
  da.est = 1;
  int kmax = 0, Cmax = 0, nEmax = 0;

  int64_t sumC = 0, sumW = 0;
  for (int b = 0; b < sa.B; ++b) {
    const int64_t N = sa.N[b], C = sa.C[b];
    double x = ceil(frac * (double)C);
    if (x < 0) x = 0;
    if (x > (double)C) x = (double)C;
    da.kreq[b] = (int32_t)x;
    kmax = da.kreq[b] > kmax ? da.kreq[b] : kmax;
    Cmax = C > Cmax ? (int)C : Cmax;
    const int nE = (int)((C + wave::DEC_SCORE_CH - 1) / wave::DEC_SCORE_CH);
    nEmax = nE > nEmax ? nE : nEmax;
    sumC += C;
    sumW += (C + 31) / 32;
    const int64_t a = n_sink < N ? n_sink : N;
    const int64_t c = (N - n_local) > a ? (N - n_local) : a;
    const int64_t nS = a + (N - c);
    if (nS < N && nS > WAVE_MAX_STEADY)
      return fail(WAVE_ERR_UNSUPPORTED, "steady zone of sequence %d has %lld tokens (> %d) without covering it", b,
                  (long long)nS, WAVE_MAX_STEADY);
  }
  da.k_max = kmax;
  int64_t nSmax = 0;
  for (int b = 0; b < sa.B; ++b) {
    const int64_t N = sa.N[b];
    const int64_t a = n_sink < N ? n_sink : N;
    const int64_t c = (N - n_local) > a ? (N - n_local) : a;
    const int64_t nS = a + (N - c);
    nSmax = nS > nSmax ? nS : nSmax;
  }
  da.scap = (int32_t)(nSmax > 0 ? nSmax : 1);
  // gathered-row workgroups per (b, h) at the average cluster size: DEC_ROWS_SMALL rows
  // each if the k_attend grid (with one estimation workgroup per 128 clusters and kv
  // head) is then resident at once, else DEC_ROWS_PER_WG
  const int64_t avg = (ix->seg_len + ix->clusters_per_seg - 1) / ix->clusters_per_seg;
  int64_t est = (int64_t)kmax * avg + nSmax;
  int64_t nest = 0;
  for (int b = 0; b < sa.B; ++b) nest += (int64_t)G * ((sa.C[b] + wave::DEC_SCORE_CH - 1) / wave::DEC_SCORE_CH);
  int64_t Pw = (est + wave::DEC_ROWS_SMALL - 1) / wave::DEC_ROWS_SMALL;
  if ((int64_t)sa.B * H * Pw + nest > wave::DEC_ATT_SLOTS)
    Pw = (est + wave::DEC_ROWS_PER_WG - 1) / wave::DEC_ROWS_PER_WG;
  if (Pw < 1) Pw = 1;
  if (Pw > 4096) Pw = 4096;
  da.P = (int32_t)Pw;
  da.PT = tail_cap > 0 ? (tail_cap + wave::DEC_TAIL_ROWS - 1) / wave::DEC_TAIL_ROWS : 0;
  da.NP = da.P + nEmax + da.PT;
  int64_t nscore = 0;
  for (int b = 0; b < sa.B; ++b) nscore += (int64_t)G * ((sa.C[b] + wave::DEC_SCORE_CH - 1) / wave::DEC_SCORE_CH);
  da.nscore = (int32_t)nscore;
  // keys per lane of the top-k (16 waves x 64 lanes): the fewest that hold every key, so
  // that every wave holds keys (its thresholds then bound the selection); 0: beyond registers
  da.NV = 0;
  for (int nv = 1; nv <= 32; nv *= 2)
    if (wave::DEC_TK_WAVES * 64 * nv >= Cmax) { da.NV = nv; break; }
  constexpr int64_t NVG_Q = (int64_t)wave::DEC_TK_WAVES * 64 * 16;  // keys per 16 a lane
  da.NVg = (int32_t)(((Cmax + NVG_Q - 1) / NVG_Q) * 16);
  int sort_stride = 0;
  if (kmax > wave::DEC_SORT_LDS) {
    sort_stride = 1;
    while (sort_stride < Cmax) sort_stride <<= 1;
  }
  da.sort_stride = sort_stride;
  const int64_t BH = (int64_t)sa.B * H;
  size_t o = 0;
  P->keys = o;   o += align256(4 * (size_t)(H * sumC));
  P->key32 = o;  o += align256(4 * (size_t)(H * sumC));
  P->span = o;   o += align256(8 * (size_t)(H * sumC));
  P->selpre = o; o += align256(4 * (size_t)(H * sumC + BH));
  P->selw = o;   o += align256(4 * (size_t)(H * sumW));
  P->corr = o;   o += align256(4 * (size_t)(BH * da.scap));
  P->counts = o; o += align256(4 * (size_t)(BH * 4));
  P->part = o;   o += align256(4 * (size_t)(BH * da.NP * wave::DEC_PART));
  P->ctop = o;   o += align256(4 * (size_t)(BH * (da.NP - da.P) * 8));
  P->sortg = o;  o += align256(8 * (size_t)(BH * sort_stride));
  P->total = o;
  return WAVE_OK;
}

// ------------------------------------------------------------------ static decode scratch
// The workspace of wave_attn_decode_static: every device holds its own copy of this
// array (from the code object's load until the process ends). Host code never passes
// the array's name to a kernel (on the host it only stands for the symbol): the set-up
// below takes each device's address with hipGetSymbolAddress, and only that address
// reaches the kernels.
__device__ __align__(256) uint8_t scratch[WAVE_STATIC_SCRATCH_BYTES];

// ------------------------------------------------------------------ per-device set-up
constexpr int MAX_DEVICES = 64;
std::once_flag g_dev_once[MAX_DEVICES];
wave::DeviceInfo g_dev_info[MAX_DEVICES];

// ------------------------------------------------------------------ timing hook
// The library's only process-wide mutable state besides the per-device set-up: the
// event pairs of the timed launches, guarded by a mutex, recorded only while enabled.
struct ProfRec {
  std::string name;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
std::vector<ProfRec> g_prof;

}  // namespace

namespace wave {

const DeviceInfo& device_info() {
  static DeviceInfo bad{hipErrorInvalidDevice, 0, nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return bad;
  std::call_once(g_dev_once[dev], [dev] {
    DeviceInfo d{hipSuccess, 0, nullptr};
    d.status = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (d.status == hipSuccess) d.status = hipGetSymbolAddress(&d.scratch, HIP_SYMBOL(scratch));
    if (d.status == hipSuccess && d.scratch == nullptr) d.status = hipErrorInvalidSymbol;
    if (d.status == hipSuccess && d.cus < 1) d.status = hipErrorInvalidDevice;
    if (d.status == hipSuccess) d.status = build_set_attrs();
    if (d.status == hipSuccess) d.status = decode_set_attrs();
    g_dev_info[dev] = d;
  });
  return g_dev_info[dev];
}

bool prof_events(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  if (!g_prof_on.load(std::memory_order_acquire)) return false;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on.load(std::memory_order_relaxed)) return false;
  ProfRec r;
  r.name = name ? name : "";
  if (hipEventCreate(&r.a) != hipSuccess) return false;
  if (hipEventCreate(&r.b) != hipSuccess) {
    (void)hipEventDestroy(r.a);
    return false;
  }
  *start = r.a;
  *stop = r.b;
  g_prof.push_back(r);
  return true;
}

}  // namespace wave

extern "C" {

const char* wave_last_error(void) { return g_err; }

wave_status wave_index_plan_cap(const wave_shape* shape, int32_t seg_len, int32_t clusters_per_seg, int32_t cap_segs,
                                wave_index_sizes* out) {
  wave_status st = check_shape(shape);
  if (st != WAVE_OK) return st;
  st = check_seg(seg_len, clusters_per_seg);
  if (st != WAVE_OK) return st;
  st = check_cap(shape, seg_len, cap_segs);
  if (st != WAVE_OK) return st;
  if (out == nullptr) return fail(WAVE_ERR_ARG, "out is NULL");
  const wave::SeqArgs sa = make_seq(shape, seg_len, clusters_per_seg, cap_segs);
  index_sizes(sa, out);
  out->build_ws_bytes = build_layout(out->clusters, out->kv_rows, false).total;
  return ok();
}

wave_status wave_index_plan(const wave_shape* shape, int32_t seg_len, int32_t clusters_per_seg,
                            wave_index_sizes* out) {
  return wave_index_plan_cap(shape, seg_len, clusters_per_seg, 0, out);
}

// checks shared by the builds; on success *sa, *z and *L describe the call
static wave_status build_checks(const wave_shape* shape, const void* K, const void* V, int32_t seg_len,
                                int32_t clusters_per_seg, const wave_index* out, const void* ws, size_t ws_bytes,
                                wave::SeqArgs* sa, wave_index_sizes* z, BuildLayout* L) {
  wave_status st = check_shape(shape);
  if (st != WAVE_OK) return st;
  st = check_seg(seg_len, clusters_per_seg);
  if (st != WAVE_OK) return st;
  if (K == nullptr || V == nullptr || out == nullptr || ws == nullptr)
    return fail(WAVE_ERR_ARG, "K, V, out and ws must be non-NULL");
  st = check_cap(shape, seg_len, out->cap_segs);
  if (st != WAVE_OK) return st;
  const void* ptrs[] = {out->k_sorted, out->v_sorted, out->perm, out->inv_perm, out->assign, out->offsets,
                        out->sizes, out->centroids, out->centroids_bf16};
  for (const void* p : ptrs)
    if (p == nullptr) return fail(WAVE_ERR_ARG, "an index array pointer is NULL");
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(WAVE_ERR_ALIGN, "index arrays must be 16-byte aligned");
  st = check_vsums(out, true);
  if (st != WAVE_OK) return st;
  if (!aligned16(K) || !aligned16(V) || !aligned16(ws))
    return fail(WAVE_ERR_ALIGN, "K, V and ws must be 16-byte aligned");
  *sa = make_seq(shape, seg_len, clusters_per_seg, out->cap_segs);
  index_sizes(*sa, z);
  *L = build_layout(z->clusters, z->kv_rows, false);
  if (ws_bytes < L->total)
    return fail(WAVE_ERR_WORKSPACE, "build workspace %zu bytes < %zu", ws_bytes, L->total);
  return hip_device_ok();
}

static wave::BuildWs carve_build(void* ws, const BuildLayout& L) {
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  wave::BuildWs bw;
  bw.norm = reinterpret_cast<float*>(w + L.norm);
  bw.rank = reinterpret_cast<int32_t*>(w + L.rank);
  bw.xn2 = reinterpret_cast<float*>(w + L.xn2);
  bw.big = reinterpret_cast<int32_t*>(w + L.big);
  return bw;
}

wave_status wave_index_build(const wave_shape* shape, const void* K, const void* V, int32_t seg_len,
                             int32_t clusters_per_seg, int32_t iters, uint64_t seed, wave_index* out, void* ws,
                             size_t ws_bytes, int32_t* assign_trace, wave_stream_t stream) {
  if (iters < 1) return fail(WAVE_ERR_SHAPE, "iters %d < 1", iters);
  if (assign_trace && !aligned16(assign_trace)) return fail(WAVE_ERR_ALIGN, "assign_trace must be 16-byte aligned");
  wave::SeqArgs sa;
  wave_index_sizes z;
  BuildLayout L;
  wave_status st = build_checks(shape, K, V, seg_len, clusters_per_seg, out, ws, ws_bytes, &sa, &z, &L);
  if (st != WAVE_OK) return st;
  out->shape = *shape;
  out->seg_len = seg_len;
  out->clusters_per_seg = clusters_per_seg;
  hipError_t e = wave::launch_build(sa, K, V, iters, seed, *out, carve_build(ws, L), assign_trace, z.rows,
                                    reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WAVE_ERR_HIP, "build launch failed: %s", hipGetErrorString(e));
  return ok();
}

wave_status wave_index_build_blocks(const wave_shape* shape, const void* K, const void* V, int32_t seg_len,
                                    int32_t clusters_per_seg, wave_index* out, void* ws, size_t ws_bytes,
                                    wave_stream_t stream) {
  wave::SeqArgs sa;
  wave_index_sizes z;
  BuildLayout L;
  wave_status st = build_checks(shape, K, V, seg_len, clusters_per_seg, out, ws, ws_bytes, &sa, &z, &L);
  if (st != WAVE_OK) return st;
  out->shape = *shape;
  out->seg_len = seg_len;
  out->clusters_per_seg = clusters_per_seg;
  hipError_t e = wave::launch_build_blocks(sa, K, V, *out, carve_build(ws, L), reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WAVE_ERR_HIP, "block build launch failed: %s", hipGetErrorString(e));
  return ok();
}

// An append of `index` to new_ctx: the checks, the longer context's SeqArgs, the old
// lengths and the workspace layout (input rows: the tokens from the first changed
// segment to the new end, per appended block).
static wave_status append_checks(const wave_index* ix, const int64_t* new_ctx, wave::SeqArgs* sa, int32_t* n_old,
                                 int64_t* appended, BuildLayout* L) {
  if (ix == nullptr || new_ctx == nullptr) return fail(WAVE_ERR_ARG, "index and new_ctx must be non-NULL");
  wave_status st = check_shape(&ix->shape);
  if (st != WAVE_OK) return st;
  st = check_seg(ix->seg_len, ix->clusters_per_seg);
  if (st != WAVE_OK) return st;
  if (ix->cap_segs < 1) return fail(WAVE_ERR_ARG, "the index has no capacity (cap_segs = %d)", ix->cap_segs);
  st = check_cap(&ix->shape, ix->seg_len, ix->cap_segs);
  if (st != WAVE_OK) return st;
  wave_shape ns = ix->shape;
  ns.ctx = new_ctx;
  st = check_shape(&ns);
  if (st != WAVE_OK) return st;
  const int64_t room = (int64_t)ix->cap_segs * ix->seg_len;
  int64_t in_rows = 0;
  *appended = 0;
  for (int b = 0; b < ns.batch; ++b) {
    const int64_t o = ix->shape.ctx[b], n = new_ctx[b];
    if (n < o) return fail(WAVE_ERR_SHAPE, "new_ctx[%d] = %lld < ctx[%d] = %lld", b, (long long)n, b, (long long)o);
    if (n > room)
      return fail(WAVE_ERR_SHAPE, "new_ctx[%d] = %lld exceeds the capacity of %lld tokens", b, (long long)n,
                  (long long)room);
    n_old[b] = (int32_t)o;
    if (n > o) {
      in_rows += (int64_t)ns.n_kv_heads * (n - (o / ix->seg_len) * ix->seg_len);
      *appended += (int64_t)ns.n_kv_heads * (n - o);
    }
  }
  *sa = make_seq(&ns, ix->seg_len, ix->clusters_per_seg, ix->cap_segs);
  wave_index_sizes z;
  index_sizes(*sa, &z);
  *L = build_layout(z.clusters, in_rows, true);
  return WAVE_OK;
}

wave_status wave_index_append_plan(const wave_index* index, const int64_t* new_ctx, size_t* ws_bytes) {
  if (ws_bytes == nullptr) return fail(WAVE_ERR_ARG, "ws_bytes is NULL");
  wave::SeqArgs sa;
  int32_t n_old[WAVE_MAX_BATCH];
  int64_t appended;
  BuildLayout L;
  wave_status st = append_checks(index, new_ctx, &sa, n_old, &appended, &L);
  if (st != WAVE_OK) return st;
  *ws_bytes = L.total;
  return ok();
}

wave_status wave_index_append(wave_index* index, const int64_t* new_ctx, const void* K_new, const void* V_new,
                              int32_t iters, uint64_t seed, void* ws, size_t ws_bytes, wave_stream_t stream) {
  if (iters < 1) return fail(WAVE_ERR_ARG, "iters %d < 1", iters);
  wave::SeqArgs sa;
  int32_t n_old[WAVE_MAX_BATCH];
  int64_t appended;
  BuildLayout L;
  wave_status st = append_checks(index, new_ctx, &sa, n_old, &appended, &L);
  if (st != WAVE_OK) return st;
  const void* ptrs[] = {index->k_sorted, index->v_sorted, index->perm, index->inv_perm, index->assign,
                        index->offsets, index->sizes, index->centroids, index->centroids_bf16};
  for (const void* p : ptrs)
    if (p == nullptr) return fail(WAVE_ERR_ARG, "an index array pointer is NULL");
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(WAVE_ERR_ALIGN, "index arrays must be 16-byte aligned");
  st = check_vsums(index, true);
  if (st != WAVE_OK) return st;
  if (appended > 0) {
    if (K_new == nullptr || V_new == nullptr || ws == nullptr)
      return fail(WAVE_ERR_ARG, "K_new, V_new and ws must be non-NULL when tokens are appended");
    if (!aligned16(K_new) || !aligned16(V_new) || !aligned16(ws))
      return fail(WAVE_ERR_ALIGN, "K_new, V_new and ws must be 16-byte aligned");
    if (ws_bytes < L.total) return fail(WAVE_ERR_WORKSPACE, "append workspace %zu bytes < %zu", ws_bytes, L.total);
    st = hip_device_ok();
    if (st != WAVE_OK) return st;
    uint8_t* w = reinterpret_cast<uint8_t*>(ws);
    hipError_t e = wave::launch_append(sa, n_old, K_new, V_new, iters, seed, *index, carve_build(ws, L),
                                       w + L.stage_k, w + L.stage_v, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(WAVE_ERR_HIP, "append launch failed: %s", hipGetErrorString(e));
  }
  index->shape.ctx = new_ctx;
  return ok();
}

wave_status wave_attn_decode_plan(const wave_index* index, int32_t n_q_heads, int32_t n_sink, int32_t n_local,
                                  double topk_frac, int32_t* k_max, size_t* ws_bytes) {
  DecodePlan P;
  wave_status st = decode_plan(index, n_q_heads, n_sink, n_local, topk_frac, &P);
  if (st != WAVE_OK) return st;
  if (k_max) *k_max = P.da.k_max;
  if (ws_bytes) *ws_bytes = P.total;
  return ok();
}

static wave_status decode_call(const wave_index* index, const void* q, int32_t n_q_heads, int32_t n_sink,
                               int32_t n_local, double topk_frac, float* out, int32_t* sel_ids, float* lse, void* ws,
                               size_t ws_bytes, wave_stream_t stream, int est, int shared,
                               const void* k_tail = nullptr, const void* v_tail = nullptr, int32_t tail_cap = 0,
                               const int32_t* tail_len = nullptr, int32_t sto_passes = 0, uint64_t sto_seed = 0) {
  DecodePlan P;
  wave_status st = decode_plan(index, n_q_heads, n_sink, n_local, topk_frac, &P, tail_cap);
  if (st != WAVE_OK) return st;
  P.da.est = est;
  P.da.shared = shared;
  P.da.sto_passes = sto_passes;
  P.da.sto_seed = sto_seed;
  P.da.kt = reinterpret_cast<const uint16_t*>(k_tail);
  P.da.vt = reinterpret_cast<const uint16_t*>(v_tail);
  P.da.tail_len = tail_len;
  P.da.tail_cap = tail_cap;
  if (q == nullptr || out == nullptr || ws == nullptr) return fail(WAVE_ERR_ARG, "q, out and ws must be non-NULL");
  if (P.da.k_max > 0 && sel_ids == nullptr) return fail(WAVE_ERR_ARG, "sel_ids is NULL but k_max = %d", P.da.k_max);
  const void* ptrs[] = {index->k_sorted, index->v_sorted, index->perm, index->inv_perm, index->assign,
                        index->offsets, index->sizes, index->centroids_bf16};
  for (const void* p : ptrs)
    if (p == nullptr) return fail(WAVE_ERR_ARG, "an index array pointer is NULL");
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(WAVE_ERR_ALIGN, "index arrays must be 16-byte aligned");
  st = check_vsums(index, est != 0);
  if (st != WAVE_OK) return st;
  if (!aligned16(q) || !aligned16(out) || !aligned16(ws) || (sel_ids && !aligned16(sel_ids)) ||
      (lse && !aligned16(lse)))
    return fail(WAVE_ERR_ALIGN, "q, out, sel_ids, lse and ws must be 16-byte aligned");
  if (ws_bytes < P.total) return fail(WAVE_ERR_WORKSPACE, "decode workspace %zu bytes < %zu", ws_bytes, P.total);
  st = hip_device_ok();
  if (st != WAVE_OK) return st;
  const wave::SeqArgs sa = make_seq(&index->shape, index->seg_len, index->clusters_per_seg, index->cap_segs);
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  wave::DecodeWs dw;
  dw.keys = reinterpret_cast<float*>(w + P.keys);
  dw.key32 = reinterpret_cast<uint32_t*>(w + P.key32);
  dw.span = reinterpret_cast<int2*>(w + P.span);
  dw.selpre = reinterpret_cast<int32_t*>(w + P.selpre);
  dw.selw = reinterpret_cast<uint32_t*>(w + P.selw);
  dw.corr = reinterpret_cast<float*>(w + P.corr);
  dw.counts = reinterpret_cast<int32_t*>(w + P.counts);
  dw.part = reinterpret_cast<float*>(w + P.part);
  dw.ctop = reinterpret_cast<uint32_t*>(w + P.ctop);
  dw.sortg = reinterpret_cast<uint64_t*>(w + P.sortg);
  hipError_t e = wave::launch_decode(sa, P.da, *index, dw, reinterpret_cast<const uint16_t*>(q), out, sel_ids, lse,
                                     reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WAVE_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

wave_status wave_attn_decode(const wave_index* index, const void* q, int32_t n_q_heads, int32_t n_sink,
                             int32_t n_local, double topk_frac, float* out, int32_t* sel_ids, float* lse, void* ws,
                             size_t ws_bytes, wave_stream_t stream) {
  return decode_call(index, q, n_q_heads, n_sink, n_local, topk_frac, out, sel_ids, lse, ws, ws_bytes, stream, 1, 0);
}

wave_status wave_attn_decode_static(const wave_index* index, const void* q, int32_t n_q_heads, int32_t n_sink,
                                    int32_t n_local, double topk_frac, float* out, int32_t* sel_ids, float* lse,
                                    wave_stream_t stream) {
  DecodePlan P;
  wave_status st = decode_plan(index, n_q_heads, n_sink, n_local, topk_frac, &P);
  if (st != WAVE_OK) return st;
  if (P.total > (size_t)WAVE_STATIC_SCRATCH_BYTES)
    return fail(WAVE_ERR_WORKSPACE, "this call needs %zu bytes of workspace, more than the %d of the static scratch",
                P.total, (int)WAVE_STATIC_SCRATCH_BYTES);
  st = hip_device_ok();
  if (st != WAVE_OK) return st;
  const wave::DeviceInfo& di = wave::device_info();
  if (di.status != hipSuccess) return fail(WAVE_ERR_HIP, "device set-up failed: %s", hipGetErrorString(di.status));
  return decode_call(index, q, n_q_heads, n_sink, n_local, topk_frac, out, sel_ids, lse, di.scratch,
                     (size_t)WAVE_STATIC_SCRATCH_BYTES, stream, 1, 0);
}

wave_status wave_attn_decode_tail_plan(const wave_index* index, int32_t n_q_heads, int32_t n_sink, int32_t n_local,
                                       double topk_frac, int32_t tail_cap, int32_t* k_max, size_t* ws_bytes) {
  if (tail_cap < 1 || tail_cap > WAVE_MAX_TAIL)
    return fail(WAVE_ERR_ARG, "tail_cap %d outside [1, %d]", tail_cap, WAVE_MAX_TAIL);
  if (k_max == nullptr || ws_bytes == nullptr) return fail(WAVE_ERR_ARG, "k_max and ws_bytes must be non-NULL");
  DecodePlan P;
  wave_status st = decode_plan(index, n_q_heads, n_sink, n_local, topk_frac, &P, tail_cap);
  if (st != WAVE_OK) return st;
  *k_max = P.da.k_max;
  *ws_bytes = P.total;
  return ok();
}

wave_status wave_attn_decode_tail(const wave_index* index, const void* q, int32_t n_q_heads, int32_t n_sink,
                                  int32_t n_local, double topk_frac, const void* k_tail, const void* v_tail,
                                  int32_t tail_cap, const int32_t* tail_len, float* out, int32_t* sel_ids,
                                  float* lse, void* ws, size_t ws_bytes, wave_stream_t stream) {
  if (tail_cap < 1 || tail_cap > WAVE_MAX_TAIL)
    return fail(WAVE_ERR_ARG, "tail_cap %d outside [1, %d]", tail_cap, WAVE_MAX_TAIL);
  if (k_tail == nullptr || v_tail == nullptr || tail_len == nullptr)
    return fail(WAVE_ERR_ARG, "k_tail, v_tail and tail_len must be non-NULL");
  if (!aligned16(k_tail) || !aligned16(v_tail) || (reinterpret_cast<uintptr_t>(tail_len) & 3) != 0)
    return fail(WAVE_ERR_ALIGN, "k_tail and v_tail must be 16-byte aligned, tail_len 4-byte aligned");
  return decode_call(index, q, n_q_heads, n_sink, n_local, topk_frac, out, sel_ids, lse, ws, ws_bytes, stream, 1, 0,
                     k_tail, v_tail, tail_cap, tail_len);
}

wave_status wave_attn_decode_shared(const wave_index* index, const void* q, int32_t n_q_heads, int32_t n_sink,
                                    int32_t n_local, double topk_frac, float* out, int32_t* sel_ids, float* lse,
                                    void* ws, size_t ws_bytes, wave_stream_t stream) {
  return decode_call(index, q, n_q_heads, n_sink, n_local, topk_frac, out, sel_ids, lse, ws, ws_bytes, stream, 1, 1);
}

wave_status wave_attn_decode_stochastic(const wave_index* index, const void* q, int32_t n_q_heads, int32_t n_sink,
                                        int32_t n_local, double topk_frac, int32_t passes, uint64_t seed, float* out,
                                        int32_t* sel_ids, float* lse, void* ws, size_t ws_bytes,
                                        wave_stream_t stream) {
  if (passes < 1 || passes > 4) return fail(WAVE_ERR_ARG, "passes %d outside [1, 4]", passes);
  if (index != nullptr && check_shape(&index->shape) == WAVE_OK && check_seg(index->seg_len, index->clusters_per_seg) == WAVE_OK)
    for (int b = 0; b < index->shape.batch; ++b)
      if (wave::num_clusters(index->shape.ctx[b], index->seg_len, index->clusters_per_seg) >= ((int64_t)1 << 26))
        return fail(WAVE_ERR_UNSUPPORTED, "sequence %d has 2^26 or more clusters per kv head", b);
  return decode_call(index, q, n_q_heads, n_sink, n_local, topk_frac, out, sel_ids, lse, ws, ws_bytes, stream, 1, 0,
                     nullptr, nullptr, 0, nullptr, passes, seed);
}

wave_status wave_attn_decode_topk(const wave_index* index, const void* q, int32_t n_q_heads, int32_t n_sink,
                                  int32_t n_local, double topk_frac, float* out, int32_t* sel_ids, float* lse,
                                  void* ws, size_t ws_bytes, wave_stream_t stream) {
  return decode_call(index, q, n_q_heads, n_sink, n_local, topk_frac, out, sel_ids, lse, ws, ws_bytes, stream, 0, 0);
}

wave_status wave_profiler_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (on) {
    for (auto& r : g_prof) {
      (void)hipEventDestroy(r.a);
      (void)hipEventDestroy(r.b);
    }
    g_prof.clear();
  }
  g_prof_on.store(on != 0, std::memory_order_release);
  return ok();
}

int32_t wave_profiler_read(char* names, int64_t* launches, double* total_ms, int32_t n_max) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  std::vector<std::string> keys;
  std::vector<int64_t> cnt;
  std::vector<double> ms;
  for (auto& r : g_prof) {
    if (hipEventSynchronize(r.b) != hipSuccess) return (int32_t)fail(WAVE_ERR_HIP, "event synchronize failed");
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return (int32_t)fail(WAVE_ERR_HIP, "elapsed time failed");
    size_t i = 0;
    while (i < keys.size() && keys[i] != r.name) ++i;
    if (i == keys.size()) {
      keys.push_back(r.name);
      cnt.push_back(0);
      ms.push_back(0.0);
    }
    cnt[i] += 1;
    ms[i] += t;
  }
  int32_t n = 0;
  for (size_t i = 0; i < keys.size() && n < n_max; ++i, ++n) {
    if (names) {
      strncpy(names + 64 * n, keys[i].c_str(), 63);
      names[64 * n + 63] = '\0';
    }
    if (launches) launches[n] = cnt[i];
    if (total_ms) total_ms[n] = ms[i];
  }
  g_err[0] = '\0';
  return n;
}

}  // extern "C"
