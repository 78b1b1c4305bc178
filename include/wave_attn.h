/*
 * wave_attn.h -- C ABI of the wave-index sparse decode attention library for
 * AMD MI355X (gfx950): retrieval-based sparse attention over a clustered,
 * HBM-resident KV cache.
 *
 * Method: RetroInfer, "A Vector Storage Engine for Scalable Long-Context LLM
 * Inference" (gist.science summary page), section 2.A: the KV cache is
 * clustered at prefill by segmented clustering; each decode query gets exact
 * attention over a steady zone (sink and recent tokens) and over the clusters
 * its index retrieves (retrieval zone), while the remaining clusters contribute
 * through their centroids (estimation zone). The split into a query-independent
 * build and a query-dependent decode follows Vortex (gist.science summary page,
 * section 2.A, two-phase decomposition into a cache pre-processing step and a
 * query-dependent indexer step).
 *
 * Conventions for every entry point:
 *  - head_dim must be 128; K, V, q and the sorted K/V are bf16 (raw 16-bit
 *    patterns), row major, 128 elements per row, rows 16-byte aligned;
 *  - ragged batch layout: sequence b owns rows [G * sum_{b'<b} N_b', ...) as G
 *    consecutive blocks of N_b rows (kv head major): row of (b, g, t) is
 *    G * sum_{b'<b} N_b' + g * N_b + t;
 *  - the caller owns and allocates every buffer (device memory unless noted
 *    "host"); the library never allocates device memory;
 *  - process-wide state: a thread-local error message; a once-per-device set-up
 *    (kernel attributes, compute-unit count; std::call_once, so concurrent first
 *    calls are safe); and the kernel timing hook below (mutex-guarded, off unless
 *    enabled). Calls on different streams, each with its own workspace and
 *    outputs, may run concurrently from several host threads over one index;
 *  - all argument checks run on the host before anything is enqueued; on an
 *    error status nothing is enqueued and no output is touched; device faults
 *    surface at the caller's next synchronisation of the stream;
 *  - work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    default stream) and never synchronises with the host.
 */
#ifndef WAVE_ATTN_H
#define WAVE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* wave_stream_t; /* same type as hipStream_t */

#define WAVE_HEAD_DIM 128
#define WAVE_MAX_BATCH 256     /* sequences per call */
#define WAVE_MAX_SEG_LEN 65536 /* tokens per segment */
#define WAVE_MAX_CLUSTERS_PER_SEG 2048
#define WAVE_MAX_STEADY 2048   /* steady tokens per sequence unless they cover it all */
#define WAVE_MAX_GROUP 8       /* q heads per kv head */
#define WAVE_MAX_TAIL 65536    /* tokens appended after a build (wave_attn_decode_tail) */

typedef enum wave_status {
  WAVE_OK = 0,
  WAVE_ERR_ARG = -1,         /* null pointer, NaN or out-of-range scalar */
  WAVE_ERR_SHAPE = -2,       /* inconsistent sizes (K_s > L_s, H % G != 0, N_b < 1, iters < 1, ...) */
  WAVE_ERR_UNSUPPORTED = -3, /* head_dim != 128 or a limit above exceeded */
  WAVE_ERR_WORKSPACE = -4,   /* workspace smaller than the plan asked for */
  WAVE_ERR_ALIGN = -5,       /* a device pointer is not 16-byte aligned */
  WAVE_ERR_HIP = -6          /* no device, or a HIP launch failed */
} wave_status;

/* Shape of a (ragged) batch of KV caches of one layer. */
typedef struct wave_shape {
  int32_t batch;        /* B, 1..WAVE_MAX_BATCH */
  int32_t n_kv_heads;   /* G >= 1 */
  int32_t head_dim;     /* must be 128 */
  int32_t reserved;     /* 0 */
  const int64_t* ctx;   /* host [B]: N_b, 1 <= N_b < 2^31 */
} wave_shape;

/*
 * Sizes of the index arrays (element counts) and of the build workspace (bytes).
 * Per (b, g) block the index arrays hold R_b rows and CS_b clusters: R_b = N_b and
 * CS_b = C_b in the dense layout; R_b = cap_segs * L_s and CS_b = cap_segs * K_s
 * with a capacity (wave_index_plan_cap).
 */
typedef struct wave_index_sizes {
  int64_t rows;          /* sum_b G * R_b: rows of k_sorted, v_sorted; length of perm, inv_perm, assign */
  int64_t clusters;      /* sum_b G * CS_b: rows of centroids, centroids_bf16, vsum; length of sizes */
  int64_t offsets_len;   /* sum_b G * (CS_b + 1): length of offsets */
  int64_t units;         /* sum_b G * ceil(N_b / seg_len): independent k-means problems */
  int32_t max_clusters;  /* max_b C_b */
  int32_t cap_segs;      /* the capacity planned for (0: dense layout) */
  size_t build_ws_bytes; /* workspace wave_index_build needs */
  int64_t kv_rows;       /* sum_b G * N_b: rows of the K and V that wave_index_build reads */
} wave_index_sizes;

/*
 * The index: host metadata plus caller-owned device arrays, all filled by
 * wave_index_build (or uploaded by the caller in exactly this layout).
 * Cluster ids are local to one (sequence b, kv head g) block, in [0, C_b),
 * segment major: segment s owns ids [s*K_s, s*K_s + K(s)).
 * Block (b, g) starts at row G*sum_{b'<b} R_b' + g*R_b, cluster
 * G*sum_{b'<b} CS_b' + g*CS_b and offsets entry G*sum_{b'<b} (CS_b'+1) + g*(CS_b+1)
 * (R_b, CS_b as in wave_index_sizes); a block's first N_b rows and C_b clusters
 * (C_b + 1 offsets entries) are filled, the rest of a capacity block is room to grow.
 */
typedef struct wave_index {
  wave_shape shape;         /* ctx points at caller host memory that must outlive the index */
  int32_t seg_len;          /* L_s */
  int32_t clusters_per_seg; /* K_s */
  int32_t cap_segs;         /* 0: dense layout; else segments of room per block. Set by the caller
                               before wave_index_build (the arrays' sizes come from the plan) */
  int32_t reserved;         /* 0 */
  void* k_sorted;           /* bf16 [rows][128]: K rows grouped by cluster, ascending position inside a cluster */
  void* v_sorted;           /* bf16 [rows][128]: V rows in the same order */
  int32_t* perm;            /* [rows]: original position (within its block) of sorted slot p */
  int32_t* inv_perm;        /* [rows]: sorted slot of original position t */
  int32_t* assign;          /* [rows]: cluster id of original position t */
  int32_t* offsets;         /* [offsets_len]: per block, C_b + 1 exclusive prefix sums of sizes */
  int32_t* sizes;           /* [clusters]: members per cluster */
  float* centroids;         /* [clusters][128]: fp32 centroids (member means) */
  void* centroids_bf16;     /* bf16 [clusters][128]: round-to-nearest-even of centroids */
  float* vsum;              /* nullable [clusters][128]: ordered fp32 sum of the members' V rows */
  void* vsum_bf16;          /* nullable bf16 [clusters][128]: round-to-nearest-even of the ordered fp32
                               sums (half the bytes). A build or append writes each of vsum and
                               vsum_bf16 that is non-NULL (at least one must be); the estimation zone
                               reads vsum_bf16 when it is non-NULL, else vsum */
} wave_index;

/*
 * wave_index_plan -- host only. Sizes of the index arrays and of the build
 * workspace for `shape`, segment length seg_len (L_s, 1..WAVE_MAX_SEG_LEN) and
 * clusters_per_seg (K_s, 1..min(L_s, WAVE_MAX_CLUSTERS_PER_SEG)).
 * Segmentation (RetroInfer page, section 2.A, segmented clustering): segments
 * [s*L_s, min((s+1)*L_s, N_b)); a full segment has K_s clusters, a shorter
 * last one of length L has ceil(L*K_s/L_s); C_b is their sum.
 */
wave_status wave_index_plan(const wave_shape* shape, int32_t seg_len, int32_t clusters_per_seg,
                            wave_index_sizes* out);

/*
 * wave_index_plan_cap -- host only. As wave_index_plan, for an index whose blocks
 * have room for cap_segs segments each (cap_segs * L_s rows and cap_segs * K_s
 * clusters per (b, g) block), which wave_index_append can then grow in place up
 * to cap_segs * L_s tokens per sequence. cap_segs 0 is the dense layout.
 * Errors: as wave_index_plan; ARG if cap_segs < 0; SHAPE if some N_b >
 * cap_segs * L_s; UNSUPPORTED if cap_segs * L_s >= 2^31.
 */
wave_status wave_index_plan_cap(const wave_shape* shape, int32_t seg_len, int32_t clusters_per_seg, int32_t cap_segs,
                                wave_index_sizes* out);

/*
 * wave_index_build -- the query-independent phase (RetroInfer page, section
 * 2.A: segmented clustering at prefill). Per (sequence, kv head, segment):
 * seeded init (SplitMix64 seeded at seed + 0x9E3779B97F4A7C15*(k+1) with the
 * segment's key k = b*2^56 + g*2^40 + s*2^16 mod 2^64, partial Fisher-Yates
 * choice of K(s) tokens), then exactly
 * `iters` Lloyd rounds: assignment to the nearest bf16-rounded centroid by
 * squared Euclidean distance (exact ties: lowest id), update to the ordered
 * fp32 mean of the members (empty clusters keep their centroid). Then the
 * layout of wave_index.
 *  K, V:   device bf16, rows [sizes.kv_rows][128] in the dense ragged layout; read only.
 *  out:    caller-filled device pointers of every wave_index array and
 *          cap_segs (sizes from wave_index_plan_cap with that cap_segs); the
 *          call writes shape, seg_len and clusters_per_seg and fills the arrays.
 *  ws:     device workspace of at least build_ws_bytes (16-byte aligned).
 *  assign_trace: nullable device int32 [iters][sizes.rows]: the assignment
 *          array after every round.
 * Errors: ARG (null pointer), SHAPE / UNSUPPORTED (as in wave_index_plan_cap,
 * iters < 1), WORKSPACE, ALIGN, HIP.
 */
wave_status wave_index_build(const wave_shape* shape, const void* K, const void* V, int32_t seg_len,
                             int32_t clusters_per_seg, int32_t iters, uint64_t seed, wave_index* out, void* ws,
                             size_t ws_bytes, int32_t* assign_trace, wave_stream_t stream);

/*
 * wave_index_append_plan -- host only. Workspace bytes of wave_index_append
 * growing `index` to new_ctx. Errors as wave_index_append's argument checks.
 */
wave_status wave_index_append_plan(const wave_index* index, const int64_t* new_ctx, size_t* ws_bytes);

/*
 * wave_index_append -- grow a capacity index in place by the tokens decoded
 * since its build (RetroInfer page, section 2.A: segments are clustered
 * independently, so the index of a longer context differs from that of the
 * shorter one only from the segment that held the old end on; IceCache page:
 * tokens generated during decoding join the indexed cache as they accumulate).
 * For every sequence b with new_ctx[b] > ctx[b] (ctx: index->shape.ctx), the
 * segments s >= floor(ctx[b] / L_s) of every kv head are clustered again over
 * the longer context, with the seeded init and the `iters` Lloyd rounds of
 * wave_index_build, and written in place: the old tokens of segment
 * floor(ctx[b] / L_s) are read from the index itself, the new ones from K_new
 * and V_new. Earlier segments are not touched. Given the build's iters and seed,
 * every array equals that of wave_index_build over the longer context.
 *  index:   a capacity index (cap_segs > 0) filled by wave_index_build or an
 *           earlier append; on success index->shape.ctx = new_ctx.
 *  new_ctx: host [B], ctx[b] <= new_ctx[b] <= cap_segs * L_s; must outlive the index.
 *  K_new, V_new: device bf16 [sum_b G * A_b][128], A_b = new_ctx[b] - ctx[b],
 *           ragged over the appended tokens: row of (b, g, i) is
 *           G * sum_{b'<b} A_b' + g * A_b + i (NULL allowed when no A_b > 0).
 *  ws:      device workspace of at least wave_index_append_plan bytes.
 * Calls on one index must not overlap one another or a decode over it.
 * Errors: ARG (null pointer, iters < 1, cap_segs = 0), SHAPE (new_ctx[b] < ctx[b]
 * or beyond the capacity), WORKSPACE, ALIGN, HIP.
 */
wave_status wave_index_append(wave_index* index, const int64_t* new_ctx, const void* K_new, const void* V_new,
                              int32_t iters, uint64_t seed, void* ws, size_t ws_bytes, wave_stream_t stream);

/*
 * wave_attn_decode_plan -- host only. Sizes of the query-dependent phase (Vortex
 * technical summary, section 2.A: the indexer step runs per query against the
 * pre-processed cache; RetroInfer page, section 2.A: the retrieval zone holds the
 * clusters most similar to the query). For q heads n_q_heads (a multiple of G,
 * at most WAVE_MAX_GROUP per kv head), steady zone (n_sink, n_local) and
 * topk_frac in [0, 1]: k_max = max_b min(ceil(topk_frac*C_b), C_b) (the id
 * columns of wave_attn_decode) and the decode workspace size in bytes.
 * UNSUPPORTED if a sequence's steady zone has more than WAVE_MAX_STEADY
 * tokens without covering the whole sequence.
 */
wave_status wave_attn_decode_plan(const wave_index* index, int32_t n_q_heads, int32_t n_sink, int32_t n_local,
                                  double topk_frac, int32_t* k_max, size_t* ws_bytes);

/*
 * wave_attn_decode -- the query-dependent phase (RetroInfer page, section 2.A,
 * the three zones), for every (sequence b, q head h), kv head g = h*G/H:
 *   S = {t < n_sink} U {t >= N_b - n_local} (steady zone, exact);
 *   n'_j, Vsum'_j = cluster j's size and value sum without its steady tokens;
 *   E = {j : n'_j > 0};  k_b = min(ceil(topk_frac*C_b), |E|);
 *   R = the k_b clusters of E with the largest rank key (a fixed-order fp32
 *       inner product of q and the bf16 centroid, each product rounded to fp32
 *       before it is added; ties: lower id);
 *   retrieval zone: exact attention over the non-steady members of R;
 *   estimation zone: every j in E \ R adds exp(s_j)*n'_j to the denominator
 *       and exp(s_j)*Vsum'_j to the numerator, s_j = q . chat_j / sqrt(128);
 *   out = numerator / denominator, lse = log(denominator) (shifted-max form).
 *  q:       device bf16 [B][n_q_heads][128].
 *  out:     device fp32 [B][n_q_heads][128].
 *  sel_ids: device int32 [B][n_q_heads][k_max] (nullable if k_max == 0): the
 *           selected cluster ids of R in rank order, then -1.
 *  lse:     nullable device fp32 [B][n_q_heads].
 *  ws:      device workspace of at least the planned size; one workspace per
 *           concurrent call (the index itself is read only and may be shared).
 * Errors: ARG, SHAPE, UNSUPPORTED, WORKSPACE, ALIGN, HIP.
 */
wave_status wave_attn_decode(const wave_index* index, const void* q, int32_t n_q_heads, int32_t n_sink,
                             int32_t n_local, double topk_frac, float* out, int32_t* sel_ids, float* lse, void* ws,
                             size_t ws_bytes, wave_stream_t stream);

/*
 * wave_attn_decode_tail -- wave attention over an index plus the tokens decoded
 * after it was built. RetroInfer page, section 2.A: the steady zone keeps the
 * recent tokens exact, and the index grows segment by segment (the segments are
 * clustered independently), so a decoded token waits among the recent tokens
 * until a full segment of them can be clustered (then a wave_index_build over
 * the longer context takes them in). Sequence b has tail_len[b] such tokens after
 * its N_b indexed ones; each is attended exactly by every q head of its kv head,
 * beside wave_attn_decode's three zones over the indexed tokens (whose steady zone
 * is still the first n_sink and the last n_local indexed tokens). S, E, k_b, R
 * and sel_ids are those of wave_attn_decode.
 *  k_tail, v_tail: device bf16 [B][G][tail_cap][128], row (b, g, t) at element
 *            128 * ((b * G + g) * tail_cap + t); rows t < tail_len[b] are read.
 *            Caller-owned, read only, 16-byte aligned.
 *  tail_cap: 1..WAVE_MAX_TAIL.
 *  tail_len: device int32 [B]; a value outside [0, tail_cap] is clamped to it.
 *  ws:       at least wave_attn_decode_tail_plan's size for this tail_cap (one
 *            partial softmax state per q head and 64 appended tokens of capacity).
 * Other arguments and errors as wave_attn_decode; ARG also for a tail_cap out of
 * range or a NULL tail pointer, ALIGN for a misaligned one.
 */
wave_status wave_attn_decode_tail_plan(const wave_index* index, int32_t n_q_heads, int32_t n_sink, int32_t n_local,
                                       double topk_frac, int32_t tail_cap, int32_t* k_max, size_t* ws_bytes);
wave_status wave_attn_decode_tail(const wave_index* index, const void* q, int32_t n_q_heads, int32_t n_sink,
                                  int32_t n_local, double topk_frac, const void* k_tail, const void* v_tail,
                                  int32_t tail_cap, const int32_t* tail_len, float* out, int32_t* sel_ids,
                                  float* lse, void* ws, size_t ws_bytes, wave_stream_t stream);

/*
 * wave_attn_decode_stochastic -- wave_attn_decode with the stochastic radix
 * top-k in place of the exact selection (Vortex page, section 2.C: the top-k
 * terminates early and samples the rest from a threshold bin); an inexact
 * variant, reported by its recall of the exact ids. Per (b, h): a radix descent
 * over the order-preserving 32-bit map of the rank keys, 8 bits a pass, for
 * `passes` passes (1..4; fewer when the threshold bin is needed whole); every
 * bin above the threshold bin is selected whole, and the m ids still missing
 * are the members r (ascending id order, n of them) of the threshold bin with
 * floor((r m + c) / n) < floor(((r + 1) m + c) / n), c = the first SplitMix64
 * output of the stream starting at seed + 0x9E3779B97F4A7C15*((b*2^32 + h) + 1),
 * mod n. Exactly k ids, in ascending order (not rank order), -1 padded.
 * Arguments, workspace (wave_attn_decode_plan) and errors as wave_attn_decode;
 * ARG if passes is outside [1, 4]; UNSUPPORTED with 2^26 or more clusters per
 * (sequence, kv head).
 */
wave_status wave_attn_decode_stochastic(const wave_index* index, const void* q, int32_t n_q_heads, int32_t n_sink,
                                        int32_t n_local, double topk_frac, int32_t passes, uint64_t seed, float* out,
                                        int32_t* sel_ids, float* lse, void* ws, size_t ws_bytes,
                                        wave_stream_t stream);

/*
 * wave_attn_decode_shared -- wave attention with one retrieval set per kv head.
 * The RetroInfer page (section 2.A) retrieves the clusters most similar to the
 * query; under grouped-query attention the q heads of a kv head read the same
 * key/value rows, and the Vortex summary (section A) names GQA backends as the
 * attention it routes to. Here the q heads of kv head g choose their clusters
 * together: the group key of cluster j is the rank keys of g's q heads (as in
 * wave_attn_decode) added in fp32 in head order, and R_{b,g} = the k_b members
 * of E with the largest group keys (ties: lower id), with S, E and k_b as in
 * wave_attn_decode. Each q head then attends exactly to the steady tokens and
 * to the non-steady members of R_{b,g}, and estimates E \ R_{b,g} from its own
 * centroid scores; sel_ids repeats R_{b,g} for every q head of g. The q heads
 * of a kv head read the same rows, which their workgroups share through the
 * L2 cache. Arguments, workspace (wave_attn_decode_plan) and errors as
 * wave_attn_decode.
 */
wave_status wave_attn_decode_shared(const wave_index* index, const void* q, int32_t n_q_heads, int32_t n_sink,
                                    int32_t n_local, double topk_frac, float* out, int32_t* sel_ids, float* lse,
                                    void* ws, size_t ws_bytes, wave_stream_t stream);

/*
 * wave_index_build_blocks -- the index of the block top-k baseline (Vortex
 * technical summary, section A, vFlow: a query-independent phase summarises
 * fixed blocks of the KV cache by their centroids; the query-dependent phase
 * scores the blocks, keeps the top-k and attends to them). Clusters are
 * contiguous blocks instead of k-means clusters: token i of a segment of L
 * tokens with K(s) clusters (as in wave_index_plan) belongs to block
 * floor(i*K(s)/L), so full segments have blocks of L_s/K_s tokens when K_s
 * divides L_s. The arrays are those wave_index_build fills, for that
 * assignment: identity order (perm, inv_perm), sizes, offsets, member means
 * (centroids), their bf16 rounding and the value sums. Arguments, ownership
 * and errors as wave_index_build (no iters, seed or trace).
 */
wave_status wave_index_build_blocks(const wave_shape* shape, const void* K, const void* V, int32_t seg_len,
                                    int32_t clusters_per_seg, wave_index* out, void* ws, size_t ws_bytes,
                                    wave_stream_t stream);

/*
 * wave_attn_decode_topk -- top-k retrieval without the estimation zone (the
 * block top-k baseline's decode; Vortex technical summary, section A): S, E,
 * k_b and R exactly as wave_attn_decode (same ids), and out / lse = exact
 * softmax attention over the steady tokens and the non-steady members of R
 * only. Arguments, workspace (wave_attn_decode_plan) and errors as
 * wave_attn_decode (index->vsum is validated like the other arrays but not read).
 */
wave_status wave_attn_decode_topk(const wave_index* index, const void* q, int32_t n_q_heads, int32_t n_sink,
                                  int32_t n_local, double topk_frac, float* out, int32_t* sel_ids, float* lse,
                                  void* ws, size_t ws_bytes, wave_stream_t stream);

/*
 * wave_attn_decode_static -- wave_attn_decode without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). The call allocates nothing: its
 * workspace is a static device array of WAVE_STATIC_SCRATCH_BYTES that every GPU the
 * library runs on holds from the library's first call there until the process ends.
 * Same kernels, results and errors as wave_attn_decode, plus WORKSPACE when
 * wave_attn_decode_plan's workspace size exceeds WAVE_STATIC_SCRATCH_BYTES (the 128K
 * layer of 32 q / 8 kv heads needs 7.4 MiB). Every call on one GPU shares that GPU's
 * array, so calls that overlap on one GPU (different streams or host threads) race:
 * serialise them, or use wave_attn_decode with one workspace per concurrent call.
 */
#define WAVE_STATIC_SCRATCH_BYTES (16 << 20)
wave_status wave_attn_decode_static(const wave_index* index, const void* q, int32_t n_q_heads, int32_t n_sink,
                                    int32_t n_local, double topk_frac, float* out, int32_t* sel_ids, float* lse,
                                    wave_stream_t stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* wave_last_error(void);

/*
 * Kernel timing hook (not part of the method): while enabled, every kernel of
 * the calls above is launched with a start/stop HIP event pair that the dispatch
 * itself records (hipExtLaunchKernel), so a pair times that kernel alone.
 * wave_profiler_read synchronises on those events and returns, per kernel name,
 * the number of launches and their summed duration.
 *  wave_profiler_enable(1) clears previous records and starts recording;
 *  wave_profiler_enable(0) stops. names: host buffer of n_max * 64 chars.
 * Returns the number of distinct kernels written (or a negative status).
 * The records are process-wide (one list for every thread and device, guarded
 * by a mutex); keep the hook off while capturing HIP graphs.
 */
wave_status wave_profiler_enable(int32_t on);
int32_t wave_profiler_read(char* names, int64_t* launches, double* total_ms, int32_t n_max);

#ifdef __cplusplus
}
#endif

#endif /* WAVE_ATTN_H */
