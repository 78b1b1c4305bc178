/*
 * oracle.c -- plain, slow CPU reference of wave-index sparse decode attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. The GPU library never links, includes or
 * calls it, and it shares no code with the GPU library.
 *
 * Method: RetroInfer, "A Vector Storage Engine for Scalable Long-Context LLM
 * Inference" (gist.science summary page), section 2.A:
 *   - the KV cache is clustered at prefill by segmented clustering (the
 *     sequence is cut into segments that are clustered independently);
 *   - steady zone: sink tokens at the start and recent local tokens get exact
 *     attention;
 *   - retrieval zone: the clusters most similar to the query are fetched and
 *     attended exactly;
 *   - estimation zone: the remaining clusters contribute through their
 *     centroids instead of their tokens.
 * The pages print no formulas for these steps. Every step below is the plainest
 * reading of that section (and of the decode-path spec this library is tested
 * against); each reading is listed with the function that takes it.
 *
 * Precision: binary64 everywhere except where a step is defined in fp32 or
 * bf16 (marked [bit-defined]); those steps are emulated exactly with C float
 * arithmetic (compile with -ffp-contract=off -fno-fast-math, FLT_EVAL_METHOD 0).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define D 128
#define GAMMA 0x9E3779B97F4A7C15ULL

/* ------------------------------------------------------------------ */
/* bf16 format [bit-defined]: IEEE binary32 rounded to an 8-bit significand,
 * round to nearest, ties to even; NaN stays NaN. */
float ref_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint16_t ref_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lower = u & 0xFFFFu, upper = u >> 16;
  /* round half to even on the discarded 16 bits */
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

void ref_f32_to_bf16_array(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = ref_f32_to_bf16(in[i]);
}

/* ------------------------------------------------------------------ */
/* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014): the state advances by the golden-ratio constant
 * and each output is the state passed through the variant-13 mixer. */
uint64_t ref_splitmix64_next(uint64_t* state) {
  *state += GAMMA;
  uint64_t z = *state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

void ref_splitmix64_stream(uint64_t state, int64_t n, uint64_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = ref_splitmix64_next(&state);
}

/*
 * Stream key of the k-means problem of (sequence b, kv head g, segment s)
 * [bit-defined]. The pages fix no initialisation. The reading keys each
 * segment's random stream by its coordinates, not by its rank in an
 * enumeration, so that a segment's seeds do not depend on how many segments
 * the sequences hold: clustering the segments of a longer context leaves the
 * earlier segments as they were, which is what an index that grows segment by
 * segment needs (RetroInfer page, section 2.A: segments are clustered
 * independently). key = b*2^56 + g*2^40 + s*2^16 (mod 2^64); with at most
 * 2^16 draws per segment the streams of distinct (b, g, s) with b < 2^8,
 * g < 2^16 and s < 2^24 never share a state.
 */
uint64_t ref_seed_key(int32_t b, int32_t g, int64_t s) {
  return ((uint64_t)(uint32_t)b << 56) + ((uint64_t)(uint32_t)g << 40) + ((uint64_t)s << 16);
}

/*
 * Seeded initial centroids of one segment [bit-defined]: a fixed-seed choice of
 * K distinct tokens of the segment. The segment with stream key `key` seeds
 * SplitMix64 with seed + GAMMA*(key+1); a partial Fisher-Yates shuffle of
 * [0, L) then picks positions: for i < K, j = i + next() mod (L-i), swap. idx
 * receives the first K entries.
 */
void ref_init_indices(int32_t L, int32_t K, uint64_t seed, uint64_t key, int32_t* idx) {
  int32_t* a = (int32_t*)malloc(sizeof(int32_t) * (size_t)L);
  for (int32_t i = 0; i < L; ++i) a[i] = i;
  uint64_t st = seed + GAMMA * (key + 1);
  for (int32_t i = 0; i < K; ++i) {
    uint64_t r = ref_splitmix64_next(&st);
    int32_t j = i + (int32_t)(r % (uint64_t)(L - i));
    int32_t t = a[i];
    a[i] = a[j];
    a[j] = t;
  }
  for (int32_t i = 0; i < K; ++i) idx[i] = a[i];
  free(a);
}

/* ------------------------------------------------------------------ */
/* Segmented clustering (section 2.A, last paragraph): the sequence of N tokens
 * is cut into segments [s*L_s, min((s+1)*L_s, N)). A full segment gets K_s
 * clusters; a shorter last segment of length L gets ceil(L*K_s/L_s), keeping
 * the average cluster size. Cluster ids of one (sequence, kv head) are
 * segment major: segment s owns ids [s*K_s, s*K_s + K(s)). */
int64_t ref_segment_clusters(int64_t L, int32_t seg_len, int32_t K_s) {
  if (L >= seg_len) return K_s;
  return (L * (int64_t)K_s + seg_len - 1) / seg_len;
}

int64_t ref_num_clusters(int64_t N, int32_t seg_len, int32_t K_s) {
  int64_t nseg = (N + seg_len - 1) / seg_len;
  int64_t last = N - (nseg - 1) * seg_len;
  return (nseg - 1) * (int64_t)K_s + ref_segment_clusters(last, seg_len, K_s);
}

/* Clusters retrieved: ceil(frac * C) evaluated in binary64, clamped to [0, C]. */
int64_t ref_k_from_frac(double frac, int64_t C) {
  double x = ceil(frac * (double)C);
  if (x < 0) x = 0;
  if (x > (double)C) x = (double)C;
  return (int64_t)x;
}

/* ------------------------------------------------------------------ */
/* k-means distance: squared Euclidean distance summed in index order, each
 * subtraction, product and sum rounded to binary64 (no fused operations). */
double ref_sq_dist(const uint16_t* x, const uint16_t* c) {
  double acc = 0.0;
  for (int i = 0; i < D; ++i) {
    double d = (double)ref_bf16_to_f32(x[i]) - (double)ref_bf16_to_f32(c[i]);
    acc = acc + d * d;
  }
  return acc;
}

/* Nearest centroid (assignment step of Lloyd's k-means): argmin over j of
 * ref_sq_dist, exact ties going to the lowest j. */
int32_t ref_assign_point(const uint16_t* x, const uint16_t* chat, int32_t K) {
  int32_t best = 0;
  double bd = ref_sq_dist(x, chat);
  for (int32_t j = 1; j < K; ++j) {
    double dj = ref_sq_dist(x, chat + (int64_t)j * D);
    if (dj < bd) { bd = dj; best = j; }
  }
  return best;
}

/*
 * Update step [bit-defined]: for cluster j with members t1 < t2 < ... < tn,
 * per dimension S = +0.0f, S = fl32(S + x_tk) for k = 1..n, and
 * c_j = fl32(S / fl32(n)) correctly rounded. An empty cluster keeps its
 * previous centroid.
 */
static void update_centroids_f32(const uint16_t* X, int32_t L, int32_t K, const int32_t* a, float* cent) {
  float* S = (float*)calloc((size_t)K * D, sizeof(float));
  int32_t* n = (int32_t*)calloc((size_t)K, sizeof(int32_t));
  for (int32_t t = 0; t < L; ++t) { /* ascending token order */
    int32_t j = a[t];
    n[j] += 1;
    for (int i = 0; i < D; ++i) S[(int64_t)j * D + i] = S[(int64_t)j * D + i] + ref_bf16_to_f32(X[(int64_t)t * D + i]);
  }
  for (int32_t j = 0; j < K; ++j)
    if (n[j] > 0)
      for (int i = 0; i < D; ++i) cent[(int64_t)j * D + i] = S[(int64_t)j * D + i] / (float)n[j];
  free(S);
  free(n);
}

static void update_centroids_exact(const uint16_t* X, int32_t L, int32_t K, const int32_t* a, double* cent) {
  double* S = (double*)calloc((size_t)K * D, sizeof(double));
  int32_t* n = (int32_t*)calloc((size_t)K, sizeof(int32_t));
  for (int32_t t = 0; t < L; ++t) {
    int32_t j = a[t];
    n[j] += 1;
    for (int i = 0; i < D; ++i) S[(int64_t)j * D + i] += (double)ref_bf16_to_f32(X[(int64_t)t * D + i]);
  }
  for (int32_t j = 0; j < K; ++j)
    if (n[j] > 0)
      for (int i = 0; i < D; ++i) cent[(int64_t)j * D + i] = S[(int64_t)j * D + i] / (double)n[j];
  free(S);
  free(n);
}

/*
 * Lloyd's k-means on one segment X[L][128], K clusters, exactly `iters` rounds
 * of (assign, update), no early stop. Spec mode (exact_mode = 0): centroids
 * are fp32, the assignment uses their bf16 rounding chat = bf16(c), the update
 * is the ordered fp32 mean above. Exact mode (exact_mode != 0): centroids stay
 * binary64 and are never rounded (Lloyd's algorithm in binary64), used to pin
 * the loop structure by the monotone objective.
 *
 * assign[L] receives the last assignment (local ids in [0, K)); cent[K][128]
 * the last centroids (fp32; in exact mode rounded to fp32 only on output);
 * trace[it][L] (nullable) every assignment; objective[it] (nullable) the
 * objective after round it: sum over tokens of the squared distance to the
 * assigned centroid (chat in spec mode, c in exact mode).
 */
void ref_kmeans_segment(const uint16_t* X, int32_t L, int32_t K, int32_t iters, uint64_t seed, uint64_t key,
                        int32_t exact_mode, int32_t* assign, float* cent, int32_t* trace, double* objective) {
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
  ref_init_indices(L, K, seed, key, idx);
  /* the bf16 inputs widened to binary64 once (exact), so the distance loops
   * below do the same operations as ref_sq_dist without re-widening */
  double* xd = (double*)malloc(sizeof(double) * (size_t)L * D);
  for (int64_t e = 0; e < (int64_t)L * D; ++e) xd[e] = (double)ref_bf16_to_f32(X[e]);
  double* cd = (double*)malloc(sizeof(double) * (size_t)K * D); /* chat (spec) or c (exact) */
  for (int32_t j = 0; j < K; ++j)
    for (int i = 0; i < D; ++i) {
      cent[(int64_t)j * D + i] = ref_bf16_to_f32(X[(int64_t)idx[j] * D + i]);
      cd[(int64_t)j * D + i] = xd[(int64_t)idx[j] * D + i];
    }
  for (int32_t it = 0; it < iters; ++it) {
    if (!exact_mode) /* chat = bf16(c) */
      for (int64_t e = 0; e < (int64_t)K * D; ++e) cd[e] = (double)ref_bf16_to_f32(ref_f32_to_bf16(cent[e]));
    /* assignment: nearest centroid, lowest j on exact ties */
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < L; ++t) {
      const double* x = xd + (int64_t)t * D;
      int32_t best = 0;
      double bd = 0.0;
      for (int32_t j = 0; j < K; ++j) {
        const double* c = cd + (int64_t)j * D;
        double acc = 0.0;
        for (int i = 0; i < D; ++i) {
          double d = x[i] - c[i];
          acc = acc + d * d;
        }
        if (j == 0 || acc < bd) { bd = acc; best = j; }
      }
      assign[t] = best;
    }
    if (!exact_mode) {
      update_centroids_f32(X, L, K, assign, cent);
    } else {
      update_centroids_exact(X, L, K, assign, cd);
    }
    if (trace) memcpy(trace + (int64_t)it * L, assign, sizeof(int32_t) * (size_t)L);
    if (objective) {
      double J = 0.0;
      for (int32_t t = 0; t < L; ++t) {
        const double* x = xd + (int64_t)t * D;
        double c_i, acc = 0.0;
        for (int i = 0; i < D; ++i) {
          c_i = exact_mode ? cd[(int64_t)assign[t] * D + i]
                           : (double)ref_bf16_to_f32(ref_f32_to_bf16(cent[(int64_t)assign[t] * D + i]));
          double d = x[i] - c_i;
          acc = acc + d * d;
        }
        J += acc;
      }
      objective[it] = J;
    }
  }
  if (exact_mode)
    for (int64_t e = 0; e < (int64_t)K * D; ++e) cent[e] = (float)cd[e];
  free(cd);
  free(xd);
  free(idx);
}

/* ------------------------------------------------------------------ */
/* Index layout of one (sequence, kv head) block of N tokens [bit-defined]:
 * tokens grouped by cluster id, ascending position inside a cluster.
 * perm[p] = original position of sorted slot p, inv_perm its inverse,
 * sizes[j] = |M_j|, offsets[j] = sum of sizes below j (C+1 entries),
 * K/V_sorted[p] = K/V[perm[p]], vsum[j] = ordered fp32 sum of the members'
 * V rows in ascending position (like the update step), chat = bf16(cent). */
static void layout_block(int64_t N, int64_t C, const uint16_t* K, const uint16_t* V, const int32_t* a,
                         const float* cent, uint16_t* k_sorted, uint16_t* v_sorted, int32_t* perm, int32_t* inv_perm,
                         int32_t* offsets, int32_t* sizes, uint16_t* chat, float* vsum) {
  for (int64_t j = 0; j < C; ++j) sizes[j] = 0;
  for (int64_t t = 0; t < N; ++t) sizes[a[t]] += 1;
  offsets[0] = 0;
  for (int64_t j = 0; j < C; ++j) offsets[j + 1] = offsets[j] + sizes[j];
  int32_t* fill = (int32_t*)calloc((size_t)(C > 0 ? C : 1), sizeof(int32_t));
  for (int64_t t = 0; t < N; ++t) {
    int32_t j = a[t];
    int32_t p = offsets[j] + fill[j];
    fill[j] += 1;
    perm[p] = (int32_t)t;
    inv_perm[t] = p;
  }
  free(fill);
  for (int64_t p = 0; p < N; ++p) {
    memcpy(k_sorted + p * D, K + (int64_t)perm[p] * D, D * sizeof(uint16_t));
    memcpy(v_sorted + p * D, V + (int64_t)perm[p] * D, D * sizeof(uint16_t));
  }
  for (int64_t j = 0; j < C; ++j) {
    for (int i = 0; i < D; ++i) {
      float S = 0.0f;
      for (int32_t p = offsets[j]; p < offsets[j + 1]; ++p) S = S + ref_bf16_to_f32(v_sorted[(int64_t)p * D + i]);
      vsum[j * D + i] = S;
      chat[j * D + i] = ref_f32_to_bf16(cent[j * D + i]);
    }
  }
}

/* per-sequence bases of the ragged layout */
typedef struct {
  int64_t row;  /* first row of sequence b: G * sum_{b'<b} N_b' */
  int64_t clu;  /* first cluster: G * sum_{b'<b} C_b' */
  int64_t off;  /* first offsets entry: G * sum_{b'<b} (C_b' + 1) */
  int64_t unit; /* first unit: G * sum_{b'<b} nseg_b' */
} seq_base;

static seq_base* make_bases(int32_t B, int32_t G, const int64_t* ctx, int32_t seg_len, int32_t K_s) {
  seq_base* sb = (seq_base*)malloc(sizeof(seq_base) * (size_t)(B + 1));
  sb[0].row = sb[0].clu = sb[0].off = sb[0].unit = 0;
  for (int32_t b = 0; b < B; ++b) {
    int64_t C = ref_num_clusters(ctx[b], seg_len, K_s);
    int64_t nseg = (ctx[b] + seg_len - 1) / seg_len;
    sb[b + 1].row = sb[b].row + (int64_t)G * ctx[b];
    sb[b + 1].clu = sb[b].clu + (int64_t)G * C;
    sb[b + 1].off = sb[b].off + (int64_t)G * (C + 1);
    sb[b + 1].unit = sb[b].unit + (int64_t)G * nseg;
  }
  return sb;
}

/*
 * Whole index build: per (b, g) block and per segment, seeded init and
 * `iters` rounds of k-means (spec mode), then the block layout. Arrays follow
 * the GPU library's ragged layout (rows [sum_b G*N_b][128], sequence major,
 * then kv head). assign holds block-level cluster ids (segment base + local
 * id). trace (nullable) is [iters][rows]. If given_assign is non-NULL the
 * k-means loop is replaced by one update with those labels from the seeded
 * init (an index over a prescribed clustering).
 */
static int build_impl(int32_t B, int32_t G, const int64_t* ctx, const uint16_t* K, const uint16_t* V, int32_t seg_len,
                      int32_t K_s, int32_t iters, uint64_t seed, const int32_t* given_assign, uint16_t* k_sorted,
                      uint16_t* v_sorted, int32_t* perm, int32_t* inv_perm, int32_t* assign, int32_t* offsets,
                      int32_t* sizes, float* centroids, uint16_t* centroids_bf16, float* vsum, int32_t* trace) {
  if (B < 1 || G < 1 || seg_len < 1 || K_s < 1 || K_s > seg_len || iters < 1) return -1;
  for (int32_t b = 0; b < B; ++b)
    if (ctx[b] < 1) return -1;
  seq_base* sb = make_bases(B, G, ctx, seg_len, K_s);
  int64_t rows = sb[B].row;
  int64_t n_units = sb[B].unit;
  int rc = 0;
  /* enumerate units (b, g, s) in order */
  int64_t* ub = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_units * 3);
  int64_t u = 0;
  for (int32_t b = 0; b < B; ++b) {
    int64_t nseg = (ctx[b] + seg_len - 1) / seg_len;
    for (int32_t g = 0; g < G; ++g)
      for (int64_t s = 0; s < nseg; ++s) { ub[3 * u] = b; ub[3 * u + 1] = g; ub[3 * u + 2] = s; ++u; }
  }
  for (int64_t uu = 0; uu < n_units; ++uu) {
    int32_t b = (int32_t)ub[3 * uu], g = (int32_t)ub[3 * uu + 1];
    int64_t s = ub[3 * uu + 2];
    int64_t N = ctx[b];
    int64_t t0 = s * seg_len;
    int32_t L = (int32_t)((N - t0 < seg_len) ? N - t0 : seg_len);
    int32_t Kc = (int32_t)ref_segment_clusters(L, seg_len, K_s);
    int64_t C = ref_num_clusters(N, seg_len, K_s);
    int64_t row0 = sb[b].row + (int64_t)g * N + t0;
    int64_t clu0 = sb[b].clu + (int64_t)g * C + s * (int64_t)K_s;
    const uint16_t* X = K + row0 * D;
    int32_t* la = (int32_t*)malloc(sizeof(int32_t) * (size_t)L);
    float* cent = centroids + clu0 * D;
    if (given_assign) {
      int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)Kc);
      ref_init_indices(L, Kc, seed, ref_seed_key(b, g, s), idx);
      for (int32_t j = 0; j < Kc; ++j)
        for (int i = 0; i < D; ++i) cent[(int64_t)j * D + i] = ref_bf16_to_f32(X[(int64_t)idx[j] * D + i]);
      free(idx);
      int bad = 0;
      for (int32_t t = 0; t < L; ++t) {
        la[t] = given_assign[row0 + t] - (int32_t)(s * K_s);
        if (la[t] < 0 || la[t] >= Kc) bad = 1;
      }
      if (bad) {
#pragma omp atomic write
        rc = -1;
        for (int32_t t = 0; t < L; ++t) la[t] = 0;
      }
      update_centroids_f32(X, L, Kc, la, cent);
    } else {
      int32_t* tr = trace ? (int32_t*)malloc(sizeof(int32_t) * (size_t)L * iters) : NULL;
      ref_kmeans_segment(X, L, Kc, iters, seed, ref_seed_key(b, g, s), 0, la, cent, tr, NULL);
      if (tr) {
        for (int32_t it = 0; it < iters; ++it)
          for (int32_t t = 0; t < L; ++t) trace[(int64_t)it * rows + row0 + t] = tr[(int64_t)it * L + t] + (int32_t)(s * K_s);
        free(tr);
      }
    }
    for (int32_t t = 0; t < L; ++t) assign[row0 + t] = la[t] + (int32_t)(s * K_s);
    free(la);
  }
  free(ub);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bg = 0; bg < (int64_t)B * G; ++bg) {
    int32_t b = (int32_t)(bg / G), g = (int32_t)(bg % G);
    int64_t N = ctx[b], C = ref_num_clusters(N, seg_len, K_s);
    int64_t row0 = sb[b].row + (int64_t)g * N, clu0 = sb[b].clu + (int64_t)g * C, off0 = sb[b].off + (int64_t)g * (C + 1);
    layout_block(N, C, K + row0 * D, V + row0 * D, assign + row0, centroids + clu0 * D, k_sorted + row0 * D,
                 v_sorted + row0 * D, perm + row0, inv_perm + row0, offsets + off0, sizes + clu0,
                 centroids_bf16 + clu0 * D, vsum + clu0 * D);
  }
  (void)rows;
  free(sb);
  return rc;
}

int ref_build(int32_t B, int32_t G, const int64_t* ctx, const uint16_t* K, const uint16_t* V, int32_t seg_len,
              int32_t K_s, int32_t iters, uint64_t seed, uint16_t* k_sorted, uint16_t* v_sorted, int32_t* perm,
              int32_t* inv_perm, int32_t* assign, int32_t* offsets, int32_t* sizes, float* centroids,
              uint16_t* centroids_bf16, float* vsum, int32_t* trace) {
  return build_impl(B, G, ctx, K, V, seg_len, K_s, iters, seed, NULL, k_sorted, v_sorted, perm, inv_perm, assign,
                    offsets, sizes, centroids, centroids_bf16, vsum, trace);
}

int ref_index_from_assign(int32_t B, int32_t G, const int64_t* ctx, const uint16_t* K, const uint16_t* V,
                          int32_t seg_len, int32_t K_s, uint64_t seed, const int32_t* given_assign, uint16_t* k_sorted,
                          uint16_t* v_sorted, int32_t* perm, int32_t* inv_perm, int32_t* assign, int32_t* offsets,
                          int32_t* sizes, float* centroids, uint16_t* centroids_bf16, float* vsum) {
  return build_impl(B, G, ctx, K, V, seg_len, K_s, 1, seed, given_assign, k_sorted, v_sorted, perm, inv_perm, assign,
                    offsets, sizes, centroids, centroids_bf16, vsum, NULL);
}

/*
 * Block clustering of the block top-k baseline (Vortex technical summary,
 * section A, vFlow: a query-independent phase builds per-block summaries such as
 * block centroids, a query-dependent phase scores the blocks, keeps the top-k and
 * attends to them; its results name block top-k as a workload). Reading: the
 * blocks are contiguous runs of tokens inside the same segments and id space as
 * the clusters, local token i of a segment of L tokens with K(s) clusters in block
 * floor(i * K(s) / L) (balanced; L_s / K_s tokens each when K_s divides L_s).
 * Writes the block-level ids (segment base + local block) of every row.
 */
void ref_block_assign(int32_t B, int32_t G, const int64_t* ctx, int32_t seg_len, int32_t K_s, int32_t* assign) {
  int64_t row = 0;
  for (int32_t b = 0; b < B; ++b)
    for (int32_t g = 0; g < G; ++g)
      for (int64_t t = 0; t < ctx[b]; ++t) {
        int64_t s = t / seg_len, i = t - s * seg_len;
        int64_t L = ctx[b] - s * seg_len < seg_len ? ctx[b] - s * seg_len : seg_len;
        int64_t Kc = ref_segment_clusters(L, seg_len, K_s);
        assign[row++] = (int32_t)(s * K_s + i * Kc / L);
      }
}

/* ------------------------------------------------------------------ */
/*
 * Rank key of a cluster for retrieval [bit-defined]. The retrieval zone ranks
 * clusters by similarity to the query; the reading is the inner product
 * q . chat_j, summed in a fixed fp32 order so that every implementation ranks
 * identically: p_i = fl32(q_i * c_i) (exact for bf16 factors unless the product
 * is below 2^-126 in magnitude or overflows); 16 lane
 * sums u_l = (((+0 + p_8l) + p_8l+1) + ... + p_8l+7); a butterfly over the 16
 * lanes, for s = 8, 4, 2, 1 at once u_l = u_l + u_(l xor s); key = u_0 + 0.0f
 * (which turns -0 into +0).
 */
float ref_rank_key(const uint16_t* q, const uint16_t* c) {
  float u[16], v[16];
  for (int l = 0; l < 16; ++l) {
    float acc = 0.0f;
    for (int m = 0; m < 8; ++m) {
      float p = ref_bf16_to_f32(q[8 * l + m]) * ref_bf16_to_f32(c[8 * l + m]);
      acc = acc + p;
    }
    u[l] = acc;
  }
  for (int s = 8; s >= 1; s >>= 1) {
    for (int l = 0; l < 16; ++l) v[l] = u[l] + u[l ^ s];
    memcpy(u, v, sizeof(u));
  }
  return u[0] + 0.0f;
}

/* order of selection: key descending, cluster id ascending */
typedef struct {
  float key;
  int32_t id;
} keyed;

static int cmp_keyed(const void* a, const void* b) {
  const keyed* x = (const keyed*)a;
  const keyed* y = (const keyed*)b;
  if (x->key > y->key) return -1;
  if (x->key < y->key) return 1;
  return (x->id < y->id) ? -1 : (x->id > y->id);
}

/*
 * Top-k cluster selection: among the candidate ids cand[0..n) with keys,
 * return the first k in (key descending, id ascending) order.
 */
void ref_select(const float* keys, const int32_t* cand, int32_t n, int32_t k, int32_t* out) {
  keyed* e = (keyed*)malloc(sizeof(keyed) * (size_t)(n > 0 ? n : 1));
  for (int32_t i = 0; i < n; ++i) { e[i].key = keys[i]; e[i].id = cand[i]; }
  qsort(e, (size_t)n, sizeof(keyed), cmp_keyed);
  for (int32_t i = 0; i < k; ++i) out[i] = e[i].id;
  free(e);
}

/*
 * Sortable key of a float: an order-preserving map to 32-bit unsigned integers
 * [bit-defined]. For f >= 0 (and for -0, which ranks equal to +0) it is
 * 2^31 + |bits|, for f < 0 it is 2^31 - 1 - |bits|, |bits| being the 31 bits of
 * magnitude. Finite floats land in [2^23, 2^32 - 2^23], so 0 is free.
 */
uint32_t ref_sortable(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  const uint32_t mag = b & 0x7FFFFFFFu;
  if (mag == 0u || !(b >> 31)) return 0x80000000u + mag;
  return 0x7FFFFFFFu - mag;
}

/*
 * Stochastic radix top-k (Vortex page, section 2.C: the top-k terminates early and
 * samples the rest from the threshold bin) [bit-defined reading]. cand[0..n) are
 * the eligible ids in ascending order with their rank keys, k <= n.
 *  - Radix descent over the sortable keys, 8 bits a pass from the top: pass r
 *    counts, among the keys whose first 8r bits equal the prefix P so far, the
 *    keys per value of their next 8 bits; the threshold bin is the value t at
 *    which the count of keys above reaches k (all keys in higher bins are taken,
 *    `above` of them), P becomes P.t. The descent stops after `passes` passes, or
 *    earlier when the threshold bin is needed whole (above + its count = k).
 *  - The m = k - above remaining ids come from the n members of the threshold bin
 *    (prefix P) by systematic sampling with a random phase: with members b_0 <
 *    b_1 < ... in ascending id order and phase c in [0, n), b_r is taken when
 *    floor((r m + c) / n) < floor(((r + 1) m + c) / n): exactly m members, evenly
 *    spread over the bin. c = splitmix64 output of the stream starting at state
 *    phase_state, mod n.
 * out[0..k) receives the selection in ascending id order.
 */
void ref_select_stochastic(const float* keys, const int32_t* cand, int32_t n, int32_t k, int32_t passes,
                           uint64_t phase_state, int32_t* out) {
  uint32_t* u = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(n > 0 ? n : 1));
  for (int32_t i = 0; i < n; ++i) u[i] = ref_sortable(keys[i]);
  uint32_t P = 0;
  int32_t above = 0, done = 0;
  while (done < passes && done < 4) {
    int64_t hist[256];
    for (int v = 0; v < 256; ++v) hist[v] = 0;
    const int shift = 24 - 8 * done;
    for (int32_t i = 0; i < n; ++i)
      if (done == 0 || (u[i] >> (shift + 8)) == P) hist[(u[i] >> shift) & 255u] += 1;
    int t = 255;
    while (t > 0 && above + hist[t] < k) above += (int32_t)hist[t--];
    P = (P << 8) | (uint32_t)t;
    ++done;
    if (above + hist[t] == k) break;
  }
  const int fs = 32 - 8 * done;  /* bits below the prefix */
  int64_t nb = 0;
  for (int32_t i = 0; i < n; ++i)
    if ((uint32_t)((uint64_t)u[i] >> fs) == P) ++nb;
  const int64_t m = k - above;
  const uint64_t c = nb > 0 ? ref_splitmix64_next(&phase_state) % (uint64_t)nb : 0;
  int32_t o = 0;
  int64_t r = 0;
  for (int32_t i = 0; i < n; ++i) {
    const uint32_t pre = (uint32_t)((uint64_t)u[i] >> fs);
    if (pre > P) {
      out[o++] = cand[i];
    } else if (pre == P) {
      if (((uint64_t)r * m + c) / nb < ((uint64_t)(r + 1) * m + c) / nb) out[o++] = cand[i];
      ++r;
    }
  }
  free(u);
}

/*
 * One decode query per (sequence b, q head h) against the index (section 2.A,
 * the three zones), in binary64 apart from the rank key:
 *   S   = steady zone: positions t < n_sink or t >= N - n_local (sink tokens at
 *         the start and recent local tokens);
 *   M_j = members of cluster j (from the index assignment); the clusters cover
 *         every token, so steady tokens are removed from them:
 *         n'_j = |M_j \ S|, Vsum'_j = Vsum_j - sum_{t in M_j cap S} V_t;
 *   E   = {j : n'_j > 0} (clusters with something left to retrieve or estimate);
 *   k   = min(ceil(topk_frac * C), |E|);
 *   R   = the k members of E with the largest rank keys (ties: lower id);
 *   retrieval zone: exact attention terms for t in M_j \ S, j in R;
 *   estimation zone: for j in E \ R the centroid stands in for its tokens:
 *         weight exp(s_j) n'_j in the denominator, exp(s_j) Vsum'_j in the
 *         numerator, s_j = q . chat_j / sqrt(d);
 *   o = numerator / denominator over all three zones, lse = max + ln(denominator).
 * Inputs: original K, V rows, block-level assignment, chat and vsum of the
 * index, q [B][H][128]. Outputs: out [B][H][128], lse [B][H], ids [B][H][k_max]
 * (rank order, -1 padded). Returns k_b per (b, h) in kcount (nullable).
 * shared: R is chosen once per kv head by the group key of each cluster (see
 * ref_decode_shared); the zones of every q head then follow from that R.
 * sto_passes > 0: R is the stochastic radix top-k (ref_select_stochastic, the
 * phase of (b, h) from the stream of key b*2^32 + h under sto_seed), ids in
 * ascending order.
 */
static int decode_impl(int32_t B, int32_t H, int32_t G, const int64_t* ctx, int32_t seg_len, int32_t K_s,
                       const uint16_t* K, const uint16_t* V, const int32_t* assign, const uint16_t* chat,
                       const float* vsum, const uint16_t* q, int32_t n_sink, int32_t n_local, double topk_frac,
                       int32_t k_max, double* out, double* lse, int32_t* ids, int32_t* kcount, int estimate,
                       int shared, const uint16_t* Kt, const uint16_t* Vt, int32_t tail_cap,
                       const int32_t* tail_len, int32_t sto_passes, uint64_t sto_seed) {
  if (B < 1 || G < 1 || H < 1 || H % G != 0 || n_sink < 0 || n_local < 0 || !(topk_frac >= 0.0 && topk_frac <= 1.0))
    return -1;
  seq_base* sb = make_bases(B, G, ctx, seg_len, K_s);
  const double tau = 1.0 / sqrt((double)D);
  int rc = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
    int32_t b = (int32_t)(bh / H), h = (int32_t)(bh % H);
    int32_t g = (int32_t)((int64_t)h * G / H);
    int64_t N = ctx[b], C = ref_num_clusters(N, seg_len, K_s);
    int64_t row0 = sb[b].row + (int64_t)g * N, clu0 = sb[b].clu + (int64_t)g * C;
    const uint16_t* qh = q + bh * D;
    double qd[D];
    for (int i = 0; i < D; ++i) qd[i] = (double)ref_bf16_to_f32(qh[i]);
    /* steady set and cluster corrections */
    int64_t* np = (int64_t*)calloc((size_t)C, sizeof(int64_t));
    double* vs = (double*)malloc(sizeof(double) * (size_t)C * D);
    for (int64_t j = 0; j < C; ++j)
      for (int i = 0; i < D; ++i) vs[j * D + i] = (double)vsum[(clu0 + j) * D + i];
    unsigned char* steady = (unsigned char*)malloc((size_t)N);
    for (int64_t t = 0; t < N; ++t) {
      steady[t] = (t < n_sink) || (t >= N - n_local);
      int32_t j = assign[row0 + t];
      if (!steady[t]) {
        np[j] += 1;
      } else {
        for (int i = 0; i < D; ++i) vs[(int64_t)j * D + i] -= (double)ref_bf16_to_f32(V[(row0 + t) * D + i]);
      }
    }
    /* eligible clusters and their rank keys */
    int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)(C > 0 ? C : 1));
    float* keys = (float*)malloc(sizeof(float) * (size_t)(C > 0 ? C : 1));
    int32_t nE = 0;
    const int32_t GS = H / G;
    for (int64_t j = 0; j < C; ++j)
      if (np[j] > 0) {
        cand[nE] = (int32_t)j;
        if (!shared) {
          keys[nE] = ref_rank_key(qh, chat + (clu0 + j) * D);
        } else {
          /* group key: the rank keys of the kv head's q heads added in head order in fp32 */
          float gk = ref_rank_key(q + ((int64_t)b * H + (int64_t)g * GS) * D, chat + (clu0 + j) * D);
          for (int32_t i = 1; i < GS; ++i)
            gk = gk + ref_rank_key(q + ((int64_t)b * H + (int64_t)g * GS + i) * D, chat + (clu0 + j) * D);
          keys[nE] = gk + 0.0f;
        }
        ++nE;
      }
    int64_t kreq = ref_k_from_frac(topk_frac, C);
    int32_t k = (int32_t)(kreq < nE ? kreq : nE);
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
    if (sto_passes > 0)
      ref_select_stochastic(keys, cand, nE, k, sto_passes,
                            sto_seed + GAMMA * ((((uint64_t)(uint32_t)b << 32) | (uint32_t)h) + 1), sel);
    else
      ref_select(keys, cand, nE, k, sel);
    if (kcount) kcount[bh] = k;
    if (ids) {
      if (k > k_max) {
#pragma omp atomic write
        rc = -2;
      }
      for (int32_t i = 0; i < k_max; ++i) ids[bh * k_max + i] = (i < k) ? sel[i] : -1;
    }
    unsigned char* inR = (unsigned char*)calloc((size_t)(C > 0 ? C : 1), 1);
    for (int32_t i = 0; i < k; ++i) inR[sel[i]] = 1;
    /* scores of every term, then one max-shifted sum */
    double m = -INFINITY;
    double* st = (double*)malloc(sizeof(double) * (size_t)N);
    for (int64_t t = 0; t < N; ++t) {
      int32_t j = assign[row0 + t];
      if (steady[t] || inR[j]) {
        double s = 0.0;
        for (int i = 0; i < D; ++i) s += qd[i] * (double)ref_bf16_to_f32(K[(row0 + t) * D + i]);
        st[t] = tau * s;
        if (st[t] > m) m = st[t];
      }
    }
    /* tokens appended after the index was built: exact, like the steady zone */
    const int64_t nT = Kt ? tail_len[b] : 0;
    const int64_t trow0 = ((int64_t)b * G + g) * tail_cap;
    double* tt = (double*)malloc(sizeof(double) * (size_t)(nT > 0 ? nT : 1));
    for (int64_t t = 0; t < nT; ++t) {
      double s = 0.0;
      for (int i = 0; i < D; ++i) s += qd[i] * (double)ref_bf16_to_f32(Kt[(trow0 + t) * D + i]);
      tt[t] = tau * s;
      if (tt[t] > m) m = tt[t];
    }
    double* sj = (double*)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1));
    for (int64_t j = 0; j < C; ++j) {
      if (estimate && np[j] > 0 && !inR[j]) {
        double s = 0.0;
        for (int i = 0; i < D; ++i) s += qd[i] * (double)ref_bf16_to_f32(chat[(clu0 + j) * D + i]);
        sj[j] = tau * s;
        if (sj[j] > m) m = sj[j];
      }
    }
    double num[D], den = 0.0;
    for (int i = 0; i < D; ++i) num[i] = 0.0;
    for (int64_t t = 0; t < N; ++t) {
      int32_t j = assign[row0 + t];
      if (steady[t] || inR[j]) {
        double w = exp(st[t] - m);
        den += w;
        for (int i = 0; i < D; ++i) num[i] += w * (double)ref_bf16_to_f32(V[(row0 + t) * D + i]);
      }
    }
    for (int64_t j = 0; j < C; ++j) {
      if (estimate && np[j] > 0 && !inR[j]) {
        double w = exp(sj[j] - m);
        den += w * (double)np[j];
        for (int i = 0; i < D; ++i) num[i] += w * vs[j * D + i];
      }
    }
    for (int64_t t = 0; t < nT; ++t) {
      double w = exp(tt[t] - m);
      den += w;
      for (int i = 0; i < D; ++i) num[i] += w * (double)ref_bf16_to_f32(Vt[(trow0 + t) * D + i]);
    }
    free(tt);
    for (int i = 0; i < D; ++i) out[bh * D + i] = num[i] / den;
    if (lse) lse[bh] = m + log(den);
    free(sj);
    free(st);
    free(inR);
    free(sel);
    free(keys);
    free(cand);
    free(steady);
    free(vs);
    free(np);
  }
  free(sb);
  return rc;
}

int ref_decode(int32_t B, int32_t H, int32_t G, const int64_t* ctx, int32_t seg_len, int32_t K_s, const uint16_t* K,
               const uint16_t* V, const int32_t* assign, const uint16_t* chat, const float* vsum, const uint16_t* q,
               int32_t n_sink, int32_t n_local, double topk_frac, int32_t k_max, double* out, double* lse,
               int32_t* ids, int32_t* kcount) {
  return decode_impl(B, H, G, ctx, seg_len, K_s, K, V, assign, chat, vsum, q, n_sink, n_local, topk_frac, k_max, out,
                     lse, ids, kcount, 1, 0, NULL, NULL, 0, NULL, 0, 0);
}

/*
 * Wave attention with the stochastic radix top-k in place of the exact top-k
 * (Vortex page, section 2.C; an inexact variant): R = ref_select_stochastic with
 * `passes` 8-bit passes, phase stream of (b, h) under `seed`; ids in ascending
 * order. Everything else as ref_decode.
 */
int ref_decode_stochastic(int32_t B, int32_t H, int32_t G, const int64_t* ctx, int32_t seg_len, int32_t K_s,
                          const uint16_t* K, const uint16_t* V, const int32_t* assign, const uint16_t* chat,
                          const float* vsum, const uint16_t* q, int32_t n_sink, int32_t n_local, double topk_frac,
                          int32_t passes, uint64_t seed, int32_t k_max, double* out, double* lse, int32_t* ids,
                          int32_t* kcount) {
  if (passes < 1 || passes > 4) return -1;
  return decode_impl(B, H, G, ctx, seg_len, K_s, K, V, assign, chat, vsum, q, n_sink, n_local, topk_frac, k_max, out,
                     lse, ids, kcount, 1, 0, NULL, NULL, 0, NULL, passes, seed);
}

/*
 * Wave attention over an index plus the tokens appended after it was built (the
 * RetroInfer page, section 2.A: the steady zone keeps the recent tokens exact, and
 * the index is built segment by segment, so decoded tokens wait in the recent window
 * until they fill a segment). Sequence b has tail_len[b] <= tail_cap such tokens, K/V
 * rows Kt, Vt [B][G][tail_cap][128] (bf16), positions N_b, N_b + 1, ...; every one is
 * attended exactly, next to ref_decode's three zones over the N_b indexed tokens
 * (whose steady zone is still the first n_sink and the last n_local of them).
 */
int ref_decode_tail(int32_t B, int32_t H, int32_t G, const int64_t* ctx, int32_t seg_len, int32_t K_s,
                    const uint16_t* K, const uint16_t* V, const int32_t* assign, const uint16_t* chat,
                    const float* vsum, const uint16_t* q, int32_t n_sink, int32_t n_local, double topk_frac,
                    const uint16_t* Kt, const uint16_t* Vt, int32_t tail_cap, const int32_t* tail_len,
                    int32_t k_max, double* out, double* lse, int32_t* ids, int32_t* kcount) {
  if (!Kt || !Vt || !tail_len || tail_cap < 0) return -1;
  for (int32_t b = 0; b < B; ++b)
    if (tail_len[b] < 0 || tail_len[b] > tail_cap) return -1;
  return decode_impl(B, H, G, ctx, seg_len, K_s, K, V, assign, chat, vsum, q, n_sink, n_local, topk_frac, k_max, out,
                     lse, ids, kcount, 1, 0, Kt, Vt, tail_cap, tail_len, 0, 0);
}

/*
 * Wave attention with the retrieval set shared by the q heads of a kv head. The
 * pages select the clusters most similar to "the current query"; with grouped
 * query attention every q head of a kv head reads the same clusters, so one
 * selection per kv head lets them share the retrieved rows. The group's key of
 * cluster j is its q heads' rank keys r_{h,j} added in fp32 in head order (the
 * inner product of their summed queries with chat_j, rounded in a fixed order):
 * R_{b,g} = the k members of E with the largest group keys (ties: lower id), the
 * same k and E as ref_decode. Every q head then has its own retrieval zone
 * (exact terms of R's non-steady members), steady zone and estimation zone
 * (E \ R by its own s_j), exactly as in ref_decode. ids [B][H][k_max] repeat the
 * group's selection for each of its q heads.
 */
int ref_decode_shared(int32_t B, int32_t H, int32_t G, const int64_t* ctx, int32_t seg_len, int32_t K_s,
                      const uint16_t* K, const uint16_t* V, const int32_t* assign, const uint16_t* chat,
                      const float* vsum, const uint16_t* q, int32_t n_sink, int32_t n_local, double topk_frac,
                      int32_t k_max, double* out, double* lse, int32_t* ids, int32_t* kcount) {
  return decode_impl(B, H, G, ctx, seg_len, K_s, K, V, assign, chat, vsum, q, n_sink, n_local, topk_frac, k_max, out,
                     lse, ids, kcount, 1, 1, NULL, NULL, 0, NULL, 0, 0);
}

/*
 * Top-k retrieval without the estimation zone (the block top-k baseline of the
 * Vortex technical summary, section A: score the blocks, keep the top-k, attend
 * to them): the same steady zone, E, k and R as ref_decode, and
 * o = softmax over the steady tokens and the non-steady members of R only.
 */
int ref_decode_topk(int32_t B, int32_t H, int32_t G, const int64_t* ctx, int32_t seg_len, int32_t K_s,
                    const uint16_t* K, const uint16_t* V, const int32_t* assign, const uint16_t* chat,
                    const uint16_t* q, int32_t n_sink, int32_t n_local, double topk_frac, int32_t k_max, double* out,
                    double* lse, int32_t* ids, int32_t* kcount) {
  int64_t clusters = 0;
  for (int32_t b = 0; b < B; ++b) clusters += (int64_t)G * ref_num_clusters(ctx[b], seg_len, K_s);
  /* the value sums are not read without the estimation zone; a zero array stands in */
  float* vz = (float*)calloc((size_t)(clusters > 0 ? clusters : 1) * D, sizeof(float));
  int rc = decode_impl(B, H, G, ctx, seg_len, K_s, K, V, assign, chat, vz, q, n_sink, n_local, topk_frac, k_max, out,
                       lse, ids, kcount, 0, 0, NULL, NULL, 0, NULL, 0, 0);
  free(vz);
  return rc;
}

/* Full attention over every token (the dense reference): softmax(q K^T / sqrt(d)) V in binary64. */
void ref_full_attention(int32_t B, int32_t H, int32_t G, const int64_t* ctx, const uint16_t* K, const uint16_t* V,
                        const uint16_t* q, double* out, double* lse) {
  int64_t* rb = (int64_t*)malloc(sizeof(int64_t) * (size_t)(B + 1));
  rb[0] = 0;
  for (int32_t b = 0; b < B; ++b) rb[b + 1] = rb[b] + (int64_t)G * ctx[b];
  const double tau = 1.0 / sqrt((double)D);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
    int32_t b = (int32_t)(bh / H), h = (int32_t)(bh % H);
    int32_t g = (int32_t)((int64_t)h * G / H);
    int64_t N = ctx[b], row0 = rb[b] + (int64_t)g * N;
    double qd[D];
    for (int i = 0; i < D; ++i) qd[i] = (double)ref_bf16_to_f32(q[bh * D + i]);
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
    double m = -INFINITY;
    for (int64_t t = 0; t < N; ++t) {
      double a = 0.0;
      for (int i = 0; i < D; ++i) a += qd[i] * (double)ref_bf16_to_f32(K[(row0 + t) * D + i]);
      s[t] = tau * a;
      if (s[t] > m) m = s[t];
    }
    double num[D], den = 0.0;
    for (int i = 0; i < D; ++i) num[i] = 0.0;
    for (int64_t t = 0; t < N; ++t) {
      double w = exp(s[t] - m);
      den += w;
      for (int i = 0; i < D; ++i) num[i] += w * (double)ref_bf16_to_f32(V[(row0 + t) * D + i]);
    }
    for (int i = 0; i < D; ++i) out[bh * D + i] = num[i] / den;
    if (lse) lse[bh] = m + log(den);
    free(s);
  }
  free(rb);
}
