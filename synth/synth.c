/*
 * synth.c -- seeded synthetic inputs for wave-index sparse decode attention.
 *
 * This module only draws inputs. It holds none of the method's arithmetic:
 * no clustering, no scoring, no attention. Both the CPU oracle and the GPU
 * library consume the arrays it writes, so the two sides see identical data.
 *
 * Workload shape (RetroInfer page, section 1 and 4: long-context KV caches of
 * Llama-3-8B-like layers, 8 kv heads x 128 dims, contexts of 120K to 1M):
 *   - per (sequence b, kv head g): a mixture of M = 1024 components with key
 *     centres mu_m ~ N(0, I) and value centres nu_m ~ N(0, I);
 *   - a per-segment drift of the key centres: d_0 = 0, d_s = d_{s-1} + N(0, 0.05^2 I);
 *   - token t of segment s picks a component m_t ~ U{0..M-1} and gets
 *     K_t = bf16(mu_{m_t} + d_s + 0.3 z), V_t = bf16(nu_{m_t} + 0.3 z');
 *   - heavy-tailed keys replace z by a Student-t variate with 4 degrees of freedom;
 *   - a query for q head h (kv head g(h) = h*G/H) is bf16(K_{t*} + 0.5 z) for a
 *     uniformly drawn t*.
 *
 * Every draw is counter based: value i of stream `key` is the i-th output of a
 * SplitMix64 generator (Steele, Lea and Flood, OOPSLA 2014) whose state starts
 * at `key`, so any element can be produced independently and in parallel.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SYN_D 128
#define SYN_M 1024
#define SYN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t syn_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* i-th output of a SplitMix64 stream started at `key`. */
static inline uint64_t syn_u64(uint64_t key, uint64_t i) { return syn_mix(key + (i + 1) * SYN_GAMMA); }

/* uniform in (0, 1) from the top 53 bits */
static inline double syn_unif(uint64_t key, uint64_t i) {
  return ((double)(syn_u64(key, i) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* standard normal by the Box-Muller transform on draws 2i and 2i+1 */
static inline double syn_normal(uint64_t key, uint64_t i) {
  double u1 = syn_unif(key, 2 * i), u2 = syn_unif(key, 2 * i + 1);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

/* Student-t with 4 dof: z / sqrt(chi2_4 / 4), chi2_4 = -2 ln(u1 u2) (a Gamma(2, 2) variate) */
static inline double syn_student4(uint64_t key, uint64_t i) {
  double z = syn_normal(key, 2 * i);
  double u1 = syn_unif(key ^ 0x5555555555555555ULL, 2 * i), u2 = syn_unif(key ^ 0x5555555555555555ULL, 2 * i + 1);
  double chi = -2.0 * log(u1 * u2);
  return z / sqrt(chi / 4.0);
}

/* round-to-nearest-even float -> bfloat16 bits, used only to store the drawn inputs */
static inline uint16_t syn_bf16(double x) {
  float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline float syn_bf16_to_f(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* stream keys: distinct tags per quantity, per (seed, b, g) */
static uint64_t syn_key(uint64_t seed, uint64_t tag, uint64_t b, uint64_t g) {
  uint64_t k = syn_mix(seed * 0xD1B54A32D192ED03ULL + tag);
  k = syn_mix(k + (b + 1) * 0x8CB92BA72F3D8DD7ULL);
  k = syn_mix(k + (g + 1) * 0xABC98388FB8FAC03ULL);
  return k;
}

enum { TAG_MU = 1, TAG_NU, TAG_DRIFT, TAG_COMP, TAG_KZ, TAG_VZ, TAG_QT, TAG_QZ, TAG_CTX };

/* context lengths N_b ~ U{lo .. hi} */
void syn_ctx_lengths(uint64_t seed, int32_t batch, int64_t lo, int64_t hi, int64_t* out) {
  uint64_t key = syn_key(seed, TAG_CTX, 0, 0);
  for (int32_t b = 0; b < batch; ++b) out[b] = lo + (int64_t)(syn_u64(key, (uint64_t)b) % (uint64_t)(hi - lo + 1));
}


/*
 * Ragged batch: K, V are [sum_b G*N_b][128] bf16, sequence b occupying rows
 * [G * sum_{b'<b} N_b', ...) as G blocks of N_b rows (kv head major).
 * V and comp may be NULL.
 */
void syn_kv(uint64_t seed, int32_t batch, int32_t n_kv_heads, const int64_t* ctx, int32_t drift_seg, int32_t heavy,
            uint16_t* K, uint16_t* V, int32_t* comp) {
  int64_t nblk = (int64_t)batch * n_kv_heads;
  int64_t* base = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nblk + 1));
  base[0] = 0;
  for (int32_t b = 0; b < batch; ++b)
    for (int32_t g = 0; g < n_kv_heads; ++g) base[b * n_kv_heads + g + 1] = base[b * n_kv_heads + g] + ctx[b];
  /* mixture centres per block: mu, nu [nblk][M][128] (float copies of the drawn normals) */
  float* mu = (float*)malloc(sizeof(float) * (size_t)(nblk * SYN_M * SYN_D));
  float* nu = V ? (float*)malloc(sizeof(float) * (size_t)(nblk * SYN_M * SYN_D)) : NULL;
#pragma omp parallel for schedule(static)
  for (int64_t bm = 0; bm < nblk * SYN_M; ++bm) {
    int64_t i = bm / SYN_M, m = bm % SYN_M;
    int64_t b = i / n_kv_heads, g = i % n_kv_heads;
    uint64_t kmu = syn_key(seed, TAG_MU, (uint64_t)b, (uint64_t)g), knu = syn_key(seed, TAG_NU, (uint64_t)b, (uint64_t)g);
    for (int d = 0; d < SYN_D; ++d) {
      mu[bm * SYN_D + d] = (float)syn_normal(kmu, (uint64_t)(m * SYN_D + d));
      if (nu) nu[bm * SYN_D + d] = (float)syn_normal(knu, (uint64_t)(m * SYN_D + d));
    }
  }
  /* parallel over (block, token chunk) so a single long block still uses all cores */
  const int64_t CH = 4096;
  int64_t nwork = 0;
  for (int64_t i = 0; i < nblk; ++i) nwork += (base[i + 1] - base[i] + CH - 1) / CH;
  int64_t* wblk = (int64_t*)malloc(sizeof(int64_t) * (size_t)nwork);
  int64_t* wst = (int64_t*)malloc(sizeof(int64_t) * (size_t)nwork);
  int64_t w = 0;
  for (int64_t i = 0; i < nblk; ++i)
    for (int64_t t = 0; t < base[i + 1] - base[i]; t += CH) { wblk[w] = i; wst[w] = t; ++w; }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t wi = 0; wi < nwork; ++wi) {
    int64_t i = wblk[wi], t0 = wst[wi];
    int64_t b = i / n_kv_heads, g = i % n_kv_heads;
    int64_t n = base[i + 1] - base[i];
    int64_t cnt = (n - t0 < CH) ? n - t0 : CH;
    uint64_t kdr = syn_key(seed, TAG_DRIFT, (uint64_t)b, (uint64_t)g), kcp = syn_key(seed, TAG_COMP, (uint64_t)b, (uint64_t)g);
    uint64_t kkz = syn_key(seed, TAG_KZ, (uint64_t)b, (uint64_t)g), kvz = syn_key(seed, TAG_VZ, (uint64_t)b, (uint64_t)g);
    /* the drift walk up to the last segment this chunk touches */
    int64_t s_hi = (t0 + cnt - 1) / drift_seg;
    double* dr = (double*)malloc(sizeof(double) * SYN_D * (size_t)(s_hi + 1));
    for (int d = 0; d < SYN_D; ++d) dr[d] = 0.0;
    for (int64_t s = 1; s <= s_hi; ++s)
      for (int d = 0; d < SYN_D; ++d)
        dr[s * SYN_D + d] = dr[(s - 1) * SYN_D + d] + 0.05 * syn_normal(kdr, (uint64_t)(s * SYN_D + d));
    for (int64_t t = t0; t < t0 + cnt; ++t) {
      int64_t s = t / drift_seg;
      int64_t m = (int64_t)(syn_u64(kcp, (uint64_t)t) % SYN_M);
      int64_t row = base[i] + t;
      const float* mrow = mu + (i * SYN_M + m) * SYN_D;
      if (comp) comp[row] = (int32_t)m;
      for (int d = 0; d < SYN_D; ++d) {
        double noise = heavy ? syn_student4(kkz, (uint64_t)(t * SYN_D + d)) : syn_normal(kkz, (uint64_t)(t * SYN_D + d));
        K[row * SYN_D + d] = syn_bf16((double)mrow[d] + dr[s * SYN_D + d] + 0.3 * noise);
      }
      if (V) {
        const float* nrow = nu + (i * SYN_M + m) * SYN_D;
        for (int d = 0; d < SYN_D; ++d)
          V[row * SYN_D + d] = syn_bf16((double)nrow[d] + 0.3 * syn_normal(kvz, (uint64_t)(t * SYN_D + d)));
      }
    }
    free(dr);
  }
  free(mu);
  free(nu);
  free(wblk);
  free(wst);
  free(base);
}

/*
 * Queries for `steps` decode steps: q[step][b][h][128] bf16 = bf16(K_{t*}[g(h)] + 0.5 z),
 * with t* ~ U[0, N_b) drawn independently per (step, b, h). K is the array syn_kv wrote.
 * tstar (optional) receives the drawn positions [step][b][h].
 */
void syn_queries(uint64_t seed, int32_t steps, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                 const int64_t* ctx, const uint16_t* K, uint16_t* q, int64_t* tstar) {
  int64_t* rb = (int64_t*)malloc(sizeof(int64_t) * (size_t)(batch + 1));
  rb[0] = 0;
  for (int32_t b = 0; b < batch; ++b) rb[b + 1] = rb[b] + (int64_t)n_kv_heads * ctx[b];
  for (int32_t st = 0; st < steps; ++st)
    for (int32_t b = 0; b < batch; ++b)
      for (int32_t h = 0; h < n_q_heads; ++h) {
        int32_t g = (int32_t)((int64_t)h * n_kv_heads / n_q_heads);
        uint64_t kt = syn_key(seed, TAG_QT, (uint64_t)st * 65536u + (uint64_t)b, (uint64_t)h);
        uint64_t kz = syn_key(seed, TAG_QZ, (uint64_t)st * 65536u + (uint64_t)b, (uint64_t)h);
        int64_t t = (int64_t)(syn_u64(kt, 0) % (uint64_t)ctx[b]);
        if (tstar) tstar[((int64_t)st * batch + b) * n_q_heads + h] = t;
        const uint16_t* krow = K + (rb[b] + (int64_t)g * ctx[b] + t) * SYN_D;
        uint16_t* qrow = q + (((int64_t)st * batch + b) * n_q_heads + h) * SYN_D;
        for (int d = 0; d < SYN_D; ++d) qrow[d] = syn_bf16((double)syn_bf16_to_f(krow[d]) + 0.5 * syn_normal(kz, (uint64_t)d));
      }
  free(rb);
}

/* raw counter-based draws, exported for the generator's own distribution tests */
void syn_normals(uint64_t seed, int64_t n, double* out) {
  uint64_t key = syn_key(seed, 99, 0, 0);
  for (int64_t i = 0; i < n; ++i) out[i] = syn_normal(key, (uint64_t)i);
}
void syn_student4s(uint64_t seed, int64_t n, double* out) {
  uint64_t key = syn_key(seed, 98, 0, 0);
  for (int64_t i = 0; i < n; ++i) out[i] = syn_student4(key, (uint64_t)i);
}
