// build.hip -- query-independent phase of wave-index attention on gfx950:
// segmented k-means over the keys of every (sequence, kv head), then the
// cluster-sorted layout.
//
// RetroInfer summary page, section 2.A (segmented clustering): the sequence is
// cut into segments that are clustered independently at prefill. One k-means
// problem ("unit") per (sequence b, kv head g, segment s), enumerated in that
// order. Launch sequence, all on the caller's stream:
//   k_init                   seeded choice of K(s) tokens per unit (bf16 centroids, norms)
//   iters x { k_assign       nearest centroid on bf16 MFMA (32x32x16), fp32, and the
//                            binary64 decision where fp32 cannot separate the two best
//                            (k_assign_lds: centroids resident in LDS, up to 512 per
//                            segment; k_assign<true>: groups of 512 from registers)
//             k_sort         stable counting sort of each unit by cluster (LSD radix in LDS
//                            for segments of at most 16384 tokens); lists the round's
//                            large clusters
//             k_update       ordered fp32 member sums, correctly rounded means, bf16
//                            centroids and norms, the listed clusters' waves first; the
//                            last round also writes the sorted K/V, inv_perm and the
//                            ordered fp32 value sums }
#include <math.h>

#include <algorithm>

#include "common.h"
#include "internal.h"

namespace wave {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ unit lookup
// The batch of one build call. first[b] is the first segment of sequence b that the
// call clusters (0 for a whole build; ceil(N_b / seg_len): none): an append re-clusters
// only the segments from the first one it changes on. The call's input rows (K, V and
// the per-row workspaces) are ragged over M_b = N_b - first[b] * seg_len tokens per
// block: row of (b, g, t) = G * sum_{b'<b} M_b' + g * M_b + t - first[b] * seg_len,
// which is the layout of the index's own rows for a whole dense build.
struct BuildSeq : SeqArgs {
  int32_t ident;  // 1: a whole dense build, where cluster F of the call is index cluster F
  int32_t first[MAXB];
};

// N_b < 2^31 and seg_len <= 2^16: the division fits 32 bits
__device__ inline int64_t nseg_of(const BuildSeq& sa, int b) {
  return (int64_t)(((uint32_t)sa.N[b] + (uint32_t)sa.seg_len - 1u) / (uint32_t)sa.seg_len);
}

// x / d and x % d for non-negative x, d > 0, in 32 bits when both fit
__device__ inline void divmod64(int64_t x, int64_t d, int64_t& q, int64_t& r) {
  if (((uint64_t)x | (uint64_t)d) < (1ull << 32)) {
    const uint32_t qq = (uint32_t)x / (uint32_t)d;
    q = qq;
    r = (int64_t)((uint32_t)x - qq * (uint32_t)d);
  } else {
    q = x / d;
    r = x % d;
  }
}

// Clusters of at least BIG_MEMBERS members, listed by the sort so that k_update starts their
// waves first: a wave adds its cluster's members in order, so a large cluster that started
// late would set the launch's end (a whole dense build only).
constexpr int BIG_MEMBERS = 64;
constexpr int BIG_CAP = BUILD_BIG_CAP;  // listed per round at most (the first waves of k_update)
struct BigList {
  int32_t* cnt;    // [2]: clusters listed in the rounds of each parity
  int32_t* ids;    // [2][BIG_CAP]
  uint8_t* flag;   // [index clusters]: 1 if the cluster is in its round's list
  int32_t parity;  // this round's
};

// A sorting workgroup stages its large clusters in LDS and takes their slots of the list
// with one atomic (one per cluster on a single counter serialised: 21 -> 30 us a sort).
constexpr int BIG_WG = 256;  // large clusters staged per sorting workgroup at most
struct BigStage {
  int32_t n;
  int32_t id[BIG_WG];
};

// the sort's note of cluster F (index id) of n members: a large one is staged, any other
// one's flag cleared (a staged one's is written by big_flush)
__device__ inline void big_note(const BuildSeq& sa, const BigList& bl, BigStage& bs, int64_t F, int32_t n) {
  if (sa.ident && n >= BIG_MEMBERS) {
    const int i = atomicAdd(&bs.n, 1);
    if (i < BIG_WG) {
      bs.id[i] = (int32_t)F;
      return;
    }
  }
  bl.flag[F] = 0;
}

// one wave, after a barrier that follows every big_note of its workgroup: slots of the
// round's list for the staged clusters, their ids and flags
__device__ inline void big_flush(const BigList& bl, const BigStage& bs) {
  const int lane = threadIdx.x & 63;
  const int m = min(bs.n, BIG_WG);
  int base = 0;
  if (lane == 0 && m > 0) base = atomicAdd(&bl.cnt[bl.parity], m);
  base = __shfl(base, 0, 64);
  for (int i = lane; i < m; i += 64) {
    const int p = base + i, F = bs.id[i];
    const bool in = p < BIG_CAP;
    if (in) bl.ids[bl.parity * BIG_CAP + p] = F;
    bl.flag[F] = in ? 1 : 0;
  }
}

struct Unit {
  int b, g, s;
  int64_t row0;   // index row of the segment's first token
  int64_t brow;   // index row of the (b, g) block's token 0
  int64_t irow0;  // input row of the segment's first token
  int64_t gclu;   // index of the segment's first cluster
  int32_t L, Kc;  // segment length and clusters
  int32_t cbase;  // block-level id of the first cluster (s * K_s)
  int32_t tok0;   // segment start within the block (s * L_s)
  int64_t boff;   // first offsets entry of the block
  int32_t N, C;
};

// unit u of the call: units in (b, g, s) order, segments s >= first[b]
__device__ inline Unit unit_of(const BuildSeq& sa, int64_t u) {
  Unit r;
  int b = 0;
  int64_t irow = 0;
  for (;; ++b) {
    const int64_t nu = nseg_of(sa, b) - sa.first[b];
    if (u < sa.G * nu) break;
    u -= sa.G * nu;
    if (nu > 0) irow += (int64_t)sa.G * (sa.N[b] - (int64_t)sa.first[b] * sa.seg_len);
  }
  const SeqBase sb = seq_base(sa, b);
  const int64_t f = sa.first[b], nu = nseg_of(sa, b) - f, M = sb.N - f * sa.seg_len;
  int64_t gq, sr;
  divmod64(u, nu, gq, sr);
  r.b = b;
  r.g = (int)gq;
  r.s = (int)(f + sr);
  r.N = sb.N;
  r.C = sb.C;
  r.brow = sb.row + (int64_t)r.g * sb.NS;
  r.tok0 = r.s * sa.seg_len;
  r.row0 = r.brow + r.tok0;
  r.irow0 = irow + (int64_t)r.g * M + (r.tok0 - f * sa.seg_len);
  r.L = (int32_t)min((int64_t)sa.seg_len, (int64_t)r.N - r.tok0);
  r.Kc = seg_clusters(r.L, sa.seg_len, sa.K_s);
  r.cbase = r.s * sa.K_s;
  r.gclu = sb.clu + (int64_t)r.g * sb.CS + r.cbase;
  r.boff = sb.off + (int64_t)r.g * (sb.CS + 1);
  return r;
}

// cluster F of the call (the clusters of its units in (b, g, id) order) -> its block
struct CluRef {
  int64_t brow, bclu, boff;
  int64_t ib;  // input row of block position t is ib + t (t >= first[b] * seg_len)
  int64_t gF;  // index of the cluster
  int32_t j, N, C;
};

__device__ inline CluRef clu_of(const BuildSeq& sa, int64_t F) {
  int b = 0;
  int64_t irow = 0;
  for (;; ++b) {
    const int64_t nu = nseg_of(sa, b) - sa.first[b];
    const int64_t nc = nu > 0 ? sa.C[b] - (int64_t)sa.first[b] * sa.K_s : 0;
    if (F < sa.G * nc) break;
    F -= sa.G * nc;
    if (nu > 0) irow += (int64_t)sa.G * (sa.N[b] - (int64_t)sa.first[b] * sa.seg_len);
  }
  const SeqBase sb = seq_base(sa, b);
  const int64_t f = sa.first[b], nc = sb.C - f * sa.K_s, M = sb.N - f * sa.seg_len;
  int64_t gq, jr;
  divmod64(F, nc, gq, jr);
  const int g = (int)gq;
  CluRef r;
  r.j = (int32_t)(f * sa.K_s + jr);
  r.N = sb.N;
  r.C = sb.C;
  r.brow = sb.row + (int64_t)g * sb.NS;
  r.bclu = sb.clu + (int64_t)g * sb.CS;
  r.boff = sb.off + (int64_t)g * (sb.CS + 1);
  r.ib = irow + (int64_t)g * M - f * sa.seg_len;
  r.gF = r.bclu + r.j;
  return r;
}


// ------------------------------------------------------------------ k_init
// Stream key of the unit (b, g, s): b*2^56 + g*2^40 + s*2^16 (mod 2^64). Keyed by the
// segment's coordinates, a segment draws the same initial tokens whatever the number
// of segments around it, so an index grown by appending segments equals one built
// over the longer context (segments are clustered independently, RetroInfer page,
// section 2.A).
__device__ __forceinline__ uint64_t seed_key(int b, int g, int s) {
  return ((uint64_t)(uint32_t)b << 56) + ((uint64_t)(uint32_t)g << 40) + ((uint64_t)(uint32_t)s << 16);
}

// One workgroup per unit. The i-th SplitMix64 draw of the unit with key k is
// mix(seed + GAMMA*(k+1) + GAMMA*(i+1)); the draws do not depend on the
// shuffle, so they are taken in parallel, and so is the outcome of the K(s)
// swaps of the partial Fisher-Yates shuffle of [0, L) (below). Centroid i
// becomes the fp32 copy of key row idx[i]; its bf16 rounding is the key itself
// and its squared norm is summed here too.
constexpr int INIT_THREADS = 1024;

__global__ __launch_bounds__(INIT_THREADS) void k_init(BuildSeq sa, uint64_t seed, const uint16_t* __restrict__ K,
                                                       float* __restrict__ cent, uint16_t* __restrict__ chat,
                                                       float* __restrict__ norm, BigList bl) {
  if (blockIdx.x == 0 && threadIdx.x < 2) bl.cnt[threadIdx.x] = 0;  // the first round's lists
  extern __shared__ uint8_t smem[];
  const Unit U = unit_of(sa, blockIdx.x);
  // LDS (all of it dynamic: the attribute allows the whole 160 KB): the pair count, the
  // draws, the (position, step) pairs a chain can meet, two bitmaps over the positions
  // (drawn at least once, more than once), the chosen rows (16-bit)
  const int Kc = U.Kc, nbw = (U.L + 31) >> 5;
  int32_t& ntab = *reinterpret_cast<int32_t*>(smem);
  int32_t* jsel = reinterpret_cast<int32_t*>(smem + 16);
  int2* tab = reinterpret_cast<int2*>(jsel + ((Kc + 3) & ~3));
  uint32_t* seen1 = reinterpret_cast<uint32_t*>(tab + Kc);
  uint32_t* seen2 = seen1 + nbw;
  uint16_t* idx = reinterpret_cast<uint16_t*>(seen2 + nbw);
  const uint64_t st0 = seed + GAMMA * (seed_key(U.b, U.g, U.s) + 1);
  for (int i = threadIdx.x; i < nbw; i += blockDim.x) {
    seen1[i] = 0u;
    seen2[i] = 0u;
  }
  if (threadIdx.x == 0) ntab = 0;
  for (int i = threadIdx.x; i < Kc; i += blockDim.x) {
    const uint64_t r = sm64_mix(st0 + GAMMA * (uint64_t)(i + 1));
    jsel[i] = i + (int32_t)(r % (uint64_t)(U.L - i));
  }
  __syncthreads();
  // The swaps, all positions at once. Step i swaps positions i and jsel[i] >= i, so position
  // t < Kc is final after step t and holds what position jsel[t] held just before it: jsel[t]
  // itself unless an earlier step s drew it too (jsel[s] == jsel[t]); then, for the last such
  // s, what position s held just before step s, found the same way (a position below Kc that
  // an earlier step drew). Such chains need a position drawn twice: the positions drawn more
  // than once are marked, the draws on them and on positions below Kc (the only draws a chain
  // can meet) listed, and a thread follows its positions' chains through that short list.
  for (int i = threadIdx.x; i < Kc; i += blockDim.x) {
    const int j = jsel[i];
    const uint32_t bit = 1u << (j & 31);
    if (atomicOr(&seen1[j >> 5], bit) & bit) atomicOr(&seen2[j >> 5], bit);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < Kc; i += blockDim.x) {
    const int j = jsel[i];
    if (j < Kc || ((seen2[j >> 5] >> (j & 31)) & 1u)) {
      tab[atomicAdd(&ntab, 1)] = make_int2(j, i);
    }
  }
  __syncthreads();
  const int nt = ntab;
  for (int t = threadIdx.x; t < Kc; t += blockDim.x) {
    int p = jsel[t], cur = t;
    if ((seen2[p >> 5] >> (p & 31)) & 1u) {
      for (;;) {
        int s = -1;  // the last step before cur that drew p
        for (int e0 = 0; e0 < nt; e0 += 8) {
          int2 pr[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) pr[u] = tab[min(e0 + u, nt - 1)];  // repeats are harmless
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (pr[u].x == p && pr[u].y < cur && pr[u].y > s) s = pr[u].y;
        }
        if (s < 0) break;
        p = s;
        cur = s;
      }
    }
    idx[t] = (uint16_t)p;
  }
  __syncthreads();
  // (centroid i, 16-byte chunk c): 16 lanes per centroid, 8 rows in flight per thread
  const int l16 = threadIdx.x & 15;
  constexpr int UI = 8;
  for (int i0 = threadIdx.x >> 4; i0 < U.Kc; i0 += (INIT_THREADS / 16) * UI) {
    u32x4 v[UI];
#pragma unroll
    for (int u = 0; u < UI; ++u) {
      const int i = min(i0 + u * (INIT_THREADS / 16), U.Kc - 1);
      v[u] = *reinterpret_cast<const u32x4*>(K + (U.irow0 + idx[i]) * D + l16 * 8);
    }
#pragma unroll
    for (int u = 0; u < UI; ++u) {
      const int i = i0 + u * (INIT_THREADS / 16);
      float f[8];
      float s2 = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = bf16_lo(v[u][e]);
        f[2 * e + 1] = bf16_hi(v[u][e]);
        s2 = fmaf(f[2 * e], f[2 * e], s2);
        s2 = fmaf(f[2 * e + 1], f[2 * e + 1], s2);
      }
      s2 = row_sum16(s2);
      if (i < U.Kc) {
        float* cr = cent + (U.gclu + i) * D + l16 * 8;
        *reinterpret_cast<float4*>(cr) = make_float4(f[0], f[1], f[2], f[3]);
        *reinterpret_cast<float4*>(cr + 4) = make_float4(f[4], f[5], f[6], f[7]);
        *reinterpret_cast<u32x4*>(chat + (U.gclu + i) * D + l16 * 8) = v[u];
        if (l16 == 0) norm[U.gclu + i] = s2;
      }
    }
  }
}

// ------------------------------------------------------------------ k_assign (bf16 MFMA)
// For a key x and bf16 centroids c_j the nearest centroid maximises
// f_j = x.c_j - |c_j|^2 / 2. D[centroid][token] = C . X^T is computed with
// v_mfma_f32_32x32x16_bf16. A workgroup is 4 waves, one per SIMD, so each wave
// has the whole register file: it keeps 128 centroid rows (four 32-row A
// tiles, all 128 dims) resident, the token tiles (B operand) stream through
// LDS, and the accumulator starts at -|c_j|^2/2. A lane of a 32x32 result holds
// one token (column) and 16 centroid rows of its A tile.
//
// Software pipeline: the 32 MFMAs of a 32-token block run as two halves of 16
// (A tiles 0-1, then 2-3); while one half runs on the matrix core, the same
// wave selects over the other half's results on the vector ALU, so one wave
// keeps both pipes busy. Units with more than 512 clusters (MULTI) take the
// centroids in groups of 512, one pass over the range's token tiles per group, the
// running best / second best / id of every token kept in LDS between passes.
//
// Selection per lane: the 6-bit position of each of its 64 values is written
// into the value's low mantissa bits, so the best and second best come from
// a tournament of triples (max3/med3) and the best's position is read back from its bits.
// The packing moves a value by less than 2^-17 |f|. The best, its position and
// the second best are then merged across the two half-waves and the 4 waves.
// When the gap between best and second best is within 2^-14 (|x| R + R^2),
// R = max_j |c_j|, plus 2^-100 for denormal flushing, the token goes to the
// exact binary64 decision at the end of the workgroup: each value is off by less
// than the fp32 accumulation error of a 128-term dot product and a norm (each
// below 2^-17 of those magnitudes) plus the packing error, i.e. by less than
// 2^-16 (|x| R + R^2), so the margin is twice what two values can move and
// every token not sent there has the exact argmin.

// scheduling of one pipeline step (see tile() in k_assign): nds LDS reads, then 16 x
// (1 MFMA, 6 vector-ALU operations), the first nvm of them followed by one global load;
// nothing moves across the step's end
#define AS_STEP_V(nds, nvm)                                                       \
  do {                                                                            \
    if ((nds) > 0) __builtin_amdgcn_sched_group_barrier(0x100, (nds), 0);         \
    _Pragma("unroll") for (int i_ = 0; i_ < 16; ++i_) {                           \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          \
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);                          \
      if (i_ < (nvm)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);         \
    }                                                                             \
    __builtin_amdgcn_sched_barrier(0);                                            \
  } while (0)
#define AS_STEP(nds) AS_STEP_V(nds, 0)

constexpr int AS_WAVES = 4;
constexpr int AS_THREADS = AS_WAVES * 64;
constexpr int AS_TT = 128;                   // tokens per LDS tile (4 blocks of 32)
constexpr int AS_CPW = 128;                  // centroids per wave
constexpr int AS_GROUP = AS_WAVES * AS_CPW;  // centroids per pass
constexpr int AS_MAXTPW = 8192;              // tokens per workgroup at most (the near-tie list fits a tile buffer)
constexpr int AS_MAXTPW_M = 4096;            // the same with more than AS_GROUP clusters (the running bests fit LDS)

// Token tiles are double buffered and loaded straight into LDS (global_load_lds,
// 16 bytes per lane); one barrier per tile. The work of a tile's start (the
// previous tile's decisions, this tile's key norms) is straight-line code, so it
// overlaps the first MFMAs of the tile. The next tile's 8 loads per wave go out two
// at a time between the MFMAs of the first four steps: issued together at the tile's
// start, the 32 loads of the workgroup queued behind each other in the address unit
// and held the issuing waves back (about 5% of the launch).
struct AssignLds {
  u32x4 tile[2][AS_TT * 16];         // token rows, 16-byte chunk c of row t stored at slot t*16 + (c ^ (t & 15))
  float red[2][AS_WAVES][AS_TT][3];  // per tile buffer and wave: best, second best, winner's position (bits)
  // near-tie flag of token i of the range at ambf[AS_TT + i]; the first AS_TT bytes
  // take the flags of the empty decision pass before the first tile
  uint8_t ambf[AS_MAXTPW + AS_TT];
  float4 nrm[WAVE_MAX_CLUSTERS_PER_SEG / 4];  // |c_j|^2 of the unit's centroids
  float part[AS_MAXTPW_M + AS_TT][3]; // more than AS_GROUP clusters: running best, second best, id per token
                                     // of the range over the centroid groups so far (+ spare slots)
  unsigned long long fd[32];         // exact decision: per token the least D_j (bits), then its id
  int32_t fj[32];
  int32_t scan[AS_THREADS];
  float rmx[AS_WAVES];               // per wave: max |c_j|^2
};

// Workgroups per unit: ceil(L / tpw) with tpw tokens per workgroup (a multiple of
// AS_TT chosen by the host); units in (b, g, s) order, segments s >= first[b].
__device__ inline void assign_wg_map(const BuildSeq& sa, int tpw, int w, Unit& U, int& tok_begin) {
  int64_t u = 0;
  for (int b = 0;; ++b) {
    const int64_t N = sa.N[b];
    const int64_t nseg = (N + sa.seg_len - 1) / sa.seg_len, nu = nseg - sa.first[b];
    const int64_t last = N - (nseg - 1) * sa.seg_len;
    const int wf = (sa.seg_len + tpw - 1) / tpw, wl = (int)((last + tpw - 1) / tpw);
    const int64_t per_g = nu > 0 ? (nu - 1) * wf + wl : 0;
    if (w < sa.G * per_g) {
      const int g = (int)(w / per_g);
      const int64_t r = w % per_g;
      int64_t s = r / wf;
      int64_t k = r % wf;
      if (s >= nu - 1) { s = nu - 1; k = r - (nu - 1) * wf; }
      U = unit_of(sa, u + (int64_t)g * nu + s);
      tok_begin = (int)(k * tpw);
      return;
    }
    w -= (int)(sa.G * per_g);
    u += sa.G * nu;
  }
}

// value with its position p (0..63) in the low 6 mantissa bits
__device__ __forceinline__ float pack6(float v, int p) {
  return __uint_as_float((__float_as_uint(v) & ~63u) | (unsigned)p);
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Best and second best of the 32 values v and a running pair b1 >= b2 (FRESH: none yet),
// by a tournament of triples: a triple's maximum goes up a level, its median is kept.
// The second best overall is the median of the triple where its path meets the best's
// (the best and it are the two largest of that triple), and no median exceeds it (a
// median is below its triple's maximum), so it is the largest median; the running pair
// enters as one more player (b1) and one more median (b2). 40 operations for 32 values,
// where folding each triple into the running pair takes 54.
template <bool FRESH>
__device__ __forceinline__ void top2_tree32(const float (&v)[32], float& b1, float& b2) {
  float up[12], md[17];
#pragma unroll
  for (int k = 0; k < 10; ++k) {
    up[k] = max3f(v[3 * k], v[3 * k + 1], v[3 * k + 2]);
    md[k] = __builtin_amdgcn_fmed3f(v[3 * k], v[3 * k + 1], v[3 * k + 2]);
  }
  up[10] = v[30];
  up[11] = v[31];
  float u2[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    u2[k] = max3f(up[3 * k], up[3 * k + 1], up[3 * k + 2]);
    md[10 + k] = __builtin_amdgcn_fmed3f(up[3 * k], up[3 * k + 1], up[3 * k + 2]);
  }
  const float u3 = max3f(u2[0], u2[1], u2[2]);
  md[14] = __builtin_amdgcn_fmed3f(u2[0], u2[1], u2[2]);
  constexpr int n = FRESH ? 16 : 17;
  if constexpr (FRESH) {
    b1 = fmaxf(u3, u2[3]);
    md[15] = fminf(u3, u2[3]);
  } else {
    md[15] = __builtin_amdgcn_fmed3f(u3, u2[3], b1);
    md[16] = b2;
    b1 = max3f(u3, u2[3], b1);
  }
  float s = max3f(md[0], md[1], md[2]);
#pragma unroll
  for (int k = 3; k + 2 <= n; k += 2) s = max3f(s, md[k], md[k + 1]);
  if constexpr ((n - 3) % 2 == 1) s = fmaxf(s, md[n - 1]);
  b2 = s;
}

template <bool MULTI>
__global__ __launch_bounds__(AS_THREADS, 1) void k_assign(BuildSeq sa, int tpw, const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ chat,
                                                          const float* __restrict__ norm,
                                                          int32_t* __restrict__ assign, float* __restrict__ xn2,
                                                          int first) {
  extern __shared__ uint8_t smem[];
  AssignLds& S = *reinterpret_cast<AssignLds*>(smem);
  Unit U;
  int tb0;
  assign_wg_map(sa, tpw, xcd_linear(blockIdx.x, gridDim.x), U, tb0);
  const int nrow = min(tpw, U.L - tb0);  // rows of the workgroup's range
  const int ntiles = (nrow + AS_TT - 1) / AS_TT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, h = lane >> 5, col = lane & 31;
  const uint16_t* Kr = K + (U.irow0 + tb0) * D;  // first input row of the range
  // rows of tile T into buffer bi: wave wv fills slots [(8 wv + m) * 64, +64), m < 8; lane i of
  // a load writes slot base + i, i.e. token t = slot / 16, chunk (slot % 16) ^ (t % 16).
  // Rows past the range end repeat its last row: their results equal that row's.
  auto issue_m = [&](int T, int bi, int m) {
    const int s0 = (wv * 8 + m) * 64;
    const int slot = s0 + lane;
    const int t = slot >> 4, c = (slot & 15) ^ (t & 15);
    const int tt = min(T * AS_TT + t, nrow - 1);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(Kr + tt * D + c * 8),
                                     (__attribute__((address_space(3))) void*)(&S.tile[bi][s0]), 16, 0, 0);
  };
  auto issue = [&](int T, int bi) {
#pragma unroll
    for (int m = 0; m < 8; ++m) issue_m(T, bi, m);
  };
  issue(0, 0);
  const int ngroups = (U.Kc + AS_GROUP - 1) / AS_GROUP;
  // A fragments live in the accumulation registers (AGPRs), which the MFMA reads as
  // its A operand directly; the architectural VGPRs hold accumulators, B fragments and
  // the selection. The empty asm only fixes the register class of its tied operand.
  // All 32 loads are issued before the first move into the accumulation registers: moved
  // one by one, each load waited for its own round trip (32 serial round trips, 13 us of
  // a 128K launch).
  u32x4 A[4][8];
  floatx16 nh[4];
  auto load_a = [&](int grp) {
    const int cb = grp * AS_GROUP + wv * AS_CPW;
    u32x4 ld[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rc = min(cb + r * 32 + col, U.Kc - 1);
#pragma unroll
      for (int st = 0; st < 8; ++st)
        ld[r][st] = *reinterpret_cast<const u32x4*>(chat + (U.gclu + rc) * D + (2 * st + h) * 8);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool in = cb + r * 32 + col < U.Kc;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const u32x4 z = in ? ld[r][st] : u32x4{0u, 0u, 0u, 0u};
        asm volatile("" : "=a"(A[r][st]) : "0"(z));
      }
    }
  };
  // accumulator start -|c_j|^2 / 2 of the rows a lane's results hold (from the LDS copy)
  auto load_nh = [&](int grp) {
    const int cb = grp * AS_GROUP + wv * AS_CPW;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int r0 = cb + r * 32 + 8 * a4 + 4 * h;
        const float4 nv = S.nrm[r0 >> 2];
        const float f[4] = {nv.x, nv.y, nv.z, nv.w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
          // rows past the unit's clusters: a finite floor that every real value beats
          nh[r][4 * a4 + k] = r0 + k < U.Kc ? -0.5f * f[k] : -__FLT_MAX__;
      }
  };
  load_a(0);
  // the unit's squared centroid norms into LDS, and their maximum (all are >= 0)
  {
    float m = 0.f;
    float* nr = reinterpret_cast<float*>(S.nrm);
    for (int j = tid; j < U.Kc; j += AS_THREADS) {
      const float v = norm[U.gclu + j];
      nr[j] = v;
      m = fmaxf(m, v);
    }
    m = wave_max(m);
    if (lane == 0) S.rmx[wv] = m;
  }
  // red buffer 1 holds the empty decision pass before the first tile
  for (int i = tid; i < AS_WAVES * AS_TT; i += AS_THREADS) {
    float* rd = S.red[1][i / AS_TT][i % AS_TT];
    rd[0] = -INFINITY;
    rd[1] = -INFINITY;
    rd[2] = 0.f;
  }
  __syncthreads();
  load_nh(0);
  const float R2 = fmaxf(fmaxf(S.rmx[0], S.rmx[1]), fmaxf(S.rmx[2], S.rmx[3])), R = __builtin_amdgcn_sqrtf(R2);
  // Decisions for tile Tm (Tm = -1: the empty pass, whose stores go to rows of tile 0 and
  // are overwritten by the real ones): wave wv takes tokens 32 wv .. 32 wv + 31, both
  // lane halves the same token; merge the 4 waves, store, flag near ties. x2: |x|^2.
  auto reduce = [&](int Tm, float x2, int grp, bool last) {
    const int bi = Tm & 1;
    const int tk = wv * 32 + col;
    float b1 = S.red[bi][0][tk][0], b2 = S.red[bi][0][tk][1];
    uint32_t meta = __float_as_uint(S.red[bi][0][tk][2]);
    int wbest = 0;
#pragma unroll
    for (int w2 = 1; w2 < AS_WAVES; ++w2) {
      const float o1 = S.red[bi][w2][tk][0], o2 = S.red[bi][w2][tk][1];
      const uint32_t om = __float_as_uint(S.red[bi][w2][tk][2]);
      const bool take = o1 > b1;
      b2 = fmaxf(fminf(b1, o1), fmaxf(b2, o2));
      b1 = fmaxf(b1, o1);
      meta = take ? om : meta;
      wbest = take ? w2 : wbest;
    }
    // id of the winner: group, wave, A tile and row i of its 32x32 block, lane half
    const int p = (int)(meta & 63u), hw = (int)((meta >> 6) & 1u), gw = (int)(meta >> 7);
    int best_id = gw * AS_GROUP + wbest * AS_CPW + (p >> 4) * 32 + 8 * ((p & 15) >> 2) + 4 * hw + (p & 3);
    const int tr = Tm * AS_TT + tk;
    if constexpr (MULTI) {
      // running best over the centroid groups (the empty pass before tile 0 uses spare slots)
      float* pp = S.part[Tm < 0 ? AS_MAXTPW_M + tk : tr];
      if (grp > 0) {
        const float q1 = pp[0], q2 = pp[1];
        const int qid = __float_as_int(pp[2]);
        const bool keep = !(b1 > q1);  // equal bests: a gap of 0, decided in binary64
        b2 = fmaxf(fminf(q1, b1), fmaxf(q2, b2));
        b1 = fmaxf(q1, b1);
        best_id = keep ? qid : best_id;
      }
      pp[0] = b1;
      pp[1] = b2;
      pp[2] = __int_as_float(best_id);
      if (!last) return;
    }
    assign[U.row0 + tb0 + min(max(tr, tk), nrow - 1)] = U.cbase + best_id;
    const float margin = 0x1p-14f * (__builtin_amdgcn_sqrtf(x2) * R + R2) + 0x1p-100f;
    // also undecided: a best at the floor of the padding rows, and keys or centroids so large
    // that a value may leave the fp32 range (|f| < |x| R + R^2 / 2 < 2^114 otherwise)
    const bool near = !(b1 - b2 > margin) || !(b1 > -0x1p127f) || !(margin < 0x1p100f);
    S.ambf[AS_TT + tr] = (near && tr < nrow) ? 1 : 0;
  };
  // |x|^2 of this wave's tokens of a tile: lane (col, h) sums the 64 dims of half h
  auto xnorm = [&](int bi) {
    const int t = wv * 32 + col;
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const u32x4 w = S.tile[bi][t * 16 + ((8 * h + q) ^ (t & 15))];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // bit-cast a named scalar: hipcc lowers a bit-cast of a vector element
        // expression inside a loop to element 0 for every iteration
        const uint32_t we = w[e];
        const bf16x2_t x = __builtin_bit_cast(bf16x2_t, we);
        s = __builtin_amdgcn_fdot2_f32_bf16(x, x, s, false);
      }
    }
    return s + swap32(s);
  };
  // B fragments of 32-token block tb of a tile: lane (col, h) holds chunks 2 st + h of token col
  auto load_b = [&](const u32x4* tl, int tb, bf16x8_t (&Bv)[8]) {
    const int t = tb * 32 + col;
#pragma unroll
    for (int st = 0; st < 8; ++st) Bv[st] = __builtin_bit_cast(bf16x8_t, tl[t * 16 + ((2 * st + h) ^ (t & 15))]);
  };
  // the 16 MFMAs of A tiles 2 hb, 2 hb + 1 against one token block
  auto mma_half = [&](const bf16x8_t (&Bv)[8], int hb, floatx16 (&acc)[2]) {
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, A[2 * hb + r][st]), Bv[st],
                                                         st == 0 ? nh[2 * hb + r] : acc[r], 0, 0, 0);
  };
  // fold the 32 values of a half block into (b1, b2); positions 32 hb + 16 r + i
  auto sel_half = [&](floatx16 (&acc)[2], int hb, float& b1, float& b2) {
    float v[32];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) v[16 * r + i] = pack6(acc[r][i], 32 * hb + 16 * r + i);
    if (hb == 0)
      top2_tree32<true>(v, b1, b2);
    else
      top2_tree32<false>(v, b1, b2);
  };
  // merge the two half-waves (the lanes of one token) and store the wave's result for the
  // block. Both halves store the same values, up to exact ties, which need no order here:
  // their gap is 0, so the token is re-decided in binary64.
  auto finish = [&](int tb, int bi, int grp, float b1, float b2) {
    const float ob1 = swap32(b1), ob2 = swap32(b2);
    const bool take = ob1 > b1;
    const float nb2 = fmaxf(fminf(b1, ob1), fmaxf(b2, ob2));
    const float nb1 = fmaxf(b1, ob1);
    // the winner's position: its packed 6 bits, its half, the centroid group
    const uint32_t meta = ((uint32_t)grp << 7) | ((uint32_t)(take ? h ^ 1 : h) << 6) | (__float_as_uint(nb1) & 63u);
    float* rd = S.red[bi][wv][tb * 32 + col];
    rd[0] = nb1;
    rd[1] = nb2;
    rd[2] = __uint_as_float(meta);
  };
  // one tile against one centroid group: 8 half-block steps, the selection of step j - 1
  // next to the MFMAs of step j. Each step is its own scheduling region: first the LDS
  // reads of a later block's B fragments, then one MFMA followed by up to 6 vector-ALU
  // operations, 16 times (the matrix core takes 32 cycles per MFMA, in which this wave
  // issues the selection work). Steps 1-4 also issue the loads of tile Tn into the other
  // buffer, which every wave finished reading before this tile's barrier.
  auto tile = [&](int bi, int grp, int Tn) {
    const u32x4* tl = S.tile[bi];
    bf16x8_t B0[8], B1[8];
    floatx16 accA[2], accB[2];
    float b1 = -INFINITY, b2 = -INFINITY;
    issue_m(Tn, bi ^ 1, 0);
    issue_m(Tn, bi ^ 1, 1);
    load_b(tl, 0, B0);
    load_b(tl, 1, B1);
    mma_half(B0, 0, accA);
    AS_STEP_V(16, 2);
    issue_m(Tn, bi ^ 1, 2);
    issue_m(Tn, bi ^ 1, 3);
    mma_half(B0, 1, accB);
    sel_half(accA, 0, b1, b2);
    AS_STEP_V(0, 2);
    issue_m(Tn, bi ^ 1, 4);
    issue_m(Tn, bi ^ 1, 5);
    mma_half(B1, 0, accA);
    sel_half(accB, 1, b1, b2);
    finish(0, bi, grp, b1, b2);
    AS_STEP_V(0, 2);
    issue_m(Tn, bi ^ 1, 6);
    issue_m(Tn, bi ^ 1, 7);
    load_b(tl, 2, B0);
    mma_half(B1, 1, accB);
    sel_half(accA, 0, b1, b2);
    AS_STEP_V(8, 2);
    mma_half(B0, 0, accA);
    sel_half(accB, 1, b1, b2);
    finish(1, bi, grp, b1, b2);
    AS_STEP(0);
    load_b(tl, 3, B1);
    mma_half(B0, 1, accB);
    sel_half(accA, 0, b1, b2);
    AS_STEP(8);
    mma_half(B1, 0, accA);
    sel_half(accB, 1, b1, b2);
    finish(2, bi, grp, b1, b2);
    AS_STEP(0);
    mma_half(B1, 1, accB);
    sel_half(accA, 0, b1, b2);
    AS_STEP(0);
    sel_half(accB, 1, b1, b2);
    finish(3, bi, grp, b1, b2);
  };
  // one pass of the range's tiles against centroid group grp; the decisions in the last.
  // The keys' |x|^2 (for the margins) are the same in every round: the first round's first
  // pass computes them from the tiles in LDS and stores them; later passes load them with
  // the tile loads, a tile ahead (the serial LDS reads of the computation cost a tenth of
  // the launch).
  auto xrow = [&](int T) { return U.irow0 + tb0 + min(T * AS_TT + wv * 32 + col, nrow - 1); };
  auto pass = [&](int grp, bool last) {
    const bool fresh = first && grp == 0;
    float xn = 0.f;                                 // |x|^2 of this wave's tokens of the previous tile
    float xc = fresh ? 0.f : xn2[xrow(0)];          // and of tile T, loaded with it
    for (int T = 0; T < ntiles; ++T) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of tile T have landed
      __syncthreads();  // tile T is in LDS; red[(T - 1) & 1] is complete
      const int bi = T & 1;
      const float xnext = fresh ? 0.f : xn2[xrow(min(T + 1, ntiles - 1))];
      reduce(T - 1, xn, grp, last);
      if (fresh) {
        xn = xnorm(bi);
        if (h == 0 && T * AS_TT + wv * 32 + col < nrow) xn2[xrow(T)] = xn;
      } else {
        xn = xc;
      }
      xc = xnext;
      // the next tile's loads go into the buffer of tile T - 1, which every wave has
      // finished; after the last tile a harmless reload of it
      tile(bi, grp, min(T + 1, ntiles - 1));
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the trailing reload has landed: the buffers are free
    __syncthreads();
    reduce(ntiles - 1, xn, grp, last);
    __syncthreads();
  };
  if (!MULTI) {
    pass(0, true);
  } else {
    // more than AS_GROUP clusters: a pass per group of them, the token tiles streamed again
    for (int grp = 0; grp < ngroups; ++grp) {
      if (grp > 0) {
        load_a(grp);
        load_nh(grp);
        issue(0, 0);
      }
      pass(grp, grp == ngroups - 1);
    }
  }
  // near-tie tokens: flags counted per thread (4 per word) and a workgroup scan
  const uint32_t* fw = reinterpret_cast<const uint32_t*>(S.ambf + AS_TT);
  const int nw = ntiles * (AS_TT / 4), per = (nw + AS_THREADS - 1) / AS_THREADS;
  const int w0 = min(tid * per, nw), w1 = min(w0 + per, nw);
  int cnt = 0;
  for (int i = w0; i < w1; ++i) cnt += __builtin_popcount(fw[i]);
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) S.scan[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w2 = 0; w2 < AS_WAVES; ++w2) {
    const int c = S.scan[w2];
    before += w2 < wv ? c : 0;
    total += c;
  }
  if (total == 0) return;
  // Exact decision in the workgroup, 32 tokens at a time: their rows go through the
  // MFMAs again, group by group (the last pass's group first, its centroids are still
  // loaded); every centroid within 2^-14 (|x| R + R^2) + 2^-40 (|x| + R)^2 + 2^-100 of
  // the best fp32 value so far (two fp32 errors and two binary64 rounding errors of the
  // sums; the best so far is at most the final best, so no centroid within the window of
  // the final best is missed) gets D_j = sum_i (x_i - c_j,i)^2 in binary64, dims in
  // order, each operation rounded; argmin with the lowest id on ties.
  int32_t* fl = reinterpret_cast<int32_t*>(S.tile[1]);  // the list (the buffer is free now)
  {
    int pos = before + incl - cnt;
    for (int i = w0; i < w1; ++i) {
      uint32_t f = fw[i];
      while (f != 0u) {
        const int b = __builtin_ctz(f);
        f &= f - 1u;
        fl[pos++] = 4 * i + (b >> 3);
      }
    }
  }
  __syncthreads();
  for (int f0 = 0; f0 < total; f0 += 32) {
    const int nb = min(32, total - f0);
    // rows of the batch into buffer 0 as block 0 of a tile; past nb the last row again
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int slot = tid + AS_THREADS * m;
      const int t = slot >> 4, c = (slot & 15) ^ (t & 15);
      S.tile[0][slot] = *reinterpret_cast<const u32x4*>(Kr + fl[f0 + min(t, nb - 1)] * D + c * 8);
    }
    if (tid < 32) {
      S.fd[tid] = ~0ull;
      S.fj[tid] = 0x7FFFFFFF;
    }
    __syncthreads();
    bf16x8_t B[8];
    load_b(S.tile[0], 0, B);
    // |x|^2 of token col in fp32
    float s2 = 0.f;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const u32x4 w = __builtin_bit_cast(u32x4, B[st]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t we = w[e];
        const float a = bf16_lo(we), b = bf16_hi(we);
        s2 = fmaf(a, a, s2);
        s2 = fmaf(b, b, s2);
      }
    }
    s2 += swap32(s2);
    const float X = sqrtf(s2);
    const float win = 0x1p-14f * (X * R + R2) + 0x1p-40f * (X + R) * (X + R) + 0x1p-100f;
    const u32x4* xr = S.tile[0] + col * 16;
    float M = -INFINITY;  // best fp32 value of token col so far
    double best = INFINITY;
    int bj = 0x7FFFFFFF;
    for (int gi = 0; gi < ngroups; ++gi) {
      const int grp = ngroups - 1 - gi;
      if (gi > 0) {
        load_a(grp);
        load_nh(grp);
      }
      floatx16 a0[2], a1[2];
      mma_half(B, 0, a0);
      mma_half(B, 1, a1);
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(a0[r][i], a1[r][i]));
      mx = fmaxf(mx, swap32(mx));
      if (h == 0) S.red[0][wv][col][0] = mx;
      __syncthreads();
      M = fmaxf(M, fmaxf(fmaxf(S.red[0][0][col][0], S.red[0][1][col][0]),
                         fmaxf(S.red[0][2][col][0], S.red[0][3][col][0])));
      __syncthreads();  // red[0] is read before the next group writes it
      const float thr = M - win;
      uint64_t cm = 0ull;  // candidates among this lane's 64 values: bit 32 hb + 16 r + i
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          // a NaN window or value (fp32 overflow) makes every centroid a candidate
          cm |= (uint64_t)!(a0[r][i] < thr) << (16 * r + i);
          cm |= (uint64_t)!(a1[r][i] < thr) << (32 + 16 * r + i);
        }
      while (cm != 0ull) {
        const int q = __builtin_ctzll(cm);
        cm &= cm - 1ull;
        const int i = q & 15;
        const int j = grp * AS_GROUP + wv * AS_CPW + 32 * (q >> 4) + 8 * (i >> 2) + 4 * h + (i & 3);
        if (j >= U.Kc) continue;
        const u32x4* cj = reinterpret_cast<const u32x4*>(chat + (U.gclu + j) * D);
        double acc = 0.0;
        for (int c = 0; c < 16; ++c) {
          const u32x4 xv = xr[c ^ (col & 15)], cv = cj[c];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t xe = xv[e], ce = cv[e];
            const double d0 = __dsub_rn((double)bf16_lo(xe), (double)bf16_lo(ce));
            acc = __dadd_rn(acc, __dmul_rn(d0, d0));
            const double d1 = __dsub_rn((double)bf16_hi(xe), (double)bf16_hi(ce));
            acc = __dadd_rn(acc, __dmul_rn(d1, d1));
          }
        }
        if (acc < best || (acc == best && j < bj)) {
          best = acc;
          bj = j;
        }
      }
    }
    // D >= 0: its bits order as its values
    const unsigned long long bd = (unsigned long long)__double_as_longlong(best);
    if (bj != 0x7FFFFFFF) atomicMin(&S.fd[col], bd);
    __syncthreads();
    if (bj != 0x7FFFFFFF && bd == S.fd[col]) atomicMin(&S.fj[col], bj);
    __syncthreads();
    if (tid < nb) assign[U.row0 + tb0 + fl[f0 + tid]] = U.cbase + S.fj[tid];
    __syncthreads();
    if (MULTI && f0 + 32 < total) {  // the next batch starts from the last group again
      load_a(ngroups - 1);
      load_nh(ngroups - 1);
    }
  }
}

// ------------------------------------------------------------------ k_assign_lds
// Units of at most 512 clusters. The unit's bf16 centroids stay in LDS for the whole
// launch (128 KB at 512 clusters, chunk-major: 16-byte chunk c of row j at slot 512 c + j, so
// an A fragment read covers two runs of 32 consecutive slots, and a block's reads differ by
// constant offsets) and every wave owns its tokens
// outright: 64 at a time (two 32-token blocks, their B fragments loaded from memory into
// registers), run against each 32-row block of centroids in turn (A fragments and the
// accumulator start -|c_j|^2/2 read from LDS, each A fragment serving both token
// blocks), the best and second best folded in on the way. No token meets another wave's
// results, so the main loop has no barrier; eight waves, two per SIMD, cover each other's
// load latency and vector-ALU work. Block r of centroids runs on the matrix core while the
// vector ALU selects over block r - 1 (two accumulator sets), and block r + 1's A fragments
// are read from LDS as block r's MFMAs free their registers.
//
// Selection: a value's position i (0..15) among the lane's 16 results of a block goes into
// its low 4 mantissa bits (moving it by less than 2^-19 |f|), the block's best and second
// best come from a tournament of triples against the running pair, and the block of the
// running best is kept beside it. The margin test and the exact binary64 decision of the
// tokens it cannot separate are the same as in k_assign (the packing error here is smaller).
constexpr int AL_WAVES = 8;
constexpr int AL_THREADS = 64 * AL_WAVES;
constexpr int AL_TPG = 64;  // tokens per wave group
constexpr int AL_MAXC = AS_GROUP;

struct AssignLdsL {
  float nh[AL_MAXC];                 // -|c_j|^2 / 2; padding rows -FLT_MAX
  u32x4 cent[16 * AL_MAXC];          // the unit's bf16 centroids, chunk c of row j at 512 c + j
                                     // (rows up to a multiple of 64 zero)
  uint32_t nearw[AS_MAXTPW / 32];    // near-tie flags of the range's tokens
  u32x4 rows[32 * 16];               // exact decision: the batch's rows (slot t*16 + (c ^ (t & 15)))
  float red[AL_WAVES][32];           // exact decision: per wave the best fp32 value of each token
  unsigned long long fd[32];         // exact decision: per token the least D_j (bits), then its id
  int32_t fj[32];
  int32_t flist[32];                 // exact decision: the batch's tokens
  int32_t wcnt[AS_MAXTPW / 32];      // near-tie flags before each flag word
  float rmx[AL_WAVES];               // per wave: max |c_j|^2
  int32_t total;
  int32_t gnext;                     // the next unclaimed token group
};

static_assert(sizeof(AssignLdsL) <= 160 * 1024, "k_assign_lds LDS");

// value with its position p (0..15) in the low 4 mantissa bits
__device__ __forceinline__ float pack4(float v, int p) {
  return __uint_as_float((__float_as_uint(v) & ~15u) | (unsigned)p);
}

// Best and second best of a block's 16 values of one token block folded into the running
// pair (b1 of block bk, b2), in four stages so that each can sit between two MFMAs: a
// triple's maximum goes up a level, its median is kept, and the second best overall is the
// largest median (with the running b2 as one more). 38 operations.
struct Top2 {
  float v[16], up[6], md[8];
  __device__ __forceinline__ void stage(int k, const floatx16& a, float& b1, float& b2, int& bk, int r) {
    if (k == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = pack4(a[i], i);
    } else if (k == 1) {
#pragma unroll
      for (int i = 8; i < 16; ++i) v[i] = pack4(a[i], i);
    } else if (k == 2) {
#pragma unroll
      for (int t = 0; t < 5; ++t) {
        up[t] = max3f(v[3 * t], v[3 * t + 1], v[3 * t + 2]);
        md[t] = __builtin_amdgcn_fmed3f(v[3 * t], v[3 * t + 1], v[3 * t + 2]);
      }
      up[5] = v[15];
    } else {
      const float z0 = max3f(up[0], up[1], up[2]), z1 = max3f(up[3], up[4], up[5]);
      md[5] = __builtin_amdgcn_fmed3f(up[0], up[1], up[2]);
      md[6] = __builtin_amdgcn_fmed3f(up[3], up[4], up[5]);
      const float nb1 = max3f(z0, z1, b1);
      md[7] = __builtin_amdgcn_fmed3f(z0, z1, b1);
      float s = max3f(md[0], md[1], md[2]);
      s = max3f(s, md[3], md[4]);
      s = max3f(s, md[5], md[6]);
      b2 = max3f(s, md[7], b2);
      bk = nb1 > b1 ? r : bk;
      b1 = nb1;
    }
  }
};

__global__ __attribute__((amdgpu_flat_work_group_size(AL_THREADS, AL_THREADS), amdgpu_waves_per_eu(2, 2))) void
k_assign_lds(BuildSeq sa, int tpw, const uint16_t* __restrict__ K, const uint16_t* __restrict__ chat,
             const float* __restrict__ norm, int32_t* __restrict__ assign) {
  extern __shared__ uint8_t smem[];
  AssignLdsL& S = *reinterpret_cast<AssignLdsL*>(smem);
  Unit U;
  int tb0;
  assign_wg_map(sa, tpw, xcd_linear(blockIdx.x, gridDim.x), U, tb0);
  const int nrow = min(tpw, U.L - tb0);  // rows of the workgroup's range
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, h = lane >> 5, col = lane & 31;
  const int Kc = U.Kc, nA2 = ((Kc + 63) >> 6) * 2;  // 32-row blocks, an even count
  const uint16_t* Kr = K + (U.irow0 + tb0) * D;    // first input row of the range
  // B fragments of the group at t: token block tb, lane (col, h) holds chunks 2 st + h of token
  // t + 32 tb + col, loaded k-step by k-step in the order the MFMAs take them; rows past the
  // range end repeat its last row (their results are not used). The first group's are loaded
  // before the centroids.
  auto load_b = [&](bf16x8_t (&Bv)[2][8], int t) {
    const uint16_t* x0 = Kr + (int64_t)min(t + col, nrow - 1) * D + h * 8;
    const uint16_t* x1 = Kr + (int64_t)min(t + 32 + col, nrow - 1) * D + h * 8;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      Bv[0][st] = *reinterpret_cast<const bf16x8_t*>(x0 + st * 16);
      Bv[1][st] = *reinterpret_cast<const bf16x8_t*>(x1 + st * 16);
    }
  };
  const int t_first = wv * AL_TPG;
  bf16x8_t B[2][8];
  load_b(B, t_first);

  // 1. the centroids into LDS (rows past Kc zero), -|c|^2/2 (padding rows: a finite floor
  // every real value beats), max |c|^2, the near-tie flags cleared
  {
    constexpr int CL = AL_MAXC * 16 / AL_THREADS;
    u32x4 cv[CL];
#pragma unroll
    for (int i = 0; i < CL; ++i) {
      const int s = tid + i * AL_THREADS, j = s >> 4, c = s & 15;
      cv[i] = *reinterpret_cast<const u32x4*>(chat + (U.gclu + min(j, Kc - 1)) * D + c * 8);
    }
#pragma unroll
    for (int i = 0; i < CL; ++i) {
      const int s = tid + i * AL_THREADS, j = s >> 4, c = s & 15;
      if (j < nA2 * 32) S.cent[c * AL_MAXC + j] = j < Kc ? cv[i] : u32x4{0u, 0u, 0u, 0u};
    }
    float m = 0.f;
    for (int j = tid; j < nA2 * 32; j += AL_THREADS) {
      const float v = j < Kc ? norm[U.gclu + j] : 0.f;
      S.nh[j] = j < Kc ? -0.5f * v : -__FLT_MAX__;
      m = fmaxf(m, v);
    }
    m = wave_max(m);
    if (lane == 0) S.rmx[wv] = m;
    for (int i = tid; i < AS_MAXTPW / 32; i += AL_THREADS) S.nearw[i] = 0u;
    if (tid == 0) S.gnext = AL_WAVES;  // groups 0..7 are the waves' first
  }
  __syncthreads();
  float R2 = S.rmx[0];
#pragma unroll
  for (int w2 = 1; w2 < AL_WAVES; ++w2) R2 = fmaxf(R2, S.rmx[w2]);
  const float R = __builtin_amdgcn_sqrtf(R2);

  // A fragments of block r, k-step st: lane (col, h) reads chunk 2 st + h of row 32 r + col
  const u32x4* cl = S.cent + h * AL_MAXC + col;
  auto read_a = [&](int r, int st) { return __builtin_bit_cast(bf16x8_t, cl[32 * r + 2 * st * AL_MAXC]); };
  // accumulator start of block r: rows 32 r + 8 a + 4 h + k at element 4 a + k
  auto read_n = [&](int r) {
    const float4* nb = reinterpret_cast<const float4*>(S.nh) + 8 * r + h;
    floatx16 n;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 t = nb[2 * a];
      n[4 * a + 0] = t.x;
      n[4 * a + 1] = t.y;
      n[4 * a + 2] = t.z;
      n[4 * a + 3] = t.w;
    }
    return n;
  };

  // 2. The wave's token groups, 64 tokens each: group wv first, then the next unclaimed one of
  // the workgroup's range, claimed when the current one starts (its B fragments are loaded as
  // soon as the current group's last MFMAs have read theirs). The two waves of a SIMD do not
  // progress alike (the arbiter favours the older one), so claimed groups keep both busy to the
  // end, where a fixed share left the younger wave running its last groups alone.
  bf16x8_t A[8];
  floatx16 nv;
  for (int t0 = t_first; t0 < nrow;) {
    int qn = 0;
    if (lane == 0) qn = atomicAdd(&S.gnext, 1);
    const int tn = __builtin_amdgcn_readfirstlane(qn) * AL_TPG;
    // |x|^2 of the group's tokens (lane (col, h): half h of token col, then both halves)
    float x2[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      float s2 = 0.f;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const u32x4 w = __builtin_bit_cast(u32x4, B[tb][st]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t we = w[e];  // bit-cast a named scalar (see xnorm in k_assign)
          const bf16x2_t x = __builtin_bit_cast(bf16x2_t, we);
          s2 = __builtin_amdgcn_fdot2_f32_bf16(x, x, s2, false);
        }
      }
      x2[tb] = s2 + swap32(s2);
    }
    nv = read_n(0);
#pragma unroll
    for (int st = 0; st < 8; ++st) A[st] = read_a(0, st);
    floatx16 accX[2], accY[2];
    float b1[2] = {-INFINITY, -INFINITY}, b2[2] = {-INFINITY, -INFINITY};
    int bk[2] = {0, 0};
    // One block step, in program order, k-step by k-step: the two MFMAs of block r (one per
    // token block: independent accumulators, so neither waits for the other), the LDS read of
    // block rn's A fragment that those MFMAs just freed (and after the first pair its start
    // values), and an eighth of the selection over the previous block (block rp, in pacc);
    // a scheduling fence after each k-step keeps that order.
    Top2 T;
    auto step = [&](floatx16 (&acc)[2], int rn, floatx16 (&pacc)[2], int rp, bool sel_prev, bool mfma) {
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        if (mfma) {
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
            acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[st], B[tb][st], st == 0 ? nv : acc[tb], 0, 0, 0);
          if (st == 0) nv = read_n(rn);
          A[st] = read_a(rn, st);
        }
        if (sel_prev) {
          // the selection at a raised wave priority, so that the arbiter takes it before the
          // other wave of the SIMD (≈ 2% faster than leaving the older wave first throughout)
          __builtin_amdgcn_s_setprio(1);
          T.stage(st & 3, pacc[st >> 2], b1[st >> 2], b2[st >> 2], bk[st >> 2], rp);
          __builtin_amdgcn_s_setprio(0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    step(accX, 1, accY, 0, false, true);  // block 0
    int r = 0;
    for (; r + 2 < nA2; r += 2) {
      step(accY, r + 2, accX, r, true, true);      // block r + 1; selection of block r
      step(accX, r + 3, accY, r + 1, true, true);  // block r + 2; selection of block r + 1
    }
    step(accY, r + 1, accX, r, true, true);  // block r + 1 (the reads of it again: harmless)
    load_b(B, tn);  // the next group's fragments (past the range end: its last row)
    step(accY, 0, accY, r + 1, true, false);
    // merge the two half-waves, the margin test, the ids
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const float ob1 = swap32(b1[tb]), ob2 = swap32(b2[tb]);
      const int obk = swap32(bk[tb]);
      const bool take = ob1 > b1[tb];
      const float nb2 = fmaxf(fminf(b1[tb], ob1), fmaxf(b2[tb], ob2));
      const float nb1 = fmaxf(b1[tb], ob1);
      const int p = (int)(__float_as_uint(nb1) & 15u), hw = take ? h ^ 1 : h, blk = take ? obk : bk[tb];
      const int best_id = 32 * blk + 8 * (p >> 2) + 4 * hw + (p & 3);
      const float margin = 0x1p-14f * (__builtin_amdgcn_sqrtf(x2[tb]) * R + R2) + 0x1p-100f;
      const bool near = !(nb1 - nb2 > margin) || !(nb1 > -0x1p127f) || !(margin < 0x1p100f);
      const int t = t0 + 32 * tb + col;
      if (h == 0 && t < nrow) {
        assign[U.row0 + tb0 + t] = U.cbase + best_id;
        if (near) atomicOr(&S.nearw[t >> 5], 1u << (t & 31));
      }
    }
    t0 = tn;
  }

  // 3. near-tie tokens: flag words counted, a workgroup scan
  __syncthreads();
  const int nwd = (nrow + 31) >> 5;
  for (int i = tid; i < nwd; i += AL_THREADS) S.wcnt[i] = __builtin_popcount(S.nearw[i]);  // its prefix below
  __syncthreads();
  if (wv == 0) {
    int run = 0;
    for (int i0 = 0; i0 < nwd; i0 += 64) {
      const int i = i0 + lane;
      const int c = i < nwd ? S.wcnt[i] : 0;
      int incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      if (i < nwd) S.wcnt[i] = run + incl - c;
      run += __shfl(incl, 63, 64);
    }
    if (lane == 0) S.total = run;
  }
  __syncthreads();
  const int total = S.total;
  if (total == 0) return;
  // Exact decision, 32 tokens at a time: their rows go through the MFMAs again (wave wv takes
  // blocks 2 wv and 2 wv + 1); every centroid within 2^-14 (|x| R + R^2) + 2^-40 (|x| + R)^2
  // + 2^-100 of the best fp32 value gets D_j = sum_i (x_i - c_j,i)^2 in binary64, dims in
  // order, each operation rounded; argmin with the lowest id on ties (as in k_assign).
  for (int f0 = 0; f0 < total; f0 += 32) {
    const int nb = min(32, total - f0);
    for (int i = tid; i < nwd; i += AL_THREADS) {
      uint32_t f = S.nearw[i];
      int k = S.wcnt[i];
      while (f != 0u) {
        const int b = __builtin_ctz(f);
        f &= f - 1u;
        if (k >= f0 && k < f0 + 32) S.flist[k - f0] = 32 * i + b;
        ++k;
      }
    }
    if (tid < 32) {
      S.fd[tid] = ~0ull;
      S.fj[tid] = 0x7FFFFFFF;
    }
    __syncthreads();
    {
      const int slot = tid, t = slot >> 4, c = (slot & 15) ^ (t & 15);
      S.rows[slot] = *reinterpret_cast<const u32x4*>(Kr + (int64_t)S.flist[min(t, nb - 1)] * D + c * 8);
    }
    __syncthreads();
    bf16x8_t Bx[8];
#pragma unroll
    for (int st = 0; st < 8; ++st)
      Bx[st] = __builtin_bit_cast(bf16x8_t, S.rows[col * 16 + ((2 * st + h) ^ (col & 15))]);
    float s2 = 0.f;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const u32x4 w = __builtin_bit_cast(u32x4, Bx[st]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t we = w[e];
        const float a = bf16_lo(we), b = bf16_hi(we);
        s2 = fmaf(a, a, s2);
        s2 = fmaf(b, b, s2);
      }
    }
    s2 += swap32(s2);
    const float X = sqrtf(s2);
    const float win = 0x1p-14f * (X * R + R2) + 0x1p-40f * (X + R) * (X + R) + 0x1p-100f;
    floatx16 av[2];
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = min(2 * wv + q, nA2 - 1);
      av[q] = read_n(r);
#pragma unroll
      for (int st = 0; st < 8; ++st) av[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_a(r, st), Bx[st], av[q], 0, 0, 0);
      if (2 * wv + q < nA2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, av[q][i]);
      }
    }
    mx = fmaxf(mx, swap32(mx));
    if (h == 0) S.red[wv][col] = mx;
    __syncthreads();
    float M = S.red[0][col];
#pragma unroll
    for (int w2 = 1; w2 < AL_WAVES; ++w2) M = fmaxf(M, S.red[w2][col]);
    const float thr = M - win;
    const u32x4* xr = S.rows + col * 16;
    double best = INFINITY;
    int bj = 0x7FFFFFFF;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (2 * wv + q >= nA2) continue;
      uint32_t cm = 0u;
#pragma unroll
      for (int i = 0; i < 16; ++i) cm |= (uint32_t)!(av[q][i] < thr) << i;  // NaN: a candidate
      while (cm != 0u) {
        const int i = __builtin_ctz(cm);
        cm &= cm - 1u;
        const int j = 32 * (2 * wv + q) + 8 * (i >> 2) + 4 * h + (i & 3);
        if (j >= Kc) continue;
        const u32x4* cj = S.cent + j;
        double acc = 0.0;
        for (int c = 0; c < 16; ++c) {
          const u32x4 xv = xr[c ^ (col & 15)], cw = cj[c * AL_MAXC];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t xe = xv[e], ce = cw[e];
            const double d0 = __dsub_rn((double)bf16_lo(xe), (double)bf16_lo(ce));
            acc = __dadd_rn(acc, __dmul_rn(d0, d0));
            const double d1 = __dsub_rn((double)bf16_hi(xe), (double)bf16_hi(ce));
            acc = __dadd_rn(acc, __dmul_rn(d1, d1));
          }
        }
        if (acc < best || (acc == best && j < bj)) {
          best = acc;
          bj = j;
        }
      }
    }
    const unsigned long long bd = (unsigned long long)__double_as_longlong(best);
    if (bj != 0x7FFFFFFF) atomicMin(&S.fd[col], bd);
    __syncthreads();
    if (bj != 0x7FFFFFFF && bd == S.fd[col]) atomicMin(&S.fj[col], bj);
    __syncthreads();
    if (tid < nb) assign[U.row0 + tb0 + S.flist[tid]] = U.cbase + S.fj[tid];
    __syncthreads();
  }
}

// ------------------------------------------------------------------ k_sort
// Stable counting sort of one unit by cluster: sorted slot of token t is
// offset(c) + #{t' < t in the unit : a(t') = c}. The 16 waves take consecutive
// token ranges; inside a wave, 64 tokens at a time, equal ids are ranked by a
// ballot loop (one iteration per distinct id); per-wave counts then become
// per-wave bases. Writes sizes, offsets (block level) and perm.
constexpr int SORT_THREADS = 1024;

__global__ __launch_bounds__(SORT_THREADS) void k_sort(BuildSeq sa, const int32_t* __restrict__ assign,
                                                       int32_t* __restrict__ rank, int32_t* __restrict__ sizes,
                                                       int32_t* __restrict__ offsets, int32_t* __restrict__ perm, BigList bl) {
  extern __shared__ uint8_t smem[];
  const Unit U = unit_of(sa, blockIdx.x);
  const int Kc = U.Kc;
  int32_t* hist = reinterpret_cast<int32_t*>(smem);  // [16][Kc]
  __shared__ uint64_t scan[17];
  __shared__ BigStage bs;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < 16 * Kc; e += SORT_THREADS) hist[e] = 0;
  if (tid == 0) bs.n = 0;
  __syncthreads();
  const int span = (U.L + 15) / 16;
  const int w0 = min(wv * span, U.L), w1 = min(w0 + span, U.L);
  const uint64_t ltmask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int t0 = w0; t0 < w1; t0 += 64) {
    const int t = t0 + lane;
    const bool valid = t < w1;
    // ids are in [0, Kc) by construction; the clamp keeps every sorted slot inside
    // the segment even if they were not
    const int c = valid ? min(max(assign[U.row0 + t] - U.cbase, 0), Kc - 1) : -1;
    uint64_t active = __ballot(valid);
    int myrank = 0, myleader = 0, old = 0;
    while (active) {
      const int leader = __ffsll((unsigned long long)active) - 1;
      const int v = __shfl(c, leader, 64);
      const uint64_t same = __ballot(c == v);
      if (c == v) {
        myrank = __popcll(same & ltmask);
        myleader = leader;
      }
      if (lane == leader) old = atomicAdd(&hist[wv * Kc + v], __popcll(same));
      active &= ~same;
    }
    const int base = __shfl(old, myleader, 64);
    if (valid) rank[U.irow0 + t] = base + myrank;
  }
  __syncthreads();
  // per-cluster totals, per-wave bases, exclusive offsets over clusters
  const int per = (Kc + SORT_THREADS - 1) / SORT_THREADS;
  const int c0 = min(tid * per, Kc), c1 = min(c0 + per, Kc);
  int64_t mysum = 0;
  for (int c = c0; c < c1; ++c) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int x = hist[w * Kc + c];
      hist[w * Kc + c] = run;
      run += x;
    }
    sizes[U.gclu + c] = run;
    big_note(sa, bl, bs, U.gclu + c, run);
    mysum += run;
  }
  // exclusive scan of mysum over threads
  {
    uint64_t x = (uint64_t)mysum;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const uint64_t y = __shfl_up(x, s, 64);
      if (lane >= s) x += y;
    }
    if (lane == 63) scan[wv] = x;
    __syncthreads();
    if (wv == 0) {
      const uint64_t v0 = lane < 16 ? scan[lane] : 0;
      uint64_t tt = v0;
#pragma unroll
      for (int s = 1; s < 16; s <<= 1) {
        const uint64_t y = __shfl_up(tt, s, 64);
        if (lane >= s) tt += y;
      }
      if (lane < 16) scan[lane] = tt - v0;
    }
    __syncthreads();
    if (wv == 1) big_flush(bl, bs);
    int64_t run = (int64_t)(scan[wv] + x - (uint64_t)mysum);
    for (int c = c0; c < c1; ++c) {
      const int sz = sizes[U.gclu + c];
      offsets[U.boff + U.cbase + c] = U.tok0 + (int32_t)run;
      for (int w = 0; w < 16; ++w) hist[w * Kc + c] += (int32_t)run;
      run += sz;
    }
  }
  if (tid == 0 && U.tok0 + U.L == U.N) offsets[U.boff + U.C] = U.N;
  __syncthreads();
  for (int t = tid; t < U.L; t += SORT_THREADS) {
    const int c = min(max(assign[U.row0 + t] - U.cbase, 0), Kc - 1);
    const int w = t / span;
    const int p = U.tok0 + hist[w * Kc + c] + rank[U.irow0 + t];
    perm[U.brow + p] = U.tok0 + t;
  }
}

// ------------------------------------------------------------------ k_sort_radix
// The same stable sort for units of at most RS_MAXL tokens, as an LSD radix sort
// of the keys (cluster << 14 | position) held in LDS, RS_DB cluster bits per pass.
// Element i of a pass is handled by thread i mod 1024 in tile i / 1024, so the
// order (tile, wave, lane) is element order. Inside a wave the elements with
// the same digit are matched with one ballot per digit bit; the per-(digit,
// tile, wave) counts are scanned over the workgroup in digit-major order, which
// makes every pass stable. After the passes the sorted keys give perm directly,
// and each cluster's first slot is found by binary search.
//
// With parts = 2 (the units alone would leave half the CUs idle) a unit's tokens are
// split between two workgroups at position Lp = ceil(L / 2): each counts the clusters of
// both halves, so that member j of cluster c in half 1 goes to slot off[c] + (members of c
// in half 0) + j, sorts its own half and writes those slots; half 0 writes sizes and
// offsets.
constexpr int RS_THREADS = 1024;
constexpr int RS_MAXL = 16384;  // positions fit 14 bits
constexpr int RS_DB = 5;
constexpr int RS_ND = 1 << RS_DB;

__device__ inline uint32_t rs_digit(uint32_t key, int pass) { return (key >> (14 + RS_DB * pass)) & (RS_ND - 1); }

// LDS slot of counter x: the counters of one (tile, wave) for the 32 digits lie 16 E words
// apart, i.e. in one bank; xor-ing bits 6.. into the bank bits spreads them over 32 banks
// (a bijection inside every 64-word block)
__device__ __forceinline__ int rs_cx(int x) { return x ^ ((x >> 6) & 63); }

// exclusive scan of one u64 per thread over a workgroup of RS_THREADS; *total gets the sum
__device__ inline uint64_t block_scan_u64(uint64_t v, uint64_t* tmp, uint64_t* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint64_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wv] = x;
  __syncthreads();
  if (wv == 0) {
    const uint64_t t = lane < RS_THREADS / 64 ? tmp[lane] : 0ull;
    uint64_t tt = t;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const uint64_t y = __shfl_up(tt, o, 64);
      if (lane >= o) tt += y;
    }
    if (lane < RS_THREADS / 64) tmp[lane] = tt - t;
    if (lane == RS_THREADS / 64 - 1) tmp[16] = tt;
  }
  __syncthreads();
  const uint64_t r = tmp[wv] + x - v;
  *total = tmp[16];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(RS_THREADS) void k_sort_radix(BuildSeq sa, int parts, const int32_t* __restrict__ assign,
                                                           int32_t* __restrict__ sizes,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm, BigList bl) {
  extern __shared__ uint8_t smem[];
  const Unit U = unit_of(sa, blockIdx.x / parts);
  const int part = (int)(blockIdx.x % parts);
  const int Kc = U.Kc, Lp = (U.L + parts - 1) / parts, p0 = part * Lp;
  const int L = min(Lp, U.L - p0);                   // this workgroup's positions [p0, p0 + L)
  const int E = (Lp + RS_THREADS - 1) / RS_THREADS;  // tiles
  uint32_t* buf0 = reinterpret_cast<uint32_t*>(smem);
  uint32_t* buf1 = buf0 + E * RS_THREADS;
  __shared__ uint64_t scan[17];
  __shared__ int32_t first[WAVE_MAX_CLUSTERS_PER_SEG + 1];  // first sorted slot of cluster c (c <= Kc)
  __shared__ int32_t hist1[WAVE_MAX_CLUSTERS_PER_SEG];      // parts = 2: members of c in half 1
  __shared__ BigStage bs;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) bs.n = 0;
  const uint64_t ltmask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int nbits = 0;
  while ((1 << nbits) < Kc) ++nbits;
  const int passes = (nbits + RS_DB - 1) / RS_DB;
  if (parts > 1) {
    // members per cluster in each half (first[] holds half 0's counts for now)
    for (int c = tid; c < Kc; c += RS_THREADS) {
      first[c] = 0;
      hist1[c] = 0;
    }
    __syncthreads();
    for (int i = tid; i < U.L; i += RS_THREADS) {
      const int c = min(max(assign[U.row0 + i] - U.cbase, 0), Kc - 1);
      atomicAdd(i < Lp ? &first[c] : &hist1[c], 1);
    }
    __syncthreads();
  }
  // keys in element (= position) order; ids are in [0, Kc) by construction, the clamp keeps
  // every sorted slot inside the segment even if they were not
  for (int e = 0; e < E; ++e) {
    const int i = e * RS_THREADS + tid;
    const int ic = min(i, L - 1);
    const int c = min(max(assign[U.row0 + p0 + ic] - U.cbase, 0), Kc - 1);
    buf0[i] = ((uint32_t)c << 14) | (uint32_t)ic;
  }
  __syncthreads();
  uint32_t* src = buf0;
  uint32_t* dst = buf1;
  const int nx = RS_ND * E * 16;           // (digit, tile, wave) counters, kept in dst
  const int per = (nx + RS_THREADS - 1) / RS_THREADS;
  for (int pass = 0; pass < passes; ++pass) {
    int32_t* cnt = reinterpret_cast<int32_t*>(dst);
    for (int x = tid; x < nx; x += RS_THREADS) cnt[x] = 0;
    __syncthreads();
    uint32_t dg[RS_MAXL / RS_THREADS];
    int rk[RS_MAXL / RS_THREADS];
#pragma unroll
    for (int e = 0; e < RS_MAXL / RS_THREADS; ++e) {
      if (e < E) {
        const int i = e * RS_THREADS + tid;
        const bool valid = i < L;
        const uint32_t d = rs_digit(src[i], pass);
        uint64_t m = __ballot(valid);
#pragma unroll
        for (int bt = 0; bt < RS_DB; ++bt) {
          const uint64_t bb = __ballot((d >> bt) & 1u);
          m &= ((d >> bt) & 1u) ? bb : ~bb;
        }
        dg[e] = d;
        rk[e] = __popcll(m & ltmask);
        if (valid && rk[e] == 0) cnt[rs_cx(((int)d * E + e) * 16 + wv)] = __popcll(m);
      }
    }
    __syncthreads();
    // exclusive scan of the counters in (digit, tile, wave) order
    {
      const int x0 = min(tid * per, nx), x1 = min(x0 + per, nx);
      uint64_t local = 0;
      for (int x = x0; x < x1; ++x) local += (uint32_t)cnt[rs_cx(x)];
      uint64_t y = local;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint64_t t = __shfl_up(y, o, 64);
        if (lane >= o) y += t;
      }
      if (lane == 63) scan[wv] = y;
      __syncthreads();
      if (wv == 0) {
        const uint64_t v0 = lane < 16 ? scan[lane] : 0;
        uint64_t tt = v0;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const uint64_t t = __shfl_up(tt, o, 64);
          if (lane >= o) tt += t;
        }
        if (lane < 16) scan[lane] = tt - v0;
      }
      __syncthreads();
      int run = (int)(scan[wv] + y - local);
      for (int x = x0; x < x1; ++x) {
        const int c = cnt[rs_cx(x)];
        cnt[rs_cx(x)] = run;
        run += c;
      }
    }
    __syncthreads();
    int pos[RS_MAXL / RS_THREADS];
    uint32_t kv[RS_MAXL / RS_THREADS];
#pragma unroll
    for (int e = 0; e < RS_MAXL / RS_THREADS; ++e) {
      if (e < E) {
        const int i = e * RS_THREADS + tid;
        kv[e] = src[i];
        pos[e] = cnt[rs_cx(((int)dg[e] * E + e) * 16 + wv)] + rk[e];
      }
    }
    __syncthreads();  // the counters are read; dst takes the keys
#pragma unroll
    for (int e = 0; e < RS_MAXL / RS_THREADS; ++e)
      if (e < E && e * RS_THREADS + tid < L) dst[pos[e]] = kv[e];
    __syncthreads();
    uint32_t* t = src;
    src = dst;
    dst = t;
  }
  if (parts > 1) {
    // slot of sorted element s of cluster c: off[c] + (half 1: members of c in half 0) +
    // (s - first element of c in this half). One scan of (total, this half's count) pairs
    // over the clusters, 2 per thread.
    const int c0 = 2 * tid;
    uint64_t v[2] = {0ull, 0ull};
#pragma unroll
    for (int r = 0; r < 2; ++r)
      if (c0 + r < Kc) {
        const uint64_t h0 = (uint32_t)first[c0 + r], h1 = (uint32_t)hist1[c0 + r];
        v[r] = ((h0 + h1) << 32) | (part == 0 ? h0 : h1);
      }
    uint64_t tot;
    const uint64_t ex = block_scan_u64(v[0] + v[1], scan, &tot);
    int32_t delta[2];
    uint64_t run = ex;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int off = (int)(run >> 32), fmy = (int)(run & 0xFFFFFFFFu);
      delta[r] = off + (part == 1 && c0 + r < Kc ? first[c0 + r] : 0) - fmy;
      if (part == 0 && c0 + r < Kc) {
        offsets[U.boff + U.cbase + c0 + r] = U.tok0 + off;
        sizes[U.gclu + c0 + r] = (int32_t)(v[r] >> 32);
        big_note(sa, bl, bs, U.gclu + c0 + r, (int32_t)(v[r] >> 32));
      }
      run += v[r];
    }
    __syncthreads();  // first[] and hist1[] are read
    if (part == 0 && wv == 0) big_flush(bl, bs);
#pragma unroll
    for (int r = 0; r < 2; ++r)
      if (c0 + r < Kc) first[c0 + r] = delta[r];
    __syncthreads();
    for (int i = tid; i < L; i += RS_THREADS) {
      const uint32_t key = src[i];
      perm[U.brow + U.tok0 + first[key >> 14] + i] = U.tok0 + p0 + (int32_t)(key & 0x3FFFu);
    }
    if (part == 0 && tid == 0 && U.tok0 + U.L == U.N) offsets[U.boff + U.C] = U.N;
    return;
  }
  // perm, and each cluster's first slot by binary search over the sorted keys
  for (int i = tid; i < L; i += RS_THREADS) perm[U.brow + U.tok0 + i] = U.tok0 + (int32_t)(src[i] & 0x3FFFu);
  for (int c = tid; c <= Kc; c += RS_THREADS) {
    int lo = 0, hi = L;  // first index whose cluster is >= c
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int)(src[mid] >> 14) < c) lo = mid + 1;
      else hi = mid;
    }
    if (c < Kc) offsets[U.boff + U.cbase + c] = U.tok0 + lo;
    first[c] = lo;
  }
  __syncthreads();
  for (int c = tid; c < Kc; c += RS_THREADS) {
    sizes[U.gclu + c] = first[c + 1] - first[c];
    big_note(sa, bl, bs, U.gclu + c, first[c + 1] - first[c]);
  }
  if (tid == 0 && U.tok0 + U.L == U.N) offsets[U.boff + U.C] = U.N;
  __syncthreads();
  if (wv == 0) big_flush(bl, bs);
}

// ------------------------------------------------------------------ k_update
// Ordered fp32 sums of the members' keys (ascending position), correctly
// rounded division by the count; empty clusters keep their centroid. One wave
// per cluster, 2 dims per lane, members fetched 16 at a time (their positions
// with one load, then 16 row loads in flight). Writes the bf16 centroid and its
// squared norm. The last round (FINAL) also copies every member's K and V row
// to its sorted slot, writes inv_perm and the ordered fp32 value sums (and/or
// their round-to-nearest-even bf16 copy).
template <bool FINAL>
__global__ __launch_bounds__(256) void k_update(BuildSeq sa, int64_t nclu, const uint16_t* __restrict__ K,
                                                const uint16_t* __restrict__ V, wave_index ix,
                                                float* __restrict__ norm, BigList bl) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (blockIdx.x == 0 && threadIdx.x == 0) bl.cnt[bl.parity ^ 1] = 0;  // the next round's list
  // a whole dense build: waves [0, BIG_CAP) take the sort's list of large clusters, the
  // rest every cluster in order except those
  int64_t Fc;
  if (sa.ident) {
    if (w < BIG_CAP) {
      if (w >= min(bl.cnt[bl.parity], BIG_CAP)) return;
      Fc = bl.ids[bl.parity * BIG_CAP + w];
    } else {
      Fc = w - BIG_CAP;
      if (Fc >= nclu || bl.flag[Fc]) return;
    }
  } else {
    Fc = w;
    if (Fc >= nclu) return;
  }
  // a whole dense build: the size load goes out before the block lookup, which then
  // overlaps its latency
  int n = sa.ident ? ix.sizes[Fc] : 0;
  const CluRef cr = clu_of(sa, Fc);
  const int64_t F = cr.gF;
  if (!sa.ident) n = ix.sizes[F];
  if (n == 0) {
    if (FINAL && ix.vsum) *reinterpret_cast<float2*>(ix.vsum + F * D + 2 * lane) = make_float2(0.f, 0.f);
    if (FINAL && ix.vsum_bf16)
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(ix.vsum_bf16) + F * D + 2 * lane) = 0u;
    return;
  }
  const int off = ix.offsets[cr.boff + cr.j];
  // input rows of the block's positions (index arithmetic: the base row alone may lie
  // before the first input row)
  const int64_t eb = cr.ib * D + 2 * lane;
  uint16_t* Ks = reinterpret_cast<uint16_t*>(ix.k_sorted) + cr.brow * D + 2 * lane;
  uint16_t* Vs = reinterpret_cast<uint16_t*>(ix.v_sorted) + cr.brow * D + 2 * lane;
  const int32_t* pb = ix.perm + cr.brow + off;
  float s0 = 0.f, s1 = 0.f, w0 = 0.f, w1 = 0.f;
  // A wave's time is the chain of its chunks' loads, so the launch ends with the largest
  // cluster's wave (615 members at 128K: 39 chunks). Before the last round each chunk's
  // member positions are loaded one chunk ahead, so a chunk waits for its rows only, not
  // for positions then rows (the last round, with V rows too, would lose occupancy).
  int ptv_next = !FINAL && lane < min(n, 16) ? pb[lane] : 0;
  for (int k0 = 0; k0 < n; k0 += 16) {
    const int m = min(16, n - k0);
    int ptv;
    if constexpr (FINAL) {
      ptv = lane < m ? pb[k0 + lane] : 0;
    } else {
      ptv = ptv_next;
      ptv_next = k0 + 16 + lane < n && lane < 16 ? pb[k0 + 16 + lane] : 0;
    }
    // unconditional loads (clamped to the last member) keep all 16 in flight
    uint32_t kr[16], vr[16];
    int tt[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      tt[u] = __shfl(ptv, min(u, m - 1), 64);
      kr[u] = *reinterpret_cast<const uint32_t*>(K + (eb + (int64_t)tt[u] * D));
      if (FINAL) vr[u] = *reinterpret_cast<const uint32_t*>(V + (eb + (int64_t)tt[u] * D));
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const bool in = u < m;
      s0 = in ? __fadd_rn(s0, bf16_lo(kr[u])) : s0;
      s1 = in ? __fadd_rn(s1, bf16_hi(kr[u])) : s1;
      if (FINAL) {
        w0 = in ? __fadd_rn(w0, bf16_lo(vr[u])) : w0;
        w1 = in ? __fadd_rn(w1, bf16_hi(vr[u])) : w1;
      }
    }
    if (FINAL) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (u < m) {
          const int p = off + k0 + u;
          *reinterpret_cast<uint32_t*>(Ks + (int64_t)p * D) = kr[u];
          *reinterpret_cast<uint32_t*>(Vs + (int64_t)p * D) = vr[u];
          if (lane == 0) ix.inv_perm[cr.brow + tt[u]] = p;
        }
      }
    }
  }
  const float fn = (float)n;
  const float c0 = __fdiv_rn(s0, fn), c1 = __fdiv_rn(s1, fn);
  *reinterpret_cast<float2*>(ix.centroids + F * D + 2 * lane) = make_float2(c0, c1);
  const uint16_t h0 = f_to_bf16(c0), h1 = f_to_bf16(c1);
  *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(ix.centroids_bf16) + F * D + 2 * lane) =
      (uint32_t)h0 | ((uint32_t)h1 << 16);
  const float a = bf16_to_f(h0), b = bf16_to_f(h1);
  const float q2 = wave_sum(fmaf(a, a, b * b));
  if (lane == 0) norm[F] = q2;
  if (FINAL && ix.vsum) *reinterpret_cast<float2*>(ix.vsum + F * D + 2 * lane) = make_float2(w0, w1);
  if (FINAL && ix.vsum_bf16)
    *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(ix.vsum_bf16) + F * D + 2 * lane) =
        (uint32_t)f_to_bf16(w0) | ((uint32_t)f_to_bf16(w1) << 16);
}

// ------------------------------------------------------------------ k_block_assign
// Block clustering of the block top-k baseline (Vortex technical summary, section A:
// per-block summaries built once, blocks scored and the top-k attended per query):
// token i of a unit of L tokens and Kc clusters goes to block floor(i Kc / L), the
// contiguous balanced blocks in the clusters' id space. One workgroup per unit.
__global__ __launch_bounds__(1024) void k_block_assign(BuildSeq sa, int32_t* __restrict__ assign, BigList bl) {
  if (blockIdx.x == 0 && threadIdx.x < 2) bl.cnt[threadIdx.x] = 0;  // the layout pass's list
  const Unit U = unit_of(sa, blockIdx.x);
  for (int i = threadIdx.x; i < U.L; i += blockDim.x)
    assign[U.row0 + i] = U.cbase + (int32_t)((int64_t)i * U.Kc / U.L);
}

// ------------------------------------------------------------------ k_stage
// Input rows of an append (RetroInfer page, section 2.A: segments are clustered
// independently, so a longer context changes only its last segments). For every
// sequence with new tokens, the tokens of each block from the start of the segment
// that held the old end (first[b] * seg_len) to the new end, in the call's input
// layout. Tokens already in the index come from its sorted copy (slot inv_perm[t]);
// the new ones from the caller's rows, ragged over the appended counts
// A_b = N_b - n_old[b]: row of (b, g, i) is G * sum_{b'<b} A_b' + g * A_b + i.
// Grid (B * G, ceil(max_b M_b / 64)); 16 lanes per row, 64 rows per workgroup.
struct StageArgs {
  int32_t B, G, seg_len, cap;
  int32_t n_new[MAXB];
  int32_t n_old[MAXB];
};

constexpr int STAGE_ROWS = 64;

__global__ __launch_bounds__(1024) void k_stage(StageArgs a, const uint16_t* __restrict__ Kn,
                                                const uint16_t* __restrict__ Vn, wave_index ix,
                                                uint16_t* __restrict__ Ko, uint16_t* __restrict__ Vo) {
  const int b = (int)blockIdx.x / a.G, g = (int)blockIdx.x % a.G;
  const int64_t A = (int64_t)a.n_new[b] - a.n_old[b];
  if (A <= 0) return;
  const int64_t t0 = (int64_t)(a.n_old[b] / a.seg_len) * a.seg_len;  // first re-clustered token
  const int64_t M = a.n_new[b] - t0;
  const int r = (int)blockIdx.y * STAGE_ROWS + (int)(threadIdx.x >> 4);
  if (r >= M) return;
  int64_t irow = 0, arow = 0;
  for (int i = 0; i < b; ++i) {
    const int64_t Ai = (int64_t)a.n_new[i] - a.n_old[i];
    if (Ai > 0) {
      irow += (int64_t)a.G * (a.n_new[i] - (int64_t)(a.n_old[i] / a.seg_len) * a.seg_len);
      arow += (int64_t)a.G * Ai;
    }
  }
  const int l16 = threadIdx.x & 15;
  const int64_t t = t0 + r;
  const int64_t brow = ((int64_t)b * a.G + g) * a.cap * a.seg_len;
  const bool old = t < a.n_old[b];
  const int64_t src = old ? brow + ix.inv_perm[brow + t] : arow + (int64_t)g * A + (t - a.n_old[b]);
  const uint16_t* SK = old ? reinterpret_cast<const uint16_t*>(ix.k_sorted) : Kn;
  const uint16_t* SV = old ? reinterpret_cast<const uint16_t*>(ix.v_sorted) : Vn;
  const int64_t dst = irow + (int64_t)g * M + r;
  *reinterpret_cast<u32x4*>(Ko + dst * D + l16 * 8) = *reinterpret_cast<const u32x4*>(SK + src * D + l16 * 8);
  *reinterpret_cast<u32x4*>(Vo + dst * D + l16 * 8) = *reinterpret_cast<const u32x4*>(SV + src * D + l16 * 8);
}

// ------------------------------------------------------------------ host side
hipError_t build_set_attrs() {
  WAVE_TRY(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_init), hipFuncAttributeMaxDynamicSharedMemorySize,
                               160 * 1024));
  WAVE_TRY(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_assign<true>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, sizeof(AssignLds)));
  WAVE_TRY(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_assign_lds),
                               hipFuncAttributeMaxDynamicSharedMemorySize, sizeof(AssignLdsL)));
  WAVE_TRY(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_sort), hipFuncAttributeMaxDynamicSharedMemorySize,
                               16 * WAVE_MAX_CLUSTERS_PER_SEG * 4));
  WAVE_TRY(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_sort_radix),
                               hipFuncAttributeMaxDynamicSharedMemorySize, 2 * RS_MAXL * 4));
  return hipSuccess;
}

// Workgroups per unit of the LDS radix sort: 2 when the units alone would leave more than
// half of the compute units idle (one 1024-thread workgroup per CU), else 1.
static int sort_parts(int64_t units, int cus) { return 2 * units <= cus ? 2 : 1; }
// Tokens per k_assign workgroup: enough workgroups per segment that the units fill
// the 256 compute units once (one workgroup per CU: its LDS and registers take the CU),
// in whole tiles.
static int assign_tpw(const SeqArgs& sa, int64_t units) {
  const int64_t per = std::max<int64_t>(1, (256 + units - 1) / units);
  int64_t t = (sa.seg_len + per - 1) / per;
  t = (t + AS_TT - 1) / AS_TT * AS_TT;
  return (int)std::min<int64_t>(sa.K_s > AS_GROUP ? AS_MAXTPW_M : AS_MAXTPW, std::max<int64_t>(AS_TT, t));
}

static int64_t host_nseg(const BuildSeq& bs, int b) { return (bs.N[b] + bs.seg_len - 1) / bs.seg_len; }

static int64_t assign_grid(const BuildSeq& bs, int tpw) {
  int64_t n = 0;
  for (int b = 0; b < bs.B; ++b) {
    const int64_t N = bs.N[b], nseg = host_nseg(bs, b), nu = nseg - bs.first[b];
    if (nu <= 0) continue;
    const int64_t last = N - (nseg - 1) * bs.seg_len;
    const int64_t wf = (bs.seg_len + tpw - 1) / tpw, wl = (last + tpw - 1) / tpw;
    n += (int64_t)bs.G * ((nu - 1) * wf + wl);
  }
  return n;
}

// units and clusters of a call
static void call_counts(const BuildSeq& bs, int64_t* units, int64_t* nclu) {
  *units = *nclu = 0;
  for (int b = 0; b < bs.B; ++b) {
    const int64_t nu = host_nseg(bs, b) - bs.first[b];
    if (nu <= 0) continue;
    *units += (int64_t)bs.G * nu;
    *nclu += (int64_t)bs.G * (bs.C[b] - (int64_t)bs.first[b] * bs.K_s);
  }
}

static BuildSeq whole(const SeqArgs& sa) {
  BuildSeq bs;
  static_cast<SeqArgs&>(bs) = sa;
  bs.ident = sa.cap == 0 ? 1 : 0;
  for (int b = 0; b < MAXB; ++b) bs.first[b] = 0;
  return bs;
}

// seeded init and `iters` Lloyd rounds of the call's units (input rows K, V), then the layout
static hipError_t run_build(const BuildSeq& bs, const uint16_t* K, const uint16_t* V, int32_t iters, uint64_t seed,
                            const wave_index& ix, const BuildWs& ws, int32_t* trace, int64_t rows, hipStream_t st) {
  const DeviceInfo& di = device_info();
  WAVE_TRY(di.status);
  int64_t units, nclu;
  call_counts(bs, &units, &nclu);
  if (units == 0) return hipSuccess;
  // k_init: count, draws and pairs (12 B per cluster), two position bitmaps, 16-bit rows
  const size_t init_lds = 16 + 4 * (((size_t)bs.K_s + 3) & ~(size_t)3) + 10 * (size_t)bs.K_s +
                          8 * (((size_t)bs.seg_len + 31) / 32);
  const size_t sort_lds = 16 * (size_t)bs.K_s * 4;
  // two key buffers of E tiles; the counters (32 digits x E tiles x 16 waves) fit in one
  const int sparts = sort_parts(units, di.cus);
  const size_t radix_tiles = ((size_t)(bs.seg_len + sparts - 1) / sparts + RS_THREADS - 1) / RS_THREADS;
  const size_t radix_lds = 2 * radix_tiles * RS_THREADS * 4;
  const unsigned cgrid = (unsigned)((nclu + 3) / 4);
  uint16_t* chat = reinterpret_cast<uint16_t*>(ix.centroids_bf16);
  BigList bl{ws.big, ws.big + 2, reinterpret_cast<uint8_t*>(ws.big + 2 + 2 * BIG_CAP), 0};
  WAVE_TRY(launch("k_init", k_init, dim3((unsigned)units), dim3(INIT_THREADS), init_lds, st, bs, seed, K,
                  ix.centroids, chat, ws.norm, bl));
  const int tpw = assign_tpw(bs, units);
  const int64_t agrid = assign_grid(bs, tpw);
  const unsigned ugrid = cgrid + (bs.ident ? BIG_CAP / 4 : 0);
  for (int it = 0; it < iters; ++it) {
    bl.parity = it & 1;
    if (bs.K_s <= AL_MAXC)
      WAVE_TRY(launch("k_assign", k_assign_lds, dim3((unsigned)agrid), dim3(AL_THREADS), sizeof(AssignLdsL), st, bs,
                      tpw, K, chat, ws.norm, ix.assign));
    else
      WAVE_TRY(launch("k_assign", k_assign<true>, dim3((unsigned)agrid), dim3(AS_THREADS), sizeof(AssignLds), st, bs,
                      tpw, K, chat, ws.norm, ix.assign, ws.xn2, it == 0 ? 1 : 0));
    if (trace != nullptr)
      WAVE_TRY(hipMemcpyAsync(trace + (int64_t)it * rows, ix.assign, sizeof(int32_t) * (size_t)rows,
                              hipMemcpyDeviceToDevice, st));
    if (bs.seg_len <= RS_MAXL)
      WAVE_TRY(launch("k_sort", k_sort_radix, dim3((unsigned)(units * sparts)), dim3(RS_THREADS), radix_lds, st, bs,
                      sparts, ix.assign, ix.sizes, ix.offsets, ix.perm, bl));
    else
      WAVE_TRY(launch("k_sort", k_sort, dim3((unsigned)units), dim3(SORT_THREADS), sort_lds, st, bs, ix.assign,
                      ws.rank, ix.sizes, ix.offsets, ix.perm, bl));
    WAVE_TRY(launch("k_update", it + 1 < iters ? k_update<false> : k_update<true>, dim3(ugrid), dim3(256), 0, st, bs,
                    nclu, K, V, ix, ws.norm, bl));
  }
  return hipSuccess;
}

hipError_t launch_build(const SeqArgs& sa, const void* Kv, const void* Vv, int32_t iters, uint64_t seed,
                        const wave_index& ix, const BuildWs& ws, int32_t* trace, int64_t rows, hipStream_t st) {
  return run_build(whole(sa), reinterpret_cast<const uint16_t*>(Kv), reinterpret_cast<const uint16_t*>(Vv), iters,
                   seed, ix, ws, trace, rows, st);
}

hipError_t launch_append(const SeqArgs& sa, const int32_t* n_old, const void* Kn, const void* Vn, int32_t iters,
                         uint64_t seed, const wave_index& ix, const BuildWs& ws, void* stage_k, void* stage_v,
                         hipStream_t st) {
  BuildSeq bs = whole(sa);
  bs.ident = 0;  // the call's clusters start at each sequence's first changed segment
  StageArgs a;
  a.B = sa.B;
  a.G = sa.G;
  a.seg_len = sa.seg_len;
  a.cap = sa.cap;
  int64_t Mmax = 0;
  for (int b = 0; b < MAXB; ++b) {
    a.n_new[b] = b < sa.B ? sa.N[b] : 0;
    a.n_old[b] = b < sa.B ? n_old[b] : 0;
  }
  for (int b = 0; b < sa.B; ++b) {
    if (sa.N[b] > n_old[b]) {
      bs.first[b] = n_old[b] / sa.seg_len;
      Mmax = std::max<int64_t>(Mmax, sa.N[b] - (int64_t)bs.first[b] * sa.seg_len);
    } else {
      bs.first[b] = (int32_t)host_nseg(bs, b);  // unchanged: no units
    }
  }
  if (Mmax == 0) return hipSuccess;
  uint16_t* Ko = reinterpret_cast<uint16_t*>(stage_k);
  uint16_t* Vo = reinterpret_cast<uint16_t*>(stage_v);
  WAVE_TRY(launch("k_stage", k_stage, dim3((unsigned)(sa.B * sa.G), (unsigned)((Mmax + STAGE_ROWS - 1) / STAGE_ROWS)),
                  dim3(STAGE_ROWS * 16), 0, st, a, reinterpret_cast<const uint16_t*>(Kn),
                  reinterpret_cast<const uint16_t*>(Vn), ix, Ko, Vo));
  return run_build(bs, Ko, Vo, iters, seed, ix, ws, nullptr, 0, st);
}

hipError_t launch_build_blocks(const SeqArgs& sa, const void* Kv, const void* Vv, const wave_index& ix,
                               const BuildWs& ws, hipStream_t st) {
  const DeviceInfo& di = device_info();
  WAVE_TRY(di.status);
  const BuildSeq bs = whole(sa);
  const uint16_t* K = reinterpret_cast<const uint16_t*>(Kv);
  const uint16_t* V = reinterpret_cast<const uint16_t*>(Vv);
  int64_t units, nclu;
  call_counts(bs, &units, &nclu);
  const size_t sort_lds = 16 * (size_t)sa.K_s * 4;
  const int sparts = sort_parts(units, di.cus);
  const size_t radix_tiles = ((size_t)(sa.seg_len + sparts - 1) / sparts + RS_THREADS - 1) / RS_THREADS;
  const size_t radix_lds = 2 * radix_tiles * RS_THREADS * 4;
  const unsigned cgrid = (unsigned)((nclu + 3) / 4);
  const BigList bl{ws.big, ws.big + 2, reinterpret_cast<uint8_t*>(ws.big + 2 + 2 * BIG_CAP), 0};
  WAVE_TRY(launch("k_block_assign", k_block_assign, dim3((unsigned)units), dim3(1024), 0, st, bs, ix.assign, bl));
  // the layout pass of the k-means build over the block labels: counts, offsets, the
  // (identity) order, member means, bf16 centroids, value sums
  if (sa.seg_len <= RS_MAXL)
    WAVE_TRY(launch("k_sort", k_sort_radix, dim3((unsigned)(units * sparts)), dim3(RS_THREADS), radix_lds, st, bs,
                    sparts, ix.assign, ix.sizes, ix.offsets, ix.perm, bl));
  else
    WAVE_TRY(launch("k_sort", k_sort, dim3((unsigned)units), dim3(SORT_THREADS), sort_lds, st, bs, ix.assign,
                    ws.rank, ix.sizes, ix.offsets, ix.perm, bl));
  WAVE_TRY(launch("k_update", k_update<true>, dim3(cgrid + (bs.ident ? BIG_CAP / 4 : 0)), dim3(256), 0, st, bs, nclu,
                  K, V, ix, ws.norm, bl));
  return hipSuccess;
}

}  // namespace wave
