// decode.hip -- query-dependent phase of wave-index attention on gfx950.
//
// RetroInfer summary page, section 2.A: each decode query is scored against
// the cluster centroids, the most similar clusters are fetched for exact
// attention (retrieval zone), sink and recent tokens are attended exactly
// (steady zone), and every other cluster contributes through its centroid
// (estimation zone). Four launches per call, all on the caller's stream:
//   k_score  -- rank keys of every centroid for the H/G q heads of a kv head
//               (one pass over the bf16 centroid rows, HBM bound)
//   k_topk   -- per (sequence, q head): steady set, eligibility, exact top-k by
//               (key desc, id asc), the selected ids and their spans
//   k_attend -- three roles in one grid: online-softmax attention over the
//               selected clusters' sorted rows (one cluster per 16-lane group),
//               over the steady rows, and the estimation term over the value
//               sums of the remaining clusters, each writing a partial state
//   k_merge  -- log-sum-exp merge of the partials of every (sequence, q head)
#include <math.h>

#include "common.h"
#include "internal.h"

namespace wave {

constexpr int SCORE_CH = 64;    // clusters per k_score workgroup
constexpr int TK_THREADS = 1024;
constexpr int TK_HASH = 4096;   // steady-cluster hash slots (>= 2 * WAVE_MAX_STEADY)
constexpr int TK_FILT = 1024;   // filter words: bit (j mod 32768)
constexpr int TK_CAND = 4096;   // threshold-bin candidates refined in LDS
constexpr int TK_EXCL = 2048;   // exclusion words kept in LDS (C <= 65536)
constexpr int TK_RANK_SMALL = 512;
constexpr int ATT_THREADS = 256;
constexpr int EST_CH = DEC_EST_CH;  // clusters per estimation workgroup (== ATT_THREADS)
constexpr int PART = DEC_PART;  // floats per partial: m, l, 2 pad, acc[128]
constexpr float LOG2E = 1.4426950408889634f;

static_assert(EST_CH == ATT_THREADS, "one estimation cluster per thread");
static_assert(TK_HASH >= 2 * WAVE_MAX_STEADY, "steady hash load factor");

// ------------------------------------------------------------------ k_score
// Rank key r_{h,j}: 16 lanes each own 8 consecutive dims of the centroid row;
// each lane sums its 8 exact bf16 products from +0 in dim order (an fma of
// two bf16 values equals a rounded product then a rounded add), then an xor
// butterfly over the 16 lanes with strides 8, 4, 2, 1, then +0.0f.
template <int GS>
__global__ __launch_bounds__(256) void k_score(SeqArgs sa, int32_t H, const uint16_t* __restrict__ chat,
                                               const uint16_t* __restrict__ q, float* __restrict__ keys) {
  __shared__ float stage[GS][SCORE_CH];
  int w = blockIdx.x, b = 0;
  int64_t clu = 0;
  for (;; ++b) {
    const int nch = (sa.C[b] + SCORE_CH - 1) / SCORE_CH;
    if (w < sa.G * nch) break;
    w -= sa.G * nch;
    clu += (int64_t)sa.G * sa.C[b];
  }
  const int C = sa.C[b];
  const int nch = (C + SCORE_CH - 1) / SCORE_CH;
  const int g = w / nch, chunk = w % nch;
  const int j0 = chunk * SCORE_CH;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, l16 = lane & 15, grp = lane >> 4;
  const uint16_t* base = chat + (clu + (int64_t)g * C) * D + l16 * 8;
  // issue the row loads first: 4 rows per wave-iteration, 4 iterations
  uint4 cv[SCORE_CH / 16];
#pragma unroll
  for (int it = 0; it < SCORE_CH / 16; ++it) {
    const int j = j0 + it * 16 + wv * 4 + grp;
    cv[it] = (j < C) ? *reinterpret_cast<const uint4*>(base + (int64_t)j * D) : make_uint4(0, 0, 0, 0);
  }
  float qf[GS][8];
#pragma unroll
  for (int hh = 0; hh < GS; ++hh) {
    const uint4 v = *reinterpret_cast<const uint4*>(q + ((int64_t)b * H + g * GS + hh) * D + l16 * 8);
    qf[hh][0] = bf16_lo(v.x); qf[hh][1] = bf16_hi(v.x);
    qf[hh][2] = bf16_lo(v.y); qf[hh][3] = bf16_hi(v.y);
    qf[hh][4] = bf16_lo(v.z); qf[hh][5] = bf16_hi(v.z);
    qf[hh][6] = bf16_lo(v.w); qf[hh][7] = bf16_hi(v.w);
  }
#pragma unroll
  for (int it = 0; it < SCORE_CH / 16; ++it) {
    const int jj = it * 16 + wv * 4 + grp;
    const uint4 v = cv[it];
    const float c[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                        bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      float u = 0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m) u = fmaf(qf[hh][m], c[m], u);
      u += xor_shfl(u, 8);
      u += xor_shfl(u, 4);
      u += xor_shfl(u, 2);
      u += xor_shfl(u, 1);
      if (l16 == hh) stage[hh][jj] = u + 0.0f;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < GS * SCORE_CH; e += blockDim.x) {
    const int hh = e / SCORE_CH, jj = e % SCORE_CH;
    if (j0 + jj < C) keys[(int64_t)GS * clu + (int64_t)(g * GS + hh) * C + j0 + jj] = stage[hh][jj];
  }
}

// ------------------------------------------------------------------ block helpers (TK_THREADS threads)
// exclusive scan of a 64-bit value over the workgroup; *total gets the sum.
__device__ inline uint64_t block_scan_excl(uint64_t v, uint64_t* tmp, uint64_t* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint64_t x = v;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const uint64_t y = __shfl_up(x, s, 64);
    if (lane >= s) x += y;
  }
  if (lane == 63) tmp[wv] = x;
  __syncthreads();
  if (wv == 0) {
    const uint64_t t = lane < nw ? tmp[lane] : 0;
    uint64_t tt = t;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const uint64_t y = __shfl_up(tt, s, 64);
      if (lane >= s) tt += y;
    }
    if (lane < nw) tmp[lane] = tt - t;
    if (lane == nw - 1) tmp[16] = tt;
  }
  __syncthreads();
  const uint64_t r = tmp[wv] + x - v;
  *total = tmp[16];
  __syncthreads();
  return r;
}

// descending bitonic sort of n (power of two) unique u64 keys (LDS or global)
__device__ inline void bitonic_desc(uint64_t* a, int n, bool global) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = a[i], y = a[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) { a[i] = y; a[ixj] = x; }
        }
      }
      if (global) __threadfence_block();
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ k_topk
constexpr int TK_BINS = 8192;   // first radix digit: the top 13 bits of the sortable key

struct TopkLds {
  int32_t hkey[TK_HASH];       // steady clusters: open-addressing hash, -1 = empty
  int32_t hcnt[TK_HASH];       // steady tokens per hashed cluster
  int32_t sj[WAVE_MAX_STEADY]; // cluster of every steady token
  uint32_t filt[TK_FILT];      // steady-cluster filter
  uint32_t hist[TK_BINS];
  union {
    struct {
      uint32_t key[TK_CAND];
      int32_t id[TK_CAND];
    } cand;
    uint64_t sortbuf[TK_CAND];
  } u;
  uint32_t excl[TK_EXCL];
  uint64_t scan[17];
  int32_t misc[16];
};

__device__ __forceinline__ uint32_t hslot(int32_t j) { return ((uint32_t)j * 2654435761u) >> 20; }

__device__ inline int steady_count(const TopkLds& L, int32_t j) {
  if (!((L.filt[(j >> 5) & (TK_FILT - 1)] >> (j & 31)) & 1u)) return 0;
  uint32_t h = hslot(j);
  for (;;) {
    const int32_t k = L.hkey[h];
    if (k == j) return L.hcnt[h];
    if (k < 0) return 0;
    h = (h + 1) & (TK_HASH - 1);
  }
}

// largest bin d of hist[0..nbins) whose suffix count reaches kk (nbins a multiple of
// TK_THREADS or equal to it); writes d and the count strictly above it to misc[1], misc[2]
__device__ inline void find_bin(TopkLds& L, int nbins, int kk) {
  const int tid = threadIdx.x;
  const int per = nbins / TK_THREADS;
  const int hi = nbins - 1 - per * tid;  // this thread's bins hi, hi-1, ..., hi-per+1
  uint64_t local = 0;
  for (int e = 0; e < per; ++e) local += L.hist[hi - e];
  uint64_t tot;
  uint64_t above = block_scan_excl(local, L.scan, &tot);
  for (int e = 0; e < per; ++e) {
    const uint64_t suf = above + L.hist[hi - e];
    if (above < (uint64_t)kk && suf >= (uint64_t)kk) {
      L.misc[1] = hi - e;
      L.misc[2] = (int)above;
    }
    above = suf;
  }
  __syncthreads();
}


// member-count prefix of the id-order selection (selpre[0..k]) and the per-(b, h)
// counts record {rows of the selected clusters, k, steady rows, 0}
__device__ inline void selection_prefix(TopkLds& L, const DecodeWs& ws, int64_t kbase, int bh, int k, int nS) {
  __threadfence_block();
  __syncthreads();
  const int tid = threadIdx.x, nt = blockDim.x;
  const int2* span = ws.span + kbase;
  int32_t* selpre = ws.selpre + kbase + bh;  // k+1 entries per (b, h)
  const int R = (k + nt - 1) / nt;
  const int q0 = min(tid * R, k), q1 = min(q0 + R, k);
  int64_t msum = 0;
  for (int i = q0; i < q1; ++i) msum += span[i].y;
  uint64_t tot;
  int64_t run = (int64_t)block_scan_excl((uint64_t)msum, L.scan, &tot);
  for (int i = q0; i < q1; ++i) {
    selpre[i] = (int32_t)run;
    run += span[i].y;
  }
  if (tid == 0) {
    selpre[k] = (int32_t)tot;
    ws.counts[4 * bh + 0] = (int32_t)tot;
    ws.counts[4 * bh + 1] = k;
    ws.counts[4 * bh + 2] = nS;
    ws.counts[4 * bh + 3] = 0;
  }
}

// Per (sequence b, q head h), any number of clusters. Ids are split into 16
// contiguous wave ranges, each walked 64 ids at a time (lane = id offset), so
// every pass is coalesced and the order of ids inside a wave follows the lanes.
// The sortable keys are kept in global memory between passes.
__global__ __launch_bounds__(TK_THREADS) void k_topk_any(SeqArgs sa, DecodeArgs da, wave_index ix, DecodeWs ws,
                                                         int32_t* __restrict__ sel_ids) {
  extern __shared__ uint8_t smem[];
  TopkLds& L = *reinterpret_cast<TopkLds*>(smem);
  const int bh = blockIdx.x;
  const int b = bh / da.H, h = bh % da.H;
  const int g = h / da.GS;
  const SeqBase sb = seq_base(sa, b);
  const int N = sb.N, C = sb.C;
  const int64_t row0 = sb.row + (int64_t)g * N;
  const int64_t clu0 = sb.clu + (int64_t)g * C;
  const int64_t off0 = sb.off + (int64_t)g * (C + 1);
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wv = tid >> 6;
  const int64_t kbase = (int64_t)da.GS * sb.clu + (int64_t)h * C;
  const int nwords = (C + 31) >> 5;
  int64_t wbase = 0;
  for (int i = 0; i < b; ++i) wbase += (int64_t)da.H * ((sa.C[i] + 31) >> 5);
  wbase += (int64_t)h * nwords;
  const float* keys = ws.keys + kbase;
  uint32_t* key32 = ws.key32 + kbase;
  uint32_t* excl_g = ws.excl + wbase;
  int2* span = ws.span + kbase;  // (first sorted slot, size) of the i-th selection in id order
  float* corr = ws.corr + (int64_t)bh * da.scap;
  const int32_t* sizes = ix.sizes + clu0;
  const int32_t* offs = ix.offsets + off0;
  const bool lds_excl = nwords <= TK_EXCL;
  // this wave's id range [w0, w1)
  const int wspan = ((C + 15) / 16 + 63) & ~63;
  const int w0 = min(wv * wspan, C), w1 = min(w0 + wspan, C);

  // 0. LDS init
  for (int i = tid; i < TK_HASH; i += nt) { L.hkey[i] = -1; L.hcnt[i] = 0; }
  for (int i = tid; i < TK_FILT; i += nt) L.filt[i] = 0u;
  for (int i = tid; i < TK_BINS; i += nt) L.hist[i] = 0u;
  if (lds_excl)
    for (int i = tid; i < nwords; i += nt) L.excl[i] = 0u;
  else
    for (int i = tid; i < nwords; i += nt) excl_g[i] = 0u;
  if (tid < 16) L.misc[tid] = 0;
  __threadfence_block();
  __syncthreads();

  // 1. steady zone S = [0, a) U [c, N): count the steady tokens of every cluster
  const int64_t a_end = min((int64_t)da.n_sink, (int64_t)N);
  const int64_t c_beg = max((int64_t)N - (int64_t)da.n_local, a_end);
  const int nS = (int)(a_end + (N - c_beg));
  const bool allS = (nS == N);
  if (!allS) {
    for (int i = tid; i < nS; i += nt) {
      const int64_t t = i < a_end ? i : c_beg + (i - a_end);
      const int32_t j = ix.assign[row0 + t];
      L.sj[i] = j;
      atomicOr(&L.filt[(j >> 5) & (TK_FILT - 1)], 1u << (j & 31));
      uint32_t hs = hslot(j);
      for (;;) {
        const int32_t prev = atomicCAS(&L.hkey[hs], -1, j);
        if (prev == -1 || prev == j) {
          atomicAdd(&L.hcnt[hs], 1);
          break;
        }
        hs = (hs + 1) & (TK_HASH - 1);
      }
    }
  }
  __syncthreads();

  // 2. eligibility (some member outside S), sortable keys, |E|, top-13-bit histogram;
  //    non-empty clusters that are not eligible are excluded from the estimation zone
  {
    int myE = 0;
    for (int j0 = w0; j0 < w1; j0 += 64) {
      const int j = j0 + lane;
      const bool in = j < w1;
      const int n = in ? sizes[j] : 0;
      const float r = in ? keys[j] : 0.f;
      bool elig = false;
      if (n > 0 && !allS) elig = (n - steady_count(L, j)) > 0;
      const uint32_t u = elig ? float_sortable(r) : 0u;
      if (in) key32[j] = u;
      if (elig) {
        ++myE;
        atomicAdd(&L.hist[u >> 19], 1u);
      } else if (n > 0) {
        if (lds_excl) atomicOr(&L.excl[j >> 5], 1u << (j & 31));
        else atomicOr(&excl_g[j >> 5], 1u << (j & 31));
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) myE += __shfl_xor(myE, o, 64);
    if (lane == 0) atomicAdd(&L.misc[0], myE);
  }
  __threadfence_block();
  __syncthreads();
  const int nE = L.misc[0];
  const int k = min(da.kreq[b], nE);

  // 3. threshold key T (the k-th largest key32) and k_eq, the number of keys equal to T taken
  uint32_t T = 0xFFFFFFFFu;
  int k_eq = 0;
  if (k > 0) {
    find_bin(L, TK_BINS, k);
    const int d1 = L.misc[1];
    int kk = k - L.misc[2];
    // candidates: keys whose top 13 bits are d1
    for (int j0 = w0; j0 < w1; j0 += 64) {
      const int j = j0 + lane;
      const uint32_t u = j < w1 ? key32[j] : 0u;
      if (j < w1 && (int)(u >> 19) == d1) {
        const int p = atomicAdd(&L.misc[3], 1);
        if (p < TK_CAND) { L.u.cand.key[p] = u; L.u.cand.id[p] = j; }
      }
    }
    __syncthreads();
    const int nc = L.misc[3];
    if (nc <= TK_RANK_SMALL) {
      // few candidates: the kk-th by (key desc, id asc) by counting
      if (tid < nc) {
        const uint32_t u = L.u.cand.key[tid];
        const int id = L.u.cand.id[tid];
        int rank = 0;
#pragma unroll 8
        for (int i = 0; i < nc; ++i) {
          const uint32_t v = L.u.cand.key[i];
          rank += (v > u) || (v == u && L.u.cand.id[i] < id);
        }
        if (rank == kk - 1) L.misc[4] = (int)u;
      }
      __syncthreads();
      T = (uint32_t)L.misc[4];
      // keys == T above the kk-th candidate are all taken: count them among candidates
      if (tid == 0) {
        int eq_gt = 0;
#pragma unroll 8
        for (int i = 0; i < nc; ++i) eq_gt += L.u.cand.key[i] > T;
        L.misc[5] = kk - eq_gt;
      }
      __syncthreads();
      k_eq = L.misc[5];
    } else {
      // radix passes over bits 18..9 and 8..0 (candidates in LDS, or all keys)
      const bool in_lds = nc <= TK_CAND;
      uint32_t prefix = (uint32_t)d1 << 19, mask = 0xFFF80000u;
      for (int pass = 0; pass < 2; ++pass) {
        const int sh = pass == 0 ? 9 : 0, nb = pass == 0 ? 1024 : 512;
        for (int i = tid; i < 1024; i += nt) L.hist[i] = 0u;
        __syncthreads();
        if (in_lds) {
          for (int i = tid; i < nc; i += nt) {
            const uint32_t u = L.u.cand.key[i];
            if ((u & mask) == prefix) atomicAdd(&L.hist[(u >> sh) & (nb - 1)], 1u);
          }
        } else {
          for (int j = tid; j < C; j += nt) {
            const uint32_t u = key32[j];
            if ((u & mask) == prefix) atomicAdd(&L.hist[(u >> sh) & (nb - 1)], 1u);
          }
        }
        __syncthreads();
        find_bin(L, 1024, kk);  // bins >= nb are empty
        prefix |= (uint32_t)L.misc[1] << sh;
        mask |= (uint32_t)(nb - 1) << sh;
        kk -= L.misc[2];
        __syncthreads();
      }
      T = prefix;
      k_eq = kk;
    }
  }

  // 4. the selection in id order: keys > T and the k_eq lowest ids with key == T
  if (k > 0) {
    int ngt = 0, neq = 0;
    for (int j0 = w0; j0 < w1; j0 += 64) {
      const int j = j0 + lane;
      const uint32_t u = j < w1 ? key32[j] : 0u;
      ngt += __popcll(__ballot(j < w1 && u > T));
      neq += __popcll(__ballot(j < w1 && u == T));
    }
    uint64_t tot;
    const uint64_t v = (lane == 0) ? (((uint64_t)ngt << 32) | (uint32_t)neq) : 0ull;
    const uint64_t pre = block_scan_excl(v, L.scan, &tot);
    const uint64_t wpre = __shfl(pre, 0, 64);
    int eq_seen = (int)(wpre & 0xFFFFFFFFu);
    int pos = (int)(wpre >> 32) + min(eq_seen, k_eq);
    const uint64_t ltmask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int j0 = w0; j0 < w1; j0 += 64) {
      const int j = j0 + lane;
      const uint32_t u = j < w1 ? key32[j] : 0u;
      const bool eq = j < w1 && u == T;
      const uint64_t eqm = __ballot(eq);
      const bool s = (j < w1 && u > T) || (eq && eq_seen + __popcll(eqm & ltmask) < k_eq);
      const uint64_t sm = __ballot(s);
      if (s) {
        const int p = pos + __popcll(sm & ltmask);
        span[p] = make_int2(offs[j], sizes[j]);
        const uint64_t comp = ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)j);
        if (k <= TK_CAND) L.u.sortbuf[p] = comp;
        else ws.sortg[(int64_t)bh * da.sort_stride + p] = comp;
        if (lds_excl) atomicOr(&L.excl[j >> 5], 1u << (j & 31));
        else atomicOr(&excl_g[j >> 5], 1u << (j & 31));
      }
      pos += __popcll(sm);
      eq_seen += __popcll(eqm);
    }
    __threadfence_block();
    __syncthreads();
    // 5. rank order (key desc, id asc) of the output ids
    int32_t* out = sel_ids + (int64_t)bh * da.k_max;
    if (k <= TK_RANK_SMALL) {
      if (tid < k) {
        const uint64_t c = L.u.sortbuf[tid];
        int rank = 0;
#pragma unroll 8
        for (int i = 0; i < k; ++i) rank += L.u.sortbuf[i] > c;
        out[rank] = (int32_t)(0xFFFFFFFFu - (uint32_t)(c & 0xFFFFFFFFu));
      }
    } else {
      int P2 = 1;
      while (P2 < k) P2 <<= 1;
      uint64_t* a = (k <= TK_CAND) ? L.u.sortbuf : ws.sortg + (int64_t)bh * da.sort_stride;
      for (int i = k + tid; i < P2; i += nt) a[i] = 0;
      if (k > TK_CAND) __threadfence_block();
      __syncthreads();
      bitonic_desc(a, P2, k > TK_CAND);
      for (int i = tid; i < k; i += nt) out[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(a[i] & 0xFFFFFFFFu));
    }
  }
  if (sel_ids != nullptr) {
    int32_t* out = sel_ids + (int64_t)bh * da.k_max;
    for (int i = k + tid; i < da.k_max; i += nt) out[i] = -1;
  }
  __threadfence_block();
  __syncthreads();
  if (lds_excl)
    for (int i = tid; i < nwords; i += nt) excl_g[i] = L.excl[i];

  // 6. steady rows: their cluster's estimation correction (rank key, NaN if none)
  for (int i = tid; i < nS; i += nt) {
    float cv = __uint_as_float(0x7FC00000u);
    if (!allS) {
      const int32_t j = L.sj[i];
      const bool elig = (sizes[j] - steady_count(L, j)) > 0;
      const uint32_t ew = lds_excl ? L.excl[j >> 5] : excl_g[j >> 5];
      if (elig && !((ew >> (j & 31)) & 1u)) cv = keys[j];
    }
    corr[i] = cv;
  }
  selection_prefix(L, ws, kbase, bh, k, nS);
}


// Per (sequence b, q head h) with C <= 16 * 64 * NV clusters. Wave w owns ids
// [w * 64 * NV, (w + 1) * 64 * NV); lane L holds ids w0 + 256 * blk + 4 * L + e
// (blk < NV / 4, e < 4), so each load instruction covers 256 consecutive ids and
// the order of ids inside a wave is (blk, lane, e). Up to 16 keys per lane stay
// in registers through every pass; larger NV keep them in global memory and
// reload 16 per lane at a time.
template <int NV>
__global__ __launch_bounds__(TK_THREADS) void k_topk_reg(SeqArgs sa, DecodeArgs da, wave_index ix, DecodeWs ws,
                                                         int32_t* __restrict__ sel_ids) {
  constexpr int CHK = NV < 16 ? NV : 16;  // keys per lane per chunk
  constexpr bool INREG = NV <= 16;
  extern __shared__ uint8_t smem[];
  TopkLds& L = *reinterpret_cast<TopkLds*>(smem);
  const int bh = blockIdx.x;
  const int b = bh / da.H, h = bh % da.H;
  const int g = h / da.GS;
  const SeqBase sb = seq_base(sa, b);
  const int N = sb.N, C = sb.C;
  const int64_t row0 = sb.row + (int64_t)g * N;
  const int64_t clu0 = sb.clu + (int64_t)g * C;
  const int64_t off0 = sb.off + (int64_t)g * (C + 1);
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wv = tid >> 6;
  const int64_t kbase = (int64_t)da.GS * sb.clu + (int64_t)h * C;
  const int nwords = (C + 31) >> 5;
  int64_t wbase = 0;
  for (int i = 0; i < b; ++i) wbase += (int64_t)da.H * ((sa.C[i] + 31) >> 5);
  wbase += (int64_t)h * nwords;
  const float* keys = ws.keys + kbase;
  uint32_t* key32 = ws.key32 + kbase;
  uint32_t* excl_g = ws.excl + wbase;
  int2* span = ws.span + kbase;
  float* corr = ws.corr + (int64_t)bh * da.scap;
  const int32_t* sizes = ix.sizes + clu0;
  const int32_t* offs = ix.offsets + off0;
  const int w0 = wv * 64 * NV;
  auto id_of = [&](int v) { return w0 + 256 * (v >> 2) + 4 * lane + (v & 3); };

  // 0. LDS init, with the lane's first chunk of sizes and keys in flight
  int nn[CHK];
  float rr[CHK];
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int v = 0; v < CHK; ++v) {
      const int j = id_of(c0 + v);
      nn[v] = j < C ? sizes[j] : 0;
      rr[v] = j < C ? keys[j] : 0.f;
    }
  };
  load_chunk(0);
  // the steady tokens' clusters (at most WAVE_MAX_STEADY = 2 per thread) in flight too
  const int64_t a_end = min((int64_t)da.n_sink, (int64_t)N);
  const int64_t c_beg = max((int64_t)N - (int64_t)da.n_local, a_end);
  const int nS = (int)(a_end + (N - c_beg));
  const bool allS = (nS == N);
  int32_t sjr[2] = {0, 0};
  if (!allS) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = tid + r * TK_THREADS;
      if (i < nS) sjr[r] = ix.assign[row0 + (i < a_end ? i : c_beg + (i - a_end))];
    }
  }
  for (int i = tid; i < TK_HASH; i += nt) { L.hkey[i] = -1; L.hcnt[i] = 0; }
  for (int i = tid; i < TK_FILT; i += nt) L.filt[i] = 0u;
  for (int i = tid; i < TK_BINS; i += nt) L.hist[i] = 0u;
  for (int i = tid; i < nwords; i += nt) L.excl[i] = 0u;
  if (tid < 16) L.misc[tid] = 0;
  __syncthreads();

  // 1. steady zone S = [0, a) U [c, N): count the steady tokens of every cluster
  if (!allS) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = tid + r * TK_THREADS;
      if (i < nS) {
        const int32_t j = sjr[r];
        L.sj[i] = j;
        atomicOr(&L.filt[(j >> 5) & (TK_FILT - 1)], 1u << (j & 31));
        uint32_t hs = hslot(j);
        for (;;) {
          const int32_t prev = atomicCAS(&L.hkey[hs], -1, j);
          if (prev == -1 || prev == j) {
            atomicAdd(&L.hcnt[hs], 1);
            break;
          }
          hs = (hs + 1) & (TK_HASH - 1);
        }
      }
    }
  }
  __syncthreads();

  // 2. eligibility, sortable keys, |E|, top-13-bit histogram, exclusions
  uint32_t ureg[INREG ? NV : 1];
  auto chunk_keys = [&](int c0, uint32_t* uc) {  // the lane's CHK keys of chunk c0
    if constexpr (INREG) {
#pragma unroll
      for (int v = 0; v < CHK; ++v) uc[v] = ureg[c0 + v];
    } else {
#pragma unroll
      for (int v = 0; v < CHK; ++v) {
        const int j = id_of(c0 + v);
        uc[v] = j < C ? key32[j] : 0u;
      }
    }
  };
  {
    int myE = 0;
#pragma unroll(INREG ? 16 : 1)
    for (int c0 = 0; c0 < NV; c0 += CHK) {
      if (c0 > 0) load_chunk(c0);
#pragma unroll
      for (int v = 0; v < CHK; ++v) {
        const int j = id_of(c0 + v);
        bool elig = false;
        if (nn[v] > 0 && !allS) elig = (nn[v] - steady_count(L, j)) > 0;
        const uint32_t x = elig ? float_sortable(rr[v]) : 0u;
        if constexpr (INREG) ureg[c0 + v] = x;
        else if (j < C) key32[j] = x;
        if (elig) {
          ++myE;
          atomicAdd(&L.hist[x >> 19], 1u);
        } else if (nn[v] > 0) {
          atomicOr(&L.excl[j >> 5], 1u << (j & 31));
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) myE += __shfl_xor(myE, o, 64);
    if (lane == 0) atomicAdd(&L.misc[0], myE);
  }
  __threadfence_block();
  __syncthreads();
  const int nE = L.misc[0];
  const int k = min(da.kreq[b], nE);

  // 3. threshold key T and k_eq
  uint32_t T = 0xFFFFFFFFu;
  int k_eq = 0;
  if (k > 0) {
    find_bin(L, TK_BINS, k);
    const int d1 = L.misc[1];
    int kk = k - L.misc[2];
#pragma unroll(INREG ? 16 : 1)
    for (int c0 = 0; c0 < NV; c0 += CHK) {
      uint32_t uc[CHK];
      chunk_keys(c0, uc);
#pragma unroll
      for (int v = 0; v < CHK; ++v) {
        if (uc[v] != 0u && (int)(uc[v] >> 19) == d1) {
          const int p = atomicAdd(&L.misc[3], 1);
          if (p < TK_CAND) { L.u.cand.key[p] = uc[v]; L.u.cand.id[p] = id_of(c0 + v); }
        }
      }
    }
    __syncthreads();
    const int nc = L.misc[3];
    if (nc <= TK_RANK_SMALL) {
      if (tid < nc) {
        const uint32_t x = L.u.cand.key[tid];
        const int id = L.u.cand.id[tid];
        int rank = 0;
#pragma unroll 8
        for (int i = 0; i < nc; ++i) {
          const uint32_t y = L.u.cand.key[i];
          rank += (y > x) || (y == x && L.u.cand.id[i] < id);
        }
        if (rank == kk - 1) L.misc[4] = (int)x;
      }
      __syncthreads();
      T = (uint32_t)L.misc[4];
      // candidates above T are taken; the rest of the kk come from keys equal to T
      if (tid < nc && L.u.cand.key[tid] > T) atomicAdd(&L.misc[5], 1);
      __syncthreads();
      k_eq = kk - L.misc[5];
    } else {
      const bool in_lds = nc <= TK_CAND;
      uint32_t prefix = (uint32_t)d1 << 19, mask = 0xFFF80000u;
      for (int pass = 0; pass < 2; ++pass) {
        const int sh = pass == 0 ? 9 : 0, nb = pass == 0 ? 1024 : 512;
        for (int i = tid; i < 1024; i += nt) L.hist[i] = 0u;
        __syncthreads();
        if (in_lds) {
          for (int i = tid; i < nc; i += nt) {
            const uint32_t x = L.u.cand.key[i];
            if ((x & mask) == prefix) atomicAdd(&L.hist[(x >> sh) & (nb - 1)], 1u);
          }
        } else {
#pragma unroll(INREG ? 16 : 1)
          for (int c0 = 0; c0 < NV; c0 += CHK) {
            uint32_t uc[CHK];
            chunk_keys(c0, uc);
#pragma unroll
            for (int v = 0; v < CHK; ++v)
              if ((uc[v] & mask) == prefix) atomicAdd(&L.hist[(uc[v] >> sh) & (nb - 1)], 1u);
          }
        }
        __syncthreads();
        find_bin(L, 1024, kk);
        prefix |= (uint32_t)L.misc[1] << sh;
        mask |= (uint32_t)(nb - 1) << sh;
        kk -= L.misc[2];
        __syncthreads();
      }
      T = prefix;
      k_eq = kk;
    }
  }

  // 4. the selection in id order (keys > T, then the k_eq lowest ids with key == T)
  if (k > 0) {
    int ngt = 0, neq = 0;
#pragma unroll(INREG ? 16 : 1)
    for (int c0 = 0; c0 < NV; c0 += CHK) {
      uint32_t uc[CHK];
      chunk_keys(c0, uc);
#pragma unroll
      for (int v = 0; v < CHK; ++v) {
        ngt += uc[v] > T;
        neq += (uc[v] == T);
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      ngt += __shfl_xor(ngt, o, 64);
      neq += __shfl_xor(neq, o, 64);
    }
    uint64_t tot;
    const uint64_t pre = block_scan_excl(lane == 0 ? (((uint64_t)ngt << 32) | (uint32_t)neq) : 0ull, L.scan, &tot);
    const uint64_t wpre = __shfl(pre, 0, 64);
    int eq_seen = (int)(wpre & 0xFFFFFFFFu);
    int pos = (int)(wpre >> 32) + min(eq_seen, k_eq);
#pragma unroll(INREG ? 16 : 1)
    for (int c0 = 0; c0 < NV; c0 += CHK) {
      uint32_t uc[CHK];
      chunk_keys(c0, uc);
      // spans of the chunk's ids, fetched unconditionally (clamped) so the loads overlap
      int ofv[CHK], szv[CHK];
#pragma unroll
      for (int v = 0; v < CHK; ++v) {
        const int j = min(id_of(c0 + v), C - 1);
        ofv[v] = offs[j];
        szv[v] = sizes[j];
      }
      // per block of 256 ids: lane-order prefix of (eq, selected) counts
#pragma unroll
      for (int bb = 0; bb < CHK / 4; ++bb) {
        int ce = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) ce += (uc[4 * bb + e] == T);
        int xe = ce;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(xe, o, 64);
          if (lane >= o) xe += y;
        }
        int er = eq_seen + xe - ce;
        bool sel[4];
        int cs = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x = uc[4 * bb + e];
          bool sv = x > T;
          if (x == T) { sv = er < k_eq; ++er; }
          sel[e] = sv;
          cs += sv;
        }
        int xs = cs;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(xs, o, 64);
          if (lane >= o) xs += y;
        }
        int p = pos + xs - cs;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (sel[e]) {
            const int j = id_of(c0 + 4 * bb + e);
            span[p] = make_int2(ofv[4 * bb + e], szv[4 * bb + e]);
            const uint64_t comp = ((uint64_t)uc[4 * bb + e] << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)j);
            if (k <= TK_CAND) L.u.sortbuf[p] = comp;
            else ws.sortg[(int64_t)bh * da.sort_stride + p] = comp;
            atomicOr(&L.excl[j >> 5], 1u << (j & 31));
            ++p;
          }
        }
        pos += __shfl(xs, 63, 64);
        eq_seen += __shfl(xe, 63, 64);
      }
    }
    __threadfence_block();
    __syncthreads();
    // 5. rank order (key desc, id asc) of the output ids
    int32_t* out = sel_ids + (int64_t)bh * da.k_max;
    if (k <= TK_RANK_SMALL) {
      if (tid < k) {
        const uint64_t c = L.u.sortbuf[tid];
        int rank = 0;
#pragma unroll 8
        for (int i = 0; i < k; ++i) rank += L.u.sortbuf[i] > c;
        out[rank] = (int32_t)(0xFFFFFFFFu - (uint32_t)(c & 0xFFFFFFFFu));
      }
    } else {
      int P2 = 1;
      while (P2 < k) P2 <<= 1;
      uint64_t* sa_ = (k <= TK_CAND) ? L.u.sortbuf : ws.sortg + (int64_t)bh * da.sort_stride;
      for (int i = k + tid; i < P2; i += nt) sa_[i] = 0;
      if (k > TK_CAND) __threadfence_block();
      __syncthreads();
      bitonic_desc(sa_, P2, k > TK_CAND);
      for (int i = tid; i < k; i += nt) out[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(sa_[i] & 0xFFFFFFFFu));
    }
  }
  if (sel_ids != nullptr) {
    int32_t* out = sel_ids + (int64_t)bh * da.k_max;
    for (int i = k + tid; i < da.k_max; i += nt) out[i] = -1;
  }
  __syncthreads();
  for (int i = tid; i < nwords; i += nt) excl_g[i] = L.excl[i];

  // 6. steady rows: their cluster's estimation correction (rank key, NaN if none)
  for (int i = tid; i < nS; i += nt) {
    float cv = __uint_as_float(0x7FC00000u);
    if (!allS) {
      const int32_t j = L.sj[i];
      const bool elig = (sizes[j] - steady_count(L, j)) > 0;
      if (elig && !((L.excl[j >> 5] >> (j & 31)) & 1u)) cv = keys[j];
    }
    corr[i] = cv;
  }
  selection_prefix(L, ws, kbase, bh, k, nS);
}

// ------------------------------------------------------------------ k_attend
__device__ inline void merge_state(float& m, float& l, float* acc, float m2, float l2, const float* acc2, int n) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  const float a = exp2f(m - M), c = exp2f(m2 - M);
  l = l * a + l2 * c;
  for (int i = 0; i < n; ++i) acc[i] = acc[i] * a + acc2[i] * c;
  m = M;
}

// running softmax state of one 16-lane group (8 dims per lane), scores in log2 units
struct RowState {
  float m, l, acc[8];
};

__device__ __forceinline__ float dot8(const float* qf, uint4 kv) {
  float s = qf[0] * bf16_lo(kv.x);
  s = fmaf(qf[1], bf16_hi(kv.x), s);
  s = fmaf(qf[2], bf16_lo(kv.y), s);
  s = fmaf(qf[3], bf16_hi(kv.y), s);
  s = fmaf(qf[4], bf16_lo(kv.z), s);
  s = fmaf(qf[5], bf16_hi(kv.z), s);
  s = fmaf(qf[6], bf16_lo(kv.w), s);
  s = fmaf(qf[7], bf16_hi(kv.w), s);
  s += xor_shfl(s, 8);
  s += xor_shfl(s, 4);
  s += xor_shfl(s, 2);
  s += xor_shfl(s, 1);
  return s;
}

// U rows at once: scores s[u] (-inf when masked), estimation corrections cs[u] (-inf if none)
template <int U>
__device__ __forceinline__ void softmax_rows(RowState& st, const float* s, const float* cs, const uint4* vv) {
  float mn = st.m;
#pragma unroll
  for (int u = 0; u < U; ++u) mn = fmaxf(mn, fmaxf(s[u], cs[u]));
  if (mn == -INFINITY) return;
  const float a = exp2f(st.m - mn);
  st.l *= a;
#pragma unroll
  for (int d = 0; d < 8; ++d) st.acc[d] *= a;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float w = exp2f(s[u] - mn) - exp2f(cs[u] - mn);
    st.l += w;
    const float v[8] = {bf16_lo(vv[u].x), bf16_hi(vv[u].x), bf16_lo(vv[u].y), bf16_hi(vv[u].y),
                        bf16_lo(vv[u].z), bf16_hi(vv[u].z), bf16_lo(vv[u].w), bf16_hi(vv[u].w)};
#pragma unroll
    for (int d = 0; d < 8; ++d) st.acc[d] = fmaf(w, v[d], st.acc[d]);
  }
  st.m = mn;
}

template <int GS>
__global__ __launch_bounds__(ATT_THREADS) void k_attend(SeqArgs sa, DecodeArgs da, wave_index ix, DecodeWs ws,
                                                        const uint16_t* __restrict__ q) {
  __shared__ float red[4][PART];
  __shared__ float wts[GS][EST_CH];
  __shared__ float hred[GS][4][2];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, l16 = lane & 15, grp = lane >> 4;
  const int gi = wv * 4 + grp;  // 16-lane group in the workgroup
  const float sc = da.tau * LOG2E;
  const int per_bh = da.P;
  const int nret = sa.B * da.H * per_bh;
  if ((int)blockIdx.x < nret) {
    // ---------------- gathered rows of one (b, h): the members of the selected
    // clusters (id order, steady members skipped), then the steady rows.
    // Workgroup `part` takes rows [part*T/P, (part+1)*T/P), each 16-lane group a
    // contiguous 1/16 of that.
    const int bh = blockIdx.x / per_bh, part = blockIdx.x % per_bh;
    const int b = bh / da.H, h = bh % da.H, g = h / da.GS;
    const SeqBase sb = seq_base(sa, b);
    const int N = sb.N;
    const int64_t row0 = sb.row + (int64_t)g * N;
    const int64_t kbase = (int64_t)da.GS * sb.clu + (int64_t)h * sb.C;
    const int M = ws.counts[4 * bh + 0], k = ws.counts[4 * bh + 1], nS = ws.counts[4 * bh + 2];
    const int T = M + nS;
    const int64_t a_end = min((int64_t)da.n_sink, (int64_t)N);
    const int64_t c_beg = max((int64_t)N - (int64_t)da.n_local, a_end);
    const int i0 = (int)((int64_t)T * part / per_bh), i1 = (int)((int64_t)T * (part + 1) / per_bh);
    const int s0 = i0 + (int)((int64_t)(i1 - i0) * gi / 16), s1 = i0 + (int)((int64_t)(i1 - i0) * (gi + 1) / 16);
    float qf[8];
    {
      const uint4 v = *reinterpret_cast<const uint4*>(q + (int64_t)bh * D + l16 * 8);
      qf[0] = bf16_lo(v.x) * sc; qf[1] = bf16_hi(v.x) * sc; qf[2] = bf16_lo(v.y) * sc; qf[3] = bf16_hi(v.y) * sc;
      qf[4] = bf16_lo(v.z) * sc; qf[5] = bf16_hi(v.z) * sc; qf[6] = bf16_lo(v.w) * sc; qf[7] = bf16_hi(v.w) * sc;
    }
    const uint16_t* Ks = reinterpret_cast<const uint16_t*>(ix.k_sorted) + row0 * D + l16 * 8;
    const uint16_t* Vs = reinterpret_cast<const uint16_t*>(ix.v_sorted) + row0 * D + l16 * 8;
    const int32_t* selpre = ws.selpre + kbase + bh;
    const int2* span = ws.span + kbase;
    const float* corr = ws.corr + (int64_t)bh * da.scap;
    RowState st;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) st.acc[d] = 0.f;
    // window of 16 selected clusters [ci0, ci0 + 16) held one per lane of the group:
    // wpre = first row of the cluster, wsx = its first sorted slot
    const int gbase = grp * 16;
    int ci0 = 0, wpre = 0x7FFFFFFF, wsx = 0, wend = 0;
    auto load_window = [&](int c0) {
      ci0 = c0;
      const int c = c0 + l16;
      wpre = c <= k ? selpre[c] : 0x7FFFFFFF;
      wsx = c < k ? span[c].x : 0;
      wend = __shfl(c0 + 16 <= k ? selpre[min(c0 + 16, k)] : 0x7FFFFFFF, gbase, 64);
    };
    if (s0 < min(s1, M)) {
      // 16-ary search for the last cluster whose first row is <= s0
      int lo = 0, hi = k;
      while (hi - lo > 1) {
        const int step = (hi - lo + 15) / 16;
        const int c = lo + l16 * step;
        const int v = c < hi ? selpre[c] : 0x7FFFFFFF;
        const uint32_t m = (uint32_t)(__ballot(v <= s0) >> gbase) & 0xFFFFu;
        const int cnt = __popc(m);
        lo = lo + (cnt - 1) * step;
        hi = min(lo + step, hi);
      }
      load_window(lo);
    }
    constexpr int U = 4;
    // members of the selected clusters: rows [s0, min(s1, M))
    const int r1 = min(s1, M);
    for (int r = s0; r < r1; r += U) {
      if (r + U - 1 >= wend) {
        // re-anchor the window at the cluster of row r; r <= wend here (the previous
        // batch ended inside the window), and r == wend starts cluster ci0 + 16. A window
        // anchored at r's cluster reaches at least 16 rows past r (clusters are non-empty).
        const uint32_t m0 = (uint32_t)(__ballot(wpre <= r) >> gbase) & 0xFFFFu;
        load_window(r >= wend ? ci0 + 16 : ci0 + __popc(m0) - 1);
      }
      uint4 kv[U], vv[U];
      int32_t t[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = min(r + u, r1 - 1);
        const uint32_t m = (uint32_t)(__ballot(wpre <= row) >> gbase) & 0xFFFFu;
        const int l = __popc(m) - 1;
        const int32_t p = __shfl(wsx, gbase + l, 64) + row - __shfl(wpre, gbase + l, 64);
        t[u] = ix.perm[row0 + p];
        kv[u] = *reinterpret_cast<const uint4*>(Ks + (int64_t)p * D);
        vv[u] = *reinterpret_cast<const uint4*>(Vs + (int64_t)p * D);
      }
      float sv[U], cs[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float x = dot8(qf, kv[u]);
        const bool keep = (r + u < r1) && !(t[u] < a_end || t[u] >= c_beg);
        sv[u] = keep ? x : -INFINITY;
        cs[u] = -INFINITY;
      }
      softmax_rows<U>(st, sv, cs, vv);
    }
    // steady rows: entries e = row - M for rows [max(s0, M), s1)
    for (int r = max(s0, M); r < s1; r += U) {
      int32_t p[U];
      float cvv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = min(r + u, s1 - 1) - M;
        const int64_t tt = e < a_end ? e : c_beg + (e - a_end);
        p[u] = ix.inv_perm[row0 + tt];
        cvv[u] = corr[e];
      }
      uint4 kv[U], vv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kv[u] = *reinterpret_cast<const uint4*>(Ks + (int64_t)p[u] * D);
        vv[u] = *reinterpret_cast<const uint4*>(Vs + (int64_t)p[u] * D);
      }
      float sv[U], cs[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float x = dot8(qf, kv[u]);
        const bool valid = r + u < s1;
        sv[u] = valid ? x : -INFINITY;
        cs[u] = (valid && cvv[u] == cvv[u]) ? cvv[u] * sc : -INFINITY;
      }
      softmax_rows<U>(st, sv, cs, vv);
    }
    // merge the 4 groups of the wave, then the 4 waves
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      const float m2 = xor_shfl(st.m, o), l2 = xor_shfl(st.l, o);
      float a2[8];
#pragma unroll
      for (int d = 0; d < 8; ++d) a2[d] = xor_shfl(st.acc[d], o);
      merge_state(st.m, st.l, st.acc, m2, l2, a2, 8);
    }
    if (grp == 0) {
      if (l16 == 0) { red[wv][0] = st.m; red[wv][1] = st.l; }
#pragma unroll
      for (int d = 0; d < 8; ++d) red[wv][4 + l16 * 8 + d] = st.acc[d];
    }
    __syncthreads();
    if (threadIdx.x < D) {
      const int d = threadIdx.x;
      float M = -INFINITY;
      for (int w2 = 0; w2 < 4; ++w2) M = fmaxf(M, red[w2][0]);
      float Ls = 0.f, A = 0.f;
      if (M != -INFINITY)
        for (int w2 = 0; w2 < 4; ++w2) {
          const float f = exp2f(red[w2][0] - M);
          Ls += red[w2][1] * f;
          A += red[w2][4 + d] * f;
        }
      float* o = ws.part + ((int64_t)bh * da.NP + part) * PART;
      if (d == 0) { o[0] = M; o[1] = Ls; }
      o[4 + d] = A;
    }
    return;
  }
  // ---------------- estimation role: clusters [j0, j0 + EST_CH) of one (b, g), all GS heads
  int w = blockIdx.x - nret, b = 0;
  for (;; ++b) {
    const int nch = (sa.C[b] + EST_CH - 1) / EST_CH;
    if (w < sa.G * nch) break;
    w -= sa.G * nch;
  }
  const SeqBase sb = seq_base(sa, b);
  const int C = sb.C;
  const int nch = (C + EST_CH - 1) / EST_CH;
  const int g = w / nch, chunk = w % nch;
  const int j0 = chunk * EST_CH;
  const int64_t clu0 = sb.clu + (int64_t)g * C;
  const int nwords = (C + 31) >> 5;
  int64_t wbase = 0;
  for (int i = 0; i < b; ++i) wbase += (int64_t)da.H * ((sa.C[i] + 31) >> 5);
  {
    const int jj = threadIdx.x;
    const int j = j0 + jj;
    const int n = j < C ? ix.sizes[clu0 + j] : 0;
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      const int h = g * GS + hh;
      float s = -INFINITY;
      if (n > 0) {
        const uint32_t ew = ws.excl[wbase + (int64_t)h * nwords + (j >> 5)];
        if (!((ew >> (j & 31)) & 1u)) s = ws.keys[(int64_t)GS * sb.clu + (int64_t)h * C + j] * sc;
      }
      float mx = s;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, xor_shfl(mx, o));
      if (lane == 0) hred[hh][wv][0] = mx;
      wts[hh][jj] = s;
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      const float M = fmaxf(fmaxf(hred[hh][0][0], hred[hh][1][0]), fmaxf(hred[hh][2][0], hred[hh][3][0]));
      const float s = wts[hh][jj];
      const float wgt = (s == -INFINITY) ? 0.f : exp2f(s - M);
      float ls = wgt * (float)n;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) ls += xor_shfl(ls, o);
      __syncthreads();
      wts[hh][jj] = wgt;
      if (lane == 0) hred[hh][wv][1] = ls;
      if (threadIdx.x == 0) hred[hh][0][0] = M;
    }
    __syncthreads();
  }
  float acc[GS][8];
#pragma unroll
  for (int hh = 0; hh < GS; ++hh)
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[hh][d] = 0.f;
  const float* vs = ix.vsum + clu0 * D + l16 * 8;
  constexpr int UE = 4;
  for (int jb = gi; jb < EST_CH; jb += 16 * UE) {
    float4 v0[UE], v1[UE];
#pragma unroll
    for (int u = 0; u < UE; ++u) {
      const int j = min(j0 + jb + 16 * u, C - 1);
      v0[u] = *reinterpret_cast<const float4*>(vs + (int64_t)j * D);
      v1[u] = *reinterpret_cast<const float4*>(vs + (int64_t)j * D + 4);
    }
#pragma unroll
    for (int u = 0; u < UE; ++u) {
      const int jj = jb + 16 * u;
      if (jj >= EST_CH || j0 + jj >= C) continue;
#pragma unroll
      for (int hh = 0; hh < GS; ++hh) {
        const float wgt = wts[hh][jj];
        acc[hh][0] = fmaf(wgt, v0[u].x, acc[hh][0]); acc[hh][1] = fmaf(wgt, v0[u].y, acc[hh][1]);
        acc[hh][2] = fmaf(wgt, v0[u].z, acc[hh][2]); acc[hh][3] = fmaf(wgt, v0[u].w, acc[hh][3]);
        acc[hh][4] = fmaf(wgt, v1[u].x, acc[hh][4]); acc[hh][5] = fmaf(wgt, v1[u].y, acc[hh][5]);
        acc[hh][6] = fmaf(wgt, v1[u].z, acc[hh][6]); acc[hh][7] = fmaf(wgt, v1[u].w, acc[hh][7]);
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < GS; ++hh) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      acc[hh][d] += xor_shfl(acc[hh][d], 16);
      acc[hh][d] += xor_shfl(acc[hh][d], 32);
    }
  }
  for (int hh = 0; hh < GS; ++hh) {
    if (grp == 0)
#pragma unroll
      for (int d = 0; d < 8; ++d) red[wv][4 + l16 * 8 + d] = acc[hh][d];
    __syncthreads();
    const int h = g * GS + hh;
    const int bh = b * da.H + h;
    if (threadIdx.x < D) {
      const int d = threadIdx.x;
      float* o = ws.part + ((int64_t)bh * da.NP + da.P + chunk) * PART;
      const float A = red[0][4 + d] + red[1][4 + d] + red[2][4 + d] + red[3][4 + d];
      const float Ls = hred[hh][0][1] + hred[hh][1][1] + hred[hh][2][1] + hred[hh][3][1];
      const float M = hred[hh][0][0];
      if (d == 0) { o[0] = (Ls > 0.f) ? M : -INFINITY; o[1] = Ls; }
      o[4 + d] = A;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ k_merge
// Log-sum-exp merge of the partials of one (b, h): thread (sub, dq) takes dims
// 4dq..4dq+3 over partials sub, sub + 8, ...; the 8 subsets meet in LDS.
__global__ __launch_bounds__(256) void k_merge(SeqArgs sa, DecodeArgs da, DecodeWs ws, float* __restrict__ out,
                                               float* __restrict__ lse) {
  __shared__ float4 accs[8][32];
  __shared__ float ls[8];
  __shared__ float mx[4];
  const int bh = blockIdx.x;
  const int b = bh / da.H;
  const int npart = da.P + (sa.C[b] + EST_CH - 1) / EST_CH;
  const float* pp = ws.part + (int64_t)bh * da.NP * PART;
  const int tid = threadIdx.x, dq = tid & 31, sub = tid >> 5;
  float M = -INFINITY;
  for (int i = tid; i < npart; i += 256) M = fmaxf(M, pp[(int64_t)i * PART]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, xor_shfl(M, o));
  if ((tid & 63) == 0) mx[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
  float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
  float Ls = 0.f;
#pragma unroll 4
  for (int i = sub; i < npart; i += 8) {
    const float* p = pp + (int64_t)i * PART;
    const float mi = p[0];
    const float4 a = *reinterpret_cast<const float4*>(p + 4 + 4 * dq);
    const float li = p[1];
    const float f = (mi == -INFINITY) ? 0.f : exp2f(mi - M);
    Ls += li * f;
    A.x += a.x * f; A.y += a.y * f; A.z += a.z * f; A.w += a.w * f;
  }
  accs[sub][dq] = A;
  if (dq == 0) ls[sub] = Ls;
  __syncthreads();
  if (tid < 32) {
    float4 s = accs[0][tid];
    float Lt = ls[0];
    for (int k = 1; k < 8; ++k) {
      const float4 t = accs[k][tid];
      s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
      Lt += ls[k];
    }
    float4 r;
    r.x = s.x / Lt; r.y = s.y / Lt; r.z = s.z / Lt; r.w = s.w / Lt;
    *reinterpret_cast<float4*>(out + (int64_t)bh * D + 4 * tid) = r;
    if (lse != nullptr && tid == 0) lse[bh] = (M + log2f(Lt)) * 0.6931471805599453f;
  }
}

// ------------------------------------------------------------------ host side
size_t topk_lds_bytes() { return sizeof(TopkLds); }

template <int GS>
static void launch_gs(const SeqArgs& sa, const DecodeArgs& da, const wave_index& ix, const DecodeWs& ws,
                      const uint16_t* q, float* out, int32_t* sel_ids, float* lse, hipStream_t st, int nscore,
                      int nest) {
  const uint16_t* chat = reinterpret_cast<const uint16_t*>(ix.centroids_bf16);
  prof_begin("k_score", st);
  hipLaunchKernelGGL(k_score<GS>, dim3(nscore), dim3(256), 0, st, sa, da.H, chat, q, ws.keys);
  prof_end(st);
  prof_begin("k_topk", st);
  const dim3 tg(sa.B * da.H), tb(TK_THREADS);
  const size_t tl = sizeof(TopkLds);
  switch (da.NV) {
    case 4: hipLaunchKernelGGL(k_topk_reg<4>, tg, tb, tl, st, sa, da, ix, ws, sel_ids); break;
    case 8: hipLaunchKernelGGL(k_topk_reg<8>, tg, tb, tl, st, sa, da, ix, ws, sel_ids); break;
    case 16: hipLaunchKernelGGL(k_topk_reg<16>, tg, tb, tl, st, sa, da, ix, ws, sel_ids); break;
    case 32: hipLaunchKernelGGL(k_topk_reg<32>, tg, tb, tl, st, sa, da, ix, ws, sel_ids); break;
    case 64: hipLaunchKernelGGL(k_topk_reg<64>, tg, tb, tl, st, sa, da, ix, ws, sel_ids); break;
    default: hipLaunchKernelGGL(k_topk_any, tg, tb, tl, st, sa, da, ix, ws, sel_ids); break;
  }
  prof_end(st);
  prof_begin("k_attend", st);
  hipLaunchKernelGGL(k_attend<GS>, dim3(sa.B * da.H * da.P + nest), dim3(ATT_THREADS), 0, st, sa, da, ix,
                     ws, q);
  prof_end(st);
  prof_begin("k_merge", st);
  hipLaunchKernelGGL(k_merge, dim3(sa.B * da.H), dim3(256), 0, st, sa, da, ws, out, lse);
  prof_end(st);
}

hipError_t launch_decode(const SeqArgs& sa, const DecodeArgs& da, const wave_index& ix, const DecodeWs& ws,
                         const uint16_t* q, float* out, int32_t* sel_ids, float* lse, hipStream_t st) {
  static bool attrs = false;
  if (!attrs) {
    const void* fns[] = {reinterpret_cast<const void*>(&k_topk_any), reinterpret_cast<const void*>(&k_topk_reg<4>),
                         reinterpret_cast<const void*>(&k_topk_reg<8>), reinterpret_cast<const void*>(&k_topk_reg<16>),
                         reinterpret_cast<const void*>(&k_topk_reg<32>),
                         reinterpret_cast<const void*>(&k_topk_reg<64>)};
    for (const void* f : fns)
      (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, sizeof(TopkLds));
    attrs = true;
  }
  int nscore = 0, nest = 0;
  for (int b = 0; b < sa.B; ++b) {
    nscore += sa.G * ((sa.C[b] + SCORE_CH - 1) / SCORE_CH);
    nest += sa.G * ((sa.C[b] + EST_CH - 1) / EST_CH);
  }
  switch (da.GS) {
    case 1: launch_gs<1>(sa, da, ix, ws, q, out, sel_ids, lse, st, nscore, nest); break;
    case 2: launch_gs<2>(sa, da, ix, ws, q, out, sel_ids, lse, st, nscore, nest); break;
    case 3: launch_gs<3>(sa, da, ix, ws, q, out, sel_ids, lse, st, nscore, nest); break;
    case 4: launch_gs<4>(sa, da, ix, ws, q, out, sel_ids, lse, st, nscore, nest); break;
    case 5: launch_gs<5>(sa, da, ix, ws, q, out, sel_ids, lse, st, nscore, nest); break;
    case 6: launch_gs<6>(sa, da, ix, ws, q, out, sel_ids, lse, st, nscore, nest); break;
    case 7: launch_gs<7>(sa, da, ix, ws, q, out, sel_ids, lse, st, nscore, nest); break;
    default: launch_gs<8>(sa, da, ix, ws, q, out, sel_ids, lse, st, nscore, nest); break;
  }
  return hipGetLastError();
}

}  // namespace wave
