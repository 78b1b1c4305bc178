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
//               (key desc, id asc), the selected ids, the rows to gather
//   k_attend -- two roles in one grid: split-K online-softmax attention over the
//               gathered rows (retrieval + steady), and the estimation term over
//               the value sums of the remaining clusters (HBM bound)
//   k_merge  -- log-sum-exp merge of every partial into out and lse
#include <math.h>

#include "common.h"
#include "internal.h"

namespace wave {

constexpr int SCORE_CH = 256;   // clusters per k_score workgroup
constexpr int TOPK_THREADS = 1024;
constexpr int ATT_THREADS = 256;
constexpr int EST_CH = 256;     // clusters per estimation workgroup
constexpr int SORT_LDS = 8192;  // selections sorted in LDS up to this many
constexpr int PART = 132;       // floats per partial: m, l, 2 pad, acc[128]
constexpr float LOG2E = 1.4426950408889634f;

// ------------------------------------------------------------------ k_score
// Rank key r_{h,j}: 16 lanes each own 8 consecutive dims of the centroid row;
// each lane sums its 8 exact bf16 products from +0 in dim order (an fma of
// two bf16 values is the same as a rounded product then a rounded add), then
// an xor butterfly over the 16 lanes with strides 8, 4, 2, 1, then +0.0f.
template <int GS>
__global__ __launch_bounds__(256) void k_score(SeqArgs sa, int32_t H, const uint16_t* __restrict__ chat,
                                               const uint16_t* __restrict__ q, float* __restrict__ keys) {
  __shared__ float stage[GS][SCORE_CH];
  // workgroup -> (sequence, kv head, chunk)
  int w = blockIdx.x, b = 0;
  int64_t clu = 0;
  for (;; ++b) {
    int nch = (sa.C[b] + SCORE_CH - 1) / SCORE_CH;
    if (w < sa.G * nch) break;
    w -= sa.G * nch;
    clu += (int64_t)sa.G * sa.C[b];
  }
  const int C = sa.C[b];
  const int nch = (C + SCORE_CH - 1) / SCORE_CH;
  const int g = w / nch, chunk = w % nch;
  const int j0 = chunk * SCORE_CH;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, l16 = lane & 15, grp = lane >> 4;
  // q slices of the GS heads of this kv head, 8 dims per lane
  float qf[GS][8];
#pragma unroll
  for (int hh = 0; hh < GS; ++hh) {
    const uint4 v = *reinterpret_cast<const uint4*>(q + ((int64_t)b * H + g * GS + hh) * D + l16 * 8);
    qf[hh][0] = bf16_lo(v.x); qf[hh][1] = bf16_hi(v.x);
    qf[hh][2] = bf16_lo(v.y); qf[hh][3] = bf16_hi(v.y);
    qf[hh][4] = bf16_lo(v.z); qf[hh][5] = bf16_hi(v.z);
    qf[hh][6] = bf16_lo(v.w); qf[hh][7] = bf16_hi(v.w);
  }
  const uint16_t* base = chat + (clu + (int64_t)g * C) * D;
#pragma unroll 4
  for (int it = 0; it < SCORE_CH / 16; ++it) {
    const int jj = it * 16 + wv * 4 + grp;  // row within chunk
    const int j = j0 + jj;
    float c[8];
    if (j < C) {
      const uint4 v = *reinterpret_cast<const uint4*>(base + (int64_t)j * D + l16 * 8);
      c[0] = bf16_lo(v.x); c[1] = bf16_hi(v.x); c[2] = bf16_lo(v.y); c[3] = bf16_hi(v.y);
      c[4] = bf16_lo(v.z); c[5] = bf16_hi(v.z); c[6] = bf16_lo(v.w); c[7] = bf16_hi(v.w);
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) c[m] = 0.f;
    }
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

// ------------------------------------------------------------------ block helpers (1024 threads)
// exclusive scan of a 64-bit value over the workgroup; returns the exclusive
// prefix, *total gets the sum. tmp: LDS of >= 17 uint64.
__device__ inline uint64_t block_scan_excl(uint64_t v, uint64_t* tmp, uint64_t* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint64_t x = v;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    uint64_t y = __shfl_up(x, s, 64);
    if (lane >= s) x += y;
  }
  if (lane == 63) tmp[wv] = x;
  __syncthreads();
  if (wv == 0) {
    uint64_t t = lane < nw ? tmp[lane] : 0;
    uint64_t tt = t;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      uint64_t y = __shfl_up(tt, s, 64);
      if (lane >= s) tt += y;
    }
    if (lane < nw) tmp[lane] = tt - t;  // exclusive wave base
    if (lane == nw - 1) tmp[16] = tt;
  }
  __syncthreads();
  uint64_t r = tmp[wv] + x - v;
  *total = tmp[16];
  __syncthreads();
  return r;
}

// descending bitonic sort of n (power of two) u64 keys
__device__ inline void bitonic_desc(uint64_t* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        int ixj = i ^ j;
        if (ixj > i) {
          uint64_t x = a[i], y = a[ixj];
          bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) { a[i] = y; a[ixj] = x; }
        }
      }
      __syncthreads();
    }
  }
}

__device__ inline void bitonic_asc_i32(int32_t* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        int ixj = i ^ j;
        if (ixj > i) {
          int32_t x = a[i], y = a[ixj];
          bool asc = (i & k) == 0;
          if (asc ? (x > y) : (x < y)) { a[i] = y; a[ixj] = x; }
        }
      }
      __syncthreads();
    }
  }
}

__device__ inline void bitonic_desc_global(uint64_t* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        int ixj = i ^ j;
        if (ixj > i) {
          uint64_t x = a[i], y = a[ixj];
          bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) { a[i] = y; a[ixj] = x; }
        }
      }
      __threadfence_block();
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ k_topk
struct TopkLds {
  int32_t sj[WAVE_MAX_STEADY];     // sorted cluster ids of the steady tokens
  uint32_t filt[4096];             // membership filter of those ids (bit j mod 2^17)
  uint64_t sortbuf[SORT_LDS];
  int32_t hist[256];
  uint64_t scan[17];
  int32_t misc[8];
};

// count of steady tokens in cluster j (0 if none)
__device__ inline int steady_count(const TopkLds& L, int nS_sorted, int32_t j) {
  if (!((L.filt[(j >> 5) & 4095] >> (j & 31)) & 1u)) return 0;
  int lo = 0, hi = nS_sorted;
  while (lo < hi) { int mid = (lo + hi) >> 1; if (L.sj[mid] < j) lo = mid + 1; else hi = mid; }
  int a = lo;
  hi = nS_sorted;
  while (lo < hi) { int mid = (lo + hi) >> 1; if (L.sj[mid] <= j) lo = mid + 1; else hi = mid; }
  return lo - a;
}

__global__ __launch_bounds__(TOPK_THREADS) void k_topk(SeqArgs sa, DecodeArgs da, wave_index ix, DecodeWs ws,
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
  const int tid = threadIdx.x, nt = blockDim.x;
  // per-(b, h) workspace slices
  const int64_t kbase = (int64_t)da.GS * sb.clu + (int64_t)h * C;  // keys / key32
  const int nwords = (C + 31) >> 5;
  int64_t wbase = 0, rbase = 0;
  for (int i = 0; i < b; ++i) {
    wbase += (int64_t)da.H * ((sa.C[i] + 31) >> 5);
    rbase += (int64_t)da.H * sa.N[i];
  }
  wbase += (int64_t)h * nwords;
  rbase += (int64_t)h * N;
  const float* keys = ws.keys + kbase;
  uint32_t* key32 = ws.key32 + kbase;
  uint32_t* excl = ws.excl + wbase;
  int32_t* rows = ws.rows + rbase;
  int32_t* selid = ws.selid + kbase;   // id-order selection (capacity C)
  int32_t* selpre = ws.selpre + (int64_t)da.GS * sb.off + (int64_t)h * (C + 1);  // member-count prefix
  float* corr = ws.corr + (int64_t)bh * da.scap;
  const int32_t* sizes = ix.sizes + clu0;
  const int32_t* offs = ix.offsets + off0;

  // 1. steady zone S = [0, a) U [c, N)
  const int64_t a_end = min((int64_t)da.n_sink, (int64_t)N);
  const int64_t c_beg = max((int64_t)N - (int64_t)da.n_local, a_end);
  const int nS = (int)(a_end + (N - c_beg));
  const bool allS = (nS == N);
  int nSs = 0;  // entries in L.sj
  if (!allS && nS > 0) {
    int P2 = 1;
    while (P2 < nS) P2 <<= 1;
    for (int i = tid; i < 4096; i += nt) L.filt[i] = 0u;
    for (int i = tid; i < P2; i += nt) {
      if (i < nS) {
        int64_t t = i < a_end ? i : c_beg + (i - a_end);
        L.sj[i] = ix.assign[row0 + t];
      } else {
        L.sj[i] = 0x7FFFFFFF;
      }
    }
    __syncthreads();
    for (int i = tid; i < nS; i += nt) {
      int32_t j = L.sj[i];
      atomicOr(&L.filt[(j >> 5) & 4095], 1u << (j & 31));
    }
    bitonic_asc_i32(L.sj, P2);
    nSs = nS;
  }
  if (tid == 0) L.misc[0] = 0;
  __syncthreads();

  // 2. eligibility, sortable keys, |E|, exclusion bits of non-empty ineligible clusters
  {
    const int lane = tid & 63;
    int myE = 0;
    for (int base = (tid >> 6) * 64; base < C; base += nt) {
      const int j = base + lane;
      bool nonempty = false, elig = false;
      float r = 0.f;
      if (j < C) {
        int n = sizes[j];
        nonempty = n > 0;
        if (nonempty && !allS) elig = (n - (nSs ? steady_count(L, nSs, j) : 0)) > 0;
        r = keys[j];
        key32[j] = elig ? float_sortable(r) : 0u;
      }
      myE += elig ? 1 : 0;
      uint64_t m = __ballot(nonempty && !elig);
      const int wd = base >> 5;
      if (lane == 0 && wd < nwords) excl[wd] = (uint32_t)m;
      if (lane == 1 && wd + 1 < nwords) excl[wd + 1] = (uint32_t)(m >> 32);
    }
    atomicAdd(&L.misc[0], myE);
  }
  __syncthreads();
  const int nE = L.misc[0];
  const int k = min(da.kreq[b], nE);

  // 3. radix select of the k-th largest key (4 passes of 8 bits) over per-thread runs
  const int R = (C + nt - 1) / nt;
  const int r0 = min(tid * R, C), r1 = min(r0 + R, C);
  uint32_t T = 0xFFFFFFFFu;
  int k_eq = 0;
  if (k > 0) {
    uint32_t prefix = 0, mask = 0;
    int kk = k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < 256; i += nt) L.hist[i] = 0;
      __syncthreads();
      for (int j = r0; j < r1; ++j) {
        uint32_t u = key32[j];
        if ((u & mask) == prefix) atomicAdd(&L.hist[(u >> shift) & 255], 1);
      }
      __syncthreads();
      if (tid < 64) {
        const int lane = tid;
        int h0 = L.hist[4 * lane], h1 = L.hist[4 * lane + 1], h2 = L.hist[4 * lane + 2], h3 = L.hist[4 * lane + 3];
        int s = h0 + h1 + h2 + h3;
        int incl = s;  // inclusive suffix over lanes >= lane
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          int y = __shfl_down(incl, o, 64);
          if (lane + o < 64) incl += y;
        }
        int above = incl - s;  // keys in lanes above
        int suf3 = above + h3, suf2 = suf3 + h2, suf1 = suf2 + h1, suf0 = suf1 + h0;
        int cand = -1, cab = 0;
        if (suf3 >= kk) { cand = 4 * lane + 3; cab = above; }
        else if (suf2 >= kk) { cand = 4 * lane + 2; cab = suf3; }
        else if (suf1 >= kk) { cand = 4 * lane + 1; cab = suf2; }
        else if (suf0 >= kk) { cand = 4 * lane; cab = suf1; }
        // highest candidate bin over the wave
        int best = cand;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) best = max(best, __shfl_xor(best, o, 64));
        if (cand == best && cand >= 0) { L.misc[1] = cand; L.misc[2] = cab; }
      }
      __syncthreads();
      const int d = L.misc[1];
      kk -= L.misc[2];
      prefix |= (uint32_t)d << shift;
      mask |= 255u << shift;
      __syncthreads();
    }
    T = prefix;
    k_eq = kk;
  }

  // 4. the selected ids in id order: every key > T and the k_eq lowest ids with key == T
  int64_t nMem = 0;
  if (k > 0) {
    int ngt = 0, neq = 0;
    for (int j = r0; j < r1; ++j) {
      uint32_t u = key32[j];
      ngt += u > T;
      neq += u == T;
    }
    uint64_t tot;
    uint64_t pre = block_scan_excl(((uint64_t)ngt << 32) | (uint32_t)neq, L.scan, &tot);
    const int gt_before = (int)(pre >> 32), eq_before = (int)(pre & 0xFFFFFFFFu);
    int take = min(max(k_eq - eq_before, 0), neq);
    int pos = gt_before + min(eq_before, k_eq);
    for (int j = r0; j < r1; ++j) {
      uint32_t u = key32[j];
      bool s = u > T;
      if (!s && u == T && take > 0) { s = true; --take; }
      if (s) {
        selid[pos] = j;
        uint64_t comp = ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)j);
        if (k <= SORT_LDS) L.sortbuf[pos] = comp; else ws.sortg[(int64_t)bh * da.sort_stride + pos] = comp;
        atomicOr(&excl[j >> 5], 1u << (j & 31));
        ++pos;
      }
    }
    __syncthreads();
    // rank order for the output ids
    int P2 = 1;
    while (P2 < k) P2 <<= 1;
    if (k <= SORT_LDS) {
      for (int i = k + tid; i < P2; i += nt) L.sortbuf[i] = 0;
      __syncthreads();
      bitonic_desc(L.sortbuf, P2);
    } else {
      uint64_t* sg = ws.sortg + (int64_t)bh * da.sort_stride;  // stride: next power of two >= max C_b
      for (int i = k + tid; i < P2; i += nt) sg[i] = 0;
      __threadfence_block();
      __syncthreads();
      bitonic_desc_global(sg, P2);
    }
    int32_t* out = sel_ids + (int64_t)bh * da.k_max;
    for (int i = tid; i < k; i += nt) {
      uint64_t comp = (k <= SORT_LDS) ? L.sortbuf[i] : ws.sortg[(int64_t)bh * da.sort_stride + i];
      out[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(comp & 0xFFFFFFFFu));
    }
    // prefix of member counts over the id-order selection
    const int Rk = (k + nt - 1) / nt;
    const int q0 = min(tid * Rk, k), q1 = min(q0 + Rk, k);
    int64_t msum = 0;
    for (int i = q0; i < q1; ++i) msum += sizes[selid[i]];
    uint64_t mtot;
    uint64_t mpre = block_scan_excl((uint64_t)msum, L.scan, &mtot);
    int64_t run = (int64_t)mpre;
    for (int i = q0; i < q1; ++i) {
      selpre[i] = (int32_t)run;
      run += sizes[selid[i]];
    }
    if (tid == 0) selpre[k] = (int32_t)mtot;
    nMem = (int64_t)mtot;
  }
  if (sel_ids != nullptr) {
    int32_t* out = sel_ids + (int64_t)bh * da.k_max;
    for (int i = k + tid; i < da.k_max; i += nt) out[i] = -1;
  }
  __threadfence_block();
  __syncthreads();

  // 5. rows to gather: non-steady members of the selected clusters, in id order
  int Tr = 0;
  if (k > 0) {
    const int64_t M = nMem;
    const int64_t Rm = (M + nt - 1) / nt;
    const int64_t f0 = min((int64_t)tid * Rm, M), f1 = min(f0 + Rm, M);
    // locate the cluster of f0
    int lo = 0, hi = k;  // last i with selpre[i] <= f0
    while (hi - lo > 1) { int mid = (lo + hi) >> 1; if (selpre[mid] <= f0) lo = mid; else hi = mid; }
    int cnt = 0;
    {
      int ci = lo;
      for (int64_t f = f0; f < f1; ++f) {
        while (selpre[ci + 1] <= f) ++ci;
        const int32_t j = selid[ci];
        const int32_t p = offs[j] + (int32_t)(f - selpre[ci]);
        const int32_t t = ix.perm[row0 + p];
        cnt += !(t < a_end || t >= c_beg);
      }
    }
    uint64_t tot;
    int pos = (int)block_scan_excl((uint64_t)cnt, L.scan, &tot);
    Tr = (int)tot;
    {
      int ci = lo;
      for (int64_t f = f0; f < f1; ++f) {
        while (selpre[ci + 1] <= f) ++ci;
        const int32_t j = selid[ci];
        const int32_t p = offs[j] + (int32_t)(f - selpre[ci]);
        const int32_t t = ix.perm[row0 + p];
        if (!(t < a_end || t >= c_beg)) rows[pos++] = p;
      }
    }
  }
  __threadfence_block();
  __syncthreads();

  // 6. steady rows, with the estimation correction of their clusters
  for (int i = tid; i < nS; i += nt) {
    const int64_t t = i < a_end ? i : c_beg + (i - a_end);
    rows[Tr + i] = ix.inv_perm[row0 + t];
    float cv = __uint_as_float(0x7FC00000u);  // NaN: no correction
    if (!allS) {
      const int32_t j = ix.assign[row0 + t];
      const int n = sizes[j];
      const bool elig = (n - steady_count(L, nSs, j)) > 0;
      const bool inR = (excl[j >> 5] >> (j & 31)) & 1u;
      if (elig && !inR) cv = keys[j];
    }
    corr[i] = cv;
  }
  if (tid == 0) {
    ws.counts[2 * bh] = Tr;
    ws.counts[2 * bh + 1] = Tr + nS;
  }
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

template <int GS>
__global__ __launch_bounds__(ATT_THREADS) void k_attend(SeqArgs sa, DecodeArgs da, wave_index ix, DecodeWs ws,
                                                        const uint16_t* __restrict__ q) {
  __shared__ float red[4][PART];
  __shared__ float wts[GS][EST_CH];
  __shared__ float hred[GS][4][2];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, l16 = lane & 15, grp = lane >> 4;
  const float sc = da.tau * LOG2E;  // scores in log2 units
  const int nret = sa.B * da.H * da.P;
  if ((int)blockIdx.x < nret) {
    // ---------------- retrieval + steady role: rows [i0, i1) of one (b, h)
    const int bh = blockIdx.x / da.P, part = blockIdx.x % da.P;
    const int b = bh / da.H, h = bh % da.H, g = h / da.GS;
    const SeqBase sb = seq_base(sa, b);
    const int N = sb.N;
    const int64_t row0 = sb.row + (int64_t)g * N;
    int64_t rbase = 0;
    for (int i = 0; i < b; ++i) rbase += (int64_t)da.H * sa.N[i];
    rbase += (int64_t)h * N;
    const int Tr = ws.counts[2 * bh], T = ws.counts[2 * bh + 1];
    const int i0 = (int)((int64_t)T * part / da.P), i1 = (int)((int64_t)T * (part + 1) / da.P);
    float qf[8];
    {
      const uint4 v = *reinterpret_cast<const uint4*>(q + (int64_t)bh * D + l16 * 8);
      qf[0] = bf16_lo(v.x) * sc; qf[1] = bf16_hi(v.x) * sc; qf[2] = bf16_lo(v.y) * sc; qf[3] = bf16_hi(v.y) * sc;
      qf[4] = bf16_lo(v.z) * sc; qf[5] = bf16_hi(v.z) * sc; qf[6] = bf16_lo(v.w) * sc; qf[7] = bf16_hi(v.w) * sc;
    }
    const uint16_t* Ks = reinterpret_cast<const uint16_t*>(ix.k_sorted) + row0 * D + l16 * 8;
    const uint16_t* Vs = reinterpret_cast<const uint16_t*>(ix.v_sorted) + row0 * D + l16 * 8;
    const int32_t* rows = ws.rows + rbase;
    const float* corr = ws.corr + (int64_t)bh * da.scap;
    float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] = 0.f;
    for (int i = i0 + wv * 4 + grp; i < i1; i += 16) {
      const int32_t p = rows[i];
      const uint4 kv = *reinterpret_cast<const uint4*>(Ks + (int64_t)p * D);
      const uint4 vv = *reinterpret_cast<const uint4*>(Vs + (int64_t)p * D);
      float s = qf[0] * bf16_lo(kv.x);
      s = fmaf(qf[1], bf16_hi(kv.x), s); s = fmaf(qf[2], bf16_lo(kv.y), s); s = fmaf(qf[3], bf16_hi(kv.y), s);
      s = fmaf(qf[4], bf16_lo(kv.z), s); s = fmaf(qf[5], bf16_hi(kv.z), s); s = fmaf(qf[6], bf16_lo(kv.w), s);
      s = fmaf(qf[7], bf16_hi(kv.w), s);
      s += xor_shfl(s, 8);
      s += xor_shfl(s, 4);
      s += xor_shfl(s, 2);
      s += xor_shfl(s, 1);
      float cs = -INFINITY;
      if (i >= Tr) {
        const float cv = corr[i - Tr];
        if (cv == cv) cs = cv * sc;
      }
      const float mn = fmaxf(m, fmaxf(s, cs));
      const float a = exp2f(m - mn);
      const float w = exp2f(s - mn) - exp2f(cs - mn);
      l = l * a + w;
      float v[8] = {bf16_lo(vv.x), bf16_hi(vv.x), bf16_lo(vv.y), bf16_hi(vv.y),
                    bf16_lo(vv.z), bf16_hi(vv.z), bf16_lo(vv.w), bf16_hi(vv.w)};
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] = fmaf(w, v[d], acc[d] * a);
      m = mn;
    }
    // merge the 4 row groups of the wave (lanes l16, l16+16, +32, +48)
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      float m2 = xor_shfl(m, o), l2 = xor_shfl(l, o), a2[8];
#pragma unroll
      for (int d = 0; d < 8; ++d) a2[d] = xor_shfl(acc[d], o);
      merge_state(m, l, acc, m2, l2, a2, 8);
    }
    if (grp == 0) {
      if (l16 == 0) { red[wv][0] = m; red[wv][1] = l; }
#pragma unroll
      for (int d = 0; d < 8; ++d) red[wv][4 + l16 * 8 + d] = acc[d];
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
      float* out = ws.part + ((int64_t)bh * da.NP + part) * PART;
      if (d == 0) { out[0] = M; out[1] = Ls; }
      out[4 + d] = A;
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
  // weights exp2(s - m_h) of valid clusters (non-empty, not excluded), chunk max per head
  {
    const int jj = threadIdx.x;  // EST_CH == blockDim
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
      if (threadIdx.x == 0) hred[hh][0][0] = M;  // keep the chunk max
    }
    __syncthreads();
  }
  // value sums, 16 lanes per row, 8 dims per lane
  float acc[GS][8];
#pragma unroll
  for (int hh = 0; hh < GS; ++hh)
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[hh][d] = 0.f;
  const float* vs = ix.vsum + clu0 * D + l16 * 8;
  for (int jj = wv * 4 + grp; jj < EST_CH; jj += 16) {
    const int j = j0 + jj;
    if (j >= C) break;
    bool any = false;
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) any |= wts[hh][jj] != 0.f;
    if (!any) continue;
    const float4 v0 = *reinterpret_cast<const float4*>(vs + (int64_t)j * D);
    const float4 v1 = *reinterpret_cast<const float4*>(vs + (int64_t)j * D + 4);
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      const float wgt = wts[hh][jj];
      acc[hh][0] = fmaf(wgt, v0.x, acc[hh][0]); acc[hh][1] = fmaf(wgt, v0.y, acc[hh][1]);
      acc[hh][2] = fmaf(wgt, v0.z, acc[hh][2]); acc[hh][3] = fmaf(wgt, v0.w, acc[hh][3]);
      acc[hh][4] = fmaf(wgt, v1.x, acc[hh][4]); acc[hh][5] = fmaf(wgt, v1.y, acc[hh][5]);
      acc[hh][6] = fmaf(wgt, v1.z, acc[hh][6]); acc[hh][7] = fmaf(wgt, v1.w, acc[hh][7]);
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
  // sum the 4 waves per head through LDS, one head at a time
  for (int hh = 0; hh < GS; ++hh) {
    if (grp == 0)
#pragma unroll
      for (int d = 0; d < 8; ++d) red[wv][4 + l16 * 8 + d] = acc[hh][d];
    __syncthreads();
    if (threadIdx.x < D) {
      const int d = threadIdx.x;
      const int h = g * GS + hh;
      const int bh = b * da.H + h;
      float* out = ws.part + ((int64_t)bh * da.NP + da.P + chunk) * PART;
      const float A = red[0][4 + d] + red[1][4 + d] + red[2][4 + d] + red[3][4 + d];
      const float Ls = hred[hh][0][1] + hred[hh][1][1] + hred[hh][2][1] + hred[hh][3][1];
      const float M = hred[hh][0][0];
      if (d == 0) { out[0] = (Ls > 0.f) ? M : -INFINITY; out[1] = Ls; }
      out[4 + d] = A;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ k_merge
__global__ __launch_bounds__(D) void k_merge(SeqArgs sa, DecodeArgs da, DecodeWs ws, float* __restrict__ out,
                                             float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const int b = bh / da.H;
  const int npart = da.P + (sa.C[b] + EST_CH - 1) / EST_CH;
  const float* pp = ws.part + (int64_t)bh * da.NP * PART;
  const int d = threadIdx.x;
  float M = -INFINITY;
  for (int i = 0; i < npart; ++i) M = fmaxf(M, pp[(int64_t)i * PART]);
  float Ls = 0.f, A = 0.f;
  for (int i = 0; i < npart; ++i) {
    const float mi = pp[(int64_t)i * PART];
    if (mi == -INFINITY) continue;
    const float f = exp2f(mi - M);
    Ls += pp[(int64_t)i * PART + 1] * f;
    A += pp[(int64_t)i * PART + 4 + d] * f;
  }
  out[(int64_t)bh * D + d] = A / Ls;
  if (lse != nullptr && d == 0) lse[bh] = (M + log2f(Ls)) * 0.6931471805599453f;
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
  hipLaunchKernelGGL(k_topk, dim3(sa.B * da.H), dim3(TOPK_THREADS), sizeof(TopkLds), st, sa, da, ix, ws, sel_ids);
  prof_end(st);
  prof_begin("k_attend", st);
  hipLaunchKernelGGL(k_attend<GS>, dim3(sa.B * da.H * da.P + nest), dim3(ATT_THREADS), 0, st, sa, da, ix, ws, q);
  prof_end(st);
  prof_begin("k_merge", st);
  hipLaunchKernelGGL(k_merge, dim3(sa.B * da.H), dim3(D), 0, st, sa, da, ws, out, lse);
  prof_end(st);
}

hipError_t launch_decode(const SeqArgs& sa, const DecodeArgs& da, const wave_index& ix, const DecodeWs& ws,
                         const uint16_t* q, float* out, int32_t* sel_ids, float* lse, hipStream_t st) {
  static bool attrs = false;
  if (!attrs) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_topk), hipFuncAttributeMaxDynamicSharedMemorySize,
                        sizeof(TopkLds));
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
