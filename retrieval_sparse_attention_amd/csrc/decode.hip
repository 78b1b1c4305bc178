// decode.hip -- query-dependent phase of wave-index attention on gfx950.
//
// RetroInfer summary page, section 2.A: each decode query is scored against
// the cluster centroids, the most similar clusters are fetched for exact
// attention (retrieval zone), sink and recent tokens are attended exactly
// (steady zone), and every other cluster contributes through its centroid
// (estimation zone). Four launches per call, all on the caller's stream:
//   k_score  -- one pass over the centroid rows of a kv head: rank keys of the
//               H/G q heads (or, selection shared by the kv head, their sum) and
//               eligibility; with tokens appended after the build, their exact
//               attention too (tail workgroups, one partial per q head)
//   k_topk   -- per (sequence, q head): exact top-k by (key desc, id asc), the
//               selected ids and spans, steady-row corrections
//   k_attend -- two roles in one grid: online-softmax attention over the selected
//               clusters' sorted rows and over the steady rows (every row of a
//               cluster whose centroid term is counted takes that term back out);
//               and the estimation term of every cluster (one pass over the value
//               sums) as partial softmax states
//   k_merge  -- log-sum-exp merge of the partials of every (sequence, q head): the
//               row workgroups', the estimation chunks' and the tail workgroups'
//
// Estimation bookkeeping. The pages' estimation zone is E \ R with the value
// sums and sizes of the clusters' non-steady members. k_score marks the clusters
// outside E (no non-steady member) with a NaN rank key, k_topk leaves each q head's
// selection bitmap in the workspace, and k_attend adds the centroid term
// e^{s_j} (n_j, Vsum_j) of every cluster of E \ R; each steady row t of such a
// cluster adds -e^{s_j} (1, v_t). Summed, this is exactly the centroid term of
// E \ R over the non-steady members, whatever the precision of the stored sums.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace wave {

constexpr int SC = DEC_SCORE_CH;  // clusters per k_score workgroup
constexpr int SCORE_THREADS = 256;
constexpr int TK_WAVES = DEC_TK_WAVES;
constexpr int TK_THREADS = 64 * TK_WAVES;
constexpr int TK_CAP = 1024;      // candidates of the fast selection
constexpr int TK_SORT = DEC_SORT_LDS;
constexpr int TK_SELW = 2048;     // selection bitmap words kept in LDS (C <= 65536)
constexpr int TK_RANK_SMALL = 512;
constexpr int ATT_THREADS = 256;
constexpr int ATT_KCAP = 4 * ATT_THREADS;  // selections whose metadata k_attend stages in LDS
constexpr int ATT_SCAP = 2 * ATT_THREADS;  // steady rows likewise
constexpr int PART = DEC_PART;    // floats per partial: m, l, 2 pad, acc[128]
constexpr float LOG2E = 1.4426950408889634f;

static_assert(SC == 128 && SCORE_THREADS == 256, "k_score thread mapping");

// ------------------------------------------------------------------ steady zone
struct Steady {
  int64_t a_end, c_beg;  // S = [0, a_end) U [c_beg, N)
  int nS;
  bool all;
};

__device__ __forceinline__ Steady steady_of(const DecodeArgs& da, int N) {
  Steady s;
  s.a_end = min((int64_t)da.n_sink, (int64_t)N);
  s.c_beg = max((int64_t)N - (int64_t)da.n_local, s.a_end);
  s.nS = (int)(s.a_end + (N - s.c_beg));
  s.all = s.nS == N;
  return s;
}

// position of steady entry i
__device__ __forceinline__ int64_t steady_pos(const Steady& s, int i) {
  return i < s.a_end ? (int64_t)i : s.c_beg + (i - s.a_end);
}

// ------------------------------------------------------------------ k_score
// Rank key r_{h,j}: 16 lanes each own 8 consecutive dims of the centroid row;
// each lane sums its 8 products in dim order, every product rounded to fp32 on
// its own before it is added (a bf16 x bf16 product is exact in fp32 unless it
// falls below 2^-126 or overflows, so a fused multiply-add would differ there),
// then an xor butterfly over the 16 lanes with strides 8, 4, 2, 1, then +0.0f.
// The lane sum starts at the first product instead of +0 + it: the two differ
// only in the sign of a zero, which every later addition either discards or
// keeps as a zero, and the final +0.0f turns -0 into +0.
//
// One workgroup per (b, g, 128 clusters), 16-lane groups over the centroid rows.
// A cluster is eligible (in E) when it has a member outside the steady zone; the
// steady tokens' clusters are counted only by workgroups whose ids can hold them
// (the first and the last segments).
template <int GS>
struct ScoreLds {
  float kw[GS][SC];   // rank keys
  int32_t nsz[SC];    // cluster sizes
  int32_t scnt[SC];   // steady members
};

template <int GS>
__device__ void tail_role(const SeqArgs& sa, const DecodeArgs& da, const uint16_t* q, const DecodeWs& ws, int w);

// maximum over the wave: rows of 16 by DPP, then lanes i ^ 16 and i ^ 32 (one LDS exchange)
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // row_ror 8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror 4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false));  // row_ror 2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false));  // row_ror 1
  v = max(v, (uint32_t)__shfl_xor((int)v, 16, 64));
  return max(v, swap32(v));
}

// TAIL: the grid also holds the appended-token workgroups (a separate instantiation, so
// that their registers do not lower the scoring workgroups' occupancy elsewhere)
template <int GS, bool TAIL>
__global__ __launch_bounds__(SCORE_THREADS) void k_score(SeqArgs sa, DecodeArgs da, wave_index ix,
                                                         const uint16_t* __restrict__ q, DecodeWs ws) {
  if constexpr (TAIL) {
    if ((int)blockIdx.x >= da.nscore) {
      tail_role<GS>(sa, da, q, ws, blockIdx.x - da.nscore);
      return;
    }
  }
  __shared__ ScoreLds<GS> S;
  int w = blockIdx.x, b = 0;
  for (;; ++b) {
    const int nch = (sa.C[b] + SC - 1) / SC;
    if (w < sa.G * nch) break;
    w -= sa.G * nch;
  }
  const SeqBase sb = seq_base(sa, b);
  const int C = sb.C, N = sb.N;
  const int nch = (C + SC - 1) / SC;
  const int g = w / nch, chunk = w % nch;
  const int j0 = chunk * SC, nc = min(SC, C - j0);
  const int64_t clu0 = sb.clu + (int64_t)g * sb.CS, row0 = sb.row + (int64_t)g * sb.NS;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, grp = lane >> 4;
  const int gi = wv * 4 + grp;

  // Loads in the order their values are needed: q, the centroid rows, then the sizes and
  // the steady tokens' clusters. The load counter drains in issue order, so the rank key
  // of row it is computed as soon as q and rows 0..it have landed, overlapping the rest.
  float qf[GS][8];
#pragma unroll
  for (int hh = 0; hh < GS; ++hh) {
    const uint4 v = *reinterpret_cast<const uint4*>(q + ((int64_t)b * da.H + g * GS + hh) * D + l16 * 8);
    qf[hh][0] = bf16_lo(v.x); qf[hh][1] = bf16_hi(v.x);
    qf[hh][2] = bf16_lo(v.y); qf[hh][3] = bf16_hi(v.y);
    qf[hh][4] = bf16_lo(v.z); qf[hh][5] = bf16_hi(v.z);
    qf[hh][6] = bf16_lo(v.w); qf[hh][7] = bf16_hi(v.w);
  }
  // 1. centroid rows: group gi takes clusters gi + 16 it
  uint4 cv[SC / 16];
  {
    const uint16_t* cb = reinterpret_cast<const uint16_t*>(ix.centroids_bf16) + (clu0 + j0) * D + l16 * 8;
#pragma unroll
    for (int it = 0; it < SC / 16; ++it)
      cv[it] = *reinterpret_cast<const uint4*>(cb + (int64_t)min(gi + 16 * it, nc - 1) * D);
  }
  const int nsz = ix.sizes[clu0 + j0 + min(tid, nc - 1)];
  // steady tokens whose clusters may lie in this chunk (the first and the last segments):
  // their clusters, up to 4 per thread in registers
  const Steady sz = steady_of(da, N);
  bool need = false;
  if (!sz.all && sz.nS > 0) {
    const int64_t sink_hi =
        sz.a_end > 0 ? min((int64_t)C, ((sz.a_end - 1) / sa.seg_len + 1) * (int64_t)sa.K_s) : 0;
    const int64_t loc_lo = sz.c_beg < N ? (sz.c_beg / sa.seg_len) * (int64_t)sa.K_s : (int64_t)C;
    need = (j0 < sink_hi) || (j0 + nc > loc_lo);
  }
  constexpr int SQ = 4;
  int32_t sjr[SQ];
  if (need) {
    // clamped loads without a per-lane branch; entries i >= nS are masked below
#pragma unroll
    for (int r = 0; r < SQ; ++r)
      sjr[r] = ix.assign[row0 + min(steady_pos(sz, min(tid + r * SCORE_THREADS, sz.nS - 1)), (int64_t)N - 1)];
  }
  if (tid < SC) S.scnt[tid] = 0;
  // 2. rank keys
#pragma unroll
  for (int it = 0; it < SC / 16; ++it) {
    const int jj = gi + 16 * it;
    const uint4 v = cv[it];
    const float c[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                        bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      float u;
      {
#pragma clang fp contract(off)
        u = qf[hh][0] * c[0];
#pragma unroll
        for (int m = 1; m < 8; ++m) u = u + qf[hh][m] * c[m];
      }
      u = row_sum16(u);
      if (l16 == hh) S.kw[hh][jj] = u + 0.0f;
    }
  }
  if (tid < SC) S.nsz[tid] = tid < nc ? nsz : 0;
  lds_barrier();
  // steady members per cluster of the chunk
  if (need) {
#pragma unroll
    for (int r = 0; r < SQ; ++r) {
      const int j = sjr[r] - j0;
      if (tid + r * SCORE_THREADS < sz.nS && j >= 0 && j < nc) atomicAdd(&S.scnt[j], 1);
    }
    for (int i = tid + SQ * SCORE_THREADS; i < sz.nS; i += SCORE_THREADS) {
      const int j = ix.assign[row0 + steady_pos(sz, i)] - j0;
      if (j >= 0 && j < nc) atomicAdd(&S.scnt[j], 1);
    }
  }
  lds_barrier();
  // 3. keys and eligibility out. Selection shared by the kv head: the sortable keys are the
  // group keys (the q heads' rank keys added in head order in fp32), in the first q head's slot.
  auto group_key = [&](int jj) {
    float s = S.kw[0][jj];
#pragma unroll
    for (int hh = 1; hh < GS; ++hh) s = s + S.kw[hh][jj];
    return s + 0.0f;
  };
  const int64_t kb = (int64_t)GS * sb.wclu + (int64_t)g * GS * C + j0;
  for (int e = tid; e < GS * SC; e += SCORE_THREADS) {
    const int hh = e / SC, jj = e % SC;
    if (jj < nc) {
      const float key = S.kw[hh][jj];
      const int n = S.nsz[jj];
      const bool elig = !sz.all && n > 0 && S.scnt[jj] < n;
      ws.keys[kb + (int64_t)hh * C + jj] = elig ? key : __uint_as_float(0x7FC00000u);  // NaN: outside E
      if (!da.shared)
        ws.key32[kb + (int64_t)hh * C + jj] = elig ? float_sortable(key) : 0u;
      else if (hh == 0)
        ws.key32[kb + jj] = elig ? float_sortable(group_key(jj)) : 0u;
    }
  }
  // per q head (a wave each): the chunk's DEC_CHUNK_TOPS largest sortable keys (a multiset) and its
  // eligible count, from which the top-k takes a threshold when its keys do not fit
  // registers (da.NV == 0)
  const int chm = da.NP - da.P;
  const int nsel = da.shared ? 1 : GS;  // rows of sortable keys
  for (int hh = wv; da.NV == 0 && hh < nsel; hh += SCORE_THREADS / 64) {
    uint32_t u[2];
    int ne = 0;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int jj = lane + 64 * r;
      const int n = jj < nc ? S.nsz[jj] : 0;
      const bool elig = jj < nc && !sz.all && n > 0 && S.scnt[jj] < n;
      u[r] = elig ? float_sortable(da.shared ? group_key(jj) : S.kw[hh][jj]) : 0u;
      ne += elig;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ne += __shfl_xor(ne, o, 64);
    uint32_t* ct = ws.ctop + ((int64_t)(b * da.H + g * GS + hh) * chm + chunk) * 8;
#pragma unroll
    for (int r4 = 0; r4 < DEC_CHUNK_TOPS; ++r4) {
      const uint32_t mx = wave_umax(max(u[0], u[1]));
      const uint64_t b0 = __ballot(u[0] == mx), b1 = __ballot(u[1] == mx);
      // take out one instance: the lowest lane's
      if (b0 != 0ull) {
        if (lane == __ffsll((unsigned long long)b0) - 1) u[0] = 0u;
      } else if (lane == __ffsll((unsigned long long)b1) - 1) {
        u[1] = 0u;
      }
      if (lane == 0) ct[r4] = mx;
    }
    if (lane == 0) ct[DEC_CHUNK_TOPS] = (uint32_t)ne;
  }
}

// ------------------------------------------------------------------ estimation role
// Workgroup (b, g, 128 clusters) of the k_attend grid: weights 2^(r tau log2(e) - m)
// of every cluster for the GS q heads of kv head g, and one partial softmax state
// per q head: (m, sum_j w_j n_j, sum_j w_j Vsum_j). It runs beside the gathering
// workgroups, whose memory latency it fills. Thread (sub, dq) takes dims
// 4dq..4dq+3 of clusters sub + 8u (16 float4 loads in flight per thread), issued
// after the keys and sizes, which the weights need first.
template <int GS>
struct EstLds {
  float kw[GS][SC];    // weights
  float red[4][GS][D]; // per wave: the q heads' weighted value sums
  float hred[GS][2][2];
};

template <int GS>
__device__ void est_role(const SeqArgs& sa, const DecodeArgs& da, const wave_index& ix, const DecodeWs& ws, int w) {
  __shared__ EstLds<GS> S;
  int b = 0;
  for (;; ++b) {
    const int nch = (sa.C[b] + SC - 1) / SC;
    if (w < sa.G * nch) break;
    w -= sa.G * nch;
  }
  const SeqBase sb = seq_base(sa, b);
  const int C = sb.C;
  const int nch = (C + SC - 1) / SC;
  const int g = w / nch, chunk = w % nch;
  const int j0 = chunk * SC, nc = min(SC, C - j0);
  const int64_t clu0 = sb.clu + (int64_t)g * sb.CS;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int sub = tid >> 5, dq = tid & 31;
  const float sc = da.tau * LOG2E;
  // weights: thread jj < 128 takes cluster jj for every head (keys and sizes loaded first)
  const int jj = tid;
  const int jc = min(jj, nc - 1);
  const int n0 = ix.sizes[clu0 + j0 + jc];
  const float* kb = ws.keys + (int64_t)GS * sb.wclu + (int64_t)g * GS * C + j0;
  float kr[GS];
#pragma unroll
  for (int hh = 0; hh < GS; ++hh) kr[hh] = kb[(int64_t)hh * C + jc];
  // the q heads' selections (k_topk's bitmaps): a selected cluster is attended row by row;
  // loaded before the value sums, so that the weights need not wait for those
  int64_t wb = 0;
  for (int i = 0; i < b; ++i) wb += (int64_t)da.H * ((sa.C[i] + 31) >> 5);
  const int nwords = (C + 31) >> 5, jw = j0 + jc;
  uint32_t selb[GS];
#pragma unroll
  for (int hh = 0; hh < GS; ++hh)
    selb[hh] = (ws.selw[wb + (int64_t)(g * GS + hh) * nwords + (jw >> 5)] >> (jw & 31)) & 1u;
  float4 vreg[SC / 8];
  if (ix.vsum_bf16 != nullptr) {
    // bf16 value sums (half the bytes), widened exactly
    const char* vsrc = reinterpret_cast<const char*>(reinterpret_cast<const uint16_t*>(ix.vsum_bf16) + (clu0 + j0) * D);
    uint2 wreg[SC / 8];
#pragma unroll
    for (int u = 0; u < SC / 8; ++u) {
      const uint32_t off = (uint32_t)(min(sub + 8 * u, nc - 1) * (D * 2) + dq * 8);
      wreg[u] = *reinterpret_cast<const uint2*>(vsrc + off);
    }
#pragma unroll
    for (int u = 0; u < SC / 8; ++u)
      vreg[u] = make_float4(bf16_lo(wreg[u].x), bf16_hi(wreg[u].x), bf16_lo(wreg[u].y), bf16_hi(wreg[u].y));
  } else {
    // a uniform base and 32-bit lane offsets: one address register per load
    const char* vsrc = reinterpret_cast<const char*>(ix.vsum + (clu0 + j0) * D);
#pragma unroll
    for (int u = 0; u < SC / 8; ++u) {
      const uint32_t off = (uint32_t)(min(sub + 8 * u, nc - 1) * (D * 4) + dq * 16);
      vreg[u] = *reinterpret_cast<const float4*>(vsrc + off);
    }
  }
  float sv[GS];
  if (tid < SC) {
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      // E \ R: eligible (a rank key, not NaN), not selected by this q head
      const bool live = jj < nc && n0 > 0 && kr[hh] == kr[hh] && selb[hh] == 0u;
      sv[hh] = live ? kr[hh] * sc : -INFINITY;
      const float mx = wave_max(sv[hh]);
      if (lane == 0) S.hred[hh][wv][0] = mx;
    }
  }
  lds_barrier();
  if (tid < SC) {
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      const float M = fmaxf(S.hred[hh][0][0], S.hred[hh][1][0]);
      const float wgt = sv[hh] == -INFINITY ? 0.f : exp2f(sv[hh] - M);
      S.kw[hh][tid] = wgt;
      const float ls = wave_sum(wgt * (float)(jj < nc ? n0 : 0));
      if (lane == 0) S.hred[hh][wv][1] = ls;
    }
  }
  lds_barrier();
  float acc[GS][4];
#pragma unroll
  for (int hh = 0; hh < GS; ++hh)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[hh][e] = 0.f;
#pragma unroll
  for (int u = 0; u < SC / 8; ++u) {
    const int c = sub + 8 * u;
    const float4 v = vreg[u];
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      const float wgt = S.kw[hh][c];  // 0 for c >= nc (not live)
      acc[hh][0] = fmaf(wgt, v.x, acc[hh][0]);
      acc[hh][1] = fmaf(wgt, v.y, acc[hh][1]);
      acc[hh][2] = fmaf(wgt, v.z, acc[hh][2]);
      acc[hh][3] = fmaf(wgt, v.w, acc[hh][3]);
    }
  }
#pragma unroll
  for (int hh = 0; hh < GS; ++hh)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[hh][e] += swap32(acc[hh][e]);
  if (lane < 32)
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
#pragma unroll
      for (int e = 0; e < 4; ++e) S.red[wv][hh][dq * 4 + e] = acc[hh][e];
  lds_barrier();
  for (int e = tid; e < GS * D; e += blockDim.x) {
    const int hh = e / D, d = e % D;
    const float A = S.red[0][hh][d] + S.red[1][hh][d] + S.red[2][hh][d] + S.red[3][hh][d];
    float* o = ws.part + (((int64_t)b * da.H + g * GS + hh) * da.NP + da.P + chunk) * PART;
    if (d == 0) {
      const float L = S.hred[hh][0][1] + S.hred[hh][1][1];
      o[0] = L > 0.f ? fmaxf(S.hred[hh][0][0], S.hred[hh][1][0]) : -INFINITY;
      o[1] = L;
    }
    o[4 + d] = A;
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

// descending bitonic sort of n (power of two) unique u64 keys in LDS. Each wave owns a
// contiguous region of R = n / waves keys; a compare-exchange step with distance j < R stays
// inside the regions, so it needs no workgroup barrier: the wave's LDS operations complete in
// order (a wait on the LDS counter between steps), and only the steps with j >= R (10 of
// the 66 for n = 2048) synchronise the workgroup.
__device__ inline void bitonic_desc_lds(uint64_t* a, int n) {
  const int nw = blockDim.x >> 6, wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int R = n / nw;
  bool waved = false;  // the previous step was wave-local
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= R || R < 2) {
        if (waved) __syncthreads();
        waved = false;
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint64_t x = a[i], y = a[ixj];
            const bool desc = (i & k) == 0;
            if (desc ? (x < y) : (x > y)) { a[i] = y; a[ixj] = x; }
          }
        }
        __syncthreads();
      } else {
        // pairs (i, i + j) of the wave's region, i with bit j clear
        for (int q = lane; q < R / 2; q += 64) {
          const int i = wv * R + ((q / j) * 2 * j) + (q % j), ixj = i + j;
          const uint64_t x = a[i], y = a[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) { a[i] = y; a[ixj] = x; }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        waved = true;
      }
    }
  }
  if (waved) __syncthreads();
}

// The same sort for n = 1024 E keys and 16 waves, the keys in registers between the steps
// that cross waves: lane l of wave w holds keys w 64 E + 64 e + l (e < E), so a step with
// partner distance j < 64 is a lane shuffle, 64 <= j < 64 E a swap between a lane's own
// registers, and only j >= 64 E goes through LDS with barriers (15 of the 78 steps of
// 4096 keys, the size it serves; up to 2048 keys take sort_desc_runs below).
__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

template <int E>
__device__ void bitonic_desc_reg(uint64_t* a, int n) {
  constexpr int R = 64 * E;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint64_t x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = a[wv * R + 64 * e + lane];
  bool inreg = true;
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= R) {
        if (inreg) {
#pragma unroll
          for (int e = 0; e < E; ++e) a[wv * R + 64 * e + lane] = x[e];
          __syncthreads();
          inreg = false;
        }
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint64_t p = a[i], q = a[ixj];
            const bool desc = (i & k) == 0;
            if (desc ? (p < q) : (p > q)) { a[i] = q; a[ixj] = p; }
          }
        }
        __syncthreads();
        continue;
      }
      if (!inreg) {
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = a[wv * R + 64 * e + lane];
        inreg = true;
      }
      if (j >= 64) {
        const int js = j >> 6;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if ((e & js) == 0) {
            const int i = wv * R + 64 * e + lane;
            const bool desc = (i & k) == 0;
            const uint64_t p = x[e], q = x[e | js];
            const uint64_t hi = p > q ? p : q, lo = p > q ? q : p;
            x[e] = desc ? hi : lo;
            x[e | js] = desc ? lo : hi;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = wv * R + 64 * e + lane;
          const uint64_t q = shfl_xor64(x[e], j);
          const bool keep_max = ((lane & j) == 0) == ((i & k) == 0);  // lower of the pair in a descending run
          x[e] = keep_max ? (x[e] > q ? x[e] : q) : (x[e] > q ? q : x[e]);
        }
      }
    }
  }
  if (inreg) {
#pragma unroll
    for (int e = 0; e < E; ++e) a[wv * R + 64 * e + lane] = x[e];
  }
  __syncthreads();
}

// Descending sort of n = 1024 E keys in LDS by 16 waves: each wave sorts its 64 E keys in
// registers (bitonic steps as lane shuffles and swaps inside a lane, no barrier), then every
// key's place in the whole is its place in its own run plus, in each other run, the number of
// keys above it (a binary search: the runs are sorted). Keys above 0 are distinct, so they
// get distinct places; the zero padding gets places after them (possibly shared, never read).
// Three barriers in all, against one per cross-wave step of a bitonic sort.
template <int E>
__device__ void sort_desc_runs(uint64_t* a, int n) {
  constexpr int R = 64 * E;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint64_t x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = a[wv * R + 64 * e + lane];
  for (int k = 2; k <= R; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= 64) {
        const int js = j >> 6;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if ((e & js) == 0) {
            const bool desc = ((64 * e + lane) & k) == 0;
            const uint64_t p = x[e], q = x[e | js];
            const uint64_t hi = p > q ? p : q, lo = p > q ? q : p;
            x[e] = desc ? hi : lo;
            x[e | js] = desc ? lo : hi;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint64_t q = shfl_xor64(x[e], j);
          const bool keep_max = ((lane & j) == 0) == (((64 * e + lane) & k) == 0);
          x[e] = keep_max ? (x[e] > q ? x[e] : q) : (x[e] > q ? q : x[e]);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) a[wv * R + 64 * e + lane] = x[e];
  __syncthreads();
  // the 16 searches of a key advance together, one LDS read each per step (a search alone
  // is a chain of 8 dependent reads); in its own run the count is its own place
  int rank[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    int pos[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) pos[r] = 0;
#pragma unroll
    for (int step = R / 2; step >= 1; step >>= 1)
#pragma unroll
      for (int r = 0; r < 16; ++r) pos[r] += a[r * R + pos[r] + step - 1] > x[e] ? step : 0;
    int rk = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) rk += pos[r] + ((pos[r] < R && a[r * R + min(pos[r], R - 1)] > x[e]) ? 1 : 0);
    rank[e] = rk;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) a[rank[e]] = x[e];
  __syncthreads();
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
// Sortable key u_j = float_sortable(r_j) for j in E, 0 otherwise; the selection
// R is the k = min(kreq, |E|) largest (u desc, id asc).
//
// Ids: wave w owns [w 64 NV, (w + 1) 64 NV); lane L holds ids
// w0 + 64 v + L (v < NV): every load is 64 consecutive ids, and a wave's order
// of (v, lane) is id order. With NV <= 32 the keys stay in registers (the fast
// path below takes NV <= 16).
//
// Fast path (keys in registers, k <= 1024): every wave finds the m-th largest
// of its 64 lane maxima, t_w (m = ceil(kreq / W) for W waves), by bisection over
// the 32 key bits with ballots, no barrier; at least m keys of the wave are >= t_w,
// so at least W m >= k keys are >= min_w t_w. A lane whose maximum is >= t holds a
// key >= t, so counting lane maxima >= each t_w bounds the keys >= t_w from below:
// X is the largest t_w with at least k lane maxima at or above it, and the keys
// >= X contain R. When there are at most 1024 of them, each one's rank and
// the summed sizes of the candidates ranked before it are counted (split over
// all threads), which yields R in rank order with its member-count prefix.
// Otherwise the general path finds the exact k-th key by bisection over the
// workgroup, selects in id order and sorts the selection.
struct TopkLds {
  union {
    struct {
      uint4 rec[TK_CAP];        // (~id, u, size, first sorted slot): the order key is (u << 32) | ~id
      int32_t rank[TK_CAP];     // candidates that order before it
      int32_t pre[TK_CAP];      // their summed sizes
    } c;                        // fast path
    uint64_t sortbuf[TK_SORT];  // general path: the selection's (u << 32) | ~id
  } u;
  uint32_t selw[TK_SELW];       // selection bitmap (C <= 65536)
  uint64_t scan[17];
  uint32_t bis[34];             // block counts of the bisection, then of keys above T
  uint32_t rhist[2][256];       // digit counts of the radix select over the chunks' top keys
  uint32_t rsel[2];             // its digit and the count above it
  alignas(16) int32_t wE[16];   // read as vectors: four reads, not a chain of sixteen
  alignas(16) uint32_t wt[16];
  alignas(16) int32_t tcnt[16]; // keys >= wt[i] over the workgroup
  int32_t misc[8];
};

// PF: prefetch every key's size and offset with the keys (as registers allow). That hides a
// load round when the heads fit the CUs; with more heads than CUs its registers (72 at 8 keys
// a lane) leave room for one workgroup per CU instead of two, so those launches take PF = false,
// compiled for two workgroups per CU (64 registers).
template <int NVR, bool PF = true>
__global__ __launch_bounds__(TK_THREADS, PF ? 1 : 2 * TK_WAVES / 4) void k_topk(SeqArgs sa, DecodeArgs da, wave_index ix, DecodeWs ws,
                                                     int32_t* __restrict__ sel_ids) {
  constexpr bool INREG = NVR > 0;
  constexpr int CHK = INREG ? (NVR < 16 ? NVR : 16) : 8;  // keys per lane per chunk
  extern __shared__ uint8_t smem[];
  TopkLds& L = *reinterpret_cast<TopkLds*>(smem);
  const int NV = INREG ? NVR : da.NVg;
  const int bh = blockIdx.x;
  const int b = bh / da.H, h = bh % da.H, g = h / da.GS;
  const SeqBase sb = seq_base(sa, b);
  const int N = sb.N, C = sb.C;
  const int64_t row0 = sb.row + (int64_t)g * sb.NS;
  const int64_t clu0 = sb.clu + (int64_t)g * sb.CS;
  const int64_t off0 = sb.off + (int64_t)g * (sb.CS + 1);
  const int64_t kbase = (int64_t)da.GS * sb.wclu + (int64_t)h * C;
  // sortable keys of the selection: the head's own, or its kv head's group keys (first q head's slot)
  const int hs = da.shared ? g * da.GS : h;
  const int64_t bhs = (int64_t)b * da.H + hs;
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wv = tid >> 6;
  const uint64_t ltmask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const uint32_t* key32 = ws.key32 + (int64_t)da.GS * sb.wclu + (int64_t)hs * C;
  const float* keys = ws.keys + kbase;
  int2* span = ws.span + kbase;
  int32_t* out = sel_ids + (int64_t)bh * da.k_max;
  const int32_t* sizes = ix.sizes + clu0;
  const int32_t* offs = ix.offsets + off0;
  const int w0 = wv * 64 * NV;
  auto id_of = [&](int v) { return w0 + 64 * v + lane; };
  const int nwords = (C + 31) >> 5;
  const bool lds_sel = INREG || nwords <= TK_SELW;  // keys in registers: C <= 32768
  int64_t wbase = 0;
  for (int i = 0; i < b; ++i) wbase += (int64_t)da.H * ((sa.C[i] + 31) >> 5);
  uint32_t* selw = lds_sel ? L.selw : ws.selw + wbase + (int64_t)h * nwords;

  // 0. loads in the order their values are needed (the load counter drains in issue
  // order): the keys, their sizes and offsets, then the steady tokens' clusters; LDS init
  // sizes and offsets of every key prefetched (as registers allow)
  constexpr bool PRE = PF && INREG && NVR <= (TK_WAVES <= 8 ? 16 : 8);
  uint32_t ureg[INREG ? NVR : 1];
  int32_t nreg[PRE ? NVR : 1], oreg[PRE ? NVR : 1];
  if constexpr (INREG) {
#pragma unroll
    for (int v = 0; v < NVR; ++v) {
      const int j = id_of(v);
      const uint32_t x = key32[min(j, C - 1)];
      ureg[v] = j < C ? x : 0u;
    }
  }
  if constexpr (PRE) {
#pragma unroll
    for (int v = 0; v < NVR; ++v) {
      const int j = min(id_of(v), C - 1);
      nreg[v] = sizes[j];
      oreg[v] = offs[j];
    }
  }
  const Steady sz = steady_of(da, N);
  // loads at a clamped position, without a branch (a value merged after a divergent
  // load would make the wave wait for every load in flight); entries i >= nS unused
  int32_t sjr[2];
  sjr[0] = ix.assign[row0 + min(steady_pos(sz, min(tid, max(sz.nS - 1, 0))), (int64_t)N - 1)];
  sjr[1] = 0;
  if (sz.nS > TK_THREADS)
    sjr[1] = ix.assign[row0 + min(steady_pos(sz, min(tid + TK_THREADS, sz.nS - 1)), (int64_t)N - 1)];
  auto chunk_keys = [&](int c0, uint32_t* uc) {  // the lane's CHK keys of chunk c0
    if constexpr (INREG) {
#pragma unroll
      for (int v = 0; v < CHK; ++v) uc[v] = ureg[c0 + v];
    } else {
#pragma unroll
      for (int v = 0; v < CHK; ++v) {
        const int j = id_of(c0 + v);
        const uint32_t x = key32[min(j, C - 1)];
        uc[v] = j < C ? x : 0u;
      }
    }
  };
  if (lds_sel) {
    for (int i = tid; i < nwords; i += nt) L.selw[i] = 0u;
  } else {
    for (int i = tid; i < nwords; i += nt) selw[i] = 0u;
  }
  if constexpr (INREG) {
    for (int i = tid; i < TK_CAP; i += nt) {
      L.u.c.rank[i] = 0;
      L.u.c.pre[i] = 0;
    }
  }
  if (tid < 34) L.bis[tid] = 0u;
  if (tid < 256) L.rhist[0][tid] = 0u;
  if (tid < 8) L.misc[tid] = 0;
  if (tid < 16) L.tcnt[tid] = 0;

  // 1. per wave: eligible keys and (keys in registers) the m-th largest key
  const int kreq = da.kreq[b];
  const int m = (kreq + TK_WAVES - 1) / TK_WAVES;
  int Ew = 0;
  uint32_t tw = 0u;
  uint32_t lmax = 0u;
  // keys read from memory: chunk t's summary record (its largest keys, then its eligible
  // count) in thread t's registers, both words loaded at once for the threshold below
  uint4 crec[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  if constexpr (INREG) {
#pragma unroll
    for (int v = 0; v < NVR; ++v) {
      Ew += __popcll(__ballot(ureg[v] != 0u));
      lmax = max(lmax, ureg[v]);
    }
    if (kreq > 0 && __popcll(__ballot(lmax != 0u)) >= m) {
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = tw | (1u << bit);
        if (__popcll(__ballot(lmax >= c)) >= m) tw = c;
      }
    }
  } else {
    // eligible keys from k_score's chunk summaries (thread t adds chunks t, t + TK_THREADS, ...)
    const int nch = (C + SC - 1) / SC;
    const uint32_t* ct = ws.ctop + bhs * (da.NP - da.P) * 8;
    if (tid < nch) {
      crec[0] = reinterpret_cast<const uint4*>(ct)[2 * tid];
      crec[1] = reinterpret_cast<const uint4*>(ct)[2 * tid + 1];
    }
    int e = (int)crec[1].w;
    for (int i = tid + nt; i < nch; i += nt) e += (int)ct[(int64_t)i * 8 + DEC_CHUNK_TOPS];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) e += __shfl_xor(e, o, 64);
    Ew = e;
  }
  // rank keys of the steady tokens' clusters, for the corrections at the end
  float kjr[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) kjr[r] = keys[min(max(sjr[r], 0), C - 1)];
  if (lane == 0) {
    L.wE[wv] = Ew;
    L.wt[wv] = tw;
  }
  lds_barrier();
  // every wave's eligible count and threshold, into registers by vector reads
  static_assert(TK_WAVES % 4 == 0 && TK_WAVES <= 16, "per-wave values read four at a time");
  uint32_t wtr[TK_WAVES];
  int nE = 0;
  uint32_t X = 0xFFFFFFFFu;
#pragma unroll
  for (int q4 = 0; q4 < TK_WAVES / 4; ++q4) {
    const int4 e4 = reinterpret_cast<const int4*>(L.wE)[q4];
    const uint4 t4 = reinterpret_cast<const uint4*>(L.wt)[q4];
    nE += e4.x + e4.y + e4.z + e4.w;
    // uniform values: scalar registers
    wtr[4 * q4 + 0] = __builtin_amdgcn_readfirstlane(t4.x);
    wtr[4 * q4 + 1] = __builtin_amdgcn_readfirstlane(t4.y);
    wtr[4 * q4 + 2] = __builtin_amdgcn_readfirstlane(t4.z);
    wtr[4 * q4 + 3] = __builtin_amdgcn_readfirstlane(t4.w);
  }
#pragma unroll
  for (int i = 0; i < TK_WAVES; ++i) X = min(X, wtr[i]);
  const int k = min(kreq, nE);
  if constexpr (INREG) {
    if (k > 0 && k == kreq && X > 0u) {
      // lane maxima >= each wave threshold; lane i < TK_WAVES of every wave adds its count for wt[i]
      int mine = 0;
#pragma unroll
      for (int i = 0; i < TK_WAVES; ++i) {
        const int cnt = __popcll(__ballot(lmax >= wtr[i]));
        mine = (lane == i) ? cnt : mine;
      }
      if (lane < TK_WAVES) atomicAdd(&L.tcnt[lane], mine);
      lds_barrier();
      // the counts by vector reads (a loop of scalar reads became a chain of round trips)
#pragma unroll
      for (int q4 = 0; q4 < TK_WAVES / 4; ++q4) {
        const int4 c4 = reinterpret_cast<const int4*>(L.tcnt)[q4];
        X = c4.x >= k ? max(X, wtr[4 * q4 + 0]) : X;
        X = c4.y >= k ? max(X, wtr[4 * q4 + 1]) : X;
        X = c4.z >= k ? max(X, wtr[4 * q4 + 2]) : X;
        X = c4.w >= k ? max(X, wtr[4 * q4 + 3]) : X;
      }
    }
  }
  if (k < kreq) X = 1u;
  X = max(X, 1u);

  // 2. fast path: candidates u >= X; rank and size prefix by counting
  // (32 keys per lane: the general path only, the keys in registers)
  bool fast = INREG && NVR <= 16 && k > 0 && k <= TK_CAP;
  if (fast) {
    if constexpr (INREG && NVR <= 16) {
      uint64_t bal[NVR];
      int tot = 0;
#pragma unroll
      for (int v = 0; v < NVR; ++v) {
        bal[v] = __ballot(ureg[v] >= X);
        tot += __popcll(bal[v]);
      }
      int base = 0;
      if (lane == 0) base = atomicAdd(&L.misc[0], tot);
      base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
      for (int v = 0; v < NVR; ++v) {
        if (ureg[v] >= X) {
          const int p = base + __popcll(bal[v] & ltmask);
          if (p < TK_CAP) {
            const int id = id_of(v);
            uint4 r;
            r.x = 0xFFFFFFFFu - (uint32_t)id;
            r.y = ureg[v];
            if constexpr (PRE) {
              r.z = (uint32_t)nreg[v];
              r.w = (uint32_t)oreg[v];
            } else {
              r.z = (uint32_t)sizes[id];
              r.w = (uint32_t)offs[id];
            }
            L.u.c.rec[p] = r;
          }
        }
        base += __popcll(bal[v]);
      }
    }
    lds_barrier();
    const int nc = L.misc[0];
    fast = nc <= TK_CAP;
    if (fast) {
      // item x = (part, candidate i) counts over that part of the candidates
      const int P = max(1, TK_THREADS / nc);
      for (int x = tid; x < nc * P; x += nt) {
        const int i = x % nc, part = x / nc;
        const uint4 ri = L.u.c.rec[i];
        const uint64_t c = ((uint64_t)ri.y << 32) | ri.x;
        const int j0 = nc * part / P, j1 = nc * (part + 1) / P;  // nc <= 1024: no overflow
        int rank = 0, pre = 0;
        auto count = [&](int j) {
          const uint4 rj = L.u.c.rec[j];
          const bool gt = (((uint64_t)rj.y << 32) | rj.x) > c;
          rank += gt;
          pre += (int)(rj.z & (0u - (uint32_t)gt));
        };
        // 16 records a batch of LDS reads (8 in the 64-register variant)
        if constexpr (PF) {
#pragma unroll 16
          for (int j = j0; j < j1; ++j) count(j);
        } else {
#pragma unroll 8
          for (int j = j0; j < j1; ++j) count(j);
        }
        atomicAdd(&L.u.c.rank[i], rank);
        atomicAdd(&L.u.c.pre[i], pre);
      }
      lds_barrier();
      int32_t* selpre = ws.selpre + kbase + bh;  // k + 1 entries per (b, h)
      for (int ci = tid; ci < nc; ci += nt) {
        const int rank = L.u.c.rank[ci];
        if (rank < k) {
          const uint4 r = L.u.c.rec[ci];
          const int id = (int)(0xFFFFFFFFu - r.x);
          const int n = (int)r.z, pre = L.u.c.pre[ci];
          out[rank] = id;
          span[rank] = make_int2((int)r.w, n);
          selpre[rank] = pre;
          atomicOr(&L.selw[id >> 5], 1u << (id & 31));
          if (rank == k - 1) {
            selpre[k] = pre + n;
            ws.counts[4 * bh + 0] = pre + n;
          }
        }
      }
    }
  }

  // 3a. keys read from memory: a threshold t from the chunks' top keys (the k-th largest
  // of them is at most the k-th largest key, so the keys >= t hold the selection), one
  // pass collecting those keys into LDS, and a sort of them
  bool done = false;
  if constexpr (!INREG) {
    const int nch = (C + SC - 1) / SC;
    const uint32_t* ct = ws.ctop + bhs * (da.NP - da.P) * 8;
    if (k > 0 && k <= DEC_CHUNK_TOPS * nch && nch <= TK_THREADS) {
      uint32_t tv[DEC_CHUNK_TOPS];
#pragma unroll
      for (int r = 0; r < DEC_CHUNK_TOPS; ++r) tv[r] = r < 4 ? crec[0][r] : crec[1][r - 4];
      // t = the k-th largest of them (zeros included): a radix select, 8 bits a pass from
      // the top; a wave counts equal digits by matching the 8 digit bits with ballots and
      // the lowest lane of each match adds the count (one LDS atomic per distinct digit)
      uint32_t t = 0u;
      {
        uint32_t pre = 0u, msk = 0u;
        int kr = k;
        for (int pass = 0; pass < 4; ++pass) {
          const int sh = 24 - 8 * pass;
          uint32_t* hist = L.rhist[pass & 1];
          if (tid < 256) L.rhist[(pass + 1) & 1][tid] = 0u;  // for the next pass (read two barriers ago)
#pragma unroll
          for (int r = 0; r < DEC_CHUNK_TOPS; ++r) {
            const uint32_t d = (tv[r] >> sh) & 255u;
            uint64_t m = __ballot((tv[r] & msk) == pre);
            if (m == 0ull) continue;  // no key of the wave still has the selected prefix
#pragma unroll
            for (int b = 0; b < 8; ++b) {
              const uint64_t bb = __ballot((d >> b) & 1u);
              m &= ((d >> b) & 1u) ? bb : ~bb;
            }
            if ((tv[r] & msk) == pre && (m & ltmask) == 0ull) atomicAdd(&hist[d], (uint32_t)__popcll(m));
          }
          lds_barrier();
          if (wv == 0) {
            // lane l: digits 4l..4l+3; suffix sums over the lanes give the count at or above
            const uint4 h4 = reinterpret_cast<const uint4*>(hist)[lane];
            const int s4 = (int)(h4.x + h4.y + h4.z + h4.w);
            int suf = s4;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
              const int v = __shfl_down(suf, o, 64);
              if (lane + o < 64) suf += v;
            }
            const int above = suf - s4;  // digits >= 4l + 4
            if (above < kr && kr <= suf) {
              int gt = above, d = 4 * lane + 3;
              if (gt + (int)h4.w < kr) {
                gt += (int)h4.w;
                d = 4 * lane + 2;
                if (gt + (int)h4.z < kr) {
                  gt += (int)h4.z;
                  d = 4 * lane + 1;
                  if (gt + (int)h4.y < kr) {
                    gt += (int)h4.y;
                    d = 4 * lane;
                  }
                }
              }
              L.rsel[0] = (uint32_t)d;
              L.rsel[1] = (uint32_t)gt;
            }
          }
          lds_barrier();
          pre |= L.rsel[0] << sh;
          msk |= 255u << sh;
          kr -= (int)L.rsel[1];
        }
        t = pre;
      }
      if (t > 0u) {
        uint64_t* cb = L.u.sortbuf;
        // the keys a chunk ahead in flight (the loads of a chunk otherwise wait for the
        // previous chunk's collection)
        uint32_t un[CHK];
        chunk_keys(0, un);
        for (int c0 = 0; c0 < NV; c0 += CHK) {
          uint32_t uc[CHK];
#pragma unroll
          for (int v = 0; v < CHK; ++v) uc[v] = un[v];
          if (c0 + CHK < NV) chunk_keys(c0 + CHK, un);
          uint64_t bal[CHK];
          int tot = 0;
#pragma unroll
          for (int v = 0; v < CHK; ++v) {
            bal[v] = __ballot(uc[v] >= t);
            tot += __popcll(bal[v]);
          }
          int base = 0;
          if (lane == 0 && tot > 0) base = atomicAdd(&L.misc[1], tot);
          base = __shfl(base, 0, 64);
#pragma unroll
          for (int v = 0; v < CHK; ++v) {
            if (uc[v] >= t) {
              const int p = base + __popcll(bal[v] & ltmask);
              if (p < TK_SORT) cb[p] = ((uint64_t)uc[v] << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)id_of(c0 + v));
            }
            base += __popcll(bal[v]);
          }
        }
        lds_barrier();
        const int nc = L.misc[1];
        if (nc <= TK_SORT) {
          int P2 = 1;
          while (P2 < nc) P2 <<= 1;
          for (int i = nc + tid; i < P2; i += nt) cb[i] = 0ull;
          __syncthreads();
          if (TK_WAVES == 16 && P2 == 1024)
            sort_desc_runs<1>(cb, P2);
          else if (TK_WAVES == 16 && P2 == 2048)
            sort_desc_runs<2>(cb, P2);
          else if (TK_WAVES == 16 && P2 == 4096)
            bitonic_desc_reg<4>(cb, P2);
          else
            bitonic_desc_lds(cb, P2);
          // (key desc, id asc): the first k are the selection in rank order. Thread t takes
          // ranks [t R, (t + 1) R) (R <= 4) and keeps their sizes for the member-count prefix
          const int R = (k + nt - 1) / nt;
          const int q0 = min(tid * R, k), q1 = min(q0 + R, k);
          int nn[TK_SORT / TK_THREADS];
          int64_t msum = 0;
#pragma unroll
          for (int u = 0; u < TK_SORT / TK_THREADS; ++u) {
            const int r = q0 + u;
            nn[u] = 0;
            if (r < q1) {
              const int id = (int)(0xFFFFFFFFu - (uint32_t)(cb[r] & 0xFFFFFFFFu));
              const int n = sizes[id];
              out[r] = id;
              span[r] = make_int2(offs[id], n);
              atomicOr(&selw[id >> 5], 1u << (id & 31));
              nn[u] = n;
              msum += n;
            }
          }
          uint64_t tot;
          int64_t run = (int64_t)block_scan_excl((uint64_t)msum, L.scan, &tot);
          int32_t* selpre = ws.selpre + kbase + bh;
#pragma unroll
          for (int u = 0; u < TK_SORT / TK_THREADS; ++u) {
            const int r = q0 + u;
            if (r < q1) {
              selpre[r] = (int32_t)run;
              run += nn[u];
            }
          }
          if (tid == 0) {
            selpre[k] = (int32_t)tot;
            ws.counts[4 * bh + 0] = (int32_t)tot;
          }
          done = true;
        }
      }
    }
  }

  // 3. general path: exact k-th key T by bisection, selection in id order, rank-order sort
  if (!fast && !done && k > 0) {
    uint32_t T = 0u;
    auto block_count = [&](uint32_t c, uint32_t* slot) {  // keys >= c over the workgroup
      int cnt = 0;
#pragma unroll(INREG ? 16 : 1)
      for (int c0 = 0; c0 < NV; c0 += CHK) {
        uint32_t uc[CHK];
        chunk_keys(c0, uc);
#pragma unroll
        for (int v = 0; v < CHK; ++v) cnt += __popcll(__ballot(uc[v] >= c));
      }
      if (lane == 0) atomicAdd(slot, (uint32_t)cnt);
      __syncthreads();
      return *slot;
    };
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = T | (1u << bit);
      if (block_count(c, &L.bis[bit]) >= (uint32_t)k) T = c;
    }
    const int cgt = T == 0xFFFFFFFFu ? 0 : (int)block_count(T + 1u, &L.bis[32]);
    const int k_eq = k - cgt;
    // selection in id order: keys > T, then the k_eq lowest ids with key == T
    int ngt = 0, neq = 0;
#pragma unroll(INREG ? 16 : 1)
    for (int c0 = 0; c0 < NV; c0 += CHK) {
      uint32_t uc[CHK];
      chunk_keys(c0, uc);
#pragma unroll
      for (int v = 0; v < CHK; ++v) {
        ngt += uc[v] > T;
        neq += uc[v] == T;
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
    uint64_t* sb_ = (k <= TK_SORT) ? L.u.sortbuf : ws.sortg + (int64_t)bh * da.sort_stride;
#pragma unroll(INREG ? 16 : 1)
    for (int c0 = 0; c0 < NV; c0 += CHK) {
      uint32_t uc[CHK];
      chunk_keys(c0, uc);
      // per 64 ids (one v): lane-order prefix of (eq, selected) counts by ballots; the
      // selected keys' offsets, sizes and rank keys are loaded where they are selected
#pragma unroll
      for (int v = 0; v < CHK; ++v) {
        const uint32_t x = uc[v];
        const uint64_t em = __ballot(x == T);
        const int er = eq_seen + __popcll(em & ltmask);
        const bool sv = x > T || (x == T && er < k_eq);
        const uint64_t sm = __ballot(sv);
        if (sv) {
          const int j = id_of(c0 + v);
          const int p = pos + __popcll(sm & ltmask);
          span[p] = make_int2(offs[j], sizes[j]);
          sb_[p] = ((uint64_t)x << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)j);
          atomicOr(&selw[j >> 5], 1u << (j & 31));
        }
        pos += __popcll(sm);
        eq_seen += __popcll(em);
      }
    }
    __threadfence_block();
    __syncthreads();
    // rank order (key desc, id asc) of the output ids
    if (k <= TK_RANK_SMALL) {
      if (tid < k) {
        const uint64_t c = sb_[tid];
        int rank = 0;
#pragma unroll 8
        for (int i = 0; i < k; ++i) rank += sb_[i] > c;
        out[rank] = (int32_t)(0xFFFFFFFFu - (uint32_t)(c & 0xFFFFFFFFu));
      }
    } else {
      int P2 = 1;
      while (P2 < k) P2 <<= 1;
      for (int i = k + tid; i < P2; i += nt) sb_[i] = 0;
      if (k > TK_SORT) __threadfence_block();
      __syncthreads();
      bitonic_desc(sb_, P2, k > TK_SORT);
      for (int i = tid; i < k; i += nt) out[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(sb_[i] & 0xFFFFFFFFu));
    }
  }

  // 4. member-count prefix of the general path's selection, counts
  if (!fast && !done) {
    int32_t* selpre = ws.selpre + kbase + bh;
    __threadfence_block();
    __syncthreads();
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
    }
  }
  if (tid == 0) {
    ws.counts[4 * bh + 1] = k;
    ws.counts[4 * bh + 2] = sz.nS;
    ws.counts[4 * bh + 3] = 0;
  }
  for (int i = k + tid; i < da.k_max; i += nt) out[i] = -1;

  // 5. steady rows: the rank key of their cluster if it is not selected, else NaN
  if (lds_sel) {
    lds_barrier();
  } else {
    __threadfence_block();
    __syncthreads();
  }
  float* corr = ws.corr + (int64_t)bh * da.scap;
  for (int i = tid; i < sz.nS; i += nt) {
    int32_t j;
    float kj;
    if (i < 2 * TK_THREADS) {
      j = i < TK_THREADS ? sjr[0] : sjr[1];
      kj = i < TK_THREADS ? kjr[0] : kjr[1];
    } else {
      j = ix.assign[row0 + steady_pos(sz, i)];
      kj = keys[j];
    }
    const bool sel = (selw[j >> 5] >> (j & 31)) & 1u;
    corr[i] = sel ? __uint_as_float(0x7FC00000u) : kj;  // NaN also outside E (its key)
  }
  // the selection bitmap for the estimation role of k_attend (in the workspace already
  // when it did not fit LDS)
  if (lds_sel) {
    uint32_t* gw = ws.selw + wbase + (int64_t)h * nwords;
    for (int i = tid; i < nwords; i += nt) gw[i] = L.selw[i];
  }
}

// ------------------------------------------------------------------ k_topk_sto
// The stochastic radix top-k (Vortex page, section 2.C: the top-k terminates early and
// samples the rest of the selection from a threshold bin), an inexact variant of k_topk
// with the same outputs (ids, spans, member prefix, counts, selection bitmap, steady
// corrections); ids in ascending order. One workgroup per (sequence, q head); wave w owns
// the clusters [w 64 per, (w + 1) 64 per) and its lane l key slot i is cluster
// w 64 per + 64 i + l, so loads are coalesced and id order is (wave, slot, lane): ranks in
// id order come from ballots within a wave and one scan over the 16 waves.
// Radix descent over the sortable keys, 8 bits a pass: a per-wave LDS histogram of the
// next digit of the keys that share the prefix so far (in the first pass, where nearly all
// keys share the top byte, a wave's equal digits are counted with one atomic), summed,
// and one wave scanning its 256 bins from the top for the threshold bin. After
// da.sto_passes passes (fewer when the threshold bin is needed whole) the bins above it
// are taken whole and its members by systematic sampling with a random phase: member r
// (in id order) of the n is taken when floor((r m + c) / n) < floor(((r + 1) m + c) / n),
// i.e. (r m + c) mod n >= n - m, m the ids still missing, c = the first SplitMix64 output
// of the stream of (b, h) under the seed, mod n (32-bit arithmetic: C < 2^26). The ids
// go to the output in ascending order, then one pass over them, split over the threads,
// writes spans, member prefixes and the bitmap. NK: key slots a lane holds in registers
// (0: re-read from memory).
template <int NK>
__global__ __launch_bounds__(TK_THREADS) void k_topk_sto(SeqArgs sa, DecodeArgs da, wave_index ix, DecodeWs ws,
                                                         int32_t* __restrict__ sel_ids) {
  __shared__ uint32_t hist[TK_WAVES][256];  // per wave, then the sum in hist[0]
  __shared__ int32_t res[4];
  __shared__ int64_t wsum[3][TK_WAVES];     // per wave: eligible keys / bin members / selected (then scan space)
  const int bh = blockIdx.x;
  const int b = bh / da.H, h = bh % da.H, g = h / da.GS;
  const SeqBase sb = seq_base(sa, b);
  const int N = sb.N, C = sb.C;
  const int64_t row0 = sb.row + (int64_t)g * sb.NS;
  const int64_t clu0 = sb.clu + (int64_t)g * sb.CS;
  const int64_t off0 = sb.off + (int64_t)g * (sb.CS + 1);
  const int64_t kbase = (int64_t)da.GS * sb.wclu + (int64_t)h * C;
  const uint32_t* key32 = ws.key32 + kbase;
  const float* keys = ws.keys + kbase;
  int2* span = ws.span + kbase;
  int32_t* selpre = ws.selpre + kbase + bh;
  int32_t* out = sel_ids + (int64_t)bh * da.k_max;
  const int32_t* sizes = ix.sizes + clu0;
  const int32_t* offs = ix.offsets + off0;
  const int nwords = (C + 31) >> 5;
  int64_t wbase = 0;
  for (int i = 0; i < b; ++i) wbase += (int64_t)da.H * ((sa.C[i] + 31) >> 5);
  uint32_t* selw = ws.selw + wbase + (int64_t)h * nwords;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint64_t ltmask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int per = (C + TK_THREADS - 1) / TK_THREADS;  // key slots per lane
  const int id0 = wv * 64 * per;
  uint32_t ur[NK > 0 ? NK : 1];
  if constexpr (NK > 0) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int j = id0 + 64 * i + lane;
      ur[i] = i < per && j < C ? key32[j] : 0u;
    }
  }
  // f(i, j, u) for every key slot of the lane, slots in order (uniform trip count; u = 0
  // past the clusters)
  auto each = [&](auto&& f) {
    if constexpr (NK > 0) {
#pragma unroll
      for (int i = 0; i < NK; ++i)
        if (i < per) f(i, id0 + 64 * i + lane, ur[i]);
    } else {
      for (int i = 0; i < per; ++i) {
        const int j = id0 + 64 * i + lane;
        f(i, j, j < C ? key32[j] : 0u);
      }
    }
  };
  // sum of a per-wave value over the waves before this one, and over all (one sync)
  auto wave_scan = [&](int slot, int64_t v, int64_t* total) {
    if (lane == 0) wsum[slot][wv] = v;
    __syncthreads();
    int64_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < TK_WAVES; ++w) {
      const int64_t x = wsum[slot][w];
      before += w < wv ? x : 0;
      all += x;
    }
    *total = all;
    return before;
  };
  for (int i = tid; i < nwords; i += TK_THREADS) selw[i] = 0u;
  int ne = 0;
  each([&](int, int, uint32_t u) { ne += __popcll(__ballot(u != 0u)); });
  int64_t nE;
  (void)wave_scan(0, ne, &nE);
  const int k = (int)min((int64_t)da.kreq[b], nE);
  // 1. radix descent
  uint32_t P = 0u;
  int above = 0, done = 0;
  while (k > 0 && done < da.sto_passes && done < 4) {
    for (int i = tid; i < TK_WAVES * 256; i += TK_THREADS) (&hist[0][0])[i] = 0u;
    __syncthreads();
    const int shift = 24 - 8 * done;
    const bool merge = done == 0;
    each([&](int, int, uint32_t u) {
      const bool valid = u != 0u && (done == 0 || (u >> (shift + 8)) == P);
      const uint32_t d = (u >> shift) & 255u;
      if (!merge) {
        if (valid) atomicAdd(&hist[wv][d], 1u);
        return;
      }
      uint64_t active = __ballot(valid);
      while (active != 0ull) {
        const int leader = __ffsll((unsigned long long)active) - 1;
        const uint32_t dv = (uint32_t)__shfl((int)d, leader, 64);
        const uint64_t same = __ballot(valid && d == dv);
        if (lane == leader) atomicAdd(&hist[wv][dv], (uint32_t)__popcll(same));
        active &= ~same;
      }
    });
    __syncthreads();
    if (tid < 256) {
      uint32_t t = 0u;
#pragma unroll
      for (int w = 0; w < TK_WAVES; ++w) t += hist[w][tid];
      hist[0][tid] = t;
    }
    __syncthreads();
    if (wv == 0) {
      // lane l holds bins 255 - 4l .. 252 - 4l; counts from the top as an inclusive scan
      uint32_t c4[4];
      int sum = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c4[e] = hist[0][255 - 4 * lane - e];
        sum += (int)c4[e];
      }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      const int excl = incl - sum;
      if (above + excl < k && k <= above + incl) {  // one lane: the k-th key's bin is here
        int cum = above + excl, t = 255 - 4 * lane, whole = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (cum + (int)c4[e] >= k) {
            t = 255 - 4 * lane - e;
            whole = cum + (int)c4[e] == k;
            break;
          }
          cum += (int)c4[e];
        }
        res[0] = t;
        res[1] = cum;
        res[2] = whole;
      }
    }
    __syncthreads();
    P = (P << 8) | (uint32_t)res[0];
    above = res[1];
    ++done;
    if (res[2]) break;
  }
  // 2. the threshold bin's members: per wave in slot order, then over the waves
  const int fs = 32 - 8 * max(done, 1);
  int nbw = 0;
  each([&](int, int, uint32_t u) { nbw += __popcll(__ballot(u != 0u && (u >> fs) == P)); });
  int64_t nbt;
  const int64_t rb = wave_scan(1, nbw, &nbt);
  // sampling: member r is taken when (r m + c) mod n >= n - m, with n = nb, m = k - above.
  // The wave tracks rem = (r0 m + c) mod n for its next member rank r0; a lane's member
  // rank is r0 + t (t < 64), so (rem + t m) mod n decides in 32 bits (n < 2^26).
  const uint32_t nb = (uint32_t)nbt, mm = (uint32_t)(k - above);
  const uint64_t c =
      nb > 0 ? sm64_mix(da.sto_seed + GAMMA * ((((uint64_t)(uint32_t)b << 32) | (uint32_t)h) + 1) + GAMMA) % nb : 0;
  const uint32_t rem0 = nb > 0 ? (uint32_t)(((uint64_t)rb * mm + c) % nb) : 0u;
  uint32_t rem = rem0;
  auto take = [&](uint32_t u) {  // called for every slot in order by the whole wave
    const bool member = u != 0u && (u >> fs) == P;
    const uint64_t mb = __ballot(member);
    const uint32_t t = (uint32_t)__popcll(mb & ltmask);
    const bool s = k > 0 && u != 0u && ((u >> fs) > P || (member && (rem + t * mm) % nb >= nb - mm));
    if (mb != 0ull) rem = (rem + (uint32_t)__popcll(mb) * mm) % nb;
    return s;
  };
  // 3. the selection: its count per wave, the waves' bases, then the ids in ascending order
  // into the output; spans, member prefixes and the bitmap from one parallel pass over them
  int cnt_w = 0;
  each([&](int, int, uint32_t u) { cnt_w += __popcll(__ballot(take(u))); });
  int64_t kk;
  int64_t pos = wave_scan(2, cnt_w, &kk);
  rem = rem0;
  each([&](int, int j, uint32_t u) {
    const bool s = take(u);
    const uint64_t sm = __ballot(s);
    if (s) out[pos + __popcll(sm & ltmask)] = j;
    pos += __popcll(sm);
  });
  __threadfence_block();
  __syncthreads();
  // entries [e0, e1) of the k per thread, in order
  const int q = (k + TK_THREADS - 1) / TK_THREADS;
  const int e0 = min(tid * q, k), e1 = min(e0 + q, k);
  int64_t mine = 0;
  for (int e = e0; e < e1; ++e)
    mine += sizes[__hip_atomic_load(&out[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)];
  uint64_t rows_all;
  int64_t pre = (int64_t)block_scan_excl((uint64_t)mine, reinterpret_cast<uint64_t*>(&wsum[0][0]), &rows_all);
  for (int e = e0; e < e1; ++e) {
    const int j = __hip_atomic_load(&out[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int n = sizes[j];
    span[e] = make_int2(offs[j], n);
    selpre[e] = (int32_t)pre;
    pre += n;
    atomicOr(&selw[j >> 5], 1u << (j & 31));
  }
  const int64_t tot_rows = (int64_t)rows_all;
  if (tid == 0) {
    selpre[k] = (int32_t)tot_rows;
    ws.counts[4 * bh + 0] = (int32_t)tot_rows;
    ws.counts[4 * bh + 1] = k;
  }
  for (int i = k + tid; i < da.k_max; i += TK_THREADS) out[i] = -1;
  // 4. steady rows: the rank key of their cluster if it is not selected (NaN outside E)
  const Steady sz = steady_of(da, N);
  if (tid == 0) {
    ws.counts[4 * bh + 2] = sz.nS;
    ws.counts[4 * bh + 3] = 0;
  }
  __threadfence_block();
  __syncthreads();
  float* corr = ws.corr + (int64_t)bh * da.scap;
  for (int i = tid; i < sz.nS; i += TK_THREADS) {
    const int32_t j = ix.assign[row0 + steady_pos(sz, i)];
    // the bitmap word as the other threads' atomics left it (read at device scope)
    const uint32_t w = __hip_atomic_load(&selw[j >> 5], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    corr[i] = ((w >> (j & 31)) & 1u) ? __uint_as_float(0x7FC00000u) : keys[j];
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
  return row_sum16(s);
}

// U rows at once: weight 2^(s - m) - 2^(cs - m) (exact term minus the centroid term it
// replaces); s = cs = -inf for padding rows
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

// ------------------------------------------------------------------ appended tokens
// Tokens decoded after the build, attended exactly. They need neither the selection nor
// the rank keys, so their workgroups run in k_score's grid: workgroup (b, g, pt) takes
// appended rows [pt DEC_TAIL_ROWS, +DEC_TAIL_ROWS) of kv head g and every q head of g,
// each row read once for all of them; one partial softmax state per q head.
template <int GS>
__device__ void tail_role(const SeqArgs& sa, const DecodeArgs& da, const uint16_t* q, const DecodeWs& ws, int w) {
  __shared__ float tred[4][GS][PART];
  const int per = sa.G * da.PT;
  const int b = w / per, g = (w / da.PT) % sa.G, pt = w % da.PT;
  const int nT = min(max(da.tail_len[b], 0), da.tail_cap);
  const int r0 = min(pt * DEC_TAIL_ROWS, nT), r1 = min(r0 + DEC_TAIL_ROWS, nT);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, l16 = lane & 15, grp = lane >> 4;
  const int gi = wv * 4 + grp;
  const int s0 = r0 + (r1 - r0) * gi / 16, s1 = r0 + (r1 - r0) * (gi + 1) / 16;
  const float sc = da.tau * LOG2E;
  float qf[GS][8];
#pragma unroll
  for (int hh = 0; hh < GS; ++hh) {
    const uint4 v = *reinterpret_cast<const uint4*>(q + ((int64_t)b * da.H + g * GS + hh) * D + l16 * 8);
    qf[hh][0] = bf16_lo(v.x) * sc; qf[hh][1] = bf16_hi(v.x) * sc; qf[hh][2] = bf16_lo(v.y) * sc;
    qf[hh][3] = bf16_hi(v.y) * sc; qf[hh][4] = bf16_lo(v.z) * sc; qf[hh][5] = bf16_hi(v.z) * sc;
    qf[hh][6] = bf16_lo(v.w) * sc; qf[hh][7] = bf16_hi(v.w) * sc;
  }
  RowState st[GS];
#pragma unroll
  for (int hh = 0; hh < GS; ++hh) {
    st[hh].m = -INFINITY;
    st[hh].l = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) st[hh].acc[d] = 0.f;
  }
  const uint16_t* Kt = da.kt + (int64_t)(b * sa.G + g) * da.tail_cap * D + l16 * 8;
  const uint16_t* Vt = da.vt + (int64_t)(b * sa.G + g) * da.tail_cap * D + l16 * 8;
  constexpr int U = 4;
  for (int r = s0; r < s1; r += U) {
    uint4 kv[U], vv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = min(r + u, s1 - 1);
      kv[u] = *reinterpret_cast<const uint4*>(Kt + e * D);
      vv[u] = *reinterpret_cast<const uint4*>(Vt + e * D);
    }
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      float sv[U], cs[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float x = dot8(qf[hh], kv[u]);
        sv[u] = r + u < s1 ? x : -INFINITY;
        cs[u] = -INFINITY;  // in no cluster: no centroid term to take back
      }
      softmax_rows<U>(st[hh], sv, cs, vv);
    }
  }
  // per q head: merge the 4 groups of a wave, then the 4 waves
#pragma unroll
  for (int hh = 0; hh < GS; ++hh) {
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      const float m2 = xor_shfl(st[hh].m, o), l2 = xor_shfl(st[hh].l, o);
      float a2[8];
#pragma unroll
      for (int d = 0; d < 8; ++d) a2[d] = xor_shfl(st[hh].acc[d], o);
      merge_state(st[hh].m, st[hh].l, st[hh].acc, m2, l2, a2, 8);
    }
    if (grp == 0) {
      if (l16 == 0) { tred[wv][hh][0] = st[hh].m; tred[wv][hh][1] = st[hh].l; }
#pragma unroll
      for (int d = 0; d < 8; ++d) tred[wv][hh][4 + l16 * 8 + d] = st[hh].acc[d];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < GS * D; e += SCORE_THREADS) {
    const int hh = e / D, d = e % D;
    float Mx = -INFINITY;
    for (int w2 = 0; w2 < 4; ++w2) Mx = fmaxf(Mx, tred[w2][hh][0]);
    float Ls = 0.f, A = 0.f;
    if (Mx != -INFINITY)
      for (int w2 = 0; w2 < 4; ++w2) {
        const float f = exp2f(tred[w2][hh][0] - Mx);
        Ls += tred[w2][hh][1] * f;
        A += tred[w2][hh][4 + d] * f;
      }
    float* o = ws.part + (((int64_t)b * da.H + g * GS + hh) * da.NP + (da.NP - da.PT) + pt) * PART;
    if (d == 0) { o[0] = Mx; o[1] = Ls; }
    o[4 + d] = A;
  }
}

// Rows of one (b, h): the members of the selected clusters in selection order,
// then the steady rows. Workgroup `part` takes rows [part*T/P, (part+1)*T/P),
// each 16-lane group a contiguous 1/16 of that.
template <int GS>
__global__ __launch_bounds__(ATT_THREADS) void k_attend(SeqArgs sa, DecodeArgs da, wave_index ix, DecodeWs ws,
                                                        const uint16_t* __restrict__ q) {
  __shared__ float red[4][PART];
  if ((int)blockIdx.x >= sa.B * da.H * da.P) {
    est_role<GS>(sa, da, ix, ws, blockIdx.x - sa.B * da.H * da.P);
    return;
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, l16 = lane & 15, grp = lane >> 4;
  const int gi = wv * 4 + grp;  // 16-lane group in the workgroup
  const float sc = da.tau * LOG2E;
  const int per_bh = da.P;
  const int bh = blockIdx.x / per_bh, part = blockIdx.x % per_bh;
  const int b = bh / da.H, h = bh % da.H, g = h / da.GS;
  const SeqBase sb = seq_base(sa, b);
  const int N = sb.N;
  const int64_t row0 = sb.row + (int64_t)g * sb.NS;
  const int64_t kbase = (int64_t)da.GS * sb.wclu + (int64_t)h * sb.C;
  const int M = ws.counts[4 * bh + 0], k = ws.counts[4 * bh + 1], nS = ws.counts[4 * bh + 2];
  const int T = M + nS;
  const Steady sz = steady_of(da, N);
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
  // The selection's metadata (member prefix, span, rank key of up to kreq clusters)
  // and the steady rows' sorted slots and corrections, loaded into LDS in the same
  // round trip as the counts and q: the searches and windows below then cost LDS
  // latency instead of one dependent global round trip each.
  __shared__ int32_t m_pre[ATT_KCAP + 1];
  __shared__ int2 m_span[ATT_KCAP];
  __shared__ int32_t m_sp[ATT_SCAP];
  __shared__ float m_corr[ATT_SCAP];
  const int kq = da.kreq[b];  // k <= kq <= C: entries up to kq are this head's
  const bool lds_meta = kq <= ATT_KCAP && sz.nS <= ATT_SCAP;
  if (lds_meta) {
    const int tid = threadIdx.x;
    int32_t rp[ATT_KCAP / ATT_THREADS + 1];
    int2 rs[ATT_KCAP / ATT_THREADS];
    int32_t rq[ATT_SCAP / ATT_THREADS];
    float rc[ATT_SCAP / ATT_THREADS];
#pragma unroll
    for (int u = 0; u <= ATT_KCAP / ATT_THREADS; ++u) {
      const int c = tid + u * ATT_THREADS;
      if (c <= kq) rp[u] = selpre[c];
      if (u < ATT_KCAP / ATT_THREADS && c < kq) rs[u] = span[c];
    }
#pragma unroll
    for (int u = 0; u < ATT_SCAP / ATT_THREADS; ++u) {
      const int e = tid + u * ATT_THREADS;
      if (e < sz.nS) {
        rq[u] = ix.inv_perm[row0 + steady_pos(sz, e)];
        rc[u] = corr[e];
      }
    }
#pragma unroll
    for (int u = 0; u <= ATT_KCAP / ATT_THREADS; ++u) {
      const int c = tid + u * ATT_THREADS;
      if (c <= kq) m_pre[c] = rp[u];
      if (u < ATT_KCAP / ATT_THREADS && c < kq) m_span[c] = rs[u];
    }
#pragma unroll
    for (int u = 0; u < ATT_SCAP / ATT_THREADS; ++u) {
      const int e = tid + u * ATT_THREADS;
      if (e < sz.nS) {
        m_sp[e] = rq[u];
        m_corr[e] = rc[u];
      }
    }
    __syncthreads();
  }
  auto pre_of = [&](int c) { return lds_meta ? m_pre[c] : selpre[c]; };
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
    wpre = c <= k ? pre_of(c) : 0x7FFFFFFF;
    wsx = c < k ? (lds_meta ? m_span[c].x : span[c].x) : 0;
    wend = __shfl(c0 + 16 <= k ? pre_of(min(c0 + 16, k)) : 0x7FFFFFFF, gbase, 64);
  };
  if (s0 < min(s1, M)) {
    // 16-ary search for the last cluster whose first row is <= s0
    int lo = 0, hi = k;
    while (hi - lo > 1) {
      const int step = (hi - lo + 15) / 16;
      const int c = lo + l16 * step;
      const int v = c < hi ? pre_of(c) : 0x7FFFFFFF;
      const uint32_t m = (uint32_t)(__ballot(v <= s0) >> gbase) & 0xFFFFu;
      const int cnt = __popc(m);
      lo = lo + (cnt - 1) * step;
      hi = min(lo + step, hi);
    }
    load_window(lo);
  }
  constexpr int U = 8;
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
      const int l = gbase + __popc(m) - 1;
      const int32_t p = __shfl(wsx, l, 64) + row - __shfl(wpre, l, 64);
      t[u] = ix.perm[row0 + p];
      kv[u] = *reinterpret_cast<const uint4*>(Ks + (int64_t)p * D);
      vv[u] = *reinterpret_cast<const uint4*>(Vs + (int64_t)p * D);
    }
    float sv[U], cs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float x = dot8(qf, kv[u]);
      const bool valid = r + u < r1;
      const bool steady = t[u] < sz.a_end || t[u] >= sz.c_beg;  // counted exactly with the steady rows
      sv[u] = (valid && !steady) ? x : -INFINITY;
      cs[u] = -INFINITY;  // a selected cluster has no centroid term to take back
    }
    softmax_rows<U>(st, sv, cs, vv);
  }
  // steady rows: entries e = row - M for rows [max(s0, M), s1)
  const int r2 = s1;
  for (int r = max(s0, M); r < r2; r += U) {
    int32_t p[U];
    float cvv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = min(r + u, r2 - 1) - M;
      p[u] = lds_meta ? m_sp[e] : ix.inv_perm[row0 + steady_pos(sz, e)];
      cvv[u] = lds_meta ? m_corr[e] : corr[e];
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
      const bool valid = r + u < r2;
      sv[u] = valid ? x : -INFINITY;
      cs[u] = (valid && da.est && cvv[u] == cvv[u]) ? cvv[u] * sc : -INFINITY;
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
    float Mx = -INFINITY;
    for (int w2 = 0; w2 < 4; ++w2) Mx = fmaxf(Mx, red[w2][0]);
    float Ls = 0.f, A = 0.f;
    if (Mx != -INFINITY)
      for (int w2 = 0; w2 < 4; ++w2) {
        const float f = exp2f(red[w2][0] - Mx);
        Ls += red[w2][1] * f;
        A += red[w2][4 + d] * f;
      }
    float* o = ws.part + ((int64_t)bh * da.NP + part) * PART;
    if (d == 0) { o[0] = Mx; o[1] = Ls; }
    o[4 + d] = A;
  }
}

// ------------------------------------------------------------------ k_merge
// Log-sum-exp merge of the partials of one (b, h): the P row partials, one centroid
// partial per estimation chunk and the tail workgroups' partials. SPLIT workgroups per
// (b, h), each 128 / SPLIT dims: all take the maximum and the total weight over every
// partial; thread (sub, dq) sums dims 4dq..4dq+3 of its workgroup's part over partials sub,
// sub + nsub, ...; the subsets meet in LDS. Row partials may carry negative sums (they take
// centroid terms back out); the total is positive. The host splits a head's merge 4 ways
// when it has many partials (the 1M layer's ~590 per head: 19 -> 11 us) and not otherwise
// (the batched layers' 512 heads with ~80 each merged 30% slower split).
constexpr int MERGE_SPLIT_MIN_PARTIALS = 256;

template <int SPLIT>
__global__ __launch_bounds__(256) void k_merge(SeqArgs sa, DecodeArgs da, DecodeWs ws, float* __restrict__ out,
                                               float* __restrict__ lse) {
  __shared__ float4 accs[256];
  __shared__ float ls[32];
  __shared__ float mx[4];
  const int bh = blockIdx.x / SPLIT, dpart = blockIdx.x % SPLIT;
  const int b = bh / da.H;
  // partials: P row workgroups, this sequence's estimation chunks, then the PT appended-token
  // workgroups (after the slots of the longest sequence's chunks)
  const int nlead = da.P + (da.est ? (sa.C[b] + SC - 1) / SC : 0);
  const int npart = nlead + da.PT;
  const int skip = da.NP - da.PT - nlead;
  auto slot = [&](int i) { return (int64_t)(i < nlead ? i : i + skip) * PART; };
  const float* pp = ws.part + (int64_t)bh * da.NP * PART;
  constexpr int nd = 32 / SPLIT, nsub = 256 / nd;  // float4 columns of the part, subsets
  const int tid = threadIdx.x, dq = tid % nd, sub = tid / nd;
  const int d0 = (D / SPLIT) * dpart;
  float M = -INFINITY;
  for (int i = tid; i < npart; i += 256) M = fmaxf(M, pp[slot(i)]);
  M = wave_max(M);
  if ((tid & 63) == 0) mx[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
  float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
  float Ls = 0.f;
#pragma unroll 4
  for (int i = sub; i < npart; i += nsub) {
    const float* p = pp + slot(i);
    const float mi = p[0];
    const float4 a = *reinterpret_cast<const float4*>(p + 4 + d0 + 4 * dq);
    const float li = p[1];
    const float f = (mi == -INFINITY) ? 0.f : exp2f(mi - M);
    Ls += li * f;
    A.x += a.x * f; A.y += a.y * f; A.z += a.z * f; A.w += a.w * f;
  }
  accs[tid] = A;
  if (dq == 0) ls[sub] = Ls;
  __syncthreads();
  if (tid < nd) {
    float4 s = accs[tid];
    float Lt = ls[0];
    for (int k = 1; k < nsub; ++k) {
      const float4 t = accs[k * nd + tid];
      s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
      Lt += ls[k];
    }
    float4 r;
    r.x = s.x / Lt; r.y = s.y / Lt; r.z = s.z / Lt; r.w = s.w / Lt;
    *reinterpret_cast<float4*>(out + (int64_t)bh * D + d0 + 4 * tid) = r;
    if (lse != nullptr && tid == 0 && dpart == 0) lse[bh] = (M + log2f(Lt)) * 0.6931471805599453f;
  }
}

// ------------------------------------------------------------------ host side
hipError_t decode_set_attrs() {
  const size_t tl = sizeof(TopkLds);
  const void* fns[] = {reinterpret_cast<const void*>(&k_topk<0>),  reinterpret_cast<const void*>(&k_topk<1>),
                       reinterpret_cast<const void*>(&k_topk<2>),  reinterpret_cast<const void*>(&k_topk<4>),
                       reinterpret_cast<const void*>(&k_topk<8>),  reinterpret_cast<const void*>(&k_topk<16>),
                       reinterpret_cast<const void*>(&k_topk<32>), reinterpret_cast<const void*>(&k_topk<8, false>)};
  for (const void* f : fns) WAVE_TRY(hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, tl));
  return hipSuccess;
}

template <int GS>
static hipError_t launch_gs(const SeqArgs& sa, const DecodeArgs& da, const wave_index& ix, const DecodeWs& ws,
                            const uint16_t* q, float* out, int32_t* sel_ids, float* lse, hipStream_t st, int nscore,
                            int nest) {
  if (da.PT > 0)
    WAVE_TRY(launch("k_score", k_score<GS, true>, dim3(nscore + sa.B * sa.G * da.PT), dim3(SCORE_THREADS), 0, st, sa,
                    da, ix, q, ws));
  else
    WAVE_TRY(launch("k_score", k_score<GS, false>, dim3(nscore), dim3(SCORE_THREADS), 0, st, sa, da, ix, q, ws));
  const dim3 tg(sa.B * da.H), tb(TK_THREADS);
  const size_t tl = sizeof(TopkLds);
  void (*tk)(SeqArgs, DecodeArgs, wave_index, DecodeWs, int32_t*);
  switch (da.NV) {
    case 1: tk = k_topk<1>; break;
    case 2: tk = k_topk<2>; break;
    case 4: tk = k_topk<4>; break;
    case 8: tk = sa.B * da.H > 256 ? k_topk<8, false> : k_topk<8, true>; break;
    case 16: tk = k_topk<16>; break;
    case 32: tk = k_topk<32>; break;
    default: tk = k_topk<0>; break;
  }
  if (da.sto_passes > 0) {
    int cmax = 0;
    for (int b = 0; b < sa.B; ++b) cmax = sa.C[b] > cmax ? sa.C[b] : cmax;
    const int per = (cmax + TK_THREADS - 1) / TK_THREADS;
    WAVE_TRY(launch("k_topk_sto", per <= 8 ? k_topk_sto<8> : per <= 64 ? k_topk_sto<64> : k_topk_sto<0>, tg, tb, 0,
                    st, sa, da, ix, ws, sel_ids));
  } else {
    WAVE_TRY(launch("k_topk", tk, tg, tb, tl, st, sa, da, ix, ws, sel_ids));
  }
  WAVE_TRY(launch("k_attend", k_attend<GS>, dim3(sa.B * da.H * da.P + (da.est ? nest : 0)), dim3(ATT_THREADS), 0, st,
                  sa, da, ix, ws, q));
  if (da.NP >= MERGE_SPLIT_MIN_PARTIALS)
    WAVE_TRY(launch("k_merge", k_merge<4>, dim3(sa.B * da.H * 4), dim3(256), 0, st, sa, da, ws, out, lse));
  else
    WAVE_TRY(launch("k_merge", k_merge<1>, dim3(sa.B * da.H), dim3(256), 0, st, sa, da, ws, out, lse));
  return hipSuccess;
}

hipError_t launch_decode(const SeqArgs& sa, const DecodeArgs& da, const wave_index& ix, const DecodeWs& ws,
                         const uint16_t* q, float* out, int32_t* sel_ids, float* lse, hipStream_t st) {
  WAVE_TRY(device_info().status);
  int nscore = 0, nest = 0;
  for (int b = 0; b < sa.B; ++b) {
    nscore += sa.G * ((sa.C[b] + SC - 1) / SC);
    nest += sa.G * ((sa.C[b] + SC - 1) / SC);
  }
  switch (da.GS) {
    case 1: return launch_gs<1>(sa, da, ix, ws, q, out, sel_ids, lse, st, nscore, nest);
    case 2: return launch_gs<2>(sa, da, ix, ws, q, out, sel_ids, lse, st, nscore, nest);
    case 3: return launch_gs<3>(sa, da, ix, ws, q, out, sel_ids, lse, st, nscore, nest);
    case 4: return launch_gs<4>(sa, da, ix, ws, q, out, sel_ids, lse, st, nscore, nest);
    case 5: return launch_gs<5>(sa, da, ix, ws, q, out, sel_ids, lse, st, nscore, nest);
    case 6: return launch_gs<6>(sa, da, ix, ws, q, out, sel_ids, lse, st, nscore, nest);
    case 7: return launch_gs<7>(sa, da, ix, ws, q, out, sel_ids, lse, st, nscore, nest);
    default: return launch_gs<8>(sa, da, ix, ws, q, out, sel_ids, lse, st, nscore, nest);
  }
}

}  // namespace wave
