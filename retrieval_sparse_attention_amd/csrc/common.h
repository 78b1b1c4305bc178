// common.h -- shared device/host helpers of the wave-index library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/wave_attn.h"

namespace wave {

constexpr int D = WAVE_HEAD_DIM;  // 128
constexpr int MAXB = WAVE_MAX_BATCH;

// Per-call description of the ragged batch, passed to kernels by value.
// N[b]: tokens of sequence b; C[b]: its clusters per kv head. cap: 0 for the dense
// ragged layout of the index arrays (block (b, g) holds N_b rows and C_b clusters),
// else the capacity of every block in segments (cap * seg_len rows, cap * K_s
// clusters, of which the first N_b and C_b are filled).
struct SeqArgs {
  int32_t B, G, seg_len, K_s;
  int32_t cap, pad_;
  int32_t N[MAXB];
  int32_t C[MAXB];
};

// Bases of sequence b (all per-sequence blocks are G-fold).
struct SeqBase {
  int64_t row;   // index: first row, G * sum_{b'<b} NS_b'
  int64_t clu;   // index: first cluster, G * sum CS_b'
  int64_t off;   // index: first offsets entry, G * sum (CS_b' + 1)
  int64_t wclu;  // G * sum_{b'<b} C_b': first cluster in the dense per-call workspaces
  int32_t N, C;
  int32_t NS, CS;  // rows and clusters of one block (kv head) of sequence b in the index arrays
};

__host__ __device__ inline SeqBase seq_base(const SeqArgs& s, int b) {
  SeqBase r{0, 0, 0, 0, 0, 0, 0, 0};
  for (int i = 0; i < b; ++i) {
    const int64_t R = s.cap ? (int64_t)s.cap * s.seg_len : s.N[i];
    const int64_t Cs = s.cap ? (int64_t)s.cap * s.K_s : s.C[i];
    r.row += (int64_t)s.G * R;
    r.clu += (int64_t)s.G * Cs;
    r.off += (int64_t)s.G * (Cs + 1);
    r.wclu += (int64_t)s.G * s.C[i];
  }
  r.N = s.N[b];
  r.C = s.C[b];
  r.NS = s.cap ? s.cap * s.seg_len : s.N[b];
  r.CS = s.cap ? s.cap * s.K_s : s.C[b];
  return r;
}

// Clusters of a segment of length L (full segments: K_s; a short last one:
// ceil(L*K_s/L_s)) and of a whole sequence.
__host__ __device__ inline int32_t seg_clusters(int64_t L, int32_t seg_len, int32_t K_s) {
  if (L >= seg_len) return K_s;
  return (int32_t)((L * (int64_t)K_s + seg_len - 1) / seg_len);
}

__host__ __device__ inline int64_t num_clusters(int64_t N, int32_t seg_len, int32_t K_s) {
  int64_t nseg = (N + seg_len - 1) / seg_len;
  return (nseg - 1) * (int64_t)K_s + seg_clusters(N - (nseg - 1) * seg_len, seg_len, K_s);
}

// ---------------------------------------------------------------- SplitMix64
// Steele, Lea and Flood, "Fast splittable pseudorandom number generators" (OOPSLA
// 2014): the state advances by GAMMA and each output is the state through this mixer
// (variant 13), so the i-th output of the stream starting at state s is
// sm64_mix(s + GAMMA * (i + 1)).
constexpr uint64_t GAMMA = 0x9E3779B97F4A7C15ULL;

__device__ __forceinline__ uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

// ---------------------------------------------------------------- XCD-aware workgroup order
// Workgroups are dispatched round robin over the 8 XCDs (workgroup w runs on XCD
// w mod 8), each with its own L2. The linear index of w in a grid of n puts
// XCD x's workgroups at one contiguous run of [0, n), so neighbouring work
// items (here: the workgroups of one k-means unit, which read the same
// centroids) share an L2. A bijection of [0, n) for any n.
__device__ __forceinline__ int xcd_linear(int w, int n) {
  const int x = w & 7, s = w >> 3;
  const int q = n >> 3, r = n & 7;  // XCD x holds q + (x < r) workgroups
  return x * q + min(x, r) + s;
}

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round to nearest, ties to even; NaN kept quiet
__device__ __forceinline__ uint16_t f_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// order-preserving map of finite floats to unsigned ints; +0 and -0 both map
// to 0x80000000, and every finite value maps to >= 0x00800000 (0 is free as a
// "not eligible" sentinel below every key)
__device__ __forceinline__ uint32_t float_sortable(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float sortable_float(uint32_t s) {
  uint32_t u = (s & 0x80000000u) ? (s & 0x7FFFFFFFu) : ~s;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T>
__device__ __forceinline__ T xor_shfl(T v, int m) {
  return __shfl_xor(v, m, 64);
}

// value held by lane (i - N) mod 16 of this lane's row of 16 (DPP row rotate; no LDS)
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a row with the association of an xor butterfly of
// strides 8, 4, 2, 1: lane i adds the value of lane (i - N) mod 16, which differs
// from lane i ^ N only in bits whose partial sums are already equal, so every
// lane ends with the bits of the xor-exchange butterfly.
__device__ __forceinline__ float row_sum16(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  v += row_ror<1>(v);
  return v;
}

__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, row_ror<8>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<2>(v));
  v = fmaxf(v, row_ror<1>(v));
  return v;
}

// value held by lane i ^ 32 (v_permlane32_swap; no LDS)
__device__ __forceinline__ uint32_t swap32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}
__device__ __forceinline__ float swap32(float v) { return __uint_as_float(swap32(__float_as_uint(v))); }
__device__ __forceinline__ int swap32(int v) { return (int)swap32((uint32_t)v); }

// workgroup barrier for LDS traffic only: waits for this wave's LDS operations,
// not for its outstanding global loads (unlike __syncthreads)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
}

// full-wave reductions: rows by DPP, then lanes i ^ 16 (LDS exchange) and i ^ 32
__device__ __forceinline__ float wave_max(float v) {
  v = row_max16(v);
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, swap32(v));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  v += __shfl_xor(v, 16, 64);
  return v + swap32(v);
}

}  // namespace wave
