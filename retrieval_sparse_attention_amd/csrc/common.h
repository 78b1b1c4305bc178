// common.h -- shared device/host helpers of the wave-index library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/wave_attn.h"

namespace wave {

constexpr int D = WAVE_HEAD_DIM;  // 128
constexpr int MAXB = WAVE_MAX_BATCH;

// Per-call description of the ragged batch, passed to kernels by value.
// N[b]: tokens of sequence b; C[b]: its clusters per kv head.
struct SeqArgs {
  int32_t B, G, seg_len, K_s;
  int32_t N[MAXB];
  int32_t C[MAXB];
};

// Bases of sequence b in the ragged arrays (all per-sequence blocks are G-fold).
struct SeqBase {
  int64_t row;   // first row: G * sum_{b'<b} N_b'
  int64_t clu;   // first cluster: G * sum C_b'
  int64_t off;   // first offsets entry: G * sum (C_b' + 1)
  int32_t N, C;
};

__host__ __device__ inline SeqBase seq_base(const SeqArgs& s, int b) {
  SeqBase r{0, 0, 0, 0, 0};
  for (int i = 0; i < b; ++i) {
    r.row += (int64_t)s.G * s.N[i];
    r.clu += (int64_t)s.G * s.C[i];
    r.off += (int64_t)s.G * (s.C[i] + 1);
  }
  r.N = s.N[b];
  r.C = s.C[b];
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

}  // namespace wave
