// internal.h -- declarations shared by the library's translation units (not installed).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "common.h"

namespace wave {

// ------------------------------------------------------------------ decode
struct DecodeArgs {
  int32_t H, GS;          // q heads, q heads per kv head
  int32_t n_sink, n_local;
  int32_t k_max;          // id columns of the output
  int32_t P;              // gathered-row workgroups per (b, h)
  int32_t NV;             // keys per lane of the register top-k (1, 2, ..., 32), 0: keys read from memory
  int32_t NP;             // partial slots per (b, h): P + max_b ceil(C_b / DEC_SCORE_CH) + PT
  int32_t scap;           // steady entries per (b, h)
  float tau;              // 1/sqrt(128)
  int32_t sort_stride;    // per-(b, h) entries of the global sort buffer
  int32_t NVg;            // keys per lane when NV == 0 (a multiple of 16)
  int32_t est;            // 1: the estimation zone (wave attention); 0: top-k retrieval only
  int32_t shared;         // 1: one selection per kv head, by the sum of its q heads' rank keys
  const uint16_t* kt;     // tokens appended after the build, keys [B][G][tail_cap][128] (nullptr: none)
  const uint16_t* vt;     // and values
  const int32_t* tail_len;  // device [B]: appended tokens of sequence b (clamped to [0, tail_cap])
  int32_t tail_cap;
  int32_t PT;             // appended-token workgroups per (b, g) in the k_score grid (0: none)
  int32_t nscore;         // scoring workgroups of the k_score grid (the tail workgroups follow)
  int32_t sto_passes;     // > 0: the stochastic radix top-k (k_topk_sto) with that many 8-bit passes
  uint64_t sto_seed;      // its sampling seed
  int32_t kreq[MAXB];     // min(ceil(topk_frac * C_b), C_b), binary64 on the host
};

struct DecodeWs {
  float* keys;       // [sum_b H*C_b] rank keys
  uint32_t* key32;   // [sum_b H*C_b] sortable keys, 0 = not eligible
  int2* span;        // [sum_b H*C_b] (first sorted slot, size) of the i-th selected cluster
  int32_t* selpre;   // [sum_b H*(C_b+1)] rows of the selection before its i-th cluster
  uint32_t* selw;    // [sum_b H*ceil(C_b/32)] each q head's selection bitmap (k_topk; read by the estimation role)
  float* corr;       // [B*H*scap] rank key of a steady row's cluster if it is not selected, else NaN
  int32_t* counts;   // [B*H*4] rows of the selected clusters, k, steady rows, 0
  float* part;       // [B*H*NP*132] partial softmax states: P row workgroups, then max_b ceil(C_b / 128)
                     // estimation chunks, then PT appended-token workgroups
  uint32_t* ctop;    // [B*H*(NP-P)*8] per 128-cluster chunk of a (b, h): its DEC_CHUNK_TOPS largest sortable keys, eligible count
  uint64_t* sortg;   // [B*H*pow2(C_max)] global sort buffer (only when k_max > 4096)
};

constexpr int DEC_SCORE_CH = 128;
// Largest sortable keys per 128-cluster chunk that k_score records for the top-k of keys
// beyond registers (slots 0..6 of the chunk's 8-word record, the eligible count in slot 7):
// the k-th largest of them bounds the k-th key from below. With 4 (1M layer: 1180 of 65,536)
// up to 2,139 keys passed that bound and a few heads sorted 4,096 candidates (the slowest
// head sets the launch time); with 7 the bound is nearly tight.
constexpr int DEC_CHUNK_TOPS = 7;
constexpr int DEC_TK_WAVES = 16;  // waves of a k_topk workgroup (one per (sequence, q head))
constexpr int DEC_PART = 132;
constexpr int DEC_SORT_LDS = 4096;
// Rows per gathering workgroup of k_attend. With fewer rows per workgroup each 16-lane
// group needs fewer dependent load rounds, which pays while the whole grid (row and
// estimation workgroups) is resident at once: DEC_ROWS_SMALL then, DEC_ROWS_PER_WG when
// the grid takes several rounds anyway (measured: a 32-head 128K layer 17.6 -> 14.0 us
// per launch at 176; the 1M and batched layers about 3% slower at 176 than at 256).
// DEC_ATT_SLOTS: k_attend workgroups resident at once on 256 CUs (4 each: 256 threads
// and at most 128 registers per lane for up to 4 q heads per kv head).
constexpr int DEC_ROWS_SMALL = 176;
constexpr int DEC_ROWS_PER_WG = 256;
constexpr int DEC_ATT_SLOTS = 1024;
// Appended tokens per tail workgroup (in the k_score grid; 4 per 16-lane group, one batch of
// loads: 4096 tokens take 64 workgroups per kv head).
constexpr int DEC_TAIL_ROWS = 64;

hipError_t launch_decode(const SeqArgs& sa, const DecodeArgs& da, const wave_index& ix, const DecodeWs& ws,
                         const uint16_t* q, float* out, int32_t* sel_ids, float* lse, hipStream_t st);

// ------------------------------------------------------------------ build
struct BuildWs {
  float* norm;        // [index clusters] |chat_j|^2 (fp32) of the current round
  int32_t* rank;      // [input rows] scratch of the counting sort
  float* xn2;         // [input rows] |x|^2 of every key (written by the first k_assign round)
  int32_t* big;       // the sort's lists of large clusters: 2 counters, 2 x BUILD_BIG_CAP ids, then a
                      // byte per index cluster (BUILD_BIG_WORDS + clusters bytes)
};
constexpr int BUILD_BIG_CAP = 4096;
constexpr int64_t BUILD_BIG_WORDS = 2 + 2 * (int64_t)BUILD_BIG_CAP;

hipError_t launch_build(const SeqArgs& sa, const void* K, const void* V, int32_t iters, uint64_t seed,
                        const wave_index& ix, const BuildWs& ws, int32_t* trace, int64_t rows, hipStream_t st);
hipError_t launch_build_blocks(const SeqArgs& sa, const void* K, const void* V, const wave_index& ix,
                               const BuildWs& ws, hipStream_t st);
// sa: the longer context (sa.cap > 0); n_old: host [B], the context the index holds.
// stage_k, stage_v: workspace of [append input rows][128] bf16 each.
hipError_t launch_append(const SeqArgs& sa, const int32_t* n_old, const void* Kn, const void* Vn, int32_t iters,
                         uint64_t seed, const wave_index& ix, const BuildWs& ws, void* stage_k, void* stage_v,
                         hipStream_t st);

// ------------------------------------------------------------------ per-device set-up
// Done once per device (std::call_once), on the first call that launches work there:
// the dynamic LDS limits of the kernels that need more than the default, the device's
// compute-unit count and the address of its static decode scratch. status is the first
// failing HIP call's code.
struct DeviceInfo {
  hipError_t status;
  int cus;
  void* scratch;  // device address of this device's copy of the static decode scratch
};
const DeviceInfo& device_info();
hipError_t build_set_attrs();   // build.hip
hipError_t decode_set_attrs();  // decode.hip

// ------------------------------------------------------------------ kernel launches
// While the timing hook is on, prof_events hands out the start/stop event pair of one
// launch (recorded by the dispatch itself through hipExtLaunchKernel, so the pair times
// the kernel alone) and files it under `name`; otherwise it returns false.
bool prof_events(const char* name, hipEvent_t* start, hipEvent_t* stop);

template <typename Tup, size_t... I>
void fill_ptrs(Tup& t, void** p, std::index_sequence<I...>) {
  void* v[] = {static_cast<void*>(&std::get<I>(t))..., nullptr};
  for (size_t i = 0; i < sizeof...(I); ++i) p[i] = v[i];
}

// Launch `kern` on `st` with arguments converted to the kernel's parameter types; returns
// the launch status. `name` files the launch's duration while the timing hook is on.
template <typename... KA, typename... A>
hipError_t launch(const char* name, void (*kern)(KA...), dim3 grid, dim3 block, size_t lds, hipStream_t st,
                  A&&... a) {
  static_assert(sizeof...(KA) == sizeof...(A), "kernel argument count");
  std::tuple<KA...> args(std::forward<A>(a)...);
  void* ptrs[sizeof...(KA) + 1];
  fill_ptrs(args, ptrs, std::index_sequence_for<KA...>{});
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (prof_events(name, &e0, &e1))
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, ptrs, lds, st, e0, e1, 0);
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, ptrs, lds, st);
}

// return the status of a HIP call from the enclosing function unless it succeeded
#define WAVE_TRY(...)                          \
  do {                                         \
    const hipError_t wave_e_ = (__VA_ARGS__);  \
    if (wave_e_ != hipSuccess) return wave_e_; \
  } while (0)

}  // namespace wave
