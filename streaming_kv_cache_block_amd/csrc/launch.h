// launch.h -- host-callable launchers of the device kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "split_plan.h"

namespace ll {

constexpr int kMaxPlan = 128;  // = LL_MAX_SLOTS
constexpr int kMaxRuns = 3;    // runs of slots holding a chunk's cached context

// One attention call: queries of one chunk against the cached runs of slots and the
// chunk's own keys.  All token tensors are [tokens][H][D], row stride H*D elements.
struct AttnParams {
  const uint16_t* Q;
  const uint16_t* Kc;   // own-chunk keys (bf16)
  const uint16_t* Vc;   // own-chunk values (bf16)
  uint16_t* out;
  const void* cK;       // cached keys: the layer's slot array (bf16, int8, fp8 or fp4 codes)
  const void* cV;
  const float* cKs;     // int8 / fp8: per (token, head) scales; MX formats: per (token,
  const float* cVs;     //   head) words of four E8M0 block-scale bytes (read as raw bits)
  int nq;               // query rows = own-chunk key rows
  int ncache;           // cached key rows (sum of the runs)
  int nrun;             // runs of cached rows (0..kMaxRuns)
  int run_row0[kMaxRuns];   // first row (slot * T) of each run in the slot array
  int run_rows[kMaxRuns];
  int H;
  float c;              // log2(e) / sqrt(D)
  // Work-split buffers of this call (the layer's own, so layers may run concurrently
  // on different streams; may be null: then no split): partial-result slots, per-block
  // arrival counters (all zero between calls), CU count.
  float* ws;
  int64_t ws_slots;
  int* cnt;
  int n_cu;
};

// Floats of one partial-result slot: O [rows][D] + m [rows] + l [rows], 256-byte aligned.
inline __host__ __device__ int64_t split_slot_floats(int D, int rows) {
  return (int64_t(rows) * (D + 2) + 63) / 64 * 64;
}

// Most query rows of one attention block (the work area's slot size is for these).
constexpr int kAttnRows = 256;

// kv_fmt: 0 bf16 cache, 1 int8 codes, 2 fp8 (E4M3) codes (+ fp32 scales), 3 MXFP4
// (E2M1 codes + E8M0 block scales), 4 MXFP8 (E4M3 codes + E8M0 block scales).
hipError_t launch_attention(const AttnParams& p, int D, int kv_fmt, hipStream_t s);

// Whether launch_attention would split the key walk of p (given a large enough work
// area): the blocks leave CUs idle and the walk is long enough.
bool attention_would_split(const AttnParams& p, int D);

// Copy (bf16) or quantise (int8 / fp8 / mxfp4 / mxfp8) whole frames of a [frames*T][H][D] bf16 tensor into
// cache slots.  plan_src[i] is the frame index in the source tensor, plan_slot[i] the
// destination slot, for i < n.
struct WriteParams {
  const uint16_t* srcK;
  const uint16_t* srcV;
  void* dstK;           // slot array of the layer: [S+W][T][H][D]
  void* dstV;
  float* dstKs;         // int8 / fp8: [S+W][T][H] fp32; MX formats: [S+W][T][H] scale words
  float* dstVs;
  int64_t rows_per_frame;  // T*H
  int n;
  int plan_src[kMaxPlan];
  int plan_slot[kMaxPlan];
};

hipError_t launch_kv_write(const WriteParams& p, int D, int kv_fmt, hipStream_t s);

// out[m][n] = sum_k h[m][k] * W[n][k] for W = W_K and W_V (bf16 in, fp32 sums,
// bf16 out).  M rows, K = d_in (multiple of 64), N = d_out (multiple of 128).
struct ProjParams {
  const uint16_t* h;
  const uint16_t* WK;
  const uint16_t* WV;
  uint16_t* outK;
  uint16_t* outV;
  int M, K, N;
};

hipError_t launch_kv_project(const ProjParams& p, hipStream_t s);

// Projection whose epilogue writes straight into cache slots: output row m (frame
// m / T, token m % T) goes to slot plan_slot[m / T]; N = H * D.  Low-bit caches get the
// quantisation of the bf16-rounded results by their format's rule (same bits as
// projecting, then quantising the stored bf16 tensor).
struct ProjToCacheParams {
  ProjParams proj;      // outK/outV unused
  int T, H, D;
  int kv_fmt;           // 0 bf16, 1 int8, 2 fp8, 3 mxfp4, 4 mxfp8
  void* slotK;          // layer slot arrays [S+W][T][H][D]
  void* slotV;
  float* scK;           // low-bit caches: [S+W][T][H] scales (fp32, or MX scale words)
  float* scV;
  int n_plan;
  int plan_slot[kMaxPlan];    // slot of frame i of the projected rows
  int plan_slot2[kMaxPlan];   // a second slot holding the same frame, or -1
};

hipError_t launch_kv_project_to_cache(const ProjToCacheParams& p, hipStream_t s);

}  // namespace ll
