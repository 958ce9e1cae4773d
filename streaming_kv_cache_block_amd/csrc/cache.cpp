// cache.cpp -- the C ABI: cache handle, host bookkeeping, validation, kernel dispatch.
//
// The handle owns one device allocation holding, per layer, the K and V slot arrays
// [S+W][T][H][D] (bf16, int8, fp8 or MXFP8; MXFP4 [S+W][T][H][D/2] bytes), for the
// low-bit caches their [S+W][T][H] scales (fp32, or for the MX formats words of E8M0
// block-scale bytes),
// and the attention work area of the split key walk (partials and counters).  Host
// bookkeeping per layer: frames seen (f0) and the frame held by each slot.  Every
// argument is checked before the first HIP call so that errors are testable on a
// machine without a GPU.
#include "../../include/ll_cache.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <mutex>
#include <string>
#include <vector>

#include "launch.h"
#include "slots.h"

static_assert(LL_MAX_SLOTS == ll::kMaxPlan, "plan table size must match LL_MAX_SLOTS");

struct ll_cache {
  int layers = 0, heads = 0, head_dim = 0, T = 0, S = 0, Ss = 0, W = 0;
  int kv_dtype = LL_KV_BF16;
  int device = -1;
  int64_t rows_per_frame = 0;   // T * heads
  size_t kv_bytes = 0;          // one K (or V) slot array of one layer
  size_t sc_bytes = 0;          // one K (or V) scale array of one layer
  int n_cu = 0;                 // compute units of the device
  // Attention work-split buffers, one set per layer (layers may run on different
  // streams at once): partial-result slots, then after all layers' slots the per-block
  // arrival counters.
  size_t ws_offset = 0;
  size_t ws_layer_bytes = 0;
  int64_t ws_slots = 0;
  size_t cnt_offset = 0;
  size_t cnt_layer_bytes = 0;
  void* mem = nullptr;
  std::vector<int64_t> f0;
  std::vector<int64_t> fs;      // first frame of the current shot (shot sink)
  std::vector<std::vector<int64_t>> slot_frame;

  ll::Layout layout() const { return ll::Layout{S, Ss, W}; }

  char* base() const { return static_cast<char*>(mem); }
  void* k(int l) const { return base() + (size_t(2) * l) * kv_bytes; }
  void* v(int l) const { return base() + (size_t(2) * l + 1) * kv_bytes; }
  float* ks(int l) const {
    return sc_bytes ? reinterpret_cast<float*>(base() + size_t(2) * layers * kv_bytes + (size_t(2) * l) * sc_bytes) : nullptr;
  }
  float* vs(int l) const {
    return sc_bytes ? reinterpret_cast<float*>(base() + size_t(2) * layers * kv_bytes + (size_t(2) * l + 1) * sc_bytes)
                    : nullptr;
  }
  float* ws(int l) const { return reinterpret_cast<float*>(base() + ws_offset + size_t(l) * ws_layer_bytes); }
  int* cnt(int l) const { return reinterpret_cast<int*>(base() + cnt_offset + size_t(l) * cnt_layer_bytes); }
};

namespace {

thread_local std::string g_err;

ll_status fail(ll_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ll_status fail(ll_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

ll_status ok() {
  g_err.clear();
  return LL_OK;
}

ll_status hip_fail(hipError_t e, const char* what) {
  (void)hipGetLastError();  // clear the sticky launch error for the next call
  return fail(LL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxRows = int64_t(1) << 30;   // token rows addressed with int arithmetic

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

ll_status check_layer(const ll_cache* c, int layer) {
  if (!c) return fail(LL_ERR_INVALID, "null cache handle");
  if (layer < 0 || layer >= c->layers) return fail(LL_ERR_INVALID, "layer %d out of range [0, %d)", layer, c->layers);
  return LL_OK;
}

ll_status check_tensor(const void* p, const char* name) {
  if (!p) return fail(LL_ERR_INVALID, "%s is NULL", name);
  if (!aligned16(p)) return fail(LL_ERR_INVALID, "%s is not 16-byte aligned", name);
  return LL_OK;
}

ll_status check_frames(const ll_cache* c, int n_frames) {
  if (n_frames <= 0) return fail(LL_ERR_INVALID, "n_frames must be >= 1 (got %d)", n_frames);
  if (int64_t(n_frames) * c->T > kMaxRows) return fail(LL_ERR_INVALID, "n_frames * tokens_per_frame too large");
  return LL_OK;
}

ll_status check_device(const ll_cache* c) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != c->device)
    return fail(LL_ERR_INVALID, "current device %d is not the cache's device %d", dev, c->device);
  return LL_OK;
}

#define LL_TRY(expr)                 \
  do {                               \
    ll_status _s = (expr);           \
    if (_s != LL_OK) return _s;      \
  } while (0)

ll_status write_frames(ll_cache* c, int layer, const void* K, const void* V, const std::vector<ll::WriteEntry>& plan,
                       hipStream_t s, const char* what) {
  ll::WriteParams wp{};
  wp.srcK = static_cast<const uint16_t*>(K);
  wp.srcV = static_cast<const uint16_t*>(V);
  wp.dstK = c->k(layer);
  wp.dstV = c->v(layer);
  wp.dstKs = c->ks(layer);
  wp.dstVs = c->vs(layer);
  wp.rows_per_frame = c->rows_per_frame;
  wp.n = int(plan.size());
  for (size_t i = 0; i < plan.size(); ++i) {
    wp.plan_src[i] = plan[i].src;
    wp.plan_slot[i] = plan[i].slot;
  }
  hipError_t e = ll::launch_kv_write(wp, c->head_dim, c->kv_dtype, s);
  if (e != hipSuccess) return hip_fail(e, what);
  return LL_OK;
}

// Arguments and parameters of one attention call (shared by the two attention entry
// points; the work area is filled in by the caller).
ll_status attn_params(ll_cache* c, int layer, const void* Q, const void* K_chunk, const void* V_chunk, int n_frames,
                      void* out, ll::AttnParams* pp) {
  LL_TRY(check_layer(c, layer));
  LL_TRY(check_tensor(Q, "Q"));
  LL_TRY(check_tensor(K_chunk, "K_chunk"));
  LL_TRY(check_tensor(V_chunk, "V_chunk"));
  LL_TRY(check_tensor(out, "out"));
  LL_TRY(check_frames(c, n_frames));
  LL_TRY(check_device(c));
  const int64_t f0 = c->f0[size_t(layer)];
  const std::vector<ll::SlotRun> runs = ll::cache_runs(f0, c->layout(), c->fs[size_t(layer)]);
#ifdef LL_DEBUG
  for (const ll::SlotRun& r : runs)
    for (int sl = r.first; sl < r.first + r.count; ++sl)
      if (c->slot_frame[size_t(layer)][size_t(sl)] < 0)
        return fail(LL_ERR_STATE, "debug check: attention of layer %d would read empty slot %d", layer, sl);
#endif
  ll::AttnParams& p = *pp;
  p.Q = static_cast<const uint16_t*>(Q);
  p.Kc = static_cast<const uint16_t*>(K_chunk);
  p.Vc = static_cast<const uint16_t*>(V_chunk);
  p.out = static_cast<uint16_t*>(out);
  p.cK = c->k(layer);
  p.cV = c->v(layer);
  p.cKs = c->ks(layer);
  p.cVs = c->vs(layer);
  p.nq = int(int64_t(n_frames) * c->T);
  p.ncache = 0;
  p.nrun = int(runs.size());
  for (size_t k = 0; k < runs.size(); ++k) {
    p.run_row0[k] = int(int64_t(runs[k].first) * c->T);
    p.run_rows[k] = int(int64_t(runs[k].count) * c->T);
    p.ncache += p.run_rows[k];
  }
  p.H = c->heads;
  p.c = float(1.4426950408889634 / std::sqrt(double(c->head_dim)));
  p.n_cu = c->n_cu;
  return LL_OK;
}

// ---- the allocation-free attention entry point's scratch ------------------------
// Partial results and arrival counters of the split key walk, for callers that cannot
// allocate: 2 x 256 partial slots of 256 rows x (128 + 2) floats (head_dim 128 on a
// 256-CU device; head_dim 64 needs half) and 1024 counters.  One copy per GPU, held
// until the process ends.  Host code never names the array itself in a launch or copy:
// it uses the per-device address from hipGetSymbolAddress.
constexpr int64_t kScratchPartialFloats = int64_t(2) * 256 * (256 * (128 + 2));
constexpr int kScratchCounters = 1024;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) float scratch[kScratchPartialFloats + kScratchCounters];

namespace {

struct ScratchDevice {
  float* ptr = nullptr;   // device address of `scratch` on this GPU
  bool cleared = false;   // counters zeroed (enqueued)
};
ScratchDevice g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

__global__ void zero_ints_kernel(int* p, int n) {
  const int i = int(blockIdx.x) * int(blockDim.x) + int(threadIdx.x);
  if (i < n) p[i] = 0;
}

// Set-up of the scratch on `dev` (the current device), once per device: look up the
// array's address on this GPU (which also makes the runtime load the code object that
// holds it) and enqueue the zeroing of its counters on stream s (a fill kernel, so that
// a later call may be captured into a graph).  Done by ll_cache_create, which waits for
// its stream; the entry point repeats it only for a device no cache was created on.
ll_status scratch_on_device(int dev, hipStream_t s, float** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(LL_ERR_INVALID, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchDevice& d = g_scratch[dev];
  if (!d.ptr) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    d.ptr = static_cast<float*>(ptr);
  }
  if (!d.cleared) {
    int* cnt = reinterpret_cast<int*>(d.ptr + kScratchPartialFloats);
    hipLaunchKernelGGL(zero_ints_kernel, dim3((kScratchCounters + 255) / 256), dim3(256), 0, s, cnt,
                       kScratchCounters);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "clearing the scratch counters");
    d.cleared = true;
  }
  if (out) *out = d.ptr;
  return LL_OK;
}

#ifdef LL_DEBUG
// Debug library: every slot starts poisoned (bf16 quiet NaN; for int8 / fp8 caches NaN
// scales, so every dequantised value is NaN) and the slots a recache rewrites are
// poisoned again just before, so an attention that reads a slot nobody wrote, or a
// rewrite that misses a slot, shows up as NaN in the outputs or the slot bytes.  Internal
// invariants of the slot arithmetic abort (slots.h, LL_CHECK): a library bug, not a
// caller error.
__global__ void poison_kernel(uint32_t* p, int64_t n_words, uint32_t pattern) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n_words; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = pattern;
}

// Scale words of a poisoned slot: fp32 NaN (int8 / fp8), or E8M0 NaN bytes (MX formats).
uint32_t scale_poison(int kv_dtype) {
  return kv_dtype == LL_KV_MXFP4 || kv_dtype == LL_KV_MXFP8 ? 0xFFFFFFFFu : 0x7FC00000u;
}

hipError_t poison(void* p, size_t bytes, uint32_t pattern, hipStream_t s) {
  const int64_t words = int64_t(bytes / 4);
  if (words == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((words + 255) / 256, 4096);
  hipLaunchKernelGGL(poison_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, static_cast<uint32_t*>(p), words, pattern);
  return hipGetLastError();
}

// Poison the slots of `layer` that the plan is about to write.
ll_status poison_planned(ll_cache* c, int layer, const std::vector<ll::WriteEntry>& plan, hipStream_t s) {
  const size_t slot_vals = size_t(c->rows_per_frame) * size_t(c->head_dim);
  for (const ll::WriteEntry& w : plan) {
    hipError_t e;
    if (c->kv_dtype == LL_KV_BF16) {
      e = poison(static_cast<char*>(c->k(layer)) + size_t(w.slot) * slot_vals * 2, slot_vals * 2, 0x7FC07FC0u, s);
      if (e == hipSuccess)
        e = poison(static_cast<char*>(c->v(layer)) + size_t(w.slot) * slot_vals * 2, slot_vals * 2, 0x7FC07FC0u, s);
    } else {
      const uint32_t pat = scale_poison(c->kv_dtype);
      e = poison(c->ks(layer) + size_t(w.slot) * size_t(c->rows_per_frame), size_t(c->rows_per_frame) * 4, pat, s);
      if (e == hipSuccess)
        e = poison(c->vs(layer) + size_t(w.slot) * size_t(c->rows_per_frame), size_t(c->rows_per_frame) * 4, pat, s);
    }
    if (e != hipSuccess) return hip_fail(e, "poisoning slots before a rewrite");
  }
  return LL_OK;
}
#endif

}  // namespace

extern "C" {

const char* ll_last_error(void) { return g_err.c_str(); }

ll_status ll_cache_create(int layers, int heads, int head_dim, int tokens_per_frame, int sink_frames,
                          int window_frames, int kv_dtype, ll_cache** out) {
  return ll_cache_create_shots(layers, heads, head_dim, tokens_per_frame, sink_frames, 0, window_frames, kv_dtype,
                               out);
}

ll_status ll_cache_create_shots(int layers, int heads, int head_dim, int tokens_per_frame, int sink_frames,
                                int shot_sink_frames, int window_frames, int kv_dtype, ll_cache** out) {
  if (!out) return fail(LL_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (layers < 1) return fail(LL_ERR_INVALID, "layers must be >= 1");
  if (heads < 1 || heads > 4096) return fail(LL_ERR_INVALID, "heads must be in [1, 4096] (got %d)", heads);
  if (head_dim != 64 && head_dim != 128) return fail(LL_ERR_INVALID, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (tokens_per_frame < 1) return fail(LL_ERR_INVALID, "tokens_per_frame must be >= 1");
  if (sink_frames < 0 || window_frames < 0 || shot_sink_frames < 0)
    return fail(LL_ERR_INVALID, "sink_frames, shot_sink_frames and window_frames must be >= 0");
  const int64_t slots = int64_t(sink_frames) + shot_sink_frames + window_frames;
  if (slots < 1 || slots > LL_MAX_SLOTS)
    return fail(LL_ERR_INVALID, "sink_frames + shot_sink_frames + window_frames must be in [1, %d]", LL_MAX_SLOTS);
  if (kv_dtype != LL_KV_BF16 && kv_dtype != LL_KV_INT8 && kv_dtype != LL_KV_FP8 && kv_dtype != LL_KV_MXFP4 &&
      kv_dtype != LL_KV_MXFP8)
    return fail(LL_ERR_INVALID, "unknown kv_dtype %d", kv_dtype);
  const int64_t rows = int64_t(tokens_per_frame) * heads;
  if (slots * tokens_per_frame > kMaxRows || rows > kMaxRows) return fail(LL_ERR_INVALID, "cache too large");
  const bool quantised = kv_dtype != LL_KV_BF16;
  // code bytes per (token, head) row: 2 per value (bf16), 1 (int8, fp8, MXFP8) or 1/2 (MXFP4)
  const int64_t row_bytes = kv_dtype == LL_KV_BF16 ? 2 * head_dim : kv_dtype == LL_KV_MXFP4 ? head_dim / 2 : head_dim;
  auto round256 = [](int64_t b) { return (b + 255) / 256 * 256; };
  const int64_t kv_bytes = round256(slots * rows * row_bytes);
  const int64_t sc_bytes = quantised ? round256(slots * rows * 4) : 0;
  const double cache_total = double(layers) * 2.0 * double(kv_bytes + sc_bytes);
  if (cache_total > double(int64_t(1) << 46)) return fail(LL_ERR_INVALID, "cache too large (%.3g bytes)", cache_total);

  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int n_cu = 0;
  e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  // Work-split buffers of the attention launches, per layer: partial-result slots (fewer
  // than two per CU, split_plan.h) and one arrival counter per block (blocks < CUs when
  // the walk is split), after the cache arrays.
  const int64_t ws_slots = ll::split_slots(n_cu);
  const int64_t ws_layer_bytes = round256(ll::split_slot_floats(head_dim, ll::kAttnRows) * ws_slots * 4);
  const int64_t cnt_layer_bytes = round256(int64_t(n_cu) * 4);
  const int64_t ws_offset = int64_t(cache_total);
  const int64_t cnt_offset = ws_offset + int64_t(layers) * ws_layer_bytes;
  const double total = double(cnt_offset) + double(layers) * double(cnt_layer_bytes);
  void* mem = nullptr;
  e = hipMalloc(&mem, size_t(total));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(LL_ERR_OOM, "hipMalloc of %.3g bytes failed: %s", total, hipGetErrorString(e));
  }
  // Zero the counters on a private stream and wait for that stream only.
  // The same stream sets up the allocation-free attention's scratch on this device.
  hipStream_t zs = nullptr;
  e = hipStreamCreateWithFlags(&zs, hipStreamNonBlocking);
  if (e == hipSuccess) {
    e = hipMemsetAsync(static_cast<char*>(mem) + cnt_offset, 0, size_t(layers) * size_t(cnt_layer_bytes), zs);
#ifdef LL_DEBUG
    if (e == hipSuccess) {   // every slot poisoned: bf16 NaN codes, or NaN scales
      if (!quantised) e = poison(mem, size_t(layers) * 2 * size_t(kv_bytes), 0x7FC07FC0u, zs);
      else e = poison(static_cast<char*>(mem) + size_t(layers) * 2 * size_t(kv_bytes), size_t(layers) * 2 * size_t(sc_bytes),
                      scale_poison(kv_dtype), zs);
    }
#endif
    if (e == hipSuccess) {
      const ll_status st = scratch_on_device(dev, zs, nullptr);
      if (st != LL_OK) {
        (void)hipStreamSynchronize(zs);
        (void)hipStreamDestroy(zs);
        (void)hipFree(mem);
        return st;
      }
    }
    const hipError_t e2 = hipStreamSynchronize(zs);
    if (e == hipSuccess) e = e2;
    const hipError_t e3 = hipStreamDestroy(zs);
    if (e == hipSuccess) e = e3;
  }
  if (e != hipSuccess) {
    (void)hipFree(mem);
    return hip_fail(e, "clearing the work-split counters");
  }
  ll_cache* c = new ll_cache;
  c->layers = layers;
  c->heads = heads;
  c->head_dim = head_dim;
  c->T = tokens_per_frame;
  c->S = sink_frames;
  c->Ss = shot_sink_frames;
  c->W = window_frames;
  c->kv_dtype = kv_dtype;
  c->device = dev;
  c->rows_per_frame = rows;
  c->kv_bytes = size_t(kv_bytes);
  c->sc_bytes = size_t(sc_bytes);
  c->n_cu = n_cu;
  c->ws_offset = size_t(ws_offset);
  c->ws_layer_bytes = size_t(ws_layer_bytes);
  c->ws_slots = ws_slots;
  c->cnt_offset = size_t(cnt_offset);
  c->cnt_layer_bytes = size_t(cnt_layer_bytes);
  c->mem = mem;
  c->f0.assign(size_t(layers), 0);
  c->fs.assign(size_t(layers), 0);
  c->slot_frame.assign(size_t(layers), std::vector<int64_t>(size_t(slots), -1));
  *out = c;
  return ok();
}

void ll_cache_destroy(ll_cache* c) {
  if (!c) return;
  if (c->mem) (void)hipFree(c->mem);
  delete c;
}

ll_status ll_cache_append(ll_cache* c, int layer, const void* K, const void* V, int n_frames, void* stream) {
  LL_TRY(check_layer(c, layer));
  LL_TRY(check_tensor(K, "K"));
  LL_TRY(check_tensor(V, "V"));
  LL_TRY(check_frames(c, n_frames));
  LL_TRY(check_device(c));
  const int64_t f0 = c->f0[size_t(layer)];
  const std::vector<ll::WriteEntry> plan = ll::append_plan(f0, n_frames, c->layout(), c->fs[size_t(layer)]);
  LL_TRY(write_frames(c, layer, K, V, plan, static_cast<hipStream_t>(stream), "append launch"));
  for (const ll::WriteEntry& w : plan) c->slot_frame[size_t(layer)][size_t(w.slot)] = w.frame;
  c->f0[size_t(layer)] = f0 + n_frames;
  return ok();
}

ll_status ll_attn_sink_window(ll_cache* c, int layer, const void* Q, const void* K_chunk, const void* V_chunk,
                              int n_frames, void* out, void* stream) {
  ll::AttnParams p{};
  LL_TRY(attn_params(c, layer, Q, K_chunk, V_chunk, n_frames, out, &p));
  p.ws = c->ws(layer);
  p.ws_slots = c->ws_slots;
  p.cnt = c->cnt(layer);
  hipError_t e = ll::launch_attention(p, c->head_dim, c->kv_dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return ok();
}

ll_status ll_attn_sink_window_noalloc(ll_cache* c, int layer, const void* Q, const void* K_chunk,
                                      const void* V_chunk, int n_frames, void* out, void* stream) {
  ll::AttnParams p{};
  LL_TRY(attn_params(c, layer, Q, K_chunk, V_chunk, n_frames, out, &p));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (ll::attention_would_split(p, c->head_dim)) {
    const int64_t slot_floats = ll::split_slot_floats(c->head_dim, ll::kAttnRows);
    const int64_t need_floats = ll::split_slots(c->n_cu) * slot_floats;
    if (need_floats > kScratchPartialFloats || c->n_cu > kScratchCounters)
      return fail(LL_ERR_INVALID,
                  "attention without allocation: the split key walk needs %lld bytes of partials and %d "
                  "counters, the library's static scratch holds %lld bytes and %d",
                  (long long)(need_floats * 4), c->n_cu, (long long)(kScratchPartialFloats * 4), kScratchCounters);
    float* base = nullptr;
    LL_TRY(scratch_on_device(c->device, s, &base));
    p.ws = base;
    p.ws_slots = kScratchPartialFloats / slot_floats;
    p.cnt = reinterpret_cast<int*>(base + kScratchPartialFloats);
  } else {
    p.ws = nullptr;   // no split: the launch needs no scratch
    p.ws_slots = 0;
    p.cnt = nullptr;
  }
  hipError_t e = ll::launch_attention(p, c->head_dim, c->kv_dtype, s);
  if (e != hipSuccess) return hip_fail(e, "attention launch (no allocation)");
  return ok();
}

ll_status ll_cache_recache(ll_cache* c, int layer, const void* K_all, const void* V_all, int n_frames,
                           void* stream) {
  LL_TRY(check_layer(c, layer));
  LL_TRY(check_tensor(K_all, "K_all"));
  LL_TRY(check_tensor(V_all, "V_all"));
  const int64_t f0 = c->f0[size_t(layer)];
  const int64_t fs = c->fs[size_t(layer)];
  const int64_t need = ll::cached_frames(f0, c->layout(), fs);
  if (need == 0) return fail(LL_ERR_STATE, "recache: layer %d holds no frames", layer);
  if (n_frames != need)
    return fail(LL_ERR_STATE, "recache: n_frames must equal the retained frames (min(f0, S+W) plus shot sink) = %lld (got %d)",
                (long long)need, n_frames);
  LL_TRY(check_frames(c, n_frames));
  LL_TRY(check_device(c));
  const std::vector<ll::WriteEntry> plan = ll::recache_plan(f0, c->layout(), fs);
#ifdef LL_DEBUG
  LL_TRY(poison_planned(c, layer, plan, static_cast<hipStream_t>(stream)));
#endif
  LL_TRY(write_frames(c, layer, K_all, V_all, plan, static_cast<hipStream_t>(stream), "recache launch"));
  return ok();
}

ll_status ll_cache_recache_window(ll_cache* c, int layer, const void* K_win, const void* V_win, int n_frames,
                                  void* stream) {
  LL_TRY(check_layer(c, layer));
  LL_TRY(check_tensor(K_win, "K_win"));
  LL_TRY(check_tensor(V_win, "V_win"));
  const int64_t f0 = c->f0[size_t(layer)];
  const int64_t need = std::min<int64_t>(std::max<int64_t>(f0 - c->S, 0), c->W);
  if (need == 0) return fail(LL_ERR_STATE, "recache_window: layer %d holds no window frames", layer);
  if (n_frames != need)
    return fail(LL_ERR_STATE, "recache_window: n_frames must equal min(max(f0-S,0), W) = %lld (got %d)",
                (long long)need, n_frames);
  LL_TRY(check_frames(c, n_frames));
  LL_TRY(check_device(c));
  const std::vector<ll::WriteEntry> plan = ll::recache_window_plan(f0, c->layout(), c->fs[size_t(layer)]);
#ifdef LL_DEBUG
  LL_TRY(poison_planned(c, layer, plan, static_cast<hipStream_t>(stream)));
#endif
  LL_TRY(write_frames(c, layer, K_win, V_win, plan, static_cast<hipStream_t>(stream), "recache_window launch"));
  return ok();
}

ll_status ll_kv_project(const void* h, const void* W_K, const void* W_V, int n_tokens, int d_in, int d_out,
                        void* K_all, void* V_all, void* stream) {
  LL_TRY(check_tensor(h, "h"));
  LL_TRY(check_tensor(W_K, "W_K"));
  LL_TRY(check_tensor(W_V, "W_V"));
  LL_TRY(check_tensor(K_all, "K_all"));
  LL_TRY(check_tensor(V_all, "V_all"));
  if (n_tokens < 1 || n_tokens > kMaxRows) return fail(LL_ERR_INVALID, "n_tokens out of range");
  if (d_in < 64 || d_in % 64 != 0 || d_in > 65536) return fail(LL_ERR_INVALID, "d_in must be a multiple of 64");
  if (d_out < 128 || d_out % 128 != 0 || d_out > 65536)
    return fail(LL_ERR_INVALID, "d_out must be a multiple of 128");
  ll::ProjParams p{};
  p.h = static_cast<const uint16_t*>(h);
  p.WK = static_cast<const uint16_t*>(W_K);
  p.WV = static_cast<const uint16_t*>(W_V);
  p.outK = static_cast<uint16_t*>(K_all);
  p.outV = static_cast<uint16_t*>(V_all);
  p.M = n_tokens;
  p.K = d_in;
  p.N = d_out;
  hipError_t e = ll::launch_kv_project(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  return ok();
}

ll_status ll_cache_recache_from_hidden(ll_cache* c, int layer, const void* h, const void* W_K, const void* W_V,
                                       int n_frames, int d_in, void* stream) {
  LL_TRY(check_layer(c, layer));
  LL_TRY(check_tensor(h, "h"));
  LL_TRY(check_tensor(W_K, "W_K"));
  LL_TRY(check_tensor(W_V, "W_V"));
  const int64_t d_out = int64_t(c->heads) * c->head_dim;
  if (d_in < 64 || d_in % 64 != 0 || d_in > 65536) return fail(LL_ERR_INVALID, "d_in must be a multiple of 64");
  if (d_out % 128 != 0 || d_out > 65536)
    return fail(LL_ERR_INVALID, "heads*head_dim = %lld must be a multiple of 128", (long long)d_out);
  const int64_t f0 = c->f0[size_t(layer)];
  const int64_t fs = c->fs[size_t(layer)];
  const int64_t need = ll::cached_frames(f0, c->layout(), fs);
  if (need == 0) return fail(LL_ERR_STATE, "recache_from_hidden: layer %d holds no frames", layer);
  if (n_frames != need)
    return fail(LL_ERR_STATE, "recache_from_hidden: n_frames must equal the retained frames = %lld (got %d)",
                (long long)need, n_frames);
  LL_TRY(check_frames(c, n_frames));
  LL_TRY(check_device(c));
  const std::vector<ll::WriteEntry> plan = ll::recache_plan(f0, c->layout(), fs);
  ll::ProjToCacheParams p{};
  p.proj.h = static_cast<const uint16_t*>(h);
  p.proj.WK = static_cast<const uint16_t*>(W_K);
  p.proj.WV = static_cast<const uint16_t*>(W_V);
  p.proj.M = n_frames * c->T;
  p.proj.K = d_in;
  p.proj.N = int(d_out);
  p.T = c->T;
  p.H = c->heads;
  p.D = c->head_dim;
  p.kv_fmt = c->kv_dtype;
  p.slotK = c->k(layer);
  p.slotV = c->v(layer);
  p.scK = c->ks(layer);
  p.scV = c->vs(layer);
  p.n_plan = n_frames;
  for (int i = 0; i < n_frames; ++i) p.plan_slot[i] = p.plan_slot2[i] = -1;
  for (const ll::WriteEntry& e : plan) {
    int& first = p.plan_slot[size_t(e.src)];
    if (first < 0) first = e.slot;
    else p.plan_slot2[size_t(e.src)] = e.slot;
  }
#ifdef LL_DEBUG
  LL_TRY(poison_planned(c, layer, plan, static_cast<hipStream_t>(stream)));
#endif
  hipError_t e = ll::launch_kv_project_to_cache(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "recache_from_hidden launch");
  return ok();
}

ll_status ll_cache_begin_shot(ll_cache* c, int layer) {
  LL_TRY(check_layer(c, layer));
  const size_t l = size_t(layer);
  c->fs[l] = c->f0[l];
  for (int s = c->S; s < c->S + c->Ss; ++s) c->slot_frame[l][size_t(s)] = -1;
  return ok();
}

ll_status ll_cache_shot_start(const ll_cache* c, int layer, int64_t* fs) {
  LL_TRY(check_layer(c, layer));
  if (!fs) return fail(LL_ERR_INVALID, "fs is NULL");
  *fs = c->fs[size_t(layer)];
  return ok();
}

ll_status ll_cache_frames_seen(const ll_cache* c, int layer, int64_t* f0) {
  LL_TRY(check_layer(c, layer));
  if (!f0) return fail(LL_ERR_INVALID, "f0 is NULL");
  *f0 = c->f0[size_t(layer)];
  return ok();
}

ll_status ll_cache_slot_frames(const ll_cache* c, int layer, int64_t* frame_of_slot) {
  LL_TRY(check_layer(c, layer));
  if (!frame_of_slot) return fail(LL_ERR_INVALID, "frame_of_slot is NULL");
  const std::vector<int64_t>& sf = c->slot_frame[size_t(layer)];
  std::memcpy(frame_of_slot, sf.data(), sf.size() * sizeof(int64_t));
  return ok();
}

ll_status ll_cache_slot_view(const ll_cache* c, int layer, void** K, void** V, void** K_scale, void** V_scale) {
  LL_TRY(check_layer(c, layer));
  if (K) *K = c->k(layer);
  if (V) *V = c->v(layer);
  if (K_scale) *K_scale = c->ks(layer);
  if (V_scale) *V_scale = c->vs(layer);
  return ok();
}

}  // extern "C"
