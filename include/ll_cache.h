/*
 * ll_cache.h -- C ABI of the MI355X (gfx950) streaming sink+window KV-cache library.
 *
 * What the library computes (sources are cited per entry point):
 *   [LL-dpshk]  "LongLive: Real-time Interactive Long Video Generation" explainer,
 *               dpshk.com: §二 frame-level autoregressive generation with a KV cache,
 *               §三 KV-recache, §五 Short Window Attention, §六 Frame Sink.
 *   [LL-tw]     "英伟达突破视频生成瓶颈：LONGLIVE让普通电脑也能实时生成超长视频",
 *               techwalker.com: §四 short window + frame sink, §六 chunk of 3 latent
 *               frames, window of 9, first 3 frames as sink, recache scope.
 *   [LL2-wmrh]  "LongLive-2.0: An NVFP4 Parallel Infrastructure for Long Video
 *               Generation" explainer, wmrh.cn: §6 autoregressive mask, §15.2-§15.3
 *               low-precision KV cache and its dequantisation.
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers on the device that was current when the
 *     cache was created, 16-byte aligned, and owned by the caller.  They must stay
 *     valid until the enqueued work has run (the library keeps no reference).
 *   - Token tensors are row-major [tokens][heads][head_dim] bf16 (IEEE binary32
 *     upper halves), contiguous.  "A frame" is tokens_per_frame consecutive tokens.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  All
 *     device work of a call is enqueued on it; nothing blocks the host.
 *   - Host-side bookkeeping (frames seen f0, which frame each slot holds) is
 *     kept per layer and updated when a call is enqueued.  Calls on ONE layer must
 *     be issued in stream order (one stream, or streams the caller orders with
 *     events) and from one host thread at a time.  Different layers may be used
 *     from different streams and host threads at the same time: each layer has
 *     its own slots, bookkeeping and attention work area.
 *   - Every function returns a status; no exception or abort crosses the ABI.
 *     Arguments are validated BEFORE any HIP call: LL_ERR_INVALID for bad
 *     arguments, LL_ERR_STATE for calls the cache's state forbids, LL_ERR_OOM when
 *     device memory cannot be allocated, LL_ERR_HIP when the HIP runtime reports
 *     an error (no device, launch failure).  ll_last_error() gives text for the
 *     last failure on the calling thread.  Device faults of enqueued work are
 *     reported by the HIP runtime at a later synchronisation.
 *
 * Debug build (libllcache_debug.so: same kernels and interface, host side compiled
 * with LL_DEBUG), for finding slot bookkeeping mistakes:
 *   - every slot of a new cache is filled with NaN (bf16 caches: NaN values;
 *     int8 / fp8 caches: NaN per-row scales), and a recache, window-only recache or
 *     fused recache fills the slots it rewrites with NaN before writing them, so a slot read
 *     before a frame reached it turns the output into NaN;
 *   - an attention call whose visible slots include one that holds no frame fails
 *     with LL_ERR_STATE before launching anything;
 *   - the slot planners check their internal invariants and abort the process on a
 *     violation (the one case where an abort leaves the library).
 *   Results of calls that pass these checks are bit-identical to the normal build.
 */
#ifndef LL_CACHE_H
#define LL_CACHE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ll_cache ll_cache; /* opaque; owns its slot memory */

typedef enum { LL_KV_BF16 = 0, LL_KV_INT8 = 1, LL_KV_FP8 = 2, LL_KV_MXFP4 = 3, LL_KV_MXFP8 = 4 } ll_kv_dtype;

typedef enum {
  LL_OK = 0,
  LL_ERR_INVALID = 1,
  LL_ERR_OOM = 2,
  LL_ERR_STATE = 3,
  LL_ERR_HIP = 4
} ll_status;

/* Largest S + W the library accepts (slots per layer). */
#define LL_MAX_SLOTS 128

/*
 * ll_cache_create -- allocate the per-layer KV cache of the sink + window policy.
 * [LL-dpshk §六]: the cache holds the sink frames' K/V permanently plus the K/V of
 * the most recent window; [LL-dpshk §五]: older K/V are evicted, so memory stays
 * bounded; [LL-tw §六]: sink = first 3 latent frames, window = 9 latent frames.
 *
 *   layers            >= 1
 *   heads             1 .. 4096 (tile copies address a 64-row tile with 32-bit
 *                     byte offsets)
 *   head_dim          64 or 128
 *   tokens_per_frame  >= 1 (T)
 *   sink_frames       S >= 0
 *   window_frames     W >= 0, 1 <= S + W <= LL_MAX_SLOTS
 *   kv_dtype          LL_KV_BF16: cached K/V stored as bf16 (bit copies of the input)
 *                     LL_KV_INT8: cached K/V stored as int8 codes with one fp32 scale
 *                     per (token, head) row:  scale = absmax/127,
 *                     q = clamp(rint((x*127)/absmax), -127, 127), 0 for an all-zero row
 *                     LL_KV_FP8: OCP E4M3 codes (sign, 4 exponent bits with bias 7,
 *                     3 mantissa bits; largest finite value 448) with one fp32 scale
 *                     per row: scale = absmax/448, q = E4M3(clamp((x*448)/absmax,
 *                     -448, 448)) rounded to nearest, ties to even, all-zero codes for
 *                     an all-zero row (the clamp acts only where x*448 overflows).
 *                     LL_KV_MXFP4: OCP MX 4-bit codes (E2M1: sign, 2 exponent bits
 *                     with bias 1, 1 mantissa bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6)
 *                     with one power-of-two scale 2^e per block of 32 consecutive
 *                     values of a row: e = max(floor(log2 absmax) - 2, -125) (-125
 *                     for an all-zero block), q = E2M1(min(|x| / 2^e, 6)) nearest,
 *                     ties to the even code, with the sign of x (so -0 and negative
 *                     values that round to zero give code 8).  Dequantised values
 *                     value(q) * 2^e are exact bf16 values.
 *                     LL_KV_MXFP8: OCP MX 8-bit codes (E4M3 as above) with one
 *                     power-of-two scale 2^e per block of 32 values of a row:
 *                     e = max(floor(log2 absmax) - 8, -117) (-117 for an all-zero
 *                     block), q = E4M3(clamp(x / 2^e, -448, 448)) nearest, ties to
 *                     even, sign kept; value(q) * 2^e is an exact bf16 value.
 *                     [LL2-wmrh §15.2-§15.3]: the history cache kept in low precision
 *                     (4-bit on the page's hardware) and dequantised where it is used.
 *                     Every division above is one IEEE binary32 division.
 *   out               receives the handle
 *
 * Device memory, one allocation made here (no later call allocates):
 * layers * 2 * (S+W) * T * heads * head_dim * (2, 1 or 1/2) bytes of slots, plus
 * layers * 2 * (S+W) * T * heads * 4 bytes of scales for the low-bit caches, plus per layer
 * an attention work area for split key walks (2 * CUs partial results of 256 rows *
 * (head_dim + 2) * 4 bytes and CUs arrival counters: about 68 MB for head_dim 128 on
 * 256 CUs).  Slot contents start undefined; no slot is visible until written.  The
 * first cache on a device also sets up the static scratch of
 * ll_attn_sink_window_noalloc there (LL_NOALLOC_SCRATCH_BYTES, held by the loaded
 * library until the process ends).  The call waits only for its own zeroing work (a
 * private stream).
 * Errors: LL_ERR_INVALID, LL_ERR_OOM, LL_ERR_HIP.
 */
ll_status ll_cache_create(int layers, int heads, int head_dim, int tokens_per_frame,
                          int sink_frames, int window_frames, int kv_dtype,
                          ll_cache **out);

/*
 * ll_cache_create_shots -- a cache with a shot sink as well as the global sink.
 * [LL2-wmrh §16]: multi-shot generation keeps a global-level sink that every shot
 * attends to and a shot-level sink holding the current shot's own context.  Reading
 * adopted (the page names the two levels only): the global sink is the first
 * sink_frames frames of the video, the shot sink the first shot_sink_frames frames of
 * the current shot (ll_cache_begin_shot), and a chunk starting at f0 in the shot that
 * started at fs sees
 *     {f < min(S, f0)} U {fs <= f < min(fs + Ss, f0)} U {max(0, f0-W) <= f < f0}
 * plus its own chunk.  Slots: [0, S) global sink, [S, S+Ss) shot sink, [S+Ss, S+Ss+W)
 * window ring; a shot-sink frame is stored in its shot slot and its ring slot.
 * ll_cache_create is this function with shot_sink_frames = 0.
 *   shot_sink_frames  Ss >= 0, 1 <= S + Ss + W <= LL_MAX_SLOTS
 * Other arguments, memory and errors as ll_cache_create.
 */
ll_status ll_cache_create_shots(int layers, int heads, int head_dim, int tokens_per_frame,
                                int sink_frames, int shot_sink_frames, int window_frames,
                                int kv_dtype, ll_cache **out);

/*
 * ll_cache_begin_shot -- the next frame appended to `layer` starts a new shot: fs = f0,
 * and the previous shot's sink is no longer visible (its shot slots are marked empty;
 * frames of it still inside the window stay visible through the window).  Host
 * bookkeeping only, no device work.  Errors: LL_ERR_INVALID.
 */
ll_status ll_cache_begin_shot(ll_cache *c, int layer);

/* First frame of the current shot of `layer` (0 until ll_cache_begin_shot). */
ll_status ll_cache_shot_start(const ll_cache *c, int layer, int64_t *fs);

/* Free the cache's device memory and the handle (NULL is accepted).  The caller
 * must make sure no enqueued work still uses it. */
void ll_cache_destroy(ll_cache *c);

/*
 * ll_cache_append -- the append/evict step after a chunk is finished.
 * [LL-dpshk §二]: after a chunk is generated its K/V enter the cache and are reused;
 * [LL-dpshk §五]: K/V older than the window are evicted; [LL-dpshk §六]: sink frames
 * stay.  Frames f0 .. f0+n_frames-1 of `layer` are written (frame f goes to slot f
 * if f < S, else to window slot S + (f-S) mod W, else it is dropped when W = 0; a
 * later frame of the same call replaces an earlier one), then f0 += n_frames.
 *   K, V       [n_frames*T][heads][head_dim] bf16 (the finished chunk's keys/values)
 *   n_frames   >= 1
 * Errors: LL_ERR_INVALID (layer, pointers, n_frames), LL_ERR_HIP.
 */
ll_status ll_cache_append(ll_cache *c, int layer, const void *K, const void *V,
                          int n_frames, void *stream);

/*
 * ll_attn_sink_window -- attention of one chunk over sink + window + own chunk.
 * [LL-dpshk §五, §六]; [LL-tw §四, §六]; [LL2-wmrh §6] (a chunk sees earlier chunks
 * and itself, never a later one).  For a chunk starting at frame f0 (the layer's
 * frames seen so far) each query token attends to every token of the frames
 *     {f < min(S, f0)} U {max(0, f0-W) <= f < f0} U {own chunk's frames}
 * with full visibility inside the own chunk:
 *     out = softmax((Q K^T) / sqrt(head_dim)) V   per head, over those keys.
 * The cache is read only (denoise passes of one chunk may call this repeatedly).
 * For the low-bit caches the cached keys/values are dequantised (value(q) * scale);
 * the own chunk is used as given.
 *   Q, K_chunk, V_chunk   [n_frames*T][heads][head_dim] bf16 (n_frames >= 1)
 *   out                   [n_frames*T][heads][head_dim] bf16, written completely
 * Arithmetic: bf16 MFMA products, fp32 accumulation and softmax statistics, bf16
 * probabilities for the P*V product, output rounded to bf16.
 * Input domain: finite inputs with scores q.k / sqrt(head_dim) below 2^14 in
 * magnitude (the exponent argument is formed as one fma of the fp32 score; beyond
 * about 2^23 the rounding of the score itself exceeds a unit and the output is not
 * meaningful).  Trained attention logits are many orders of magnitude smaller.
 * Errors: LL_ERR_INVALID, LL_ERR_HIP.
 */
ll_status ll_attn_sink_window(ll_cache *c, int layer, const void *Q, const void *K_chunk,
                              const void *V_chunk, int n_frames, void *out, void *stream);

/*
 * ll_attn_sink_window_noalloc -- ll_attn_sink_window for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, computation, results and errors as
 * ll_attn_sink_window; it allocates nothing and calls no allocating routine.  The
 * split key walk keeps its partial results and arrival counters in one static device
 * array per GPU owned by the library (LL_NOALLOC_SCRATCH_BYTES: the partials of
 * head_dim 128 on a 256-CU device plus 1024 counters, held until the process ends)
 * instead of the layer's work area.  ll_cache_create sets the array up on its device
 * (address looked up, counters zeroed before create returns); each merge leaves its
 * counter at zero again.  All calls of this function on one GPU share the
 * array, whatever cache or stream they use: calls that overlap in time on one GPU race
 * (wrong outputs), so issue them in one stream order.  A call whose split walk would
 * need more than the array holds (a device with more than 256 compute units) returns
 * LL_ERR_INVALID and launches nothing.
 * Errors: LL_ERR_INVALID, LL_ERR_HIP.
 */
#define LL_NOALLOC_SCRATCH_BYTES (2 * 256 * 256 * 130 * 4 + 1024 * 4)
ll_status ll_attn_sink_window_noalloc(ll_cache *c, int layer, const void *Q, const void *K_chunk,
                                      const void *V_chunk, int n_frames, void *out, void *stream);

/*
 * ll_cache_recache -- rewrite the retained cache at a prompt switch.
 * [LL-dpshk §三 items 3 and 5]: the recache context is the sink latents plus the
 * recent-window latents; the old KV cache is dropped and a new one computed from
 * them under the new prompt replaces it.  K_all/V_all hold the recomputed K/V of
 * the retained frames in logical order -- sink frames ascending, then window
 * frames oldest to newest -- and every retained slot is overwritten; f0 is
 * unchanged.
 *   K_all, V_all  [n_frames*T][heads][head_dim] bf16
 *   n_frames      must equal min(f0, S+W) (else LL_ERR_STATE; 0 frames cached is
 *                 LL_ERR_STATE too); with a shot sink, the number of retained
 *                 frames (the cached visible set), in ascending frame order; a
 *                 frame held in two slots gets its block in both
 * Errors: LL_ERR_INVALID, LL_ERR_STATE, LL_ERR_HIP.
 */
ll_status ll_cache_recache(ll_cache *c, int layer, const void *K_all, const void *V_all,
                           int n_frames, void *stream);

/*
 * ll_cache_recache_window -- recache variant that keeps the sink.
 * [LL-tw §六]: recomputation is limited to the most recent W frames and the sink
 * tokens stay unchanged.  K_win/V_win hold the window frames oldest to newest.
 *   n_frames  must equal min(max(f0 - S, 0), W) and be >= 1 (else LL_ERR_STATE)
 * Errors: LL_ERR_INVALID, LL_ERR_STATE, LL_ERR_HIP.
 */
ll_status ll_cache_recache_window(ll_cache *c, int layer, const void *K_win,
                                  const void *V_win, int n_frames, void *stream);

/*
 * ll_kv_project -- recompute keys and values from hidden states (the recache
 * projection).  [LL-dpshk §三 item 4]: K = W_K h', V = W_V h'.  Row form:
 *     K_all = h W_K^T,  V_all = h W_V^T
 *   h         [n_tokens][d_in] bf16
 *   W_K, W_V  [d_out][d_in] bf16 (the matrices of the column form K = W_K h')
 *   K_all, V_all  [n_tokens][d_out] bf16 (= [tokens][heads][head_dim] when
 *             d_out = heads*head_dim), rounded to nearest-even from fp32 sums
 *   n_tokens >= 1; d_in a multiple of 64; d_out a multiple of 128
 * Errors: LL_ERR_INVALID, LL_ERR_HIP.
 */
ll_status ll_kv_project(const void *h, const void *W_K, const void *W_V, int n_tokens,
                        int d_in, int d_out, void *K_all, void *V_all, void *stream);

/*
 * ll_cache_recache_from_hidden -- recache straight from hidden states: the
 * projection of ll_kv_project with its results written into the retained slots
 * (and, for the low-bit caches, quantised on the way) instead of into K_all/V_all.
 * [LL-dpshk §三 items 4 and 5]: the retained latents' K and V are recomputed from
 * the hidden state under the new prompt and replace the old cache.  The cache
 * bytes equal those of ll_kv_project followed by ll_cache_recache bit for bit;
 * the [n_frames*T][heads*head_dim] intermediate never reaches memory.
 *   h         [n_frames*T][d_in] bf16, retained frames in logical order (sink
 *             frames ascending, then window frames oldest to newest)
 *   W_K, W_V  [heads*head_dim][d_in] bf16
 *   n_frames  must equal min(f0, S+W) (else LL_ERR_STATE)
 *   d_in      a multiple of 64; heads*head_dim must be a multiple of 128
 * Every cache format (the low-bit ones quantised by the same rule as append).
 * Errors: LL_ERR_INVALID, LL_ERR_STATE, LL_ERR_HIP.
 */
ll_status ll_cache_recache_from_hidden(ll_cache *c, int layer, const void *h, const void *W_K,
                                       const void *W_V, int n_frames, int d_in, void *stream);

/* ---- introspection (host-side, no device work) --------------------------- */

/* Frames appended to `layer` so far (f0). */
ll_status ll_cache_frames_seen(const ll_cache *c, int layer, int64_t *f0);

/* For each of the S+Ss+W slots of `layer`, the frame it holds, or -1 if empty.
 * frame_of_slot must have room for S+Ss+W entries (host memory; S+W without a
 * shot sink). */
ll_status ll_cache_slot_frames(const ll_cache *c, int layer, int64_t *frame_of_slot);

/* Device pointers of `layer`'s slot arrays (read them after synchronising):
 *   K, V        [S+Ss+W][T][heads][head_dim], bf16, int8 or E4M3 bytes (kv_dtype:
 *               bf16, int8, fp8 or MXFP8);
 *               for LL_KV_MXFP4 [S+Ss+W][T][heads][head_dim/2] bytes, byte k holding
 *               value 2k in its low 4 bits and value 2k+1 in its high 4 bits
 *   K_scale, V_scale  [S+Ss+W][T][heads] fp32 for int8 / fp8 caches; for the MX caches
 *               [S+Ss+W][T][heads] uint32, byte b = e + 127 of the row's block b
 *               (bytes past head_dim/32 are 0); NULL for bf16
 * Any output pointer may be NULL. */
ll_status ll_cache_slot_view(const ll_cache *c, int layer, void **K, void **V,
                             void **K_scale, void **V_scale);

/* Text of the last failure on the calling thread ("" if none). */
const char *ll_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LL_CACHE_H */
