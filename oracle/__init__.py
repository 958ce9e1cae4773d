"""CPU oracle for streaming sink+window KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP library (no kernels, headers, helpers, tables or constants), and it never
models the ring buffer the GPU path uses when it decides what a query sees.

It is plain, slow and meant to be checked by eye against the pages:

* "LongLive: Real-time Interactive Long Video Generation" explainer
  (dpshk.com): §三 KV-recache (items 3 and 5), §五 Short Window Attention,
  §六 Frame Sink.
* "英伟达突破视频生成瓶颈：LONGLIVE让普通电脑也能实时生成超长视频"
  (techwalker.com): §四 short-window attention and frame sink, §六 technical
  details (chunk of 3 latent frames, local window of 9, first 3 frames as
  sink; recache scope).
* "LongLive-2.0: An NVFP4 Parallel Infrastructure for Long Video
  Generation" explainer (wmrh.cn): §6 (the autoregressive mask example),
  §15.2-§15.3 (KV-cache quantisation and its dequantisation).

Modules
-------
``bf16``       bit-level bfloat16 <-> float32 helpers (the oracle's own).
``visibility`` which frames a chunk may attend to (the visible set V(f0)).
``attention``  masked softmax attention with an explicit boolean mask
               (fp32 and fp64), a triple-loop brute force, and the per-chunk
               driver that builds the mask from ``visibility``.
``ring``       an independent model of the fixed-capacity slot store
               (append/evict, recache rewrite) used to check cache bytes.
``quant``      int8 and fp8 per-(token, head) absmax quantisation and dequantisation.
``mxfp4``      4-bit E2M1 codes with a power-of-two scale per block of 32 values.
``mxfp8``      E4M3 codes with a power-of-two scale per block of 32 values.
``gemm``       the recache projection K = W_K h (row form) rounded to bf16.

Every function states the passage it follows.  Parity status of each part
(pinned or not) is listed in the tests that pin it; no part is unpinned.
"""

from . import bf16, visibility, attention, ring, quant, mxfp4, mxfp8, gemm  # noqa: F401
