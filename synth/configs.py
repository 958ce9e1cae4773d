"""The five synthetic workloads (shapes, lengths, seeds).  No arithmetic here.

Sizes follow the pages where they give them: a chunk of 3 latent frames,
3 sink frames and windows of 9-21 latent frames (techwalker.com article on
LONGLIVE, §四 and §六); 832x480 video from the Wan2.1-T2V-1.3B base model
(same article, §六) taken as 30x52 = 1560 tokens per latent frame; videos up
to 240 s.  Head count, head size and layer count are those of a 1.3B DiT.
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    heads: int
    head_dim: int
    tokens_per_frame: int
    chunk_frames: int
    sink: int
    window: int
    chunks: int          # chunks generated in the rollout
    passes: int          # denoise passes per chunk (cache read-only)
    sigma: float         # std of the Gaussian inputs
    seed: int
    kv_int8: bool = False
    recache_every: int = 0   # prompt switch before chunks k*recache_every (k >= 1)
    prefill_chunks: int = 0  # chunks appended before the measured step
    hidden: int = 0          # recache projection width (heads * head_dim)

    @property
    def nq(self) -> int:
        return self.chunk_frames * self.tokens_per_frame

    @property
    def row_elems(self) -> int:
        return self.heads * self.head_dim


# 1. tiny streaming toy: fp32 N(0,1) rounded to bf16, scale 1/sqrt(64)
TOY = Workload("toy_h2_d64_t16_s3_w6", layers=1, heads=2, head_dim=64, tokens_per_frame=16,
               chunk_frames=3, sink=3, window=6, chunks=12, passes=2, sigma=1.0, seed=0)

# 2. single-layer steady-state step at 1.3B-DiT shape, cache already full
STEADY = Workload("steady_h12_d128_t1560_s3_w12", layers=1, heads=12, head_dim=128,
                  tokens_per_frame=1560, chunk_frames=3, sink=3, window=12, chunks=1,
                  passes=4, sigma=0.5, seed=1, prefill_chunks=10)

# 3. 30-layer rollout, 80 chunks (240 latent frames)
ROLLOUT = Workload("rollout_l30_80chunks_s3_w12", layers=30, heads=12, head_dim=128,
                   tokens_per_frame=1560, chunk_frames=3, sink=3, window=12, chunks=80,
                   passes=4, sigma=0.5, seed=2)

# 4. KV-recache at a prompt switch, 30 layers, hidden 1536 = 12 x 128
RECACHE = Workload("recache_l30_h1536_23400tok", layers=30, heads=12, head_dim=128,
                   tokens_per_frame=1560, chunk_frames=3, sink=3, window=12, chunks=1,
                   passes=1, sigma=1.0, seed=3, prefill_chunks=6, hidden=1536)

# 5. long-horizon int8 KV cache: 400 chunks (1200 frames), window 21, recache every 50
LONG_INT8 = Workload("long_int8_l30_400chunks_s3_w21", layers=30, heads=12, head_dim=128,
                     tokens_per_frame=1560, chunk_frames=3, sink=3, window=21, chunks=400,
                     passes=4, sigma=0.5, seed=4, kv_int8=True, recache_every=50)

ALL = [TOY, STEADY, ROLLOUT, RECACHE, LONG_INT8]
