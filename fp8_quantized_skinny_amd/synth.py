"""Seeded synthetic inputs: float32 weights and fp16 activations.

This module only draws random numbers.  It holds none of the GEMM's
arithmetic: no decoding, quantization, contraction or argmax.  Both the CPU
oracle (through the tests) and the library consume what it draws.

Recipe, per workload and per M, independently:
  rng = numpy.random.default_rng(seed)          seed 0 unless stated
  W   = float32(rng.standard_normal((K, N)) * 0.02)   drawn first, row-major K x N
  x   = float16(rng.standard_normal((M, K)))          drawn second
Large W are drawn in row chunks; numpy fills a Generator's normal draws from
one sequential stream, so the chunked draw equals the one-shot draw (a CPU test
checks this).

The shapes are the decode shapes of a 27B-class hybrid model at one GPU's
full size (the author's post serves such a model with 4-way tensor
parallelism; its kernel table is measured at per-rank shapes that it does not
list).
"""

import numpy as np

# name: (format, M values, K, N)
WORKLOADS = {
    "tiny":    ("nvfp4", (1,), 256, 512),
    "up":      ("nvfp4", (1,), 5120, 17408),
    "gate_up": ("nvfp4", (8,), 5120, 34816),
    "down":    ("nvfp4", (8,), 17408, 5120),
    "qkv":     ("fp8", (1, 2, 4), 5120, 7168),
    "o_proj":  ("fp8", (1, 2, 4), 6144, 5120),
    "lm_head": ("nvfp4", (1, 8), 5120, 151936),
    # the gate+up shape as a SwiGLU pair: two 5120 x 17408 projections, output h[M, 17408]
    "gate_up_swiglu": ("swiglu", (8,), 5120, 17408),
    # the lm_head shape verifying one speculative round (k = 7 drafts, M = 8 rows)
    "lm_head_verify": ("nvfp4", (8,), 5120, 151936),
    # one rank's share under 4-way tensor parallelism (column shards; down and
    # o_proj shard K), at M = 1, 4 (k = 3 drafts) and 8 (k = 7 drafts)
    "up_tp4":      ("nvfp4", (1, 4, 8), 5120, 4352),
    "gate_up_tp4": ("nvfp4", (1, 4, 8), 5120, 8704),
    "down_tp4":    ("nvfp4", (1, 4, 8), 4352, 5120),
    "qkv_tp4":     ("fp8", (1, 2, 4), 5120, 1792),
    "o_proj_tp4":  ("fp8", (1, 2, 4), 1536, 5120),
    "lm_head_tp4": ("nvfp4", (1, 8), 5120, 37984),
    # the FP8 shapes with the codes reordered by fp8_pack
    "qkv_packed":    ("fp8p", (1, 2, 4), 5120, 7168),
    "o_proj_packed": ("fp8p", (1, 2, 4), 6144, 5120),
}


def draw_weights(rng, K, N, scale=0.02, chunk_rows=None):
    """float32 [K, N] = float32(standard_normal * scale), drawn in row chunks.

    The default chunk holds about 4 MB of float64 draws, which stays in cache."""
    if chunk_rows is None:
        chunk_rows = max(1, (1 << 19) // N)
    w = np.empty((K, N), np.float32)
    buf = np.empty((min(chunk_rows, K), N), np.float64)
    for r0 in range(0, K, chunk_rows):
        r1 = min(K, r0 + chunk_rows)
        b = buf[:r1 - r0]
        rng.standard_normal(out=b)
        np.multiply(b, scale, out=b)
        w[r0:r1] = b
    return w


def draw_activations(rng, M, K):
    """float16 [M, K] = float16(standard_normal)."""
    return rng.standard_normal((M, K)).astype(np.float16)


def draw(M, K, N, seed=0):
    """(W float32 [K, N], x float16 [M, K]) drawn in that order from one seeded stream."""
    rng = np.random.default_rng(seed)
    w = draw_weights(rng, K, N)
    x = draw_activations(rng, M, K)
    return w, x
