"""Model shapes and seeded synthetic inputs for the Slow-AR decode step.

Shapes follow the Slow-AR dimension table of the s2.cpp analysis pages
("Overall architecture & Dual-AR data flow", section 2; "Model loading and
GGUF", section 2.2): 36 layers, dim 2560, 32 query / 8 KV heads, head_dim 128,
SwiGLU width 9728, vocabulary 155776, RoPE base 1e6, eps 1e-6, codebook_size
4096, 10 codebooks, semantic ids 151678..155773.  The end-of-speech id
(im_end) is not on the pages; the S2 Pro shape uses 151645, an id below the
semantic range, and the tiny shape also puts it below, the ragged shape above.

Synthetic recipe (no trained weights exist here):
  * matrices and embedding tables ~ 0.02 * N(0,1), norm weights
    ~ 1 + 0.05 * N(0,1); bf16 shapes round them to bfloat16 and both sides
    consume exactly those values;
  * the KV cache is pre-filled with N(0,1) keys and values (bf16 for bf16
    shapes) at positions 0..n_fill-1;
  * the previous frame's main token is uniform over the semantic ids and its
    10 codes uniform over the codebook;
  * uniforms are (k + 0.5) * 2^-23 (exact float32 in (0,1)); a frame takes
    two for the Slow-AR draw (the main draw and the repetition resample) and
    num_codebooks-1 for the Fast-AR draws.

Every tensor has its own PCG64 stream, seeded with (seed, tensor index), so
the large shape can be drawn on several threads with the same result.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Dict, List, Optional

import numpy as np

from .inputs import bf16_bits_from_f32, exact_uniforms


@dataclass(frozen=True)
class SlowShape:
    name: str
    dim: int
    n_layer: int
    n_head: int
    n_head_kv: int
    head_dim: int
    ffn_dim: int
    vocab: int
    codebook_size: int
    sem_begin: int
    end_id: int
    max_ctx: int          # KV cache positions the context holds
    num_codebooks: int = 10
    rope_base: float = 1.0e6
    norm_eps: float = 1.0e-6
    has_qk_norm: bool = True
    weight_dtype: str = "bf16"   # also the KV cache's element type

    @property
    def sem_end(self) -> int:
        return self.sem_begin + self.codebook_size - 1

    @property
    def qkv_dim(self) -> int:
        return (self.n_head + 2 * self.n_head_kv) * self.head_dim

    @property
    def attn_dim(self) -> int:
        return self.n_head * self.head_dim


SLOW_TINY = SlowShape("slow_tiny", dim=256, n_layer=2, n_head=4, n_head_kv=2, head_dim=64, ffn_dim=768,
                      vocab=1024, codebook_size=256, sem_begin=700, end_id=650, max_ctx=80,
                      weight_dtype="f32")
SLOW_S2PRO = SlowShape("slow_s2pro", dim=2560, n_layer=36, n_head=32, n_head_kv=8, head_dim=128,
                       ffn_dim=9728, vocab=155776, codebook_size=4096, sem_begin=151678,
                       end_id=151645, max_ctx=2560)
# the measured shape's head layout (bf16, head_dim 128, 4 query heads per KV
# group) at small widths
SLOW_MID = SlowShape("slow_mid", dim=512, n_layer=2, n_head=8, n_head_kv=2, head_dim=128, ffn_dim=1024,
                     vocab=3000, codebook_size=512, sem_begin=2400, end_id=100, max_ctx=700)
# the same with a cache too long for a chunk to be held in LDS
SLOW_MID_LONG = replace(SLOW_MID, name="slow_mid_long", max_ctx=13000)
# awkward sizes: nothing a multiple of the kernels' tiles, end id above the
# semantic range, bf16 weights and cache
SLOW_RAGGED = SlowShape("slow_ragged", dim=176, n_layer=3, n_head=6, n_head_kv=2, head_dim=40,
                        ffn_dim=344, vocab=1500, codebook_size=300, sem_begin=1111, end_id=1420,
                        max_ctx=300)


def weight_names(shape: SlowShape) -> List[str]:
    names = ["embeddings", "codebook_embeddings"]
    for i in range(shape.n_layer):
        p = f"layers.{i}."
        names += [p + "attention_norm", p + "attention.wqkv", p + "attention.q_norm",
                  p + "attention.k_norm", p + "attention.wo", p + "ffn_norm",
                  p + "feed_forward.w1", p + "feed_forward.w3", p + "feed_forward.w2"]
    names.append("norm")
    return names


def weight_shape(shape: SlowShape, name: str):
    s = shape
    leaf = name.split(".")[-1] if name.startswith("layers.") else name
    return {
        "embeddings": (s.vocab, s.dim),
        "codebook_embeddings": (s.num_codebooks * s.codebook_size, s.dim),
        "attention_norm": (s.dim,),
        "wqkv": (s.qkv_dim, s.dim),
        "q_norm": (s.head_dim,),
        "k_norm": (s.head_dim,),
        "wo": (s.dim, s.attn_dim),
        "ffn_norm": (s.dim,),
        "w1": (s.ffn_dim, s.dim),
        "w3": (s.ffn_dim, s.dim),
        "w2": (s.dim, s.ffn_dim),
        "norm": (s.dim,),
    }[leaf]


def _draw(shape: SlowShape, seed: int, idx: int, name: str) -> np.ndarray:
    rng = np.random.default_rng([seed, idx])
    w = rng.standard_normal(size=weight_shape(shape, name), dtype=np.float32)
    if name.endswith("norm"):
        w *= np.float32(0.05)
        w += np.float32(1.0)
    else:
        w *= np.float32(0.02)
    return bf16_bits_from_f32(w, inplace=True) if shape.weight_dtype == "bf16" else w


def make_weights(shape: SlowShape, seed: int, threads: int = 8) -> Dict[str, np.ndarray]:
    """Every Slow-AR tensor: uint16 bf16 bits (bf16 shapes) or float32."""
    names = weight_names(shape)
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        arrs = list(ex.map(lambda t: _draw(shape, seed, t[0], t[1]), enumerate(names)))
    return dict(zip(names, arrs))


def make_kv_cache(shape: SlowShape, n_fill: int, seed: int) -> np.ndarray:
    """Cache [n_layer, n_head_kv, max_ctx, 2, head_dim] (key then value per
    position); positions >= n_fill are zero.  uint16 bf16 bits for bf16
    shapes, float32 otherwise."""
    s = shape
    assert 0 <= n_fill <= s.max_ctx
    bf = s.weight_dtype == "bf16"
    kv = np.zeros((s.n_layer, s.n_head_kv, s.max_ctx, 2, s.head_dim), np.uint16 if bf else np.float32)

    def fill(l):
        rng = np.random.default_rng([seed, 7, l])
        v = rng.standard_normal(size=(s.n_head_kv, n_fill, 2, s.head_dim), dtype=np.float32)
        kv[l, :, :n_fill] = bf16_bits_from_f32(v, inplace=True) if bf else v
    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(fill, range(s.n_layer)))
    return kv


@dataclass
class SlowWorkload:
    index: int
    name: str
    shape: SlowShape
    n_fill: int              # cache positions before the first frame
    frames: int
    temperature: float = 0.8
    top_p: float = 0.8
    top_k: int = 30

    def seed(self, k: int) -> int:
        return 1000 * self.index + k


SLOW_WORKLOADS: Dict[str, SlowWorkload] = {
    "full_s2pro": SlowWorkload(5, "full_s2pro", SLOW_S2PRO, n_fill=2048, frames=512),
    "slow_tiny": SlowWorkload(11, "slow_tiny", SLOW_TINY, n_fill=37, frames=4),
    "slow_mid": SlowWorkload(13, "slow_mid", SLOW_MID, n_fill=333, frames=3),
    "slow_mid_long": SlowWorkload(14, "slow_mid_long", SLOW_MID_LONG, n_fill=12345, frames=2),
    "slow_ragged": SlowWorkload(12, "slow_ragged", SLOW_RAGGED, n_fill=130, frames=3,
                                temperature=0.9, top_p=0.85),
}


def make_step_inputs(w: SlowWorkload, n_frames: Optional[int] = None):
    """Per-frame inputs: the previous frame's main token [F] and codes
    [F, num_codebooks], Slow-AR uniforms [F, 2], Fast-AR uniforms
    [F, num_codebooks-1]; sampling settings (scalars)."""
    F = w.frames if n_frames is None else n_frames
    s = w.shape
    rng = np.random.default_rng(w.seed(2))
    main = rng.integers(s.sem_begin, s.sem_end + 1, size=F).astype(np.int32)
    codes = rng.integers(0, s.codebook_size, size=(F, s.num_codebooks)).astype(np.int32)
    rng_u = np.random.default_rng(w.seed(3))
    u_slow = exact_uniforms(rng_u, (F, 2))
    u_fast = exact_uniforms(rng_u, (F, s.num_codebooks - 1))
    return dict(main=main, codes=codes, u_slow=u_slow, u_fast=u_fast,
                temperature=np.float32(w.temperature), top_p=np.float32(w.top_p), top_k=np.int32(w.top_k))
