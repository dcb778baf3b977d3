"""Model shapes and seeded synthetic inputs for the Fast-AR codebook decoder.

Shapes follow the dimension tables of the s2.cpp analysis pages ("Overall
architecture & Dual-AR data flow", section 2; "Model loading and GGUF",
section 2.2): Fast-AR has 4 layers, 32 query / 8 KV heads, head_dim 128, a
window of at most 11 positions, codebook_size 4096 and 10 codebooks.  The
FFN width of the fast transformer is not on the pages; 9728 (the Slow-AR
FFN width) is assumed.

No trained weights exist here, so every workload is synthetic:
  * matrices ~ 0.02 * N(0,1), norm weights ~ 1 + 0.05 * N(0,1);
    bf16 workloads round them to bfloat16 (round to nearest even) and both
    sides consume exactly those bf16 values;
  * the Slow-AR hidden state ~ N(0,1), scaled to unit root-mean-square
    (the pages feed Fast-AR the slow model's normalised hidden state);
  * semantic codes uniform or Zipf(1.1) over the codebook;
  * the caller's uniforms are (k + 0.5) * 2^-23 for integer k in [0, 2^23),
    so every value is an exact float32 strictly inside (0, 1).

Seeds: workload c draws with numpy's PCG64 from seeds 1000*c + {0 weights,
1 hidden, 2 semantic codes, 3 uniforms, 4 per-request settings}.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Callable, Dict, List, Optional

import numpy as np


@dataclass(frozen=True)
class ModelShape:
    name: str
    in_dim: int          # width of the Slow-AR hidden state handed to Fast-AR
    dim: int             # fast_dim
    n_layer: int
    n_head: int
    n_head_kv: int
    head_dim: int
    ffn_dim: int
    codebook_size: int   # V: logits per call and codes per codebook
    num_codebooks: int = 10
    context: int = 11
    rope_base: float = 1.0e6
    norm_eps: float = 1.0e-6
    has_project_in: bool = False
    has_qk_norm: bool = True
    weight_dtype: str = "bf16"   # "bf16", "f32" or "q8" (int8 matrices, bf16 vectors)

    @property
    def qkv_dim(self) -> int:
        return (self.n_head + 2 * self.n_head_kv) * self.head_dim

    @property
    def attn_dim(self) -> int:
        return self.n_head * self.head_dim

    @property
    def n_steps(self) -> int:
        return self.num_codebooks - 1


TINY = ModelShape("tiny", in_dim=256, dim=256, n_layer=2, n_head=4, n_head_kv=2,
                  head_dim=64, ffn_dim=768, codebook_size=256, weight_dtype="f32")
S2PRO = ModelShape("s2pro", in_dim=2560, dim=2560, n_layer=4, n_head=32, n_head_kv=8,
                   head_dim=128, ffn_dim=9728, codebook_size=4096)
S2PRO_PROJ = replace(S2PRO, name="s2pro_proj", has_project_in=True)
# Deliberately awkward sizes: nothing is a multiple of the kernels' tiles,
# the projection is rectangular and head_dim is not a power of two.
RAGGED = ModelShape("ragged", in_dim=176, dim=200, n_layer=2, n_head=6, n_head_kv=2,
                    head_dim=40, ffn_dim=520, codebook_size=300, has_project_in=True)
# Weight-only int8: every weight matrix int8 with one float32 scale per
# output row; norm weights and fast_embeddings stay bf16.  Widths are
# multiples of 16 (one 16-byte load holds 16 weights).
S2PRO_Q8 = replace(S2PRO, name="s2pro_q8", weight_dtype="q8")
TINY_Q8 = replace(TINY, name="tiny_q8", weight_dtype="q8")
RAGGED_Q8 = ModelShape("ragged_q8", in_dim=176, dim=208, n_layer=2, n_head=6, n_head_kv=2,
                       head_dim=48, ffn_dim=528, codebook_size=300, has_project_in=True, weight_dtype="q8")


def weight_names(shape: ModelShape) -> List[str]:
    """Tensor names in draw order (GGUF-style names from "Model loading and
    GGUF", section 3: fast_project_in, fast_embeddings, fast_layers.i.*,
    fast_norm, fast_output)."""
    names = []
    if shape.has_project_in:
        names.append("fast_project_in")
    names.append("fast_embeddings")
    for i in range(shape.n_layer):
        p = f"fast_layers.{i}."
        names += [p + "attention_norm", p + "attention.wqkv", p + "attention.q_norm",
                  p + "attention.k_norm", p + "attention.wo", p + "ffn_norm",
                  p + "feed_forward.w1", p + "feed_forward.w3", p + "feed_forward.w2"]
    names += ["fast_norm", "fast_output"]
    return names


def weight_shape(shape: ModelShape, name: str):
    """Row-major [out, in] for matrices, [n] for norm weights."""
    s = shape
    leaf = name.split(".")[-1] if name.startswith("fast_layers") else name
    table = {
        "fast_project_in": (s.dim, s.in_dim),
        "fast_embeddings": (s.codebook_size, s.dim),
        "attention_norm": (s.dim,),
        "wqkv": (s.qkv_dim, s.dim),
        "q_norm": (s.head_dim,),
        "k_norm": (s.head_dim,),
        "wo": (s.dim, s.attn_dim),
        "ffn_norm": (s.dim,),
        "w1": (s.ffn_dim, s.dim),
        "w3": (s.ffn_dim, s.dim),
        "w2": (s.dim, s.ffn_dim),
        "fast_norm": (s.dim,),
        "fast_output": (s.codebook_size, s.dim),
    }
    return table[leaf]


def is_norm(name: str) -> bool:
    return name.endswith("norm")


def bf16_bits_from_f32(x: np.ndarray, inplace: bool = False) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16
    bit patterns.  Inputs here are always finite.  With inplace, x (float32,
    contiguous) is used as scratch and destroyed."""
    if inplace:
        b = x.view(np.uint32)
        t = b >> np.uint32(16)
        t &= np.uint32(1)
        b += t
        del t
        b += np.uint32(0x7FFF)
        b >>= np.uint32(16)
        return b.astype(np.uint16)
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_rows(w: np.ndarray):
    """Symmetric per-row int8 of a float matrix [N, K]: scale[r] =
    max_k |w[r, k]| / 127 (float64, then float32), q = round-half-even of
    w / scale clipped to [-127, 127]; an all-zero row gets scale 0 and
    q = 0.  Returns (q int8, scale float32)."""
    w64 = np.asarray(w, dtype=np.float64)
    amax = np.max(np.abs(w64), axis=1)
    scale = (amax / 127.0).astype(np.float32)
    s64 = scale.astype(np.float64)
    safe = np.where(s64 > 0, s64, 1.0)
    q = np.clip(np.rint(w64 / safe[:, None]), -127, 127)
    q[s64 == 0] = 0
    return q.astype(np.int8), scale


def is_matrix(name: str) -> bool:
    return not is_norm(name) and name != "fast_embeddings"


def make_weights(shape: ModelShape, seed: int) -> Dict[str, np.ndarray]:
    """Draw every weight tensor in `weight_names` order from one PCG64 stream.

    bf16 shapes return uint16 bit arrays, f32 shapes float32 arrays.  q8
    shapes draw the same bf16 model and store each weight matrix as int8
    (quantize_rows of its bf16 values) with its float32 row scales under
    name + ".scale"; norm weights and fast_embeddings stay bf16.
    """
    rng = np.random.default_rng(seed)
    out: Dict[str, np.ndarray] = {}
    for name in weight_names(shape):
        shp = weight_shape(shape, name)
        w = rng.standard_normal(size=shp, dtype=np.float32)
        if is_norm(name):            # 1 + 0.05 z, float32
            w *= np.float32(0.05)
            w += np.float32(1.0)
        else:                        # 0.02 z, float32
            w *= np.float32(0.02)
        if shape.weight_dtype == "f32":
            out[name] = w
            continue
        bits = bf16_bits_from_f32(w, inplace=True)
        if shape.weight_dtype == "q8" and is_matrix(name):
            out[name], out[name + ".scale"] = quantize_rows(f32_from_bf16_bits(bits))
        else:
            out[name] = bits
    return out


@dataclass
class Workload:
    """One measured / tested configuration: shape, batch, frames, sampling."""
    index: int
    name: str
    shape: ModelShape
    batch: int
    frames: int
    sem_dist: str = "uniform"        # "uniform" or "zipf"
    sampling: str = "fixed"          # "fixed", "per_request", "mixed", "greedy"
    temperature: float = 0.8
    top_p: float = 0.8
    top_k: int = 30

    def seed(self, k: int) -> int:
        return 1000 * self.index + k


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(1, "tiny", TINY, batch=1, frames=1),
    "s2pro_b1": Workload(2, "s2pro_b1", S2PRO, batch=1, frames=256),
    "s2pro_b16": Workload(3, "s2pro_b16", S2PRO, batch=16, frames=128,
                          sem_dist="zipf", sampling="per_request"),
    "s2pro_b64": Workload(4, "s2pro_b64", S2PRO_PROJ, batch=64, frames=64,
                          sampling="mixed", temperature=1.0, top_p=0.9),
    # not one of the measured workloads: awkward sizes for the parity tests
    "ragged": Workload(9, "ragged", RAGGED, batch=3, frames=4, sampling="mixed",
                       temperature=0.9, top_p=0.85),
    # weight-only int8 (the next row after the measured bf16 workloads): the
    # batch-1 workload's settings on the int8 model
    "s2pro_q8": Workload(6, "s2pro_q8", S2PRO_Q8, batch=1, frames=256),
    "tiny_q8": Workload(7, "tiny_q8", TINY_Q8, batch=1, frames=1),
    "ragged_q8": Workload(8, "ragged_q8", RAGGED_Q8, batch=3, frames=4, sampling="mixed",
                          temperature=0.9, top_p=0.85),
}


def exact_uniforms(rng: np.random.Generator, size) -> np.ndarray:
    """Uniforms (k + 0.5) * 2^-23, k integer in [0, 2^23): exact float32 in (0,1)."""
    k = rng.integers(0, 1 << 23, size=size, dtype=np.int64)
    return ((k.astype(np.float64) + 0.5) * 2.0 ** -23).astype(np.float32)


def unit_rms(h: np.ndarray) -> np.ndarray:
    """Scale each row to unit root-mean-square (input shaping for the
    synthetic Slow-AR hidden state; not part of Fast-AR)."""
    h64 = h.astype(np.float64)
    return (h64 / np.sqrt(np.mean(h64 * h64, axis=-1, keepdims=True) + 1e-6)).astype(np.float32)


def make_frames(w: Workload, n_frames: Optional[int] = None, batch: Optional[int] = None):
    """Per-frame inputs for `n_frames` frames of `batch` requests.

    Returns a dict: hidden [F,B,in_dim] f32, sem_code [F,B] int32,
    uniforms [F,B,9] f32, temperature/top_p [B] f32, top_k [B] int32.
    Per-request sampling settings are fixed over frames.
    """
    F = w.frames if n_frames is None else n_frames
    B = w.batch if batch is None else batch
    s = w.shape
    n_steps = s.n_steps

    rng_h = np.random.default_rng(w.seed(1))
    hidden = unit_rms(rng_h.standard_normal(size=(F, B, s.in_dim), dtype=np.float32))

    rng_c = np.random.default_rng(w.seed(2))
    V = s.codebook_size
    if w.sem_dist == "zipf":
        p = (np.arange(V, dtype=np.float64) + 1.0) ** -1.1
        p /= p.sum()
        sem = rng_c.choice(V, size=(F, B), p=p)
    else:
        sem = rng_c.integers(0, V, size=(F, B))
    sem = sem.astype(np.int32)

    rng_u = np.random.default_rng(w.seed(3))
    uniforms = exact_uniforms(rng_u, (F, B, n_steps))

    rng_p = np.random.default_rng(w.seed(4))
    temperature = np.full(B, w.temperature, dtype=np.float32)
    top_p = np.full(B, w.top_p, dtype=np.float32)
    top_k = np.full(B, w.top_k, dtype=np.int32)
    if w.sampling == "per_request":
        temperature = rng_p.uniform(0.6, 1.0, size=B).astype(np.float32)
        top_p = rng_p.uniform(0.7, 0.95, size=B).astype(np.float32)
    elif w.sampling == "mixed":
        temperature[: B // 2] = 0.0          # first half of the requests decode greedily
    elif w.sampling == "greedy":
        temperature[:] = 0.0
    return dict(hidden=hidden, sem_code=sem, uniforms=uniforms,
                temperature=temperature, top_p=top_p, top_k=top_k)
