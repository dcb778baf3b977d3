"""Oracle forward pass and frame loop of the Fast-AR codebook decoder.

TEST INFRASTRUCTURE ONLY (see the package header).

Plain float32 numpy.  Every call recomputes its whole window from scratch,
as the pages describe it (no KV cache: "Fast-AR codebook decoding and the
generation main loop", section 1; causal mask with offset 0, section 3).
A batch of B requests at the same step is computed as B independent windows
of equal length; nothing is shared between requests.

Readings of points the pages leave open:
  * pre-norm residual blocks, x += attn(norm(x)); x += ffn(norm(x)) — the
    pages call the block "almost isomorphic" to the Qwen3-shaped Slow-AR;
  * the fused wqkv output is [Q (n_head*hd) | K (n_kv*hd) | V (n_kv*hd)],
    each head-major;
  * SwiGLU is w2(silu(w1 n) * w3 n);
  * Fast-AR uses the Slow-AR RoPE base (1e6) and RMSNorm eps (1e-6), also
    for the per-head q/k norms;
  * query head h reads KV head floor(h / (n_head / n_kv)) (repeat_interleave);
  * fast_project_in, when present, has no bias and maps position 0 only;
  * every step's logits cover the full codebook (4096); nothing is masked.

Pins: tests/test_oracle_forward.py (float64 brute force, torch library
formulation, invariants) and tests/test_oracle_pins.py (closed forms).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np

from . import sampler as _sampler

F32 = np.float32


class FastARError(ValueError):
    """Raised for inputs the pages' entry checks reject."""


def as_f32_weight(w: np.ndarray) -> np.ndarray:
    """Weights arrive as float32 or as bfloat16 bit patterns (uint16);
    bf16 widens exactly to float32."""
    w = np.asarray(w)
    if w.dtype == np.uint16:
        return (w.astype(np.uint32) << np.uint32(16)).view(F32)
    return w.astype(F32, copy=False)


SCALE_SUFFIX = ".scale"


def dequantize_rows(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Weight-only int8 matrices with one float32 scale per output row:
    W[r, k] = scale[r] * q[r, k], rounded to float32.  (The pages name GGUF
    quantised tensors, "Overall architecture & Dual-AR data flow", section 5
    and "Model loading and GGUF", section 4, but no Fast-AR format; per-row
    symmetric int8 is the library's reading.)"""
    q = np.asarray(q)
    assert q.dtype == np.int8 and q.ndim == 2
    scale = np.asarray(scale, dtype=F32).reshape(-1)
    assert scale.shape[0] == q.shape[0]
    return (scale.astype(np.float64)[:, None] * q.astype(np.float64)).astype(F32)


@dataclass
class Model:
    """Shape hyper-parameters plus float32 weights keyed by GGUF-style name."""
    shape: object
    w: Dict[str, np.ndarray]

    @classmethod
    def from_weights(cls, shape, weights: Dict[str, np.ndarray]) -> "Model":
        """Weights as float32 or bf16 bits; an int8 matrix comes with its
        per-row scales under name + ".scale" and is dequantized."""
        out = {}
        for k, v in weights.items():
            if k.endswith(SCALE_SUFFIX):
                continue
            if np.asarray(v).dtype == np.int8:
                out[k] = dequantize_rows(v, weights[k + SCALE_SUFFIX])
            else:
                out[k] = as_f32_weight(v)
        return cls(shape, out)

    def layer(self, i: int, name: str) -> np.ndarray:
        return self.w[f"fast_layers.{i}.{name}"]


# --------------------------------------------------------------------------
# building blocks
# --------------------------------------------------------------------------

def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis in float32: x / sqrt(mean(x^2) + eps) * w.
    ("Model loading and GGUF" section 2.2 gives eps 1e-6; the Mizuoto page,
    section "What matches upstream", computes it in float32.)"""
    x = np.asarray(x, dtype=F32)
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=F32)
    return (x / np.sqrt(ms + F32(eps))) * weight


def bf16_round_f64(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits),
    ties to even, directly from float64; returned as float64."""
    m, e = np.frexp(np.asarray(v, dtype=np.float64))
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def rope_table(head_dim: int, context: int, base: float, bf16: bool = True):
    """cos/sin table [context, head_dim/2] for positions 0..context-1.

    theta(p, i) = p * base^(-2i/head_dim), evaluated in float64; the Mizuoto
    page (section "What matches upstream") rounds the frequency table to bfloat16.  Returns
    float32 arrays holding the (bf16-rounded) values."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / head_dim)
    theta = np.arange(context, dtype=np.float64)[:, None] * inv_freq[None, :]
    c, s = np.cos(theta), np.sin(theta)
    if bf16:
        c, s = bf16_round_f64(c), bf16_round_f64(s)
    return c.astype(F32), s.astype(F32)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs (x[2i], x[2i+1]) by the angle of position p.

    x: [..., T, H, hd]; cos/sin: [T, hd/2] (rows = window positions).
    (a, b) -> (a cos - b sin, a sin + b cos), float32."""
    a = x[..., 0::2]
    b = x[..., 1::2]
    c = cos[:, None, :]
    s = sin[:, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Scaled dot-product attention with a causal mask of offset 0.

    q: [B, T, H, hd]; k, v: [B, T, Hkv, hd].  Position i attends to j <= i
    ("Fast-AR codebook decoding ...", section 3: the window always starts at
    position 0, so the mask offset is 0).  Scale 1/sqrt(head_dim) (section 1).
    Query head h reads KV head h // (H / Hkv).  Returns [B, T, H*hd]."""
    B, T, H, hd = q.shape
    Hkv = k.shape[2]
    group = H // Hkv
    kx = np.repeat(k, group, axis=2)          # repeat_interleave over heads
    vx = np.repeat(v, group, axis=2)
    qh = q.transpose(0, 2, 1, 3)              # [B, H, T, hd]
    kh = kx.transpose(0, 2, 3, 1)             # [B, H, hd, T]
    vh = vx.transpose(0, 2, 1, 3)             # [B, H, T, hd]
    scale = F32(1.0 / np.sqrt(hd))
    s = np.matmul(qh, kh) * scale             # [B, H, T, T]
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    s = np.where(mask, F32(-np.inf), s)
    s = s - np.max(s, axis=-1, keepdims=True)
    e = np.exp(s)
    p = e / np.sum(e, axis=-1, keepdims=True)
    o = np.matmul(p, vh)                      # [B, H, T, hd]
    return o.transpose(0, 2, 1, 3).reshape(B, T, H * hd)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (F32(1.0) + np.exp(-z))


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """x [..., in] times a row-major [out, in] weight: x @ w.T in float32.
    The leading axes are flattened first, so a batch of windows is one
    matrix product over all of its rows (each output is still the dot
    product of one input row with one weight row)."""
    x = np.asarray(x)
    y = np.matmul(x.reshape(-1, x.shape[-1]), w.T)
    return y.reshape(x.shape[:-1] + (w.shape[0],))


# --------------------------------------------------------------------------
# the forward pass
# --------------------------------------------------------------------------

def check_inputs(model: Model, hidden: np.ndarray, prefix: np.ndarray) -> None:
    """Entry checks of fast_decode ("Fast-AR codebook decoding ...",
    section 1): the hidden state has exactly in_dim values and the prefix
    holds fewer codes than there are codebooks."""
    s = model.shape
    if hidden.ndim != 2 or hidden.shape[1] != s.in_dim:
        raise FastARError(f"hidden must be [B, {s.in_dim}], got {hidden.shape}")
    if prefix.ndim != 2 or prefix.shape[0] != hidden.shape[0]:
        raise FastARError("prefix must be [B, k]")
    if prefix.shape[1] >= s.num_codebooks:
        raise FastARError(f"prefix length {prefix.shape[1]} must be < {s.num_codebooks}")
    if prefix.size and (prefix.min() < 0 or prefix.max() >= s.codebook_size):
        raise FastARError("prefix codes must lie in [0, codebook_size)")


def window(model: Model, hidden: np.ndarray, prefix: np.ndarray) -> np.ndarray:
    """Assemble the window ("Fast-AR codebook decoding ...", section 2):
    position 0 is the Slow-AR hidden (through fast_project_in if present),
    positions 1..k are fast_embeddings rows of the codes so far."""
    s = model.shape
    h = np.asarray(hidden, dtype=F32)
    x0 = linear(h, model.w["fast_project_in"]) if s.has_project_in else h
    emb = model.w["fast_embeddings"][prefix]          # [B, k, dim]
    return np.concatenate([x0[:, None, :], emb], axis=1).astype(F32)


def block(model: Model, i: int, x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """One transformer layer over the whole window, x: [B, T, dim]
    ("Fast-AR codebook decoding ...", section 3: RMSNorm, fused wqkv, view
    split, optional q/k norm, RoPE, 4x GQA expansion, scaled dot-product
    attention, wo, SwiGLU FFN)."""
    s = model.shape
    B, T, _ = x.shape
    H, Hkv, hd = s.n_head, s.n_head_kv, s.head_dim
    a = rms_norm(x, model.layer(i, "attention_norm"), s.norm_eps)
    qkv = linear(a, model.layer(i, "attention.wqkv"))
    q = qkv[..., : H * hd].reshape(B, T, H, hd)
    k = qkv[..., H * hd: (H + Hkv) * hd].reshape(B, T, Hkv, hd)
    v = qkv[..., (H + Hkv) * hd:].reshape(B, T, Hkv, hd)
    if s.has_qk_norm:
        q = rms_norm(q, model.layer(i, "attention.q_norm"), s.norm_eps)
        k = rms_norm(k, model.layer(i, "attention.k_norm"), s.norm_eps)
    q = apply_rope(q, cos[:T], sin[:T])
    k = apply_rope(k, cos[:T], sin[:T])
    o = causal_attention(q, k, v)
    x = x + linear(o, model.layer(i, "attention.wo"))
    n = rms_norm(x, model.layer(i, "ffn_norm"), s.norm_eps)
    g = silu(linear(n, model.layer(i, "feed_forward.w1"))) * linear(n, model.layer(i, "feed_forward.w3"))
    x = x + linear(g, model.layer(i, "feed_forward.w2"))
    return x.astype(F32)


def hidden_states(model: Model, hidden: np.ndarray, prefix: np.ndarray) -> np.ndarray:
    """Final-layer states of every window position, [B, T, dim] (before
    fast_norm).  Positions restart at 0 on every call (section 2)."""
    s = model.shape
    hidden = np.asarray(hidden, dtype=F32)
    prefix = np.asarray(prefix, dtype=np.int64).reshape(hidden.shape[0], -1)
    check_inputs(model, hidden, prefix)
    cos, sin = rope_table(s.head_dim, s.context, s.rope_base)
    x = window(model, hidden, prefix)
    if x.shape[1] > s.context:
        raise FastARError("window longer than the RoPE context")
    for i in range(s.n_layer):
        x = block(model, i, x, cos, sin)
    return x


def fast_forward(model: Model, hidden: np.ndarray, prefix: np.ndarray) -> np.ndarray:
    """One Fast-AR call: logits [B, V] for the code after `prefix`.

    Only the last window position feeds the head: fast_norm, then the untied
    fast_output matrix ("Fast-AR codebook decoding ...", section 4)."""
    s = model.shape
    x = hidden_states(model, hidden, prefix)
    y = rms_norm(x[:, -1, :], model.w["fast_norm"], s.norm_eps)
    return linear(y, model.w["fast_output"]).astype(F32)


def clamp_sem_code(sem_code, V: int) -> np.ndarray:
    """sem_code = main_token - semantic_begin, clamped to [0, V-1] in both
    directions as the caller does ("Fast-AR codebook decoding ...", sections
    5.1 and 5.2)."""
    return np.clip(np.asarray(sem_code, dtype=np.int64), 0, V - 1)


def sem_code_from_main_token(main_token, semantic_begin: int = 151678, V: int = 4096):
    """The frame's codebook-0 code from the Slow-AR main token ("Overall
    architecture ...", section 3.3)."""
    return clamp_sem_code(np.asarray(main_token, dtype=np.int64) - semantic_begin, V)


@dataclass
class FrameResult:
    codes: np.ndarray      # [B, num_codebooks] int32
    logits: np.ndarray     # [B, n_steps, V] float32, logits of each step
    fragile: np.ndarray    # [B, n_steps] bool, knife-edge decisions
    alts: list = None      # [B][n_steps] tuples: every defensible code of each draw


def decode_frame(model: Model, hidden, sem_code, uniforms, temperature, top_p, top_k,
                 forced: Optional[np.ndarray] = None) -> FrameResult:
    """One frame: codes [sem_code, r_1, ..., r_9].

    Step k = 1..9 calls fast_forward on [hidden, codes so far] and samples
    r_k ("Fast-AR codebook decoding ...", section 5.1, step 3).  `uniforms`
    is [B, 9]: column k-1 drives step k.  With `forced` ([B, 10]) the prefix
    of every step is taken from it instead of from the draws (teacher
    forcing); the draws are still reported."""
    s = model.shape
    hidden = np.asarray(hidden, dtype=F32)
    B = hidden.shape[0]
    codes = np.zeros((B, s.num_codebooks), dtype=np.int64)
    codes[:, 0] = clamp_sem_code(sem_code, s.codebook_size)
    prefix_src = codes if forced is None else np.asarray(forced, dtype=np.int64).copy()
    if forced is not None:
        prefix_src[:, 0] = codes[:, 0]
    logits = np.zeros((B, s.n_steps, s.codebook_size), dtype=F32)
    fragile = np.zeros((B, s.n_steps), dtype=bool)
    alts = [[None] * s.n_steps for _ in range(B)]
    for k in range(1, s.num_codebooks):
        lg = fast_forward(model, hidden, prefix_src[:, :k])
        logits[:, k - 1] = lg
        for b in range(B):
            d = _sampler.sample(lg[b], temperature[b], top_p[b], top_k[b], uniforms[b][k - 1])
            codes[b, k] = d.code
            fragile[b, k - 1] = d.fragile
            alts[b][k - 1] = d.alts
    return FrameResult(codes.astype(np.int32), logits, fragile, alts)
