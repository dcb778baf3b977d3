"""Float64 brute-force forward of the Fast-AR decoder, for small shapes.

TEST INFRASTRUCTURE ONLY (see the package header).

Written independently of ``fast_ar`` to pin it: one window at a time, one
position at a time, one head at a time, in float64, with the rotary
embedding done as complex multiplication and attention as explicit loops
over the visible keys.  It follows the same reading of the pages as
``fast_ar`` ("Fast-AR codebook decoding and the generation main loop",
sections 1-4; Mizuoto "Fish Speech" page, section "What matches upstream"), but shares no
code with it.  Slow: meant for the tiny and ragged shapes only.
"""
from __future__ import annotations

import math
from typing import Dict, List

import numpy as np
import torch


def _w64(w) -> np.ndarray:
    w = np.asarray(w)
    if w.dtype == np.uint16:
        return torch.from_numpy(w.astype(np.int16)).view(torch.bfloat16).double().numpy()
    return w.astype(np.float64)


def _bf16(v: float) -> float:
    return float(torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).double())


def rotations(head_dim: int, context: int, base: float) -> List[List[complex]]:
    """rot[p][i] = bf16(cos t) + 1j*bf16(sin t), t = p * base**(-2i/head_dim)."""
    out = []
    for p in range(context):
        row = []
        for i in range(head_dim // 2):
            t = p * base ** (-2.0 * i / head_dim)
            row.append(complex(_bf16(math.cos(t)), _bf16(math.sin(t))))
        out.append(row)
    return out


def _rms(v: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    return v / math.sqrt(float(np.dot(v, v)) / v.size + eps) * w


def _rotate(v: np.ndarray, rot_p: List[complex]) -> np.ndarray:
    out = np.empty_like(v)
    for i, r in enumerate(rot_p):
        z = complex(v[2 * i], v[2 * i + 1]) * r
        out[2 * i], out[2 * i + 1] = z.real, z.imag
    return out


def forward_one(shape, weights: Dict[str, np.ndarray], hidden: np.ndarray, prefix) -> np.ndarray:
    """Logits (float64) for a single window [hidden, emb(prefix...)]."""
    s = shape
    W = {k: _w64(v) for k, v in weights.items()}
    rot = rotations(s.head_dim, s.context, s.rope_base)
    h = np.asarray(hidden, dtype=np.float64)
    if s.has_project_in:
        h = W["fast_project_in"] @ h
    xs = [h] + [W["fast_embeddings"][int(c)].copy() for c in prefix]
    T = len(xs)
    H, G, hd = s.n_head, s.n_head_kv, s.head_dim
    per_group = H // G
    for li in range(s.n_layer):
        L = lambda n: W[f"fast_layers.{li}.{n}"]
        qs, ks, vs = [], [], []
        for p in range(T):
            a = _rms(xs[p], L("attention_norm"), s.norm_eps)
            qkv = L("attention.wqkv") @ a
            q_heads, k_heads, v_heads = [], [], []
            for hh in range(H):
                q = qkv[hh * hd:(hh + 1) * hd]
                if s.has_qk_norm:
                    q = _rms(q, L("attention.q_norm"), s.norm_eps)
                q_heads.append(_rotate(q, rot[p]))
            for g in range(G):
                off = H * hd + g * hd
                k = qkv[off:off + hd]
                if s.has_qk_norm:
                    k = _rms(k, L("attention.k_norm"), s.norm_eps)
                k_heads.append(_rotate(k, rot[p]))
                voff = (H + G) * hd + g * hd
                v_heads.append(qkv[voff:voff + hd].copy())
            qs.append(q_heads)
            ks.append(k_heads)
            vs.append(v_heads)
        new_xs = []
        for i in range(T):
            o = np.zeros(H * hd)
            for hh in range(H):
                g = hh // per_group
                scores = [float(np.dot(qs[i][hh], ks[j][g])) / math.sqrt(hd) for j in range(i + 1)]
                mx = max(scores)
                ex = [math.exp(sc - mx) for sc in scores]
                tot = sum(ex)
                acc = np.zeros(hd)
                for j in range(i + 1):
                    acc += (ex[j] / tot) * vs[j][g]
                o[hh * hd:(hh + 1) * hd] = acc
            x = xs[i] + L("attention.wo") @ o
            n = _rms(x, L("ffn_norm"), s.norm_eps)
            u1 = L("feed_forward.w1") @ n
            u3 = L("feed_forward.w3") @ n
            g_act = np.array([z / (1.0 + math.exp(-z)) for z in u1]) * u3
            new_xs.append(x + L("feed_forward.w2") @ g_act)
        xs = new_xs
    y = _rms(xs[-1], W["fast_norm"], s.norm_eps)
    return W["fast_output"] @ y
