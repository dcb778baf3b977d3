"""Pins of the oracle's building blocks against closed forms, library
routines and invariants (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import fast_ar as fa
from oracle import brute
from synth import inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_dimensions_match_pages():
    d = json.load(open(os.path.join(GOLDEN, "s2pro_dims.json")))
    s = si.S2PRO
    assert s.dim == d["fast_dim"] and s.in_dim == d["slow_dim"]
    assert s.n_layer == d["fast_layers"]
    assert (s.n_head, s.n_head_kv, s.head_dim) == (d["n_head"], d["n_head_kv"], d["fast_head_dim"])
    # head_dim is given explicitly; it is not dim / n_head
    assert d["slow_dim"] // d["n_head"] == d["head_dim_without_qk_norm"] != s.head_dim
    assert s.codebook_size == d["codebook_size"] == d["semantic_count"]
    assert d["semantic_end"] - d["semantic_begin"] + 1 == d["semantic_count"]
    assert s.num_codebooks == d["num_codebooks"]
    assert s.n_steps == d["fast_calls_per_frame"] == d["num_codebooks"] - 1
    assert s.context == d["fast_window_max"] == d["num_codebooks"] + 1
    assert s.rope_base == d["rope_base"] and s.norm_eps == d["norm_eps"]
    assert abs(d["sample_rate"] / d["samples_per_frame"] - 21.53) < 0.01


def test_sem_code_convention():
    d = json.load(open(os.path.join(GOLDEN, "s2pro_dims.json")))
    b, e = d["semantic_begin"], d["semantic_end"]
    toks = np.arange(b, e + 1)
    codes = fa.sem_code_from_main_token(toks, b, 4096)
    assert np.array_equal(codes, np.arange(4096))
    # out-of-range ids clamp both ways (defensive clamp of the main loop)
    assert list(fa.sem_code_from_main_token([b - 1, 0, e + 1, 10 ** 6], b, 4096)) == [0, 0, 4095, 4095]


def test_rms_norm_closed_form_and_library():
    w = (1 + 0.05 * np.random.default_rng(0).standard_normal(64)).astype(np.float32)
    for c in (0.0, 1e-4, 0.5, 3.0, -7.0):
        x = np.full(64, c, dtype=np.float32)
        want = c / math.sqrt(c * c + 1e-6) * w.astype(np.float64)
        np.testing.assert_allclose(fa.rms_norm(x, w, 1e-6), want, rtol=2e-7, atol=1e-12)
    x = np.random.default_rng(1).standard_normal((5, 64)).astype(np.float32) * 3
    ref = F.rms_norm(torch.from_numpy(x).double(), (64,), torch.from_numpy(w).double(), eps=1e-6).numpy()
    np.testing.assert_allclose(fa.rms_norm(x, w, 1e-6), ref, rtol=1e-6, atol=1e-7)


def test_bf16_rounding_matches_library():
    x = np.random.default_rng(2).standard_normal(100000).astype(np.float32) * 0.02
    x[:4] = [1.0, -0.0, 1.00390625, 1.01171875]   # exact and tie cases
    mine = si.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(si.f32_from_bf16_bits(mine), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_rope_table_values():
    for hd, base in ((128, 1e6), (64, 1e6), (40, 1e6)):
        c, s = fa.rope_table(hd, 11, base)
        # position 0 is the identity, exactly, even after bf16 rounding
        assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)
        # every entry is a bf16 value
        assert np.all((c.view(np.uint32) & 0xFFFF) == 0) and np.all((s.view(np.uint32) & 0xFFFF) == 0)
        # the unrounded table is cos/sin of p * base^(-2i/hd)
        c64, s64 = fa.rope_table(hd, 11, base, bf16=False)
        th = np.arange(11)[:, None] * base ** (-2.0 * np.arange(hd // 2) / hd)[None, :]
        np.testing.assert_allclose(c64, np.cos(th), atol=1e-7)
        np.testing.assert_allclose(s64, np.sin(th), atol=1e-7)
        # bf16 rounding is within half a bf16 ulp (2^-8 relative) of the exact value
        assert np.all(np.abs(c - np.cos(th)) <= 2.0 ** -8 * np.abs(np.cos(th)))
        assert np.all(np.abs(s - np.sin(th)) <= 2.0 ** -8 * np.abs(np.sin(th)))
        # an independent evaluation with the library's bf16 conversion agrees bit for bit
        rot = brute.rotations(hd, 11, base)
        assert np.array_equal(c, np.array([[r.real for r in row] for row in rot], dtype=np.float32))
        assert np.array_equal(s, np.array([[r.imag for r in row] for row in rot], dtype=np.float32))


def test_apply_rope_is_complex_rotation():
    rng = np.random.default_rng(3)
    hd, T, H = 128, 11, 3
    x = rng.standard_normal((2, T, H, hd)).astype(np.float32)
    c, s = fa.rope_table(hd, 11, 1e6)
    y = fa.apply_rope(x, c, s)
    z = (x[..., 0::2].astype(np.float64) + 1j * x[..., 1::2]) * (c + 1j * s.astype(np.float64))[None, :, None, :]
    np.testing.assert_allclose(y[..., 0::2], z.real, rtol=0, atol=1e-5)
    np.testing.assert_allclose(y[..., 1::2], z.imag, rtol=0, atol=1e-5)
    assert np.array_equal(y[:, 0], x[:, 0])            # p = 0 leaves x unchanged


def test_rope_relative_position():
    """With an exact (unrounded) table, q(p).k(p') depends only on p - p'."""
    rng = np.random.default_rng(4)
    hd = 128
    c, s = fa.rope_table(hd, 11, 1e6, bf16=False)
    q = rng.standard_normal(hd).astype(np.float32)
    k = rng.standard_normal(hd).astype(np.float32)
    Q = fa.apply_rope(np.broadcast_to(q, (11, 1, hd)).copy(), c, s)[:, 0]
    K = fa.apply_rope(np.broadcast_to(k, (11, 1, hd)).copy(), c, s)[:, 0]
    for d in range(0, 6):
        dots = [float(np.dot(Q[p + d].astype(np.float64), K[p])) for p in range(11 - d)]
        assert max(dots) - min(dots) < 1e-4 * (1 + abs(dots[0]))
    # pair norms are preserved up to the bf16 table error
    cb, sb = fa.rope_table(hd, 11, 1e6)
    Qb = fa.apply_rope(np.broadcast_to(q, (11, 1, hd)).copy(), cb, sb)[:, 0]
    n0 = q[0::2] ** 2 + q[1::2] ** 2
    for p in range(11):
        n = Qb[p, 0::2] ** 2 + Qb[p, 1::2] ** 2
        assert np.all(np.abs(n - n0) <= 2 * 2.0 ** -8 * n0 + 1e-6)


def _sdpa(q, k, v, gqa):
    qt = torch.from_numpy(q).double().permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).double().permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).double().permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, enable_gqa=gqa)
    B, H, T, hd = o.shape
    return o.permute(0, 2, 1, 3).reshape(B, T, H * hd).numpy()


def test_attention_matches_library_gqa_and_mha():
    rng = np.random.default_rng(5)
    for (H, G) in ((32, 8), (4, 2), (6, 6), (6, 2)):
        q = rng.standard_normal((2, 7, H, 16)).astype(np.float32)
        k = rng.standard_normal((2, 7, G, 16)).astype(np.float32)
        v = rng.standard_normal((2, 7, G, 16)).astype(np.float32)
        np.testing.assert_allclose(fa.causal_attention(q, k, v), _sdpa(q, k, v, H != G), rtol=1e-5, atol=1e-5)


def test_attention_invariants():
    rng = np.random.default_rng(6)
    H, G, hd = 8, 2, 32
    # one-position window: the output is the value row of the head's KV group
    q = rng.standard_normal((1, 1, H, hd)).astype(np.float32)
    k = rng.standard_normal((1, 1, G, hd)).astype(np.float32)
    v = rng.standard_normal((1, 1, G, hd)).astype(np.float32)
    o = fa.causal_attention(q, k, v).reshape(H, hd)
    for h in range(H):
        assert np.array_equal(o[h], v[0, 0, h // (H // G)])
    # equal scores: every visible value row gets the same weight
    T = 6
    q0 = np.zeros((1, T, H, hd), np.float32)
    k = rng.standard_normal((1, T, G, hd)).astype(np.float32)
    v = rng.standard_normal((1, T, G, hd)).astype(np.float32)
    o = fa.causal_attention(q0, k, v).reshape(T, H, hd)
    for i in range(T):
        for h in range(H):
            np.testing.assert_allclose(o[i, h], v[0, : i + 1, h // (H // G)].mean(axis=0), rtol=1e-5, atol=1e-6)
    # adding the same constant (+1) to every score changes nothing
    q = rng.standard_normal((1, T, H, hd)).astype(np.float32)
    base = fa.causal_attention(np.concatenate([q, np.zeros((1, T, H, 1), np.float32)], -1),
                               np.concatenate([k, np.zeros((1, T, G, 1), np.float32)], -1),
                               np.concatenate([v, np.zeros((1, T, G, 1), np.float32)], -1))
    a = np.float32(math.sqrt(hd + 1))
    shifted = fa.causal_attention(np.concatenate([q, np.full((1, T, H, 1), a, np.float32)], -1),
                                  np.concatenate([k, np.ones((1, T, G, 1), np.float32)], -1),
                                  np.concatenate([v, np.zeros((1, T, G, 1), np.float32)], -1))
    np.testing.assert_allclose(shifted, base, rtol=1e-5, atol=1e-6)


def test_silu_and_linear_library():
    rng = np.random.default_rng(7)
    z = rng.standard_normal(1000).astype(np.float32) * 4
    np.testing.assert_allclose(fa.silu(z), F.silu(torch.from_numpy(z).double()).numpy(), rtol=1e-6, atol=1e-7)
    wb = si.bf16_bits_from_f32(rng.standard_normal((96, 320)).astype(np.float32) * 0.02)
    w = fa.as_f32_weight(wb)
    x = rng.standard_normal((3, 320)).astype(np.float32)
    ref = F.linear(torch.from_numpy(x).double(), torch.from_numpy(wb.astype(np.int16)).view(torch.bfloat16).double())
    np.testing.assert_allclose(fa.linear(x, w), ref.numpy(), rtol=1e-5, atol=1e-6)


def test_exact_uniforms():
    u = si.exact_uniforms(np.random.default_rng(8), 100000)
    assert u.dtype == np.float32 and np.all(u > 0) and np.all(u < 1)
    k = (u.astype(np.float64) * 2 ** 23 - 0.5)
    assert np.array_equal(k, np.round(k))     # exact (k + 0.5) * 2^-23 in float32
