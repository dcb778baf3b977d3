"""Pins of the oracle's whole forward pass and frame loop (CPU only)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import brute
from oracle import fast_ar as fa
from synth import inputs as si


@pytest.fixture(scope="module")
def tiny():
    w = si.make_weights(si.TINY, si.WORKLOADS["tiny"].seed(0))
    return si.TINY, w, fa.Model.from_weights(si.TINY, w)


@pytest.fixture(scope="module")
def ragged():
    w = si.make_weights(si.RAGGED, si.WORKLOADS["ragged"].seed(0))
    return si.RAGGED, w, fa.Model.from_weights(si.RAGGED, w)


def _inputs(shape, seed, k):
    rng = np.random.default_rng(seed)
    h = si.unit_rms(rng.standard_normal((1, shape.in_dim)).astype(np.float32))
    prefix = rng.integers(0, shape.codebook_size, size=(1, k))
    return h, prefix


@pytest.mark.parametrize("which", ["tiny", "ragged"])
def test_forward_matches_float64_brute_force(which, tiny, ragged):
    shape, w, model = tiny if which == "tiny" else ragged
    for k in (0, 1, 4, 9):
        h, prefix = _inputs(shape, 100 + k, k)
        got = fa.fast_forward(model, h, prefix)[0]
        ref = brute.forward_one(shape, w, h[0], prefix[0])
        assert np.max(np.abs(got - ref)) <= 1e-4 * np.max(np.abs(ref)), k


def _torch_forward(shape, w, h, prefix):
    """The same network written with torch library routines in float64:
    F.rms_norm, F.linear, scaled_dot_product_attention (causal, GQA via
    repeat_interleave semantics), F.silu, and RoPE as complex multiplication."""
    W = {}
    for kname, v in w.items():
        t = torch.from_numpy(v.astype(np.int16)).view(torch.bfloat16) if v.dtype == np.uint16 else torch.from_numpy(v)
        W[kname] = t.double()
    s = shape
    x0 = torch.from_numpy(h).double()
    if s.has_project_in:
        x0 = F.linear(x0, W["fast_project_in"])
    x = torch.cat([x0[None], W["fast_embeddings"][torch.from_numpy(prefix)]], 0)[None]  # [1,T,D]
    T = x.shape[1]
    hd = s.head_dim
    i = torch.arange(hd // 2, dtype=torch.float64)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * s.rope_base ** (-2.0 * i / hd)
    rot = torch.complex(torch.cos(ang).to(torch.bfloat16).double(), torch.sin(ang).to(torch.bfloat16).double())

    def rope(t):  # t [1,T,H,hd]
        c = torch.view_as_complex(t.reshape(*t.shape[:-1], hd // 2, 2).contiguous())
        return torch.view_as_real(c * rot[None, :, None, :]).reshape(t.shape)

    for li in range(s.n_layer):
        L = lambda n: W[f"fast_layers.{li}.{n}"]
        a = F.rms_norm(x, (s.dim,), L("attention_norm"), eps=s.norm_eps)
        qkv = F.linear(a, L("attention.wqkv"))
        H, G = s.n_head, s.n_head_kv
        q = qkv[..., : H * hd].reshape(1, T, H, hd)
        k = qkv[..., H * hd:(H + G) * hd].reshape(1, T, G, hd)
        v = qkv[..., (H + G) * hd:].reshape(1, T, G, hd)
        q = rope(F.rms_norm(q, (hd,), L("attention.q_norm"), eps=s.norm_eps))
        k = rope(F.rms_norm(k, (hd,), L("attention.k_norm"), eps=s.norm_eps))
        o = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2),
                                           is_causal=True, enable_gqa=True)
        x = x + F.linear(o.transpose(1, 2).reshape(1, T, H * hd), L("attention.wo"))
        n = F.rms_norm(x, (s.dim,), L("ffn_norm"), eps=s.norm_eps)
        x = x + F.linear(F.silu(F.linear(n, L("feed_forward.w1"))) * F.linear(n, L("feed_forward.w3")),
                         L("feed_forward.w2"))
    y = F.rms_norm(x[0, -1], (s.dim,), W["fast_norm"], eps=s.norm_eps)
    return F.linear(y, W["fast_output"]).numpy()


@pytest.mark.parametrize("which", ["tiny", "ragged"])
def test_forward_matches_torch_library_formulation(which, tiny, ragged):
    shape, w, model = tiny if which == "tiny" else ragged
    for k in (0, 3, 9):
        h, prefix = _inputs(shape, 200 + k, k)
        got = fa.fast_forward(model, h, prefix)[0]
        ref = _torch_forward(shape, w, h[0], prefix[0])
        assert np.max(np.abs(got - ref)) <= 1e-4 * np.max(np.abs(ref)), k


def test_appending_codes_never_changes_earlier_positions(tiny):
    shape, w, model = tiny
    h, prefix = _inputs(shape, 300, 9)
    full = fa.hidden_states(model, h, prefix)
    for k in range(0, 9):
        part = fa.hidden_states(model, h, prefix[:, :k])
        np.testing.assert_allclose(part, full[:, : k + 1], rtol=1e-5, atol=1e-5)


def test_entry_checks(tiny):
    shape, w, model = tiny
    h, prefix = _inputs(shape, 301, 9)
    with pytest.raises(fa.FastARError):
        fa.fast_forward(model, np.zeros((1, shape.in_dim + 1), np.float32), prefix)
    with pytest.raises(fa.FastARError):
        fa.fast_forward(model, h, np.zeros((1, 10), np.int64))    # prefix must be < 10 codes
    with pytest.raises(fa.FastARError):
        fa.fast_forward(model, h, np.full((1, 2), shape.codebook_size))


def test_batch_rows_are_independent(ragged):
    shape, w, model = ragged
    rng = np.random.default_rng(302)
    h = si.unit_rms(rng.standard_normal((3, shape.in_dim)).astype(np.float32))
    prefix = rng.integers(0, shape.codebook_size, size=(3, 5))
    both = fa.fast_forward(model, h, prefix)
    for b in range(3):
        np.testing.assert_allclose(both[b], fa.fast_forward(model, h[b:b + 1], prefix[b:b + 1])[0],
                                   rtol=1e-5, atol=1e-6)


def test_frame_loop_greedy_and_teacher_forcing(tiny):
    shape, w, model = tiny
    fr = si.make_frames(si.WORKLOADS["tiny"], n_frames=1)
    B = 1
    T0 = np.zeros(B, np.float32)
    r = fa.decode_frame(model, fr["hidden"][0], fr["sem_code"][0], fr["uniforms"][0], T0, fr["top_p"], fr["top_k"])
    assert r.codes.shape == (1, 10) and r.codes[0, 0] == fr["sem_code"][0, 0]
    for k in range(1, 10):
        assert r.codes[0, k] == int(np.argmax(r.logits[0, k - 1]))
        # each step's logits are a fresh call on the codes so far
        np.testing.assert_array_equal(r.logits[0, k - 1],
                                      fa.fast_forward(model, fr["hidden"][0], r.codes[:, :k].astype(np.int64))[0])
    forced = fa.decode_frame(model, fr["hidden"][0], fr["sem_code"][0], fr["uniforms"][0], T0,
                             fr["top_p"], fr["top_k"], forced=r.codes)
    np.testing.assert_array_equal(forced.logits, r.logits)
    # sem_code is clamped into the codebook
    r2 = fa.decode_frame(model, fr["hidden"][0], np.array([shape.codebook_size + 7]), fr["uniforms"][0], T0,
                         fr["top_p"], fr["top_k"])
    assert r2.codes[0, 0] == shape.codebook_size - 1
