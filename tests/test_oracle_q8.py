"""Pins of the oracle's weight-only int8 matrices (CPU only).

Format (the library's reading; the pages name GGUF quantised tensors but no
Fast-AR format): every weight matrix int8 with one float32 scale per output
row, W[r, k] = scale[r] * q[r, k]; norm weights and fast_embeddings stay
bf16."""
import numpy as np
import pytest
import torch

from oracle import brute
from oracle import fast_ar as fa
from synth import inputs as si


def test_dequantize_closed_form():
    """Distinct scales per row and per sign: a scale applied along the
    wrong axis, a dropped scale or a sign error changes these values."""
    q = np.array([[1, -2, 127, 0], [0, 5, -127, 3], [-1, 1, 2, -2]], np.int8)
    s = np.array([0.5, 0.25, 3.0], np.float32)
    want = np.array([[0.5, -1.0, 63.5, 0.0], [0.0, 1.25, -31.75, 0.75], [-3.0, 3.0, 6.0, -6.0]], np.float32)
    assert np.array_equal(fa.dequantize_rows(q, s), want)


def test_quantizer_round_trip_bound():
    """Each dequantized weight lies within half a step of the bf16 value it
    came from (the step is the row's scale); the largest |q| of a row is
    127; an all-zero row stays zero."""
    rng = np.random.default_rng(3)
    w = si.f32_from_bf16_bits(si.bf16_bits_from_f32((rng.standard_normal((64, 320)) * 0.02).astype(np.float32)))
    w[7] = 0.0
    q, s = si.quantize_rows(w)
    assert q.dtype == np.int8 and s.dtype == np.float32
    d = fa.dequantize_rows(q, s).astype(np.float64)
    err = np.abs(d - w.astype(np.float64))
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 1e-6) + 1e-12)
    nz = np.arange(64) != 7
    assert np.all(np.max(np.abs(q[nz].astype(np.int32)), axis=1) == 127)
    assert s[7] == 0 and not q[7].any() and not d[7].any()


@pytest.mark.parametrize("shape", [si.TINY_Q8, si.RAGGED_Q8], ids=["tiny_q8", "ragged_q8"])
def test_q8_forward_matches_float64_brute_force(shape):
    """The oracle's forward on the int8 model equals the float64 brute
    force run on the dequantized weights (dequantized here with torch)."""
    w = si.make_weights(shape, 77)
    model = fa.Model.from_weights(shape, w)
    wd = {}
    for k, v in w.items():
        if k.endswith(".scale"):
            continue
        if v.dtype == np.int8:
            wd[k] = (torch.from_numpy(v).double() * torch.from_numpy(w[k + ".scale"]).double()[:, None]).numpy()
        else:
            wd[k] = v
    rng = np.random.default_rng(5)
    for k in (0, 3, 9):
        h = si.unit_rms(rng.standard_normal((1, shape.in_dim)).astype(np.float32))
        prefix = rng.integers(0, shape.codebook_size, size=(1, k))
        got = fa.fast_forward(model, h, prefix)[0]
        ref = brute.forward_one(shape, wd, h[0], prefix[0])
        assert np.max(np.abs(got - ref)) <= 1e-4 * np.max(np.abs(ref)), k


def test_q8_model_stays_near_the_bf16_model():
    """The int8 model quantizes the bf16 model's matrices (steps of about
    1/127 of each row's largest weight): its logits stay within a few
    percent of the bf16 model's (informational bound for the workload)."""
    from dataclasses import replace
    s8 = si.TINY_Q8
    sb = replace(s8, name="tiny_bf16", weight_dtype="bf16")
    m8 = fa.Model.from_weights(s8, si.make_weights(s8, 11))
    mb = fa.Model.from_weights(sb, si.make_weights(sb, 11))
    rng = np.random.default_rng(2)
    h = si.unit_rms(rng.standard_normal((1, s8.in_dim)).astype(np.float32))
    prefix = rng.integers(0, s8.codebook_size, size=(1, 5))
    l8, lb = fa.fast_forward(m8, h, prefix)[0], fa.fast_forward(mb, h, prefix)[0]
    assert 0 < np.max(np.abs(l8 - lb)) <= 0.05 * np.max(np.abs(lb))
