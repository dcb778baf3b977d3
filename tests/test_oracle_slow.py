"""Pins of the Slow-AR oracle (CPU only): the cached decode step against a
full causal recompute, the input combine and the mask against closed forms,
and the repetition-aware draw against the sampler it reduces to."""
import json
import math
import os

import numpy as np
import pytest

from oracle import fast_ar as fa
from oracle import sampler as sp
from oracle import slow_ar as sa
from synth import inputs as si
from synth import slow_inputs as ssi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


@pytest.fixture(scope="module")
def tiny():
    s = ssi.SLOW_TINY
    return sa.SlowModel.from_weights(s, ssi.make_weights(s, 11))


def test_s2pro_shape_matches_pages():
    d = json.load(open(os.path.join(GOLDEN, "slow_ar.json")))
    s = ssi.SLOW_S2PRO
    assert (s.vocab, s.dim, s.ffn_dim, s.n_layer) == (d["vocab_size"], d["slow_dim"], d["slow_ffn"], d["slow_layers"])
    assert (s.n_head, s.n_head_kv, s.rope_base, s.norm_eps) == (d["n_head"], d["n_head_kv"], d["rope_base"], d["norm_eps"])
    assert (s.sem_begin, s.sem_end) == (d["semantic_begin"], d["semantic_end"])
    assert s.codebook_size == d["codebook_size"] and s.num_codebooks == d["num_codebooks"]
    assert ssi.weight_shape(s, "codebook_embeddings")[0] == d["codebook_table_rows"]
    assert s.max_ctx <= d["max_context"]
    assert s.num_codebooks + 1 == d["sem_scale_inverse_square"]
    assert not (s.sem_begin <= s.end_id <= s.sem_end)
    assert (sa.RAS_WINDOW, sa.RAS_TEMPERATURE, sa.RAS_TOP_P) == (d["ras_window"], d["ras_temperature"], d["ras_top_p"])


def test_combine_closed_form():
    """Row r of each table filled with the value r: the combine is then
    main/sqrt(11) + sum_j (j*cbs + c_j) in every column."""
    s = ssi.SLOW_TINY
    w = {"embeddings": np.repeat(np.arange(s.vocab, dtype=F32)[:, None], s.dim, 1),
         "codebook_embeddings": np.repeat(np.arange(s.num_codebooks * s.codebook_size, dtype=F32)[:, None], s.dim, 1)}
    m = sa.SlowModel(s, w)
    rng = np.random.default_rng(0)
    for _ in range(5):
        main = int(rng.integers(s.sem_begin, s.sem_end + 1))   # a position that carries codes
        codes = rng.integers(0, s.codebook_size, size=s.num_codebooks)
        x = sa.combine(m, main, codes)
        want = main / math.sqrt(11.0) + sum(j * s.codebook_size + int(c) for j, c in enumerate(codes))
        np.testing.assert_allclose(x, np.full(s.dim, want), rtol=2e-7)


def test_sem_mask_and_allowed_ids():
    for s in (ssi.SLOW_S2PRO, ssi.SLOW_TINY, ssi.SLOW_RAGGED):
        m = sa.sem_mask(s)
        ids = sa.allowed_ids(s)
        assert m.shape == (s.vocab,)
        assert ids.size == s.codebook_size + 1
        assert np.all(m[ids] == 0) and np.all(np.isneginf(np.delete(m, ids)))
        assert m[s.sem_begin] == 0 and m[s.sem_end] == 0 and m[s.end_id] == 0
        assert np.isneginf(m[s.sem_begin - 1]) or s.end_id == s.sem_begin - 1
        assert np.all(np.diff(ids) > 0)
    d = json.load(open(os.path.join(GOLDEN, "slow_ar.json")))
    assert sa.allowed_ids(ssi.SLOW_S2PRO).size == d["mask_finite_count_without_end"] + 1


def test_sem_code_clamp():
    s = ssi.SLOW_S2PRO
    assert sa.sem_code(s, s.sem_begin) == 0 and sa.sem_code(s, s.sem_end) == 4095
    assert sa.sem_code(s, s.end_id) == 0            # below the range: clamped up
    assert sa.sem_code(s, s.vocab - 1) == 4095       # above: clamped down


def test_attend_single_position_is_value():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((4, 8)).astype(F32)
    K = rng.standard_normal((2, 1, 8)).astype(F32)
    V = rng.standard_normal((2, 1, 8)).astype(F32)
    o = sa.attend(q, K, V).reshape(4, 8)
    for h in range(4):
        np.testing.assert_array_equal(o[h], V[h // 2, 0])


def test_attend_equal_keys_average_values():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((4, 8)).astype(F32)
    K = np.repeat(rng.standard_normal((2, 1, 8)).astype(F32), 5, axis=1)
    V = rng.standard_normal((2, 5, 8)).astype(F32)
    o = sa.attend(q, K, V).reshape(4, 8)
    for h in range(4):
        np.testing.assert_allclose(o[h], V[h // 2].mean(axis=0), rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("T", [1, 2, 9])
def test_cached_steps_equal_full_causal_recompute(tiny, T):
    """T decode steps from an empty cache give, at the last position, the
    final-layer state of one causal forward over all T inputs (positions
    0..T-1, mask offset 0) computed by the Fast-AR block."""
    s = tiny.shape
    rng = np.random.default_rng(3)
    xs = rng.standard_normal((T, s.dim)).astype(F32)
    kv = np.zeros((s.n_layer, s.n_head_kv, T, 2, s.head_dim), F32)
    for p in range(T):
        st = sa.step(tiny, xs[p], kv, p)
        kv[:, :, p] = st.kv_new
    cos, sin = fa.rope_table(s.head_dim, T, s.rope_base)
    x = xs[None].copy()
    for i in range(s.n_layer):
        x = fa.block(tiny, i, x, cos, sin)
    h = fa.rms_norm(x[0, -1], tiny.get("norm"), s.norm_eps)
    np.testing.assert_allclose(st.hidden, h, rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(st.logits, fa.linear(h, tiny.get("embeddings")), rtol=1e-4, atol=1e-5)


def test_step_positions_matter(tiny):
    """The same input at another position gives another state (RoPE sees
    the position), and an unrelated cache changes it too."""
    s = tiny.shape
    rng = np.random.default_rng(4)
    kv = rng.standard_normal((s.n_layer, s.n_head_kv, 6, 2, s.head_dim)).astype(F32)
    x = rng.standard_normal(s.dim).astype(F32)
    a = sa.step(tiny, x, kv, 5).hidden
    b = sa.step(tiny, x, kv, 4).hidden
    kv2 = kv.copy()
    kv2[:, :, 0] += 1.0
    c = sa.step(tiny, x, kv2, 5).hidden
    assert np.abs(a - b).max() > 1e-4 and np.abs(a - c).max() > 1e-4


def test_bf16_cache_entries_are_rounded():
    s = ssi.SLOW_RAGGED
    m = sa.SlowModel.from_weights(s, ssi.make_weights(s, 5))
    kv = si.f32_from_bf16_bits(ssi.make_kv_cache(s, 4, 6))
    st = sa.step(m, np.ones(s.dim, F32), kv, 4)
    bits = st.kv_new.view(np.uint32)
    assert np.all(bits & np.uint32(0xFFFF) == 0)
    # bf16 keeps 8 significant bits (ulp 2^-7 at 1.0); halfway cases go to the even neighbour
    x = np.array([1.0 + 2 ** -9, 1.0 + 3 * 2 ** -9, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], F32)
    want = np.array([1.0, 1.0 + 2 ** -7, 1.0, 1.0 + 2 ** -6], F32)
    np.testing.assert_array_equal(sa.bf16_round_f32(x), want)


def _logits(s, rng):
    return (rng.standard_normal(s.vocab) * 3).astype(F32)


def test_main_draw_stays_in_allowed_set():
    s = ssi.SLOW_S2PRO
    rng = np.random.default_rng(5)
    allowed = set(sa.allowed_ids(s).tolist())
    for _ in range(20):
        l = _logits(s, rng)
        u = si.exact_uniforms(rng, 2)
        d = sa.draw_main(s, l, [], 0.8, 0.8, 30, u[0], u[1])
        assert d.token in allowed and not d.resampled
    # greedy: argmax over the allowed ids only
    l = _logits(s, rng)
    l[0] = 100.0                                   # a masked id with the largest logit
    d = sa.draw_main(s, l, [], 0.0, 0.8, 30, 0.5, 0.5)
    ids = sa.allowed_ids(s)
    assert d.token == ids[np.argmax(l[ids])]


def test_repetition_resample():
    s = ssi.SLOW_S2PRO
    rng = np.random.default_rng(6)
    l = _logits(s, rng)
    u = si.exact_uniforms(rng, 2)
    d0 = sa.draw_main(s, l, [], 0.8, 0.8, 30, u[0], u[1])
    # the first draw is in the window: redrawn at T=1.0, top_p=0.9 with u_ras
    win = [s.sem_begin + 3, d0.first, s.sem_begin + 7]
    d1 = sa.draw_main(s, l, win, 0.8, 0.8, 30, u[0], u[1])
    masked = l + sa.sem_mask(s)
    assert d1.first == d0.first and d1.resampled
    assert d1.token == sp.sample(masked, F32(1.0), F32(0.9), 30, u[1]).code
    # not in the window: kept
    d2 = sa.draw_main(s, l, [s.sem_begin + 1], 0.8, 0.8, 30, u[0], u[1])
    assert d2.token == d0.first and not d2.resampled


def test_repetition_skips_end_id():
    s = ssi.SLOW_S2PRO
    rng = np.random.default_rng(7)
    l = _logits(s, rng)
    l[s.end_id] = 50.0
    d = sa.draw_main(s, l, [s.end_id], 0.8, 0.8, 30, 0.3, 0.6)
    assert d.first == s.end_id and d.token == s.end_id and not d.resampled


def test_window_keeps_newest_ten():
    w = []
    for t in range(13):
        w = sa.push_window(w, 100 + t)
    assert w == list(range(103, 113))


def test_decode_frame_tiny(tiny):
    s = tiny.shape
    fs = si.TINY
    fast = fa.Model.from_weights(fs, si.make_weights(fs, 1000))
    kv = ssi.make_kv_cache(s, 9, 3)
    inp = ssi.make_step_inputs(ssi.SLOW_WORKLOADS["slow_tiny"], 1)
    r = sa.decode_frame(tiny, fast, kv, 9, inp["main"][0], inp["codes"][0], [], inp["u_slow"][0],
                        inp["u_fast"][0], 0.8, 0.8, 30)
    assert r.codes[0] == r.sem_code == sa.sem_code(s, r.main.token)
    assert r.main.token in set(sa.allowed_ids(s).tolist())
    rms = np.sqrt(np.mean((r.hidden / tiny.get("norm")).astype(np.float64) ** 2))
    assert abs(rms - 1.0) < 1e-3
    assert r.window == [r.main.token]
    want = fa.decode_frame(fast, r.hidden[None], np.array([r.sem_code]), inp["u_fast"][:1],
                           np.array([0.8], F32), np.array([0.8], F32), np.array([30]))
    np.testing.assert_array_equal(r.codes, want.codes[0])


def test_combine_text_position_has_no_codebook_terms():
    """A row-0 token outside the semantic ids (text, markers, the end id)
    takes its scaled embedding only."""
    s = ssi.SLOW_TINY
    w = {"embeddings": np.repeat(np.arange(s.vocab, dtype=F32)[:, None], s.dim, 1),
         "codebook_embeddings": np.repeat(np.arange(s.num_codebooks * s.codebook_size, dtype=F32)[:, None], s.dim, 1)}
    m = sa.SlowModel(s, w)
    codes = np.arange(s.num_codebooks) + 5
    for tok in (0, 17, s.sem_begin - 1, s.end_id, s.sem_end + 1, s.vocab - 1):
        np.testing.assert_allclose(sa.combine(m, tok, codes), np.full(s.dim, tok / math.sqrt(11.0)), rtol=2e-7)
    assert sa.is_semantic(s, s.sem_begin) and sa.is_semantic(s, s.sem_end)
    assert not sa.is_semantic(s, s.end_id)


def test_prefill_equals_full_causal_forward(tiny):
    """Prefill of a mixed prompt (text tokens, then semantic positions with
    codes) from an empty cache gives, at its last position, the final state
    of one causal forward over the combined inputs."""
    s = tiny.shape
    rng = np.random.default_rng(8)
    T = 7
    toks = np.zeros((T, 1 + s.num_codebooks), np.int64)
    toks[:3, 0] = rng.integers(0, s.sem_begin, size=3)                     # text
    toks[3:, 0] = rng.integers(s.sem_begin, s.sem_end + 1, size=T - 3)     # reference audio
    toks[3:, 1:] = rng.integers(0, s.codebook_size, size=(T - 3, s.num_codebooks))
    kv = np.zeros((s.n_layer, s.n_head_kv, T, 2, s.head_dim), F32)
    st = sa.prefill(tiny, toks, kv, 0)
    xs = np.stack([sa.combine(tiny, toks[t, 0], toks[t, 1:]) for t in range(T)])[None]
    cos, sin = fa.rope_table(s.head_dim, T, s.rope_base)
    for i in range(s.n_layer):
        xs = fa.block(tiny, i, xs, cos, sin)
    h = fa.rms_norm(xs[0, -1], tiny.get("norm"), s.norm_eps)
    np.testing.assert_allclose(st.hidden, h, rtol=1e-4, atol=1e-5)
    assert np.all(kv[:, :, T - 1] == st.kv_new)
    # the same prompt in two parts gives the same state
    kv2 = np.zeros_like(kv)
    sa.prefill(tiny, toks[:4], kv2, 0)
    st2 = sa.prefill(tiny, toks[4:], kv2, 4)
    np.testing.assert_array_equal(st2.hidden, st.hidden)


# ------------------------------------------------------------ rounding follow
# A bf16 cache rounds every new key and value.  Two implementations whose
# float32 values differ in the last bits can round a value that sits next to
# a rounding midpoint to different neighbours; the oracle then follows the
# other implementation's entry, after checking it is such a rounding.

def _deep_mid_shape():
    from dataclasses import replace
    return replace(ssi.SLOW_MID, name="deep_mid", n_layer=36)


def test_rounding_flips_compound_over_36_layers_and_following_removes_them():
    """At position 0 the attention output is the rounded value itself, so
    flips feed straight into the residual stream.  Emulate an implementation
    whose float32 keys/values differ by ~1e-6 relative before rounding: a few
    entries round the other way, the hidden state moves by about 1e-3 of its
    largest element (more than a 1e-3 * max + 1e-4 bound allows room for),
    and following its entries reproduces its hidden state exactly."""
    shp = _deep_mid_shape()
    m = sa.SlowModel.from_weights(shp, ssi.make_weights(shp, 7))
    kv = np.zeros((shp.n_layer, shp.n_head_kv, 1, 2, shp.head_dim), np.float32)
    x = sa.combine(m, shp.sem_begin + 3, np.arange(shp.num_codebooks))
    own = sa.step(m, x, kv, 0)
    rng = np.random.default_rng(1)
    exact_round = sa.cache_round

    def other(s, v):
        v = np.asarray(v, np.float32)
        return exact_round(s, (v.astype(np.float64) * (1 + rng.standard_normal(v.shape) * 1e-6)).astype(np.float32))

    sa.cache_round = other
    try:
        theirs = sa.step(m, x, kv, 0)
    finally:
        sa.cache_round = exact_round
    followed = sa.step(m, x, kv, 0, follow=theirs.kv_new)
    M = float(np.abs(theirs.hidden).max())
    assert followed.flips >= 1
    assert float(np.abs(own.hidden - theirs.hidden).max()) > 5e-4 * M
    assert np.array_equal(followed.hidden, theirs.hidden)
    assert np.array_equal(followed.kv_new, theirs.kv_new)


def test_follow_rounding_accepts_only_defensible_entries():
    s = ssi.SLOW_MID                                   # bf16 cache
    lo = np.float32(1.0)                               # bf16 neighbours 1.0 and 1.0078125
    hi = np.float32(1.0078125)
    mid = (np.float64(lo) + np.float64(hi)) / 2
    near = np.float32(mid * (1 + 3e-6))                # rounds to hi; within the band of the midpoint
    far = np.float32(1.002)                            # rounds to lo; far from the midpoint
    tiny = np.float32(-1.5057623e-05)                  # far below the band: several roundings are defensible
    exact = np.array([near, far, -near, tiny], np.float32)
    mine = sa.cache_round(s, exact)
    assert list(mine[:3]) == [hi, lo, -hi]
    got, flips = sa.follow_rounding(s, exact, mine)
    assert flips == 0 and np.array_equal(got, mine)
    other_tiny = np.float32(-1.50203705e-05)           # a bf16 value one ulp from the oracle's rounding
    got, flips = sa.follow_rounding(s, exact, np.array([lo, lo, -lo, other_tiny], np.float32))
    assert flips == 3 and list(got) == [lo, lo, -lo, other_tiny]
    for bad in ([lo, hi, -hi, mine[3]],                # a flip away from any midpoint
                [np.float32(1.015625), lo, -hi, mine[3]],   # two ulps off
                [hi, lo, np.float32(1.0078125), mine[3]],   # wrong sign
                [hi, lo, -hi, np.float32(-1.0e-3)],    # a small value far outside the band
                [hi, np.float32(1.0000001), -hi, mine[3]]):  # not a bf16 value
        with pytest.raises(sa.CacheFollowError):
            sa.follow_rounding(s, exact, np.array(bad, np.float32))
    # float32 caches are not rounded: the oracle keeps its own values
    got, flips = sa.follow_rounding(ssi.SLOW_TINY, exact, exact + 1)
    assert flips == 0 and np.array_equal(got, exact)
