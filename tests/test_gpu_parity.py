"""Parity of the HIP path (through the C ABI) with the oracle, on the GPU.

Logits: |delta| <= 1e-2 * max|logit| + 1e-3 under teacher-forced prefixes.
Codes: bit-exact except at decisions the oracle reports as knife-edges
(greedy top-2 gap < 1e-3; sampled top-k boundary, nucleus boundary or race
within the sampler's margins)."""
import numpy as np
import pytest
import torch

from dual_ar_neural_amd import binding as bd
from oracle import sampler as sm
from synth import inputs as si
from tests import parity as pr

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.fixture(scope="module")
def tiny():
    _announce("tiny model")
    return pr.make_pair(si.TINY, si.WORKLOADS["tiny"].seed(0), max_batch=4)


@pytest.fixture(scope="module")
def ragged():
    _announce("ragged model")
    return pr.make_pair(si.RAGGED, si.WORKLOADS["ragged"].seed(0), max_batch=4)


@pytest.fixture(scope="module")
def s2pro():
    _announce("s2pro model (bf16, 828 MB)")
    return pr.make_pair(si.S2PRO, si.WORKLOADS["s2pro_b1"].seed(0), max_batch=64)


# ------------------------------------------------------------------ sampler

def _sampler_cases():
    rng = np.random.default_rng(123)
    cases = []
    for V in (4096, 256, 300, 50, 8192, 64, 2):
        for T, tp, tk in ((0.8, 0.8, 30), (1.0, 0.9, 30), (0.0, 0.8, 30), (-1.0, 0.5, 30), (0.05, 0.95, 64),
                          (3.0, 1.0, 100), (0.7, 0.0, 30), (0.9, 1e-9, 1), (1.2, 0.99, 0), (0.6, 0.7, 13)):
            for kind in ("normal", "ties", "flat", "spiky", "outlier", "bf16"):
                if kind == "normal":
                    l = rng.standard_normal(V).astype(np.float32) * rng.uniform(0.5, 4)
                elif kind == "ties":
                    l = (np.round(rng.standard_normal(V) * 2) / 2).astype(np.float32)
                elif kind == "flat":
                    l = np.full(V, 0.25, np.float32)
                elif kind == "spiky":
                    l = rng.standard_normal(V).astype(np.float32)
                    l[rng.integers(0, V, size=3)] += 8.0
                elif kind == "outlier":      # a huge range: many threshold-search rounds
                    l = rng.standard_normal(V).astype(np.float32)
                    l[rng.integers(0, V)] = 1e6
                    l[rng.integers(0, V)] = -1e6
                else:                        # bf16-quantised logits: near-ties at every scale
                    l = (rng.standard_normal(V) * 3).astype(np.float32)
                    l = (l.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
                u = np.float32((rng.integers(0, 1 << 23) + 0.5) * 2.0 ** -23)
                cases.append((l, np.float32(T), np.float32(tp), np.int32(tk), u))
    return cases


def test_sampler_bit_exact_with_oracle():
    cases = _sampler_cases()
    by_v = {}
    for c in cases:
        by_v.setdefault(c[0].size, []).append(c)
    n = 0
    for V, cs in by_v.items():
        logits = pr.to_dev(np.stack([c[0] for c in cs]))
        T = pr.to_dev(np.array([c[1] for c in cs], np.float32))
        tp = pr.to_dev(np.array([c[2] for c in cs], np.float32))
        tk = pr.to_dev(np.array([c[3] for c in cs], np.int32))
        u = pr.to_dev(np.array([c[4] for c in cs], np.float32))
        got = bd.sample(logits, T, tp, tk, u).cpu().numpy()
        for i, c in enumerate(cs):
            want = sm.sample(*c).code
            assert got[i] == want, (V, i, c[1:], got[i], want)
            n += 1
    _announce(f"sampler: {n} cases bit-exact")


def test_sampler_many_uniforms_one_logit_vector():
    rng = np.random.default_rng(7)
    V, B = 4096, 512
    l = rng.standard_normal(V).astype(np.float32) * 2
    us = ((rng.integers(0, 1 << 23, size=B) + 0.5) * 2.0 ** -23).astype(np.float32)
    got = bd.sample(pr.to_dev(np.tile(l, (B, 1))), pr.to_dev(np.full(B, 0.8, np.float32)),
                    pr.to_dev(np.full(B, 0.8, np.float32)), pr.to_dev(np.full(B, 30, np.int32)),
                    pr.to_dev(us)).cpu().numpy()
    want = [sm.sample(l, 0.8, 0.8, 30, u).code for u in us]
    assert list(got) == want


# ------------------------------------------------------------------ model parity

def _frames(w, n, B):
    fr = si.make_frames(w, n_frames=n, batch=B)
    return fr


@pytest.mark.parametrize("mode", ["greedy", "sampled"])
def test_tiny_codes_and_logits(tiny, mode):
    w = si.WORKLOADS["tiny"]
    fr = _frames(w, 6, 1)
    temp = np.zeros(1, np.float32) if mode == "greedy" else fr["temperature"]
    rep = pr.FrameReport()
    for f in range(6):
        codes = pr.gpu_decode(tiny, fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f], temp,
                              fr["top_p"], fr["top_k"])
        rep = rep.add(pr.check_frame(tiny, fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f], temp,
                                     fr["top_p"], fr["top_k"], codes))
    _announce(f"tiny {mode}: 6 frames, {rep}")
    rep.assert_ok(1e-4)   # far inside the bar: float32 accumulation on both sides


def test_ragged_batch(ragged):
    w = si.WORKLOADS["ragged"]
    fr = _frames(w, 3, 3)
    rep = pr.FrameReport()
    for f in range(3):
        codes = pr.gpu_decode(ragged, fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f], fr["temperature"],
                              fr["top_p"], fr["top_k"])
        rep = rep.add(pr.check_frame(ragged, fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f],
                                     fr["temperature"], fr["top_p"], fr["top_k"], codes))
    _announce(f"ragged B=3: {rep}")
    rep.assert_ok(1e-4)


# The measured workloads, each at the size the parity protocol names: the
# batch-1 workload over its first 64 frames, batch 16 over 8 frames and
# batch 64 (with fast_project_in) over 4 frames, every request's codes and
# teacher-forced logits against the oracle.

def test_s2pro_b1_protocol(s2pro):
    """64 frames of the batch-1 workload (one launch of the batch-1 kernel
    per frame); the oracle runs the 64 frames as one batch of windows."""
    w = si.WORKLOADS["s2pro_b1"]
    F = 64
    fr = _frames(w, F, 1)
    codes = np.concatenate([pr.gpu_decode(s2pro, fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f],
                                          fr["temperature"], fr["top_p"], fr["top_k"]) for f in range(F)])
    _announce(f"s2pro B=1: {F} frames decoded; oracle pass")
    rep = pr.check_frame(s2pro, fr["hidden"][:, 0], fr["sem_code"][:, 0], fr["uniforms"][:, 0],
                         np.repeat(fr["temperature"], F), np.repeat(fr["top_p"], F), np.repeat(fr["top_k"], F),
                         codes, one_by_one=True)
    _announce(f"s2pro B=1, {F} frames: {rep}")
    rep.assert_ok(1e-4)


def test_s2pro_greedy_b2(s2pro):
    w = si.WORKLOADS["s2pro_b1"]
    fr = _frames(w, 1, 2)
    T = np.zeros(2, np.float32)
    codes = pr.gpu_decode(s2pro, fr["hidden"][0], fr["sem_code"][0], fr["uniforms"][0], T, fr["top_p"], fr["top_k"])
    rep = pr.check_frame(s2pro, fr["hidden"][0], fr["sem_code"][0], fr["uniforms"][0], T, fr["top_p"],
                         fr["top_k"], codes)
    rep.assert_ok(1e-3)


# ------------------------------------------------------------------ batched decoding
# Batches of 2..64 requests share one launch (skinny GEMMs on the matrix
# cores; a pass takes up to 128 rows in wave groups of 32, so step 1 of a
# group of 64 is one pass); larger batches run in groups of 64.

@pytest.mark.parametrize("frame", range(8))
def test_s2pro_b16_protocol(s2pro, frame):
    """Frame `frame` of the batch-16 workload (per-request temperature and
    top_p, Zipf semantic codes): all 16 requests' codes and logits."""
    w = si.WORKLOADS["s2pro_b16"]
    fr = _frames(w, frame + 1, 16)
    f = frame
    codes = pr.gpu_decode(s2pro, fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f], fr["temperature"],
                          fr["top_p"], fr["top_k"])
    rep = pr.check_frame(s2pro, fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f], fr["temperature"],
                         fr["top_p"], fr["top_k"], codes)
    _announce(f"s2pro B=16 frame {f}: {rep}")
    rep.assert_ok(1e-3)


def test_s2pro_batched_teacher_forced_all_rows(s2pro):
    """Teacher-forced logits of a full group of 64 (every row of the skinny
    GEMMs: four wave groups of 32; step 1's 128 rows in one pass)."""
    w = si.WORKLOADS["s2pro_b16"]
    fr = _frames(w, 1, 64)
    rng = np.random.default_rng(5)
    codes = rng.integers(0, w.shape.codebook_size, size=(64, w.shape.num_codebooks)).astype(np.int32)
    worst, rel, _, _ = pr.check_logits(s2pro, fr["hidden"][0], codes)
    _announce(f"s2pro B=64 teacher-forced: worst |d|/tol {worst:.2e}, |d|/max {rel:.2e}")
    assert worst <= 1.0 and rel < 1e-3, (worst, rel)


def test_two_groups_with_project_in():
    """B = 34 with project_in, first half greedy: every request."""
    w = si.WORKLOADS["s2pro_b64"]
    pair = pr.make_pair(w.shape, w.seed(0), max_batch=34)
    fr = _frames(w, 1, 34)
    assert (fr["temperature"][:17] == 0).all() and (fr["temperature"][17:] > 0).all()
    codes = pr.gpu_decode(pair, fr["hidden"][0], fr["sem_code"][0], fr["uniforms"][0], fr["temperature"],
                          fr["top_p"], fr["top_k"])
    rep = pr.check_frame(pair, fr["hidden"][0], fr["sem_code"][0], fr["uniforms"][0], fr["temperature"],
                         fr["top_p"], fr["top_k"], codes)
    _announce(f"project_in B=34: {rep}")
    rep.assert_ok(1e-3)
    pair.ctx.close()


@pytest.fixture(scope="module")
def s2pro_b64():
    _announce("s2pro model with fast_project_in (bf16)")
    w = si.WORKLOADS["s2pro_b64"]
    pair = pr.make_pair(w.shape, w.seed(0), max_batch=64)
    yield pair
    pair.ctx.close()


@pytest.mark.parametrize("frame", range(4))
def test_s2pro_b64_protocol(s2pro_b64, frame):
    """Frame `frame` of the batch-64 workload as bench.py times it (with
    fast_project_in, half greedy): all 64 requests' codes and logits."""
    w = si.WORKLOADS["s2pro_b64"]
    fr = _frames(w, frame + 1, 64)
    f = frame
    codes = pr.gpu_decode(s2pro_b64, fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f], fr["temperature"],
                          fr["top_p"], fr["top_k"])
    assert codes.shape == (64, w.shape.num_codebooks)
    rep = pr.check_frame(s2pro_b64, fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f], fr["temperature"],
                         fr["top_p"], fr["top_k"], codes)
    _announce(f"s2pro B=64 frame {f}: {rep}")
    rep.assert_ok(1e-3)


def test_tiny_f32_batched_groups():
    """float32 weights (float32 MFMA path), B = 36 = 32 + 4, mixed settings."""
    w = si.WORKLOADS["tiny"]
    pair = pr.make_pair(w.shape, w.seed(0), max_batch=36)
    fr = _frames(w, 2, 36)
    rng = np.random.default_rng(11)
    temp = rng.uniform(0.5, 1.2, size=36).astype(np.float32)
    temp[::3] = 0.0
    top_p = rng.uniform(0.5, 1.0, size=36).astype(np.float32)
    top_k = rng.integers(1, 80, size=36).astype(np.int32)
    rep = pr.FrameReport()
    for f in range(2):
        codes = pr.gpu_decode(pair, fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f], temp, top_p, top_k)
        rep = rep.add(pr.check_frame(pair, fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f], temp, top_p,
                                     top_k, codes))
    _announce(f"tiny f32 B=36: {rep}")
    rep.assert_ok(1e-4)
    pair.ctx.close()


# ------------------------------------------------------------------ weight-only int8
# int8 matrices with per-row scales (bf16 norm weights and embeddings); the
# oracle dequantizes them.  Every request runs the batch-1 kernel.

@pytest.mark.parametrize("wname,frames,B", [("tiny_q8", 6, 1), ("ragged_q8", 3, 3)])
def test_q8_small_shapes(wname, frames, B):
    w = si.WORKLOADS[wname]
    pair = pr.make_pair(w.shape, w.seed(0), max_batch=B)
    fr = _frames(w, frames, B)
    rep = pr.FrameReport()
    for f in range(frames):
        codes = pr.gpu_decode(pair, fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f], fr["temperature"],
                              fr["top_p"], fr["top_k"])
        rep = rep.add(pr.check_frame(pair, fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f],
                                     fr["temperature"], fr["top_p"], fr["top_k"], codes))
    _announce(f"{wname}: {rep}")
    rep.assert_ok(1e-4)
    pair.ctx.close()


def test_q8_s2pro_protocol():
    """16 frames of the int8 S2 Pro model at batch 1 (the batch-1
    workload's settings), codes and teacher-forced logits; the oracle runs
    them as one batch of windows."""
    w = si.WORKLOADS["s2pro_q8"]
    pair = pr.make_pair(w.shape, w.seed(0), max_batch=1)
    F = 16
    fr = _frames(w, F, 1)
    codes = np.concatenate([pr.gpu_decode(pair, fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f],
                                          fr["temperature"], fr["top_p"], fr["top_k"]) for f in range(F)])
    rep = pr.check_frame(pair, fr["hidden"][:, 0], fr["sem_code"][:, 0], fr["uniforms"][:, 0],
                         np.repeat(fr["temperature"], F), np.repeat(fr["top_p"], F), np.repeat(fr["top_k"], F),
                         codes, one_by_one=True)
    _announce(f"s2pro q8 B=1, {F} frames: {rep}")
    rep.assert_ok(1e-4)
    pair.ctx.close()


# ------------------------------------------------------------------ behaviour

def test_deterministic(tiny):
    fr = _frames(si.WORKLOADS["tiny"], 1, 2)
    a = pr.gpu_decode(tiny, fr["hidden"][0], fr["sem_code"][0], fr["uniforms"][0], fr["temperature"],
                      fr["top_p"], fr["top_k"])
    b = pr.gpu_decode(tiny, fr["hidden"][0], fr["sem_code"][0], fr["uniforms"][0], fr["temperature"],
                      fr["top_p"], fr["top_k"])
    assert np.array_equal(a, b)
    la = pr.gpu_forward_logits(tiny, fr["hidden"][0], a)
    lb = pr.gpu_forward_logits(tiny, fr["hidden"][0], a)
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))


def test_sem_code_is_clamped(tiny):
    fr = _frames(si.WORKLOADS["tiny"], 1, 2)
    V = si.TINY.codebook_size
    sem = np.array([-5, V + 10], np.int32)
    codes = pr.gpu_decode(tiny, fr["hidden"][0], sem, fr["uniforms"][0], np.zeros(2, np.float32),
                          fr["top_p"], fr["top_k"])
    assert list(codes[:, 0]) == [0, V - 1]
    pr.check_frame(tiny, fr["hidden"][0], sem, fr["uniforms"][0], np.zeros(2, np.float32), fr["top_p"],
                   fr["top_k"], codes).assert_ok(1e-4)


def test_batch_limits(tiny):
    fr = _frames(si.WORKLOADS["tiny"], 1, 5)
    with pytest.raises(bd.S2FastError) as e:
        pr.gpu_decode(tiny, fr["hidden"][0], fr["sem_code"][0], fr["uniforms"][0], fr["temperature"],
                      fr["top_p"], fr["top_k"])
    assert e.value.code == 5
