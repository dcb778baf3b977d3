"""Helpers shared by the GPU parity tests: build a model on both sides from
one seeded weight draw, and compare the HIP path with the oracle."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from dual_ar_neural_amd import binding as bd
from oracle import fast_ar as fa
from oracle import sampler as sm
from synth import inputs as si


@dataclass
class Pair:
    shape: object
    host: dict
    oracle: fa.Model
    dev: dict
    ctx: bd.FastAR


def make_pair(shape, seed: int, max_batch: int) -> Pair:
    host = si.make_weights(shape, seed)
    dev = bd.device_weights(shape, host)
    ctx = bd.FastAR(shape, dev, max_batch=max_batch)
    return Pair(shape, host, fa.Model.from_weights(shape, host), dev, ctx)


def logit_tolerance(ref: np.ndarray) -> float:
    """|delta| <= 1e-2 * max|logit| + 1e-3 (per call)."""
    return 1e-2 * float(np.max(np.abs(ref))) + 1e-3


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def gpu_forward_logits(p: Pair, hidden: np.ndarray, codes: np.ndarray) -> np.ndarray:
    out = p.ctx.forward_logits(to_dev(hidden, torch.float32), to_dev(codes.astype(np.int32)))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def gpu_decode(p: Pair, hidden, sem, uniforms, temperature, top_p, top_k) -> np.ndarray:
    out = p.ctx.decode_frame(to_dev(hidden, torch.float32), to_dev(np.asarray(sem, np.int32)),
                             to_dev(uniforms, torch.float32), to_dev(temperature, torch.float32),
                             to_dev(top_p, torch.float32), to_dev(np.asarray(top_k, np.int32)))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_logits(p: Pair, hidden: np.ndarray, codes: np.ndarray):
    """Teacher-forced logits of every step vs the oracle; returns the worst
    |delta| / tolerance ratio and the worst |delta| / max|logit|."""
    got = gpu_forward_logits(p, hidden, codes)
    ref = fa.decode_frame(p.oracle, hidden, codes[:, 0], np.full((len(codes), p.shape.n_steps), 0.5, np.float32),
                          np.zeros(len(codes), np.float32), np.ones(len(codes), np.float32),
                          np.full(len(codes), 30, np.int32), forced=codes).logits
    worst, worst_rel = logit_errors(got, ref)
    return worst, worst_rel, got, ref


def logit_errors(got: np.ndarray, ref: np.ndarray):
    """Worst |delta| / tolerance and worst |delta| / max|logit| over calls."""
    worst, worst_rel = 0.0, 0.0
    for b in range(ref.shape[0]):
        for k in range(ref.shape[1]):
            d = float(np.max(np.abs(got[b, k] - ref[b, k])))
            worst = max(worst, d / logit_tolerance(ref[b, k]))
            worst_rel = max(worst_rel, d / float(np.max(np.abs(ref[b, k]))))
    return worst, worst_rel


# At most this share of draws may come out as the oracle's alternative
# rather than its own code (plus one).  The GPU's logits differ from the
# oracle's by about 1e-6 of their largest magnitude, a hundred times less
# than the smallest margin, so a legitimate flip is rare even among the
# draws the oracle marks.
EXCUSED_SHARE = 0.02


@dataclass
class FrameReport:
    draws: int = 0         # decode steps compared
    marked: int = 0        # draws with more than one defensible code
    excused: int = 0       # draws where the GPU took a defensible alternative
    worst: float = 0.0     # worst |delta logit| / tolerance
    worst_rel: float = 0.0  # worst |delta logit| / max|logit|

    def add(self, o: "FrameReport") -> "FrameReport":
        return FrameReport(self.draws + o.draws, self.marked + o.marked, self.excused + o.excused,
                           max(self.worst, o.worst), max(self.worst_rel, o.worst_rel))

    def assert_ok(self, rel_bound: float):
        assert self.excused <= self.marked, self
        assert self.excused <= EXCUSED_SHARE * self.draws + 1, self
        assert self.worst <= 1.0 and self.worst_rel < rel_bound, self


def check_frame(p: Pair, hidden, sem, uniforms, temperature, top_p, top_k, gpu_codes,
                logits: bool = True, one_by_one: bool = False) -> FrameReport:
    """One frame of B requests decoded on the GPU, against one oracle pass
    teacher-forced along the GPU's own codes: at every step the oracle
    computes the logits of the GPU's prefix and the draw from them, and the
    GPU's code must be one of that draw's defensible codes (the oracle's own
    code unless a decision sits within a margin).  With `logits`, the GPU's
    teacher-forced logits of the same prefixes are compared with the
    oracle's; `one_by_one` runs them one request per call (the batch-1
    kernel) instead of as one batch.  Raises AssertionError on a code
    outside the set."""
    V = p.shape.codebook_size
    gpu_codes = np.asarray(gpu_codes)
    B = len(gpu_codes)
    c0 = np.clip(np.asarray(sem, np.int64), 0, V - 1)
    assert np.array_equal(gpu_codes[:, 0], c0), (gpu_codes[:, 0], c0)
    ref = fa.decode_frame(p.oracle, hidden, sem, uniforms, temperature, top_p, top_k, forced=gpu_codes)
    rep = FrameReport()
    for b in range(B):
        for k in range(1, p.shape.num_codebooks):
            g = int(gpu_codes[b, k])
            alts = ref.alts[b][k - 1]
            assert g in alts, f"request {b} step {k}: gpu {g}, oracle {ref.codes[b, k]}, defensible {alts}"
            rep.draws += 1
            rep.marked += len(alts) > 1
            rep.excused += g != int(ref.codes[b, k])
    if logits:
        gc = gpu_codes.astype(np.int32)
        if one_by_one:
            got = np.concatenate([gpu_forward_logits(p, hidden[b:b + 1], gc[b:b + 1]) for b in range(B)])
        else:
            got = gpu_forward_logits(p, hidden, gc)
        rep.worst, rep.worst_rel = logit_errors(got, ref.logits)
    return rep


def check_codes(p: Pair, hidden, sem, uniforms, temperature, top_p, top_k, gpu_codes):
    """Codes only (see check_frame); returns the number of excused draws."""
    return check_frame(p, hidden, sem, uniforms, temperature, top_p, top_k, gpu_codes, logits=False).excused
