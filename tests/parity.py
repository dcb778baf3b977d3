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
    worst, worst_rel = 0.0, 0.0
    for b in range(len(codes)):
        for k in range(p.shape.n_steps):
            d = float(np.max(np.abs(got[b, k] - ref[b, k])))
            worst = max(worst, d / logit_tolerance(ref[b, k]))
            worst_rel = max(worst_rel, d / float(np.max(np.abs(ref[b, k]))))
    return worst, worst_rel, got, ref


def check_codes(p: Pair, hidden, sem, uniforms, temperature, top_p, top_k, gpu_codes):
    """Walk the oracle along the GPU's codes.  A step must match exactly
    unless the oracle reports that decision as a knife-edge; after an excused
    difference the walk continues on the GPU's code.  Returns the number of
    excused steps; raises AssertionError on a real mismatch."""
    V = p.shape.codebook_size
    excused = 0
    for b in range(len(gpu_codes)):
        c0 = int(np.clip(sem[b], 0, V - 1))
        assert gpu_codes[b, 0] == c0, (b, gpu_codes[b, 0], c0)
        prefix = [c0]
        for k in range(1, p.shape.num_codebooks):
            lg = fa.fast_forward(p.oracle, hidden[b:b + 1], np.array([prefix]))[0]
            d = sm.sample(lg, temperature[b], top_p[b], top_k[b], uniforms[b][k - 1])
            g = int(gpu_codes[b, k])
            if g != d.code:
                assert d.fragile, f"request {b} step {k}: gpu {g} oracle {d.code} (not a knife-edge)"
                excused += 1
            prefix.append(g)
    return excused
