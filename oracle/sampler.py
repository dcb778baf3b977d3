"""Oracle sampler: turns one request's Fast-AR logits into the next code.

TEST INFRASTRUCTURE ONLY (see the package header).

What the pages fix (Mizuoto "Fish Speech" engine page, sections
"What matches upstream" and "Limitations"): a draw is argmax(probs / -log(u)); top-k is fixed at 30;
temperature and top-p are per request.  The s2.cpp sampler chapter is not
among the pages, so the order and the tie/rounding details below are this
oracle's stated reading:

  1. temperature <= 0 (or NaN) decodes greedily: argmax of the raw logits,
     lowest index on ties.
  2. n = clamp(top_k, 1, min(V, 64)); the candidates are the n largest
     logits ordered by (value descending, index ascending).
  3. z_j = l_j / T in float32; e_j = f32(exp(f64(z_j - z_0))); S is the
     float32 sum of e_j taken in rank order; p_j = e_j / S in float32.
  4. Nucleus (Holtzman et al. 2020): running float32 sums c_j in rank order;
     keep ranks 0..m with m = min{j : c_j >= top_p}, or n-1 if none.
  5. One exponential per kept candidate, from the caller's single uniform u:
     u_j = (floor(splitmix64(bits(u) * 2^32 + j) / 2^40) + 0.5) * 2^-24
     (float64), E_j = f32(-log(u_j)).  SplitMix64 is Steele, Lea & Flood,
     "Fast splittable pseudorandom number generators", OOPSLA 2014.
  6. The code is the kept candidate with the largest float32 p_j / E_j,
     lowest rank on ties.  With independent Exp(1) variables E_j this picks
     candidate j with probability p_j / sum(kept p) (the exponential race).

Pins (tests/test_oracle_sampler.py): SplitMix64 against the published
reference sequence; greedy/T->0+/top_k=1/top_p->0+ all reduce to argmax;
the code is always inside the top-k set; the kept set is the minimal prefix;
draw frequencies match p_j (chi-square).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F32 = np.float32
MASK64 = (1 << 64) - 1
TOPK_MAX = 64

# Margins below which a decision is reported as a knife-edge: a legitimately
# different code may come out of an implementation whose logits differ from
# these in the last bits.
GREEDY_GAP = 1.0e-3      # absolute logit gap between the top two (greedy)
TOPK_GAP = 1.0e-3        # absolute logit gap at the top-k boundary
TOPP_GAP = 1.0e-4        # |c_j - top_p| at the nucleus boundary
RACE_GAP = 1.0e-4        # relative gap between the two best race keys


def splitmix64(x: int) -> int:
    """One SplitMix64 output for state `x` (add the golden gamma, then the
    two xor-shift-multiply rounds and a final xor-shift), all mod 2^64."""
    z = (x + 0x9E3779B97F4A7C15) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def f32_bits(u) -> int:
    return int(np.asarray(u, dtype=F32).reshape(()).view(np.uint32))


def candidate_uniform(u, j: int) -> float:
    """Per-candidate uniform u_j in (0,1), float64, from the caller's u."""
    h = splitmix64((f32_bits(u) << 32) + j)
    return (float(h >> 40) + 0.5) * 2.0 ** -24


def candidate_exponential(u, j: int) -> np.float32:
    return F32(-np.log(np.float64(candidate_uniform(u, j))))


@dataclass
class Draw:
    code: int
    fragile: bool          # knife-edge: another code is also defensible
    kept: int = 0          # number of kept candidates (m + 1); 0 for greedy
    ranks: np.ndarray = None  # candidate indices in rank order (sampled only)


def greedy(logits: np.ndarray) -> Draw:
    l = np.asarray(logits, dtype=F32)
    code = int(np.argmax(l))              # first occurrence = lowest index
    top2 = np.sort(l)[-2:] if l.size > 1 else np.array([l[0], -np.inf], F32)
    fragile = bool(l.size > 1 and float(top2[1]) - float(top2[0]) < GREEDY_GAP)
    return Draw(code, fragile)


def rank_order(l: np.ndarray) -> np.ndarray:
    """Indices ordered by (value descending, index ascending)."""
    return np.argsort(-l, kind="stable")


def sample(logits, temperature, top_p, top_k, u) -> Draw:
    """Draw one code from a request's logits (steps 1-6 of the header)."""
    l = np.asarray(logits, dtype=F32)
    V = l.size
    T = F32(temperature)
    if not (T > 0):
        return greedy(l)
    n = int(min(max(int(top_k), 1), min(V, TOPK_MAX)))
    order = rank_order(l)
    ranks = order[:n]
    lv = l[ranks]
    z = (lv / T).astype(F32)
    d = (z - z[0]).astype(F32)
    e = np.exp(d.astype(np.float64)).astype(F32)
    S = F32(0.0)
    for j in range(n):
        S = F32(S + e[j])
    p = (e / S).astype(F32)
    tp = F32(top_p)
    c = F32(0.0)
    cum = np.empty(n, F32)
    m = n - 1
    for j in range(n):
        c = F32(c + p[j])
        cum[j] = c
    for j in range(n):
        if cum[j] >= tp:
            m = j
            break
    E = np.array([candidate_exponential(u, j) for j in range(m + 1)], dtype=F32)
    key = (p[: m + 1] / E).astype(F32)
    best = int(np.argmax(key))            # first occurrence = lowest rank

    # knife-edge report
    fragile = False
    if n < V:
        nxt = l[order[n]]
        fragile |= float(lv[-1]) - float(nxt) < TOPK_GAP
    fragile |= abs(float(cum[m]) - float(tp)) < TOPP_GAP
    if m > 0:
        fragile |= abs(float(cum[m - 1]) - float(tp)) < TOPP_GAP
    if m > 0:
        srt = np.sort(key)
        fragile |= (float(srt[-1]) - float(srt[-2])) <= RACE_GAP * float(srt[-1])
    return Draw(int(ranks[best]), bool(fragile), m + 1, ranks)


def sample_batch(logits, temperature, top_p, top_k, u):
    """Row-wise `sample` over a batch: logits [B,V], settings [B], u [B]."""
    return [sample(logits[b], temperature[b], top_p[b], top_k[b], u[b])
            for b in range(len(logits))]
