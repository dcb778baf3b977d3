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

Besides the code, a draw reports every code another implementation may
defensibly return when its logits differ from these in the last bits (the
margins below): the parity tests accept exactly those.

Pins (tests/test_oracle_sampler.py): SplitMix64 against the published
reference sequence; greedy/T->0+/top_k=1/top_p->0+ all reduce to argmax;
the code is always inside the top-k set; the kept set is the minimal prefix;
draw frequencies match p_j (chi-square); draws on slightly perturbed logits
always land in the reported set, which is the code alone away from the
margins.
"""
from __future__ import annotations

import itertools
from dataclasses import dataclass

import numpy as np

F32 = np.float32
MASK64 = (1 << 64) - 1
TOPK_MAX = 64

# Margins below which a decision is reported as a knife-edge: an
# implementation whose logits differ from these in the last bits may take the
# other side of such a decision.  Each margin names the alternative it
# allows (see `sample`).
GREEDY_GAP = 1.0e-3      # any logit within this of the maximum may be the argmax
ORDER_GAP = 1.0e-3       # two logits closer than this may rank either way
                         # (this covers the top-k boundary: rank n-1 against rank n)
TOPP_GAP = 1.0e-4        # |c_j - top_p| at the nucleus boundary: rank j kept or dropped
RACE_GAP = 1.0e-4        # relative gap between the two best race keys: either wins


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
    alts: tuple = ()       # every defensible code (sorted; always holds `code`)


def greedy(logits: np.ndarray) -> Draw:
    """argmax, lowest index on ties; every index whose logit is within
    GREEDY_GAP of the maximum is a defensible alternative."""
    l = np.asarray(logits, dtype=F32)
    code = int(np.argmax(l))              # first occurrence = lowest index
    alts = tuple(int(i) for i in np.flatnonzero(l.astype(np.float64) >= float(l[code]) - GREEDY_GAP))
    if code not in alts:                  # NaN-free inputs always hold it; keep the invariant regardless
        alts = tuple(sorted(set(alts) | {code}))
    return Draw(code, len(alts) > 1, alts=alts)


def rank_order(l: np.ndarray) -> np.ndarray:
    """Indices ordered by (value descending, index ascending)."""
    return np.argsort(-l, kind="stable")


def _nucleus(lv: np.ndarray, T, top_p):
    """Steps 3-4 on candidate logits lv given in rank order: float32
    probabilities p, running sums cum and the last kept rank m."""
    n = lv.size
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
    for j in range(n):
        c = F32(c + p[j])
        cum[j] = c
    m = n - 1
    for j in range(n):
        if cum[j] >= tp:
            m = j
            break
    return p, cum, m


def _race(p: np.ndarray, E: np.ndarray, m: int):
    """Step 6 over ranks 0..m: the winning rank, and the runner-up rank when
    its key is within RACE_GAP (relative) of the winner's, else None."""
    key = (p[: m + 1] / E[: m + 1]).astype(F32)
    best = int(np.argmax(key))            # first occurrence = lowest rank
    runner = None
    if m > 0:
        k2 = key.astype(np.float64).copy()
        k2[best] = -np.inf
        r = int(np.argmax(k2))
        if float(key[best]) - float(key[r]) <= RACE_GAP * float(key[best]):
            runner = r
    return best, runner


def _order_variants(l: np.ndarray, order: np.ndarray, n: int):
    """Rank orders an implementation with slightly different logits may
    see: in every run of consecutive ranked logits whose neighbours differ by
    less than ORDER_GAP and that reaches into the first n ranks (or across
    the boundary at rank n), each permutation of the run (runs of up to four
    logits; longer runs: each swap of two of its members).  Only one run is
    disturbed at a time.  Yields the first n indices of each variant."""
    V = l.size
    lim = min(V, n + TOPK_MAX + 1)
    lv = l[order[:lim]].astype(np.float64)
    j = 0
    while j < min(n, lim - 1):
        a = j
        while j + 1 < lim and lv[j] - lv[j + 1] < ORDER_GAP:
            j += 1
        b = j                                  # run [a, b]
        j += 1
        if b == a:
            continue
        run = list(order[a:b + 1])
        if len(run) <= 4:
            perms = [list(q) for q in itertools.permutations(run) if list(q) != run]
        else:
            # pairs of members (adjacent pairs only in runs longer than 16)
            perms = []
            for x in range(len(run)):
                for y in range(x + 1, len(run) if len(run) <= 16 else min(x + 2, len(run))):
                    q = list(run)
                    q[x], q[y] = q[y], q[x]
                    perms.append(q)
        for q in perms:
            var = np.array(order[:lim])
            var[a:b + 1] = q
            yield var[:n]


def sample(logits, temperature, top_p, top_k, u) -> Draw:
    """Draw one code from a request's logits (steps 1-6 of the header).

    The draw also reports every code that is defensible for logits which
    differ from these by less than the margins above: the draws under each
    rank order of near-equal logits (`_order_variants`; the top-k boundary
    is the pair at ranks n-1 and n), each with the nucleus cut one rank
    earlier or later where a running sum lies within TOPP_GAP of top_p, and
    the race's runner-up where its key is within RACE_GAP of the winner's."""
    l = np.asarray(logits, dtype=F32)
    V = l.size
    T = F32(temperature)
    if not (T > 0):
        return greedy(l)
    n = int(min(max(int(top_k), 1), min(V, TOPK_MAX)))
    order = rank_order(l)
    ranks = order[:n]
    tp = F32(top_p)
    E = np.array([candidate_exponential(u, j) for j in range(n)], dtype=F32)
    p, cum, m = _nucleus(l[ranks], T, tp)
    best, _ = _race(p, E, m)
    code = int(ranks[best])

    alts = set()
    for cand in [ranks] + list(_order_variants(l, order, n)):
        pv, cv, mv = _nucleus(l[cand], T, tp)
        cuts = {mv}
        if mv + 1 < n and abs(float(cv[mv]) - float(tp)) < TOPP_GAP:
            cuts.add(mv + 1)
        if mv > 0 and abs(float(cv[mv - 1]) - float(tp)) < TOPP_GAP:
            cuts.add(mv - 1)
        for mm in cuts:
            b, r = _race(pv, E, mm)
            alts.add(int(cand[b]))
            if r is not None:
                alts.add(int(cand[r]))
    alts.add(code)
    alts = tuple(sorted(alts))
    return Draw(code, len(alts) > 1, m + 1, ranks, alts)
