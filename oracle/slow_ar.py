"""Oracle Slow-AR decode step and full Dual-AR frame.

TEST INFRASTRUCTURE ONLY (see the package header).

Plain float32 numpy, one request at a time.  What it follows:
  * input of a position: sem_scale * embeddings[main token] plus, for a
    position that carries codes, codebook_embeddings[j * codebook_size +
    code_j] summed over the codebooks j; sem_scale = 1/sqrt(num_codebooks+1)
    ("Overall architecture & Dual-AR data flow", section 3.2);
  * 36 pre-norm layers of the same block as Fast-AR (RMSNorm, fused wqkv,
    per-head q/k RMSNorm, pair RoPE, GQA attention, wo, SwiGLU; same
    section), attending over the KV cache of every earlier position plus
    the new one (section 3.4: the cache keeps the whole history);
  * hidden = RMSNorm(last position, norm) and tied logits hidden x
    embeddings^T (section 3.2);
  * sem_mask: -inf except the semantic ids and the end id; main token drawn
    from logits + sem_mask ("Fast-AR codebook decoding and the generation
    main loop", section 5);
  * repetition-aware sampling: a semantic main token already in the window
    of the last 10 main tokens is redrawn at temperature 1.0, top_p 0.9 from
    the same masked logits; every frame pushes its main token and the window
    keeps the newest 10 (section 6);
  * sem_code = main token - semantic_begin, clamped (section 5.2), then the
    nine Fast-AR draws on the Slow-AR hidden state (section 5.1).

Readings of points the pages leave open:
  * the codebook index j runs 0..num_codebooks-1 over the frame's codes
    c_0..c_9 (the shared table has num_codebooks * codebook_size rows);
  * sem_scale multiplies the semantic embedding only, as the formula on the
    architecture page and the measured configuration write it (the engine
    page's remark that inference scales the codebook embeddings is not
    followed);
  * a position's codebook terms count exactly when its row-0 token is a
    semantic id (the mask of the prompt matrix: codes are present only in
    reference-audio positions; every generated frame's main token is
    semantic);
  * prefill runs the prompt's positions through the same cached step one
    at a time (the engine's CUDA path takes one token per chunk; any chunk
    size gives the same result), and only the last position's logits feed
    the first main-token draw;
  * the KV cache stores keys after q/k-norm and RoPE; new entries are
    rounded to the cache type (bf16 for bf16 models) before the attention
    reads them;
  * the hidden state handed to Fast-AR is the normalised one the tied head
    reads;
  * the main draw uses the request's temperature / top_p / top_k, the
    redraw temperature 1.0, top_p 0.9 and the same top_k; the two draws
    take separate caller uniforms;
  * the end id is a parameter (the pages name im_end without its id);
    repetition checks skip it; a frame whose main token is the end id
    still runs its Fast-AR draws (the caller stops the loop).

Pins: tests/test_oracle_slow.py.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from . import fast_ar as _fa
from . import sampler as _sampler

F32 = np.float32
RAS_WINDOW = 10
RAS_TEMPERATURE = 1.0
RAS_TOP_P = 0.9


@dataclass
class SlowModel:
    """Shape hyper-parameters plus weights keyed by tensor name, float32 or
    bf16 bits; each access widens to float32 (the 36-layer model is kept in
    its storage type and widened one tensor at a time)."""
    shape: object
    w: Dict[str, np.ndarray]

    @classmethod
    def from_weights(cls, shape, weights: Dict[str, np.ndarray]) -> "SlowModel":
        return cls(shape, dict(weights))

    def get(self, name: str) -> np.ndarray:
        return _fa.as_f32_weight(self.w[name])

    def row(self, name: str, r: int) -> np.ndarray:
        return _fa.as_f32_weight(self.w[name][r])

    def layer(self, i: int, name: str) -> np.ndarray:
        return self.get(f"layers.{i}.{name}")


def bf16_round_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32."""
    b = np.ascontiguousarray(x, dtype=F32).view(np.uint32)
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)) << np.uint32(16)
    return r.view(F32)


def cache_round(shape, x: np.ndarray) -> np.ndarray:
    return bf16_round_f32(x) if shape.weight_dtype == "bf16" else np.asarray(x, dtype=F32)


# Two implementations whose float32 sums run in different orders compute
# keys and values that differ by about 1e-6 of the vector's largest
# magnitude (the error of a dot product scales with its terms, not with its
# result).  A cache entry is a defensible rounding when it is the bfloat16
# rounding of some float32 value within ROUND_BAND times that magnitude of
# the oracle's value.
ROUND_BAND = 1.0e-5


class CacheFollowError(AssertionError):
    """A followed cache entry is not a defensible rounding of the oracle's
    value."""


def follow_rounding(shape, exact: np.ndarray, theirs: np.ndarray):
    """The cache entries to continue with when another implementation wrote
    `theirs` for the float32 values `exact` (one layer's keys or values): its
    entries, provided each one lies between the bfloat16 roundings of
    exact - band and exact + band, band = ROUND_BAND * max|exact| (rounding
    is monotone, so those are exactly the roundings of values within the
    band).  float32 caches are not rounded, so their entries are compared,
    not followed (the oracle's values are returned).  Returns (entries,
    number of entries that differ from the oracle's rounding); raises
    CacheFollowError otherwise."""
    exact = np.asarray(exact, dtype=F32)
    mine = cache_round(shape, exact)
    if shape.weight_dtype != "bf16":
        return mine, 0
    theirs = np.asarray(theirs, dtype=F32)
    band = ROUND_BAND * float(np.max(np.abs(exact))) if exact.size else 0.0
    e64 = exact.astype(np.float64)
    lo = bf16_round_f32((e64 - band).astype(F32)).astype(np.float64)
    hi = bf16_round_f32((e64 + band).astype(F32)).astype(np.float64)
    t64 = theirs.astype(np.float64)
    is_bf16 = (theirs.view(np.uint32) & np.uint32(0xFFFF)) == 0
    ok = is_bf16 & (t64 >= lo) & (t64 <= hi)
    if not ok.all():
        i = np.flatnonzero(~ok.reshape(-1))[0]
        raise CacheFollowError(f"entry {i}: exact {exact.reshape(-1)[i]!r}, theirs {theirs.reshape(-1)[i]!r}, "
                               f"oracle {mine.reshape(-1)[i]!r}, band {band:.3g}")
    same = theirs.view(np.uint32) == mine.view(np.uint32)
    return theirs.copy(), int((~same).sum())


# --------------------------------------------------------------------------
# input, mask, head
# --------------------------------------------------------------------------

def is_semantic(shape, token) -> bool:
    return shape.sem_begin <= int(token) <= shape.sem_end


def combine(model: SlowModel, main_token: int, codes) -> np.ndarray:
    """Input vector of one position [dim] (architecture page, section 3.2):
    the row-0 token's embedding scaled by sem_scale, plus the codebook rows
    when the position carries codes (its row-0 token is a semantic id)."""
    s = model.shape
    codes = np.asarray(codes, dtype=np.int64)
    assert codes.shape == (s.num_codebooks,)
    scale = F32(1.0 / np.sqrt(np.float64(s.num_codebooks + 1)))
    x = scale * model.row("embeddings", int(main_token))
    if is_semantic(s, main_token):
        rows = np.arange(s.num_codebooks) * s.codebook_size + codes
        for r in rows:
            x = x + model.row("codebook_embeddings", int(r))
    return x.astype(F32)


def sem_mask(shape) -> np.ndarray:
    """0 at the semantic ids and the end id, -inf elsewhere [vocab]
    (main-loop page, section 5)."""
    m = np.full(shape.vocab, -np.inf, dtype=F32)
    m[shape.sem_begin: shape.sem_end + 1] = 0.0
    m[shape.end_id] = 0.0
    return m


def allowed_ids(shape) -> np.ndarray:
    """The ids sem_mask leaves finite, ascending."""
    return np.flatnonzero(np.isfinite(sem_mask(shape)))


def sem_code(shape, main_token) -> int:
    return int(_fa.clamp_sem_code(int(main_token) - shape.sem_begin, shape.codebook_size))


# --------------------------------------------------------------------------
# the cached decode step
# --------------------------------------------------------------------------

def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """One query position over n cached positions: q [H, hd], K/V [G, n, hd]
    -> [H * hd].  Query head h reads KV head h // (H / G); scale
    1/sqrt(hd); every cached position is visible (the new position is the
    last one, so the causal mask hides nothing)."""
    H, hd = q.shape
    G = K.shape[0]
    out = np.empty((H, hd), dtype=F32)
    scale = F32(1.0 / np.sqrt(hd))
    for h in range(H):
        g = h // (H // G)
        sc = (K[g] @ q[h]) * scale             # [n]
        e = np.exp(sc - np.max(sc))
        p = e / np.sum(e)
        out[h] = p @ V[g]
    return out.reshape(H * hd)


@dataclass
class StepResult:
    hidden: np.ndarray       # [dim] RMSNorm(x_last, norm): the tied head's input
    logits: np.ndarray       # [vocab] unmasked tied logits
    kv_new: np.ndarray       # [n_layer, n_head_kv, 2, head_dim] entries written at position n_past
    flips: int = 0           # followed entries that took the other bf16 neighbour


def step(model: SlowModel, x: np.ndarray, kv: np.ndarray, n_past: int,
         follow: Optional[np.ndarray] = None) -> StepResult:
    """One Slow-AR position at index n_past over a cache holding positions
    0..n_past-1.  kv: [n_layer, n_head_kv, >= n_past, 2, head_dim] float32
    (key then value); it is not modified.  With `follow` ([n_layer,
    n_head_kv, 2, head_dim], the entries another implementation wrote at
    n_past) the step continues with those entries wherever they are a
    defensible rounding of this step's values (follow_rounding), so that a
    comparison tracks that implementation's rounding decisions."""
    s = model.shape
    H, G, hd = s.n_head, s.n_head_kv, s.head_dim
    cos, sin = _fa.rope_table(hd, n_past + 1, s.rope_base)
    cos, sin = cos[n_past:n_past + 1], sin[n_past:n_past + 1]
    x = np.asarray(x, dtype=F32)
    kv_new = np.zeros((s.n_layer, G, 2, hd), dtype=F32)
    flips = 0
    for i in range(s.n_layer):
        a = _fa.rms_norm(x, model.layer(i, "attention_norm"), s.norm_eps)
        qkv = _fa.linear(a, model.layer(i, "attention.wqkv"))
        q = qkv[: H * hd].reshape(1, H, hd)
        k = qkv[H * hd: (H + G) * hd].reshape(1, G, hd)
        v = qkv[(H + G) * hd:].reshape(G, hd)
        if s.has_qk_norm:
            q = _fa.rms_norm(q, model.layer(i, "attention.q_norm"), s.norm_eps)
            k = _fa.rms_norm(k, model.layer(i, "attention.k_norm"), s.norm_eps)
        q = _fa.apply_rope(q, cos, sin)[0]
        k = _fa.apply_rope(k, cos, sin)[0]
        if follow is None:
            kv_new[i, :, 0] = cache_round(s, k)
            kv_new[i, :, 1] = cache_round(s, v)
        else:
            try:
                kv_new[i, :, 0], f0 = follow_rounding(s, k, follow[i, :, 0])
                kv_new[i, :, 1], f1 = follow_rounding(s, v, follow[i, :, 1])
            except CacheFollowError as e:
                raise CacheFollowError(f"position {n_past}, layer {i}: {e}") from None
            flips += f0 + f1
        K = np.concatenate([kv[i, :, :n_past, 0], kv_new[i, :, None, 0]], axis=1)
        V = np.concatenate([kv[i, :, :n_past, 1], kv_new[i, :, None, 1]], axis=1)
        o = attend(q, K, V)
        x = x + _fa.linear(o, model.layer(i, "attention.wo"))
        n = _fa.rms_norm(x, model.layer(i, "ffn_norm"), s.norm_eps)
        g = _fa.silu(_fa.linear(n, model.layer(i, "feed_forward.w1"))) * _fa.linear(n, model.layer(i, "feed_forward.w3"))
        x = (x + _fa.linear(g, model.layer(i, "feed_forward.w2"))).astype(F32)
    h = _fa.rms_norm(x, model.get("norm"), s.norm_eps).astype(F32)
    logits = _fa.linear(h, model.get("embeddings")).astype(F32)
    return StepResult(h, logits, kv_new, flips)


def prefill(model: SlowModel, tokens, kv: np.ndarray, n_past0: int, follow: Optional[np.ndarray] = None):
    """The prompt's positions n_past0 .. n_past0 + T - 1 (tokens [T, 1 +
    num_codebooks]: row-0 token, then the codebook codes) through the cached
    step in order; `kv` receives every new entry.  Returns the last
    position's StepResult ("Overall architecture & Dual-AR data flow",
    section 4: prefill in chunks, one token per chunk on CUDA; main-loop
    page, section 5: the first main token is drawn from the prefill
    logits)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    st = None
    flips = 0
    for t in range(tokens.shape[0]):
        x = combine(model, tokens[t, 0], tokens[t, 1:])
        st = step(model, x, kv, n_past0 + t, None if follow is None else follow[:, :, t])
        kv[:, :, n_past0 + t] = st.kv_new
        flips += st.flips
    st.flips = flips
    return st


# --------------------------------------------------------------------------
# main-token draw with repetition-aware resampling
# --------------------------------------------------------------------------

@dataclass
class MainDraw:
    token: int
    first: int               # the draw before any repetition resample
    resampled: bool
    fragile: bool
    alts: tuple = ()         # every defensible main token (see sampler.sample)


def draw_main(shape, logits: np.ndarray, window: List[int], temperature, top_p, top_k,
              u_main, u_ras) -> MainDraw:
    """Main token from logits + sem_mask; a semantic token already in
    `window` is redrawn at temperature 1.0 / top_p 0.9 (main-loop page,
    sections 5 and 6).  `window` is not modified.  The defensible tokens
    follow each defensible first draw through the repetition check."""
    masked = (np.asarray(logits, dtype=F32) + sem_mask(shape)).astype(F32)
    d = _sampler.sample(masked, temperature, top_p, top_k, u_main)
    repeats = lambda t: shape.sem_begin <= t <= shape.sem_end and t in window
    d2 = None
    if any(repeats(a) for a in d.alts):
        d2 = _sampler.sample(masked, F32(RAS_TEMPERATURE), F32(RAS_TOP_P), top_k, u_ras)
    first = d.code
    tok, resampled = first, False
    if repeats(first):
        tok, resampled = d2.code, True
    alts = set()
    for a in d.alts:
        alts |= set(d2.alts) if repeats(a) else {a}
    alts = tuple(sorted(alts))
    return MainDraw(int(tok), int(first), resampled, len(alts) > 1, alts)


def push_window(window: List[int], token: int) -> List[int]:
    """The window after a frame: newest last, at most RAS_WINDOW entries."""
    w = list(window) + [int(token)]
    return w[-RAS_WINDOW:]


# --------------------------------------------------------------------------
# the full frame
# --------------------------------------------------------------------------

@dataclass
class FrameResult:
    main: MainDraw
    sem_code: int
    hidden: np.ndarray       # [dim]
    codes: np.ndarray        # [num_codebooks] int32 Fast-AR output [sem_code, c_1..c_9]
    fast_fragile: np.ndarray
    kv_new: np.ndarray
    window: List[int]
    logits: np.ndarray       # [vocab] unmasked
    fast_alts: list = None   # [n_steps] tuples: every defensible code of each Fast-AR draw


def decode_frame(slow: SlowModel, fast: "_fa.Model", kv: np.ndarray, n_past: int, prev_main: int, prev_codes,
                 window: List[int], u_slow, u_fast, temperature, top_p, top_k,
                 follow: Optional[np.ndarray] = None, main_token: Optional[int] = None,
                 fast_codes=None) -> FrameResult:
    """One Dual-AR frame: the Slow-AR step on the previous frame's 11 values,
    the main-token draw with repetition check, then the nine Fast-AR draws
    (main-loop page, section 5.1).

    To compare another implementation's frame along its own path: `follow`
    takes its new cache entries (see step), `main_token` its main token
    (which must be one of the draw's defensible tokens) and `fast_codes` its
    Fast-AR codes, which then form the prefixes of the Fast-AR draws
    (teacher forcing; the draws and their defensible codes are reported)."""
    x = combine(slow, prev_main, prev_codes)
    st = step(slow, x, kv, n_past, follow)
    md = draw_main(slow.shape, st.logits, window, temperature, top_p, top_k, u_slow[0], u_slow[1])
    tok = md.token
    if main_token is not None:
        tok = int(main_token)
        if tok not in md.alts:
            raise AssertionError(f"main token {tok} is not defensible (oracle {md.token}, defensible {md.alts})")
    sc = sem_code(slow.shape, tok)
    one = lambda v, dt: np.asarray([v], dtype=dt)
    forced = None if fast_codes is None else np.asarray(fast_codes, dtype=np.int64).reshape(1, -1)
    fr = _fa.decode_frame(fast, st.hidden[None, :], one(sc, np.int64), np.asarray(u_fast, F32)[None, :],
                          one(temperature, F32), one(top_p, F32), one(top_k, np.int64), forced=forced)
    return FrameResult(md, sc, st.hidden, fr.codes[0], fr.fragile[0], st.kv_new,
                       push_window(window, tok), st.logits, fr.alts[0])
