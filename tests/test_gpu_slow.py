"""Parity of the Slow-AR step and the full frame (HIP path through the C ABI)
with the oracle, on the GPU.

Tolerances (float32 accumulation in another order than the oracle's):
  logits: |delta| <= 1e-2 * max|logit| + 1e-3 (the Fast-AR logit bound);
  hidden: |delta| <= 1e-3 * max|hidden| + 1e-4;
  new cache entries: bf16 caches round each float32 key and value, and where
    the two sides' float32 values differ in the last bits a value next to a
    rounding midpoint may round either way (one bf16 ulp, 2^-8 relative).
    The oracle checks every GPU entry element by element (it must be the
    oracle's rounding, or the other neighbour of a value within 1e-4 of a
    midpoint) and then continues with the GPU's entries, so one such flip
    is not compounded over 36 layers (a CPU test shows those flips alone
    move the hidden state by about 1e-3 of its largest element at position
    0); float32 caches are compared within the hidden-state bound;
  main token and codes: the oracle's, or one of the draw's defensible
  alternatives (then the comparison follows the GPU's draw), with the
  excused count bounded."""
import numpy as np
import pytest
import torch

from dual_ar_neural_amd import binding as bd
from oracle import fast_ar as fa
from oracle import slow_ar as sa
from synth import inputs as si
from synth import slow_inputs as ssi

pytestmark = pytest.mark.gpu
F32 = np.float32
HIDDEN_RTOL, HIDDEN_ATOL = 1e-3, 1e-4
EXCUSED_SHARE = 0.02    # excused draws at most this share of all draws, plus one


def _announce(msg):
    print(f"[gpu] {msg}", flush=True)


class SlowPair:
    def __init__(self, shape, seed):
        self.shape = shape
        self.host = ssi.make_weights(shape, seed)
        self.oracle = sa.SlowModel.from_weights(shape, self.host)
        self.dev = bd.device_weights(shape, self.host)
        self.gpu = bd.SlowAR(shape, self.dev)


@pytest.fixture(scope="module")
def slow_tiny():
    _announce("slow tiny model")
    return SlowPair(ssi.SLOW_TINY, ssi.SLOW_WORKLOADS["slow_tiny"].seed(0))


@pytest.fixture(scope="module")
def slow_ragged():
    _announce("slow ragged model")
    return SlowPair(ssi.SLOW_RAGGED, ssi.SLOW_WORKLOADS["slow_ragged"].seed(0))


def _host_kv(shape, n_past, seed):
    """Cache with positions < n_past filled; positions >= n_past hold NaN,
    which no correct step reads."""
    kv = ssi.make_kv_cache(shape, n_past, seed)
    if shape.weight_dtype == "bf16":
        kv[:, :, n_past:] = 0x7FC0          # bf16 NaN
        return kv, si.f32_from_bf16_bits(kv)
    kv[:, :, n_past:] = np.nan
    return kv, kv.copy()


def _dev_kv(kv):
    if kv.dtype == np.uint16:
        return torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(kv).cuda()


def _kv_f32(t):
    return t.float().cpu().numpy()


def _i32(a):
    return torch.tensor(np.asarray(a, dtype=np.int32).reshape(-1)).cuda()


def _f32(a):
    return torch.tensor(np.asarray(a, dtype=F32).reshape(-1)).cuda()


def _window_dev(win):
    w = np.zeros(1 + bd.RAS_WINDOW, np.int32)
    w[0] = len(win)
    w[1:1 + len(win)] = win
    return _i32(w)


def _check_new_entries(s, gpu_new, oracle_new):
    """float32 caches: the GPU's new entries within the hidden-state bound
    (bf16 caches were checked entry by entry while the oracle followed them)."""
    if s.weight_dtype != "bf16":
        d = np.abs(gpu_new - oracle_new).max()
        assert d <= HIDDEN_RTOL * np.abs(oracle_new).max() + HIDDEN_ATOL, d


def _check_step(p, n_past, main, codes, win, u, T=0.8, top_p=0.8, top_k=30, seed=77):
    s = p.shape
    kv_host, kv_f = _host_kv(s, n_past, seed)
    kv = _dev_kv(kv_host)
    logits = torch.empty(p.gpu.n_allowed, dtype=torch.float32, device="cuda")
    window = _window_dev(win)
    _announce(f"slow step {s.name} n_past={n_past} window={len(win)}")
    m_out, sem_out, h_out = p.gpu.step(kv, n_past, _i32([main]), _i32(codes), window, _f32(u), _f32([T]),
                                       _f32([top_p]), _i32([top_k]), logits_out=logits)
    torch.cuda.synchronize()
    kv_after = _kv_f32(kv)
    st = sa.step(p.oracle, sa.combine(p.oracle, main, codes), kv_f, n_past, follow=kv_after[:, :, n_past])
    _check_new_entries(s, kv_after[:, :, n_past], st.kv_new)
    ids = sa.allowed_ids(s)
    assert ids.size == p.gpu.n_allowed
    ref = st.logits[ids]
    got = logits.cpu().numpy()
    tol = 1e-2 * np.abs(ref).max() + 1e-3
    assert np.abs(got - ref).max() <= tol, (np.abs(got - ref).max(), tol)
    h = h_out.cpu().numpy()
    dh = np.abs(h - st.hidden).max()
    assert dh <= HIDDEN_RTOL * np.abs(st.hidden).max() + HIDDEN_ATOL, (dh, st.flips)
    # every other position is untouched
    assert np.array_equal(np.delete(kv_after, n_past, axis=2), np.delete(kv_f, n_past, axis=2), equal_nan=True)
    md = sa.draw_main(s, st.logits, list(win), T, top_p, top_k, u[0], u[1])
    tok = int(m_out.item())
    assert tok in md.alts, (tok, md)
    assert tok in set(ids.tolist())
    assert int(sem_out.item()) == sa.sem_code(s, tok)
    w = window.cpu().numpy()
    want = sa.push_window(list(win), tok)
    assert w[0] == len(want) and list(w[1:1 + w[0]]) == want
    _announce(f"  rounding flips followed {st.flips}, |dh|/max {dh / np.abs(st.hidden).max():.1e}, "
              f"main {'excused' if tok != md.token else 'exact'}")
    return md, tok


@pytest.mark.parametrize("n_past", [0, 1, 37, 79])
def test_slow_step_tiny(slow_tiny, n_past):
    s = slow_tiny.shape
    inp = ssi.make_step_inputs(ssi.SLOW_WORKLOADS["slow_tiny"], 1)
    _check_step(slow_tiny, n_past, inp["main"][0], inp["codes"][0], [], inp["u_slow"][0])


@pytest.fixture(scope="module")
def slow_mid():
    _announce("slow mid model")
    return SlowPair(ssi.SLOW_MID, ssi.SLOW_WORKLOADS["slow_mid"].seed(0))


@pytest.mark.parametrize("n_past", [0, 3, 95, 96, 333, 699])
def test_slow_step_mid(slow_mid, n_past):
    """The measured shape's attention path (bf16, head_dim 128, 4 heads per
    group) at chunk sizes from empty to a few positions."""
    inp = ssi.make_step_inputs(ssi.SLOW_WORKLOADS["slow_mid"], 2)
    win = [int(inp["main"][1])]
    _check_step(slow_mid, n_past, inp["main"][0], inp["codes"][0], win, inp["u_slow"][0])


@pytest.mark.parametrize("n_past", [97, 12345, 12999])
def test_slow_step_mid_long_context(n_past):
    """The same attention path over a long cache: chunks of up to 102
    positions, more than one load batch per wave."""
    w = ssi.SLOW_WORKLOADS["slow_mid_long"]
    p = SlowPair(w.shape, ssi.SLOW_WORKLOADS["slow_mid"].seed(0))
    inp = ssi.make_step_inputs(w, 1)
    _check_step(p, n_past, inp["main"][0], inp["codes"][0], [], inp["u_slow"][0])
    p.gpu.close()


@pytest.mark.parametrize("n_past", [0, 5, 130, 299])
def test_slow_step_ragged(slow_ragged, n_past):
    inp = ssi.make_step_inputs(ssi.SLOW_WORKLOADS["slow_ragged"], 2)
    win = [int(x) for x in (inp["main"][1], slow_ragged.shape.sem_begin + 3)]
    _check_step(slow_ragged, n_past, inp["main"][0], inp["codes"][0], win, inp["u_slow"][0], T=0.9, top_p=0.85)


def test_slow_step_greedy_and_full_window(slow_ragged):
    s = slow_ragged.shape
    inp = ssi.make_step_inputs(ssi.SLOW_WORKLOADS["slow_ragged"], 1)
    win = list(range(s.sem_begin, s.sem_begin + bd.RAS_WINDOW))
    _check_step(slow_ragged, 64, inp["main"][0], inp["codes"][0], win, inp["u_slow"][0], T=0.0)


def test_slow_step_repetition_redraw(slow_ragged):
    """A window holding the oracle's first draw forces the redraw at
    temperature 1.0 / top_p 0.9 with the second uniform."""
    s = slow_ragged.shape
    inp = ssi.make_step_inputs(ssi.SLOW_WORKLOADS["slow_ragged"], 1)
    main, codes, u = inp["main"][0], inp["codes"][0], inp["u_slow"][0]
    kv_host, kv_f = _host_kv(s, 40, 77)
    st = sa.step(slow_ragged.oracle, sa.combine(slow_ragged.oracle, main, codes), kv_f, 40)
    first = sa.draw_main(s, st.logits, [], 0.9, 0.85, 30, u[0], u[1])
    assert s.sem_begin <= first.token <= s.sem_end
    md, tok = _check_step(slow_ragged, 40, main, codes, [s.sem_begin, first.token], u, T=0.9, top_p=0.85)
    assert md.resampled


def test_slow_step_rejects_bad_arguments(slow_tiny):
    s = slow_tiny.shape
    kv = torch.zeros((s.n_layer, s.n_head_kv, s.max_ctx, 2, s.head_dim), dtype=torch.float32, device="cuda")
    args = (_i32([s.sem_begin]), _i32(np.zeros(s.num_codebooks)), _window_dev([]), _f32([0.5, 0.5]),
            _f32([0.8]), _f32([0.8]), _i32([30]))
    for n_past in (-1, s.max_ctx):
        with pytest.raises(bd.S2FastError) as e:
            slow_tiny.gpu.step(kv, n_past, *args)
        assert e.value.code == 1


def _full_frames(p, fast_pair, n_frames, n_fill, u_slow, u_fast, main0, codes0, T, top_p, top_k=30):
    """Chained frames on the device (each frame's outputs feed the next)
    against the oracle's frame loop, which follows the GPU's path: its new
    cache entries (checked entry by entry), its main token (one of the
    draw's defensible tokens) and its Fast-AR codes (each one of its draw's
    defensible codes, teacher-forced as the next prefix).  Returns (draws,
    excused)."""
    s = p.shape
    kv_host, kv_f = _host_kv(s, n_fill + n_frames, 91)
    kv_host[:, :, n_fill:] = 0x7FC0 if s.weight_dtype == "bf16" else np.nan
    kv_f = si.f32_from_bf16_bits(kv_host) if s.weight_dtype == "bf16" else kv_host.copy()
    kv = _dev_kv(kv_host)
    window = _window_dev([])
    main_d, codes_d = _i32([main0]), _i32(codes0)
    hid = torch.empty(s.dim, dtype=torch.float32, device="cuda")
    o_main, o_codes, o_win = int(main0), np.asarray(codes0), []
    allowed = set(sa.allowed_ids(s).tolist())
    draws = excused = 0
    for f in range(n_frames):
        _announce(f"full frame {s.name} frame {f}")
        pos = n_fill + f
        m_new = torch.empty(1, dtype=torch.int32, device="cuda")
        c_new = torch.empty(s.num_codebooks, dtype=torch.int32, device="cuda")
        p.gpu.full_frame(fast_pair.gpu, kv, pos, main_d, codes_d, window, _f32(u_slow[f]), _f32(u_fast[f]),
                         _f32([T]), _f32([top_p]), _i32([top_k]), main_out=m_new, hidden_out=hid, codes_out=c_new)
        torch.cuda.synchronize()
        tok, codes = int(m_new.item()), c_new.cpu().numpy()
        assert tok in allowed and codes.min() >= 0 and codes.max() < s.codebook_size
        gpu_new = _kv_f32(kv)[:, :, pos]
        r = sa.decode_frame(p.oracle, fast_pair.oracle, kv_f, pos, o_main, o_codes, o_win, u_slow[f], u_fast[f],
                            T, top_p, top_k, follow=gpu_new, main_token=tok, fast_codes=codes)
        _check_new_entries(s, gpu_new, r.kv_new)
        h = hid.cpu().numpy()
        assert np.abs(h - r.hidden).max() <= HIDDEN_RTOL * np.abs(r.hidden).max() + HIDDEN_ATOL
        assert codes[0] == r.sem_code
        for k in range(1, s.num_codebooks):
            assert codes[k] in r.fast_alts[k - 1], (f, k, codes, r.codes, r.fast_alts[k - 1])
            excused += int(codes[k] != r.codes[k])
        draws += s.num_codebooks
        excused += int(tok != r.main.token)
        kv_f[:, :, pos] = r.kv_new
        # the next frame starts from the GPU's draws on both sides
        o_main, o_codes, o_win = tok, codes, sa.push_window(o_win, tok)
        main_d, codes_d = m_new, c_new
    assert excused <= EXCUSED_SHARE * draws + 1, (excused, draws)
    return draws, excused


class FastPair:
    def __init__(self, shape, seed):
        self.oracle = fa.Model.from_weights(shape, si.make_weights(shape, seed))
        self.gpu = bd.FastAR(shape, bd.device_weights(shape, si.make_weights(shape, seed)), max_batch=1)


def test_full_frame_tiny(slow_tiny):
    fast = FastPair(si.TINY, si.WORKLOADS["tiny"].seed(0))
    w = ssi.SLOW_WORKLOADS["slow_tiny"]
    inp = ssi.make_step_inputs(w, 4)
    draws, excused = _full_frames(slow_tiny, fast, 4, w.n_fill, inp["u_slow"], inp["u_fast"], inp["main"][0],
                                  inp["codes"][0], 0.8, 0.8)
    _announce(f"full frames tiny: {draws} draws, {excused} excused")


def test_full_frame_ragged(slow_ragged):
    fast = FastPair(si.RAGGED, si.WORKLOADS["ragged"].seed(0))
    w = ssi.SLOW_WORKLOADS["slow_ragged"]
    inp = ssi.make_step_inputs(w, 3)
    draws, excused = _full_frames(slow_ragged, fast, 3, w.n_fill, inp["u_slow"], inp["u_fast"], inp["main"][0],
                                  inp["codes"][0], 0.9, 0.85)
    _announce(f"full frames {w.name}: {draws} draws, {excused} excused")


@pytest.fixture(scope="module")
def slow_s2pro():
    w = ssi.SLOW_WORKLOADS["full_s2pro"]
    _announce("slow s2pro weights (7.3 GB bf16)")
    p = SlowPair(w.shape, w.seed(0))
    yield p
    p.gpu.close()


@pytest.mark.timeout(600)
def test_slow_step_s2pro_full_size(slow_s2pro):
    """The measured shape: 36 layers, 2048 cached positions (N(0,1) bf16),
    vocabulary 155776; steps at positions 2048 and 2559 (the last) against
    the full oracle step (positions past n_past hold NaN)."""
    w = ssi.SLOW_WORKLOADS["full_s2pro"]
    s = w.shape
    p = slow_s2pro
    inp = ssi.make_step_inputs(w, 2)
    _check_step(p, w.n_fill, inp["main"][0], inp["codes"][0], [], inp["u_slow"][0], seed=w.seed(5))
    # the cache's last position (chunks of 80 positions)
    _check_step(p, s.max_ctx - 1, inp["main"][1], inp["codes"][1], [int(inp["main"][0])], inp["u_slow"][1],
                seed=w.seed(6))


# ------------------------------------------------------------------ prefill

def _prompt(s, T, seed, n_text):
    """T prompt positions: n_text text tokens (ids below the semantic range,
    codes present but masked), then semantic ids with codes, one of them the
    end id's row turned into a text-like position."""
    rng = np.random.default_rng(seed)
    toks = np.zeros((T, 1 + s.num_codebooks), np.int32)
    toks[:, 1:] = rng.integers(0, s.codebook_size, size=(T, s.num_codebooks))
    toks[:n_text, 0] = rng.integers(0, min(s.sem_begin, s.vocab), size=n_text)
    toks[n_text:, 0] = rng.integers(s.sem_begin, s.sem_end + 1, size=T - n_text)
    if T - n_text >= 3:
        toks[n_text + 1, 0] = s.end_id
    return toks


def _check_prefill(p, n_past0, toks, win, u, T_=0.8, top_p=0.8, top_k=30, seed=55):
    s = p.shape
    T = toks.shape[0]
    kv_host, kv_f = _host_kv(s, n_past0, seed)
    kv = _dev_kv(kv_host)
    logits = torch.empty(p.gpu.n_allowed, dtype=torch.float32, device="cuda")
    window = _window_dev(win)
    _announce(f"prefill {s.name} n_past0={n_past0} T={T}")
    m_out, sem_out, h_out = p.gpu.prefill(kv, n_past0, torch.from_numpy(toks).cuda(), window, _f32(u), _f32([T_]),
                                          _f32([top_p]), _i32([top_k]), logits_out=logits)
    torch.cuda.synchronize()
    kv_before = kv_f.copy()
    kv_after = _kv_f32(kv)
    new = slice(n_past0, n_past0 + T)
    st = sa.prefill(p.oracle, toks, kv_f, n_past0, follow=kv_after[:, :, new])
    _check_new_entries(s, kv_after[:, :, new], kv_f[:, :, new])
    ref = st.logits[sa.allowed_ids(s)]
    got = logits.cpu().numpy()
    assert np.abs(got - ref).max() <= 1e-2 * np.abs(ref).max() + 1e-3
    h = h_out.cpu().numpy()
    dh = np.abs(h - st.hidden).max()
    assert dh <= HIDDEN_RTOL * np.abs(st.hidden).max() + HIDDEN_ATOL, (dh, st.flips)
    keep = np.r_[0:n_past0, n_past0 + T:s.max_ctx]
    assert np.array_equal(kv_after[:, :, keep], kv_before[:, :, keep], equal_nan=True)
    md = sa.draw_main(s, st.logits, list(win), T_, top_p, top_k, u[0], u[1])
    tok = int(m_out.item())
    assert tok in md.alts, (tok, md)
    _announce(f"  rounding flips followed {st.flips}, |dh|/max {dh / np.abs(st.hidden).max():.1e}")
    assert tok in set(sa.allowed_ids(s).tolist())
    assert int(sem_out.item()) == sa.sem_code(s, tok)
    w = window.cpu().numpy()
    want = sa.push_window(list(win), tok)
    assert w[0] == len(want) and list(w[1:1 + w[0]]) == want


@pytest.mark.parametrize("n_past0,T,n_text", [(0, 1, 1), (0, 9, 4), (30, 5, 0), (70, 10, 3)])
def test_prefill_tiny(slow_tiny, n_past0, T, n_text):
    _check_prefill(slow_tiny, n_past0, _prompt(slow_tiny.shape, T, 100 + T, n_text), [], [0.3, 0.7])


@pytest.mark.parametrize("n_past0,T,n_text", [(0, 6, 2), (90, 8, 3)])
def test_prefill_mid(slow_mid, n_past0, T, n_text):
    _check_prefill(slow_mid, n_past0, _prompt(slow_mid.shape, T, 200 + T, n_text), [], [0.6, 0.2])


def test_prefill_ragged(slow_ragged):
    s = slow_ragged.shape
    _check_prefill(slow_ragged, 100, _prompt(s, 7, 300, 2), [s.sem_begin + 9], [0.45, 0.55], T_=0.9, top_p=0.85)


def test_prefill_rejects_bad_arguments(slow_tiny):
    s = slow_tiny.shape
    kv = torch.zeros((s.n_layer, s.n_head_kv, s.max_ctx, 2, s.head_dim), dtype=torch.float32, device="cuda")
    args = (_window_dev([]), _f32([0.5, 0.5]), _f32([0.8]), _f32([0.8]), _i32([30]))
    toks = torch.zeros((3, 1 + s.num_codebooks), dtype=torch.int32, device="cuda")
    for n0 in (-1, s.max_ctx - 2):
        with pytest.raises(bd.S2FastError) as e:
            slow_tiny.gpu.prefill(kv, n0, toks, *args)
        assert e.value.code == 1


# Chunked prefill: the positions before the last run up to 64 a launch on
# the matrix cores; these prompts take several chunks and a ragged last one.
@pytest.mark.parametrize("n_past0,T,n_text", [(0, 80, 30), (5, 75, 0), (1, 66, 2)])
def test_prefill_chunks_tiny(slow_tiny, n_past0, T, n_text):
    _check_prefill(slow_tiny, n_past0, _prompt(slow_tiny.shape, T, 600 + T, n_text), [], [0.4, 0.6])


@pytest.mark.parametrize("which,n_past0,T", [("tiny", 0, 2), ("mid", 0, 2), ("mid", 635, 65), ("ragged", 233, 67)])
def test_prefill_chunk_edges(slow_tiny, slow_mid, slow_ragged, which, n_past0, T):
    """A chunk of one position (T = 2), and prompts whose last position is
    the cache's last (a full chunk of 64 ending there; 66 positions in two
    chunks at the ragged shape)."""
    p = {"tiny": slow_tiny, "mid": slow_mid, "ragged": slow_ragged}[which]
    assert n_past0 + T <= p.shape.max_ctx
    _check_prefill(p, n_past0, _prompt(p.shape, T, 1400 + T, min(T, 3)), [], [0.45, 0.55])


def test_prefill_chunks_ragged(slow_ragged):
    s = slow_ragged.shape
    _check_prefill(slow_ragged, 100, _prompt(s, 150, 700, 20), [s.sem_begin + 3], [0.55, 0.45], T_=0.9, top_p=0.85)


def test_prefill_chunks_mid(slow_mid):
    _check_prefill(slow_mid, 3, _prompt(slow_mid.shape, 200, 800, 40), [], [0.7, 0.3])


def test_prefill_chunks_off_matches(slow_mid):
    """The comparison path (two positions a launch) still runs when the
    chunks are switched off."""
    slow_mid.gpu.prefill_chunks(False)
    try:
        _check_prefill(slow_mid, 10, _prompt(slow_mid.shape, 9, 900, 3), [], [0.2, 0.8])
    finally:
        slow_mid.gpu.prefill_chunks(True)


def test_prefill_device_failure_is_reported_and_recovered(slow_mid):
    """Every launch's first grid-wide wait made to give up (the test hook),
    through a chunked prefill: every block leaves normally, the status
    reports the failure once, no token is drawn; then the same context
    prefills correctly (the K-split counts were restored)."""
    s = slow_mid.shape
    kv_host, _ = _host_kv(s, 20, 61)
    kv = _dev_kv(kv_host)
    main_out = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    window = _window_dev([])
    slow_mid.gpu.test_watchdog(True)
    try:
        slow_mid.gpu.prefill(kv, 20, torch.from_numpy(_prompt(s, 70, 1300, 10)).cuda(), window, _f32([0.5, 0.5]),
                             _f32([0.8]), _f32([0.8]), _i32([30]), main_out=main_out)
        torch.cuda.synchronize()
    finally:
        slow_mid.gpu.test_watchdog(False)
    assert slow_mid.gpu.status() == 6 and slow_mid.gpu.status() == 0
    assert int(main_out.item()) == -7 and int(window[0].item()) == 0
    _check_prefill(slow_mid, 20, _prompt(s, 70, 1300, 10), [], [0.5, 0.5])
    assert slow_mid.gpu.status() == 0


def test_prefill_mid_long_context():
    """A prompt at cache positions near 7000 of a 13000-position cache: the
    attention splits each query block's cache positions over 16 workgroups
    and merges their partial results."""
    w = ssi.SLOW_WORKLOADS["slow_mid_long"]
    p = SlowPair(w.shape, ssi.SLOW_WORKLOADS["slow_mid"].seed(0))
    _check_prefill(p, 6990, _prompt(w.shape, 30, 1000, 5), [], [0.3, 0.7], seed=w.seed(3))
    p.gpu.close()


@pytest.mark.parametrize("which", ["tiny", "mid"])
def test_prefill_chunk_limit(slow_tiny, slow_mid, which):
    """Chunks only below a cache position (as where an f32 cache's on-chip
    score buffer ends): the positions below it run chunked, the rest two a
    launch, the last with the head."""
    p = slow_tiny if which == "tiny" else slow_mid
    p.gpu.prefill_chunks(40)
    try:
        _check_prefill(p, 5, _prompt(p.shape, 70, 1200, 10), [], [0.65, 0.35])
    finally:
        p.gpu.prefill_chunks(True)


def _check_prefill_sampled(p, n_past0, toks, samples, u, T_=0.8, top_p=0.8, top_k=30, seed=55):
    """A long prefill at full size, checked at sampled positions: the oracle
    runs each sampled position's step over the cache the GPU wrote before it
    (following its rounding) and checks the entries the GPU wrote there; the
    last position's logits and hidden state the same way."""
    s = p.shape
    T = toks.shape[0]
    kv_host, kv_f = _host_kv(s, n_past0, seed)
    kv = _dev_kv(kv_host)
    logits = torch.empty(p.gpu.n_allowed, dtype=torch.float32, device="cuda")
    window = _window_dev([])
    _announce(f"prefill {s.name} n_past0={n_past0} T={T}, sampled at {samples}")
    m_out, _, h_out = p.gpu.prefill(kv, n_past0, torch.from_numpy(toks).cuda(), window, _f32(u), _f32([T_]),
                                    _f32([top_p]), _i32([top_k]), logits_out=logits)
    torch.cuda.synchronize()
    kv_after = _kv_f32(kv)
    keep = np.r_[0:n_past0, n_past0 + T:s.max_ctx]
    assert np.array_equal(kv_after[:, :, keep], kv_f[:, :, keep], equal_nan=True)
    assert np.isfinite(kv_after[:, :, n_past0:n_past0 + T]).all()
    for t in sorted(set(samples) | {T - 1}):
        pos = n_past0 + t
        x = sa.combine(p.oracle, toks[t, 0], toks[t, 1:])
        st = sa.step(p.oracle, x, kv_after, pos, follow=kv_after[:, :, pos])
        _check_new_entries(s, kv_after[:, :, pos], st.kv_new)
        _announce(f"  position {pos}: entries ok ({st.flips} rounding flips followed)")
    ref = st.logits[sa.allowed_ids(s)]
    got = logits.cpu().numpy()
    assert np.abs(got - ref).max() <= 1e-2 * np.abs(ref).max() + 1e-3
    h = h_out.cpu().numpy()
    assert np.abs(h - st.hidden).max() <= HIDDEN_RTOL * np.abs(st.hidden).max() + HIDDEN_ATOL
    assert int(m_out.item()) in sa.draw_main(s, st.logits, [], T_, top_p, top_k, u[0], u[1]).alts


@pytest.mark.timeout(900)
def test_prefill_chunks_s2pro_full_size(slow_s2pro):
    """130 prompt positions over the 2000 cached ones at the measured shape:
    chunks of 64, 64 and 1, then the last position with the head; sampled
    at each chunk's first and last position."""
    w = ssi.SLOW_WORKLOADS["full_s2pro"]
    _check_prefill_sampled(slow_s2pro, 2000, _prompt(w.shape, 130, 1100, 10), [0, 63, 64, 127, 128], [0.5, 0.5],
                           seed=w.seed(10))


@pytest.mark.timeout(600)
def test_prefill_s2pro_full_size(slow_s2pro):
    """Three prompt positions (a text token, then two semantic positions)
    over the 2048-position cache at the measured shape."""
    w = ssi.SLOW_WORKLOADS["full_s2pro"]
    _check_prefill(slow_s2pro, w.n_fill - 1, _prompt(w.shape, 3, 400, 1), [], [0.25, 0.75], seed=w.seed(7))


@pytest.mark.timeout(600)
def test_full_frame_s2pro_full_size(slow_s2pro):
    """Two chained full frames at the measured shapes (36-layer Slow-AR over
    the 2048-position cache, then the S2 Pro Fast-AR), as bench.py runs
    them."""
    fast = FastPair(si.S2PRO, si.WORKLOADS["s2pro_b1"].seed(0))
    w = ssi.SLOW_WORKLOADS["full_s2pro"]
    inp = ssi.make_step_inputs(w, 2)
    draws, excused = _full_frames(slow_s2pro, fast, 2, w.n_fill, inp["u_slow"], inp["u_fast"], inp["main"][0],
                                  inp["codes"][0], 0.8, 0.8)
    _announce(f"full frames {w.name}: {draws} draws, {excused} excused")
    fast.gpu.close()


@pytest.mark.timeout(600)
def test_slow_edges_s2pro_full_size(slow_s2pro):
    """The measured shape at the cache's first position (every attention
    chunk but the last is empty) and an odd prefill from position 0 (two
    pairs, then a one-position launch)."""
    w = ssi.SLOW_WORKLOADS["full_s2pro"]
    inp = ssi.make_step_inputs(w, 1)
    _check_step(slow_s2pro, 0, inp["main"][0], inp["codes"][0], [], inp["u_slow"][0], seed=w.seed(8))
    _check_prefill(slow_s2pro, 0, _prompt(w.shape, 5, 500, 2), [], [0.35, 0.65], seed=w.seed(9))
