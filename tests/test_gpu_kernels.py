"""Per-kernel parity of the frame kernel's building blocks (test exports of
the C ABI), and the entry points around the frame: the single Fast-AR call
and the device-side failure report.

GEMV (s2fast_test_gemv) at the six S2 Pro shapes (wqkv 6144x2560, wo
2560x4096, w1 and w3 9728x2560 as one SwiGLU pair, w2 2560x9728, head
4096x2560) and the tiny and ragged shapes, one and two activation rows:
  * small integer weights and activations: every product and partial sum is
    an integer below 2^24, exact in float32 in any order, so the GPU must
    return the integer dot products bit for bit (a wrong row, a dropped or
    repeated term or a misplaced activation cannot hide in a tolerance);
  * random values with the RMSNorm and SwiGLU epilogues against float64:
    per element |delta| <= 64 * 2^-24 * sum_k |W_ik n_k| (a float32 dot
    product summed in chunks of at most a few dozen terms, then trees over
    lanes and waves), plus the epilogue's own rounding.
q/k norm + RoPE + attention (s2fast_test_norm_rope_attn) against the
oracle's functions within 1e-4 * max|out| + 1e-5: scores of 128-term float32
dot products carry about 1e-5 absolute error, which the softmax passes on
as relative error of the weights."""
import numpy as np
import pytest
import torch

from dual_ar_neural_amd import binding as bd
from oracle import fast_ar as fa
from synth import inputs as si
from tests import parity as pr

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def _announce(msg):
    print(f"[gpu] {msg}", flush=True)


S2PRO_GEMVS = [   # (name, N, K, swiglu, norm)
    ("wqkv", 6144, 2560, False, True), ("wo", 2560, 4096, False, False), ("w1w3", 9728, 2560, True, True),
    ("w2", 2560, 9728, False, False), ("head", 4096, 2560, False, True), ("project_in", 2560, 2560, False, False)]
SMALL_GEMVS = [
    ("tiny_wqkv", 512, 256, False, True, torch.float32), ("tiny_w1w3", 768, 256, True, True, torch.float32),
    ("tiny_w2", 256, 768, False, False, torch.float32), ("ragged_wqkv", 400, 200, False, True, torch.bfloat16),
    ("ragged_w2", 200, 520, False, False, torch.bfloat16), ("ragged_head", 300, 200, False, True, torch.bfloat16),
    ("ragged_proj", 200, 176, False, False, torch.bfloat16), ("odd_rows", 7, 64, True, False, torch.bfloat16)]
CASES = [(n, N, K, sw, nm, torch.bfloat16) for n, N, K, sw, nm in S2PRO_GEMVS] + SMALL_GEMVS


@pytest.mark.parametrize("name,N,K,swiglu,norm,dt", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("M", [1, 2])
def test_gemv_integer_exact(name, N, K, swiglu, norm, dt, M):
    g = torch.Generator().manual_seed(N * 7 + K + M)
    W = torch.randint(-4, 5, (N, K), generator=g).to(dt).cuda()
    W3 = torch.randint(-4, 5, (N, K), generator=g).to(dt).cuda() if swiglu else None
    x = torch.randint(-4, 5, (M, K), generator=g).float().cuda()
    y = bd.gemv(W, x, W3=W3).cpu().double()
    a1 = (x.double() @ W.double().T).cpu()
    if swiglu:
        a3 = (x.double() @ W3.double().T).cpu()
        # a1 and a3 are exact; the epilogue rounds silu and the product in float32
        want = (a1 / (1 + torch.exp(-a1))) * a3
        assert torch.all((y - want).abs() <= 8 * U * want.abs() + 1e-30), name
    else:
        assert torch.equal(y, a1), (name, (y - a1).abs().max().item())
    _announce(f"gemv {name} M={M}: exact")


@pytest.mark.parametrize("name,N,K,swiglu,norm,dt", CASES, ids=[c[0] for c in CASES])
def test_gemv_norm_swiglu_random(name, N, K, swiglu, norm, dt):
    rng = np.random.default_rng(N + 3 * K)
    M = 2
    Wh = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W3h = (rng.standard_normal((N, K)) * 0.02).astype(np.float32) if swiglu else None
    wn = (1 + 0.05 * rng.standard_normal(K)).astype(np.float32) if norm else None
    x = rng.standard_normal((M, K)).astype(np.float32)
    to = lambda a: torch.from_numpy(a).to(dt).cuda()
    W, W3, nw = to(Wh), (to(W3h) if swiglu else None), (to(wn) if norm else None)
    y = bd.gemv(W, torch.from_numpy(x).cuda(), W3=W3, norm_w=nw, eps=1e-6).cpu().numpy().astype(np.float64)
    # the same bf16-valued weights, float64 arithmetic
    Wd = W.double().cpu().numpy()
    n = x.astype(np.float64)
    if norm:
        n = n * nw.double().cpu().numpy() / np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1, keepdims=True) + 1e-6)
    a1 = n @ Wd.T
    s1 = np.abs(n) @ np.abs(Wd).T
    bound = 64 * U * s1 + 8 * U * np.abs(a1)
    if swiglu:
        W3d = W3.double().cpu().numpy()
        a3 = n @ W3d.T
        s3 = np.abs(n) @ np.abs(W3d).T
        sig = 1 / (1 + np.exp(-a1))
        want = a1 * sig * a3
        dsilu = sig * (1 + a1 * (1 - sig))
        bound = (np.abs(dsilu * a3) * (64 * U * s1 + 8 * U * np.abs(a1)) + np.abs(a1 * sig) * (64 * U * s3 + 8 * U * np.abs(a3))
                 + 8 * U * np.abs(want))
    else:
        want = a1
    err = np.abs(y - want)
    assert np.all(err <= bound + 1e-30), (name, float((err / (bound + 1e-30)).max()))
    _announce(f"gemv {name} random: worst |d|/bound {float((err / (bound + 1e-30)).max()):.2e}")


ATTN_SHAPES = [("s2pro", 32, 8, 128, 11), ("tiny", 4, 2, 64, 11), ("ragged", 6, 2, 40, 11), ("mha", 4, 4, 64, 16)]


@pytest.mark.parametrize("name,H,G,hd,ctx", ATTN_SHAPES, ids=[a[0] for a in ATTN_SHAPES])
@pytest.mark.parametrize("qk_norm", [True, False])
def test_norm_rope_attn(name, H, G, hd, ctx, qk_norm):
    rng = np.random.default_rng(H * hd + ctx)
    T = min(10, ctx)
    qkv = rng.standard_normal((T, (H + 2 * G) * hd)).astype(np.float32)
    qn = (1 + 0.05 * rng.standard_normal(hd)).astype(np.float32)
    kn = (1 + 0.05 * rng.standard_normal(hd)).astype(np.float32)
    dev = lambda a: torch.from_numpy(a).cuda()
    got = bd.norm_rope_attn(dev(qkv), H, G, hd, ctx, 1e6, 1e-6, q_norm=dev(qn) if qk_norm else None,
                            k_norm=dev(kn) if qk_norm else None).cpu().numpy()
    # the oracle's own functions over the whole window
    q = qkv[:, : H * hd].reshape(1, T, H, hd)
    k = qkv[:, H * hd:(H + G) * hd].reshape(1, T, G, hd)
    v = qkv[:, (H + G) * hd:].reshape(1, T, G, hd)
    if qk_norm:
        q, k = fa.rms_norm(q, qn, 1e-6), fa.rms_norm(k, kn, 1e-6)
    cos, sin = fa.rope_table(hd, ctx, 1e6)
    q, k = fa.apply_rope(q, cos[:T], sin[:T]), fa.apply_rope(k, cos[:T], sin[:T])
    want = fa.causal_attention(q, k, v)[0]
    d = np.abs(got - want).max()
    assert d <= 1e-4 * np.abs(want).max() + 1e-5, (name, d)
    _announce(f"norm_rope_attn {name} qk_norm={qk_norm}: |d|/max {d / np.abs(want).max():.1e}")


# ------------------------------------------------------------ fast_decode

@pytest.mark.parametrize("shape_name,B", [("tiny", 1), ("tiny", 3), ("ragged", 2), ("s2pro", 1), ("s2pro", 4)])
def test_fast_decode_matches_oracle(shape_name, B):
    """One Fast-AR call per prefix length 1..9 against the oracle's
    fast_forward (the window [hidden, emb(prefix)]); B = 1 runs the batch-1
    kernel, B >= 2 the batched one."""
    w = si.WORKLOADS["s2pro_b1" if shape_name == "s2pro" else shape_name]
    p = pr.make_pair(w.shape, w.seed(0), max_batch=max(B, 2))
    rng = np.random.default_rng(B)
    hidden = si.make_frames(w, n_frames=1, batch=B)["hidden"][0]
    worst = 0.0
    for k in range(1, w.shape.num_codebooks):
        prefix = rng.integers(0, w.shape.codebook_size, size=(B, k)).astype(np.int32)
        got = p.ctx.fast_decode(pr.to_dev(hidden), pr.to_dev(prefix)).cpu().numpy()
        want = fa.fast_forward(p.oracle, hidden, prefix)
        for b in range(B):
            r = float(np.abs(got[b] - want[b]).max()) / pr.logit_tolerance(want[b])
            worst = max(worst, r)
    assert worst <= 1.0, worst
    _announce(f"fast_decode {shape_name} B={B}: worst |d|/tol {worst:.2e}")
    p.ctx.close()


def test_fast_decode_entry_checks():
    """The pages' entry checks, in their order: hidden width, then prefix
    length; nothing is enqueued on an error."""
    w = si.WORKLOADS["tiny"]
    p = pr.make_pair(w.shape, w.seed(0), max_batch=2)
    h = torch.zeros((1, w.shape.in_dim), dtype=torch.float32, device="cuda")
    good = torch.zeros((1, 3), dtype=torch.int32, device="cuda")
    for kw, code in (({"hidden_dim": w.shape.in_dim + 8}, 3),):
        with pytest.raises(bd.S2FastError) as e:
            p.ctx.fast_decode(h, good, **kw)
        assert e.value.code == code
    for plen in (0, w.shape.num_codebooks, w.shape.num_codebooks + 3):
        pre = torch.zeros((1, plen), dtype=torch.int32, device="cuda")
        with pytest.raises(bd.S2FastError) as e:
            p.ctx.fast_decode(h, pre)
        assert e.value.code == 4
    with pytest.raises(bd.S2FastError) as e:           # width is checked before the prefix
        p.ctx.fast_decode(h, torch.zeros((1, 0), dtype=torch.int32, device="cuda"), hidden_dim=17)
    assert e.value.code == 3
    h3 = torch.zeros((3, w.shape.in_dim), dtype=torch.float32, device="cuda")
    with pytest.raises(bd.S2FastError) as e:
        p.ctx.fast_decode(h3, torch.zeros((3, 2), dtype=torch.int32, device="cuda"))
    assert e.value.code == 5
    p.ctx.close()


def test_mixed_launches_on_one_context():
    """Batch-1 frames, one-call decodes of falling prefix lengths (launches of
    9 steps down to 1), a batched frame and the allocation-free path, in turn
    on one context.  Every launch writes its hand-over values with a tag no
    earlier launch used (the epoch advances by at least one a launch), so
    each result matches the oracle whatever earlier launches, of any length
    or kernel, left in the arena."""
    w = si.WORKLOADS["tiny"]
    p = pr.make_pair(w.shape, w.seed(0), max_batch=3)
    f1 = si.make_frames(w, n_frames=3, batch=1)
    f3 = si.make_frames(w, n_frames=1, batch=3)
    rng = np.random.default_rng(11)

    def frame(fr, f, static=False):
        args = (fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f], fr["temperature"], fr["top_p"], fr["top_k"])
        if static:
            d = pr.to_dev
            codes = p.ctx.decode_frame(d(args[0], torch.float32), d(np.asarray(args[1], np.int32)),
                                       d(args[2], torch.float32), d(args[3], torch.float32), d(args[4], torch.float32),
                                       d(np.asarray(args[5], np.int32)), static_scratch=True)
            torch.cuda.synchronize()
            codes = codes.cpu().numpy()
        else:
            codes = pr.gpu_decode(p, *args)
        pr.check_frame(p, *args, codes).assert_ok(1e-3)

    frame(f1, 0)
    hidden = f1["hidden"][1]
    for k in range(w.shape.num_codebooks - 1, 0, -1):
        prefix = rng.integers(0, w.shape.codebook_size, size=(1, k)).astype(np.int32)
        got = p.ctx.fast_decode(pr.to_dev(hidden), pr.to_dev(prefix)).cpu().numpy()
        want = fa.fast_forward(p.oracle, hidden, prefix)
        assert float(np.abs(got[0] - want[0]).max()) <= pr.logit_tolerance(want[0]), k
    frame(f3, 0)
    frame(f1, 1, static=True)
    frame(f1, 2)
    assert p.ctx.status() == 0
    _announce("mixed launches on one context: every result matches the oracle")
    p.ctx.close()


# ------------------------------------------------------------ failure report

@pytest.mark.parametrize("B", [1, 3])
def test_device_failure_is_reported_and_recovered(B):
    """Every block's first grid-wide wait is made to give up (the test hook:
    it waits for an epoch no block publishes, for two polls), so every block
    still leaves the kernel normally.  The launch reports the failure
    through s2fast_status, keeps the semantic codes and zero-fills codebooks
    1..; the next frame on the same context decodes correctly."""
    w = si.WORKLOADS["tiny"]
    p = pr.make_pair(w.shape, w.seed(0), max_batch=4)
    fr = si.make_frames(w, n_frames=2, batch=B)
    assert p.ctx.status() == 0
    p.ctx.test_watchdog(True)
    codes = pr.gpu_decode(p, fr["hidden"][0], fr["sem_code"][0], fr["uniforms"][0], fr["temperature"],
                          fr["top_p"], fr["top_k"])
    assert p.ctx.status() == 6                     # S2FAST_ERR_HIP
    assert p.ctx.status() == 0                     # the report is cleared by reading it
    assert np.array_equal(codes[:, 0], np.clip(fr["sem_code"][0], 0, w.shape.codebook_size - 1))
    assert (codes[:, 1:] == 0).all()
    p.ctx.test_watchdog(False)
    for f in range(2):
        codes = pr.gpu_decode(p, fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f], fr["temperature"],
                              fr["top_p"], fr["top_k"])
        pr.check_frame(p, fr["hidden"][f], fr["sem_code"][f], fr["uniforms"][f], fr["temperature"], fr["top_p"],
                       fr["top_k"], codes).assert_ok(1e-4)
    assert p.ctx.status() == 0
    _announce(f"failure path B={B}: reported, zero-filled, recovered")
    p.ctx.close()


def test_slow_device_failure_is_reported_and_recovered():
    from oracle import slow_ar as sa
    from synth import slow_inputs as ssi
    sw = ssi.SLOW_WORKLOADS["slow_tiny"]
    s = sw.shape
    host = ssi.make_weights(s, sw.seed(0))
    slow = bd.SlowAR(s, bd.device_weights(s, host))
    model = sa.SlowModel.from_weights(s, host)
    kvh = ssi.make_kv_cache(s, sw.n_fill, sw.seed(5))
    inp = ssi.make_step_inputs(sw, 1)
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
    args = (t(inp["main"][:1], torch.int32), t(inp["codes"][0], torch.int32))
    window = torch.zeros(11, dtype=torch.int32, device="cuda")
    main_out = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    slow.test_watchdog(True)
    kv = torch.from_numpy(kvh.copy()).cuda()
    slow.step(kv, sw.n_fill, *args, window, t(inp["u_slow"][0], torch.float32), t([0.8], torch.float32),
              t([0.8], torch.float32), t([30], torch.int32), main_out=main_out)
    assert slow.status() == 6 and slow.status() == 0
    assert int(main_out.item()) == -7 and int(window[0].item()) == 0   # no draw, window unchanged
    slow.test_watchdog(False)
    kv = torch.from_numpy(kvh.copy()).cuda()
    m_out, _, h_out = slow.step(kv, sw.n_fill, *args, window, t(inp["u_slow"][0], torch.float32),
                                t([0.8], torch.float32), t([0.8], torch.float32), t([30], torch.int32))
    torch.cuda.synchronize()
    assert slow.status() == 0
    st = sa.step(model, sa.combine(model, inp["main"][0], inp["codes"][0]), kvh, sw.n_fill,
                 follow=kv.float().cpu().numpy()[:, :, sw.n_fill])
    h = h_out.cpu().numpy()
    assert np.abs(h - st.hidden).max() <= 1e-3 * np.abs(st.hidden).max() + 1e-4
    md = sa.draw_main(s, st.logits, [], 0.8, 0.8, 30, inp["u_slow"][0][0], inp["u_slow"][0][1])
    assert int(m_out.item()) in md.alts
    slow.close()


# ------------------------------------------------------------ weight-only int8

Q8_GEMVS = [("wqkv", 6144, 2560, False, True), ("wo", 2560, 4096, False, False), ("w1w3", 9728, 2560, True, True),
            ("w2", 2560, 9728, False, False), ("head", 4096, 2560, False, True), ("small", 400, 208, True, True),
            ("odd_rows", 7, 64, False, False)]


@pytest.mark.parametrize("name,N,K,swiglu,norm", Q8_GEMVS, ids=[c[0] for c in Q8_GEMVS])
@pytest.mark.parametrize("M", [1, 2])
def test_gemv_q8_integer_exact(name, N, K, swiglu, norm, M):
    """int8 weights, power-of-two row scales and small integer activations:
    every product, partial sum and scaled result is exact in float32."""
    g = torch.Generator().manual_seed(N + K + 31 * M)
    W = torch.randint(-127, 128, (N, K), generator=g, dtype=torch.int8).cuda()
    W3 = torch.randint(-127, 128, (N, K), generator=g, dtype=torch.int8).cuda() if swiglu else None
    sc = (2.0 ** torch.randint(-6, 2, (N,), generator=g).float()).cuda()
    sc3 = (2.0 ** torch.randint(-6, 2, (N,), generator=g).float()).cuda() if swiglu else None
    x = torch.randint(-3, 4, (M, K), generator=g).float().cuda()
    y = bd.gemv(W, x, W3=W3, scale=sc, scale3=sc3).cpu().double()
    a1 = (x.double() @ W.double().T).cpu() * sc.double().cpu()
    if swiglu:
        a3 = (x.double() @ W3.double().T).cpu() * sc3.double().cpu()
        want = (a1 / (1 + torch.exp(-a1))) * a3
        assert torch.all((y - want).abs() <= 8 * U * want.abs() + 1e-30), name
    else:
        assert torch.equal(y, a1), (name, (y - a1).abs().max().item())
    _announce(f"gemv q8 {name} M={M}: exact")


@pytest.mark.parametrize("name,N,K,swiglu,norm", Q8_GEMVS, ids=[c[0] for c in Q8_GEMVS])
def test_gemv_q8_random(name, N, K, swiglu, norm):
    rng = np.random.default_rng(N * 5 + K)
    q, s = si.quantize_rows((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    q3, s3 = si.quantize_rows((rng.standard_normal((N, K)) * 0.02).astype(np.float32)) if swiglu else (None, None)
    wn = si.bf16_bits_from_f32((1 + 0.05 * rng.standard_normal(K)).astype(np.float32)) if norm else None
    x = rng.standard_normal((2, K)).astype(np.float32)
    d = lambda a: torch.from_numpy(a).cuda()
    nw = torch.from_numpy(wn.view(np.int16)).view(torch.bfloat16).cuda() if norm else None
    y = bd.gemv(d(q), d(x), W3=d(q3) if swiglu else None, norm_w=nw, eps=1e-6, scale=d(s),
                scale3=d(s3) if swiglu else None).cpu().numpy().astype(np.float64)
    Wd = q.astype(np.float64) * s.astype(np.float64)[:, None]
    n = x.astype(np.float64)
    if norm:
        n = n * si.f32_from_bf16_bits(wn).astype(np.float64) / np.sqrt(np.mean(n ** 2, axis=1, keepdims=True) + 1e-6)
    a1 = n @ Wd.T
    b1 = 64 * U * (np.abs(n) @ np.abs(Wd).T) + 8 * U * np.abs(a1)
    if swiglu:
        W3d = q3.astype(np.float64) * s3.astype(np.float64)[:, None]
        a3 = n @ W3d.T
        b3 = 64 * U * (np.abs(n) @ np.abs(W3d).T) + 8 * U * np.abs(a3)
        sig = 1 / (1 + np.exp(-a1))
        want = a1 * sig * a3
        bound = np.abs(sig * (1 + a1 * (1 - sig)) * a3) * b1 + np.abs(a1 * sig) * b3 + 8 * U * np.abs(want)
    else:
        want, bound = a1, b1
    r = np.abs(y - want) / (bound + 1e-30)
    assert np.all(r <= 1.0), (name, float(r.max()))
    _announce(f"gemv q8 {name} random: worst |d|/bound {float(r.max()):.2e}")


# ------------------------------------------------------------------ streaming-read probe

@pytest.mark.gpu
@pytest.mark.parametrize("nbytes,grid,in_flight", [(16, 1, 4), (1 << 20, 256, 4), ((1 << 20) + 48, 7, 8),
                                                   (64 << 20, 256, 8), ((64 << 20) + 16 * 513, 1024, 4)])
def test_stream_read_reads_every_byte(nbytes, grid, in_flight):
    """The probe's XOR of every 32-bit word equals numpy's over the same
    random buffer: every byte was read exactly once (a word read twice
    would cancel out, one skipped would be missing)."""
    _announce(f"stream_read {nbytes} B, grid {grid}, {in_flight} in flight")
    rng = np.random.default_rng(nbytes + grid)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = bd.stream_read(buf, grid=grid, in_flight=in_flight)
    torch.cuda.synchronize()
    want = int(np.bitwise_xor.reduce(host))
    got = int(sink.cpu().numpy().view(np.uint32)[0])
    assert got == want, (hex(got), hex(want))
