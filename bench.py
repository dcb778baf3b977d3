"""Benchmark of the Fast-AR frame decoder on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A "step" is one s2fast_decode_frame call: the nine decode calls of one frame
for a batch of requests.  The measured workload is the S2 Pro-shaped Fast-AR
(4 layers, dim 2560, 32/8 heads, head_dim 128, ffn 9728, 4096 codes, bf16
weights, float32 arithmetic) at batch 1 with independent synthetic frames
(temperature 0.8, top_p 0.8, top_k 30).  All inputs are on the device before
the timed region; HIP events on the launch stream bracket exactly K frames.

Prints one JSON line: frames/s, per-frame time, the decoder kernel's
achieved algorithmic HBM bandwidth against the 8 TB/s peak, the float32
oracle timed on this host's cores on a few frames, a batch 16/64 sweep, and
the full frame (Slow-AR step from 2048 cached positions, then the Fast-AR
frame) with the Slow-AR kernel's own bandwidth.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "Fast-AR frames/sec (9 codebooks) at batch 1/16/64; achieved HBM GB/s"


def algorithmic_bytes_per_frame(shape, batch: int, qkv0_table: bool) -> int:
    """Bytes a frame of `batch` requests must move at minimum: every weight
    read once per decode step (matrices, norm vectors and one embedding row
    per request), plus each request's inputs and codes.  With qkv0_table the
    steps after the first take their one new row's layer-0 q/k/v from the
    context's precomputed table (one float32 row of qkv_dim per request)
    instead of streaming layer 0's wqkv and attention_norm."""
    s = shape
    wb = 2 if s.weight_dtype == "bf16" else 4
    per_layer = (s.qkv_dim * s.dim + s.dim * s.attn_dim + 2 * s.ffn_dim * s.dim + s.dim * s.ffn_dim
                 + 2 * s.dim + (2 * s.head_dim if s.has_qk_norm else 0)) * wb
    per_step = s.n_layer * per_layer + (s.codebook_size * s.dim + s.dim) * wb + batch * s.dim * wb
    per_frame = s.n_steps * per_step
    if qkv0_table:
        per_frame -= (s.n_steps - 1) * ((s.qkv_dim * s.dim + s.dim) * wb - batch * s.qkv_dim * 4)
    if s.has_project_in:
        per_frame += s.dim * s.in_dim * wb
    io = batch * (s.in_dim * 4 + 4 + s.n_steps * 4 + 3 * 4 + s.num_codebooks * 4)
    return per_frame + io


def scope_bytes_per_frame(shape, batch: int) -> int:
    """The roofline's algorithmic bytes of one frame of `batch` requests:
    every weight matrix (wqkv, wo, w1, w3, w2 of each layer and the untied
    head) once per decode step, fast_project_in once per frame, plus each
    request's inputs and codes (hidden state, semantic code, nine uniforms,
    three sampling settings, ten codes).  7,455,375,360 + 10,332 bytes at
    the S2 Pro shape and batch 1."""
    s = shape
    wb = {"bf16": 2, "f32": 4, "q8": 1}[s.weight_dtype]
    per_step = (s.n_layer * (s.qkv_dim * s.dim + s.dim * s.attn_dim + 3 * s.ffn_dim * s.dim)
                + s.codebook_size * s.dim) * wb
    proj = s.dim * s.in_dim * wb if s.has_project_in else 0
    if s.weight_dtype == "q8":   # plus one float32 scale per matrix row
        per_step += (s.n_layer * (s.qkv_dim + 2 * s.dim + 2 * s.ffn_dim) + s.codebook_size) * 4
        proj += s.dim * 4 if s.has_project_in else 0
    io = batch * (s.in_dim * 4 + 4 + s.n_steps * 4 + 3 * 4 + s.num_codebooks * 4)
    return s.n_steps * per_step + proj + io


def slow_step_bytes(shape, n_past: int, head: bool = True, M: int = 1) -> int:
    """Bytes one Slow-AR launch must move at minimum for the M positions
    n_past .. n_past + M - 1: every layer matrix and norm vector once, the
    input rows (one embedding row and one codebook row per codebook, per
    position), the cache keys/values of positions 0..n_past-1 read and the
    M new positions' written, and the head rows the mask leaves open
    (semantic ids and the end id) plus the final norm."""
    s = shape
    wb = 2 if s.weight_dtype == "bf16" else 4
    per_layer = (s.qkv_dim * s.dim + s.dim * s.attn_dim + 3 * s.ffn_dim * s.dim + 2 * s.dim
                 + (2 * s.head_dim if s.has_qk_norm else 0)) * wb
    kv_pos = s.n_head_kv * 2 * s.head_dim * wb
    kv = s.n_layer * (n_past + M) * kv_pos
    n_allowed = s.codebook_size + (0 if s.sem_begin <= s.end_id <= s.sem_end else 1)
    head_b = (n_allowed + 1) * s.dim * wb + s.dim * 4 if head else 0
    inputs = M * (1 + s.num_codebooks) * s.dim * wb
    return s.n_layer * per_layer + kv + head_b + inputs


def prefill_traffic():
    """HBM bytes per chunked-prefill launch (mean over the profiled chunks)
    from the committed counter summary, if it was taken on the current
    kernel code (else None)."""
    csrc = os.path.join(ROOT, "dual_ar_neural_amd", "csrc")
    rec = traffic_from_profile(os.path.join(ROOT, "profiles", "prefill_kernel_b_s2pro_prefill_hbm_traffic.md"),
                               [os.path.join(csrc, f) for f in ("s2fast.hip", "batched.h", "prefill.h", "slow_host.h",
                                                                "device_common.h")])
    return rec["hbm_bytes_per_launch"] if rec else None


def prefill_launches(T: int, chunks: bool, chunk: int = 64):
    """(first position offset, positions, kind) of each launch the library
    makes for a T-position prefill whose cache positions all fit the chunked
    attention: kind "chunk" (the chunk kernel), "step" (the step kernel:
    layers, head and draw) or "head" (a head-only step launch).  With chunks
    on, the whole prompt runs in chunks of up to `chunk`, the last chunk
    holding the last position, then a head-only launch; when that chunk
    would hold the last position alone ((T - 1) a multiple of `chunk`), the
    positions before the last run in chunks and the last as a step.  With
    chunks off, two positions a launch, the last launch with the head."""
    out, t = [], 0
    if chunks and T >= 2 and (T - 1) % chunk != 0:
        while t < T:
            c = min(chunk, T - t)
            out.append((t, c, "chunk"))
            t += c
        return out + [(T - 1, 1, "head")]
    if chunks:
        while t < T - 1:
            c = min(chunk, T - 1 - t)
            out.append((t, c, "chunk"))
            t += c
    while t < T:
        m = min(2, T - t)
        out.append((t, m, "step"))
        t += m
    return out


def head_only_bytes(shape) -> int:
    """A head-only step launch: the open head rows, the final norm, the
    hidden state written and the last layer's output row read."""
    return slow_step_bytes(shape, 0, head=True, M=1) - slow_step_bytes(shape, 0, head=False, M=1) + shape.dim * 4


def prefill_bytes(shape, n_past0: int, T: int, chunks: bool) -> int:
    """Minimum bytes of a prefill as the library splits it into launches:
    slow_step_bytes of each chunk or step launch (chunks without the head),
    head_only_bytes of a head-only launch."""
    total = 0
    for t, m, kind in prefill_launches(T, chunks):
        if kind == "head":
            total += head_only_bytes(shape)
        else:
            total += slow_step_bytes(shape, n_past0 + t, head=(kind == "step" and t + m == T), M=m)
    return total


def slow_traffic():
    """HBM bytes per Slow-AR launch from the committed counter summary, if it
    was taken on the current kernel code (else None)."""
    csrc = os.path.join(ROOT, "dual_ar_neural_amd", "csrc")
    rec = traffic_from_profile(os.path.join(ROOT, "profiles", "slow_kernel_s2pro_full_frame_hbm_traffic.md"),
                               [os.path.join(csrc, f) for f in ("s2fast.hip", "slow_step.h", "slow_host.h",
                                                                "device_common.h", "sampler.h")])
    return rec["hbm_bytes_per_launch"] if rec else None


def full_frame_cpu(host_slow, kvh, fast_host, fast_shape, inp, n_fill, frames: int):
    """The oracle's full frame (Slow-AR step over the cache, masked draw,
    nine Fast-AR draws) on this host: `frames` chained frames after one
    warm-up frame."""
    from oracle import fast_ar as fa
    from oracle import slow_ar as sa
    from synth import inputs as si
    from synth import slow_inputs as ssi
    s = ssi.SLOW_WORKLOADS["full_s2pro"].shape
    slow = sa.SlowModel.from_weights(s, host_slow)
    fast = fa.Model.from_weights(fast_shape, fast_host)
    kv = si.f32_from_bf16_bits(kvh)
    main, codes, win = int(inp["main"][0]), inp["codes"][0], []
    T, tp, tk = inp["temperature"], inp["top_p"], inp["top_k"]
    t0 = 0.0
    for f in range(frames + 1):
        if f == 1:
            t0 = time.perf_counter()
        r = sa.decode_frame(slow, fast, kv, n_fill + f, main, codes, win, inp["u_slow"][f], inp["u_fast"][f],
                            T, tp, tk)
        kv[:, :, n_fill + f] = r.kv_new
        main, codes, win = r.main.token, r.codes, r.window
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    threads = os.environ.get("OMP_NUM_THREADS")
    if threads and threads.isdigit():
        cores = min(cores, int(threads))
    return {"value": round(frames / dt, 4), "unit": "frames/s", "cores": cores, "kind": "oracle", **host_description(),
            "sample": f"{frames} chained full frames from position {n_fill + 1} after one warm-up frame, "
                      f"{dt:.1f} s wall clock"}


def full_frame_bench(torch, bd, fast_ctx, fast_shape, frames: int, warmup: int, fast_host=None, cpu_frames=0):
    """The full frame (one Slow-AR step, then the Fast-AR frame) at batch 1,
    chained on the device for `frames` frames from 2048 cached positions;
    then the Slow-AR step alone with per-call events for its kernel time.
    With fast_host and cpu_frames > 0, the oracle's full frame is timed on
    the host afterwards."""
    from synth import slow_inputs as ssi
    w = ssi.SLOW_WORKLOADS["full_s2pro"]
    s = w.shape
    frames = max(1, min(frames, s.max_ctx - w.n_fill))
    print(f"[bench] generating {w.name} Slow-AR weights", file=sys.stderr, flush=True)
    host = ssi.make_weights(s, w.seed(0), threads=16)
    dev = bd.device_weights(s, host)
    keep_host = fast_host is not None and cpu_frames > 0
    if not keep_host:
        del host
    kvh = ssi.make_kv_cache(s, w.n_fill, w.seed(5))
    kv = torch.from_numpy(kvh.view(np.int16)).view(torch.bfloat16).cuda()
    if not keep_host:
        del kvh
    slow = bd.SlowAR(s, dev)
    inp = ssi.make_step_inputs(w, frames)
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
    u_slow, u_fast = t(inp["u_slow"], torch.float32), t(inp["u_fast"], torch.float32)
    temp, tp, tk = t([inp["temperature"]], torch.float32), t([inp["top_p"]], torch.float32), t([inp["top_k"]], torch.int32)
    main = t(inp["main"][:1], torch.int32)
    codes = t(inp["codes"][0], torch.int32)
    window = torch.zeros(1 + bd.RAS_WINDOW, dtype=torch.int32, device="cuda")
    hidden = torch.empty(s.dim, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def run(f, pos):
        slow.full_frame(fast_ctx, kv, pos, main, codes, window, u_slow[f], u_fast[f], temp, tp, tk,
                        main_out=main, hidden_out=hidden, codes_out=codes, stream=stream)

    for i in range(warmup):
        run(i % frames, w.n_fill + i)
    torch.cuda.synchronize()
    window.zero_()
    print(f"[bench] timing {frames} full frames", file=sys.stderr, flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for f in range(frames):
        run(f, w.n_fill + f)
    e1.record(stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3
    # the Slow-AR kernel alone, each call between its own events
    n_slow = min(frames, 64)
    sem = torch.empty(1, dtype=torch.int32, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_slow)]
    for f in range(n_slow):
        ev[f][0].record(stream)
        slow.step(kv, w.n_fill + f, main, codes, window, u_slow[f], temp, tp, tk, main_out=main, sem_out=sem,
                  hidden_out=hidden, stream=stream)
        ev[f][1].record(stream)
    torch.cuda.synchronize()
    slow_s = sum(a.elapsed_time(b) for a, b in ev) / 1e3 / n_slow
    slow_b = sum(slow_step_bytes(s, w.n_fill + f) for f in range(n_slow)) / n_slow
    fast_b = algorithmic_bytes_per_frame(fast_shape, 1, True)
    frame_b = sum(slow_step_bytes(s, w.n_fill + f) for f in range(frames)) / frames + fast_b
    out = {"workload": "S2 Pro-shaped full frame: 36-layer Slow-AR step (2048 cached positions, bf16 cache, "
                       "tied head masked to 4096 semantic ids + end id, repetition window 10) then the "
                       "9-codebook Fast-AR frame, batch 1, frames chained on the device",
           "frames": frames, "frames_per_s": round(frames / sec, 2), "ms_per_frame": round(sec * 1e3 / frames, 3),
           "frame_bytes": int(frame_b), "frame_hbm_gbs": round(frame_b * frames / sec / 1e9, 1),
           "frame_frac": round(frame_b * frames / sec / 1e9 / PEAK_HBM_GBS, 4),
           "slow_kernel": {"kernel": "slow_kernel<bf16, 1>", "avg_launch_us": round(slow_s * 1e6, 2),
                           "traffic": slow_traffic(),
                           "bytes_per_launch": int(slow_b), "achieved_gbs": round(slow_b / slow_s / 1e9, 1),
                           "frac": round(slow_b / slow_s / 1e9 / PEAK_HBM_GBS, 4), "syncs": slow.syncs(),
                           "launches": n_slow}}
    # prefill: a prompt of 64 text tokens and 192 reference-audio positions
    # (semantic ids with codes) from position 0; the positions before the
    # last in chunks of up to 64 a launch, then the last with the head and
    # the draw; and the same prompt two positions a launch for comparison
    P, n_text = 256, 64
    rng = np.random.default_rng(w.seed(6))
    toks = np.zeros((P, 1 + s.num_codebooks), np.int32)
    toks[:, 1:] = rng.integers(0, s.codebook_size, size=(P, s.num_codebooks))
    toks[:n_text, 0] = rng.integers(0, s.sem_begin, size=n_text)
    toks[n_text:, 0] = rng.integers(s.sem_begin, s.sem_end + 1, size=P - n_text)
    toks_d = torch.from_numpy(toks).cuda()

    def time_prefill(chunks):
        slow.prefill_chunks(chunks)
        window.zero_()
        slow.prefill(kv, 0, toks_d, window, u_slow[0], temp, tp, tk, main_out=main, sem_out=sem, hidden_out=hidden,
                     stream=stream)
        torch.cuda.synchronize()
        print(f"[bench] timing a {P}-position prefill ({'chunks of 64' if chunks else 'two positions a launch'})",
              file=sys.stderr, flush=True)
        window.zero_()
        e0.record(stream)
        slow.prefill(kv, 0, toks_d, window, u_slow[0], temp, tp, tk, main_out=main, sem_out=sem, hidden_out=hidden,
                     stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3

    psec2 = time_prefill(False)
    psec = time_prefill(True)
    pb = prefill_bytes(s, 0, P, True)
    pb2 = prefill_bytes(s, 0, P, False)
    out["prefill"] = {"workload": f"S2 Pro-shaped Slow-AR prefill of {P} prompt positions ({n_text} text tokens, "
                                  f"{P - n_text} reference-audio positions with codes) from an empty cache: the "
                                  "prompt in chunks of up to 64 positions a launch on the matrix cores (the last "
                                  "chunk runs the last layer in full for the last position), then a head-only "
                                  "launch with the first main-token draw",
                      "positions": P, "positions_per_s": round(P / psec, 1), "ms": round(psec * 1e3, 2),
                      "launches": len(prefill_launches(P, True)),
                      "chunk_traffic": prefill_traffic(),
                      "bytes": int(pb), "hbm_gbs": round(pb / psec / 1e9, 1),
                      "frac": round(pb / psec / 1e9 / PEAK_HBM_GBS, 4),
                      "two_per_launch": {"positions_per_s": round(P / psec2, 1), "ms": round(psec2 * 1e3, 2),
                                         "launches": len(prefill_launches(P, False)), "bytes": int(pb2),
                                         "hbm_gbs": round(pb2 / psec2 / 1e9, 1)}}
    slow.close()
    del dev, kv
    torch.cuda.empty_cache()
    if keep_host:
        print("[bench] timing the oracle's full frame on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = full_frame_cpu(host, kvh, fast_host, fast_shape, ssi.make_step_inputs(w, cpu_frames + 1),
                                             w.n_fill, cpu_frames)
    return out


def probe_hbm(torch, bd):
    """The achievable HBM read rate: the library's streaming-read probe (the
    frame kernel's 16-byte non-temporal load form) over a 2 GiB buffer, eight
    times the memory-side cache, at a few grid sizes and loads in flight;
    the best of five timed launches after one warm-up each."""
    nbytes = 2 << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(7)
    sink = torch.empty(1, dtype=torch.int32, device="cuda")
    best = None
    for grid, inflight in ((256, 4), (256, 8), (512, 4), (1024, 4), (1024, 8)):
        bd.stream_read(buf, grid, inflight, sink)
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            bd.stream_read(buf, grid, inflight, sink)
            e1.record()
            e1.synchronize()
            gbs = nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, grid, inflight)
    del buf, sink
    torch.cuda.empty_cache()
    return {"probe_gbs": round(best[0], 1), "probe_config": f"{best[1]} workgroups x 512 threads, {best[2]} 16-byte "
            f"non-temporal loads in flight a thread, 2 GiB read"}


RUNS = 5   # timed runs of each line; the line reports the median run


def time_frames(torch, ctx, dev_in, B, frames, warmup, runs=1):
    """Decode `warmup` then `frames` frames on the current stream, `runs`
    times (the warm-up only before the first).  Returns (seconds over the
    timed region, mean seconds per decode call) of the median run, and the
    list of every run's (seconds, per call): every call is bracketed by its
    own pair of HIP events on that stream, so the second figure excludes the
    host's gaps between launches."""
    hidden, sem, uni, temp, tp, tk, out = dev_in
    F = hidden.shape[0]
    for i in range(warmup):
        f = i % F
        ctx.decode_frame(hidden[f], sem[f], uni[f], temp, tp, tk, codes=out[f])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    res = []
    for _ in range(runs):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(frames)]
        torch.cuda.synchronize()
        for i in range(frames):
            f = i % F
            ev[i][0].record(stream)
            ctx.decode_frame(hidden[f], sem[f], uni[f], temp, tp, tk, codes=out[f], stream=stream)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        res.append((ev[0][0].elapsed_time(ev[-1][1]) / 1e3, sum(a.elapsed_time(b) for a, b in ev) / 1e3 / frames))
    total, per_call = sorted(res)[len(res) // 2]
    if runs > 1:
        return total, per_call, res
    return total, per_call


def upload(torch, fr):
    d = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
    hidden = d(fr["hidden"], torch.float32)
    F, B = hidden.shape[:2]
    return (hidden, d(fr["sem_code"], torch.int32), d(fr["uniforms"], torch.float32),
            d(fr["temperature"], torch.float32), d(fr["top_p"], torch.float32), d(fr["top_k"], torch.int32),
            torch.empty((F, B, 10), dtype=torch.int32, device="cuda"))


def code_digest(source_files) -> str:
    """sha256 of the kernel sources with comments and whitespace removed, so
    that only code changes count as a kernel change."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in source_files:
        text = open(f).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def traffic_from_profile(path: str, source_files) -> dict | None:
    """HBM bytes per launch of the frame kernel from the committed counter
    summary, if it was taken on the current kernel code (else None)."""
    import re
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("code_sha256") != code_digest(source_files):
        return None
    return rec


def host_description() -> dict:
    """The host the oracle runs on: CPU model and numpy's BLAS."""
    out = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    out["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        out["blas"] = f"{blas.get('name', '?')} {blas.get('version', '')}".strip()
    except Exception:
        pass
    return out


def oracle_leg(workload, frames: int, host_weights, gpu_codes, gpu_logits, batched=()):
    """The oracle on this host: the literal-recompute float32 numpy decoder
    as it stands, BLAS on every core the process may use.  It decodes the
    first `frames` frames of the batch-1 workload teacher-forced along the
    GPU's codes of the timed run (the same windows a free decode computes),
    timed after one warm-up frame; the same run supplies the parity of
    those frames: each GPU code must be one of the oracle draw's defensible
    codes, and the GPU's teacher-forced logits of the same prefixes must lie
    within 1e-2 * max|logit| + 1e-3.  `batched` adds one frame of each batch
    line (workload, host weights, GPU codes, GPU logits), checked the same
    way but not timed."""
    from oracle import fast_ar as fa
    from synth import inputs as si
    w = workload
    model = fa.Model.from_weights(w.shape, host_weights)
    fr = si.make_frames(w, n_frames=frames + 1)

    def one(m, fr_, f, codes):
        return fa.decode_frame(m, fr_["hidden"][f], fr_["sem_code"][f], fr_["uniforms"][f], fr_["temperature"],
                               fr_["top_p"], fr_["top_k"], forced=codes)

    one(model, fr, 0, gpu_codes[0])
    t0 = time.perf_counter()
    refs = [one(model, fr, f, gpu_codes[f]) for f in range(1, frames + 1)]
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    threads = os.environ.get("OMP_NUM_THREADS")
    if threads and threads.isdigit():
        cores = min(cores, int(threads))
    base = {"value": round(w.batch * frames / dt, 4), "unit": "frames/s", "cores": cores, "kind": "oracle",
            **host_description(),
            "sample": f"{frames} frames of {w.name} (batch {w.batch}) after one warm-up frame, teacher-forced "
                      f"along the GPU's codes, {dt:.1f} s wall clock"}

    def check(refs_, codes_, logits_):
        draws = marked = excused = 0
        worst = 0.0
        for r, c, lg in zip(refs_, codes_, logits_):
            for b in range(c.shape[0]):
                for k in range(1, c.shape[1]):
                    alts = r.alts[b][k - 1]
                    draws += 1
                    marked += len(alts) > 1
                    excused += int(c[b, k]) != int(r.codes[b, k])
                    if int(c[b, k]) not in alts:
                        raise AssertionError(f"parity: request {b} step {k}: GPU code {int(c[b, k])} is not "
                                             f"defensible (oracle {int(r.codes[b, k])}, {alts})")
                for k in range(lg.shape[1]):
                    ref = r.logits[b, k]
                    d = float(np.max(np.abs(lg[b, k] - ref)))
                    worst = max(worst, d / (1e-2 * float(np.max(np.abs(ref))) + 1e-3))
        if worst > 1.0:
            raise AssertionError(f"parity: logits {worst:.3g} x the tolerance")
        return {"frames": len(refs_), "draws": draws, "marked": marked, "excused": excused,
                "worst_logit_err_over_tol": float(f"{worst:.3g}")}

    parity = {"b1": check(refs, gpu_codes[1:frames + 1], gpu_logits[1:frames + 1])}
    for name, wb, hw, codes_b, logits_b in batched:
        mb = fa.Model.from_weights(wb.shape, hw)
        frb = si.make_frames(wb, n_frames=1)
        parity[name] = check([one(mb, frb, 0, codes_b)], [codes_b], [logits_b])
    return base, parity


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256, help="timed frames")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the batch 16/64 lines")
    ap.add_argument("--sweep-frames", type=int, default=16, help="timed frames of each batch line")
    ap.add_argument("--cpu-frames", type=int, default=96)
    ap.add_argument("--no-q8", action="store_true", help="skip the weight-only int8 line")
    ap.add_argument("--q8-frames", type=int, default=64)
    ap.add_argument("--no-full-frame", action="store_true", help="skip the full-frame (Slow-AR + Fast-AR) line")
    ap.add_argument("--full-frames", type=int, default=512)
    ap.add_argument("--cpu-full-frames", type=int, default=3)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the decoder runs on a single MI355X; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from dual_ar_neural_amd import binding as bd
    from synth import inputs as si

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = si.WORKLOADS["s2pro_b1"]
    shape = w.shape
    print(f"[bench] generating {w.name} weights", file=sys.stderr, flush=True)
    host = si.make_weights(shape, w.seed(0))
    dev = bd.device_weights(shape, host)
    if args.no_cpu_baseline:
        del host
    ctx = bd.FastAR(shape, dev, max_batch=64)
    n_in = max(args.steps, args.cpu_frames + 1 if not args.no_cpu_baseline else 1)
    fr = si.make_frames(w, n_frames=min(w.frames, n_in))
    dev_in = upload(torch, fr)

    # one elementwise kernel of known traffic (reads 256 MiB, writes 256 MiB),
    # so that counter runs can calibrate their byte counts
    cal = torch.zeros(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
    cal2 = torch.empty_like(cal)
    torch.add(cal, 1.0, out=cal2)
    torch.cuda.synchronize()
    del cal, cal2

    print("[bench] streaming-read probe", file=sys.stderr, flush=True)
    probe = probe_hbm(torch, bd)
    print(f"[bench] timing {args.steps} frames at batch 1", file=sys.stderr, flush=True)
    secs, kern_s, runs = time_frames(torch, ctx, dev_in, 1, args.steps, args.warmup, runs=RUNS)
    B = 1
    frames_per_s = B * args.steps / secs
    ms = secs * 1e3 / args.steps
    bytes_frame = scope_bytes_per_frame(shape, B)                # one launch is one frame at batch 1
    path_bytes = algorithmic_bytes_per_frame(shape, B, True)
    achieved = bytes_frame / kern_s / 1e9
    csrc = os.path.join(ROOT, "dual_ar_neural_amd", "csrc")
    prof = traffic_from_profile(os.path.join(ROOT, "profiles", "frame_kernel_s2pro_b1_hbm_traffic.md"),
                                [os.path.join(csrc, f) for f in ("s2fast.hip", "device_common.h", "sampler.h")])
    traffic = prof["hbm_bytes_per_launch"] if prof else None
    result = {
        "metric": METRIC,
        "value": round(frames_per_s, 3),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "S2 Pro-shaped Fast-AR frame decode, batch 1, independent frames",
                   "batch": 1, "weights": "bf16 (float32 arithmetic)", "dim": shape.dim, "layers": shape.n_layer,
                   "heads": f"{shape.n_head}/{shape.n_head_kv}", "head_dim": shape.head_dim,
                   "ffn": shape.ffn_dim, "codebook": shape.codebook_size, "codebooks": shape.num_codebooks,
                   "sampling": "T 0.8, top_p 0.8, top_k 30"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": "frame_kernel<bf16>", "bytes_per_launch": bytes_frame,
                     "avg_launch_us": round(kern_s * 1e6, 2),
                     "path_bytes_per_launch": path_bytes,
                     "path_frac": round(path_bytes / kern_s / 1e9 / PEAK_HBM_GBS, 4),
                     **probe, "frac_of_probe": round(achieved / probe["probe_gbs"], 4)},
        "syncs_per_frame": ctx.syncs_per_frame(1),
        "timing": f"median of {RUNS} timed runs of {args.steps} frames each (one warm-up of {args.warmup} frames "
                  "before the first); every run's frames/s in runs_frames_per_s",
        "runs_frames_per_s": [round(args.steps / t, 2) for t, _ in runs],
    }
    n_chk = 0 if args.no_cpu_baseline else min(args.cpu_frames + 1, dev_in[0].shape[0])
    if n_chk:
        # the codes of the frames the oracle leg checks (decoded again after
        # the timed region: the decoder is deterministic, so a frame the
        # timed run decoded gets the same codes), and the batch-1 kernel's
        # teacher-forced logits of the same prefixes
        for f in range(n_chk):
            ctx.decode_frame(dev_in[0][f], dev_in[1][f], dev_in[2][f], dev_in[3], dev_in[4], dev_in[5],
                             codes=dev_in[6][f])
        gpu_codes = dev_in[6][:n_chk].cpu().numpy()
        gpu_logits = np.stack([ctx.forward_logits(dev_in[0][f], dev_in[6][f]).cpu().numpy() for f in range(n_chk)])
    batched_chk = []
    if not args.no_sweep:
        sweep = {}
        for Bs, wname in ((16, "s2pro_b16"), (64, "s2pro_b64")):
            ws = si.WORKLOADS[wname]
            hs = None
            if ws.shape is not shape:
                hs = si.make_weights(ws.shape, ws.seed(0))
                ds = bd.device_weights(ws.shape, hs)
                cs = bd.FastAR(ws.shape, ds, max_batch=Bs)
            else:
                ds, cs = None, ctx
            nf = args.sweep_frames
            frs = si.make_frames(ws, n_frames=nf)
            di = upload(torch, frs)
            print(f"[bench] timing {nf} frames at batch {Bs}", file=sys.stderr, flush=True)
            sec, per_call, rs = time_frames(torch, cs, di, Bs, nf, 2, runs=RUNS)
            fb = scope_bytes_per_frame(ws.shape, Bs)
            sweep[f"b{Bs}"] = {"frames_per_s": round(Bs * nf / sec, 2), "ms_per_frame": round(sec * 1e3 / nf, 3),
                               "hbm_gbs": round(fb * nf / sec / 1e9, 1),
                               "frac": round(fb * nf / sec / 1e9 / PEAK_HBM_GBS, 4), "frames": nf,
                               "bytes_per_frame": fb, "kernel_ms_per_frame": round(per_call * 1e3, 3),
                               "launches_per_frame": (Bs + 63) // 64, "workload": ws.name,
                               "runs_frames_per_s": [round(Bs * nf / t, 2) for t, _ in rs]}
            if n_chk:
                c0 = di[6][0].cpu().numpy()
                l0 = cs.forward_logits(di[0][0], di[6][0]).cpu().numpy()
                batched_chk.append((f"b{Bs}", ws, hs if hs is not None else host, c0, l0))
            if cs is not ctx:
                cs.close()
                del ds
            del di
            torch.cuda.empty_cache()
        result["batch_sweep"] = sweep
    if not args.no_q8:
        # weight-only int8 model (int8 matrices with per-row scales), batch 1
        wq = si.WORKLOADS["s2pro_q8"]
        print(f"[bench] generating {wq.name} weights", file=sys.stderr, flush=True)
        hq = si.make_weights(wq.shape, wq.seed(0))
        dq = bd.device_weights(wq.shape, hq)
        cq = bd.FastAR(wq.shape, dq, max_batch=1)
        nq = args.q8_frames
        frq = si.make_frames(wq, n_frames=nq)
        diq = upload(torch, frq)
        print(f"[bench] timing {nq} frames of the int8 model at batch 1", file=sys.stderr, flush=True)
        sec, per_call = time_frames(torch, cq, diq, 1, nq, 4)
        fbq = scope_bytes_per_frame(wq.shape, 1)
        result["q8"] = {"workload": "S2 Pro-shaped Fast-AR with weight-only int8 matrices (one float32 scale per "
                                    "row; bf16 norms and embeddings), batch 1, independent frames",
                        "frames_per_s": round(nq / sec, 2), "ms_per_frame": round(sec * 1e3 / nq, 4),
                        "frames": nq, "kernel": "frame_kernel<int8>", "bytes_per_launch": fbq,
                        "avg_launch_us": round(per_call * 1e6, 2),
                        "achieved_gbs": round(fbq / per_call / 1e9, 1),
                        "frac": round(fbq / per_call / 1e9 / PEAK_HBM_GBS, 4)}
        if n_chk:
            batched_chk.append(("q8", wq, hq, diq[6][0].cpu().numpy(),
                                cq.forward_logits(diq[0][0], diq[6][0]).cpu().numpy()))
        cq.close()
        del dq, diq
        torch.cuda.empty_cache()
    if not args.no_full_frame:
        result["full_frame"] = full_frame_bench(torch, bd, ctx, shape, args.full_frames, 4,
                                                None if args.no_cpu_baseline else host, args.cpu_full_frames)
    ctx.close()
    del dev, dev_in
    torch.cuda.synchronize()
    if n_chk:
        print("[bench] the oracle on the host: timing and parity of the timed frames", file=sys.stderr, flush=True)
        result["cpu_baseline"], result["parity"] = oracle_leg(w, n_chk - 1, host, gpu_codes, gpu_logits,
                                                               batched_chk)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
