"""ctypes binding of libs2fast (include/s2fast.h).

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every computation runs in the library's kernels.  The
binding raises if the library is missing — there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import sys
from typing import Dict, Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libs2fast.so")
MAX_LAYERS = 8
BF16, F32, Q8 = 0, 1, 2
DTYPES = {"bf16": BF16, "f32": F32, "q8": Q8}

ERRORS = {
    0: "OK", 1: "ERR_ARG", 2: "ERR_NO_FAST_DECODER", 3: "ERR_HIDDEN_DIM", 4: "ERR_PREFIX_LEN",
    5: "ERR_BATCH", 6: "ERR_HIP", 7: "ERR_NOMEM", 8: "ERR_DEVICE", 9: "ERR_SCRATCH",
}


class S2FastError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {ERRORS.get(code, code)} ({_strerror(code)})")


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "in_dim", "dim", "n_layer", "n_head", "n_head_kv", "head_dim", "ffn_dim",
        "codebook_size", "num_codebooks", "context")] + [
        ("rope_base", ctypes.c_float), ("norm_eps", ctypes.c_float),
        ("has_project_in", ctypes.c_int32), ("has_qk_norm", ctypes.c_int32),
        ("weight_dtype", ctypes.c_int32), ("max_batch", ctypes.c_int32)]


LAYER_FIELDS = ("attention_norm", "wqkv", "q_norm", "k_norm", "wo", "ffn_norm", "w1", "w3", "w2")


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_FIELDS]


Q8_FIELDS = (("wqkv", "attention.wqkv"), ("wo", "attention.wo"), ("w1", "feed_forward.w1"),
             ("w3", "feed_forward.w3"), ("w2", "feed_forward.w2"))


class Q8LayerScales(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n, _ in Q8_FIELDS]


class Q8Scales(ctypes.Structure):
    _fields_ = [("project_in", ctypes.c_void_p), ("output", ctypes.c_void_p),
                ("layers", Q8LayerScales * MAX_LAYERS)]


class Weights(ctypes.Structure):
    _fields_ = [("project_in", ctypes.c_void_p), ("embeddings", ctypes.c_void_p),
                ("norm", ctypes.c_void_p), ("output", ctypes.c_void_p),
                ("layers", LayerWeights * MAX_LAYERS), ("q8_scales", ctypes.POINTER(Q8Scales))]


SLOW_MAX_LAYERS = 64
RAS_WINDOW = 10


class SlowConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "dim", "n_layer", "n_head", "n_head_kv", "head_dim", "ffn_dim", "vocab", "codebook_size",
        "num_codebooks", "semantic_begin", "end_id", "max_context")] + [
        ("rope_base", ctypes.c_float), ("norm_eps", ctypes.c_float),
        ("has_qk_norm", ctypes.c_int32), ("weight_dtype", ctypes.c_int32)]


class SlowWeights(ctypes.Structure):
    _fields_ = [("embeddings", ctypes.c_void_p), ("codebook_embeddings", ctypes.c_void_p),
                ("norm", ctypes.c_void_p), ("layers", LayerWeights * SLOW_MAX_LAYERS)]


_lib = None


def library() -> ctypes.CDLL:
    """Load libs2fast.so (built in-tree by dual_ar_neural_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m dual_ar_neural_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, I, F, V = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
        lib.s2fast_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), ctypes.POINTER(ctypes.c_void_p)]
        lib.s2fast_create.restype = ctypes.c_int
        lib.s2fast_destroy.argtypes = [P]
        lib.s2fast_destroy.restype = None
        lib.s2fast_strerror.argtypes = [ctypes.c_int]
        lib.s2fast_strerror.restype = ctypes.c_char_p
        lib.s2fast_decode_frame.argtypes = [P, I, P, P, P, P, P, P, P, V]
        lib.s2fast_decode_frame.restype = ctypes.c_int
        lib.s2fast_forward_logits.argtypes = [P, I, P, P, P, V]
        lib.s2fast_forward_logits.restype = ctypes.c_int
        lib.s2fast_test_rope_table.argtypes = [I, I, F, P, P]
        lib.s2fast_test_rope_table.restype = ctypes.c_int
        lib.s2fast_test_sample.argtypes = [I, I, P, P, P, P, P, P, V]
        lib.s2fast_test_sample.restype = ctypes.c_int
        lib.s2fast_test_timeline.argtypes = [P, I, P, I]
        lib.s2fast_test_timeline.restype = ctypes.c_int
        lib.s2fast_syncs_per_frame.argtypes = [P, I]
        lib.s2fast_syncs_per_frame.restype = ctypes.c_int
        lib.s2fast_slow_create.argtypes = [ctypes.POINTER(SlowConfig), ctypes.POINTER(SlowWeights),
                                           ctypes.POINTER(ctypes.c_void_p)]
        lib.s2fast_slow_create.restype = ctypes.c_int
        lib.s2fast_slow_destroy.argtypes = [P]
        lib.s2fast_slow_destroy.restype = None
        lib.s2fast_slow_step.argtypes = [P, P, I, P, P, P, P, P, P, P, P, P, P, P, V]
        lib.s2fast_slow_step.restype = ctypes.c_int
        lib.s2fast_slow_prefill.argtypes = [P, P, I, I, P, P, P, P, P, P, P, P, P, P, V]
        lib.s2fast_slow_prefill.restype = ctypes.c_int
        lib.s2fast_full_frame.argtypes = [P, P, P, I, P, P, P, P, P, P, P, P, P, P, P, V]
        lib.s2fast_full_frame.restype = ctypes.c_int
        lib.s2fast_slow_syncs.argtypes = [P]
        lib.s2fast_slow_syncs.restype = ctypes.c_int
        lib.s2fast_slow_allowed.argtypes = [P]
        lib.s2fast_slow_allowed.restype = ctypes.c_int
        lib.s2fast_test_slow_timeline.argtypes = [P, I, P, I]
        lib.s2fast_test_slow_timeline.restype = ctypes.c_int
        lib.s2fast_decode_frame_static.argtypes = [P, I, P, P, P, P, P, P, P, V]
        lib.s2fast_decode_frame_static.restype = ctypes.c_int
        lib.s2fast_fast_decode.argtypes = [P, I, P, I, P, I, P, V]
        lib.s2fast_fast_decode.restype = ctypes.c_int
        lib.s2fast_status.argtypes = [P, V]
        lib.s2fast_status.restype = ctypes.c_int
        lib.s2fast_slow_status.argtypes = [P, V]
        lib.s2fast_slow_status.restype = ctypes.c_int
        lib.s2fast_test_watchdog.argtypes = [P, I]
        lib.s2fast_test_watchdog.restype = ctypes.c_int
        lib.s2fast_test_slow_watchdog.argtypes = [P, I]
        lib.s2fast_test_slow_watchdog.restype = ctypes.c_int
        lib.s2fast_test_slow_prefill_chunks.argtypes = [P, I]
        lib.s2fast_test_slow_prefill_chunks.restype = ctypes.c_int
        lib.s2fast_test_gemv.argtypes = [I, I, I, I, P, P, P, P, P, F, P, P, V]
        lib.s2fast_test_gemv.restype = ctypes.c_int
        lib.s2fast_test_norm_rope_attn.argtypes = [I, I, I, I, I, F, F, P, P, P, P, V]
        lib.s2fast_test_norm_rope_attn.restype = ctypes.c_int
        lib.s2fast_test_stream_read.argtypes = [P, ctypes.c_uint64, I, I, P, V]
        lib.s2fast_test_stream_read.restype = ctypes.c_int
        _lib = lib
    return _lib


EXPORTS = ("s2fast_create", "s2fast_destroy", "s2fast_strerror", "s2fast_decode_frame",
           "s2fast_forward_logits", "s2fast_test_rope_table", "s2fast_test_sample",
           "s2fast_syncs_per_frame", "s2fast_test_timeline", "s2fast_slow_create", "s2fast_slow_destroy",
           "s2fast_slow_step", "s2fast_slow_prefill", "s2fast_full_frame", "s2fast_slow_syncs", "s2fast_slow_allowed",
           "s2fast_test_slow_timeline", "s2fast_fast_decode", "s2fast_status", "s2fast_slow_status",
           "s2fast_test_watchdog", "s2fast_test_slow_watchdog", "s2fast_test_gemv", "s2fast_test_norm_rope_attn",
           "s2fast_decode_frame_static", "s2fast_test_stream_read", "s2fast_test_slow_prefill_chunks")


def _strerror(code: int) -> str:
    try:
        return library().s2fast_strerror(code).decode()
    except Exception:
        return "?"


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise S2FastError(rc, what)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t: torch.Tensor, dtype: torch.dtype, shape: Sequence[int], name: str) -> torch.Tensor:
    if not (t.is_cuda and t.dtype == dtype and tuple(t.shape) == tuple(shape) and t.is_contiguous()):
        raise ValueError(f"{name}: expected contiguous {dtype} CUDA tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")
    return t


def make_config(shape, max_batch: int) -> Config:
    return Config(in_dim=shape.in_dim, dim=shape.dim, n_layer=shape.n_layer, n_head=shape.n_head,
                  n_head_kv=shape.n_head_kv, head_dim=shape.head_dim, ffn_dim=shape.ffn_dim,
                  codebook_size=shape.codebook_size, num_codebooks=shape.num_codebooks,
                  context=shape.context, rope_base=shape.rope_base, norm_eps=shape.norm_eps,
                  has_project_in=int(shape.has_project_in), has_qk_norm=int(shape.has_qk_norm),
                  weight_dtype=DTYPES[shape.weight_dtype], max_batch=max_batch)


def device_weights(shape, weights: Dict[str, "object"], device="cuda") -> Dict[str, torch.Tensor]:
    """Copy host weights (numpy: uint16 bf16 bits, int8 matrices with their
    float32 row scales, or float32) to device tensors."""
    import numpy as np
    out = {}
    for k, v in weights.items():
        if isinstance(v, torch.Tensor):
            out[k] = v.to(device).contiguous()
        elif v.dtype == np.uint16:
            out[k] = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(device).contiguous()
        elif v.dtype == np.int8:
            out[k] = torch.from_numpy(np.ascontiguousarray(v)).to(device)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(device)
    return out


class FastAR:
    """One s2fast context over device-resident weights."""

    def __init__(self, shape, weights: Dict[str, torch.Tensor], max_batch: int = 1):
        self.shape = shape
        self.weights = weights           # keep the device tensors alive
        self.max_batch = max_batch
        lib = library()
        cfg = make_config(shape, max_batch)
        w = Weights()
        g = lambda n: _ptr(weights.get(n))
        w.project_in = g("fast_project_in")
        w.embeddings = g("fast_embeddings")
        w.norm = g("fast_norm")
        w.output = g("fast_output")
        for i in range(shape.n_layer):
            p = f"fast_layers.{i}."
            L = w.layers[i]
            L.attention_norm = g(p + "attention_norm")
            L.wqkv = g(p + "attention.wqkv")
            L.q_norm = g(p + "attention.q_norm")
            L.k_norm = g(p + "attention.k_norm")
            L.wo = g(p + "attention.wo")
            L.ffn_norm = g(p + "ffn_norm")
            L.w1 = g(p + "feed_forward.w1")
            L.w3 = g(p + "feed_forward.w3")
            L.w2 = g(p + "feed_forward.w2")
        if shape.weight_dtype == "q8":
            q = Q8Scales()
            q.project_in = g("fast_project_in.scale")
            q.output = g("fast_output.scale")
            for i in range(shape.n_layer):
                for f, n in Q8_FIELDS:
                    setattr(q.layers[i], f, g(f"fast_layers.{i}.{n}.scale"))
            self._q8 = q
            w.q8_scales = ctypes.pointer(q)
        ctx = ctypes.c_void_p()
        _check(lib.s2fast_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ctx)), "s2fast_create")
        self._ctx = ctx

    def close(self) -> None:
        if getattr(self, "_ctx", None):
            library().s2fast_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        # Never touch the device while the interpreter shuts down: the HIP
        # runtime (or a profiler attached to it) may already be torn down.
        # Close contexts explicitly; at exit the process releases them.
        try:
            if sys.is_finalizing():
                return
            self.close()
        except Exception:
            pass

    def timeline(self, enable: bool = True, fetch: bool = False):
        """Turn per-block phase timing on/off; with fetch, return the last
        frame's marks as numpy [blocks, 256, 8] (100 MHz ticks): per sync
        point, phase done, released, then in-phase marks."""
        import numpy as np
        out = None
        if fetch:
            import torch as _t
            nb = _t.cuda.get_device_properties(0).multi_processor_count
            out = np.zeros((nb, 256, 8), np.uint32)
        _check(library().s2fast_test_timeline(self._ctx, int(enable), None if out is None else out.ctypes.data,
                                              0 if out is None else out.size), "s2fast_test_timeline")
        return out

    def syncs_per_frame(self, B: int) -> int:
        return library().s2fast_syncs_per_frame(self._ctx, B)

    def decode_frame(self, hidden, sem_code, uniforms, temperature, top_p, top_k, codes=None, stream=None,
                     static_scratch: bool = False):
        """One frame for B requests; with static_scratch, through
        s2fast_decode_frame_static (no allocation: the library's static
        per-GPU scratch, the batch-1 kernel per request)."""
        s = self.shape
        B = hidden.shape[0]
        _dev(hidden, torch.float32, (B, s.in_dim), "hidden")
        _dev(sem_code, torch.int32, (B,), "sem_code")
        _dev(uniforms, torch.float32, (B, s.n_steps), "uniforms")
        _dev(temperature, torch.float32, (B,), "temperature")
        _dev(top_p, torch.float32, (B,), "top_p")
        _dev(top_k, torch.int32, (B,), "top_k")
        if codes is None:
            codes = torch.empty((B, s.num_codebooks), dtype=torch.int32, device=hidden.device)
        _dev(codes, torch.int32, (B, s.num_codebooks), "codes")
        fn = library().s2fast_decode_frame_static if static_scratch else library().s2fast_decode_frame
        rc = fn(self._ctx, B, _ptr(hidden), _ptr(sem_code), _ptr(uniforms), _ptr(temperature), _ptr(top_p),
                _ptr(top_k), _ptr(codes), _stream(stream))
        _check(rc, "s2fast_decode_frame_static" if static_scratch else "s2fast_decode_frame")
        return codes

    def status(self, stream=None) -> int:
        """S2FAST_OK, or S2FAST_ERR_HIP if a launch on this context gave up
        a grid-wide wait since the last call (waits for the stream)."""
        return library().s2fast_status(self._ctx, _stream(stream))

    def test_watchdog(self, give_up: bool) -> None:
        _check(library().s2fast_test_watchdog(self._ctx, int(give_up)), "s2fast_test_watchdog")

    def fast_decode(self, hidden, prefix, logits=None, hidden_dim=None, stream=None):
        """One Fast-AR call: logits [B, V] after `prefix` [B, k] (int32)."""
        s = self.shape
        B = hidden.shape[0]
        if not (hidden.is_cuda and hidden.dtype == torch.float32 and hidden.is_contiguous() and hidden.dim() == 2):
            raise ValueError("hidden: expected a contiguous float32 CUDA tensor [B, width]")
        if not (prefix.is_cuda and prefix.dtype == torch.int32 and prefix.is_contiguous() and prefix.dim() == 2
                and prefix.shape[0] == B):
            raise ValueError("prefix: expected a contiguous int32 CUDA tensor [B, k]")
        if logits is None:
            logits = torch.empty((B, s.codebook_size), dtype=torch.float32, device=hidden.device)
        _dev(logits, torch.float32, (B, s.codebook_size), "logits")
        hd = hidden.shape[1] if hidden_dim is None else hidden_dim
        rc = library().s2fast_fast_decode(self._ctx, B, _ptr(hidden), int(hd), _ptr(prefix), int(prefix.shape[1]),
                                          _ptr(logits), _stream(stream))
        _check(rc, "s2fast_fast_decode")
        return logits

    def forward_logits(self, hidden, codes, logits=None, stream=None):
        s = self.shape
        B = hidden.shape[0]
        _dev(hidden, torch.float32, (B, s.in_dim), "hidden")
        _dev(codes, torch.int32, (B, s.num_codebooks), "codes")
        if logits is None:
            logits = torch.empty((B, s.n_steps, s.codebook_size), dtype=torch.float32, device=hidden.device)
        _dev(logits, torch.float32, (B, s.n_steps, s.codebook_size), "logits")
        rc = library().s2fast_forward_logits(self._ctx, B, _ptr(hidden), _ptr(codes), _ptr(logits), _stream(stream))
        _check(rc, "s2fast_forward_logits")
        return logits


def make_slow_config(shape) -> SlowConfig:
    return SlowConfig(dim=shape.dim, n_layer=shape.n_layer, n_head=shape.n_head, n_head_kv=shape.n_head_kv,
                      head_dim=shape.head_dim, ffn_dim=shape.ffn_dim, vocab=shape.vocab,
                      codebook_size=shape.codebook_size, num_codebooks=shape.num_codebooks,
                      semantic_begin=shape.sem_begin, end_id=shape.end_id, max_context=shape.max_ctx,
                      rope_base=shape.rope_base, norm_eps=shape.norm_eps, has_qk_norm=int(shape.has_qk_norm),
                      weight_dtype=BF16 if shape.weight_dtype == "bf16" else F32)


class SlowAR:
    """One Slow-AR step context over device-resident weights."""

    def __init__(self, shape, weights: Dict[str, torch.Tensor]):
        self.shape = shape
        self.weights = weights
        lib = library()
        cfg = make_slow_config(shape)
        w = SlowWeights()
        g = lambda n: _ptr(weights.get(n))
        w.embeddings = g("embeddings")
        w.codebook_embeddings = g("codebook_embeddings")
        w.norm = g("norm")
        for i in range(shape.n_layer):
            p = f"layers.{i}."
            L = w.layers[i]
            for f, n in zip(LAYER_FIELDS, ("attention_norm", "attention.wqkv", "attention.q_norm",
                                           "attention.k_norm", "attention.wo", "ffn_norm", "feed_forward.w1",
                                           "feed_forward.w3", "feed_forward.w2")):
                setattr(L, f, g(p + n))
        ctx = ctypes.c_void_p()
        _check(lib.s2fast_slow_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ctx)), "s2fast_slow_create")
        self._ctx = ctx
        self.n_allowed = lib.s2fast_slow_allowed(ctx)

    def close(self) -> None:
        if getattr(self, "_ctx", None):
            library().s2fast_slow_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        # Never touch the device while the interpreter shuts down: the HIP
        # runtime (or a profiler attached to it) may already be torn down.
        # Close contexts explicitly; at exit the process releases them.
        try:
            if sys.is_finalizing():
                return
            self.close()
        except Exception:
            pass

    def syncs(self) -> int:
        return library().s2fast_slow_syncs(self._ctx)

    def status(self, stream=None) -> int:
        return library().s2fast_slow_status(self._ctx, _stream(stream))

    def test_watchdog(self, give_up: bool) -> None:
        _check(library().s2fast_test_slow_watchdog(self._ctx, int(give_up)), "s2fast_test_slow_watchdog")

    def prefill_chunks(self, enable) -> None:
        """Chunked prefill on (True, the default), off (False: two positions a
        launch), or an int N > 1: chunks only below cache position N."""
        _check(library().s2fast_test_slow_prefill_chunks(self._ctx, int(enable)), "s2fast_test_slow_prefill_chunks")

    def timeline(self, enable: bool = True, fetch: bool = False):
        """Per-block phase timing of later steps (see FastAR.timeline)."""
        import numpy as np
        out = None
        if fetch:
            nb = torch.cuda.get_device_properties(0).multi_processor_count
            out = np.zeros((nb, 256, 8), np.uint32)
        _check(library().s2fast_test_slow_timeline(self._ctx, int(enable), None if out is None else out.ctypes.data,
                                                   0 if out is None else out.size), "s2fast_test_slow_timeline")
        return out

    def kv_dtype(self):
        return torch.bfloat16 if self.shape.weight_dtype == "bf16" else torch.float32

    def _common(self, kv, prev_main, prev_codes, window, temperature, top_p, top_k):
        s = self.shape
        _dev(kv, self.kv_dtype(), (s.n_layer, s.n_head_kv, s.max_ctx, 2, s.head_dim), "kv_cache")
        _dev(prev_main, torch.int32, (1,), "prev_main")
        _dev(prev_codes, torch.int32, (s.num_codebooks,), "prev_codes")
        _dev(window, torch.int32, (1 + RAS_WINDOW,), "window")
        _dev(temperature, torch.float32, (1,), "temperature")
        _dev(top_p, torch.float32, (1,), "top_p")
        _dev(top_k, torch.int32, (1,), "top_k")

    def step(self, kv, n_past: int, prev_main, prev_codes, window, u, temperature, top_p, top_k,
             main_out=None, sem_out=None, hidden_out=None, logits_out=None, stream=None):
        s = self.shape
        self._common(kv, prev_main, prev_codes, window, temperature, top_p, top_k)
        _dev(u, torch.float32, (2,), "u")
        dev = kv.device
        if main_out is None:
            main_out = torch.empty(1, dtype=torch.int32, device=dev)
        if sem_out is None:
            sem_out = torch.empty(1, dtype=torch.int32, device=dev)
        if hidden_out is None:
            hidden_out = torch.empty(s.dim, dtype=torch.float32, device=dev)
        _dev(hidden_out, torch.float32, (s.dim,), "hidden_out")
        if logits_out is not None:
            _dev(logits_out, torch.float32, (self.n_allowed,), "logits_out")
        rc = library().s2fast_slow_step(self._ctx, _ptr(kv), int(n_past), _ptr(prev_main), _ptr(prev_codes),
                                        _ptr(window), _ptr(u), _ptr(temperature), _ptr(top_p), _ptr(top_k),
                                        _ptr(main_out), _ptr(sem_out), _ptr(hidden_out), _ptr(logits_out),
                                        _stream(stream))
        _check(rc, "s2fast_slow_step")
        return main_out, sem_out, hidden_out

    def prefill(self, kv, n_past0: int, tokens, window, u, temperature, top_p, top_k, main_out=None,
                sem_out=None, hidden_out=None, logits_out=None, stream=None):
        """Positions n_past0 .. n_past0 + T - 1 of a prompt (tokens [T, 1 +
        num_codebooks] int32: row-0 token, then codes), then the first main
        token from the last position's logits."""
        s = self.shape
        T = tokens.shape[0]
        _dev(tokens, torch.int32, (T, 1 + s.num_codebooks), "tokens")
        _dev(kv, self.kv_dtype(), (s.n_layer, s.n_head_kv, s.max_ctx, 2, s.head_dim), "kv_cache")
        _dev(window, torch.int32, (1 + RAS_WINDOW,), "window")
        _dev(u, torch.float32, (2,), "u")
        dev = kv.device
        if main_out is None:
            main_out = torch.empty(1, dtype=torch.int32, device=dev)
        if sem_out is None:
            sem_out = torch.empty(1, dtype=torch.int32, device=dev)
        if hidden_out is None:
            hidden_out = torch.empty(s.dim, dtype=torch.float32, device=dev)
        if logits_out is not None:
            _dev(logits_out, torch.float32, (self.n_allowed,), "logits_out")
        rc = library().s2fast_slow_prefill(self._ctx, _ptr(kv), int(n_past0), int(T), _ptr(tokens), _ptr(window),
                                           _ptr(u), _ptr(temperature), _ptr(top_p), _ptr(top_k), _ptr(main_out),
                                           _ptr(sem_out), _ptr(hidden_out), _ptr(logits_out), _stream(stream))
        _check(rc, "s2fast_slow_prefill")
        return main_out, sem_out, hidden_out

    def full_frame(self, fast: "FastAR", kv, n_past: int, prev_main, prev_codes, window, u_slow, u_fast,
                   temperature, top_p, top_k, main_out=None, hidden_out=None, codes_out=None, stream=None):
        s = self.shape
        self._common(kv, prev_main, prev_codes, window, temperature, top_p, top_k)
        _dev(u_slow, torch.float32, (2,), "u_slow")
        _dev(u_fast, torch.float32, (s.num_codebooks - 1,), "u_fast")
        dev = kv.device
        if main_out is None:
            main_out = torch.empty(1, dtype=torch.int32, device=dev)
        if hidden_out is None:
            hidden_out = torch.empty(s.dim, dtype=torch.float32, device=dev)
        if codes_out is None:
            codes_out = torch.empty(s.num_codebooks, dtype=torch.int32, device=dev)
        _dev(hidden_out, torch.float32, (s.dim,), "hidden_out")
        _dev(codes_out, torch.int32, (s.num_codebooks,), "codes_out")
        rc = library().s2fast_full_frame(self._ctx, fast._ctx, _ptr(kv), int(n_past), _ptr(prev_main),
                                         _ptr(prev_codes), _ptr(window), _ptr(u_slow), _ptr(u_fast),
                                         _ptr(temperature), _ptr(top_p), _ptr(top_k), _ptr(main_out),
                                         _ptr(hidden_out), _ptr(codes_out), _stream(stream))
        _check(rc, "s2fast_full_frame")
        return main_out, hidden_out, codes_out


def rope_table(head_dim: int, context: int, base: float):
    """The library's host-built RoPE table (cos, sin) as numpy [context, head_dim/2]."""
    import numpy as np
    c = np.zeros((context, head_dim // 2), np.float32)
    s = np.zeros((context, head_dim // 2), np.float32)
    _check(library().s2fast_test_rope_table(head_dim, context, base, c.ctypes.data, s.ctypes.data),
           "s2fast_test_rope_table")
    return c, s


def stream_read(buf, grid: int = 256, in_flight: int = 4, sink=None, stream=None):
    """The streaming-read probe over a contiguous device tensor (test
    export); returns the int32 device tensor holding the XOR of its words."""
    if not (isinstance(buf, torch.Tensor) and buf.is_cuda and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous device tensor")
    if sink is None:
        sink = torch.empty(1, dtype=torch.int32, device=buf.device)
    _check(library().s2fast_test_stream_read(_ptr(buf), buf.numel() * buf.element_size(), grid, in_flight,
                                             _ptr(sink), _stream(stream)), "s2fast_test_stream_read")
    return sink


def sample(logits, temperature, top_p, top_k, u, stream=None):
    """The device sampler on given logits [B, V] (test export)."""
    B, V = logits.shape
    _dev(logits, torch.float32, (B, V), "logits")
    _dev(temperature, torch.float32, (B,), "temperature")
    _dev(top_p, torch.float32, (B,), "top_p")
    _dev(top_k, torch.int32, (B,), "top_k")
    _dev(u, torch.float32, (B,), "u")
    codes = torch.empty(B, dtype=torch.int32, device=logits.device)
    _check(library().s2fast_test_sample(B, V, _ptr(logits), _ptr(temperature), _ptr(top_p), _ptr(top_k),
                                        _ptr(u), _ptr(codes), _stream(stream)), "s2fast_test_sample")
    return codes


def gemv(W, x, W3=None, norm_w=None, eps: float = 1e-6, scale=None, scale3=None, stream=None):
    """The frame kernel's GEMV on its own (test export): y [M, N] = W . n
    with n = x * norm_w / rms(x) if norm_w is given, or the SwiGLU pair
    silu(W . n) * (W3 . n) if W3 is given.  int8 W (and W3) take their
    float32 row scales."""
    N, K = W.shape
    M = x.shape[0]
    dt = {torch.bfloat16: BF16, torch.float32: F32, torch.int8: Q8}[W.dtype]
    _dev(W, W.dtype, (N, K), "W")
    if W3 is not None:
        _dev(W3, W.dtype, (N, K), "W3")
    if norm_w is not None:
        _dev(norm_w, torch.bfloat16 if dt == Q8 else W.dtype, (K,), "norm_w")
    for t, n in ((scale, "scale"), (scale3, "scale3")):
        if t is not None:
            _dev(t, torch.float32, (N,), n)
    _dev(x, torch.float32, (M, K), "x")
    y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check(library().s2fast_test_gemv(dt, N, K, M, _ptr(W), _ptr(W3), _ptr(scale), _ptr(scale3), _ptr(norm_w),
                                      float(eps), _ptr(x), _ptr(y), _stream(stream)), "s2fast_test_gemv")
    return y


def norm_rope_attn(qkv, n_head: int, n_head_kv: int, head_dim: int, context: int, rope_base: float, eps: float,
                   q_norm=None, k_norm=None, stream=None):
    """q/k RMSNorm + pair RoPE + causal attention of the frame kernel on its
    own (test export): qkv [T, (H + 2 G) hd] raw wqkv outputs -> [T, H hd]."""
    T = qkv.shape[0]
    _dev(qkv, torch.float32, (T, (n_head + 2 * n_head_kv) * head_dim), "qkv")
    for t, n in ((q_norm, "q_norm"), (k_norm, "k_norm")):
        if t is not None:
            _dev(t, torch.float32, (head_dim,), n)
    out = torch.empty((T, n_head * head_dim), dtype=torch.float32, device=qkv.device)
    _check(library().s2fast_test_norm_rope_attn(n_head, n_head_kv, head_dim, T, context, float(rope_base), float(eps),
                                                _ptr(qkv), _ptr(q_norm), _ptr(k_norm), _ptr(out), _stream(stream)),
           "s2fast_test_norm_rope_attn")
    return out
