"""The C-ABI library: loads, exports what include/s2fast.h declares, validates
arguments on the host, and builds the same RoPE table as the oracle.
CPU only: nothing here launches a kernel."""
import ctypes
import os
import re

import numpy as np
import pytest

from dual_ar_neural_amd import binding as bd
from oracle import fast_ar as fa
from synth import inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "s2fast.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(s2fast_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = bd.library()
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(bd.EXPORTS)


def test_strerror():
    lib = bd.library()
    assert lib.s2fast_strerror(0) == b"ok"
    for code in range(1, 9):
        assert len(lib.s2fast_strerror(code)) > 5
    assert lib.s2fast_strerror(99) == b"unknown error"


@pytest.mark.parametrize("hd,ctx,base", [(128, 11, 1e6), (64, 11, 1e6), (40, 11, 1e6), (128, 16, 1e4)])
def test_rope_table_bit_exact_with_oracle(hd, ctx, base):
    c, s = bd.rope_table(hd, ctx, base)
    oc, os_ = fa.rope_table(hd, ctx, base)
    assert np.array_equal(c.view(np.uint32), oc.view(np.uint32))
    assert np.array_equal(s.view(np.uint32), os_.view(np.uint32))


def _fake_weights(shape, with_layers=True):
    """Distinct aligned fake addresses: enough for host-side validation,
    which never dereferences them."""
    w = bd.Weights()
    addr = [0x100000]

    def nxt():
        addr[0] += 0x1000
        return addr[0]
    w.embeddings, w.norm, w.output = nxt(), nxt(), nxt()
    if shape.has_project_in:
        w.project_in = nxt()
    if with_layers:
        for i in range(shape.n_layer):
            for f in bd.LAYER_FIELDS:
                setattr(w.layers[i], f, nxt())
    return w


def _create(cfg, w):
    ctx = ctypes.c_void_p()
    rc = bd.library().s2fast_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ctx))
    return rc, ctx


def test_create_rejects_missing_fast_decoder():
    cfg = bd.make_config(si.S2PRO, 1)
    w = _fake_weights(si.S2PRO, with_layers=False)
    rc, ctx = _create(cfg, w)
    assert rc == 2 and not ctx.value          # S2FAST_ERR_NO_FAST_DECODER
    w = _fake_weights(si.S2PRO)
    w.output = None
    assert _create(cfg, w)[0] == 2
    w = _fake_weights(si.S2PRO)
    w.layers[3].k_norm = None                 # q/k norm declared but missing
    assert _create(cfg, w)[0] == 2
    cfg_p = bd.make_config(si.S2PRO_PROJ, 1)
    w = _fake_weights(si.S2PRO)               # no project_in pointer
    assert _create(cfg_p, w)[0] == 2


@pytest.mark.parametrize("field,value", [
    ("head_dim", 130), ("head_dim", 63), ("head_dim", 60), ("n_head_kv", 3), ("dim", 2564), ("ffn_dim", 9730),
    ("codebook_size", 9000), ("num_codebooks", 12), ("context", 17), ("n_layer", 9), ("n_layer", 0),
    ("max_batch", 0), ("weight_dtype", 7), ("in_dim", 2048)])
def test_create_rejects_bad_shapes(field, value):
    cfg = bd.make_config(si.S2PRO, 1)
    setattr(cfg, field, value)
    assert _create(cfg, _fake_weights(si.S2PRO))[0] == 1      # S2FAST_ERR_ARG


def test_create_rejects_misaligned_weights():
    cfg = bd.make_config(si.S2PRO, 1)
    w = _fake_weights(si.S2PRO)
    w.layers[1].wo = w.layers[1].wo + 2
    assert _create(cfg, w)[0] == 1


def test_null_arguments():
    lib = bd.library()
    assert lib.s2fast_create(None, None, None) == 1
    assert lib.s2fast_decode_frame(None, 1, None, None, None, None, None, None, None, None) == 1
    assert lib.s2fast_forward_logits(None, 1, None, None, None, None) == 1
    assert lib.s2fast_test_sample(0, 10, None, None, None, None, None, None, None) == 1
    assert lib.s2fast_syncs_per_frame(None, 1) == -1
    assert lib.s2fast_fast_decode(None, 1, None, 256, None, 1, None, None) == 1
    assert lib.s2fast_status(None, None) == 1
    assert lib.s2fast_test_watchdog(None, 1) == 1
    lib.s2fast_destroy(None)


def test_kernel_test_exports_reject_bad_arguments():
    """Checked on the host before any device call."""
    lib = bd.library()
    fake = 0x7F0000000000
    # weight dtype, K not a multiple of the weight vector, M outside 1..2, NULL / misaligned pointers
    assert lib.s2fast_test_gemv(5, 16, 64, 1, fake, None, None, None, None, 1e-6, fake, fake, None) == 1
    assert lib.s2fast_test_gemv(0, 16, 60, 1, fake, None, None, None, None, 1e-6, fake, fake, None) == 1
    assert lib.s2fast_test_gemv(0, 16, 64, 3, fake, None, None, None, None, 1e-6, fake, fake, None) == 1
    assert lib.s2fast_test_gemv(0, 16, 64, 1, None, None, None, None, None, 1e-6, fake, fake, None) == 1
    assert lib.s2fast_test_gemv(0, 16, 64, 1, fake + 4, None, None, None, None, 1e-6, fake, fake, None) == 1
    assert lib.s2fast_test_gemv(0, 0, 64, 1, fake, None, None, None, None, 1e-6, fake, fake, None) == 1
    # heads that do not divide, head_dim not a multiple of 8, T past the context, one norm weight only
    assert lib.s2fast_test_norm_rope_attn(6, 4, 64, 4, 11, 1e6, 1e-6, fake, None, None, fake, None) == 1
    assert lib.s2fast_test_norm_rope_attn(4, 2, 60, 4, 11, 1e6, 1e-6, fake, None, None, fake, None) == 1
    assert lib.s2fast_test_norm_rope_attn(4, 2, 64, 12, 11, 1e6, 1e-6, fake, None, None, fake, None) == 1
    assert lib.s2fast_test_norm_rope_attn(4, 2, 64, 4, 11, 1e6, 1e-6, fake, fake, None, fake, None) == 1
    # streaming probe: NULL / misaligned buffer, size 0 or not a multiple of 16, grid, loads in flight
    assert lib.s2fast_test_stream_read(None, 1024, 256, 4, fake, None) == 1
    assert lib.s2fast_test_stream_read(fake + 8, 1024, 256, 4, fake, None) == 1
    assert lib.s2fast_test_stream_read(fake, 0, 256, 4, fake, None) == 1
    assert lib.s2fast_test_stream_read(fake, 1000, 256, 4, fake, None) == 1
    assert lib.s2fast_test_stream_read(fake, 1024, 0, 4, fake, None) == 1
    assert lib.s2fast_test_stream_read(fake, 1024, 256, 3, fake, None) == 1
    assert lib.s2fast_test_stream_read(fake, 1024, 256, 4, None, None) == 1


# ---------------------------------------------------------------- Slow-AR

def _fake_slow_weights(shape, with_layers=True):
    """Distinct 256-byte-aligned fake device addresses (never dereferenced:
    every case below is rejected before any device call)."""
    from synth import slow_inputs as ssi  # noqa: F401
    base = [0x7F0000000000]

    def nxt():
        base[0] += 1 << 20
        return base[0]
    w = bd.SlowWeights()
    w.embeddings, w.codebook_embeddings, w.norm = nxt(), nxt(), nxt()
    if with_layers:
        for i in range(shape.n_layer):
            for f in bd.LAYER_FIELDS:
                setattr(w.layers[i], f, nxt())
    return w


def _slow_create(cfg, w):
    ctx = ctypes.c_void_p()
    rc = bd.library().s2fast_slow_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ctx))
    return rc, ctx


def test_slow_create_rejects_missing_weights():
    from synth import slow_inputs as ssi
    s = ssi.SLOW_S2PRO
    cfg = bd.make_slow_config(s)
    rc, ctx = _slow_create(cfg, _fake_slow_weights(s, with_layers=False))
    assert rc == 2 and not ctx.value
    w = _fake_slow_weights(s)
    w.codebook_embeddings = None
    assert _slow_create(cfg, w)[0] == 2
    w = _fake_slow_weights(s)
    w.layers[35].q_norm = None
    assert _slow_create(cfg, w)[0] == 2


@pytest.mark.parametrize("field,value", [
    ("num_codebooks", 11), ("num_codebooks", 0), ("head_dim", 12), ("head_dim", 136), ("n_head_kv", 5),
    ("n_head", 96), ("n_layer", 65), ("n_layer", 0), ("semantic_begin", 155000), ("semantic_begin", -1),
    ("end_id", 155776), ("end_id", -3), ("max_context", 0), ("codebook_size", 8192), ("dim", 2564),
    ("ffn_dim", 9730), ("weight_dtype", 3)])
def test_slow_create_rejects_bad_shapes(field, value):
    from synth import slow_inputs as ssi
    s = ssi.SLOW_S2PRO
    cfg = bd.make_slow_config(s)
    setattr(cfg, field, value)
    assert _slow_create(cfg, _fake_slow_weights(s))[0] == 1


def test_slow_create_rejects_misaligned_weights():
    from synth import slow_inputs as ssi
    s = ssi.SLOW_S2PRO
    cfg = bd.make_slow_config(s)
    w = _fake_slow_weights(s)
    w.layers[7].w2 = w.layers[7].w2 + 8
    assert _slow_create(cfg, w)[0] == 1
    w = _fake_slow_weights(s)
    w.embeddings = w.embeddings + 4
    assert _slow_create(cfg, w)[0] == 1


def test_slow_null_arguments():
    lib = bd.library()
    assert lib.s2fast_slow_create(None, None, None) == 1
    assert lib.s2fast_slow_step(None, None, 0, None, None, None, None, None, None, None, None, None, None, None,
                                None) == 1
    assert lib.s2fast_full_frame(None, None, None, 0, None, None, None, None, None, None, None, None, None, None,
                                 None, None) == 1
    assert lib.s2fast_slow_prefill(None, None, 0, 1, None, None, None, None, None, None, None, None, None, None,
                                   None) == 1
    assert lib.s2fast_slow_syncs(None) == -1 and lib.s2fast_slow_allowed(None) == -1
    assert lib.s2fast_test_slow_timeline(None, 1, None, 0) == 1
    assert lib.s2fast_slow_status(None, None) == 1 and lib.s2fast_test_slow_watchdog(None, 0) == 1
    assert lib.s2fast_test_slow_prefill_chunks(None, 1) == 1
    lib.s2fast_slow_destroy(None)


# ---------------------------------------------------------------- weight-only int8

def _fake_q8_scales(shape):
    q = bd.Q8Scales()
    base = [0x7E0000000000]

    def nxt():
        base[0] += 1 << 16
        return base[0]
    q.output = nxt()
    if shape.has_project_in:
        q.project_in = nxt()
    for i in range(shape.n_layer):
        for f, _ in bd.Q8_FIELDS:
            setattr(q.layers[i], f, nxt())
    return q


def test_create_q8_needs_every_row_scale():
    cfg = bd.make_config(si.S2PRO_Q8, 1)
    w = _fake_weights(si.S2PRO_Q8)
    assert _create(cfg, w)[0] == 2                       # no scales at all
    q = _fake_q8_scales(si.S2PRO_Q8)
    q.layers[2].w3 = None
    w.q8_scales = ctypes.pointer(q)
    assert _create(cfg, w)[0] == 2
    q = _fake_q8_scales(si.S2PRO_Q8)
    q.output = None
    w.q8_scales = ctypes.pointer(q)
    assert _create(cfg, w)[0] == 2


def test_create_rejects_scales_without_q8_and_q8_widths():
    cfg = bd.make_config(si.S2PRO, 1)
    w = _fake_weights(si.S2PRO)
    w.q8_scales = ctypes.pointer(_fake_q8_scales(si.S2PRO))
    assert _create(cfg, w)[0] == 1
    cfg = bd.make_config(si.S2PRO_Q8, 1)
    cfg.dim = cfg.in_dim = 2568                          # a multiple of 8, not of 16
    w = _fake_weights(si.S2PRO_Q8)
    w.q8_scales = ctypes.pointer(_fake_q8_scales(si.S2PRO_Q8))
    assert _create(cfg, w)[0] == 1


def test_test_gemv_q8_arguments():
    lib = bd.library()
    fake = 0x7F0000000000
    assert lib.s2fast_test_gemv(2, 16, 64, 1, fake, None, None, None, None, 1e-6, fake, fake, None) == 1  # no scale
    assert lib.s2fast_test_gemv(2, 16, 56, 1, fake, None, fake, None, None, 1e-6, fake, fake, None) == 1  # K % 16
    assert lib.s2fast_test_gemv(0, 16, 64, 1, fake, None, fake, None, None, 1e-6, fake, fake, None) == 1  # scale on bf16
    assert lib.s2fast_test_gemv(2, 16, 64, 1, fake, fake, fake, None, None, 1e-6, fake, fake, None) == 1  # W3 unscaled
