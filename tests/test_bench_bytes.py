"""The algorithmic byte counts bench.py divides by kernel time, recomputed
from the tensor shapes of the synthetic models (CPU only)."""
import numpy as np

import bench
from oracle import slow_ar as sa
from synth import inputs as si
from synth import slow_inputs as ssi


def _tensor_bytes(shape_fn, names, wb):
    return sum(int(np.prod(shape_fn(n))) * wb for n in names)


def test_slow_step_bytes_from_shapes():
    s = ssi.SLOW_S2PRO
    wb = 2
    layer_names = [n for n in ssi.weight_names(s) if n.startswith("layers.")]
    weights = _tensor_bytes(lambda n: ssi.weight_shape(s, n), layer_names, wb)
    head_rows = sa.allowed_ids(s).size
    for n_past in (0, 2048, 2559):
        want = (weights
                + s.n_layer * s.n_head_kv * 2 * s.head_dim * wb * (n_past + 1)    # cache read + the new row
                + (1 + s.num_codebooks) * s.dim * wb                              # input rows
                + head_rows * s.dim * wb + s.dim * wb + s.dim * 4)               # open head rows, norm, hidden
        assert bench.slow_step_bytes(s, n_past) == want
    # a two-position prefill launch: one weight pass, two input rows sets
    want2 = (weights + s.n_layer * s.n_head_kv * 2 * s.head_dim * wb * (100 + 2)
             + 2 * (1 + s.num_codebooks) * s.dim * wb)
    assert bench.slow_step_bytes(s, 100, head=False, M=2) == want2


def test_fast_frame_bytes_from_shapes():
    s = si.S2PRO
    wb = 2
    names = si.weight_names(s)
    layer = [n for n in names if n.startswith("fast_layers.")]
    per_step = (_tensor_bytes(lambda n: si.weight_shape(s, n), layer, wb)
                + _tensor_bytes(lambda n: si.weight_shape(s, n), ["fast_output", "fast_norm"], wb)
                + s.dim * wb)                                                    # one embedding row
    l0 = _tensor_bytes(lambda n: si.weight_shape(s, n), ["fast_layers.0.attention.wqkv",
                                                         "fast_layers.0.attention_norm"], wb)
    io = s.in_dim * 4 + 4 + s.n_steps * 4 + 3 * 4 + s.num_codebooks * 4
    # steps 2..9 take their layer-0 q/k/v from the table (one float32 row)
    want = s.n_steps * per_step - (s.n_steps - 1) * (l0 - s.qkv_dim * 4) + io
    assert bench.algorithmic_bytes_per_frame(s, 1, True) == want


def test_scope_bytes_are_the_scope_tables_figure():
    """The roofline's bytes: every weight matrix once per decode step
    (7,455,375,360 B a frame at the S2 Pro shape, 828,375,040 a step) plus
    10,332 B of each request's inputs and codes; fast_project_in once per
    frame for the batch-64 workload."""
    s = si.S2PRO
    mats = [n for n in si.weight_names(s) if not n.endswith("norm") and n != "fast_embeddings"]
    per_step = _tensor_bytes(lambda n: si.weight_shape(s, n), mats, 2)
    assert per_step == 828_375_040
    assert bench.scope_bytes_per_frame(s, 1) == 7_455_375_360 + 10_332
    assert bench.scope_bytes_per_frame(s, 16) == 7_455_375_360 + 16 * 10_332
    assert bench.scope_bytes_per_frame(si.S2PRO_PROJ, 64) == 7_455_375_360 + 13_107_200 + 64 * 10_332


def test_scope_bytes_of_the_int8_model():
    """int8 matrices: one byte a weight plus one float32 scale a row."""
    s = si.S2PRO_Q8
    w = si.make_weights(si.TINY_Q8, 1)           # the same tensor set at a small shape
    mats = [n for n in w if w[n].dtype == np.int8]
    per_step_tiny = sum(w[n].size + 4 * w[n].shape[0] for n in mats)
    io = si.TINY_Q8.in_dim * 4 + 4 + 9 * 4 + 12 + 40
    assert bench.scope_bytes_per_frame(si.TINY_Q8, 1) == 9 * per_step_tiny + io
    rows = 4 * (s.qkv_dim + 2 * s.dim + 2 * s.ffn_dim) + s.codebook_size   # wqkv, wo, w1, w3, w2, head
    assert bench.scope_bytes_per_frame(s, 1) == 7_455_375_360 // 2 + 9 * rows * 4 + 10_332


def test_prefill_launch_split_and_bytes():
    """The chunked prefill's launches: the whole prompt in chunks of up to
    64 and a head-only launch, unless the last chunk would hold the last
    position alone (then the positions before it in chunks and the last as
    a step); the comparison path two a launch.  Bytes: every launch's weight
    pass, its cache reads and writes and its input rows; a head-only launch
    its head rows, the final norm and two rows of the state."""
    assert bench.prefill_launches(1, True) == [(0, 1, "step")]
    assert bench.prefill_launches(2, True) == [(0, 2, "chunk"), (1, 1, "head")]
    assert bench.prefill_launches(256, True) == [(0, 64, "chunk"), (64, 64, "chunk"), (128, 64, "chunk"),
                                                 (192, 64, "chunk"), (255, 1, "head")]
    assert bench.prefill_launches(65, True) == [(0, 64, "chunk"), (64, 1, "step")]
    assert bench.prefill_launches(5, False) == [(0, 2, "step"), (2, 2, "step"), (4, 1, "step")]
    s = ssi.SLOW_S2PRO
    wb = 2
    layer_names = [n for n in ssi.weight_names(s) if n.startswith("layers.")]
    weights = _tensor_bytes(lambda n: ssi.weight_shape(s, n), layer_names, wb)
    kv_pos = s.n_layer * s.n_head_kv * 2 * s.head_dim * wb
    row = (1 + s.num_codebooks) * s.dim * wb
    head = sa.allowed_ids(s).size * s.dim * wb + s.dim * wb + s.dim * 4
    assert bench.head_only_bytes(s) == head + s.dim * 4
    # 130 positions from 10: chunks at 10 (64), 74 (64), 138 (2), then the head
    want = (3 * weights + kv_pos * ((10 + 64) + (74 + 64) + (138 + 2)) + 130 * row + head + s.dim * 4)
    assert bench.prefill_bytes(s, 10, 130, True) == want
    # 129 positions from 0: chunks at 0 (64), 64 (64), then position 128 as a step
    want = (3 * weights + kv_pos * (64 + 128 + 129) + 129 * row + head)
    assert bench.prefill_bytes(s, 0, 129, True) == want
