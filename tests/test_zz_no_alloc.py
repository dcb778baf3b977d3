"""s2fast_decode_frame_static, the entry point for callers that cannot
allocate (its frame arena and barrier flags live in the library's static
per-GPU scratch), against s2fast_decode_frame on the same inputs: two calls
in a row, the second with fewer requests, each request's codes identical to
a batch-1 s2fast_decode_frame call (the same kernel) and inside the oracle's
defensible set."""
import numpy as np
import pytest
import torch

from dual_ar_neural_amd import binding as bd
from synth import inputs as si
from tests import parity as pr

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[gpu] {msg}", flush=True)


# the three shapes lay the shared scratch out differently, one after another
@pytest.mark.parametrize("wname,batches", [("tiny", (3, 2)), ("ragged", (3, 1)), ("s2pro_b1", (2, 1)),
                                           ("tiny", (1, 1))])
def test_static_scratch_matches_decode_frame(wname, batches):
    w = si.WORKLOADS[wname]
    p = pr.make_pair(w.shape, w.seed(0), max_batch=4)
    fr = si.make_frames(w, n_frames=len(batches), batch=max(batches))
    for call, B in enumerate(batches):
        h, sem, u = fr["hidden"][call][:B], fr["sem_code"][call][:B], fr["uniforms"][call][:B]
        T, tp, tk = fr["temperature"][:B], fr["top_p"][:B], fr["top_k"][:B]
        d = pr.to_dev
        got = p.ctx.decode_frame(d(h), d(sem), d(u), d(T), d(tp), d(tk), static_scratch=True)
        torch.cuda.synchronize()
        got = got.cpu().numpy()
        want = np.concatenate([pr.gpu_decode(p, h[b:b + 1], sem[b:b + 1], u[b:b + 1], T[b:b + 1], tp[b:b + 1],
                                             tk[b:b + 1]) for b in range(B)])
        assert np.array_equal(got, want), (call, got, want)
        pr.check_frame(p, h, sem, u, T, tp, tk, got, logits=False).assert_ok(1e-4)
        _announce(f"static scratch {wname} call {call} B={B}: codes identical")
    assert p.ctx.status() == 0
    p.ctx.close()


def test_static_scratch_rejects_a_shape_larger_than_the_scratch():
    """dim 8192, 8 layers, 16 codebooks: a 23 MiB batch-1 arena."""
    s = si.ModelShape("wide", in_dim=8192, dim=8192, n_layer=8, n_head=1, n_head_kv=1, head_dim=128, ffn_dim=8,
                      codebook_size=2, num_codebooks=16, context=16)
    wts = {n: torch.zeros(si.weight_shape(s, n), dtype=torch.bfloat16, device="cuda") for n in si.weight_names(s)}
    ctx = bd.FastAR(s, wts, max_batch=1)
    z = lambda *shape, dt=torch.float32: torch.zeros(shape, dtype=dt, device="cuda")
    with pytest.raises(bd.S2FastError) as e:
        ctx.decode_frame(z(1, 8192), z(1, dt=torch.int32), z(1, 15), z(1), z(1), z(1, dt=torch.int32),
                         static_scratch=True)
    assert e.value.code == 9
    ctx.close()
