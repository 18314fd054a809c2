"""GPU parity of the optional input gradients (grad_x = dL/dx_k for every
step, grad_h0 = dL/dh_0) against the float64 oracle, through the C ABI, for
every backward kernel and both entry points; requesting them must leave the
other outputs bitwise unchanged.
"""
import numpy as np
import pytest

from parity_util import assert_close, host, oracle_threads, say, to_dev
from oracle import oracle as O
from cfc_recurrent_cell_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but torch sees no GPU")
    import cfc_recurrent_cell_amd as C
    C.load_library()
    return torch.device("cuda:0")


def _separate(d, accumulate=False, input_grads=True):
    import torch
    import cfc_recurrent_cell_amd as C
    h = C.cfc_forward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], d["dt"])
    scratch = torch.zeros((d["x"].shape[0], C.cfc_scratch_row_len(d["x"].shape[2], d["w_rec"].shape[0])),
                          device="cuda") if accumulate else None
    r = C.cfc_backward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], h, d["y"], d["dt"],
                       scratch=scratch, accumulate=accumulate, input_grads=input_grads)
    return (h,) + tuple(r)


def _fused(d, input_grads=True):
    import cfc_recurrent_cell_amd as C
    return C.cfc_forward_backward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], d["y"],
                                  d["dt"], input_grads=input_grads)


SHAPES = [
    # (B, K, n_in, H, dt, seed, note)
    (3, 5, 21, 37, 0.9, 61, "one row per workgroup"),
    (2, 64, 128, 128, 0.5, 62, "one row per workgroup, both limits"),
    (1, 1, 1, 1, 0.7, 63, "degenerate"),
    (2, 70, 20, 100, 0.4, 64, "general backward (K > 64)"),
    (5, 7, 130, 129, 0.6, 65, "16-row kernels, masked"),
    (3, 6, 256, 256, 1.0, 66, "16-row kernels, unmasked"),
    (37, 5, 200, 256, 0.8, 67, "16-row kernels, ragged last group"),
    (3, 21, 256, 160, 0.7, 68, "general backward (wide, K > 20)"),
    (4, 3, 7, 200, 0.0, 69, "dt = 0"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}_K{}_n{}_H{}".format(*s[:4]))
@pytest.mark.parametrize("path", ["separate", "fused"])
def test_input_grads_match_oracle(shape, path):
    B, K, n_in, H, dt, seed, note = shape
    inp = W.make_random_cfc_inputs(B, K, n_in, H, dt, seed)
    what = f"{path} B{B} K{K} n{n_in} H{H} ({note})"
    say(f"[input grads] {what}")
    d = to_dev(inp)
    run = _separate if path == "separate" else _fused
    h, s, l, gx, gh = [host(t) for t in run(d)]
    ref = O.cfc_step(inp, threads=oracle_threads(), input_grads=True)
    assert_close(gx, ref["grad_x"], what + " grad_x")
    assert_close(gh, ref["grad_h0"], what + " grad_h0")
    assert_close(s, ref["scratch"], what + " scratch")
    # asking for the input gradients changes nothing else
    h2, s2, l2 = [host(t) for t in run(d, input_grads=False)]
    for a, b_, name in ((h, h2, "h_seq"), (s, s2, "scratch"), (l, l2, "loss")):
        assert np.array_equal(a.view(np.uint32), b_.view(np.uint32)), f"{what}: {name} changed"


def test_input_grads_accumulate_mode_wide():
    """Accumulate mode at width > 128 takes the general backward: its input
    gradients are overwritten (not accumulated) and match the oracle."""
    inp = W.make_random_cfc_inputs(3, 4, 140, 160, 0.7, 70)
    d = to_dev(inp)
    say("[input grads] accumulate, wide")
    _, s, _, gx, gh = [host(t) for t in _separate(d, accumulate=True)]
    ref = O.cfc_step(inp, threads=oracle_threads(), input_grads=True)
    assert_close(gx, ref["grad_x"], "accumulate grad_x")
    assert_close(gh, ref["grad_h0"], "accumulate grad_h0")
    assert_close(s, ref["scratch"], "accumulate scratch (onto zeros)")


def test_input_grads_training_workload():
    """The training-scale workload through the one-kernel path."""
    cfg = W.TRAIN
    inp = W.make_cfc_inputs(cfg)
    say(f"[input grads] {cfg.name}")
    d = to_dev(inp)
    _, _, _, gx, gh = [host(t) for t in _fused(d)]
    ref = O.cfc_step(inp, threads=oracle_threads(), input_grads=True)
    assert_close(gx, ref["grad_x"], cfg.name + " grad_x")
    assert_close(gh, ref["grad_h0"], cfg.name + " grad_h0")


def test_input_grads_large_shape_rows():
    """The large-batch workload's shape (K=8, 256/256) on 40 of its rows:
    three 16-row workgroups, the last one ragged."""
    cfg = W.LARGE
    inp = W.make_cfc_inputs(cfg, B=40)
    say(f"[input grads] {cfg.name}, 40 rows")
    d = to_dev(inp)
    _, s, _, gx, gh = [host(t) for t in _separate(d)]
    ref = O.cfc_step(inp, threads=oracle_threads(), input_grads=True)
    assert_close(gx, ref["grad_x"], "large grad_x")
    assert_close(gh, ref["grad_h0"], "large grad_h0")
    assert_close(s, ref["scratch"], "large scratch")


@pytest.mark.parametrize("dims", [(40, 56), (200, 256)], ids=["n40_H56", "n200_H256"])
def test_input_grads_b1_rows_bitwise_equal_batched(dims):
    n_in, H = dims
    inp = W.make_random_cfc_inputs(5, 6, n_in, H, 0.8, 71)
    say(f"[input grads] B=1 vs batched {dims}")
    _, _, _, gx, gh = [host(t) for t in _separate(to_dev(inp))]
    for r in range(5):
        one = W.CfcInputs(inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x[r:r + 1], inp.h0[r:r + 1],
                          inp.y[r:r + 1], inp.dt)
        _, _, _, gx1, gh1 = [host(t) for t in _separate(to_dev(one))]
        assert np.array_equal(gx1[0].view(np.uint32), gx[r].view(np.uint32))
        assert np.array_equal(gh1[0].view(np.uint32), gh[r].view(np.uint32))
