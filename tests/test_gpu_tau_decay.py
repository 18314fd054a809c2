"""GPU parity of the tau-decay cell (the cell the pages print: a per-unit
decay exp(-dt / max(tau, 1e-6)) instead of the gated cell's sigmoid) against
the float64 oracle, through the C ABI, for every kernel and both entry points:
h_seq, every scratch row (dL/dtau in the last slot), the loss, the reduced
gradient and the input gradients.
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


def _run(d, path, accumulate=False, scratch=None):
    import cfc_recurrent_cell_amd as C
    args = (d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"])
    if path == "fused":
        h, s, l, gx, gh = C.cfc_forward_backward(*args, d["y"], d["dt"], scratch=scratch, accumulate=accumulate,
                                                 input_grads=True, cell="tau_decay")
    else:
        h = C.cfc_forward(*args, d["dt"], cell="tau_decay")
        s, l, gx, gh = C.cfc_backward(*args, h, d["y"], d["dt"], scratch=scratch, accumulate=accumulate,
                                      input_grads=True, cell="tau_decay")
    out = C.reduce_axis0(s)
    return [host(t) for t in (h, s, l, gx, gh, out)]


def _check(inp, what, path):
    say(f"[tau decay] {what} ({path})")
    h, s, l, gx, gh, out = _run(to_dev(inp), path)
    ref = O.cfc_step(inp, threads=oracle_threads(), input_grads=True)
    assert_close(h, ref["h_seq"], what + " h_seq")
    assert_close(s, ref["scratch"], what + " scratch")
    assert_close(l, ref["loss"], what + " loss")
    assert_close(out, ref["out"], what + " out")
    assert_close(gx, ref["grad_x"], what + " grad_x")
    assert_close(gh, ref["grad_h0"], what + " grad_h0")
    return h, s


@pytest.mark.parametrize("path", ["separate", "fused"])
def test_tau_tiny_workload(path):
    _check(W.make_cfc_inputs(W.TAU_TINY), W.TAU_TINY.name, path)


@pytest.mark.parametrize("path", ["separate", "fused"])
def test_tau_training_workload(path):
    _check(W.make_cfc_inputs(W.TAU_TRAIN), W.TAU_TRAIN.name, path)


SHAPES = [
    # (B, K, n_in, H, dt, seed, note)
    (3, 5, 21, 37, 0.3, 81, "one row per workgroup"),
    (2, 70, 20, 100, 0.05, 82, "general backward (K > 64)"),
    (5, 7, 130, 129, 0.2, 83, "16-row kernels, masked"),
    (3, 6, 256, 256, 0.5, 84, "16-row kernels, unmasked"),
    (3, 21, 256, 160, 0.1, 85, "general backward (wide, K > 20)"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}_K{}_n{}_H{}".format(*s[:4]))
@pytest.mark.parametrize("path", ["separate", "fused"])
def test_tau_shapes(shape, path):
    B, K, n_in, H, dt, seed, note = shape
    _check(W.make_random_cfc_inputs(B, K, n_in, H, dt, seed, cell="tau_decay"),
           f"B{B} K{K} n{n_in} H{H} ({note})", path)


@pytest.mark.parametrize("dims", [(12, 20), (140, 160), (256, 256)], ids=["small", "masked16", "full16"])
def test_tau_guard_units(dims):
    """Units with tau <= 1e-6 decay to 0 (h = tanh(a)) and get dL/dtau = 0
    exactly, on every kernel family."""
    n_in, H = dims
    inp = W.make_random_cfc_inputs(4, 5, n_in, H, 0.5, 86, cell="tau_decay")
    tau = inp.w_tau.copy()
    tau[[0, 3, H - 1]] = [0.0, -1.0, 1e-7]
    inp = W.CfcInputs(inp.w_in, inp.w_rec, inp.b, tau, inp.x, inp.h0, inp.y, inp.dt, "tau_decay")
    h, s = _check(inp, f"guard {dims}", "separate")
    N = s.shape[1]
    for u in (0, 3, H - 1):
        assert np.all(s[:, N - H + u] == 0.0)


@pytest.mark.parametrize("dims", [(12, 20), (140, 160)], ids=["small", "wide"])
def test_tau_accumulate_mode(dims):
    """Accumulate mode onto zeros equals the oracle; twice doubles it."""
    import torch
    n_in, H = dims
    inp = W.make_random_cfc_inputs(3, 4, n_in, H, 0.3, 87, cell="tau_decay")
    d = to_dev(inp)
    say(f"[tau decay] accumulate {dims}")
    z = torch.zeros((3, W.scratch_row_len(n_in, H)), device="cuda")
    _run(d, "separate", accumulate=True, scratch=z)
    ref = O.cfc_step(inp, threads=oracle_threads())
    assert_close(host(z), ref["scratch"], "tau accumulate once")
    _run(d, "separate", accumulate=True, scratch=z)
    assert_close(host(z), 2.0 * ref["scratch"], "tau accumulate twice")


def test_tau_cells_differ_and_rows_independent():
    """The two cells give different results on the same arrays, and tau-decay
    rows run alone (B=1) equal their batched rows bitwise."""
    inp = W.make_random_cfc_inputs(4, 6, 30, 40, 0.3, 88, cell="tau_decay")
    d = to_dev(inp)
    say("[tau decay] cells differ, B=1 vs batched")
    h, s, l, gx, gh, _ = _run(d, "fused")
    import cfc_recurrent_cell_amd as C
    hg = host(C.cfc_forward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], d["dt"]))
    assert not np.allclose(hg, h)
    for r in range(4):
        one = W.CfcInputs(inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x[r:r + 1], inp.h0[r:r + 1],
                          inp.y[r:r + 1], inp.dt, "tau_decay")
        h1, s1, l1, gx1, gh1, _ = _run(to_dev(one), "fused")
        for a, b_ in ((h1[0], h[r]), (s1[0], s[r]), (gx1[0], gx[r]), (gh1[0], gh[r])):
            assert np.array_equal(a.view(np.uint32), b_.view(np.uint32))
