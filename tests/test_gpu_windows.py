"""GPU parity of the windowed backward (cfc_backward_window: steps
[k_begin, k_end) with dL/dh carried in and out) against the float64 oracle's
whole-sequence backward, through the C ABI -- including sequences longer than
the one-call backward accepts -- and its relation to cfc_backward.
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


def _forward(d, cell="gated"):
    import cfc_recurrent_cell_amd as C
    return C.cfc_forward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], d["dt"], cell=cell)


CASES = [
    # (B, K, n_in, H, dt, seed, window, cell, note)
    (3, 150, 128, 128, 0.5, 91, 64, "gated", "K = 150 > 76 at 128/128: one-row kernels per window"),
    (2, 90, 20, 100, 0.4, 92, 70, "gated", "70-step windows: the general backward"),
    (2, 61, 40, 56, 0.6, 93, 16, "tau_decay", "tau-decay cell, ragged last window"),
    (3, 45, 256, 256, 1.0, 94, 20, "gated", "K = 45 > 37 at 256/256: 16-row kernel, accumulating windows "
                                            "parked in a workspace"),
    (2, 7, 12, 20, 0.9, 95, 1, "gated", "one step per window, as the pages' K launches"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_K{}_n{}_H{}_w{}".format(*c[:4], c[6]))
def test_windowed_backward_matches_oracle(case):
    import torch
    import cfc_recurrent_cell_amd as C
    B, K, n_in, H, dt, seed, window, cell, note = case
    inp = W.make_random_cfc_inputs(B, K, n_in, H, dt, seed, cell=cell)
    say(f"[windows] B={B} K={K} {n_in}/{H} window={window} {cell}: {note}")
    d = to_dev(inp)
    h = _forward(d, cell)
    gx = torch.full((B, K, n_in), float("nan"), device="cuda")
    s, l, gx, gh = C.cfc_backward_windows(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], h, d["y"],
                                          d["dt"], window, grad_x=gx, cell=cell)
    out = C.reduce_axis0(s)
    ref = O.cfc_step(inp, threads=oracle_threads(), input_grads=True)
    assert_close(host(h), ref["h_seq"], "h_seq")
    assert_close(host(s), ref["scratch"], "windowed scratch")
    assert_close(host(l), ref["loss"], "windowed loss")
    assert_close(host(gx), ref["grad_x"], "windowed grad_x")
    assert_close(host(gh), ref["grad_h0"], "windowed grad_h0")
    assert_close(host(out), ref["out"], "windowed out")


@pytest.mark.parametrize("dims", [(20, 30), (140, 160)], ids=["small", "wide"])
def test_one_window_is_cfc_backward(dims):
    """The window [0, K) seeded from y is cfc_backward, bitwise."""
    import torch
    import cfc_recurrent_cell_amd as C
    n_in, H = dims
    inp = W.make_random_cfc_inputs(3, 9, n_in, H, 0.7, 96)
    d = to_dev(inp)
    say(f"[windows] one window {dims}")
    h = _forward(d)
    s_ref, l_ref, gx_ref, gh_ref = C.cfc_backward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], h,
                                                  d["y"], d["dt"], input_grads=True)
    N = s_ref.shape[1]
    s = torch.empty((3, N), device="cuda")
    l = torch.empty((3,), device="cuda")
    gx = torch.empty_like(gx_ref)
    gh = torch.empty_like(gh_ref)
    C.cfc_backward_window(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], h, d["dt"], 0, 9, s,
                          y=d["y"], delta_out=gh, loss=l, grad_x=gx)
    for a, b_ in ((s, s_ref), (l, l_ref), (gx, gx_ref), (gh, gh_ref)):
        assert torch.equal(a.view(torch.int32), b_.view(torch.int32))


def test_upstream_gradient_and_in_place_carry():
    """delta_in supplies dL/dh_K directly (here h_K - y in float32, so the
    result matches the seeded backward to float32 rounding of the seed), and
    carrying the gradient in place equals carrying it between two buffers."""
    import torch
    import cfc_recurrent_cell_amd as C
    inp = W.make_random_cfc_inputs(4, 30, 24, 40, 0.5, 97)
    d = to_dev(inp)
    say("[windows] upstream gradient, in-place carry")
    h = _forward(d)
    args = (d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], h, d["dt"])
    seed = (h[:, -1] - d["y"]).contiguous()
    N = W.scratch_row_len(24, 40)
    # two buffers
    s1 = torch.empty((4, N), device="cuda")
    d_a, d_b = seed.clone(), torch.empty_like(seed)
    C.cfc_backward_window(*args, 12, 30, s1, delta_in=d_a, delta_out=d_b)
    C.cfc_backward_window(*args, 0, 12, s1, delta_in=d_b, delta_out=d_a, accumulate=True)
    # in place
    s2 = torch.empty((4, N), device="cuda")
    d_c = seed.clone()
    C.cfc_backward_window(*args, 12, 30, s2, delta_in=d_c, delta_out=d_c)
    C.cfc_backward_window(*args, 0, 12, s2, delta_in=d_c, delta_out=d_c, accumulate=True)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(d_a.view(torch.int32), d_c.view(torch.int32))
    ref = O.cfc_step(inp, threads=oracle_threads(), input_grads=True)
    assert_close(host(s2), ref["scratch"], "upstream-seeded scratch")
    assert_close(host(d_c), ref["grad_h0"], "upstream-seeded grad_h0")


def test_seeded_window_must_end_at_K():
    import cfc_recurrent_cell_amd as C
    import torch
    inp = W.make_random_cfc_inputs(2, 6, 8, 16, 0.5, 98)
    d = to_dev(inp)
    h = _forward(d)
    s = torch.empty((2, W.scratch_row_len(8, 16)), device="cuda")
    with pytest.raises(C.CfcError) as e:
        C.cfc_backward_window(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], h, d["dt"], 0, 4, s,
                              y=d["y"])
    assert e.value.code == C.CFC_ERR_DIM


@pytest.mark.parametrize("K", [64, 128], ids=["one_window", "two_windows"])
def test_whole_shape_backward_instance_matches_generic(K):
    """64-step windows at 128 x 128 with 16-byte-aligned inputs run an instance
    whose staging fetches the recomputation's weights while [x | h_prev] is
    staged; x one float off alignment runs the generic one.  Same arithmetic:
    scratch, loss, grad_x and dL/dh_0 bitwise equal (the second window's first
    h_prev row comes from h_seq, the first's from h0)."""
    import torch
    import cfc_recurrent_cell_amd as C
    B, n = 3, 128
    inp = W.make_random_cfc_inputs(B, K, n, n, 0.5, 96)
    d = to_dev(inp)
    h = _forward(d)
    buf = torch.empty(B * K * n + 1, device="cuda")
    x_off = buf[1:].view(B, K, n)
    x_off.copy_(d["x"])
    assert d["x"].data_ptr() % 16 == 0 and x_off.data_ptr() % 16 == 4
    say(f"[windows] whole-shape backward instance vs generic, K={K}")
    outs = []
    for xx in (d["x"], x_off):
        gx = torch.empty((B, K, n), device="cuda")
        s, l, gx, gh = C.cfc_backward_windows(d["w_in"], d["w_rec"], d["b"], d["w_tau"], xx, d["h0"], h, d["y"],
                                              d["dt"], 64, grad_x=gx)
        outs.append([host(t) for t in (s, l, gx, gh)])
    for name, a, b_ in zip(("scratch", "loss", "grad_x", "grad_h0"), *outs):
        assert np.array_equal(a.view(np.uint32), b_.view(np.uint32)), f"K={K}: {name} differs between instances"
    ref = O.cfc_step(inp, threads=oracle_threads())
    assert_close(outs[0][0], ref["scratch"], f"K={K} scratch")
    assert_close(outs[0][1], ref["loss"], f"K={K} loss")
