"""GPU parity of cfc_forward_backward (forward and backward in one call)
against the float64 oracle, through the C ABI, at the same per-element
tolerance as the separate calls; plus its relation to the separate calls:
h_seq bitwise equal to cfc_forward's, scratch equal to cfc_backward's to
float32 rounding of the pre-activations (the one-kernel path keeps them in
float64 instead of recomputing them from the float32 h_seq).
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


def fused_step(d, h_seq=None, scratch=None, out=None, accumulate=False):
    import cfc_recurrent_cell_amd as C
    h_seq, scratch, loss = C.cfc_forward_backward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"],
                                                  d["h0"], d["y"], d["dt"], h_seq=h_seq,
                                                  scratch=scratch, accumulate=accumulate)
    out = C.reduce_axis0(scratch, out=out)
    return h_seq, scratch, loss, out


def separate_step(d):
    import cfc_recurrent_cell_amd as C
    h = C.cfc_forward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], d["dt"])
    s, l = C.cfc_backward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], h, d["y"], d["dt"])
    return h, s, l


def _check(inp, what, compare_separate=True):
    say(f"[fused] {what}: B={inp.x.shape[0]} K={inp.x.shape[1]} n_in={inp.x.shape[2]} "
        f"H={inp.w_rec.shape[0]} dt={float(inp.dt)}")
    d = to_dev(inp)
    h, s, l, o = [host(t) for t in fused_step(d)]
    ref = O.cfc_step(inp, threads=oracle_threads())
    assert_close(h, ref["h_seq"], what + " h_seq")
    assert_close(s, ref["scratch"], what + " scratch")
    assert_close(l, ref["loss"], what + " loss")
    assert_close(o, ref["out"], what + " out")
    if compare_separate:
        hs, ss, ls = [host(t) for t in separate_step(d)]
        assert np.array_equal(h.view(np.uint32), hs.view(np.uint32)), what + ": h_seq differs from cfc_forward"
        assert np.array_equal(l.view(np.uint32), ls.view(np.uint32)), what + ": loss differs from cfc_backward"
        assert_close(s, ss, what + " scratch vs cfc_backward", rtol=1e-5, atol=1e-6)
    return d, (h, s, l, o)


def test_fused_tiny():
    _check(W.make_cfc_inputs(W.TINY), W.TINY.name)


def test_fused_smoke():
    _check(W.make_cfc_inputs(W.SMOKE), W.SMOKE.name)


def test_fused_train_ten_steps_bitwise():
    """Training-scale workload through the one-call path: oracle parity, then
    10 repeats with every output poisoned in between, all bitwise equal."""
    import torch
    cfg = W.TRAIN
    d, first = _check(W.make_cfc_inputs(cfg), cfg.name)
    N = W.scratch_row_len(cfg.n_in, cfg.n_hid)
    h_seq = torch.empty((cfg.B, cfg.K, cfg.n_hid), device="cuda")
    scratch = torch.empty((cfg.B, N), device="cuda")
    out = torch.empty((N,), device="cuda")
    for step in range(cfg.steps):
        for t in (h_seq, scratch, out):
            t.fill_(float("nan"))
        got = [host(t) for t in fused_step(d, h_seq=h_seq, scratch=scratch, out=out)]
        for a, b_, name in zip(got, first, ("h_seq", "scratch", "loss", "out")):
            assert np.array_equal(a.view(np.uint32), b_.view(np.uint32)), f"step {step} {name} differs"


FUSED_SHAPES = [
    # (B, K, n_in, H, dt, seed): the one-kernel path ...
    (1, 1, 1, 1, 0.7, 41),
    (3, 5, 21, 37, 0.9, 42),
    (2, 9, 5, 3, 1.3, 43),
    (5, 64, 128, 128, 0.5, 44),    # its K limit at the maximum width
    (4, 17, 128, 7, 1.1, 45),
    (6, 4, 64, 100, 0.0, 46),      # dt = 0
    # ... and the shapes that fall back to two launches
    (3, 65, 16, 24, 0.6, 47),      # K above the one-kernel limit
    (5, 7, 130, 129, 0.6, 48),     # wider than 128
    (2, 6, 256, 256, 1.0, 49),
]


@pytest.mark.parametrize("shape", FUSED_SHAPES, ids=lambda s: "B{}_K{}_n{}_H{}_dt{}".format(*s[:5]))
def test_fused_shapes(shape):
    B, K, n_in, H, dt, seed = shape
    inp = W.make_random_cfc_inputs(B, K, n_in, H, dt, seed)
    _check(inp, f"fused B{B} K{K} n{n_in} H{H}")


def test_fused_b1_rows_bitwise_equal_batched():
    """Rows are independent: each row run alone (B=1) equals its row of the
    batched run bitwise."""
    inp = W.make_random_cfc_inputs(5, 12, 40, 56, 0.8, 50)
    say("[fused] B=1 vs batched")
    h, s, l, _ = [host(t) for t in fused_step(to_dev(inp))]
    for r in range(5):
        one = W.CfcInputs(inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x[r:r + 1], inp.h0[r:r + 1],
                          inp.y[r:r + 1], inp.dt)
        h1, s1, l1, o1 = [host(t) for t in fused_step(to_dev(one))]
        assert np.array_equal(h1[0].view(np.uint32), h[r].view(np.uint32))
        assert np.array_equal(s1[0].view(np.uint32), s[r].view(np.uint32))
        assert np.array_equal(l1.view(np.uint32), l[r:r + 1].view(np.uint32))
        assert np.array_equal(o1.view(np.uint32), s[r].view(np.uint32))   # B=1 reduce is a copy


def test_fused_overwrite_and_accumulate():
    """Overwrite ignores a poisoned scratch; accumulate onto zeros equals
    overwrite bitwise (same kernel); a second accumulate doubles."""
    import torch
    inp = W.make_random_cfc_inputs(4, 10, 24, 40, 0.7, 51)
    d = to_dev(inp)
    say("[fused] overwrite / accumulate")
    _, s_ref, _, _ = fused_step(d)
    s_ref = s_ref.clone()
    poisoned = torch.full_like(s_ref, float("nan"))
    _, s_p, _, _ = fused_step(d, scratch=poisoned)
    assert torch.equal(s_p.view(torch.int32), s_ref.view(torch.int32))
    z = torch.zeros_like(s_ref)
    fused_step(d, scratch=z, accumulate=True)
    assert torch.equal(z.view(torch.int32), s_ref.view(torch.int32))
    fused_step(d, scratch=z, accumulate=True)
    assert_close(host(z), 2.0 * host(s_ref).astype(np.float64), "accumulate twice", rtol=1e-6, atol=1e-7)


def test_fused_refusal_enqueues_nothing():
    """A shape the backward refuses (K = 77 at 128/128) is refused before the
    forward runs: h_seq keeps its poison."""
    import torch
    import cfc_recurrent_cell_amd as C
    inp = W.make_random_cfc_inputs(2, 77, 128, 128, 0.5, 52)
    d = to_dev(inp)
    h_seq = torch.full((2, 77, 128), float("nan"), device="cuda")
    with pytest.raises(C.CfcError) as e:
        C.cfc_forward_backward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], d["y"],
                               d["dt"], h_seq=h_seq)
    assert e.value.code == C.CFC_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(h_seq).all()


WIDE_PARKED = [
    # (B, K, n_in, H, dt, seed, cell): the one-call entry's 16-row path, where
    # the forward parks a_k in the head of each scratch row and the backward
    # reads it back (overwrite mode, even N)
    (37, 7, 200, 256, 0.8, 53, "gated"),     # masked widths, ragged last group
    (17, 20, 256, 256, 0.6, 54, "gated"),    # the 16-row backward's K limit, one row in the last group
    (20, 9, 256, 200, 0.1, 55, "tau_decay"),
    # exactly 256 x 256 with K <= 8: the 32-row forward and phase 2 on the
    # vector units (one workgroup per row)
    (33, 8, 256, 256, 0.7, 56, "gated"),     # a ragged last 32-row group
    (21, 3, 256, 256, 0.3, 57, "tau_decay"),
    # the float64 weight copy lives in scratch rows 0..3: B = 4 is the
    # fewest rows that hold it, B = 3 reads the float32 weights
    (4, 5, 256, 256, 0.5, 58, "gated"),
    (3, 6, 256, 256, 0.5, 59, "tau_decay"),
    (6, 1, 256, 256, 0.4, 60, "gated"),      # one step: no next x, h_prev = h0 only
]


@pytest.mark.parametrize("case", WIDE_PARKED, ids=lambda c: "B{}_K{}_n{}_H{}_{}".format(c[0], c[1], c[2], c[3], c[6]))
def test_fused_wide_parked_preactivations(case):
    """Every scratch element is overwritten (NaN poison gone, oracle parity),
    the input gradients match, and rows run alone equal their batched rows."""
    import torch
    import cfc_recurrent_cell_amd as C
    B, K, n_in, H, dt, seed, cell = case
    inp = W.make_random_cfc_inputs(B, K, n_in, H, dt, seed, cell=cell)
    assert W.scratch_row_len(n_in, H) % 2 == 0
    say(f"[fused] parked a_k: B={B} K={K} n_in={n_in} H={H} {cell}")
    d = to_dev(inp)
    args = (d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], d["y"], d["dt"])
    scratch = torch.full((B, W.scratch_row_len(n_in, H)), float("nan"), device="cuda")
    h, s, l, gx, gh = C.cfc_forward_backward(*args, scratch=scratch, input_grads=True, cell=cell)
    out = C.reduce_axis0(s)
    h, s, l, gx, gh, out = [host(t) for t in (h, s, l, gx, gh, out)]
    assert np.isfinite(s).all()
    ref = O.cfc_step(inp, threads=oracle_threads(), input_grads=True)
    for got, name in ((h, "h_seq"), (s, "scratch"), (l, "loss"), (out, "out"), (gx, "grad_x"), (gh, "grad_h0")):
        assert_close(got, ref[name], f"parked {name}")
    for r in (0, B - 1):
        one = W.CfcInputs(inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x[r:r + 1], inp.h0[r:r + 1],
                          inp.y[r:r + 1], inp.dt, cell)
        d1 = to_dev(one)
        h1, s1, l1 = [host(t) for t in C.cfc_forward_backward(d1["w_in"], d1["w_rec"], d1["b"], d1["w_tau"], d1["x"],
                                                               d1["h0"], d1["y"], d1["dt"], cell=cell)]
        assert np.array_equal(h1[0].view(np.uint32), h[r].view(np.uint32))
        assert np.array_equal(s1[0].view(np.uint32), s[r].view(np.uint32))


@pytest.mark.parametrize("entry", ["fused", "separate"])
def test_accumulate_at_full_width_adds_float32(entry):
    """At 128 x 128 the weight gradients are stored from float32 tiles: in
    accumulate mode every scratch element becomes the float32 sum of its old
    value and the overwrite-mode value (bitwise), and onto zeros accumulate
    equals overwrite."""
    import torch
    import cfc_recurrent_cell_amd as C
    inp = W.make_random_cfc_inputs(3, 64, 128, 128, 0.5, 56)
    d = to_dev(inp)
    say(f"[fused] accumulate at 128x128, {entry}")
    args = (d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"])

    def run(scratch, accumulate):
        if entry == "fused":
            C.cfc_forward_backward(*args, d["y"], d["dt"], scratch=scratch, accumulate=accumulate)
        else:
            h = C.cfc_forward(*args, d["dt"])
            C.cfc_backward(*args, h, d["y"], d["dt"], scratch=scratch, accumulate=accumulate)
        return scratch

    N = W.scratch_row_len(128, 128)
    over = host(run(torch.full((3, N), float("nan"), device="cuda"), False)).copy()
    zero = host(run(torch.zeros((3, N), device="cuda"), True))
    assert np.array_equal(zero.view(np.uint32), over.view(np.uint32))
    base = W.make_random_matrix(3, N, seed=57)
    acc = host(run(torch.from_numpy(base.copy()).cuda(), True))
    want = base.astype(np.float32) + over.astype(np.float32)
    assert np.array_equal(acc.view(np.uint32), want.view(np.uint32))
    ref = O.cfc_step(inp, threads=oracle_threads())
    assert_close(over, ref["scratch"], "overwrite scratch at 128x128")


@pytest.mark.parametrize("cell", ["gated", "tau_decay"])
def test_fused_whole_shape_instance_matches_generic(cell):
    """At K = 64, n_in = H = 128 with 16-byte-aligned x, W_in and W_rec the
    library launches an instance whose staging fetches the projection's
    weights while x is staged and reads W_rec as float4; with x, or W_rec, one
    float off alignment it launches the generic one.  Same arithmetic: every
    output (with the input gradients) bitwise equal, and the aligned one
    within tolerance of the oracle."""
    import torch
    import cfc_recurrent_cell_amd as C
    B, K, n = 4, 64, 128
    inp = W.make_random_cfc_inputs(B, K, n, n, 0.5, 58, cell=cell)
    d = to_dev(inp)
    buf = torch.empty(B * K * n + 1, device="cuda")
    x_off = buf[1:].view(B, K, n)
    x_off.copy_(d["x"])
    wbuf = torch.empty(n * n + 1, device="cuda")
    w_rec_off = wbuf[1:].view(n, n)
    w_rec_off.copy_(d["w_rec"])
    assert d["x"].data_ptr() % 16 == 0 and d["w_in"].data_ptr() % 16 == 0 and x_off.data_ptr() % 16 == 4
    assert d["w_rec"].data_ptr() % 16 == 0 and w_rec_off.data_ptr() % 16 == 4
    say(f"[fused] whole-shape instance vs generic, {cell}")
    outs = []
    for xx, wr in ((d["x"], d["w_rec"]), (x_off, d["w_rec"]), (d["x"], w_rec_off)):
        outs.append([host(t) for t in C.cfc_forward_backward(d["w_in"], wr, d["b"], d["w_tau"], xx, d["h0"],
                                                             d["y"], d["dt"], input_grads=True, cell=cell)])
    for other, what in ((outs[1], "x off alignment"), (outs[2], "W_rec off alignment")):
        for name, a, b_ in zip(("h_seq", "scratch", "loss", "grad_x", "grad_h0"), outs[0], other):
            assert np.array_equal(a.view(np.uint32), b_.view(np.uint32)), f"{cell}, {what}: {name} differs"
    ref = O.cfc_step(inp, threads=oracle_threads())
    assert_close(outs[0][0], ref["h_seq"], cell + " h_seq")
    assert_close(outs[0][1], ref["scratch"], cell + " scratch")
    assert_close(outs[0][2], ref["loss"], cell + " loss")


@pytest.mark.parametrize("cell", ["gated", "tau_decay"])
def test_fused_256_dispatch_variants(cell):
    """At exactly 256 x 256, K <= 8 the one-call entry picks its kernels by
    alignment: the float64 weight copy needs a 16-byte-aligned scratch, the
    vector-unit weight-gradient phase also 16-byte-aligned x, h0 and h_seq.
    All aligned (weight copy, vector phase 2), with x one float off
    alignment (weight copy, matrix-core phase 2) and with the scratch two
    floats off (float32 weights, matrix-core phase 2) every output must be
    bitwise the same -- the widening is exact, and both phase-2 forms sum each
    element's K products in step order -- and within tolerance of the
    oracle."""
    import torch
    import cfc_recurrent_cell_amd as C
    B, K, n = 37, 8, 256
    inp = W.make_random_cfc_inputs(B, K, n, n, 0.7, 61, cell=cell)
    d = to_dev(inp)
    N = W.scratch_row_len(n, n)
    xbuf = torch.empty(B * K * n + 1, device="cuda")
    x_off = xbuf[1:].view(B, K, n)
    x_off.copy_(d["x"])
    sbuf = torch.full((B * N + 2,), float("nan"), device="cuda")
    s_off = sbuf[2:].view(B, N)
    assert x_off.data_ptr() % 16 == 4 and s_off.data_ptr() % 16 == 8 and d["x"].data_ptr() % 16 == 0
    say(f"[fused] 256x256 dispatch variants, {cell}")
    outs = {}
    for name, xx, sc in (("aligned", d["x"], None), ("x_off", x_off, None), ("scratch_off", d["x"], s_off)):
        h, s, l, gx, gh = C.cfc_forward_backward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], xx, d["h0"], d["y"],
                                                 d["dt"], scratch=sc, input_grads=True, cell=cell)
        outs[name] = [host(t) for t in (h, s, l, gx, gh)]
    for other in ("x_off", "scratch_off"):
        for name, a, b_ in zip(("h_seq", "scratch", "loss", "grad_x", "grad_h0"), outs["aligned"], outs[other]):
            assert np.array_equal(a.view(np.uint32), b_.view(np.uint32)), f"{cell}: {name} differs ({other})"
    ref = O.cfc_step(inp, threads=oracle_threads(), input_grads=True)
    for variant, o in outs.items():
        assert np.isfinite(o[1]).all(), variant
        for got, name in zip(o, ("h_seq", "scratch", "loss", "grad_x", "grad_h0")):
            assert_close(got, ref[name], f"{cell} {variant} {name}")
