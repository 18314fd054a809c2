"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Every workload is compared element by element -- h_seq, every scratch row,
the per-row loss and the reduced gradient -- at the tolerance rule in
parity_util.  The reducer is also checked against the exact float64 column
sum of the GPU's own scratch ("split parity"), so a reducer error cannot hide
behind a cell error or the other way round.
"""
import numpy as np
import pytest

from parity_util import (assert_close, gpu_step, host, oracle_threads, say, to_dev)
from oracle import oracle as O
from cfc_recurrent_cell_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but torch sees no GPU")
    import cfc_recurrent_cell_amd as C
    C.load_library()          # raises if the HIP library is missing: no fallback
    return torch.device("cuda:0")


def _own_sum_check(out_gpu, scratch_gpu_host, what):
    """GPU reduce vs the float64 sum of the GPU's own float32 rows: the float32
    result must be within one float32 ulp of that sum."""
    own = O.reduce_axis0_f32(scratch_gpu_host)
    want = own.astype(np.float32)
    diff = np.abs(out_gpu.astype(np.float64) - own)
    ulp = np.spacing(np.abs(want)).astype(np.float64)
    bad = np.flatnonzero(diff > ulp)
    assert bad.size == 0, f"{what}: reduce differs from the exact sum of its input by >1 ulp at {bad[:5]}"


def _ulp_check(got_f32, want_f64, what):
    """The forward is float64 inside from float32 inputs, so each h_seq element
    must be within one float32 ulp of the float64 oracle value."""
    want = np.asarray(want_f64, dtype=np.float64)
    diff = np.abs(np.asarray(got_f32, dtype=np.float64) - want)
    ulp = np.spacing(np.abs(want.astype(np.float32))).astype(np.float64)
    bad = np.flatnonzero(diff.ravel() > ulp.ravel())
    assert bad.size == 0, f"{what}: {bad.size} h_seq elements more than 1 float32 ulp from the oracle"


def _full_check(inp, what, threads=None):
    threads = threads or oracle_threads()
    say(f"[parity] {what}: B={inp.x.shape[0]} K={inp.x.shape[1]} n_in={inp.x.shape[2]} "
        f"H={inp.w_rec.shape[0]} dt={float(inp.dt)}")
    d = to_dev(inp)
    h_seq, scratch, loss, out = gpu_step(d)
    g_h, g_s, g_l, g_o = host(h_seq), host(scratch), host(loss), host(out)
    ref = O.cfc_step(inp, threads=threads)
    assert_close(g_h, ref["h_seq"], what + " h_seq")
    _ulp_check(g_h, ref["h_seq"], what)
    assert_close(g_s, ref["scratch"], what + " scratch")
    assert_close(g_l, ref["loss"], what + " loss")
    assert_close(g_o, ref["out"], what + " out")
    _own_sum_check(g_o, g_s, what)
    return d, (g_h, g_s, g_l, g_o)


def test_tiny_workload():
    _full_check(W.make_cfc_inputs(W.TINY), W.TINY.name)


def test_smoke_workload():
    _full_check(W.make_cfc_inputs(W.SMOKE), W.SMOKE.name)


def test_train_workload_ten_steps_bitwise():
    """Training-scale workload, repeated for 10 steps with the scratch cleared at
    each step start: every step matches the oracle and all 10 are bitwise equal
    (the scratch is poisoned with NaN between steps to prove it is rewritten)."""
    import torch
    cfg = W.TRAIN
    inp = W.make_cfc_inputs(cfg)
    d, first = _full_check(inp, cfg.name)
    scratch = torch.empty((cfg.B, W.scratch_row_len(cfg.n_in, cfg.n_hid)), device="cuda")
    out = torch.empty((W.scratch_row_len(cfg.n_in, cfg.n_hid),), device="cuda")
    for step in range(cfg.steps):
        scratch.fill_(float("nan"))
        out.fill_(float("nan"))
        h_seq, scratch, loss, out = gpu_step(d, scratch=scratch, out=out)
        for a, b_, name in zip((host(h_seq), host(scratch), host(loss), host(out)), first,
                               ("h_seq", "scratch", "loss", "out")):
            assert np.array_equal(a.view(np.uint32), b_.view(np.uint32)), f"step {step} {name} differs"


def test_large_workload_all_rows():
    """B=8192, K=8, 256/256 (a 4.31 GB scratch, row offsets past 2^32 bytes),
    through each way the library runs this shape, against the same oracle rows:
      separate    cfc_forward + cfc_backward (16-row forward, recomputing
                  16-row backward);
      one_call    cfc_forward_backward in overwrite mode onto a NaN-poisoned
                  scratch (the forward parks a_k in the head of each scratch
                  row, the backward's two stages read it back and park dL/da
                  in the row's tail);
      accumulate  cfc_forward_backward_ws accumulating onto a base that
                  depends on row and column (a_k and dL/da parked in the
                  workspace, the float64 weight copy after them), compared as
                  result - base;
      bwd_accumulate  cfc_forward + cfc_backward accumulating onto the same
                  base with the workspace (the recomputing reverse pass alone,
                  then the vector weight-gradient phase adding into the
                  scratch), compared as result - base.
    Every h_seq element, every scratch row (block by block), the loss and the
    reduced gradient; each path is then run again and must repeat bitwise."""
    import torch
    import cfc_recurrent_cell_amd as C
    cfg = W.LARGE
    inp = W.make_cfc_inputs(cfg)
    d = to_dev(inp)
    B, K, H, n_in = cfg.B, cfg.K, cfg.n_hid, cfg.n_in
    N = W.scratch_row_len(n_in, H)
    args = (d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"])
    # base[b, j] = (b % 7 - 3) + (j % 5 - 2): small integers, exact in float32
    rowval = (torch.arange(B, device="cuda") % 7 - 3).float()
    colval = (torch.arange(N, device="cuda") % 5 - 2).float()
    ws = torch.empty((C.cfc_forward_backward_workspace(B, K, n_in, H),), dtype=torch.uint8, device="cuda")

    def run(path):
        scratch = torch.empty((B, N), device="cuda")
        if path == "separate":
            h_seq, scratch, loss, out = gpu_step(d, scratch=scratch)
            return h_seq, scratch, loss, out
        if path == "one_call":
            scratch.fill_(float("nan"))
            h_seq, scratch, loss = C.cfc_forward_backward(*args, d["y"], d["dt"], scratch=scratch)
        elif path == "accumulate":
            torch.add(rowval[:, None], colval[None, :], out=scratch)
            h_seq, scratch, loss = C.cfc_forward_backward(*args, d["y"], d["dt"], scratch=scratch,
                                                          accumulate=True, workspace=ws)
        else:
            torch.add(rowval[:, None], colval[None, :], out=scratch)
            h_seq = C.cfc_forward(*args, d["dt"])
            scratch, loss = C.cfc_backward(*args, h_seq, d["y"], d["dt"], scratch=scratch, accumulate=True,
                                           workspace=ws)
        return h_seq, scratch, loss, C.reduce_axis0(scratch)

    paths = ("separate", "one_call", "accumulate", "bwd_accumulate")
    res = {}
    for p in paths:
        say(f"[parity] {cfg.name}: GPU step, {p}")
        res[p] = run(p)
    torch.cuda.synchronize()
    threads = oracle_threads()
    say(f"[parity] {cfg.name}: oracle forward ({threads} threads)")
    ref_h = O.cfc_forward(inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x, inp.h0, inp.dt, threads=threads)
    for p in paths:
        assert_close(host(res[p][0]), ref_h, f"{cfg.name} {p} h_seq")
        _ulp_check(host(res[p][0]), ref_h, f"{cfg.name} {p}")
    ref_out = np.zeros(N)
    own_out = {p: np.zeros(N) for p in paths}
    losses = {p: host(res[p][2]) for p in paths}
    blk = 512
    for r0 in range(0, B, blk):
        r1 = min(B, r0 + blk)
        s, l = O.cfc_backward(inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x[r0:r1], inp.h0[r0:r1],
                              ref_h[r0:r1], inp.y[r0:r1], inp.dt, threads=threads)
        base = None
        for p in paths:
            g = res[p][1][r0:r1].cpu().numpy()
            own_out[p] += O.reduce_axis0_f32(g)
            if p in ("accumulate", "bwd_accumulate"):
                base = (np.arange(r0, r1)[:, None] % 7 - 3) + (np.arange(N)[None, :] % 5 - 2)
                g = g.astype(np.float64) - base
            assert_close(g, s, f"{cfg.name} {p} scratch rows {r0}..{r1}")
            assert_close(losses[p][r0:r1], l, f"{cfg.name} {p} loss rows {r0}..{r1}")
        for r in range(r1 - r0):
            ref_out += s[r]
        say(f"[parity] {cfg.name}: rows {r0}..{r1} ok on every path")
    col_base = float(sum((b % 7) - 3 for b in range(B))) + (np.arange(N) % 5 - 2) * B
    for p in paths:
        g_out = host(res[p][3])
        own = own_out[p]
        diff = np.abs(g_out.astype(np.float64) - own)
        assert np.all(diff <= np.spacing(np.abs(own.astype(np.float32))).astype(np.float64) * 1.0001), p
        if p in ("accumulate", "bwd_accumulate"):
            # the reduced base is an exact integer; the gradient part is checked
            # against the oracle at float32 resolution of the combined sum
            assert_close(g_out.astype(np.float64) - col_base, ref_out, f"{cfg.name} {p} out - base",
                         atol=max(1e-5, float(np.spacing(np.float32(np.abs(col_base).max())))))
        else:
            assert_close(g_out, ref_out, f"{cfg.name} {p} out")
    # a second run of each path is bitwise identical
    for p in paths:
        say(f"[parity] {cfg.name}: bitwise repeat, {p}")
        again = run(p)
        for a, b_, name in zip(again, res[p], ("h_seq", "scratch", "loss", "out")):
            assert torch.equal(a.view(torch.int32), b_.view(torch.int32)), f"{p}: {name} differs on repeat"
        del again
        torch.cuda.synchronize()


RAGGED = [
    # (B, K, n_in, H, dt, seed)
    (1, 1, 1, 1, 0.7, 21),
    (3, 5, 21, 37, 0.9, 22),
    (2, 9, 5, 3, 1.3, 23),
    (5, 7, 130, 129, 0.6, 24),     # H > 128: one thread per unit
    (3, 70, 20, 100, 0.4, 25),     # forward spans two windows of steps
    (4, 3, 256, 256, 1.0, 26),     # the compiled maxima
    (2, 37, 256, 256, 0.3, 27),    # the backward's K limit at 256/256
    (2, 76, 128, 128, 0.5, 28),    # the backward's K limit at 128/128
    (6, 4, 64, 200, 0.0, 29),      # dt = 0
    (7, 2, 3, 64, 2.0, 30),
    (37, 5, 200, 256, 0.8, 36),    # 16-row groups with a ragged last group
    (3, 21, 256, 160, 0.7, 37),    # wide shapes, K above the 16-row backward's limit
]


@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "B{}_K{}_n{}_H{}_dt{}".format(*s[:5]))
def test_ragged_and_edge_shapes(shape):
    B, K, n_in, H, dt, seed = shape
    inp = W.make_random_cfc_inputs(B, K, n_in, H, dt, seed)
    _full_check(inp, f"ragged B{B} K{K} n{n_in} H{H}")


def test_long_forward_only():
    """The forward has no K limit: K = 300 (five windows) against the oracle."""
    import cfc_recurrent_cell_amd as C
    inp = W.make_random_cfc_inputs(3, 300, 16, 24, 0.2, 31, w_scale=0.8)
    say("[parity] forward K=300")
    d = to_dev(inp)
    h = C.cfc_forward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], d["dt"])
    ref = O.cfc_forward(inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x, inp.h0, inp.dt)
    assert_close(host(h), ref, "forward K=300")
    _ulp_check(host(h), ref, "forward K=300")


def test_backward_rejects_k_beyond_lds():
    import torch
    import cfc_recurrent_cell_amd as C
    inp = W.make_random_cfc_inputs(1, 77, 128, 128, 0.5, 32)
    d = to_dev(inp)
    h = C.cfc_forward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], d["dt"])
    with pytest.raises(C.CfcError) as e:
        C.cfc_backward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], h, d["y"], d["dt"])
    assert e.value.code == C.CFC_ERR_UNSUPPORTED
    torch.cuda.synchronize()


def test_b1_rows_bitwise_equal_batched():
    """The pages' B=1 oracle test, on the GPU: each row computed alone gives the
    batched scratch row bit for bit, and the reduce at B=1 is a copy."""
    inp = W.make_cfc_inputs(W.SMOKE)
    say("[parity] B=1 vs batched")
    _, s, l, _ = [host(t) for t in gpu_step(to_dev(inp))]
    for r in (0, 7, 31):
        one = W.CfcInputs(inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x[r:r + 1], inp.h0[r:r + 1],
                          inp.y[r:r + 1], inp.dt)
        _, s1, l1, o1 = [host(t) for t in gpu_step(to_dev(one))]
        assert np.array_equal(s1[0].view(np.uint32), s[r].view(np.uint32))
        assert np.array_equal(o1.view(np.uint32), s1[0].view(np.uint32))
        assert l1[0] == l[r]


def test_permuted_rows():
    inp = W.make_random_cfc_inputs(9, 6, 24, 40, 0.8, 33)
    perm = np.array([4, 8, 0, 3, 7, 1, 6, 2, 5])
    pinp = W.CfcInputs(inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x[perm], inp.h0[perm], inp.y[perm], inp.dt)
    say("[parity] permutation")
    _, s, _, o = [host(t) for t in gpu_step(to_dev(inp))]
    _, sp, _, op = [host(t) for t in gpu_step(to_dev(pinp))]
    assert np.array_equal(sp.view(np.uint32), s[perm].view(np.uint32))
    assert_close(op, o, "permuted out", rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("dims", [(12, 20), (140, 160)], ids=["n12_H20", "n140_H160"])
def test_scratch_clear_and_accumulate_modes(dims):
    """Overwrite mode ignores what the scratch held (NaN poison); accumulate mode
    on a zeroed scratch equals overwrite bitwise (both modes run the same
    kernel: at 140/160 the binding gives accumulate mode the workspace of the
    16-row backward); a second accumulate adds."""
    import torch
    import cfc_recurrent_cell_amd as C
    n_in, H = dims
    a = W.make_random_cfc_inputs(4, 6, n_in, H, 0.7, 34)
    bb = W.make_random_cfc_inputs(4, 6, n_in, H, 0.7, 35)
    say("[parity] scratch clears / accumulate")
    da, db = to_dev(a), to_dev(bb)
    _, fresh_b, _, _ = gpu_step(db)
    fresh_b = fresh_b.clone()
    _, sA, _, _ = gpu_step(da)                  # step A leaves its gradient behind
    _, sB, _, _ = gpu_step(db, scratch=sA)      # step B on different data, same buffer
    assert torch.equal(sB.view(torch.int32), fresh_b.view(torch.int32))
    sA.fill_(float("nan"))
    _, sB2, _, _ = gpu_step(db, scratch=sA)
    assert torch.equal(sB2.view(torch.int32), fresh_b.view(torch.int32))
    z = torch.zeros_like(fresh_b)
    h = C.cfc_forward(db["w_in"], db["w_rec"], db["b"], db["w_tau"], db["x"], db["h0"], db["dt"])
    C.cfc_backward(db["w_in"], db["w_rec"], db["b"], db["w_tau"], db["x"], db["h0"], h, db["y"],
                   db["dt"], scratch=z, accumulate=True)
    assert torch.equal(z.view(torch.int32), fresh_b.view(torch.int32))
    C.cfc_backward(db["w_in"], db["w_rec"], db["b"], db["w_tau"], db["x"], db["h0"], h, db["y"],
                   db["dt"], scratch=z, accumulate=True)
    assert_close(host(z), 2.0 * host(fresh_b).astype(np.float64), "accumulate twice", rtol=1e-6, atol=1e-7)


# ------------------------------------------------------------------ reducer
def test_reduce_workload_normal_and_integer():
    import torch
    import cfc_recurrent_cell_amd as C
    cfg = W.REDUCE
    for integer in (False, True):
        a = W.make_reduce_input(cfg, integer=integer)
        say(f"[parity] reduce {cfg.name} integer={integer}")
        t = torch.from_numpy(a).cuda()
        out = torch.full((cfg.N,), float("nan"), device="cuda")
        C.reduce_axis0(t, out=out)
        g = host(out)
        assert not np.isnan(g).any()
        ref = O.reduce_axis0(a)
        if integer:
            assert np.array_equal(g.astype(np.float64), ref)
            assert np.array_equal(g.astype(np.int64), a.astype(np.int64).sum(0))
        else:
            assert_close(g, ref, "reduce normal")
            _own_sum_check(g, a, "reduce normal")


@pytest.mark.parametrize("B,N", [(0, 37), (1, 7), (3, 4), (5, 1001), (17, 64), (33, 4099),
                                 (1000, 12), (2, 65), (300, 1)])
def test_reduce_edge_sizes(B, N):
    import torch
    import cfc_recurrent_cell_amd as C
    a = W.make_random_matrix(B, N, seed=B * 1000 + N)
    say(f"[parity] reduce B={B} N={N}")
    t = torch.from_numpy(a).cuda()
    out = torch.full((N,), float("nan"), device="cuda")
    C.reduce_axis0(t, out=out)
    g = host(out)
    if B == 0:
        assert np.array_equal(g, np.zeros(N, np.float32))
    else:
        _own_sum_check(g, a, f"reduce B={B} N={N}")
        if B == 1:
            assert np.array_equal(g.view(np.uint32), a[0].view(np.uint32))


def test_reduce_misaligned_rows():
    """A view that starts one float into its storage takes the scalar path."""
    import torch
    import cfc_recurrent_cell_amd as C
    a = W.make_random_matrix(6, 4096, seed=77, integer=True)
    base = torch.zeros(6 * 4096 + 1, device="cuda")
    base[1:] = torch.from_numpy(a.ravel()).cuda()
    view = base[1:].view(6, 4096)
    out = C.reduce_axis0(view)
    assert np.array_equal(host(out).astype(np.int64), a.astype(np.int64).sum(0))


@pytest.mark.parametrize("B,N", [(520, 131580), (70000, 964)])
def test_reduce_inputs_above_256_mb(B, N):
    """Inputs of more than 256 MB take 128-column tiles with 16 rows' loads in
    flight per slot: exact integer sums (a ragged last tile: N % 128 != 0)
    and, on real values, within one float32 ulp of the float64 sum, bitwise
    repeatable."""
    import torch
    import cfc_recurrent_cell_amd as C
    assert B * N * 4 > 256 * 1024 * 1024 and N % 128 != 0
    say(f"[parity] reduce above 256 MB: B={B} N={N}")
    a = W.make_random_matrix(B, N, seed=B + N, integer=True)
    t = torch.from_numpy(a).cuda()
    assert np.array_equal(host(C.reduce_axis0(t)).astype(np.int64), a.astype(np.int64).sum(axis=0))
    del t
    a = W.make_random_matrix(B, N, seed=B + 3 * N)
    t = torch.from_numpy(a).cuda()
    g = host(C.reduce_axis0(t)).copy()
    _own_sum_check(g, a, f"reduce B={B} N={N}")
    assert np.array_equal(g.view(np.uint32), host(C.reduce_axis0(t)).view(np.uint32))
