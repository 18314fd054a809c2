"""GPU parity of accumulate mode at widths above 128 with a caller workspace
(cfc_backward_window_ws): the 16-row backward parks dL/da in the workspace
instead of the scratch tail and adds its float32 gradient into the scratch.
Checked bitwise against the same kernel's overwrite mode, against the float64
oracle, and against the general backward that accumulate mode runs without a
workspace.
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


CASES = [
    # (B, K, n_in, H, dt, seed, cell, note)
    (20, 8, 256, 256, 1.0, 131, "gated", "unmasked 256 x 256, two row groups (16 + 4)"),
    (19, 20, 200, 140, 0.7, 132, "gated", "masked widths, K at the 16-row bound"),
    (17, 5, 256, 256, 0.05, 133, "tau_decay", "tau-decay cell, unmasked"),
    (3, 11, 130, 96, 0.8, 134, "tau_decay", "one partial row group, n_in alone above 128"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_K{}_n{}_H{}_{}".format(*c[:4], c[6]))
def test_wide_accumulate_with_workspace(case):
    """Onto zeros, accumulate equals overwrite bitwise; onto random values it
    is their float32 sum with the overwrite gradient, bitwise; loss, grad_x and
    grad_h0 are the overwrite call's; the workspace's contents on entry do not
    matter; and the result is within tolerance of the oracle and of the
    general backward's accumulate mode."""
    import torch
    import cfc_recurrent_cell_amd as C
    B, K, n_in, H, dt, seed, cell, note = case
    say(f"[wide accumulate] B={B} K={K} {n_in}/{H} {cell}: {note}")
    inp = W.make_random_cfc_inputs(B, K, n_in, H, dt, seed, cell=cell)
    d = to_dev(inp)
    args = (d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"])
    h = C.cfc_forward(*args, d["dt"], cell=cell)
    N = W.scratch_row_len(n_in, H)
    need = C.cfc_backward_workspace(B, K, n_in, H, accumulate=True)
    assert need == 8 * B * K * H
    ws = torch.full((need // 4,), float("nan"), device="cuda")   # float32 NaN words: contents ignored

    def run(scratch, accumulate, workspace, general=False):
        gx = torch.full((B, K, n_in), float("nan"), device="cuda")
        gh = torch.full((B, H), float("nan"), device="cuda")
        loss = torch.full((B,), float("nan"), device="cuda")
        if general:   # cfc_backward_window without a workspace: the general backward
            C.cfc_backward_window(*args, h, d["dt"], 0, K, scratch, y=d["y"], delta_out=gh, loss=loss,
                                  grad_x=gx, accumulate=accumulate, cell=cell)
        else:
            C.cfc_backward(*args, h, d["y"], d["dt"], scratch=scratch, loss=loss, grad_x=gx, grad_h0=gh,
                           accumulate=accumulate, cell=cell, workspace=workspace)
        return [host(t).copy() for t in (scratch, loss, gx, gh)]

    over = run(torch.full((B, N), float("nan"), device="cuda"), False, None)
    zero = run(torch.zeros((B, N), device="cuda"), True, ws)
    for a, b, name in zip(zero, over, ("scratch", "loss", "grad_x", "grad_h0")):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"accumulate onto zeros: {name}"
    base = W.make_random_matrix(B, N, seed=seed + 1000)
    acc = run(torch.from_numpy(base.copy()).cuda(), True, ws)
    want = base.astype(np.float32) + over[0]
    assert np.array_equal(acc[0].view(np.uint32), want.view(np.uint32))
    for a, b, name in zip(acc[1:], over[1:], ("loss", "grad_x", "grad_h0")):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"accumulate onto values: {name}"
    ref = O.cfc_step(inp, threads=oracle_threads(), input_grads=True)
    assert_close(over[0], ref["scratch"], "overwrite scratch")
    assert_close(acc[0] - base.astype(np.float32), ref["scratch"], "accumulated gradient")
    assert_close(acc[2], ref["grad_x"], "grad_x")
    assert_close(acc[3], ref["grad_h0"], "grad_h0")
    # the general backward (no workspace) accumulates the same gradient in
    # another summation order
    gen = run(torch.from_numpy(base.copy()).cuda(), True, None, general=True)
    assert_close(gen[0], acc[0], "general backward's accumulate mode")
    # the binding sizes the workspace itself when none is given: the 16-row
    # kernel's bits, not the general backward's
    auto = run(torch.from_numpy(base.copy()).cuda(), True, None)
    for a, b, name in zip(auto, acc, ("scratch", "loss", "grad_x", "grad_h0")):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"binding's own workspace: {name}"


ONE_CALL = [
    # (B, K, cell, dt, seed, note)
    (21, 8, "gated", 1.0, 161, "parked path: two row groups of 16, a ragged one of 5"),
    (21, 8, "tau_decay", 0.3, 163, "parked path, tau-decay cell"),
    (1, 3, "gated", 0.6, 165, "parked path, one row"),
    (37, 5, "gated", 0.8, 167, "parked path, three row groups"),
    (6, 1, "tau_decay", 0.4, 171, "parked path, one step"),
    (21, 9, "gated", 1.0, 169, "K = 9: forward, then the recomputing backward"),
]


@pytest.mark.parametrize("case", ONE_CALL, ids=lambda c: "B{}_K{}_{}".format(*c[:3]))
def test_one_call_entry_with_workspace(case):
    """cfc_forward_backward_ws in accumulate mode at 256 x 256.  At K <= 8 the
    forward parks a_k in the workspace and the parked backward follows, so the
    result is the one-call overwrite path's gradient added to the old values
    in float32, bitwise, with the same h_seq, loss, grad_x and grad_h0; onto
    zeros it equals that path bitwise, and a workspace that is 8- but not
    16-byte aligned gives the same bits.  At K = 9 the call is cfc_forward then
    the workspace backward, bitwise.  Every case is checked against the oracle."""
    import torch
    import cfc_recurrent_cell_amd as C
    B, K, cell, dt, seed, note = case
    n = 256
    say(f"[wide accumulate] one-call entry with a workspace, B={B} K={K} {cell}: {note}")
    inp = W.make_random_cfc_inputs(B, K, n, n, dt, seed, cell=cell)
    d = to_dev(inp)
    args = (d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"])
    N = W.scratch_row_len(n, n)
    need = C.cfc_backward_workspace(B, K, n, n)
    ws_mem = torch.full(((need + 16) // 4,), float("nan"), device="cuda")   # contents on entry ignored
    base = W.make_random_matrix(B, N, seed=seed + 1)

    def run(start, ws):
        out = C.cfc_forward_backward(*args, d["y"], d["dt"], scratch=start, accumulate=True, cell=cell,
                                     workspace=ws, input_grads=True)
        return [host(t).copy() for t in out]

    acc = run(torch.from_numpy(base.copy()).cuda(), ws_mem.view(torch.uint8)[:need])
    names = ("h_seq", "scratch", "loss", "grad_x", "grad_h0")
    if K <= 8:
        over = [host(t).copy() for t in C.cfc_forward_backward(*args, d["y"], d["dt"], cell=cell,
                                                               input_grads=True)]
        want = base.astype(np.float32) + over[1]
        assert np.array_equal(acc[1].view(np.uint32), want.view(np.uint32)), "base + one-call gradient"
        for i in (0, 2, 3, 4):
            assert np.array_equal(acc[i].view(np.uint32), over[i].view(np.uint32)), names[i]
        zero = run(torch.zeros((B, N), device="cuda"), ws_mem.view(torch.uint8)[:need])
        for a, b_, name in zip(zero, over, names):
            assert np.array_equal(a.view(np.uint32), b_.view(np.uint32)), f"onto zeros: {name}"
        odd = run(torch.from_numpy(base.copy()).cuda(), ws_mem.view(torch.uint8)[8:8 + need])
        for a, b_, name in zip(odd, acc, names):
            assert np.array_equal(a.view(np.uint32), b_.view(np.uint32)), f"8-byte-aligned workspace: {name}"
        # room for the float64 weight copy: the widened weights give the same
        # bits; 8- but not 16-byte aligned, the copy is skipped
        full = C.cfc_forward_backward_workspace(B, K, n, n)
        assert full == need + (1 << 20)
        big = torch.full(((full + 16) // 4,), float("nan"), device="cuda").view(torch.uint8)
        for off, what in ((0, "float64 weight copy"), (8, "8-byte-aligned full-size workspace")):
            got = run(torch.from_numpy(base.copy()).cuda(), big[off:off + full])
            for a, b_, name in zip(got, acc, names):
                assert np.array_equal(a.view(np.uint32), b_.view(np.uint32)), f"{what}: {name}"
    else:
        h2 = C.cfc_forward(*args, d["dt"], cell=cell)
        s2, l2, gx2, gh2 = C.cfc_backward(*args, h2, d["y"], d["dt"],
                                          scratch=torch.from_numpy(base.copy()).cuda(), accumulate=True,
                                          cell=cell, workspace=ws_mem.view(torch.uint8)[:need], input_grads=True)
        for a, b_, name in zip(acc, (h2, s2, l2, gx2, gh2), names):
            assert np.array_equal(a.view(np.uint32), host(b_).view(np.uint32)), name
    ref = O.cfc_step(inp, threads=oracle_threads(), input_grads=True)
    assert_close(acc[1] - base.astype(np.float32), ref["scratch"], "accumulated one-call gradient")
    assert_close(acc[2], ref["loss"], "loss")
    assert_close(acc[3], ref["grad_x"], "grad_x")
    assert_close(acc[4], ref["grad_h0"], "grad_h0")
    # no workspace given: the binding allocates one, same bits
    auto = run(torch.from_numpy(base.copy()).cuda(), None)
    for a, b_, name in zip(auto, acc, names):
        assert np.array_equal(a.view(np.uint32), b_.view(np.uint32)), "binding's workspace: " + name


def test_workspace_reuse_over_calls_and_shapes():
    """One workspace serves consecutive calls of different sizes (a larger
    call, then a smaller one), each checked against a fresh overwrite."""
    import torch
    import cfc_recurrent_cell_amd as C
    say("[wide accumulate] one workspace, two calls of different sizes")
    big = C.cfc_backward_workspace(18, 9, 256, 256, accumulate=True)
    ws = torch.empty((big,), dtype=torch.uint8, device="cuda")
    for B, K, seed in ((18, 9, 141), (5, 4, 142)):
        inp = W.make_random_cfc_inputs(B, K, 256, 256, 0.9, seed)
        d = to_dev(inp)
        args = (d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"])
        h = C.cfc_forward(*args, d["dt"])
        N = W.scratch_row_len(256, 256)
        over, _ = C.cfc_backward(*args, h, d["y"], d["dt"], scratch=torch.empty((B, N), device="cuda"))
        base = W.make_random_matrix(B, N, seed=seed + 7)
        acc, _ = C.cfc_backward(*args, h, d["y"], d["dt"], scratch=torch.from_numpy(base.copy()).cuda(),
                                accumulate=True, workspace=ws)
        want = base.astype(np.float32) + host(over)
        assert np.array_equal(host(acc).view(np.uint32), want.view(np.uint32))


def test_too_small_workspace_is_refused_before_launch():
    import torch
    import cfc_recurrent_cell_amd as C
    say("[wide accumulate] refusal of a short workspace")
    B, K = 4, 3
    inp = W.make_random_cfc_inputs(B, K, 256, 256, 1.0, 151)
    d = to_dev(inp)
    args = (d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"])
    h = C.cfc_forward(*args, d["dt"])
    N = W.scratch_row_len(256, 256)
    base = W.make_random_matrix(B, N, seed=152)
    scratch = torch.from_numpy(base.copy()).cuda()
    need = C.cfc_backward_workspace(B, K, 256, 256, accumulate=True)
    ws = torch.empty((need - 8,), dtype=torch.uint8, device="cuda")
    with pytest.raises(C.CfcError):
        C.cfc_backward(*args, h, d["y"], d["dt"], scratch=scratch, accumulate=True, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(scratch).view(np.uint32), base.view(np.uint32))   # nothing was enqueued
