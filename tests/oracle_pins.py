"""Pins that tie the float64 oracle to facts other than itself.

Each pin takes an oracle library handle so the same checks can be run against
deliberately broken copies of the oracle (see test_oracle_mutants.py): a pin
set is only useful if a plausible mistake anywhere in the oracle fails it.

What pins what:
  * hand-solved examples (tests/golden/hand_examples.json): forward values,
    loss and every gradient slot in closed form, including the orientation of
    W_rec going forward and of W_rec^T going backward;
  * the zero-weight closed form: h_k = 2^-k h0 and the backward recurrences it
    implies, derived by hand;
  * dt = 0: gate exactly 1/2 and dw_tau exactly 0;
  * central finite differences of the oracle's own forward loss: pins the whole
    backward (every gradient slot, and the gradients with respect to x and
    h0) to the forward without sharing a formula;
  * float64 torch autograd of the forward: a second, independent gradient
    (parameters, x and h0);
  * batch-row independence, scratch clearing, permutation equivariance;
  * reduce_axis0 against exact integer sums and math.fsum.
"""
from __future__ import annotations

import json
import math
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from oracle import oracle as O
from cfc_recurrent_cell_amd.workloads import make_random_cfc_inputs, CfcInputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _ev(s: str) -> float:
    return float(eval(s, {"__builtins__": {}}, {"ln2": math.log(2.0), "e": math.e, "log": math.log}))


def _loss_from_hseq(h_seq, y) -> float:
    d = h_seq[:, -1, :] - y
    return float(0.5 * np.sum(d * d))


def _full_step(lib, w_in, w_rec, b, w_tau, x, h0, y, dt, cell="gated"):
    h_seq = O.cfc_forward(w_in, w_rec, b, w_tau, x, h0, dt, lib=lib, cell=cell)
    scratch, loss = O.cfc_backward(w_in, w_rec, b, w_tau, x, h0, h_seq, y, dt, lib=lib, cell=cell)
    out = O.reduce_axis0(scratch, lib=lib)
    return h_seq, scratch, loss, out


# ---------------------------------------------------------------- hand examples
def pin_hand_examples(lib) -> None:
    with open(GOLDEN) as f:
        data = json.load(f)
    for ex in data["examples"]:
        n_in, H, K = ex["n_in"], ex["n_hid"], ex["K"]
        arr = lambda key, shape: np.array([_ev(s) for s in ex[key]], dtype=np.float64).reshape(shape)
        w_in = arr("w_in", (H, n_in))
        w_rec = arr("w_rec", (H, H))
        b = arr("b", (H,))
        w_tau = arr("w_tau", (H,))
        x = arr("x", (1, K, n_in))
        h0 = arr("h0", (1, H))
        y = arr("y", (1, H))
        dt = _ev(ex["dt"])
        cell = ex.get("cell", "gated")
        h_seq, scratch, loss, out = _full_step(lib, w_in, w_rec, b, w_tau, x, h0, y, dt, cell)
        want_h = arr("h_seq", (1, K, H))
        want_s = arr("scratch", (1, H * (n_in + H + 2)))
        np.testing.assert_allclose(h_seq, want_h, rtol=1e-13, atol=1e-15, err_msg=ex["name"] + " h_seq")
        np.testing.assert_allclose(loss[0], _ev(ex["loss"]), rtol=1e-13, err_msg=ex["name"] + " loss")
        np.testing.assert_allclose(scratch, want_s, rtol=1e-12, atol=1e-15, err_msg=ex["name"] + " scratch")
        np.testing.assert_array_equal(out, scratch[0], err_msg=ex["name"] + " reduce at B=1 is a copy")
        _, _, gx, gh = O.cfc_backward_inputs(w_in, w_rec, b, w_tau, x, h0, h_seq, y, dt, lib=lib, cell=cell)
        np.testing.assert_allclose(gx, arr("grad_x", (1, K, n_in)), rtol=1e-12, atol=1e-15,
                                   err_msg=ex["name"] + " grad_x")
        np.testing.assert_allclose(gh, arr("grad_h0", (1, H)), rtol=1e-12, atol=1e-15,
                                   err_msg=ex["name"] + " grad_h0")


# ------------------------------------------------------- zero-weight closed form
def pin_zero_weights(lib, K=6, n_in=3, H=4, dt=0.8, seed=5) -> None:
    """W_in = W_rec = 0, b = 0: a = 0, g = 1/2, c = 0, so h_k = 2^-k h0 exactly.
    Backward by hand: with d_{k+1} = dL/dh_{k+1} = 2^-(K-1-k) (h_K - y),
      da_k = d_{k+1}/2 - sp dt d_{k+1} h_k / 4,  dw_tau = 0,  d_k = d_{k+1}/2."""
    rng = np.random.default_rng(seed)
    w_in = np.zeros((H, n_in))
    w_rec = np.zeros((H, H))
    b = np.zeros(H)
    w_tau = rng.standard_normal(H)
    x = rng.standard_normal((2, K, n_in))
    h0 = rng.standard_normal((2, H))
    y = rng.standard_normal((2, H))
    h_seq, scratch, loss, _ = _full_step(lib, w_in, w_rec, b, w_tau, x, h0, y, dt)
    for k in range(K):
        np.testing.assert_array_equal(h_seq[:, k, :], h0 * 2.0 ** -(k + 1))
    sp = np.log1p(np.exp(-np.abs(w_tau))) + np.maximum(w_tau, 0)   # softplus, by definition
    for r in range(2):
        hK = h0[r] * 2.0 ** -K
        gWin = np.zeros((H, n_in))
        gWrec = np.zeros((H, H))
        gb = np.zeros(H)
        for k in range(K):
            d = 2.0 ** -(K - 1 - k) * (hK - y[r])
            hk = h0[r] * 2.0 ** -k
            da = d / 2 - sp * dt * d * hk / 4
            gWin += np.outer(da, x[r, k])
            gWrec += np.outer(da, hk)
            gb += da
        want = np.concatenate([gWin.ravel(), gWrec.ravel(), gb, np.zeros(H)])
        np.testing.assert_allclose(scratch[r], want, rtol=1e-12, atol=1e-14)
        np.testing.assert_array_equal(scratch[r, -H:], np.zeros(H))
        np.testing.assert_allclose(loss[r], 0.5 * np.sum((hK - y[r]) ** 2), rtol=1e-14)
    # input gradients: W_in = 0 gives dL/dx = 0; d_k = d_k+1 / 2 gives dL/dh_0 = 2^-K (h_K - y)
    _, _, gx, gh = O.cfc_backward_inputs(w_in, w_rec, b, w_tau, x, h0, h_seq, y, dt, lib=lib)
    np.testing.assert_array_equal(gx, np.zeros_like(gx))
    np.testing.assert_array_equal(gh, 2.0 ** -K * (h_seq[:, -1] - y))


# ---------------------------------------------------------------------- dt = 0
def pin_dt_zero(lib, seed=6) -> None:
    """dt = 0: g = 1/2 exactly, so h_{k+1} - h_k/2 = tanh(a)/2 and dw_tau = 0."""
    inp = make_random_cfc_inputs(3, 5, 4, 6, 0.0, seed)
    h_seq, scratch, _, _ = _full_step(lib, inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x, inp.h0,
                                      inp.y, 0.0)
    H = inp.w_rec.shape[0]
    assert np.all(scratch[:, -H:] == 0.0)
    prev = inp.h0.astype(np.float64)
    for k in range(inp.x.shape[1]):
        a = inp.x[:, k].astype(np.float64) @ inp.w_in.T.astype(np.float64) + \
            prev @ inp.w_rec.T.astype(np.float64) + inp.b
        np.testing.assert_allclose(h_seq[:, k], 0.5 * prev + 0.5 * np.tanh(a), rtol=1e-13, atol=1e-15)
        prev = h_seq[:, k]


# ------------------------------------------------------ central finite differences
def pin_finite_differences(lib, inp: CfcInputs = None, eps=1e-6, rtol=2e-6, atol=1e-9,
                           max_params=None) -> float:
    """d(sum_b L_b)/d theta by central differences of the oracle's own forward, for
    every parameter, against the reduced gradient from its backward."""
    if inp is None:
        inp = make_random_cfc_inputs(2, 4, 3, 5, 0.7, seed=7)
    cell = inp.cell
    w = [np.array(a, dtype=np.float64) for a in (inp.w_in, inp.w_rec, inp.b, inp.w_tau)]
    x, h0, y, dt = inp.x, inp.h0, inp.y, float(inp.dt)
    _, _, _, out = _full_step(lib, *w, x, h0, y, dt, cell)

    def L(params):
        return _loss_from_hseq(O.cfc_forward(*params, x, h0, dt, lib=lib, cell=cell), y)

    fd = []
    for t in range(4):
        flat = w[t].ravel()
        for idx in range(flat.size):
            p = [a.copy() for a in w]
            p[t].ravel()[idx] = flat[idx] + eps
            lp = L(p)
            p[t].ravel()[idx] = flat[idx] - eps
            lm = L(p)
            fd.append((lp - lm) / (2 * eps))
    fd = np.array(fd)
    if max_params is not None:
        fd, out = fd[:max_params], out[:max_params]
    np.testing.assert_allclose(out, fd, rtol=rtol, atol=atol)
    return float(np.max(np.abs(out - fd)))


def pin_input_grad_finite_differences(lib, inp: CfcInputs = None, eps=1e-6, rtol=2e-6, atol=1e-9):
    """d(sum_b L_b)/dx and d(sum_b L_b)/dh0 by central differences of the
    oracle's own forward, against the backward's grad_x and grad_h0."""
    if inp is None:
        inp = make_random_cfc_inputs(2, 4, 3, 5, 0.7, seed=13)
    cell = inp.cell
    w = [np.array(a, dtype=np.float64) for a in (inp.w_in, inp.w_rec, inp.b, inp.w_tau)]
    x, h0, y, dt = np.array(inp.x, np.float64), np.array(inp.h0, np.float64), inp.y, float(inp.dt)
    h_seq = O.cfc_forward(*w, x, h0, dt, lib=lib, cell=cell)
    _, _, gx, gh = O.cfc_backward_inputs(*w, x, h0, h_seq, y, dt, lib=lib, cell=cell)

    def L(xv, hv):
        return _loss_from_hseq(O.cfc_forward(*w, xv, hv, dt, lib=lib, cell=cell), y)

    for arr, got, is_x in ((x, gx, True), (h0, gh, False)):
        fd = np.empty(arr.size)
        for idx in range(arr.size):
            p = arr.copy()
            p.ravel()[idx] += eps
            lp = L(p, h0) if is_x else L(x, p)
            p.ravel()[idx] -= 2 * eps
            lm = L(p, h0) if is_x else L(x, p)
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(got.ravel(), fd, rtol=rtol, atol=atol)


# ---------------------------------------------------------------- torch autograd
def pin_autograd(lib, inp: CfcInputs = None) -> None:
    """Independent float64 gradient: torch autograd of the forward definition."""
    import torch
    if inp is None:
        inp = make_random_cfc_inputs(3, 5, 4, 6, 0.7, seed=8)
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=False)
    w_in, w_rec, b, w_tau = (t(a).requires_grad_(True) for a in (inp.w_in, inp.w_rec, inp.b, inp.w_tau))
    x, h0, y = t(inp.x).requires_grad_(True), t(inp.h0).requires_grad_(True), t(inp.y)
    dt = float(inp.dt)
    cell = inp.cell
    h = h0
    hs = []
    for k in range(x.shape[1]):
        a = x[:, k] @ w_in.T + h @ w_rec.T + b
        if cell == "tau_decay":    # the pages' cell: a per-unit decay from tau, clamped at 1e-6
            g = torch.exp(-dt / torch.clamp(w_tau, min=1e-6))
        else:
            g = torch.sigmoid(-torch.nn.functional.softplus(w_tau) * a * dt)
        h = g * h + (1 - g) * torch.tanh(a)
        hs.append(h)
    loss = 0.5 * ((h - y) ** 2).sum()
    loss.backward()
    want = torch.cat([w_in.grad.ravel(), w_rec.grad.ravel(), b.grad, w_tau.grad]).numpy()
    h_seq, _, lossv, out = _full_step(lib, inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x, inp.h0,
                                      inp.y, dt, cell)
    np.testing.assert_allclose(h_seq, torch.stack(hs, 1).detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lossv.sum(), loss.item(), rtol=1e-12)
    np.testing.assert_allclose(out, want, rtol=1e-10, atol=1e-13)
    _, _, gx, gh = O.cfc_backward_inputs(inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x, inp.h0, h_seq,
                                         inp.y, dt, lib=lib, cell=cell)
    np.testing.assert_allclose(gx, x.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(gh, h0.grad.numpy(), rtol=1e-10, atol=1e-13)


# ------------------------------------------------------------- tau-decay cell
def pin_tau_zero_weights(lib, K=5, n_in=3, H=4, dt=0.3, seed=14) -> None:
    """Tau-decay cell with W_in = W_rec = 0, b = 0: a = 0, c = 0, so
    h_k+1 = d h_k with d = exp(-dt/tau) per unit; backward by hand:
    da_k = (1 - d) delta_k+1, dtau += delta_k+1 h_k d dt / tau^2,
    delta_k = d delta_k+1."""
    rng = np.random.default_rng(seed)
    w_in, w_rec, b = np.zeros((H, n_in)), np.zeros((H, H)), np.zeros(H)
    tau = rng.uniform(0.05, 2.0, H)
    x = rng.standard_normal((2, K, n_in))
    h0 = rng.standard_normal((2, H))
    y = rng.standard_normal((2, H))
    h_seq, scratch, loss, _ = _full_step(lib, w_in, w_rec, b, tau, x, h0, y, dt, "tau_decay")
    _, _, gx, gh = O.cfc_backward_inputs(w_in, w_rec, b, tau, x, h0, h_seq, y, dt, lib=lib, cell="tau_decay")
    d = np.exp(-dt / tau)
    for r in range(2):
        hs = [h0[r]]
        for k in range(K):
            hs.append(d * hs[-1])
        np.testing.assert_allclose(h_seq[r], np.array(hs[1:]), rtol=1e-14, atol=1e-300)
        delta = hs[-1] - y[r]
        gWin, gWrec, gb, gtau = np.zeros((H, n_in)), np.zeros((H, H)), np.zeros(H), np.zeros(H)
        for k in range(K - 1, -1, -1):
            da = (1 - d) * delta
            gWin += np.outer(da, x[r, k])
            gWrec += np.outer(da, hs[k])
            gb += da
            gtau += delta * hs[k] * d * dt / tau ** 2
            delta = d * delta
        want = np.concatenate([gWin.ravel(), gWrec.ravel(), gb, gtau])
        np.testing.assert_allclose(scratch[r], want, rtol=1e-12, atol=1e-14)
        np.testing.assert_array_equal(gx[r], np.zeros((K, n_in)))
        np.testing.assert_allclose(gh[r], delta, rtol=1e-13, atol=1e-300)


def pin_tau_guard(lib, seed=15) -> None:
    """Units with tau <= 1e-6 (the pages' guard): the decay is exp(-dt/1e-6),
    which is 0 in float64 for dt = 0.5, so h_k+1 = tanh(a) exactly, and their
    dL/dtau slot is exactly 0; the other units are unaffected."""
    inp = make_random_cfc_inputs(3, 4, 5, 6, 0.5, seed, cell="tau_decay")
    tau = inp.w_tau.astype(np.float64).copy()
    tau[[1, 4]] = [0.0, -0.3]
    h_seq, scratch, _, _ = _full_step(lib, inp.w_in, inp.w_rec, inp.b, tau, inp.x, inp.h0, inp.y, 0.5,
                                      "tau_decay")
    H = 6
    assert scratch[0, -H + 1] == 0.0 and scratch[0, -H + 4] == 0.0
    assert np.all(scratch[:, -H:][:, [0, 2, 3, 5]] != 0.0)
    prev = inp.h0.astype(np.float64)
    for k in range(4):
        a = inp.x[:, k].astype(np.float64) @ inp.w_in.T.astype(np.float64) + \
            prev @ inp.w_rec.T.astype(np.float64) + inp.b
        np.testing.assert_allclose(h_seq[:, k, [1, 4]], np.tanh(a[:, [1, 4]]), rtol=1e-14, atol=1e-16)
        prev = h_seq[:, k]


def pin_tau_finite_differences(lib) -> None:
    pin_finite_differences(lib, make_random_cfc_inputs(2, 4, 3, 5, 0.4, seed=16, cell="tau_decay"))
    pin_input_grad_finite_differences(lib, make_random_cfc_inputs(2, 4, 3, 5, 0.4, seed=17, cell="tau_decay"))


def pin_tau_autograd(lib) -> None:
    pin_autograd(lib, make_random_cfc_inputs(3, 5, 4, 6, 0.7, seed=18, cell="tau_decay"))


# ------------------------------------------------------------ structural pins
def pin_row_independence(lib, seed=9) -> None:
    """A row's scratch is bitwise the same computed alone (B=1) or in a batch."""
    inp = make_random_cfc_inputs(4, 5, 3, 5, 0.9, seed)
    h_seq, scratch, loss, _ = _full_step(lib, inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x, inp.h0,
                                         inp.y, float(inp.dt))
    for r in range(4):
        h1, s1, l1, o1 = _full_step(lib, inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x[r:r + 1],
                                    inp.h0[r:r + 1], inp.y[r:r + 1], float(inp.dt))
        np.testing.assert_array_equal(h1[0], h_seq[r])
        np.testing.assert_array_equal(s1[0], scratch[r])
        np.testing.assert_array_equal(o1, s1[0])   # reduce at B=1 is a copy
        assert l1[0] == loss[r]


def pin_scratch_clears(lib, seed=10) -> None:
    """Step A then step B on different data into a scratch poisoned with A's
    values or NaN: B's scratch must equal a fresh run on B's data."""
    a = make_random_cfc_inputs(3, 4, 3, 5, 0.6, seed)
    bb = make_random_cfc_inputs(3, 4, 3, 5, 0.6, seed + 1)
    fresh = _full_step(lib, bb.w_in, bb.w_rec, bb.b, bb.w_tau, bb.x, bb.h0, bb.y, 0.6)[1]
    hA = O.cfc_forward(a.w_in, a.w_rec, a.b, a.w_tau, a.x, a.h0, 0.6, lib=lib)
    sA, _ = O.cfc_backward(a.w_in, a.w_rec, a.b, a.w_tau, a.x, a.h0, hA, a.y, 0.6, lib=lib)
    hB = O.cfc_forward(bb.w_in, bb.w_rec, bb.b, bb.w_tau, bb.x, bb.h0, 0.6, lib=lib)
    for poison in (sA.copy(), np.full_like(sA, np.nan)):
        sB, _ = O.cfc_backward(bb.w_in, bb.w_rec, bb.b, bb.w_tau, bb.x, bb.h0, hB, bb.y, 0.6,
                               lib=lib, scratch=poison)
        np.testing.assert_array_equal(sB, fresh)
    assert not np.array_equal(fresh, sA)


def pin_permutation(lib, seed=12) -> None:
    inp = make_random_cfc_inputs(5, 4, 3, 4, 0.5, seed)
    perm = np.array([3, 0, 4, 1, 2])
    _, s, _, out = _full_step(lib, inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x, inp.h0, inp.y, 0.5)
    _, sp, _, outp = _full_step(lib, inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x[perm], inp.h0[perm],
                                inp.y[perm], 0.5)
    np.testing.assert_array_equal(sp, s[perm])
    np.testing.assert_allclose(outp, out, rtol=1e-13, atol=1e-16)


def pin_reduce_exact(lib) -> None:
    from cfc_recurrent_cell_amd.workloads import make_reduce_input, REDUCE
    a = make_reduce_input(REDUCE, integer=True)
    exact = a.astype(np.int64).sum(axis=0)                 # exact integer arithmetic
    out = O.reduce_axis0(a, lib=lib)
    np.testing.assert_array_equal(out, exact.astype(np.float64))
    out32 = O.reduce_axis0_f32(a, lib=lib)
    np.testing.assert_array_equal(out32, exact.astype(np.float64))
    # real-valued data: within a few ulps of the correctly rounded sum
    g = make_reduce_input(REDUCE, integer=False)[:, :512]
    o = O.reduce_axis0(g, lib=lib)
    fs = np.array([math.fsum(g[:, j].astype(np.float64)) for j in range(g.shape[1])])
    np.testing.assert_allclose(o, fs, rtol=0, atol=1e-13)
    # degenerate sizes: B = 0 writes zeros; N = 0 is a no-op
    np.testing.assert_array_equal(O.reduce_axis0(np.zeros((0, 7)), lib=lib), np.zeros(7))
    assert O.reduce_axis0(np.zeros((3, 0)), lib=lib).shape == (0,)


ALL_PINS = {
    "hand_examples": pin_hand_examples,
    "zero_weights": pin_zero_weights,
    "dt_zero": pin_dt_zero,
    "finite_differences": pin_finite_differences,
    "input_grad_finite_differences": pin_input_grad_finite_differences,
    "autograd": pin_autograd,
    "row_independence": pin_row_independence,
    "scratch_clears": pin_scratch_clears,
    "permutation": pin_permutation,
    "reduce_exact": pin_reduce_exact,
    "tau_zero_weights": pin_tau_zero_weights,
    "tau_guard": pin_tau_guard,
    "tau_finite_differences": pin_tau_finite_differences,
    "tau_autograd": pin_tau_autograd,
}
