"""GPU parity at the cell's edge values, for every kernel family and both cells.

Saturation: biases of +-20 on a quarter of the units, +-400 on an eighth and
+-800 on two, both weight matrices scaled by 5 and dt = 2, so tanh and the gate
saturate and |2a| (the tanh argument) and |softplus(w_tau) a dt| (the gate
argument) pass 700, where the kernels select the saturated value instead of
evaluating the exponential.  Every output is compared with the float64 oracle
element by element at the usual tolerance, and the forward within one float32
ulp.  (The pages' invariant tests for a sigmoid head drive the bias to +-20 to
saturate it near 1 and near 0: the plans commit log, invariant-only tests.)

NaN: a NaN in one row's x (at one step) and in another row's h_0 must give NaN
wherever the definition does -- that row's h_seq from the step on, its whole
scratch row and loss, and every reduced column -- and leave the other rows, and
the rows that share a 16-row workgroup with them, equal to the oracle.

Families (each runs the kernels named):
  fused_row      cfc_forward_backward, n_in, H <= 128: cfc_fb_small_kernel
  fused_whole    the same at K = 64, 128 x 128 (its whole-shape instance)
  separate_row   cfc_forward + cfc_backward: cfc_fwd_small / cfc_bwd_small
  separate_16    cfc_forward + cfc_backward at 200 x 256: the 16-row kernels
  parked_16      cfc_forward_backward at 256 x 256: forward parking a_k, then
                 the two backward stages
  accumulate_16  cfc_forward_backward_ws accumulating onto zeros at 256 x 256:
                 the forward parking a_k in the workspace, then the two
                 backward stages (the second adding into the scratch)
  general        cfc_forward + cfc_backward at K = 24, 140 x 160: the general
                 one-row-per-workgroup backward
"""
import numpy as np
import pytest

from parity_util import assert_close, close_mask, host, oracle_threads, say, to_dev
from oracle import oracle as O
from cfc_recurrent_cell_amd import workloads as W

pytestmark = pytest.mark.gpu

FAMILIES = {
    # name: (B, K, n_in, H)
    "fused_row": (5, 12, 40, 56),
    "fused_whole": (3, 64, 128, 128),
    "separate_row": (5, 12, 40, 56),
    "separate_16": (21, 6, 200, 256),
    "parked_16": (21, 6, 256, 256),
    "accumulate_16": (19, 5, 256, 256),
    "general": (3, 24, 140, 160),
}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but torch sees no GPU")
    import cfc_recurrent_cell_amd as C
    C.load_library()
    return torch.device("cuda:0")


def saturating_inputs(B, K, n_in, H, cell, seed):
    """Random inputs, then saturating biases, weights x 5 and dt = 2."""
    inp = W.make_random_cfc_inputs(B, K, n_in, H, 2.0, seed, w_scale=5.0, cell=cell)
    rng = np.random.Generator(np.random.PCG64(seed + 500))
    units = rng.permutation(H)
    sign = np.where(rng.random(H) < 0.5, -1.0, 1.0)
    b = inp.b.astype(np.float64)
    q, e = max(1, H // 4), max(1, H // 8)
    b[units[:q]] = 20.0 * sign[units[:q]]
    b[units[q:q + e]] = 400.0 * sign[units[q:q + e]]
    b[units[q + e:q + e + 2]] = 800.0 * sign[units[q + e:q + e + 2]]
    inp.b = np.ascontiguousarray(b, dtype=np.float32)
    return inp


def run_family(family, inp):
    """The family's entry points on device copies of inp; returns host arrays
    (h_seq, scratch, loss, out)."""
    import torch
    import cfc_recurrent_cell_amd as C
    d = to_dev(inp)
    cell = inp.cell
    args = (d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"])
    B, K, n_in = inp.x.shape
    H = inp.w_rec.shape[0]
    N = W.scratch_row_len(n_in, H)
    scratch = torch.full((B, N), float("nan"), device="cuda")
    if family in ("fused_row", "fused_whole", "parked_16"):
        h, s, l = C.cfc_forward_backward(*args, d["y"], d["dt"], scratch=scratch, cell=cell)
    elif family == "accumulate_16":
        scratch.zero_()
        ws = torch.empty((C.cfc_backward_workspace(B, K, n_in, H),), dtype=torch.uint8, device="cuda")
        h, s, l = C.cfc_forward_backward(*args, d["y"], d["dt"], scratch=scratch, accumulate=True, cell=cell,
                                         workspace=ws)
    else:
        h = C.cfc_forward(*args, d["dt"], cell=cell)
        s, l = C.cfc_backward(*args, h, d["y"], d["dt"], scratch=scratch, cell=cell)
    o = C.reduce_axis0(s)
    return [host(t).copy() for t in (h, s, l, o)]


def _ulp_check(got_f32, want_f64, what):
    want = np.asarray(want_f64, dtype=np.float64)
    diff = np.abs(np.asarray(got_f32, dtype=np.float64) - want)
    ulp = np.spacing(np.abs(want.astype(np.float32))).astype(np.float64)
    bad = np.flatnonzero(diff.ravel() > ulp.ravel())
    assert bad.size == 0, f"{what}: {bad.size} h_seq elements more than 1 float32 ulp from the oracle"


@pytest.mark.parametrize("cell", ["gated", "tau_decay"])
@pytest.mark.parametrize("family", sorted(FAMILIES))
def test_saturating_inputs_match_oracle(family, cell):
    B, K, n_in, H = FAMILIES[family]
    inp = saturating_inputs(B, K, n_in, H, cell, seed=700 + sorted(FAMILIES).index(family))
    say(f"[saturation] {family} {cell}: B={B} K={K} n_in={n_in} H={H} dt=2, |b| up to 800, W x 5")
    h, s, l, o = run_family(family, inp)
    ref = O.cfc_step(inp, threads=oracle_threads())
    # the inputs do reach the saturated regime: some tanh values are exactly +-1
    assert np.any(np.abs(ref["h_seq"]) > 0.999999), "inputs failed to saturate the cell"
    assert_close(h, ref["h_seq"], f"{family} {cell} h_seq")
    _ulp_check(h, ref["h_seq"], f"{family} {cell}")
    assert_close(s, ref["scratch"], f"{family} {cell} scratch")
    assert_close(l, ref["loss"], f"{family} {cell} loss")
    assert_close(o, ref["out"], f"{family} {cell} out")


def _nan_consistent(got, want, what):
    """NaN exactly where the oracle has NaN; elsewhere within tolerance."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(want, dtype=np.float64)
    gn, rn = np.isnan(g), np.isnan(r)
    mism = np.flatnonzero((gn != rn).ravel())
    assert mism.size == 0, (f"{what}: NaN pattern differs from the oracle at {mism.size} elements "
                            f"(first {mism[:5]}: got {g.ravel()[mism[:5]]}, want {r.ravel()[mism[:5]]})")
    ok = close_mask(g[~rn], r[~rn])
    assert ok.all(), f"{what}: {int((~ok).sum())} finite elements outside the tolerance"


@pytest.mark.parametrize("cell", ["gated", "tau_decay"])
@pytest.mark.parametrize("family", sorted(FAMILIES))
def test_nan_propagates_like_the_definition(family, cell):
    B, K, n_in, H = FAMILIES[family]
    inp = W.make_random_cfc_inputs(B, K, n_in, H, 0.7, 800 + sorted(FAMILIES).index(family), cell=cell)
    x = inp.x.copy()
    h0 = inp.h0.copy()
    r_x, k_x = 1, K // 2
    r_h = B - 1
    x[r_x, k_x, 0] = np.nan
    h0[r_h, H // 2] = np.nan
    inp.x, inp.h0 = x, h0
    say(f"[nan] {family} {cell}: NaN in x[{r_x},{k_x},0] and h0[{r_h},{H // 2}]")
    h, s, l, o = run_family(family, inp)
    ref = O.cfc_step(inp, threads=oracle_threads())
    # the definition: row r_x is NaN from step k_x on, row r_h everywhere
    assert np.isnan(ref["h_seq"][r_x, k_x:]).all() and np.isfinite(ref["h_seq"][r_x, :k_x]).all()
    assert np.isnan(ref["scratch"][r_x]).all() and np.isnan(ref["scratch"][r_h]).all()
    clean = [r for r in range(B) if r not in (r_x, r_h)]
    assert np.isfinite(ref["scratch"][clean]).all()
    _nan_consistent(h, ref["h_seq"], f"{family} {cell} h_seq")
    _nan_consistent(s, ref["scratch"], f"{family} {cell} scratch")
    _nan_consistent(l, ref["loss"], f"{family} {cell} loss")
    _nan_consistent(o, ref["out"], f"{family} {cell} out")
