"""The library's calls inside a HIP graph and on a side stream.

Every call only validates its arguments on the host and enqueues kernels on
the stream it is given (no allocation, no synchronisation, no host copy, no
memset), so a training step -- cfc_forward_backward then reduce_axis0 on
preallocated buffers -- can be captured once and replayed.  The pages make
capture safety an invariant of this path (the ml-alpha commit log's
graph-capture-safety commit: no host branches or allocations inside the
captured step).

The captured graph is replayed several times; before each replay new inputs
are copied into the captured input buffers and every output is poisoned with
NaN, with eager work and a device synchronisation between replays.  Each
replay must equal an eager run on the same inputs bitwise, and the eager runs
match the float64 oracle.  The same step enqueued on a side stream equals the
default-stream step bitwise.
"""
import numpy as np
import pytest

from parity_util import assert_close, host, oracle_threads, say, to_dev
from oracle import oracle as O
from cfc_recurrent_cell_amd import workloads as W

pytestmark = pytest.mark.gpu

SHAPES = [
    # (B, K, n_in, H, dt, seed, note)
    (256, 64, 128, 128, 0.5, 901, "one kernel per row (training-scale shape)"),
    (21, 6, 256, 256, 1.0, 902, "four launches: weight widening, forward parking a_k, two backward stages"),
    (5, 30, 140, 160, 0.7, 903, "two launches: 16-row forward, general backward"),
]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but torch sees no GPU")
    import cfc_recurrent_cell_amd as C
    C.load_library()
    return torch.device("cuda:0")


class Step:
    """Static input and output buffers of one training step."""

    def __init__(self, inp):
        import torch
        d = to_dev(inp)
        self.d = d
        B, K, n_in = inp.x.shape
        H = inp.w_rec.shape[0]
        N = W.scratch_row_len(n_in, H)
        self.h_seq = torch.empty((B, K, H), device="cuda")
        self.scratch = torch.empty((B, N), device="cuda")
        self.loss = torch.empty((B,), device="cuda")
        self.out = torch.empty((N,), device="cuda")

    def load(self, inp):
        """Copy a new input set into the static input buffers."""
        import torch
        for name in ("x", "h0", "y"):
            self.d[name].copy_(torch.from_numpy(np.ascontiguousarray(getattr(inp, name))))

    def poison(self):
        for t in (self.h_seq, self.scratch, self.loss, self.out):
            t.fill_(float("nan"))

    def __call__(self, stream=None):
        import cfc_recurrent_cell_amd as C
        d = self.d
        C.cfc_forward_backward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], d["y"], d["dt"],
                               h_seq=self.h_seq, scratch=self.scratch, loss=self.loss, stream=stream)
        C.reduce_axis0(self.scratch, out=self.out, stream=stream)

    def outputs(self):
        return [host(t).copy() for t in (self.h_seq, self.scratch, self.loss, self.out)]


def _same(a, b):
    return all(np.array_equal(x.view(np.uint32), y.view(np.uint32)) for x, y in zip(a, b))


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}_K{}_n{}_H{}".format(*s[:4]))
def test_captured_step_replays_match_eager(shape):
    import torch
    B, K, n_in, H, dt, seed, note = shape
    say(f"[capture] B={B} K={K} {n_in}/{H}: {note}")
    sets = [W.make_random_cfc_inputs(B, K, n_in, H, dt, seed + i) for i in range(2)]
    for s in sets[1:]:           # one parameter set; only x, h0 and y change
        s.w_in, s.w_rec, s.b, s.w_tau = sets[0].w_in, sets[0].w_rec, sets[0].b, sets[0].w_tau
    step = Step(sets[0])
    eager = []
    for inp in sets:
        step.load(inp)
        step.poison()
        step()
        eager.append(step.outputs())
    for inp, e in zip(sets, eager):
        ref = O.cfc_step(inp, threads=oracle_threads())
        for got, name in zip(e, ("h_seq", "scratch", "loss", "out")):
            assert_close(got, ref[name], f"eager {name}")
    # warm up on a side stream, as torch asks before a capture, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for replay, which in enumerate((1, 0, 1, 1, 0)):
        step.load(sets[which])
        step.poison()
        graph.replay()
        torch.cuda.synchronize()
        got = step.outputs()
        assert _same(got, eager[which]), f"replay {replay} (input set {which}) differs from the eager step"
        # unrelated eager work between replays
        torch.randn(1 << 20, device="cuda").sum().item()


def test_step_on_a_side_stream():
    """The binding enqueues on torch's current stream, or on the stream it is
    given: either way on a non-default stream the step equals the
    default-stream step bitwise."""
    import torch
    inp = W.make_random_cfc_inputs(64, 64, 128, 128, 0.5, 911)
    step = Step(inp)
    say("[stream] default stream vs side stream")
    step.poison()
    step()
    base = step.outputs()
    side = torch.cuda.Stream()
    for how in ("current", "explicit"):
        step.poison()
        torch.cuda.synchronize()
        side.wait_stream(torch.cuda.current_stream())
        if how == "current":
            with torch.cuda.stream(side):
                step()
        else:
            step(stream=side)
        torch.cuda.current_stream().wait_stream(side)
        got = step.outputs()
        assert _same(got, base), f"side stream ({how}) differs from the default stream"
