"""Capture and concurrency: the step recorded in a HIP graph and replayed
several times (with unrelated eager work and synchronizations between the
replays) equals the same steps run eagerly, bitwise; two lists with their own
workspaces stepped on two streams at once equal the same steps run one after
the other.  For fp32 and 8-bit moments, and for both two-launch forms of the
step (three calls, and the one clipped-step call).

A list's tables are uploaded by its first call (a host-to-device copy), so a
caller records a graph after one eager call on the list; the norm alone
changes no state and serves for that."""
import numpy as np
import pytest
import torch

from gpu_harness import say
from mixed_precision_sharded_amd import binding

pytestmark = pytest.mark.gpu
HP = (3e-4, 0.9, 0.95, 1e-8, 0.1)


def inputs(sizes, seed, q8=False):
    gen = torch.Generator().manual_seed(seed)
    d = {"w": [], "m": [], "v": [], "g": [], "p": [], "st": []}
    for n in sizes:
        d["w"].append((torch.randn(n, generator=gen) * 0.02).cuda())
        d["m"].append((torch.randn(n, generator=gen) * 1e-4).cuda())
        d["v"].append((torch.randn(n, generator=gen) * 1e-8).abs().cuda())
        d["g"].append((torch.randn(n, generator=gen) * 1e-2).to(torch.bfloat16).cuda())
        d["p"].append(torch.zeros(n, dtype=torch.bfloat16, device="cuda"))
        if q8:
            st = binding.zeros_q8_state(n, "cuda")
            binding.adamw8_quantize(d["m"][-1], binding.MPS_Q8_E4M3, st[0], st[1])
            binding.adamw8_quantize(d["v"][-1], binding.MPS_Q8_E5M2, st[2], st[3])
            d["st"].append(st)
    torch.cuda.synchronize()
    return d


def clone(d):
    return {k: [tuple(x.clone() for x in t) if isinstance(t, tuple) else t.clone() for t in v]
            for k, v in d.items()}


class Runner:
    def __init__(self, d, q8, clipped=False):
        self.q8 = q8
        self.clipped = clipped
        self.d = d
        if q8:
            self.tl = binding.TensorList8(d["w"], d["st"], d["g"], d["p"])
        else:
            self.tl = binding.TensorList(d["w"], d["m"], d["v"], d["g"], d["p"])
        self.sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
        self.coef = torch.zeros(1, dtype=torch.float32, device="cuda")
        self.step = torch.tensor([7], dtype=torch.int32, device="cuda")

    def norm(self, stream=None):
        f = binding.adamw8_grad_norm_sq if self.q8 else binding.grad_norm_sq
        f(self.tl, self.sumsq, 1.0, self.coef, stream=stream)

    def update(self, stream=None):
        f = binding.adamw8_multi_tensor_step if self.q8 else binding.adamw_multi_tensor_step
        f(self.tl, self.coef, self.step, *HP, stream=stream)

    def full_step(self, stream=None):
        if self.clipped:
            f = binding.adamw8_clipped_step if self.q8 else binding.adamw_clipped_step
            f(self.tl, self.step, *HP, 1.0, sumsq_out=self.sumsq, coef_out=self.coef,
              stream=stream)
        else:
            self.norm(stream)
            self.update(stream)

    def state(self):
        torch.cuda.synchronize()
        out = [self.sumsq.clone(), self.coef.clone(), self.step.clone()]
        out += [t.clone() for t in self.d["w"] + self.d["p"]]
        if self.q8:
            out += [x.clone() for st in self.d["st"] for x in st]
        else:
            out += [t.clone() for t in self.d["m"] + self.d["v"]]
        return out


def same(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        xb = x.view(torch.uint8) if x.dtype != torch.uint8 else x
        yb = y.view(torch.uint8) if y.dtype != torch.uint8 else y
        assert torch.equal(xb, yb), f"{what}: buffer {i} differs"


FORMS = [False, True]
FORM_IDS = ["three_calls", "clipped"]


@pytest.mark.parametrize("clipped", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("q8", [False, True], ids=["fp32_moments", "8bit_moments"])
def test_graph_replays_equal_eager_steps(q8, clipped):
    say(f"graph capture, 8-bit={q8}, clipped={clipped}")
    sizes = [5, 4096 + 3, 100000]
    base = inputs(sizes, 61, q8)
    eager, graphed = Runner(clone(base), q8, clipped), Runner(clone(base), q8, clipped)
    graphed.norm()                      # uploads the tables; changes no state
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.full_step()
    scratch = torch.randn(1 << 20, device="cuda")
    for k in range(3):
        eager.full_step()
        g.replay()
        scratch.mul_(1.0001).add_(1.0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        same(eager.state(), graphed.state(), f"replay {k}")
    assert int(graphed.step.item()) == 10
    eager.tl.release()
    graphed.tl.release()


@pytest.mark.parametrize("clipped", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("q8", [False, True], ids=["fp32_moments", "8bit_moments"])
def test_two_lists_on_two_streams(q8, clipped):
    say(f"two streams, 8-bit={q8}, clipped={clipped}")
    a0, b0 = inputs([70000, 33], 62, q8), inputs([123457], 63, q8)
    seq_a, seq_b = Runner(clone(a0), q8, clipped), Runner(clone(b0), q8, clipped)
    for _ in range(3):
        seq_a.full_step()
        seq_b.full_step()
    con_a, con_b = Runner(clone(a0), q8, clipped), Runner(clone(b0), q8, clipped)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        if clipped:
            con_a.full_step(s1); con_b.full_step(s2)
        else:
            con_a.norm(s1); con_b.norm(s2)
            con_a.update(s1); con_b.update(s2)
    torch.cuda.synchronize()
    same(seq_a.state(), con_a.state(), "list a")
    same(seq_b.state(), con_b.state(), "list b")
    for r in (seq_a, seq_b, con_a, con_b):
        r.tl.release()


def test_host_threads_with_their_own_workspaces():
    """Three host threads, each with its own list, workspace and stream,
    stepping at once (the binding's calls release the interpreter lock):
    every list ends bitwise where a sequential run ends."""
    import threading
    say("three host threads")
    bases = [inputs([50000 + 17 * k, 4096], 70 + k) for k in range(3)]
    seq = [Runner(clone(b), False) for b in bases]
    for r in seq:
        for _ in range(4):
            r.norm(); r.update()
    con = [Runner(clone(b), False) for b in bases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in con]
    errors = []

    def work(r, st):
        try:
            with torch.cuda.stream(st):
                for _ in range(4):
                    r.norm(st); r.update(st)
            st.synchronize()
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(r, st)) for r, st in zip(con, streams)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    torch.cuda.synchronize()
    for k, (a, b) in enumerate(zip(seq, con)):
        same(a.state(), b.state(), f"thread {k}")
    for r in seq + con:
        r.tl.release()
