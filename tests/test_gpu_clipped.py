"""GPU parity of the two-launch whole step (adamw_clipped_step): the norm's
blocks leave partial sums, and every block of the update finishes S from
them before it updates.  Checked against the oracle on the cases of the
three-call path, and bitwise against that path itself (same norm blocks and
summation order, so the same S, coefficient and state)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_harness import NORM_REL_TOL, Step, compare_state, host_copy, oracle_norm, oracle_step, say
from mixed_precision_sharded_amd import synth
from mixed_precision_sharded_amd.configs import WORKLOADS
from test_gpu_parity import HP, RAGGED, make_cols

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def clipped_and_check(cols, t, hp=HP, max_norm=1.0, grad_scale=1.0, what=""):
    host = host_copy(cols)
    st = Step(cols, completed_steps=t - 1)
    st.clipped(max_norm, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["wd"],
               grad_scale=grad_scale)
    S, c, step = st.results()
    assert step == t, what
    S_ref = oracle_norm(host["grad"])
    assert abs(S - S_ref) <= NORM_REL_TOL * abs(S_ref), (what, S, S_ref)
    assert c == oracle.default().clip_coef(S, max_norm, grad_scale), what
    oracle_step(host, c, t, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["wd"])
    stats = compare_state(cols, host, what)
    say(f"[clipped {what}] S rel {abs(S - S_ref) / max(S_ref, 1e-300):.1e} c={c} "
        f"non-bitwise w/m/v/p = {stats['w'][0]}/{stats['m'][0]}/{stats['v'][0]}/{stats['p'][0]}")
    return stats


@pytest.mark.parametrize("grad_bf16,copy", [(False, False), (True, True), (False, True)])
def test_clipped_ragged(grad_bf16, copy):
    cols = make_cols(RAGGED, grad_bf16, copy, seed=70)
    stats = clipped_and_check(cols, t=3, what=f"ragged bf16={grad_bf16} copy={copy}")
    assert stats["w"][0] == stats["m"][0] == stats["v"][0] == 0


def test_clipped_many_tensors_and_scale():
    rng = np.random.default_rng(71)
    cols = make_cols(rng.integers(0, 5000, 400).tolist(), True, True, seed=71, grad_std=1e-1)
    clipped_and_check(cols, t=12, grad_scale=0.125, what="400 tensors, scale 1/8")


def test_clipped_one_tensor_among_empty_ones():
    """A list whose chunks all belong to its second tensor (the one-tensor
    lookup with a non-zero index), and a misaligned view."""
    cols = make_cols([0, 123457, 0], False, True, seed=72)
    stats = clipped_and_check(cols, t=2, what="[0, 123457, 0]")
    assert stats["w"][0] == 0
    base = make_cols([70001], True, True, seed=73)
    cols = {k: [None if t is None else t[3:] for t in v] for k, v in base.items()}
    stats = clipped_and_check(cols, t=5, what="view at element 3")
    assert stats["w"][0] == 0


def test_clipped_list_without_elements():
    cols = make_cols([0, 0], True, True, seed=74)
    st = Step(cols, completed_steps=6)
    st.clipped(1.0, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"])
    S, c, step = st.results()
    assert S == 0.0 and c == 1.0 and step == 7


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_clipped_workloads(cfg):
    w = WORKLOADS[cfg]
    say(f"clipped, workload {w.name}")
    cols = synth.workload_inputs(w, "cuda")
    clipped_and_check(cols, t=w.step, max_norm=w.max_norm, what=w.name,
                      hp=dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                              wd=w.weight_decay))


def test_clipped_consecutive_launches_match_the_oracle():
    cols = make_cols([300001, 77], False, True, seed=75)
    host = host_copy(cols)
    st = Step(cols, completed_steps=0)
    o = oracle.default()
    for t in range(1, 6):
        st.clipped(1.0, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"])
        S, c, step = st.results()
        assert step == t
        assert c == o.clip_coef(S, 1.0)
        oracle_step(host, c, t, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"])
    stats = compare_state(cols, host, "5 clipped steps")
    assert stats["w"][0] == 0


def test_clipped_interleaved_with_the_three_call_step_and_a_counter_reset():
    """The step number travels from the norm launch to the update launch in
    the workspace: calls of the other path in between, and a counter set by
    the host, must not disturb it."""
    cols = make_cols([200003, 5], True, True, seed=78)
    host = host_copy(cols)
    st = Step(cols, completed_steps=0)
    o = oracle.default()
    hp = (HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"])
    for kind, expect_t in (("clipped", 1), ("three-call", 2), ("reset", 40), ("clipped", 41),
                           ("clipped", 42)):
        if kind == "reset":
            st.step.fill_(expect_t - 1)
            kind = "three-call"
        if kind == "clipped":
            st.clipped(1.0, *hp)
        else:
            st.norm_clip(1.0).update(*hp)
        S, c, step = st.results()
        assert step == expect_t, kind
        assert c == o.clip_coef(S, 1.0)
        oracle_step(host, c, expect_t, *hp)
    stats = compare_state(cols, host, "interleaved")
    assert stats["w"][0] == stats["m"][0] == stats["v"][0] == 0


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_clipped_skip_if_nonfinite(bad):
    cols = make_cols([40000, 9], True, True, seed=76)
    cols["grad"][1][4] = bad
    before = {k: [t.clone() for t in v] for k, v in cols.items()}
    st = Step(cols, completed_steps=4)
    st.clipped(1.0, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"],
               skip_if_nonfinite=True)
    S, c, step = st.results()
    assert not np.isfinite(S) and step == 4
    assert c == oracle.default().clip_coef(S, 1.0) or (np.isnan(c) and np.isnan(S))
    for k in ("master", "exp_avg", "exp_avg_sq", "param_bf16"):
        for x, y in zip(cols[k], before[k]):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), k


@pytest.mark.parametrize("sizes,grad_bf16", [([250000, 3], False), (RAGGED, True),
                                             ([1 << 20], True)])
def test_clipped_is_bitwise_the_three_call_step(sizes, grad_bf16):
    """The same S, coefficient, counter and state as grad_norm_sq with the
    clip output followed by adamw_multi_tensor_step, on a two-step run (the
    second step also compares the skip path's reads of S)."""
    a = make_cols(sizes, grad_bf16, True, seed=77)
    b = make_cols(sizes, grad_bf16, True, seed=77)
    sa = Step(a, completed_steps=1)
    sb = Step(b, completed_steps=1)
    for _ in range(2):
        sa.clipped(1.0, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"], grad_scale=0.5,
                   skip_if_nonfinite=True)
        sb.norm_clip(1.0, grad_scale=0.5).update(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"],
                                                 HP["wd"], skip_if_nonfinite=True)
        Sa, ca, ta = sa.results()
        Sb, cb, tb = sb.results()
        assert np.float64(Sa).tobytes() == np.float64(Sb).tobytes()
        assert np.float32(ca).tobytes() == np.float32(cb).tobytes() and ta == tb
    for k in ("master", "exp_avg", "exp_avg_sq", "param_bf16"):
        for x, y in zip(a[k], b[k]):
            if x is not None:
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), k


def big_cols(sizes, seed):
    """fp32 state and bf16 gradients drawn on the GPU (lists of a billion
    elements and more; only GPU results are compared with each other)."""
    gen = torch.Generator(device="cuda").manual_seed(seed)
    cols = {"master": [], "exp_avg": [], "exp_avg_sq": [], "grad": [], "param_bf16": []}
    for n in sizes:
        cols["master"].append(torch.randn(n, device="cuda", generator=gen).mul_(0.02))
        cols["exp_avg"].append(torch.randn(n, device="cuda", generator=gen).mul_(1e-4))
        cols["exp_avg_sq"].append(torch.randn(n, device="cuda", generator=gen).abs_().mul_(1e-8))
        cols["grad"].append(torch.randn(n, device="cuda", generator=gen).mul_(1e-3)
                            .to(torch.bfloat16))
        cols["param_bf16"].append(torch.zeros(n, dtype=torch.bfloat16, device="cuda"))
    return cols


def test_long_walks_are_bitwise_the_three_call_step():
    """A list of 41.9M parameters in 4096-element chunks (10,244 chunks,
    ragged ends, bf16 gradients): each of the 256 update blocks walks 40
    chunks in turn with tiles of two groups of four per thread.  The clipped
    step and the three-call step must give the same bits for every element,
    on two steps in a row (each is checked against the oracle elsewhere;
    here the long walks of both forms are compared in full)."""
    sizes = [10240 * 4096 - 5000, 7, 40000]
    say("generating two copies of a 41.9M-parameter list")
    a = big_cols(sizes, seed=91)
    b = {k: [t.clone() for t in v] for k, v in a.items()}
    sa = Step(a, completed_steps=41)
    sb = Step(b, completed_steps=41)
    for i in range(2):
        say(f"step {i + 1}")
        sa.clipped(1.0, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"])
        sb.norm_clip(1.0).update(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"])
        Sa, ca, ta = sa.results()
        Sb, cb, tb = sb.results()
        assert np.float64(Sa).tobytes() == np.float64(Sb).tobytes()
        assert np.float32(ca).tobytes() == np.float32(cb).tobytes() and ta == tb == 42 + i
    for k in ("master", "exp_avg", "exp_avg_sq", "param_bf16"):
        for x, y in zip(a[k], b[k]):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), k
    del sa, sb, a, b
