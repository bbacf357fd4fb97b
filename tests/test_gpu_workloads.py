"""GPU parity at the full sizes of the two largest workloads, in the launch
configuration bench.py times (adamw_clipped_step on the same list; one case
runs the three-call step instead).

The sum of squares is checked against the oracle over every gradient.  The
update is checked against the oracle on EVERY element of the 405B share
(792.7M parameters, 1137 tensors, cold and warm moments) and of the
8B-parameter list (8.03e9 parameters, 291 tensors): each tensor's inputs are
generated a second time from their seeds (the generator is deterministic on
the device), copied to the host, and stepped by the oracle with the GPU's
coefficient, one tensor at a time; so is the single tensor of 2^31 + 1003
elements (offsets past 32 bits), whose three-call step is also checked on
sampled positions (random ones, its first and last elements, chunk edges
and the elements around 2^31 and 2^30), and so are two lists just past the
whole-model threshold (2^30 elements) built from ragged, element-misaligned
views, one with fp32 and one with bf16 gradients (the fp32 one also
through the three-call step).
"""
import time

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import (NORM_REL_TOL, Step, check_bf16, check_bf16_bitwise_first, check_f32,
                         check_f32_bitwise_first, oracle_step_threads, sample_indices, say)
from mixed_precision_sharded_amd import synth
from mixed_precision_sharded_amd.configs import WORKLOADS, Workload, warm
from mixed_precision_sharded_amd.synth import to_numpy

pytestmark = pytest.mark.gpu

FIELDS = ("master", "exp_avg", "exp_avg_sq")


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def whole_tensor_parity(w, cols, i, c):
    """Every element of tensor i after the step against the oracle stepped
    from the tensor's regenerated inputs with the GPU's coefficient.  The
    oracle's results are copied to the device and compared bitwise there
    (torch.equal); a tensor that is not bitwise equal is brought to the host
    and checked element by element against the tolerances."""
    fresh = synth.tensor_inputs(w, i, "cuda")
    host = {k: to_numpy(fresh[k]).copy() for k in FIELDS + ("grad",)}
    del fresh
    pv = np.zeros(host["master"].size, np.uint16) if w.copy_bf16 else None
    oracle_step_threads(host["master"], host["exp_avg"], host["exp_avg_sq"], host["grad"], pv, c,
                        w.step, w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)
    nbit = 0
    for k in FIELDS:
        got = cols[k][i]
        if torch.equal(got.view(torch.int32), torch.from_numpy(host[k]).to(got.device).view(torch.int32)):
            continue
        nb, _ = check_f32_bitwise_first(to_numpy(got), host[k], f"{w.name} tensor {i} {k}")
        nbit += nb
    if w.copy_bf16:
        got = cols["param_bf16"][i]
        want = torch.from_numpy(pv.view(np.int16)).to(got.device)
        if not torch.equal(got.view(torch.int16), want):
            nb, _ = check_bf16_bitwise_first(to_numpy(got), pv, f"{w.name} tensor {i} param_bf16")
            nbit += nb
    return host["master"].size, nbit


def full_parity(w, clipped=True, cols=None):
    """Every element of every tensor of workload w against the oracle
    (`cols`: the workload's inputs already placed, else generated here)."""
    say(f"workload {w.name}: {w.numel:,} params in {w.n_tensors} tensors; generating")
    if cols is None:
        cols = synth.workload_inputs(w, "cuda")
    torch.cuda.synchronize()
    o = oracle.default()
    S_ref = o.grad_norm_sq(to_numpy(g) for g in cols["grad"])
    say(f"GPU step ({'clipped' if clipped else 'three calls'})")
    st = Step(cols, completed_steps=w.step - 1)
    if clipped:
        st.clipped(w.max_norm, w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)
    else:
        st.full(w)
    S, c, step = st.results()
    assert step == w.step
    assert abs(S - S_ref) <= NORM_REL_TOL * S_ref, (S, S_ref)
    assert c == o.clip_coef(S, w.max_norm)
    say(f"S={S:.9e} oracle {S_ref:.9e} rel {abs(S - S_ref) / S_ref:.2e} c={c}; "
        "every element against the oracle")
    n_checked = nbit = 0
    t0 = time.time()
    for i in range(w.n_tensors):
        n, nb = whole_tensor_parity(w, cols, i, c)
        n_checked += n
        nbit += nb
        if i % 25 == 24:
            say(f"  {i + 1} tensors, {n_checked:,} elements checked ({time.time() - t0:.0f} s)")
    assert n_checked == w.numel
    say(f"{n_checked:,} elements checked (master, m, v{', copy' if w.copy_bf16 else ''}); "
        f"{nbit} not bitwise equal")
    del st, cols


def sampled_parity(w, per_tensor, seed, extra=(), clipped=True):
    """`extra`: more element indices to check in every tensor (where they
    exist).  `clipped`: one adamw_clipped_step call, else grad_norm_sq with
    the clip output followed by adamw_multi_tensor_step."""
    say(f"workload {w.name}: {w.numel:,} params in {w.n_tensors} tensors; generating")
    cols = synth.workload_inputs(w, "cuda")
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(seed)
    idx = [sorted(set(sample_indices(n, per_tensor, gen)) | {e for e in extra if 0 <= e < n})
           for _, n in w.tensors]
    idx_dev = [torch.tensor(ix, dtype=torch.int64, device="cuda") for ix in idx]
    before = {k: [to_numpy(t[ix]) for t, ix in zip(cols[k], idx_dev)] for k in FIELDS + ("grad",)}

    say("oracle sum of squares over every gradient")
    o = oracle.default()
    S_ref = o.grad_norm_sq(to_numpy(g) for g in cols["grad"])  # one tensor on the host at a time

    say(f"GPU step ({'clipped' if clipped else 'three calls'})")
    st = Step(cols, completed_steps=w.step - 1)
    if clipped:
        st.clipped(w.max_norm, w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)
    else:
        st.full(w)
    S, c, step = st.results()
    assert step == w.step
    assert abs(S - S_ref) <= NORM_REL_TOL * S_ref, (S, S_ref)
    assert c == o.clip_coef(S, w.max_norm)
    say(f"S={S:.9e} oracle {S_ref:.9e} rel {abs(S - S_ref) / S_ref:.2e} c={c}")

    nbit = 0
    n_checked = 0
    for i in range(w.n_tensors):
        wv, mv, vv = (before[k][i].copy() for k in FIELDS)
        gv = before["grad"][i]
        pv = np.zeros(wv.size, np.uint16) if w.copy_bf16 else None
        o.adamw_step(wv, mv, vv, gv, pv, c, w.step, w.lr, w.beta1, w.beta2, w.eps,
                     w.weight_decay)
        for k, want in zip(FIELDS, (wv, mv, vv)):
            got = to_numpy(cols[k][i][idx_dev[i]])
            nb, _ = check_f32(got, want, f"{w.name} tensor {i} {k}")
            nbit += nb
        if w.copy_bf16:
            check_bf16(to_numpy(cols["param_bf16"][i][idx_dev[i]]), pv,
                       f"{w.name} tensor {i} param_bf16")
        n_checked += wv.size
        assert bool(torch.isfinite(cols["master"][i]).all()), i
    say(f"{n_checked:,} sampled elements checked; {nbit} not bitwise equal")
    del st, cols


def test_llama405b_share_every_element():
    full_parity(WORKLOADS[5])


def test_llama405b_share_warm_moments_every_element():
    full_parity(warm(WORKLOADS[5]), clipped=False)


def test_llama8b_full_list_every_element():
    """8,030,261,248 parameters (128.5 GB of state) on one GPU, in the launch
    configuration bench.py times (the whole-model walk: 1280 blocks,
    16384-element chunks): every element of every tensor against the
    oracle."""
    w = WORKLOADS[3]
    free, total = torch.cuda.mem_get_info()
    need = w.numel * w.state_bytes_per_param() + (16 << 30)
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB free, {free / 2**30:.0f} GiB available")
    full_parity(w)


# A list just past the whole-model threshold of 2^30 elements, with ragged
# sizes and element-misaligned views: the whole-model walk (1280 blocks,
# 16384-element chunks) through heads, tails, tiny tensors and the
# element-wise path, with fp32 and with bf16 gradients.
RAGGED_BIG = (((1 << 29) + 13, 1), (1, 0), (3, 3), (65, 2), (4097, 1), ((1 << 28) + 4001, 0),
              (2049, 3), ((1 << 28) + 1023, 2),
              (100003, {"master": 1, "exp_avg": 2, "exp_avg_sq": 0, "grad": 3, "param_bf16": 1}))


def placed_inputs(w, offsets):
    """The workload's seeded inputs, each stream of tensor i a view starting
    offsets[i] elements into a buffer of its own (one offset for every
    stream, or one per stream)."""
    cols = {k: [] for k in FIELDS + ("grad", "param_bf16")}
    for i, (_, n) in enumerate(w.tensors):
        fresh = synth.tensor_inputs(w, i, "cuda")
        for k in cols:
            src = fresh.get(k)
            if src is None:
                cols[k].append(None)
                continue
            off = offsets[i] if isinstance(offsets[i], int) else offsets[i][k]
            view = torch.empty(n + off, dtype=src.dtype, device="cuda")[off:off + n]
            view.copy_(src)
            cols[k].append(view)
        del fresh
    torch.cuda.synchronize()
    return cols


@pytest.mark.parametrize("grad_bf16,clipped", [(False, True), (True, True), (False, False)])
def test_whole_model_walk_ragged_misaligned_every_element(grad_bf16, clipped):
    w = Workload(cfg=92 + int(grad_bf16), name=f"ragged_past_2p30_{'bf16' if grad_bf16 else 'f32'}",
                 tensors=tuple((f"t{i}", n) for i, (n, _) in enumerate(RAGGED_BIG)),
                 grad_bf16=grad_bf16, copy_bf16=grad_bf16, step=7, m_std=1e-4, v_std=1e-8)
    assert w.numel >= 1 << 30
    free, _ = torch.cuda.mem_get_info()
    need = w.numel * (w.state_bytes_per_param() + 4) + (8 << 30)
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB free, {free / 2**30:.0f} GiB available")
    full_parity(w, clipped=clipped, cols=placed_inputs(w, [off for _, off in RAGGED_BIG]))


# A single tensor of more than 2^31 elements: element offsets, chunk indices
# and buffer pieces must not wrap at 32 bits.
HUGE = Workload(cfg=90, name="single_tensor_2g", tensors=(("huge", (1 << 31) + 1003),),
                grad_bf16=True, copy_bf16=True, step=5, m_std=1e-4, v_std=1e-8)
AROUND_2G = [(1 << 31) + d for d in range(-40, 41)] + [(1 << 30) + d for d in range(-8, 9)]


def test_single_tensor_over_2g_elements_every_element():
    """One tensor of 2^31 + 1003 elements (a whole-model walk: 1280 blocks,
    16384-element chunks, 131,073 of them): every element against the
    oracle, those past element 2^31 included."""
    free, _ = torch.cuda.mem_get_info()
    need = HUGE.numel * (HUGE.state_bytes_per_param() + 4) * 2 + (8 << 30)
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB free, {free / 2**30:.0f} GiB available")
    full_parity(HUGE)


def test_single_tensor_over_2g_elements_three_calls_sampled():
    """The same tensor through the three-call step, on sampled positions
    around element 2^31 and 2^30 and elsewhere."""
    free, _ = torch.cuda.mem_get_info()
    need = HUGE.numel * (HUGE.state_bytes_per_param() + 4) + (8 << 30)
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB free, {free / 2**30:.0f} GiB available")
    sampled_parity(HUGE, per_tensor=20000, seed=53, extra=AROUND_2G, clipped=False)
