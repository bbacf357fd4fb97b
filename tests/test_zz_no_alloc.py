"""GPU: adamw_clipped_step_noalloc (the clipped step on the library-held
workspace, for callers that cannot allocate) against adamw_clipped_step on
a workspace of the caller's, through the C ABI, on identical inputs: two
calls in a row on different lists, the second smaller, then the second list
again (its tables are still in the array), and the call recorded in a HIP
graph and replayed.  S, the coefficient, the counter and every element of
master, m, v and the bf16 copy must be bitwise equal (the same kernels,
grids and summation order), and the no-alloc results are also checked
against the oracle (relative error <= 2e-6, bf16 copy <= 1 ulp).  A list
whose tables exceed the array is refused before anything runs."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

from gpu_harness import NORM_REL_TOL, Step, compare_state, host_copy, oracle_norm, oracle_step, say
from mixed_precision_sharded_amd import binding
from test_gpu_parity import HP, make_cols

pytestmark = pytest.mark.gpu

FIELDS = ("master", "exp_avg", "exp_avg_sq", "grad", "param_bf16")


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def clone(cols):
    return {k: [None if t is None else t.clone() for t in v] for k, v in cols.items()}


def noalloc_against_workspace_step(cols, t, what):
    twin = clone(cols)
    host = host_copy(cols)
    hp = (HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"])

    ref = Step(cols, completed_steps=t - 1)
    ref.clipped(1.0, *hp)
    S_ref, c_ref, t_ref = ref.results()

    dev = twin["master"][0].device
    tl = binding.TensorList(*(twin[k] for k in FIELDS), workspace=False)
    sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
    coef = torch.zeros(1, dtype=torch.float32, device=dev)
    step = torch.tensor([t - 1], dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    allocated = torch.cuda.memory_allocated()
    binding.adamw_clipped_step_noalloc(tl, step, *hp, 1.0, sumsq_out=sumsq, coef_out=coef)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == allocated, "the call allocated through torch"
    S, c, t_got = float(sumsq.item()), np.float32(coef.item()), int(step.item())

    say(f"[no-alloc {what}] S={S:.9e} (workspace step {S_ref:.9e}) c={c} t={t_got}")
    assert np.float64(S).view(np.int64) == np.float64(S_ref).view(np.int64), (S, S_ref)
    assert c.view(np.int32) == c_ref.view(np.int32) and t_got == t_ref == t
    for k in ("master", "exp_avg", "exp_avg_sq", "param_bf16"):
        for i, (x, y) in enumerate(zip(twin[k], cols[k])):
            if x is None:
                continue
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (what, k, i)

    # The bar against the oracle as well (its own norm and, given the GPU's
    # coefficient, its update).
    S_o = oracle_norm(host["grad"])
    assert abs(S - S_o) <= NORM_REL_TOL * S_o
    oracle_step(host, c, t, *hp)
    stats = compare_state(twin, host, f"no-alloc {what}")
    assert stats["w"][0] == stats["m"][0] == stats["v"][0] == 0
    return twin


def test_noalloc_equals_the_workspace_step_on_consecutive_lists():
    big = make_cols([300001, 5, 77, 0, 4096, 1 << 20], True, True, seed=70)
    noalloc_against_workspace_step(big, t=3, what="first list, 1.35M params, bf16 + copy")
    small = make_cols([70001, 3], False, False, seed=71)
    after = noalloc_against_workspace_step(small, t=1, what="second list, smaller, fp32")
    # The same (smaller) list once more: its tables are already in the array.
    noalloc_against_workspace_step(after, t=2, what="second list again")


def test_noalloc_step_replays_from_a_graph():
    """The use the entry point is for: after one eager call on a list (which
    puts its tables in the library's array), the call recorded in a HIP graph
    and replayed three times, with unrelated eager work and synchronizations
    between the replays; after every replay S, the coefficient, the counter
    and every element equal the same step run eagerly on a workspace of the
    caller's, bitwise."""
    cols = make_cols([100003, 4097, 5], True, True, seed=72)
    twin = clone(cols)
    hp = (HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"])
    dev = cols["master"][0].device
    ref_tl = binding.TensorList(*(cols[k] for k in FIELDS))
    tl = binding.TensorList(*(twin[k] for k in FIELDS), workspace=False)
    scalars = [(torch.zeros(1, dtype=torch.float64, device=dev),
                torch.zeros(1, dtype=torch.float32, device=dev),
                torch.zeros(1, dtype=torch.int32, device=dev)) for _ in range(2)]
    (rs, rc, rt), (s, c, t) = scalars

    def reference_step():
        binding.adamw_clipped_step(ref_tl, rt, *hp, 1.0, sumsq_out=rs, coef_out=rc)

    def noalloc_step():
        binding.adamw_clipped_step_noalloc(tl, t, *hp, 1.0, sumsq_out=s, coef_out=c)

    def check(what):
        torch.cuda.synchronize()
        for x, y in ((s, rs), (c, rc), (t, rt)):
            assert torch.equal(x, y), (what, x.item(), y.item())
        for k in ("master", "exp_avg", "exp_avg_sq", "param_bf16"):
            for i, (x, y) in enumerate(zip(twin[k], cols[k])):
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (what, k, i)

    reference_step()
    noalloc_step()  # uploads the list's tables into the library's array
    check("eager call")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        noalloc_step()
    scratch = torch.randn(1 << 20, device=dev)
    for k in range(3):
        reference_step()
        g.replay()
        scratch.mul_(1.0001).add_(1.0)  # unrelated eager work between replays
        check(f"replay {k}")
    say(f"[no-alloc graph] four steps, S={s.item():.9e} c={c.item()} t={t.item()}, bitwise")
    assert int(t.item()) == 4
    ref_tl.release()


def test_noalloc_refuses_a_list_beyond_its_workspace():
    """270,000 one-element tensors need 64 bytes of table each: 17.3 MB, more
    than the 4 MiB array.  The records point into one real buffer (nothing
    would be touched anyway: the call is refused before anything is
    enqueued)."""
    n = 270000
    dev = torch.device("cuda")
    buf = torch.zeros(4 * n, device=dev)
    grads = torch.zeros(n, dtype=torch.bfloat16, device=dev)
    arr = (binding.MpsTensor * n)()
    w0, g0 = buf.data_ptr(), grads.data_ptr()
    for i in range(n):
        arr[i] = binding.MpsTensor(w0 + 4 * i, w0 + 4 * (n + i), w0 + 4 * (2 * n + i),
                                   g0 + 2 * i, None, 1)
    tl = SimpleNamespace(array=arr, n=n, grad_dtype=binding.MPS_DTYPE_BF16, device=buf.device)
    step = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(binding.MpsError) as err:
        binding.adamw_clipped_step_noalloc(tl, step, *(3e-4, 0.9, 0.95, 1e-8, 0.1), 1.0)
    assert err.value.code == -28 and "more than the library's" in str(err.value)
    torch.cuda.synchronize()
    assert int(step.item()) == 0
