"""Lists whose elements all sit in one tensor.  Such a tensor travels with
each launch (no table is read) and every update kernel starts it its own
way: the first tile's loads go out with the scalar reads, the tag is
checked before the first store.  Each case here runs the three-call and
the clipped step, fp32 and 8-bit moments, against the oracle, bitwise: at
sizes around the chunk (2048 elements here) and grid boundaries, as views
that share a misalignment (peeled head) or do not (element path), among
empty tensors, and with the update's optional inputs present and absent
(the library then reads its workspace constants)."""
import numpy as np
import pytest
import torch

from gpu_harness import (NORM_REL_TOL, Step, compare_state, host_copy, oracle_norm, oracle_step,
                         say)
from test_gpu_parity import HP, make_cols
from test_gpu_q8 import Step8, check_norm, compare, make_host
from test_gpu_q8 import oracle_step as oracle_step8

pytestmark = pytest.mark.gpu
DEV = "cuda"

# 2048 elements per chunk for lists below 12,582,912 elements, 4096 from
# there; the fp32 update's grid is one block per chunk up to 1280 chunks,
# then at most 256 blocks (one per CU) walking several chunks each; the
# 8-bit update's grid is at most 1280 blocks, the norm's 256.
SIZES = [1, 5, 2047, 2048, 2049, 3 * 2048 + 17, 256 * 2048 + 1, 768 * 2048 + 33,
         1280 * 2048 - 3, 1280 * 2048 + 5, 2560 * 2048 + 2049, 12582912 + 4097]


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def fp32_case(cols, form, t=4, use_coef=True, skip=False, what=""):
    """One step of `form` on cols vs the oracle; the state must match bitwise."""
    host = host_copy(cols)
    st = Step(cols, completed_steps=t - 1)
    if form == "clipped":
        st.clipped(1.0, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"],
                   skip_if_nonfinite=skip)
    else:
        st.norm_clip(1.0).update(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"],
                                 use_coef=use_coef, skip_if_nonfinite=skip)
    S, c, step = st.results()
    assert step == t, what
    S_ref = oracle_norm(host["grad"])
    assert abs(S - S_ref) <= NORM_REL_TOL * S_ref, f"{what}: S {S} vs {S_ref}"
    oracle_step(host, c if use_coef else np.float32(1.0), t, HP["lr"], HP["beta1"], HP["beta2"],
                HP["eps"], HP["wd"])
    stats = compare_state(cols, host, what)
    assert stats["w"][0] == stats["m"][0] == stats["v"][0] == 0, what
    st.tl.release()


@pytest.mark.parametrize("form", ["three calls", "clipped"])
@pytest.mark.parametrize("grad_bf16,copy", [(False, False), (True, True)])
def test_one_tensor_sizes(form, grad_bf16, copy):
    for n in SIZES:
        what = f"{form} n={n} bf16={grad_bf16}"
        say(what)
        fp32_case(make_cols([n], grad_bf16, copy, seed=n % 997), form, what=what)


@pytest.mark.parametrize("form", ["three calls", "clipped"])
def test_one_tensor_among_empty_tensors(form):
    cols = make_cols([0, 0, 70001, 0], True, True, seed=5)
    fp32_case(cols, form, what=f"{form} among empty tensors")


@pytest.mark.parametrize("form", ["three calls", "clipped"])
@pytest.mark.parametrize("offsets", [(1, 1, 1), (2, 2, 2), (1, 2, 1), (0, 0, 3)],
                         ids=["shared 1", "shared 2", "mixed", "grad only"])
def test_one_tensor_misaligned_views(form, offsets):
    """Views into larger buffers: a misalignment every stream shares is
    peeled; otherwise the whole tensor takes the element path."""
    off_w, off_m, off_g = offsets
    gen = torch.Generator().manual_seed(sum(offsets))
    n = 3 * 2048 + 11
    w = (torch.randn(n + 8, generator=gen) * 0.02).to(DEV)[off_w:off_w + n]
    m = (torch.randn(n + 8, generator=gen) * 1e-4).to(DEV)[off_m:off_m + n]
    v = (torch.randn(n + 8, generator=gen) * 1e-8).abs().to(DEV)[off_w:off_w + n]
    g = (torch.randn(n + 8, generator=gen) * 1e-3).to(torch.bfloat16).to(DEV)[off_g:off_g + n]
    p = torch.zeros(n + 8, dtype=torch.bfloat16, device=DEV)[off_w:off_w + n]
    cols = {"master": [w], "exp_avg": [m], "exp_avg_sq": [v], "grad": [g], "param_bf16": [p]}
    fp32_case(cols, form, what=f"{form} offsets {offsets}")


@pytest.mark.parametrize("use_coef,skip", [(False, False), (False, True), (True, True)],
                         ids=["no coefficient", "no coefficient, skip pointer", "both"])
def test_one_tensor_optional_inputs(use_coef, skip):
    """The three-call update with its coefficient or skip pointer left out
    (the library passes its workspace constants 1 and 0 instead) or given."""
    for n in (7, 2049, 512 * 2048 + 5):
        fp32_case(make_cols([n], False, False, seed=n), "three calls", use_coef=use_coef,
                  skip=skip, what=f"n={n} coef={use_coef} skip={skip}")


def test_one_tensor_skip_if_nonfinite_writes_nothing():
    """A non-finite norm with skipping asked for leaves every buffer and the
    counter alone, in both forms (one tensor, several chunks)."""
    for form in ("three calls", "clipped"):
        cols = make_cols([3 * 2048 + 5], False, True, seed=9)
        cols["grad"][0][4100] = float("inf")
        before = [t.clone() for t in (cols["master"][0], cols["exp_avg"][0],
                                      cols["exp_avg_sq"][0], cols["param_bf16"][0])]
        st = Step(cols, completed_steps=6)
        if form == "clipped":
            st.clipped(1.0, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"],
                       skip_if_nonfinite=True)
        else:
            st.norm_clip(1.0).update(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"],
                                     skip_if_nonfinite=True)
        S, _, step = st.results()
        assert np.isinf(S) and step == 6, form
        after = (cols["master"][0], cols["exp_avg"][0], cols["exp_avg_sq"][0],
                 cols["param_bf16"][0])
        assert all(torch.equal(a, b) for a, b in zip(after, before)), form


# ----------------------------------------------------------- 8-bit moments ---

def q8_case(host, clipped, offset=0, what=""):
    s8 = Step8(host, offset=offset, completed_steps=2)
    S, c, t = s8.run(1.0, clipped=clipped)
    check_norm(S, host, what)
    assert t == 3, what
    oracle_step8(host, c, t)
    assert compare(s8, host, what) == 0, what
    s8.tl.release()


@pytest.mark.parametrize("clipped", [False, True], ids=["three calls", "clipped"])
@pytest.mark.parametrize("bf16", [False, True])
def test_q8_one_tensor_sizes(clipped, bf16):
    for n in (1, 31, 33, 2048, 2049, 3 * 2048 + 17, 768 * 2048 + 33, 1280 * 2048 + 33):
        what = f"q8 clipped={clipped} n={n} bf16={bf16}"
        say(what)
        q8_case(make_host([n], seed=n % 991, bf16=bf16), clipped, what=what)


@pytest.mark.parametrize("clipped", [False, True], ids=["three calls", "clipped"])
def test_q8_one_tensor_misaligned_and_among_empty(clipped):
    """A view one element into its buffers takes the element path; a tensor
    between empty ones keeps its first chunk at 0."""
    q8_case(make_host([3 * 2048 + 40], seed=71, bf16=True), clipped, offset=1,
            what=f"q8 clipped={clipped} misaligned")
    q8_case(make_host([0, 5000, 0], seed=72, bf16=False), clipped,
            what=f"q8 clipped={clipped} among empty")
