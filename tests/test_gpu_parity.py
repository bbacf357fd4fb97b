"""GPU parity: the HIP path through the C ABI against the CPU oracle, element
by element, on seeded inputs (small and ragged cases, and the workloads).

Tolerances: sum of squares <= 1e-5 relative; master, m, v <= 2e-6 relative
per element (exact where the oracle gives 0) with the oracle fed the GPU's
own clip coefficient; bf16 copy <= 1 ulp.  Bitwise agreement is expected
and its count is printed.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_harness import (NORM_REL_TOL, Step, check_bf16, check_f32, compare_state, host_copy,
                         oracle_norm, oracle_step, say)
from mixed_precision_sharded_amd import binding, synth
from mixed_precision_sharded_amd.configs import WORKLOADS, Workload

pytestmark = pytest.mark.gpu

DEV = "cuda"
HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1)


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def make_cols(sizes, grad_bf16, copy, seed, warm=True, grad_std=1e-3, device=DEV):
    gen = torch.Generator(device="cpu").manual_seed(seed)
    cols = {"master": [], "exp_avg": [], "exp_avg_sq": [], "grad": [], "param_bf16": []}
    for n in sizes:
        cols["master"].append((torch.randn(n, generator=gen) * 0.02).to(device))
        if warm:
            cols["exp_avg"].append((torch.randn(n, generator=gen) * 1e-4).to(device))
            cols["exp_avg_sq"].append((torch.randn(n, generator=gen) * 1e-8).abs().to(device))
        else:
            cols["exp_avg"].append(torch.zeros(n, device=device))
            cols["exp_avg_sq"].append(torch.zeros(n, device=device))
        g = (torch.randn(n, generator=gen) * grad_std).to(device)
        cols["grad"].append(g.to(torch.bfloat16) if grad_bf16 else g)
        cols["param_bf16"].append(torch.zeros(n, dtype=torch.bfloat16, device=device)
                                  if copy else None)
    return cols


def run_and_check(cols, t, max_norm=1.0, what="", hp=HP, use_coef=True, fused=True):
    """One GPU step vs the oracle; returns (S_gpu, c_gpu, stats).  `fused`:
    the clip coefficient comes from the norm's launch (else from clip_coef)."""
    host = host_copy(cols)
    st = Step(cols, completed_steps=t - 1)
    st = st.norm_clip(max_norm) if fused else st.norm().clip(max_norm)
    st.update(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["wd"], use_coef=use_coef)
    S, c, step = st.results()
    assert step == t, f"{what}: step counter {step}, expected {t}"
    S_ref = oracle_norm(host["grad"])
    if np.isfinite(S_ref):
        assert abs(S - S_ref) <= NORM_REL_TOL * abs(S_ref), f"{what}: norm {S} vs {S_ref}"
    else:
        assert (np.isnan(S) and np.isnan(S_ref)) or S == S_ref, f"{what}: norm {S} vs {S_ref}"
    c_ref = oracle.default().clip_coef(S, max_norm)
    assert c == c_ref or (np.isnan(c) and np.isnan(c_ref)), f"{what}: coef {c} vs {c_ref}"
    oracle_step(host, c if use_coef else np.float32(1.0), t, hp["lr"], hp["beta1"], hp["beta2"],
                hp["eps"], hp["wd"])
    stats = compare_state(cols, host, what)
    rel = abs(S - S_ref) / max(S_ref, 1e-300) if np.isfinite(S_ref) else 0.0
    say(f"[{what}] S={S:.6e} (oracle {S_ref:.6e}, rel {rel:.1e}) "
        f"c={c} non-bitwise w/m/v/p = {stats['w'][0]}/{stats['m'][0]}/{stats['v'][0]}/"
        f"{stats['p'][0]}")
    return S, c, stats


# ------------------------------------------------------- small and ragged ---

RAGGED = [0, 1, 3, 4, 5, 7, 8, 9, 63, 64, 65, 2047, 2048, 2049, 4097, 100003]


@pytest.mark.parametrize("grad_bf16,copy,fused", [(False, False, True), (True, True, True),
                                                  (False, True, False), (True, False, False)])
def test_ragged_list(grad_bf16, copy, fused):
    say(f"ragged list grad_bf16={grad_bf16} copy={copy} fused clip={fused}")
    cols = make_cols(RAGGED, grad_bf16, copy, seed=1)
    _, _, stats = run_and_check(cols, t=3, what=f"ragged bf16={grad_bf16} copy={copy}",
                                fused=fused)
    assert stats["w"][0] == stats["m"][0] == stats["v"][0] == 0, "expected bitwise agreement"


def test_large_tensor_many_chunks_ragged_tail():
    say("one tensor of 3,000,003 elements, bf16 grads with copy, clipping active")
    cols = make_cols([3_000_003], True, True, seed=2, grad_std=1e-2)
    S, c, stats = run_and_check(cols, t=7, what="3M+3")
    assert c < 1.0
    assert stats["w"][0] == 0


def _views(base_numel, offsets, dtype, gen):
    out = []
    for off in offsets:
        buf = torch.randn(base_numel + 8, generator=gen).to(dtype)
        out.append(buf.to(DEV)[off:off + base_numel])
    return out


@pytest.mark.parametrize("grad_bf16", [False, True])
def test_misaligned_views(grad_bf16):
    """Views starting at every element offset mod 8, with the streams either
    sharing an alignment (peeled head) or not (element-wise path)."""
    say(f"misaligned views grad_bf16={grad_bf16}")
    gen = torch.Generator().manual_seed(3)
    n = 9001
    cols = {"master": [], "exp_avg": [], "exp_avg_sq": [], "grad": [], "param_bf16": []}
    for off_w, off_m, off_g in [(0, 0, 0), (1, 1, 1), (2, 2, 2), (3, 3, 3), (5, 5, 5),
                                (1, 2, 1), (0, 3, 0), (0, 0, 1), (7, 7, 3)]:
        w = (torch.randn(n + 8, generator=gen) * 0.02).to(DEV)[off_w:off_w + n]
        m = (torch.randn(n + 8, generator=gen) * 1e-4).to(DEV)[off_m:off_m + n]
        v = (torch.randn(n + 8, generator=gen) * 1e-8).abs().to(DEV)[off_w:off_w + n]
        g = (torch.randn(n + 8, generator=gen) * 1e-3)
        g = (g.to(torch.bfloat16) if grad_bf16 else g).to(DEV)[off_g:off_g + n]
        p = torch.zeros(n + 8, dtype=torch.bfloat16, device=DEV)[off_w:off_w + n]
        for k, t in zip(cols, (w, m, v, g, p)):
            cols[k].append(t)
    _, _, stats = run_and_check(cols, t=2, what=f"misaligned bf16={grad_bf16}")
    assert stats["w"][0] == 0


def test_many_small_tensors():
    say("600 tensors of 0..3000 elements")
    rng = np.random.default_rng(4)
    sizes = rng.integers(0, 3000, 600).tolist()
    cols = make_cols(sizes, True, True, seed=4)
    run_and_check(cols, t=11, what="600 small")


def test_all_empty_list():
    say("list of empty tensors")
    cols = make_cols([0, 0, 0], False, False, seed=5)
    st = Step(cols, completed_steps=41).norm().clip(1.0).update(**_hp())
    S, c, step = st.results()
    assert S == 0.0 and c == 1.0 and step == 42


def _hp():
    return dict(lr=HP["lr"], beta1=HP["beta1"], beta2=HP["beta2"], eps=HP["eps"], wd=HP["wd"])


@pytest.mark.parametrize("blocks", [1, 2, 7, 8, 9, 15, 17, 100])
def test_ticket_tree_at_every_group_shape(blocks):
    """One tensor of `blocks` chunks of 2048 elements: both the norm and the
    three-call update run `blocks` blocks, so their ticket trees have groups
    of equal and unequal sizes, or fewer groups than eight.  Four steps in a
    row: the norm's last block must finish S every time and the counter must
    advance by exactly one per update."""
    n = blocks * 2048
    cols = make_cols([n], True, True, seed=400 + blocks)
    host = host_copy(cols)
    st = Step(cols, completed_steps=10)
    o = oracle.default()
    S_ref = o.grad_norm_sq(host["grad"])
    for t in range(11, 15):
        st.norm_clip(1.0).update(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"])
        S, c, step = st.results()
        assert step == t, (blocks, t, step)
        assert abs(S - S_ref) <= NORM_REL_TOL * S_ref, (blocks, S, S_ref)
        oracle_step(host, c, t, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"])
    stats = compare_state(cols, host, f"{blocks} blocks")
    assert stats["w"][0] == stats["m"][0] == stats["v"][0] == 0


def test_no_coef_means_no_clipping():
    cols = make_cols([5000, 77], False, True, seed=6, grad_std=1.0)
    run_and_check(cols, t=1, what="no coef", use_coef=False)


@pytest.mark.parametrize("t", [1, 2, 10, 1000, 123456])
def test_step_counter_and_bias_corrections(t):
    cols = make_cols([4099], True, True, seed=7)
    _, _, stats = run_and_check(cols, t=t, what=f"t={t}")
    assert stats["w"][0] == 0 and stats["v"][0] == 0


@pytest.mark.parametrize("hp", [dict(lr=0.0, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1),
                                dict(lr=1e-2, beta1=0.0, beta2=0.0, eps=1e-6, wd=0.0),
                                dict(lr=1e-3, beta1=0.5, beta2=0.999, eps=0.0, wd=1.0)])
def test_hyperparameter_corners(hp):
    cols = make_cols([3001, 5], False, True, seed=8)
    run_and_check(cols, t=5, what=f"hp {hp}", hp=hp)


# ------------------------------------------------------------------ clip ---

def test_clip_bitwise_given_the_same_sum():
    o = oracle.default()
    vals = [0.0, 1e-300, 1e-12, 0.25, 1.0, 1.049, 4.0, 2.0 ** 40, 1e300, float("inf"),
            float("nan")] + list(np.random.default_rng(9).lognormal(0, 10, 200))
    for max_norm in (1.0, 0.5, 3.0, 1e-3):
        S = torch.tensor(vals, dtype=torch.float64, device=DEV)
        c = torch.empty(len(vals), dtype=torch.float32, device=DEV)
        for i in range(len(vals)):
            binding.clip_coef(S[i:i + 1], max_norm, c[i:i + 1])
        got = c.cpu().numpy()
        want = np.array([o.clip_coef(s, max_norm) for s in vals], np.float32)
        same = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
        assert same.all(), (max_norm, np.array(vals)[~same], got[~same], want[~same])


def test_fused_clip_equals_standalone_clip():
    """The coefficient written by the norm's launch equals clip_coef's."""
    for seed, std, max_norm in ((20, 1e-3, 1.0), (21, 1.0, 0.5), (22, 1e-6, 1.0), (23, 1e2, 3.0)):
        cols = make_cols([100003, 17, 4096], seed % 2 == 0, False, seed=seed, grad_std=std)
        st = Step(cols).norm_clip(max_norm)
        S1, c1, _ = st.results()
        st.clip(max_norm)
        S2, c2, _ = st.results()
        assert S1 == S2 and c1 == c2 == oracle.default().clip_coef(S1, max_norm), (seed, c1, c2)


@pytest.mark.parametrize("grad_scale", [1.0, 0.25, 1.0 / 3, 2.0 ** -16, 1.0 / 7])
def test_scaled_clip_and_step(grad_scale):
    """Gradient scale folded into the coefficient (fused and standalone),
    then the step, against the oracle."""
    say(f"grad_scale {grad_scale}")
    o = oracle.default()
    cols = make_cols([100003, 4097, 5], True, True, seed=40, grad_std=5e-2 / grad_scale)
    host = host_copy(cols)
    st = Step(cols, completed_steps=6).norm_clip(1.0, grad_scale)
    S, c_fused, _ = st.results()
    st.clip(1.0, grad_scale)
    _, c_alone, _ = st.results()
    assert c_fused == c_alone == o.clip_coef(S, 1.0, grad_scale), (c_fused, c_alone)
    st.update(**_hp())
    _, _, step = st.results()
    assert step == 7
    oracle_step(host, c_fused, 7, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"])
    stats = compare_state(cols, host, f"scale {grad_scale}")
    assert stats["w"][0] == stats["m"][0] == stats["v"][0] == 0


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_skip_if_nonfinite_leaves_everything(bad):
    """A non-finite sum of squares skips the whole step: state, copy and the
    counter stay bitwise as they were."""
    cols = make_cols([70001, 33], True, True, seed=41)
    cols["grad"][0][123] = bad
    before = {k: [t.clone() for t in v] for k, v in cols.items()}
    st = Step(cols, completed_steps=9).norm_clip(1.0).update(**_hp(), skip_if_nonfinite=True)
    S, _, step = st.results()
    assert not np.isfinite(S) and step == 9
    for k in ("master", "exp_avg", "exp_avg_sq", "param_bf16"):
        for x, y in zip(cols[k], before[k]):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), k


def test_skip_pointer_with_finite_gradients_steps_normally():
    a = make_cols([50000, 7], False, True, seed=42)
    b = make_cols([50000, 7], False, True, seed=42)
    sa = Step(a, completed_steps=3).norm_clip(1.0).update(**_hp(), skip_if_nonfinite=True)
    sb = Step(b, completed_steps=3).norm_clip(1.0).update(**_hp())
    assert sa.results()[2] == sb.results()[2] == 4
    for k in ("master", "exp_avg", "exp_avg_sq"):
        for x, y in zip(a[k], b[k]):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), k


# ---------------------------------------------------- determinism, resume ---

def test_repeatable_bitwise():
    outs = []
    for _ in range(2):
        cols = make_cols([1_000_003, 4096, 17], True, True, seed=10)
        st = Step(cols, completed_steps=4).norm().clip(1.0).update(**_hp())
        S, c, _ = st.results()
        outs.append((S, c, [t.cpu() for k in ("master", "exp_avg", "exp_avg_sq", "param_bf16")
                            for t in cols[k]]))
    assert outs[0][0] == outs[1][0] and outs[0][1] == outs[1][1]
    for a, b in zip(outs[0][2], outs[1][2]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_resume_equals_straight_run():
    """Two steps in a row = one step, a host save/restore of the state and the
    counter, then one more step (bitwise)."""
    sizes = [70001, 129]
    a = make_cols(sizes, False, True, seed=11)
    b = make_cols(sizes, False, True, seed=11)
    sa = Step(a, completed_steps=9)
    for _ in range(2):
        sa.norm().clip(1.0).update(**_hp())
    sb = Step(b, completed_steps=9)
    sb.norm().clip(1.0).update(**_hp())
    torch.cuda.synchronize()
    saved = {k: [None if t is None else t.cpu().clone() for t in v] for k, v in b.items()}
    saved_step = sb.step.cpu().clone()
    for k in ("master", "exp_avg", "exp_avg_sq"):
        for t in b[k]:
            t.zero_()
    for k in ("master", "exp_avg", "exp_avg_sq"):
        for t, s in zip(b[k], saved[k]):
            t.copy_(s)
    sb.step.copy_(saved_step)
    sb.norm().clip(1.0).update(**_hp())
    torch.cuda.synchronize()
    assert sa.step.item() == sb.step.item() == 11
    for k in ("master", "exp_avg", "exp_avg_sq"):
        for x, y in zip(a[k], b[k]):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), k


def test_list_equals_flat():
    """The same data as one flat tensor or as a list: bitwise identical state
    and copy given the same coefficient."""
    sizes = [12345, 1, 99999, 4096]
    lst = make_cols(sizes, True, True, seed=12)
    flat = {k: [torch.cat(v)] for k, v in lst.items()}  # concatenation copies
    coef = torch.tensor([0.8125], dtype=torch.float32, device=DEV)
    for cols in (lst, flat):
        st = Step(cols, completed_steps=2)
        st.coef.copy_(coef)
        st.update(**_hp())
    torch.cuda.synchronize()
    for k in ("master", "exp_avg", "exp_avg_sq"):
        assert torch.equal(torch.cat(lst[k]).view(torch.int32), flat[k][0].view(torch.int32))
    assert torch.equal(torch.cat(lst["param_bf16"]).view(torch.int16),
                       flat["param_bf16"][0].view(torch.int16))


def test_nonfinite_gradients():
    cols = make_cols([1000, 50], False, False, seed=13)
    cols["grad"][0][17] = float("nan")
    st = Step(cols, completed_steps=0).norm().clip(1.0).update(**_hp())
    S, c, step = st.results()
    assert np.isnan(S) and np.isnan(c) and step == 1
    assert torch.isnan(cols["master"][0]).all() and torch.isnan(cols["master"][1]).all()
    cols = make_cols([1000], True, True, seed=14)
    cols["grad"][0][3] = float("inf")
    run_and_check(cols, t=1, what="inf grad")


@pytest.mark.parametrize("form", ["three calls", "clipped"])
@pytest.mark.parametrize("sizes", [[5000], [5000, 300]], ids=["one tensor", "two tensors"])
@pytest.mark.parametrize("overwrite", ["header", "everything"])
def test_overwritten_workspace_is_detected(form, sizes, overwrite):
    """If the workspace tables are overwritten behind the library's back the
    kernels leave every buffer alone (the norm reports NaN).  A one-tensor
    list takes its tensor from the launch and checks the tag after its first
    reads, a longer list before; both are covered in both two-launch forms.
    The header alone is zeroed, or every byte of the workspace set to 0xFF:
    then the chunk map holds 0xFFFFFFFF, which the prologues (reading a table
    entry before the tag has been compared) clamp into the tensor table."""
    cols = make_cols(sizes, False, False, seed=15)
    before = [t.clone() for t in cols["master"] + cols["exp_avg"] + cols["exp_avg_sq"]]
    st = Step(cols, completed_steps=0)
    st.norm().results()  # uploads the tables
    ws = st.tl._ws_storage
    off = st.tl.workspace_ptr - ws.data_ptr()
    if overwrite == "header":
        ws[off:off + 64].zero_()
    else:
        ws[off:off + st.tl.workspace_bytes].fill_(0xFF)
    if form == "clipped":
        st.clipped(1.0, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"])
    else:
        st.norm().clip(1.0).update(**_hp())
    S, c, step = st.results()
    assert np.isnan(S) and np.isnan(c) and step == 0
    after = cols["master"] + cols["exp_avg"] + cols["exp_avg_sq"]
    assert all(torch.equal(a, b) for a, b in zip(after, before))


def test_one_workspace_shared_by_two_lists():
    """Two lists step in turn on one workspace, in both two-launch forms: each
    call finds the other list's tables there, so the library's cached plan
    must not be reused; every step matches the oracle bitwise."""
    a = make_cols([300000, 5, 77], True, True, seed=90)
    b = make_cols([70001], False, True, seed=91)
    ha, hb = host_copy(a), host_copy(b)
    sa, sb = Step(a, completed_steps=0), Step(b, completed_steps=5)
    assert sa.tl.workspace_bytes >= sb.tl.workspace_bytes
    sb.tl.release()
    sb.tl._ws_storage = sa.tl._ws_storage
    sb.tl.workspace_ptr, sb.tl.workspace_bytes = sa.tl.workspace_ptr, sa.tl.workspace_bytes
    hp = (HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["wd"])
    for k in range(4):
        for st, h in ((sa, ha), (sb, hb)):
            t_next = int(st.step.item()) + 1
            if k % 2:
                st.clipped(1.0, *hp)
            else:
                st.norm_clip(1.0).update(*hp)
            S, c, t = st.results()
            assert t == t_next, (k, t, t_next)
            S_ref = oracle_norm(h["grad"])
            assert abs(S - S_ref) <= NORM_REL_TOL * S_ref, (k, S, S_ref)
            oracle_step(h, c, t, *hp)
    for cols, h, what in ((a, ha, "list a"), (b, hb, "list b")):
        stats = compare_state(cols, h, what)
        assert stats["w"][0] == stats["m"][0] == stats["v"][0] == 0, what


def test_norm_only_list_then_step_still_checks_state_pointers():
    """A list without state pointers is valid for the norm; the same tensor
    array passed to a step on the same workspace must still be refused,
    although the library has a plan for it."""
    L = binding.lib()
    g = torch.randn(4096, device=DEV) * 1e-2
    arr = (binding.MpsTensor * 1)()
    arr[0] = binding.MpsTensor(None, None, None, g.data_ptr(), None, 4096)
    nbytes = L.adamw_workspace_bytes(arr, 1)
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=DEV)
    ws = (buf.data_ptr() + 255) // 256 * 256
    S = torch.zeros(1, dtype=torch.float64, device=DEV)
    step = torch.zeros(1, dtype=torch.int32, device=DEV)
    assert L.grad_norm_sq(arr, 1, binding.MPS_DTYPE_F32, S.data_ptr(), 1.0, 1.0, None, ws,
                          nbytes, None) == 0
    torch.cuda.synchronize()
    assert abs(S.item() - float((g.double() ** 2).sum())) <= 1e-12 * S.item()
    assert L.adamw_multi_tensor_step(arr, 1, binding.MPS_DTYPE_F32, None, None, step.data_ptr(),
                                     3e-4, 0.9, 0.95, 1e-8, 0.1, ws, nbytes, None) == -22
    assert "NULL" in binding.last_error()
    assert L.adamw_clipped_step(arr, 1, binding.MPS_DTYPE_F32, 1.0, 1.0, 0, None, None,
                                step.data_ptr(), 3e-4, 0.9, 0.95, 1e-8, 0.1, ws, nbytes, None,
                                None) == -22
    assert L.grad_norm_sq(arr, 1, binding.MPS_DTYPE_F32, S.data_ptr(), 1.0, 1.0, None, ws,
                          nbytes, None) == 0
    torch.cuda.synchronize()
    assert int(step.item()) == 0
    L.adamw_workspace_release(ws)


# ------------------------------------------------------------- workloads ---

def _workload_cols(w):
    cols = synth.workload_inputs(w, DEV)
    return cols


@pytest.mark.parametrize("cfg", [1, 2])
def test_workload_full_parity(cfg):
    w = WORKLOADS[cfg]
    say(f"workload {cfg} {w.name}: full element-wise parity")
    cols = _workload_cols(w)
    S, c, stats = run_and_check(cols, t=w.step, max_norm=w.max_norm, what=w.name,
                                hp=dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                                        wd=w.weight_decay))
    if cfg == 2:
        assert c < 0.1, "the outliers force clipping"
    del cols


def test_workload_70b_share_full_parity():
    w = WORKLOADS[4]
    say(f"workload 4 {w.name}: full element-wise parity over {w.n_tensors} tensors")
    cols = _workload_cols(w)
    run_and_check(cols, t=w.step, max_norm=w.max_norm, what=w.name,
                  hp=dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, wd=w.weight_decay))
    del cols


def test_bf16_copy_rounds_to_nearest_even():
    """lr = 0 and zero moments and gradients keep every master as it is, so
    the copy is exactly the bf16 rounding of the crafted masters: ties, one
    unit off a tie, subnormals, overflow to infinity, zeros, infinities, NaN;
    aligned (vector path) and one element off (scalar peel)."""
    from gpu_harness import crafted_bf16_masters
    from mixed_precision_sharded_amd.synth import to_numpy
    w = crafted_bf16_masters(np.random.default_rng(31))
    n = w.size
    buf = torch.zeros(n + 1, dtype=torch.float32, device=DEV)
    buf[1:] = torch.from_numpy(w).to(DEV)
    masters = [torch.from_numpy(w).to(DEV), buf[1:]]
    cols = {"master": masters,
            "exp_avg": [torch.zeros(n, device=DEV) for _ in range(2)],
            "exp_avg_sq": [torch.zeros(n, device=DEV) for _ in range(2)],
            "grad": [torch.zeros(n, dtype=torch.bfloat16, device=DEV) for _ in range(2)],
            "param_bf16": [torch.zeros(n, dtype=torch.bfloat16, device=DEV) for _ in range(2)]}
    st = Step(cols).norm_clip(1.0).update(0.0, HP["beta1"], HP["beta2"], HP["eps"], HP["wd"])
    S, c, _ = st.results()
    assert S == 0.0 and c == np.float32(1.0)
    want = oracle.default().f32_to_bf16(w)
    nan = np.isnan(w)
    for i in range(2):
        got = to_numpy(cols["param_bf16"][i])
        assert ((got & 0x7FFF) > 0x7F80)[nan].all(), f"tensor {i}: NaN copies"
        bad = np.nonzero(got[~nan] != want[~nan])[0]
        assert bad.size == 0, (f"tensor {i}: {bad.size} copies differ, e.g. "
                               f"{w[~nan][bad[0]].view(np.uint32):#010x} -> {got[~nan][bad[0]]:#06x}"
                               f" vs {want[~nan][bad[0]]:#06x}")
        kept = to_numpy(cols["master"][i])
        assert np.array_equal(kept[~nan].view(np.uint32), w[~nan].view(np.uint32))
    say(f"bf16 copy: {n} crafted values, every non-NaN copy bitwise equal to the oracle's")
