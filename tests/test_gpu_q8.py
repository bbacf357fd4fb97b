"""GPU parity of the step with 8-bit moments (m: E4M3 codes, v: E5M2 codes,
one scale byte per run of 32) against the oracle, through the C ABI.

The bar is the oracle's own arithmetic: the master and its bf16 copy are
fp32 / bf16 results (relative error <= 2e-6, copy within 1 ulp; expected
bitwise), the codes and scale bytes are integers decided in fp32 on both
sides and must match exactly.  The oracle's update is fed the device's clip
coefficient; the sum of squares is checked on its own (relative 1e-5).
"""
import time

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import NORM_REL_TOL, check_bf16, check_f32, say
from mixed_precision_sharded_amd import binding

pytestmark = pytest.mark.gpu

E4M3, E5M2 = oracle.E4M3, oracle.E5M2
HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1)


def make_host(sizes, seed, bf16, copy_every=1, warm=True, grad_std=1e-3):
    """Seeded host arrays per tensor: fp32 master, the 8-bit state of a warm
    (or zero) m and v, the gradient (fp32 or bf16 words), the copy buffer."""
    o = oracle.default()
    rng = np.random.default_rng(seed)
    host = []
    for i, n in enumerate(sizes):
        w = (rng.standard_normal(n) * 0.02).astype(np.float32)
        g = (rng.standard_normal(n) * grad_std).astype(np.float32)
        if warm:
            m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
            v = np.abs(rng.standard_normal(n) * 1e-8).astype(np.float32)
        else:
            m = np.zeros(n, np.float32)
            v = np.zeros(n, np.float32)
        mc, ms = o.quantize(m, E4M3)
        vc, vs = o.quantize(v, E5M2)
        host.append(dict(w=w, mc=mc, ms=ms, vc=vc, vs=vs,
                         g=o.f32_to_bf16(g) if bf16 else g,
                         p=np.zeros(n, np.uint16) if copy_every and i % copy_every == 0 else None))
    return host


def to_device(a, offset=0):
    """Device copy of a host array; with offset > 0 a view that starts
    `offset` elements into a larger buffer."""
    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 \
        else torch.from_numpy(a)
    if offset == 0:
        return t.cuda()
    buf = torch.zeros(a.size + offset, dtype=t.dtype, device="cuda")
    buf[offset:] = t.cuda()
    return buf[offset:]


def to_host(t):
    t = t.detach().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


class Step8:
    def __init__(self, host, offset=0, completed_steps=0):
        self.dev = [{k: (None if a is None else to_device(a, offset)) for k, a in h.items()}
                    for h in host]
        self.tl = binding.TensorList8([d["w"] for d in self.dev],
                                      [(d["mc"], d["ms"], d["vc"], d["vs"]) for d in self.dev],
                                      [d["g"] for d in self.dev], [d["p"] for d in self.dev])
        self.sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
        self.coef = torch.zeros(1, dtype=torch.float32, device="cuda")
        self.step = torch.tensor([completed_steps], dtype=torch.int32, device="cuda")

    def run(self, max_norm, hp=HP, skip_if_nonfinite=False, clipped=False):
        """Three calls (norm with the clip output, update), or one
        adamw8_clipped_step."""
        if clipped:
            binding.adamw8_clipped_step(self.tl, self.step, hp["lr"], hp["beta1"], hp["beta2"],
                                        hp["eps"], hp["wd"], max_norm,
                                        skip_if_nonfinite=skip_if_nonfinite,
                                        sumsq_out=self.sumsq, coef_out=self.coef)
        else:
            binding.adamw8_grad_norm_sq(self.tl, self.sumsq, max_norm, self.coef)
            binding.adamw8_multi_tensor_step(
                self.tl, self.coef, self.step, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                hp["wd"], skip_if_nonfinite=self.sumsq if skip_if_nonfinite else None)
        torch.cuda.synchronize()
        return float(self.sumsq.item()), np.float32(self.coef.item()), int(self.step.item())


def oracle_step(host, c, t, hp=HP):
    o = oracle.default()
    for h in host:
        o.adamw8_step(h["w"], h["mc"], h["ms"], h["vc"], h["vs"], h["g"], h["p"], c, t,
                      hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["wd"])


def check_norm(S_gpu, host, what):
    S = oracle.default().grad_norm_sq([h["g"] for h in host])
    if np.isfinite(S):
        assert abs(S_gpu - S) <= NORM_REL_TOL * abs(S), f"{what}: S {S_gpu} vs {S}"
    else:
        assert np.isnan(S_gpu) == np.isnan(S) and np.isinf(S_gpu) == np.isinf(S), what
    return S


def compare(step8, host, what):
    nbit = 0
    for i, (d, h) in enumerate(zip(step8.dev, host)):
        nb, _ = check_f32(to_host(d["w"]), h["w"], f"{what} tensor {i} master")
        nbit += nb
        for k in ("mc", "ms", "vc", "vs"):
            got = to_host(d[k])
            bad = np.nonzero(got != h[k])[0]
            assert bad.size == 0, (f"{what} tensor {i} {k}: {bad.size} bytes differ, first at "
                                   f"{int(bad[0])}: {int(got[bad[0]])} vs {int(h[k][bad[0]])}")
        if h["p"] is not None:
            check_bf16(to_host(d["p"]), h["p"], f"{what} tensor {i} copy")
    return nbit


def step_and_compare(host, what, max_norm=1.0, hp=HP, offset=0, steps=1, completed=0,
                     clipped=False):
    s8 = Step8(host, offset=offset, completed_steps=completed)
    for k in range(steps):
        S_gpu, c, t = s8.run(max_norm, hp, clipped=clipped)
        check_norm(S_gpu, host, f"{what} step {k}")
        assert t == completed + k + 1
        oracle_step(host, c, t, hp)
        nbit = compare(s8, host, f"{what} step {k}")
        say(f"{what} step {k}: S={S_gpu:.6e} c={float(c):.6f} master not bitwise: {nbit}")
    s8.tl.release()


SIZES = [1, 31, 32, 33, 100, 2048, 4096 + 5, 3 * 16384 + 17, 70000]


def test_q8_ragged_list_fp32_grads():
    say("q8 ragged list, fp32 gradients, warm state, t = 9")
    step_and_compare(make_host(SIZES, 101, bf16=False, copy_every=0), "fp32", completed=8)


def test_q8_ragged_list_bf16_grads_with_copy():
    say("q8 ragged list, bf16 gradients, copy, cold start, two steps")
    step_and_compare(make_host(SIZES, 102, bf16=True, copy_every=2, warm=False), "bf16",
                     steps=2)


@pytest.mark.parametrize("bf16", [False, True])
def test_q8_clipped_ragged_two_steps(bf16):
    say(f"q8 clipped step, ragged list, bf16 gradients={bf16}")
    step_and_compare(make_host(SIZES, 105 + bf16, bf16=bf16, copy_every=2), f"clipped bf16={bf16}",
                     steps=2, completed=4, clipped=True)


def test_q8_clipped_is_bitwise_the_three_call_step():
    host = make_host(SIZES + [0, 250000], 107, bf16=True, copy_every=1)
    a, b = Step8(host, completed_steps=2), Step8(host, completed_steps=2)
    for _ in range(2):
        ra = a.run(1.0, clipped=True, skip_if_nonfinite=True)
        rb = b.run(1.0, clipped=False, skip_if_nonfinite=True)
        assert np.float64(ra[0]).tobytes() == np.float64(rb[0]).tobytes()
        assert np.float32(ra[1]).tobytes() == np.float32(rb[1]).tobytes() and ra[2] == rb[2]
    for da, db in zip(a.dev, b.dev):
        for k, x in da.items():
            if x is not None and x.numel():
                assert torch.equal(x.view(torch.uint8), db[k].view(torch.uint8)), k
    a.tl.release()
    b.tl.release()


def test_q8_clipped_skip_if_nonfinite():
    host = make_host([5000, 77], 108, bf16=True, copy_every=1)
    host[1]["g"][10] = 0x7FC0  # a bf16 NaN
    s8 = Step8(host, completed_steps=6)
    before = [{k: x.clone() for k, x in d.items() if x is not None} for d in s8.dev]
    S, _, t = s8.run(1.0, clipped=True, skip_if_nonfinite=True)
    assert np.isnan(S) and t == 6
    for d, b in zip(s8.dev, before):
        for k, x in b.items():
            if x.numel():
                assert torch.equal(d[k].view(torch.uint8), x.view(torch.uint8)), k
    s8.tl.release()


def test_q8_misaligned_views_take_the_element_path():
    say("q8 views one element past an aligned start")
    host = make_host([5, 64, 1000, 40000 + 3], 103, bf16=True, copy_every=1)
    step_and_compare(host, "misaligned", offset=1, completed=3)


def test_q8_five_steps_track_the_oracle():
    say("q8 five consecutive steps, bf16 gradients with outliers")
    host = make_host([300000, 12345, 64], 104, bf16=True, copy_every=1)
    o = oracle.default()
    g = o.bf16_to_f32(host[0]["g"][:2000]) * np.float32(50.0)
    host[0]["g"][:2000] = o.f32_to_bf16(g)
    step_and_compare(host, "five", steps=5, completed=20)


def crafted_run(rng):
    """Gradients that, with beta1 = beta2 = 0 and no clipping, make the new
    moments land on rounding ties and in the subnormal codes: m = g exactly,
    v = g * g exactly."""
    runs = []
    # E4M3 ties: the run's largest |m| is 448 * 2^-(20+k); the others sit
    # halfway between neighbouring codes at the same scale.
    grid = np.unique(np.abs(torch.arange(128, dtype=torch.uint8).view(
        torch.float8_e4m3fn).double().numpy()[1:0x7F]))
    mids = (grid[:-1] + grid[1:]) / 2
    for k in range(6):
        r = np.empty(32)
        r[0] = 448.0
        r[1:] = rng.choice(mids, 31)
        r[1:] *= rng.choice([-1.0, 1.0], 31)
        r[5] = 2.0 ** -10                         # half the smallest subnormal: ties to 0
        r[6] = 3 * 2.0 ** -11                     # rounds up to the smallest subnormal
        runs.append(r * 2.0 ** (-20 - k))
    # E5M2 ties in v: largest v = 2^-4 (scale exponent -19); v = 9 * 2^-12 scales
    # to 1152, halfway between 1024 and 1280.
    r = np.full(32, 3 * 2.0 ** -6)
    r[0] = 0.25
    r[1::2] *= -1
    runs.append(r)
    # a run of tiny values: largest |m| below 448 * 2^-127, clamped exponent
    runs.append(rng.standard_normal(32) * 1e-37)
    # exactly on an exponent boundary, and a negative zero
    r = rng.standard_normal(32) * 2.0 ** -15
    r[0] = 448.0 * 2.0 ** -16
    r[3] = -0.0
    runs.append(r)
    return np.concatenate(runs).astype(np.float32)


def test_q8_rounding_ties_and_tiny_runs():
    say("q8 crafted ties, subnormal codes, clamped exponents")
    rng = np.random.default_rng(105)
    g = crafted_run(rng)
    n = g.size
    o = oracle.default()
    host = [dict(w=(rng.standard_normal(n) * 0.02).astype(np.float32),
                 mc=np.zeros(n, np.uint8), ms=np.zeros(n // 32, np.uint8),
                 vc=np.zeros(n, np.uint8), vs=np.zeros(n // 32, np.uint8), g=g,
                 p=np.zeros(n, np.uint16))]
    hp = dict(HP, beta1=0.0, beta2=0.0)
    # with max_norm huge the coefficient is exactly 1, so m = g and v = g * g
    s8 = Step8(host)
    S_gpu, c, t = s8.run(1e30, hp)
    assert c == np.float32(1.0)
    check_norm(S_gpu, host, "crafted")
    oracle_step(host, c, t, hp)
    compare(s8, host, "crafted")
    # the tie runs did exercise ties: half of their elements sit on midpoints
    first = host[0]["mc"][:32]
    assert (o.fp8_value(first & 0x7F, E4M3) * 2.0 ** 20 != np.abs(g[:32].astype(np.float64) * 2.0 ** 20)).sum() >= 28
    s8.tl.release()


def test_q8_nonfinite_gradient_poisons_its_run_only():
    say("q8 NaN gradient")
    host = make_host([200, 64], 106, bf16=False, copy_every=1)
    host[0]["g"][70] = np.nan
    s8 = Step8(host)
    S_gpu, c, t = s8.run(1.0)
    assert np.isnan(S_gpu) and np.isnan(c)
    oracle_step(host, c, t)
    compare(s8, host, "nan")
    ms = to_host(s8.dev[0]["ms"])
    assert (ms == 255).all()  # c is NaN, so every run is NaN
    s8.tl.release()
    # with the skip rule nothing is written and the counter stays
    host = make_host([200, 64], 106, bf16=False, copy_every=1)
    host[0]["g"][70] = np.nan
    s8 = Step8(host, completed_steps=4)
    before = {k: to_host(v).copy() for k, v in s8.dev[0].items() if v is not None}
    S_gpu, c, t = s8.run(1.0, skip_if_nonfinite=True)
    assert t == 4
    for k, v in before.items():  # bytes, so that the NaN gradient compares equal
        assert np.array_equal(to_host(s8.dev[0][k]).view(np.uint8), v.view(np.uint8)), k
    s8.tl.release()


def test_q8_nan_in_one_run_with_finite_coefficient():
    """An infinite gradient gives c = 0: its element's moments become NaN
    (inf * 0), so only that run is stored as non-finite."""
    say("q8 infinite gradient")
    host = make_host([200], 107, bf16=False, copy_every=1)
    host[0]["g"][100] = np.inf
    s8 = Step8(host)
    S_gpu, c, t = s8.run(1.0)
    assert np.isinf(S_gpu) and c == 0.0
    oracle_step(host, c, t)
    compare(s8, host, "inf")
    ms = to_host(s8.dev[0]["ms"])
    assert ms[3] == 255 and (np.delete(ms, 3) != 255).all()
    s8.tl.release()


def test_q8_zero_state_and_zero_gradient():
    say("q8 zero state, zero gradient")
    n = 5000
    rng = np.random.default_rng(108)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    dev_w = torch.from_numpy(w).cuda()
    state = binding.zeros_q8_state(n, "cuda")
    g = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    tl = binding.TensorList8([dev_w], [state], [g])
    coef = torch.ones(1, dtype=torch.float32, device="cuda")
    step = torch.zeros(1, dtype=torch.int32, device="cuda")
    binding.adamw8_multi_tensor_step(tl, coef, step, **{k if k != "wd" else "weight_decay": v
                                                        for k, v in HP.items()})
    torch.cuda.synchronize()
    decay = np.float32(1.0 - 3e-4 * 0.1)
    assert np.array_equal(dev_w.cpu().numpy().view(np.uint32), (w * decay).view(np.uint32))
    for a in state:
        assert not a.cpu().numpy().any()
    tl.release()


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_q8_quantize_and_dequantize_match_oracle(fmt):
    say(f"q8 conversion kernels, format {fmt}")
    rng = np.random.default_rng(109 + fmt)
    n = 32 * 5000 + 19
    x = rng.standard_normal(n) * 10.0 ** rng.integers(-40, 35, size=(n + 31) // 32).repeat(32)[:n]
    x = x.astype(np.float32)
    x[32:64] = 0.0
    x[100] = np.nan
    x[200] = -np.inf
    x[300] = -0.0
    x[400:432] = (rng.standard_normal(32) * 1e-40).astype(np.float32)
    o = oracle.default()
    rc, rs = o.quantize(x, fmt)
    xd = torch.from_numpy(x).cuda()
    codes = torch.empty(n, dtype=torch.uint8, device="cuda")
    scales = torch.empty((n + 31) // 32, dtype=torch.uint8, device="cuda")
    binding.adamw8_quantize(xd, fmt, codes, scales)
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    binding.adamw8_dequantize(codes, scales, fmt, out)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy(), rs)
    want = o.dequantize(rc, rs, fmt)
    got = out.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok].view(np.uint32), want[ok].view(np.uint32))
    # every code of both formats decodes like the oracle (all 256, at scale 2^0)
    allc = torch.arange(256, dtype=torch.uint8, device="cuda").repeat(2)
    sc = torch.full((16,), 127, dtype=torch.uint8, device="cuda")
    out = torch.empty(512, dtype=torch.float32, device="cuda")
    binding.adamw8_dequantize(allc, sc, fmt, out)
    torch.cuda.synchronize()
    want = o.fp8_value(np.arange(256), fmt)
    got = out.cpu().numpy()[:256].astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[~np.isnan(want)], want[~np.isnan(want)])


def test_q8_empty_and_single_tensor_lists():
    say("q8 empty tensors in the list")
    host = make_host([0, 45, 0], 110, bf16=True, copy_every=1)
    step_and_compare(host, "empty")


def test_q8_bf16_copy_rounds_to_nearest_even():
    """The 8-bit kernel's copy on crafted masters (lr = 0, zero state and
    gradients keep the master): vector path and element path."""
    from gpu_harness import crafted_bf16_masters
    w = crafted_bf16_masters(np.random.default_rng(32))
    n = w.size - w.size % 32            # whole runs: vector path ...
    w = w[:n]
    host = []
    for extra in (0, 5):                # ... and a partial run: element path
        m = w.size + extra
        wm = np.concatenate([w, np.float32([1.0, -2.5, 3e-39, 0.1, 7.0])[:extra]]).astype(np.float32)
        host.append(dict(w=wm, mc=np.zeros(m, np.uint8), ms=np.zeros((m + 31) // 32, np.uint8),
                         vc=np.zeros(m, np.uint8), vs=np.zeros((m + 31) // 32, np.uint8),
                         g=np.zeros(m, np.float32), p=np.zeros(m, np.uint16)))
    s8 = Step8(host)
    S_gpu, c, t = s8.run(1.0, dict(HP, lr=0.0))
    assert S_gpu == 0.0 and c == np.float32(1.0)
    o = oracle.default()
    for d, h in zip(s8.dev, host):
        want = o.f32_to_bf16(h["w"])
        got = to_host(d["p"])
        nan = np.isnan(h["w"])
        assert ((got & 0x7FFF) > 0x7F80)[nan].all()
        assert np.array_equal(got[~nan], want[~nan])
    s8.tl.release()


@pytest.mark.parametrize("t", [1, 2, 10, 1000, 123456])
def test_q8_step_counter_and_bias_corrections(t):
    say(f"q8 bias corrections at t = {t}")
    step_and_compare(make_host([4099, 64], 111, bf16=True, copy_every=1), f"t={t}",
                     completed=t - 1)


@pytest.mark.parametrize("hp", [dict(lr=0.0, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1),
                                dict(lr=1e-2, beta1=0.0, beta2=0.0, eps=1e-6, wd=0.0),
                                dict(lr=1e-3, beta1=0.5, beta2=0.999, eps=0.0, wd=1.0)])
def test_q8_hyperparameter_corners(hp):
    say(f"q8 hyperparameters {hp}")
    step_and_compare(make_host([3000, 33], 112, bf16=False, copy_every=1), "hp", hp=hp,
                     completed=4)


# ------------------------------------------------------- full sizes ---

def random_q8_state(n, rng, warm):
    """A valid seeded 8-bit state without the encoder: random finite codes and
    scale bytes near those of m ~ N(0, 1e-4) and v = |N(0, 1e-8)| (warm), or
    all zero."""
    nb = (n + 31) // 32
    if not warm:
        return (np.zeros(n, np.uint8), np.zeros(nb, np.uint8), np.zeros(n, np.uint8),
                np.zeros(nb, np.uint8))
    mc = rng.integers(0, 0x7F, size=n, dtype=np.uint8) | (rng.integers(0, 2, size=n, dtype=np.uint8) << 7)
    vc = rng.integers(0, 0x7C, size=n, dtype=np.uint8)
    ms = rng.integers(105, 109, size=nb, dtype=np.uint8)
    vs = rng.integers(85, 89, size=nb, dtype=np.uint8)
    return mc, ms, vc, vs


def sampled_runs(n, k, rng):
    """Run indices: the first and last run, runs at chunk edges, k random."""
    nr = (n + 31) // 32
    fixed = {0, nr - 1} | {r for q in range(64, min(nr, 2048) + 1, 64) for r in (q - 1, q) if r < nr}
    return sorted(fixed | set(rng.integers(0, nr, size=min(k, nr)).tolist()))


@pytest.mark.parametrize("cfg,clipped", [(2, True), (5, True), (4, True), (3, True), (2, False)])
def test_q8_full_size_sampled(cfg, clipped):
    """The bench's workload and launches with 8-bit moments (the clipped
    step; once also the three-call step): the sum of squares over every
    gradient, and sampled runs of 32 recomputed by the oracle from their
    inputs gathered before the step."""
    from mixed_precision_sharded_amd.configs import WORKLOADS
    w = WORKLOADS[cfg]
    free, _ = torch.cuda.mem_get_info()
    need = w.numel * (w.state8_bytes_per_param() + 4) + (8 << 30)
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB free, {free / 2**30:.0f} GiB available")
    q8_sampled_parity(w, seed=200 + cfg, clipped=clipped)


@pytest.mark.parametrize("cfg", [2, 4, 5])
def test_q8_full_size_every_element(cfg):
    """The bench's workload and launch with 8-bit moments, every element of
    every tensor against the oracle stepped with the GPU's coefficient:
    master (bitwise first, else the tolerance), both code arrays and both
    scale arrays exactly.  The 8-bit oracle's nearest-code search takes 15M
    elements/s on 16 threads, so the 8B full list (8.03e9 elements, about
    nine minutes) is left to the sampled test above."""
    from concurrent.futures import ThreadPoolExecutor
    from mixed_precision_sharded_amd import synth
    from mixed_precision_sharded_amd.configs import WORKLOADS
    from mixed_precision_sharded_amd.synth import to_numpy

    w = WORKLOADS[cfg]
    free, _ = torch.cuda.mem_get_info()
    need = w.numel * (w.state8_bytes_per_param() + 4) + (8 << 30)
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB free, {free / 2**30:.0f} GiB available")
    warm = w.m_std is not None
    say(f"q8 every element: {w.name}, {w.numel:,} params in {w.n_tensors} tensors, warm={warm}")
    cols = synth.workload_inputs(w, "cuda")
    del cols["exp_avg"], cols["exp_avg_sq"]
    rng = np.random.default_rng(300 + cfg)
    host = [random_q8_state(n, rng, warm) for _, n in w.tensors]
    states = [tuple(torch.from_numpy(a).cuda() for a in st) for st in host]
    before_w = [to_numpy(t).copy() for t in cols["master"]]
    grads = [to_numpy(t).copy() for t in cols["grad"]]
    o = oracle.default()
    S_ref = o.grad_norm_sq(grads)

    say("GPU step (8-bit moments, clipped)")
    tl = binding.TensorList8(cols["master"], states, cols["grad"], cols["param_bf16"])
    sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    coef = torch.zeros(1, dtype=torch.float32, device="cuda")
    step = torch.tensor([w.step - 1], dtype=torch.int32, device="cuda")
    binding.adamw8_clipped_step(tl, step, w.lr, w.beta1, w.beta2, w.eps, w.weight_decay,
                                w.max_norm, sumsq_out=sumsq, coef_out=coef)
    torch.cuda.synchronize()
    S, c, t = float(sumsq.item()), np.float32(coef.item()), int(step.item())
    assert t == w.step
    assert abs(S - S_ref) <= NORM_REL_TOL * S_ref, (S, S_ref)
    assert c == o.clip_coef(S, w.max_norm)
    say(f"S={S:.9e} oracle {S_ref:.9e} c={float(c)}; the oracle over every element")

    # The oracle on the pre-step host state, in slices cut at multiples of
    # the 32-element runs (one scale byte each), 16 threads.
    copies = [np.zeros(n, np.uint16) if w.copy_bf16 else None for _, n in w.tensors]
    piece = 1 << 20
    items = [(i, lo, min(lo + piece, n)) for i, (_, n) in enumerate(w.tensors)
             for lo in range(0, n, piece)]

    def one(item):
        i, lo, hi = item
        mc, ms, vc, vs = host[i]
        r0, r1 = lo // 32, (hi + 31) // 32
        o.adamw8_step(before_w[i][lo:hi], mc[lo:hi], ms[r0:r1], vc[lo:hi], vs[r0:r1],
                      grads[i][lo:hi], None if copies[i] is None else copies[i][lo:hi], c, w.step,
                      w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)

    t0 = time.time()
    with ThreadPoolExecutor(max_workers=16) as pool:
        list(pool.map(one, items))
    say(f"oracle done in {time.time() - t0:.0f} s; comparing")

    nbit = 0
    for i, (_, n) in enumerate(w.tensors):
        got_w = to_numpy(cols["master"][i])
        if not np.array_equal(got_w.view(np.uint32), before_w[i].view(np.uint32)):
            nb, _ = check_f32(got_w, before_w[i], f"{w.name} tensor {i} master")
            nbit += nb
        for k, name in enumerate(("m codes", "m scales", "v codes", "v scales")):
            got = states[i][k].cpu().numpy()
            if not np.array_equal(got, host[i][k]):
                bad = np.flatnonzero(got != host[i][k])
                raise AssertionError(f"{w.name} tensor {i} {name}: {bad.size} differ, first at "
                                     f"{bad[0]}: {got[bad[0]]} against {host[i][k][bad[0]]}")
        if w.copy_bf16:
            check_bf16(to_numpy(cols["param_bf16"][i]), copies[i], f"{w.name} tensor {i} copy")
    say(f"{w.numel:,} elements checked (master, codes, scales{', copy' if w.copy_bf16 else ''}); "
        f"{nbit} master elements not bitwise equal")
    tl.release()
    del tl, cols, states
    torch.cuda.empty_cache()


def test_q8_single_tensor_over_2g_elements_sampled():
    """One tensor of 2^31 + 1003 elements (runs around element 2^31
    included): 64-bit offsets throughout."""
    from mixed_precision_sharded_amd.configs import Workload
    w = Workload(cfg=91, name="single_tensor_2g", tensors=(("huge", (1 << 31) + 1003),),
                 grad_bf16=True, copy_bf16=True, step=5, m_std=1e-4, v_std=1e-8)
    free, _ = torch.cuda.mem_get_info()
    need = w.numel * 16 + (8 << 30)
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB free, {free / 2**30:.0f} GiB available")
    q8_sampled_parity(w, seed=210, extra_runs=[((1 << 31) >> 5) + d for d in range(-3, 4)])


def q8_sampled_parity(w, seed, extra_runs=(), clipped=True):
    from mixed_precision_sharded_amd import synth
    from mixed_precision_sharded_amd.synth import to_numpy

    warm = w.m_std is not None
    say(f"q8 full size: {w.name}, {w.numel:,} params in {w.n_tensors} tensors, warm={warm}")
    cols = synth.workload_inputs(w, "cuda")
    del cols["exp_avg"], cols["exp_avg_sq"]
    rng = np.random.default_rng(seed)
    states, picks, before = [], [], []
    per_tensor = max(4, 6000 // w.n_tensors)
    for i, (_, n) in enumerate(w.tensors):
        st = tuple(torch.from_numpy(a).cuda() for a in random_q8_state(n, rng, warm))
        states.append(st)
        runs = sorted(set(sampled_runs(n, per_tensor, rng)) |
                      {r for r in extra_runs if 0 <= r < (n + 31) // 32})
        elems = torch.tensor([e for r in runs for e in range(32 * r, min(32 * r + 32, n))],
                             dtype=torch.int64, device="cuda")
        rix = torch.tensor(runs, dtype=torch.int64, device="cuda")
        picks.append((runs, elems, rix))
        before.append(dict(w=to_numpy(cols["master"][i][elems]), g=to_numpy(cols["grad"][i][elems]),
                           mc=st[0][elems].cpu().numpy(), ms=st[1][rix].cpu().numpy(),
                           vc=st[2][elems].cpu().numpy(), vs=st[3][rix].cpu().numpy()))
    torch.cuda.synchronize()
    say("oracle sum of squares over every gradient")
    o = oracle.default()
    S_ref = o.grad_norm_sq(to_numpy(g) for g in cols["grad"])

    say("GPU step (8-bit moments)")
    tl = binding.TensorList8(cols["master"], states, cols["grad"], cols["param_bf16"])
    sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    coef = torch.zeros(1, dtype=torch.float32, device="cuda")
    step = torch.tensor([w.step - 1], dtype=torch.int32, device="cuda")
    if clipped:
        binding.adamw8_clipped_step(tl, step, w.lr, w.beta1, w.beta2, w.eps, w.weight_decay,
                                    w.max_norm, sumsq_out=sumsq, coef_out=coef)
    else:
        binding.adamw8_grad_norm_sq(tl, sumsq, w.max_norm, coef)
        binding.adamw8_multi_tensor_step(tl, coef, step, w.lr, w.beta1, w.beta2, w.eps,
                                         w.weight_decay)
    torch.cuda.synchronize()
    S, c, t = float(sumsq.item()), np.float32(coef.item()), int(step.item())
    assert t == w.step
    assert abs(S - S_ref) <= NORM_REL_TOL * S_ref, (S, S_ref)
    assert c == o.clip_coef(S, w.max_norm)
    say(f"S={S:.9e} oracle {S_ref:.9e} c={float(c)}")

    n_runs = nbit = 0
    for i, (_, n) in enumerate(w.tensors):
        runs, elems, rix = picks[i]
        b = before[i]
        got_w = to_numpy(cols["master"][i][elems])
        got = [states[i][0][elems].cpu().numpy(), states[i][1][rix].cpu().numpy(),
               states[i][2][elems].cpu().numpy(), states[i][3][rix].cpu().numpy()]
        got_p = to_numpy(cols["param_bf16"][i][elems]) if w.copy_bf16 else None
        off = 0
        for j, r in enumerate(runs):
            k = min(32 * r + 32, n) - 32 * r
            sl = slice(off, off + k)
            ww = b["w"][sl].copy()
            mc, vc = b["mc"][sl].copy(), b["vc"][sl].copy()
            ms, vs = b["ms"][j:j + 1].copy(), b["vs"][j:j + 1].copy()
            pv = np.zeros(k, np.uint16) if w.copy_bf16 else None
            o.adamw8_step(ww, mc, ms, vc, vs, np.ascontiguousarray(b["g"][sl]), pv, c, w.step,
                          w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)
            nb, _ = check_f32(got_w[sl], ww, f"{w.name} tensor {i} run {r} master")
            nbit += nb
            assert np.array_equal(got[0][sl], mc), (i, r, "m codes")
            assert got[1][j] == ms[0], (i, r, "m scale")
            assert np.array_equal(got[2][sl], vc), (i, r, "v codes")
            assert got[3][j] == vs[0], (i, r, "v scale")
            if w.copy_bf16:
                check_bf16(got_p[sl], pv, f"{w.name} tensor {i} run {r} copy")
            off += k
            n_runs += 1
        assert bool(torch.isfinite(cols["master"][i]).all()), i
    say(f"{n_runs:,} sampled runs checked; {nbit} master elements not bitwise equal")
    tl.release()
    del tl, cols, states
    torch.cuda.empty_cache()
