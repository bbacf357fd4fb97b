"""Pins of the CPU oracle: checks against things other than the oracle itself.

Each `pin_*(o)` takes an `oracle.Oracle` and raises AssertionError when the
oracle disagrees with
  - a library routine computing the same quantity (torch's bf16 conversion,
    torch.optim.AdamW and torch.nn.utils.clip_grad_norm_ in float64),
  - exact rational arithmetic (fractions; sqrt to 60 digits),
  - closed forms (first step from zero state, zero gradient, lr = 0,
    beta1 = beta2 = 0, clipping at S = 0 and S = 4 max_norm^2),
  - invariants (v >= 0, the Cauchy-Schwarz bound |m| <= 1.165 sqrt(v),
    independence of m and v from lr / wd / master, list = flat concatenation).
The same functions run against deliberately broken copies of the oracle in
test_oracle_mutants.py, which checks that every planted mistake is caught.
"""
import math
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import torch

U32 = 2.0 ** -24  # unit roundoff of fp32

LR, B1, B2, EPS, WD = 3e-4, 0.9, 0.95, 1e-8, 0.1


# ------------------------------------------------------------- helpers ---

def fr(x) -> Fraction:
    """Exact value of a binary float (float, np.float32, np.float64)."""
    return Fraction(float(x))


def dec(s: str) -> Fraction:
    """Exact value of a decimal literal."""
    return Fraction(s)


def sqrt_fr(x: Fraction) -> Fraction:
    """sqrt(x) to 60 significant digits."""
    if x == 0:
        return Fraction(0)
    with localcontext() as ctx:
        ctx.prec = 60
        d = (Decimal(x.numerator) / Decimal(x.denominator)).sqrt()
    return Fraction(d)


def round_f32(x: Fraction) -> np.float32:
    """Round an exact value to the nearest fp32, ties to even (normal range)."""
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while a >= Fraction(2) ** (e + 1):
        e += 1
    while a < Fraction(2) ** e:
        e -= 1
    assert -126 <= e <= 127, "round_f32 covers the normal range only"
    scaled = a * Fraction(2) ** (23 - e)
    q, r = divmod(scaled.numerator, scaled.denominator)
    rem = Fraction(r, scaled.denominator)
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    return np.float32(sign * float(Fraction(q) * Fraction(2) ** (e - 23)))


def ulp32(x) -> float:
    x = np.abs(np.float32(x))
    return float(np.spacing(x)) if x > 0 else float(np.spacing(np.float32(0)))


def bf16_bits_torch(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def rand_state(n, seed, warm=True):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    if warm:
        m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        v = np.abs(rng.standard_normal(n) * 1e-8).astype(np.float32)
    else:
        m = np.zeros(n, np.float32)
        v = np.zeros(n, np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    return w, m, v, g


def run_step(o, w, m, v, g, c, t, lr=LR, b1=B1, b2=B2, eps=EPS, wd=WD, copy=False):
    w, m, v = w.copy(), m.copy(), v.copy()
    p = np.zeros(w.size, np.uint16) if copy else None
    o.adamw_step(w, m, v, g, p, c, t, lr, b1, b2, eps, wd)
    return (w, m, v, p) if copy else (w, m, v)


def assert_within(actual, exact, bound, what):
    actual = np.asarray(actual, dtype=np.float64)
    exact = np.asarray(exact, dtype=np.float64)
    err = np.abs(actual - exact)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} beyond bound; worst err "
                           f"{float(err.max()):.3e} vs bound {float(np.asarray(bound).min()):.3e}")


# --------------------------------------------------------------- bf16 ---

def pin_bf16_rounding_matches_torch(o):
    rng = np.random.default_rng(1)
    vals = [rng.standard_normal(20000).astype(np.float32) * s for s in (1e-30, 1e-3, 1.0, 1e30)]
    words = np.array([
        0x3f808000, 0x3f818000, 0x3f807fff, 0x3f808001,   # ties to even (down, up), near ties
        0x7f7fffff, 0x7f7f8000, 0x7f7f7fff, 0xff7f8000,   # top of the range
        0x00000001, 0x00008000, 0x00018000, 0x007fffff,   # denormals, including ties
        0x00000000, 0x80000000, 0x7f800000, 0xff800000,   # zeros and infinities
    ], dtype=np.uint32).view(np.float32)
    x = np.concatenate(vals + [words])
    got = o.f32_to_bf16(x)
    want = bf16_bits_torch(x)
    mismatch = np.nonzero(got != want)[0]
    assert mismatch.size == 0, f"bf16 rounding differs from torch at {x[mismatch[:5]]}"


def pin_bf16_nan_is_quiet_and_signed(o):
    nans = np.array([0x7f800001, 0xff800001, 0x7fc00000, 0xffffffff, 0x7fa00000],
                    dtype=np.uint32).view(np.float32)
    got = o.f32_to_bf16(nans)
    assert np.all((got & 0x7f80) == 0x7f80) and np.all((got & 0x7f) != 0), "NaN must stay NaN"
    assert np.all(got & 0x0040), "NaN must come out quiet"
    assert np.array_equal(got >> 15, (nans.view(np.uint32) >> 31).astype(np.uint16)), "NaN sign kept"


def pin_bf16_widening_is_exact(o):
    words = np.arange(0, 1 << 16, 97, dtype=np.uint32).astype(np.uint16)
    got = o.bf16_to_f32(words)
    want = torch.from_numpy(words.view(np.int16)).view(torch.bfloat16).float().numpy()
    both_nan = np.isnan(got) & np.isnan(want)
    assert np.all((got.view(np.uint32) == want.view(np.uint32)) | both_nan)


# --------------------------------------------------------------- norm ---

def pin_norm_exact_on_dyadic_values(o):
    rng = np.random.default_rng(2)
    a = (rng.integers(-64, 65, 5000) / 8.0).astype(np.float32)
    b = (rng.integers(-8, 9, 3001) / 4.0).astype(np.float32)
    exact = sum(fr(x) ** 2 for x in a) + sum(fr(x) ** 2 for x in b)
    assert Fraction(o.grad_norm_sq([a, b])) == exact
    c = np.ones(777, np.float32)
    c[::3] = -1.0
    assert o.grad_norm_sq([c]) == 777.0
    hb = o.f32_to_bf16(a)  # a's values are exact in bf16
    assert Fraction(o.grad_norm_sq([hb])) == sum(fr(x) ** 2 for x in a)


def pin_norm_matches_fsum(o):
    rng = np.random.default_rng(3)
    parts = [(rng.standard_normal(n) * 10.0 ** rng.integers(-4, 2)).astype(np.float32)
             for n in (100000, 7, 33333)]
    S = o.grad_norm_sq(parts)
    exact = math.fsum(float(x) * float(x) for p in parts for x in p)
    n = sum(p.size for p in parts)
    assert abs(S - exact) <= n * 2.0 ** -53 * exact
    hb = [o.f32_to_bf16(p) for p in parts]
    Sb = o.grad_norm_sq(hb)
    exact_b = math.fsum(float(x) ** 2 for p in hb
                        for x in torch.from_numpy(p.view(np.int16)).view(torch.bfloat16).double().numpy())
    assert abs(Sb - exact_b) <= n * 2.0 ** -53 * exact_b


def pin_norm_list_equals_concatenation(o):
    rng = np.random.default_rng(4)
    a = rng.standard_normal(1000).astype(np.float32)
    b = rng.standard_normal(2345).astype(np.float32)
    assert o.grad_norm_sq([a, b]) == o.grad_norm_sq([np.concatenate([a, b])])


# --------------------------------------------------------------- clip ---

def pin_clip_closed_forms(o):
    assert o.clip_coef(0.0, 1.0) == np.float32(1.0)
    assert o.clip_coef(1e-20, 1.0) == np.float32(1.0)
    for mn in ("1.0", "0.5", "3.0", "0.25"):
        m = float(mn)
        want = round_f32(dec(mn) / (2 * dec(mn) + dec("1e-6")))
        got = o.clip_coef(4.0 * m * m, m)
        assert abs(float(got) - float(want)) <= ulp32(want), (mn, got, want)
        assert got < np.float32(0.5)
        want1 = round_f32(dec(mn) / (dec(mn) + dec("1e-6")))
        assert abs(float(o.clip_coef(m * m, m)) - float(want1)) <= ulp32(want1)
        assert o.clip_coef(m * m, m) < np.float32(1.0)
    assert np.isnan(o.clip_coef(float("nan"), 1.0))
    assert o.clip_coef(float("inf"), 1.0) == np.float32(0.0)
    # the 2^20-parameter bf16 workload's norm is just above 1: clipping must act
    c = o.clip_coef(1.049, 1.0)
    assert np.float32(0.97) < c < np.float32(0.98)


def pin_clip_matches_torch(o):
    rng = np.random.default_rng(5)
    for scale, mn in ((1e-3, 1.0), (1.0, 1.0), (1e-2, 0.05), (1e-5, 1.0)):
        parts = [(rng.standard_normal(n) * scale).astype(np.float32) for n in (3000, 500)]
        S = o.grad_norm_sq(parts)
        c = o.clip_coef(S, mn)
        ps = [torch.nn.Parameter(torch.zeros(p.size, dtype=torch.float64)) for p in parts]
        for p, g in zip(ps, parts):
            p.grad = torch.from_numpy(g.astype(np.float64))
        before = [p.grad.clone() for p in ps]
        torch.nn.utils.clip_grad_norm_(ps, mn)
        k = int(np.argmax(np.abs(parts[0])))
        coef = float(ps[0].grad[k] / before[0][k])
        assert abs(float(c) - coef) <= ulp32(coef) + 1e-15, (scale, mn, c, coef)


def pin_scaled_clip_reduces_to_unscaled(o):
    rng = np.random.default_rng(30)
    for S in [0.0, 1e-12, 0.25, 1.0, 1.049, 4.0, 1e6, float("inf"), float("nan")] + \
            list(rng.lognormal(0, 8, 100)):
        for mn in (1.0, 0.5, 3.0):
            a, b = o.clip_coef(S, mn), o.clip_coef(S, mn, 1.0)
            assert a.view(np.uint32) == b.view(np.uint32) or (np.isnan(a) and np.isnan(b)), (S, mn)


def pin_scaled_clip_matches_torch(o):
    """The multiplier for stored g equals s times torch's clip coefficient of s*g."""
    rng = np.random.default_rng(31)
    for scale, s, mn in ((1e-3, 0.125, 1.0), (1.0, 1 / 3, 1.0), (1e-2, 1 / 65536, 0.05),
                         (1e2, 0.25, 1.0), (1e-4, 1.0 / 7, 0.3)):
        parts = [(rng.standard_normal(n) * scale).astype(np.float32) for n in (3000, 41)]
        S = o.grad_norm_sq(parts)
        c = o.clip_coef(S, mn, s)
        ps = [torch.nn.Parameter(torch.zeros(p.size, dtype=torch.float64)) for p in parts]
        for p, g in zip(ps, parts):
            p.grad = torch.from_numpy(g.astype(np.float64)) * s
        before = [p.grad.clone() for p in ps]
        torch.nn.utils.clip_grad_norm_(ps, mn)
        k = int(np.argmax(np.abs(parts[0])))
        want = s * float(ps[0].grad[k] / before[0][k])
        assert abs(float(c) - want) <= ulp32(want) + 1e-300, (scale, s, mn, c, want)


def pin_power_of_two_scale_is_exact(o):
    """With s = 2^-k and S scaled by 4^k, the coefficient is 2^-k times the
    unscaled one, bitwise."""
    rng = np.random.default_rng(32)
    for S in list(rng.lognormal(0, 4, 200)) + [0.0, 1.0, 4.0]:
        for k in (1, 3, 10, 16):
            got = o.clip_coef(S * 4.0 ** k, 1.0, 2.0 ** -k)
            want = np.float32(o.clip_coef(S, 1.0) * np.float32(2.0 ** -k))
            assert got.view(np.uint32) == want.view(np.uint32), (S, k, got, want)


def pin_accumulation_scale_equals_averaged_gradient(o):
    """Lecture 9 exercises page, gradient-accumulation answer: summing K
    micro-batch gradients and dividing by K gives the large-batch gradient.
    Stepping on the summed gradient with s = 1/K matches stepping on the
    averaged one with s = 1 (K a power of two, so the average is exact)."""
    rng = np.random.default_rng(33)
    for K in (2, 4, 8):
        micro = [(rng.standard_normal(5000) * 1e-2).astype(np.float32) for _ in range(K)]
        summed = np.sum(np.stack(micro).astype(np.float64), axis=0).astype(np.float32)
        avg = (summed / np.float32(K)).astype(np.float32)
        c_sum = o.clip_coef(o.grad_norm_sq([summed]), 1.0, 1.0 / K)
        c_avg = o.clip_coef(o.grad_norm_sq([avg]), 1.0)
        assert c_sum.view(np.uint32) == np.float32(c_avg / np.float32(K)).view(np.uint32), K
        w, m, v, _ = rand_state(5000, 34 + K, warm=True)
        a = run_step(o, w, m, v, summed, c_sum, 3)
        b = run_step(o, w, m, v, avg, c_avg, 3)
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), K


def pin_skip_rule(o):
    assert o.skips(float("nan")) and o.skips(float("inf")) and o.skips(float("-inf"))
    assert not o.skips(0.0) and not o.skips(1e300)


# ------------------------------------------------------------ scalars ---

def pin_power_matches_exact(o):
    for beta in (0.9, 0.95, 0.999, 0.5):
        for t in (0, 1, 2, 3, 7, 100, 1000, 4095):
            exact = fr(beta) ** t
            if exact < Fraction(2) ** -1000:
                continue  # below the fp64 normal range
            got = Fraction(o.pow_int(beta, t))
            # each squaring doubles the relative error carried so far
            bound = 2 * max(t, 1) * Fraction(2) ** -53 * exact
            assert abs(got - exact) <= bound, (beta, t)


def pin_scalars_match_exact(o):
    for t in (1, 2, 3, 10, 100, 1000, 4321):
        for lr, b1, b2, eps, wd in (("3e-4", "0.9", "0.95", "1e-8", "0.1"),
                                    ("1.5e-4", "0.9", "0.95", "1e-8", "0.1"),
                                    ("1e-3", "0.8", "0.999", "1e-6", "0.01")):
            s = o.step_scalars(t, float(lr), float(b1), float(b2), float(eps), float(wd))
            L, P1, P2 = dec(lr), dec(b1), dec(b2)
            want = {
                "beta1": P1, "beta2": P2, "one_m_b1": 1 - P1, "one_m_b2": 1 - P2,
                "decay": 1 - L * dec(wd), "step_size": L / (1 - P1 ** t),
                "bc2_sqrt": sqrt_fr(1 - P2 ** t), "eps": dec(eps),
            }
            for k, exact in want.items():
                r = round_f32(exact)
                assert abs(float(s[k]) - float(r)) <= ulp32(r), (t, lr, k, s[k], r)


# ------------------------------------------------------------- update ---

def exact_step(w, m, v, g, c, t, lr="3e-4", b1="0.9", b2="0.95", eps="1e-8", wd="0.1"):
    """The AdamW step on exact values with decimal hyperparameters."""
    L, P1, P2, E, D = dec(lr), dec(b1), dec(b2), dec(eps), dec(wd)
    G = fr(g) * fr(c)
    M = P1 * fr(m) + (1 - P1) * G
    V = P2 * fr(v) + (1 - P2) * G * G
    mhat = M / (1 - P1 ** t)
    vhat_root = sqrt_fr(V / (1 - P2 ** t))
    W = fr(w) * (1 - L * D) - L * mhat / (vhat_root + E)
    return W, M, V


def step_bounds(w, m, v, g, c, t, lr=LR, b1=B1, b2=B2, wd=WD, eps=EPS):
    """Generous fp32 rounding bounds of one step (about ten roundings each,
    measured against the sizes of the terms, not of the result)."""
    w, m, v, g = (np.asarray(a, np.float64) for a in (w, m, v, g))
    gc = np.abs(g * c)
    m_terms = b1 * np.abs(m) + (1 - b1) * gc
    v_terms = b2 * np.abs(v) + (1 - b2) * gc * gc
    m_new = np.abs(b1 * m + (1 - b1) * g * c)
    v_new = b2 * v + (1 - b2) * gc * gc
    den = np.sqrt(v_new / (1 - b2 ** t)) + eps
    step = lr / (1 - b1 ** t)
    upd_terms = step * (m_terms + m_new) / den
    bw = 16 * U32 * (np.abs(w) * (1 - lr * wd) + upd_terms) + 1e-45
    return bw, 8 * U32 * m_terms + 1e-45, 8 * U32 * v_terms + 1e-45


def pin_update_matches_exact_rationals(o):
    for warm, t, c in ((True, 7, 0.8), (False, 1, 1.0), (True, 1000, 0.125), (True, 2, 1.0)):
        w, m, v, g = rand_state(24, 10 + t, warm)
        w1, m1, v1 = run_step(o, w, m, v, g, np.float32(c), t)
        bw, bm, bv = step_bounds(w, m, v, g, c, t)
        for i in range(w.size):
            W, M, V = exact_step(w[i], m[i], v[i], g[i], np.float32(c), t)
            assert abs(fr(w1[i]) - W) <= Fraction(float(bw[i])), ("w", i, t, w1[i], float(W))
            assert abs(fr(m1[i]) - M) <= Fraction(float(bm[i])), ("m", i, t)
            assert abs(fr(v1[i]) - V) <= Fraction(float(bv[i])), ("v", i, t)


def pin_update_each_op_rounds_once(o):
    """Replays the reading 'each fp32 operation rounds once, in order' with
    exact arithmetic and explicit rounding: the oracle must agree bitwise,
    i.e. its build neither contracts to FMA nor keeps excess precision."""
    w, m, v, g = rand_state(32, 21, True)
    t, c = 9, np.float32(0.75)
    s = o.step_scalars(t, LR, B1, B2, EPS, WD)
    w1, m1, v1 = run_step(o, w, m, v, g, c, t)
    R = round_f32
    for i in range(w.size):
        gg = R(fr(g[i]) * fr(c))
        mm = R(fr(R(fr(s["beta1"]) * fr(m[i]))) + fr(R(fr(s["one_m_b1"]) * fr(gg))))
        g2 = R(fr(gg) * fr(gg))
        vv = R(fr(R(fr(s["beta2"]) * fr(v[i]))) + fr(R(fr(s["one_m_b2"]) * fr(g2))))
        den = R(fr(R(fr(R(sqrt_fr(fr(vv)))) / fr(s["bc2_sqrt"]))) + fr(s["eps"]))
        ww = R(fr(R(fr(w[i]) * fr(s["decay"]))) - fr(R(fr(s["step_size"]) * fr(R(fr(mm) / fr(den))))))
        assert (m1[i], v1[i], w1[i]) == (mm, vv, ww), i


def pin_matches_torch_adamw_fp64(o):
    rng = np.random.default_rng(6)
    sizes = (2000, 1, 777)
    w = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
    m = [(rng.standard_normal(n) * 1e-4).astype(np.float32) for n in sizes]
    v = [np.abs(rng.standard_normal(n) * 1e-8).astype(np.float32) for n in sizes]
    for step in range(1, 5):
        g = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for n in sizes]
        g[0][rng.integers(0, sizes[0], 5)] *= 1000.0  # forces clipping
        for lr, wd, mn in ((LR, WD, 1.0), (1e-2, 0.5, 0.3)):
            S = o.grad_norm_sq(g)
            c = o.clip_coef(S, mn)
            assert c < 1.0
            params = [torch.nn.Parameter(torch.from_numpy(x.astype(np.float64))) for x in w]
            opt = torch.optim.AdamW(params, lr=lr, betas=(B1, B2), eps=EPS, weight_decay=wd,
                                    foreach=False)
            for p, gi, mi, vi in zip(params, g, m, v):
                p.grad = torch.from_numpy(gi.astype(np.float64))
                opt.state[p] = {"step": torch.tensor(float(step - 1), dtype=torch.float64),
                                "exp_avg": torch.from_numpy(mi.astype(np.float64)),
                                "exp_avg_sq": torch.from_numpy(vi.astype(np.float64))}
            torch.nn.utils.clip_grad_norm_(params, mn)
            opt.step()
            for k in range(len(sizes)):
                w1, m1, v1 = run_step(o, w[k], m[k], v[k], g[k], c, step, lr=lr, wd=wd)
                bw, bm, bv = step_bounds(w[k], m[k], v[k], g[k], float(c), step, lr=lr, wd=wd)
                st = opt.state[params[k]]
                assert_within(m1, st["exp_avg"].numpy(), bm, f"m step {step}")
                assert_within(v1, st["exp_avg_sq"].numpy(), bv, f"v step {step}")
                assert_within(w1, params[k].detach().numpy(), bw, f"w step {step}")
        w = [run_step(o, w[k], m[k], v[k], g[k], o.clip_coef(o.grad_norm_sq(g), 1.0), step)
             for k in range(len(sizes))]
        w, m, v = [x[0] for x in w], [x[1] for x in w], [x[2] for x in w]


def pin_first_step_closed_form(o):
    """m = v = 0, t = 1: w1 = w0 (1 - lr wd) - lr g / (|g| + eps), ~ lr sign(g)."""
    w, m, v, g = rand_state(4096, 7, warm=False)
    for c in (np.float32(1.0), np.float32(0.5)):
        w1, m1, v1 = run_step(o, w, m, v, g, c, 1)
        gc = g.astype(np.float64) * float(c)
        want = w.astype(np.float64) * (1 - LR * WD) - LR * gc / (np.abs(gc) + EPS)
        assert_within(w1, want, 8 * U32 * (np.abs(w) + LR) + 1e-12, "first-step w")
        big = np.abs(gc) > 1e-5
        assert_within((w.astype(np.float64) * (1 - LR * WD) - w1)[big], LR * np.sign(gc[big]),
                      LR * 2e-3, "first step ~ lr*sign(g)")
        assert_within(m1, (1 - B1) * gc, 3 * U32 * np.abs((1 - B1) * gc) + 1e-45, "m1")
        assert_within(v1, (1 - B2) * gc * gc, 4 * U32 * (1 - B2) * gc * gc + 1e-45, "v1")


def pin_zero_gradient(o):
    w, m, v, _ = rand_state(1000, 8, warm=False)
    g = np.zeros_like(w)
    w1, m1, v1 = run_step(o, w, m, v, g, np.float32(1.0), 1)
    decay = round_f32(1 - dec("3e-4") * dec("0.1"))
    assert np.array_equal(w1.view(np.uint32), (w * decay).view(np.uint32))
    assert not m1.any() and not v1.any()
    hb = o.f32_to_bf16(g)
    w2, m2, v2 = run_step(o, w, m, v, hb, np.float32(1.0), 1)
    assert np.array_equal(w2, w1) and not m2.any() and not v2.any()


def pin_lr_zero_keeps_master(o):
    w, m, v, g = rand_state(1000, 9, warm=True)
    w1, m1, v1 = run_step(o, w, m, v, g, np.float32(0.9), 5, lr=0.0)
    assert np.array_equal(w1.view(np.uint32), w.view(np.uint32))
    _, m2, v2 = run_step(o, w, m, v, g, np.float32(0.9), 5)
    assert np.array_equal(m1, m2) and np.array_equal(v1, v2)


def pin_moments_independent_of_lr_wd_master(o):
    w, m, v, g = rand_state(1000, 11, warm=True)
    _, m1, v1 = run_step(o, w, m, v, g, np.float32(0.6), 3)
    _, m2, v2 = run_step(o, -3 * w, m, v, g, np.float32(0.6), 3, lr=0.1, wd=0.0)
    assert np.array_equal(m1, m2) and np.array_equal(v1, v2)


def pin_no_momentum_closed_form(o):
    """beta1 = beta2 = 0: the step is lr g / (|g| + eps) at any t."""
    w, m, v, g = rand_state(2000, 12, warm=True)
    w1, _, _ = run_step(o, w, m, v, g, np.float32(1.0), 5, b1=0.0, b2=0.0)
    gd = g.astype(np.float64)
    want = w.astype(np.float64) * (1 - LR * WD) - LR * gd / (np.abs(gd) + EPS)
    assert_within(w1, want, 8 * U32 * (np.abs(w) + LR), "beta=0 step")


def pin_cauchy_schwarz_bound(o):
    rng = np.random.default_rng(13)
    n = 5000
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    k = (1 - B1) / math.sqrt((1 - B2) * (1 - B1 * B1 / B2))
    for t in range(1, 31):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-5, -1, n)).astype(np.float32)
        w, m, v = run_step(o, w, m, v, g, np.float32(1.0), t)
        assert np.all(v >= 0)
        assert np.all(np.abs(m) <= k * np.sqrt(v.astype(np.float64)) * (1 + 1e-5) + 1e-30), t


def pin_copy_is_rounded_master(o):
    w, m, v, g = rand_state(3000, 14, warm=True)
    w1, _, _, p = run_step(o, w, m, v, g, np.float32(1.0), 4, copy=True)
    assert np.array_equal(p, bf16_bits_torch(w1))


def pin_list_equals_flat_and_repeats(o):
    w, m, v, g = rand_state(3000, 15, warm=True)
    a, b = slice(0, 1234), slice(1234, 3000)
    whole = run_step(o, w, m, v, g, np.float32(0.7), 6)
    pa = run_step(o, w[a], m[a], v[a], g[a], np.float32(0.7), 6)
    pb = run_step(o, w[b], m[b], v[b], g[b], np.float32(0.7), 6)
    for k in range(3):
        assert np.array_equal(whole[k], np.concatenate([pa[k], pb[k]]))
    again = run_step(o, w, m, v, g, np.float32(0.7), 6)
    for k in range(3):
        assert np.array_equal(whole[k].view(np.uint32), again[k].view(np.uint32))


def pin_nonfinite_propagation(o):
    """A NaN gradient gives a NaN norm, a NaN coefficient and NaN updates;
    an infinite one gives c = 0, so inf * 0 = NaN at that element only."""
    w, m, v, g = rand_state(64, 16, warm=True)
    gn = g.copy()
    gn[5] = np.nan
    S = o.grad_norm_sq([gn])
    assert math.isnan(S) and np.isnan(o.clip_coef(S, 1.0))
    w1, m1, v1 = run_step(o, w, m, v, gn, o.clip_coef(S, 1.0), 3)
    assert np.isnan(w1).all() and np.isnan(m1).all()
    gi = g.copy()
    gi[7] = np.inf
    S = o.grad_norm_sq([gi])
    c = o.clip_coef(S, 1.0)
    assert math.isinf(S) and c == 0.0
    w1, m1, v1 = run_step(o, w, m, v, gi, c, 3)
    assert np.isnan(w1[7]) and np.isnan(m1[7]) and np.isnan(v1[7])
    rest = np.arange(64) != 7
    assert np.isfinite(w1[rest]).all()
    assert np.array_equal(m1[rest], (np.float32(B1) * m[rest]) + np.float32(0.0))


# ------------------------------------------------- 8-bit moment state ---
# Codes of m are E4M3, codes of v E5M2; 32 elements share a power-of-two
# scale.  The library routine pinned against is torch's fp32 -> float8 cast
# (round to nearest even) and its float8 -> fp32 widening; the block
# exponent is re-derived here from frexp.

Q_E4M3, Q_E5M2 = 0, 1
Q_LARGEST = {Q_E4M3: 448.0, Q_E5M2: 57344.0}
Q_TORCH = {Q_E4M3: torch.float8_e4m3fn, Q_E5M2: torch.float8_e5m2}
Q_HALF_STEP = {Q_E4M3: (2.0 ** -4, 2.0 ** -10), Q_E5M2: (2.0 ** -3, 2.0 ** -17)}


def q8_exponent_ref(absmax: float, fmt) -> int:
    """Smallest e >= -127 with absmax <= largest * 2^e, from frexp."""
    if absmax == 0.0:
        return -127
    mant, ex = math.frexp(absmax)                 # absmax = mant 2^ex, mant in [0.5, 1)
    lmant, lex = math.frexp(Q_LARGEST[fmt])      # 448 = 0.875 2^9, 57344 = 0.875 2^16
    e = ex - lex if mant <= lmant else ex - lex + 1
    return max(e, -127)


def q8_quantize_ref(x, fmt):
    """Independent quantizer: frexp exponent, codes from torch's float8 cast."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    codes = np.empty(x.size, np.uint8)
    scales = np.empty((x.size + 31) // 32, np.uint8)
    for b in range(0, x.size, 32):
        blk = x[b:b + 32]
        if not np.isfinite(blk).all():
            scales[b // 32] = 255
            codes[b:b + 32] = 255
            continue
        e = q8_exponent_ref(float(np.max(np.abs(blk))), fmt)
        scales[b // 32] = e + 127
        scaled = (blk.astype(np.float64) * 2.0 ** -e).astype(np.float32)
        codes[b:b + 32] = torch.from_numpy(scaled).to(Q_TORCH[fmt]).view(torch.uint8).numpy()
    return codes, scales


def q8_state(o, m, v):
    mc, ms = o.quantize(m, Q_E4M3)
    vc, vs = o.quantize(v, Q_E5M2)
    return mc, ms, vc, vs


def q8_step(o, w, state, g, c, t, copy=True, **hp):
    h = dict(lr=LR, beta1=B1, beta2=B2, eps=EPS, wd=WD)
    h.update(hp)
    w = w.copy()
    mc, ms, vc, vs = (a.copy() for a in state)
    p = np.zeros(w.size, np.uint16) if copy else None
    o.adamw8_step(w, mc, ms, vc, vs, g, p, c, t, h["lr"], h["beta1"], h["beta2"], h["eps"], h["wd"])
    return w, (mc, ms, vc, vs), p


def q8_blocks(n, seed):
    """Values spread over many magnitudes, ragged, with special blocks."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n) * 10.0 ** rng.integers(-40, 30, size=(n + 31) // 32).repeat(32)[:n]
    x = x.astype(np.float32)
    x[32:64] = 0.0                                  # all-zero block
    x[64:96] *= np.float32(1e-4)
    x[70] = np.float32(3.0)                         # one large value, the rest flush
    x[96:128] = (rng.standard_normal(32) * 1e-39).astype(np.float32)   # fp32 subnormals
    x[128] = -0.0
    x[160:192] = np.float32(448.0) * np.float32(2.0 ** -30)            # exactly on a boundary
    return x


def pin_q8_codes_decode_like_torch(o):
    for fmt in (Q_E4M3, Q_E5M2):
        ours = o.fp8_value(np.arange(256), fmt)
        ref = torch.arange(256, dtype=torch.uint8).view(Q_TORCH[fmt]).double().numpy()
        assert np.array_equal(np.isnan(ours), np.isnan(ref)), fmt
        keep = ~np.isnan(ref)
        assert np.array_equal(ours[keep], ref[keep]), fmt


def q8_probe_values() -> np.ndarray:
    """Every bf16-grid fp32 value, every code value and midpoint of both
    formats (and the overflow points), each with its fp32 neighbours."""
    grid = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    pts = [np.float32([464.0, 480.0, 61440.0, 65536.0, 2.0 ** -10, 2.0 ** -17])]
    for fmt in (Q_E4M3, Q_E5M2):
        v = torch.arange(128, dtype=torch.uint8).view(Q_TORCH[fmt]).double().numpy()
        v = np.unique(v[np.isfinite(v)])
        pts += [v.astype(np.float32), ((v[:-1] + v[1:]) / 2).astype(np.float32)]
    p = np.concatenate(pts)
    up = np.nextafter(p, np.float32(np.inf))
    down = np.nextafter(p, np.float32(-np.inf))
    p = np.concatenate([p, up, down])
    return np.concatenate([grid, p, -p, np.float32([np.inf, -np.inf, np.nan, -np.nan])])


def pin_q8_rounding_matches_torch(o):
    x = q8_probe_values()
    for fmt in (Q_E4M3, Q_E5M2):
        ours = o.fp8_round(x, fmt)
        ref = torch.from_numpy(x).to(Q_TORCH[fmt]).view(torch.uint8).numpy()
        bad = np.nonzero(ours != ref)[0]
        assert bad.size == 0, (fmt, [(float(x[i]), int(ours[i]), int(ref[i])) for i in bad[:5]])


def pin_q8_block_exponent(o):
    rng = np.random.default_rng(21)
    bits = rng.integers(0, 0x7F7FFFFF, size=4000, dtype=np.uint32)
    samples = [0.0] + [float(a) for a in bits.view(np.float32)]
    for fmt in (Q_E4M3, Q_E5M2):
        edges = []
        for k in range(-140, 122):
            if Q_LARGEST[fmt] * 2.0 ** k > 3.4e38:
                break
            b = np.float32(Q_LARGEST[fmt] * 2.0 ** k)
            if b > 0:
                edges += [float(b), float(np.nextafter(b, np.float32(np.inf))),
                          float(np.nextafter(b, np.float32(0)))]
        for a in samples + edges:
            e = o.block_exponent(a, fmt)
            assert e == q8_exponent_ref(a, fmt), (fmt, a, e)
            assert a <= math.ldexp(Q_LARGEST[fmt], e)
            assert e == -127 or a > math.ldexp(Q_LARGEST[fmt], e - 1)


def pin_q8_quantize_matches_reference(o):
    x = q8_blocks(32 * 41 + 13, 22)
    xn = x.copy()
    xn[200] = np.nan
    xn[260] = -np.inf
    for fmt in (Q_E4M3, Q_E5M2):
        for arr in (x, xn, x[:17], x[:0]):
            codes, scales = o.quantize(arr, fmt)
            rc, rs = q8_quantize_ref(arr, fmt)
            assert np.array_equal(scales, rs), fmt
            assert np.array_equal(codes, rc), fmt


def pin_q8_roundtrip_error_bound(o):
    x = q8_blocks(32 * 60 + 7, 23)
    for fmt in (Q_E4M3, Q_E5M2):
        codes, scales = o.quantize(x, fmt)
        y = o.dequantize(codes, scales, fmt)
        e = scales.astype(np.int64).repeat(32)[:x.size] - 127
        rel, sub = Q_HALF_STEP[fmt]
        bound = np.maximum(rel * np.abs(x.astype(np.float64)), sub * np.exp2(e.astype(np.float64)))
        assert_within(y, x, bound, f"round trip, format {fmt}")
        # The largest element of every block sits in the top binade: its code
        # is at least half the largest code, unless the exponent is clamped.
        for b in range(0, x.size, 32):
            blk = np.abs(x[b:b + 32])
            if blk.max() > 0 and scales[b // 32] > 0:
                top = np.abs(y[b:b + 32]).max() * 2.0 ** -(int(scales[b // 32]) - 127)
                assert Q_LARGEST[fmt] / 2 <= top <= Q_LARGEST[fmt], (fmt, b)
    # Values already on a block's grid come back exactly.
    rng = np.random.default_rng(24)
    for fmt in (Q_E4M3, Q_E5M2):
        codes = rng.integers(0, 0x78 if fmt == Q_E5M2 else 0x7E, size=320).astype(np.uint8)
        codes |= rng.integers(0, 2, size=320).astype(np.uint8) << 7
        codes[::32] = 0x7E if fmt == Q_E4M3 else 0x7B            # the block maximum
        scales = rng.integers(1, 200, size=10).astype(np.uint8)
        x = o.dequantize(codes, scales, fmt)
        c2, s2 = o.quantize(x, fmt)
        assert np.array_equal(s2, scales) and np.array_equal(o.dequantize(c2, s2, fmt), x)


def pin_q8_step_is_fp32_step_on_decoded_state(o):
    n = 32 * 9 + 5
    w, m, v, g = rand_state(n, 25, warm=True)
    g[::17] *= np.float32(100.0)
    state = q8_state(o, m, v)
    m_dec = o.dequantize(state[0], state[1], Q_E4M3)
    v_dec = o.dequantize(state[2], state[3], Q_E5M2)
    for grad in (g, o.f32_to_bf16(g)):
        for c, t in ((np.float32(0.37), 7), (np.float32(1.0), 1)):
            w8, (mc, ms, vc, vs), p8 = q8_step(o, w, state, grad, c, t)
            w32, m32, v32, p32 = run_step(o, w, m_dec, v_dec, grad, c, t, copy=True)
            assert np.array_equal(w8.view(np.uint32), w32.view(np.uint32))
            assert np.array_equal(p8, p32)
            rc, rs = q8_quantize_ref(m32, Q_E4M3)
            assert np.array_equal(mc, rc) and np.array_equal(ms, rs)
            rc, rs = q8_quantize_ref(v32, Q_E5M2)
            assert np.array_equal(vc, rc) and np.array_equal(vs, rs)


def pin_q8_zero_state_zero_gradient(o):
    w, _, _, _ = rand_state(100, 26, warm=False)
    zeros = np.zeros(100, np.float32)
    state = (np.zeros(100, np.uint8), np.zeros(4, np.uint8), np.zeros(100, np.uint8),
             np.zeros(4, np.uint8))
    w1, st1, _ = q8_step(o, w, state, zeros, np.float32(1.0), 1)
    decay = round_f32(1 - dec("3e-4") * dec("0.1"))
    assert np.array_equal(w1.view(np.uint32), (w * decay).view(np.uint32))
    for a in st1:
        assert not a.any()


def pin_q8_first_step_closed_form(o):
    """From zero state the master follows the fp32 closed form and the stored
    moments are (1 - b1) g and (1 - b2) g^2 within half a code step."""
    w, _, _, g = rand_state(32 * 20, 27, warm=False)
    state = (np.zeros(w.size, np.uint8), np.zeros(20, np.uint8)) * 2
    c = np.float32(0.5)
    w1, (mc, ms, vc, vs), _ = q8_step(o, w, state, g, c, 1)
    gc = g.astype(np.float64) * float(c)
    want = w.astype(np.float64) * (1 - LR * WD) - LR * gc / (np.abs(gc) + EPS)
    assert_within(w1, want, 8 * U32 * (np.abs(w) + LR) + 1e-12, "first-step w (8-bit)")
    for codes, scales, fmt, exact in ((mc, ms, Q_E4M3, (1 - B1) * gc),
                                      (vc, vs, Q_E5M2, (1 - B2) * gc * gc)):
        y = o.dequantize(codes, scales, fmt)
        e = scales.astype(np.float64).repeat(32) - 127
        rel, sub = Q_HALF_STEP[fmt]
        bound = (rel * np.abs(exact) + sub * np.exp2(e)) * (1 + 1e-6) + 4 * U32 * np.abs(exact)
        assert_within(y, exact, bound, f"stored moment, format {fmt}")


def pin_q8_nonfinite_block(o):
    """A NaN gradient poisons its own block of 32 (stored as NaN), nothing else."""
    w, m, v, g = rand_state(96, 28, warm=True)
    state = q8_state(o, m, v)
    g[40] = np.nan
    w1, st1, _ = q8_step(o, w, state, g, np.float32(1.0), 2)
    assert np.isnan(w1[40]) and np.isfinite(np.delete(w1, 40)).all()
    for codes, scales in ((st1[0], st1[1]), (st1[2], st1[3])):
        assert scales[1] == 255 and (codes[32:64] == 255).all()
        assert scales[0] != 255 and scales[2] != 255
    g[40] = 0.0
    w2, st2, _ = q8_step(o, w1, st1, g, np.float32(1.0), 3)
    assert np.isnan(w2[32:64]).all()
    assert np.isfinite(w2[:32]).all() and np.isfinite(w2[64:]).all()


def pin_q8_list_equals_flat_on_block_multiples(o):
    w, m, v, g = rand_state(32 * 30, 29, warm=True)
    state = q8_state(o, m, v)
    whole = q8_step(o, w, state, g, np.float32(0.8), 4)
    cut = 32 * 11
    parts = []
    for lo, hi in ((0, cut), (cut, w.size)):
        sub = (state[0][lo:hi], state[1][lo // 32:hi // 32], state[2][lo:hi], state[3][lo // 32:hi // 32])
        parts.append(q8_step(o, w[lo:hi], tuple(np.ascontiguousarray(a) for a in sub), g[lo:hi],
                             np.float32(0.8), 4))
    assert np.array_equal(whole[0], np.concatenate([parts[0][0], parts[1][0]]))
    for k in range(4):
        assert np.array_equal(whole[1][k], np.concatenate([parts[0][1][k], parts[1][1][k]]))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
