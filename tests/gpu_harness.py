"""Helpers shared by the GPU tests: run the three-call step through the C ABI
(via the binding) and compare with the oracle on the same seeded inputs."""
import sys

import numpy as np
import torch

import oracle
from mixed_precision_sharded_amd import binding
from mixed_precision_sharded_amd.synth import to_numpy

REL_TOL = 2e-6       # master, m, v: relative error per element
NORM_REL_TOL = 1e-5  # sum of squares
BF16_ULP_TOL = 1     # bf16 copy


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Step:
    """Device buffers of one list plus the scalars of one call sequence."""

    def __init__(self, cols, completed_steps=0):
        self.cols = cols
        dev = cols["master"][0].device
        self.tl = binding.TensorList(cols["master"], cols["exp_avg"], cols["exp_avg_sq"],
                                     cols["grad"], cols["param_bf16"])
        self.sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
        self.coef = torch.zeros(1, dtype=torch.float32, device=dev)
        self.step = torch.tensor([completed_steps], dtype=torch.int32, device=dev)

    def norm(self):
        binding.grad_norm_sq(self.tl, self.sumsq)
        return self

    def norm_clip(self, max_norm, grad_scale=1.0):
        """Norm and clip coefficient from one launch."""
        binding.grad_norm_sq(self.tl, self.sumsq, max_norm, self.coef, grad_scale=grad_scale)
        return self

    def clip(self, max_norm, grad_scale=1.0):
        binding.clip_coef(self.sumsq, max_norm, self.coef, grad_scale=grad_scale)
        return self

    def update(self, lr, beta1, beta2, eps, wd, use_coef=True, skip_if_nonfinite=False):
        binding.adamw_multi_tensor_step(self.tl, self.coef if use_coef else None, self.step, lr,
                                        beta1, beta2, eps, wd,
                                        skip_if_nonfinite=self.sumsq if skip_if_nonfinite else None)
        return self

    def fused(self, max_norm, lr, beta1, beta2, eps, wd, grad_scale=1.0, skip_if_nonfinite=False):
        """Norm, clip and update in one launch (adamw_fused_step)."""
        binding.adamw_fused_step(self.tl, self.step, lr, beta1, beta2, eps, wd, max_norm,
                                 grad_scale=grad_scale, skip_if_nonfinite=skip_if_nonfinite,
                                 sumsq_out=self.sumsq, coef_out=self.coef)
        return self

    def clipped(self, max_norm, lr, beta1, beta2, eps, wd, grad_scale=1.0,
                skip_if_nonfinite=False):
        """Norm, clip and update in two launches, the clip finished inside the
        update (adamw_clipped_step)."""
        binding.adamw_clipped_step(self.tl, self.step, lr, beta1, beta2, eps, wd, max_norm,
                                   grad_scale=grad_scale, skip_if_nonfinite=skip_if_nonfinite,
                                   sumsq_out=self.sumsq, coef_out=self.coef)
        return self

    def header_words(self):
        """The workspace header as 64-bit words (for the barrier counters)."""
        torch.cuda.synchronize()
        ws = self.tl._ws_storage
        off = self.tl.workspace_ptr - ws.data_ptr()
        return ws[off:off + 64].cpu().view(torch.int64).tolist()

    def full(self, w):
        """norm + clip (one launch) -> update with a workload's hyperparameters."""
        return self.norm_clip(w.max_norm).update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)

    def results(self):
        torch.cuda.synchronize()
        return float(self.sumsq.item()), np.float32(self.coef.item()), int(self.step.item())


def host_copy(cols):
    return {k: [None if t is None else to_numpy(t).copy() for t in v] for k, v in cols.items()}


def oracle_step(host, c, t, lr, beta1, beta2, eps, wd):
    """The oracle's step on host copies (in place)."""
    o = oracle.default()
    for i in range(len(host["master"])):
        o.adamw_step(host["master"][i], host["exp_avg"][i], host["exp_avg_sq"][i],
                     host["grad"][i], host["param_bf16"][i], c, t, lr, beta1, beta2, eps, wd)
    return host


def oracle_norm(grads_host):
    return oracle.default().grad_norm_sq(grads_host)


def check_f32(got, want, what, rel=REL_TOL):
    """Per-element relative error <= rel (exact where the reference is 0);
    NaN must match NaN.  Returns (elements not bitwise equal, worst rel)."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape, what
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    wi = np.isinf(want)
    assert np.array_equal(got[wi], want[wi]) and not np.isinf(got[~wi & ~wn]).any(), \
        f"{what}: infinities differ"
    ok = ~wn & ~wi
    g64, w64 = got[ok].astype(np.float64), want[ok].astype(np.float64)
    diff = np.abs(g64 - w64)
    zero = w64 == 0
    assert not (diff[zero] > 0).any(), f"{what}: nonzero where the oracle gives 0"
    relerr = np.zeros_like(diff)
    relerr[~zero] = diff[~zero] / np.abs(w64[~zero])
    worst = float(relerr.max()) if relerr.size else 0.0
    bad = int((relerr > rel).sum())
    assert bad == 0, f"{what}: {bad} elements beyond rel {rel}; worst {worst:.3e}"
    nbit = int((got[ok].view(np.uint32) != want[ok].view(np.uint32)).sum())
    return nbit, worst


def check_f32_bitwise_first(got, want, what, rel=REL_TOL, piece=1 << 26):
    """check_f32 for very long arrays: elements that are bitwise equal meet
    every condition of check_f32 (zero error, NaN for NaN, the same infinity),
    so only the others go through it; in pieces, to bound the temporaries."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape, what
    nbit, worst = 0, 0.0
    for lo in range(0, got.size, piece):
        g, w = got[lo:lo + piece], want[lo:lo + piece]
        neq = g.view(np.uint32) != w.view(np.uint32)
        if neq.any():
            nb, wr = check_f32(g[neq], w[neq], f"{what} [{lo}:]", rel)
            nbit += nb
            worst = max(worst, wr)
    return nbit, worst


def check_bf16_bitwise_first(got, want, what, ulps=BF16_ULP_TOL, piece=1 << 26):
    """check_bf16 for very long arrays, bitwise-equal elements skipped."""
    got = np.asarray(got, np.uint16)
    want = np.asarray(want, np.uint16)
    assert got.shape == want.shape, what
    nbit, worst = 0, 0
    for lo in range(0, got.size, piece):
        g, w = got[lo:lo + piece], want[lo:lo + piece]
        neq = g != w
        if neq.any():
            nb, wr = check_bf16(g[neq], w[neq], f"{what} [{lo}:]", ulps)
            nbit += nb
            worst = max(worst, wr)
    return nbit, worst


def oracle_step_threads(w, m, v, g, p, c, t, lr, beta1, beta2, eps, wd, threads=16):
    """The oracle's step on host arrays (in place), each array cut into
    `threads` contiguous slices stepped by one thread each: the oracle's
    arithmetic is per element, so slicing changes nothing in the results
    (its C code runs outside the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor

    o = oracle.default()
    n = w.size
    cuts = [n * k // threads for k in range(threads)] + [n]

    def one(k):
        lo, hi = cuts[k], cuts[k + 1]
        if hi > lo:
            o.adamw_step(w[lo:hi], m[lo:hi], v[lo:hi], g[lo:hi], None if p is None else p[lo:hi],
                         c, t, lr, beta1, beta2, eps, wd)

    with ThreadPoolExecutor(max_workers=threads) as pool:
        list(pool.map(one, range(threads)))


def bf16_order(bits):
    """Map bf16 bit patterns to integers ordered like their values."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7fff), b)


def check_bf16(got, want, what, ulps=BF16_ULP_TOL):
    got = np.asarray(got, np.uint16)
    want = np.asarray(want, np.uint16)
    gn = (got & 0x7fff) > 0x7f80
    wn = (want & 0x7fff) > 0x7f80
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    d = np.abs(bf16_order(got[~gn]) - bf16_order(want[~wn]))
    worst = int(d.max()) if d.size else 0
    assert worst <= ulps, f"{what}: {int((d > ulps).sum())} copies beyond {ulps} ulp"
    return int((d != 0).sum()), worst


def compare_state(cols, host, what=""):
    """Device state (after the step) against host oracle results, per tensor."""
    stats = {"w": [0, 0.0], "m": [0, 0.0], "v": [0, 0.0], "p": [0, 0]}
    for i in range(len(host["master"])):
        for key, dev_key in (("w", "master"), ("m", "exp_avg"), ("v", "exp_avg_sq")):
            nb, worst = check_f32(to_numpy(cols[dev_key][i]), host[dev_key][i],
                                  f"{what} tensor {i} {dev_key}")
            stats[key][0] += nb
            stats[key][1] = max(stats[key][1], worst)
        if host["param_bf16"][i] is not None:
            nb, worst = check_bf16(to_numpy(cols["param_bf16"][i]), host["param_bf16"][i],
                                   f"{what} tensor {i} param_bf16")
            stats["p"][0] += nb
            stats["p"][1] = max(stats["p"][1], worst)
    return stats


def sample_indices(n, k, gen):
    """k random indices of [0, n) plus the first and last 8 and the elements
    around every multiple of 2048 up to 64 Ki (chunk edges)."""
    fixed = list(range(min(n, 8))) + list(range(max(0, n - 8), n))
    for q in range(2048, min(n, 65536) + 1, 2048):
        fixed += [q - 1, q] if q < n else [q - 1]
    rnd = torch.randint(0, n, (min(k, n),), generator=gen).tolist() if n else []
    return sorted(set(i for i in fixed + rnd if 0 <= i < n))


def crafted_bf16_masters(rng, n_random=4000):
    """fp32 values at the corners of bf16 rounding: exact ties below odd and
    even kept halves, one unit either side of a tie, fp32 subnormals (also at
    ties), the largest finite values (which round up to infinity), signed
    zeros, infinities and NaNs."""
    hi = rng.integers(0, 1 << 16, size=n_random, dtype=np.uint32) << 16
    lows = np.array([0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    sub = rng.integers(1, 0x00800000, size=500, dtype=np.uint32)
    sub_ties = (rng.integers(0, 0x80, size=500, dtype=np.uint32) << 16) | 0x8000
    special = np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0xFF7FFFFF, 0x00000000, 0x80000000,
                        0x7F800000, 0xFF800000, 0x7FC00001, 0xFFA00000, 0x00008000, 0x80018000],
                       dtype=np.uint32)
    bits = np.concatenate([bits, sub, sub | 0x80000000, sub_ties, special])
    # keep the exponent field away from all-ones except for the specials
    body = bits[:-special.size]
    body = np.where((body & 0x7F800000) == 0x7F800000, body & 0xBFFFFFFF, body)
    return np.concatenate([body, special]).view(np.float32)
