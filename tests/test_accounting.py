"""The workloads' byte accounting against the pages' 16N figures.

tests/golden/state_accounting_7b.json holds the numbers the Lecture 9
exercises page prints for a 7B model (16N = 112 GB either way, itemized
14/14/28/28/28 for mixed precision; 10N = 70 GB with 8-bit moments; 14 GB
per card when all of it is sharded 8 ways).  The per-parameter state bytes
the workloads use must reproduce them, and the harness must allocate exactly
that much.
"""
import json
import os

import torch

from mixed_precision_sharded_amd import synth
from mixed_precision_sharded_amd.configs import WORKLOADS, Workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "state_accounting_7b.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_state_bytes_reproduce_the_16n_table():
    g = _golden()
    N = g["N"]
    mixed = WORKLOADS[1]      # bf16 gradients + bf16 copy: the mixed basis
    pure = WORKLOADS[2]       # fp32 gradients, no copy: the pure-fp32 basis
    assert mixed.state_bytes_per_param() * N / 1e9 == g["mixed_adam"]["total"]
    assert pure.state_bytes_per_param() * N / 1e9 == g["fp32_adam"]["total"]
    # itemized: 2 (bf16 copy) + 2 (bf16 grad) + 4 + 4 (m, v) + 4 (master)
    items = {"params": 2, "grads": 2, "m": 4, "v": 4, "master": 4}
    assert {k: b * N / 1e9 for k, b in items.items()} == {
        k: g["mixed_adam"][k] for k in items}
    assert (4 + 4 + 4) * N / 1e9 / g["mixed_adam"]["total"] == g["optimizer_related_fraction"]
    # 8-bit moments: m and v shrink from 8 to 2 bytes per parameter
    eight = (mixed.state_bytes_per_param() - 8 + 2) * N / 1e9
    assert eight == g["mixed_adam_8bit_moments"]["total"]
    assert 1 - eight / g["mixed_adam"]["total"] == g["mixed_adam_8bit_moments"]["saving_fraction"]
    assert mixed.state_bytes_per_param() * N / 8 / 1e9 == g["zero3_k8_per_card_total"]


def test_every_workload_keeps_16_bytes_of_state_per_param():
    for w in WORKLOADS.values():
        assert w.state_bytes_per_param() == 16, w.name


def test_algorithmic_bytes_per_param():
    # the norm reads the gradient once more than the update does
    assert WORKLOADS[1].algorithmic_bytes_per_param() == 30
    assert WORKLOADS[2].algorithmic_bytes_per_param() == 32
    for w in WORKLOADS.values():
        g = 2 if w.grad_bf16 else 4
        assert w.algorithmic_bytes_per_param() == w.update_bytes_per_param() + g


def test_workload_sizes():
    sizes = {k: (w.n_tensors, w.numel) for k, w in WORKLOADS.items()}
    assert sizes == {1: (1, 1 << 20), 2: (1, 62_736_416), 3: (291, 8_030_261_248),
                     4: (723, 276_254_720), 5: (1137, 792_682_400)}


def test_harness_allocates_exactly_the_state():
    w = Workload(cfg=1, name="tiny", tensors=(("a", 1000), ("b", 24)), grad_bf16=True,
                 copy_bf16=True, step=1)
    ins = synth.workload_inputs(w, "cpu")
    nbytes = sum(t.numel() * t.element_size() for col in ins.values() for t in col
                 if t is not None)
    assert nbytes == w.state_bytes_per_param() * w.numel


def test_inputs_are_seeded_per_tensor():
    w = WORKLOADS[4]
    a = synth.tensor_inputs(w, 3, "cpu")
    b = synth.tensor_inputs(w, 3, "cpu")
    for k in a:
        assert torch.equal(a[k], b[k])
    c = synth.tensor_inputs(w, 4, "cpu")
    assert not torch.equal(a["master"], c["master"])


def test_8bit_state_reproduces_the_10n_row():
    """The 8-bit moment layout (codes + one scale byte per 32 elements) on the
    mixed basis lands on the page's 10N = 70 GB for 7B, up to the scale
    bytes (0.0625 B per parameter, under 1 %)."""
    g = _golden()
    N = g["N"]
    mixed = WORKLOADS[1]
    total = mixed.state8_bytes_per_param() * N / 1e9
    assert abs(total - g["mixed_adam_8bit_moments"]["total"]) / total < 0.01
    # the codes alone are exactly the page's 2N for the optimizer state
    assert (mixed.state8_bytes_per_param() - 2 / 32 - 8) * N / 1e9 == 2 * N / 1e9


def test_8bit_update_bytes():
    # bf16 gradient + copy: 2 + 4 + 4 + (1 + 1) * 2 + 2 * 2/32 + 2 = 16.125
    assert WORKLOADS[1].update8_bytes_per_param() == 16.125
    assert WORKLOADS[2].update8_bytes_per_param() == 16.125   # fp32 gradient, no copy
    assert WORKLOADS[2].algorithmic8_bytes_per_param() == 20.125
