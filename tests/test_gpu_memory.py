"""Device memory of a step on the GPU: the resident state of a workload is
exactly its accounted bytes (16 per parameter; 10.0625 with 8-bit moments
plus gradient and copy), the workspace grows with tensors and chunks only,
and stepping allocates nothing — neither through PyTorch's allocator nor
below it (the device's free memory does not move)."""
import pytest
import torch

from gpu_harness import say
from mixed_precision_sharded_amd import binding, synth
from mixed_precision_sharded_amd.configs import WORKLOADS

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def tensor_bytes(cols):
    return sum(t.numel() * t.element_size() for col in cols.values() for t in col
               if t is not None)


@pytest.mark.parametrize("cfg", [2, 5])
def test_state_is_the_accounted_bytes_and_steps_allocate_nothing(cfg):
    w = WORKLOADS[cfg]
    say(f"memory: {w.name}")
    cols = synth.workload_inputs(w, "cuda")
    assert tensor_bytes(cols) == w.numel * w.state_bytes_per_param()
    tl = binding.TensorList(cols["master"], cols["exp_avg"], cols["exp_avg_sq"], cols["grad"],
                            cols["param_bf16"])
    # The workspace: tables for the tensors and chunks, nothing per element.
    assert tl.workspace_bytes < 64 * w.n_tensors + 4 * (w.numel // 2048 + w.n_tensors) + (1 << 16)
    S = torch.zeros(1, dtype=torch.float64, device="cuda")
    c = torch.zeros(1, dtype=torch.float32, device="cuda")
    step = torch.zeros(1, dtype=torch.int32, device="cuda")
    hp = (w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)

    def steps(k):
        for _ in range(k):
            binding.adamw_clipped_step(tl, step, *hp, w.max_norm, sumsq_out=S, coef_out=c)
            binding.grad_norm_sq(tl, S, w.max_norm, c)
            binding.adamw_multi_tensor_step(tl, c, step, *hp)
        torch.cuda.synchronize()

    steps(1)  # the tables' upload and the runtime's first-launch setup
    allocated = torch.cuda.memory_allocated()
    free, _ = torch.cuda.mem_get_info()
    steps(5)
    assert torch.cuda.memory_allocated() == allocated
    free_after, _ = torch.cuda.mem_get_info()
    assert abs(free_after - free) <= (4 << 20), (free, free_after)
    assert int(step.item()) == 12
    tl.release()


def test_8bit_state_is_the_accounted_bytes():
    w = WORKLOADS[2]
    cols = synth.workload_inputs(w, "cuda")
    states = [binding.zeros_q8_state(m.numel(), "cuda") for m in cols["exp_avg"]]
    del cols["exp_avg"], cols["exp_avg_sq"]
    state8 = sum(x.numel() * x.element_size() for st in states for x in st)
    total = tensor_bytes(cols) + state8
    assert total == pytest.approx(w.numel * w.state8_bytes_per_param(), abs=2 * w.n_tensors)
    tl = binding.TensorList8(cols["master"], states, cols["grad"], cols["param_bf16"])
    step = torch.zeros(1, dtype=torch.int32, device="cuda")
    binding.adamw8_clipped_step(tl, step, w.lr, w.beta1, w.beta2, w.eps, w.weight_decay,
                                w.max_norm)
    torch.cuda.synchronize()
    allocated = torch.cuda.memory_allocated()
    for _ in range(3):
        binding.adamw8_clipped_step(tl, step, w.lr, w.beta1, w.beta2, w.eps, w.weight_decay,
                                    w.max_norm)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == allocated
    tl.release()
