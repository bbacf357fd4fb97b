"""The five synthetic shard workloads: tensor lists, dtypes, hyperparameters
and value distributions.  Pure data, no optimizer arithmetic.

Shapes are one GPU's share of the Llama 3.1 models the TorchTitan digest
reports on ("TorchTitan: a one-stop PyTorch-native solution for production
LLM pre-training", section 1: 8B on 128 GPUs with 1D FSDP, 70B on 256 GPUs
with 2D FSDP x TP, 405B on 512 GPUs with 3D); the tensor order follows the
decoder layout of the TorchTitan composability article (embedding, the
layers in order, final norm, output head).  Precision bases follow the
Lecture 9 exercises page's 16N table: bf16 gradients with a bf16 parameter
copy (mixed basis) or fp32 gradients without a copy (pure-fp32 basis).
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple


@dataclass(frozen=True)
class Workload:
    cfg: int                       # 1..5
    name: str
    tensors: Tuple[Tuple[str, int], ...]  # (name, numel) in list order
    grad_bf16: bool                # bf16 gradients (else fp32)
    copy_bf16: bool                # write a bf16 parameter copy
    step: int                      # t of the step under test (completed = t - 1)
    lr: float = 3e-4
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    max_norm: float = 1.0
    master_std: float = 0.02
    grad_std: float = 1e-3
    m_std: Optional[float] = None  # None: m starts at zero
    v_std: Optional[float] = None  # None: v starts at zero; else |N(0, v_std)|
    outlier_frac: float = 0.0      # fraction of gradient entries scaled ...
    outlier_scale: float = 1.0     # ... by this factor
    note: str = field(default="", compare=False)

    @property
    def numel(self) -> int:
        return sum(n for _, n in self.tensors)

    @property
    def n_tensors(self) -> int:
        return len(self.tensors)

    def algorithmic_bytes_per_param(self) -> int:
        """HBM bytes one step must move per parameter: the norm reads the
        gradient once; the update reads master, m, v and the gradient and
        writes master, m, v and the optional bf16 copy."""
        g = 2 if self.grad_bf16 else 4
        return g + (12 + g) + 12 + (2 if self.copy_bf16 else 0)

    def update_bytes_per_param(self) -> int:
        """The update kernel's share of algorithmic_bytes_per_param."""
        g = 2 if self.grad_bf16 else 4
        return 12 + g + 12 + (2 if self.copy_bf16 else 0)

    # With 8-bit moments (one code byte each for m and v, one scale byte per
    # 32 elements for each) the update moves master 4 + codes 2 + scales
    # 2/32 bytes each way instead of 12.
    def update8_bytes_per_param(self) -> float:
        g = 2 if self.grad_bf16 else 4
        return g + 2 * (4 + 2 + 2 / 32) + (2 if self.copy_bf16 else 0)

    def algorithmic8_bytes_per_param(self) -> float:
        return (2 if self.grad_bf16 else 4) + self.update8_bytes_per_param()

    def state8_bytes_per_param(self) -> float:
        """Resident state with 8-bit moments: the 10N row of the accounting
        (plus the scale bytes) on the mixed basis."""
        g = 2 if self.grad_bf16 else 4
        return 4 + 2 + 2 / 32 + g + (2 if self.copy_bf16 else 0)

    def state_bytes_per_param(self) -> int:
        """Resident state per parameter under the 16N accounting: fp32
        master, m and v (12 B) plus the gradient and the parameter copy.
        With fp32 gradients and no bf16 copy (the pure-fp32 basis) the
        master is the parameter itself."""
        g = 2 if self.grad_bf16 else 4
        return 12 + g + (2 if self.copy_bf16 else 0)


def _llama(dim: int, kv_dim: int, ffn: int, vocab: int, n_layers: int, div: int,
           norm_numel: int) -> Tuple[Tuple[str, int], ...]:
    """Tensor list of a Llama decoder, every matrix divided by `div`."""
    def mat(rows, cols):
        assert (rows * cols) % div == 0
        return rows * cols // div
    out: List[Tuple[str, int]] = [("tok_embeddings", mat(vocab, dim))]
    for i in range(n_layers):
        p = f"layers.{i}."
        out += [(p + "attention.wq", mat(dim, dim)), (p + "attention.wk", mat(kv_dim, dim)),
                (p + "attention.wv", mat(kv_dim, dim)), (p + "attention.wo", mat(dim, dim)),
                (p + "feed_forward.w1", mat(ffn, dim)), (p + "feed_forward.w2", mat(dim, ffn)),
                (p + "feed_forward.w3", mat(ffn, dim)), (p + "attention_norm", norm_numel),
                (p + "ffn_norm", norm_numel)]
    out += [("norm", norm_numel), ("output", mat(vocab, dim))]
    return tuple(out)


LLAMA_8B_NUMEL = 8_030_261_248

WORKLOADS = {
    1: Workload(
        cfg=1, name="flat_1m_bf16", tensors=(("flat", 1 << 20),), grad_bf16=True,
        copy_bf16=True, step=1,
        note="single flat fp32 shard of 2^20 params, bf16 grads, bf16 copy out"),
    2: Workload(
        cfg=2, name="llama8b_fsdp128_shard", tensors=(("flat", LLAMA_8B_NUMEL // 128),),
        grad_bf16=False, copy_bf16=False, step=100, m_std=1e-4, v_std=1e-8,
        outlier_frac=1e-3, outlier_scale=100.0,
        note="one GPU's FSDP2 shard of Llama-3.1-8B at 128-way: 62.7M fp32 params, "
             "fp32 grads with 0.1% outliers x100, warm m/v, step 100"),
    3: Workload(
        cfg=3, name="llama8b_full_list",
        tensors=_llama(4096, 1024, 14336, 128256, 32, 1, 4096), grad_bf16=True,
        copy_bf16=True, step=1,
        note="full Llama-3.1-8B as a 291-tensor list, bf16 grads, bf16 copy out"),
    4: Workload(
        cfg=4, name="llama70b_tp8_fsdp32_share",
        tensors=_llama(8192, 1024, 28672, 128256, 80, 256, 4096), grad_bf16=False,
        copy_bf16=False, step=1, lr=1.5e-4, grad_std=5e-4,
        note="one GPU's share of Llama-70B under TP8 x FSDP32: 723 tensors, 276M params"),
    5: Workload(
        cfg=5, name="llama405b_512way_share",
        tensors=_llama(16384, 1024, 53248, 128256, 126, 512, 32), grad_bf16=True,
        copy_bf16=True, step=1000, grad_std=2e-4,
        note="one GPU's share of Llama-405B at 512-way: 1137 tensors, 792.7M params, "
             "bf16 grads, bf16 copy out, step 1000"),
}


def warm(w: Workload) -> Workload:
    """The same workload with m and v warmed as in the 8B shard workload."""
    from dataclasses import replace
    return replace(w, m_std=1e-4, v_std=1e-8, name=w.name + "_warm")
