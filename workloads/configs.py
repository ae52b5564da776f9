"""The five synthetic workloads of the shard step, as plain data.

Each workload is one FSDP unit (or a set of DDP buckets) seen from one
rank: the tensor shapes that make up the FlatParameter, the number of
data-parallel ranks N_d, the number of accumulated micro-batches, the
ranks whose shard is computed, the value distributions and the AdamW
hyperparameters.

Sources of the shapes:
* three (4, 2) weights split over two ranks -- the FSDP1 figure of
  "Infra: Data Parallel" (section "FSDP1: pack first, then split");
* one Transformer block as an FSDP unit -- "Infra: Data Parallel",
  FSDP1 section, and "PyTorch FSDP ..." summary, section 3.1;
* DDP buckets of about 25 MB -- "4.1 数据并行详解", section 4.2 (bucket
  mechanism); the 611M model size is the T5-611M of the FSDP summary,
  section 4.1;
* the GPT-175B-shaped layer (d=12288, ffn=49152) and the 10k ragged
  tensors are synthetic stand-ins with the sizes the workload list fixes.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class AdamW:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    world: int                      # N_d, simulated data-parallel ranks
    n_micro: int                    # accumulated micro-batches per step
    ranks: Tuple[int, ...]          # ranks whose shard is computed
    grad_sigma: float               # per-rank bf16 gradient ~ N(0, grad_sigma)
    master_sigma: float             # fp32 master weights ~ N(0, master_sigma)
    shapes: Optional[Tuple[Tuple[int, ...], ...]] = None   # one FlatParameter
    names: Optional[Tuple[str, ...]] = None
    bucket_elems: Optional[int] = None   # DDP bucket size in elements
    total_elems: Optional[int] = None    # flat model size when bucketed
    inf_fraction: float = 0.0            # share of gradient elements set to +inf
    seed: int = 0
    hp: AdamW = AdamW()

    # ---- geometry helpers (pure integer bookkeeping of the workload) ----
    def units(self) -> List[int]:
        """Element count T of every unit (FlatParameter or bucket)."""
        if self.shapes is not None:
            return [sum(math.prod(s) for s in self.shapes)]
        n_full = self.total_elems // self.bucket_elems
        sizes = [self.bucket_elems] * n_full
        tail = self.total_elems - n_full * self.bucket_elems
        if tail:
            sizes.append(tail)
        return sizes


def transformer_unit_shapes(d: int, ffn: int):
    """One Transformer block as an FSDP unit, in registration order.

    Order: qkv weight/bias, attention output weight/bias, the two MLP
    weights/biases, then the two LayerNorm weight/bias pairs.  Weights are
    (out_features, in_features) as nn.Linear stores them.
    """
    names = ("qkv.weight", "qkv.bias", "out.weight", "out.bias",
             "ff1.weight", "ff1.bias", "ff2.weight", "ff2.bias",
             "ln1.weight", "ln1.bias", "ln2.weight", "ln2.bias")
    shapes = ((3 * d, d), (3 * d,), (d, d), (d,),
              (ffn, d), (ffn,), (d, ffn), (d,),
              (d,), (d,), (d,), (d,))
    return names, shapes


def c5_tensor_sizes(n_tensors: int = 10_000, max_elems: int = 4_194_304,
                    seed: int = 0) -> np.ndarray:
    """Ragged 1-D tensor sizes, log-uniform on [1, max_elems].

    n_i = max(1, floor(exp(u_i * ln(max_elems)))) with u_i uniform on [0, 1)
    drawn from numpy's PCG64 with the given seed.  With the default
    arguments the total is 2,728,745,331 elements.
    """
    u = np.random.default_rng(seed).random(n_tensors)
    return np.maximum(1, np.floor(np.exp(u * math.log(max_elems)))).astype(np.int64)


_C2_NAMES, _C2_SHAPES = transformer_unit_shapes(1024, 4096)
_C4_NAMES, _C4_SHAPES = transformer_unit_shapes(12288, 49152)

CONFIGS = {
    # three fp32 (4,2) weights, two ranks, one AdamW step
    "c1_three_4x2_nd2": Config(
        name="c1_three_4x2_nd2", world=2, n_micro=1, ranks=(0, 1),
        grad_sigma=1.0, master_sigma=1.0,
        shapes=((4, 2), (4, 2), (4, 2)), names=("W1", "W2", "W3")),
    # one Transformer layer unit d=1024, ffn=4096, eight ranks
    "c2_layer_d1024_nd8": Config(
        name="c2_layer_d1024_nd8", world=8, n_micro=1, ranks=(1, 7, 0),
        grad_sigma=1e-3, master_sigma=0.02,
        shapes=_C2_SHAPES, names=_C2_NAMES),
    # 611M flat model in 25 MiB bf16 buckets, 16 ranks, 4 micro-batches
    "c3_611m_buckets_nd16": Config(
        name="c3_611m_buckets_nd16", world=16, n_micro=4, ranks=(0,),
        grad_sigma=1e-3, master_sigma=0.02,
        bucket_elems=25 * 1024 * 1024 // 2, total_elems=611_000_000),
    # GPT-175B-shaped layer unit d=12288, ffn=49152, eight ranks
    "c4_layer_d12288_nd8": Config(
        name="c4_layer_d12288_nd8", world=8, n_micro=1, ranks=(0,),
        grad_sigma=1e-3, master_sigma=0.02,
        shapes=_C4_SHAPES, names=_C4_NAMES),
    # 10k ragged tensors, 64 ranks, 0.01% injected +inf in the gradients
    "c5_ragged10k_nd64": Config(
        name="c5_ragged10k_nd64", world=64, n_micro=1, ranks=(0, 63),
        grad_sigma=1e-3, master_sigma=0.02,
        shapes=tuple((int(n),) for n in c5_tensor_sizes()),
        inf_fraction=1e-4),
}
