"""Seeded synthetic workloads for the TIDE placement collectives.

This module holds only parameter shapes and random draws.  It holds none of
the method's arithmetic (no shard geometry, no sums), so both the HIP path
and the CPU oracle can be fed from it without sharing any of the method.

The workloads take architecture shapes from the models the TIDE article
trains ("FSDP通信终局：TIDE零拷贝集合通信优化", §"FSDP2通信开销的根源" and
§"性能表现：步时降低与干扰削减": Llama-3.1 70B at 8K tokens per GPU,
Qwen3-30B-A3B).  No dataset or trained weight is involved: gradients are
fp32 normal draws scaled by sigma and rounded to bf16 (round-to-nearest-even).

Seeds: rank r draws from seed ``base + r`` (base 0), one generator per rank,
parameters in list order.  The tiny workload draws on the CPU so that it can
be reproduced without a GPU; the large ones draw on the device because the
biggest (64 ranks of a 70B layer, ~110 GB) cannot pass through host memory.
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import torch

Shape = Tuple[int, ...]


@dataclass(frozen=True)
class Workload:
    name: str
    params: List[Tuple[str, Shape]]
    world: int
    sigma: float
    rank: Optional[int] = None          # the rank a single-rank run uses
    zero_expert_frac: float = 0.0       # fraction of experts with all-zero grads
    n_experts: int = 0
    corun_gemm: Optional[Tuple[int, int, int]] = None
    grad_seed_base: int = 0
    description: str = field(default="", compare=False)

    @property
    def shapes(self) -> List[Shape]:
        return [s for _, s in self.params]

    @property
    def psi(self) -> int:
        n = 0
        for s in self.shapes:
            k = 1
            for d in s:
                k *= d
            n += k
        return n


def _llama_layer(hidden, kv, ffn):
    return [
        ("q_proj", (hidden, hidden)),
        ("k_proj", (kv, hidden)),
        ("v_proj", (kv, hidden)),
        ("o_proj", (hidden, hidden)),
        ("gate_proj", (ffn, hidden)),
        ("up_proj", (ffn, hidden)),
        ("down_proj", (hidden, ffn)),
        ("input_norm", (hidden,)),
        ("post_attn_norm", (hidden,)),
    ]


def _qwen_moe_layer():
    p = [
        ("q_proj", (4096, 2048)),
        ("k_proj", (512, 2048)),
        ("v_proj", (512, 2048)),
        ("o_proj", (2048, 4096)),
        ("router", (128, 2048)),
    ]
    for e in range(128):
        p += [
            (f"expert{e}.gate_proj", (768, 2048)),
            (f"expert{e}.up_proj", (768, 2048)),
            (f"expert{e}.down_proj", (2048, 768)),
        ]
    p += [("input_norm", (2048,)), ("post_attn_norm", (2048,))]
    return p


WORKLOADS = {
    "tiny": Workload(
        name="tiny",
        params=[("a", (5, 7)), ("b", (16,)), ("c", (33, 4))],
        world=4, sigma=1.0, rank=1,
        description="3 params [5,7],[16],[33,4]; 4 ranks; rank 1; bf16 ~N(0,1)"),
    "llama3_8b_layer": Workload(
        name="llama3_8b_layer", params=_llama_layer(4096, 1024, 14336),
        world=8, sigma=0.02,
        description="Llama-3-8B-shaped decoder layer, 8 ranks, bf16 ~N(0,0.02^2)"),
    "llama31_70b_layer": Workload(
        name="llama31_70b_layer", params=_llama_layer(8192, 1024, 28672),
        world=8, sigma=0.01,
        description="Llama-3.1-70B-shaped decoder layer, 8 ranks, bf16 ~N(0,0.01^2)"),
    "qwen3_30b_a3b_moe_layer": Workload(
        name="qwen3_30b_a3b_moe_layer", params=_qwen_moe_layer(),
        world=16, sigma=0.02, zero_expert_frac=0.1, n_experts=128,
        description="Qwen3-30B-A3B-shaped MoE layer (391 params), 16 ranks, "
                    "bf16 ~N(0,0.02^2), 10% of experts all-zero per rank"),
    "llama31_70b_layer_n64": Workload(
        name="llama31_70b_layer_n64", params=_llama_layer(8192, 1024, 28672),
        world=64, sigma=0.01, corun_gemm=(8192, 8192, 8192),
        description="Llama-3.1-70B-shaped layer, 64 ranks (~110 GB of bf16 grads), "
                    "co-run with a bf16 8192^3 GEMM"),
}


def zero_experts(w: Workload, r: int) -> List[int]:
    """Experts whose gradients are all +0.0 on rank r (none if the workload
    has no experts): the first round(frac*E) entries of a permutation drawn
    from a CPU generator seeded 10000 + r."""
    if w.n_experts == 0 or w.zero_expert_frac <= 0:
        return []
    k = int(round(w.zero_expert_frac * w.n_experts))
    g = torch.Generator().manual_seed(10000 + r)
    perm = torch.randperm(w.n_experts, generator=g)
    return sorted(int(e) for e in perm[:k])


def rank_grads(w: Workload, r: int, device="cpu", shapes=None, sigma=None, seed_base=None):
    """Rank r's bf16 gradients, one tensor (own allocation) per parameter."""
    shapes = w.shapes if shapes is None else shapes
    sigma = w.sigma if sigma is None else sigma
    base = w.grad_seed_base if seed_base is None else seed_base
    dev = torch.device(device)
    gen = torch.Generator(device=dev).manual_seed(base + r)
    out = []
    for s in shapes:
        x = torch.randn(s, generator=gen, device=dev, dtype=torch.float32)
        x.mul_(sigma)
        out.append(x.to(torch.bfloat16))
        del x
    zeros = set(zero_experts(w, r))
    if zeros:
        names = [n for n, _ in w.params]
        for idx, n in enumerate(names):
            if n.startswith("expert") and int(n.split(".")[0][6:]) in zeros:
                out[idx].zero_()
    return out


def all_grads(w: Workload, device="cpu", **kw):
    """grads[r][i] for every rank r of the workload."""
    return [rank_grads(w, r, device=device, **kw) for r in range(w.world)]


def random_bf16(numel: int, seed: int, sigma: float = 1.0, device="cpu"):
    """A flat bf16 buffer of `numel` normal draws (e.g. a gathered buffer)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev).manual_seed(seed)
    x = torch.randn(numel, generator=gen, device=dev, dtype=torch.float32)
    x.mul_(sigma)
    return x.to(torch.bfloat16)


def random_grads_for_shapes(shapes, world, seed_base=0, sigma=1.0, device="cpu"):
    """Per-rank bf16 gradients for an ad-hoc parameter list (test cases)."""
    w = Workload(name="adhoc", params=[(f"p{i}", tuple(s)) for i, s in enumerate(shapes)],
                 world=world, sigma=sigma, grad_seed_base=seed_base)
    return all_grads(w, device=device)


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a CPU bf16 tensor's bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")
