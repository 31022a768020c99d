"""Seeded synthetic inputs for the fused clip + AdamW optimizer step.

This module only describes tensor lists (shapes, groups, trainable and owner
flags, gradient dtypes), hyperparameter schedules and random values.  It holds
none of the optimizer's arithmetic: both the HIP path and the fp64 oracle take
what it produces as plain inputs.

Workloads (all synthetic; no dataset or trained weight is involved):

* ``tiny``          64 fp32 tensors, log-uniform sizes in [1, 65536], one group,
                    effective-batch divisor 4, max_norm 1, one step.
* ``action_expert`` an 18-block d=1024 transformer action head (q/k/v/o, up/gate/
                    down, two RMSNorms per block, plus action in/out projections),
                    bf16 gradients, fp32 state, two groups, ten steps.
* ``launch_bound``  20,000 fp32 tensors of 1..4096 elements, 30% frozen, three
                    groups with a linear lr warm-up over ten steps.
* ``backbone_7b``   a 32-layer d=4096 / MLP 11008 / vocab 32064 backbone
                    (6,738,939,904 elements), bf16 gradients whose global norm
                    alternates between 0.5 and 5 times max_norm (two seeded
                    draws, scaled per step, repeating with period 2).
* ``sharded_7b``    the backbone's matrices cut into four contiguous shards held
                    together on one device, with every RMSNorm replicated in each
                    shard and owned only by shard 0; cosine lr schedule.

Hyperparameter constants come from the veRL training-process page (section
"Training Configuration": actor lr 5e-6, grad_clip 1; section 4.2: the loss is
divided by the number of micro-batches, 128 // 8 = 16 there).

Seeds follow ``1000 * config + purpose``; per-tensor streams add the tensor's
logical index so that a sharded layout reproduces the unsharded values exactly.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Callable, List, Optional, Sequence

import numpy as np

F32 = "f32"
BF16 = "bf16"
F16 = "f16"

# Purposes that enter the seed (seed = 1000 * config + purpose).
SEED_SIZES = 1
SEED_PARAMS = 2
SEED_GRADS = 3
SEED_FROZEN = 4

# Page constants (veRL training-process page, "Training Configuration").
PAGE_LR = 5e-6
PAGE_MAX_NORM = 1.0


@dataclass(frozen=True)
class GroupHP:
    """Per-parameter-group AdamW settings (base values before any schedule)."""

    lr: float
    weight_decay: float
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8


@dataclass(frozen=True)
class TensorSpec:
    """One logical tensor of the model."""

    name: str
    numel: int
    group: int
    grad_dtype: str = F32
    trainable: bool = True


@dataclass
class Workload:
    """A tensor list plus the step-level settings that drive the optimizer."""

    name: str
    config: int                      # 1-based configuration number (seed base)
    tensors: List[TensorSpec]
    groups: List[GroupHP]
    max_norm: float
    grad_divisor: float
    steps: int
    p_std: float = 0.02
    g_std: float = 0.05
    schedule: str = "constant"        # constant | warmup | cosine
    nan_frozen_grads: bool = False     # fill frozen tensors' grads with NaN
    norm_targets: Optional[Sequence[float]] = None  # per-step target global norm
    grad_period: Optional[int] = None  # >0: gradient draws repeat with this period
    meta: dict = field(default_factory=dict)

    # ----------------------------------------------------------------- sizes
    @property
    def n_tensors(self) -> int:
        return len(self.tensors)

    @property
    def trainable_numel(self) -> int:
        return sum(t.numel for t in self.tensors if t.trainable)

    @property
    def total_numel(self) -> int:
        return sum(t.numel for t in self.tensors)

    # -------------------------------------------------------------- schedule
    def lrs_for_step(self, k: int) -> List[float]:
        """Per-group lr for update k (1-based): the caller's schedule."""
        out = []
        for g in self.groups:
            if self.schedule == "constant":
                out.append(g.lr)
            elif self.schedule == "warmup":
                out.append(g.lr * k / self.steps)
            elif self.schedule == "cosine":
                out.append(0.5 * g.lr * (1.0 + math.cos(math.pi * (k - 1) / self.steps)))
            else:
                raise ValueError(f"unknown schedule {self.schedule!r}")
        return out

    def grad_std(self, k: int) -> float:
        """Standard deviation of the synthetic gradients at update k."""
        if self.norm_targets is None:
            return self.g_std
        n_owned = self.trainable_numel
        target = self.norm_targets[(k - 1) % len(self.norm_targets)]
        return target * self.grad_divisor / math.sqrt(max(n_owned, 1))

    # ----------------------------------------------------------------- seeds
    def seed(self, purpose: int, index: int = 0, step: int = 0) -> int:
        return (1000 * self.config + purpose) * 1_000_003 + index * 101 + step


# --------------------------------------------------------------------------
# Workload constructors
# --------------------------------------------------------------------------

def tiny(seed_offset: int = 0, n_tensors: int = 64, max_numel: int = 65536) -> Workload:
    """64 fp32 tensors, sizes clip(rint(exp(U(0, ln 65536))), 1, 65536)."""
    rng = np.random.default_rng(1000 * 1 + SEED_SIZES + seed_offset)
    u = rng.uniform(0.0, math.log(max_numel), size=n_tensors)
    sizes = np.clip(np.rint(np.exp(u)), 1, max_numel).astype(np.int64)
    tensors = [TensorSpec(f"t{i}", int(s), 0, F32) for i, s in enumerate(sizes)]
    return Workload(
        name="tiny", config=1, tensors=tensors,
        groups=[GroupHP(lr=PAGE_LR, weight_decay=0.01)],
        max_norm=PAGE_MAX_NORM, grad_divisor=4.0, steps=1,
        p_std=0.02, g_std=0.05)


def _action_expert_tensors(blocks: int, d: int, mlp: int, action_dim: int) -> List[TensorSpec]:
    t: List[TensorSpec] = [TensorSpec("action_in_proj", d * action_dim, 0, BF16)]
    for b in range(blocks):
        for nm in ("q", "k", "v", "o"):
            t.append(TensorSpec(f"blk{b}.{nm}", d * d, 0, BF16))
        t.append(TensorSpec(f"blk{b}.up", mlp * d, 0, BF16))
        t.append(TensorSpec(f"blk{b}.gate", mlp * d, 0, BF16))
        t.append(TensorSpec(f"blk{b}.down", d * mlp, 0, BF16))
        t.append(TensorSpec(f"blk{b}.norm1", d, 1, BF16))
        t.append(TensorSpec(f"blk{b}.norm2", d, 1, BF16))
    t.append(TensorSpec("action_out_proj", action_dim * d, 0, BF16))
    return t


def action_expert(blocks: int = 18, d: int = 1024, mlp: int = 4096,
                  action_dim: int = 32, steps: int = 10) -> Workload:
    """Action-expert head; group 0 = matrices (wd 0.01), group 1 = RMSNorms (wd 0)."""
    return Workload(
        name="action_expert" if (blocks, d, mlp) == (18, 1024, 4096)
        else f"action_expert_b{blocks}_d{d}_m{mlp}",
        config=2, tensors=_action_expert_tensors(blocks, d, mlp, action_dim),
        groups=[GroupHP(lr=PAGE_LR, weight_decay=0.01), GroupHP(lr=PAGE_LR, weight_decay=0.0)],
        max_norm=PAGE_MAX_NORM, grad_divisor=1.0, steps=steps,
        p_std=0.02, g_std=0.1,
        meta=dict(blocks=blocks, d=d, mlp=mlp, action_dim=action_dim))


def launch_bound(n_tensors: int = 20000, max_numel: int = 4096, frozen_frac: float = 0.3,
                 max_norm: float = 10.0, steps: int = 10) -> Workload:
    """Many small fp32 tensors; an exact 30% are frozen (seeded permutation)."""
    rng = np.random.default_rng(1000 * 3 + SEED_SIZES)
    sizes = rng.integers(1, max_numel + 1, size=n_tensors)
    perm = np.random.default_rng(1000 * 3 + SEED_FROZEN).permutation(n_tensors)
    frozen = np.zeros(n_tensors, dtype=bool)
    frozen[perm[: int(round(frozen_frac * n_tensors))]] = True
    tensors = [TensorSpec(f"t{i}", int(sizes[i]), i % 3, F32, trainable=not frozen[i])
               for i in range(n_tensors)]
    return Workload(
        name="launch_bound" if n_tensors == 20000 else f"launch_bound_{n_tensors}",
        config=3, tensors=tensors,
        groups=[GroupHP(lr=5e-6, weight_decay=0.01), GroupHP(lr=1e-5, weight_decay=0.0),
                GroupHP(lr=2.5e-6, weight_decay=0.01)],
        max_norm=max_norm, grad_divisor=1.0, steps=steps,
        p_std=0.02, g_std=1e-3, schedule="warmup", nan_frozen_grads=True)


def _backbone_tensors(layers: int, d: int, mlp: int, vocab: int) -> List[TensorSpec]:
    t: List[TensorSpec] = [TensorSpec("embed", vocab * d, 0, BF16)]
    for layer in range(layers):
        for nm in ("q", "k", "v", "o"):
            t.append(TensorSpec(f"l{layer}.{nm}", d * d, 0, BF16))
        t.append(TensorSpec(f"l{layer}.gate", mlp * d, 0, BF16))
        t.append(TensorSpec(f"l{layer}.up", mlp * d, 0, BF16))
        t.append(TensorSpec(f"l{layer}.down", d * mlp, 0, BF16))
        t.append(TensorSpec(f"l{layer}.input_norm", d, 1, BF16))
        t.append(TensorSpec(f"l{layer}.post_norm", d, 1, BF16))
    t.append(TensorSpec("final_norm", d, 1, BF16))
    t.append(TensorSpec("lm_head", vocab * d, 0, BF16))
    return t


def backbone_7b(layers: int = 32, d: int = 4096, mlp: int = 11008, vocab: int = 32064,
                steps: int = 10) -> Workload:
    """7B-scale backbone state; grads scaled so the global norm alternates 0.5 / 5."""
    full = (layers, d, mlp, vocab) == (32, 4096, 11008, 32064)
    return Workload(
        name="backbone_7b" if full else f"backbone_l{layers}_d{d}_m{mlp}_v{vocab}",
        config=4, tensors=_backbone_tensors(layers, d, mlp, vocab),
        groups=[GroupHP(lr=PAGE_LR, weight_decay=0.01), GroupHP(lr=PAGE_LR, weight_decay=0.0)],
        max_norm=PAGE_MAX_NORM, grad_divisor=1.0, steps=steps,
        p_std=0.02, norm_targets=(0.5 * PAGE_MAX_NORM, 5.0 * PAGE_MAX_NORM), grad_period=2,
        meta=dict(layers=layers, d=d, mlp=mlp, vocab=vocab))


@dataclass(frozen=True)
class Piece:
    """A contiguous piece of a logical tensor placed inside one shard."""

    tensor: int        # logical tensor index in the unsharded workload
    t_offset: int      # first element of the piece inside that tensor
    numel: int
    shard: int
    s_offset: int      # first element of the piece inside the shard allocation
    owner: bool


@dataclass
class ShardLayout:
    """Four contiguous shards of the matrices plus replicated RMSNorm tensors."""

    base: Workload                 # the unsharded workload (oracle side)
    n_shards: int
    shard_numel: List[int]         # elements per shard allocation
    pieces: List[Piece]            # descriptor order = piece order
    schedule: str = "cosine"

    @property
    def n_descriptors(self) -> int:
        return len(self.pieces)


def sharded_7b(n_shards: int = 4, **backbone_kw) -> ShardLayout:
    """Cut the backbone's matrices (unsharded order) into equal contiguous shards.

    Every shard also holds a full replica of all RMSNorm tensors; only shard 0
    owns them, so each element enters the global norm exactly once.
    """
    base = replace(backbone_7b(**backbone_kw), schedule="cosine", config=5)
    mats = [i for i, t in enumerate(base.tensors) if t.group == 0]
    norms = [i for i, t in enumerate(base.tensors) if t.group == 1]
    total = sum(base.tensors[i].numel for i in mats)
    if total % n_shards:
        raise ValueError("matrix elements do not divide evenly into shards")
    per = total // n_shards
    norm_numel = sum(base.tensors[i].numel for i in norms)
    pieces: List[Piece] = []
    flat = 0
    for i in mats:
        n = base.tensors[i].numel
        off = 0
        while off < n:
            shard = (flat + off) // per
            s_off = (flat + off) - shard * per
            take = min(n - off, per - s_off)
            pieces.append(Piece(i, off, take, shard, s_off, True))
            off += take
        flat += n
    # replicas go after the shard's matrix elements, in tensor order
    by_shard: List[List[Piece]] = [[p for p in pieces if p.shard == s] for s in range(n_shards)]
    out: List[Piece] = []
    for s in range(n_shards):
        out.extend(by_shard[s])
        off = per
        for i in norms:
            n = base.tensors[i].numel
            out.append(Piece(i, 0, n, s, off, s == 0))
            off += n
    return ShardLayout(base=base, n_shards=n_shards,
                       shard_numel=[per + norm_numel] * n_shards, pieces=out)


# Elements per buffer of the per-kind arena layout (4 GiB of fp32).
ARENA_CHUNK = 1 << 30


def arena_layout(wl: Workload, align: int = 64, max_elems: int = ARENA_CHUNK):
    """Placement of every tensor in per-kind buffers (one set of buffers for
    each of p, g, m, v): tensors in table order, each starting at a multiple of
    ``align`` elements, a new buffer whenever the current one would pass
    ``max_elems``.  Returns ([(buffer, offset)] per tensor, [elements per
    buffer]); every kind uses the same placement."""
    place, sizes = [], [0]
    for t in wl.tensors:
        n = -(-t.numel // align) * align
        if sizes[-1] > 0 and sizes[-1] + n > max_elems:
            sizes.append(0)
        place.append((len(sizes) - 1, sizes[-1]))
        sizes[-1] += n
    return place, sizes


WORKLOADS: dict = {
    "tiny": tiny,
    "action_expert": action_expert,
    "launch_bound": launch_bound,
    "backbone_7b": backbone_7b,
}


# --------------------------------------------------------------------------
# Values.  Generation uses torch only as a seeded random-number source; the
# CPU and GPU generators give different (but each reproducible) streams.
# --------------------------------------------------------------------------

def _torch():
    import torch  # local import: host-only tests of the oracle do not need torch
    return torch


def _gen(seed: int, device):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def param_values(wl: Workload, index: int, device="cpu"):
    """fp32 initial weights of logical tensor ``index`` (N(0, p_std))."""
    torch = _torch()
    n = wl.tensors[index].numel
    x = torch.randn(n, generator=_gen(wl.seed(SEED_PARAMS, index), device),
                    device=device, dtype=torch.float32)
    return x.mul_(wl.p_std)


def grad_values(wl: Workload, index: int, step: int, device="cpu"):
    """Gradient of logical tensor ``index`` at update ``step`` (1-based).

    fp32 tensors get fp32 values; bf16 tensors get N(0, std) rounded to bf16.
    Frozen tensors get NaN when the workload asks for it (they must never be
    read).
    """
    torch = _torch()
    spec = wl.tensors[index]
    dt = torch_dtype(spec.grad_dtype)
    if not spec.trainable and wl.nan_frozen_grads:
        return torch.full((spec.numel,), float("nan"), dtype=dt, device=device)
    draw = step if not wl.grad_period else 1 + (step - 1) % wl.grad_period
    x = torch.randn(spec.numel, generator=_gen(wl.seed(SEED_GRADS, index, draw), device),
                    device=device, dtype=torch.float32)
    x.mul_(wl.grad_std(step))
    return x.to(dt)


def torch_dtype(name: str):
    torch = _torch()
    return {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}[name]


def bf16_bits(t) -> np.ndarray:
    """Raw uint16 bit patterns of a bf16 torch tensor (host copy)."""
    torch = _torch()
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def to_numpy_grad(t) -> np.ndarray:
    """Host copy of a gradient: float32/float16 array, or uint16 bf16 bit patterns."""
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.detach().cpu().numpy()
