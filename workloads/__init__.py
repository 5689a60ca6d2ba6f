"""Seeded synthetic workloads for paged decode attention.

This module is shared by the tests, the benchmark and the oracle's callers.  It
holds NONE of the method's arithmetic: no slot, block-table, copy-on-write or
attention computation.  It draws context lengths, free-list orders, fork
points and random q/K/V values, and describes each workload as a script of
block-manager operations that each side (the HIP library's block manager, the
oracle's) executes with its own code.

Workloads (the pages name no model or hardware; these shapes are the decode
batches the path is measured on):

=================  ====  =====  ===  ====  ==  =================================
name               B     Hq/Hkv  d   type  bs  context lengths before the step
=================  ====  =====  ===  ====  ==  =================================
tiny_fp32          2     1/1    64   f32   4   10 and 7 (the pages' example)
mha7b_fp16         64    32/32  128  f16   16  uniform [128, 2048]
gqa70b_bf16        256   64/8   128  bf16  16  log-uniform [256, 4096]
prefix_share_fp16  256   32/32  128  f16   16  1024 shared + tail U[16, 512]
long_splitk_bf16   8     8/1    128  bf16  32  uniform [32768, 131072]
=================  ====  =====  ===  ====  ==  =================================

Values: each q/K/V element is N(0, 1) scaled by ``value_scale`` (1/√128 for the
head_dim-128 workloads, 1 for tiny_fp32) and rounded to the storage type
(round-to-nearest-even).  Seeds are ``1000 * workload_index + repetition``.
"""
from dataclasses import dataclass, field
import math

import numpy as np

F32, F16, BF16 = "f32", "f16", "bf16"


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    dtype: str
    block_size: int
    value_scale: float
    partition_tokens: int = 0          # 0 → the library's automatic choice
    pool_blocks: int = 0               # 0 → sized from the lengths (×1.1)
    notes: str = ""

    @property
    def group(self):
        return self.q_heads // self.kv_heads


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32", 0, 2, 1, 1, 64, F32, 4, 1.0, pool_blocks=16,
                 notes="the pages' 10-token example plus a 7-token sequence"),
        Workload("mha7b_fp16", 1, 64, 32, 32, 128, F16, 16, 1.0 / math.sqrt(128),
                 pool_blocks=12288, notes="Llama-2-7B-shaped MHA decode"),
        Workload("gqa70b_bf16", 2, 256, 64, 8, 128, BF16, 16, 1.0 / math.sqrt(128),
                 notes="70B-layer GQA shape (group 8)"),
        Workload("prefix_share_fp16", 3, 256, 32, 32, 128, F16, 16, 1.0 / math.sqrt(128),
                 pool_blocks=12288, notes="32 prompts x 8 samples, shared 1024-token prefix"),
        Workload("long_splitk_bf16", 4, 8, 8, 1, 128, BF16, 32, 1.0 / math.sqrt(128),
                 partition_tokens=512, notes="long-context split-K decode (group 8)"),
    ]
}


def seed_for(workload, repetition=0):
    return 1000 * workload.index + repetition


# ----------------------------------------------------------------------------
# Scenario: the block-manager calls that build a workload's state
# ----------------------------------------------------------------------------
@dataclass
class Scenario:
    """A workload instance: pool size, free-list order and the call script.

    ``setup`` is a list of ("add", seq_id, n_tokens) / ("fork", parent, child)
    / ("step", [seq_ids]) operations run in order; ``measured`` is the batch of
    sequence ids appended and decoded in the measured decode step.
    ``cow_step`` (prefix sharing only) is the first append after the fork,
    whose writes hit the shared, part-filled last block.
    """
    workload: Workload
    seed: int
    num_blocks: int
    free_order: np.ndarray
    setup: list = field(default_factory=list)
    cow_step: list = None
    growth: list = field(default_factory=list)
    measured: list = field(default_factory=list)
    lengths_before: dict = field(default_factory=dict)

    def all_ops(self):
        """setup, the copy-on-write step (if any) and growth, as one script."""
        ops = list(self.setup)
        if self.cow_step is not None:
            ops.append(("step", list(self.cow_step)))
        ops.extend(("step", ids) for ids in self.growth)
        return ops


def _blocks(n, bs):
    return -(-n // bs)


def make_scenario(workload, repetition=0, batch=None):
    """Draw a seeded instance of ``workload``.  ``batch`` shrinks B for quick tests."""
    w = workload
    seed = seed_for(w, repetition)
    rng = np.random.default_rng(seed)
    B = w.batch if batch is None else batch
    bs = w.block_size

    if w.name == "tiny_fp32":
        lengths = [10, 7][:B]
        head = [5, 12, 3, 9, 0]
        rest = [b for b in range(w.pool_blocks) if b not in head]
        order = np.array(head + list(rng.permutation(rest)), dtype=np.int64)
        sc = Scenario(w, seed, w.pool_blocks, order)
        for i, n in enumerate(lengths):
            sc.setup.append(("add", i, n))
            sc.lengths_before[i] = n
        sc.measured = list(range(len(lengths)))
        return sc

    if w.name == "prefix_share_fp16":
        samples = 8
        prompts = max(1, B // samples)
        fork_extra = rng.integers(1, 16, size=prompts)          # shared tokens past 1024
        tails = rng.integers(16, 513, size=prompts * samples)   # per-sample tail length
        nb = w.pool_blocks
        sc = Scenario(w, seed, nb, rng.permutation(nb).astype(np.int64))
        for p in range(prompts):
            parent = p * samples
            sc.setup.append(("add", parent, 1024 + int(fork_extra[p])))
            for j in range(1, samples):
                sc.setup.append(("fork", parent, parent + j))
        ids = list(range(prompts * samples))
        sc.cow_step = ids
        # after the copy-on-write step each sample holds 1024 + r + 1 tokens;
        # growth steps bring it to 1024 + tail before the measured step
        remaining = [int(tails[s]) - int(fork_extra[s // samples]) - 1 for s in ids]
        for k in range(max(remaining) if remaining else 0):
            sc.growth.append([s for s in ids if remaining[s] > k])
        for s in ids:
            sc.lengths_before[s] = 1024 + int(tails[s])
        sc.measured = ids
        return sc

    if w.name == "mha7b_fp16":
        lengths = rng.integers(128, 2049, size=B)
    elif w.name == "gqa70b_bf16":
        lengths = np.floor(np.exp(rng.uniform(math.log(256), math.log(4096), size=B)))
        lengths = np.clip(lengths, 256, 4096).astype(np.int64)
    elif w.name == "long_splitk_bf16":
        lengths = rng.integers(32768, 131073, size=B)
    else:
        raise KeyError(w.name)
    lengths = [int(n) for n in lengths]
    if w.pool_blocks:
        nb = w.pool_blocks
    else:
        nb = math.ceil(1.1 * sum(_blocks(n + 1, bs) for n in lengths))
    sc = Scenario(w, seed, nb, rng.permutation(nb).astype(np.int64))
    for i, n in enumerate(lengths):
        sc.setup.append(("add", i, n))
        sc.lengths_before[i] = n
    sc.measured = list(range(B))
    return sc


# ----------------------------------------------------------------------------
# Values
# ----------------------------------------------------------------------------
def round_to_bits(x, dtype):
    """Round float32/float64 values to the storage type; return the bit patterns."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == F32:
        return x.view(np.uint32).copy()
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    import torch  # bf16 rounding (nearest-even) via the library's conversion
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


class ValueStream:
    """Deterministic stream of random rows in a storage type.

    Each call draws fresh N(0,1)·scale values, rounded to ``dtype`` and returned
    as bit patterns, so two consumers that make the same calls in the same order
    see the same values.
    """

    def __init__(self, seed, dtype, scale):
        self.rng = np.random.default_rng(seed + 7_000_000)
        self.dtype = dtype
        self.scale = scale

    def draw(self, *shape):
        return round_to_bits(self.rng.standard_normal(shape, dtype=np.float32) * np.float32(self.scale),
                             self.dtype)


def torch_dtype(dtype):
    import torch
    return {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}[dtype]


def bits_torch_dtype(dtype):
    import torch
    return torch.int32 if dtype == F32 else torch.int16


def device_fill_(tensor, seed, scale):
    """Fill a device tensor in place with N(0,1)·scale from a seeded device generator."""
    import torch
    gen = torch.Generator(device=tensor.device)
    gen.manual_seed(seed)
    flat = tensor.view(-1)
    chunk = 1 << 26
    for start in range(0, flat.numel(), chunk):
        part = flat[start:start + chunk]
        part.copy_(torch.randn(part.shape, generator=gen, device=tensor.device,
                               dtype=torch.float32) * scale)
    return tensor
