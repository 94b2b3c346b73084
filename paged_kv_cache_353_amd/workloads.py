"""Seeded synthetic inputs for paged decode attention and the KV append.

This module only draws inputs: sequence lengths, the order in which physical
blocks leave the free pool, Block Tables, and N(0,1) values for q and for every
slot of the K/V pools.  It holds none of the attention arithmetic and serves the
HIP path, the oracle and the benchmark alike.

Every slot that a correct kernel must never read is filled with NaN (unused
blocks, the slots past the end of each sequence's last block, and the block
that padding entries of the Block Tables point at): the pages reclaim blocks for
reuse without clearing them ("PagedAttention技术解析" section 4.2; CSDN answer
section 四), so their contents are arbitrary and must not leak into a result.

Integer structure comes from ``numpy.random.default_rng(seed)`` and values from
a ``torch.Generator`` seeded with the same number on the target device, so a
workload is reproducible on a given device type.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from .block_pool import BlockManager, BlockPool

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def seed_for(config_no: int) -> int:
    return 353_000 + int(config_no)


@dataclass
class DecodeInputs:
    """One decode step: append one token per sequence, then attend."""
    q: torch.Tensor                 # [S, Hq, D]
    k_cache: torch.Tensor           # [NB, Hkv, BS, D]
    v_cache: torch.Tensor
    block_tables: torch.Tensor      # int32 [S, MB]
    context_lens: torch.Tensor      # int32 [S] (includes the appended token)
    k_new: torch.Tensor             # [S, Hkv, D] the token appended this step
    v_new: torch.Tensor
    slot_mapping: torch.Tensor      # int64 [S]; slot of position L-1, -1 if L == 0
    block_size: int
    scale: float
    dtype: str
    poison_block: int
    lens: np.ndarray                # host copy of context_lens
    name: str = ""
    meta: Dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_cache.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[2])

    @property
    def max_context_len(self) -> int:
        return int(self.lens.max()) if self.lens.size else 0

    def kv_read_bytes(self) -> int:
        """K and V bytes of the attended tokens, each counted once per sequence."""
        return int(self.lens.sum()) * self.num_kv_heads * self.head_dim * 2 * DTYPE_BYTES[self.dtype]

    def kv_unique_bytes(self) -> int:
        """K and V bytes of the attended tokens counted once per physical slot:
        blocks shared by several sequences (forked prefixes) count once."""
        tables = self.block_tables.cpu().numpy()
        rows = {}
        bs = self.block_size
        for i, L in enumerate(self.lens):
            L = int(L)
            for j in range(-(-L // bs)):
                b = int(tables[i, j])
                rows[b] = max(rows.get(b, 0), min(bs, L - j * bs))
        return sum(rows.values()) * self.num_kv_heads * self.head_dim * 2 * DTYPE_BYTES[self.dtype]


def _randn_into(t: torch.Tensor, gen: torch.Generator, chunk_elems: int = 1 << 28) -> None:
    """Fill ``t`` (contiguous) with N(0,1) drawn in fp32, rounded to t's dtype."""
    flat = t.view(-1)
    n = flat.numel()
    for a in range(0, n, chunk_elems):
        b = min(n, a + chunk_elems)
        flat[a:b] = torch.randn(b - a, generator=gen, device=t.device,
                                dtype=torch.float32).to(t.dtype)


def _poison(k_cache: torch.Tensor, v_cache: torch.Tensor, used: np.ndarray,
            tails: List[tuple]) -> None:
    """NaN-fill unused blocks and the slots past each sequence's end."""
    dev = k_cache.device
    unused = torch.from_numpy(np.flatnonzero(~used)).to(dev)
    if unused.numel():
        k_cache.index_fill_(0, unused, float("nan"))
        v_cache.index_fill_(0, unused, float("nan"))
    for blk, first in tails:
        k_cache[blk, :, first:, :] = float("nan")
        v_cache[blk, :, first:, :] = float("nan")


def build_decode_inputs(lens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                        head_dim: int, block_size: int, dtype: str, num_blocks: int,
                        seed: int, device="cpu", scale: Optional[float] = None,
                        max_blocks_per_seq: Optional[int] = None,
                        block_order: Optional[np.ndarray] = None,
                        name: str = "") -> DecodeInputs:
    """Deal shuffled physical blocks to sequences in order and draw all values.

    ``lens[i]`` is the context length of sequence i after the appended token.
    Blocks leave a free list that is a seeded permutation of the pool (or
    ``block_order``); sequence i takes the next ``ceil(lens[i]/block_size)``
    of them.  The first block left over is the NaN block that every padding
    entry of the tables points at.
    """
    lens = np.asarray(lens, dtype=np.int64)
    S = len(lens)
    rng = np.random.default_rng(seed)
    order = rng.permutation(num_blocks) if block_order is None else np.asarray(block_order)
    nblk = -(-lens // block_size)
    used_total = int(nblk.sum())
    if used_total >= num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {used_total} blocks plus a spare")
    MB = int(max(1, nblk.max() if S else 1)) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    if S and MB < nblk.max():
        raise ValueError("max_blocks_per_seq too small")
    poison = int(order[used_total])
    tables = np.full((S, MB), poison, dtype=np.int32)
    used = np.zeros(num_blocks, dtype=bool)
    tails = []
    pos = 0
    for i in range(S):
        n = int(nblk[i])
        tables[i, :n] = order[pos:pos + n]
        used[order[pos:pos + n]] = True
        pos += n
        r = int(lens[i]) % block_size
        if n and r:
            tails.append((int(tables[i, n - 1]), r))

    tdt = TORCH_DTYPES[dtype]
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    q = torch.empty((S, num_q_heads, head_dim), dtype=tdt, device=device)
    k_cache = torch.empty((num_blocks, num_kv_heads, block_size, head_dim), dtype=tdt, device=device)
    v_cache = torch.empty_like(k_cache)
    k_new = torch.empty((S, num_kv_heads, head_dim), dtype=tdt, device=device)
    v_new = torch.empty_like(k_new)
    for t in (q, k_cache, v_cache, k_new, v_new):
        _randn_into(t, gen)
    _poison(k_cache, v_cache, used, tails)

    slots = np.full(S, -1, dtype=np.int64)
    for i in range(S):
        L = int(lens[i])
        if L > 0:
            slots[i] = int(tables[i, (L - 1) // block_size]) * block_size + (L - 1) % block_size
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return DecodeInputs(
        q=q, k_cache=k_cache, v_cache=v_cache,
        block_tables=torch.from_numpy(tables).to(device),
        context_lens=torch.from_numpy(lens.astype(np.int32)).to(device),
        k_new=k_new, v_new=v_new,
        slot_mapping=torch.from_numpy(slots).to(device),
        block_size=int(block_size), scale=float(scale), dtype=dtype,
        poison_block=poison, lens=lens, name=name,
        meta=dict(seed=int(seed), num_blocks=int(num_blocks)))


# ---------------------------------------------------------------------------
# the five named workloads
# ---------------------------------------------------------------------------

def tiny(device="cpu") -> DecodeInputs:
    """4 seqs, lengths uniform in [17,200], 8 q = 8 kv heads, head_dim 64,
    block_size 16, fp32, a 64-block pool dealt in a seeded random order."""
    seed = seed_for(1)
    lens = np.random.default_rng(seed + 1_000_000).integers(17, 201, size=4)
    return build_decode_inputs(lens, 8, 8, 64, 16, "f32", 64, seed, device,
                               scale=1.0 / 8.0, name="tiny_fp32")


def llama8b_decode(device="cpu") -> DecodeInputs:
    """64 seqs, lengths uniform in [128,2048], 32 q / 8 kv heads, head_dim 128,
    block_size 16, bf16, blocks shuffled across an 8192-block pool."""
    seed = seed_for(2)
    lens = np.random.default_rng(seed + 1_000_000).integers(128, 2049, size=64)
    return build_decode_inputs(lens, 32, 8, 128, 16, "bf16", 8192, seed, device,
                               name="llama8b_bf16_bs16")


def block_size_sweep(block_size: int, device="cpu") -> DecodeInputs:
    """128 seqs, lengths log-uniform in [64,8192], 32 q / 8 kv heads, head_dim
    128, fp16, pool holding 2^20 tokens (2^20/block_size blocks)."""
    if block_size not in (16, 32, 64, 128):
        raise ValueError("block size sweep covers 16, 32, 64 and 128")
    seed = seed_for(3)
    u = np.random.default_rng(seed + 1_000_000).uniform(math.log(64), math.log(8192), size=128)
    lens = np.clip(np.floor(np.exp(u)).astype(np.int64), 64, 8192)
    return build_decode_inputs(lens, 32, 8, 128, block_size, "f16", (1 << 20) // block_size,
                               seed, device, name=f"sweep_fp16_bs{block_size}")


def long_context(device="cpu", lengths=(1 << 17, 1 << 18, 1 << 19, 1 << 20),
                 num_blocks: int = 139_264) -> DecodeInputs:
    """4 seqs at 128k, 256k, 512k and 1M tokens, 32 q / 8 kv heads, head_dim
    128, block_size 16, bf16, blocks scattered through a 139,264-block pool
    (over 2^31 elements per cache, so offsets need 64 bits)."""
    seed = seed_for(5)
    return build_decode_inputs(np.asarray(lengths), 32, 8, 128, 16, "bf16", num_blocks,
                               seed, device, name="long_context_bf16")


def shared_prefix(device="cpu", prompt_len: int = 1024, num_prompts: int = 16,
                  samples: int = 8, suffix_len: int = 256, num_blocks: int = 4096,
                  num_q_heads: int = 32, num_kv_heads: int = 8, head_dim: int = 128,
                  block_size: int = 16, dtype: str = "bf16") -> DecodeInputs:
    """Parallel sampling: each prompt is forked into ``samples`` sequences whose
    tables share the prompt's physical blocks; every sample then appends its
    own ``suffix_len`` tokens, copying a shared partial last block on its first
    write (copy-on-write).  The query attends over prompt + suffix.

    Values are drawn for every slot of the pool up front; a copy-on-write
    duplicates the source block's valid rows into the fresh block, so all
    samples of a prompt read identical prefix data.
    """
    seed = seed_for(4)
    rng = np.random.default_rng(seed)
    pool = BlockPool(num_blocks, order=rng.permutation(num_blocks))
    mgr = BlockManager(pool, block_size)
    sample_ids: List[int] = []
    cows = []
    for _ in range(num_prompts):
        root = mgr.new_sequence()
        for _ in range(prompt_len):
            mgr.append_token(root)
        group = [root] + [mgr.fork(root) for _ in range(samples - 1)]
        sample_ids.extend(group)
    for _ in range(suffix_len):
        for sid in sample_ids:
            _, cow = mgr.append_token(sid)
            if cow is not None:
                cows.append(cow)
    assert np.array_equal(mgr.table_refs(), pool.ref)
    S = len(sample_ids)
    lens = np.array([mgr.seqs[s].length for s in sample_ids], dtype=np.int64)
    MB = max(len(mgr.seqs[s].table) for s in sample_ids)
    free_left = pool._free[::-1]
    if not free_left:
        raise ValueError("no spare block left for table padding")
    poison = int(free_left[0])
    tables = np.full((S, MB), poison, dtype=np.int32)
    for r, s in enumerate(sample_ids):
        tables[r, :len(mgr.seqs[s].table)] = mgr.seqs[s].table

    tdt = TORCH_DTYPES[dtype]
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    q = torch.empty((S, num_q_heads, head_dim), dtype=tdt, device=device)
    k_cache = torch.empty((num_blocks, num_kv_heads, block_size, head_dim), dtype=tdt, device=device)
    v_cache = torch.empty_like(k_cache)
    k_new = torch.empty((S, num_kv_heads, head_dim), dtype=tdt, device=device)
    v_new = torch.empty_like(k_new)
    for t in (q, k_cache, v_cache, k_new, v_new):
        _randn_into(t, gen)
    for c in cows:   # in the order the writes happened
        k_cache[c.dst, :, :c.valid_tokens] = k_cache[c.src, :, :c.valid_tokens]
        v_cache[c.dst, :, :c.valid_tokens] = v_cache[c.src, :, :c.valid_tokens]
    used = pool.ref > 0
    tails = []
    for r in range(S):
        n = -(-int(lens[r]) // block_size)
        rem = int(lens[r]) % block_size
        if rem:
            tails.append((int(tables[r, n - 1]), rem))
    _poison(k_cache, v_cache, used, tails)
    slots = np.array([int(tables[r, (int(lens[r]) - 1) // block_size]) * block_size
                      + (int(lens[r]) - 1) % block_size for r in range(S)], dtype=np.int64)
    # the appended token of this step is the sample's last suffix token: it
    # already sits in its slot, so the append writes the same bytes again
    k_new = torch.stack([k_cache[int(s) // block_size, :, int(s) % block_size] for s in slots])
    v_new = torch.stack([v_cache[int(s) // block_size, :, int(s) % block_size] for s in slots])
    unique_blocks = int(used.sum())
    return DecodeInputs(
        q=q, k_cache=k_cache, v_cache=v_cache,
        block_tables=torch.from_numpy(tables).to(device),
        context_lens=torch.from_numpy(lens.astype(np.int32)).to(device),
        k_new=k_new.contiguous(), v_new=v_new.contiguous(),
        slot_mapping=torch.from_numpy(slots).to(device),
        block_size=block_size, scale=1.0 / math.sqrt(head_dim), dtype=dtype,
        poison_block=poison, lens=lens, name=f"shared_prefix_{prompt_len}",
        meta=dict(seed=seed, num_blocks=num_blocks, cow_copies=len(cows),
                  unique_blocks=unique_blocks,
                  groups=[sample_ids[i:i + samples] for i in range(0, S, samples)]))


def multi_query(inputs: DecodeInputs, num_query_tokens: int, seed: int) -> torch.Tensor:
    """Queries for several new tokens per sequence: N(0,1) values of shape
    [num_seqs, num_query_tokens, num_q_heads, head_dim] in the inputs' dtype.
    The new tokens themselves are the last ``num_query_tokens`` positions of
    each sequence, whose K/V the cache already holds."""
    gen = torch.Generator(device=inputs.q.device)
    gen.manual_seed(int(seed))
    S, Hq, D = inputs.q.shape
    q = torch.empty((S, int(num_query_tokens), Hq, D), dtype=inputs.q.dtype, device=inputs.q.device)
    _randn_into(q, gen)
    return q


def speculative_llama8b(device="cpu", num_query_tokens: int = 4) -> tuple:
    """The Llama-8B-shaped batch (64 sequences, lengths uniform in [128, 2048],
    32 q / 8 kv heads, head_dim 128, bf16, block_size 16) verifying
    ``num_query_tokens`` drafted tokens per sequence: returns (inputs, q)."""
    inp = llama8b_decode(device)
    inp.name = f"llama8b_bf16_bs16_q{num_query_tokens}"
    return inp, multi_query(inp, num_query_tokens, seed_for(2) + 17)


CONFIG_BUILDERS = {
    1: tiny,
    2: llama8b_decode,
    3: block_size_sweep,
    4: shared_prefix,
    5: long_context,
}


# ---------------------------------------------------------------------------
# host-side views for the oracle (stored bits as numpy arrays)
# ---------------------------------------------------------------------------

def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Stored representation of ``t`` as a numpy array (bf16 -> uint16 bits)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
