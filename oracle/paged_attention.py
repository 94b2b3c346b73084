"""Plain fp64 CPU oracle for paged-KV-cache decode attention and the KV append.

TEST INFRASTRUCTURE ONLY.  This module is the checker that the HIP kernels are
compared against.  Only the test suite, the smoke check and the CPU-baseline leg
of the benchmark may import it; the library itself never does, and this module
imports nothing from the library.  It is written for clarity, not speed.

What it follows (pages named by title and section):

* "PagedAttention核心思想" (vLLM memory-management chapter), section 2.2: a
  request's KV cache is a sequence of logical blocks; the Block Table maps each
  logical block to a physical block anywhere in the pool, and through that table
  the blocks behave exactly like one contiguous buffer.  Hence the result of
  paged decode attention *is* ordinary softmax attention of the query over the
  contiguous logical K/V sequence, and that plain definition is what is written
  out here (gather, then a two-pass softmax).
* Same chapter, section 2.3: a block holds ``block_size`` tokens for every
  attention head; the cache tensors here are laid out
  ``[num_blocks, num_kv_heads, block_size, head_dim]``.
* Same chapter, section 2.5: attention is computed by looking up each block's
  physical id in the table, scoring the query against the block's keys and
  weighting the block's values; block after block until all are done.
* "VLLM中PagedAttention如何降低显存碎片？" (CSDN answer), section 三 items 4 and 9:
  the kernel turns a token position into a logical page number plus an offset
  and looks the page up in the table; every attention head addresses the same
  set of pages.
* "PagedAttention技术解析", section 2.2 item 3: tokens past the end of the
  sequence inside the last block are masked out, never computed with.
* "PagedAttention核心思想" section 2.4.2: appending a token writes its K/V into
  the next slot of the sequence's last block (a fresh block once it is full).

Readings taken where the pages are silent (each one also listed in the design
notes): the in-block offset is ``t % block_size``; scores are
``scale * (q . k)``; query head ``h`` uses KV head ``h // (Hq // Hkv)``;
positions ``[0, context_len)`` are attended; ``context_len == 0`` gives a zero
output; stale data in table padding, in unused blocks and in the tail of the
last block never influences the result.

Precision: every stored value is decoded exactly to float64 (fp32 as is, fp16
through numpy's half type, bf16 by placing its 16 bits in the top half of an
fp32 word), and all arithmetic is float64.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

DTYPES = ("f32", "f16", "bf16")


# ---------------------------------------------------------------------------
# exact decoding of stored values
# ---------------------------------------------------------------------------

def to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode stored elements to float64 exactly.

    ``bits`` holds the stored representation: float32 values for "f32",
    float16 values (or their uint16 bit patterns) for "f16", and uint16 bit
    patterns for "bf16" (bfloat16 is the top half of an IEEE fp32 word).
    """
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        a = np.asarray(bits)
        if a.dtype == np.uint16:
            a = a.view(np.float16)
        return a.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        a = np.asarray(bits)
        if a.dtype != np.uint16:
            raise TypeError("bf16 input must be given as uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# address translation (logical token position -> physical slot)
# ---------------------------------------------------------------------------

def physical_slot(block_table_row: np.ndarray, t: int, block_size: int) -> Tuple[int, int]:
    """Token position ``t`` of a sequence -> (physical block id, in-block offset).

    The logical page is ``t // block_size``; its physical id comes from the
    sequence's Block Table row; the offset inside the page is
    ``t % block_size`` (the pages make an explicit offset field optional).
    """
    return int(block_table_row[t // block_size]), t % block_size


def gather_rows(cache: np.ndarray, block_table_row: np.ndarray, kv_head: int,
                start: int, stop: int, block_size: int, dtype: str) -> np.ndarray:
    """Logical rows ``[start, stop)`` of one KV head of one sequence, as float64.

    Walks the Block Table block by block; only the first
    ``ceil(stop / block_size)`` entries of the row are ever read, so padding
    entries past the sequence's last block are never touched.
    """
    num_blocks = cache.shape[0]
    rows = []
    t = start
    while t < stop:
        phys, off = physical_slot(block_table_row, t, block_size)
        if not 0 <= phys < num_blocks:
            raise IndexError(f"block id {phys} outside the pool of {num_blocks} blocks")
        n = min(block_size - off, stop - t)
        rows.append(cache[phys, kv_head, off:off + n, :])
        t += n
    if not rows:
        return np.zeros((0, cache.shape[3]), dtype=np.float64)
    return to_f64(np.concatenate(rows, axis=0), dtype)


# ---------------------------------------------------------------------------
# decode attention
# ---------------------------------------------------------------------------

def kv_head_of(q_head: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by a query head.  The pages only say that every head
    addresses the same set of pages (CSDN answer section 三 item 9); the
    reading taken is that contiguous groups of ``num_q_heads // num_kv_heads``
    query heads share one KV head."""
    return q_head // (num_q_heads // num_kv_heads)


def softmax_weights(scores: np.ndarray) -> np.ndarray:
    """Normalised softmax weights of a score vector, max-shifted for range."""
    m = scores.max()
    w = np.exp(scores - m)
    return w / w.sum()


def _attend_one(qv: np.ndarray, cache_k: np.ndarray, cache_v: np.ndarray,
                table_row: np.ndarray, kv_head: int, L: int, block_size: int,
                scale: float, dtype: str, chunk_tokens: int,
                want_probs: bool):
    """Softmax attention of one query vector over logical positions [0, L).

    Two passes over the sequence: scores and their maximum first, then the
    normalised weights times the values.  Long sequences are processed in
    chunks of ``chunk_tokens`` logical positions so that memory stays bounded;
    the chunking only bounds memory, every score is computed independently.
    """
    D = qv.shape[0]
    if L == 0:
        return np.zeros(D, dtype=np.float64), (np.zeros(0) if want_probs else None)
    scores = np.empty(L, dtype=np.float64)
    for a in range(0, L, chunk_tokens):
        b = min(L, a + chunk_tokens)
        K = gather_rows(cache_k, table_row, kv_head, a, b, block_size, dtype)
        scores[a:b] = scale * (K @ qv)
    p = softmax_weights(scores)
    out = np.zeros(D, dtype=np.float64)
    for a in range(0, L, chunk_tokens):
        b = min(L, a + chunk_tokens)
        V = gather_rows(cache_v, table_row, kv_head, a, b, block_size, dtype)
        out += p[a:b] @ V
    return out, (p if want_probs else None)


def paged_attn_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                      block_tables: np.ndarray, context_lens: np.ndarray,
                      block_size: int, scale: float, dtype: str,
                      pairs: Optional[Iterable[Tuple[int, int]]] = None,
                      return_probs: bool = False,
                      chunk_tokens: int = 1 << 16):
    """Single-token decode attention over a paged KV cache, in float64.

    Arguments (stored representation, see ``to_f64``):
      q             [num_seqs, num_q_heads, head_dim]
      k_cache       [num_blocks, num_kv_heads, block_size, head_dim]
      v_cache       same shape as k_cache
      block_tables  int [num_seqs, max_blocks_per_seq]; row i maps sequence i's
                    logical block j to a physical block id
      context_lens  int [num_seqs]; number of cached tokens attended by seq i
      block_size    tokens per block (must equal k_cache.shape[2])
      scale         score scale applied to q . k before the softmax
      pairs         optional iterable of (seq, q_head); if given, only those
                    outputs are computed and the rest of ``out`` is NaN
      return_probs  also return a dict (seq, q_head) -> softmax weights

    Returns ``out`` float64 [num_seqs, num_q_heads, head_dim] (and the dict).
    """
    S, Hq, D = q.shape
    NB, Hkv, BS, D2 = k_cache.shape
    if BS != block_size or D2 != D or v_cache.shape != k_cache.shape:
        raise ValueError("cache shape does not match q / block_size")
    if Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    qf = to_f64(q, dtype)
    if pairs is None:
        pairs = [(i, h) for i in range(S) for h in range(Hq)]
        out = np.zeros((S, Hq, D), dtype=np.float64)
    else:
        pairs = list(pairs)
        out = np.full((S, Hq, D), np.nan, dtype=np.float64)
    probs = {}
    for i, h in pairs:
        L = int(context_lens[i])
        if L < 0:
            raise ValueError("negative context length")
        kv_head = kv_head_of(h, Hq, Hkv)
        o, p = _attend_one(qf[i, h], k_cache, v_cache, np.asarray(block_tables[i]),
                           kv_head, L, block_size, float(scale), dtype,
                           chunk_tokens, return_probs)
        out[i, h] = o
        if return_probs:
            probs[(i, h)] = p
    if return_probs:
        return out, probs
    return out


def query_context_len(L: int, num_query_tokens: int, j: int) -> int:
    """Positions attended by query token ``j`` of ``num_query_tokens`` new
    tokens of a sequence whose cache holds ``L`` tokens.

    Reading taken (the pages describe one query per step; several queries per
    sequence arise from parallel sampling, beam search and draft
    verification, "PagedAttention核心思想" section 2.4.3): the new tokens are
    the last ``num_query_tokens`` positions of the sequence, already written to
    the cache, and each attends to every position up to and including its own,
    so query ``j`` sees ``[0, L - num_query_tokens + j + 1)``; a query with no
    such position gets the empty (zero) output.
    """
    return max(0, L - num_query_tokens + j + 1)


def paged_attn_decode_multi(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                            block_tables: np.ndarray, context_lens: np.ndarray,
                            block_size: int, scale: float, dtype: str,
                            triples: Optional[Iterable[Tuple[int, int, int]]] = None,
                            chunk_tokens: int = 1 << 16):
    """Decode attention with several query tokens per sequence, in float64.

    ``q`` is [num_seqs, num_query_tokens, num_q_heads, head_dim]; query token
    ``j`` of sequence ``i`` is ordinary softmax attention over the logical
    positions ``query_context_len(L_i, T, j)`` walks, read block by block
    through the sequence's table ("PagedAttention核心思想" section 2.5).
    ``triples`` optionally restricts the work to (seq, query token, q head)
    outputs (the others are NaN).  Returns float64 of q's shape.
    """
    S, T, Hq, D = q.shape
    NB, Hkv, BS, D2 = k_cache.shape
    if BS != block_size or D2 != D or v_cache.shape != k_cache.shape:
        raise ValueError("cache shape does not match q / block_size")
    if Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    qf = to_f64(q, dtype)
    if triples is None:
        triples = [(i, j, h) for i in range(S) for j in range(T) for h in range(Hq)]
        out = np.zeros((S, T, Hq, D), dtype=np.float64)
    else:
        triples = list(triples)
        out = np.full((S, T, Hq, D), np.nan, dtype=np.float64)
    for i, j, h in triples:
        L = int(context_lens[i])
        if L < 0:
            raise ValueError("negative context length")
        o, _ = _attend_one(qf[i, j, h], k_cache, v_cache, np.asarray(block_tables[i]),
                           kv_head_of(h, Hq, Hkv), query_context_len(L, T, j), block_size,
                           float(scale), dtype, chunk_tokens, False)
        out[i, j, h] = o
    return out


# ---------------------------------------------------------------------------
# KV append (scatter of new tokens into their slots)
# ---------------------------------------------------------------------------

def paged_kv_write(k: np.ndarray, v: np.ndarray, k_cache: np.ndarray,
                   v_cache: np.ndarray, slot_mapping: Sequence[int]):
    """Copy each new token's K/V rows into its slot; returns new cache arrays.

    ``k``, ``v``: [num_tokens, num_kv_heads, head_dim] in the cache's stored
    representation.  ``slot_mapping[n]`` is ``physical_block * block_size +
    offset``; a negative slot means the token is skipped.  The copy is a bit
    copy (no conversion), so the result is compared byte for byte.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    NB, Hkv, BS, D = kc.shape
    if k.shape[1:] != (Hkv, D) or v.shape != k.shape:
        raise ValueError("k/v shape does not match the cache")
    for n, s in enumerate(slot_mapping):
        s = int(s)
        if s < 0:
            continue
        b, off = s // BS, s % BS
        if b >= NB:
            raise IndexError(f"slot {s} outside the pool")
        kc[b, :, off, :] = k[n]
        vc[b, :, off, :] = v[n]
    return kc, vc


# ---------------------------------------------------------------------------
# block copy (copy-on-write)
# ---------------------------------------------------------------------------

def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, block_pairs):
    """Whole-block bit copy for copy-on-write; returns new cache arrays.

    "PagedAttention核心思想" section 2.4.3: shared blocks are read-only, and a
    write into a block referenced more than once first copies it.  Every pair
    (src, dst) with both ids non-negative makes block ``dst`` (all KV heads,
    all rows) a copy of block ``src``; pairs are applied in order.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    for src, dst in block_pairs:
        src, dst = int(src), int(dst)
        if src < 0 or dst < 0:
            continue
        if not (src < kc.shape[0] and dst < kc.shape[0]):
            raise IndexError("block id outside the pool")
        kc[dst] = kc[src]
        vc[dst] = vc[src]
    return kc, vc


__all__ = ["DTYPES", "to_f64", "physical_slot", "gather_rows", "kv_head_of",
           "softmax_weights", "paged_attn_decode", "query_context_len",
           "paged_attn_decode_multi", "paged_kv_write", "copy_blocks"]
