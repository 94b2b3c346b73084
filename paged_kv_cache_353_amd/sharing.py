"""Host-side discovery of shared prefixes for ``paged_attn_decode_shared``.

Forks of one request point their Block Tables at the same physical blocks for
the prompt they share ("PagedAttention核心思想" section 2.4.3).  The scheduler
that owns the tables can describe that sharing to the decode kernel as groups
of consecutive sequences plus, per sequence, the number of leading positions
it shares with its group.  This module derives that description from host
copies of the tables; it reads nothing from the device.
"""

from __future__ import annotations

from typing import Tuple

import numpy as np


def _common_blocks(a: np.ndarray, b: np.ndarray, n: int) -> int:
    """Leading entries of two table rows (within the first n) that are equal."""
    neq = np.flatnonzero(a[:n] != b[:n])
    return int(neq[0]) if neq.size else n


def shared_prefix_groups(block_tables: np.ndarray, context_lens: np.ndarray,
                         block_size: int, min_shared_tokens: int = 1
                         ) -> Tuple[np.ndarray, np.ndarray]:
    """Group consecutive sequences that share leading physical blocks.

    A group starts at a sequence and takes in the following sequences for as
    long as each shares at least ``min_shared_tokens`` leading positions with
    the group's first member.  The group's shared length is the smallest of
    those counts, never more than any member's length, so positions below it
    lie in the same physical blocks for every member.  A sequence alone in its
    group shares nothing.

    Returns ``group_starts`` (int32 [num_groups + 1]) and ``prefix_lens``
    (int32 [num_seqs]) in the form ``paged_attn_decode_shared`` takes.
    """
    tables = np.asarray(block_tables)
    lens = np.asarray(context_lens).astype(np.int64)
    S = len(lens)
    starts = [0]
    prefix = np.zeros(S, dtype=np.int32)
    i = 0
    while i < S:
        first = i
        shared = int(lens[first])
        j = i + 1
        while j < S:
            n = int(min(-(-lens[first] // block_size), -(-lens[j] // block_size)))
            common = min(_common_blocks(tables[first], tables[j], n) * block_size,
                         int(lens[first]), int(lens[j]))
            if common < max(1, min_shared_tokens):
                break
            shared = min(shared, common)
            j += 1
        if j - first > 1:
            prefix[first:j] = shared
        starts.append(j)
        i = j
    return np.asarray(starts, dtype=np.int32), prefix


def check_shared_prefix(block_tables: np.ndarray, context_lens: np.ndarray, block_size: int,
                        group_starts: np.ndarray, prefix_lens: np.ndarray) -> None:
    """Raise ValueError unless the description meets the preconditions of
    ``paged_attn_decode_shared`` (the kernel cannot check device data)."""
    tables = np.asarray(block_tables)
    lens = np.asarray(context_lens).astype(np.int64)
    gs = np.asarray(group_starts).astype(np.int64)
    pl = np.asarray(prefix_lens).astype(np.int64)
    S = len(lens)
    if gs.ndim != 1 or len(gs) < 2 or gs[0] != 0 or gs[-1] != S or np.any(np.diff(gs) < 0):
        raise ValueError("group_starts must run from 0 to num_seqs, non-decreasing")
    if pl.shape != (S,) or np.any(pl < 0) or np.any(pl > lens):
        raise ValueError("prefix_lens must lie in [0, context_len]")
    for g in range(len(gs) - 1):
        a, b = int(gs[g]), int(gs[g + 1])
        if a == b:
            continue
        if np.any(pl[a:b] != pl[a]):
            raise ValueError(f"group {g}: members disagree on the shared length")
        nb = -(-int(pl[a]) // block_size)
        for k in range(a + 1, b):
            if not np.array_equal(tables[k, :nb], tables[a, :nb]):
                raise ValueError(f"group {g}: sequence {k} does not share the prefix blocks")
