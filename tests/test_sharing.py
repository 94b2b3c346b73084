"""Host logic of the shared-prefix description (no GPU)."""

import numpy as np
import pytest

from paged_kv_cache_353_amd.block_pool import BlockManager, BlockPool
from paged_kv_cache_353_amd.sharing import check_shared_prefix, shared_prefix_groups


def _forked_batch(prompt_lens, samples, suffix, bs, seed):
    pool = BlockPool(4096, order=np.random.default_rng(seed).permutation(4096))
    mgr = BlockManager(pool, bs)
    ids = []
    for P in prompt_lens:
        root = mgr.new_sequence()
        for _ in range(P):
            mgr.append_token(root)
        ids += [root] + mgr.fork_many(root, samples - 1)
    for _ in range(suffix):
        mgr.append_batch(ids)
    MB = max(len(mgr.seqs[s].table) for s in ids)
    tables = np.zeros((len(ids), MB), dtype=np.int32)
    for r, s in enumerate(ids):
        tables[r, :len(mgr.seqs[s].table)] = mgr.seqs[s].table
    lens = np.array([mgr.seqs[s].length for s in ids])
    return tables, lens


@pytest.mark.parametrize("prompt_lens,samples,suffix", [([64, 40, 17], 4, 10), ([1000], 8, 3), ([16], 2, 0)])
def test_groups_follow_the_forks(prompt_lens, samples, suffix):
    bs = 16
    tables, lens = _forked_batch(prompt_lens, samples, suffix, bs, seed=5)
    gs, pl = shared_prefix_groups(tables, lens, bs)
    check_shared_prefix(tables, lens, bs, gs, pl)
    assert gs.tolist() == [samples * g for g in range(len(prompt_lens) + 1)]
    for g, P in enumerate(prompt_lens):
        got = int(pl[g * samples])
        if suffix == 0:
            assert got == P                       # nothing written yet: the whole prompt is shared
        else:
            assert got == (P // bs) * bs          # the partial last block was copied on write


def test_singletons_share_nothing_and_bad_descriptions_are_rejected():
    bs = 16
    tables = np.array([[1, 2], [3, 4], [3, 5]], dtype=np.int32)
    lens = np.array([20, 30, 18])
    gs, pl = shared_prefix_groups(tables, lens, bs)
    assert gs.tolist() == [0, 1, 3] and pl.tolist() == [0, 16, 16]
    check_shared_prefix(tables, lens, bs, gs, pl)
    with pytest.raises(ValueError):
        check_shared_prefix(tables, lens, bs, np.array([0, 3]), np.array([16, 16, 16]))
    with pytest.raises(ValueError):
        check_shared_prefix(tables, lens, bs, gs, np.array([0, 16, 20]))
    with pytest.raises(ValueError):
        check_shared_prefix(tables, lens, bs, np.array([0, 2, 3]), np.array([16, 16, 0]))
