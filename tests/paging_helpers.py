"""Test-local helpers that build paged inputs from logical (contiguous) K/V.

They are written independently of the oracle's gather and of the workload
generator so that the oracle can be checked against plain dense attention on
the logical arrays.
"""

import numpy as np


def page_in(logical_k, logical_v, lens, block_size, num_blocks, order, fill=np.nan):
    """Place logical sequences into a pool, one block after another.

    logical_k[i] has shape [L_i, Hkv, D] (float64 here).  Blocks are taken
    from ``order`` in sequence order.  Returns (k_pool, v_pool, tables) with
    pool shape [num_blocks, Hkv, block_size, D]; unused slots hold ``fill``.
    """
    Hkv, D = logical_k[0].shape[1], logical_k[0].shape[2]
    kp = np.full((num_blocks, Hkv, block_size, D), fill, dtype=np.float64)
    vp = np.full_like(kp, fill)
    nblk = [-(-int(L) // block_size) for L in lens]
    MB = max(max(nblk), 1)
    tables = np.zeros((len(lens), MB), dtype=np.int64)
    pos = 0
    for i, L in enumerate(lens):
        for j in range(nblk[i]):
            b = int(order[pos])
            pos += 1
            tables[i, j] = b
            for o in range(block_size):
                t = j * block_size + o
                if t < L:
                    for h in range(Hkv):
                        kp[b, h, o, :] = logical_k[i][t, h, :]
                        vp[b, h, o, :] = logical_v[i][t, h, :]
    # padding entries point at the first unused block
    if pos < num_blocks:
        for i in range(len(lens)):
            tables[i, nblk[i]:] = int(order[pos])
    return kp, vp, tables


def brute_force_decode(q, logical_k, logical_v, scale, group):
    """Pure-Python scalar loops (math.exp, math.fsum): softmax attention of
    each query head over its sequence's logical keys and values."""
    import math
    S = len(q)
    out = []
    for i in range(S):
        Hq = len(q[i])
        rows = []
        for h in range(Hq):
            g = h // group
            L = len(logical_k[i])
            if L == 0:
                rows.append([0.0] * len(q[i][h]))
                continue
            s = [scale * math.fsum(q[i][h][d] * logical_k[i][t][g][d] for d in range(len(q[i][h])))
                 for t in range(L)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            Z = math.fsum(w)
            rows.append([math.fsum(w[t] / Z * logical_v[i][t][g][d] for t in range(L))
                         for d in range(len(q[i][h]))])
        out.append(rows)
    return np.array(out, dtype=np.float64)
