"""Top-k block selection for block-sparse long-range attention, step by step.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[K25-arch] section 2.2 "direction two": besides the local window, each query
looks only at its top-64 most similar keys (section 2.3: 64 was chosen from
reference statistics).  The page finds those keys through an inverted index
that needs corpus statistics; the block form used here scores whole 64-token
blocks instead:

  1. sum Q over each 64-token query block and K over each 64-token key block
     (per head), in fp64;
  2. score(h, qb, kb) = (sumQ / 64) . (sumK / 64) in fp64, only for key blocks
     strictly earlier than the query block (kb < qb); the softmax scale is left
     out, it does not change the ranking;
  3. keep the ``topk`` highest scores, ties going to the lower block index
     (sort key (-score, kb)); when qb <= topk every earlier block is kept;
  4. write the kept block indices in ascending order, padded with -1.

Query head h is scored against KV head h // (Hq / Hkv).
"""

from __future__ import annotations

import numpy as np


def block_sums(x, block: int) -> np.ndarray:
    """x [L, H, D] -> [H, L/block, D] fp64 block sums."""
    xf = np.asarray(x, dtype=np.float64)
    L, H, D = xf.shape
    if L % block != 0:
        raise ValueError("sequence length must be a multiple of the block size")
    return xf.reshape(L // block, block, H, D).sum(axis=1).transpose(1, 0, 2)


def block_scores(q, k, block: int, h: int) -> np.ndarray:
    """Score matrix [nb, nb] for query head h: mean(Q_qb) . mean(K_kb), fp64.

    Entries with kb >= qb are meaningless and are not used by the selection.
    """
    Hq = q.shape[1]
    Hkv = k.shape[1]
    g = h // (Hq // Hkv)
    qm = block_sums(q[:, h:h + 1], block)[0] / block
    km = block_sums(k[:, g:g + 1], block)[0] / block
    return qm @ km.T


def block_select(q, k, block: int, topk: int, heads=None, return_scores: bool = False):
    """Selected key blocks [Hq, L/block, topk] int32 (ascending, -1 padded).

    ``heads`` optionally restricts the heads computed (others stay -1).  With
    ``return_scores`` the fp64 score matrices of those heads are returned too
    (dict head -> [nb, nb]).
    """
    L, Hq, D = q.shape
    nb = L // block
    heads = range(Hq) if heads is None else heads
    sel = np.full((Hq, nb, max(topk, 0)), -1, dtype=np.int32)
    scores_out = {}
    qb_idx = np.arange(nb)[:, None]
    kb_idx = np.arange(nb)[None, :]
    for h in heads:
        sc = block_scores(q, k, block, h)
        if return_scores:
            scores_out[h] = sc
        if topk <= 0:
            continue
        key = np.where(kb_idx < qb_idx, -sc, np.inf)      # ascending (-score), invalid last
        order = np.argsort(key, axis=1, kind="stable")    # stable: equal keys keep kb order
        for qb in range(nb):
            n = min(qb, topk)
            chosen = np.sort(order[qb, :n])
            sel[h, qb, :n] = chosen
    if return_scores:
        return sel, scores_out
    return sel
