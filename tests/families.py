"""Brute-force definitions of the mask families, written from what each family means (who may
attend to whom), not from the four-vector encoding.  Used to pin both the encodings in
``workloads.masks`` and the oracle's ``dense_mask``.  True = masked."""

import numpy as np


def _ij(n, nq=None):
    nq = n if nq is None else nq
    i = np.arange(nq)[:, None]
    j = np.arange(n)[None, :]
    return i, j


def causal(n):
    i, j = _ij(n)
    return j > i


def sliding_window(n, w):
    # row i sees the w most recent keys, itself included
    i, j = _ij(n)
    return ~((j <= i) & (j > i - w))


def document(n, lengths):
    doc = np.repeat(np.arange(len(lengths)), lengths)
    i, j = _ij(n)
    same = doc[i] == doc[j]
    return ~(same & (j <= i))


def prefix_lm(n, prefix):
    i, j = _ij(n)
    visible = (j < prefix) | (j <= i)
    return ~visible


def share_question(n, q_len, answers):
    seg = np.concatenate([np.zeros(q_len, dtype=int)] +
                         [np.full(a, k + 1) for k, a in enumerate(answers)])
    i, j = _ij(n)
    # question keys: visible to every later row (question rows causally, all answers);
    # answer keys: visible only inside the same answer, causally.
    vis_question_key = (seg[j] == 0) & (j <= i)
    vis_answer_key = (seg[j] > 0) & (seg[i] == seg[j]) & (j <= i)
    return ~(vis_question_key | vis_answer_key)


def block_sparse(n, starts, ends, block=128):
    i, j = _ij(n)
    b = j // block
    hole = (i >= starts[b]) & (i < ends[b])
    return (j > i) | hole


def unmasked_closed_form(family, n, **p):
    """Closed-form count of unmasked entries per head."""
    if family == "causal":
        return n * (n + 1) // 2
    if family == "sliding_window":
        w = p["w"]
        return w * (n - w) + w * (w + 1) // 2
    if family == "document":
        return int(sum(L * (L + 1) // 2 for L in p["lengths"]))
    if family == "prefix_lm":
        P = p["prefix"]
        return P * n + (n - P) * (n - P + 1) // 2
    if family == "share_question":
        Q = p["q_len"]
        return Q * n - Q * (Q - 1) // 2 + int(sum(a * (a + 1) // 2 for a in p["answers"]))
    if family == "block_sparse":
        starts, ends, block = p["starts"], p["ends"], p.get("block", 128)
        sizes = np.minimum(block, n - block * np.arange(len(starts)))
        return n * (n + 1) // 2 - int(np.sum(sizes * (np.asarray(ends) - np.asarray(starts))))
    raise ValueError(family)
