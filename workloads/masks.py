"""Mask families encoded as the column-wise sparse mask, plus the seeded draws of their parameters.

Encoding (FlashMask-3 explainer, "four vectors" paragraph; FlashMask-3 abstract): for every key
column j the four int32 numbers LTS[j], LTE[j], UTS[j], UTE[j] give at most two stretches of
query rows that are closed to that key.  Stretches are half-open: row i is masked for key j iff
LTS[j] <= i < LTE[j] or UTS[j] <= i < UTE[j].  An empty stretch is written canonically as
LT = (nq, nq) and UT = (0, 0).

The families are the ones the pages list (abstract: document, prefix-LM, share-question,
sliding-window, block-sparse; plus plain causal).  Their parameters are drawn from numpy
``default_rng`` generators that the caller seeds.  Nothing here evaluates a mask: the brute-force
definitions that check these encodings live in the tests.
"""

from __future__ import annotations

import numpy as np

I32 = np.int32


def _empty(n: int, nq: int | None = None):
    nq = n if nq is None else nq
    LTS = np.full(n, nq, dtype=np.int64)
    LTE = np.full(n, nq, dtype=np.int64)
    UTS = np.zeros(n, dtype=np.int64)
    UTE = np.zeros(n, dtype=np.int64)
    return LTS, LTE, UTS, UTE


def _pack(LTS, LTE, UTS, UTE):
    return tuple(np.ascontiguousarray(x, dtype=I32) for x in (LTS, LTE, UTS, UTE))


# --------------------------------------------------------------------------------------------
# encodings (deterministic given the family parameters)
# --------------------------------------------------------------------------------------------

def no_mask(n: int, nq: int | None = None):
    """Every stretch empty: plain (bidirectional) attention."""
    return _pack(*_empty(n, nq))


def causal(n: int):
    """Row i sees keys j <= i: the stretch above the diagonal is rows [0, j)."""
    LTS, LTE, UTS, UTE = _empty(n)
    UTE[:] = np.arange(n)
    return _pack(LTS, LTE, UTS, UTE)


def sliding_window(n: int, w: int):
    """Causal window of w keys: row i sees keys j with i - w < j <= i.

    Below the diagonal the closed stretch is rows [min(j + w, n), n)."""
    j = np.arange(n, dtype=np.int64)
    LTS = np.minimum(j + w, n)
    LTE = np.full(n, n, dtype=np.int64)
    UTS = np.zeros(n, dtype=np.int64)
    UTE = j.copy()
    return _pack(LTS, LTE, UTS, UTE)


def document(n: int, lengths):
    """Causal attention inside each document; documents are consecutive and cover [0, n).

    For key j in document [s, e): rows [e, n) (later documents) and rows [0, j) are closed."""
    lengths = np.asarray(lengths, dtype=np.int64)
    assert lengths.min() >= 1 and lengths.sum() == n
    ends = np.cumsum(lengths)
    doc_end = np.repeat(ends, lengths)
    j = np.arange(n, dtype=np.int64)
    return _pack(doc_end, np.full(n, n), np.zeros(n, dtype=np.int64), j)


def prefix_lm(n: int, prefix: int):
    """Bidirectional inside the prefix [0, P), causal after it; every row sees the whole prefix."""
    LTS, LTE, UTS, UTE = _empty(n)
    j = np.arange(n, dtype=np.int64)
    UTE[:] = np.where(j >= prefix, j, 0)
    return _pack(LTS, LTE, UTS, UTE)


def share_question(n: int, q_len: int, answer_lengths):
    """One question [0, Q) followed by answers that fill the rest of the sequence.

    The question attends causally to itself; each answer attends to the whole question and
    causally to itself, never to another answer."""
    answer_lengths = np.asarray(answer_lengths, dtype=np.int64)
    assert answer_lengths.min() >= 1 and q_len + answer_lengths.sum() == n
    LTS, LTE, UTS, UTE = _empty(n)
    j = np.arange(n, dtype=np.int64)
    UTE[:] = j
    ends = q_len + np.cumsum(answer_lengths)
    LTS[q_len:] = np.repeat(ends, answer_lengths)
    LTE[q_len:] = n
    return _pack(LTS, LTE, UTS, UTE)


def block_sparse(n: int, starts, ends, block: int = 128):
    """Causal plus, for every block of ``block`` keys, one closed stretch [a_b, z_b) of rows
    below the diagonal shared by all keys of that block.  An empty stretch is stored as (n, n)."""
    starts = np.asarray(starts, dtype=np.int64)
    ends = np.asarray(ends, dtype=np.int64)
    n_blk = -(-n // block)
    assert starts.shape == (n_blk,) and ends.shape == (n_blk,)
    j = np.arange(n, dtype=np.int64)
    b = j // block
    a = starts[b]
    z = ends[b]
    empty = a >= z
    LTS = np.where(empty, n, a)
    LTE = np.where(empty, n, z)
    return _pack(LTS, LTE, np.zeros(n, dtype=np.int64), j)


# --------------------------------------------------------------------------------------------
# seeded parameter draws
# --------------------------------------------------------------------------------------------

def uniform_cut_lengths(rng: np.random.Generator, n: int, k: int):
    """k lengths summing to n: k - 1 distinct cut points drawn uniformly from {1, ..., n - 1}."""
    if k == 1:
        return np.array([n], dtype=np.int64)
    cuts = np.sort(rng.choice(np.arange(1, n), size=k - 1, replace=False))
    return np.diff(np.concatenate([[0], cuts, [n]])).astype(np.int64)


def lognormal_lengths(rng: np.random.Generator, n: int, k: int, median: float = 512.0,
                      sigma: float = 1.0, max_len: int = 8192):
    """k document lengths summing to n with a log-normal shape (median ``median``, tail clipped
    at ``max_len``).  Draws are clipped to [1, max_len], scaled to sum to n and floored; the
    remainder goes to the longest document, and anything that pushes it past ``max_len`` is
    handed to the shortest documents."""
    raw = rng.lognormal(mean=np.log(median), sigma=sigma, size=k)
    raw = np.clip(raw, 1.0, float(max_len))
    lens = np.maximum(np.floor(raw * (n / raw.sum())).astype(np.int64), 1)
    rem = n - int(lens.sum())
    big = int(np.argmax(lens))
    lens[big] += rem
    excess = int(lens[big]) - max_len
    if excess > 0:
        lens[big] = max_len
        while excess > 0:
            i = int(np.argmin(lens))
            give = min(excess, max_len - int(lens[i]))
            lens[i] += give
            excess -= give
    assert lens.sum() == n and lens.min() >= 1 and lens.max() <= max_len
    return lens


def draw_prefix(rng: np.random.Generator, lo: int = 1024, hi: int = 4096) -> int:
    return int(rng.integers(lo, hi, endpoint=True))


def draw_share_question(rng: np.random.Generator, n: int, n_answers: int = 4,
                        q_lo: int = 512, q_hi: int = 2048):
    q_len = int(rng.integers(q_lo, q_hi, endpoint=True))
    return q_len, uniform_cut_lengths(rng, n - q_len, n_answers)


def draw_block_sparse(rng: np.random.Generator, n: int, block: int = 128):
    """For block b: a_b uniform on [block*(b+1), n], z_b uniform on [a_b, n]."""
    n_blk = -(-n // block)
    a = np.empty(n_blk, dtype=np.int64)
    z = np.empty(n_blk, dtype=np.int64)
    for b in range(n_blk):
        lo = min(block * (b + 1), n)
        a[b] = rng.integers(lo, n, endpoint=True)
        z[b] = rng.integers(a[b], n, endpoint=True)
    return a, z


def random_vectors(rng: np.random.Generator, nk: int, nq: int, spread: int = 0):
    """Arbitrary int32 vectors (no structure): stretch ends drawn on [-spread, nq + spread],
    in either order, so empty, reversed and out-of-range stretches all occur."""
    lo, hi = -spread, nq + spread
    return _pack(*(rng.integers(lo, hi, size=nk, endpoint=True) for _ in range(4)))
