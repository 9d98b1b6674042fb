"""Plain, slow, float64 CPU oracle for FlashMask-style mask-aware attention.

TEST INFRASTRUCTURE ONLY: imported by tests, by the smoke check and by the benchmark's CPU
baseline.  It shares no code with the HIP library and never calls it.

Sources (cited by page title and paragraph):
  [abstract]  "FlashMask-3: Efficient and Expressive Mask-Aware Distributed Attention", the
              paper's abstract (acceptodds.com).
  [explainer] "FlashMask-3 sends each GPU its mask without sending any mask -- Four-vector
              sparse attention masks" (learnaivisually.com): the four-vector paragraph (keys
              as avenues, query rows as street numbers), the clip-shift-max paragraph (with
              Theorem 1), the tile-classification paragraph, the byte-arithmetic paragraph.

Every floating-point function works in float64 on inputs upcast from whatever dtype the caller
holds (bf16 or fp32 values are represented exactly).  Where the pages leave a step open the
reading taken is stated in the function's docstring.

Parity pins: every function here is pinned by tests marked "not gpu" against closed forms,
brute-force family definitions, library routines (torch SDPA / autograd in fp64) and finite
differences; none is "parity unpinned".
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# --------------------------------------------------------------------------------------------
# the mask
# --------------------------------------------------------------------------------------------


def dense_mask(LTS, LTE, UTS, UTE, rows) -> np.ndarray:
    """Dense boolean mask (True = masked) of the given query rows against every key column.

    [explainer, four-vector paragraph; abstract]: the vectors are indexed by key position and
    hold query-row boundaries; each key has at most two closed stretches, one below the diagonal
    (LTS..LTE) and one above it (UTS..UTE).  Reading: the stretches are half-open, so row i is
    masked for key j iff LTS[j] <= i < LTE[j] or UTS[j] <= i < UTE[j]; a stretch whose start is
    not below its end is empty.  Shape: [len(rows), len(LTS)].
    """
    i = np.asarray(rows, dtype=np.int64)[:, None]
    lts, lte, uts, ute = (np.asarray(x, dtype=np.int64)[None, :] for x in (LTS, LTE, UTS, UTE))
    return ((lts <= i) & (i < lte)) | ((uts <= i) & (i < ute))


def unmasked_count(LTS, LTE, UTS, UTE, nq: int) -> int:
    """Number of unmasked (i, j) entries over rows [0, nq): the union of the two closed stretches
    of each key, clipped to [0, nq), is subtracted from nq (plain interval arithmetic on the
    definition in ``dense_mask``)."""
    def clip(a):
        return np.clip(np.asarray(a, dtype=np.int64), 0, nq)
    a1, b1, a2, b2 = clip(LTS), clip(LTE), clip(UTS), clip(UTE)
    len1 = np.maximum(b1 - a1, 0)
    len2 = np.maximum(b2 - a2, 0)
    inter = np.maximum(np.minimum(b1, b2) - np.maximum(a1, a2), 0)
    inter = np.where((len1 > 0) & (len2 > 0), inter, 0)
    masked = len1 + len2 - inter
    return int(nq * len(a1) - masked.sum())


def mask_storage_bytes(n: int, dense_bytes_per_entry: int = 1, vector_bytes: int = 4):
    """Bytes of a dense n x n mask versus the four length-n boundary vectors
    ([explainer, byte-arithmetic paragraph], one byte per dense entry and four bytes per number
    as the explainer assumes)."""
    dense = n * n * dense_bytes_per_entry
    vec = 4 * n * vector_bytes
    return dense, vec


# --------------------------------------------------------------------------------------------
# attention forward / backward (the plain definition, row by row)
# --------------------------------------------------------------------------------------------


def _f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def fwd_rows(q, K, V, masked, scale):
    """Masked softmax attention for a set of query rows of one (batch, head).

    q: [r, d]; K, V: [nk, d]; masked: [r, nk] bool (True = masked); scale: softmax scale.
    Returns O [r, d] and LSE [r] (natural log, scale included).

    Definition: S = scale * q K^T, with masked entries set to -inf; LSE_i = log sum_j exp(S_ij);
    P = exp(S - LSE); O = P V.  Reading where the pages are silent: a row whose every entry is
    masked has O = 0 and LSE = -inf.
    """
    q, K, V = _f64(q), _f64(K), _f64(V)
    S = float(scale) * (q @ K.T)
    S = np.where(masked, -np.inf, S)
    m = S.max(axis=1)
    live = np.isfinite(m)
    O = np.zeros((q.shape[0], V.shape[1]))
    LSE = np.full(q.shape[0], -np.inf)
    if live.any():
        Sl = S[live]
        ml = m[live]
        LSE[live] = ml + np.log(np.exp(Sl - ml[:, None]).sum(axis=1))
        P = np.exp(Sl - LSE[live][:, None])
        O[live] = P @ V
    return O, LSE


def bwd_rows(q, K, V, dO, masked, scale, cols=None):
    """Gradients of L = sum(O * dO) for a set of query rows of one (batch, head).

    Returns dq [r, d] (complete for these rows) and the contribution of these rows to dK and dV
    ([nk, d], or [len(cols), d] when ``cols`` selects key columns).  Summing the contributions of
    every row gives the full dK and dV; rows whose mask row is all masked at ``cols`` contribute
    exactly zero there.

    Definition (exact gradient of masked softmax attention, using this oracle's own O and LSE):
      P = exp(S - LSE) (0 where masked and on fully masked rows); dV = P^T dO; dP = dO V^T;
      D_i = sum_d dO_id O_id; dS = P * (dP - D); dQ = scale dS K; dK = scale dS^T Q.
    """
    q, K, V, dO = _f64(q), _f64(K), _f64(V), _f64(dO)
    O, LSE = fwd_rows(q, K, V, masked, scale)
    S = float(scale) * (q @ K.T)
    live = np.isfinite(LSE)
    P = np.zeros_like(S)
    P[live] = np.exp(np.where(masked[live], -np.inf, S[live]) - LSE[live][:, None])
    dP = dO @ V.T
    D = (dO * O).sum(axis=1)
    dS = P * (dP - D[:, None])
    dq = float(scale) * (dS @ K)
    if cols is None:
        dk = float(scale) * (dS.T @ q)
        dv = P.T @ dO
    else:
        cols = np.asarray(cols)
        dk = float(scale) * (dS[:, cols].T @ q)
        dv = P[:, cols].T @ dO
    return dq, dk, dv


def _blocks(n, size):
    return [(s, min(s + size, n)) for s in range(0, n, size)]


def attention_fwd(Q, K, V, vectors, scale, row_block: int = 256, workers: int = 1,
                  rows=None):
    """O [B,H,nq,d] and LSE [B,H,nq] for Q [B,H,nq,d], K/V [B,H,nk,d] and one mask (four
    vectors of length nk, shared by every batch and head).  Row blocks are independent.

    ``rows`` (optional) gives the mask-row index of each query row (default 0..nq-1); the
    context-parallel check passes global row numbers here together with the global vectors.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B, H, nq, d = Q.shape
    rows = np.arange(nq) if rows is None else np.asarray(rows)
    O = np.zeros((B, H, nq, V.shape[-1]))
    LSE = np.zeros((B, H, nq))
    jobs = [(b, h, r0, r1) for b in range(B) for h in range(H) for r0, r1 in _blocks(nq, row_block)]

    def run(job):
        b, h, r0, r1 = job
        m = dense_mask(*vectors, rows[r0:r1])
        O[b, h, r0:r1], LSE[b, h, r0:r1] = fwd_rows(Q[b, h, r0:r1], K[b, h], V[b, h], m, scale)

    _run_jobs(run, jobs, workers)
    return O, LSE


def attention_bwd(Q, K, V, dO, vectors, scale, row_block: int = 256, workers: int = 1,
                  rows=None):
    """dQ, dK, dV for the same shapes as ``attention_fwd`` (dO like Q)."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    B, H, nq, d = Q.shape
    nk = K.shape[2]
    rows = np.arange(nq) if rows is None else np.asarray(rows)
    dQ = np.zeros_like(Q)
    blocks = _blocks(nq, row_block)
    parts = {}
    jobs = [(b, h, i) for b in range(B) for h in range(H) for i in range(len(blocks))]

    def run(job):
        b, h, i = job
        r0, r1 = blocks[i]
        m = dense_mask(*vectors, rows[r0:r1])
        dq, dk, dv = bwd_rows(Q[b, h, r0:r1], K[b, h], V[b, h], dO[b, h, r0:r1], m, scale)
        dQ[b, h, r0:r1] = dq
        parts[job] = (dk, dv)

    _run_jobs(run, jobs, workers)
    dK = np.zeros((B, H, nk, d))
    dV = np.zeros((B, H, nk, V.shape[-1]))
    for (b, h, _i), (dk, dv) in sorted(parts.items()):
        dK[b, h] += dk
        dV[b, h] += dv
    return dQ, dK, dV


def _run_jobs(fn, jobs, workers):
    if workers <= 1:
        for j in jobs:
            fn(j)
        return
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(fn, jobs))


# --------------------------------------------------------------------------------------------
# tile classification
# --------------------------------------------------------------------------------------------


def block_minmax(vec, BN: int):
    """Per key block b (keys [b*BN, min((b+1)*BN, nk))): the minimum and the maximum of the
    vector over that block only (the explainer's tile-classification paragraph reduces each
    vector to its extremes over the keys of a block).  Returns (mins, maxs) as int64 arrays of length ceil(nk/BN)."""
    v = np.asarray(vec, dtype=np.int64)
    nk = v.shape[0]
    n_kb = -(-nk // BN)
    mins = np.array([v[b * BN:min((b + 1) * BN, nk)].min() for b in range(n_kb)], dtype=np.int64)
    maxs = np.array([v[b * BN:min((b + 1) * BN, nk)].max() for b in range(n_kb)], dtype=np.int64)
    return mins, maxs


def classify(LTS, LTE, UTS, UTE, nq: int, BM: int, BN: int):
    """Sort every (query block, key block) tile as fully masked (0), partly masked (1) or
    unmasked (2) from the per-key-block min/max of the four vectors, and list the tiles that are
    not fully masked ([explainer, tile-classification paragraph]).

    Reading of the rule (the pages give it in words only): for rows [r0, r1) of the query block,
      a stretch [S, E) covers every row of the tile for every key of the block when
          max S <= r0 and min E >= r1;
      it misses every row of the tile for every key of the block when
          max E <= r0 or min S >= r1.
    The tile is fully masked if either stretch covers it; unmasked if both stretches miss it;
    partly masked otherwise.  This is sound for arbitrary int32 vectors (class 0 implies every
    entry masked, class 2 implies none is) and may put a truly full or truly empty tile in
    class 1.

    Lists hold the tiles of class != 0 in ascending order, entry = index * 2 + (class == 1):
    ``qlist[qb]`` over key blocks (forward orientation), ``klist[kb]`` over query blocks
    (backward orientation).  Returns dict(cls [n_qb, n_kb] uint8, qcnt, qlist, kcnt, klist) with
    the lists as Python lists of int.
    """
    nk = len(LTS)
    n_qb = -(-nq // BM)
    n_kb = -(-nk // BN)
    lts_lo, lts_hi = block_minmax(LTS, BN)
    lte_lo, lte_hi = block_minmax(LTE, BN)
    uts_lo, uts_hi = block_minmax(UTS, BN)
    ute_lo, ute_hi = block_minmax(UTE, BN)

    r0 = (np.arange(n_qb, dtype=np.int64) * BM)[:, None]
    r1 = np.minimum(r0 + BM, nq)

    lt_full = (lts_hi[None, :] <= r0) & (lte_lo[None, :] >= r1)
    ut_full = (uts_hi[None, :] <= r0) & (ute_lo[None, :] >= r1)
    lt_none = (lte_hi[None, :] <= r0) | (lts_lo[None, :] >= r1)
    ut_none = (ute_hi[None, :] <= r0) | (uts_lo[None, :] >= r1)

    cls = np.where(lt_full | ut_full, 0, np.where(lt_none & ut_none, 2, 1)).astype(np.uint8)

    qlist = [[kb * 2 + int(cls[qb, kb] == 1) for kb in range(n_kb) if cls[qb, kb] != 0]
             for qb in range(n_qb)]
    klist = [[qb * 2 + int(cls[qb, kb] == 1) for qb in range(n_qb) if cls[qb, kb] != 0]
             for kb in range(n_kb)]
    return {
        "cls": cls,
        "qcnt": np.array([len(x) for x in qlist], dtype=np.int64),
        "qlist": qlist,
        "kcnt": np.array([len(x) for x in klist], dtype=np.int64),
        "klist": klist,
    }


def prune_chunks(LTS, LTE, UTS, UTE, n_local: int, BM: int, chunk: int):
    """Which key/value chunks a context-parallel rank needs ([explainer, across-ranks
    paragraph]: the forward all-gather skips key-value chunks that are fully masked; [abstract]:
    mask-driven communication pruning).

    The vectors are the rank's localised ones (values in local row numbering, indexed by global
    key).  Reading: the same min/max tile classification as inside one GPU, with key blocks of
    `chunk` keys (the unit the all-gather moves) and query blocks of BM local rows.  Returns, per
    chunk c, the number of BM-row blocks of the rank's rows whose tile in column c is not fully
    masked (int64 [ceil(nk / chunk)]); 0 means the rank never needs chunk c.  With BM equal to the
    rank's chunk length every query block is one contiguous run of global rows, and the rule is
    then exact for the causal, document and sliding-window families.
    """
    cls = classify(LTS, LTE, UTS, UTE, n_local, BM, chunk)["cls"]
    return (cls != 0).sum(axis=0).astype(np.int64)


# --------------------------------------------------------------------------------------------
# rank-local mask: clip-shift-max
# --------------------------------------------------------------------------------------------


def localize_chunks_check(chunk_start, chunk_len, nq_global: int):
    """Validate a rank's chunk table: ascending offsets, non-empty, disjoint, inside
    [0, nq_global].  Raises ValueError otherwise."""
    o = np.asarray(chunk_start, dtype=np.int64)
    L = np.asarray(chunk_len, dtype=np.int64)
    if o.ndim != 1 or o.shape != L.shape or o.size == 0:
        raise ValueError("chunk table must be two equal-length non-empty 1-D arrays")
    if (L <= 0).any() or (o < 0).any() or (o + L > nq_global).any():
        raise ValueError("chunks must be non-empty and inside [0, nq_global]")
    if (o[1:] < o[:-1] + L[:-1]).any():
        raise ValueError("chunks must be sorted by offset and disjoint")
    return o, L


def localize(LTS, LTE, UTS, UTE, chunk_start, chunk_len, nq_global: int):
    """Rank-local boundary vectors by clip-shift-max ([abstract]; [explainer, clip-shift-max
    paragraph]).

    The rank owns the query-row chunks [o_k, o_k + L_k) (ascending), concatenated into a local
    numbering with chunk k starting at P_k = L_0 + ... + L_{k-1}.  For every mark x (each entry
    of each of the four vectors):
        clip  x to the chunk:            min(x, o_k + L_k)
        shift into the local numbering:  ... - o_k + P_k
        take the maximum over the rank's chunks, floored at 0 (the start of local numbering).
    Reading: the clip is one-sided (only the chunk's upper end), which makes the result the
    number of owned rows below x; the literal two-sided clamp breaks Theorem 1 when a rank owns
    two or more chunks.  Keys are not renumbered (the vectors stay indexed by global key).

    Returns (LTS_l, LTE_l, UTS_l, UTE_l, n_local) with int32 vectors.
    """
    o, L = localize_chunks_check(chunk_start, chunk_len, nq_global)
    P = np.concatenate([[0], np.cumsum(L)[:-1]])

    def ell(x):
        x = np.asarray(x, dtype=np.int64)
        best = np.zeros_like(x)
        for ok, Lk, Pk in zip(o, L, P):
            best = np.maximum(best, np.minimum(x, ok + Lk) - ok + Pk)
        return best.astype(np.int32)

    return ell(LTS), ell(LTE), ell(UTS), ell(UTE), int(L.sum())


# --------------------------------------------------------------------------------------------
# work counts
# --------------------------------------------------------------------------------------------


def flops(unmasked: int, d: int, B: int = 1, H: int = 1):
    """Forward and backward FLOPs counted over unmasked entries only: 4*d per entry forward
    (two matrix products), 10*d backward (five).  The pages quote "achieved TFLOPs" without a
    formula; this is the FlashAttention convention."""
    return 4 * d * B * H * unmasked, 10 * d * B * H * unmasked


__all__ = [n for n in dir() if not n.startswith("_") and n not in ("annotations", "math",
                                                                     "np", "ThreadPoolExecutor")]
