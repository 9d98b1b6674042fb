"""The five synthetic workloads (plus their sub-masks) and their seeded tensors.

Seeds: the generator for config c and stream s is ``default_rng(SeedSequence([c, s, ...]))``,
with stream 0 = mask structure, 1 = Q, 2 = K, 3 = V, 4 = dO.  Values are drawn in float32 and
rounded to the compute dtype (bf16 with round-to-nearest-even).  Q, K, V have the config's
standard deviation; the configs give none for dO, which is drawn with half of it (DO_STD_RATIO):
at the full deviation the gradient of a document's first keys (a sum over the document's rows,
dominated by its first rows) reaches 4-5.5 at the 32K workload, where bf16's own spacing of
2^-5 leaves under 0.005 of the 2e-2 max-abs bar for the arithmetic.

The pages benchmark 12 unpublished structured masks at 4K-128K on one H100 (FlashMask-3
abstract); these shapes and mask families stand in for that suite.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import masks


@dataclass(frozen=True)
class Workload:
    key: str            # short id, e.g. "c3"
    cfg: int            # config index 1..5 (seed root)
    sub: int            # sub-mask index inside the config (seed)
    name: str           # human-readable workload name
    dtype: str          # "bf16" | "fp32"
    B: int
    H: int
    nq: int             # query rows seen by the attention call (local rows for c5)
    nk: int             # key columns
    d: int
    std: float
    family: str
    params: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))


def _rng(*key):
    return np.random.default_rng(np.random.SeedSequence(list(key)))


# Context-parallel share of the 128K workload: 32 chunks of 4096, CP degree 16, dual-chunk
# assignment (rank r owns chunks r and 2R - 1 - r); rank 5 owns chunks 5 and 26.
C5_CHUNK = 4096
C5_RANK, C5_DEGREE = 5, 16
C5_CHUNKS = (C5_RANK, 2 * C5_DEGREE - 1 - C5_RANK)
C5_CHUNK_START = tuple(c * C5_CHUNK for c in C5_CHUNKS)
C5_CHUNK_LEN = (C5_CHUNK, C5_CHUNK)

WORKLOADS = {
    "c1": Workload("c1", 1, 0, "tiny fp32 causal-document n256", "fp32", 1, 2, 256, 256, 64,
                   1.0, "document_uniform", {"docs": 3}),
    "c2a": Workload("c2a", 2, 0, "n8192 causal", "bf16", 1, 16, 8192, 8192, 128, 1.0, "causal"),
    "c2b": Workload("c2b", 2, 1, "n8192 sliding-window w1024", "bf16", 1, 16, 8192, 8192, 128,
                    1.0, "sliding_window", {"w": 1024}),
    "c2c": Workload("c2c", 2, 2, "n8192 causal-document x12", "bf16", 1, 16, 8192, 8192, 128,
                    1.0, "document_uniform", {"docs": 12}),
    "c2d": Workload("c2d", 2, 3, "n8192 prefix-LM", "bf16", 1, 16, 8192, 8192, 128, 1.0,
                    "prefix_lm"),
    "c2e": Workload("c2e", 2, 4, "n8192 share-question", "bf16", 1, 16, 8192, 8192, 128, 1.0,
                    "share_question"),
    "c2f": Workload("c2f", 2, 5, "n8192 block-sparse", "bf16", 1, 16, 8192, 8192, 128, 1.0,
                    "block_sparse"),
    "c3": Workload("c3", 3, 0, "n32768 log-normal causal-document x40", "bf16", 1, 32, 32768,
                   32768, 128, 1.0, "document_lognormal", {"docs": 40}),
    # The same generator at the draw whose unmasked count is the median of draws 0..199 (29.6M
    # per head against 45.6M for draw 0, whose one 7,265-row document holds 58% of the work): a
    # sensitivity case for the benchmark; Q/K/V/dO are those of the 32K workload.
    "c3m": Workload("c3m", 3, 198, "n32768 log-normal causal-document x40, median-U draw",
                    "bf16", 1, 32, 32768, 32768, 128, 1.0, "document_lognormal", {"docs": 40}),
    "c4swa": Workload("c4swa", 4, 0, "n131072 sliding-window w4096", "bf16", 1, 8, 131072,
                      131072, 128, 0.5, "sliding_window", {"w": 4096}),
    "c4doc": Workload("c4doc", 4, 1, "n131072 causal-document x16", "bf16", 1, 8, 131072,
                      131072, 128, 0.5, "document_uniform", {"docs": 16}),
    "c5": Workload("c5", 5, 0, "CP rank 5/16 share: 8192 local rows x 131072 keys, "
                   "causal-document x24", "bf16", 1, 16, 8192, 131072, 128, 1.0,
                   "document_uniform", {"docs": 24, "global_n": 131072}),
}


def global_mask(w: Workload):
    """The four vectors of the workload's (global) mask as int32 numpy arrays."""
    n = w.params.get("global_n", w.nk)
    rng = _rng(w.cfg, 0, w.sub)
    f = w.family
    if f == "causal":
        return masks.causal(n)
    if f == "sliding_window":
        return masks.sliding_window(n, w.params["w"])
    if f == "document_uniform":
        return masks.document(n, masks.uniform_cut_lengths(rng, n, w.params["docs"]))
    if f == "document_lognormal":
        return masks.document(n, masks.lognormal_lengths(rng, n, w.params["docs"]))
    if f == "prefix_lm":
        return masks.prefix_lm(n, masks.draw_prefix(rng))
    if f == "share_question":
        q_len, ans = masks.draw_share_question(rng, n)
        return masks.share_question(n, q_len, ans)
    if f == "block_sparse":
        a, z = masks.draw_block_sparse(rng, n)
        return masks.block_sparse(n, a, z)
    raise ValueError(f)


def family_params(w: Workload):
    """The drawn family parameters (for brute-force checks and reports)."""
    n = w.params.get("global_n", w.nk)
    rng = _rng(w.cfg, 0, w.sub)
    f = w.family
    if f == "document_uniform":
        return {"lengths": masks.uniform_cut_lengths(rng, n, w.params["docs"])}
    if f == "document_lognormal":
        return {"lengths": masks.lognormal_lengths(rng, n, w.params["docs"])}
    if f == "prefix_lm":
        return {"prefix": masks.draw_prefix(rng)}
    if f == "share_question":
        q_len, ans = masks.draw_share_question(rng, n)
        return {"q_len": q_len, "answers": ans}
    if f == "block_sparse":
        a, z = masks.draw_block_sparse(rng, n)
        return {"starts": a, "ends": z}
    return dict(w.params)


def owned_rows(w: Workload):
    """Global row indices of the query rows this workload's attention call sees."""
    if w.key == "c5":
        return np.concatenate([np.arange(s, s + L) for s, L in zip(C5_CHUNK_START, C5_CHUNK_LEN)])
    return np.arange(w.nq)


def _normal(rng, shape, std):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


# standard deviation of dO relative to the config's Q/K/V deviation
DO_STD_RATIO = 0.5


def tensor_f32(w: Workload, stream: int, heads=None) -> np.ndarray:
    """One seeded input tensor as float32 [B, H, rows, d] before rounding to the compute dtype.

    stream 1 = Q, 2 = K, 3 = V, 4 = dO.  Q and dO have the call's query rows; K and V the keys.
    For the context-parallel share (c5) the query-side tensors are generated chunk by chunk from
    (cfg, stream, chunk) so that any rank can generate exactly its own rows of the global tensor.
    ``heads`` restricts to a subset of heads (same values as the full draw only for heads=None;
    the subset path is used by small CPU checks that draw their own tensors)."""
    rows = w.nk if stream in (2, 3) else w.nq
    std = w.std * (DO_STD_RATIO if stream == 4 else 1.0)
    if w.key == "c5" and stream in (1, 4):
        parts = [_normal(_rng(w.cfg, stream, c), (w.B, w.H, C5_CHUNK, w.d), std)
                 for c in C5_CHUNKS]
        x = np.concatenate(parts, axis=2)
    else:
        x = _normal(_rng(w.cfg, stream), (w.B, w.H, rows, w.d), std)
    if heads is not None:
        x = x[:, heads]
    return x


def to_compute_dtype(x_f32: np.ndarray, dtype: str):
    """Round float32 values to the compute dtype; returns a CPU torch tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "fp32":
        return t.clone()
    raise ValueError(dtype)


def tensors(w: Workload, streams=(1, 2, 3, 4)):
    """Seeded Q/K/V/dO as CPU torch tensors in the compute dtype, keyed 'q', 'k', 'v', 'do'."""
    names = {1: "q", 2: "k", 3: "v", 4: "do"}
    return {names[s]: to_compute_dtype(tensor_f32(w, s), w.dtype) for s in streams}
