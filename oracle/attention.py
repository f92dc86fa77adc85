"""Exact causal GQA softmax attention, float64, over contiguous K/V.

TEST INFRASTRUCTURE ONLY (see the package header): the GPU path never
imports this module.

What is computed (the plain definition; no blocking, fusion or reordering
beyond it):

* A query at absolute position ``p`` attends to the keys at positions
  ``0 .. p`` inclusive.  In chunked prefill a chunk starting at ``S`` with
  ``T`` tokens has its queries at ``S .. S+T-1``; each sees every earlier
  chunk and the causal part of its own chunk, which is why chunking is
  lossless ([L7] section 2.3, chunked prefill; section 9, pitfall 1).
  Decode is the same rule with one query at ``p = L-1`` over ``L`` cached
  keys ([L7] section 1.1: one new token per request per step, reading the
  whole KV).
* GQA: q-head ``h`` uses KV head ``h // G`` with ``G = Hq / Hkv``.  The
  pages only say the models are GQA ([DISAGG] "传输的代价"; [L7] section
  3); contiguous grouping is the reading taken here.
* Score ``s_j = (q . k_j) * scale``; the default scale is ``1/sqrt(D)``
  (the pages never state the scale; this is the standard reading).
* ``o = sum_j w_j v_j / sum_j w_j`` with ``w_j = exp(s_j - max_j s_j)``.

The result does not depend on how queries are batched into calls: a row's
value is a function of its own query, its position and the keys it sees.
"""

from __future__ import annotations

import numpy as np


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def attend(q, k, v, positions, scale: float | None = None, row_tile: int = 1024) -> np.ndarray:
    """Causal GQA attention rows.

    q:          [M, Hq, D]   queries (any float dtype; upcast to float64).
    k, v:       [Lk, Hkv, D] the request's keys / values in position order.
    positions:  [M] int      absolute position of each query row; row m sees
                             keys ``0 .. positions[m]`` (must be < Lk).
    scale:      softmax scale, default ``1/sqrt(D)``.
    row_tile:   rows per GEMM (a memory bound only; results do not depend
                on it).

    Returns [M, Hq, D] float64.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    positions = np.asarray(positions, dtype=np.int64)
    m_rows, hq, d = q.shape
    lk, hkv, dk = k.shape
    if dk != d or v.shape != k.shape:
        raise ValueError("q, k, v head dims / shapes disagree")
    if hq % hkv:
        raise ValueError("q heads must be a multiple of kv heads")
    if positions.shape != (m_rows,):
        raise ValueError("one position per query row")
    if m_rows and (positions.min() < 0 or positions.max() >= lk):
        raise ValueError("a query position has no key at or before it")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    group = hq // hkv
    out = np.empty((m_rows, hq, d), dtype=np.float64)
    for h in range(hq):
        kh = k[:, h // group, :]
        vh = v[:, h // group, :]
        for r0 in range(0, m_rows, row_tile):
            pos = positions[r0:r0 + row_tile]
            nkeys = int(pos.max()) + 1
            s = (q[r0:r0 + row_tile, h, :] @ kh[:nkeys].T) * scale
            s[np.arange(nkeys)[None, :] > pos[:, None]] = -np.inf
            w = np.exp(s - s.max(axis=1, keepdims=True))
            out[r0:r0 + row_tile, h, :] = (w @ vh[:nkeys]) / w.sum(axis=1, keepdims=True)
    return out


def prefill(q, k, v, scale: float | None = None) -> np.ndarray:
    """One-shot causal prefill of an N-token prompt: rows at positions 0..N-1.

    q [N, Hq, D]; k, v [N, Hkv, D].  A chunk ``[S, S+T)`` of a chunked
    prefill must equal rows ``S .. S+T-1`` of this result ([L7] 2.3).
    """
    n = np.asarray(q).shape[0]
    return attend(q, k, v, np.arange(n), scale)


def prefill_chunk(q_chunk, k, v, start: int, scale: float | None = None) -> np.ndarray:
    """Rows of one chunk: queries at ``start .. start+T-1`` over keys ``[0, start+T)``.

    ``k``/``v`` need hold at least ``start+T`` positions; later keys are
    never looked at.
    """
    t = np.asarray(q_chunk).shape[0]
    return attend(q_chunk, k, v, start + np.arange(t), scale)


def decode(q, k, v, scale: float | None = None) -> np.ndarray:
    """One decode query per request: q [Hq, D] at position L-1 over k, v [L, Hkv, D].

    Returns [Hq, D] float64.
    """
    q = _as_f64(q)
    lk = np.asarray(k).shape[0]
    return attend(q[None], k, v, np.array([lk - 1]), scale)[0]


def decode_batch(q, ks, vs, scale: float | None = None) -> np.ndarray:
    """Decode for a batch: q [B, Hq, D]; ks[b], vs[b] are [L_b, Hkv, D]."""
    q = _as_f64(q)
    return np.stack([decode(q[b], ks[b], vs[b], scale) for b in range(q.shape[0])])


def error_metrics(got, ref) -> dict:
    """max |got - ref| and ||got - ref||_2 / ||ref||_2 (both in float64)."""
    got = _as_f64(got)
    ref = _as_f64(ref)
    diff = got - ref
    denom = float(np.linalg.norm(ref.ravel()))
    return {
        "max_abs": float(np.abs(diff).max()) if diff.size else 0.0,
        "rel_l2": float(np.linalg.norm(diff.ravel()) / denom) if denom > 0 else float(np.linalg.norm(diff.ravel())),
    }
