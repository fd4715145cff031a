"""CPU oracle for the TriAttention KV-cache eviction pass.  TEST INFRASTRUCTURE ONLY.

Only the test-suite, the package's smoke check and the CPU-baseline leg of the
benchmark may import this module.  The GPU path never calls it and shares no
code with it.  Everything here is plain float64 NumPy, one (layer, sequence,
KV head) unit at a time, written to be checked by eye against the pages.

Sources (cited by title and section):
  [S] "TriAttention：基于三角函数 KV 压缩的高效长推理" (paper summary page)
  [C] "WeianMao/triattention" (project card page), section "How it works"
  [N] "TriAttention助力：单张RTX 4090跑通32B大模型…" (news page)

What the pass computes, in the pages' order ([S] 流程详解 steps 2-5; [C] How it works):
  * score every cached key by a trigonometric series in the distance between the
    key's position and future query positions, built from the pre-rotation query
    centre of each head, plus a norm-weighting term ([S] steps 2 and 3);
  * keep the highest-scoring keys up to a budget and evict the rest ([S] step 4);
  * later attention reads the compacted cache ([S] step 5).

The pages never write the score out.  The definition used here (a reading,
listed with the others in the design notes) is, for one unit with stored
post-rotation keys K[p], query-centre group qbar[g] (g < G, the query heads of
this KV head), norm coefficients c[g, i], offsets D and decode position t:

  s(p) = (1/G) sum_g [ (1/|D|) sum_{Delta in D} RoPE(qbar_g, t + Delta) . K[p]
                       + sum_i c[g, i] * |z_i(K[p])| ]

with z_i(x) the i-th rotary pair as a complex number and RoPE(x, n) multiplying
z_i by exp(1j * n * omega_i), omega_i = theta^(-2i/d).  Written through the
pre-rotation key k = RoPE(K[p], -pos[p]) the first term is the series
|z_i(qbar)| |z_i(k)| cos(omega_i (t + Delta - pos[p]) + arg z_i(qbar) - arg z_i(k))
summed over pairs: sinusoids of the query-key distance ([S] step 2, [C]).

Parity pins for every function live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math
from typing import Sequence

import numpy as np

__all__ = [
    "frequencies", "to_pairs", "from_pairs", "rotate", "group_rows",
    "score", "score_trig_series", "score_collapsed", "centre_vector", "abs_terms",
    "rank_values", "select", "select_bruteforce", "compact", "paged_tables",
    "boundary_set", "evict_unit", "logical_unit", "calibration_stats", "decode_attention",
    "score_variant", "abs_terms_variant",
]


# --------------------------------------------------------------------------- rotary pairs

def frequencies(d: int, theta: float) -> np.ndarray:
    """omega_i = theta^(-2i/d), i = 0 .. d/2-1 (float64): the rotary frequencies whose
    sinusoids make up the distance series ([S] 流程详解 step 2)."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / d)


def to_pairs(x: np.ndarray, rope: str = "half") -> np.ndarray:
    """Rotary pairs of the last axis as complex numbers.

    "half": pair i is (x[i], x[i + d/2]) (the rotate-half layout of Qwen-family models);
    "interleaved": pair i is (x[2i], x[2i+1]).
    """
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    if rope == "half":
        return x[..., :h] + 1j * x[..., h:]
    if rope == "interleaved":
        return x[..., 0::2] + 1j * x[..., 1::2]
    raise ValueError(rope)


def from_pairs(z: np.ndarray, rope: str = "half") -> np.ndarray:
    """Inverse of to_pairs."""
    if rope == "half":
        return np.concatenate([z.real, z.imag], axis=-1)
    if rope == "interleaved":
        return np.stack([z.real, z.imag], axis=-1).reshape(z.shape[:-1] + (2 * z.shape[-1],))
    raise ValueError(rope)


def rotate(x: np.ndarray, n, theta: float, rope: str = "half") -> np.ndarray:
    """RoPE(x, n): every pair z_i(x) times exp(1j * n * omega_i), angles formed in float64.

    x [..., d]; n a scalar position or an array broadcasting against x's leading axes.
    """
    x = np.asarray(x, dtype=np.float64)
    w = frequencies(x.shape[-1], theta)
    ang = np.asarray(n, dtype=np.float64)[..., None] * w
    return from_pairs(to_pairs(x, rope) * np.exp(1j * ang), rope)


def group_rows(per_query_head: np.ndarray, h: int, G: int) -> np.ndarray:
    """Rows of the G query heads that share KV head h (query head hq belongs to KV head hq // G)."""
    return per_query_head[h * G:(h + 1) * G]


# --------------------------------------------------------------------------- score (step a2)

def score(K, qbar, c, theta, offsets: Sequence[int], t: int, rope: str = "half") -> np.ndarray:
    """Score of every key: the plain definition (module docstring), float64.

    K [L, d] stored post-rotation keys; qbar [G, d] query centres of the group; c [G, d/2]
    norm coefficients; offsets the future offsets Delta; t the decode position.
    The distance part averages the rotary logit of every query centre placed at every
    future position t + Delta ([S] 流程详解 step 2); the norm part weights each key pair's
    magnitude ([S] 流程详解 step 3); query heads of a group are averaged.
    """
    K = np.asarray(K, dtype=np.float64)
    qbar = np.asarray(qbar, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    G = qbar.shape[0]
    # every (query head, future position) rotated centre, one row each
    Q = np.stack([rotate(qbar[g], t + dl, theta, rope) for g in range(G) for dl in offsets])
    distance_part = (K @ Q.T).reshape(K.shape[0], G, len(offsets)).mean(axis=2).mean(axis=1)
    norms = np.abs(to_pairs(K, rope))                      # [L, d/2]
    norm_part = (norms @ c.T).mean(axis=1)                 # mean over the G heads
    return distance_part + norm_part


def score_trig_series(K, pos, qbar, c, theta, offsets, t, rope: str = "half") -> np.ndarray:
    """The same score written as the pages frame it: a sum of sinusoids of the distance
    t + Delta - pos[p] with amplitudes |z_i(qbar)||z_i(k)| and phases arg z_i(qbar) - arg z_i(k),
    where k = RoPE(K[p], -pos[p]) is the pre-rotation key ([S] 流程详解 step 2, [C] How it works),
    plus the norm weighting of the pre-rotation key pairs ([S] step 3).  Float64, small inputs."""
    K = np.asarray(K, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.float64)
    qbar = np.asarray(qbar, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    w = frequencies(K.shape[-1], theta)
    k_pre = rotate(K, -pos, theta, rope)                   # undo the rotation each key was stored with
    zk = to_pairs(k_pre, rope)                             # [L, d/2]
    zq = to_pairs(qbar, rope)                              # [G, d/2]
    amp = np.abs(zq)[:, None, :] * np.abs(zk)[None, :, :]  # [G, L, d/2]
    phase = np.angle(zq)[:, None, :] - np.angle(zk)[None, :, :]
    series = np.zeros(K.shape[0])
    for dl in offsets:
        dist = (t + dl) - pos                              # [L]
        series += (amp * np.cos(dist[None, :, None] * w + phase)).sum(axis=2).mean(axis=0)
    series /= len(offsets)
    norm_part = (np.abs(zk) @ c.T).mean(axis=1)
    return series + norm_part


def centre_vector(qbar, theta, offsets, rope: str = "half") -> np.ndarray:
    """u = mean over the group's heads g and offsets Delta of RoPE(qbar_g, Delta), float64 [d]."""
    qbar = np.asarray(qbar, dtype=np.float64)
    return np.mean([rotate(qbar[g], dl, theta, rope) for g in range(qbar.shape[0]) for dl in offsets], axis=0)


def score_collapsed(K, qbar, c, theta, offsets, t, rope: str = "half") -> np.ndarray:
    """The same score, collapsed: because the distance part is linear in the key it equals
    w . K[p] with w = RoPE(u, t), u = centre_vector(...); the norm part equals
    chat . |z(K[p])| with chat the group mean of c.  Float64; a cross-check of `score`."""
    K = np.asarray(K, dtype=np.float64)
    w = rotate(centre_vector(qbar, theta, offsets, rope), t, theta, rope)
    chat = np.asarray(c, dtype=np.float64).mean(axis=0)
    return K @ w + np.abs(to_pairs(K, rope)) @ chat


def abs_terms(K, qbar, c, theta, offsets, t, rope: str = "half") -> np.ndarray:
    """A(p) = sum_j |w_j K_j[p]| + sum_i |chat_i| |z_i(K[p])| >= |s(p)|: the size of the terms a
    float32 evaluation of the collapsed form sums, used to scale score tolerances."""
    K = np.asarray(K, dtype=np.float64)
    w = rotate(centre_vector(qbar, theta, offsets, rope), t, theta, rope)
    chat = np.asarray(c, dtype=np.float64).mean(axis=0)
    return np.abs(K * w).sum(axis=1) + np.abs(to_pairs(K, rope)) @ np.abs(chat)


# --------------------------------------------------------------------------- selection (step a3)

def rank_values(s) -> np.ndarray:
    """Values used for ranking: NaN ranks as -inf and -0 as +0 (float64)."""
    s = np.asarray(s, dtype=np.float64)
    s = np.where(np.isnan(s), -np.inf, s)
    return s + 0.0                                         # -0 + 0 = +0


def select(scores, pos, budget: int, recent: int) -> np.ndarray:
    """Slots kept for one unit, ascending ([S] 流程详解 step 4: keep the most important keys,
    evict the rest).

    If L <= budget every slot stays.  Otherwise the last `recent` slots are always kept and the
    remaining budget - recent places go to the best of slots 0 .. L-recent-1, ordered by score
    (higher first) and then by position (lower first).  Result int64 [min(L, budget)].
    """
    if not (0 <= recent <= budget and budget >= 1):
        raise ValueError("need 0 <= recent <= budget and budget >= 1")
    s = rank_values(scores)
    pos = np.asarray(pos, dtype=np.int64)
    L = s.shape[0]
    if L <= budget:
        return np.arange(L, dtype=np.int64)
    n_cand = L - recent
    order = np.lexsort((pos[:n_cand], -s[:n_cand]))      # primary: score descending; then position
    chosen = order[:budget - recent]
    return np.sort(np.concatenate([chosen, np.arange(n_cand, L)])).astype(np.int64)


def select_bruteforce(scores, pos, budget: int, recent: int) -> np.ndarray:
    """Same contract as `select`, by a plain Python stable sort (small inputs only)."""
    s = list(rank_values(scores))
    L = len(s)
    if L <= budget:
        return np.arange(L, dtype=np.int64)
    cand = sorted(range(L - recent), key=lambda p: (-s[p], int(pos[p])))
    return np.array(sorted(cand[:budget - recent] + list(range(L - recent, L))), dtype=np.int64)


def boundary_set(ref_scores, A, budget: int, recent: int, rel_tol: float) -> np.ndarray:
    """Candidate slots whose reference score lies within rel_tol * A(p) of the threshold score
    (the (budget-recent)-th best candidate): their membership may legitimately differ between
    two evaluations whose scores differ by less than that tolerance.  Empty when L <= budget."""
    s = rank_values(ref_scores)
    L = s.shape[0]
    if L <= budget or budget == recent:
        return np.zeros(0, dtype=np.int64)
    cand = s[:L - recent]
    tau = np.sort(cand)[::-1][budget - recent - 1]
    return np.nonzero(np.abs(cand - tau) <= rel_tol * np.asarray(A)[:L - recent])[0].astype(np.int64)


# --------------------------------------------------------------------------- compaction (step a4)

def compact(K, V, pos, keep):
    """Retained rows moved to the front in slot order ([S] 流程详解 step 5: later attention reads
    the compressed cache): row j of the result is row keep[j] of the input, bit for bit."""
    keep = np.asarray(keep, dtype=np.int64)
    return np.asarray(K)[keep], np.asarray(V)[keep], np.asarray(pos)[keep]


def paged_tables(table_row, L: int, L_new: int, block_size: int):
    """Paged cache: after compaction a sequence's first ceil(L_new/bs) blocks hold its slots; the
    blocks after them, up to ceil(L/bs), are freed in logical order.  Returns (new_row, freed)."""
    n_old = -(-L // block_size)
    n_new = -(-L_new // block_size)
    row = np.asarray(table_row)
    return row[:n_new].copy(), row[n_new:n_old].copy()


def logical_unit(pool, table_row, L: int, h: int, block_size: int) -> np.ndarray:
    """Rows 0..L-1 of KV head h of one sequence, gathered through its block table.

    pool [num_blocks, block_size, H_kv, ...]; returns [L, ...]."""
    s = np.arange(L)
    blocks = np.asarray(table_row)[s // block_size]
    return np.asarray(pool)[blocks, s % block_size, h]


# --------------------------------------------------------------------------- one unit end to end

def evict_unit(K, V, pos, qbar, c, theta, offsets, t, budget, recent, rope: str = "half") -> dict:
    """The whole pass for one (layer, sequence, KV head): score, select, compact."""
    s = score(K, qbar, c, theta, offsets, t, rope)
    keep = select(s, pos, budget, recent)
    k2, v2, p2 = compact(K, V, pos, keep)
    return {"scores": s, "keep": keep, "k": k2, "v": v2, "pos": p2, "new_len": int(keep.shape[0])}


# --------------------------------------------------------------------------- calibration statistics

def calibration_stats(Q, rope: str = "half"):
    """Query centre and norm coefficients of one (layer, query head) from its calibration queries:
    the centre is the mean pre-rotation query ([S] 流程详解 step 1, centres measured on a calibration
    set; 核心洞见: pre-rotation queries concentrate around it), and c_i is the pair-norm mass the centre
    misses, mean_n |z_i(q_n)| - |z_i(qbar)| (the norm weighting of [S] step 3; >= 0 by the triangle
    inequality).  Q [n, d] pre-rotation queries; returns (qbar [d], c [d/2]), float64."""
    Q = np.asarray(Q, dtype=np.float64)
    qbar = Q.mean(axis=0)
    c = np.abs(to_pairs(Q, rope)).mean(axis=0) - np.abs(to_pairs(qbar, rope))
    return qbar, c


# --------------------------------------------------------------------------- decode attention over the kept cache

def decode_attention(q, K, V, scale: float) -> np.ndarray:
    """One decode step of attention over a compacted unit ([S] 流程详解 step 5: inference reads the
    compressed cache): for each query row g, softmax over the kept keys of scale * q_g . K[p], applied
    to V.  q [G, d] post-rotation queries of the KV head's query group; K, V [L, d] (L >= 1).
    Float64; the softmax subtracts the row maximum before exponentiating."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    s = scale * (q @ K.T)                                   # [G, L]
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return (p @ V) / p.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------- aggregation variants

def _logits(K, qbar, theta, offsets, t, rope):
    """logit[p, g, k] = RoPE(qbar_g, t + offsets[k]) . K[p]: the rotary logit of every query centre at every
    future position ([S] 流程详解 step 2), float64 [L, G, |D|]."""
    K = np.asarray(K, dtype=np.float64)
    qbar = np.asarray(qbar, dtype=np.float64)
    W = np.stack([[rotate(qbar[g], t + dl, theta, rope) for dl in offsets] for g in range(qbar.shape[0])])
    return np.einsum("pd,gkd->pgk", K, W)


def score_variant(K, qbar, c, theta, offsets, t, rope: str = "half", agg: str = "max") -> np.ndarray:
    """Scores whose distance part aggregates the logits of the query group's centres over the future offsets
    with something other than a mean, so that they no longer collapse to one dot product (the pages leave the
    aggregation of the series open, [S] 复现注意事项):
      "mean"     mean over heads and offsets (the collapsible score: equals `score`);
      "max"      max over heads and offsets;
      "head_max" mean over heads of the max over offsets.
    The norm term is the same as in `score`.  Float64 [L]."""
    lg = _logits(K, qbar, theta, offsets, t, rope)
    if agg == "mean":
        dist = lg.mean(axis=(1, 2))
    elif agg == "max":
        dist = lg.max(axis=(1, 2))
    elif agg == "head_max":
        dist = lg.max(axis=2).mean(axis=1)
    else:
        raise ValueError(agg)
    norms = np.abs(to_pairs(np.asarray(K, dtype=np.float64), rope))
    return dist + (norms @ np.asarray(c, dtype=np.float64).T).mean(axis=1)


def abs_terms_variant(K, qbar, c, theta, offsets, t, rope: str = "half") -> np.ndarray:
    """Error scale of a variant score: the largest sum of |W_j K_j| over the group's rotated centres W plus the
    norm term's absolute sum (every aggregation above errs by at most the worst logit's error)."""
    K = np.asarray(K, dtype=np.float64)
    qbar = np.asarray(qbar, dtype=np.float64)
    W = np.stack([rotate(qbar[g], t + dl, theta, rope) for g in range(qbar.shape[0]) for dl in offsets])
    dist = (np.abs(K) @ np.abs(W).T).max(axis=1)
    chat = np.asarray(c, dtype=np.float64).mean(axis=0)
    return dist + np.abs(to_pairs(K, rope)) @ np.abs(chat)
