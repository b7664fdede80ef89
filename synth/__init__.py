"""Seeded synthetic inputs for the QSA indexer hot path.

Shared by the oracle's tests and the GPU parity tests and benchmark.  This
module draws random numbers and lays out buffers; it holds none of the
method's arithmetic (no pooling, norm, rotary, scoring or selection).  bf16
values are produced from float32 draws by torch's CPU conversion.

Workloads (4 query heads, head dim 128, 4-token blocks, rotary_dim 64,
theta 1e4, eps 1e-6, norm weights N(0, 0.05) unless stated):
  1  tiny prefill: 512 tokens, all 512 rows as queries, budget 64; 6 blocks
     (about 5% of 128) take their left neighbour's pooled key, so equal
     scores exercise the ascending-index tie fill.
  2  prefill: 4096 tokens, all 4096 rows, budget 2048.
  3  decode-shaped: 64 rows at positions uniform in [60000, 65535] over a
     65536-token cache; 10% of blocks get a +2.0 shift on all raw elements.
  4  long-context decode: 16 rows at positions 262140..262143 (4 each,
     distinct queries) over a 262144-token cache.
  5  prefill chunk: 8192 rows at positions 57344..65535 over 65536 tokens;
     keys and queries drawn from {-1, 0, +1} with p = 0.25 / 0.5 / 0.25.
Seed = 1000 + workload number.  Draw order: raw keys, queries, k norm
weight, q norm weight, positions, then structure.
"""

from __future__ import annotations

import numpy as np
import torch

HEADS = 4
HEAD_DIM = 128

WORKLOADS = {
    1: dict(name="tiny-prefill-512", tokens=512, rows=512, budget=64),
    2: dict(name="prefill-4096", tokens=4096, rows=4096, budget=2048),
    3: dict(name="decode-64k-x64", tokens=65536, rows=64, budget=2048),
    4: dict(name="decode-256k-x16", tokens=262144, rows=16, budget=2048),
    5: dict(name="prefill-chunk-8192-over-64k", tokens=65536, rows=8192, budget=2048),
}

ROTARY_DIM = 64
THETA = 10000.0
EPS = 1e-6


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16) via torch's CPU conversion."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _ternary(rng, shape):
    u = rng.random(shape)
    return np.where(u < 0.25, -1.0, np.where(u < 0.75, 0.0, 1.0)).astype(np.float32)


def _non_adjacent(rng, lo, hi, count):
    while True:
        pick = np.sort(rng.choice(np.arange(lo, hi), size=count, replace=False))
        if np.all(np.diff(pick) > 1):
            return pick


def make_workload(wid: int, rows: int | None = None) -> dict:
    """Inputs of workload `wid` (1..5).  `rows` limits the query rows drawn
    (the first `rows` rows of the full workload; same values).

    Returns a dict with bf16 bit arrays raw_keys [T,128], queries [Q,4,128],
    k_norm_w [128], q_norm_w [128]; int32 pos [Q]; tokens, budget,
    rotary_dim, theta, eps; dup_blocks (blocks whose pooled key is replaced
    by block-1's, applied in ascending order after pooling).
    """
    spec = WORKLOADS[wid]
    T, Q = spec["tokens"], spec["rows"]
    rng = np.random.Generator(np.random.PCG64(1000 + wid))
    if wid == 5:
        keys = _ternary(rng, (T, HEAD_DIM))
        qs = _ternary(rng, (Q, HEADS, HEAD_DIM))
    else:
        keys = rng.standard_normal((T, HEAD_DIM), dtype=np.float32)
        qs = rng.standard_normal((Q, HEADS, HEAD_DIM), dtype=np.float32)
    w_k = (rng.standard_normal(HEAD_DIM) * 0.05).astype(np.float32)
    w_q = (rng.standard_normal(HEAD_DIM) * 0.05).astype(np.float32)
    dup = np.zeros(0, dtype=np.int64)
    if wid == 1:
        pos = np.arange(Q, dtype=np.int32)
        dup = _non_adjacent(rng, 1, T // 4, 6)
    elif wid == 2:
        pos = np.arange(Q, dtype=np.int32)
    elif wid == 3:
        pos = rng.integers(60000, 65536, size=Q).astype(np.int32)
        nb = T // 4
        shifted = rng.choice(nb, size=int(round(0.1 * nb)), replace=False)
        view = keys.reshape(nb, 4, HEAD_DIM)
        view[shifted] += np.float32(2.0)
    elif wid == 4:
        pos = np.repeat(np.arange(262140, 262144, dtype=np.int32), 4)
    else:
        pos = np.arange(57344, 57344 + Q, dtype=np.int32)
    if rows is not None:
        qs, pos = qs[:rows], pos[:rows]
    return dict(
        wid=wid, name=spec["name"], tokens=T, budget=spec["budget"],
        rotary_dim=ROTARY_DIM, theta=THETA, eps=EPS,
        raw_keys=bf16_bits(keys), queries=bf16_bits(qs),
        k_norm_w=bf16_bits(w_k), q_norm_w=bf16_bits(w_q),
        pos=np.ascontiguousarray(pos, dtype=np.int32), dup_blocks=dup,
    )


def apply_dups(pooled: np.ndarray, dup_blocks) -> np.ndarray:
    """Copy pooled[b-1] into pooled[b] for each b, ascending (a buffer copy)."""
    out = np.array(pooled, copy=True)
    for b in sorted(int(x) for x in dup_blocks):
        out[b] = out[b - 1]
    return out


def rope_sweep(rotary_dim: int, theta: float, tokens: int = 262147, rows: int = 8190, seed: int = 31) -> dict:
    """Inputs for checking the rotary embedding over a whole cache: raw keys
    N(0, 1) for `tokens` tokens (every 4-token block anchor up to the longest
    cache the library accepts), `rows` N(0, 1) query rows at positions 0..15,
    the last 16 positions and uniform ones between, norm weights N(0, 0.05).
    The draws do not depend on rotary_dim or theta, which are only recorded."""
    rng = np.random.Generator(np.random.PCG64(seed))
    keys = rng.standard_normal((tokens, HEAD_DIM), dtype=np.float32)
    qs = rng.standard_normal((rows, HEADS, HEAD_DIM), dtype=np.float32)
    w_k = (rng.standard_normal(HEAD_DIM) * 0.05).astype(np.float32)
    w_q = (rng.standard_normal(HEAD_DIM) * 0.05).astype(np.float32)
    ends = np.concatenate([np.arange(16), np.arange(tokens - 16, tokens)])
    pos = np.concatenate([ends, rng.integers(16, tokens - 16, size=rows - len(ends))])
    return dict(
        wid=0, name=f"rope-sweep-{tokens}", tokens=tokens, budget=2048,
        rotary_dim=rotary_dim, theta=theta, eps=EPS,
        raw_keys=bf16_bits(keys), queries=bf16_bits(qs),
        k_norm_w=bf16_bits(w_k), q_norm_w=bf16_bits(w_q),
        pos=np.ascontiguousarray(pos, dtype=np.int32), dup_blocks=np.zeros(0, dtype=np.int64),
    )


def single_row(wid: int, position: int) -> dict:
    """One query row (workload wid's first query) at `position` over that
    workload's key cache: the pages' one-row select shapes (64k, 256k)."""
    w = make_workload(wid, rows=1)
    w["pos"] = np.array([position], dtype=np.int32)
    return w


# ----------------------------------------------------------------------------
# Selector-only fixtures: score rows fed straight to the selector.
# ----------------------------------------------------------------------------

FIXTURE_POSITIONS = (0, 1, 2, 3, 4, 67, 2050, 2051, 2052, 2055, 8191, 65535, 262143, 262146)


def _blocks(p):
    return (p + 1) // 4


def selector_fixture(kind: str, positions=FIXTURE_POSITIONS, seed: int = 77,
                     spare_cols: int = 0):
    """Score rows of one fixture kind for rows at `positions`.

    Returns (scores [R, cols] f32, cols, pos int32 [R], tokens).  Columns at
    or past a row's visible block count hold a NaN sentinel (must be
    ignored).  Kinds:
      zeros    cut inside a run of mixed +0.0 / -0.0 scores
      ties     scores on a 0.25 grid, ties away from zero
      lowbyte  1.0 + k ulp, k < 256 (keys differ only in the low byte)
      wild     negatives, subnormals and large magnitudes
      equal    every score equal
      poison   one NaN or +-Inf inside the prefix of every other row
      random   N(0, 1) scores
    spare_cols > 0 adds that many sentinel-filled columns past tokens/4.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    pos = np.asarray(positions, dtype=np.int32)
    tokens = int(pos.max()) + 1
    cols = tokens // 4 + spare_cols
    R = len(pos)
    scores = np.full((R, max(cols, 1)), np.nan, dtype=np.float32)
    for r, p in enumerate(pos):
        n = _blocks(int(p))
        if n == 0:
            continue
        if kind == "zeros":
            pos_count = int(rng.integers(0, max(1, min(n, 600))))
            v = np.where(rng.random(n) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
            hot = rng.choice(n, size=pos_count, replace=False)
            v[hot] = rng.random(pos_count).astype(np.float32) + np.float32(0.5)
            neg = rng.random(n) < 0.05
            v[neg] = -rng.random(int(neg.sum())).astype(np.float32) - np.float32(0.1)
        elif kind == "ties":
            v = (rng.integers(0, 12, size=n) * 0.25 + 0.25).astype(np.float32)
        elif kind == "lowbyte":
            v = (np.float32(1.0).view(np.uint32) + rng.integers(0, 256, size=n).astype(np.uint32)).view(np.float32)
        elif kind == "wild":
            mag = np.float32(10.0) ** rng.uniform(-44, 38, size=n).astype(np.float32)
            sign = np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
            v = (mag * sign).astype(np.float32)
            sub = rng.random(n) < 0.1
            v[sub] = (rng.integers(1, 1 << 23, size=int(sub.sum())).astype(np.uint32)).view(np.float32)
        elif kind == "equal":
            v = np.full(n, 0.75, dtype=np.float32)
        elif kind == "poison":
            v = rng.standard_normal(n).astype(np.float32)
            if r % 2 == 1:
                v[int(rng.integers(0, n))] = [np.nan, np.inf, -np.inf][r % 3]
        elif kind == "random":
            v = rng.standard_normal(n).astype(np.float32)
        else:
            raise ValueError(kind)
        scores[r, :n] = v
    return scores, cols, pos, tokens


def random_rows(n_rows: int, max_blocks: int, seed: int, tie_grid: float | None = None):
    """Random score rows with positions spread over [0, 4*max_blocks + 3]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    pos = rng.integers(0, 4 * max_blocks + 4, size=n_rows).astype(np.int32)
    tokens = int(pos.max()) + 1
    cols = tokens // 4
    scores = rng.standard_normal((n_rows, max(cols, 1))).astype(np.float32)
    if tie_grid is not None:
        scores = (np.round(scores / tie_grid) * tie_grid).astype(np.float32)
    return scores, cols, pos, tokens
