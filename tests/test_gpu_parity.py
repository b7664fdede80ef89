"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: pooled keys bit-exact; scores within 5e-3 absolute (the parity bound
the score pages settle on); the selector fed the oracle's scores bit-exact;
end-to-end masks may differ from the oracle's only at blocks whose oracle
score lies within 5e-3 of the row's cut, and are structurally valid.
"""

import functools

import numpy as np
import pytest
import torch

import oracle as O
import synth
import sparse_attention_token_qsa_amd as qsa
from tests.gpu_util import (DEV, gpu_pool, gpu_prep, gpu_scores, gpu_scores_prepped, gpu_select,
                            gpu_select_indices, gpu_select_indices_ws, gpu_select_ws, i32_dev, note, status_word,
                            u16_dev, u16_host, workload)
from tests.test_oracle_pins import check_structure

pytestmark = pytest.mark.gpu

SCORE_ATOL = 5e-3


@functools.lru_cache(maxsize=8)
def oracle_pooled(wid):
    w = workload(wid)
    p = O.pool_keys(w["raw_keys"], w["k_norm_w"], w["rotary_dim"], w["theta"], w["eps"])
    return synth.apply_dups(p, w["dup_blocks"])


def sample_rows(wid):
    """Rows checked against the oracle: all, except the 8192-row chunk."""
    w = workload(wid)
    R = len(w["pos"])
    if R <= 4096:
        return np.arange(R)
    rng = np.random.default_rng(9)
    return np.unique(np.concatenate([[0, 1, R - 2, R - 1], rng.choice(R, 92, replace=False)]))


def oracle_scores(wid, rows):
    w = workload(wid)
    qhat = O.prep_queries(w["queries"][rows], w["pos"][rows], w["q_norm_w"], w["rotary_dim"],
                          w["theta"], w["eps"])
    return O.score_rows(qhat, w["pos"][rows], oracle_pooled(wid), w["tokens"])


@functools.lru_cache(maxsize=8)
def oracle_sample_scores(wid):
    return oracle_scores(wid, sample_rows(wid))


SCORERS = {"fused": gpu_scores, "prepped": gpu_scores_prepped}


def dense(score_list, cols):
    out = np.full((len(score_list), max(cols, 1)), np.nan, dtype=np.float32)
    for r, s in enumerate(score_list):
        out[r, : len(s)] = s
    return out


# ------------------------------------------------------------------ pool ----

@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_pool_bit_exact(wid):
    w = workload(wid)
    note(f"pool parity: workload {wid} ({w['name']}), tokens {w['tokens']}")
    got = u16_host(gpu_pool(w))
    want = O.pool_keys(w["raw_keys"], w["k_norm_w"], w["rotary_dim"], w["theta"], w["eps"])
    diff = np.nonzero(got != want)
    assert len(diff[0]) == 0, (len(diff[0]), got[diff][:8], want[diff][:8], diff[0][:8], diff[1][:8])


def test_pool_block_range_fused_row_stride_and_unaligned_stride():
    w = workload(1)
    T = w["tokens"]
    want = O.pool_keys(w["raw_keys"], w["k_norm_w"], 64, 1e4, 1e-6)
    # keys as the last 128 columns of a 640-wide fused row (4 query heads first)
    fused = np.zeros((T, 640), dtype=np.uint16)
    fused[:, 512:] = w["raw_keys"]
    fused_dev = u16_dev(fused)
    note("pool: fused 640-wide rows, blocks [37, 57)")
    got = u16_host(gpu_pool(w, first_block=37, n_blocks=20, key_stride_view=fused_dev[:, 512:]))
    assert np.array_equal(got[37:57], want[37:57])
    assert np.all(got[:37] == 0x5A5A) and np.all(got[57:] == 0x5A5A)
    # odd row stride (scalar loads)
    odd = np.zeros((T, 129), dtype=np.uint16)
    odd[:, :128] = w["raw_keys"]
    note("pool: odd row stride 129")
    got = u16_host(gpu_pool(w, key_stride_view=u16_dev(odd)))
    assert np.array_equal(got, want)


def test_pool_nan_key_poisons_only_its_block():
    w = dict(workload(1))
    raw = w["raw_keys"].copy()
    raw[4 * 50 + 2, 7] = 0x7FC0
    w["raw_keys"] = raw
    got = O.f32_from_bf16(u16_host(gpu_pool(w)))
    assert np.all(np.isnan(got[50]))
    assert not np.any(np.isnan(np.delete(got, 50, axis=0)))


# ------------------------------------------------------------------ prep ----

@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_prep_bit_exact(wid):
    w = workload(wid)
    note(f"prep parity: workload {wid} ({w['name']}), {len(w['pos'])} rows")
    qhat, st = gpu_prep(w)
    assert st == 0
    got = u16_host(qhat)
    want = O.prep_queries(w["queries"], w["pos"], w["q_norm_w"], w["rotary_dim"], w["theta"],
                          w["eps"])
    diff = np.nonzero(got != want)
    assert len(diff[0]) == 0, (len(diff[0]), got[diff][:8], want[diff][:8], diff[0][:8])


def test_prep_nan_query_and_bad_positions():
    w = workload(1)
    pos = np.array([0, 5, 511, -1, 512, 77, 2**31 - 1], dtype=np.int32)
    q = w["queries"][: len(pos)].copy()
    q[1, 2, 9] = 0x7FC0   # NaN in one head: that head is NaN, the others finite
    q[5, 0, 3] = 0xFFC1   # negative NaN with a payload: written as 0x7FC0
    note("prep: NaN queries and out-of-range positions")
    qhat, st = gpu_prep(w, pos=pos, q=q)
    assert st == O.STATUS_BAD_POSITION
    got = u16_host(qhat)
    valid = [0, 1, 2, 5]
    want = O.prep_queries(q[valid], pos[valid], w["q_norm_w"], w["rotary_dim"], w["theta"],
                          w["eps"])
    assert np.array_equal(got[valid], want)
    assert np.all(got[1, 2] == 0x7FC0) and np.all(got[5, 0] == 0x7FC0)
    assert not np.any(got[1, [0, 1, 3]] == 0x7FC0)
    assert np.all(got[[3, 4, 6]] == 0)


@pytest.mark.parametrize("rd", [0, 2, 36, 128])
def test_prep_other_rotary_dims(rd):
    w = workload(1)
    rows = np.arange(0, 512, 7)
    pos, q = w["pos"][rows], w["queries"][rows]
    note(f"prep: rotary_dim {rd}")
    ww = dict(w, rotary_dim=rd, theta=5e5)
    qhat, st = gpu_prep(ww, pos=pos, q=q)
    assert st == 0
    want = O.prep_queries(q, pos, w["q_norm_w"], rd, 5e5, w["eps"])
    assert np.array_equal(u16_host(qhat), want)


# ---------------------------------------------------------------- select ----

@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_select_on_oracle_scores_bit_exact(wid):
    w = workload(wid)
    rows = sample_rows(wid)
    if wid == 5:
        rows = rows[:48]
    note(f"select parity on oracle scores: workload {wid}, {len(rows)} rows")
    T = w["tokens"]
    cols = T // 4
    sc = dense(oracle_scores(wid, rows), cols)
    pos = w["pos"][rows]
    want, wst = O.select_mask(sc, cols, pos, T, w["budget"])
    got, gst = gpu_select(sc, cols, pos, T, w["budget"])
    assert gst == wst == 0
    bad = [r for r in range(len(rows)) if not np.array_equal(got[r], want[r])]
    assert not bad, (bad[:5], pos[bad[:5]])


@pytest.mark.parametrize("kind", ["zeros", "ties", "lowbyte", "wild", "equal", "random", "poison"])
def test_select_fixtures_bit_exact(kind):
    scores, cols, pos, T = synth.selector_fixture(kind)
    note(f"select fixture {kind}: rows {len(pos)}, tokens {T}")
    for budget in (2048, 64, 4):
        want, wst = O.select_mask(scores, cols, pos, T, budget)
        got, gst = gpu_select(scores, cols, pos, T, budget)
        assert gst == wst
        bad = [r for r in range(len(pos)) if not np.array_equal(got[r], want[r])]
        assert not bad, (budget, bad[:5], pos[bad[:5]])


def test_select_spare_columns_ragged_tokens_and_bad_positions():
    for T in (4099, 4098, 64, 5, 3, 1):
        pos = np.array([T - 1, 0, T // 2, -1, T, 2 * T + 5], dtype=np.int32)
        cols = T // 4 + 11
        scores = np.full((len(pos), cols), np.nan, np.float32)
        rng = np.random.default_rng(T)
        for r, p in enumerate(pos):
            n = (int(p) + 1) // 4 if 0 <= p < T else 0
            scores[r, :n] = rng.standard_normal(n)
        note(f"select ragged: tokens {T}")
        want, wst = O.select_mask(scores, cols, pos, T, 64)
        got, gst = gpu_select(scores, cols, pos, T, 64)
        assert gst == wst == O.STATUS_BAD_POSITION
        assert np.array_equal(got, want)


def test_select_longest_supported_row():
    T = 262147
    pos = np.array([262146, 262145, 262144, 262143, 131071], dtype=np.int32)
    for kind in ("random", "ties", "equal"):
        scores, cols, pos2, _ = synth.selector_fixture(kind, positions=pos)
        note(f"select longest rows: {kind}")
        want, _ = O.select_mask(scores, cols, pos2, T, 2048)
        got, st = gpu_select(scores, cols, pos2, T, 2048)
        assert st == 0 and np.array_equal(got, want)


@pytest.mark.parametrize("copies", [1, 2])
def test_select_prefill_batch_on_oracle_scores_bit_exact(copies):
    """The benchmarked prefill select: 1024 rows of the prefill chunk over 64k
    (ternary keys and queries, many exact ties), fed the oracle's scores as
    one batch of 1024 * copies rows (the oracle rows repeated), so the
    launch is the prefill one: 512 threads per row with the two-per-thread
    prefilter, 16-byte loads and stores, and rows visited in the 128-row
    group order of a 1024 k-row batch.  Masks, index lists and counts are
    bit-exact against the oracle's, and so is the split-capable entry point
    (which takes the same kernel for this many rows)."""
    from tests import oracle_cache as C
    w = workload(5)
    T = w["tokens"]
    cols = T // 4
    pos1, _, sc1, mask1, idx1, cnt1 = C.prefill_slice()
    pos = np.tile(pos1, copies)
    sc = np.tile(sc1, (copies, 1))
    note(f"select, prefill batch on oracle scores: {len(pos)} rows over {T} tokens")
    got, gst = gpu_select(sc, cols, pos, T, w["budget"])
    assert gst == 0
    bad = [r for r in range(len(pos)) if not np.array_equal(got[r], mask1[r % len(pos1)])]
    assert not bad, (bad[:5], pos[bad[:5]])
    got_ws, gst, nbytes = gpu_select_ws(sc, cols, pos, T, w["budget"])
    assert gst == 0 and nbytes == 0 and np.array_equal(got_ws, got)
    gi, gc, gst = gpu_select_indices(sc, cols, pos, T, w["budget"])
    assert gst == 0
    assert np.array_equal(gc, np.tile(cnt1, copies))
    assert np.array_equal(gi, np.tile(idx1, (copies, 1)))


def _template_positions(T):
    """Sixteen row positions over a T-token cache: the last tokens (every
    tail length), around the budget boundary, the middle, tiny rows."""
    p = [T - 1, T - 2, T - 3, T - 4, T - 5, T // 2 + 1, T // 2 - 1, 3 * T // 4, T // 4,
         2047, 2050, 2051, 2055, 67, 4, 0]
    return np.array([min(x, T - 1) for x in p], dtype=np.int32)


@pytest.mark.parametrize("rows", [16, 1024])
@pytest.mark.parametrize("T", [4096, 8192, 16384, 32768, 65536, 131072, 262144])
def test_select_fixture_batches_reach_every_template_bit_exact(T, rows):
    """The selector fixtures (signed zeros, ties, low-byte keys, wild
    magnitudes, all equal, random, non-finite) over caches of 4k to 256k
    tokens (multiples of 16: the vectorised load and store forms), as
    batches of 16 and 1024 rows (the 16 fixture rows repeated): every
    one-workgroup-per-row select template, with and without the prefilter,
    in index order and in the group order of 1024-row batches.  Masks,
    index lists and counts bit-exact against the oracle's on every row."""
    pos16 = _template_positions(T)
    reps = rows // len(pos16)
    for kind in ("zeros", "ties", "lowbyte", "wild", "equal", "random", "poison"):
        sc16, cols, p16, T2 = synth.selector_fixture(kind, positions=pos16)
        assert T2 == T and cols == T // 4
        sc = np.tile(sc16, (reps, 1))
        pos = np.tile(p16, reps)
        for budget in (2048, 64, 4):
            want, wst = O.select_mask(sc16, cols, p16, T, budget)
            wi, wc, wst2 = O.select_indices(sc16, cols, p16, T, budget)
            note(f"select fixture batch: {kind}, {rows} rows over {T} tokens, budget {budget}")
            got, gst = gpu_select(sc, cols, pos, T, budget)
            assert gst == wst
            bad = [r for r in range(len(pos)) if not np.array_equal(got[r], want[r % 16])]
            assert not bad, (kind, budget, bad[:5], pos[bad[:5]])
            gi, gc, gst = gpu_select_indices(sc, cols, pos, T, budget)
            assert gst == wst2
            assert np.array_equal(gc, np.tile(wc, reps)), (kind, budget)
            assert np.array_equal(gi, np.tile(wi, (reps, 1))), (kind, budget)


# ------------------------------------------------- select, index lists ----

def _check_indices(got, gcnt, want, wcnt, budget, stride):
    bad = [r for r in range(len(wcnt))
           if gcnt[r] != wcnt[r] or not np.array_equal(got[r, : budget + 3], want[r])]
    assert not bad, bad[:5]
    assert np.all(got[:, budget + 3: stride] == -77), "wrote past budget + 3"


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_select_indices_on_oracle_scores_bit_exact(wid):
    w = workload(wid)
    rows = sample_rows(wid)
    if wid == 5:
        rows = rows[:48]
    T = w["tokens"]
    cols = T // 4
    sc = dense(oracle_scores(wid, rows), cols)
    pos = w["pos"][rows]
    b = w["budget"]
    note(f"index lists on oracle scores: workload {wid}, {len(rows)} rows")
    want, wcnt, wst = O.select_indices(sc, cols, pos, T, b)
    got, gcnt, gst = gpu_select_indices(sc, cols, pos, T, b, stride=b + 9)
    assert gst == wst == 0
    _check_indices(got, gcnt, want, wcnt, b, b + 9)


@pytest.mark.parametrize("kind", ["zeros", "ties", "lowbyte", "wild", "equal", "random", "poison"])
def test_select_indices_fixtures_bit_exact(kind):
    scores, cols, pos, T = synth.selector_fixture(kind)
    note(f"index lists, fixture {kind}: rows {len(pos)}, tokens {T}")
    for budget in (2048, 64, 4):
        want, wcnt, wst = O.select_indices(scores, cols, pos, T, budget)
        got, gcnt, gst = gpu_select_indices(scores, cols, pos, T, budget)
        assert gst == wst
        _check_indices(got, gcnt, want, wcnt, budget, budget + 3)


def test_select_indices_ragged_tokens_spare_columns_bad_positions():
    for T in (4099, 16387, 65541, 5, 1):
        pos = np.array([T - 1, 0, T // 2, -1, T, 2 * T + 5, max(T - 3, 0)], dtype=np.int32)
        cols = T // 4 + 11
        scores = np.full((len(pos), cols), np.nan, np.float32)
        rng = np.random.default_rng(T)
        for r, p in enumerate(pos):
            n = (int(p) + 1) // 4 if 0 <= p < T else 0
            scores[r, :n] = rng.standard_normal(n)
        note(f"index lists ragged: tokens {T}")
        want, wcnt, wst = O.select_indices(scores, cols, pos, T, 64)
        got, gcnt, gst = gpu_select_indices(scores, cols, pos, T, 64, stride=70)
        assert gst == wst
        _check_indices(got, gcnt, want, wcnt, 64, 70)


# ------------------------------------------------- select, split rows ----

@pytest.mark.parametrize("wid", [3, 4])
def test_select_ws_on_oracle_scores_bit_exact(wid):
    """Decode batches through the split selector: the oracle's scores of
    every sampled row, masks equal to the oracle's byte for byte."""
    w = workload(wid)
    rows = sample_rows(wid)
    T = w["tokens"]
    cols = T // 4
    sc = dense(oracle_scores(wid, rows), cols)
    pos = w["pos"][rows]
    note(f"split select on oracle scores: workload {wid}, {len(rows)} rows")
    want, wst = O.select_mask(sc, cols, pos, T, w["budget"])
    got, gst, nbytes = gpu_select_ws(sc, cols, pos, T, w["budget"])
    assert (nbytes > 0) == (T > 65539), "the split path runs on caches past 64k tokens"
    assert gst == wst == 0
    bad = [r for r in range(len(rows)) if not np.array_equal(got[r], want[r])]
    assert not bad, (bad[:5], pos[bad[:5]])


@pytest.mark.parametrize("kind", ["zeros", "ties", "lowbyte", "wild", "equal", "random", "poison"])
def test_select_ws_fixtures_bit_exact(kind):
    scores, cols, pos, T = synth.selector_fixture(kind)
    note(f"split select fixture {kind}: rows {len(pos)}, tokens {T}")
    for budget in (2048, 64, 4):
        want, wst = O.select_mask(scores, cols, pos, T, budget)
        got, gst, nbytes = gpu_select_ws(scores, cols, pos, T, budget)
        assert nbytes > 0
        assert gst == wst
        bad = [r for r in range(len(pos)) if not np.array_equal(got[r], want[r])]
        assert not bad, (budget, bad[:5], pos[bad[:5]])


def test_select_ws_kept_blocks_in_one_chunk_and_across_boundaries():
    """Kept sets that sit in one 4096-block chunk (rising scores: the last
    chunk; all equal: the first 512 indices), ties straddling a chunk
    boundary, and a single kept block."""
    T = 65536 + 4 * 4096 + 7
    n = T // 4
    pos = np.array([T - 1, T - 2, 4 * 8192 + 3, 4 * 4096 - 1, 4 * 4096 + 3, T - 1], dtype=np.int32)
    cols = n
    sc = np.full((len(pos), cols), np.nan, np.float32)
    nb = (pos.astype(np.int64) + 1) // 4
    sc[0, : nb[0]] = np.arange(nb[0], dtype=np.float32)          # rising: last chunk
    sc[1, : nb[1]] = 1.5                                          # all equal: lowest indices
    v = np.zeros(nb[2], np.float32)
    v[4096 - 300: 4096 + 300] = 2.0                               # 600 ties across a boundary
    sc[2, : nb[2]] = v
    rng = np.random.default_rng(5)
    sc[3, : nb[3]] = rng.standard_normal(nb[3])                   # exactly one chunk
    sc[4, : nb[4]] = rng.standard_normal(nb[4])                   # one chunk plus one block
    sc[5, : nb[5]] = -np.arange(nb[5], dtype=np.float32)          # falling: first chunk
    note(f"split select boundaries: tokens {T}")
    for budget in (2048, 4):
        want, wst = O.select_mask(sc, cols, pos, T, budget)
        got, gst, nbytes = gpu_select_ws(sc, cols, pos, T, budget)
        assert nbytes > 0 and gst == wst == 0
        bad = [r for r in range(len(pos)) if not np.array_equal(got[r], want[r])]
        assert not bad, (budget, bad)


@pytest.mark.parametrize("T", [65541, 65554, 131075, 262147])
def test_select_ws_ragged_tokens_spare_columns_bad_positions(T):
    """Token counts off the 16-byte grid (byte-wise mask path), a score row
    stride off the 4-float grid (scalar loads), out-of-range positions and a
    non-finite score in one row."""
    pos = np.array([T - 1, 0, 3, 4, 2051, T // 2, -1, T, 2 * T + 5, T - 3], dtype=np.int32)
    cols = T // 4 + 3
    scores = np.full((len(pos), cols), np.nan, np.float32)
    rng = np.random.default_rng(T)
    for r, p in enumerate(pos):
        n = (int(p) + 1) // 4 if 0 <= p < T else 0
        scores[r, :n] = rng.standard_normal(n)
    scores[9, 17] = np.inf
    note(f"split select ragged: tokens {T}")
    want, wst = O.select_mask(scores, cols, pos, T, 2048)
    got, gst, nbytes = gpu_select_ws(scores, cols, pos, T, 2048)
    assert nbytes > 0
    assert gst == wst == O.STATUS_BAD_POSITION | O.STATUS_NONFINITE_SCORE
    assert np.array_equal(got, want)


def _check_split_indices(sc, cols, pos, T, budget, stride=None):
    stride = budget + 3 if stride is None else stride
    want, wcnt, wst = O.select_indices(sc, cols, pos, T, budget)
    got, gcnt, gst, nbytes = gpu_select_indices_ws(sc, cols, pos, T, budget, stride=stride)
    assert gst == wst, (gst, wst)
    assert np.array_equal(gcnt, wcnt), np.nonzero(gcnt != wcnt)[0][:8]
    bad = [r for r in range(len(pos)) if not np.array_equal(got[r, : budget + 3], want[r])]
    assert not bad, (budget, bad[:5], pos[bad[:5]])
    assert np.all(got[:, budget + 3:] == -77), "wrote past budget + 3"
    return nbytes, wst


@pytest.mark.parametrize("wid", [3, 4])
def test_select_indices_ws_on_oracle_scores_bit_exact(wid):
    """Index lists through the split selector on the oracle's scores of the
    decode workloads: equal to the oracle's lists and counts."""
    w = workload(wid)
    rows = sample_rows(wid)
    T = w["tokens"]
    cols = T // 4
    note(f"split index lists on oracle scores: workload {wid}")
    nbytes, st = _check_split_indices(dense(oracle_scores(wid, rows), cols), cols, w["pos"][rows], T, w["budget"])
    assert (nbytes > 0) == (T > 65539) and st == 0


@pytest.mark.parametrize("kind", ["zeros", "ties", "lowbyte", "wild", "equal", "random", "poison"])
def test_select_indices_ws_fixtures_bit_exact(kind):
    scores, cols, pos, T = synth.selector_fixture(kind)
    note(f"split index lists fixture {kind}")
    for budget in (2048, 64, 4):
        nbytes, _ = _check_split_indices(scores, cols, pos, T, budget)
        assert nbytes > 0


def test_select_indices_ws_kept_blocks_in_one_chunk_and_across_boundaries():
    T = 65536 + 4 * 4096 + 7
    n = T // 4
    pos = np.array([T - 1, T - 2, 4 * 8192 + 3, 4 * 4096 - 1, 4 * 4096 + 3, T - 1], dtype=np.int32)
    sc = np.full((len(pos), n), np.nan, np.float32)
    nb = (pos.astype(np.int64) + 1) // 4
    sc[0, : nb[0]] = np.arange(nb[0], dtype=np.float32)
    sc[1, : nb[1]] = 1.5
    v = np.zeros(nb[2], np.float32)
    v[4096 - 300: 4096 + 300] = 2.0
    sc[2, : nb[2]] = v
    rng = np.random.default_rng(5)
    sc[3, : nb[3]] = rng.standard_normal(nb[3])
    sc[4, : nb[4]] = rng.standard_normal(nb[4])
    sc[5, : nb[5]] = -np.arange(nb[5], dtype=np.float32)
    note(f"split index lists at chunk boundaries: tokens {T}")
    for budget in (2048, 4):
        _check_split_indices(sc, n, pos, T, budget, stride=budget + 11)


@pytest.mark.parametrize("T", [65541, 131075, 262147])
def test_select_indices_ws_ragged_tokens_bad_positions(T):
    pos = np.array([T - 1, 0, 3, 4, 2051, T // 2, -1, T, 2 * T + 5, T - 3], dtype=np.int32)
    cols = T // 4 + 3
    scores = np.full((len(pos), cols), np.nan, np.float32)
    rng = np.random.default_rng(T)
    for r, p in enumerate(pos):
        nn = (int(p) + 1) // 4 if 0 <= p < T else 0
        scores[r, :nn] = rng.standard_normal(nn)
    scores[9, 17] = np.inf
    note(f"split index lists ragged: tokens {T}")
    nbytes, st = _check_split_indices(scores, cols, pos, T, 2048, stride=2060)
    assert nbytes > 0 and st == O.STATUS_BAD_POSITION | O.STATUS_NONFINITE_SCORE


def test_select_ws_equals_select_and_reuses_its_workspace():
    """Two calls in a row on one workspace (the second over shorter rows)
    match qsa_select_mask bit for bit; many rows take the one-workgroup path
    and need no workspace."""
    w = workload(4)
    T = w["tokens"]
    cols = T // 4
    rng = np.random.default_rng(11)
    rows = 24
    pos = np.sort(rng.integers(T // 2, T, size=rows)).astype(np.int32)
    sc = rng.standard_normal((rows, cols)).astype(np.float32)
    nbytes = qsa.qsa_select_workspace_bytes(rows, T)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    from tests.gpu_util import f32_dev
    for p2 in (pos, pos // 3):
        mask = torch.full((rows, T), 0xAB, dtype=torch.uint8, device=DEV)
        st = status_word()
        qsa.qsa_select_mask_ws(f32_dev(sc.reshape(-1)), cols, i32_dev(p2), T, 2048, mask, st, ws)
        assert qsa.check_status(st) == 0
        ref, rst = gpu_select(sc, cols, p2, T, 2048)
        assert rst == 0 and np.array_equal(mask.cpu().numpy(), ref)
    assert qsa.qsa_select_workspace_bytes(4096, T) == 0


@pytest.mark.parametrize("rows,T", [(1024, 4096), (2048, 65536), (3072, 8192)])
def test_select_row_order_of_whole_row_groups(rows, T):
    """Batches of a multiple of 1024 rows are visited in a group order, not
    by row index: every row is written, and each equals the same row selected
    in batches of other sizes (index order) and, on a sample, the oracle."""
    from tests.gpu_util import f32_dev
    note(f"select row order: {rows} rows over {T} tokens")
    rng = np.random.default_rng(rows + T)
    cols = T // 4
    pos = rng.integers(0, T, size=rows).astype(np.int32)
    sc = rng.standard_normal((rows, cols)).astype(np.float32)
    budget = 2048
    mask = torch.full((rows, T), 0xAB, dtype=torch.uint8, device=DEV)
    st = status_word()
    qsa.qsa_select_mask(f32_dev(sc.reshape(-1)), cols, i32_dev(pos), T, budget, mask, st)
    assert qsa.check_status(st) == 0
    got = mask.cpu().numpy()
    assert got.max() <= 1  # no row left unwritten
    cut = 1000
    head, hst = gpu_select(sc[:cut], cols, pos[:cut], T, budget)
    tail, tst = gpu_select(sc[cut:], cols, pos[cut:], T, budget)
    assert hst == 0 and tst == 0
    assert np.array_equal(got[:cut], head) and np.array_equal(got[cut:], tail)
    sample = np.sort(rng.choice(rows, 12, replace=False))
    want, wst = O.select_mask(sc[sample], cols, pos[sample], T, budget)
    assert wst == 0 and np.array_equal(got[sample], want)


# ----------------------------------------------------------------- score ----

@pytest.mark.parametrize("path", ["fused", "prepped"])
@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_score_within_bound_and_prefix_only(wid, path):
    w = workload(wid)
    rows = sample_rows(wid)
    T = w["tokens"]
    cols = T // 4 + (7 if wid in (1, 3) else 0)
    note(f"score parity ({path}): workload {wid}, {len(rows)} rows, score_cols {cols}")
    pooled = u16_dev(oracle_pooled(wid))
    sentinel = np.float32(-7.25)
    got, st = SCORERS[path](w, pooled, pos=w["pos"][rows], q=w["queries"][rows], score_cols=cols,
                            sentinel=sentinel)
    assert st == 0
    want = oracle_sample_scores(wid)
    worst = 0.0
    for r, s in enumerate(want):
        n = len(s)
        assert np.all(got[r, n:] == sentinel), "wrote past the visible prefix"
        if n:
            d = np.abs(got[r, :n].astype(np.float64) - s)
            worst = max(worst, float(d.max()))
    note(f"  max |gpu - oracle| = {worst:.3e}")
    assert worst <= SCORE_ATOL


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_score_prepped_equals_fused_bitwise(wid):
    w = workload(wid)
    rows = sample_rows(wid)
    note(f"score: prepped vs fused, workload {wid}")
    pooled = u16_dev(oracle_pooled(wid))
    a, s1 = gpu_scores(w, pooled, pos=w["pos"][rows], q=w["queries"][rows])
    b, s2 = gpu_scores_prepped(w, pooled, pos=w["pos"][rows], q=w["queries"][rows])
    assert s1 == s2 == 0
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def few_row_positions(T, R):
    """Ragged positions for a batch of R <= 4 rows: the cache's last token,
    a mid-cache row, a row inside its first block and a row with a partial
    last block."""
    return np.array([T - 1, T // 2 + 3, 2, 4 * 1001 + 2][:R], dtype=np.int32)


@pytest.mark.parametrize("R", [1, 2, 3, 4])
@pytest.mark.parametrize("wid", [3, 4])
def test_score_few_rows_against_oracle(wid, R):
    """Batches of one to four rows (one row: the streaming scorer; more: the
    matrix kernels): both entry points within the bound of the oracle on
    ragged rows, nothing written past a row's prefix into the spare columns,
    and the two entry points equal bit for bit."""
    w = workload(wid)
    T = w["tokens"]
    pos = few_row_positions(T, R)
    q = w["queries"][:R]
    cols = T // 4 + 5
    sentinel = np.float32(-7.25)
    note(f"score: {R} rows over workload {wid} ({T} tokens), both entry points")
    pooled = u16_dev(oracle_pooled(wid))
    a, s1 = gpu_scores(w, pooled, pos=pos, q=q, score_cols=cols, sentinel=sentinel)
    b, s2 = gpu_scores_prepped(w, pooled, pos=pos, q=q, score_cols=cols, sentinel=sentinel)
    assert s1 == s2 == 0
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    qhat = O.prep_queries(q, pos, w["q_norm_w"], w["rotary_dim"], w["theta"], w["eps"])
    want = O.score_rows(qhat, pos, oracle_pooled(wid), T)
    worst = 0.0
    for r, sc in enumerate(want):
        n = len(sc)
        assert n == (pos[r] + 1) // 4
        assert np.all(a[r, n:] == sentinel), "wrote past the visible prefix"
        if n:
            worst = max(worst, float(np.abs(a[r, :n].astype(np.float64) - sc).max()))
    note(f"  max |gpu - oracle| = {worst:.3e}")
    assert worst <= SCORE_ATOL


@pytest.mark.parametrize("path", ["fused", "prepped"])
def test_score_few_rows_nan_key_and_bad_positions(path):
    """The streaming scorer's edges: a NaN key poisons exactly its block,
    rows with out-of-range positions are flagged and left untouched."""
    w = workload(1)
    pooled = oracle_pooled(1).copy()
    pooled[50] = 0x7FC0
    pos = np.array([203, -3, 512, 60], dtype=np.int32)
    q = w["queries"][: len(pos)]
    note(f"score ({path}): 4 rows, NaN key, bad positions")
    got, st = SCORERS[path](w, u16_dev(pooled), pos=pos, q=q)
    assert st == O.STATUS_BAD_POSITION
    assert np.all(got[1] == np.float32(-7.25)) and np.all(got[2] == np.float32(-7.25))
    assert np.isnan(got[0, 50]) and np.all(np.isfinite(np.delete(got[0, :51], 50)))
    assert np.all(np.isfinite(got[3, :15])) and np.all(got[3, 15:] == np.float32(-7.25))
    qhat = O.prep_queries(q[[0, 3]], pos[[0, 3]], w["q_norm_w"], w["rotary_dim"], w["theta"], w["eps"])
    want = O.score_rows(qhat, pos[[0, 3]], pooled, 512)
    ok = ~np.isnan(want[0])
    assert np.all(np.abs(got[0, :51][ok].astype(np.float64) - want[0][ok]) <= SCORE_ATOL)
    assert np.all(np.abs(got[3, :15].astype(np.float64) - want[1]) <= SCORE_ATOL)


@pytest.mark.parametrize("path", ["fused", "prepped"])
def test_score_one_row_nan_key_and_bad_position(path):
    """The streaming scorer (one row): a NaN key poisons exactly its block;
    a row at a position past the cache is flagged and left untouched."""
    w = workload(1)
    pooled = oracle_pooled(1).copy()
    pooled[50] = 0x7FC0
    note(f"score ({path}): one row, NaN key; one row, bad position")
    got, st = SCORERS[path](w, u16_dev(pooled), pos=np.array([203], np.int32), q=w["queries"][:1])
    assert st == 0
    assert np.isnan(got[0, 50]) and np.all(np.isfinite(np.delete(got[0, :51], 50)))
    assert np.all(got[0, 51:] == np.float32(-7.25))
    qhat = O.prep_queries(w["queries"][:1], np.array([203], np.int32), w["q_norm_w"], w["rotary_dim"],
                          w["theta"], w["eps"])
    want = O.score_rows(qhat, np.array([203], np.int32), pooled, 512)[0]
    ok = ~np.isnan(want)
    assert np.all(np.abs(got[0, :51][ok].astype(np.float64) - want[ok]) <= SCORE_ATOL)
    got, st = SCORERS[path](w, u16_dev(pooled), pos=np.array([512], np.int32), q=w["queries"][:1])
    assert st == O.STATUS_BAD_POSITION
    assert np.all(got == np.float32(-7.25))


def test_score_duplicate_blocks_tie_exactly():
    w = workload(1)
    pooled = u16_dev(oracle_pooled(1))
    got, _ = gpu_scores(w, pooled)
    for b in w["dup_blocks"]:
        vis = (w["pos"] + 1) // 4 > b
        assert np.array_equal(got[vis, b].view(np.uint32), got[vis, b - 1].view(np.uint32))


@pytest.mark.parametrize("path", ["fused", "prepped"])
def test_score_nan_key_and_bad_positions(path):
    w = workload(1)
    pooled = oracle_pooled(1).copy()
    pooled[50] = 0x7FC0
    pos = np.array([199, 200, 202, 203, 204, 511, -3, 512, 700], dtype=np.int32)
    q = w["queries"][: len(pos)]
    note(f"score ({path}): NaN key, bad positions")
    got, st = SCORERS[path](w, u16_dev(pooled), pos=pos, q=q)
    assert st == O.STATUS_BAD_POSITION
    for r, p in enumerate(pos):
        if not 0 <= p < 512:
            assert np.all(got[r] == np.float32(-7.25))
            continue
        n = (p + 1) // 4
        if n > 50:
            assert np.isnan(got[r, 50]) and np.all(np.isfinite(np.delete(got[r, :n], 50)))
        else:
            assert np.all(np.isfinite(got[r, :n]))


def test_score_long_batches_ragged_rows_bad_positions_nan_key():
    """The prepared-query scorer on batches of 128 rows and more (the shape
    prefill uses): a row count that is not a multiple of 128, ragged prefixes
    from position 0 to the last token, out-of-range positions, a NaN key and
    spare score columns.  Valid rows match the oracle within the bound, the
    NaN key poisons exactly block 50 of the rows that see it, nothing is
    written outside a row's prefix, and the scores equal the one-call
    scorer's bit for bit."""
    w = workload(2)
    T = w["tokens"]
    rng = np.random.default_rng(77)
    R = 301
    pos = rng.integers(0, T, size=R).astype(np.int32)
    pos[:6] = [0, 3, 4, T - 1, T - 2, 203]
    pos[[10, 150, 300]] = [-1, T, 1 << 30]
    q = w["queries"][rng.choice(len(w["pos"]), size=R, replace=False)]
    pooled = oracle_pooled(2).copy()
    pooled[50] = 0x7FC0
    cols = T // 4 + 3
    sentinel = np.float32(-7.25)
    note(f"score long batch: {R} rows over {T} tokens, score_cols {cols}")
    got, st = gpu_scores_prepped(w, u16_dev(pooled), pos=pos, q=q, score_cols=cols, sentinel=sentinel)
    assert st == O.STATUS_BAD_POSITION
    ref, st2 = gpu_scores(w, u16_dev(pooled), pos=pos, q=q, score_cols=cols, sentinel=sentinel)
    assert st2 == O.STATUS_BAD_POSITION
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    valid = (pos >= 0) & (pos < T)
    assert np.all(got[~valid] == sentinel)
    vrows = np.nonzero(valid)[0]
    qhat = O.prep_queries(q[vrows], pos[vrows], w["q_norm_w"], w["rotary_dim"], w["theta"], w["eps"])
    want = O.score_rows(qhat, pos[vrows], pooled, T)
    worst = 0.0
    for i, r in enumerate(vrows):
        s = want[i]
        n = len(s)
        assert np.all(got[r, n:] == sentinel), "wrote past the visible prefix"
        if n > 50:
            assert np.isnan(got[r, 50]) and np.isnan(s[50])
            s = np.delete(s, 50)
            g = np.delete(got[r, :n], 50)
        else:
            g = got[r, :n]
        if len(s):
            worst = max(worst, float(np.max(np.abs(g.astype(np.float64) - s))))
    note(f"  max |gpu - oracle| = {worst:.3e}")
    assert worst <= SCORE_ATOL


@pytest.mark.parametrize("R", [1152, 3072, 4096])
def test_ring_scorer_row_group_shares(R):
    """The ring scorer deals its 128-row groups to the 8 XCDs by group count:
    9 groups (1152 rows) in contiguous eighths of the tasks, 24 groups (3072
    rows) every eighth group, 32 groups (4096 rows) mirror pairs of 16-group
    bands.  On causal rows over 4k tokens (positions from 0 to the last
    token) every score equals the one-call scorer's bit for bit, columns past
    each prefix keep their sentinel, and 64 sampled rows are within the bound
    of the oracle."""
    w = workload(2)
    T = w["tokens"]
    rng = np.random.default_rng(1000 + R)
    pos = np.sort(rng.integers(0, T, size=R)).astype(np.int32)
    pos[-1] = T - 1
    q = w["queries"][rng.integers(0, len(w["pos"]), size=R)]
    pooled = oracle_pooled(2)
    cols = T // 4
    sentinel = np.float32(-7.25)
    note(f"ring shares: {R} rows ({-(-R // 128)} groups) over {T} tokens")
    got, st = gpu_scores_prepped(w, u16_dev(pooled), pos=pos, q=q, score_cols=cols, sentinel=sentinel)
    ref, st2 = gpu_scores(w, u16_dev(pooled), pos=pos, q=q, score_cols=cols, sentinel=sentinel)
    assert st == 0 and st2 == 0
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    n = (pos.astype(np.int64) + 1) // 4
    assert np.all(got[np.arange(cols)[None, :] >= n[:, None]] == sentinel)
    rows = rng.choice(R, size=64, replace=False)
    qhat = O.prep_queries(q[rows], pos[rows], w["q_norm_w"], w["rotary_dim"], w["theta"], w["eps"])
    want = O.score_rows(qhat, pos[rows], pooled, T)
    worst = 0.0
    for i, r in enumerate(rows):
        if len(want[i]):
            worst = max(worst, float(np.max(np.abs(got[r, : len(want[i])].astype(np.float64) - want[i]))))
    note(f"  max |gpu - oracle| over 64 rows = {worst:.3e}")
    assert worst <= SCORE_ATOL


def test_score_full_prefill_chunk_ring_equals_one_call_scorer():
    """Every score of the 8192-row prefill chunk over 64k (125.8 M pairs, the
    benchmarked launch: the 128-row ring scorer, one step loop over 32-block
    tiles streamed through a four-stage LDS ring) equals the one-call
    scorer's bit for bit (a different kernel: 32 rows per workgroup, queries
    normed and roped in its prologue), and the columns past each row's
    prefix keep their sentinel.  Compared on the device; the oracle checks
    of the same launch are in test_end_to_end_masks and
    test_ring_scorer_prefill_rows_within_bound."""
    w = workload(5)
    T = w["tokens"]
    rows = len(w["pos"])
    cols = T // 4
    note(f"score full chunk: {rows} rows over {T} tokens, ring vs one-call scorer")
    pooled = gpu_pool(w)
    pos = i32_dev(w["pos"])
    qhat, s0 = gpu_prep(w)
    assert s0 == 0
    a = torch.full((rows * cols,), -7.25, dtype=torch.float32, device=DEV)
    b = torch.full((rows * cols,), -7.25, dtype=torch.float32, device=DEV)
    st = status_word()
    qsa.qsa_score_prepped(qhat, pos, pooled, T, a, cols, st)
    qsa.qsa_score_rows(u16_dev(w["queries"].reshape(rows, 512)), pos, u16_dev(w["q_norm_w"]), w["rotary_dim"],
                       w["theta"], w["eps"], pooled, T, b, cols, st)
    assert qsa.check_status(st) == 0
    same = torch.equal(a.view(torch.int32), b.view(torch.int32))
    if not same:
        bad = torch.nonzero((a.view(torch.int32) != b.view(torch.int32)).view(rows, cols).any(dim=1)).flatten()
        raise AssertionError(f"ring and one-call scores differ in rows {bad[:8].tolist()}")
    n = (torch.from_numpy(w["pos"]).to(DEV).to(torch.int64) + 1) // 4
    col = torch.arange(cols, device=DEV)
    outside = col[None, :] >= n[:, None]
    assert bool((a.view(rows, cols)[outside] == -7.25).all())


def test_ring_scorer_prefill_rows_within_bound():
    """The ring scorer (128 rows per workgroup, the prefill launch) on 1024
    consecutive rows of the prefill chunk over 64k, against the oracle:
    15.8 M scores within 5e-3, nothing written past any row's prefix."""
    from tests import oracle_cache as C
    w = workload(5)
    T = w["tokens"]
    cols = T // 4
    pos, q, want, _, _, _ = C.prefill_slice()
    note(f"ring scorer vs oracle: {len(pos)} rows over {T} tokens")
    got, st = gpu_scores_prepped(w, u16_dev(C.pooled(5)), pos=pos, q=q, score_cols=cols)
    assert st == 0
    n = (pos.astype(np.int64) + 1) // 4
    inside = np.arange(cols)[None, :] < n[:, None]
    assert np.all(got[~inside] == np.float32(-7.25)), "wrote past the visible prefix"
    worst = float(np.max(np.abs(got[inside].astype(np.float64) - want[inside])))
    note(f"  max |gpu - oracle| = {worst:.3e}")
    assert worst <= SCORE_ATOL


def _huge_dot_inputs(R, seed=31):
    """Prepared queries and pooled keys whose head dots reach past half the
    f32 range (one head: 128 * (1.5e18)^2 ~ 2.9e38 < FLT_MAX) or overflow
    to -Inf (a key of -1.5e19 against a query of 1.5e18), beside ordinary
    N(0, 1) values.  T = 256 tokens, rows at the last position."""
    rng = np.random.default_rng(seed)
    T = 256
    nb = T // 4
    keys = rng.standard_normal((nb, 128)).astype(np.float32)
    keys[5] = 1.5e18
    keys[9] = -1.5e19
    keys[20] = 1.5e18
    keys[20, :64] = -1.5e18          # a zero-sum huge key: the dot cancels exactly
    qs = rng.standard_normal((R, 4, 128)).astype(np.float32)
    qs[:, 0] = 1.5e18                 # head 0: 2.9e38 on block 5, -Inf on block 9
    qs[::3, 1] = 1.5e18               # every third row: two such heads, the sum overflows
    qs[1::3, 2] = -1.5e18             # others: a huge negative head (relu 0)
    pos = np.full(R, T - 1, dtype=np.int32)
    return T, synth.bf16_bits(keys), synth.bf16_bits(qs), pos


def _compare_huge(got, want, pos):
    """Finite oracle scores: within 5e-3 + 2^-16 relative (f32 accumulation
    of 128 products near 1e36); non-finite ones: the same class."""
    for r, s in enumerate(want):
        n = len(s)
        g = got[r, :n].astype(np.float64)
        fin = np.isfinite(s)
        assert np.array_equal(np.isnan(g[~fin]), np.isnan(s[~fin])), r
        assert np.array_equal(g[~fin & ~np.isnan(s)], s[~fin & ~np.isnan(s)].astype(np.float64)), r
        assert np.all(np.isfinite(g[fin])), (r, np.nonzero(~np.isfinite(g) & fin)[0][:5])
        err = np.abs(g[fin] - s[fin])
        assert np.all(err <= 5e-3 + 2.0 ** -16 * np.abs(s[fin])), (r, float(err.max()))


@pytest.mark.parametrize("R", [1, 4, 8, 70, 130])
def test_score_head_dots_past_half_range_and_minus_inf(R):
    """relu is a comparison: a head dot of -Inf contributes 0, and head dots
    above 2^127 (whose doubled relu terms would overflow) keep their finite
    score, as in the oracle; two such heads overflow the f32 head sum to
    +Inf there too.  Prepared queries through the streaming scorer (1 and 4
    rows), the decode kernels (8 and 70 rows) and the ring scorer (130
    rows)."""
    T, keys, qs, pos = _huge_dot_inputs(R)
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", RuntimeWarning)
        want = O.score_rows(qs, pos, keys, T)
    assert any(np.isinf(s).any() for s in want) and all(np.isfinite(s[5]) for s in want[1::3])
    cols = T // 4
    scores = torch.full((R * cols,), -7.25, dtype=torch.float32, device=DEV)
    st = status_word()
    note(f"score: huge head dots, {R} prepared rows")
    qsa.qsa_score_prepped(u16_dev(qs.reshape(R, 4, 128)), i32_dev(pos), u16_dev(keys), T, scores, cols, st)
    assert qsa.check_status(st) == 0
    _compare_huge(scores.cpu().numpy().reshape(R, cols), want, pos)


def test_score_rows_huge_norm_weights():
    """The one-call scorer with a (1 + w) query weight of 1.5e18 on every
    channel and no rotary channels.  Head 0 is constant (normed to 1.5e18 on
    every channel), heads 1 and 2 one-hot with opposite signs (1.7e19 on one
    channel), head 3 zero: against the constant keys head 0 reaches 2.9e38
    (and the relu sum 3.1e38, whose doubled form overflows) or -Inf, whose
    doubled form is NaN; the oracle's finite scores stay finite and within
    bound.  Every dot is deterministic: no partial sum of any accumulation
    order overflows unless the exact one does."""
    R = 40
    T, keys, _, pos = _huge_dot_inputs(R)
    q = np.zeros((R, 4, 128), np.float32)
    q[:, 0] = 1.0
    q[:, 1, 7] = 1.0
    q[:, 2, 9] = -1.0
    qb = synth.bf16_bits(q)
    wq = synth.bf16_bits(np.full(128, 1.5e18, np.float32))
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", RuntimeWarning)
        qhat = O.prep_queries(qb, pos, wq, 0, 1e4, 1e-6)
        want = O.score_rows(qhat, pos, keys, T)
    cols = T // 4
    scores = torch.full((R * cols,), -7.25, dtype=torch.float32, device=DEV)
    st = status_word()
    note("score: one-call scorer, huge query norm weight")
    qsa.qsa_score_rows(u16_dev(qb.reshape(R, 512)), i32_dev(pos), u16_dev(wq), 0, 1e4, 1e-6, u16_dev(keys), T,
                       scores, cols, st)
    assert qsa.check_status(st) == 0
    _compare_huge(scores.cpu().numpy().reshape(R, cols), want, pos)


def _wide_range(shape, rng):
    """bf16 values with magnitudes spread over 2^-60 .. 2^60 (the double sum
    of their squares is no longer exact), random signs, some zeros."""
    mag = np.exp2(rng.uniform(-60, 60, size=shape)).astype(np.float32)
    v = mag * np.where(rng.random(shape) < 0.5, -1.0, 1.0).astype(np.float32)
    v[rng.random(shape) < 0.02] = 0.0
    return v.astype(np.float32)


def test_pool_and_prep_wide_dynamic_range_bit_exact():
    """Keys whose channels span 2^120 in magnitude within a block, keys with
    one outlier channel (1e3 against 1e-4: a span past 2^18), and queries of
    the same kinds: pooled keys and prepared queries bit-exact against the
    oracle (both sum the squares in double; past a 2^18 span the sum is
    rounded, in different orders, and these seeded inputs are checked to
    give identical bf16 outputs)."""
    rng = np.random.default_rng(41)
    T = 4096
    raw = _wide_range((T, 128), rng)
    out = rng.standard_normal((T // 2, 128)).astype(np.float32) * np.float32(1e-4)
    out[:, 17] = 1e3
    raw[: T // 2] = out
    rawb = synth.bf16_bits(raw)
    wk = synth.bf16_bits((rng.standard_normal(128) * 0.05).astype(np.float32))
    w = dict(workload(2), raw_keys=rawb, k_norm_w=wk)
    note("pool: wide dynamic range")
    got = u16_host(gpu_pool(w))
    want = O.pool_keys(rawb, wk, 64, 1e4, 1e-6)
    diff = np.nonzero(got != want)
    assert len(diff[0]) == 0, (len(diff[0]), diff[0][:8], diff[1][:8])
    R = 256
    q = _wide_range((R, 4, 128), rng)
    q[: R // 2, :, :] = rng.standard_normal((R // 2, 4, 128)).astype(np.float32) * np.float32(1e-4)
    q[: R // 2, :, 3] = 1e3
    qb = synth.bf16_bits(q)
    pos = rng.integers(0, T, size=R).astype(np.int32)
    note("prep: wide dynamic range")
    qhat, st = gpu_prep(dict(w, queries=qb), pos=pos, q=qb)
    assert st == 0
    wantq = O.prep_queries(qb, pos, w["q_norm_w"], 64, 1e4, 1e-6)
    diff = np.nonzero(u16_host(qhat) != wantq)
    assert len(diff[0]) == 0, (len(diff[0]), diff[0][:8])


# ------------------------------------------------------------ end to end ----

@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_end_to_end_masks(wid):
    w = workload(wid)
    T = w["tokens"]
    cols = T // 4
    note(f"end to end: workload {wid}")
    pooled_dev = gpu_pool(w)
    if len(w["dup_blocks"]):
        p = u16_host(pooled_dev)
        pooled_dev = u16_dev(synth.apply_dups(p, w["dup_blocks"]))
    scores, st = gpu_scores_prepped(w, pooled_dev)
    assert st == 0
    mask, st = gpu_select(scores, cols, w["pos"], T, w["budget"])
    assert st == 0
    rows = sample_rows(wid)
    want_scores = oracle_sample_scores(wid)
    # the scores of this launch (for the 8192-row chunk: the benchmarked ring
    # scorer over the whole batch) on the sampled rows, against the oracle
    worst = 0.0
    for i, r in enumerate(rows):
        n = len(want_scores[i])
        if n:
            worst = max(worst, float(np.max(np.abs(scores[r, :n].astype(np.float64) - want_scores[i]))))
    note(f"  max |gpu - oracle| over the sampled rows = {worst:.3e}")
    assert worst <= SCORE_ATOL
    want_dense = dense(want_scores, cols)
    want_mask, _ = O.select_mask(want_dense, cols, w["pos"][rows], T, w["budget"])
    loose = 0
    for i, r in enumerate(rows):
        p = int(w["pos"][r])
        check_structure(mask[r], scores[r], p, T, w["budget"])
        if np.array_equal(mask[r], want_mask[i]):
            continue
        n = (p + 1) // 4
        keep = min(w["budget"] // 4, n)
        s = want_scores[i]
        cut = np.sort(s)[::-1][keep - 1]
        gb = mask[r][: 4 * n].reshape(n, 4)[:, 0]
        wb = want_mask[i][: 4 * n].reshape(n, 4)[:, 0]
        diff = np.nonzero(gb != wb)[0]
        assert np.all(np.abs(s[diff].astype(np.float64) - cut) <= SCORE_ATOL), (r, diff[:8])
        loose += 1
    note(f"  rows differing only at the cut: {loose} of {len(rows)}")


def test_repeat_launches_are_bit_identical():
    w = workload(3)
    pooled_a = u16_host(gpu_pool(w))
    pooled_b = u16_host(gpu_pool(w))
    assert np.array_equal(pooled_a, pooled_b)
    s1, _ = gpu_scores(w, u16_dev(pooled_a))
    s2, _ = gpu_scores(w, u16_dev(pooled_a))
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    T = w["tokens"]
    m1, _ = gpu_select(s1, T // 4, w["pos"], T, 2048)
    for _ in range(3):
        m2, _ = gpu_select(s1, T // 4, w["pos"], T, 2048)
        assert np.array_equal(m1, m2)
