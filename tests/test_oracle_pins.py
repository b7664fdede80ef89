"""Pins of the CPU oracle to facts fixed outside it: library routines, closed
forms, special cases and invariants.  CPU only.

Each test names the mistake it would catch in the oracle.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden_values():
    vals = {}
    with open(os.path.join(GOLDEN, "closed_forms.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, value = line.split()[:2]
            vals[name] = float(value)
    return vals


def torch_bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


# ---------------------------------------------------------------- bf16 ------

def test_bf16_rounding_matches_torch_on_random_and_edge_patterns():
    """Library routine: torch's CPU float32 -> bfloat16 conversion (RNE)."""
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    edges = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x00000001, 0x807FFFFF,
                      0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F80FFFF, 0x7F7FFFFF,
                      0x7F7F8000, 0x7F7F7FFF, 0x00008000, 0x00018000, 0x0000FFFF],
                     dtype=np.uint32)
    x = np.concatenate([bits, edges]).view(np.float32)
    finite = np.isfinite(x) | np.isinf(x)
    ours = O.bf16_from_f32(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours[finite], ref[finite])
    nan = np.isnan(x)
    assert np.all(np.isnan(O.f32_from_bf16(ours[nan])))


def test_bf16_widening_is_exact():
    b = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f = O.f32_from_bf16(b)
    ok = ~np.isnan(f)
    assert np.array_equal(O.bf16_from_f32(f[ok]), b[ok])


# ---------------------------------------------------------------- rotary ----

def test_inv_freq_closed_forms():
    """theta^(-2i/d): i=0 -> 1, 2i/d = 1/4 -> theta^-1/4, 2i/d = 1/2 -> theta^-1/2.
    Catches a wrong exponent (e.g. -i/d or -2i/(d/2))."""
    f = O.rope_inv_freq(64, 10000.0)
    assert f.shape == (32,) and f.dtype == np.float32
    assert f[0] == np.float32(1.0)
    assert f[8] == np.float32(0.1)
    assert f[16] == np.float32(0.01)
    assert f[24] == np.float32(0.001)
    assert np.all(np.diff(f) < 0)
    g = O.rope_inv_freq(128, 1e7)
    assert g[32] == np.float32(1e7 ** -0.5)


def test_cos_sin_position_zero_and_known_angles():
    inv = O.rope_inv_freq(64, 10000.0)
    c, s = O.rope_cos_sin(np.array([0]), inv)
    assert np.all(c == 1.0) and np.all(s == 0.0)
    # frequency 0 is 1 rad/token: angle = P exactly in f32
    for P in (1, 3, 1000, 262143):
        c, s = O.rope_cos_sin(np.array([P]), inv)
        assert c[0, 0] == torch_bf16(np.float32(math.cos(P)))
        assert s[0, 0] == torch_bf16(np.float32(math.sin(P)))


def test_rope_position_zero_is_identity_in_value():
    rng = np.random.default_rng(1)
    x = synth.bf16_bits(rng.standard_normal((16, 128)).astype(np.float32))
    y = O.rope_partial(x, np.zeros(16, dtype=np.int64), 64, O.rope_inv_freq(64, 1e4))
    assert np.array_equal(O.f32_from_bf16(x), O.f32_from_bf16(y))


@pytest.mark.parametrize("P", [1, 7, 4096, 65532])
def test_rope_rotates_pairs_i_and_i_plus_half(P):
    """A one-hot in channel i comes out as (a cos, a sin) in channels
    (i, i+32); a one-hot in i+32 as (-a sin, a cos); channels >= 64 pass.
    Catches an interleaved pair layout, a wrong sign, rotating all 128."""
    inv = O.rope_inv_freq(64, 10000.0)
    for i in (0, 5, 31):
        ang = np.float32(P) * inv[i]
        c = torch_bf16(np.float32(math.cos(float(ang))))
        s = torch_bf16(np.float32(math.sin(float(ang))))
        x = np.zeros(128, dtype=np.float32)
        x[i] = 1.0
        x[100] = 3.0
        y = O.f32_from_bf16(O.rope_partial(synth.bf16_bits(x)[None], np.array([P]), 64, inv))[0]
        assert y[i] == c and y[i + 32] == s and y[100] == 3.0
        assert np.count_nonzero(y) <= 3
        x = np.zeros(128, dtype=np.float32)
        x[i + 32] = 1.0
        y = O.f32_from_bf16(O.rope_partial(synth.bf16_bits(x)[None], np.array([P]), 64, inv))[0]
        assert y[i] == -s and y[i + 32] == c


# ---------------------------------------------------------------- norm ------

def test_rms_norm_closed_forms():
    g = golden_values()
    w0 = np.zeros(128, dtype=np.uint16)
    x = np.zeros(128, dtype=np.float32)
    x[17] = 2.0
    y = O.f32_from_bf16(O.rms_norm_1pw(synth.bf16_bits(x), w0, 1e-6))
    assert y[17] == g["onehot_norm_a2"] and np.count_nonzero(y) == 1
    w = np.zeros(128, dtype=np.float32)
    w[17] = 0.5
    y = O.f32_from_bf16(O.rms_norm_1pw(synth.bf16_bits(x), synth.bf16_bits(w), 1e-6))
    assert y[17] == g["onehot_norm_a2_w05"]
    y = O.f32_from_bf16(O.rms_norm_1pw(synth.bf16_bits(np.full(128, 3.0, np.float32)), w0, 1e-6))
    assert np.all(y == g["const_norm_c3"])
    y = O.f32_from_bf16(O.rms_norm_1pw(synth.bf16_bits(np.full(128, 1e-3, np.float32)), w0, 1e-6))
    assert np.all(y == g["const_norm_eps"])


def test_rms_norm_matches_unit_rms_within_bf16():
    """Random rows: the output (w = 0) has mean square 1 up to bf16 rounding."""
    rng = np.random.default_rng(2)
    x = synth.bf16_bits(rng.standard_normal((64, 128)).astype(np.float32) * 7)
    y = O.f32_from_bf16(O.rms_norm_1pw(x, np.zeros(128, np.uint16), 1e-6)).astype(np.float64)
    ms = np.mean(y * y, axis=1)
    assert np.all(np.abs(ms - 1.0) < 2e-3)


# ---------------------------------------------------------------- pool ------

def _raw(rows):
    return synth.bf16_bits(np.asarray(rows, dtype=np.float32))


def test_block_mean_is_a_mean_rounded_to_bf16():
    r = np.zeros((8, 128), dtype=np.float32)
    r[0:4, 0] = [1, 2, 3, 4]
    r[0:4, 1] = [1, 1, 1, 1 + 2**-7]           # 1 + 2^-9 -> 1.0
    r[0:4, 2] = [1, 1, 1 + 2**-7, 1 + 2**-7]   # 1 + 2^-8 (tie) -> 1.0
    r[0:4, 3] = [1, 1 + 2**-7, 1 + 2**-7, 1 + 2**-7]  # 1 + 3*2^-9 -> 1 + 2^-7
    r[4:8, 0] = [2**24, 1, 1, -2**24]           # f32 token-order sum: 0
    m = O.f32_from_bf16(O.block_mean(_raw(r), 0, 2))
    assert m[0, 0] == 2.5
    assert m[0, 1] == 1.0 and m[0, 2] == 1.0 and m[0, 3] == np.float32(1 + 2**-7)
    assert m[1, 0] == 0.0


def test_pool_constant_block_closed_form():
    """Four equal all-ones tokens, w = 0: mean 1, norm 1, then RoPE at 4b:
    channels i < 32 hold rb(c - s), i+32 hold rb(c + s), the rest stay 1."""
    T = 64
    raw = _raw(np.ones((T, 128), dtype=np.float32))
    pooled = O.f32_from_bf16(O.pool_keys(raw, np.zeros(128, np.uint16), 64, 1e4, 1e-6))
    inv = O.rope_inv_freq(64, 1e4)
    for b in (0, 1, 9, 15):
        for i in (0, 3, 31):
            ang = float(np.float32(4 * b) * inv[i])
            c = torch_bf16(np.float32(math.cos(ang)))
            s = torch_bf16(np.float32(math.sin(ang)))
            assert pooled[b, i] == torch_bf16(np.float32(c - s))
            assert pooled[b, i + 32] == torch_bf16(np.float32(c + s))
        assert np.all(pooled[b, 64:] == 1.0)


def test_pool_first_block_offset_matches_whole_pool():
    w = synth.make_workload(1)
    allp = O.pool_keys(w["raw_keys"], w["k_norm_w"], 64, 1e4, 1e-6)
    part = O.pool_keys(w["raw_keys"], w["k_norm_w"], 64, 1e4, 1e-6, first_block=37, n_blocks=20)
    assert np.array_equal(allp[37:57], part)


def test_pool_scale_invariance_up_to_eps():
    """RMSNorm removes a power-of-two scale of the raw keys (exact in bf16)
    except through eps: nearly every pooled element is bit-identical."""
    rng = np.random.default_rng(3)
    raw = rng.standard_normal((256, 128)).astype(np.float32)
    a = O.pool_keys(_raw(raw), np.zeros(128, np.uint16), 64, 1e4, 1e-6)
    b = O.pool_keys(_raw(raw * 4), np.zeros(128, np.uint16), 64, 1e4, 1e-6)
    assert np.mean(a == b) > 0.99


# ---------------------------------------------------------------- score -----

def _score_setup(q_rows, key_rows, pos, tokens, w_zero=True):
    wk = np.zeros(128, np.uint16)
    pooled = O.pool_keys(_raw(key_rows), wk, 64, 1e4, 1e-6)
    qhat = O.prep_queries(_raw(q_rows), np.asarray(pos), wk, 64, 1e4, 1e-6)
    return O.score_rows(qhat, np.asarray(pos), pooled, tokens)


def test_score_closed_forms_head_sum_relu_and_scale():
    g = golden_values()
    T = 16
    keys = np.ones((T, 128), dtype=np.float32)
    q = np.zeros((2, 4, 128), dtype=np.float32)
    q[0, :, 100] = 2.0           # every head: pass-through one-hot
    q[1, :, 100] = 2.0
    q[1, 0, 100] = -2.0          # head 0 dot is negative
    s = _score_setup(q, keys, [15, 15], T)
    assert len(s[0]) == 4
    np.testing.assert_allclose(s[0], g["score_four_heads"], rtol=2e-7)
    np.testing.assert_allclose(s[1], g["score_three_heads"], rtol=2e-7)
    assert not np.any(np.isclose(s[1], g["score_post_sum_relu_fault"], rtol=1e-3))


@pytest.mark.parametrize("i", [0, 5, 20])
def test_score_rope_anchor_is_block_first_token(i):
    """q and every key one-hot in rotary channel i: the dot is about
    128 cos(theta_i (p - 4b)), so the anchor (4b, not 4b+3) and the pair
    layout are both visible in the score."""
    T = 256
    keys = np.zeros((T, 128), dtype=np.float32)
    keys[:, i] = 2.0
    q = np.zeros((3, 4, 128), dtype=np.float32)
    q[:, :, i] = 2.0
    pos = np.array([255, 130, 61])
    s = _score_setup(q, keys, pos, T)
    inv = O.rope_inv_freq(64, 1e4)
    for r, p in enumerate(pos):
        b = np.arange(len(s[r]))
        want = 4 * 128 * np.cos(np.float64(inv[i]) * (p - 4 * b)) / math.sqrt(128)
        want = np.maximum(want, 0)
        assert np.max(np.abs(s[r] - want)) < 0.6, (r, np.max(np.abs(s[r] - want)))
        if i == 0:
            wrong = np.maximum(4 * 128 * np.cos(1.0 * (p - 4 * b - 3)) / math.sqrt(128), 0)
            assert np.max(np.abs(s[r] - wrong)) > 5


def test_score_relative_position_invariance():
    """Shifting a query and a key block by the same 4*d tokens keeps the
    score up to bf16 rounding of cos/sin."""
    rng = np.random.default_rng(4)
    T = 1024
    keys = np.zeros((T, 128), dtype=np.float32)
    blk = rng.standard_normal((4, 128)).astype(np.float32)
    keys[8:12] = blk          # block 2
    keys[808:812] = blk       # block 202 = 2 + 200
    q = rng.standard_normal((2, 4, 128)).astype(np.float32)
    q[1] = q[0]
    s = _score_setup(q, keys, [40, 840], T)
    a, b = s[0][2], s[1][202]
    assert abs(a - b) < 0.02 * max(1.0, abs(a)), (a, b)


def test_score_nan_poison_reaches_exactly_the_rows_that_see_the_block():
    w = synth.make_workload(1)
    raw = w["raw_keys"].copy()
    raw[4 * 50 + 2, 7] = 0x7FC0  # NaN in block 50
    pooled = O.pool_keys(raw, w["k_norm_w"], 64, 1e4, 1e-6)
    assert np.all(np.isnan(O.f32_from_bf16(pooled[50])))
    assert not np.any(np.isnan(O.f32_from_bf16(np.delete(pooled, 50, axis=0))))
    pos = np.array([199, 200, 202, 203, 204, 511])
    qhat = O.prep_queries(w["queries"][:6], pos, w["q_norm_w"], 64, 1e4, 1e-6)
    s = O.score_rows(qhat, pos, pooled, 512)
    for r, p in enumerate(pos):
        n = (p + 1) // 4
        assert len(s[r]) == n
        if n > 50:
            assert np.isnan(s[r][50]) and np.all(np.isfinite(np.delete(s[r], 50)))
        else:
            assert np.all(np.isfinite(s[r]))


def test_score_out_of_range_row_is_empty():
    w = synth.make_workload(1, rows=3)
    pooled = O.pool_keys(w["raw_keys"], w["k_norm_w"], 64, 1e4, 1e-6)
    pos = np.array([-1, 512, 5])
    qhat = O.prep_queries(w["queries"], pos, w["q_norm_w"], 64, 1e4, 1e-6)
    s = O.score_rows(qhat, pos, pooled, 512)
    assert len(s[0]) == 0 and len(s[1]) == 0 and len(s[2]) == 1


# ---------------------------------------------------------------- select ----

def load_geometry():
    rows = []
    with open(os.path.join(GOLDEN, "select_geometry.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append(tuple(int(v) for v in line.split()))
    return rows


def test_select_geometry_golden():
    rng = np.random.default_rng(5)
    for p, budget, blocks, tail, keep, pop in load_geometry():
        assert O.visible_blocks(p) == blocks and (p + 1) % 4 == tail
        s = rng.standard_normal(max(blocks, 1)).astype(np.float32)
        m, st = O.select_mask_row(s, p, p + 5, budget)
        assert st == 0
        assert int(m.sum()) == pop
        assert np.all(m[p + 1:] == 0)
        assert np.all(m[4 * blocks: p + 1] == 1)


def check_structure(mask_row, scores, p, tokens, budget):
    """The invariants of a valid mask row (selection contract).  Returns the
    kept block set; asserts on any violation."""
    n = (p + 1) // 4
    keep = min(budget // 4, n)
    assert mask_row.shape == (tokens,)
    assert set(np.unique(mask_row)).issubset({0, 1})
    assert np.all(mask_row[p + 1:] == 0), "bit past p"
    assert np.all(mask_row[4 * n: p + 1] == 1), "tail"
    blocks = mask_row[: 4 * n].reshape(n, 4) if n else np.zeros((0, 4), np.uint8)
    assert np.all((blocks.sum(1) == 0) | (blocks.sum(1) == 4)), "partial block"
    kept = np.nonzero(blocks[:, 0])[0]
    assert len(kept) == keep, "count"
    assert int(mask_row.sum()) == 4 * keep + (p + 1) % 4
    if n <= budget // 4:
        assert np.all(mask_row[: p + 1] == 1)
    s = np.where(scores[:n] == 0, np.float32(0), scores[:n])
    excl = np.setdiff1d(np.arange(n), kept)
    if len(kept) and len(excl):
        cut = s[kept].min()
        assert cut >= s[excl].max(), "order"
        eq_kept = kept[s[kept] == cut]
        eq_excl = excl[s[excl] == cut]
        if len(eq_excl):
            assert eq_kept.max() < eq_excl.min(), "tie fill not ascending"
    return kept


def rank_definition(scores, keep):
    """O(n^2): b is kept iff fewer than keep blocks precede it in the order."""
    s = np.where(scores == 0, np.float32(0), scores)
    n = len(s)
    out = []
    for b in range(n):
        ahead = np.sum((s > s[b]) | ((s == s[b]) & (np.arange(n) < b)))
        if ahead < keep:
            out.append(b)
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("kind", ["zeros", "ties", "lowbyte", "wild", "equal", "random"])
def test_select_fixtures_structure_and_rank_definition(kind):
    pos_list = (0, 1, 2, 3, 4, 67, 2050, 2051, 2052, 2055, 8191)
    scores, cols, pos, T = synth.selector_fixture(kind, positions=pos_list)
    mask, st = O.select_mask(scores, cols, pos, T, 2048)
    assert st == 0
    for r, p in enumerate(pos):
        kept = check_structure(mask[r], scores[r], int(p), T, 2048)
        n = (int(p) + 1) // 4
        if n <= 3000:
            assert np.array_equal(kept, rank_definition(scores[r, :n], min(512, n)))


def test_select_exhaustive_small_rows():
    """Every keep-subset of up to 12 blocks: exactly one is ordered before
    its complement; it is the oracle's."""
    import itertools
    rng = np.random.default_rng(6)
    for trial in range(300):
        n = int(rng.integers(1, 13))
        p = 4 * n - 1 + int(rng.integers(0, 4))
        budget = 4 * int(rng.integers(1, n + 2))
        grid = rng.integers(0, 4, size=n).astype(np.float32) * np.float32(0.5) - 0.5
        if trial % 3 == 0:
            grid = np.where(grid == 0, np.float32(-0.0), grid)
        keep = min(budget // 4, n)
        m, st = O.select_mask_row(grid, p, p + 1, budget)
        got = np.nonzero(m[: 4 * n].reshape(n, 4)[:, 0])[0]
        valid = []
        for sub in itertools.combinations(range(n), keep):
            inside = set(sub)
            ok = True
            for a in inside:
                for e in range(n):
                    if e in inside:
                        continue
                    sa, se = grid[a] + 0, grid[e] + 0
                    if not (sa > se or (sa == se and a < e)):
                        ok = False
            if ok:
                valid.append(sub)
        assert len(valid) == 1
        assert tuple(got) == valid[0]


def test_select_refuses_nonfinite_and_bad_positions():
    scores, cols, pos, T = synth.selector_fixture("poison", positions=(7, 11, 67, 2055, 4095, 9))
    mask, st = O.select_mask(scores, cols, pos, T, 2048)
    for r in range(len(pos)):
        n = (int(pos[r]) + 1) // 4
        bad = not np.all(np.isfinite(scores[r, :n]))
        assert bad == (r % 2 == 1)
        if bad:
            assert mask[r].sum() == 0
        else:
            check_structure(mask[r], scores[r], int(pos[r]), T, 2048)
    assert st == O.STATUS_NONFINITE_SCORE
    m, st = O.select_mask(np.zeros((2, 4), np.float32), 4, np.array([-1, 16]), 16, 64)
    assert st == O.STATUS_BAD_POSITION and m.sum() == 0


def test_select_ignores_nan_past_the_prefix_and_spare_columns():
    scores, cols, pos, T = synth.selector_fixture("random", positions=(67, 2055, 9), spare_cols=13)
    assert np.all(np.isnan(scores[:, T // 4:]))
    mask, st = O.select_mask(scores, cols, pos, T, 2048)
    assert st == 0
    for r, p in enumerate(pos):
        check_structure(mask[r], scores[r], int(p), T, 2048)


@pytest.mark.parametrize("budget", [0, -4, 6, 2052, 4096])
def test_select_refuses_bad_budget(budget):
    with pytest.raises(ValueError):
        O.select_mask(np.zeros((1, 4), np.float32), 4, np.array([15]), 16, budget)


def test_mutation_controls_are_caught_by_the_invariants():
    """The five selection faults of pull request 1178's mutation table
    (drop the tail, keep one fewer, keep one more, ignore causality, invert
    the order), planted in copies of the oracle's output, each fail the
    structural check."""
    scores, cols, pos, T = synth.selector_fixture("random", positions=(2054, 3000, 66, 4095))
    mask, _ = O.select_mask(scores, cols, pos, T, 2048)
    faults = {}
    for r, p in enumerate(pos):
        p = int(p)
        n = (p + 1) // 4
        keep = min(512, n)
        kept = np.nonzero(mask[r][: 4 * n].reshape(n, 4)[:, 0])[0]
        s = scores[r, :n]
        m = mask[r].copy(); m[4 * n: p + 1] = 0; faults[("tail", r)] = m
        if keep:
            worst = kept[np.argmin(s[kept])]
            m = mask[r].copy(); m[4 * worst: 4 * worst + 4] = 0; faults[("fewer", r)] = m
        excl = np.setdiff1d(np.arange(n), kept)
        if len(excl):
            best = excl[np.argmax(s[excl])]
            m = mask[r].copy(); m[4 * best: 4 * best + 4] = 1; faults[("more", r)] = m
        m = mask[r].copy(); m[p + 1:] = 1; faults[("causal", r)] = m
        inv = O.kept_blocks(-s, keep)
        m = np.zeros_like(mask[r])
        for b in inv:
            m[4 * b: 4 * b + 4] = 1
        m[4 * n: p + 1] = 1
        faults[("invert", r)] = m
    caught = 0
    for key, m in faults.items():
        r = key[1]
        if np.array_equal(m, mask[r]):
            continue  # the fault is a no-op on this row (e.g. all-kept row)
        with pytest.raises(AssertionError):
            check_structure(m, scores[r], int(pos[r]), T, 2048)
        caught += 1
    assert caught >= 15


# ------------------------------------------------------------ index lists ----

def check_index_list(idx_row, count, mask_row, p, budget):
    """An index row is the ascending list of the mask row's set tokens,
    4 keep + tail long, padded with -1 to budget + 3 entries."""
    n = (p + 1) // 4
    keep = min(budget // 4, n)
    assert idx_row.shape == (budget + 3,)
    assert count == 4 * keep + (p + 1) % 4, "count"
    assert np.all(idx_row[count:] == -1), "padding"
    got = idx_row[:count]
    assert np.all(np.diff(got) > 0), "not ascending"
    assert np.array_equal(got, np.flatnonzero(mask_row)), "tokens differ from the mask"


@pytest.mark.parametrize("kind", ["zeros", "ties", "lowbyte", "wild", "equal", "random", "poison"])
def test_select_indices_are_the_mask_tokens_in_order(kind):
    scores, cols, pos, T = synth.selector_fixture(kind)
    for budget in (2048, 64, 4):
        mask, mst = O.select_mask(scores, cols, pos, T, budget)
        idx, counts, ist = O.select_indices(scores, cols, pos, T, budget)
        assert ist == mst
        for r, p in enumerate(pos):
            if mask[r].sum() == 0 and counts[r] == 0:
                assert np.all(idx[r] == -1)  # refused row
                continue
            check_index_list(idx[r], int(counts[r]), mask[r], int(p), budget)


def test_select_indices_brute_force_small_rows():
    """Index lists of small rows from the O(n^2) rank definition: kept blocks
    ascending, each as its 4 tokens, then the tail."""
    rng = np.random.default_rng(8)
    for trial in range(200):
        n = int(rng.integers(0, 40))
        p = 4 * n + int(rng.integers(0, 4)) - (1 if n and trial % 5 == 0 else 0)
        p = max(p, 0)
        n = (p + 1) // 4
        budget = 4 * int(rng.integers(1, 20))
        s = (rng.integers(-3, 4, size=max(n, 1)) * 0.5).astype(np.float32)
        idx, count, st = O.select_indices_row(s, p, p + 1, budget)
        assert st == 0
        want = []
        for b in rank_definition(s[:n], min(budget // 4, n)):
            want.extend(range(4 * b, 4 * b + 4))
        want.extend(range(4 * n, p + 1))
        assert count == len(want) and np.array_equal(idx[:count], want)
        assert np.all(idx[count:] == -1)


def test_select_indices_under_budget_rows_are_the_prefix():
    for p in (0, 1, 2, 3, 4, 67, 2047, 2050):
        s = np.random.default_rng(p).standard_normal((p + 1) // 4 or 1).astype(np.float32)
        idx, count, st = O.select_indices_row(s, p, 4096, 2048)
        assert st == 0 and count == p + 1
        assert np.array_equal(idx[:count], np.arange(p + 1)) and np.all(idx[count:] == -1)


def test_select_indices_refusals_and_format_faults():
    idx, count, st = O.select_indices_row(np.array([1.0, np.nan], np.float32), 7, 8, 64)
    assert st == O.STATUS_NONFINITE_SCORE and count == 0 and np.all(idx == -1)
    idx, count, st = O.select_indices_row(np.zeros(4, np.float32), 16, 16, 64)
    assert st == O.STATUS_BAD_POSITION and count == 0 and np.all(idx == -1)
    # planted faults in a copy of a good list are caught by the checks
    scores, cols, pos, T = synth.selector_fixture("random", positions=(2054,))
    mask, _ = O.select_mask(scores, cols, pos, T, 2048)
    idx, counts, _ = O.select_indices(scores, cols, pos, T, 2048)
    c = int(counts[0])
    bad = {"no tail": (idx[0].copy(), c - 3), "unsorted": (idx[0].copy(), c),
           "block start": (idx[0].copy(), c)}
    bad["no tail"][0][c - 3:] = -1
    bad["unsorted"][0][[0, 5]] = bad["unsorted"][0][[5, 0]]
    bad["block start"][0][:c - 3] += 1
    for name, (row, cnt) in bad.items():
        with pytest.raises(AssertionError):
            check_index_list(row, cnt, mask[0], 2054, 2048)


# ---------------------------------------------------------------- K/V gather

def encoded_cache(n_pages, page_size, kv_dim, page_of_logical, salt):
    """A paged cache whose vector for token t carries t in its first three
    elements (base-256 digits, exact in bf16) and `salt` in the fourth, the
    rest a fixed pattern; page_of_logical maps logical page -> physical."""
    k = np.zeros((n_pages, page_size, kv_dim), dtype=np.uint16)
    for lp, pp in enumerate(page_of_logical):
        for s in range(page_size):
            t = lp * page_size + s
            digits = np.array([t & 255, (t >> 8) & 255, (t >> 16) & 255, salt], dtype=np.float32)
            k[pp, s, :4] = O.bf16_from_f32(digits)
            k[pp, s, 4:] = O.bf16_from_f32(np.float32(0.5))
    return k


def decode_token(vec):
    d = O.f32_from_bf16(vec[:4]).astype(np.int64)
    return int(d[0] + 256 * d[1] + 65536 * d[2]), int(d[3])


@pytest.mark.parametrize("shared", [True, False])
def test_gather_returns_each_listed_token_through_the_page_table(shared):
    """Every gathered vector decodes to the token the list names (K salt 1,
    V salt 2), in list order, whatever physical page holds it; entries past
    the count are zero; the identity table is row-major over the scratch."""
    rng = np.random.default_rng(11)
    page_size, kv_dim, rows, slots = 16, 24, 3, 48
    n_log = 40
    perm = rng.permutation(n_log + 7)[:n_log]  # physical pages, 7 unused
    kc = encoded_cache(n_log + 7, page_size, kv_dim, perm, 1)
    vc = encoded_cache(n_log + 7, page_size, kv_dim, perm, 2)
    if shared:
        table, tstride = perm.astype(np.int32), 0
    else:
        # row r's sequence is the shared one shifted by r pages
        table = np.concatenate([np.roll(perm, -r) for r in range(rows)]).astype(np.int32)
        tstride = n_log
    idx_stride = 50
    idx = np.full((rows, idx_stride), -1, np.int32)
    counts = np.array([45, 0, 17], np.int32)
    for r in range(rows):
        pick = np.sort(rng.choice(n_log * page_size, counts[r], replace=False))
        idx[r, : counts[r]] = pick
    ko, vo, tab, st = O.gather_kv(kc, vc, page_size, table, tstride, n_log, idx, idx_stride, counts,
                                  rows, slots)
    assert st == 0
    for r in range(rows):
        for i in range(slots):
            if i < counts[r]:
                t = int(idx[r, i])
                shift = 0 if shared else r * page_size
                want = (t + shift) % (n_log * page_size)
                assert decode_token(ko[r, i]) == (want, 1), (r, i)
                assert decode_token(vo[r, i]) == (want, 2), (r, i)
            else:
                assert not ko[r, i].any() and not vo[r, i].any()
        assert np.array_equal(tab[r], r * (slots // page_size) + np.arange(slots // page_size))


def test_gather_with_identity_paging_is_plain_indexing():
    """With physical page = logical page, the gather is numpy indexing of the
    flattened cache."""
    rng = np.random.default_rng(12)
    page_size, kv_dim, n_pages, rows, slots = 8, 16, 30, 4, 64
    kc = rng.integers(0, 1 << 16, size=(n_pages, page_size, kv_dim), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(n_pages, page_size, kv_dim), dtype=np.uint16)
    counts = rng.integers(0, slots + 1, size=rows).astype(np.int32)
    idx = np.full((rows, slots), -1, np.int32)
    for r in range(rows):
        idx[r, : counts[r]] = np.sort(rng.choice(n_pages * page_size, counts[r], replace=False))
    ko, vo, _, st = O.gather_kv(kc, vc, page_size, np.arange(n_pages, dtype=np.int32), 0, n_pages, idx,
                                slots, counts, rows, slots)
    assert st == 0
    flat_k, flat_v = kc.reshape(-1, kv_dim), vc.reshape(-1, kv_dim)
    for r in range(rows):
        c = counts[r]
        assert np.array_equal(ko[r, :c], flat_k[idx[r, :c]])
        assert np.array_equal(vo[r, :c], flat_v[idx[r, :c]])


def test_gather_bad_indices_and_counts_write_zeros_and_flag():
    page_size, kv_dim = 4, 8
    kc = np.full((3, page_size, kv_dim), 7, np.uint16)
    vc = np.full((3, page_size, kv_dim), 9, np.uint16)
    table = np.array([2, 5, 0], np.int32)  # logical page 1 -> physical 5: outside the cache
    idx = np.array([[0, -3, 5, 11, 12, 3, 0, 0]], np.int32)
    ko, vo, _, st = O.gather_kv(kc, vc, page_size, table, 0, 3, idx, 8, np.array([6]), 1, 8)
    assert st == O.STATUS_BAD_INDEX
    good = [0, 3, 5]  # entries 0 (t 0), 3 (t 11, page 0), 5 (t 3)
    for i in range(8):
        if i in good:
            assert np.all(ko[0, i] == 7) and np.all(vo[0, i] == 9)
        else:
            assert not ko[0, i].any() and not vo[0, i].any(), i
    for bad_count in (-1, 9):
        ko, _, _, st = O.gather_kv(kc, vc, page_size, table, 0, 3, np.zeros((1, 8), np.int32), 8,
                                   np.array([bad_count]), 1, 8)
        assert st == O.STATUS_BAD_INDEX
        assert np.all(ko[0, :8 if bad_count > 0 else 0] == 7) and not ko[0, 8:].any()
    # a list row shorter than the scratch bounds the count too
    ko, _, _, st = O.gather_kv(kc, vc, page_size, table, 0, 3, np.zeros((1, 6), np.int32), 6,
                               np.array([7]), 1, 8)
    assert st == O.STATUS_BAD_INDEX and np.all(ko[0, :6] == 7) and not ko[0, 6:].any()
