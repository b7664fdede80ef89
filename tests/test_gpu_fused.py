"""GPU parity of qsa_score_select_mask, the fused score -> select call.

It must give the same mask bytes and status bits as qsa_score_prepped
followed by qsa_select_mask, bit for bit, whatever its sampled thresholds do:
on the workloads, on ragged batches with bad positions and a NaN key, on
inputs built so that the sampled threshold is useless (every score equal;
only the sampled blocks score high), across the budget boundary, and with a
dirty, reused workspace.  One workload is also checked against the oracle
directly, to the end-to-end bar.
"""

import numpy as np
import pytest
import torch

import oracle as O
from tests.gpu_util import DEV, gpu_pool, gpu_prep, i32_dev, note, u16_dev, workload
from tests.test_oracle_pins import check_structure
import sparse_attention_token_qsa_amd as qsa

pytestmark = pytest.mark.gpu


def status_word():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def separate(qhat, pos, pooled, T, budget):
    """Mask (device) and status of qsa_score_prepped + qsa_select_mask."""
    rows = pos.numel()
    cols = max(T // 4, 1)
    scores = torch.full((rows * cols,), -3.5, dtype=torch.float32, device=DEV)
    st = status_word()
    qsa.qsa_score_prepped(qhat, pos, pooled, T, scores, cols, st)
    mask = torch.full((rows, T), 0xAB, dtype=torch.uint8, device=DEV)
    qsa.qsa_select_mask(scores, cols, pos, T, budget, mask, st)
    torch.cuda.synchronize()
    return mask, int(st.item())


def fused(qhat, pos, pooled, T, budget, ws=None, fill=0x5A, flags=False):
    """Mask (device) and status of qsa_score_select_mask; with flags=True
    also the per-row fallback flags it leaves in its workspace (1: the row
    was scored and selected in full)."""
    rows = pos.numel()
    n = qsa.qsa_score_select_workspace_bytes(rows, T, budget)
    if ws is None:
        ws = torch.full((max(n, 256),), fill, dtype=torch.uint8, device=DEV)
    assert ws.numel() >= n
    mask = torch.full((rows, T), 0xCD, dtype=torch.uint8, device=DEV)
    st = status_word()
    qsa.qsa_score_select_mask(qhat, pos, pooled, T, budget, mask, st, ws)
    torch.cuda.synchronize()
    if not flags:
        return mask, int(st.item())
    off = qsa.qsa_score_select_flags_offset(rows, T, budget)
    fl = ws[off: off + 4 * rows].view(torch.int32).cpu().numpy()
    return mask, int(st.item()), fl


def assert_same(qhat, pos, pooled, T, budget, label, ws=None, with_flags=False):
    note(f"fused vs separate: {label}: {pos.numel()} rows, {T} tokens, budget {budget}")
    out = fused(qhat, pos, pooled, T, budget, ws=ws, flags=with_flags)
    mf, sf = out[0], out[1]
    ms, ss = separate(qhat, pos, pooled, T, budget)
    assert sf == ss, (sf, ss)
    if not torch.equal(mf, ms):
        bad = torch.nonzero((mf != ms).any(dim=1)).flatten()[:8].tolist()
        raise AssertionError(f"{label}: masks differ in rows {bad}")
    return out


def prepped(w, pos=None, q=None):
    qhat, st = gpu_prep(w, pos=pos, q=q)
    return qhat


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_fused_equals_separate_on_workloads(wid):
    w = workload(wid)
    pooled = gpu_pool(w)
    qhat = prepped(w)
    pos = i32_dev(w["pos"])
    _, st = assert_same(qhat, pos, pooled, w["tokens"], w["budget"], f"workload {wid}")
    assert st == 0


def test_fused_ragged_rows_bad_positions_nan_key_odd_tokens():
    """301 rows (odd, not a multiple of 128), positions anywhere in a cache of
    65543 tokens (not a multiple of 16: the bytewise mask path), positions
    out of range, and a NaN key at block 50 (rows that see it are refused)."""
    w = workload(5)
    T = 65543
    rng = np.random.default_rng(5)
    pooled = gpu_pool(w)
    extra = torch.from_numpy(rng.standard_normal((1, 128)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    pooled = torch.cat([pooled, extra.view(torch.int16)], dim=0).contiguous()
    pooled[50] = 0x7FC0
    R = 301
    p = rng.integers(0, T, size=R).astype(np.int32)
    p[:8] = [0, 3, 4, 202, 203, T - 1, T - 2, 2050]
    p[[10, 150, 300]] = [-1, T, 1 << 30]
    q = w["queries"][rng.choice(len(w["pos"]), size=R, replace=False)]
    pos = i32_dev(p)
    qhat, _ = gpu_prep(dict(w, tokens=T), pos=p, q=q)
    _, st = assert_same(qhat, pos, pooled, T, 2048, "ragged")
    assert st == O.STATUS_BAD_POSITION | O.STATUS_NONFINITE_SCORE


def test_fused_fallback_when_every_score_ties():
    """Every block has the same key: each row's scores are all equal, every
    block reaches the sampled threshold and the candidate regions overflow,
    so every truncating row takes the full-score fallback (kept set: the
    lowest block indices)."""
    w = workload(5)
    rng = np.random.default_rng(6)
    T = 65536
    key = rng.standard_normal(128).astype(np.float32)
    pooled = torch.from_numpy(np.tile(key, (T // 4, 1))).to(DEV).to(torch.bfloat16).view(torch.int16).contiguous()
    sel = rng.choice(len(w["pos"]), size=256, replace=False)
    p = w["pos"][sel]
    qhat = prepped(w, pos=p, q=w["queries"][sel])
    mf, st, fl = assert_same(qhat, i32_dev(p), pooled, T, 2048, "all ties", with_flags=True)
    assert st == 0
    # every truncating row fell back to the full path
    n_all = (p.astype(np.int64) + 1) // 4
    assert np.array_equal(fl, (n_all > 512).astype(np.int32))
    # lowest indices win ties: blocks 0..511, then the tail
    row = mf[0].cpu().numpy()
    n = (int(p[0]) + 1) // 4
    assert row[: 4 * 512].all() and not row[4 * 512: 4 * n].any()


def test_fused_fallback_when_the_sample_overrates_the_row():
    """Only every 16th block (the sampled ones) scores high, so the sampled
    threshold admits n/16 < budget/4 blocks: the row falls back, and the kept
    set is those blocks plus the lowest-index ties among the rest."""
    rng = np.random.default_rng(7)
    T = 16384
    n = T // 4
    hi = rng.standard_normal(128).astype(np.float32)
    keys = np.tile(-hi, (n, 1))
    keys[::16] = hi
    keys[1::16] += 0.01 * rng.standard_normal((len(keys[1::16]), 128)).astype(np.float32)
    pooled = torch.from_numpy(keys).to(DEV).to(torch.bfloat16).view(torch.int16).contiguous()
    R = 130
    p = (T - 1 - np.arange(R)).astype(np.int32)
    qh = np.tile(np.concatenate([hi] * 4), (R, 1)).astype(np.float32)
    qh += 0.05 * rng.standard_normal(qh.shape).astype(np.float32)
    qhat = torch.from_numpy(qh).to(DEV).to(torch.bfloat16).view(torch.int16).reshape(R, 4, 128).contiguous()
    _, st, fl = assert_same(qhat, i32_dev(p), pooled, T, 2048, "overrated sample", with_flags=True)
    assert st == 0
    assert np.all(fl == 1), "every row's sampled threshold admits too few blocks"


def test_fused_rows_across_the_budget_and_tiny_caches():
    """Rows just under, at and over the budget (pairs that straddle it), rows
    with no complete block, a cache shorter than one block, budget 4."""
    w = workload(2)
    pooled = gpu_pool(w)
    T = w["tokens"]
    p = np.array([0, 1, 2, 3, 4, 7, 2043, 2044, 2045, 2046, 2047, 2048, 2049, 2050, 2051, 2052, 2055,
                  4095, 4094, 3000, 129], dtype=np.int32)
    sel = np.arange(len(p))
    qhat = prepped(w, pos=p, q=w["queries"][sel])
    for budget in (2048, 4, 64, 2044):
        assert_same(qhat, i32_dev(p), pooled, T, budget, f"budget {budget}")
    # caches of 3 and 7 tokens
    for Tt in (3, 7):
        pt = np.array([0, 1, 2, Tt - 1], dtype=np.int32)
        assert_same(qhat[:4].contiguous(), i32_dev(pt), pooled, Tt, 2048, f"{Tt}-token cache")


def test_fused_dirty_reused_workspace():
    """Contents on entry do not matter: a junk-filled workspace, then a
    second, smaller call on the same workspace."""
    w = workload(5)
    pooled = gpu_pool(w)
    T = w["tokens"]
    qhat = prepped(w)
    rows = len(w["pos"])
    n = qsa.qsa_score_select_workspace_bytes(rows, T, 2048)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=DEV)
    assert_same(qhat, i32_dev(w["pos"]), pooled, T, 2048, "junk workspace", ws=ws)
    sub = np.arange(1000, 1517)
    assert_same(qhat[sub].contiguous(), i32_dev(w["pos"][sub]), pooled, T, 2048, "reused workspace", ws=ws)


def test_fused_against_the_oracle():
    """Workload 1 (ties by duplicated keys) end to end against the oracle:
    masks may differ only at blocks within 5e-3 of a row's cut."""
    w = workload(1)
    T = w["tokens"]
    pooled_np = O.pool_keys(w["raw_keys"], w["k_norm_w"], w["rotary_dim"], w["theta"], w["eps"])
    import synth
    pooled_np = synth.apply_dups(pooled_np, w["dup_blocks"])
    qhat_np = O.prep_queries(w["queries"], w["pos"], w["q_norm_w"], w["rotary_dim"], w["theta"], w["eps"])
    want_scores = O.score_rows(qhat_np, w["pos"], pooled_np, T)
    cols = T // 4
    dense = np.full((len(w["pos"]), cols), np.nan, dtype=np.float32)
    for r, s in enumerate(want_scores):
        dense[r, : len(s)] = s
    want_mask, _ = O.select_mask(dense, cols, w["pos"], T, w["budget"])
    qhat = prepped(w)
    mask, st = fused(qhat, i32_dev(w["pos"]), u16_dev(pooled_np), T, w["budget"])
    assert st == 0
    mask = mask.cpu().numpy()
    for r in range(len(w["pos"])):
        p = int(w["pos"][r])
        check_structure(mask[r], dense[r], p, T, w["budget"])
        if np.array_equal(mask[r], want_mask[r]):
            continue
        n = (p + 1) // 4
        keep = min(w["budget"] // 4, n)
        s = want_scores[r]
        cut = np.sort(s)[::-1][keep - 1]
        gb = mask[r][: 4 * n].reshape(n, 4)[:, 0]
        wb = want_mask[r][: 4 * n].reshape(n, 4)[:, 0]
        diff = np.nonzero(gb != wb)[0]
        assert np.all(np.abs(s[diff].astype(np.float64) - cut) <= 5e-3), (r, diff[:8])


def test_fused_sampled_threshold_against_the_oracle():
    """1024 consecutive rows of the prefill chunk over 64k (ternary keys and
    queries: many exact score ties), pooled keys from the oracle.  Every row
    truncates and has over 900 sampled blocks, so its threshold comes from
    the samples and the row is selected from its candidates (its fallback
    flag stays 0).  Masks equal the oracle's, or keep the right number of
    whole blocks plus the tail and differ from it only at blocks within 5e-3
    of the row's cut."""
    from tests import oracle_cache as C
    w = workload(5)
    T = w["tokens"]
    pos, q, want_sc, want_mask, _, _ = C.prefill_slice()
    qhat, st = gpu_prep(w, pos=pos, q=q)
    assert st == 0
    note(f"fused vs oracle: {len(pos)} prefill rows over {T} tokens")
    mask, st, fl = fused(qhat, i32_dev(pos), u16_dev(C.pooled(5)), T, w["budget"], flags=True)
    assert st == 0
    assert np.all(fl == 0), f"{int(fl.sum())} rows fell back"
    mask = mask.cpu().numpy()
    loose = 0
    for r in range(len(pos)):
        p = int(pos[r])
        n = (p + 1) // 4
        if np.array_equal(mask[r], want_mask[r]):
            continue
        s = want_sc[r, :n].astype(np.float64)
        keep = min(w["budget"] // 4, n)
        cut = np.sort(s)[::-1][keep - 1]
        gb = mask[r][: 4 * n].reshape(n, 4)[:, 0]
        wb = want_mask[r][: 4 * n].reshape(n, 4)[:, 0]
        assert gb.sum() == keep and np.all(mask[r][4 * n: p + 1] == 1) and not mask[r][p + 1:].any()
        diff = np.nonzero(gb != wb)[0]
        assert np.all(np.abs(s[diff] - cut) <= 5e-3), (r, diff[:8])
        loose += 1
    note(f"  rows differing only at the cut: {loose} of {len(pos)}")
