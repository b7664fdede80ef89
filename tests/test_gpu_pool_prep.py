"""The combined pool + prep launch (qsa_pool_prep, qsa_pool_prep_dev) against
the oracle, bit for bit: the pooled keys against oracle.pool_keys and the
prepared query heads against oracle.prep_queries, on every workload and on
the edges of the combined call (either stage alone, a block range, refused
positions next to pooled blocks, the unaligned key-stride path, and the
device-count form's window and geometry flag)."""

import functools

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_token_qsa_amd as qsa
from tests.gpu_util import DEV, i32_dev, note, status_word, u16_dev, u16_host, workload

pytestmark = pytest.mark.gpu

FILL = 0x5A5A  # bytes the calls must leave untouched


@functools.lru_cache(maxsize=6)
def oracle_pool(wid):
    w = workload(wid)
    return O.pool_keys(w["raw_keys"], w["k_norm_w"], w["rotary_dim"], w["theta"], w["eps"])


@functools.lru_cache(maxsize=6)
def oracle_prep(wid):
    w = workload(wid)
    return O.prep_queries(w["queries"], w["pos"], w["q_norm_w"], w["rotary_dim"], w["theta"], w["eps"])


def run(w, pos=None, q=None, first_block=0, n_blocks=None, raw=None):
    """qsa_pool_prep on workload w: (pooled [T/4, 128], qhat [rows, 4, 128], status)."""
    T = w["tokens"]
    pos = w["pos"] if pos is None else pos
    q = w["queries"] if q is None else q
    rows = len(pos)
    raw = u16_dev(w["raw_keys"]) if raw is None else raw
    pooled = torch.full((T // 4, 128), FILL, dtype=torch.int16, device=DEV)
    qhat = torch.full((max(rows, 1), 4, 128), FILL, dtype=torch.int16, device=DEV)
    st = status_word()
    qsa.qsa_pool_prep(raw, u16_dev(w["k_norm_w"]), u16_dev(np.asarray(q).reshape(rows, 512)), i32_dev(pos),
                      u16_dev(w["q_norm_w"]), w["rotary_dim"], w["theta"], w["eps"], pooled, qhat, st,
                      first_block=first_block, n_blocks=n_blocks)
    s = qsa.check_status(st)
    return u16_host(pooled), u16_host(qhat)[:rows], s


def assert_equal(got, want, what):
    diff = np.nonzero(got != want)
    assert len(diff[0]) == 0, (what, len(diff[0]), got[diff][:8], want[diff][:8], diff[0][:8])


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_pool_prep_bit_exact(wid):
    w = workload(wid)
    note(f"pool+prep parity: workload {wid} ({w['name']}), tokens {w['tokens']}, rows {len(w['pos'])}")
    pooled, qhat, st = run(w)
    assert st == 0
    assert_equal(pooled, oracle_pool(wid), "pooled")
    assert_equal(qhat, oracle_prep(wid), "qhat")


def test_pool_prep_each_stage_alone():
    w = workload(3)
    note("pool+prep: prep only (n_blocks 0), then pool only (0 rows)")
    pooled, qhat, st = run(w, n_blocks=0)
    assert st == 0
    assert np.all(pooled == FILL)
    assert_equal(qhat, oracle_prep(3), "qhat, prep only")
    pooled, qhat, st = run(w, pos=np.zeros(0, np.int32), q=np.zeros((0, 4, 128), np.uint16))
    assert st == 0
    assert_equal(pooled, oracle_pool(3), "pooled, pool only")


def test_pool_prep_block_range_and_refused_positions():
    """A ragged block range (not a multiple of the 16 blocks a workgroup
    pools) beside query rows with NaN heads and out-of-range positions."""
    w = workload(1)
    T = w["tokens"]
    pos = np.array([0, 5, 511, -1, 512, 77, 2**31 - 1], dtype=np.int32)
    q = w["queries"][: len(pos)].copy()
    q[1, 2, 9] = 0x7FC0
    q[5, 0, 3] = 0xFFC1
    first, n = 7, 53
    note(f"pool+prep: blocks [{first}, {first + n}) of {T // 4}, refused positions")
    pooled, qhat, st = run(w, pos=pos, q=q, first_block=first, n_blocks=n)
    assert st == O.STATUS_BAD_POSITION
    want = oracle_pool(1)
    assert_equal(pooled[first:first + n], want[first:first + n], "pooled range")
    assert np.all(pooled[:first] == FILL) and np.all(pooled[first + n:] == FILL)
    valid = [0, 1, 2, 5]
    wq = O.prep_queries(q[valid], pos[valid], w["q_norm_w"], w["rotary_dim"], w["theta"], w["eps"])
    assert_equal(qhat[valid], wq, "qhat valid rows")
    assert np.all(qhat[[3, 4, 6]] == 0)


def test_pool_prep_unaligned_key_stride():
    """Keys in the first 128 columns of 129-wide rows: the element-wise path."""
    w = workload(1)
    T = w["tokens"]
    wide = np.zeros((T, 129), dtype=np.uint16)
    wide[:, :128] = w["raw_keys"]
    wide[:, 128] = 0xFFFF
    note("pool+prep: key stride 129")
    pooled, qhat, st = run(w, raw=u16_dev(wide))
    assert st == 0
    assert_equal(pooled, oracle_pool(1), "pooled, stride 129")
    assert_equal(qhat, oracle_prep(1), "qhat")


def test_pool_prep_dev_window_and_geometry():
    """Device cache length T_live below the ceiling: the window of the last n
    complete blocks of raw[:T_live] is pooled, rows at or past T_live are
    refused; a length above the ceiling sets the geometry flag."""
    w = workload(3)
    T = w["tokens"]
    t_live = T - 4 * 37 - 2  # 2 tokens into an incomplete block
    n = 21
    rows = np.arange(0, 64, 3)
    pos = w["pos"][rows].copy()
    pos[[0, 5]] = [t_live - 1, t_live]  # one last visible position, one past the cache
    q = w["queries"][rows]
    note(f"pool+prep dev: T_live {t_live} of {T}, window {n} blocks, {len(rows)} rows")
    raw = u16_dev(w["raw_keys"])
    pooled = torch.full((T // 4, 128), FILL, dtype=torch.int16, device=DEV)
    qhat = torch.full((len(rows), 4, 128), FILL, dtype=torch.int16, device=DEV)
    st = status_word()
    dev_t = i32_dev([t_live])
    qsa.qsa_pool_prep_dev(raw, u16_dev(w["k_norm_w"]), u16_dev(q.reshape(len(rows), 512)), i32_dev(pos),
                          u16_dev(w["q_norm_w"]), w["rotary_dim"], w["theta"], w["eps"], dev_t, n, pooled,
                          qhat, st)
    assert qsa.check_status(st) == O.STATUS_BAD_POSITION
    got_p, got_q = u16_host(pooled), u16_host(qhat)
    nb = t_live // 4
    # complete blocks below T_live pool the same under any cache length
    assert_equal(got_p[nb - n:nb], oracle_pool(3)[nb - n:nb], "pooled window")
    assert np.all(got_p[:nb - n] == FILL) and np.all(got_p[nb:] == FILL)
    ok = pos < t_live
    wq = O.prep_queries(q[ok], pos[ok], w["q_norm_w"], w["rotary_dim"], w["theta"], w["eps"])
    assert_equal(got_q[ok], wq, "qhat valid rows")
    assert np.all(got_q[~ok] == 0)
    # a device length above the ceiling: clamped to it, geometry flag set
    st2 = status_word()
    qsa.qsa_pool_prep_dev(raw, u16_dev(w["k_norm_w"]), u16_dev(q.reshape(len(rows), 512)), i32_dev(pos),
                          u16_dev(w["q_norm_w"]), w["rotary_dim"], w["theta"], w["eps"], i32_dev([T + 8]), 4,
                          pooled, qhat, st2)
    assert qsa.check_status(st2) & qsa.STATUS_BAD_GEOMETRY
    torch.cuda.synchronize()
