"""GPU parity of qsa_gather_kv, the decode K/V gather: bit-exact against the
oracle (a copy has one right answer), through permuted and per-row page
tables, on the vectorised and the element-wise paths, with bad indices and
counts, and downstream of the selector's index lists."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
import sparse_attention_token_qsa_amd as qsa
from tests.gpu_util import DEV, f32_dev, i32_dev, note

pytestmark = pytest.mark.gpu


def run_gpu(kc, vc, table, tstride, tlen, idx, counts, slots, offset=0):
    """qsa_gather_kv on device copies; `offset` > 0 places every bf16 buffer
    `offset` elements into a larger allocation (unaligned path)."""
    n_pages, ps, kv_dim = kc.shape
    rows = idx.shape[0]

    def dev_u16(a):
        flat = torch.from_numpy(np.ascontiguousarray(a).reshape(-1).view(np.int16))
        buf = torch.zeros(flat.numel() + offset, dtype=torch.int16)
        buf[offset:] = flat
        return buf.to(DEV)[offset:].view(a.shape)

    def out_u16(shape):
        n = int(np.prod(shape))
        buf = torch.full((n + offset,), 0x5A5A, dtype=torch.int16, device=DEV)
        return buf[offset:].view(shape)

    ko = out_u16((rows, slots, kv_dim))
    vo = out_u16((rows, slots, kv_dim))
    tab = torch.full((rows, slots // ps), -9, dtype=torch.int32, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    qsa.qsa_gather_kv(dev_u16(kc), dev_u16(vc), i32_dev(table), tstride, tlen, i32_dev(idx),
                      i32_dev(counts), ko, vo, tab, st)
    torch.cuda.synchronize()
    return (ko.cpu().numpy().view(np.uint16), vo.cpu().numpy().view(np.uint16), tab.cpu().numpy(),
            int(st.item()))


def check(kc, vc, table, tstride, tlen, idx, counts, slots, offset=0, label=""):
    note(f"gather {label}: {idx.shape[0]} rows, {slots} slots, kv_dim {kc.shape[2]}, offset {offset}")
    got = run_gpu(kc, vc, table, tstride, tlen, idx, counts, slots, offset)
    want = O.gather_kv(kc, vc, kc.shape[1], table, tstride, tlen, idx, idx.shape[1], counts,
                       idx.shape[0], slots)
    assert got[3] == want[3], (got[3], want[3])
    assert np.array_equal(got[2], want[2])
    assert np.array_equal(got[0], want[0])
    assert np.array_equal(got[1], want[1])
    return want[3]


def random_case(rng, rows, n_log, spare, page_size, kv_dim, idx_stride, per_row=False):
    n_pages = n_log + spare
    kc = rng.integers(0, 1 << 16, size=(n_pages, page_size, kv_dim), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(n_pages, page_size, kv_dim), dtype=np.uint16)
    if per_row:
        table = np.stack([rng.permutation(n_pages)[:n_log] for _ in range(rows)]).astype(np.int32)
        tstride = n_log
    else:
        table = rng.permutation(n_pages)[:n_log].astype(np.int32)
        tstride = 0
    idx = np.full((rows, idx_stride), -1, np.int32)
    counts = rng.integers(0, idx_stride + 1, size=rows).astype(np.int32)
    counts[0] = idx_stride
    for r in range(rows):
        idx[r, : counts[r]] = np.sort(rng.choice(n_log * page_size, counts[r], replace=False))
    return kc, vc, table, tstride, idx, counts


@pytest.mark.parametrize("per_row", [False, True])
def test_gather_bit_exact_budget_lists(per_row):
    rng = np.random.default_rng(31)
    kc, vc, table, ts, idx, counts = random_case(rng, 5, 200, 9, 16, 512, 2051, per_row)
    assert check(kc, vc, table, ts, 200, idx, counts, 2064, label="budget lists") == 0


@pytest.mark.parametrize("kv_dim,offset", [(20, 0), (512, 3), (72, 1)])
def test_gather_elementwise_path(kv_dim, offset):
    rng = np.random.default_rng(32 + kv_dim)
    kc, vc, table, ts, idx, counts = random_case(rng, 3, 40, 3, 8, kv_dim, 100)
    assert check(kc, vc, table, ts, 40, idx, counts, 104, offset=offset, label="element-wise") == 0


@pytest.mark.parametrize("per_row", [False, True])
def test_gather_bit_exact_large_batch(per_row):
    """A batch of 40 rows x 2064 entries (at least 65536 entries: the form
    that moves two entries per wave), random counts up to the whole list,
    against the oracle."""
    rng = np.random.default_rng(35)
    kc, vc, table, ts, idx, counts = random_case(rng, 40, 300, 11, 16, 64, 2051, per_row)
    assert check(kc, vc, table, ts, 300, idx, counts, 2064, label="large batch") == 0


def test_gather_bad_indices_and_counts():
    rng = np.random.default_rng(33)
    kc, vc, table, ts, idx, counts = random_case(rng, 4, 30, 2, 16, 64, 64)
    table = table.copy()
    table[3] = 99                 # a page outside the cache
    idx[0, 5] = -2                # negative
    idx[0, 6] = 30 * 16           # past the table
    idx[0, 7] = 3 * 16 + 1        # lands in the bad page
    counts[1] = 65                # longer than the list row
    counts[2] = -3
    assert check(kc, vc, table, ts, 30, idx, counts, 80, label="bad") == O.STATUS_BAD_INDEX


def test_gather_after_the_selector():
    """Index lists from qsa_select_indices (on seeded scores the oracle also
    selects from) feed the gather; both sides are compared to the oracle."""
    rng = np.random.default_rng(34)
    scores, cols, pos, T = synth.selector_fixture("random", positions=(65535, 60001, 2052, 3000))
    want_idx, want_cnt, st = O.select_indices(scores, cols, pos, T, 2048)
    assert st == 0
    rows = len(pos)
    idx = torch.full((rows, 2051), -77, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(rows, dtype=torch.int32, device=DEV)
    sw = torch.zeros(1, dtype=torch.int32, device=DEV)
    qsa.qsa_select_indices(f32_dev(scores.reshape(-1)), cols, i32_dev(pos), T, 2048, idx, cnt, sw)
    assert int(sw.item()) == 0
    assert np.array_equal(idx.cpu().numpy(), want_idx) and np.array_equal(cnt.cpu().numpy(), want_cnt)
    n_log = T // 16
    kc = rng.integers(0, 1 << 16, size=(n_log + 5, 16, 256), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(n_log + 5, 16, 256), dtype=np.uint16)
    table = rng.permutation(n_log + 5)[:n_log].astype(np.int32)
    n_pages, ps, kv_dim = kc.shape
    ko = torch.empty((rows, 2064, kv_dim), dtype=torch.int16, device=DEV)
    vo = torch.empty_like(ko)
    tab = torch.empty((rows, 2064 // 16), dtype=torch.int32, device=DEV)
    qsa.qsa_gather_kv(torch.from_numpy(kc.view(np.int16)).to(DEV), torch.from_numpy(vc.view(np.int16)).to(DEV),
                      i32_dev(table), 0, n_log, idx, cnt, ko, vo, tab, sw)
    torch.cuda.synchronize()
    want = O.gather_kv(kc, vc, 16, table, 0, n_log, want_idx, 2051, want_cnt, rows, 2064)
    assert int(sw.item()) == want[3] == 0
    assert np.array_equal(ko.cpu().numpy().view(np.uint16), want[0])
    assert np.array_equal(vo.cpu().numpy().view(np.uint16), want[1])
    assert np.array_equal(tab.cpu().numpy(), want[2])
