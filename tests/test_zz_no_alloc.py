"""qsa_select_mask_noalloc (library-owned device scratch, no allocation)
against qsa_select_mask_ws (caller workspace) through the C ABI: two calls
in a row on the split path, the second smaller, then calls that take the
one-workgroup-per-row path and one past the scratch limit.  Mask bytes and
status bits must be identical (integer work: bit-exact), and a few rows are
also checked against the oracle."""

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_token_qsa_amd as qsa
from tests.gpu_util import DEV, f32_dev, i32_dev, note, status_word

pytestmark = pytest.mark.gpu


def _rows(seed, rows, T, nan_row=None):
    rng = np.random.default_rng(seed)
    pos = rng.integers(T // 2, T, size=rows).astype(np.int32)
    pos[0] = T - 1
    cols = T // 4
    sc = rng.standard_normal((rows, cols)).astype(np.float32)
    sc[1, : cols // 3] = 0.5          # a long run of ties
    if nan_row is not None:
        sc[nan_row, 7] = np.nan       # a refused row
    return sc, cols, pos


def _both(sc, cols, pos, T, budget=2048):
    rows = len(pos)
    s = f32_dev(sc.reshape(-1))
    p = i32_dev(pos)
    m_ws = torch.full((rows, T), 0xAB, dtype=torch.uint8, device=DEV)
    st_ws = status_word()
    n = qsa.qsa_select_workspace_bytes(rows, T)
    ws = torch.full((max(n, 16),), 0x5A, dtype=torch.uint8, device=DEV) if n else None
    qsa.qsa_select_mask_ws(s, cols, p, T, budget, m_ws, st_ws, ws)
    m_na = torch.full((rows, T), 0xCD, dtype=torch.uint8, device=DEV)
    st_na = status_word()
    qsa.qsa_select_mask_noalloc(s, cols, p, T, budget, m_na, st_na)
    torch.cuda.synchronize()
    return m_ws.cpu().numpy(), qsa.check_status(st_ws), m_na.cpu().numpy(), qsa.check_status(st_na), n


def test_noalloc_equals_workspace_select_on_two_calls_in_a_row():
    # 1: 16 rows over a 256k-token cache (the split select: 16 chunks per row)
    T = 262144
    sc, cols, pos = _rows(1, 16, T, nan_row=5)
    note(f"noalloc select, call 1: {len(pos)} rows over {T} tokens")
    a, sa, b, sb, n = _both(sc, cols, pos, T)
    assert n > 0, "the split path must run"
    assert sa == sb == O.STATUS_NONFINITE_SCORE
    assert np.array_equal(a, b)
    want, wst = O.select_mask(sc[[0, 1, 5]], cols, pos[[0, 1, 5]], T, 2048)
    assert np.array_equal(b[[0, 1, 5]], want)
    # 2: a smaller call on the same scratch (its contents left by call 1)
    T = 131075
    sc, cols, pos = _rows(2, 5, T)
    note(f"noalloc select, call 2: {len(pos)} rows over {T} tokens")
    a, sa, b, sb, n = _both(sc, cols, pos, T)
    assert n > 0
    assert sa == sb == 0
    assert np.array_equal(a, b)
    want, _ = O.select_mask(sc[:2], cols, pos[:2], T, 2048)
    assert np.array_equal(b[:2], want)


def test_noalloc_one_workgroup_per_row_and_the_scratch_limit():
    T = 4096
    sc, cols, pos = _rows(3, 300, T)
    note("noalloc select: 300 rows over 4096 tokens (no scratch needed)")
    a, sa, b, sb, n = _both(sc, cols, pos, T)
    assert n == 0 and sa == sb == 0 and np.array_equal(a, b)
    # past the scratch: 120 rows fit at 256k tokens, 121 do not
    T = 262144
    assert qsa.qsa_select_workspace_bytes(120, T) <= qsa._lib.NOALLOC_SCRATCH_BYTES
    assert qsa.qsa_select_workspace_bytes(121, T) > qsa._lib.NOALLOC_SCRATCH_BYTES
    rows = 121
    s = torch.zeros(rows * (T // 4), dtype=torch.float32, device=DEV)
    p = torch.full((rows,), T - 1, dtype=torch.int32, device=DEV)
    m = torch.zeros((rows, T), dtype=torch.uint8, device=DEV)
    with pytest.raises(qsa.QsaError) as e:
        qsa.qsa_select_mask_noalloc(s, T // 4, p, T, 2048, m, status_word())
    assert e.value.code == qsa._lib.QSA_ERR_CAPACITY
