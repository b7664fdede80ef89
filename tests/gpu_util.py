"""Helpers for the GPU tests: move seeded inputs to the device, run the three
C-ABI calls through the binding, read results back.  No method arithmetic."""

from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import sparse_attention_token_qsa_amd as qsa
import synth

DEV = "cuda:0"


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def u16_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def u16_host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def i32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def f32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


@functools.lru_cache(maxsize=8)
def workload(wid: int):
    return synth.make_workload(wid)


def status_word() -> torch.Tensor:
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def gpu_pool(w, first_block=0, n_blocks=None, raw_dev=None, key_stride_view=None):
    T = w["tokens"]
    raw = u16_dev(w["raw_keys"]) if raw_dev is None else raw_dev
    if key_stride_view is not None:
        raw = key_stride_view
    pooled = torch.full((T // 4, 128), 0x5A5A, dtype=torch.int16, device=DEV)
    qsa.qsa_pool_keys(raw, u16_dev(w["k_norm_w"]), w["rotary_dim"], w["theta"], w["eps"], pooled,
                      first_block=first_block, n_blocks=n_blocks)
    torch.cuda.synchronize()
    return pooled


def gpu_scores(w, pooled_dev, pos=None, q=None, score_cols=None, sentinel=np.float32(-7.25)):
    """Scores [rows, score_cols] (read back), prefilled with `sentinel`, and status."""
    T = w["tokens"]
    pos = w["pos"] if pos is None else pos
    q = w["queries"] if q is None else q
    rows = len(pos)
    cols = T // 4 if score_cols is None else score_cols
    scores = torch.full((rows * max(cols, 1),), float(sentinel), dtype=torch.float32, device=DEV)
    st = status_word()
    qsa.qsa_score_rows(u16_dev(q.reshape(rows, 512)), i32_dev(pos), u16_dev(w["q_norm_w"]),
                       w["rotary_dim"], w["theta"], w["eps"], pooled_dev, T, scores, cols, st)
    s = qsa.check_status(st)
    return scores.cpu().numpy().reshape(rows, max(cols, 1)), s


def gpu_prep(w, pos=None, q=None):
    """Prepared queries [rows, 4, 128] (bf16 bits, read back) and status."""
    T = w["tokens"]
    pos = w["pos"] if pos is None else pos
    q = w["queries"] if q is None else q
    rows = len(pos)
    qhat = torch.full((rows, 4, 128), 0x5A5A, dtype=torch.int16, device=DEV)
    st = status_word()
    qsa.qsa_prep_queries(u16_dev(q.reshape(rows, 512)), i32_dev(pos), u16_dev(w["q_norm_w"]),
                         w["rotary_dim"], w["theta"], w["eps"], T, qhat, st)
    s = qsa.check_status(st)
    return qhat, s


def gpu_scores_prepped(w, pooled_dev, pos=None, q=None, score_cols=None,
                       sentinel=np.float32(-7.25)):
    """gpu_scores through qsa_prep_queries + qsa_score_prepped."""
    T = w["tokens"]
    pos = w["pos"] if pos is None else pos
    rows = len(pos)
    cols = T // 4 if score_cols is None else score_cols
    qhat, s1 = gpu_prep(w, pos=pos, q=q)
    scores = torch.full((rows * max(cols, 1),), float(sentinel), dtype=torch.float32, device=DEV)
    st = status_word()
    qsa.qsa_score_prepped(qhat, i32_dev(pos), pooled_dev, T, scores, cols, st)
    s2 = qsa.check_status(st)
    return scores.cpu().numpy().reshape(rows, max(cols, 1)), s1 | s2


def gpu_select(scores: np.ndarray, cols: int, pos, tokens: int, budget: int):
    rows = len(pos)
    mask = torch.full((rows, tokens), 0xAB, dtype=torch.uint8, device=DEV)
    st = status_word()
    qsa.qsa_select_mask(f32_dev(scores.reshape(-1)), cols, i32_dev(pos), tokens, budget, mask, st)
    s = qsa.check_status(st)
    return mask.cpu().numpy(), s


def gpu_select_ws(scores: np.ndarray, cols: int, pos, tokens: int, budget: int, fill: int = 0x5A):
    """qsa_select_mask_ws with a workspace of exactly the reported size,
    prefilled with junk (its contents on entry must not matter)."""
    rows = len(pos)
    mask = torch.full((rows, tokens), 0xAB, dtype=torch.uint8, device=DEV)
    st = status_word()
    nbytes = qsa.qsa_select_workspace_bytes(rows, tokens)
    ws = torch.full((max(nbytes, 16),), fill, dtype=torch.uint8, device=DEV) if nbytes else None
    qsa.qsa_select_mask_ws(f32_dev(scores.reshape(-1)), cols, i32_dev(pos), tokens, budget, mask, st, ws)
    s = qsa.check_status(st)
    return mask.cpu().numpy(), s, nbytes


def gpu_select_indices(scores: np.ndarray, cols: int, pos, tokens: int, budget: int, stride=None):
    """qsa_select_indices: (idx [rows, stride] read back, counts, status);
    idx is prefilled with a sentinel so untouched columns show."""
    rows = len(pos)
    stride = budget + 3 if stride is None else stride
    idx = torch.full((rows, stride), -77, dtype=torch.int32, device=DEV)
    counts = torch.full((rows,), -77, dtype=torch.int32, device=DEV)
    st = status_word()
    qsa.qsa_select_indices(f32_dev(scores.reshape(-1)), cols, i32_dev(pos), tokens, budget, idx, counts, st)
    s = qsa.check_status(st)
    return idx.cpu().numpy(), counts.cpu().numpy(), s


def gpu_select_indices_ws(scores: np.ndarray, cols: int, pos, tokens: int, budget: int, stride=None,
                          fill: int = 0x5A):
    """qsa_select_indices_ws with a junk-filled workspace of exactly the
    reported size: (idx read back, counts, status, workspace bytes)."""
    rows = len(pos)
    stride = budget + 3 if stride is None else stride
    idx = torch.full((rows, stride), -77, dtype=torch.int32, device=DEV)
    counts = torch.full((rows,), -77, dtype=torch.int32, device=DEV)
    st = status_word()
    nbytes = qsa.qsa_select_workspace_bytes(rows, tokens)
    ws = torch.full((max(nbytes, 16),), fill, dtype=torch.uint8, device=DEV) if nbytes else None
    qsa.qsa_select_indices_ws(f32_dev(scores.reshape(-1)), cols, i32_dev(pos), tokens, budget, idx, counts, st, ws)
    s = qsa.check_status(st)
    return idx.cpu().numpy(), counts.cpu().numpy(), s, nbytes
