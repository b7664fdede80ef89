"""QSA token indexer hot path on AMD Instinct MI355X (gfx950).

Thin torch-facing binding of libqsa.so (C ABI: include/qsa.h).  Each function
has the name of the C entry point it marshals to; torch tensors supply device
memory, torch's current HIP stream is used unless one is given.  All
computation runs in the library's HIP kernels; there is no CPU path.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (EXPORTS, HEAD_DIM, HEADS, MAX_KEEP_BLOCKS, MAX_TOKENS, RATIO,  # noqa: F401
                   STATUS_BAD_GEOMETRY, STATUS_BAD_INDEX, STATUS_BAD_POSITION,
                   STATUS_NONFINITE_SCORE, QsaError,
                   abi_version, load,
                   strerror)

__all__ = ["qsa_pool_keys", "qsa_score_rows", "qsa_prep_queries", "qsa_pool_prep", "qsa_score_prepped",
           "qsa_select_mask", "qsa_select_indices", "qsa_select_workspace_bytes",
           "qsa_select_mask_ws", "qsa_select_mask_noalloc", "qsa_score_select_workspace_bytes",
           "qsa_score_select_flags_offset",
           "qsa_score_select_mask",
           "qsa_gather_kv", "qsa_pool_window", "qsa_prep_queries_dev", "qsa_pool_prep_dev",
           "qsa_score_prepped_dev", "qsa_select_indices_dev", "qsa_select_indices_ws",
           "qsa_rope_inv_freq",
           "check_status", "load", "abi_version", "strerror", "QsaError"]

_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _dev(t: torch.Tensor, name: str, dtypes) -> None:
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.is_cuda, f"{name} must be on the GPU")
    _need(t.dtype in dtypes, f"{name} has dtype {t.dtype}, expected one of {dtypes}")


def _rows_2d(t: torch.Tensor, name: str, min_cols: int) -> int:
    """Row stride (elements) of a 2-D tensor with unit column stride."""
    _need(t.dim() == 2, f"{name} must be 2-D")
    _need(t.stride(1) == 1 or t.shape[1] == 1, f"{name} must have unit column stride")
    _need(t.shape[1] >= min_cols, f"{name} needs at least {min_cols} columns")
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def _check(code: int, what: str) -> None:
    if code != 0:
        raise QsaError(code, what)


def qsa_pool_keys(raw_keys: torch.Tensor, k_norm_w: torch.Tensor, rotary_dim: int,
                  rope_theta: float, rms_eps: float, pooled: torch.Tensor,
                  first_block: int = 0, n_blocks: int | None = None, stream=None) -> None:
    """Pool blocks [first_block, first_block + n_blocks) of raw_keys
    [tokens, >=128] (bf16, unit column stride) into pooled [tokens/4, 128]."""
    _dev(raw_keys, "raw_keys", _BF16_LIKE)
    _dev(k_norm_w, "k_norm_w", _BF16_LIKE)
    _dev(pooled, "pooled", _BF16_LIKE)
    key_stride = _rows_2d(raw_keys, "raw_keys", HEAD_DIM)
    tokens = raw_keys.shape[0]
    _need(k_norm_w.numel() == HEAD_DIM and k_norm_w.is_contiguous(), "k_norm_w must hold 128 values")
    _need(pooled.is_contiguous() and pooled.dim() == 2 and pooled.shape[1] == HEAD_DIM
          and pooled.shape[0] >= tokens // RATIO, "pooled must be contiguous [tokens/4, 128]")
    if n_blocks is None:
        n_blocks = tokens // RATIO - first_block
    lib = load()
    _check(lib.qsa_pool_keys(_ptr(raw_keys), key_stride, tokens, _ptr(k_norm_w), rotary_dim,
                             rope_theta, rms_eps, first_block, n_blocks, _ptr(pooled),
                             _stream_ptr(stream)), "qsa_pool_keys")


def _pool_prep_args(raw_keys, k_norm_w, q, pos, q_norm_w, pooled, qhat, dev_status):
    """Shared checks of the combined pool + prep calls; returns (key_stride,
    q_stride, tokens, rows)."""
    for t, name in ((raw_keys, "raw_keys"), (k_norm_w, "k_norm_w"), (pooled, "pooled"), (q, "q"),
                    (q_norm_w, "q_norm_w"), (qhat, "qhat")):
        _dev(t, name, _BF16_LIKE)
    _dev(pos, "pos", (torch.int32,))
    _dev(dev_status, "dev_status", (torch.int32,))
    key_stride = _rows_2d(raw_keys, "raw_keys", HEAD_DIM)
    q_stride = _rows_2d(q, "q", HEADS * HEAD_DIM)
    tokens, rows = raw_keys.shape[0], q.shape[0]
    _need(k_norm_w.numel() == HEAD_DIM and k_norm_w.is_contiguous(), "k_norm_w must hold 128 values")
    _need(q_norm_w.numel() == HEAD_DIM and q_norm_w.is_contiguous(), "q_norm_w must hold 128 values")
    _need(pooled.is_contiguous() and pooled.dim() == 2 and pooled.shape[1] == HEAD_DIM
          and pooled.shape[0] >= tokens // RATIO, "pooled must be contiguous [tokens/4, 128]")
    _need(pos.is_contiguous() and pos.numel() == rows, "pos must be contiguous [rows]")
    _need(qhat.is_contiguous() and qhat.numel() >= rows * HEADS * HEAD_DIM,
          "qhat must be contiguous [rows, 4, 128]")
    _need(dev_status.numel() >= 1, "dev_status needs one int32")
    return key_stride, q_stride, tokens, rows


def qsa_pool_prep(raw_keys: torch.Tensor, k_norm_w: torch.Tensor, q: torch.Tensor, pos: torch.Tensor,
                  q_norm_w: torch.Tensor, rotary_dim: int, rope_theta: float, rms_eps: float,
                  pooled: torch.Tensor, qhat: torch.Tensor, dev_status: torch.Tensor,
                  first_block: int = 0, n_blocks: int | None = None, stream=None) -> None:
    """qsa_pool_keys (blocks [first_block, first_block + n_blocks) of raw_keys)
    and qsa_prep_queries (q at pos, valid below raw_keys' row count) in one launch."""
    key_stride, q_stride, tokens, rows = _pool_prep_args(raw_keys, k_norm_w, q, pos, q_norm_w, pooled,
                                                         qhat, dev_status)
    if n_blocks is None:
        n_blocks = tokens // RATIO - first_block
    lib = load()
    _check(lib.qsa_pool_prep(_ptr(raw_keys), key_stride, tokens, _ptr(k_norm_w), first_block, n_blocks,
                             _ptr(pooled), _ptr(q), q_stride, _ptr(pos), rows, _ptr(q_norm_w), _ptr(qhat),
                             rotary_dim, rope_theta, rms_eps, _ptr(dev_status), _stream_ptr(stream)),
           "qsa_pool_prep")


def qsa_score_rows(q: torch.Tensor, pos: torch.Tensor, q_norm_w: torch.Tensor, rotary_dim: int,
                   rope_theta: float, rms_eps: float, pooled: torch.Tensor, tokens: int,
                   scores: torch.Tensor, score_cols: int, dev_status: torch.Tensor,
                   stream=None) -> None:
    """Scores of query rows q [rows, >=512] (4 heads x 128, bf16) at positions
    pos (int32 [rows]) against pooled keys; writes scores[r*score_cols + b]
    for b < (pos[r]+1)/4 into the flat f32 buffer `scores`."""
    _dev(q, "q", _BF16_LIKE)
    _dev(pos, "pos", (torch.int32,))
    _dev(q_norm_w, "q_norm_w", _BF16_LIKE)
    _dev(pooled, "pooled", _BF16_LIKE)
    _dev(scores, "scores", (torch.float32,))
    _dev(dev_status, "dev_status", (torch.int32,))
    q_stride = _rows_2d(q, "q", HEADS * HEAD_DIM)
    rows = q.shape[0]
    _need(pos.is_contiguous() and pos.numel() == rows, "pos must be contiguous [rows]")
    _need(q_norm_w.numel() == HEAD_DIM and q_norm_w.is_contiguous(), "q_norm_w must hold 128 values")
    _need(pooled.is_contiguous() and pooled.numel() >= (tokens // RATIO) * HEAD_DIM,
          "pooled must be contiguous and cover tokens/4 blocks")
    _need(scores.is_contiguous(), "scores must be contiguous")
    _need(dev_status.numel() >= 1, "dev_status needs one int32")
    lib = load()
    _check(lib.qsa_score_rows(_ptr(q), q_stride, _ptr(pos), rows, _ptr(q_norm_w), rotary_dim,
                              rope_theta, rms_eps, _ptr(pooled), tokens, _ptr(scores),
                              score_cols, scores.numel(), _ptr(dev_status), _stream_ptr(stream)),
           "qsa_score_rows")


def qsa_prep_queries(q: torch.Tensor, pos: torch.Tensor, q_norm_w: torch.Tensor,
                     rotary_dim: int, rope_theta: float, rms_eps: float, tokens: int,
                     qhat: torch.Tensor, dev_status: torch.Tensor, stream=None) -> None:
    """Normed, roped query heads of q [rows, >=512] at positions pos into
    qhat [rows, 4, 128] (bf16 bits, contiguous)."""
    _dev(q, "q", _BF16_LIKE)
    _dev(pos, "pos", (torch.int32,))
    _dev(q_norm_w, "q_norm_w", _BF16_LIKE)
    _dev(qhat, "qhat", _BF16_LIKE)
    _dev(dev_status, "dev_status", (torch.int32,))
    q_stride = _rows_2d(q, "q", HEADS * HEAD_DIM)
    rows = q.shape[0]
    _need(pos.is_contiguous() and pos.numel() == rows, "pos must be contiguous [rows]")
    _need(q_norm_w.numel() == HEAD_DIM and q_norm_w.is_contiguous(), "q_norm_w must hold 128 values")
    _need(qhat.is_contiguous() and qhat.numel() >= rows * HEADS * HEAD_DIM,
          "qhat must be contiguous [rows, 4, 128]")
    _need(dev_status.numel() >= 1, "dev_status needs one int32")
    lib = load()
    _check(lib.qsa_prep_queries(_ptr(q), q_stride, _ptr(pos), rows, _ptr(q_norm_w), rotary_dim,
                                rope_theta, rms_eps, tokens, _ptr(qhat), _ptr(dev_status),
                                _stream_ptr(stream)), "qsa_prep_queries")


def qsa_score_prepped(qhat: torch.Tensor, pos: torch.Tensor, pooled: torch.Tensor, tokens: int,
                      scores: torch.Tensor, score_cols: int, dev_status: torch.Tensor,
                      stream=None) -> None:
    """qsa_score_rows on queries prepared by qsa_prep_queries."""
    _dev(qhat, "qhat", _BF16_LIKE)
    _dev(pos, "pos", (torch.int32,))
    _dev(pooled, "pooled", _BF16_LIKE)
    _dev(scores, "scores", (torch.float32,))
    _dev(dev_status, "dev_status", (torch.int32,))
    rows = pos.numel()
    _need(pos.is_contiguous(), "pos must be contiguous")
    _need(qhat.is_contiguous() and qhat.numel() >= rows * HEADS * HEAD_DIM,
          "qhat must be contiguous [rows, 4, 128]")
    _need(pooled.is_contiguous() and pooled.numel() >= (tokens // RATIO) * HEAD_DIM,
          "pooled must be contiguous and cover tokens/4 blocks")
    _need(scores.is_contiguous(), "scores must be contiguous")
    _need(dev_status.numel() >= 1, "dev_status needs one int32")
    lib = load()
    _check(lib.qsa_score_prepped(_ptr(qhat), _ptr(pos), rows, _ptr(pooled), tokens, _ptr(scores),
                                 score_cols, scores.numel(), _ptr(dev_status), _stream_ptr(stream)),
           "qsa_score_prepped")


def qsa_select_mask(scores: torch.Tensor, score_cols: int, pos: torch.Tensor, tokens: int,
                    budget: int, mask: torch.Tensor, dev_status: torch.Tensor,
                    stream=None) -> None:
    """Top-(budget/4) block select of each row and its u8 mask [rows, tokens]."""
    _dev(scores, "scores", (torch.float32,))
    _dev(pos, "pos", (torch.int32,))
    _dev(mask, "mask", (torch.uint8,))
    _dev(dev_status, "dev_status", (torch.int32,))
    rows = pos.numel()
    _need(pos.is_contiguous(), "pos must be contiguous")
    _need(scores.is_contiguous(), "scores must be contiguous")
    _need(mask.is_contiguous() and mask.numel() >= rows * tokens, "mask must be contiguous [rows, tokens]")
    _need(dev_status.numel() >= 1, "dev_status needs one int32")
    lib = load()
    _check(lib.qsa_select_mask(_ptr(scores), score_cols, scores.numel(), _ptr(pos), rows, tokens,
                               budget, _ptr(mask), _ptr(dev_status), _stream_ptr(stream)),
           "qsa_select_mask")


def qsa_select_indices(scores: torch.Tensor, score_cols: int, pos: torch.Tensor, tokens: int,
                       budget: int, idx: torch.Tensor, counts: torch.Tensor,
                       dev_status: torch.Tensor, stream=None) -> None:
    """Kept token indices of each row: idx [rows, >= budget + 3] int32
    (ascending, -1 after counts[r]) and counts [rows] int32."""
    _dev(scores, "scores", (torch.float32,))
    _dev(pos, "pos", (torch.int32,))
    _dev(idx, "idx", (torch.int32,))
    _dev(counts, "counts", (torch.int32,))
    _dev(dev_status, "dev_status", (torch.int32,))
    rows = pos.numel()
    _need(pos.is_contiguous(), "pos must be contiguous")
    _need(scores.is_contiguous(), "scores must be contiguous")
    idx_stride = _rows_2d(idx, "idx", budget + RATIO - 1)
    _need(idx.shape[0] >= rows, "idx needs a row per position")
    _need(counts.is_contiguous() and counts.numel() >= rows, "counts must be contiguous [rows]")
    _need(dev_status.numel() >= 1, "dev_status needs one int32")
    lib = load()
    _check(lib.qsa_select_indices(_ptr(scores), score_cols, scores.numel(), _ptr(pos), rows, tokens,
                                  budget, _ptr(idx), idx_stride, _ptr(counts), _ptr(dev_status),
                                  _stream_ptr(stream)), "qsa_select_indices")


def qsa_select_workspace_bytes(rows: int, tokens: int) -> int:
    """Device workspace bytes qsa_select_mask_ws needs (0: none)."""
    n = load().qsa_select_workspace_bytes(rows, tokens)
    if n < 0:
        raise QsaError(int(n), "qsa_select_workspace_bytes")
    return int(n)


def qsa_select_mask_ws(scores: torch.Tensor, score_cols: int, pos: torch.Tensor, tokens: int,
                       budget: int, mask: torch.Tensor, dev_status: torch.Tensor,
                       workspace: torch.Tensor | None, stream=None) -> None:
    """qsa_select_mask for few long rows, split over workgroups; `workspace`
    is a device tensor of at least qsa_select_workspace_bytes(rows, tokens)
    bytes (may be None when that is 0)."""
    _dev(scores, "scores", (torch.float32,))
    _dev(pos, "pos", (torch.int32,))
    _dev(mask, "mask", (torch.uint8,))
    _dev(dev_status, "dev_status", (torch.int32,))
    rows = pos.numel()
    _need(pos.is_contiguous(), "pos must be contiguous")
    _need(scores.is_contiguous(), "scores must be contiguous")
    _need(mask.is_contiguous() and mask.numel() >= rows * tokens, "mask must be contiguous [rows, tokens]")
    _need(dev_status.numel() >= 1, "dev_status needs one int32")
    ws_bytes = 0
    if workspace is not None:
        _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous GPU tensor")
        ws_bytes = workspace.numel() * workspace.element_size()
    lib = load()
    _check(lib.qsa_select_mask_ws(_ptr(scores), score_cols, scores.numel(), _ptr(pos), rows, tokens,
                                  budget, _ptr(mask), _ptr(dev_status), _ptr(workspace), ws_bytes,
                                  _stream_ptr(stream)), "qsa_select_mask_ws")


def qsa_select_mask_noalloc(scores: torch.Tensor, score_cols: int, pos: torch.Tensor, tokens: int,
                            budget: int, mask: torch.Tensor, dev_status: torch.Tensor, stream=None) -> None:
    """qsa_select_mask_ws with the library's own device scratch in place of a
    workspace: allocates nothing (for graph capture and allocation-free
    loops).  Calls overlapping on one GPU share the scratch and race."""
    _dev(scores, "scores", (torch.float32,))
    _dev(pos, "pos", (torch.int32,))
    _dev(mask, "mask", (torch.uint8,))
    _dev(dev_status, "dev_status", (torch.int32,))
    rows = pos.numel()
    _need(pos.is_contiguous(), "pos must be contiguous")
    _need(scores.is_contiguous(), "scores must be contiguous")
    _need(mask.is_contiguous() and mask.numel() >= rows * tokens, "mask must be contiguous [rows, tokens]")
    _need(dev_status.numel() >= 1, "dev_status needs one int32")
    _check(load().qsa_select_mask_noalloc(_ptr(scores), score_cols, scores.numel(), _ptr(pos), rows, tokens,
                                          budget, _ptr(mask), _ptr(dev_status), _stream_ptr(stream)),
           "qsa_select_mask_noalloc")


def qsa_score_select_workspace_bytes(rows: int, tokens: int, budget: int) -> int:
    """Device workspace bytes qsa_score_select_mask needs."""
    n = load().qsa_score_select_workspace_bytes(rows, tokens, budget)
    if n < 0:
        raise QsaError(int(n), "qsa_score_select_workspace_bytes")
    return int(n)


def qsa_score_select_flags_offset(rows: int, tokens: int, budget: int) -> int:
    """Byte offset, in qsa_score_select_mask's workspace, of the int32 [rows]
    flags that mark the rows the call selected in full."""
    n = load().qsa_score_select_flags_offset(rows, tokens, budget)
    if n < 0:
        raise QsaError(int(n), "qsa_score_select_flags_offset")
    return int(n)


def qsa_score_select_mask(qhat: torch.Tensor, pos: torch.Tensor, pooled: torch.Tensor, tokens: int,
                          budget: int, mask: torch.Tensor, dev_status: torch.Tensor,
                          workspace: torch.Tensor, stream=None) -> None:
    """qsa_score_prepped followed by qsa_select_mask in one call, without the
    score matrix: `workspace` is a device tensor of at least
    qsa_score_select_workspace_bytes(rows, tokens, budget) bytes, 256-byte
    aligned (torch's allocations are)."""
    _dev(qhat, "qhat", _BF16_LIKE)
    _dev(pos, "pos", (torch.int32,))
    _dev(pooled, "pooled", _BF16_LIKE)
    _dev(mask, "mask", (torch.uint8,))
    _dev(dev_status, "dev_status", (torch.int32,))
    rows = pos.numel()
    _need(pos.is_contiguous() and qhat.is_contiguous() and pooled.is_contiguous(),
          "qhat, pos and pooled must be contiguous")
    _need(qhat.numel() >= rows * HEADS * HEAD_DIM, "qhat must hold [rows, 4, 128]")
    _need(pooled.numel() >= (tokens // RATIO) * HEAD_DIM, "pooled must hold [tokens/4, 128]")
    _need(mask.is_contiguous() and mask.numel() >= rows * tokens, "mask must be contiguous [rows, tokens]")
    _need(dev_status.numel() >= 1, "dev_status needs one int32")
    _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    lib = load()
    _check(lib.qsa_score_select_mask(_ptr(qhat), _ptr(pos), rows, _ptr(pooled), tokens, budget, _ptr(mask),
                                     _ptr(dev_status), _ptr(workspace), ws_bytes, _stream_ptr(stream)),
           "qsa_score_select_mask")


def qsa_gather_kv(k_cache: torch.Tensor, v_cache: torch.Tensor, page_table: torch.Tensor,
                  table_stride: int, table_len: int, idx: torch.Tensor, counts: torch.Tensor,
                  k_out: torch.Tensor, v_out: torch.Tensor, out_table: torch.Tensor,
                  dev_status: torch.Tensor, stream=None) -> None:
    """Selected tokens' K/V from a paged cache into contiguous scratch plus the
    identity page table.  k_cache, v_cache: [n_pages, page_size, kv_dim] bf16;
    idx: [rows, idx_stride] int32 lists with counts [rows]; k_out, v_out:
    [rows, slots, kv_dim] bf16; out_table: [rows, slots / page_size] int32."""
    for t, name in ((k_cache, "k_cache"), (v_cache, "v_cache"), (k_out, "k_out"), (v_out, "v_out")):
        _dev(t, name, _BF16_LIKE)
        _need(t.dim() == 3 and t.is_contiguous(), f"{name} must be a contiguous 3-D tensor")
    for t, name in ((page_table, "page_table"), (idx, "idx"), (counts, "counts"), (out_table, "out_table"),
                    (dev_status, "dev_status")):
        _dev(t, name, (torch.int32,))
        _need(t.is_contiguous(), f"{name} must be contiguous")
    n_pages, page_size, kv_dim = k_cache.shape
    _need(tuple(v_cache.shape) == tuple(k_cache.shape), "v_cache must match k_cache")
    rows, slots, kd = k_out.shape
    _need(kd == kv_dim and tuple(v_out.shape) == tuple(k_out.shape), "k_out/v_out must be [rows, slots, kv_dim]")
    _need(idx.dim() == 2 and idx.shape[0] == rows, "idx must be [rows, idx_stride]")
    _need(counts.numel() >= rows, "counts needs one entry per row")
    _need(out_table.numel() >= rows * (slots // max(page_size, 1)), "out_table too small")
    need = table_len if table_stride == 0 else rows * table_stride
    _need(page_table.numel() >= need, "page_table too small")
    lib = load()
    _check(lib.qsa_gather_kv(_ptr(k_cache), _ptr(v_cache), n_pages, page_size, kv_dim, _ptr(page_table),
                             table_stride, table_len, _ptr(idx), idx.shape[1], _ptr(counts), rows, slots,
                             _ptr(k_out), _ptr(v_out), _ptr(out_table), _ptr(dev_status), _stream_ptr(stream)),
           "qsa_gather_kv")


def _dev_tokens(dev_tokens: torch.Tensor) -> None:
    _dev(dev_tokens, "dev_tokens", (torch.int32,))
    _need(dev_tokens.numel() >= 1, "dev_tokens needs one int32")


def qsa_pool_window(raw_keys: torch.Tensor, k_norm_w: torch.Tensor, rotary_dim: int,
                    rope_theta: float, rms_eps: float, dev_tokens: torch.Tensor, n_blocks: int,
                    pooled: torch.Tensor, dev_status: torch.Tensor, stream=None) -> None:
    """Pool the last n_blocks complete blocks of a cache of dev_tokens[0] tokens;
    raw_keys [max_tokens, >=128] bf16 (its rows are the ceiling)."""
    _dev(raw_keys, "raw_keys", _BF16_LIKE)
    _dev(k_norm_w, "k_norm_w", _BF16_LIKE)
    _dev(pooled, "pooled", _BF16_LIKE)
    _dev(dev_status, "dev_status", (torch.int32,))
    _dev_tokens(dev_tokens)
    key_stride = _rows_2d(raw_keys, "raw_keys", HEAD_DIM)
    max_tokens = raw_keys.shape[0]
    _need(k_norm_w.numel() == HEAD_DIM and k_norm_w.is_contiguous(), "k_norm_w must hold 128 values")
    _need(pooled.is_contiguous() and pooled.dim() == 2 and pooled.shape[1] == HEAD_DIM
          and pooled.shape[0] >= max_tokens // RATIO, "pooled must be contiguous [max_tokens/4, 128]")
    lib = load()
    _check(lib.qsa_pool_window(_ptr(raw_keys), key_stride, max_tokens, _ptr(k_norm_w), rotary_dim, rope_theta,
                               rms_eps, _ptr(dev_tokens), n_blocks, _ptr(pooled), _ptr(dev_status),
                               _stream_ptr(stream)), "qsa_pool_window")


def qsa_pool_prep_dev(raw_keys: torch.Tensor, k_norm_w: torch.Tensor, q: torch.Tensor, pos: torch.Tensor,
                      q_norm_w: torch.Tensor, rotary_dim: int, rope_theta: float, rms_eps: float,
                      dev_tokens: torch.Tensor, n_blocks: int, pooled: torch.Tensor, qhat: torch.Tensor,
                      dev_status: torch.Tensor, stream=None) -> None:
    """qsa_pool_window and qsa_prep_queries_dev in one launch; raw_keys' row
    count is the ceiling max_tokens."""
    key_stride, q_stride, max_tokens, rows = _pool_prep_args(raw_keys, k_norm_w, q, pos, q_norm_w, pooled,
                                                             qhat, dev_status)
    _dev_tokens(dev_tokens)
    lib = load()
    _check(lib.qsa_pool_prep_dev(_ptr(raw_keys), key_stride, max_tokens, _ptr(k_norm_w), n_blocks, _ptr(pooled),
                                 _ptr(q), q_stride, _ptr(pos), rows, _ptr(q_norm_w), _ptr(qhat), rotary_dim,
                                 rope_theta, rms_eps, _ptr(dev_tokens), _ptr(dev_status), _stream_ptr(stream)),
           "qsa_pool_prep_dev")


def qsa_prep_queries_dev(q: torch.Tensor, pos: torch.Tensor, q_norm_w: torch.Tensor, rotary_dim: int,
                         rope_theta: float, rms_eps: float, dev_tokens: torch.Tensor, max_tokens: int,
                         qhat: torch.Tensor, dev_status: torch.Tensor, stream=None) -> None:
    """qsa_prep_queries with the live cache length in dev_tokens[0]."""
    _dev(q, "q", _BF16_LIKE)
    _dev(pos, "pos", (torch.int32,))
    _dev(q_norm_w, "q_norm_w", _BF16_LIKE)
    _dev(qhat, "qhat", _BF16_LIKE)
    _dev(dev_status, "dev_status", (torch.int32,))
    _dev_tokens(dev_tokens)
    q_stride = _rows_2d(q, "q", HEADS * HEAD_DIM)
    rows = q.shape[0]
    _need(pos.is_contiguous() and pos.numel() == rows, "pos must be contiguous [rows]")
    _need(q_norm_w.numel() == HEAD_DIM and q_norm_w.is_contiguous(), "q_norm_w must hold 128 values")
    _need(qhat.is_contiguous() and qhat.numel() >= rows * HEADS * HEAD_DIM,
          "qhat must be contiguous [rows, 4, 128]")
    lib = load()
    _check(lib.qsa_prep_queries_dev(_ptr(q), q_stride, _ptr(pos), rows, _ptr(q_norm_w), rotary_dim, rope_theta,
                                    rms_eps, _ptr(dev_tokens), max_tokens, _ptr(qhat), _ptr(dev_status),
                                    _stream_ptr(stream)), "qsa_prep_queries_dev")


def qsa_score_prepped_dev(qhat: torch.Tensor, pos: torch.Tensor, pooled: torch.Tensor,
                          dev_tokens: torch.Tensor, max_tokens: int, scores: torch.Tensor, score_cols: int,
                          dev_status: torch.Tensor, stream=None) -> None:
    """qsa_score_prepped with the live cache length in dev_tokens[0]."""
    _dev(qhat, "qhat", _BF16_LIKE)
    _dev(pos, "pos", (torch.int32,))
    _dev(pooled, "pooled", _BF16_LIKE)
    _dev(scores, "scores", (torch.float32,))
    _dev(dev_status, "dev_status", (torch.int32,))
    _dev_tokens(dev_tokens)
    rows = pos.numel()
    _need(pos.is_contiguous(), "pos must be contiguous")
    _need(qhat.is_contiguous() and qhat.numel() >= rows * HEADS * HEAD_DIM,
          "qhat must be contiguous [rows, 4, 128]")
    _need(pooled.is_contiguous() and pooled.numel() >= (max_tokens // RATIO) * HEAD_DIM,
          "pooled must hold [max_tokens/4, 128]")
    _need(scores.is_contiguous(), "scores must be contiguous")
    lib = load()
    _check(lib.qsa_score_prepped_dev(_ptr(qhat), _ptr(pos), rows, _ptr(pooled), _ptr(dev_tokens), max_tokens,
                                     _ptr(scores), score_cols, scores.numel(), _ptr(dev_status),
                                     _stream_ptr(stream)), "qsa_score_prepped_dev")


def _workspace(workspace):
    if workspace is None:
        return 0
    _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous GPU tensor")
    return workspace.numel() * workspace.element_size()


def qsa_select_indices_ws(scores: torch.Tensor, score_cols: int, pos: torch.Tensor, tokens: int,
                          budget: int, idx: torch.Tensor, counts: torch.Tensor, dev_status: torch.Tensor,
                          workspace: torch.Tensor | None, stream=None) -> None:
    """qsa_select_indices, split over workgroups for few long rows; `workspace`
    holds qsa_select_workspace_bytes(rows, tokens) bytes (None when 0)."""
    _dev(scores, "scores", (torch.float32,))
    _dev(pos, "pos", (torch.int32,))
    _dev(idx, "idx", (torch.int32,))
    _dev(counts, "counts", (torch.int32,))
    _dev(dev_status, "dev_status", (torch.int32,))
    rows = pos.numel()
    _need(pos.is_contiguous() and scores.is_contiguous(), "pos and scores must be contiguous")
    idx_stride = _rows_2d(idx, "idx", budget + RATIO - 1)
    _need(idx.shape[0] >= rows, "idx needs a row per position")
    _need(counts.is_contiguous() and counts.numel() >= rows, "counts must be contiguous [rows]")
    lib = load()
    _check(lib.qsa_select_indices_ws(_ptr(scores), score_cols, scores.numel(), _ptr(pos), rows, tokens, budget,
                                     _ptr(idx), idx_stride, _ptr(counts), _ptr(dev_status), _ptr(workspace),
                                     _workspace(workspace), _stream_ptr(stream)), "qsa_select_indices_ws")


def qsa_select_indices_dev(scores: torch.Tensor, score_cols: int, pos: torch.Tensor,
                           dev_tokens: torch.Tensor, max_tokens: int, budget: int, idx: torch.Tensor,
                           counts: torch.Tensor, dev_status: torch.Tensor, workspace: torch.Tensor | None = None,
                           stream=None) -> None:
    """qsa_select_indices_ws with the live cache length in dev_tokens[0];
    `workspace` holds qsa_select_workspace_bytes(rows, max_tokens) bytes."""
    _dev(scores, "scores", (torch.float32,))
    _dev(pos, "pos", (torch.int32,))
    _dev(idx, "idx", (torch.int32,))
    _dev(counts, "counts", (torch.int32,))
    _dev(dev_status, "dev_status", (torch.int32,))
    _dev_tokens(dev_tokens)
    rows = pos.numel()
    _need(pos.is_contiguous() and scores.is_contiguous(), "pos and scores must be contiguous")
    idx_stride = _rows_2d(idx, "idx", budget + RATIO - 1)
    _need(idx.shape[0] >= rows, "idx needs a row per position")
    _need(counts.is_contiguous() and counts.numel() >= rows, "counts must be contiguous [rows]")
    lib = load()
    _check(lib.qsa_select_indices_dev(_ptr(scores), score_cols, scores.numel(), _ptr(pos), rows, _ptr(dev_tokens),
                                      max_tokens, budget, _ptr(idx), idx_stride, _ptr(counts), _ptr(dev_status),
                                      _ptr(workspace), _workspace(workspace), _stream_ptr(stream)),
           "qsa_select_indices_dev")


def qsa_rope_inv_freq(rotary_dim: int, rope_theta: float) -> list:
    """The library's rotary frequencies (host computation), as Python floats."""
    lib = load()
    buf = (ctypes.c_float * max(1, rotary_dim // 2))()
    _check(lib.qsa_rope_inv_freq(rotary_dim, rope_theta, buf), "qsa_rope_inv_freq")
    return [buf[i] for i in range(rotary_dim // 2)]


def check_status(dev_status: torch.Tensor) -> int:
    """Synchronise and return the status word (QSA_STATUS_* bits)."""
    torch.cuda.synchronize(dev_status.device)
    return int(dev_status.view(-1)[0].item())
