"""Plain CPU oracle for the QSA token indexer's hot path: pool -> score -> select/mask.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
this module: only the test suite, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code, table or helper with the HIP library.

Sources (web pages; cited by title and section):
  [SEL]   pegainfer pull request 1178, "select QSA indexer blocks and their tail"
  [SCORE] pegainfer pull request 1160, "score QSA token-indexer blocks in native CUDA"
  [QSA]   metrale model layers, layers/qsa.rs (source view)
  [PRE]   atlas spark_model, layers/qsa_select.rs (source view)

Geometry fixed by the pages: 4 query heads, head dim 128, 4-token micro-blocks,
at most 512 kept blocks per row ([SCORE] "Frozen semantics"; [SEL] "Exact
semantics").

Precision.  Where the pages fix a precision it is followed: the block mean is
a float32 mean cast back to bf16, RoPE cos/sin are bf16 values, the RoPE
products and sums round to bf16 after each op, the score is float32
([SCORE] summary and the review's mutation table).  Where they do not, the
oracle computes in float64 and rounds once at the next bf16/f32 point:
the RMSNorm statistic and scale, the RoPE angle trig, and the q.k dot product.
Readings of points the pages leave open are listed per function.

Parity status: every function below is pinned by tests/test_oracle_*.py
against closed forms, invariants, library routines or brute force.
"""

from __future__ import annotations

import numpy as np

HEADS = 4
HEAD_DIM = 128
RATIO = 4
MAX_KEEP_BLOCKS = 512

STATUS_BAD_POSITION = 1
STATUS_NONFINITE_SCORE = 2
STATUS_BAD_INDEX = 4


# ----------------------------------------------------------------------------
# bf16 helpers
# ----------------------------------------------------------------------------

def bf16_from_f32(x) -> np.ndarray:
    """Round float32 values to bf16 bit patterns, round-to-nearest-even.

    Written from the IEEE definition: keep the top 16 bits of the float32
    pattern, rounding on the dropped 16 bits with ties to even.  NaN maps to
    the quiet NaN 0x7FC0; +-Inf stay +-Inf; overflow past the largest bf16
    rounds to Inf as the definition requires.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), rounded).astype(np.uint16)


def f32_from_bf16(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def rb(x) -> np.ndarray:
    """The value of x rounded to bf16, returned as float32."""
    return f32_from_bf16(bf16_from_f32(x))


# ----------------------------------------------------------------------------
# Rotary position embedding (partial)
# ----------------------------------------------------------------------------

def rope_inv_freq(rotary_dim: int, theta: float) -> np.ndarray:
    """Rotary frequencies theta^(-2i/rotary_dim), i < rotary_dim/2, as float32.

    [SCORE] review: the indexer rotates with the same position embeddings as
    attention.  Reading (pages silent on the table's arithmetic): the standard
    rotary table, each frequency evaluated in float64 and rounded once to f32.
    """
    half = rotary_dim // 2
    out = np.empty(half, dtype=np.float32)
    for i in range(half):
        out[i] = np.float32(float(theta) ** (-(2.0 * i) / float(rotary_dim)))
    return out


def rope_cos_sin(position, inv_freq: np.ndarray):
    """bf16-valued cos/sin at integer positions, shape [..., rotary_dim/2].

    The angle is one float32 product position*freq; cos and sin of that f32
    angle are evaluated in float64, rounded to f32 and then to bf16.
    [SCORE] review mutation table: keeping cos/sin in f32 instead of bf16 is a
    detected fault, so the bf16 rounding is part of the definition.
    """
    p = np.asarray(position, dtype=np.int64)
    pf = p.astype(np.float32)[..., None]
    angle = pf * inv_freq.astype(np.float32)  # f32 multiply, correctly rounded
    a64 = angle.astype(np.float64)
    c = rb(np.cos(a64).astype(np.float32))
    s = rb(np.sin(a64).astype(np.float32))
    return c, s


def rope_partial(x_bits: np.ndarray, position, rotary_dim: int, inv_freq: np.ndarray) -> np.ndarray:
    """Partial RoPE on the last axis (128 channels), bf16 in, bf16 out.

    [SCORE] summary: "partial RoPE" with rotary_dim 64 of head dim 128; a
    fault that rotates all 128 channels is detected.  Reading (pages silent on
    the pair layout): channels [0, rotary_dim) rotate as pairs (i, i + half)
    with frequency i, channels [rotary_dim, 128) pass through unchanged, and
    every product and every sum rounds to bf16 (the bf16 tensor-op chain):
        o[i]        = rb(rb(x[i] * c) - rb(x[i+half] * s))
        o[i + half] = rb(rb(x[i+half] * c) + rb(x[i] * s))
    position broadcasts against x's leading axes.
    """
    half = rotary_dim // 2
    x = f32_from_bf16(x_bits)
    out = x.copy()
    if half == 0:
        return bf16_from_f32(out)
    c, s = rope_cos_sin(position, inv_freq)  # [..., half]
    x1 = x[..., :half]
    x2 = x[..., half:rotary_dim]
    o1 = rb(rb(x1 * c) - rb(x2 * s))
    o2 = rb(rb(x2 * c) + rb(x1 * s))
    out[..., :half] = o1
    out[..., half:rotary_dim] = o2
    return bf16_from_f32(out)


# ----------------------------------------------------------------------------
# (1 + w) RMSNorm
# ----------------------------------------------------------------------------

def rms_norm_1pw(x_bits: np.ndarray, w_bits: np.ndarray, eps: float) -> np.ndarray:
    """(1 + w) RMSNorm over the last axis, bf16 in, bf16 out.

    [SCORE] summary: the pooled key goes through a "(1 + w)" RMSNorm; the
    review's table shows the eps is live (eps x100 is a detected fault).
    Reading: y = x / sqrt(mean(x^2) + eps) * (1 + w), evaluated in float64
    with eps taken as the float32 argument value, rounded to f32 then bf16.
    """
    x = f32_from_bf16(x_bits).astype(np.float64)
    w = f32_from_bf16(w_bits).astype(np.float64)
    n = x.shape[-1]
    ms = np.sum(x * x, axis=-1, keepdims=True) / float(n)
    r = 1.0 / np.sqrt(ms + float(np.float32(eps)))
    y = (x * r) * (1.0 + w)
    return bf16_from_f32(y.astype(np.float32))


# ----------------------------------------------------------------------------
# Stage 1: block pooling
# ----------------------------------------------------------------------------

def block_mean(raw_bits: np.ndarray, first_block: int, n_blocks: int) -> np.ndarray:
    """bf16 bits of the float32 mean of each 4-token block's raw keys.

    [SCORE] summary: the block's raw keys are averaged in float32 and cast
    back to bf16; the review shows the bf16 round trip is load-bearing.
    Reading: the f32 sum runs in token order ((k0 + k1) + k2) + k3 and is
    divided by 4.
    """
    rows = f32_from_bf16(raw_bits[RATIO * first_block: RATIO * (first_block + n_blocks)])
    k = rows.reshape(n_blocks, RATIO, -1)
    s = k[:, 0] + k[:, 1]
    s = s + k[:, 2]
    s = s + k[:, 3]
    return bf16_from_f32(s / np.float32(RATIO))


def pool_keys(raw_bits: np.ndarray, k_norm_w_bits: np.ndarray, rotary_dim: int,
              theta: float, eps: float, first_block: int = 0,
              n_blocks: int | None = None) -> np.ndarray:
    """Pooled, normed, roped key of blocks [first_block, first_block + n_blocks).

    [SCORE] summary: mean in float32 -> bf16 -> (1 + w) RMSNorm -> partial
    RoPE at the block's first token; [QSA] module doc: blocks are roped at
    their first position; the review's table shows RoPE at the block end is a
    detected fault.  raw_bits: [tokens, 128] uint16 (bf16); returns
    [n_blocks, 128] uint16.
    """
    raw_bits = np.asarray(raw_bits, dtype=np.uint16)
    if n_blocks is None:
        n_blocks = raw_bits.shape[0] // RATIO - first_block
    if n_blocks == 0:
        return np.zeros((0, HEAD_DIM), dtype=np.uint16)
    m = block_mean(raw_bits, first_block, n_blocks)
    y = rms_norm_1pw(m, k_norm_w_bits, eps)
    anchor = RATIO * (first_block + np.arange(n_blocks, dtype=np.int64))
    return rope_partial(y, anchor, rotary_dim, rope_inv_freq(rotary_dim, theta))


# ----------------------------------------------------------------------------
# Stage 2: query prep + scoring
# ----------------------------------------------------------------------------

def prep_queries(q_bits: np.ndarray, pos: np.ndarray, q_norm_w_bits: np.ndarray,
                 rotary_dim: int, theta: float, eps: float) -> np.ndarray:
    """Per head (1 + w) RMSNorm with q_norm_w, then partial RoPE at the row's
    own position ([SCORE] summary: "norms each of a query row's four heads at
    the row's own position").  q_bits: [rows, 4, 128]; returns the same shape.
    """
    q_bits = np.asarray(q_bits, dtype=np.uint16)
    y = rms_norm_1pw(q_bits, q_norm_w_bits, eps)
    p = np.asarray(pos, dtype=np.int64)[:, None]  # broadcast over heads
    return rope_partial(y, p, rotary_dim, rope_inv_freq(rotary_dim, theta))


def visible_blocks(p: int) -> int:
    """Complete 4-token blocks visible at position p ([SEL] "Exact semantics")."""
    return (p + 1) // RATIO


SCORE_SCALE = np.float32(1.0 / np.sqrt(np.float64(HEAD_DIM)))


def score_rows(qhat_bits: np.ndarray, pos: np.ndarray, pooled_bits: np.ndarray,
               tokens: int) -> list:
    """Block scores of each row: sum_h relu(q_h . k_b) / sqrt(128), b < n(p).

    [SCORE] summary and [QSA] module doc give the formula; the review pins the
    order relu -> head sum -> scale (relu after the sum is a detected fault)
    and that relu keeps NaN like torch.relu.
    Readings: each head dot product is the exact sum rounded once to f32
    (float64 matmul of bf16 values); relu is "d < 0 ? 0 : d"; heads add in
    order ((r0 + r1) + r2) + r3 in f32; the scale is a multiply by the f32
    value of 1/sqrt(128).  Rows whose position is outside [0, tokens) get an
    empty array (the GPU writes nothing for them).
    Returns a list of float32 arrays, one per row, of length n(p).
    """
    qhat = f32_from_bf16(qhat_bits).astype(np.float64)  # [R, 4, 128]
    k = f32_from_bf16(pooled_bits).astype(np.float64)  # [NB, 128]
    out = []
    for r in range(qhat.shape[0]):
        p = int(pos[r])
        if p < 0 or p >= tokens:
            out.append(np.zeros(0, dtype=np.float32))
            continue
        n = visible_blocks(p)
        d = (qhat[r] @ k[:n].T).astype(np.float32)  # [4, n]
        rel = np.where(d < np.float32(0), np.float32(0), d)
        s = rel[0] + rel[1]
        s = s + rel[2]
        s = s + rel[3]
        out.append((s * SCORE_SCALE).astype(np.float32))
    return out


# ----------------------------------------------------------------------------
# Stage 3: exact top-(budget/4) select and the visibility mask
# ----------------------------------------------------------------------------

def check_budget(budget: int) -> None:
    """[SEL] "Exact semantics": budget is a positive multiple of 4 keeping at
    most 512 blocks."""
    if budget <= 0 or budget % RATIO != 0 or budget // RATIO > MAX_KEEP_BLOCKS:
        raise ValueError(f"bad budget {budget}")


def kept_blocks(row_scores: np.ndarray, keep: int) -> np.ndarray:
    """Indices of the `keep` first blocks under the canonical order, ascending.

    [SEL] "Exact semantics": descending score, ascending block index; -0.0
    ties +0.0.  Same order as the host sorts in [QSA] decode_select and
    [PRE] prefill_select.  Computed by a full stable sort.
    """
    s = np.asarray(row_scores, dtype=np.float32)
    s = np.where(s == np.float32(0), np.float32(0), s)  # fold -0.0 onto +0.0
    idx = np.arange(s.shape[0])
    order = np.lexsort((idx, -s))
    return np.sort(order[:keep])


def select_mask_row(row_scores: np.ndarray, p: int, tokens: int, budget: int):
    """One row's u8 mask over [0, tokens) and its status bits.

    [SEL] "Exact semantics": blocks = (p+1)/4, tail = (p+1)%4 tokens at
    4*blocks..=p, keep = min(budget/4, blocks); the mask is 1 on each kept
    block's four tokens and on the tail, 0 elsewhere.  A non-finite score in
    the block prefix is refused (the pages trap; here the row is all zero
    and status bit 2 is set).  Reading: the finiteness check covers every
    row, all-kept rows included.  A position outside [0, tokens) is refused
    with status bit 1 and an all-zero row.
    """
    mask = np.zeros(tokens, dtype=np.uint8)
    if p < 0 or p >= tokens:
        return mask, STATUS_BAD_POSITION
    n = visible_blocks(p)
    s = np.asarray(row_scores[:n], dtype=np.float32)
    if not np.all(np.isfinite(s)):
        return mask, STATUS_NONFINITE_SCORE
    keep = min(budget // RATIO, n)
    for b in kept_blocks(s, keep):
        mask[RATIO * b: RATIO * b + RATIO] = 1
    mask[RATIO * n: p + 1] = 1
    return mask, 0


def select_mask(scores: np.ndarray, score_cols: int, pos: np.ndarray, tokens: int,
                budget: int):
    """Masks of all rows from a row-major [rows, score_cols] f32 score buffer.

    Returns (mask [rows, tokens] uint8, status bits OR-ed over rows).
    """
    check_budget(budget)
    flat = np.asarray(scores, dtype=np.float32).reshape(-1)
    rows = len(pos)
    mask = np.zeros((rows, tokens), dtype=np.uint8)
    status = 0
    for r in range(rows):
        row = flat[r * score_cols: (r + 1) * score_cols]
        m, st = select_mask_row(row, int(pos[r]), tokens, budget)
        mask[r] = m
        status |= st
    return mask, status


def select_indices_row(row_scores: np.ndarray, p: int, tokens: int, budget: int):
    """One row's kept token indices (int32, ascending), padded with -1 to
    budget + 3 entries, their count, and the status bits.

    [QSA] decode_select: the kept blocks (the keep first under the canonical
    order) are sorted ascending and each contributes its RATIO tokens
    RATIO*b .. RATIO*b + RATIO - 1; the tail tokens RATIO*n .. p follow.
    [SCORE] "Next: P3" bounds the list by budget + RATIO - 1 entries.
    Refusals as in select_mask_row: count 0, all entries -1.
    """
    cap = budget + RATIO - 1
    out = np.full(cap, -1, dtype=np.int32)
    if p < 0 or p >= tokens:
        return out, 0, STATUS_BAD_POSITION
    n = visible_blocks(p)
    s = np.asarray(row_scores[:n], dtype=np.float32)
    if not np.all(np.isfinite(s)):
        return out, 0, STATUS_NONFINITE_SCORE
    keep = min(budget // RATIO, n)
    sel = []
    for b in kept_blocks(s, keep):
        sel.extend(range(RATIO * int(b), RATIO * int(b) + RATIO))
    sel.extend(range(RATIO * n, p + 1))
    out[: len(sel)] = sel
    return out, len(sel), 0


def select_indices(scores: np.ndarray, score_cols: int, pos: np.ndarray, tokens: int,
                   budget: int):
    """Index lists of all rows from a row-major [rows, score_cols] f32 score
    buffer.  Returns (idx [rows, budget + 3] int32, counts [rows] int32,
    status bits OR-ed over rows)."""
    check_budget(budget)
    flat = np.asarray(scores, dtype=np.float32).reshape(-1)
    rows = len(pos)
    idx = np.full((rows, budget + RATIO - 1), -1, dtype=np.int32)
    counts = np.zeros(rows, dtype=np.int32)
    status = 0
    for r in range(rows):
        row = flat[r * score_cols: (r + 1) * score_cols]
        idx[r], counts[r], st = select_indices_row(row, int(pos[r]), tokens, budget)
        status |= st
    return idx, counts, status


# ----------------------------------------------------------------------------
# Decode K/V gather
# ----------------------------------------------------------------------------

def gather_kv(k_cache, v_cache, page_size: int, page_table, table_stride: int,
              table_len: int, idx, idx_stride: int, counts, rows: int, slots: int):
    """The selected tokens' K and V vectors copied out of a paged cache into
    contiguous per-row scratch, and the identity page table over it.

    [QSA] module notes and decode_select: the kept token list (ascending kept
    blocks' tokens, then the tail) indexes the sequence's paged K/V cache;
    each listed token's vector is copied, in list order, into a contiguous
    NHD scratch, which the paged decode attention then reads through an
    identity block table of ceil(n_sel / block_size) pages with sequence
    length n_sel.

    Readings where the page is silent, one row per sequence (rows may share
    a cache):
      - cache layout [n_pages, page_size, kv_dim] (page, slot, then the
        kv_heads x head_dim vector), token t of row r at page
        page_table[r * table_stride + t // page_size], slot t % page_size;
        table_stride 0 shares one table;
      - row r's scratch holds `slots` (a multiple of page_size) entries:
        entry i < counts[r] is token idx[r * idx_stride + i], the rest zero;
      - the identity table presents all rows' scratch as one paged pool:
        row r's page j is pool page r * (slots / page_size) + j;
      - a token index that is negative, at or past table_len * page_size, or
        whose page lies outside the cache is written as zeros and sets
        STATUS_BAD_INDEX; so does a count outside [0, min(slots,
        idx_stride)] (a list never outgrows its row), clamped there.

    k_cache, v_cache: [n_pages, page_size, kv_dim] uint16 (bf16 bits).
    Returns (k_out, v_out [rows, slots, kv_dim] uint16, table [rows,
    slots // page_size] int32, status).
    """
    k_cache = np.asarray(k_cache, dtype=np.uint16)
    v_cache = np.asarray(v_cache, dtype=np.uint16)
    n_pages, ps, kv_dim = k_cache.shape
    assert ps == page_size and slots % page_size == 0
    page_table = np.asarray(page_table, dtype=np.int64).reshape(-1)
    idx = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = np.asarray(counts, dtype=np.int64).reshape(-1)
    k_out = np.zeros((rows, slots, kv_dim), dtype=np.uint16)
    v_out = np.zeros((rows, slots, kv_dim), dtype=np.uint16)
    ppr = slots // page_size
    table = np.zeros((rows, ppr), dtype=np.int32)
    status = 0
    for r in range(rows):
        for j in range(ppr):
            table[r, j] = r * ppr + j
        c = int(counts[r])
        cmax = min(slots, idx_stride)
        if c < 0 or c > cmax:
            status |= STATUS_BAD_INDEX
            c = min(max(c, 0), cmax)
        for i in range(c):
            t = int(idx[r * idx_stride + i])
            lp = t // page_size if t >= 0 else -1
            if t < 0 or lp >= table_len:
                status |= STATUS_BAD_INDEX
                continue
            page = int(page_table[r * table_stride + lp])
            if page < 0 or page >= n_pages:
                status |= STATUS_BAD_INDEX
                continue
            k_out[r, i] = k_cache[page, t % page_size]
            v_out[r, i] = v_cache[page, t % page_size]
    return k_out, v_out, table, status


# ----------------------------------------------------------------------------
# Whole path
# ----------------------------------------------------------------------------

def index_mask(raw_bits, q_bits, pos, k_norm_w_bits, q_norm_w_bits, rotary_dim,
               theta, eps, budget, tokens, pooled_edit=None):
    """pool -> score -> select for rows `pos` over a `tokens`-long key cache.

    pooled_edit, if given, is applied to the pooled keys before scoring (a
    test-input construction step, e.g. duplicating a neighbour's pooled key).
    Returns (pooled, per-row scores, mask, status).
    """
    pooled = pool_keys(raw_bits[:tokens], k_norm_w_bits, rotary_dim, theta, eps)
    if pooled_edit is not None:
        pooled = pooled_edit(pooled)
    qhat = prep_queries(q_bits, pos, q_norm_w_bits, rotary_dim, theta, eps)
    scores = score_rows(qhat, pos, pooled, tokens)
    cols = max(1, tokens // RATIO)
    dense = np.zeros((len(pos), cols), dtype=np.float32)
    for r, s in enumerate(scores):
        dense[r, : s.shape[0]] = s
    mask, status = select_mask(dense, cols, pos, tokens, budget)
    return pooled, scores, mask, status
