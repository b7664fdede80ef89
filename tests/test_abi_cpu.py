"""libqsa.so on the host: it loads, exports every symbol include/qsa.h
declares, and refuses bad arguments before any HIP call (no GPU needed)."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from sparse_attention_token_qsa_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")

# Fake, never dereferenced device addresses: every call below is refused (or
# is an empty launch) before the library touches HIP.
P = 0x1000
OK, NULL, EXTENT, BUDGET, STRIDE, CAP, PARAM = 0, -1, -2, -3, -4, -5, -6


# These calls pass fake addresses that a launch would dereference; they are
# meant for a host with no GPU (on a GPU host a validation bug would fault).
pytestmark = pytest.mark.skipif(__import__("torch").cuda.device_count() > 0,
                                reason="fake-pointer refusal checks run on a host without a GPU")


@pytest.fixture(scope="module")
def lib():
    return L.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(L.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_abi_version_and_strerror(lib):
    assert lib.qsa_abi_version() == L.ABI_VERSION == 10
    for code in range(-7, 1):
        assert lib.qsa_strerror(code)
    assert b"unknown" in lib.qsa_strerror(-99)


@pytest.mark.parametrize("rd,theta", [(64, 1e4), (64, 1e7), (128, 5e5), (2, 1e4), (36, 123.5)])
def test_host_rope_frequencies_match_the_oracle_bitwise(lib, rd, theta):
    buf = (ctypes.c_float * (rd // 2))()
    assert lib.qsa_rope_inv_freq(rd, theta, buf) == OK
    ours = np.frombuffer(buf, dtype=np.float32)
    assert np.array_equal(ours.view(np.uint32), O.rope_inv_freq(rd, theta).view(np.uint32))


def test_rope_frequency_refusals(lib):
    buf = (ctypes.c_float * 64)()
    assert lib.qsa_rope_inv_freq(63, 1e4, buf) == PARAM
    assert lib.qsa_rope_inv_freq(130, 1e4, buf) == PARAM
    assert lib.qsa_rope_inv_freq(64, 0.0, buf) == PARAM
    assert lib.qsa_rope_inv_freq(64, float("inf"), buf) == PARAM
    assert lib.qsa_rope_inv_freq(64, 1e4, None) == NULL
    assert lib.qsa_rope_inv_freq(0, 1e4, None) == OK


def pool(lib, **kw):
    a = dict(raw=P, key_stride=128, tokens=64, w=P, rd=64, theta=1e4, eps=1e-6,
             first_block=0, n_blocks=16, pooled=P)
    a.update(kw)
    return lib.qsa_pool_keys(a["raw"], a["key_stride"], a["tokens"], a["w"], a["rd"], a["theta"],
                             a["eps"], a["first_block"], a["n_blocks"], a["pooled"], None)


def test_pool_refusals(lib):
    assert pool(lib, n_blocks=0) == OK              # empty launch
    assert pool(lib, tokens=3, n_blocks=0) == OK
    assert pool(lib, raw=None) == NULL
    assert pool(lib, w=None) == NULL
    assert pool(lib, pooled=None) == NULL
    assert pool(lib, tokens=-1) == EXTENT
    assert pool(lib, first_block=-1) == EXTENT
    assert pool(lib, n_blocks=-1) == EXTENT
    assert pool(lib, n_blocks=17) == EXTENT
    assert pool(lib, first_block=10, n_blocks=7) == EXTENT
    assert pool(lib, first_block=17, n_blocks=0) == EXTENT
    assert pool(lib, key_stride=127) == STRIDE
    assert pool(lib, rd=63) == PARAM
    assert pool(lib, rd=130) == PARAM
    assert pool(lib, rd=-2) == PARAM
    assert pool(lib, theta=0.0) == PARAM
    assert pool(lib, theta=float("nan")) == PARAM
    assert pool(lib, eps=-1e-6) == PARAM
    assert pool(lib, eps=float("nan")) == PARAM
    assert pool(lib, eps=float("inf")) == PARAM
    assert pool(lib, tokens=2**62, key_stride=2**10, n_blocks=1) == CAP


def score(lib, **kw):
    a = dict(q=P, q_stride=512, pos=P, rows=8, w=P, rd=64, theta=1e4, eps=1e-6, pooled=P,
             tokens=64, scores=P, score_cols=16, scores_len=128, status=P)
    a.update(kw)
    return lib.qsa_score_rows(a["q"], a["q_stride"], a["pos"], a["rows"], a["w"], a["rd"],
                              a["theta"], a["eps"], a["pooled"], a["tokens"], a["scores"],
                              a["score_cols"], a["scores_len"], a["status"], None)


def test_score_refusals(lib):
    assert score(lib, rows=0) == OK
    assert score(lib, tokens=0, score_cols=0) == OK
    for k in ("q", "pos", "w", "pooled", "scores", "status"):
        assert score(lib, **{k: None}) == NULL, k
    assert score(lib, rows=-1) == EXTENT
    assert score(lib, tokens=-4) == EXTENT
    assert score(lib, q_stride=511) == STRIDE
    assert score(lib, score_cols=15) == STRIDE
    assert score(lib, scores_len=127) == CAP
    assert score(lib, tokens=262148, score_cols=65537, scores_len=8 * 65537) == CAP
    assert score(lib, rows=2**40, scores_len=2**62, score_cols=2**40) == CAP
    assert score(lib, rd=65) == PARAM
    assert score(lib, theta=-1.0) == PARAM
    assert score(lib, eps=float("nan")) == PARAM


def select(lib, **kw):
    a = dict(scores=P, score_cols=16, scores_len=128, pos=P, rows=8, tokens=64, budget=2048,
             mask=P, status=P)
    a.update(kw)
    return lib.qsa_select_mask(a["scores"], a["score_cols"], a["scores_len"], a["pos"], a["rows"],
                               a["tokens"], a["budget"], a["mask"], a["status"], None)


def test_select_refusals(lib):
    assert select(lib, rows=0) == OK
    assert select(lib, tokens=0, score_cols=0) == OK
    for k in ("scores", "pos", "mask", "status"):
        assert select(lib, **{k: None}) == NULL, k
    assert select(lib, rows=-1) == EXTENT
    assert select(lib, score_cols=-1) == EXTENT
    for b in (0, -4, 2, 6, 2052, 4096):
        assert select(lib, budget=b) == BUDGET, b
    assert select(lib, score_cols=15) == STRIDE
    assert select(lib, scores_len=127) == CAP
    assert select(lib, tokens=262148, score_cols=65537, scores_len=8 * 65537) == CAP
    assert select(lib, rows=2**40, score_cols=16, scores_len=2**62) == CAP


def select_idx(lib, **kw):
    a = dict(scores=P, score_cols=16, scores_len=128, pos=P, rows=8, tokens=64, budget=2048,
             idx=P, idx_stride=2051, counts=P, status=P)
    a.update(kw)
    return lib.qsa_select_indices(a["scores"], a["score_cols"], a["scores_len"], a["pos"], a["rows"],
                                  a["tokens"], a["budget"], a["idx"], a["idx_stride"], a["counts"],
                                  a["status"], None)


def test_select_indices_refusals(lib):
    assert select_idx(lib, rows=0) == OK
    assert select_idx(lib, tokens=0, score_cols=0) == OK
    for k in ("scores", "pos", "idx", "counts", "status"):
        assert select_idx(lib, **{k: None}) == NULL, k
    assert select_idx(lib, rows=-1) == EXTENT
    assert select_idx(lib, idx_stride=-1) == EXTENT
    for b in (0, -4, 2, 2052):
        assert select_idx(lib, budget=b) == BUDGET, b
    assert select_idx(lib, score_cols=15) == STRIDE
    assert select_idx(lib, idx_stride=2050) == STRIDE
    assert select_idx(lib, budget=64, idx_stride=66) == STRIDE
    assert select_idx(lib, budget=64, idx_stride=67, rows=0) == OK
    assert select_idx(lib, scores_len=127) == CAP
    assert select_idx(lib, rows=2**40, score_cols=16, scores_len=2**62, idx_stride=2**30) == CAP


def select_ws(lib, **kw):
    a = dict(scores=P, score_cols=16385, scores_len=8 * 16385, pos=P, rows=8, tokens=65540,
             budget=2048, mask=P, status=P, ws=P, ws_bytes=1 << 20)
    a.update(kw)
    return lib.qsa_select_mask_ws(a["scores"], a["score_cols"], a["scores_len"], a["pos"], a["rows"],
                                  a["tokens"], a["budget"], a["mask"], a["status"], a["ws"],
                                  a["ws_bytes"], None)


def test_select_workspace_sizes(lib):
    # one workgroup per row: no workspace
    assert lib.qsa_select_workspace_bytes(8192, 65536) == 0
    assert lib.qsa_select_workspace_bytes(8, 16384) == 0
    assert lib.qsa_select_workspace_bytes(0, 65536) == 0
    # few long rows: one list of 512 composites per 16384-token slice, plus counts
    assert lib.qsa_select_workspace_bytes(16, 262144) == 16 * 16 * (4096 + 256)
    assert lib.qsa_select_workspace_bytes(1, 262147) == 17 * (4096 + 256)
    assert lib.qsa_select_workspace_bytes(64, 65536) == 0
    assert lib.qsa_select_workspace_bytes(64, 65540) == 64 * 5 * (4096 + 256)
    assert lib.qsa_select_workspace_bytes(129, 262144) == 0
    assert lib.qsa_select_workspace_bytes(-1, 64) == EXTENT
    assert lib.qsa_select_workspace_bytes(8, 262148) == CAP


def test_select_ws_refusals(lib):
    assert select_ws(lib, rows=0) == OK
    assert select_ws(lib, tokens=0, score_cols=0) == OK
    for k in ("scores", "pos", "mask", "status", "ws"):
        assert select_ws(lib, **{k: None}) == NULL, k
    assert select_ws(lib, rows=-1) == EXTENT
    assert select_ws(lib, ws_bytes=-1) == EXTENT
    for b in (0, -4, 2, 2052):
        assert select_ws(lib, budget=b) == BUDGET, b
    assert select_ws(lib, score_cols=16384) == STRIDE
    assert select_ws(lib, scores_len=8 * 16385 - 1) == CAP
    assert select_ws(lib, ws_bytes=8 * 5 * (4096 + 256) - 1) == CAP
    assert select_ws(lib, ws=P + 8) == PARAM


def fused(lib, **kw):
    a = dict(qhat=P, pos=P, rows=8, pooled=P, tokens=4096, budget=2048, mask=P, status=P, ws=0x100000,
             ws_bytes=1 << 40)
    a.update(kw)
    return lib.qsa_score_select_mask(a["qhat"], a["pos"], a["rows"], a["pooled"], a["tokens"], a["budget"],
                                     a["mask"], a["status"], a["ws"], a["ws_bytes"], None)


def test_score_select_workspace_sizes(lib):
    assert lib.qsa_score_select_workspace_bytes(0, 65536, 2048) == 0
    assert lib.qsa_score_select_workspace_bytes(8, 0, 2048) == 0
    big = lib.qsa_score_select_workspace_bytes(8192, 65536, 2048)
    # at least the fallback score matrix and the sampled scores
    assert big >= 8192 * 16384 * 4 + 8192 * 1024 * 4
    assert big < 1 << 30
    assert lib.qsa_score_select_workspace_bytes(8, 64, 4) > 0
    assert lib.qsa_score_select_workspace_bytes(8, 64, 4) % 256 == 0
    assert lib.qsa_score_select_workspace_bytes(-1, 64, 4) == EXTENT
    assert lib.qsa_score_select_workspace_bytes(8, -1, 4) == EXTENT
    assert lib.qsa_score_select_workspace_bytes(8, 64, 6) == BUDGET
    assert lib.qsa_score_select_workspace_bytes(8, 64, 2052) == BUDGET
    assert lib.qsa_score_select_workspace_bytes(8, 262148, 4) == CAP
    assert lib.qsa_score_select_workspace_bytes(2**31, 64, 4) == CAP


def test_score_select_refusals(lib):
    assert fused(lib, rows=0) == OK
    assert fused(lib, tokens=0) == OK
    assert fused(lib, rows=0, qhat=None, pos=None, mask=None, status=None, ws=None) == OK
    for k in ("qhat", "pos", "pooled", "mask", "status", "ws"):
        assert fused(lib, **{k: None}) == NULL, k
    assert fused(lib, tokens=3, pooled=None, ws_bytes=0) != NULL  # no complete block: no pooled keys read
    assert fused(lib, rows=-1) == EXTENT
    assert fused(lib, tokens=-1) == EXTENT
    assert fused(lib, ws_bytes=-1) == EXTENT
    for b in (0, -4, 2, 2052):
        assert fused(lib, budget=b) == BUDGET, b
    assert fused(lib, tokens=262148) == CAP
    assert fused(lib, rows=2**31) == CAP
    need = lib.qsa_score_select_workspace_bytes(8, 4096, 2048)
    assert fused(lib, ws_bytes=need - 1) == CAP
    assert fused(lib, ws=0x100000 + 16, ws_bytes=need) == PARAM


def gather(lib, **kw):
    a = dict(k=P, v=P, n_pages=64, page_size=16, kv_dim=512, table=P, table_stride=0, table_len=64,
             idx=P, idx_stride=2051, counts=P, rows=4, slots=2064, ko=P, vo=P, otab=P, status=P)
    a.update(kw)
    return lib.qsa_gather_kv(a["k"], a["v"], a["n_pages"], a["page_size"], a["kv_dim"], a["table"],
                             a["table_stride"], a["table_len"], a["idx"], a["idx_stride"], a["counts"],
                             a["rows"], a["slots"], a["ko"], a["vo"], a["otab"], a["status"], None)


def test_gather_kv_refusals(lib):
    assert gather(lib, rows=0) == OK
    assert gather(lib, slots=0) == OK
    assert gather(lib, rows=0, k=None, v=None, ko=None, vo=None, otab=None, status=None) == OK
    for k in ("k", "v", "table", "idx", "counts", "ko", "vo", "otab", "status"):
        assert gather(lib, **{k: None}) == NULL, k
    for k in ("n_pages", "table_len", "table_stride", "idx_stride", "rows", "slots"):
        assert gather(lib, **{k: -1}) == EXTENT, k
    assert gather(lib, page_size=0) == PARAM
    assert gather(lib, kv_dim=0) == PARAM
    assert gather(lib, slots=2051) == PARAM
    assert gather(lib, table_stride=63) == STRIDE
    assert gather(lib, rows=2**40, slots=2**20) == CAP
    assert gather(lib, n_pages=2**50) == CAP
    assert gather(lib, rows=2**33, slots=16) == CAP


def pool_window(lib, **kw):
    a = dict(raw=P, ks=128, mt=4096, w=P, rd=64, th=1e4, eps=1e-6, dt=P, nb=1, out=P, st=P)
    a.update(kw)
    return lib.qsa_pool_window(a["raw"], a["ks"], a["mt"], a["w"], a["rd"], a["th"], a["eps"], a["dt"], a["nb"],
                               a["out"], a["st"], None)


def test_device_geometry_refusals(lib):
    def pw(**kw):
        return pool_window(lib, **kw)
    assert pw(nb=0) == OK
    for k in ("raw", "w", "dt", "out", "st"):
        assert pw(**{k: None}) == NULL, k
    assert pw(nb=-1) == EXTENT and pw(mt=-4) == EXTENT
    assert pw(nb=1025) == EXTENT
    assert pw(ks=127) == STRIDE
    assert pw(rd=3) == PARAM
    assert pw(mt=262148, nb=1) == CAP
    # prep / score / select with a device count refuse like their host-count twins, and need the word
    assert lib.qsa_prep_queries_dev(P, 512, P, 8, P, 64, 1e4, 1e-6, None, 4096, P, P, None) == NULL
    assert lib.qsa_prep_queries_dev(P, 500, P, 8, P, 64, 1e4, 1e-6, P, 4096, P, P, None) == STRIDE
    assert lib.qsa_prep_queries_dev(P, 512, P, 0, P, 64, 1e4, 1e-6, None, 4096, P, P, None) == OK
    assert lib.qsa_score_prepped_dev(P, P, 8, P, None, 4096, P, 1024, 8 * 1024, P, None) == NULL
    assert lib.qsa_score_prepped_dev(P, P, 8, P, P, 4096, P, 1023, 8 * 1024, P, None) == STRIDE
    assert lib.qsa_score_prepped_dev(P, P, 8, P, P, 4096, P, 1024, 8 * 1024 - 1, P, None) == CAP
    sid = lambda *a: lib.qsa_select_indices_dev(*a, None)  # noqa: E731
    assert sid(P, 1024, 8 * 1024, P, 8, None, 4096, 2048, P, 2051, P, P, None, 0) == NULL
    assert sid(P, 1024, 8 * 1024, P, 8, P, 4096, 2046, P, 2051, P, P, None, 0) == BUDGET
    assert sid(P, 1024, 8 * 1024, P, 8, P, 4096, 2048, P, 2050, P, P, None, 0) == STRIDE
    assert sid(P, 1024, 8 * 1024, P, 0, None, 4096, 2048, P, 2051, P, P, None, 0) == OK
    # long rows need the split workspace
    assert sid(P, 65536, 8 * 65536, P, 8, P, 262144, 2048, P, 2051, P, P, None, 0) == NULL
    need = lib.qsa_select_workspace_bytes(8, 262144)
    assert sid(P, 65536, 8 * 65536, P, 8, P, 262144, 2048, P, 2051, P, P, P, need - 1) == CAP
    assert sid(P, 65536, 8 * 65536, P, 8, P, 262144, 2048, P, 2051, P, P, P + 8, need) == PARAM
    assert sid(P, 65536, 8 * 65536, P, 8, P, 262144, 2048, P, 2051, P, P, P, -1) == EXTENT


def test_select_indices_ws_refusals(lib):
    siw = lambda *a: lib.qsa_select_indices_ws(*a, None)  # noqa: E731
    assert siw(P, 16385, 8 * 16385, P, 0, 65540, 2048, P, 2051, P, P, None, 0) == OK
    for i, name in ((0, "scores"), (3, "pos"), (7, "idx"), (9, "counts"), (10, "status"), (11, "ws")):
        a = [P, 16385, 8 * 16385, P, 8, 65540, 2048, P, 2051, P, P, P, 1 << 20]
        a[i] = None
        assert siw(*a) == NULL, name
    assert siw(P, 16385, 8 * 16385, P, 8, 65540, 2048, P, 2050, P, P, P, 1 << 20) == STRIDE
    assert siw(P, 16385, 8 * 16385, P, 8, 65540, 2046, P, 2051, P, P, P, 1 << 20) == BUDGET
    assert siw(P, 16385, 8 * 16385, P, 8, 65540, 2048, P, 2051, P, P, P, 8 * 5 * (4096 + 256) - 1) == CAP


def prep(lib, **kw):
    a = dict(q=P, q_stride=512, pos=P, rows=8, w=P, rd=64, theta=1e4, eps=1e-6, tokens=64,
             qhat=P, status=P)
    a.update(kw)
    return lib.qsa_prep_queries(a["q"], a["q_stride"], a["pos"], a["rows"], a["w"], a["rd"],
                                a["theta"], a["eps"], a["tokens"], a["qhat"], a["status"], None)


def test_prep_refusals(lib):
    assert prep(lib, rows=0) == OK
    for k in ("q", "pos", "w", "qhat", "status"):
        assert prep(lib, **{k: None}) == NULL, k
    assert prep(lib, rows=-1) == EXTENT
    assert prep(lib, tokens=-1) == EXTENT
    assert prep(lib, q_stride=500) == STRIDE
    assert prep(lib, tokens=262148) == CAP
    assert prep(lib, rows=2**31) == CAP
    assert prep(lib, rows=2**40, q_stride=2**40) == CAP
    assert prep(lib, rd=3) == PARAM
    assert prep(lib, theta=float("inf")) == PARAM
    assert prep(lib, eps=-0.5) == PARAM


def score_prepped(lib, **kw):
    a = dict(qhat=P, pos=P, rows=8, pooled=P, tokens=64, scores=P, score_cols=16, scores_len=128,
             status=P)
    a.update(kw)
    return lib.qsa_score_prepped(a["qhat"], a["pos"], a["rows"], a["pooled"], a["tokens"],
                                 a["scores"], a["score_cols"], a["scores_len"], a["status"], None)


def test_score_prepped_refusals(lib):
    assert score_prepped(lib, rows=0) == OK
    assert score_prepped(lib, tokens=0, score_cols=0) == OK
    for k in ("qhat", "pos", "pooled", "scores", "status"):
        assert score_prepped(lib, **{k: None}) == NULL, k
    assert score_prepped(lib, rows=-1) == EXTENT
    assert score_prepped(lib, scores_len=-1) == EXTENT
    assert score_prepped(lib, score_cols=15) == STRIDE
    assert score_prepped(lib, scores_len=127) == CAP
    assert score_prepped(lib, tokens=262148, score_cols=65537, scores_len=8 * 65537) == CAP
    assert score_prepped(lib, rows=2**40, scores_len=2**62, score_cols=2**20) == CAP


def test_fused_fallback_flags_lie_inside_the_workspace(lib):
    """qsa_score_select_flags_offset: an aligned int32 [rows] array inside the
    fused call's workspace; the workspace-size refusals apply."""
    for rows, T, b in ((8192, 65536, 2048), (8, 64, 4), (301, 65543, 2048), (1024, 65536, 64)):
        n = lib.qsa_score_select_workspace_bytes(rows, T, b)
        off = lib.qsa_score_select_flags_offset(rows, T, b)
        assert 0 < off and off % 256 == 0 and off + 4 * rows <= n, (rows, T, b, off, n)
    assert lib.qsa_score_select_flags_offset(0, 64, 4) == 0
    assert lib.qsa_score_select_flags_offset(8, 0, 4) == 0
    assert lib.qsa_score_select_flags_offset(8, 64, 6) == BUDGET
    assert lib.qsa_score_select_flags_offset(-1, 64, 4) == EXTENT
    assert lib.qsa_score_select_flags_offset(8, 262148, 4) == CAP
