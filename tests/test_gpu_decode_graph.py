"""A graph-capturable decode step: pool_window -> prep_dev -> score_dev ->
select_indices_dev -> gather, with the live cache length in a device word.

Checked at every cache length, eagerly and as one captured HIP graph
replayed while the cache grows (eager work and synchronisation between
replays, every replay compared), against the oracle: pooled keys and
prepared queries bit-exact, scores within 5e-3, index lists equal to the
oracle's or differing only at blocks within 5e-3 of a row's cut, and the
gathered K/V and page table bit-exact against the oracle's gather of the
lists.  The host-count calls give the same bytes again."""

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_token_qsa_amd as qsa
from tests.gpu_util import DEV, note, workload

pytestmark = pytest.mark.gpu

CEIL = 65536 + 256
ROWS = 4
BUDGET = 2048
WINDOW = 4       # blocks re-pooled per step: covers up to 16 new tokens
KV_DIM, PAGE = 64, 16


class Setup:
    def __init__(self):
        w = workload(3)
        self.w = w
        g = torch.Generator().manual_seed(4321)
        raw = torch.randn((CEIL, 128), generator=g).to(torch.bfloat16)
        self.raw_np = raw.view(torch.int16).numpy().view(np.uint16).copy()
        self.raw = raw.view(torch.int16).to(DEV)
        self.wk = torch.from_numpy(w["k_norm_w"].view(np.int16)).to(DEV)
        self.wq = torch.from_numpy(w["q_norm_w"].view(np.int16)).to(DEV)
        self.q = torch.from_numpy(w["queries"][:ROWS].reshape(ROWS, 512).view(np.int16)).to(DEV)
        n_pages = CEIL // PAGE
        kc = torch.randint(-(1 << 15), 1 << 15, (n_pages, PAGE, KV_DIM), dtype=torch.int16, generator=g)
        vc = torch.randint(-(1 << 15), 1 << 15, (n_pages, PAGE, KV_DIM), dtype=torch.int16, generator=g)
        table = torch.randperm(n_pages, generator=g).to(torch.int32)
        self.kc_np, self.vc_np = kc.numpy().view(np.uint16), vc.numpy().view(np.uint16)
        self.table_np = table.numpy()
        self.kc, self.vc, self.table = kc.to(DEV), vc.to(DEV), table.to(DEV)
        self.n_pages = n_pages
        self.slots = -(-(BUDGET + 3) // PAGE) * PAGE

    def rope(self):
        w = self.w
        return w["rotary_dim"], w["theta"], w["eps"]

    def buffers(self):
        b = {
            "pooled": torch.zeros((CEIL // 4, 128), dtype=torch.int16, device=DEV),
            "qhat": torch.zeros((ROWS, 4, 128), dtype=torch.int16, device=DEV),
            "scores": torch.zeros(ROWS * (CEIL // 4), dtype=torch.float32, device=DEV),
            "idx": torch.full((ROWS, BUDGET + 3), -5, dtype=torch.int32, device=DEV),
            "counts": torch.zeros(ROWS, dtype=torch.int32, device=DEV),
            "ko": torch.zeros((ROWS, self.slots, KV_DIM), dtype=torch.int16, device=DEV),
            "vo": torch.zeros((ROWS, self.slots, KV_DIM), dtype=torch.int16, device=DEV),
            "tab": torch.zeros((ROWS, self.slots // PAGE), dtype=torch.int32, device=DEV),
            "st": torch.zeros(1, dtype=torch.int32, device=DEV),
            "ws": torch.full((max(qsa.qsa_select_workspace_bytes(ROWS, CEIL), 16),), 0x5A, dtype=torch.uint8,
                             device=DEV),
            "pos": torch.zeros(ROWS, dtype=torch.int32, device=DEV),
            "dt": torch.zeros(1, dtype=torch.int32, device=DEV),
        }
        return b

    def reference(self, T):
        """The host-count path at cache length T: every complete block pooled,
        rows at position T - 1."""
        rd, th, eps = self.rope()
        b = self.buffers()
        b["pos"].fill_(T - 1)
        qsa.qsa_pool_keys(self.raw[:T], self.wk, rd, th, eps, b["pooled"])
        qsa.qsa_prep_queries(self.q, b["pos"], self.wq, rd, th, eps, T, b["qhat"], b["st"])
        qsa.qsa_score_prepped(b["qhat"], b["pos"], b["pooled"], T, b["scores"], CEIL // 4, b["st"])
        qsa.qsa_select_indices(b["scores"], CEIL // 4, b["pos"], T, BUDGET, b["idx"], b["counts"], b["st"])
        qsa.qsa_gather_kv(self.kc, self.vc, self.table, 0, self.n_pages, b["idx"], b["counts"], b["ko"], b["vo"],
                          b["tab"], b["st"])
        torch.cuda.synchronize()
        return b

    def step(self, b):
        """The device-geometry step; reads T from b["dt"] and positions from b["pos"]."""
        rd, th, eps = self.rope()
        qsa.qsa_pool_window(self.raw, self.wk, rd, th, eps, b["dt"], WINDOW, b["pooled"], b["st"])
        qsa.qsa_prep_queries_dev(self.q, b["pos"], self.wq, rd, th, eps, b["dt"], CEIL, b["qhat"], b["st"])
        qsa.qsa_score_prepped_dev(b["qhat"], b["pos"], b["pooled"], b["dt"], CEIL, b["scores"], CEIL // 4, b["st"])
        qsa.qsa_select_indices_dev(b["scores"], CEIL // 4, b["pos"], b["dt"], CEIL, BUDGET, b["idx"], b["counts"],
                                   b["st"], b["ws"])
        qsa.qsa_gather_kv(self.kc, self.vc, self.table, 0, self.n_pages, b["idx"], b["counts"], b["ko"], b["vo"],
                          b["tab"], b["st"])


class OracleRef:
    """The oracle's pooled keys of the whole ceiling (a block depends only
    on its own four tokens), and per cache length the oracle's prepared
    queries, scores and index lists of the step's rows at position T - 1."""

    def __init__(self, s):
        self.s = s
        w = s.w
        self.pooled = O.pool_keys(s.raw_np, w["k_norm_w"], w["rotary_dim"], w["theta"], w["eps"])
        self.q = w["queries"][:ROWS]

    def at(self, T):
        w = self.s.w
        pos = np.full(ROWS, T - 1, dtype=np.int32)
        qhat = O.prep_queries(self.q, pos, w["q_norm_w"], w["rotary_dim"], w["theta"], w["eps"])
        sc = O.score_rows(qhat, pos, self.pooled[: T // 4], T)
        cols = CEIL // 4
        dense = np.full((ROWS, cols), np.nan, np.float32)
        for r, v in enumerate(sc):
            dense[r, : len(v)] = v
        idx, cnt, st = O.select_indices(dense, cols, pos, T, BUDGET)
        assert st == 0
        return qhat, sc, idx, cnt


def assert_oracle(got, oref, T, label):
    """The step's outputs at cache length T against the oracle."""
    n = T // 4
    qhat, sc, idx, cnt = oref.at(T)
    pooled = got["pooled"][:n].cpu().numpy().view(np.uint16)
    assert np.array_equal(pooled, oref.pooled[:n]), f"{label}: pooled keys differ from the oracle at T={T}"
    assert np.array_equal(got["qhat"].cpu().numpy().view(np.uint16), qhat), f"{label}: qhat differs at T={T}"
    gs = got["scores"].view(ROWS, CEIL // 4)[:, :n].cpu().numpy().astype(np.float64)
    for r in range(ROWS):
        assert np.max(np.abs(gs[r] - sc[r])) <= 5e-3, f"{label}: scores past the bound at T={T}"
    gi = got["idx"].cpu().numpy()
    gc = got["counts"].cpu().numpy()
    p = T - 1
    keep = min(BUDGET // 4, n)
    tail = (p + 1) % 4
    for r in range(ROWS):
        assert gc[r] == cnt[r] == 4 * keep + tail, f"{label}: count at T={T}"
        if np.array_equal(gi[r, : BUDGET + 3], idx[r]):
            continue
        lst = gi[r, : gc[r]]
        assert np.all(gi[r, gc[r]: BUDGET + 3] == -1)
        assert np.all(np.diff(lst) > 0) and np.array_equal(lst[4 * keep:], np.arange(4 * n, p + 1))
        gb = lst[: 4 * keep].reshape(keep, 4)
        assert np.all(gb % 4 == np.arange(4)) and np.all(gb[:, 1:] - gb[:, :1] == np.arange(1, 4))
        gset, wset = set(gb[:, 0] // 4), set(idx[r, : 4 * keep: 4] // 4)
        cut = np.sort(sc[r])[::-1][keep - 1]
        diff = np.array(sorted(gset ^ wset))
        assert np.all(np.abs(sc[r][diff].astype(np.float64) - cut) <= 5e-3), f"{label}: lists at T={T}"
    s = oref.s
    ko, vo, tab, st = O.gather_kv(s.kc_np, s.vc_np, PAGE, s.table_np, 0, s.n_pages, gi, gi.shape[1], gc, ROWS,
                                  s.slots)
    assert st == 0
    assert np.array_equal(got["ko"].cpu().numpy().view(np.uint16), ko), f"{label}: gathered K at T={T}"
    assert np.array_equal(got["vo"].cpu().numpy().view(np.uint16), vo), f"{label}: gathered V at T={T}"
    assert np.array_equal(got["tab"].cpu().numpy(), tab), f"{label}: page table at T={T}"


def assert_same(got, ref, T, label):
    n = T // 4
    pooled_ok = torch.equal(got["pooled"][:n], ref["pooled"][:n])
    sc_g = got["scores"].view(ROWS, CEIL // 4)[:, :n]
    sc_r = ref["scores"].view(ROWS, CEIL // 4)[:, :n]
    assert pooled_ok, f"{label}: pooled keys differ at T={T}"
    assert torch.equal(got["qhat"], ref["qhat"]), f"{label}: prepared queries differ at T={T}"
    assert torch.equal(sc_g.view(torch.int32), sc_r.view(torch.int32)), f"{label}: scores differ at T={T}"
    assert torch.equal(got["idx"], ref["idx"]) and torch.equal(got["counts"], ref["counts"]), \
        f"{label}: index lists differ at T={T}"
    for k in ("ko", "vo", "tab"):
        assert torch.equal(got[k], ref[k]), f"{label}: {k} differs at T={T}"


def test_device_geometry_calls_equal_host_count_calls():
    s = Setup()
    oref = OracleRef(s)
    b = s.buffers()
    T0 = CEIL - 200
    rd, th, eps = s.rope()
    qsa.qsa_pool_keys(s.raw[:T0 - 1], s.wk, rd, th, eps, b["pooled"])  # the cache before the first step
    for T in (T0, T0 + 1, T0 + 2, T0 + 3, T0 + 4, T0 + 11, T0 + 27):
        note(f"device geometry, eager: T={T}")
        b["dt"].fill_(T)
        b["pos"].fill_(T - 1)
        b["st"].zero_()
        s.step(b)
        torch.cuda.synchronize()
        assert int(b["st"].item()) == 0
        assert_oracle(b, oref, T, "eager")
        assert_same(b, s.reference(T), T, "eager")


def test_captured_decode_step_replays_as_the_cache_grows():
    s = Setup()
    oref = OracleRef(s)
    b = s.buffers()
    T0 = CEIL - 120
    rd, th, eps = s.rope()
    qsa.qsa_pool_keys(s.raw[:T0 - 1], s.wk, rd, th, eps, b["pooled"])
    b["dt"].fill_(T0)
    b["pos"].fill_(T0 - 1)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        s.step(b)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    note("capturing the decode step")
    with torch.cuda.graph(graph):
        s.step(b)
    torch.cuda.synchronize()
    T = T0
    for k, add in enumerate((0, 1, 1, 1, 1, 3, 5, 16, 2, 1)):
        T += add
        note(f"replay {k}: T={T}")
        b["dt"].fill_(T)
        b["pos"].fill_(T - 1)
        b["st"].zero_()
        b["idx"].fill_(-9)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(b["st"].item()) == 0
        assert_oracle(b, oref, T, f"replay {k}")
        assert_same(b, s.reference(T), T, f"replay {k}")


def test_device_count_past_the_ceiling_is_clamped_and_flagged():
    s = Setup()
    b = s.buffers()
    rd, th, eps = s.rope()
    qsa.qsa_pool_keys(s.raw, s.wk, rd, th, eps, b["pooled"])
    b["dt"].fill_(CEIL + 9)
    b["pos"].fill_(CEIL - 1)
    s.step(b)
    torch.cuda.synchronize()
    assert int(b["st"].item()) == qsa.STATUS_BAD_GEOMETRY
    ref = s.reference(CEIL)
    assert torch.equal(b["idx"], ref["idx"]) and torch.equal(b["ko"], ref["ko"])


def test_one_row_device_count_scorer_against_the_oracle():
    """The one-row streaming scorer with the live cache length on the device
    (its key loads are clamped to the live blocks, not the ceiling): one row
    at T - 1 for cache lengths well below the ceiling, with no complete
    block, and past the ceiling (clamped and flagged); scores within the
    bound of the oracle, nothing written past the prefix, and equal bit for
    bit to the host-count call at the same length."""
    s = Setup()
    oref = OracleRef(s)
    w = s.w
    rd, th, eps = s.rope()
    pooled = torch.from_numpy(oref.pooled.view(np.int16)).to(DEV)
    q1 = s.q[:1]
    cols = CEIL // 4
    for T in (CEIL, CEIL - 200, 40001, 7, 3):
        note(f"one-row device-count scorer: T={T} of {CEIL}")
        pos = torch.full((1,), T - 1, dtype=torch.int32, device=DEV)
        dt = torch.full((1,), T, dtype=torch.int32, device=DEV)
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        qhat = torch.zeros((1, 4, 128), dtype=torch.int16, device=DEV)
        qsa.qsa_prep_queries(q1, pos, s.wq, rd, th, eps, T, qhat, st)
        sc = torch.full((cols,), -7.25, dtype=torch.float32, device=DEV)
        qsa.qsa_score_prepped_dev(qhat, pos, pooled, dt, CEIL, sc, cols, st)
        ref = torch.full((cols,), -7.25, dtype=torch.float32, device=DEV)
        qsa.qsa_score_prepped(qhat, pos, pooled, T, ref, cols, st)
        assert qsa.check_status(st) == 0
        n = T // 4
        got = sc.cpu().numpy()
        assert np.all(got[n:] == np.float32(-7.25)), f"wrote past the prefix at T={T}"
        assert torch.equal(sc.view(torch.int32), ref.view(torch.int32)), f"device count vs host count at T={T}"
        qh = O.prep_queries(w["queries"][:1], np.array([T - 1], np.int32), w["q_norm_w"], rd, th, eps)
        want = O.score_rows(qh, np.array([T - 1], np.int32), oref.pooled[:n], T)[0]
        if n:
            assert np.max(np.abs(got[:n].astype(np.float64) - want)) <= 5e-3, f"scores past the bound at T={T}"
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    sc = torch.full((cols,), -7.25, dtype=torch.float32, device=DEV)
    qsa.qsa_score_prepped_dev(qhat, torch.full((1,), CEIL - 1, dtype=torch.int32, device=DEV), pooled,
                              torch.full((1,), CEIL + 9, dtype=torch.int32, device=DEV), CEIL, sc, cols, st)
    assert qsa.check_status(st) == qsa.STATUS_BAD_GEOMETRY
