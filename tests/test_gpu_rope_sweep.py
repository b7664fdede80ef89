"""Pooled keys and prepared queries over a whole cache at several rotary
tables, bit-exact against the oracle.

The kernels evaluate each (position, frequency) cos/sin in single precision
and keep it only when its error bound cannot move the bf16 rounding, else in
double; the CPU tests check that certificate on every f32 angle with the host
build of the same code.  Here the device path itself meets the oracle at
every block anchor 4b of a 262147-token cache (the longest accepted) and at
8190 query positions spread over it (the last prep workgroup partly empty), for rotary tables of the pages'
geometry (rotary_dim 64, the launch's fixed-pair kernel) and others (the
general kernel): [SCORE] summary, keys roped at the block's first token and
queries at the row's own position, with bf16 rounding after every rotary
product and sum.
"""

import functools

import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import gpu_pool, gpu_prep, note, u16_host

pytestmark = pytest.mark.gpu

CASES = [(1e4, 64), (1e7, 64), (123.5, 64), (5e5, 128), (1e4, 36)]


@functools.lru_cache(maxsize=1)
def _inputs():
    return synth.rope_sweep(64, 1e4)


def _mismatch(got, want):
    bad = np.nonzero(got != want)
    return len(bad[0]), [tuple(int(i) for i in ix[:4]) for ix in bad]


@pytest.mark.parametrize("theta,rd", CASES)
def test_pool_every_block_anchor_bit_exact(theta, rd):
    w = dict(_inputs(), rotary_dim=rd, theta=theta)
    note(f"rope sweep pool: theta {theta}, rotary_dim {rd}, tokens {w['tokens']}")
    got = u16_host(gpu_pool(w))
    want = O.pool_keys(w["raw_keys"], w["k_norm_w"], rd, theta, w["eps"])
    assert got.shape == want.shape == (w["tokens"] // 4, 128)
    n, where = _mismatch(got, want)
    assert n == 0, (n, where)


@pytest.mark.parametrize("theta,rd", CASES)
def test_prep_positions_across_the_cache_bit_exact(theta, rd):
    w = dict(_inputs(), rotary_dim=rd, theta=theta)
    note(f"rope sweep prep: theta {theta}, rotary_dim {rd}, rows {len(w['pos'])}")
    qhat, st = gpu_prep(w)
    assert st == 0
    want = O.prep_queries(w["queries"], w["pos"], w["q_norm_w"], rd, theta, w["eps"])
    n, where = _mismatch(u16_host(qhat), want)
    assert n == 0, (n, where)
