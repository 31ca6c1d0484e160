"""Pins of the append oracle (oracle/append.py): closed forms and the
algebra of rotations, not a re-typing of its formula."""
import math

import numpy as np

from oracle.append import kv_append, rope


def test_rope_position_zero_is_identity():
    k = np.random.default_rng(1).standard_normal(128)
    assert np.array_equal(rope(k, 0, 10000.0), k)


def test_rope_first_pair_rotates_by_position_radians():
    # j = 0: frequency theta^0 = 1, so the pair (k0, k_{D/2}) turns by pos rad.
    k = np.zeros(64)
    k[0] = 1.0
    out = rope(k, 3, 10000.0)
    assert abs(out[0] - math.cos(3.0)) < 1e-15 and abs(out[32] - math.sin(3.0)) < 1e-15


def test_rope_middle_pair_frequency():
    # D = 64, j = 16: theta^(-2*16/64) = theta^(-1/2) = 1/100 for theta = 1e4;
    # at pos = 100 the pair turns by exactly 1 rad.
    k = np.zeros(64)
    k[16] = 2.0
    out = rope(k, 100, 10000.0)
    assert abs(out[16] - 2 * math.cos(1.0)) < 1e-14
    assert abs(out[48] - 2 * math.sin(1.0)) < 1e-14


def test_rope_preserves_pair_norms_and_composes():
    rng = np.random.default_rng(2)
    k = rng.standard_normal(256)
    a = rope(k, 77, 10000.0)
    H = 128
    assert np.allclose(a[:H] ** 2 + a[H:] ** 2, k[:H] ** 2 + k[H:] ** 2, rtol=0, atol=1e-12)
    assert np.allclose(rope(a, 23, 10000.0), rope(k, 100, 10000.0), rtol=0, atol=1e-12)


def test_rope_scores_depend_on_relative_position():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    d1 = rope(q, 40, 500000.0) @ rope(k, 12, 500000.0)
    d2 = rope(q, 1040, 500000.0) @ rope(k, 1012, 500000.0)
    assert abs(d1 - d2) < 1e-9


def test_append_writes_only_the_slot():
    rng = np.random.default_rng(4)
    nb, Hkv, bs, D, S = 6, 2, 8, 16, 3
    kc = rng.standard_normal((nb, Hkv, bs, D)).astype(np.float16)
    vc = rng.standard_normal((nb, Hkv, bs, D)).astype(np.float16)
    bt = np.array([[4, 1], [0, -1], [5, 2]], dtype=np.int32)
    pos = np.array([11, 5, -1], dtype=np.int32)          # seq 2 skipped
    kn = rng.standard_normal((S, Hkv, D)).astype(np.float16)
    vn = rng.standard_normal((S, Hkv, D)).astype(np.float16)
    k2, v2 = kv_append(kc, vc, bt, pos, kn, vn)
    changed = np.argwhere(np.any(k2.view(np.uint16) != kc.view(np.uint16), axis=-1))
    assert {tuple(x) for x in changed} <= {(1, 0, 3), (1, 1, 3), (0, 0, 5), (0, 1, 5)}
    assert np.array_equal(k2[1, :, 3], kn[0]) and np.array_equal(v2[0, :, 5], vn[1])
    # past the table and invalid page ids write nothing
    k3, _ = kv_append(kc, vc, bt, np.array([16, 9, 0], dtype=np.int32), kn, vn)
    assert np.array_equal(k3[:, :, :, :].view(np.uint16)[np.arange(nb) != 5],
                          kc.view(np.uint16)[np.arange(nb) != 5])
