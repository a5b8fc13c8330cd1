"""Pins of oracle/sparse.py (2:4 magnitude pruning and its compressed form) against a
hand-worked fixture, brute force over every pair of a group, and invariants. CPU only."""
import itertools

import numpy as np

import tel_inputs as ti
from oracle import encoder as enc
from oracle import sparse as sp
from tests.test_oracle_encoder import golden_rows


def _golden():
    rows = {}
    for tok in golden_rows("prune_2of4.txt"):
        rows.setdefault(tok[0], {})[int(tok[1])] = [float(v) for v in tok[2:]]
    return rows


def test_golden_prune_and_compress():
    """tests/golden/prune_2of4.txt, worked by hand from the pruning rule."""
    g = _golden()
    w = np.array([g["w"][0], g["w"][1]])
    assert np.array_equal(sp.prune_2of4(w), np.array([g["pruned"][0], g["pruned"][1]]))
    values, index = sp.compress_2of4(w)
    assert np.array_equal(values, np.array([g["values"][0], g["values"][1]]))
    assert index.dtype == np.uint16
    assert index[:, 0].tolist() == [int(g["index"][0][0]), int(g["index"][1][0])]


def _brute_keep(group):
    """The pair of positions with the largest sum of magnitudes; among equal sums the
    lexicographically smallest pair (equivalent to: largest first, ties to lower k)."""
    best = None
    for pair in itertools.combinations(range(4), 2):
        s = abs(group[pair[0]]) + abs(group[pair[1]])
        if best is None or s > best[0]:
            best = (s, pair)
    return best[1]


def test_keep_positions_brute_force():
    rng = np.random.default_rng(0)
    # small integers make ties (and zeros) frequent
    w = rng.integers(-3, 4, size=(64, 64)).astype(np.float64) * 0.5
    pos = sp.keep_positions(w)
    for n in range(w.shape[0]):
        for q in range(w.shape[1] // 4):
            assert tuple(pos[n, q]) == _brute_keep(w[n, 4 * q:4 * q + 4]), (n, q)


def test_prune_invariants():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((48, 96))
    p = sp.prune_2of4(w)
    groups = w.reshape(48, 24, 4)
    kept = p.reshape(48, 24, 4) != 0
    assert (kept.sum(axis=-1) == 2).all()              # continuous values: no zero ties
    # every kept magnitude is at least every dropped one in its group
    kmin = np.where(kept, np.abs(groups), np.inf).min(axis=-1)
    dmax = np.where(~kept, np.abs(groups), -np.inf).max(axis=-1)
    assert (kmin >= dmax).all()
    assert np.array_equal(sp.prune_2of4(p), p)         # idempotent
    assert np.array_equal(p[p != 0], w[p != 0])         # kept weights unchanged


def test_compress_roundtrip_and_index_range():
    rng = np.random.default_rng(2)
    w = rng.integers(-2, 3, size=(40, 128)).astype(np.float64)
    values, index = sp.compress_2of4(w)
    assert values.shape == (40, 64) and index.shape == (40, 8)
    assert np.array_equal(sp.decompress_2of4(values, index, 128), sp.prune_2of4(w))
    # in every group the two positions differ and increase
    for shift in range(0, 16, 4):
        p0 = (index.astype(np.int64) >> shift) & 3
        p1 = (index.astype(np.int64) >> (shift + 2)) & 3
        assert (p0 < p1).all()


def test_sparse_linear_is_dense_linear_on_pruned_weights():
    """Zeroed weights contribute nothing: the product over the kept weights only (brute
    force over the compressed form) equals the dense product with the pruned matrix."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 32))
    w = rng.standard_normal((6, 32))
    b = rng.standard_normal(6)
    values, index = sp.compress_2of4(w)
    ref = np.zeros((5, 6))
    for m in range(5):
        for n in range(6):
            s = b[n]
            for wd in range(2):
                word = int(index[n, wd])
                for g in range(4):
                    for j in range(2):
                        k = 16 * wd + 4 * g + ((word >> (4 * g + 2 * j)) & 3)
                        s += x[m, k] * values[n, 8 * wd + 2 * g + j]
            ref[m, n] = s
    assert np.allclose(sp.linear_2of4(x, w, b), ref, rtol=0, atol=1e-12)


def test_pruned_layer_changes_only_projections():
    cfg = ti.ENCODER_CONFIGS["tiny"]
    w = ti.encoder_layer_weights(cfg, 0, variant=True)
    p = sp.prune_layer_weights(w)
    for k, v in w.items():
        if k in sp.SPARSE_WEIGHTS:
            assert np.array_equal(p[k], sp.prune_2of4(v))
            assert (p[k] == 0).mean() >= 0.5
        else:
            assert p[k] is v
    lens, x = ti.encoder_input(cfg)
    y = enc.encoder_forward(x, lens, [p], cfg["heads"], ti.LN_EPS)
    assert np.isfinite(y).all()
