"""Pins of the oracle's routing (MegaGate order: score -> bias ranking ->
Top-K -> score extraction -> normalise -> scale; HashRouter ids from
tid2eid[input_ids] weighted from the gate logits).

- Top-K against brute-force enumeration of every k-subset on tiny E, with
  forced exact ties, under the total order (biased score desc, expert asc).
- Library cross-check against numpy's lexsort.
- Weights against the textbook normalised sigmoid in fp64 (which fails if the
  biased score, a wrong slot or no normalisation were used).
- Closed forms: k = 1 gives w = scale exactly; scale = 0 gives 0.
"""
import itertools

import numpy as np
import pytest

U = 2.0 ** -24


def _ranked(orc, logits, bias_rows):
    """(r desc, e asc) ranking inputs: r = fl32(S(l) + b) per token."""
    s = orc.score(logits)
    return (s + bias_rows).astype(np.float32), s


def _beats(r, a, b):
    """Expert a precedes expert b: larger biased score, then smaller index."""
    return r[a] > r[b] or (r[a] == r[b] and a < b)


@pytest.mark.parametrize("E,k", [(5, 1), (6, 2), (8, 2), (9, 3), (12, 4), (7, 7)])
@pytest.mark.parametrize("ties", [False, True])
def test_topk_brute_force(orc, E, k, ties):
    rng = np.random.default_rng(100 * E + k + ties)
    T = 60
    if ties:
        logits = rng.choice([-1.0, 0.0, 1.0], size=(T, E)).astype(np.float32)
        bias = rng.choice([0.0, 0.25], size=(1, E)).astype(np.float32)
    else:
        logits = rng.normal(0, 1, (T, E)).astype(np.float32)
        bias = rng.uniform(-0.1, 0.1, (1, E)).astype(np.float32)
    ids, w, flags = orc.route(logits, k, 1.0, bias=bias)
    assert flags == 0
    r, _ = _ranked(orc, logits, bias[0][None, :])
    for t in range(T):
        dominant = []
        for sub in itertools.combinations(range(E), k):
            rest = [e for e in range(E) if e not in sub]
            if all(_beats(r[t], a, b) for a in sub for b in rest):
                dominant.append(set(sub))
        assert len(dominant) == 1
        assert set(ids[t].tolist()) == dominant[0]
        # slots listed in ranking order
        for j in range(k - 1):
            assert _beats(r[t], ids[t, j], ids[t, j + 1])


def test_topk_matches_lexsort(orc):
    rng = np.random.default_rng(7)
    T, E, k = 500, 384, 6
    logits = rng.normal(0, 1, (T, E)).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, (2, E)).astype(np.float32)
    modality = (rng.random(T) < 0.3).astype(np.uint8)
    ids, _, _ = orc.route(logits, k, 2.5, bias=bias, modality=modality)
    r, _ = _ranked(orc, logits, bias[modality.astype(np.int64)])
    for t in range(T):
        order = np.lexsort((np.arange(E), -r[t].astype(np.float64)))
        assert ids[t].tolist() == order[:k].tolist()


def _textbook_weights(logits, ids, scale):
    l = np.take_along_axis(logits.astype(np.float64), ids.astype(np.int64), axis=1)
    s = 1.0 / (1.0 + np.exp(-l))
    return scale * s / s.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("scale", [1.0, 2.5])
def test_weights_textbook(orc, scale):
    rng = np.random.default_rng(11)
    T, E, k = 400, 64, 6
    logits = rng.normal(0, 1.5, (T, E)).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, (1, E)).astype(np.float32)
    ids, w, _ = orc.route(logits, k, scale, bias=bias)
    ref = _textbook_weights(logits, ids, scale)
    rel = np.abs(w - ref) / ref
    assert rel.max() <= (3 + k + 3) * U * 2
    # normalised weights sum to the scale factor
    assert np.max(np.abs(w.astype(np.float64).sum(axis=1) - scale)) <= 8 * k * U * scale


def test_weights_closed_forms(orc):
    rng = np.random.default_rng(12)
    logits = rng.normal(0, 1, (50, 16)).astype(np.float32)
    _, w1, _ = orc.route(logits, 1, 2.5)
    assert np.all(w1 == np.float32(2.5))
    _, w0, _ = orc.route(logits, 4, 0.0)
    assert np.all(w0 == 0)


def test_modality_selects_bias_row(orc):
    T, E, k = 4, 8, 2
    logits = np.zeros((T, E), np.float32)
    bias = np.zeros((2, E), np.float32)
    bias[0, [1, 2]] = 0.5   # text prefers experts 1, 2
    bias[1, [6, 7]] = 0.5   # vision prefers experts 6, 7
    modality = np.array([0, 1, 1, 0], np.uint8)
    ids, w, _ = orc.route(logits, k, 1.0, bias=bias, modality=modality)
    assert ids.tolist() == [[1, 2], [6, 7], [6, 7], [1, 2]]
    # bias only ranks: equal logits give equal weights
    assert np.all(w == np.float32(0.5))


def test_hash_router(orc):
    rng = np.random.default_rng(13)
    V, E, k, T = 1000, 384, 6, 300
    tab = np.stack([rng.choice(E, k, replace=False) for _ in range(V)]).astype(np.int32)
    input_ids = rng.integers(0, V, T).astype(np.int32)
    logits = rng.normal(0, 1, (T, E)).astype(np.float32)
    ids, w, flags = orc.route(logits, k, 2.5, input_ids=input_ids, tid2eid=tab,
                              mode=orc.MODE_HASH)
    assert flags == 0
    assert np.array_equal(ids, tab[input_ids])
    ref = _textbook_weights(logits, ids, 2.5)
    assert (np.abs(w - ref) / ref).max() <= (3 + k + 3) * U * 2
    # equal input ids and equal logits give equal routing
    logits[1] = logits[0]
    input_ids[1] = input_ids[0]
    ids, w, _ = orc.route(logits, k, 2.5, input_ids=input_ids, tid2eid=tab,
                          mode=orc.MODE_HASH)
    assert np.array_equal(ids[0], ids[1]) and np.array_equal(w[0], w[1])


def test_hash_router_bad_ids(orc):
    V, E, k = 4, 8, 2
    tab = np.array([[0, 1], [2, 3], [4, 9], [5, 6]], np.int32)  # row 2 holds 9 >= E
    input_ids = np.array([0, 7, 2, 3, -1], np.int32)
    logits = np.zeros((5, E), np.float32)
    ids, w, flags = orc.route(logits, k, 1.0, input_ids=input_ids, tid2eid=tab,
                              mode=orc.MODE_HASH)
    assert flags == orc.FLAG_BAD_INPUT_ID | orc.FLAG_BAD_EXPERT_ID
    assert ids.tolist() == [[0, 1], [-1, -1], [-1, -1], [5, 6], [-1, -1]]
    assert np.all(w[[1, 2, 4]] == 0)
