"""The streaming recurrence the GPU kernels implement, run in fp64 against the oracle.

This pins the algebra of the online formulation (technical summary, Method 1:
five running scalars m1, m2, l1, l2, acc and L = acc/l1 + LSE2 - LSE1), in the
exact form the kernels use: logits in base-2 units y = S * log2(e), each key
tile updating (M1, l1, A, M2, l2), the tile's sum of p1 * (y1 - y2) split into
p1 * (t1 - t2) plus (M1 - M2) * sum(p1), partial states over disjoint key sets
merged with the associative rule, and empty partials (no visible key) carried
as (-inf, 0, 0, -inf, 0).  Any tiling and any split of the keys must give the
definition to ~1e-13.
"""
import math

import numpy as np
import pytest

import oracle

LOG2E = 1.0 / math.log(2.0)
LN2 = math.log(2.0)


def empty_state():
    return [-math.inf, 0.0, 0.0, -math.inf, 0.0]


def tile_update(st, y1, y2):
    """y1, y2: base-2 logits of the visible keys of one tile (may be empty)."""
    M1, l1, A, M2, l2 = st
    mx1 = max(y1) if len(y1) else -math.inf
    mx2 = max(y2) if len(y2) else -math.inf
    M1n, M2n = max(M1, mx1), max(M2, mx2)
    M1s = 0.0 if M1n == -math.inf else M1n
    M2s = 0.0 if M2n == -math.inf else M2n
    a1 = 2.0 ** (M1 - M1s)
    a2 = 2.0 ** (M2 - M2s)
    t1 = np.asarray(y1) - M1s
    t2 = np.asarray(y2) - M2s
    p1, p2 = 2.0 ** t1, 2.0 ** t2
    tl1, tl2 = p1.sum(), p2.sum()
    tA = (p1 * (t1 - t2)).sum()
    return [M1n, a1 * l1 + tl1, a1 * A + tA + (M1s - M2s) * tl1, M2n, a2 * l2 + tl2]


def merge(a, b):
    M1, M2 = max(a[0], b[0]), max(a[3], b[3])
    M1s = 0.0 if M1 == -math.inf else M1
    M2s = 0.0 if M2 == -math.inf else M2
    wa1, wb1 = 2.0 ** (a[0] - M1s), 2.0 ** (b[0] - M1s)
    wa2, wb2 = 2.0 ** (a[3] - M2s), 2.0 ** (b[3] - M2s)
    return [M1, wa1 * a[1] + wb1 * b[1], wa1 * a[2] + wb1 * b[2], M2, wa2 * a[4] + wb2 * b[4]]


def finish(st):
    M1, l1, A, M2, l2 = st
    lse1_2 = M1 + math.log2(l1)
    lse2_2 = M2 + math.log2(l2)
    return LN2 * (A / l1 + lse2_2 - lse1_2), LN2 * lse1_2, LN2 * lse2_2


def streaming_row(S1row, S2row, vis, tile, lanes, splits):
    """keys split into `splits` contiguous ranges; inside each range keys go in
    tiles; within a tile, key j belongs to lane partial (j // 4) % lanes."""
    n_k = len(S1row)
    bounds = np.linspace(0, n_k, splits + 1).astype(int)
    parts = []
    for s in range(splits):
        lane_states = [empty_state() for _ in range(lanes)]
        for t0 in range(bounds[s], bounds[s + 1], tile):
            t1_ = min(t0 + tile, bounds[s + 1])
            for ln in range(lanes):
                js = [j for j in range(t0, t1_) if ((j - t0) // 4) % lanes == ln and vis[j]]
                lane_states[ln] = tile_update(lane_states[ln], [S1row[j] * LOG2E for j in js],
                                              [S2row[j] * LOG2E for j in js])
        st = lane_states[0]
        for o in lane_states[1:]:
            st = merge(st, o)
        parts.append(st)
    st = parts[0]
    for o in parts[1:]:
        st = merge(st, o)
    return finish(st)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tile,lanes,splits", [(64, 2, 1), (8, 2, 3), (16, 1, 7), (4, 2, 40)])
def test_streaming_recurrence_equals_definition(causal, tile, lanes, splits):
    r = np.random.default_rng(3)
    n_q, n_k, d = 9, 37, 8
    q1, k1 = r.normal(size=(n_q, d)), r.normal(size=(n_k, d))
    q2, k2 = q1 + 0.5 * r.normal(size=(n_q, d)), k1 + 0.5 * r.normal(size=(n_k, d))
    k1[5] += 4.0  # a key with much larger logits: exercises the max rescaling
    kl, l1, l2 = oracle.head_forward(q1, k1, q2, k2, causal)
    S1, S2 = oracle.scores(q1, k1, d ** -0.5), oracle.scores(q2, k2, d ** -0.5)
    for i in range(n_q):
        vis = oracle.valid_mask(np.array([i]), n_q, n_k, causal)[0]
        got = streaming_row(S1[i], S2[i], vis, tile, lanes, splits)
        assert got[0] == pytest.approx(kl[i], rel=1e-12, abs=1e-13)
        assert got[1] == pytest.approx(l1[i], rel=1e-13)
        assert got[2] == pytest.approx(l2[i], rel=1e-13)


def test_empty_partials_merge_to_nothing():
    st = merge(empty_state(), empty_state())
    assert st[0] == -math.inf and st[1] == 0.0 and st[2] == 0.0
    full = tile_update(empty_state(), [0.5, -1.0], [0.25, 2.0])
    assert merge(full, empty_state()) == pytest.approx(full)
    assert merge(empty_state(), full) == pytest.approx(full)


CAP = 2.0 ** 64


def tile_update_held(st, y1, y2):
    """The long-range forward's update of an unmasked tile with the state's
    offsets held: the terms are taken against the offsets the state has (0
    for a state with none). A state with no offset yet, or a tile whose sums
    pass 2^64, takes the tile maxima as offsets instead, never lowering them,
    and sums the tile again."""
    M1, l1, A, M2, l2 = st
    y1, y2 = np.asarray(y1), np.asarray(y2)
    fresh = M1 == -math.inf or M2 == -math.inf
    m1 = 0.0 if M1 == -math.inf else M1
    m2 = 0.0 if M2 == -math.inf else M2
    t1, t2 = y1 - m1, y2 - m2
    if not fresh:
        p1, p2 = 2.0 ** t1, 2.0 ** t2
        s1, s2 = p1.sum(), p2.sum()
        if s1 <= CAP and s2 <= CAP:
            return [m1, l1 + s1, A + (p1 * (t1 - t2)).sum() + (m1 - m2) * s1, m2, l2 + s2]
    h1 = t1.max() if fresh else max(t1.max(), 0.0)
    h2 = t2.max() if fresh else max(t2.max(), 0.0)
    n1, n2 = m1 + h1, m2 + h2
    a1 = 0.0 if fresh else 2.0 ** -h1
    a2 = 0.0 if fresh else 2.0 ** -h2
    u1, u2 = t1 - h1, t2 - h2
    p1, p2 = 2.0 ** u1, 2.0 ** u2
    return [n1, a1 * l1 + p1.sum(), a1 * A + (p1 * (u1 - u2)).sum() + (n1 - n2) * p1.sum(), n2, a2 * l2 + p2.sum()]


def _far_keys(kind, n_k, d, tile, r):
    """Keys whose base-2 logits (against queries near all-ones) move by
    about 80 per tile ("rising") or sit near -270 ("sinking")."""
    k = 1.0 + 0.3 * r.normal(size=(n_k, d))
    unit = LOG2E * math.sqrt(d)
    t = np.arange(n_k) // tile
    scale = (80.0 * t + 1.0) / unit if kind == "rising" else (-270.0 + t) / unit
    return k * scale[:, None]


@pytest.mark.parametrize("kind", ["random", "rising", "sinking"])
@pytest.mark.parametrize("causal", [False, True])
def test_held_offsets_equal_definition(kind, causal):
    """Unmasked tiles with held offsets, masked tiles with the exact update:
    the definition to ~1e-12, and after every tile no term exceeds 2^64 and
    the offsets never pass the largest logit seen."""
    r = np.random.default_rng(11)
    n_q, n_k, d, tile = 12, 96, 8, 8
    q1 = 1.0 + 0.3 * r.normal(size=(n_q, d))
    q2 = 1.0 + 0.3 * r.normal(size=(n_q, d))
    if kind == "random":
        k1, k2 = r.normal(size=(n_k, d)), r.normal(size=(n_k, d))
    else:
        k1, k2 = _far_keys(kind, n_k, d, tile, r), 0.9 * _far_keys(kind, n_k, d, tile, r)
    kl, l1, l2 = oracle.head_forward(q1, k1, q2, k2, causal)
    S1, S2 = oracle.scores(q1, k1, d ** -0.5), oracle.scores(q2, k2, d ** -0.5)
    raised = 0
    for i in range(n_q):
        vis = oracle.valid_mask(np.array([i]), n_q, n_k, causal)[0]
        st, seen1, seen2 = empty_state(), -math.inf, -math.inf
        for t0 in range(0, n_k, tile):
            js = [j for j in range(t0, t0 + tile) if vis[j]]
            y1, y2 = [S1[i, j] * LOG2E for j in js], [S2[i, j] * LOG2E for j in js]
            if not js:
                continue
            if len(js) == tile:
                before = st[0]
                st = tile_update_held(st, y1, y2)
                raised += st[0] != before
            else:
                st = tile_update(st, y1, y2)
            seen1, seen2 = max(seen1, max(y1)), max(seen2, max(y2))
            assert st[0] <= seen1 and st[3] <= seen2
            assert seen1 - st[0] <= 64.0 and seen2 - st[3] <= 64.0
        got = finish(st)
        assert got[0] == pytest.approx(kl[i], rel=1e-11, abs=1e-12)
        assert got[1] == pytest.approx(l1[i], rel=1e-13)
        assert got[2] == pytest.approx(l2[i], rel=1e-13)
    if kind == "rising":
        assert raised > n_q  # the offsets were raised past the first tile
