"""Pins of the oracle's router-live top-k gate (verification rows below the
survival threshold take their anchor row's experts, weighted by their own
logits; every pair is bucketed) against the plain top-k gate, numpy
softmax and brute-force bucketing."""
import numpy as np

import oracle


def verify_rows(streams=4, drafts=5, E=64, seed=0):
    """streams x (1 anchor + drafts) rows: logits N(0,1), survival U(0,1) (1.0 for anchors)."""
    rng = np.random.default_rng(seed)
    T = streams * (drafts + 1)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    surv = rng.random(T).astype(np.float32)
    surv[:: drafts + 1] = 1.0
    anchor = (np.arange(T) // (drafts + 1) * (drafts + 1)).astype(np.int32)
    return logits, surv, anchor


def softmax_f32(v):
    v = v.astype(np.float64)
    e = np.exp(v - v.max())
    return (e / e.sum()).astype(np.float32)


def check_buckets(r, T, k, E):
    ids, offsets, perm, slot_pos = r["ids"], r["offsets"], r["perm"], r["slot_pos"]
    assert offsets[E] == T * k and offsets[0] == 0
    assert np.array_equal(np.sort(perm), np.arange(T * k))
    want = sorted(((ids[t, j], t, j) for t in range(T) for j in range(k)))
    assert [(int(p) // k, int(p) % k) for p in perm] == [(t, j) for _, t, j in want]
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(ids.ravel()[seg] == e)
    assert np.array_equal(slot_pos.ravel()[perm], np.arange(T * k))


def test_without_reuse_it_is_the_plain_gate():
    logits, surv, anchor = verify_rows()
    T, k, E = logits.shape[0], 6, logits.shape[1]
    plain = oracle.route(logits, k)
    for s, a in [(np.ones_like(surv), anchor), (surv, np.arange(T, dtype=np.int32)), (None, anchor)]:
        r = oracle.route_live(logits, k, s, a, reuse_below=0.3)
        for key in ("ids", "w", "offsets", "perm", "slot_pos"):
            assert np.array_equal(r[key], plain[key]), key


def test_reusing_rows_take_the_anchor_experts_with_their_own_weights():
    logits, surv, anchor = verify_rows(seed=1)
    T, k, E = logits.shape[0], 8, logits.shape[1]
    plain = oracle.route(logits, k)
    r = oracle.route_live(logits, k, surv, anchor, reuse_below=0.5)
    reuse = (surv < np.float32(0.5)) & (anchor != np.arange(T))
    assert reuse.sum() >= 4
    for t in range(T):
        src = anchor[t] if reuse[t] else t
        assert np.array_equal(r["ids"][t], plain["ids"][src]), t
        want = softmax_f32(logits[t, r["ids"][t]])
        assert np.all(np.abs(r["w"][t] - want) <= np.spacing(want)), t
        assert abs(float(r["w"][t].astype(np.float64).sum()) - 1.0) < k * 2.0 ** -23
    check_buckets(r, T, k, E)
    # no expert is read that a live row does not read
    live_experts = set(plain["ids"][~reuse].ravel().tolist())
    assert set(r["ids"].ravel().tolist()) == live_experts


def test_anchor_chains_and_bad_anchors():
    logits, surv, _ = verify_rows(streams=1, drafts=7, seed=2)
    T, k = logits.shape[0], 4
    plain = oracle.route(logits, k)
    surv = np.full(T, 0.05, np.float32)
    surv[0] = 1.0
    anchor = np.array([0, 0, 1, 2, -1, T, 6, 3], np.int32)       # 2 -> 1 (itself reusing), bad and self anchors
    r = oracle.route_live(logits, k, surv, anchor, reuse_below=0.1)
    want_src = [0, 0, 1, 2, 4, 5, 6, 3]                          # a reusing anchor still lends its own top-k
    for t in range(T):
        assert np.array_equal(r["ids"][t], plain["ids"][want_src[t]]), t
    check_buckets(r, T, k, logits.shape[1])


def test_threshold_is_strict():
    logits, surv, anchor = verify_rows(streams=1, drafts=3, seed=3)
    surv[:] = np.float32(0.1)
    surv[0] = 1.0
    r = oracle.route_live(logits, 2, surv, anchor, reuse_below=0.1)
    assert np.array_equal(r["ids"], oracle.route(logits, 2)["ids"])
