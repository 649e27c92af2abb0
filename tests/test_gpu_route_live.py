"""GPU parity of the router-live top-k gate (moe_route_live) against the
oracle: bit-exact ids, offsets, perm and slot_pos, weights within 2^-22, on
verification-shaped rows (streams of one anchor and five drafts, rows below
the threshold taking their anchor's experts) for every route kernel (one
row, one workgroup, chunked), edge cases, and the routed-expert FFN run on
such a routing."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp8xfp4_amd import mxmoe, synth
from block_scaled_fp8xfp4_amd.layer import Route
from gpu_common import dev, host, moe_workload, say
from gpu_common import ffn_parity

pytestmark = pytest.mark.gpu


def anchors_of(T, group):
    return (np.arange(T) // group * group).astype(np.int32)


def check_route_live(logits, k, survival, anchor, thr):
    T, E = logits.shape
    r = oracle.route_live(logits, k, survival, anchor, thr)
    g = Route(T, E, k)
    g(dev(logits), None if survival is None else dev(survival), thr, anchor=dev(anchor))
    assert mxmoe.last_variant().startswith("route_live:")
    for key in ("ids", "offsets", "perm", "slot_pos"):
        assert np.array_equal(host(getattr(g, key)), r[key]), key
    w = host(g.w)
    assert np.all(np.abs(w - r["w"]) <= 2.0 ** -22 * np.abs(r["w"]))
    return g, r


@pytest.mark.parametrize("thr", [0.1, 0.5])
def test_verify_workload(thr):
    inp = synth.moe_inputs("verify")
    c = inp.cfg
    anchor = anchors_of(c.T, c.drafts + 1)
    g, r = check_route_live(inp.logits, c.k, inp.survival, anchor, thr)
    reuse = (inp.survival < np.float32(thr)) & (anchor != np.arange(c.T))
    say(f"route_live verify thr={thr}: {int(reuse.sum())} rows reuse their anchor's experts")
    assert reuse.any()
    # no weight is read that a row keeping its own experts does not read
    offs = host(g.offsets)
    touched = set(np.nonzero(np.diff(offs))[0].tolist())
    own = oracle.route(inp.logits, c.k)["ids"]
    assert touched == set(own[~reuse].ravel().tolist())


def test_every_route_kernel():
    rng = np.random.default_rng(7)
    # one row: its anchor is itself
    check_route_live(rng.standard_normal((1, 256)).astype(np.float32), 8, np.array([0.01], np.float32),
                     np.zeros(1, np.int32), 0.1)
    # chunked path: streams of 6 rows cross the 256-row chunk boundaries
    T = 600
    surv = rng.random(T).astype(np.float32)
    surv[::6] = 1.0
    check_route_live(rng.standard_normal((T, 256)).astype(np.float32), 8, surv, anchors_of(T, 6), 0.3)
    # one workgroup, exact ties, -0, bad anchors and chains
    ties = np.round(rng.standard_normal((40, 64)) * 2).astype(np.float32)
    ties[3, ::2] = -0.0
    surv = np.full(40, 0.05, np.float32)
    surv[::8] = 1.0
    anchor = anchors_of(40, 8)
    anchor[[1, 2, 3, 4]] = [-5, 40, 3, 1]                       # out of range, self, a reusing anchor
    check_route_live(ties, 4, surv, anchor, 0.1)
    assert mxmoe.last_variant() == "route_live:topk_wave+bucket_single_workgroup"
    # the same rows, few enough to be ranked inside the bucketing workgroup
    check_route_live(ties[:24], 4, surv[:24], np.minimum(anchor[:24], 23), 0.1)
    assert mxmoe.last_variant() == "route_live:fused_single_workgroup"
    # no survival: every row keeps its own experts (the plain gate with every row live)
    lg = rng.standard_normal((20, 32)).astype(np.float32)
    g, r = check_route_live(lg, 2, None, anchors_of(20, 5), 0.1)
    assert np.array_equal(r["ids"], oracle.route(lg, 2)["ids"])


def test_empty_batch():
    for live in (False, True):
        g = Route(0, 16, 2)
        g.offsets.fill_(7)
        g(torch.empty((0, 16), device="cuda"), None, 0.1, anchor=torch.empty(0, dtype=torch.int32, device="cuda")
          if live else None)
        assert mxmoe.last_variant() == "route:empty"
        assert not host(g.offsets).any()


def test_ffn_on_router_live_routing():
    """The verification layer routed in router-live mode: every row gets an
    output (reusing rows through their anchor's experts), staged and
    end-to-end parity with the oracle."""
    inp, _, layer = moe_workload("verify")
    c = inp.cfg
    anchor = anchors_of(c.T, c.drafts + 1)
    # at the layer's own skip threshold every row that keeps its experts has
    # weights in the workload (only experts of such rows are generated)
    g, r = check_route_live(inp.logits, c.k, inp.survival, anchor, 0.2)
    yg = ffn_parity(inp, r, layer, what="verify router-live", route=g)
    assert np.all(np.any(yg != 0, axis=1))                      # no row is skipped
