"""moe_route_permute_noalloc (the routing call that takes no workspace and allocates
nothing) against moe_route_permute with a caller workspace: every output byte-equal, on
consecutive calls that share the library's static per-GPU workspace, the second one
smaller than the first, then a third of another expert count; a small call is also
checked against the oracle's routing and grouping. Sizes past the static workspace are
refused on the host before anything is launched."""

import numpy as np
import pytest
import torch

from oracle.route import group_pairs, topk_route
from synth import CONFIGS, moe_inputs
from synth.inputs import router_logits
from tests.gpu_util import assert_bytes_equal, dev, host

pytestmark = pytest.mark.gpu


def _both(logits, k, xq=None, xs=None, xsum=None):
    import fp8_moe_prefill_amd as f
    lg = dev(logits)
    g = {} if xq is None else dict(xq=dev(xq), xs=dev(xs), xsum=dev(xsum))
    ref = f.moe_route_permute(lg, k, **g)
    torch.cuda.synchronize()
    ref = {n: host(t).copy() for n, t in ref.items()}
    # outputs preallocated and poisoned, so every byte must come from the call
    out = {n: torch.full_like(dev(v), 0x5A if v.dtype == np.uint8 else -7) for n, v in ref.items()}
    got = f.moe_route_permute_noalloc(lg, k, out=out, **g)
    torch.cuda.synchronize()
    assert set(got) == set(ref)
    for n in ref:
        assert got[n] is out[n]
        assert_bytes_equal(host(got[n]), ref[n], n)
    return ref


def test_noalloc_matches_workspace_call_on_consecutive_calls():
    import fp8_moe_prefill_amd as f
    # 1: the 4096-token layer (64 experts, top-8) with the row, scale and code-sum gathers
    c = CONFIGS["moe_prefill"]
    inp = moe_inputs(c)
    xq, xs, xsum = (host(t) for t in f.fp8_quant_act(dev(inp["x"]), 128, with_sums=True))
    _both(inp["logits"], c.k, xq, xs, xsum)
    # 2: a smaller, ragged call right after it (37 tokens: two chunks plus a tail)
    lg = router_logits(7, "noalloc.small", 37, c.E, 0.0)
    r = _both(lg, c.k)
    ids, w = topk_route(lg, c.k)
    off, sorted_, pos = group_pairs(ids, c.E)
    assert_bytes_equal(r["ids"], ids, "ids")
    assert_bytes_equal(r["offsets"], off, "offsets")
    assert_bytes_equal(r["sorted"], sorted_, "sorted")
    assert_bytes_equal(r["pos"], pos, "pos")
    assert np.all(np.abs(r["weights"] - w) <= 1e-5 * w + 1e-7)
    # 3: another expert count and a skewed router (empty experts), 1000 tokens
    s = CONFIGS["moe_skewed"]
    lg = router_logits(s.seed, "noalloc.skewed", 1000, s.E, s.zipf_s)
    r = _both(lg, s.k)
    assert (np.diff(r["offsets"]) == 0).any()


def test_noalloc_refuses_sizes_past_its_static_workspace():
    import fp8_moe_prefill_amd as f
    from fp8_moe_prefill_amd._lib import OP_ROUTE_PERMUTE, Fp8MoeError
    T, E, k = 1 << 17, 256, 8
    assert f.workspace_bytes(OP_ROUTE_PERMUTE, T, E, k) > 4 << 20
    lg = torch.zeros((T, E), dtype=torch.float32, device="cuda:0")
    with pytest.raises(Fp8MoeError, match="workspace"):
        f.moe_route_permute_noalloc(lg, k)
    # the largest token count that fits still runs and matches the workspace call
    T = ((4 << 20) // 4 - E) // E * 16
    assert f.workspace_bytes(OP_ROUTE_PERMUTE, T, E, k) <= 4 << 20
    lg = router_logits(3, "noalloc.max", T, E, 0.0)
    _both(lg, k)
