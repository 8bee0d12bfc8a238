"""moe_route_permute on the GPU vs the oracle: ids, offsets, sorted, pos and the gathered
rows bit-exact; weights within 1e-5 relative."""

import numpy as np
import pytest
import torch

from oracle.route import group_pairs, permute_rows, topk_route
from synth import CONFIGS, moe_inputs
from tests.gpu_util import assert_bytes_equal, dev, host

pytestmark = pytest.mark.gpu


def _gpu_route(logits, k, xq=None, xs=None):
    import fp8_moe_prefill_amd as f
    r = f.moe_route_permute(dev(logits), k, xq=None if xq is None else dev(xq),
                            xs=None if xs is None else dev(xs))
    torch.cuda.synchronize()
    return {n: host(t) for n, t in r.items()}


def _check(logits, k, gpu):
    E = logits.shape[1]
    ids, w = topk_route(logits, k)
    off, sorted_, pos = group_pairs(ids, E)
    assert_bytes_equal(gpu["ids"], ids, "ids")
    assert_bytes_equal(gpu["offsets"], off, "offsets")
    assert_bytes_equal(gpu["sorted"], sorted_, "sorted")
    assert_bytes_equal(gpu["pos"], pos, "pos")
    err = np.abs(gpu["weights"].astype(np.float64) - w)
    assert np.all(err <= 1e-5 * w + 1e-7), err.max()
    return ids, off, sorted_, pos


@pytest.mark.parametrize("cfg", ["moe_tiny", "moe_prefill", "moe_skewed"])
def test_config_routing(cfg):
    c = CONFIGS[cfg]
    from synth.inputs import router_logits
    logits = router_logits(c.seed, f"{c.name}.logits", c.T, c.E, c.zipf_s)
    gpu = _gpu_route(logits, c.k)
    _, off, _, _ = _check(logits, c.k, gpu)
    if cfg == "moe_skewed":
        assert (np.diff(off) == 0).sum() >= 1  # some experts receive no rows


def test_ties_and_degenerate_shapes():
    rng = np.random.default_rng(0)
    lg = np.round(rng.standard_normal((37, 16))).astype(np.float32)  # many exact ties
    lg[3] = 0.0  # all equal
    lg[4, :] = -0.0
    lg[4, 7] = 0.0
    _check(lg, 4, _gpu_route(lg, 4))
    _check(lg, 16, _gpu_route(lg, 16))  # k = E
    one = rng.standard_normal((5, 1)).astype(np.float32)
    _check(one, 1, _gpu_route(one, 1))  # E = 1
    t1 = rng.standard_normal((1, 64)).astype(np.float32)
    _check(t1, 8, _gpu_route(t1, 8))  # T = 1


@pytest.mark.parametrize("E,k", [(1024, 8), (200, 32), (65, 3)])
def test_wide_expert_counts(E, k):
    rng = np.random.default_rng(E)
    lg = rng.standard_normal((50, E)).astype(np.float32)
    _check(lg, k, _gpu_route(lg, k))


def test_one_hot_expert_and_empty_experts():
    lg = np.full((300, 32), -5.0, np.float32)
    lg[:, 3] = 5.0  # every token's first choice
    lg[:, 9] = 4.0
    gpu = _gpu_route(lg, 2)
    _, off, _, _ = _check(lg, 2, gpu)
    counts = np.diff(off)
    assert counts[3] == 300 and counts[9] == 300 and counts.sum() == 600


def test_gather_rows_and_scales():
    c = CONFIGS["moe_tiny"]
    rng = np.random.default_rng(1)
    xq = rng.integers(0, 256, size=(c.T, c.H), dtype=np.uint8)
    xs = rng.uniform(0.001, 1, size=(c.T, c.H // 128)).astype(np.float32)
    logits = moe_inputs(c)["logits"]
    gpu = _gpu_route(logits, c.k, xq, xs)
    _, _, sorted_, _ = _check(logits, c.k, gpu)
    assert_bytes_equal(gpu["xq_perm"], permute_rows(xq, sorted_, c.k), "gathered rows")
    assert_bytes_equal(gpu["xs_perm"].view(np.uint32),
                       np.ascontiguousarray(permute_rows(xs, sorted_, c.k).T).view(np.uint32),
                       "gathered scales")


def test_repeat_runs_identical():
    c = CONFIGS["moe_prefill"]
    logits = moe_inputs(c)["logits"]
    a = _gpu_route(logits, c.k)
    b = _gpu_route(logits, c.k)
    for n in a:
        assert np.array_equal(a[n].view(np.uint8), b[n].view(np.uint8)), n


def test_code_sum_gather():
    """xsum rides the scale gather: xsum_perm[g, r] = xsum[sorted[r] // k, g], bit-exact, with
    the scales' gather unchanged beside it."""
    import fp8_moe_prefill_amd as f
    c = CONFIGS["moe_tiny"]
    from synth.inputs import router_logits
    logits = router_logits(c.seed, f"{c.name}.logits", c.T, c.E, c.zipf_s)
    rng = np.random.default_rng(3)
    G = 4
    xs = rng.uniform(0.01, 1, (c.T, G)).astype(np.float32)
    xsum = rng.standard_normal((c.T, G)).astype(np.float32) * 100
    r = f.moe_route_permute(dev(logits), c.k, xs=dev(xs), xsum=dev(xsum))
    torch.cuda.synchronize()
    ids, _ = topk_route(logits, c.k)
    _, sorted_, _ = group_pairs(ids, c.E)
    assert_bytes_equal(host(r["xs_perm"]), np.ascontiguousarray(permute_rows(xs, sorted_, c.k).T),
                       "xs_perm")
    assert_bytes_equal(host(r["xsum_perm"]),
                       np.ascontiguousarray(permute_rows(xsum, sorted_, c.k).T), "xsum_perm")


@pytest.mark.parametrize("T,H,E,k,with_sums", [(4096, 2048, 64, 8, True), (77, 256, 64, 8, True),
                                               (1, 128, 8, 2, True), (300, 384, 128, 8, False),
                                               (130, 512, 1024, 32, True), (2000, 1024, 256, 4,
                                                                            True)])
def test_quant_route_equals_the_two_calls(T, H, E, k, with_sums):
    """fp8moe_quant_route (the group quantiser and the top-k in one launch) writes the
    same bytes as fp8_quant_act(group 128) followed by moe_route_permute, for every
    output; the routing is also checked against the oracle. Expert counts 64, 128-256 and
    1024 take the three top-k kernels; ragged T leaves a partial chunk."""
    import fp8_moe_prefill_amd as f
    from synth import bf16_bits_from_f32
    rng = np.random.default_rng(T + 7 * H + E)
    x = bf16_bits_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    xd, ld = dev(x), dev(logits)
    q, s, sums, r = f.quant_route(xd, ld, k, with_sums=with_sums)
    ref = f.fp8_quant_act(xd, f.GROUP, with_sums=with_sums)
    rr = f.moe_route_permute(ld, k)
    torch.cuda.synchronize()
    assert_bytes_equal(host(q), host(ref[0]), "codes")
    assert_bytes_equal(host(s), host(ref[1]), "scales")
    if with_sums:
        assert_bytes_equal(host(sums), host(ref[2]), "code sums")
    else:
        assert sums is None
    for name in ("ids", "weights", "offsets", "sorted", "pos"):
        assert_bytes_equal(host(r[name]), host(rr[name]), name)
    _check(logits, k, {n: host(t) for n, t in r.items()})


@pytest.mark.parametrize("T,E,k", [
    (16384, 64, 8),   # C * E = 1024 * 64 = 65536: the largest table scanned inside the scatter
    (16400, 64, 8),   # 1025 chunks: one past it, the separate chunk scan
    (4000, 256, 4),   # E = 256, one thread per expert in the scatter's table sums
    (1000, 257, 4),   # E = 257: past the scatter's scan, the separate chunk scan
    (333, 3, 2),      # E = 3: 85 threads per expert over interleaved chunks, one idle
])
def test_scan_inside_scatter_and_separate_scan(T, E, k):
    """Both ways of forming the per-expert chunk bases (the scan inside the scatter for small
    count tables, the separate scan kernel otherwise) against the oracle, bit for bit, at
    shapes on both sides of the limit and with ties in the logits."""
    rng = np.random.default_rng(T + E)
    lg = np.round(rng.standard_normal((T, E)) * 4).astype(np.float32) / 4  # many exact ties
    _check(lg, k, _gpu_route(lg, k))


@pytest.mark.parametrize("T", [1, 7, 16, 17])
@pytest.mark.parametrize("E,k", [(1, 1), (3, 2), (64, 8), (257, 32), (1024, 32), (1024, 1)])
def test_one_chunk_grouping_in_the_topk_launch(T, E, k):
    """A batch of at most 16 tokens (one chunk) is grouped by the top-k workgroup itself (its
    histogram scanned for the offsets, the pairs ranked in LDS); 17 tokens take the separate
    launches. Both against the oracle, bit for bit, with ties in the logits, through
    moe_route_permute (with the row and scale gather) and through the fused quantiser +
    routing call."""
    import fp8_moe_prefill_amd as f
    from synth import bf16_bits_from_f32
    rng = np.random.default_rng(1000 * T + E + k)
    lg = np.round(rng.standard_normal((T, E)) * 2).astype(np.float32) / 2  # many exact ties
    H = 256
    xq = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
    xs = rng.uniform(0.001, 1, size=(T, H // 128)).astype(np.float32)
    gpu = _gpu_route(lg, k, xq, xs)
    _, _, sorted_, _ = _check(lg, k, gpu)
    assert_bytes_equal(gpu["xq_perm"], permute_rows(xq, sorted_, k), "gathered rows")
    assert_bytes_equal(gpu["xs_perm"].view(np.uint32),
                       np.ascontiguousarray(permute_rows(xs, sorted_, k).T).view(np.uint32),
                       "gathered scales")
    x = bf16_bits_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    q, s, _, r = f.quant_route(dev(x), dev(lg), k)
    torch.cuda.synchronize()
    _check(lg, k, {n: host(t) for n, t in r.items()})
