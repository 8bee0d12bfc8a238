"""The library's calls captured in HIP graphs (torch.cuda.CUDAGraph over the launch stream):
each replay must give the bytes the same calls give eagerly.

Every entry point only launches kernels on the given stream (no allocation, memset, copy or
host synchronisation), so a whole layer can be captured once and replayed. The graphs are
replayed several times, in a changing order, with eager runs of the same runner on other
inputs and host synchronisations in between, and every replay's output is compared with
the eager output for its inputs.
"""

import numpy as np
import pytest
import torch

from synth import CONFIGS, dense_inputs, moe_inputs
from tests.gpu_util import assert_bytes_equal, host

pytestmark = pytest.mark.gpu


def _capture(fn):
    """Warm fn up on a side stream, then capture one call of it."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("cfg,T,act", [("moe_tiny", None, "e4m3"), ("moe_prefill", 512, "e4m3"),
                                       ("moe_tiny", None, "mxfp4")])
def test_moe_layer_runner_graph_replays(cfg, T, act):
    import fp8_moe_prefill_amd as f
    c = CONFIGS[cfg]
    dev = torch.device("cuda:0")
    sets = []
    for seed in range(3):
        inp = moe_inputs(c, seed=seed, T=T)
        x = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)
        lg = torch.from_numpy(inp["logits"]).to(dev)
        sets.append((x, lg, f.ExpertBank.from_host(inp, dev, act=act)))
    Tn = sets[0][0].shape[0]
    runner = f.MoELayerRunner(Tn, c.H, c.E, c.k, c.I, dev, act=act)
    eager = []
    for x, lg, bank in sets:
        runner.run(x, lg, bank)
        torch.cuda.synchronize()
        eager.append(host(runner.out).copy())
    graphs = [_capture(lambda x=x, lg=lg, bank=bank: runner.run(x, lg, bank))
              for x, lg, bank in sets]
    for order in ([0, 1, 2], [2, 0, 1], [1, 1, 0, 2]):
        for r in order:
            graphs[r].replay()
            torch.cuda.synchronize()
            assert_bytes_equal(host(runner.out), eager[r], f"replay of input set {r}")
            # eager work on another input set between replays
            o = (r + 1) % 3
            runner.run(*sets[o])
            torch.cuda.synchronize()
            assert_bytes_equal(host(runner.out), eager[o], f"eager run of input set {o}")


def test_w8a8_projection_graph_replays():
    """Per-tensor activation quantisation (amax pass + cast over a partials workspace) and the
    W8A8 GEMM, captured with their buffers allocated once."""
    import fp8_moe_prefill_amd as f
    from fp8_moe_prefill_amd import _lib
    d = dense_inputs(CONFIGS["dense_w8a8"])
    dev = torch.device("cuda:0")
    x = torch.from_numpy(d["x"].view(np.int16)).to(dev).view(torch.bfloat16)[:512].contiguous()
    w = torch.from_numpy(d["w_o"].view(np.int16)).to(dev).view(torch.bfloat16)
    wq, sw = f.quantize_weight(w)
    M, K = x.shape
    N = w.shape[0]
    q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    blk = torch.empty(4, dtype=torch.float32, device=dev)
    nws = _lib.workspace_bytes(_lib.OP_QUANT_ACT, M, K, 0)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    xs = [x, (x.float() * 3.0).to(torch.bfloat16)]
    src = torch.empty_like(x)

    def step():
        _lib.fp8_quant_act(src, 0, q=q, scales=blk, ws=ws)
        _lib.fp8_dense_gemm(q, blk, wq, sw, torch.bfloat16, out=y)

    eager = []
    for xi in xs:
        src.copy_(xi)
        step()
        torch.cuda.synchronize()
        eager.append(host(y).copy())
    g = _capture(step)
    for r in (0, 1, 1, 0):
        src.copy_(xs[r])
        g.replay()
        torch.cuda.synchronize()
        assert_bytes_equal(host(y), eager[r], f"replay {r}")
        step()  # eager in between
        torch.cuda.synchronize()
        assert_bytes_equal(host(y), eager[r], f"eager {r}")
