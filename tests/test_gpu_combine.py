"""moe_unpermute_combine on the GPU vs the oracle (identical inputs): fp32 output within
1e-6 relative of sum_j |w_j y_j|; bf16 output additionally within half a bf16 ulp."""

import numpy as np
import pytest
import torch

from oracle.moe import combine
from oracle.tol import half_ulp_bf16
from synth import bf16_bits_from_f32
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,k,H,ydt", [(64, 2, 256, "bf16"), (100, 8, 2048, "bf16"),
                                       (7, 1, 8, "f32"), (33, 32, 136, "f32"),
                                       (29, 11, 64, "bf16"), (5, 17, 24, "f32")])
def test_combine(T, k, H, ydt):
    import fp8_moe_prefill_amd as f
    rng = np.random.default_rng(T * k + H)
    R = T * k
    y32 = (rng.standard_normal((R, H)) * 3).astype(np.float32)
    if ydt == "bf16":
        ybits = bf16_bits_from_f32(y32)
        yv = (ybits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        yd = dev(ybits)
    else:
        yv = y32.astype(np.float64)
        yd = dev(y32)
    pos = rng.permutation(R).astype(np.int32)
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    for odt in (torch.float32, torch.bfloat16):
        out = f.moe_unpermute_combine(yd, dev(pos), dev(w), odt)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        ref = combine(yv, pos, w.astype(np.float64))
        mag = np.zeros((T, H))
        p2 = pos.reshape(T, k)
        for j in range(k):
            mag += np.abs(w[:, j:j + 1].astype(np.float64) * yv[p2[:, j]])
        tol = 1e-6 * mag + 1e-30
        if odt == torch.bfloat16:
            tol = tol + half_ulp_bf16(ref)
        assert np.all(np.abs(got - ref) <= tol), np.abs(got - ref).max()
