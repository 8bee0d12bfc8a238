"""Pins of the oracle's depth stack.

* RMSNorm closed form: a constant row c normalises to sign(c) / sqrt(1 + eps / c^2);
* attention: T = 1 returns v; a pure-Python loop over (query, key) on a tiny case; with
  identical keys every query averages the causal prefix of v;
* the FP8 stack vs the bf16 path on a tiny random stack: logit cosine well above 0.99
  (the FP8 grouped-expert prefill note, section 1, gates on final-logit cosine).
"""

import math

import numpy as np

from oracle.numeric import cosine
from oracle.stack import EPS, causal_gqa_attention, rmsnorm, stack_forward
from synth import StackConfig, stack_inputs

TINY = StackConfig("stack_tiny", L=2, T=24, H=256, n_q=4, n_kv=2, head_dim=64, E=4, k=2,
                   I=256, V=300)


def test_rmsnorm_constant_rows():
    for c in [3.0, -0.5, 1e-2]:
        r = rmsnorm(np.full((1, 64), c))
        assert np.allclose(r, math.copysign(1, c) / math.sqrt(1 + EPS / c ** 2), rtol=1e-14)


def test_attention_single_token_and_loops():
    rng = np.random.default_rng(0)
    n_q, n_kv, d = 4, 2, 8
    q, k, v = (rng.standard_normal((1, h * d)) for h in (n_q, n_kv, n_kv))
    out = causal_gqa_attention(q, k, v, n_q, n_kv, d)
    for h in range(n_q):
        assert np.allclose(out[0, h * d:(h + 1) * d], v[0, (h // 2) * d:(h // 2 + 1) * d])
    T = 5
    q, k, v = (rng.standard_normal((T, h * d)) for h in (n_q, n_kv, n_kv))
    out = causal_gqa_attention(q, k, v, n_q, n_kv, d)
    for t in range(T):
        for h in range(n_q):
            kv = h // (n_q // n_kv)
            sc = [sum(q[t, h * d + i] * k[s, kv * d + i] for i in range(d)) / math.sqrt(d)
                  for s in range(t + 1)]
            m = max(sc)
            p = [math.exp(x - m) for x in sc]
            z = sum(p)
            for i in range(d):
                ref = sum(p[s] * v[s, kv * d + i] for s in range(t + 1)) / z
                assert abs(out[t, h * d + i] - ref) < 1e-12
    kk = np.tile(rng.standard_normal((1, n_kv * d)), (T, 1))
    out = causal_gqa_attention(q, kk, v, n_q, n_kv, d)
    cm = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None]
    assert np.allclose(out[:, :d], cm[:, :d])


def test_fp8_stack_vs_bf16_path():
    inp = stack_inputs(TINY)
    a = stack_forward(inp, TINY.n_q, TINY.n_kv, TINY.head_dim, TINY.k, fp8=True)
    b = stack_forward(inp, TINY.n_q, TINY.n_kv, TINY.head_dim, TINY.k, fp8=False)
    assert a.shape == (TINY.T, TINY.V)
    c = cosine(a, b)
    assert 0.99 < c < 1.0, c
