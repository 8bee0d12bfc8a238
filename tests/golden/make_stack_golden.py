"""Write the expected values of the depth-stack workloads (T=2048, L=8 and L=12) from the
oracle alone: ``python -m tests.golden.make_stack_golden`` (minutes of CPU per stack).

The whole-stack oracle takes minutes, too long to rerun inside a GPU test, and its full
logits (T x V fp32) are too large to store. What is stored, per stack, in
``<name>.npz``:

* ``rows``: 8 token positions spread over the sequence (first and last included), and
  ``row_logits``: the oracle's logits at those rows, as fp16 (relative rounding 2^-11,
  negligible against a cosine gate of 0.999);
* ``argmax``, ``margin``: for every token, the oracle's top logit index and the gap
  between its two largest logits (a token whose gap is below the GPU/oracle difference
  may legitimately change its argmax);
* ``norm``: every token's logit-vector norm;
* ``cos_bf16``: cosine of the oracle's FP8 logits against the oracle's bf16 path (the
  FP8 grouped-expert prefill note, section 1, gates on final-logit cosine), computed here
  so the GPU run need not.

Inputs: ``synth.stack_inputs`` with the preset's seed; nothing here comes from the GPU.
"""

from __future__ import annotations

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle.numeric import cosine  # noqa: E402
from oracle.stack import stack_forward  # noqa: E402
from synth import CONFIGS, stack_inputs  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
N_ROWS = 8


def golden_path(name: str) -> str:
    return os.path.join(HERE, f"{name}.npz")


def sample_rows(T: int) -> np.ndarray:
    return np.unique(np.round(np.linspace(0, T - 1, N_ROWS)).astype(np.int64))


def make(name: str) -> None:
    cfg = CONFIGS[name]
    t0 = time.time()
    inp = stack_inputs(cfg)
    a = stack_forward(inp, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.k, fp8=True)
    print(f"{name}: fp8 oracle {time.time() - t0:.0f} s", flush=True)
    b = stack_forward(inp, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.k, fp8=False)
    print(f"{name}: bf16 path {time.time() - t0:.0f} s", flush=True)
    rows = sample_rows(cfg.T)
    top2 = np.sort(np.partition(a, -2, axis=1)[:, -2:], axis=1)
    np.savez_compressed(
        golden_path(name), rows=rows, row_logits=a[rows].astype(np.float16),
        argmax=np.argmax(a, axis=1).astype(np.int32),
        margin=(top2[:, 1] - top2[:, 0]).astype(np.float32),
        norm=np.linalg.norm(a, axis=1), cos_bf16=np.float64(cosine(a, b)))
    print(f"{name}: cos(fp8, bf16 path) = {cosine(a, b):.6f}", flush=True)


if __name__ == "__main__":
    for n in (sys.argv[1:] or ["stack_L8", "stack_L12"]):
        make(n)
