"""Seeded synthetic workloads (inputs only; none of the method's arithmetic).

The pages measure on real checkpoints (Qwen-Image 2.1 INT8, MiniMax-H3 DiTs)
that are not available; these generators stand in for them with the shapes the
pages quote and the value distributions stated per workload below:

* ``c1``  tiny int8_linear, no input activation: x [64, 256], W [128, 256]
* ``c2``  fused SwiGLU down projection, M=2048, K=3072 -> N=1024
  (sglang PR #44196, "Accuracy Tests": the (2048, 3072->1024) case)
* ``c3``  fused SwiGLU down projection, M=4096, K=12288 -> N=4096
  (same section: the (4096, 12288->4096) case)
* ``c4``  square int8_linear, M=N=K=4096, no input activation
  (comfy-kitchen PR #277, "Summary": the 4096^3 GEMM)
* ``c5``  DiT-style SwiGLU MLP block, M=4096 tokens, hidden 3072,
  intermediate 12288 (sglang PR #44196, "Motivation": packed [gate | up] GEMM
  then the SwiGLU down projection)

Recipe: ``numpy.random.default_rng([seed, tensor_id])`` (PCG64),
``standard_normal`` in float64, cast to float32.  Tensor ids: 0 = x or gate,
1 = up, 2 = W (or W_gate), 3 = W_up, 4 = W_down, 5 = outlier channel set.
Activations: a channel set S of round(K/100) channels (2 for c1) is drawn
without replacement; those columns are multiplied by 20 in float32; the result
is rounded to BF16 (nearest even).  The same S applies to gate and up.
Weights: sigma * N(0, 1) in float64, rounded to float32.
BF16 tensors are returned as uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TID_X, TID_UP, TID_W, TID_WUP, TID_WDOWN, TID_OUTLIERS = 0, 1, 2, 3, 4, 5
_CHUNK = 1 << 24


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "linear" or "mlp"
    m: int
    k: int               # in_features (hidden size for "mlp")
    n: int               # out_features (intermediate size for "mlp")
    act: int             # 0 = none, 1 = swiglu (linear only)
    sigma: float         # weight std (W_gate/W_up for "mlp")
    sigma_down: float = 0.0
    n_outliers: int | None = None
    group: int = 128
    seed: int = 0
    desc: str = ""

    @property
    def outliers(self) -> int:
        return self.n_outliers if self.n_outliers is not None else round(self.k / 100)

    @property
    def int8_ops(self) -> int:
        """INT8 multiply-add work, counted 2 ops per multiply-add."""
        if self.kind == "mlp":
            return 6 * self.m * self.k * self.n
        return 2 * self.m * self.n * self.k


WORKLOADS = {
    "c1": Workload("c1", "linear", 64, 256, 128, 0, 0.02, n_outliers=2,
                   desc="tiny int8_linear 64x256->128, no input act"),
    "c2": Workload("c2", "linear", 2048, 3072, 1024, 1, 0.02,
                   desc="fused SwiGLU down projection M=2048, K=3072->N=1024"),
    "c3": Workload("c3", "linear", 4096, 12288, 4096, 1, 0.01,
                   desc="fused SwiGLU down projection M=4096, K=12288->N=4096"),
    "c4": Workload("c4", "linear", 4096, 4096, 4096, 0, 0.02,
                   desc="square int8_linear M=N=K=4096, no input act"),
    "c5": Workload("c5", "mlp", 4096, 3072, 12288, 1, 0.02, sigma_down=0.01,
                   desc="SwiGLU MLP block M=4096, hidden 3072, intermediate 12288"),
}


def _normal(seed: int, tid: int, shape) -> np.ndarray:
    """float32 array of standard normals, drawn in float64 and rounded."""
    rng = np.random.default_rng([seed, tid])
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        out[lo:hi] = rng.standard_normal(hi - lo, dtype=np.float64)
    return out.reshape(shape)


def _weights(seed: int, tid: int, shape, sigma: float) -> np.ndarray:
    rng = np.random.default_rng([seed, tid])
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        out[lo:hi] = sigma * rng.standard_normal(hi - lo, dtype=np.float64)
    return out.reshape(shape)


def outlier_channels(seed: int, k: int, count: int) -> np.ndarray:
    rng = np.random.default_rng([seed, TID_OUTLIERS])
    return np.sort(rng.choice(k, size=count, replace=False))


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 to BF16 (nearest even) using torch's conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def activation(seed: int, tid: int, m: int, k: int, outliers: np.ndarray) -> np.ndarray:
    x = _normal(seed, tid, (m, k))
    if len(outliers):
        x[:, outliers] *= np.float32(20.0)
    return to_bf16_bits(x)


def linear_inputs(w: Workload, m: int | None = None):
    """Inputs of an int8_linear workload: dict(x=[m, K or 2K] BF16 bits, w=[N, K] f32)."""
    m = w.m if m is None else m
    s = outlier_channels(w.seed, w.k, w.outliers)
    if w.act == 1:
        gate = activation(w.seed, TID_X, m, w.k, s)
        up = activation(w.seed, TID_UP, m, w.k, s)
        x = np.concatenate([gate, up], axis=1)
    else:
        x = activation(w.seed, TID_X, m, w.k, s)
    return dict(x=np.ascontiguousarray(x), w=_weights(w.seed, TID_W, (w.n, w.k), w.sigma))


def mlp_inputs(w: Workload, m: int | None = None):
    """Inputs of the MLP block: x [m, H] BF16 bits, w_gu [2I, H] (gate rows then
    up rows), w_down [H, I], all f32."""
    m = w.m if m is None else m
    s = outlier_channels(w.seed, w.k, w.outliers)
    x = activation(w.seed, TID_X, m, w.k, s)
    w_gate = _weights(w.seed, TID_W, (w.n, w.k), w.sigma)
    w_up = _weights(w.seed, TID_WUP, (w.n, w.k), w.sigma)
    w_down = _weights(w.seed, TID_WDOWN, (w.k, w.n), w.sigma_down)
    return dict(x=x, w_gu=np.concatenate([w_gate, w_up], axis=0), w_down=w_down)


def case(m: int, k: int, n: int, act: int, seed: int, sigma: float = 0.02,
         outlier_frac: float = 0.01, zero_rows=()):
    """An arbitrary-size int8_linear case with the same recipe (test cases)."""
    w = Workload("case", "linear", m, k, n, act, sigma,
                 n_outliers=max(1, round(k * outlier_frac)), seed=seed)
    d = linear_inputs(w)
    for r in zero_rows:
        d["x"][r, :] = 0
    return d
