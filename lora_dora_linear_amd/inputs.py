"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random tensors and stores them in the dtypes the layer takes
(bf16 as raw uint16 bits, float32, int8).  It holds none of the layer's
arithmetic: no products, no norms of the adapted weight, no quantisation.

Recipe (one stream per tensor):
  rng = numpy.random.default_rng(SeedSequence([config_id, tensor_id])) (PCG64),
  draw float32 standard normals, multiply by the std, then round to bf16 by
  round-to-nearest-even on the float32 bits when the dtype is bf16.
  Tensor ids: X 0, W0 1, A 2, B 3, dY 4, magnitude factor 5, bias 6;
  the MLP uses gate (W, A, B) = 10, 11, 12; up = 20, 21, 22; down = 30, 31, 32.

Distributions (the workloads of the layer as the configurations state them):
  X, dY ~ N(0, 1);  W0, A ~ N(0, 1/fan_in);  B ~ N(0, 0.02) read as a
  variance (std = sqrt(0.02));  DoRA magnitude m_n = ||W0_n|| . U(0.9, 1.1) (row
  form) or m_k = ||W0[:,k]|| . U(0.9, 1.1) (column form).
"""

from dataclasses import dataclass, field

import numpy as np

B_STD = float(np.sqrt(0.02))


# ----------------------------------------------------------------------------- dtype helpers
def f32_to_bf16_bits(x):
    """Round float32 to bf16 (nearest, ties to even) and return the uint16 bit patterns."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits):
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def to_f64(arr, dtype):
    """Exact float64 value of a stored tensor ('bf16' bits, 'f32' or 'i8')."""
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    return np.asarray(arr, dtype=np.float64)


# ----------------------------------------------------------------------------- draws
def _rng(config_id, tensor_id):
    return np.random.default_rng(np.random.SeedSequence([int(config_id), int(tensor_id)]))


def normal(config_id, tensor_id, shape, std, dtype):
    x = _rng(config_id, tensor_id).standard_normal(size=shape, dtype=np.float32)
    x = (x * np.float32(std)).astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def uniform(config_id, tensor_id, shape, lo, hi):
    return _rng(config_id, tensor_id).uniform(lo, hi, size=shape).astype(np.float32)


# ----------------------------------------------------------------------------- workloads
@dataclass
class LinearCase:
    """One adapted linear layer: shapes, scale, dtype and the stored tensors."""
    M: int
    N: int
    K: int
    r: int
    s: float
    dtype: str
    t: dict = field(default_factory=dict)

    def f64(self, name):
        return to_f64(self.t[name], self.dtype if name in ("X", "W0", "A", "B", "dY", "bias") else "f32")


def linear_case(config_id, M, N, K, r, s, dtype, with_bias=False, dora=False,
                zero_B=False, zero_W0=False, dora_cols=False):
    """X, W0, A, B, dY (+ bias, + DoRA magnitude m) for a LoRA / DoRA layer."""
    c = LinearCase(M, N, K, r, float(s), dtype)
    c.t["X"] = normal(config_id, 0, (M, K), 1.0, dtype)
    c.t["W0"] = normal(config_id, 1, (N, K), 1.0 / np.sqrt(K), dtype)
    c.t["A"] = normal(config_id, 2, (r, K), 1.0 / np.sqrt(K), dtype)
    c.t["B"] = normal(config_id, 3, (N, r), B_STD, dtype)
    c.t["dY"] = normal(config_id, 4, (M, N), 1.0, dtype)
    if zero_B:
        c.t["B"] = np.zeros_like(c.t["B"])
    if zero_W0:
        c.t["W0"] = np.zeros_like(c.t["W0"])
    if with_bias:
        c.t["bias"] = normal(config_id, 6, (N,), 0.5, dtype)
    if dora:
        w0 = to_f64(c.t["W0"], dtype)
        rownorm = np.sqrt(np.sum(w0 * w0, axis=1))
        c.t["m"] = (rownorm * uniform(config_id, 5, (N,), 0.9, 1.1)).astype(np.float32)
    if dora_cols:
        w0 = to_f64(c.t["W0"], dtype)
        colnorm = np.sqrt(np.sum(w0 * w0, axis=0))
        c.t["m"] = (colnorm * uniform(config_id, 5, (K,), 0.9, 1.1)).astype(np.float32)
    return c


def multi_case(config_id, M, K, n_leaf, r, s_leaf, with_bias=False):
    """Several adapters over one concatenated weight (bf16): X, W0 [sum n_leaf, K],
    A = [A_1; ..; A_L] [L r, K], B = [B_1; ..; B_L] [sum n_leaf, r], dY (+ bias).  The
    leaf widths and scales ride along as c.n_leaf / c.s_leaf."""
    N, L = int(sum(n_leaf)), len(n_leaf)
    c = LinearCase(M, N, K, r, 1.0, "bf16")
    c.n_leaf, c.s_leaf = [int(n) for n in n_leaf], [float(v) for v in s_leaf]
    c.t["X"] = normal(config_id, 0, (M, K), 1.0, "bf16")
    c.t["W0"] = normal(config_id, 1, (N, K), 1.0 / np.sqrt(K), "bf16")
    c.t["A"] = normal(config_id, 2, (L * r, K), 1.0 / np.sqrt(K), "bf16")
    c.t["B"] = normal(config_id, 3, (N, r), B_STD, "bf16")
    c.t["dY"] = normal(config_id, 4, (M, N), 1.0, "bf16")
    if with_bias:
        c.t["bias"] = normal(config_id, 6, (N,), 0.5, "bf16")
    return c


@dataclass
class MlpCase:
    M: int
    K: int
    H: int
    r: int
    s: float
    t: dict = field(default_factory=dict)

    def f64(self, name):
        return bf16_bits_to_f64(self.t[name])

    def proj(self, p):
        """(W, A, B, s) for projection p in 'gate' | 'up' | 'down' as float64 arrays."""
        return (self.f64("W" + p[0]), self.f64("A" + p[0]), self.f64("B" + p[0]), self.s)


def mlp_case(config_id, M, K, H, r, s, zero_B=False):
    """SwiGLU LoRA MLP: gate/up [H,K] with adapters, down [K,H] with an adapter; bf16."""
    c = MlpCase(M, K, H, r, float(s))
    c.t["X"] = normal(config_id, 0, (M, K), 1.0, "bf16")
    c.t["dY"] = normal(config_id, 4, (M, K), 1.0, "bf16")
    for tag, base, n_out, n_in in (("g", 10, H, K), ("u", 20, H, K), ("d", 30, K, H)):
        c.t["W" + tag] = normal(config_id, base, (n_out, n_in), 1.0 / np.sqrt(n_in), "bf16")
        c.t["A" + tag] = normal(config_id, base + 1, (r, n_in), 1.0 / np.sqrt(n_in), "bf16")
        c.t["B" + tag] = normal(config_id, base + 2, (n_out, r), B_STD, "bf16")
        if zero_B:
            c.t["B" + tag] = np.zeros_like(c.t["B" + tag])
    return c


# ----------------------------------------------------------------------------- named configurations
CONFIGS = {
    # id: (name, kind, params)
    1: ("tiny_fp32_lora", "lora", dict(M=64, N=256, K=256, r=8, s=2.0, dtype="f32")),
    2: ("bf16_lora_4096", "lora", dict(M=4096, N=4096, K=4096, r=16, s=0.5, dtype="bf16")),
    3: ("bf16_dora_3072", "dora", dict(M=4096, N=3072, K=3072, r=32, s=1.0, dtype="bf16", eps=1e-12)),
    4: ("bf16_swiglu_mlp", "mlp", dict(M=8192, K=4096, H=14336, r=64, s=0.25)),
    5: ("w8a8_lora_5120", "w8a8", dict(M_sweep=(1024, 2048, 4096, 8192, 16384), N=5120, K=5120, r=32, s=0.5)),
}
