"""Seeded synthetic KV-cache generators and the workload table.

This module only makes inputs. It holds none of the codec's arithmetic (no
centering, projection, quantization or packing), so that the CPU oracle and the
HIP library, which must not share code, can both be fed the same tensors.

The pages evaluate KV transform coding on real model caches (Llama 3.1/3.3,
Mistral NeMo, Qwen 2.5; "KV Cache Transform Coding for Compact Storage in LLM
Inference", section 4). No weights or datasets are available here, so these
generators stand in for those caches at the same shapes:

* family "A" (the tiny workload): X = (Z * sigma) B^T + eps, Z ~ N(0,1) of rank
  16, sigma_k = 0.8^k, B ~ N(0,1) fixed per layer, eps ~ N(0, 0.01^2); fp32.
* family "B" (model-shaped workloads): one latent z in R^r per token shared by
  all heads, a fixed orthonormal U (head_dim x r) and a Haar-random rotation R_h
  per head, x_h = R_h U (sigma * z) with sigma_k = k^-alpha; a fixed per-feature
  mean offset; for keys, 4 distinct channels per head scaled by 10; rounded to
  bfloat16 (round to nearest even).  The shared latent is what makes the heads
  alike after an orthogonal transform, the property the pages build on
  (same page, section 2A).

Seeds: numpy PCG64 from SeedSequence([251101815, cfg, layer, kind, role, req]),
role 0 = per-tensor structure, 1 = calibration tokens, 2 = evaluation tokens.
"""
from __future__ import annotations

import dataclasses
import numpy as np

SEED_ROOT = 251101815
K, V = 0, 1
ROLE_STRUCT, ROLE_CALIB, ROLE_EVAL = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    n_layers: int
    kinds: tuple
    kv_heads: int
    head_dim: int
    n_tokens: int          # tokens per request
    n_requests: int
    calib_tokens: int
    dtype: str             # "f32" | "bf16"
    sink: int
    window: int
    group: int
    bits_per_value: float
    family: str            # "A" | "B"
    rank: int
    alpha: float = 1.2
    decay: float = 0.8
    noise: float = 0.01
    paged: bool = False
    block_size: int = 16
    mean_scale: float = 0.5    # family B: std of the per-feature mean offset

    @property
    def features(self) -> int:
        return self.kv_heads * self.head_dim

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def n_tensors(self) -> int:
        return self.n_layers * len(self.kinds) * self.n_requests

    @property
    def kv_bytes(self) -> int:
        """Uncompressed bytes of the whole cache."""
        return self.n_tensors * self.n_tokens * self.features * self.elem_bytes


# The five workloads of the pages, then two small shapes whose feature
# count is an odd multiple of 64 (parity cases only).  bits_per_value =
# 16 / ratio for 16-bit KV.
WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, (K,), 2, 64, 512, 1, 2048, "f32", 4, 64, 16,
                     2.0, "A", 16),
    "llama31_8b": Workload("llama31_8b", 1, 32, (K, V), 8, 128, 8192, 1, 16384,
                           "bf16", 4, 128, 16, 1.0, "B", 96),
    "nemo12b": Workload("nemo12b", 2, 40, (K, V), 8, 128, 32768, 1, 16384,
                        "bf16", 4, 128, 32, 0.5, "B", 128),
    "llama33_70b_16x": Workload("llama33_70b_16x", 3, 80, (K, V), 8, 128, 16384,
                                1, 16384, "bf16", 4, 128, 16, 1.0, "B", 96),
    "llama33_70b_64x": Workload("llama33_70b_64x", 3, 80, (K, V), 8, 128, 16384,
                                1, 16384, "bf16", 4, 128, 16, 0.25, "B", 96),
    "qwen25_7b_paged": Workload("qwen25_7b_paged", 4, 28, (K, V), 4, 128, 8192,
                                16, 16384, "bf16", 4, 128, 16, 0.8, "B", 96,
                                paged=True),
    "odd3_bf16": Workload("odd3_bf16", 5, 1, (K, V), 3, 64, 1100, 1, 2048,
                          "bf16", 4, 64, 16, 2.0, "B", 48),
    "odd1_f32": Workload("odd1_f32", 6, 1, (K,), 1, 64, 2100, 1, 2048, "f32", 4,
                         32, 16, 3.0, "A", 16),
    # Llama-3.1-8B-shaped layer whose features carry large mean offsets
    # (std 50 against a unit spread; x10 on the key outlier channels): the
    # centring must not lose precision when |mean| >> spread.
    "offsets_bf16": Workload("offsets_bf16", 7, 1, (K, V), 8, 128, 4096, 1, 4096,
                             "bf16", 4, 128, 16, 1.0, "B", 96, mean_scale=50.0),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _rng(cfg: int, layer: int, kind: int, role: int, req: int = 0):
    ss = np.random.SeedSequence([SEED_ROOT, cfg, layer, kind, role, req])
    return np.random.Generator(np.random.PCG64(ss))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest-even bfloat16 value, returned as fp32 (input storage)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16).astype(np.uint32) << 16
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 storage of fp32 values that are already bfloat16-representable."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(b & 0xFFFF):
        raise ValueError("values are not bfloat16-representable")
    return (b >> 16).astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _haar(rng, n):
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))


@dataclasses.dataclass
class _Structure:
    kind: str
    basis: np.ndarray          # A: B [F, rank]; B: per-head (R_h U) stacked [F, rank]
    sigma: np.ndarray
    mean: np.ndarray           # [F]
    chan_scale: np.ndarray     # [F]


def structure(w: Workload, layer: int, kind: int) -> _Structure:
    """The fixed per-(layer, kind) generator structure (role 0 stream)."""
    rng = _rng(w.index, layer, kind, ROLE_STRUCT)
    F = w.features
    if w.family == "A":
        B = rng.standard_normal((F, w.rank))
        sigma = w.decay ** np.arange(w.rank, dtype=np.float64)
        return _Structure("A", B, sigma, np.zeros(F), np.ones(F))
    d, r = w.head_dim, w.rank
    U, _ = np.linalg.qr(rng.standard_normal((d, r)))
    blocks = [_haar(rng, d) @ U for _ in range(w.kv_heads)]
    M = np.concatenate(blocks, axis=0)                      # [F, r]
    sigma = np.arange(1, r + 1, dtype=np.float64) ** (-w.alpha)
    amp = np.sqrt(d / np.sum(sigma ** 2))                   # unit per-channel std
    mean = w.mean_scale * rng.standard_normal(F)
    scale = np.ones(F)
    if kind == K:
        for h in range(w.kv_heads):
            ch = rng.choice(d, size=4, replace=False)
            scale[h * d + ch] = 10.0
    return _Structure("B", M, sigma * amp, mean, scale)


def gen_kv(w: Workload, layer: int, kind: int, role: int, n_tokens: int,
           req: int = 0) -> np.ndarray:
    """Seeded synthetic KV for one (layer, kind): fp32 array [n_tokens, F].

    For bf16 workloads every value is bfloat16-representable (use bf16_bits to
    get the uint16 storage)."""
    st = structure(w, layer, kind)
    rng = _rng(w.index, layer, kind, role, req)
    z = rng.standard_normal((n_tokens, st.basis.shape[1]))
    x = (z * st.sigma) @ st.basis.T
    if st.kind == "A":
        x = x + w.noise * rng.standard_normal(x.shape)
        return x.astype(np.float32)
    x = (x + st.mean) * st.chan_scale
    return round_to_bf16(x.astype(np.float32))


def storage(w: Workload, x: np.ndarray) -> np.ndarray:
    """The raw element storage of a generated tensor (uint16 for bf16, f32)."""
    return bf16_bits(x) if w.dtype == "bf16" else np.ascontiguousarray(x, np.float32)
