"""Seeded synthetic inputs for the quantized INT8 linear layer.

This module only draws random numbers and casts them; it holds none of the
layer's arithmetic.  Both the CPU oracle (in the tests) and the HIP library
consume the arrays it returns.

The pages measure on real models (a 7B model, a 70B FFN, a 530B model); no
weights or datasets are used here.  Instead each workload draws Gaussian
activations and weights of the stated layer shape, with a few seeded
"outlier" input channels scaled up, which is the activation structure the pages
describe (a handful of channels tens of times larger than the rest).

Draw order per workload (numpy default_rng(seed)):
  1. outlier channel indices: sorted(rng.choice(K, n, replace=False)),
     n = round(fraction * K)
  2. per-channel factors or per-entry magnitudes
  3. X = standard_normal((M, K), float32)
  4. W = standard_normal((N, K), float32) * sigma   (one matrix after another)
  5. the calibration batch, where the workload has one
then the cast to the stated dtype (numpy astype: round to nearest even).
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np


@dataclass
class Workload:
    name: str
    M: int
    K: int
    alpha: Optional[float]                # None: no smoothing (LLM.int8())
    gran: int                             # 0 per-channel weight scale, 1 per-tensor
    out_dtype: type                       # np.float16 or np.float32
    X: np.ndarray
    weights: Dict[str, np.ndarray]        # name -> [N, K]
    outlier_idx: np.ndarray
    X_cal: Optional[np.ndarray] = None    # calibration batch (else X itself)
    threshold: Optional[float] = None     # LLM.int8() outlier threshold
    decode_rows: List[int] = field(default_factory=list)

    @property
    def calib(self):
        return self.X if self.X_cal is None else self.X_cal


def _pick(rng, K, n):
    return np.sort(rng.choice(K, n, replace=False))


def single_w8a8(seed: int = 0) -> Workload:
    """16 tokens x 512, fp32, four fixed outlier channels x50; W 512x512 N(0,0.02)."""
    rng = np.random.default_rng(seed)
    M, K, N = 16, 512, 512
    idx = np.array([37, 128, 300, 451], dtype=np.int64)
    X = rng.standard_normal((M, K), dtype=np.float32)
    X[:, idx] *= np.float32(50.0)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    return Workload("single_w8a8_16x512x512_f32", M, K, 0.5, 0, np.float32, X, {"w": W}, idx)


def prefill_7b(seed: int = 0, which=("qkv", "up")) -> Workload:
    """2048 tokens x 4096, fp16, 0.5% channels x U(20,60); fused QKV 12288x4096
    and FFN-up 11008x4096, N(0,0.02)."""
    rng = np.random.default_rng(seed)
    M, K = 2048, 4096
    n = round(0.005 * K)
    idx = _pick(rng, K, n)
    fac = rng.uniform(20.0, 60.0, n).astype(np.float32)
    X = rng.standard_normal((M, K), dtype=np.float32)
    X[:, idx] *= fac
    weights = {}
    for name, N in (("qkv", 12288), ("up", 11008)):
        W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
        if name in which:
            weights[name] = W.astype(np.float16)
        del W
    return Workload("prefill_7b_2048x4096_qkv12288_up11008_f16", M, K, 0.5, 0, np.float16,
                    X.astype(np.float16), weights, idx)


def decode_70b(seed: int = 0, n_rows: int = 28672) -> Workload:
    """Decode: X [16 x 8192] fp16 (M=1,4,16 use its first rows), 0.3% channels x50,
    FFN-up W [28672 x 8192] N(0,0.02); a 512-token calibration batch with the
    same outlier channels supplies act_max.  n_rows < 28672 gives a smaller
    slice of the same distribution for quick tests."""
    rng = np.random.default_rng(seed)
    M, K, N = 16, 8192, n_rows
    n = round(0.003 * K)
    idx = _pick(rng, K, n)
    X = rng.standard_normal((M, K), dtype=np.float32)
    X[:, idx] *= np.float32(50.0)
    W = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)).astype(np.float16)
    Xc = rng.standard_normal((512, K), dtype=np.float32)
    Xc[:, idx] *= np.float32(50.0)
    return Workload("decode_70b_ffn_up_Mx8192x28672_f16", M, K, 0.5, 0, np.float16,
                    X.astype(np.float16), {"w": W}, idx, X_cal=Xc.astype(np.float16),
                    decode_rows=[1, 4, 16])


def llm_int8_4096(seed: int = 0) -> Workload:
    """X [4096 x 8192] fp16 N(0,1) with 0.1% of columns whose every entry is
    +-U(6,100) (random sign); W16 [8192 x 8192] N(0,0.02); threshold 6.0."""
    rng = np.random.default_rng(seed)
    M, K, N = 4096, 8192, 8192
    n = round(0.001 * K)
    idx = _pick(rng, K, n)
    mag = rng.uniform(6.0, 100.0, (M, n)).astype(np.float32)
    sign = rng.choice(np.array([-1.0, 1.0], np.float32), (M, n))
    X = rng.standard_normal((M, K), dtype=np.float32)
    X[:, idx] = sign * mag
    W = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)).astype(np.float16)
    return Workload("llm_int8_4096x8192x8192_thr6_f16", M, K, None, 0, np.float16,
                    X.astype(np.float16), {"w": W}, idx, threshold=6.0)


def slice_530b(seed: int = 0) -> Workload:
    """X [4096 x 20480] fp16, 1% of channels replaced by Student-t (nu=2) clipped
    to +-200; W [10240 x 20480] N(0,0.01); alpha 0.7, per-tensor weight scale."""
    rng = np.random.default_rng(seed)
    M, K, N = 4096, 20480, 10240
    n = round(0.01 * K)
    idx = _pick(rng, K, n)
    t = np.clip(rng.standard_t(2.0, (M, n)), -200.0, 200.0).astype(np.float32)
    X = rng.standard_normal((M, K), dtype=np.float32)
    X[:, idx] = t
    X16 = X.astype(np.float16)
    del X
    W = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.01)).astype(np.float16)
    return Workload("slice_530b_ffn_up_4096x20480x10240_f16", M, K, 0.7, 1, np.float16,
                    X16, {"w": W}, idx)


def ffn_down_7b_post_activation(seed: int = 0, M: int = 2048) -> Workload:
    """The 7B FFN-down projection, whose input is the output of the FFN's activation
    function and so is not centred on zero (the case zero-point activations are for):
    X [M x 11008] = h * sigmoid(h) for h ~ N(0, 1) times a per-row factor U(0.5, 3)
    (the SiLU activation; a long positive tail, negatives only down to about -0.28
    times the factor); W_down [4096 x 11008] N(0, 0.02).  Draw order: the per-row
    factors, h, then W; fp16 casts at the end.  No smoothing."""
    rng = np.random.default_rng(seed)
    K, N = 11008, 4096
    fac = rng.uniform(0.5, 3.0, (M, 1)).astype(np.float32)
    h = rng.standard_normal((M, K), dtype=np.float32) * fac
    X = h / (np.float32(1.0) + np.exp(-h))
    del h
    W = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)).astype(np.float16)
    return Workload(f"ffn_down_7b_silu_{M}x11008x4096_f16", M, K, None, 0, np.float16, X.astype(np.float16),
                    {"down": W}, np.zeros(0, np.int64))


def random_layer(seed: int, M: int, K: int, N: int, dtype=np.float16, n_outliers: int = 0,
                 factor: float = 50.0, w_sigma: float = 0.02):
    """Small generic case for tests: (X [M,K], W [N,K], outlier idx)."""
    rng = np.random.default_rng(seed)
    idx = _pick(rng, K, n_outliers) if n_outliers else np.zeros(0, np.int64)
    X = rng.standard_normal((M, K), dtype=np.float32)
    if n_outliers:
        X[:, idx] *= np.float32(factor)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(w_sigma)
    return X.astype(dtype), W.astype(dtype), idx


def kv_cache(seed: int = 0, T: int = 4096, H: int = 8, D: int = 128, T_cal: int = 512):
    """One layer's K and V cache, [T x H x D] fp16, with a calibration prefix.

    Heads differ in range (the reason for per-head scales): head h is drawn as
    N(0, 1) times a per-head factor, log-uniform in [0.25, 8]; a few (head, dim)
    lanes per head are 10x larger.  Draw order: per-head factors (K, then V),
    outlier lanes (K, then V), K_cal, V_cal [T_cal x H x D], then K, V [T x H x D].
    Returns (K_cal, V_cal, K, V) as float16 arrays.
    """
    rng = np.random.default_rng(seed)
    fac = [np.exp(rng.uniform(np.log(0.25), np.log(8.0), H)).astype(np.float32) for _ in range(2)]
    lanes = [np.stack([_pick(rng, D, 2) for _ in range(H)]) for _ in range(2)]

    def draw(n, which):
        x = rng.standard_normal((n, H, D), dtype=np.float32) * fac[which][None, :, None]
        for h in range(H):
            x[:, h, lanes[which][h]] *= np.float32(10.0)
        return x.astype(np.float16)

    K_cal, V_cal = draw(T_cal, 0), draw(T_cal, 1)
    return K_cal, V_cal, draw(T, 0), draw(T, 1)


WORKLOADS = {
    "single_w8a8": single_w8a8,
    "prefill_7b": prefill_7b,
    "decode_70b": decode_70b,
    "llm_int8": llm_int8_4096,
    "slice_530b": slice_530b,
}
