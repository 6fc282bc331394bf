"""Seeded synthetic inputs for the MoE expert layer.

This module is shared by the tests, the bench and the oracle's callers. It draws
random tensors and nothing else: it holds none of the layer's arithmetic
(routing, matmuls, activations, quantisation), so the HIP path and the oracle
stay independent of each other while consuming identical input bytes.

Workload shapes mirror the five layer configurations the library is measured
on. Every headline number on the pages is taken under random routing
(Ai2 Olmo-core 3 on kongchang.com, section on the conditions behind the
throughput numbers), so router logits are i.i.d. normal; the skewed workload
adds a fixed Zipf-shaped per-expert bias. The pages also warn that input values
change compute time at fixed matrix sizes (bytechap.com, "Why this matters"),
so no workload uses zeros or constants.

Streams: tensor s of seed `seed` uses numpy PCG64(SeedSequence([seed, s])),
s = 0 logits, 1 X, 2 W1, 3 W2, 4 dOut. Large tensors can instead be drawn on
the GPU with a seeded torch generator (`device_inputs`); both produce float32
draws which are then scaled and rounded once to the storage dtype.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

STREAM_LOGITS, STREAM_X, STREAM_W1, STREAM_W2, STREAM_DOUT = range(5)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens
    d: int          # model width
    E: int          # experts
    k: int          # experts per token
    h: int          # SwiGLU hidden width per expert
    dtype: str      # "f32" | "bf16" | "mxfp8"
    logit_scale: float
    x_scale: float
    w_scale: float
    zipf_s: float = 0.0     # 0 = no expert bias
    backward: bool = True

    @property
    def R(self) -> int:
        return self.T * self.k

    def fwd_flops(self) -> int:
        # GEMM1 (2h outputs) + GEMM2, useful rows only
        return 6 * self.R * self.d * self.h

    def fwd_bwd_flops(self) -> int:
        return 18 * self.R * self.d * self.h


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 256, 128, 8, 2, 256, "f32", 0.02, 0.02, 0.02),
    "e8_bf16_fwd": Workload("e8_bf16_fwd", 8192, 2048, 8, 4, 1024, "bf16", 1.0, 1.0, 0.02,
                            backward=False),
    "e128_bf16": Workload("e128_bf16", 16384, 2048, 128, 4, 1024, "bf16", 1.0, 1.0, 0.02),
    "e128_bf16_zipf": Workload("e128_bf16_zipf", 16384, 2048, 128, 4, 1024, "bf16", 1.0, 1.0,
                               0.02, zipf_s=1.2),
    "e128_mxfp8": Workload("e128_mxfp8", 32768, 4096, 128, 4, 2048, "mxfp8", 1.0, 1.0, 0.02),
    # one GPU's share of the E=128 fwd+bwd layer if its experts were spread
    # over 8 GPUs: 16 experts with ~512 rows each (the same rows per expert,
    # d, h and k; an eighth of the tokens)
    "e16_bf16_ep_share": Workload("e16_bf16_ep_share", 2048, 2048, 16, 4, 1024, "bf16", 1.0,
                                  1.0, 0.02),
}


def zipf_bias(E: int, s: float) -> np.ndarray:
    """Per-expert logit bias ln p_e with p_e proportional to (e+1)^-s, normalised."""
    p = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    return np.log(p).astype(np.float32)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def normal(shape, seed: int, stream: int, scale: float = 1.0) -> np.ndarray:
    """float32 N(0, scale^2) draws from the given stream."""
    a = _rng(seed, stream).standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def host_inputs(w: Workload, seed: int = 0, with_dout: bool = True):
    """All layer inputs as float32 numpy arrays (values already representable in
    the storage dtype when it is bf16: rounded once, to nearest even, via torch)."""
    import torch

    logits = normal((w.T, w.E), seed, STREAM_LOGITS, w.logit_scale)
    if w.zipf_s:
        logits = logits + zipf_bias(w.E, w.zipf_s)[None, :]
    x = normal((w.T, w.d), seed, STREAM_X, w.x_scale)
    w1 = normal((w.E, 2 * w.h, w.d), seed, STREAM_W1, w.w_scale)
    w2 = normal((w.E, w.d, w.h), seed, STREAM_W2, w.w_scale)
    dout = normal((w.T, w.d), seed, STREAM_DOUT, 1.0) if with_dout else None

    def store(a):
        if a is None or w.dtype == "f32":
            return a
        return torch.from_numpy(a).to(torch.bfloat16).float().numpy()

    # weights of the mxfp8 workload stay fp32 masters; activations are bf16
    w_store = (lambda a: a) if w.dtype == "mxfp8" else store
    return dict(logits=logits.astype(np.float32), x=store(x), w1=w_store(w1),
                w2=w_store(w2), dout=store(dout))


def device_inputs(w: Workload, seed: int = 0, device="cuda", with_dout: bool = True):
    """The same workload drawn directly on the GPU with a seeded torch generator
    (for the full-size configurations, where host generation is slow). Values
    differ from host_inputs, but the recipe (distribution, scale, rounding) is
    identical. Returns torch tensors on `device`."""
    import torch

    def draw(shape, stream, scale, dtype):
        g = torch.Generator(device=device)
        g.manual_seed(seed * 1000003 + stream)
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            t.mul_(scale)
        return t.to(dtype)

    act = torch.float32 if w.dtype == "f32" else torch.bfloat16
    wdt = torch.float32 if w.dtype in ("f32", "mxfp8") else torch.bfloat16
    logits = draw((w.T, w.E), STREAM_LOGITS, w.logit_scale, torch.float32)
    if w.zipf_s:
        logits += torch.from_numpy(zipf_bias(w.E, w.zipf_s)).to(device)[None, :]
    out = dict(
        logits=logits,
        x=draw((w.T, w.d), STREAM_X, w.x_scale, act),
        w1=draw((w.E, 2 * w.h, w.d), STREAM_W1, w.w_scale, wdt),
        w2=draw((w.E, w.d, w.h), STREAM_W2, w.w_scale, wdt),
        dout=draw((w.T, w.d), STREAM_DOUT, 1.0, act) if with_dout else None,
    )
    return out


def sample_indices(n: int, count: int, seed: int, stream: int = 99) -> np.ndarray:
    """Sorted distinct sample of range(n) (for sampled parity at full size)."""
    count = min(count, n)
    return np.sort(_rng(seed, stream).choice(n, size=count, replace=False)).astype(np.int64)


def capacity(w: Workload, factor: float = 1.25) -> int:
    """Uniform per-expert capacity of the padded baseline: ceil(factor * T*k / E)."""
    return int(math.ceil(factor * w.R / w.E))
