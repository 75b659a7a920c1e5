"""Seeded synthetic inputs for the decoder-layer tests, smoke run and benchmark.

This module is the only code that both the CPU oracle side and the HIP side
use.  It holds none of the layer's arithmetic: it draws numbers and names the
workloads (shapes, seeds, distributions).

Generator (counter-based, order independent, so any element can be drawn on
its own and any slice gives the same values as the whole tensor):

    base     = splitmix64(seed XOR (tensor_id << 32))
    a_i, b_i = splitmix64(base + 2 i), splitmix64(base + 2 i + 1)     (mod 2^64)
    u1       = ((a_i >> 11) + 1) * 2^-53          in (0, 1]
    u2       =  (b_i >> 11)      * 2^-53          in [0, 1)
    n_i      = sqrt(-2 ln u1) * cos(2 pi u2)       (Box-Muller, fp64)

splitmix64 is Steele, Lea and Flood's SplitMix64 output function
("Fast splittable pseudorandom number generators", OOPSLA 2014):
z += 0x9E3779B97F4A7C15; z = (z ^ z>>30) * 0xBF58476D1CE4E5B9;
z = (z ^ z>>27) * 0x94D049BB133111EB; return z ^ z>>31.

Values are scaled by the requested standard deviation in fp64, rounded to
fp32 (round-to-nearest-even) and, for bf16 workloads, rounded once more to
bf16 by torch's conversion.  Whatever tensor is handed to the GPU is the very
tensor (copied to the host) that the oracle receives.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK = (1 << 64) - 1

# tensor ids
TID_X = 1
TID_WQ, TID_WK, TID_WV, TID_WO, TID_WGATE, TID_WUP, TID_WDOWN = 2, 3, 4, 5, 6, 7, 8
TID_KCACHE, TID_VCACHE = 9, 10
TID_GAIN1, TID_GAIN2 = 11, 12
TID_DECODE_BASE = 100  # decode step s draws its input with tensor id 100 + s
TID_EMBED, TID_FINAL_NORM, TID_LMHEAD, TID_UNIFORM = 13, 14, 15, 16
TID_LAYER_SEED_STRIDE = 1000  # layer l of a stack uses seed + 1000 l


def splitmix64_int(z: int) -> int:
    """SplitMix64 output function on one Python int (mod 2^64)."""
    z = (z + _GOLDEN) & _MASK
    z = ((z ^ (z >> 30)) * _M1) & _MASK
    z = ((z ^ (z >> 27)) * _M2) & _MASK
    return z ^ (z >> 31)


def _base(seed: int, tensor_id: int) -> int:
    return splitmix64_int((seed ^ (tensor_id << 32)) & _MASK)


def _splitmix64_np(z: np.ndarray) -> np.ndarray:
    z = z + np.uint64(_GOLDEN)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
    return z ^ (z >> np.uint64(31))


def normal_np(seed: int, tensor_id: int, start: int, count: int) -> np.ndarray:
    """fp64 N(0,1) draws for flat indices [start, start+count) on the host."""
    base = np.uint64(_base(seed, tensor_id))
    idx = np.arange(start, start + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        a = _splitmix64_np(base + np.uint64(2) * idx)
        b = _splitmix64_np(base + np.uint64(2) * idx + np.uint64(1))
    u1 = ((a >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0**-53
    u2 = (b >> np.uint64(11)).astype(np.float64) * 2.0**-53
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def _s64(v: int) -> int:
    """Unsigned 64-bit constant as the int64 with the same bits."""
    return v - (1 << 64) if v >= (1 << 63) else v


def _normal_torch(seed: int, tensor_id: int, start: int, count: int, device):
    """Same draws as normal_np, computed with int64 tensors on a torch device.

    int64 multiplication wraps modulo 2^64 on the GPU, which gives the same
    bits as the unsigned arithmetic above; right shifts are made logical by
    masking the sign-extended bits.
    """
    import torch

    def lsr(z, k):
        return (z >> k) & ((1 << (64 - k)) - 1)

    def mix(z):
        z = z + _s64(_GOLDEN)
        z = (z ^ lsr(z, 30)) * _s64(_M1)
        z = (z ^ lsr(z, 27)) * _s64(_M2)
        return z ^ lsr(z, 31)

    base = _s64(_base(seed, tensor_id))
    idx = torch.arange(start, start + count, dtype=torch.int64, device=device)
    a = mix(idx * 2 + base)
    b = mix(idx * 2 + (base + 1 if base + 1 < (1 << 63) else base + 1 - (1 << 64)))
    u1 = (lsr(a, 11).to(torch.float64) + 1.0) * 2.0**-53
    u2 = lsr(b, 11).to(torch.float64) * 2.0**-53
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(2.0 * math.pi * u2)


def normal_tensor(seed: int, tensor_id: int, shape, std: float, dtype, device="cpu",
                  chunk: int = 1 << 24):
    """A torch tensor of N(0, std^2) draws, rounded fp64 -> fp32 -> dtype.

    On a CUDA/HIP device the draws are made there (int64 torch ops); on the
    host they are made with numpy's unsigned arithmetic.  Both give the same
    integers; the fp64 transcendental step may differ in the last bit between
    the two, which is why a test always hands the oracle a host copy of the
    exact tensor the GPU used.
    """
    import torch

    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = torch.empty(n, dtype=dtype, device=device)
    on_gpu = torch.device(device).type == "cuda"
    for s in range(0, n, chunk):
        c = min(chunk, n - s)
        if on_gpu:
            v = _normal_torch(seed, tensor_id, s, c, device) * std
            out[s:s + c] = v.to(torch.float32).to(dtype)
        else:
            v = normal_np(seed, tensor_id, s, c) * std
            out[s:s + c] = torch.from_numpy(v.astype(np.float32)).to(dtype)
    return out.view(shape)


# --------------------------------------------------------------------------
# Workloads.  Shapes are the LLaMA layer shapes the pages discuss (7B
# 4096/11008, 13B 5120/13824, 70B 8192/28672 with grouped-query attention),
# plus a tiny fp32 layer.  Weights ~ N(0, 0.02), activations ~ N(0, 1),
# RMSNorm gains 1, eps 1e-6, RoPE base 10000, no biases.
# --------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str              # "f32" or "bf16"
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    batch: int
    seq: int                # prefill tokens per sequence (0: decode only)
    prior: int = 0          # cache slots already filled before the call
    decode_steps: int = 0   # sequential single-token decode calls after prefill
    seed: int = 20261203
    rms_eps: float = 1e-6
    rope_base: float = 10000.0
    w_std: float = 0.02
    x_std: float = 1.0
    cache_std: float = 1.0  # std of random prior cache entries

    @property
    def max_pos(self) -> int:
        return self.prior + self.seq + self.decode_steps

    @property
    def tokens(self) -> int:
        return self.batch * max(self.seq, 1)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "f32", 64, 4, 4, 16, 172, 1, 16, seed=20261203),
    "llama7b_prefill": Workload("llama7b_prefill", "bf16", 4096, 32, 32, 128, 11008, 1, 2048,
                                seed=20261204),
    "llama13b_prefill": Workload("llama13b_prefill", "bf16", 5120, 40, 40, 128, 13824, 2, 4096,
                                 seed=20261205),
    "llama7b_decode": Workload("llama7b_decode", "bf16", 4096, 32, 32, 128, 11008, 32, 0,
                               prior=4095, decode_steps=1, seed=20261206),
    "llama70b_gqa": Workload("llama70b_gqa", "bf16", 8192, 64, 8, 128, 28672, 1, 4096,
                             decode_steps=64, seed=20261207),
    # one GPU's share of llama70b_gqa under 8-way tensor parallelism (heads
    # and the MLP's intermediate dimension split 8 ways; d unchanged)
    "llama70b_tp8_shard": Workload("llama70b_tp8_shard", "bf16", 8192, 8, 1, 128, 3584, 1, 4096,
                                   decode_steps=64, seed=20261208),
}


def torch_dtype(wl: Workload):
    import torch
    return torch.float32 if wl.dtype == "f32" else torch.bfloat16


def make_weights(wl: Workload, device="cpu", random_gains: bool = False):
    """nn.Linear-layout ([out, in]) weights and RMSNorm gains for a workload."""
    import torch

    dt = torch_dtype(wl)
    d, H, Hkv, dh, f = wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.d_ff
    s = wl.seed
    w = {
        "wq": normal_tensor(s, TID_WQ, (H * dh, d), wl.w_std, dt, device),
        "wk": normal_tensor(s, TID_WK, (Hkv * dh, d), wl.w_std, dt, device),
        "wv": normal_tensor(s, TID_WV, (Hkv * dh, d), wl.w_std, dt, device),
        "wo": normal_tensor(s, TID_WO, (d, H * dh), wl.w_std, dt, device),
        "w_gate": normal_tensor(s, TID_WGATE, (f, d), wl.w_std, dt, device),
        "w_up": normal_tensor(s, TID_WUP, (f, d), wl.w_std, dt, device),
        "w_down": normal_tensor(s, TID_WDOWN, (d, f), wl.w_std, dt, device),
    }
    if random_gains:
        w["attn_norm"] = (1.0 + normal_tensor(s, TID_GAIN1, (d,), 0.1, torch.float32, device)).to(dt)
        w["ffn_norm"] = (1.0 + normal_tensor(s, TID_GAIN2, (d,), 0.1, torch.float32, device)).to(dt)
    else:
        w["attn_norm"] = torch.ones(d, dtype=dt, device=device)
        w["ffn_norm"] = torch.ones(d, dtype=dt, device=device)
    return w


def make_x(wl: Workload, tokens_shape, tensor_id: int = TID_X, device="cpu"):
    return normal_tensor(wl.seed, tensor_id, tuple(tokens_shape) + (wl.d_model,), wl.x_std,
                         torch_dtype(wl), device)


def make_cache(wl: Workload, device="cpu", batch: int | None = None):
    """K and V caches [B, Hkv, max_pos, dh]; the first `prior` slots hold
    N(0, cache_std^2) entries (keys taken as already rotated), the rest zero."""
    import torch

    B = wl.batch if batch is None else batch
    shape = (B, wl.n_kv_heads, wl.max_pos, wl.head_dim)
    dt = torch_dtype(wl)
    k = torch.zeros(shape, dtype=dt, device=device)
    v = torch.zeros(shape, dtype=dt, device=device)
    if wl.prior > 0:
        pshape = (B, wl.n_kv_heads, wl.prior, wl.head_dim)
        k[:, :, :wl.prior] = normal_tensor(wl.seed, TID_KCACHE, pshape, wl.cache_std, dt, device)
        v[:, :, :wl.prior] = normal_tensor(wl.seed, TID_VCACHE, pshape, wl.cache_std, dt, device)
    return k, v


def prefill_positions(batch: int, seq: int, start: int = 0, device="cpu"):
    import torch
    p = torch.arange(start, start + seq, dtype=torch.int32, device=device)
    return p.unsqueeze(0).expand(batch, seq).contiguous()


def scaled(wl: Workload, **changes) -> Workload:
    """A copy of a workload with some fields changed (e.g. a shorter sequence)."""
    return dataclasses.replace(wl, **changes)


def uniform_np(seed: int, tensor_id: int, count: int) -> np.ndarray:
    """U[0, 1) draws (53-bit) from the same counter-based generator, fp64."""
    base = np.uint64(_base(seed, tensor_id))
    idx = np.arange(count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        a = _splitmix64_np(base + idx)
    return (a >> np.uint64(11)).astype(np.float64) * 2.0**-53


def make_model_weights(wl: Workload, n_layers: int, vocab: int, device="cpu", random_gains: bool = False,
                       lm_std: float = 0.05):
    """Embedding [V, d] ~ N(0, 1), final gain, LM head [V, d] ~ N(0, lm_std^2),
    and n_layers layer weight dicts (layer l drawn with seed + 1000 l)."""
    import torch

    dt = torch_dtype(wl)
    d, s = wl.d_model, wl.seed
    layers = [make_weights(dataclasses.replace(wl, seed=s + TID_LAYER_SEED_STRIDE * (l + 1)), device, random_gains)
              for l in range(n_layers)]
    final = ((1.0 + normal_tensor(s, TID_FINAL_NORM, (d,), 0.1, torch.float32, device)).to(dt)
             if random_gains else torch.ones(d, dtype=dt, device=device))
    return {"embed": normal_tensor(s, TID_EMBED, (vocab, d), 1.0, dt, device), "final_norm": final,
            "lm_head": normal_tensor(s, TID_LMHEAD, (vocab, d), lm_std, dt, device), "layers": layers}
