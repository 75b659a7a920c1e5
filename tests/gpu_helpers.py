"""Shared helpers of the GPU parity tests: build a layer from a workload, run
it through the C ABI, run the oracle on host copies of the very same tensors,
and compare."""
from __future__ import annotations

import numpy as np
import torch

import synth
from oracle import llama_oracle as O

# bf16 gate: max-abs error <= 2e-2 x RMS of the oracle output (rounding-point oracle)
BF16_RMS_GATE = 2e-2
# fp32 gate: max-abs error <= 1e-4 against the plain oracle
F32_ABS_GATE = 1e-4


def f64(t) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def layer_config(lib, wl: synth.Workload, max_tokens: int, max_pos: int | None = None,
                 bidirectional: bool = False):
    return lib.make_config(wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.d_ff,
                           max_pos or wl.max_pos, max_tokens, wl.dtype, wl.rms_eps, wl.rope_base,
                           bidirectional=bidirectional)


def oracle_weights(w: dict) -> dict:
    return {k: f64(v) for k, v in w.items()}


def oracle_prefill(wl, w64, x, pos, kc, vc, rows=None, bf16_points=None, bidirectional=False):
    if bf16_points is None:
        bf16_points = wl.dtype == "bf16"
    return O.decoder_layer(f64(x), f64(pos).astype(np.int64), w64, f64(kc), f64(vc),
                           n_heads=wl.n_heads, n_kv_heads=wl.n_kv_heads, eps=wl.rms_eps,
                           rope_base=wl.rope_base, bf16_points=bf16_points, rows=rows,
                           bidirectional=bidirectional)


def rms(a) -> float:
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a)))


def rel_err(got, ref) -> float:
    """max |got - ref| / RMS(ref)"""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(rms(ref), 1e-30))


def assert_bf16_output(got, ref, what=""):
    """The bf16 gate: every element within 0.02 x RMS(ref) of the unrounded
    oracle value, beyond the half bf16 ulp that rounding the output itself
    must cost.  A correctly rounded exact result is off by up to half an ulp
    of |ref|, which alone reaches 0.0165 x RMS on the 70B-shape sample (max|y|
    of 40 at RMS 7.6), so the gate bounds the compute error on top of that."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    e = rel_err(got, ref)
    r = max(rms(ref), 1e-30)
    beyond = float(np.max(np.maximum(np.abs(got - ref) - bf16_ulp(ref) / 2, 0.0)) / r)
    print(f"  {what}: max|err|/rms = {e:.5f}; beyond the output's half ulp {beyond:.5f} (gate {BF16_RMS_GATE})",
          flush=True)
    assert np.all(np.isfinite(got)), what
    assert beyond <= BF16_RMS_GATE, f"{what}: {beyond} beyond half an ulp ({e} in all)"


def bf16_ulp(a):
    """Spacing of bf16 values at |a| (8 significant bits): 2^(floor(log2|a|) - 7)."""
    a = np.abs(np.asarray(a, np.float64))
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    return np.where(a > 0, np.ldexp(1.0, e - 8), 0.0)


def xn_flip_floor(x, gain, w, eps=1e-6):
    """Largest cache-entry shift that one legitimate rounding-point difference
    upstream can cause.  Both sides round the normalised activations xn to bf16
    at the same point, but from fp32 (GPU) and fp64 (oracle) values, so a rare
    element can land one bf16 step apart; that step (at most one ulp of
    max|xn|) reaches k or v through one weight (at most max|W|).  Two such
    flips in one token are allowed for."""
    xn = O.rms_norm(np.asarray(x, np.float64).reshape(-1, np.shape(x)[-1]), gain, eps)
    return 2.0 * float(np.max(bf16_ulp(np.max(np.abs(xn))))) * float(np.max(np.abs(w)))


def assert_bf16_storage(got, ref, what="", floor=None):
    """Cache entries are stored as bf16 on both sides: the GPU rounds its fp32
    result, the rounding-point oracle rounds its fp64 one.  Two correct
    roundings of values that agree to accumulation noise are equal or one bf16
    step apart, so each entry must lie within one ulp of the oracle's, plus an
    absolute floor for upstream rounding-point differences (xn_flip_floor)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    if floor is None:
        floor = 2e-3 * rms(ref)
    bound = bf16_ulp(ref) + floor
    worst = float(np.max(np.abs(got - ref) - bound))
    flips = int(np.count_nonzero(got != ref))
    print(f"  {what}: max|err|/rms = {rel_err(got, ref):.5f}, {flips}/{got.size} entries differ, "
          f"worst excess over one ulp + {floor:.2e} = {worst:.3g}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert worst <= 0.0, f"{what}: exceeds the bound by {worst}"
    # correctly rounded results agree almost everywhere; a systematic rounding
    # error (truncation, double rounding) flips a large share of entries
    assert flips <= 0.05 * got.size, f"{what}: {flips} of {got.size} entries differ"


def kv_floors(x, w):
    """(K floor, V floor) for assert_bf16_storage from the inputs of a call."""
    xx, g = f64(x), f64(w["attn_norm"])
    return xn_flip_floor(xx, g, f64(w["wk"])), xn_flip_floor(xx, g, f64(w["wv"]))


def assert_f32(got, ref, what=""):
    e = float(np.max(np.abs(np.asarray(got, np.float64) - ref)))
    print(f"  {what}: max|err| = {e:.3g} (gate {F32_ABS_GATE})", flush=True)
    assert e <= F32_ABS_GATE, f"{what}: {e}"


def sample_rows(B, T, seed, extra=8):
    """Flat token indices: tile edges, the ends, and a few random rows per sequence."""
    rng = np.random.default_rng(seed)
    base = [0, 1, 2, 31, 32, 63, 64, 127, 128, 129, 255, 256, 511, 1000, 2047, 2048, T - 2, T - 1]
    rows = []
    for b in range(B):
        ts = {t for t in base if 0 <= t < T} | set(rng.integers(0, T, size=extra).tolist())
        rows += [b * T + t for t in sorted(ts)]
    return rows
