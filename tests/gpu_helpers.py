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


def oracle_prefill(wl, w64, x, pos, kc, vc, rows=None, bf16_points=None, bidirectional=False,
                   kv_exact=None):
    if bf16_points is None:
        bf16_points = wl.dtype == "bf16"
    return O.decoder_layer(f64(x), f64(pos).astype(np.int64), w64, f64(kc), f64(vc),
                           n_heads=wl.n_heads, n_kv_heads=wl.n_kv_heads, eps=wl.rms_eps,
                           rope_base=wl.rope_base, bf16_points=bf16_points, rows=rows,
                           bidirectional=bidirectional, kv_exact=kv_exact)


def rms(a) -> float:
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a)))


def rel_err(got, ref) -> float:
    """max |got - ref| / RMS(ref)"""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(rms(ref), 1e-30))


def bf16_ulp(a):
    """Spacing of bf16 values at |a| (8 significant bits): 2^(floor(log2|a|) - 7)."""
    a = np.abs(np.asarray(a, np.float64))
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    return np.where(a > 0, np.ldexp(1.0, e - 8), 0.0)


def assert_bf16_output(got, ref, what=""):
    """The bf16 gate: max |got - ref| <= 0.02 x RMS(ref), where ref is the
    rounding-point oracle's unrounded output.  Printed beside it: the error
    beyond the half bf16 ulp that rounding an exact result to bf16 costs (a
    diagnostic of the compute error alone; not the gate)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    e = rel_err(got, ref)
    r = max(rms(ref), 1e-30)
    beyond = float(np.max(np.maximum(np.abs(got - ref) - bf16_ulp(ref) / 2, 0.0)) / r)
    mean = float(np.mean(np.abs(got - ref)) / r)
    print(f"  {what}: max|err|/rms = {e:.5f} (gate {BF16_RMS_GATE}); mean {mean:.2e}; "
          f"beyond the output's half ulp {beyond:.5f}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert e <= BF16_RMS_GATE, f"{what}: max|err|/rms = {e} > {BF16_RMS_GATE}"


def assert_bf16_cache(got, exact, rounded, what=""):
    """Cache entries written by a bf16 call.  Gate: max |got - exact| <=
    0.02 x RMS(exact) against the oracle's unrounded keys/values (kv_exact).
    Also: both sides store the bf16 rounding of values that agree to
    accumulation noise, so at most 5% of the entries may differ from the
    oracle's own rounding at all (a systematic rounding error, such as
    truncation or double rounding, flips far more)."""
    got, exact, rounded = (np.asarray(a, np.float64) for a in (got, exact, rounded))
    e = rel_err(got, exact)
    flips = int(np.count_nonzero(got != rounded))
    over_ulp = float(np.max(np.abs(got - rounded) / np.maximum(bf16_ulp(rounded), 1e-30)))
    print(f"  {what}: max|err|/rms = {e:.5f} (gate {BF16_RMS_GATE}) against the unrounded oracle; "
          f"{flips}/{got.size} entries differ from its bf16 rounding, by at most {over_ulp:.2f} ulp",
          flush=True)
    assert np.all(np.isfinite(got)), what
    assert e <= BF16_RMS_GATE, f"{what}: max|err|/rms = {e} > {BF16_RMS_GATE}"
    assert flips <= 0.05 * got.size, f"{what}: {flips} of {got.size} entries differ"


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
