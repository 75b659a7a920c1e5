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


def _gate(got, ref, what, extra=""):
    """max |got - ref| <= 0.02 x RMS(ref), element by element, where ref is
    the oracle's unrounded value.  The one exception is an element whose
    correctly rounded bf16 value is itself farther from ref than that (the
    format cannot do better there: e.g. |ref| >= 8 at RMS 1.4): it must then
    be exactly that value.  Returns the raw max |err| / RMS."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    r = max(rms(ref), 1e-30)
    err = np.abs(got - ref)
    nearest = O.bf16_round(ref)
    tol = BF16_RMS_GATE * r
    beyond_format = np.abs(nearest - ref) > tol
    ok = (err <= tol) | (beyond_format & (got == nearest))
    e = float(np.max(err) / r)
    beyond = float(np.max(np.maximum(err - bf16_ulp(ref) / 2, 0.0)) / r)
    mean = float(np.mean(err) / r)
    print(f"  {what}: max|err|/rms = {e:.5f} (gate {BF16_RMS_GATE}); mean {mean:.2e}; beyond the "
          f"output's half ulp {beyond:.5f}; {int(beyond_format.sum())} entries whose nearest bf16 is "
          f"beyond the gate{extra}", flush=True)
    assert np.all(np.isfinite(got)), what
    bad = np.nonzero(~ok)
    assert bad[0].size == 0, (f"{what}: {bad[0].size} elements off by more than {BF16_RMS_GATE} x RMS, e.g. "
                              f"index {tuple(int(i[0]) for i in bad)}: got {got[tuple(i[0] for i in bad)]}, "
                              f"oracle {ref[tuple(i[0] for i in bad)]}")
    return e


def assert_bf16_output(got, ref, what=""):
    """The bf16 gate on a layer output (see _gate), against the rounding-point
    oracle's unrounded output.  The error beyond the half bf16 ulp that
    rounding an exact result costs is printed as a diagnostic."""
    return _gate(got, ref, what)


def assert_bf16_cache(got, exact, rounded, what=""):
    """Cache entries written by a bf16 call: the same gate (see _gate) against
    the oracle's unrounded keys/values (kv_exact).  Also: both sides store
    the bf16 rounding of values that agree to accumulation noise, so at most
    5% of the entries may differ from the oracle's own rounding at all (a
    systematic rounding error, such as truncation or double rounding, flips
    far more)."""
    got, exact, rounded = (np.asarray(a, np.float64) for a in (got, exact, rounded))
    flips = int(np.count_nonzero(got != rounded))
    e = _gate(got, exact, what, f"; {flips}/{got.size} entries differ from the oracle's bf16 rounding")
    assert flips <= 0.05 * got.size, f"{what}: {flips} of {got.size} entries differ"
    return e


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
