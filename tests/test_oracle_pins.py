"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a worked
example printed on the pages (fixtures under tests/golden/), a closed form, an
invariant, a library routine (torch CPU fp64) or brute force on tiny inputs.
No GPU is needed.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import llama_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_round_matches_torch_conversion():
    """Library routine: torch's fp32 -> bf16 conversion is round-to-nearest-even."""
    x = _rng(1).standard_normal(200000).astype(np.float32) * np.float32(3.0)
    x = np.concatenate([x, np.float32([0.0, -0.0, 1.0, 1e-30, -7.5e20])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_round(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: the even neighbour is 1.
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6.
    got = O.bf16_round(np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 1 + 2**-8 + 2**-30]))
    np.testing.assert_array_equal(got, [1.0, 1 + 2**-6, -1.0, 1 + 2**-7])


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_worked_example():
    g = _golden("rmsnorm_worked_example.json")
    x = np.array(g["x"])
    assert np.mean(x * x) == pytest.approx(g["mean_square"], rel=1e-15)
    assert round(np.mean(x * x), 2) == g["page_mean_square_approx"]
    y = O.rms_norm(x, 1.0, g["eps"])
    np.testing.assert_array_equal(np.round(y, g["page_decimals"]), g["page_output_approx"])
    np.testing.assert_allclose(y, x / math.sqrt(14.0 / 3.0 + 1e-6), rtol=1e-15)


def test_rmsnorm_unit_rms_and_library_routine():
    """Notes runnable example 05: output RMS ~ 1 and equal to F.rms_norm."""
    rng = _rng(2)
    x = rng.standard_normal((7, 96)) * 3.0
    y1 = O.rms_norm(x, 1.0, 1e-6)
    np.testing.assert_allclose(np.sqrt(np.mean(y1 * y1, axis=-1)), 1.0, atol=1e-6)
    g = 1.0 + 0.1 * rng.standard_normal(96)
    ref = F.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), 1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, g, 1e-6), ref, rtol=1e-12, atol=1e-13)


def test_rmsnorm_eps_inside_sqrt_closed_form():
    # x = 1e-3 everywhere: mean square 1e-6, so x / sqrt(1e-6 + 1e-6) = 1/sqrt(2).
    y = O.rms_norm(np.full(64, 1e-3), 1.0, 1e-6)
    np.testing.assert_allclose(y, 1 / math.sqrt(2.0), rtol=1e-12)
    # the zero vector maps to zero (eps prevents 0/0)
    assert np.all(O.rms_norm(np.zeros(16), 1.0, 1e-6) == 0.0)


# ---------------------------------------------------------------- RoPE

def test_rope_worked_example():
    g = _golden("rope_worked_example.json")
    inv = O.rope_inv_freq(g["head_dim"], g["base"])
    np.testing.assert_allclose(inv, g["page_inv_freq"], rtol=1e-15)
    np.testing.assert_allclose(g["pos"] * inv, g["page_freqs"], rtol=1e-15)
    cos, sin = O.rope_cos_sin(g["pos"], g["head_dim"], g["base"])
    np.testing.assert_allclose(cos, g["page_cos_approx"], atol=g["page_cos_sin_abs_tol"])
    np.testing.assert_allclose(sin, g["page_sin_approx"], atol=g["page_cos_sin_abs_tol"])
    # the page's pairing: q0' = q0 cos(2) - q2 sin(2), q1' = q1 cos(0.02) - q3 sin(0.02)
    q = np.array([1.0, 2.0, 3.0, 4.0])
    out = O.rope(q, g["pos"], g["base"])
    assert out[0] == pytest.approx(1.0 * math.cos(2.0) - 3.0 * math.sin(2.0), rel=1e-14)
    assert out[1] == pytest.approx(2.0 * math.cos(0.02) - 4.0 * math.sin(0.02), rel=1e-14)


def test_rope_equals_complex_rotation():
    """Closed form: rotate-half RoPE is multiplication of z_i = x_i + j x_{i+half}
    by exp(j p theta_i)."""
    rng = _rng(3)
    dh, base = 128, 10000.0
    x = rng.standard_normal((5, dh))
    pos = np.array([0, 1, 17, 2047, 4159])
    theta = base ** (-np.arange(0, dh, 2) / dh)
    z = x[:, : dh // 2] + 1j * x[:, dh // 2:]
    zr = z * np.exp(1j * pos[:, None] * theta[None, :])
    ref = np.concatenate([zr.real, zr.imag], axis=-1)
    np.testing.assert_allclose(O.rope(x, pos, base), ref, rtol=1e-12, atol=1e-12)


def test_rope_invariants():
    """Notes §02.2 and runnable example 04: norm kept, position 0 is the identity,
    the q.k product depends only on the position difference."""
    rng = _rng(4)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    assert np.linalg.norm(O.rope(q, 7, 10000.0)) == pytest.approx(np.linalg.norm(q), rel=1e-13)
    np.testing.assert_array_equal(O.rope(q, 0, 10000.0), q)
    dot_a = O.rope(q, 2, 10000.0) @ O.rope(k, 5, 10000.0)
    dot_b = O.rope(q, 9, 10000.0) @ O.rope(k, 12, 10000.0)
    assert dot_a == pytest.approx(dot_b, abs=1e-12)
    # and a different offset gives a different product (the map is not trivial)
    dot_c = O.rope(q, 2, 10000.0) @ O.rope(k, 6, 10000.0)
    assert abs(dot_c - dot_a) > 1e-3


# ---------------------------------------------------------------- attention

def test_causal_mask_zero_future_rows_sum_to_one():
    """Notes §02.1, runnable example 03 and lab 02: future weight exactly 0,
    rows sum to 1, query 3 reads keys 0..3 only."""
    rng = _rng(5)
    T, dh = 8, 16
    q, k, v = (rng.standard_normal((T, dh)) * 3 for _ in range(3))
    _, a = O.masked_softmax_attention(q, k, v, np.arange(T), np.arange(T))
    future = np.triu(np.ones((T, T), dtype=bool), 1)
    assert np.all(a[future] == 0.0)
    np.testing.assert_allclose(a.sum(-1), 1.0, atol=1e-14)
    assert np.all(a[3, :4] > 0) and np.all(a[3, 4:] == 0)


def test_attention_matches_sdpa_and_single_token():
    rng = _rng(6)
    T, dh = 11, 32
    q, k, v = (rng.standard_normal((T, dh)) for _ in range(3))
    o, _ = O.masked_softmax_attention(q, k, v, np.arange(T), np.arange(T))
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(t)[None, None] for t in (q, k, v)),
                                         is_causal=True)[0, 0].numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    # the first query sees only the first key: its output is v_0
    np.testing.assert_allclose(o[0], v[0], rtol=1e-15)


def test_repeat_kv_head_map_matches_library_gqa():
    """GQA: torch's enable_gqa maps query head h to kv head h // (H/Hkv)."""
    rng = _rng(7)
    H, Hkv, T, dh = 8, 2, 9, 16
    q = rng.standard_normal((H, T, dh))
    k = rng.standard_normal((Hkv, T, dh))
    v = rng.standard_normal((Hkv, T, dh))
    kk, vv = O.repeat_kv(k, H // Hkv), O.repeat_kv(v, H // Hkv)
    got = np.stack([O.masked_softmax_attention(q[h], kk[h], vv[h], np.arange(T), np.arange(T))[0]
                    for h in range(H)])
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None], torch.from_numpy(k)[None],
                                         torch.from_numpy(v)[None], is_causal=True,
                                         enable_gqa=True)[0].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- SwiGLU

def test_mlp_param_table():
    g = _golden("mlp_param_table.json")
    for row in g["rows"]:
        n = O.mlp_param_count(row["d"], row["f"])
        assert n == pytest.approx(row["page_params"], rel=g["relative_tolerance"])
        # three bias-free d x f matrices (gate [f,d], up [f,d], down [d,f])
        assert n == row["f"] * row["d"] + row["f"] * row["d"] + row["d"] * row["f"]


def test_silu_library_and_limits():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(O.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-14,
                               atol=1e-300)
    assert O.silu(0.0) == 0.0
    assert O.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(O.silu(-40.0)) < 1e-15


def test_swiglu_is_not_relu_squared():
    """Notes runnable example 06: same shape, different numbers."""
    rng = _rng(8)
    x = rng.standard_normal((4, 32))
    wg, wu, wd = rng.standard_normal((64, 32)), rng.standard_normal((64, 32)), rng.standard_normal((32, 64))
    y = O.swiglu_hidden(x, wg, wu) @ wd.T
    relu2 = np.maximum(x @ wg.T, 0.0) ** 2 @ wd.T
    assert y.shape == x.shape
    assert not np.allclose(y, relu2)
    # the activation sits on the gate branch only: swapping gate and up changes the result
    assert not np.allclose(y, O.swiglu_hidden(x, wu, wg) @ wd.T)


# ---------------------------------------------------------------- KV cache accounting

def test_kv_cache_bytes_formula():
    """Notes Ch.04 memory accounting and runnable example 08 (fp32: 4 bytes)."""
    T, layers, batch, heads, head_dim = 37, 3, 2, 4, 16
    assert O.kv_cache_bytes(layers, batch, T, heads, head_dim, 4) == \
        T * layers * batch * heads * head_dim * 2 * 4
    # the notes' lab default shape per layer: [1, 4096, 8, 128] for K and for V, bf16
    assert O.kv_cache_bytes(1, 1, 4096, 8, 128, 2) == 2 * 4096 * 8 * 128 * 2


# ---------------------------------------------------------------- whole layer

def _tiny(seed, B=2, T=6, d=32, H=4, Hkv=2, f=48, S=None, gains=True):
    rng = _rng(seed)
    dh = d // H
    S = S or T
    w = {
        "wq": rng.standard_normal((H * dh, d)) * 0.2, "wk": rng.standard_normal((Hkv * dh, d)) * 0.2,
        "wv": rng.standard_normal((Hkv * dh, d)) * 0.2, "wo": rng.standard_normal((d, H * dh)) * 0.2,
        "w_gate": rng.standard_normal((f, d)) * 0.2, "w_up": rng.standard_normal((f, d)) * 0.2,
        "w_down": rng.standard_normal((d, f)) * 0.2,
        "attn_norm": 1 + 0.1 * rng.standard_normal(d) if gains else np.ones(d),
        "ffn_norm": 1 + 0.1 * rng.standard_normal(d) if gains else np.ones(d),
    }
    x = rng.standard_normal((B, T, d))
    kc = np.zeros((B, Hkv, S, dh))
    vc = np.zeros((B, Hkv, S, dh))
    return x, w, kc, vc


def _round_via_odd_fp32(a, dtype):
    """fp64 -> dtype (bf16 or fp16) rounded to nearest even with torch's own
    conversions, without double rounding: round to fp32 *to odd* first, then
    let torch round fp32 -> dtype.  Boldo and Melquiond, "Emulation of FMA and
    correctly rounded sums: proved algorithms using rounding to odd" (IEEE
    Trans. Computers, 2008): exact when the intermediate format has at least
    two more bits (fp32 has 24; bf16 8, fp16 11).  Round to odd keeps exact
    values and otherwise takes, of the two fp32 neighbours of the value, the
    one whose last significand bit is 1."""
    a = torch.as_tensor(a, dtype=torch.float64)
    f = a.to(torch.float32)                        # nearest fp32
    back = f.to(torch.float64)
    inexact = back != a
    even = (f.view(torch.int32) & 1) == 0
    away = torch.where(back < a, torch.full_like(f, math.inf), torch.full_like(f, -math.inf))
    odd = torch.where(inexact & even, torch.nextafter(f, away), f)
    return odd.to(dtype).to(torch.float64)


def _f16_torch(a):
    return _round_via_odd_fp32(a, torch.float16)


def _bf16_torch(a):
    """fp64 -> bf16 (round to nearest, ties to even) with torch's own
    conversions, as an independent check of the oracle's frexp/rint rounding.

    torch converts fp64 to bf16 through fp32, and rounding twice can differ
    from rounding once (a value just off a bf16 midpoint can land on it in
    fp32).  Rounding to fp32 *to odd* first makes the second rounding exact:
    Boldo and Melquiond, "Emulation of FMA and correctly rounded sums: proved
    algorithms using rounding to odd" (IEEE Trans. Computers, 2008), which
    needs at least two more bits in the intermediate format (fp32 has 24,
    bf16 8).  Round to odd keeps exact values and otherwise takes, of the two
    fp32 neighbours of the value, the one whose last significand bit is 1."""
    return _round_via_odd_fp32(a, torch.bfloat16)


def _torch_layer(x, pos, w, kc, vc, H, Hkv, eps=1e-6, base=10000.0, bidirectional=False,
                 rnd=None, rnd16=None, kv_exact=None):
    """Independent fp64 re-derivation from library routines: F.rms_norm,
    F.linear, RoPE as complex multiplication, SDPA with enable_gqa and an
    explicit boolean position mask (bidirectional: every new token of a
    sequence sees the slots up to the sequence's largest new position), F.silu.
    rnd (default: none) is applied at the bf16 layer's bf16 rounding points
    (the normalised activations, q and k after RoPE, v), rnd16 at its fp16
    ones (the attention output and the SwiGLU product)."""
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))  # noqa: E731
    r = rnd or (lambda a: a)  # noqa: E731
    r16 = rnd16 or (lambda a: a)  # noqa: E731
    x, kc, vc = t(x), t(kc).clone(), t(vc).clone()
    W = {k: t(v) for k, v in w.items()}
    B, T, d = x.shape
    dh = d // H
    pos = torch.as_tensor(pos, dtype=torch.int64)

    def rot(a, p):  # a [B, h, T, dh], p [B, T]
        theta = base ** (-torch.arange(0, dh, 2, dtype=torch.float64) / dh)
        ang = p[:, None, :, None].to(torch.float64) * theta
        z = torch.complex(a[..., : dh // 2], a[..., dh // 2:]) * torch.exp(1j * ang)
        return torch.cat([z.real, z.imag], dim=-1)

    xn = r(F.rms_norm(x, (d,), W["attn_norm"], eps))
    q = F.linear(xn, W["wq"]).view(B, T, H, dh).transpose(1, 2)
    k = F.linear(xn, W["wk"]).view(B, T, Hkv, dh).transpose(1, 2)
    v = F.linear(xn, W["wv"]).view(B, T, Hkv, dh).transpose(1, 2)
    q, k = r(rot(q, pos)), rot(k, pos)
    if kv_exact is not None:
        kv_exact["k"], kv_exact["v"] = k.numpy().copy(), v.numpy().copy()
    k, v = r(k), r(v)
    for b in range(B):
        kc[b, :, pos[b]] = k[b]
        vc[b, :, pos[b]] = v[b]
    S = kc.shape[2]
    lim = pos.max(dim=1, keepdim=True).values.expand(B, T) if bidirectional else pos
    allowed = torch.arange(S)[None, None, :] <= lim[:, :, None]      # [B, T, S]
    o = F.scaled_dot_product_attention(q, kc, vc, attn_mask=allowed[:, None], enable_gqa=True)
    o = r16(o.transpose(1, 2).reshape(B, T, H * dh))
    x1 = x + F.linear(o, W["wo"])
    xn2 = r(F.rms_norm(x1, (d,), W["ffn_norm"], eps))
    h = r16(F.silu(F.linear(xn2, W["w_gate"])) * F.linear(xn2, W["w_up"]))
    y = x1 + F.linear(h, W["w_down"])
    return y.numpy(), kc.numpy(), vc.numpy()


@pytest.mark.parametrize("H,Hkv", [(4, 4), (4, 2), (4, 1)])
def test_layer_matches_library_rederivation(H, Hkv):
    x, w, kc, vc = _tiny(10 + Hkv, H=H, Hkv=Hkv)
    pos = np.tile(np.arange(6), (2, 1))
    y, k2, v2 = O.decoder_layer(x, pos, w, kc, vc, n_heads=H, n_kv_heads=Hkv)
    yr, kr, vr = _torch_layer(x, pos, w, kc, vc, H, Hkv)
    np.testing.assert_allclose(y, yr, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(k2, kr, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(v2, vr, rtol=1e-12, atol=1e-12)


def test_layer_with_prior_cache_matches_library_rederivation():
    """Chunked prefill: 4 new tokens at positions 5..8 over 5 prior cache slots."""
    H, Hkv = 4, 2
    x, w, kc, vc = _tiny(20, B=2, T=4, H=H, Hkv=Hkv, S=12)
    rng = _rng(21)
    kc[:, :, :5] = rng.standard_normal(kc[:, :, :5].shape)
    vc[:, :, :5] = rng.standard_normal(vc[:, :, :5].shape)
    pos = np.tile(np.arange(5, 9), (2, 1))
    y, k2, v2 = O.decoder_layer(x, pos, w, kc, vc, n_heads=H, n_kv_heads=Hkv)
    yr, kr, vr = _torch_layer(x, pos, w, kc, vc, H, Hkv)
    np.testing.assert_allclose(y, yr, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(k2, kr, atol=1e-12)
    # slots the call did not write are untouched
    np.testing.assert_array_equal(k2[:, :, :5], kc[:, :, :5])
    np.testing.assert_array_equal(k2[:, :, 9:], 0.0)


def test_layer_shape_and_zero_output_projections():
    """Notes runnable example 02 (shape kept); with W_o = W_down = 0 both
    residual branches add exactly zero, so y == x bit for bit."""
    x, w, kc, vc = _tiny(30)
    pos = np.tile(np.arange(6), (2, 1))
    y, _, _ = O.decoder_layer(x, pos, w, kc, vc, n_heads=4, n_kv_heads=2)
    assert y.shape == x.shape
    w0 = dict(w, wo=np.zeros_like(w["wo"]), w_down=np.zeros_like(w["w_down"]))
    y0, _, _ = O.decoder_layer(x, pos, w0, kc, vc, n_heads=4, n_kv_heads=2)
    np.testing.assert_array_equal(y0, x)


def test_layer_is_causal():
    """Changing later tokens leaves earlier outputs unchanged."""
    x, w, kc, vc = _tiny(31, B=1, T=8)
    pos = np.arange(8)[None]
    y, _, _ = O.decoder_layer(x, pos, w, kc, vc, n_heads=4, n_kv_heads=2)
    x2 = x.copy()
    x2[0, 5:] = _rng(32).standard_normal(x2[0, 5:].shape)
    y2, _, _ = O.decoder_layer(x2, pos, w, kc, vc, n_heads=4, n_kv_heads=2)
    np.testing.assert_array_equal(y2[0, :5], y[0, :5])
    assert not np.allclose(y2[0, 5:], y[0, 5:])


@pytest.mark.parametrize("prior", [0, 5])
def test_bidirectional_layer_matches_library_rederivation(prior):
    """The encoder-style variant (LARQL page: the SigLIP encoder's attention is
    the causal one without the mask), fresh and over a prior cache."""
    H, Hkv, T = 4, 2, 5
    x, w, kc, vc = _tiny(40 + prior, B=2, T=T, H=H, Hkv=Hkv, S=prior + T + 3)
    if prior:
        rng = _rng(41)
        kc[:, :, :prior] = rng.standard_normal(kc[:, :, :prior].shape)
        vc[:, :, :prior] = rng.standard_normal(vc[:, :, :prior].shape)
    pos = np.tile(np.arange(prior, prior + T), (2, 1))
    y, k2, _ = O.decoder_layer(x, pos, w, kc, vc, n_heads=H, n_kv_heads=Hkv, bidirectional=True)
    yr, kr, _ = _torch_layer(x, pos, w, kc, vc, H, Hkv, bidirectional=True)
    np.testing.assert_allclose(y, yr, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(k2, kr, atol=1e-12)


def test_bidirectional_sees_later_tokens_and_agrees_at_the_last():
    """Without the mask an earlier token's output depends on later tokens; the
    token at the largest position sees the same slots either way, so its
    output equals the causal layer's."""
    x, w, kc, vc = _tiny(42, B=1, T=8)
    pos = np.arange(8)[None]
    kw = dict(n_heads=4, n_kv_heads=2)
    yb, _, _ = O.decoder_layer(x, pos, w, kc, vc, bidirectional=True, **kw)
    yc, _, _ = O.decoder_layer(x, pos, w, kc, vc, **kw)
    np.testing.assert_allclose(yb[0, -1], yc[0, -1], rtol=1e-13, atol=1e-13)
    assert not np.allclose(yb[0, 0], yc[0, 0])
    x2 = x.copy()
    x2[0, 5:] = _rng(43).standard_normal(x2[0, 5:].shape)
    yb2, _, _ = O.decoder_layer(x2, pos, w, kc, vc, bidirectional=True, **kw)
    assert not np.allclose(yb2[0, :5], yb[0, :5])


def test_decode_equals_last_row_of_prefill():
    """Notes runnable examples 07/08: prefill T tokens, then decode token T at
    position T (the cache length) equals row T of a prefill of T+1 tokens."""
    H, Hkv, T = 4, 2, 7
    x, w, kc, vc = _tiny(40, B=2, T=T + 1, H=H, Hkv=Hkv, S=T + 1)
    pos = np.tile(np.arange(T + 1), (2, 1))
    y_full, k_full, v_full = O.decoder_layer(x, pos, w, kc, vc, n_heads=H, n_kv_heads=Hkv)
    _, k1, v1 = O.decoder_layer(x[:, :T], pos[:, :T], w, kc, vc, n_heads=H, n_kv_heads=Hkv)
    # the cache position advances: slots 0..T-1 written, slot T still empty
    assert np.all(k1[:, :, T] == 0) and np.all(np.any(k1[:, :, :T] != 0, axis=-1))
    y_dec, k2, v2 = O.decoder_layer_decode(x[:, T], np.full(2, T), w, k1, v1,
                                           n_heads=H, n_kv_heads=Hkv)
    np.testing.assert_allclose(y_dec, y_full[:, T], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(k2, k_full, atol=1e-13)
    np.testing.assert_allclose(v2, v_full, atol=1e-13)


def test_rows_subset_equals_full_rows():
    x, w, kc, vc = _tiny(50, B=2, T=6)
    pos = np.tile(np.arange(6), (2, 1))
    for bf in (False, True):
        y, k2, _ = O.decoder_layer(x, pos, w, kc, vc, n_heads=4, n_kv_heads=2, bf16_points=bf)
        ys, k3, _ = O.decoder_layer(x, pos, w, kc, vc, n_heads=4, n_kv_heads=2, bf16_points=bf,
                                    rows=[1, 6, 11])
        flat, flats = y.reshape(12, -1), ys.reshape(12, -1)
        # BLAS may block a 3-row product differently from a 12-row one: equal
        # up to fp64 rounding (a bf16 rounding point can move by one ulp)
        np.testing.assert_allclose(flats[[1, 6, 11]], flat[[1, 6, 11]],
                                   rtol=1e-12, atol=(2e-2 if bf else 1e-12))
        assert np.all(np.isnan(flats[[0, 2, 3, 4, 5, 7, 8, 9, 10]]))
        np.testing.assert_array_equal(k3, k2)


def test_bf16_points_mode_is_close_but_rounded():
    x, w, kc, vc = _tiny(60, B=1, T=6)
    pos = np.arange(6)[None]
    y, k, v = O.decoder_layer(x, pos, w, kc, vc, n_heads=4, n_kv_heads=2)
    yb, kb, vb = O.decoder_layer(x, pos, w, kc, vc, n_heads=4, n_kv_heads=2, bf16_points=True)
    # written cache entries are bf16 values in this mode
    np.testing.assert_array_equal(O.bf16_round(kb), kb)
    np.testing.assert_array_equal(O.bf16_round(vb), vb)
    rms = np.sqrt(np.mean(y * y))
    assert 0 < np.max(np.abs(yb - y)) < 0.05 * rms


# ------------------------------------------------- the bf16 rounding-point mode

def test_bf16_torch_rounding_helper_is_correct_rounding():
    """The test's own fp64 -> bf16 route (round to odd, then torch's fp32 ->
    bf16) against the exact midpoint cases where rounding twice would go wrong,
    and against torch's fp32 -> bf16 on values fp32 holds exactly."""
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7; a hair above it must round up,
    # though its fp32 rounding (1 + 2^-8 exactly) would round to even (down)
    vals = torch.tensor([1 + 2**-8 + 2**-40, 1 + 2**-8 - 2**-40, 1 + 2**-8, 1 + 3 * 2**-8,
                         -(1 + 2**-8 + 2**-40)], dtype=torch.float64)
    want = torch.tensor([1 + 2**-7, 1.0, 1.0, 1 + 2**-6, -(1 + 2**-7)], dtype=torch.float64)
    assert torch.equal(_bf16_torch(vals), want)
    x = torch.randn(100000, dtype=torch.float32, generator=torch.Generator().manual_seed(3))
    assert torch.equal(_bf16_torch(x.double()), x.to(torch.bfloat16).double())


def test_fp16_round_matches_library_conversion():
    """Library routine: numpy's fp32 -> fp16 conversion (round to nearest
    even) on values fp32 holds exactly, across normal and subnormal fp16
    ranges; ties; saturation at the largest finite value."""
    rng = _rng(7)
    x = np.concatenate([rng.standard_normal(100000) * s for s in (1e-6, 1e-4, 1.0, 100.0, 1e4)])
    x32 = x.astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(O.fp16_round(x32), x32.astype(np.float16).astype(np.float64))
    # 1 + 2^-11 is the midpoint of 1 and 1 + 2^-10 (to even: 1); 1 + 3 2^-11 -> 1 + 2^-9
    np.testing.assert_array_equal(O.fp16_round(np.array([1 + 2**-11, 1 + 3 * 2**-11, 1 + 2**-11 + 2**-40])),
                                  [1.0, 1 + 2**-9, 1 + 2**-10])
    assert O.fp16_round(np.array([1e5, -7e4])).tolist() == [65504.0, -65504.0]
    assert O.fp16_round(np.array([2.0**-25, 3 * 2.0**-25])).tolist() == [0.0, 2.0**-23]


def test_rounding_helper_fp16_is_correct_rounding():
    """The test's fp64 -> fp16 route, like the bf16 one: a value a hair above
    a midpoint must round up although its fp32 rounding lands on the midpoint."""
    vals = torch.tensor([1 + 2**-11 + 2**-40, 1 + 2**-11 - 2**-40], dtype=torch.float64)
    assert torch.equal(_f16_torch(vals), torch.tensor([1 + 2**-10, 1.0], dtype=torch.float64))
    x = torch.randn(100000, dtype=torch.float32, generator=torch.Generator().manual_seed(4))
    assert torch.equal(_f16_torch(x.double()), x.half().double())


def _bf16_case(seed=61, B=1, T=7, H=4, Hkv=2, prior=0):
    x, w, kc, vc = _tiny(seed, B=B, T=T, H=H, Hkv=Hkv, S=prior + T + 2)
    if prior:
        rng = _rng(seed + 1)
        kc[:, :, :prior] = O.bf16_round(rng.standard_normal(kc[:, :, :prior].shape))
        vc[:, :, :prior] = O.bf16_round(rng.standard_normal(vc[:, :, :prior].shape))
    pos = np.tile(np.arange(prior, prior + T), (B, 1))
    return x, w, kc, vc, pos


@pytest.mark.parametrize("B,H,Hkv,prior", [(1, 4, 2, 0), (2, 4, 4, 0), (2, 4, 1, 5)])
def test_bf16_points_mode_matches_library_rederivation(B, H, Hkv, prior):
    """The rounding-point mode (the reference of every bf16 comparison) against
    the torch re-derivation with independent roundings at the same seven
    points: bf16 (_bf16_torch) at xn, q, k, v and xn2, fp16 (_f16_torch) at
    the attention output and h.
    Agreement to 1e-12: the two sides' pre-rounding values differ only by fp64
    evaluation order (~1e-16 relative), so they round differently only for a
    value within that distance of a bf16 midpoint (a tie; none occurs in these
    seeded cases, about 1e-13 per element)."""
    x, w, kc, vc, pos = _bf16_case(61 + 7 * B + Hkv + prior, B=B, H=H, Hkv=Hkv, prior=prior)
    ex, exr = {}, {}
    y, k2, v2 = O.decoder_layer(x, pos, w, kc, vc, n_heads=H, n_kv_heads=Hkv, bf16_points=True,
                                kv_exact=ex)
    yr, kr, vr = _torch_layer(x, pos, w, kc, vc, H, Hkv, rnd=_bf16_torch, rnd16=_f16_torch, kv_exact=exr)
    np.testing.assert_allclose(y, yr, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(k2, kr)
    np.testing.assert_array_equal(v2, vr)
    np.testing.assert_allclose(ex["k"], exr["k"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(ex["v"], exr["v"], rtol=0, atol=1e-12)
    # the cache holds the rounding of the exact values, and the rounding moved them
    for b in range(B):
        np.testing.assert_array_equal(k2[b][:, pos[b]], O.bf16_round(ex["k"][b]))
    assert np.max(np.abs(k2[:, :, prior:prior + x.shape[1]] - ex["k"])) > 0


_ROUNDING_POINTS = ("xn", "k", "v", "q", "o", "xn2", "h")  # the order decoder_layer rounds them in (B = 1)


@pytest.mark.parametrize("dropped", range(len(_ROUNDING_POINTS)), ids=list(_ROUNDING_POINTS))
def test_bf16_points_pin_catches_a_dropped_rounding(dropped, monkeypatch):
    """Planted mistakes in the oracle: skipping any one of its seven bf16
    rounding points makes it disagree with the re-derivation above (in y or
    in the cache), so the pin covers every point."""
    x, w, kc, vc, pos = _bf16_case(61 + 7 + 2)
    yr, kr, vr = _torch_layer(x, pos, w, kc, vc, 4, 2, rnd=_bf16_torch, rnd16=_f16_torch)
    real = O._maybe_round
    calls = []

    def mutant(a, bf16_points, fmt="bf16"):
        calls.append(len(calls))
        return a if len(calls) - 1 == dropped else real(a, bf16_points, fmt)
    monkeypatch.setattr(O, "_maybe_round", mutant)
    y, k2, v2 = O.decoder_layer(x, pos, w, kc, vc, n_heads=4, n_kv_heads=2, bf16_points=True)
    assert len(calls) == len(_ROUNDING_POINTS)
    diff = max(np.max(np.abs(y - yr)), np.max(np.abs(k2 - kr)), np.max(np.abs(v2 - vr)))
    assert diff > 1e-6, f"dropping the rounding of {_ROUNDING_POINTS[dropped]} went unnoticed ({diff})"


# ----------------------------------------------------------- paged KV cache

def test_gather_pages_hand_worked():
    """Two sequences, pages of 2 slots, one kv head of width 1: the page pool
    holds the values 10 * page + row, and the block tables [2, 0] and [1, 3]
    lay sequence 0's slots 0..3 over pages 2, 2, 0, 0 and sequence 1's over
    1, 1, 3, 3."""
    pool = np.array([[[[10 * pg + r] for r in range(2)]] for pg in range(4)], dtype=np.float64)  # [4,1,2,1]
    got = O.gather_pages(pool, [[2, 0], [1, 3]], 2, 4)
    np.testing.assert_array_equal(got[:, 0, :, 0], [[20, 21, 0, 1], [10, 11, 30, 31]])


def test_scatter_then_gather_is_identity_on_written_slots():
    rng = _rng(70)
    B, Hkv, ps, dh, nblk = 3, 2, 4, 5, 3
    perm = rng.permutation(B * nblk + 2)[:B * nblk].reshape(B, nblk)   # distinct pages, two spare
    pool = rng.standard_normal((B * nblk + 2, Hkv, ps, dh))
    cache = rng.standard_normal((B, Hkv, ps * nblk, dh))
    slots = [[0, 5, 11], [3], [4, 7, 8, 9]]
    new = O.scatter_pages(cache, pool, perm, ps, slots)
    back = O.gather_pages(new, perm, ps, ps * nblk)
    for b in range(B):
        np.testing.assert_array_equal(back[b][:, slots[b]], cache[b][:, slots[b]])
        others = [p for p in range(ps * nblk) if p not in slots[b]]
        np.testing.assert_array_equal(back[b][:, others], O.gather_pages(pool, perm, ps, ps * nblk)[b][:, others])
    # pages no sequence maps are untouched
    spare = sorted(set(range(B * nblk + 2)) - set(perm.ravel().tolist()))
    np.testing.assert_array_equal(new[spare], pool[spare])


def test_paged_layer_equals_contiguous_layer():
    """A prefill over a prior cache, then a decode step, on a shuffled page
    table equal the contiguous layer on the gathered cache (the paging only
    moves where slots live)."""
    H, Hkv, T, prior, ps = 4, 2, 5, 6, 4
    x, w, _, _ = _tiny(71, B=2, T=T, H=H, Hkv=Hkv)
    dh = 32 // H
    nblk = 4                                               # capacity 16 >= prior + T + 1
    rng = _rng(72)
    bt = rng.permutation(2 * nblk + 3)[:2 * nblk].reshape(2, nblk)
    kp = rng.standard_normal((2 * nblk + 3, Hkv, ps, dh))
    vp = rng.standard_normal((2 * nblk + 3, Hkv, ps, dh))
    pos = np.tile(np.arange(prior, prior + T), (2, 1))
    kw = dict(n_heads=H, n_kv_heads=Hkv, bf16_points=True)
    y, kp2, vp2 = O.decoder_layer_paged(x, pos, w, kp, vp, bt, ps, nblk * ps, **kw)
    kc, vc = O.gather_pages(kp, bt, ps, nblk * ps), O.gather_pages(vp, bt, ps, nblk * ps)
    yc, kc2, vc2 = O.decoder_layer(x, pos, w, kc, vc, **kw)
    np.testing.assert_array_equal(y, yc)
    np.testing.assert_array_equal(O.gather_pages(kp2, bt, ps, nblk * ps), kc2)
    np.testing.assert_array_equal(O.gather_pages(vp2, bt, ps, nblk * ps), vc2)
    xd = _rng(73).standard_normal((2, 32))
    yd, _, _ = O.decoder_layer_paged(xd[:, None], np.full((2, 1), prior + T), w, kp2, vp2, bt, ps, nblk * ps, **kw)
    ydc, _, _ = O.decoder_layer_decode(xd, np.full(2, prior + T), w, kc2, vc2, **kw)
    np.testing.assert_array_equal(yd[:, 0], ydc)


# --------------------------------------------------------------------------
# int8 KV cache (the reading: symmetric int8 codes, one fp32 scale per row;
# Notes Ch.04 and "Llama MLP deep dive" §6.4 name cache quantisation, no scheme)
# --------------------------------------------------------------------------

def test_kv_int8_worked_example():
    """[1, -2, 0.5, 0]: amax 2, 127/2 = 63.5 exactly, so 1 -> 63.5 -> 64 (half
    to even), -2 -> -127, 0.5 -> 31.75 -> 32, 0 -> 0; scale fp32(2/127)."""
    c, s = O.kv_int8_quantize(np.array([[1.0, -2.0, 0.5, 0.0], [0.0, 0.0, 0.0, 0.0]]))
    assert c.dtype == np.int8 and s.dtype == np.float32
    np.testing.assert_array_equal(c, [[64, -127, 32, 0], [0, 0, 0, 0]])
    assert s[0] == np.float32(2.0) / np.float32(127.0) and s[1] == 0.0
    # 2.5 * 127 / 5 = 63.5 again, now from a row whose amax is 5; 1.5 * 25.4 = 38.1
    c, s = O.kv_int8_quantize(np.array([2.5, -5.0, 1.5, -0.0]))
    np.testing.assert_array_equal(c, [64, -127, 38, 0])
    # a tie that half-to-even and half-away-from-zero round apart: amax
    # 127/32 makes 127/amax = 32 exactly, and 62.5/32 * 32 = 62.5 -> 62
    c, s = O.kv_int8_quantize(np.array([62.5 / 32, -127 / 32, -61.5 / 32, 0.5 / 32]))
    np.testing.assert_array_equal(c, [62, -127, -62, 0])
    assert s == np.float32(1 / 32)
    # rows below 2^-100 are stored as zeros; just above, quantized as usual
    c, s = O.kv_int8_quantize(np.array([[2.0 ** -101, -(2.0 ** -102)], [2.0 ** -99, -(2.0 ** -100)]]))
    np.testing.assert_array_equal(c, [[0, 0], [127, -64]])
    assert s[0] == 0 and s[1] == np.float32(2.0 ** -99) / np.float32(127)


def test_kv_int8_properties():
    """On seeded bf16 rows: codes in [-127, 127], each row's largest magnitude
    maps to +-127, every code is the nearest integer to x * 127/amax (error at
    most half a step, up to fp32 rounding), negation flips the codes and keeps
    the scale, and quantizing the dequantized row gives the same codes."""
    rng = _rng(71)
    x = O.bf16_round(rng.standard_normal((64, 128)) * rng.uniform(0.01, 100, (64, 1)))
    c, s = O.kv_int8_quantize(x)
    ci = c.astype(np.int64)
    assert np.all(np.abs(ci) <= 127)
    am = np.argmax(np.abs(x), axis=1)
    np.testing.assert_array_equal(np.abs(ci[np.arange(64), am]), 127)
    deq = O.kv_int8_dequantize(c, s)
    step = s.astype(np.float64)[:, None]
    # half a step, plus what the fp32 roundings of inv, s and x * inv add:
    # |x| |1 - inv s| + s |x inv| 2^-24 <= 127 s (2^-23 + 2^-24 + 2^-24) < 4e-5 s
    assert np.all(np.abs(x - deq) <= (0.5 + 4e-5) * step)
    cn, sn = O.kv_int8_quantize(-x)
    np.testing.assert_array_equal(cn.astype(np.int64), -ci)
    np.testing.assert_array_equal(sn, s)
    c2, s2 = O.kv_int8_quantize(deq)
    np.testing.assert_array_equal(c2, c)
    np.testing.assert_allclose(s2, s, rtol=1e-6)


def test_kv_int8_decode_wiring():
    """The int8 decode step: the new token's key and value rows are the
    quantization of the rows the bf16 cache would hold (plain mode: the exact
    ones), written at slot p, every other slot unchanged; the output is the
    bf16-cache decode's up to the quantization error (a few 1e-3 here), and
    attends to the quantized new row, not the exact one."""
    x, w, kc, vc = _tiny(73, B=2, T=1, S=12)
    rng = _rng(74)
    kc[:, :, :9] = rng.standard_normal((2, 2, 9, 8))
    vc[:, :, :9] = rng.standard_normal((2, 2, 9, 8))
    kq, ks = O.kv_int8_quantize(kc)
    vq, vs = O.kv_int8_quantize(vc)
    kw = dict(n_heads=4, n_kv_heads=2)
    pos = np.array([9, 5])
    ex = {}
    y8, kq2, ks2, vq2, vs2 = O.decoder_layer_decode_int8(x[:, 0], pos, w, kq, ks, vq, vs, kv_exact=ex, **kw)
    for b in range(2):
        cb, sb = O.kv_int8_quantize(ex["k"][b, :, 0])
        np.testing.assert_array_equal(kq2[b, :, pos[b]], cb)
        np.testing.assert_array_equal(ks2[b, :, pos[b]], sb)
        cv, sv = O.kv_int8_quantize(ex["v"][b, :, 0])
        np.testing.assert_array_equal(vq2[b, :, pos[b]], cv)
        others = [j for j in range(12) if j != pos[b]]
        np.testing.assert_array_equal(kq2[b][:, others], kq[b][:, others])
        np.testing.assert_array_equal(vs2[b][:, others], vs[b][:, others])
    # against the bf16-format decode over the dequantized prior cache
    yd, _, _ = O.decoder_layer_decode(x[:, 0], pos, w, O.kv_int8_dequantize(kq, ks),
                                      O.kv_int8_dequantize(vq, vs), **kw)
    err = np.max(np.abs(y8 - yd)) / np.sqrt(np.mean(yd ** 2))
    assert 1e-5 < err < 2e-2, err
    # with the new rows stored exactly, the int8 step reproduces that decode
    ye, _, _ = O.decoder_layer(x[:, :1], pos.reshape(2, 1), w, O.kv_int8_dequantize(kq, ks),
                               O.kv_int8_dequantize(vq, vs), kv_store=O.kv_int8_store, **kw)
    np.testing.assert_allclose(y8, ye.reshape(2, -1), rtol=0, atol=1e-12)
def test_kv_int8_prefill_is_a_run_of_decode_steps():
    """A causal chunk over the int8 cache equals the same tokens fed one decode
    step at a time: every new row is quantized on its own (per token and kv
    head, not over the chunk), lands in its own slot, and every query reads the
    chunk's earlier rows as c * s, not exactly.  Both rounding modes; the two
    sequences start at different positions over different prior lengths; and
    the rows= subset gives the same rows."""
    T = 5
    x, w, kc, vc = _tiny(75, B=2, T=T, S=16)
    rng = _rng(76)
    kc[:, :, :9] = rng.standard_normal((2, 2, 9, 8))
    vc[:, :, :9] = rng.standard_normal((2, 2, 9, 8)) * 3
    kq, ks = O.kv_int8_quantize(kc)
    vq, vs = O.kv_int8_quantize(vc)
    pos = np.array([[9, 10, 11, 12, 13], [4, 5, 6, 7, 8]])
    for bf in (False, True):
        kw = dict(n_heads=4, n_kv_heads=2, bf16_points=bf)
        y, kq2, ks2, vq2, vs2 = O.decoder_layer_int8(x, pos, w, kq, ks, vq, vs, **kw)
        st = (kq, ks, vq, vs)
        ys = []
        for t in range(T):
            yt, *st = O.decoder_layer_decode_int8(x[:, t], pos[:, t], w, *st, **kw)
            ys.append(yt)
        np.testing.assert_allclose(y, np.stack(ys, axis=1), rtol=0, atol=1e-12)
        for a, b_ in zip((kq2, ks2, vq2, vs2), st):
            np.testing.assert_array_equal(a, b_)
        # a chunk quantized as a whole (one amax per chunk) would differ
        assert not np.array_equal(ks2[0, 0, 9:14], np.full(5, ks2[0, 0, 9]))
        yr, *_ = O.decoder_layer_int8(x, pos, w, kq, ks, vq, vs, rows=[1, 7], **kw)
        np.testing.assert_allclose(yr.reshape(10, -1)[[1, 7]], y.reshape(10, -1)[[1, 7]], rtol=0, atol=1e-12)
        assert np.all(np.isnan(yr.reshape(10, -1)[[0, 2, 9]]))




def test_paged_int8_layer_equals_contiguous_int8_layer():
    """int8 page pools (codes and per-row scales) on a shuffled table with
    spare pages: a prefill over prior rows and then a decode step equal the
    contiguous int8 layer on the gathered cache; a new slot's code row and
    scale land in page table[b, p // page] at row p % page; unmapped pages
    are untouched."""
    H, Hkv, T, prior, ps, nblk = 4, 2, 5, 6, 4, 4
    x, w, _, _ = _tiny(77, B=2, T=T, H=H, Hkv=Hkv)
    dh = 32 // H
    rng = _rng(78)
    n_pages = 2 * nblk + 3
    bt = rng.permutation(n_pages)[:2 * nblk].reshape(2, nblk)
    kq, ks = O.kv_int8_quantize(rng.standard_normal((n_pages, Hkv, ps, dh)))
    vq, vs = O.kv_int8_quantize(rng.standard_normal((n_pages, Hkv, ps, dh)) * 2)
    pos = np.array([np.arange(prior, prior + T), np.arange(prior - 3, prior - 3 + T)])
    cap = nblk * ps
    kw = dict(n_heads=H, n_kv_heads=Hkv, bf16_points=True)
    y, kq2, ks2, vq2, vs2 = O.decoder_layer_paged_int8(x, pos, w, kq, ks, vq, vs, bt, ps, cap, **kw)

    def g(c, s):
        return (O.gather_pages(c, bt, ps, cap).astype(np.int8),
                O.gather_pages(s[..., None], bt, ps, cap)[..., 0].astype(np.float32))
    yc, kqc, ksc, vqc, vsc = O.decoder_layer_int8(x, pos, w, *g(kq, ks), *g(vq, vs), **kw)
    np.testing.assert_array_equal(y, yc)
    for (c2, s2), (cc, sc) in zip((g(kq2, ks2), g(vq2, vs2)), ((kqc, ksc), (vqc, vsc))):
        np.testing.assert_array_equal(c2, cc)
        np.testing.assert_array_equal(s2, sc)
    p = pos[1, 2]
    np.testing.assert_array_equal(kq2[bt[1, p // ps], :, p % ps], kqc[1, :, p])
    assert np.array_equal(ks2[bt[1, p // ps], :, p % ps], ksc[1, :, p])
    spare = sorted(set(range(n_pages)) - set(bt.ravel().tolist()))
    np.testing.assert_array_equal(kq2[spare], kq[spare])
    np.testing.assert_array_equal(vs2[spare], vs[spare])
    xd = _rng(79).standard_normal((2, 1, 32))
    pd = np.array([[prior + T], [prior + 4]])
    yd, *_ = O.decoder_layer_paged_int8(xd, pd, w, kq2, ks2, vq2, vs2, bt, ps, cap, **kw)
    ydc, *_ = O.decoder_layer_int8(xd, pd, w, kqc, ksc, vqc, vsc, **kw)
    np.testing.assert_array_equal(yd, ydc)
