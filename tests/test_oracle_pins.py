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


def _torch_layer(x, pos, w, kc, vc, H, Hkv, eps=1e-6, base=10000.0, bidirectional=False):
    """Independent fp64 re-derivation from library routines: F.rms_norm,
    F.linear, RoPE as complex multiplication, SDPA with enable_gqa and an
    explicit boolean position mask (bidirectional: every new token of a
    sequence sees the slots up to the sequence's largest new position), F.silu."""
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))  # noqa: E731
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

    xn = F.rms_norm(x, (d,), W["attn_norm"], eps)
    q = F.linear(xn, W["wq"]).view(B, T, H, dh).transpose(1, 2)
    k = F.linear(xn, W["wk"]).view(B, T, Hkv, dh).transpose(1, 2)
    v = F.linear(xn, W["wv"]).view(B, T, Hkv, dh).transpose(1, 2)
    q, k = rot(q, pos), rot(k, pos)
    for b in range(B):
        kc[b, :, pos[b]] = k[b]
        vc[b, :, pos[b]] = v[b]
    S = kc.shape[2]
    lim = pos.max(dim=1, keepdim=True).values.expand(B, T) if bidirectional else pos
    allowed = torch.arange(S)[None, None, :] <= lim[:, :, None]      # [B, T, S]
    o = F.scaled_dot_product_attention(q, kc, vc, attn_mask=allowed[:, None], enable_gqa=True)
    x1 = x + F.linear(o.transpose(1, 2).reshape(B, T, H * dh), W["wo"])
    xn2 = F.rms_norm(x1, (d,), W["ffn_norm"], eps)
    y = x1 + F.linear(F.silu(F.linear(xn2, W["w_gate"])) * F.linear(xn2, W["w_up"]), W["w_down"])
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
