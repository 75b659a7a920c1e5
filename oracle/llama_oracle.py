"""Plain CPU oracle for one pre-norm LLaMA decoder layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

Everything is computed in fp64 with numpy, materialising every intermediate
(full score matrices, an explicitly repeated K/V for grouped-query attention).
Sources, cited by page title and section:

  [LMDrive]   "LMDrive 大语言模型（LLM）核心推理单元" (LMDrive LLM core
              inference unit): §2.1 LlamaRMSNorm, §2.2 LlamaRotaryEmbedding,
              §2.3 LlamaAttention, §2.4 LlamaMLP, §2.5 LlamaDecoderLayer.
  [Notes]     "LLM 核心机制交互讲义" (LLM mechanics lecture notes):
              Ch.02 §02.1 causal mask, §02.2 RoPE, §02.3 RMSNorm, §02.4 SwiGLU,
              the pre-norm block equation; Ch.04 prefill/decode, KV cache and
              its memory accounting.
  [MLP]       "深入解析Llama MLP模块：SwiGLU激活函数与参数配置详解" (Llama MLP
              deep dive): §2.2 the gate/up/down computation, §3 parameter counts.
  [LARQL]     "从纯文本到视觉理解：LARQL多模态支持(SigLIP)架构解析" (LARQL
              multimodal support): the SigLIP encoder's bidirectional attention,
              the causal kernel without its future-column mask.

Two modes:
  plain       no intermediate rounding (the gate for fp32 layers);
  bf16 points round-to-nearest-even (this module's own rounding) of exactly
              the tensors a bf16 layer stores or feeds to 16-bit matrix
              products, in the format it uses for them: bf16 for the
              normalised activations, q, k and v (the cache dtype); fp16 for
              the attention output and the SwiGLU product (the A operands of
              o_proj and down, kept with 11 significant bits; the pages fix
              bf16 weights and activations with fp32 accumulation, not the
              format of these internal operands).  Scores, softmax weights,
              the residual stream X' and the returned y are never rounded.

It also holds the paged cache (gather / scatter around the same layer), the
int8 cache (the row quantizer, and a layer call -- a prefill chunk or a
decode step -- over int8 rows), and the two combined (int8 page pools).

Parity status: every function below is pinned by a CPU test against what the
pages or the mathematics fix (worked examples, invariants, library routines
on tiny inputs); see tests/test_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# bf16 rounding (used only in the "bf16 points" mode)
# --------------------------------------------------------------------------

def bf16_round(a):
    """Round fp64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits (1 implicit + 7 stored) and fp32's exponent
    range.  frexp gives a = m * 2^e with 0.5 <= |m| < 1, so m * 2^8 carries
    exactly the 8 bits to keep; np.rint rounds half to even.  Values this
    layer produces never reach bf16's overflow or subnormal range.
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def fp16_round(a):
    """Round fp64 values to the nearest IEEE half-precision value, ties to
    even, saturating at the largest finite value (+-65504).

    fp16 keeps 11 significant bits for |a| >= 2^-14 (normal numbers) and a
    fixed spacing of 2^-24 below that (subnormal numbers)."""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    normal = np.ldexp(np.rint(m * 2048.0), e - 11)
    sub = np.ldexp(np.rint(np.ldexp(a, 24)), -24)
    r = np.where(np.abs(a) >= 2.0**-14, normal, sub)
    return np.clip(r, -65504.0, 65504.0)


def _maybe_round(a, bf16_points: bool, fmt: str = "bf16"):
    if not bf16_points:
        return a
    return fp16_round(a) if fmt == "fp16" else bf16_round(a)


# --------------------------------------------------------------------------
# RMSNorm  [LMDrive §2.1; Notes §02.3]
# --------------------------------------------------------------------------

def rms_norm(x, g, eps):
    """g * x / sqrt(mean(x^2) + eps) over the last axis.

    eps sits inside the square root, next to the mean square.  The gain is
    applied after normalising, in the same precision (the order in the notes'
    runnable example 05, one rounding at the end)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(g, dtype=np.float64) * (x / np.sqrt(ms + eps))


# --------------------------------------------------------------------------
# RoPE, rotate-half convention  [LMDrive §2.2; Notes §02.2]
# --------------------------------------------------------------------------

def rope_inv_freq(head_dim, base):
    """theta_i = base^(-2i/head_dim), i = 0 .. head_dim/2 - 1."""
    i = np.arange(0, head_dim // 2, dtype=np.float64)
    return 1.0 / (float(base) ** (2.0 * i / head_dim))


def rope_cos_sin(positions, head_dim, base):
    """cos and sin of angle p * theta_i, shape positions.shape + (head_dim/2,)."""
    ang = np.asarray(positions, dtype=np.float64)[..., None] * rope_inv_freq(head_dim, base)
    return np.cos(ang), np.sin(ang)


def rope(x, positions, base):
    """Rotate-half RoPE of x[..., head_dim] at the given positions.

    Dimension i (i < head_dim/2) is paired with i + head_dim/2 and the pair is
    turned by the angle p * theta_i:
        x'_i          = x_i cos - x_{i+half} sin
        x'_{i+half}   = x_{i+half} cos + x_i sin
    `positions` broadcasts against x's leading axes (no head axis)."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    cos, sin = rope_cos_sin(positions, x.shape[-1], base)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


# --------------------------------------------------------------------------
# Attention  [LMDrive §2.3; Notes §02.1, Ch.04]
# --------------------------------------------------------------------------

def repeat_kv(kv, n_rep):
    """[..., Hkv, S, dh] -> [..., Hkv*n_rep, S, dh]; kv head g serves query
    heads g*n_rep .. g*n_rep + n_rep - 1 (each kv head repeated in place)."""
    return np.repeat(kv, n_rep, axis=-3)


def masked_softmax_attention(q, k, v, q_pos, k_pos):
    """softmax(q k^T / sqrt(dh) + M) v for one head.

    q [Tq, dh], k/v [S, dh]; M_ij = 0 if k_pos[j] <= q_pos[i] else -inf,
    added before the softmax.  Returns (output [Tq, dh], weights [Tq, S])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dh = q.shape[-1]
    scores = (q @ k.T) / np.sqrt(dh)
    mask = np.where(np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None], 0.0, -np.inf)
    s = scores + mask
    s = s - np.max(s, axis=-1, keepdims=True)
    e = np.exp(s)
    a = e / np.sum(e, axis=-1, keepdims=True)
    return a @ v, a


# --------------------------------------------------------------------------
# SwiGLU MLP  [LMDrive §2.4; MLP §2.2; Notes §02.4]
# --------------------------------------------------------------------------

def silu(z):
    """z * sigmoid(z)."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu_hidden(xn, w_gate, w_up):
    """SiLU(xn W_gate^T) * (xn W_up^T); the activation acts on the gate branch only."""
    return silu(xn @ np.asarray(w_gate, np.float64).T) * (xn @ np.asarray(w_up, np.float64).T)


def mlp_param_count(d_model, d_ff):
    """Parameters of the bias-free gate/up/down MLP: three d x f matrices."""
    return 3 * d_model * d_ff


def kv_cache_bytes(layers, batch, tokens, n_kv_heads, head_dim, elem_bytes):
    """L x 2 (K and V) x B x T x H_kv x d_h x bytes per element [Notes Ch.04]."""
    return layers * 2 * batch * tokens * n_kv_heads * head_dim * elem_bytes


# --------------------------------------------------------------------------
# The decoder layer  [LMDrive §2.5; Notes Ch.02 block equation, Ch.04]
# --------------------------------------------------------------------------

def _f64(a):
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().to("cpu")
        import torch
        a = a.to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def decoder_layer(x, positions, weights, k_cache, v_cache, *, n_heads, n_kv_heads,
                  eps=1e-6, rope_base=10000.0, bf16_points=False, rows=None,
                  bidirectional=False, kv_exact=None, kv_store=None):
    """One pre-norm decoder layer forward over B sequences with a KV cache.

        X'  = x  + o_proj(CausalAttn(RoPE(q, k), v))      q,k,v = proj(RMSNorm1(x))
        y   = X' + down(SiLU(gate(RMSNorm2(X'))) * up(RMSNorm2(X')))

    x          [B, T, d]       token (b, t) sits at position positions[b, t]
    positions  [B, T] ints     its post-RoPE key and raw value are written to
                               cache slot positions[b, t]; its query sees every
                               slot j <= positions[b, t] of sequence b.
    weights    dict of nn.Linear-layout [out, in] matrices wq, wk, wv, wo,
               w_gate, w_up, w_down and gains attn_norm, ffn_norm.
    k_cache, v_cache [B, Hkv, S, dh]: slots below a sequence's first position
               hold its prior (already rotated) keys and values.
    rows       optional list of flat token indices b*T + t; when given, the
               output is computed for those tokens only (keys and values are
               still computed for every token, as the cache needs them).
    bidirectional  the encoder-style variant without the causal mask: every
               new token of sequence b sees every slot up to the largest
               position among the sequence's new tokens.  [LARQL: the SigLIP
               encoder's attention is the causal one without the mask.]
    kv_exact   optional dict; receives "k" and "v" [B, Hkv, T, dh], the new
               tokens' rotated keys and values before the cache dtype's
               rounding (in the bf16 points mode they are computed from the
               rounded normalised activations; the cache holds their bf16
               rounding).  Token (b, t) is [b, :, t].
    kv_store   optional function applied to the new tokens' keys and values
               [B, Hkv, T, dh] (after the cache dtype's rounding) before they
               are written to the cache: the int8 cache stores
               dequantize(quantize(.)) of each row (kv_int8_store).

    Returns (y [B, T, d] (rows not asked for are NaN), k_cache', v_cache').
    """
    x = _f64(x)
    B, T, d = x.shape
    pos = np.asarray(_f64(positions), dtype=np.int64).reshape(B, T)
    W = {k_: _f64(v_) for k_, v_ in weights.items()}
    kc = _f64(k_cache).copy()
    vc = _f64(v_cache).copy()
    H, Hkv = n_heads, n_kv_heads
    dh = W["wq"].shape[0] // H
    n_rep = H // Hkv
    r = lambda a, fmt="bf16": _maybe_round(a, bf16_points, fmt)  # noqa: E731

    xn = r(rms_norm(x, W["attn_norm"], eps))                         # [B,T,d]

    # keys and values for every token: cache write at slot = position
    k = xn @ W["wk"].T                                               # [B,T,Hkv*dh]
    v = xn @ W["wv"].T
    k = k.reshape(B, T, Hkv, dh).transpose(0, 2, 1, 3)               # [B,Hkv,T,dh]
    v = v.reshape(B, T, Hkv, dh).transpose(0, 2, 1, 3)
    k = rope(k, pos[:, None, :], rope_base)
    if kv_exact is not None:
        kv_exact["k"], kv_exact["v"] = k.copy(), v.copy()
    k = r(k)
    v = r(v)
    if kv_store is not None:
        k, v = kv_store(k), kv_store(v)
    for b in range(B):
        kc[b][:, pos[b], :] = k[b]
        vc[b][:, pos[b], :] = v[b]

    want = np.zeros(B * T, dtype=bool)
    if rows is None:
        want[:] = True
    else:
        want[np.asarray(rows, dtype=np.int64)] = True
    want = want.reshape(B, T)

    y = np.full((B, T, d), np.nan)
    for b in range(B):
        ts = np.nonzero(want[b])[0]
        if ts.size == 0:
            continue
        xb, xnb, pb = x[b, ts], xn[b, ts], pos[b, ts]               # [n,d]
        q = (xnb @ W["wq"].T).reshape(ts.size, H, dh).transpose(1, 0, 2)   # [H,n,dh]
        q = r(rope(q, pb[None, :], rope_base))
        # the position each query may see up to: its own, or (bidirectional)
        # the sequence's largest new position
        lim = np.full(ts.size, pos[b].max()) if bidirectional else pb
        S = int(lim.max()) + 1                                       # slots 0 .. max position
        kk = repeat_kv(kc[b][:, :S], n_rep)                          # [H,S,dh]
        vv = repeat_kv(vc[b][:, :S], n_rep)
        heads = [masked_softmax_attention(q[h], kk[h], vv[h], lim, np.arange(S))[0]
                 for h in range(H)]
        o = r(np.stack(heads, axis=1).reshape(ts.size, H * dh), "fp16")  # heads concatenated
        x1 = xb + o @ W["wo"].T                                      # X', never rounded
        xn2 = r(rms_norm(x1, W["ffn_norm"], eps))
        h_ = r(swiglu_hidden(xn2, W["w_gate"], W["w_up"]), "fp16")
        y[b, ts] = x1 + h_ @ W["w_down"].T
    return y, kc, vc


# --------------------------------------------------------------------------
# int8 KV cache  [Notes Ch.04 (KV-cache memory: bytes = 2 B T Hkv dh x the
# element size, and quantising the cache as a lever beside GQA/MQA); "Llama
# MLP deep dive" §6.4 (KV-cache quantisation named)].  The pages give no
# scheme; the reading here: symmetric int8 codes with one fp32 scale per
# cached row (one token's 128 dims of one kv head), taken from the row's bf16
# values.  The code decision is made in fp32, the format the GPU decides it in:
#   amax = max |x|;  s = fp32(amax / 127);  inv = fp32(127 / amax);
#   c = rint(fp32(x * inv))  (round half to even), in [-127, 127];
#   a row whose amax is below 2^-100 (zeros among them) has s = 0 and codes
#   0, which keeps 127 / amax finite.  The row stands for c * s.
# --------------------------------------------------------------------------

def kv_int8_quantize(rows):
    """rows [..., dh] (values exact in fp32, e.g. bf16) -> (codes int8
    [..., dh], scales float32 [...])."""
    x = np.asarray(rows, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(x), axis=-1)
    zero = amax < np.float32(2.0 ** -100)
    safe = np.where(zero, np.float32(1), amax).astype(np.float32)
    inv = (np.float32(127) / safe).astype(np.float32)
    codes = np.rint((x * inv[..., None]).astype(np.float32))
    codes = np.clip(codes, -127, 127)
    codes = np.where(zero[..., None], 0, codes).astype(np.int8)
    scales = np.where(zero, np.float32(0), (safe / np.float32(127)).astype(np.float32)).astype(np.float32)
    return codes, scales


def kv_int8_dequantize(codes, scales):
    """codes int8 [..., dh], scales [...] -> the values they stand for (fp64)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def kv_int8_store(rows):
    """What the int8 cache holds for rows [..., dh]: dequantize(quantize(rows))."""
    return kv_int8_dequantize(*kv_int8_quantize(rows))


def decoder_layer_int8(x, positions, weights, k_codes, k_scales, v_codes, v_scales, **kw):
    """One layer call over an int8 cache: x [B, T, d] at positions [B, T]; the
    cache as codes [B, Hkv, S, dh] and scales [B, Hkv, S].  Each new token's
    key and value rows (bf16-rounded in the bf16 points mode, as the bf16
    cache would hold them) are quantized, row by row, into slot positions[b, t]
    before any query reads the cache; attention reads every visible slot,
    the new ones included, as c * s.  Other keywords as for decoder_layer
    (rows, bidirectional, kv_exact ...).  Returns (y [B, T, d], k_codes',
    k_scales', v_codes', v_scales')."""
    x = _f64(x)
    B, T, d = x.shape
    pos = np.asarray(_f64(positions), dtype=np.int64).reshape(B, T)
    kc = kv_int8_dequantize(k_codes, k_scales)
    vc = kv_int8_dequantize(v_codes, v_scales)
    new = {}

    def store(a):  # called for k, then v: a [B, Hkv, T, dh]
        key = "k" if "k" not in new else "v"
        new[key] = kv_int8_quantize(a)
        return kv_int8_dequantize(*new[key])
    y, _, _ = decoder_layer(x, pos, weights, kc, vc, kv_store=store, **kw)
    kq, ks = np.array(k_codes, dtype=np.int8), np.array(k_scales, dtype=np.float32)
    vq, vs = np.array(v_codes, dtype=np.int8), np.array(v_scales, dtype=np.float32)
    for b in range(B):
        kq[b][:, pos[b]], ks[b][:, pos[b]] = new["k"][0][b], new["k"][1][b]
        vq[b][:, pos[b]], vs[b][:, pos[b]] = new["v"][0][b], new["v"][1][b]
    return y, kq, ks, vq, vs


def decoder_layer_decode_int8(x, positions, weights, k_codes, k_scales, v_codes, v_scales, **kw):
    """One decode step over an int8 cache: x [B, d], positions [B] (the
    one-token case of decoder_layer_int8).  Returns (y [B, d], k_codes',
    k_scales', v_codes', v_scales')."""
    x = _f64(x)
    B, d = x.shape
    pos = np.asarray(_f64(positions), dtype=np.int64).reshape(B, 1)
    y, kq, ks, vq, vs = decoder_layer_int8(x.reshape(B, 1, d), pos, weights, k_codes, k_scales, v_codes,
                                           v_scales, **kw)
    return y.reshape(B, d), kq, ks, vq, vs


# --------------------------------------------------------------------------
# Paged KV cache  ["Llama MLP deep dive" §6.4 (PagedAttention named as the
# KV-memory lever); Notes Ch.04 (the cache as [layers, 2, B, T, Hkv, dh]
# memory that grows with context)]
# --------------------------------------------------------------------------

def gather_pages(pool, block_table, page_size, capacity):
    """The contiguous cache [B, Hkv, capacity, dh] a paged one stands for.

    pool [n_pages, Hkv, page_size, dh]; block_table [B, blocks_per_seq] of
    page ids: slot p of sequence b lives in page block_table[b, p // page_size]
    at row p % page_size.  capacity <= blocks_per_seq * page_size."""
    pool = _f64(pool)
    bt = np.asarray(block_table, dtype=np.int64)
    B, nblk = bt.shape
    n_pages, Hkv, ps, dh = pool.shape
    assert ps == page_size and capacity <= nblk * page_size
    out = np.zeros((B, Hkv, capacity, dh))
    for b in range(B):
        for p in range(capacity):
            out[b, :, p] = pool[bt[b, p // page_size], :, p % page_size]
    return out


def scatter_pages(cache, pool, block_table, page_size, slots):
    """Write slots[b] (a list of positions) of the contiguous cache [B, Hkv, S,
    dh] back into a copy of the page pool; returns the new pool."""
    pool = _f64(pool).copy()
    cache = _f64(cache)
    bt = np.asarray(block_table, dtype=np.int64)
    for b, ps_ in enumerate(slots):
        for p in ps_:
            pool[bt[b, p // page_size], :, p % page_size] = cache[b, :, p]
    return pool


def decoder_layer_paged(x, positions, weights, k_pool, v_pool, block_table, page_size, capacity, **kw):
    """The decoder layer over a paged cache: gather the pages into the
    contiguous layout, run decoder_layer, write the new tokens' slots back.
    Returns (y, k_pool', v_pool'); kv_exact (if given) as in decoder_layer."""
    x = _f64(x)
    pos = np.asarray(_f64(positions), dtype=np.int64).reshape(x.shape[0], x.shape[1])
    kc = gather_pages(k_pool, block_table, page_size, capacity)
    vc = gather_pages(v_pool, block_table, page_size, capacity)
    y, kc, vc = decoder_layer(x, pos, weights, kc, vc, **kw)
    slots = [list(pos[b]) for b in range(pos.shape[0])]
    return (y, scatter_pages(kc, k_pool, block_table, page_size, slots),
            scatter_pages(vc, v_pool, block_table, page_size, slots))


def decoder_layer_paged_int8(x, positions, weights, k_pool, k_scale_pool, v_pool, v_scale_pool, block_table,
                             page_size, capacity, **kw):
    """The int8 layer call over paged pools: codes [n_pages, Hkv, page, dh]
    and scales [n_pages, Hkv, page], slot p of sequence b in page
    block_table[b, p // page] at row p % page.  Gathers codes and scales into
    the contiguous int8 cache, runs decoder_layer_int8 there and writes the new
    tokens' slots back.  Returns (y, k_pool', k_scale_pool', v_pool',
    v_scale_pool')."""
    x = _f64(x)
    pos = np.asarray(_f64(positions), dtype=np.int64).reshape(x.shape[0], x.shape[1])

    def gather(pool, scale_pool):
        c = gather_pages(pool, block_table, page_size, capacity).astype(np.int8)
        s = gather_pages(np.asarray(scale_pool)[..., None], block_table, page_size, capacity)[..., 0]
        return c, s.astype(np.float32)
    kq, ks = gather(k_pool, k_scale_pool)
    vq, vs = gather(v_pool, v_scale_pool)
    y, kq, ks, vq, vs = decoder_layer_int8(x, pos, weights, kq, ks, vq, vs, **kw)
    slots = [list(pos[b]) for b in range(pos.shape[0])]

    def scatter(c, s, pool, scale_pool):
        cp = scatter_pages(c, pool, block_table, page_size, slots).astype(np.int8)
        sp = scatter_pages(s[..., None], np.asarray(scale_pool)[..., None], block_table, page_size, slots)[..., 0]
        return cp, sp.astype(np.float32)
    kp, ksp = scatter(kq, ks, k_pool, k_scale_pool)
    vp, vsp = scatter(vq, vs, v_pool, v_scale_pool)
    return y, kp, ksp, vp, vsp


def decoder_layer_decode(x, positions, weights, k_cache, v_cache, **kw):
    """One decode step: x [B, d], positions [B] (= each sequence's cache length).
    The same layer with T = 1; returns (y [B, d], k_cache', v_cache')."""
    x = _f64(x)
    B, d = x.shape
    pos = np.asarray(_f64(positions), dtype=np.int64).reshape(B, 1)
    y, kc, vc = decoder_layer(x.reshape(B, 1, d), pos, weights, k_cache, v_cache, **kw)
    return y.reshape(B, d), kc, vc
