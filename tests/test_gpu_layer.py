"""GPU parity of the HIP decoder layer against the CPU oracle at small shapes
that still span several tiles and ragged tails, plus edge cases and
properties.  Every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import synth
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

import llama_decoder_block_amd as lib  # noqa: E402  (fails loudly if the library is not built)

DEV = "cuda"


def _wl(name="small", dtype="bf16", d=512, H=4, Hkv=2, f=1408, B=2, T=300, prior=0, steps=0,
        seed=7):
    return synth.Workload(name, dtype, d, H, Hkv, 128 if dtype == "bf16" else d // H, f, B, T,
                          prior=prior, decode_steps=steps, seed=seed)


def _setup(wl, random_gains=False, max_tokens=None, bidirectional=False):
    w = synth.make_weights(wl, DEV, random_gains=random_gains)
    x = synth.make_x(wl, (wl.batch, wl.seq), device=DEV)
    kc, vc = synth.make_cache(wl, DEV)
    pos = synth.prefill_positions(wl.batch, wl.seq, start=wl.prior, device=DEV)
    layer = lib.LlamaLayer(G.layer_config(lib, wl, max_tokens or wl.batch * wl.seq,
                                          bidirectional=bidirectional), w)
    return w, x, kc, vc, pos, layer


def _check_prefill(wl, w, x, kc0, vc0, pos, y, kc, vc, bidirectional=False):
    torch.cuda.synchronize()
    w64 = G.oracle_weights(w)
    ex = {}
    yo, ko, vo = G.oracle_prefill(wl, w64, x, pos, kc0, vc0, bidirectional=bidirectional, kv_exact=ex)
    written = slice(wl.prior, wl.prior + wl.seq)
    kg, vg = G.f64(kc), G.f64(vc)
    if wl.dtype == "bf16":
        G.assert_bf16_output(G.f64(y), yo, "y")
        G.assert_bf16_cache(kg[:, :, written], ex["k"], ko[:, :, written], "K written")
        G.assert_bf16_cache(vg[:, :, written], ex["v"], vo[:, :, written], "V written")
        yp, _, _ = G.oracle_prefill(wl, w64, x, pos, kc0, vc0, bf16_points=False, bidirectional=bidirectional)
        print(f"  (vs plain oracle: y max|err|/rms = {G.rel_err(G.f64(y), yp):.5f})")
    else:
        G.assert_f32(G.f64(y), yo, "y")
        G.assert_f32(kg, ko, "K cache")
        G.assert_f32(vg, vo, "V cache")
    # slots this call did not write are untouched
    np.testing.assert_array_equal(kg[:, :, :wl.prior], G.f64(kc0)[:, :, :wl.prior])
    np.testing.assert_array_equal(kg[:, :, wl.prior + wl.seq:], G.f64(kc0)[:, :, wl.prior + wl.seq:])
    np.testing.assert_array_equal(vg[:, :, wl.prior + wl.seq:], G.f64(vc0)[:, :, wl.prior + wl.seq:])


def test_tiny_fp32_layer():
    """The tiny fp32 workload: B=1, T=16, d=64, 4 heads of 16, f=172."""
    wl = synth.WORKLOADS["tiny_f32"]
    print(f"case {wl}", flush=True)
    w, x, kc, vc, pos, layer = _setup(wl)
    kc0, vc0 = kc.clone(), vc.clone()
    y = layer.prefill(x, pos, kc, vc)
    _check_prefill(wl, w, x, kc0, vc0, pos, y, kc, vc)


@pytest.mark.parametrize("shape", [
    dict(d=512, H=4, Hkv=2, f=1408, B=2, T=300),      # tiled GEMMs, ragged M and query tile
    dict(d=512, H=4, Hkv=2, f=1536, B=2, T=300),      # 2f a multiple of 512: 128 x 512 gate/up tiles
    dict(d=384, H=3, Hkv=1, f=640, B=1, T=129),       # odd heads, MQA, N not a multiple of 256
    dict(d=256, H=2, Hkv=2, f=384, B=3, T=5),         # 15 tokens: weight-streaming GEMMs
    dict(d=1024, H=8, Hkv=2, f=2816, B=1, T=1),       # single token prefill
    dict(d=512, H=4, Hkv=4, f=1408, B=1, T=64),       # 64 tokens: two token blocks of weight streaming
    dict(d=512, H=4, Hkv=4, f=1408, B=1, T=65),       # 65 tokens: the four-block weight-streaming GEMMs
    dict(d=512, H=4, Hkv=2, f=1408, B=1, T=127),      # one short of four token blocks
    dict(d=1024, H=8, Hkv=2, f=2816, B=2, T=64),      # 128 tokens: the largest weight-streaming call
    dict(d=512, H=4, Hkv=4, f=1408, B=1, T=129),      # 129 tokens: the smallest tiled call (split K)
    dict(d=512, H=4, Hkv=1, f=1408, B=1, T=1000),     # long ragged sequence, MQA
])
def test_bf16_prefill_small(shape):
    wl = _wl(**shape)
    print(f"case {shape}", flush=True)
    w, x, kc, vc, pos, layer = _setup(wl, random_gains=True)
    kc0, vc0 = kc.clone(), vc.clone()
    y = layer.prefill(x, pos, kc, vc)
    _check_prefill(wl, w, x, kc0, vc0, pos, y, kc, vc)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunked_prefill_over_prior_cache(dtype):
    """Positions p0..p0+T-1 over a cache whose first p0 slots hold earlier K/V."""
    if dtype == "bf16":
        wl = _wl(dtype="bf16", d=512, H=4, Hkv=2, f=1408, B=2, T=100, prior=150)
    else:
        wl = _wl(dtype="f32", d=64, H=4, Hkv=2, f=96, B=2, T=7, prior=9)
    print(f"case {wl}", flush=True)
    w, x, kc, vc, pos, layer = _setup(wl)
    kc0, vc0 = kc.clone(), vc.clone()
    y = layer.prefill(x, pos, kc, vc)
    _check_prefill(wl, w, x, kc0, vc0, pos, y, kc, vc)


@pytest.mark.parametrize("dtype,T", [("bf16", 100), ("bf16", 20), ("f32", 9)])
def test_chunked_prefill_with_a_different_start_per_sequence(dtype, T):
    """Sequence 0 starts at position 0, sequence 1 continues its cache at 150
    (tiled and weight-streaming shapes): causal limits differ per sequence."""
    if dtype == "bf16":
        wl = _wl(dtype="bf16", d=512, H=4, Hkv=2, f=1408, B=2, T=T, prior=150, seed=37)
    else:
        wl = _wl(dtype="f32", d=64, H=4, Hkv=2, f=96, B=2, T=T, prior=150, seed=37)
    print(f"case {wl}", flush=True)
    w, x, kc, vc, _, layer = _setup(wl)
    pos = torch.stack([torch.arange(T), torch.arange(150, 150 + T)]).to(torch.int32).to(DEV)
    kc0, vc0 = kc.clone(), vc.clone()
    y = layer.prefill(x, pos, kc, vc)
    torch.cuda.synchronize()
    w64 = G.oracle_weights(w)
    ex = {}
    yo, ko, vo = G.oracle_prefill(wl, w64, x, pos, kc0, vc0, kv_exact=ex)
    kg, vg = G.f64(kc), G.f64(vc)
    if dtype == "bf16":
        G.assert_bf16_output(G.f64(y), yo, "y")
        for b, lo in ((0, 0), (1, 150)):
            G.assert_bf16_cache(kg[b, :, lo:lo + T], ex["k"][b], ko[b, :, lo:lo + T], f"K written, sequence {b}")
            G.assert_bf16_cache(vg[b, :, lo:lo + T], ex["v"][b], vo[b, :, lo:lo + T], f"V written, sequence {b}")
    else:
        G.assert_f32(G.f64(y), yo, "y")
        G.assert_f32(kg, ko, "K cache")
        G.assert_f32(vg, vo, "V cache")
    # slots the call did not write are untouched
    k0, v0 = G.f64(kc0), G.f64(vc0)
    for b, lo in ((0, 0), (1, 150)):
        np.testing.assert_array_equal(np.delete(kg[b], np.s_[lo:lo + T], axis=1), np.delete(k0[b], np.s_[lo:lo + T], axis=1))
        np.testing.assert_array_equal(np.delete(vg[b], np.s_[lo:lo + T], axis=1), np.delete(v0[b], np.s_[lo:lo + T], axis=1))


@pytest.mark.parametrize("shape", [
    dict(dtype="bf16", d=512, H=4, Hkv=2, f=1408, B=2, T=300),             # tiled GEMMs, ragged query tile
    dict(dtype="bf16", d=256, H=2, Hkv=2, f=384, B=3, T=5),                # weight-streaming GEMMs
    dict(dtype="bf16", d=512, H=4, Hkv=2, f=1408, B=2, T=100, prior=150),  # over a prior cache
    dict(dtype="f32", d=64, H=4, Hkv=2, f=96, B=2, T=7, prior=9),
])
def test_bidirectional_prefill(shape):
    """The encoder-style variant: every new token sees its sequence's slots up
    to the largest position in the call."""
    wl = _wl(**shape)
    print(f"case {shape}", flush=True)
    w, x, kc, vc, pos, layer = _setup(wl, random_gains=True, bidirectional=True)
    kc0, vc0 = kc.clone(), vc.clone()
    y = layer.prefill(x, pos, kc, vc)
    _check_prefill(wl, w, x, kc0, vc0, pos, y, kc, vc, bidirectional=True)


@pytest.mark.parametrize("bidirectional", [False, True])
def test_attention_with_several_workgroup_rounds(bidirectional):
    """576 query-tile workgroups (more than two per CU): the attention kernel
    with one wave group per tile, checked on sampled rows of every sequence."""
    wl = _wl(d=1024, H=8, Hkv=2, f=1408, B=8, T=1100, seed=9)
    print(f"case {wl} bidirectional={bidirectional}", flush=True)
    w, x, kc, vc, pos, layer = _setup(wl, bidirectional=bidirectional)
    kc0, vc0 = kc.clone(), vc.clone()
    y = layer.prefill(x, pos, kc, vc)
    torch.cuda.synchronize()
    rows = G.sample_rows(wl.batch, wl.seq, seed=3)
    yo, _, _ = G.oracle_prefill(wl, G.oracle_weights(w), x, pos, kc0, vc0, rows=rows,
                                bidirectional=bidirectional)
    G.assert_bf16_output(G.f64(y).reshape(-1, wl.d_model)[rows], yo.reshape(-1, wl.d_model)[rows], "y rows")


@pytest.mark.parametrize("shape", [
    # 8 query-tile workgroups: the kernel with two wave groups per tile; all rows checked
    # (slot 70 and 250 are tiles of the second group, 150 of the first)
    dict(d=512, H=4, Hkv=2, B=2, T=100, prior=300, slots=(70, 150, 250), rows=None),
    # 576 workgroups: one wave group per tile, several rounds; sampled rows
    dict(d=1024, H=8, Hkv=2, B=8, T=1100, prior=200, slots=(70, 100, 150), rows=5),
])
def test_planted_keys_move_the_reference_max(shape):
    """Keys of a prior cache scaled by 40, 40 and 4 at three slots past the
    first key tile: the scores against them reach hundreds, so many queries'
    maxima jump far past the value their weights were taken against when the
    tile arrives, and the attention output is then dominated by one value row
    (the causal softmax of the LMDrive page §2.3 with the notes' Ch.04 cache,
    evaluated by the oracle in fp64)."""
    wl = _wl(d=shape["d"], H=shape["H"], Hkv=shape["Hkv"], f=1408, B=shape["B"], T=shape["T"],
             prior=shape["prior"], seed=43)
    print(f"case {wl} planted slots {shape['slots']}", flush=True)
    w, x, kc, vc, pos, layer = _setup(wl)
    kf = kc.float()
    for slot, s in zip(shape["slots"], (40.0, 40.0, 4.0)):
        kf[:, :, slot] *= s
    kc.copy_(kf.to(kc.dtype))
    kc0, vc0 = kc.clone(), vc.clone()
    y = layer.prefill(x, pos, kc, vc)
    if shape["rows"] is None:
        _check_prefill(wl, w, x, kc0, vc0, pos, y, kc, vc)
        return
    torch.cuda.synchronize()
    rows = G.sample_rows(wl.batch, wl.seq, seed=shape["rows"])
    yo, _, _ = G.oracle_prefill(wl, G.oracle_weights(w), x, pos, kc0, vc0, rows=rows)
    G.assert_bf16_output(G.f64(y).reshape(-1, wl.d_model)[rows], yo.reshape(-1, wl.d_model)[rows], "y rows")


@pytest.mark.parametrize("B,H,Hkv", [(5, 4, 2), (1, 4, 1), (40, 4, 4),
                                     # query heads per kv head 3, 5, 6, 7: every decode
                                     # attention width below 8 (5 and up: one workgroup per CU)
                                     (3, 3, 1), (3, 10, 2), (2, 6, 1), (4, 14, 2)])
def test_bf16_decode_steps(B, H, Hkv):
    """Prefill 37 tokens, then 3 decode steps; each step checked against the
    oracle continuing from its own cache."""
    wl = _wl(d=512, H=H, Hkv=Hkv, f=1408, B=B, T=37, steps=3, seed=11)
    print(f"case B={B} H={H} Hkv={Hkv}", flush=True)
    w, x, kc, vc, pos, layer = _setup(wl, max_tokens=B * 37)
    w64 = G.oracle_weights(w)
    kc0, vc0 = kc.clone(), vc.clone()
    layer.prefill(x, pos, kc, vc)
    torch.cuda.synchronize()
    _, ko, vo = G.oracle_prefill(wl, w64, x, pos, kc0, vc0)
    from oracle import llama_oracle as O
    for s in range(wl.decode_steps):
        p = wl.seq + s
        xs = synth.make_x(wl, (B,), tensor_id=synth.TID_DECODE_BASE + s, device=DEV)
        ps = torch.full((B,), p, dtype=torch.int32, device=DEV)
        ys = layer.decode(xs, ps, kc, vc)
        torch.cuda.synchronize()
        ex = {}
        yo, ko, vo = O.decoder_layer_decode(G.f64(xs), np.full(B, p), w64, ko, vo,
                                            n_heads=wl.n_heads, n_kv_heads=wl.n_kv_heads,
                                            bf16_points=True, kv_exact=ex)
        G.assert_bf16_output(G.f64(ys), yo, f"decode step {s} y")
        G.assert_bf16_cache(G.f64(kc)[:, :, p], ex["k"][:, :, 0], ko[:, :, p], f"decode step {s} K")
        G.assert_bf16_cache(G.f64(vc)[:, :, p], ex["v"][:, :, 0], vo[:, :, p], f"decode step {s} V")


@pytest.mark.parametrize("shape", [
    # one GPU's share of the 70B layer under 8-way tensor parallelism: 8 query
    # heads and their one kv head (q width 1024 != d = 8192), f / 8 = 3584
    dict(d=8192, H=8, Hkv=1, f=3584, B=1, T=300),
    # the 13B layer's 4-way share: 10 heads, f / 4 = 3456
    dict(d=5120, H=10, Hkv=10, f=3456, B=2, T=200),
])
def test_tensor_parallel_shard_shapes(shape):
    """A layer whose projections are one GPU's tensor-parallel share (H dh
    below d): prefill (tiled GEMMs, ragged tiles), then 2 decode steps
    (weight-streaming GEMMs), each against the oracle at the same shape."""
    wl = _wl(d=shape["d"], H=shape["H"], Hkv=shape["Hkv"], f=shape["f"], B=shape["B"], T=shape["T"], steps=2,
             seed=19)
    print(f"case {shape}", flush=True)
    B = wl.batch
    w, x, kc, vc, pos, layer = _setup(wl, random_gains=True)
    kc0, vc0 = kc.clone(), vc.clone()
    y = layer.prefill(x, pos, kc, vc)
    _check_prefill(wl, w, x, kc0, vc0, pos, y, kc, vc)
    w64 = G.oracle_weights(w)
    _, ko, vo = G.oracle_prefill(wl, w64, x, pos, kc0, vc0)
    from oracle import llama_oracle as O
    for s in range(wl.decode_steps):
        p = wl.seq + s
        xs = synth.make_x(wl, (B,), tensor_id=synth.TID_DECODE_BASE + s, device=DEV)
        ps = torch.full((B,), p, dtype=torch.int32, device=DEV)
        ys = layer.decode(xs, ps, kc, vc)
        torch.cuda.synchronize()
        yo, ko, vo = O.decoder_layer_decode(G.f64(xs), np.full(B, p), w64, ko, vo, n_heads=wl.n_heads,
                                            n_kv_heads=wl.n_kv_heads, bf16_points=True)
        G.assert_bf16_output(G.f64(ys), yo, f"decode step {s} y")
    layer.close()


@pytest.mark.parametrize("dtype,H,Hkv", [("bf16", 4, 2), ("bf16", 4, 4), ("f32", 4, 2),
                                          # 3 .. 8 query heads per kv head: every width of
                                          # the decode attention kernel over several of its
                                          # loop iterations (the prefetch hand-off)
                                          ("bf16", 6, 2), ("bf16", 8, 2), ("bf16", 10, 2),
                                          ("bf16", 12, 2), ("bf16", 14, 2), ("bf16", 16, 2)])
def test_decode_with_ragged_cache_lengths(dtype, H, Hkv):
    """One decode step where every sequence sits at a different position over a
    random prior cache of 2048 slots (continuous batching): the short
    sequences leave most split-K ranges of the attention empty."""
    from oracle import llama_oracle as O
    if dtype == "bf16":
        wl = _wl(d=128 * H, H=H, Hkv=Hkv, f=1408, B=6, T=1, prior=2047, seed=31 + H)
    else:
        wl = _wl(dtype="f32", d=64, H=H, Hkv=Hkv, f=96, B=6, T=1, prior=2047, seed=31)
    print(f"case {dtype} H={H} Hkv={Hkv} max_pos={wl.max_pos}", flush=True)
    w = synth.make_weights(wl, DEV, random_gains=True)
    kc, vc = synth.make_cache(wl, DEV)
    layer = lib.LlamaLayer(G.layer_config(lib, wl, wl.batch), w)
    w64 = G.oracle_weights(w)
    k64, v64 = G.f64(kc), G.f64(vc)
    p = np.array([0, 5, 100, 1000, 2047, 1531])
    xs = synth.make_x(wl, (wl.batch,), tensor_id=synth.TID_DECODE_BASE, device=DEV)
    ys = layer.decode(xs, torch.tensor(p, dtype=torch.int32, device=DEV), kc, vc)
    torch.cuda.synchronize()
    ex = {}
    yo, ko, vo = O.decoder_layer_decode(G.f64(xs), p, w64, k64, v64, n_heads=wl.n_heads,
                                        n_kv_heads=wl.n_kv_heads, bf16_points=dtype == "bf16", kv_exact=ex)
    kg, vg = G.f64(kc), G.f64(vc)
    bi = np.arange(wl.batch)
    if dtype == "bf16":
        G.assert_bf16_output(G.f64(ys), yo, "ragged decode y")
        G.assert_bf16_cache(kg[bi, :, p], ex["k"][:, :, 0], ko[bi, :, p], "K of every sequence")
        G.assert_bf16_cache(vg[bi, :, p], ex["v"][:, :, 0], vo[bi, :, p], "V of every sequence")
    else:
        G.assert_f32(G.f64(ys), yo, "ragged decode y")
        for b in range(wl.batch):
            G.assert_f32(kg[b, :, p[b]], ko[b, :, p[b]], f"K of sequence {b}")
            G.assert_f32(vg[b, :, p[b]], vo[b, :, p[b]], f"V of sequence {b}")
    # every other cache slot is untouched
    kg[np.arange(wl.batch), :, p] = k64[np.arange(wl.batch), :, p]
    vg[np.arange(wl.batch), :, p] = v64[np.arange(wl.batch), :, p]
    assert np.array_equal(kg, k64) and np.array_equal(vg, v64)


@pytest.mark.parametrize("B", [3, 40, 64])
def test_decode_gate_up_wider_than_the_grid(B):
    """f = 8704: the gate/up projection has 272 column groups, more than the
    CUs, so each workgroup of the weight-streaming GEMM streams a share that
    spans parts of several groups (one or two 32-token blocks)."""
    from oracle import llama_oracle as O
    wl = _wl(d=512, H=4, Hkv=2, f=8704, B=B, T=9, steps=2, seed=29)
    print(f"case B={B}", flush=True)
    w, x, kc, vc, pos, layer = _setup(wl, random_gains=True, max_tokens=B * 9)
    w64 = G.oracle_weights(w)
    kc0, vc0 = kc.clone(), vc.clone()
    layer.prefill(x, pos, kc, vc)
    torch.cuda.synchronize()
    _, ko, vo = G.oracle_prefill(wl, w64, x, pos, kc0, vc0)
    for s in range(wl.decode_steps):
        p = wl.seq + s
        xs = synth.make_x(wl, (B,), tensor_id=synth.TID_DECODE_BASE + s, device=DEV)
        ys = layer.decode(xs, torch.full((B,), p, dtype=torch.int32, device=DEV), kc, vc)
        torch.cuda.synchronize()
        yo, ko, vo = O.decoder_layer_decode(G.f64(xs), np.full(B, p), w64, ko, vo, n_heads=wl.n_heads,
                                            n_kv_heads=wl.n_kv_heads, bf16_points=True)
        G.assert_bf16_output(G.f64(ys), yo, f"decode step {s} y")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_with_wide_rows(dtype):
    """d = 2048: the calls of <= 64 rows normalise each row with a whole
    workgroup (a separate RMSNorm kernel from the one-wave-per-row one)."""
    from oracle import llama_oracle as O
    wl = _wl(dtype=dtype, d=2048, H=16, Hkv=4, f=5632, B=3, T=20, steps=2, seed=23)
    print(f"case {dtype}", flush=True)
    w, x, kc, vc, pos, layer = _setup(wl, random_gains=True, max_tokens=3 * 20)
    w64 = G.oracle_weights(w)
    kc0, vc0 = kc.clone(), vc.clone()
    layer.prefill(x, pos, kc, vc)
    torch.cuda.synchronize()
    _, ko, vo = G.oracle_prefill(wl, w64, x, pos, kc0, vc0)
    for s in range(wl.decode_steps):
        p = wl.seq + s
        xs = synth.make_x(wl, (wl.batch,), tensor_id=synth.TID_DECODE_BASE + s, device=DEV)
        ys = layer.decode(xs, torch.full((wl.batch,), p, dtype=torch.int32, device=DEV), kc, vc)
        torch.cuda.synchronize()
        yo, ko, vo = O.decoder_layer_decode(G.f64(xs), np.full(wl.batch, p), w64, ko, vo, n_heads=wl.n_heads,
                                            n_kv_heads=wl.n_kv_heads, bf16_points=dtype == "bf16")
        if dtype == "bf16":
            G.assert_bf16_output(G.f64(ys), yo, f"decode step {s} y")
        else:
            G.assert_f32(G.f64(ys), yo, f"decode step {s} y")


@pytest.mark.parametrize("d", [3072, 5120])
def test_rmsnorm_row_widths(d):
    """Widths that take the RMSNorm kernels with 2 wavefronts per row
    (prefill rows: d/1024 = 3 or 5 vectors per lane) and, for decode rows,
    2 (d = 3072) or d/512 = 10 (d = 5120) wavefronts per row: a prefill of 70
    tokens (tiled GEMMs) and two single-sequence decode steps against the
    oracle."""
    from oracle import llama_oracle as O
    wl = _wl(d=d, H=d // 128, Hkv=8, f=1024, B=1, T=70, steps=2, seed=31 + d // 1024)
    print(f"case d={d}", flush=True)
    w, x, kc, vc, pos, layer = _setup(wl, random_gains=True)
    kc0, vc0 = kc.clone(), vc.clone()
    y = layer.prefill(x, pos, kc, vc)
    _check_prefill(wl, w, x, kc0, vc0, pos, y, kc, vc)
    w64 = G.oracle_weights(w)
    _, ko, vo = G.oracle_prefill(wl, w64, x, pos, kc0, vc0)  # the oracle continues from its own cache
    for s in range(wl.decode_steps):
        p = wl.seq + s
        xs = synth.make_x(wl, (wl.batch,), tensor_id=synth.TID_DECODE_BASE + s, device=DEV)
        ys = layer.decode(xs, torch.full((wl.batch,), p, dtype=torch.int32, device=DEV), kc, vc)
        torch.cuda.synchronize()
        yo, ko, vo = O.decoder_layer_decode(G.f64(xs), np.full(wl.batch, p), w64, ko, vo, n_heads=wl.n_heads,
                                            n_kv_heads=wl.n_kv_heads, bf16_points=True)
        G.assert_bf16_output(G.f64(ys), yo, f"d={d} decode step {s} y")
    layer.close()


def test_decode_matches_prefill_of_one_more_token():
    """Prefill T, decode token T == row T of a prefill of T+1 (within bf16)."""
    wl = _wl(d=512, H=4, Hkv=2, f=1408, B=2, T=81, seed=13)
    w = synth.make_weights(wl, DEV)
    x = synth.make_x(wl, (2, 82), device=DEV)
    cfg = G.layer_config(lib, wl, max_tokens=2 * 82, max_pos=82)
    layer = lib.LlamaLayer(cfg, w)
    kc1 = torch.zeros((2, 2, 82, 128), dtype=torch.bfloat16, device=DEV)
    vc1 = torch.zeros_like(kc1)
    y_full = layer.prefill(x, synth.prefill_positions(2, 82, device=DEV), kc1, vc1)
    kc2, vc2 = torch.zeros_like(kc1), torch.zeros_like(kc1)
    layer.prefill(x[:, :81].contiguous(), synth.prefill_positions(2, 81, device=DEV), kc2, vc2)
    y_dec = layer.decode(x[:, 81].contiguous(), torch.full((2,), 81, dtype=torch.int32, device=DEV),
                         kc2, vc2)
    torch.cuda.synchronize()
    G.assert_bf16_output(G.f64(y_dec), G.f64(y_full[:, 81]), "decode vs prefill row")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_extreme_inputs(dtype):
    """Rows of zeros, rows scaled by 1e-3 and by 1e3, and a sharp softmax (the
    query and key weights scaled so the scores have a standard deviation near
    10, which moves the attention's reference max often): a prefill over
    several key tiles, then one decode step with extreme rows.  Each row
    group is checked on its own scale (RMSNorm makes the layer's work scale
    free, so a row scaled by s is held to s times the unit-scale gate)."""
    from oracle import llama_oracle as O
    if dtype == "bf16":
        wl, sharpen = _wl(d=512, H=4, Hkv=2, f=1408, B=2, T=130, steps=1, seed=21), 7.0
    else:
        wl, sharpen = _wl(dtype="f32", d=64, H=4, Hkv=2, f=96, B=2, T=20, steps=1, seed=21), 20.0
    print(f"case {dtype}", flush=True)
    w = synth.make_weights(wl, DEV, random_gains=True)
    for name in ("wq", "wk"):
        w[name] = (w[name].float() * sharpen).to(w[name].dtype)
    x = synth.make_x(wl, (wl.batch, wl.seq), device=DEV).float()
    groups = {"zero": [(0, 5), (1, 0)], "x1e-3": [(0, 6), (0, 7), (0, 8)], "x1e3": [(1, 10), (1, 11), (1, 12)]}
    for b, t in groups["zero"]:
        x[b, t] = 0.0
    for b, t in groups["x1e-3"]:
        x[b, t] *= 1e-3
    for b, t in groups["x1e3"]:
        x[b, t] *= 1e3
    x = x.to(synth.torch_dtype(wl))
    special = {bt for v in groups.values() for bt in v}
    groups["unscaled"] = [(b, t) for b in range(wl.batch) for t in range(wl.seq) if (b, t) not in special]
    scale = {"zero": 1.0, "x1e-3": 1.0, "x1e3": 1e3, "unscaled": 1.0}
    kc, vc = synth.make_cache(wl, DEV)
    pos = synth.prefill_positions(wl.batch, wl.seq, device=DEV)
    layer = lib.LlamaLayer(G.layer_config(lib, wl, wl.batch * wl.seq), w)
    kc0, vc0 = kc.clone(), vc.clone()
    y = layer.prefill(x, pos, kc, vc)
    torch.cuda.synchronize()
    w64 = G.oracle_weights(w)
    ex = {}
    yo, ko, vo = G.oracle_prefill(wl, w64, x, pos, kc0, vc0, kv_exact=ex)
    yg = G.f64(y)

    def check(got, ref, what, s):
        if dtype == "bf16":
            G.assert_bf16_output(got / s, ref / s, what)
        else:
            G.assert_f32(got / s, ref / s, what)
    # a zero row at position 0 sees only itself, whose key and value are
    # zero: every step maps zeros to zeros, so its y is exactly zero on both
    # sides (it is checked on its own, as its RMS is zero)
    assert np.all(yo[1, 0] == 0.0) and np.all(yg[1, 0] == 0.0)
    groups["zero"] = [(0, 5)]
    for name, rows in groups.items():
        idx = tuple(np.array(rows).T)
        check(yg[idx], yo[idx], f"y, {name} rows", scale[name])
    written = slice(0, wl.seq)
    # the scores' spread the sharpening reaches (sequence 0, head 0, unscaled rows)
    q0 = G.f64(x)[0, 9:40] @ G.f64(w["wq"])[:wl.head_dim].T
    k0 = G.f64(x)[0, 9:40] @ G.f64(w["wk"])[:wl.head_dim].T
    print(f"  score std ~ {np.std(q0 @ k0.T) / np.sqrt(wl.head_dim):.1f}", flush=True)
    if dtype == "bf16":
        G.assert_bf16_cache(G.f64(kc)[:, :, written], ex["k"], ko[:, :, written], "K written")
        G.assert_bf16_cache(G.f64(vc)[:, :, written], ex["v"], vo[:, :, written], "V written")
    else:
        G.assert_f32(G.f64(kc), ko, "K cache")
        G.assert_f32(G.f64(vc), vo, "V cache")
    # a decode step with a zero row and a 1e3-scaled row
    xs = synth.make_x(wl, (wl.batch,), tensor_id=synth.TID_DECODE_BASE, device=DEV).float()
    xs[0] = 0.0
    xs[1] *= 1e3
    xs = xs.to(synth.torch_dtype(wl))
    p = wl.seq
    ys = layer.decode(xs, torch.full((wl.batch,), p, dtype=torch.int32, device=DEV), kc, vc)
    torch.cuda.synchronize()
    yo_d, ko_d, vo_d = O.decoder_layer_decode(G.f64(xs), np.full(wl.batch, p), w64, ko, vo, n_heads=wl.n_heads,
                                              n_kv_heads=wl.n_kv_heads, bf16_points=dtype == "bf16")
    check(G.f64(ys)[0], yo_d[0], "decode y, zero row", 1.0)
    check(G.f64(ys)[1], yo_d[1], "decode y, 1e3 row", 1e3)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_output_projections_give_identity(dtype):
    wl = _wl(dtype=dtype, d=256 if dtype == "bf16" else 64, H=2 if dtype == "bf16" else 4, Hkv=2,
             f=384 if dtype == "bf16" else 96, B=2, T=70)
    w = synth.make_weights(wl, DEV)
    w["wo"].zero_()
    w["w_down"].zero_()
    x = synth.make_x(wl, (2, 70), device=DEV)
    kc, vc = synth.make_cache(wl, DEV)
    layer = lib.LlamaLayer(G.layer_config(lib, wl, 140), w)
    y = layer.prefill(x, synth.prefill_positions(2, 70, device=DEV), kc, vc)
    torch.cuda.synchronize()
    assert torch.equal(y, x)


def test_gqa_equals_mha_with_repeated_kv_weights():
    """GQA with Hkv=2 computes what MHA computes when each kv head's weights
    are repeated for its group of query heads."""
    wl = _wl(d=512, H=4, Hkv=2, f=1408, B=1, T=200, seed=17)
    w = synth.make_weights(wl, DEV)
    x = synth.make_x(wl, (1, 200), device=DEV)
    pos = synth.prefill_positions(1, 200, device=DEV)
    kc, vc = synth.make_cache(wl, DEV)
    y_gqa = lib.LlamaLayer(G.layer_config(lib, wl, 200), w).prefill(x, pos, kc, vc)
    wl_mha = synth.scaled(wl, n_kv_heads=4)
    w_mha = dict(w)
    w_mha["wk"] = w["wk"].view(2, 128, 512).repeat_interleave(2, dim=0).reshape(512, 512).contiguous()
    w_mha["wv"] = w["wv"].view(2, 128, 512).repeat_interleave(2, dim=0).reshape(512, 512).contiguous()
    kc2, vc2 = synth.make_cache(wl_mha, DEV)
    y_mha = lib.LlamaLayer(G.layer_config(lib, wl_mha, 200), w_mha).prefill(x, pos, kc2, vc2)
    torch.cuda.synchronize()
    assert torch.equal(y_gqa, y_mha)
    assert torch.equal(kc2[:, 0::2], kc) and torch.equal(kc2[:, 1::2], kc)


def test_bitwise_deterministic():
    wl = _wl(d=512, H=4, Hkv=2, f=1408, B=2, T=300, seed=19)
    w, x, kc, vc, pos, layer = _setup(wl)
    y1 = layer.prefill(x, pos, kc, vc).clone()
    k1 = kc.clone()
    y2 = layer.prefill(x, pos, kc, vc)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(k1, kc)


def test_in_place_output():
    wl = _wl(d=512, H=4, Hkv=2, f=1408, B=1, T=90, seed=23)
    w, x, kc, vc, pos, layer = _setup(wl)
    y = layer.prefill(x, pos, kc, vc)
    x2 = x.clone()
    kc.zero_(); vc.zero_()
    layer.prefill(x2, pos, kc, vc, y=x2)
    torch.cuda.synchronize()
    assert torch.equal(x2, y)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_position_check_mode(dtype, monkeypatch):
    """LLAMA_LAYER_CHECK=1 at creation: calls with a position outside [0, max_pos)
    or repeated within a sequence fail with INVALID before touching the cache;
    valid calls give the same bits as a handle without the check."""
    wl = _wl(dtype=dtype, d=256 if dtype == "bf16" else 64, H=2, Hkv=2, f=384 if dtype == "bf16" else 96,
             B=2, T=8, steps=1)
    print(f"case {wl}", flush=True)
    w, x, kc, vc, pos, plain = _setup(wl)
    monkeypatch.setenv("LLAMA_LAYER_CHECK", "1")
    checked = lib.LlamaLayer(G.layer_config(lib, wl, wl.batch * wl.seq), w)
    kc2, vc2 = kc.clone(), vc.clone()
    y1 = plain.prefill(x, pos, kc, vc)
    y2 = checked.prefill(x, pos, kc2, vc2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(kc, kc2) and torch.equal(vc, vc2)
    flat = pos.reshape(-1)
    bad_cases = {"outside": (5, wl.max_pos), "negative": (9, -1), "repeats": (12, int(flat[10]))}
    for what, (i, v) in bad_cases.items():
        bad = pos.clone()
        bad.view(-1)[i] = v
        k0, v0 = kc2.clone(), vc2.clone()
        with pytest.raises(lib.LlamaLayerError) as e:
            checked.prefill(x, bad, kc2, vc2)
        assert e.value.status == lib.LLAMA_ERR_INVALID, what
        assert torch.equal(kc2, k0) and torch.equal(vc2, v0), what
    # decode: one position per sequence
    xd = synth.make_x(wl, (wl.batch,), tensor_id=100, device=DEV)
    with pytest.raises(lib.LlamaLayerError) as e:
        checked.decode(xd, torch.tensor([3, wl.max_pos], dtype=torch.int32, device=DEV), kc2, vc2)
    assert e.value.status == lib.LLAMA_ERR_INVALID
    checked.decode(xd, torch.tensor([wl.seq, wl.seq], dtype=torch.int32, device=DEV), kc2, vc2)
    torch.cuda.synchronize()


def test_capacity_and_alignment_errors():
    wl = _wl(d=256, H=2, Hkv=2, f=384, B=1, T=8)
    w, x, kc, vc, pos, layer = _setup(wl, max_tokens=8)
    big = synth.make_x(wl, (2, 8), device=DEV)
    with pytest.raises(lib.LlamaLayerError) as e:
        layer.prefill(big, synth.prefill_positions(2, 8, device=DEV), kc, vc)
    assert e.value.status == lib.LLAMA_ERR_CAPACITY
    flat = torch.zeros(8 * 256 + 1, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(lib.LlamaLayerError) as e:
        lib.llama_layer_prefill(layer.handle, x, flat[1:], pos, 1, 8, kc, vc)
    assert e.value.status == lib.LLAMA_ERR_INVALID
