"""The paged KV cache through the C ABI: parity with the oracle's paged layer
(gather pages, run the layer, scatter the new slots) and bit-identity with
the contiguous calls on the cache the pages stand for, with shuffled block
tables, at small shapes (tiled and weight-streaming paths, both attention
kernels) and at the full 7B decode and 70B prefill + 64 decode workloads."""
import numpy as np
import pytest
import torch

import llama_decoder_block_amd as lib
import synth
from oracle import llama_oracle as O
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu
DEV = "cuda"


def to_pages(kc, page, seed, spare=3):
    """Scatter a contiguous cache [B, Hkv, S, dh] (S a multiple of page) into a
    shuffled page pool with `spare` unmapped pages; returns (pool, block_table)."""
    B, Hkv, S, dh = kc.shape
    nb = S // page
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(B * nb + spare, generator=g)
    bt = perm[:B * nb].view(B, nb).to(torch.int32)
    pool = torch.zeros(B * nb + spare, Hkv, page, dh, dtype=kc.dtype, device=kc.device)
    for b in range(B):
        for i in range(nb):
            pool[int(bt[b, i])] = kc[b, :, i * page:(i + 1) * page]
    return pool, bt.to(kc.device)


def from_pages(pool, bt, page):
    B, nb = bt.shape
    idx = bt.long()
    return torch.stack([torch.cat([pool[int(idx[b, i])] for i in range(nb)], dim=1) for b in range(B)])


def _same(a, b):
    return int((a.view(torch.int16) != b.view(torch.int16)).sum())


@pytest.mark.parametrize("shape", [
    dict(d=512, H=4, Hkv=2, f=1408, B=2, T=300, prior=212, page=64),    # tiled GEMMs, 8-wave attention
    dict(d=256, H=2, Hkv=2, f=384, B=3, T=5, prior=123, page=128),      # weight-streaming GEMMs, pages of 128
    dict(d=1024, H=8, Hkv=2, f=1408, B=8, T=300, prior=212, page=64),   # 4-wave attention kernel, rounds
])
def test_paged_prefill_then_decode(shape):
    page = shape["page"]
    wl = synth.Workload("paged", "bf16", shape["d"], shape["H"], shape["Hkv"], 128, shape["f"], shape["B"], shape["T"],
                        prior=shape["prior"], decode_steps=1, seed=41)
    cap = -(-wl.max_pos // page) * page                   # whole pages
    print(f"case {shape} capacity {cap}", flush=True)
    B, T = wl.batch, wl.seq
    w = synth.make_weights(wl, DEV, random_gains=True)
    x = synth.make_x(wl, (B, T), device=DEV)
    kc, vc = synth.make_cache(wl, DEV)
    kc = torch.nn.functional.pad(kc, (0, 0, 0, cap - wl.max_pos)).contiguous()
    vc = torch.nn.functional.pad(vc, (0, 0, 0, cap - wl.max_pos)).contiguous()
    kp, bt = to_pages(kc, page, seed=1)
    vp, _ = to_pages(vc, page, seed=1)
    kp0, vp0 = kp.clone(), vp.clone()
    pos = synth.prefill_positions(B, T, start=wl.prior, device=DEV)
    cfg = G.layer_config(lib, wl, B * T, max_pos=cap)
    layer = lib.LlamaLayer(cfg, w)
    y = layer.prefill_paged(x, pos, kp, vp, bt)
    yc = layer.prefill(x, pos, kc, vc)                     # contiguous, same cache
    torch.cuda.synchronize()
    assert _same(y, yc) == 0
    assert _same(from_pages(kp, bt, page), kc) == 0 and _same(from_pages(vp, bt, page), vc) == 0
    spare = sorted(set(range(kp.shape[0])) - set(bt.view(-1).tolist()))
    assert torch.equal(kp[spare], kp0[spare]) and torch.equal(vp[spare], vp0[spare])  # unmapped pages untouched
    # against the oracle's paged layer
    w64 = G.oracle_weights(w)
    ex = {}
    yo, kpo, vpo = O.decoder_layer_paged(G.f64(x), G.f64(pos), w64, G.f64(kp0), G.f64(vp0), bt.cpu().numpy(), page,
                                         cap, n_heads=wl.n_heads, n_kv_heads=wl.n_kv_heads, bf16_points=True,
                                         kv_exact=ex)
    G.assert_bf16_output(G.f64(y), yo, "paged prefill y")
    new = slice(wl.prior, wl.prior + T)
    ko = O.gather_pages(kpo, bt.cpu().numpy(), page, cap)
    G.assert_bf16_cache(G.f64(from_pages(kp, bt, page))[:, :, new], ex["k"], ko[:, :, new], "paged K written")
    # one decode step at ragged positions
    xd = synth.make_x(wl, (B,), tensor_id=synth.TID_DECODE_BASE, device=DEV)
    pd = torch.tensor([wl.prior + T - (37 * b) % 50 for b in range(B)], dtype=torch.int32, device=DEV)
    kd, vd = kp.clone(), vp.clone()
    yd = layer.decode_paged(xd, pd, kd, vd, bt)
    kdc, vdc = kc.clone(), vc.clone()
    ydc = layer.decode(xd, pd, kdc, vdc)
    torch.cuda.synchronize()
    assert _same(yd, ydc) == 0 and _same(from_pages(kd, bt, page), kdc) == 0
    # the oracle continues from its own pools
    ydo, _, _ = O.decoder_layer_paged(G.f64(xd)[:, None], G.f64(pd)[:, None], w64, kpo, vpo,
                                      bt.cpu().numpy(), page, cap, n_heads=wl.n_heads, n_kv_heads=wl.n_kv_heads,
                                      bf16_points=True)
    G.assert_bf16_output(G.f64(yd), ydo[:, 0], "paged decode y")
    layer.close()


def test_paged_position_check_rejects_bad_pages(monkeypatch):
    """LLAMA_LAYER_CHECK=1: a block table entry outside [0, n_pages) in a page
    a token uses, or a position beyond the paged capacity, fails with INVALID
    before anything is written."""
    wl = synth.Workload("pc", "bf16", 256, 2, 2, 128, 384, 2, 8, prior=0, decode_steps=1, seed=5)
    monkeypatch.setenv("LLAMA_LAYER_CHECK", "1")
    layer = lib.LlamaLayer(G.layer_config(lib, wl, 16, max_pos=256), synth.make_weights(wl, DEV))
    kc = torch.zeros(2, 2, 256, 128, dtype=torch.bfloat16, device=DEV)
    kp, bt = to_pages(kc, 64, seed=2)
    vp = kp.clone()
    x = synth.make_x(wl, (2, 8), device=DEV)
    pos = synth.prefill_positions(2, 8, device=DEV)
    layer.prefill_paged(x, pos, kp, vp, bt)
    torch.cuda.synchronize()
    bad = bt.clone()
    bad[1, 0] = kp.shape[0]
    k0 = kp.clone()
    with pytest.raises(lib.LlamaLayerError) as e:
        layer.prefill_paged(x, pos, kp, vp, bad)
    assert e.value.status == lib.LLAMA_ERR_INVALID and torch.equal(kp, k0)
    with pytest.raises(lib.LlamaLayerError) as e:   # one page per sequence holds 64 slots
        layer.decode_paged(x[:, 0].contiguous(), torch.tensor([64, 3], dtype=torch.int32, device=DEV), kp, vp,
                           bt[:, :1].contiguous())
    assert e.value.status == lib.LLAMA_ERR_INVALID
    for kw, status in ((dict(page_size=100), lib.LLAMA_ERR_INVALID), (dict(page_size=0), lib.LLAMA_ERR_INVALID)):
        with pytest.raises(lib.LlamaLayerError) as e:
            lib.llama_layer_prefill_paged(layer.handle, x, torch.empty_like(x), pos, 2, 8, kp, vp, bt, kw["page_size"])
        assert e.value.status == status


@pytest.mark.slow
def test_paged_llama7b_decode_is_bit_identical():
    """The 7B decode workload (32 sequences at position 4095) on pages of 64
    slots shuffled over the pool: y and the appended slots bit-identical to
    the contiguous call."""
    wl = synth.WORKLOADS["llama7b_decode"]
    B, p = wl.batch, wl.prior
    w = synth.make_weights(wl, DEV)
    x = synth.make_x(wl, (B,), device=DEV)
    kc, vc = synth.make_cache(wl, DEV)
    kp, bt = to_pages(kc, 64, seed=3)
    vp, _ = to_pages(vc, 64, seed=3)
    pos = torch.full((B,), p, dtype=torch.int32, device=DEV)
    layer = lib.LlamaLayer(G.layer_config(lib, wl, B), w)
    yc = layer.decode(x, pos, kc, vc)
    yp = layer.decode_paged(x, pos, kp, vp, bt)
    torch.cuda.synchronize()
    print(f"  y: {_same(yp, yc)} elements differ", flush=True)
    assert _same(yp, yc) == 0
    assert _same(from_pages(kp, bt, 64), kc) == 0 and _same(from_pages(vp, bt, 64), vc) == 0


@pytest.mark.slow
def test_paged_llama70b_prefill_and_64_decode_steps_are_bit_identical():
    """The 70B GQA workload: a 4096-token prefill, then 64 decode steps, over
    65 pages of 64 slots in shuffled order, bit-identical to the contiguous
    calls at every step."""
    wl = synth.WORKLOADS["llama70b_gqa"]
    T = wl.seq
    w = synth.make_weights(wl, DEV)
    x = synth.make_x(wl, (1, T), device=DEV)
    kc, vc = synth.make_cache(wl, DEV)
    kp, bt = to_pages(kc, 64, seed=4, spare=5)
    vp, _ = to_pages(vc, 64, seed=4, spare=5)
    pos = synth.prefill_positions(1, T, device=DEV)
    layer = lib.LlamaLayer(G.layer_config(lib, wl, T), w)
    yc = layer.prefill(x, pos, kc, vc)
    yp = layer.prefill_paged(x, pos, kp, vp, bt)
    torch.cuda.synchronize()
    assert _same(yp, yc) == 0, "prefill"
    for s in range(wl.decode_steps):
        xs = synth.make_x(wl, (1,), tensor_id=synth.TID_DECODE_BASE + s, device=DEV)
        ps = torch.full((1,), T + s, dtype=torch.int32, device=DEV)
        a = layer.decode(xs, ps, kc, vc)
        b = layer.decode_paged(xs, ps, kp, vp, bt)
        torch.cuda.synchronize()
        assert _same(a, b) == 0, f"decode step {s}"
    assert _same(from_pages(kp, bt, 64), kc) == 0 and _same(from_pages(vp, bt, 64), vc) == 0
    print("  prefill and 64 decode steps bit-identical", flush=True)


@pytest.mark.parametrize("shape", [
    dict(d=512, H=4, Hkv=2, f=1408, B=2, T=300, prior=212, page=64),    # tiled GEMMs, 8-wave attention
    dict(d=256, H=2, Hkv=2, f=384, B=3, T=5, prior=123, page=128),      # weight-streaming GEMMs, pages of 128
    dict(d=1024, H=8, Hkv=2, f=1408, B=8, T=300, prior=212, page=64),   # 4-wave attention kernel, rounds
])
def test_paged_int8_prefill_then_decode(shape):
    """int8 page pools (codes and per-row scales, shuffled table, spare pages):
    a prefill over converted prior rows, then a decode step at ragged
    positions, bit-identical to the contiguous int8 calls on the cache the
    pages stand for, unmapped pages untouched, and y against the oracle's
    paged int8 call at the 0.02 x RMS gate."""
    page = shape["page"]
    wl = synth.Workload("paged8", "bf16", shape["d"], shape["H"], shape["Hkv"], 128, shape["f"], shape["B"],
                        shape["T"], prior=shape["prior"], decode_steps=1, seed=43)
    cap = -(-wl.max_pos // page) * page
    print(f"case {shape} capacity {cap}", flush=True)
    B, T = wl.batch, wl.seq
    w = synth.make_weights(wl, DEV, random_gains=True)
    x = synth.make_x(wl, (B, T), device=DEV)
    kc, vc = synth.make_cache(wl, DEV)
    kc = torch.nn.functional.pad(kc, (0, 0, 0, cap - wl.max_pos)).contiguous()
    vc = torch.nn.functional.pad(vc, (0, 0, 0, cap - wl.max_pos)).contiguous()
    cfg = G.layer_config(lib, wl, B * T, max_pos=cap)
    layer = lib.LlamaLayer(cfg, w)
    kq = torch.empty(kc.shape, dtype=torch.int8, device=DEV)
    vq = torch.empty_like(kq)
    ks = torch.empty(kc.shape[:3], dtype=torch.float32, device=DEV)
    vs = torch.empty_like(ks)
    layer.kv_quantize(kc, vc, cap, kq, vq, ks, vs)
    torch.cuda.synchronize()

    def pages(t):  # scales [B, Hkv, cap] ride as rows of one element
        pool, bt = to_pages(t if t.dim() == 4 else t.unsqueeze(-1), page, seed=1)
        return (pool if t.dim() == 4 else pool.squeeze(-1).contiguous()), bt
    (kp, bt), (vp, _), (ksp, _), (vsp, _) = pages(kq), pages(vq), pages(ks), pages(vs)
    pools0 = [t.clone() for t in (kp, ksp, vp, vsp)]
    pos = synth.prefill_positions(B, T, start=wl.prior, device=DEV)
    y = layer.prefill_paged_int8(x, pos, kp, vp, ksp, vsp, bt)
    c = [t.clone() for t in (kq, vq, ks, vs)]
    yc = layer.prefill_int8(x, pos, *c)
    torch.cuda.synchronize()

    def gathered():
        return (from_pages(kp, bt, page), from_pages(vp, bt, page), from_pages(ksp.unsqueeze(-1), bt, page)[..., 0],
                from_pages(vsp.unsqueeze(-1), bt, page)[..., 0])
    assert _same(y, yc) == 0
    for a, b_ in zip(gathered(), c):
        assert torch.equal(a, b_)
    spare = sorted(set(range(kp.shape[0])) - set(bt.view(-1).tolist()))
    for t, t0 in zip((kp, ksp, vp, vsp), pools0):
        assert torch.equal(t[spare], t0[spare])  # unmapped pages untouched
    w64 = G.oracle_weights(w)
    btn = bt.cpu().numpy()
    kw = dict(n_heads=wl.n_heads, n_kv_heads=wl.n_kv_heads, eps=wl.rms_eps, rope_base=wl.rope_base, bf16_points=True)
    yo, *opools = O.decoder_layer_paged_int8(G.f64(x), G.f64(pos), w64, pools0[0].cpu().numpy(),
                                             pools0[1].cpu().numpy(), pools0[2].cpu().numpy(),
                                             pools0[3].cpu().numpy(), btn, page, cap, **kw)
    G.assert_bf16_output(G.f64(y), yo, "paged int8 prefill y")
    # one decode step at ragged positions
    xd = synth.make_x(wl, (B,), tensor_id=synth.TID_DECODE_BASE, device=DEV)
    pd = torch.tensor([wl.prior + T - (37 * b) % 50 for b in range(B)], dtype=torch.int32, device=DEV)
    yd = layer.decode_paged_int8(xd, pd, kp, vp, ksp, vsp, bt)
    ydc = layer.decode_int8(xd, pd, *c)
    torch.cuda.synchronize()
    assert _same(yd, ydc) == 0
    for a, b_ in zip(gathered(), c):
        assert torch.equal(a, b_)
    ydo, *_ = O.decoder_layer_paged_int8(G.f64(xd)[:, None], G.f64(pd)[:, None], w64, *opools, btn, page, cap, **kw)
    G.assert_bf16_output(G.f64(yd), ydo[:, 0], "paged int8 decode y")
    layer.close()


def test_paged_decode_of_more_sequences_than_one_attention_chunk():
    """80 sequences (the decode attention runs in chunks of 64, the block
    table advancing with them; the GEMMs take the tiled path) at ragged
    positions over shuffled pages: the bf16 and the int8 paged decode
    bit-identical to their contiguous calls, appended slots included."""
    B, page = 80, 64
    wl = synth.Workload("paged80", "bf16", 512, 4, 2, 128, 1408, B, 0, prior=255, decode_steps=1, seed=47)
    cap = 256
    print(f"case B={B} capacity {cap}", flush=True)
    w = synth.make_weights(wl, DEV, random_gains=True)
    x = synth.make_x(wl, (B,), device=DEV)
    kc, vc = synth.make_cache(wl, DEV)
    pos = torch.tensor([(97 * b) % 256 for b in range(B)], dtype=torch.int32, device=DEV)
    layer = lib.LlamaLayer(G.layer_config(lib, wl, B, max_pos=cap), w)
    kp, bt = to_pages(kc, page, seed=5)
    vp, _ = to_pages(vc, page, seed=5)
    yp = layer.decode_paged(x, pos, kp, vp, bt)
    kcc, vcc = kc.clone(), vc.clone()
    yc = layer.decode(x, pos, kcc, vcc)
    torch.cuda.synchronize()
    print(f"  bf16 y: {_same(yp, yc)} elements differ", flush=True)
    assert _same(yp, yc) == 0
    assert _same(from_pages(kp, bt, page), kcc) == 0 and _same(from_pages(vp, bt, page), vcc) == 0
    kq = torch.empty(kc.shape, dtype=torch.int8, device=DEV)
    vq = torch.empty_like(kq)
    ks = torch.empty(kc.shape[:3], dtype=torch.float32, device=DEV)
    vs = torch.empty_like(ks)
    layer.kv_quantize(kc, vc, cap, kq, vq, ks, vs)
    pools = [to_pages(t if t.dim() == 4 else t.unsqueeze(-1), page, seed=5)[0] for t in (kq, vq, ks, vs)]
    pools[2], pools[3] = pools[2].squeeze(-1).contiguous(), pools[3].squeeze(-1).contiguous()
    yq = layer.decode_paged_int8(x, pos, *pools, bt)
    c = [t.clone() for t in (kq, vq, ks, vs)]
    yqc = layer.decode_int8(x, pos, *c)
    torch.cuda.synchronize()
    print(f"  int8 y: {_same(yq, yqc)} elements differ", flush=True)
    assert _same(yq, yqc) == 0
    assert torch.equal(from_pages(pools[0], bt, page), c[0]) and torch.equal(from_pages(pools[1], bt, page), c[1])
    assert torch.equal(from_pages(pools[2].unsqueeze(-1), bt, page)[..., 0], c[2])
    assert torch.equal(from_pages(pools[3].unsqueeze(-1), bt, page)[..., 0], c[3])
    layer.close()
