"""GPU parity of the int8 KV cache (symmetric int8 codes, one fp32 scale per
cached row) against the oracle's quantizer and its int8 decode step: the
conversion of a bf16 cache bit for bit, and decode steps over the int8 cache
at the raw 0.02 x RMS gate.  Every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import synth
from oracle import llama_oracle as O
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

import llama_decoder_block_amd as lib  # noqa: E402  (fails loudly if the library is not built)

DEV = "cuda"


def _wl(d=512, H=4, Hkv=2, f=1408, B=3, prior=300, steps=0, seed=51):
    """max_pos = prior + 1 + steps: room for the appended slots"""
    return synth.Workload("int8", "bf16", d, H, Hkv, 128, f, B, 1, prior=prior, decode_steps=steps, seed=seed)


def _int8_cache(wl):
    B, Hkv, S = wl.batch, wl.n_kv_heads, wl.max_pos
    kq = torch.full((B, Hkv, S, 128), 85, dtype=torch.int8, device=DEV)  # sentinels: slots not written keep them
    vq = torch.full((B, Hkv, S, 128), -86, dtype=torch.int8, device=DEV)
    ks = torch.full((B, Hkv, S), 7.25, dtype=torch.float32, device=DEV)
    vs = torch.full((B, Hkv, S), -3.5, dtype=torch.float32, device=DEV)
    return kq, vq, ks, vs


def test_convert_matches_the_oracle_bit_for_bit():
    """llama_layer_kv_quantize on a bf16 cache with N(0,1) rows, rows scaled
    by 1e-30 and 1e30, a zero row and a row below 2^-100: codes and scales
    equal the oracle's (the same fp32 decision on the same bf16 values);
    slots past n_slots keep their contents."""
    wl = _wl(prior=300)
    print(f"case {wl}", flush=True)
    w = synth.make_weights(wl, DEV)
    layer = lib.LlamaLayer(G.layer_config(lib, wl, 64), w)
    kc, vc = synth.make_cache(wl, DEV)
    kf = kc.float()
    kf[0, 0, 3] = 0.0
    kf[0, 1, 4] *= 1e-30
    kf[1, 0, 5] *= 1e30
    kf[2, 1, 6] = 2.0 ** -110
    kc.copy_(kf.to(kc.dtype))
    kq, vq, ks, vs = _int8_cache(wl)
    n = 257
    layer.kv_quantize(kc, vc, n, kq, vq, ks, vs)
    torch.cuda.synchronize()
    for name, cache, q, s in (("K", kc, kq, ks), ("V", vc, vq, vs)):
        co, so = O.kv_int8_quantize(G.f64(cache)[:, :, :n])
        np.testing.assert_array_equal(q[:, :, :n].cpu().numpy(), co, err_msg=f"{name} codes")
        np.testing.assert_array_equal(s[:, :, :n].cpu().numpy(), so, err_msg=f"{name} scales")
    assert torch.all(kq[:, :, n:] == 85) and torch.all(vq[:, :, n:] == -86)
    assert torch.all(ks[:, :, n:] == 7.25) and torch.all(vs[:, :, n:] == -3.5)
    assert torch.all(kq[0, 0, 3] == 0) and ks[0, 0, 3] == 0 and ks[2, 1, 6] == 0
    layer.close()


@pytest.mark.parametrize("shape", [
    # 2 query heads per kv head, three sequences at different lengths, one split
    dict(d=512, H=4, Hkv=2, B=3, prior=300, pos=(300, 150, 77), steps=3),
    # 4 query heads per kv head over 4096 slots: several splits and their merge
    dict(d=2048, H=16, Hkv=4, B=2, prior=4095, pos=(4095, 3000), steps=2),
    # 80 sequences: more tokens than the weight-streaming GEMMs take, so the
    # tiled QKV GEMM's epilogue stages the rows (and the attention runs in
    # chunks of sequences)
    dict(d=512, H=4, Hkv=2, B=80, prior=200, pos=tuple(range(120, 200)), steps=1),
])
def test_decode_steps_over_the_int8_cache(shape):
    """A random bf16 cache converted to int8, then decode steps that append
    quantized rows and attend over code * scale: y against the oracle's int8
    step (bf16 rounding points, the oracle continuing from its own int8
    cache) at the raw 0.02 x RMS gate; the appended rows within one code step
    of the oracle's int8 rows, their codes equal to the oracle's but where
    the two sides' bf16 values differ (then one apart, for at most 5%);
    every other slot untouched."""
    wl = _wl(d=shape["d"], H=shape["H"], Hkv=shape["Hkv"], B=shape["B"], prior=shape["prior"], steps=shape["steps"])
    print(f"case {shape}", flush=True)
    w = synth.make_weights(wl, DEV)
    w64 = G.oracle_weights(w)
    layer = lib.LlamaLayer(G.layer_config(lib, wl, max(64, wl.batch)), w)
    kc, vc = synth.make_cache(wl, DEV)
    kq, vq, ks, vs = _int8_cache(wl)
    layer.kv_quantize(kc, vc, wl.max_pos, kq, vq, ks, vs)
    torch.cuda.synchronize()
    okq, oks = O.kv_int8_quantize(G.f64(kc))
    ovq, ovs = O.kv_int8_quantize(G.f64(vc))
    kw = dict(n_heads=wl.n_heads, n_kv_heads=wl.n_kv_heads, eps=wl.rms_eps, rope_base=wl.rope_base,
              bf16_points=True)
    for step in range(shape["steps"]):
        p = np.array(shape["pos"]) + step  # below max_pos = prior + 1 + steps
        x = synth.make_x(wl, (wl.batch,), tensor_id=synth.TID_DECODE_BASE + step, device=DEV)
        pos = torch.tensor(p, dtype=torch.int32, device=DEV)
        before = (kq.clone(), vq.clone(), ks.clone(), vs.clone())
        y = layer.decode_int8(x, pos, kq, vq, ks, vs)
        torch.cuda.synchronize()
        ex = {}
        yo, okq, oks, ovq, ovs = O.decoder_layer_decode_int8(G.f64(x), p, w64, okq, oks, ovq, ovs, kv_exact=ex, **kw)
        G.assert_bf16_output(G.f64(y), yo, f"decode step {step} y")
        for name, q, s, oq, os_, kx, prev in (("K", kq, ks, okq, oks, ex["k"], before[0]),
                                             ("V", vq, vs, ovq, ovs, ex["v"], before[1])):
            qn, sn = q.cpu().numpy(), s.cpu().numpy()
            got = np.stack([O.kv_int8_dequantize(qn[b, :, p[b]], sn[b, :, p[b]]) for b in range(wl.batch)])
            want = np.stack([O.kv_int8_dequantize(oq[b, :, p[b]], os_[b, :, p[b]]) for b in range(wl.batch)])
            step_ = np.maximum(np.stack([sn[b, :, p[b]] for b in range(wl.batch)]),
                               np.stack([os_[b, :, p[b]] for b in range(wl.batch)]))[..., None]
            ref = kx[:, :, 0]  # [B, Hkv, dh], exact (before any rounding)
            print(f"  {name} appended: max|err|/rms against the exact values = "
                  f"{np.max(np.abs(got - ref)) / G.rms(ref):.5f} (the int8 format's own error included); "
                  f"against the oracle's int8 row: {np.max(np.abs(got - want) / step_):.3f} steps")
            # the two sides round the same bf16 values but where those differ: one code step at most
            assert np.all(np.abs(got - want) <= 1.01 * step_)
            gc = np.stack([qn[b, :, p[b]] for b in range(wl.batch)]).astype(np.int64)
            oc = np.stack([oq[b, :, p[b]] for b in range(wl.batch)]).astype(np.int64)
            diff = np.abs(gc - oc)
            print(f"  {name} appended codes: {int((diff > 0).sum())}/{diff.size} differ from the oracle's, max {diff.max()}")
            assert diff.max() <= 1 and (diff > 0).mean() <= 0.05
            # every other slot is untouched
            mask = np.ones(qn.shape[:3], dtype=bool)
            for b in range(wl.batch):
                mask[b, :, p[b]] = False
            np.testing.assert_array_equal(qn[mask], prev.cpu().numpy()[mask])
        # the oracle carries its own cache on: the two sides' appended rows may
        # differ by a step where their bf16 keys differ (counted above)
    layer.close()


def _check_appended(name, q, s, oq, os_, slots, prev_q, prev_s):
    """The rows written at slots[b] (a list per sequence) of the int8 cache
    (codes q [B, Hkv, S, dh], scales s) against the oracle's (oq, os_): within
    one code step, codes equal but where the two sides' bf16 values differ (then
    one apart, for at most 5%); every other slot unchanged from prev_q / prev_s."""
    qn, sn = q.cpu().numpy(), s.cpu().numpy()
    gd, od, stp, gc, oc = [], [], [], [], []
    for b, sl in enumerate(slots):
        gd.append(O.kv_int8_dequantize(qn[b][:, sl], sn[b][:, sl]).ravel())
        od.append(O.kv_int8_dequantize(oq[b][:, sl], os_[b][:, sl]).ravel())
        stp.append(np.repeat(np.maximum(sn[b][:, sl], os_[b][:, sl]).ravel(), qn.shape[-1]))
        gc.append(qn[b][:, sl].astype(np.int64).ravel())
        oc.append(oq[b][:, sl].astype(np.int64).ravel())
    gd, od, stp, gc, oc = (np.concatenate(a) for a in (gd, od, stp, gc, oc))
    diff = np.abs(gc - oc)
    print(f"  {name} appended: {np.max(np.abs(gd - od) / np.maximum(stp, 1e-30)):.3f} steps from the oracle's "
          f"int8 rows; codes {int((diff > 0).sum())}/{diff.size} differ, max {diff.max()}", flush=True)
    assert np.all(np.abs(gd - od) <= 1.01 * stp)
    assert diff.max() <= 1 and (diff > 0).mean() <= 0.05
    mask = np.ones(qn.shape[:3], dtype=bool)
    for b, sl in enumerate(slots):
        mask[b][:, sl] = False
    np.testing.assert_array_equal(qn[mask], prev_q.cpu().numpy()[mask])
    np.testing.assert_array_equal(sn[mask], prev_s.cpu().numpy()[mask])


@pytest.mark.parametrize("shape", [
    # two sequences, one continuing its converted cache at 120, one a fresh
    # prompt at 0 (ragged query tiles; few workgroups: the eight-wavefront
    # attention kernel)
    dict(d=512, H=4, Hkv=2, f=1408, B=2, T=150, prior=120, starts=(120, 0)),
    # 544 query tiles: the four-wavefront kernel in several rounds, GQA 4:1,
    # a ragged last tile; sampled rows
    dict(d=2048, H=16, Hkv=4, f=5632, B=2, T=2100, prior=64, starts=(64, 64), sampled=True),
    # 15 tokens: the weight-streaming GEMMs stage the rows
    dict(d=256, H=2, Hkv=2, f=384, B=3, T=5, prior=40, starts=(40, 7, 0)),
    # the bidirectional variant
    dict(d=512, H=4, Hkv=2, f=1408, B=2, T=100, prior=50, starts=(50, 20), bidirectional=True),
])
def test_prefill_over_the_int8_cache(shape):
    """A chunk of T tokens per sequence over a converted int8 cache: the new
    rows are quantized into their slots and every query reads code * scale
    (its own chunk's rows included).  y against the oracle's int8 layer call
    at the raw 0.02 x RMS gate; the appended rows as in the decode test; every
    other slot untouched."""
    bidir = shape.get("bidirectional", False)
    wl = synth.Workload("int8p", "bf16", shape["d"], shape["H"], shape["Hkv"], 128, shape["f"], shape["B"],
                        shape["T"], prior=shape["prior"], seed=53)
    print(f"case {shape}", flush=True)
    B, T = wl.batch, wl.seq
    w = synth.make_weights(wl, DEV, random_gains=True)
    layer = lib.LlamaLayer(G.layer_config(lib, wl, B * T, bidirectional=bidir), w)
    kc, vc = synth.make_cache(wl, DEV)
    kq, vq, ks, vs = _int8_cache(wl)
    layer.kv_quantize(kc, vc, wl.max_pos, kq, vq, ks, vs)
    torch.cuda.synchronize()
    before = (kq.clone(), ks.clone(), vq.clone(), vs.clone())
    x = synth.make_x(wl, (B, T), device=DEV)
    p = np.stack([np.arange(s0, s0 + T) for s0 in shape["starts"]])  # below max_pos = prior + T
    pos = torch.tensor(p, dtype=torch.int32, device=DEV)
    y = layer.prefill_int8(x, pos, kq, vq, ks, vs)
    torch.cuda.synchronize()
    rows = G.sample_rows(B, T, seed=54) if shape.get("sampled") else None
    okq, oks = O.kv_int8_quantize(G.f64(kc))
    ovq, ovs = O.kv_int8_quantize(G.f64(vc))
    yo, okq, oks, ovq, ovs = O.decoder_layer_int8(
        G.f64(x), p, G.oracle_weights(w), okq, oks, ovq, ovs, rows=rows, n_heads=wl.n_heads,
        n_kv_heads=wl.n_kv_heads, eps=wl.rms_eps, rope_base=wl.rope_base, bf16_points=True, bidirectional=bidir)
    yg = G.f64(y).reshape(B * T, -1)
    yo = yo.reshape(B * T, -1)
    sel = rows if rows is not None else slice(None)
    G.assert_bf16_output(yg[sel], yo[sel], "y")
    slots = [list(p[b]) for b in range(B)]
    _check_appended("K", kq, ks, okq, oks, slots, before[0], before[1])
    _check_appended("V", vq, vs, ovq, ovs, slots, before[2], before[3])
    layer.close()


@pytest.mark.slow
def test_llama7b_int8_prefill():
    """The 7B prefill workload over an int8 cache, as the benchmark runs it: a
    2048-token prompt from position 0 quantized into its slots while every
    query attends over code * scale; y of all 2048 rows at the raw gate and
    every appended row against the oracle's int8 call."""
    wl = synth.WORKLOADS["llama7b_prefill"]
    B, T = wl.batch, wl.seq
    print(f"case llama7b_prefill int8: B={B} T={T}", flush=True)
    w = synth.make_weights(wl, DEV)
    x = synth.make_x(wl, (B, T), device=DEV)
    pos = synth.prefill_positions(B, T, device=DEV)
    kq, vq, ks, vs = _int8_cache(wl)
    before = (kq.clone(), ks.clone(), vq.clone(), vs.clone())
    layer = lib.LlamaLayer(G.layer_config(lib, wl, B * T), w)
    y = layer.prefill_int8(x, pos, kq, vq, ks, vs)
    torch.cuda.synchronize()
    print("  gpu done; running the oracle on every row", flush=True)
    p = pos.cpu().numpy()
    yo, okq, oks, ovq, ovs = O.decoder_layer_int8(
        G.f64(x), p, G.oracle_weights(w), *(t.cpu().numpy() for t in (before[0], before[1], before[2], before[3])),
        n_heads=wl.n_heads, n_kv_heads=wl.n_kv_heads, eps=wl.rms_eps, rope_base=wl.rope_base, bf16_points=True)
    G.assert_bf16_output(G.f64(y).reshape(B * T, -1), yo.reshape(B * T, -1), f"y (all {B * T} rows)")
    slots = [list(p[b]) for b in range(B)]
    _check_appended("K", kq, ks, okq, oks, slots, before[0], before[1])
    _check_appended("V", vq, vs, ovq, ovs, slots, before[2], before[3])
    layer.close()


@pytest.mark.slow
def test_llama7b_int8_decode_and_its_paged_form():
    """The 7B decode workload over an int8 cache, as the benchmark runs it:
    32 sequences at position 4095 whose 4096 random bf16 rows per head are
    converted (codes and scales bit for bit the oracle's at this size), then
    one step: y of every sequence at the raw gate and the appended rows
    against the oracle's int8 step.  The same step over the codes and scales
    on shuffled pages of 64 slots is bit-identical to the contiguous one."""
    from tests.test_gpu_paged import from_pages, to_pages
    wl = synth.WORKLOADS["llama7b_decode"]
    B, p = wl.batch, wl.prior
    print(f"case llama7b_decode int8: B={B} pos={p}", flush=True)
    w = synth.make_weights(wl, DEV)
    x = synth.make_x(wl, (B,), device=DEV)
    kc, vc = synth.make_cache(wl, DEV)
    kq, vq, ks, vs = _int8_cache(wl)
    layer = lib.LlamaLayer(G.layer_config(lib, wl, B), w)
    layer.kv_quantize(kc, vc, wl.max_pos, kq, vq, ks, vs)
    torch.cuda.synchronize()
    okq, oks = O.kv_int8_quantize(G.f64(kc))
    ovq, ovs = O.kv_int8_quantize(G.f64(vc))
    del kc, vc
    for name, q, s, oq, os_ in (("K", kq, ks, okq, oks), ("V", vq, vs, ovq, ovs)):
        np.testing.assert_array_equal(q.cpu().numpy(), oq, err_msg=f"{name} codes")
        np.testing.assert_array_equal(s.cpu().numpy(), os_, err_msg=f"{name} scales")
    print("  conversion bit-identical to the oracle's", flush=True)

    def pages(t):  # scales [B, Hkv, S] ride as rows of one element
        pool, bt = to_pages(t if t.dim() == 4 else t.unsqueeze(-1), 64, seed=5)
        return (pool if t.dim() == 4 else pool.squeeze(-1).contiguous()), bt
    (kp, bt), (vp, _), (ksp, _), (vsp, _) = pages(kq), pages(vq), pages(ks), pages(vs)
    before = (kq.clone(), ks.clone(), vq.clone(), vs.clone())
    pos = torch.full((B,), p, dtype=torch.int32, device=DEV)
    y = layer.decode_int8(x, pos, kq, vq, ks, vs)
    yp = layer.decode_paged_int8(x, pos, kp, vp, ksp, vsp, bt)
    torch.cuda.synchronize()
    nd = int((yp.view(torch.int16) != y.view(torch.int16)).sum())
    print(f"  paged y: {nd} elements differ from the contiguous call", flush=True)
    assert nd == 0
    for a, b_ in ((from_pages(kp, bt, 64), kq), (from_pages(vp, bt, 64), vq),
                  (from_pages(ksp.unsqueeze(-1), bt, 64)[..., 0], ks), (from_pages(vsp.unsqueeze(-1), bt, 64)[..., 0], vs)):
        assert torch.equal(a, b_)
    del kp, vp, ksp, vsp
    pn = np.full(B, p)
    yo, okq, oks, ovq, ovs = O.decoder_layer_decode_int8(
        G.f64(x), pn, G.oracle_weights(w), okq, oks, ovq, ovs, n_heads=wl.n_heads, n_kv_heads=wl.n_kv_heads,
        eps=wl.rms_eps, rope_base=wl.rope_base, bf16_points=True)
    G.assert_bf16_output(G.f64(y), yo, f"y (all {B} sequences)")
    slots = [[p] for _ in range(B)]
    _check_appended("K", kq, ks, okq, oks, slots, before[0], before[1])
    _check_appended("V", vq, vs, ovq, ovs, slots, before[2], before[3])
    layer.close()
