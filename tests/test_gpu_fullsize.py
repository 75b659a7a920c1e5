"""GPU parity at the full workload sizes (LLaMA-7B/13B/70B layer shapes), in
the launch configuration the benchmark times, on outputs the oracle computes
one by one: sampled token rows of y (the oracle still builds every key and
value those rows attend to) and every cache entry the call writes."""
import numpy as np
import pytest
import torch

import llama_decoder_block_amd as lib
import synth
from oracle import llama_oracle as O
from tests import gpu_helpers as G

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda"


def _prefill_case(name, seed):
    wl = synth.WORKLOADS[name]
    B, T = wl.batch, wl.seq
    print(f"case {name}: B={B} T={T} d={wl.d_model} H={wl.n_heads}/{wl.n_kv_heads} f={wl.d_ff}",
          flush=True)
    w = synth.make_weights(wl, DEV)
    x = synth.make_x(wl, (B, T), device=DEV)
    kc, vc = synth.make_cache(wl, DEV)
    kc0, vc0 = kc.clone(), vc.clone()
    pos = synth.prefill_positions(B, T, device=DEV)
    layer = lib.LlamaLayer(G.layer_config(lib, wl, B * T), w)
    y = layer.prefill(x, pos, kc, vc)
    torch.cuda.synchronize()
    print("  gpu done; running oracle", flush=True)
    w64 = G.oracle_weights(w)
    rows = G.sample_rows(B, T, seed)
    yo, ko, vo = G.oracle_prefill(wl, w64, x, pos, kc0, vc0, rows=rows)
    yg = G.f64(y).reshape(B * T, -1)[rows]
    G.assert_bf16_output(yg, yo.reshape(B * T, -1)[rows], f"y ({len(rows)} sampled rows)")
    kg, vg = G.f64(kc), G.f64(vc)
    fk, fv = G.kv_floors(x, w)
    G.assert_bf16_storage(kg[:, :, :T], ko[:, :, :T], "K written", fk)
    G.assert_bf16_storage(vg[:, :, :T], vo[:, :, :T], "V written", fv)
    return wl, w, w64, layer, kc, vc, ko, vo


def test_llama7b_prefill():
    _prefill_case("llama7b_prefill", 101)


def test_llama7b_prefill_repeatable_with_cold_caches():
    """The same 7B-shape call, repeated with L2 and the Infinity Cache evicted
    (a 512 MB read) before each one, gives bit-identical y, K and V: a
    pipeline whose LDS hand-off depends on load timing shows up here as
    differing elements, because cold loads arrive late and unevenly."""
    wl = synth.WORKLOADS["llama7b_prefill"]
    B, T = wl.batch, wl.seq
    w = synth.make_weights(wl, DEV)
    x = synth.make_x(wl, (B, T), device=DEV)
    kc0, vc0 = synth.make_cache(wl, DEV)
    pos = synth.prefill_positions(B, T, device=DEV)
    layer = lib.LlamaLayer(G.layer_config(lib, wl, B * T), w)
    flush = torch.ones(128 << 20, dtype=torch.int32, device=DEV)
    first = None
    for rep in range(6):
        kc, vc = kc0.clone(), vc0.clone()
        y = torch.empty_like(x)
        flush.sum()
        layer.prefill(x, pos, kc, vc, y=y)
        torch.cuda.synchronize()
        cur = [t.view(torch.int16).clone() for t in (y, kc, vc)]
        if first is None:
            first = cur
            continue
        for name, a, b in zip(("y", "K", "V"), first, cur):
            nd = int((a != b).sum())
            assert nd == 0, f"rep {rep}: {nd} elements of {name} differ from the first call"


def test_llama13b_prefill():
    _prefill_case("llama13b_prefill", 102)


def test_llama7b_decode():
    """32 sequences, one new token each at position 4095 over 4095 random prior slots."""
    wl = synth.WORKLOADS["llama7b_decode"]
    B, p = wl.batch, wl.prior
    print(f"case llama7b_decode: B={B} pos={p}", flush=True)
    w = synth.make_weights(wl, DEV)
    x = synth.make_x(wl, (B,), device=DEV)
    kc, vc = synth.make_cache(wl, DEV)
    kc0, vc0 = kc.clone(), vc.clone()
    pos = torch.full((B,), p, dtype=torch.int32, device=DEV)
    layer = lib.LlamaLayer(G.layer_config(lib, wl, B), w)
    y = layer.decode(x, pos, kc, vc)
    torch.cuda.synchronize()
    w64 = G.oracle_weights(w)
    idx = [0, 9, 22, 31]
    yo, ko, vo = O.decoder_layer_decode(G.f64(x)[idx], np.full(len(idx), p), w64,
                                        G.f64(kc0[idx]), G.f64(vc0[idx]), n_heads=wl.n_heads,
                                        n_kv_heads=wl.n_kv_heads, bf16_points=True)
    G.assert_bf16_output(G.f64(y)[idx], yo, "y (4 sampled sequences)")
    fk, fv = G.kv_floors(x[idx], w)
    G.assert_bf16_storage(G.f64(kc[idx])[:, :, p], ko[:, :, p], "K appended", fk)
    G.assert_bf16_storage(G.f64(vc[idx])[:, :, p], vo[:, :, p], "V appended", fv)
    # prior slots untouched
    assert torch.equal(kc[:, :, :p], kc0[:, :, :p]) and torch.equal(vc[:, :, :p], vc0[:, :, :p])


def test_llama70b_gqa_prefill_then_64_decode_steps():
    wl, w, w64, layer, kc, vc, ko, vo = _prefill_case("llama70b_gqa", 103)
    T = wl.seq
    for s in range(wl.decode_steps):
        p = T + s
        xs = synth.make_x(wl, (1,), tensor_id=synth.TID_DECODE_BASE + s, device=DEV)
        ys = layer.decode(xs, torch.full((1,), p, dtype=torch.int32, device=DEV), kc, vc)
        torch.cuda.synchronize()
        yo, ko, vo = O.decoder_layer_decode(G.f64(xs), np.array([p]), w64, ko, vo,
                                            n_heads=wl.n_heads, n_kv_heads=wl.n_kv_heads,
                                            bf16_points=True)
        if s in (0, 1, 31, 63):
            G.assert_bf16_output(G.f64(ys), yo, f"decode step {s} y")
        else:
            assert G.rel_err(G.f64(ys), yo) <= G.BF16_RMS_GATE, s
    xs_all = torch.stack([synth.make_x(wl, (1,), tensor_id=synth.TID_DECODE_BASE + s, device=DEV)
                          for s in range(wl.decode_steps)])
    fk, fv = G.kv_floors(xs_all, w)
    G.assert_bf16_storage(G.f64(kc)[:, :, T:], ko[:, :, T:], "K appended by 64 steps", fk)
    G.assert_bf16_storage(G.f64(vc)[:, :, T:], vo[:, :, T:], "V appended by 64 steps", fv)
