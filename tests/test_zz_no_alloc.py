"""The allocation-free decode entry point (llama_layer_decode_noalloc, scratch
in the library's static device array) against the ordinary decode
(llama_layer_decode, scratch in the handle), through the C ABI: two calls in
a row on one handle, the second with fewer sequences, each bit-identical to
the ordinary call on the same inputs (same kernels, same arithmetic)."""
import pytest
import torch

import llama_decoder_block_amd as lib
import synth
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("name,shape,calls", [
    # GQA layer over a 2048-slot random cache: 40 sequences (two 32-token
    # blocks in the weight-streaming GEMMs, split attention), then 5
    ("gqa_small", dict(d=1024, H=8, Hkv=2, f=2816, prior=2047), [40, 5]),
    # the LLaMA-7B decode shape: 32 sequences at position 4095, then 8
    ("llama7b", None, [32, 8]),
])
def test_noalloc_decode_matches_decode(name, shape, calls):
    if shape is None:
        wl = synth.WORKLOADS["llama7b_decode"]
    else:
        wl = synth.Workload(name, "bf16", shape["d"], shape["H"], shape["Hkv"], 128, shape["f"], max(calls), 0,
                            prior=shape["prior"], decode_steps=1, seed=77)
    print(f"case {name}: calls with B = {calls}", flush=True)
    w = synth.make_weights(wl, DEV, random_gains=True)
    kc0, vc0 = synth.make_cache(wl, DEV, batch=max(calls))
    layer = lib.LlamaLayer(G.layer_config(lib, wl, max(calls)), w)
    for i, B in enumerate(calls):
        x = synth.make_x(wl, (B,), tensor_id=synth.TID_DECODE_BASE + i, device=DEV)
        # ragged positions at the small shape, the workload's position at 7B
        if shape is None:
            pos = torch.full((B,), wl.prior, dtype=torch.int32, device=DEV)
        else:
            pos = ((torch.arange(B, device=DEV) * 397 + 11 * i) % (wl.prior + 1)).to(torch.int32)
        ka, va = kc0[:B].clone(), vc0[:B].clone()
        kb, vb = kc0[:B].clone(), vc0[:B].clone()
        ya = layer.decode(x, pos, ka, va)
        yb = torch.empty_like(x)
        layer.decode_noalloc(x, pos, kb, vb, y=yb)
        torch.cuda.synchronize()
        for what, a, b in (("y", ya, yb), ("K cache", ka, kb), ("V cache", va, vb)):
            nd = int((a.view(torch.int16) != b.view(torch.int16)).sum())
            print(f"  call {i} (B={B}): {what}: {nd} elements differ", flush=True)
            assert nd == 0, f"call {i}: {what} differs in {nd} elements"
    layer.close()


def test_noalloc_decode_rejects_what_it_cannot_serve():
    wl = synth.Workload("t", "bf16", 256, 2, 2, 128, 384, 1, 0, prior=8, decode_steps=1)
    w = synth.make_weights(wl, DEV)
    layer = lib.LlamaLayer(G.layer_config(lib, wl, 128), w)
    kc, vc = synth.make_cache(wl, DEV, batch=65)
    x = synth.make_x(wl, (65,), device=DEV)
    pos = torch.full((65,), 3, dtype=torch.int32, device=DEV)
    with pytest.raises(lib.LlamaLayerError) as e:
        layer.decode_noalloc(x, pos, kc, vc, y=torch.empty_like(x))
    assert e.value.status == lib.LLAMA_ERR_CAPACITY
    wf = synth.Workload("t32", "f32", 64, 4, 4, 16, 96, 1, 0, prior=8, decode_steps=1)
    lf = lib.LlamaLayer(G.layer_config(lib, wf, 4), synth.make_weights(wf, DEV))
    kf, vf = synth.make_cache(wf, DEV, batch=2)
    xf = synth.make_x(wf, (2,), device=DEV)
    with pytest.raises(lib.LlamaLayerError) as e:
        lf.decode_noalloc(xf, pos[:2], kf, vf, y=torch.empty_like(xf))
    assert e.value.status == lib.LLAMA_ERR_UNSUPPORTED
