"""GPU parity of the generation stack (embedding, layers, final norm, LM head,
sampling, the native loop) against the CPU oracle.  Every call goes through
the C ABI.

Where floating point decides a token (argmax, nucleus boundary, inverse
CDF), the GPU decides in fp32 and the oracle in fp64: a token that differs
from the oracle's must be the one the oracle's rule gives with its decision
boundaries moved by at most 1e-4 (relative), and a generated sequence is
compared token by token up to the first such step."""
import numpy as np
import pytest
import torch

import synth
from oracle import generation_oracle as GO
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

import llama_decoder_block_amd as lib  # noqa: E402

DEV = "cuda"


def _check_pick(pick, z, temperature, top_p, penalty, generated, u, tol=1e-4):
    """True if the oracle picks the same token; otherwise assert that the GPU's
    token is what the oracle's rule gives after moving its fp64 decision
    boundaries by at most tol (relative), and return False."""
    want = GO.sample(z, temperature=temperature, top_p=top_p, penalty=penalty, generated=generated, u=u)
    if pick == want:
        return True
    if penalty != 1.0:
        z = GO.repetition_penalty(z, generated, penalty)
    if temperature == 0.0:
        assert z[pick] >= z.max() - tol * max(abs(z.max()), 1.0), (pick, want)
        return False
    p = GO.softmax_temperature(z, temperature)
    members = GO.nucleus(p, top_p)
    if pick not in set(members.tolist()):
        # only the token at the nucleus boundary may differ: its mass must sit
        # within tol of top_p
        order = np.lexsort((np.arange(p.size), -p))
        c = np.cumsum(p[order])
        k = int(np.flatnonzero(order == pick)[0])
        assert abs(c[k - 1] - top_p) <= tol or abs(c[k] - top_p) <= tol, (pick, want)
        return False
    ids = np.sort(members)
    q = p[ids] / p[ids].sum()
    c = np.cumsum(q)
    i = int(np.flatnonzero(ids == pick)[0])
    lo = c[i - 1] if i else 0.0
    assert lo - tol <= u <= c[i] + tol, (pick, want, lo, c[i], u)
    return False


@pytest.mark.parametrize("V", [1000, 32000])
@pytest.mark.parametrize("params", [
    dict(temperature=0.0),
    dict(temperature=0.8),
    dict(temperature=1.0, top_p=0.9),
    dict(temperature=0.7, top_p=0.5, repetition_penalty=1.3),
    dict(temperature=0.0, repetition_penalty=1.5),
])
def test_sampling_matches_oracle(V, params):
    rng = np.random.default_rng(V + int(100 * params.get("top_p", 1.0)))
    B = 16
    z = (rng.standard_normal((B, V)) * 3.0).astype(np.float32)
    hist = rng.integers(-5, V + 5, size=(B, 12)).astype(np.int32)  # some ids out of range (ignored)
    hist[:, 6:] = hist[:, :6]  # duplicates count once
    hlen = rng.integers(0, 13, size=B).astype(np.int32)
    u = rng.uniform(size=B).astype(np.float32)
    sp = lib.make_sampling(**params)
    got = lib.llama_sample(torch.tensor(z, device=DEV), sp, torch.tensor(hist, device=DEV),
                           torch.tensor(hlen, device=DEV), torch.tensor(u, device=DEV)).cpu().numpy()
    exact = 0
    for b in range(B):
        gen = [int(t) for t in hist[b, :hlen[b]] if 0 <= t < V]
        exact += _check_pick(int(got[b]), z[b].astype(np.float64), sp.temperature, sp.top_p,
                             sp.repetition_penalty, gen, float(u[b]))
    print(f"  {exact}/{B} rows identical to the oracle, the rest within its boundaries' fp32 shift")
    if V <= 1000:  # coarse distributions: the fp32 and fp64 decisions agree
        assert exact >= B - 1


def test_sampling_ties_take_the_smaller_ids():
    """Equal probabilities: the nucleus takes the smallest ids among the tied
    tokens (the descending-probability order with ties by id)."""
    V = 64
    z = np.full((4, V), -5.0, dtype=np.float32)
    z[:, [3, 7, 11, 40, 50]] = 2.0  # five tokens tied at the top
    sp = lib.make_sampling(temperature=1.0, top_p=0.5)
    u = torch.tensor([0.0, 0.3, 0.6, 0.999], dtype=torch.float32, device=DEV)
    got = lib.llama_sample(torch.tensor(z, device=DEV), sp, uniforms=u).cpu().numpy()
    for b in range(4):
        p = GO.softmax_temperature(z[b].astype(np.float64), 1.0)
        want = GO.draw(p, GO.nucleus(p, 0.5), float(u[b]))
        assert got[b] == want
    assert set(got.tolist()) <= {3, 7, 11}  # 3 of the 5 tied tokens reach half the mass


# ---------------------------------------------------------------- the model

def _model(wl, n_layers, vocab, random_gains=True, lm_std=0.05):
    mw = synth.make_model_weights(wl, n_layers, vocab, DEV, random_gains=random_gains, lm_std=lm_std)
    return mw


def _oracle_model(wl, mw):
    return {"config": {"n_heads": wl.n_heads, "n_kv_heads": wl.n_kv_heads, "eps": wl.rms_eps,
                       "rope_base": wl.rope_base},
            "embed": G.f64(mw["embed"]), "final_norm": G.f64(mw["final_norm"]), "lm_head": G.f64(mw["lm_head"]),
            "layers": [G.oracle_weights(w) for w in mw["layers"]]}


def _gpu_model(wl, mw, n_layers, vocab, max_tokens):
    cfg = G.layer_config(lib, wl, max_tokens)
    return lib.LlamaModel(cfg, n_layers, vocab, mw["embed"], mw["final_norm"], mw["lm_head"], mw["layers"])


def _caches(wl, B, n_layers):
    kc = [torch.zeros(B, wl.n_kv_heads, wl.max_pos, wl.head_dim, dtype=synth.torch_dtype(wl), device=DEV)
          for _ in range(n_layers)]
    vc = [torch.zeros_like(k) for k in kc]
    return kc, vc


def _oracle_caches(wl, B, n_layers):
    z = np.zeros((B, wl.n_kv_heads, wl.max_pos, wl.head_dim))
    return [(z, z) for _ in range(n_layers)]


def test_tiny_fp32_model_logits_and_greedy_generation():
    wl = synth.Workload("tiny_model", "f32", 64, 4, 2, 16, 96, 2, 5, decode_steps=6, seed=31)
    L, V, B, T = 2, 300, 2, 5
    mw = _model(wl, L, V)
    om = _oracle_model(wl, mw)
    model = _gpu_model(wl, mw, L, V, B * T)
    prompt = np.random.default_rng(1).integers(0, V, size=(B, T)).astype(np.int32)
    kc, vc = _caches(wl, B, L)
    logits = model.prefill(torch.tensor(prompt, device=DEV), kc, vc)
    torch.cuda.synchronize()
    want, _ = GO.model_forward(prompt, np.tile(np.arange(T), (B, 1)), om, _oracle_caches(wl, B, L))
    G.assert_f32(G.f64(logits), want, "prefill logits")
    kc, vc = _caches(wl, B, L)
    got = model.generate(prompt, 6, lib.make_sampling(), kc, vc)
    ref, seen = GO.generate(prompt, om, _oracle_caches(wl, B, L), max_new=6, temperature=0.0)
    for b in range(B):
        # identical until a step whose decision the oracle itself puts within
        # fp32 reach of a boundary (then the GPU's token must still be valid there)
        for s_, t in enumerate(ref[b]):
            if not _check_pick(got[b][s_], seen[s_, b], 0.0, 1.0, 1.0, [], 0.0):
                break
            assert got[b][s_] == t
    model.close()


def test_sampled_generation_matches_oracle():
    """Temperature, top-p and the repetition penalty with the same uniforms on
    both sides (fp32 model), up to the first step whose decision is marginal."""
    wl = synth.Workload("tiny_model", "f32", 64, 4, 2, 16, 96, 3, 4, decode_steps=8, seed=32)
    L, V, B, T, N = 2, 200, 3, 4, 8
    mw = _model(wl, L, V, lm_std=0.3)
    om = _oracle_model(wl, mw)
    model = _gpu_model(wl, mw, L, V, B * T)
    prompt = np.random.default_rng(2).integers(0, V, size=(B, T)).astype(np.int32)
    us = synth.uniform_np(wl.seed, synth.TID_UNIFORM, N * B).reshape(N, B).astype(np.float32)
    kw = dict(temperature=0.9, top_p=0.9, penalty=1.2)
    kc, vc = _caches(wl, B, L)
    got = model.generate(prompt, N, lib.make_sampling(0.9, 0.9, 1.2), kc, vc, uniforms=us)
    ref, seen = GO.generate(prompt, om, _oracle_caches(wl, B, L), max_new=N, uniforms=us.astype(np.float64), **kw)
    compared = 0
    for b in range(B):
        for s_ in range(min(len(ref[b]), len(got[b]))):
            if not _check_pick(got[b][s_], seen[s_, b], 0.9, 0.9, 1.2, ref[b][:s_], float(us[s_, b])):
                break  # a boundary case: the sequences may part from here on
            compared += 1
        else:
            assert len(got[b]) == len(ref[b])
    print(f"  {compared} tokens identical to the oracle's")
    assert compared >= B * N // 2
    model.close()


@pytest.mark.parametrize("B,T", [
    (3, 40),
    # 100 sequences: the logits rows and the decode steps take the four-block
    # weight-streaming GEMMs, the decode attention two chunks of sequences
    (100, 8),
])
def test_bf16_model_logits_and_decode_steps(B, T):
    """A 2-layer bf16 model, vocab 1000 (not a multiple of 128: padded LM
    head): prefill logits and teacher-forced decode-step logits against the
    oracle in its bf16-rounding-point mode."""
    wl = synth.Workload("small_model", "bf16", 512, 4, 2, 128, 1408, B, T, decode_steps=3, seed=33)
    L, V = 2, 1000
    print(f"case B={B} T={T}", flush=True)
    mw = _model(wl, L, V)
    om = _oracle_model(wl, mw)
    model = _gpu_model(wl, mw, L, V, B * T)
    rng = np.random.default_rng(3)
    prompt = rng.integers(0, V, size=(B, T)).astype(np.int32)
    kc, vc = _caches(wl, B, L)
    logits = model.prefill(torch.tensor(prompt, device=DEV), kc, vc)
    torch.cuda.synchronize()
    caches = _oracle_caches(wl, B, L)
    want, caches = GO.model_forward(prompt, np.tile(np.arange(T), (B, 1)), om, caches, bf16_points=True)
    G.assert_bf16_output(G.f64(logits), want, "prefill logits")
    for step in range(3):
        nxt = rng.integers(0, V, size=B).astype(np.int32)
        pos = np.full(B, T + step, dtype=np.int32)
        logits = model.decode(torch.tensor(nxt, device=DEV), torch.tensor(pos, device=DEV), kc, vc)
        torch.cuda.synchronize()
        want, caches = GO.model_forward(nxt[:, None], pos[:, None], om, caches, bf16_points=True)
        G.assert_bf16_output(G.f64(logits), want, f"decode step {step} logits")
    model.close()


def test_generation_stops_at_eos_as_in_the_notes():
    """The notes' example on the GPU: identity layers (W_o = W_down = 0),
    equal embedding rows and an LM head giving logits (3.0, 2.5, 0.1, 2.2)
    every step; greedy with penalty 1.5 generates [0, 1] and stops at EOS 3.
    A second row with no EOS runs to max_new."""
    wl = synth.Workload("eos_model", "f32", 8, 2, 1, 4, 8, 2, 2, decode_steps=6, seed=34)
    L, V = 2, 4
    mw = _model(wl, L, V, random_gains=False)
    for w in mw["layers"]:
        w["wo"].zero_()
        w["w_down"].zero_()
    mw["embed"].fill_(1.0)
    mw["lm_head"].zero_()
    mw["lm_head"][:, 0] = torch.tensor([3.0, 2.5, 0.1, 2.2])
    model = _gpu_model(wl, mw, L, V, 4)
    kc, vc = _caches(wl, 2, L)
    got = model.generate([[2, 2], [1, 3]], 6, lib.make_sampling(repetition_penalty=1.5, eos_id=3), kc, vc)
    assert got == [[0, 1], [0, 1]]
    kc, vc = _caches(wl, 2, L)
    got = model.generate([[2, 2], [1, 3]], 5, lib.make_sampling(), kc, vc)  # no penalty, no EOS
    assert got == [[0] * 5, [0] * 5]
    model.close()


def test_bf16_gqa_batch_generation_with_eos_and_edges():
    """A bf16 GQA stack (4 query heads over 1 kv head), three prompts of one
    token, greedy with an EOS taken from the oracle's own output so that one
    row stops early; max_new = 1 as the smallest loop.  Tokens compared with
    the oracle up to the first fp32-marginal step."""
    wl = synth.Workload("gqa_model", "bf16", 512, 4, 1, 128, 1408, 3, 1, decode_steps=6, seed=35)
    L, V, B, T, N = 2, 512, 3, 1, 6
    mw = _model(wl, L, V, lm_std=0.5)
    om = _oracle_model(wl, mw)
    model = _gpu_model(wl, mw, L, V, B * T)
    prompt = np.array([[5], [77], [300]], dtype=np.int32)
    ref, seen = GO.generate(prompt, om, _oracle_caches(wl, B, L), max_new=N, temperature=0.0, bf16_points=True)
    kc, vc = _caches(wl, B, L)
    got = model.generate(prompt, N, lib.make_sampling(), kc, vc)
    same = 0
    for b in range(B):
        for s_, t in enumerate(ref[b]):
            if not _check_pick(got[b][s_], seen[s_, b], 0.0, 1.0, 1.0, [], 0.0, tol=2e-2):
                break
            assert got[b][s_] == t
            same += 1
    print(f"  {same} greedy tokens identical to the oracle's")
    eos = ref[0][2]
    kc, vc = _caches(wl, B, L)
    got2 = model.generate(prompt, N, lib.make_sampling(eos_id=eos), kc, vc)
    for b in range(B):  # every row is the greedy sequence cut at its first EOS
        k = got[b].index(eos) if eos in got[b] else len(got[b])
        assert got2[b] == got[b][:k]
    kc, vc = _caches(wl, B, L)
    got1 = model.generate(prompt, 1, lib.make_sampling(), kc, vc)
    assert got1 == [g[:1] for g in got]
    model.close()
