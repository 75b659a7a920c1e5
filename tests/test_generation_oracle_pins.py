"""Pins of the generation-stack oracle (embedding, layers, final norm, LM
head, sampling, the loop) against what the pages and the mathematics fix:
hand-worked nucleus sets and draws, closed forms and limits of the
temperature softmax, the sign rule of the repetition penalty, library
routines (torch CPU fp64), the notes' stop-at-EOS example, and invariants.
No GPU is needed."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import generation_oracle as G
from oracle import llama_oracle as O


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- sampling

def test_nucleus_hand_worked_sets():
    """p = [0.05, 0.5, 0.15, 0.3]: descending order 1, 3, 2, 0 with cumulative
    0.5, 0.8, 0.95, 1.0; the set is the shortest prefix reaching top_p."""
    p = np.array([0.05, 0.5, 0.15, 0.3])
    assert list(G.nucleus(p, 0.5)) == [1]          # 0.5 reaches 0.5
    assert list(G.nucleus(p, 0.75)) == [1, 3]
    assert list(G.nucleus(p, 0.85)) == [1, 3, 2]   # the notes' lab default top-p
    assert list(G.nucleus(p, 0.97)) == [1, 3, 2, 0]
    assert sorted(G.nucleus(p, 1.0)) == [0, 1, 2, 3]


def test_nucleus_ties_go_to_the_smaller_id():
    p = np.array([0.2, 0.3, 0.2, 0.3])
    assert list(G.nucleus(p, 0.55)) == [1, 3]
    assert list(G.nucleus(p, 0.65)) == [1, 3, 0]


def test_nucleus_is_minimal_and_takes_the_largest():
    """Invariants on random distributions: the set reaches top_p, dropping its
    smallest member falls below it, and no excluded token is more likely than
    an included one."""
    rng = _rng(3)
    for _ in range(200):
        p = rng.dirichlet(np.full(rng.integers(2, 40), rng.uniform(0.05, 3.0)))
        tp = rng.uniform(0.05, 0.999)
        s = G.nucleus(p, tp)
        mass = p[s].sum()
        assert mass >= tp - 1e-15
        assert mass - p[s].min() < tp
        out = np.setdiff1d(np.arange(p.size), s)
        if out.size:
            assert p[out].max() <= p[s].min()


def test_draw_inverse_cdf_in_ascending_id():
    """Members {1, 3} of p = [0.05, 0.5, 0.15, 0.3] renormalise to 0.625 and
    0.375: u in [0, 0.625) picks 1, u in [0.625, 1) picks 3."""
    p = np.array([0.05, 0.5, 0.15, 0.3])
    assert G.draw(p, [3, 1], 0.0) == 1
    assert G.draw(p, [3, 1], 0.62) == 1
    assert G.draw(p, [3, 1], 0.63) == 3
    assert G.draw(p, [3, 1], 0.999) == 3
    # frequencies over a uniform grid of u reproduce the renormalised probabilities
    us = (np.arange(10000) + 0.5) / 10000
    picks = np.array([G.draw(p, [0, 1, 2, 3], u) for u in us])
    np.testing.assert_allclose(np.bincount(picks, minlength=4) / us.size, p, atol=1e-4)


def test_temperature_softmax_closed_form_and_limits():
    z = np.array([1.5, -0.25, 3.0, 0.0, 2.75])
    for tau in (0.3, 1.0, 1.5):
        p = G.softmax_temperature(z, tau)
        # ratio p_i / p_j = exp((z_i - z_j) / tau)
        np.testing.assert_allclose(p[0] / p[3], np.exp(1.5 / tau), rtol=1e-13)
        np.testing.assert_allclose(p, torch.softmax(torch.tensor(z / tau), 0).numpy(), rtol=1e-13)
    # tau below 1 sharpens, above 1 flattens (the notes' statement), and the
    # tau -> 0+ limit is the greedy choice
    assert G.softmax_temperature(z, 0.5).max() > G.softmax_temperature(z, 1.0).max() > \
        G.softmax_temperature(z, 2.0).max()
    assert np.argmax(G.softmax_temperature(z, 1e-3)) == G.greedy(z) == 2
    assert G.softmax_temperature(z, 1e-3).max() > 1 - 1e-12


def test_greedy_ties_and_explicit_path():
    assert G.greedy([0.5, 2.0, 2.0, -1.0]) == 1
    # temperature 0 takes the explicit argmax path (no division by zero)
    assert G.sample(np.array([0.5, 2.0, 2.0]), temperature=0.0) == 1


def test_repetition_penalty_sign_rule():
    """Positive logits are divided by r, negative ones multiplied, zero stays;
    each distinct generated token once."""
    z = np.array([2.0, -2.0, 0.0, 3.0])
    got = G.repetition_penalty(z, [0, 1, 2, 0], 2.0)
    np.testing.assert_array_equal(got, [1.0, -4.0, 0.0, 3.0])


def test_notes_example_stops_after_two_tokens():
    """The notes' runnable example 10: greedy with penalty 1.5 over set(generated)
    on fixed logits generates [0, 1] and then stops at EOS.  Logits 3.0, 2.5,
    0.1 and EOS (id 3) 2.2: 0 wins, then 2.0 < 2.5 so 1 wins, then 2.0 and
    1.67 fall below EOS's 2.2."""
    logits = np.array([3.0, 2.5, 0.1, 2.2])
    eos, generated = 3, []
    for _ in range(10):
        t = G.sample(logits, temperature=0.0, penalty=1.5, generated=generated)
        if t == eos:
            break
        generated.append(t)
    assert generated == [0, 1]


# ---------------------------------------------------------------- model and loop

def _model(seed, V=12, d=16, H=2, Hkv=1, f=24, layers=2, zero_out=False):
    rng = _rng(seed)
    dh = d // H
    lw = []
    for _ in range(layers):
        w = {"wq": rng.standard_normal((H * dh, d)) * 0.3, "wk": rng.standard_normal((Hkv * dh, d)) * 0.3,
             "wv": rng.standard_normal((Hkv * dh, d)) * 0.3, "wo": rng.standard_normal((d, H * dh)) * 0.3,
             "w_gate": rng.standard_normal((f, d)) * 0.3, "w_up": rng.standard_normal((f, d)) * 0.3,
             "w_down": rng.standard_normal((d, f)) * 0.3,
             "attn_norm": 1 + 0.1 * rng.standard_normal(d), "ffn_norm": 1 + 0.1 * rng.standard_normal(d)}
        if zero_out:
            w["wo"] = np.zeros_like(w["wo"])
            w["w_down"] = np.zeros_like(w["w_down"])
        lw.append(w)
    return {"config": {"n_heads": H, "n_kv_heads": Hkv, "eps": 1e-6, "rope_base": 10000.0},
            "embed": rng.standard_normal((V, d)), "final_norm": 1 + 0.1 * rng.standard_normal(d),
            "lm_head": rng.standard_normal((V, d)) * 0.5, "layers": lw}


def _caches(model, B, S):
    d = model["embed"].shape[1]
    H, Hkv = model["config"]["n_heads"], model["config"]["n_kv_heads"]
    z = np.zeros((B, Hkv, S, d // H))
    return [(z, z) for _ in model["layers"]]


def test_lm_logits_matches_library_routines():
    m = _model(5)
    h = _rng(6).standard_normal((3, 16))
    ref = F.linear(F.rms_norm(torch.tensor(h), (16,), torch.tensor(m["final_norm"]), 1e-6),
                   torch.tensor(m["lm_head"])).numpy()
    np.testing.assert_allclose(G.lm_logits(h, m["final_norm"], m["lm_head"]), ref, rtol=1e-12, atol=1e-12)


def test_identity_layers_give_closed_form_logits():
    """With W_o = W_down = 0 every layer is the identity, so the logits are
    lm_head . RMSNorm(E[last id]) in closed form."""
    m = _model(7, zero_out=True)
    ids = np.array([[3, 1, 4, 1, 5]])
    logits, _ = G.model_forward(ids, np.arange(5)[None], m, _caches(m, 1, 8))
    e = m["embed"][5]
    ref = m["lm_head"] @ (m["final_norm"] * e / np.sqrt(np.mean(e * e) + 1e-6))
    np.testing.assert_allclose(logits[0], ref, rtol=1e-13)


def test_generate_stops_at_eos_as_in_the_notes():
    """The same fixed logits produced by a model: identical embedding rows and
    identity layers make every step's logits equal, and the LM head is built
    so they are (3.0, 2.5, 0.1, 2.2) times RMSNorm's 1/sqrt(1 + eps)."""
    V, d = 4, 4
    m = _model(8, V=V, d=d, H=2, Hkv=1, f=8, layers=2, zero_out=True)
    m["embed"] = np.ones((V, d))
    m["final_norm"] = np.ones(d)
    m["lm_head"] = np.zeros((V, d))
    m["lm_head"][:, 0] = [3.0, 2.5, 0.1, 2.2]
    out, _ = G.generate(np.array([[2, 2]]), m, _caches(m, 1, 16), max_new=8, temperature=0.0,
                        penalty=1.5, eos_id=3)
    assert out == [[0, 1]]


def test_generate_rows_stop_independently_and_respect_max_new():
    m = _model(9)
    prompt = np.array([[1, 2, 3], [4, 5, 6]])
    out, seen = G.generate(prompt, m, _caches(m, 2, 16), max_new=5, temperature=0.0)
    assert [len(o) for o in out] == [5, 5]
    eos = out[0][2]  # make row 0's third token the EOS: each row stops at its first EOS
    out2, seen2 = G.generate(prompt, m, _caches(m, 2, 16), max_new=5, temperature=0.0, eos_id=eos)
    for b in range(2):
        k = out[b].index(eos) if eos in out[b] else len(out[b])
        assert out2[b] == out[b][:k]
        assert np.isnan(seen2[k + 1:, b]).all()  # a finished row takes no further steps


def test_decode_logits_equal_a_longer_prefill():
    """Step s's logits (decode over the cache) equal the last logits of one
    prefill over the prompt plus the s tokens generated before it."""
    m = _model(10)
    prompt = np.array([[7, 2, 9, 4]])
    out, seen = G.generate(prompt, m, _caches(m, 1, 16), max_new=4, temperature=0.0)
    for s in range(1, 4):
        ids = np.concatenate([prompt[0], out[0][:s]])[None]
        full, _ = G.model_forward(ids, np.arange(ids.shape[1])[None], m, _caches(m, 1, 16))
        np.testing.assert_allclose(seen[s, 0], full[0], rtol=1e-11, atol=1e-11)


def test_sampled_generation_uses_the_given_uniforms():
    """Temperature + top-p: each step's token is the oracle's draw with that
    step's u; the same uniforms reproduce the same tokens."""
    m = _model(11)
    prompt = np.array([[1, 2], [3, 4]])
    us = _rng(12).uniform(size=(6, 2))
    kw = dict(max_new=6, temperature=0.8, top_p=0.9, penalty=1.2, uniforms=us)
    out, seen = G.generate(prompt, m, _caches(m, 2, 16), **kw)
    out2, _ = G.generate(prompt, m, _caches(m, 2, 16), **kw)
    assert out == out2
    for b in range(2):
        for s, t in enumerate(out[b]):
            z = G.repetition_penalty(seen[s, b], out[b][:s], 1.2)
            p = G.softmax_temperature(z, 0.8)
            assert t in set(G.nucleus(p, 0.9).tolist())
            assert t == G.draw(p, G.nucleus(p, 0.9), us[s, b])
