"""Plain CPU oracle for the generation stack around the decoder layer:
embedding, L decoder layers, final RMSNorm, LM head, and the sampling step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

Sources, cited by page title and section:

  [Notes]  "LLM 核心机制交互讲义" (LLM mechanics lecture notes):
           Ch.02, the decoder-only data flow [B,T,d] embedding -> L blocks ->
           [B,T,V] logits, X_0 = E[ids], generation reads the last position's
           logits; Ch.04 prefill then single-token decode over the cache;
           Ch.05 sampling: temperature softmax(z / tau), greedy as an explicit
           argmax, the top-p nucleus (sort by probability, descending; the
           smallest prefix whose cumulative probability reaches p;
           renormalise and draw inside it), the sign-aware repetition penalty
           (a positive logit is divided by r > 1, a negative one multiplied by
           r) on the tokens generated so far, EOS as a per-row stop state with
           max tokens as a hard bound, and the end-to-end loop (prefill, take
           the last logits, penalise, sample, stop at EOS, decode the new
           token, repeat).
  [LMDrive] "LMDrive 大语言模型（LLM）核心推理单元": §2.1 RMSNorm (used once
           more after the last layer, before the LM head).

Readings where the pages leave a step open (each listed in the design notes):
  * the final RMSNorm has a gain and the LM head has no bias and its own
    weights (not tied to the embedding);
  * the repetition penalty applies once per distinct token among the tokens
    generated so far (the notes' example passes set(generated)); the prompt
    is not penalised;
  * ties in the nucleus order (equal probabilities) go to the smaller token
    id; greedy ties likewise;
  * the draw inside the nucleus: with u uniform in [0, 1), the token is the
    first, in ascending token id, whose cumulative renormalised probability
    exceeds u (inverse CDF; the random number is an input, never drawn here).

Everything is fp64 numpy.  In the "bf16 points" mode the final normalised
activation is rounded to bf16 (it feeds a bf16 matrix product), as the layer
oracle rounds its own operands; logits are never rounded.
"""
from __future__ import annotations

import numpy as np

from oracle import llama_oracle as L


# --------------------------------------------------------------------------
# Model: embedding, layers, final norm, LM head  [Notes Ch.02, Ch.04]
# --------------------------------------------------------------------------

def embed(ids, table):
    """X_0 = E[ids]: rows of the [vocab, d] table."""
    return np.asarray(table, dtype=np.float64)[np.asarray(ids, dtype=np.int64)]


def lm_logits(h, final_norm, lm_head, eps=1e-6, bf16_points=False):
    """logits = RMSNorm(h) W_lm^T for hidden states h [..., d]."""
    xn = L.rms_norm(h, final_norm, eps)
    if bf16_points:
        xn = L.bf16_round(xn)
    return xn @ np.asarray(lm_head, dtype=np.float64).T


def model_forward(ids, positions, model, caches, *, bf16_points=False, last_only=True):
    """Run the embedding and every layer over tokens ids [B, T] at positions
    [B, T]; caches is a list of (k_cache, v_cache) per layer, updated (new
    arrays returned).  Returns (logits of the last position [B, V] (or of all
    positions [B, T, V]), new caches)."""
    cfg = model["config"]
    x = embed(ids, model["embed"])
    if bf16_points:
        x = L.bf16_round(x)  # the activations between layers are bf16 tensors
    new = []
    for lw, (kc, vc) in zip(model["layers"], caches):
        y, kc2, vc2 = L.decoder_layer(x, positions, lw, kc, vc, n_heads=cfg["n_heads"],
                                      n_kv_heads=cfg["n_kv_heads"], eps=cfg["eps"],
                                      rope_base=cfg["rope_base"], bf16_points=bf16_points)
        x = L.bf16_round(y) if bf16_points else y
        new.append((kc2, vc2))
    h = x[:, -1] if last_only else x
    return lm_logits(h, model["final_norm"], model["lm_head"], cfg["eps"], bf16_points), new


# --------------------------------------------------------------------------
# Sampling  [Notes Ch.05]
# --------------------------------------------------------------------------

def repetition_penalty(z, generated, r):
    """Sign-aware penalty on every distinct generated token: z / r if z > 0,
    z * r otherwise (zero stays zero)."""
    z = np.array(z, dtype=np.float64)
    for t in sorted(set(int(i) for i in generated)):
        z[t] = z[t] / r if z[t] > 0 else z[t] * r
    return z


def greedy(z):
    """argmax, the smallest id among equal maxima."""
    z = np.asarray(z, dtype=np.float64)
    return int(np.flatnonzero(z == z.max())[0])


def softmax_temperature(z, tau):
    """p_i = exp(z_i / tau) / sum_j exp(z_j / tau), max-subtracted."""
    s = np.asarray(z, dtype=np.float64) / tau
    e = np.exp(s - s.max())
    return e / e.sum()


def nucleus(p, top_p):
    """The smallest set of tokens, taken in descending probability (ties: the
    smaller id first), whose cumulative probability reaches top_p.  Returns
    the token ids of the set (in that order)."""
    p = np.asarray(p, dtype=np.float64)
    if top_p >= 1.0:
        return np.argsort(-p, kind="stable")
    order = np.lexsort((np.arange(p.size), -p))  # primary: -p, secondary: id
    c = np.cumsum(p[order])
    k = int(np.searchsorted(c, top_p, side="left")) + 1  # first prefix with c >= top_p
    return order[:min(k, p.size)]


def draw(p, members, u):
    """Inverse CDF inside the set: renormalise p over members, walk them in
    ascending id and return the first whose cumulative probability exceeds u."""
    ids = np.sort(np.asarray(members, dtype=np.int64))
    q = np.asarray(p, dtype=np.float64)[ids]
    c = np.cumsum(q) / q.sum()
    i = int(np.searchsorted(c, u, side="right"))
    return int(ids[min(i, ids.size - 1)])


def sample(z, *, temperature, top_p=1.0, penalty=1.0, generated=(), u=0.0):
    """One token from logits z: penalty, then greedy (temperature 0) or a
    temperature softmax restricted to the top-p nucleus and drawn with u."""
    if penalty != 1.0:
        z = repetition_penalty(z, generated, penalty)
    if temperature == 0.0:
        return greedy(z)
    p = softmax_temperature(z, temperature)
    return draw(p, nucleus(p, top_p), u)


# --------------------------------------------------------------------------
# The generation loop  [Notes Ch.05 end-to-end loop]
# --------------------------------------------------------------------------

def generate(prompt, model, caches, *, max_new, temperature, top_p=1.0, penalty=1.0,
             eos_id=-1, uniforms=None, bf16_points=False):
    """prompt [B, T] ids (positions 0..T-1); uniforms [max_new, B] (used when
    temperature > 0).  Each row stops at EOS (not appended) or after max_new
    tokens; a finished row appends nothing more.  Returns (list of generated
    id lists, the logits of every step [max_new, B, V] (NaN after a row's
    stop))."""
    prompt = np.asarray(prompt, dtype=np.int64)
    B, T = prompt.shape
    pos = np.tile(np.arange(T), (B, 1))
    logits, caches = model_forward(prompt, pos, model, caches, bf16_points=bf16_points)
    out = [[] for _ in range(B)]
    done = [False] * B
    V = logits.shape[-1]
    seen = np.full((max_new, B, V), np.nan)
    for step in range(max_new):
        nxt = np.zeros(B, dtype=np.int64)
        for b in range(B):
            if done[b]:
                continue
            seen[step, b] = logits[b]
            u = 0.0 if uniforms is None else float(uniforms[step][b])
            t = sample(logits[b], temperature=temperature, top_p=top_p, penalty=penalty,
                       generated=out[b], u=u)
            if t == eos_id:
                done[b] = True
                continue
            out[b].append(t)
            nxt[b] = t
            if len(out[b]) == max_new:
                done[b] = True
        if all(done):
            break
        p = np.full((B, 1), T + step)
        logits, caches = model_forward(nxt[:, None], p, model, caches, bf16_points=bf16_points)
    return out, seen
