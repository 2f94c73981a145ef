"""Oracle runs of whole workloads (test infrastructure only).

Inputs are regenerated layer by layer from the seeded recipes in ``synth``, so a
64-layer step never holds more than one layer's weights and caches in memory.
"""
import numpy as np

import oracle as O
from synth import workloads as W


def layer_inputs(wl, layer, n_cached=None, seq=0):
    m = wl.model
    T = W.layer_tensors(m, wl.seed, layer)
    Kc, Vc = W.kv_cache(m, wl.seed, layer, wl.n_cached if n_cached is None else n_cached, wl.t_max, seq)
    return T, Kc, Vc


def run_layer(wl, layer=0, x=None, trace=None):
    """One layer of workload ``wl`` at pos = wl.n_cached. Returns (y, Kc, Vc)."""
    m = wl.model
    T, Kc, Vc = layer_inputs(wl, layer)
    if x is None:
        x = W.x_in(m, wl.seed)
    y = O.layer_step(m, m.layer_types[layer], T, x, Kc, Vc, wl.n_cached, trace)
    return y, Kc, Vc


def decode_token(wl):
    """The token the decode workload feeds (first draw of the prompt stream)."""
    return int(W.prompt_tokens(wl.model, wl.seed, 1)[0])


def run_decode(wl, n_layers=None, token=None, keep_hidden=False, seq=0, keep_kv=False):
    """Full decode step: embed -> n_layers layers -> final norm -> bf16 lm_head ->
    argmax, for sequence ``seq`` of the workload (its own caches, at position
    wl.seq_cached(seq)). Returns dict(logits, argmax, y, hidden=[per-layer outputs],
    and with keep_kv the new key/value of every layer: kv=[(k, v)])."""
    m = wl.model
    n_layers = m.n_layers if n_layers is None else n_layers
    if token is None:
        token = decode_token(wl)
    pos = wl.seq_cached(seq)
    x = O.embed(W.embedding_rows(m, wl.seed, token, 1)[0])
    hidden = []
    kv = []
    for l in range(n_layers):
        T, Kc, Vc = layer_inputs(wl, l, pos, seq)
        tr = {} if keep_kv else None
        x = O.layer_step(m, m.layer_types[l], T, x, Kc, Vc, pos, tr)
        if keep_kv:
            kv.append((tr["k"], tr["v"]))
        if keep_hidden:
            hidden.append(x.copy())
        del T, Kc, Vc
    out = {"y": x, "token": token, "hidden": hidden, "kv": kv}
    if wl.final_head:
        lm = W.lm_head_rows(m, wl.seed, 0, m.vocab)
        logits, yh = O.final_logits(x, W.final_gain(m, wl.seed), lm, m.eps)
        out.update(logits=logits, argmax=O.argmax(logits), y_hat=yh)
    return out


def run_decode_batch(wl, n_layers=None, keep_kv=False):
    """A batched decode step is, by definition, one independent decode step per
    sequence (own token, position and caches; shared weights)."""
    toks = W.batch_tokens(wl)
    return [run_decode(wl, n_layers, int(toks[b]), seq=b, keep_kv=keep_kv) for b in range(wl.batch)]


def run_prefill(wl, tokens, n_layers=None, final=True):
    """Prefill as its definition: teacher-forced decode of ``tokens`` at positions
    start..start+n-1 over n_layers layers, writing every KV slot. Returns
    dict(K=[layer caches], V=[...], logits, argmax, y) for the last token."""
    m = wl.model
    n_layers = m.n_layers if n_layers is None else n_layers
    start = wl.n_cached
    Ts = [W.layer_tensors(m, wl.seed, l) for l in range(n_layers)]
    caches = [W.kv_cache(m, wl.seed, l, wl.n_cached, wl.t_max) for l in range(n_layers)]
    emb_rows = {}
    x = None
    for t, tok in enumerate(tokens):
        tok = int(tok)
        if tok not in emb_rows:
            emb_rows[tok] = W.embedding_rows(m, wl.seed, tok, 1)[0]
        x = O.embed(emb_rows[tok])
        for l in range(n_layers):
            Kc, Vc = caches[l]
            x = O.layer_step(m, m.layer_types[l], Ts[l], x, Kc, Vc, start + t)
    out = {"K": [c[0] for c in caches], "V": [c[1] for c in caches], "y": x}
    if final and wl.final_head:
        lm = W.lm_head_rows(m, wl.seed, 0, m.vocab)
        logits, _ = O.final_logits(x, W.final_gain(m, wl.seed), lm, m.eps)
        out.update(logits=logits, argmax=O.argmax(logits))
    return out
