"""Algorithmic byte and FLOP counts of the decode step and the prefill.

"Algorithmic" bytes are the bytes the step must move at least once per token: every
W4 weight (packed codes, f16 group scales, packed uint4 zeros), the KV entries the
attention reads (f32 or bf16 elements), the bf16 lm_head, the norm gains and the embedding row. Achieved
bandwidth is these bytes divided by measured time.
"""
from dataclasses import dataclass


def w4_bytes(N, K, group=128, scale_bytes=2, zeros=True):
    """Bytes of one W4 linear [N][K]: codes K/2 per row, a scale per group, and the
    group zero points packed eight to a 32-bit word."""
    G = -(-K // group)
    zb = 4 * (-(-G // 8)) if zeros else 0
    return N * (K // 2 + scale_bytes * G + zb)


def layer_w4_bytes(m):
    """W4 bytes of one layer in the model's format (bf16 and f16 scales are both two
    bytes; a symmetric model has no zero table)."""
    zeros = not getattr(m, "symmetric", False)
    return sum(w4_bytes(N, K, m.group, 2, zeros) for _, _, N, K in m.linears())


def layer_weight_count(m):
    return sum(N * K for _, _, N, K in m.linears())


def layer_gain_count(m):
    return m.hq * m.hd + m.hkv * m.hd + 2 * m.d


def keys_read(layer_type, pos, window):
    """Keys a decode step at position pos attends (the window counts the new token)."""
    if layer_type == 1 or window <= 0:
        return pos + 1
    return min(window, pos + 1)


def kv_elem_bytes(m):
    """Bytes of one cached key or value element: 2 for a bf16 cache, else 4."""
    return 2 if getattr(m, "kv_dtype", 0) == 1 else 4


def layer_kv_read_bytes(m, layer_type, pos):
    return 2 * m.hkv * m.hd * kv_elem_bytes(m) * keys_read(layer_type, pos, m.window)


@dataclass
class StepBytes:
    w4: int
    kv: int
    lm_head: int
    small: int

    @property
    def total(self):
        return self.w4 + self.kv + self.lm_head + self.small


def decode_step_bytes(m, pos, n_layers=None, head=True):
    """Algorithmic bytes of one decode step at position pos over n_layers layers
    (plus the embedding row, final gain and bf16 lm_head when ``head``)."""
    n_layers = m.n_layers if n_layers is None else n_layers
    w4 = n_layers * layer_w4_bytes(m)
    kv = sum(layer_kv_read_bytes(m, m.layer_types[l], pos) for l in range(n_layers))
    # gains (f32), the new k/v written to the cache
    small = n_layers * (4 * layer_gain_count(m) + 2 * m.hkv * m.hd * kv_elem_bytes(m))
    lm = 0
    if head:
        lm = m.vocab * m.d * 2
        small += 2 * m.d + 4 * m.d
    return StepBytes(w4, kv, lm, small)


def decode_batch_bytes(m, positions, n_layers=None, head=True):
    """Algorithmic bytes of one batched step: the weights and lm_head once, the KV and
    small vectors of every sequence (sequence b at positions[b])."""
    per = [decode_step_bytes(m, p, n_layers, head) for p in positions]
    return StepBytes(per[0].w4, sum(x.kv for x in per), per[0].lm_head, sum(x.small for x in per))


def decode_flops(m, context, n_layers=None, head=True):
    """2 FLOPs per weight for every linear, 4 per (query head, dim, key) for the
    score and value products, plus the lm_head."""
    n_layers = m.n_layers if n_layers is None else n_layers
    f = 2 * n_layers * layer_weight_count(m)
    f += n_layers * m.hq * m.hd * 4 * context
    if head:
        f += 2 * m.vocab * m.d
    return f


def prefill_flops(m, T, n_layers=None, head=True, window=None):
    """Projections for T tokens plus causal attention (token t attends t+1 keys,
    capped at the window on sliding-window layers) and the last row's lm_head."""
    n_layers = m.n_layers if n_layers is None else n_layers
    f = 2 * n_layers * layer_weight_count(m) * T
    for l in range(n_layers):
        if window is False or m.layer_types[l] == 1:
            keys = T * (T + 1) // 2
        else:
            W = m.window
            keys = sum(min(t + 1, W) for t in range(T)) if T > W else T * (T + 1) // 2
        f += m.hq * m.hd * 4 * keys
    if head:
        f += 2 * m.vocab * m.d
    return f


def param_counts(m):
    per_layer = layer_weight_count(m) + layer_gain_count(m)
    backbone = m.n_layers * per_layer + m.d       # + final norm
    emb_head = 2 * m.vocab * m.d
    return {"per_layer": per_layer, "backbone": backbone, "emb_head": emb_head,
            "total": backbone + emb_head}
