"""Workload recipes: shapes, seeds and value distributions of the synthetic inputs.

A recipe says *what* the decode step is run on (the model's configuration fields
and where every input tensor's bits come from); it says nothing about how the
step is computed. Model fields follow the OLMo-3-32B configuration listed on the
architecture pages (hidden 5,120; 40 query / 8 KV heads of 128; SwiGLU 27,648;
64 layers laid out as three sliding-window layers then one full-attention layer;
window 4,096; RoPE theta 500,000 with YaRN x8 from 8,192 on the full layers;
RMSNorm eps 1e-6; vocabulary 100,278).

Tensor ids are (model_id << 48) | (layer << 16) | kind; the global tensors use
layer 0xFFFF.
"""
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

import synth as S

SWA, FULL = 0, 1

# tensor kinds
K_QKV, K_O, K_GATE, K_UP, K_DOWN = 1, 4, 7, 10, 13  # +0 codes, +1 scales, +2 zeros
K_GQ, K_GK, K_GPA, K_GPF, K_KC, K_VC = 16, 17, 18, 19, 20, 21
K_XIN, K_EMB, K_LM, K_GFIN, K_TOK = 32, 33, 34, 35, 36
GLOBAL_LAYER = 0xFFFF


@dataclass
class Model:
    d: int
    hq: int
    hkv: int
    hd: int
    dff: int
    n_layers: int
    layer_types: List[int]
    window: int = 4096
    group: int = 128
    theta: float = 500000.0
    yarn_factor: float = 8.0          # applied on FULL layers only
    yarn_orig_max: int = 8192
    yarn_beta_fast: float = 32.0
    yarn_beta_slow: float = 1.0
    eps: float = 1e-6
    vocab: int = 100278
    model_id: int = 0
    scale_dtype: int = 0              # 0: f16 group scales, 1: bf16
    symmetric: bool = False           # True: no zero table, every zero point is 8
    kv_dtype: int = 0                 # KV cache elements: 0 f32, 1 bf16
    swa_ring: bool = False            # True: sliding-window layers keep a ring of `window` slots

    @property
    def n_qkv(self):
        return (self.hq + 2 * self.hkv) * self.hd

    def linears(self):
        """(name, tensor kind, N rows, K columns) of every W4 linear in one layer."""
        return [("qkv", K_QKV, self.n_qkv, self.d),
                ("o", K_O, self.d, self.hq * self.hd),
                ("gate", K_GATE, self.dff, self.d),
                ("up", K_UP, self.dff, self.d),
                ("down", K_DOWN, self.d, self.dff)]


def olmo3_32b(model_id=3, n_layers=64):
    types = [FULL if (l % 4) == 3 else SWA for l in range(n_layers)]
    return Model(d=5120, hq=40, hkv=8, hd=128, dff=27648, n_layers=n_layers, layer_types=types,
                 model_id=model_id)


def card_format(m):
    """The card's own W4 recipe on model m: symmetric codes (zero point 8, no zero
    table), group 32, bf16 scales."""
    m.group, m.scale_dtype, m.symmetric = 32, 1, True
    return m


def bf16_ring_kv(m):
    """The card's planned KV format on model m: bf16 elements, and on the
    sliding-window layers a ring of `window` slots (key j in slot j mod window)."""
    m.kv_dtype, m.swa_ring = 1, True
    return m


def tiny(model_id=0):
    return Model(d=640, hq=5, hkv=1, hd=128, dff=1728, n_layers=1, layer_types=[SWA],
                 window=64, model_id=model_id)


@dataclass
class Workload:
    name: str
    model: Model
    seed: int
    n_cached: int              # KV positions 0..n_cached-1 pre-filled; new token at pos = n_cached
    t_max: int                 # KV slots allocated per layer
    layer_types: Optional[List[int]] = None
    use_tokens: bool = False   # config 3/4: embedding input; else x ~ N(0,1)
    final_head: bool = False   # final norm + lm_head + argmax
    prompt_len: int = 0        # prefill only
    batch: int = 1             # batched decode: sequences decoded together
    batch_gap: int = 0         # sequence b holds n_cached - b * batch_gap positions (ragged batch)
    extra: dict = field(default_factory=dict)

    def seq_cached(self, b):
        """Cached positions of sequence b of a batch (its new token sits there)."""
        return self.n_cached - b * self.batch_gap


def config(i):
    """The workload configurations. 0: tiny layer, 1: SWA layer at 4,096 keys, 2: full
    layer at 16,385 keys with YaRN, 3: 64-layer step at 16K, 4: prefill of 1,200 tokens;
    5: config 3 and 6: config 1 in the card's own W4 recipe (symmetric, group 32, bf16
    scales); 7: config 3 with a bf16 KV cache and rings on the sliding-window layers;
    8: the same at 65,535 cached tokens (the YaRN context limit of 65,536); 9: one
    full-size SWA layer at 16,384 cached keys in that KV format (the ring has wrapped); 10:
    config 7 for a batch of 8 sequences decoded together."""
    if i == 0:
        return Workload("tiny-swa-layer", tiny(0), seed=0, n_cached=256, t_max=257)
    if i == 1:
        m = olmo3_32b(model_id=1, n_layers=1)
        m.layer_types = [SWA]
        return Workload("olmo3-32b-swa-layer-4k", m, seed=0, n_cached=4096, t_max=4097)
    if i == 2:
        m = olmo3_32b(model_id=2, n_layers=1)
        m.layer_types = [FULL]
        return Workload("olmo3-32b-full-layer-16k-yarn", m, seed=0, n_cached=16384, t_max=16385)
    if i == 3:
        return Workload("olmo3-32b-w4-decode-16k", olmo3_32b(3), seed=0, n_cached=16384,
                        t_max=16385, use_tokens=True, final_head=True)
    if i == 4:
        return Workload("olmo3-32b-w4-prefill-1200", olmo3_32b(3), seed=0, n_cached=0,
                        t_max=1200, use_tokens=True, final_head=True, prompt_len=1200)
    if i == 5:
        return Workload("olmo3-32b-w4sym-g32-decode-16k", card_format(olmo3_32b(5)), seed=0, n_cached=16384,
                        t_max=16385, use_tokens=True, final_head=True)
    if i == 6:
        m = card_format(olmo3_32b(model_id=6, n_layers=1))
        m.layer_types = [SWA]
        return Workload("olmo3-32b-w4sym-g32-swa-layer-4k", m, seed=0, n_cached=4096, t_max=4097)
    if i == 7:
        return Workload("olmo3-32b-w4-decode-16k-bf16kv-ring", bf16_ring_kv(olmo3_32b(3)), seed=0,
                        n_cached=16384, t_max=16385, use_tokens=True, final_head=True)
    if i == 8:
        return Workload("olmo3-32b-w4-decode-64k-bf16kv-ring", bf16_ring_kv(olmo3_32b(3)), seed=0,
                        n_cached=65535, t_max=65536, use_tokens=True, final_head=True)
    if i == 10:
        return Workload("olmo3-32b-w4-decode-16k-bf16kv-ring-batch8", bf16_ring_kv(olmo3_32b(3)), seed=0,
                        n_cached=16384, t_max=16385, use_tokens=True, final_head=True, batch=8)
    if i == 9:
        m = bf16_ring_kv(olmo3_32b(model_id=1, n_layers=1))
        m.layer_types = [SWA]
        return Workload("olmo3-32b-swa-layer-16k-bf16kv-ring", m, seed=0, n_cached=16384, t_max=16385)
    raise ValueError(i)


def tid(model, layer, kind, seq=0):
    """Tensor id; ``seq`` numbers the sequences of a batch (their caches and tokens),
    sequence 0 being the single-sequence workload's."""
    return (model.model_id << 48) | (layer << 16) | (seq << 8) | kind


def key(wl_or_model, seed, layer, kind):
    m = wl_or_model.model if isinstance(wl_or_model, Workload) else wl_or_model
    return S.key(seed, tid(m, layer, kind))


# ---- per-layer inputs --------------------------------------------------------

def w4_linear(model, seed, layer, kind, N, K):
    """Packed codes [N][K/8] u32, scale bits [N][G] u16 (f16, or bf16 when
    model.scale_dtype == 1), packed zeros [N][ceil(G/8)] u32 (None when the model is
    symmetric). Codes and zeros ~ U{0..15}; scales ~ U(0.002, 0.02) rounded to the
    scale type."""
    G = -(-K // model.group)
    codes = S.codes(S.key(seed, tid(model, layer, kind)), N * K // 8).reshape(N, K // 8)
    uni = S.uniform_bf16 if model.scale_dtype == 1 else S.uniform_f16
    scales = uni(S.key(seed, tid(model, layer, kind + 1)), N * G, 0.002, 0.02).reshape(N, G)
    zeros = None if model.symmetric else S.zeros(S.key(seed, tid(model, layer, kind + 2)), N, G)
    return codes, scales, zeros


def gains(model, seed, layer):
    """RMSNorm gains ~ N(1, 0.02): q-norm [hq*hd], k-norm [hkv*hd], post-attention [d],
    post-feedforward [d]."""
    def g(kind, n):
        return S.normal_f32(S.key(seed, tid(model, layer, kind)), n, 1.0, 0.02)
    return {"g_q": g(K_GQ, model.hq * model.hd), "g_k": g(K_GK, model.hkv * model.hd),
            "g_pa": g(K_GPA, model.d), "g_pf": g(K_GPF, model.d)}


def layer_tensors(model, seed, layer):
    out = {}
    for name, kind, N, K in model.linears():
        out[name] = w4_linear(model, seed, layer, kind, N, K)
    out.update(gains(model, seed, layer))
    return out


def kv_slots(model, layer_type, t_max):
    """Positions stored per KV head: `window` on a sliding-window layer kept as a ring,
    else t_max."""
    return model.window if (model.swa_ring and layer_type == SWA and model.window > 0) else t_max


def kv_np_dtype(model):
    return np.uint16 if model.kv_dtype == 1 else np.float32


def kv_cache_into(model, seed, layer, n_cached, t_max, kdst, vdst, seq=0):
    """K and V caches [hkv][slots][hd] in the model's KV format (f32, or bf16 bits)
    holding positions 0..n_cached-1 ~ N(0,1) (a ring holds the last `slots` of them
    at slot j mod slots); ``seq``: sequence of a batch. Slots not written are left as
    the caller's buffer holds them."""
    slots = kv_slots(model, model.layer_types[layer], t_max)
    j0 = max(0, n_cached - slots)
    for kind, dst in ((K_KC, kdst), (K_VC, vdst)):
        if n_cached > 0:
            S.normal_kv_into(S.key(seed, tid(model, layer, kind, seq)), model.hkv, n_cached, model.hd, j0, slots,
                             model.kv_dtype, 0.0, 1.0, dst)


def kv_cache(model, seed, layer, n_cached, t_max, seq=0):
    slots = kv_slots(model, model.layer_types[layer], t_max)
    Kc = np.zeros((model.hkv, slots, model.hd), kv_np_dtype(model))
    Vc = np.zeros((model.hkv, slots, model.hd), kv_np_dtype(model))
    kv_cache_into(model, seed, layer, n_cached, t_max, Kc, Vc, seq)
    return Kc, Vc


# ---- global inputs -----------------------------------------------------------

def x_in(model, seed):
    return S.normal_f32(S.key(seed, tid(model, GLOBAL_LAYER, K_XIN)), model.d, 0.0, 1.0)


def final_gain(model, seed):
    return S.normal_f32(S.key(seed, tid(model, GLOBAL_LAYER, K_GFIN)), model.d, 1.0, 0.02)


def prompt_tokens(model, seed, n, stream=0):
    return S.tokens(S.key(seed, tid(model, GLOBAL_LAYER, K_TOK) + (stream << 8)), n, model.vocab)


def batch_tokens(wl):
    """The token each sequence of a batch feeds (sequence 0: the single-sequence
    workload's token)."""
    return np.array([int(prompt_tokens(wl.model, wl.seed, 1, stream=b * 16)[0]) for b in range(wl.batch)], np.int32)


def embedding_rows(model, seed, r0, nr):
    """bf16 bits of embedding rows [r0, r0+nr) ~ N(0, 0.02)."""
    return S.normal_bf16_rows(S.key(seed, tid(model, GLOBAL_LAYER, K_EMB)), r0, nr, model.d, 0.0, 0.02)


def lm_head_rows(model, seed, r0, nr):
    """bf16 bits of lm_head rows [r0, r0+nr) ~ N(0, 0.02)."""
    return S.normal_bf16_rows(S.key(seed, tid(model, GLOBAL_LAYER, K_LM)), r0, nr, model.d, 0.0, 0.02)


def emb_key(model, seed):
    return S.key(seed, tid(model, GLOBAL_LAYER, K_EMB))


def lm_key(model, seed):
    return S.key(seed, tid(model, GLOBAL_LAYER, K_LM))
