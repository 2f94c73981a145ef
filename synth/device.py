"""Upload seeded synthetic workloads to device memory (torch tensors) and wrap them
as the C-ABI descriptors of swa_attention_amd.ops. Input plumbing only."""
import numpy as np
import torch

from synth import workloads as W


def _t(arr, device):
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device, non_blocking=False)


def w4_to_device(codes, scales, zeros, K, device, group=128, scale_dtype=0):
    from swa_attention_amd.ops import W4
    N = codes.shape[0]
    return W4(_t(codes, device), _t(scales, device), None if zeros is None else _t(zeros, device), N, K, group,
              scale_dtype)


def rope_structs(model):
    from swa_attention_amd.ops import rope_params
    swa = rope_params(model.theta, 1.0, model.yarn_orig_max, model.yarn_beta_fast, model.yarn_beta_slow, 0.0)
    full = rope_params(model.theta, model.yarn_factor, model.yarn_orig_max, model.yarn_beta_fast,
                       model.yarn_beta_slow, 0.0)
    return swa, full


def layer_to_device(model, seed, layer, n_cached, t_max, device, tensors=None, seq_cached=None):
    """One layer's weights, gains and caches on the device. seq_cached: cached
    positions of each sequence of a batch (the caches then hold the sequences back to
    back, [batch][hkv][slots][hd]); None: one sequence with n_cached positions."""
    from swa_attention_amd.ops import Layer
    T = tensors if tensors is not None else W.layer_tensors(model, seed, layer)
    ws = {}
    for name, kind, N, K in model.linears():
        c, s, z = T[name]
        ws[name] = w4_to_device(c, s, z, K, device, model.group, model.scale_dtype)
    # caches in the model's KV format: [hkv][slots][hd] f32, or bf16 bits held as int16
    slots = W.kv_slots(model, model.layer_types[layer], t_max)
    tdt = torch.int16 if model.kv_dtype == 1 else torch.float32
    seqs = [n_cached] if seq_cached is None else list(seq_cached)
    shape = (model.hkv, slots, model.hd) if seq_cached is None else (len(seqs), model.hkv, slots, model.hd)
    Kc = torch.zeros(shape, dtype=tdt, device=device)
    Vc = torch.zeros_like(Kc)
    for b, nc in enumerate(seqs):
        if nc > 0:
            hk = np.zeros((model.hkv, slots, model.hd), W.kv_np_dtype(model))
            hv = np.zeros((model.hkv, slots, model.hd), W.kv_np_dtype(model))
            W.kv_cache_into(model, seed, layer, nc, t_max, hk, hv, seq=b)
            kd = Kc if seq_cached is None else Kc[b]
            vd = Vc if seq_cached is None else Vc[b]
            kd.copy_(torch.from_numpy(hk.view(np.int16) if model.kv_dtype == 1 else hk))
            vd.copy_(torch.from_numpy(hv.view(np.int16) if model.kv_dtype == 1 else hv))
    g = {k: _t(T[k], device) for k in ("g_q", "g_k", "g_pa", "g_pf")}
    return Layer(ws["qkv"], ws["o"], ws["gate"], ws["up"], ws["down"], g["g_q"], g["g_k"], g["g_pa"], g["g_pf"],
                 Kc, Vc, model.layer_types[layer])


def bf16_table_to_device(model, seed, which, device, chunk_rows=8192):
    """bf16 [vocab][d] table ('emb' or 'lm') generated in row chunks."""
    out = torch.empty((model.vocab, model.d), dtype=torch.int16, device=device)
    gen = W.embedding_rows if which == "emb" else W.lm_head_rows
    for r0 in range(0, model.vocab, chunk_rows):
        nr = min(chunk_rows, model.vocab - r0)
        out[r0:r0 + nr].copy_(torch.from_numpy(gen(model, seed, r0, nr).view(np.int16)))
    return out


def build_model(wl, device="cuda", n_layers=None, head=None, progress=None):
    """Device model of workload ``wl`` (layers 0..n_layers-1, caches pre-filled with
    wl.n_cached positions)."""
    from swa_attention_amd.ops import Model
    m = wl.model
    n_layers = m.n_layers if n_layers is None else n_layers
    head = wl.final_head if head is None else head
    swa, full = rope_structs(m)
    dm = Model(m.d, m.hq, m.hkv, m.hd, m.dff, m.window, m.vocab, m.eps, wl.t_max, swa, full,
               kv_dtype=m.kv_dtype, swa_ring=int(m.swa_ring))
    seq_cached = [wl.seq_cached(b) for b in range(wl.batch)] if wl.batch > 1 else None
    for l in range(n_layers):
        dm.layers.append(layer_to_device(m, wl.seed, l, wl.n_cached, wl.t_max, device, seq_cached=seq_cached))
        if progress:
            progress(l)
    if wl.use_tokens or head:
        dm.embedding = bf16_table_to_device(m, wl.seed, "emb", device)
    if head:
        dm.lm_head = bf16_table_to_device(m, wl.seed, "lm", device)
        dm.g_final = _t(W.final_gain(m, wl.seed), device)
    return dm
