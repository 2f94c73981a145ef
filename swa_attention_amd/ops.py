"""Thin Python wrappers over the C ABI with the entry points' names.

Tensors are torch CUDA (HIP) tensors; PyTorch provides device memory and the
stream, every computation runs in libatlas.so. Each wrapper validates dtype and
contiguity, marshals pointers and raises AtlasError on a non-zero status.
"""
import ctypes
from dataclasses import dataclass, field
from typing import List, Optional

import torch

from . import _lib as L

F32, U16, I32 = torch.float32, torch.int16, torch.int32


def _dev(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


# ---- W4 linear --------------------------------------------------------------------------------

@dataclass
class W4:
    """A packed W4 linear held in device memory: qweight int32 [N][K/8], scales int16
    (f16 or bf16 bits) [N][G], zeros int32 [N][ceil(G/8)] or None."""
    qweight: torch.Tensor
    scales: torch.Tensor
    zeros: Optional[torch.Tensor]
    N: int
    K: int
    group: int = 128
    scale_dtype: int = 0

    def c(self):
        return L.atlas_w4(self.qweight.data_ptr(), self.scales.data_ptr(),
                          self.zeros.data_ptr() if self.zeros is not None else None,
                          self.N, self.K, self.group, self.scale_dtype)


def atlas_w4_gemv_workspace_bytes(w: W4):
    return L.lib().atlas_w4_gemv_workspace_bytes(ctypes.byref(w.c()))


def atlas_w4_gemv(w: W4, x, y=None, ws=None, stream=None):
    _dev(x, F32, "x")
    if y is None:
        y = torch.empty(w.N, dtype=F32, device=x.device)
    _dev(y, F32, "y")
    need = atlas_w4_gemv_workspace_bytes(w)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    L.call("atlas_w4_gemv", ctypes.byref(w.c()), L.ptr(x), L.ptr(y), L.ptr(ws), ws.numel(), L.stream_ptr(stream))
    return y


def atlas_w4_gemv_batch_workspace_bytes(w: W4, B: int):
    return L.lib().atlas_w4_gemv_batch_workspace_bytes(ctypes.byref(w.c()), int(B))


def atlas_w4_gemv_batch(w: W4, x, y=None, ws=None, stream=None):
    """x: f32 [B][K] on the device; returns y f32 [B][N]."""
    _dev(x, F32, "x")
    if x.dim() != 2 or x.shape[1] != w.K or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B][K] tensor")
    B = x.shape[0]
    if y is None:
        y = torch.empty((B, w.N), dtype=F32, device=x.device)
    _dev(y, F32, "y")
    need = atlas_w4_gemv_batch_workspace_bytes(w, B)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    L.call("atlas_w4_gemv_batch", ctypes.byref(w.c()), L.ptr(x), B, L.ptr(y), L.ptr(ws), ws.numel(),
           L.stream_ptr(stream))
    return y


def atlas_w4_dequant(w: W4, out=None, stream=None):
    if out is None:
        out = torch.empty((w.N, w.K), dtype=F32, device=w.qweight.device)
    _dev(out, F32, "out")
    L.call("atlas_w4_dequant", ctypes.byref(w.c()), L.ptr(out), L.stream_ptr(stream))
    return out


def atlas_w4_gemm_workspace_bytes(w: W4, M):
    return L.lib().atlas_w4_gemm_workspace_bytes(ctypes.byref(w.c()), M)


def atlas_w4_gemm(w: W4, A, C=None, ws=None, stream=None):
    """C [M][N] = A [M][K] W^T on the matrix cores (A f32, row-major)."""
    _dev(A, F32, "A")
    M = A.shape[0]
    if C is None:
        C = torch.empty((M, w.N), dtype=F32, device=A.device)
    _dev(C, F32, "C")
    need = atlas_w4_gemm_workspace_bytes(w, M)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=A.device)
    L.call("atlas_w4_gemm", ctypes.byref(w.c()), L.ptr(A), M, L.ptr(C), L.ptr(ws), ws.numel(), L.stream_ptr(stream))
    return C


# ---- norms, rotary, attention -------------------------------------------------------------------

def atlas_rmsnorm_residual(x, g, resid=None, out=None, eps=1e-6, stream=None):
    _dev(x, F32, "x"), _dev(g, F32, "g"), _dev(resid, F32, "resid")
    if out is None:
        out = torch.empty_like(x)
    L.call("atlas_rmsnorm_residual", L.ptr(x), L.ptr(g), L.ptr(resid), L.ptr(out), x.numel(), eps,
           L.stream_ptr(stream))
    return out


def rope_params(theta=500000.0, yarn_factor=1.0, orig_max_pos=8192, beta_fast=32.0, beta_slow=1.0,
                attention_factor=0.0):
    return L.atlas_rope(theta, yarn_factor, float(orig_max_pos), beta_fast, beta_slow, attention_factor)


def atlas_qk_norm_rope(q, k, gq, gk, Hq, Hkv, D, d_pos, rope, eps=1e-6, stream=None):
    for t, n in ((q, "q"), (k, "k"), (gq, "gq"), (gk, "gk")):
        _dev(t, F32, n)
    _dev(d_pos, I32, "d_pos")
    L.call("atlas_qk_norm_rope", L.ptr(q), L.ptr(k), L.ptr(gq), L.ptr(gk), Hq, Hkv, D, L.ptr(d_pos),
           ctypes.byref(rope), eps, L.stream_ptr(stream))
    return q, k


def atlas_gqa_decode_workspace_bytes(Hq, Hkv, D, T_max):
    return L.lib().atlas_gqa_decode_workspace_bytes(Hq, Hkv, D, T_max)


def atlas_gqa_decode(q, k_cache, v_cache, Hq, Hkv, D, T_max, d_pos, window, scale=None, out=None, ws=None,
                     stream=None):
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, F32, n)
    _dev(d_pos, I32, "d_pos")
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty(Hq * D, dtype=F32, device=q.device)
    need = atlas_gqa_decode_workspace_bytes(Hq, Hkv, D, T_max)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    L.call("atlas_gqa_decode", L.ptr(q), L.ptr(k_cache), L.ptr(v_cache), Hq, Hkv, D, T_max, L.ptr(d_pos), window,
           scale, L.ptr(out), L.ptr(ws), ws.numel(), L.stream_ptr(stream))
    return out


def atlas_gqa_decode_kv(q, k_cache, v_cache, Hq, Hkv, D, d_pos, window, ring=False, scale=None, out=None, ws=None,
                        stream=None):
    """Decode attention over caches [Hkv][slots][D] of f32 or bf16 (torch.bfloat16 or
    raw int16/uint16 bits); ``ring``: key j in slot j mod slots."""
    _dev(q, F32, "q")
    if k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must share a dtype")
    if k_cache.dtype == F32:
        kv_dtype = 0
    elif k_cache.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        kv_dtype = 1
    else:
        raise TypeError(f"unsupported cache dtype {k_cache.dtype}")
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, k_cache.dtype, n)
    _dev(d_pos, I32, "d_pos")
    slots = k_cache.numel() // (Hkv * D)
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty(Hq * D, dtype=F32, device=q.device)
    need = atlas_gqa_decode_workspace_bytes(Hq, Hkv, D, slots)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    layout = L.atlas_kv_layout(kv_dtype, int(bool(ring)), slots)
    L.call("atlas_gqa_decode_kv", L.ptr(q), L.ptr(k_cache), L.ptr(v_cache), ctypes.byref(layout), Hq, Hkv, D,
           L.ptr(d_pos), window, scale, L.ptr(out), L.ptr(ws), ws.numel(), L.stream_ptr(stream))
    return out


# ---- model --------------------------------------------------------------------------------------

@dataclass
class Layer:
    qkv: W4
    o: W4
    gate: W4
    up: W4
    down: W4
    g_q: torch.Tensor
    g_k: torch.Tensor
    g_pa: torch.Tensor
    g_pf: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    type: int

    def c(self):
        return L.atlas_layer(self.qkv.c(), self.o.c(), self.gate.c(), self.up.c(), self.down.c(),
                             self.g_q.data_ptr(), self.g_k.data_ptr(), self.g_pa.data_ptr(), self.g_pf.data_ptr(),
                             self.k_cache.data_ptr(), self.v_cache.data_ptr(), self.type)


@dataclass
class Model:
    d: int
    hq: int
    hkv: int
    hd: int
    dff: int
    window: int
    vocab: int
    eps: float
    t_max: int
    rope_swa: object
    rope_full: object
    layers: List[Layer] = field(default_factory=list)
    embedding: Optional[torch.Tensor] = None
    g_final: Optional[torch.Tensor] = None
    lm_head: Optional[torch.Tensor] = None
    kv_dtype: int = 0          # 0: f32 caches, 1: bf16
    swa_ring: int = 0          # 1: sliding-window layers keep a ring of `window` slots
    _c: object = None
    _arr: object = None

    def c(self):
        """The atlas_model struct (rebuilt when the layer list changes)."""
        arr = (L.atlas_layer * len(self.layers))(*[l.c() for l in self.layers])
        self._arr = arr
        self._c = L.atlas_model(self.d, self.hq, self.hkv, self.hd, self.dff, len(self.layers), self.window,
                                self.vocab, self.eps, self.t_max, self.rope_swa, self.rope_full,
                                ctypes.cast(arr, ctypes.POINTER(L.atlas_layer)),
                                None if self.embedding is None else self.embedding.data_ptr(),
                                None if self.g_final is None else self.g_final.data_ptr(),
                                None if self.lm_head is None else self.lm_head.data_ptr(),
                                self.kv_dtype, self.swa_ring)
        return self._c


def atlas_decode_workspace_bytes(m: Model):
    return L.lib().atlas_decode_workspace_bytes(ctypes.byref(m.c()))


def atlas_decode_step(m: Model, d_pos, d_token=None, hidden_in=None, hidden_out=None, logits=None, argmax=None,
                      ws=None, stream=None, cm=None):
    """One decode step. ``cm``: a prebuilt atlas_model struct (m.c()) to skip rebuilding."""
    cm = cm if cm is not None else m.c()
    L.call("atlas_decode_step", ctypes.byref(cm), L.ptr(d_token), L.ptr(hidden_in), L.ptr(d_pos),
           L.ptr(hidden_out), L.ptr(logits), L.ptr(argmax), L.ptr(ws), 0 if ws is None else ws.numel(),
           L.stream_ptr(stream))


def atlas_decode_step_noalloc(m: Model, d_pos, d_token=None, hidden_in=None, hidden_out=None, logits=None,
                              argmax=None, status_out=None, stream=None, cm=None):
    """One decode step on the library's fixed scratch area (no workspace argument)."""
    for t, n, dt in ((d_pos, "d_pos", I32), (d_token, "d_token", I32), (hidden_in, "hidden_in", F32),
                     (hidden_out, "hidden_out", F32), (logits, "logits", F32), (argmax, "argmax", I32),
                     (status_out, "status_out", I32)):
        _dev(t, dt, n)
    cm = cm if cm is not None else m.c()
    L.call("atlas_decode_step_noalloc", ctypes.byref(cm), L.ptr(d_token), L.ptr(hidden_in), L.ptr(d_pos),
           L.ptr(hidden_out), L.ptr(logits), L.ptr(argmax), L.ptr(status_out), L.stream_ptr(stream))


def atlas_decode_batch_workspace_bytes(m: Model, batch):
    return L.lib().atlas_decode_batch_workspace_bytes(ctypes.byref(m.c()), batch)


def atlas_decode_batch(m: Model, d_tokens, d_pos, hidden_out=None, logits=None, argmax=None, ws=None, stream=None,
                       cm=None):
    """One token for each of len(d_tokens) sequences; every layer's caches hold the
    sequences back to back ([batch][Hkv][slots][D])."""
    _dev(d_tokens, I32, "d_tokens")
    _dev(d_pos, I32, "d_pos")
    B = d_tokens.numel()
    if d_pos.numel() != B:
        raise ValueError("d_tokens and d_pos must have one entry per sequence")
    for t, n, dt in ((hidden_out, "hidden_out", F32), (logits, "logits", F32), (argmax, "argmax", I32)):
        _dev(t, dt, n)
    c = cm if cm is not None else m.c()
    if ws is None:
        ws = torch.empty(max(L.lib().atlas_decode_batch_workspace_bytes(ctypes.byref(c), B), 1), dtype=torch.uint8,
                         device=d_tokens.device)
    L.call("atlas_decode_batch", ctypes.byref(c), L.ptr(d_tokens), L.ptr(d_pos), B, L.ptr(hidden_out), L.ptr(logits),
           L.ptr(argmax), L.ptr(ws), ws.numel(), L.stream_ptr(stream))
    return ws


def atlas_device_status(ws, stream=None):
    out = ctypes.c_int32(-1)
    L.call("atlas_device_status", L.ptr(ws), L.stream_ptr(stream), ctypes.byref(out))
    return out.value


def atlas_prefill_workspace_bytes(m: Model, n_tokens):
    return L.lib().atlas_prefill_workspace_bytes(ctypes.byref(m.c()), n_tokens)


def atlas_prefill(m: Model, d_tokens, start_pos=0, logits=None, argmax=None, ws=None, stream=None, cm=None):
    cm = cm if cm is not None else m.c()
    _dev(d_tokens, I32, "tokens")
    L.call("atlas_prefill", ctypes.byref(cm), L.ptr(d_tokens), d_tokens.numel(), start_pos, L.ptr(logits),
           L.ptr(argmax), L.ptr(ws), 0 if ws is None else ws.numel(), L.stream_ptr(stream))


# ---- read-bandwidth probe (measurement aid) ------------------------------------------------------

def atlas_sample_workspace_bytes(vocab):
    return L.lib().atlas_sample_workspace_bytes(vocab)


def atlas_sample(logits, temperature, top_p=1.0, d_u=None, token=None, ws=None, stream=None):
    """Next token from device logits (f32 [vocab]) with temperature and nucleus
    filtering; d_u: device f32 [1] uniform variate (unused when temperature == 0)."""
    _dev(logits, F32, "logits")
    if d_u is not None:
        _dev(d_u, F32, "d_u")
    if token is None:
        token = torch.empty(1, dtype=I32, device=logits.device)
    _dev(token, I32, "token")
    V = logits.numel()
    if ws is None:
        ws = torch.empty(max(atlas_sample_workspace_bytes(V), 1), dtype=torch.uint8, device=logits.device)
    L.call("atlas_sample", L.ptr(logits), V, float(temperature), float(top_p), L.ptr(d_u), L.ptr(token), L.ptr(ws),
           ws.numel(), L.stream_ptr(stream))
    return token


def atlas_stream_read(buf, blocks=512, sink=None, stream=None):
    """Plain streaming read of the device tensor `buf` (its bytes, a multiple of 16) by
    `blocks` blocks of 256 threads; returns the one-word sink."""
    if not buf.is_cuda:
        raise ValueError("buf must be a device tensor")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    L.call("atlas_stream_read", L.ptr(buf), buf.numel() * buf.element_size(), L.ptr(sink), blocks,
           L.stream_ptr(stream))
    return sink


# ---- launch timing -------------------------------------------------------------------------------

def atlas_profile_start(capacity=100000):
    L.call("atlas_profile_start", capacity)


def atlas_profile_stop(max_entries=64):
    """{label: (launch count, total ms)} of the launches since atlas_profile_start."""
    arr = (L.atlas_profile_entry * max_entries)()
    n = ctypes.c_int32(0)
    L.call("atlas_profile_stop", arr, max_entries, ctypes.byref(n))
    return {arr[i].name.decode(): (arr[i].count, arr[i].total_ms) for i in range(n.value)}
