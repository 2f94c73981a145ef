"""CPU oracle of the W4 decode step (test infrastructure only).

The arithmetic lives in ``oracle.c`` (plain loops, double accumulation, one f32
rounding per operation); this module binds it with ctypes and composes the
operations in the order the pages give for one decoder layer:

  qkv projection -> full-projection RMSNorm of q and of k -> RoPE (YaRN and its
  magnitude factor on full-attention layers only) -> append k, v at slot pos ->
  GQA attention over the window -> o projection -> h = x + RMSNorm(attn) ->
  gate/up projections -> SwiGLU -> down projection -> y = h + RMSNorm(mlp).

Only tests, the smoke check and the CPU-baseline leg of ``bench.py`` may import
this package. Nothing here is shared with the HIP library.
"""
import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

vp, i64, f64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int


def build(verbose=False):
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-Wall", "-Wextra", "-shared", "-fPIC",
           os.path.join(_HERE, "oracle.c"), "-o", _LIB_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_f16_to_f64.restype = f64
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f64.restype = f64
        L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_unpack_codes.argtypes = [vp, i64, i64, vp]
        L.orc_dequant.argtypes = [vp, vp, vp, i64, i64, i64, ci, vp]
        L.orc_w4_gemv.argtypes = [vp, vp, vp, i64, i64, i64, ci, vp, vp]
        L.orc_bf16_gemv.argtypes = [vp, i64, i64, vp, vp]
        L.orc_rmsnorm.argtypes = [vp, vp, i64, f64, vp]
        L.orc_rmsnorm_residual.argtypes = [vp, vp, vp, i64, f64, vp]
        L.orc_rope_inv_freq.argtypes = [ci, f64, f64, f64, f64, f64, vp]
        L.orc_yarn_attention_factor.restype = f64
        L.orc_yarn_attention_factor.argtypes = [f64]
        L.orc_rope.argtypes = [vp, ci, ci, i64, vp, f64]
        L.orc_attention.argtypes = [vp, vp, vp, ci, ci, ci, i64, i64, i64, f64, vp]
        L.orc_attention_kv.argtypes = [vp, vp, vp, ci, i64, ci, ci, ci, ci, i64, i64, f64, vp]
        L.orc_round_bf16.argtypes = [vp, i64, vp]
        L.orc_swiglu.argtypes = [vp, vp, i64, vp]
        L.orc_argmax.restype = i64
        L.orc_argmax.argtypes = [vp, i64]
        L.orc_embed.argtypes = [vp, i64, vp]
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return a.ctypes.data if a is not None else None


# ---- single operations ---------------------------------------------------------

def f16_to_f64(bits):
    return lib().orc_f16_to_f64(int(bits))


def bf16_to_f64(bits):
    return lib().orc_bf16_to_f64(int(bits))


def unpack_codes(qw, K):
    qw = _c(qw, np.uint32)
    N = qw.size // (K // 8)
    out = np.empty((N, K), np.uint8)
    lib().orc_unpack_codes(_p(qw), N, K, _p(out))
    return out


def dequant(qw, scales, zeros, K, group=128, scale_dtype=0):
    qw = _c(qw, np.uint32)
    sc = _c(scales, np.uint16)
    zw = None if zeros is None else _c(zeros, np.uint32)
    N = qw.size // (K // 8)
    out = np.empty((N, K), np.float32)
    lib().orc_dequant(_p(qw), _p(sc), _p(zw), N, K, group, scale_dtype, _p(out))
    return out


def w4_gemv(qw, scales, zeros, K, x, group=128, scale_dtype=0):
    qw = _c(qw, np.uint32)
    sc = _c(scales, np.uint16)
    zw = None if zeros is None else _c(zeros, np.uint32)
    x = _c(x, np.float32)
    N = qw.size // (K // 8)
    assert x.size == K
    y = np.empty(N, np.float32)
    lib().orc_w4_gemv(_p(qw), _p(sc), _p(zw), N, K, group, scale_dtype, _p(x), _p(y))
    return y


def bf16_gemv(W_bits, x):
    W = _c(W_bits, np.uint16)
    x = _c(x, np.float32)
    N, K = W.shape
    y = np.empty(N, np.float32)
    lib().orc_bf16_gemv(_p(W), N, K, _p(x), _p(y))
    return y


def rmsnorm(x, g, eps=1e-6):
    x = _c(x, np.float32)
    g = _c(g, np.float32)
    y = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(g), x.size, eps, _p(y))
    return y


def rmsnorm_residual(x, g, resid, eps=1e-6):
    x, g, resid = _c(x, np.float32), _c(g, np.float32), _c(resid, np.float32)
    out = np.empty_like(x)
    lib().orc_rmsnorm_residual(_p(x), _p(g), _p(resid), x.size, eps, _p(out))
    return out


def rope_inv_freq(D, theta, yarn_factor=1.0, orig_max=8192, beta_fast=32.0, beta_slow=1.0):
    inv = np.empty(D // 2, np.float64)
    lib().orc_rope_inv_freq(D, theta, yarn_factor, float(orig_max), beta_fast, beta_slow, _p(inv))
    return inv


def yarn_attention_factor(s):
    return lib().orc_yarn_attention_factor(s)


def rope(x, H, D, pos, inv, mscale=1.0):
    x = _c(x, np.float32).copy()
    inv = _c(inv, np.float64)
    lib().orc_rope(_p(x), H, D, pos, _p(inv), mscale)
    return x


def attention(q, Kc, Vc, Hq, Hkv, D, pos, window, scale=None):
    """Attention over f32 caches [Hkv][T_max][D] with key j in slot j."""
    return attention_kv(q, _c(Kc, np.float32), _c(Vc, np.float32), Hq, Hkv, D, pos, window, False, scale)


def attention_kv(q, Kc, Vc, Hq, Hkv, D, pos, window, ring, scale=None):
    """Attention over caches [Hkv][slots][D] in storage layout: f32, or bf16 bits
    (uint16 arrays); key j in slot j mod slots when ``ring``, else in slot j."""
    q = _c(q, np.float32)
    dt = 1 if Kc.dtype == np.uint16 else 0
    Kc, Vc = _c(Kc, Kc.dtype), _c(Vc, Vc.dtype)
    if Vc.dtype != Kc.dtype:
        raise ValueError("K and V caches must share a dtype")
    slots = Kc.size // (Hkv * D)
    if not ring and pos >= slots:
        raise ValueError("position beyond the cache")
    if ring and not (0 < window <= slots):
        raise ValueError("a ring must hold the whole window")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.empty(Hq * D, np.float32)
    lib().orc_attention_kv(_p(q), _p(Kc), _p(Vc), dt, slots, int(bool(ring)), Hq, Hkv, D, pos, window, scale,
                           _p(out))
    return out


def round_bf16(x):
    """bfloat16 bits of f32 values, rounded to nearest even (the store into a bf16
    KV cache)."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_round_bf16(_p(x), x.size, _p(out))
    return out


def swiglu(u, v):
    u, v = _c(u, np.float32), _c(v, np.float32)
    z = np.empty_like(u)
    lib().orc_swiglu(_p(u), _p(v), u.size, _p(z))
    return z


def argmax(x):
    x = _c(x, np.float32)
    return int(lib().orc_argmax(_p(x), x.size))


def sample_top_p(logits, temperature, top_p, u):
    """Token drawn from the logits with temperature and nucleus (top-p) filtering, the
    card's sampling settings being temperature 0.6 and top-p 0.95 ("ATLAS-OLMo-3-32B-
    Think-v4", Benchmarks; Prompting guide). In float64:

      temperature <= 0: greedy, the first index of the maximum;
      p_i proportional to e_i = exp((l_i - max l) / temperature);
      nucleus: the fewest most-probable tokens whose mass reaches top_p (of the total),
        tokens tied with the last one included, i.e. N = {i : e_i >= tau} with tau the
        e of the k-th largest token, k the smallest count whose mass reaches top_p;
      draw: u in [0, 1) is the uniform variate; the token is the first i of N, in
        ascending index order, whose cumulative mass over N exceeds u * mass(N).

    The random variate is an input, so the result is a function of (logits, u)."""
    l = np.asarray(logits, np.float64)
    if temperature <= 0:
        return int(np.argmax(l))
    e = np.exp((l - l.max()) / float(temperature))
    total = e.sum()
    order = np.argsort(-e, kind="stable")        # descending, ties by index
    cum = np.cumsum(e[order])
    k = int(np.searchsorted(cum, float(top_p) * total, side="left"))   # first prefix reaching top_p
    k = min(k, e.size - 1)
    tau = e[order[k]]
    members = np.nonzero(e >= tau)[0]            # ascending index order
    cn = np.cumsum(e[members])
    target = float(u) * cn[-1]
    return int(members[np.searchsorted(cn, target, side="right")])


def embed(row_bits):
    r = _c(row_bits, np.uint16)
    x = np.empty(r.size, np.float32)
    lib().orc_embed(_p(r), r.size, _p(x))
    return x


# ---- one decoder layer ------------------------------------------------------------

FULL = 1


def rope_params(model, layer_type):
    """(inverse frequencies, magnitude factor) of a layer: YaRN and its factor on
    full-attention layers only, plain RoPE on sliding-window layers."""
    if layer_type == FULL and model.yarn_factor > 1.0:
        inv = rope_inv_freq(model.hd, model.theta, model.yarn_factor, model.yarn_orig_max,
                            model.yarn_beta_fast, model.yarn_beta_slow)
        return inv, yarn_attention_factor(model.yarn_factor)
    return rope_inv_freq(model.hd, model.theta), 1.0


def layer_step(model, layer_type, T, x, Kc, Vc, pos, trace=None):
    """One decoder layer for the token at position ``pos``.

    T: the layer's tensors (W4 triples 'qkv', 'o', 'gate', 'up', 'down'; gains
    'g_q', 'g_k', 'g_pa', 'g_pf'). Kc, Vc: [hkv][slots][hd] caches in the model's KV
    format (f32, or bf16 bits when model.kv_dtype == 1; on a sliding-window layer of
    a model with swa_ring, a ring of `window` slots), updated in place at the slot
    of pos. Returns y; fills ``trace`` (a dict) with the intermediates."""
    hq, hkv, hd, d, g = model.hq, model.hkv, model.hd, model.d, model.group
    sd = getattr(model, "scale_dtype", 0)
    kv_dtype = getattr(model, "kv_dtype", 0)
    ring = bool(getattr(model, "swa_ring", False)) and layer_type != FULL and model.window > 0
    qkv = w4_gemv(*T["qkv"], d, x, g, sd)
    q, k, v = qkv[:hq * hd], qkv[hq * hd:(hq + hkv) * hd], qkv[(hq + hkv) * hd:]
    qn = rmsnorm(q, T["g_q"], model.eps)
    kn = rmsnorm(k, T["g_k"], model.eps)
    inv, m = rope_params(model, layer_type)
    qr = rope(qn, hq, hd, pos, inv, m)
    kr = rope(kn, hkv, hd, pos, inv, m)
    slot = pos % Kc.shape[1] if ring else pos
    if kv_dtype == 1:
        Kc[:, slot, :] = round_bf16(kr).reshape(hkv, hd)
        Vc[:, slot, :] = round_bf16(v).reshape(hkv, hd)
    else:
        Kc[:, slot, :] = kr.reshape(hkv, hd)
        Vc[:, slot, :] = v.reshape(hkv, hd)
    window = model.window if layer_type != FULL else 0
    o = attention_kv(qr, Kc, Vc, hq, hkv, hd, pos, window, ring)
    a = w4_gemv(*T["o"], hq * hd, o, g, sd)
    h = rmsnorm_residual(a, T["g_pa"], x, model.eps)
    u = w4_gemv(*T["gate"], d, h, g, sd)
    vv = w4_gemv(*T["up"], d, h, g, sd)
    z = swiglu(u, vv)
    mm = w4_gemv(*T["down"], model.dff, z, g, sd)
    y = rmsnorm_residual(mm, T["g_pf"], h, model.eps)
    if trace is not None:
        trace.update(qkv=qkv, q=qr, k=kr, v=v, o=o, a=a, h=h, u=u, up=vv, z=z, m=mm, y=y)
    return y


def final_logits(y, g_final, lm_head_bits, eps=1e-6):
    """Final RMSNorm (our reading: a post-norm stack normalises the residual stream
    once before the untied bf16 lm_head), then logits = W_lm y_hat."""
    yh = rmsnorm(y, g_final, eps)
    return bf16_gemv(lm_head_bits, yh), yh
