"""Seeded synthetic inputs shared by the oracle runner and the GPU harness.

Only bit generation and distribution mapping live here (see ``synth.c`` for the
exact definition); none of the decode step's arithmetic does. Every function has
two forms: one returning a fresh numpy array, and one writing into a caller
buffer given as a numpy array or a raw host address (for pinned staging memory).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

u64, i64, f32, f64 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float, ctypes.c_double
vp = ctypes.c_void_p


def build(verbose=False):
    """Compile libsynth.so with gcc (OpenMP, no FP contraction)."""
    import subprocess
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-Wall", "-shared", "-fPIC",
           os.path.join(_HERE, "synth.c"), "-o", _LIB_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(_LIB_PATH)
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u64]
        L.synth_hash.restype = u64
        L.synth_hash.argtypes = [u64, u64]
        L.synth_codes_u32.argtypes = [u64, i64, vp]
        L.synth_zeros_u32.argtypes = [u64, i64, i64, vp]
        L.synth_uniform_f16.argtypes = [u64, i64, f64, f64, vp]
        L.synth_uniform_bf16.argtypes = [u64, i64, f64, f64, vp]
        L.synth_normal_f32_3d.argtypes = [u64, i64, i64, i64, i64, i64, f32, f32, vp]
        L.synth_normal_f32.argtypes = [u64, i64, f32, f32, vp]
        L.synth_normal_kv.argtypes = [u64, i64, i64, i64, i64, i64, ctypes.c_int, f32, f32, vp]
        L.synth_normal_bf16_rows.argtypes = [u64, i64, i64, i64, f32, f32, vp]
        L.synth_tokens.argtypes = [u64, i64, i64, vp]
        L.synth_raw.argtypes = [u64, i64, vp]
        L.synth_f64_to_f16.restype = ctypes.c_uint16
        L.synth_f64_to_f16.argtypes = [f64]
        _lib = L
    return _lib


def _ptr(buf, nbytes_needed):
    if isinstance(buf, np.ndarray):
        if not buf.flags["C_CONTIGUOUS"]:
            raise ValueError("destination must be C-contiguous")
        if buf.nbytes < nbytes_needed:
            raise ValueError(f"destination too small: {buf.nbytes} < {nbytes_needed}")
        return buf.ctypes.data
    return int(buf)  # raw host address; caller guarantees the size


def key(seed, tensor_id):
    return lib().synth_key(seed & (2**64 - 1), tensor_id & (2**64 - 1))


def raw(k, n):
    out = np.empty(n, np.uint64)
    lib().synth_raw(k, n, out.ctypes.data)
    return out


def codes_into(k, n_words, dst):
    lib().synth_codes_u32(k, n_words, _ptr(dst, 4 * n_words))


def codes(k, n_words):
    out = np.empty(n_words, np.uint32)
    codes_into(k, n_words, out)
    return out


def zeros_into(k, N, G, dst):
    lib().synth_zeros_u32(k, N, G, _ptr(dst, 4 * N * ((G + 7) // 8)))


def zeros(k, N, G):
    out = np.empty((N, (G + 7) // 8), np.uint32)
    zeros_into(k, N, G, out)
    return out


def uniform_f16_into(k, n, a, b, dst):
    lib().synth_uniform_f16(k, n, a, b, _ptr(dst, 2 * n))


def uniform_f16(k, n, a, b):
    """Raw binary16 bits (uint16) of U(a, b) draws."""
    out = np.empty(n, np.uint16)
    uniform_f16_into(k, n, a, b, out)
    return out


def uniform_bf16(k, n, a, b):
    out = np.empty(n, np.uint16)
    lib().synth_uniform_bf16(k, n, a, b, out.ctypes.data)
    return out


def normal_f32_3d_into(k, A, B, C, sa, sb, mu, sigma, dst):
    need = 4 * ((A - 1) * sa + (B - 1) * sb + C) if A and B and C else 0
    lib().synth_normal_f32_3d(k, A, B, C, sa, sb, mu, sigma, _ptr(dst, need))


def normal_kv_into(k, A, B, C, j0, slots, dtype, mu, sigma, dst):
    """Positions [j0, B) of an [A][B][C] N(mu, sigma) stream into slot j mod slots of
    dst ([A][slots][C], f32 for dtype 0, bf16 bits for dtype 1); see synth.c."""
    if not (0 <= j0 <= B and slots >= 1 and (B - j0) <= slots):
        raise ValueError("positions do not fit the slots")
    need = A * slots * C * (2 if dtype == 1 else 4)
    lib().synth_normal_kv(k, A, B, C, j0, slots, dtype, mu, sigma, _ptr(dst, need))


def normal_f32(k, n, mu=0.0, sigma=1.0):
    out = np.empty(n, np.float32)
    lib().synth_normal_f32(k, n, mu, sigma, out.ctypes.data)
    return out


def normal_bf16_rows_into(k, r0, nr, C, mu, sigma, dst):
    lib().synth_normal_bf16_rows(k, r0, nr, C, mu, sigma, _ptr(dst, 2 * nr * C))


def normal_bf16_rows(k, r0, nr, C, mu=0.0, sigma=1.0):
    """Raw bfloat16 bits (uint16) of rows [r0, r0+nr) of an N(mu, sigma) matrix."""
    out = np.empty((nr, C), np.uint16)
    normal_bf16_rows_into(k, r0, nr, C, mu, sigma, out)
    return out


def tokens(k, n, vocab):
    out = np.empty(n, np.int32)
    lib().synth_tokens(k, n, vocab, out.ctypes.data)
    return out


def f64_to_f16_bits(v):
    return lib().synth_f64_to_f16(float(v))
