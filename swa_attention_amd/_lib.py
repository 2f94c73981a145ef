"""ctypes binding of libatlas.so: the C-ABI structs and entry points under the same
names as include/atlas.h. Argument marshalling only; every step runs in the HIP
library. Loading fails loudly when the library has not been built."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libatlas.so")

c_int32, c_int64, c_size_t, c_float, c_double, c_void_p = (
    ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_double, ctypes.c_void_p)

ATLAS_OK, ATLAS_ERR_INVALID_ARG, ATLAS_ERR_UNSUPPORTED_SHAPE, ATLAS_ERR_WORKSPACE_TOO_SMALL, ATLAS_ERR_HIP = range(5)


class atlas_w4(ctypes.Structure):
    _fields_ = [("qweight", c_void_p), ("scales", c_void_p), ("zeros", c_void_p),
                ("N", c_int32), ("K", c_int32), ("group", c_int32), ("scale_dtype", c_int32)]


class atlas_rope(ctypes.Structure):
    _fields_ = [("theta", c_double), ("yarn_factor", c_double), ("orig_max_pos", c_double),
                ("beta_fast", c_double), ("beta_slow", c_double), ("attention_factor", c_double)]


class atlas_layer(ctypes.Structure):
    _fields_ = [("qkv", atlas_w4), ("o", atlas_w4), ("gate", atlas_w4), ("up", atlas_w4), ("down", atlas_w4),
                ("g_q", c_void_p), ("g_k", c_void_p), ("g_pa", c_void_p), ("g_pf", c_void_p),
                ("k_cache", c_void_p), ("v_cache", c_void_p), ("type", c_int32)]


class atlas_model(ctypes.Structure):
    _fields_ = [("d", c_int32), ("hq", c_int32), ("hkv", c_int32), ("hd", c_int32), ("dff", c_int32),
                ("n_layers", c_int32), ("window", c_int32), ("vocab", c_int32), ("eps", c_float),
                ("t_max", c_int64), ("rope_swa", atlas_rope), ("rope_full", atlas_rope),
                ("layers", ctypes.POINTER(atlas_layer)), ("embedding", c_void_p), ("g_final", c_void_p),
                ("lm_head", c_void_p), ("kv_dtype", c_int32), ("swa_ring", c_int32)]


class atlas_kv_layout(ctypes.Structure):
    _fields_ = [("kv_dtype", c_int32), ("ring", c_int32), ("slots", c_int64)]


class atlas_profile_entry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("count", c_int32), ("total_ms", c_double)]


P = ctypes.POINTER
_SIGS = {
    "atlas_version": (ctypes.c_char_p, []),
    "atlas_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "atlas_last_error": (ctypes.c_char_p, []),
    "atlas_w4_gemv_workspace_bytes": (c_size_t, [P(atlas_w4)]),
    "atlas_w4_gemv": (ctypes.c_int, [P(atlas_w4), c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "atlas_w4_dequant": (ctypes.c_int, [P(atlas_w4), c_void_p, c_void_p]),
    "atlas_w4_gemv_batch_workspace_bytes": (c_size_t, [P(atlas_w4), c_int32]),
    "atlas_w4_gemv_batch": (ctypes.c_int, [P(atlas_w4), c_void_p, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "atlas_w4_gemm_workspace_bytes": (c_size_t, [P(atlas_w4), c_int32]),
    "atlas_w4_gemm": (ctypes.c_int, [P(atlas_w4), c_void_p, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "atlas_rmsnorm_residual": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float, c_void_p]),
    "atlas_qk_norm_rope": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                          c_void_p, P(atlas_rope), c_float, c_void_p]),
    "atlas_gqa_decode_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int64]),
    "atlas_gqa_decode": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int64,
                                        c_void_p, c_int32, c_float, c_void_p, c_void_p, c_size_t, c_void_p]),
    "atlas_gqa_decode_kv": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, P(atlas_kv_layout), c_int32, c_int32,
                                           c_int32, c_void_p, c_int32, c_float, c_void_p, c_void_p, c_size_t,
                                           c_void_p]),
    "atlas_decode_workspace_bytes": (c_size_t, [P(atlas_model)]),
    "atlas_decode_step": (ctypes.c_int, [P(atlas_model), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_size_t, c_void_p]),
    "atlas_device_status": (ctypes.c_int, [c_void_p, c_void_p, P(c_int32)]),
    "atlas_decode_step_noalloc": (ctypes.c_int, [P(atlas_model), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                                 c_void_p, c_void_p, c_void_p]),
    "atlas_prefill_workspace_bytes": (c_size_t, [P(atlas_model), c_int32]),
    "atlas_prefill": (ctypes.c_int, [P(atlas_model), c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                     c_size_t, c_void_p]),
    "atlas_decode_batch_workspace_bytes": (c_size_t, [P(atlas_model), c_int32]),
    "atlas_decode_batch": (ctypes.c_int, [P(atlas_model), c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_size_t, c_void_p]),
    "atlas_sample_workspace_bytes": (c_size_t, [c_int32]),
    "atlas_sample": (ctypes.c_int, [c_void_p, c_int32, c_float, c_float, c_void_p, c_void_p, c_void_p, c_size_t,
                                    c_void_p]),
    "atlas_stream_read": (ctypes.c_int, [c_void_p, c_size_t, c_void_p, c_int32, c_void_p]),
    "atlas_profile_start": (ctypes.c_int, [c_int32]),
    "atlas_profile_stop": (ctypes.c_int, [P(atlas_profile_entry), c_int32, P(c_int32)]),
}

_lib = None


class AtlasError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: the HIP library must be built "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


def check(fn, rc):
    if rc != ATLAS_OK:
        raise AtlasError(fn, rc, lib().atlas_last_error().decode())
    return rc


def call(name, *args):
    """Call entry point ``name`` and raise AtlasError on a non-zero status."""
    return check(name, getattr(lib(), name)(*args))


def ptr(t):
    """Device address of a torch tensor (None -> NULL)."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream_ptr(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)
