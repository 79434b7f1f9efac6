"""ctypes wrapper of the plain C oracle (``mla_oracle.c``).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg import this module.  Inputs are host arrays: numpy arrays or
CPU torch tensors (bf16 tensors are passed as their raw 16-bit patterns).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

C_LATENT, R_ROPE, D_NOPE, D_V, BLOCK = 512, 64, 128, 128, 128


class _DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("max_seq_len", ctypes.c_int),
        ("s", ctypes.c_int), ("fp8", ctypes.c_int), ("topk", ctypes.c_int), ("softmax_scale", ctypes.c_double),
        ("q_nope", ctypes.c_void_p), ("q_pe", ctypes.c_void_p), ("wkv_b", ctypes.c_void_p),
        ("kv_cache", ctypes.c_void_p), ("kv_scale", ctypes.c_void_p),
        ("pe_cache", ctypes.c_void_p), ("cache_lens", ctypes.c_void_p),
        ("topk_idx", ctypes.c_void_p),
    ]


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB") or _build.LIB  # ORACLE_LIB: e.g. a sanitizer build
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.oracle_bf16_value.restype = ctypes.c_double
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_round.restype = ctypes.c_uint16
        L.oracle_bf16_round.argtypes = [ctypes.c_float]
        L.oracle_e4m3fn_value.restype = ctypes.c_double
        L.oracle_e4m3fn_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3fn_encode.restype = ctypes.c_uint8
        L.oracle_e4m3fn_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3fn_encode_array.restype = None
        L.oracle_e4m3fn_encode_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]
        L.oracle_values_per_position.restype = ctypes.c_int
        L.oracle_latent_bytes.restype = ctypes.c_double
        L.oracle_latent_bytes.argtypes = [ctypes.c_double, ctypes.c_int]
        L.oracle_cache_write.restype = ctypes.c_int
        L.oracle_cache_write.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 6
        L.oracle_decode.restype = ctypes.c_int
        L.oracle_decode.argtypes = [ctypes.POINTER(_DecodeArgs), ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_decode_latent.restype = ctypes.c_int
        L.oracle_decode_latent.argtypes = [ctypes.POINTER(_DecodeArgs), ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p]
        L.oracle_output_projection.restype = ctypes.c_int
        L.oracle_output_projection.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 3
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _np(x, dtype):
    """Host array with the given raw dtype (bf16 torch tensors -> uint16 bits)."""
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16)
            x = x.numpy()
    except ImportError:
        pass
    a = np.ascontiguousarray(x)
    if a.dtype != dtype:
        a = a.view(dtype) if a.dtype.itemsize == np.dtype(dtype).itemsize else a.astype(dtype)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def bf16_value(bits: int) -> float:
    return lib().oracle_bf16_value(bits)


def bf16_round(x: float) -> int:
    return lib().oracle_bf16_round(x)


def e4m3fn_value(code: int) -> float:
    return lib().oracle_e4m3fn_value(code)


def e4m3fn_encode(v: float) -> int:
    return lib().oracle_e4m3fn_encode(v)


def e4m3fn_encode_array(values) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float32))
    out = np.zeros(v.shape, np.uint8)
    lib().oracle_e4m3fn_encode_array(_ptr(v), _ptr(out), v.size)
    return out


def values_per_position() -> int:
    return lib().oracle_values_per_position()


def latent_bytes(seq_len: float, bytes_per_elem: int) -> float:
    return lib().oracle_latent_bytes(seq_len, bytes_per_elem)


def num_threads() -> int:
    return lib().oracle_num_threads()


def cache_write(kv_new, pe_new, start_pos, max_seq_len, fp8, kv_cache=None, kv_scale=None,
                pe_cache=None):
    """Writes new rows into (host) caches; returns (kv_cache, kv_scale, pe_cache).

    kv_new [B][s][512] bf16, pe_new [B][s][64] bf16, start_pos int32 [B].
    Caches are allocated (zeros) when not given.
    """
    kv_new = _np(kv_new, np.uint16)
    pe_new = _np(pe_new, np.uint16)
    start_pos = _np(start_pos, np.int32)
    B, s = kv_new.shape[0], kv_new.shape[1]
    if kv_cache is None:
        kv_cache = np.zeros((B, max_seq_len, C_LATENT), np.uint8 if fp8 else np.uint16)
    if fp8 and kv_scale is None:
        kv_scale = np.zeros((B, max_seq_len, C_LATENT // BLOCK), np.float32)
    if pe_cache is None:
        pe_cache = np.zeros((B, max_seq_len, R_ROPE), np.uint16)
    rc = lib().oracle_cache_write(B, s, max_seq_len, int(fp8), _ptr(kv_new), _ptr(pe_new),
                                  _ptr(start_pos), _ptr(kv_cache), _ptr(kv_scale),
                                  _ptr(pe_cache))
    if rc != 0:
        raise ValueError("oracle_cache_write rejected its arguments")
    return kv_cache, kv_scale, pe_cache


def _decode_args(q_nope, q_pe, wkv_b, kv_cache, pe_cache, cache_lens, softmax_scale, kv_scale,
                 topk_idx):
    qn = _np(q_nope, np.uint16)
    qp = _np(q_pe, np.uint16)
    w = _np(wkv_b, np.uint16)
    fp8 = kv_scale is not None
    kv = _np(kv_cache, np.uint8 if fp8 else np.uint16)
    sc = _np(kv_scale, np.float32) if fp8 else None
    pe = _np(pe_cache, np.uint16)
    lens = _np(cache_lens, np.int32)
    B, T = kv.shape[0], kv.shape[1]
    H = w.shape[0]
    s = qn.size // (B * H * D_NOPE) if B > 0 else 1
    assert qn.size == B * s * H * D_NOPE and qp.size == B * s * H * R_ROPE
    assert w.shape == (H, D_NOPE + D_V, C_LATENT)
    assert kv.shape == (B, T, C_LATENT) and pe.shape == (B, T, R_ROPE) and lens.shape == (B,)
    k = 0
    ti = None
    if topk_idx is not None:
        ti = _np(topk_idx, np.int32)
        k = ti.shape[-1]
        assert ti.size == B * s * k
    args = _DecodeArgs(B, H, T, s, int(fp8), k, float(softmax_scale), _ptr(qn), _ptr(qp), _ptr(w),
                       _ptr(kv), _ptr(sc), _ptr(pe), _ptr(lens), _ptr(ti))
    keep = (qn, qp, w, kv, sc, pe, lens, ti)  # the arrays the pointers refer to
    return args, keep, (B, s, H, T)


def _pairs(pairs, n_all):
    if pairs is None:
        return None, n_all
    pr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    return pr, pr.shape[0]


def decode(q_nope, q_pe, wkv_b, kv_cache, pe_cache, cache_lens, softmax_scale, kv_scale=None,
           topk_idx=None, pairs=None, want_probs=False):
    """Oracle decode; returns out (float64) [B][H][128] for one query token,
    [B][s][H][128] for s > 1, or [n_pairs][128] (+ probs).

    q_nope [B][s][H][128], q_pe [B][s][H][64], wkv_b [H][256][512] (bf16);
    kv_cache bf16 [B][T][512] or uint8 E4M3FN codes (then kv_scale fp32 [B][T][4]);
    pe_cache bf16 [B][T][64]; cache_lens int32 [B]; topk_idx int32 [B][s][k] or None;
    pairs: optional int array [n][2] of (q, h) to evaluate, q = b * s + i.
    The s query tokens are the last s cached positions; token i sees rows
    t < end_b - (s - 1 - i).
    """
    args, keep, (B, s, H, T) = _decode_args(q_nope, q_pe, wkv_b, kv_cache, pe_cache, cache_lens,
                                            softmax_scale, kv_scale, topk_idx)
    pr, n = _pairs(pairs, B * s * H)
    out = np.zeros((n, D_V), np.float64)
    probs = np.zeros((n, T), np.float64) if want_probs else None
    rc = lib().oracle_decode(ctypes.byref(args), n, _ptr(pr), _ptr(out), _ptr(probs))
    del keep
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    if pairs is None:
        out = out.reshape((B, H, D_V) if s == 1 else (B, s, H, D_V))
        if want_probs:
            probs = probs.reshape((B, H, T) if s == 1 else (B, s, H, T))
    return (out, probs) if want_probs else out


def decode_latent(q_nope, q_pe, wkv_b, kv_cache, pe_cache, cache_lens, softmax_scale, kv_scale=None,
                  topk_idx=None, pairs=None):
    """The latent output of the decode before the value up-projection,
    o[c] = sum_t p[t] c_KV[t, c] (float64): [B][s][H][512], or [n_pairs][512]."""
    args, keep, (B, s, H, T) = _decode_args(q_nope, q_pe, wkv_b, kv_cache, pe_cache, cache_lens,
                                            softmax_scale, kv_scale, topk_idx)
    pr, n = _pairs(pairs, B * s * H)
    olat = np.zeros((n, C_LATENT), np.float64)
    rc = lib().oracle_decode_latent(ctypes.byref(args), n, _ptr(pr), _ptr(olat))
    del keep
    if rc != 0:
        raise ValueError("oracle_decode_latent rejected its arguments")
    return olat.reshape(B, s, H, C_LATENT) if pairs is None else olat


def output_projection(x, w):
    """y[m][n] = sum_k x[m][k] w[n][k] in float64.  x: [..., K] (float64, or a
    bf16 tensor), w: [N, K] (bf16 tensor or float array); returns [..., N]."""
    def f64(a):
        try:
            import torch
            if isinstance(a, torch.Tensor):
                return a.detach().cpu().to(torch.float64).numpy()
        except ImportError:
            pass
        return np.asarray(a, dtype=np.float64)
    xa = np.ascontiguousarray(f64(x))
    wa = np.ascontiguousarray(f64(w))
    K = xa.shape[-1]
    N = wa.shape[0]
    assert wa.shape == (N, K)
    M = xa.size // K
    y = np.zeros(xa.shape[:-1] + (N,), np.float64)
    if lib().oracle_output_projection(M, K, N, _ptr(xa), _ptr(wa), _ptr(y)) != 0:
        raise ValueError("oracle_output_projection rejected its arguments")
    return y
