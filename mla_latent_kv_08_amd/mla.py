"""Python binding of the C-ABI library ``libmla.so`` (same entry-point names).

Argument marshalling only: every step of the decode runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  The library
must be built (``python -m mla_latent_kv_08_amd.build`` or
``__graft_entry__.build()``); importing this module without it raises.
"""
import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MLA_LIB overrides the library path (the sanitizer test loads a host-only,
# ASan/UBSan build of the same sources through it)
LIB_PATH = os.environ.get("MLA_LIB") or os.path.join(_PKG, "libmla.so")

C_LATENT, R_ROPE, D_NOPE, D_V = 512, 64, 128, 128
KV_BF16, KV_FP8_E4M3_B128 = 0, 1
NOALLOC_SCRATCH_BYTES = 64 << 20  # MLA_NOALLOC_SCRATCH_BYTES
OPROJ_WO, OPROJ_WOV = 0, 1
DEFAULT_SOFTMAX_SCALE = 1.0 / math.sqrt(D_NOPE + R_ROPE)

STATUS = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED",
          3: "MLA_ERR_WORKSPACE", 4: "MLA_ERR_HIP"}


class MLAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


class Params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("seqlen_q", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32), ("kv_lora_rank", ctypes.c_int32),
        ("qk_nope_dim", ctypes.c_int32), ("qk_rope_dim", ctypes.c_int32),
        ("v_head_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("reserved", ctypes.c_int32),
        ("trace_events", ctypes.c_void_p),
    ]


def make_params(batch, num_heads, max_seq_len, kv_dtype=KV_BF16, topk=0, seqlen_q=1,
                softmax_scale=DEFAULT_SOFTMAX_SCALE, trace_events=None) -> Params:
    return Params(batch, seqlen_q, num_heads, max_seq_len, C_LATENT, D_NOPE, R_ROPE, D_V,
                  kv_dtype, topk, softmax_scale, 0, trace_events)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    vp, P = ctypes.c_void_p, ctypes.POINTER(Params)
    L.mla_cache_write.restype = ctypes.c_int
    L.mla_cache_write.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    L.mla_decode_workspace_size.restype = ctypes.c_int
    L.mla_decode_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    L.mla_decode.restype = ctypes.c_int
    L.mla_decode.argtypes = [P] + [vp] * 10 + [ctypes.c_size_t, vp]
    L.mla_decode_step.restype = ctypes.c_int
    L.mla_decode_step.argtypes = [P] + [vp] * 12 + [ctypes.c_size_t, vp]
    L.mla_decode_latent.restype = ctypes.c_int
    L.mla_decode_latent.argtypes = [P] + [vp] * 10 + [ctypes.c_size_t, vp]
    L.mla_output_projection.restype = ctypes.c_int
    L.mla_output_projection.argtypes = [P, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp]
    L.mla_decode_noalloc.restype = ctypes.c_int
    L.mla_decode_noalloc.argtypes = [P] + [vp] * 10
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_status_string.argtypes = [ctypes.c_int]
    L.mla_last_error.restype = ctypes.c_char_p
    L.mla_abi_version.restype = ctypes.c_int
    return L


lib = _load()


def _check(status: int):
    if status != 0:
        raise MLAError(status, lib.mla_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def decode_workspace_size(params: Params) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.mla_decode_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return n.value


def cache_write(kv_new, pe_new, start_pos, kv_cache, pe_cache, kv_scale=None, stream=None,
                trace_events=None):
    """mla_cache_write: rows start_pos[b] + i of the caches get kv_new/pe_new.

    kv_new [B,s,512] bf16, pe_new [B,s,64] bf16, start_pos int32 [B];
    kv_cache bf16 [>=B,T,512] or uint8 [>=B,T,512] with kv_scale fp32 [>=B,T,4];
    pe_cache bf16 [>=B,T,64].
    """
    _dev(kv_new, pe_new, start_pos, kv_cache, pe_cache, kv_scale)
    B, s = kv_new.shape[0], kv_new.shape[1]
    fp8 = kv_scale is not None
    p = make_params(B, 1, kv_cache.shape[1], KV_FP8_E4M3_B128 if fp8 else KV_BF16, seqlen_q=s,
                    trace_events=trace_events)
    _check(lib.mla_cache_write(ctypes.byref(p), _ptr(kv_new), _ptr(pe_new), _ptr(start_pos),
                               _ptr(kv_cache), _ptr(kv_scale), _ptr(pe_cache), _stream(stream)))


def decode(q_nope, q_pe, wkv_b, kv_cache, pe_cache, cache_lens, kv_scale=None, topk_idx=None,
           out=None, workspace=None, softmax_scale=DEFAULT_SOFTMAX_SCALE, stream=None,
           trace_events=None):
    """mla_decode: returns out [B,s,H,128] bf16 (allocated when not given).

    q_nope [B,s,H,128], q_pe [B,s,H,64], wkv_b [H,256,512] bf16; caches as for
    cache_write; cache_lens int32 [B]; topk_idx int32 [B,s,k] or None.  The s
    query tokens are the last s cached positions; token i sees rows
    t < cache_lens - (s - 1 - i).
    """
    _dev(q_nope, q_pe, wkv_b, kv_cache, pe_cache, cache_lens, kv_scale, topk_idx, out, workspace)
    B, s, H = q_nope.shape[0], q_nope.shape[1], q_nope.shape[2]
    fp8 = kv_scale is not None
    k = 0 if topk_idx is None else topk_idx.shape[-1]
    p = make_params(B, H, kv_cache.shape[1], KV_FP8_E4M3_B128 if fp8 else KV_BF16, topk=k,
                    seqlen_q=s, softmax_scale=softmax_scale, trace_events=trace_events)
    if out is None:
        out = torch.empty(B, s, H, D_V, dtype=torch.bfloat16, device=q_nope.device)
    if workspace is None:
        workspace = torch.empty(max(decode_workspace_size(p), 16), dtype=torch.uint8,
                                device=q_nope.device)
    _check(lib.mla_decode(ctypes.byref(p), _ptr(q_nope), _ptr(q_pe), _ptr(wkv_b), _ptr(kv_cache),
                          _ptr(kv_scale), _ptr(pe_cache), _ptr(cache_lens), _ptr(topk_idx),
                          _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def decode_step(kv_new, pe_new, q_nope, q_pe, wkv_b, kv_cache, pe_cache, cache_lens,
                kv_scale=None, topk_idx=None, out=None, workspace=None,
                softmax_scale=DEFAULT_SOFTMAX_SCALE, stream=None, trace_events=None):
    """mla_decode_step: store rows cache_lens[b] - s .. - 1, then decode; returns out.

    kv_new [B,s,512] and pe_new [B,s,64] bf16; every other argument as for
    decode (the caches are written).
    """
    _dev(kv_new, pe_new, q_nope, q_pe, wkv_b, kv_cache, pe_cache, cache_lens, kv_scale, topk_idx,
         out, workspace)
    B, s, H = q_nope.shape[0], q_nope.shape[1], q_nope.shape[2]
    if tuple(kv_new.shape[:2]) != (B, s) or tuple(pe_new.shape[:2]) != (B, s):
        raise ValueError("kv_new and pe_new need one row per query token")
    fp8 = kv_scale is not None
    k = 0 if topk_idx is None else topk_idx.shape[-1]
    p = make_params(B, H, kv_cache.shape[1], KV_FP8_E4M3_B128 if fp8 else KV_BF16, topk=k,
                    seqlen_q=s, softmax_scale=softmax_scale, trace_events=trace_events)
    if out is None:
        out = torch.empty(B, s, H, D_V, dtype=torch.bfloat16, device=q_nope.device)
    if workspace is None:
        workspace = torch.empty(max(decode_workspace_size(p), 16), dtype=torch.uint8,
                                device=q_nope.device)
    _check(lib.mla_decode_step(ctypes.byref(p), _ptr(kv_new), _ptr(pe_new), _ptr(q_nope),
                               _ptr(q_pe), _ptr(wkv_b), _ptr(kv_cache), _ptr(kv_scale),
                               _ptr(pe_cache), _ptr(cache_lens), _ptr(topk_idx), _ptr(out),
                               _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def decode_latent(q_nope, q_pe, wkv_b, kv_cache, pe_cache, cache_lens, kv_scale=None, topk_idx=None,
                  o_lat=None, workspace=None, softmax_scale=DEFAULT_SOFTMAX_SCALE, stream=None,
                  trace_events=None):
    """mla_decode_latent: returns the latent output o_lat [B,s,H,512] bf16 (the
    attention output before the value up-projection); arguments as for decode."""
    _dev(q_nope, q_pe, wkv_b, kv_cache, pe_cache, cache_lens, kv_scale, topk_idx, o_lat, workspace)
    B, s, H = q_nope.shape[0], q_nope.shape[1], q_nope.shape[2]
    fp8 = kv_scale is not None
    k = 0 if topk_idx is None else topk_idx.shape[-1]
    p = make_params(B, H, kv_cache.shape[1], KV_FP8_E4M3_B128 if fp8 else KV_BF16, topk=k,
                    seqlen_q=s, softmax_scale=softmax_scale, trace_events=trace_events)
    if o_lat is None:
        o_lat = torch.empty(B, s, H, C_LATENT, dtype=torch.bfloat16, device=q_nope.device)
    if workspace is None:
        workspace = torch.empty(max(decode_workspace_size(p), 16), dtype=torch.uint8,
                                device=q_nope.device)
    _check(lib.mla_decode_latent(ctypes.byref(p), _ptr(q_nope), _ptr(q_pe), _ptr(wkv_b), _ptr(kv_cache),
                                 _ptr(kv_scale), _ptr(pe_cache), _ptr(cache_lens), _ptr(topk_idx),
                                 _ptr(o_lat), _ptr(workspace), workspace.numel(), _stream(stream)))
    return o_lat


def output_projection(x, w, kind, y=None, stream=None, trace_events=None):
    """mla_output_projection: y [B,s,d_model] bf16 = x [B,s,H,F] . w[d_model, H*F]^T with
    (kind, F) = (OPROJ_WO, 128) for W_O after decode, or (OPROJ_WOV, 512) for the fused
    W_OV after decode_latent."""
    _dev(x, w, y)
    B, s, H, F = x.shape
    if F != (D_V if kind == OPROJ_WO else C_LATENT) or tuple(w.shape[1:]) != (H * F,):
        raise ValueError("x and w do not match the projection kind")
    d_model = w.shape[0]
    p = make_params(B, H, 1, seqlen_q=s, trace_events=trace_events)
    if y is None:
        y = torch.empty(B, s, d_model, dtype=torch.bfloat16, device=x.device)
    _check(lib.mla_output_projection(ctypes.byref(p), d_model, kind, _ptr(x), _ptr(w), _ptr(y),
                                     _stream(stream)))
    return y


def decode_noalloc(q_nope, q_pe, wkv_b, kv_cache, pe_cache, cache_lens, out, kv_scale=None,
                   topk_idx=None, softmax_scale=DEFAULT_SOFTMAX_SCALE, stream=None):
    """mla_decode_noalloc: mla_decode on the library's static device scratch
    (no workspace argument); `out` [B,s,H,128] bf16 must be given, since this
    path allocates nothing.  Calls that may overlap on one GPU race."""
    _dev(q_nope, q_pe, wkv_b, kv_cache, pe_cache, cache_lens, kv_scale, topk_idx, out)
    B, s, H = q_nope.shape[0], q_nope.shape[1], q_nope.shape[2]
    fp8 = kv_scale is not None
    k = 0 if topk_idx is None else topk_idx.shape[-1]
    p = make_params(B, H, kv_cache.shape[1], KV_FP8_E4M3_B128 if fp8 else KV_BF16, topk=k,
                    seqlen_q=s, softmax_scale=softmax_scale)
    _check(lib.mla_decode_noalloc(ctypes.byref(p), _ptr(q_nope), _ptr(q_pe), _ptr(wkv_b),
                                  _ptr(kv_cache), _ptr(kv_scale), _ptr(pe_cache), _ptr(cache_lens),
                                  _ptr(topk_idx), _ptr(out), _stream(stream)))
    return out
