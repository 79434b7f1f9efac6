"""Host-side checks of the C-ABI library (no GPU needed).

The library loads, exports every entry point include/mla.h declares, and
rejects bad arguments before any HIP call (so these run on a machine without
a GPU).  No call here reaches a kernel launch.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


@pytest.fixture(scope="module")
def m():
    import torch  # noqa: F401  (load torch's HIP runtime first, as every user does)
    from mla_latent_kv_08_amd import mla
    return mla


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(m):
    names = declared_functions()
    assert {"mla_cache_write", "mla_decode", "mla_decode_step", "mla_decode_workspace_size",
            "mla_decode_latent", "mla_output_projection", "mla_decode_noalloc",
            "mla_status_string", "mla_last_error", "mla_abi_version"} <= set(names)
    for n in names:
        assert hasattr(m.lib, n), n
    assert m.lib.mla_abi_version() == 2


def test_params_struct_matches_header(m):
    # mla_params: 12 x int32/float then one pointer
    assert ctypes.sizeof(m.Params) == 12 * 4 + 8
    assert m.Params.trace_events.offset == 48


def test_status_strings(m):
    for s in range(5):
        assert m.lib.mla_status_string(s).decode().startswith(m.STATUS[s])
    assert b"unknown" in m.lib.mla_status_string(99)


FAKE = ctypes.c_void_p(0x100000)  # 16-byte aligned, never dereferenced: calls fail first


def _decode(m, p, **kw):
    a = dict(q_nope=FAKE, q_pe=FAKE, wkv_b=FAKE, kv=FAKE, scale=None, pe=FAKE, lens=FAKE,
             topk=None, out=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return m.lib.mla_decode(ctypes.byref(p), a["q_nope"], a["q_pe"], a["wkv_b"], a["kv"],
                            a["scale"], a["pe"], a["lens"], a["topk"], a["out"], a["ws"],
                            a["ws_bytes"], None)


def test_decode_rejects_bad_arguments(m):
    P = m.make_params
    assert m.lib.mla_decode(None, *([None] * 10), 0, None) == 1
    assert _decode(m, P(1, 128, 4096, seqlen_q=0)) == 1                 # no query token
    assert _decode(m, P(40000, 16, 100, seqlen_q=2)) == 2               # > 65535 query tokens
    assert _decode(m, P(1, 0, 4096)) == 1                               # no heads
    assert _decode(m, P(1, 129, 4096)) == 1                             # too many heads
    assert _decode(m, P(1, 16, 0)) == 1                                 # empty cache buffer
    assert _decode(m, P(1, 16, 100, topk=101), topk=FAKE) == 1          # topk > T
    assert _decode(m, P(1, 16, 100, topk=4)) == 1                       # topk without indices
    assert _decode(m, P(1, 16, 100), topk=FAKE) == 1                    # indices without topk
    assert _decode(m, P(1, 16, 100, kv_dtype=7)) == 1                   # unknown kv dtype
    assert _decode(m, P(1, 16, 100, kv_dtype=1)) == 1                   # fp8 without scales
    assert _decode(m, P(1, 16, 100), scale=FAKE) == 1                   # scales with bf16
    assert _decode(m, P(1, 16, 100, softmax_scale=0.0)) == 1
    assert _decode(m, P(1, 16, 100, softmax_scale=float("inf"))) == 1
    assert _decode(m, P(1, 16, 100), q_pe=None) == 1                    # null tensor
    assert _decode(m, P(1, 16, 100), out=ctypes.c_void_p(0x100002)) == 1  # misaligned
    assert _decode(m, P(1, 16, 100), ws=None) == 3                      # no workspace
    assert _decode(m, P(1, 16, 100), ws_bytes=16) == 3                  # workspace too small
    p = P(1, 16, 100)
    p.kv_lora_rank = 256
    assert _decode(m, p) == 2                                           # other widths
    assert _decode(m, P(0, 16, 100)) == 0                               # empty batch: no-op
    assert "workspace" in m.lib.mla_last_error().decode() or True


def test_last_error_detail(m):
    _decode(m, m.make_params(1, 16, 100), ws_bytes=16)
    assert "workspace needs" in m.lib.mla_last_error().decode()
    assert _decode(m, m.make_params(0, 16, 100)) == 0
    assert m.lib.mla_last_error().decode() == ""


def test_cache_write_rejects_bad_arguments(m):
    P = m.make_params

    def cw(p, kv_new=FAKE, pe_new=FAKE, sp=FAKE, kv=FAKE, sc=None, pe=FAKE):
        return m.lib.mla_cache_write(ctypes.byref(p), kv_new, pe_new, sp, kv, sc, pe, None)

    assert cw(P(2, 1, 64, seqlen_q=-1)) == 1
    assert cw(P(2, 1, 64, seqlen_q=1), kv_new=None) == 1
    assert cw(P(2, 1, 64, seqlen_q=1, kv_dtype=1)) == 1           # fp8 without scales
    assert cw(P(2, 1, 64, seqlen_q=1), sc=FAKE) == 1              # scales with bf16
    assert cw(P(2, 1, 64, seqlen_q=1), kv=ctypes.c_void_p(0x100008)) == 1
    assert cw(P(2, 1, 64, seqlen_q=0)) == 0                       # nothing to write
    assert cw(P(0, 1, 64, seqlen_q=3)) == 0


def test_workspace_size_is_host_only_and_monotone(m):
    sizes = []
    for T in (256, 4096, 16384, 65536):
        p = m.make_params(8, 128, T)
        sizes.append(m.decode_workspace_size(p))
    assert all(s > 0 for s in sizes) and sizes == sorted(sizes)
    # partials: one per attention workgroup, at most max(256, B) of them for a
    # dense selection whatever the buffer length; a top-k selection of more
    # than 32 tiles per workgroup needs more workgroups
    assert m.decode_workspace_size(m.make_params(512, 128, 4096)) > sizes[1]
    small_k = m.decode_workspace_size(m.make_params(8, 128, 65536, topk=2048))
    assert m.decode_workspace_size(m.make_params(8, 128, 65536, topk=65536)) > small_k
    # s query tokens per sequence plan like batch x s sequences
    assert m.decode_workspace_size(m.make_params(8, 128, 4096, seqlen_q=4)) == \
        m.decode_workspace_size(m.make_params(32, 128, 4096))
    with pytest.raises(m.MLAError):
        m.decode_workspace_size(m.make_params(8, 200, 4096))
    with pytest.raises(m.MLAError):
        m.decode_workspace_size(m.make_params(8, 128, 4096, seqlen_q=0))


def test_workspace_size_applies_the_decode_limits(m):
    # the same query-token limit as mla_decode, checked before any plan is
    # formed: batch x seqlen_q beyond 2^31 must not wrap to a small size
    for batch, s in ((40000, 2), (65536, 1), (1 << 20, 1 << 12), (0x7FFFFFFF, 2)):
        n = ctypes.c_size_t(12345)
        st = m.lib.mla_decode_workspace_size(ctypes.byref(m.make_params(batch, 16, 100, seqlen_q=s)),
                                             ctypes.byref(n))
        assert st == 2 and n.value == 12345, (batch, s, st)
        assert "65535" in m.lib.mla_last_error().decode()
    assert m.decode_workspace_size(m.make_params(65535, 16, 100)) > 0
    with pytest.raises(m.MLAError):
        m.decode_workspace_size(m.make_params(1, 16, 100, topk=101))


def test_decode_step_rejects_bad_arguments(m):
    P = m.make_params

    def step(p, kv_new=FAKE, pe_new=FAKE, ws_bytes=1 << 40, **kw):
        a = dict(q_nope=FAKE, q_pe=FAKE, wkv_b=FAKE, kv=FAKE, scale=None, pe=FAKE, lens=FAKE,
                 topk=None, out=FAKE, ws=FAKE)
        a.update(kw)
        return m.lib.mla_decode_step(ctypes.byref(p), kv_new, pe_new, a["q_nope"], a["q_pe"],
                                     a["wkv_b"], a["kv"], a["scale"], a["pe"], a["lens"],
                                     a["topk"], a["out"], a["ws"], ws_bytes, None)

    assert step(P(1, 16, 100), kv_new=None) == 1
    assert step(P(1, 16, 100), pe_new=ctypes.c_void_p(0x100004)) == 1      # misaligned
    assert step(P(1, 16, 100, kv_dtype=1)) == 1                             # fp8 without scales
    assert step(P(1, 16, 100, seqlen_q=0)) == 1
    assert step(P(1, 16, 100), ws_bytes=16) == 3
    assert step(P(0, 16, 100), kv_new=None) == 0                            # empty batch: no-op


def test_decode_noalloc_rejects_before_any_hip_call(m):
    P = m.make_params

    def na(p, **kw):
        a = dict(q_nope=FAKE, q_pe=FAKE, wkv_b=FAKE, kv=FAKE, scale=None, pe=FAKE, lens=FAKE,
                 topk=None, out=FAKE)
        a.update(kw)
        return m.lib.mla_decode_noalloc(ctypes.byref(p), a["q_nope"], a["q_pe"], a["wkv_b"], a["kv"],
                                        a["scale"], a["pe"], a["lens"], a["topk"], a["out"], None)

    # a call whose workspace exceeds the static scratch: MLA_ERR_WORKSPACE, nothing enqueued
    big = P(2000, 128, 4096)
    assert m.decode_workspace_size(big) > m.NOALLOC_SCRATCH_BYTES
    assert na(big) == 3
    assert "static scratch holds %d" % m.NOALLOC_SCRATCH_BYTES in m.lib.mla_last_error().decode()
    # the benchmark's workloads fit it
    for B, T, k, s in ((32, 16384, 0, 1), (16, 32768, 0, 1), (8, 65536, 2048, 1), (1, 4096, 0, 1),
                       (32, 16384, 0, 2)):
        assert m.decode_workspace_size(P(B, 128, T, topk=k, seqlen_q=s)) <= m.NOALLOC_SCRATCH_BYTES
    # the same argument checks as mla_decode
    assert na(P(1, 16, 100), q_pe=None) == 1
    assert na(P(1, 16, 100, kv_dtype=1)) == 1
    assert na(P(1, 129, 100)) == 1
    assert na(P(40000, 16, 100, seqlen_q=2)) == 2
    assert na(P(0, 16, 100)) == 0
