"""GPU test of mla_decode_noalloc, the entry point that allocates nothing.

Through the C ABI, its output must equal mla_decode's bit for bit (the same
kernels on the library's static scratch instead of a caller workspace), and
meet the oracle's bar, on two calls in a row, the second smaller than the
first (the scratch keeps the first call's contents, which the second must
not depend on).
"""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_08_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(m, w, label, s=1):
    x = synth.make_inputs(w)
    if s > 1:
        x = synth.add_query_tokens(x, s, seed=w.seed + 1000)
    print(f"[noalloc {label}] B={w.batch} s={s} H={w.heads} T={w.max_seq_len} fp8={w.fp8} topk={w.topk}",
          flush=True)
    d = {k: (None if v is None else v.to(DEV).contiguous()) for k, v in x.items()}
    kv, sc, pe = d["kv"], None, d["pe"]
    if w.fp8:
        B, T = w.batch, w.max_seq_len
        kv = torch.zeros(B, T, 512, dtype=torch.uint8, device=DEV)
        sc = torch.zeros(B, T, 4, dtype=torch.float32, device=DEV)
        pe = torch.zeros(B, T, 64, dtype=torch.bfloat16, device=DEV)
        m.cache_write(d["kv"], d["pe"], torch.zeros(B, dtype=torch.int32, device=DEV), kv, pe,
                      kv_scale=sc)
    args = (d["q_nope"], d["q_pe"], d["wkv_b"], kv, pe, d["cache_lens"])
    ref = m.decode(*args, kv_scale=sc, topk_idx=d["topk_idx"])
    out = torch.full_like(ref, float("nan"))
    m.decode_noalloc(*args, out, kv_scale=sc, topk_idx=d["topk_idx"])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), label
    if w.fp8:
        codes, scales, ope = oracle.cache_write(x["kv"], x["pe"], torch.zeros(w.batch, dtype=torch.int32),
                                                w.max_seq_len, True)
    else:
        codes, scales, ope = x["kv"], None, x["pe"]
    o = oracle.decode(x["q_nope"], x["q_pe"], x["wkv_b"], codes, ope, x["cache_lens"],
                      synth.SOFTMAX_SCALE, kv_scale=scales, topk_idx=x["topk_idx"])
    g = out.float().cpu().double().numpy().reshape(o.shape)
    rel = float(np.linalg.norm(g - o) / np.linalg.norm(o))
    mx = float(np.abs(g - o).max())
    print(f"[noalloc {label}] relL2={rel:.3e} max|err|={mx:.3e}", flush=True)
    assert rel <= 1e-2 and mx <= 5e-2 * max(1.0, float(np.abs(o).max())), (label, rel, mx)


def test_noalloc_matches_decode_two_calls_second_smaller():
    from mla_latent_kv_08_amd import mla as m
    first = synth.Workload("na1", 6, 128, 3000, ragged=(1, 3000), seed=91)
    second = synth.Workload("na2", 2, 64, 700, ragged=(1, 700), seed=92)
    _case(m, first, "first")
    _case(m, second, "second, smaller")


def test_noalloc_fp8_topk_then_smaller_dense():
    from mla_latent_kv_08_amd import mla as m
    _case(m, synth.Workload("na3", 4, 128, 2500, fp8=True, topk=600, outlier_frac=0.01,
                            outlier_mult=20.0, seed=93), "fp8 top-k")
    _case(m, synth.Workload("na4", 1, 16, 256, seed=94), "tiny dense")


def test_noalloc_packed_tokens_then_smaller():
    """Several query tokens per sequence at few heads (the tokens share one
    work item: s H packed query rows), then a smaller call of the same kind."""
    from mla_latent_kv_08_amd import mla as m
    _case(m, synth.Workload("na5", 5, 16, 900, ragged=(4, 900), seed=95), "packed H=16 s=4", s=4)
    _case(m, synth.Workload("na6", 2, 32, 300, ragged=(3, 300), seed=96), "packed H=32 s=3, smaller", s=3)


def test_noalloc_in_a_captured_graph():
    """The use it is for: recorded into a HIP graph (after one eager call, which
    looks up the scratch address), replayed several times with eager work in
    between, every replay bit for bit equal to mla_decode's output."""
    from mla_latent_kv_08_amd import mla as m
    w = synth.Workload("na5", 3, 128, 1500, ragged=(1, 1500), seed=95)
    x = synth.make_inputs(w)
    print(f"[noalloc graph] B={w.batch} H={w.heads} T={w.max_seq_len}", flush=True)
    d = {k: (None if v is None else v.to(DEV).contiguous()) for k, v in x.items()}
    args = (d["q_nope"], d["q_pe"], d["wkv_b"], d["kv"], d["pe"], d["cache_lens"])
    ref = m.decode(*args)
    out = torch.zeros_like(ref)
    m.decode_noalloc(*args, out)  # eager first call on this device
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            m.decode_noalloc(*args, out, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        m.decode(*args)  # eager work between replays (its own workspace)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep
