"""Error study of an FP8 latent reduction for the FP8 cache (CPU only).

An FP8 matrix-core product for the latent reduction of an E4M3FN cache would
take both operands in FP8: the codes as they are stored, and the
probabilities with each row's block scale folded in, P'_w[h][t] =
p[h][t] * scale[t][w] for the 128-column block w of the latent, rounded to
E4M3FN (with a power-of-two factor per head and block that puts the largest
value near 448).  The cache-write excerpt of "DeepSeek-V3.2-Exp . KV cache"
fixes the cache (E4M3FN codes, scale = blockmax / 448); it says nothing on
the probabilities, which this path keeps in bf16.

The same holds for the score contraction in FP8: the codes times the absorbed
query rounded to E4M3FN (one scale per head, its maximum mapped to 448), the
128-column blocks summed separately and each multiplied by its row's scale.

This test measures these choices on sequences drawn like the FP8 workload
(N(0, 1) latent with 1 % of entries x20, bf16 queries and weights), against
the fp64 result over the same dequantised latent, and records why the path
keeps bf16 probabilities: their error is about 5e-4 relative L2, while E4M3
probabilities alone cost about 2.8e-2, above the 1e-2 bar the GPU path is
held to and close to the 3e-2 stated for an FP8 cache; an E4M3 query in the
score contraction costs about 9e-2 by itself (the outliers multiply the
query's rounding errors into the logits), far above either bar.
"""
import math

import numpy as np
import torch

import oracle
from mla_latent_kv_08_amd import synth


def _fp8(a):
    return torch.from_numpy(np.clip(a, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()


def _bf16(a):
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).double().numpy()


def test_fp8_probabilities_cost_versus_bf16():
    B, H, T = 2, 32, 8192
    w = synth.Workload("fp8pv", B, H, T, fp8=True, outlier_frac=0.01, outlier_mult=20.0, seed=3)
    x = synth.make_inputs(w)
    codes, scales, _ = oracle.cache_write(x["kv"], x["pe"], torch.zeros(B, dtype=torch.int32), T, True)
    cv = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    sc = scales.astype(np.float64)
    # the cache's latent as the page decodes it: bf16(code * scale)
    deq = _bf16((cv.reshape(B, T, 4, 128) * sc[..., None]).reshape(B, T, 512))
    wkv = x["wkv_b"].double().numpy()
    qn, qp, pe = x["q_nope"].double().numpy()[:, 0], x["q_pe"].double().numpy()[:, 0], x["pe"].double().numpy()
    err = {"bf16": [0.0, 0.0], "fp8": [0.0, 0.0], "fp8_scores": [0.0, 0.0], "fp8_both": [0.0, 0.0]}
    for b in range(B):
        qa = np.einsum("hd,hdc->hc", qn[b], wkv[:, :128, :])
        s = (qa @ deq[b].T + qp[b] @ pe[b].T) / math.sqrt(192.0)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        l = p.sum(axis=1, keepdims=True)
        ref = np.einsum("hc,hdc->hd", (p @ deq[b]) / l, wkv[:, 128:, :])
        pb = _bf16(p)
        o_bf = (pb @ deq[b]) / l
        o_f8 = np.zeros_like(o_bf)
        for blk in range(4):
            pp = pb * sc[b, :, blk][None, :]
            e = np.floor(np.log2(448.0 / np.maximum(pp.max(axis=1, keepdims=True), 1e-300)))
            o_f8[:, 128 * blk:128 * blk + 128] = (_fp8(pp * 2.0 ** e) / 2.0 ** e) @ cv[b][:, 128 * blk:128 * blk + 128] / l
        # scores with the absorbed query in E4M3 (per-head scale), block partial sums times the row scales
        qs = np.abs(qa).max(axis=1, keepdims=True) / 448.0
        q8 = _fp8(qa / qs) * qs
        s8 = sum((q8[:, 128 * blk:128 * blk + 128] @ cv[b][:, 128 * blk:128 * blk + 128].T) * sc[b, :, blk][None, :]
                 for blk in range(4))
        s8 = (s8 + qp[b] @ pe[b].T) / math.sqrt(192.0)
        p8 = np.exp(s8 - s8.max(axis=1, keepdims=True))
        l8 = p8.sum(axis=1, keepdims=True)
        o_s8 = (_bf16(p8) @ deq[b]) / l8
        o_both = np.zeros_like(o_bf)
        for blk in range(4):
            pp = _bf16(p8) * sc[b, :, blk][None, :]
            e = np.floor(np.log2(448.0 / np.maximum(pp.max(axis=1, keepdims=True), 1e-300)))
            o_both[:, 128 * blk:128 * blk + 128] = (_fp8(pp * 2.0 ** e) / 2.0 ** e) @ cv[b][:, 128 * blk:128 * blk + 128] / l8
        for name, o in (("bf16", o_bf), ("fp8", o_f8), ("fp8_scores", o_s8), ("fp8_both", o_both)):
            out = np.einsum("hc,hdc->hd", o, wkv[:, 128:, :])
            err[name][0] += float(np.sum((out - ref) ** 2))
            err[name][1] += float(np.sum(ref ** 2))
    rel = {k: math.sqrt(v[0] / v[1]) for k, v in err.items()}
    print(f"relative L2 of the output: bf16 probabilities {rel['bf16']:.3e}, E4M3 probabilities {rel['fp8']:.3e}, "
          f"E4M3 query in the scores {rel['fp8_scores']:.3e}, both {rel['fp8_both']:.3e}")
    assert rel["bf16"] < 1e-3
    assert 1e-2 < rel["fp8"] < 3e-2
    assert rel["fp8_scores"] > 3e-2
    assert rel["fp8_both"] > 3e-2
