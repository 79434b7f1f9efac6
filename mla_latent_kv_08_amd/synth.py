"""Seeded synthetic decode workloads (host tensors).

This module only draws inputs; it holds none of the decode arithmetic.  The
GPU path and the CPU oracle are both fed from it, so the two always see the
same bits.  Draws use a CPU ``torch.Generator`` in a fixed order per
workload: q_nope, q_pe, wkv_b, latent rows, rotary rows, then the
workload-specific structure (lengths, outlier mask, top-k indices).

Distributions (shapes and roles follow the DeepSeek-V3 decode layer: latent
512 wide, rotary key 64 wide, q_nope and v 128 wide per head):
  q_nope, q_pe, latent, rotary  ~ N(0, 1), rounded to bf16
  wkv_b                          ~ N(0, variance 1/512), rounded to bf16
With these variances the scaled logits have unit variance:
  var(absorbed q) = 128/512, content term 512 * 0.25, rotary term 64,
  total 192, times softmax_scale^2 = 1/192.
"""
from dataclasses import dataclass, field
import math
from typing import Optional

import torch

C_LATENT, R_ROPE, D_NOPE, D_V = 512, 64, 128, 128
SOFTMAX_SCALE = 1.0 / math.sqrt(D_NOPE + R_ROPE)


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    max_seq_len: int          # second dimension of the cache buffers
    fp8: bool = False         # latent stored as E4M3FN codes + per-128 scales
    ragged: Optional[tuple] = None   # (lo, hi): lengths uniform on {lo..hi}
    topk: int = 0             # >0: positions selected per sequence
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    seed: int = 0
    note: str = field(default="", compare=False)


# The five decode workloads (seed = position in this list).
WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_b1_h16_t256", 1, 16, 256, seed=0,
                 note="B=1, H=16, T=256, dense bf16 (one GPU's share of 128 heads on 8)"),
        Workload("dense_b1_h128_t4096", 1, 128, 4096, seed=1,
                 note="DeepSeek-V3-shaped decode, B=1, H=128, T=4096, dense bf16"),
        Workload("ragged_b32_h128_t16384", 32, 128, 16384, ragged=(1024, 16384), seed=2,
                 note="B=32, H=128, lengths U{1024..16384} in a 16384-row buffer, bf16"),
        Workload("fp8_b16_h128_t32768", 16, 128, 32768, fp8=True, outlier_frac=0.01,
                 outlier_mult=20.0, seed=3,
                 note="B=16, H=128, T=32768, E4M3FN latent with per-128 fp32 scales, "
                      "1% of latent entries x20"),
        Workload("topk2048_b8_h128_t65536", 8, 128, 65536, topk=2048, seed=4,
                 note="B=8, H=128, T=65536 bf16 cache, 2048 distinct sorted positions per "
                      "sequence"),
    ]
}
ORDER = list(WORKLOADS)


def scaled(w: Workload, **over) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    d = {k: getattr(w, k) for k in w.__dataclass_fields__}
    d.update(over)
    return Workload(**d)


def make_inputs(w: Workload, seed: Optional[int] = None, poison_tail: bool = False) -> dict:
    """Draws one decode batch for workload ``w`` on the host.

    Returns a dict of CPU tensors:
      q_nope [B,1,H,128] bf16, q_pe [B,1,H,64] bf16, wkv_b [H,256,512] bf16,
      kv [B,T,512] bf16 (pre-quantisation latent rows), pe [B,T,64] bf16,
      cache_lens int32 [B], topk_idx int32 [B,1,k] or None.
    Rows at or beyond a sequence's length are zero (NaN when ``poison_tail``).
    """
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)
    B, H, T = w.batch, w.heads, w.max_seq_len
    bf = torch.bfloat16
    q_nope = torch.randn(B, 1, H, D_NOPE, generator=g).to(bf)
    q_pe = torch.randn(B, 1, H, R_ROPE, generator=g).to(bf)
    wkv_b = (torch.randn(H, D_NOPE + D_V, C_LATENT, generator=g) / math.sqrt(C_LATENT)).to(bf)
    kv = torch.randn(B, T, C_LATENT, generator=g)
    pe = torch.randn(B, T, R_ROPE, generator=g)
    if w.ragged is not None:
        lo, hi = w.ragged
        lens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    else:
        lens = torch.full((B,), T, dtype=torch.int32)
    if w.outlier_frac > 0:
        mask = torch.rand(B, T, C_LATENT, generator=g) < w.outlier_frac
        kv = torch.where(mask, kv * w.outlier_mult, kv)
    topk_idx = None
    if w.topk > 0:
        rows = []
        for b in range(B):
            n = int(lens[b])
            perm = torch.randperm(n, generator=g)[: w.topk]
            rows.append(torch.sort(perm).values.to(torch.int32))
        topk_idx = torch.stack(rows).reshape(B, 1, w.topk)
    kv = kv.to(bf)
    pe = pe.to(bf)
    if w.ragged is not None:
        fill = float("nan") if poison_tail else 0.0
        pos = torch.arange(T).reshape(1, T)
        tail = pos >= lens.reshape(B, 1).to(torch.int64)
        kv[tail] = fill
        pe[tail] = fill
    return dict(q_nope=q_nope, q_pe=q_pe, wkv_b=wkv_b, kv=kv, pe=pe, cache_lens=lens,
                topk_idx=topk_idx)


def add_query_tokens(x: dict, s: int, seed: int) -> dict:
    """Inputs with s query tokens per sequence: the workload's token first,
    then s - 1 more seeded draws of the same distributions (q ~ N(0, 1)); a
    top-k index row is repeated for every token."""
    g = torch.Generator().manual_seed(seed)
    B, _, H, _ = x["q_nope"].shape
    y = dict(x)
    y["q_nope"] = torch.cat([x["q_nope"], torch.randn(B, s - 1, H, 128, generator=g).to(torch.bfloat16)], 1)
    y["q_pe"] = torch.cat([x["q_pe"], torch.randn(B, s - 1, H, 64, generator=g).to(torch.bfloat16)], 1)
    if x["topk_idx"] is not None:
        y["topk_idx"] = x["topk_idx"].expand(B, s, x["topk_idx"].shape[-1]).contiguous()
    return y


D_MODEL = 7168  # DeepSeek-V3 hidden size: the output projection's width


def make_w_o(heads: int, d_model: int = D_MODEL, seed: int = 0) -> torch.Tensor:
    """Seeded synthetic output projection W_O, bf16 [d_model][heads * 128]
    (a linear layer's weight: [out features][in features]), N(0, variance
    1/(heads * 128)) so that unit-variance head outputs give unit-variance
    layer outputs."""
    g = torch.Generator().manual_seed(seed)
    k = heads * D_V
    return (torch.randn(d_model, k, generator=g) / math.sqrt(k)).to(torch.bfloat16)
