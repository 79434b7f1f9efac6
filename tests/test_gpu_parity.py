"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (float outputs are compared in float64 against the oracle's fp64 result):
  bf16 latent cache:  relative L2 <= 1e-2 and max |err| <= 5e-2
  FP8 latent cache:   relative L2 <= 1e-2 and max |err| <= 5e-2 * max(1, max|ref|).
                      Both sides read the same dequantised values
                      bf16(code * scale), so the FP8 cache gets the bf16 bar; only
                      the absolute bound follows the outputs' magnitude (with 1 %
                      of latent entries x20 they reach |out| ~ 5).  The looser
                      3e-2 relative bound stated for an FP8 cache would not see a
                      several-fold regression of this path.
  FP8 codes and scales written by mla_cache_write: bit-exact.
Small cases span several 32-row tiles with ragged tails and are compared in
full; the five decode workloads at full size run in the launch configuration
the benchmark uses and are compared on sampled (sequence, head) rows.
"""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_08_amd import synth

pytestmark = pytest.mark.gpu

REL_BF16, ABS_MAX = 1e-2, 5e-2
DEV = "cuda:0"


@pytest.fixture(scope="module")
def m():
    from mla_latent_kv_08_amd import mla
    return mla


def to_dev(x):
    return None if x is None else x.to(DEV).contiguous()


def errors(out_gpu, ref):
    g = out_gpu.float().cpu().double().numpy().reshape(ref.shape)
    assert np.isfinite(g).all(), "non-finite GPU output"
    rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
    return float(rel), float(np.abs(g - ref).max())


def abs_bar(ref, fp8):
    return ABS_MAX * max(1.0, float(np.abs(ref).max())) if fp8 else ABS_MAX


def check(out_gpu, ref, fp8=False, label=""):
    rel, mx = errors(out_gpu, ref)
    print(f"[{label}] relL2={rel:.3e} max|err|={mx:.3e} max|ref|={np.abs(ref).max():.3e}", flush=True)
    assert rel <= REL_BF16, (label, rel)
    assert mx <= abs_bar(ref, fp8), (label, mx)


def gpu_caches(m, w, x):
    """Device caches for inputs x: bf16 rows as given, or FP8 via mla_cache_write."""
    B, T = w.batch, w.max_seq_len
    pe = to_dev(x["pe"])
    if not w.fp8:
        return to_dev(x["kv"]), None, pe
    kv8 = torch.zeros(B, T, 512, dtype=torch.uint8, device=DEV)
    sc = torch.zeros(B, T, 4, dtype=torch.float32, device=DEV)
    pe_c = torch.zeros(B, T, 64, dtype=torch.bfloat16, device=DEV)
    m.cache_write(to_dev(x["kv"]), pe, torch.zeros(B, dtype=torch.int32, device=DEV), kv8, pe_c,
                  kv_scale=sc)
    return kv8, sc, pe_c


def oracle_caches(w, x):
    if not w.fp8:
        return x["kv"], None, x["pe"]
    codes, scales, pe = oracle.cache_write(x["kv"], x["pe"], torch.zeros(w.batch, dtype=torch.int32),
                                           w.max_seq_len, True)
    return codes, scales, pe


def run_case(m, w, x, pairs=None, label=""):
    print(f"[{label}] GPU decode B={w.batch} H={w.heads} T={w.max_seq_len} fp8={w.fp8} "
          f"topk={w.topk}", flush=True)
    kv, sc, pe = gpu_caches(m, w, x)
    out = m.decode(to_dev(x["q_nope"]), to_dev(x["q_pe"]), to_dev(x["wkv_b"]), kv, pe,
                   to_dev(x["cache_lens"]), kv_scale=sc, topk_idx=to_dev(x["topk_idx"]))
    torch.cuda.synchronize()
    okv, osc, ope = oracle_caches(w, x)
    if w.fp8:
        assert np.array_equal(kv.cpu().numpy(), okv), "FP8 codes differ"
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), osc.view(np.uint32)), "scales differ"
    ref = oracle.decode(x["q_nope"], x["q_pe"], x["wkv_b"], okv, ope, x["cache_lens"],
                        synth.SOFTMAX_SCALE, kv_scale=osc, topk_idx=x["topk_idx"], pairs=pairs)
    if pairs is not None:
        got = out.reshape(w.batch, w.heads, 128)[[p[0] for p in pairs], [p[1] for p in pairs]]
        check(got, ref, w.fp8, label)
    else:
        check(out, ref.reshape(w.batch, 1, w.heads, 128), w.fp8, label)
    return out


# ---------------------------------------------------------------- small cases, full compare

# The attention grid depends on the plan: B=1 T=8192 at H=128 (128 plan
# workgroups) splits each one's heads over two workgroups of two head blocks;
# B=4 T=4096 at H=64 (256) runs unsplit workgroups of two head blocks; the
# short cases split four ways into single head blocks.
@pytest.mark.parametrize("B,H,T", [(1, 16, 256), (2, 128, 300), (3, 48, 97), (1, 100, 33),
                                   (2, 32, 1), (1, 128, 64), (1, 128, 8192), (4, 64, 4096)])
def test_dense_small(m, B, H, T):
    w = synth.Workload("dense", B, H, T, seed=100 + T)
    run_case(m, w, synth.make_inputs(w), label=f"dense B{B} H{H} T{T}")


def test_ragged_small_with_poison(m):
    w = synth.Workload("ragged", 6, 64, 1000, ragged=(0, 1000), seed=5)
    x = synth.make_inputs(w)
    x["kv"] = x["kv"].clone()
    x["pe"] = x["pe"].clone()
    x["cache_lens"] = torch.tensor([0, 1, 31, 33, 1000, 517], dtype=torch.int32)
    T = w.max_seq_len
    tail = torch.arange(T).reshape(1, T) >= x["cache_lens"].reshape(-1, 1).long()
    x["kv"][tail] = float("nan")
    x["pe"][tail] = float("nan")
    out = run_case(m, w, x, label="ragged+poison")
    assert (out[0].float() == 0).all()  # length 0 -> zeros


def test_many_sequences(m):
    # more sequences than the work planner keeps in LDS (2048): the rest of the
    # plan takes the per-sequence path; lengths include empty and full ones
    w = synth.Workload("many", 2100, 16, 70, ragged=(0, 70), seed=11)
    x = synth.make_inputs(w)
    lens = x["cache_lens"].clone()
    lens[::7] = 0
    lens[3::11] = 70
    x["cache_lens"] = lens
    run_case(m, w, x, label="B2100")


def test_topk_small(m):
    w = synth.Workload("topk", 3, 128, 2000, topk=300, seed=6)
    x = synth.make_inputs(w)
    idx = x["topk_idx"].clone()
    idx[0, 0, :7] = -1          # padding
    idx[1, 0, -3:] = 5000       # out of range
    x["topk_idx"] = idx
    x["cache_lens"] = torch.tensor([2000, 1500, 2000], dtype=torch.int32)  # b1: entries >= 1500 skipped
    run_case(m, w, x, label="topk300")


@pytest.mark.parametrize("H", [128, 48])
def test_fp8_topk_small(m, H):
    """FP8 cache with a top-k selection: the staging loads take each lane's
    row from the staged indices (H = 48 leaves waves without score heads)."""
    w = synth.Workload("fp8topk", 3, H, 2000, fp8=True, topk=300, outlier_frac=0.01, outlier_mult=20.0,
                       seed=9 + H)
    x = synth.make_inputs(w)
    idx = x["topk_idx"].clone()
    idx[0, 0, :7] = -1          # padding
    idx[1, 0, -3:] = 5000       # out of range
    x["topk_idx"] = idx
    x["cache_lens"] = torch.tensor([2000, 1500, 2000], dtype=torch.int32)  # b1: entries >= 1500 skipped
    run_case(m, w, x, label=f"fp8 topk300 H{H}")


@pytest.mark.parametrize("fp8", [False, True])
def test_topk_unsplit_workgroups(m, fp8):
    """Top-k with 144 plan workgroups (9 sequences x 2048 selected rows, 4 tiles
    each): no head split, every workgroup scores all four head blocks; the
    2048-of-65536 workload (8 sequences, 128 workgroups) splits them in two."""
    w = synth.Workload("topk_unsplit", 9, 128, 3000, fp8=fp8, topk=2048, seed=21 + int(fp8))
    x = synth.make_inputs(w)
    idx = x["topk_idx"].clone()
    idx[0, 0, :11] = -1         # padding
    idx[4, 0, -2:] = 7000       # out of range
    x["topk_idx"] = idx
    run_case(m, w, x, pairs=sample_pairs(w, 48, w.seed), label=f"topk unsplit fp8={fp8}")


def test_topk_all_positions_equals_dense(m):
    w = synth.Workload("dense", 2, 128, 160, seed=7)
    x = synth.make_inputs(w)
    args = [to_dev(x["q_nope"]), to_dev(x["q_pe"]), to_dev(x["wkv_b"]), to_dev(x["kv"]),
            to_dev(x["pe"]), to_dev(x["cache_lens"])]
    dense = m.decode(*args)
    idx = torch.arange(160, dtype=torch.int32).flip(0).reshape(1, 1, 160).expand(2, 1, 160)
    tk = m.decode(*args, topk_idx=to_dev(idx.contiguous()))
    rel, mx = errors(tk, dense.float().cpu().double().numpy())
    assert rel < 1e-2 and mx < 5e-2


def test_fp8_small(m):
    w = synth.Workload("fp8", 2, 128, 200, fp8=True, outlier_frac=0.01, outlier_mult=20.0, seed=8)
    run_case(m, w, synth.make_inputs(w), label="fp8 small")


def test_cache_write_rows_and_dropping(m):
    for fp8 in (False, True):
        B, s, T = 4, 5, 12
        g = torch.Generator().manual_seed(9)
        kv_new = torch.randn(B, s, 512, generator=g).to(torch.bfloat16)
        pe_new = torch.randn(B, s, 64, generator=g).to(torch.bfloat16)
        sp = torch.tensor([0, 9, -2, 3], dtype=torch.int32)
        kv = torch.zeros(B, T, 512, dtype=torch.uint8 if fp8 else torch.bfloat16, device=DEV)
        sc = torch.zeros(B, T, 4, dtype=torch.float32, device=DEV) if fp8 else None
        pe = torch.zeros(B, T, 64, dtype=torch.bfloat16, device=DEV)
        m.cache_write(to_dev(kv_new), to_dev(pe_new), to_dev(sp), kv, pe, kv_scale=sc)
        okv, osc, ope = oracle.cache_write(kv_new, pe_new, sp, T, fp8)
        got_kv = kv.cpu().numpy() if fp8 else kv.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got_kv, okv)
        assert np.array_equal(pe.cpu().view(torch.int16).numpy().view(np.uint16), ope)
        if fp8:
            assert np.array_equal(sc.cpu().numpy().view(np.uint32), osc.view(np.uint32))


def test_fp8_codec_edge_values(m):
    # blocks built to hit ties, saturation, signed zeros, subnormal codes and a zero block
    vals = []
    for c in range(0x7F):
        vals.append(oracle.e4m3fn_value(c))
    v = np.array(vals, np.float32)
    mids = ((v[1:].astype(np.float64) + v[:-1]) / 2).astype(np.float32)
    pool = np.concatenate([v, mids, -mids, [0.0, -0.0, 448.0, -448.0, 1e-3, -1e-3]]).astype(np.float32)
    n_rows = (pool.size + 127) // 128 + 2
    x = np.zeros(n_rows * 512, np.float32)
    x[: pool.size] = pool
    x[-512:-384] = 0.0                       # an all-zero block
    x[-384:-256] = np.float32(3e-39)         # tiny block (scale underflows)
    kv_new = torch.from_numpy(x.reshape(1, n_rows, 512)).to(torch.bfloat16)
    pe_new = torch.zeros(1, n_rows, 64, dtype=torch.bfloat16)
    kv = torch.zeros(1, n_rows, 512, dtype=torch.uint8, device=DEV)
    sc = torch.zeros(1, n_rows, 4, dtype=torch.float32, device=DEV)
    pe = torch.zeros(1, n_rows, 64, dtype=torch.bfloat16, device=DEV)
    m.cache_write(to_dev(kv_new), to_dev(pe_new), torch.zeros(1, dtype=torch.int32, device=DEV),
                  kv, pe, kv_scale=sc)
    okv, osc, _ = oracle.cache_write(kv_new, pe_new, torch.zeros(1, dtype=torch.int32), n_rows, True)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    assert np.array_equal(kv.cpu().numpy(), okv)


def test_deterministic_and_no_out_of_bounds_writes(m):
    w = synth.Workload("det", 3, 128, 700, ragged=(1, 700), seed=10)
    x = synth.make_inputs(w)
    args = [to_dev(x["q_nope"]), to_dev(x["q_pe"]), to_dev(x["wkv_b"]), to_dev(x["kv"]),
            to_dev(x["pe"]), to_dev(x["cache_lens"])]
    guard = 4096
    buf = torch.full((2 * guard + 3 * 128 * 128,), -7.0, dtype=torch.bfloat16, device=DEV)
    out = buf[guard: guard + 3 * 128 * 128].view(3, 1, 128, 128)
    m.decode(*args, out=out)
    first = out.clone()
    m.decode(*args, out=out)
    assert torch.equal(first.view(torch.int16), out.view(torch.int16))
    assert (buf[:guard] == -7.0).all() and (buf[-guard:] == -7.0).all()


# Latent and rotary rows scaled up along the sequence (x 0.5 at row 0 to x 4.5
# at the last row), so the logits keep growing and the running maximum moves
# by more than the lazy-rescale threshold after the first tile (once or twice
# for every head of the bf16 cases): the rescale of non-zero accumulators
# runs, and several waves set the shared rescale flag at once.
# Each instance of the attention kernel runs ten times on the same inputs;
# every output must equal the first bit for bit, and the first the oracle.
@pytest.mark.parametrize("B,H,T,topk,fp8", [(2, 128, 3000, 0, False),    # four head blocks
                                            (1, 128, 4096, 0, False),    # one block, heads split four ways
                                            (4, 128, 8192, 1024, False), # top-k, two blocks
                                            (2, 128, 3000, 0, True)])    # FP8 cache
def test_rescale_path_repeatable(m, B, H, T, topk, fp8):
    w = synth.Workload(f"ramp_b{B}_h{H}_t{T}", B, H, T, fp8=fp8, topk=topk, seed=31 + B)
    x = synth.make_inputs(w)
    ramp = (0.5 + 4.0 * torch.arange(T, dtype=torch.float32) / T).reshape(1, T, 1)
    x["kv"] = (x["kv"].float() * ramp).to(torch.bfloat16)
    x["pe"] = (x["pe"].float() * ramp).to(torch.bfloat16)
    label = f"{w.name} topk={topk} fp8={fp8}"
    print(f"[{label}] GPU decode x10", flush=True)
    kv, sc, pe = gpu_caches(m, w, x)
    args = [to_dev(x["q_nope"]), to_dev(x["q_pe"]), to_dev(x["wkv_b"]), kv, pe, to_dev(x["cache_lens"])]
    kw = dict(kv_scale=sc, topk_idx=to_dev(x["topk_idx"]))
    first = m.decode(*args, **kw)
    torch.cuda.synchronize()
    for rep in range(9):
        again = m.decode(*args, **kw)
        torch.cuda.synchronize()
        assert torch.equal(first.view(torch.int16), again.view(torch.int16)), (label, rep)
    okv, osc, ope = oracle_caches(w, x)
    ref = oracle.decode(x["q_nope"], x["q_pe"], x["wkv_b"], okv, ope, x["cache_lens"],
                        synth.SOFTMAX_SCALE, kv_scale=osc, topk_idx=x["topk_idx"])
    # The output is a convex combination of latent rows scaled by up to 4.5,
    # then up-projected: absolute rounding errors scale with the rows, so the
    # bf16 max |err| bar is scaled by the ramp's maximum; relative L2 is not.
    rel, mx = errors(first, ref.reshape(B, 1, H, 128))
    print(f"[{label}] relL2={rel:.3e} max|err|={mx:.3e}", flush=True)
    assert rel <= REL_BF16, (label, rel)
    assert mx <= abs_bar(ref, fp8) * 4.5, (label, mx)


def test_concurrent_streams_match_sequential(m):
    """The library keeps no device state between calls: two decodes with their
    own workspaces, issued alternately on two streams (default priority) so
    that they may overlap, give bit for bit the outputs of the same calls
    made one after another."""
    cases = []
    for w in [synth.Workload("concA", 4, 128, 3000, ragged=(100, 3000), seed=71),
              synth.Workload("concB", 3, 128, 2000, fp8=True, topk=300, seed=72)]:
        x = synth.make_inputs(w)
        kv, sc, pe = gpu_caches(m, w, x)
        args = [to_dev(x["q_nope"]), to_dev(x["q_pe"]), to_dev(x["wkv_b"]), kv, pe, to_dev(x["cache_lens"])]
        kw = dict(kv_scale=sc, topk_idx=to_dev(x["topk_idx"]))
        ref = m.decode(*args, **kw)
        p = m.make_params(w.batch, w.heads, w.max_seq_len, 1 if w.fp8 else 0, topk=w.topk)
        ws = torch.empty(m.decode_workspace_size(p), dtype=torch.uint8, device=DEV)
        cases.append((args, kw, ref, torch.empty_like(ref), ws))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(5):
        for (args, kw, _, out, ws), st in zip(cases, streams):
            m.decode(*args, **kw, out=out, workspace=ws, stream=st)
        torch.cuda.synchronize()
        for args, kw, ref, out, ws in cases:
            assert torch.equal(ref.view(torch.int16), out.view(torch.int16)), rep


# ---------------------------------------------------------------- the five workloads, full size

def sample_pairs(w, n, seed):
    """n (sequence, head) rows: the four corners, then one random head of
    every sequence (so no ragged length goes unchecked), then random rows."""
    rng = np.random.default_rng(seed)
    b = rng.integers(0, w.batch, n)
    h = rng.integers(0, w.heads, n)
    b[:4] = [0, w.batch - 1, 0, w.batch - 1]
    h[:4] = [0, w.heads - 1, w.heads - 1, 0]
    every = np.arange(w.batch)[: max(0, n - 4)]
    b[4:4 + len(every)] = every
    return [(int(i), int(j)) for i, j in zip(b, h)]


def test_workload_tiny_full(m):
    w = synth.WORKLOADS["tiny_b1_h16_t256"]
    run_case(m, w, synth.make_inputs(w), label=w.name)


def test_workload_dense_4k_full(m):
    w = synth.WORKLOADS["dense_b1_h128_t4096"]
    run_case(m, w, synth.make_inputs(w), label=w.name)


@pytest.mark.parametrize("name", ["ragged_b32_h128_t16384", "fp8_b16_h128_t32768",
                                  "topk2048_b8_h128_t65536"])
def test_workload_full_sampled(m, name):
    w = synth.WORKLOADS[name]
    x = synth.make_inputs(w)
    run_case(m, w, x, pairs=sample_pairs(w, 64, w.seed), label=name)


def test_long_sequences_past_2gib_offsets(m):
    """Maximum-size offsets: two sequences of 2^20 + 64 rows (2 GiB of bf16
    latent).  The second is full, so its last rows sit past byte offset 2^31 of
    the cache; the first ends 7 rows short of the buffer, with NaN in the rows
    it must not read.  Sampled (sequence, head) outputs against the oracle."""
    T = (1 << 20) + 64
    w = synth.Workload("long_b2_h128_t1048640", 2, 128, T, seed=77)
    x = synth.make_inputs(w)
    x["cache_lens"] = torch.tensor([T - 7, T], dtype=torch.int32)
    x["kv"][0, T - 7:] = float("nan")
    x["pe"][0, T - 7:] = float("nan")
    run_case(m, w, x, pairs=sample_pairs(w, 6, w.seed), label=w.name)


# ---------------------------------------------------------------- fused decode step

def _upload_caches(m, w, x):
    """Device copies of the host caches of x (FP8: the oracle's codes and scales)."""
    if not w.fp8:
        return x["kv"].clone(), None, x["pe"].clone()
    codes, scales, pe = oracle.cache_write(x["kv"], x["pe"], torch.zeros(w.batch, dtype=torch.int32),
                                           w.max_seq_len, True)
    return torch.from_numpy(codes), torch.from_numpy(scales), torch.from_numpy(pe.view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("fp8,topk,B", [(False, 0, 5), (True, 0, 5), (False, 96, 3), (True, 96, 3),
                                        (True, 0, 2100), (False, 0, 2100)])
def test_decode_step_writes_then_attends(m, fp8, topk, B):
    T = 70 if B > 100 else 300
    w = synth.Workload("step", B, 16 if B > 100 else 128, T, fp8=fp8, topk=topk, ragged=(0, T), seed=12 + B)
    x = synth.make_inputs(w)
    lens = x["cache_lens"].clone()
    lens[0] = 0              # nothing written, empty attention
    lens[1] = T              # row T - 1 written
    if B > 2:
        lens[2] = T + 5      # row outside the buffer: dropped, attention over T rows
    x["cache_lens"] = lens
    g = torch.Generator().manual_seed(13)
    kv_new = torch.randn(B, 1, 512, generator=g).to(torch.bfloat16)
    pe_new = torch.randn(B, 1, 64, generator=g).to(torch.bfloat16)
    kv_h, sc_h, pe_h = _upload_caches(m, w, x)
    kv, sc, pe = to_dev(kv_h), to_dev(sc_h), to_dev(pe_h)
    print(f"[step] B={B} T={T} fp8={fp8} topk={topk}", flush=True)
    args = [to_dev(x["q_nope"]), to_dev(x["q_pe"]), to_dev(x["wkv_b"])]
    out = m.decode_step(to_dev(kv_new), to_dev(pe_new), *args, kv, pe, to_dev(lens), kv_scale=sc,
                        topk_idx=to_dev(x["topk_idx"]))
    torch.cuda.synchronize()
    # caches: the oracle's cache write at start_pos = cache_lens - 1 on the same old caches
    okv, osc, ope = oracle.cache_write(kv_new, pe_new, (lens - 1).to(torch.int32), T, fp8,
                                       kv_cache=kv_h.numpy().copy() if fp8 else kv_h.view(torch.int16).numpy().view(np.uint16).copy(),
                                       kv_scale=None if sc_h is None else sc_h.numpy().copy(),
                                       pe_cache=pe_h.view(torch.int16).numpy().view(np.uint16).copy())
    got_kv = kv.cpu().numpy() if fp8 else kv.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got_kv, okv), "latent cache differs"
    assert np.array_equal(pe.cpu().view(torch.int16).numpy().view(np.uint16), ope), "rotary cache differs"
    if fp8:
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), osc.view(np.uint32)), "scales differ"
    ref = oracle.decode(x["q_nope"], x["q_pe"], x["wkv_b"], okv, ope, lens, synth.SOFTMAX_SCALE,
                        kv_scale=osc, topk_idx=x["topk_idx"])
    check(out, ref.reshape(B, 1, w.heads, 128), fp8, f"step B{B} fp8={fp8} topk={topk}")
    assert (out[0].float() == 0).all()
    # the same as the two separate calls on the GPU, bit for bit
    kv2, sc2, pe2 = to_dev(kv_h), to_dev(sc_h), to_dev(pe_h)
    m.cache_write(to_dev(kv_new), to_dev(pe_new), to_dev((lens - 1).to(torch.int32)), kv2, pe2,
                  kv_scale=sc2)
    out2 = m.decode(*args, kv2, pe2, to_dev(lens), kv_scale=sc2, topk_idx=to_dev(x["topk_idx"]))
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


# ---------------------------------------------------------------- s > 1 query tokens

def multitoken_case(B, s, H, T, fp8, topk, seed):
    g = torch.Generator().manual_seed(seed)
    bf = lambda *shape, std=1.0: (torch.randn(*shape, generator=g) * std).to(torch.bfloat16)
    x = {"q_nope": bf(B, s, H, 128), "q_pe": bf(B, s, H, 64), "wkv_b": bf(H, 256, 512, std=512 ** -0.5),
         "kv": bf(B, T, 512), "pe": bf(B, T, 64)}
    lens = torch.randint(s, T + 1, (B,), generator=g, dtype=torch.int32)
    lens[0] = T
    if B > 2:
        lens[2] = s - 1  # its first token sees no row
    x["cache_lens"] = lens
    x["topk_idx"] = None
    if topk:
        idx = torch.stack([torch.stack([torch.randperm(T, generator=g)[:topk] for _ in range(s)])
                           for _ in range(B)]).to(torch.int32)
        idx[0, 0, :5] = -1
        x["topk_idx"] = idx
    return x


def host_caches(x, T, fp8):
    """Caches as host tensors: bf16 as drawn, or the oracle's FP8 codes and scales."""
    if not fp8:
        return x["kv"], None, x["pe"]
    B = x["kv"].shape[0]
    codes, scales, pe = oracle.cache_write(x["kv"], x["pe"], torch.zeros(B, dtype=torch.int32), T, True)
    return torch.from_numpy(codes), torch.from_numpy(scales), torch.from_numpy(pe.view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("B,s,H,T,fp8,topk", [(3, 3, 32, 150, False, 0), (2, 2, 128, 300, False, 0),
                                              (3, 4, 16, 97, True, 0), (2, 2, 128, 400, False, 64),
                                              (2, 2, 128, 400, True, 64)])
def test_multitoken_decode(m, B, s, H, T, fp8, topk):
    x = multitoken_case(B, s, H, T, fp8, topk, seed=31 + s + T)
    kv, sc, pe = host_caches(x, T, fp8)
    print(f"[multitoken] B={B} s={s} H={H} T={T} fp8={fp8} topk={topk}", flush=True)
    out = m.decode(to_dev(x["q_nope"]), to_dev(x["q_pe"]), to_dev(x["wkv_b"]), to_dev(kv), to_dev(pe),
                   to_dev(x["cache_lens"]), kv_scale=to_dev(sc), topk_idx=to_dev(x["topk_idx"]))
    torch.cuda.synchronize()
    ref = oracle.decode(x["q_nope"], x["q_pe"], x["wkv_b"], kv, pe, x["cache_lens"], synth.SOFTMAX_SCALE,
                        kv_scale=None if sc is None else sc.numpy(), topk_idx=x["topk_idx"])
    assert tuple(out.shape) == (B, s, H, 128)
    check(out, ref, fp8, f"multitoken B{B} s{s} H{H}")
    if B > 2:
        assert (out[2, 0].float() == 0).all()


# A sequence's s tokens share one attention work item when the selection is
# dense and s x H <= 128: query rows are packed as token i, head h -> row
# i H + h, and each row is masked at its own token's length.  Cases: one, two
# and four row blocks, padding rows (48 and 100 of a 64- or 128-row block, a
# head count that is not a multiple of 16), the FP8 cache, lengths at and
# around the token count and the 32-row tile boundaries, a length past the
# buffer, a sequence of many tiles split over several workgroups, and the
# latent output of the same path.
@pytest.mark.parametrize("B,s,H,T,fp8", [(6, 2, 16, 700, False), (6, 3, 16, 300, False),
                                         (5, 8, 16, 1200, False), (6, 5, 20, 450, False),
                                         (4, 2, 64, 2000, True), (6, 4, 32, 333, True),
                                         (6, 7, 1, 260, False), (6, 40, 3, 500, True)])
def test_packed_tokens(m, B, s, H, T, fp8):
    x = multitoken_case(B, s, H, T, fp8, 0, seed=13 * s + H + T)
    lens = x["cache_lens"]
    edge = [T, 0, s - 1, s, 32 + s - 1, T + 3]  # (a length past T is clamped to T)
    for i in range(min(B, len(edge))):
        lens[i] = edge[i] if i == 5 else min(edge[i], T)
    kv, sc, pe = host_caches(x, T, fp8)
    print(f"[packed] B={B} s={s} H={H} T={T} fp8={fp8} lens={lens.tolist()}", flush=True)
    args = (to_dev(x["q_nope"]), to_dev(x["q_pe"]), to_dev(x["wkv_b"]), to_dev(kv), to_dev(pe),
            to_dev(lens))
    out = m.decode(*args, kv_scale=to_dev(sc))
    lat = m.decode_latent(*args, kv_scale=to_dev(sc))
    torch.cuda.synchronize()
    oargs = (x["q_nope"], x["q_pe"], x["wkv_b"], kv, pe, lens, synth.SOFTMAX_SCALE)
    osc = None if sc is None else sc.numpy()
    ref = oracle.decode(*oargs, kv_scale=osc)
    check(out, ref, fp8, f"packed B{B} s{s} H{H} fp8={fp8}")
    check(lat, oracle.decode_latent(*oargs, kv_scale=osc), fp8, f"packed latent B{B} s{s} H{H}")
    assert (out[1].float() == 0).all()      # length 0: no token sees a row
    assert (out[2, 0].float() == 0).all()   # length s - 1: the first token sees none
    assert not (out[2, 1:].float() == 0).all()


def test_packed_tokens_full_size_sampled(m):
    """The benchmark's packed configuration at full size, with its inputs (the
    same seeds): ragged B=32 over a 16384-row buffer at 16 heads with two query
    tokens per sequence (one work item of 32 packed rows per sequence); both
    tokens of every sequence are checked, at two heads each, plus the corners."""
    w = synth.scaled(synth.WORKLOADS["ragged_b32_h128_t16384"], heads=16, name="ragged_b32_h128_t16384_h16")
    s = 2
    x = synth.add_query_tokens(synth.make_inputs(w), s, seed=w.seed + 1000)
    print(f"[packed full] B={w.batch} s={s} H={w.heads} T={w.max_seq_len}", flush=True)
    out = m.decode(to_dev(x["q_nope"]), to_dev(x["q_pe"]), to_dev(x["wkv_b"]), to_dev(x["kv"]),
                   to_dev(x["pe"]), to_dev(x["cache_lens"]))
    torch.cuda.synchronize()
    rng = np.random.default_rng(77)
    pairs = [(q, int(h)) for q in range(w.batch * s) for h in rng.choice(w.heads, 2, replace=False)]
    pairs += [(0, 0), (w.batch * s - 1, w.heads - 1)]
    ref = oracle.decode(x["q_nope"], x["q_pe"], x["wkv_b"], x["kv"], x["pe"], x["cache_lens"],
                        synth.SOFTMAX_SCALE, pairs=pairs)
    got = out.reshape(w.batch * s, w.heads, 128)[[p[0] for p in pairs], [p[1] for p in pairs]]
    check(got, ref, False, "packed full-size sampled")


def _sweep_configs(n=20, seed=2026):
    """Deterministic draw of small shapes over every plan path: batch, query
    tokens, head count (whole, padded and odd head blocks, so the head split
    and the one-, two- and four-block attention instances), ragged lengths,
    top-k or dense, bf16 or FP8."""
    rng = np.random.default_rng(seed)
    cfgs = []
    while len(cfgs) < n:
        B = int(rng.integers(1, 7))
        s = int(rng.choice([1, 1, 2, 3]))
        H = int(rng.choice([16, 32, 48, 64, 96, 100, 128]))
        T = int(rng.integers(s, 1500))
        fp8 = bool(rng.random() < 0.3)
        topk = int(rng.integers(1, T + 1)) if rng.random() < 0.3 else 0
        if B * s * H * T <= 1_500_000:
            cfgs.append((B, s, H, T, fp8, topk))
    return cfgs


@pytest.mark.parametrize("B,s,H,T,fp8,topk", _sweep_configs())
def test_sweep_random_shapes(m, B, s, H, T, fp8, topk):
    x = multitoken_case(B, s, H, T, fp8, topk, seed=7 * B + 11 * s + H + T)
    kv, sc, pe = host_caches(x, T, fp8)
    print(f"[sweep] B={B} s={s} H={H} T={T} fp8={fp8} topk={topk}", flush=True)
    out = m.decode(to_dev(x["q_nope"]), to_dev(x["q_pe"]), to_dev(x["wkv_b"]), to_dev(kv), to_dev(pe),
                   to_dev(x["cache_lens"]), kv_scale=to_dev(sc), topk_idx=to_dev(x["topk_idx"]))
    torch.cuda.synchronize()
    ref = oracle.decode(x["q_nope"], x["q_pe"], x["wkv_b"], kv, pe, x["cache_lens"], synth.SOFTMAX_SCALE,
                        kv_scale=None if sc is None else sc.numpy(), topk_idx=x["topk_idx"])
    check(out, ref, fp8, f"sweep B{B} s{s} H{H} T{T} fp8={fp8} topk={topk}")


def test_multitoken_full_size_sampled(m):
    B, s, H, T = 4, 2, 128, 4096
    x = multitoken_case(B, s, H, T, False, 0, seed=41)
    print(f"[multitoken] B={B} s={s} H={H} T={T} sampled", flush=True)
    out = m.decode(to_dev(x["q_nope"]), to_dev(x["q_pe"]), to_dev(x["wkv_b"]), to_dev(x["kv"]),
                   to_dev(x["pe"]), to_dev(x["cache_lens"]))
    torch.cuda.synchronize()
    rng = np.random.default_rng(42)
    pairs = [(int(q), int(h)) for q, h in zip(rng.integers(0, B * s, 48), rng.integers(0, H, 48))]
    ref = oracle.decode(x["q_nope"], x["q_pe"], x["wkv_b"], x["kv"], x["pe"], x["cache_lens"],
                        synth.SOFTMAX_SCALE, pairs=pairs)
    got = out.reshape(B * s, H, 128)[[p[0] for p in pairs], [p[1] for p in pairs]]
    check(got, ref, False, "multitoken sampled")


@pytest.mark.parametrize("fp8", [False, True])
def test_multitoken_decode_step(m, fp8):
    B, s, H, T = 3, 2, 64, 120
    x = multitoken_case(B, s, H, T, fp8, 0, seed=51)
    kv_h, sc_h, pe_h = host_caches(x, T, fp8)
    g = torch.Generator().manual_seed(52)
    kv_new = torch.randn(B, s, 512, generator=g).to(torch.bfloat16)
    pe_new = torch.randn(B, s, 64, generator=g).to(torch.bfloat16)
    lens = x["cache_lens"]
    print(f"[multitoken step] B={B} s={s} fp8={fp8}", flush=True)
    kv, sc, pe = to_dev(kv_h), to_dev(sc_h), to_dev(pe_h)
    args = [to_dev(x["q_nope"]), to_dev(x["q_pe"]), to_dev(x["wkv_b"])]
    out = m.decode_step(to_dev(kv_new), to_dev(pe_new), *args, kv, pe, to_dev(lens), kv_scale=sc)
    torch.cuda.synchronize()
    u16 = lambda t: t.view(torch.int16).numpy().view(np.uint16).copy()
    okv, osc, ope = oracle.cache_write(kv_new, pe_new, (lens - s).to(torch.int32), T, fp8,
                                       kv_cache=kv_h.numpy().copy() if fp8 else u16(kv_h),
                                       kv_scale=None if sc_h is None else sc_h.numpy().copy(),
                                       pe_cache=u16(pe_h))
    got_kv = kv.cpu().numpy() if fp8 else kv.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got_kv, okv), "latent cache differs"
    assert np.array_equal(pe.cpu().view(torch.int16).numpy().view(np.uint16), ope), "rotary cache differs"
    if fp8:
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), osc.view(np.uint32)), "scales differ"
    ref = oracle.decode(x["q_nope"], x["q_pe"], x["wkv_b"], okv, ope, lens, synth.SOFTMAX_SCALE, kv_scale=osc)
    check(out, ref, fp8, f"multitoken step fp8={fp8}")
    kv2, sc2, pe2 = to_dev(kv_h), to_dev(sc_h), to_dev(pe_h)
    m.cache_write(to_dev(kv_new), to_dev(pe_new), to_dev((lens - s).to(torch.int32)), kv2, pe2, kv_scale=sc2)
    out2 = m.decode(*args, kv2, pe2, to_dev(lens), kv_scale=sc2)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


# ---------------------------------------------------------------- HIP graph capture

@pytest.mark.parametrize("fp8", [False, True])
def test_decode_step_graph_replays(m, fp8):
    """The fused step recorded into a HIP graph gives, on every replay, the eager
    result bit for bit (the header promises capture safety; the benchmark relies on it)."""
    w = synth.Workload("graph", 4, 128, 700, fp8=fp8, ragged=(1, 700), seed=61)
    x = synth.make_inputs(w)
    kv_h, sc_h, pe_h = _upload_caches(m, w, x)
    lens = x["cache_lens"]
    B, T = w.batch, w.max_seq_len
    # the new row of every sequence is the row already cached there, so the
    # step leaves the caches as they are and every call sees the same inputs
    rows = (lens.long() - 1).clamp(min=0)
    kv_new = x["kv"][torch.arange(B), rows].reshape(B, 1, 512).contiguous()
    pe_new = x["pe"][torch.arange(B), rows].reshape(B, 1, 64).contiguous()
    if fp8:  # FP8: the re-quantised row must reproduce its stored codes
        codes, scales, _ = oracle.cache_write(kv_new, pe_new, (lens - 1).to(torch.int32), T, True,
                                              kv_cache=kv_h.numpy().copy(), kv_scale=sc_h.numpy().copy(),
                                              pe_cache=pe_h.view(torch.int16).numpy().view(np.uint16).copy())
        assert np.array_equal(codes, kv_h.numpy()) and np.array_equal(scales.view(np.uint32), sc_h.numpy().view(np.uint32))
    d = {k: to_dev(v) for k, v in dict(q_nope=x["q_nope"], q_pe=x["q_pe"], wkv_b=x["wkv_b"], kv=kv_h, sc=sc_h,
                                        pe=pe_h, lens=lens, kv_new=kv_new, pe_new=pe_new).items()}
    p = m.make_params(B, w.heads, T, 1 if fp8 else 0)
    ws = torch.empty(m.decode_workspace_size(p), dtype=torch.uint8, device=DEV)
    out = torch.empty(B, 1, w.heads, 128, dtype=torch.bfloat16, device=DEV)
    step = lambda: m.decode_step(d["kv_new"], d["pe_new"], d["q_nope"], d["q_pe"], d["wkv_b"], d["kv"], d["pe"],
                                 d["lens"], kv_scale=d["sc"], out=out, workspace=ws)
    print(f"[graph] fp8={fp8}", flush=True)
    step()
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        out.fill_(-1.0)          # eager work between the replays
        ws.fill_(0x7F)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r} differs"
