"""GPU parity of the 8-bit KV formats with one scale per head (E4M3 and INT8),
through the C ABI's *_head_scales entry points, against the oracle.

* The cache write of every f16 and bf16 bit pattern into every head, each
  head with its own scale, bit for bit against the oracle's encoders.
* The decode of every E4M3 code and INT8 byte, each head with its own
  power-of-two scale, exactly.
* The per-head fp8 and INT8 workloads (C5 and C6 shapes, scales drawn per
  head), small on every sequence and full size on sampled sequences, within
  the stated 3e-2; and both formats with per-head scales from U[0.01, 0.1].
* Equal per-head scales give the per-pool form's bits: pools and outputs of
  the cache write, the decode (one call, two phases, appending form) and the
  prompt attention (plain and appending).
* Prompt attention over per-head 8-bit pools against the oracle.
* The decode step captured as a HIP graph with per-head scales: replays are
  bitwise equal to the eager step and read the scales' current contents.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_common import (assert_tolerance_budget, check_step, check_untouched, oracle_step, out_f64, require_gpu,
                        run_gpu_step, sample_seqs, touched)

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[head-scales] {msg}", flush=True)


def _u8(t):
    return t.contiguous().view(torch.uint8)


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
@pytest.mark.parametrize("src", ["f16", "bf16"])
def test_encode_all_16bit_patterns_per_head(fmt, src):
    """Every pattern through every head; the five heads' scales are those
    the per-pool pattern tests use, one per head."""
    pkv = require_gpu()
    scales = [1.0, 0.0123, 0.0625, 0.1 if fmt == "e4m3" else 0.04, 3.7]
    H, D, BS = len(scales), 128, 32
    T = 65536 // D
    pat = np.arange(65536, dtype=np.uint16).reshape(T, 1, D).repeat(H, axis=1)     # [T, H, D]
    rev = pat[::-1].copy()
    tdt = torch.float16 if src == "f16" else torch.bfloat16
    key = torch.from_numpy(pat.view(np.int16)).view(tdt).to("cuda")
    value = torch.from_numpy(rev.view(np.int16)).view(tdt).to("cuda")
    NB = T // BS + 1
    pool_dt = torch.uint8 if fmt == "e4m3" else torch.int8
    kc = torch.full((NB, H, BS, D), 0x55, dtype=pool_dt, device="cuda")
    vc = torch.full_like(kc, 0x55)
    slots = np.random.default_rng(3).permutation(NB * BS)[:T].astype(np.int32)
    ks = np.array(scales, dtype=np.float32)
    vs = ks[::-1].copy()
    pkv.reshape_and_cache(key, value, kc, vc, torch.from_numpy(slots).to("cuda"), torch.from_numpy(ks).cuda(),
                          torch.from_numpy(vs).cuda())
    torch.cuda.synchronize()
    k0 = np.full((NB, H, BS, D), 0x55, np.uint8)
    ko, vo = oracle.reshape_and_cache(pat, rev, k0, k0.copy(), slots, src, fmt, ks, vs)
    assert np.array_equal(_u8(kc).cpu().numpy(), ko)
    assert np.array_equal(_u8(vc).cpu().numpy(), vo)


def _many_scales():
    """64 scales: powers of two, 1 and its neighbours, significands of all
    ones, thirds and tenths, and log-uniform draws over 2^-24 .. 2^24."""
    f32 = np.float32
    fixed = [1.0, 0.5, 2.0, 2.0 ** -20, 2.0 ** 20, float(np.nextafter(f32(1), f32(2))),
             float(np.nextafter(f32(1), f32(0))), float(np.nextafter(f32(2), f32(0))), 3.0, 1.0 / 3.0, 0.1, 0.7,
             7.0, 0.0123, 0.04, 448.0]
    rng = np.random.default_rng(2024)
    drawn = np.exp2(rng.uniform(-24.0, 24.0, size=64 - len(fixed)))
    return np.array(fixed + drawn.tolist(), dtype=np.float32)


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
@pytest.mark.parametrize("src", ["f16", "bf16"])
def test_encode_all_16bit_patterns_over_many_scales(fmt, src):
    """Every 16-bit pattern divided by 64 scales spread over 2^-24 .. 2^24
    (one per head, K and V in opposite orders) and encoded: bit for bit the
    oracle's IEEE fp32 division and encoder, so the kernel's division is
    correctly rounded at every quotient these give, from zeros, subnormals
    and infinities to the saturation range."""
    pkv = require_gpu()
    scales = _many_scales()
    H, D, BS = len(scales), 128, 32
    T = 65536 // D
    pat = np.arange(65536, dtype=np.uint16).reshape(T, 1, D).repeat(H, axis=1)     # [T, H, D]
    rev = pat[::-1].copy()
    tdt = torch.float16 if src == "f16" else torch.bfloat16
    key = torch.from_numpy(pat.view(np.int16)).view(tdt).to("cuda")
    value = torch.from_numpy(rev.view(np.int16)).view(tdt).to("cuda")
    NB = T // BS + 1
    pool_dt = torch.uint8 if fmt == "e4m3" else torch.int8
    kc = torch.full((NB, H, BS, D), 0x55, dtype=pool_dt, device="cuda")
    vc = torch.full_like(kc, 0x55)
    slots = np.random.default_rng(5).permutation(NB * BS)[:T].astype(np.int32)
    ks = scales
    vs = ks[::-1].copy()
    _announce(f"encode all patterns over {H} scales, {src} -> {fmt}")
    pkv.reshape_and_cache(key, value, kc, vc, torch.from_numpy(slots).to("cuda"), torch.from_numpy(ks).cuda(),
                          torch.from_numpy(vs).cuda())
    torch.cuda.synchronize()
    k0 = np.full((NB, H, BS, D), 0x55, np.uint8)
    ko, vo = oracle.reshape_and_cache(pat, rev, k0, k0.copy(), slots, src, fmt, ks, vs)
    got_k, got_v = _u8(kc).cpu().numpy(), _u8(vc).cpu().numpy()
    for name, got, want in (("K", got_k, ko), ("V", got_v, vo)):
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{name}: {len(bad)} bytes differ, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
def test_decode_all_codes_per_head(fmt):
    """n = 1: out = decode(byte) * v_scale[h] exactly, for every byte in
    every head (power-of-two scales keep every product exact in fp16)."""
    pkv = require_gpu()
    H, D, BS = 4, 256, 32
    codes = np.arange(256, dtype=np.uint8)
    pool_dt = torch.uint8 if fmt == "e4m3" else torch.int8
    kc = torch.zeros((2, H, BS, D), dtype=pool_dt, device="cuda")
    vc = torch.zeros_like(kc)
    vc[1, :, 0, :] = torch.from_numpy(np.tile(codes, (H, 1))).view(pool_dt).to("cuda")
    q = torch.zeros((1, H, D), dtype=torch.float16, device="cuda")
    out = torch.empty_like(q)
    bt = torch.tensor([[1]], dtype=torch.int32, device="cuda")
    cl = torch.tensor([1], dtype=torch.int32, device="cuda")
    vs = torch.tensor([1.0, 2.0, 0.5, 4.0], dtype=torch.float32, device="cuda")
    ks = torch.tensor([0.25, 1.0, 8.0, 0.125], dtype=torch.float32, device="cuda")
    pkv.paged_attention_decode(out, q, kc, vc, bt, cl, 0.1, ks, vs)
    torch.cuda.synchronize()
    got = out_f64(out[0])                                   # [H, D]
    dec = oracle.decode(codes, fmt)
    for h in range(H):
        want = dec * float(vs[h])
        nan = np.isnan(want)
        assert (np.isnan(got[h]) == nan).all()
        assert (got[h][~nan] == want[~nan]).all(), h


@pytest.mark.parametrize("cfg", [W.CONFIG_5_HEAD_SCALES, W.CONFIG_6_HEAD_SCALES], ids=["e4m3", "i8"])
def test_small_head_scale_workload_all_sequences(cfg):
    pkv = require_gpu()
    _announce(f"{cfg.name} small")
    case = W.make_case(cfg, device="cpu", S=24, H=4)
    g = run_gpu_step(pkv, case)
    o = oracle_step(case, g.k_pre, g.v_pre)
    err = check_step(case, g, o, f"{cfg.name}-small")
    assert_tolerance_budget(case, o)
    check_untouched(g, touched(case))
    _announce(f"{cfg.name} small: max abs err {err:.3g}")


@pytest.mark.parametrize("cfg", [W.CONFIG_5_HEAD_SCALES, W.CONFIG_6_HEAD_SCALES], ids=["e4m3", "i8"])
def test_full_head_scale_workload_sampled(cfg):
    pkv = require_gpu()
    _announce(f"{cfg.name} full size, generated on the GPU")
    case = W.make_case(cfg, device="cuda")
    g = run_gpu_step(pkv, case)
    seqs = sample_seqs(case, 8, seed=cfg.index)
    o = oracle_step(case, g.k_pre, g.v_pre, seqs)
    err = check_step(case, g, o, f"{cfg.name}-full")
    assert_tolerance_budget(case, o)
    check_untouched(g, touched(case))
    _announce(f"{cfg.name} full: {len(seqs)} sequences, max abs err {err:.3g}")
    del g, case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
def test_head_scales_over_the_wide_range(fmt):
    """Per-head scales from U[0.01, 0.1] for both formats (INT8 then
    saturates often at the small scales; the stored bytes decide)."""
    pkv = require_gpu()
    base = W.CONFIG_5_HEAD_SCALES if fmt == "e4m3" else W.CONFIG_6_HEAD_SCALES
    cfg = replace(base, name=f"{fmt}-head-scales-wide", scale_lo=0.01, scale_hi=0.1)
    case = W.make_case(cfg, device="cpu", S=16, H=6)
    assert case.k_scale.min() < 0.04 and case.k_scale.max() > 0.04
    g = run_gpu_step(pkv, case)
    o = oracle_step(case, g.k_pre, g.v_pre)
    check_step(case, g, o, cfg.name)


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
def test_equal_head_scales_give_the_per_pool_bits(fmt):
    pkv = require_gpu()
    cfg = W.CONFIGS[5] if fmt == "e4m3" else W.CONFIGS[6]
    lens = [1, 31, 32, 33, 500, 2047, 2048, 2049, 3000, 4096]      # one to two partitions
    case = W.make_case(cfg, device="cpu", H=3, context_lens=lens).to("cuda")
    ks = torch.full((case.H,), case.k_scale, dtype=torch.float32, device="cuda")
    vs = torch.full((case.H,), case.v_scale, dtype=torch.float32, device="cuda")
    slots = torch.from_numpy(case.slot_mapping).cuda()
    bt = torch.from_numpy(case.block_tables).cuda()
    cl = torch.from_numpy(case.context_lens).cuda()
    assert int(case.context_lens.max()) > 2048                   # the merge runs
    ws = pkv.alloc_decode_workspace(case.S, case.H, case.D, case.BS, case.MB)
    results = {}
    for mode, (a, b) in (("pool", (case.k_scale, case.v_scale)), ("head", (ks, vs))):
        kc, vc = case.k_cache.clone(), case.v_cache.clone()
        pkv.reshape_and_cache(case.key, case.value, kc, vc, slots, a, b)
        out1 = torch.empty_like(case.q)
        pkv.paged_attention_decode(out1, case.q, kc, vc, bt, cl, case.scale, a, b, workspace=ws)
        out2 = torch.empty_like(case.q)
        pkv.paged_attention_decode_partitions(out2, case.q, kc, vc, bt, cl, case.scale, a, b, workspace=ws)
        pkv.paged_attention_decode_merge(out2, cl, case.BS, case.MB, kc.dtype, b, workspace=ws)
        kc3, vc3 = case.k_cache.clone(), case.v_cache.clone()
        out3 = torch.empty_like(case.q)
        pkv.paged_attention_decode_append(out3, case.q, case.key, case.value, kc3, vc3, slots, bt, cl, case.scale,
                                          a, b, workspace=ws)
        torch.cuda.synchronize()
        results[mode] = [_u8(x).clone() for x in (kc, vc, out1, out2, kc3, vc3, out3)]
    for i, (x, y) in enumerate(zip(results["pool"], results["head"])):
        assert torch.equal(x, y), f"{fmt}: result {i} differs between per-pool and equal per-head scales"
    # prompt attention over the same pools
    pc = replace(W.PREFILL_CONFIGS[1], cache_dtype=fmt)
    p = W.make_prefill_case(pc, device="cuda")
    ph = torch.full((p.H,), p.k_scale, dtype=torch.float32, device="cuda")
    pv = torch.full((p.H,), p.v_scale, dtype=torch.float32, device="cuda")
    pbt, pcl = torch.from_numpy(p.block_tables).cuda(), torch.from_numpy(p.context_lens).cuda()
    pcu, psl = torch.from_numpy(p.cu_q_lens).cuda(), torch.from_numpy(p.slot_mapping).cuda()
    outs = {}
    for mode, (a, b) in (("pool", (p.k_scale, p.v_scale)), ("head", (ph, pv))):
        kc, vc = p.k_cache.clone(), p.v_cache.clone()
        o1 = torch.empty_like(p.q)
        pkv.paged_attention_prefill_append(o1, p.q, p.key, p.value, kc, vc, psl, pbt, pcl, pcu, p.max_q_len, p.scale,
                                           a, b)
        o2 = torch.empty_like(p.q)
        pkv.paged_attention_prefill(o2, p.q, kc, vc, pbt, pcl, pcu, p.max_q_len, p.scale, a, b)
        torch.cuda.synchronize()
        outs[mode] = [_u8(x).clone() for x in (kc, vc, o1, o2)]
    for i, (x, y) in enumerate(zip(outs["pool"], outs["head"])):
        assert torch.equal(x, y), f"{fmt}: prompt result {i} differs between per-pool and equal per-head scales"


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
def test_prefill_with_head_scales_against_the_oracle(fmt):
    import test_gpu_prefill as P
    pkv = require_gpu()
    for base in (W.PREFILL_CONFIGS[1], W.PREFILL_CONFIGS[3]):
        cfg = replace(base, cache_dtype=fmt, head_scales=True)
        case = W.make_prefill_case(cfg, device="cuda" if base.index == 3 else "cpu")
        assert case.k_scale.shape == (case.H,)
        _announce(f"prompt {cfg.name} / {fmt} per head")
        k_pre, v_pre, gk, gv, gout = P.run_gpu(pkv, case)
        seqs = None if base.index == 1 else P.sample(case, 2, seed=5)
        o = P.oracle_run(case, k_pre, v_pre, seqs)
        err = P.check(case, gk, gv, gout, o, f"prompt {cfg.name} {fmt} per head")
        _announce(f"prompt {cfg.name} / {fmt} per head: max abs err {err:.3g}")
        del case, k_pre, v_pre, gk, gv, gout
        torch.cuda.empty_cache()


@pytest.mark.parametrize("append", [False, True])
def test_graph_with_head_scales(append):
    pkv = require_gpu()
    case = W.make_case(W.CONFIG_5_HEAD_SCALES, device="cpu", S=12, H=4).to("cuda")
    ks = torch.from_numpy(case.k_scale).cuda()
    vs = torch.from_numpy(case.v_scale).cuda()
    slots = torch.from_numpy(case.slot_mapping).cuda()
    bt = torch.from_numpy(case.block_tables).cuda()
    cl = torch.from_numpy(case.context_lens).cuda()
    ws = pkv.alloc_decode_workspace(case.S, case.H, case.D, case.BS, case.MB)

    def eager():
        kc, vc = case.k_cache.clone(), case.v_cache.clone()
        out = torch.empty_like(case.q)
        pkv.reshape_and_cache(case.key, case.value, kc, vc, slots, ks, vs)
        pkv.paged_attention_decode(out, case.q, kc, vc, bt, cl, case.scale, ks, vs, workspace=ws)
        torch.cuda.synchronize()
        return [_u8(x).clone() for x in (kc, vc, out)]

    want = eager()
    kc, vc = case.k_cache.clone(), case.v_cache.clone()
    out = torch.empty_like(case.q)
    g = pkv.DecodeGraph(kc, vc, case.key, case.value, slots, case.q, out, bt, cl, case.scale, ks, vs,
                        workspace=torch.empty_like(ws) if ws is not None else None, append=append)
    for rep in range(3):
        kc.copy_(case.k_cache)
        vc.copy_(case.v_cache)
        g.launch()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip([_u8(t) for t in (kc, vc, out)], want)):
            assert torch.equal(x, y), f"replay {rep}: result {i} differs from the eager step"
    # the graph reads the scales' current contents at every replay
    ks.mul_(2.0)
    vs.mul_(0.5)
    want2 = eager()
    kc.copy_(case.k_cache)
    vc.copy_(case.v_cache)
    g.launch()
    torch.cuda.synchronize()
    for i, (x, y) in enumerate(zip([_u8(t) for t in (kc, vc, out)], want2)):
        assert torch.equal(x, y), f"changed scales: result {i} differs from the eager step"
    g.destroy()
