"""GPU edge cases and invariants through the C ABI.

* Context lengths at every boundary the kernel has (1, a block, a block + 1,
  a partition, a partition + 1, a full block table), and n = 0 (zeros).
* One token: the output is that token's V, bit for bit.
* Placement invariance: permuting the physical blocks gives bitwise-equal
  outputs; a shared prefix gives the same bits as private copies of it
  ("在A10G上榨干LLaMA-7B：vLLM与PagedAttention实战" §2.1 and §2.2).  The
  kernel's arithmetic order depends only on logical token positions.
* Block size 16 versus 32 for the same tokens: within tolerance.
* The fp8 decode of all 256 E4M3 codes and the fp8 encode of all 65536 fp16 and bf16
  bit patterns, against the oracle's codecs; the same for INT8.
* The block gather, bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_common import TOL, check_step, oracle_step, out_f64, require_gpu, run_gpu_step

pytestmark = pytest.mark.gpu

PART_TOKENS = 2048   # tokens per decode partition


def _announce(msg):
    print(f"[edges] {msg}", flush=True)


def _decode(pkv, case, kc=None, vc=None, tables=None, lens=None):
    dev = "cuda"
    kc = case.k_cache if kc is None else kc
    vc = case.v_cache if vc is None else vc
    bt = torch.from_numpy(case.block_tables if tables is None else tables).to(dev)
    cl = torch.from_numpy(case.context_lens if lens is None else lens).to(dev)
    out = torch.empty_like(case.q)
    pkv.paged_attention_decode(out, case.q, kc, vc, bt, cl, case.scale, case.k_scale, case.v_scale)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("idx", [1, 2, 3, 5, 6])
def test_boundary_lengths(idx):
    pkv = require_gpu()
    cfg = W.CONFIGS[idx]
    BS, part = cfg.BS, PART_TOKENS
    lens = [1, 2, BS - 1, BS, BS + 1, part - 1, part, part + 1, 2 * part + 3, cfg.MB * BS]
    _announce(f"config {idx} lengths {lens}")
    case = W.make_case(cfg, device="cpu", H=2, context_lens=lens)
    g = run_gpu_step(pkv, case)
    o = oracle_step(case, g.k_pre, g.v_pre)
    check_step(case, g, o, f"C{idx}-boundaries")


@pytest.mark.parametrize("idx", [1, 2, 3])
def test_single_token_is_v0_bitwise(idx):
    pkv = require_gpu()
    cfg = W.CONFIGS[idx]
    case = W.make_case(cfg, device="cpu", H=3, context_lens=[1, 1, 1, 1]).to("cuda")
    g = run_gpu_step(pkv, case, keep_pre=False)
    for s in range(case.S):
        blk, off = divmod(int(case.slot_mapping[s]), case.BS)
        v0 = g.v_post[blk, :, off, :]
        assert torch.equal(g.out[s].view(torch.int16 if cfg.q_dtype != "f32" else torch.int32),
                           v0.view(torch.int16 if cfg.q_dtype != "f32" else torch.int32))


@pytest.mark.parametrize("idx", [1, 3, 5, 6])
def test_zero_length_gives_zeros(idx):
    pkv = require_gpu()
    cfg = W.CONFIGS[idx]
    case = W.make_case(cfg, device="cpu", H=2, context_lens=[5, 40, 300]).to("cuda")
    run_gpu_step(pkv, case, keep_pre=False)          # the new tokens are written first
    lens = np.array([0, 40, 0], dtype=np.int32)
    out = _decode(pkv, case, lens=lens)
    assert (out[0] == 0).all() and (out[2] == 0).all() and torch.isfinite(out[1].float()).all()


def _permuted(case, perm):
    """Move physical block b to perm[b] (tables follow)."""
    p = torch.as_tensor(perm, device=case.k_cache.device)
    kc = torch.empty_like(case.k_cache)
    vc = torch.empty_like(case.v_cache)
    kc[p] = case.k_cache
    vc[p] = case.v_cache
    return kc, vc, perm[case.block_tables].astype(np.int32)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5, 6])
def test_block_permutation_is_bitwise_invariant(idx):
    pkv = require_gpu()
    cfg = W.CONFIGS[idx]
    kw = {} if idx in (1, 2) else dict(S=12, H=2)
    case = W.make_case(cfg, device="cpu", **kw).to("cuda")
    g = run_gpu_step(pkv, case, keep_pre=False)
    perm = np.random.default_rng(idx).permutation(case.NB)
    kc, vc, tables = _permuted(case, perm)
    out2 = _decode(pkv, case, kc, vc, tables)
    assert torch.equal(g.out.view(torch.uint8), out2.view(torch.uint8))


def test_shared_prefix_equals_duplicated_bitwise():
    pkv = require_gpu()
    case = W.make_case(W.CONFIGS[4], device="cpu", S=16, H=4).to("cuda")
    g = run_gpu_step(pkv, case, keep_pre=False)
    # duplicate: give every sequence private copies of all the blocks it shares
    tables = case.block_tables.copy()
    use = {}
    for s in range(case.S):
        for j in range(-(-int(case.context_lens[s]) // case.BS)):
            use.setdefault(int(tables[s, j]), []).append((s, j))
    extra = [(b, sj) for b, sj in use.items() if len(sj) > 1]
    n_new = sum(len(sj) - 1 for _, sj in extra)
    kc = torch.cat([case.k_cache, torch.empty((n_new,) + tuple(case.k_cache.shape[1:]),
                                              dtype=case.k_cache.dtype, device="cuda")])
    vc = torch.cat([case.v_cache, torch.empty_like(kc[case.NB:])])
    nxt = case.NB
    for b, sj in extra:
        for s, j in sj[1:]:
            kc[nxt] = kc[b]
            vc[nxt] = vc[b]
            tables[s, j] = nxt
            nxt += 1
    assert n_new > 0
    out2 = _decode(pkv, case, kc, vc, tables)
    assert torch.equal(g.out.view(torch.uint8), out2.view(torch.uint8))


def test_block_size_change_within_tolerance():
    pkv = require_gpu()
    # the same logical tokens laid out with BS = 16 and with BS = 32
    cfg16 = W.CONFIGS[2]
    case = W.make_case(cfg16, device="cpu", H=4).to("cuda")
    g = run_gpu_step(pkv, case, keep_pre=False)
    S, H, D = case.S, case.H, case.D
    MB32 = -(-int(case.context_lens.max()) // 32)
    NB32 = S * MB32 + 1
    kc = torch.full((NB32, H, 32, D), float("nan"), dtype=case.k_cache.dtype, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    tables = np.zeros((S, MB32), dtype=np.int32)
    for s in range(S):
        n = int(case.context_lens[s])
        t = torch.arange(n, device="cuda")
        src_b = torch.from_numpy(case.block_tables[s]).to("cuda").long()[t // 16]
        rows_k = case.k_cache[src_b, :, t % 16, :]          # [n, H, D]
        rows_v = case.v_cache[src_b, :, t % 16, :]
        for j in range(-(-n // 32)):
            b = 1 + s * MB32 + j
            tables[s, j] = b
            m = min(32, n - 32 * j)
            kc[b, :, :m, :] = rows_k[32 * j:32 * j + m].transpose(0, 1)
            vc[b, :, :m, :] = rows_v[32 * j:32 * j + m].transpose(0, 1)
    bt = torch.from_numpy(tables).to("cuda")
    cl = torch.from_numpy(case.context_lens).to("cuda")
    out2 = torch.empty_like(case.q)
    pkv.paged_attention_decode(out2, case.q, kc, vc, bt, cl, case.scale)
    torch.cuda.synchronize()
    err = float((g.out.float() - out2.float()).abs().max())
    assert err <= TOL["f16"]


def test_fp8_decode_all_256_codes():
    pkv = require_gpu()
    # n = 1, v_scale = 1: out = decode(v0) exactly (every E4M3 value fits fp16)
    H, D, BS = 2, 128, 32
    codes = np.arange(256, dtype=np.uint8).reshape(H, D)
    kc = torch.zeros((2, H, BS, D), dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    vc[1, :, 0, :] = torch.from_numpy(codes).to("cuda")
    q = torch.zeros((1, H, D), dtype=torch.float16, device="cuda")
    out = torch.empty_like(q)
    bt = torch.tensor([[1]], dtype=torch.int32, device="cuda")
    cl = torch.tensor([1], dtype=torch.int32, device="cuda")
    pkv.paged_attention_decode(out, q, kc, vc, bt, cl, 0.1, 1.0, 1.0)
    torch.cuda.synchronize()
    got = out_f64(out[0]).reshape(-1)
    want = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == want[~nan]).all()
    # the sign of a nonzero value survives; a zero's sign does not survive the
    # weighted sum (the accumulator starts at +0), and has no meaning there
    nz = ~nan & (want != 0)
    assert (np.signbit(got[nz]) == np.signbit(want[nz])).all()


@pytest.mark.parametrize("src", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 0.0123, 0.0625, 0.1, 3.7])
def test_fp8_encode_all_16bit_patterns(src, scale):
    """Every f16 and bf16 bit pattern through the quantising cache write.
    bf16 sources span fp32's whole exponent range (saturation, infinities,
    NaN, underflow to zero), and at scale 1 they hit every rounding
    midpoint of E4M3 exactly, and one bf16 step on either side of it."""
    pkv = require_gpu()
    H, D, BS = 2, 128, 32
    T = 65536 // (H * D)
    pat = np.arange(65536, dtype=np.uint16).reshape(T, H, D)
    tdt = torch.float16 if src == "f16" else torch.bfloat16
    key = torch.from_numpy(pat.view(np.int16)).view(tdt).to("cuda")
    value = torch.from_numpy(pat[::-1].copy().view(np.int16)).view(tdt).to("cuda")
    NB = T // BS + 1
    kc = torch.full((NB, H, BS, D), 0x55, dtype=torch.uint8, device="cuda")
    vc = torch.full_like(kc, 0x55)
    slots = np.random.default_rng(1).permutation(NB * BS)[:T].astype(np.int32)
    s32 = float(np.float32(scale))
    pkv.reshape_and_cache(key, value, kc, vc, torch.from_numpy(slots).to("cuda"), s32, s32)
    torch.cuda.synchronize()
    k0 = np.full((NB, H, BS, D), 0x55, np.uint8)
    ko, vo = oracle.reshape_and_cache(pat, pat[::-1].copy(), k0, k0.copy(), slots, src, "e4m3", s32, s32)
    assert np.array_equal(kc.cpu().numpy(), ko)
    assert np.array_equal(vc.cpu().numpy(), vo)


@pytest.mark.parametrize("idx", [1, 3, 5, 6])
def test_gather_kv_bitwise(idx):
    pkv = require_gpu()
    cfg = W.CONFIGS[idx]
    kw = {} if idx == 1 else dict(S=10, H=2)
    case = W.make_case(cfg, device="cpu", **kw)
    g = run_gpu_step(pkv, case)
    total = int(case.context_lens.sum())
    ko = torch.empty((total, case.H, case.D), dtype=g.k_post.dtype, device="cuda")
    vo = torch.empty_like(ko)
    cu = np.zeros(case.S + 1, dtype=np.int32)
    cu[1:] = np.cumsum(case.context_lens)
    pkv.gather_kv(ko, vo, torch.from_numpy(cu).to("cuda"), g.k_post, g.v_post, g.block_tables, g.context_lens)
    torch.cuda.synchronize()
    o = oracle_step(case, g.k_pre, g.v_pre)        # the oracle's own post-step pools
    # every sequence's blocks, renumbered: gather from the oracle's mini pools
    tables = np.zeros_like(case.block_tables)
    remap = {int(b): i for i, b in enumerate(o.blocks)}
    for s in range(case.S):
        nb = -(-int(case.context_lens[s]) // case.BS)
        tables[s, :nb] = [remap[int(b)] for b in case.block_tables[s, :nb]]
    ke, ve, cu_e = oracle.gather_kv(o.k_post, o.v_post, tables, case.context_lens)
    assert np.array_equal(W.bits(ko, case.cache_dtype), ke)
    assert np.array_equal(W.bits(vo, case.cache_dtype), ve)


def test_int8_decode_all_256_bytes():
    pkv = require_gpu()
    # n = 1, v_scale = 1: out = the byte's integer value exactly (all fit fp16)
    H, D, BS = 2, 128, 32
    codes = np.arange(256, dtype=np.uint8).reshape(H, D)
    kc = torch.zeros((2, H, BS, D), dtype=torch.int8, device="cuda")
    vc = torch.zeros_like(kc)
    vc[1, :, 0, :] = torch.from_numpy(codes.view(np.int8)).to("cuda")
    q = torch.zeros((1, H, D), dtype=torch.float16, device="cuda")
    out = torch.empty_like(q)
    bt = torch.tensor([[1]], dtype=torch.int32, device="cuda")
    cl = torch.tensor([1], dtype=torch.int32, device="cuda")
    pkv.paged_attention_decode(out, q, kc, vc, bt, cl, 0.1, 1.0, 1.0)
    torch.cuda.synchronize()
    got = out_f64(out[0]).reshape(-1)
    assert np.array_equal(got, oracle.i8_decode(np.arange(256, dtype=np.uint8)))


@pytest.mark.parametrize("src", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 0.0123, 0.0625, 0.04, 3.7])
def test_int8_encode_all_16bit_patterns(src, scale):
    pkv = require_gpu()
    H, D, BS = 2, 128, 32
    T = 65536 // (H * D)
    pat = np.arange(65536, dtype=np.uint16).reshape(T, H, D)
    tdt = torch.float16 if src == "f16" else torch.bfloat16
    key = torch.from_numpy(pat.view(np.int16)).view(tdt).to("cuda")
    value = torch.from_numpy(pat[::-1].copy().view(np.int16)).view(tdt).to("cuda")
    NB = T // BS + 1
    kc = torch.full((NB, H, BS, D), 0x55, dtype=torch.int8, device="cuda")
    vc = torch.full_like(kc, 0x55)
    slots = np.random.default_rng(2).permutation(NB * BS)[:T].astype(np.int32)
    s32 = float(np.float32(scale))
    pkv.reshape_and_cache(key, value, kc, vc, torch.from_numpy(slots).to("cuda"), s32, s32)
    torch.cuda.synchronize()
    k0 = np.full((NB, H, BS, D), 0x55, np.uint8)
    ko, vo = oracle.reshape_and_cache(pat, pat[::-1].copy(), k0, k0.copy(), slots, src, "i8", s32, s32)
    assert np.array_equal(kc.cpu().view(torch.uint8).numpy(), ko)
    assert np.array_equal(vc.cpu().view(torch.uint8).numpy(), vo)
