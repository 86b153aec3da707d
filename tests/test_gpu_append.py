"""GPU: the decode that appends the step's tokens itself
(pkv_paged_attention_decode_append).

The fused call must give, bit for bit in the output and in both whole pools,
what the cache write followed by the decode gives on the same inputs; it is
also checked against the oracle.  Cases: every workload shape, contexts on
both sides of the 2048-token partition boundaries (the writing workgroup is
then partition 0, 1 or 2 and the merge runs), padding sequences, the two-phase
form, and the host-side checks.
"""

import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import GpuStep, check_step, oracle_step, require_gpu

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _device_case(case):
    return case if case.k_cache.device.type == "cuda" else case.to("cuda")


def _pools(pkv, c, case):
    """Fresh copies of the pre-step pools, with the step's block copies applied."""
    kc, vc = c.k_cache.clone(), c.v_cache.clone()
    if case.copy_pairs.shape[0]:
        pkv.copy_blocks(kc, vc, torch.from_numpy(case.copy_pairs).cuda())
    return kc, vc


def run_separate(pkv, case, lens, slots):
    c = _device_case(case)
    kc, vc = _pools(pkv, c, case)
    bt = torch.from_numpy(case.block_tables).cuda()
    pkv.reshape_and_cache(c.key, c.value, kc, vc, torch.from_numpy(slots).cuda(), case.k_scale, case.v_scale)
    out = torch.full_like(c.q, float("nan"))
    pkv.paged_attention_decode(out, c.q, kc, vc, bt, torch.from_numpy(lens).cuda(), case.scale, case.k_scale,
                               case.v_scale)
    torch.cuda.synchronize()
    return kc, vc, out


def run_append(pkv, case, lens, slots, two_phase=False):
    c = _device_case(case)
    kc, vc = _pools(pkv, c, case)
    bt = torch.from_numpy(case.block_tables).cuda()
    cl = torch.from_numpy(lens).cuda()
    sl = torch.from_numpy(slots).cuda()
    out = torch.full_like(c.q, float("nan"))
    if two_phase:
        ws = pkv.alloc_decode_workspace(case.S, case.H, case.D, case.BS, case.MB)
        pkv.paged_attention_decode_append_partitions(out, c.q, c.key, c.value, kc, vc, sl, bt, cl, case.scale,
                                                     case.k_scale, case.v_scale, workspace=ws)
        pkv.paged_attention_decode_merge(out, cl, case.BS, case.MB, kc.dtype, case.v_scale, workspace=ws)
    else:
        pkv.paged_attention_decode_append(out, c.q, c.key, c.value, kc, vc, sl, bt, cl, case.scale, case.k_scale,
                                          case.v_scale)
    torch.cuda.synchronize()
    return kc, vc, out


def assert_same(case, a, b, label):
    for name, x, y in zip(("K pool", "V pool", "output"), a, b):
        assert torch.equal(_bits(x), _bits(y)), f"{label}: {name} differs between the fused and the separate calls"


SHAPES = [(1, {}), (2, {}), (3, {"S": 16, "H": 8}), (4, {"S": 16, "H": 4}), (5, {"S": 32, "H": 4}),
          (6, {"S": 32, "H": 4})]


@pytest.mark.parametrize("idx,kw", SHAPES, ids=[f"C{i}" for i, _ in SHAPES])
def test_append_equals_cache_write_then_decode(idx, kw):
    pkv = require_gpu()
    case = W.make_case(W.CONFIGS[idx], device="cuda", **kw)
    print(f"[append] C{idx} S={case.S} H={case.H}", flush=True)
    lens, slots = case.context_lens, case.slot_mapping
    assert_same(case, run_append(pkv, case, lens, slots), run_separate(pkv, case, lens, slots), f"C{idx}")


def test_append_into_a_copied_block():
    """Copy-on-write inside the step (the new token lands in the block each
    writer just copied, at offset 4): the fused call equals the copies, the
    cache write and the decode in order."""
    pkv = require_gpu()
    case = W.make_case(W.CONFIG_4_ON_WRITE, device="cuda", S=16, H=4)
    print(f"[append] C4' S={case.S} pairs={case.copy_pairs.shape[0]}", flush=True)
    lens, slots = case.context_lens, case.slot_mapping
    assert_same(case, run_append(pkv, case, lens, slots), run_separate(pkv, case, lens, slots), "C4'")


def test_append_full_size_long_context_bitwise():
    """The Llama2-13B-shaped long-context step at full size, as the benchmark runs it."""
    pkv = require_gpu()
    case = W.make_case(W.CONFIGS[3], device="cuda")
    print(f"[append] C3 full size S={case.S} H={case.H} NB={case.NB}", flush=True)
    lens, slots = case.context_lens, case.slot_mapping
    assert_same(case, run_append(pkv, case, lens, slots), run_separate(pkv, case, lens, slots), "C3 full")


@pytest.mark.parametrize("idx", [2, 5, 6])
def test_append_matches_oracle(idx):
    pkv = require_gpu()
    case = W.make_case(W.CONFIGS[idx], device="cpu", **({"S": 24, "H": 2} if idx != 2 else {}))
    print(f"[append] oracle C{idx} S={case.S} H={case.H}", flush=True)
    c = case.to("cuda")
    k_pre, v_pre = c.k_cache.clone(), c.v_cache.clone()
    kc, vc, out = run_append(pkv, c, case.context_lens, case.slot_mapping)
    g = GpuStep(k_pre, v_pre, kc, vc, out, torch.from_numpy(case.block_tables).cuda(),
                torch.from_numpy(case.context_lens).cuda())
    check_step(case, g, oracle_step(case, k_pre, v_pre), f"append C{idx}")


@pytest.mark.parametrize("idx", [3, 5])
@pytest.mark.parametrize("two_phase", [False, True])
def test_append_partition_boundaries(idx, two_phase):
    """Contexts ending just before, on and after the 2048-token partition
    boundaries: the writing workgroup is partition 0, 1 or 2."""
    pkv = require_gpu()
    BS = W.CONFIGS[idx].BS
    lens = [1, 2, BS - 1, BS, BS + 1, 2047, 2048, 2049, 4095, 4096, 4097, 5000]
    case = W.make_case(W.CONFIGS[idx], device="cpu", H=2, context_lens=lens, seed=idx + 50)
    print(f"[append] boundaries C{idx} two_phase={two_phase} lens={lens}", flush=True)
    c = case.to("cuda")
    k_pre, v_pre = c.k_cache.clone(), c.v_cache.clone()
    fused = run_append(pkv, c, case.context_lens, case.slot_mapping, two_phase=two_phase)
    assert_same(case, fused, run_separate(pkv, c, case.context_lens, case.slot_mapping), f"C{idx} boundaries")
    kc, vc, out = fused
    g = GpuStep(k_pre, v_pre, kc, vc, out, torch.from_numpy(case.block_tables).cuda(),
                torch.from_numpy(case.context_lens).cuda())
    check_step(case, g, oracle_step(case, k_pre, v_pre), f"append C{idx} boundaries")


@pytest.mark.parametrize("idx", [2, 5])
def test_append_padding_sequences(idx):
    """Idle batch slots (slot -1, n = 0) write nothing and give zeros; a
    sequence with n = 0 but a slot still gets its token written, as the cache
    write would."""
    pkv = require_gpu()
    case = W.make_case(W.CONFIGS[idx], device="cuda", **({"S": 16, "H": 4} if idx == 5 else {}))
    lens = case.context_lens.copy()
    slots = case.slot_mapping.copy()
    lens[1::3] = 0
    slots[1::3] = -1
    lens[2] = 0                                   # keeps its slot: written, then a zero output
    print(f"[append] padding C{idx} idle={np.flatnonzero(slots < 0).tolist()}", flush=True)
    fused = run_append(pkv, case, lens, slots)
    assert_same(case, fused, run_separate(pkv, case, lens, slots), f"C{idx} padding")
    out = fused[2]
    assert torch.count_nonzero(out[torch.from_numpy(lens == 0).cuda()].float()) == 0
    blk, off = divmod(int(slots[2]), case.BS)
    assert not torch.equal(_bits(fused[0][blk, :, off]), _bits(case.k_cache[blk, :, off])), \
        "the n = 0 sequence's token was not written"


def test_append_status_codes():
    pkv = require_gpu()
    lib = pkv.lib()
    case = W.make_case(W.CONFIGS[3], device="cuda", H=2, context_lens=[100, 2047, 2049, 4000])
    bt = torch.from_numpy(case.block_tables).cuda()
    cl = torch.from_numpy(case.context_lens).cuda()
    sl = torch.from_numpy(case.slot_mapping).cuda()
    out = torch.empty_like(case.q)
    need = pkv.decode_workspace_bytes(case.S, case.H, case.D, case.BS, case.MB)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    P = ctypes.c_void_p
    key_bytes = case.key.reshape(-1).view(torch.uint8)

    def call(key=case.key.data_ptr(), value=case.value.data_ptr(), slots=sl.data_ptr(), S=case.S, ws_bytes=need):
        return lib.pkv_paged_attention_decode_append(
            P(out.data_ptr()), P(case.q.data_ptr()), P(key), P(value), P(case.k_cache.data_ptr()),
            P(case.v_cache.data_ptr()), P(slots), P(bt.data_ptr()), P(cl.data_ptr()), S, case.H, case.D, case.BS,
            case.MB, case.NB, case.scale, 2, 2, 1.0, 1.0, P(ws.data_ptr()), ws_bytes, None)

    assert call(key=0) == pkv.PKV_ERR_INVALID_ARG
    assert call(value=0) == pkv.PKV_ERR_INVALID_ARG
    assert call(slots=0) == pkv.PKV_ERR_INVALID_ARG
    assert call(key=key_bytes[2:].data_ptr()) == pkv.PKV_ERR_INVALID_ARG          # misaligned
    assert call(ws_bytes=need - 1) == pkv.PKV_ERR_WORKSPACE
    assert call(S=0) == pkv.PKV_OK
    with pytest.raises(ValueError):
        pkv.paged_attention_decode_append(out, case.q, case.key[:2].contiguous(), case.value, case.k_cache,
                                          case.v_cache, sl, bt, cl, case.scale)
    torch.cuda.synchronize()
