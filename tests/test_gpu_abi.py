"""Status codes of the C ABI with real device buffers (GPU).

Every call returns before enqueueing anything when its host-side checks fail,
and an in-range call on the null stream and on a side stream both work.
"""

import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import require_gpu

pytestmark = pytest.mark.gpu


def _args(case):
    dev = "cuda"
    c = case.to(dev)
    return c, torch.from_numpy(case.block_tables).to(dev), torch.from_numpy(case.context_lens).to(dev)


def test_decode_status_codes():
    pkv = require_gpu()
    lib = pkv.lib()
    # contexts past one 2048-token partition, so the decode needs a workspace
    case = W.make_case(W.CONFIGS[3], device="cpu", H=2, context_lens=[100, 2047, 2049, 4000])
    c, bt, cl = _args(case)
    out = torch.empty_like(c.q)
    need = pkv.decode_workspace_bytes(c.S, c.H, c.D, c.BS, c.MB)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    P = ctypes.c_void_p

    def call(ws_ptr=ws.data_ptr(), ws_bytes=need, S=c.S, D=c.D, BS=c.BS, scale=c.scale, qd=2, cd=2, out_ptr=None):
        return lib.pkv_paged_attention_decode(P(out.data_ptr() if out_ptr is None else out_ptr), P(c.q.data_ptr()),
                                              P(c.k_cache.data_ptr()), P(c.v_cache.data_ptr()), P(bt.data_ptr()),
                                              P(cl.data_ptr()), S, c.H, D, BS, c.MB, c.NB, scale, qd, cd, 1.0, 1.0,
                                              P(ws_ptr), ws_bytes, None)

    assert call() == pkv.PKV_OK
    torch.cuda.synchronize()
    assert call(ws_bytes=need - 1) == pkv.PKV_ERR_WORKSPACE
    assert call(ws_ptr=0) == pkv.PKV_ERR_WORKSPACE
    assert call(S=-1) == pkv.PKV_ERR_INVALID_ARG
    assert call(S=0) == pkv.PKV_OK
    assert call(D=72) == pkv.PKV_ERR_UNSUPPORTED
    assert call(BS=8) == pkv.PKV_ERR_UNSUPPORTED
    assert call(qd=0, cd=2) == pkv.PKV_ERR_UNSUPPORTED
    assert call(cd=7) == pkv.PKV_ERR_INVALID_ARG
    assert call(scale=float("nan")) == pkv.PKV_ERR_INVALID_ARG
    assert call(scale=0.0) == pkv.PKV_ERR_INVALID_ARG
    assert call(out_ptr=0) == pkv.PKV_ERR_INVALID_ARG
    torch.cuda.synchronize()


def test_binding_raises_and_side_stream():
    pkv = require_gpu()
    case = W.make_case(W.CONFIGS[2], device="cpu", S=4, H=2)
    c, bt, cl = _args(case)
    out = torch.empty_like(c.q)
    with pytest.raises(pkv.PagedKVError) as ei:
        pkv.paged_attention_decode(out, c.q, c.k_cache, c.v_cache, bt, cl, float("inf"))
    assert ei.value.status == pkv.PKV_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        pkv.paged_attention_decode(out, c.q.cpu(), c.k_cache, c.v_cache, bt, cl, c.scale)
    ref = pkv.paged_attention_decode(torch.empty_like(c.q), c.q, c.k_cache, c.v_cache, bt, cl, c.scale)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = pkv.paged_attention_decode(torch.empty_like(c.q), c.q, c.k_cache, c.v_cache, bt, cl, c.scale)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))


def test_cache_ops_status_codes():
    pkv = require_gpu()
    lib = pkv.lib()
    case = W.make_case(W.CONFIGS[5], device="cpu", S=4, H=2)
    c, bt, cl = _args(case)
    P = ctypes.c_void_p
    slots = torch.from_numpy(case.slot_mapping).to("cuda")
    args = [P(c.key.data_ptr()), P(c.value.data_ptr()), P(c.k_cache.data_ptr()), P(c.v_cache.data_ptr()),
            P(slots.data_ptr()), c.S, c.H, c.D, c.BS, c.NB, 1, 3]
    assert lib.pkv_reshape_and_cache(*args, 0.05, 0.05, None) == pkv.PKV_OK
    assert lib.pkv_reshape_and_cache(*args, -0.05, 0.05, None) == pkv.PKV_ERR_INVALID_ARG
    assert lib.pkv_reshape_and_cache(*args[:-2], 0, 3, 0.05, 0.05, None) == pkv.PKV_ERR_UNSUPPORTED
    a2 = list(args)
    a2[5] = 0
    assert lib.pkv_reshape_and_cache(*a2, 0.05, 0.05, None) == pkv.PKV_OK
    pairs = torch.tensor([[1, 2]], dtype=torch.int32, device="cuda")
    assert lib.pkv_copy_blocks(P(c.k_cache.data_ptr()), P(c.v_cache.data_ptr()), P(pairs.data_ptr()), 0,
                               c.H, c.D, c.BS, c.NB, 3, None) == pkv.PKV_OK
    assert lib.pkv_copy_blocks(P(c.k_cache.data_ptr()), P(c.v_cache.data_ptr()), P(0), 1,
                               c.H, c.D, c.BS, c.NB, 3, None) == pkv.PKV_ERR_INVALID_ARG
    torch.cuda.synchronize()


@pytest.mark.parametrize("idx", [3, 5, 6])
def test_two_phase_decode_equals_decode(idx):
    pkv = require_gpu()
    # lengths on both sides of the 2048-token partition boundary
    lens = [W.CONFIGS[idx].BS, 2047, 2048, 2049, 3000, 4096, 300, 2500]
    case = W.make_case(W.CONFIGS[idx], device="cpu", H=2, context_lens=lens)
    c, bt, cl = _args(case)
    pkv.reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, torch.from_numpy(case.slot_mapping).cuda(),
                          case.k_scale, case.v_scale)
    ref = pkv.paged_attention_decode(torch.empty_like(c.q), c.q, c.k_cache, c.v_cache, bt, cl, case.scale,
                                     case.k_scale, case.v_scale)
    ws = pkv.alloc_decode_workspace(case.S, case.H, case.D, case.BS, case.MB)
    assert ws is not None
    out = torch.empty_like(c.q)
    pkv.paged_attention_decode_partitions(out, c.q, c.k_cache, c.v_cache, bt, cl, case.scale, case.k_scale,
                                          case.v_scale, workspace=ws)
    pkv.paged_attention_decode_merge(out, cl, case.BS, case.MB, c.k_cache.dtype, case.v_scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), out.view(torch.int16))
