"""The decode over the library's static workspace (pkv_paged_attention_decode_
static, for callers that cannot allocate) against pkv_paged_attention_decode
with a caller workspace, through the C ABI (GPU).

Both run the same kernels on the same inputs, so their outputs must agree
bit for bit.  Two calls in a row share the GPU's one static buffer: a larger
step first, then a smaller one, both with contexts over several partitions
so that the partials in the buffer are written and read; the second call
must not see anything of the first.  A third call over a step whose contexts
fit one partition uses no partials at all.
"""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import require_gpu

pytestmark = pytest.mark.gpu


def _inputs(case):
    dev = "cuda"
    c = case.to(dev)
    slots = torch.from_numpy(case.slot_mapping).to(dev)
    bt = torch.from_numpy(case.block_tables).to(dev)
    cl = torch.from_numpy(case.context_lens).to(dev)
    return c, slots, bt, cl


def _compare(pkv, case, label):
    c, slots, bt, cl = _inputs(case)
    pkv.reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, slots, case.k_scale, case.v_scale)
    need = pkv.decode_workspace_bytes(case.S, case.H, case.D, case.BS, case.MB)
    assert need <= pkv.STATIC_WORKSPACE_BYTES
    ws = pkv.alloc_decode_workspace(case.S, case.H, case.D, case.BS, case.MB)
    want = torch.full_like(c.q, float("nan"))
    pkv.paged_attention_decode(want, c.q, c.k_cache, c.v_cache, bt, cl, case.scale, case.k_scale, case.v_scale,
                               workspace=ws)
    got = torch.full_like(c.q, float("nan"))
    pkv.paged_attention_decode_static(got, c.q, c.k_cache, c.v_cache, bt, cl, case.scale, case.k_scale, case.v_scale)
    torch.cuda.synchronize()
    assert torch.isfinite(got.float()).all(), f"{label}: non-finite output"
    assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"{label}: differs from the workspace decode"
    print(f"[no-alloc] {label}: S={case.S} H={case.H} partials {need} B, bitwise equal", flush=True)
    return need


def test_static_workspace_decode_matches_two_calls_in_a_row():
    pkv = require_gpu()
    # 1: the fp8 workload's shape on 96 sequences x 8 heads, contexts up to
    #    4096 tokens (two partitions)
    big = W.make_case(W.CONFIGS[5], device="cpu", S=96, H=8)
    assert int(big.context_lens.max()) > 2048
    need1 = _compare(pkv, big, "fp8 KV, 96 x 8")
    # 2: smaller: bf16, 6 sequences x 3 heads with contexts across one to
    #    four partitions
    from dataclasses import replace
    cfg = replace(W.CONFIGS[3], name="no-alloc-small", MB=512)
    small = W.make_case(cfg, device="cpu", H=3, context_lens=[1, 2047, 2049, 4100, 6000, 8192])
    need2 = _compare(pkv, small, "bf16, 6 x 3")
    assert 0 < need2 < need1
    # 3: every context fits one partition: no partials
    tiny = W.make_case(W.CONFIGS[2], device="cpu", S=4, H=2)
    assert _compare(pkv, tiny, "f16, one partition") == 0
