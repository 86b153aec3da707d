"""GPU parity over the supported head sizes, block sizes and formats.

Head sizes 64, 80, 96, 128 and 256 with block sizes 16 and 32, for every
(query, cache) format pair, through one decode step (cache write, then the
decode) against the oracle: pools bit for bit, outputs within the format's
tolerance.  The lengths cross a block, the decode's sub-tiles of a block and
its 2048-token partitions.  80 and 96 leave lanes of a row idle in the
decode; 256 splits each block into several register stages.  The decode that
appends the step's tokens itself must match the separate calls bit for bit on
every one of these shapes.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_common import check_step, oracle_step, require_gpu, run_gpu_step

pytestmark = pytest.mark.gpu

PAIRS = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f16", "e4m3"), ("bf16", "i8")]


def _cfg(D, BS, qd, cd):
    scales = dict(scale_lo=0.03, scale_hi=0.05) if cd in ("e4m3", "i8") else {}
    return replace(W.CONFIGS[1], name=f"shape-D{D}-BS{BS}-{qd}-{cd}", D=D, BS=BS, q_dtype=qd, cache_dtype=cd,
                   MB=140, NB_fixed=None, **scales)


@pytest.mark.parametrize("D", [64, 80, 96, 128, 256])
@pytest.mark.parametrize("BS", [16, 32])
@pytest.mark.parametrize("qd,cd", PAIRS)
def test_decode_head_and_block_sizes(D, BS, qd, cd):
    pkv = require_gpu()
    cfg = _cfg(D, BS, qd, cd)
    part = 2048                                # tokens per decode partition
    lens = [1, BS - 1, BS + 1, 3 * BS + 5, part + 1, 2 * part + BS - 3]
    print(f"[shapes] D={D} BS={BS} {qd}/{cd} lens={lens}", flush=True)
    case = W.make_case(cfg, device="cpu", H=3, context_lens=lens, seed=D + BS)
    g = run_gpu_step(pkv, case)
    o = oracle_step(case, g.k_pre, g.v_pre)
    check_step(case, g, o, f"D{D} BS{BS} {qd}/{cd}")
    # the same step through the appending decode, from the same pre-step pools
    kc, vc = g.k_pre.clone(), g.v_pre.clone()
    c = case.to("cuda")
    out = torch.empty_like(c.q)
    pkv.paged_attention_decode_append(out, c.q, c.key, c.value, kc, vc, torch.from_numpy(case.slot_mapping).cuda(),
                                      g.block_tables, g.context_lens, case.scale, case.k_scale, case.v_scale)
    torch.cuda.synchronize()
    for name, x, y in (("K pool", kc, g.k_post), ("V pool", vc, g.v_post), ("output", out, g.out)):
        assert torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8)), \
            f"D{D} BS{BS} {qd}/{cd}: appending decode's {name} differs from the separate calls"


@pytest.mark.parametrize("D", [80, 96, 256])
def test_gather_kv_head_sizes_bitwise(D):
    pkv = require_gpu()
    cfg = _cfg(D, 16, "bf16", "bf16")
    case = W.make_case(cfg, device="cpu", H=2, context_lens=[5, 33, 70], seed=D)
    g = run_gpu_step(pkv, case)
    total = int(case.context_lens.sum())
    ko = torch.empty((total, case.H, case.D), dtype=g.k_post.dtype, device="cuda")
    vo = torch.empty_like(ko)
    cu = np.zeros(case.S + 1, dtype=np.int32)
    cu[1:] = np.cumsum(case.context_lens)
    pkv.gather_kv(ko, vo, torch.from_numpy(cu).to("cuda"), g.k_post, g.v_post, g.block_tables, g.context_lens)
    torch.cuda.synchronize()
    kb, vb = W.bits(g.k_post, "bf16"), W.bits(g.v_post, "bf16")
    ke, ve, _ = oracle.gather_kv(kb, vb, case.block_tables, case.context_lens)
    assert np.array_equal(W.bits(ko, "bf16"), ke) and np.array_equal(W.bits(vo, "bf16"), ve)
