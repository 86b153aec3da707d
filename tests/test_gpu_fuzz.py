"""Seeded random decode steps against the oracle (GPU).

Each case draws a head size, block size, format pair, sequence and head
count and a mix of context lengths: one token, whole blocks and one token
either side, partition boundaries (2048 tokens) and one token either side,
and uniform lengths, in a table with spare width.  One decode step (cache
write, then the decode) is checked against the oracle: pools bit for bit,
outputs within the format's tolerance.  The decode that appends the step's
tokens itself must give the same pools and output bit for bit.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import check_step, oracle_step, require_gpu, run_gpu_step

pytestmark = pytest.mark.gpu

PAIRS = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f16", "e4m3"), ("bf16", "e4m3"), ("f16", "i8"),
         ("bf16", "i8")]
PART = 2048


def _draw(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    D = int(rng.choice([64, 80, 96, 128, 256]))
    BS = int(rng.choice([16, 32]))
    qd, cd = PAIRS[int(rng.integers(len(PAIRS)))]
    S, H = int(rng.integers(1, 9)), int(rng.integers(1, 5))
    pool = [1, BS, BS + 1, 2 * BS - 1, PART - 1, PART, PART + 1, 2 * PART + 1]
    lens = [int(rng.choice(pool)) if rng.random() < 0.6 else int(rng.integers(1, 3 * PART)) for _ in range(S)]
    MB = -(-max(lens) // BS) + int(rng.integers(0, 4))
    scales = dict(scale_lo=0.03, scale_hi=0.05) if cd in ("e4m3", "i8") else {}
    cfg = replace(W.CONFIGS[1], name=f"fuzz-{seed}", D=D, BS=BS, q_dtype=qd, cache_dtype=cd, MB=MB, NB_fixed=None,
                  **scales)
    return cfg, S, H, lens


@pytest.mark.parametrize("seed", range(24))
def test_random_decode_steps(seed):
    pkv = require_gpu()
    cfg, S, H, lens = _draw(4230 + seed)
    print(f"[fuzz {seed}] D={cfg.D} BS={cfg.BS} {cfg.q_dtype}/{cfg.cache_dtype} S={S} H={H} MB={cfg.MB} "
          f"lens={lens}", flush=True)
    case = W.make_case(cfg, device="cpu", S=S, H=H, context_lens=lens, seed=4230 + seed)
    g = run_gpu_step(pkv, case)
    o = oracle_step(case, g.k_pre, g.v_pre)
    check_step(case, g, o, f"fuzz {seed}")
    kc, vc = g.k_pre.clone(), g.v_pre.clone()
    c = case.to("cuda")
    out = torch.empty_like(c.q)
    ws = pkv.alloc_decode_workspace(case.S, case.H, case.D, case.BS, case.MB)
    pkv.paged_attention_decode_append(out, c.q, c.key, c.value, kc, vc, torch.from_numpy(case.slot_mapping).cuda(),
                                      g.block_tables, g.context_lens, case.scale, case.k_scale, case.v_scale,
                                      workspace=ws)
    torch.cuda.synchronize()
    for name, x, y in (("K pool", kc, g.k_post), ("V pool", vc, g.v_post), ("output", out, g.out)):
        assert torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8)), \
            f"fuzz {seed}: appending decode's {name} differs from the separate calls"
