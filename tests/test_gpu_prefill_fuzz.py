"""Seeded random prompt steps against the oracle (GPU).

Each case draws a head size, block size, q format, pool format (the q
format, E4M3 or INT8), head count and, per sequence, a number of new tokens
(none, one, around the 32-key tile and the 128-query workgroup tile, or
uniform) and of cached ones (none, or uniform).  One prompt step (copies,
cache write, prompt attention) is checked against the oracle: pools bit for
bit, outputs within the bound derived in test_gpu_prefill.  The same step
through the appending entry point (the cache write inside the prompt kernel
for 16-bit pools) must give the same pools and output bit for bit.
"""

from dataclasses import replace

import numpy as np
import pytest

import workloads as W
from gpu_common import require_gpu
from test_gpu_prefill import check, oracle_run, run_gpu
from test_gpu_prefill_append import assert_same, run_append, run_separate

pytestmark = pytest.mark.gpu


def _draw(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    D = int(rng.choice([64, 80, 96, 128, 256]))
    BS = int(rng.choice([16, 32]))
    dtype = str(rng.choice(["f16", "bf16"]))
    cache = str(rng.choice(["", "e4m3", "i8"]))
    S, H = int(rng.integers(1, 7)), int(rng.integers(1, 4))
    edges = [0, 1, 31, 32, 33, 127, 128, 129, 255, 256, 257]
    q_lens = [int(rng.choice(edges)) if rng.random() < 0.6 else int(rng.integers(1, 400)) for _ in range(S)]
    if sum(q_lens) == 0:
        q_lens[0] = 1
    cached = [0 if rng.random() < 0.4 else int(rng.integers(1, 700)) for _ in range(S)]
    cfg = replace(W.PREFILL_CONFIGS[1], name=f"prefill-fuzz-{seed}", D=D, BS=BS, dtype=dtype, cache_dtype=cache, H=H)
    return cfg, q_lens, cached


@pytest.mark.parametrize("seed", range(16))
def test_random_prompt_steps(seed):
    pkv = require_gpu()
    cfg, q_lens, cached = _draw(5230 + seed)
    print(f"[prefill fuzz {seed}] D={cfg.D} BS={cfg.BS} {cfg.dtype}/{cfg.cache_dtype or cfg.dtype} H={cfg.H} "
          f"q={q_lens} cached={cached}", flush=True)
    case = W.make_prefill_case(cfg, device="cuda", q_lens=q_lens, cached=cached, seed=5230 + seed)
    k_pre, v_pre, gk, gv, gout = run_gpu(pkv, case)
    err = check(case, gk, gv, gout, oracle_run(case, k_pre, v_pre), f"prefill fuzz {seed}")
    print(f"[prefill fuzz {seed}] max abs error {err:.3g}", flush=True)
    case.k_cache.copy_(k_pre)                  # both forms from the pre-step pools
    case.v_cache.copy_(v_pre)
    assert_same(run_append(pkv, case), run_separate(pkv, case), f"prefill fuzz {seed}")
