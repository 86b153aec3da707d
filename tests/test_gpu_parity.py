"""GPU parity: the five decode workloads through the C ABI against the oracle.

Each test runs one decode step (copy-on-write copies if any, the cache write
of one new token per sequence, then the decode) on the GPU and in the oracle
from the same generator inputs.  Pools must match bit for bit; outputs must
be within the stated max-abs tolerance (fp32 1e-5, fp16/bf16 2e-3, fp8 KV
3e-2) at every element: on these workloads the output format's own rounding
fits in the tolerance everywhere, which the tests assert too.  Small variants (fewer sequences/heads, the same lengths, so several
partitions and ragged tails) are checked on every sequence; the full-size
workloads, generated on the GPU in the launch configuration the benchmark
times, are checked on sampled sequences plus the whole-pool untouched check.
"""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import (assert_tolerance_budget, check_step, check_untouched, oracle_step, require_gpu, run_gpu_step,
                        sample_seqs, touched)

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[parity] {msg}", flush=True)


SMALL = {1: dict(), 2: dict(), 3: dict(S=6, H=3), 4: dict(S=16, H=2), 5: dict(S=24, H=2), 6: dict(S=24, H=2)}


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5, 6])
def test_small_workload_all_sequences(idx):
    pkv = require_gpu()
    cfg = W.CONFIGS[idx]
    _announce(f"config {idx} small {SMALL[idx]}")
    case = W.make_case(cfg, device="cpu", **SMALL[idx])
    g = run_gpu_step(pkv, case)
    o = oracle_step(case, g.k_pre, g.v_pre)
    err = check_step(case, g, o, f"C{idx}-small")
    assert_tolerance_budget(case, o)
    check_untouched(g, touched(case))
    _announce(f"config {idx} small: max abs err {err:.3g}")


def test_shared_prefix_copy_on_write_on_write():
    pkv = require_gpu()
    _announce("config 4' (append inside the shared block)")
    case = W.make_case(W.CONFIG_4_ON_WRITE, device="cpu", S=64, H=8)
    g = run_gpu_step(pkv, case)
    o = oracle_step(case, g.k_pre, g.v_pre)
    check_step(case, g, o, "C4'")
    check_untouched(g, touched(case))
    # the copy sources still hold the prefix as it was (only seq 7 of each group wrote into one)
    src = torch.as_tensor(case.copy_pairs[:, 0].astype(np.int64), device="cuda")
    dst = torch.as_tensor(case.copy_pairs[:, 1].astype(np.int64), device="cuda")
    written = {int(x) // case.BS: int(x) % case.BS for x in case.slot_mapping}
    ks = g.k_post.index_select(0, src).view(torch.int16)
    kd = g.k_post.index_select(0, dst).view(torch.int16)
    for i in range(src.numel()):
        # copy and source agree on every row except the one each writer appended
        rows = [r for r in range(case.BS) if r != written.get(int(dst[i]), -1) and r != written.get(int(src[i]), -1)]
        assert torch.equal(ks[i][:, rows], kd[i][:, rows])


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5, 6])
def test_full_workload_sampled(idx):
    pkv = require_gpu()
    cfg = W.CONFIGS[idx]
    _announce(f"config {idx} full size, generated on the GPU")
    case = W.make_case(cfg, device="cuda")
    g = run_gpu_step(pkv, case)
    seqs = sample_seqs(case, 8 if idx in (3, 5, 6) else case.S, seed=idx)
    o = oracle_step(case, g.k_pre, g.v_pre, seqs)
    err = check_step(case, g, o, f"C{idx}-full")
    assert_tolerance_budget(case, o)
    check_untouched(g, touched(case))
    _announce(f"config {idx} full: {len(seqs)} sequences, max abs err {err:.3g}")
    del g, case
    torch.cuda.empty_cache()
