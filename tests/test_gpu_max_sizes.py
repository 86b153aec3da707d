"""GPU: the largest shapes the entry points accept.

* 65,535 sequences, the grid limit of the decode (one workgroup row per
  sequence), through the cache write, the decode, the appending decode and
  the grouped appending decode;
* one 32,768-token context next to short ones: 16 partitions merged;
* a 4,096-token prompt after a cached prefix of 1,000 tokens (32 query tiles
  of 128), through the prompt attention and the prompt step in one pass.

Outputs are compared with the oracle on a sample of sequences (the first,
the last and a spread in between), pools bit for bit on the blocks those
sequences map; the fused forms must equal the separate calls bit for bit.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import check_step, oracle_step, require_gpu, run_gpu_step

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.uint8)


def test_decode_at_the_sequence_grid_limit():
    pkv = require_gpu()
    S = 65535
    rng = np.random.default_rng(65535)
    lens = rng.integers(1, 40, size=S).tolist()
    cfg = replace(W.CONFIGS[1], NB_fixed=None)       # a pool sized for the batch
    case = W.make_case(cfg, device="cpu", H=1, context_lens=lens, seed=5)
    print(f"[max] decode S={case.S} NB={case.NB}", flush=True)
    g = run_gpu_step(pkv, case)
    seqs = sorted({0, 1, S // 3, S // 2, S - 2, S - 1} | set(rng.integers(0, S, size=40).tolist()))
    check_step(case, g, oracle_step(case, g.k_pre, g.v_pre, seqs), f"S={S}")
    assert torch.isfinite(g.out.float()).all()
    # the appending decode from the same pre-step pools
    kc, vc = g.k_pre.clone(), g.v_pre.clone()
    c = case.to("cuda")
    out = torch.empty_like(c.q)
    pkv.paged_attention_decode_append(out, c.q, c.key, c.value, kc, vc, torch.from_numpy(case.slot_mapping).cuda(),
                                      g.block_tables, g.context_lens, case.scale)
    torch.cuda.synchronize()
    for name, x, y in (("K pool", kc, g.k_post), ("V pool", vc, g.v_post), ("output", out, g.out)):
        assert torch.equal(_bits(x), _bits(y)), f"S={S}: appending decode's {name} differs"
    # the grouped appending decode over the whole batch (its grid's last
    # dimension: ceil(S / group size) groups times the chunks of a group)
    for gs in (3, 8):
        kc, vc = g.k_pre.clone(), g.v_pre.clone()
        out = torch.empty_like(c.q)
        pkv.paged_attention_decode_grouped(out, c.q, kc, vc, g.block_tables, g.context_lens, case.scale, gs,
                                           key=c.key, value=c.value,
                                           slot_mapping=torch.from_numpy(case.slot_mapping).cuda())
        torch.cuda.synchronize()
        for name, x, y in (("K pool", kc, g.k_post), ("V pool", vc, g.v_post), ("output", out, g.out)):
            assert torch.equal(_bits(x), _bits(y)), f"S={S}: grouped decode's {name} differs (groups of {gs})"


def test_decode_long_context_many_partitions():
    pkv = require_gpu()
    lens = [32768, 1, 2048, 2049, 10000, 16]
    case = W.make_case(W.CONFIGS[3], device="cpu", H=2, context_lens=lens, seed=32768)
    print(f"[max] decode lens={lens} MB={case.MB} (partitions of 2048 tokens)", flush=True)
    g = run_gpu_step(pkv, case)
    err = check_step(case, g, oracle_step(case, g.k_pre, g.v_pre), "32k context")
    print(f"[max] 32k context: max abs error {err:.3g}", flush=True)
    kc, vc = g.k_pre.clone(), g.v_pre.clone()
    c = case.to("cuda")
    out = torch.empty_like(c.q)
    pkv.paged_attention_decode_append(out, c.q, c.key, c.value, kc, vc, torch.from_numpy(case.slot_mapping).cuda(),
                                      g.block_tables, g.context_lens, case.scale)
    torch.cuda.synchronize()
    for name, x, y in (("K pool", kc, g.k_post), ("V pool", vc, g.v_post), ("output", out, g.out)):
        assert torch.equal(_bits(x), _bits(y)), f"32k context: appending decode's {name} differs"


def test_prefill_long_prompt_after_cached_prefix():
    pkv = require_gpu()
    from test_gpu_prefill import check, oracle_run, run_gpu
    cfg = replace(W.PREFILL_CONFIGS[1], D=128, BS=16, dtype="bf16", H=2)
    q_lens, cached = [4096, 7, 300], [1000, 4000, 0]
    case = W.make_prefill_case(cfg, device="cuda", q_lens=q_lens, cached=cached, seed=4096)
    print(f"[max] prompt q_lens={q_lens} cached={cached} max_q_len={case.max_q_len}", flush=True)
    k_pre, v_pre, gk, gv, gout = run_gpu(pkv, case)
    err = check(case, gk, gv, gout, oracle_run(case, k_pre, v_pre), "4096-token prompt")
    print(f"[max] 4096-token prompt: max abs error {err:.3g}", flush=True)
    # the prompt step in one pass, from the same pre-step pools
    kc, vc = k_pre.clone(), v_pre.clone()
    out = torch.full_like(case.q, float("nan"))
    pkv.paged_attention_prefill_append(out, case.q, case.key, case.value, kc, vc,
                                       torch.from_numpy(case.slot_mapping).cuda(),
                                       torch.from_numpy(case.block_tables).cuda(),
                                       torch.from_numpy(case.context_lens).cuda(),
                                       torch.from_numpy(case.cu_q_lens).cuda(), case.max_q_len, case.scale)
    torch.cuda.synchronize()
    for name, x, y in (("K pool", kc, gk), ("V pool", vc, gv), ("output", out, gout)):
        assert torch.equal(_bits(x), _bits(y)), f"4096-token prompt: prompt step in one pass, {name} differs"
