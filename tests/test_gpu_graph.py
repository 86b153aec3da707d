"""GPU: the decode step captured into a HIP graph (pkv_decode_graph_*).

A replay must give bit for bit what the eager calls give on the same
buffer contents.  Every test replays the graph several times, with new
contents written into the fixed buffers and other eager work (and
synchronisations) between replays, and checks every replay; one replay is
also checked against the oracle.
"""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import GpuStep, check_step, oracle_step, require_gpu

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.uint8) if t.dtype != torch.uint8 else t


class Buffers:
    """Fixed device buffers of one decode step of ``case``."""

    def __init__(self, case: W.Case):
        dev = "cuda"
        self.key = case.key.to(dev).clone()
        self.value = case.value.to(dev).clone()
        self.q = case.q.to(dev).clone()
        self.slots = torch.from_numpy(case.slot_mapping).to(dev)
        self.tables = torch.from_numpy(case.block_tables).to(dev)
        self.lens = torch.from_numpy(case.context_lens).to(dev)
        self.pairs = torch.from_numpy(case.copy_pairs).to(dev) if case.copy_pairs.shape[0] else None


def eager_step(pkv, case, b: Buffers, kc, vc, out):
    if b.pairs is not None:
        pkv.copy_blocks(kc, vc, b.pairs)
    pkv.reshape_and_cache(b.key, b.value, kc, vc, b.slots, case.k_scale, case.v_scale)
    pkv.paged_attention_decode(out, b.q, kc, vc, b.tables, b.lens, case.scale, case.k_scale, case.v_scale)


def next_contents(case, b: Buffers, gen, step):
    """New token values and queries; some sequences drop out of the batch
    (slot -1, length 0) and come back, so replays see changing contents."""
    for t in (b.key, b.value, b.q):
        t.copy_(torch.randn(t.shape, generator=gen, device="cuda", dtype=torch.float32).to(t.dtype))
    lens = torch.from_numpy(case.context_lens).cuda()
    slots = torch.from_numpy(case.slot_mapping).cuda()
    idle = torch.zeros(case.S, dtype=torch.bool, device="cuda")
    idle[step % 3::3] = True
    b.lens.copy_(torch.where(idle, torch.zeros_like(lens), lens))
    b.slots.copy_(torch.where(idle, torch.full_like(slots, -1), slots))


@pytest.mark.parametrize("append", [False, True], ids=["separate-write", "append"])
@pytest.mark.parametrize("idx", [1, 2, 4, 5])
def test_graph_replays_match_eager(idx, append):
    """Every replay equals the eager separate calls bit for bit, whether the
    graph records them as such or as the decode that appends the tokens."""
    pkv = require_gpu()
    cfg = W.CONFIGS[idx]
    case = W.make_case(cfg, device="cuda", **({"S": 32} if idx == 5 else {}))
    print(f"[graph] config {idx}: S={case.S} append={append}", flush=True)
    b = Buffers(case)
    kc_e, vc_e = case.k_cache.clone(), case.v_cache.clone()
    kc_g, vc_g = case.k_cache.clone(), case.v_cache.clone()
    out_e = torch.empty_like(b.q)
    out_g = torch.empty_like(b.q)
    g = pkv.DecodeGraph(kc_g, vc_g, b.key, b.value, b.slots, b.q, out_g, b.tables, b.lens, case.scale,
                        case.k_scale, case.v_scale, copy_pairs=b.pairs, append=append)
    gen = torch.Generator(device="cuda").manual_seed(idx)
    scratch = torch.zeros(1 << 20, device="cuda")
    for step in range(4):
        if step:
            next_contents(case, b, gen, step)
        eager_step(pkv, case, b, kc_e, vc_e, out_e)
        scratch.add_(1.0)                        # unrelated eager work between the two
        g.launch()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out_e), _bits(out_g)), f"replay {step}: output differs from the eager step"
        assert torch.equal(_bits(kc_e), _bits(kc_g)) and torch.equal(_bits(vc_e), _bits(vc_g)), \
            f"replay {step}: pools differ from the eager step"
        if step:
            idle = b.lens == 0
            assert torch.count_nonzero(out_g[idle].float()) == 0, "an idle batch slot got a nonzero output"
    g.destroy()


def test_graph_replay_matches_oracle():
    pkv = require_gpu()
    case = W.make_case(W.CONFIGS[2], device="cpu")
    b = Buffers(case)
    kc, vc = case.k_cache.cuda(), case.v_cache.cuda()
    k_pre, v_pre = kc.clone(), vc.clone()
    out = torch.empty_like(b.q)
    g = pkv.DecodeGraph(kc, vc, b.key, b.value, b.slots, b.q, out, b.tables, b.lens, case.scale)
    g.launch()
    torch.cuda.synchronize()
    o = oracle_step(case, k_pre, v_pre)
    err = check_step(case, GpuStep(k_pre, v_pre, kc, vc, out, b.tables, b.lens), o, "graph C2")
    print(f"[graph] C2 replay vs oracle: max abs err {err:.3g}", flush=True)
    g.destroy()


def test_graph_padded_batch_equals_smaller_eager_batch():
    """A graph captured for 16 batch slots with 10 live sequences gives the
    10-sequence eager result bit for bit and zeros in the idle slots."""
    pkv = require_gpu()
    case = W.make_case(W.CONFIGS[2], device="cuda")
    live = 10
    b = Buffers(case)
    b.slots[live:] = -1
    b.lens[live:] = 0
    kc_g, vc_g = case.k_cache.clone(), case.v_cache.clone()
    out_g = torch.full_like(b.q, float("nan"))
    g = pkv.DecodeGraph(kc_g, vc_g, b.key, b.value, b.slots, b.q, out_g, b.tables, b.lens, case.scale)
    for _ in range(3):
        g.launch()
        torch.cuda.synchronize()
    kc_e, vc_e = case.k_cache.clone(), case.v_cache.clone()
    out_e = torch.empty_like(b.q[:live])
    # the eager batch rewrites the same tokens once; the graph rewrote them thrice with the same values
    pkv.reshape_and_cache(b.key[:live].contiguous(), b.value[:live].contiguous(), kc_e, vc_e,
                          b.slots[:live].contiguous())
    pkv.paged_attention_decode(out_e, b.q[:live].contiguous(), kc_e, vc_e, b.tables[:live].contiguous(),
                               b.lens[:live].contiguous(), case.scale)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out_e), _bits(out_g[:live].contiguous()))
    assert torch.count_nonzero(out_g[live:].float()) == 0
    assert torch.equal(_bits(kc_e), _bits(kc_g)) and torch.equal(_bits(vc_e), _bits(vc_g))
    g.destroy()


def test_graph_create_checks():
    pkv = require_gpu()
    case = W.make_case(W.CONFIGS[1], device="cuda")
    b = Buffers(case)
    out = torch.empty_like(b.q)
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.DecodeGraph(case.k_cache, case.v_cache, b.key, b.value, b.slots, b.q, out, b.tables, b.lens,
                        float("inf"))
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    # a 72-dim head is outside the supported set
    q72 = torch.zeros((case.S, case.H, 72), dtype=torch.float32, device="cuda")
    kc72 = torch.zeros((case.NB, case.H, case.BS, 72), dtype=torch.float32, device="cuda")
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.DecodeGraph(kc72, kc72.clone(), q72, q72.clone(), b.slots, q72.clone(), q72.clone(), b.tables, b.lens,
                        case.scale)
    assert e.value.status == pkv.PKV_ERR_UNSUPPORTED
    # a workspace that is too small (tables wide enough to need one)
    wide = torch.zeros((case.S, 256), dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.DecodeGraph(case.k_cache, case.v_cache, b.key, b.value, b.slots, b.q, out, wide, b.lens, case.scale,
                        workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == pkv.PKV_ERR_WORKSPACE
