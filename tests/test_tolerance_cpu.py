"""CPU checks of the decode parity bound used by the GPU tests.

* half_ulp agrees with the formats' own spacing (NumPy float16 / float32,
  torch bfloat16) at normal and subnormal magnitudes.
* The bound is exactly the stated tolerance wherever the output format's
  half-ulp is at most half of it (bf16: every |out| < 0.5; fp16 and fp32:
  every magnitude the workloads produce).
* The exact result rounded to the output format, the best any kernel can
  return, passes the bound on short bf16 contexts, where |out| reaches 1 to 4.
"""

import numpy as np
import torch

import oracle
import workloads as W
from gpu_common import TOL, decode_bound, fp32_error_bound, half_ulp


def test_half_ulp_matches_the_formats_spacing():
    x = np.concatenate([np.logspace(-12, 4, 400), [2.0 ** -14, 2.0 ** -20, 1.0, 0.5, 3.999]])
    f16 = x[x < 60000.0].astype(np.float16)
    assert np.array_equal(half_ulp(f16.astype(np.float64), "f16"), np.spacing(f16).astype(np.float64) / 2)
    f32 = x.astype(np.float32)
    assert np.array_equal(half_ulp(f32.astype(np.float64), "f32"), np.spacing(f32).astype(np.float64) / 2)
    b = torch.tensor(x, dtype=torch.float64).to(torch.bfloat16)
    nxt = (b.view(torch.int16) + 1).view(torch.bfloat16)           # the next bf16 above each value
    assert torch.equal(nxt.double() - b.double(), 2 * torch.from_numpy(half_ulp(b.double().numpy(), "bf16")))


def _short_case(fmt_q, fmt_c):
    from dataclasses import replace
    cfg = replace(W.CONFIGS[1], name="bound", D=128, q_dtype=fmt_q, cache_dtype=fmt_c, MB=8, NB_fixed=None)
    return W.make_case(cfg, device="cpu", H=4, context_lens=[1, 2, 3, 5, 16, 17, 40, 100])


def _oracle(case):
    kb, vb = oracle.reshape_and_cache(W.bits(case.key, case.q_dtype), W.bits(case.value, case.q_dtype),
                                      W.bits(case.k_cache, case.cache_dtype), W.bits(case.v_cache, case.cache_dtype),
                                      case.slot_mapping, case.q_dtype, case.cache_dtype, case.k_scale, case.v_scale)
    q = W.bits(case.q, case.q_dtype)
    out = oracle.paged_attention_decode(q, kb, vb, case.block_tables, case.context_lens, case.scale, case.q_dtype,
                                        case.cache_dtype, case.k_scale, case.v_scale)
    err = fp32_error_bound(case, q, kb, vb, case.block_tables, case.context_lens)
    return out, err


def test_bound_is_the_tolerance_where_rounding_leaves_room():
    case = _short_case("bf16", "bf16")
    want, err = _oracle(case)
    bound = decode_bound(case, want, err)
    small = np.abs(want) < 0.5
    assert small.any() and (~small).any()
    assert (bound[small] == TOL["bf16"]).all()
    assert (bound[~small] >= TOL["bf16"]).all()
    # the fp32 term is a small fraction of the tolerance on these inputs
    assert 0 < err.max() < 1e-3
    case16 = _short_case("f16", "f16")
    want16, err16 = _oracle(case16)
    assert (decode_bound(case16, want16, err16) == TOL["f16"]).all()
    case32 = _short_case("f32", "f32")
    want32, err32 = _oracle(case32)
    assert (decode_bound(case32, want32, err32) == TOL["f32"]).all()


def test_correctly_rounded_output_passes():
    case = _short_case("bf16", "bf16")
    want, err = _oracle(case)
    got = torch.from_numpy(want).to(torch.bfloat16).double().numpy()
    assert (np.abs(got - want) <= decode_bound(case, want, err)).all()
    # rounding alone exceeds 2e-3 somewhere: the allowance is needed there
    assert (np.abs(got - want) > TOL["bf16"]).any()
