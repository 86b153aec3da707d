"""GPU parity of pkv_check_step_inputs with the oracle's validator.

The mask is integer work, so it must equal the oracle's bit for bit:

* on every decode workload's real index inputs at full size (the pools are
  not needed: only the tables, lengths, slots and copy pairs are checked),
  and on the prompt workloads' (one slot per new token): mask 0;
* on the copy-on-write variant, the tables before the copy (the write lands
  in a block eight sequences map) and after it;
* on single planted faults and on 300 seeded random small steps with and
  without faults, in both modes;
* on full-size workloads with faults planted at random positions (so that
  the entries of many workgroups and every kind of input are involved);
* the host-side status codes.
"""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import require_gpu
from oracle import checks as C

pytestmark = pytest.mark.gpu


def _dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def _gpu_mask(pkv, tables, lens, BS, NB, slots=None, pairs=None, append=False):
    pairs_t = None if pairs is None else _dev(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    return pkv.check_step_inputs(_dev(tables), _dev(lens), BS, NB, _dev(slots), pairs_t, append)


def _both(pkv, tables, lens, BS, NB, slots=None, pairs=None, append=False, label=""):
    want = C.step_input_violations(tables, lens, BS, NB, slots, pairs, append=append)
    got = _gpu_mask(pkv, tables, lens, BS, NB, slots, pairs, append)
    assert got == want, f"{label}: device mask {got:#x}, oracle {want:#x}"
    return got


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5, 6])
def test_decode_workloads_are_well_formed(idx):
    pkv = require_gpu()
    print(f"check decode workload C{idx}", flush=True)
    case = W.make_case(W.CONFIGS[idx], device="cpu", H=1)
    m = _both(pkv, case.block_tables, case.context_lens, case.BS, case.NB, case.slot_mapping, case.copy_pairs,
              append=True, label=f"C{idx}")
    assert m == 0


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_prompt_workloads_are_well_formed(idx):
    pkv = require_gpu()
    print(f"check prompt workload P{idx}", flush=True)
    case = W.make_prefill_case(W.PREFILL_CONFIGS[idx], device="cpu", H=1)
    m = _both(pkv, case.block_tables, case.context_lens, case.BS, case.NB, case.slot_mapping, case.copy_pairs,
              label=f"P{idx}")
    assert m == 0


def test_copy_on_write_before_and_after_the_copy():
    pkv = require_gpu()
    case = W.make_case(W.CONFIG_4_ON_WRITE, device="cpu", H=1)
    assert _both(pkv, case.block_tables, case.context_lens, case.BS, case.NB, case.slot_mapping, case.copy_pairs,
                 append=True, label="after") == 0
    pre = np.full_like(case.block_tables, case.poison_block)
    for s, row in enumerate(case.pre_tables):
        pre[s, :len(row)] = row
    m = _both(pkv, pre, case.context_lens, case.BS, case.NB, case.slot_mapping, None, label="before")
    assert m & C.SHARED_WRITE


def _random_step(rng, S_max=5, MB_max=5, NB_max=10):
    S, MB = int(rng.integers(1, S_max)), int(rng.integers(1, MB_max))
    BS = int(rng.choice([1, 2, 4, 16]))
    NB = int(rng.integers(2, NB_max))
    bad = rng.random() < 0.5
    lens = rng.integers(0 if not bad else -1, MB * BS + (2 if bad else 1), S)
    tables = rng.integers(-1 if bad else 0, NB + (1 if bad else 0), (S, MB))
    slots = np.empty(S, dtype=np.int64)
    for i in range(S):
        n = min(max(int(lens[i]), 0), MB * BS)
        if n > 0 and rng.random() < 0.8:
            slots[i] = tables[i, (n - 1) // BS] * BS + (n - 1) % BS
        else:
            slots[i] = rng.integers(-1, NB * BS + (1 if bad else 0))
    pairs = rng.integers(0 if not bad else -1, NB + (1 if bad else 0), (int(rng.integers(0, 4)), 2))
    return (tables.astype(np.int32), lens.astype(np.int32), slots.astype(np.int32), pairs.astype(np.int32),
            BS, NB)


def test_random_small_steps_match_the_oracle():
    pkv = require_gpu()
    rng = np.random.Generator(np.random.PCG64(4231))
    seen = 0
    for k in range(300):
        t, n, s, p, BS, NB = _random_step(rng)
        for append in (False, True):
            seen |= _both(pkv, t, n, BS, NB, s, p, append=append, label=f"step {k} append={append}")
    assert seen == 0xFF, f"not every condition was exercised: {seen:#x}"


@pytest.mark.parametrize("idx", [3, 5])
def test_faults_planted_in_full_size_workloads(idx):
    pkv = require_gpu()
    print(f"check planted faults C{idx}", flush=True)
    case = W.make_case(W.CONFIGS[idx], device="cpu", H=1)
    rng = np.random.Generator(np.random.PCG64(423 + idx))
    S, MB, BS, NB = case.S, case.MB, case.BS, case.NB
    for k in range(12):
        t = case.block_tables.copy()
        n = case.context_lens.copy()
        s = case.slot_mapping.copy()
        kind = k % 6
        i = int(rng.integers(0, S))
        if kind == 0:
            n[i] = MB * BS + 1 + int(rng.integers(0, 5))
        elif kind == 1:
            j = int(rng.integers(0, -(-int(n[i]) // BS)))
            t[i, j] = NB + int(rng.integers(0, 3))
        elif kind == 2:
            s[i] = NB * BS + int(rng.integers(0, 100))
        elif kind == 3:
            s[i] = s[(i + 1 + int(rng.integers(0, S - 1))) % S]
        elif kind == 4:
            s[i] += 1 if (int(n[i]) - 1) % BS < BS - 1 else -1
        else:                                  # another sequence maps i's last block
            o = (i + 1) % S
            t[o, 0] = t[i, (int(n[i]) - 1) // BS]
        m = _both(pkv, t, n, BS, NB, s, None, append=True, label=f"C{idx} fault {k} kind {kind}")
        assert m != 0


def test_status_codes():
    pkv = require_gpu()
    lib = pkv.lib()
    P = ctypes.c_void_p
    t = _dev(np.array([[0, 0, 0], [1, 0, 0]], dtype=np.int32))
    n = _dev(np.array([1, 2], dtype=np.int32))
    s = _dev(np.array([0, 17], dtype=np.int32))    # positions n - 1: block 0 offset 0, block 1 offset 1
    need = pkv.check_workspace_bytes(8, 16)
    assert need >= 256 and need % 4 == 0
    assert pkv.check_workspace_bytes(0, 16) == 0 and pkv.check_workspace_bytes(8, 0) == 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    mask = ctypes.c_uint32(77)

    def call(tp=t.data_ptr(), np_=n.data_ptr(), S=2, MB=3, sp=s.data_ptr(), T=2, pp=None, N=0, BS=16, NB=8,
             append=1, wp=ws.data_ptr(), wb=need):
        return lib.pkv_check_step_inputs(P(tp), P(np_), S, MB, P(sp), T, P(pp), N, BS, NB, append, P(wp), wb,
                                         ctypes.byref(mask), None)

    assert call() == pkv.PKV_OK and mask.value == 0
    assert call(S=-1) == pkv.PKV_ERR_INVALID_ARG
    assert call(MB=0) == pkv.PKV_ERR_INVALID_ARG
    assert call(NB=0) == pkv.PKV_ERR_INVALID_ARG
    assert call(tp=None) == pkv.PKV_ERR_INVALID_ARG
    assert call(sp=None) == pkv.PKV_ERR_INVALID_ARG
    assert call(N=1) == pkv.PKV_ERR_INVALID_ARG            # pairs NULL with N > 0
    assert call(T=1) == pkv.PKV_ERR_INVALID_ARG            # append needs T == S
    assert call(wp=None) == pkv.PKV_ERR_INVALID_ARG
    assert call(wb=need - 4) == pkv.PKV_ERR_WORKSPACE
    assert call(S=0, tp=None, np_=None, T=0, sp=None, append=0) == pkv.PKV_OK
    bad = _dev(np.array([0, 0], dtype=np.int32))           # two tokens, one slot
    assert call(sp=bad.data_ptr(), append=0) == pkv.PKV_ERR_DEVICE_CHECK
    assert mask.value == C.SLOT_DUP
    assert pkv.status_string(pkv.PKV_ERR_DEVICE_CHECK) == "device-side input check failed"


def test_maximum_sequence_count_and_inputs_untouched():
    """65,535 sequences (the grid's limit elsewhere), a well-formed appending
    step, then one fault in the very last table entry and one in the last
    slot; the inputs are left as they were."""
    pkv = require_gpu()
    rng = np.random.Generator(np.random.PCG64(65535))
    S, MB, BS = 65535, 4, 16
    NB = S * MB + 1
    perm = rng.permutation(NB - 1).astype(np.int32)
    t = perm.reshape(S, MB)
    n = rng.integers(1, MB * BS + 1, S).astype(np.int32)
    last = (n - 1)
    s = (t[np.arange(S), last // BS].astype(np.int64) * BS + last % BS).astype(np.int32)
    tg, ng, sg = _dev(t), _dev(n), _dev(s)
    print("check max sequences", flush=True)
    assert pkv.check_step_inputs(tg, ng, BS, NB, sg, None, True) == 0
    assert np.array_equal(tg.cpu().numpy(), t) and np.array_equal(ng.cpu().numpy(), n)
    assert np.array_equal(sg.cpu().numpy(), s)
    t2 = t.copy()
    t2[S - 1, (int(n[S - 1]) - 1) // BS] = NB                 # the last used entry past the pool
    assert _both(pkv, t2, n, BS, NB, s, None, append=True, label="last entry") & C.BLOCK_ID
    s2 = s.copy()
    s2[S - 1] = s[0]                                          # the last slot collides with the first
    assert _both(pkv, t, n, BS, NB, s2, None, append=True, label="last slot") & C.SLOT_DUP
