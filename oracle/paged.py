"""The oracle's operations on a paged KV cache, in float64 / raw bits.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages cited (titles as published):

* [P1] "vLLM-v0.17.1技术解析：PagedAttention内存管理与显存优化技巧"
  (cnnetsun.cn/a/1550967)
* [P2] "在A10G上榨干LLaMA-7B：vLLM与PagedAttention实战"
  (devpress.csdn.net/awstech)
* [P3] the l189.com article on KV cache, PagedAttention, slot mapping and
  CUDA graphs (www.l189.com/news/180929)

Cache layout read from the pages: K and V live in two pools of fixed-size
physical blocks ([P1] §2.2, [P3] §2.1).  [P3] §2.1 sizes one block as
block_size * num_heads * head_size * 2 (K and V) * element size; the layout
taken here is one pool per K and V, shaped [num_blocks, num_heads,
block_size, head_size], with each token's head row of head_size elements
contiguous.  Logical block j of a sequence holds its tokens
[j*block_size, (j+1)*block_size) ([P2] §2.1), and the block table maps
logical block j to a physical block id ([P1] §2.2, [P2] §2.1).  A cache slot
is numbered physical_block * block_size + offset_in_block ([P3] §2.2, where
the int32 slot mapping addresses a pool of blocks with 16 slots each).

Every function validates its arguments and raises ValueError where the
operation is undefined (out-of-range ids, duplicate destinations).
"""

from __future__ import annotations

import numpy as np

from .codecs import SCALED, bits_dtype, decode, e4m3_encode, f32_div_rn, i8_encode


def _check_bits(name, arr, fmt):
    want = bits_dtype(fmt)
    if arr.dtype != want:
        raise ValueError(f"{name}: expected raw bits as {np.dtype(want)} for {fmt}, got {arr.dtype}")


def head_scales(tensor_scale, H):
    """The fp32 scale of each of the H heads of an 8-bit pool: one value for
    the whole pool (a number) or one per head (a sequence of H numbers).

    The pages name 8-bit KV formats without saying how finely a scale
    applies ("vLLM-v0.17.1技术解析" §3.3 lists FP8 and INT8; the l189.com
    article §4 turns on an FP8 cache).  Both readings are supported: a
    per-pool scale is the special case of equal per-head scales.  Scales
    must be finite and positive."""
    s = np.asarray(tensor_scale, dtype=np.float64)
    if s.ndim == 0:
        s = np.full(H, float(s))
    elif s.shape != (H,):
        raise ValueError(f"expected one scale per pool or one per head ({H}), got shape {s.shape}")
    if not (np.isfinite(s).all() and (s > 0).all()):
        raise ValueError("scales must be finite and positive")
    return s


def _cache_value(bits, cache_dtype, tensor_scale):
    """Values held in the cache for rows [..., H, D]: the stored elements,
    times head h's scale for the 8-bit formats (see oracle.codecs)."""
    vals = decode(bits, cache_dtype)
    if cache_dtype in SCALED:
        vals = vals * head_scales(tensor_scale, bits.shape[-2])[:, None]
    return vals


def gather_seq_rows(cache_bits, block_table_row, n, block_size):
    """Raw rows of one sequence's logical tokens 0..n-1, as [n, H, D].

    Token t sits in logical block t // block_size, at offset t % block_size
    of the physical block the table names for that logical block
    ([P2] §2.1; [P3] §2.2).
    """
    t = np.arange(n, dtype=np.int64)
    logical = t // block_size
    offset = t % block_size
    phys = np.asarray(block_table_row, dtype=np.int64)[logical]
    # cache_bits[phys, :, offset, :] -> [n, H, D]
    return cache_bits[phys, :, offset, :]


def paged_attention_decode_seq(q_bits_s, k_cache_bits, v_cache_bits, block_table_row, n,
                               scale, q_dtype, cache_dtype, k_scale=1.0, v_scale=1.0):
    """Decode attention of one sequence, all heads: returns float64 [H, D].

    The paged form computes exactly the attention of the contiguous cache
    ([P2] §2.1: the block mapping is invisible to the model; [P1] §2.1 and
    [P3] §1 describe the contiguous cache it replaces), so the oracle gathers
    the sequence's K and V into contiguous arrays and applies the textbook
    formula per head h:

        z_t = scale * sum_d q[h, d] * K[t, h, d]      for t < n
        p   = exp(z - max z) / sum_t exp(z - max z)
        out[h, :] = sum_t p_t * V[t, h, :]

    n = 0 gives zeros (no token to attend to; the pages do not define this
    case, and zeros are the reading taken).
    """
    H, D = q_bits_s.shape
    if n == 0:
        return np.zeros((H, D), dtype=np.float64)
    BS = k_cache_bits.shape[2]
    q = decode(q_bits_s, q_dtype)                                   # [H, D]
    K = _cache_value(gather_seq_rows(k_cache_bits, block_table_row, n, BS), cache_dtype, k_scale)
    V = _cache_value(gather_seq_rows(v_cache_bits, block_table_row, n, BS), cache_dtype, v_scale)
    z = float(scale) * np.einsum("thd,hd->ht", K, q)                # [H, n]
    z = z - z.max(axis=1, keepdims=True)
    w = np.exp(z)
    p = w / w.sum(axis=1, keepdims=True)                            # [H, n]
    return np.einsum("ht,thd->hd", p, V)                            # [H, D]


def paged_attention_decode(q_bits, k_cache_bits, v_cache_bits, block_tables, context_lens,
                           scale, q_dtype, cache_dtype, k_scale=1.0, v_scale=1.0, seqs=None):
    """Single-query decode over a paged KV cache: float64 [S, H, D].

    Arguments:
      q_bits        [S, H, D] raw bits of q_dtype (one query token per head).
      k/v_cache_bits [NB, H, BS, D] raw bits of cache_dtype.
      block_tables  int32 [S, MB]; entries past ceil(n_s / BS) are never read.
      context_lens  int32 [S]; n_s tokens are attended, n_s <= MB * BS.
      scale         softmax scale (typically 1/sqrt(D)), applied to q . k.
      k_scale, v_scale  scales of the 8-bit pools (ignored for other formats):
                    one per pool, or one per head (a sequence of H values).
      seqs          optional list of sequence indices; rows of the result not
                    listed are left as NaN (for sampled checks of big inputs).
    """
    _check_bits("q", q_bits, q_dtype)
    _check_bits("k_cache", k_cache_bits, cache_dtype)
    _check_bits("v_cache", v_cache_bits, cache_dtype)
    S, H, D = q_bits.shape
    NB, Hc, BS, Dc = k_cache_bits.shape
    if (Hc, Dc) != (H, D) or v_cache_bits.shape != k_cache_bits.shape:
        raise ValueError("q / cache shapes disagree")
    block_tables = np.asarray(block_tables)
    context_lens = np.asarray(context_lens)
    MB = block_tables.shape[1]
    out = np.full((S, H, D), np.nan, dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        n = int(context_lens[s])
        if n < 0 or n > MB * BS:
            raise ValueError(f"context_lens[{s}]={n} outside [0, {MB * BS}]")
        used = block_tables[s, : (n + BS - 1) // BS]
        if used.size and (used.min() < 0 or used.max() >= NB):
            raise ValueError(f"block table of sequence {s} names a block outside [0, {NB})")
        out[s] = paged_attention_decode_seq(q_bits[s], k_cache_bits, v_cache_bits, block_tables[s],
                                            n, scale, q_dtype, cache_dtype, k_scale, v_scale)
    return out


def _convert_for_cache(src_bits, src_dtype, cache_dtype, tensor_scale):
    """Element conversion done by the cache write.

    Same format: the bits are copied unchanged.  Into fp8 or INT8: the source
    value of head h (exact in binary32 for f16/bf16/f32) is divided by head
    h's scale (the pool's one scale, or its own) as one IEEE binary32
    division, then encoded with round-to-nearest-even and saturation
    (oracle.codecs.e4m3_encode / i8_encode).  src_bits is [T, H, D].
    """
    if src_dtype == cache_dtype:
        return src_bits.copy()
    if cache_dtype in SCALED and src_dtype in ("f16", "bf16", "f32"):
        x32 = decode(src_bits, src_dtype).astype(np.float32)   # exact: every source value fits binary32
        q = f32_div_rn(x32, head_scales(tensor_scale, src_bits.shape[1])[None, :, None])
        return e4m3_encode(q) if cache_dtype == "e4m3" else i8_encode(q)
    raise ValueError(f"no conversion {src_dtype} -> {cache_dtype}")


def reshape_and_cache(key_bits, value_bits, k_cache_bits, v_cache_bits, slot_mapping,
                      src_dtype, cache_dtype, k_scale=1.0, v_scale=1.0):
    """Write new tokens' K/V into their cache slots; returns new (k_cache, v_cache).

    For token i with slot = slot_mapping[i] >= 0, every head h gets
    cache[slot // BS, h, slot % BS, :] = conv_h(src[i, h, :]), conv_h dividing
    by head h's scale for 8-bit pools (k_scale / v_scale: one per pool or one
    per head) ([P3] §2.2: the
    int32 slot mapping names each token's slot; [P2] §2.1: a generated
    token's K/V is stored into the block its sequence maps).  A negative slot
    marks a padding token that is skipped (the pages do not cover padding).
    Two tokens naming one slot is undefined and raises.
    """
    _check_bits("key", key_bits, src_dtype)
    _check_bits("value", value_bits, src_dtype)
    _check_bits("k_cache", k_cache_bits, cache_dtype)
    _check_bits("v_cache", v_cache_bits, cache_dtype)
    T, H, D = key_bits.shape
    NB, Hc, BS, Dc = k_cache_bits.shape
    if (Hc, Dc) != (H, D) or value_bits.shape != key_bits.shape or v_cache_bits.shape != k_cache_bits.shape:
        raise ValueError("key / value / cache shapes disagree")
    slots = np.asarray(slot_mapping, dtype=np.int64)
    if slots.shape != (T,):
        raise ValueError("slot_mapping must hold one slot per token")
    live = slots[slots >= 0]
    if live.size and live.max() >= NB * BS:
        raise ValueError("slot outside the pool")
    if np.unique(live).size != live.size:
        raise ValueError("two tokens name the same slot")
    k_new = k_cache_bits.copy()
    v_new = v_cache_bits.copy()
    kc = _convert_for_cache(key_bits, src_dtype, cache_dtype, k_scale)
    vc = _convert_for_cache(value_bits, src_dtype, cache_dtype, v_scale)
    for i in range(T):
        slot = int(slots[i])
        if slot < 0:
            continue
        blk, off = slot // BS, slot % BS
        k_new[blk, :, off, :] = kc[i]
        v_new[blk, :, off, :] = vc[i]
    return k_new, v_new


def copy_blocks(k_cache_bits, v_cache_bits, pairs):
    """Copy whole physical blocks (K and V, all heads); returns new pools.

    Copy-on-write ([P2] §2.2): when a request is about to write a physical
    block that other requests still share, that block is first duplicated
    into a fresh one, which the writer then maps instead.  Each (src, dst)
    pair sets block dst to the contents block src had before the call.  A dst
    that repeats, or that is also a src, makes the result depend on order and
    is rejected.
    """
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    NB = k_cache_bits.shape[0]
    if pairs.size:
        if pairs.min() < 0 or pairs.max() >= NB:
            raise ValueError("block id outside the pool")
        dst = pairs[:, 1]
        if np.unique(dst).size != dst.size:
            raise ValueError("repeated destination block")
        if np.intersect1d(dst, pairs[:, 0]).size:
            raise ValueError("a destination is also a source")
    k_new = k_cache_bits.copy()
    v_new = v_cache_bits.copy()
    for src, dst in pairs:
        k_new[dst] = k_cache_bits[src]
        v_new[dst] = v_cache_bits[src]
    return k_new, v_new


def gather_kv(k_cache_bits, v_cache_bits, block_tables, context_lens):
    """Each sequence's K and V rows laid out contiguously, raw bits.

    Returns (k_out, v_out, cu_lens): k_out[cu_lens[s] + t] is token t of
    sequence s, shape [sum n_s, H, D]; cu_lens is int64 [S + 1].  This is the
    block gather of the decode ([P2] §2.1) on its own.
    """
    BS = k_cache_bits.shape[2]
    context_lens = np.asarray(context_lens, dtype=np.int64)
    cu = np.zeros(context_lens.size + 1, dtype=np.int64)
    cu[1:] = np.cumsum(context_lens)
    H, D = k_cache_bits.shape[1], k_cache_bits.shape[3]
    k_out = np.empty((int(cu[-1]), H, D), dtype=k_cache_bits.dtype)
    v_out = np.empty_like(k_out)
    for s, n in enumerate(context_lens):
        n = int(n)
        k_out[cu[s]:cu[s + 1]] = gather_seq_rows(k_cache_bits, block_tables[s], n, BS)
        v_out[cu[s]:cu[s + 1]] = gather_seq_rows(v_cache_bits, block_tables[s], n, BS)
    return k_out, v_out, cu


def paged_attention_prefill_seq(q_bits_s, k_cache_bits, v_cache_bits, block_table_row, n,
                                scale, q_dtype, cache_dtype, k_scale=1.0, v_scale=1.0):
    """Multi-query attention of one sequence's new tokens, all heads:
    returns float64 [q, H, D] for q_bits_s of shape [q, H, D].

    The sequence holds n tokens in the cache, its q newest ones included
    (their K/V were stored first, as a prompt's are when its blocks are
    allocated: [P2] §2.1 step 1 and the allocate-for-prompt sketch in §2.2).
    New token i sits at position n - q + i and, as in any decoder-only
    language model, attends to the positions up to and including its own:

        z_t = scale * q_i . K[t]        for t <= n - q + i
        out_i = sum_t softmax(z)_t V[t]

    With q = n this is a whole prompt; with q < n the first n - q tokens were
    cached before (for example a prefix shared with other requests,
    [P2] §2.2).  Gathering through the block table gives the contiguous
    cache's rows, so the result is the textbook masked attention.
    """
    qn, H, D = q_bits_s.shape
    if qn > n:
        raise ValueError(f"{qn} new tokens but only {n} cached")
    if qn == 0:
        return np.zeros((0, H, D), dtype=np.float64)
    BS = k_cache_bits.shape[2]
    q = decode(q_bits_s, q_dtype)                                   # [q, H, D]
    K = _cache_value(gather_seq_rows(k_cache_bits, block_table_row, n, BS), cache_dtype, k_scale)
    V = _cache_value(gather_seq_rows(v_cache_bits, block_table_row, n, BS), cache_dtype, v_scale)
    pos = (n - qn) + np.arange(qn)                                  # position of each new token
    visible = np.arange(n)[None, :] <= pos[:, None]                 # [q, n]
    out = np.empty((qn, H, D), dtype=np.float64)
    for h in range(H):
        z = float(scale) * (q[:, h, :] @ K[:, h, :].T)              # [q, n]
        z = np.where(visible, z, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        w = np.exp(z)
        p = w / w.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[:, h, :]
    return out


def paged_attention_prefill(q_bits, k_cache_bits, v_cache_bits, block_tables, context_lens, cu_q_lens,
                            scale, q_dtype, cache_dtype, k_scale=1.0, v_scale=1.0, seqs=None):
    """Multi-query (prompt) attention over a paged KV cache: float64 [Tq, H, D].

    Arguments:
      q_bits        [Tq, H, D] raw bits of q_dtype: the new tokens of all
                    sequences, sequence s owning rows cu_q_lens[s] ..
                    cu_q_lens[s + 1] - 1.
      k/v_cache_bits [NB, H, BS, D] raw bits of cache_dtype, the new tokens'
                    K/V already stored.
      block_tables  int32 [S, MB]; context_lens int32 [S] (n_s, new tokens
                    included); cu_q_lens int [S + 1], non-decreasing from 0,
                    with q_s = cu_q_lens[s + 1] - cu_q_lens[s] <= n_s.
      seqs          optional list of sequences; rows of other sequences are
                    left as NaN.
    See paged_attention_prefill_seq for the formula.  With q_s = 1 for every
    s this is paged_attention_decode.
    """
    _check_bits("q", q_bits, q_dtype)
    _check_bits("k_cache", k_cache_bits, cache_dtype)
    _check_bits("v_cache", v_cache_bits, cache_dtype)
    Tq, H, D = q_bits.shape
    NB, Hc, BS, Dc = k_cache_bits.shape
    if (Hc, Dc) != (H, D) or v_cache_bits.shape != k_cache_bits.shape:
        raise ValueError("q / cache shapes disagree")
    block_tables = np.asarray(block_tables)
    context_lens = np.asarray(context_lens)
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    S, MB = block_tables.shape
    if cu.shape != (S + 1,) or cu[0] != 0 or cu[-1] != Tq or (np.diff(cu) < 0).any():
        raise ValueError("cu_q_lens must run from 0 to the number of query rows, non-decreasing")
    out = np.full((Tq, H, D), np.nan, dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        n = int(context_lens[s])
        if n < 0 or n > MB * BS:
            raise ValueError(f"context_lens[{s}]={n} outside [0, {MB * BS}]")
        used = block_tables[s, : (n + BS - 1) // BS]
        if used.size and (used.min() < 0 or used.max() >= NB):
            raise ValueError(f"block table of sequence {s} names a block outside [0, {NB})")
        a, b = int(cu[s]), int(cu[s + 1])
        out[a:b] = paged_attention_prefill_seq(q_bits[a:b], k_cache_bits, v_cache_bits, block_tables[s], n,
                                               scale, q_dtype, cache_dtype, k_scale, v_scale)
    return out


def swap_blocks(src_k_bits, src_v_bits, dst_k_bits, dst_v_bits, pairs):
    """Copy whole blocks from one pair of pools to another; returns new
    (dst_k, dst_v).

    The pools are a GPU cache and a swap space in host memory, either way
    round: when GPU memory runs short, part of the KV cache is moved to CPU
    memory and brought back when needed ([P1] §4.1, the swap-space launch
    flag; [P2] §5.2, which says this costs speed but lifts the GPU memory
    limit).  Each (src, dst) pair sets block dst of the destination pools to
    block src of the source pools (all heads, K and V).  The two pools may
    hold different numbers of blocks; everything else about their shape and
    element format must match.  A repeated destination is rejected.
    """
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if src_k_bits.shape != src_v_bits.shape or dst_k_bits.shape != dst_v_bits.shape:
        raise ValueError("K and V pools of one side must match")
    if src_k_bits.shape[1:] != dst_k_bits.shape[1:] or src_k_bits.dtype != dst_k_bits.dtype:
        raise ValueError("source and destination pools differ in block shape or format")
    if pairs.size:
        if pairs[:, 0].min() < 0 or pairs[:, 0].max() >= src_k_bits.shape[0]:
            raise ValueError("source block outside its pool")
        if pairs[:, 1].min() < 0 or pairs[:, 1].max() >= dst_k_bits.shape[0]:
            raise ValueError("destination block outside its pool")
        if np.unique(pairs[:, 1]).size != pairs.shape[0]:
            raise ValueError("repeated destination block")
    k_new = dst_k_bits.copy()
    v_new = dst_v_bits.copy()
    for src, dst in pairs:
        k_new[dst] = src_k_bits[src]
        v_new[dst] = src_v_bits[src]
    return k_new, v_new
