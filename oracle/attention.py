"""fp64 reference for the cache write, decode attention and causal packed prefill.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Parity is pinned by
tests/test_oracle_attention.py.

Layouts ([vllm] §3.3):
  NHD  cache[num_blocks, block_size, num_kv_heads, head_size]
  HND  cache[num_blocks, num_kv_heads, block_size, head_size]  (head-major)

Caches are handled as raw bit arrays (uint32 for float32, uint16 for
bfloat16/float16) so the write is a bit copy; attention upcasts the bits to
float64 exactly.
"""
from __future__ import annotations

import numpy as np

from .fp8 import E4M3, quantize

NHD, HND = 0, 1


def bits_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of stored values to float64.

    dtype "f32": float32 values (or their uint32 bits); "bf16": uint16 bit
    patterns of bfloat16 (the upper half of a float32); "f16": uint16 bits of
    IEEE half.
    """
    if dtype == "f32":
        return np.asarray(a).view(np.float32).astype(np.float64) if a.dtype != np.float32 \
            else a.astype(np.float64)
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)) \
            .view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "e4m3":  # FP8 codes (uint8), unscaled values
        return E4M3[np.asarray(a, dtype=np.uint8)]
    raise ValueError(dtype)


def _cache_f64(rows, dtype, kv_dtype, scale):
    """Gathered cache rows as float64: the stored values, times the scale for
    an FP8 cache (oracle.fp8: a code reads back as its value times scale)."""
    if kv_dtype is None or kv_dtype == dtype:
        return bits_to_f64(rows, dtype)
    assert kv_dtype == "e4m3", kv_dtype
    return bits_to_f64(rows, "e4m3") * float(np.float32(scale))


def _raw(a: np.ndarray) -> np.ndarray:
    """View float arrays as same-width unsigned bits (bit-copy semantics)."""
    if a.dtype == np.float32:
        return a.view(np.uint32)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    return a


# --------------------------------------------------------------------- write
def write_ref(key_cache, value_cache, key, value, slot_mapping, block_size, layout=NHD):
    """Scatter new tokens' K/V rows into copies of the block pool.

    [vllm] §3.2 and §7.4: each token i carries a global slot
    ``slot = block_number * block_size + block_offset``; a negative slot marks
    a padding token, which is skipped.  Row i ([num_kv_heads, head_size]) is
    copied bit for bit to (block = slot // block_size, offset = slot %
    block_size); every other slot of the pool is left as it was.  Non-negative
    slots must be distinct (asserted).

    Returns (new_key_cache, new_value_cache) as raw bit arrays.
    """
    kc = _raw(np.array(key_cache, copy=True))
    vc = _raw(np.array(value_cache, copy=True))
    k = _raw(np.asarray(key))
    v = _raw(np.asarray(value))
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = slots[slots >= 0]
    assert len(np.unique(live)) == len(live), "duplicate slots"
    for i, s in enumerate(slots):
        if s < 0:
            continue
        b, o = divmod(int(s), block_size)
        if layout == NHD:
            kc[b, o] = k[i]
            vc[b, o] = v[i]
        else:
            kc[b, :, o] = k[i]
            vc[b, :, o] = v[i]
    return kc, vc


def write_ref_fp8(key_cache, value_cache, key, value, slot_mapping, block_size, src_dtype,
                  k_scale, v_scale, layout=NHD):
    """Cache write into an FP8 (E4M3) pool ([vllm] §6.3, §7.4 flash variant):
    every new row is quantised (``oracle.fp8.quantize``: x / scale in fp32,
    nearest E4M3 with ties to even, saturated to +-448) and scattered exactly
    as ``write_ref`` scatters; padding rows are skipped.  Caches are uint8
    codes; returns the new (key, value) code arrays."""
    kq = quantize(key, src_dtype, k_scale)
    vq = quantize(value, src_dtype, v_scale)
    return write_ref(key_cache, value_cache, kq, vq, slot_mapping, block_size, layout)


# -------------------------------------------------------------------- gather
def gather_seq(cache, block_table_row, L, block_size, layout=NHD):
    """Logical rows 0..L-1 of one sequence, read through its block table.

    [k4i] #the-block-table and [vllm] §3.1: token t lives in physical block
    ``block_table[t // block_size]`` at offset ``t % block_size``.  Entries of
    the table past ceil(L / block_size) are never read.  Returns raw rows
    [L, num_kv_heads, head_size].
    """
    t = np.arange(int(L))
    blk = np.asarray(block_table_row)[t // block_size]
    off = t % block_size
    if layout == NHD:
        return cache[blk, off]
    return cache[blk, :, off]


# ----------------------------------------------------------------- attention
def attention_dense(q, K, V, scale):
    """softmax(scale * K q) V for one query over contiguous K, V (float64).

    This is the plain definition the paged kernels must reproduce ([tut] §3.4:
    paging does not change the attention math; [k4i] #paged-attention-kernel:
    the block-wise computation equals softmax over the concatenated sequence).
    Returns (out [D], p [L]).  With no keys (L = 0) the output is 0.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[-1]), np.zeros(0)
    z = scale * (K @ q)
    w = np.exp(z - z.max())
    p = w / w.sum()
    return p @ V, p


def decode_ref(query, key_cache, value_cache, block_tables, context_lens, scale,
               block_size, dtype, layout=NHD, return_probs=False, kv_dtype=None,
               k_scale=1.0, v_scale=1.0):
    """Decode attention over the paged cache, float64.

    For sequence s and query head h: kv head ``h // (H / Hkv)`` (contiguous
    GQA groups), keys/values are the first ``context_lens[s]`` logical tokens
    gathered through ``block_tables[s]`` ([vllm] §3.1, §6.2 with
    ``seqlen_k = seq_lens``), and the output is ``attention_dense``.
    ``query`` is [S, H, D] raw; returns out [S, H, D] (and the probability
    vectors per (s, h) if asked).  ``kv_dtype`` "e4m3": the caches hold FP8
    codes that read back as value * k_scale (keys) and value * v_scale
    (values), the query keeps ``dtype``.
    """
    qf = bits_to_f64(np.asarray(query), dtype)
    S, H, D = qf.shape
    Hkv = key_cache.shape[2] if layout == NHD else key_cache.shape[1]
    G = H // Hkv
    out = np.zeros((S, H, D))
    probs = {}
    for s in range(S):
        L = int(context_lens[s])
        K = _cache_f64(gather_seq(key_cache, block_tables[s], L, block_size, layout), dtype,
                       kv_dtype, k_scale)
        V = _cache_f64(gather_seq(value_cache, block_tables[s], L, block_size, layout), dtype,
                       kv_dtype, v_scale)
        for h in range(H):
            o, p = attention_dense(qf[s, h], K[:, h // G], V[:, h // G], scale)
            out[s, h] = o
            if return_probs:
                probs[(s, h)] = p
    return (out, probs) if return_probs else out


def prefill_ref(query, key_cache, value_cache, block_tables, query_start_loc, context_lens,
                scale, block_size, dtype, layout=NHD, kv_dtype=None, k_scale=1.0, v_scale=1.0):
    """Causal packed-sequence prefill over the paged cache, float64.

    Queries of all sequences are packed without padding; sequence s owns rows
    ``query_start_loc[s] .. query_start_loc[s+1]-1`` ([packed] §2.3; [vllm]
    §5.4 ``query_start_loc``).  With n = that row count and L =
    ``context_lens[s]`` (all L tokens already cached), row j is the token at
    absolute position ``L - n + j`` and attends to keys 0 .. L - n + j (causal,
    aligned to the end of the context: [vllm] §6.2 ``causal=True`` with
    ``seqlen_k = seq_lens``).  Returns out [num_tokens, H, D].  ``kv_dtype``
    and the scales as in ``decode_ref``.
    """
    qf = bits_to_f64(np.asarray(query), dtype)
    T, H, D = qf.shape
    Hkv = key_cache.shape[2] if layout == NHD else key_cache.shape[1]
    G = H // Hkv
    out = np.zeros((T, H, D))
    qsl = np.asarray(query_start_loc)
    for s in range(len(qsl) - 1):
        n = int(qsl[s + 1] - qsl[s])
        L = int(context_lens[s])
        assert n <= L
        K = _cache_f64(gather_seq(key_cache, block_tables[s], L, block_size, layout), dtype,
                       kv_dtype, k_scale)
        V = _cache_f64(gather_seq(value_cache, block_tables[s], L, block_size, layout), dtype,
                       kv_dtype, v_scale)
        for j in range(n):
            a = L - n + j  # absolute position of query row j
            for h in range(H):
                o, _ = attention_dense(qf[qsl[s] + j, h], K[:a + 1, h // G], V[:a + 1, h // G], scale)
                out[qsl[s] + j, h] = o
    return out


# ------------------------------------------------ block-wise form (cross-check)
def partition_stats(q, K, V, scale):
    """Statistics (m_p, l_p, o_p) of one key range ([vllm] §7.3, V2):
    m_p = the range's largest score, l_p = sum exp(score - m_p), o_p = sum
    exp(score - m_p) v (unnormalised).  The softmax over the range alone is
    o_p / l_p."""
    q = np.asarray(q, dtype=np.float64)
    a = scale * (np.asarray(K, dtype=np.float64) @ q)
    m = a.max()
    e = np.exp(a - m)
    return m, e.sum(), e @ np.asarray(V, dtype=np.float64)


def combine_stats(x, y):
    """Statistics of the union of two disjoint key ranges from theirs: both
    are re-expressed relative to the larger maximum M, after which the
    normalisers and the unnormalised outputs simply add."""
    (mx, lx, ox), (my, ly, oy) = x, y
    M = max(mx, my)
    cx, cy = np.exp(mx - M), np.exp(my - M)
    return M, cx * lx + cy * ly, cx * ox + cy * oy


def merge_partitions(stats):
    """Reduce step of split-K ([vllm] §7.3): all partitions' statistics
    combined at once, M = max_p m_p, out = sum_p e^(m_p - M) o_p /
    sum_p e^(m_p - M) l_p."""
    M = max(m for m, _, _ in stats)
    num = sum(np.exp(m - M) * o for m, _, o in stats)
    den = sum(np.exp(m - M) * l for m, l, _ in stats)
    return num / den


def online_softmax_blocks(q, K, V, scale, block):
    """Attention over K, V taken ``block`` keys at a time ([k4i]
    #paged-attention-kernel: a sequence's blocks may be visited one by one):
    the running statistics are the left fold of ``combine_stats`` over the
    blocks' ``partition_stats``, and the output is o / l of the fold.  Pinned
    against ``attention_dense`` in float64."""
    stats = [partition_stats(q, K[b0:b0 + block], V[b0:b0 + block], scale)
             for b0 in range(0, np.asarray(K).shape[0], block)]
    if not stats:
        return np.zeros(np.asarray(V).shape[-1])
    m, l, o = stats[0]
    for st in stats[1:]:
        m, l, o = combine_stats((m, l, o), st)
    return o / l
