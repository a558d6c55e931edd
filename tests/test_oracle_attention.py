"""Pins for the fp64 oracle's write, gather, decode and prefill (CPU only).

Each test ties the oracle to something other than itself: a worked example
printed on the pages (tests/golden), a closed form, an invariant, or a
brute-force formulation written independently (matrix form with a mask, no
block table).
"""
import math

import numpy as np
import pytest

import workloads
from oracle import attention as A
from oracle.state import build_pool, build_state, empty_pool
from tests.conftest import golden


def _f64_rand(rng, *shape):
    return rng.standard_normal(shape)


# ------------------------------------------------------------ address pins
@pytest.mark.parametrize("layout", [A.NHD, A.HND])
def test_block_table_worked_example(layout):
    g = golden("block_table_example.json")
    bs, table = g["block_size"], g["block_table"]
    nb = max(table) + 1
    # pool whose every slot stores (block, offset) so a gather reveals the address
    if layout == A.NHD:
        cache = np.zeros((nb, bs, 1, 2), np.int64)
        for b in range(nb):
            for o in range(bs):
                cache[b, o, 0] = (b, o)
    else:
        cache = np.zeros((nb, 1, bs, 2), np.int64)
        for b in range(nb):
            for o in range(bs):
                cache[b, 0, o] = (b, o)
    rows = A.gather_seq(cache, np.array(table), g["num_tokens"], bs, layout)
    for t, b, o in g["lookups"]:
        assert tuple(rows[t, 0]) == (b, o)
    counts = [int(np.sum(rows[:, 0, 0] == b)) for b in table]
    assert counts == g["tokens_per_block"]


def test_write_matches_slot_formula_and_skips_padding():
    """slot = block * block_size + offset, negative slots skipped ([vllm] §3.2)."""
    rng = np.random.default_rng(0)
    nb, bs, hkv, d = 6, 4, 2, 3
    kc = np.full((nb, bs, hkv, d), 0xFFFF, np.uint16)
    vc = kc.copy()
    T = 9
    K = rng.integers(0, 0x7F00, (T, hkv, d)).astype(np.uint16)
    V = rng.integers(0, 0x7F00, (T, hkv, d)).astype(np.uint16)
    slots = np.array([5, -1, 0, 23, -7, 12, 11, -1, 2], np.int64)
    SENT = np.uint16(0xBEEF)
    for r in np.where(slots < 0)[0]:
        K[r] = SENT
        V[r] = SENT
    nk, nv = A.write_ref(kc, vc, K, V, slots, bs, A.NHD)
    for i, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(nk[s // bs, s % bs], K[i])
            assert np.array_equal(nv[s // bs, s % bs], V[i])
    touched = {int(s) for s in slots if s >= 0}
    for b in range(nb):
        for o in range(bs):
            if b * bs + o not in touched:
                assert np.all(nk[b, o] == 0xFFFF) and np.all(nv[b, o] == 0xFFFF)
    assert not np.any(nk == SENT) and not np.any(nv == SENT)
    # HND writes the same rows head-major
    hk, hv = A.write_ref(kc.transpose(0, 2, 1, 3).copy(), vc.transpose(0, 2, 1, 3).copy(),
                         K, V, slots, bs, A.HND)
    assert np.array_equal(hk.transpose(0, 2, 1, 3), nk)


def test_write_then_gather_round_trip():
    """Un-scattering the pool through the slots returns the rows exactly."""
    w = workloads.make(1)
    st = build_state(w)
    kc, vc = build_pool(w, st, include_step=True)
    for s in range(w.S):
        L = int(w.context_lens[s])
        k, v = w.kv(s)
        gk = A.gather_seq(kc, st.block_tables[s], L, w.bs)
        assert np.array_equal(gk.view(np.float32), k)
        gv = A.gather_seq(vc, st.block_tables[s], L, w.bs)
        assert np.array_equal(gv.view(np.float32), v)


# --------------------------------------------------------- attention pins
def test_dense_closed_forms():
    D, L, c = 8, 6, 3.0
    scale = 1.0 / math.sqrt(D)
    K = np.zeros((L, D))
    K[np.arange(L), np.arange(L)] = 1.0           # orthonormal keys
    V = np.arange(L * D, dtype=np.float64).reshape(L, D) * 0.25 - 3.0
    q = np.zeros(D)
    q[2] = c
    out, p = A.attention_dense(q, K, V, scale)
    e = math.exp(c * scale)
    expect_p = np.full(L, 1.0 / (e + L - 1))
    expect_p[2] = e / (e + L - 1)
    assert np.allclose(p, expect_p, rtol=0, atol=1e-15)
    assert np.allclose(out, expect_p @ V, rtol=0, atol=1e-13)
    # q = 0: uniform weights, output = mean of V
    out0, p0 = A.attention_dense(np.zeros(D), K, V, scale)
    assert np.allclose(out0, V.mean(0), atol=1e-14)
    # two keys: weight of key 1 = sigmoid(scale * (k1 - k0) . q)
    K2 = np.array([[1.0, 0, 0, 0], [0, 2.0, 0, 0]])
    q2 = np.array([0.5, -1.5, 0, 0])
    V2 = np.array([[1.0, 2, 3, 4], [-4.0, 0, 1, 7]])
    o2, p2 = A.attention_dense(q2, K2, V2, 0.5)
    w1 = 1.0 / (1.0 + math.exp(-0.5 * ((0 * 0.5 + 2 * -1.5) - (1 * 0.5))))
    assert abs(p2[1] - w1) < 1e-15
    assert np.allclose(o2, (1 - w1) * V2[0] + w1 * V2[1], atol=1e-14)


def test_empty_context_gives_zero():
    out, p = A.attention_dense(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 0.5)
    assert np.all(out == 0) and len(p) == 0


def _tiny_decode(seed=0, S=3, H=4, Hkv=2, D=16, bs=4, lens=(1, 5, 11), nb=16, layout=A.NHD):
    """Random tiny paged decode problem with its logical (un-paged) K/V."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(nb)
    Klog = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    Vlog = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    q = rng.standard_normal((S, H, D)).astype(np.float32)
    maxb = max(-(-L // bs) for L in lens)
    bt = np.full((S, maxb), nb, np.int32)          # nb = poison block
    shape = (nb + 1, bs, Hkv, D) if layout == A.NHD else (nb + 1, Hkv, bs, D)
    kc = np.full(shape, 0xFFFFFFFF, np.uint32)
    vc = kc.copy()
    nxt = 0
    for s, L in enumerate(lens):
        nblk = -(-L // bs)
        bt[s, :nblk] = perm[nxt:nxt + nblk]
        nxt += nblk
        slots = np.array([bt[s, t // bs] * bs + t % bs for t in range(L)], np.int64)
        kc, vc = A.write_ref(kc, vc, Klog[s], Vlog[s], slots, bs, layout)
    return dict(q=q, kc=kc, vc=vc, bt=bt, lens=np.array(lens), Klog=Klog, Vlog=Vlog,
                bs=bs, layout=layout, H=H, Hkv=Hkv, D=D, perm=perm)


@pytest.mark.parametrize("layout", [A.NHD, A.HND])
def test_decode_matches_brute_force_on_logical_kv(layout):
    t = _tiny_decode(layout=layout)
    scale = 1.0 / math.sqrt(t["D"])
    out, probs = A.decode_ref(t["q"], t["kc"], t["vc"], t["bt"], t["lens"], scale, t["bs"], "f32",
                              layout, return_probs=True)
    G = t["H"] // t["Hkv"]
    for s, L in enumerate(t["lens"]):
        K = t["Klog"][s].astype(np.float64)
        V = t["Vlog"][s].astype(np.float64)
        for h in range(t["H"]):
            z = scale * K[:, h // G] @ t["q"][s, h].astype(np.float64)
            w = np.exp(z - z.max())
            ref = (w / w.sum()) @ V[:, h // G]
            assert np.max(np.abs(out[s, h] - ref)) < 1e-12
            assert abs(probs[(s, h)].sum() - 1.0) < 1e-14 * max(L, 1)


def test_context_len_one_returns_v_exactly():
    t = _tiny_decode(lens=(1, 1, 1))
    out = A.decode_ref(t["q"], t["kc"], t["vc"], t["bt"], t["lens"], 0.25, t["bs"], "f32")
    G = t["H"] // t["Hkv"]
    for s in range(3):
        for h in range(t["H"]):
            assert np.array_equal(out[s, h], t["Vlog"][s][0, h // G].astype(np.float64))


def test_placement_invariance_bitwise():
    a = _tiny_decode(seed=3)
    rng = np.random.default_rng(99)
    # same logical contents, different physical placement
    b = dict(a)
    nb = 16
    perm = rng.permutation(nb)
    bt = np.full_like(a["bt"], nb)
    kc = np.full_like(a["kc"], 0xFFFFFFFF)
    vc = kc.copy()
    nxt = 0
    for s, L in enumerate(a["lens"]):
        nblk = -(-int(L) // a["bs"])
        bt[s, :nblk] = perm[nxt:nxt + nblk]
        nxt += nblk
        slots = np.array([bt[s, t // a["bs"]] * a["bs"] + t % a["bs"] for t in range(L)])
        kc, vc = A.write_ref(kc, vc, a["Klog"][s], a["Vlog"][s], slots, a["bs"])
    assert not np.array_equal(bt, a["bt"])
    o1 = A.decode_ref(a["q"], a["kc"], a["vc"], a["bt"], a["lens"], 0.25, a["bs"], "f32")
    o2 = A.decode_ref(a["q"], kc, vc, bt, a["lens"], 0.25, a["bs"], "f32")
    assert np.array_equal(o1, o2)


def test_gqa_equals_mha_with_repeated_kv():
    t = _tiny_decode(H=8, Hkv=2)
    G = 4
    kc_rep = np.repeat(t["kc"], G, axis=2)
    vc_rep = np.repeat(t["vc"], G, axis=2)
    o_gqa = A.decode_ref(t["q"], t["kc"], t["vc"], t["bt"], t["lens"], 0.3, t["bs"], "f32")
    o_mha = A.decode_ref(t["q"], kc_rep, vc_rep, t["bt"], t["lens"], 0.3, t["bs"], "f32")
    assert np.array_equal(o_gqa, o_mha)
    # G = 1 with Hkv = H is plain MHA: each head uses its own kv head
    t1 = _tiny_decode(H=2, Hkv=2)
    o = A.decode_ref(t1["q"], t1["kc"], t1["vc"], t1["bt"], t1["lens"], 0.3, t1["bs"], "f32")
    s = 2
    ref, _ = A.attention_dense(t1["q"][s, 1], t1["Klog"][s][:, 1], t1["Vlog"][s][:, 1], 0.3)
    assert np.max(np.abs(o[s, 1] - ref)) < 1e-13


@pytest.mark.parametrize("block", [1, 3, 16, 512, 10_000])
def test_online_softmax_identity(block):
    """Block-wise LSE merge equals softmax over the concatenation ([k4i])."""
    rng = np.random.default_rng(block)
    L, D = 1100, 32
    q, K, V = rng.standard_normal(D), rng.standard_normal((L, D)) * 3, rng.standard_normal((L, D))
    ref, _ = A.attention_dense(q, K, V, 0.2)
    assert np.max(np.abs(A.online_softmax_blocks(q, K, V, 0.2, block) - ref)) < 1e-12


def test_partition_merge_equals_dense():
    rng = np.random.default_rng(5)
    L, D, P = 2049, 16, 512
    q, K, V = rng.standard_normal(D), rng.standard_normal((L, D)) * 4, rng.standard_normal((L, D))
    stats = [A.partition_stats(q, K[i:i + P], V[i:i + P], 0.25) for i in range(0, L, P)]
    ref, _ = A.attention_dense(q, K, V, 0.25)
    assert np.max(np.abs(A.merge_partitions(stats) - ref)) < 1e-12


def test_bf16_upcast_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], np.uint16)
    expect = [1.0, -1.0, 3.140625, 2.0 ** -133, 3.3895313892515355e38]
    assert list(A.bits_to_f64(bits, "bf16")) == expect


def _binary16_value(c: int) -> float:
    """IEEE 754 binary16 from its fields: sign bit 15, exponent bits 14..10
    (bias 15), fraction bits 9..0; exponent 0 holds the subnormals
    frac * 2^-24, exponent 31 the infinities (fraction 0) and NaNs."""
    sign = -1.0 if c >> 15 else 1.0
    e, f = (c >> 10) & 0x1F, c & 0x3FF
    if e == 0x1F:
        return sign * np.inf if f == 0 else np.nan
    if e == 0:
        return sign * f * 2.0 ** -24
    return sign * (1.0 + f / 1024.0) * 2.0 ** (e - 15)


def test_f16_upcast_exact():
    """The f16 branches of both oracle upcasts (attention and the FP8 write's
    source read) against IEEE binary16: printed values of the format, then
    every one of the 65,536 codes against the field definition.  Reading the
    bits as bfloat16 instead (0x3C00 would be 2^-7) fails here."""
    from oracle import fp8 as F
    bits = np.array([0x3C00, 0xC000, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0x3555, 0x7C00, 0xFC00,
                     0x8000], np.uint16)
    expect = [1.0, -2.0, 2.0 ** -24, 1023 * 2.0 ** -24, 2.0 ** -14, 65504.0, 0.333251953125,
              np.inf, -np.inf, -0.0]
    for got in (A.bits_to_f64(bits, "f16"), F.f32_of(bits, "f16").astype(np.float64)):
        assert list(got) == expect
        assert np.signbit(got[-1])
    every = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = np.array([_binary16_value(int(c)) for c in every])
    for got in (A.bits_to_f64(every, "f16"), F.f32_of(every, "f16").astype(np.float64)):
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], ref[~nan])
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ------------------------------------------------------------- prefill pins
def _brute_causal(Q, K, V, scale):
    """Masked dense causal attention in matrix form; query row j of n sits at
    position L - n + j and sees keys 0 .. L - n + j."""
    n, L = Q.shape[0], K.shape[0]
    Sm = scale * Q @ K.T
    mask = np.arange(L)[None, :] <= (L - n + np.arange(n))[:, None]
    Sm = np.where(mask, Sm, -np.inf)
    Pm = np.exp(Sm - Sm.max(1, keepdims=True))
    Pm /= Pm.sum(1, keepdims=True)
    return Pm @ V


def _tiny_prefill(qlens, lens, seed=1, H=2, Hkv=1, D=8, bs=4, nb=40):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(nb)
    S = len(lens)
    Klog = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    Vlog = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    Q = rng.standard_normal((int(qsl[-1]), H, D)).astype(np.float32)
    maxb = max(-(-L // bs) for L in lens)
    bt = np.full((S, maxb), nb, np.int32)
    kc = np.full((nb + 1, bs, Hkv, D), 0xFFFFFFFF, np.uint32)
    vc = kc.copy()
    nxt = 0
    for s, L in enumerate(lens):
        k = -(-L // bs)
        bt[s, :k] = perm[nxt:nxt + k]
        nxt += k
        slots = [bt[s, t // bs] * bs + t % bs for t in range(L)]
        kc, vc = A.write_ref(kc, vc, Klog[s], Vlog[s], slots, bs)
    return Q, kc, vc, bt, qsl, np.array(lens), Klog, Vlog


def test_prefill_matches_brute_force_and_edges():
    qlens, lens = [3, 1, 6, 5], [3, 9, 6, 13]
    Q, kc, vc, bt, qsl, L, Klog, Vlog = _tiny_prefill(qlens, lens)
    H, G, scale = 2, 2, 0.35
    out = A.prefill_ref(Q, kc, vc, bt, qsl, L, scale, 4, "f32")
    for s in range(len(lens)):
        rows = slice(qsl[s], qsl[s + 1])
        for h in range(H):
            ref = _brute_causal(Q[rows, h].astype(np.float64), Klog[s][:, h // G].astype(np.float64),
                                Vlog[s][:, h // G].astype(np.float64), scale)
            assert np.max(np.abs(out[rows, h] - ref)) < 1e-12
    # fresh sequence (n == L): its first row sees only key 0, so equals V[0] exactly
    for s in (0, 2):
        for h in range(H):
            assert np.array_equal(out[qsl[s], h], Vlog[s][0, h // G].astype(np.float64))
    # last row of every sequence equals decode with the full context
    last = np.array([qsl[s + 1] - 1 for s in range(len(lens))])
    dec = A.decode_ref(Q[last], kc, vc, bt, L, scale, 4, "f32")
    assert np.max(np.abs(out[last] - dec)) == 0.0


def test_prefill_packed_equals_each_sequence_alone():
    g = golden("packed_offsets.json")
    assert list(np.concatenate([[0], np.cumsum(g["lengths"])])[:-1]) == g["offsets"]
    qlens = [n // 15 + 1 for n in g["lengths"]]     # 6, 9, 4, 15 rows: same structure, small
    lens = [n + 2 for n in qlens]
    Q, kc, vc, bt, qsl, L, _, _ = _tiny_prefill(qlens, lens, seed=7)
    packed = A.prefill_ref(Q, kc, vc, bt, qsl, L, 0.3, 4, "f32")
    for s in range(len(lens)):
        rows = slice(qsl[s], qsl[s + 1])
        alone = A.prefill_ref(Q[rows], kc, vc, bt[s:s + 1], np.array([0, qlens[s]]), L[s:s + 1],
                              0.3, 4, "f32")
        assert np.array_equal(packed[rows], alone)


def test_workload_state_pool_is_nan_outside_written_slots():
    """Free blocks, tail slots and the poison block keep the NaN fill."""
    w = workloads.make(1)
    st = build_state(w)
    kc, _ = build_pool(w, st, include_step=True)
    written = np.zeros(kc.shape[:2], bool)
    for s in range(w.S):
        for sl in st.seq_slots[s]:
            written[sl // w.bs, sl % w.bs] = True
    assert np.all(kc[~written] == 0xFFFFFFFF)
    assert np.all(kc[written] != 0xFFFFFFFF)
    assert np.all(kc[st.poison] == 0xFFFFFFFF)
    assert empty_pool(w).shape[0] == w.NB + 1
