"""GPU parity at the workloads' full sizes, in the launch configuration the
bench times (HND pools; split-K decode at the workload's own partition size
where it names one, and at the library's choice), on whole outputs where the
oracle finishes in seconds and on every head of sampled sequences / rows
otherwise, plus properties that hold at any size (every output finite,
sampled pool slots bit-exact).

The oracle side derives its own slots (allocator model) and computes each
sampled output as the plain definition over the sequence's logical K/V.
"""
import numpy as np
import pytest

from tests.gpu_util import TOL, announce, need_gpu, torch

import workloads
from oracle import attention as A
from oracle.state import build_state

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

P = pytest.importorskip("paged_kv_cache_134_amd")
from paged_kv_cache_134_amd import metadata as M  # noqa: E402


def _pool_rows(dw, slots, kvh):
    """K and V rows of kv head kvh at the given slots, read back from the device."""
    w = dw.w
    idx = torch.from_numpy(np.asarray(slots, np.int64)).cuda()
    blk, off = idx // w.bs, idx % w.bs
    if dw.layout == P.NHD:
        k, v = dw.key_cache[blk, off, kvh], dw.value_cache[blk, off, kvh]
    else:
        k, v = dw.key_cache[blk, kvh, off], dw.value_cache[blk, kvh, off]
    view = torch.int32 if w.dtype == "f32" else torch.int16
    raw = np.uint32 if w.dtype == "f32" else np.uint16
    return k.contiguous().view(view).cpu().numpy().view(raw), \
        v.contiguous().view(view).cpu().numpy().view(raw)


def _check_pool_samples(dw, st, seqs):
    w = dw.w
    for s in seqs:
        L = int(w.context_lens[s])
        pos = sorted({0, min(w.bs - 1, L - 1), min(w.bs, L - 1), L // 2, L - 1})
        k_log, v_log = [], []
        for t in pos:
            k, v = w.kv(s, t, t + 1)
            k_log.append(k[0])
            v_log.append(v[0])
        for kvh in sorted({0, w.Hkv - 1}):
            kg, vg = _pool_rows(dw, st.seq_slots[s][pos], kvh)
            raw = lambda x: np.asarray(x).view(np.uint32 if w.dtype == "f32" else np.uint16)  # noqa
            assert np.array_equal(kg, raw(np.stack(k_log)[:, kvh])), (s, kvh)
            assert np.array_equal(vg, raw(np.stack(v_log)[:, kvh])), (s, kvh)


def _oracle_heads(w, s, qf, heads, rows=None):
    """The plain definition for sequence s at the given query heads: decode
    (rows None) or the prefill rows given as packed row indices.  K/V are the
    sequence's logical values, upcast one kv head at a time."""
    K, V = w.kv(s)
    out = {}
    by_g = {}
    for h in heads:
        by_g.setdefault(h // w.G, []).append(h)
    n, L = (int(w.query_lens[s]), int(w.context_lens[s])) if rows is not None else (0, 0)
    for g, hs in by_g.items():
        Kf, Vf = A.bits_to_f64(K[:, g], w.dtype), A.bits_to_f64(V[:, g], w.dtype)
        for h in hs:
            if rows is None:
                out[h], _ = A.attention_dense(qf[s, h], Kf, Vf, w.scale)
            else:
                q0 = int(w.query_start_loc[s])
                for r in rows:
                    a = L - n + (r - q0)  # absolute position of the row's token
                    out[(r, h)], _ = A.attention_dense(qf[r, h], Kf[:a + 1], Vf[:a + 1], w.scale)
    return out


# (workload, partition size: None = the library's choice, else the workload's own)
DECODE_FULL = [(2, None), (3, None), (4, 512), (4, None), ("5a", None)]


@pytest.mark.parametrize("cfg,part", DECODE_FULL)
def test_decode_full_size(cfg, part):
    """Full-size decode in the bench's launch configuration.  The 7B-like and
    70B-like workloads are compared whole (every sequence and head); the
    long-context (at its 512-token partitions and at the library's choice)
    and shared-prefix workloads on every head of sampled sequences."""
    need_gpu()
    w = workloads.make(cfg)
    ps = part if part is not None else P.pa_decode_auto_partition(
        w.S, w.H, w.Hkv, P.KV_DTYPE[w.dtype], w.max_context_len, int(w.context_lens.sum()))
    assert ps > 0
    announce("full-size decode", w.name, "partition", ps)
    dw = M.setup(w, layout=P.HND, write_step=True)
    st = build_state(w)
    assert np.array_equal(dw.block_tables_host, st.block_tables)
    ws = torch.empty(P.pa_decode_workspace_size(w.S, w.H, w.D, dw.max_context_len, ps),
                     dtype=torch.uint8, device="cuda")
    out = torch.full(w.query_shape, float("nan"), dtype=torch.float32, device="cuda")
    P.pa_decode_partitions(out, dw.query, dw.key_cache, dw.value_cache, dw.block_tables,
                           dw.context_lens, dw.max_context_len, w.scale, ps, ws, layout=dw.layout)
    P.pa_decode_reduce(out, dw.context_lens, dw.max_context_len, w.Hkv, ps, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    lens = w.context_lens
    whole = cfg in (2, 3)
    seqs = range(w.S) if whole else sorted({0, w.S // 2, w.S - 1, int(np.argmax(lens)),
                                            int(np.argmin(lens))})
    _check_pool_samples(dw, st, sorted({0, w.S // 2, w.S - 1, int(np.argmax(lens))}))
    del dw
    assert np.all(np.isfinite(got))
    qf = A.bits_to_f64(w.query, w.dtype)
    worst = 0.0
    for s in seqs:
        ref = _oracle_heads(w, s, qf, range(w.H))
        for h in range(w.H):
            worst = max(worst, float(np.max(np.abs(got[s, h] - ref[h]))))
    announce("max-abs", worst, "over", len(seqs), "sequences x", w.H, "heads")
    assert worst <= TOL[w.dtype]


@pytest.mark.parametrize("cfg", ["5b", "5c"])
def test_prefill_full_size(cfg):
    """Full-size prefill.  The packed prefill of the printed lengths is
    compared whole (all 460 rows, every head); the prefix-cached suffix
    prefill on every head of sampled rows (first, second, middle, last) of
    sampled sequences."""
    need_gpu()
    w = workloads.make(cfg)
    announce("full-size prefill", w.name)
    dw = M.setup(w, layout=P.HND, write_step=True)
    st = build_state(w)
    assert np.array_equal(dw.block_tables_host, st.block_tables)
    out = torch.full(w.query_shape, float("nan"), dtype=torch.float32, device="cuda")
    P.pa_prefill(out, dw.query, dw.key_cache, dw.value_cache, dw.block_tables, dw.query_start_loc,
                 dw.context_lens, int(w.query_lens.max()), dw.max_context_len, w.scale,
                 layout=dw.layout)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    seqs = range(w.S) if cfg == "5b" else sorted({0, w.S // 2, w.S - 1})
    _check_pool_samples(dw, st, sorted({0, w.S // 2, w.S - 1}))
    del dw
    assert np.all(np.isfinite(got))
    qf = A.bits_to_f64(w.query, w.dtype)
    worst = 0.0
    for s in seqs:
        n, q0 = int(w.query_lens[s]), int(w.query_start_loc[s])
        rows = range(q0, q0 + n) if cfg == "5b" else [q0 + j for j in sorted({0, 1, n // 2, n - 1})]
        ref = _oracle_heads(w, s, qf, range(w.H), rows=rows)
        for (r, h), o in ref.items():
            worst = max(worst, float(np.max(np.abs(got[r, h] - o))))
    announce("max-abs", worst)
    assert worst <= TOL[w.dtype]


def test_cascade_decode_full_size_sampled():
    """The shared-prefix workload through the cascade path (common prefix =
    its fully shared blocks), sampled against the plain definition."""
    need_gpu()
    w = workloads.make("5a")
    announce("full-size cascade decode", w.name)
    dw = M.setup(w, layout=P.HND, write_step=True)
    st = build_state(w)
    common = (w.prefix_len // w.bs) * w.bs
    nbc = common // w.bs
    assert np.all(st.block_tables[:, :nbc] == st.block_tables[0, :nbc])
    ws = torch.empty(P.pa_decode_cascade_workspace_size(w.S, w.H, w.D, dw.max_context_len, common, -1),
                     dtype=torch.uint8, device="cuda")
    out = torch.full(w.query_shape, float("nan"), dtype=torch.float32, device="cuda")
    P.pa_decode_cascade(out, dw.query, dw.key_cache, dw.value_cache, dw.block_tables,
                        dw.context_lens, dw.max_context_len, common, w.scale, ws, layout=dw.layout)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    qf = A.bits_to_f64(w.query, w.dtype)
    worst = 0.0
    for s in sorted({0, w.S // 2, w.S - 1}):
        ref = _oracle_heads(w, s, qf, range(w.H))
        for h in range(w.H):
            worst = max(worst, float(np.max(np.abs(got[s, h] - ref[h]))))
    announce("max-abs", worst)
    assert worst <= TOL[w.dtype]


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_fp8_decode_full_size_sampled(cfg, layout):
    """FP8 pools at full size, as `bench.py --kv fp8` runs them: sampled pool
    codes bit-exact against the oracle's quantisation of the same rows, and
    sampled outputs against the plain definition over the codes read back."""
    from oracle import fp8 as F
    need_gpu()
    w = workloads.make(cfg)
    ks, vs = workloads.FP8_K_SCALE, workloads.FP8_V_SCALE
    lay = P.NHD if layout == "nhd" else P.HND
    announce("full-size fp8 decode", w.name, layout)
    dw = M.setup(w, layout=lay, write_step=True, kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    st = build_state(w)
    # the bench's partition: the workload's own (512 for the long context), else the library's
    ps = w.partition_size or P.pa_decode_auto_partition(w.S, w.H, w.Hkv, P.PA_FP8_E4M3,
                                                        dw.max_context_len, int(w.context_lens.sum()))
    announce("partition", ps)
    ws = torch.empty(max(16, P.pa_decode_workspace_size(w.S, w.H, w.D, dw.max_context_len, ps)),
                     dtype=torch.uint8, device="cuda")
    out = torch.full(w.query_shape, float("nan"), dtype=torch.float32, device="cuda")
    P.pa_decode_partitions_fp8(out, dw.query, dw.key_cache, dw.value_cache, dw.block_tables,
                               dw.context_lens, dw.max_context_len, w.scale, ks, vs, ps, ws,
                               layout=lay)
    P.pa_decode_reduce(out, dw.context_lens, dw.max_context_len, w.Hkv, ps, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    lens = w.context_lens
    seqs = sorted({0, w.S // 2, w.S - 1, int(np.argmax(lens)), int(np.argmin(lens))})
    qf = A.bits_to_f64(w.query, w.dtype)
    worst = 0.0
    for s in seqs:
        K, V = w.kv(s)
        kq, vq = F.quantize(K, w.dtype, ks), F.quantize(V, w.dtype, vs)
        # the device pool holds exactly these codes at the sequence's slots
        idx = torch.from_numpy(st.seq_slots[s].astype(np.int64)).cuda()
        blk, off = idx // w.bs, idx % w.bs
        kd = dw.key_cache[blk, off] if lay == P.NHD else dw.key_cache[blk, :, off]
        vd = dw.value_cache[blk, off] if lay == P.NHD else dw.value_cache[blk, :, off]
        assert np.array_equal(kd.cpu().numpy(), kq) and np.array_equal(vd.cpu().numpy(), vq), s
        Kf, Vf = F.dequantize(kq, ks), F.dequantize(vq, vs)
        for h in sorted({0, w.G - 1, w.H // 2, w.H - 1}):
            g = h // w.G
            ref, _ = A.attention_dense(qf[s, h], Kf[:, g], Vf[:, g], w.scale)
            worst = max(worst, float(np.max(np.abs(got[s, h] - ref))))
    announce("max-abs", worst)
    assert worst <= TOL[w.dtype]


def test_fp8_prefill_full_size_sampled():
    """The prefix-cached suffix prefill over FP8 pools at full size, as
    `bench.py --config 5c --kv fp8` runs it (the 3-waves-per-SIMD FP8 kernel):
    sampled pool codes bit-exact against the oracle's quantisation, sampled
    rows against the plain definition over the codes read back."""
    from oracle import fp8 as F
    need_gpu()
    w = workloads.make("5c")
    ks, vs = workloads.FP8_K_SCALE, workloads.FP8_V_SCALE
    announce("full-size fp8 prefill", w.name)
    dw = M.setup(w, layout=P.HND, write_step=True, kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    st = build_state(w)
    out = torch.full(w.query_shape, float("nan"), dtype=torch.float32, device="cuda")
    P.pa_prefill_fp8(out, dw.query, dw.key_cache, dw.value_cache, dw.block_tables,
                     dw.query_start_loc, dw.context_lens, int(w.query_lens.max()),
                     dw.max_context_len, w.scale, ks, vs, layout=P.HND)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    seqs = sorted({0, w.S // 2, w.S - 1})
    qf = A.bits_to_f64(w.query, w.dtype)
    worst = 0.0
    for s in seqs:
        K, V = w.kv(s)
        kq, vq = F.quantize(K, w.dtype, ks), F.quantize(V, w.dtype, vs)
        idx = torch.from_numpy(st.seq_slots[s].astype(np.int64)).cuda()
        blk, off = idx // w.bs, idx % w.bs
        assert np.array_equal(dw.key_cache[blk, :, off].cpu().numpy(), kq), s
        assert np.array_equal(dw.value_cache[blk, :, off].cpu().numpy(), vq), s
        Kf, Vf = F.dequantize(kq, ks), F.dequantize(vq, vs)
        n, L = int(w.query_lens[s]), int(w.context_lens[s])
        for h in sorted({0, w.H - 1}):
            g = h // w.G
            for j in sorted({0, 1, n // 2, n - 1}):
                a = L - n + j
                r = int(w.query_start_loc[s]) + j
                ref, _ = A.attention_dense(qf[r, h], Kf[:a + 1, g], Vf[:a + 1, g], w.scale)
                worst = max(worst, float(np.max(np.abs(got[r, h] - ref))))
    announce("max-abs", worst)
    assert worst <= TOL["bf16"]
