"""Seeded random shapes through the C ABI against the fp64 oracle.

Each case draws a group size, kv head count, head size, block size, layout,
cache type (fp32, bf16, FP8), partition size and context lengths (or packed
prompt lengths for prefill) from a fixed seed, so every run checks the same
cases; the hand-picked cases of the other parity files stay as they are.
"""
import numpy as np
import pytest

from tests.gpu_util import TOL, announce, max_abs, need_gpu, torch

import workloads
from oracle import attention as A
from oracle.state import build_pool, build_state

pytestmark = pytest.mark.gpu

P = pytest.importorskip("paged_kv_cache_134_amd")
from paged_kv_cache_134_amd import metadata as M  # noqa: E402

KS, VS = workloads.FP8_K_SCALE, workloads.FP8_V_SCALE


def _decode_case(i):
    rng = np.random.default_rng([2024, i])
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2, 3]))
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128, 256]))
    S = int(rng.integers(1, 6))
    lens = rng.integers(1, 2600, S).tolist()
    kv = str(rng.choice(["f32", "bf16", "e4m3"]))
    layout = int(rng.integers(0, 2))
    part = int(rng.choice([0, -1, 16 * int(rng.integers(1, 80))]))
    return dict(G=G, Hkv=Hkv, D=D, bs=bs, lens=lens, kv=kv, layout=layout, part=part)


@pytest.mark.parametrize("i", range(16))
def test_decode_random_shapes(i):
    need_gpu()
    c = _decode_case(i)
    announce("random decode", i, c)
    dt = "f32" if c["kv"] == "f32" else "bf16"
    w = workloads.make(4, S=len(c["lens"]), H=c["G"] * c["Hkv"], Hkv=c["Hkv"], D=c["D"], bs=c["bs"],
                       lens=c["lens"], dtype=dt)
    fp8 = c["kv"] == "e4m3"
    kw = dict(kv_dtype="e4m3", k_scale=KS, v_scale=VS) if fp8 else {}
    dw = M.setup(w, layout=c["layout"], write_step=True, **kw)
    st = build_state(w)
    kc, vc = build_pool(w, st, layout=c["layout"], include_step=True, **kw)
    ref = A.decode_ref(w.query, kc, vc, st.block_tables, w.context_lens, w.scale, w.bs, w.dtype,
                       c["layout"], **kw)
    out = torch.full(w.query_shape, float("nan"), dtype=torch.float32, device="cuda")
    part = c["part"]
    ws = None
    if part != 0:
        nbytes = P.pa_decode_workspace_size(w.S, w.H, w.D, dw.max_context_len, part)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    if fp8:
        P.pa_decode_fp8(out, dw.query, dw.key_cache, dw.value_cache, dw.block_tables,
                        dw.context_lens, dw.max_context_len, w.scale, KS, VS, layout=c["layout"],
                        partition_size=part, workspace=ws)
    else:
        P.pa_decode(out, dw.query, dw.key_cache, dw.value_cache, dw.block_tables, dw.context_lens,
                    dw.max_context_len, w.scale, layout=c["layout"], partition_size=part,
                    workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    err, where = max_abs(got, ref)
    announce("max-abs", err)
    assert np.all(np.isfinite(got))
    assert err <= TOL[w.dtype], (c, err, where)


def _prefill_case(i):
    rng = np.random.default_rng([4048, i])
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2]))
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([4, 8, 16, 32, 64, 128, 256]))
    kv = str(rng.choice(["bf16", "e4m3"]))
    layout = int(rng.integers(0, 2))
    if rng.random() < 0.5:
        spec = ("5b", dict(packed_lens=rng.integers(1, 300, int(rng.integers(1, 6))).tolist()))
    else:
        spec = ("5c", dict(S=int(rng.integers(1, 4)), prefix=int(rng.integers(1, 700)),
                           suffix_lo=1, suffix_hi=int(rng.integers(2, 260))))
    return dict(G=G, Hkv=Hkv, D=D, bs=bs, kv=kv, layout=layout, spec=spec)


@pytest.mark.parametrize("i", range(10))
def test_prefill_random_shapes(i):
    need_gpu()
    c = _prefill_case(i)
    announce("random prefill", i, c)
    cfg, over = c["spec"]
    w = workloads.make(cfg, H=c["G"] * c["Hkv"], Hkv=c["Hkv"], D=c["D"], bs=c["bs"], **over)
    fp8 = c["kv"] == "e4m3"
    kw = dict(kv_dtype="e4m3", k_scale=KS, v_scale=VS) if fp8 else {}
    dw = M.setup(w, layout=c["layout"], write_step=True, **kw)
    st = build_state(w)
    kc, vc = build_pool(w, st, layout=c["layout"], include_step=True, **kw)
    ref = A.prefill_ref(w.query, kc, vc, st.block_tables, w.query_start_loc, w.context_lens,
                        w.scale, w.bs, w.dtype, c["layout"], **kw)
    out = torch.full(w.query_shape, float("nan"), dtype=torch.float32, device="cuda")
    args = (out, dw.query, dw.key_cache, dw.value_cache, dw.block_tables, dw.query_start_loc,
            dw.context_lens, int(w.query_lens.max()), dw.max_context_len, w.scale)
    if fp8:
        P.pa_prefill_fp8(*args, KS, VS, layout=c["layout"])
    else:
        P.pa_prefill(*args, layout=c["layout"])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    err, where = max_abs(got, ref)
    announce("max-abs", err)
    assert np.all(np.isfinite(got))
    assert err <= TOL[w.dtype], (c, err, where)
