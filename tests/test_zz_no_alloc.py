"""pa_decode_static_scratch (decode that allocates nothing: its split-K
workspace is the library's static per-GPU array) against pa_decode with a
caller workspace, through the C ABI: two calls in a row, the second on a
smaller batch, each bitwise equal to pa_decode's output at the same partition
size (same kernels, same launch configuration) and within the oracle's
tolerance; a shape whose workspace exceeds the array is refused before any
device call.
"""
import ctypes

import numpy as np
import pytest

from tests.gpu_util import TOL, announce, max_abs, need_gpu, torch

import workloads
from oracle import attention as A
from oracle.state import build_pool, build_state

pytestmark = pytest.mark.gpu

P = pytest.importorskip("paged_kv_cache_134_amd")
from paged_kv_cache_134_amd import metadata as M  # noqa: E402

_i32, _f32, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
_fn = P._lib.pa_decode_static_scratch
_fn.restype = _i32
_fn.argtypes = [_vp, _i32, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                _i32, _i32, _i32, _f32, _i32, _vp]
SCRATCH = 96 << 20


def _static(dw, part):
    w = dw.w
    out = torch.full(w.query_shape, float("nan"), dtype=torch.float32, device="cuda")
    nb = dw.key_cache.shape[0]
    st = _fn(out.data_ptr(), P.PA_F32, dw.query.data_ptr(), dw.key_cache.data_ptr(),
             dw.value_cache.data_ptr(), P.KV_DTYPE[w.dtype], dw.layout, dw.block_tables.data_ptr(),
             dw.block_tables.shape[1], dw.context_lens.data_ptr(), dw.max_context_len, w.S, w.H,
             w.Hkv, w.D, w.bs, nb, w.scale, part, torch.cuda.current_stream().cuda_stream)
    assert st == 0, (st, P._lib.pa_last_error())
    return out


def _workspace_decode(dw, part):
    w = dw.w
    out = torch.full(w.query_shape, float("nan"), dtype=torch.float32, device="cuda")
    ws = None
    if part != 0:
        nbytes = P.pa_decode_workspace_size(w.S, w.H, w.D, dw.max_context_len, part)
        ws = torch.full((max(nbytes, 16),), 0x5A, dtype=torch.uint8, device="cuda")
    P.pa_decode(out, dw.query, dw.key_cache, dw.value_cache, dw.block_tables, dw.context_lens,
                dw.max_context_len, w.scale, layout=dw.layout, partition_size=part, workspace=ws)
    return out


@pytest.mark.parametrize("G", [1, 8])
def test_static_scratch_decode_matches_pa_decode(G):
    need_gpu()
    big = workloads.make(3, S=24, H=8 * G, Hkv=8, len_median=2000, len_cap=8192)
    small = workloads.make(3, S=5, H=8 * G, Hkv=8, len_median=300, len_cap=900, seed=11)
    for w in (big, small):  # two calls in a row, the second smaller
        announce("static scratch decode", "G", G, "S", w.S, "max len", w.max_context_len)
        dw = M.setup(w, layout=P.HND, write_step=True)
        st = build_state(w)
        kc, vc = build_pool(w, st, layout=P.HND, include_step=True)
        ref = A.decode_ref(w.query, kc, vc, st.block_tables, w.context_lens, w.scale, w.bs,
                           w.dtype, P.HND)
        for part in (-1, 512, 0):
            got = _static(dw, part)
            expect = _workspace_decode(dw, part)
            torch.cuda.synchronize()
            g, e = got.cpu().numpy(), expect.cpu().numpy()
            assert np.array_equal(g, e), (G, w.S, part)
            err, where = max_abs(g, ref)
            announce("partition", part, "max-abs", err)
            assert err <= TOL[w.dtype], (part, err, where)


def test_static_scratch_refuses_oversized_shapes():
    """The long-context shape with 64 sequences at 512-token partitions needs
    about 545 MB of workspace: refused before any device call (null device
    pointers are never touched)."""
    need_gpu()
    S, H, Hkv, D, L, ps = 64, 64, 8, 128, 131072, 512
    need = P.pa_decode_workspace_size(S, H, D, L, ps)
    assert need > SCRATCH
    st = _fn(None, P.PA_F32, None, None, None, P.PA_BF16, P.HND, None, L // 16, None, L, S, H, Hkv,
             D, 16, 1 << 20, 0.088, ps, None)
    assert P.STATUS_NAMES[st] == "PA_ERR_WORKSPACE_TOO_SMALL"
    assert b"static scratch" in P._lib.pa_last_error()
    # the long-context workload itself (8 sequences) fits
    assert P.pa_decode_workspace_size(8, H, D, L, ps) <= SCRATCH
