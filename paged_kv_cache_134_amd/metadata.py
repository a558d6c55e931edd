"""Device-side metadata and cache set-up for seeded workloads.

Builds, with the library only, what one step of the hot path consumes:
block tables and slot mappings from the host block pool (pa_pool_*), the K/V
pools filled through pa_reshape_and_cache and pa_copy_blocks, and the step's
inputs (new K/V rows, their slot_mapping, queries, lengths, packed offsets).
The block manager's role follows the "Paged attention" post (k4i.top, block
manager and copy-on-write sections) and the metadata fields the
CommonAttentionMetadata of "PagedAttention 在 vLLM 中的实现分析" §5.4.

Pools hold NB + 1 blocks; the last one (id NB) is a poison block that pads
every block table.  Every slot starts as all-ones bits (NaN for float32,
bfloat16 and float16), so a kernel that reads an unwritten slot, a tail slot
past a context or a padding table entry produces NaN.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

from . import NHD, BlockPool, pa_copy_blocks, pa_reshape_and_cache, pa_reshape_and_cache_fp8

_CHUNK_ROWS = 16384  # rows per set-up upload


def _torch():
    import torch
    return torch


def torch_dtype(name: str):
    torch = _torch()
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[name]


def to_device(raw: np.ndarray, dtype: str, device="cuda"):
    """Upload raw values (float32, or uint16 bits of bf16/f16) as a typed tensor."""
    torch = _torch()
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(raw, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).to(device)
    return t.view(torch_dtype(dtype))


def nan_pool(shape, dtype: str, device="cuda"):
    torch = _torch()
    if dtype == "e4m3":  # code 0xFF is NaN
        return torch.full(shape, 255, dtype=torch.uint8, device=device)
    if dtype == "f32":
        return torch.full(shape, -1, dtype=torch.int32, device=device).view(torch.float32)
    return torch.full(shape, -1, dtype=torch.int16, device=device).view(torch_dtype(dtype))


@dataclass
class DeviceWorkload:
    w: object                      # workloads.Workload
    layout: int
    pool: BlockPool
    seq_ids: List[int]
    seq_slots: List[np.ndarray]    # host: slot of every position of every sequence
    copies: List[Tuple[int, int]]
    block_tables_host: np.ndarray  # int32 [S, max_blocks]
    key_cache: object = None
    value_cache: object = None
    block_tables: object = None    # device int32 [S, max_blocks]
    context_lens: object = None    # device int32 [S]
    step_k: object = None          # device [T, Hkv, D]
    step_v: object = None
    step_slots: object = None      # device int64 [T]
    step_slots_host: Optional[np.ndarray] = None
    query: object = None
    query_start_loc: object = None  # device int32 [S+1] (prefill)
    kv_dtype: Optional[str] = None  # "e4m3": FP8 pools written by the quantising write
    k_scale: float = 1.0
    v_scale: float = 1.0
    notes: dict = field(default_factory=dict)

    @property
    def max_context_len(self) -> int:
        return int(self.w.context_lens.max()) if self.w.S else 0

    @property
    def num_blocks(self) -> int:
        return self.w.NB + 1


def allocate(w, max_blocks: Optional[int] = None):
    """Run the block pool for workload w: returns (pool, seq ids, per-sequence
    slots, copy-on-write pairs, padded block tables)."""
    pool = BlockPool(w.NB, w.bs, w.free_order)
    S, P = w.S, w.prefix_len
    lens = [int(x) for x in w.context_lens]
    copies: List[Tuple[int, int]] = []
    seq_slots: List[np.ndarray] = []
    if P:
        parent = pool.add_seq()
        ps, _ = pool.append(parent, P)
        sids = [parent] + [pool.fork(parent) for _ in range(S - 1)]
        for s, sid in enumerate(sids):
            sl, cow = pool.append(sid, lens[s] - P)
            copies.extend(cow)
            seq_slots.append(np.concatenate([ps, sl]))
    else:
        sids = []
        for s in range(S):
            sid = pool.add_seq()
            sl, _ = pool.append(sid, lens[s])
            seq_slots.append(sl)
            sids.append(sid)
    tabs = [pool.block_table(sid) for sid in sids]
    nb = max((len(t) for t in tabs), default=0)
    mb = nb if max_blocks is None else max_blocks
    if mb < nb:
        raise ValueError("max_blocks smaller than the longest table")
    bt = np.full((S, max(mb, 1)), w.NB, np.int32)
    for s, t in enumerate(tabs):
        bt[s, :len(t)] = t
    return pool, sids, seq_slots, copies, bt


def _write_rows(dw: "DeviceWorkload", k: np.ndarray, v: np.ndarray, slots: np.ndarray) -> None:
    torch = _torch()
    w = dw.w
    for a in range(0, len(slots), _CHUNK_ROWS):
        b = min(len(slots), a + _CHUNK_ROWS)
        kd = to_device(k[a:b], w.dtype)
        vd = to_device(v[a:b], w.dtype)
        sd = torch.from_numpy(np.ascontiguousarray(slots[a:b], dtype=np.int64)).cuda()
        _write(dw, kd, vd, sd)


def _write(dw: "DeviceWorkload", k, v, slots) -> None:
    if dw.kv_dtype == "e4m3":
        pa_reshape_and_cache_fp8(k, v, dw.key_cache, dw.value_cache, slots, dw.k_scale,
                                 dw.v_scale, dw.layout)
    else:
        pa_reshape_and_cache(k, v, dw.key_cache, dw.value_cache, slots, dw.layout)


def setup(w, layout: int = NHD, write_step: bool = False, max_blocks: Optional[int] = None,
          device="cuda", kv_dtype: Optional[str] = None, k_scale: float = 1.0,
          v_scale: float = 1.0) -> DeviceWorkload:
    """Allocate, fill the pools with every position that is not a row of the
    step, and stage the step's inputs on the device.  kv_dtype "e4m3": FP8
    pools, every row written by the quantising write with k_scale / v_scale
    (queries and new rows keep the workload's dtype)."""
    torch = _torch()
    pool, sids, seq_slots, copies, bt = allocate(w, max_blocks)
    dw = DeviceWorkload(w=w, layout=layout, pool=pool, seq_ids=sids, seq_slots=seq_slots,
                        copies=copies, block_tables_host=bt, kv_dtype=kv_dtype,
                        k_scale=float(k_scale), v_scale=float(v_scale))
    shape = ((w.NB + 1, w.bs, w.Hkv, w.D) if layout == NHD else (w.NB + 1, w.Hkv, w.bs, w.D))
    dw.key_cache = nan_pool(shape, kv_dtype or w.dtype, device)
    dw.value_cache = nan_pool(shape, kv_dtype or w.dtype, device)
    # step rows and their slots
    step = np.full(w.T, -1, np.int64)
    step_pos = {}
    for r in range(w.T):
        s = int(w.row_seq[r])
        if s >= 0:
            step[r] = seq_slots[s][int(w.row_pos[r])]
            step_pos.setdefault(s, []).append(int(w.row_pos[r]))
    # shared prefix once, then copy-on-write copies, then each sequence's own positions
    P = w.prefix_len
    if P:
        for a in range(0, P, _CHUNK_ROWS):
            b = min(P, a + _CHUNK_ROWS)
            k, v = w.kv(0, a, b)
            _write_rows(dw, k, v, seq_slots[0][a:b])
    if copies:
        pairs = torch.from_numpy(np.asarray(copies, np.int32).reshape(-1, 2)).to(device)
        pa_copy_blocks(dw.key_cache, dw.value_cache, pairs, layout)
    for s in range(w.S):
        L = int(w.context_lens[s])
        skip = set(step_pos.get(s, ()))
        a = P
        while a < L:
            b = min(L, a + _CHUNK_ROWS)
            pos = np.arange(a, b)
            if skip:
                pos = pos[~np.isin(pos, list(skip))]
            if len(pos):
                k, v = w.kv(s, a, b)
                _write_rows(dw, k[pos - a], v[pos - a], seq_slots[s][pos])
            a = b
    K, V = w.new_rows()
    dw.step_k = to_device(K, w.dtype, device)
    dw.step_v = to_device(V, w.dtype, device)
    dw.step_slots_host = step
    dw.step_slots = torch.from_numpy(step).to(device)
    dw.block_tables = torch.from_numpy(bt).to(device)
    dw.context_lens = torch.from_numpy(np.asarray(w.context_lens, np.int32)).to(device)
    dw.query = to_device(w.query, w.dtype, device)
    if w.query_start_loc is not None:
        dw.query_start_loc = torch.from_numpy(np.asarray(w.query_start_loc, np.int32)).to(device)
    if write_step:
        write_step_rows(dw)
    return dw


def write_step_rows(dw: DeviceWorkload) -> None:
    """The step's cache write: the new rows through their slot_mapping."""
    _write(dw, dw.step_k, dw.step_v, dw.step_slots)
