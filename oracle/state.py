"""Oracle-side construction of a workload's block tables, slot mappings and pool.

TEST INFRASTRUCTURE ONLY (see the package docstring).

From the seeded draws of ``workloads.Workload`` this derives, with the
allocator model and ``write_ref`` only:

* every sequence's block table and the slot of each of its positions;
* the copy-on-write block copies that sharing a prefix causes;
* the step's ``slot_mapping`` (padding rows get -1);
* optionally the host pool after set-up and after the step's write.

Set-up order: the shared prefix (if any) is written once through the first
sequence's slots; the other sequences fork it; every sequence then appends
its own tokens (the first append into the prefix's partly filled last block
copies it, see the allocator model); the copies are applied; then every
position that is not a row of the step is written.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

import numpy as np

from .allocator import BlockManagerModel
from .attention import NHD, write_ref, write_ref_fp8


@dataclass
class OracleState:
    block_tables: np.ndarray        # int32 [S, max_blocks], unused entries = poison block id
    seq_slots: List[np.ndarray]     # per sequence: int64 slot of positions 0..L-1
    copies: List[Tuple[int, int]]   # copy-on-write (src, dst) block copies, in order
    step_slots: np.ndarray          # int64 [T] slot_mapping of the step's rows
    setup_positions: List[np.ndarray]  # per sequence: private positions written at set-up
    prefix_slots: Optional[np.ndarray]  # slots of the shared prefix (written once)
    poison: int                     # id of the all-NaN block that pads the tables
    model: BlockManagerModel


def build_state(w, max_blocks: Optional[int] = None) -> OracleState:
    model = BlockManagerModel(w.NB, w.bs, w.free_order)
    S, P = w.S, w.prefix_len
    lens = [int(x) for x in w.context_lens]
    copies: List[Tuple[int, int]] = []
    seq_slots: List[np.ndarray] = [None] * S
    prefix_slots = None
    if P:
        parent = model.add_seq()
        ps, _ = model.append(parent, P)
        prefix_slots = np.asarray(ps, np.int64)
        sids = [parent] + [model.fork(parent) for _ in range(S - 1)]
        for s, sid in enumerate(sids):
            sl, cow = model.append(sid, lens[s] - P)
            copies.extend(cow)
            seq_slots[s] = np.concatenate([prefix_slots, np.asarray(sl, np.int64)])
    else:
        sids = []
        for s in range(S):
            sid = model.add_seq()
            sl, _ = model.append(sid, lens[s])
            seq_slots[s] = np.asarray(sl, np.int64)
            sids.append(sid)
    nb = max((len(model.tables[sid]) for sid in sids), default=0)
    mb = nb if max_blocks is None else max_blocks
    assert mb >= nb
    poison = w.NB
    bt = np.full((S, max(mb, 1)), poison, np.int32)
    for s, sid in enumerate(sids):
        tab = model.tables[sid]
        bt[s, :len(tab)] = tab
    # the step's rows
    step = np.full(w.T, -1, np.int64)
    step_pos: Dict[int, set] = {}
    for r in range(w.T):
        s = int(w.row_seq[r])
        if s >= 0:
            step[r] = seq_slots[s][int(w.row_pos[r])]
            step_pos.setdefault(s, set()).add(int(w.row_pos[r]))
    setup_positions = []
    for s in range(S):
        pos = np.arange(P, lens[s])
        if s in step_pos:
            pos = pos[~np.isin(pos, list(step_pos[s]))]
        setup_positions.append(pos.astype(np.int64))
    return OracleState(bt, seq_slots, copies, step, setup_positions, prefix_slots, poison, model)


def empty_pool(w, layout=NHD, kv_dtype=None) -> np.ndarray:
    """All-NaN pool of NB + 1 blocks (the extra one is the poison block);
    all-ones bits are NaN in every element type, E4M3 codes included."""
    raw = np.uint8 if kv_dtype == "e4m3" else np.uint32 if w.dtype == "f32" else np.uint16
    shape = (w.NB + 1, w.bs, w.Hkv, w.D) if layout == NHD else (w.NB + 1, w.Hkv, w.bs, w.D)
    return np.full(shape, np.iinfo(raw).max, dtype=raw)


def build_pool(w, st: OracleState, layout=NHD, include_step: bool = False, seqs=None,
               kv_dtype=None, k_scale=1.0, v_scale=1.0):
    """Host K and V pools after set-up (and after the step's write if asked).

    ``seqs`` restricts the per-sequence writes (and the step rows) to those
    sequences; the shared prefix and the copies are always applied.
    ``kv_dtype`` "e4m3": every write quantises (``write_ref_fp8``) into pools
    of E4M3 codes.
    """
    def write(kc, vc, k, v, slots, bs, lay):
        if kv_dtype == "e4m3":
            return write_ref_fp8(kc, vc, k, v, slots, bs, w.dtype, k_scale, v_scale, lay)
        return write_ref(kc, vc, k, v, slots, bs, lay)

    kc, vc = empty_pool(w, layout, kv_dtype), empty_pool(w, layout, kv_dtype)
    if st.prefix_slots is not None:
        k, v = w.kv(0, 0, w.prefix_len)
        kc, vc = write(kc, vc, k, v, st.prefix_slots, w.bs, layout)
    for src, dst in st.copies:
        kc[dst] = kc[src]
        vc[dst] = vc[src]
    ks, vs, ss = [], [], []
    for s in (range(w.S) if seqs is None else seqs):
        pos = st.setup_positions[s]
        if len(pos) == 0:
            continue
        lo, hi = int(pos.min()), int(pos.max()) + 1
        k, v = w.kv(s, lo, hi)
        ks.append(k[pos - lo])
        vs.append(v[pos - lo])
        ss.append(st.seq_slots[s][pos])
    if ss:
        kc, vc = write(kc, vc, np.concatenate(ks), np.concatenate(vs), np.concatenate(ss),
                       w.bs, layout)
    if include_step:
        K, V = w.new_rows()
        slots = st.step_slots.copy()
        if seqs is not None:
            slots[~np.isin(w.row_seq, list(seqs))] = -1
        kc, vc = write(kc, vc, K, V, slots, w.bs, layout)
    return kc, vc
