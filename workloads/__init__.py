"""Seeded synthetic inputs shared by the HIP path's tests/bench and by the oracle.

This module only *draws* inputs: lengths, the order in which pool blocks are
handed out, query values, per-sequence logical K/V values, padding rows.  It
holds none of the paged-attention arithmetic: no slot computation, no block
table, no scatter and no softmax.  Both sides build their own block tables and
slot mappings from these draws (the product through its C++ block allocator,
the oracle through its own allocator model) and the tests compare the two.

Values follow the workloads named for the method (decode of 7B-like and
70B-like layers, long-context split-K decode, shared-prefix + packed prefill):
N(0, 1) drawn in float32, rounded to bfloat16 (round-to-nearest-even) for the
bf16 workloads.  Per-sequence K/V values come from child streams
``default_rng([seed, tag, seq, chunk])``, one per CHUNK positions, and the
queries from ``default_rng([seed, tag])``, so any slice of any sequence can be
re-drawn alone, at any size, without drawing the rest.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

# stream tags for the child generators
_TAG_K, _TAG_V, _TAG_PAD, _TAG_Q = 1, 2, 3, 4
_TAG_PREFIX = 1 << 20  # sequence index used for the shared prefix stream
CHUNK = 128            # positions per K/V child stream

F32, BF16 = "f32", "bf16"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    Inputs here are finite N(0,1) draws, so NaN/Inf handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def _normal(rng: np.random.Generator, shape, dtype: str, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x = x * np.float32(std)
    return x if dtype == F32 else f32_to_bf16_bits(x)


# FP8 (E4M3) cache scales used with these standard-normal K/V draws: x / scale
# stays below the format's 448 up to |x| = 7.7 (keys) and 6.9 (values)
# standard deviations.
FP8_K_SCALE = 0.0171
FP8_V_SCALE = 0.0153


@dataclass
class Workload:
    """One seeded synthetic workload.

    Raw arrays are float32 (dtype "f32") or uint16 bfloat16 bit patterns
    (dtype "bf16").  Shapes use S = sequences, H = query heads, Hkv = kv heads,
    D = head size, bs = block size (tokens per block), NB = usable pool blocks.
    """

    cfg: int
    name: str
    kind: str                 # "decode" or "prefill"
    dtype: str
    seed: int
    S: int
    H: int
    Hkv: int
    D: int
    bs: int
    NB: int                   # usable blocks; the pool tensor has NB + 1 blocks (last = poison)
    context_lens: np.ndarray  # int32 [S]: tokens attended (decode: includes the new token)
    free_order: np.ndarray    # int32 [NB]: order in which the allocator hands out blocks
    query_shape: Tuple[int, int, int]  # [S, H, D] (decode) or [T, H, D] packed (prefill)
    # decode: write rows (new tokens + padding); prefill: packed new tokens
    row_seq: np.ndarray       # int32 [T]: sequence of each new-token row, -1 for padding
    row_pos: np.ndarray       # int32 [T]: absolute position of the row's token, -1 for padding
    pad_k: np.ndarray         # [T_pad, Hkv, D] garbage rows for padding (same dtype)
    pad_v: np.ndarray
    query_start_loc: Optional[np.ndarray] = None  # int32 [S+1] packed offsets (prefill)
    prefix_len: int = 0       # shared prefix length (all sequences share it), 0 = none
    partition_size: int = 0   # split-K partition size named by the workload (0 = none)
    v_std: float = 1.0        # V drawn from N(0, v_std^2) (a power of two keeps bf16 exact)
    notes: Dict[str, object] = field(default_factory=dict)
    _query: Optional[np.ndarray] = field(default=None, repr=False)

    # ------------------------------------------------------------------ K/V
    def kv(self, s: int, lo: int = 0, hi: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
        """Logical K and V of sequence s for positions [lo, hi): arrays [n, Hkv, D].

        Positions below ``prefix_len`` come from the shared prefix streams, the
        rest from the sequence's own streams (position prefix_len is its row 0).
        Each stream covers CHUNK positions, so a slice draws only what it needs.
        """
        L = int(self.context_lens[s])
        hi = L if hi is None else int(hi)
        lo = int(lo)
        assert 0 <= lo <= hi <= L
        P = self.prefix_len
        parts_k, parts_v = [], []
        if lo < P:
            k, v = self._range(_TAG_PREFIX, lo, min(hi, P))
            parts_k.append(k)
            parts_v.append(v)
        if hi > P:
            k, v = self._range(s, max(lo, P) - P, hi - P)
            parts_k.append(k)
            parts_v.append(v)
        if len(parts_k) == 1:
            return parts_k[0], parts_v[0]
        if not parts_k:
            return self._range(s, 0, 0)
        return np.concatenate(parts_k), np.concatenate(parts_v)

    def _range(self, idx: int, lo: int, hi: int):
        dt = np.float32 if self.dtype == F32 else np.uint16
        n = hi - lo
        K = np.empty((n, self.Hkv, self.D), dt)
        V = np.empty((n, self.Hkv, self.D), dt)
        c = lo // CHUNK
        while c * CHUNK < hi:
            a, b = c * CHUNK, (c + 1) * CHUNK
            shape = (CHUNK, self.Hkv, self.D)
            k = _normal(np.random.default_rng([self.seed, _TAG_K, idx, c]), shape, self.dtype)
            v = _normal(np.random.default_rng([self.seed, _TAG_V, idx, c]), shape, self.dtype,
                        self.v_std)
            x0, x1 = max(a, lo), min(b, hi)
            K[x0 - lo:x1 - lo] = k[x0 - a:x1 - a]
            V[x0 - lo:x1 - lo] = v[x0 - a:x1 - a]
            c += 1
        return K, V

    @property
    def query(self) -> np.ndarray:
        """Queries, drawn from their own stream (cached after the first use)."""
        if self._query is None:
            self._query = _normal(np.random.default_rng([self.seed, _TAG_Q]), self.query_shape,
                                  self.dtype)
        return self._query

    # ------------------------------------------------------------ new rows
    def new_rows(self) -> Tuple[np.ndarray, np.ndarray]:
        """K and V rows [T, Hkv, D] of this step's new tokens in row order (padding included)."""
        T = len(self.row_seq)
        shape = (T, self.Hkv, self.D)
        dt = np.float32 if self.dtype == F32 else np.uint16
        K = np.empty(shape, dt)
        V = np.empty(shape, dt)
        pad_i = 0
        # group real rows per sequence so each sequence stream is drawn once
        by_seq: Dict[int, List[int]] = {}
        for r in range(T):
            s = int(self.row_seq[r])
            if s < 0:
                K[r] = self.pad_k[pad_i]
                V[r] = self.pad_v[pad_i]
                pad_i += 1
            else:
                by_seq.setdefault(s, []).append(r)
        for s, rows in by_seq.items():
            pos = self.row_pos[rows]
            lo, hi = int(pos.min()), int(pos.max()) + 1
            k, v = self.kv(s, lo, hi)
            K[rows] = k[pos - lo]
            V[rows] = v[pos - lo]
        return K, V

    @property
    def T(self) -> int:
        return int(len(self.row_seq))

    @property
    def G(self) -> int:
        return self.H // self.Hkv

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(head_size), as the float32 value both sides use."""
        return float(np.float32(1.0 / math.sqrt(self.D)))

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.S else 0

    @property
    def query_lens(self) -> np.ndarray:
        assert self.query_start_loc is not None
        return np.diff(self.query_start_loc).astype(np.int32)


def _pool_blocks(lens: np.ndarray, bs: int, factor: float = 1.2) -> int:
    """Pool sizing: ``factor`` times the blocks the sequences need (rounded up)."""
    need = int(sum(-(-int(L) // bs) for L in lens))
    return int(math.ceil(factor * need))


def _decode_rows(rng, S, lens, n_pad):
    """Write rows for a decode step: one new token per sequence (its last
    position) plus ``n_pad`` padding rows, in a seeded shuffled order."""
    T = S + n_pad
    order = rng.permutation(T)
    row_seq = np.full(T, -1, np.int32)
    row_pos = np.full(T, -1, np.int32)
    for r, src in enumerate(order):
        if src < S:
            row_seq[r] = src
            row_pos[r] = lens[src] - 1
    return row_seq, row_pos


def make(cfg: int, seed: Optional[int] = None, **over) -> Workload:
    """Build workload ``cfg`` (1..5 plus the cfg-5 variants "5a", "5b", "5c").

    ``over`` scales a workload down for tests (e.g. S=8) while keeping its
    structure; any key of the config table may be overridden.
    """
    spec = dict(CONFIGS[cfg])
    spec.update(over)
    seed = spec.get("seed", _default_seed(cfg)) if seed is None else seed
    return spec["builder"](cfg, seed, spec)


def _default_seed(cfg) -> int:
    return int(str(cfg)[0])


def _build_decode(cfg, seed, sp) -> Workload:
    rng = np.random.default_rng(seed)
    S = sp["S"]
    # 1. lengths
    lens = sp["lens_fn"](rng, S, sp)
    lens = np.asarray(lens, dtype=np.int32)
    # 2. pool and the allocator's free order
    NB = sp.get("pool_blocks") or _pool_blocks(lens, sp["bs"], sp.get("pool_factor", 1.2))
    free_order = rng.permutation(NB).astype(np.int32)
    # 3. new-token rows and padding rows (queries and K/V come from child streams)
    n_pad = int(sp.get("n_pad", 0))
    row_seq, row_pos = _decode_rows(rng, S, lens, n_pad)
    prng = np.random.default_rng([seed, _TAG_PAD])
    pad_k = _normal(prng, (n_pad, sp["Hkv"], sp["D"]), sp["dtype"])
    pad_v = _normal(prng, (n_pad, sp["Hkv"], sp["D"]), sp["dtype"])
    return Workload(cfg=cfg, name=sp["name"], kind="decode", dtype=sp["dtype"], seed=seed,
                    S=S, H=sp["H"], Hkv=sp["Hkv"], D=sp["D"], bs=sp["bs"], NB=NB,
                    context_lens=lens, free_order=free_order, query_shape=(S, sp["H"], sp["D"]),
                    row_seq=row_seq, row_pos=row_pos, pad_k=pad_k, pad_v=pad_v,
                    partition_size=int(sp.get("partition_size", 0)),
                    v_std=float(sp.get("v_std", 1.0)))


def _build_shared(cfg, seed, sp) -> Workload:
    """Shared-prefix workloads: every sequence starts with the same ``prefix``
    tokens (physically shared blocks, refcount = number of sequences), then a
    private suffix of U[lo, hi] tokens.  Variants:

    * "5a": decode step, the new token is each suffix's last token;
    * "5c": packed prefill of all suffix tokens over the cached prefix;
    * "5b": packed prefill of fresh prompts with the lengths printed for the
      packed format (no prefix).
    """
    rng = np.random.default_rng(seed)
    variant = sp["variant"]
    H, Hkv, D, bs = sp["H"], sp["Hkv"], sp["D"], sp["bs"]
    if variant == "5b":
        qlens = np.asarray(sp["packed_lens"], dtype=np.int32)
        S = len(qlens)
        lens = qlens.copy()
        prefix = 0
    else:
        S = sp["S"]
        qlens = rng.integers(sp["suffix_lo"], sp["suffix_hi"] + 1, S).astype(np.int32)
        prefix = sp["prefix"]
        lens = (prefix + qlens).astype(np.int32)
    # pool: blocks held after every sequence appended its suffix (prefix held once)
    if prefix:
        pb = -(-prefix // bs)
        need = pb + sum(-(-int(L) // bs) - (prefix // bs) for L in lens)
    else:
        need = sum(-(-int(L) // bs) for L in lens)
    NB = sp.get("pool_blocks") or int(math.ceil(sp.get("pool_factor", 1.2) * need))
    free_order = rng.permutation(NB).astype(np.int32)
    qsl = np.zeros(S + 1, np.int32)
    qsl[1:] = np.cumsum(qlens)
    if variant == "5a":
        qshape = (S, H, D)
        row_seq = np.arange(S, dtype=np.int32)
        row_pos = (lens - 1).astype(np.int32)
        kind, q_start = "decode", None
    else:
        qshape = (int(qsl[-1]), H, D)
        row_seq = np.repeat(np.arange(S, dtype=np.int32), qlens)
        row_pos = np.concatenate([np.arange(L - n, L, dtype=np.int32)
                                  for L, n in zip(lens, qlens)]) if S else np.zeros(0, np.int32)
        kind, q_start = "prefill", qsl
    empty = np.zeros((0, Hkv, D), np.uint16 if sp["dtype"] == BF16 else np.float32)
    return Workload(cfg=cfg, name=sp["name"], kind=kind, dtype=sp["dtype"], seed=seed,
                    S=S, H=H, Hkv=Hkv, D=D, bs=bs, NB=NB, context_lens=lens,
                    free_order=free_order, query_shape=qshape, row_seq=row_seq, row_pos=row_pos,
                    pad_k=empty, pad_v=empty, query_start_loc=q_start, prefix_len=prefix,
                    notes={"suffix_lens": qlens}, v_std=float(sp.get("v_std", 1.0)))


def _lens_fixed(rng, S, sp):
    return np.asarray(sp["lens"], dtype=np.int32)


def _lens_uniform(rng, S, sp):
    return rng.integers(sp["len_lo"], sp["len_hi"] + 1, S)


def _lens_lognormal(rng, S, sp):
    x = np.exp(rng.normal(math.log(sp["len_median"]), sp["len_sigma"], S))
    return np.clip(np.rint(x), 1, sp["len_cap"]).astype(np.int64)


CONFIGS = {
    1: dict(name="tiny-decode", builder=_build_decode, dtype=F32, S=4, H=8, Hkv=8, D=64, bs=16,
            lens_fn=_lens_fixed, lens=[1, 17, 130, 300], pool_blocks=128),
    2: dict(name="7b-mha-decode", builder=_build_decode, dtype=BF16, S=64, H=32, Hkv=32, D=128,
            bs=16, lens_fn=_lens_uniform, len_lo=200, len_hi=2048, n_pad=7),
    3: dict(name="70b-gqa-decode", builder=_build_decode, dtype=BF16, S=128, H=64, Hkv=8, D=128,
            bs=32, lens_fn=_lens_lognormal, len_median=1024, len_sigma=1.0, len_cap=8192),
    4: dict(name="long-context-splitk-decode", builder=_build_decode, dtype=BF16, S=8, H=64, Hkv=8,
            D=128, bs=16, lens_fn=_lens_fixed, lens=[131072] * 8, partition_size=512),
    "5a": dict(name="shared-prefix-decode", builder=_build_shared, variant="5a", dtype=BF16, S=100,
               H=32, Hkv=32, D=128, bs=256, prefix=2000, suffix_lo=50, suffix_hi=500),
    "5b": dict(name="packed-prefill", builder=_build_shared, variant="5b", dtype=BF16, H=32, Hkv=32,
               D=128, bs=256, packed_lens=[85, 120, 45, 210]),
    "5c": dict(name="prefix-cached-suffix-prefill", builder=_build_shared, variant="5c", dtype=BF16,
               S=100, H=32, Hkv=32, D=128, bs=256, prefix=2000, suffix_lo=50, suffix_hi=500),
}
CONFIGS[5] = CONFIGS["5c"]
