"""Pins of the FP8 (E4M3) oracle: the code table, rounding, saturation, the
quantising cache write and attention over an FP8 cache.

Independent references: torch's float8_e4m3fn conversions (a library
implementation of the same OCP format; torch does not saturate, so it is
used only within +-448), the format's defining fields, and closed-form
error bounds.
"""
import numpy as np
import torch

from oracle import attention as A
from oracle import fp8

F8 = torch.float8_e4m3fn


def _torch_codes(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(F8).view(torch.uint8).numpy()


def test_table_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(F8).float().numpy().astype(np.float64)
    same = (ref == fp8.E4M3) | (np.isnan(ref) & np.isnan(fp8.E4M3))
    assert same.all()


def test_table_fields():
    T = fp8.E4M3
    assert T[0x38] == 1.0 and T[0xB8] == -1.0
    assert T[0x7E] == 448.0 and T[0xFE] == -448.0
    assert T[0x01] == 2.0 ** -9 and T[0x08] == 2.0 ** -6 and T[0x07] == 7 * 2.0 ** -9
    assert T[0x00] == 0.0 and T[0x80] == 0.0 and np.signbit(T[0x80])
    assert np.isnan(T[0x7F]) and np.isnan(T[0xFF])
    assert np.isfinite(T).sum() == 254
    assert np.all(np.diff(T[:0x7F]) > 0)
    assert np.array_equal(T[0x80:0xFF], -T[0x00:0x7F])


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(100_000) * np.exp(rng.uniform(-13, 6.5, 100_000))).astype(np.float32)
    x = x[np.abs(x) <= fp8.SAT]
    assert len(x) > 90_000
    assert np.array_equal(fp8.e4m3_from_f32(x), _torch_codes(x))


def test_ties_go_to_the_even_code():
    lo, hi = fp8._POS[:-1], fp8._POS[1:]
    mids = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (lo + hi) / 2)  # midpoints exact in fp32
    got = fp8.e4m3_from_f32(np.concatenate([mids, -mids]))
    assert np.all(got[:len(mids)] % 2 == 0)
    assert np.array_equal(got, _torch_codes(np.concatenate([mids, -mids])))
    # worked cases: 1.0625 lies between 1.0 (0x38) and 1.125 (0x39) -> 0x38;
    # 1.1875 between 1.125 and 1.25 (0x3A) -> 0x3A; 2^-10 between 0 and 2^-9 -> 0
    assert list(fp8.e4m3_from_f32(np.array([1.0625, 1.1875, 2.0 ** -10], np.float32))) == [0x38, 0x3A, 0x00]


def test_saturation_nan_and_zero():
    x = np.array([448.0, 449.0, 464.0, 470.0, 1e30, np.inf, -470.0, -np.inf], np.float32)
    assert list(fp8.e4m3_from_f32(x)) == [0x7E] * 6 + [0xFE] * 2
    c = fp8.e4m3_from_f32(np.array([np.nan, -0.0, 0.0, -1e-30, 1e-30], np.float32))
    assert c[0] & 0x7F == 0x7F and list(c[1:]) == [0x80, 0x00, 0x80, 0x00]


def test_nan_elements_keep_their_sign():
    """A NaN element is stored as S.1111.111 with its own sign bit, from every
    source type: 0x7F for a positive NaN, 0xFF for a negative one."""
    f32 = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF800001], np.uint32)
    assert list(fp8.quantize(f32, "f32", 0.37)) == [0x7F, 0xFF, 0x7F, 0xFF]
    bf16 = np.array([0x7FC0, 0xFFC0, 0x7F81, 0xFF81], np.uint16)
    assert list(fp8.quantize(bf16, "bf16", 1.0)) == [0x7F, 0xFF, 0x7F, 0xFF]
    f16 = np.array([0x7E00, 0xFE00, 0x7C01, 0xFC01], np.uint16)
    assert list(fp8.quantize(f16, "f16", 2.5)) == [0x7F, 0xFF, 0x7F, 0xFF]
    # infinities are not NaN: they saturate to +-448 (0x7E / 0xFE)
    assert list(fp8.quantize(np.array([0x7C00, 0xFC00], np.uint16), "f16", 1.0)) == [0x7E, 0xFE]


def test_round_trip_and_error_bound():
    finite = np.flatnonzero(np.isfinite(fp8.E4M3)).astype(np.uint8)
    assert np.array_equal(fp8.e4m3_from_f32(fp8.E4M3[finite].astype(np.float32)), finite)
    rng = np.random.default_rng(3)
    y = (rng.uniform(-1, 1, 200_000) * np.exp(rng.uniform(-14, 6.1, 200_000))).astype(np.float32)
    y = y[np.abs(y) <= fp8.SAT]
    back = fp8.E4M3[fp8.e4m3_from_f32(y)]
    err = np.abs(back - y.astype(np.float64))
    normal = np.abs(y) >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(y[normal]))  # half a 3-bit ulp
    assert np.all(err[~normal] <= 2.0 ** -10)                     # half the subnormal step


def test_quantize_divides_in_fp32():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(50_000).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)  # bf16 by truncation: any bf16 values do
    scale = np.float32(0.0171)
    xf = (bits.astype(np.uint32) << 16).view(np.float32)
    ref = _torch_codes((torch.from_numpy(xf) / torch.tensor(scale)).numpy())
    assert np.array_equal(fp8.quantize(bits, "bf16", scale), ref)
    # dequantised values stay within half a step of x
    back = fp8.dequantize(fp8.quantize(bits, "bf16", scale), scale)
    assert np.all(np.abs(back - xf) <= 2.0 ** -4 * np.abs(xf) + 2.0 ** -10 * float(scale))


def test_write_ref_fp8_quantises_and_scatters():
    rng = np.random.default_rng(5)
    NB, bs, Hkv, D = 4, 8, 2, 16
    kc = np.full((NB, bs, Hkv, D), 0xFF, np.uint8)
    vc = kc.copy()
    T = 5
    k = (rng.standard_normal((T, Hkv, D)) * 3).astype(np.float32)
    v = (rng.standard_normal((T, Hkv, D)) * 3).astype(np.float32)
    slots = np.array([9, -1, 30, 0, -1], np.int64)
    ks, vs = np.float32(0.005), np.float32(0.5)
    nk, nv = A.write_ref_fp8(kc, vc, k, v, slots, bs, "f32", ks, vs, A.NHD)
    for i, s in enumerate(slots):
        if s >= 0:
            b, o = divmod(int(s), bs)
            assert np.array_equal(nk[b, o], fp8.e4m3_from_f32(k[i] / ks))
            assert np.array_equal(nv[b, o], fp8.e4m3_from_f32(v[i] / vs))
    written = np.zeros((NB, bs), bool)
    for s in slots[slots >= 0]:
        written[divmod(int(s), bs)] = True
    assert np.all(nk[~written] == 0xFF) and np.all(nv[~written] == 0xFF)
    assert np.any(nk[written] == 0x7E) or np.any(nk[written] == 0xFE)  # k / 0.005 saturates somewhere


def test_decode_over_fp8_equals_decode_over_the_same_values_in_bf16():
    """With power-of-two scales every dequantised value is exact in bf16, so
    attention over the FP8 cache must equal attention over a bf16 cache that
    holds those values (checks the read-back and the scale wiring)."""
    rng = np.random.default_rng(9)
    NB, bs, Hkv, D, S, G = 6, 16, 2, 32, 3, 2
    finite = np.flatnonzero(np.isfinite(fp8.E4M3) & (np.abs(fp8.E4M3) <= 16)).astype(np.uint8)
    kc = rng.choice(finite, (NB, bs, Hkv, D)).astype(np.uint8)
    vc = rng.choice(finite, (NB, bs, Hkv, D)).astype(np.uint8)
    ks, vs = 2.0 ** -3, 2.0 ** 2

    def bf16_bits(vals):
        b = vals.astype(np.float32).view(np.uint32)
        assert np.all(b & 0xFFFF == 0)
        return (b >> 16).astype(np.uint16)

    kb, vb = bf16_bits(fp8.E4M3[kc] * ks), bf16_bits(fp8.E4M3[vc] * vs)
    q = bf16_bits(np.round(rng.standard_normal((S, Hkv * G, D)) * 8) / 8)
    bt = np.stack([rng.permutation(NB)[:4] for _ in range(S)]).astype(np.int32)
    lens = np.array([1, 37, 64], np.int32)
    scale = 1 / np.sqrt(D)
    a = A.decode_ref(q, kc, vc, bt, lens, scale, bs, "bf16", kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    b = A.decode_ref(q, kb, vb, bt, lens, scale, bs, "bf16")
    assert np.array_equal(a, b)
    # the scales matter: a wrong v_scale changes the result
    c = A.decode_ref(q, kc, vc, bt, lens, scale, bs, "bf16", kv_dtype="e4m3", k_scale=ks, v_scale=1.0)
    assert not np.array_equal(c, b)
