"""The seeded generator: determinism, first-draw sums, encodings (CPU only)."""
import numpy as np

import workloads


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20,
                  3.14159265], np.float32)
    assert list(workloads.f32_to_bf16_bits(x)) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81, 0x4049]


def test_first_draw_sums():
    assert int(workloads.make(2).context_lens.sum()) == 75661
    assert int(workloads.make(3).context_lens.sum()) == 207090
    assert int(workloads.make("5c").notes["suffix_lens"].sum()) == 25952
    w1 = workloads.make(1)
    assert list(w1.context_lens) == [1, 17, 130, 300] and w1.NB == 128


def test_determinism_and_streams():
    a, b = workloads.make(2, S=5), workloads.make(2, S=5)
    assert np.array_equal(a.query, b.query)
    assert np.array_equal(a.free_order, b.free_order)
    ka, va = a.kv(3)
    kb, vb = b.kv(3)
    assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    # a slice of a stream equals the same positions of the whole stream
    k_part, _ = a.kv(3, 10, 20)
    assert np.array_equal(k_part, ka[10:20])


def test_decode_rows_and_padding():
    w = workloads.make(2)
    assert w.T == 71 and int((w.row_seq < 0).sum()) == 7
    real = w.row_seq >= 0
    assert sorted(w.row_seq[real]) == list(range(64))
    assert np.array_equal(w.row_pos[real], w.context_lens[w.row_seq[real]] - 1)
    K, V = w.new_rows()
    s, r = int(w.row_seq[real][0]), int(np.where(real)[0][0])
    k, v = w.kv(s, w.context_lens[s] - 1)
    assert np.array_equal(K[r], k[0]) and np.array_equal(V[r], v[0])


def test_shared_prefix_positions_come_from_one_stream():
    w = workloads.make("5c", S=3, prefix=300, suffix_lo=5, suffix_hi=9, bs=16)
    k0, _ = w.kv(0, 0, 300)
    k2, _ = w.kv(2, 0, 300)
    assert np.array_equal(k0, k2)
    assert w.query.shape[0] == int(w.query_start_loc[-1])
    assert np.array_equal(np.diff(w.query_start_loc), w.notes["suffix_lens"])


def test_packed_prefill_lengths():
    w = workloads.make("5b")
    assert list(w.query_start_loc) == [0, 85, 205, 250, 460]
    assert np.array_equal(w.context_lens, [85, 120, 45, 210])
