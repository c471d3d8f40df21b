"""Pins of the oracle's fused producers (rotary embedding + fp8 quantiser +
cache write, query scale folded into the head weights) against hand-worked
values, complex multiplication, identity tables and invariants.  CPU only."""
import numpy as np

import oracle as O
from sparse_attention_indexer_paged_amd import synth


def _tables(P, rope_dim, base=10000.0):
    """Unit-circle tables cos(p * f_i), sin(p * f_i), f_i = base^(-2i/rope_dim),
    computed in float64 and rounded to float32 (a test input, any angles do)."""
    half = rope_dim // 2
    f = base ** (-2.0 * np.arange(half) / max(rope_dim, 1))
    ang = np.arange(P)[:, None] * f[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def test_rotation_hand_worked():
    # pair 0 (1, 2) by 90 degrees -> (-2, 1); pair 1 (3, 4) identity
    x = np.arange(1, 9, dtype=np.float32)[None, :]
    c = np.array([[0.0, 1.0]], np.float32)
    s = np.array([[1.0, 0.0]], np.float32)
    assert O.rope_rotate(x, [0], c, s, 4).tolist() == [[-2, 1, 3, 4, 5, 6, 7, 8]]
    # exact binary fractions: (2, 4) with cos 0.5, sin 0.75 -> (1 - 3, 2 + 1.5)
    x = np.array([[2.0, 4.0, 9.0]], np.float32)
    y = O.rope_rotate(x, [0], np.array([[0.5]], np.float32), np.array([[0.75]], np.float32), 2)
    assert y.tolist() == [[-2.0, 3.5, 9.0]]


def test_rotation_equals_complex_multiplication():
    """(x1 + i x2)(cos + i sin) in complex128, rounded to float32, is the
    rotation; the float32 steps may differ from it by the rounding of two
    products and one sum (<= 3 ulp of the larger term)."""
    rng = np.random.default_rng(0)
    T, L, rope_dim, P = 50, 128, 64, 300
    x = rng.standard_normal((T, L)).astype(np.float32)
    pos = rng.integers(0, P, T)
    c, s = _tables(P, rope_dim)
    y = O.rope_rotate(x, pos, c, s, rope_dim)
    z = (x[:, 0:rope_dim:2].astype(np.float64) + 1j * x[:, 1:rope_dim:2]) * \
        (c[pos].astype(np.float64) + 1j * s[pos])
    mag = np.abs(x[:, 0:rope_dim:2]) + np.abs(x[:, 1:rope_dim:2])
    tol = 3 * np.spacing(mag.astype(np.float32)).astype(np.float64) + 1e-30
    assert np.all(np.abs(y[:, 0:rope_dim:2] - z.real) <= tol)
    assert np.all(np.abs(y[:, 1:rope_dim:2] - z.imag) <= tol)
    assert np.array_equal(y[:, rope_dim:], x[:, rope_dim:])        # the rest untouched


def test_rotation_preserves_pair_norms_and_inverts():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, 128)).astype(np.float32)
    pos = rng.integers(0, 100, 40)
    c, s = _tables(100, 128)
    y = O.rope_rotate(x, pos, c, s, 128)
    n0 = x[:, 0::2].astype(np.float64) ** 2 + x[:, 1::2].astype(np.float64) ** 2
    n1 = y[:, 0::2].astype(np.float64) ** 2 + y[:, 1::2].astype(np.float64) ** 2
    assert np.all(np.abs(n1 - n0) <= 1e-5 * n0 + 1e-30)
    back = O.rope_rotate(y, pos, c, -s, 128)                         # rotate by -theta
    assert np.all(np.abs(back - x) <= 1e-5 * (np.abs(x) + 1))


def test_rope_dim_zero_and_identity_tables_reduce_to_the_plain_quantisers():
    wl = synth.custom(2, 1, [130, 70], num_blocks=8, bt_width=3, seed=5)
    k = synth.bf16_bits_to_f32(wl.k_all())
    slots = wl.slot_mapping()
    pos = np.arange(len(slots)) % 50
    ones = np.ones((50, 64), np.float32)
    zeros = np.zeros((50, 64), np.float32)
    want = O.k_cache_write(k, slots, wl.poisoned_pool())
    assert np.array_equal(O.k_rope_cache_write(k, pos, ones, zeros, 128, slots, wl.poisoned_pool()), want)
    c, s = _tables(50, 128)
    assert np.array_equal(O.k_rope_cache_write(k, pos, c, s, 0, slots, wl.poisoned_pool()), want)
    q = synth.bf16_bits_to_f32(wl.q())
    w = wl.w()
    qpos = np.array([3, 9])
    for a, b in zip(O.quantize_q_rope(q, qpos, ones, zeros, 128, w), O.quantize_q(q, w)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_quantiser_sees_the_rotated_values():
    """The scale is amax over the rotated row: (3, 4) rotated by (cos 0.5,
    sin 0.75) becomes (-1.5, 4.25), so amax 4.25 (not 4) sets the scale."""
    k = np.zeros((1, 128), np.float32)
    k[0, 0], k[0, 1] = 3.0, 4.0
    pool = np.zeros((1, O.BLOCK_BYTES), np.uint8)
    O.k_rope_cache_write(k, [0], np.array([[0.5]], np.float32), np.array([[0.75]], np.float32), 2,
                         [5], pool)
    scale = pool[0, 8192 + 4 * 5:8192 + 4 * 6].view(np.float32)[0]
    assert scale == np.float32(np.float32(4.25) * O.INV_448)
    codes = pool[0, 5 * 128:5 * 128 + 2]
    want, _ = O.quantize_rows(np.array([[-1.5, 4.25] + [0.0] * 126], np.float32))
    assert codes.tolist() == want[0, :2].tolist()


def test_each_token_uses_its_own_position_row():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 128)).astype(np.float32)
    c, s = _tables(20, 64)
    y = O.rope_rotate(x, [4, 17, 4], c, s, 64)
    for t, p in enumerate([4, 17, 4]):
        assert np.array_equal(y[t], O.rope_rotate(x[t:t + 1], [0], c[p:p + 1], s[p:p + 1], 64)[0])
    assert not np.array_equal(y[0], y[1])


def test_head_rotation_of_queries_is_per_head():
    """Every head of a query token rotates with the token's position; the
    fold multiplies each head weight by the token's one scale."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 64, 128)).astype(np.float32)
    w = rng.standard_normal((2, 64)).astype(np.float32)
    c, s = _tables(10, 64)
    codes, w_eff, scale = O.quantize_q_rope(q, [2, 7], c, s, 64, w)
    rot = np.stack([O.rope_rotate(q[t], np.full(64, p), c, s, 64) for t, p in enumerate([2, 7])])
    want = O.quantize_q(rot, w)
    assert np.array_equal(codes, want[0]) and np.array_equal(w_eff, want[1])
    assert np.array_equal(scale, want[2])


def test_positions_outside_the_table_give_nan():
    k = np.ones((3, 128), np.float32)
    pool = np.zeros((1, O.BLOCK_BYTES), np.uint8)
    c, s = _tables(4, 64)
    O.k_rope_cache_write(k, [0, 4, -1], c, s, 64, [0, 1, 2], pool)
    scales = pool[0, 8192:8192 + 12].view(np.float32)
    assert np.isfinite(scales[0]) and np.isnan(scales[1]) and np.isnan(scales[2])
    assert (pool[0, 128:384] == 0x7F).all() and (pool[0, :128] != 0x7F).all()
    q = np.ones((2, 64, 128), np.float32)
    codes, w_eff, scale = O.quantize_q_rope(q, [1, 9], c, s, 64, np.ones((2, 64), np.float32))
    assert (codes[1] == 0x7F).all() and np.isnan(w_eff[1]).all() and np.isnan(scale[1])
    assert np.isfinite(w_eff[0]).all()
