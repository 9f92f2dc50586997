"""Pins for the oracle's 3D rotary encoding with a global time index
("Accelerating Video Generation Inference with Sequential-Parallel 3D
Positional Encoding Using a Global Time Index", section 2.2)."""
import math

import numpy as np

from oracle import fva_oracle as O


def test_pair_split_is_even_t_first():
    # D/2 pairs over (t, h, w) as evenly as possible, the remainder to t then h:
    # 64 = 22+21+21, 48 = 16+16+16, 32 = 11+11+10, 5 = 2+2+1, 4 = 2+1+1, 3 = 1+1+1
    assert O.rope_pairs(128) == (22, 21, 21)
    assert O.rope_pairs(96) == (16, 16, 16)
    assert O.rope_pairs(64) == (11, 11, 10)
    assert O.rope_pairs(10) == (2, 2, 1)
    assert O.rope_pairs(8) == (2, 1, 1)
    assert O.rope_pairs(6) == (1, 1, 1)


def test_hand_worked_frequencies_small_base():
    # D = 12: two pairs per axis; base 16 makes pair i of an axis turn by
    # pos * 16**(-i/2), i.e. by pos and by pos/4.  Token (t=1, h=2, w=3) of a
    # (2, 3, 4) grid with t_offset 1 sits at raster n = (1*3 + 2)*4 + 3 = 23
    # and has positions t = 2, h = 2, w = 3, so the six pair angles are
    # 2, 0.5 (t), 2, 0.5 (h), 3, 0.75 (w).
    x = np.zeros((1, 24, 1, 12))
    x[0, 23, 0] = [1, 0, 0, 1, 1, 0, 0, 1, 1, 0, 0, 1]
    out = O.rope(x, (2, 3, 4), t_offset=1, base=16.0)[0, 23, 0]
    c, s = math.cos, math.sin
    want = [c(2), s(2), -s(0.5), c(0.5),      # t pairs: (1,0) by 2, (0,1) by 0.5
            c(2), s(2), -s(0.5), c(0.5),      # h pairs
            c(3), s(3), -s(0.75), c(0.75)]    # w pairs
    assert np.allclose(out, want, atol=1e-15)


def test_hand_worked_example():
    # D = 6: one pair per axis, each turning by its position (base**0 = 1).
    x = np.array([1.0, 0.0, 0.0, 1.0, 1.0, 1.0]).reshape(1, 1, 1, 6)
    grid = (2, 1, 3)                       # token n = (t*1 + h)*3 + w
    full = np.zeros((1, 6, 1, 6))
    full[:, 5] = x[:, 0]                   # token (t=1, h=0, w=2)
    out = O.rope(full, grid)[0, 5, 0]
    want = [math.cos(1), math.sin(1),                          # (1,0) by 1 rad
            0.0, 1.0,                                          # (0,1) by 0 rad
            math.cos(2) - math.sin(2), math.sin(2) + math.cos(2)]   # (1,1) by 2 rad
    assert np.allclose(out, want, atol=1e-15)


def test_position_zero_is_identity_and_norms_are_kept():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 2 * 3 * 4, 2, 64))
    out = O.rope(x, (2, 3, 4), t_offset=5)
    pair = lambda a: a[..., 0::2] ** 2 + a[..., 1::2] ** 2
    assert np.allclose(pair(out), pair(x), rtol=1e-13)
    zero = O.rope(x, (2, 3, 4))[:, 0]
    assert np.array_equal(zero, x[:, 0])


def test_scores_depend_only_on_relative_position():
    # q.k after encoding is unchanged when both positions shift by the same offset
    rng = np.random.default_rng(1)
    grid = (3, 2, 2)
    q = rng.standard_normal((1, 12, 1, 64))
    k = rng.standard_normal((1, 12, 1, 64))
    a = O.rope(q, grid, t_offset=0)[0, :, 0] @ O.rope(k, grid, t_offset=0)[0, :, 0].T
    b = O.rope(q, grid, t_offset=7)[0, :, 0] @ O.rope(k, grid, t_offset=7)[0, :, 0].T
    assert np.allclose(a, b, rtol=1e-11, atol=1e-11)


def test_chunk_with_start_frame_equals_full_sequence():
    # encoding frames [s, s+Tc) as their own chunk with offset s equals the
    # same frames of the whole sequence encoded at once (global time index)
    rng = np.random.default_rng(2)
    T, Hh, W, s, Tc = 6, 2, 3, 2, 3
    full = rng.standard_normal((1, T * Hh * W, 1, 32))
    enc = O.rope(full, (T, Hh, W))
    chunk = full[:, s * Hh * W:(s + Tc) * Hh * W]
    assert np.allclose(O.rope(chunk, (Tc, Hh, W), t_offset=s), enc[:, s * Hh * W:(s + Tc) * Hh * W], atol=1e-13)
