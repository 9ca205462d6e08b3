"""Host checks of the seeded input generator (no GPU): the Hadamard option yields
+-1 sign vectors, deterministic per seed, whose oracle matrices are orthogonal."""

import numpy as np

import kvq_inputs as I
from oracle import kvq_oracle as O


def test_hadamard_case_holds_sign_vectors():
    a = I.make_case("h", 5, B=2, Hq=8, Hkv=2, seq_lens=[30, 2], rotation="hadamard")
    b = I.make_case("h", 5, B=2, Hq=8, Hkv=2, seq_lens=[30, 2], rotation="hadamard")
    assert a.rotation == "hadamard" and a.r_k.shape == (2, 128) and a.r_v.shape == (2, 128)
    assert np.all(np.abs(a.r_k) == 1) and np.all(np.abs(a.r_v) == 1)
    assert not np.array_equal(a.r_k, a.r_v)  # K and V draw their own signs
    np.testing.assert_array_equal(a.r_k, b.r_k)
    for r in (*O.hadamard_rotation(a.r_k), *O.hadamard_rotation(a.r_v)):
        O.check_orthogonal(r)
    d = I.make_case("h", 5, B=2, Hq=8, Hkv=2, seq_lens=[30, 2])
    assert d.rotation == "dense" and d.r_k.shape == (2, 128, 128)
