"""GPU parity of 3- and 4-bit values (K3V3, K2V4, K4V4 budgets) through the C ABI.

A cache with val_bits = 3 or 4 adds a plane holding each value code's high
bits (256 bytes for 3 bits, 512 for 4; after the keys' plane when keys are wide
too), for every group size.  Gates as for 2-bit values: the kernel's rotated rows within the
fp32 bound of the fp64 rotation and the bytes bit-exact to the oracle's
quantizer and packing on those rows (both append kernels, partial and full
pages); the fused step writing the append's bytes; decode within 2e-3 of the
oracle reading the same pool; the output-error evaluator reading the plane.
"""

import numpy as np
import pytest

import kvq_inputs as I
from oracle import kvq_oracle as O
from tests.gpu_util import DeviceCase, dense_rotations, max_abs_rel, require_gpu, rotation_error_bound
from tests.test_gpu_step import _append_newest, _new_kv, _newest, _prefill

pytestmark = pytest.mark.gpu

TOL = 2e-3
BUDGETS = [(3, 3), (2, 4), (4, 4), (2, 3)]  # (key bits, value bits)


@pytest.mark.parametrize("dtype,lens,rotation,group", [
    ("bf16", [40, 9], "dense", 32),       # the tiled kernel
    ("f32", [30, 2], "hadamard", 32),
    ("bf16", [300, 77], "dense", 32),     # the bulk kernel, full and partial pages
    ("f32", [129, 64], "hadamard", 128),
    ("bf16", [200, 50], "dense", 64),
])
@pytest.mark.parametrize("kb,vb", BUDGETS, ids=lambda b: str(b))
def test_append_bytes_match_the_oracle(dtype, lens, rotation, group, kb, vb):
    dev = require_gpu()
    case = I.make_case("v4", 400 + sum(lens) + kb + 3 * vb, B=2, Hq=8, Hkv=4, seq_lens=lens, dtype=dtype,
                       table_policy="interleaved", rotation=rotation)
    r_k, r_v = dense_rotations(case)
    dc = DeviceCase(case, dev, group_size=group, key_bits=kb, val_bits=vb)
    rot = dc.append(rot_out=True).cpu().numpy()
    xg, wg = rot[:, :, 0, :], rot[:, :, 1, :]
    a = O.centre_keys(case.k, case.mu)
    x64, w64 = O.rotate(a, r_k), O.rotate(case.v, r_v)
    for h in range(case.Hkv):
        assert np.all(np.abs(xg[:, h] - x64[:, h]) <= rotation_error_bound(a[:, h], r_k[h]) + 1e-30)
        assert np.all(np.abs(wg[:, h] - w64[:, h]) <= rotation_error_bound(case.v[:, h], r_v[h]) + 1e-30)
    expect = np.zeros_like(dc.pool_np())
    O.quantize_append(expect, case.Hkv, case.slots, xg, wg, group=group, key_bits=kb, val_bits=vb)
    np.testing.assert_array_equal(dc.pool_np(), expect)
    if vb > 2:  # the values really use more than four levels
        _, _, _, vc, _, _ = O.unpack_blocks(dc.pool_np().reshape(-1, O.block_bytes(kb, vb, group)), kb, vb, group)
        assert vc.max() > 3


SHAPES = [
    (1, 4, 1, [256]),
    (2, 2, 2, [77, 300]),         # g = 1
    (2, 32, 8, [1000, 257]),      # g = 4
    (2, 64, 8, [513, 1024]),      # g = 8
    (1, 16, 1, [300]),            # g = 16
    (3, 8, 2, [0, 5, 100]),
]


@pytest.mark.parametrize("kb,vb,group", [b + (32,) for b in BUDGETS] + [(3, 3, 128), (2, 3, 64), (4, 4, 64)],
                         ids=lambda b: str(b))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}_Hq{s[1]}_Hkv{s[2]}_T{'-'.join(map(str, s[3]))}")
def test_decode_parity(shape, kb, vb, group):
    dev = require_gpu()
    B, Hq, Hkv, lens = shape
    case = I.make_case("v4d", 410 + sum(lens) + Hq + kb, B=B, Hq=Hq, Hkv=Hkv, seq_lens=lens,
                       table_policy="interleaved")
    dc = DeviceCase(case, dev, key_bits=kb, val_bits=vb, group_size=group)
    dc.append(rot_out=False)
    ref = O.decode_attention(case.q, dc.pool_np(), case.Hkv, case.page_table, case.seq_lens, case.r_k, case.r_v,
                             **dc.layout)
    for ns in (0, 1, 3):
        got = dc.decode("f32", num_splits=ns)
        assert max_abs_rel(got, ref) <= TOL, ns
    got16 = dc.decode("bf16")
    assert np.array_equal(got16, I.bf16_bits(dc.decode("f32").astype(np.float32)))


@pytest.mark.parametrize("kb,vb", [(2, 3), (4, 4)], ids=lambda b: str(b))
@pytest.mark.parametrize("shape", [(2, 32, 8, [1000, 257]), (2, 64, 8, [513, 1024]), (1, 16, 1, [300])],
                         ids=lambda s: f"B{s[0]}_Hq{s[1]}_Hkv{s[2]}_T{'-'.join(map(str, s[3]))}")
def test_hadamard_decode_parity(shape, kb, vb):
    """A Hadamard R_V with wide values: the kernel's correction for the fp16 rounding of p * s_v is taken about
    the tensor's own middle code (3.5 or 7.5), and one split per sequence gives the longest sums."""
    dev = require_gpu()
    B, Hq, Hkv, lens = shape
    case = I.make_case("v4h", 430 + sum(lens) + Hq + kb, B=B, Hq=Hq, Hkv=Hkv, seq_lens=lens,
                       table_policy="interleaved", rotation="hadamard")
    r_k, r_v = dense_rotations(case)
    dc = DeviceCase(case, dev, key_bits=kb, val_bits=vb)
    dc.append(rot_out=False)
    ref = O.decode_attention(case.q, dc.pool_np(), case.Hkv, case.page_table, case.seq_lens, r_k, r_v,
                             key_bits=kb, val_bits=vb)
    for ns in (0, 1, 3):
        got = dc.decode("f32", num_splits=ns)
        assert max_abs_rel(got, ref) <= TOL, ns


@pytest.mark.parametrize("shape", [(2, 32, 8, [1000, 17], "bf16"), (2, 64, 8, [513, 16], "f32"),
                                   (1, 16, 1, [300], "bf16"), (3, 8, 2, [0, 5, 100], "bf16")],
                         ids=lambda s: f"Hq{s[1]}_Hkv{s[2]}_{s[4]}")
@pytest.mark.parametrize("kb,vb,group", [(3, 3, 32), (2, 4, 32), (3, 3, 64), (2, 3, 128)], ids=lambda b: str(b))
def test_step_writes_the_appended_bytes(shape, kb, vb, group):
    dev = require_gpu()
    B, Hq, Hkv, lens, dtype = shape
    case = I.make_case("v4s", 420 + sum(lens) + Hq + vb, B=B, Hq=Hq, Hkv=Hkv, seq_lens=lens, dtype=dtype,
                       table_policy="interleaved")
    newest = _newest(case)
    a = DeviceCase(case, dev, key_bits=kb, val_bits=vb, group_size=group)
    _prefill(a, case, newest)
    b = DeviceCase(case, dev, key_bits=kb, val_bits=vb, group_size=group)
    b.pool.copy_(a.pool)
    _append_newest(a, newest)
    k_new, v_new = _new_kv(case, b, newest, dev)
    got = b.step(k_new, v_new, "f32")
    np.testing.assert_array_equal(b.pool_np(), a.pool_np())
    ref = O.decode_attention(case.q, b.pool_np(), Hkv, case.page_table, case.seq_lens, case.r_k, case.r_v,
                             **b.layout)
    assert max_abs_rel(got, ref) <= TOL


@pytest.mark.parametrize("kb,vb", [(3, 3), (4, 4)], ids=lambda b: str(b))
def test_window_with_wide_values(kb, vb):
    dev = require_gpu()
    case = I.make_case("v4w", 430 + kb, B=2, Hq=32, Hkv=8, seq_lens=[700, 90], table_policy="interleaved")
    dc = DeviceCase(case, dev, key_bits=kb, val_bits=vb)
    dc.append(rot_out=False)
    win = dc.window(4, 64)
    got = dc.decode("f32", window=win)
    ks = [case.k[case.tok_seq == b] for b in range(case.B)]
    vs = [case.v[case.tok_seq == b] for b in range(case.B)]
    ref = O.decode_attention_window(case.q, dc.pool_np(), case.Hkv, case.page_table, case.seq_lens, case.mu,
                                    case.r_k, case.r_v, ks, vs, 4, 64, key_bits=kb, val_bits=vb)
    assert max_abs_rel(got, ref) <= TOL


@pytest.mark.parametrize("kb,vb,group", [(3, 3, 32), (2, 4, 32), (3, 3, 128), (4, 3, 64)], ids=lambda b: str(b))
def test_output_error_with_wide_values(kb, vb, group):
    """The evaluator reads the values' plane (256 bytes for 3 bits, 512 for 4) after the keys' one."""
    from tests.test_gpu_eval import Evaluated, _check
    dev = require_gpu()
    case = I.make_case("v4e", 440 + kb + vb, B=2, Hq=32, Hkv=8, seq_lens=[700, 65], table_policy="interleaved")
    ev = Evaluated(case, dev, key_bits=kb, val_bits=vb, group=group)
    _check(ev.run(), ev.oracle())


def test_full_size_k3v3_sampled_heads():
    """The 8B shape at 128K with K3V3: bulk append, one decode, sampled heads."""
    dev = require_gpu()
    case = I.llama8b_case(131072)
    dc = DeviceCase(case, dev, key_bits=3, val_bits=3)
    dc.append(rot_out=False, chunk=1 << 20)
    got = dc.decode("f32")
    heads = [(0, 0), (0, 17), (0, 31)]
    ref = O.decode_attention(case.q, dc.pool_np(), case.Hkv, case.page_table, case.seq_lens, case.r_k, case.r_v,
                             heads=heads, key_bits=3, val_bits=3)
    for b, j in heads:
        assert max_abs_rel(got[b, j], ref[b, j]) <= TOL, j
