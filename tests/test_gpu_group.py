"""GPU parity of Q2 with group size G = 64 and 128 through the C ABI.

The cache's group_size selects G; the block keeps one metadata pair per group
(80 and 72 bytes per token for G = 64 and 128), and every kernel reads the pair
of a channel's group.
Gates as for G = 32: the kernel's rotated rows within the fp32 bound of the
fp64 rotation, codes and metadata bit-exact to the oracle's quantizer (with the
same G) on those rows, in both append kernels; the fused step writing the
append's bytes (G = 128 combines a group's range across two waves there); decode
within 2e-3 of the oracle.
"""

import numpy as np
import pytest

import kvq_inputs as I
from oracle import kvq_oracle as O
from tests.gpu_util import DeviceCase, dense_rotations, max_abs_rel, require_gpu, rotation_error_bound
from tests.test_gpu_step import _append_newest, _new_kv, _newest, _prefill

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.mark.parametrize("group", [64, 128])
@pytest.mark.parametrize("dtype,lens,rotation", [
    ("bf16", [40, 9], "dense"),        # 49 tokens: the tiled kernel
    ("f32", [30, 2], "hadamard"),
    ("bf16", [300, 77], "dense"),      # the bulk kernel
    ("f32", [129, 64], "hadamard"),
])
def test_append_codes_match_the_oracle(group, dtype, lens, rotation):
    dev = require_gpu()
    case = I.make_case("g", 130 + sum(lens), B=2, Hq=8, Hkv=4, seq_lens=lens, dtype=dtype,
                       table_policy="interleaved", rotation=rotation)
    r_k, r_v = dense_rotations(case)
    dc = DeviceCase(case, dev, group_size=group)
    rot = dc.append(rot_out=True).cpu().numpy()
    xg, wg = rot[:, :, 0, :], rot[:, :, 1, :]
    a = O.centre_keys(case.k, case.mu)
    x64, w64 = O.rotate(a, r_k), O.rotate(case.v, r_v)
    for h in range(case.Hkv):
        assert np.all(np.abs(xg[:, h] - x64[:, h]) <= rotation_error_bound(a[:, h], r_k[h]) + 1e-30)
        assert np.all(np.abs(wg[:, h] - w64[:, h]) <= rotation_error_bound(case.v[:, h], r_v[h]) + 1e-30)
    expect = np.zeros_like(dc.pool_np())
    O.quantize_append(expect, case.Hkv, case.slots, xg, wg, group=group)
    np.testing.assert_array_equal(dc.pool_np(), expect)
    # one metadata pair per G channels: the blocks are smaller than G = 32's
    assert expect.size == O.pool_bytes(dc.num_pages, case.Hkv, group=group) < O.pool_bytes(dc.num_pages, case.Hkv)


@pytest.mark.parametrize("group", [64, 128])
@pytest.mark.parametrize("shape", [(2, 32, 8, [1000, 257]), (2, 64, 8, [513, 100]), (1, 16, 1, [300])],
                         ids=lambda s: f"B{s[0]}_Hq{s[1]}_Hkv{s[2]}" if isinstance(s, tuple) else str(s))
def test_decode_parity(group, shape):
    dev = require_gpu()
    B, Hq, Hkv, lens = shape
    case = I.make_case("gd", 140 + sum(lens) + Hq, B=B, Hq=Hq, Hkv=Hkv, seq_lens=lens, table_policy="interleaved")
    dc = DeviceCase(case, dev, group_size=group)
    dc.append(rot_out=False)
    ref = O.decode_attention(case.q, dc.pool_np(), case.Hkv, case.page_table, case.seq_lens, case.r_k, case.r_v,
                             group=group)
    for ns in (0, 3):
        assert max_abs_rel(dc.decode("f32", num_splits=ns), ref) <= TOL, ns


@pytest.mark.parametrize("group", [64, 128])
@pytest.mark.parametrize("shape", [(2, 32, 8, [1000, 17], "bf16"), (2, 64, 8, [513, 16], "f32"),
                                   (1, 16, 1, [300], "bf16")],
                         ids=lambda s: f"Hq{s[1]}_Hkv{s[2]}_{s[4]}" if isinstance(s, tuple) else str(s))
def test_step_writes_the_appended_bytes(group, shape):
    dev = require_gpu()
    B, Hq, Hkv, lens, dtype = shape
    case = I.make_case("gs", 150 + sum(lens) + Hq, B=B, Hq=Hq, Hkv=Hkv, seq_lens=lens, dtype=dtype,
                       table_policy="interleaved")
    newest = _newest(case)
    a = DeviceCase(case, dev, group_size=group)
    _prefill(a, case, newest)
    b = DeviceCase(case, dev, group_size=group)
    b.pool.copy_(a.pool)
    _append_newest(a, newest)
    k_new, v_new = _new_kv(case, b, newest, dev)
    got = b.step(k_new, v_new, "f32")
    np.testing.assert_array_equal(b.pool_np(), a.pool_np())
    ref = O.decode_attention(case.q, b.pool_np(), Hkv, case.page_table, case.seq_lens, case.r_k, case.r_v,
                             group=group)
    assert max_abs_rel(got, ref) <= TOL


def test_full_size_group128_sampled_heads():
    """The 8B shape at 32K with G = 128: the bulk append over the whole context, then
    one decode; sampled heads against the oracle on the GPU's pool."""
    dev = require_gpu()
    case = I.llama8b_case(32768)
    dc = DeviceCase(case, dev, group_size=128)
    dc.append(rot_out=False)
    got = dc.decode("f32")
    heads = [(0, 0), (0, 19)]
    ref = O.decode_attention(case.q, dc.pool_np(), case.Hkv, case.page_table, case.seq_lens, case.r_k, case.r_v,
                             heads=heads, group=128)
    for b, j in heads:
        assert max_abs_rel(got[b, j], ref[b, j]) <= TOL, j
