"""GPU parity of the fused decode attention against the oracle (through the C ABI).

The oracle runs on the kernel's own pool bytes, so both sides read the same
dequantized cache.  The gate is 2e-3 max-abs-relative per (sequence, head) row
on the fp32 output; the bf16 output must equal the fp32 output rounded to
nearest even.
"""

import numpy as np
import pytest

import kvq_inputs as I
from oracle import kvq_oracle as O
from tests.gpu_util import DeviceCase, dev_tensor, max_abs_rel, require_gpu

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _oracle_decode(case, pool, heads=None):
    return O.decode_attention(case.q, pool, case.Hkv, case.page_table, case.seq_lens, case.r_k, case.r_v, heads=heads)


def _rne_bf16(x: np.ndarray) -> np.ndarray:
    """Reference fp32 -> bf16 rounding (nearest even) for the output-format check."""
    return I.bf16_bits(np.asarray(x, np.float32))


def test_tiny_case_parity_and_split_counts():
    dev = require_gpu()
    case = I.tiny_case()
    dc = DeviceCase(case, dev)
    dc.append(rot_out=False)
    ref = _oracle_decode(case, dc.pool_np())
    for ns in (0, 1, 2, 3, 16):
        got = dc.decode("f32", num_splits=ns)
        err = max_abs_rel(got, ref)
        assert err <= TOL, (ns, err)


SHAPES = [
    # (B, Hq, Hkv, seq_lens, policy)
    (1, 4, 1, [1], "contiguous"),
    (1, 4, 1, [15], "contiguous"),
    (1, 4, 1, [16], "permuted"),
    (1, 4, 1, [17], "permuted"),
    (1, 8, 2, [31], "permuted"),
    (1, 8, 2, [33], "permuted"),
    (3, 8, 2, [0, 5, 100], "interleaved"),
    (2, 2, 2, [77, 300], "interleaved"),        # g = 1
    (2, 4, 2, [129, 64], "interleaved"),        # g = 2
    (2, 32, 8, [1000, 257], "interleaved"),     # g = 4, Llama-3.1-8B heads
    (2, 64, 8, [513, 1024], "interleaved"),     # g = 8, 70B-class heads
    (1, 6, 1, [150], "permuted"),               # g = 6 (second quad padded)
    (1, 12, 1, [200], "permuted"),              # g = 12 (padded quad)
    (1, 16, 1, [300], "permuted"),              # g = 16
    (2, 10, 2, [400, 77], "interleaved"),       # g = 5: three padded heads of the octet layout
    (1, 7, 1, [260], "permuted"),               # g = 7
    (1, 9, 1, [500], "permuted"),               # g = 9: seven padded heads of the hexadeca layout
    (2, 30, 2, [333, 1200], "interleaved"),     # g = 15
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}_Hq{s[1]}_Hkv{s[2]}_T{'-'.join(map(str, s[3]))}")
def test_decode_parity_shapes(shape):
    dev = require_gpu()
    B, Hq, Hkv, lens, policy = shape
    case = I.make_case("d", 100 + sum(lens) + Hq, B=B, Hq=Hq, Hkv=Hkv, seq_lens=lens, table_policy=policy)
    dc = DeviceCase(case, dev)
    dc.append(rot_out=False)
    ref = _oracle_decode(case, dc.pool_np())
    for ns in (0, 1, 7):
        got = dc.decode("f32", num_splits=ns)
        assert np.isfinite(got).all()
        err = max_abs_rel(got, ref)
        assert err <= TOL, (ns, err)
    for b in range(B):
        if lens[b] == 0:
            assert not got[b].any()


def test_bf16_output_is_rounded_fp32_output():
    dev = require_gpu()
    case = I.make_case("o", 7, B=2, Hq=32, Hkv=8, seq_lens=[333, 4000], table_policy="interleaved")
    dc = DeviceCase(case, dev)
    dc.append(rot_out=False)
    f32 = dc.decode("f32")
    b16 = dc.decode("bf16")
    np.testing.assert_array_equal(b16, _rne_bf16(f32))
    assert max_abs_rel(f32, _oracle_decode(case, dc.pool_np())) <= TOL


def test_page_permutation_gives_identical_output():
    """The same tokens under a different physical page placement: bit-identical output."""
    dev = require_gpu()
    base = dict(B=2, Hq=32, Hkv=8, seq_lens=[700, 1500])
    a = I.make_case("q", 9, table_policy="contiguous", **base)
    b = I.make_case("q", 9, table_policy="interleaved", **base)
    assert not np.array_equal(a.page_table, b.page_table)
    outs = []
    for case in (a, b):
        dc = DeviceCase(case, dev)
        dc.append(rot_out=False)
        outs.append(dc.decode("f32"))
    np.testing.assert_array_equal(outs[0], outs[1])


@pytest.mark.parametrize("Hq,B", [(4, 800), (8, 600)], ids=["g4_B800", "g8_B600"])
def test_large_ragged_batch(Hq, B):
    """The automatic plan sizes splits from the batch's total length inside the
    kernel (a prefix scan over the sequence lengths, in chunks of one
    workgroup's threads): a batch larger than a workgroup, lengths 0..60 with
    empty sequences, every row against the oracle, under the automatic and a
    fixed split plan."""
    dev = require_gpu()
    rng = np.random.default_rng(B)
    lens = rng.integers(0, 61, size=B)
    lens[::97] = 0
    case = I.make_case("lb", 500 + B, B=B, Hq=Hq, Hkv=1, seq_lens=lens, table_policy="interleaved")
    dc = DeviceCase(case, dev)
    dc.append(rot_out=False)
    ref = _oracle_decode(case, dc.pool_np())
    for ns in (0, 2):
        got = dc.decode("f32", num_splits=ns)
        assert np.isfinite(got).all()
        assert not got[lens == 0].any()
        assert max_abs_rel(got, ref) <= TOL, ns


def test_ragged_batch_rows():
    """Automatic plan on a ragged batch: the long sequences take many splits, the
    short ones one, a one-token sequence a single page; every row matches the
    oracle."""
    dev = require_gpu()
    lens = [4000, 70, 1, 2500]
    case = I.make_case("rb", 77, B=4, Hq=32, Hkv=8, seq_lens=lens, table_policy="interleaved")
    dc = DeviceCase(case, dev)
    dc.append(rot_out=False)
    got = dc.decode("f32")
    ref = _oracle_decode(case, dc.pool_np())
    for b in range(4):
        assert max_abs_rel(got[b], ref[b]) <= TOL, b


def test_length_beyond_max_seq_len_is_cut():
    """A sequence length above the host's max_seq_len is cut there: the row equals
    attention over the first max_seq_len tokens (both split plans)."""
    dev = require_gpu()
    case = I.make_case("cut", 78, B=2, Hq=8, Hkv=2, seq_lens=[300, 120], table_policy="permuted")
    dc = DeviceCase(case, dev)
    dc.append(rot_out=False)
    cut = np.array([200, 120], dtype=np.int32)
    ref = O.decode_attention(case.q, dc.pool_np(), case.Hkv, case.page_table, cut, case.r_k, case.r_v)
    for ns in (0, 3):
        got = dc.decode("f32", num_splits=ns, max_seq=200)
        assert max_abs_rel(got, ref) <= TOL, ns


def test_repeated_calls_are_deterministic():
    dev = require_gpu()
    case = I.make_case("r", 11, B=1, Hq=32, Hkv=8, seq_lens=[5000])
    dc = DeviceCase(case, dev)
    dc.append(rot_out=False)
    first = dc.decode("f32")
    for _ in range(3):
        np.testing.assert_array_equal(dc.decode("f32"), first)


def test_one_workspace_reused_across_calls_and_shapes():
    """The split tickets in the workspace return to zero after every call: one workspace
    serves calls of different lengths and split counts, each equal to a fresh-workspace run."""
    import torch
    dev = require_gpu()
    a = DeviceCase(I.make_case("wa", 15, B=2, Hq=32, Hkv=8, seq_lens=[3000, 100]), dev)
    b = DeviceCase(I.make_case("wb", 16, B=1, Hq=32, Hkv=8, seq_lens=[9000]), dev)
    for dc in (a, b):
        dc.append(rot_out=False)
    fresh = {(id(dc), ns): dc.decode("f32", num_splits=ns) for dc in (a, b) for ns in (0, 5)}
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=dev)
    for dc, ns in [(a, 0), (b, 0), (a, 5), (b, 5), (a, 0), (b, 5), (a, 5)]:
        np.testing.assert_array_equal(dc.decode("f32", num_splits=ns, ws=ws), fresh[(id(dc), ns)])


def test_workspace_reused_across_batches_beyond_one_counter_block():
    """Shapes with more than 64 (sequence, KV head) pairs, which would spill past a
    256-byte ticket block: a batch of 20 x 8 KV heads, a batch of one, and the
    batch of 20 again, all through one workspace, each equal to a fresh run."""
    import torch
    dev = require_gpu()
    a = DeviceCase(I.make_case("wc", 17, B=20, Hq=32, Hkv=8, seq_lens=list(range(40, 840, 40))), dev)
    b = DeviceCase(I.make_case("wd", 18, B=1, Hq=32, Hkv=8, seq_lens=[5000]), dev)
    for dc in (a, b):
        dc.append(rot_out=False)
    fresh = {id(dc): dc.decode("f32") for dc in (a, b)}
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=dev)
    for dc in (a, b, a, b, a):
        np.testing.assert_array_equal(dc.decode("f32", ws=ws), fresh[id(dc)])


def test_centering_is_invisible_to_attention_on_exact_cache():
    """OptR section 1: centering shifts every logit of a query by <q, mu>, so softmax is
    unchanged.  Keys k = mu + 0.5 * levels and values 0.25 * levels (R = I) quantize
    exactly once centred, so the kernel's output must equal plain Eq. (1)-(2) attention
    on the raw, uncentred k and v."""
    dev = require_gpu()
    rng = np.random.default_rng(12)
    case = I.make_case("c", 13, B=1, Hq=4, Hkv=1, seq_lens=[64], dtype="f32", identity_rotation=True,
                       mu_zero=True)

    def levels():
        lv = rng.integers(0, 4, size=(64, 1, 128)).astype(np.float32)
        lv[:, :, 0::32] = 0
        lv[:, :, 1::32] = 3
        return lv

    mu = (np.round(rng.standard_normal((1, 128)) * 4) / 4).astype(np.float32)
    case.k = (levels() * np.float32(0.5) + mu[None]).astype(np.float32)
    case.v = (levels() * np.float32(0.25)).astype(np.float32)
    case.mu = mu
    dc = DeviceCase(case, dev)
    dc.append(rot_out=False)
    got = dc.decode("f32")
    for j in range(case.Hq):
        ref = O.softmax_attention(case.q[0, j], case.k[:, 0], case.v[:, 0], 1 / np.sqrt(128))
        assert max_abs_rel(got[0, j], ref) <= TOL


FULL = {
    "llama8b_t32k": lambda: I.llama8b_case(32768),
    "llama8b_t128k": lambda: I.llama8b_case(131072),
    "llama8b_batch16": lambda: I.batched_case(),
    "gqa70b_b4_t128k": lambda: I.seventy_b_case(),
    "gqa405b_t128k": lambda: I.gqa405b_case(),
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled_heads(name):
    """Workload sizes: bulk append of the whole context, one decode step, and the oracle
    on sampled (sequence, head) rows over the kernel's own pool."""
    dev = require_gpu()
    case = FULL[name]()
    dc = DeviceCase(case, dev)
    dc.append(rot_out=False, chunk=1 << 20)
    got = dc.decode("f32")
    assert np.isfinite(got).all()
    rng = np.random.default_rng(3)
    heads = sorted({(int(rng.integers(case.B)), int(rng.integers(case.Hq))) for _ in range(4)} |
                   {(case.B - 1, case.Hq - 1), (0, 0)})
    ref = _oracle_decode(case, dc.pool_np(), heads=heads)
    for b, j in heads:
        err = max_abs_rel(got[b, j], ref[b, j])
        assert err <= TOL, (b, j, err)


@pytest.mark.parametrize("num_splits", [64, 100])
def test_many_splits_take_the_register_merge(num_splits):
    """With more (split, head) partial rows than the ring holds (64 splits x 4 heads x
    132 floats > the g <= 4 ring), the merging workgroup loads them per thread instead
    of staging them by DMA; both merges must agree with the oracle."""
    dev = require_gpu()
    case = I.make_case("ms", 91 + num_splits, B=2, Hq=8, Hkv=2, seq_lens=[4096, 3000], table_policy="interleaved")
    dc = DeviceCase(case, dev)
    dc.append(rot_out=False, chunk=1 << 20)
    ref = O.decode_attention(case.q, dc.pool_np(), case.Hkv, case.page_table, case.seq_lens, case.r_k, case.r_v)
    got = dc.decode("f32", num_splits=num_splits)
    assert max_abs_rel(got, ref) <= TOL
    auto = dc.decode("f32")  # the automatic plan stages the rows
    assert max_abs_rel(auto, ref) <= TOL
