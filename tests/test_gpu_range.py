"""GPU parity of decode over the value range the cache format stores (through the C ABI).

The P.V product runs on the matrix cores with an fp16 operand p * s_v, so the
kernel keeps it in a per-group power-of-two unit; these tests drive it with
value groups whose stored scale s_v spans 1e-4 .. 4e3 (about 2^-13 .. 2^12),
and with keys built so that the logits climb 3 to 8 log2 units at a time past
the running maximum (every climb moves the online softmax's reference).  The
cache is written from given rotated rows (KVQ_F32_ROTATED), and the oracle
reads the GPU's own pool, so both sides attend over the same dequantized
cache; the gate is the 2e-3 max-abs-relative error per (sequence, head) row of
the fp32 output (OptR section 3, Eq. (1)-(2); section 3.2, Eq. (5)).

A second test fills the pool with 0xff bytes (fp16 NaN metadata) before
appending: stale slots past a sequence's end and an absent page then hold NaN
scales and zeros, which must weigh nothing.
"""

import dataclasses

import numpy as np
import pytest

import kvq_inputs as I
from oracle import kvq_oracle as O
from tests.gpu_util import DeviceCase, dense_rotations, dev_tensor, max_abs_rel, require_gpu

pytestmark = pytest.mark.gpu

TOL = 2e-3
LOG2E = 1.4426950408889634


def _scales(kind: str, rng, n: int) -> np.ndarray:
    """Half-width c of each (position, value group) [n][4]; s_v is about 2c/3."""
    lo, hi = np.log10(1.5e-4), np.log10(6e3)
    if kind == "per_position":
        return 10.0 ** rng.uniform(lo, hi, (n, 4))
    if kind == "phases":  # constant over stretches of 256 positions, per group
        per = 10.0 ** rng.uniform(lo, hi, (n // 256 + 1, 4))
        return np.repeat(per, 256, axis=0)[:n]
    if kind == "big_then_small":
        c = np.where(np.arange(n)[:, None] < n // 2, 6e3, 1.5e-4) * np.ones((1, 4))
        return c * (1.0 + 0.1 * rng.random((n, 4)))
    raise ValueError(kind)


def _range_case(kind: str, g: int, Hkv: int, lens, seed: int, rotation: str = "dense"):
    """A case with constructed queries and rotated rows: returns (case, x, w)."""
    B = len(lens)
    case = I.make_case(f"rng_{kind}", seed, B=B, Hq=g * Hkv, Hkv=Hkv, seq_lens=lens, dtype="f32",
                       table_policy="interleaved", rotation=rotation)
    rng = np.random.default_rng(seed)
    r_k, _ = dense_rotations(case)
    # queries of one KV head share a direction (every head sees the climbs), plus head noise
    base = rng.standard_normal((B, Hkv, 128))
    q = np.repeat(base, g, axis=1) + 0.3 * rng.standard_normal((B, Hkv * g, 128))
    case = dataclasses.replace(case, q=q.astype(np.float32))
    n = case.n_tokens
    x = np.zeros((n, Hkv, 128))
    w = np.zeros((n, Hkv, 128))
    sm = 1.0 / np.sqrt(128.0)
    for b in range(B):
        sel = np.nonzero(case.tok_seq == b)[0]
        T = len(sel)
        for h in range(Hkv):
            qh = case.q[b, h * g].astype(np.float64) @ r_k[h].astype(np.float64)  # q_hat of the head's first query
            d = qh / np.linalg.norm(qh)
            # logit staircase (log2 units): a climb of 3..8 with probability 0.02 per position
            climb = np.cumsum(np.where(rng.random(T) < 0.02, rng.uniform(3.0, 8.0, T), 0.0))
            beta = climb / (np.linalg.norm(qh) * sm * LOG2E)
            x[sel, h] = 0.5 * rng.standard_normal((T, 128)) + beta[:, None] * d[None, :]
            c = _scales(kind, rng, T)
            off = c * 2.0 * rng.standard_normal((T, 4))
            u = rng.uniform(-1.0, 1.0, (T, 128))
            w[sel, h] = np.repeat(off, 32, axis=1) + np.repeat(c, 32, axis=1) * u
    return case, x.astype(np.float32), w.astype(np.float32)


def _prerotated(dc, x, w):
    from rotated_int2_kv_centering_amd import kvq
    import torch
    c = dc.c
    kvq.kvq_quant_append(dc.cache, dev_tensor(x, dc.dev), dev_tensor(w, dc.dev), kvq.KVQ_F32_ROTATED, c.n_tokens,
                         dc.slots, None, None, None, None)
    torch.cuda.synchronize()


CASES = [
    # (kind, g, Hkv, lens)
    ("per_position", 4, 2, [1500, 333]),
    ("phases", 4, 2, [2049, 700]),
    ("big_then_small", 4, 1, [1800]),
    ("per_position", 8, 1, [1200, 517]),
    ("big_then_small", 8, 1, [1024]),
    ("phases", 8, 2, [2049, 700]),
    ("per_position", 16, 1, [900]),
    ("phases", 16, 1, [1300]),
]


@pytest.mark.parametrize("case_def", CASES, ids=lambda c: f"{c[0]}_g{c[1]}_T{'-'.join(map(str, c[3]))}")
def test_decode_value_scales_across_fp16_range(case_def):
    dev = require_gpu()
    kind, g, Hkv, lens = case_def
    case, x, w = _range_case(kind, g, Hkv, lens, seed=900 + g + len(lens) + lens[0])
    dc = DeviceCase(case, dev)
    _prerotated(dc, x, w)
    pool = dc.pool_np()
    ref = O.decode_attention(case.q, pool, case.Hkv, case.page_table, case.seq_lens, case.r_k, case.r_v)
    for ns in (0, 1, 3):
        got = dc.decode("f32", num_splits=ns)
        assert np.isfinite(got).all(), ns
        err = max_abs_rel(got, ref)
        assert err <= TOL, (ns, err)


@pytest.mark.parametrize("val_bits", [2, 4])
def test_decode_value_scales_hadamard_and_wide_values(val_bits):
    """The Hadamard kernels (their P.V rounding correction included) and 4-bit values
    over the same range."""
    dev = require_gpu()
    case, x, w = _range_case("per_position", 4, 2, [1400, 260], seed=977 + val_bits, rotation="hadamard")
    dc = DeviceCase(case, dev, val_bits=val_bits)
    _prerotated(dc, x, w)
    r_k, r_v = dense_rotations(case)
    ref = O.decode_attention(case.q, dc.pool_np(), case.Hkv, case.page_table, case.seq_lens, r_k, r_v,
                             val_bits=val_bits)
    for ns in (0, 2):
        got = dc.decode("f32", num_splits=ns)
        assert np.isfinite(got).all()
        assert max_abs_rel(got, ref) <= TOL, ns


def test_stored_value_scales_span_the_range():
    """The constructed cache really stores value scales from about 1e-4 to 4e3."""
    dev = require_gpu()
    case, x, w = _range_case("per_position", 4, 1, [1000], seed=990)
    dc = DeviceCase(case, dev)
    _prerotated(dc, x, w)
    pool = dc.pool_np()
    T = int(case.seq_lens[0])
    s_v = np.concatenate([O.unpack_block(O.block_view(pool, case.page_table[0, i], 0, case.Hkv))[4]
                          for i in range((T + 15) // 16)]).astype(np.float64)[:T]
    assert s_v.min() < 2e-4 and s_v.max() > 2e3


@pytest.mark.parametrize("g", [4, 8, 16])
def test_nan_metadata_in_unread_slots_weighs_nothing(g):
    """Pool bytes 0xff (NaN scales and zeros) in stale slots past each sequence's end and
    on an absent page: the output is finite and equals the oracle's."""
    dev = require_gpu()
    import torch
    lens = [333, 70]
    case = I.make_case("nanmeta", 1200 + g, B=2, Hq=g * 2, Hkv=2, seq_lens=lens, dtype="f32",
                       table_policy="interleaved")
    table = case.page_table.copy()
    table[0, 5] = -1  # an absent page in the middle of sequence 0
    case = dataclasses.replace(case, page_table=table)
    dc = DeviceCase(case, dev)
    dc.pool.fill_(255)
    keep = np.nonzero(~((case.tok_seq == 0) & (case.tok_pos // 16 == 5)))[0]
    x, w = O.rotated_inputs(case.k, case.v, case.mu, case.r_k, case.r_v)
    from rotated_int2_kv_centering_amd import kvq
    kvq.kvq_quant_append(dc.cache, dev_tensor(x[keep].astype(np.float32), dev),
                         dev_tensor(w[keep].astype(np.float32), dev), kvq.KVQ_F32_ROTATED, len(keep),
                         dev_tensor(case.slots[keep].astype(np.int32), dev), None, None, None, None)
    torch.cuda.synchronize()
    pool = dc.pool_np()
    ref = O.decode_attention(case.q, pool, case.Hkv, table, case.seq_lens, case.r_k, case.r_v)
    for ns in (0, 1, 4):
        got = dc.decode("f32", num_splits=ns)
        assert np.isfinite(got).all(), ns
        assert max_abs_rel(got, ref) <= TOL, ns
