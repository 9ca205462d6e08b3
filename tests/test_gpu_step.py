"""GPU parity of the fused decode step (append of the newest token + decode in one
kernel, kvq_decode_step) through the C ABI.

Each case first fills the cache with every token except the newest of each
sequence, and plants a different token's codes in the newest token's slot, so a
step that read the old slot contents would be caught.  Then:
* the pool after kvq_decode_step equals, byte for byte, the pool after
  kvq_quant_append of the newest tokens (both kernels quantize identically);
* the step's output is within 2e-3 max-abs-rel of the oracle decode on the
  step's own pool, and its bf16 output is the fp32 output rounded to nearest even.
"""

import numpy as np
import pytest

import kvq_inputs as I
from oracle import kvq_oracle as O
from tests.gpu_util import DeviceCase, bf16_tensor, dev_tensor, max_abs_rel, require_gpu

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _newest(case):
    """Token index of position T_b - 1 per sequence (-1 for empty sequences)."""
    idx = np.full(case.B, -1, np.int64)
    for b in range(case.B):
        sel = np.nonzero(case.tok_seq == b)[0]
        if len(sel):
            idx[b] = sel[-1]
    return idx


def _new_kv(case, dc, newest, dev):
    """k_new, v_new device tensors [B][H_kv][128] in the case's dtype (zeros for empty sequences)."""
    take = np.where(newest >= 0, newest, 0)
    if case.dtype == "bf16":
        kb = np.where((newest >= 0)[:, None, None], case.k_bits[take], 0).astype(np.uint16)
        vb = np.where((newest >= 0)[:, None, None], case.v_bits[take], 0).astype(np.uint16)
        return bf16_tensor(kb, dev), bf16_tensor(vb, dev)
    k = np.where((newest >= 0)[:, None, None], case.k[take], 0).astype(np.float32)
    v = np.where((newest >= 0)[:, None, None], case.v[take], 0).astype(np.float32)
    return dev_tensor(k, dev), dev_tensor(v, dev)


def _prefill(dc, case, newest):
    """Append every token but the newest ones; then plant another token's codes in the newest slots."""
    from rotated_int2_kv_centering_amd import kvq
    import torch

    old = np.setdiff1d(np.arange(case.n_tokens), newest[newest >= 0])
    sel = dev_tensor(old, dc.dev)
    if len(old):
        kvq.kvq_quant_append(dc.cache, dc.k[sel].contiguous(), dc.v[sel].contiguous(), dc.in_dtype, len(old),
                             dc.slots[sel].contiguous(), dc.mu, dc.r_k, dc.r_v)
    new_idx = newest[newest >= 0]
    if len(new_idx):  # stale content: token 0's key/value written into the newest slots
        src = dev_tensor(np.zeros(len(new_idx), np.int64), dc.dev)
        kvq.kvq_quant_append(dc.cache, dc.k[src].contiguous(), dc.v[src].contiguous(), dc.in_dtype, len(new_idx),
                             dc.slots[dev_tensor(new_idx, dc.dev)].contiguous(), dc.mu, dc.r_k, dc.r_v)
    torch.cuda.synchronize()


def _append_newest(dc, newest):
    from rotated_int2_kv_centering_amd import kvq
    import torch

    new_idx = newest[newest >= 0]
    if len(new_idx):
        sel = dev_tensor(new_idx, dc.dev)
        kvq.kvq_quant_append(dc.cache, dc.k[sel].contiguous(), dc.v[sel].contiguous(), dc.in_dtype, len(new_idx),
                             dc.slots[sel].contiguous(), dc.mu, dc.r_k, dc.r_v)
    torch.cuda.synchronize()


STEP_SHAPES = [
    # (B, Hq, Hkv, seq_lens, policy, dtype)
    (1, 4, 1, [256], "contiguous", "f32"),      # the tiny case's shape
    (1, 4, 1, [1], "contiguous", "bf16"),       # the new token is the whole context
    (1, 4, 1, [16], "permuted", "bf16"),        # last slot of a page
    (1, 4, 1, [17], "permuted", "bf16"),        # first slot of a fresh page
    (3, 8, 2, [0, 5, 100], "interleaved", "bf16"),
    (2, 2, 2, [77, 300], "interleaved", "bf16"),     # g = 1
    (2, 32, 8, [1000, 257], "interleaved", "bf16"),  # g = 4
    (2, 64, 8, [513, 1024], "interleaved", "bf16"),  # g = 8
    (1, 16, 1, [300], "permuted", "f32"),            # g = 16
]


@pytest.mark.parametrize("shape", STEP_SHAPES,
                         ids=lambda s: f"B{s[0]}_Hq{s[1]}_Hkv{s[2]}_T{'-'.join(map(str, s[3]))}_{s[5]}")
def test_step_equals_append_then_decode(shape):
    dev = require_gpu()
    B, Hq, Hkv, lens, policy, dtype = shape
    case = I.make_case("s", 300 + sum(lens) + Hq, B=B, Hq=Hq, Hkv=Hkv, seq_lens=lens, dtype=dtype,
                       table_policy=policy, n_outliers=4 if dtype == "f32" else 3)
    newest = _newest(case)
    a = DeviceCase(case, dev)
    _prefill(a, case, newest)
    b = DeviceCase(case, dev)
    b.pool.copy_(a.pool)
    k_new, v_new = _new_kv(case, b, newest, dev)

    _append_newest(a, newest)
    for ns in (0, 1, 7):  # the step is idempotent: it rewrites the same token each time
        got = b.step(k_new, v_new, "f32", num_splits=ns)
        assert np.array_equal(b.pool_np(), a.pool_np()), f"pool differs from kvq_quant_append's (splits {ns})"
        ref = O.decode_attention(case.q, b.pool_np(), Hkv, case.page_table, case.seq_lens, case.r_k, case.r_v)
        err = max_abs_rel(got, ref)
        assert err <= TOL, (ns, err)
    got16 = b.step(k_new, v_new, "bf16")
    got32 = b.step(k_new, v_new, "f32")
    assert np.array_equal(got16, I.bf16_bits(got32.astype(np.float32)))


def test_step_reads_no_stale_slot():
    """Two different stale contents in the newest slot give the same step output."""
    dev = require_gpu()
    case = I.make_case("s2", 71, B=2, Hq=8, Hkv=2, seq_lens=[40, 97], table_policy="permuted")
    newest = _newest(case)
    outs = []
    for stale in (0, 5):
        dc = DeviceCase(case, dev)
        from rotated_int2_kv_centering_amd import kvq
        import torch
        old = np.setdiff1d(np.arange(case.n_tokens), newest)
        sel = dev_tensor(old, dev)
        kvq.kvq_quant_append(dc.cache, dc.k[sel].contiguous(), dc.v[sel].contiguous(), dc.in_dtype, len(old),
                             dc.slots[sel].contiguous(), dc.mu, dc.r_k, dc.r_v)
        src = dev_tensor(np.full(len(newest), stale, np.int64), dev)
        kvq.kvq_quant_append(dc.cache, dc.k[src].contiguous(), dc.v[src].contiguous(), dc.in_dtype, len(newest),
                             dc.slots[dev_tensor(newest, dev)].contiguous(), dc.mu, dc.r_k, dc.r_v)
        torch.cuda.synchronize()
        k_new, v_new = _new_kv(case, dc, newest, dev)
        outs.append(dc.step(k_new, v_new, "f32"))
    assert np.array_equal(outs[0], outs[1])


def test_step_with_absent_last_page_appends_nothing():
    """The page holding position T-1 is outside the pool: nothing is written and that
    page's positions are not attended (oracle with the same absent page)."""
    dev = require_gpu()
    case = I.make_case("s3", 72, B=2, Hq=8, Hkv=2, seq_lens=[40, 33], table_policy="contiguous")
    newest = _newest(case)
    dc = DeviceCase(case, dev)
    _prefill(dc, case, newest)
    before = dc.pool_np().copy()
    table = case.page_table.copy()
    table[1, 2] = case.num_pages + 3  # page of position 32 of sequence 1
    dc.table = dev_tensor(table.astype(np.int32), dev)
    k_new, v_new = _new_kv(case, dc, newest, dev)
    got = dc.step(k_new, v_new, "f32")
    after = dc.pool_np()
    # sequence 0's newest token was written; nothing else changed
    blk = lambda p, h: slice((p * case.Hkv + h) * 1536, (p * case.Hkv + h + 1) * 1536)
    p0 = int(table[0, 39 // 16])
    mask = np.ones_like(before, bool)
    for h in range(case.Hkv):
        mask[blk(p0, h)] = False
    assert np.array_equal(after[mask], before[mask])
    ref = O.decode_attention(case.q, after, case.Hkv, table, case.seq_lens, case.r_k, case.r_v,
                             num_pages=case.num_pages)
    assert max_abs_rel(got, ref) <= TOL


def test_step_without_mu_matches_zero_mu():
    dev = require_gpu()
    case = I.make_case("s4", 73, B=1, Hq=4, Hkv=1, seq_lens=[50], table_policy="contiguous", mu_zero=True)
    newest = _newest(case)
    outs = []
    for mu in ("case", None):
        dc = DeviceCase(case, dev)
        _prefill(dc, case, newest)
        k_new, v_new = _new_kv(case, dc, newest, dev)
        outs.append((dc.step(k_new, v_new, "f32", mu=mu), dc.pool_np()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_step_with_clip_ratio_writes_the_appended_bytes():
    """The step quantizes the new token with the cache's clip ratio: its pool equals
    kvq_quant_append's with the same c, and differs from the unclipped one."""
    dev = require_gpu()
    case = I.make_case("s5", 74, B=2, Hq=8, Hkv=2, seq_lens=[300, 41], table_policy="interleaved")
    newest = _newest(case)
    dc = DeviceCase(case, dev, clip_ratio=0.75)
    _prefill(dc, case, newest)
    k_new, v_new = _new_kv(case, dc, newest, dev)
    got = dc.step(k_new, v_new, "f32")
    ref_dc = DeviceCase(case, dev, clip_ratio=0.75)
    ref_dc.pool.copy_(dc.pool)
    _append_newest(ref_dc, newest)
    assert np.array_equal(ref_dc.pool_np(), dc.pool_np())
    plain = DeviceCase(case, dev)
    plain.pool.copy_(dc.pool)
    _append_newest(plain, newest)
    assert not np.array_equal(plain.pool_np(), dc.pool_np())
    ref = O.decode_attention(case.q, dc.pool_np(), case.Hkv, case.page_table, case.seq_lens, case.r_k, case.r_v)
    assert max_abs_rel(got, ref) <= TOL


@pytest.mark.parametrize("name", ["llama8b_t128k"])
def test_full_size_step_all_heads(name):
    """The bench's workload and launch configuration: one step at 128K context, all 32 query heads."""
    dev = require_gpu()
    case = I.llama8b_case(131072)
    newest = _newest(case)
    dc = DeviceCase(case, dev)
    _prefill(dc, case, newest)
    k_new, v_new = _new_kv(case, dc, newest, dev)
    got = dc.step(k_new, v_new, "f32")
    pool = dc.pool_np()
    # the cache after the step equals the cache after kvq_quant_append of the newest token
    ref_dc = DeviceCase(case, dev)
    ref_dc.pool.copy_(dc.pool)
    _append_newest(ref_dc, newest)
    assert np.array_equal(ref_dc.pool_np(), pool)
    # every query head of the step, each against the oracle on the step's pool
    ref = O.decode_attention(case.q, pool, case.Hkv, case.page_table, case.seq_lens, case.r_k, case.r_v)
    for j in range(case.Hq):
        assert max_abs_rel(got[0, j], ref[0, j]) <= TOL, j
