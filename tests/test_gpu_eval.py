"""GPU parity of the output-error evaluator (OptR section 3.2, Eq. (6)-(10)) and
of the append's per-token squared errors, through the C ABI.

The cache is written by kvq_quant_append_err over every token of the case (rows
in sequence order, so row_offsets are the cumulative lengths); the oracle's
output_error then reads the GPU's own pool with the exact k, v and W_O.

Tolerances (fp32 kernel against the fp64 oracle):
* dy_k, dy_v: 2e-3 max-abs-rel per (sequence, head) row.  Each is a difference
  of two attention readouts (B - A, C - B) whose fp32 accumulation errors are
  ~1e-6 of max |v|, while the differences themselves are the INT2 error's
  effect, a few percent of the readouts or more; W_O maps both alike.
* e_out: 5e-3 relative (it is quadratic in dy).
* e_rec and the per-token squared errors: 1e-4 relative (fp32 sums of squares
  of fp32 differences; the fp32 rotation's own error is ~1e-7 of |x|).
"""

import numpy as np
import pytest

import kvq_inputs as I
from oracle import kvq_oracle as O
from tests.gpu_util import DeviceCase, bf16_tensor, dense_rotations, dev_tensor, max_abs_rel, require_gpu

pytestmark = pytest.mark.gpu

TOL_DY = 2e-3
TOL_EOUT = 5e-3
TOL_EREC = 1e-4


def _rows_max_rel(got, ref):
    """max over rows of max |got - ref| / max |ref| (a zero row must be matched exactly)."""
    got = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    worst = 0.0
    for g, r in zip(got, ref):
        den = np.abs(r).max()
        if den == 0:
            if np.abs(g).max() != 0:
                return float("inf")
            continue
        worst = max(worst, np.abs(g - r).max() / den)
    return worst


class Evaluated:
    """Append with squared errors, then kvq_output_error; results on the host."""

    def __init__(self, case, dev, d_model=96, w_dtype="bf16", table=None, with_err=True, seed=7, key_bits=2,
                 val_bits=2, group=32):
        import torch
        from rotated_int2_kv_centering_amd import kvq
        self.c = c = case
        self.key_bits = key_bits
        self.val_bits = val_bits
        self.dc = dc = DeviceCase(case, dev, key_bits=key_bits, val_bits=val_bits, group_size=group)
        n = c.n_tokens
        self.sq_err = torch.zeros((max(n, 1), c.Hkv, 2, 2), dtype=torch.float32, device=dev)
        kvq.kvq_quant_append_err(dc.cache, dc.k, dc.v, dc.in_dtype, n, dc.slots, dc.mu, dc.r_k, dc.r_v, None,
                                 self.sq_err)
        torch.cuda.synchronize()
        rng = np.random.default_rng(seed)
        w = (rng.standard_normal((d_model, c.Hq * 128)) / np.sqrt(128)).astype(np.float32)
        if w_dtype == "bf16":
            self.w_bits = I.bf16_bits(w)
            self.w_o = I.bf16_to_f32(self.w_bits)
            w_dev, w_kind = bf16_tensor(self.w_bits, dev), kvq.KVQ_BF16
        else:
            self.w_o = w
            w_dev, w_kind = dev_tensor(w, dev), kvq.KVQ_F32
        self.table = c.page_table if table is None else table
        table_dev = dev_tensor(self.table.astype(np.int32), dev)
        max_seq = int(c.seq_lens.max(initial=0))
        ws_bytes = kvq.kvq_output_error_workspace_bytes(c.B, c.Hq, c.Hkv, max_seq, d_model)
        self.ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        row_off = np.concatenate([[0], np.cumsum(c.seq_lens)[:-1]]).astype(np.int64)
        outs = dict(dy_k=(c.B, c.Hq, d_model), dy_v=(c.B, c.Hq, d_model), e_out=(c.B, c.Hq), e_rec=(c.B, c.Hkv))
        self.t = {k: torch.full(s, float("nan"), dtype=torch.float32, device=dev) for k, s in outs.items()}
        self.args = (dc.cache, dc.q, dc.in_dtype, c.B, c.Hq, table_dev, int(self.table.shape[1]), dc.seq_lens, max_seq,
                     dc.k, dc.v, dc.in_dtype, dev_tensor(row_off, dev), self.sq_err if with_err else None, dc.r_k,
                     dc.r_v, 0.0, w_dev, w_kind, d_model)
        self.run()

    def run(self):
        import torch
        from rotated_int2_kv_centering_amd import kvq
        t = self.t
        kvq.kvq_output_error(*self.args, t["dy_k"], t["dy_v"], t["e_out"], t["e_rec"], self.ws, self.ws.numel())
        torch.cuda.synchronize()
        return {k: v.cpu().numpy() for k, v in t.items()}

    def oracle(self):
        c = self.c
        r_k, r_v = dense_rotations(c)
        ks = [c.k[c.tok_seq == b] for b in range(c.B)]
        vs = [c.v[c.tok_seq == b] for b in range(c.B)]
        dy_k, dy_v, e_out, e_rec = O.output_error(c.q, self.dc.pool_np(), c.Hkv, self.table, c.seq_lens, ks, vs, c.mu,
                                                  r_k, r_v, self.w_o, num_pages=c.num_pages, **self.dc.layout)
        return dict(dy_k=dy_k, dy_v=dy_v, e_out=e_out, e_rec=e_rec)


def _check(got, ref, erec=True):
    assert _rows_max_rel(got["dy_k"], ref["dy_k"]) <= TOL_DY, _rows_max_rel(got["dy_k"], ref["dy_k"])
    assert _rows_max_rel(got["dy_v"], ref["dy_v"]) <= TOL_DY, _rows_max_rel(got["dy_v"], ref["dy_v"])
    np.testing.assert_allclose(got["e_out"], ref["e_out"], rtol=TOL_EOUT, atol=0)
    if erec:
        np.testing.assert_allclose(got["e_rec"], ref["e_rec"], rtol=TOL_EREC, atol=0)


SHAPES = [
    # (B, Hq, Hkv, lens, dtype, w_dtype, rotation)
    (3, 8, 2, [50, 0, 33], "bf16", "bf16", "dense"),        # g = 4, an empty sequence
    (2, 2, 2, [77, 300], "f32", "f32", "dense"),            # g = 1, fp32 inputs and W_O
    (2, 64, 8, [513, 100], "bf16", "bf16", "dense"),        # g = 8
    (1, 16, 1, [300], "bf16", "f32", "dense"),              # g = 16: two head chunks
    (2, 32, 8, [1000, 17], "bf16", "bf16", "hadamard"),     # Hadamard rotation
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}_Hq{s[1]}_Hkv{s[2]}_{s[4]}_{s[6]}")
def test_output_error_matches_the_oracle(shape):
    dev = require_gpu()
    B, Hq, Hkv, lens, dtype, w_dtype, rot = shape
    case = I.make_case("ev", 200 + sum(lens) + Hq, B=B, Hq=Hq, Hkv=Hkv, seq_lens=lens, dtype=dtype,
                       table_policy="interleaved", rotation=rot)
    ev = Evaluated(case, dev, w_dtype=w_dtype)
    got = ev.run()
    _check(got, ev.oracle())
    # a second call on the same workspace gives the same bytes (counters were reset)
    again = ev.run()
    for k in got:
        np.testing.assert_array_equal(got[k], again[k])


def test_absent_page_and_missing_errors():
    """A page outside the pool drops out of every readout (oracle with the same table);
    without sq_err, e_rec is 0 and nothing else changes."""
    dev = require_gpu()
    case = I.make_case("eva", 211, B=2, Hq=8, Hkv=2, seq_lens=[40, 70], table_policy="contiguous")
    table = case.page_table.copy()
    table[1, 2] = case.num_pages + 5
    ev = Evaluated(case, dev, table=table)
    got = ev.run()
    _check(got, ev.oracle())
    ev2 = Evaluated(case, dev, table=table, with_err=False)
    got2 = ev2.run()
    assert np.all(got2["e_rec"] == 0)
    for k in ("dy_k", "dy_v", "e_out"):
        np.testing.assert_array_equal(got2[k], got[k])


@pytest.mark.parametrize("dtype,lens", [("bf16", [40, 33]), ("f32", [300, 77])])
def test_append_squared_errors(dtype, lens):
    """kvq_quant_append_err writes the same cache bytes as kvq_quant_append, and each
    token's two half sums equal sum (x - level)^2 over the kernel's own rotated rows
    (rot_out) and the oracle quantizer's levels."""
    import torch
    from rotated_int2_kv_centering_amd import kvq
    dev = require_gpu()
    case = I.make_case("eve", 222, B=2, Hq=8, Hkv=4, seq_lens=lens, dtype=dtype, table_policy="interleaved")
    ref = DeviceCase(case, dev)
    ref.append(rot_out=False)
    dc = DeviceCase(case, dev)
    n = case.n_tokens
    rot = torch.empty((n, case.Hkv, 2, 128), dtype=torch.float32, device=dev)
    err = torch.full((n, case.Hkv, 2, 2), float("nan"), dtype=torch.float32, device=dev)
    kvq.kvq_quant_append_err(dc.cache, dc.k, dc.v, dc.in_dtype, n, dc.slots, dc.mu, dc.r_k, dc.r_v, rot, err)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dc.pool_np(), ref.pool_np())
    rot = rot.cpu().numpy()
    err = err.cpu().numpy()
    for t in range(2):
        x = rot[:, :, t, :]
        lv = O.int2_dequantize(*O.int2_quantize(x))
        sq = ((x.astype(np.float64) - lv) ** 2).reshape(n, case.Hkv, 2, 64).sum(-1)
        np.testing.assert_allclose(err[:, :, t, :], sq, rtol=TOL_EREC, atol=1e-30)


def test_full_size_llama8b_t32k():
    """The 8B shape at 32K with a 4096-wide W_O: every head against the oracle."""
    dev = require_gpu()
    case = I.llama8b_case(32768)
    ev = Evaluated(case, dev, d_model=4096)
    _check(ev.run(), ev.oracle())


def test_full_size_llama8b_t128k():
    """The evaluator's benchmark configuration: the 8B shape at 128K with a 4096-wide
    bf16 W_O, every head against the oracle."""
    dev = require_gpu()
    case = I.llama8b_case(131072)
    ev = Evaluated(case, dev, d_model=4096)
    _check(ev.run(), ev.oracle())


@pytest.mark.parametrize("bits,group", [(3, 32), (4, 32), (3, 128), (4, 64)])
@pytest.mark.parametrize("shape", [(2, 32, 8, [700, 65]), (1, 64, 8, [400])], ids=lambda s: f"Hq{s[1]}")
def test_output_error_with_wide_keys(shape, bits, group):
    """3- and 4-bit keys: the evaluator reads the keys' high-bit plane (one word per record for 3 bits, two
    for 4) after the metadata, whose size follows the group size."""
    dev = require_gpu()
    B, Hq, Hkv, lens = shape
    case = I.make_case("evk", 240 + sum(lens) + Hq + bits, B=B, Hq=Hq, Hkv=Hkv, seq_lens=lens,
                       table_policy="interleaved")
    ev = Evaluated(case, dev, key_bits=bits, group=group)
    _check(ev.run(), ev.oracle())
