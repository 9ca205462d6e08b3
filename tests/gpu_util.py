"""Helpers for the GPU tests: move a synthetic case to the device and call libkvq.

Only marshalling lives here; every computation under test runs in the HIP
kernels behind the C ABI, and every expected value comes from the oracle.
"""

from __future__ import annotations

import numpy as np
import pytest

import kvq_inputs as I
from oracle import kvq_oracle as O

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None


def require_gpu():
    if torch is None or not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from rotated_int2_kv_centering_amd import kvq
    kvq.load()  # raises if the library is missing: no fallback exists
    return torch.device("cuda:0")


def dev_tensor(a: np.ndarray, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_tensor(bits: np.ndarray, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


class DeviceCase:
    """Device copies of a case's inputs and one zeroed pool."""

    def __init__(self, case: I.Case, dev, num_pages=None, clip_ratio=0.0, group_size=32, key_bits=2, val_bits=2):
        from rotated_int2_kv_centering_amd import kvq
        self.c = case
        self.dev = dev
        self.num_pages = int(num_pages or case.num_pages)
        self.key_bits = key_bits
        self.val_bits = val_bits
        self.group_size = group_size
        # the block layout's parameters, as the oracle's layout functions take them
        self.layout = dict(key_bits=key_bits, val_bits=val_bits, group=group_size)
        self.pool = torch.zeros(O.pool_bytes(self.num_pages, case.Hkv, key_bits, val_bits, group_size),
                                dtype=torch.uint8, device=dev)
        self.cache = kvq.make_cache(case.Hkv, self.num_pages, self.pool, clip_ratio=clip_ratio, group_size=group_size,
                                    key_bits=key_bits, val_bits=val_bits,
                                    rotation=kvq.KVQ_ROT_HADAMARD if case.rotation == "hadamard" else kvq.KVQ_ROT_DENSE)
        if case.dtype == "bf16":
            self.k = bf16_tensor(case.k_bits, dev)
            self.v = bf16_tensor(case.v_bits, dev)
            self.q = bf16_tensor(case.q_bits, dev)
            self.in_dtype = kvq.KVQ_BF16
        else:
            self.k = dev_tensor(case.k.astype(np.float32), dev)
            self.v = dev_tensor(case.v.astype(np.float32), dev)
            self.q = dev_tensor(case.q.astype(np.float32), dev)
            self.in_dtype = kvq.KVQ_F32
        self.slots = dev_tensor(case.slots.astype(np.int32), dev)
        self.mu = dev_tensor(case.mu.astype(np.float32), dev)
        self.r_k = dev_tensor(case.r_k.astype(np.float32), dev)
        self.r_v = dev_tensor(case.r_v.astype(np.float32), dev)
        self.table = dev_tensor(case.page_table.astype(np.int32), dev)
        self.seq_lens = dev_tensor(case.seq_lens.astype(np.int32), dev)

    def append(self, rot_out=True, chunk=None):
        """Quantize-append every token of the case (optionally in chunks); returns rot_out or None."""
        from rotated_int2_kv_centering_amd import kvq
        n = self.c.n_tokens
        rot = torch.empty((n, self.c.Hkv, 2, 128), dtype=torch.float32, device=self.dev) if rot_out else None
        chunk = chunk or max(n, 1)
        for s in range(0, n, chunk):
            e = min(n, s + chunk)
            kvq.kvq_quant_append(self.cache, self.k[s:e], self.v[s:e], self.in_dtype, e - s, self.slots[s:e], self.mu,
                                 self.r_k, self.r_v, rot[s:e] if rot is not None else None)
        torch.cuda.synchronize()
        return rot

    def window(self, sinks, recent, fill=True, tokens=None, mu="case"):
        """A zeroed exact-window buffer for the case (kept alive on self), filled by
        kvq_window_fill with every token (or the token indices ``tokens``)."""
        from rotated_int2_kv_centering_amd import kvq
        c = self.c
        probe = kvq.make_window(sinks, recent, c.B)
        nbytes = kvq.kvq_window_bytes(probe, c.Hkv)
        self.win_buf = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=self.dev)
        self.win = kvq.make_window(sinks, recent, c.B, self.win_buf, self.mu if mu == "case" else mu)
        if fill:
            sel = np.arange(c.n_tokens) if tokens is None else np.asarray(tokens, np.int64)
            if len(sel):
                idx = dev_tensor(sel, self.dev)
                kvq.kvq_window_fill(self.win, c.Hkv, self.k[idx].contiguous(), self.v[idx].contiguous(), self.in_dtype,
                                    len(sel), dev_tensor(c.tok_seq[sel].astype(np.int32), self.dev),
                                    dev_tensor(c.tok_pos[sel].astype(np.int32), self.dev), self.seq_lens)
            torch.cuda.synchronize()
        return self.win

    def decode(self, out_dtype="f32", num_splits=0, q=None, table=None, ws=None, max_seq=None, window=None):
        from rotated_int2_kv_centering_amd import kvq
        c = self.c
        max_seq = int(c.seq_lens.max(initial=0)) if max_seq is None else int(max_seq)
        ws_bytes = kvq.kvq_decode_workspace_bytes(c.B, c.Hq, c.Hkv, max_seq, num_splits)
        if ws is None:
            ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=self.dev)
        else:
            assert ws.numel() >= ws_bytes
            ws_bytes = ws.numel()
        tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
        out = torch.full((c.B, c.Hq, 128), float("nan"), dtype=tdt, device=self.dev)
        table = self.table if table is None else table
        kvq.kvq_decode_attn(self.cache, self.q if q is None else q, self.in_dtype, c.B, c.Hq, table,
                            int(table.shape[1]), self.seq_lens, max_seq, self.r_k, self.r_v, 0.0, out,
                            kvq.KVQ_F32 if out_dtype == "f32" else kvq.KVQ_BF16, ws, ws_bytes, num_splits,
                            window=window)
        torch.cuda.synchronize()
        if out_dtype == "f32":
            return out.cpu().numpy()
        return out.view(torch.int16).cpu().numpy().view(np.uint16)

    def step(self, k_new, v_new, out_dtype="f32", num_splits=0, ws=None, mu="case", window=None):
        """kvq_decode_step with the case's queries, tables and lengths; k_new/v_new are
        device tensors [B][H_kv][128] in the case's dtype."""
        from rotated_int2_kv_centering_amd import kvq
        c = self.c
        max_seq = int(c.seq_lens.max(initial=0))
        ws_bytes = kvq.kvq_decode_workspace_bytes(c.B, c.Hq, c.Hkv, max_seq, num_splits)
        if ws is None:
            ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=self.dev)
        else:
            ws_bytes = ws.numel()
        tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
        out = torch.full((c.B, c.Hq, 128), float("nan"), dtype=tdt, device=self.dev)
        kvq.kvq_decode_step(self.cache, k_new, v_new, self.in_dtype, self.mu if mu == "case" else mu, self.q,
                            self.in_dtype, c.B, c.Hq, self.table, int(self.table.shape[1]), self.seq_lens, max_seq,
                            self.r_k, self.r_v, 0.0, out, kvq.KVQ_F32 if out_dtype == "f32" else kvq.KVQ_BF16, ws,
                            ws_bytes, num_splits, window=window)
        torch.cuda.synchronize()
        if out_dtype == "f32":
            return out.cpu().numpy()
        return out.view(torch.int16).cpu().numpy().view(np.uint16)

    def pool_np(self) -> np.ndarray:
        return self.pool.cpu().numpy()


def dense_rotations(case):
    """(R_K, R_V) as dense [H_kv][128][128] matrices for oracle calls: the case's own,
    or the oracle's matrices of its Hadamard signs."""
    if case.rotation == "hadamard":
        return O.hadamard_rotation(case.r_k), O.hadamard_rotation(case.r_v)
    return case.r_k, case.r_v


def max_abs_rel(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of max_c |got - ref| / max_c |ref| (rows of zeros must match exactly)."""
    got = np.asarray(got, np.float64).reshape(-1, 128)
    ref = np.asarray(ref, np.float64).reshape(-1, 128)
    worst = 0.0
    for g, r in zip(got, ref):
        den = np.abs(r).max()
        if den == 0:
            if np.abs(g).max() != 0:
                return float("inf")
            continue
        worst = max(worst, np.abs(g - r).max() / den)
    return worst


def rotation_error_bound(a_rows: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Bound on |fp32 sequential-FMA (a R) - fp64 (a R) rounded to fp32| per output.

    With u = 2^-24, 128 fused multiply-adds, one rounding of the centred input
    and the oracle's final rounding: (130 u) * sum_i |a_i| |R_ij| + u |x_j|.
    """
    u = 2.0 ** -24
    mag = np.abs(a_rows.astype(np.float64)) @ np.abs(r.astype(np.float64))
    return 2 * 130 * u * mag
