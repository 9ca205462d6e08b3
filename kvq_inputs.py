"""Seeded synthetic inputs for rotated INT2 KV-cache decode.

This module only draws data.  It holds none of the method's arithmetic: no
centering, rotation, quantization, packing or attention.  Both the CPU oracle's
tests and the GPU path's tests/benchmark take their inputs from here.

Recipe (one ``numpy.random.Generator`` per named stream, so the order in which
streams are drawn never changes any value):

* keys    k = N(0,1); a few outlier channels per KV head are multiplied by 20;
          a per-(KV head, channel) offset ~ N(0, 3^2) is added.
* values  v = N(0,1); queries q = N(0,1).
* outlier channels: 4 per KV head for the tiny case, round(0.02*128) = 3 for
          the Llama-shaped cases, chosen without replacement.
* R_K, R_V: Q of a QR factorisation of a seeded 128x128 Gaussian, with the
          columns' signs fixed by sign(diag(R_qr)); computed in fp64 and stored
          fp32.  The tiny case uses one matrix for both K and V.
* mu:     per-(KV head, channel) mean of the (dtype-rounded) keys of the first
          ``mu_tokens`` positions of sequence 0, fp64 mean stored fp32.
* dtype:  the tiny case keeps fp32; the others round q, k, v to bf16
          (round-to-nearest-even), carried here as uint16 bit patterns.
* page tables: contiguous, a seeded permutation of the pool, or an
          interleaved allocator (free list = a seeded permutation; for page
          index i = 0, 1, ... visit the sequences in a fresh seeded order and
          pop one page for each sequence that still needs page i).
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

HEAD_DIM = 128
PAGE_SIZE = 16

_STREAMS = {
    "q": 1, "k": 2, "v": 3, "outliers": 4, "offsets": 5, "r_k": 6, "r_v": 7,
    "lengths": 8, "pages": 9, "append": 10, "misc": 11,
}


def rng_for(seed: int, stream: str, sub: int = 0) -> np.random.Generator:
    """Independent generator for one named stream of one case."""
    return np.random.default_rng(np.random.SeedSequence([int(seed), _STREAMS[stream], int(sub)]))


# ---------------------------------------------------------------- bf16 helpers
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even); return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # round-to-nearest-even on the 16 discarded bits (finite inputs only)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------ random matrices
def random_orthogonal(rng: np.random.Generator, d: int = HEAD_DIM) -> np.ndarray:
    """Haar-like random orthogonal d x d matrix, fp32."""
    a = rng.standard_normal((d, d))
    qm, rm = np.linalg.qr(a)
    qm = qm * np.sign(np.diag(rm))[None, :]
    return qm.astype(np.float32)


# ----------------------------------------------------------------- page tables
def page_table_contiguous(seq_lens: np.ndarray, page_size: int = PAGE_SIZE):
    pages_per = (np.asarray(seq_lens) + page_size - 1) // page_size
    max_pages = int(max(1, pages_per.max(initial=0)))
    table = np.full((len(seq_lens), max_pages), -1, dtype=np.int32)
    nxt = 0
    for b, n in enumerate(pages_per):
        table[b, :n] = np.arange(nxt, nxt + n, dtype=np.int32)
        nxt += int(n)
    return table, nxt


def page_table_permuted(seq_lens: np.ndarray, rng: np.random.Generator, page_size: int = PAGE_SIZE,
                        num_pages: Optional[int] = None):
    pages_per = (np.asarray(seq_lens) + page_size - 1) // page_size
    total = int(pages_per.sum())
    num_pages = total if num_pages is None else int(num_pages)
    assert num_pages >= total
    perm = rng.permutation(num_pages).astype(np.int32)
    max_pages = int(max(1, pages_per.max(initial=0)))
    table = np.full((len(seq_lens), max_pages), -1, dtype=np.int32)
    nxt = 0
    for b, n in enumerate(pages_per):
        table[b, :n] = perm[nxt:nxt + n]
        nxt += int(n)
    return table, num_pages


def page_table_interleaved(seq_lens: np.ndarray, rng: np.random.Generator, page_size: int = PAGE_SIZE,
                           num_pages: Optional[int] = None):
    pages_per = (np.asarray(seq_lens) + page_size - 1) // page_size
    total = int(pages_per.sum())
    num_pages = total if num_pages is None else int(num_pages)
    assert num_pages >= total
    free = list(rng.permutation(num_pages).astype(np.int32)[::-1])  # pop() from the end
    max_pages = int(max(1, pages_per.max(initial=0)))
    table = np.full((len(seq_lens), max_pages), -1, dtype=np.int32)
    for i in range(max_pages):
        for b in rng.permutation(len(seq_lens)):
            if i < pages_per[b]:
                table[b, i] = free.pop()
    return table, num_pages


def slots_for_positions(table: np.ndarray, b: np.ndarray, pos: np.ndarray, page_size: int = PAGE_SIZE):
    """Global slot index page*page_size + offset for (sequence, position) pairs."""
    b = np.asarray(b, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    return (table[b, pos // page_size].astype(np.int64) * page_size + pos % page_size).astype(np.int32)


# ----------------------------------------------------------------- the cases
@dataclasses.dataclass
class Case:
    """One synthetic decode workload.

    Token arrays are flattened over (sequence, position) in that order:
    ``k[n, h, :]`` is KV head ``h`` of token ``n``; ``tok_seq[n]`` and
    ``tok_pos[n]`` name its sequence and position; ``slots[n]`` its cache slot.
    ``q[b, j, :]`` is query head ``j`` of the decode step of sequence ``b``.
    Float tensors are float32 views of the stored dtype's values; when
    ``dtype == "bf16"`` the ``*_bits`` fields hold the raw uint16 patterns.
    """
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    seq_lens: np.ndarray
    page_table: np.ndarray
    num_pages: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    tok_seq: np.ndarray
    tok_pos: np.ndarray
    slots: np.ndarray
    mu: np.ndarray
    r_k: np.ndarray
    r_v: np.ndarray
    q_bits: Optional[np.ndarray] = None
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None
    outlier_channels: Optional[np.ndarray] = None
    # "dense": r_k, r_v are [H_kv][128][128] orthogonal matrices; "hadamard": they
    # are [H_kv][128] sign vectors (+-1) of a randomized Hadamard rotation
    rotation: str = "dense"

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def n_tokens(self) -> int:
        return int(self.k.shape[0])


def _draw_keys(seed, n_tok, Hkv, outlier_ch, offsets, sub):
    k = rng_for(seed, "k", sub).standard_normal((n_tok, Hkv, HEAD_DIM), dtype=np.float32)
    for h in range(Hkv):
        k[:, h, outlier_ch[h]] *= np.float32(20.0)
    k += offsets[None, :, :]
    return k


def make_case(name: str, seed: int, B: int, Hq: int, Hkv: int, seq_lens, dtype: str = "bf16",
              n_outliers: int = 3, mu_tokens: int = 2048, table_policy: str = "permuted",
              shared_rotation: bool = False, num_pages: Optional[int] = None,
              mu_zero: bool = False, identity_rotation: bool = False, rotation: str = "dense") -> Case:
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape == (B,) and Hq % Hkv == 0
    out_rng = rng_for(seed, "outliers")
    outlier_ch = np.stack([out_rng.choice(HEAD_DIM, size=n_outliers, replace=False) for _ in range(Hkv)])
    offsets = (rng_for(seed, "offsets").standard_normal((Hkv, HEAD_DIM)) * 3.0).astype(np.float32)

    if table_policy == "contiguous":
        table, npages = page_table_contiguous(seq_lens)
        if num_pages is not None:
            npages = max(npages, int(num_pages))
    elif table_policy == "permuted":
        table, npages = page_table_permuted(seq_lens, rng_for(seed, "pages"), num_pages=num_pages)
    elif table_policy == "interleaved":
        table, npages = page_table_interleaved(seq_lens, rng_for(seed, "pages"), num_pages=num_pages)
    else:
        raise ValueError(table_policy)

    ks, vs, seqs, poss = [], [], [], []
    for b in range(B):
        T = int(seq_lens[b])
        kb = _draw_keys(seed, T, Hkv, outlier_ch, offsets, sub=b)
        vb = rng_for(seed, "v", b).standard_normal((T, Hkv, HEAD_DIM), dtype=np.float32)
        ks.append(kb)
        vs.append(vb)
        seqs.append(np.full(T, b, dtype=np.int32))
        poss.append(np.arange(T, dtype=np.int32))
    k = np.concatenate(ks) if ks else np.zeros((0, Hkv, HEAD_DIM), np.float32)
    v = np.concatenate(vs) if vs else np.zeros((0, Hkv, HEAD_DIM), np.float32)
    tok_seq = np.concatenate(seqs)
    tok_pos = np.concatenate(poss)
    q = rng_for(seed, "q").standard_normal((B, Hq, HEAD_DIM), dtype=np.float32)

    q_bits = k_bits = v_bits = None
    if dtype == "bf16":
        q_bits, k_bits, v_bits = bf16_bits(q), bf16_bits(k), bf16_bits(v)
        q, k, v = bf16_to_f32(q_bits), bf16_to_f32(k_bits), bf16_to_f32(v_bits)
    elif dtype != "f32":
        raise ValueError(dtype)

    if rotation == "hadamard":  # seeded +-1 signs per KV head
        r_k = np.stack([rng_for(seed, "r_k", h).choice(np.array([-1.0, 1.0], np.float32), HEAD_DIM)
                        for h in range(Hkv)]).astype(np.float32)
        r_v = r_k.copy() if shared_rotation else np.stack(
            [rng_for(seed, "r_v", h).choice(np.array([-1.0, 1.0], np.float32), HEAD_DIM)
             for h in range(Hkv)]).astype(np.float32)
    elif rotation != "dense":
        raise ValueError(rotation)
    elif identity_rotation:
        r_k = np.broadcast_to(np.eye(HEAD_DIM, dtype=np.float32), (Hkv, HEAD_DIM, HEAD_DIM)).copy()
        r_v = r_k.copy()
    else:
        r_k = np.stack([random_orthogonal(rng_for(seed, "r_k", h)) for h in range(Hkv)])
        r_v = r_k.copy() if shared_rotation else np.stack([random_orthogonal(rng_for(seed, "r_v", h))
                                                           for h in range(Hkv)])
    if mu_zero:
        mu = np.zeros((Hkv, HEAD_DIM), np.float32)
    else:
        n_mu = min(int(mu_tokens), int(seq_lens[0]))
        first = k[tok_seq == 0][:n_mu].astype(np.float64)
        mu = first.mean(axis=0).astype(np.float32) if n_mu > 0 else np.zeros((Hkv, HEAD_DIM), np.float32)

    slots = slots_for_positions(table, tok_seq, tok_pos) if len(tok_seq) else np.zeros(0, np.int32)
    return Case(name=name, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, seq_lens=seq_lens, page_table=table,
                num_pages=int(npages), q=q, k=k, v=v, tok_seq=tok_seq, tok_pos=tok_pos, slots=slots,
                mu=mu, r_k=r_k, r_v=r_v, q_bits=q_bits, k_bits=k_bits, v_bits=v_bits,
                outlier_channels=outlier_ch, rotation=rotation)


# Named workloads.  Sizes follow the tiny case and the Llama-3.1-8B-shaped and
# 70B-class GQA decode shapes used throughout the tests and the benchmark.
def tiny_case(seed: int = 1) -> Case:
    """1 KV head, 4 query heads, d=128, 256 cached tokens, fp32, contiguous pages, one R."""
    return make_case("tiny_t256", seed, B=1, Hq=4, Hkv=1, seq_lens=[256], dtype="f32", n_outliers=4,
                     mu_tokens=256, table_policy="contiguous", shared_rotation=True)


def llama8b_case(T: int, seed: int = 2, B: int = 1, rotation: str = "dense") -> Case:
    """32 query / 8 KV heads, bf16, permuted page table, mu from the first 2048 tokens."""
    return make_case(f"llama8b_b{B}_t{T}", seed, B=B, Hq=32, Hkv=8, seq_lens=[T] * B, dtype="bf16",
                     n_outliers=3, mu_tokens=2048, table_policy="permuted", rotation=rotation)


def batched_lengths(B: int = 16, lo: int = 4096, hi: int = 65536, seed: int = 4) -> np.ndarray:
    return rng_for(seed, "lengths").integers(lo, hi + 1, size=B).astype(np.int32)


def batched_case(seed: int = 4, B: int = 16, lo: int = 4096, hi: int = 65536, rotation: str = "dense") -> Case:
    """8B shape, batch 16, lengths uniform in [4K, 64K], interleaved page allocator."""
    lens = batched_lengths(B, lo, hi, seed)
    return make_case(f"llama8b_batch{B}", seed, B=B, Hq=32, Hkv=8, seq_lens=lens, dtype="bf16",
                     n_outliers=3, mu_tokens=2048, table_policy="interleaved", rotation=rotation)


def seventy_b_case(T: int = 131072, B: int = 4, seed: int = 5, rotation: str = "dense") -> Case:
    """64 query / 8 KV heads (group 8), bf16, interleaved page allocator."""
    return make_case(f"gqa70b_b{B}_t{T}", seed, B=B, Hq=64, Hkv=8, seq_lens=[T] * B, dtype="bf16",
                     n_outliers=3, mu_tokens=2048, table_policy="interleaved", rotation=rotation)


def gqa405b_case(T: int = 131072, B: int = 1, seed: int = 6, rotation: str = "dense") -> Case:
    """128 query / 8 KV heads (group 16, the 405B-class head layout), bf16, interleaved page allocator."""
    return make_case(f"gqa405b_b{B}_t{T}", seed, B=B, Hq=128, Hkv=8, seq_lens=[T] * B, dtype="bf16",
                     n_outliers=3, mu_tokens=2048, table_policy="interleaved", rotation=rotation)


def list_cases() -> List[str]:
    return ["tiny_t256", "llama8b_t32k", "llama8b_t128k", "llama8b_batch16", "gqa70b_b4_t128k"]
