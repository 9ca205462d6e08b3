"""CPU oracle for rotated INT2 KV-cache quantization with key centering.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain reference that the
GPU path is checked against.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import or run it; the product path never
calls it and shares no code with it.

Sources.  "OptR" below is the page *Output-Oriented Rotation for INT2 KV-Cache
Quantization* (arXiv 2608.02691):

* §3, Eq. (1)-(2): GQA attention of query head j over KV head h,
  a_s = <q_j, k_s>/sqrt(d), p = softmax_{s<=t}(a), o_j = sum_s p_s v_s.
* §3.1, Eq. (4): the rotated INT2 quantizer D_R(z) = Q2(zR; c, G) R^T with an
  orthogonal R; with Q2 replaced by the identity, D_R(z) = z.
* §3.2, Eq. (5): attention on the effective (quantized) keys and values.
* §3.2, Eq. (6)-(8): the exact split of the output error into a key-induced and
  a value-induced term, Eq. (9)-(10): E_rec and E_out.
* §1 (and the contributions list): keys are centred before rotation and
  quantization; this shifts every logit of one query by the same constant, so
  the softmax is unchanged.

Readings where the page leaves a step open (each is listed with its reason in
the design notes of the repository):

* Q2 is asymmetric with group size G (32 by default; 64 or 128) consecutive
  rotated channels of one token and clip ratio c (default 1): with mn, mx = c*min, c*max,
  scale s = (mx - mn)/3, zero z = mn, code = clamp(round_half_even((x - z)/s),
  0, 3), level = z + s*code.
  The exact fp32/fp16 operation order is fixed in ``int2_quantize``.
* mu is an input; it is subtracted from keys only and never added back.
* R^T is applied to the query (as qR) and once to the attention output, which
  equals dequantize-then-rotate-back per token because R is orthogonal.
* A sequence of length 0 attends to nothing and its output is zero.
* A page-table entry outside [0, num_pages) marks an absent page: its
  positions are neither written nor attended.
* The BF16 window (optional): the first ``sinks`` and the last ``recent``
  positions of a sequence are attended from their exact BF16 keys and values,
  the rest from INT2; the page leaves its size open (``window_mask``).

Packed page layout.  The pages fix only that rotation keeps a regular paged
layout; the byte layout below is this repository's format, stated here in
full so the oracle can be read without any other file.  One block holds the 16
token slots of one (page p, KV head h) and starts at byte (p*H_kv + h)*B,
B the block size below:

* bytes [0, 1024): 64 records of 16 bytes.  Record r = 16*a + b
  (a in 0..3, b in 0..15) is four little-endian uint32 words at byte 16*r:
  K0, K1, V0, V1.
  - K code of slot s, channel c: kk = c // 32, a = (c % 32) // 8, e = c % 8;
    record 16*a + s, word K[kk // 2], bit 2*(4*(kk % 2) + e // 2) + 16*(e % 2).
  - V code of slot s, channel c: t = c // 16, b = c % 16, a = s // 4,
    i = s % 4; record 16*a + b, word V[i // 2], bit 2*t + 16*(i % 2).
  Each code occupies that bit and the one above it (low bit first).
* bytes [1024, 1024 + M), M = 128 * (128 / G) (512, 256 or 128 bytes for
  G = 32, 64, 128): 128 / G * 4 records of 32 bytes.  Record m = 4*grp + a
  holds, for the four slots s = 4*a + i (i in 0..3) and channel group grp
  (channels G*grp .. G*grp + G - 1): at byte 1024 + 32*m + 4*i the K pair and
  at byte 1024 + 32*m + 16 + 4*i the V pair, each pair being the fp16 scale
  (low two bytes) then the fp16 zero, little-endian.  The base block is
  1024 + M bytes: 96, 80 or 72 bytes per token and KV head.

Keys or values of 3 or 4 bits (key_bits, val_bits: the page's K3V2, K3V3 and
K4V2 budgets) keep the low two bits of each code (code & 3) in the words
above and the rest in a plane appended to the block, the keys' plane first
(at P_K = 1024 + M), then the values' (at P_V = P_K + the keys' plane size):

* 4 bits: a 512-byte plane, 64 records of 8 bytes.  Record r holds words
  H0, H1 (keys) or VH0, VH1 (values) at byte P + 8*r: the high two bits
  (code >> 2) of a code sit in the same record and word index as its low
  bits (record 16*a + s, word H[kk // 2] for the key of slot s, channel c;
  record 16*a + b, word VH[i // 2] for the value), at the same bit.
* 3 bits: a 256-byte plane, 64 records of 4 bytes, one word W per record at
  byte P + 4*r holding the high bit (code >> 2) of every code of the record:
  keys: the code at bit j of word K[w] (j even) has its high bit at bit
  j + w of W (the two K words interleaved); values: the code of slot
  4*a + i, channel 16*t + b (record 16*a + b) has its high bit at bit 8*i + t
  of W (one byte per slot).

So a K2V2 block is 1536 bytes for G = 32, a K3V3 block 2048 (128 bytes per
token) and a K4V2 block 2048.
"""

from __future__ import annotations

import numpy as np

HEAD_DIM = 128
GROUP = 32
N_GROUPS = HEAD_DIM // GROUP
PAGE = 16
CODE_BYTES = 1024


def meta_bytes(group: int = GROUP) -> int:
    """Metadata bytes of a block: 16 slots x (K, V) x 4 bytes per group."""
    assert group in (32, 64, 128), "group size must be 32, 64 or 128"
    return PAGE * 2 * 4 * (HEAD_DIM // group)


def plane_bytes(bits: int) -> int:
    """Bytes of the high-bit plane of 3- or 4-bit codes (none for 2-bit codes)."""
    assert bits in (2, 3, 4), "codes are 2, 3 or 4 bits"
    return {2: 0, 3: 256, 4: 512}[bits]


def key_plane(group: int = GROUP) -> int:
    """Byte offset of the keys' high-bit plane: after codes and metadata."""
    return CODE_BYTES + meta_bytes(group)


def value_plane(key_bits: int = 2, group: int = GROUP) -> int:
    """Byte offset of the values' high-bit plane: after the keys' plane, if any."""
    return key_plane(group) + plane_bytes(key_bits)


def block_bytes(key_bits: int = 2, val_bits: int = 2, group: int = GROUP) -> int:
    """Bytes of one (page, KV head) block: codes, metadata, then the planes."""
    return value_plane(key_bits, group) + plane_bytes(val_bits)


# --------------------------------------------------------------------- checks
def check_orthogonal(r: np.ndarray, tol: float = 1e-6) -> None:
    """OptR §3.1: R must be in O(d).  Asserts max|R^T R - I| <= tol."""
    r64 = np.asarray(r, dtype=np.float64)
    err = np.abs(r64.T @ r64 - np.eye(r64.shape[0])).max()
    assert err <= tol, f"rotation is not orthogonal (max |R^T R - I| = {err:.3g})"


# -------------------------------------------------- structured rotation
def hadamard_rotation(signs: np.ndarray) -> np.ndarray:
    """Randomized Hadamard rotation per KV head, R = diag(s) H / sqrt(d) (fp64).

    The rotation baseline the pages build OptR on (QuaRot) is a randomized
    Hadamard transform; this is its plain matrix: H is Sylvester's Hadamard
    matrix, H[i][j] = (-1)^popcount(i & j), and s a +-1 sign vector, so
    (x R)_j = sum_i x_i s_i (-1)^popcount(i & j) / sqrt(d).  R is orthogonal
    and enters every rotation function here like any other R.
    ``signs`` is [H_kv, d] of +-1; returns [H_kv, d, d].
    """
    s = np.asarray(signs, np.float64)
    assert np.all(np.abs(s) == 1.0), "signs must be +-1"
    d = s.shape[-1]
    idx = np.arange(d)
    parity = np.vectorize(lambda v: bin(int(v)).count("1") & 1)(idx[:, None] & idx[None, :])
    h = np.where(parity == 0, 1.0, -1.0)
    return s[:, :, None] * h[None, :, :] / np.sqrt(d)


# ---------------------------------------------- centering and rotation (fp64)
def centre_keys(k: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """OptR §1: attention-equivalent key reparameterisation, k - mu (fp64).

    ``k`` is [..., H_kv, d]; ``mu`` is [H_kv, d] and broadcasts over tokens.
    """
    return np.asarray(k, np.float64) - np.asarray(mu, np.float64)


def rotate(z: np.ndarray, r: np.ndarray) -> np.ndarray:
    """OptR §3.1, Eq. (4): row vector z maps to zR, per KV head (fp64).

    ``z`` is [n, H_kv, d]; ``r`` is [H_kv, d, d]; out[n, h, j] = sum_i z[n,h,i] R[h,i,j].
    """
    z = np.asarray(z, np.float64)
    r = np.asarray(r, np.float64)
    return np.einsum("nhi,hij->nhj", z, r)


def rotated_inputs(k, v, mu, r_k, r_v):
    """fp32 inputs of the quantizer: x = fp32((k - mu) R_K), w = fp32(v R_V).

    The products are formed in fp64 and rounded once to fp32 (OptR §1 centres
    keys only; §3.1 Eq. (4) rotates both K and V).
    """
    x = rotate(centre_keys(k, mu), r_k).astype(np.float32)
    w = rotate(np.asarray(v, np.float64), r_v).astype(np.float32)
    return x, w


# ---------------------------------------------------------- INT2 quantizer Q2
def int2_quantize(x: np.ndarray, clip: float = 1.0, group: int = GROUP, bits: int = 2):
    """OptR §3.1: Q2(.; c, G), asymmetric, on fp32 rows of 128 channels;
    ``bits`` = 3 or 4 gives the same quantizer with 8 or 16 levels (3- and 4-bit
    keys of K3V2 / K4V2 budgets): the divisor 3 below becomes 2^bits - 1 and
    codes run 0..2^bits - 1.

    ``x`` is float32 [..., 128].  Groups are G = ``group`` (32, 64 or 128)
    consecutive channels.  For each
    group, with every operation in IEEE fp32 (round to nearest even) unless
    stated:

      mn, mx = c * min, c * max of the group   (c = ``clip``, exact when c = 1)
      s32 = (mx - mn) / 3
      s16 = fp16(s32), z16 = fp16(mn)          (round to nearest even)
      s, z = float(s16), float(z16)
      if s == 0: every code is 0
      else code = clamp(round_half_even((x - z) / s), 0, 3)

    The clip ratio c in (0, 1] narrows the range the four levels span (the page
    names Q2(.; c, G) without defining c; reading: both ends of the group's
    range are scaled by c, as the rotation baselines it builds on clip KV
    groups); values past the narrowed range take the end codes.
    Returns (codes uint8 [..., 128], scale float16 [..., 128/G], zero float16 [..., 128/G]).
    Inputs must be finite with group ranges inside the fp16 range.
    """
    x = np.asarray(x)
    assert x.dtype == np.float32 and x.shape[-1] == HEAD_DIM
    assert np.isfinite(x).all(), "quantizer input must be finite"
    c = np.float32(clip)
    assert np.float32(0.0) < c <= np.float32(1.0), "clip ratio must be in (0, 1]"
    assert group in (32, 64, 128), "group size must be 32, 64 or 128"
    assert bits in (2, 3, 4), "2, 3 or 4 bits"
    n_lv = np.float32((1 << bits) - 1)
    xg = x.reshape(x.shape[:-1] + (HEAD_DIM // group, group))
    mn = (xg.min(axis=-1) * c).astype(np.float32)
    mx = (xg.max(axis=-1) * c).astype(np.float32)
    rng = (mx - mn).astype(np.float32)
    s32 = (rng / n_lv).astype(np.float32)
    s16 = s32.astype(np.float16)
    z16 = mn.astype(np.float16)
    assert np.isfinite(s16).all() and np.isfinite(z16).all(), "group range exceeds fp16"
    s = s16.astype(np.float32)[..., None]
    z = z16.astype(np.float32)[..., None]
    t = (xg - z).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(s > 0, t / np.where(s > 0, s, np.float32(1.0)), np.float32(0.0)).astype(np.float32)
    codes = np.clip(np.rint(u), 0, int(n_lv)).astype(np.uint8)
    return codes.reshape(x.shape), s16, z16


def int2_dequantize(codes: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """Level of each code, z + s*code, exact in fp64 (OptR §3.1, four levels per group).
    The group size is 128 / (number of scale entries per row)."""
    n_g = np.asarray(s16).shape[-1]
    c = np.asarray(codes, np.float64).reshape(codes.shape[:-1] + (n_g, HEAD_DIM // n_g))
    lv = np.asarray(z16, np.float64)[..., None] + np.asarray(s16, np.float64)[..., None] * c
    return lv.reshape(codes.shape)


# ------------------------------------------------------------ pack / unpack
def _k_position(slot: int, c: int):
    kk, a, e = c // 32, (c % 32) // 8, c % 8
    rec = 16 * a + slot
    word = kk // 2
    bit = 2 * (4 * (kk % 2) + e // 2) + 16 * (e % 2)
    return rec, word, bit


def _v_position(slot: int, c: int):
    t, b, a, i = c // 16, c % 16, slot // 4, slot % 4
    rec = 16 * a + b
    word = 2 + i // 2
    bit = 2 * t + 16 * (i % 2)
    return rec, word, bit


# Position tables [slot, channel] -> (record, word, bit), built by looping the
# formulas above once.
_K_POS = np.array([[_k_position(s, c) for c in range(HEAD_DIM)] for s in range(PAGE)], dtype=np.int64)
_V_POS = np.array([[_v_position(s, c) for c in range(HEAD_DIM)] for s in range(PAGE)], dtype=np.int64)


def _set_bits(words, idx, bit, val, width):
    """words[idx] <- field of ``width`` bits at ``bit`` replaced by val (all arrays flat)."""
    mask = np.uint32((1 << width) - 1)
    np.bitwise_and.at(words, idx, ~(mask << bit))
    np.bitwise_or.at(words, idx, (val & mask) << bit)


def _plane_position(pos, bits: int, value: bool):
    """Plane (word index, bit) of the codes at code-word positions pos [..., (record, word, bit)]:
    4-bit planes mirror the code words (two words per record, same bit); 3-bit planes hold one
    word per record, keys' high bits at bit + w (w = 0, 1 the K word), values' at 8 * i + t
    (slot 4a + i, channel tile t)."""
    rec, word, bit = pos[..., 0], pos[..., 1] - (2 if value else 0), pos[..., 2]
    if bits == 4:
        return rec * 2 + word, bit
    if not value:
        return rec, bit + word
    i = 2 * word + bit // 16
    return rec, 8 * i + (bit % 16) // 2


def pack_block(k_codes, k_s16, k_z16, v_codes, v_s16, v_z16, block: np.ndarray | None = None,
               slots=None, key_bits: int = 2, val_bits: int = 2, group: int = GROUP) -> np.ndarray:
    """Write token slots of one (page, KV head) block in the layout above.

    ``k_codes``/``v_codes`` are uint8 [n, 128]; scales/zeros float16 [n, 128/G];
    ``slots`` (default 0..n-1, distinct) are the slot indices inside the page.
    Bits of slots not written are left as they were in ``block``.
    """
    nb = block_bytes(key_bits, val_bits, group)
    blk = np.zeros(nb, np.uint8) if block is None else block
    assert blk.shape == (nb,) and blk.dtype == np.uint8
    n = np.asarray(k_codes).shape[0]
    slots = np.arange(n) if slots is None else np.asarray(slots, np.int64)
    assert len(np.unique(slots)) == len(slots)
    words = blk[:CODE_BYTES].view("<u4").reshape(-1)           # 64 records x 4 words
    k_codes = np.asarray(k_codes, np.uint32)
    v_codes = np.asarray(v_codes, np.uint32)
    assert k_codes.max(initial=0) < (1 << key_bits) and v_codes.max(initial=0) < (1 << val_bits)
    for codes, table in ((k_codes, _K_POS), (v_codes, _V_POS)):
        pos = table[slots]                                      # [n, 128, (record, word, bit)]
        _set_bits(words, (pos[..., 0] * 4 + pos[..., 1]).reshape(-1), pos[..., 2].reshape(-1).astype(np.uint32),
                  codes.reshape(-1), 2)
    for bits, codes, table, off, value in ((key_bits, k_codes, _K_POS, key_plane(group), False),
                                           (val_bits, v_codes, _V_POS, value_plane(key_bits, group), True)):
        if bits == 2:
            continue
        plane = blk[off:off + plane_bytes(bits)].view("<u4").reshape(-1)
        idx, bit = _plane_position(table[slots], bits, value)
        _set_bits(plane, idx.reshape(-1), bit.reshape(-1).astype(np.uint32), (codes >> np.uint32(2)).reshape(-1),
                  bits - 2)
    n_g = HEAD_DIM // group
    meta = blk[CODE_BYTES:CODE_BYTES + meta_bytes(group)].view("<u2").reshape(4 * n_g, 2, 4, 2)  # [m][K/V][i][s/z]
    for idx, s in enumerate(slots):
        a, i = int(s) // 4, int(s) % 4
        for grp in range(n_g):
            m = 4 * grp + a
            meta[m, 0, i, 0] = np.asarray(k_s16[idx, grp], np.float16).view(np.uint16)
            meta[m, 0, i, 1] = np.asarray(k_z16[idx, grp], np.float16).view(np.uint16)
            meta[m, 1, i, 0] = np.asarray(v_s16[idx, grp], np.float16).view(np.uint16)
            meta[m, 1, i, 1] = np.asarray(v_z16[idx, grp], np.float16).view(np.uint16)
    return blk


def unpack_blocks(blocks: np.ndarray, key_bits: int = 2, val_bits: int = 2, group: int = GROUP):
    """Inverse of ``pack_block`` for a stack of blocks [n, block_bytes] (all 16 slots each).

    Returns (k_codes, k_s16, k_z16, v_codes, v_s16, v_z16) with codes uint8
    [n, 16, 128] and scales/zeros float16 [n, 16, 128/G].
    """
    blk = np.ascontiguousarray(blocks, np.uint8).reshape(-1, block_bytes(key_bits, val_bits, group))
    words = blk[:, :CODE_BYTES].view("<u4").reshape(-1, 256).astype(np.int64)
    n_g = HEAD_DIM // group
    meta = blk[:, CODE_BYTES:CODE_BYTES + meta_bytes(group)].view("<f2").reshape(-1, 4 * n_g, 2, 4, 2)

    def gather(bits, table, off, value):
        pos = table                                                  # [16, 128, 3]
        low = (words[:, pos[..., 0] * 4 + pos[..., 1]] >> pos[..., 2][None]) & 3
        if bits > 2:
            plane = blk[:, off:off + plane_bytes(bits)].view("<u4").reshape(blk.shape[0], -1).astype(np.int64)
            idx, bit = _plane_position(pos, bits, value)
            low = low + (((plane[:, idx] >> bit[None]) & ((1 << (bits - 2)) - 1)) << 2)
        return low.astype(np.uint8)

    slots = np.arange(PAGE)
    rec = 4 * np.arange(n_g)[None, :] + (slots // 4)[:, None]          # [slot, grp] -> record m
    i = np.broadcast_to((slots % 4)[:, None], rec.shape)
    k = gather(key_bits, _K_POS, key_plane(group), False)
    v = gather(val_bits, _V_POS, value_plane(key_bits, group), True)
    return (k, meta[:, rec, 0, i, 0], meta[:, rec, 0, i, 1],
            v, meta[:, rec, 1, i, 0], meta[:, rec, 1, i, 1])


def unpack_block(block: np.ndarray, key_bits: int = 2, val_bits: int = 2, group: int = GROUP):
    """``unpack_blocks`` for a single block: codes [16, 128], scales/zeros [16, 128/G]."""
    return tuple(x[0] for x in unpack_blocks(np.asarray(block, np.uint8)[None], key_bits, val_bits, group))


def pool_bytes(num_pages: int, num_kv_heads: int, key_bits: int = 2, val_bits: int = 2, group: int = GROUP) -> int:
    return int(num_pages) * int(num_kv_heads) * block_bytes(key_bits, val_bits, group)


def block_view(pool: np.ndarray, page: int, h: int, num_kv_heads: int, key_bits: int = 2, val_bits: int = 2,
               group: int = GROUP) -> np.ndarray:
    nb = block_bytes(key_bits, val_bits, group)
    off = (int(page) * num_kv_heads + int(h)) * nb
    return pool[off:off + nb]


# ------------------------------------------------------------- quantize-append
def quantize_append(pool: np.ndarray, num_kv_heads: int, slots, x: np.ndarray, w: np.ndarray,
                    clip: float = 1.0, group: int = GROUP, key_bits: int = 2, val_bits: int = 2) -> None:
    """Quantize rotated fp32 rows and store them at the given cache slots.

    ``x``/``w`` are float32 [n, H_kv, 128] (already centred and rotated);
    ``slots[n]`` = page*16 + offset, all distinct; ``clip`` and ``group`` are
    Q2's clip ratio c and group size G.  Writes ``pool`` (uint8) in place.
    """
    kc, ks, kz = int2_quantize(x, clip, group, key_bits)
    vc, vs, vz = int2_quantize(w, clip, group, val_bits)
    slots = np.asarray(slots, np.int64)
    assert len(np.unique(slots)) == len(slots), "slots must be distinct"
    pages = slots // PAGE
    for page in np.unique(pages):
        sel = np.nonzero(pages == page)[0]
        offs = slots[sel] % PAGE
        for h in range(num_kv_heads):
            pack_block(kc[sel, h], ks[sel, h], kz[sel, h], vc[sel, h], vs[sel, h], vz[sel, h],
                       block=block_view(pool, page, h, num_kv_heads, key_bits, val_bits, group), slots=offs,
                       key_bits=key_bits, val_bits=val_bits, group=group)


def append_tokens(pool, num_kv_heads, slots, k, v, mu, r_k, r_v, clip: float = 1.0, group: int = GROUP,
                  key_bits: int = 2, val_bits: int = 2) -> None:
    """Full write path: centre keys, rotate K and V, quantize, pack (OptR §1, §3.1 Eq. (4))."""
    check_orthogonal_all(r_k)
    check_orthogonal_all(r_v)
    x, w = rotated_inputs(k, v, mu, r_k, r_v)
    quantize_append(pool, num_kv_heads, slots, x, w, clip, group, key_bits, val_bits)


def check_orthogonal_all(r: np.ndarray, tol: float = 1e-6) -> None:
    for h in range(r.shape[0]):
        check_orthogonal(r[h], tol)


# ----------------------------------------------------------- reading the cache
def gather_sequence(pool, num_kv_heads, table_row, seq_len, h, num_pages=None, key_bits: int = 2, val_bits: int = 2,
                    group: int = GROUP):
    """Dequantized rotated keys x_hat and values w_hat [T', 128] of one sequence and KV head (fp64).

    A table entry outside [0, num_pages) marks an absent page: its positions
    are left out, so T' = T minus the positions on absent pages.  ``num_pages``
    defaults to the pool's size.
    """
    T = int(seq_len)
    if T == 0:
        return np.zeros((0, HEAD_DIM)), np.zeros((0, HEAD_DIM))
    n_pages = (T + PAGE - 1) // PAGE
    nb = block_bytes(key_bits, val_bits, group)
    if num_pages is None:
        num_pages = np.asarray(pool).size // (num_kv_heads * nb)
    pages = np.asarray(table_row[:n_pages], np.int64)
    present = (pages >= 0) & (pages < num_pages)
    offs = (np.where(present, pages, 0) * num_kv_heads + int(h)) * nb
    blocks = np.asarray(pool, np.uint8)[offs[:, None] + np.arange(nb)[None, :]]
    kc, ks, kz, vc, vs, vz = unpack_blocks(blocks, key_bits, val_bits, group)
    keep = np.repeat(present, PAGE)[:T]
    x = int2_dequantize(kc, ks, kz).reshape(-1, HEAD_DIM)[:T][keep]
    w = int2_dequantize(vc, vs, vz).reshape(-1, HEAD_DIM)[:T][keep]
    return x, w


def softmax_attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """OptR §3, Eq. (1)-(2) in fp64: softmax_s(<q, k_s> * scale) weighted sum of v_s.

    ``q`` is [d] or [m, d]; keys/values [T, d].  T = 0 gives a zero output.
    """
    q = np.asarray(q, np.float64)
    keys = np.asarray(keys, np.float64)
    values = np.asarray(values, np.float64)
    if keys.shape[0] == 0:
        return np.zeros(q.shape[:-1] + (values.shape[-1],))
    a = (q @ keys.T) * scale
    a = a - a.max(axis=-1, keepdims=True)
    p = np.exp(a)
    p = p / p.sum(axis=-1, keepdims=True)
    return p @ values


def decode_attention(q, pool, num_kv_heads, page_table, seq_lens, r_k, r_v, sm_scale=None,
                     heads=None, bypass=None, num_pages=None, key_bits: int = 2, val_bits: int = 2,
                     group: int = GROUP) -> np.ndarray:
    """Decode attention read from the packed cache (OptR §3.2 Eq. (5), §3.1 Eq. (4)).

    For query head j of sequence b, with h = j // g:
      q_hat = q_j R_K,h ;  a_s = <q_hat, x_hat_s> * sm_scale for s < T_b
      p = softmax(a) ;     o_rot = sum_s p_s w_hat_s ;  o_j = o_rot R_V,h^T
    x_hat, w_hat are the dequantized rotated cache rows.  Since R is
    orthogonal, <q_hat, x_hat_s> = <q_j, x_hat_s R_K^T>: the key used is
    D_R(k - mu), and the dropped <q_j, mu> shifts every logit of j equally.

    ``q`` is [B, H_q, 128]; returns fp64 [B, H_q, 128] (only ``heads`` = list
    of (b, j) pairs are filled when given; others stay zero).  ``bypass`` =
    (x, w, tok_seq) replaces the packed cache with unquantized rotated rows.
    Pages whose table entry lies outside [0, num_pages) are absent: their
    positions are not attended (a sequence with no present position outputs 0).
    """
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    g = Hq // num_kv_heads
    sm_scale = 1.0 / np.sqrt(d) if sm_scale is None else float(sm_scale)
    out = np.zeros((B, Hq, d))
    todo = [(b, j) for b in range(B) for j in range(Hq)] if heads is None else list(heads)
    cache = {}
    for b, j in todo:
        h = j // g
        if (b, h) not in cache:
            if bypass is None:
                cache[(b, h)] = gather_sequence(pool, num_kv_heads, page_table[b], seq_lens[b], h, num_pages,
                                                key_bits, val_bits, group)
            else:
                x, w, tok_seq = bypass
                sel = np.asarray(tok_seq) == b
                cache[(b, h)] = (np.asarray(x, np.float64)[sel, h][:seq_lens[b]],
                                 np.asarray(w, np.float64)[sel, h][:seq_lens[b]])
        xh, wh = cache[(b, h)]
        q_hat = q[b, j] @ np.asarray(r_k[h], np.float64)
        o_rot = softmax_attention(q_hat, xh, wh, sm_scale)
        out[b, j] = o_rot @ np.asarray(r_v[h], np.float64).T
    return out


# --------------------------------------------------- exact (BF16) window
def window_mask(seq_len: int, sinks: int, recent: int) -> np.ndarray:
    """Positions of a sequence of length T kept exact next to the INT2 history.

    OptR §3.1 (the text after Eq. (4)) stores the long history in INT2 and
    keeps a small BF16 window, and attends the keys and values that remain
    after the rotated INT2 quantization and the BF16 window restore; the page
    does not size the window.  Reading: the first ``sinks`` positions and the
    last ``recent`` positions (s >= T - recent) are exact, the rest INT2.
    """
    pos = np.arange(int(seq_len))
    return (pos < sinks) | (pos >= int(seq_len) - recent)


def window_slot(t: int, sinks: int, recent: int) -> int:
    """Slot of position t in a sequence's window buffer: t for a sink, else
    sinks + t mod recent (a ring over the recent positions)."""
    return int(t) if t < sinks else sinks + int(t) % recent


def effective_kv_window(pool, num_kv_heads, table_row, seq_len, h, mu_h, r_k_h, r_v_h, k_exact, v_exact,
                        sinks, recent, num_pages=None, key_bits: int = 2, val_bits: int = 2, group: int = GROUP):
    """Keys and values attention uses for one sequence and KV head, in the original basis (fp64).

    Window positions (``window_mask``) take k_exact[s], v_exact[s] (the BF16
    window restore); every other position takes the INT2 cache's
    D_R(k - mu) + mu = x_hat R_K^T + mu and D_R(v) = w_hat R_V^T (OptR §3.1
    Eq. (4), with the §1 centering undone).  INT2 positions on absent pages
    (table entry outside [0, num_pages)) are left out; window positions never
    are.  k_exact, v_exact are [>= T, 128].
    """
    T = int(seq_len)
    if T == 0:
        return np.zeros((0, HEAD_DIM)), np.zeros((0, HEAD_DIM))
    win = window_mask(T, sinks, recent)
    n_pages = (T + PAGE - 1) // PAGE
    nb = block_bytes(key_bits, val_bits, group)
    if num_pages is None:
        num_pages = np.asarray(pool).size // (num_kv_heads * nb)
    pages = np.asarray(table_row[:n_pages], np.int64)
    present = (pages >= 0) & (pages < num_pages)
    offs = (np.where(present, pages, 0) * num_kv_heads + int(h)) * nb
    blocks = np.asarray(pool, np.uint8)[offs[:, None] + np.arange(nb)[None, :]]
    kc, ks, kz, vc, vs, vz = unpack_blocks(blocks, key_bits, val_bits, group)
    x_hat = int2_dequantize(kc, ks, kz).reshape(-1, HEAD_DIM)[:T]
    w_hat = int2_dequantize(vc, vs, vz).reshape(-1, HEAD_DIM)[:T]
    k_int2 = x_hat @ np.asarray(r_k_h, np.float64).T + np.asarray(mu_h, np.float64)
    v_int2 = w_hat @ np.asarray(r_v_h, np.float64).T
    k_eff = np.where(win[:, None], np.asarray(k_exact, np.float64)[:T], k_int2)
    v_eff = np.where(win[:, None], np.asarray(v_exact, np.float64)[:T], v_int2)
    keep = win | np.repeat(present, PAGE)[:T]
    return k_eff[keep], v_eff[keep]


def decode_attention_window(q, pool, num_kv_heads, page_table, seq_lens, mu, r_k, r_v, k_seqs, v_seqs,
                            sinks, recent, sm_scale=None, heads=None, num_pages=None, key_bits: int = 2, val_bits: int = 2,
                            group: int = GROUP) -> np.ndarray:
    """OptR §3.2 Eq. (5) with the BF16 window: Eq. (1)-(2) attention of query
    head j of sequence b over ``effective_kv_window`` of KV head h = j // g.

    k_seqs[b], v_seqs[b] are the exact (BF16-valued) keys and values of
    sequence b, [T_b, H_kv, 128], position-ordered; mu is [H_kv, 128] (None =
    0).  Returns fp64 [B, H_q, 128] (only ``heads`` filled when given).
    """
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    g = Hq // num_kv_heads
    sm_scale = 1.0 / np.sqrt(d) if sm_scale is None else float(sm_scale)
    mu = np.zeros((num_kv_heads, d)) if mu is None else np.asarray(mu, np.float64)
    out = np.zeros((B, Hq, d))
    todo = [(b, j) for b in range(B) for j in range(Hq)] if heads is None else list(heads)
    cache = {}
    for b, j in todo:
        h = j // g
        if (b, h) not in cache:
            cache[(b, h)] = effective_kv_window(pool, num_kv_heads, page_table[b], seq_lens[b], h, mu[h], r_k[h],
                                                r_v[h], np.asarray(k_seqs[b])[:, h], np.asarray(v_seqs[b])[:, h],
                                                sinks, recent, num_pages, key_bits, val_bits, group)
        k_eff, v_eff = cache[(b, h)]
        out[b, j] = softmax_attention(q[b, j], k_eff, v_eff, sm_scale)
    return out


# ------------------------------------------------------ split-K form (partials)
def split_partials(q_hat: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float, bounds):
    """Per-split softmax partials (m, l, acc) over token ranges ``bounds`` (fp64).

    m = max logit of the split, l = sum exp(a - m), acc = sum exp(a - m) v.
    An empty split has m = -inf, l = 0, acc = 0.
    """
    parts = []
    for lo, hi in bounds:
        if hi <= lo:
            parts.append((-np.inf, 0.0, np.zeros(values.shape[-1])))
            continue
        a = (keys[lo:hi] @ q_hat) * scale
        m = a.max()
        e = np.exp(a - m)
        parts.append((m, e.sum(), e @ values[lo:hi]))
    return parts


def merge_partials(parts) -> np.ndarray:
    """Log-sum-exp merge of split partials into the normalised output (fp64)."""
    ms = np.array([p[0] for p in parts])
    if len(ms) == 0 or not np.isfinite(ms).any():
        return np.zeros_like(parts[0][2]) if parts else np.zeros(HEAD_DIM)
    m = ms[np.isfinite(ms)].max()
    wts = np.where(np.isfinite(ms), np.exp(np.where(np.isfinite(ms), ms, 0.0) - m), 0.0)
    l_tot = sum(w * p[1] for w, p in zip(wts, parts))
    acc = sum(w * p[2] for w, p in zip(wts, parts))
    return acc / l_tot


# ------------------------------------------------- output-error decomposition
def output_error_terms(q, keys, values, keys_q, values_q, w_o, scale=None):
    """OptR §3.2 Eq. (6)-(10) for one query row (fp64).

    Returns (dy, dy_k, dy_v, e_rec, e_out) with
      dy   = y_tilde - y
      dy_k = (sum_s (p_tilde_s - p_s) v_s) W_O^T      (key-induced)
      dy_v = (sum_s p_tilde_s (v_tilde_s - v_s)) W_O^T  (value-induced)
      e_rec = ||K - K_tilde||_F^2 + ||V - V_tilde||_F^2,  e_out = ||dy||^2.
    """
    q = np.asarray(q, np.float64)
    d = q.shape[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale

    def probs(kk):
        a = (np.asarray(kk, np.float64) @ q) * scale
        a = a - a.max()
        e = np.exp(a)
        return e / e.sum()

    p, pt = probs(keys), probs(keys_q)
    w_o = np.asarray(w_o, np.float64)
    y = (p @ values) @ w_o.T
    yt = (pt @ values_q) @ w_o.T
    dy_k = ((pt - p) @ values) @ w_o.T
    dy_v = (pt @ (np.asarray(values_q, np.float64) - values)) @ w_o.T
    e_rec = float(((keys - keys_q) ** 2).sum() + ((values - values_q) ** 2).sum())
    return yt - y, dy_k, dy_v, e_rec, float(((yt - y) ** 2).sum())


def present_positions(table_row, seq_len: int, num_pages: int) -> np.ndarray:
    """Mask [T] of the positions whose page is present (table entry in [0, num_pages))."""
    T = int(seq_len)
    n_pages = (T + PAGE - 1) // PAGE
    pages = np.asarray(table_row[:n_pages], np.int64)
    return np.repeat((pages >= 0) & (pages < num_pages), PAGE)[:T]


def output_error(q, pool, num_kv_heads, page_table, seq_lens, k_seqs, v_seqs, mu, r_k, r_v, w_o,
                 sm_scale=None, num_pages=None, kv_heads=None, key_bits: int = 2, val_bits: int = 2,
                 group: int = GROUP):
    """OptR §3.2 Eq. (6)-(10) at the decode position of every sequence, from the packed cache (fp64).

    Query head j of sequence b (KV head h = j // g) attends positions 0..T_b-1.
    Exact keys/values are k_seqs[b][:, h], v_seqs[b][:, h]; the effective ones
    (§3.1) are k~ = x_hat R_K^T + mu and v~ = w_hat R_V^T from the pool.
    Positions on absent pages are left out of both, as in decode.  W_O,j is
    columns [j d, (j + 1) d) of ``w_o`` [d_model, H_q d] (a model's output
    projection, row-major).  Per (b, j) this is ``output_error_terms``.
    Returns dy_k, dy_v [B, H_q, d_model], e_out [B, H_q] (Eq. (10)) and
    e_rec [B, H_kv] (Eq. (9), the cache of sequence b and KV head h).
    ``kv_heads`` (default all) limits the work to those KV heads and their query
    heads; the other entries stay zero.
    """
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    g = Hq // num_kv_heads
    sm_scale = 1.0 / np.sqrt(d) if sm_scale is None else float(sm_scale)
    w_o = np.asarray(w_o, np.float64)
    d_model = w_o.shape[0]
    if num_pages is None:
        num_pages = np.asarray(pool).size // (num_kv_heads * block_bytes(key_bits, val_bits, group))
    dy_k = np.zeros((B, Hq, d_model))
    dy_v = np.zeros((B, Hq, d_model))
    e_out = np.zeros((B, Hq))
    e_rec = np.zeros((B, num_kv_heads))
    for b in range(B):
        T = int(seq_lens[b])
        keep = present_positions(page_table[b], T, num_pages)
        for h in (range(num_kv_heads) if kv_heads is None else kv_heads):
            x_hat, w_hat = gather_sequence(pool, num_kv_heads, page_table[b], T, h, num_pages, key_bits,
                                           val_bits, group)
            k_eff = x_hat @ np.asarray(r_k[h], np.float64).T + np.asarray(mu[h], np.float64)
            v_eff = w_hat @ np.asarray(r_v[h], np.float64).T
            k_ex = np.asarray(k_seqs[b], np.float64)[:T, h][keep]
            v_ex = np.asarray(v_seqs[b], np.float64)[:T, h][keep]
            if k_ex.shape[0] == 0:
                continue
            for j in range(h * g, (h + 1) * g):
                w_oj = w_o[:, j * d:(j + 1) * d]
                _, dk, dv, er, eo = output_error_terms(q[b, j], k_ex, v_ex, k_eff, v_eff, w_oj, sm_scale)
                dy_k[b, j], dy_v[b, j], e_out[b, j] = dk, dv, eo
                e_rec[b, h] = er
    return dy_k, dy_v, e_out, e_rec
