"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  None re-types the oracle's own formula: each
checks a hand-derived worked example, a closed form, an invariant or a brute
force search.
"""

import os

import numpy as np
import pytest

import kvq_inputs as I
from oracle import kvq_oracle as O


# ------------------------------------------------------------------ helpers
def _parse_runs(tokens, dtype):
    out = []
    for t in tokens:
        if "*" in t:
            val, cnt = t.split("*")
            out += [dtype(val)] * int(cnt)
        else:
            out.append(dtype(t))
    return out


def _load_groups(golden_dir):
    cases = {}
    with open(os.path.join(golden_dir, "int2_groups.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, field, *rest = line.split()
            c = cases.setdefault(name, {})
            if field == "values":
                c[field] = np.array(_parse_runs(rest, float), dtype=np.float32)
            elif field == "codes":
                c[field] = np.array(_parse_runs(rest, int), dtype=np.uint8)
            else:
                c[field] = float(rest[0])
    return cases


def _random_rows(rng, n, scale=1.0, offset=0.0):
    return (rng.standard_normal((n, 128)) * scale + offset).astype(np.float32)


# ---------------------------------------------------- Q2: worked examples
def test_quantizer_golden_groups(golden_dir):
    """OptR §3.1 Q2: hand-derived groups (ties to even, fp16 scale use, constant group)."""
    cases = _load_groups(golden_dir)
    assert set(cases) == {"A", "B", "C", "D"}
    for name, c in cases.items():
        assert c["values"].shape == (32,) and c["codes"].shape == (32,)
        row = np.tile(c["values"], 4)[None, :]          # same group in all 4 positions
        codes, s16, z16 = O.int2_quantize(row)
        for grp in range(4):
            assert float(s16[0, grp]) == c["scale"], (name, grp)
            assert float(z16[0, grp]) == c["zero"], (name, grp)
            np.testing.assert_array_equal(codes[0, 32 * grp:32 * grp + 32], c["codes"], err_msg=name)


def test_quantizer_golden_groups_independent_positions(golden_dir):
    """Each of the 4 groups of a row is quantized on its own (no cross-group leakage)."""
    cases = _load_groups(golden_dir)
    order = ["A", "B", "C", "D"]
    row = np.concatenate([cases[n]["values"] for n in order])[None, :]
    codes, s16, z16 = O.int2_quantize(row)
    for grp, n in enumerate(order):
        np.testing.assert_array_equal(codes[0, 32 * grp:32 * grp + 32], cases[n]["codes"])
        assert float(s16[0, grp]) == cases[n]["scale"]
        assert float(z16[0, grp]) == cases[n]["zero"]


# ---------------------------------------------------- Q2: properties
def test_quantizer_at_most_four_levels_and_nearest():
    """OptR §1: only four INT2 levels per group; each code picks the nearest level.

    Brute force over the four candidate levels in fp64.  Ties and fp32 rounding
    of u allow a slack of a few fp32 ulps of the group's scale.
    """
    rng = np.random.default_rng(11)
    x = np.concatenate([_random_rows(rng, 200), _random_rows(rng, 50, 20.0, 3.0),
                        _random_rows(rng, 50, 1e-3, -2.0)])
    codes, s16, z16 = O.int2_quantize(x)
    lv = O.int2_dequantize(codes, s16, z16)
    for n in range(x.shape[0]):
        for grp in range(4):
            sl = slice(32 * grp, 32 * grp + 32)
            assert len(np.unique(lv[n, sl])) <= 4
            s, z = float(s16[n, grp]), float(z16[n, grp])
            cand = z + s * np.arange(4.0)
            dist = np.abs(x[n, sl].astype(np.float64)[:, None] - cand[None, :])
            chosen = dist[np.arange(32), codes[n, sl]]
            assert np.all(chosen <= dist.min(axis=1) + 4 * np.spacing(np.float32(max(s, 1e-30))) + 1e-12)


def test_quantizer_extremes_and_error_bound():
    """Min element gets code 0, max gets 3; |x - level| <= s/2 (+ fp16 rounding of z and s)."""
    rng = np.random.default_rng(12)
    x = _random_rows(rng, 300, 4.0, 1.0)
    codes, s16, z16 = O.int2_quantize(x)
    xg = x.reshape(-1, 4, 32)
    cg = codes.reshape(-1, 4, 32)
    rows = np.arange(xg.shape[0])[:, None]
    grps = np.arange(4)[None, :]
    assert np.all(cg[rows, grps, xg.argmin(-1)] == 0)
    assert np.all(cg[rows, grps, xg.argmax(-1)] == 3)
    lv = O.int2_dequantize(codes, s16, z16).reshape(-1, 4, 32)
    s = s16.astype(np.float64)
    rng_true = (xg.max(-1) - xg.min(-1)).astype(np.float64)
    # stored scale/zero differ from the exact ones by at most half an fp16 ulp (relative 2^-11)
    slack = 2.0 ** -10 * (np.abs(z16.astype(np.float64)) + rng_true)
    assert np.all(np.abs(xg - lv).max(-1) <= s / 2 + slack + 1e-7)


def test_quantizer_arithmetic_progression_is_exact():
    """A group already on an fp16-exact grid z + s*{0,1,2,3} reconstructs with zero error."""
    rng = np.random.default_rng(13)
    for _ in range(50):
        z = float(np.float16(rng.uniform(-8, 8)))
        s = float(2.0 ** rng.integers(-6, 3))
        lvls = z + s * rng.integers(0, 4, size=(4, 32)).astype(np.float64)
        lvls[:, 0], lvls[:, 1] = z, z + 3 * s                   # make min and max present
        x = lvls.reshape(1, 128).astype(np.float32)
        codes, s16, z16 = O.int2_quantize(x)
        np.testing.assert_array_equal(O.int2_dequantize(codes, s16, z16), x.astype(np.float64))


def test_quantizer_constant_and_degenerate_groups():
    x = np.full((3, 128), 0.0, np.float32)
    x[1] = -3.5
    x[2, :32] = 1e-9                                           # range underflows fp16 scale
    x[2, 1] = 2e-9
    codes, s16, z16 = O.int2_quantize(x)
    assert not codes.any()
    assert float(z16[1, 0]) == -3.5
    assert float(s16[2, 0]) == 0.0


# ---------------------------------------------------- pack / unpack
def test_block_layout_golden(golden_dir):
    """Hand-derived byte positions of single codes and metadata in a block."""
    with open(os.path.join(golden_dir, "block_layout.txt")) as f:
        lines = [l.split() for l in f if l.strip() and not l.startswith("#")]
    z = np.zeros((1, 128), np.uint8)
    zf = np.zeros((1, 4), np.float16)
    n_checked = 0
    for parts in lines:
        if parts[0] in ("K", "V"):
            tensor, slot, ch, code, byte, val = parts[0], *map(int, parts[1:])
            kc, vc = z.copy(), z.copy()
            (kc if tensor == "K" else vc)[0, ch] = code
            blk = O.pack_block(kc, zf, zf, vc, zf, zf, slots=[slot])
            nz = np.nonzero(blk)[0]
            assert list(nz) == [byte] and blk[byte] == val, parts
            n_checked += 1
        elif parts[0] == "META":
            tensor, slot, grp, byte = parts[1], int(parts[2]), int(parts[3]), int(parts[4])
            sc = np.zeros((1, 4), np.float16)
            zc = np.zeros((1, 4), np.float16)
            sc[0, grp], zc[0, grp] = 1.5, -2.0                 # 0x3E00, 0xC000
            args = (z, sc, zc, z, zf, zf) if tensor == "K" else (z, zf, zf, z, sc, zc)
            blk = O.pack_block(*args, slots=[slot])
            assert list(np.nonzero(blk)[0]) == [byte + 1, byte + 3], parts
            assert blk[byte + 1] == 0x3E and blk[byte + 3] == 0xC0
            n_checked += 1
    assert n_checked == 10


LAYOUTS = [(2, 2, 32), (2, 2, 64), (2, 2, 128), (3, 3, 32), (4, 2, 64), (3, 4, 128), (2, 3, 64)]


@pytest.mark.parametrize("kb,vb,g", LAYOUTS)
def test_pack_unpack_roundtrip_and_partial_writes(kb, vb, g):
    """Every layout round-trips, and slot-by-slot writes in any order onto a dirty
    block give the bytes of one whole-block write (no slot's bits touch another's)."""
    rng = np.random.default_rng(14 + kb + 3 * vb + g)
    kc = rng.integers(0, 1 << kb, (16, 128)).astype(np.uint8)
    vc = rng.integers(0, 1 << vb, (16, 128)).astype(np.uint8)
    f = lambda: rng.standard_normal((16, 128 // g)).astype(np.float16)
    ks, kz, vs, vz = f(), f(), f(), f()
    full = O.pack_block(kc, ks, kz, vc, vs, vz, key_bits=kb, val_bits=vb, group=g)
    assert full.size == O.block_bytes(kb, vb, g)
    got = O.unpack_block(full, kb, vb, g)
    for a, b in zip(got, (kc, ks, kz, vc, vs, vz)):
        np.testing.assert_array_equal(a.view(np.uint8) if a.dtype == np.float16 else a,
                                      b.view(np.uint8) if b.dtype == np.float16 else b)
    # slot-by-slot writes in a scrambled order onto a dirty block give the same bytes
    blk = rng.integers(0, 256, O.block_bytes(kb, vb, g)).astype(np.uint8)
    for s in rng.permutation(16):
        O.pack_block(kc[s:s + 1], ks[s:s + 1], kz[s:s + 1], vc[s:s + 1], vs[s:s + 1], vz[s:s + 1],
                     block=blk, slots=[s], key_bits=kb, val_bits=vb, group=g)
    np.testing.assert_array_equal(blk, full)


def test_storage_arithmetic():
    """OptR §1: INT2 codes take 1/8 of BF16 storage; with fp16 scale+zero per group
    the block is 96, 80 or 72 bytes per token per KV head for G = 32, 64, 128 (3,
    2.5 and 2.25 bits per element); 3-bit codes add one bit per element, 4-bit two."""
    assert O.CODE_BYTES // 16 // 2 == 128 * 2 // 8            # K (or V) codes per token = bf16 bytes / 8
    for g, per_token in ((32, 96), (64, 80), (128, 72)):
        assert O.block_bytes(group=g) // 16 == per_token
        assert O.block_bytes(group=g) * 8 / (16 * 2 * 128) == 2 + 32 / g
    assert O.block_bytes(3, 3) // 16 == 128                   # K3V3: 4 bits per element
    assert O.block_bytes(3, 2) * 8 / (16 * 2 * 128) == 3.5
    assert O.block_bytes(4, 4) // 16 == 160


def test_compact_layout_golden(golden_dir):
    """Hand-derived block sizes, metadata positions for G = 64 and 128, and 3-bit
    key planes (tests/golden/block_layout_compact.txt)."""
    with open(os.path.join(golden_dir, "block_layout_compact.txt")) as f:
        lines = [l.split() for l in f if l.strip() and not l.startswith("#")]
    n_seen = {"BLOCK": 0, "META": 0, "KEY3": 0}
    for parts in lines:
        kind, nums = parts[0], list(map(int, parts[1:]))
        n_seen[kind] += 1
        if kind == "BLOCK":
            kb, vb, g, size = nums
            assert O.block_bytes(kb, vb, g) == size
            continue
        if kind == "META":
            g, slot, grp, tensor, sbits, zbits, *pairs = nums
            kb = 2
            z = np.zeros((1, 128), np.uint8)
            m0 = np.zeros((1, 128 // g), np.float16)
            pair = [m0.copy() for _ in range(4)]
            pair[2 * tensor][0, grp] = np.uint16(sbits).view(np.float16)
            pair[2 * tensor + 1][0, grp] = np.uint16(zbits).view(np.float16)
            blk = O.pack_block(z, pair[0], pair[1], z, pair[2], pair[3], slots=[slot], group=g)
        else:
            kb, g, slot, ch, code, *pairs = nums
            kc = np.zeros((1, 128), np.uint8)
            kc[0, ch] = code
            z = np.zeros((1, 128), np.uint8)
            m0 = np.zeros((1, 128 // g), np.float16)
            blk = O.pack_block(kc, m0, m0, z, m0, m0, slots=[slot], key_bits=kb, group=g)
        want = dict(zip(pairs[0::2], pairs[1::2]))
        nz = np.nonzero(blk)[0]
        assert set(nz) == set(want) and all(blk[b] == v for b, v in want.items()), parts
        back = O.unpack_block(blk, kb, 2, g)
        if kind == "KEY3":
            assert back[0][slot, ch] == code and np.count_nonzero(back[0]) == 1
    assert n_seen == {"BLOCK": 6, "META": 3, "KEY3": 3}


# ---------------------------------------------------- attention pins
def _brute_attention(q, keys, values, scale):
    """Eq. (1)-(2) with explicit loops."""
    T = len(keys)
    a = [sum(float(q[c]) * float(keys[s][c]) for c in range(len(q))) * scale for s in range(T)]
    m = max(a)
    e = [np.exp(x - m) for x in a]
    tot = sum(e)
    return np.array([sum(e[s] / tot * float(values[s][c]) for s in range(T)) for c in range(values.shape[1])])


def test_softmax_attention_matches_brute_force():
    rng = np.random.default_rng(15)
    for T in (1, 2, 7, 33):
        q = rng.standard_normal(16)
        k = rng.standard_normal((T, 16)) * 3
        v = rng.standard_normal((T, 16))
        np.testing.assert_allclose(O.softmax_attention(q, k, v, 0.25), _brute_attention(q, k, v, 0.25),
                                   rtol=0, atol=1e-13)


def test_split_merge_equals_one_pass():
    rng = np.random.default_rng(16)
    T = 37
    q = rng.standard_normal(128)
    k = rng.standard_normal((T, 128)) * 2
    v = rng.standard_normal((T, 128))
    ref = O.softmax_attention(q, k, v, 1 / np.sqrt(128))
    for n_split in range(1, T + 1):
        edges = np.linspace(0, T, n_split + 1).round().astype(int)
        parts = O.split_partials(q, k, v, 1 / np.sqrt(128), list(zip(edges[:-1], edges[1:])))
        np.testing.assert_allclose(O.merge_partials(parts), ref, rtol=0, atol=1e-13)
    # empty splits are neutral
    parts = O.split_partials(q, k, v, 1 / np.sqrt(128), [(0, 0), (0, T), (T, T)])
    np.testing.assert_allclose(O.merge_partials(parts), ref, rtol=0, atol=1e-13)


def test_key_centering_shift_invariance_fp64():
    """OptR §1: centering shifts every logit of a query by one constant; softmax unchanged."""
    rng = np.random.default_rng(17)
    for _ in range(20):
        q = rng.standard_normal(128)
        k = rng.standard_normal((64, 128)) + rng.standard_normal(128) * 3
        mu = k.mean(axis=0)
        a = k @ q / np.sqrt(128)
        ac = (k - mu) @ q / np.sqrt(128)
        shift = ac - a
        assert np.ptp(shift) <= 1e-12 * max(1.0, np.abs(a).max())
        pa = np.exp(a - a.max()); pa /= pa.sum()
        pc = np.exp(ac - ac.max()); pc /= pc.sum()
        assert np.abs(pa - pc).max() <= 1e-14


def _tiny(seed=1, **kw):
    return I.make_case("t", seed, B=kw.pop("B", 1), Hq=kw.pop("Hq", 4), Hkv=kw.pop("Hkv", 1),
                       seq_lens=kw.pop("seq_lens", [64]), dtype=kw.pop("dtype", "f32"), n_outliers=4,
                       mu_tokens=kw.pop("mu_tokens", 64), table_policy=kw.pop("table_policy", "contiguous"),
                       **kw)


def _fp64_orthogonal(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        qm, rm = np.linalg.qr(rng.standard_normal((128, 128)))
        out.append(qm * np.sign(np.diag(rm))[None, :])
    return np.stack(out)


def test_bypass_equals_plain_attention_any_rotation_and_mu():
    """OptR §3.1 Eq. (4): with Q2 = identity, D_R(z) = z for orthogonal R, so the rotated,
    centred path (q R_K against (k - mu) R_K, output mapped back by R_V^T) equals plain
    Eq. (1)-(2) attention on the raw k, v.  The rotations are fp64-orthogonal so the
    identity holds to fp64 rounding."""
    c = _tiny(B=2, Hq=8, Hkv=2, seq_lens=[40, 23])
    c.r_k, c.r_v = _fp64_orthogonal(101, 2), _fp64_orthogonal(102, 2)
    x = O.rotate(O.centre_keys(c.k, c.mu), c.r_k)
    w = O.rotate(c.v, c.r_v)
    got = O.decode_attention(c.q, None, c.Hkv, c.page_table, c.seq_lens, c.r_k, c.r_v,
                             bypass=(x, w, c.tok_seq))
    for b in range(c.B):
        kb = c.k[c.tok_seq == b].astype(np.float64)
        vb = c.v[c.tok_seq == b].astype(np.float64)
        for j in range(c.Hq):
            ref = O.softmax_attention(c.q[b, j].astype(np.float64), kb[:, j // 4], vb[:, j // 4], 1 / np.sqrt(128))
            np.testing.assert_allclose(got[b, j], ref, rtol=0, atol=1e-12)
    # the rotations must be non-trivial for the test to mean anything
    assert np.abs(c.r_k[0] - c.r_k[0].T).max() > 0.1 and np.abs(c.r_k[0] - np.eye(128)).max() > 0.1


def test_orthogonal_rotation_preserves_norms_and_products():
    c = _tiny()
    O.check_orthogonal(c.r_k[0])
    z = c.k[:, 0].astype(np.float64)
    zr = O.rotate(c.k, c.r_k)[:, 0]
    np.testing.assert_allclose(np.linalg.norm(zr, axis=1), np.linalg.norm(z, axis=1), rtol=1e-6)
    with pytest.raises(AssertionError):
        O.check_orthogonal(c.r_k[0] * 1.001)


def test_identity_rotation_zero_mu_equals_direct_int2():
    """R = I and mu = 0: the quantized cache equals INT2 applied directly to raw k and v (bit-exact)."""
    c = _tiny(identity_rotation=True, mu_zero=True)
    pool = np.zeros(O.pool_bytes(c.num_pages, c.Hkv), np.uint8)
    O.append_tokens(pool, c.Hkv, c.slots, c.k, c.v, c.mu, c.r_k, c.r_v)
    dk = O.int2_quantize(c.k.astype(np.float32))
    dv = O.int2_quantize(c.v.astype(np.float32))
    for n in range(c.n_tokens):
        page, off = divmod(int(c.slots[n]), 16)
        kc, ks, kz, vc, vs, vz = O.unpack_block(O.block_view(pool, page, 0, 1))
        np.testing.assert_array_equal(kc[off], dk[0][n, 0])
        np.testing.assert_array_equal(vc[off], dv[0][n, 0])
        np.testing.assert_array_equal(ks[off], dk[1][n, 0])
        np.testing.assert_array_equal(vz[off], dv[2][n, 0])


def test_decode_from_pool_equals_attention_on_effective_kv():
    """OptR §3.2 Eq. (5): decode over the packed cache equals Eq. (1)-(2) attention on the
    effective keys k~ = Q2((k - mu) R_K) R_K^T + mu and values v~ = Q2(v R_V) R_V^T."""
    c = _tiny(B=2, Hq=8, Hkv=2, seq_lens=[50, 33], table_policy="permuted")
    pool = np.zeros(O.pool_bytes(c.num_pages, c.Hkv), np.uint8)
    O.append_tokens(pool, c.Hkv, c.slots, c.k, c.v, c.mu, c.r_k, c.r_v)
    got = O.decode_attention(c.q, pool, c.Hkv, c.page_table, c.seq_lens, c.r_k, c.r_v)
    x, w = O.rotated_inputs(c.k, c.v, c.mu, c.r_k, c.r_v)
    kq = O.int2_dequantize(*O.int2_quantize(x))
    vq = O.int2_dequantize(*O.int2_quantize(w))
    for b in range(c.B):
        sel = c.tok_seq == b
        for j in range(c.Hq):
            h = j // 4
            k_eff = kq[sel, h] @ c.r_k[h].astype(np.float64).T + c.mu[h]
            v_eff = vq[sel, h] @ c.r_v[h].astype(np.float64).T
            ref = O.softmax_attention(c.q[b, j], k_eff, v_eff, 1 / np.sqrt(128))
            np.testing.assert_allclose(got[b, j], ref, rtol=0, atol=1e-11)


def test_page_permutation_and_batch_independence():
    """The result depends only on the tokens of each sequence, not on where pages live."""
    base = dict(B=2, Hq=4, Hkv=1, seq_lens=[45, 70])
    a = _tiny(table_policy="contiguous", **base)
    b = _tiny(table_policy="interleaved", **base)
    assert not np.array_equal(a.page_table, b.page_table)
    outs = []
    for c in (a, b):
        pool = np.zeros(O.pool_bytes(c.num_pages, c.Hkv), np.uint8)
        O.append_tokens(pool, c.Hkv, c.slots, c.k, c.v, c.mu, c.r_k, c.r_v)
        outs.append(O.decode_attention(c.q, pool, c.Hkv, c.page_table, c.seq_lens, c.r_k, c.r_v))
    np.testing.assert_array_equal(outs[0], outs[1])
    # sequence 1 alone, in a pool of its own, gives the same output
    c = a
    sel = c.tok_seq == 1
    table, npg = I.page_table_contiguous(np.array([70]))
    pool = np.zeros(O.pool_bytes(npg, 1), np.uint8)
    O.append_tokens(pool, 1, I.slots_for_positions(table, np.zeros(70, int), np.arange(70)),
                    c.k[sel], c.v[sel], c.mu, c.r_k, c.r_v)
    alone = O.decode_attention(c.q[1:2], pool, 1, table, np.array([70]), c.r_k, c.r_v)
    np.testing.assert_array_equal(alone[0], outs[0][1])


def test_gqa_group_of_one_is_mha():
    """g = 1: every query head reads its own KV head (OptR §3, G_h = {h})."""
    c = _tiny(Hq=2, Hkv=2)
    c.r_k, c.r_v = _fp64_orthogonal(103, 2), _fp64_orthogonal(104, 2)
    x = O.rotate(O.centre_keys(c.k, c.mu), c.r_k)
    w = O.rotate(c.v, c.r_v)
    got = O.decode_attention(c.q, None, 2, c.page_table, c.seq_lens, c.r_k, c.r_v, bypass=(x, w, c.tok_seq))
    for j in range(2):
        ref = O.softmax_attention(c.q[0, j], c.k[:, j], c.v[:, j], 1 / np.sqrt(128))
        np.testing.assert_allclose(got[0, j], ref, rtol=0, atol=1e-12)


def test_empty_sequence_gives_zero():
    c = _tiny(B=2, seq_lens=[0, 20])
    pool = np.zeros(O.pool_bytes(c.num_pages, 1), np.uint8)
    O.append_tokens(pool, 1, c.slots, c.k, c.v, c.mu, c.r_k, c.r_v)
    out = O.decode_attention(c.q, pool, 1, c.page_table, c.seq_lens, c.r_k, c.r_v)
    assert not out[0].any() and np.abs(out[1]).max() > 0


def test_absent_page_is_left_out():
    """A page-table entry outside the pool marks an absent page: decode equals decode of the
    same sequence with that page's tokens removed, laid out on fresh pages (brute-force layout)."""
    c = _tiny(seq_lens=[64])  # 4 pages, contiguous 0..3
    pool = np.zeros(O.pool_bytes(c.num_pages, 1), np.uint8)
    O.append_tokens(pool, 1, c.slots, c.k, c.v, c.mu, c.r_k, c.r_v)
    for bad in (c.num_pages, -1, 1 << 20):
        table = c.page_table.copy()
        table[0, 1] = bad  # positions 16..31 absent
        got = O.decode_attention(c.q, pool, 1, table, c.seq_lens, c.r_k, c.r_v, num_pages=c.num_pages)
        keep = np.r_[0:16, 32:64]
        pool2 = np.zeros(O.pool_bytes(3, 1), np.uint8)
        O.append_tokens(pool2, 1, np.arange(48), c.k[keep], c.v[keep], c.mu, c.r_k, c.r_v)
        ref = O.decode_attention(c.q, pool2, 1, np.array([[0, 1, 2]]), np.array([48]), c.r_k, c.r_v)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    table = np.full_like(c.page_table, -1)  # every page absent: nothing attended
    assert not O.decode_attention(c.q, pool, 1, table, c.seq_lens, c.r_k, c.r_v).any()


def test_output_error_decomposition_eq8():
    """OptR §3.2 Eq. (8): dy = dy_K + dy_V exactly (random W_O), Eq. (10) E_out = ||dy||^2."""
    rng = np.random.default_rng(18)
    T, d = 40, 128
    q = rng.standard_normal(d)
    k = rng.standard_normal((T, d)) * 2
    v = rng.standard_normal((T, d))
    kq = k + rng.standard_normal((T, d)) * 0.3
    vq = v + rng.standard_normal((T, d)) * 0.3
    w_o = rng.standard_normal((64, d))
    dy, dyk, dyv, e_rec, e_out = O.output_error_terms(q, k, v, kq, vq, w_o)
    np.testing.assert_allclose(dy, dyk + dyv, rtol=0, atol=1e-12)
    assert abs(e_out - float(dy @ dy)) <= 1e-9 * max(1.0, e_out)
    assert abs(e_rec - (np.linalg.norm(k - kq) ** 2 + np.linalg.norm(v - vq) ** 2)) <= 1e-9 * e_rec
    # no key error -> no key-induced term; no value error -> no value-induced term
    _, dyk0, _, _, _ = O.output_error_terms(q, k, v, k, vq, w_o)
    _, _, dyv0, _, _ = O.output_error_terms(q, k, v, kq, v, w_o)
    assert np.abs(dyk0).max() == 0 and np.abs(dyv0).max() == 0


def test_centering_reduces_int2_key_error_with_offsets():
    """OptR §1: with large per-channel key offsets, centering before rotation shrinks the
    INT2 key reconstruction error (a direction check on synthetic data)."""
    c = I.tiny_case()
    errs = []
    for mu in (np.zeros_like(c.mu), c.mu):
        x = O.rotate(O.centre_keys(c.k, mu), c.r_k).astype(np.float32)
        xq = O.int2_dequantize(*O.int2_quantize(x))
        errs.append(np.linalg.norm(x - xq))
    assert errs[1] < errs[0]


# ------------------------------------------------------- exact (BF16) window
def _seqs(c, a):
    """Per-sequence, position-ordered copies [T_b, H_kv, 128] of a token array."""
    out = []
    for b in range(c.B):
        sel = np.nonzero(c.tok_seq == b)[0]
        out.append(np.asarray(a)[sel[np.argsort(c.tok_pos[sel])]])
    return out


def _window_case(**kw):
    c = _tiny(B=2, Hq=8, Hkv=2, seq_lens=kw.pop("seq_lens", [50, 33]), table_policy="permuted", dtype="bf16", **kw)
    pool = np.zeros(O.pool_bytes(c.num_pages, c.Hkv), np.uint8)
    O.append_tokens(pool, c.Hkv, c.slots, c.k, c.v, c.mu, c.r_k, c.r_v)
    return c, pool


def test_window_covering_every_position_is_plain_attention():
    """sinks + recent >= T: every key and value is restored exactly, so the output is
    Eq. (1)-(2) attention on the raw (bf16) k and v, whatever the INT2 cache holds."""
    c, pool = _window_case()
    ks, vs = _seqs(c, c.k), _seqs(c, c.v)
    for sinks, recent in ((0, 50), (4, 46), (50, 0), (8, 128)):
        got = O.decode_attention_window(c.q, pool, c.Hkv, c.page_table, c.seq_lens, c.mu, c.r_k, c.r_v, ks, vs,
                                        sinks, recent)
        for b in range(c.B):
            for j in range(c.Hq):
                ref = _brute_attention(c.q[b, j], ks[b][:, j // 4], vs[b][:, j // 4], 1 / np.sqrt(128))
                np.testing.assert_allclose(got[b, j], ref, rtol=0, atol=1e-12)


def test_empty_window_equals_int2_decode():
    """sinks = recent = 0: the original-basis effective-KV form equals the rotated-basis
    decode (q R_K against x_hat, mu dropped, output mapped back by R_V^T)."""
    c, pool = _window_case()
    got = O.decode_attention_window(c.q, pool, c.Hkv, c.page_table, c.seq_lens, c.mu, c.r_k, c.r_v,
                                    _seqs(c, c.k), _seqs(c, c.v), 0, 0)
    ref = O.decode_attention(c.q, pool, c.Hkv, c.page_table, c.seq_lens, c.r_k, c.r_v)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)


def test_window_positions_brute_force():
    """Which positions are exact, built independently with list slicing, then explicit
    per-position effective keys/values and looped attention."""
    c, pool = _window_case(seq_lens=[40, 9])
    ks, vs = _seqs(c, c.k), _seqs(c, c.v)
    x, w = O.rotated_inputs(c.k, c.v, c.mu, c.r_k, c.r_v)
    kq = _seqs(c, O.int2_dequantize(*O.int2_quantize(x)))
    vq = _seqs(c, O.int2_dequantize(*O.int2_quantize(w)))
    for sinks, recent in ((3, 7), (0, 1), (5, 0), (6, 6), (12, 30)):
        got = O.decode_attention_window(c.q, pool, c.Hkv, c.page_table, c.seq_lens, c.mu, c.r_k, c.r_v, ks, vs,
                                        sinks, recent)
        for b in range(c.B):
            T = int(c.seq_lens[b])
            positions = list(range(T))
            exact = set(positions[:sinks]) | (set(positions[-recent:]) if recent else set())
            for j in (0, 5):
                h = j // 4
                keys, vals = [], []
                for s in positions:
                    if s in exact:
                        keys.append(ks[b][s, h])
                        vals.append(vs[b][s, h])
                    else:
                        keys.append(kq[b][s, h] @ c.r_k[h].astype(np.float64).T + c.mu[h])
                        vals.append(vq[b][s, h] @ c.r_v[h].astype(np.float64).T)
                ref = _brute_attention(c.q[b, j], np.array(keys), np.array(vals), 1 / np.sqrt(128))
                np.testing.assert_allclose(got[b, j], ref, rtol=0, atol=1e-11)
    # one more exact position changes the output (the boundary is not off by one)
    a = O.decode_attention_window(c.q, pool, c.Hkv, c.page_table, c.seq_lens, c.mu, c.r_k, c.r_v, ks, vs, 0, 7)
    b_ = O.decode_attention_window(c.q, pool, c.Hkv, c.page_table, c.seq_lens, c.mu, c.r_k, c.r_v, ks, vs, 0, 8)
    assert np.abs(a[0] - b_[0]).max() > 1e-6


def test_window_slots_golden(golden_dir):
    """window_slot and window_mask against hand-derived slots and positions
    (tests/golden/window_slots.txt).  A ring over the recent positions started at
    the first recent position (sinks + (t - sinks) mod recent) would differ."""
    n_slot = n_mask = 0
    with open(os.path.join(golden_dir, "window_slots.txt")) as f:
        for line in f:
            f_ = line.split()
            if not f_ or f_[0].startswith("#"):
                continue
            if f_[0] == "slot":
                sinks, recent, t, slot = map(int, f_[1:])
                assert O.window_slot(t, sinks, recent) == slot, line
                n_slot += 1
            else:
                sinks, recent, T = map(int, f_[1:4])
                want = [int(x) for x in f_[4:]]
                assert list(np.nonzero(O.window_mask(T, sinks, recent))[0]) == want, line
                n_mask += 1
    assert n_slot >= 20 and n_mask >= 6


def test_window_slots_are_distinct():
    """Within any length, the window positions map to distinct slots of the buffer."""
    for sinks, recent in ((4, 128), (0, 5), (3, 1), (8, 0), (2, 16)):
        for T in range(0, 300):
            pos = np.nonzero(O.window_mask(T, sinks, recent))[0]
            slots = [O.window_slot(t, sinks, recent) for t in pos]
            assert len(set(slots)) == len(slots)
            assert all(0 <= s < sinks + recent for s in slots)


def test_window_positions_survive_absent_pages():
    """An absent page drops its INT2 positions but not the window positions on it."""
    c = _tiny(seq_lens=[64], dtype="bf16")
    pool = np.zeros(O.pool_bytes(c.num_pages, 1), np.uint8)
    O.append_tokens(pool, 1, c.slots, c.k, c.v, c.mu, c.r_k, c.r_v)
    table = c.page_table.copy()
    table[0, 0] = -1  # positions 0..15 absent from the INT2 cache; sinks 0..3 stay
    ks, vs = _seqs(c, c.k), _seqs(c, c.v)
    got = O.decode_attention_window(c.q, pool, 1, table, c.seq_lens, c.mu, c.r_k, c.r_v, ks, vs, 4, 10,
                                    num_pages=c.num_pages)
    k_eff, v_eff = O.effective_kv_window(pool, 1, c.page_table[0], 64, 0, c.mu[0], c.r_k[0], c.r_v[0], ks[0][:, 0],
                                         vs[0][:, 0], 4, 10)
    keep = np.r_[0:4, 16:64]
    for j in range(c.Hq):
        ref = _brute_attention(c.q[0, j], k_eff[keep], v_eff[keep], 1 / np.sqrt(128))
        np.testing.assert_allclose(got[0, j], ref, rtol=0, atol=1e-11)


# ------------------------------------------------------- Q2 clip ratio c < 1
def test_quantizer_clip_golden_groups(golden_dir):
    """OptR §3.1 Q2(.; c, G): hand-derived groups with c = 0.5 and c = 0.8 (both range ends
    scale by c; values past the narrowed range take the end codes)."""
    cases = {}
    with open(os.path.join(golden_dir, "int2_clip_groups.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, field, *rest = line.split()
            c = cases.setdefault(name, {})
            if field == "values":
                c[field] = np.array(_parse_runs(rest, float), dtype=np.float32)
            elif field == "codes":
                c[field] = np.array(_parse_runs(rest, int), dtype=np.uint8)
            else:
                c[field] = float(rest[0])
    assert set(cases) == {"E", "F"}
    for name, c in cases.items():
        assert c["values"].shape == (32,) and c["codes"].shape == (32,)
        row = np.tile(c["values"], 4)[None, :]
        codes, s16, z16 = O.int2_quantize(row, clip=c["clip"])
        for grp in range(4):
            assert float(s16[0, grp]) == c["scale"], (name, grp)
            assert float(z16[0, grp]) == c["zero"], (name, grp)
            np.testing.assert_array_equal(codes[0, 32 * grp:32 * grp + 32], c["codes"], err_msg=name)


def test_quantizer_clip_one_is_the_default_and_clipped_codes_are_nearest():
    """c = 1 is the unclipped quantizer bit for bit; for c < 1 each code is the level of
    z + s*{0..3} nearest to the value (ties aside), the ends absorbing values outside."""
    rng = np.random.default_rng(31)
    x = _random_rows(rng, 64, scale=3.0, offset=0.5)
    np.testing.assert_array_equal(O.int2_quantize(x, clip=1.0)[0], O.int2_quantize(x)[0])
    for c in (0.95, 0.8, 0.6):
        codes, s16, z16 = O.int2_quantize(x, clip=c)
        xg = x.reshape(64, 4, 32).astype(np.float64)
        s = s16.astype(np.float64)[..., None]
        z = z16.astype(np.float64)[..., None]
        levels = z[..., None] + s[..., None] * np.arange(4)  # [64, 4, 1, 4]
        dist = np.abs(xg[..., None] - levels)
        got = np.take_along_axis(dist, codes.reshape(64, 4, 32)[..., None].astype(np.int64), -1)[..., 0]
        best = dist.min(-1)
        # the chosen level is nearest up to fp32 rounding of (x - z) / s
        assert np.all(got <= best + 1e-5 * (np.abs(xg) + s[..., 0:1])), c
        # a negative group minimum lies below the narrowed range (c * min > min): code 0
        cg = codes.reshape(64, 4, 32)
        at_min = (xg == xg.min(-1, keepdims=True)) & (xg < 0)
        assert at_min.any() and np.all(cg[at_min] == 0), c


# ------------------------------------------------ structured (Hadamard) rotation
def _sylvester(d):
    """Sylvester's construction by the Kronecker recursion H_2n = [[H, H], [H, -H]]."""
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def _fwht_recursive(x):
    """Walsh-Hadamard transform of a vector by recursion on halves (unnormalised)."""
    n = len(x)
    if n == 1:
        return x.copy()
    a, b = _fwht_recursive(x[: n // 2]), _fwht_recursive(x[n // 2:])
    return np.concatenate([a + b, a - b])


def test_hadamard_rotation_matches_sylvester_and_fwht():
    """hadamard_rotation(s) = diag(s) H / sqrt(128): H equals the Kronecker-recursive
    Sylvester matrix, x R equals the recursive Walsh-Hadamard transform of x * s, R is
    orthogonal, and with all signs +1 it is symmetric (its own inverse)."""
    rng = np.random.default_rng(77)
    signs = rng.choice([-1.0, 1.0], size=(2, 128))
    r = O.hadamard_rotation(signs)
    h = _sylvester(128)
    for k in range(2):
        np.testing.assert_array_equal(r[k] * np.sqrt(128), signs[k][:, None] * h)
        assert np.abs(r[k].T @ r[k] - np.eye(128)).max() < 1e-14
        x = rng.standard_normal(128)
        np.testing.assert_allclose(x @ r[k], _fwht_recursive(x * signs[k]) / np.sqrt(128), rtol=0, atol=1e-13)
    plain = O.hadamard_rotation(np.ones((1, 128)))[0]
    np.testing.assert_allclose(plain @ plain, np.eye(128), atol=1e-14)
    np.testing.assert_array_equal(plain, plain.T)


# ------------------------------------------------ Q2 group size G = 64, 128
def _group_row():
    """One row whose 32-channel halves have different ranges, so G = 32, 64 and 128
    give different scales: channels 0-31 alternate 0, 3; 32-63 alternate -3, 0;
    64-95 alternate 10, 10.75; 96-127 alternate 10.25, 10.5 (all exact in fp16)."""
    alt = lambda a, b: np.where(np.arange(32) % 2 == 0, a, b)
    return np.concatenate([alt(0.0, 3.0), alt(-3.0, 0.0), alt(10.0, 10.75), alt(10.25, 10.5)]).astype(np.float32)[None]


def test_quantizer_group_sizes_hand_derived():
    """Hand-derived codes of _group_row for each G (closed forms, no quantizer call):
    G = 64: group 0 spans [-3, 3]: s = 2, z = -3, levels -3, -1, 1, 3, so 0 -> 1.5 -> 2
            (half to even), 3 -> 3, -3 -> 0; group 1 spans [10, 10.75]: s = 0.25, z = 10,
            so 10 -> 0, 10.75 -> 3, 10.25 -> 1, 10.5 -> 2.
    G = 128: one group spanning [-3, 10.75]: s32 = 13.75 / 3 = 4.58333..., fp16 of it is
            1173 * 2^-8 = 4.58203125, z = -3; (x + 3) / s = 0, 0.655, 1.309, 2.837, 2.892,
            2.946, 3.0017 for x = -3, 0, 3, 10, 10.25, 10.5, 10.75: codes 0, 1, 1, 3, 3, 3, 3.
    G = 32: channels 0-31 alone span [0, 3]: s = 1, z = 0, so 0 -> 0 (unlike G = 64)."""
    x = _group_row()
    alt = lambda a, b: np.where(np.arange(32) % 2 == 0, a, b)
    c64, s64, z64 = O.int2_quantize(x, group=64)
    np.testing.assert_array_equal(s64[0], np.array([2.0, 0.25], np.float16))
    np.testing.assert_array_equal(z64[0], np.array([-3.0, 10.0], np.float16))
    np.testing.assert_array_equal(c64[0], np.concatenate([alt(2, 3), alt(0, 2), alt(0, 3), alt(1, 2)]))
    c128, s128, z128 = O.int2_quantize(x, group=128)
    assert s128[0, 0] == np.float16(4.58203125) and z128[0, 0] == np.float16(-3.0)
    np.testing.assert_array_equal(c128[0], np.concatenate([alt(1, 1), alt(0, 1), alt(3, 3), alt(3, 3)]))
    c32, s32, _ = O.int2_quantize(x, group=32)
    assert s32[0, 0] == np.float16(1.0) and c32[0, 0] == 0 and c32[0, 1] == 3


def test_quantizer_group_sizes_nearest_level_and_shared_metadata():
    """For G = 64 and 128: four levels per group, each code the nearest level (brute
    force), G = 32 the default; a packed block keeps one pair per group, and
    unpacking gives back the same levels."""
    rng = np.random.default_rng(41)
    x = np.concatenate([_random_rows(rng, 40), _random_rows(rng, 24, 5.0, -1.0)])
    np.testing.assert_array_equal(O.int2_quantize(x)[0], O.int2_quantize(x, group=32)[0])
    for g in (64, 128):
        codes, s16, z16 = O.int2_quantize(x, group=g)
        assert s16.shape == (64, 128 // g)
        xg = x.reshape(64, 128 // g, g).astype(np.float64)
        levels = z16.astype(np.float64)[..., None, None] + s16.astype(np.float64)[..., None, None] * np.arange(4)
        dist = np.abs(xg[..., None] - levels)
        got = np.take_along_axis(dist, codes.reshape(64, 128 // g, g)[..., None].astype(np.int64), -1)[..., 0]
        tol = 4 * np.spacing(np.maximum(s16.astype(np.float32), np.float32(1e-30))).astype(np.float64)[..., None]
        assert np.all(got <= dist.min(-1) + tol + 1e-12), g
        # pack 16 rows into one block (one metadata pair per group) and read it back
        blk = O.pack_block(codes[:16], s16[:16], z16[:16], codes[16:32], s16[16:32], z16[16:32], group=g)
        assert blk.size == 1024 + 128 * (128 // g)
        kc, ks, kz, vc, vs, vz = O.unpack_block(blk, group=g)
        np.testing.assert_array_equal(ks, s16[:16])
        np.testing.assert_array_equal(vz, z16[16:32])
        np.testing.assert_array_equal(O.int2_dequantize(kc, ks, kz), O.int2_dequantize(codes[:16], s16[:16], z16[:16]))
        np.testing.assert_array_equal(O.int2_dequantize(vc, vs, vz),
                                      O.int2_dequantize(codes[16:32], s16[16:32], z16[16:32]))


def test_decode_with_group_size_equals_attention_on_effective_kv():
    """Decode over a pool written with G = 64 or 128 equals attention on the effective
    K/V of Q2(.; 1, G), as for G = 32 (OptR §3.2, Eq. (5))."""
    c = _tiny(B=2, Hq=8, Hkv=2, seq_lens=[50, 33], table_policy="permuted")
    x, w = O.rotated_inputs(c.k, c.v, c.mu, c.r_k, c.r_v)
    for g in (64, 128):
        pool = np.zeros(O.pool_bytes(c.num_pages, c.Hkv, group=g), np.uint8)
        O.append_tokens(pool, c.Hkv, c.slots, c.k, c.v, c.mu, c.r_k, c.r_v, group=g)
        got = O.decode_attention(c.q, pool, c.Hkv, c.page_table, c.seq_lens, c.r_k, c.r_v, group=g)
        kq = O.int2_dequantize(*O.int2_quantize(x, group=g))
        vq = O.int2_dequantize(*O.int2_quantize(w, group=g))
        for b in range(c.B):
            sel = c.tok_seq == b
            for j in range(c.Hq):
                h = j // 4
                k_eff = kq[sel, h] @ c.r_k[h].astype(np.float64).T + c.mu[h]
                v_eff = vq[sel, h] @ c.r_v[h].astype(np.float64).T
                ref = O.softmax_attention(c.q[b, j], k_eff, v_eff, 1 / np.sqrt(128))
                np.testing.assert_allclose(got[b, j], ref, rtol=0, atol=1e-11)


# ----------------------------------------------- output-error evaluator (Eq. 6-10)
def _eval_case(lens=(50, 0, 33), Hq=8, Hkv=2, d_model=96, seed=81):
    c = _tiny(B=len(lens), Hq=Hq, Hkv=Hkv, seq_lens=list(lens), table_policy="permuted")
    pool = np.zeros(O.pool_bytes(c.num_pages, c.Hkv), np.uint8)
    O.append_tokens(pool, c.Hkv, c.slots, c.k, c.v, c.mu, c.r_k, c.r_v)
    ks = [c.k[c.tok_seq == b] for b in range(c.B)]
    vs = [c.v[c.tok_seq == b] for b in range(c.B)]
    w_o = np.random.default_rng(seed).standard_normal((d_model, Hq * 128)) / np.sqrt(128)
    return c, pool, ks, vs, w_o


def test_output_error_matches_decode_and_plain_attention():
    """dy_K + dy_V equals (decode read from the pool - exact attention) W_O,j^T: the
    decode oracle works in the rotated basis (q R_K against x_hat), this one on the
    effective keys in the original basis.  dy_K alone equals the exact values read
    with the INT2-key probabilities minus exact attention; e_out = ||dy||^2; an empty
    sequence gives zeros."""
    c, pool, ks, vs, w_o = _eval_case()
    dy_k, dy_v, e_out, e_rec = O.output_error(c.q, pool, c.Hkv, c.page_table, c.seq_lens, ks, vs, c.mu, c.r_k,
                                              c.r_v, w_o)
    o_q = O.decode_attention(c.q, pool, c.Hkv, c.page_table, c.seq_lens, c.r_k, c.r_v)
    s = 1 / np.sqrt(128)
    g = c.Hq // c.Hkv
    for b in range(c.B):
        for j in range(c.Hq):
            h = j // g
            w_oj = w_o[:, j * 128:(j + 1) * 128]
            if c.seq_lens[b] == 0:
                assert not dy_k[b, j].any() and not dy_v[b, j].any() and e_out[b, j] == 0 and e_rec[b, h] == 0
                continue
            o = O.softmax_attention(c.q[b, j], ks[b][:, h], vs[b][:, h], s)
            np.testing.assert_allclose(dy_k[b, j] + dy_v[b, j], (o_q[b, j] - o) @ w_oj.T, rtol=0, atol=1e-10)
            x_hat, _ = O.gather_sequence(pool, c.Hkv, c.page_table[b], c.seq_lens[b], h)
            k_eff = x_hat @ c.r_k[h].astype(np.float64).T + c.mu[h]
            o_kq = O.softmax_attention(c.q[b, j], k_eff, vs[b][:, h], s)
            np.testing.assert_allclose(dy_k[b, j], (o_kq - o) @ w_oj.T, rtol=0, atol=1e-10)
            dy = dy_k[b, j] + dy_v[b, j]
            assert abs(e_out[b, j] - dy @ dy) <= 1e-9 * max(e_out[b, j], 1e-30)


def test_output_error_reconstruction_term_per_token():
    """e_rec (Eq. (9)) summed token by token: each slot unpacked alone, its levels
    rotated back, mu added to the key; the squared distances to the exact rows."""
    c, pool, ks, vs, w_o = _eval_case(lens=(37, 16))
    *_, e_rec = O.output_error(c.q, pool, c.Hkv, c.page_table, c.seq_lens, ks, vs, c.mu, c.r_k, c.r_v, w_o)
    for b in range(c.B):
        for h in range(c.Hkv):
            tot = 0.0
            for t in range(int(c.seq_lens[b])):
                page = int(c.page_table[b, t // 16])
                kc, ksc, kz, vc, vsc, vz = O.unpack_block(O.block_view(pool, page, h, c.Hkv))
                xk = O.int2_dequantize(kc[t % 16][None], ksc[t % 16][None], kz[t % 16][None])[0]
                xv = O.int2_dequantize(vc[t % 16][None], vsc[t % 16][None], vz[t % 16][None])[0]
                kt = xk @ c.r_k[h].astype(np.float64).T + c.mu[h]
                vt = xv @ c.r_v[h].astype(np.float64).T
                tot += ((ks[b][t, h] - kt) ** 2).sum() + ((vs[b][t, h] - vt) ** 2).sum()
            assert abs(e_rec[b, h] - tot) <= 1e-10 * tot


def test_output_error_leaves_out_absent_pages_and_exact_cache_gives_zero():
    """An absent page's positions drop out of the exact and the INT2 readouts alike
    (so e_rec shrinks by their terms); with the effective K/V passed as the exact
    ones every term is zero."""
    c, pool, ks, vs, w_o = _eval_case(lens=(40,))
    table = c.page_table.copy()
    table[0, 1] = c.num_pages + 7
    full = O.output_error(c.q, pool, c.Hkv, c.page_table, c.seq_lens, ks, vs, c.mu, c.r_k, c.r_v, w_o)
    cut = O.output_error(c.q, pool, c.Hkv, table, c.seq_lens, ks, vs, c.mu, c.r_k, c.r_v, w_o)
    keep = np.r_[0:16, 32:40]
    ks2 = [ks[0][keep]]
    vs2 = [vs[0][keep]]
    # the same as a sequence made of the present positions only (exact rows and cache rows)
    for h in range(c.Hkv):
        x_hat, w_hat = O.gather_sequence(pool, c.Hkv, table[0], 40, h)
        assert x_hat.shape[0] == 24
    assert cut[3][0].sum() < full[3][0].sum()
    o_q = O.decode_attention(c.q, pool, c.Hkv, table, c.seq_lens, c.r_k, c.r_v)
    for j in range(c.Hq):
        h = j // (c.Hq // c.Hkv)
        o = O.softmax_attention(c.q[0, j], ks2[0][:, h], vs2[0][:, h], 1 / np.sqrt(128))
        np.testing.assert_allclose(cut[0][0, j] + cut[1][0, j], (o_q[0, j] - o) @ w_o[:, j * 128:(j + 1) * 128].T,
                                   rtol=0, atol=1e-10)
    # exact rows equal to the effective ones: no error at all
    eff_k, eff_v = [], []
    for h in range(c.Hkv):
        x_hat, w_hat = O.gather_sequence(pool, c.Hkv, c.page_table[0], 40, h)
        eff_k.append(x_hat @ c.r_k[h].astype(np.float64).T + c.mu[h])
        eff_v.append(w_hat @ c.r_v[h].astype(np.float64).T)
    z = O.output_error(c.q, pool, c.Hkv, c.page_table, c.seq_lens, [np.stack(eff_k, 1)], [np.stack(eff_v, 1)],
                       c.mu, c.r_k, c.r_v, w_o)
    assert max(np.abs(z[0]).max(), np.abs(z[1]).max(), z[2].max(), z[3].max()) < 1e-20


# ------------------------------------------------- 4-bit keys (K4V2 budget)
def test_k4_block_layout_golden(golden_dir):
    """Hand-derived byte positions of 4-bit key codes (low bits in place, high
    bits in the plane at byte 1536); values and metadata are unaffected."""
    with open(os.path.join(golden_dir, "block_layout_k4.txt")) as f:
        lines = [l.split() for l in f if l.strip() and not l.startswith("#")]
    z = np.zeros((1, 128), np.uint8)
    zf = np.zeros((1, 4), np.float16)
    for parts in lines:
        slot, ch, code, *pairs = map(int, parts[1:])
        kc = z.copy()
        kc[0, ch] = code
        blk = O.pack_block(kc, zf, zf, z, zf, zf, slots=[slot], key_bits=4)
        assert blk.size == 2048
        want = dict(zip(pairs[0::2], pairs[1::2]))
        nz = np.nonzero(blk)[0]
        assert set(nz) == set(want) and all(blk[b] == v for b, v in want.items()), parts
        back = O.unpack_block(blk, key_bits=4)[0]
        assert back[slot, ch] == code and np.count_nonzero(back) == 1
    assert len(lines) == 4


def test_quantizer_four_bits_hand_derived_and_nearest():
    """bits = 4: a group holding 0..15 twice is exact (s = 1, z = 0); 7.5 ties to 8;
    a group spanning [-1, 2] has s = fp16(0.2) = 0.199951171875, so 0 -> 5.  Every
    code is the nearest of 16 levels (brute force); 2-bit and 4-bit agree on
    the range (z and the span of the levels)."""
    row = np.zeros(128, np.float32)
    row[:32] = np.tile(np.arange(16, dtype=np.float32), 2)
    row[32:64] = np.float32(0.0)
    row[32], row[33], row[34] = 0.0, 7.5, 15.0
    row[64:96] = np.float32(0.0)
    row[64], row[65] = -1.0, 2.0
    row[96:] = np.float32(3.0)
    codes, s16, z16 = O.int2_quantize(row[None], bits=4)
    np.testing.assert_array_equal(codes[0, :32], np.tile(np.arange(16), 2))
    assert s16[0, 0] == np.float16(1.0) and z16[0, 0] == np.float16(0.0)
    assert codes[0, 33] == 8 and codes[0, 34] == 15 and codes[0, 32] == 0
    assert s16[0, 2] == np.float16(0.199951171875) and z16[0, 2] == np.float16(-1.0)
    assert codes[0, 66] == 5 and codes[0, 64] == 0 and codes[0, 65] == 15
    assert s16[0, 3] == 0 and np.all(codes[0, 96:] == 0)  # constant group
    rng = np.random.default_rng(43)
    x = _random_rows(rng, 64, 3.0, 0.5)
    codes, s16, z16 = O.int2_quantize(x, bits=4)
    assert codes.max() <= 15
    xg = x.reshape(64, 4, 32).astype(np.float64)
    levels = z16.astype(np.float64)[..., None, None] + s16.astype(np.float64)[..., None, None] * np.arange(16)
    dist = np.abs(xg[..., None] - levels)
    got = np.take_along_axis(dist, codes.reshape(64, 4, 32)[..., None].astype(np.int64), -1)[..., 0]
    tol = 4 * np.spacing(np.maximum(s16.astype(np.float32), np.float32(1e-30))).astype(np.float64)[..., None]
    assert np.all(got <= dist.min(-1) + tol + 1e-12)
    c2, s2, z2 = O.int2_quantize(x)
    np.testing.assert_array_equal(z2, z16)
    np.testing.assert_allclose(3 * s2.astype(np.float64), 15 * s16.astype(np.float64), rtol=2e-3)


def test_k4_pack_unpack_roundtrip_and_partial_writes():
    rng = np.random.default_rng(44)
    kc = rng.integers(0, 16, (16, 128)).astype(np.uint8)
    vc = rng.integers(0, 4, (16, 128)).astype(np.uint8)
    ks, kz, vs, vz = (rng.standard_normal((16, 4)).astype(np.float16) for _ in range(4))
    blk = O.pack_block(kc, ks, kz, vc, vs, vz, key_bits=4)
    out = O.unpack_block(blk, key_bits=4)
    for got, want in zip(out, (kc, ks, kz, vc, vs, vz)):
        np.testing.assert_array_equal(got, want)
    # the 2-bit reading of the first 1536 bytes sees the low bits
    np.testing.assert_array_equal(O.unpack_block(blk[:1536])[0], kc & 3)
    # rewriting slots 3 and 9 leaves the other slots intact
    kc2 = rng.integers(0, 16, (2, 128)).astype(np.uint8)
    O.pack_block(kc2, ks[:2], kz[:2], vc[:2], vs[:2], vz[:2], block=blk, slots=[3, 9], key_bits=4)
    back = O.unpack_block(blk, key_bits=4)[0]
    np.testing.assert_array_equal(back[[3, 9]], kc2)
    keep = np.setdiff1d(np.arange(16), [3, 9])
    np.testing.assert_array_equal(back[keep], kc[keep])


def test_k4_decode_equals_attention_on_effective_kv_and_is_closer():
    """Decode over a 4-bit-key pool equals Eq. (1)-(2) attention on k~ = Q4((k - mu) R_K)
    R_K^T + mu and v~ = Q2(v R_V) R_V^T (OptR §3.2, Eq. (5)); its key error is below
    the 2-bit one."""
    c = _tiny(B=2, Hq=8, Hkv=2, seq_lens=[50, 33], table_policy="permuted")
    pool = np.zeros(O.pool_bytes(c.num_pages, c.Hkv, key_bits=4), np.uint8)
    O.append_tokens(pool, c.Hkv, c.slots, c.k, c.v, c.mu, c.r_k, c.r_v, key_bits=4)
    got = O.decode_attention(c.q, pool, c.Hkv, c.page_table, c.seq_lens, c.r_k, c.r_v, key_bits=4)
    x, w = O.rotated_inputs(c.k, c.v, c.mu, c.r_k, c.r_v)
    kq = O.int2_dequantize(*O.int2_quantize(x, bits=4))
    vq = O.int2_dequantize(*O.int2_quantize(w))
    for b in range(c.B):
        sel = c.tok_seq == b
        for j in range(c.Hq):
            h = j // 4
            k_eff = kq[sel, h] @ c.r_k[h].astype(np.float64).T + c.mu[h]
            v_eff = vq[sel, h] @ c.r_v[h].astype(np.float64).T
            ref = O.softmax_attention(c.q[b, j], k_eff, v_eff, 1 / np.sqrt(128))
            np.testing.assert_allclose(got[b, j], ref, rtol=0, atol=1e-11)
    e4 = np.abs(kq - x).mean()
    e2 = np.abs(O.int2_dequantize(*O.int2_quantize(x)) - x).mean()
    assert e4 < 0.3 * e2


def test_quantizer_three_bits_hand_derived_and_nearest():
    """bits = 3 (K3V2 keys): a group holding 0..7 four times is exact (s = 1, z = 0);
    3.5 ties to 4; codes stay in 0..7, each the nearest of 8 levels (brute force);
    a 3-bit pool decodes like attention on its effective keys."""
    row = np.zeros(128, np.float32)
    row[:32] = np.tile(np.arange(8, dtype=np.float32), 4)
    row[32:64] = 0.0
    row[32], row[33], row[34] = 0.0, 3.5, 7.0
    codes, s16, z16 = O.int2_quantize(row[None], bits=3)
    np.testing.assert_array_equal(codes[0, :32], np.tile(np.arange(8), 4))
    assert s16[0, 0] == np.float16(1.0) and codes[0, 33] == 4 and codes[0, 34] == 7
    rng = np.random.default_rng(45)
    x = _random_rows(rng, 64, 2.0, -0.5)
    codes, s16, z16 = O.int2_quantize(x, bits=3)
    assert codes.max() <= 7
    xg = x.reshape(64, 4, 32).astype(np.float64)
    levels = z16.astype(np.float64)[..., None, None] + s16.astype(np.float64)[..., None, None] * np.arange(8)
    dist = np.abs(xg[..., None] - levels)
    got = np.take_along_axis(dist, codes.reshape(64, 4, 32)[..., None].astype(np.int64), -1)[..., 0]
    tol = 4 * np.spacing(np.maximum(s16.astype(np.float32), np.float32(1e-30))).astype(np.float64)[..., None]
    assert np.all(got <= dist.min(-1) + tol + 1e-12)
    c = _tiny(B=1, Hq=4, Hkv=1, seq_lens=[40], table_policy="permuted")
    pool = np.zeros(O.pool_bytes(c.num_pages, c.Hkv, key_bits=3), np.uint8)
    O.append_tokens(pool, c.Hkv, c.slots, c.k, c.v, c.mu, c.r_k, c.r_v, key_bits=3)
    got = O.decode_attention(c.q, pool, c.Hkv, c.page_table, c.seq_lens, c.r_k, c.r_v, key_bits=3)
    xr, wr = O.rotated_inputs(c.k, c.v, c.mu, c.r_k, c.r_v)
    kq = O.int2_dequantize(*O.int2_quantize(xr, bits=3))
    vq = O.int2_dequantize(*O.int2_quantize(wr))
    for j in range(c.Hq):
        ref = O.softmax_attention(c.q[0, j], kq[:, 0] @ c.r_k[0].astype(np.float64).T + c.mu[0],
                                  vq[:, 0] @ c.r_v[0].astype(np.float64).T, 1 / np.sqrt(128))
        np.testing.assert_allclose(got[0, j], ref, rtol=0, atol=1e-11)


# ------------------------------------------- 3- and 4-bit values (K3V3 budget)
def test_wide_value_block_layout_golden(golden_dir):
    """Hand-derived byte positions of wide value codes (low bits in place, high
    bits in the value plane after the keys' plane); keys and metadata are
    unaffected and the block grows by the planes (256 bytes for 3 bits, 512 for 4)."""
    with open(os.path.join(golden_dir, "block_layout_wide_v.txt")) as f:
        lines = [l.split() for l in f if l.strip() and not l.startswith("#")]
    z = np.zeros((1, 128), np.uint8)
    zf = np.zeros((1, 4), np.float16)
    for parts in lines:
        kb, vb, slot, ch, code, *pairs = map(int, parts[1:])
        vc = z.copy()
        vc[0, ch] = code
        blk = O.pack_block(z, zf, zf, vc, zf, zf, slots=[slot], key_bits=kb, val_bits=vb)
        assert blk.size == 1536 + {2: 0, 3: 256, 4: 512}[kb] + {2: 0, 3: 256, 4: 512}[vb]
        want = dict(zip(pairs[0::2], pairs[1::2]))
        nz = np.nonzero(blk)[0]
        assert set(nz) == set(want) and all(blk[b] == v for b, v in want.items()), parts
        back = O.unpack_block(blk, key_bits=kb, val_bits=vb)[3]
        assert back[slot, ch] == code and np.count_nonzero(back) == 1
    assert len(lines) == 4


def test_wide_value_pack_unpack_roundtrip_and_planes_independent():
    """K3V3 and K4V4 blocks round-trip; the key plane and the value plane do not
    overlap (rewriting values leaves every key bit as it was and vice versa)."""
    rng = np.random.default_rng(46)
    for kb, vb in ((3, 3), (4, 4), (2, 4)):
        kc = rng.integers(0, 1 << kb, (16, 128)).astype(np.uint8)
        vc = rng.integers(0, 1 << vb, (16, 128)).astype(np.uint8)
        ks, kz, vs, vz = (rng.standard_normal((16, 4)).astype(np.float16) for _ in range(4))
        blk = O.pack_block(kc, ks, kz, vc, vs, vz, key_bits=kb, val_bits=vb)
        for got, want in zip(O.unpack_block(blk, key_bits=kb, val_bits=vb), (kc, ks, kz, vc, vs, vz)):
            np.testing.assert_array_equal(got, want)
        # the 2-bit reading of the first 1536 bytes sees the low bits of both
        lo = O.unpack_block(blk[:1536])
        np.testing.assert_array_equal(lo[0], kc & 3)
        np.testing.assert_array_equal(lo[3], vc & 3)
        vc2 = rng.integers(0, 1 << vb, (16, 128)).astype(np.uint8)
        O.pack_block(kc, ks, kz, vc2, vs, vz, block=blk, key_bits=kb, val_bits=vb)
        back = O.unpack_block(blk, key_bits=kb, val_bits=vb)
        np.testing.assert_array_equal(back[0], kc)
        np.testing.assert_array_equal(back[3], vc2)


def test_wide_value_decode_equals_attention_on_effective_kv_and_is_closer():
    """Decode over a K3V3 pool equals Eq. (1)-(2) attention on k~ = Q3((k - mu) R_K)
    R_K^T + mu and v~ = Q3(v R_V) R_V^T (OptR §3.2, Eq. (5)); its value
    reconstruction error is below the 2-bit one, and so is the value part of
    the output error (Eq. (8))."""
    c = _tiny(B=2, Hq=8, Hkv=2, seq_lens=[50, 33], table_policy="permuted")
    pools = {}
    for vb in (2, 3):
        pool = np.zeros(O.pool_bytes(c.num_pages, c.Hkv, key_bits=3, val_bits=vb), np.uint8)
        O.append_tokens(pool, c.Hkv, c.slots, c.k, c.v, c.mu, c.r_k, c.r_v, key_bits=3, val_bits=vb)
        pools[vb] = pool
    got = O.decode_attention(c.q, pools[3], c.Hkv, c.page_table, c.seq_lens, c.r_k, c.r_v, key_bits=3,
                             val_bits=3)
    x, w = O.rotated_inputs(c.k, c.v, c.mu, c.r_k, c.r_v)
    kq = O.int2_dequantize(*O.int2_quantize(x, bits=3))
    vq = O.int2_dequantize(*O.int2_quantize(w, bits=3))
    for b in range(c.B):
        sel = c.tok_seq == b
        for j in range(c.Hq):
            h = j // 4
            k_eff = kq[sel, h] @ c.r_k[h].astype(np.float64).T + c.mu[h]
            v_eff = vq[sel, h] @ c.r_v[h].astype(np.float64).T
            ref = O.softmax_attention(c.q[b, j], k_eff, v_eff, 1 / np.sqrt(128))
            np.testing.assert_allclose(got[b, j], ref, rtol=0, atol=1e-11)
    assert np.abs(vq - w).mean() < 0.6 * np.abs(O.int2_dequantize(*O.int2_quantize(w)) - w).mean()
    rng = np.random.default_rng(47)
    w_o = rng.standard_normal((64, c.Hq * 128)) / np.sqrt(c.Hq * 128)
    k_seqs = [c.k[c.tok_seq == b] for b in range(c.B)]
    v_seqs = [c.v[c.tok_seq == b] for b in range(c.B)]
    dv = {vb: O.output_error(c.q, pools[vb], c.Hkv, c.page_table, c.seq_lens, k_seqs, v_seqs, c.mu, c.r_k,
                             c.r_v, w_o, key_bits=3, val_bits=vb)[1] for vb in (2, 3)}
    assert np.linalg.norm(dv[3]) < 0.6 * np.linalg.norm(dv[2])
