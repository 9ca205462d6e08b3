"""Host-side checks of the C ABI (no GPU): the library loads, exports exactly
the entry points include/kvq.h declares, and its host logic (sizes, page
tables, argument validation) behaves as documented.  No call here reaches a
kernel launch: every failing call is rejected by host validation first.
"""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


@pytest.fixture(scope="module")
def K():
    from rotated_int2_kv_centering_amd import kvq

    if not os.path.exists(kvq.LIB_PATH):  # fresh checkout: build once, as __graft_entry__.build() does
        from rotated_int2_kv_centering_amd import build

        build.build()
    # KVQ_TEST_LIB: another build of the same library (the host-sanitized one, see
    # test_host_sanitizers.py)
    kvq.load(os.environ.get("KVQ_TEST_LIB", kvq.LIB_PATH))
    return kvq


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(kvq_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["kvq_pool_bytes", "kvq_quant_append", "kvq_quant_append_err", "kvq_decode_workspace_bytes",
                            "kvq_decode_attn", "kvq_decode_attn_noalloc", "kvq_decode_attn_traced", "kvq_decode_step",
                            "kvq_window_bytes",
                            "kvq_window_fill", "kvq_output_error_workspace_bytes", "kvq_output_error",
                            "kvq_page_table", "kvq_last_error"]), names


def test_library_exports_exactly_the_declared_symbols(K):
    lib = K.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", K.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if l.split()[-2:-1] == ["T"] and "kvq_" in l.split()[-1]})
    assert exported == declared_functions()


def test_python_binding_has_the_same_names(K):
    for name in declared_functions():
        assert callable(getattr(K, name)), name


def test_pool_bytes(K):
    assert K.kvq_pool_bytes(K.make_cache(8, 8192)) == 8192 * 8 * 1536
    assert K.kvq_pool_bytes(K.make_cache(1, 16)) == 16 * 1536
    assert K.kvq_pool_bytes(K.make_cache(0, 16)) == 0
    assert K.kvq_pool_bytes(K.make_cache(8, 0)) == 0
    # the metadata holds one pair per group: 80 and 72 bytes per token for G = 64 and 128
    assert K.kvq_pool_bytes(K.make_cache(8, 16, group_size=64)) == 16 * 8 * 1280
    assert K.kvq_pool_bytes(K.make_cache(8, 16, group_size=128)) == 16 * 8 * 1152
    assert K.kvq_pool_bytes(K.make_cache(8, 16, group_size=48)) == 0  # unsupported group size
    assert K.kvq_pool_bytes(K.make_cache(8, 16, key_bits=5)) == 0


def test_pool_bytes_agree_with_the_oracle_layout(K):
    from oracle import kvq_oracle as O
    for g in (32, 64, 128):
        for kb in (2, 3, 4):
            for vb in (2, 3, 4):
                got = K.kvq_pool_bytes(K.make_cache(3, 5, group_size=g, key_bits=kb, val_bits=vb))
                assert got == O.pool_bytes(5, 3, kb, vb, g), (g, kb, vb)


CTR = 4096 * 4  # the fixed ticket prefix


def test_workspace_bytes_with_explicit_splits(K):
    # counters (a fixed 16 KiB prefix: up to 4096 (sequence, KV head) int32 tickets)
    # + B*Hq*n_splits partial rows of 132 floats + B*Hq window rows of 132 floats;
    # 1000 tokens = 63 pages: 7 splits of 9 pages
    assert K.kvq_decode_workspace_bytes(2, 8, 2, 1000, 7) == CTR + 4 * 2 * 8 * 7 * 132 + 4 * 2 * 8 * 132
    # a request of more splits than pages gives one page per split
    assert K.kvq_decode_workspace_bytes(1, 4, 1, 40, 16) == CTR + 4 * 1 * 4 * 3 * 132 + 4 * 4 * 132
    # at most 512 splits: pages per split grow instead
    big = 600 * 16
    assert K.kvq_decode_workspace_bytes(1, 4, 1, big, 600) == CTR + 4 * 4 * 300 * 132 + 4 * 4 * 132


def test_workspace_bytes_automatic_plan(K):
    # Automatic plan, 256 compute units: split slots per KV head
    # S = min(B * ceil(pages / pps_min), max(ceil(W / H_kv), ceil(B * pages / 2048)) + B - 1),
    # pps_min = max(8, ceil(pages / 512)); partial rows = H_q * S; window rows = B * H_q.
    # W = 256 workgroups, or 768 for a batch of g <= 4 (the narrow shape: three per compute unit).
    assert K.kvq_decode_workspace_bytes(1, 32, 8, 131072, 0) == CTR + 4 * 32 * 32 * 132 + 4 * 32 * 132
    assert K.kvq_decode_workspace_bytes(16, 32, 8, 65536, 0) == CTR + 4 * 32 * (96 + 15) * 132 + 4 * 16 * 32 * 132
    # one split per sequence
    assert K.kvq_decode_workspace_bytes(3, 8, 2, 100, 0) == CTR + 4 * 8 * 3 * 132 + 4 * 3 * 8 * 132
    # B = 4, 8192 pages: max(32, ceil(4 * 8192 / 2048) = 16) + 3 = 35 slots
    assert K.kvq_decode_workspace_bytes(4, 64, 8, 131072, 0) == CTR + 4 * 64 * 35 * 132 + 4 * 4 * 64 * 132


def test_workspace_ticket_prefix_grows_past_4096_pairs(K):
    # batch 600 x 8 KV heads = 4800 tickets: 19200 bytes (a multiple of 256)
    n = K.kvq_decode_workspace_bytes(600, 32, 8, 160, 1)
    assert n == 19200 + 4 * 600 * 32 * 1 * 132 + 4 * 600 * 32 * 132


def test_workspace_bytes_rejects_bad_shapes(K):
    assert K.kvq_decode_workspace_bytes(1, 6, 4, 100, 1) == 0   # Hq not a multiple of Hkv
    assert K.kvq_decode_workspace_bytes(-1, 4, 1, 100, 1) == 0
    assert K.kvq_decode_workspace_bytes(1, 4, 1, -5, 1) == 0
    assert K.kvq_decode_workspace_bytes(1, 4, 1, 512 * 2048 * 16 + 1, 1) == 0  # beyond the longest context


def test_page_table_contiguous_and_slots(K):
    lens = [5, 33, 0, 16]
    table, slots = K.kvq_page_table(K.KVQ_PT_CONTIGUOUS, 0, lens, 16, 10, 4)
    assert table.tolist() == [[0, -1, -1, -1], [1, 2, 3, -1], [-1, -1, -1, -1], [4, -1, -1, -1]]
    assert slots.tolist() == [4, 3 * 16 + 0, -1, 4 * 16 + 15]


@pytest.mark.parametrize("policy", ["KVQ_PT_PERMUTED", "KVQ_PT_INTERLEAVED"])
def test_page_table_random_policies_give_valid_tables(K, policy):
    rng = np.random.default_rng(5)
    lens = rng.integers(0, 400, size=9).astype(np.int32)
    need = (lens + 15) // 16
    table, slots = K.kvq_page_table(getattr(K, policy), 1234, lens, 16, int(need.sum()) + 7, int(need.max()))
    used = np.concatenate([table[b, :need[b]] for b in range(len(lens))])
    assert len(np.unique(used)) == len(used) == need.sum()
    assert used.min() >= 0 and used.max() < need.sum() + 7
    for b in range(len(lens)):
        assert (table[b, need[b]:] == -1).all()
        t = lens[b] - 1
        assert slots[b] == (-1 if t < 0 else table[b, t // 16] * 16 + t % 16)
    # the same seed gives the same table; the validator accepts it
    again, _ = K.kvq_page_table(getattr(K, policy), 1234, lens, 16, int(need.sum()) + 7, int(need.max()))
    assert (again == table).all()
    K.kvq_page_table(K.KVQ_PT_VALIDATE, 0, lens, 16, int(need.sum()) + 7, int(need.max()), table)


def test_page_table_validation_errors(K):
    lens = [20, 20]
    table = np.array([[0, 1], [2, 1]], dtype=np.int32)  # page 1 twice
    with pytest.raises(K.KvqError) as e:
        K.kvq_page_table(K.KVQ_PT_VALIDATE, 0, lens, 16, 4, 2, table)
    assert e.value.status == K.KVQ_EINVAL and "twice" in str(e.value)
    table = np.array([[0, 1], [2, 4]], dtype=np.int32)  # page 4 outside a pool of 4
    with pytest.raises(K.KvqError) as e:
        K.kvq_page_table(K.KVQ_PT_VALIDATE, 0, lens, 16, 4, 2, table)
    assert e.value.status == K.KVQ_EINVAL
    with pytest.raises(K.KvqError) as e:  # 4 pages needed, 3 in the pool
        K.kvq_page_table(K.KVQ_PT_PERMUTED, 0, lens, 16, 3, 2)
    assert e.value.status == K.KVQ_ENOSPACE
    with pytest.raises(K.KvqError) as e:  # a row of 1 page cannot hold 20 tokens
        K.kvq_page_table(K.KVQ_PT_PERMUTED, 0, lens, 16, 8, 1)
    assert e.value.status == K.KVQ_ENOSPACE
    with pytest.raises(K.KvqError) as e:
        K.kvq_page_table(K.KVQ_PT_CONTIGUOUS, 0, lens, 32, 8, 2)
    assert e.value.status == K.KVQ_EUNSUPPORTED


FAKE = 1 << 20  # a non-NULL, 16-byte aligned address; never dereferenced by rejected calls


def test_append_argument_validation(K):
    lib = K.load()
    ok = K.make_cache(2, 4, FAKE)
    assert lib.kvq_quant_append(None, FAKE, FAKE, K.KVQ_BF16, 1, FAKE, None, FAKE, FAKE, None, None) == K.KVQ_EINVAL
    bad_geom = K.make_cache(2, 4, FAKE, head_dim=64)
    assert lib.kvq_quant_append(ctypes.byref(bad_geom), FAKE, FAKE, K.KVQ_BF16, 1, FAKE, None, FAKE, FAKE, None,
                                None) == K.KVQ_EUNSUPPORTED
    assert "head_dim=64" in K.kvq_last_error()
    for g in (16, 48, 256):  # Q2 group sizes other than 32, 64, 128
        assert lib.kvq_quant_append(ctypes.byref(K.make_cache(2, 4, FAKE, group_size=g)), FAKE, FAKE, K.KVQ_BF16, 1,
                                    FAKE, None, FAKE, FAKE, None, None) == K.KVQ_EUNSUPPORTED
        assert f"group_size={g}" in K.kvq_last_error()
        assert _decode(K, K.make_cache(1, 8, FAKE, group_size=g)) == K.KVQ_EUNSUPPORTED
    assert lib.kvq_quant_append(ctypes.byref(ok), FAKE, FAKE, 7, 1, FAKE, None, FAKE, FAKE, None,
                                None) == K.KVQ_EUNSUPPORTED
    assert lib.kvq_quant_append(ctypes.byref(ok), FAKE, FAKE, K.KVQ_BF16, -1, FAKE, None, FAKE, FAKE, None,
                                None) == K.KVQ_EINVAL
    # zero tokens: nothing to do, OK without touching any pointer
    assert lib.kvq_quant_append(ctypes.byref(ok), None, None, K.KVQ_BF16, 0, None, None, None, None, None,
                                None) == K.KVQ_OK
    assert lib.kvq_quant_append(ctypes.byref(ok), FAKE, FAKE, K.KVQ_BF16, 1, FAKE, None, None, FAKE, None,
                                None) == K.KVQ_EINVAL  # rotation required for raw input
    empty = K.make_cache(2, 0, None)
    assert lib.kvq_quant_append(ctypes.byref(empty), FAKE, FAKE, K.KVQ_BF16, 1, FAKE, None, FAKE, FAKE, None,
                                None) == K.KVQ_ENOSPACE
    misaligned = K.make_cache(2, 4, FAKE + 4)
    assert lib.kvq_quant_append(ctypes.byref(misaligned), FAKE, FAKE, K.KVQ_BF16, 1, FAKE, None, FAKE, FAKE, None,
                                None) == K.KVQ_EINVAL


def _decode(K, cache, batch=1, hq=4, max_pages=4, max_seq=64, sm_scale=0.0, q_dtype=None, out_dtype=None,
            ws_bytes=1 << 20, num_splits=1, q=FAKE, window=None):
    lib = K.load()
    q_dtype = K.KVQ_BF16 if q_dtype is None else q_dtype
    out_dtype = K.KVQ_F32 if out_dtype is None else out_dtype
    return lib.kvq_decode_attn(ctypes.byref(cache) if cache is not None else None, q, q_dtype, batch, hq, FAKE,
                               max_pages, FAKE, max_seq, FAKE, FAKE, sm_scale, FAKE, out_dtype, FAKE, ws_bytes,
                               num_splits, ctypes.byref(window) if window is not None else None, None)


def test_decode_argument_validation(K):
    c = K.make_cache(1, 8, FAKE)
    assert _decode(K, None) == K.KVQ_EINVAL
    assert _decode(K, c, hq=3 * 1, batch=-1) == K.KVQ_EINVAL
    assert _decode(K, K.make_cache(2, 8, FAKE), hq=3) == K.KVQ_EINVAL          # 3 q heads over 2 KV heads
    assert _decode(K, c, hq=17) == K.KVQ_EUNSUPPORTED                           # g > 16
    assert _decode(K, c, q_dtype=K.KVQ_F32_ROTATED) == K.KVQ_EUNSUPPORTED
    assert _decode(K, c, out_dtype=5) == K.KVQ_EUNSUPPORTED
    assert _decode(K, c, max_pages=3, max_seq=64) == K.KVQ_EINVAL               # 64 tokens need 4 pages
    assert _decode(K, c, sm_scale=float("nan")) == K.KVQ_EINVAL
    assert _decode(K, c, sm_scale=-1.0) == K.KVQ_EINVAL
    assert _decode(K, c, num_splits=-2) == K.KVQ_EINVAL
    assert _decode(K, c, q=None) == K.KVQ_EINVAL
    need = K.kvq_decode_workspace_bytes(1, 4, 1, 64, 1)
    assert _decode(K, c, ws_bytes=need - 1) == K.KVQ_ENOSPACE
    assert "workspace" in K.kvq_last_error()
    assert _decode(K, c, max_pages=512 * 2048 + 1, max_seq=512 * 2048 * 16 + 1) == K.KVQ_EUNSUPPORTED
    assert _decode(K, K.make_cache(1, 0, None)) == K.KVQ_ENOSPACE
    # an empty batch is a no-op
    assert _decode(K, c, batch=0) == K.KVQ_OK


def test_binding_raises_with_the_library_message(K):
    c = K.make_cache(1, 8, FAKE, page_size=32)
    with pytest.raises(K.KvqError) as e:
        K.kvq_quant_append(c, FAKE, FAKE, K.KVQ_BF16, 1, FAKE, None, FAKE, FAKE, stream=0)
    assert e.value.status == K.KVQ_EUNSUPPORTED and "page_size=32" in str(e.value)


def test_binding_rejects_non_contiguous_arrays(K):
    a = np.zeros((4, 4), dtype=np.int32)[:, ::2]
    with pytest.raises(ValueError):
        K._ptr(a)


def test_probe_library_exports_its_declared_symbol():
    """The HBM read-rate probe (a measurement aid) is built beside libkvq and
    exports exactly what include/kvq_probe.h declares; bad arguments are
    rejected on the host, before any launch."""
    from rotated_int2_kv_centering_amd import build

    if not os.path.exists(build.PROBE_LIB):
        build.build()
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "kvq_probe.h")).read(), flags=re.S)
    declared = sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(kvq_\w+)\s*\(", text, flags=re.M)))
    assert declared == ["kvq_probe_read_stream"]
    out = subprocess.run(["nm", "-D", "--defined-only", build.PROBE_LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if l.split()[-2:-1] == ["T"] and "kvq_" in l.split()[-1]})
    assert exported == declared
    lib = ctypes.CDLL(build.PROBE_LIB)
    f = lib.kvq_probe_read_stream
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(None, 16, ctypes.c_void_p(256), 1, None) == 1          # null source
    assert f(ctypes.c_void_p(256), 15, ctypes.c_void_p(256), 1, None) == 1  # not a multiple of 16
    assert f(ctypes.c_void_p(264), 16, ctypes.c_void_p(256), 1, None) == 1  # misaligned
    assert f(ctypes.c_void_p(256), 16, ctypes.c_void_p(256), 0, None) == 1  # no workgroups
    assert f(ctypes.c_void_p(256), 0, ctypes.c_void_p(256), 1, None) == 0   # nothing to read: no launch


def test_window_bytes_and_host_validation(K):
    """The exact window: buffer size, and every bad window rejected on the host."""
    W = K.make_window
    assert K.kvq_window_bytes(W(4, 128, 2, FAKE), 8) == 2 * 8 * 132 * 512
    assert K.kvq_window_bytes(W(0, 0, 2, FAKE), 8) == 0
    assert K.kvq_window_bytes(W(9, 0, 1, FAKE), 1) == 0
    assert K.kvq_window_bytes(W(0, 129, 1, FAKE), 1) == 0
    assert K.kvq_window_bytes(W(1, 1, -1, FAKE), 1) == 0
    assert K.kvq_window_bytes(None, 1) == 0
    c = K.make_cache(1, 8, FAKE)
    assert _decode(K, c, window=W(9, 4, 1, FAKE)) == K.KVQ_EINVAL          # too many sinks
    assert _decode(K, c, window=W(4, 129, 1, FAKE)) == K.KVQ_EINVAL        # too many recent positions
    assert _decode(K, c, window=W(4, 4, 1, None)) == K.KVQ_EINVAL          # no buffer
    assert _decode(K, c, window=W(4, 4, 1, FAKE + 8)) == K.KVQ_EINVAL      # misaligned buffer
    assert _decode(K, c, batch=2, window=W(4, 4, 1, FAKE)) == K.KVQ_EINVAL  # holds one sequence
    # g = 16 with a window passes validation (without a GPU the call then stops at
    # its first HIP runtime query)
    assert _decode(K, c, hq=16, window=W(4, 4, 1, FAKE)) not in (K.KVQ_EINVAL, K.KVQ_EUNSUPPORTED)
    lib = K.load()
    w = W(4, 4, 2, FAKE)
    fill = lib.kvq_window_fill
    assert fill(None, 1, FAKE, FAKE, K.KVQ_BF16, 1, FAKE, FAKE, FAKE, None) == K.KVQ_EINVAL
    assert fill(ctypes.byref(w), 0, FAKE, FAKE, K.KVQ_BF16, 1, FAKE, FAKE, FAKE, None) == K.KVQ_EINVAL
    assert fill(ctypes.byref(w), 1, FAKE, FAKE, K.KVQ_BF16, -1, FAKE, FAKE, FAKE, None) == K.KVQ_EINVAL
    assert fill(ctypes.byref(w), 1, FAKE, FAKE, K.KVQ_F32_ROTATED, 1, FAKE, FAKE, FAKE, None) == K.KVQ_EUNSUPPORTED
    assert fill(ctypes.byref(w), 1, None, FAKE, K.KVQ_BF16, 1, FAKE, FAKE, FAKE, None) == K.KVQ_EINVAL
    assert fill(ctypes.byref(w), 1, FAKE, FAKE, K.KVQ_BF16, 0, FAKE, FAKE, FAKE, None) == K.KVQ_OK  # no tokens
    empty = W(0, 0, 2, None)
    assert fill(ctypes.byref(empty), 1, FAKE, FAKE, K.KVQ_BF16, 5, FAKE, FAKE, FAKE, None) == K.KVQ_OK  # no window
    bad = W(4, 4, 2, FAKE + 4)
    assert fill(ctypes.byref(bad), 1, FAKE, FAKE, K.KVQ_BF16, 5, FAKE, FAKE, FAKE, None) == K.KVQ_EINVAL


def test_cache_clip_ratio_layout_and_validation(K):
    """kvq_cache.clip_ratio sits after the pool pointer; values outside [0, 1] (or NaN)
    are rejected on the host before any launch."""
    assert ctypes.sizeof(K.kvq_cache) == 48 and K.kvq_cache.clip_ratio.offset == 32
    assert K.kvq_cache.rotation.offset == 36 and K.kvq_cache.key_bits.offset == 40
    assert K.kvq_pool_bytes(K.make_cache(2, 8, FAKE, key_bits=4)) == 2 * 8 * 2048
    assert K.kvq_pool_bytes(K.make_cache(2, 8, FAKE, key_bits=0)) == 2 * 8 * 1536
    assert _decode(K, K.make_cache(1, 8, FAKE, key_bits=5)) == K.KVQ_EUNSUPPORTED and "key_bits" in K.kvq_last_error()
    assert K.kvq_pool_bytes(K.make_cache(2, 8, FAKE, key_bits=3)) == 2 * 8 * 1792
    # 3- and 4-bit values add the values' plane (256 or 512 bytes)
    assert K.kvq_cache.val_bits.offset == 44
    assert K.kvq_pool_bytes(K.make_cache(2, 8, FAKE, val_bits=4)) == 2 * 8 * 2048
    assert K.kvq_pool_bytes(K.make_cache(2, 8, FAKE, key_bits=3, val_bits=3)) == 2 * 8 * 2048
    assert K.kvq_pool_bytes(K.make_cache(2, 8, FAKE, key_bits=4, val_bits=4)) == 2 * 8 * 2560
    assert K.kvq_pool_bytes(K.make_cache(2, 8, FAKE, key_bits=4, val_bits=2)) == 2 * 8 * 2048
    assert _decode(K, K.make_cache(1, 8, FAKE, val_bits=1)) == K.KVQ_EUNSUPPORTED and "val_bits" in K.kvq_last_error()
    assert _decode(K, K.make_cache(1, 8, FAKE, rotation=2)) == K.KVQ_EINVAL  # unknown rotation kind
    assert "rotation" in K.kvq_last_error()
    lib = K.load()
    for bad in (1.5, -0.25, float("nan")):
        c = K.make_cache(2, 4, FAKE, clip_ratio=bad)
        assert lib.kvq_quant_append(ctypes.byref(c), FAKE, FAKE, K.KVQ_BF16, 1, FAKE, None, FAKE, FAKE, None,
                                    None) == K.KVQ_EINVAL
        assert "clip_ratio" in K.kvq_last_error()
        assert _decode(K, K.make_cache(1, 8, FAKE, clip_ratio=bad)) == K.KVQ_EINVAL


def _eval(K, cache, batch=1, hq=4, max_pages=4, max_seq=64, d_model=96, ws_bytes=1 << 22, sq_err=FAKE, k=FAKE,
          w_o=FAKE, kv_dtype=None, w_dtype=None, row_offsets=FAKE):
    lib = K.load()
    kv_dtype = K.KVQ_BF16 if kv_dtype is None else kv_dtype
    w_dtype = K.KVQ_BF16 if w_dtype is None else w_dtype
    return lib.kvq_output_error(ctypes.byref(cache) if cache is not None else None, FAKE, K.KVQ_BF16, batch, hq, FAKE,
                                max_pages, FAKE, max_seq, k, FAKE, kv_dtype, row_offsets, sq_err, FAKE, FAKE, 0.0,
                                w_o, w_dtype, d_model, FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)


def test_output_error_workspace_and_validation(K):
    """The evaluator's host checks (no launch is reached): sizes, shapes, dtypes,
    alignment, the batch cap, and the append-with-errors entry point's checks."""
    ws = K.kvq_output_error_workspace_bytes
    assert ws(1, 32, 8, 131072, 4096) > 0 and ws(1, 32, 8, 131072, 4096) % 256 == 0
    assert ws(64, 32, 8, 1024, 4096) > ws(1, 32, 8, 1024, 4096)
    assert ws(65, 32, 8, 1024, 4096) == 0          # batch above 64
    assert ws(1, 34, 2, 1024, 4096) == 0           # g = 17
    assert ws(1, 3, 2, 1024, 4096) == 0            # 3 q heads over 2 KV heads
    assert ws(1, 4, 1, 1024, 0) == 0               # d_model < 1
    c = K.make_cache(1, 8, FAKE)
    assert _eval(K, None) == K.KVQ_EINVAL
    assert _eval(K, c, batch=65) == K.KVQ_EUNSUPPORTED
    assert "64" in K.kvq_last_error()
    assert _eval(K, c, hq=17) == K.KVQ_EUNSUPPORTED
    assert _eval(K, c, kv_dtype=K.KVQ_F32_ROTATED) == K.KVQ_EUNSUPPORTED
    assert _eval(K, c, w_dtype=9) == K.KVQ_EUNSUPPORTED
    assert _eval(K, c, d_model=0) == K.KVQ_EINVAL
    assert _eval(K, c, max_pages=3) == K.KVQ_EINVAL
    assert _eval(K, c, k=None) == K.KVQ_EINVAL
    assert _eval(K, c, row_offsets=None) == K.KVQ_EINVAL
    assert _eval(K, c, w_o=FAKE + 4) == K.KVQ_EINVAL and "aligned" in K.kvq_last_error()
    assert _eval(K, c, sq_err=FAKE + 8) == K.KVQ_EINVAL
    need = K.kvq_output_error_workspace_bytes(1, 4, 1, 64, 96)
    assert _eval(K, c, ws_bytes=need - 1) == K.KVQ_ENOSPACE
    assert _eval(K, c, batch=0) == K.KVQ_OK        # an empty batch is a no-op
    assert _eval(K, K.make_cache(1, 8, FAKE, rotation=3)) == K.KVQ_EINVAL
    lib = K.load()
    assert lib.kvq_quant_append_err(ctypes.byref(c), None, None, K.KVQ_BF16, 0, None, None, None, None, None, None,
                                    None) == K.KVQ_OK
    assert lib.kvq_quant_append_err(ctypes.byref(c), FAKE, FAKE, K.KVQ_BF16, -1, FAKE, None, FAKE, FAKE, None, FAKE,
                                    None) == K.KVQ_EINVAL
