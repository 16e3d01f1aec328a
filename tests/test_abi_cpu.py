"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/dense_gemm.h declares, and its argument checks, status
codes, configuration table and tile order behave as documented."""
import ctypes
import os
import re

import pytest

import dense_gemm_run_amd as dg
from dense_gemm_run_amd import _lib
from oracle import exact

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dense_gemm.h")

OK, INVALID, BADTYPE, NODEV, TOOBIG, ALIAS, HIPERR, MISMATCH = range(8)


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(_lib.LIB_PATH):
        from dense_gemm_run_amd import build
        build.build()
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 10
    L = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_header_status_codes_match_binding():
    text = open(HEADER).read()
    for name, code in _lib.STATUS_CODE.items():
        assert re.search(rf"\b{name}\s*=\s*{code}\b", text), name
    for s in range(8):
        assert dg.status_string(s) and dg.status_string(s) != "unknown status"
    assert dg.status_string(99) == "unknown status"


A, B, C = 0x10000, 0x200000, 0x4000000   # fake, never dereferenced


@pytest.mark.parametrize("args,want", [
    ((A, B, C, 4, 5, 6, 1), OK),
    ((A, B, C, -1, 5, 6, 1), INVALID),
    ((A, B, C, 4, -5, 6, 1), INVALID),
    ((A, B, C, 4, 5, -6, 1), INVALID),
    ((A, B, C, 4, 5, 6, 5), BADTYPE),
    ((A, B, C, 4, 5, 6, -1), BADTYPE),
    ((A, B, C, 4, 5, 6, 3), OK),          # 8-bit inputs, bf16 C
    ((A, B, C, 4, 5, 6, 4), OK),
    ((A, B, A + 24, 4, 5, 6, 3), OK),     # A holds 24 one-byte elements: adjacent, no overlap
    ((A, B, A + 23, 4, 5, 6, 3), ALIAS),
    ((A + 40, B, A, 4, 5, 6, 3), OK),     # C holds 20 bf16 = 40 bytes: adjacent
    ((A + 39, B, A, 4, 5, 6, 3), ALIAS),
    ((A, B, C, 1 << 16, 1 << 14, 1, 3), TOOBIG),   # C = 2^30 bf16 = 2^31 bytes
    ((A, B, C, 1 << 16, 1 << 14, 1 << 15, 3), TOOBIG),  # A = 2^31 one-byte elements
    ((A, 1 << 33, 1 << 34, 1 << 16, (1 << 14) - 1, (1 << 15) - 1, 3), OK),   # just below both limits
    ((0, B, C, 4, 5, 6, 1), INVALID),
    ((A, 0, C, 4, 5, 6, 1), INVALID),
    ((A, B, 0, 4, 5, 6, 1), INVALID),
    ((0, 0, C, 4, 5, 0, 1), OK),          # K = 0: A and B hold nothing
    ((0, B, 0, 0, 5, 6, 1), OK),          # M = 0
    ((A, 0, 0, 4, 0, 6, 1), OK),          # N = 0
    ((A, B, C, 2 ** 31, 1, 1, 1), TOOBIG),
    ((A, B, C, 1 << 16, 1 << 14, 1, 1), TOOBIG),   # C = 2^30 fp16 elements = 2^31 bytes
    ((A, B, C, (1 << 16) - 1, 1 << 14, 1, 1), OK),
    ((A, B, C, 1 << 15, 1 << 14, 1, 0), TOOBIG),   # fp32: 2^29 elements = 2^31 bytes
    ((A, B, A + 4, 4, 5, 6, 1), ALIAS),   # C starts inside A
    ((A, B, B - 10, 4, 5, 6, 1), ALIAS),  # C ends inside B
    ((A, B, A + 48, 4, 5, 6, 1), OK),     # A holds 24 fp16 = 48 bytes: adjacent, no overlap
])
def test_check_args(args, want):
    assert dg.gemm_check_args(*args) == want


def test_run_without_handle_is_rejected_before_any_launch():
    assert _lib.lib().gemm_run(None, A, B, C, 4, 5, 6, 1, None) == INVALID
    assert _lib.lib().gemm_run(None, A, B, C, 4, 5, 6, 7, None) == BADTYPE
    assert _lib.lib().gemm_run_config(None, A, B, C, 4, 5, 6, 1, 999, None) == INVALID


def test_create_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    with pytest.raises(dg.GemmError) as e:
        dg.gemm_create()
    assert e.value.status == NODEV
    assert _lib.lib().gemm_create(None) == INVALID
    assert _lib.lib().gemm_destroy(None) == OK


def test_config_table():
    n = dg.gemm_config_count()
    assert n >= 1
    names = set()
    for i in range(n):
        info = dg.gemm_config_info(i)
        assert info["id"] == i
        assert info["bm"] > 0 and info["bn"] > 0 and info["bk"] > 0 and info["group_m"] > 0
        assert info["threads"] % 64 == 0
        names.add(info["name"])
    assert len(names) == n
    assert dg.gemm_config_info(0)["dtype_mask"] == 0x1f and dg.gemm_config_info(0)["needs_vec_align"] == 0
    with pytest.raises(dg.GemmError):
        dg.gemm_config_info(n)


def test_selection_rules():
    # the generic configuration takes anything small (16-bit), ragged or
    # unaligned; aligned fp32 rows run the fp32 MFMA kernel at any size
    assert dg.gemm_select_config(A, B, C, 64, 64, 64, 1) == 0
    assert dg.gemm_config_info(dg.gemm_select_config(A, B, C, 64, 64, 64, 0))["name"] == "fp32_64x64x32"
    assert dg.gemm_select_config(A, B, C, 127, 255, 65, 1) == 0
    assert dg.gemm_select_config(A + 2, B, C, 4096, 4096, 4096, 1) == 0   # misaligned A
    assert dg.gemm_select_config(A, B, C, 4096, 4096, 4094, 1) in (0,)   # K not a multiple of 8
    assert dg.gemm_select_config(A, B, C, -1, 4, 4, 1) == -1
    for M, N, K, dt in [(4096, 4096, 4096, 1), (8192, 8192, 8192, 2), (8192, 12288, 4096, 2),
                        (8192, 4096, 14336, 2), (1000, 1000, 1000, 1)]:
        Cb = C + (1 << 32)
        cid = dg.gemm_select_config(A, A + (M * K * 2 + 4096) // 16 * 16, Cb, M, N, K, dt)
        assert 0 <= cid < dg.gemm_config_count()
        info = dg.gemm_config_info(cid)
        assert (info["dtype_mask"] >> dt) & 1


@pytest.mark.parametrize("cid", range(64))
def test_tile_order_is_a_bijection(cid):
    if cid >= dg.gemm_config_count():
        pytest.skip("no such configuration")
    info = dg.gemm_config_info(cid)
    for M, N in [(1, 1), (127, 255), (4096, 4096), (8192, 12288), (300, 5000), (8192, 4096)]:
        tm_n = -(-M // info["bm"])
        tn_n = -(-N // info["bn"])
        total = tm_n * tn_n
        if total > 2000:
            continue
        seen = [dg.gemm_tile_of_block(cid, M, N, b) for b in range(total)]
        assert sorted(seen) == [(r, c) for r in range(tm_n) for c in range(tn_n)]
        if not info["xcd_remap"]:
            # without the XCD remap the order is exactly the pages' grouped order
            assert seen == [exact.grouped_tile(b, tm_n, tn_n, info["group_m"]) for b in range(total)]
        with pytest.raises(dg.GemmError):
            dg.gemm_tile_of_block(cid, M, N, total)


def test_xcd_remap_gives_each_xcd_a_compact_block():
    remapped = [i for i in range(dg.gemm_config_count()) if dg.gemm_config_info(i)["xcd_remap"]]
    if not remapped:
        pytest.skip("no configuration remaps workgroups")
    cid = remapped[0]
    info = dg.gemm_config_info(cid)
    M = N = 16 * info["bm"] if info["bm"] == info["bn"] else 4096
    tm_n, tn_n = -(-M // info["bm"]), -(-N // info["bn"])
    total = tm_n * tn_n
    for x in range(8):
        tiles = [dg.gemm_tile_of_block(cid, M, N, b) for b in range(x, total, 8)]
        rows = {t[0] for t in tiles}
        cols = {t[1] for t in tiles}
        # a compact block touches far fewer rows+columns than a scattered one
        assert len(rows) * len(cols) <= 2 * len(tiles), (x, len(rows), len(cols))


# ---------------------------------------------------------------- batched
@pytest.mark.parametrize("args,want", [
    # (A, B, C, batch, M, N, K, sa, sb, sc, dtype)
    ((A, B, C, 3, 4, 5, 6, 24, 30, 20, 1), OK),
    ((A, B, C, 0, 4, 5, 6, 24, 30, 20, 1), OK),            # empty batch
    ((0, 0, 0, 0, 4, 5, 6, 24, 30, 20, 1), OK),            # ... with no data at all
    ((A, B, C, 3, 4, 5, 6, 0, 0, 20, 1), OK),              # A and B shared by every product
    ((A, B, C, -1, 4, 5, 6, 24, 30, 20, 1), INVALID),
    ((A, B, C, 3, 4, 5, 6, -24, 30, 20, 1), INVALID),
    ((A, B, C, 3, 4, 5, 6, 24, 30, -20, 1), INVALID),
    ((A, B, C, 3, 4, 5, 6, 24, 30, 20, 5), BADTYPE),
    ((0, B, C, 3, 4, 5, 6, 24, 30, 20, 1), INVALID),
    ((A, B, C, 3, 4, 5, 6, 24, 30, 19, 1), ALIAS),         # C matrices overlap each other
    ((A, B, C, 1, 4, 5, 6, 24, 30, 0, 1), OK),             # ... unless there is one
    ((A, B, A + 2 * 48, 3, 4, 5, 6, 48, 30, 20, 1), ALIAS),  # C inside A's span, between matrices
    ((A, B, C, 2 ** 31, 4, 5, 6, 24, 30, 20, 1), TOOBIG),
    ((A, B, C, 2, 1 << 16, 1 << 14, 1, 0, 0, 1 << 30, 1), TOOBIG),   # one C matrix of 2^31 bytes
    ((A, B, C, 3, 4, 5, 6, 1 << 62, 30, 20, 1), TOOBIG),   # A's span overflows
    ((A, B, C, 1 << 20, 4096, 4096, 8, 0, 0, 1 << 24, 1), TOOBIG),   # grid of 2^32 workgroups
    # batched matrix-vector products (4 rows of A per 256-lane workgroup):
    # 1024 workgroups per product, so 16383 products are 2^32 - 2^18 lanes
    # and 16384 are 2^32, one more than a grid holds
    ((A, B, C, 16383, 4096, 1, 4096, 0, 0, 4096, 1), OK),
    ((A, B, C, 16384, 4096, 1, 4096, 0, 0, 4096, 1), TOOBIG),
])
def test_check_args_batched(args, want):
    assert dg.gemm_check_args_batched(*args) == want


def test_grid_limit_is_checked_before_the_handle():
    """A batched matrix-vector product whose grid would exceed 2^32-1 lanes
    is refused as too large by gemm_run_batched itself, before anything
    else (here: the missing handle) is looked at; one product fewer reaches
    the handle check."""
    assert dg.gemm_select_config_batched(A, B, C, 16384, 4096, 1, 4096, 0, 0, 4096, 1) == 34
    info = dg.gemm_config_info(34)
    assert (info["bm"], info["threads"]) == (4, 256)
    L = _lib.lib()
    assert L.gemm_run_batched(None, A, B, C, 16384, 4096, 1, 4096, 0, 0, 4096, 1, None) == TOOBIG
    assert L.gemm_run_batched(None, A, B, C, 16383, 4096, 1, 4096, 0, 0, 4096, 1, None) == INVALID
    # a batch of 2^21 products would wrap a 32-bit workgroup count
    assert L.gemm_run_batched(None, A, B, C, 1 << 21, 4096, 1, 4096, 0, 0, 4096, 1, None) == TOOBIG
    # forced configurations: the grid of the configuration that was asked for
    assert L.gemm_run_batched_config(None, A, B, C, 16384, 4096, 1, 4096, 0, 0, 4096, 1, 34, None) == TOOBIG


def test_single_calls_are_the_batch_of_one():
    for args in [(A, B, C, 4, 5, 6, 1), (A, B, A + 4, 4, 5, 6, 1), (0, B, C, 4, 5, 6, 1),
                 (A, B, C, 4096, 4096, 4096, 1)]:
        a, b, c, M, N, K, dt = args
        assert dg.gemm_check_args(*args) == dg.gemm_check_args_batched(a, b, c, 1, M, N, K,
                                                                       M * K, K * N, M * N, dt)
    Cb = C + (1 << 32)
    for M, N, K, dt in [(4096, 4096, 4096, 1), (1000, 1000, 1000, 1), (64, 64, 64, 0)]:
        Bb = A + (M * K * 2 + 4096) // 16 * 16
        assert dg.gemm_select_config(A, Bb, Cb, M, N, K, dt) == dg.gemm_select_config_batched(
            A, Bb, Cb, 1, M, N, K, M * K, K * N, M * N, dt)
    for cid in (0, 6):
        for b in range(0, 64, 7):
            assert dg.gemm_tile_of_block(cid, 4096, 2048, b) == \
                dg.gemm_tile_of_block_batched(cid, 4096, 2048, 1, b)[1:]


def test_batched_selection_counts_the_whole_batch():
    Cb = C + (1 << 34)
    M = N = K = 2048          # 64 tiles of 256 x 256: too few alone, enough 16 at a time
    Bb = A + (1 << 33)
    alone = dg.gemm_select_config_batched(A, Bb, Cb, 1, M, N, K, M * K, K * N, M * N, 2)
    many = dg.gemm_select_config_batched(A, Bb, Cb, 16, M, N, K, M * K, K * N, M * N, 2)
    assert dg.gemm_config_info(alone)["bm"] * dg.gemm_config_info(alone)["bn"] < 256 * 256
    assert (dg.gemm_config_info(many)["bm"], dg.gemm_config_info(many)["bn"]) == (256, 256)
    # strides that break 16-byte alignment rule out the vector-load kernels
    odd = dg.gemm_select_config_batched(A, Bb, Cb, 16, M, N, K, M * K + 1, K * N, M * N, 2)
    assert dg.gemm_config_info(odd)["needs_vec_align"] == 0


@pytest.mark.parametrize("cid", [0, 2, 6, 9, 48])
def test_batched_tile_order_is_a_bijection(cid):
    info = dg.gemm_config_info(cid)
    for M, N, batch in [(300, 700, 3), (1024, 1024, 8), (100, 100, 17)]:
        tm_n, tn_n = -(-M // info["bm"]), -(-N // info["bn"])
        total = tm_n * tn_n * batch
        seen = [dg.gemm_tile_of_block_batched(cid, M, N, batch, b) for b in range(total)]
        assert sorted(seen) == [(i, r, c) for i in range(batch) for r in range(tm_n)
                                for c in range(tn_n)]
        with pytest.raises(dg.GemmError):
            dg.gemm_tile_of_block_batched(cid, M, N, batch, total)


def test_few_columns_select_the_vector_kernel():
    Cb = C + (1 << 34)
    Bb = A + (1 << 33)
    for M, N, K in [(14336, 1, 4096), (4096, 1, 14336), (12288, 4, 4096), (1, 1, 8), (300, 3, 1040)]:
        cid = dg.gemm_select_config(A, Bb, Cb, M, N, K, 2)
        info = dg.gemm_config_info(cid)
        assert info["name"].startswith("gemv") and N <= info["bn"], (M, N, K, info["name"])
    # five columns, K not a multiple of 8, a misaligned B, or fp32: not the vector kernel
    for args in [(A, Bb, Cb, 4096, 5, 4096, 2), (A, Bb, Cb, 4096, 1, 4090, 2),
                 (A, Bb + 2, Cb, 4096, 1, 4096, 2), (A, Bb, Cb, 4096, 1, 4096, 0)]:
        assert not dg.gemm_config_info(dg.gemm_select_config(*args))["name"].startswith("gemv")
    # C needs no alignment for it
    assert dg.gemm_config_info(dg.gemm_select_config(A, Bb, Cb + 2, 4096, 1, 4096, 2))["name"].startswith("gemv")


def test_8bit_inputs_select_their_kernels():
    Cb = C + (1 << 34)
    Bb = A + (1 << 33)
    fp8_cfgs = [i for i in range(dg.gemm_config_count())
                if dg.gemm_config_info(i)["dtype_mask"] == 0x18]
    assert len(fp8_cfgs) >= 1
    for dt in (3, 4):
        for M, N, K in [(4096, 4096, 4096), (8192, 8192, 8192), (1000, 1008, 1024)]:
            cid = dg.gemm_select_config(A, Bb, Cb, M, N, K, dt)
            assert cid in fp8_cfgs, (M, N, K, dt, cid)
        # rows of A or B not whole 16-byte pieces, a misaligned pointer, or a
        # small product: the generic kernel (which widens to bf16)
        for args in [(A, Bb, Cb, 4096, 4096, 4088, dt), (A, Bb, Cb, 4096, 4088, 4096, dt),
                     (A + 8, Bb, Cb, 4096, 4096, 4096, dt), (A, Bb, Cb + 8, 4096, 4096, 4096, dt),
                     (A, Bb, Cb, 64, 64, 64, dt), (A, Bb, Cb, 4096, 1, 4096, dt)]:
            assert dg.gemm_select_config(*args) == 0, args
    # the 16-bit kernels refuse 8-bit inputs and the 8-bit ones refuse the rest
    for i in range(dg.gemm_config_count()):
        m = dg.gemm_config_info(i)["dtype_mask"]
        assert i == 0 or (m & 0x18) == 0 or (m & 0x7) == 0
    # batch strides: in one-byte elements for A and B, bf16 elements for C
    assert dg.gemm_select_config_batched(A, Bb, Cb, 4, 1024, 1024, 1024, 1024 * 1024,
                                         1024 * 1024, 1024 * 1024, 3) in fp8_cfgs
    assert dg.gemm_select_config_batched(A, Bb, Cb, 4, 1024, 1024, 1024, 1024 * 1024 + 8,
                                         1024 * 1024, 1024 * 1024, 3) == 0
    assert dg.gemm_select_config_batched(A, Bb, Cb, 4, 1024, 1024, 1024, 1024 * 1024,
                                         1024 * 1024, 1024 * 1024 + 8, 3) in fp8_cfgs


def test_few_rows_select_the_few_row_kernels():
    Cb = C + (1 << 34)
    Bb = A + (1 << 33)
    name = lambda *args: dg.gemm_config_info(dg.gemm_select_config(*args))["name"]
    # 16-bit: the one-launch few-row kernel (8-, 16-, 32- and 64-row
    # workgroups) in configurations that fit one wave of 256 workgroups, the
    # 64 x 128 tiles where none does, the strip kernel for wide B with short K
    expect16 = {(16, 4096, 4096): "fewrow_16x16x64", (1, 4096, 4096): "fewrow_8x16x64",
                (8, 4096, 14336): "fewrow_8x16x64", (9, 4096, 4096): "fewrow_16x16x64",
                (16, 4096, 14336): "fewrow_16x16x64", (16, 4096, 2048): "fewrow_16x32x32",
                (16, 2048, 2048): "fewrow_16x16x32", (1, 3072, 3072): "fewrow_16x16x32",
                (32, 4096, 4096): "fewrow_16x32x32",
                (24, 4096, 4096): "fewrow_16x32x32", (16, 8192, 4096): "fewrow_16x32x32",
                (16, 14336, 4096): "mfma16x16_64x128x32_adma", (32, 14336, 4096): "mfma16x16_64x128x32_adma",
                (16, 14336, 512): "skinny_16x32x64", (16, 65536, 4096): "fewrow_16x32x32",
                (16, 32768, 4096): "mfma16x16_64x128x32_adma", (32, 8192, 4096): "fewrow_32x32x32",
                (48, 4096, 4096): "fewrow_32x32x32", (64, 4096, 4096): "fewrow_32x32x32",
                (64, 8192, 4096): "fewrow_64x32x32", (96, 4096, 4096): "fewrow_64x32x32",
                (128, 4096, 4096): "fewrow_64x32x32", (128, 4096, 14336): "fewrow_64x32x32",
                # one wave: 192 strips of 32 columns rather than 384 of 16, and so on
                (1, 6144, 4096): "fewrow_16x32x32", (16, 6144, 4096): "fewrow_16x32x32",
                (24, 6144, 4096): "fewrow_32x32x32", (40, 6144, 4096): "fewrow_64x32x32",
                (96, 6144, 4096): "mfma16x16_64x128x32_adma", (24, 11008, 4096): "mfma16x16_64x128x32_adma",
                (1, 11008, 4096): "fewrow_16x32x32", (16, 11008, 4096): "mfma16x16_64x128x32_adma",
                (24, 2048, 8192): "fewrow_16x16x64", (40, 2048, 8192): "fewrow_32x16x32",
                (40, 2048, 2048): "fewrow_16x32x32"}
    for (M, N, K), want in expect16.items():
        for dt in (1, 2):
            assert name(A, Bb, Cb, M, N, K, dt) == want, (M, N, K, dt)
    # wide B from 33 rows up, many rows, fp32, unaligned rows: none of them
    for args in [(A, Bb, Cb, 64, 14336, 4096, 2), (A, Bb, Cb, 256, 4096, 4096, 2),
                 (A, Bb, Cb, 16, 4096, 4096, 0), (A, Bb, Cb, 16, 4096, 4092, 2)]:
        n = name(*args)
        assert not n.startswith("skinny") and not n.startswith("fewrow"), args
    # 8-bit: the 8-bit few-row configurations where one fits one wave
    expect8 = {(1, 4096, 4096): "fewrow8_8x32x128", (8, 1024, 8192): "fewrow8_8x32x128",
               (8, 4096, 14336): "fewrow8_16x16x128", (16, 4096, 4096): "fewrow8_16x32x128",
               (32, 4096, 4096): "fewrow8_32x32x128", (16, 8192, 4096): "fewrow8_16x32x128",
               (16, 4096, 14336): "fewrow8_16x16x128", (16, 4096, 8192): "fewrow8_16x16x128",
               (64, 4096, 4096): "fewrow8_32x32x128", (24, 4096, 14336): "fewrow8_16x32x128",
               (96, 4096, 4096): "fp8_64x128x64_adma", (16, 14336, 4096): "fp8_64x128x64_adma",
               (4, 11008, 4096): "fp8_64x128x64_adma", (96, 2048, 4096): "fewrow8_32x32x128",
               (40, 6144, 4096): "fp8_64x128x64_adma", (16, 8192, 8192): "fewrow8_16x32x128",
               (1, 3072, 8192): "fewrow8_16x16x128", (24, 1024, 4096): "fewrow8_16x32x128",
               (40, 2048, 8192): "fewrow8_32x32x128", (40, 2048, 2048): "fewrow8_16x32x128"}
    for (M, N, K), want in expect8.items():
        for dt in (3, 4):
            assert name(A, Bb, Cb, M, N, K, dt) == want, (M, N, K, dt)
    for M, N, K in [(128, 4096, 4096), (16, 4096, 4088)]:
        n = name(A, Bb, Cb, M, N, K, 3)
        assert not n.startswith("skinny") and not n.startswith("fewrow"), (M, N, K)


def test_few_row_picks_fit_one_wave():
    """Over a grid of 1-128 rows, the few-row kernel is picked in a shape
    whose workgroups fit one wave of 256 (one per CU) whenever one of its
    shapes does; more only up to 8 rows (16-bit, at most 384 strips of 32
    columns) and up to 32 rows where the 64 x 128 tiles do not fit one wave
    either."""
    Cb = C + (1 << 34)
    Bb = A + (1 << 33)
    cd = lambda a, b: -(-a // b)
    fewrow = {c: dg.gemm_config_info(c) for c in range(dg.gemm_config_count())
              if dg.gemm_config_info(c)["name"].startswith("fewrow")}
    for dt in (2, 3):
        eight = dt == 3
        shapes_ok = [c for c, i in fewrow.items() if (i["dtype_mask"] == 0x18) == eight]
        for M in (1, 5, 8, 9, 16, 17, 24, 32, 33, 48, 64, 65, 96, 128):
            for N in (512, 1024, 2048, 3072, 4096, 5120, 6144, 8192, 11008, 12288, 14336, 28672):
                for K in (1024, 2048, 4096, 8192, 14336):
                    cid = dg.gemm_select_config(A, Bb, Cb, M, N, K, dt)
                    fits = [c for c in shapes_ok
                            if cd(M, fewrow[c]["bm"]) * cd(N, fewrow[c]["bn"]) <= 256]
                    if cid in fewrow:
                        wgs = cd(M, fewrow[cid]["bm"]) * cd(N, fewrow[cid]["bn"])
                        assert (wgs <= 256 or (not eight and M <= 8 and wgs <= 384)
                                or (not fits and M <= 32 and cd(N, 128) > 256)), (M, N, K, dt, wgs)
                    elif fits:
                        # a one-wave few-row shape exists: only the generic kernel
                        # (tiny products) may take its place
                        assert cid == 0 and M * N * K < 128 ** 3, (M, N, K, dt, cid)


def test_192_row_tiles_where_256_leaves_a_partial_wave():
    Cb = C + (1 << 34)
    Bb = A + (1 << 33)
    name = lambda *args: dg.gemm_config_info(dg.gemm_select_config(*args))["name"]
    # 144 tiles of 256 x 256 -> one wave of 192 x 256; 576 (2.25 waves) -> 768 (3 whole waves)
    for M, N, K in [(3072, 3072, 3072), (6144, 6144, 6144)]:
        for dt in (1, 2):
            assert name(A, Bb, Cb, M, N, K, dt) == "mfma16x16_192x256x32_apair", (M, N, K)
    # whole waves of 256 x 256 tiles keep them
    for M, N, K in [(4096, 4096, 4096), (8192, 8192, 8192), (8192, 12288, 4096), (8192, 14336, 4096),
                    (5120, 5120, 5120)]:
        assert name(A, Bb, Cb, M, N, K, 2) == "mfma16x16_256x256x32_apair", (M, N, K)
    # operands beyond the 256 MB Infinity Cache: A direct to LDS as well
    assert name(A, Bb, Cb, 8192, 4096, 14336, 2) == "mfma16x16_256x256x32_apair"
    assert name(A, Bb, Cb, 12288, 12288, 12288, 2) == "mfma16x16_256x256x32_apair"
    assert name(A, Bb, Cb, 6144, 6144, 16384, 2) == "mfma16x16_192x256x32_apair"
    # fewer than 128 tiles: 128 x 128, A direct to LDS
    assert name(A, Bb, Cb, 2048, 2048, 2048, 1) == "mfma16x16_128x128x32_adma"
    info = dg.gemm_config_info(28)
    assert (info["bm"], info["bn"], info["bk"]) == (192, 256, 32)


def test_8bit_tile_size_follows_the_tile_count():
    Cb = C + (1 << 34)
    Bb = A + (1 << 33)
    name = lambda *args: dg.gemm_config_info(dg.gemm_select_config(*args))["name"]
    # fewer than 128 tiles of 256 x 256 (half the CUs): 64 x 128 tiles while they fit one
    # wave, else 128 x 128
    for M, N, K in [(512, 4096, 4096), (128, 4096, 4096), (64, 14336, 4096), (1024, 1024, 1024)]:
        assert name(A, Bb, Cb, M, N, K, 3) == "fp8_64x128x64_adma", (M, N, K)
    for M, N, K in [(2048, 2048, 2048), (1536, 1536, 1536), (2816, 2816, 1024)]:
        assert name(A, Bb, Cb, M, N, K, 3).startswith("fp8_128x128"), (M, N, K)
    for M, N, K in [(4096, 4096, 4096), (8192, 14336, 4096), (8192, 8192, 8192)]:
        assert name(A, Bb, Cb, M, N, K, 4).startswith("fp8_256x256"), (M, N, K)
    # a partial last wave of 256 x 256 tiles that 192 x 256 tiles fill: 3072^2, 6144^2
    for n in (3072, 6144):
        assert name(A, Bb, Cb, n, n, n, 3) == "fp8_192x256x128_k128", n
    # the 128-deep kernel from 128 tiles of 256 x 256 on (a partial single wave included,
    # where 192 x 256 tiles do not fill it better)
    assert name(A, Bb, Cb, 4096, 4096, 4096, 3) == "fp8_256x256x128_k128"
    for M, N, K in [(2048, 6144, 4096), (1024, 14336, 4096)]:
        assert name(A, Bb, Cb, M, N, K, 3) == "fp8_256x256x128_k128", (M, N, K)
    assert name(A, Bb, Cb, 2048, 2048, 2048, 3) == "fp8_128x128x64_adma"
    # the batch counts: 16 products of 1024^2 are 256 tiles of 256 x 256
    cid = dg.gemm_select_config_batched(A, Bb, Cb, 16, 1024, 1024, 1024, 1024 * 1024, 1024 * 1024,
                                        1024 * 1024, 3)
    assert dg.gemm_config_info(cid)["name"].startswith("fp8_256x256")


# ---------------------------------------------------------------- split K with a workspace
def test_workspace_sizes_follow_the_split_rule():
    L = _lib.lib()
    # up to 256 rows the tiles are 64 x 128: 256 x 4096 is 128 of them -> 2 splits
    assert L.gemm_workspace_size(256, 4096, 4096, 2) == 2 * 256 * 4096 * 4
    # 128 x 4096: 64 tiles -> 4 splits; 64 x 14336: 112 tiles -> 2 splits
    assert L.gemm_workspace_size(128, 4096, 4096, 2) == 4 * 128 * 4096 * 4
    assert L.gemm_workspace_size(64, 14336, 4096, 1) == 2 * 64 * 14336 * 4
    # 16 rows: 32 tiles -> 8 splits; 512 x 4096 is 256 tiles, one wave: no split;
    # 1024 x 1024 x 16384: 128 tiles -> 2 splits of 256 K-steps
    assert L.gemm_workspace_size(16, 4096, 4096, 2) == 8 * 16 * 4096 * 4
    assert L.gemm_workspace_size(512, 4096, 4096, 2) == 0
    assert L.gemm_workspace_size(1024, 1024, 16384, 2) == 2 * 1024 * 1024 * 4
    # 8-bit inputs up to 128 rows: 64 x 4096 x 8192 -> 8 splits of 16 K-steps of 64; K = 14336 -> 8
    assert L.gemm_workspace_size(64, 4096, 8192, 3) == 8 * 64 * 4096 * 4
    assert L.gemm_workspace_size(16, 4096, 14336, 4) == 8 * 16 * 4096 * 4
    assert L.gemm_workspace_size(16, 14336, 4096, 3) == 2 * 16 * 14336 * 4
    # 8-bit tiles are 64 x 128: up to 64 rows each split keeps at least 16 K-steps
    # (32 x 8192 x 4096: 4 splits), beyond that 32: 128 x 4096 x 4096 -> 2
    assert L.gemm_workspace_size(32, 8192, 4096, 3) == 4 * 32 * 8192 * 4
    assert L.gemm_workspace_size(128, 4096, 4096, 3) == 2 * 128 * 4096 * 4
    # 1 to 8 rows split too (8 splits of the 32 tiles of 64 x 128)
    assert L.gemm_workspace_size(8, 4096, 4096, 2) == 8 * 8 * 4096 * 4
    assert L.gemm_workspace_size(1, 4096, 4096, 1) == 8 * 1 * 4096 * 4
    # where the one-launch few-row kernel is faster: no split (16-bit K <= 2048, or
    # K <= 4096 with N <= 2048; 8-bit up to 64 rows with K and N <= 4096)
    for args in [(16, 2048, 2048, 2), (16, 4096, 2048, 1), (16, 2048, 4096, 2), (8, 2048, 2048, 2),
                 (16, 4096, 4096, 3), (1, 2048, 4096, 4), (16, 3072, 3072, 3), (24, 4096, 4096, 3),
                 (64, 4096, 4096, 3)]:
        assert L.gemm_workspace_size(*args) == 0, args
    assert L.gemm_workspace_size(16, 3072, 3072, 2) > 0
    assert L.gemm_workspace_size(96, 4096, 4096, 3) > 0
    # enough tiles, GEMV, fp32, K < 2048, K = 0, and 8-bit inputs beyond 128 rows: no split
    for args in [(4096, 4096, 4096, 1), (2048, 2048, 2048, 2), (256, 14336, 4096, 2),
                 (4096, 4, 4096, 2), (256, 4096, 4096, 0), (256, 4096, 4096, 3),
                 (129, 4096, 4096, 3), (64, 4096, 1024, 4),
                 (1024, 1024, 1024, 2), (256, 4096, 2016, 2), (256, 4096, 0, 2), (0, 4096, 4096, 2),
                 (256, 4096, 4092, 2)]:
        assert L.gemm_workspace_size(*args) == 0, args
    # the split count never leaves a split without K-steps, and each has >= 16 of them
    for M, N, K in [(128, 1024, 4096), (256, 512, 8192), (256, 4096, 2048), (100, 200, 30000)]:
        ws = L.gemm_workspace_size(M, N, K, 2)
        s = ws // (M * N * 4)
        assert ws == 0 or (2 <= s <= 16 and -(-K // 32) >= 16 * s), (M, N, K, s)
    assert L.gemm_workspace_size(-1, 4, 4, 2) == -1
    assert L.gemm_workspace_size(4, 4, 4, 9) == -1


def test_select_config_ws_falls_back_when_the_workspace_is_short():
    need = dg.gemm_workspace_size(256, 4096, 4096, 2)
    cid, s = dg.gemm_select_config_ws(A, A + (1 << 30), A + (1 << 31), 256, 4096, 4096, 2, need)
    assert dg.gemm_config_info(cid)["name"] == "mfma16x16_64x128x32_adma" and s == 2
    # one wave of 64 x 128 tiles: one pass on them
    cid, s = dg.gemm_select_config_ws(A, A + (1 << 30), A + (1 << 31), 512, 4096, 4096, 2, 1 << 40)
    assert dg.gemm_config_info(cid)["name"] == "mfma16x16_64x128x32_adma" and s == 1
    cid, s = dg.gemm_select_config_ws(A, A + (1 << 30), A + (1 << 31), 256, 4096, 4096, 2, need - 1)
    assert s == 1 and cid == dg.gemm_select_config(A, A + (1 << 30), A + (1 << 31), 256, 4096, 4096, 2)
    # misaligned A: the generic kernel, no split
    cid, s = dg.gemm_select_config_ws(A + 2, A + (1 << 30), A + (1 << 31), 256, 4096, 4096, 2, need)
    assert (cid, s) == (0, 1)
    assert dg.gemm_select_config_ws(A, B, C, -1, 4, 4, 2, need)[0] == -1


def test_workspace_argument_errors():
    L = _lib.lib()
    M, N, K = 256, 4096, 4096
    Bb, Cb = A + (1 << 30), A + (1 << 31)
    W = A + (1 << 33)
    need = 4 * M * N * 4
    run = lambda *a: L.gemm_run_ws(None, A, Bb, Cb, M, N, K, 2, *a, None)
    assert run(W, -1) == INVALID
    assert run(None, 64) == INVALID
    assert run(W + 8, need) == INVALID                 # not 16-byte aligned
    assert run(Cb + 1024, need) == ALIAS               # overlaps C
    assert run(A, need) == ALIAS                       # overlaps A
    assert run(W, need) == INVALID                     # valid arguments, but no handle
    cfg = lambda cid, s, w, nb: L.gemm_run_ws_config(None, A, Bb, Cb, M, N, K, 2, cid, s, w, nb, None)
    assert cfg(12, 0, W, need) == INVALID
    assert cfg(12, 65, W, need) == INVALID
    assert cfg(0, 2, W, need) == MISMATCH               # the generic kernel does not split
    assert cfg(15, 2, W, need) == MISMATCH              # nor does the strip kernel
    assert cfg(22, 2, W, need) == MISMATCH              # nor the 8-bit strip kernel
    assert cfg(12, 4, W, need - 1) == INVALID           # workspace too small for 4 splits
    assert cfg(12, 4, W, need) == INVALID               # valid, but no handle
    assert cfg(99, 2, W, need) == INVALID


def test_short_k_selects_128x128_tiles_with_a_through_registers():
    Cb = C + (1 << 34)
    Bb = A + (1 << 33)
    name = lambda *args: dg.gemm_config_info(dg.gemm_select_config(*args))["name"]
    # at most 8 K-steps of 32 (16-bit) or 4 of 64 (8-bit); 16-bit products
    # with K <= 128 over at least 1024 tiles of 128 x 128 take the persistent
    # short-K kernel
    for M, N, K in [(8192, 8192, 64), (4096, 4096, 128), (8192, 8192, 8)]:
        for dt in (1, 2):
            assert name(A, Bb, Cb, M, N, K, dt) == "shortk_128x128x128", (M, N, K, dt)
    for M, N, K in [(8192, 8192, 136), (8192, 8192, 256), (2048, 2048, 208), (2048, 2048, 128),
                    (4096, 3968, 128)]:
        for dt in (1, 2):
            assert name(A, Bb, Cb, M, N, K, dt) == "mfma16x16_128x128x32", (M, N, K, dt)
    for M, N, K in [(8192, 8192, 64), (8192, 8192, 256), (4096, 4096, 128), (2048, 2048, 208)]:
        for dt in (3, 4):
            assert name(A, Bb, Cb, M, N, K, dt) == "fp8_128x128x64", (M, N, K, dt)
    cid = dg.gemm_select_config_batched(A, Bb, Cb, 64, 2048, 2048, 128, 2048 * 128, 128 * 2048,
                                        2048 * 2048, 2)
    assert dg.gemm_config_info(cid)["name"] == "shortk_128x128x128"
    cid = dg.gemm_select_config_batched(A, Bb, Cb, 3, 2048, 2048, 128, 2048 * 128, 128 * 2048,
                                        2048 * 2048, 2)
    assert dg.gemm_config_info(cid)["name"] == "mfma16x16_128x128x32"   # 768 tiles
    info = dg.gemm_config_info(48)
    assert (info["bm"], info["bn"], info["bk"], info["dtype_mask"], info["threads"]) == (128, 128, 128, 6, 256)
    # from K = 264 on, the tile-count rules again
    assert name(A, Bb, Cb, 8192, 8192, 264, 2) == "mfma16x16_256x256x32_apair"
    assert name(A, Bb, Cb, 8192, 8192, 512, 3) == "fp8_256x256x128_k128"
    # few rows keep the few-row kernels, few columns the vector kernel
    assert name(A, Bb, Cb, 16, 4096, 128, 2).startswith("fewrow")
    assert name(A, Bb, Cb, 16, 4096, 128, 3).startswith("fewrow8")
    assert name(A, Bb, Cb, 4096, 1, 128, 2).startswith("gemv")


def test_wide_few_rows_select_64x128_tiles_while_they_fit_one_wave():
    Cb = C + (1 << 34)
    Bb = A + (1 << 33)
    name = lambda *args: dg.gemm_config_info(dg.gemm_select_config(*args))["name"]
    for M, N, K in [(40, 14336, 4096), (128, 14336, 4096), (96, 8192, 4096), (128, 8192, 8192)]:
        for dt in (1, 2):
            assert name(A, Bb, Cb, M, N, K, dt) == "mfma16x16_64x128x32_adma", (M, N, K, dt)
    # 448 tiles of 64 x 128: back to 128 x 128; up to 32 rows of a wide B the
    # 64 x 128 tiles from K = 1024, the strip kernel below
    assert name(A, Bb, Cb, 128, 28672, 4096, 2) == "mfma16x16_128x128x32_adma"
    # beyond one wave of 128 x 128 tiles: A staged two K-steps at a time
    for M, N, K in [(2560, 2560, 2048), (2304, 2304, 4096), (2816, 2816, 1024)]:
        assert name(A, Bb, Cb, M, N, K, 2) == "mfma16x16_128x128x32_apair", (M, N, K)
    # a partial single wave of 256 x 256 tiles that at most 512 tiles of 128 x 128 cover
    for M, N, K in [(2048, 4096, 4096), (1024, 8192, 4096), (4096, 2048, 8192)]:
        assert name(A, Bb, Cb, M, N, K, 2) == "mfma16x16_128x128x32_apair", (M, N, K)
    assert name(A, Bb, Cb, 32, 14336, 4096, 2) == "mfma16x16_64x128x32_adma"
    assert name(A, Bb, Cb, 32, 14336, 512, 2).startswith("skinny")


def test_few_tiles_select_64x128_tiles_while_they_fit_one_wave():
    Cb = C + (1 << 34)
    Bb = A + (1 << 33)
    name = lambda *args: dg.gemm_config_info(dg.gemm_select_config(*args))["name"]
    for n in (512, 768, 1024):
        assert name(A, Bb, Cb, n, n, n, 2) == "mfma16x16_64x128x32_adma", n
    assert name(A, Bb, Cb, 512, 4096, 4096, 1) == "mfma16x16_64x128x32_adma"
    # 288 and 512 tiles of 64 x 128: 128 x 128
    for n in (1536, 2048):
        assert name(A, Bb, Cb, n, n, n, 2) == "mfma16x16_128x128x32_adma", n


def test_noalloc_entry_point_host_checks():
    """gemm_run_noalloc's host side: the scratch size in the header and the
    binding agree, every split the selection makes fits it (so its
    too-large refusal is a guard, not a case the split rule reaches), and
    argument errors come before any device work."""
    text = open(HEADER).read()
    m = re.search(r"#define GEMM_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES
    most = 0
    for dtype in (1, 2, 3, 4):
        for M in list(range(1, 130)) + [200, 256, 300, 512]:
            for N in (8, 128, 1000, 4096, 10240, 14336, 20480, 28672):
                for K in (2048, 4096, 14336, 65536):
                    most = max(most, dg.gemm_workspace_size(M, N, K, dtype))
    assert 0 < most <= _lib.NOALLOC_SCRATCH_BYTES, most
    L = _lib.lib()
    assert L.gemm_run_noalloc(None, A, B, C, 16, 4096, 4096, 2, None) == INVALID
    assert L.gemm_run_noalloc(None, A, B, C, 16, 4096, 4096, 9, None) == BADTYPE
    assert L.gemm_run_noalloc(None, A, B, A + 8, 16, 4096, 4096, 2, None) == ALIAS


def test_fp32_selects_the_mfma_kernel_for_aligned_rows():
    """fp32 products with 16-byte rows (K and N multiples of 4) run the fp32
    MFMA kernel, on 128 x 128 tiles from 1024 of them and on 64 x 64 tiles
    below; ragged or misaligned ones the generic kernel."""
    Cb = C + (1 << 34)
    Bb = A + (1 << 33)
    name = lambda *args: dg.gemm_config_info(dg.gemm_select_config(*args))["name"]
    for M, N, K in [(4096, 4096, 4096), (8192, 8192, 128), (4096, 4096 - 124, 64)]:
        assert name(A, Bb, Cb, M, N, K, 0) == "fp32_128x128x32", (M, N, K)
    for M, N, K in [(3072, 3072, 3072), (4096, 4096 - 128, 64), (1024, 1024, 1024), (128, 128, 128),
                    (8192, 4, 4096), (300, 1000, 8), (64, 64, 64), (127, 128, 128), (1, 4, 4)]:
        assert name(A, Bb, Cb, M, N, K, 0) == "fp32_64x64x32", (M, N, K)
    for M, N, K in [(4096, 4096, 4094), (4096, 4094, 4096), (64, 62, 64), (3, 5, 7)]:
        assert name(A, Bb, Cb, M, N, K, 0) == "generic_64x64", (M, N, K)
    assert name(A + 4, Bb, Cb, 1024, 1024, 1024, 0) == "generic_64x64"   # A not 16-byte aligned
    info = dg.gemm_config_info(45)
    assert (info["bm"], info["bn"], info["bk"], info["dtype_mask"], info["threads"]) == (128, 128, 32, 1, 256)


def test_clocked_run_checks_its_arguments_on_the_host():
    L = _lib.lib()
    Cb = C + (1 << 34)
    Bb = A + (1 << 33)
    assert L.gemm_run_clocked(None, A, Bb, Cb, 64, 64, 64, 1, None, None) == INVALID          # no clk
    assert L.gemm_run_clocked(None, A, Bb, Cb, 64, 64, 64, 1, A + (1 << 35) + 4, None) == INVALID   # misaligned
    assert L.gemm_run_clocked(None, A, Bb, Cb, 64, 64, 64, 1, A + (1 << 35), None) == INVALID       # no handle
    assert L.gemm_run_clocked(None, A, Bb, Cb, 64, 64, 64, 9, A + (1 << 35), None) == BADTYPE
