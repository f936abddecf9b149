"""CPU checks of the C ABI: the library loads, exports every symbol snm.h declares, and
rejects bad arguments on the host before any HIP call (no compute runs here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def _lib():
    from structured_sparse_matrix_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libsnm.so not built (run __graft_entry__.build())")
    return L.load()


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(snm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("snm_prune_encode_nm", "snm_prune_encode_vnm", "snm_spmm_nm", "snm_spmm_vnm",
              "snm_sddmm_prune_nm", "snm_softmax_nm_rows", "snm_sddmm_prune_nm_rowmax",
              "snm_spmm_nm_softmax", "snm_bitmap_sizes", "snm_bitmap_count", "snm_bitmap_encode",
              "snm_spmm_bitmap", "snm_sddmm_prune_nm_bf16", "snm_softmax_nm_rows_bf16",
              "snm_spmm_nm_bf16", "snm_spmm_nm_softmax_bf16", "snm_sddmm_prune_1of2_f32",
              "snm_softmax_nm_rows_f32", "snm_spmm_1of2_f32", "snm_prune_encode_vnm_tiled",
              "snm_spmm_vnm_tiled", "snm_spmm_nm_tiled_ws_bytes", "snm_spmm_nm_tiled_ws"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    from structured_sparse_matrix_amd import _lib as L
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in snm.h but not exported"
        assert name in L.SIGNATURES, f"{name} has no ctypes signature in the binding"


def test_exported_symbols_are_c_linkage():
    # nm -D lists dynamic symbols; every declared name must appear unmangled
    import subprocess
    from structured_sparse_matrix_amd import _lib as L
    _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in syms


def test_version_and_status_strings():
    lib = _lib()
    assert lib.snm_abi_version() == 1
    for s in range(7):
        assert lib.snm_status_string(s)
    assert lib.snm_status_string(99) == b"unknown status"


def test_size_queries():
    from structured_sparse_matrix_amd import nm_sizes, vnm_sizes, SnmError
    _lib()
    assert nm_sizes(4096, 4096) == (4096 * 2048, 4096 * 512)
    assert nm_sizes(2, 16) == (16, 4)
    # V:2:M, V=128 M=16 on 8192 x 8192: values 8192 x 1024, midx 8192 x 256 B, colloc 64 x 512 x 4
    assert vnm_sizes(8192, 8192, 128, 16) == (8192 * 1024, 8192 * 256, 64 * 512 * 4)
    assert vnm_sizes(11008, 4096, 64, 8) == (11008 * 1024, 11008 * 256, 172 * 512 * 4)
    with pytest.raises(SnmError):
        nm_sizes(4, 8)            # K % 16 != 0
    with pytest.raises(SnmError):
        vnm_sizes(100, 64, 64, 8)  # R % V != 0
    with pytest.raises(SnmError):
        vnm_sizes(64, 48, 64, 8)   # (K/M) % 4 != 0
    with pytest.raises(SnmError):
        vnm_sizes(64, 1024, 64, 2)  # M < 4


P = ctypes.c_void_p
FAKE = P(0x1000)          # never dereferenced: every call below fails validation first
MISALIGNED = P(0x1008)


def _nm(args, at, n=2, m=4):
    """The argument tuple with the N:M pattern (n, m) inserted at position `at`."""
    return tuple(args[:at]) + (n, m) + tuple(args[at:])


def _vnm(args, at, n=2):
    """The argument tuple with the V:N:M n inserted at position `at` (between V and M)."""
    return tuple(args[:at]) + (n,) + tuple(args[at:])


# The pattern arguments are checked first: anything but 2:4 (N:M) or n = 2 (V:N:M) is
# SNM_E_UNSUPPORTED even where every other argument is valid, and nothing is enqueued.
@pytest.mark.parametrize("n,m", [(1, 2), (2, 8), (4, 8), (1, 4), (2, 2), (0, 0)])
def test_nm_pattern_arguments_rejected(n, m):
    lib = _lib()
    v, mb = ctypes.c_int64(), ctypes.c_int64()
    assert lib.snm_nm_sizes(64, 64, n, m, ctypes.byref(v), ctypes.byref(mb)) == 4
    assert lib.snm_prune_encode_nm(FAKE, 4, 16, 16, n, m, FAKE, FAKE, P(0)) == 4
    assert lib.snm_spmm_nm(FAKE, FAKE, 16, 32, n, m, FAKE, 8, 8, 0, FAKE, 8, 1, 0, 0, 0, 0, P(0)) == 4
    assert lib.snm_sddmm_prune_nm(FAKE, FAKE, 1, 16, 32, 64, ctypes.c_float(0.125), n, m, FAKE, FAKE,
                                  P(0), P(0)) == 4
    # the same calls with (2, 4) get past the pattern check (to the size query's result, or
    # to the empty-problem early return with nothing enqueued)
    assert lib.snm_nm_sizes(64, 64, 2, 4, ctypes.byref(v), ctypes.byref(mb)) == 0 and v.value == 64 * 32
    assert lib.snm_prune_encode_nm(P(0), 0, 16, 16, 2, 4, P(0), P(0), P(0)) == 0


@pytest.mark.parametrize("n", [1, 3, 4, 0])
def test_vnm_pattern_argument_rejected(n):
    lib = _lib()
    v, mi, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    assert lib.snm_vnm_sizes(128, 64, 64, n, 8, ctypes.byref(v), ctypes.byref(mi), ctypes.byref(c)) == 4
    assert lib.snm_prune_encode_vnm(FAKE, 128, 64, 64, 64, n, 8, FAKE, FAKE, FAKE, P(0)) == 4
    assert lib.snm_prune_encode_vnm_tiled(FAKE, 128, 64, 64, 64, n, 8, FAKE, FAKE, FAKE, P(0)) == 4
    assert lib.snm_spmm_vnm(FAKE, FAKE, FAKE, 64, 64, 64, n, 8, FAKE, 8, 8, FAKE, 8, P(0)) == 4
    assert lib.snm_spmm_vnm_tiled(FAKE, FAKE, FAKE, 64, 64, 64, n, 8, FAKE, 64, 64, FAKE, 64, P(0)) == 4
    assert lib.snm_vnm_sizes(128, 64, 64, 2, 8, ctypes.byref(v), ctypes.byref(mi), ctypes.byref(c)) == 0


@pytest.mark.parametrize("args,status", [
    ((P(0), 4, 16, 16, FAKE, FAKE, P(0)), 1),           # A NULL
    ((FAKE, 4, 12, 16, FAKE, FAKE, P(0)), 2),           # K % 16
    ((FAKE, 4, 16, 8, FAKE, FAKE, P(0)), 2),            # lda < K
    ((FAKE, 4, 16, 20, FAKE, FAKE, P(0)), 3),           # lda % 8
    ((MISALIGNED, 4, 16, 16, FAKE, FAKE, P(0)), 3),     # pointer alignment
    ((FAKE, -1, 16, 16, FAKE, FAKE, P(0)), 2),          # negative R
    ((P(0), 0, 16, 16, P(0), P(0), P(0)), 0),           # empty: ok, nothing enqueued
])
def test_prune_encode_nm_validation(args, status):
    assert _lib().snm_prune_encode_nm(*_nm(args, 4)) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, 128, 64, 64, 64, 3, FAKE, FAKE, FAKE, P(0)), 4),     # M < 4
    ((FAKE, 128, 64, 64, 0, 8, FAKE, FAKE, FAKE, P(0)), 4),      # V < 1
    ((FAKE, 100, 64, 64, 64, 8, FAKE, FAKE, FAKE, P(0)), 2),     # R % V
    ((FAKE, 128, 48, 48, 64, 8, FAKE, FAKE, FAKE, P(0)), 2),     # (K/M) % 4
    ((FAKE, 128, 64, 64, 64, 8, P(0), FAKE, FAKE, P(0)), 1),     # values NULL
])
def test_prune_encode_vnm_validation(args, status):
    assert _lib().snm_prune_encode_vnm(*_vnm(args, 5)) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, 16, 24, FAKE, 8, 8, 0, FAKE, 8, 1, 0, 0, 0, 0, P(0)), 2),      # K % 16
    ((FAKE, FAKE, 16, 32, FAKE, 8, 4, 0, FAKE, 8, 1, 0, 0, 0, 0, P(0)), 2),      # ldb < C
    ((FAKE, FAKE, 16, 32, FAKE, 8, 16, 1, FAKE, 8, 1, 0, 0, 0, 0, P(0)), 2),     # column-major: ldb < K
    ((FAKE, FAKE, 16, 32, FAKE, 8, 8, 2, FAKE, 8, 1, 0, 0, 0, 0, P(0)), 4),      # unknown layout
    ((FAKE, FAKE, 16, 32, FAKE, 8, 8, 0, P(0x1001), 12, 1, 0, 0, 0, 0, P(0)), 3),  # odd Y pointer
    ((FAKE, P(0), 16, 32, FAKE, 8, 8, 0, FAKE, 8, 1, 0, 0, 0, 0, P(0)), 1),      # meta NULL
    ((FAKE, FAKE, 16, 32, FAKE, 8, 8, 0, FAKE, 8, 2, 8, 64, 256, 128, P(0)), 2),  # stride_values too small
    ((FAKE, FAKE, 16, 32, FAKE, 8, 8, 0, FAKE, 8, -1, 0, 0, 0, 0, P(0)), 2),     # negative batch
    ((P(0), P(0), 16, 32, P(0), 0, 0, 0, P(0), 0, 1, 0, 0, 0, 0, P(0)), 0),      # C == 0: ok
])
def test_spmm_nm_validation(args, status):
    assert _lib().snm_spmm_nm(*_nm(args, 4)) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, FAKE, 64, 64, 8, 8, FAKE, 8, 8, FAKE, 8, P(0)), 4),    # V not a multiple of 16
    ((FAKE, FAKE, FAKE, 64, 48, 64, 8, FAKE, 8, 8, FAKE, 8, P(0)), 2),   # (K/M) % 4
    ((FAKE, FAKE, P(0), 64, 64, 64, 8, FAKE, 8, 8, FAKE, 8, P(0)), 1),   # colloc NULL
])
def test_spmm_vnm_validation(args, status):
    assert _lib().snm_spmm_vnm(*_vnm(args, 6)) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, 128, 64, 64, 16, 8, FAKE, FAKE, FAKE, P(0)), 4),     # V % 32
    ((FAKE, 128, 48, 48, 64, 8, FAKE, FAKE, FAKE, P(0)), 2),     # (K/M) % 4
    ((FAKE, 128, 64, 64, 64, 8, FAKE, P(0), FAKE, P(0)), 1),     # midx NULL
    ((FAKE, 128, 64, 60, 64, 8, FAKE, FAKE, FAKE, P(0)), 2),     # lda < K
])
def test_prune_encode_vnm_tiled_validation(args, status):
    assert _lib().snm_prune_encode_vnm_tiled(*_vnm(args, 5)) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, FAKE, 64, 64, 16, 8, FAKE, 64, 64, FAKE, 64, P(0)), 4),         # V % 32
    ((FAKE, FAKE, FAKE, 64, 64, 64, 8, FAKE, 60, 64, FAKE, 64, P(0)), 4),         # C % 8
    ((FAKE, FAKE, FAKE, 64, 64, 64, 8, FAKE, 64, 68, FAKE, 64, P(0)), 4),         # ldb % 8
    ((FAKE, FAKE, FAKE, 64, 64, 64, 8, P(0x1008), 64, 64, FAKE, 64, P(0)), 3),    # B not 16-byte aligned
    ((FAKE, FAKE, FAKE, 64, 8 * 4100 * 4, 64, 8, FAKE, 64, 64, FAKE, 64, P(0)), 4),  # 4K/M > 16384
    ((FAKE, FAKE, P(0), 64, 64, 64, 8, FAKE, 64, 64, FAKE, 64, P(0)), 1),         # colloc NULL
    ((P(0), P(0), P(0), 64, 64, 64, 8, P(0), 0, 0, P(0), 0, P(0)), 0),            # C == 0: ok
])
def test_spmm_vnm_tiled_validation(args, status):
    assert _lib().snm_spmm_vnm_tiled(*_vnm(args, 6)) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, 1, 16, 32, 48, ctypes.c_float(0.125), FAKE, FAKE, P(0), P(0)), 4),   # d unsupported
    ((FAKE, FAKE, 1, 16, 40, 64, ctypes.c_float(0.125), FAKE, FAKE, P(0), P(0)), 2),   # Lk % 32
    ((FAKE, P(0), 1, 16, 32, 64, ctypes.c_float(0.125), FAKE, FAKE, P(0), P(0)), 1),   # Kmat NULL
    ((FAKE, FAKE, 1, 16, 32, 64, ctypes.c_float(0.125), FAKE, FAKE, MISALIGNED, P(0)), 3),
])
def test_sddmm_validation(args, status):
    assert _lib().snm_sddmm_prune_nm(*_nm(args, 7)) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, 1, 16, 32, 48, ctypes.c_float(0.125), FAKE, FAKE, FAKE, P(0)), 4),   # d unsupported
    ((FAKE, FAKE, 1, 16, 32, 64, ctypes.c_float(0.125), FAKE, FAKE, P(0), P(0)), 1),   # row_max NULL
    ((FAKE, FAKE, 1, 16, 32, 64, ctypes.c_float(0.125), FAKE, FAKE, P(0x1002), P(0)), 3),  # row_max % 4
    ((P(0), P(0), 0, 16, 32, 64, ctypes.c_float(0.125), P(0), P(0), P(0), P(0)), 0),   # empty batch
])
def test_sddmm_rowmax_validation(args, status):
    assert _lib().snm_sddmm_prune_nm_rowmax(*args) == status


# values, meta, row_max, R, K, B, C, ldb, Y, ldy, batch, s_values, s_meta, s_rowmax, s_B, s_Y, stream
@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, FAKE, 16, 24, FAKE, 8, 8, FAKE, 8, 1, 0, 0, 0, 0, 0, P(0)), 2),      # K % 16
    ((FAKE, FAKE, P(0), 16, 32, FAKE, 8, 8, FAKE, 8, 1, 0, 0, 0, 0, 0, P(0)), 1),      # row_max NULL
    ((FAKE, FAKE, FAKE, 16, 32, FAKE, 12, 12, FAKE, 12, 1, 0, 0, 0, 0, 0, P(0)), 3),   # C % 8
    ((FAKE, FAKE, FAKE, 16, 32, FAKE, 8, 12, FAKE, 8, 1, 0, 0, 0, 0, 0, P(0)), 3),     # ldb % 8
    ((FAKE, FAKE, FAKE, 16, 32, P(0x1008), 8, 8, FAKE, 8, 1, 0, 0, 0, 0, 0, P(0)), 3),  # B 16-byte alignment
    ((FAKE, FAKE, P(0x1002), 16, 32, FAKE, 8, 8, FAKE, 8, 1, 0, 0, 0, 0, 0, P(0)), 3),  # row_max % 4
    ((FAKE, FAKE, FAKE, 16, 0, FAKE, 8, 8, FAKE, 8, 1, 0, 0, 0, 0, 0, P(0)), 2),       # K == 0: no softmax
    ((FAKE, FAKE, FAKE, 16, 32, FAKE, 8, 8, FAKE, 8, 2, 256, 64, 8, 256, 128, P(0)), 2),  # stride_row_max < R
    ((FAKE, FAKE, FAKE, 16, 1 << 24, FAKE, 8, 8, FAKE, 8, 1, 0, 0, 0, 0, 0, P(0)), 2),  # 128*K >= 2^31
    ((P(0), P(0), P(0), 0, 32, P(0), 8, 8, P(0), 8, 1, 0, 0, 0, 0, 0, P(0)), 0),       # R == 0: ok
])
def test_spmm_softmax_validation(args, status):
    assert _lib().snm_spmm_nm_softmax(*args) == status


def test_bitmap_sizes_and_validation():
    from structured_sparse_matrix_amd import bitmap_sizes, SnmError
    _lib()
    assert bitmap_sizes(9216, 9216) == (9216 * 144, 9216 * 144 + 1)
    assert bitmap_sizes(0, 64) == (0, 1)
    with pytest.raises(SnmError):
        bitmap_sizes(4, 100)                     # K % 64
    with pytest.raises(SnmError):
        bitmap_sizes(1 << 16, 1 << 15)           # R*K >= 2^31
    lib = _lib()
    # count: A, R, K, lda, bitmaps, offsets, stream
    assert lib.snm_bitmap_count(FAKE, 4, 96, 96, FAKE, FAKE, P(0)) == 2          # K % 64
    assert lib.snm_bitmap_count(FAKE, 4, 64, 64, FAKE, P(0), P(0)) == 1          # offsets NULL
    assert lib.snm_bitmap_count(FAKE, 4, 64, 60, FAKE, FAKE, P(0)) == 2          # lda < K
    assert lib.snm_bitmap_count(FAKE, 4, 64, 72, P(0x1004), FAKE, P(0)) == 3     # bitmaps % 8
    assert lib.snm_bitmap_count(MISALIGNED, 4, 64, 64, FAKE, FAKE, P(0)) == 3    # A % 16
    # encode: A, R, K, lda, bitmaps, offsets, values, stream
    assert lib.snm_bitmap_encode(FAKE, 4, 64, 64, P(0), FAKE, FAKE, P(0)) == 1   # bitmaps NULL
    assert lib.snm_bitmap_encode(P(0), 0, 64, 64, P(0), FAKE, P(0), P(0)) == 0   # empty
    # spmm: bitmaps, offsets, values, R, K, B, C, ldb, b_layout, Y, ldy, stream
    assert lib.snm_spmm_bitmap(FAKE, FAKE, FAKE, 16, 64, FAKE, 40, 64, 1, FAKE, 40, P(0)) == 4   # C > 32
    assert lib.snm_spmm_bitmap(FAKE, FAKE, FAKE, 16, 64, FAKE, 8, 64, 2, FAKE, 8, P(0)) == 4     # layout
    assert lib.snm_spmm_bitmap(FAKE, FAKE, FAKE, 16, 64, FAKE, 8, (1 << 25) + 1, 0, FAKE, 8, P(0)) == 4  # row stride
    assert lib.snm_spmm_bitmap(FAKE, FAKE, MISALIGNED, 16, 64, FAKE, 8, 64, 1, FAKE, 8, P(0)) == 3
    assert lib.snm_spmm_bitmap(FAKE, FAKE, FAKE, 16, 64, FAKE, 8, 68, 1, FAKE, 8, P(0)) == 3     # ldb % 8
    assert lib.snm_spmm_bitmap(FAKE, FAKE, FAKE, 16, 64, FAKE, 8, 32, 1, FAKE, 8, P(0)) == 2     # ldb < K
    assert lib.snm_spmm_bitmap(P(0), P(0), P(0), 0, 64, P(0), 8, 64, 1, P(0), 8, P(0)) == 0      # R == 0


def test_spmm_ws_plan_and_validation():
    from structured_sparse_matrix_amd import spmm_nm_tiled_ws_bytes, SnmError
    # 4096 x 14336: 64 groups of 4 row tiles x 4 splits; counters (256-byte rounded) then
    # fp32 tiles of 64 rows x 32 (C > 16) or 16 columns
    assert spmm_nm_tiled_ws_bytes(4096, 14336, 32) == 256 + 4 * 64 * (64 * 32) * 4
    assert spmm_nm_tiled_ws_bytes(4096, 14336, 16) == 256 + 4 * 64 * (64 * 16) * 4
    assert spmm_nm_tiled_ws_bytes(4096, 14336, 8) == 0     # K*C < 163840 with 256 row tiles
    assert spmm_nm_tiled_ws_bytes(4096, 4096, 32) == 0     # the unsplit kernel is faster there
    assert spmm_nm_tiled_ws_bytes(2048, 8192, 8) == 256 + 4 * 64 * (32 * 16) * 4   # 128 row tiles: 64 groups of 2, 4 splits
    assert spmm_nm_tiled_ws_bytes(1024, 16384, 32) == 256 + 4 * 32 * (32 * 32) * 4  # at most 4 splits
    assert spmm_nm_tiled_ws_bytes(64, 512, 32) == 0        # 8 chunks: fewer than one per wave
    assert spmm_nm_tiled_ws_bytes(0, 4096, 32) == 0
    with pytest.raises(SnmError):
        spmm_nm_tiled_ws_bytes(16, 64, 33)                  # C > 32
    with pytest.raises(SnmError):
        spmm_nm_tiled_ws_bytes(16, 72, 8)                   # K % 16
    lib = _lib()
    need = spmm_nm_tiled_ws_bytes(64, 2048, 32)
    assert need > 0
    # values_t, meta_t, R, K, B, C, ldb, Y, ldy, workspace, workspace_bytes, stream
    assert lib.snm_spmm_nm_tiled_ws(FAKE, FAKE, 64, 2048, FAKE, 32, 2048, FAKE, 32, FAKE, need - 1, P(0)) == 2
    assert lib.snm_spmm_nm_tiled_ws(FAKE, FAKE, 64, 2048, FAKE, 32, 2048, FAKE, 32, P(0), need, P(0)) == 1
    assert lib.snm_spmm_nm_tiled_ws(FAKE, FAKE, 64, 2048, FAKE, 32, 2048, FAKE, 32, MISALIGNED, need, P(0)) == 3
    assert lib.snm_spmm_nm_tiled_ws(FAKE, FAKE, 64, 2048, FAKE, 40, 2048, FAKE, 40, FAKE, need, P(0)) == 4
    assert lib.snm_spmm_nm_tiled_ws(FAKE, FAKE, 64, 2048, FAKE, 32, 2040, FAKE, 32, FAKE, need, P(0)) == 2  # ldb < K
    assert lib.snm_spmm_nm_tiled_ws(FAKE, FAKE, 64, 2048, FAKE, 32, 2048, FAKE, 32, FAKE, -1, P(0)) == 2
    assert lib.snm_spmm_nm_tiled_ws(P(0), P(0), 0, 2048, P(0), 32, 2048, P(0), 32, P(0), 0, P(0)) == 0    # R == 0
    # the no-allocation variant: the same checks without the workspace
    assert lib.snm_spmm_nm_tiled_noalloc(FAKE, FAKE, 64, 2048, FAKE, 40, 2048, FAKE, 40, P(0)) == 4
    assert lib.snm_spmm_nm_tiled_noalloc(FAKE, FAKE, 64, 2048, FAKE, 32, 2040, FAKE, 32, P(0)) == 2  # ldb < K
    assert lib.snm_spmm_nm_tiled_noalloc(P(0), FAKE, 64, 2048, FAKE, 32, 2048, FAKE, 32, P(0)) == 1
    assert lib.snm_spmm_nm_tiled_noalloc(P(0), P(0), 0, 2048, P(0), 32, 2048, P(0), 32, P(0)) == 0    # R == 0


def test_softmax_validation():
    lib = _lib()
    assert lib.snm_softmax_nm_rows(FAKE, 4, 16, 8, P(0)) == 2       # ld < kept
    assert lib.snm_softmax_nm_rows(P(0), 4, 16, 16, P(0)) == 1
    assert lib.snm_softmax_nm_rows(MISALIGNED, 4, 16, 16, P(0)) == 3
    assert lib.snm_softmax_nm_rows(P(0), 0, 16, 16, P(0)) == 0


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    from structured_sparse_matrix_amd import _lib as L
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(L, "_lib", None)
    with pytest.raises(ImportError):
        L.load()


def test_binding_never_imports_the_oracle():
    # the product package must not reach the CPU oracle
    pkg = os.path.join(ROOT, "structured_sparse_matrix_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), f
                assert not re.search(r"import_module\(\s*['\"]oracle", text), f


# Q, K, batch, Lq, Lk, d, scale, values, meta, S_dense, row_max, stream
@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, 1, 16, 32, 48, ctypes.c_float(0.125), FAKE, FAKE, P(0), P(0), P(0)), 4),   # d unsupported
    ((FAKE, FAKE, 1, 16, 40, 64, ctypes.c_float(0.125), FAKE, FAKE, P(0), P(0), P(0)), 2),   # Lk % 32
    ((FAKE, P(0), 1, 16, 32, 64, ctypes.c_float(0.125), FAKE, FAKE, P(0), P(0), P(0)), 1),   # Kmat NULL
    ((FAKE, FAKE, 1, 16, 32, 64, ctypes.c_float(0.125), FAKE, FAKE, MISALIGNED, P(0), P(0)), 3),
    ((FAKE, FAKE, 1, 16, 32, 64, ctypes.c_float(0.125), FAKE, FAKE, P(0), P(0x1002), P(0)), 3),  # row_max % 4
    ((P(0), P(0), 0, 16, 32, 64, ctypes.c_float(0.125), P(0), P(0), P(0), P(0), P(0)), 0),   # empty batch
])
def test_sddmm_bf16_validation(args, status):
    assert _lib().snm_sddmm_prune_nm_bf16(*args) == status


# values, meta, R, K, B, C, ldb, Y, ldy, batch, s_values, s_meta, s_B, s_Y, stream
@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, 16, 24, FAKE, 8, 8, FAKE, 8, 1, 0, 0, 0, 0, P(0)), 2),       # K % 16
    ((FAKE, P(0), 16, 32, FAKE, 8, 8, FAKE, 8, 1, 0, 0, 0, 0, P(0)), 1),       # meta NULL
    ((FAKE, FAKE, 16, 32, FAKE, 12, 12, FAKE, 12, 1, 0, 0, 0, 0, P(0)), 3),    # C % 8
    ((FAKE, FAKE, 16, 32, FAKE, 8, 12, FAKE, 8, 1, 0, 0, 0, 0, P(0)), 3),      # ldb % 8
    ((FAKE, FAKE, 16, 32, P(0x1008), 8, 8, FAKE, 8, 1, 0, 0, 0, 0, P(0)), 3),  # B 16-byte alignment
    ((FAKE, FAKE, 16, 1 << 24, FAKE, 8, 8, FAKE, 8, 1, 0, 0, 0, 0, P(0)), 2),  # 128*K >= 2^31
    ((P(0), P(0), 0, 32, P(0), 8, 8, P(0), 8, 1, 0, 0, 0, 0, P(0)), 0),        # R == 0: ok
])
def test_spmm_bf16_validation(args, status):
    assert _lib().snm_spmm_nm_bf16(*args) == status


def test_bf16_softmax_and_fused_validation():
    lib = _lib()
    assert lib.snm_softmax_nm_rows_bf16(FAKE, 4, 16, 8, P(0)) == 2        # ld < kept
    assert lib.snm_softmax_nm_rows_bf16(MISALIGNED, 4, 16, 16, P(0)) == 3
    assert lib.snm_softmax_nm_rows_bf16(P(0), 0, 16, 16, P(0)) == 0
    # values, meta, row_max, R, K, B, C, ldb, Y, ldy, batch, strides x 5, stream
    assert lib.snm_spmm_nm_softmax_bf16(FAKE, FAKE, P(0), 16, 32, FAKE, 8, 8, FAKE, 8, 1,
                                        0, 0, 0, 0, 0, P(0)) == 1       # row_max NULL
    assert lib.snm_spmm_nm_softmax_bf16(FAKE, FAKE, FAKE, 16, 0, FAKE, 8, 8, FAKE, 8, 1,
                                        0, 0, 0, 0, 0, P(0)) == 2       # K == 0


def test_f32_1of2_validation():
    lib = _lib()
    f = ctypes.c_float(0.125)
    # Q, K, batch, Lq, Lk, d, scale, values, meta, S_dense, row_max, stream
    assert lib.snm_sddmm_prune_1of2_f32(FAKE, FAKE, 1, 16, 32, 48, f, FAKE, FAKE, P(0), P(0), P(0)) == 4
    assert lib.snm_sddmm_prune_1of2_f32(FAKE, FAKE, 1, 16, 48, 64, f, FAKE, FAKE, P(0), P(0), P(0)) == 2
    assert lib.snm_sddmm_prune_1of2_f32(FAKE, FAKE, 1, 16, 32, 64, f, P(0), FAKE, P(0), P(0), P(0)) == 1
    assert lib.snm_sddmm_prune_1of2_f32(FAKE, FAKE, 1, 16, 32, 64, f, FAKE, FAKE, P(0), P(0x1002), P(0)) == 3
    assert lib.snm_softmax_nm_rows_f32(FAKE, 4, 16, 8, P(0)) == 2
    assert lib.snm_softmax_nm_rows_f32(MISALIGNED, 4, 16, 16, P(0)) == 3
    # values, meta, row_max, R, K, B, C, ldb, Y, ldy, batch, s_values, s_meta, s_rowmax, s_B, s_Y, stream
    def spmm(*a):
        return lib.snm_spmm_1of2_f32(*a)
    assert spmm(FAKE, FAKE, P(0), 16, 48, FAKE, 8, 8, FAKE, 8, 1, 0, 0, 0, 0, 0, P(0)) == 2       # K % 32
    assert spmm(FAKE, P(0), P(0), 16, 64, FAKE, 8, 8, FAKE, 8, 1, 0, 0, 0, 0, 0, P(0)) == 1       # meta NULL
    assert spmm(FAKE, FAKE, P(0), 16, 64, FAKE, 6, 8, FAKE, 8, 1, 0, 0, 0, 0, 0, P(0)) == 3       # C % 4
    assert spmm(FAKE, FAKE, P(0), 16, 64, FAKE, 8, 10, FAKE, 8, 1, 0, 0, 0, 0, 0, P(0)) == 3      # ldb % 4
    assert spmm(FAKE, P(0x1004), P(0), 16, 64, FAKE, 8, 8, FAKE, 8, 1, 0, 0, 0, 0, 0, P(0)) == 3  # meta % 8
    assert spmm(FAKE, FAKE, FAKE, 16, 0, FAKE, 8, 8, FAKE, 8, 1, 0, 0, 0, 0, 0, P(0)) == 2        # softmax, K == 0
    assert spmm(FAKE, FAKE, P(0), 16, 64, FAKE, 8, 8, FAKE, 8, 2, 100, 256, 0, 512, 128, P(0)) == 2  # stride_values
    assert spmm(P(0), P(0), P(0), 0, 64, P(0), 8, 8, P(0), 8, 1, 0, 0, 0, 0, 0, P(0)) == 0         # R == 0


def test_empty_reduction_strides_carry_no_alignment_rule():
    # values, meta, R, K, B, C, ldb, b_layout, Y, ldy, batch, s_values, s_meta, s_B, s_Y, stream
    lib = _lib()
    # K = 16: a metadata batch stride that is not a multiple of 16 bytes is rejected
    assert lib.snm_spmm_nm(FAKE, FAKE, 40, 16, 2, 4, FAKE, 8, 8, 0, FAKE, 8, 2, 320, 88, 128, 320, P(0)) == 3
    # K = 0 (nothing is read): the same strides pass validation; without a GPU the call then
    # stops at the device check (SNM_E_DEVICE), with one it writes zeros (GPU test)
    st = lib.snm_spmm_nm(FAKE, FAKE, 40, 0, 2, 4, FAKE, 8, 8, 0, FAKE, 8, 2, 40, 40, 0, 320, P(0))
    assert st in (0, 5)


def test_validation_unit_builds_with_the_host_compiler(tmp_path):
    # validate.cpp is HIP-free: it must compile with a plain host compiler (where it can be
    # built with host sanitizers), warnings treated as errors
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    src = os.path.join(ROOT, "structured_sparse_matrix_amd", "csrc", "validate.cpp")
    out = subprocess.run([gxx, "-std=c++17", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                          "-c", src, "-o", str(tmp_path / "validate.o")], capture_output=True, text=True)
    assert out.returncode == 0, out.stderr


def test_split_workspace_is_bounded():
    # the split reduction keeps about 256 workgroups with at most 4 splits, so S * groups
    # < 512 tiles of at most 8 KiB, plus 1 KiB of counters, whatever the shape
    from structured_sparse_matrix_amd import spmm_nm_tiled_ws_bytes
    _lib()
    worst = 0
    for R in [16 * t for t in (1, 63, 64, 255, 256, 257, 1020, 1021, 4096)] + [12288, 16320, 16384, 1 << 20]:
        for K in (1984, 2048, 4096, 14336, 1 << 20):
            for C in (1, 16, 17, 32):
                worst = max(worst, spmm_nm_tiled_ws_bytes(R, K, C))
    assert 0 < worst <= (4 << 20) + 1024


def test_ceiling_validation():
    lib = _lib()
    # src, bytes, sink, stream
    assert lib.snm_ceiling_read(FAKE, 100, FAKE, P(0)) == 2            # bytes % 16
    assert lib.snm_ceiling_read(P(0), 1024, FAKE, P(0)) == 1
    assert lib.snm_ceiling_read(MISALIGNED, 1024, FAKE, P(0)) == 3
    assert lib.snm_ceiling_read(P(0), 0, P(0), P(0)) == 0
    assert lib.snm_ceiling_copy(FAKE, MISALIGNED, 1024, P(0)) == 3
    assert lib.snm_ceiling_copy(FAKE, FAKE, -16, P(0)) == 2
    # kind, workgroups, iters, out, stream
    assert lib.snm_ceiling_matrix(2, 8, 8, FAKE, P(0)) == 4
    assert lib.snm_ceiling_matrix(1, -1, 8, FAKE, P(0)) == 2
    assert lib.snm_ceiling_matrix(0, 8, 8, P(0), P(0)) == 1
    assert lib.snm_ceiling_lds_fill(FAKE, 3 << 20, 8, 8, FAKE, P(0)) == 2   # window not a power of two
    assert lib.snm_ceiling_lds_fill(FAKE, 512, 8, 8, FAKE, P(0)) == 2       # window < one copy
    assert lib.snm_ceiling_lds_fill(FAKE, 1 << 21, -1, 8, FAKE, P(0)) == 2
    assert lib.snm_ceiling_lds_fill(P(0), 1 << 21, 8, 8, FAKE, P(0)) == 1
    assert lib.snm_ceiling_lds_fill(MISALIGNED, 1 << 21, 8, 8, FAKE, P(0)) == 3
    assert lib.snm_ceiling_lds_fill(P(0), 1 << 21, 0, 8, P(0), P(0)) == 0   # empty: nothing enqueued
    assert lib.snm_ceiling_matrix(1, 0, 8, P(0), P(0)) == 0
