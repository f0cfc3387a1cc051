"""Host-side tests of the C ABI (no GPU, no compute calls).

The library must load, export every function include/mm.h declares, and
reject bad arguments on the host before touching HIP.  Pointers passed here
are never dereferenced: validation fails first.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import quantized_skinny_gemm_amd as qs

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "mm.h")

OK, NULL, SHAPE, ALIGN, WS, ALIAS, DEVICE, HIP, ARG = 0, -1, -2, -3, -4, -5, -6, -7, -8
F32, F16, Q4, Q8 = qs.MM_TYPE_F32, qs.MM_TYPE_F16, qs.MM_TYPE_Q4_0, qs.MM_TYPE_Q8_0


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mm_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_five_entry_points():
    names = _declared()
    for n in ("mm_quantize_q4_0", "mm_quantize_q8_0", "mm_mul_mat_q4_0_f32",
              "mm_mul_mat_f16_f32", "mm_mul_mat_f32"):
        assert n in names


def test_header_is_plain_c_and_returns_mm_status():
    """include/mm.h compiles as C99 (plain pointers and sizes, no C++ or HIP
    types), and every call that reports a status declares the mm_status enum."""
    import shutil
    import subprocess
    import tempfile
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        with open(c, "w") as f:
            f.write('#include "mm.h"\nint main(void) { return mm_status_string(MM_OK) == 0; }\n')
        r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                            "-I", os.path.dirname(HEADER), c], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for n in ("mm_quantize_q4_0", "mm_quantize_q8_0", "mm_mul_mat_q4_0_f32",
              "mm_mul_mat_q4_0_f32_noalloc", "mm_q4_0_init", "mm_q4_0_compute",
              "mm_mul_mat_q4_0_f32_group", "mm_repack_q4_0", "mm_unpack_q4_0",
              "mm_mul_mat_q4_0r_f32", "mm_mul_mat_q8_0_f32", "mm_mul_mat_f16_f32",
              "mm_mul_mat_f32", "mm_dispatch", "mm_debug_mul_mat"):
        assert re.search(r"\bmm_status\s+%s\s*\(" % n, src), n


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(qs.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n


def test_status_strings():
    for s in (OK, NULL, SHAPE, ALIGN, WS, ALIAS, DEVICE, HIP, ARG):
        assert qs.status_string(s)
    assert qs.status_string(12345) == "unknown status"


def test_row_bytes():
    assert qs.row_bytes(Q4, 4096) == 4096 // 32 * 18
    assert qs.row_bytes(Q8, 4096) == 4096 // 32 * 34
    assert qs.row_bytes(F16, 37) == 74
    assert qs.row_bytes(F32, 37) == 148
    assert qs.row_bytes(Q4, 48) == -1
    assert qs.row_bytes(99, 32) == -1


FAKE = 0x7f0000000000      # 256-byte aligned, never dereferenced


def _mm_q4(src0, src1, dst, m, n, k, ws, wsb):
    return qs.lib.mm_mul_mat_q4_0_f32(src0, src1, dst, m, n, k, ws, wsb, None)


def test_q4_shape_errors():
    assert _mm_q4(FAKE, FAKE + 2**30, FAKE + 2**31, 1, 16, 48, None, 0) == SHAPE
    assert _mm_q4(FAKE, FAKE + 2**30, FAKE + 2**31, -1, 16, 64, None, 0) == SHAPE
    assert _mm_q4(FAKE, FAKE + 2**30, FAKE + 2**31, 1, -3, 64, None, 0) == SHAPE
    assert _mm_q4(FAKE, FAKE + 2**30, FAKE + 2**31, 1, 16, -32, None, 0) == SHAPE
    assert _mm_q4(FAKE, FAKE + 2**30, FAKE + 2**31, 1, 2**31, 64, None, 0) == SHAPE


def test_empty_problems_are_noops():
    # M == 0 or N == 0: nothing to do, no pointer is looked at
    assert _mm_q4(None, None, None, 0, 16, 64, None, 0) == OK
    assert _mm_q4(None, None, None, 4, 0, 64, None, 0) == OK
    assert qs.lib.mm_mul_mat_f32(None, None, None, 0, 0, 0, None, 0, None) == OK
    assert qs.lib.mm_quantize_q4_0(None, None, 0, 64, None) == OK
    assert qs.lib.mm_quantize_q8_0(None, None, 5, 0, None) == OK


def test_null_pointers():
    ws = qs.workspace_size(Q4, 1, 64, 64)
    assert _mm_q4(FAKE, FAKE + 2**30, None, 1, 64, 64, FAKE + 2**32, ws) == NULL
    assert _mm_q4(None, FAKE + 2**30, FAKE + 2**31, 1, 64, 64, FAKE + 2**32, ws) == NULL
    assert _mm_q4(FAKE, None, FAKE + 2**31, 1, 64, 64, FAKE + 2**32, ws) == NULL
    assert qs.lib.mm_quantize_q8_0(None, FAKE, 1, 64, None) == NULL


def test_alignment():
    ws = qs.workspace_size(Q4, 1, 64, 64)
    args = dict(src0=FAKE, src1=FAKE + 2**30, dst=FAKE + 2**31, ws=FAKE + 2**32)
    assert _mm_q4(FAKE + 1, args["src1"], args["dst"], 1, 64, 64, args["ws"], ws) == ALIGN
    assert _mm_q4(FAKE, args["src1"] + 4, args["dst"], 1, 64, 64, args["ws"], ws) == ALIGN
    assert _mm_q4(FAKE, args["src1"], args["dst"] + 2, 1, 64, 64, args["ws"], ws) == ALIGN
    assert _mm_q4(FAKE, args["src1"], args["dst"], 1, 64, 64, args["ws"] + 64, ws) == ALIGN
    assert qs.lib.mm_quantize_q4_0(FAKE + 4, FAKE + 2**30, 1, 64, None) == ALIGN
    assert qs.lib.mm_quantize_q8_0(FAKE, FAKE + 2**30 + 1, 1, 64, None) == ALIGN
    assert qs.lib.mm_mul_mat_f16_f32(FAKE + 1, FAKE + 2**30, FAKE + 2**31, 1, 8, 8, None, 0, None) == ALIGN
    assert qs.lib.mm_mul_mat_f32(FAKE + 2, FAKE + 2**30, FAKE + 2**31, 1, 8, 8, None, 0, None) == ALIGN


def test_workspace_too_small():
    need = qs.workspace_size(Q4, 4, 256, 512)
    assert need > 0
    assert _mm_q4(FAKE, FAKE + 2**30, FAKE + 2**31, 4, 256, 512, FAKE + 2**32, need - 1) == WS
    assert _mm_q4(FAKE, FAKE + 2**30, FAKE + 2**31, 4, 256, 512, None, need) == WS


def test_aliasing():
    need = qs.workspace_size(Q4, 4, 256, 512)
    # dst overlapping src1
    assert _mm_q4(FAKE, FAKE + 2**30, FAKE + 2**30 + 256, 4, 256, 512, FAKE + 2**32, need) == ALIAS
    # dst overlapping src0
    assert _mm_q4(FAKE, FAKE + 2**30, FAKE + 1024, 4, 256, 512, FAKE + 2**32, need) == ALIAS
    # workspace overlapping dst
    assert _mm_q4(FAKE, FAKE + 2**30, FAKE + 2**31, 4, 256, 512, FAKE + 2**31, need) == ALIAS
    # quantize output overlapping its input
    assert qs.lib.mm_quantize_q8_0(FAKE, FAKE + 64, 4, 64, None) == ALIAS


def test_debug_entry_argument_checks():
    assert qs.lib.mm_debug_mul_mat(Q4, FAKE, FAKE, FAKE, None, 1, 64, 64, 0, 0, 7, None, 0, None) == ARG
    # variants 1-3 only; the wide F kernel is for F16 only
    for t in (F16, F32, Q4):
        assert qs.lib.mm_debug_mul_mat(t, FAKE, FAKE, FAKE, None, 1, 64, 64, 0, 0, 4, None, 0, None) == ARG
    assert qs.lib.mm_debug_mul_mat(F32, FAKE, FAKE, FAKE, None, 1, 64, 64, 0, 0, 2, None, 0, None) == ARG
    # the skinny MFMA variant exists for every type
    for t in (F16, F32, Q4):
        assert qs.lib.mm_debug_workspace_size(t, 4, 64, 64, 3) >= 0
    assert qs.lib.mm_debug_mul_mat(Q4, FAKE, FAKE, FAKE, None, 1, 64, 64, 0, 0, 5, None, 0, None) == ARG
    assert qs.lib.mm_debug_mul_mat(Q4, FAKE, FAKE, FAKE, None, 1, 64, 64, 5, 3, 0, None, 0, None) == SHAPE
    assert qs.lib.mm_debug_mul_mat(Q4, FAKE, FAKE, FAKE, None, 1, 64, 64, 0, 65, 0, None, 0, None) == SHAPE
    assert qs.lib.mm_debug_mul_mat(Q4, FAKE, FAKE, FAKE, None, 1, 64, 64, 0, 8, 0, None, 0, None) == NULL
    assert qs.lib.mm_debug_mul_mat(9, FAKE, FAKE, FAKE, None, 1, 64, 64, 0, 0, 0, None, 0, None) == ARG



def test_tall_products_keep_the_grid_y_limit():
    """The narrow and skinny kernels put src1 row tiles in the grid's y
    dimension (at most 65535 workgroups): beyond 65535 rows the block types
    take the wide kernel whatever the table says, forcing the narrow or
    skinny kernel there is a shape error (before any HIP call), and F16 /
    F32 keep their kernels (launched over row ranges)."""
    R4 = qs.MM_TYPE_Q4_0R
    Q8 = qs.MM_TYPE_Q8_0
    for t in (Q4, R4, Q8):
        assert qs.dispatch(t, 65536, 4096, 4096)[0] == 2
        for v in (1, 3):
            assert qs.lib.mm_debug_workspace_size(t, 65536, 4096, 4096, v) == 0
            assert qs.lib.mm_debug_mul_mat(t, FAKE, FAKE, FAKE, None, 65536, 4096, 4096, 0, 0,
                                           v, None, 0, None) in (SHAPE, ARG)
        assert qs.lib.mm_debug_workspace_size(t, 65536, 4096, 4096, 2) > 0
    # the measured table still applies up to 65535 rows (4096 x 4096: skinny)
    assert qs.dispatch(Q4, 65535, 4096, 4096)[0] == 3
    assert qs.lib.mm_debug_workspace_size(Q4, 65535, 4096, 4096, 1) > 0
    assert qs.dispatch(F32, 2 * 65535 * 16 + 5, 40, 64)[0] == 3
    assert qs.dispatch(F16, 70000, 40, 64)[0] == 2
    d = (ctypes.c_int * 5)()
    assert qs.lib.mm_dispatch(F32, 2 * 65535 * 16 + 5, 40, 64, d) == 0


# The built-in rules, at shapes the measured dispatch table does not list
# (4100 rows); the table itself is tested in test_dispatch_table.py.
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 9, 16, 17, 32, 33, 64, 100, 128, 512])
def test_dispatch_threshold_and_workspace(m):
    variant, split, rows, cols, launches = qs.dispatch(Q4, m, 4100, 4096)
    # M <= 2: narrow kernel with INIT fused (one launch); up to 32 src1 rows:
    # the skinny MFMA kernel; beyond: the wide kernel.  Both of the latter
    # run INIT first, and a split adds the reduce kernel.
    want = 1 if m <= 2 else 3 if m <= 32 else 2
    assert variant == want
    assert launches == (0 if m <= 2 else 1) + 1 + (1 if split > 1 else 0)
    assert split >= 1
    ws = qs.workspace_size(Q4, m, 4100, 4096)
    # at least the wdata: codes + scale + bias per block
    assert ws >= m * 4096 + 2 * 4 * m * 128
    if variant == 1:
        assert rows >= m or rows == 8
    if variant == 3:
        # workgroups of 4, 8 or 16 waves, passes of 8 (two blocks per
        # MFMA), 16 or 32 src1 rows
        assert rows == (8 if m <= 8 else 16 if m <= 16 else 32) and cols in (4, 8, 16)
        assert split == 1
    # F16: M = 1 narrow, up to 16 rows the skinny MFMA kernel, beyond the
    # wide kernel; F32: narrow at M = 1, skinny MFMA from 2 rows
    for t in (F16, F32):
        fv, fsplit, frows, fcols, flaunch = qs.dispatch(t, m, 4100, 4096)
        # (F16 up to 64 rows at this N = 4096 also takes the skinny kernel)
        fwant = 1 if m == 1 else 3 if (m <= 64 or t == F32) else 2
        assert fv == fwant
        if fv == 3:
            # 16-row passes, workgroups of 4 to 16 waves that split K among
            # themselves: one launch, no workspace
            assert frows == 16 and fcols in (4, 8, 16)
            assert fsplit == 1 and flaunch == 1
            assert qs.workspace_size(t, m, 4100, 4096) == 0
        elif fv == 2:
            # the wide F16 kernel converts src1 to binary16 in the workspace,
            # with one power-of-two exponent per row, and with a K split (few
            # tiles) the partial tiles too
            part = fsplit * m * 4100 * 4 if fsplit > 1 else 0
            assert qs.workspace_size(t, m, 4100, 4096) >= m * 4096 * 2 + 4 * m + part
            assert flaunch == 2 + (1 if fsplit > 1 else 0)
        else:
            assert fsplit == 1 and qs.workspace_size(t, m, 4100, 4096) == 0


def test_split_k_when_grid_is_small():
    # the skinny MFMA kernel splits K among the waves of a workgroup, never
    # across workgroups: no partials in the workspace even for a narrow N
    v, split, _, cols, _ = qs.dispatch(Q4, 32, 64, 14336)
    assert v == 3 and split == 1 and cols == 8
    # the wdata (codes, scales, bias) and its operand-order copy (codes and
    # scales: 36 bytes per src1 row and block), nothing for partial sums
    need = 32 * 14336 + 2 * 4 * 32 * 448 + 36 * 32 * 448
    assert need <= qs.workspace_size(Q4, 32, 64, 14336) < need + 4096
    # the wide kernels split across workgroups
    v, split, _, _, _ = qs.dispatch(Q4, 64, 64, 14336)
    assert v == 2 and split > 1
    v, split, _, _, _ = qs.dispatch(Q4, 256, 64, 14336)
    assert v == 2 and split > 1
    # large grids do not split
    assert qs.dispatch(Q4, 512, 14336, 4096)[1] == 1
    assert qs.dispatch(Q4, 1, 11008, 4096)[1] == 1
    assert qs.dispatch(Q4, 16, 14336, 4096)[1] == 1


def test_skinny_mfma_waves_per_workgroup():
    # waves per 16-row workgroup: about 16 waves per CU over the grid (8 with
    # 32-row passes), every wave at least one phase of 4 block pairs, at most
    # 16 waves with 8-row passes and 8 with 16- or 32-row passes
    for m, n, k, want in ((8, 14336, 4096, 8), (16, 4096, 14336, 8), (32, 4096, 14336, 8),
                          (16, 11008, 4096, 8), (8, 256, 512, 4), (4, 4096, 4096, 16),
                          (8, 4096, 14336, 16), (32, 14336, 4096, 4), (32, 4096, 4096, 8)):
        v, split, rows, cols, _ = qs.dispatch(Q4, m, n, k)
        assert v == 3 and split == 1
        assert rows == (8 if m <= 8 else 16 if m <= 16 else 32)
        assert cols == want, (m, n, k, cols)


def test_workspace_size_of_invalid_shapes_is_zero():
    assert qs.workspace_size(Q4, 1, 16, 48) == 0
    assert qs.workspace_size(7, 1, 16, 64) == 0


def test_group_argument_checks():
    n = (ctypes.c_int64 * 2)(64, 64)
    src = (ctypes.c_void_p * 2)(FAKE, FAKE + 2**20)
    dst = (ctypes.c_void_p * 2)(FAKE + 2**31, FAKE + 2**31 + 4 * 64)
    g = qs.lib.mm_mul_mat_q4_0_f32_group
    assert g(0, src, dst, n, FAKE + 2**30, 1, 64, None, 0, None) == ARG
    assert g(9, src, dst, n, FAKE + 2**30, 1, 64, None, 0, None) == ARG
    assert g(2, None, dst, n, FAKE + 2**30, 1, 64, None, 0, None) == NULL
    assert g(2, src, dst, None, FAKE + 2**30, 1, 64, None, 0, None) == NULL
    ws = qs.group_workspace_size([64, 64], 1, 64)
    assert ws > 0
    assert g(2, src, dst, n, FAKE + 2**30, 1, 64, FAKE + 2**32, ws - 1, None) == WS
    # overlapping outputs
    dst2 = (ctypes.c_void_p * 2)(FAKE + 2**31, FAKE + 2**31 + 4)
    assert g(2, src, dst2, n, FAKE + 2**30, 1, 64, FAKE + 2**32, ws, None) == ALIAS
    # an output overlapping another member's weights
    dst3 = (ctypes.c_void_p * 2)(FAKE + 2**31, FAKE + 2**20 + 8)
    assert g(2, src, dst3, n, FAKE + 2**30, 1, 64, FAKE + 2**32, ws, None) == ALIAS
    assert qs.group_workspace_size([64, -1], 1, 64) == 0


def test_measured_tile_and_wave_choices():
    # Q4_0 wide int8 tiles (rows, cols): 64 x 128 up to M = 64 with few weight
    # rows and from M = 65 to 128 with many, 64 x 64 / 128 x 128 otherwise
    # (built-in rules: shapes off the measured table, 16 rows more)
    for m, n, want in ((64, 4096, (64, 128)), (64, 14336, (64, 64)), (128, 14336, (64, 128)),
                       (100, 11008, (64, 128)), (128, 4096, (128, 128)), (512, 14336, (128, 128))):
        v, _, rows, cols, _ = qs.dispatch(Q4, m, n + 16, 4096 if n > 4096 else 14336)
        assert v == 2 and (rows, cols) == want, (m, n, rows, cols)
    # Q4_0 at M = 1 (the fused kernel): one weight row per wave at every size
    for n, k in ((256, 512), (4096, 4096), (4096, 11008), (11008, 4096), (12288, 4096)):
        assert qs.dispatch(Q4, 1, n, k)[3] == 1, (n, k)
    # M = 2: one row per wave only with long K at up to 8192 rows
    assert qs.dispatch(Q4, 2, 4096, 11008)[3] == 1
    assert qs.dispatch(Q4, 2, 4096, 4096)[3] == 2
    # F16 / F32 at M = 1: one weight row per wave, except F16 beyond 8192 rows
    assert qs.dispatch(F32, 1, 11008, 4096)[3] == 1
    assert qs.dispatch(F16, 1, 4096, 4096)[3] == 1
    assert qs.dispatch(F16, 1, 11008, 4096)[3] == 4
    # skinny F MFMA (built-in rules: shapes off the measured table): 8 waves
    # per 16-row workgroup in one pass, 4 per 32-row workgroup when src1
    # takes several passes; fewer only for short K
    assert qs.dispatch(F32, 4, 11008 + 16, 4096)[:4:3] == (3, 8)
    assert qs.dispatch(F16, 16, 11008 + 16, 4096)[:4:3] == (3, 8)
    assert qs.dispatch(F16, 40, 4096 + 16, 4096)[:4:3] == (3, 4)
    assert qs.dispatch(F16, 4, 100, 64)[3] == 4
    # wide F16: the src1 pre-pass, the product, and with at most one 64 x 64
    # tile per two CUs a K split (at least four 128-k stages a slice) and its
    # reduce
    assert qs.dispatch(F16, 512, 14336 + 16, 4096)[:2] == (2, 1)
    assert qs.dispatch(F16, 512, 14336 + 16, 4096)[4] == 2
    v, split, rows, cols, launches = qs.dispatch(F16, 100, 2048 + 16, 4096)   # 66 tiles
    assert (v, rows, cols) == (2, 64, 64) and 2 <= split <= 8 and launches == 3
    assert qs.dispatch(F16, 100, 4096 + 16, 4096)[1] == 1        # 130 tiles: no split
    assert qs.dispatch(F16, 100, 2048 + 16, 512)[1] == 1         # 4 stages: no split


def test_noalloc_entry_point_host_checks():
    # shapes whose workspace exceeds the fixed 64 MiB array are rejected
    # before any pointer is looked at or any HIP call is made
    assert qs.workspace_size(Q4, 4096, 64, 16384) > 64 << 20
    assert qs.lib.mm_mul_mat_q4_0_f32_noalloc(None, None, None, 4096, 64, 16384, None) == WS
    # the usual shape checks and empty problems
    assert qs.lib.mm_mul_mat_q4_0_f32_noalloc(FAKE, FAKE, FAKE, 1, 16, 48, None) == SHAPE
    assert qs.lib.mm_mul_mat_q4_0_f32_noalloc(None, None, None, 0, 16, 64, None) == OK
    # pointer checks come before the device is touched
    assert qs.lib.mm_mul_mat_q4_0_f32_noalloc(FAKE, FAKE + 2**30, None, 1, 64, 64, None) == NULL
    assert qs.lib.mm_mul_mat_q4_0_f32_noalloc(FAKE, FAKE + 2**30 + 4, FAKE + 2**31, 1, 64, 64,
                                              None) == ALIGN


def test_repack_host_checks():
    R = qs.MM_TYPE_Q4_0R
    assert qs.repacked_bytes(16, 256) == 2304
    assert qs.repacked_bytes(17, 256) == 2 * 2304
    assert qs.repacked_bytes(4096, 4096) == 256 * 16 * 2304 == 4096 * 4096 // 32 * 18
    assert qs.repacked_bytes(16, 288) == 2 * 2304       # 9 blocks: a padded second phase
    assert qs.repacked_bytes(16, 48) == -1
    assert qs.row_bytes(R, 4096) == -1
    # argument checks before any HIP call
    assert qs.lib.mm_repack_q4_0(FAKE, FAKE + 2**30, 16, 48, None) == SHAPE
    assert qs.lib.mm_repack_q4_0(None, FAKE, 16, 64, None) == NULL
    assert qs.lib.mm_repack_q4_0(FAKE + 1, FAKE + 2**30, 16, 64, None) == ALIGN
    assert qs.lib.mm_repack_q4_0(FAKE, FAKE + 2**30 + 8, 16, 64, None) == ALIGN
    assert qs.lib.mm_unpack_q4_0(FAKE + 8, FAKE + 2**30, 16, 64, None) == ALIGN
    assert qs.lib.mm_repack_q4_0(FAKE, FAKE + 16, 16, 64, None) == ALIAS
    assert qs.lib.mm_repack_q4_0(None, None, 0, 64, None) == OK
    # products on repacked weights (built-in rules, a shape off the measured
    # table): the skinny kernel from M = 1, the wide one past 32
    for m, want in ((1, 3), (2, 3), (8, 3), (32, 3), (33, 2), (512, 2)):
        v, split, rows, cols, launches = qs.dispatch(R, m, 4112, 4096)
        assert v == want, (m, v)
        assert launches == 2 + (1 if split > 1 else 0)
    assert qs.lib.mm_debug_mul_mat(R, FAKE, FAKE, FAKE, None, 1, 64, 64, 0, 0, 1, None, 0, None) == ARG
    need = qs.workspace_size(R, 4, 256, 512)
    assert need > 0
    st = qs.lib.mm_mul_mat_q4_0r_f32(FAKE + 8, FAKE + 2**30, FAKE + 2**31, 4, 256, 512,
                                     FAKE + 2**32, need, None)
    assert st == ALIGN


def test_q8_0_weights_host_rules():
    """Q8_0 weights: the fused kernel at M <= 2 when K/32 is even (one launch,
    no workspace use), the skinny kernel at 2 < M <= 32 (INIT, then the
    product; passes of 8, 16 or 32 rows), the wide kernel otherwise (INIT,
    product and maybe a reduce); the skinny kernel needs K/32 even; 4-byte
    alignment of src0; K % 32."""
    d = (ctypes.c_int * 5)()
    assert qs.lib.mm_dispatch(Q8, 1, 4096, 4096, d) == OK and d[0] == 1 and d[4] == 1
    assert qs.lib.mm_dispatch(Q8, 2, 11008, 4096, d) == OK and d[0] == 1 and d[2] == 2 and d[4] == 1
    assert qs.lib.mm_dispatch(Q8, 1, 100, 96, d) == OK and d[0] == 2           # K/32 odd
    assert qs.lib.mm_dispatch(Q8, 3, 4096, 4096, d) == OK and d[0] == 3 and d[4] == 2
    assert qs.lib.mm_dispatch(Q8, 8, 14336, 4096, d) == OK and d[0] == 3 and d[4] == 2
    assert qs.lib.mm_dispatch(Q8, 5, 300, 96, d) == OK and d[0] == 2           # K/32 odd: wide
    assert qs.lib.mm_dispatch(Q8, 9, 4096, 4096, d) == OK and d[0] == 3 and d[2] == 16
    assert qs.lib.mm_dispatch(Q8, 32, 4096, 4096, d) == OK and d[0] == 3 and d[2] == 32
    assert qs.lib.mm_dispatch(Q8, 33, 4096, 4096, d) == OK and d[0] == 2
    assert qs.lib.mm_dispatch(Q8, 512, 14336, 4096, d) == OK and d[0] == 2 and (d[2], d[3]) == (128, 64)
    assert qs.lib.mm_dispatch(Q8, 1, 64, 48, d) == SHAPE
    assert qs.lib.mm_debug_workspace_size(Q8, 40, 64, 64, 3) > 0                # 32-row passes
    assert qs.lib.mm_debug_mul_mat(Q8, FAKE, FAKE, FAKE, None, 4, 64, 96, 0, 0, 3, None, 0, None) == ARG
    assert qs.lib.mm_debug_mul_mat(Q8, FAKE, FAKE, FAKE, None, 4, 64, 96, 0, 0, 1, None, 0, None) == ARG
    ws = qs.workspace_size(Q8, 8, 256, 512)
    assert ws > 0
    call = qs.lib.mm_mul_mat_q8_0_f32
    assert call(FAKE + 2, FAKE + 2**30, FAKE + 2**31, 8, 256, 512, FAKE + 2**32, ws, None) == ALIGN
    assert call(FAKE, FAKE + 2**30 + 4, FAKE + 2**31, 8, 256, 512, FAKE + 2**32, ws, None) == ALIGN
    assert call(FAKE, FAKE + 2**30, FAKE + 2**31, 8, 256, 512, FAKE + 2**32, ws - 1, None) == WS
    assert call(FAKE, FAKE + 2**30, FAKE + 2**31, 8, 256, 48, FAKE + 2**32, ws, None) == SHAPE
    assert call(None, FAKE + 2**30, FAKE + 2**31, 8, 256, 512, FAKE + 2**32, ws, None) == NULL
    assert qs.row_bytes(Q8, 4096) == 4096 // 32 * 34


def _dispatch_in_subprocess(env, shapes):
    """mm_dispatch for (type, M, N, K) shapes in a fresh process with `env`
    set (the library reads its environment overrides once per process)."""
    import json
    import os
    import subprocess
    import sys
    code = ("import json, sys, ctypes\n"
            "import quantized_skinny_gemm_amd as qs\n"
            "out = []\n"
            "for t, m, n, k in json.loads(sys.argv[1]):\n"
            "    d = (ctypes.c_int * 5)()\n"
            "    st = qs.lib.mm_dispatch(t, m, n, k, d)\n"
            "    out.append([st] + list(d))\n"
            "print(json.dumps(out))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, "-c", code, json.dumps(shapes)], capture_output=True,
                       text=True, env=e, cwd=root, timeout=120)
    assert r.returncode == 0, r.stderr
    return json.loads(r.stdout.strip().splitlines()[-1])


def test_env_overrides_narrow_max_m_and_split_k():
    """MM_NARROW_MAX_M moves the narrow kernel's M range for Q4_0 (0: never);
    MM_SPLIT_K sets the K split of the narrow and wide kernels (clamped);
    values that are not counts are ignored."""
    Q4 = qs.MM_TYPE_Q4_0
    shapes = [[Q4, 5, 4096, 4096], [Q4, 9, 4096, 4096], [Q4, 1, 4096, 4096], [Q4, 512, 14336, 4096]]
    base = _dispatch_in_subprocess({}, shapes)
    assert [r[1] for r in base] == [3, 3, 1, 2]
    wide_split = base[3][2]
    got = _dispatch_in_subprocess({"MM_NARROW_MAX_M": "8"}, shapes)
    assert [r[1] for r in got] == [1, 3, 1, 2]
    got = _dispatch_in_subprocess({"MM_NARROW_MAX_M": "0"}, shapes)
    assert got[2][1] == 3                                # M = 1 off the narrow kernel
    got = _dispatch_in_subprocess({"MM_SPLIT_K": "4", "MM_NARROW_MAX_M": "8"},
                                  shapes + [[Q4, 5, 4096, 16384]])
    assert got[0][1] == 1 and got[0][2] == 1             # K = 4096: one pair per lane, no split
    assert got[4][1] == 1 and got[4][2] == 4             # narrow, split 4
    assert got[3][1] == 2 and got[3][2] == 4             # wide, split 4
    got = _dispatch_in_subprocess({"MM_SPLIT_K": "1000000"}, [[Q4, 512, 14336, 4096]])
    assert got[0][2] == 4096 // 32 // 4                  # at most one split per stage
    got = _dispatch_in_subprocess({"MM_SPLIT_K": "two", "MM_NARROW_MAX_M": "-3"}, shapes)
    assert got == base
    assert wide_split >= 1
