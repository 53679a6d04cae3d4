"""The C-ABI library on the host (CPU only, no GPU needed).

Loads libmmq.so, checks that it exports every function include/mmq.h declares, and
exercises the size queries, the LDS-budget guard (mmq_plan) and the argument validation
of every entry point. Validation happens before any device access, so each bad call must
return its error code here; a well-formed call reaches the device check.
"""
import ctypes
import subprocess

import pytest

mmq = pytest.importorskip("q4_q8_int8_amd")


def test_exports_every_declared_symbol():
    names = mmq.exported_symbols()
    assert set(names) >= {"quantize_q8_1", "repack_q4_K", "mmq_q4K_q8_1", "mmq_plan"}
    out = subprocess.run(["nm", "-D", "--defined-only", mmq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in names:
        assert name in exported, name
        assert hasattr(mmq._lib, name)


def test_sizes():
    # q, words, pad to 256, (da, nda) plane, pad to 256, 48 bytes of pieces per (row,
    # super-block)
    assert mmq.mmq_q8_1_bytes(2048, 4096) == (2048 * 4096 * 9 // 8 + 8 * 2048 * 128
                                              + 48 * 2048 * 16)
    assert mmq.mmq_q8_1_bytes(1, 32) == 256 + 256 + 48
    assert mmq.mmq_q8_1_bytes(3, 96) == 512 + 256 + 48 * 3
    assert mmq.mmq_q8_1_bytes(2, 288) == 768 + 256 + 48 * 2 * 2
    assert mmq.mmq_q4K_bytes(4096, 4096) == 4096 * 16 * 144
    assert mmq.mmq_q4K_repacked_bytes(4096, 4096) == 128 * 16 * 4608 == 4096 * 4096 * 9 // 16
    assert mmq.mmq_q4K_repacked_bytes(33, 256) == 2 * 4608
    assert mmq.mmq_q4K_repacked_bytes(11008, 4096) == 344 * 16 * 4608


@pytest.mark.parametrize("fn,args,status", [
    ("mmq_q8_1_bytes", (0, 32), mmq.MMQ_E_ARG),
    ("mmq_q8_1_bytes", (4, 33), mmq.MMQ_E_SHAPE),
    ("mmq_q4K_bytes", (4, 128), mmq.MMQ_E_SHAPE),
    ("mmq_q4K_bytes", (-1, 256), mmq.MMQ_E_ARG),
    ("mmq_q4K_repacked_bytes", (4, 300), mmq.MMQ_E_SHAPE),
    ("mmq_q8_1_bytes", (1 << 31, 32), mmq.MMQ_E_SHAPE),
])
def test_size_errors(fn, args, status):
    n = ctypes.c_size_t()
    assert mmq.raw_call(fn, *args, ctypes.byref(n)) == status
    assert mmq.mmq_last_error()


def test_size_null_out():
    assert mmq.raw_call("mmq_q8_1_bytes", 1, 32, None) == mmq.MMQ_E_ARG


# two stages of: token tile [BM][272], (da, nda) [8][BM][2] f32, token pieces [3][BM][8]
# bf16, and per wavefront dsv [8][32] f32 + dmv pieces [3][32][8] bf16 + the 32 row headers
# [32][16] they are expanded from
LARGE, SMALL = mmq.MMQ_TILE_LARGE, mmq.MMQ_TILE_SMALL
LARGE_LDS = 2 * (128 * 272 + 128 * 64 + 128 * 48 + 8 * 3072)
SMALL_LDS = 2 * (32 * 272 + 32 * 64 + 32 * 48 + 2 * 3072)


def test_plan_large_when_it_fits():
    p = mmq.mmq_plan(2048, 4096, 4096, 160 * 1024)
    assert p["tile"] == mmq.MMQ_TILE_LARGE and p["reason"] == mmq.MMQ_REASON_LARGE
    assert p["fallback"] == 0 and p["lds_bytes"] == LARGE_LDS
    assert p["block_m"] == 128 and p["block_n"] == 256 and p["threads"] == 512
    assert p["grid"] == 16 * 16


HALF_LDS = 2 * (64 * 272 + 64 * 64 + 64 * 48 + 8 * 3072)


def test_plan_half_tile_forced():
    p = mmq.mmq_plan(1000, 3000, 4096, 160 * 1024, force_tile=mmq.MMQ_TILE_HALF)
    assert p["tile"] == mmq.MMQ_TILE_HALF and p["reason"] == mmq.MMQ_REASON_FORCED
    assert p["block_m"] == 64 and p["block_n"] == 256 and p["threads"] == 512
    assert p["lds_bytes"] == HALF_LDS
    assert p["grid"] == 16 * 12                 # ceil(1000/64) x ceil(ceil(3000/32)/8)
    # a budget below its stages refuses it (MMQ_E_LDS), as for every forced tile
    with pytest.raises(mmq.MMQError) as e:
        mmq.mmq_plan(1000, 3000, 4096, HALF_LDS - 1, force_tile=mmq.MMQ_TILE_HALF)
    assert e.value.status == mmq.MMQ_E_LDS
    p = mmq.mmq_plan(1000, 3000, 4096, 160 * 1024, force_tile=mmq.MMQ_TILE_HALF, splits=4,
                     workspace_bytes=4 * 1000 * 3000 * 4)
    assert p["tile"] == mmq.MMQ_TILE_HALF and p["splits"] == 4 and p["grid"] == 16 * 12 * 4


def test_plan_lds_fallback_and_refusal():
    p = mmq.mmq_plan(2048, 4096, 4096, LARGE_LDS - 1)
    assert p["tile"] == mmq.MMQ_TILE_SMALL and p["fallback"] == 1
    assert p["reason"] == mmq.MMQ_REASON_LDS_FALLBACK and p["lds_bytes"] == SMALL_LDS
    assert p["grid"] == 64 * 64
    p = mmq.mmq_plan(2048, 4096, 4096, LARGE_LDS)
    assert p["tile"] == mmq.MMQ_TILE_LARGE
    with pytest.raises(mmq.MMQError) as e:
        mmq.mmq_plan(2048, 4096, 4096, SMALL_LDS - 1)
    assert e.value.status == mmq.MMQ_E_LDS


SKINNY = mmq.MMQ_TILE_SKINNY
GEMV = mmq.MMQ_TILE_GEMV
MEDIUM = mmq.MMQ_TILE_MEDIUM
HALF = mmq.MMQ_TILE_HALF
REASON = {LARGE: mmq.MMQ_REASON_LARGE, SMALL: mmq.MMQ_REASON_SMALL_GRID,
          MEDIUM: mmq.MMQ_REASON_SMALL_GRID, HALF: mmq.MMQ_REASON_SMALL_GRID,
          SKINNY: mmq.MMQ_REASON_FEW_TOKENS, GEMV: mmq.MMQ_REASON_DECODE}


@pytest.mark.parametrize("M,N,tile", [
    (1, 4096, GEMV),        # decode: the vector-ALU form of the decode tile
    (8, 4096, GEMV),
    (1, 65536, GEMV),       # whatever the large grid would be
    (9, 4096, GEMV),        # the matrix-unit form
    (16, 4096, GEMV),
    (17, 4096, SKINNY),     # large grid 1 x 16, few tokens
    (128, 4096, SKINNY),
    (256, 4096, SKINNY),
    (257, 4096, SMALL),     # 3 x 16
    (512, 4096, MEDIUM),    # 4 x 16 = 64 < 256 compute units; 32 x 256 tiles: 16 x 16
    (768, 4096, HALF),      # 6 x 16 = 96; 64 x 256 tiles: 12 x 16
    (1024, 4096, HALF),     # 8 x 16 = 128; 16 x 16
    (256, 11008, HALF),     # 2 x 43 = 86; 4 x 43
    (2048, 4096, LARGE),    # 16 x 16 = 256
    (1024, 11008, LARGE),   # 8 x 43 = 344
    (128, 65536, LARGE),    # 1 x 256
    (8192, 4096, LARGE),
])
def test_plan_prefers_a_grid_that_fills_the_gpu(M, N, tile):
    p = mmq.mmq_plan(M, N, 4096, 160 * 1024)
    assert p["tile"] == tile and p["reason"] == REASON[tile]
    assert p["fallback"] == 0


@pytest.mark.parametrize("M,N,K,tile", [
    (128, 256, 512, SMALL),     # 2 super-blocks for the skinny kernel's 8 wavefronts
    (32, 4096, 1792, SMALL),    # 7
    (32, 4096, 2048, SKINNY),   # 8: one each
    (128, 256, 2048, SKINNY),
])
def test_plan_skinny_needs_a_super_block_per_wavefront(M, N, K, tile):
    assert mmq.mmq_plan(M, N, K, 160 * 1024)["tile"] == tile


def test_plan_min_workgroups_option():
    assert mmq.mmq_plan(512, 4096, 4096, 160 * 1024, min_workgroups=64)["tile"] == LARGE
    p = mmq.mmq_plan(512, 4096, 4096, 160 * 1024, min_workgroups=65)
    assert p["tile"] in (SMALL, MEDIUM, HALF) and p["grid"] >= 65
    assert mmq.mmq_plan(64, 4096, 4096, 160 * 1024, min_workgroups=16)["tile"] == LARGE
    p = mmq.mmq_plan(2048, 4096, 4096, 160 * 1024, min_workgroups=257)
    assert p["tile"] in (SMALL, MEDIUM, HALF) and p["grid"] >= 257


def test_plan_skinny_tile():
    p = mmq.mmq_plan(16, 4096, 4096, 160 * 1024, force_tile=mmq.MMQ_TILE_SKINNY)
    assert p["tile"] == mmq.MMQ_TILE_SKINNY and p["reason"] == mmq.MMQ_REASON_FORCED
    assert p["block_m"] == 32 and p["block_n"] == 32 and p["threads"] == 512
    assert p["lds_bytes"] == 8 * 16 * 65 * 4 and p["grid"] == 1 * 128
    p = mmq.mmq_plan(70, 100, 512, 160 * 1024, force_tile=mmq.MMQ_TILE_SKINNY)
    assert p["grid"] == 3 * 4
    with pytest.raises(mmq.MMQError) as e:
        mmq.mmq_plan(16, 4096, 4096, 160 * 1024, force_tile=mmq.MMQ_TILE_SKINNY,
                     opt_lds_budget=8 * 16 * 65 * 4 - 1)
    assert e.value.status == mmq.MMQ_E_LDS


def test_blockdots_refuse_the_skinny_tile():
    opt = mmq.mmq_options(mmq.MMQ_TILE_SKINNY, 0, 0)
    assert mmq.raw_call("mmq_q4K_q8_1_blockdots", 4, 8, 256, A, B, 0, 4, 0, 8, Cp, None,
                        ctypes.byref(opt)) == mmq.MMQ_E_ARG


def test_blockdots_refuse_the_gemv_tile():
    opt = mmq.mmq_options(mmq.MMQ_TILE_GEMV, 0, 0)
    assert mmq.raw_call("mmq_q4K_q8_1_blockdots", 4, 8, 256, A, B, 0, 4, 0, 8, Cp, None,
                        ctypes.byref(opt)) == mmq.MMQ_E_ARG


# the matrix-unit form's LDS per wavefront: its expanded weight scales per 16-row half (dsv
# [8][16] f32, dmv pieces [3][16][8]), its partial sums [16 tokens][rows] and its super-block's
# token bytes [16][256], (da, nda) pairs [8][16] and pieces [3][16][8]
def mfma_wave_lds(rows):
    return rows // 16 * (512 + 768) + 16 * rows * 4 + 16 * 256 + 8 * 16 * 8 + 3 * 16 * 16


MFMA_WAVE_LDS = mfma_wave_lds(16)
MFMA_GEMV_LDS = 16 * MFMA_WAVE_LDS


def dot_lds(group):
    """The vector-ALU form, per wavefront and K-slice: its half's 128 token bytes and 4
    (da, sa) pairs per token, 16 padding."""
    return 8 * 4 * (160 * group + 16)


@pytest.mark.parametrize("M,N,group,grid,waves,rows", [
    (1, 4096, 1, 256, 0, 16), (2, 4096, 2, 256, 0, 16), (3, 4096, 4, 256, 0, 16),
    (4, 4096, 4, 256, 0, 16), (2, 11008, 2, 688, 0, 16), (4, 11008, 4, 688, 0, 16),
    # up to 4 tokens the vector ALU; from 5 the matrix unit, whose N/16 workgroups fit 256
    # compute units once: 16 wavefronts
    (5, 4096, 16, 256, 16, 16), (8, 4096, 16, 256, 16, 16), (16, 4096, 16, 256, 16, 16),
    # N/32 workgroups fit once: 32 rows, 8 wavefronts
    (5, 4097, 16, 129, 8, 32), (9, 8192, 16, 256, 8, 32), (16, 5120, 16, 160, 8, 32),
    # beyond: 16 rows, 4 wavefronts
    (9, 8208, 16, 513, 4, 16), (8, 11008, 16, 688, 4, 16), (16, 11008, 16, 688, 4, 16),
    (5, 16400, 16, 1025, 4, 16)])
def test_plan_gemv_tile(M, N, group, grid, waves, rows):
    auto = mmq.mmq_plan(M, N, 4096, 160 * 1024)
    assert (auto["tile"], auto["reason"]) == (GEMV, mmq.MMQ_REASON_DECODE)
    p = mmq.mmq_plan(M, N, 4096, 160 * 1024, force_tile=GEMV)
    assert p["tile"] == GEMV
    assert p["block_m"] == group and p["block_n"] == rows
    assert p["threads"] == (512 if waves == 0 else 64 * waves)
    lds = dot_lds(group) if waves == 0 else waves * mfma_wave_lds(rows)
    assert p["lds_bytes"] == lds and p["grid"] == grid


@pytest.mark.parametrize("M,N,waves,rows", [(8, 4096, 16, 16), (5, 4096, 16, 16),
                                            (5, 4097, 8, 32), (7, 8192, 8, 32)])
def test_plan_gemv_form_falls_back_within_the_budget(M, N, waves, rows):
    """5-8 tokens take the vector-ALU form where the matrix-unit form's LDS (at the shape the
    row blocks call for) does not fit."""
    need = waves * mfma_wave_lds(rows)
    group = 8
    p = mmq.mmq_plan(M, N, 4096, 160 * 1024, opt_lds_budget=need - 1)
    assert p["tile"] == GEMV and p["threads"] == 512 and p["block_m"] == group
    assert p["lds_bytes"] == dot_lds(group)
    p = mmq.mmq_plan(M, N, 4096, 160 * 1024, opt_lds_budget=need)
    assert p["tile"] == GEMV and p["threads"] == 64 * waves and p["block_m"] == 16
    assert p["block_n"] == rows


def test_plan_gemv_matrix_form_only_from_9_tokens():
    # from 9 tokens only the matrix-unit form serves: below its LDS another tile is taken
    p = mmq.mmq_plan(9, 4096, 4096, 160 * 1024, opt_lds_budget=MFMA_GEMV_LDS - 1)
    assert p["tile"] != GEMV
    # at 5-8 tokens with 4 wavefronts (32 KiB) the vector-ALU form (40.5 KiB) needs more, and
    # so does every other tile
    with pytest.raises(mmq.MMQError) as e:
        mmq.mmq_plan(8, 11008, 4096, 160 * 1024, opt_lds_budget=4 * MFMA_WAVE_LDS - 1)
    assert e.value.status == mmq.MMQ_E_LDS


def test_plan_above_decode_tile_is_skinny():
    """From 17 tokens the guard leaves the decode tile for the skinny one (K >= 2048)."""
    p = mmq.mmq_plan(17, 4096, 4096, 160 * 1024)
    assert (p["tile"], p["reason"]) == (SKINNY, mmq.MMQ_REASON_FEW_TOKENS)


def test_plan_gemv_forced_limits():
    p = mmq.mmq_plan(16, 4096, 4096, 160 * 1024, force_tile=GEMV)
    assert p["tile"] == GEMV and p["reason"] == mmq.MMQ_REASON_FORCED
    with pytest.raises(mmq.MMQError) as e:
        mmq.mmq_plan(17, 4096, 4096, 160 * 1024, force_tile=GEMV)
    assert e.value.status == mmq.MMQ_E_SHAPE
    with pytest.raises(mmq.MMQError) as e:
        mmq.mmq_plan(8, 8192, 4096, 160 * 1024, force_tile=GEMV, opt_lds_budget=41471)
    assert e.value.status == mmq.MMQ_E_LDS
    # the vector-ALU tile needs the least LDS: under 6 KiB it is the only one that fits
    p = mmq.mmq_plan(1, 4096, 4096, 160 * 1024, opt_lds_budget=5632)
    assert p["tile"] == GEMV and p["lds_bytes"] == 5632
    with pytest.raises(mmq.MMQError) as e:
        mmq.mmq_plan(1, 4096, 4096, 160 * 1024, opt_lds_budget=5631)
    assert e.value.status == mmq.MMQ_E_LDS


def test_plan_forced_tiles():
    p = mmq.mmq_plan(16, 4096, 4096, 160 * 1024, force_tile=mmq.MMQ_TILE_LARGE)
    assert p["tile"] == mmq.MMQ_TILE_LARGE and p["reason"] == mmq.MMQ_REASON_FORCED
    p = mmq.mmq_plan(2048, 4096, 4096, 160 * 1024, force_tile=mmq.MMQ_TILE_SMALL)
    assert p["tile"] == mmq.MMQ_TILE_SMALL and p["reason"] == mmq.MMQ_REASON_FORCED
    with pytest.raises(mmq.MMQError) as e:   # a forced tile over budget is refused, not swapped
        mmq.mmq_plan(2048, 4096, 4096, 160 * 1024, force_tile=mmq.MMQ_TILE_LARGE,
                     opt_lds_budget=LARGE_LDS - 1)
    assert e.value.status == mmq.MMQ_E_LDS
    # the option's budget overrides the argument
    p = mmq.mmq_plan(2048, 4096, 4096, 160 * 1024, opt_lds_budget=SMALL_LDS)
    assert p["tile"] == mmq.MMQ_TILE_SMALL and p["lds_budget"] == SMALL_LDS


def test_plan_ragged_grid():
    p = mmq.mmq_plan(2047, 11008, 4096, 160 * 1024)
    assert p["grid"] == 16 * 43
    p = mmq.mmq_plan(1, 33, 256, 160 * 1024)
    assert p["grid"] == 3 and p["tile"] == GEMV       # 33 rows: three blocks of 16
    p = mmq.mmq_plan(1, 33, 256, 160 * 1024, force_tile=mmq.MMQ_TILE_SKINNY)
    assert p["grid"] == 2
    p = mmq.mmq_plan(1, 33, 256, 160 * 1024, force_tile=mmq.MMQ_TILE_SMALL)
    assert p["grid"] == 1


@pytest.mark.parametrize("args,status", [
    ((0, 4096, 4096), mmq.MMQ_E_ARG),
    ((16, 4096, 4000), mmq.MMQ_E_SHAPE),
    ((16, -5, 4096), mmq.MMQ_E_ARG),
    ((1 << 20, 64, 4096), mmq.MMQ_E_SHAPE),
    ((4, 64, 1 << 25), mmq.MMQ_E_SHAPE),
])
def test_plan_shape_errors(args, status):
    info = mmq.mmq_kernel_info()
    assert mmq.raw_call("mmq_plan", *args, None, 65536, ctypes.byref(info)) == status


# well-formed-looking device addresses (never dereferenced: validation fails first)
A = 0x10000000
B = 0x20000000
Cp = 0x30000000


@pytest.mark.parametrize("call,status", [
    (("quantize_q8_1", None, 4, 64, B, None), mmq.MMQ_E_ARG),
    (("quantize_q8_1", A, 4, 64, None, None), mmq.MMQ_E_ARG),
    (("quantize_q8_1", A + 4, 4, 64, B, None), mmq.MMQ_E_ARG),
    (("quantize_q8_1", A, 4, 48, B, None), mmq.MMQ_E_SHAPE),
    (("quantize_q8_1", A, 0, 64, B, None), mmq.MMQ_E_ARG),
    (("repack_q4_K", A, 4, 200, B, None), mmq.MMQ_E_SHAPE),
    (("repack_q4_K", None, 4, 256, B, None), mmq.MMQ_E_ARG),
    (("repack_q4_K", A, 4, 256, B + 8, None), mmq.MMQ_E_ARG),
    (("quantize_q8_1", A, 1 << 20, 1 << 14, B, None), mmq.MMQ_E_SHAPE),   # M*K = 2^34
    (("repack_q4_K", A, 1 << 30, 1 << 14, B, None), mmq.MMQ_E_SHAPE),     # 2^25 x 64 workgroups
    (("mmq_q4K_q8_1", 4, 8, 100, A, B, Cp, None), mmq.MMQ_E_SHAPE),
    (("mmq_q4K_q8_1", 4, 8, 256, None, B, Cp, None), mmq.MMQ_E_ARG),
    (("mmq_q4K_q8_1", 4, 8, 256, A, B, Cp + 4, None), mmq.MMQ_E_ARG),
    (("mmq_q4K_q8_1", 0, 8, 256, A, B, Cp, None), mmq.MMQ_E_ARG),
    (("mmq_q4K_q8_1_blockdots", 4, 8, 256, A, B, 0, 5, 0, 8, Cp, None, None), mmq.MMQ_E_SHAPE),
    (("mmq_q4K_q8_1_blockdots", 4, 8, 256, A, B, 2, 2, 0, 8, Cp, None, None), mmq.MMQ_E_SHAPE),
    (("mmq_q4K_q8_1_blockdots", 4, 8, 256, A, B, 0, 4, -1, 8, Cp, None, None), mmq.MMQ_E_SHAPE),
    (("mmq_q4K_q8_1_blockdots", 4, 8, 256, A, B, 0, 4, 0, 8, None, None, None), mmq.MMQ_E_ARG),
    (("mmq_q4K_f32", 129, 8, 256, A, B, Cp, None), mmq.MMQ_E_SHAPE),     # few tokens only
    (("mmq_q4K_f32", 4, 8, 100, A, B, Cp, None), mmq.MMQ_E_SHAPE),
    (("mmq_q4K_f32", 4, 8, 256, None, B, Cp, None), mmq.MMQ_E_ARG),
    (("mmq_q4K_f32", 4, 8, 256, A + 4, B, Cp, None), mmq.MMQ_E_ARG),
    (("mmq_q4K_f32", 0, 8, 256, A, B, Cp, None), mmq.MMQ_E_ARG),
])
def test_hot_path_validation(call, status):
    assert mmq.raw_call(*call) == status
    assert mmq.mmq_last_error() != ""


def test_bad_options_rejected():
    bad = mmq.mmq_options(7, 0, 0)
    assert mmq.raw_call("mmq_q4K_q8_1_ex", 4, 8, 256, A, B, Cp, None, ctypes.byref(bad)) == mmq.MMQ_E_ARG
    neg = mmq.mmq_options(0, 0, -1)
    assert mmq.raw_call("mmq_q4K_q8_1_ex", 4, 8, 256, A, B, Cp, None, ctypes.byref(neg)) == mmq.MMQ_E_ARG
    neg_wg = mmq.mmq_options(0, -1, 0)
    assert mmq.raw_call("mmq_q4K_q8_1_ex", 4, 8, 256, A, B, Cp, None,
                        ctypes.byref(neg_wg)) == mmq.MMQ_E_ARG


def test_status_strings():
    for s in range(6):
        assert mmq.mmq_status_str(s).startswith("MMQ_")
    assert "unknown" in mmq.mmq_status_str(99)


# ---------------------------------------------------------------- the f16 comparator path
def test_f16_sizes():
    assert mmq.mmq_f16_bytes(2048, 4096) == 2 * 2048 * 4096
    assert mmq.mmq_f16_bytes(1, 1) == 2
    assert mmq.mmq_f16_bytes(3, 5) == 30
    n = ctypes.c_size_t()
    assert mmq.raw_call("mmq_f16_bytes", 0, 8, ctypes.byref(n)) == mmq.MMQ_E_ARG
    assert mmq.raw_call("mmq_f16_bytes", 1 << 31, 8, ctypes.byref(n)) == mmq.MMQ_E_SHAPE
    assert mmq.raw_call("mmq_f16_bytes", 4, 8, None) == mmq.MMQ_E_ARG


@pytest.mark.parametrize("call,status", [
    (("convert_f32_f16", None, 4, 64, B, None), mmq.MMQ_E_ARG),
    (("convert_f32_f16", A, 4, 64, None, None), mmq.MMQ_E_ARG),
    (("convert_f32_f16", A + 4, 4, 64, B, None), mmq.MMQ_E_ARG),
    (("convert_f32_f16", A, 4, 64, B + 2, None), mmq.MMQ_E_ARG),
    (("convert_f32_f16", A, 0, 64, B, None), mmq.MMQ_E_ARG),
    (("convert_f32_f16", A, 4, -1, B, None), mmq.MMQ_E_ARG),
    (("dequantize_q4_K_f16", A, 4, 200, B, None), mmq.MMQ_E_SHAPE),
    (("dequantize_q4_K_f16", None, 4, 256, B, None), mmq.MMQ_E_ARG),
    (("dequantize_q4_K_f16", A, 4, 256, B + 8, None), mmq.MMQ_E_ARG),
    (("dequantize_q4_K_f16", A, 0, 256, B, None), mmq.MMQ_E_ARG),
    (("gemm_f16", 0, 8, 16, A, B, Cp, None), mmq.MMQ_E_ARG),
    (("gemm_f16", 4, 8, 12, A, B, Cp, None), mmq.MMQ_E_SHAPE),        # K % 8
    (("gemm_f16", 1 << 20, 8, 1 << 10, A, B, Cp, None), mmq.MMQ_E_SHAPE),  # M*K = 2^30
    (("gemm_f16", 4, 1 << 21, 1 << 9, A, B, Cp, None), mmq.MMQ_E_SHAPE),   # N*K = 2^30
    (("gemm_f16", 4, 8, 16, None, B, Cp, None), mmq.MMQ_E_ARG),
    (("gemm_f16", 4, 8, 16, A, B + 8, Cp, None), mmq.MMQ_E_ARG),
    (("gemm_f16", 4, 8, 16, A, B, Cp + 4, None), mmq.MMQ_E_ARG),
])
def test_f16_path_validation(call, status):
    assert mmq.raw_call(*call) == status
    assert mmq.mmq_last_error() != ""


@pytest.mark.parametrize("call", [
    ("convert_f32_f16", A, 4, 64, B, None),
    ("dequantize_q4_K_f16", A, 4, 256, B, None),
    ("gemm_f16", 4, 8, 16, A, B, Cp, None),
])
def test_f16_path_reaches_the_device_check(call):
    # well-formed arguments pass validation; without a GPU the device check refuses them
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the call would run")
    assert mmq.raw_call(*call) == mmq.MMQ_E_DEVICE


def test_fused_path_reaches_the_device_check():
    # M = 128 is the largest accepted; without a GPU the device check refuses the call
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the call would run")
    assert mmq.raw_call("mmq_q4K_f32", 128, 8, 256, A, B, Cp, None) == mmq.MMQ_E_DEVICE


# ---------------------------------------------------------------- the binding's tensor checks
def _t(n, dtype=None):
    import torch
    return torch.zeros(n, dtype=dtype or torch.uint8)


def test_binding_refuses_unfit_tensors():
    """Each wrapper checks type, dtype, contiguity and byte size (and, on a GPU machine, that the
    tensor is on the current CUDA device) before calling the library, which cannot check
    buffer sizes itself."""
    import torch
    M, N, K = 4, 40, 256
    q8 = _t(mmq.mmq_q8_1_bytes(M, K))
    rep = _t(mmq.mmq_q4K_repacked_bytes(N, K))
    C = _t(M * N, torch.float32)
    x = _t(M * K, torch.float32)
    bad = [
        lambda: mmq.mmq_q4K_q8_1(M, N, K, q8[:-1], rep, C),                  # q8 one byte short
        lambda: mmq.mmq_q4K_q8_1(M, N, K, q8, rep[:-16], C),                 # w_rep short
        lambda: mmq.mmq_q4K_q8_1(M, N, K, q8, rep, C[:-1]),                  # C short
        lambda: mmq.mmq_q4K_q8_1(M, N, K, q8, rep, C.to(torch.float16)),     # C not f32
        lambda: mmq.mmq_q4K_q8_1(M, N, K, q8, rep, C.view(M, N).t()),        # C not contiguous
        lambda: mmq.mmq_q4K_q8_1(M, N, K, 12345, rep, C),                    # not a tensor
        lambda: mmq.quantize_q8_1(x.to(torch.float64), M, K, q8),            # x not f32
        lambda: mmq.quantize_q8_1(x[:-1], M, K, q8),
        lambda: mmq.repack_q4_K(_t(mmq.mmq_q4K_bytes(N, K) - 1), N, K, rep),
        lambda: mmq.mmq_q4K_f32(M, N, K, x.view(M, K)[:, ::2], rep, C),
        lambda: mmq.mmq_q4K_q8_1_blockdots(M, N, K, q8, rep, 0, M, 0, N,
                                           _t(K // 32 * M * N, torch.int32)[:-1]),
        lambda: mmq.mmq_q4K_q8_1_blockdots(M, N, K, q8, rep, 0, M, 0, N,
                                           _t(K // 32 * M * N, torch.float32)),
        lambda: mmq.convert_f32_f16(x, M, K, _t(2 * M * K - 1)),
        lambda: mmq.gemm_f16(M, N, K, _t(2 * M * K), _t(2 * N * K), C[:-1]),
    ]
    for i, call in enumerate(bad):
        with pytest.raises(mmq.MMQArgumentError):
            call()
    # well-sized host tensors pass every check but the device one
    with pytest.raises(mmq.MMQArgumentError, match="CUDA tensor"):
        mmq.mmq_q4K_q8_1(M, N, K, q8, rep, C)


# ---------------------------------------------------------------- split-K planning
MEDIUM = mmq.MMQ_TILE_MEDIUM


@pytest.mark.parametrize("M,N,K", [(128, 4096, 11008), (2048, 512, 4096), (2048, 512, 11008),
                                   (256, 4096, 11008), (64, 4096, 11008)])
def test_plan_splits_with_a_workspace(M, N, K):
    p = mmq.mmq_plan(M, N, K, 160 * 1024, workspace_bytes=1 << 40)
    assert p["reason"] == mmq.MMQ_REASON_SPLIT_K and p["splits"] > 1
    assert p["splits"] <= K // 256 and p["splits"] & (p["splits"] - 1) == 0
    assert p["workspace_bytes"] == p["splits"] * M * N * 4
    assert mmq.mmq_workspace_bytes(M, N, K) == p["workspace_bytes"]
    gm = -(-M // p["block_m"])
    gn = -(-N // p["block_n"])
    assert p["grid"] == gm * gn * p["splits"]
    # without a workspace the same product is not split
    q = mmq.mmq_plan(M, N, K, 160 * 1024)
    assert q["splits"] == 1 and q["workspace_bytes"] == 0


@pytest.mark.parametrize("M,N,K", [(2048, 4096, 4096), (2048, 11008, 4096), (8192, 4096, 4096),
                                   (1, 4096, 4096), (16, 4096, 4096)])
def test_plan_does_not_split_what_fills_the_gpu(M, N, K):
    p = mmq.mmq_plan(M, N, K, 160 * 1024, workspace_bytes=1 << 40)
    assert p["splits"] == 1 and p["workspace_bytes"] == 0
    assert mmq.mmq_workspace_bytes(M, N, K) == 0


def test_plan_splits_within_the_workspace():
    M, N, K = 2048, 512, 11008
    full = mmq.mmq_plan(M, N, K, 160 * 1024, workspace_bytes=1 << 40)
    half = mmq.mmq_plan(M, N, K, 160 * 1024, workspace_bytes=full["workspace_bytes"] // 2)
    assert 1 < half["splits"] < full["splits"]
    assert half["workspace_bytes"] <= full["workspace_bytes"] // 2
    one = mmq.mmq_plan(M, N, K, 160 * 1024, workspace_bytes=2 * M * N * 4 - 1)
    assert one["splits"] == 1


def test_forced_splits():
    p = mmq.mmq_plan(150, 300, 2816, 160 * 1024, force_tile=MEDIUM, splits=11,
                     workspace_bytes=11 * 150 * 300 * 4)
    assert p["tile"] == MEDIUM and p["splits"] == 11 and p["grid"] == 5 * 2 * 11
    p = mmq.mmq_plan(150, 300, 2816, 160 * 1024, force_tile=MEDIUM, splits=1)
    assert p["splits"] == 1 and p["workspace_bytes"] == 0


@pytest.mark.parametrize("kw", [
    dict(force_tile=MEDIUM, splits=12, workspace_bytes=1 << 30),   # 11 super-blocks only
    dict(splits=2, workspace_bytes=1 << 30),                        # split-K needs a tile
    dict(force_tile=mmq.MMQ_TILE_SKINNY, splits=2, workspace_bytes=1 << 30),
    dict(force_tile=MEDIUM, splits=2, workspace_bytes=2 * 150 * 300 * 4 - 1),  # no room
    dict(splits=-1),
    dict(workspace_bytes=-1),
])
def test_split_option_errors(kw):
    with pytest.raises(mmq.MMQError) as e:
        mmq.mmq_plan(150, 300, 2816, 160 * 1024, **kw)
    assert e.value.status == mmq.MMQ_E_ARG


def test_reserved_option_must_be_zero():
    bad = mmq.mmq_options(0, 0, 0, None, 0, 0, 1)
    info = mmq.mmq_kernel_info()
    assert mmq.raw_call("mmq_plan", 128, 256, 512, ctypes.byref(bad), 65536,
                        ctypes.byref(info)) == mmq.MMQ_E_ARG


def test_ex_refuses_a_workspace_size_without_a_pointer():
    opt = mmq.mmq_options(0, 0, 0, None, 1 << 20, 0, 0)
    assert mmq.raw_call("mmq_q4K_q8_1_ex", 128, 256, 512, A, B, Cp, None,
                        ctypes.byref(opt)) == mmq.MMQ_E_ARG
    opt = mmq.mmq_options(0, 0, 0, B + 8, 1 << 20, 0, 0)
    assert mmq.raw_call("mmq_q4K_q8_1_ex", 128, 256, 512, A, B, Cp, None,
                        ctypes.byref(opt)) == mmq.MMQ_E_ARG


# ---------------------------------------------------------------- the static-scratch entry point
@pytest.mark.parametrize("call,status", [
    (("mmq_q4K_q8_1_static", 4, 8, 100, A, B, Cp, None, None), mmq.MMQ_E_SHAPE),
    (("mmq_q4K_q8_1_static", 4, 8, 256, None, B, Cp, None, None), mmq.MMQ_E_ARG),
    (("mmq_q4K_q8_1_static", 4, 8, 256, A, B, Cp + 4, None, None), mmq.MMQ_E_ARG),
    (("mmq_q4K_q8_1_static", 0, 8, 256, A, B, Cp, None, None), mmq.MMQ_E_ARG),
])
def test_static_entry_validation(call, status):
    assert mmq.raw_call(*call) == status
    assert mmq.mmq_last_error() != ""


def test_static_entry_refuses_a_workspace_and_oversized_splits():
    opt = mmq.mmq_options(0, 0, 0, B, 1 << 20, 0, 0)
    assert mmq.raw_call("mmq_q4K_q8_1_static", 128, 256, 512, A, B, Cp, None,
                        ctypes.byref(opt)) == mmq.MMQ_E_ARG
    # 4 splits of 256 x 16384 floats are 64 MiB
    opt = mmq.mmq_options(mmq.MMQ_TILE_MEDIUM, 0, 0, None, 0, 4, 0)
    assert mmq.raw_call("mmq_q4K_q8_1_static", 256, 16384, 1024, A, B, Cp, None,
                        ctypes.byref(opt)) == mmq.MMQ_E_ARG
    assert "32 MiB" in mmq.mmq_last_error()
    # more splits than super-blocks, on the largest output: refused before any device access
    # (and before the size of their planes is formed)
    opt = mmq.mmq_options(mmq.MMQ_TILE_MEDIUM, 0, 0, None, 0, (1 << 31) - 1, 0)
    assert mmq.raw_call("mmq_q4K_q8_1_static", 1 << 20, 1 << 20, 1024, A, B, Cp, None,
                        ctypes.byref(opt)) == mmq.MMQ_E_ARG
    assert "super-blocks" in mmq.mmq_last_error()


def test_static_entry_reaches_the_device_check():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the call would run")
    assert mmq.raw_call("mmq_q4K_q8_1_static", 128, 256, 512, A, B, Cp, None,
                        None) == mmq.MMQ_E_DEVICE
