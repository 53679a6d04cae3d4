"""Host-side arithmetic of bench.py's report (no GPU)."""
import bench


def test_epilogue_ceiling_at_qproj():
    e = bench.epilogue_ceiling(2048, 4096, 4096, 87.83)
    # 2 FMAs per element-block, 2048*4096*128 element-blocks, 2 flops per FMA, at the
    # non-packed FP32 rate of 78.6 TFLOP/s (16 FMA lanes per SIMD per cycle)
    assert abs(e["floor_us"] - 2 * 2048 * 4096 * 128 * 2 / 78.6e12 * 1e6) < 0.01
    assert abs(e["floor_us"] - 54.6) < 0.1
    # the GEMM rate that floor allows: 2*M*N*K ops in floor_us, against 5000 TOP/s
    assert abs(e["ceiling_frac_of_int8_peak"] - 0.2515) < 1e-3
    assert abs(e["gemm_frac_of_ceiling"] - e["floor_us"] / 87.83) < 1e-3
    # and at the FMA rate measured at the GEMM's occupancy (67.8 TFLOP/s)
    assert abs(e["floor_at_occupancy_us"] - 2 * 2048 * 4096 * 128 * 2 / 67.8e12 * 1e6) < 0.01


def test_sizes_in_the_report_match_the_library():
    # the quantize's algorithmic bytes: f32 in, the q8 buffer out
    import q4_q8_int8_amd as mmq
    assert bench.quant_bytes(2048, 4096) == 4 * 2048 * 4096 + mmq.mmq_q8_1_bytes(2048, 4096)
