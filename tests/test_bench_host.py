"""Host-side arithmetic of bench.py's report (no GPU)."""
import bench


def test_epilogue_ceiling_at_qproj():
    e = bench.epilogue_ceiling(2048, 4096, 4096, 87.83)
    # 2 FMAs per element-block, 2048*4096*128 element-blocks, 2 flops per FMA, 157.3 TFLOP/s
    assert abs(e["floor_us"] - 2 * 2048 * 4096 * 128 * 2 / 157.3e12 * 1e6) < 0.01
    assert abs(e["floor_us"] - 27.3) < 0.05
    # the GEMM rate that floor allows: 2*M*N*K ops in floor_us, against 5000 TOP/s
    assert abs(e["ceiling_frac_of_int8_peak"] - 0.5034) < 1e-3
    assert abs(e["gemm_frac_of_ceiling"] - 27.3 / 87.83) < 1e-3


def test_sizes_in_the_report_match_the_library():
    # the quantize's algorithmic bytes: f32 in, the q8 buffer out
    import q4_q8_int8_amd as mmq
    assert bench.quant_bytes(2048, 4096) == 4 * 2048 * 4096 + mmq.mmq_q8_1_bytes(2048, 4096)
