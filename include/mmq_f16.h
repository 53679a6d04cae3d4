/*
 * mmq_f16.h -- C ABI of the float16 comparator path of libmmq.so, beside the q4_K x q8_1
 * integer product of mmq.h: the weights are dequantized to f16, the activations converted to
 * f16, and the product is taken by an f16 matrix-core GEMM with float32 accumulation.
 *
 * On the r15 page ("f32-accumulate mma probe + rank-1 term2 rescale", section 5) and the r12
 * page ("16-chain warp tile + ldmatrix", sections 1 and 5) this f16 path is the default
 * prefill path that the integer product is measured against. The audit page "Round 31 Track
 * C Audit: dq_f16 & DW<F>" (sections 1-2) describes its dequantize step (dq_f16): quantized
 * weights in, an f16 weight matrix out, a kernel bound by writing that matrix. It is a
 * comparator, not a replacement: f16 rounds the activations to 11 significant bits, so its
 * result is checked against the exact product of its own f16 operands, not against the
 * integer product's result.
 *
 * The conventions of mmq.h hold here too: DEVICE pointers owned by the caller, 16-byte
 * aligned, not overlapping; `stream` is a hipStream_t; every argument is validated on the
 * host before anything is launched; return values are mmq_status codes; mmq_last_error
 * reports the calling thread's last error.
 */
#ifndef MMQ_F16_H
#define MMQ_F16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of a row-major f16 matrix rows x K: 2*rows*K (host only). rows, K >= 1. */
int mmq_f16_bytes(int64_t rows, int64_t K, size_t* bytes);

/*
 * convert_f32_f16: x[M][K] float32 -> x_f16[M][K] float16 (row-major, leading dimension K),
 * each value rounded to the nearest f16, ties to even, with f16 subnormals; magnitudes of
 * 65520 and above become infinity. The activation side of the f16 path.
 * Errors: MMQ_E_ARG (null or misaligned pointer, M or K <= 0), MMQ_E_SHAPE (M*K above 2^40),
 *         MMQ_E_DEVICE, MMQ_E_HIP.
 */
int convert_f32_f16(const float* x, int64_t M, int64_t K, void* x_f16, void* stream);

/*
 * dequantize_q4_K_f16: q4_K weights (the GGUF layout of mmq.h, [N][K/256] super-blocks of 144
 * bytes) -> w_f16[N][K] float16, row-major. The dq_f16 step of the audit page (sections 1-2)
 * for the q4_K format, whose fields the r15 page gives (section 2.1): per sub-block b of 32,
 *   w = dsv*v + dmv,  dsv = d*sc, dmv = -(dmin*m)
 * evaluated in float32 (dsv*v is exact, so the sum is rounded once) and then rounded to the
 * nearest f16, ties to even.
 * Errors: MMQ_E_ARG, MMQ_E_SHAPE (K % 256), MMQ_E_DEVICE, MMQ_E_HIP.
 */
int dequantize_q4_K_f16(const void* w_q4K, int64_t N, int64_t K, void* w_f16, void* stream);

/*
 * gemm_f16: C[M][N] (float32, row-major, overwritten) = sum_k x_f16[i][k] * w_f16[j][k]
 * for row-major f16 operands x_f16[M][K] and w_f16[N][K], on the f16 matrix instruction
 * (v_mfma_f32_32x32x16_f16) with float32 accumulation. Each product of two f16 values is
 * exact in float32; the order of the float32 additions is fixed by the kernel (deterministic).
 * Preconditions: K % 8 == 0 (rows of whole 16-byte words); M*K and N*K below 2^30.
 * Errors: MMQ_E_ARG (null or misaligned pointer, M, N or K <= 0), MMQ_E_SHAPE, MMQ_E_LDS (the
 *         device allows less than the kernel's 144 KiB of LDS), MMQ_E_DEVICE, MMQ_E_HIP.
 */
int gemm_f16(int64_t M, int64_t N, int64_t K, const void* x_f16, const void* w_f16, float* C,
             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MMQ_F16_H */
