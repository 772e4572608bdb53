// fp8_mfma_probe.hip -- test instrument: evaluates 64-term fp8 dot products
// with the fp8 matrix instruction the fp8 attention kernel uses
// (v_mfma_f32_32x32x64_f8f6f4, E4M3 operands, no block scaling), so that
// tests/test_gpu_fp8_mfma.py can compare its sums with exact ones.
//
// Case c: bytes a[64 c .. 64 c + 63] and b[64 c .. 64 c + 63] are E4M3
// codes; every row of the A operand holds a and every column of B holds b,
// so each element of the 32 x 32 result is sum_k a_k b_k; out[c] gets
// element (0, 0).  Operand layout: lane l holds the 32 consecutive k values
// 32 (l / 32) .. 32 (l / 32) + 31 of its row (A) or column (B), four per
// register, low byte first.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(64) void fp8_dot_kernel(const uint8_t *a, const uint8_t *b, float *out) {
    const int c = blockIdx.x, l = threadIdx.x;
    const uint32_t *ac = reinterpret_cast<const uint32_t *>(a + (int64_t)c * 64 + 32 * (l / 32));
    const uint32_t *bc = reinterpret_cast<const uint32_t *>(b + (int64_t)c * 64 + 32 * (l / 32));
    i32x8 A, B;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        A[w] = (int)ac[w];
        B[w] = (int)bc[w];
    }
    const f32x16 z = {};
    const f32x16 r = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, z, 0, 0, 0, 0, 0, 0);
    if (l == 0) out[c] = r[0];
}

// a, b: device arrays of 64 n bytes; out: device array of n floats.
// Returns 0, or -1 for a bad argument or launch failure.
extern "C" int fp8_mfma_probe(const void *a, const void *b, float *out, int n, hipStream_t stream) {
    if (n < 0 || (n > 0 && (!a || !b || !out))) return -1;
    if (n == 0) return 0;
    hipLaunchKernelGGL(fp8_dot_kernel, dim3((unsigned)n), dim3(64), 0, stream, static_cast<const uint8_t *>(a),
                       static_cast<const uint8_t *>(b), out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
