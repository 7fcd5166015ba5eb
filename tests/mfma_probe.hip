// Test probe for the FP32 leaf's block rule: runs v_mfma_f32_16x16x32_bf16 or
// v_mfma_f32_16x16x32_f16 directly on given operands and accumulator, so the
// rule the oracle declares for a leaf can be checked against the instruction
// itself (test infrastructure; not part of the library).
//
// Case c is one wave.  Lane l holds, for MFMA step s of the case, the 8
// operand values A[row = l % 16][k = 8 (l / 16) .. +8] and B[k = 8 (l / 16)
// .. +8][col = l % 16] at slot (c * steps + s) * 64 + l, and the accumulator
// C / D[row = 4 (l / 16) + i][col = l % 16], i < 4, at slot c * 64 + l.  The
// steps chain: D = mfma(A_s, B_s, D) from D = C.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool F16>
__global__ __launch_bounds__(64) void k_probe(const u16x8 *A, const u16x8 *B, const f32x4 *C, f32x4 *D, int ncases,
                                              int steps) {
  const int c = blockIdx.x, l = threadIdx.x;
  if (c >= ncases) return;
  f32x4 acc = C[c * 64 + l];
  for (int s = 0; s < steps; ++s) {
    const int i = (c * steps + s) * 64 + l;
    if constexpr (F16)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, A[i]), __builtin_bit_cast(f16x8, B[i]),
                                                   acc, 0, 0, 0);
    else
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[i]), __builtin_bit_cast(bf16x8, B[i]),
                                                    acc, 0, 0, 0);
  }
  D[c * 64 + l] = acc;
}

// dtype 0: BF16 operands, 1: FP16.  A, B: ncases * steps * 64 slots of 16
// bytes; C, D: ncases * 64 slots of 16 bytes; device pointers.  Returns a
// hipError_t after the kernel has finished.
extern "C" int mfma_probe(int dtype, const void *A, const void *B, const void *C, void *D, int ncases, int steps) {
  if (ncases <= 0) return 0;
  if (steps < 1 || steps > 64 || ncases > (1 << 20) || (dtype != 0 && dtype != 1)) return (int)hipErrorInvalidValue;
  if (dtype == 1)
    hipLaunchKernelGGL(k_probe<true>, dim3(ncases), dim3(64), 0, 0, (const u16x8 *)A, (const u16x8 *)B,
                       (const f32x4 *)C, (f32x4 *)D, ncases, steps);
  else
    hipLaunchKernelGGL(k_probe<false>, dim3(ncases), dim3(64), 0, 0, (const u16x8 *)A, (const u16x8 *)B,
                       (const f32x4 *)C, (f32x4 *)D, ncases, steps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  return (int)hipDeviceSynchronize();
}
