// Input projection (the only dense contraction of the path): xproj = x W^T + bias.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prn {

// C[M, N] = A[M, K] * B[N, K]^T + bias[N]; A, B, C row-major, K contiguous.
// bf16 = false: fp32 storage, fp32 matrix-core products.
// bf16 = true : bf16 storage, bf16 products with fp32 accumulation, result
//               rounded to bf16 (nearest even).
// Requires K % 4 == 0 (fp32) or K % 8 == 0 (bf16) and 16-byte aligned A, B, C.
void launch_proj(bool bf16, const void* A, const void* B, const float* bias, void* C, int64_t M, int64_t N,
                 int64_t K, hipStream_t stream);

}  // namespace prn
