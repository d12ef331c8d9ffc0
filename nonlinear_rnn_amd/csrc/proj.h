// Input projection (the only dense contraction of the path): xproj = x W^T + bias.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prn {

// C[M, N] = A[M, K] * B[N, K]^T + bias[N]; A, B, C row-major, K contiguous.
// bf16 = false: fp32 storage; fp32-accurate products on the bf16 matrix
//               cores (six products of exact three-term bf16 splits,
//               bf16split.h), fp32 accumulation.
// bf16 = true : bf16 storage, bf16 products with fp32 accumulation, result
//               rounded to bf16 (nearest even).
// Requires K % 4 == 0 (fp32) or K % 8 == 0 (bf16) and 16-byte aligned A, B, C.
void launch_proj(bool bf16, const void* A, const void* B, const float* bias, void* C, int64_t M, int64_t N,
                 int64_t K, hipStream_t stream);

// The same product without bias, with operand rows lda / ldb bytes apart
// (16-byte multiples, at least K elements).
void launch_proj_ld(bool bf16, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t M,
                    int64_t N, int64_t K, hipStream_t stream);

// Split-K: slice z (0 <= z < splits) multiplies elements [z K, (z+1) K) of
// every operand row and writes its fp32 sums, unrounded, to P + z M N
// (M x N row-major).  128 x 128 tiles.
void launch_proj_splitk(bool bf16, const void* A, int64_t lda, const void* B, int64_t ldb, float* P, int64_t M,
                        int64_t N, int64_t K, int splits, hipStream_t stream);

// Helpers of the projection's backward (elements of the storage dtype):
// out (C x Rp) = the transpose of in (R x C, rows ld_in apart), zero for
// R <= r < Rp; csum (optional, ceil(Rp/64) x C fp32): column sums of every
// 64 input rows, in row order; out may be null.
void launch_transpose(bool bf16, const void* in, int64_t R, int64_t C, int64_t ld_in, void* out, int64_t Rp,
                      float* csum, hipStream_t stream);
// out (R x Cp) = in (R x C) with zero columns appended
void launch_pad_rows(bool bf16, const void* in, int64_t R, int64_t C, void* out, int64_t Cp, hipStream_t stream);
// P[z][n][j] = sum over tokens t of slice z (tokens [z ks, min((z+1) ks, M)))
// of A[t][n] B[t][j]: A tokens x N, B tokens x Kd, rows lda / ldb bytes
// apart, both 16-byte aligned; N and Kd multiples of 256; fp32 sums,
// unrounded (P: splits x N x Kd).  No transposed copies.  csum (optional,
// splits x N): csum[z][n] = the sum of A[t][n] over the tokens of slice z,
// in a fixed order.
void launch_proj_tn(bool bf16, const void* A, int64_t lda, const void* B, int64_t ldb, float* P, int64_t M, int64_t N,
                    int64_t Kd, int64_t ks, int splits, float* csum, hipStream_t stream);
// csum (n_rt x C) = column sums of every 64 rows of in (R x C, row-major,
// zero past R), in row order; in 16-byte aligned, C a multiple of 16 bytes
void launch_colsum64(bool bf16, const void* in, int64_t R, int64_t C, int64_t n_rt, float* csum, hipStream_t stream);
// out[i] = sum_z P[z n + i] in z order, rounded once to the storage dtype
void launch_splitk_sum(bool bf16, const float* P, int S, int64_t n, void* out, hipStream_t stream);

}  // namespace prn
