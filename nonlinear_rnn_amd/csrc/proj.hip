// Input projection GEMM on the CDNA4 matrix cores.
//
//   xproj[m, n] = sum_k x[m, k] W[n, k] + bias[n],  m = (b, t), n = (gate, channel)
//
// Tiling: a 256-thread workgroup computes a 128 x 128 output tile; its four
// waves each own a 64 x 64 quadrant made of 2 x 2 blocks of 32 x 32.  K is
// walked in stages of BK elements (128 bytes of every row): x and W tiles are
// staged through LDS, double buffered, with the next stage's global loads in
// flight while the current one is multiplied.
//
// Operand layout of the 32 x 32 matrix instructions (wave64): lane l feeds
// row (l % 32) of A and column (l % 32) of B; lane half h = l / 32 feeds the
// k values of that half.  Only the pairing of A's and B's k values matters to
// a dot product, so each lane reads 16 contiguous bytes of its LDS row
// (4 fp32 or 8 bf16 k values) and A and B use the same k order.
//   fp32: v_mfma_f32_32x32x2_f32 takes one k per half; the 4 values of a
//         16-byte read feed 4 instructions (k = 8 kb + 4 h + s, s = 0..3).
//   bf16: v_mfma_f32_32x32x16_bf16 takes 8 k per half (k = 16 kb + 8 h + e).
// Result layout: lane l, accumulator r holds row 8 (r / 4) + 4 (l / 32) +
// (r % 4), column l % 32.
//
// Workgroups are numbered so that the column tiles of one row tile run on the
// same XCD (blocks are dealt round-robin to the 8 XCDs), letting that XCD's
// L2 serve the x tile to all of them.
#include <hip/hip_runtime.h>

#include "proj.h"

namespace prn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int BM = 128, BN = 128;
constexpr int ROWB = 128;              // bytes of one row per K stage
constexpr int PADB = 16;               // LDS row padding (bytes)
constexpr int LDS_ROW = ROWB + PADB;   // LDS row stride (bytes)
constexpr int VPR = ROWB / 16;         // 16-byte vectors per row per stage
constexpr int NTHR = 256;
constexpr int VPT = BM * VPR / NTHR;   // vectors per thread per tile per stage
constexpr int NXCD = 8;

__device__ __forceinline__ uint16_t bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <bool BF16>
__global__ void __launch_bounds__(NTHR)
k_proj(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, const float* __restrict__ bias,
       uint8_t* __restrict__ C, int64_t M, int64_t N, int64_t K, int n_tiles_n, int remap) {
  constexpr int ELT = BF16 ? 2 : 4;       // bytes per element
  constexpr int BK = ROWB / ELT;          // k per stage
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][BM * LDS_ROW];

  // block -> tile, keeping the column tiles of a row tile on one XCD
  int64_t bid = blockIdx.x;
  if (remap) {
    const int64_t per = gridDim.x / NXCD;
    bid = (bid % NXCD) * per + bid / NXCD;
  }
  const int64_t tm = bid / n_tiles_n, tn = bid % n_tiles_n;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t rowbytes = K * ELT;

  // global -> register staging of one K stage
  f32x4 ra[VPT], rb[VPT];
  auto gload = [&](int64_t kt) {
#pragma unroll
    for (int p = 0; p < VPT; ++p) {
      const int v = tid + p * NTHR;
      const int r = v / VPR, kv = v % VPR;
      const int64_t kbyte = kt * ROWB + kv * 16;
      const bool kin = kbyte < rowbytes;
      const int64_t gm = m0 + r, gn = n0 + r;
      ra[p] = (kin && gm < M) ? *reinterpret_cast<const f32x4*>(A + gm * rowbytes + kbyte) : f32x4{0, 0, 0, 0};
      rb[p] = (kin && gn < N) ? *reinterpret_cast<const f32x4*>(B + gn * rowbytes + kbyte) : f32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < VPT; ++p) {
      const int v = tid + p * NTHR;
      const int r = v / VPR, kv = v % VPR;
      *reinterpret_cast<f32x4*>(&lds[buf][0][r * LDS_ROW + kv * 16]) = ra[p];
      *reinterpret_cast<f32x4*>(&lds[buf][1][r * LDS_ROW + kv * 16]) = rb[p];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t nk = (K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int half = lane >> 5, l32 = lane & 31;
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* la = lds[cur][0];
    const uint8_t* lb = lds[cur][1];
#pragma unroll
    for (int kb = 0; kb < VPR / 2; ++kb) {  // 32 bytes of k per step: two 16-byte halves
      const int off = kb * 32 + half * 16;
      f32x4 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        av[i] = *reinterpret_cast<const f32x4*>(la + (wr * 64 + i * 32 + l32) * LDS_ROW + off);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bv[j] = *reinterpret_cast<const f32x4*>(lb + (wc * 64 + j * 32 + l32) * LDS_ROW + off);
      if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[i]),
                                                                __builtin_bit_cast(bf16x8, bv[j]), acc[i][j], 0, 0, 0);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i][s], bv[j][s], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: bias, round to the storage dtype, store
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t gn = n0 + wc * 64 + j * 32 + l32;
    const bool nin = gn < N;
    const float bv = (bias && nin) ? bias[gn] : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t gm = m0 + wr * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (nin && gm < M) {
          const float v = acc[i][j][r] + bv;
          if constexpr (BF16)
            reinterpret_cast<uint16_t*>(C)[gm * N + gn] = bf16_rne(v);
          else
            reinterpret_cast<float*>(C)[gm * N + gn] = v;
        }
      }
    }
  }
}

}  // namespace

void launch_proj(bool bf16, const void* A, const void* B, const float* bias, void* C, int64_t M, int64_t N,
                 int64_t K, hipStream_t stream) {
  const int tn = static_cast<int>((N + BN - 1) / BN);
  const int64_t tm = (M + BM - 1) / BM;
  const int64_t nb = tm * tn;
  const int remap = (nb % NXCD == 0) ? 1 : 0;
  const dim3 grid(static_cast<unsigned>(nb));
  if (bf16)
    k_proj<true><<<grid, NTHR, 0, stream>>>(static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(B), bias,
                                           static_cast<uint8_t*>(C), M, N, K, tn, remap);
  else
    k_proj<false><<<grid, NTHR, 0, stream>>>(static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(B), bias,
                                            static_cast<uint8_t*>(C), M, N, K, tn, remap);
}

}  // namespace prn
