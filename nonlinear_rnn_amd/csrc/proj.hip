// Input projection GEMM on the CDNA4 matrix cores.
//
//   xproj[m, n] = sum_k x[m, k] W[n, k] + bias[n],  m = (b, t), n = (gate, channel)
//
// Tiling: a 256-thread workgroup computes a 128 x 128 output tile; its four
// waves each own a 64 x 64 quadrant made of 2 x 2 blocks of 32 x 32.  K is
// walked in stages of 128 bytes of every row: the stage's x rows and W rows
// share one LDS buffer, double buffered, with the next stage's global loads
// in flight while the current one is multiplied.
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
//
// Two kernels share this operand layout and k order (so they produce the
// same bits):
//   k_proj_dl  large problems.  A 1024-thread workgroup computes a 256 x 256
//              tile (16 waves, each a 64 x 64 quadrant).  Operands go from
//              global memory straight into LDS (global_load_lds_dwordx4: lane
//              l of a wave's load lands at LDS base + 16 l), with no register
//              staging and no LDS store instructions; two 128-byte K stages
//              are double buffered (128 KB of LDS, one workgroup per CU).
//              LDS rows are unpadded; the 16-byte chunk kv of row r sits at
//              position kv ^ ((r / 2) % 8), which spreads the 32 rows one
//              matrix-instruction operand read touches over all banks.
//              Rows past M or N load the last row (their results are not
//              stored); chunks past K load a zero chunk.  Those guards live
//              in a separate instance (EDGE): problems that tile exactly run
//              without them (the guarded instance took 1.22 ms against 1.14
//              at the size below).  Results are stored non-temporally (they
//              are not read again by this kernel).
//              At 262144 x 1024 x 256 fp32: 1.12 ms against 1.31 ms for
//              k_proj; bf16 at 262144 x 1536 x 512: 0.58 against 0.88 ms.
//   k_proj     grids too small to fill the device with 256 x 256 tiles
//              (128 x 128 tiles, 256 threads, operands staged through
//              registers into padded LDS rows).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "proj.h"

namespace prn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int WM = 2, WN = 2;                       // 32x32 blocks per wave (rows, columns)
constexpr int WR = 2, WC = 2;                       // waves per workgroup (rows, columns)
constexpr int BM = WR * WM * 32, BN = WC * WN * 32;  // workgroup tile: 128 x 128
constexpr int ROWB = 128;                           // bytes of one row per K stage
constexpr int LDS_ROW = ROWB + 16;                  // LDS row stride (bytes), padded
constexpr int VPR = ROWB / 16;                      // 16-byte vectors per row per stage
constexpr int NTHR = 64 * WR * WC;
constexpr int NROWS = BM + BN;                      // A rows then B rows in one LDS buffer
constexpr int VPT = NROWS * VPR / NTHR;             // vectors per thread per stage
constexpr int NXCD = 8;
static_assert(NROWS * VPR % NTHR == 0, "a stage must split evenly over the workgroup");

// round to nearest even; NaN stays a quiet NaN (branch-free)
__device__ __forceinline__ uint16_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t q = (u >> 16) | 0x40u;
  return static_cast<uint16_t>((u & 0x7fffffffu) > 0x7f800000u ? q : r);
}

template <bool BF16>
__global__ void __launch_bounds__(NTHR)
k_proj(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, const float* __restrict__ bias,
       uint8_t* __restrict__ C, int64_t M, int64_t N, int64_t K, int n_tiles_n, int remap) {
  constexpr int ELT = BF16 ? 2 : 4;  // bytes per element
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][NROWS * LDS_ROW];

  // block -> tile, keeping the column tiles of a row tile on one XCD
  int64_t bid = blockIdx.x;
  if (remap) {
    const int64_t per = gridDim.x / NXCD;
    bid = (bid % NXCD) * per + bid / NXCD;
  }
  const int64_t m0 = (bid / n_tiles_n) * BM, n0 = (bid % n_tiles_n) * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / WC, wc = wave % WC;
  const int64_t rowbytes = K * ELT;

  // global -> register staging of one K stage: rows [0, BM) of the tile come
  // from x, rows [BM, BM + BN) from W
  f32x4 rv[VPT];
  auto gload = [&](int64_t kt) {
#pragma unroll
    for (int p = 0; p < VPT; ++p) {
      const int v = tid + p * NTHR;
      const int r = v / VPR, kv = v % VPR;
      const int64_t kbyte = kt * ROWB + kv * 16;
      const bool kin = kbyte < rowbytes;
      if (r < BM) {
        const int64_t g = m0 + r;
        rv[p] = (kin && g < M) ? *reinterpret_cast<const f32x4*>(A + g * rowbytes + kbyte) : f32x4{0, 0, 0, 0};
      } else {
        const int64_t g = n0 + (r - BM);
        rv[p] = (kin && g < N) ? *reinterpret_cast<const f32x4*>(B + g * rowbytes + kbyte) : f32x4{0, 0, 0, 0};
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < VPT; ++p) {
      const int v = tid + p * NTHR;
      const int r = v / VPR, kv = v % VPR;
      *reinterpret_cast<f32x4*>(&lds[buf][r * LDS_ROW + kv * 16]) = rv[p];
    }
  };

  // bias of this lane's output columns, loaded up front (the epilogue must
  // not wait on a load between its stores)
  float bcol[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int64_t gn = n0 + wc * WN * 32 + j * 32 + (lane & 31);
    bcol[j] = (bias && gn < N) ? bias[gn] : 0.0f;
  }

  f32x16 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t nk = (rowbytes + ROWB - 1) / ROWB;
  gload(0);
  lstore(0);
  __syncthreads();
  const int half = lane >> 5, l32 = lane & 31;
  const int arow = wr * WM * 32 + l32;       // this lane's A row (block i adds 32 i)
  const int brow = BM + wc * WN * 32 + l32;  // this lane's B row (block j adds 32 j)
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* L = lds[cur];
#pragma unroll
    for (int kb = 0; kb < VPR / 2; ++kb) {  // 32 bytes of k per step: two 16-byte halves
      const int off = kb * 32 + half * 16;
      f32x4 av[WM], bv[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) av[i] = *reinterpret_cast<const f32x4*>(L + (arow + 32 * i) * LDS_ROW + off);
#pragma unroll
      for (int j = 0; j < WN; ++j) bv[j] = *reinterpret_cast<const f32x4*>(L + (brow + 32 * j) * LDS_ROW + off);
      if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[i]),
                                                                __builtin_bit_cast(bf16x8, bv[j]), acc[i][j], 0, 0, 0);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int i = 0; i < WM; ++i)
#pragma unroll
            for (int j = 0; j < WN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i][s], bv[j][s], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: bias, round to the storage dtype, store (bounds checks only
  // for tiles that overhang M or N)
  auto put = [&](int64_t gm, int64_t gn, float v) {
    if constexpr (BF16)
      reinterpret_cast<uint16_t*>(C)[gm * N + gn] = bf16_rne(v);
    else
      reinterpret_cast<float*>(C)[gm * N + gn] = v;
  };
  const bool full = m0 + BM <= M && n0 + BN <= N;
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int64_t gn = n0 + wc * WN * 32 + j * 32 + l32;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t gm = m0 + wr * WM * 32 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (full || (gm < M && gn < N)) put(gm, gn, acc[i][j][r] + bcol[j]);
      }
    }
  }
}

// ---- large problems: 256 x 256 tiles, direct global -> LDS operand loads ----
constexpr int DL_WR = 4, DL_WC = 4;                      // waves (rows, columns): 16 waves
constexpr int DL_BM = DL_WR * WM * 32, DL_BN = DL_WC * WN * 32;  // 256 x 256
constexpr int DL_NTHR = 64 * DL_WR * DL_WC;
constexpr int DL_ROWB = 128;                             // bytes of every row per K stage
constexpr int DL_CPR = DL_ROWB / 16;                     // 16-byte chunks per row
constexpr int DL_RPG = 16 / DL_CPR;                      // rows per 256 bytes (64 banks)
constexpr int DL_NROWS = DL_BM + DL_BN;
constexpr int DL_STAGE = DL_NROWS * DL_ROWB;
constexpr int DL_IPW = DL_STAGE / 1024 / (DL_WR * DL_WC);  // 1 KB wave loads per wave per stage
constexpr int64_t DL_MIN_TILES = 1024;                   // below this, k_proj's smaller tiles fill the device better
static_assert(DL_STAGE % (1024 * DL_WR * DL_WC) == 0, "a stage must split evenly over the waves");

__device__ __attribute__((aligned(16))) const uint32_t kZeroChunk[4] = {0, 0, 0, 0};

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

__device__ __forceinline__ int dl_pos(int r, int kv) { return kv ^ ((r / DL_RPG) & (DL_CPR - 1)); }

template <bool BF16, bool EDGE>
__global__ void __launch_bounds__(DL_NTHR)
k_proj_dl(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, const float* __restrict__ bias,
          uint8_t* __restrict__ C, int64_t M, int64_t N, int64_t K, int n_tiles_n, int remap) {
  constexpr int ELT = BF16 ? 2 : 4;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * DL_STAGE];
  int64_t bid = blockIdx.x;
  if (remap) {
    const int64_t per = gridDim.x / NXCD;
    bid = (bid % NXCD) * per + bid / NXCD;
  }
  const int64_t m0 = (bid / n_tiles_n) * DL_BM, n0 = (bid % n_tiles_n) * DL_BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / DL_WC, wc = wave % DL_WC;
  const int64_t rowbytes = K * ELT;

  // the chunk each of this lane's loads fetches: wave load p fills LDS bytes
  // [1024 (wave IPW + p), +1024) of a stage, lane l the 16 bytes at 16 l,
  // i.e. position q of row r with 16 (r CPR + q) = 1024 (wave IPW + p) + 16 l
  const uint8_t* src[DL_IPW];
  int kvb[DL_IPW];
#pragma unroll
  for (int p = 0; p < DL_IPW; ++p) {
    const int v = (wave * DL_IPW + p) * 64 + lane;
    const int r = v / DL_CPR, q = v % DL_CPR;
    kvb[p] = dl_pos(r, q) * 16;
    int64_t g = r < DL_BM ? m0 + r : n0 + r - DL_BM;
    if (EDGE) g = r < DL_BM ? (g < M ? g : M - 1) : (g < N ? g : N - 1);
    src[p] = (r < DL_BM ? A : B) + g * rowbytes + kvb[p];
  }
  auto issue = [&](int64_t kt, int buf) {
    uint8_t* base = lds + buf * DL_STAGE + wave * DL_IPW * 1024;
#pragma unroll
    for (int p = 0; p < DL_IPW; ++p) {
      const void* g = src[p] + kt * DL_ROWB;
      if (EDGE && kt * DL_ROWB + kvb[p] >= rowbytes) g = kZeroChunk;
      __builtin_amdgcn_global_load_lds((gptr_t)g, (lptr_t)(base + p * 1024), 16, 0, 0);
    }
  };

  float bcol[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int64_t gn = n0 + wc * WN * 32 + j * 32 + (lane & 31);
    bcol[j] = (bias && (!EDGE || gn < N)) ? bias[gn] : 0.0f;
  }
  f32x16 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t nk = (rowbytes + DL_ROWB - 1) / DL_ROWB;
  const int half = lane >> 5, l32 = lane & 31;
  issue(0, 0);
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    // this wave's loads of stage kt have landed and its reads of the other
    // buffer are done; after the barrier the same holds for every wave.  (A
    // bare barrier: a workgroup fence would also wait for nothing more.)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + 1 < nk) issue(kt + 1, cur ^ 1);
    const uint8_t* L = lds + cur * DL_STAGE;
#pragma unroll
    for (int kb = 0; kb < DL_CPR / 2; ++kb) {
      const int kv = kb * 2 + half;
      f32x4 av[WM], bv[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const int r = wr * WM * 32 + i * 32 + l32;
        av[i] = *reinterpret_cast<const f32x4*>(L + r * DL_ROWB + 16 * dl_pos(r, kv));
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int r = DL_BM + wc * WN * 32 + j * 32 + l32;
        bv[j] = *reinterpret_cast<const f32x4*>(L + r * DL_ROWB + 16 * dl_pos(r, kv));
      }
      if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[i]),
                                                                __builtin_bit_cast(bf16x8, bv[j]), acc[i][j], 0, 0, 0);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int i = 0; i < WM; ++i)
#pragma unroll
            for (int j = 0; j < WN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i][s], bv[j][s], acc[i][j], 0, 0, 0);
      }
    }
  }

  const bool full = !EDGE || (m0 + DL_BM <= M && n0 + DL_BN <= N);
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int64_t gn = n0 + wc * WN * 32 + j * 32 + l32;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t gm = m0 + wr * WM * 32 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const float v = acc[i][j][r] + bcol[j];
        if (full || (gm < M && gn < N)) {
          if constexpr (BF16)
            __builtin_nontemporal_store(bf16_rne(v), reinterpret_cast<uint16_t*>(C) + gm * N + gn);
          else
            __builtin_nontemporal_store(v, reinterpret_cast<float*>(C) + gm * N + gn);
        }
      }
    }
  }
}

}  // namespace

void launch_proj(bool bf16, const void* A, const void* B, const float* bias, void* C, int64_t M, int64_t N,
                 int64_t K, hipStream_t stream) {
  const int64_t dl_tn = (N + DL_BN - 1) / DL_BN, dl_nb = ((M + DL_BM - 1) / DL_BM) * dl_tn;
  if (dl_nb >= DL_MIN_TILES) {
    const int remap = (dl_nb % NXCD == 0) ? 1 : 0;
    const dim3 grid(static_cast<unsigned>(dl_nb));
    const bool edge = M % DL_BM != 0 || N % DL_BN != 0 || (K * (bf16 ? 2 : 4)) % DL_ROWB != 0;
    auto go = [&](auto bf, auto ed) {
      k_proj_dl<decltype(bf)::value, decltype(ed)::value><<<grid, DL_NTHR, 0, stream>>>(
          static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(B), bias, static_cast<uint8_t*>(C), M, N, K,
          int(dl_tn), remap);
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    if (bf16) {
      if (edge) go(T_{}, T_{}); else go(T_{}, F_{});
    } else {
      if (edge) go(F_{}, T_{}); else go(F_{}, F_{});
    }
    return;
  }
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
