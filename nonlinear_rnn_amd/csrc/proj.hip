// Input projection GEMM on the CDNA4 matrix cores.
//
//   xproj[m, n] = sum_k x[m, k] W[n, k] + bias[n],  m = (b, t), n = (gate, channel)
//
// Tiling: each wave owns a 64 x 64 quadrant of the workgroup's tile, made of
// 2 x 2 blocks of 32 x 32.  Large problems (at least 768 tiles of 256 x 256)
// take 256 x 256 tiles of 16 waves (1024 threads, one workgroup per CU);
// smaller ones 128 x 128 tiles of 4 waves, which give the device enough
// workgroups.  K is walked in stages of 128 bytes of every row, double
// buffered in LDS: the x rows and W rows of the next stage are in flight
// while the current one is multiplied.
//
// Operands go from global memory straight into LDS (global_load_lds_dwordx4:
// lane l of a wave's load lands at LDS base + 16 l), with no register staging
// and no LDS store instructions.  LDS rows are unpadded; the 16-byte chunk kv
// of row r sits at position kv ^ ((r / 2) % 8), which spreads the 32 rows one
// matrix-instruction operand read touches over all banks.  The stage barrier
// is a bare s_barrier after an explicit wait for this wave's loads: a
// workgroup fence (__syncthreads) would make the compiler drain every load in
// flight, the next stage's included.
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
// Ragged edges (EDGE instances): rows past M or N load the last row and are
// not stored; chunks past K load a zero chunk.  Problems that tile exactly
// run the instance without these guards (1.13 against 1.22 ms at
// 262144 x 1024 x 256 fp32).  Results are stored non-temporally: this kernel
// never reads them again.
//
// Measured (262144 x 1024 x 256 fp32; 262144 x 1536 x 512 bf16): 1.12 ms and
// 0.57 ms with 256 x 256 tiles, against 1.31 and 0.88 ms for 128 x 128 tiles
// staged through registers into padded LDS rows.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "proj.h"

namespace prn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

constexpr int WM = 2, WN = 2;                  // 32 x 32 blocks per wave (rows, columns)
constexpr int ROWB = 128;                      // bytes of every row per K stage
constexpr int CPR = ROWB / 16;                 // 16-byte chunks per row
constexpr int RPG = 16 / CPR;                  // rows per 256 bytes (64 banks)
constexpr int NXCD = 8;
// 256 x 256 tiles from three per CU on (measured: 65536 x 768 x 256, 768
// tiles, 0.208 ms against 0.215 ms with 128 x 128; 32768 x 768 x 256, 384
// tiles, 0.135 ms against 0.111)
constexpr int64_t kLargeTiles = 768;

__device__ __attribute__((aligned(16))) const uint32_t kZeroChunk[4] = {0, 0, 0, 0};

// LDS position of chunk kv of row r
__device__ __forceinline__ int lds_pos(int r, int kv) { return kv ^ ((r / RPG) & (CPR - 1)); }

// round to nearest even (v_cvt_pk_bf16_f32); NaN stays a quiet NaN
__device__ __forceinline__ uint16_t bf16_rne(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }

template <int WR, int WC>
struct Tile {
  static constexpr int NW = WR * WC;
  static constexpr int BM = WR * WM * 32, BN = WC * WN * 32;
  static constexpr int NTHR = 64 * NW;
  static constexpr int NROWS = BM + BN;          // x rows, then W rows
  static constexpr int STAGE = NROWS * ROWB;
  static constexpr int IPW = STAGE / 1024 / NW;  // 1 KB wave loads per wave per stage
  static_assert(STAGE % (1024 * NW) == 0, "a stage must split evenly over the waves");
};

template <bool BF16, bool EDGE, int WR, int WC>
__global__ void __launch_bounds__(64 * WR * WC)
k_proj(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, const float* __restrict__ bias,
       uint8_t* __restrict__ C, int64_t M, int64_t N, int64_t K, int n_tiles_n, int remap) {
  using Tl = Tile<WR, WC>;
  constexpr int BM = Tl::BM, BN = Tl::BN, IPW = Tl::IPW, STAGE = Tl::STAGE;
  constexpr int ELT = BF16 ? 2 : 4;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];
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

  // the chunk each of this lane's loads fetches: wave load p fills LDS bytes
  // [1024 (wave IPW + p), +1024) of a stage, lane l the 16 bytes at 16 l,
  // i.e. position q of row r with 16 (r CPR + q) = 1024 (wave IPW + p) + 16 l
  const uint8_t* src[IPW];
  int kvb[IPW];
#pragma unroll
  for (int p = 0; p < IPW; ++p) {
    const int v = (wave * IPW + p) * 64 + lane;
    const int r = v / CPR, q = v % CPR;
    kvb[p] = lds_pos(r, q) * 16;
    int64_t g = r < BM ? m0 + r : n0 + r - BM;
    if (EDGE) g = r < BM ? (g < M ? g : M - 1) : (g < N ? g : N - 1);
    src[p] = (r < BM ? A : B) + g * rowbytes + kvb[p];
  }
  auto issue = [&](int64_t kt, int buf) {
    uint8_t* base = lds + buf * STAGE + wave * IPW * 1024;
#pragma unroll
    for (int p = 0; p < IPW; ++p) {
      const void* g = src[p] + kt * ROWB;
      if (EDGE && kt * ROWB + kvb[p] >= rowbytes) g = kZeroChunk;
      __builtin_amdgcn_global_load_lds((gptr_t)g, (lptr_t)(base + p * 1024), 16, 0, 0);
    }
  };

  // bias of this lane's output columns, loaded up front (the epilogue must
  // not wait on a load between its stores)
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

  const int64_t nk = (rowbytes + ROWB - 1) / ROWB;
  const int half = lane >> 5, l32 = lane & 31;
  issue(0, 0);
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    // this wave's loads of stage kt have landed and its reads of the other
    // buffer are done; after the barrier the same holds for every wave
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + 1 < nk) issue(kt + 1, cur ^ 1);
    const uint8_t* L = lds + cur * STAGE;
#pragma unroll
    for (int kb = 0; kb < CPR / 2; ++kb) {  // 32 bytes of k per step: two 16-byte halves
      const int kv = kb * 2 + half;
      f32x4 av[WM], bv[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const int r = wr * WM * 32 + i * 32 + l32;
        av[i] = *reinterpret_cast<const f32x4*>(L + r * ROWB + 16 * lds_pos(r, kv));
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int r = BM + wc * WN * 32 + j * 32 + l32;
        bv[j] = *reinterpret_cast<const f32x4*>(L + r * ROWB + 16 * lds_pos(r, kv));
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

  // epilogue: bias, round to the storage dtype, store
  const bool full = !EDGE || (m0 + BM <= M && n0 + BN <= N);
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

template <int WR, int WC>
void launch_tiles(bool bf16, const void* A, const void* B, const float* bias, void* C, int64_t M, int64_t N,
                  int64_t K, hipStream_t stream) {
  using Tl = Tile<WR, WC>;
  const int64_t tn = (N + Tl::BN - 1) / Tl::BN, nb = ((M + Tl::BM - 1) / Tl::BM) * tn;
  const int remap = (nb % NXCD == 0) ? 1 : 0;
  const bool edge = M % Tl::BM != 0 || N % Tl::BN != 0 || (K * (bf16 ? 2 : 4)) % ROWB != 0;
  const dim3 grid(static_cast<unsigned>(nb));
  auto go = [&](auto bf, auto ed) {
    k_proj<decltype(bf)::value, decltype(ed)::value, WR, WC><<<grid, Tl::NTHR, 0, stream>>>(
        static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(B), bias, static_cast<uint8_t*>(C), M, N, K,
        int(tn), remap);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (bf16) {
    if (edge) go(T_{}, T_{}); else go(T_{}, F_{});
  } else {
    if (edge) go(F_{}, T_{}); else go(F_{}, F_{});
  }
}

}  // namespace

void launch_proj(bool bf16, const void* A, const void* B, const float* bias, void* C, int64_t M, int64_t N,
                 int64_t K, hipStream_t stream) {
  using Large = Tile<4, 4>;
  const int64_t large = ((M + Large::BM - 1) / Large::BM) * ((N + Large::BN - 1) / Large::BN);
  if (large >= kLargeTiles)
    launch_tiles<4, 4>(bf16, A, B, bias, C, M, N, K, stream);
  else
    launch_tiles<2, 2>(bf16, A, B, bias, C, M, N, K, stream);
}

}  // namespace prn
