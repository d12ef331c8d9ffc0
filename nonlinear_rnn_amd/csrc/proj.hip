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
// a dot product, so each lane reads contiguous bytes of its LDS row and A
// and B use the same k order.
//   bf16: v_mfma_f32_32x32x16_bf16 takes 8 k per half (k = 16 kb + 8 h + e),
//         one 16-byte read.
//   fp32: the same bf16 instruction on the exact three-term bf16 splits of
//         the operands (bf16split.h), six term products per 16 k
//         (k = 16 ks + 8 h + e, e = 0..7).  The sums agree with fp32
//         products to fp32 rounding, in 3/8 of the matrix-core time of
//         v_mfma_f32_32x32x2_f32.  The 16-wave tiles split every stage once,
//         cooperatively, into three bf16 term planes in LDS (each value by
//         one thread) and multiply from the planes while the next stage is
//         split; the 4-wave tiles, which have room for the registers but not
//         the LDS of that, split the two 16-byte chunks each lane reads.
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
// staged through registers into padded LDS rows; the fp32 case takes
// 0.75 ms on the split bf16 products from term planes (0.79 ms splitting in
// registers, 1.13 ms on v_mfma_f32_32x32x2_f32).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "bf16split.h"
#include "proj.h"

namespace prn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

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

// LDS address (byte offset) of a pointer into __shared__ memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lptr_t)const_cast<void*>(p)));
}

// One direct-to-LDS load of 16 bytes per lane (lane l lands at LDS byte
// lds + 16 l; lds is wave-uniform, the instruction takes it from M0).
// Issued from asm so that the compiler does not track it: it would make
// every later LDS read wait for all such loads in flight, the next stage's
// included, although the reads touch only the stage buffer that the stage
// barrier has already made complete.  The kernel waits for these loads
// itself (vmcnt(0) before every stage barrier).  M0 written by a scalar
// instruction needs one wait state before the load reads it; nothing else
// in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is a reserved register
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// round to nearest even (v_cvt_pk_bf16_f32); NaN stays a quiet NaN
__device__ __forceinline__ uint16_t bf16_rne(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }


// WR x WC waves, each owning WM x WN blocks of 32 x 32
template <int WR, int WC, int WM_ = 2, int WN_ = 2>
struct Tile {
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int NW = WR * WC;
  static constexpr int BM = WR * WM * 32, BN = WC * WN * 32;
  static constexpr int NTHR = 64 * NW;
  static constexpr int NROWS = BM + BN;          // x rows, then W rows
  static constexpr int STAGE = NROWS * ROWB;
  static constexpr int IPW = STAGE / 1024 / NW;  // 1 KB wave loads per wave per stage
  static_assert(STAGE % (1024 * NW) == 0, "a stage must split evenly over the waves");
};

// OUTF32: store the fp32 sums as they are (no bias, no rounding), for the
// split-K partial products of the weight gradient.  Operand rows are lda /
// ldb bytes apart (16-byte multiples); slice z = blockIdx.y of a split-K
// launch starts K elements into every operand row and writes its own M x N
// block of C.
template <bool BF16, bool EDGE, int WR, int WC, bool OUTF32, int WM, int WN>
__global__ void __launch_bounds__(64 * WR * WC)
k_proj(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, const float* __restrict__ bias,
       uint8_t* __restrict__ C, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int n_tiles_n, int remap) {
  using Tl = Tile<WR, WC, WM, WN>;
  constexpr int BM = Tl::BM, BN = Tl::BN, IPW = Tl::IPW, STAGE = Tl::STAGE;
  constexpr int ELT = BF16 ? 2 : 4;
  // fp32 with 16 waves (PLANES): two K stages of 64 bytes per row, then two
  // sets of the three bf16 term planes of a stage (32 bytes per row each):
  // 320 bytes per row.  Otherwise two K stages of 128 bytes per row.
  constexpr bool PLANES = !BF16 && Tl::NW == 16;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[PLANES ? Tl::NROWS * 320 : 2 * STAGE];
  {
    const int64_t z = blockIdx.y;
    A += z * K * ELT;
    B += z * K * ELT;
    C += z * M * N * (OUTF32 ? 4 : ELT);
  }
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
  //
  // Without edges (EDGE = false) the 64 lanes of a wave load cover 64 / CPR
  // whole rows, which lie all in the x rows or all in the W rows: the first
  // row's address is wave-uniform (scalar registers) and each lane adds a
  // 32-bit offset (fewer vector registers than a 64-bit address per load).
  static_assert(BM % (64 / CPR) == 0, "a wave load must not straddle the x and W rows");
  const uint8_t* src[EDGE ? IPW : 1];
  int kvb[EDGE ? IPW : 1];
  const uint8_t* gbase[EDGE ? 1 : IPW];
  uint32_t voff[EDGE ? 1 : IPW];
#pragma unroll
  for (int p = 0; p < IPW; ++p) {
    const int v = (wave * IPW + p) * 64 + lane;
    const int r = v / CPR, q = v % CPR;
    if constexpr (EDGE) {
      kvb[p] = lds_pos(r, q) * 16;
      int64_t g = r < BM ? m0 + r : n0 + r - BM;
      g = r < BM ? (g < M ? g : M - 1) : (g < N ? g : N - 1);
      src[p] = (r < BM ? A + g * lda : B + g * ldb) + kvb[p];
    } else {
      const int r0 = (wave * IPW + p) * (64 / CPR);
      gbase[p] = r0 < BM ? A + (m0 + r0) * lda : B + (n0 + r0 - BM) * ldb;
      voff[p] = static_cast<uint32_t>((r - r0) * (r0 < BM ? lda : ldb) + lds_pos(r, q) * 16);
    }
  }
  auto issue = [&](int64_t kt, int buf) {
    uint8_t* base = lds + buf * STAGE + wave * IPW * 1024;
#pragma unroll
    for (int p = 0; p < IPW; ++p) {
      const void* g;
      if constexpr (EDGE) {
        g = src[p] + kt * ROWB;
        if (kt * ROWB + kvb[p] >= rowbytes) g = kZeroChunk;
      } else {
        g = gbase[p] + kt * ROWB + voff[p];
      }
      dma16(g, lds_addr(base + p * 1024));
    }
  };

  f32x16 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int half = lane >> 5, l32 = lane & 31;
  if constexpr (!PLANES) {
    const int64_t nk = (rowbytes + ROWB - 1) / ROWB;
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
      if constexpr (BF16) {
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
#pragma unroll
          for (int i = 0; i < WM; ++i)
#pragma unroll
            for (int j = 0; j < WN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, av[i]), __builtin_bit_cast(bf16x8, bv[j]), acc[i][j], 0, 0, 0);
        }
      } else {
        // fp32: 16 k per step, half h takes chunks 4 ks + 2 h and 4 ks + 2 h + 1
        // (k = 16 ks + 8 h + e); six bf16 products per block and step
#pragma unroll
        for (int ks = 0; ks < CPR / 4; ++ks) {
          const int kv = ks * 4 + half * 2;
          bf16x8 bp[WN][3];
#pragma unroll
          for (int j = 0; j < WN; ++j) {
            const int r = BM + wc * WN * 32 + j * 32 + l32;
            split3(*reinterpret_cast<const f32x4*>(L + r * ROWB + 16 * lds_pos(r, kv)),
                   *reinterpret_cast<const f32x4*>(L + r * ROWB + 16 * lds_pos(r, kv + 1)), bp[j][0], bp[j][1],
                   bp[j][2]);
          }
          // the x blocks are split one at a time (registers)
#pragma unroll
          for (int i = 0; i < WM; ++i) {
            const int r = wr * WM * 32 + i * 32 + l32;
            bf16x8 ap[3];
            split3(*reinterpret_cast<const f32x4*>(L + r * ROWB + 16 * lds_pos(r, kv)),
                   *reinterpret_cast<const f32x4*>(L + r * ROWB + 16 * lds_pos(r, kv + 1)), ap[0], ap[1], ap[2]);
#pragma unroll
            for (int t = 0; t < 6; ++t)
#pragma unroll
              for (int j = 0; j < WN; ++j)
                acc[i][j] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap[kSplitU[t]], bp[j][kSplitV[t]], acc[i][j], 0, 0, 0);
          }
          // keep the scheduler from hoisting the next step's reads and splits
          // above these products (their registers would not fit)
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  } else {
    // fp32 with 16 waves (bf16split.h): K stages of 16 k (64 bytes per row) double
    // buffered; every stage is split once, cooperatively (each operand value
    // by one thread, not by each of the four waves that read it), into
    // three bf16 term planes, also double buffered.  While the planes of
    // stage kt are multiplied, the same waves split stage kt + 1 and stage
    // kt + 2 is in flight.  Stage rows: 16-byte chunk kv of row r at
    // position kv ^ ((r / 4) % 4); plane rows: 16 k as two chunks of 8 bf16
    // (k = 8 c + e), chunk c at position c ^ ((r / 8) % 2).
    constexpr int SROW = 64, SCPR = SROW / 16, FST = Tl::NROWS * SROW;
    constexpr int PROW = 32, PLANE = Tl::NROWS * PROW, PST = 3 * PLANE;
    constexpr int IPW2 = FST / 1024 / Tl::NW;
    constexpr int UPT = Tl::NROWS * 2 / Tl::NTHR;   // 8-value units per thread and stage
    static_assert(FST % (1024 * Tl::NW) == 0 && Tl::NROWS * 2 % Tl::NTHR == 0 && IPW2 < 16,
                  "stage split over the waves and threads");
    static_assert(2 * FST + 2 * PST == Tl::NROWS * 320, "LDS layout");
    uint8_t* const Fb = lds;
    uint8_t* const Pb = lds + 2 * FST;
    auto fpos = [](int r, int kv) { return kv ^ ((r >> 2) & 3); };
    auto ppos = [](int r, int c) { return c ^ ((r >> 3) & 1); };
    const uint8_t* src2[IPW2];
    int kvb2[IPW2];
#pragma unroll
    for (int p = 0; p < IPW2; ++p) {
      const int v = (wave * IPW2 + p) * 64 + lane;
      const int r = v / SCPR, q = v % SCPR;
      kvb2[p] = fpos(r, q) * 16;
      int64_t g = r < BM ? m0 + r : n0 + r - BM;
      if (EDGE) g = r < BM ? (g < M ? g : M - 1) : (g < N ? g : N - 1);
      src2[p] = (r < BM ? A + g * lda : B + g * ldb) + kvb2[p];
    }
    auto issue2 = [&](int64_t kt, int buf) {
#pragma unroll
      for (int p = 0; p < IPW2; ++p) {
        const void* g = src2[p] + kt * SROW;
        if (EDGE && kt * SROW + kvb2[p] >= rowbytes) g = kZeroChunk;
        dma16(g, lds_addr(Fb + buf * FST + (wave * IPW2 + p) * 1024));
      }
    };
    auto split_stage = [&](int buf) {
#pragma unroll
      for (int q = 0; q < UPT; ++q) {
        const int v = tid + q * Tl::NTHR;
        const int r = v >> 1, c = v & 1;
        const uint8_t* f = Fb + buf * FST + r * SROW;
        bf16x8 t0, t1, t2;
        split3(*reinterpret_cast<const f32x4*>(f + 16 * fpos(r, 2 * c)),
               *reinterpret_cast<const f32x4*>(f + 16 * fpos(r, 2 * c + 1)), t0, t1, t2);
        uint8_t* d = Pb + buf * PST + r * PROW + 16 * ppos(r, c);
        *reinterpret_cast<bf16x8*>(d) = t0;
        *reinterpret_cast<bf16x8*>(d + PLANE) = t1;
        *reinterpret_cast<bf16x8*>(d + 2 * PLANE) = t2;
      }
    };
    const int64_t nk = (rowbytes + SROW - 1) / SROW;
    issue2(0, 0);
    if (nk > 1) issue2(1, 1);
    asm volatile("" ::: "memory");
    if (nk > 1)
      __builtin_amdgcn_s_waitcnt((IPW2 & 15) | (7 << 4) | (15 << 8));   // vmcnt(IPW2): stage 0 has landed
    else
      __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    split_stage(0);
    for (int64_t kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      // the planes of stage kt are complete and stage kt + 1 has landed;
      // every wave is done with the planes of stage kt - 1 and with the
      // stage buffer of stage kt
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (kt + 2 < nk) issue2(kt + 2, cur);
      if (kt + 1 < nk) split_stage(cur ^ 1);
      // six term products per block: half h takes plane chunk h
      // (k = 16 kt + 8 h + e); the x blocks one at a time (registers)
      const uint8_t* P = Pb + cur * PST;
      bf16x8 bp[WN][3];
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int r = BM + wc * WN * 32 + j * 32 + l32;
#pragma unroll
        for (int u = 0; u < 3; ++u)
          bp[j][u] = *reinterpret_cast<const bf16x8*>(P + u * PLANE + r * PROW + 16 * ppos(r, half));
      }
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const int r = wr * WM * 32 + i * 32 + l32;
        bf16x8 ap[3];
#pragma unroll
        for (int u = 0; u < 3; ++u)
          ap[u] = *reinterpret_cast<const bf16x8*>(P + u * PLANE + r * PROW + 16 * ppos(r, half));
#pragma unroll
        for (int t = 0; t < 6; ++t)
#pragma unroll
          for (int j = 0; j < WN; ++j)
            acc[i][j] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap[kSplitU[t]], bp[j][kSplitV[t]], acc[i][j], 0, 0, 0);
      }
    }
  }

  // epilogue: bias, round to the storage dtype, store.  The bias of this
  // lane's columns is loaded here, before the first store (not held in
  // registers through the main loop, nor awaited between stores)
  float bcol[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int64_t gn = n0 + wc * WN * 32 + j * 32 + (lane & 31);
    bcol[j] = (bias && (!EDGE || gn < N)) ? bias[gn] : 0.0f;
  }
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
          if constexpr (OUTF32)
            reinterpret_cast<float*>(C)[gm * N + gn] = v;
          else if constexpr (BF16)
            __builtin_nontemporal_store(bf16_rne(v), reinterpret_cast<uint16_t*>(C) + gm * N + gn);
          else
            __builtin_nontemporal_store(v, reinterpret_cast<float*>(C) + gm * N + gn);
        }
      }
    }
  }
}

template <int WR, int WC, bool OUTF32, int WM = 2, int WN = 2>
void launch_tiles(bool bf16, const void* A, const void* B, const float* bias, void* C, int64_t M, int64_t N,
                  int64_t K, int64_t lda, int64_t ldb, int splits, hipStream_t stream) {
  using Tl = Tile<WR, WC, WM, WN>;
  const int64_t tn = (N + Tl::BN - 1) / Tl::BN, nb = ((M + Tl::BM - 1) / Tl::BM) * tn;
  const int remap = (nb % NXCD == 0) ? 1 : 0;
  const bool edge = M % Tl::BM != 0 || N % Tl::BN != 0 || (K * (bf16 ? 2 : 4)) % ROWB != 0;
  const dim3 grid(static_cast<unsigned>(nb), static_cast<unsigned>(splits));
  auto go = [&](auto bf, auto ed) {
    k_proj<decltype(bf)::value, decltype(ed)::value, WR, WC, OUTF32, WM, WN><<<grid, Tl::NTHR, 0, stream>>>(
        static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(B), bias, static_cast<uint8_t*>(C), M, N, K,
        lda, ldb, int(tn), remap);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (bf16) {
    if (edge) go(T_{}, T_{}); else go(T_{}, F_{});
  } else {
    if (edge) go(F_{}, T_{}); else go(F_{}, F_{});
  }
}


// Products whose reduction index runs along the operand rows, as in the
// weight gradient dW = dxproj^T x:
//   P[z][n][j] = sum over tokens t of slice z of A[t][n] B[t][j]
// (A: tokens x N, B: tokens x Kd, row-major, rows lda / ldb bytes apart),
// fp32 sums, unrounded; slice z = blockIdx.y covers tokens
// [z ks, min((z + 1) ks, M)) (ks a multiple of the stage).  256 x 256
// output tiles (N and Kd multiples of 256), 16 waves of 64 x 64 as in
// k_proj.  fp32 operands (bf16 ones: k_proj_tn_tr).  A K stage is 16
// tokens: the stage buffer holds, per token, the tile's 256 A values and
// 256 B values (loaded straight into LDS, 1 KB of a row per wave load); the
// split into bf16 term planes (bf16split.h) reads each plane row's 8 tokens
// down a column of the stage, so the planes come out in the layout k_proj's
// planes have, with k = t, and no transposed copy of either operand is ever
// made.  Stages and planes are double buffered as in k_proj.
// csum (optional): csum[z][n] = the sum of A[t][n] over the slice's tokens,
// taken by the workgroups of the first column tile (bid % n_tiles_j == 0)
// on the split, where each value passes one thread: the thread of column n
// and token half h (tokens 16 s + 8 h .. + 7 of every stage s) sums its
// values in token order, and the two halves are added last (h = 0 first).
__global__ void __launch_bounds__(1024)
k_proj_tn(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, float* __restrict__ P, int64_t M, int64_t N,
          int64_t Kd, int64_t lda, int64_t ldb, int64_t ks, int n_tiles_j, float* __restrict__ csum) {
  constexpr int BM = 256, BN = 256, NROWS = BM + BN, NW = 16, NTHR = 64 * NW, WC = 4, WM = 2, WN = 2;
  constexpr int ELT = 4, NPL = 3, NTERM = 6, KS = 16;
  constexpr int FROW = NROWS * ELT, FST = KS * FROW;  // a token's row of the stage; the stage
  constexpr int PCH = KS / 8, PROW = 16 * PCH;        // 16-byte chunks (8 tokens) of a plane row
  constexpr int PLANE = NROWS * PROW, PST = NPL * PLANE;
  constexpr int NLD = FST / 1024, IPW = NLD / NW;     // 1 KB wave loads per stage; per wave
  constexpr int UPT = NROWS * PCH / NTHR;             // split units of each thread per stage
  static_assert(NLD % NW == 0 && IPW < 16 && NROWS * PCH % NTHR == 0, "stage geometry");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * FST + 2 * PST];
  uint8_t* const Fb = lds;
  uint8_t* const Pb = lds + 2 * FST;
  // chunk c of plane row r (rows of 32 bytes) changes key every 8 rows (16
  // consecutive rows read at one chunk: all banks)
  auto ppos = [](int r, int c) { return c ^ ((r >> 3) & 1); };

  const int64_t z = blockIdx.y;
  const int64_t t0 = z * ks, t1 = t0 + ks < M ? t0 + ks : M;
  const int64_t bid = blockIdx.x;
  const int64_t n0 = (bid / n_tiles_j) * BM, j0 = (bid % n_tiles_j) * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / WC, wc = wave % WC;
  const int half = lane >> 5, l32 = lane & 31;
  // this thread's column sum (threads of the A rows, first column tile)
  const bool sums = csum && bid % n_tiles_j == 0 && (tid & (NROWS - 1)) < BM;
  float cs = 0.0f;

  // wave load li = wave IPW + p fills stage bytes [1024 li, +1024): token
  // row 1024 li / FROW of the stage, from byte 1024 li % FROW of that row
  // (its A values first); lane l the 16 bytes at 16 l past that
  const uint8_t* src[IPW];
  int64_t ldr[IPW];
  int trow[IPW];
#pragma unroll
  for (int p = 0; p < IPW; ++p) {
    const int li = wave * IPW + p;
    trow[p] = li * 1024 / FROW;
    const int off = li * 1024 % FROW + 16 * lane;
    const bool in_a = off < BM * ELT;
    src[p] = in_a ? A + n0 * ELT + off : B + j0 * ELT + (off - BM * ELT);
    ldr[p] = in_a ? lda : ldb;
  }
  auto issue = [&](int64_t kt, int buf) {
#pragma unroll
    for (int p = 0; p < IPW; ++p) {
      const int64_t t = t0 + kt * KS + trow[p];
      const void* g = t < t1 ? static_cast<const void*>(src[p] + t * ldr[p]) : static_cast<const void*>(kZeroChunk);
      dma16(g, lds_addr(Fb + buf * FST + (wave * IPW + p) * 1024));
    }
  };
  // unit v: plane row r (A rows, then B rows), tokens 8 kc .. 8 kc + 7 of the stage
  auto split_unit = [&](int buf, int v) {
    const int r = v & (NROWS - 1), kc = v / NROWS;
    const uint8_t* f = Fb + buf * FST + 8 * kc * FROW + r * ELT;
    uint8_t* d = Pb + buf * PST + r * PROW + 16 * ppos(r, kc);
    f32x4 va, vb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      va[e] = *reinterpret_cast<const float*>(f + e * FROW);
      vb[e] = *reinterpret_cast<const float*>(f + (4 + e) * FROW);
    }
    if (sums) {
#pragma unroll
      for (int e = 0; e < 4; ++e) cs += va[e];
#pragma unroll
      for (int e = 0; e < 4; ++e) cs += vb[e];
    }
    bf16x8 h0, h1, h2;
    split3(va, vb, h0, h1, h2);
    *reinterpret_cast<bf16x8*>(d) = h0;
    *reinterpret_cast<bf16x8*>(d + PLANE) = h1;
    *reinterpret_cast<bf16x8*>(d + 2 * PLANE) = h2;
  };
  auto split_stage = [&](int buf) {
#pragma unroll
    for (int q = 0; q < UPT; ++q) split_unit(buf, tid + q * NTHR);
  };

  f32x16 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t nk = (ks + KS - 1) / KS;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  asm volatile("" ::: "memory");
  if (nk > 1)
    __builtin_amdgcn_s_waitcnt((IPW & 15) | (7 << 4) | (15 << 8));   // vmcnt(IPW): stage 0 has landed
  else
    __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  split_stage(0);
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    // the planes of stage kt are complete and stage kt + 1 has landed;
    // every wave is done with the planes of stage kt - 1 and the stage
    // buffer of stage kt
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + 2 < nk) issue(kt + 2, cur);
    if (kt + 1 < nk) split_stage(cur ^ 1);
    const uint8_t* Pl = Pb + cur * PST;
#pragma unroll
    for (int ks2 = 0; ks2 < KS / 16; ++ks2) {
      // 16 tokens per step: half h takes plane chunk 2 ks2 + h
      const int c = 2 * ks2 + half;
      bf16x8 bp[WN][NPL];
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int r = BM + wc * WN * 32 + j * 32 + l32;
#pragma unroll
        for (int u = 0; u < NPL; ++u)
          bp[j][u] = *reinterpret_cast<const bf16x8*>(Pl + u * PLANE + r * PROW + 16 * ppos(r, c));
      }
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const int r = wr * WM * 32 + i * 32 + l32;
        bf16x8 ap[NPL];
#pragma unroll
        for (int u = 0; u < NPL; ++u)
          ap[u] = *reinterpret_cast<const bf16x8*>(Pl + u * PLANE + r * PROW + 16 * ppos(r, c));
#pragma unroll
        for (int t = 0; t < NTERM; ++t)
#pragma unroll
          for (int j = 0; j < WN; ++j)
            acc[i][j] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap[kSplitU[t]], bp[j][kSplitV[t]], acc[i][j], 0, 0, 0);
      }
    }
  }

  if (csum && bid % n_tiles_j == 0) {
    // the two token halves of each column: h = 1 hands its sum over through
    // LDS (the stage buffers are free once every wave has left the loop)
    float* const hand = reinterpret_cast<float*>(lds);
    __syncthreads();
    if (sums && tid >= NROWS) hand[tid - NROWS] = cs;
    __syncthreads();
    if (sums && tid < NROWS) csum[z * N + n0 + tid] = cs + hand[tid];
  }

  // lane l, accumulator r of block (i, j): row n0 + .. + 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
  float* Pz = P + z * N * Kd;
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int64_t gj = j0 + wc * WN * 32 + j * 32 + l32;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t gn = n0 + wr * WM * 32 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        Pz[gn * Kd + gj] = acc[i][j][r];
      }
    }
  }
}

}  // namespace

void launch_proj(bool bf16, const void* A, const void* B, const float* bias, void* C, int64_t M, int64_t N,
                 int64_t K, hipStream_t stream) {
  using Large = Tile<4, 4>;
  const int64_t large = ((M + Large::BM - 1) / Large::BM) * ((N + Large::BN - 1) / Large::BN);
  const int64_t ld = K * (bf16 ? 2 : 4);
  if (large >= kLargeTiles)
    launch_tiles<4, 4, false>(bf16, A, B, bias, C, M, N, K, ld, ld, 1, stream);
  else
    launch_tiles<2, 2, false>(bf16, A, B, bias, C, M, N, K, ld, ld, 1, stream);
}

void launch_proj_ld(bool bf16, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t M,
                    int64_t N, int64_t K, hipStream_t stream) {
  using Large = Tile<4, 4>;
  const int64_t large = ((M + Large::BM - 1) / Large::BM) * ((N + Large::BN - 1) / Large::BN);
  if (large >= kLargeTiles)
    launch_tiles<4, 4, false>(bf16, A, B, nullptr, C, M, N, K, lda, ldb, 1, stream);
  else
    launch_tiles<2, 2, false>(bf16, A, B, nullptr, C, M, N, K, lda, ldb, 1, stream);
}

void launch_proj_splitk(bool bf16, const void* A, int64_t lda, const void* B, int64_t ldb, float* P, int64_t M,
                        int64_t N, int64_t K, int splits, hipStream_t stream) {
  launch_tiles<2, 2, true>(bf16, A, B, nullptr, P, M, N, K, lda, ldb, splits, stream);
}

// ---------------------------------------------- backward helpers ---------

namespace {

template <bool BF16> struct Elt;
template <> struct Elt<false> {
  using T = float;
  static __device__ __forceinline__ float ld(T v) { return v; }
  static __device__ __forceinline__ T st(float v) { return v; }
};
template <> struct Elt<true> {
  using T = uint16_t;
  static __device__ __forceinline__ float ld(T v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
  static __device__ __forceinline__ T st(float v) { return bf16_rne(v); }
};

// out[c, r] = in[r, c] (in: R x C, rows ld_in elements apart; out: C x Rp,
// zero for R <= r < Rp), through a 64 x 64 LDS tile: reads coalesced along
// the input rows, writes along the output rows.  bf16 values pass through
// fp32 exactly.  csum (optional): the column sums of the tile's 64 input
// rows, taken in row order, at csum[blockIdx.x * C + c].  out may be null
// (column sums only).
template <bool BF16>
__global__ void __launch_bounds__(256) k_transpose(const typename Elt<BF16>::T* __restrict__ in, int64_t R, int64_t C,
                                                   int64_t ld_in, typename Elt<BF16>::T* __restrict__ out, int64_t Rp,
                                                   float* __restrict__ csum) {
  using E = Elt<BF16>;
  __shared__ float tile[64][65];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 64, c0 = static_cast<int64_t>(blockIdx.y) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t r = r0 + ty + 4 * i, c = c0 + tx;
    tile[ty + 4 * i][tx] = (r < R && c < C) ? E::ld(in[r * ld_in + c]) : 0.0f;
  }
  __syncthreads();
  if (csum && ty == 0 && c0 + tx < C) {
    float sum = 0.0f;
    for (int i = 0; i < 64; ++i) sum += tile[i][tx];
    csum[static_cast<int64_t>(blockIdx.x) * C + c0 + tx] = sum;
  }
  if (!out) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t c = c0 + ty + 4 * i, r = r0 + tx;
    if (c < C && r < Rp) out[c * Rp + r] = E::st(tile[tx][ty + 4 * i]);
  }
}

// out[r, c] = in[r, c] for c < C, 0 for C <= c < Cp (rows of Cp elements)
template <bool BF16>
__global__ void __launch_bounds__(256) k_pad_rows(const typename Elt<BF16>::T* __restrict__ in, int64_t R, int64_t C,
                                                  typename Elt<BF16>::T* __restrict__ out, int64_t Cp) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= R * Cp) return;
  const int64_t r = i / Cp, c = i - r * Cp;
  out[i] = c < C ? in[r * C + c] : Elt<BF16>::st(0.0f);
}

// The bf16 weight-gradient tile (P as in k_proj_tn, bf16 operands) without a
// repack: the stage keeps the tokens as rows, as loaded, and the operand
// fragments come straight from it through ds_read_b64_tr_b16.  That
// instruction treats each 16 lanes as a group: lane j of the group names an
// 8-byte run (four 16-bit values) and lane i receives value i % 4 of the
// runs named by lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4, in that order
// (checked by an in-bounds probe).  So if lane j names token row
// t0 + j / 4, columns c0 + 4 (j % 4) .. + 3, lane i receives tokens
// t0 .. t0 + 3 of column c0 + i: four consecutive k of one row of the
// operand, half of what a lane holds for a 32 x 32 x 16 product.  The
// fragments hold the same k in the same places as the planes of k_proj_tn,
// so the sums are bitwise the same.  Three 32-token stages (one being read,
// two in flight).  Within a token row the 16-byte chunk c sits at c ^
// swz(t), so the eight rows one transposed read touches (t0 + 0..3 and
// t0 + 8..11) fall into eight different 64-byte segments.  csum (optional)
// as in k_proj_tn: in the workgroups of the first column tile, the thread
// of column n and token quarter q sums tokens 32 s + 8 q .. + 7 of every
// stage s in token order, and the quarters are added last, in order.
__global__ void __launch_bounds__(1024)
k_proj_tn_tr(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, float* __restrict__ P, int64_t M,
             int64_t N, int64_t Kd, int64_t lda, int64_t ldb, int64_t ks, int n_tiles_j, float* __restrict__ csum) {
  constexpr int BM = 256, BN = 256, NROWS = BM + BN, NW = 16, WC = 4, WM = 2, WN = 2;
  constexpr int KS = 32, FROW = NROWS * 2, FST = KS * FROW, NBUF = 3;
  constexpr int NLD = FST / 1024, IPW = NLD / NW;   // a wave load fills one token row (1 KB)
  static_assert(FROW == 1024 && NLD % NW == 0 && IPW < 16, "stage geometry");
  typedef __attribute__((ext_vector_type(4))) short s16x4;
  typedef __attribute__((ext_vector_type(8))) short s16x8;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NBUF * FST];
  auto swz = [](int t) { return 4 * ((t & 3) | (((t >> 3) & 1) << 2)); };

  const int64_t z = blockIdx.y;
  const int64_t t0 = z * ks, t1 = t0 + ks < M ? t0 + ks : M;
  const int64_t bid = blockIdx.x;
  const int64_t n0 = (bid / n_tiles_j) * BM, j0 = (bid % n_tiles_j) * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / WC, wc = wave % WC;
  const int half = lane >> 5, l32 = lane & 31;
  const bool sums = csum && bid % n_tiles_j == 0;   // wave-uniform
  const int scol = tid & (BM - 1), sq = tid / BM;   // this thread's column and token quarter
  float cs = 0.0f;

  // wave load li = wave IPW + p fills token row li of the stage: lane l the
  // 16 bytes at position l, i.e. chunk l ^ swz(li) of the row (chunks 0..31:
  // the A columns n0 .., 32..63: the B columns j0 ..)
  const uint8_t* src[IPW];
  int64_t ldr[IPW];
#pragma unroll
  for (int p = 0; p < IPW; ++p) {
    const int li = wave * IPW + p, c = lane ^ swz(li);
    src[p] = c < 32 ? A + n0 * 2 + 16 * c : B + j0 * 2 + 16 * (c - 32);
    ldr[p] = c < 32 ? lda : ldb;
  }
  auto issue = [&](int64_t kt, int buf) {
#pragma unroll
    for (int p = 0; p < IPW; ++p) {
      const int li = wave * IPW + p;
      const int64_t t = t0 + kt * KS + li;
      const void* g = t < t1 ? static_cast<const void*>(src[p] + t * ldr[p]) : static_cast<const void*>(kZeroChunk);
      dma16(g, lds_addr(lds + buf * FST + li * 1024));
    }
  };
  // this lane's part of a transposed read: group g = lane / 16 takes columns
  // c0 + 16 (g % 2) .. + 15 and tokens 8 (g / 2) .. + 7 of the 16-token step
  const int grp = lane >> 4, jl = lane & 15;
  const int rsub = 8 * (grp >> 1) + (jl >> 2);          // token row within the step, before + 4 call
  const int csub = 16 * (grp & 1) + 4 * (jl & 3);       // column offset within the 32-column block
  auto frag = [&](const uint8_t* st, int step, int c0) {
    s16x8 v;
#pragma unroll
    for (int call = 0; call < 2; ++call) {
      const int t = 16 * step + rsub + 4 * call, col = c0 + csub;
      const uint8_t* a = st + t * FROW + 16 * ((col >> 3) ^ swz(t)) + 2 * (col & 7);
      const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(a));
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * call + e] = r[e];
    }
    return __builtin_bit_cast(bf16x8, v);
  };

  f32x16 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t nk = (ks + KS - 1) / KS;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = static_cast<int>(kt % NBUF);
    // stage kt has landed (stage kt + 1 may still be in flight); every wave
    // is done with the buffer of stage kt - 1, which stage kt + 2 refills
    asm volatile("" ::: "memory");
    if (kt + 1 < nk)
      __builtin_amdgcn_s_waitcnt((IPW & 15) | (7 << 4) | (15 << 8));
    else
      __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + 2 < nk) issue(kt + 2, static_cast<int>((kt + 2) % NBUF));
    const uint8_t* st = lds + cur * FST;
    if (sums) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = 8 * sq + e;
        const uint16_t v = *reinterpret_cast<const uint16_t*>(st + t * FROW + 16 * ((scol >> 3) ^ swz(t)) + 2 * (scol & 7));
        cs += __uint_as_float(static_cast<uint32_t>(v) << 16);
      }
    }
#pragma unroll
    for (int step = 0; step < KS / 16; ++step) {
      bf16x8 bp[WN];
#pragma unroll
      for (int j = 0; j < WN; ++j) bp[j] = frag(st, step, BM + wc * WN * 32 + j * 32);
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const bf16x8 ap = frag(st, step, wr * WM * 32 + i * 32);
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap, bp[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  if (sums) {
    // the four token quarters of each column, added in order
    float* const hand = reinterpret_cast<float*>(lds);
    __syncthreads();
    hand[tid] = cs;
    __syncthreads();
    if (tid < BM) csum[z * N + n0 + tid] = ((hand[tid] + hand[BM + tid]) + hand[2 * BM + tid]) + hand[3 * BM + tid];
  }

  // lane l, accumulator r of block (i, j): row n0 + .. + 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
  float* Pz = P + z * N * Kd;
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int64_t gj = j0 + wc * WN * 32 + j * 32 + l32;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t gn = n0 + wr * WM * 32 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        Pz[gn * Kd + gj] = acc[i][j][r];
      }
    }
  }
}

// csum[rt * C + c] = the sum of in[r][c] over the rows r = 64 rt ..
// 64 rt + 63 (0 at r >= R), in row order: the column sums k_transpose takes.
// A thread sums the 16 bytes of columns at c0 .. (C a multiple of those, in
// 16-byte aligned rows), so every load is a whole 16-byte chunk.
template <bool BF16>
__global__ void __launch_bounds__(256) k_colsum64(const typename Elt<BF16>::T* __restrict__ in, int64_t R, int64_t C,
                                                  float* __restrict__ csum) {
  constexpr int V = 16 / sizeof(typename Elt<BF16>::T);
  const int64_t c0 = (static_cast<int64_t>(blockIdx.y) * 256 + threadIdx.x) * V, r0 = static_cast<int64_t>(blockIdx.x) * 64;
  if (c0 >= C) return;
  float sum[V];
#pragma unroll
  for (int e = 0; e < V; ++e) sum[e] = 0.0f;
  // the rows past R add zeros, which leave a sum that started at +0 unchanged
  const int n = static_cast<int>(R - r0 < 64 ? R - r0 : 64);
  const typename Elt<BF16>::T* src = in + r0 * C + c0;
  for (int i = 0; i < n; ++i, src += C) {
    const uint4 q = *reinterpret_cast<const uint4*>(src);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < V; ++e)
      sum[e] += BF16 ? __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16)) : __uint_as_float(w[e]);
  }
#pragma unroll
  for (int e = 0; e < V; ++e) csum[static_cast<int64_t>(blockIdx.x) * C + c0 + e] = sum[e];
}

// out[i] = the sum over z = 0 .. S-1, in that order, of P[z * n + i],
// rounded once to the storage dtype
template <bool BF16>
__global__ void __launch_bounds__(256) k_splitk_sum(const float* __restrict__ P, int S, int64_t n,
                                                    typename Elt<BF16>::T* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float sum = 0.0f;
  for (int z = 0; z < S; ++z) sum += P[z * n + i];
  out[i] = Elt<BF16>::st(sum);
}

}  // namespace

void launch_transpose(bool bf16, const void* in, int64_t R, int64_t C, int64_t ld_in, void* out, int64_t Rp,
                      float* csum, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((Rp + 63) / 64), static_cast<unsigned>((C + 63) / 64));
  if (bf16)
    k_transpose<true><<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(in), R, C, ld_in,
                                                static_cast<uint16_t*>(out), Rp, csum);
  else
    k_transpose<false><<<grid, 256, 0, stream>>>(static_cast<const float*>(in), R, C, ld_in,
                                                 static_cast<float*>(out), Rp, csum);
}

void launch_pad_rows(bool bf16, const void* in, int64_t R, int64_t C, void* out, int64_t Cp, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((R * Cp + 255) / 256));
  if (bf16)
    k_pad_rows<true><<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(in), R, C, static_cast<uint16_t*>(out), Cp);
  else
    k_pad_rows<false><<<grid, 256, 0, stream>>>(static_cast<const float*>(in), R, C, static_cast<float*>(out), Cp);
}

void launch_proj_tn(bool bf16, const void* A, int64_t lda, const void* B, int64_t ldb, float* P, int64_t M, int64_t N,
                    int64_t Kd, int64_t ks, int splits, float* csum, hipStream_t stream) {
  const int tj = static_cast<int>(Kd / 256);
  const dim3 grid(static_cast<unsigned>((N / 256) * tj), static_cast<unsigned>(splits));
  if (bf16)
    k_proj_tn_tr<<<grid, 1024, 0, stream>>>(static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(B), P, M, N, Kd,
                                            lda, ldb, ks, tj, csum);
  else
    k_proj_tn<<<grid, 1024, 0, stream>>>(static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(B), P, M, N, Kd,
                                         lda, ldb, ks, tj, csum);
}

void launch_colsum64(bool bf16, const void* in, int64_t R, int64_t C, int64_t n_rt, float* csum, hipStream_t stream) {
  const int64_t v = bf16 ? 8 : 4;
  const dim3 grid(static_cast<unsigned>(n_rt), static_cast<unsigned>((C / v + 255) / 256));
  if (bf16)
    k_colsum64<true><<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(in), R, C, csum);
  else
    k_colsum64<false><<<grid, 256, 0, stream>>>(static_cast<const float*>(in), R, C, csum);
}

void launch_splitk_sum(bool bf16, const float* P, int S, int64_t n, void* out, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  if (bf16)
    k_splitk_sum<true><<<grid, 256, 0, stream>>>(P, S, n, static_cast<uint16_t*>(out));
  else
    k_splitk_sum<false><<<grid, 256, 0, stream>>>(P, S, n, static_cast<float*>(out));
}

}  // namespace prn
