// The input projection of one Newton chunk, computed inside the Newton
// workgroup on the matrix cores.
//
// A single-pass Newton workgroup owns LC = LS * NW consecutive steps of one
// row and one 64-channel tile, and keeps that tile's projected inputs
//   xproj[t, g, c] = sum_j x[t, j] W[g d_h + c, j] + bias[g d_h + c]
// (t in the chunk, g a gate, c a channel of the tile) in LDS for all K
// iterations.  Computing the tile here instead of reading it from HBM means
// the projected inputs never travel through HBM at all (the separate
// projection writes them once and the Newton kernel reads them once), and
// the matrix-core work of one resident workgroup overlaps the vector-ALU
// Newton work of another.
//
// The tile is an (LC x 64 G) block of x W^T: LC token rows of x and 64 G rows
// of W.  Both go from global memory straight into LDS (global_load_lds_dwordx4,
// no register round trip) in K stages of 64 bytes per row, through a ring of
// three stage buffers, so that two stages are in flight while a third is
// multiplied; the ring lives in the memory the tile itself occupies
// afterwards (the staging is dead before the first result is written).  Rows
// are unpadded and their four 16-byte chunks are XOR-swizzled by row so that
// 16 consecutive rows read at one k fall in distinct banks.  Each wave owns
// the 32-column blocks cb = w, w + NW, ... and all LC / 32 row blocks.
//
// The products use the instruction, the operand layout and the k order of
// the stand-alone projection kernel (proj.hip): bf16 v_mfma_f32_32x32x16_bf16
// with k = 16 kb + 8 h + e; fp32 the same instruction on the exact bf16
// splits of the operands (bf16split.h), six term products per 16 k in the
// same order, k = 16 ks + 8 h + e; accumulators from 0 and the bias added
// last, so the tile is bitwise the stand-alone projection's output.
#pragma once

#include "bf16split.h"
#include "prn_device.h"

namespace prn {

struct FxArgs {
  const void* x;       // (rows, T, d_in) storage dtype
  const void* W;       // (G d_h, d_in) storage dtype
  const float* bias;   // (G d_h) fp32 or NULL
  int64_t d_in;
  void* xproj_out;     // optional (rows, T, G, d_h) storage dtype: the tile is also stored
};

template <class C, int LS, int NW>
struct FxGeom {
  static constexpr int LC = LS * NW;               // token rows of the tile
  static constexpr int NCOL = C::G * kWave;        // gate-channel columns
  static constexpr int ROWB = 64;                  // bytes of every row per K stage
  static constexpr int CPR = ROWB / 16;            // 16-byte chunks per row per stage
  static constexpr int NROWS = LC + NCOL;          // x rows, then W rows
  static constexpr int STAGE = NROWS * ROWB;
  static constexpr int NBUF = 3;                   // stage ring
  static constexpr int BYTES = NBUF * STAGE;
  static constexpr int NI = STAGE / 1024;          // 1 KB wave loads per stage
  static constexpr int IPW = (NI + NW - 1) / NW;   // wave loads of one wave per stage (at most)
  static constexpr int IPW_MIN = NI / NW;          // (at least)
  static constexpr int NRB = LC / 32;              // 32-row blocks
  static constexpr int NCB_ALL = NCOL / 32;        // 32-column blocks (2 G)
  static constexpr int NCB = (NCB_ALL + NW - 1) / NW;  // column blocks of one wave (at most)
  static_assert(LC % 32 == 0, "the fused projection needs chunks of a multiple of 32 steps");
  static_assert(STAGE % 1024 == 0, "a stage must be whole 1 KB wave loads");
  static_assert(IPW_MIN < 16, "the stage wait encodes at most 15 outstanding loads");
};

// LDS position of 16-byte chunk kv of row r (rows of 64 bytes: four rows
// span the 256 bytes of all banks, so the key changes every four rows)
__device__ __forceinline__ int fx_pos(int r, int kv) { return kv ^ ((r >> 2) & 3); }

// s_waitcnt immediate that waits until at most n vector memory operations
// are outstanding (lgkm and export counts left alone)
constexpr int fx_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// 16 zero bytes: the source of every chunk past T or past d_in
static __device__ __attribute__((aligned(16))) const uint32_t kFxZeroChunk[4] = {0, 0, 0, 0};

typedef __attribute__((address_space(1))) const void* fx_gptr_t;
typedef __attribute__((address_space(3))) void* fx_lptr_t;

typedef __attribute__((ext_vector_type(8))) __bf16 fx_bf16x8;
typedef __attribute__((ext_vector_type(16))) float fx_f32x16;
typedef __attribute__((ext_vector_type(4))) float fx_f32x4;

// Fills xsh[j][g][w * 64 + c] (step t0 + w LS + j of the chunk, gate g,
// channel c of the tile) with the projected input scaled for the gate, as
// load_xs would have read it.  Lanes past d_h take the last channel's row of
// W, so that they compute what the lane they shadow computes.  Must be
// called by every thread of the workgroup (it has workgroup barriers); ends
// with a barrier after which xsh is complete.
template <class C, int DT, int LS, int NW>
__device__ __forceinline__ void fused_tile(uint8_t* lds, const FxArgs& fx, int64_t b, int64_t T, int64_t tc0,
                                           int64_t tile, int64_t d_h, float (*xsh)[C::G][kWave * NW]) {
  using Gm = FxGeom<C, LS, NW>;
  using ST = Storage<DT>;
  constexpr int G = C::G;
  constexpr int ELT = DT == kF32 ? 4 : 2;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int64_t rowbytes = fx.d_in * ELT;
  const uint8_t* X = static_cast<const uint8_t*>(fx.x);
  const uint8_t* Wm = static_cast<const uint8_t*>(fx.W);

  // wave load p of this wave (stage-relative index wl = w + p NW) fills LDS
  // bytes [1024 wl, +1024) of a stage, lane l the 16 bytes at 16 l: row
  // r = (64 wl + l) / 4, position q = l % 4, i.e. chunk kv = fx_pos(r, q) of
  // the row (the same rows every stage; only k moves)
  const uint8_t* src[Gm::IPW];
  int kvb[Gm::IPW];
#pragma unroll
  for (int p = 0; p < Gm::IPW; ++p) {
    const int v = (w + p * NW) * kWave + lane;
    const int r = v / Gm::CPR, q = v % Gm::CPR;
    kvb[p] = fx_pos(r, q) * 16;
    src[p] = nullptr;
    if (r < Gm::LC) {
      const int64_t t = tc0 + r;
      if (t < T) src[p] = X + (b * T + t) * rowbytes + kvb[p];
    } else if (r < Gm::NROWS) {
      const int col = r - Gm::LC, g = col / kWave, c = col % kWave;
      const int64_t ch = imin(tile * kWave + c, d_h - 1);
      src[p] = Wm + (g * d_h + ch) * rowbytes + kvb[p];
    }
  }
  auto issue = [&](int64_t kt, int buf) {
#pragma unroll
    for (int p = 0; p < Gm::IPW; ++p) {
      const int wl = w + p * NW;   // wave-uniform
      if (Gm::NI % NW == 0 || wl < Gm::NI) {
        const void* g = (src[p] && kt * Gm::ROWB + kvb[p] < rowbytes) ? static_cast<const void*>(src[p] + kt * Gm::ROWB)
                                                                      : static_cast<const void*>(kFxZeroChunk);
        // the destination goes through an opaque SGPR copy: the compiler then
        // does not tie the later LDS reads to these writes with a full vmcnt
        // wait of its own; the waits before the stage barrier order them
        fx_lptr_t d = (fx_lptr_t)(lds + buf * Gm::STAGE + wl * 1024);
        asm volatile("" : "+s"(d));
        __builtin_amdgcn_global_load_lds((fx_gptr_t)g, d, 16, 0, 0);
      }
    }
  };

  const int half = lane >> 5, l32 = lane & 31;
  // this wave's column blocks, their gate / channel and bias (loaded ahead:
  // nothing waits on a global load between the results)
  int gcol[Gm::NCB], ccol[Gm::NCB];
  float bcol[Gm::NCB];
#pragma unroll
  for (int j = 0; j < Gm::NCB; ++j) {
    const int cb = w + j * NW;
    const int col = (cb < Gm::NCB_ALL ? cb : 0) * 32 + l32;
    gcol[j] = col / kWave;
    ccol[j] = col % kWave;
    const int64_t ch = imin(tile * kWave + ccol[j], d_h - 1);
    bcol[j] = (fx.bias && cb < Gm::NCB_ALL) ? fx.bias[gcol[j] * d_h + ch] : 0.0f;
  }
  fx_f32x16 acc[Gm::NRB][Gm::NCB];
#pragma unroll
  for (int i = 0; i < Gm::NRB; ++i)
#pragma unroll
    for (int j = 0; j < Gm::NCB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t nk = (rowbytes + Gm::ROWB - 1) / Gm::ROWB;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  for (int64_t kt = 0; kt < nk; ++kt) {
    // this wave's loads of stage kt have landed (those of stage kt + 1 may
    // still be in flight); after the barrier the same holds for every wave,
    // and every wave is done with stage kt - 1, whose buffer takes kt + 2
    asm volatile("" ::: "memory");
    if (kt + 1 < nk)
      __builtin_amdgcn_s_waitcnt(fx_vmcnt(Gm::IPW_MIN));
    else
      __builtin_amdgcn_s_waitcnt(fx_vmcnt(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + 2 < nk) issue(kt + 2, static_cast<int>((kt + 2) % Gm::NBUF));
    const uint8_t* L = lds + static_cast<int>(kt % Gm::NBUF) * Gm::STAGE;
    if constexpr (DT == kF32) {
      // 16 k per stage: half h takes chunks 2 h and 2 h + 1 (k = 16 kt + 8 h + e)
      static_assert(Gm::CPR == 4, "the fp32 split path takes 16 k per stage");
      const int kv = 2 * half;
      sp_bf16x8 bp[Gm::NCB][3];
#pragma unroll
      for (int j = 0; j < Gm::NCB; ++j) {
        const int cb = w + j * NW;
        const int r = Gm::LC + cb * 32 + l32;
        if (cb < Gm::NCB_ALL)
          split3(*reinterpret_cast<const fx_f32x4*>(L + r * Gm::ROWB + 16 * fx_pos(r, kv)),
                 *reinterpret_cast<const fx_f32x4*>(L + r * Gm::ROWB + 16 * fx_pos(r, kv + 1)), bp[j][0], bp[j][1],
                 bp[j][2]);
      }
#pragma unroll
      for (int i = 0; i < Gm::NRB; ++i) {
        const int r = i * 32 + l32;
        sp_bf16x8 ap[3];
        split3(*reinterpret_cast<const fx_f32x4*>(L + r * Gm::ROWB + 16 * fx_pos(r, kv)),
               *reinterpret_cast<const fx_f32x4*>(L + r * Gm::ROWB + 16 * fx_pos(r, kv + 1)), ap[0], ap[1], ap[2]);
#pragma unroll
        for (int t = 0; t < 6; ++t)
#pragma unroll
          for (int j = 0; j < Gm::NCB; ++j)
            if (w + j * NW < Gm::NCB_ALL)
              acc[i][j] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap[kSplitU[t]], bp[j][kSplitV[t]], acc[i][j], 0, 0, 0);
      }
      continue;
    }
#pragma unroll
    for (int kb = 0; kb < Gm::CPR / 2; ++kb) {
      const int kv = kb * 2 + half;
      fx_f32x4 av[Gm::NRB], bv[Gm::NCB];
#pragma unroll
      for (int i = 0; i < Gm::NRB; ++i) {
        const int r = i * 32 + l32;
        av[i] = *reinterpret_cast<const fx_f32x4*>(L + r * Gm::ROWB + 16 * fx_pos(r, kv));
      }
#pragma unroll
      for (int j = 0; j < Gm::NCB; ++j) {
        const int cb = w + j * NW;
        const int r = Gm::LC + cb * 32 + l32;
        if (cb < Gm::NCB_ALL) bv[j] = *reinterpret_cast<const fx_f32x4*>(L + r * Gm::ROWB + 16 * fx_pos(r, kv));
      }
#pragma unroll
      for (int i = 0; i < Gm::NRB; ++i)
#pragma unroll
        for (int j = 0; j < Gm::NCB; ++j)
          if (w + j * NW < Gm::NCB_ALL)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(fx_bf16x8, av[i]),
                                                                __builtin_bit_cast(fx_bf16x8, bv[j]), acc[i][j], 0, 0,
                                                                0);
    }
  }
  __syncthreads();   // every wave is done with the last stage

  // results: the staging is dead (every wave is past the last barrier)
  typename ST::T* xo = static_cast<typename ST::T*>(fx.xproj_out);
#pragma unroll
  for (int j = 0; j < Gm::NCB; ++j) {
    if (w + j * NW >= Gm::NCB_ALL) continue;
    const int g = gcol[j], c = ccol[j];
    const float sc = C::scale(g);
    const bool cok = tile * kWave + c < d_h;
#pragma unroll
    for (int i = 0; i < Gm::NRB; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tau = i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const float v = acc[i][j][r] + bcol[j];
        xsh[tau % LS][g][(tau / LS) * kWave + c] = ST::round(v) * sc;
        if (xo && cok && tc0 + tau < T) xo[((b * T + tc0 + tau) * G + g) * d_h + tile * kWave + c] = ST::pack(v);
      }
    }
  }
  __syncthreads();
}

}  // namespace prn
