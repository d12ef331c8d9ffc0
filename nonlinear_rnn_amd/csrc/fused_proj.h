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
// of W.  Both are staged through LDS in K stages of 64 bytes per row, double
// buffered, in the memory the tile itself occupies afterwards (the staging is
// dead before the first result is written).  Each wave owns the 32-column
// blocks cb = w, w + NW, ... and all LC / 32 row blocks.
//
// The products use the instruction, the operand layout and the k order of
// the stand-alone projection kernel (proj.hip): fp32 v_mfma_f32_32x32x2_f32
// with k = 8 kb + 4 h + s, bf16 v_mfma_f32_32x32x16_bf16 with
// k = 16 kb + 8 h + e, accumulators from 0 and the bias added last, so the
// tile is bitwise the stand-alone projection's output.
#pragma once

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
  static constexpr int LDS_ROW = ROWB + 16;        // padded LDS row
  static constexpr int NROWS = LC + NCOL;          // x rows, then W rows
  static constexpr int STAGE = NROWS * LDS_ROW;
  static constexpr int BYTES = 2 * STAGE;          // double buffered
  static constexpr int NRB = LC / 32;              // 32-row blocks
  static constexpr int NCB_ALL = NCOL / 32;        // 32-column blocks (2 G)
  static constexpr int NCB = (NCB_ALL + NW - 1) / NW;  // column blocks of one wave (at most)
  static_assert(LC % 32 == 0, "the fused projection needs chunks of a multiple of 32 steps");
};

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
  constexpr int VPR = Gm::ROWB / 16;  // 16-byte vectors per row per stage
  constexpr int NT = kWave * NW;
  constexpr int NV = Gm::NROWS * VPR;
  constexpr int VPT = (NV + NT - 1) / NT;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int64_t rowbytes = fx.d_in * ELT;
  const uint8_t* X = static_cast<const uint8_t*>(fx.x);
  const uint8_t* Wm = static_cast<const uint8_t*>(fx.W);

  // the rows this thread stages (same rows every stage; only k moves)
  const uint8_t* rp[VPT];
  int lo[VPT], ko[VPT];
#pragma unroll
  for (int p = 0; p < VPT; ++p) {
    const int v = tid + p * NT;
    rp[p] = nullptr;
    lo[p] = -1;
    ko[p] = 0;
    if (NV % NT == 0 || v < NV) {
      const int r = v / VPR, kv = v % VPR;
      if (r < Gm::LC) {
        const int64_t t = tc0 + r;
        if (t < T) rp[p] = X + (b * T + t) * rowbytes;
      } else {
        const int col = r - Gm::LC, g = col / kWave, c = col % kWave;
        const int64_t ch = imin(tile * kWave + c, d_h - 1);
        rp[p] = Wm + (g * d_h + ch) * rowbytes;
      }
      lo[p] = r * Gm::LDS_ROW + kv * 16;
      ko[p] = kv * 16;
    }
  }
  fx_f32x4 rv[VPT];
  auto gload = [&](int64_t kt) {
#pragma unroll
    for (int p = 0; p < VPT; ++p) {
      const int64_t kb = kt * Gm::ROWB + ko[p];
      rv[p] = (rp[p] && kb < rowbytes) ? *reinterpret_cast<const fx_f32x4*>(rp[p] + kb) : fx_f32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < VPT; ++p)
      if (NV % NT == 0 || lo[p] >= 0) *reinterpret_cast<fx_f32x4*>(lds + buf * Gm::STAGE + lo[p]) = rv[p];
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
  gload(0);
  lstore(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* L = lds + cur * Gm::STAGE;
#pragma unroll
    for (int kb = 0; kb < VPR / 2; ++kb) {
      const int off = kb * 32 + half * 16;
      fx_f32x4 av[Gm::NRB], bv[Gm::NCB];
#pragma unroll
      for (int i = 0; i < Gm::NRB; ++i)
        av[i] = *reinterpret_cast<const fx_f32x4*>(L + (i * 32 + l32) * Gm::LDS_ROW + off);
#pragma unroll
      for (int j = 0; j < Gm::NCB; ++j) {
        const int cb = w + j * NW;
        if (cb < Gm::NCB_ALL)
          bv[j] = *reinterpret_cast<const fx_f32x4*>(L + (Gm::LC + cb * 32 + l32) * Gm::LDS_ROW + off);
      }
      if constexpr (DT == kBF16) {
#pragma unroll
        for (int i = 0; i < Gm::NRB; ++i)
#pragma unroll
          for (int j = 0; j < Gm::NCB; ++j)
            if (w + j * NW < Gm::NCB_ALL)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(fx_bf16x8, av[i]),
                                                                  __builtin_bit_cast(fx_bf16x8, bv[j]), acc[i][j], 0,
                                                                  0, 0);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int i = 0; i < Gm::NRB; ++i)
#pragma unroll
            for (int j = 0; j < Gm::NCB; ++j)
              if (w + j * NW < Gm::NCB_ALL)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i][s], bv[j][s], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

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
