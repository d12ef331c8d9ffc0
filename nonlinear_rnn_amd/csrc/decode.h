// One T = 1 step of the sequential cell for B independent slots (the serving
// decode step of the FAQs: a fixed-size carry (slots, d_h) per layer, the
// token's input projection then one cell step): projection and cell fused
// in one launch.
//
// One wave takes one channel and a group of 16 slots.  Lanes run along d_in
// (each weight row and each token is read in coalesced 64-element pieces),
// and every lane keeps a partial sum for each of the 4 x 16 (gate, slot)
// outputs (the GRU's three gates padded to four).  A transpose-reduce
// butterfly (at each lane bit a lane keeps the half of its partials that
// bit selects and adds its partner's copy of that half: 63 exchange-adds in
// all, through cross-lane swaps and DPP, not LDS) leaves lane l with the
// complete sum of output l.
// The sum gets its bias, is rounded to the storage dtype (as the
// projection's output would be), and lanes 0..15 gather their slot's gates
// and step the cell from the carry.  Waves are independent: no LDS, no
// barrier.
#pragma once

#include <type_traits>

#include "newton_kernels.h"

namespace prn {

constexpr int kDecodeSlots = 16;  // slots per wave
constexpr int kDecodeWaves = 4;   // channels (waves) per workgroup

template <class C, int DT>
__global__ void __launch_bounds__(kWave * kDecodeWaves)
k_decode(const typename Storage<DT>::T* __restrict__ x, const typename Storage<DT>::T* __restrict__ W,
         const float* __restrict__ bias, const float* __restrict__ a, int64_t n_slots, int64_t d_in, int64_t d_h,
         const typename Storage<DT>::T* __restrict__ sin, typename Storage<DT>::T* __restrict__ sout,
         typename Storage<DT>::T* __restrict__ hout) {
  using ST = Storage<DT>;
  constexpr int G = C::G, S = C::S, GP = 4, SB = kDecodeSlots;
  static_assert(G <= GP && GP * SB == kWave, "one output per lane after the reduction");
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t ch = static_cast<int64_t>(blockIdx.x) * kDecodeWaves + threadIdx.x / kWave;
  if (ch >= d_h) return;  // whole wave
  const int64_t s0 = static_cast<int64_t>(blockIdx.y) * SB;
  const int n_s = static_cast<int>(imin(SB, n_slots - s0));

  // what the cell step needs besides the projection (this lane's bias term,
  // the channel's recurrent weights, the carry of this lane's slot) is read
  // here, so that those loads are in flight with the projection's instead of
  // after them (lanes past the last slot read the last slot's carry and
  // store nothing)
  const int g_l = lane / SB;
  const float bv = (bias && g_l < G) ? bias[g_l * d_h + ch] : 0.0f;
  ChanCoef<C> cf;
  cf.load(a, d_h, ch);
  const int64_t slot = s0 + imin(lane & (SB - 1), n_s - 1);
  float s[S];
#pragma unroll
  for (int q = 0; q < S; ++q) s[q] = 0.0f;
  if (sin) load_state<DT, S>(sin + slot * S * d_h + ch, d_h, s);

  // partial dot products: p[g * SB + s] over this lane's k = lane, lane + 64,
  // ...; U row pieces per round, their loads issued together (the loop is
  // bound by load latency, not by the multiply-adds).  The loads carry no
  // guard (a guard per load becomes a branch per load, which serialises
  // them): a k past d_in reads the last column with a zero weight, a slot
  // past the last one rereads the last slot, whose outputs nobody stores.
  constexpr int U = 4;
  float p[GP * SB];
#pragma unroll
  for (int i = 0; i < GP * SB; ++i) p[i] = 0.0f;
  for (int64_t k0 = lane; k0 < d_in; k0 += U * kWave) {
    float wv[U][G], xv[U][SB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = k0 + u * kWave;
      const bool ok = k < d_in;
      const int64_t kc = ok ? k : d_in - 1;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float v = ST::load(W + (g * d_h + ch) * d_in + kc);
        wv[u][g] = ok ? v : 0.0f;
      }
#pragma unroll
      for (int s = 0; s < SB; ++s) xv[u][s] = ST::load(x + (s0 + imin(s, n_s - 1)) * d_in + kc);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int s = 0; s < SB; ++s) p[g * SB + s] = fmaf(wv[u][g], xv[u][s], p[g * SB + s]);
  }
  // transpose-reduce: after the stage of lane bit b, lane l holds 2^b
  // partials, those of the outputs whose bit b equals l's bit b.  The
  // partner of a lane differs from it in bit b and agrees on the bits above
  // (it holds the same outputs).  Bits 5 and 4: the half-wave and row swaps
  // exchange one register of each pair across the halves (rows), and the
  // sum of the two swapped registers is own + partner's copy of the half
  // each lane keeps.  Bits 3..0: a lane sends the half it does not keep,
  // read by its partner through DPP: rotate by 8 in a row (partner l ^ 8),
  // mirror in 8 lanes (l ^ 7: bit 2 flips, bits 3 and up agree), quad
  // permutations (l ^ 2, l ^ 1).  No LDS traffic.
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[i]), __float_as_uint(p[i + 32]), false, false);
    p[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(p[i]), __float_as_uint(p[i + 16]), false, false);
    p[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  auto dpp_stage = [&](auto m_t, auto ctrl_t) __attribute__((always_inline)) {
    constexpr int m = decltype(m_t)::value, ctrl = decltype(ctrl_t)::value;
    const bool hi = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < m; ++i) {
      const float keep = hi ? p[i + m] : p[i];
      const float send = hi ? p[i] : p[i + m];
      p[i] = keep + __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(send), ctrl, 0xf, 0xf, false));
    }
  };
  dpp_stage(std::integral_constant<int, 8>{}, std::integral_constant<int, 0x128>{});  // row_ror:8
  dpp_stage(std::integral_constant<int, 4>{}, std::integral_constant<int, 0x141>{});  // row_half_mirror
  dpp_stage(std::integral_constant<int, 2>{}, std::integral_constant<int, 0x4e>{});   // quad_perm [2,3,0,1]
  dpp_stage(std::integral_constant<int, 1>{}, std::integral_constant<int, 0xb1>{});   // quad_perm [1,0,3,2]
  // lane l = g * SB + s holds the projected value of gate g, slot s
  float v = p[0];
  if (g_l < G) {
    if (bias) v += bv;
    v = ST::round(v);
  }
  float xs[G];
#pragma unroll
  for (int g = 0; g < G; ++g) xs[g] = __shfl(v, g * SB + (lane & (SB - 1)), kWave) * C::scale(g);
  if (lane >= n_s) return;  // lanes 0..n_s-1: one slot each (slot = s0 + lane)

  float o[S];
  C::f(xs, s, cf.as, cf.a, o);
#pragma unroll
  for (int q = 0; q < S; ++q) sout[(slot * S + q) * d_h + ch] = ST::pack(o[q]);
  if (hout) hout[slot * d_h + ch] = ST::pack(o[S - 1]);
}

}  // namespace prn
