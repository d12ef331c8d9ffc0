// One T = 1 step of the sequential cell for B independent slots (the serving
// decode step of the FAQs: a fixed-size carry (slots, d_h) per layer, the
// token's input projection then one cell step): projection and cell fused
// in one launch.
//
// A workgroup takes 64 channels of one slot; its four waves each sum a
// quarter of d_in for all G gates (lane = channel, 16-byte loads along the
// weight row), the quarters are added in a fixed order through LDS with the
// bias, the projected value is rounded to the storage dtype (as the
// projection's output would be), and wave 0 steps the cell from the carry.
#pragma once

#include "newton_kernels.h"

namespace prn {

template <class C, int DT>
__global__ void __launch_bounds__(256)
k_decode(const typename Storage<DT>::T* __restrict__ x, const typename Storage<DT>::T* __restrict__ W,
         const float* __restrict__ bias, const float* __restrict__ a, int64_t d_in, int64_t d_h,
         const typename Storage<DT>::T* __restrict__ sin, typename Storage<DT>::T* __restrict__ sout,
         typename Storage<DT>::T* __restrict__ hout) {
  using ST = Storage<DT>;
  constexpr int G = C::G, S = C::S;
  constexpr int VE = 16 / sizeof(typename ST::T);  // elements per 16-byte load
  const int lane = threadIdx.x & (kWave - 1), part = threadIdx.x / kWave;
  const int64_t ch_l = static_cast<int64_t>(blockIdx.x) * kWave + lane;
  const bool ch_ok = ch_l < d_h;
  const int64_t ch = ch_ok ? ch_l : d_h - 1;
  const int64_t slot = blockIdx.y;
  __shared__ float red[4][G][kWave];

  // this wave's quarter of the reduction dimension, in whole 16-byte vectors
  const int64_t nvec = d_in / VE;
  const int64_t v0 = part * nvec / 4, v1 = (part + 1) * nvec / 4;
  const typename ST::T* xr = x + slot * d_in;
  float acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.0f;
  for (int64_t v = v0; v < v1; ++v) {
    float xv[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) xv[e] = ST::load(xr + v * VE + e);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const typename ST::T* wr = W + (g * d_h + ch) * d_in + v * VE;
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[g] = fmaf(xv[e], ST::load(wr + e), acc[g]);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) red[part][g][lane] = acc[g];
  __syncthreads();
  if (part != 0 || !ch_ok) return;

  ChanCoef<C> cf;
  cf.load(a, d_h, ch);
  float xs[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float v = ((red[0][g][lane] + red[1][g][lane]) + red[2][g][lane]) + red[3][g][lane];
    if (bias) v += bias[g * d_h + ch];
    xs[g] = ST::round(v) * C::scale(g);
  }
  float s[S], o[S];
#pragma unroll
  for (int q = 0; q < S; ++q) s[q] = 0.0f;
  if (sin) load_state<DT, S>(sin + slot * S * d_h + ch, d_h, s);
  C::f(xs, s, cf.as, cf.a, o);
#pragma unroll
  for (int q = 0; q < S; ++q) sout[(slot * S + q) * d_h + ch] = ST::pack(o[q]);
  if (hout) hout[slot * d_h + ch] = ST::pack(o[S - 1]);
}

}  // namespace prn
