// Parallel Newton kernels: the chunked three-phase affine scan over time,
// fused with the cell / Jacobian evaluation and the residual reduction.
//
// One Newton iteration linearises every step at the previous trajectory
// guess, giving maps s_t = J_t s_{t-1} + b_t (J = 0 at segment heads,
// shapes/layout page), and solves them with an associative scan:
//   phase 1  each chunk composes its maps into one aggregate;
//   phase 2  an exclusive scan over the chunk aggregates gives every chunk
//            its carry-in state;
//   phase 3  each chunk re-runs its maps from the carry-in and writes the
//            new iterate.
// Phase 3 of iteration k is fused with phase 1 of iteration k+1: the new
// state s_t is in a register the moment it is produced, so the next
// linearisation at s_t and its chunk aggregate come out of the same pass.
//
// Work decomposition (all kernels): a workgroup owns one chunk of LC = NW*LS
// consecutive steps of one row and 64 consecutive channels.  Lane = channel
// (so every load and store of a (step, gate) row is 64 consecutive elements:
// coalesced), wave w = the w-th sub-chunk of LS steps, walked serially by
// each lane.  Sub-chunk aggregates are combined across the NW waves through
// LDS; chunk aggregates are scanned by k_tp_scan.
#pragma once

#include "prn_device.h"

namespace prn {

template <int S> __device__ __forceinline__ void store_map(float* base, int64_t stride, const Aff<S>& m);
template <> __device__ __forceinline__ void store_map<1>(float* p, int64_t st, const Aff<1>& m) {
  p[0] = m.a;
  p[st] = m.b;
}
template <> __device__ __forceinline__ void store_map<2>(float* p, int64_t st, const Aff<2>& m) {
  p[0] = m.a00; p[st] = m.a01; p[2 * st] = m.a10; p[3 * st] = m.a11; p[4 * st] = m.b0; p[5 * st] = m.b1;
}
template <int S> __device__ __forceinline__ Aff<S> load_map(const float* p, int64_t st);
template <> __device__ __forceinline__ Aff<1> load_map<1>(const float* p, int64_t st) { return {p[0], p[st]}; }
template <> __device__ __forceinline__ Aff<2> load_map<2>(const float* p, int64_t st) {
  return {p[0], p[st], p[2 * st], p[3 * st], p[4 * st], p[5 * st]};
}

// Residual max of one workgroup: max over each wave, then over the waves
// through LDS; thread 0 writes the workgroup's partial to part[block id].
// (One partial per workgroup and a separate reduction, rather than a
// same-address atomic per wave: those serialise in the memory system.)
template <int NW>
__device__ __forceinline__ void residual_partial(float r, float* __restrict__ part) {
  __shared__ float red[NW];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) r = fmaxf(r, __shfl_xor(r, o, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = r;
  __syncthreads();
  if (threadIdx.x == 0 && part) {
#pragma unroll
    for (int v = 1; v < NW; ++v) r = fmaxf(r, red[v]);
    const int64_t bid = blockIdx.x + static_cast<int64_t>(gridDim.x) * (blockIdx.y + static_cast<int64_t>(gridDim.y) * blockIdx.z);
    part[bid] = r;
  }
}

// residual_out[k] = max over the n partials of slot k; one 1024-thread
// workgroup per slot, four independent running maxima per thread.
__global__ void __launch_bounds__(1024) k_residual_reduce(const float* __restrict__ part, int64_t n,
                                                          float* __restrict__ out) {
  __shared__ float red[16];
  const float* p = part + blockIdx.x * n;
  float r0 = 0.0f, r1 = 0.0f, r2 = 0.0f, r3 = 0.0f;
  int64_t i = threadIdx.x;
  for (; i + 3 * 1024 < n; i += 4 * 1024) {
    r0 = fmaxf(r0, p[i]);
    r1 = fmaxf(r1, p[i + 1024]);
    r2 = fmaxf(r2, p[i + 2048]);
    r3 = fmaxf(r3, p[i + 3072]);
  }
  for (; i < n; i += 1024) r0 = fmaxf(r0, p[i]);
  float r = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) r = fmaxf(r, __shfl_xor(r, o, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = r;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int v = 1; v < 16; ++v) r = fmaxf(r, red[v]);
    out[blockIdx.x] = r;
  }
}

template <int DT, int S>
__device__ __forceinline__ void load_state(const typename Storage<DT>::T* p, int64_t d_h, float* s) {
#pragma unroll
  for (int q = 0; q < S; ++q) s[q] = Storage<DT>::load(p + q * d_h);
}

// ----------------------------------------------------------------------------
// Phase 1 of iteration 1.  The guess H^(0) is zero, so the linearisation
// point is 0 (or the segment's h0 at a head) and nothing but the projected
// inputs is read.  Also r_0 = max|0 - f(prev_t)|.
// agg layout: (rows, n_ch, S*S + S, d_h) fp32.
template <class C, int DT, int LS, int NW>
__global__ void __launch_bounds__(kWave * NW)
k_tp_first(const typename Storage<DT>::T* __restrict__ xproj, const typename Storage<DT>::T* __restrict__ h0,
           const int32_t* __restrict__ cu, const float* __restrict__ a, int64_t T, int64_t d_h,
           int64_t n_seqs, int64_t n_ch, float* __restrict__ agg, float* __restrict__ rpart) {
  using ST = Storage<DT>;
  using Map = typename C::Map;
  constexpr int G = C::G, S = C::S, NC = S * S + S, LC = LS * NW;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int64_t chunk = blockIdx.x, b = blockIdx.z;
  const int64_t ch = static_cast<int64_t>(blockIdx.y) * kWave + lane;
  const int64_t t0 = chunk * LC + static_cast<int64_t>(w) * LS;
  __shared__ Map part[NW][kWave];

  Map acc = Map::identity();
  float rmax = 0.0f;
  if (ch < d_h && t0 < T) {
    ChanCoef<C> cf;
    cf.load(a, d_h, ch);
    SegTracker sg;
    sg.init(cu, n_seqs, b, t0);
    const typename ST::T* xp = xproj + ((b * T + t0) * G) * d_h + ch;
    const int n = static_cast<int>(imin(LS, T - t0));
#pragma unroll
    for (int j = 0; j < LS; ++j) {
      if (j < n) {
        const bool head = sg.at(t0 + j);
        float prev[S];
#pragma unroll
        for (int q = 0; q < S; ++q) prev[q] = 0.0f;
        if (head && h0) load_state<DT, S>(h0 + sg.seg * S * d_h + ch, d_h, prev);
        float x[G];
        load_xs<C, DT>(xp + j * G * d_h, d_h, x);
        float fv[S];
        const Map m = C::fj(x, prev, cf.as, cf.a, head, fv);
        acc = compose(m, acc);
#pragma unroll
        for (int q = 0; q < S; ++q) rmax = fmaxf(rmax, abs_nan_inf(fv[q]));
      }
    }
  }
  part[w][lane] = acc;
  __syncthreads();
  if (w == 0 && ch < d_h) {
    Map tot = part[0][lane];
#pragma unroll
    for (int v = 1; v < NW; ++v) tot = compose(part[v][lane], tot);
    store_map<S>(agg + ((b * n_ch + chunk) * NC) * d_h + ch, d_h, tot);
  }
  residual_partial<NW>(rmax, rpart);
}

// ----------------------------------------------------------------------------
// Phase 2: exclusive scan of the chunk aggregates of every (row, channel),
// producing the carry-in state of every chunk (the state just before its
// first step).  NSEG segments of chunks per channel are composed in
// parallel, combined through LDS, then re-walked to emit the carries.  The
// state entering chunk 0 is 0; every row starts with a head (J = 0), so it
// never reaches the output.
// carry layout: (rows, n_ch, S, d_h) fp32.
template <int S, int NSEG>
__global__ void __launch_bounds__(kWave * NSEG)
k_tp_scan(const float* __restrict__ agg, float* __restrict__ carry, int64_t d_h, int64_t n_ch) {
  using Map = Aff<S>;
  constexpr int NC = S * S + S;
  const int lane = threadIdx.x & (kWave - 1), sgm = threadIdx.x / kWave;
  const int64_t ch = static_cast<int64_t>(blockIdx.x) * kWave + lane;
  const int64_t b = blockIdx.y;
  const int64_t per = (n_ch + NSEG - 1) / NSEG;
  const int64_t c0 = imin(n_ch, sgm * per), c1 = imin(n_ch, c0 + per);
  __shared__ Map part[NSEG][kWave];
  const bool act = ch < d_h;
  const float* ap = agg + (b * n_ch * NC) * d_h + ch;

  // U maps are loaded before any is used, so their latencies overlap
  constexpr int U = 8;
  Map acc = Map::identity();
  if (act) {
    for (int64_t c = c0; c < c1; c += U) {
      Map m[U];
#pragma unroll
      for (int u = 0; u < U; ++u) m[u] = (c + u < c1) ? load_map<S>(ap + (c + u) * NC * d_h, d_h) : Map::identity();
#pragma unroll
      for (int u = 0; u < U; ++u) acc = compose(m[u], acc);
    }
  }
  part[sgm][lane] = acc;
  __syncthreads();
  if (!act) return;
  float st[S];
#pragma unroll
  for (int q = 0; q < S; ++q) st[q] = 0.0f;
  for (int v = 0; v < sgm; ++v) apply(part[v][lane], st);
  float* cp = carry + (b * n_ch * S) * d_h + ch;
  for (int64_t c = c0; c < c1; c += U) {
    Map m[U];
#pragma unroll
    for (int u = 0; u < U; ++u) m[u] = (c + u < c1) ? load_map<S>(ap + (c + u) * NC * d_h, d_h) : Map::identity();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c + u < c1) {
#pragma unroll
        for (int q = 0; q < S; ++q) cp[((c + u) * S + q) * d_h] = st[q];
        apply(m[u], st);
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Phase 3 of iteration k (fix-up), optionally fused with phase 1 of
// iteration k+1 (NEXT) or closing the solve (LAST).
//   walk A: re-linearise at H^(k-1) (cheaper than storing J and b), compose
//           the sub-chunk aggregate; LDS gives each wave its carry-in.
//   walk B: s_t = J_t s_{t-1} + b_t from the carry-in (fp32 chain), store
//           H^(k) rounded to the storage dtype; with NEXT, linearise at the
//           stored H^(k)_{t-1} for iteration k+1 and compose its aggregate;
//           r_k = max|H^(k)_t - f(H^(k)_{t-1})| comes from the same cell
//           evaluation (with LAST it is the final residual r_K).
// Hprev = null means H^(k-1) = 0 (k = 1).
template <class C, int DT, int LS, int NW, bool NEXT, bool LAST>
__global__ void __launch_bounds__(kWave * NW)
k_tp_fix(const typename Storage<DT>::T* __restrict__ xproj, const typename Storage<DT>::T* __restrict__ Hprev,
         const typename Storage<DT>::T* __restrict__ h0, const int32_t* __restrict__ cu,
         const float* __restrict__ a, int64_t T, int64_t d_h, int64_t n_seqs, int64_t n_ch,
         const float* __restrict__ carry, typename Storage<DT>::T* __restrict__ Hnext,
         typename Storage<DT>::T* __restrict__ Hout, typename Storage<DT>::T* __restrict__ slast,
         typename Storage<DT>::T* __restrict__ sout, float* __restrict__ agg_next, float* __restrict__ rpart) {
  using ST = Storage<DT>;
  using Map = typename C::Map;
  constexpr int G = C::G, S = C::S, NC = S * S + S, LC = LS * NW;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int64_t chunk = blockIdx.x, b = blockIdx.z;
  const int64_t ch = static_cast<int64_t>(blockIdx.y) * kWave + lane;
  const int64_t t0 = chunk * LC + static_cast<int64_t>(w) * LS;
  const bool act = ch < d_h && t0 < T;
  const int n = act ? static_cast<int>(imin(LS, T - t0)) : 0;
  __shared__ Map part[NW][kWave];

  ChanCoef<C> cf;
  float xs[LS][G];
  Map ms[LS];
  Map acc = Map::identity();
  SegTracker sg;
  if (act) {
    cf.load(a, d_h, ch);
    sg.init(cu, n_seqs, b, t0);
    const typename ST::T* xp = xproj + ((b * T + t0) * G) * d_h + ch;
    const typename ST::T* hp = Hprev ? Hprev + ((b * T + t0 - 1) * S) * d_h + ch : nullptr;
#pragma unroll
    for (int j = 0; j < LS; ++j) {
      if (j < n) {
        const bool head = sg.at(t0 + j);
        float prev[S];
#pragma unroll
        for (int q = 0; q < S; ++q) prev[q] = 0.0f;
        if (head) {
          if (h0) load_state<DT, S>(h0 + sg.seg * S * d_h + ch, d_h, prev);
        } else if (hp) {
          load_state<DT, S>(hp + j * S * d_h, d_h, prev);
        }
        load_xs<C, DT>(xp + j * G * d_h, d_h, xs[j]);
        float fv[S];
        ms[j] = C::fj(xs[j], prev, cf.as, cf.a, head, fv);
        acc = compose(ms[j], acc);
      }
    }
  }
  part[w][lane] = acc;
  __syncthreads();
  float s[S];
  if (act) {
    const float* cp = carry + ((b * n_ch + chunk) * S) * d_h + ch;
#pragma unroll
    for (int q = 0; q < S; ++q) s[q] = cp[q * d_h];
    for (int v = 0; v < w; ++v) apply(part[v][lane], s);
  }
  if (NEXT) __syncthreads();  // part[] is reused for the next aggregate

  Map acc2 = Map::identity();
  float rmax = 0.0f;
  if (act) {
    float pr[S];
#pragma unroll
    for (int q = 0; q < S; ++q) pr[q] = ST::round(s[q]);
    sg.init(cu, n_seqs, b, t0);
#pragma unroll
    for (int j = 0; j < LS; ++j) {
      if (j < n) {
        const int64_t t = t0 + j;
        const bool head = sg.at(t);
        apply(ms[j], s);
        float sr[S];
#pragma unroll
        for (int q = 0; q < S; ++q) sr[q] = ST::round(s[q]);
        if (!LAST) {
          typename ST::T* hn = Hnext + ((b * T + t) * S) * d_h + ch;
#pragma unroll
          for (int q = 0; q < S; ++q) hn[q * d_h] = ST::pack(s[q]);
        } else {
          Hout[(b * T + t) * d_h + ch] = ST::pack(s[S - 1]);
          if (sout) {
#pragma unroll
            for (int q = 0; q < S; ++q) sout[((b * T + t) * S + q) * d_h + ch] = ST::pack(s[q]);
          }
          if (slast && sg.last(t, T)) {
#pragma unroll
            for (int q = 0; q < S; ++q) slast[(sg.seg * S + q) * d_h + ch] = ST::pack(s[q]);
          }
        }
        if (NEXT || LAST) {
          float p[S];
#pragma unroll
          for (int q = 0; q < S; ++q) p[q] = pr[q];
          if (head) {
#pragma unroll
            for (int q = 0; q < S; ++q) p[q] = 0.0f;
            if (h0) load_state<DT, S>(h0 + sg.seg * S * d_h + ch, d_h, p);
          }
          float fv[S];
          if (NEXT) {
            const Map m2 = C::fj(xs[j], p, cf.as, cf.a, head, fv);
            acc2 = compose(m2, acc2);
          } else {
            C::f(xs[j], p, cf.as, cf.a, fv);
          }
#pragma unroll
          for (int q = 0; q < S; ++q) rmax = fmaxf(rmax, abs_nan_inf(sr[q] - fv[q]));
        }
#pragma unroll
        for (int q = 0; q < S; ++q) pr[q] = sr[q];
      }
    }
  }
  if (NEXT) {
    part[w][lane] = acc2;
    __syncthreads();
    if (w == 0 && ch < d_h) {
      Map tot = part[0][lane];
#pragma unroll
      for (int v = 1; v < NW; ++v) tot = compose(part[v][lane], tot);
      store_map<S>(agg_next + ((b * n_ch + chunk) * NC) * d_h + ch, d_h, tot);
    }
  }
  residual_partial<NW>(rmax, rpart);
}

// ----------------------------------------------------------------------------
// Sequential unroll (eval mode): one lane per (sequence, channel) walks its
// whole sequence, s_t = f(s_{t-1}, x_t), state kept in fp32 between steps.
template <class C, int DT>
__global__ void __launch_bounds__(kWave)
k_sequential(const typename Storage<DT>::T* __restrict__ xproj, const typename Storage<DT>::T* __restrict__ h0,
             const int32_t* __restrict__ cu, const float* __restrict__ a, int64_t T, int64_t d_h,
             int64_t n_seqs, typename Storage<DT>::T* __restrict__ Hout,
             typename Storage<DT>::T* __restrict__ slast, typename Storage<DT>::T* __restrict__ sout) {
  using ST = Storage<DT>;
  constexpr int G = C::G, S = C::S;
  const int64_t ch = static_cast<int64_t>(blockIdx.x) * kWave + threadIdx.x;
  const int64_t r = blockIdx.y;  // row (rectangular) or segment (ragged)
  if (ch >= d_h) return;
  int64_t base, len;
  if (cu) {
    const int64_t lo = cu[r], hi = cu[r + 1];
    base = imax(0, imin(lo, T));
    len = imax(0, imin(hi, T) - base);
  } else {
    base = r * T;
    len = T;
  }
  ChanCoef<C> cf;
  cf.load(a, d_h, ch);
  float s[S];
#pragma unroll
  for (int q = 0; q < S; ++q) s[q] = 0.0f;
  if (h0) load_state<DT, S>(h0 + r * S * d_h + ch, d_h, s);
  const typename ST::T* xp = xproj + base * G * d_h + ch;
  typename ST::T* hp = Hout + base * d_h + ch;
  typename ST::T* sp = sout ? sout + base * S * d_h + ch : nullptr;
  constexpr int U = 4;
  int64_t t = 0;
  for (; t + U <= len; t += U) {
    float x[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) load_xs<C, DT>(xp + (t + u) * G * d_h, d_h, x[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float o[S];
      C::f(x[u], s, cf.as, cf.a, o);
#pragma unroll
      for (int q = 0; q < S; ++q) s[q] = o[q];
      hp[(t + u) * d_h] = ST::pack(s[S - 1]);
      if (sp) {
#pragma unroll
        for (int q = 0; q < S; ++q) sp[((t + u) * S + q) * d_h] = ST::pack(s[q]);
      }
    }
  }
  for (; t < len; ++t) {
    float x[G];
    load_xs<C, DT>(xp + t * G * d_h, d_h, x);
    float o[S];
    C::f(x, s, cf.as, cf.a, o);
#pragma unroll
    for (int q = 0; q < S; ++q) s[q] = o[q];
    hp[t * d_h] = ST::pack(s[S - 1]);
    if (sp) {
#pragma unroll
      for (int q = 0; q < S; ++q) sp[(t * S + q) * d_h] = ST::pack(s[q]);
    }
  }
  if (slast) {
#pragma unroll
    for (int q = 0; q < S; ++q) slast[(r * S + q) * d_h + ch] = ST::pack(s[q]);
  }
}

// Final state of empty segments of a ragged pack: their h0 (or zero).
template <int DT, int S>
__global__ void k_empty_segments(const int32_t* __restrict__ cu, int64_t n_seqs, int64_t d_h,
                                 const typename Storage<DT>::T* __restrict__ h0,
                                 typename Storage<DT>::T* __restrict__ slast) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n_seqs * S * d_h) return;
  const int64_t j = i / (S * d_h);
  if (cu[j + 1] > cu[j]) return;
  slast[i] = h0 ? h0[i] : Storage<DT>::pack(0.0f);
}

template <class T>
__global__ void k_copy_or_zero(const T* __restrict__ src, T* __restrict__ dst, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : T(0);
}

__global__ void k_zero_u32(unsigned* __restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

__global__ void k_zero_f32(float* __restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

}  // namespace prn
