// Backward pass of the diagonal recurrences: gradients of a loss through
// s_t = f(s_{t-1}, x_t) at a given trajectory, by the adjoint recurrence
//
//   lam_t = g_t + J_{t+1}^T lam_{t+1}     (0 where step t+1 is a segment head
//                                          or past the row's end)
//
// with g_t = dL/ds_t arriving directly at step t (dL/dh_t, plus dL/d(final
// state) at a sequence's last step).  The quantity carried between steps is
// the gradient flowing out of a step into the one before it,
//
//   mu_{t-1} = J_t^T lam_t,   lam_t = g_t + [step t+1 not a cut] mu_t,
//
// and one step is the affine map  P_t(mu) = J_t^T (g_t + c_{t+1} mu)  with
// c_{t+1} = 0 at a cut, 1 otherwise.  The maps compose backwards in time, so
// the forward's chunked three-phase scan runs unchanged on reversed chunks:
//   phase 1 (k_bw_reduce)  each chunk composes P_{t0} o ... o P_{t1-1} and
//                          stores it at chunk index n_ch - 1 - chunk;
//   phase 2 (k_tp_scan)    the forward's exclusive scan over increasing
//                          index: every chunk gets the mu entering it from
//                          all later chunks of its row;
//   phase 3 (k_bw_fix)     each chunk re-derives its waves' maps, gives each
//                          wave its carry-in, and walks its steps backwards
//                          from it: lam_t, then the step's vector-Jacobian
//                          product (C::vjp) gives dL/dx_t (stored), dL/da
//                          (accumulated per lane) and mu_{t-1}; at a head,
//                          mu_{t-1} is dL/dh0 of that segment.
// dL/da is reduced over rows and chunks in a fixed order (k_bw_da_reduce).
//
// The default schedule is the single-pass kernel k_bw_sp, the backward twin
// of the forward's single-pass kernel: chunks are taken by ticket in reverse
// time order, each workgroup composes its chunk's maps, obtains the gradient
// entering it from the later chunks by the same decoupled look-back (chunk
// records indexed in processing order; the result does not depend on
// timing), publishes what leaves it, and walks
// its steps backwards; inputs cross HBM once and no scan pass is needed.
// The three-phase kernels above remain as the PRN_ALGO=tp schedule.
//
// Work decomposition as in the forward kernels: lane = channel, wave w = the
// w-th sub-chunk of LS steps of a chunk of LC = NW LS steps, walked serially.
#pragma once

#include "newton_kernels.h"
#include "newton_sp.h"

namespace prn {

// Segment of steps walked backwards (t non-increasing): [start, end) is the
// segment holding the current step.  Rectangular batch: one segment per row.
struct RevSegTracker {
  const int32_t* cu;
  int64_t seg, start, end;

  __device__ __forceinline__ void init(const int32_t* cu_, int64_t n_seqs, int64_t row, int64_t t, int64_t T) {
    cu = cu_;
    if (!cu) {
      seg = row;
      start = 0;
      end = T;
      return;
    }
    // largest j in [0, n_seqs) with cu[j] <= t (skips empty segments)
    int64_t lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (static_cast<int64_t>(cu[mid]) <= t) lo = mid; else hi = mid - 1;
    }
    seg = lo;
    start = cu[seg];
    end = cu[seg + 1];
  }
  // init by a whole wave (every lane active, t wave-uniform): the forward's
  // wave-wide segment search
  __device__ __forceinline__ void init_wave(const int32_t* cu_, int64_t n_seqs, int64_t row, int64_t t, int64_t T) {
    cu = cu_;
    if (!cu) {
      seg = row;
      start = 0;
      end = T;
      return;
    }
    SegTracker f;
    f.init_wave(cu_, n_seqs, 0, t);
    seg = f.seg;
    start = f.start;
    end = cu[seg + 1];
  }
  __device__ __forceinline__ void at(int64_t t) {
    if (cu) {
      while (seg > 0 && start > t) {
        --seg;
        start = cu[seg];
        end = cu[seg + 1];
      }
    }
  }
  __device__ __forceinline__ bool head(int64_t t) const { return t == start || t == 0; }
  // nothing flows into t from t + 1: t is its segment's (or row's) last step
  __device__ __forceinline__ bool last(int64_t t, int64_t T) const { return t + 1 == end || t + 1 == T; }
};

// P_t = (c J^T, J^T g): the transposed step map, cut (A = 0) at a segment end
__device__ __forceinline__ Aff<1> bw_step_map(const Aff<1>& m, const float* g, bool cut) {
  return {cut ? 0.0f : m.a, m.a * g[0]};
}
__device__ __forceinline__ Aff<2> bw_step_map(const Aff<2>& m, const float* g, bool cut) {
  Aff<2> p;
  p.a00 = cut ? 0.0f : m.a00;
  p.a01 = cut ? 0.0f : m.a10;
  p.a10 = cut ? 0.0f : m.a01;
  p.a11 = cut ? 0.0f : m.a11;
  p.b0 = fmaf(m.a00, g[0], m.a10 * g[1]);
  p.b1 = fmaf(m.a01, g[0], m.a11 * g[1]);
  return p;
}

// Everything a step of the backward reads: the state it starts from (the
// segment's h0 at a head), its scaled projected inputs and g_t.
template <class C, int DT>
struct BwStep {
  float prev[C::S], xs[C::G], g[C::S];

  __device__ __forceinline__ void load(const typename Storage<DT>::T* __restrict__ xproj,
                                       const typename Storage<DT>::T* __restrict__ states,
                                       const typename Storage<DT>::T* __restrict__ h0,
                                       const typename Storage<DT>::T* __restrict__ dH,
                                       const typename Storage<DT>::T* __restrict__ dsl, int64_t b, int64_t t,
                                       int64_t T, int64_t d_h, int64_t ch, const RevSegTracker& rs) {
    constexpr int G = C::G, S = C::S;
#pragma unroll
    for (int q = 0; q < S; ++q) prev[q] = 0.0f;
    if (rs.head(t)) {
      if (h0) load_state<DT, S>(h0 + rs.seg * S * d_h + ch, d_h, prev);
    } else {
      load_state<DT, S>(states + ((b * T + t - 1) * S) * d_h + ch, d_h, prev);
    }
    load_xs<C, DT>(xproj + ((b * T + t) * G) * d_h + ch, d_h, xs);
#pragma unroll
    for (int q = 0; q < S - 1; ++q) g[q] = 0.0f;
    g[S - 1] = Storage<DT>::load(dH + (b * T + t) * d_h + ch);
    if (dsl && rs.last(t, T)) {
#pragma unroll
      for (int q = 0; q < S; ++q) g[q] += Storage<DT>::load(dsl + (rs.seg * S + q) * d_h + ch);
    }
  }
};

// Phase 1.  agg layout: (B, n_ch, S*S + S, d_h) fp32, chunk order reversed.
template <class C, int DT, int LS, int NW>
__global__ void __launch_bounds__(kWave * NW)
k_bw_reduce(const typename Storage<DT>::T* __restrict__ xproj, const typename Storage<DT>::T* __restrict__ states,
            const typename Storage<DT>::T* __restrict__ h0, const int32_t* __restrict__ cu,
            const float* __restrict__ a, const typename Storage<DT>::T* __restrict__ dH,
            const typename Storage<DT>::T* __restrict__ dsl, int64_t T, int64_t d_h, int64_t n_seqs, int64_t n_ch,
            float* __restrict__ agg) {
  using Map = typename C::Map;
  constexpr int S = C::S, NC = S * S + S, LC = LS * NW;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int64_t chunk = blockIdx.x, b = blockIdx.z;
  const int64_t ch = static_cast<int64_t>(blockIdx.y) * kWave + lane;
  const int64_t t0 = chunk * LC + static_cast<int64_t>(w) * LS;
  const bool act = ch < d_h && t0 < T;
  const int n = act ? static_cast<int>(imin(LS, T - t0)) : 0;
  __shared__ Map part[NW][kWave];

  Map acc = Map::identity();
  if (act) {
    ChanCoef<C> cf;
    cf.load(a, d_h, ch);
    RevSegTracker rs;
    rs.init(cu, n_seqs, b, t0 + n - 1, T);
#pragma unroll
    for (int j = LS - 1; j >= 0; --j) {
      if (j < n) {
        const int64_t t = t0 + j;
        rs.at(t);
        BwStep<C, DT> st;
        st.load(xproj, states, h0, dH, dsl, b, t, T, d_h, ch, rs);
        float fv[S];
        const Map m = C::template fj<false>(st.xs, st.prev, cf.as, cf.a, false, fv);
        acc = compose(bw_step_map(m, st.g, rs.last(t, T)), acc);
      }
    }
  }
  part[w][lane] = acc;
  __syncthreads();
  if (w == 0 && ch < d_h) {
    Map tot = part[NW - 1][lane];
#pragma unroll
    for (int v = NW - 2; v >= 0; --v) tot = compose(part[v][lane], tot);
    store_map<S>(agg + ((b * n_ch + (n_ch - 1 - chunk)) * NC) * d_h + ch, d_h, tot);
  }
}

// Phase 3.  carry layout: (B, n_ch, S, d_h) fp32, chunk order reversed (as
// k_tp_scan writes it for the reversed aggregates).  dap: (B, n_ch, G, d_h)
// fp32 per-chunk partial sums of dL/da.
template <class C, int DT, int LS, int NW>
__global__ void __launch_bounds__(kWave * NW)
k_bw_fix(const typename Storage<DT>::T* __restrict__ xproj, const typename Storage<DT>::T* __restrict__ states,
         const typename Storage<DT>::T* __restrict__ h0, const int32_t* __restrict__ cu,
         const float* __restrict__ a, const typename Storage<DT>::T* __restrict__ dH,
         const typename Storage<DT>::T* __restrict__ dsl, int64_t T, int64_t d_h, int64_t n_seqs, int64_t n_ch,
         const float* __restrict__ carry, typename Storage<DT>::T* __restrict__ dxproj,
         typename Storage<DT>::T* __restrict__ dh0, float* __restrict__ dap) {
  using ST = Storage<DT>;
  using Map = typename C::Map;
  constexpr int G = C::G, S = C::S, LC = LS * NW;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int64_t chunk = blockIdx.x, b = blockIdx.z;
  const int64_t ch = static_cast<int64_t>(blockIdx.y) * kWave + lane;
  const int64_t t0 = chunk * LC + static_cast<int64_t>(w) * LS;
  const bool act = ch < d_h && t0 < T;
  const int n = act ? static_cast<int>(imin(LS, T - t0)) : 0;
  __shared__ Map part[NW][kWave];
  __shared__ float dash[NW][G][kWave];

  // walk A: this wave's map, kept with the steps' inputs for walk B
  ChanCoef<C> cf;
  BwStep<C, DT> st[LS];
  Map acc = Map::identity();
  RevSegTracker rs;
  if (act) {
    cf.load(a, d_h, ch);
    rs.init(cu, n_seqs, b, t0 + n - 1, T);
#pragma unroll
    for (int j = LS - 1; j >= 0; --j) {
      if (j < n) {
        const int64_t t = t0 + j;
        rs.at(t);
        st[j].load(xproj, states, h0, dH, dsl, b, t, T, d_h, ch, rs);
        float fv[S];
        const Map m = C::template fj<false>(st[j].xs, st[j].prev, cf.as, cf.a, false, fv);
        acc = compose(bw_step_map(m, st[j].g, rs.last(t, T)), acc);
      }
    }
  }
  part[w][lane] = acc;
  __syncthreads();

  // the gradient entering this wave: the chunk's carry-in through the later waves
  float mu[S];
  float da[G];
#pragma unroll
  for (int g = 0; g < G; ++g) da[g] = 0.0f;
  if (act) {
    const float* cp = carry + ((b * n_ch + (n_ch - 1 - chunk)) * S) * d_h + ch;
#pragma unroll
    for (int q = 0; q < S; ++q) mu[q] = cp[q * d_h];
    for (int v = NW - 1; v > w; --v) apply(part[v][lane], mu);

    // walk B: lam_t, the step's vector-Jacobian product, mu_{t-1}
    rs.init(cu, n_seqs, b, t0 + n - 1, T);
#pragma unroll
    for (int j = LS - 1; j >= 0; --j) {
      if (j < n) {
        const int64_t t = t0 + j;
        rs.at(t);
        const bool cut = rs.last(t, T);
        float lam[S];
#pragma unroll
        for (int q = 0; q < S; ++q) lam[q] = cut ? st[j].g[q] : st[j].g[q] + mu[q];
        float dx[G], dac[G];
        C::vjp(st[j].xs, st[j].prev, cf.as, cf.a, lam, dx, dac, mu);
        typename ST::T* dp = dxproj + ((b * T + t) * G) * d_h + ch;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          dp[g * d_h] = ST::pack(dx[g]);
          da[g] += dac[g];
        }
        if (dh0 && rs.head(t)) {
#pragma unroll
          for (int q = 0; q < S; ++q) dh0[(rs.seg * S + q) * d_h + ch] = ST::pack(mu[q]);
        }
      }
    }
  }
  // dL/da of the chunk: waves summed in a fixed order
#pragma unroll
  for (int g = 0; g < G; ++g) dash[w][g][lane] = da[g];
  __syncthreads();
  if (w == 0 && ch < d_h) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = dash[0][g][lane];
#pragma unroll
      for (int v = 1; v < NW; ++v) s += dash[v][g][lane];
      dap[((b * n_ch + chunk) * G + g) * d_h + ch] = s;
    }
  }
}

// Single-pass backward.  Ticket i takes chain i mod n_chains and processing
// index r = i / n_chains, i.e. time chunk n_ch - 1 - r: a chunk only waits on
// chunks later in time, which hold smaller tickets and have started.  Chunk
// records (status, aggregate map, outgoing gradient) are indexed by r; the
// look-back is the forward's (lookback_carry), so are its bounded waits and
// its timing-independent (bitwise reproducible) arithmetic.
template <class C, int DT, int LS, int NW>
__global__ void __launch_bounds__(kWave * NW)
k_bw_sp(const typename Storage<DT>::T* __restrict__ xproj, const typename Storage<DT>::T* __restrict__ states,
        const typename Storage<DT>::T* __restrict__ h0, const int32_t* __restrict__ cu,
        const float* __restrict__ a, const typename Storage<DT>::T* __restrict__ dH,
        const typename Storage<DT>::T* __restrict__ dsl, int64_t T, int64_t d_h, int64_t n_seqs, int64_t n_ch,
        int64_t n_tiles, int64_t n_chains, typename Storage<DT>::T* __restrict__ dxproj,
        typename Storage<DT>::T* __restrict__ dh0, float* __restrict__ dap, SpRecords rec, unsigned spin_limit,
        bool agg_first) {
  using ST = Storage<DT>;
  using Map = typename C::Map;
  constexpr int G = C::G, S = C::S, LC = LS * NW;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  __shared__ Map part[NW][kWave];
  __shared__ float carry_sh[S][kWave];
  __shared__ float dash[NW][G][kWave];
  __shared__ unsigned tk;

  if (threadIdx.x == 0) tk = atomicAdd(rec.ticket, 1u);
  __syncthreads();
  const int64_t ticket = static_cast<unsigned>(__builtin_amdgcn_readfirstlane(tk));
  const int64_t n_wg = n_ch * n_chains;
  const int64_t rchunk = ticket / n_chains, chain = ticket - rchunk * n_chains;
  const int64_t chunk = n_ch - 1 - rchunk;
  const int64_t b = chain / n_tiles, tile = chain - b * n_tiles;
  const int64_t ch_l = tile * kWave + lane;
  const bool ch_ok = ch_l < d_h;
  const int64_t ch = ch_ok ? ch_l : d_h - 1;  // lanes past d_h shadow the last channel (stores masked)
  const int64_t t0 = chunk * LC + static_cast<int64_t>(w) * LS;
  const bool wact = ticket < n_wg && t0 < T;
  const int n = wact ? static_cast<int>(imin(LS, T - t0)) : 0;

  // walk A: this wave's map, kept with the steps' inputs for walk B
  ChanCoef<C> cf;
  cf.load(a, d_h, ch);
  BwStep<C, DT> st[LS];
  Map acc = Map::identity();
  RevSegTracker rs;
  if (wact) {
    rs.init_wave(cu, n_seqs, b, t0 + n - 1, T);
#pragma unroll
    for (int j = LS - 1; j >= 0; --j) {
      if (j < n) {
        const int64_t t = t0 + j;
        rs.at(t);
        st[j].load(xproj, states, h0, dH, dsl, b, t, T, d_h, ch, rs);
        float fv[S];
        const Map m = C::template fj<false>(st[j].xs, st[j].prev, cf.as, cf.a, false, fv);
        acc = compose(bw_step_map(m, st[j].g, rs.last(t, T)), acc);
      }
    }
  }
  part[w][lane] = acc;
  __syncthreads();

  // the gradient entering the chunk from later chunks: one wave looks back
  const int64_t base = chain * n_ch;
  if (w == NW - 1 && ticket < n_wg) {
    Map tot = part[NW - 1][lane];
#pragma unroll
    for (int v = NW - 2; v >= 0; --v) tot = compose(part[v][lane], tot);
    float cin[S];
    // four records in flight per batch (not the forward's eight): with eight
    // the fp32 LSTM instance needs 148 registers, three waves per SIMD and so
    // one 8-wave workgroup per CU; with four, 124 and two workgroups
    // (measured: 0.98 -> 0.74 ms at 2 x 131072 x 256)
    lookback_carry<S, 4>(rec, base, rchunk, tot, lane, spin_limit, agg_first, cin);
#pragma unroll
    for (int q = 0; q < S; ++q) carry_sh[q][lane] = cin[q];
    // what leaves the chunk towards earlier ones goes out before the barrier,
    // its status right after it
    float outg[S];
#pragma unroll
    for (int q = 0; q < S; ++q) outg[q] = cin[q];
    apply(tot, outg);
#pragma unroll
    for (int q = 0; q < S; ++q) rec_store(rec.pre + (base + rchunk) * S * kWave + q * kWave + lane, outg[q]);
  }
  __syncthreads();
  if (w == NW - 1 && ticket < n_wg) rec_publish(rec.status + base + rchunk, kRecPrefix, lane);

  // walk B from this wave's carry-in
  float da[G];
#pragma unroll
  for (int g = 0; g < G; ++g) da[g] = 0.0f;
  if (wact) {
    float mu[S];
#pragma unroll
    for (int q = 0; q < S; ++q) mu[q] = carry_sh[q][lane];
    for (int v = NW - 1; v > w; --v) apply(part[v][lane], mu);
    rs.init_wave(cu, n_seqs, b, t0 + n - 1, T);
#pragma unroll
    for (int j = LS - 1; j >= 0; --j) {
      if (j < n) {
        const int64_t t = t0 + j;
        rs.at(t);
        const bool cut = rs.last(t, T);
        float lam[S];
#pragma unroll
        for (int q = 0; q < S; ++q) lam[q] = cut ? st[j].g[q] : st[j].g[q] + mu[q];
        float dx[G], dac[G];
        C::vjp(st[j].xs, st[j].prev, cf.as, cf.a, lam, dx, dac, mu);
        if (ch_ok) {
          typename ST::T* dp = dxproj + ((b * T + t) * G) * d_h + ch;
#pragma unroll
          for (int g = 0; g < G; ++g) dp[g * d_h] = ST::pack(dx[g]);
          if (dh0 && rs.head(t)) {
#pragma unroll
            for (int q = 0; q < S; ++q) dh0[(rs.seg * S + q) * d_h + ch] = ST::pack(mu[q]);
          }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) da[g] += dac[g];
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) dash[w][g][lane] = da[g];
  __syncthreads();
  if (w == 0 && ch_ok && ticket < n_wg) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = dash[0][g][lane];
#pragma unroll
      for (int v = 1; v < NW; ++v) s += dash[v][g][lane];
      dap[((b * n_ch + chunk) * G + g) * d_h + ch] = s;
    }
  }
}

// First level of the dL/da reduction: slice z of the units (per = units per
// slice) summed for every (gate, channel) in a fixed order; out is
// (n_slices, G, d_h).  k_bw_da_reduce then sums the slices.
template <int G>
__global__ void __launch_bounds__(256) k_bw_da_partial(const float* __restrict__ dap, int64_t n_units, int64_t per,
                                                       int64_t d_h, float* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1), y = threadIdx.x / kWave;
  const int64_t ch = static_cast<int64_t>(blockIdx.x) * kWave + lane;
  const int g = blockIdx.y;
  const int64_t z = blockIdx.z, u0 = z * per, u1 = imin(n_units, u0 + per);
  __shared__ float sh[4][kWave];
  float s = 0.0f;
  if (ch < d_h) {
    for (int64_t u = u0 + y; u < u1; u += 4) s += dap[(u * G + g) * d_h + ch];
  }
  sh[y][lane] = s;
  __syncthreads();
  if (y == 0 && ch < d_h) out[(z * G + g) * d_h + ch] = ((sh[0][lane] + sh[1][lane]) + sh[2][lane]) + sh[3][lane];
}

// dL/da = sum of the n_units per-chunk partials (units = B * n_ch), for every
// (gate, channel): 4 waves take every 4th unit in order, then add in order.
template <int G>
__global__ void __launch_bounds__(256) k_bw_da_reduce(const float* __restrict__ dap, int64_t n_units, int64_t d_h,
                                                      float* __restrict__ da) {
  const int lane = threadIdx.x & (kWave - 1), y = threadIdx.x / kWave;
  const int64_t ch = static_cast<int64_t>(blockIdx.x) * kWave + lane;
  const int g = blockIdx.y;
  __shared__ float sh[4][kWave];
  float s = 0.0f;
  if (ch < d_h) {
    constexpr int U = 8;
    int64_t u = y;
    for (; u + 4 * (U - 1) < n_units; u += 4 * U) {
      float v[U];
#pragma unroll
      for (int k = 0; k < U; ++k) v[k] = dap[((u + 4 * k) * G + g) * d_h + ch];
#pragma unroll
      for (int k = 0; k < U; ++k) s += v[k];
    }
    for (; u < n_units; u += 4) s += dap[(u * G + g) * d_h + ch];
  }
  sh[y][lane] = s;
  __syncthreads();
  if (y == 0 && ch < d_h) da[g * d_h + ch] = ((sh[0][lane] + sh[1][lane]) + sh[2][lane]) + sh[3][lane];
}

// dL/dh0 of an empty segment (its final state is its h0): dstate_last, or 0.
template <int DT, int S>
__global__ void k_bw_empty_dh0(const int32_t* __restrict__ cu, int64_t n_seqs, int64_t d_h,
                               const typename Storage<DT>::T* __restrict__ dsl,
                               typename Storage<DT>::T* __restrict__ dh0) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n_seqs * S * d_h) return;
  const int64_t j = i / (S * d_h);
  if (cu[j + 1] > cu[j]) return;
  dh0[i] = dsl ? dsl[i] : Storage<DT>::pack(0.0f);
}

}  // namespace prn
