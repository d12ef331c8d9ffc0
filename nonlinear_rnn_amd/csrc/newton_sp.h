// Single-pass parallel Newton: all K iterations of one chunk in one
// workgroup, the chunk's projected inputs held in registers throughout,
// carries obtained by a decoupled look-back over the preceding chunks whose
// result does not depend on timing (bitwise reproducible).
//
// The three phases of the chunked affine scan are still there, per
// iteration:  (1) the workgroup composes its chunk's maps (lane-serial over
// LS steps, then across waves through LDS);  (2) the carry across chunks
// comes from the chunk records of the predecessors: each chunk publishes its
// aggregate map, then looks back until it meets a predecessor whose
// inclusive prefix (the state after its last step) is published, composing
// aggregates on the way, and publishes its own inclusive prefix;  (3) each
// lane re-runs its steps from its carry-in (the fix-up), and the same pass
// linearises the new states for the next iteration.
//
// What this buys over separate phase kernels: the projected inputs cross
// HBM once per forward instead of once per phase, no iterate is ever
// written (only the final h), and the linearisation of iteration k+1 comes
// from the fix-up pass of iteration k (K + 1 cell evaluations per step in
// all, the last one for the final residual).
//
// Forward progress: a workgroup takes a ticket from a global counter when it
// starts, and the ticket (not blockIdx) decides its chunk, chunk-major over
// the independent chains (row, 64-channel tile).  A chunk therefore only
// ever waits for chunks with smaller tickets, which have started; chunk 0 of
// every chain never waits.  Every wait is bounded (spin_limit polls); on
// timeout the carry becomes NaN (so the residual reads +Inf) and an error
// word (the caller's, or one in the workspace) is set: the kernel always
// terminates.
//
// Memory ordering of the chunk records: every record word is written and
// read with relaxed agent-scope atomics, which gfx950 performs at the
// device-wide coherence point (sc1), never from a per-XCD cache.  A
// publishing wave stores the record's data, waits until all its stores are
// acknowledged (s_waitcnt vmcnt(0)), and only then stores the status word;
// a reader issues its data loads only after its status load has returned.
// A reader that sees a status therefore sees the data it announces.  (This
// avoids the L2 write-back / invalidate of agent-scope release / acquire
// fences, which cost about 2 us per publication here.)
#pragma once

#include "fused_proj.h"
#include "newton_kernels.h"

namespace prn {

constexpr unsigned kRecEmpty = 0, kRecAggregate = 1, kRecPrefix = 2;  // status word of a chunk record

// coherent (device-scope) record accesses
__device__ __forceinline__ void rec_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float rec_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// publish a status once every record store of this wave has completed
__device__ __forceinline__ void rec_publish(unsigned* status, unsigned v, int lane) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (lane == 0) __hip_atomic_store(status, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <int S> __device__ __forceinline__ void rec_store_map(float* p, const Aff<S>& m);
template <> __device__ __forceinline__ void rec_store_map<1>(float* p, const Aff<1>& m) {
  rec_store(p, m.a);
  rec_store(p + kWave, m.b);
}
template <> __device__ __forceinline__ void rec_store_map<2>(float* p, const Aff<2>& m) {
  rec_store(p, m.a00); rec_store(p + kWave, m.a01); rec_store(p + 2 * kWave, m.a10);
  rec_store(p + 3 * kWave, m.a11); rec_store(p + 4 * kWave, m.b0); rec_store(p + 5 * kWave, m.b1);
}
template <int S> __device__ __forceinline__ Aff<S> rec_load_map(const float* p);
template <> __device__ __forceinline__ Aff<1> rec_load_map<1>(const float* p) {
  return {rec_load(p), rec_load(p + kWave)};
}
template <> __device__ __forceinline__ Aff<2> rec_load_map<2>(const float* p) {
  return {rec_load(p), rec_load(p + kWave), rec_load(p + 2 * kWave),
          rec_load(p + 3 * kWave), rec_load(p + 4 * kWave), rec_load(p + 5 * kWave)};
}

// an LDS map slot reused for a wave's carry-in (its first S floats)
__device__ __forceinline__ void map_put_carry(Aff<1>& m, const float* c) { m.a = c[0]; }
__device__ __forceinline__ void map_put_carry(Aff<2>& m, const float* c) {
  m.a00 = c[0];
  m.a01 = c[1];
}
__device__ __forceinline__ void map_get_carry(const Aff<1>& m, float* c) { c[0] = m.a; }
__device__ __forceinline__ void map_get_carry(const Aff<2>& m, float* c) {
  c[0] = m.a00;
  c[1] = m.a01;
}

struct SpRecords {
  unsigned* status;    // [K][n_chains][n_ch]
  float* agg;          // [K][n_chains][n_ch][NC][64]
  float* pre;          // [K][n_chains][n_ch][S][64]
  unsigned* ticket;    // 1 counter
  unsigned* error;     // 1 word: set when a look-back wait timed out
};

// Carry-in E(c) of chunk c (the state just before its first step) by a
// decoupled look-back whose arithmetic does not depend on timing.  The carry
// is defined by the serial recurrence over chunks
//     E(0) = 0,   E(c+1) = A_c applied to E(c)
// (A_c the chunk's composed map; apply() is a fixed sequence of fused
// multiply-adds), and every chunk publishes its inclusive prefix E(c+1)
// computed that way.  A chunk that finds the prefix E(p+1) of a predecessor
// p behind an unbroken run of published aggregates A_{p+1} .. A_{c-1}
// applies those aggregates to that prefix, oldest first: exactly the
// operations of the serial definition, so E(c) comes out bit for bit the
// same whichever predecessor's prefix happened to be found, and repeated
// runs agree bitwise.  (Composing the run into one map first, then applying
// it, would round differently for every run length, hence with timing.)
// Executed by one whole wave (lane = channel).  Each round reads the status
// words of 64 predecessors with one load (lane i looks at chunk jh - i) and
// finds the nearest published prefix behind an unbroken run of published
// aggregates; a window of published aggregates without a prefix moves the
// scan one window further back; a run broken by an unpublished chunk before
// any prefix waits for that chunk (a chunk publishes its aggregate as soon
// as its first poll cannot resolve its own carry, or at once with few
// chains).  The aggregates are loaded RB at a time, their latencies
// overlapped.  Chunk 0 of a chain has carry 0 (its first step is a segment
// head, J = 0).  Every wait is bounded: after spin_limit polls without
// progress (none at all for spin_limit = 0) the carry becomes NaN and the
// error word is set, and the chunk goes on, so the kernel terminates.
template <int S, int RB = 8>
__device__ __forceinline__ void lookback_carry(const SpRecords& rec, int64_t base, int64_t chunk,
                                               const Aff<S>& tot, int lane, unsigned spin_limit, bool agg_first, float* cin) {
  using Map = Aff<S>;
  constexpr int NC = S * S + S;
#pragma unroll
  for (int q = 0; q < S; ++q) cin[q] = 0.0f;
  if (chunk == 0) return;
  int64_t jh = chunk - 1;
  // Our aggregate's data are stored, and the first poll is issued without
  // waiting for them: the wait for the poll also covers the stores, so the
  // status can go out right after it.  With few chains (consecutive chunks
  // of a chain start close together, so successors are already waiting) the
  // aggregate status is published after the first poll in any case; with
  // many chains the predecessor is usually done, and it is published only if
  // the first poll cannot resolve the carry.
  rec_store_map<S>(rec.agg + (base + chunk) * NC * kWave + lane, tot);
  bool published = false;
  unsigned spins = 0;
  while (true) {
    if (spins >= spin_limit) {  // gave up: poison the carry, flag the error, stop waiting
      if (lane == 0) atomicOr(rec.error, 1u);
      if (!published) rec_publish(rec.status + base + chunk, kRecAggregate, lane);
#pragma unroll
      for (int q = 0; q < S; ++q) cin[q] = __builtin_nanf("");
      return;
    }
    const int64_t jj = jh - lane;
    const unsigned st = jj >= 0 ? __hip_atomic_load(rec.status + base + jj, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                : kRecEmpty;
    const unsigned long long ready = __ballot(st != kRecEmpty);
    const unsigned long long pref = __ballot(st == kRecPrefix);
    const int n_ready = ~ready ? __builtin_ctzll(~ready) : 64;
    const int i_p = pref ? __builtin_ctzll(pref) : 64;
    const bool hit = i_p < n_ready;
    if ((agg_first || !hit) && !published) {
      rec_publish(rec.status + base + chunk, kRecAggregate, lane);
      published = true;
    }
    if (hit) {
      // E(c) = A_{c-1}( ... A_{p+1}(E(p+1)) ... ), p = jh - i_p; the
      // prefix is loaded in the same batch as the first aggregates
      const int64_t p = jh - i_p, n_app = chunk - 1 - p;
      float e[S];
      const float* pp = rec.pre + (base + p) * S * kWave + lane;
#pragma unroll
      for (int q = 0; q < S; ++q) e[q] = rec_load(pp + q * kWave);
      for (int64_t r0 = 0; r0 < n_app; r0 += RB) {
        Map mb[RB];
#pragma unroll
        for (int u = 0; u < RB; ++u)
          mb[u] = (r0 + u < n_app) ? rec_load_map<S>(rec.agg + (base + p + 1 + r0 + u) * NC * kWave + lane)
                                   : Map::identity();
#pragma unroll
        for (int u = 0; u < RB; ++u)
          if (r0 + u < n_app) apply(mb[u], e);
      }
#pragma unroll
      for (int q = 0; q < S; ++q) cin[q] = e[q];
      return;
    }
    if (n_ready == kWave) {  // 64 published aggregates and no prefix: look one window further back
      jh -= kWave;
      continue;
    }
    ++spins;   // the run breaks at a chunk that has published nothing yet
    __builtin_amdgcn_s_sleep(2);
  }
}

// WS: also write every state of the final trajectory to sout (the training
// forward); a separate instance, so that the plain forward's registers are
// not spent on it.  PIC: P = picard >= 1 Picard (Jacobi) sweeps
// H <- f(shift(H), x) from H = 0 before the Newton iterations, so iteration
// 1 linearises at the guess H^(P) rather than at 0, and r_0 is the residual
// of H^(P).  H^(P)_t depends on the P steps up to t only (it is the unroll
// started from 0 P steps back, or from h0 at a head inside that window), so
// every wave builds the guess of its own sub-chunk: P sweeps over its steps
// in registers, each starting from H^(p-1) of the step before the sub-chunk,
// which a short unroll over the p - 1 steps before it (from xproj, or from
// h0 at the segment's head) supplies.
// Waves per SIMD the compiler must leave room for: two for the longest
// chunk (LS = 16, fp32 LSTM: 205 registers, 207 with states_out; a bound
// that only matters if a change pushes it past 256, where one wave per SIMD
// would halve the resident waves); no constraint otherwise.  The
// fused-projection instances (FX) hold the projection's accumulators on top
// of the Newton state and are capped the same way.
template <class C, int DT, int LS, bool FX>
constexpr int sp_min_waves() {
  return (FX || (C::S == 2 && DT == kF32 && LS >= 16)) ? 2 : 1;
}

// LDS of the chunk's projected inputs; with the fused projection (FX) the
// same memory first stages that projection's operands
template <class C, int LS, int NW, bool FX>
constexpr int sp_xsh_bytes() {
  constexpr int xsh = LS * C::G * kWave * NW * 4;
  if constexpr (FX) {
    constexpr int st = FxGeom<C, LS, NW>::BYTES;
    return st > xsh ? st : xsh;
  } else {
    return xsh;
  }
}

// FX: the chunk's projected inputs are computed here from x and W on the
// matrix cores (fused_tile) instead of being read from xproj.
template <class C, int DT, int LS, int NW, bool WS, bool PIC, bool FX>
__global__ void __launch_bounds__(kWave * NW) __attribute__((amdgpu_waves_per_eu(sp_min_waves<C, DT, LS, FX>())))
k_newton_sp(const typename Storage<DT>::T* __restrict__ xproj, const typename Storage<DT>::T* __restrict__ h0,
            const int32_t* __restrict__ cu, const float* __restrict__ a, int64_t T, int64_t d_h,
            int64_t n_seqs, int64_t n_ch, int64_t n_tiles, int64_t n_chains, int K,
            typename Storage<DT>::T* __restrict__ Hout, typename Storage<DT>::T* __restrict__ slast,
            typename Storage<DT>::T* __restrict__ sout, float* __restrict__ rpart, SpRecords rec,
            unsigned spin_limit, bool agg_first, FxArgs fx, int picard) {
  using ST = Storage<DT>;
  using Map = typename C::Map;
  constexpr int G = C::G, S = C::S, LC = LS * NW;
  static_assert(!(FX && PIC), "the Picard sweep reads the step before the chunk, which the fused tile lacks");
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform, kept in SGPRs
  // part[w][lane]: wave w's sub-chunk map, written before an iteration's
  // first barrier; the look-back wave reads every slot and overwrites it
  // with that wave's carry-in (map_put_carry) before the second barrier.
  // A wave reads only its own slot after that and rewrites it only in the
  // next iteration, so one buffer serves every iteration.
  __shared__ Map part[NW][kWave];
  __shared__ unsigned red[NW];
  __shared__ unsigned tk;
  // the chunk's scaled projected inputs, read-only after the first walk:
  // [step][gate][thread] (consecutive lanes, consecutive banks)
  __shared__ __attribute__((aligned(16))) float xraw[sp_xsh_bytes<C, LS, NW, FX>() / 4];
  float(*xsh)[G][kWave * NW] = reinterpret_cast<float(*)[G][kWave * NW]>(xraw);

  if (threadIdx.x == 0) tk = atomicAdd(rec.ticket, 1u);
  __syncthreads();
  const int64_t ticket = static_cast<unsigned>(__builtin_amdgcn_readfirstlane(tk));
  const int64_t n_wg = n_ch * n_chains;
  const int64_t chunk = ticket / n_chains, chain = ticket - chunk * n_chains;
  const int64_t b = chain / n_tiles, tile = chain - b * n_tiles;
  const int64_t ch_l = tile * kWave + lane;
  const bool ch_ok = ch_l < d_h;
  const int64_t ch = ch_ok ? ch_l : d_h - 1;  // lanes past d_h shadow the last channel (stores masked)
  const int64_t t0 = chunk * LC + static_cast<int64_t>(w) * LS;
  const bool wact = ticket < n_wg && t0 < T;
  const int n = wact ? static_cast<int>(imin(LS, T - t0)) : 0;
  SegTracker sg;
  sg.init_wave(cu, n_seqs, b, t0);
  // a full sub-chunk without a segment head needs no per-step guards
  const bool fast = n == LS && t0 != 0 && sg.start != t0 && sg.next >= t0 + LS;
  if constexpr (FX) fused_tile<C, DT, LS, NW>(reinterpret_cast<uint8_t*>(xraw), fx, b, T, chunk * LC, tile, d_h, xsh);

  ChanCoef<C> cf;
  cf.load(a, d_h, ch);
  Map ms[LS];
  auto xs_put = [&](int j, const float* v) {
#pragma unroll
    for (int g = 0; g < G; ++g) xsh[j][g][threadIdx.x] = v[g];
  };
  auto xs_get = [&](int j, float* v) {
#pragma unroll
    for (int g = 0; g < G; ++g) v[g] = xsh[j][g][threadIdx.x];
  };
  Map acc = Map::identity();
  unsigned rmax = 0;
  const typename ST::T* xp = xproj + ((b * T + t0) * G) * d_h + ch;
  typename ST::T* hp = Hout + (b * T + t0) * d_h + ch;
  typename ST::T* sp = WS ? sout + (b * T + t0) * S * d_h + ch : nullptr;

  // H^(p)_{t0-1}, the Picard iterate p of the step before the sub-chunk
  // (PIC; t0 not a head, so that step lies in the segment of t0): the
  // unroll over the p steps before t0, started from 0, or from h0 at the
  // segment's head where that falls inside them; every value is rounded to
  // the storage type like a stored sweep
  auto picard_before = [&](int p, float* pm) {
#pragma unroll
    for (int q = 0; q < S; ++q) pm[q] = 0.0f;
    int64_t s0 = t0 - p;
    if (s0 <= sg.start) {
      s0 = sg.start;
      if (h0) load_state<DT, S>(h0 + sg.seg * S * d_h + ch, d_h, pm);
    }
    for (int64_t t = s0; t < t0; ++t) {
      float xm[G], nx[S];
      load_xs<C, DT>(xp - (t0 - t) * G * d_h, d_h, xm);
      C::f(xm, pm, cf.as, cf.a, nx);
#pragma unroll
      for (int q = 0; q < S; ++q) pm[q] = ST::round(nx[q]);
    }
  };
  // the Picard guess H^(picard) at the sub-chunk's n steps, in place in hv;
  // HD: the sub-chunk may hold segment heads (h0 there instead of the step
  // before); t0 at a head needs no step before
  auto picard_guess = [&](const float(*xs)[G], float(*hv)[S], int n, auto hd) {
    constexpr bool HD = decltype(hd)::value;
    const bool before = t0 != 0 && sg.start != t0;
#pragma unroll
    for (int j = 0; j < LS; ++j) {
#pragma unroll
      for (int q = 0; q < S; ++q) hv[j][q] = 0.0f;   // H^(0)
    }
    for (int p = 1; p <= picard; ++p) {
      float c[S];   // H^(p-1) of the step before the one being swept
      if (p > 1 && before) {
        picard_before(p - 1, c);
      } else {
#pragma unroll
        for (int q = 0; q < S; ++q) c[q] = 0.0f;
      }
      SegTracker st = sg;
#pragma unroll
      for (int j = 0; j < LS; ++j) {
        if (!HD || j < n) {
          float prev[S];
#pragma unroll
          for (int q = 0; q < S; ++q) prev[q] = c[q];
          if (HD && st.at(t0 + j)) {
#pragma unroll
            for (int q = 0; q < S; ++q) prev[q] = 0.0f;
            if (h0) load_state<DT, S>(h0 + st.seg * S * d_h + ch, d_h, prev);
          }
          float nx[S];
          C::f(xs[j], prev, cf.as, cf.a, nx);
#pragma unroll
          for (int q = 0; q < S; ++q) {
            c[q] = hv[j][q];
            hv[j][q] = ST::round(nx[q]);
          }
        }
      }
    }
  };

  // ---- load the tile; linearise iteration 1 at H^(0) = 0 (h0 at heads), or
  // at the Picard guess H^(P) ----
  if (fast) {
    float xs[LS][G];
#pragma unroll
    for (int j = 0; j < LS; ++j) {
      if constexpr (FX)
        xs_get(j, xs[j]);
      else
        load_xs<C, DT>(xp + j * G * d_h, d_h, xs[j]);
    }
    float hv[PIC ? LS : 1][S];
    float pm[S];
    if constexpr (PIC) {
      picard_guess(xs, hv, LS, std::false_type{});
      picard_before(picard, pm);
    }
#pragma unroll
    for (int j = 0; j < LS; ++j) {
      if constexpr (!FX) xs_put(j, xs[j]);
      float fv[S];
      if constexpr (PIC) {
        ms[j] = C::template fj<false>(xs[j], j ? hv[j - 1] : pm, cf.as, cf.a, false, fv);
#pragma unroll
        for (int q = 0; q < S; ++q) rmax = rmax_bits(rmax, hv[j][q] - fv[q]);
      } else {
        ms[j] = C::fj0(xs[j], cf.a, fv);  // linearised at H^(0) = 0
#pragma unroll
        for (int q = 0; q < S; ++q) rmax = rmax_bits(rmax, fv[q]);
      }
      acc = compose(ms[j], acc);
    }
  } else if (wact) {
    float xs[LS][G];
#pragma unroll
    for (int j = 0; j < LS; ++j) {
      if (j < n) {
        if constexpr (FX)
          xs_get(j, xs[j]);
        else
          load_xs<C, DT>(xp + j * G * d_h, d_h, xs[j]);
      }
    }
    float hv[PIC ? LS : 1][S];
    float pm[S];
    if constexpr (PIC) {
      picard_guess(xs, hv, n, std::true_type{});
#pragma unroll
      for (int q = 0; q < S; ++q) pm[q] = 0.0f;
      if (t0 != 0 && sg.start != t0) picard_before(picard, pm);
    }
    SegTracker st = sg;
#pragma unroll
    for (int j = 0; j < LS; ++j) {
      if (j < n) {
        if constexpr (!FX) xs_put(j, xs[j]);
        const bool head = st.at(t0 + j);
        float prev[S], fv[S];
        if constexpr (PIC) {
#pragma unroll
          for (int q = 0; q < S; ++q) prev[q] = j ? hv[j - 1][q] : pm[q];
        } else {
#pragma unroll
          for (int q = 0; q < S; ++q) prev[q] = 0.0f;
        }
        if (head) {
#pragma unroll
          for (int q = 0; q < S; ++q) prev[q] = 0.0f;
          if (h0) load_state<DT, S>(h0 + st.seg * S * d_h + ch, d_h, prev);
        }
        ms[j] = C::fj(xs[j], prev, cf.as, cf.a, head, fv);
        acc = compose(ms[j], acc);
        if constexpr (PIC) {
#pragma unroll
          for (int q = 0; q < S; ++q) rmax = rmax_bits(rmax, hv[j][q] - fv[q]);
        } else {
#pragma unroll
          for (int q = 0; q < S; ++q) rmax = rmax_bits(rmax, fv[q]);
        }
      }
    }
  }

  // residual r_k: each wave leaves its maximum in red[], and after the next
  // workgroup barrier (the one that exchanges the waves' maps) thread 0
  // combines them; red[] is not written again before the look-back barrier
  auto residual_put = [&](unsigned r) {
    r = wave_max_u32(r);
    if (lane == 0) red[w] = r;
  };
  auto residual_finish = [&](int k) {
    if (threadIdx.x == 0 && rpart && ticket < n_wg) {
      unsigned r = red[0];
#pragma unroll
      for (int v = 1; v < NW; ++v) r = max(r, red[v]);
      rpart[k * n_wg + ticket] = rmax_finish(r);
    }
  };
  residual_put(rmax);

  // iteration k; the last one (LAST) is a separate copy after the loop, so
  // that the maps the loop carries keep one register assignment (with the
  // last iteration inside the loop, the compiler copied all LS maps at both
  // ends of the loop body)
  auto iteration = [&](int k, auto last_t) __attribute__((always_inline)) {
    constexpr bool last = decltype(last_t)::value;
    part[w][lane] = acc;
    __syncthreads();
    residual_finish(k);

    // ---- carry across chunks: one wave publishes and looks back ----
    if (w == NW - 1 && ticket < n_wg) {
      Map tot = part[0][lane];
#pragma unroll
      for (int v = 1; v < NW; ++v) tot = compose(part[v][lane], tot);
      const int64_t base = (static_cast<int64_t>(k) * n_chains + chain) * n_ch;
      float cin[S];
      lookback_carry<S>(rec, base, chunk, tot, lane, spin_limit, agg_first, cin);
      // each wave's carry-in: the chunk's, through the maps of the waves
      // before it, applied in wave order
      float c[S];
#pragma unroll
      for (int q = 0; q < S; ++q) c[q] = cin[q];
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const Map m = part[v][lane];
        map_put_carry(part[v][lane], c);
        if (v + 1 < NW) apply(m, c);
      }
      // the inclusive prefix (state after the chunk's last step) goes out
      // before the barrier; its status is published right after it, while
      // the other waves already start their fix-up
      float incl[S];
#pragma unroll
      for (int q = 0; q < S; ++q) incl[q] = cin[q];
      apply(tot, incl);
#pragma unroll
      for (int q = 0; q < S; ++q) rec_store(rec.pre + (base + chunk) * S * kWave + q * kWave + lane, incl[q]);
    }
    __syncthreads();
    if (w == NW - 1 && ticket < n_wg)
      rec_publish(rec.status + (static_cast<int64_t>(k) * n_chains + chain) * n_ch + chunk, kRecPrefix, lane);

    // ---- fix-up of iteration k+1, linearisation of iteration k+2 ----
    // The output addresses are formed at the stores: an opaque copy of the
    // bases per iteration keeps the compiler from hoisting LS 64-bit
    // addresses out of the iteration loop, which would hold their registers
    // through every iteration (fp32 LSTM at LS = 12: 236 -> 213 VGPRs, which
    // is what lets LS = 16 fit two waves per SIMD).  The fp32 GRU fits three
    // waves per SIMD either way and measured faster with the hoisted form.
    typename ST::T* hq = hp;
    typename ST::T* sq = sp;
    typename ST::T* lq = slast;
    int64_t dq = d_h;
    if constexpr (!(S == 1 && DT == kF32)) asm volatile("" : "+v"(hq), "+v"(sq), "+s"(lq), "+s"(dq));
    acc = Map::identity();
    rmax = 0;
    float s[S];
    map_get_carry(part[w][lane], s);
    float pr[S];
#pragma unroll
    for (int q = 0; q < S; ++q) pr[q] = ST::round(s[q]);
    if (fast) {
      if constexpr (!last) {
#pragma unroll
        for (int j = 0; j < LS; ++j) {
          apply(ms[j], s);
          float fv[S], xj[G];
          xs_get(j, xj);
          ms[j] = C::template fj<false>(xj, pr, cf.as, cf.a, false, fv);
          acc = compose(ms[j], acc);
#pragma unroll
          for (int q = 0; q < S; ++q) {
            const float sr = ST::round(s[q]);
            rmax = rmax_bits(rmax, sr - fv[q]);
            pr[q] = sr;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < LS; ++j) {
          apply(ms[j], s);
          float fv[S], xj[G];
          xs_get(j, xj);
          C::f(xj, pr, cf.as, cf.a, fv);
          if (ch_ok) {
            gstore(hq + j * dq, ST::pack(s[S - 1]));
            if constexpr (WS) {
#pragma unroll
              for (int q = 0; q < S; ++q) gstore(sq + (j * S + q) * dq, ST::pack(s[q]));
            }
          }
#pragma unroll
          for (int q = 0; q < S; ++q) {
            const float sr = ST::round(s[q]);
            rmax = rmax_bits(rmax, sr - fv[q]);
            pr[q] = sr;
          }
        }
        if (slast && ch_ok && (t0 + LS == T || sg.next == t0 + LS)) {
#pragma unroll
          for (int q = 0; q < S; ++q) gstore(lq + (sg.seg * S + q) * dq + ch, ST::pack(s[q]));
        }
      }
    } else if (wact) {
      SegTracker st = sg;
#pragma unroll
      for (int j = 0; j < LS; ++j) {
        if (j < n) {
          const int64_t t = t0 + j;
          const bool head = st.at(t);
          apply(ms[j], s);
          float p[S];
#pragma unroll
          for (int q = 0; q < S; ++q) p[q] = pr[q];
          if (head) {
#pragma unroll
            for (int q = 0; q < S; ++q) p[q] = 0.0f;
            if (h0) load_state<DT, S>(h0 + st.seg * S * d_h + ch, d_h, p);
          }
          float fv[S], xj[G];
          xs_get(j, xj);
          if constexpr (!last) {
            ms[j] = C::fj(xj, p, cf.as, cf.a, head, fv);
            acc = compose(ms[j], acc);
          } else {
            C::f(xj, p, cf.as, cf.a, fv);
            if (ch_ok) {
              gstore(hq + j * dq, ST::pack(s[S - 1]));
              if constexpr (WS) {
#pragma unroll
                for (int q = 0; q < S; ++q) gstore(sq + (j * S + q) * dq, ST::pack(s[q]));
              }
              if (slast && st.last(t, T)) {
#pragma unroll
                for (int q = 0; q < S; ++q) gstore(lq + (st.seg * S + q) * dq + ch, ST::pack(s[q]));
              }
            }
          }
#pragma unroll
          for (int q = 0; q < S; ++q) {
            const float sr = ST::round(s[q]);
            rmax = rmax_bits(rmax, sr - fv[q]);
            pr[q] = sr;
          }
        }
      }
    }
    residual_put(rmax);
  };
  for (int k = 0; k < K - 1; ++k) iteration(k, std::false_type{});
  iteration(K - 1, std::true_type{});
  __syncthreads();
  residual_finish(K);
}

}  // namespace prn
