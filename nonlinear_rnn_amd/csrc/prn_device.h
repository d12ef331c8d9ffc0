// Device building blocks shared by the Newton, scan and sequential kernels:
// storage-dtype loads/stores, fast transcendentals, the two diagonal cells
// with their closed-form per-channel Jacobians, and per-channel affine maps.
//
// Everything is fp32 arithmetic whatever the storage dtype (FAQs, "What about
// Turing GPUs": the algebra inside the kernel stays fp32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prn {

constexpr int kWave = 64;

__device__ __forceinline__ int64_t imin(int64_t x, int64_t y) { return x < y ? x : y; }
__device__ __forceinline__ int64_t imax(int64_t x, int64_t y) { return x > y ? x : y; }

// ----------------------------------------------------------- dtypes -------

enum StorageType { kF32 = 0, kBF16 = 1 };

template <int DT> struct Storage;
template <> struct Storage<kF32> {
  using T = float;
  static __device__ __forceinline__ float load(const T* p) { return *p; }
  static __device__ __forceinline__ T pack(float v) { return v; }
  static __device__ __forceinline__ float round(float v) { return v; }
};
template <> struct Storage<kBF16> {
  using T = uint16_t;
  static __device__ __forceinline__ float load(const T* p) {
    return __uint_as_float(static_cast<uint32_t>(*p) << 16);
  }
  // round to nearest, ties to even (gfx950's v_cvt_pk_bf16_f32; a NaN stays
  // a quiet NaN); two instructions per rounding instead of a software
  // sequence of about seven
  static __device__ __forceinline__ T pack(float v) { return __builtin_bit_cast(T, static_cast<__bf16>(v)); }
  static __device__ __forceinline__ float round(float v) { return static_cast<float>(static_cast<__bf16>(v)); }
};

// A store through the global address space.  A pointer that went through an
// empty asm statement (to keep the compiler from hoisting addresses) is only
// known as a generic pointer, and a plain store to it becomes a flat store,
// which the LDS counter tracks as well: every later wait for an LDS read then
// also waits for the store to complete.
template <class T>
__device__ __forceinline__ void gstore(T* p, T v) {
  *(__attribute__((address_space(1))) T*)p = v;
}

// ------------------------------------------------- transcendentals -------
// v_exp_f32 computes 2^x and v_rcp_f32 1/x, each to about 1 ulp.  Gate
// pre-activations are carried pre-multiplied by the factor that turns them
// into the exponent the gate needs ("scaled" values v):
//   sig(u)  = 1 / (1 + 2^v),        v = -log2(e) u
//   tanh(u) = 2 / (1 + 2^v) - 1,    v = -2 log2(e) u
// so a gate costs one fma (v = as * h + xs), one exp, one add, one rcp.
// Saturation is exact at both ends (2^(+big) = inf -> rcp = 0).

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSigScale = -kLog2e;          // logistic gates
constexpr float kTanhScale = -2.0f * kLog2e;  // tanh gates

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float sig_s(float v) { return rcp(1.0f + ex2(v)); }
__device__ __forceinline__ float tanh_s(float v) { return fmaf(2.0f, rcp(1.0f + ex2(v)), -1.0f); }

// |x| with NaN mapped to +Inf, so that a max over residuals never drops a NaN
__device__ __forceinline__ float abs_nan_inf(float x) {
  const float v = fabsf(x);
  return __builtin_isnan(v) ? __builtin_inff() : v;
}
// running max of |x| on IEEE bit patterns: every NaN pattern of |x| orders
// above +Inf, so NaN survives (mapped to +Inf by rmax_finish)
__device__ __forceinline__ unsigned rmax_bits(unsigned r, float x) { return max(r, __float_as_uint(x) & 0x7fffffffu); }
__device__ __forceinline__ float rmax_finish(unsigned r) {
  return r > 0x7f800000u ? __builtin_inff() : __uint_as_float(r);
}
// maximum of r over the wave, in every lane, without LDS: within each
// 16-lane row by DPP (partners l ^ 1, l ^ 2 by quad permutations, then the
// mirror images in 8 and in 16 lanes), then across rows and halves by the
// gfx950 row swaps (the two results of a swap hold, in each lane, its own
// row's value and the partner row's)
__device__ __forceinline__ unsigned wave_max_u32(unsigned r) {
  r = max(r, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(r), 0xb1, 0xf, 0xf, false)));
  r = max(r, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(r), 0x4e, 0xf, 0xf, false)));
  r = max(r, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(r), 0x141, 0xf, 0xf, false)));
  r = max(r, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(r), 0x140, 0xf, 0xf, false)));
  const auto x = __builtin_amdgcn_permlane16_swap(r, r, false, false);
  r = max(x[0], x[1]);
  const auto y = __builtin_amdgcn_permlane32_swap(r, r, false, false);
  return max(y[0], y[1]);
}

// ---------------------------------------------------- affine maps --------
// One channel's map s -> A s + b (S = 1 or 2).  compose(m2, m1) is "m2 after
// m1": (A2 A1, A2 b1 + b2).

template <int S> struct Aff;
template <> struct Aff<1> {
  float a, b;
  static __device__ __forceinline__ Aff identity() { return {1.0f, 0.0f}; }
};
template <> struct Aff<2> {
  float a00, a01, a10, a11, b0, b1;
  static __device__ __forceinline__ Aff identity() { return {1.0f, 0.0f, 0.0f, 1.0f, 0.0f, 0.0f}; }
};

__device__ __forceinline__ Aff<1> compose(const Aff<1>& m2, const Aff<1>& m1) {
  return {m2.a * m1.a, fmaf(m2.a, m1.b, m2.b)};
}
__device__ __forceinline__ Aff<2> compose(const Aff<2>& m2, const Aff<2>& m1) {
  Aff<2> r;
  r.a00 = fmaf(m2.a00, m1.a00, m2.a01 * m1.a10);
  r.a01 = fmaf(m2.a00, m1.a01, m2.a01 * m1.a11);
  r.a10 = fmaf(m2.a10, m1.a00, m2.a11 * m1.a10);
  r.a11 = fmaf(m2.a10, m1.a01, m2.a11 * m1.a11);
  r.b0 = fmaf(m2.a00, m1.b0, fmaf(m2.a01, m1.b1, m2.b0));
  r.b1 = fmaf(m2.a10, m1.b0, fmaf(m2.a11, m1.b1, m2.b1));
  return r;
}
__device__ __forceinline__ void apply(const Aff<1>& m, float* s) { s[0] = fmaf(m.a, s[0], m.b); }
__device__ __forceinline__ void apply(const Aff<2>& m, float* s) {
  const float c = s[0], h = s[1];
  s[0] = fmaf(m.a00, c, fmaf(m.a01, h, m.b0));
  s[1] = fmaf(m.a10, c, fmaf(m.a11, h, m.b1));
}

// --------------------------------------------------------- cells ---------
// Per-channel constants: a (recurrent weights, for the Jacobian) and as =
// a * scale(gate) (for the scaled pre-activations).  Projected inputs are
// passed scaled the same way: xs[g] = x[g] * scale(g) (Cell::scale(g)).
//
// fj(): f(s) and the per-channel Jacobian J = df/ds at state s, packed as the
// Newton map (J, b = f - J s).  At a segment head the caller passes head =
// true: J := 0 and b := f(h0) (shapes/layout page: J = 0 on the scan).
// f(): the cell value only (residual of the final iterate).

struct CellGRU {
  static constexpr int G = 3, S = 1;
  using Map = Aff<1>;
  // gates [z, r, c]; state [h]
  static constexpr __host__ __device__ float scale(int g) { return g == 2 ? kTanhScale : kSigScale; }
  static __device__ __forceinline__ void f(const float* xs, const float* s, const float* as, const float* /*a*/,
                                           float* out) {
    const float h = s[0];
    const float z = sig_s(fmaf(as[0], h, xs[0]));
    const float r = sig_s(fmaf(as[1], h, xs[1]));
    const float c = tanh_s(fmaf(as[2], r * h, xs[2]));
    out[0] = fmaf(z, c - h, h);
  }
  template <bool HEAD_POSSIBLE = true>
  static __device__ __forceinline__ Map fj(const float* xs, const float* s, const float* as, const float* a,
                                           bool head, float* fout) {
    const float h = s[0];
    const float z = sig_s(fmaf(as[0], h, xs[0]));
    const float r = sig_s(fmaf(as[1], h, xs[1]));
    const float c = tanh_s(fmaf(as[2], r * h, xs[2]));
    const float fv = fmaf(z, c - h, h);
    fout[0] = fv;
    if (HEAD_POSSIBLE && head) return {0.0f, fv};
    const float omz = 1.0f - z;
    const float dz = z * omz * a[0];
    const float dr = r * (1.0f - r) * a[1];
    const float dc = fmaf(-c, c, 1.0f) * a[2] * fmaf(h, dr, r);
    const float J = fmaf(z, dc, fmaf(c - h, dz, omz));
    return {J, fmaf(-J, h, fv)};
  }
  // fj at the zero state (the first linearisation, from H = 0, away from a
  // segment head): the terms that vanish with h are left out.  Equal to
  // fj(xs, {0}) for finite operands.
  static __device__ __forceinline__ Map fj0(const float* xs, const float* a, float* fout) {
    const float z = sig_s(xs[0]);
    const float r = sig_s(xs[1]);
    const float c = tanh_s(xs[2]);
    const float fv = z * c;
    fout[0] = fv;
    const float omz = 1.0f - z;
    const float dz = z * omz * a[0];
    const float dc = fmaf(-c, c, 1.0f) * a[2] * r;
    return {fmaf(z, dc, fmaf(c, dz, omz)), fv};
  }
  // Backward of one step at (s, x) with cotangent lam = dL/dh': the
  // pre-activation gradients du_g (= dL/dx_g), dL/da_g = du_g * m_g (m = h,
  // h, r h) and dL/dh = J^T lam.
  static __device__ __forceinline__ void vjp(const float* xs, const float* s, const float* as, const float* a,
                                             const float* lam, float* dx, float* da, float* dprev) {
    const float h = s[0];
    const float z = sig_s(fmaf(as[0], h, xs[0]));
    const float r = sig_s(fmaf(as[1], h, xs[1]));
    const float rh = r * h;
    const float c = tanh_s(fmaf(as[2], rh, xs[2]));
    const float L = lam[0];
    const float zl = z * L;
    const float du_z = L * (c - h) * z * (1.0f - z);
    const float du_c = zl * fmaf(-c, c, 1.0f);
    const float du_r = du_c * a[2] * h * r * (1.0f - r);
    dx[0] = du_z;
    dx[1] = du_r;
    dx[2] = du_c;
    da[0] = du_z * h;
    da[1] = du_r * h;
    da[2] = du_c * rh;
    dprev[0] = fmaf(du_c * a[2], r, fmaf(du_r, a[1], fmaf(du_z, a[0], L - zl)));
  }
};

struct CellLSTM {
  static constexpr int G = 4, S = 2;
  using Map = Aff<2>;
  // gates [i, f, o, g]; state [c, h]
  static constexpr __host__ __device__ float scale(int g) { return g == 3 ? kTanhScale : kSigScale; }
  static __device__ __forceinline__ void f(const float* xs, const float* s, const float* as, const float* /*a*/,
                                           float* out) {
    const float c = s[0], h = s[1];
    const float ig = sig_s(fmaf(as[0], h, xs[0]));
    const float fg = sig_s(fmaf(as[1], h, xs[1]));
    const float og = sig_s(fmaf(as[2], h, xs[2]));
    const float gg = tanh_s(fmaf(as[3], h, xs[3]));
    const float c1 = fmaf(fg, c, ig * gg);
    out[0] = c1;
    out[1] = og * tanh_s(c1 * kTanhScale);
  }
  template <bool HEAD_POSSIBLE = true>
  static __device__ __forceinline__ Map fj(const float* xs, const float* s, const float* as, const float* a,
                                           bool head, float* fout) {
    const float c = s[0], h = s[1];
    const float ig = sig_s(fmaf(as[0], h, xs[0]));
    const float fg = sig_s(fmaf(as[1], h, xs[1]));
    const float og = sig_s(fmaf(as[2], h, xs[2]));
    const float gg = tanh_s(fmaf(as[3], h, xs[3]));
    const float c1 = fmaf(fg, c, ig * gg);
    const float tc = tanh_s(c1 * kTanhScale);
    const float h1 = og * tc;
    fout[0] = c1;
    fout[1] = h1;
    if (HEAD_POSSIBLE && head) return {0.0f, 0.0f, 0.0f, 0.0f, c1, h1};
    const float di = ig * (1.0f - ig) * a[0];
    const float df = fg * (1.0f - fg) * a[1];
    const float dO = og * (1.0f - og) * a[2];
    const float dg = fmaf(-gg, gg, 1.0f) * a[3];
    const float j01 = fmaf(c, df, fmaf(gg, di, ig * dg));   // dc'/dh
    const float odt = og * fmaf(-tc, tc, 1.0f);             // o (1 - tanh^2 c')
    const float j10 = odt * fg;                             // dh'/dc
    const float j11 = fmaf(tc, dO, odt * j01);              // dh'/dh
    Map m;
    m.a00 = fg;
    m.a01 = j01;
    m.a10 = j10;
    m.a11 = j11;
    m.b0 = c1 - fmaf(fg, c, j01 * h);
    m.b1 = h1 - fmaf(j10, c, j11 * h);
    return m;
  }
  // fj at the zero state (c, h) = 0 (the first linearisation, from H = 0,
  // away from a segment head): the terms that vanish with c and h are left
  // out.  Equal to fj(xs, {0, 0}) for finite operands.
  static __device__ __forceinline__ Map fj0(const float* xs, const float* a, float* fout) {
    const float ig = sig_s(xs[0]);
    const float fg = sig_s(xs[1]);
    const float og = sig_s(xs[2]);
    const float gg = tanh_s(xs[3]);
    const float c1 = ig * gg;
    const float tc = tanh_s(c1 * kTanhScale);
    const float h1 = og * tc;
    fout[0] = c1;
    fout[1] = h1;
    const float di = ig * (1.0f - ig) * a[0];
    const float dO = og * (1.0f - og) * a[2];
    const float dg = fmaf(-gg, gg, 1.0f) * a[3];
    const float j01 = fmaf(gg, di, ig * dg);
    const float odt = og * fmaf(-tc, tc, 1.0f);
    Map m;
    m.a00 = fg;
    m.a01 = j01;
    m.a10 = odt * fg;
    m.a11 = fmaf(tc, dO, odt * j01);
    m.b0 = c1;
    m.b1 = h1;
    return m;
  }
  // Backward of one step at (s, x) with cotangent lam = (dL/dc', dL/dh'):
  // pre-activation gradients du_g (= dL/dx_g), dL/da_g = du_g * h and
  // (dL/dc, dL/dh) = J^T lam.
  static __device__ __forceinline__ void vjp(const float* xs, const float* s, const float* as, const float* a,
                                             const float* lam, float* dx, float* da, float* dprev) {
    const float c = s[0], h = s[1];
    const float ig = sig_s(fmaf(as[0], h, xs[0]));
    const float fg = sig_s(fmaf(as[1], h, xs[1]));
    const float og = sig_s(fmaf(as[2], h, xs[2]));
    const float gg = tanh_s(fmaf(as[3], h, xs[3]));
    const float c1 = fmaf(fg, c, ig * gg);
    const float tc = tanh_s(c1 * kTanhScale);
    const float dc1 = fmaf(lam[1] * og, fmaf(-tc, tc, 1.0f), lam[0]);  // total dL/dc'
    const float du_i = dc1 * gg * ig * (1.0f - ig);
    const float du_f = dc1 * c * fg * (1.0f - fg);
    const float du_o = lam[1] * tc * og * (1.0f - og);
    const float du_g = dc1 * ig * fmaf(-gg, gg, 1.0f);
    dx[0] = du_i;
    dx[1] = du_f;
    dx[2] = du_o;
    dx[3] = du_g;
#pragma unroll
    for (int g = 0; g < 4; ++g) da[g] = dx[g] * h;
    dprev[0] = dc1 * fg;
    dprev[1] = fmaf(du_g, a[3], fmaf(du_o, a[2], fmaf(du_f, a[1], du_i * a[0])));
  }
};

// per-channel constants of a cell
template <class C>
struct ChanCoef {
  float a[C::G], as[C::G];
  __device__ __forceinline__ void load(const float* __restrict__ aw, int64_t d_h, int64_t ch) {
#pragma unroll
    for (int g = 0; g < C::G; ++g) {
      a[g] = aw[g * d_h + ch];
      as[g] = a[g] * C::scale(g);
    }
  }
};

// load one step's projected inputs (G values, stride d_h apart) scaled for the gates
template <class C, int DT>
__device__ __forceinline__ void load_xs(const typename Storage<DT>::T* p, int64_t d_h, float* xs) {
#pragma unroll
  for (int g = 0; g < C::G; ++g) xs[g] = Storage<DT>::load(p + g * d_h) * C::scale(g);
}

// ------------------------------------------------ segment tracking -------
// Which steps are segment heads, and which segment a step belongs to.
// Rectangular batch: row b is one segment (index b) starting at t = 0.
// Ragged pack: segment j covers [cu[j], cu[j+1]); empty segments are
// skipped.  Indices stay in [0, n_seqs) whatever cu holds.

struct SegTracker {
  const int32_t* cu;  // null for a rectangular batch
  int64_t n_seqs;
  int64_t seg;        // current segment (row b for a rectangular batch)
  int64_t start;      // first step of the current segment
  int64_t next;       // first step of the next segment (INT64_MAX if none)

  __device__ __forceinline__ void init(const int32_t* cu_, int64_t n_seqs_, int64_t row, int64_t t0) {
    cu = cu_;
    n_seqs = n_seqs_;
    if (!cu) {
      seg = row;
      start = 0;
      next = INT64_MAX;
      return;
    }
    // largest j in [0, n_seqs) with cu[j] <= t0
    int64_t lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (static_cast<int64_t>(cu[mid]) <= t0) lo = mid; else hi = mid - 1;
    }
    seg = lo;
    start = cu[seg];
    next = (seg + 1 < n_seqs) ? static_cast<int64_t>(cu[seg + 1]) : INT64_MAX;
  }
  // The same as init, searched by a whole wave at once (every lane active,
  // t0 wave-uniform): each load probes 64 offsets, a ballot narrows the
  // range, so a pack of up to 64 segments costs two dependent loads instead
  // of a binary search's six or more.  Stays in bounds for any cu contents.
  __device__ __forceinline__ void init_wave(const int32_t* cu_, int64_t n_seqs_, int64_t row, int64_t t0) {
    cu = cu_;
    n_seqs = n_seqs_;
    if (!cu) {
      seg = row;
      start = 0;
      next = INT64_MAX;
      return;
    }
    const int lane = threadIdx.x & 63;
    int64_t lo = 0, hi = n_seqs;   // the answer lies in [lo, hi); cu[lo] <= t0 once lo has been probed
    while (hi - lo > 63) {
      const int64_t step = (hi - lo + 63) / 64;
      const int64_t j = lo + lane * step;
      const bool ok = j < hi && static_cast<int64_t>(cu[j < hi ? j : lo]) <= t0;
      const unsigned long long m = __ballot(ok);
      const int k = m ? 63 - __builtin_clzll(m) : 0;
      lo += k * step;
      hi = imin(hi, lo + step);
    }
    // the last range has at most 63 candidates: lane i probes lo + i, and the
    // next lane holds the following offset (lo + i + 1 <= n_seqs)
    const int64_t j = lo + lane;
    const int64_t v = j <= n_seqs ? static_cast<int64_t>(cu[j <= n_seqs ? j : n_seqs]) : 0;
    const unsigned long long m = __ballot(j < hi && v <= t0);
    const int k = m ? 63 - __builtin_clzll(m) : 0;
    seg = lo + k;
    start = __shfl(v, k, 64);
    const int64_t nx = __shfl(v, k + 1, 64);
    next = (seg + 1 < n_seqs) ? nx : INT64_MAX;
  }
  // advance to step t (t non-decreasing); returns true if t is a head
  __device__ __forceinline__ bool at(int64_t t) {
    if (cu) {
      while (next <= t) {
        ++seg;
        start = next;
        next = (seg + 1 < n_seqs) ? static_cast<int64_t>(cu[seg + 1]) : INT64_MAX;
      }
    }
    return t == start || t == 0;  // the first step of a row is always a head
  }
  // is t the last step of its segment (T = steps in the row)?
  __device__ __forceinline__ bool last(int64_t t, int64_t T) const { return t + 1 == next || t + 1 == T; }
};

}  // namespace prn
