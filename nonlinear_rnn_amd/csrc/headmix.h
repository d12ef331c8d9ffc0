// Head-mix GRU (dense d_head x d_head recurrent blocks, d_head = 16): the
// parallel Newton forward and the sequential unroll, fp32 storage.
//
// Cell (per head, A_g the head's block of gate g, h the head's 16 channels):
//   z = sig(x_z + A_z h)  r = sig(x_r + A_r h)  c = tanh(x_c + A_c (r h))
//   h' = (1 - z) h + z c
// Its Jacobian is never formed.  With the per-channel vectors
//   alpha = 1 - z, beta = (c - h) z (1 - z), gamma = z (1 - c^2),
//   rho = r, delta = h r (1 - r)
// J X = diag(alpha) X + diag(beta) (A_z X) + diag(gamma) A_c (diag(rho) X +
// diag(delta) (A_r X)) for a vector or a 16 x 16 matrix X: three products
// with the constant blocks.
//
// Lane layout (one wave per (row, head, chunk)): lane = 4 i + q holds
// channel i of the head, and columns 4q..4q+3 of a 16 x 16 map.  Vectors are
// held by all four lanes of a channel.  A matrix-vector product takes its
// operand's four columns by shuffles and sums the row over the four lanes;
// a matrix-matrix product reads the right operand from a 16 x 16 LDS tile.
//
// Schedule per Newton iteration k (three phases over chunks of kHmChunk
// steps): k_hm_reduce linearises at H^(k-1) and composes each chunk's maps
// (and reduces r_(k-1) on the way); k_hm_scan carries across the chunks of
// one (row, head) serially; k_hm_fix replays each chunk from its carry and
// writes H^(k).  A last k_hm_reduce without composition gives r_K.
#pragma once

#include "newton_kernels.h"

namespace prn {

constexpr int kHmD = 16;       // d_head
constexpr int kHmChunk = 64;   // steps per chunk
constexpr int kHmNC = kHmD * kHmD + kHmD;  // floats of one chunk aggregate (M row-major, then v)

struct HmBlocks {
  float row[3][kHmD];  // A_g[i][0..15]: the full row (matrix-matrix products)
  float quad[3][4];    // A_g[i][4q..4q+3]: this lane's columns (matrix-vector products)
};

__device__ __forceinline__ void hm_load_blocks(const float* A, int64_t n_heads, int64_t head, int i, int q,
                                               HmBlocks& blk) {
#pragma unroll
  for (int g = 0; g < 3; ++g) {
    const float* base = A + ((g * n_heads + head) * kHmD + i) * kHmD;
#pragma unroll
    for (int m = 0; m < kHmD; ++m) blk.row[g][m] = base[m];
#pragma unroll
    for (int u = 0; u < 4; ++u) blk.quad[g][u] = base[4 * q + u];
  }
}

// sum over the four lanes of a channel
__device__ __forceinline__ float hm_rowsum(float x) {
  x += __shfl_xor(x, 1, kWave);
  x += __shfl_xor(x, 2, kWave);
  return x;
}

// (A v)_i for a vector held per channel (all four lanes of channel j hold v_j)
__device__ __forceinline__ float hm_matvec(const float* aq, float v, int q) {
  float s = 0.0f;
#pragma unroll
  for (int u = 0; u < 4; ++u) s = fmaf(aq[u], __shfl(v, 4 * (4 * q + u), kWave), s);
  return hm_rowsum(s);
}

// (A X)[i][4q..4q+3] with X in LDS (row-major 16 x 16)
__device__ __forceinline__ void hm_matmat(const float* arow, const float* X, int q, float* out) {
#pragma unroll
  for (int c = 0; c < 4; ++c) out[c] = 0.0f;
#pragma unroll
  for (int m = 0; m < kHmD; ++m) {
    const float4 x = *reinterpret_cast<const float4*>(X + m * kHmD + 4 * q);
    out[0] = fmaf(arow[m], x.x, out[0]);
    out[1] = fmaf(arow[m], x.y, out[1]);
    out[2] = fmaf(arow[m], x.z, out[2]);
    out[3] = fmaf(arow[m], x.w, out[3]);
  }
}

// one cell evaluation at h (the channel's previous state) with inputs x[3]:
// f and the Jacobian's per-channel coefficients
struct HmLin {
  float fv, alpha, beta, gamma, rho, delta;
};
__device__ __forceinline__ HmLin hm_linearise(const HmBlocks& blk, const float* x, float h, int q) {
  const float uz = x[0] + hm_matvec(blk.quad[0], h, q);
  const float ur = x[1] + hm_matvec(blk.quad[1], h, q);
  const float z = sig_s(kSigScale * uz);
  const float r = sig_s(kSigScale * ur);
  const float uc = x[2] + hm_matvec(blk.quad[2], r * h, q);
  const float c = tanh_s(kTanhScale * uc);
  HmLin l;
  l.fv = fmaf(z, c - h, h);
  l.alpha = 1.0f - z;
  l.beta = (c - h) * z * (1.0f - z);
  l.gamma = z * fmaf(-c, c, 1.0f);
  l.rho = r;
  l.delta = h * r * (1.0f - r);
  return l;
}

// J d for a vector d held per channel
__device__ __forceinline__ float hm_jvec(const HmBlocks& blk, const HmLin& l, float d, int q) {
  const float y3 = hm_matvec(blk.quad[0], d, q);
  const float y1 = hm_matvec(blk.quad[1], d, q);
  const float w = fmaf(l.delta, y1, l.rho * d);
  const float y2 = hm_matvec(blk.quad[2], w, q);
  return fmaf(l.gamma, y2, fmaf(l.beta, y3, l.alpha * d));
}

// inputs of step t for channel ch: x_z, x_r, x_c
__device__ __forceinline__ void hm_load_x(const float* xproj, int64_t b, int64_t t, int64_t T, int64_t d_h,
                                          int64_t ch, float* x) {
  const float* p = xproj + ((b * T + t) * 3) * d_h + ch;
#pragma unroll
  for (int g = 0; g < 3; ++g) x[g] = p[g * d_h];
}

// previous state of step t under the iterate Hprev (zero iterate if null),
// h0 (zero if null) at t = 0
__device__ __forceinline__ float hm_prev(const float* Hprev, const float* h0, int64_t b, int64_t t, int64_t T,
                                         int64_t d_h, int64_t ch) {
  if (t == 0) return h0 ? h0[b * d_h + ch] : 0.0f;
  return Hprev ? Hprev[(b * T + t - 1) * d_h + ch] : 0.0f;
}

// Phase 1 (COMPOSE) or the residual pass (!COMPOSE): linearise every step
// of the chunk at Hprev; r = max |Hprev_t - f(prev_t)| (Hprev = 0 when null);
// with COMPOSE also the chunk aggregate (M, v) of the maps
// h -> J_t h + f_t - J_t prev_t, J_0 := 0.
template <bool COMPOSE>
__global__ void __launch_bounds__(kWave)
k_hm_reduce(const float* __restrict__ xproj, const float* __restrict__ A, const float* __restrict__ h0,
            const float* __restrict__ Hprev, int64_t T, int64_t d_h, int64_t n_ch, float* __restrict__ agg,
            float* __restrict__ rpart) {
  const int lane = threadIdx.x, i = lane >> 2, q = lane & 3;
  const int64_t chunk = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int64_t n_heads = gridDim.y;
  const int64_t ch = head * kHmD + i;
  __shared__ __attribute__((aligned(16))) float Mt[kHmD * kHmD];
  __shared__ __attribute__((aligned(16))) float Wt[kHmD * kHmD];
  HmBlocks blk;
  hm_load_blocks(A, n_heads, head, i, q, blk);
  const int64_t t0 = chunk * kHmChunk, t1 = imin(T, t0 + kHmChunk);
  float M[4], v = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) M[c] = (4 * q + c == i) ? 1.0f : 0.0f;
  unsigned rmax = 0;
  for (int64_t t = t0; t < t1; ++t) {
    float x[3];
    hm_load_x(xproj, b, t, T, d_h, ch, x);
    const float prev = hm_prev(Hprev, h0, b, t, T, d_h, ch);
    const float cur = Hprev ? Hprev[(b * T + t) * d_h + ch] : 0.0f;
    const HmLin l = hm_linearise(blk, x, prev, q);
    rmax = rmax_bits(rmax, cur - l.fv);
    if constexpr (COMPOSE) {
      if (t == 0) {  // the sequence's first step: J = 0
#pragma unroll
        for (int c = 0; c < 4; ++c) M[c] = 0.0f;
        v = l.fv;
      } else {
        // M <- J M
#pragma unroll
        for (int c = 0; c < 4; ++c) Mt[i * kHmD + 4 * q + c] = M[c];
        __syncthreads();
        float y3[4], y1[4], y2[4];
        hm_matmat(blk.row[0], Mt, q, y3);
        hm_matmat(blk.row[1], Mt, q, y1);
#pragma unroll
        for (int c = 0; c < 4; ++c) Wt[i * kHmD + 4 * q + c] = fmaf(l.delta, y1[c], l.rho * M[c]);
        __syncthreads();
        hm_matmat(blk.row[2], Wt, q, y2);
#pragma unroll
        for (int c = 0; c < 4; ++c) M[c] = fmaf(l.gamma, y2[c], fmaf(l.beta, y3[c], l.alpha * M[c]));
        // v <- J v + f - J prev = f + J (v - prev)
        v = l.fv + hm_jvec(blk, l, v - prev, q);
        __syncthreads();  // Mt and Wt are rewritten at the next step
      }
    }
  }
  if constexpr (COMPOSE) {
    float* out = agg + ((b * n_heads + head) * n_ch + chunk) * kHmNC;
    *reinterpret_cast<float4*>(out + i * kHmD + 4 * q) = make_float4(M[0], M[1], M[2], M[3]);
    if (q == 0) out[kHmD * kHmD + i] = v;
  }
  if (rpart) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) rmax = max(rmax, static_cast<unsigned>(__shfl_xor(static_cast<int>(rmax), o, kWave)));
    if (lane == 0) rpart[(b * n_heads + head) * n_ch + chunk] = rmax_finish(rmax);
  }
}

// Phase 2: carries across the chunks of one (row, head): carry_0 = 0,
// carry_(c+1) = M_c carry_c + v_c (carry_c is the state before chunk c).
// The aggregates are read eight chunks ahead of the serial chain.
__global__ void __launch_bounds__(kWave)
k_hm_scan(const float* __restrict__ agg, int64_t n_ch, float* __restrict__ carry) {
  const int lane = threadIdx.x, i = lane >> 2, q = lane & 3;
  const int64_t head = blockIdx.x, b = blockIdx.y, n_heads = gridDim.x;
  const float* a = agg + (b * n_heads + head) * n_ch * kHmNC;
  float* cout = carry + (b * n_heads + head) * n_ch * kHmD;
  constexpr int PB = 8;
  float s = 0.0f;
  for (int64_t c0 = 0; c0 < n_ch; c0 += PB) {
    float4 m[PB];
    float vv[PB];
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int64_t c = imin(c0 + u, n_ch - 1);
      m[u] = *reinterpret_cast<const float4*>(a + c * kHmNC + i * kHmD + 4 * q);
      vv[u] = a[c * kHmNC + kHmD * kHmD + i];
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      if (c0 + u < n_ch) {
        if (q == 0) cout[(c0 + u) * kHmD + i] = s;
        float p = m[u].x * __shfl(s, 4 * (4 * q + 0), kWave);
        p = fmaf(m[u].y, __shfl(s, 4 * (4 * q + 1), kWave), p);
        p = fmaf(m[u].z, __shfl(s, 4 * (4 * q + 2), kWave), p);
        p = fmaf(m[u].w, __shfl(s, 4 * (4 * q + 3), kWave), p);
        s = hm_rowsum(p) + vv[u];
      }
    }
  }
}

// Phase 3: replay each chunk from its carry with the maps of the old
// linearisation point Hprev: H_t = f_t + J_t (H_(t-1) - prev_t) (H_0 = f_0),
// written to Hout; the final state of each row to slast at the last step.
__global__ void __launch_bounds__(kWave)
k_hm_fix(const float* __restrict__ xproj, const float* __restrict__ A, const float* __restrict__ h0,
         const float* __restrict__ Hprev, const float* __restrict__ carry, int64_t T, int64_t d_h, int64_t n_ch,
         float* __restrict__ Hout, float* __restrict__ slast) {
  const int lane = threadIdx.x, i = lane >> 2, q = lane & 3;
  const int64_t chunk = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int64_t n_heads = gridDim.y;
  const int64_t ch = head * kHmD + i;
  HmBlocks blk;
  hm_load_blocks(A, n_heads, head, i, q, blk);
  const int64_t t0 = chunk * kHmChunk, t1 = imin(T, t0 + kHmChunk);
  float s = carry[((b * n_heads + head) * n_ch + chunk) * kHmD + i];
  for (int64_t t = t0; t < t1; ++t) {
    float x[3];
    hm_load_x(xproj, b, t, T, d_h, ch, x);
    const float prev = hm_prev(Hprev, h0, b, t, T, d_h, ch);
    const HmLin l = hm_linearise(blk, x, prev, q);
    s = (t == 0) ? l.fv : l.fv + hm_jvec(blk, l, s - prev, q);
    if (q == 0) Hout[(b * T + t) * d_h + ch] = s;
  }
  if (slast && t1 == T && q == 0) slast[b * d_h + ch] = s;
}

// The sequential unroll: one wave per (row, head), h_t = f(h_(t-1), x_t).
__global__ void __launch_bounds__(kWave)
k_hm_sequential(const float* __restrict__ xproj, const float* __restrict__ A, const float* __restrict__ h0,
                int64_t T, int64_t d_h, float* __restrict__ Hout, float* __restrict__ slast) {
  const int lane = threadIdx.x, i = lane >> 2, q = lane & 3;
  const int64_t head = blockIdx.x, b = blockIdx.y, n_heads = gridDim.x;
  const int64_t ch = head * kHmD + i;
  HmBlocks blk;
  hm_load_blocks(A, n_heads, head, i, q, blk);
  float h = h0 ? h0[b * d_h + ch] : 0.0f;
  for (int64_t t = 0; t < T; ++t) {
    float x[3];
    hm_load_x(xproj, b, t, T, d_h, ch, x);
    h = hm_linearise(blk, x, h, q).fv;
    if (q == 0) Hout[(b * T + t) * d_h + ch] = h;
  }
  if (slast && q == 0) slast[b * d_h + ch] = h;
}

}  // namespace prn
