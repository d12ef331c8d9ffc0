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
// Lane layouts (one wave per (row, head, chunk)).  Vectors: lane = 4 i + q
// holds channel i of the head (all four lanes of a channel hold it); a
// matrix-vector product takes its operand's four columns q by shuffles and
// sums the row over the four lanes.  Maps: the chunk's running 16 x 16 map
// lives in the output layout of v_mfma_f32_16x16x4_f32 (lane L holds rows
// 4 (L / 16) .. + 3 of column L % 16).  A block product X M is four such
// instructions; in instruction p lane L supplies X[L % 16][4 (L / 16) + p]
// and M[4 (L / 16) + p][L % 16], which is M's own register p, so the
// running map never moves between lanes.
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
constexpr int kHmChunk = 32;   // steps per chunk
constexpr int kHmSeqBlock = 64;  // steps of inputs the unroll stages at a time

typedef __attribute__((ext_vector_type(4))) float hm_f4;
constexpr int kHmNC = kHmD * kHmD + kHmD;  // floats of one chunk aggregate (M row-major, then v)

struct HmBlocks {
  float quad[3][4];  // A_g[i][4q..4q+3]: this lane's columns (matrix-vector products)
  float mf[3][4];    // A_g[L % 16][4 (L / 16) + p]: the operand of block-product instruction p
};

__device__ __forceinline__ void hm_load_blocks(const float* A, int64_t n_heads, int64_t head, int lane,
                                               HmBlocks& blk) {
  const int i = lane >> 2, q = lane & 3, mr = lane & 15, mk = 4 * (lane >> 4);
#pragma unroll
  for (int g = 0; g < 3; ++g) {
    const float* base = A + (g * n_heads + head) * kHmD * kHmD;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      blk.quad[g][u] = base[i * kHmD + 4 * q + u];
      blk.mf[g][u] = base[mr * kHmD + mk + u];
    }
  }
}

// X M for the constant block X (operands xm) and M in the product layout
__device__ __forceinline__ hm_f4 hm_blockmul(const float* xm, const hm_f4& m) {
  hm_f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int p = 0; p < 4; ++p) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xm[p], m[p], acc, 0, 0, 0);
  return acc;
}

// a per-channel vector (vector layout) read at rows 4 (L / 16) + r
__device__ __forceinline__ hm_f4 hm_rows(float c, int lane) {
  const int r0 = 4 * (lane >> 4);
  return {__shfl(c, 4 * (r0 + 0), kWave), __shfl(c, 4 * (r0 + 1), kWave), __shfl(c, 4 * (r0 + 2), kWave),
          __shfl(c, 4 * (r0 + 3), kWave)};
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

// The chunk's inputs and previous-iterate states staged in LDS with all
// loads in flight at once (a load per step would put a memory round trip
// on every step of the serial chain): xs[j][g][i] = x_g of step t0 + j,
// hs[j][i] = the state before step t0 + j under Hprev (hs[0]: h0 at t = 0),
// hs[n][i] = Hprev at the chunk's last step.
struct HmStage {
  float xs[kHmChunk][3][kHmD];
  float hs[kHmChunk + 1][kHmD];
};
__device__ __forceinline__ void hm_stage(HmStage& sm, const float* xproj, const float* Hprev, const float* h0,
                                         int64_t b, int64_t head, int64_t t0, int n, int64_t T, int64_t d_h,
                                         int lane) {
  const float* xb = xproj + ((b * T + t0) * 3) * d_h + head * kHmD;
#pragma unroll 8
  for (int e = lane; e < n * 3 * kHmD; e += kWave) {
    const int j = e / (3 * kHmD), r = e - j * 3 * kHmD, g = r / kHmD, i = r - g * kHmD;
    sm.xs[j][g][i] = xb[(static_cast<int64_t>(j) * 3 + g) * d_h + i];
  }
#pragma unroll 4
  for (int e = lane; e < (n + 1) * kHmD; e += kWave) {
    const int j = e / kHmD, i = e - j * kHmD;
    const int64_t t = t0 + j - 1;  // the step whose state this is
    float v = 0.0f;
    if (t < 0) v = h0 ? h0[b * d_h + head * kHmD + i] : 0.0f;
    else if (Hprev) v = Hprev[(b * T + t) * d_h + head * kHmD + i];
    sm.hs[j][i] = v;
  }
  __syncthreads();
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
  __shared__ HmStage sm;
  HmBlocks blk;
  hm_load_blocks(A, n_heads, head, lane, blk);
  const int64_t t0 = chunk * kHmChunk;
  const int n = static_cast<int>(imin(T - t0, kHmChunk));
  hm_stage(sm, xproj, Hprev, h0, b, head, t0, n, T, d_h, lane);
  const int mr = lane & 15, mk = 4 * (lane >> 4);  // product layout: rows mk..mk+3 of column mr
  hm_f4 M;
  float v = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) M[r] = (mk + r == mr) ? 1.0f : 0.0f;
  unsigned rmax = 0;
  for (int j = 0; j < n; ++j) {
    const int64_t t = t0 + j;
    const float x[3] = {sm.xs[j][0][i], sm.xs[j][1][i], sm.xs[j][2][i]};
    const float prev = sm.hs[j][i];
    const float cur = sm.hs[j + 1][i];
    const HmLin l = hm_linearise(blk, x, prev, q);
    rmax = rmax_bits(rmax, cur - l.fv);
    if constexpr (COMPOSE) {
      if (t == 0) {  // the sequence's first step: J = 0
#pragma unroll
        for (int r = 0; r < 4; ++r) M[r] = 0.0f;
        v = l.fv;
      } else {
        // M <- J M = alpha M + beta (A_z M) + gamma A_c (rho M + delta (A_r M))
        const hm_f4 y3 = hm_blockmul(blk.mf[0], M);
        const hm_f4 y1 = hm_blockmul(blk.mf[1], M);
        const hm_f4 rho = hm_rows(l.rho, lane), del = hm_rows(l.delta, lane);
        hm_f4 W;
#pragma unroll
        for (int r = 0; r < 4; ++r) W[r] = fmaf(del[r], y1[r], rho[r] * M[r]);
        const hm_f4 y2 = hm_blockmul(blk.mf[2], W);
        const hm_f4 al = hm_rows(l.alpha, lane), be = hm_rows(l.beta, lane), ga = hm_rows(l.gamma, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) M[r] = fmaf(ga[r], y2[r], fmaf(be[r], y3[r], al[r] * M[r]));
        // v <- J v + f - J prev = f + J (v - prev)
        v = l.fv + hm_jvec(blk, l, v - prev, q);
      }
    }
  }
  if constexpr (COMPOSE) {
    float* out = agg + ((b * n_heads + head) * n_ch + chunk) * kHmNC;
#pragma unroll
    for (int r = 0; r < 4; ++r) out[(mk + r) * kHmD + mr] = M[r];
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
  __shared__ HmStage sm;
  HmBlocks blk;
  hm_load_blocks(A, n_heads, head, lane, blk);
  const int64_t t0 = chunk * kHmChunk;
  const int n = static_cast<int>(imin(T - t0, kHmChunk));
  hm_stage(sm, xproj, Hprev, h0, b, head, t0, n, T, d_h, lane);
  float s = carry[((b * n_heads + head) * n_ch + chunk) * kHmD + i];
  for (int j = 0; j < n; ++j) {
    const int64_t t = t0 + j;
    const float x[3] = {sm.xs[j][0][i], sm.xs[j][1][i], sm.xs[j][2][i]};
    const float prev = sm.hs[j][i];
    const HmLin l = hm_linearise(blk, x, prev, q);
    s = (t == 0) ? l.fv : l.fv + hm_jvec(blk, l, s - prev, q);
    if (q == 0) Hout[(b * T + t) * d_h + ch] = s;
  }
  if (slast && t0 + n == T && q == 0) slast[b * d_h + ch] = s;
}

// The sequential unroll: one wave per (row, head), h_t = f(h_(t-1), x_t).
__global__ void __launch_bounds__(kWave)
k_hm_sequential(const float* __restrict__ xproj, const float* __restrict__ A, const float* __restrict__ h0,
                int64_t T, int64_t d_h, float* __restrict__ Hout, float* __restrict__ slast) {
  const int lane = threadIdx.x, i = lane >> 2, q = lane & 3;
  const int64_t head = blockIdx.x, b = blockIdx.y, n_heads = gridDim.x;
  const int64_t ch = head * kHmD + i;
  __shared__ float xs[kHmSeqBlock][3][kHmD];
  HmBlocks blk;
  hm_load_blocks(A, n_heads, head, lane, blk);
  float h = h0 ? h0[b * d_h + ch] : 0.0f;
  for (int64_t t0 = 0; t0 < T; t0 += kHmSeqBlock) {
    // the next block's inputs, all loads in flight at once
    const int n = static_cast<int>(imin(T - t0, kHmSeqBlock));
    const float* xb = xproj + ((b * T + t0) * 3) * d_h + head * kHmD;
    __syncthreads();  // the previous block's reads are done
#pragma unroll 8
    for (int e = lane; e < n * 3 * kHmD; e += kWave) {
      const int j = e / (3 * kHmD), r = e - j * 3 * kHmD, g = r / kHmD, c = r - g * kHmD;
      xs[j][g][c] = xb[(static_cast<int64_t>(j) * 3 + g) * d_h + c];
    }
    __syncthreads();
    for (int j = 0; j < n; ++j) {
      const float x[3] = {xs[j][0][i], xs[j][1][i], xs[j][2][i]};
      h = hm_linearise(blk, x, h, q).fv;
      if (q == 0) Hout[(b * T + t0 + j) * d_h + ch] = h;
    }
  }
  if (slast && q == 0) slast[b * d_h + ch] = h;
}

}  // namespace prn
