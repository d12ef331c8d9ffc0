// Head-mix GRU (dense d_head x d_head recurrent blocks, d_head = 16): the
// parallel Newton forward and the sequential unroll, fp32 or bf16 storage
// (xproj, h0, the iterates and H; the blocks A and all arithmetic fp32; a
// stored iterate is rounded once, the chain it came from is not).
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
// steps): k_hm_pass<kHmReduce> linearises at H^(k-1) and composes each
// chunk's maps (and reduces r_(k-1) on the way); k_hm_scan carries across
// the chunks of one (row, head) serially; k_hm_pass<kHmFix> replays each
// chunk from its carry and writes H^(k).  A last k_hm_pass<kHmResidual>
// gives r_K.
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

// sum over the four lanes of a channel (one quad: DPP quad permutations
// [1,0,3,2] and [2,3,0,1], no LDS)
__device__ __forceinline__ float hm_rowsum(float x) {
  x += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), 0xb1, 0xf, 0xf, false));
  x += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), 0x4e, 0xf, 0xf, false));
  return x;
}

// (A v)_i for a vector held per channel (all four lanes of channel j hold v_j)
__device__ __forceinline__ float hm_matvec(const float* aq, float v, int q) {
  float s = 0.0f;
#pragma unroll
  for (int u = 0; u < 4; ++u) s = fmaf(aq[u], __shfl(v, 4 * (4 * q + u), kWave), s);
  return hm_rowsum(s);
}

// one cell step h' = f(h, x) in the vector layout (the unroll)
__device__ __forceinline__ float hm_step(const HmBlocks& blk, const float* x, float h, int q) {
  const float z = sig_s(kSigScale * (x[0] + hm_matvec(blk.quad[0], h, q)));
  const float r = sig_s(kSigScale * (x[1] + hm_matvec(blk.quad[1], h, q)));
  const float c = tanh_s(kTanhScale * (x[2] + hm_matvec(blk.quad[2], r * h, q)));
  return fmaf(z, c - h, h);
}

// ---- the Newton passes over one chunk of one (row, head) ----
//
// Phase A, per block of 16 steps: the linearisation of every step is
// independent (the previous states come from the previous iterate), so the
// gate pre-activations of the block are block products too: with P the
// 16 x 16 matrix of previous states (channels x steps) in the product
// layout, U_z = A_z P, U_r = A_r P and U_c = A_c (R * P) are four
// matrix-core instructions each, and the per-(channel, step) coefficients
// f, alpha, beta, gamma, rho, delta (and P itself) go to LDS as
// [coefficient][step][channel].  The residual max |H_t - f_t| is reduced
// here.  Phase B walks the block's steps serially: the chunk map
// M <- J M on the matrix cores (rows of the coefficients read back as
// 16-byte LDS words), and the vector chain d <- f + J (d - prev) in the
// vector layout, whose matrix-vector products read their operand from a
// 16-float LDS vector (one 16-byte read per lane) instead of shuffles.
enum HmMode { kHmReduce = 0, kHmFix = 1, kHmResidual = 2 };
constexpr int kHmBlk = 16;  // steps per block of phase A
enum { kCf = 0, kCalpha, kCbeta, kCgamma, kCrho, kCdelta, kCprev, kNCoef };

struct HmShared {
  __attribute__((aligned(16))) float cf[kNCoef][kHmBlk][kHmD];
  __attribute__((aligned(16))) float dv[kHmD];
  __attribute__((aligned(16))) float wv[kHmD];
};

__device__ __forceinline__ hm_f4 hm_ld4(const float* p) { return *reinterpret_cast<const hm_f4*>(p); }
// four consecutive stored values (16 bytes fp32, 8 bytes bf16) as floats
__device__ __forceinline__ hm_f4 hm_ld4s(const float* p) { return hm_ld4(p); }
__device__ __forceinline__ hm_f4 hm_ld4s(const uint16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return hm_f4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
               __uint_as_float(w.y & 0xffff0000u)};
}

// phase A for steps jb .. jb + 15 of the chunk (lane L: step jb + L % 16,
// channels 4 (L / 16) .. + 3 of the head); steps at or past n are computed
// on clamped inputs and ignored
template <bool RES, class E>
__device__ __forceinline__ void hm_phase_a(const HmBlocks& blk, const E* xproj, const E* Hprev, const E* h0,
                                           int64_t b, int64_t head, int64_t t0, int jb, int n, int64_t T,
                                           int64_t d_h, int lane, HmShared& sh, unsigned& rmax) {
  const int col = lane & 15, mk = 4 * (lane >> 4);
  const int j = jb + col;
  const bool valid = j < n;
  const int64_t t = t0 + (valid ? j : n - 1);
  const int64_t c0 = head * kHmD + mk;
  const E* xp = xproj + ((b * T + t) * 3) * d_h + c0;
  const hm_f4 xz = hm_ld4s(xp), xr = hm_ld4s(xp + d_h), xc = hm_ld4s(xp + 2 * d_h);
  hm_f4 P = {0.0f, 0.0f, 0.0f, 0.0f}, cur = {0.0f, 0.0f, 0.0f, 0.0f};
  if (Hprev) {
    cur = hm_ld4s(Hprev + (b * T + t) * d_h + c0);
    if (t > 0) P = hm_ld4s(Hprev + (b * T + t - 1) * d_h + c0);
  }
  if (t == 0 && h0) P = hm_ld4s(h0 + b * d_h + c0);
  else if (t == 0) P = hm_f4{0.0f, 0.0f, 0.0f, 0.0f};
  // linearising at H = 0 (the first iteration; no h0 in this block): the
  // recurrent terms A_g P vanish, and so do their block products
  const bool pzero = !Hprev && (!h0 || t0 + jb > 0);
  const hm_f4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  const hm_f4 uz = pzero ? zero4 : hm_blockmul(blk.mf[0], P), ur = pzero ? zero4 : hm_blockmul(blk.mf[1], P);
  hm_f4 z, rr, rh;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    z[r] = sig_s(kSigScale * (xz[r] + uz[r]));
    rr[r] = sig_s(kSigScale * (xr[r] + ur[r]));
    rh[r] = rr[r] * P[r];
  }
  const hm_f4 uc = pzero ? zero4 : hm_blockmul(blk.mf[2], rh);
  hm_f4 fv, al, be, ga, de;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float c = tanh_s(kTanhScale * (xc[r] + uc[r]));
    fv[r] = fmaf(z[r], c - P[r], P[r]);
    al[r] = 1.0f - z[r];
    be[r] = (c - P[r]) * z[r] * (1.0f - z[r]);
    ga[r] = z[r] * fmaf(-c, c, 1.0f);
    de[r] = P[r] * rr[r] * (1.0f - rr[r]);
    if (RES && valid) rmax = rmax_bits(rmax, cur[r] - fv[r]);
  }
  *reinterpret_cast<hm_f4*>(&sh.cf[kCf][col][mk]) = fv;
  *reinterpret_cast<hm_f4*>(&sh.cf[kCalpha][col][mk]) = al;
  *reinterpret_cast<hm_f4*>(&sh.cf[kCbeta][col][mk]) = be;
  *reinterpret_cast<hm_f4*>(&sh.cf[kCgamma][col][mk]) = ga;
  *reinterpret_cast<hm_f4*>(&sh.cf[kCrho][col][mk]) = rr;
  *reinterpret_cast<hm_f4*>(&sh.cf[kCdelta][col][mk]) = de;
  *reinterpret_cast<hm_f4*>(&sh.cf[kCprev][col][mk]) = P;
}

// sum_u a[u] * x[4q + u] over the channel's four lanes, x a 16-float LDS vector
__device__ __forceinline__ float hm_matvec_lds(const float* aq, const float* x, int q) {
  const hm_f4 v = hm_ld4(x + 4 * q);
  return hm_rowsum(fmaf(aq[3], v[3], fmaf(aq[2], v[2], fmaf(aq[1], v[1], aq[0] * v[0]))));
}

// one step of the vector chain, vector layout (channel i = L / 4):
// returns f + J (d - prev) for step s of the block.  zprev: the previous
// iterate is 0 (the first iteration), so delta = h r (1 - r) is 0 and the
// A_r product drops out.
__device__ __forceinline__ float hm_chain_step(const HmBlocks& blk, HmShared& sh, int s, float d, int i, int q,
                                               bool zprev) {
  const float dl = d - sh.cf[kCprev][s][i];
  if (q == 0) sh.dv[i] = dl;
  __syncthreads();
  const float y3 = hm_matvec_lds(blk.quad[0], sh.dv, q);
  const float rdl = sh.cf[kCrho][s][i] * dl;
  const float w = zprev ? rdl : fmaf(sh.cf[kCdelta][s][i], hm_matvec_lds(blk.quad[1], sh.dv, q), rdl);
  if (q == 0) sh.wv[i] = w;
  __syncthreads();
  const float y2 = hm_matvec_lds(blk.quad[2], sh.wv, q);
  return sh.cf[kCf][s][i] +
         fmaf(sh.cf[kCgamma][s][i], y2, fmaf(sh.cf[kCbeta][s][i], y3, sh.cf[kCalpha][s][i] * dl));
}

// kHmReduce: compose the chunk's maps (M, v) into agg, and reduce r_(k-1)
//   (max |Hprev_t - f_t|, Hprev = 0 when null) into rpart;
// kHmFix: replay the chunk from its carry, H_t = f_t + J_t (H_(t-1) -
//   prev_t), into Hout (and the row's final state into slast);
// kHmResidual: only the residual of Hprev.
// J_0 := 0 (the map of a sequence's first step is constant, f_0).
template <int MODE, int DT>
__global__ void __launch_bounds__(kWave)
k_hm_pass(const typename Storage<DT>::T* __restrict__ xproj, const float* __restrict__ A,
          const typename Storage<DT>::T* __restrict__ h0, const typename Storage<DT>::T* __restrict__ Hprev,
          const float* __restrict__ carry, int64_t T, int64_t d_h, int64_t n_ch, float* __restrict__ agg,
          float* __restrict__ rpart, typename Storage<DT>::T* __restrict__ Hout,
          typename Storage<DT>::T* __restrict__ slast) {
  using ST = Storage<DT>;
  const int lane = threadIdx.x, i = lane >> 2, q = lane & 3;
  const int mr = lane & 15, mk = 4 * (lane >> 4);  // product layout: rows mk..mk+3 of column mr
  const int64_t chunk = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int64_t n_heads = gridDim.y;
  __shared__ HmShared sh;
  HmBlocks blk;
  hm_load_blocks(A, n_heads, head, lane, blk);
  const int64_t t0 = chunk * kHmChunk;
  const int n = static_cast<int>(imin(T - t0, kHmChunk));
  hm_f4 M;
#pragma unroll
  for (int r = 0; r < 4; ++r) M[r] = (mk + r == mr) ? 1.0f : 0.0f;
  float d = 0.0f;  // kHmReduce: the map's offset v; kHmFix: the state
  // linearisation at H = 0: past a sequence's first step (whose map is
  // constant) every previous state is 0
  const bool zprev = Hprev == nullptr;
  if (MODE == kHmFix) d = carry[((b * n_heads + head) * n_ch + chunk) * kHmD + i];
  unsigned rmax = 0;
  for (int jb = 0; jb < n; jb += kHmBlk) {
    hm_phase_a<MODE != kHmFix>(blk, xproj, Hprev, h0, b, head, t0, jb, n, T, d_h, lane, sh, rmax);
    __syncthreads();
    if constexpr (MODE != kHmResidual) {
      const int nb = static_cast<int>(imin(n - jb, kHmBlk));
      for (int s = 0; s < nb; ++s) {
        if (t0 + jb + s == 0) {  // the sequence's first step: J = 0
          if constexpr (MODE == kHmReduce) {
#pragma unroll
            for (int r = 0; r < 4; ++r) M[r] = 0.0f;
          }
          d = sh.cf[kCf][s][i];
        } else {
          if constexpr (MODE == kHmReduce) {
            // M <- J M = alpha M + beta (A_z M) + gamma A_c (rho M + delta (A_r M));
            // delta = 0 when linearising at H = 0
            const hm_f4 y3 = hm_blockmul(blk.mf[0], M);
            const hm_f4 rho = hm_ld4(&sh.cf[kCrho][s][mk]);
            hm_f4 W;
            if (zprev) {
#pragma unroll
              for (int r = 0; r < 4; ++r) W[r] = rho[r] * M[r];
            } else {
              const hm_f4 y1 = hm_blockmul(blk.mf[1], M);
              const hm_f4 del = hm_ld4(&sh.cf[kCdelta][s][mk]);
#pragma unroll
              for (int r = 0; r < 4; ++r) W[r] = fmaf(del[r], y1[r], rho[r] * M[r]);
            }
            const hm_f4 y2 = hm_blockmul(blk.mf[2], W);
            const hm_f4 al = hm_ld4(&sh.cf[kCalpha][s][mk]), be = hm_ld4(&sh.cf[kCbeta][s][mk]),
                        ga = hm_ld4(&sh.cf[kCgamma][s][mk]);
#pragma unroll
            for (int r = 0; r < 4; ++r) M[r] = fmaf(ga[r], y2[r], fmaf(be[r], y3[r], al[r] * M[r]));
          }
          d = hm_chain_step(blk, sh, s, d, i, q, zprev);
        }
        if (MODE == kHmFix && q == 0) Hout[(b * T + t0 + jb + s) * d_h + head * kHmD + i] = ST::pack(d);
      }
    }
    __syncthreads();  // the coefficients are rewritten by the next block
  }
  if constexpr (MODE == kHmReduce) {
    float* out = agg + ((b * n_heads + head) * n_ch + chunk) * kHmNC;
#pragma unroll
    for (int r = 0; r < 4; ++r) out[(mk + r) * kHmD + mr] = M[r];
    if (q == 0) out[kHmD * kHmD + i] = d;
  }
  if (MODE == kHmFix && slast && t0 + n == T && q == 0) slast[b * d_h + head * kHmD + i] = ST::pack(d);
  if (MODE != kHmFix && rpart) {
    rmax = wave_max_u32(rmax);
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

// Two-level carries for long chunk sequences: k_hm_group composes the
// aggregates of each group of kHmGroup consecutive chunks (in parallel over
// groups, the matrix products on the matrix cores), k_hm_scan then runs
// over the groups, and k_hm_expand turns each group's incoming carry into
// the carries of its chunks.  The serial chain is n_ch / kHmGroup + 2
// kHmGroup steps long instead of n_ch.
constexpr int kHmGroup = 16;

// the map of the whole group: (M, v) <- (M_c, v_c) o (M, v), c in order
__global__ void __launch_bounds__(kWave)
k_hm_group(const float* __restrict__ agg, int64_t n_ch, int64_t n_groups, float* __restrict__ gagg) {
  const int lane = threadIdx.x, i = lane >> 2, q = lane & 3;
  const int mr = lane & 15, mk = 4 * (lane >> 4);
  const int64_t g = blockIdx.x, head = blockIdx.y, b = blockIdx.z, n_heads = gridDim.y;
  const float* a = agg + (b * n_heads + head) * n_ch * kHmNC;
  __shared__ __attribute__((aligned(16))) float vs[kHmD];
  const int64_t c0 = g * kHmGroup, c1 = imin(n_ch, c0 + kHmGroup);
  hm_f4 M;
#pragma unroll
  for (int r = 0; r < 4; ++r) M[r] = (mk + r == mr) ? 1.0f : 0.0f;
  float v = 0.0f;
  for (int64_t c = c0; c < c1; ++c) {
    const float* ac = a + c * kHmNC;
    const hm_f4 xm = hm_ld4(ac + mr * kHmD + mk);     // operands of M_c as the left factor
    const hm_f4 row = hm_ld4(ac + i * kHmD + 4 * q);   // row i of M_c, columns 4q..4q+3
    const float vc = ac[kHmD * kHmD + i];
    hm_f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int p = 0; p < 4; ++p) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xm[p], M[p], acc, 0, 0, 0);
    M = acc;
    if (q == 0) vs[i] = v;
    __syncthreads();
    const hm_f4 vv = hm_ld4(vs + 4 * q);
    v = hm_rowsum(fmaf(row[3], vv[3], fmaf(row[2], vv[2], fmaf(row[1], vv[1], row[0] * vv[0])))) + vc;
    __syncthreads();  // vs is rewritten at the next chunk
  }
  float* out = gagg + ((b * n_heads + head) * n_groups + g) * kHmNC;
#pragma unroll
  for (int r = 0; r < 4; ++r) out[(mk + r) * kHmD + mr] = M[r];
  if (q == 0) out[kHmD * kHmD + i] = v;
}

// the carries of a group's chunks from the carry entering the group
__global__ void __launch_bounds__(kWave)
k_hm_expand(const float* __restrict__ agg, const float* __restrict__ gcarry, int64_t n_ch, int64_t n_groups,
            float* __restrict__ carry) {
  const int lane = threadIdx.x, i = lane >> 2, q = lane & 3;
  const int64_t g = blockIdx.x, head = blockIdx.y, b = blockIdx.z, n_heads = gridDim.y;
  const float* a = agg + (b * n_heads + head) * n_ch * kHmNC;
  float* cout = carry + (b * n_heads + head) * n_ch * kHmD;
  __shared__ __attribute__((aligned(16))) float ss[kHmD];
  const int64_t c0 = g * kHmGroup, c1 = imin(n_ch, c0 + kHmGroup);
  float s = gcarry[((b * n_heads + head) * n_groups + g) * kHmD + i];
  for (int64_t c = c0; c < c1; ++c) {
    const float* ac = a + c * kHmNC;
    const hm_f4 row = hm_ld4(ac + i * kHmD + 4 * q);
    const float vc = ac[kHmD * kHmD + i];
    if (q == 0) {
      cout[c * kHmD + i] = s;
      ss[i] = s;
    }
    __syncthreads();
    const hm_f4 sv = hm_ld4(ss + 4 * q);
    s = hm_rowsum(fmaf(row[3], sv[3], fmaf(row[2], sv[2], fmaf(row[1], sv[1], row[0] * sv[0])))) + vc;
    __syncthreads();
  }
}

// The sequential unroll: one wave per (row, head), h_t = f(h_(t-1), x_t).
template <int DT>
__global__ void __launch_bounds__(kWave)
k_hm_sequential(const typename Storage<DT>::T* __restrict__ xproj, const float* __restrict__ A,
                const typename Storage<DT>::T* __restrict__ h0, int64_t T, int64_t d_h,
                typename Storage<DT>::T* __restrict__ Hout, typename Storage<DT>::T* __restrict__ slast) {
  using ST = Storage<DT>;
  const int lane = threadIdx.x, i = lane >> 2, q = lane & 3;
  const int64_t head = blockIdx.x, b = blockIdx.y, n_heads = gridDim.x;
  const int64_t ch = head * kHmD + i;
  __shared__ float xs[kHmSeqBlock][3][kHmD];
  HmBlocks blk;
  hm_load_blocks(A, n_heads, head, lane, blk);
  float h = h0 ? ST::load(h0 + b * d_h + ch) : 0.0f;
  for (int64_t t0 = 0; t0 < T; t0 += kHmSeqBlock) {
    // the next block's inputs, all loads in flight at once
    const int n = static_cast<int>(imin(T - t0, kHmSeqBlock));
    const typename ST::T* xb = xproj + ((b * T + t0) * 3) * d_h + head * kHmD;
    __syncthreads();  // the previous block's reads are done
#pragma unroll 8
    for (int e = lane; e < n * 3 * kHmD; e += kWave) {
      const int j = e / (3 * kHmD), r = e - j * 3 * kHmD, g = r / kHmD, c = r - g * kHmD;
      xs[j][g][c] = ST::load(xb + (static_cast<int64_t>(j) * 3 + g) * d_h + c);
    }
    __syncthreads();
    for (int j = 0; j < n; ++j) {
      const float x[3] = {xs[j][0][i], xs[j][1][i], xs[j][2][i]};
      h = hm_step(blk, x, h, q);
      if (q == 0) Hout[(b * T + t0 + j) * d_h + ch] = ST::pack(h);
    }
  }
  if (slast && q == 0) slast[b * d_h + ch] = ST::pack(h);
}

}  // namespace prn
