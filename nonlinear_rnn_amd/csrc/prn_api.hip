// Host side of libprn: argument validation, workspace planning and the
// launch sequence of every entry point declared in include/prn.h.
//
// Nothing here synchronises with the device; everything is enqueued on the
// caller's stream (FAQs, "Does torch.compile / autocast work?": a fixed-K
// loop with no residual host sync).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <type_traits>

#include "backward.h"
#include "decode.h"
#include "headmix.h"
#include "newton_kernels.h"
#include "newton_sp.h"
#include "proj.h"
#include "prn.h"

namespace {

thread_local std::string g_err;

prn_status fail(prn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// three-phase geometry: lanes = 64 channels, NW waves of LS serial steps
constexpr int kLS = 8;
constexpr int kNW = 8;
constexpr int kLC = kLS * kNW;
constexpr int kScanSeg = 16;
// single-pass geometry (lane = channel, NW waves of LS serial steps).
// Longer chunks mean fewer carry look-backs per step, which is what bounds
// the kernel when few chains (rows x 64-channel tiles) run side by side:
// every chunk of a chain waits on the look-back of the chunks before it.
// Measured at the long LSTM shape (8 chains): LS = 6, 8, 10, 12 took 1.00,
// 0.97, 0.86, 0.78 ms; once the output addresses stopped being hoisted out
// of the iteration loop (236 -> 213 registers at LS = 12), LS = 14 and 16
// fit too: 0.756 and 0.713 ms (LS = 16 under a two-waves-per-SIMD register
// cap, no spills).  Shorter chunks under a three-waves-per-SIMD cap do not
// pay for their extra look-backs: LS = 8 (168 registers, 45 KB of LDS, three
// workgroups per CU) took 0.84 ms and LS = 10 (spills) 0.95 ms, against
// 0.69 ms for LS = 16 at two.  A Picard sweep takes the same LS = 16 (0.78 ms
// at K = 2, against 0.92 ms at LS = 10).  The GRU takes LS = 16 below 64
// chains (4 chains: 0.25 -> 0.18 ms against LS = 8) and LS = 12 above (128
// chains: 0.96 -> 0.91 ms; LS = 16 took 1.05 ms there).  With few chains the
// four-wave 64-step chunk also beat the other shapes tried on the 4-chain
// ragged pack (LS x NW = 16 x 4: 0.24 ms; 12 x 4: 0.27; 16 x 3: 0.27;
// 8 x 4: 0.32; 24 x 2: 0.31; 16 x 2: 0.34).  Once the last iteration was
// peeled out of the iteration loop (fp32 GRU at LS = 16: 168 -> 96
// registers), eight waves of 10 steps (80-step chunks, 69 KB of LDS, two
// workgroups per CU) beat it (MALL flushed; 32-chain GRU 8 x 4096 x 256 /
// 4-chain ragged pack): 16 x 4 0.105 / 0.255 ms; 10 x 8 0.099 / 0.220;
// 9 x 8 0.100 / 0.227; 8 x 8 0.098 / 0.236; 6 x 8 0.098 / 0.244; 4 x 16
// 0.127 / 0.290; 12 x 8 0.118 / 0.285; 10 x 6 0.108 / 0.264.  Eight waves
// lost where the chains are many or the state is wider: bf16 GRU at 128
// chains 8 x 8 0.978 and 5 x 8 0.953 ms against 0.836 at 10 x 4; the long
// LSTM 8 x 8 0.909 against 0.678 at 16 x 4.  With the waves' maps in one
// LDS buffer instead of two (the slot of each wave then carries its
// carry-in), 12 x 8 fits two workgroups per CU (77 KB) and took the ragged
// pack from 0.216 to 0.204 ms (32 chains: 0.0965 -> 0.0961 ms); the long
// LSTM at 8 x 8 (two workgroups per CU then) still took 0.894 ms, at 7 x 8
// 0.947, against 0.666 at 16 x 4.  The bf16 GRU at 128 chains then took
// 0.812 / 0.781 / 0.758 / 0.824 ms at LS = 10 / 11 / 12 / 13 (four waves);
// the long LSTM at LS = 18 (72-step chunks, 80 KB, still two per CU) 0.662
// against 0.673 ms, not taken: the fused forward's chunks must be multiples
// of 32 steps, and at equal chunks both forwards give the same bits.  Other
// long-LSTM shapes on the same build: 11 x 4 and 12 x 4 under a
// three-waves-per-SIMD cap 0.723 / 0.761 ms, 16 x 2 0.841, 16 x 3 0.823.
// bf16 storage needs more registers per step (unpacking): the bf16 LSTM
// keeps LS = 8 (LS = 12 needed 256 registers before the peel, LS = 16
// spilled); the bf16 GRU with many chains took LS = 10 while that was the
// longest chunk that kept four waves per SIMD (measured at 16 x 16384 x
// 512: LS = 8 / 10 took 1.06 / 0.97 ms then), and takes 12 since (above).
constexpr int kSpNW = 4;
constexpr int kSpLsLstm = 16, kSpLsLstmBf16 = 8, kSpLsGruMany = 12, kSpLsGruManyBf16 = 12;
constexpr int kSpNwLstm = 4, kSpNwLstmBf16 = 4, kSpNwGruMany = 4, kSpNwGruManyBf16 = 4;
constexpr int kSpLsGruFew = 12, kSpNwGruFew = 8;   // GRU below kSpManyChains chains
constexpr int kSpLsFusedGru = 16, kSpLsFusedLstm = 16;
// fused GRU below kSpManyChains chains: eight waves lost there (MALL flushed,
// 32-chain GRU / 4-chain ragged pack: 16 x 4 0.189 / 0.343 ms, 8 x 8 0.205 /
// 0.407, 4 x 8 0.227 / 0.508)
constexpr int kSpLsFusedGruFew = 16, kSpNwFusedGruFew = 4;
constexpr int64_t kSpManyChains = 64;
struct SpGeo {
  int ls, nw;   // steps per wave, waves per workgroup
};
SpGeo sp_geo(int cell, int dtype, int64_t n_chains) {
  if (cell != PRN_CELL_DIAG_GRU)
    return dtype == PRN_BF16 ? SpGeo{kSpLsLstmBf16, kSpNwLstmBf16} : SpGeo{kSpLsLstm, kSpNwLstm};
  if (n_chains < kSpManyChains) return {kSpLsGruFew, kSpNwGruFew};
  return dtype == PRN_BF16 ? SpGeo{kSpLsGruManyBf16, kSpNwGruManyBf16} : SpGeo{kSpLsGruMany, kSpNwGruMany};
}
// With the projection fused into the Newton kernel, a chunk must be a
// multiple of 32 steps (the projection's 32-row blocks), and longer chunks
// stream W from L2 fewer times per token: every fused GRU takes 64-step
// chunks (16 per lane), also with many chains where the unfused kernel takes
// 48 or 40 (bf16 GRU at 128 chains: 32-step chunks 2.54 ms, 64-step 1.76 ms).
SpGeo sp_geo_fused(int cell, int dtype, int64_t n_chains) {
  if (cell == PRN_CELL_DIAG_GRU)
    return n_chains < kSpManyChains ? SpGeo{kSpLsFusedGruFew, kSpNwFusedGruFew} : SpGeo{kSpLsFusedGru, kSpNW};
  if (dtype == PRN_F32) return {kSpLsFusedLstm, kSpNW};
  return {kSpLsLstmBf16, kSpNW};
}
constexpr unsigned kSpinLimit = 1u << 16;   // polls (~1 us each) of one look-back wait before giving up
// PRN_SPIN_LIMIT overrides the poll limit at every call; 0 makes every
// look-back wait give up at once (every chunk but the first of each chain),
// which exercises the error path without any fault or hang.
unsigned spin_limit() {
  const char* e = getenv("PRN_SPIN_LIMIT");
  if (e && *e) return unsigned(strtoul(e, nullptr, 10));
  return kSpinLimit;
}
// below this many independent chains, chunks publish their aggregate before
// polling (measured: helps 4-32 chains, hurts 128)
constexpr int64_t kAggFirstBelowChains = 64;

// PRN_ALGO=tp selects the multi-kernel three-phase schedule; the default is
// the single-pass kernel.  Read at every call, so workspace sizing and the
// forward agree within a process.
bool use_three_phase() {
  const char* e = getenv("PRN_ALGO");
  return e && (e[0] == 't' || e[0] == 'T');
}
constexpr int64_t kMaxGrid = 65535;
constexpr int64_t kMaxGrid1D = (int64_t(1) << 31) - 1;  // workgroups of a one-dimensional launch

struct Shape {
  int G, S;
  size_t elt;       // bytes per stored element
  int64_t rows;     // sequences: B, or n_seqs for a ragged pack
  bool ragged;
};

prn_status check_common(const prn_params* p, Shape* sh) {
  if (!p) return fail(PRN_ERR_INVALID_ARG, "params is NULL");
  if (p->cell != PRN_CELL_DIAG_GRU && p->cell != PRN_CELL_DIAG_LSTM)
    return fail(PRN_ERR_INVALID_ARG, "unknown cell %d", p->cell);
  if (p->dtype != PRN_F32 && p->dtype != PRN_BF16)
    return fail(PRN_ERR_INVALID_ARG, "unknown storage dtype %d", p->dtype);
  if (p->B < 1 || p->T < 0 || p->d_h < 1)
    return fail(PRN_ERR_INVALID_ARG, "bad sizes B=%lld T=%lld d_h=%lld", (long long)p->B,
                (long long)p->T, (long long)p->d_h);
  if (p->n_seqs < 0) return fail(PRN_ERR_INVALID_ARG, "n_seqs < 0");
  if (p->n_seqs > 0 && p->B != 1)
    return fail(PRN_ERR_INVALID_ARG, "a ragged pack (n_seqs > 0) needs B == 1, got B=%lld", (long long)p->B);
  if (p->B > kMaxGrid || p->n_seqs > kMaxGrid || (p->d_h + 63) / 64 > kMaxGrid)
    return fail(PRN_ERR_UNSUPPORTED, "B, n_seqs and d_h/64 must each be <= %lld", (long long)kMaxGrid);
  sh->G = p->cell == PRN_CELL_DIAG_GRU ? 3 : 4;
  sh->S = p->cell == PRN_CELL_DIAG_GRU ? 1 : 2;
  sh->elt = p->dtype == PRN_F32 ? 4 : 2;
  sh->ragged = p->n_seqs > 0;
  sh->rows = sh->ragged ? p->n_seqs : p->B;
  const double elems = double(p->B) * double(p->T) * sh->G * double(p->d_h);
  if (elems > 4.0e18) return fail(PRN_ERR_INVALID_ARG, "tensor too large");
  return PRN_OK;
}

bool misaligned(const void* ptr, size_t elt) { return ptr && (reinterpret_cast<uintptr_t>(ptr) % elt) != 0; }

prn_status check_newton_args(const prn_params* p, const Shape& sh, const void* xproj, const void* h0,
                             const int32_t* cu, const void* H_out) {
  if (!p->a) return fail(PRN_ERR_INVALID_ARG, "recurrent weights a is NULL");
  if (p->T > 0 && (!xproj || !H_out)) return fail(PRN_ERR_INVALID_ARG, "xproj or H_out is NULL");
  if (sh.ragged && !cu) return fail(PRN_ERR_INVALID_ARG, "n_seqs > 0 but cu_seqlens is NULL");
  if (!sh.ragged && cu) return fail(PRN_ERR_INVALID_ARG, "cu_seqlens given but n_seqs == 0");
  if (misaligned(xproj, sh.elt) || misaligned(h0, sh.elt) || misaligned(H_out, sh.elt) ||
      misaligned(p->state_last_out, sh.elt) || misaligned(p->states_out, sh.elt) || misaligned(p->a, 4) ||
      misaligned(p->error_out, 4) ||
      misaligned(cu, 4))
    return fail(PRN_ERR_INVALID_ARG, "a tensor pointer is not aligned to its element size");
  return PRN_OK;
}

// backward geometry.  Single pass (default): per-cell chunks of LS steps
// per lane times NW waves; workspace: status words, chunk records and the da
// partials.  Three-phase (PRN_ALGO=tp): chunks of kLC steps; aggregates,
// carries, da partials.
// Measured with the MALL flushed (ms; LS x NW): long LSTM 8 x 8: 0.77,
// 8 x 16: 0.70-0.73, 7 x 16: 0.74, 6 x 16: 0.75, 8 x 12: 0.79, 8 x 4: 0.93,
// 12 x 8: 0.93; GRU below 64 chains (8 x 4096 x 256 / one 65536-step ragged
// row): 16 x 8: 0.125-0.133 / 0.190, 16 x 16: 0.117-0.120 / 0.177-0.179,
// 12 x 16: 0.110 / 0.204, 20 x 16: 0.112 / 0.210, 16 x 12: 0.139 / 0.213;
// the bf16 GRU at 128 chains: 8 x 8: 0.925, 8 x 4: 0.909, 6 x 8: 0.97,
// 12 x 8: 1.14, 4 x 16: 1.36.  Sixteen waves of 1024 threads fill a CU as
// two eight-wave workgroups did (the LSTM instance keeps 124 registers, four
// waves per SIMD) with half the look-backs per step; long chunks pay off
// only with few chains, as in the forward.
struct BwGeo {
  int ls, nw;
};
constexpr BwGeo kBwLstm{8, 16}, kBwGruFew{16, 16}, kBwGruMany{8, 8};
BwGeo bw_geo(int cell, int64_t n_chains) {
  if (cell != PRN_CELL_DIAG_GRU) return kBwLstm;
  return n_chains < kSpManyChains ? kBwGruFew : kBwGruMany;
}
int bw_chunk(int cell, int64_t n_chains, bool sp) {
  if (!sp) return kLC;
  const BwGeo g = bw_geo(cell, n_chains);
  return g.ls * g.nw;
}
// dL/da is reduced from per-chunk partials in two fixed-order levels: up to
// kDaSlices slices of chunks, then the slices (one level with only
// G x d_h/64 workgroups took 70 us at the long LSTM shape).
constexpr int64_t kDaSlices = 64;

struct PlanBw {
  bool sp;
  int lc;  // steps per chunk
  int64_t n_ch, n_tiles, n_chains;
  size_t words_off, n_words, agg_off, pre_off, carry_off, da_off, dslice_off, total;
};

PlanBw plan_bw(const prn_params* p, const Shape& sh) {
  PlanBw pl{};
  pl.sp = !use_three_phase();
  pl.n_tiles = (p->d_h + 63) / 64;
  pl.n_chains = p->B * pl.n_tiles;
  pl.lc = bw_chunk(p->cell, pl.n_chains, pl.sp);
  pl.n_ch = (p->T + pl.lc - 1) / pl.lc;
  const size_t NC = sh.S * sh.S + sh.S;
  const size_t units = size_t(p->B) * pl.n_ch * p->d_h;
  size_t off = 0;
  if (pl.sp) {
    const size_t nrec = size_t(pl.n_chains) * pl.n_ch;
    pl.n_words = 2 + nrec;
    pl.words_off = 0;
    pl.agg_off = align_up(pl.n_words * 4);
    pl.pre_off = pl.agg_off + align_up(nrec * NC * 64 * 4);
    off = pl.pre_off + align_up(nrec * sh.S * 64 * 4);
  } else {
    pl.agg_off = 0;
    pl.carry_off = align_up(units * NC * 4);
    off = pl.carry_off + align_up(units * sh.S * 4);
  }
  pl.da_off = off;
  pl.dslice_off = pl.da_off + align_up(units * sh.G * 4);
  pl.total = pl.dslice_off + align_up(size_t(kDaSlices) * sh.G * p->d_h * 4);
  return pl;
}

struct Plan {
  int64_t n_ch;
  int64_t n_wg;  // workgroups of a Newton-pass launch (residual partials per iteration)
  int nbuf;      // iterate buffers: H^(k) for k = 1..K-1 lives in buffer (k - 1) % 2
  size_t agg_off, carry_off, rpart_off, it_off[2], it_bytes, total;
};

Plan plan_tp(const prn_params* p, const Shape& sh, int K) {
  Plan pl{};
  pl.n_ch = (p->T + kLC - 1) / kLC;
  const size_t NC = sh.S * sh.S + sh.S;
  const size_t agg = align_up(size_t(p->B) * pl.n_ch * NC * p->d_h * 4);
  const size_t car = align_up(size_t(p->B) * pl.n_ch * sh.S * p->d_h * 4);
  const size_t it = align_up(size_t(p->B) * p->T * sh.S * p->d_h * sh.elt);
  pl.n_wg = pl.n_ch * ((p->d_h + 63) / 64) * p->B;
  const size_t rp = align_up(size_t(K + 1) * pl.n_wg * 4);
  pl.nbuf = K >= 3 ? 2 : (K == 2 ? 1 : 0);
  pl.agg_off = 0;
  pl.carry_off = agg;
  pl.rpart_off = agg + car;
  pl.it_off[0] = agg + car + rp;
  pl.it_off[1] = agg + car + rp + it;
  pl.it_bytes = it;
  pl.total = agg + car + rp + pl.nbuf * it;
  return pl;
}

struct PlanSp {
  int ls;  // steps per lane
  int nw;  // waves per workgroup
  int64_t n_ch, n_tiles, n_chains, n_wg;
  size_t status_off, n_status;  // words zeroed per launch: ticket, error, K*n_chains*n_ch statuses
  size_t agg_off, pre_off, rpart_off, total;
};

PlanSp plan_sp(const prn_params* p, const Shape& sh, int K, bool fused = false) {
  PlanSp pl{};
  pl.n_tiles = (p->d_h + 63) / 64;
  pl.n_chains = p->B * pl.n_tiles;
  const SpGeo geo = fused ? sp_geo_fused(p->cell, p->dtype, pl.n_chains) : sp_geo(p->cell, p->dtype, pl.n_chains);
  pl.ls = geo.ls;
  pl.nw = geo.nw;
  const int lc = pl.ls * pl.nw;
  pl.n_ch = (p->T + lc - 1) / lc;
  pl.n_wg = pl.n_ch * pl.n_chains;
  const size_t nrec = size_t(K) * pl.n_chains * pl.n_ch;
  const size_t NC = sh.S * sh.S + sh.S;
  pl.n_status = 2 + nrec;
  pl.status_off = 0;
  pl.agg_off = align_up(pl.n_status * 4);
  pl.pre_off = pl.agg_off + align_up(nrec * NC * 64 * 4);
  pl.rpart_off = pl.pre_off + align_up(nrec * sh.S * 64 * 4);
  pl.total = pl.rpart_off + align_up(size_t(K + 1) * pl.n_wg * 4);
  return pl;
}

size_t workspace_needed(const prn_params* p, const Shape& sh, int K) {
  return use_three_phase() ? plan_tp(p, sh, K).total : plan_sp(p, sh, K).total;
}
// the fused forward always runs the single-pass schedule
size_t fused_workspace_needed(const prn_params* p, const Shape& sh, int K) {
  return p->T > 0 ? plan_sp(p, sh, K, true).total : 0;
}

prn_status launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PRN_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return PRN_OK;
}

template <int DT>
void final_states_empty(const prn_params* p, const Shape& sh, const void* h0, const int32_t* cu,
                        hipStream_t st) {
  using T = typename prn::Storage<DT>::T;
  if (!p->state_last_out || !sh.ragged) return;
  const int64_t n = p->n_seqs * sh.S * p->d_h;
  const int S = sh.S;
  const dim3 grid(unsigned((n + 255) / 256));
  if (S == 1)
    prn::k_empty_segments<DT, 1><<<grid, 256, 0, st>>>(cu, p->n_seqs, p->d_h, static_cast<const T*>(h0),
                                                      static_cast<T*>(p->state_last_out));
  else
    prn::k_empty_segments<DT, 2><<<grid, 256, 0, st>>>(cu, p->n_seqs, p->d_h, static_cast<const T*>(h0),
                                                      static_cast<T*>(p->state_last_out));
}

template <class C, int DT>
prn_status newton_tp(const prn_params* p, const Shape& sh, const void* xproj_v, const void* h0_v, int K,
                     const int32_t* cu, void* Hout_v, float* res) {
  using T = typename prn::Storage<DT>::T;
  constexpr int S = C::S;
  hipStream_t st = static_cast<hipStream_t>(p->stream);
  const Plan pl = plan_tp(p, sh, K);
  const T* xproj = static_cast<const T*>(xproj_v);
  const T* h0 = static_cast<const T*>(h0_v);
  T* Hout = static_cast<T*>(Hout_v);
  T* slast = static_cast<T*>(p->state_last_out);
  char* ws = static_cast<char*>(p->workspace);
  float* agg = reinterpret_cast<float*>(ws + pl.agg_off);
  float* carry = reinterpret_cast<float*>(ws + pl.carry_off);
  // H^(k) (k = 1..K-1) is stored in iterate buffer (k - 1) % 2; iteration k
  // reads buffer (k - 2) % 2 and writes (k - 1) % 2, never the same one.
  auto iter_buf = [&](int k) -> T* {
    const int i = (k - 1) & 1;
    if (k < 1 || k >= K || i >= pl.nbuf || pl.it_off[i] + pl.it_bytes > pl.total) return nullptr;
    return reinterpret_cast<T*>(ws + pl.it_off[i]);
  };
  for (int k = 1; k < K; ++k)
    if (!iter_buf(k)) return fail(PRN_ERR_WORKSPACE, "internal: iterate %d has no workspace buffer", k);
  float* rpart = reinterpret_cast<float*>(ws + pl.rpart_off);
  auto slot = [&](int k) { return res ? rpart + k * pl.n_wg : nullptr; };

  const dim3 grid(unsigned(pl.n_ch), unsigned((p->d_h + 63) / 64), unsigned(p->B));
  const dim3 block(64 * kNW);
  const dim3 sgrid(unsigned((p->d_h + 63) / 64), unsigned(p->B));
  const dim3 sblock(64 * kScanSeg);
  if (p->T > 0) {
    prn::k_tp_first<C, DT, kLS, kNW><<<grid, block, 0, st>>>(xproj, h0, cu, p->a, p->T, p->d_h, p->n_seqs,
                                                             pl.n_ch, agg, slot(0));
    prn::k_tp_scan<S, kScanSeg><<<sgrid, sblock, 0, st>>>(agg, carry, p->d_h, pl.n_ch);
    for (int k = 1; k < K; ++k) {
      const T* hprev = k == 1 ? nullptr : iter_buf(k - 1);
      prn::k_tp_fix<C, DT, kLS, kNW, true, false><<<grid, block, 0, st>>>(
          xproj, hprev, h0, cu, p->a, p->T, p->d_h, p->n_seqs, pl.n_ch, carry, iter_buf(k), nullptr, nullptr,
          nullptr, agg, slot(k));
      prn::k_tp_scan<S, kScanSeg><<<sgrid, sblock, 0, st>>>(agg, carry, p->d_h, pl.n_ch);
    }
    const T* hprev = K == 1 ? nullptr : iter_buf(K - 1);
    prn::k_tp_fix<C, DT, kLS, kNW, false, true><<<grid, block, 0, st>>>(
        xproj, hprev, h0, cu, p->a, p->T, p->d_h, p->n_seqs, pl.n_ch, carry, nullptr, Hout, slast,
        static_cast<T*>(p->states_out), nullptr, slot(K));
    if (res) prn::k_residual_reduce<<<unsigned(K + 1), 1024, 0, st>>>(rpart, pl.n_wg, res);
  } else {
    if (res) prn::k_zero_f32<<<unsigned((K + 256) / 256), 256, 0, st>>>(res, K + 1);
  }
  if (p->T == 0 && slast && !sh.ragged) {
    // zero-length rows: the final state is the initial state
    const int64_t n = p->B * S * p->d_h;
    prn::k_copy_or_zero<T><<<unsigned((n + 255) / 256), 256, 0, st>>>(h0, slast, n);
  }
  final_states_empty<DT>(p, sh, h0_v, cu, st);
  return launched("prn_newton_forward");
}

// fx != NULL: the projection is fused into the Newton kernel (xproj_v unused)
template <class C, int DT>
prn_status newton_sp(const prn_params* p, const Shape& sh, const void* xproj_v, const void* h0_v, int K,
                     const int32_t* cu, void* Hout_v, float* res, const prn::FxArgs* fx = nullptr) {
  using T = typename prn::Storage<DT>::T;
  constexpr int S = C::S;
  hipStream_t st = static_cast<hipStream_t>(p->stream);
  const PlanSp pl = plan_sp(p, sh, K, fx != nullptr);
  if (pl.n_wg > kMaxGrid1D) return fail(PRN_ERR_UNSUPPORTED, "too many chunks for one launch (%lld)", (long long)pl.n_wg);
  const T* h0 = static_cast<const T*>(h0_v);
  T* slast = static_cast<T*>(p->state_last_out);
  char* ws = static_cast<char*>(p->workspace);
  if (p->T > 0) {
    prn::SpRecords rec;
    unsigned* words = reinterpret_cast<unsigned*>(ws + pl.status_off);
    rec.ticket = words;
    rec.error = p->error_out ? static_cast<unsigned*>(p->error_out) : words + 1;
    rec.status = words + 2;
    rec.agg = reinterpret_cast<float*>(ws + pl.agg_off);
    rec.pre = reinterpret_cast<float*>(ws + pl.pre_off);
    float* rpart = res ? reinterpret_cast<float*>(ws + pl.rpart_off) : nullptr;
    prn::k_zero_u32<<<unsigned((pl.n_status + 255) / 256), 256, 0, st>>>(words, int64_t(pl.n_status));
    using T_ = std::true_type;
    using F_ = std::false_type;
    const prn::FxArgs fa = fx ? *fx : prn::FxArgs{nullptr, nullptr, nullptr, 0, nullptr};
    // sweeps beyond T change nothing (every step's window already reaches
    // its segment's head), so the kernel never runs more than T of them
    const int picard = static_cast<int>(std::min<int64_t>(p->picard_iters, p->T));
    auto launch = [&](auto ls, auto nw, auto fxc) {
      constexpr int LS = decltype(ls)::value, NW = decltype(nw)::value;
      constexpr bool FX = decltype(fxc)::value;
      T* sout = static_cast<T*>(p->states_out);
      auto go = [&](auto ws, auto pic) {
        prn::k_newton_sp<C, DT, LS, NW, decltype(ws)::value, decltype(pic)::value, FX>
            <<<unsigned(pl.n_wg), 64 * NW, 0, st>>>(
                static_cast<const T*>(xproj_v), h0, cu, p->a, p->T, p->d_h, p->n_seqs, pl.n_ch, pl.n_tiles,
                pl.n_chains, K, static_cast<T*>(Hout_v), slast, sout, rpart, rec, spin_limit(),
                pl.n_chains < kAggFirstBelowChains, fa, picard);
      };
      if constexpr (FX) {
        if (sout) go(T_{}, F_{}); else go(F_{}, F_{});
      } else if (p->picard_iters > 0) {
        if (sout) go(T_{}, T_{}); else go(F_{}, T_{});
      } else {
        if (sout) go(T_{}, F_{}); else go(F_{}, F_{});
      }
    };
    using NW4 = std::integral_constant<int, kSpNW>;
    if (fx) {
      if constexpr (S == 2) {
        if constexpr (DT == prn::kBF16)
          launch(std::integral_constant<int, kSpLsLstmBf16>{}, NW4{}, T_{});
        else
          launch(std::integral_constant<int, kSpLsFusedLstm>{}, NW4{}, T_{});
      } else if (pl.n_chains < kSpManyChains) {
        launch(std::integral_constant<int, kSpLsFusedGruFew>{}, std::integral_constant<int, kSpNwFusedGruFew>{}, T_{});
      } else {
        launch(std::integral_constant<int, kSpLsFusedGru>{}, NW4{}, T_{});
      }
    } else if constexpr (S == 2) {
      if constexpr (DT == prn::kBF16)
        launch(std::integral_constant<int, kSpLsLstmBf16>{}, std::integral_constant<int, kSpNwLstmBf16>{}, F_{});
      else
        launch(std::integral_constant<int, kSpLsLstm>{}, std::integral_constant<int, kSpNwLstm>{}, F_{});
    } else {
      if (pl.n_chains < kSpManyChains)
        launch(std::integral_constant<int, kSpLsGruFew>{}, std::integral_constant<int, kSpNwGruFew>{}, F_{});
      else if constexpr (DT == prn::kBF16)
        launch(std::integral_constant<int, kSpLsGruManyBf16>{}, std::integral_constant<int, kSpNwGruManyBf16>{}, F_{});
      else
        launch(std::integral_constant<int, kSpLsGruMany>{}, std::integral_constant<int, kSpNwGruMany>{}, F_{});
    }
    if (res) prn::k_residual_reduce<<<unsigned(K + 1), 1024, 0, st>>>(rpart, pl.n_wg, res);
  } else {
    if (res) prn::k_zero_f32<<<unsigned((K + 256) / 256), 256, 0, st>>>(res, K + 1);
    if (slast && !sh.ragged) {
      const int64_t n = p->B * S * p->d_h;
      prn::k_copy_or_zero<T><<<unsigned((n + 255) / 256), 256, 0, st>>>(h0, slast, n);
    }
  }
  final_states_empty<DT>(p, sh, h0_v, cu, st);
  return launched("prn_newton_forward");
}

template <class C, int DT>
prn_status newton(const prn_params* p, const Shape& sh, const void* xproj, const void* h0, int K,
                  const int32_t* cu, void* Hout, float* res) {
  if (use_three_phase()) return newton_tp<C, DT>(p, sh, xproj, h0, K, cu, Hout, res);
  return newton_sp<C, DT>(p, sh, xproj, h0, K, cu, Hout, res);
}

template <class C, int DT>
prn_status sequential(const prn_params* p, const Shape& sh, const void* xproj_v, const void* h0_v,
                      const int32_t* cu, void* Hout_v) {
  using T = typename prn::Storage<DT>::T;
  hipStream_t st = static_cast<hipStream_t>(p->stream);
  const dim3 grid(unsigned((p->d_h + 63) / 64), unsigned(sh.rows));
  prn::k_sequential<C, DT><<<grid, 64, 0, st>>>(static_cast<const T*>(xproj_v), static_cast<const T*>(h0_v), cu,
                                                p->a, p->T, p->d_h, p->n_seqs, static_cast<T*>(Hout_v),
                                                static_cast<T*>(p->state_last_out), static_cast<T*>(p->states_out));
  return launched("prn_sequential_forward");
}

template <class C, int DT>
prn_status backward(const prn_params* p, const Shape& sh, const void* xproj_v, const void* h0_v, const int32_t* cu,
                    const void* states_v, const void* dH_v, const void* dsl_v, void* dxproj_v, float* da,
                    void* dh0_v) {
  using T = typename prn::Storage<DT>::T;
  constexpr int G = C::G, S = C::S;
  hipStream_t st = static_cast<hipStream_t>(p->stream);
  const PlanBw pl = plan_bw(p, sh);
  const T* xproj = static_cast<const T*>(xproj_v);
  const T* h0 = static_cast<const T*>(h0_v);
  const T* states = static_cast<const T*>(states_v);
  const T* dH = static_cast<const T*>(dH_v);
  const T* dsl = static_cast<const T*>(dsl_v);
  T* dxproj = static_cast<T*>(dxproj_v);
  T* dh0 = static_cast<T*>(dh0_v);
  if (p->T > 0) {
    char* ws = static_cast<char*>(p->workspace);
    float* dap = reinterpret_cast<float*>(ws + pl.da_off);
    if (pl.sp) {
      prn::SpRecords rec;
      unsigned* words = reinterpret_cast<unsigned*>(ws + pl.words_off);
      rec.ticket = words;
      rec.error = p->error_out ? static_cast<unsigned*>(p->error_out) : words + 1;
      rec.status = words + 2;
      rec.agg = reinterpret_cast<float*>(ws + pl.agg_off);
      rec.pre = reinterpret_cast<float*>(ws + pl.pre_off);
      prn::k_zero_u32<<<unsigned((pl.n_words + 255) / 256), 256, 0, st>>>(words, int64_t(pl.n_words));
      auto launch = [&](auto ls, auto nw) {
        constexpr int LS = decltype(ls)::value, NW = decltype(nw)::value;
        prn::k_bw_sp<C, DT, LS, NW><<<unsigned(pl.n_ch * pl.n_chains), 64 * NW, 0, st>>>(
            xproj, states, h0, cu, p->a, dH, dsl, p->T, p->d_h, p->n_seqs, pl.n_ch, pl.n_tiles, pl.n_chains, dxproj,
            dh0, dap, rec, spin_limit(), pl.n_chains < kAggFirstBelowChains);
      };
      // the geometry bw_chunk planned the workspace for
      if constexpr (S == 1) {
        if (pl.n_chains < kSpManyChains)
          launch(std::integral_constant<int, kBwGruFew.ls>{}, std::integral_constant<int, kBwGruFew.nw>{});
        else
          launch(std::integral_constant<int, kBwGruMany.ls>{}, std::integral_constant<int, kBwGruMany.nw>{});
      } else {
        launch(std::integral_constant<int, kBwLstm.ls>{}, std::integral_constant<int, kBwLstm.nw>{});
      }
    } else {
      float* agg = reinterpret_cast<float*>(ws + pl.agg_off);
      float* carry = reinterpret_cast<float*>(ws + pl.carry_off);
      const dim3 grid(unsigned(pl.n_ch), unsigned((p->d_h + 63) / 64), unsigned(p->B));
      const dim3 block(64 * kNW);
      prn::k_bw_reduce<C, DT, kLS, kNW><<<grid, block, 0, st>>>(xproj, states, h0, cu, p->a, dH, dsl, p->T, p->d_h,
                                                                p->n_seqs, pl.n_ch, agg);
      prn::k_tp_scan<S, kScanSeg><<<dim3(unsigned((p->d_h + 63) / 64), unsigned(p->B)), 64 * kScanSeg, 0, st>>>(
          agg, carry, p->d_h, pl.n_ch);
      prn::k_bw_fix<C, DT, kLS, kNW><<<grid, block, 0, st>>>(xproj, states, h0, cu, p->a, dH, dsl, p->T, p->d_h,
                                                             p->n_seqs, pl.n_ch, carry, dxproj, dh0, dap);
    }
    float* dsl_part = reinterpret_cast<float*>(ws + pl.dslice_off);
    const int64_t n_units = p->B * pl.n_ch;
    const int64_t per = (n_units + kDaSlices - 1) / kDaSlices;
    const int64_t n_slices = (n_units + per - 1) / per;
    prn::k_bw_da_partial<G><<<dim3(unsigned((p->d_h + 63) / 64), unsigned(G), unsigned(n_slices)), 256, 0, st>>>(
        dap, n_units, per, p->d_h, dsl_part);
    prn::k_bw_da_reduce<G><<<dim3(unsigned((p->d_h + 63) / 64), unsigned(G)), 256, 0, st>>>(
        dsl_part, n_slices, p->d_h, da);
  } else {
    prn::k_zero_f32<<<unsigned((G * p->d_h + 255) / 256), 256, 0, st>>>(da, G * p->d_h);
    if (dh0 && !sh.ragged) {
      const int64_t n = p->B * S * p->d_h;
      prn::k_copy_or_zero<T><<<unsigned((n + 255) / 256), 256, 0, st>>>(dsl, dh0, n);
    }
  }
  if (dh0 && sh.ragged) {
    const int64_t n = p->n_seqs * S * p->d_h;
    prn::k_bw_empty_dh0<DT, S><<<unsigned((n + 255) / 256), 256, 0, st>>>(cu, p->n_seqs, p->d_h, dsl, dh0);
  }
  return launched("prn_newton_backward");
}

// ---- head-mix GRU (dense d_head x d_head recurrent blocks) ----
struct PlanHm {
  int64_t n_heads, n_ch, n_wg, n_groups;  // n_groups = 0: one-level carries
  size_t iter_off, n_iter, agg_off, carry_off, rpart_off, gagg_off, gcarry_off, total;
};

PlanHm plan_hm(const prn_params* p, int K) {
  PlanHm pl{};
  pl.n_heads = p->d_h / prn::kHmD;
  pl.n_ch = (p->T + prn::kHmChunk - 1) / prn::kHmChunk;
  pl.n_wg = p->B * pl.n_heads * pl.n_ch;
  pl.n_iter = size_t(std::min(K - 1, 2));  // ping-pong iterates H^(1..K-1); H^(K) goes to H_out
  const size_t it = align_up(size_t(p->B) * p->T * p->d_h * (p->dtype == PRN_BF16 ? 2 : 4));
  pl.iter_off = 0;
  pl.agg_off = pl.n_iter * it;
  pl.carry_off = pl.agg_off + align_up(size_t(pl.n_wg) * prn::kHmNC * 4);
  pl.rpart_off = pl.carry_off + align_up(size_t(pl.n_wg) * prn::kHmD * 4);
  pl.gagg_off = pl.rpart_off + align_up(size_t(K + 1) * pl.n_wg * 4);
  // two-level carries once the chunk chain is longer than two groups
  pl.n_groups = pl.n_ch > 2 * prn::kHmGroup ? (pl.n_ch + prn::kHmGroup - 1) / prn::kHmGroup : 0;
  const size_t ng = size_t(p->B) * pl.n_heads * pl.n_groups;
  pl.gcarry_off = pl.gagg_off + align_up(ng * prn::kHmNC * 4);
  pl.total = pl.gcarry_off + align_up(ng * prn::kHmD * 4);
  return pl;
}

// Head-mix support: the GRU, fp32 or bf16 storage, rectangular batches (the
// pages' head-mix fused path takes no ragged pack), d_head = 16.
prn_status check_head(const prn_params* p, Shape* sh, int32_t d_head) {
  prn_status s = check_common(p, sh);
  if (s != PRN_OK) return s;
  if (p->cell != PRN_CELL_DIAG_GRU) return fail(PRN_ERR_UNSUPPORTED, "head-mix blocks are built for the GRU cell");
  if (p->n_seqs != 0) return fail(PRN_ERR_UNSUPPORTED, "head-mix takes rectangular batches, not a ragged pack");
  if (d_head != prn::kHmD) return fail(PRN_ERR_UNSUPPORTED, "d_head = %d: head-mix is built for d_head = 16", d_head);
  if (p->d_h % d_head != 0) return fail(PRN_ERR_INVALID_ARG, "d_h = %lld is not a multiple of d_head", (long long)p->d_h);
  if (p->d_h / d_head > kMaxGrid) return fail(PRN_ERR_UNSUPPORTED, "more than %lld heads", (long long)kMaxGrid);
  if (p->states_out || p->picard_iters)
    return fail(PRN_ERR_UNSUPPORTED, "head-mix has no states_out or Picard sweep");
  return PRN_OK;
}

// ---- the projection's backward ----
// dW = dxproj^T x reduces over tokens, the row index of both operands.
// When G d_h and d_in are multiples of 256, the dW tiles read both operands
// along their rows (token-major K stages; fp32 through the split into term
// planes, bf16 through transposed LDS reads) and take dxproj's column sums
// per token slice on the way (dbias).  Otherwise both operands are first
// transposed into the workspace (token-padded with zeros to splits x ks) for
// the split-K instance of the forward's tile, and dbias comes from the
// column sums the dxproj transpose takes (per 64 tokens).  Either way slice
// z multiplies tokens [z ks, (z+1) ks) into its own fp32 block and the
// blocks are summed in slice order.  dx = dxproj W only needs W transposed;
// dxproj is read in place when its rows are whole 16-byte chunks, else from
// a zero-padded copy.  Every column-sum set is reduced in two fixed-order
// levels.
struct PlanPb {
  int64_t M, N, Kd;      // tokens, G d_h, d_in
  bool do_dx, do_dw, do_db;
  bool pad_g;            // dxproj rows are not whole 16-byte chunks: use a padded copy for dx
  bool tn;               // dW without transposed copies (G d_h and d_in multiples of 256)
  int64_t Np;            // row length (elements) of W^T and of the padded dxproj
  int splits;
  int64_t ks, Mp, n_rt;  // tokens per slice, padded tokens, 64-token tiles of the dxproj transpose
  int64_t n_cs;           // rows of column sums: a row per slice (dW along the rows), else per 64-token tile
  int64_t n_slices, per;  // the column sums: n_cs rows reduced in n_slices slices of per rows
  size_t wt_off, gp_off, gt_off, xt_off, part_off, csum_off, cslice_off, total;
};
constexpr int64_t kPbWgTarget = 1024;   // workgroups the split-K product aims for (128 x 128 tiles)
constexpr int64_t kPbWgTargetTn = 256;  // the same for 256 x 256 tiles, one workgroup per CU
constexpr int64_t kPbTok = 256;         // slices are multiples of 256 tokens

PlanPb plan_pb(const prn_params* p, const Shape& sh, bool dx, bool dw, bool db) {
  PlanPb pl{};
  pl.M = p->B * p->T;
  pl.N = sh.G * p->d_h;
  pl.Kd = p->d_in;
  pl.do_dx = dx && pl.M > 0;
  pl.do_dw = dw && pl.M > 0;
  pl.do_db = db && pl.M > 0;
  const int64_t vec = 16 / int64_t(sh.elt);
  pl.pad_g = pl.N % vec != 0;
  pl.Np = pl.pad_g ? (pl.N + vec - 1) / vec * vec : pl.N;
  pl.tn = pl.N % 256 == 0 && pl.Kd % 256 == 0;
  const int64_t tiles = pl.tn ? (pl.N / 256) * (pl.Kd / 256) : ((pl.N + 127) / 128) * ((pl.Kd + 127) / 128);
  const int64_t target = pl.tn ? kPbWgTargetTn : kPbWgTarget;
  // 128 x 128 tiles: at least the target; 256 x 256 tiles (one workgroup
  // per CU): at most, so that the slices run in one round
  int64_t splits = pl.tn ? std::max<int64_t>(1, target / tiles) : (target + tiles - 1) / tiles;
  splits = std::max<int64_t>(1, std::min<int64_t>(splits, (pl.M + kPbTok - 1) / kPbTok));
  pl.ks = ((pl.M + splits - 1) / splits + kPbTok - 1) / kPbTok * kPbTok;
  if (pl.tn) splits = std::max<int64_t>(1, (pl.M + pl.ks - 1) / pl.ks);   // no slice left empty
  pl.splits = int(splits);
  pl.Mp = pl.ks * splits;
  pl.n_rt = (pl.Mp + 63) / 64;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  if (pl.do_dx) {
    pl.wt_off = take(size_t(pl.Kd) * pl.Np * sh.elt);
    if (pl.pad_g) pl.gp_off = take(size_t(pl.M) * pl.Np * sh.elt);
  }
  if (pl.do_dw) {
    if (!pl.tn) {
      pl.gt_off = take(size_t(pl.N) * pl.Mp * sh.elt);
      pl.xt_off = take(size_t(pl.Kd) * pl.Mp * sh.elt);
    }
    pl.part_off = take(size_t(pl.splits) * pl.N * pl.Kd * 4);
  }
  if (pl.do_db) {
    pl.n_cs = pl.do_dw && pl.tn ? pl.splits : pl.n_rt;
    pl.per = (pl.n_cs + kDaSlices - 1) / kDaSlices;
    pl.n_slices = (pl.n_cs + pl.per - 1) / pl.per;
    // sized for the 64-token tiles (at least the slices) whichever outputs
    // are asked for, so the size queried with every output covers any call
    pl.csum_off = take(size_t(std::max(pl.n_rt, int64_t(pl.splits))) * pl.N * 4);
    auto slices_for = [](int64_t n) {
      const int64_t per = (n + kDaSlices - 1) / kDaSlices;
      return (n + per - 1) / per;
    };
    pl.cslice_off = take(size_t(std::max(slices_for(pl.n_rt), slices_for(pl.splits))) * pl.N * 4);
  }
  pl.total = off;
  return pl;
}

// ---- scratch of the allocation-free forward ----
// One file-scope device array per GPU, alive until the process ends.  Host
// code never uses the array's name as an address (on the host it names a
// stand-in, not device memory): each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = PRN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

prn_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PRN_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PRN_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(PRN_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PRN_OK;
}

}  // namespace

extern "C" {

prn_status prn_newton_forward_noalloc(const void* xproj, const prn_params* p, const void* h0, int32_t K,
                                      const int32_t* cu, void* H_out, float* residual_out) {
  Shape sh;
  prn_status s = check_common(p, &sh);
  if (s != PRN_OK) return s;
  if (K < 1) return fail(PRN_ERR_INVALID_ARG, "K must be >= 1, got %d", K);
  if (p->picard_iters < 0) return fail(PRN_ERR_INVALID_ARG, "picard_iters must be >= 0");
  if ((s = check_newton_args(p, sh, xproj, h0, cu, H_out)) != PRN_OK) return s;
  if (misaligned(residual_out, 4)) return fail(PRN_ERR_INVALID_ARG, "residual_out is not 4-byte aligned");
  const PlanSp pl = plan_sp(p, sh, K);
  if (pl.total > kScratchBytes)
    return fail(PRN_ERR_WORKSPACE, "this call needs %zu bytes of scratch; the allocation-free forward holds %zu "
                "(use prn_newton_forward with a caller workspace)", pl.total, kScratchBytes);
  prn_params q = *p;
  q.workspace = nullptr;
  q.workspace_bytes = kScratchBytes;
  if (p->T > 0 && (s = scratch_of_current_device(&q.workspace)) != PRN_OK) return s;
  if (p->cell == PRN_CELL_DIAG_GRU) {
    if (p->dtype == PRN_F32) return newton_sp<prn::CellGRU, prn::kF32>(&q, sh, xproj, h0, K, cu, H_out, residual_out);
    return newton_sp<prn::CellGRU, prn::kBF16>(&q, sh, xproj, h0, K, cu, H_out, residual_out);
  }
  if (p->dtype == PRN_F32) return newton_sp<prn::CellLSTM, prn::kF32>(&q, sh, xproj, h0, K, cu, H_out, residual_out);
  return newton_sp<prn::CellLSTM, prn::kBF16>(&q, sh, xproj, h0, K, cu, H_out, residual_out);
}

prn_status prn_decode_step(const void* x, const void* W, const float* bias, const prn_params* p,
                           const void* state_in, void* state_out, void* h_out) {
  Shape sh;
  prn_status s = check_common(p, &sh);
  if (s != PRN_OK) return s;
  if (p->T != 1) return fail(PRN_ERR_INVALID_ARG, "a decode step has T = 1, got T=%lld", (long long)p->T);
  if (sh.ragged) return fail(PRN_ERR_INVALID_ARG, "a decode step takes slots (B), not a ragged pack");
  if (p->d_in < 1) return fail(PRN_ERR_INVALID_ARG, "d_in must be >= 1");
  if (!x || !W || !p->a || !state_out) return fail(PRN_ERR_INVALID_ARG, "x, W, a or state_out is NULL");
  if (misaligned(x, sh.elt) || misaligned(W, sh.elt) || misaligned(bias, 4) || misaligned(p->a, 4) ||
      misaligned(state_in, sh.elt) || misaligned(state_out, sh.elt) || misaligned(h_out, sh.elt))
    return fail(PRN_ERR_INVALID_ARG, "a tensor pointer is not aligned to its element size");
  if (state_in && state_in == state_out) return fail(PRN_ERR_INVALID_ARG, "state_in and state_out alias");
  hipStream_t st = static_cast<hipStream_t>(p->stream);
  // one wave per (channel, group of 16 slots); 4 channels per workgroup
  const dim3 grid(unsigned((p->d_h + prn::kDecodeWaves - 1) / prn::kDecodeWaves),
                  unsigned((p->B + prn::kDecodeSlots - 1) / prn::kDecodeSlots));
  auto go = [&](auto cell, auto dt) {
    using C = decltype(cell);
    constexpr int DT = decltype(dt)::value;
    using T = typename prn::Storage<DT>::T;
    prn::k_decode<C, DT><<<grid, 64 * prn::kDecodeWaves, 0, st>>>(
        static_cast<const T*>(x), static_cast<const T*>(W), bias, p->a, p->B, p->d_in, p->d_h,
        static_cast<const T*>(state_in), static_cast<T*>(state_out), static_cast<T*>(h_out));
  };
  using F32 = std::integral_constant<int, prn::kF32>;
  using BF16 = std::integral_constant<int, prn::kBF16>;
  if (p->cell == PRN_CELL_DIAG_GRU) {
    if (p->dtype == PRN_F32) go(prn::CellGRU{}, F32{}); else go(prn::CellGRU{}, BF16{});
  } else {
    if (p->dtype == PRN_F32) go(prn::CellLSTM{}, F32{}); else go(prn::CellLSTM{}, BF16{});
  }
  return launched("prn_decode_step");
}

size_t prn_backward_workspace_bytes(const prn_params* p) {
  g_err.clear();  // a 0 result with no message means no workspace is needed
  Shape sh;
  if (check_common(p, &sh) != PRN_OK) return 0;
  return plan_bw(p, sh).total;
}

prn_status prn_newton_backward(const void* xproj, const prn_params* p, const void* h0, const int32_t* cu,
                               const void* states, const void* dH, const void* dstate_last, void* dxproj_out,
                               float* da_out, void* dh0_out) {
  Shape sh;
  prn_status s = check_common(p, &sh);
  if (s != PRN_OK) return s;
  if (!p->a) return fail(PRN_ERR_INVALID_ARG, "recurrent weights a is NULL");
  if (!da_out) return fail(PRN_ERR_INVALID_ARG, "da_out is NULL");
  if (p->T > 0 && (!xproj || !states || !dH || !dxproj_out))
    return fail(PRN_ERR_INVALID_ARG, "xproj, states, dH or dxproj_out is NULL");
  if (sh.ragged && !cu) return fail(PRN_ERR_INVALID_ARG, "n_seqs > 0 but cu_seqlens is NULL");
  if (!sh.ragged && cu) return fail(PRN_ERR_INVALID_ARG, "cu_seqlens given but n_seqs == 0");
  if (misaligned(xproj, sh.elt) || misaligned(h0, sh.elt) || misaligned(states, sh.elt) || misaligned(dH, sh.elt) ||
      misaligned(dstate_last, sh.elt) || misaligned(dxproj_out, sh.elt) || misaligned(dh0_out, sh.elt) ||
      misaligned(da_out, 4) || misaligned(p->a, 4) || misaligned(cu, 4) || misaligned(p->error_out, 4))
    return fail(PRN_ERR_INVALID_ARG, "a tensor pointer is not aligned to its element size");
  const PlanBw pl = plan_bw(p, sh);
  if (p->T > 0) {
    if (!p->workspace || p->workspace_bytes < pl.total)
      return fail(PRN_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed", p->workspace_bytes,
                  p->workspace, pl.total);
    if (reinterpret_cast<uintptr_t>(p->workspace) % kAlign)
      return fail(PRN_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
    if (pl.n_ch > 0x7fffffff) return fail(PRN_ERR_UNSUPPORTED, "sequence too long");
  }
  if (p->cell == PRN_CELL_DIAG_GRU) {
    if (p->dtype == PRN_F32)
      return backward<prn::CellGRU, prn::kF32>(p, sh, xproj, h0, cu, states, dH, dstate_last, dxproj_out, da_out,
                                                dh0_out);
    return backward<prn::CellGRU, prn::kBF16>(p, sh, xproj, h0, cu, states, dH, dstate_last, dxproj_out, da_out,
                                               dh0_out);
  }
  if (p->dtype == PRN_F32)
    return backward<prn::CellLSTM, prn::kF32>(p, sh, xproj, h0, cu, states, dH, dstate_last, dxproj_out, da_out,
                                               dh0_out);
  return backward<prn::CellLSTM, prn::kBF16>(p, sh, xproj, h0, cu, states, dH, dstate_last, dxproj_out, da_out,
                                              dh0_out);
}

int32_t prn_version(void) { return 200; }

const char* prn_last_error(void) { return g_err.c_str(); }

prn_status prn_validate_cu_seqlens(const int32_t* cu, int64_t n_seqs, int64_t N) {
  if (!cu) return fail(PRN_ERR_INVALID_ARG, "cu_seqlens is NULL");
  if (n_seqs < 1) return fail(PRN_ERR_INVALID_ARG, "cu_seqlens needs at least 2 entries (n_seqs >= 1)");
  if (cu[0] != 0) return fail(PRN_ERR_INVALID_ARG, "cu_seqlens[0] = %d, expected 0", cu[0]);
  for (int64_t j = 0; j < n_seqs; ++j)
    if (cu[j + 1] < cu[j])
      return fail(PRN_ERR_INVALID_ARG, "cu_seqlens decreases at %lld (%d -> %d)", (long long)j, cu[j], cu[j + 1]);
  if (cu[n_seqs] != N)
    return fail(PRN_ERR_INVALID_ARG, "cu_seqlens[-1] = %d, expected N = %lld", cu[n_seqs], (long long)N);
  return PRN_OK;
}

size_t prn_workspace_bytes(const prn_params* p, int32_t K) {
  g_err.clear();  // a 0 result with no message means no workspace is needed
  Shape sh;
  if (check_common(p, &sh) != PRN_OK) return 0;
  if (K < 1) {
    fail(PRN_ERR_INVALID_ARG, "K must be >= 1, got %d", K);
    return 0;
  }
  const size_t a = workspace_needed(p, sh, K), b = fused_workspace_needed(p, sh, K);
  return a > b ? a : b;
}

prn_status prn_newton_forward(const void* xproj, const prn_params* p, const void* h0, int32_t K,
                              const int32_t* cu, void* H_out, float* residual_out) {
  Shape sh;
  prn_status s = check_common(p, &sh);
  if (s != PRN_OK) return s;
  if (K < 1) return fail(PRN_ERR_INVALID_ARG, "K must be >= 1, got %d", K);
  if (p->picard_iters < 0) return fail(PRN_ERR_INVALID_ARG, "picard_iters must be >= 0");
  if (p->picard_iters > 0 && use_three_phase())
    return fail(PRN_ERR_UNSUPPORTED, "Picard warm-start runs in the single-pass schedule only (PRN_ALGO=tp)");
  if ((s = check_newton_args(p, sh, xproj, h0, cu, H_out)) != PRN_OK) return s;
  if (misaligned(residual_out, 4)) return fail(PRN_ERR_INVALID_ARG, "residual_out is not 4-byte aligned");
  const size_t need = workspace_needed(p, sh, K);
  if (need > 0 && (!p->workspace || p->workspace_bytes < need))
    return fail(PRN_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed", p->workspace_bytes,
                p->workspace, need);
  if (reinterpret_cast<uintptr_t>(p->workspace) % kAlign)
    return fail(PRN_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  if (p->cell == PRN_CELL_DIAG_GRU) {
    if (p->dtype == PRN_F32) return newton<prn::CellGRU, prn::kF32>(p, sh, xproj, h0, K, cu, H_out, residual_out);
    return newton<prn::CellGRU, prn::kBF16>(p, sh, xproj, h0, K, cu, H_out, residual_out);
  }
  if (p->dtype == PRN_F32) return newton<prn::CellLSTM, prn::kF32>(p, sh, xproj, h0, K, cu, H_out, residual_out);
  return newton<prn::CellLSTM, prn::kBF16>(p, sh, xproj, h0, K, cu, H_out, residual_out);
}

prn_status prn_newton_forward_fused(const void* x, const void* W, const float* bias, const prn_params* p,
                                    const void* h0, int32_t K, const int32_t* cu, void* H_out, float* residual_out,
                                    void* xproj_out) {
  Shape sh;
  prn_status s = check_common(p, &sh);
  if (s != PRN_OK) return s;
  if (K < 1) return fail(PRN_ERR_INVALID_ARG, "K must be >= 1, got %d", K);
  if (p->picard_iters < 0) return fail(PRN_ERR_INVALID_ARG, "picard_iters must be >= 0");
  if (p->picard_iters > 0)
    return fail(PRN_ERR_UNSUPPORTED, "the fused forward has no Picard sweep (use prn_input_proj + prn_newton_forward)");
  if (p->d_in < 1) return fail(PRN_ERR_INVALID_ARG, "d_in must be >= 1");
  if (p->T > 0 && (!x || !W)) return fail(PRN_ERR_INVALID_ARG, "x or W is NULL");
  if ((s = check_newton_args(p, sh, x, h0, cu, H_out)) != PRN_OK) return s;
  if (misaligned(x, 16) || misaligned(W, 16) || misaligned(xproj_out, 16) || misaligned(bias, 4))
    return fail(PRN_ERR_INVALID_ARG, "x, W and xproj_out must be 16-byte aligned, bias 4-byte aligned");
  if (misaligned(residual_out, 4)) return fail(PRN_ERR_INVALID_ARG, "residual_out is not 4-byte aligned");
  const int kvec = p->dtype == PRN_F32 ? 4 : 8;
  if (p->d_in % kvec != 0)
    return fail(PRN_ERR_UNSUPPORTED, "the fused projection needs d_in %% %d == 0 for this storage dtype", kvec);
  const size_t need = fused_workspace_needed(p, sh, K);
  if (need > 0 && (!p->workspace || p->workspace_bytes < need))
    return fail(PRN_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed", p->workspace_bytes,
                p->workspace, need);
  if (reinterpret_cast<uintptr_t>(p->workspace) % kAlign)
    return fail(PRN_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  const prn::FxArgs fx{x, W, bias, p->d_in, xproj_out};
  if (p->cell == PRN_CELL_DIAG_GRU) {
    if (p->dtype == PRN_F32)
      return newton_sp<prn::CellGRU, prn::kF32>(p, sh, nullptr, h0, K, cu, H_out, residual_out, &fx);
    return newton_sp<prn::CellGRU, prn::kBF16>(p, sh, nullptr, h0, K, cu, H_out, residual_out, &fx);
  }
  if (p->dtype == PRN_F32)
    return newton_sp<prn::CellLSTM, prn::kF32>(p, sh, nullptr, h0, K, cu, H_out, residual_out, &fx);
  return newton_sp<prn::CellLSTM, prn::kBF16>(p, sh, nullptr, h0, K, cu, H_out, residual_out, &fx);
}

prn_status prn_sequential_forward(const void* xproj, const prn_params* p, const void* h0, const int32_t* cu,
                                  void* H_out) {
  Shape sh;
  prn_status s = check_common(p, &sh);
  if (s != PRN_OK) return s;
  if ((s = check_newton_args(p, sh, xproj, h0, cu, H_out)) != PRN_OK) return s;
  if (p->cell == PRN_CELL_DIAG_GRU) {
    if (p->dtype == PRN_F32) return sequential<prn::CellGRU, prn::kF32>(p, sh, xproj, h0, cu, H_out);
    return sequential<prn::CellGRU, prn::kBF16>(p, sh, xproj, h0, cu, H_out);
  }
  if (p->dtype == PRN_F32) return sequential<prn::CellLSTM, prn::kF32>(p, sh, xproj, h0, cu, H_out);
  return sequential<prn::CellLSTM, prn::kBF16>(p, sh, xproj, h0, cu, H_out);
}

prn_status prn_input_proj(const void* x, const void* W, const float* bias, const prn_params* p, void* xproj_out) {
  Shape sh;
  prn_status s = check_common(p, &sh);
  if (s != PRN_OK) return s;
  if (p->d_in < 1) return fail(PRN_ERR_INVALID_ARG, "d_in must be >= 1");
  const int64_t M = p->B * p->T, N = sh.G * p->d_h, Kd = p->d_in;
  if (M == 0) return PRN_OK;
  if (!x || !W || !xproj_out) return fail(PRN_ERR_INVALID_ARG, "x, W or xproj_out is NULL");
  if (misaligned(x, 16) || misaligned(W, 16) || misaligned(xproj_out, 16) || misaligned(bias, 4))
    return fail(PRN_ERR_INVALID_ARG, "x, W and xproj_out must be 16-byte aligned");
  const int kvec = p->dtype == PRN_F32 ? 4 : 8;
  if (Kd % kvec != 0)
    return fail(PRN_ERR_UNSUPPORTED, "input projection needs d_in %% %d == 0 for this storage dtype", kvec);
  // one workgroup per output tile (at most 128 x 128 of them): the grid must fit
  if (M > (int64_t(1) << 31) * 128 || N > (int64_t(1) << 31) || ((M + 127) / 128) * ((N + 127) / 128) > kMaxGrid1D)
    return fail(PRN_ERR_UNSUPPORTED, "input projection too large");
  prn::launch_proj(p->dtype == PRN_BF16, x, W, bias, xproj_out, M, N, Kd, static_cast<hipStream_t>(p->stream));
  return launched("prn_input_proj");
}

size_t prn_input_proj_backward_workspace_bytes(const prn_params* p) {
  g_err.clear();  // a 0 result with no message means no workspace is needed
  Shape sh;
  if (check_common(p, &sh) != PRN_OK) return 0;
  if (p->d_in < 1) {
    fail(PRN_ERR_INVALID_ARG, "d_in must be >= 1");
    return 0;
  }
  return plan_pb(p, sh, true, true, true).total;
}

prn_status prn_input_proj_backward(const void* dxproj, const void* x, const void* W, const prn_params* p,
                                   void* dx_out, void* dW_out, float* dbias_out) {
  Shape sh;
  prn_status s = check_common(p, &sh);
  if (s != PRN_OK) return s;
  if (sh.ragged) return fail(PRN_ERR_INVALID_ARG, "the projection's backward takes (B, T) rows, n_seqs must be 0");
  if (p->d_in < 1) return fail(PRN_ERR_INVALID_ARG, "d_in must be >= 1");
  const int64_t M = p->B * p->T, N = sh.G * p->d_h, Kd = p->d_in;
  if (M > 0 && !dxproj) return fail(PRN_ERR_INVALID_ARG, "dxproj is NULL");
  if (dW_out && M > 0 && !x) return fail(PRN_ERR_INVALID_ARG, "x is NULL");
  if (dx_out && M > 0 && !W) return fail(PRN_ERR_INVALID_ARG, "W is NULL");
  if (misaligned(dxproj, 16) || misaligned(x, sh.elt) || misaligned(W, sh.elt) || misaligned(dx_out, sh.elt) ||
      misaligned(dW_out, sh.elt) || misaligned(dbias_out, 4))
    return fail(PRN_ERR_INVALID_ARG, "dxproj must be 16-byte aligned, the other tensors aligned to their element size");
  const PlanPb pl = plan_pb(p, sh, dx_out != nullptr, dW_out != nullptr, dbias_out != nullptr);
  if (pl.do_dw && pl.tn && misaligned(x, 16))
    return fail(PRN_ERR_INVALID_ARG, "x must be 16-byte aligned for the weight gradient when G*d_h and d_in are "
                                     "multiples of 256");
  if (pl.total > 0) {
    if (!p->workspace || p->workspace_bytes < pl.total)
      return fail(PRN_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed", p->workspace_bytes,
                  p->workspace, pl.total);
    if (reinterpret_cast<uintptr_t>(p->workspace) % kAlign)
      return fail(PRN_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  }
  // grids: transposes take (rows / 64) x (columns / 64) workgroups, the products one per 128 x 128 tile
  if (pl.Mp / 64 > kMaxGrid1D || (pl.N + 63) / 64 > kMaxGrid || (Kd + 63) / 64 > kMaxGrid ||
      ((M + 127) / 128) * ((Kd + 127) / 128) > kMaxGrid1D || pl.splits > kMaxGrid)
    return fail(PRN_ERR_UNSUPPORTED, "projection backward too large");
  hipStream_t st = static_cast<hipStream_t>(p->stream);
  const bool bf = p->dtype == PRN_BF16;
  const size_t elt = sh.elt;
  char* ws = static_cast<char*>(p->workspace);
  if (M == 0) {
    if (dW_out) {
      if (bf)
        prn::k_copy_or_zero<uint16_t><<<unsigned((N * Kd + 255) / 256), 256, 0, st>>>(
            nullptr, static_cast<uint16_t*>(dW_out), N * Kd);
      else
        prn::k_zero_f32<<<unsigned((N * Kd + 255) / 256), 256, 0, st>>>(static_cast<float*>(dW_out), N * Kd);
    }
    if (dbias_out) prn::k_zero_f32<<<unsigned((N + 255) / 256), 256, 0, st>>>(dbias_out, N);
    return launched("prn_input_proj_backward");
  }
  if (pl.do_dx) {
    // dx (M x Kd) = dxproj (M x N) W (N x Kd): W^T rows of Np elements, zero past N
    void* wt = ws + pl.wt_off;
    prn::launch_transpose(bf, W, N, Kd, Kd, wt, pl.Np, nullptr, st);
    const void* g = dxproj;
    if (pl.pad_g) {
      prn::launch_pad_rows(bf, dxproj, M, N, ws + pl.gp_off, pl.Np, st);
      g = ws + pl.gp_off;
    }
    prn::launch_proj_ld(bf, g, pl.Np * elt, wt, pl.Np * elt, dx_out, M, Kd, pl.Np, st);
  }
  float* csum = pl.do_db ? reinterpret_cast<float*>(ws + pl.csum_off) : nullptr;
  if (pl.do_dw && pl.tn) {
    // dW (N x Kd) = dxproj^T x, split-K over tokens, read along the rows of
    // both operands (no transposed copies); the same tiles take dxproj's
    // column sums per slice on the way (dbias)
    float* part = reinterpret_cast<float*>(ws + pl.part_off);
    prn::launch_proj_tn(bf, dxproj, N * elt, x, Kd * elt, part, M, N, Kd, pl.ks, pl.splits, csum, st);
    prn::launch_splitk_sum(bf, part, pl.splits, N * Kd, dW_out, st);
  } else if (pl.do_dw) {
    // dW (N x Kd) = dxproj^T x, split-K over tokens
    void* gt = ws + pl.gt_off;
    void* xt = ws + pl.xt_off;
    float* part = reinterpret_cast<float*>(ws + pl.part_off);
    prn::launch_transpose(bf, dxproj, M, N, N, gt, pl.Mp, csum, st);
    prn::launch_transpose(bf, x, M, Kd, Kd, xt, pl.Mp, nullptr, st);
    prn::launch_proj_splitk(bf, gt, pl.Mp * elt, xt, pl.Mp * elt, part, N, Kd, pl.ks, pl.splits, st);
    prn::launch_splitk_sum(bf, part, pl.splits, N * Kd, dW_out, st);
  } else if (pl.do_db && N % (16 / int64_t(elt)) == 0) {
    prn::launch_colsum64(bf, dxproj, M, N, pl.n_rt, csum, st);
  } else if (pl.do_db) {
    prn::launch_transpose(bf, dxproj, M, N, N, nullptr, pl.Mp, csum, st);
  }
  if (pl.do_db) {
    float* cslice = reinterpret_cast<float*>(ws + pl.cslice_off);
    prn::k_bw_da_partial<1><<<dim3(unsigned((N + 63) / 64), 1u, unsigned(pl.n_slices)), 256, 0, st>>>(
        csum, pl.n_cs, pl.per, N, cslice);
    prn::k_bw_da_reduce<1><<<dim3(unsigned((N + 63) / 64), 1u), 256, 0, st>>>(cslice, pl.n_slices, N, dbias_out);
  }
  return launched("prn_input_proj_backward");
}

size_t prn_head_workspace_bytes(const prn_params* p, int32_t d_head, int32_t K) {
  g_err.clear();  // a 0 result with no message means no workspace is needed
  Shape sh;
  if (check_head(p, &sh, d_head) != PRN_OK) return 0;
  if (K < 1) {
    fail(PRN_ERR_INVALID_ARG, "K must be >= 1, got %d", K);
    return 0;
  }
  return p->T > 0 ? plan_hm(p, K).total : 0;
}

}  // extern "C"

namespace {
// the head-mix Newton passes for storage dtype DT (validated by the caller)
template <int DT>
void head_newton_launch(const void* xproj_v, const prn_params* p, const float* A, const void* h0_v, int32_t K,
                        void* H_out_v, float* residual_out, const PlanHm& pl, hipStream_t st) {
  using T = typename prn::Storage<DT>::T;
  char* ws = static_cast<char*>(p->workspace);
  const size_t it = align_up(size_t(p->B) * p->T * p->d_h * sizeof(T));
  T* iter[2] = {reinterpret_cast<T*>(ws + pl.iter_off), reinterpret_cast<T*>(ws + pl.iter_off + it)};
  float* agg = reinterpret_cast<float*>(ws + pl.agg_off);
  float* carry = reinterpret_cast<float*>(ws + pl.carry_off);
  float* rpart = residual_out ? reinterpret_cast<float*>(ws + pl.rpart_off) : nullptr;
  float* gagg = reinterpret_cast<float*>(ws + pl.gagg_off);
  float* gcarry = reinterpret_cast<float*>(ws + pl.gcarry_off);
  const T* xp = static_cast<const T*>(xproj_v);
  const T* h0 = static_cast<const T*>(h0_v);
  T* Hout = static_cast<T*>(H_out_v);
  T* slast = static_cast<T*>(p->state_last_out);
  const dim3 grid(unsigned(pl.n_ch), unsigned(pl.n_heads), unsigned(p->B));
  const dim3 sgrid(unsigned(pl.n_heads), unsigned(p->B));
  const T* Hprev = nullptr;
  for (int k = 0; k < K; ++k) {
    T* Hk = (k == K - 1) ? Hout : iter[k % 2];
    prn::k_hm_pass<prn::kHmReduce, DT><<<grid, 64, 0, st>>>(xp, A, h0, Hprev, nullptr, p->T, p->d_h, pl.n_ch, agg,
                                                            rpart ? rpart + k * pl.n_wg : nullptr, nullptr, nullptr);
    if (pl.n_groups) {
      const dim3 ggrid(unsigned(pl.n_groups), unsigned(pl.n_heads), unsigned(p->B));
      prn::k_hm_group<<<ggrid, 64, 0, st>>>(agg, pl.n_ch, pl.n_groups, gagg);
      prn::k_hm_scan<<<sgrid, 64, 0, st>>>(gagg, pl.n_groups, gcarry);
      prn::k_hm_expand<<<ggrid, 64, 0, st>>>(agg, gcarry, pl.n_ch, pl.n_groups, carry);
    } else {
      prn::k_hm_scan<<<sgrid, 64, 0, st>>>(agg, pl.n_ch, carry);
    }
    prn::k_hm_pass<prn::kHmFix, DT><<<grid, 64, 0, st>>>(xp, A, h0, Hprev, carry, p->T, p->d_h, pl.n_ch, nullptr,
                                                         nullptr, Hk, k == K - 1 ? slast : nullptr);
    Hprev = Hk;
  }
  if (rpart) {
    prn::k_hm_pass<prn::kHmResidual, DT><<<grid, 64, 0, st>>>(xp, A, h0, Hout, nullptr, p->T, p->d_h, pl.n_ch,
                                                              nullptr, rpart + K * pl.n_wg, nullptr, nullptr);
    prn::k_residual_reduce<<<unsigned(K + 1), 1024, 0, st>>>(rpart, pl.n_wg, residual_out);
  }
}
}  // namespace

extern "C" {

prn_status prn_head_newton_forward(const void* xproj, const prn_params* p, const float* A, int32_t d_head,
                                   const void* h0, int32_t K, void* H_out, float* residual_out) {
  Shape sh;
  prn_status s = check_head(p, &sh, d_head);
  if (s != PRN_OK) return s;
  if (!A) return fail(PRN_ERR_INVALID_ARG, "the recurrent blocks A are NULL");
  if (misaligned(A, 4)) return fail(PRN_ERR_INVALID_ARG, "A is not 4-byte aligned");
  if (K < 1) return fail(PRN_ERR_INVALID_ARG, "K must be >= 1, got %d", K);
  if (p->T > 0 && (!xproj || !H_out)) return fail(PRN_ERR_INVALID_ARG, "xproj or H_out is NULL");
  const size_t vec = 4 * sh.elt;   // four channels per vector load
  if (misaligned(xproj, vec) || misaligned(h0, vec) || misaligned(H_out, vec))
    return fail(PRN_ERR_INVALID_ARG, "xproj, h0 and H_out must be %zu-byte aligned (4-channel vector loads)", vec);
  if (misaligned(p->state_last_out, sh.elt) || misaligned(residual_out, 4))
    return fail(PRN_ERR_INVALID_ARG, "a tensor pointer is not aligned to its element size");
  hipStream_t st = static_cast<hipStream_t>(p->stream);
  if (p->T == 0) {
    if (residual_out) prn::k_zero_f32<<<unsigned((K + 256) / 256), 256, 0, st>>>(residual_out, K + 1);
    if (p->state_last_out) {
      const int64_t n = p->B * p->d_h;
      if (p->dtype == PRN_BF16)
        prn::k_copy_or_zero<uint16_t><<<unsigned((n + 255) / 256), 256, 0, st>>>(
            static_cast<const uint16_t*>(h0), static_cast<uint16_t*>(p->state_last_out), n);
      else
        prn::k_copy_or_zero<float><<<unsigned((n + 255) / 256), 256, 0, st>>>(
            static_cast<const float*>(h0), static_cast<float*>(p->state_last_out), n);
    }
    return launched("prn_head_newton_forward");
  }
  const PlanHm pl = plan_hm(p, K);
  if (!p->workspace || p->workspace_bytes < pl.total)
    return fail(PRN_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed", p->workspace_bytes,
                p->workspace, pl.total);
  if (reinterpret_cast<uintptr_t>(p->workspace) % kAlign)
    return fail(PRN_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  if (p->dtype == PRN_BF16)
    head_newton_launch<prn::kBF16>(xproj, p, A, h0, K, H_out, residual_out, pl, st);
  else
    head_newton_launch<prn::kF32>(xproj, p, A, h0, K, H_out, residual_out, pl, st);
  return launched("prn_head_newton_forward");
}

prn_status prn_head_sequential_forward(const void* xproj, const prn_params* p, const float* A, int32_t d_head,
                                       const void* h0, void* H_out) {
  Shape sh;
  prn_status s = check_head(p, &sh, d_head);
  if (s != PRN_OK) return s;
  if (!A) return fail(PRN_ERR_INVALID_ARG, "the recurrent blocks A are NULL");
  if (misaligned(A, 4)) return fail(PRN_ERR_INVALID_ARG, "A is not 4-byte aligned");
  if (p->T > 0 && (!xproj || !H_out)) return fail(PRN_ERR_INVALID_ARG, "xproj or H_out is NULL");
  if (misaligned(xproj, sh.elt) || misaligned(h0, sh.elt) || misaligned(H_out, sh.elt) ||
      misaligned(p->state_last_out, sh.elt))
    return fail(PRN_ERR_INVALID_ARG, "a tensor pointer is not aligned to its element size");
  hipStream_t st = static_cast<hipStream_t>(p->stream);
  const dim3 sgrid(unsigned(p->d_h / prn::kHmD), unsigned(p->B));
  if (p->dtype == PRN_BF16)
    prn::k_hm_sequential<prn::kBF16><<<sgrid, 64, 0, st>>>(
        static_cast<const uint16_t*>(xproj), A, static_cast<const uint16_t*>(h0), p->T, p->d_h,
        static_cast<uint16_t*>(H_out), static_cast<uint16_t*>(p->state_last_out));
  else
    prn::k_hm_sequential<prn::kF32><<<sgrid, 64, 0, st>>>(
        static_cast<const float*>(xproj), A, static_cast<const float*>(h0), p->T, p->d_h,
        static_cast<float*>(H_out), static_cast<float*>(p->state_last_out));
  return launched("prn_head_sequential_forward");
}

}  // extern "C"
