// Deep-pipelined MFMA mainloop for bf16 operands (gfx950).
//
// Same problems, tile semantics and epilogues as gemm.hpp, different data
// path: operands move from global memory straight into LDS with
// global_load_lds_dwordx4 (lane l of an instruction writes LDS bytes
// 16l..16l+15 of a 1 KB block), through a ring of STAGES buffers.  The loads
// of k-tile kt+STAGES-1 are issued while the MFMAs of k-tile kt run, so about
// STAGES-1 k-tiles of each operand are in flight per work-group, without
// staging registers.
//
// LDS layout per stage: BF weight rows then BT token rows, 128 bytes each
// (one k-tile), as eight 16-byte chunks with chunk c of row r stored at
// position c ^ swz(r).  A DMA instruction fills 8 consecutive rows; each lane
// fetches the global chunk that belongs at its LDS slot.  The MFMA fragment
// reads (16 bytes per lane, 32 rows x 2 chunks per instruction) then hit
// distinct bank groups.
//
// Synchronisation per k-tile: s_waitcnt vmcnt(n) for the stage about to be
// read (n = DMA instructions this wave issued after it; every wave issues the
// same fixed count per stage, rows past the end are redirected to a valid
// row), then s_barrier, then the DMA for the stage STAGES-1 ahead into the
// buffer everyone finished reading in the previous iteration.
#pragma once

#include "gemm.hpp"

namespace lmoe {

typedef __attribute__((address_space(3))) void lds_void;

template <int BF_, int BT_, int WF_, int WT_, int STAGES_, int WAUX_ = 0>
struct Tile2 {
  static constexpr int BF = BF_, BT = BT_, WF = WF_, WT = WT_, STAGES = STAGES_;
  static constexpr int WAUX = WAUX_;  // cache policy of the weight loads
  static constexpr int NT = WF * WT * kWave, NW = WF * WT;
  static constexpr int FW = BF / WF, TW = BT / WT;
  static constexpr int FI = FW / 32, TI = TW / 32;
  static constexpr int QW = BF / 8, QX = BT / 8;  // DMA instructions per stage
  static constexpr int NQ = (QW + QX) / NW;       // ... per wave
  static constexpr int STAGE_BYTES = (BF + BT) * 128;
  static constexpr int LDS = STAGES * STAGE_BYTES;
  static constexpr bool kDma = true;
  static constexpr int kKind = 2;
  static_assert(FW % 64 == 0 && TW % 32 == 0, "wave tile");
  static_assert((QW + QX) % NW == 0, "DMA instructions split evenly over the waves");
  static_assert(STAGES >= 2 && NQ * (STAGES - 2) <= 63, "vmcnt range");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Dense GEMMs over many tokens / few tokens (weight streaming); experts
// holding many rows, a few dozen rows, or one or two rows (decode).
// Split-ring tile (gemm3_kernel below): weights three stages deep, tokens two.
template <int BF_, int BT_, int WF_, int WT_, int WAUX_>
struct Tile3 {
  static constexpr int BF = BF_, BT = BT_, WF = WF_, WT = WT_, WAUX = WAUX_;
  static constexpr int NT = WF * WT * kWave, NW = WF * WT;
  static constexpr int FW = BF / WF, TW = BT / WT;
  static constexpr int FI = FW / 32, TI = TW / 32;
  static constexpr int QW = BF / 8, QX = BT / 8;
  static constexpr int NQW = QW / NW, NQX = QX / NW;
  static constexpr int SW = 3, SX = 2;
  static constexpr int X_OFF = SW * BF * 128;
  static constexpr int LDS = SW * BF * 128 + SX * BT * 128;
  static constexpr bool kDma = true;
  static constexpr int kKind = 3;
  static_assert(FW % 64 == 0 && TW % 32 == 0, "wave tile");
  static_assert(QW % NW == 0 && QX % NW == 0, "DMA instructions split evenly over the waves");
  static_assert(NQW <= 63, "vmcnt range");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Tile configurations (full types, overridable at build time for tuning
// sweeps).  Tile2: one ring for both operands; Tile3: weight ring 3 deep,
// token ring 2 deep.  Expert gate/value and down GEMMs of one size class
// share the token tile (and so the expert tile list).
#ifndef LMOE_T_DENSE
#define LMOE_T_DENSE Tile3<256, 256, 4, 4, 0>
#endif
#ifndef LMOE_T_THIN
#define LMOE_T_THIN Tile2<64, 32, 1, 1, 4, 0>
#endif
#ifndef LMOE_T_EXPERT_GV
#define LMOE_T_EXPERT_GV Tile3<256, 256, 4, 4, 0>
#endif
#ifndef LMOE_T_EXPERT_DN
#define LMOE_T_EXPERT_DN Tile3<256, 256, 4, 4, 0>
#endif
#ifndef LMOE_T_MID_GV
#define LMOE_T_MID_GV Tile2<256, 64, 4, 1, 3, 0>
#endif
#ifndef LMOE_T_MID_DN
#define LMOE_T_MID_DN Tile2<256, 64, 4, 1, 3, 0>
#endif
#ifndef LMOE_T_SMALL_GV
#define LMOE_T_SMALL_GV Tile2<256, 32, 4, 1, 4, 2>
#endif
#ifndef LMOE_T_SMALL_DN
#define LMOE_T_SMALL_DN Tile2<256, 32, 4, 1, 4, 2>
#endif
typedef LMOE_T_DENSE T2Dense;
typedef LMOE_T_THIN T2Thin;
typedef LMOE_T_EXPERT_GV T2ExpertGV;
typedef LMOE_T_EXPERT_DN T2ExpertDn;
typedef LMOE_T_MID_GV T2MidGV;
typedef LMOE_T_MID_DN T2MidDn;
typedef LMOE_T_SMALL_GV T2SmallGV;
typedef LMOE_T_SMALL_DN T2SmallDn;
static_assert(T2ExpertGV::BT == T2ExpertDn::BT && T2MidGV::BT == T2MidDn::BT && T2SmallGV::BT == T2SmallDn::BT,
              "expert GEMMs of one size class share the token tile");

#ifndef LMOE_X_AUX
#define LMOE_X_AUX 0
#endif

// XOR swizzle of the 16-byte chunks of an LDS row (0: none, 1: (r >> 1) & 7,
// 2: r & 7).  DMA writes are contiguous whatever the choice; it only moves
// the fragment reads between banks.
#ifndef LMOE_SWZ
#define LMOE_SWZ 1
#endif
__device__ __forceinline__ int swz(int r) { return LMOE_SWZ == 1 ? ((r >> 1) & 7) : LMOE_SWZ == 2 ? (r & 7) : 0; }

// 16 bytes per lane from `g` into LDS at `lds` + 16 * lane (lds wave-uniform).
// A __device__ function, not a lambda: lambdas are also compiled for the host,
// where the builtin does not exist.
template <int AUX>
__device__ __forceinline__ void dma16(const char* g, char* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, AUX);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// One k-tile (64 bf16 of K) of a wave's FI x TI block of 32x32 MFMAs, from
// the swizzled LDS stage (W rows at sW, token rows at sX).  Fragments are
// double-buffered across the four 16-wide k-steps so the LDS reads of step
// ks+1 overlap the MFMAs of step ks; no per-block predicates, so the MFMA
// sequence is straight-line code.
template <int FI, int TI>
__device__ __forceinline__ void mma_ktile(f32x16 (&acc)[FI][TI], const char* sW, const char* sX, int wf0, int wt0,
                                          int lane) {
  const int lr = lane & 31;
  const int sw = swz(lr);  // fragment row offsets are multiples of 32
  const char* pw = sW + (wf0 + lr) * 128;
  const char* px = sX + (wt0 + lr) * 128;
  bf16x8 a[2][FI], b[2][TI];
  auto load = [&](int ks, int buf) {
    const int ch = ((2 * ks + (lane >> 5)) ^ sw) << 4;
#pragma unroll
    for (int i = 0; i < FI; ++i) a[buf][i] = *reinterpret_cast<const bf16x8*>(pw + i * 32 * 128 + ch);
#pragma unroll
    for (int j = 0; j < TI; ++j) b[buf][j] = *reinterpret_cast<const bf16x8*>(px + j * 32 * 128 + ch);
  };
  load(0, 0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (ks + 1 < 4) load(ks + 1, (ks + 1) & 1);
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < TI; ++j) acc[i][j] = mfma32(a[ks & 1][i], b[ks & 1][j], acc[i][j]);
  }
}

template <class Cfg, class Prob>
__global__ __launch_bounds__(Cfg::NT) void gemm2_kernel(const Prob p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  typename Prob::State st;
  if (!p.setup(blockIdx.x, st)) return;

  constexpr int FI = Cfg::FI, TI = Cfg::TI, NQ = Cfg::NQ, S = Cfg::STAGES, NW = Cfg::NW;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf0 = (wid % Cfg::WF) * Cfg::FW;
  const int wt0 = (wid / Cfg::WF) * Cfg::TW;

  // a wave whose token or feature slab lies wholly past the end skips its MFMAs
  const bool active = wt0 < p.tokens_valid(st) && wf0 < p.feats_valid(st);

  f32x16 acc[FI][TI];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < TI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // k-tiles over all K segments
  const int nks = p.num_ksegs();
  int nkt = 0;
  for (int s = 0; s < nks; ++s) nkt += p.seg_ktiles(s);

  // ---- issue side: segment cursor and one source pointer per DMA slot ----
  int is = 0, ik = 0;
  while (is < nks && p.seg_ktiles(is) == 0) ++is;
  const char* src[NQ];
  auto set_src = [&](int s) {
    const float* dummy = nullptr;
    const char* w0 = p.w_row(st, s, 0, &dummy);
    const char* x0 = p.x_row(st, s, 0);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int q = wid + NW * i;  // uniform per wave
      const char* rp;
      int row;
      if (q < Cfg::QW) {
        row = q * 8 + (lane >> 3);
        rp = p.w_row(st, s, row, &dummy);
        if (!rp) rp = w0;
      } else {
        row = (q - Cfg::QW) * 8 + (lane >> 3);
        rp = p.x_row(st, s, row);
        if (!rp) rp = x0;
      }
      src[i] = rp + (((lane & 7) ^ swz(row)) << 4);
    }
  };
  if (is < nks) set_src(is);
  auto issue = [&](int buf) {
    char* base = smem + buf * Cfg::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int q = wid + NW * i;
      if (q < Cfg::QW) dma16<Cfg::WAUX>(src[i] + (int64_t)ik * 128, base + q * 1024);
      else dma16<LMOE_X_AUX>(src[i] + (int64_t)ik * 128, base + q * 1024);
    }
    if (++ik == p.seg_ktiles(is)) {
      ik = 0;
      do { ++is; } while (is < nks && p.seg_ktiles(is) == 0);
      if (is < nks) set_src(is);
    }
  };

  // ---- compute side ----
  auto compute = [&](int buf) {
    const char* sW = smem + buf * Cfg::STAGE_BYTES;
    if (active) mma_ktile<FI, TI>(acc, sW, sW + Cfg::BF * 128, wf0, wt0, lane);
  };

#pragma unroll
  for (int st = 0; st < S - 1; ++st)
    if (st < nkt) issue(st);
  for (int kt = 0; kt < nkt; ++kt) {
    // stages issued after kt: min(S-2, nkt-1-kt), NQ instructions each
    const int after = min(S - 2, nkt - 1 - kt);
    if constexpr (S >= 4) {
      if (after >= 2) wait_vmcnt_barrier<2 * NQ>();
      else if (after == 1) wait_vmcnt_barrier<NQ>();
      else wait_vmcnt_barrier<0>();
    } else {
      if (after >= 1) wait_vmcnt_barrier<NQ * (S - 2)>();
      else wait_vmcnt_barrier<0>();
    }
    if (kt + S - 1 < nkt) issue((kt + S - 1) % S);
    compute(kt % S);
  }
  p.epilogue(st, acc, wf0, wt0, lane);
}

// ---------------------------------------------------------------------------
// Split rings: the weight operand (streamed from HBM) gets three LDS stages
// and runs two k-tiles ahead; the token operand (re-read by neighbouring
// tiles, mostly from L2) gets two stages and runs one k-tile ahead.  Issue
// order: X(0) W(0) W(1) before the loop, then X(kt+1) W(kt+2) in iteration
// kt.  At the top of iteration kt the only DMA issued after the newest
// operand that iteration kt needs (X(kt), or W(0) when kt = 0) is W(kt+1), so
// the wait is vmcnt(NQW) while W(kt+1) exists and vmcnt(0) after.
// ---------------------------------------------------------------------------
template <class Cfg, class Prob>
__global__ __launch_bounds__(Cfg::NT) void gemm3_kernel(const Prob p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  typename Prob::State st;
  if (!p.setup(blockIdx.x, st)) return;

  constexpr int FI = Cfg::FI, TI = Cfg::TI, NQW = Cfg::NQW, NQX = Cfg::NQX, NW = Cfg::NW;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf0 = (wid % Cfg::WF) * Cfg::FW;
  const int wt0 = (wid / Cfg::WF) * Cfg::TW;

  // a wave whose token or feature slab lies wholly past the end skips its MFMAs
  const bool active = wt0 < p.tokens_valid(st) && wf0 < p.feats_valid(st);

  f32x16 acc[FI][TI];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < TI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nks = p.num_ksegs();
  int nkt = 0;
  for (int s = 0; s < nks; ++s) nkt += p.seg_ktiles(s);

  // issue cursors (segment, k-tile within it) and source pointers per operand
  int wsg = 0, wk = 0, xsg = 0, xk = 0;
  while (wsg < nks && p.seg_ktiles(wsg) == 0) ++wsg;
  xsg = wsg;
  const char* srcW[NQW];
  const char* srcX[NQX];
  auto set_w = [&](int s) {
    const float* dummy = nullptr;
    const char* w0 = p.w_row(st, s, 0, &dummy);
#pragma unroll
    for (int i = 0; i < NQW; ++i) {
      const int row = (wid + NW * i) * 8 + (lane >> 3);
      const char* rp = p.w_row(st, s, row, &dummy);
      srcW[i] = (rp ? rp : w0) + (((lane & 7) ^ swz(row)) << 4);
    }
  };
  auto set_x = [&](int s) {
    const char* x0 = p.x_row(st, s, 0);
#pragma unroll
    for (int i = 0; i < NQX; ++i) {
      const int row = (wid + NW * i) * 8 + (lane >> 3);
      const char* rp = p.x_row(st, s, row);
      srcX[i] = (rp ? rp : x0) + (((lane & 7) ^ swz(row)) << 4);
    }
  };
  if (wsg < nks) {
    set_w(wsg);
    set_x(xsg);
  }
  auto issue_w = [&](int buf) {
    char* base = smem + buf * Cfg::BF * 128;
#pragma unroll
    for (int i = 0; i < NQW; ++i) dma16<Cfg::WAUX>(srcW[i] + (int64_t)wk * 128, base + (wid + NW * i) * 1024);
    if (++wk == p.seg_ktiles(wsg)) {
      wk = 0;
      do { ++wsg; } while (wsg < nks && p.seg_ktiles(wsg) == 0);
      if (wsg < nks) set_w(wsg);
    }
  };
  auto issue_x = [&](int buf) {
    char* base = smem + Cfg::X_OFF + buf * Cfg::BT * 128;
#pragma unroll
    for (int i = 0; i < NQX; ++i) dma16<LMOE_X_AUX>(srcX[i] + (int64_t)xk * 128, base + (wid + NW * i) * 1024);
    if (++xk == p.seg_ktiles(xsg)) {
      xk = 0;
      do { ++xsg; } while (xsg < nks && p.seg_ktiles(xsg) == 0);
      if (xsg < nks) set_x(xsg);
    }
  };

  auto compute = [&](int wbuf, int xbuf) {
    if (active)
      mma_ktile<FI, TI>(acc, smem + wbuf * Cfg::BF * 128, smem + Cfg::X_OFF + xbuf * Cfg::BT * 128, wf0, wt0, lane);
  };

  if (nkt > 0) {
    issue_x(0);
    issue_w(0);
    if (nkt > 1) issue_w(1);
  }
  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) wait_vmcnt_barrier<NQW>();
    else wait_vmcnt_barrier<0>();
    if (kt + 1 < nkt) issue_x((kt + 1) & 1);
    if (kt + 2 < nkt) issue_w((kt + 2) % 3);
    compute(kt % 3, kt & 1);
  }
  p.epilogue(st, acc, wf0, wt0, lane);
}

}  // namespace lmoe
