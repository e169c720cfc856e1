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

template <int BF_, int BT_, int WF_, int WT_, int STAGES_>
struct Tile2 {
  static constexpr int BF = BF_, BT = BT_, WF = WF_, WT = WT_, STAGES = STAGES_;
  static constexpr int NT = WF * WT * kWave, NW = WF * WT;
  static constexpr int FW = BF / WF, TW = BT / WT;
  static constexpr int FI = FW / 32, TI = TW / 32;
  static constexpr int QW = BF / 8, QX = BT / 8;  // DMA instructions per stage
  static constexpr int NQ = (QW + QX) / NW;       // ... per wave
  static constexpr int STAGE_BYTES = (BF + BT) * 128;
  static constexpr int LDS = STAGES * STAGE_BYTES;
  static constexpr bool kDma = true;
  static_assert(FW % 64 == 0 && TW % 32 == 0, "wave tile");
  static_assert((QW + QX) % NW == 0, "DMA instructions split evenly over the waves");
  static_assert(STAGES >= 2 && NQ * (STAGES - 2) <= 63, "vmcnt range");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Dense GEMMs over many tokens / few tokens (weight streaming); experts
// holding many rows, a few dozen rows, or one or two rows (decode).
typedef Tile2<256, 128, 2, 2, 3> T2Dense;
typedef Tile2<64, 32, 1, 1, 4> T2Thin;
typedef Tile2<128, 256, 2, 2, 3> T2Expert;
typedef Tile2<256, 64, 4, 1, 3> T2Mid;
typedef Tile2<256, 32, 4, 1, 4> T2Small;

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// 16 bytes per lane from `g` into LDS at `lds` + 16 * lane (lds wave-uniform).
// A __device__ function, not a lambda: lambdas are also compiled for the host,
// where the builtin does not exist.
__device__ __forceinline__ void dma16(const char* g, char* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <class Cfg, class Prob>
__global__ __launch_bounds__(Cfg::NT) void gemm2_kernel(const Prob p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  typename Prob::State st;
  if (!p.setup(blockIdx.x, st)) return;

  constexpr int FI = Cfg::FI, TI = Cfg::TI, NQ = Cfg::NQ, S = Cfg::STAGES, NW = Cfg::NW;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wf0 = (wid % Cfg::WF) * Cfg::FW;
  const int wt0 = (wid / Cfg::WF) * Cfg::TW;

  const int tvalid = p.tokens_valid(st);
  const int fvalid = p.feats_valid(st);
  bool tok[TI], fea[FI];
#pragma unroll
  for (int i = 0; i < TI; ++i) tok[i] = wt0 + i * 32 < tvalid;
#pragma unroll
  for (int i = 0; i < FI; ++i) fea[i] = wf0 + i * 32 < fvalid;

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
      dma16(src[i] + (int64_t)ik * 128, base + q * 1024);
    }
    if (++ik == p.seg_ktiles(is)) {
      ik = 0;
      do { ++is; } while (is < nks && p.seg_ktiles(is) == 0);
      if (is < nks) set_src(is);
    }
  };

  // ---- compute side ----
  const int lr = lane & 31;
  const int sw = swz(lr);  // row offsets of fragments are multiples of 32
  auto compute = [&](int buf) {
    const char* sW = smem + buf * Cfg::STAGE_BYTES;
    const char* sX = sW + Cfg::BF * 128;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ch = ((2 * ks + (lane >> 5)) ^ sw) << 4;
      bf16x8 a[FI], b[TI];
#pragma unroll
      for (int i = 0; i < FI; ++i) a[i] = *reinterpret_cast<const bf16x8*>(sW + (wf0 + i * 32 + lr) * 128 + ch);
#pragma unroll
      for (int j = 0; j < TI; ++j) b[j] = *reinterpret_cast<const bf16x8*>(sX + (wt0 + j * 32 + lr) * 128 + ch);
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < TI; ++j)
          if (fea[i] && tok[j]) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
    }
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

}  // namespace lmoe
