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
  static constexpr int XF8 = 0;  // tokens are never e4m3 here
  static_assert(FW % 64 == 0 && TW % 32 == 0, "wave tile");
  static_assert((QW + QX) % NW == 0, "DMA instructions split evenly over the waves");
  static_assert(STAGES >= 2 && NQ * (STAGES - 2) <= 63, "vmcnt range");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Dense GEMMs over many tokens / few tokens (weight streaming); experts
// holding many rows, a few dozen rows, or one or two rows (decode).
// Split-ring tile (gemm3_kernel below): weights three stages deep, tokens two.
template <int BF_, int BT_, int WF_, int WT_, int WAUX_, int PERSIST_ = 0, int WF8_ = 0, int SW_ = 3, int XF8_ = 0,
          int WTR_ = 0>
struct Tile3 {
  static constexpr int BF = BF_, BT = BT_, WF = WF_, WT = WT_, WAUX = WAUX_;
  // WTR: the weights are stored transposed ([K, F] per matrix, features
  // contiguous, as the backward's data gradients read the forward's
  // weights).  A stage then holds the k-tile's 64 k-rows of the tile's 256
  // features (512 bytes each, two per DMA instruction), and the MFMA's weight
  // fragments come out of it through transposing LDS reads.
  static constexpr int WTR = WTR_;
  // PERSIST: a grid of resident work-groups walks the tile list with one
  // continuous DMA pipeline (gemm3p_kernel) instead of one tile per group
  static constexpr int PERSIST = PERSIST_;
  // WF8: e4m3 weights staged as such (64 bytes per row per 64-column k-tile)
  // and widened to bf16 with their block scale at the fragment load
  static constexpr int WF8 = WF8_;
  // XF8: token rows staged as e4m3 codes as well (W8A8), multiplied by
  // e4m3 x e4m3 MFMAs; the fp32 scale of each row's 128-column block rides
  // with the token tile into a pair of LDS scale slots
  static constexpr int XF8 = XF8_;
  static constexpr int SW = SW_, SX = 2;  // weight / token ring depths
  static constexpr int RBW = WF8 ? 64 : 128;              // weight row bytes per k-tile
  static constexpr int RPIW = 1024 / RBW;                 // weight rows per DMA instruction
  static constexpr int RBX = XF8 ? 64 : 128;              // token row bytes per k-tile
  static constexpr int RPIX = 1024 / RBX;                 // token rows per DMA instruction
  static constexpr int NT = WF * WT * kWave, NW = WF * WT;
  static constexpr int FW = BF / WF, TW = BT / WT;
  static constexpr int FI = FW / 32, TI = TW / 32;
  static constexpr int QW = BF / RPIW, QX = BT / RPIX;
  static constexpr int NQW = QW / NW, NQX = QX / NW;
  static constexpr int WSTAGE = BF * RBW, XSTAGE = BT * RBX;
  static constexpr int X_OFF = SW * WSTAGE;
  static constexpr int SC_OFF = X_OFF + SX * XSTAGE;
  static constexpr int LDS = SC_OFF + (XF8 ? SX * BT * 4 : 0);
  static constexpr bool kDma = true;
  static constexpr int kKind = PERSIST ? 4 : 3;
  static_assert(FW % 64 == 0 && TW % 32 == 0, "wave tile");
  static_assert(QW % NW == 0 && QX % NW == 0, "DMA instructions split evenly over the waves");
  static_assert(NQW <= 63, "vmcnt range");
  static_assert(SW >= 3, "the weight ring runs at least two k-tiles ahead");
  static_assert(PERSIST || (!WF8 && SW == 3), "one-tile-per-group kernel: bf16 weights, three stages");
  static_assert(!XF8 || (WF8 && PERSIST), "e4m3 tokens go with e4m3 weights in the persistent kernel");
  static_assert(!XF8 || (BT % 64 == 0 && BT / 64 <= NW), "one 4-byte scale DMA per 64 token rows");
  static_assert(!WTR || (PERSIST && !WF8 && !XF8 && BF == 256), "transposed weights: bf16, 256 features");
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
#define LMOE_T_EXPERT_GV Tile3<256, 256, 4, 4, 0, 1>
#endif
#ifndef LMOE_T_EXPERT_DN
#define LMOE_T_EXPERT_DN Tile3<256, 256, 4, 4, 0, 1>
#endif
// e4m3 expert weights with bf16 activations (many rows per expert): half the
// weight bytes per stage, so a five-deep weight ring fits beside the tokens.
#ifndef LMOE_T_EXPERT_GV_F8
#define LMOE_T_EXPERT_GV_F8 Tile3<256, 256, 4, 4, 0, 1, 1, 5>
#endif
#ifndef LMOE_T_EXPERT_DN_F8
#define LMOE_T_EXPERT_DN_F8 Tile3<256, 256, 4, 4, 0, 1, 1, 5>
#endif
// W8A8 experts: 64-byte rows on both sides (64 columns per k-tile), so a
// seven-deep weight ring fits beside the token ring and its scale slots.
#ifndef LMOE_T_EXPERT_GV_A8
#define LMOE_T_EXPERT_GV_A8 Tile3<256, 256, 4, 4, 0, 1, 1, 7, 1>
#endif
#ifndef LMOE_T_EXPERT_DN_A8
#define LMOE_T_EXPERT_DN_A8 Tile3<256, 256, 4, 4, 0, 1, 1, 7, 1>
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
typedef LMOE_T_EXPERT_GV_F8 T2ExpertGVF8;
typedef LMOE_T_EXPERT_DN_F8 T2ExpertDnF8;
typedef LMOE_T_EXPERT_GV_A8 T2ExpertGVA8;
typedef LMOE_T_EXPERT_DN_A8 T2ExpertDnA8;
typedef LMOE_T_MID_GV T2MidGV;
typedef LMOE_T_MID_DN T2MidDn;
typedef LMOE_T_SMALL_GV T2SmallGV;
typedef LMOE_T_SMALL_DN T2SmallDn;
static_assert(T2ExpertGV::BT == T2ExpertDn::BT && T2MidGV::BT == T2MidDn::BT && T2SmallGV::BT == T2SmallDn::BT &&
                  T2ExpertGVF8::BT == T2ExpertDnF8::BT && T2ExpertGVF8::WF8 && T2ExpertDnF8::WF8 &&
                  T2ExpertGVA8::BT == T2ExpertDnA8::BT && T2ExpertGVA8::XF8 && T2ExpertDnA8::XF8,
              "expert GEMMs of one size class share the token tile");
static_assert(T2ExpertGV::BF == kPackRows && T2ExpertDn::BF == kPackRows && T2MidGV::BF == kPackRows &&
                  T2MidDn::BF == kPackRows && T2SmallGV::BF == kPackRows && T2SmallDn::BF == kPackRows,
              "every bf16 expert tile reads whole packed weight blocks");

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
// 64-byte rows (e4m3 weights, 4 chunks): chunk c of row r at position
// c ^ ((r >> 2) & 3), so 16 consecutive rows of one chunk hit distinct banks.
__device__ __forceinline__ int swz64(int r) { return (r >> 2) & 3; }

// 16 bytes per lane from `g` into LDS at `lds` + 16 * lane (lds wave-uniform).
// A __device__ function, not a lambda: lambdas are also compiled for the host,
// where the builtin does not exist.
//
// With the default cache policy the instruction is written out (M0 = the LDS
// address) instead of issued through the builtin: after a builtin LDS DMA the
// compiler puts an s_waitcnt vmcnt(0) in front of the next transposed
// (ds_read_b64_tr_b16) or e4m3 LDS read it cannot tell apart from the DMA's
// target, which drains the whole ring once per k-tile.  The kernels' own
// s_waitcnt + s_barrier at the top of each k-tile order every LDS read after
// the DMA that fills its stage, so no compiler wait is needed.
__device__ __forceinline__ uint32_t lds_u32(const char* lds) {
  return (uint32_t)(uintptr_t)(lds_void*)lds;
}
template <int AUX>
__device__ __forceinline__ void dma16(const char* g, char* lds) {
  if constexpr (AUX == 0) {
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds_u32(lds)) : "memory");
  } else {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, AUX);
  }
}

// Packs the routed expert weights into 32 KB blocks, each the LDS image of
// one 256-row weight tile at one 64-column k-tile (layout at
// lmoe_pack_experts).  One work-group per block; thread t writes chunks t,
// t + 256, ... (coalesced 16-byte stores), and the 8 chunks of a row come
// from one 128-byte run of the source row.  Rows past I (gate/value) or L
// (out) are zero.
__global__ __launch_bounds__(256) void pack_experts_kernel(const char* wg, const char* wv, const char* wo, char* dst,
                                                          int E, int I, int L) {
  const int64_t nft_gv = (I + 127) / 128, nkt_gv = L / 64;
  const int64_t nft_dn = (L + 255) / 256, nkt_dn = I / 64;
  const int64_t gv_blocks = (int64_t)E * nft_gv * nkt_gv;
  const int64_t b = blockIdx.x;
  const bool gv = b < gv_blocks;
  int64_t rem = gv ? b : b - gv_blocks;
  const int64_t nkt = gv ? nkt_gv : nkt_dn, nft = gv ? nft_gv : nft_dn;
  const int kt = (int)(rem % nkt);
  rem /= nkt;
  const int ft = (int)(rem % nft);
  const int64_t e = rem / nft;
  char* out = dst + b * kPackBlock;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = threadIdx.x + 256 * j;  // chunk 0 .. 2047 of the block
    const int r = c >> 3, ch = (c & 7) ^ swz(r);
    const char* src = nullptr;
    if (gv) {
      const int m = r & 63;
      const int u = ft * 128 + (r >> 6) * 32 + (m & 31);
      if (u < I) src = (m >= 32 ? wv : wg) + ((e * I + u) * L + kt * 64 + ch * 8) * 2;
    } else {
      const int f = ft * 256 + r;
      if (f < L) src = wo + ((e * L + f) * I + kt * 64 + ch * 8) * 2;
    }
    uint4 v = {0u, 0u, 0u, 0u};
    if (src) v = *reinterpret_cast<const uint4*>(src);
    *reinterpret_cast<uint4*>(out + c * 16) = v;
  }
}

// 4 bytes per lane from `g` into LDS at `lds` + 4 * lane (lds wave-uniform);
// written out like dma16.
__device__ __forceinline__ void dma4(const void* g, char* lds) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds_u32(lds)) : "memory");
}

// Stacked e4m3 matrices [n, R, C] with one fp32 scale per 128x128 block
// ([n, R/128, C/128]) -> bf16 of code * scale, rounded exactly as the
// register-staged GEMMs widen codes (widen_e4m3).  8 codes per thread.
__global__ __launch_bounds__(256) void dequant_blocks_kernel(const char* q, const float* s, int64_t n, int R, int C,
                                                             char* out) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= n * R * (int64_t)(C / 8)) return;
  const int64_t e = g * 8;
  const int64_t row = e / C;
  const int c = (int)(e - row * C);
  const int64_t m = row / R;
  const int r = (int)(row - m * R);
  const float sc = s[(m * (R / 128) + r / 128) * (C / 128) + c / 128];
  *reinterpret_cast<uint4*>(out + e * 2) = widen_e4m3(*reinterpret_cast<const uint2*>(q + e), sc);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// One k-tile (64 bf16 of K) of a wave's FI x TI block of 32x32 MFMAs, from
// the swizzled LDS stage (W rows at sW, token rows at sX).  Fragments are
// double-buffered across the four 16-wide k-steps so the LDS reads of step
// ks+1 overlap the MFMAs of step ks.  Token blocks j >= tiv (rows all past
// the valid ones) are skipped, loads and MFMAs alike; the test is uniform
// across the wave.  Dense GEMMs, whose extra token rows are never stored,
// use the unconditional mma_ktile_full below instead.
template <int FI, int TI, bool DB = true>
__device__ __forceinline__ void mma_ktile(f32x16 (&acc)[FI][TI], const char* sW, const char* sX, int wf0, int wt0,
                                          int lane, int tiv) {
  const int lr = lane & 31;
  const int sw = swz(lr);  // fragment row offsets are multiples of 32
  const char* pw = sW + (wf0 + lr) * 128;
  const char* px = sX + (wt0 + lr) * 128;
  constexpr int NB = DB ? 2 : 1;
  bf16x8 a[NB][FI], b[NB][TI];
  auto load = [&](int ks, int buf) __attribute__((always_inline)) {
    const int ch = ((2 * ks + (lane >> 5)) ^ sw) << 4;
#pragma unroll
    for (int i = 0; i < FI; ++i) a[buf][i] = *reinterpret_cast<const bf16x8*>(pw + i * 32 * 128 + ch);
#pragma unroll
    for (int j = 0; j < TI; ++j)
      if (j < tiv) b[buf][j] = *reinterpret_cast<const bf16x8*>(px + j * 32 * 128 + ch);
  };
  if (DB) load(0, 0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int cur = DB ? (ks & 1) : 0;
    if (DB) {
      if (ks + 1 < 4) load(ks + 1, (ks + 1) & 1);
    } else {
      load(ks, 0);
    }
#pragma unroll
    for (int j = 0; j < TI; ++j)
      if (j < tiv) {
#pragma unroll
        for (int i = 0; i < FI; ++i) acc[i][j] = mfma32(a[cur][i], b[cur][j], acc[i][j]);
      }
  }
}

// Problems whose token rows past the valid ones may be multiplied like the
// rest declare kDenseRows (dense GEMMs: whatever such LDS rows hold only
// reaches accumulator columns of tokens the epilogue never stores); their
// k-tiles take the branch-free fragment path.
template <class P, class = void>
struct dense_rows : std::false_type {};
template <class P>
struct dense_rows<P, std::void_t<decltype(P::kDenseRows)>> : std::bool_constant<P::kDenseRows> {};

// mma_ktile for a wave that multiplies all its token blocks: no conditional
// loads or MFMAs, and the fragments of k-step ks+1 are read while the MFMAs
// of k-step ks run (3-5% faster on the 256x256 dense GEMMs at K3 shape than
// the guarded loop, bitwise the same sums).
template <int FI, int TI>
__device__ __forceinline__ void mma_ktile_full(f32x16 (&acc)[FI][TI], const char* sW, const char* sX, int wf0, int wt0,
                                               int lane) {
  const int lr = lane & 31;
  const int sw = swz(lr);  // fragment row offsets are multiples of 32
  const char* pw = sW + (wf0 + lr) * 128;
  const char* px = sX + (wt0 + lr) * 128;
  bf16x8 a[2][FI], b[2][TI];
  auto load = [&](int ks, int buf) __attribute__((always_inline)) {
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
    for (int j = 0; j < TI; ++j)
#pragma unroll
      for (int i = 0; i < FI; ++i) acc[i][j] = mfma32(a[ks & 1][i], b[ks & 1][j], acc[i][j]);
    // scheduling order within the k-step: the next k-step's LDS reads, then
    // this k-step's MFMAs (the reads land under them: two fragment buffers);
    // nothing moves across k-steps, which keeps register use at two buffers
    if (ks + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, FI + TI, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, FI * TI, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// As mma_ktile, with the weight operand as e4m3 codes (64-byte rows): lane l
// reads the 8 codes of k-step ks, half l / 32 of chunk ks, and widens them to
// bf16 unscaled (exact: every e4m3 value is a bf16 value); the caller applies
// the block scales to the accumulators once per 128 columns.  Raw codes are
// double-buffered across k-steps.
__device__ __forceinline__ bf16x8 widen_e4m3_exact(uint2 q) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)q.x, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)q.x, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)q.y, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)q.y, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
template <int FI, int TI>
__device__ __forceinline__ void mma_ktile_f8(f32x16 (&acc)[FI][TI], const char* sW, const char* sX, int wf0, int wt0,
                                             int lane, int tiv) {
  const int lr = lane & 31;
  const int sw = swz(lr), sw64 = swz64(lr);  // fragment row offsets are multiples of 32
  const char* pw = sW + (wf0 + lr) * 64 + ((lane >> 5) << 3);
  const char* px = sX + (wt0 + lr) * 128;
  uint2 q[2][FI];
  auto loadw = [&](int ks, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FI; ++i) q[buf][i] = *reinterpret_cast<const uint2*>(pw + i * 32 * 64 + ((ks ^ sw64) << 4));
  };
  loadw(0, 0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (ks + 1 < 4) loadw(ks + 1, (ks + 1) & 1);
    const int ch = ((2 * ks + (lane >> 5)) ^ sw) << 4;
    bf16x8 b[TI];
#pragma unroll
    for (int j = 0; j < TI; ++j)
      if (j < tiv) b[j] = *reinterpret_cast<const bf16x8*>(px + j * 32 * 128 + ch);
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const bf16x8 a = widen_e4m3_exact(q[ks & 1][i]);
#pragma unroll
      for (int j = 0; j < TI; ++j)
        if (j < tiv) acc[i][j] = mfma32(a, b[j], acc[i][j]);
    }
  }
}

// One k-tile (64 columns) with both operands as e4m3 codes in swizzled
// 64-byte rows: one 32x32x64 MFMA per block.  Lane l supplies chunks
// 2 (l / 32) and 2 (l / 32) + 1 of row l % 32 of each operand; the two
// operands use the same lane-to-column map, so every code meets its partner.
template <int FI, int TI>
__device__ __forceinline__ void mma_ktile_a8(f32x16 (&acc)[FI][TI], const char* sW, const char* sX, int wf0, int wt0,
                                             int lane, int tiv) {
  const int lr = lane & 31, h = lane >> 5;
  const int s = swz64(lr);  // fragment row offsets are multiples of 32
  const int c0 = ((2 * h) ^ s) << 4, c1 = ((2 * h + 1) ^ s) << 4;
  const char* pw = sW + (wf0 + lr) * 64;
  const char* px = sX + (wt0 + lr) * 64;
  auto frag = [&](const char* p) __attribute__((always_inline)) {
    const i32x4 u = *reinterpret_cast<const i32x4*>(p + c0);
    const i32x4 v = *reinterpret_cast<const i32x4*>(p + c1);
    return i32x8{u[0], u[1], u[2], u[3], v[0], v[1], v[2], v[3]};
  };
  i32x8 a[FI];
#pragma unroll
  for (int i = 0; i < FI; ++i) a[i] = frag(pw + i * 32 * 64);
#pragma unroll
  for (int j = 0; j < TI; ++j)
    if (j < tiv) {
      const i32x8 b = frag(px + j * 32 * 64);
#pragma unroll
      for (int i = 0; i < FI; ++i) acc[i][j] = mfma8(a[i], b, acc[i][j]);
    }
}

// Transposed weight stage (Tile3 WTR): k-row kr (0..63) of the tile's 256
// features at kr * 512 bytes, its 16-byte chunk c stored at position
// c ^ ((kr & 3) << 2), so the four k-rows one transposing read spans fall in
// different bank windows.
__device__ __forceinline__ int wtr_off(int kr, int f) {
  return kr * 512 + ((((f >> 3) ^ ((kr & 3) << 2))) << 4) + (f & 7) * 2;
}

// As mma_ktile, with the weight fragments (32 features x 16 k per MFMA)
// read from a transposed stage with ds_read_b64_tr_b16: within each 16-lane
// group, lane i receives element i % 4 of the 4-element loads of lanes
// 4 j + i / 4 (j = 0..3).  So lane q of group G loads k-row
// 8 (G / 2) + q / 4 of the k-step at features r0 + 16 (G % 2) + 4 (q % 4)
// .. + 3, and a second load 4 k-rows further gives its other 4 k: lane l
// ends up with the 8 consecutive k (8 (l / 32) .. + 7) of feature
// r0 + l % 32, the fragment mma_ktile reads from a k-contiguous stage.
typedef short i16x4 __attribute__((ext_vector_type(4)));
template <int FI, int TI>
__device__ __forceinline__ void mma_ktile_wt(f32x16 (&acc)[FI][TI], const char* sW, const char* sX, int wf0, int wt0,
                                             int lane, int tiv) {
  const int lr = lane & 31;
  const int sw = swz(lr);  // token fragment row offsets are multiples of 32
  const char* px = sX + (wt0 + lr) * 128;
  const int G = lane >> 4, q = lane & 15;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int kr = ks * 16 + 8 * (G >> 1) + (q >> 2);
    bf16x8 a[FI];
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const char* pa = sW + wtr_off(kr, wf0 + i * 32 + 16 * (G & 1) + 4 * (q & 3));
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa + 4 * 512));
      const short v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      a[i] = *reinterpret_cast<const bf16x8*>(v);
    }
    const int ch = ((2 * ks + (lane >> 5)) ^ sw) << 4;
#pragma unroll
    for (int j = 0; j < TI; ++j)
      if (j < tiv) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(px + j * 32 * 128 + ch);
#pragma unroll
        for (int i = 0; i < FI; ++i) acc[i][j] = mfma32(a[i], b, acc[i][j]);
      }
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

  // token blocks of this wave holding valid rows; a wave with none, or whose
  // feature slab lies wholly past the end, skips its MFMAs
  const int tiv = min(TI, max(0, (p.tokens_valid(st) - wt0 + 31) >> 5));
  const bool active = tiv > 0 && wf0 < p.feats_valid(st);

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
  const char* wblk = p.w_block(st);
  const int64_t wstep = wblk ? kPackBlock : 128;
  auto set_src = [&](int s) __attribute__((always_inline)) {
    const float* dummy = nullptr;
    const char* w0 = p.w_row(st, s, 0, &dummy);
    const char* x0 = p.x_row(st, s, 0);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int q = wid + NW * i;  // uniform per wave
      int row;
      if (q < Cfg::QW) {
        row = q * 8 + (lane >> 3);
        if (wblk) {
          src[i] = wblk + q * 1024 + lane * 16;
        } else {
          const char* rp = p.w_row(st, s, row, &dummy);
          src[i] = (rp ? rp : w0) + (((lane & 7) ^ swz(row)) << 4);
        }
      } else {
        row = (q - Cfg::QW) * 8 + (lane >> 3);
        const char* rp = p.x_row(st, s, row);
        src[i] = (rp ? rp : x0) + (((lane & 7) ^ swz(row)) << 4);
      }
    }
  };
  if (is < nks) set_src(is);
  auto issue = [&](int buf) __attribute__((always_inline)) {
    char* base = smem + buf * Cfg::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int q = wid + NW * i;
      if (q < Cfg::QW) dma16<Cfg::WAUX>(src[i] + ik * wstep, base + q * 1024);
      else dma16<LMOE_X_AUX>(src[i] + (int64_t)ik * 128, base + q * 1024);
    }
    if (++ik == p.seg_ktiles(is)) {
      ik = 0;
      do { ++is; } while (is < nks && p.seg_ktiles(is) == 0);
      if (is < nks) set_src(is);
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
    const char* sW = smem + (kt % S) * Cfg::STAGE_BYTES;
    if (active) {
      if constexpr (dense_rows<Prob>::value) mma_ktile_full<FI, TI>(acc, sW, sW + Cfg::BF * 128, wf0, wt0, lane);
      else mma_ktile<FI, TI>(acc, sW, sW + Cfg::BF * 128, wf0, wt0, lane, tiv);
    }
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
// the wait is vmcnt(NQW) while W(kt+1) exists and vmcnt(0) after.  Token DMA
// instructions whose 8 rows all lie past the valid ones are not issued: their
// LDS rows feed only token blocks no wave computes, and since the weight
// instructions come last in every iteration the waits do not depend on how
// many token instructions went out.
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

  const int xrows = p.tokens_valid(st);
  const int tiv = min(TI, max(0, (xrows - wt0 + 31) >> 5));
  const bool active = tiv > 0 && wf0 < p.feats_valid(st);

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
  bool xon[NQX];
#pragma unroll
  for (int i = 0; i < NQX; ++i) xon[i] = (wid + NW * i) * 8 < xrows;
  const char* wblk = p.w_block(st);
  const int64_t wstep = wblk ? kPackBlock : 128;
  auto set_w = [&](int s) __attribute__((always_inline)) {
    const float* dummy = nullptr;
    const char* w0 = p.w_row(st, s, 0, &dummy);
#pragma unroll
    for (int i = 0; i < NQW; ++i) {
      const int q = wid + NW * i;
      if (wblk) {
        srcW[i] = wblk + q * 1024 + lane * 16;
      } else {
        const int row = q * 8 + (lane >> 3);
        const char* rp = p.w_row(st, s, row, &dummy);
        srcW[i] = (rp ? rp : w0) + (((lane & 7) ^ swz(row)) << 4);
      }
    }
  };
  auto set_x = [&](int s) __attribute__((always_inline)) {
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
  auto issue_w = [&](int buf) __attribute__((always_inline)) {
    char* base = smem + buf * Cfg::BF * 128;
#pragma unroll
    for (int i = 0; i < NQW; ++i) dma16<Cfg::WAUX>(srcW[i] + wk * wstep, base + (wid + NW * i) * 1024);
    if (++wk == p.seg_ktiles(wsg)) {
      wk = 0;
      do { ++wsg; } while (wsg < nks && p.seg_ktiles(wsg) == 0);
      if (wsg < nks) set_w(wsg);
    }
  };
  auto issue_x = [&](int buf) __attribute__((always_inline)) {
    char* base = smem + Cfg::X_OFF + buf * Cfg::BT * 128;
#pragma unroll
    for (int i = 0; i < NQX; ++i)
      if (xon[i]) dma16<LMOE_X_AUX>(srcX[i] + (int64_t)xk * 128, base + (wid + NW * i) * 1024);
    if (++xk == p.seg_ktiles(xsg)) {
      xk = 0;
      do { ++xsg; } while (xsg < nks && p.seg_ktiles(xsg) == 0);
      if (xsg < nks) set_x(xsg);
    }
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
    if (active) {
      const char* sW = smem + (kt % 3) * Cfg::BF * 128;
      const char* sX = smem + Cfg::X_OFF + (kt & 1) * Cfg::BT * 128;
      if constexpr (dense_rows<Prob>::value) mma_ktile_full<FI, TI>(acc, sW, sX, wf0, wt0, lane);
      else mma_ktile<FI, TI>(acc, sW, sX, wf0, wt0, lane, tiv);
    }
  }
  p.epilogue(st, acc, wf0, wt0, lane);
}

// ---------------------------------------------------------------------------
// Persistent split-ring GEMM.  The grid holds a multiple of 8 work-groups, all
// resident; work-group b serves XCD b % 8 and walks that XCD's contiguous
// range of logical tiles with stride (grid / 8), so tiles that share operands
// still run side by side in one L2.  The k-tiles of all its tiles form one
// sequence g = 0 .. G-1 (nkt per tile) through the same rings, issued as in
// gemm3_kernel: X(g+1) then W(g+2) in iteration g, wait vmcnt(NQW) at the top
// of each iteration.  A finished tile's epilogue runs in the next
// iteration, after its wait and barrier (with bf16 weights after that
// iteration's DMAs, with e4m3 weights before them).
// ---------------------------------------------------------------------------
// Vector stores a wave's epilogue issues, at least, per 32-row token block
// whose rows are all valid (0: not declared).
template <class P, class = void>
struct epi_stores : std::integral_constant<int, 0> {};
template <class P>
struct epi_stores<P, std::void_t<decltype(P::kEpiStores)>> : std::integral_constant<int, P::kEpiStores> {};

// wait_vmcnt_barrier<min(63, (W ? NQW : 0) + NB * SB)> for a runtime NB in
// 0 .. 4: the count past the awaited DMAs of the youngest weight tile (when
// issued) and of the previous epilogue's stores.
template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier_c() {
  wait_vmcnt_barrier<(N < 63 ? N : 63)>();
}
template <int NQW, int SB>
__device__ __forceinline__ void wait_past_stores(bool w, int nb) {
  if (w) {
    switch (nb) {
      case 0: wait_vmcnt_barrier_c<NQW>(); break;
      case 1: wait_vmcnt_barrier_c<NQW + SB>(); break;
      case 2: wait_vmcnt_barrier_c<NQW + 2 * SB>(); break;
      case 3: wait_vmcnt_barrier_c<NQW + 3 * SB>(); break;
      default: wait_vmcnt_barrier_c<NQW + 4 * SB>(); break;
    }
  } else {
    switch (nb) {
      case 0: wait_vmcnt_barrier_c<0>(); break;
      case 1: wait_vmcnt_barrier_c<SB>(); break;
      case 2: wait_vmcnt_barrier_c<2 * SB>(); break;
      case 3: wait_vmcnt_barrier_c<3 * SB>(); break;
      default: wait_vmcnt_barrier_c<4 * SB>(); break;
    }
  }
}

template <class Cfg, class Prob>
__global__ __launch_bounds__(Cfg::NT) void gemm3p_kernel(const Prob p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  constexpr int FI = Cfg::FI, TI = Cfg::TI, NQW = Cfg::NQW, NQX = Cfg::NQX, NW = Cfg::NW;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf0 = (wid % Cfg::WF) * Cfg::FW;
  const int wt0 = (wid / Cfg::WF) * Cfg::TW;

  // this work-group's tiles: logical xcd * per + slot + j * nslot
  const int R = p.num_logical();
  const int per = (R + kXcds - 1) / kXcds;
  const int nslot = (int)gridDim.x / kXcds;
  const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
  const int lim = min(per, R - xcd * per);
  const int ntile = lim > slot ? (lim - slot + nslot - 1) / nslot : 0;
  if (ntile == 0) return;
  auto tile_lg = [&](int j) __attribute__((always_inline)) { return xcd * per + slot + j * nslot; };

  const int nks = p.num_ksegs();
  int nkt = 0;
  for (int s = 0; s < nks; ++s) nkt += p.seg_ktiles(s);
  if (nkt == 0) return;
  const int G = ntile * nkt;
  int first_seg = 0;
  while (first_seg < nks && p.seg_ktiles(first_seg) == 0) ++first_seg;

  // compute side: current tile and its wave masks
  typename Prob::State cst;
  p.setup_lg(tile_lg(0), cst);
  int cj = 0, ckt = 0;
  int tiv = 0;
  bool active = false;
  auto masks = [&]() __attribute__((always_inline)) {
    tiv = min(TI, max(0, (p.tokens_valid(cst) - wt0 + 31) >> 5));
    active = tiv > 0 && wf0 < p.feats_valid(cst);
  };
  masks();

  f32x16 acc[FI][TI];
  auto zero = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < TI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  };
  zero();

  // weight issue side (bf16 rows: 8 rows of 128 bytes per DMA instruction;
  // e4m3 rows: 16 rows of 64 bytes)
  typename Prob::State wst = cst;
  int wj = 0, wsg = first_seg, wk = 0;
  const char* srcW[NQW];
  const char* wblk = nullptr;
  int64_t wstep = Cfg::RBW;
  auto set_w = [&]() __attribute__((always_inline)) {
    if constexpr (Cfg::WTR) {
      // instruction q stages k-rows 2 q and 2 q + 1; lane l fetches the chunk
      // that belongs at position l % 32 of k-row 2 q + l / 32
      wstep = p.w_tstep(wst, wsg);
#pragma unroll
      for (int i = 0; i < NQW; ++i) {
        const int q = wid + NW * i, kr = 2 * q + (lane >> 5);
        srcW[i] = p.w_tsrc(wst, wsg, kr, (lane & 31) ^ ((kr & 3) << 2));
      }
      return;
    }
    wblk = Cfg::WF8 ? nullptr : p.w_block(wst);
    wstep = wblk ? kPackBlock : Cfg::RBW;
    const float* dummy = nullptr;
    const char* w0 = p.w_row(wst, wsg, 0, &dummy);
#pragma unroll
    for (int i = 0; i < NQW; ++i) {
      const int q = wid + NW * i;
      if (wblk) {
        srcW[i] = wblk + q * 1024 + lane * 16;
      } else {
        constexpr int CPR = Cfg::RBW / 16;
        const int row = q * Cfg::RPIW + lane / CPR;
        const int chunk = (lane % CPR) ^ (Cfg::WF8 ? swz64(row) : swz(row));
        const char* rp = p.w_row(wst, wsg, row, &dummy);
        srcW[i] = (rp ? rp : w0) + (chunk << 4);
      }
    }
  };
  // token issue side
  typename Prob::State xst = cst;
  int xj = 0, xsg = first_seg, xk = 0;
  const char* srcX[NQX];
  bool xon[NQX];
  int xrows = 0, xg = 0;  // valid rows of the issue-side tile; X k-tiles issued
  // (row groups wholly past the valid rows are never issued and need no
  // source; x_row_grp maps the missing rows of a partial group to a valid one)
  auto set_x = [&]() __attribute__((always_inline)) {
    xrows = p.tokens_valid(xst);
#pragma unroll
    for (int i = 0; i < NQX; ++i) {
      const int r0 = (wid + NW * i) * Cfg::RPIX;
      xon[i] = r0 < xrows;
      if (xon[i]) {
        if constexpr (Cfg::XF8)
          srcX[i] = p.template x_row_grp<Cfg::RPIX>(xst, xsg, r0, lane) + (((lane & 3) ^ swz64(r0 + (lane >> 2))) << 4);
        else
          srcX[i] = p.x_row_grp(xst, xsg, r0, lane) + (((lane & 7) ^ swz(r0 + (lane >> 3))) << 4);
      }
    }
  };
  set_w();
  set_x();
  auto issue_w = [&](int buf) __attribute__((always_inline)) {
    char* base = smem + buf * Cfg::WSTAGE;
#pragma unroll
    for (int i = 0; i < NQW; ++i) dma16<Cfg::WAUX>(srcW[i] + wk * wstep, base + (wid + NW * i) * 1024);
    if (++wk == p.seg_ktiles(wsg)) {
      wk = 0;
      do { ++wsg; } while (wsg < nks && p.seg_ktiles(wsg) == 0);
      if (wsg == nks && ++wj < ntile) {
        p.setup_lg(tile_lg(wj), wst);
        wsg = first_seg;
      }
      if (wsg < nks) set_w();
    }
  };
  auto issue_x = [&](int buf) __attribute__((always_inline)) {
    char* base = smem + Cfg::X_OFF + buf * Cfg::XSTAGE;
#pragma unroll
    for (int i = 0; i < NQX; ++i)
      if (xon[i]) dma16<LMOE_X_AUX>(srcX[i] + (int64_t)xk * Cfg::RBX, base + (wid + NW * i) * 1024);
    if constexpr (Cfg::XF8) {
      // the k-tile that opens a 128-column block brings the block's row
      // scales: wave w loads rows 64 w .. 64 w + 63 (clamped to valid rows)
      // into scale slot (block index & 1)
      if ((xk & 1) == 0 && wid * 64 < xrows)
        dma4(p.x_scale(xst, xk >> 1) + min(wid * 64 + lane, xrows - 1),
             smem + Cfg::SC_OFF + ((xg >> 1) & 1) * (Cfg::BT * 4) + wid * 256);
    }
    ++xg;
    if (++xk == p.seg_ktiles(xsg)) {
      xk = 0;
      do { ++xsg; } while (xsg < nks && p.seg_ktiles(xsg) == 0);
      if (xsg == nks && ++xj < ntile) {
        p.setup_lg(tile_lg(xj), xst);
        xsg = first_seg;
      }
      if (xsg < nks) set_x();
    }
  };

  // prologue: X(0), then W(0) .. W(SW-2); iteration g issues X(g+1) then
  // W(g+SW-1).  At the top of iteration g the DMAs issued after X(g) are the
  // weight tile W(g+SW-2) alone (NQW instructions, all older weight tiles
  // precede X(g) or are older still), so vmcnt(NQW) completes X(g) and W(g);
  // once W(g+SW-2) no longer exists the wait is vmcnt(0).
  constexpr int SW = Cfg::SW;
  if constexpr (Cfg::XF8) {
    // scale slots start at 1 (entries of row groups that are never loaded
    // stay positive and finite); ordered before the first scale DMA
    for (int i = tid; i < Cfg::SX * Cfg::BT; i += Cfg::NT) reinterpret_cast<float*>(smem + Cfg::SC_OFF)[i] = 1.f;
    __syncthreads();
  }
  issue_x(0);
#pragma unroll
  for (int s = 0; s < SW - 1; ++s)
    if (s < G) issue_w(s);
  float sc[FI];
#pragma unroll
  for (int i = 0; i < FI; ++i) sc[i] = 1.f;
  // e4m3 weights: acc holds the sum over 128-column blocks divided by sp,
  // the current block's weight scale (times the row scale under W8A8);
  // entering a new block multiplies acc by old / new, the epilogue by sp.
  float sp[FI][TI];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < TI; ++j) sp[i][j] = 1.f;
  auto finish = [&]() __attribute__((always_inline)) {
    if constexpr (Cfg::WF8) {
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < TI; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] *= sp[i][j];
    }
    p.epilogue(cst, acc, wf0, wt0, lane);
  };
  bool pending = false;  // a finished tile's accumulators await their epilogue
  // bf16 weights: the epilogue's stores follow the iteration's DMAs, and the
  // next wait lets those this wave certainly issued stay in flight (vector
  // memory operations complete in issue order, so they count past X(g)):
  // eb = the finished tile's 32-row token blocks all of whose rows, and all
  // of the wave's features, are valid
  constexpr int SB = Cfg::WF8 ? 0 : epi_stores<Prob>::value;
  static_assert(SB == 0 || TI <= 4, "wait_past_stores covers four token blocks");
  int eb = 0;
  for (int g = 0; g < G; ++g) {
    if constexpr (SB > 0) {
      wait_past_stores<NQW, SB>(g + SW - 2 < G, eb);
      eb = 0;
    } else {
      if (g + SW - 2 < G) wait_vmcnt_barrier<NQW>();
      else wait_vmcnt_barrier<0>();
    }
    auto retire = [&]() __attribute__((always_inline)) {
      if (pending) {
        if constexpr (SB > 0)
          eb = wf0 + Cfg::FW <= p.feats_valid(cst) ? min(TI, max(0, (p.tokens_valid(cst) - wt0) >> 5)) : 0;
        finish();
        zero();
        ++cj;
        p.setup_lg(tile_lg(cj), cst);
        masks();
        pending = false;
      }
    };
    // bf16 weights: this iteration's DMAs go out before the finished tile's
    // epilogue, so its VALU work does not hold up the weight stream (measured
    // 4% on the gate/value GEMM) and its stores can drain under the next
    // k-tiles (the wait above); with e4m3 weights the other order measured
    // better, and the next wait then covers the stores too.
    if constexpr (Cfg::WF8) retire();
    if (g + 1 < G) issue_x((g + 1) & 1);
    if (g + SW - 1 < G) issue_w((g + SW - 1) % SW);
    if constexpr (!Cfg::WF8) retire();
    if (active) {
      const char* sW = smem + (g % SW) * Cfg::WSTAGE;
      const char* sX = smem + Cfg::X_OFF + (g & 1) * Cfg::XSTAGE;
      if constexpr (Cfg::WF8) {
        if ((ckt & 1) == 0) {
          // a new 128-column block: weight scales, and under W8A8 the row
          // scales from the slot this block's first k-tile filled.  Every
          // scale is positive and finite (the slots start at 1 and hold real
          // row scales after), so the ratio is finite; at a tile's first
          // block acc is zero and stays zero
          p.w_scales(cst, wf0, ckt >> 1, sc);
          const float* sxs =
              reinterpret_cast<const float*>(smem + Cfg::SC_OFF + ((g >> 1) & 1) * (Cfg::BT * 4)) + wt0 + (lane & 31);
#pragma unroll
          for (int j = 0; j < TI; ++j) {
            const float sx = Cfg::XF8 ? sxs[j * 32] : 1.f;
#pragma unroll
            for (int i = 0; i < FI; ++i) {
              const float sn = sc[i] * sx;
              const float r = sp[i][j] * __builtin_amdgcn_rcpf(sn);
#pragma unroll
              for (int q = 0; q < 16; ++q) acc[i][j][q] *= r;
              sp[i][j] = sn;
            }
          }
        }
        if constexpr (Cfg::XF8) mma_ktile_a8<FI, TI>(acc, sW, sX, wf0, wt0, lane, tiv);
        else mma_ktile_f8<FI, TI>(acc, sW, sX, wf0, wt0, lane, tiv);
      } else if constexpr (Cfg::WTR) {
        mma_ktile_wt<FI, TI>(acc, sW, sX, wf0, wt0, lane, tiv);
      } else {
        mma_ktile<FI, TI, false>(acc, sW, sX, wf0, wt0, lane, tiv);
      }
    }
    if (++ckt == nkt) {
      ckt = 0;
      pending = true;
    }
  }
  finish();
}

}  // namespace lmoe
