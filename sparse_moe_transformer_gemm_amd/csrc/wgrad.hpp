// Weight gradients on a persistent DMA pipeline (gfx950): the routed
// experts', and in a second mode up to kWgSegs dense products over all T rows
// in one launch (the dense projections' weight gradients).
//
//   C_e[m, n] = sum over expert e's assignment rows t of P[t, m] Q[t, n]
//
// dW_o[e] = dO_e^T A_e (P = dO, Q = A), dW_g[e] = dG_e^T z_e and
// dW_v[e] = dV_e^T z_e (Q = the latent rows z, gathered through the sorted
// assignment ids).  P and Q are stored row by row (an assignment row's M or N
// values contiguous), so both operands reach LDS as k-rows: per 64-row
// k-tile, 64 rows of the tile's 256 columns (512 bytes each, two per DMA
// instruction, 16-byte chunks swizzled by k-row as in the transposed weight
// stage of gemm3p_kernel), and both MFMA fragments come out through
// ds_read_b64_tr_b16.
//
// Every expert's [M, N] matrix is written, an expert without rows as zeros:
// its tiles run one k-tile whose rows all read a zero page.  A tile's K is
// the expert's row count, so the k-tiles per tile vary; the walk, the rings,
// the waits and the epilogue placement are those of gemm3p_kernel (token
// ring two deep, weight ring three deep, vmcnt(NQW) + s_barrier at the top
// of each k-tile, a finished tile's stores after the next iteration's DMAs).
// Rows past an expert's last read the zero page, so every k-tile issues the
// same DMAs and the waits stay exact.
#pragma once

#include "gemm2.hpp"

namespace lmoe {

constexpr int kWgSegs = 12;

// A dense product C = P^T Q over all rows [0, rows) of P [rows, ldp] and
// Q [rows, ldq] (bf16), C fp32 [M, N] row-major; N a multiple of 256, M of 8
// (the last 256-row tile stores only C's rows below M, and reads P's
// columns past M from the zero page).
struct WgSeg {
  const char* p;
  const char* q;
  float* c;
  int64_t ldp, ldq;
  int M, N;
  int first;  // first logical tile of the segment
};

struct WGradArgs {
  // routed experts (nseg == 0)
  const char* p;          // P rows, assignment order, bf16 [T*k, ldp]
  int64_t ldp;
  const char* q;          // Q rows, bf16 [rows, ldq]
  int64_t ldq;
  const int* gather_q;    // Q row of assignment a: gather_q[a] / gk (NULL: a)
  int gk;
  float* c;               // C_e at c + e * M * N, row-major [M, N]
  int M, N, E;
  const int* offsets;     // [E + 1]
  // dense segments (nseg > 0), all in one launch
  int nseg;
  int rows;
  int tiles;              // logical tiles over all segments
  WgSeg seg[kWgSegs];
  const char* zero;       // 512 zero bytes
};

typedef Tile3<256, 256, 4, 4, 0, 1, 0, 3, 0, 1> TWGrad;

// The zero page: 512 bytes, one 4-byte store per thread of a 128-thread group
// (a kernel rather than a memset, so the call stays capturable in a graph).
__global__ __launch_bounds__(128) void zero_page_kernel(uint32_t* z) { z[threadIdx.x] = 0u; }

// Both operands from transposed stages (wtr_off layout): 16 k per MFMA,
// KS k-steps per stage of 16 KS k-rows.
template <int FI, int TI, int KS>
__device__ __forceinline__ void mma_ktile_tt(f32x16 (&acc)[FI][TI], const char* sW, const char* sX, int wf0, int wt0,
                                             int lane) {
  const int G = lane >> 4, q = lane & 15;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  auto frag = [&](const char* s, int kr, int r0) __attribute__((always_inline)) {
    const char* pa = s + wtr_off(kr, r0 + 16 * (G & 1) + 4 * (q & 3));
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa + 4 * 512));
    const short v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return *reinterpret_cast<const bf16x8*>(v);
  };
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int kr = ks * 16 + 8 * (G >> 1) + (q >> 2);
    bf16x8 a[FI], b[TI];
#pragma unroll
    for (int i = 0; i < FI; ++i) a[i] = frag(sW, kr, wf0 + i * 32);
#pragma unroll
    for (int j = 0; j < TI; ++j) b[j] = frag(sX, kr, wt0 + j * 32);
    // P side as the MFMA's A operand: a block's output rows (registers) run
    // along m and its columns (lanes) along n, so each accumulator register
    // holds 32 consecutive n of one row m per half-wave
#pragma unroll
    for (int j = 0; j < TI; ++j)
#pragma unroll
      for (int i = 0; i < FI; ++i) acc[i][j] = mfma32(b[j], a[i], acc[i][j]);
  }
}

template <class Cfg, int KR>
__global__ __launch_bounds__(Cfg::NT) void wgrad3p_kernel(const WGradArgs p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  constexpr int FI = Cfg::FI, TI = Cfg::TI, NW = Cfg::NW;
  // Stages of KR k-rows (a k-row holds the tile's 256 columns, 512 bytes),
  // as many as fit per operand in half the LDS: 32 k-rows 5 deep (the DMAs
  // run D = 4 stages ahead) for the routed experts, whose K is a few hundred
  // rows and whose stores bound them; 64 k-rows 2 deep for the dense
  // segments (K = T), whose MFMA loop gains from the longer k-tiles.  One
  // DMA instruction stages two k-rows.
  static_assert(KR == 32 || KR == 64, "stage height");
  constexpr int STG = KR * 512, P = Cfg::LDS / 2 / STG, D = P - 1;
  constexpr int NQ = KR / 2 / NW;
  static_assert(NQ * NW * 2 == KR && Cfg::BF == 256 && Cfg::BT == 256, "DMAs split evenly over the waves");
  static_assert(D >= 1 && D <= 4, "the stage wait counts up to three later groups");
  static_assert(2 * P * STG <= Cfg::LDS, "the rings fit the launch's LDS");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf0 = (wid % Cfg::WF) * Cfg::FW;  // columns n of the tile (Q side, MFMA A operand)
  const int wt0 = (wid / Cfg::WF) * Cfg::TW;  // rows m of the tile (P side, MFMA B operand)

  // logical tiles, dealt to the XCDs in contiguous ranges
  const int R = p.nseg == 0 ? p.E * (p.M / 256) * (p.N / 256) : p.tiles;
  const int per = (R + kXcds - 1) / kXcds;
  const int nslot = (int)gridDim.x / kXcds;
  const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
  const int lim = min(per, R - xcd * per);
  const int ntile = lim > slot ? (lim - slot + nslot - 1) / nslot : 0;
  if (ntile == 0) return;

  struct T {
    const char* pb;  // P at (the tile's first row, column m0)
    const char* qb;  // Q at column n0 (row index absolute)
    float* cb;       // C at (m0, n0)
    int64_t ldp, ldq, ldc;
    int off, rows, nkt;
    int mv;          // rows of C in the tile (dense segments: M - m0, up to 256)
  };
  // experts: expert-major, then m tiles, then n tiles; dense: segment after
  // segment, m tiles, then n tiles
  auto locate = [&](int j, T& t) __attribute__((always_inline)) {
    const int lg = xcd * per + slot + j * nslot;
    if (p.nseg == 0) {
      const int ntn = p.N / 256, per_e = (p.M / 256) * ntn;
      const int e = lg / per_e, rem = lg - e * per_e;
      const int m0 = (rem / ntn) * 256, n0 = (rem % ntn) * 256;
      const i32x2 ob = sload2(p.offsets + e);
      t.off = ob.x;
      t.rows = ob.y - ob.x;
      t.ldp = p.ldp;
      t.ldq = p.ldq;
      t.ldc = p.N;
      t.pb = p.p + ((int64_t)t.off * p.ldp + m0) * 2;
      t.qb = p.q + (int64_t)n0 * 2;
      t.cb = p.c + (int64_t)e * p.M * p.N + (int64_t)m0 * p.N + n0;
      t.mv = 256;
    } else {
      int s = 0;
#pragma unroll
      for (int u = 1; u < kWgSegs; ++u)
        if (u < p.nseg && lg >= p.seg[u].first) s = u;
      const WgSeg& sg = p.seg[s];
      const int ntn = sg.N / 256, rem = lg - sg.first;
      const int m0 = (rem / ntn) * 256, n0 = (rem % ntn) * 256;
      t.off = 0;
      t.rows = p.rows;
      t.ldp = sg.ldp;
      t.ldq = sg.ldq;
      t.ldc = sg.N;
      t.pb = sg.p + (int64_t)m0 * 2;
      t.qb = sg.q + (int64_t)n0 * 2;
      t.cb = sg.c + (int64_t)m0 * sg.N + n0;
      t.mv = min(256, sg.M - m0);
    }
    t.nkt = max(1, (t.rows + KR - 1) / KR);
  };
  int G = 0;
  for (int j = 0; j < ntile; ++j) {
    T t;
    locate(j, t);
    G += t.nkt;
  }

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

  // issue sides: tile and k-tile cursors per operand
  T xt, wt;
  locate(0, xt);
  wt = xt;
  int xj = 0, xk = 0, wj = 0, wk = 0;
  // instruction q of a k-tile stages k-rows 2 q and 2 q + 1 of it; lane l the
  // chunk that belongs at position l % 32 of k-row 2 q + l / 32
  auto issue_x = [&](int buf) __attribute__((always_inline)) {
    char* base = smem + P * STG + buf * STG;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int q = wid + NW * i, kr = 2 * q + (lane >> 5), c = (lane & 31) ^ ((kr & 3) << 2);
      const int t = xk * KR + kr;
      // dense segments: P's columns past M come from the zero page too
      const bool in = t < xt.rows && (KR == 32 || 8 * c < xt.mv);
      const char* src = in ? xt.pb + ((int64_t)t * xt.ldp + 8 * c) * 2 : p.zero + 16 * c;
      dma16<0>(src, base + q * 1024);
    }
    if (++xk == xt.nkt) {
      xk = 0;
      if (++xj < ntile) locate(xj, xt);
    }
  };
  auto issue_w = [&](int buf) __attribute__((always_inline)) {
    char* base = smem + buf * STG;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int q = wid + NW * i, c = (lane & 31) ^ (((2 * q + (lane >> 5)) & 3) << 2);
      // the two k-rows' Q rows, read through the scalar cache (no vector
      // load may join the DMA count); clamped into the expert's rows
      const int t0 = wk * KR + 2 * q;
      int r0 = 0, r1 = 0;
      if (wt.rows > 0) {
        const int a0 = wt.off + min(t0, wt.rows - 1), a1 = wt.off + min(t0 + 1, wt.rows - 1);
        if (p.nseg == 0 && p.gather_q) {
          const i32x2 g = sload_pair(p.gather_q + a0, p.gather_q + a1);
          r0 = g.x / p.gk;
          r1 = g.y / p.gk;
        } else {
          r0 = a0;
          r1 = a1;
        }
      }
      const int t = t0 + (lane >> 5);
      const int row = (lane >> 5) ? r1 : r0;
      const char* src = t < wt.rows ? wt.qb + ((int64_t)row * wt.ldq + 8 * c) * 2 : p.zero + 16 * c;
      dma16<0>(src, base + q * 1024);
    }
    if (++wk == wt.nkt) {
      wk = 0;
      if (++wj < ntile) locate(wj, wt);
    }
  };

  // compute side
  T ct = xt;
  int cj = 0, ckt = 0;
  auto finish = [&]() __attribute__((always_inline)) {
    // block (i, j), register 4 g + r: row m = wt0 + 32 j + 8 g + 4 (lane / 32)
    // + r, column n = wf0 + 32 i + lane % 32; one store instruction writes two
    // 128-byte row segments
    const int m1 = wt0 + 4 * (lane >> 5);
    float* ce = ct.cb + (int64_t)m1 * ct.ldc + wf0 + (lane & 31);
    // dense segments: only rows of C below M (lim < 128 only in a last,
    // partial 256-row tile)
    const int lim = KR == 32 ? 256 : ct.mv - m1;
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < TI; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (KR == 32 || 32 * j + 8 * g + r < lim) ce[(int64_t)(32 * j + 8 * g + r) * ct.ldc + 32 * i] = acc[i][j][4 * g + r];
  };

  // Group g = X(g) then W(g), NQ instructions each per wave.  The prologue
  // issues groups 0 .. D-1; iteration g waits for group g, issues group
  // g + D into the stages group g - 1 used, multiplies stage g, and before
  // that stores a finished tile (64 stores per wave) after its DMAs.  The
  // wait needs group g done; after it the wave has issued the groups up to
  // g + D - 1 and the stores of the last D iterations.  When any of those
  // iterations stored, at least 64 operations follow group g, so
  // vmcnt(63) covers it and leaves the stores in flight; otherwise the
  // count is exact: 2 NQ per later group.  A wave whose rows of a dense
  // segment's last, partial tile hold fewer than 64 rows of C skips the
  // stores of the missing rows (their instructions are branched over), so
  // it drains its counter right after its stores instead.
  constexpr int SB = FI * TI * 16;
  static_assert(SB >= 63, "a tile's stores alone exceed the wait's cap");
  for (int g = 0; g < D && g < G; ++g) {
    issue_x(g);
    issue_w(g);
  }
  bool pending = false;
  unsigned hist = 0;  // bit i: iteration g - 1 - i stored a tile
  for (int g = 0; g < G; ++g) {
    if (hist & ((1u << D) - 1)) {
      wait_vmcnt_barrier<63>();
    } else {
      switch (min(D - 1, G - 1 - g)) {
        case 0: wait_vmcnt_barrier<0>(); break;
        case 1: wait_vmcnt_barrier_c<2 * NQ>(); break;
        case 2: wait_vmcnt_barrier_c<4 * NQ>(); break;
        default: wait_vmcnt_barrier_c<6 * NQ>(); break;
      }
    }
    if (g + D < G) {
      issue_x((g + D) % P);
      issue_w((g + D) % P);
    }
    hist <<= 1;
    if (pending) {
      const bool all_rows = KR == 32 || ct.mv - wt0 >= Cfg::TW;  // uniform over the wave
      finish();
      if (!all_rows) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      zero();
      locate(++cj, ct);
      pending = false;
      hist |= 1;
    }
    mma_ktile_tt<FI, TI, KR / 16>(acc, smem + (g % P) * STG, smem + P * STG + (g % P) * STG, wf0, wt0, lane);
    if (++ckt == ct.nkt) {
      ckt = 0;
      pending = true;
    }
  }
  finish();
}

}  // namespace lmoe
