// Weight gradients of the routed experts on a persistent DMA pipeline
// (gfx950).
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

struct WGradArgs {
  const char* p;          // P rows, assignment order, bf16 [T*k, ldp]
  int64_t ldp;
  const char* q;          // Q rows, bf16 [rows, ldq]
  int64_t ldq;
  const int* gather_q;    // Q row of assignment a: gather_q[a] / gk (NULL: a)
  int gk;
  float* c;               // C_e at c + e * M * N, row-major [M, N]
  int M, N, E;
  const int* offsets;     // [E + 1]
  const char* zero;       // 512 zero bytes
};

typedef Tile3<256, 256, 4, 4, 0, 1, 0, 3, 0, 1> TWGrad;

// The zero page: 512 bytes, one 4-byte store per thread of a 128-thread group
// (a kernel rather than a memset, so the call stays capturable in a graph).
__global__ __launch_bounds__(128) void zero_page_kernel(uint32_t* z) { z[threadIdx.x] = 0u; }

// Both operands from transposed stages (wtr_off layout): 16 k per MFMA,
// 4 k-steps per 64-row k-tile.
template <int FI, int TI>
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
  for (int ks = 0; ks < 4; ++ks) {
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

template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void wgrad3p_kernel(const WGradArgs p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  constexpr int FI = Cfg::FI, TI = Cfg::TI, NQW = Cfg::NQW, NQX = Cfg::NQX, NW = Cfg::NW;
  static_assert(NQW == NQX && Cfg::QW == 32 && Cfg::QX == 32, "32 DMA instructions per operand per k-tile");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf0 = (wid % Cfg::WF) * Cfg::FW;  // columns n of the tile (Q side, MFMA A operand)
  const int wt0 = (wid / Cfg::WF) * Cfg::TW;  // rows m of the tile (P side, MFMA B operand)

  // logical tiles: expert-major, then m tiles, then n tiles
  const int ntm = p.M / 256, ntn = p.N / 256, per_e = ntm * ntn;
  const int R = p.E * per_e;
  const int per = (R + kXcds - 1) / kXcds;
  const int nslot = (int)gridDim.x / kXcds;
  const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
  const int lim = min(per, R - xcd * per);
  const int ntile = lim > slot ? (lim - slot + nslot - 1) / nslot : 0;
  if (ntile == 0) return;

  struct T {
    int e, m0, n0, off, rows, nkt;
  };
  auto locate = [&](int j, T& t) __attribute__((always_inline)) {
    const int lg = xcd * per + slot + j * nslot;
    t.e = lg / per_e;
    const int rem = lg - t.e * per_e;
    t.m0 = (rem / ntn) * 256;
    t.n0 = (rem % ntn) * 256;
    const i32x2 ob = sload2(p.offsets + t.e);
    t.off = ob.x;
    t.rows = ob.y - ob.x;
    t.nkt = max(1, (t.rows + 63) >> 6);
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
    char* base = smem + Cfg::X_OFF + buf * Cfg::XSTAGE;
#pragma unroll
    for (int i = 0; i < NQX; ++i) {
      const int q = wid + NW * i, kr = 2 * q + (lane >> 5), c = (lane & 31) ^ ((kr & 3) << 2);
      const int t = xk * 64 + kr;
      const char* src = t < xt.rows ? p.p + (((int64_t)xt.off + t) * p.ldp + xt.m0 + 8 * c) * 2 : p.zero + 16 * c;
      dma16<0>(src, base + q * 1024);
    }
    if (++xk == xt.nkt) {
      xk = 0;
      if (++xj < ntile) locate(xj, xt);
    }
  };
  auto issue_w = [&](int buf) __attribute__((always_inline)) {
    char* base = smem + buf * Cfg::WSTAGE;
#pragma unroll
    for (int i = 0; i < NQW; ++i) {
      const int q = wid + NW * i, c = (lane & 31) ^ (((2 * q + (lane >> 5)) & 3) << 2);
      // the two k-rows' Q rows, read through the scalar cache (no vector
      // load may join the DMA count); clamped into the expert's rows
      const int t0 = wk * 64 + 2 * q;
      int r0 = 0, r1 = 0;
      if (wt.rows > 0) {
        const int a0 = wt.off + min(t0, wt.rows - 1), a1 = wt.off + min(t0 + 1, wt.rows - 1);
        if (p.gather_q) {
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
      const char* src = t < wt.rows ? p.q + ((int64_t)row * p.ldq + wt.n0 + 8 * c) * 2 : p.zero + 16 * c;
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
    float* ce = p.c + (int64_t)ct.e * p.M * p.N + ((int64_t)ct.m0 + wt0 + 4 * (lane >> 5)) * p.N + ct.n0 + wf0 + (lane & 31);
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < TI; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) ce[(int64_t)(32 * j + 8 * g + r) * p.N + 32 * i] = acc[i][j][4 * g + r];
  };

  // prologue and iterations as gemm3p_kernel: X(0), W(0), W(1); iteration g
  // issues X(g + 1) then W(g + 2), after waiting for X(g) and W(g)
  issue_x(0);
  issue_w(0);
  if (1 < G) issue_w(1);
  bool pending = false;
  for (int g = 0; g < G; ++g) {
    if (g + 1 < G) wait_vmcnt_barrier<NQW>();
    else wait_vmcnt_barrier<0>();
    if (g + 1 < G) issue_x((g + 1) & 1);
    if (g + 2 < G) issue_w((g + 2) % 3);
    if (pending) {
      finish();
      zero();
      locate(++cj, ct);
      pending = false;
    }
    mma_ktile_tt<FI, TI>(acc, smem + (g % 3) * Cfg::WSTAGE, smem + Cfg::X_OFF + (g & 1) * Cfg::XSTAGE, wf0, wt0,
                         lane);
    if (++ckt == ct.nkt) {
      ckt = 0;
      pending = true;
    }
  }
  finish();
}

}  // namespace lmoe
