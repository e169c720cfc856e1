// Backward pass of the layer: a generic MFMA GEMM for the gradient GEMMs
// (dense and per-expert, with either operand stored k-contiguous or
// row-contiguous) and the elementwise gradient kernels (SiTU-GLU, RMSNorm,
// weighted combine, router).  Gradients are fp32.
//
// Sources: P2 wpnews.pro "The 2.8-Trillion-Parameter Problem", stabilizer
// passage (the cap and the norm are there to keep training stable); the
// chain rule of the forward steps of P2's Stable LatentMoE passage.
#pragma once

#include "common.hpp"

namespace lmoe {

// ---------------------------------------------------------------------------
// Generic GEMM: C[m, n] (= or +=) sum_k A(m, k) B(n, k), fp32 out (or bf16),
// bf16 32x32x16 MFMAs with fp32 accumulation; fp32 operands are rounded to
// bf16 (nearest even) as they are staged into LDS.
//
// An operand element (r, k) -- r the operand's row (m for A, n for B) -- is
// stored at  base + sr * ld + k   (RC = 0: k contiguous), or
//            base + sr * ld + r   (RC = 1: rows contiguous),
// where the stored row sr is r (RC = 0) or k (RC = 1), plus the group's first
// assignment row when `grow` is set, and then mapped through `gather`
// (sr -> gather[sr] / gk) when that is given.  `gstride` moves the base by
// group (stacked expert weights).
//
// Modes: BG_DENSE (one matrix); BG_GROUP_M (per expert, M = the expert's
// assignment rows, walked through the expert tile list of 128-row tiles; C
// rows are assignment rows); BG_GROUP_K (per expert, K = the expert's
// assignment rows, one grid slice per expert; C moves by cgstride).
// ---------------------------------------------------------------------------
enum { BG_DENSE = 0, BG_GROUP_M = 1, BG_GROUP_K = 2 };

struct BgOp {
  const char* p;
  int64_t ld;
  int64_t gstride;
  const int* gather;
  int gk;
  int grow;
};

struct BgArgs {
  BgOp a, b;
  char* c;
  int64_t ldc, cgstride;
  int M, N, K;
  int accumulate, cbf16;
  const int* offsets;
  const int4* tiles;
  const int* tile_count;
};

#ifndef LMOE_BG_K
#define LMOE_BG_K 32
#endif
constexpr int kBgM = 128, kBgN = 128, kBgK = LMOE_BG_K;
constexpr int kBgPitch = kBgK * 2 + 16;       // LDS row: the k-tile in bf16 + 16 B pad
constexpr int kBgRcPitch = (kBgM + 8) * 2;    // row-contiguous tiles: one k per LDS row, 128 rows + pad
constexpr int kBgTileBytes = kBgM * kBgPitch > kBgK * kBgRcPitch ? kBgM * kBgPitch : kBgK * kBgRcPitch;
constexpr int kBgVec = kBgM * kBgK / 8 / 256;  // 8-element vectors per thread per operand tile

__device__ __forceinline__ unsigned short f2bf(float f) {
  const bf16 h = (bf16)f;  // round to nearest even
  return *reinterpret_cast<const unsigned short*>(&h);
}

// Loads 8 consecutive stored elements (along the contiguous dimension) as
// bf16; `n` of them are valid (the rest are zero).
template <int F32>
__device__ __forceinline__ uint4 bg_load8(const char* p, int n, bool vec) {
  if (F32) {
    const float* f = reinterpret_cast<const float*>(p);
    float v[8];
    if (vec && n == 8) {
      const float4 u = *reinterpret_cast<const float4*>(f);
      const float4 w = *reinterpret_cast<const float4*>(f + 4);
      v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w; v[4] = w.x; v[5] = w.y; v[6] = w.z; v[7] = w.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = i < n ? f[i] : 0.f;
    }
    uint4 o;
    o.x = f2bf(v[0]) | ((unsigned)f2bf(v[1]) << 16);
    o.y = f2bf(v[2]) | ((unsigned)f2bf(v[3]) << 16);
    o.z = f2bf(v[4]) | ((unsigned)f2bf(v[5]) << 16);
    o.w = f2bf(v[6]) | ((unsigned)f2bf(v[7]) << 16);
    return o;
  } else {
    if (vec && n == 8) return *reinterpret_cast<const uint4*>(p);
    const unsigned short* h = reinterpret_cast<const unsigned short*>(p);
    unsigned short v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = i < n ? h[i] : (unsigned short)0;
    return uint4{v[0] | ((unsigned)v[1] << 16), v[2] | ((unsigned)v[3] << 16), v[4] | ((unsigned)v[5] << 16),
                 v[6] | ((unsigned)v[7] << 16)};
  }
}

// One operand tile (128 rows x kBgK) of one k-tile into registers, kBgVec
// vectors of 8 elements per thread.  rows / kv: valid rows and k.
template <int RC, int F32>
struct BgTile {
  uint4 v[kBgVec];
  __device__ __forceinline__ void load(const BgOp& o, const char* base, int rowbase, int r0, int rows, int k0,
                                       int kv, bool vec, int tid) {
    constexpr int ES = F32 ? 4 : 2, VPR = kBgK / 8;  // vectors per k-contiguous row
#pragma unroll
    for (int q = 0; q < kBgVec; ++q) {
      const int vi = tid + 256 * q;
      if (!RC) {
        const int r = vi / VPR, kk = (vi % VPR) * 8;
        const int n = min(8, kv - kk);
        if (r < rows && n > 0) {
          int sr = r0 + r + (o.grow ? rowbase : 0);
          if (o.gather) sr = o.gather[sr] / o.gk;
          v[q] = bg_load8<F32>(base + ((int64_t)sr * o.ld + k0 + kk) * ES, n, vec);
        } else {
          v[q] = uint4{0u, 0u, 0u, 0u};
        }
      } else {
        const int kk = vi >> 4, r8 = (vi & 15) * 8;
        const int n = min(8, rows - r8);
        if (kk < kv && n > 0) {
          int sr = k0 + kk + (o.grow ? rowbase : 0);
          if (o.gather) sr = o.gather[sr] / o.gk;
          v[q] = bg_load8<F32>(base + ((int64_t)sr * o.ld + r0 + r8) * ES, n, vec);
        } else {
          v[q] = uint4{0u, 0u, 0u, 0u};
        }
      }
    }
  }
  // LDS image.  k-contiguous operands: row r at r * kBgPitch, k contiguous.
  // Row-contiguous operands keep their layout: k at k * kBgRcPitch, rows
  // contiguous (the fragments are read with transposing LDS reads).
  __device__ __forceinline__ void store(char* s, int tid) const {
    constexpr int VPR = kBgK / 8;
#pragma unroll
    for (int q = 0; q < kBgVec; ++q) {
      const int vi = tid + 256 * q;
      if (!RC) {
        const int r = vi / VPR, kk = (vi % VPR) * 8;
        *reinterpret_cast<uint4*>(s + r * kBgPitch + kk * 2) = v[q];
      } else {
        const int kk = vi >> 4, r8 = (vi & 15) * 8;
        *reinterpret_cast<uint4*>(s + kk * kBgRcPitch + r8 * 2) = v[q];
      }
    }
  }
};

typedef short bgv4 __attribute__((ext_vector_type(4)));

// MFMA fragment of rows r0 .. r0 + 31 at k-step ks: lane l holds the 8
// consecutive k (8 (l / 32) .. + 7 within the step) of row r0 + l % 32.
// Row-contiguous tiles are read with ds_read_b64_tr_b16: in each 16-lane
// group, lane i receives element i % 4 of the 4-element loads of lanes
// 4 j + i / 4 (j = 0..3), so lane q of group G points at k-row
// 8 (G / 2) + q / 4 and rows r0 + 16 (G % 2) + 4 (q % 4) .. + 3; a second read
// 4 k-rows further gives the other 4 k.
template <int RC>
__device__ __forceinline__ bf16x8 bg_frag(const char* s, int r0, int ks, int lane) {
  if (!RC) {
    return *reinterpret_cast<const bf16x8*>(s + (r0 + (lane & 31)) * kBgPitch + (ks * 16 + (lane >> 5) * 8) * 2);
  } else {
    const int G = lane >> 4, q = lane & 15;
    const char* p = s + (ks * 16 + 8 * (G >> 1) + (q >> 2)) * kBgRcPitch + (r0 + 16 * (G & 1) + 4 * (q & 3)) * 2;
    typedef __attribute__((address_space(3))) bgv4 lds_v4;
    const bgv4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(p));
    const bgv4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(p + 4 * kBgRcPitch));
    const short v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return *reinterpret_cast<const bf16x8*>(v);
  }
}

// 16-byte loads need the row pitch and the base 16-byte aligned.
__device__ __forceinline__ bool bg_vec_ok(const char* base, int64_t ld, int es) {
  return ((reinterpret_cast<uintptr_t>(base) & 15) == 0) && ((ld * es) % 16 == 0);
}

// The grouped modes (per-expert wgrads with a few k-tiles per work-group, and
// the row-tiled dgrads over each expert's rows) are latency-bound: they ask
// for 4 waves per SIMD, i.e. at most 128 registers. The dgrads spill a few
// registers at that bound and are still faster (measured); the dense mode keeps
// its full register budget.
template <int MODE, int ARC, int AF32, int BRC, int BF32>
__global__ __launch_bounds__(256, MODE != BG_DENSE ? 4 : 1) void bgemm_kernel(const BgArgs p) {
  // operand double buffers; after the k-loop the grouped-K mode reuses them
  // to stage its output tile (below)
  __shared__ __attribute__((aligned(16))) char smem[4 * kBgTileBytes];
  char (*sA)[kBgTileBytes] = reinterpret_cast<char (*)[kBgTileBytes]>(smem);
  char (*sB)[kBgTileBytes] = reinterpret_cast<char (*)[kBgTileBytes]>(smem + 2 * kBgTileBytes);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int e = 0, rowbase = 0, M = p.M, K = p.K, m0 = 0;
  const int n0 = blockIdx.x * kBgN;
  if (MODE == BG_DENSE) {
    m0 = blockIdx.y * kBgM;
  } else if (MODE == BG_GROUP_M) {
    const int j = blockIdx.y;
    if (j >= *p.tile_count) return;
    const int4 te = p.tiles[j];
    e = te.x;
    rowbase = p.offsets[e];
    M = p.offsets[e + 1] - rowbase;
    m0 = (j - te.y) * kBgM;
  } else {
    e = blockIdx.z;
    m0 = blockIdx.y * kBgM;
    rowbase = p.offsets[e];
    K = p.offsets[e + 1] - rowbase;
  }
  if (m0 >= M || n0 >= p.N) return;
  const int rows_a = min(kBgM, M - m0), rows_b = min(kBgN, p.N - n0);
  const char* abase = p.a.p + (int64_t)e * p.a.gstride * (AF32 ? 4 : 2);
  const char* bbase = p.b.p + (int64_t)e * p.b.gstride * (BF32 ? 4 : 2);
  const bool avec = bg_vec_ok(abase, p.a.ld, AF32 ? 4 : 2);
  const bool bvec = bg_vec_ok(bbase, p.b.ld, BF32 ? 4 : 2);

  const int wm = (wid & 1) * 64, wn = (wid >> 1) * 64;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  BgTile<ARC, AF32> ta;
  BgTile<BRC, BF32> tb;
  const int nk = (K + kBgK - 1) / kBgK;
  auto load = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kt * kBgK, kv = min(kBgK, K - k0);
    ta.load(p.a, abase, rowbase, m0, rows_a, k0, kv, avec, tid);
    tb.load(p.b, bbase, rowbase, n0, rows_b, k0, kv, bvec, tid);
  };
  if (nk > 0) {
    load(0);
    ta.store(sA[0], tid);
    tb.store(sB[0], tid);
  }
  __syncthreads();
  const int lr = lane & 31;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load(kt + 1);
#pragma unroll
    for (int ks = 0; ks < kBgK / 16; ++ks) {
      // 32-row blocks with no valid row (an expert's last, partial row
      // tile; a tile past N) are skipped, reads and MFMAs alike: the test is
      // uniform across the wave
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (wm + i * 32 < rows_a) a[i] = bg_frag<ARC>(sA[cur], wm + i * 32, ks, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (wn + j * 32 < rows_b) b[j] = bg_frag<BRC>(sB[cur], wn + j * 32, ks, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (wm + i * 32 < rows_a && wn + j * 32 < rows_b) {
            // dense and grouped-K modes: transposed blocks, for row-vector
            // stores (below)
            if constexpr (MODE != BG_GROUP_M)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
          }
    }
    if (kt + 1 < nk) {
      ta.store(sA[cur ^ 1], tid);
      tb.store(sB[cur ^ 1], tid);
    }
    __syncthreads();
  }

  char* cbase = p.c + (int64_t)e * p.cgstride * (p.cbf16 ? 2 : 4);
  const int crow0 = (MODE == BG_GROUP_M ? rowbase : 0) + m0;
  if constexpr (MODE == BG_GROUP_K) {
    // The weight gradients are the backward's largest writes (fp32, every
    // expert's full matrices).  The tile goes out through LDS in two halves of
    // 64 rows: the two waves holding a half write their transposed blocks
    // (lane l: row l % 32, 4 consecutive columns per group g), then all 256
    // threads store it row by row, 16 bytes per lane, so each store
    // instruction covers two whole 512-byte row segments.
    constexpr int CP = kBgN + 4;  // staged row pitch in floats
    static_assert(64 * CP * 4 <= 4 * kBgTileBytes, "half tile in LDS");
    float* sc = reinterpret_cast<float*>(smem);
    const bool cvec = !p.cbf16 && (p.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(cbase) & 15) == 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if ((wid & 1) == half) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int m = i * 32 + lr, n = wn + j * 32 + g * 8 + (lane >> 5) * 4;
              *reinterpret_cast<f32x4*>(sc + m * CP + n) =
                  f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
            }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int ml = q * 8 + (tid >> 5), n = (tid & 31) * 4;
        const int m = half * 64 + ml;
        if (m < rows_a && n < rows_b) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(sc + ml * CP + n);
          const int64_t off = (int64_t)(crow0 + m) * p.ldc + n0 + n;
          if (cvec && n + 3 < rows_b) {
            float* cp = reinterpret_cast<float*>(cbase) + off;
            f32x4 o = v;
            if (p.accumulate) o += *reinterpret_cast<const f32x4*>(cp);
            *reinterpret_cast<f32x4*>(cp) = o;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (n + r >= rows_b) continue;
              if (p.cbf16) {
                reinterpret_cast<unsigned short*>(cbase)[off + r] = f2bf(v[r]);
              } else {
                float* cp = reinterpret_cast<float*>(cbase) + off + r;
                *cp = p.accumulate ? *cp + v[r] : v[r];
              }
            }
          }
        }
      }
      __syncthreads();
    }
    return;
  }
  if constexpr (MODE == BG_DENSE) {
    // acc[i][j] is the transposed 32x32 block: lane l holds row m = l % 32 of
    // C and its columns 8 g + 4 (l / 32) + r (g, r < 4), so each g is four
    // consecutive elements of one C row, stored as one 16-byte (fp32) or
    // 8-byte (bf16) vector where aligned and wholly inside the tile.  (The
    // grouped-M mode measured slower this way and keeps the layout below.)
    const bool cvec = (p.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(cbase) & (p.cbf16 ? 7 : 15)) == 0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int m = wm + i * 32 + lr;
        if (m >= rows_a || wn + j * 32 >= rows_b) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = wn + j * 32 + g * 8 + (lane >> 5) * 4;
          if (n >= rows_b) continue;
          const int64_t off = (int64_t)(crow0 + m) * p.ldc + n0 + n;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * g + r];
          if (p.cbf16) {
            unsigned short* cp = reinterpret_cast<unsigned short*>(cbase) + off;
            if (cvec && n + 3 < rows_b) {
              *reinterpret_cast<uint2*>(cp) =
                  uint2{f2bf(v[0]) | ((unsigned)f2bf(v[1]) << 16), f2bf(v[2]) | ((unsigned)f2bf(v[3]) << 16)};
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (n + r < rows_b) cp[r] = f2bf(v[r]);
            }
          } else {
            float* cp = reinterpret_cast<float*>(cbase) + off;
            if (cvec && n + 3 < rows_b) {
              float4 o = {v[0], v[1], v[2], v[3]};
              if (p.accumulate) {
                const float4 c = *reinterpret_cast<const float4*>(cp);
                o.x += c.x;
                o.y += c.y;
                o.z += c.z;
                o.w += c.w;
              }
              *reinterpret_cast<float4*>(cp) = o;
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (n + r < rows_b) cp[r] = p.accumulate ? cp[r] + v[r] : v[r];
            }
          }
        }
      }
    return;
  }
  // lane l holds column n = l % 32 of each 32x32 block and rows
  // 8 g + 4 (l / 32) + r (g, r < 4)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = wn + j * 32 + lr;
      if (n >= rows_b) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = wm + i * 32 + g * 8 + (lane >> 5) * 4 + r;
          if (m >= rows_a) continue;
          const int64_t off = (int64_t)(crow0 + m) * p.ldc + n0 + n;
          float v = acc[i][j][4 * g + r];
          if (p.cbf16) {
            reinterpret_cast<unsigned short*>(cbase)[off] = f2bf(v);
          } else {
            float* cp = reinterpret_cast<float*>(cbase) + off;
            if (p.accumulate) v += *cp;
            *cp = v;
          }
        }
    }
}

// ---------------------------------------------------------------------------
// Elementwise gradient kernels.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bw_sigmoid(float u) { return 1.f / (1.f + expf(-u)); }

// SiTU-GLU on flat arrays, four elements per thread (n a multiple of 4):
// mode 0 writes a = silu(cap g) cap v; mode 1 writes dg, dv of a given da.
// Outputs are bf16 (the next GEMM's operand precision).
__global__ __launch_bounds__(256) void bw_situ_kernel(int mode, const float* g, const float* v, const float* da,
                                                      unsigned short* o1, unsigned short* o2, int64_t n, float cap,
                                                      float inv_cap) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const f32x4 g4 = *reinterpret_cast<const f32x4*>(g + i), v4 = *reinterpret_cast<const f32x4*>(v + i);
  f32x4 d4 = {0.f, 0.f, 0.f, 0.f};
  if (mode != 0) d4 = *reinterpret_cast<const f32x4*>(da + i);
  unsigned short a1[4], a2[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float gg = g4[e], vv = v4[e];
    float cg = gg, cv = vv, dcg = 1.f, dcv = 1.f;
    if (inv_cap > 0.f) {
      const float tg = tanhf(gg * inv_cap), tv = tanhf(vv * inv_cap);
      cg = cap * tg;
      cv = cap * tv;
      dcg = 1.f - tg * tg;
      dcv = 1.f - tv * tv;
    }
    const float sg = bw_sigmoid(cg);
    if (mode == 0) {
      a1[e] = f2bf(cg * sg * cv);
    } else {
      const float d = d4[e];
      a1[e] = f2bf(d * cv * sg * (1.f + cg * (1.f - sg)) * dcg);
      a2[e] = f2bf(d * cg * sg * dcv);
    }
  }
  *reinterpret_cast<uint2*>(o1 + i) = uint2{a1[0] | ((unsigned)a1[1] << 16), a1[2] | ((unsigned)a1[3] << 16)};
  if (mode != 0)
    *reinterpret_cast<uint2*>(o2 + i) = uint2{a2[0] | ((unsigned)a2[1] << 16), a2[2] | ((unsigned)a2[3] << 16)};
}

// Block sum of one float per thread (256 threads); every thread gets it.
__device__ __forceinline__ float bw_block_sum(float v, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ float bf2f(unsigned short h) { return __uint_as_float((unsigned)h << 16); }

// Per token: dc = r u - r^3 c (u . c) / L with u = gamma dn; then for each
// slot j, dO[pos(t, j)] = w_tj dc (bf16) and dw_tj = dc . O[pos(t, j)] (fp32
// dc).  Thread c holds 8-element chunks c, c + 256, ... of the row (L a
// multiple of 8, at most 256 * 8 * MAXC): dc stays in registers across the
// k slots, every load and store moves 16 or 32 bytes per lane, and the k
// dot products are reduced together at the end.
template <int MAXC>
__global__ __launch_bounds__(256) void bw_norm_combine_grad_kernel(const float* dn, const float* c, const float* r,
                                                                   const float* gamma, const unsigned short* O,
                                                                   const int32_t* pos, const float* w, int L, int k,
                                                                   unsigned short* dO, float* dw) {
  constexpr int KMAX = 64;
  __shared__ float red[4];
  __shared__ float part[4 * KMAX];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nch = L / 8;
  const float rr = r[t];
  float dc[MAXC][8];
  float uc = 0.f;
#pragma unroll
  for (int q = 0; q < MAXC; ++q) {
    const int ch = tid + q * 256;
    if (ch < nch) {
      const int64_t o = t * L + ch * 8;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dn + o + 4 * h);
        const f32x4 c4 = *reinterpret_cast<const f32x4*>(c + o + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ge = gamma[ch * 8 + 4 * h + e];  // a caller's pointer: element loads
          uc += ge * d4[e] * c4[e];
          dc[q][4 * h + e] = rr * ge * d4[e];  // the c part is subtracted below
        }
      }
    }
  }
  const float coef = rr * rr * rr * bw_block_sum(uc, red) / L;
#pragma unroll
  for (int q = 0; q < MAXC; ++q) {
    const int ch = tid + q * 256;
    if (ch < nch) {
      const int64_t o = t * L + ch * 8;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4 c4 = *reinterpret_cast<const f32x4*>(c + o + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) dc[q][4 * h + e] -= coef * c4[e];
      }
    }
  }
  for (int j = 0; j < k; ++j) {
    const int64_t a = pos[t * k + j];
    const float wj = w[t * k + j];
    float dot = 0.f;
#pragma unroll
    for (int q = 0; q < MAXC; ++q) {
      const int ch = tid + q * 256;
      if (ch < nch) {
        const uint4 ov = *reinterpret_cast<const uint4*>(O + a * L + ch * 8);
        const unsigned ow[4] = {ov.x, ov.y, ov.z, ov.w};
        unsigned pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = dc[q][2 * e], hi = dc[q][2 * e + 1];
          dot += lo * bf2f((unsigned short)(ow[e] & 0xffffu)) + hi * bf2f((unsigned short)(ow[e] >> 16));
          pk[e] = f2bf(wj * lo) | ((unsigned)f2bf(wj * hi) << 16);
        }
        *reinterpret_cast<uint4*>(dO + a * L + ch * 8) = uint4{pk[0], pk[1], pk[2], pk[3]};
      }
    }
    // wave partial of slot j (j < KMAX: the shape check bounds k by 64)
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) dot += __shfl_xor(dot, m);
    if (lane == 0) part[wv * KMAX + j] = dot;
  }
  __syncthreads();
  for (int j = tid; j < k; j += 256) dw[t * k + j] = part[j] + part[KMAX + j] + part[2 * KMAX + j] + part[3 * KMAX + j];
}

// dgamma partials: part[y, l] = sum over tokens t of chunk y of dn c r.
__global__ __launch_bounds__(256) void bw_dgamma_part_kernel(const float* dn, const float* c, const float* r,
                                                             int64_t T, int L, int64_t chunk, float* part) {
  const int l = blockIdx.x * 256 + threadIdx.x;
  if (l >= L) return;
  const int64_t t0 = (int64_t)blockIdx.y * chunk, t1 = min(T, t0 + chunk);
  float s = 0.f;
  for (int64_t t = t0; t < t1; ++t) s += dn[t * L + l] * c[t * L + l] * r[t];
  part[(int64_t)blockIdx.y * L + l] = s;
}

// Sum of `rows` partial rows [rows, L] into out[L] (rows in order).
__global__ __launch_bounds__(256) void bw_sum_rows_kernel(const float* part, int rows, int L, float* out) {
  const int l = blockIdx.x * 256 + threadIdx.x;
  if (l >= L) return;
  float s = 0.f;
  for (int y = 0; y < rows; ++y) s += part[(int64_t)y * L + l];
  out[l] = s;
}

// Router: per token, dlogit = ds s (1 - s) at the selected experts (0
// elsewhere), ds_j = (dw_j - sum_j' dw_j' w_j') / S, S = sum of the selected
// sigmoid scores, w_j = s_j / S.
// dl16 (optional): the same row in bf16, the operand precision of the
// GEMMs that consume it.
__global__ __launch_bounds__(256) void bw_route_grad_kernel(const float* logits, const int32_t* idx, const float* dw,
                                                            int E, int k, float* dlogits, unsigned short* dl16) {
  const int64_t t = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) {
    dlogits[t * E + e] = 0.f;
    if (dl16) dl16[t * E + e] = 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float S = 0.f, dot = 0.f;
    for (int j = 0; j < k; ++j) S += bw_sigmoid(logits[t * E + idx[t * k + j]]);
    for (int j = 0; j < k; ++j) dot += dw[t * k + j] * bw_sigmoid(logits[t * E + idx[t * k + j]]) / S;
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      const float s = bw_sigmoid(logits[t * E + e]);
      const float d = (dw[t * k + j] - dot) / S * s * (1.f - s);
      dlogits[t * E + e] = d;
      if (dl16) dl16[t * E + e] = f2bf(d);
    }
  }
}

// dz_t = sum_j dzrows[pos(t, j)] (j ascending, fp32); written as fp32 to
// out32, or as bf16 to out16 (the next GEMM's operand).  Four consecutive
// elements per thread (L a multiple of 4).
__global__ __launch_bounds__(256) void bw_gather_sum_kernel(const float* rows, const int32_t* pos, int L, int k,
                                                            float* out32, unsigned short* out16) {
  const int64_t t = blockIdx.y;
  const int l = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (l >= L) return;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(rows + (int64_t)pos[t * k + j] * L + l);
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] += v[e];
  }
  if (out16)
    *reinterpret_cast<uint2*>(out16 + t * L + l) =
        uint2{f2bf(s[0]) | ((unsigned)f2bf(s[1]) << 16), f2bf(s[2]) | ((unsigned)f2bf(s[3]) << 16)};
  else
    *reinterpret_cast<f32x4*>(out32 + t * L + l) = s;
}

// bf16 -> fp32 of n elements.
__global__ __launch_bounds__(256) void bw_widen_kernel(const unsigned short* x, float* y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = __uint_as_float((unsigned)x[i] << 16);
}

}  // namespace lmoe
