// Router top-k, counting-sort permute, expert tile list and combine + RMSNorm.
//
// Sources: P1 aitrending.vip "The 2.8-Trillion-Parameter Problem", Technical
// Details (router keeps 16 of 896 experts; RMSNorm before the up-projection);
// P2 wpnews.pro, same title, MoE, Stable LatentMoE and stabilizer passages
// (selected experts' outputs are combined, then normalised, then projected
// back); P3 daily-ai-frontier "苏神复盘 Kimi K3", Merged summary (norm after
// expert aggregation).
#include <float.h>
#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace lmoe {

// ---------------------------------------------------------------------------
// Top-k: one wavefront per token.  Lane l holds experts l, l+64, ... as one
// 64-bit key each: the order-preserving image of the biased score s + b in
// the high word and the complement of the expert index in the low word, so
// the largest key is the largest score, lower index first on equal scores.
// NaN and -inf scores rank as -FLT_MAX: below every real expert, above
// padding and retired entries (key 0).  Each of the k rounds takes the
// wave's largest key with DPP steps inside each 16-lane row and scalar reads
// across the four rows, then retires the winner; all state stays in
// registers and no round needs an LDS round trip.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t topk_max(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t topk_dpp(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Largest key over the wave, the same value in every lane.
__device__ __forceinline__ uint64_t topk_wave_max(uint64_t v) {
  v = topk_max(v, topk_dpp<0xB1>(v));   // quad_perm [1,0,3,2]: lane ^ 1
  v = topk_max(v, topk_dpp<0x4E>(v));   // quad_perm [2,3,0,1]: lane ^ 2
  v = topk_max(v, topk_dpp<0x141>(v));  // row_half_mirror: the other quad of 8
  v = topk_max(v, topk_dpp<0x140>(v));  // row_mirror: the other half of 16
  uint64_t r = 0;
#pragma unroll
  for (int row = 0; row < 4; ++row) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, row * 16);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), row * 16);
    r = topk_max(r, ((uint64_t)hi << 32) | lo);
  }
  return r;
}

template <int NPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, const float* __restrict__ bias,
                                                   int64_t T, int E, int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + t * E;
  uint64_t key[NPL];
  float sc[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      const float s = 1.f / (1.f + expf(-row[e]));
      float v = s + bias[e];
      v = (v == v) ? fmaxf(v, -FLT_MAX) : -FLT_MAX;
      uint32_t b = __float_as_uint(v);
      b = b == 0x80000000u ? 0u : b;  // -0 ranks as +0 (equal scores)
      const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
      key[i] = ((uint64_t)ord << 32) | (uint32_t)~(uint32_t)e;
      sc[i] = s;
    } else {
      key[i] = 0;
      sc[i] = 0.f;
    }
  }
  int my_e = 0;
  float my_s = 0.f, ssum = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) best = topk_max(best, key[i]);
    best = topk_wave_max(best);
    const int be = (int)~(uint32_t)best;  // uniform across the wave
    const int wl = be & 63, wi = be >> 6;
    float s_w = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (i == wi) {
        s_w = sc[i];
        if (lane == wl) key[i] = 0;
      }
    const float bs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_w), wl));
    if (lane == j) {
      my_e = be;
      my_s = bs;
    }
    ssum += bs;
  }
  if (lane < k) {
    idx[t * k + lane] = my_e;
    wout[t * k + lane] = my_s / ssum;
  }
}

hipError_t launch_topk(const float* logits, const float* bias, int64_t T, int E, int k, int32_t* idx,
                       float* w, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  const int npl = (E + 63) / 64;
  if (npl <= 1) hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, st, logits, bias, T, E, k, idx, w);
  else if (npl <= 2) hipLaunchKernelGGL(topk_kernel<2>, grid, block, 0, st, logits, bias, T, E, k, idx, w);
  else if (npl <= 4) hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, st, logits, bias, T, E, k, idx, w);
  else if (npl <= 8) hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, st, logits, bias, T, E, k, idx, w);
  else hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, st, logits, bias, T, E, k, idx, w);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Permute: stable counting sort of the T*k assignments by expert.  A
// work-group covers 256 tokens (one per thread, 4 waves) and marks, per expert,
// the tokens that chose it in a 256-bit LDS mask (4 x 64 bits, one word per
// wave).  The mask's population gives the group's count per expert; the
// population of the lower bits gives a token's rank inside the group.  Group
// counts are scanned across groups per expert (in token order, so the sort is
// stable), then across experts for the offsets.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void perm_mark(const int32_t* __restrict__ idx, int64_t T, int E, int k,
                                          unsigned long long* mask, uint64_t* dup) {
  const int tid = threadIdx.x;
  for (int i = tid; i < E * 4; i += kPermTokens) mask[i] = 0ull;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kPermTokens + tid;
  const unsigned long long bit = 1ull << (tid & 63);
  const int w = tid >> 6;
  uint64_t d = 0;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e < 0 || e >= E) { d |= 1ull << j; continue; }
      const unsigned long long old = atomicOr(&mask[e * 4 + w], bit);
      if (old & bit) d |= 1ull << j;  // repeat of an expert already listed for this token
    }
  }
  *dup = d;
  __syncthreads();
}

__global__ __launch_bounds__(kPermTokens) void perm_count_kernel(const int32_t* __restrict__ idx, int64_t T, int E,
                                                                 int k, int32_t* __restrict__ bcounts) {
  extern __shared__ unsigned long long mask[];
  uint64_t dup;
  perm_mark(idx, T, E, k, mask, &dup);
  for (int e = threadIdx.x; e < E; e += kPermTokens)
    bcounts[(int64_t)blockIdx.x * E + e] = __popcll(mask[e * 4]) + __popcll(mask[e * 4 + 1]) +
                                           __popcll(mask[e * 4 + 2]) + __popcll(mask[e * 4 + 3]);
}

// One work-group: per expert, exclusive scan of the group counts in place;
// then exclusive scan of the expert totals into offsets.
__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t* __restrict__ bcounts, int nb, int E,
                                                         int32_t* __restrict__ offsets) {
  __shared__ int lds[1024 / 64 + 1];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int b = 0; b < nb; ++b) {
      const int c = bcounts[(int64_t)b * E + e];
      bcounts[(int64_t)b * E + e] = run;
      run += c;
    }
  }
  int total;
  const int ex = block_exclusive_scan<1024>(e < E ? run : 0, lds, &total);
  if (e < E) offsets[e] = ex;
  if (e == 0) offsets[E] = total;
}

__global__ __launch_bounds__(kPermTokens) void perm_scatter_kernel(const int32_t* __restrict__ idx, int64_t T, int E,
                                                                   int k, const int32_t* __restrict__ bprefix,
                                                                   const int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ sorted,
                                                                   int32_t* __restrict__ pos) {
  extern __shared__ unsigned long long mask[];
  uint64_t dup;
  perm_mark(idx, T, E, k, mask, &dup);
  const int tid = threadIdx.x;
  const int64_t t = (int64_t)blockIdx.x * kPermTokens + tid;
  if (t >= T) return;
  const int w = tid >> 6;
  const unsigned long long below = (1ull << (tid & 63)) - 1ull;
  for (int j = 0; j < k; ++j) {
    const int64_t a = t * k + j;
    if (dup >> j & 1ull) { pos[a] = -1; continue; }
    const int e = idx[a];
    int rank = __popcll(mask[e * 4 + w] & below);
    for (int q = 0; q < w; ++q) rank += __popcll(mask[e * 4 + q]);
    const int dst = offsets[e] + bprefix[(int64_t)blockIdx.x * E + e] + rank;
    sorted[dst] = (int32_t)a;
    pos[a] = dst;
  }
}

hipError_t launch_permute(const int32_t* idx, int64_t T, int E, int k, int32_t* bcounts, int32_t* offsets,
                          int32_t* sorted, int32_t* pos, hipStream_t st) {
  const int nb = (int)((T + kPermTokens - 1) / kPermTokens);
  const size_t lds = (size_t)E * 4 * sizeof(unsigned long long);
  if (nb > 0) {
    hipLaunchKernelGGL(perm_count_kernel, dim3(nb), dim3(kPermTokens), lds, st, idx, T, E, k, bcounts);
    if (hipError_t e = hipGetLastError()) return e;
  }
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, st, bcounts, nb, E, offsets);
  if (hipError_t e = hipGetLastError()) return e;
  if (nb > 0)
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(nb), dim3(kPermTokens), lds, st, idx, T, E, k, bcounts, offsets,
                       sorted, pos);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Tile list: expert e with c_e rows gets ceil(c_e / bt) token tiles; entry q
// = {e, first tile of e, tiles of e, 0}.  One work-group, one expert a thread.
// ---------------------------------------------------------------------------
__device__ void write_tiles(int e, int E, int c, int bt, int4* tiles, int32_t* cnt, int* lds) {
  const int nt = (e < E) ? (c + bt - 1) / bt : 0;
  int total;
  const int tb = block_exclusive_scan<1024>(nt, lds, &total);
  for (int q = 0; q < nt; ++q) tiles[tb + q] = int4{e, tb, nt, 0};
  if (threadIdx.x == 0) *cnt = total;
}

__global__ __launch_bounds__(1024) void tiles_kernel(const int32_t* __restrict__ offsets, int E, int bt_a,
                                                     int4* tiles_a, int32_t* cnt_a, int bt_b, int4* tiles_b,
                                                     int32_t* cnt_b) {
  __shared__ int lds[1024 / 64 + 1];
  const int e = threadIdx.x;
  const int c = e < E ? offsets[e + 1] - offsets[e] : 0;
  write_tiles(e, E, c, bt_a, tiles_a, cnt_a, lds);
  if (bt_b > 0) write_tiles(e, E, c, bt_b, tiles_b, cnt_b, lds);
}

// Permute and tile list of a batch of at most kPermTokens tokens in one
// work-group (decode-sized batches): the same marks, ranks, scans and tile
// entries as perm_count + perm_scan + perm_scatter + tiles_kernel with a
// single token group, in one launch instead of four.
__global__ __launch_bounds__(1024) void permute_small_kernel(const int32_t* __restrict__ idx, int64_t T, int E, int k,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ sorted, int32_t* __restrict__ pos,
                                                             int bt, int4* __restrict__ tiles,
                                                             int32_t* __restrict__ cnt) {
  extern __shared__ unsigned long long mask[];  // E x 4 words: tokens 64 w .. 64 w + 63 of expert e at e * 4 + w
  __shared__ int soff[1024];
  __shared__ int lds[1024 / 64 + 1];
  const int tid = threadIdx.x;
  for (int i = tid; i < E * 4; i += 1024) mask[i] = 0ull;
  __syncthreads();
  const bool tok = tid < kPermTokens && tid < T;
  const int w = tid >> 6;
  const unsigned long long bit = 1ull << (tid & 63);
  uint64_t dup = 0;
  if (tok) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[(int64_t)tid * k + j];
      if (e < 0 || e >= E) { dup |= 1ull << j; continue; }
      const unsigned long long old = atomicOr(&mask[e * 4 + w], bit);
      if (old & bit) dup |= 1ull << j;  // repeat of an expert already listed for this token
    }
  }
  __syncthreads();
  // expert tid: its count, then the exclusive scan over experts
  const int c = tid < E ? __popcll(mask[tid * 4]) + __popcll(mask[tid * 4 + 1]) + __popcll(mask[tid * 4 + 2]) +
                              __popcll(mask[tid * 4 + 3])
                        : 0;
  int total;
  const int ex = block_exclusive_scan<1024>(c, lds, &total);
  if (tid < E) {
    offsets[tid] = ex;
    soff[tid] = ex;
  }
  if (tid == 0) offsets[E] = total;
  __syncthreads();
  if (tok) {
    const unsigned long long below = bit - 1ull;
    for (int j = 0; j < k; ++j) {
      const int64_t a = (int64_t)tid * k + j;
      if (dup >> j & 1ull) { pos[a] = -1; continue; }
      const int e = idx[a];
      int rank = __popcll(mask[e * 4 + w] & below);
      for (int q = 0; q < w; ++q) rank += __popcll(mask[e * 4 + q]);
      const int dst = soff[e] + rank;
      sorted[dst] = (int32_t)a;
      pos[a] = dst;
    }
  }
  write_tiles(tid, E, c, bt, tiles, cnt, lds);
}

hipError_t launch_permute_small(const int32_t* idx, int64_t T, int E, int k, int32_t* offsets, int32_t* sorted,
                                int32_t* pos, int bt, int4* tiles, int32_t* cnt, hipStream_t st) {
  const size_t lds = (size_t)E * 4 * sizeof(unsigned long long);
  hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(1024), lds, st, idx, T, E, k, offsets, sorted, pos, bt,
                     tiles, cnt);
  return hipGetLastError();
}

hipError_t launch_tiles(const int32_t* offsets, int E, int bt_a, int4* tiles_a, int32_t* cnt_a, int bt_b,
                        int4* tiles_b, int32_t* cnt_b, hipStream_t st) {
  hipLaunchKernelGGL(tiles_kernel, dim3(1), dim3(1024), 0, st, offsets, E, bt_a, tiles_a, cnt_a, bt_b, tiles_b,
                     cnt_b);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine + RMSNorm: one work-group per token.  Thread c accumulates 16-byte
// chunks c, c+256, ... of the token's k expert rows (slot order j ascending)
// in fp32, the block reduces the sum of squares, and the normalised row is
// written in the activation dtype.
// ---------------------------------------------------------------------------
// The backward's recompute also takes the combined row c (fp32, c_out) and
// the row's 1/rms (r_out); the forward passes NULL for both.
template <typename CT, int MAXC>
__global__ __launch_bounds__(256) void combine_norm_kernel(const CT* __restrict__ O, const int32_t* __restrict__ pos,
                                                           const float* __restrict__ w,
                                                           const float* __restrict__ gamma, int L, int k, float eps,
                                                           CT* __restrict__ out, float* __restrict__ c_out,
                                                           float* __restrict__ r_out) {
  constexpr int EPC = 16 / sizeof(CT);
  typedef CT vec_t __attribute__((ext_vector_type(EPC)));
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int nch = L / EPC;
  float acc[MAXC][EPC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c)
#pragma unroll
    for (int i = 0; i < EPC; ++i) acc[c][i] = 0.f;
  // rows of JB assignments are loaded together (more loads in flight per
  // thread), then added in ascending j; a missing row (pos < 0) adds nothing
  constexpr int JB = 16 / MAXC;
  for (int j0 = 0; j0 < k; j0 += JB) {
    vec_t v[JB][MAXC];
    float wj[JB];
    bool ok[JB];
#pragma unroll
    for (int u = 0; u < JB; ++u) {
      const int p = j0 + u < k ? pos[t * k + j0 + u] : -1;
      ok[u] = p >= 0;
      wj[u] = ok[u] ? w[t * k + j0 + u] : 0.f;
      const CT* row = O + (int64_t)(ok[u] ? p : 0) * L;
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int ch = tid + c * 256;
        if (ok[u] && ch < nch) v[u][c] = *reinterpret_cast<const vec_t*>(row + ch * EPC);
      }
    }
#pragma unroll
    for (int u = 0; u < JB; ++u) {
      if (!ok[u]) continue;
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int ch = tid + c * 256;
        if (ch < nch) {
#pragma unroll
          for (int i = 0; i < EPC; ++i) acc[c][i] += wj[u] * to_f32(v[u][c][i]);
        }
      }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c)
#pragma unroll
    for (int i = 0; i < EPC; ++i) ss += acc[c][i] * acc[c][i];
  ss = wave_sum_f(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float inv = 1.f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)L + eps);
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int ch = tid + c * 256;
    if (ch < nch) {
      vec_t o;
#pragma unroll
      for (int i = 0; i < EPC; ++i) o[i] = from_f32<CT>(gamma[ch * EPC + i] * acc[c][i] * inv);
      *reinterpret_cast<vec_t*>(out + t * L + ch * EPC) = o;
      if (c_out) {
#pragma unroll
        for (int i = 0; i < EPC; i += 4)
          *reinterpret_cast<f32x4*>(c_out + t * L + ch * EPC + i) =
              f32x4{acc[c][i], acc[c][i + 1], acc[c][i + 2], acc[c][i + 3]};
      }
    }
  }
  if (r_out && tid == 0) r_out[t] = inv;
}

hipError_t launch_combine_norm(bool bf16_act, const void* O, const int32_t* pos, const float* w, const float* gamma,
                               int64_t T, int L, int k, float eps, void* n, hipStream_t st, float* c_out,
                               float* r_out) {
  if (T == 0) return hipSuccess;
  if (bf16_act && L <= 2 * 256 * 8)
    hipLaunchKernelGGL((combine_norm_kernel<bf16, 2>), dim3((unsigned)T), dim3(256), 0, st, (const bf16*)O, pos, w,
                       gamma, L, k, eps, (bf16*)n, c_out, r_out);
  else if (bf16_act)
    hipLaunchKernelGGL((combine_norm_kernel<bf16, 4>), dim3((unsigned)T), dim3(256), 0, st, (const bf16*)O, pos, w,
                       gamma, L, k, eps, (bf16*)n, c_out, r_out);
  else
    hipLaunchKernelGGL((combine_norm_kernel<float, 8>), dim3((unsigned)T), dim3(256), 0, st, (const float*)O, pos, w,
                       gamma, L, k, eps, (float*)n, c_out, r_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Quantile Balancing thresholds: tau_e = (1 - k/E) quantile over the batch of
// expert e's sigmoid scores, linear between the order statistics floor(h) and
// floor(h) + 1 with h = (T - 1)(1 - k/E); bias_e = -tau_e.
// ---------------------------------------------------------------------------
// Order-preserving fp32 <-> uint32 keys (unsigned key order = numeric order).
__device__ __forceinline__ uint32_t f2key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k); }

// logits [T, E] -> keys [E, T] of sigmoid(logit), through a 64 x 64 LDS tile
// (coalesced reads along E, coalesced writes along T).
__global__ __launch_bounds__(256) void qb_keys_kernel(const float* logits, int64_t T, int E, uint32_t* keys) {
  __shared__ uint32_t tile[64][65];
  const int tid = threadIdx.x;
  const int e0 = blockIdx.x * 64;
  const int64_t t0 = (int64_t)blockIdx.y * 64;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = (tid >> 6) + 4 * i, c = tid & 63;
    const int64_t t = t0 + r;
    const int e = e0 + c;
    if (t < T && e < E) tile[r][c] = f2key(1.f / (1.f + expf(-logits[t * E + e])));
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = (tid >> 6) + 4 * i, r = tid & 63;
    const int64_t t = t0 + r;
    const int e = e0 + c;
    if (t < T && e < E) keys[(int64_t)e * T + t] = tile[r][c];
  }
}

// Keys of an expert held in LDS by the select kernel (64 KB); longer batches
// are read from global memory in every pass.
constexpr int64_t kQbLdsKeys = 16384;

// Inclusive sum over the 256 threads of a work-group (4 waves).
__device__ __forceinline__ uint32_t qb_block_scan(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  for (int i = 0; i < w; ++i) v += wsum[i];
  return v;
}

// One work-group per expert: the lower order statistic s_(lo) by radix
// selection (4 passes of 8 bits, most significant first) over the expert's
// keys, held in LDS; then s_(lo+1), which is the same key when enough keys
// tie with it and otherwise the smallest key above it (one more pass).
__global__ __launch_bounds__(256) void qb_select_kernel(const uint32_t* keys, int64_t T, int E, int k, float* bias) {
  extern __shared__ uint32_t sk[];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[4];
  __shared__ int64_t rank_s;
  __shared__ uint32_t bin_s, min_s[4];
  const int tid = threadIdx.x;
  const int e = blockIdx.x;
  const uint32_t* col = keys + (int64_t)e * T;
  const bool inl = T <= kQbLdsKeys;
  if (inl)
    for (int64_t t = tid; t < T; t += 256) sk[t] = col[t];
  const double h = (double)(T - 1) * (1.0 - (double)k / (double)E);
  const int64_t lo = (int64_t)floor(h);
  const int64_t hi = lo + 1 < T ? lo + 1 : T - 1;
  int64_t r = lo;  // 0-based rank among the keys that match the prefix
  uint32_t prefix = 0, mask = 0, ties = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int64_t t = tid; t < T; t += 256) {
      const uint32_t v = inl ? sk[t] : col[t];
      if ((v & mask) == prefix) atomicAdd(&hist[(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    const uint32_t c = hist[tid];
    const uint32_t incl = qb_block_scan(c, wsum);
    const uint32_t excl = incl - c;
    if ((int64_t)excl <= r && r < (int64_t)incl) {
      bin_s = (uint32_t)tid;
      rank_s = r - (int64_t)excl;
    }
    __syncthreads();
    prefix |= bin_s << shift;
    mask |= 255u << shift;
    r = rank_s;
    ties = hist[bin_s];  // after the last pass: the keys equal to s_(lo)
    __syncthreads();
  }
  const uint32_t klo = prefix;
  uint32_t khi = klo;
  if (hi != lo && r + 1 >= (int64_t)ties) {
    // s_(lo+1) is the smallest key above s_(lo)
    uint32_t m = 0xffffffffu;
    for (int64_t t = tid; t < T; t += 256) {
      const uint32_t v = inl ? sk[t] : col[t];
      if (v > klo && v < m) m = v;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) m = min(m, (uint32_t)__shfl_xor(m, d));
    if ((tid & 63) == 0) min_s[tid >> 6] = m;
    __syncthreads();
    khi = min(min(min_s[0], min_s[1]), min(min_s[2], min_s[3]));
  }
  if (tid == 0) {
    const double xl = key2f(klo), xh = key2f(khi);
    bias[e] = (float)(-(xl + (h - (double)lo) * (xh - xl)));
  }
}

hipError_t launch_quantile_bias(const float* logits, int64_t T, int E, int k, uint32_t* keys, float* bias,
                                hipStream_t st) {
  if (T <= 0 || (T + 63) / 64 > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(qb_keys_kernel, dim3((unsigned)((E + 63) / 64), (unsigned)((T + 63) / 64)), dim3(256), 0, st,
                     logits, T, E, keys);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = T <= kQbLdsKeys ? (size_t)T * 4 : 0;
  hipLaunchKernelGGL(qb_select_kernel, dim3((unsigned)E), dim3(256), lds, st, keys, T, E, k, bias);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// W8A8 activations: per row, per 128 consecutive columns, scale = amax / 448
// in fp32 (1 for an all-zero block) and code = e4m3fn(x / scale): a correctly
// rounded fp32 division, then the hardware conversion, which rounds to
// nearest even.  Every |x / scale| <= 448 up to one rounding of the quotient,
// which the conversion rounds back to 448.  Sixteen lanes share one block,
// eight values each (bf16: one 16-byte load; fp32: two), one 8-byte store.
// The fp32 form reads the layer's own activations as the GEMMs accumulated
// them, so the code decisions see no intermediate rounding.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load8(const uint16_t* p, float (&f)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&f)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x, f[1] = a.y, f[2] = a.z, f[3] = a.w, f[4] = b.x, f[5] = b.y, f[6] = b.z, f[7] = b.w;
}

template <typename In>
__global__ __launch_bounds__(256) void quant_1x128_kernel(const In* __restrict__ x, int64_t R, int C,
                                                          uint8_t* __restrict__ q, float* __restrict__ sc) {
  const int nb = C >> 7;
  const int64_t unit = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // (row, block)
  if (unit >= R * nb) return;  // whole 16-lane groups leave together
  const int64_t r = unit / nb;
  const int b = (int)(unit - r * nb);
  const int sub = threadIdx.x & 15;
  const int64_t off = r * C + b * 128 + sub * 8;
  float f[8];
  load8(x + off, f);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
  const float s = amax > 0.f ? amax / 448.f : 1.f;
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0] / s, f[1] / s, 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2] / s, f[3] / s, lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4] / s, f[5] / s, 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6] / s, f[7] / s, hi, true);
  *reinterpret_cast<uint2*>(q + off) = uint2{(unsigned)lo, (unsigned)hi};
  if (sub == 0) sc[(int64_t)b * R + r] = s;
}
hipError_t launch_quant_1x128(const void* x, bool x_f32, int64_t R, int C, void* q, float* sc, hipStream_t st) {
  const int64_t units = R * (C / 128);
  if (units == 0) return hipSuccess;
  const int64_t blocks = (units + 15) / 16;
  if (blocks > INT_MAX) return hipErrorInvalidValue;
  if (x_f32)
    hipLaunchKernelGGL(quant_1x128_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const float*>(x), R, C, static_cast<uint8_t*>(q), sc);
  else
    hipLaunchKernelGGL(quant_1x128_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), R, C, static_cast<uint8_t*>(q), sc);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void gather_scales_kernel(const float* __restrict__ s_tok, int64_t T, int nb,
                                                            const int32_t* __restrict__ sorted, int64_t tk, int k,
                                                            float* __restrict__ out) {
  const int64_t a = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (a >= tk) return;
  // entries past the last expert's range may hold anything: clamp the token
  const int64_t t = min(max((int64_t)(sorted[a] / k), (int64_t)0), T - 1);
  for (int b = 0; b < nb; ++b) out[b * tk + a] = s_tok[b * T + t];
}

hipError_t launch_gather_scales(const float* s_tok, int64_t T, int nb, const int32_t* sorted, int k, float* out,
                                hipStream_t st) {
  const int64_t tk = T * k;
  if (tk == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_scales_kernel, dim3((unsigned)((tk + 255) / 256)), dim3(256), 0, st, s_tok, T, nb, sorted,
                     tk, k, out);
  return hipGetLastError();
}

}  // namespace lmoe
