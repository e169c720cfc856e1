// Shared device helpers for the Stable Latent MoE kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lmoe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

enum Dtype : int { DT_F32 = 0, DT_BF16 = 1, DT_F8 = 2 };

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, WGs dealt round-robin
// Packed expert weights: one block = 256 rows x 64 bf16 columns (32 KB), the
// on-chip image of one weight tile of the expert GEMMs.
constexpr int kPackRows = 256;
constexpr int kPackBlock = kPackRows * 128;

__host__ __device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }  // RNE

// SiTU-GLU: silu(cap(g)) * cap(v), cap(u) = c * tanh(u / c); an infinite cap
// (inv_c == 0) leaves g and v unchanged (plain SwiGLU).
__device__ __forceinline__ float situ_cap(float u, float c, float inv_c) {
  return inv_c == 0.f ? u : c * tanhf(u * inv_c);
}
__device__ __forceinline__ float situ_glu(float g, float v, float c, float inv_c) {
  const float gc = situ_cap(g, c, inv_c);
  const float vc = situ_cap(v, c, inv_c);
  return gc / (1.f + expf(-gc)) * vc;
}

// Uniform reads, through the scalar cache, of index data that no kernel in
// flight writes (expert tile list, offsets, the sorted assignment order).
// Each returns with the value loaded (the wait is inside), so no vector-memory
// counter is involved: the GEMM main loops' DMA accounting stays exact and no
// compiler-inserted vmcnt(0) drains their pipeline.  Reads only.
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
// Every address passed to these loads is wave-uniform by construction; the
// compiler's divergence analysis does not always prove it, so the address is
// taken from the first lane, which places it in scalar registers.
__device__ __forceinline__ const int* su(const int* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const int*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int sload1(const int* p) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(su(p)) : "memory");
  return v;
}
__device__ __forceinline__ i32x2 sload2(const int* p) {
  i32x2 v;
  asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(su(p)) : "memory");
  return v;
}
__device__ __forceinline__ i32x4 sload4(const int* p) {
  i32x4 v;
  asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(su(p)) : "memory");
  return v;
}
// Two uniform ints *a, *b in one round trip.
__device__ __forceinline__ i32x2 sload_pair(const int* a, const int* b) {
  int v0, v1;
  asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(v0), "=&s"(v1)
               : "s"(su(a)), "s"(su(b))
               : "memory");
  i32x2 v = {v0, v1};
  return v;
}
// Eight uniform ints p[idx[0..7]] (any addresses) in one round trip.
__device__ __forceinline__ i32x8 sload_gather8(const int* p, const int (&idx)[8]) {
  int v0, v1, v2, v3, v4, v5, v6, v7;
  asm volatile(
      "s_load_dword %0, %8, 0x0\n\ts_load_dword %1, %9, 0x0\n\ts_load_dword %2, %10, 0x0\n\t"
      "s_load_dword %3, %11, 0x0\n\ts_load_dword %4, %12, 0x0\n\ts_load_dword %5, %13, 0x0\n\t"
      "s_load_dword %6, %14, 0x0\n\ts_load_dword %7, %15, 0x0\n\ts_waitcnt lgkmcnt(0)"
      : "=&s"(v0), "=&s"(v1), "=&s"(v2), "=&s"(v3), "=&s"(v4), "=&s"(v5), "=&s"(v6), "=&s"(v7)
      : "s"(su(p + idx[0])), "s"(su(p + idx[1])), "s"(su(p + idx[2])), "s"(su(p + idx[3])), "s"(su(p + idx[4])),
        "s"(su(p + idx[5])), "s"(su(p + idx[6])), "s"(su(p + idx[7]))
      : "memory");
  i32x8 v = {v0, v1, v2, v3, v4, v5, v6, v7};
  return v;
}

// Work-group id -> logical index so that each XCD receives a contiguous range
// of logical tiles (neighbouring tiles share operands in that XCD's L2).
// `padded` is a multiple of kXcds and the grid size.
__device__ __forceinline__ int xcd_remap(int bid, int padded) {
  const int per = padded / kXcds;
  return (bid % kXcds) * per + bid / kXcds;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64, <= 1024).
// `lds` holds NT/64 + 1 ints.  Returns the exclusive prefix; *total = block sum.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(inc, o);
    if (lane >= o) inc += u;
  }
  if (lane == 63) lds[wid] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < NT / 64; ++w) {
      const int c = lds[w];
      lds[w] = run;
      run += c;
    }
    lds[NT / 64] = run;
  }
  __syncthreads();
  const int ex = lds[wid] + inc - v;
  *total = lds[NT / 64];
  __syncthreads();
  return ex;
}

}  // namespace lmoe
