// MFMA GEMM core for the Stable Latent MoE layer (gfx950).
//
// Every GEMM of the layer has the form  C[t, f] = sum_k X[t, k] * W[f, k]  with
// both operands K-contiguous (activations [tokens, K], weights [features, K]).
// A work-group owns a BF x BT tile (features x tokens).  Per k-tile (128 bytes
// of K per row) the work-group stages the W and X rows into LDS (double
// buffered through registers: the global loads of k-tile kt+1 are in flight
// while the MFMAs of k-tile kt run), then each wave multiplies its
// (BF/WF) x (BT/WT) sub-tile with 32x32 MFMA blocks: v_mfma_f32_32x32x16_bf16
// for bf16 operands, v_mfma_f32_32x32x2_f32 for fp32.  The weight operand sits
// in the MFMA's A slot, so each lane's accumulator holds 4 consecutive
// features of one token: stores are 8/16-byte packets along the output row.
//
// e4m3 weights are widened in the LDS store path (two codes per
// v_cvt_pk_f32_fp8, times the block scale, rounded to bf16), so the MFMA
// always sees bf16.  A "problem" object supplies the tile coordinates, the row
// addresses of both operands for each K-segment, and the epilogue.
#pragma once

#include "common.hpp"

namespace lmoe {

constexpr int kPitch = 144;  // LDS bytes per staged row: 128 data + 16 pad

template <int BF_, int BT_, int WF_, int WT_>
struct TileCfg {
  static constexpr int BF = BF_, BT = BT_, WF = WF_, WT = WT_;
  static constexpr int NT = WF * WT * kWave;
  static constexpr int FW = BF / WF, TW = BT / WT;
  static constexpr int FI = FW / 32, TI = TW / 32;
  static constexpr int CW = BF * 8 / NT;  // 16-byte LDS chunks per thread, W tile
  static constexpr int CX = BT * 8 / NT;  // same, X tile
  static constexpr int LDS = 2 * (BF + BT) * kPitch;
  static constexpr bool kDma = false;
  static constexpr int kKind = 1;
  static constexpr int XF8 = 0;  // tokens are never e4m3 here
  static_assert(FW % 64 == 0, "a wave covers whole gate/value pairs");
  static_assert(TW % 32 == 0 && CW >= 1 && CX >= 1, "tile shape");
  static_assert((BF * 8) % NT == 0 && (BT * 8) % NT == 0, "chunk split");
};

// Big tiles for prefill-sized token counts, small ones for decode / sparse experts.
typedef TileCfg<128, 128, 2, 2> CfgBig;
typedef TileCfg<128, 32, 2, 1> CfgSmall;

enum Epi : int { EPI_F32 = 0, EPI_STORE = 1, EPI_GLU = 2 };

// ---------------------------------------------------------------------------
// Stores of 4 consecutive outputs (features f..f+3 of one token row).
// ---------------------------------------------------------------------------
template <typename OT>
__device__ __forceinline__ void store4(OT* row, int f, const float* v, int fvalid, bool vec) {
  if (vec && f + 3 < fvalid) {
    if constexpr (sizeof(OT) == 4) {
      *reinterpret_cast<f32x4*>(row + f) = f32x4{v[0], v[1], v[2], v[3]};
    } else {
      bf16x4 p = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
      *reinterpret_cast<bf16x4*>(row + f) = p;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (f + j < fvalid) row[f + j] = from_f32<OT>(v[j]);
  }
}

// bf16 outputs, 16 bytes per lane.  In a 32x32 MFMA block, lanes l and l + 32
// hold the same output row: of the 16 features b .. b + 15 that accumulator
// groups 2h and 2h + 1 cover, lane l has b .. b+3 (va) and b+8 .. b+11 (vb),
// lane l + 32 has b+4 .. b+7 and b+12 .. b+15.  One exchange between the
// half-waves leaves b .. b+7 with lane l and b+8 .. b+15 with lane l + 32, so
// a wave stores a row's 16 features with one 16-byte store per lane instead
// of two 8-byte ones (half the store instructions, each covering 32 bytes
// of a row).  The values and their rounding are those of store4.  Every lane
// of the wave calls it (the exchange reads the partner lane); `ok` says
// whether the row is stored and is the same for both lanes of a pair.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {(bf16)a, (bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
// a0, a1 are va packed in pairs by pack_bf16x2, b0, b1 likewise vb.
__device__ __forceinline__ void store16_pair(bf16* row, int b, uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                             int fvalid, bool ok, bool vec, int lane) {
  // v_permlane32_swap trades the upper half-wave of its first operand with
  // the lower half-wave of its second: afterwards lane l < 32 holds its own a
  // and lane l + 32's a, lane l + 32 holds lane l's b and its own b.
  const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
  if (!ok) return;
  const uint32_t w[4] = {s0[0], s1[0], s0[1], s1[1]};
  const int f = b + (lane >= 32 ? 8 : 0);
  if (vec && f + 7 < fvalid) {
    *reinterpret_cast<uint4*>(row + f) = uint4{w[0], w[1], w[2], w[3]};
  } else {
    uint16_t* r16 = reinterpret_cast<uint16_t*>(row);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (f + e < fvalid) r16[f + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
  }
}

// ---------------------------------------------------------------------------
// Problem: x-GEMM (router logits, latent z, shared-expert gate/value) -- one
// GEMM over x with the weight matrices concatenated along the features.
// ---------------------------------------------------------------------------
struct NSeg {
  const char* w;      // [rows, K] (GLU: gate matrix)
  const char* w2;     // GLU: value matrix
  const float* sc;    // e4m3 block scales of w / w2, [rows/128, K/128]
  const float* sc2;
  char* out;          // output matrix
  int64_t ldo;        // its leading dimension, elements
  int col0;           // first output column
  int rows;           // features (GLU: units)
  int ft0;            // first feature tile of this segment
  int kind;           // Epi
  int f8;             // weights are e4m3 codes
  int vec;            // output rows allow vector stores
};

// Tile walk of a dense GEMM.  The output is cut into big tiles (the main
// launch's tile size), numbered with 8 token tiles per group and the feature
// tiles running over the group, so 8 neighbours share one weight tile.  A
// launch covers big tiles first .. first + count - 1, each as sf x st
// sub-tiles (sf along the features, st along the tokens; 1 x 1 = the big tile
// itself): the tail launch re-cuts the last, partial wave of big tiles into
// smaller tiles so that it spreads over every CU.  Every tile runs the same
// k-tile sequence, so an output element's sum is the same in any tile shape.
struct DenseWalk {
  int nft, ntt;       // big-tile grid: feature tiles, token tiles
  int first, count;   // big tiles of this launch
  int sf, st;         // sub-tiles per big tile
  __device__ int num_logical() const { return count * sf * st; }
  __host__ __device__ bool map(int lg, int& ttb, int& ftb, int& qf, int& qt) const {
    const int n = sf * st;
    if (lg >= count * n) return false;
    const int b = first + lg / n, q = lg - (lg / n) * n;
    const int grp = b / (8 * nft);
    const int gsz = min(8, ntt - grp * 8);
    const int within = b - grp * 8 * nft;
    ftb = within / gsz;
    ttb = grp * 8 + within % gsz;
    qf = q % sf;
    qt = q / sf;
    return true;
  }
};

template <class Cfg, typename CT>
struct DenseXProb {
  static constexpr bool kDenseRows = true;  // rows past T: loaded from row 0, never stored
  const char* x;
  int64_t T;
  int K;              // H
  int nseg, padded;
  DenseWalk walk;
  float cap, inv_cap;
  NSeg seg[3];        // ft0: first big feature tile of the segment

  struct State {
    int tt, f0;       // token tile, first feature (GLU: unit) of the tile
    NSeg s;           // its feature segment
  };

  __device__ bool setup(int bid, State& st) const {
    if (bid >= padded) return false;
    return setup_lg(xcd_remap(bid, padded), st);
  }
  __device__ int num_logical() const { return walk.num_logical(); }
  // logical tile -> (token tile, feature tile) of this launch's tile size;
  // an XCD's window of neighbours covers a few weight tiles
  __device__ bool setup_lg(int lg, State& st) const {
    int ttb, ftb, qf, qt;
    if (!walk.map(lg, ttb, ftb, qf, qt)) return false;
    st.tt = ttb * walk.st + qt;
    // constant indices only: the argument block stays in kernarg memory
    st.s = seg[0];
    if (nseg > 1 && ftb >= seg[1].ft0) st.s = seg[1];
    if (nseg > 2 && ftb >= seg[2].ft0) st.s = seg[2];
    const int per = st.s.kind == EPI_GLU ? Cfg::BF / 2 : Cfg::BF;
    st.f0 = ((ftb - st.s.ft0) * walk.sf + qf) * per;
    return true;
  }
  __device__ int num_ksegs() const { return 1; }
  __device__ int seg_ktiles(int) const { return K * (int)sizeof(CT) / 128; }
  __device__ bool seg_f8(const State& st, int) const { return st.s.f8; }
  __device__ int tokens_valid(const State& st) const { return (int)imin64(Cfg::BT, T - (int64_t)st.tt * Cfg::BT); }
  __device__ int feats_valid(const State& st) const {
    // GLU tiles interleave gate/value blocks: missing units load as zeros.
    const NSeg& s = st.s;
    return s.kind == EPI_GLU ? Cfg::BF : min(Cfg::BF, s.rows - st.f0);
  }
  __device__ const char* x_row(const State& st, int, int r) const {
    const int64_t t = (int64_t)st.tt * Cfg::BT + r;
    return t < T ? x + t * K * (int64_t)sizeof(CT) : nullptr;
  }
  __device__ const char* x_row_grp(const State& st, int s, int r0, int lane) const {
    return x_row(st, s, min(r0 + (lane >> 3), tokens_valid(st) - 1));
  }
  __device__ const char* w_row(const State& st, int, int r, const float** scrow) const {
    const NSeg& s = st.s;
    const int64_t wes = s.f8 ? 1 : sizeof(CT);
    const char* base = s.w;
    const float* sb = s.sc;
    int u;
    if (s.kind == EPI_GLU) {
      const int m = r & 63;
      u = st.f0 + (r >> 6) * 32 + (m & 31);
      if (m >= 32) { base = s.w2; sb = s.sc2; }
    } else {
      u = st.f0 + r;
    }
    if (u >= s.rows) {
      // Row 0 stands in for every missing row of its tile.  A re-cut
      // sub-tile can lie wholly past the segment (the second half of a last
      // big tile with <= BF/2 rows): its stand-in is then the segment's
      // first row, so its DMAs read in bounds; nothing computed from them is
      // stored.
      if (r != 0) return nullptr;
      u = 0;
      base = s.w;
      sb = s.sc;
    }
    if (s.f8) *scrow = sb + (int64_t)(u >> 7) * (K >> 7);
    return base + (int64_t)u * K * wes;
  }
  __device__ const char* w_block(const State&) const { return nullptr; }
  template <class Acc>
  __device__ __forceinline__ void epilogue(const State& st, const Acc& acc, int wf0, int wt0, int lane) const;
};

// ---------------------------------------------------------------------------
// Problem: up-projection + shared-expert down-projection, one GEMM with the K
// ranges concatenated: y = [n | hs] . [W_up | W_so[0] | ... ]^T (+ addend).
// ---------------------------------------------------------------------------
struct KSeg {
  const char* x;      // activations of this K range, rows of ldx elements
  int64_t ldx;
  const char* w;      // weights [N, K_seg], rows of ldw elements
  int64_t ldw;
  const float* sc;    // e4m3 scales [N/128, ldw/128]
  int nkt;            // k-tiles in this range
  int f8;
};

template <class Cfg, typename CT>
struct UpProb {
  static constexpr bool kDenseRows = true;  // rows past T: never stored
  int64_t T;
  int N;              // H
  int nks, padded;
  DenseWalk walk;
  char* y;
  const char* addend; // [T, N] act dtype, or null (identity up-projection adds n)
  int vec;
  KSeg ks[9];

  struct State {
    int tt, ft;
  };

  __device__ bool setup(int bid, State& st) const {
    if (bid >= padded) return false;
    return setup_lg(xcd_remap(bid, padded), st);
  }
  __device__ int num_logical() const { return walk.num_logical(); }
  __device__ bool setup_lg(int lg, State& st) const {
    int ttb, ftb, qf, qt;
    if (!walk.map(lg, ttb, ftb, qf, qt)) return false;
    st.ft = ftb * walk.sf + qf;
    st.tt = ttb * walk.st + qt;
    return true;
  }
  __device__ int num_ksegs() const { return nks; }
  __device__ int seg_ktiles(int s) const { return ks[s].nkt; }
  __device__ bool seg_f8(const State&, int s) const { return ks[s].f8; }
  __device__ int tokens_valid(const State& st) const { return (int)imin64(Cfg::BT, T - (int64_t)st.tt * Cfg::BT); }
  __device__ int feats_valid(const State& st) const { return min(Cfg::BF, N - st.ft * Cfg::BF); }
  __device__ const char* x_row(const State& st, int s, int r) const {
    const int64_t t = (int64_t)st.tt * Cfg::BT + r;
    return t < T ? ks[s].x + t * ks[s].ldx * (int64_t)sizeof(CT) : nullptr;
  }
  __device__ const char* x_row_grp(const State& st, int s, int r0, int lane) const {
    return x_row(st, s, min(r0 + (lane >> 3), tokens_valid(st) - 1));
  }
  __device__ const char* w_row(const State& st, int s, int r, const float** scrow) const {
    int f = st.ft * Cfg::BF + r;
    if (f >= N) {
      // row 0 of a re-cut sub-tile wholly past N (the stand-in for its
      // missing rows): the first row, so that its DMAs read in bounds
      if (r != 0) return nullptr;
      f = 0;
    }
    const KSeg& q = ks[s];
    if (q.f8) {
      *scrow = q.sc + (int64_t)(f >> 7) * (q.ldw >> 7);
      return q.w + (int64_t)f * q.ldw;
    }
    return q.w + (int64_t)f * q.ldw * (int64_t)sizeof(CT);
  }
  __device__ const char* w_block(const State&) const { return nullptr; }
  template <class Acc>
  __device__ __forceinline__ void epilogue(const State& st, const Acc& acc, int wf0, int wt0, int lane) const;
};

// ---------------------------------------------------------------------------
// Problems over the expert tile list.  Entry q of `tiles` = {e, first tile of
// e, tiles of e, 0}; an expert's tiles are consecutive.  Logical work index
// -> (expert, feature tile, token tile) with the token tiles innermost, so
// work-groups that share one weight slab run next to each other on one XCD.
// ---------------------------------------------------------------------------
struct ExpertState {
  int e, ft, m0, rows;
};

template <class Cfg>
struct ExpertTiles {
  const int* offsets;
  const int4* tiles;
  const int* tile_count;
  int nft;

  __device__ int num_logical() const { return sload1(tile_count) * nft; }
  __device__ bool locate(int bid, ExpertState& st) const {
    const int R = num_logical();
    const int per = (R + kXcds - 1) / kXcds;
    if (bid >= per * kXcds) return false;
    return locate_lg((bid % kXcds) * per + bid / kXcds, R, st);
  }
  __device__ bool locate_lg(int lg, int R, ExpertState& st) const {
    if (lg >= R) return false;
    const i32x4 te = sload4(reinterpret_cast<const int*>(tiles + lg / nft));
    const int local = lg - te.y * nft;
    st.ft = local / te.z;
    const int mt = local - st.ft * te.z;
    st.e = te.x;
    const i32x2 ob = sload2(offsets + st.e);
    st.m0 = ob.x + mt * Cfg::BT;
    st.rows = min(Cfg::BT, ob.y - st.m0);
    return st.rows > 0;
  }
};

// RAW = 1: the epilogue stores the gate and value pre-activations (fp32,
// graw / vraw [T*k, I] in assignment order) instead of their SiTU-GLU.
// RAW = 2: the SiTU-GLU output is stored in fp32 (W8A8: the quantiser's input).
template <class Cfg, typename CT, int RAW = 0>
struct ExpertGVProb {
  ExpertTiles<Cfg> et;
  const char* z;      // [T, ldz]
  int64_t ldz;
  const int* sorted;
  const char* wg;     // [E, I, L]
  const char* wv;
  const float* sg;    // [E, I/128, L/128]
  const float* sv;
  char* act;          // [T*k, I] act dtype (fp32 with RAW = 2)
  float* graw;        // RAW = 1: [T*k, I]
  float* vraw;
  const char* wpk;    // packed gate/value blocks (see lmoe_pack_experts) or NULL
  const float* xs;    // W8A8: z block scales in expert order, [L/128, ldxs]
  int64_t ldxs;
  int I, L, k, f8, a8;  // a8: z holds e4m3 codes (W8A8)
  float cap, inv_cap;

  typedef ExpertState State;
  __device__ bool setup(int bid, State& st) const { return et.locate(bid, st); }
  __device__ int num_logical() const { return et.num_logical(); }
  __device__ bool setup_lg(int lg, State& st) const { return et.locate_lg(lg, et.num_logical(), st); }
  __device__ int num_ksegs() const { return 1; }
  __device__ int seg_ktiles(int) const { return L * (int)sizeof(CT) / 128; }
  __device__ bool seg_f8(const State&, int) const { return f8; }
  __device__ int tokens_valid(const State& st) const { return st.rows; }
  // GLU rows: 64-row groups of 32 gate and 32 value rows of one 32-unit
  // range, so a wave's rows [wf0, wf0 + FW) hold only valid units iff
  // wf0 + FW <= 2 * (units left in the tile).  The raw-output instantiation
  // reports that (its epilogue stores are counted past the next wait, which
  // needs every counted block's stores issued); the others keep the whole
  // tile (missing units load as zeros and are never stored).
  __device__ int feats_valid(const State& st) const {
    if constexpr (RAW == 1) return min(Cfg::BF, 2 * (I - st.ft * (Cfg::BF / 2)));
    return Cfg::BF;
  }
  // RAW = 1: vector stores per wave per fully valid 32-row token block (a
  // gate and a value store4 per accumulator group)
  static constexpr int kEpiStores = RAW == 1 ? Cfg::FI * 4 : 0;
  __device__ int64_t xes() const { return a8 ? 1 : (int64_t)sizeof(CT); }
  __device__ const char* x_row(const State& st, int, int r) const {
    if (r >= st.rows) return nullptr;
    const int t = sorted[st.m0 + r] / k;
    return z + (int64_t)t * ldz * xes();
  }
  // Row r0 + lane / (64 / RPI) for r0 < rows (rows past the valid ones map to
  // the last valid row): the group's RPI assignment ids are read as uniform
  // scalars, so the call needs no vector-memory wait.
  template <int RPI = 8>
  __device__ const char* x_row_grp(const State& st, int, int r0, int lane) const {
    static_assert(RPI == 8 || RPI == 16, "8 or 16 rows per DMA instruction");
    const int q = lane / (64 / RPI);
    int a = 0;
#pragma unroll
    for (int h = 0; h < RPI / 8; ++h) {
      int idx[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) idx[u] = st.m0 + min(r0 + 8 * h + u, st.rows - 1);
      const i32x8 v = sload_gather8(sorted, idx);
#pragma unroll
      for (int u = 0; u < 8; ++u) a = q == 8 * h + u ? v[u] : a;
    }
    return z + (int64_t)(a / k) * ldz * xes();
  }
  // W8A8: scales of 128-column block kb of this tile's rows (row r at + r)
  __device__ const float* x_scale(const State& st, int kb) const { return xs + kb * ldxs + st.m0; }
  __device__ const char* w_row(const State& st, int, int r, const float** scrow) const {
    const int m = r & 63;
    const int u = st.ft * (Cfg::BF / 2) + (r >> 6) * 32 + (m & 31);
    if (u >= I) return nullptr;  // last tile of an I that is not a multiple of BF/2
    const bool val = m >= 32;
    const int64_t wes = f8 ? 1 : sizeof(CT);
    const int64_t off = ((int64_t)st.e * I + u) * L * wes;
    if (f8) *scrow = (val ? sv : sg) + ((int64_t)st.e * (I >> 7) + (u >> 7)) * (L >> 7);
    return (val ? wv : wg) + off;
  }
  // e4m3 block scales of the 32-row blocks r0 + 32 i (i < N) at 128-column
  // block kb: a block's rows are all gate or all value rows of one 128-unit
  // block (read through the scalar cache).
  template <int N>
  __device__ void w_scales(const State& st, int r0, int kb, float (&sc)[N]) const {
    const float* p[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int r = r0 + 32 * i, m = r & 63;
      const int u = st.ft * (Cfg::BF / 2) + (r >> 6) * 32;
      p[i] = (m >= 32 ? sv : sg) + ((int64_t)st.e * (I >> 7) + (u >> 7)) * (L >> 7) + kb;
    }
#pragma unroll
    for (int i = 0; i < N; i += 2) {
      if (i + 1 < N) {
        const i32x2 v = sload_pair(reinterpret_cast<const int*>(p[i]), reinterpret_cast<const int*>(p[i + 1]));
        sc[i] = __int_as_float(v.x);
        sc[i + 1] = __int_as_float(v.y);
      } else {
        sc[i] = __int_as_float(sload1(reinterpret_cast<const int*>(p[i])));
      }
    }
  }
  // k-tile 0 block of this tile in the packed layout (k-tile kt at + kt * 32 KB)
  __device__ const char* w_block(const State& st) const {
    if (!wpk) return nullptr;
    return wpk + ((int64_t)st.e * et.nft + st.ft) * (int64_t)(L / 64) * kPackBlock;
  }
  template <class Acc>
  __device__ __forceinline__ void epilogue(const State& st, const Acc& acc, int wf0, int wt0, int lane) const;
};

template <class Cfg, typename CT>
struct ExpertDownProb {
  ExpertTiles<Cfg> et;
  const char* act;    // [T*k, I]
  const char* wo;     // [E, L, I]
  const float* so;    // [E, L/128, I/128]
  char* out;          // [T*k, L]
  const char* wpk;    // packed out blocks (see lmoe_pack_experts) or NULL
  const float* xs;    // W8A8: act block scales, [I/128, ldxs]
  int64_t ldxs;
  int I, L, f8, a8;   // a8: act holds e4m3 codes (W8A8)

  typedef ExpertState State;
  __device__ bool setup(int bid, State& st) const { return et.locate(bid, st); }
  __device__ int num_logical() const { return et.num_logical(); }
  __device__ bool setup_lg(int lg, State& st) const { return et.locate_lg(lg, et.num_logical(), st); }
  __device__ int num_ksegs() const { return 1; }
  __device__ int seg_ktiles(int) const { return I * (int)sizeof(CT) / 128; }
  __device__ bool seg_f8(const State&, int) const { return f8; }
  __device__ int tokens_valid(const State& st) const { return st.rows; }
  __device__ int feats_valid(const State& st) const { return min(Cfg::BF, L - st.ft * Cfg::BF); }
  __device__ const char* x_row(const State& st, int, int r) const {
    if (r >= st.rows) return nullptr;
    return act + (int64_t)(st.m0 + r) * I * (a8 ? 1 : (int64_t)sizeof(CT));
  }
  template <int RPI = 8>
  __device__ const char* x_row_grp(const State& st, int s, int r0, int lane) const {
    return x_row(st, s, min(r0 + lane / (64 / RPI), tokens_valid(st) - 1));
  }
  __device__ const float* x_scale(const State& st, int kb) const { return xs + kb * ldxs + st.m0; }
  __device__ const char* w_row(const State& st, int, int r, const float** scrow) const {
    const int f = st.ft * Cfg::BF + r;
    if (f >= L) return nullptr;
    const int64_t wes = f8 ? 1 : sizeof(CT);
    if (f8) *scrow = so + ((int64_t)st.e * (L >> 7) + (f >> 7)) * (I >> 7);
    return wo + ((int64_t)st.e * L + f) * I * wes;
  }
  __device__ const char* w_block(const State& st) const {
    if (!wpk) return nullptr;
    return wpk + ((int64_t)st.e * et.nft + st.ft) * (int64_t)(I / 64) * kPackBlock;
  }
  // e4m3 block scales of the 32-row blocks r0 + 32 i at 128-column block kb.
  // A wave's rows (r0 a multiple of its 64- or 128-row slab) lie in one
  // 128-row block, so they share one scale.
  template <int N>
  __device__ void w_scales(const State& st, int r0, int kb, float (&sc)[N]) const {
    static_assert(N * 32 <= 128, "a wave slab within one 128-row scale block");
    const int f0 = st.ft * Cfg::BF + r0;
    const float s = __int_as_float(
        sload1(reinterpret_cast<const int*>(so + ((int64_t)st.e * (L >> 7) + (f0 >> 7)) * (I >> 7) + kb)));
#pragma unroll
    for (int i = 0; i < N; ++i) sc[i] = s;
  }
  template <class Acc>
  __device__ __forceinline__ void epilogue(const State& st, const Acc& acc, int wf0, int wt0, int lane) const;
};

// Backward data gradients of the routed experts on the persistent engine
// (Tile3 WTR): C[r, f] = sum over the K segments s of X_s[r, k] W_s[e][k, f],
// the expert matrices read as the forward stores them ([E, K_s, F], features
// contiguous) and transposed between LDS and the MFMAs.  X_s: rows in
// assignment (expert) order, [T*k, K_s], bf16.  C: fp32 [T*k, F].
//   dA = dO W_o[e]        (one segment, K = L, F = I)
//   dz rows = dG W_g[e] + dV W_v[e]   (two segments, K = I each, F = L)
template <class Cfg, typename CT>
struct ExpertTGradProb {
  // vector stores (at least) a wave's epilogue issues per 32-row token block
  // whose rows are all valid: the persistent loop's next wait lets them drain
  // (declared where the fp32 output tile is large; on the forward's bf16
  // expert GEMMs it measured no better)
  static constexpr int kEpiStores = Cfg::FI * 4;
  ExpertTiles<Cfg> et;
  const char* x[2];   // [T*k, kd[s]]
  const char* w[2];   // [E, kd[s], F]
  int kd[2];
  int nseg, F;
  float* out;         // [T*k, F]

  typedef ExpertState State;
  __device__ bool setup(int bid, State& st) const { return et.locate(bid, st); }
  __device__ int num_logical() const { return et.num_logical(); }
  __device__ bool setup_lg(int lg, State& st) const { return et.locate_lg(lg, et.num_logical(), st); }
  __device__ int num_ksegs() const { return nseg; }
  __device__ int seg_ktiles(int s) const { return kd[s] * (int)sizeof(CT) / 128; }
  __device__ bool seg_f8(const State&, int) const { return false; }
  __device__ int tokens_valid(const State& st) const { return st.rows; }
  __device__ int feats_valid(const State& st) const { return min(Cfg::BF, F - st.ft * Cfg::BF); }
  __device__ const char* x_row(const State& st, int s, int r) const {
    if (r >= st.rows) return nullptr;
    return x[s] + (int64_t)(st.m0 + r) * kd[s] * (int64_t)sizeof(CT);
  }
  template <int RPI = 8>
  __device__ const char* x_row_grp(const State& st, int s, int r0, int lane) const {
    return x_row(st, s, min(r0 + lane / (64 / RPI), tokens_valid(st) - 1));
  }
  // 16-byte chunk c (features ft * BF + 8 c ..) of k-row kr of the first
  // k-tile of segment s; each k-tile moves it by w_tstep bytes.  Chunks past
  // F (a last, partial feature tile) read the row's last chunk instead: they
  // only feed accumulator columns that are never stored, and no read leaves
  // the matrix.
  __device__ const char* w_tsrc(const State& st, int s, int kr, int c) const {
    const int f = min(st.ft * Cfg::BF + 8 * c, F - 8);
    return w[s] + (((int64_t)st.e * kd[s] + kr) * F + f) * (int64_t)sizeof(CT);
  }
  __device__ int64_t w_tstep(const State&, int) const { return (int64_t)64 * F * sizeof(CT); }
  __device__ const char* w_row(const State&, int, int, const float**) const { return nullptr; }
  __device__ const char* w_block(const State&) const { return nullptr; }
  template <class Acc>
  __device__ __forceinline__ void epilogue(const State& st, const Acc& acc, int wf0, int wt0, int lane) const;
};

// Backward data gradients of the dense projections on the persistent engine
// (Tile3 WTR): C[t, f] = sum over the K segments s of X_s[t, k] W_s[k, f],
// with each W_s read as the forward stores it (features contiguous) and
// transposed between LDS and the MFMAs.  The F features may span several
// matrices of fsplit features each (a stack, wms elements apart: the shared
// experts' out matrices); each 8-feature chunk lies in one of them.
//   dn = dy W_up;  dh = dy [W_so[0] | W_so[1] ...];
//   dx = dz W_dn + dg_s W_sg + dv_s W_sv  (three K segments)
// X_s: bf16 [T, ldx], C: fp32 [T, ldo].
template <class Cfg, typename CT>
struct DenseTProb {
  static constexpr bool kDenseRows = false;
  static constexpr int kEpiStores = Cfg::FI * 4;  // as ExpertTGradProb
  int64_t T;
  int F, fsplit;      // features; features per stacked matrix
  int nks, ntt, nft;
  const char* x[3];
  int64_t ldx[3];
  int kd[3];
  const char* w[3];   // W_s: [K_s, fsplit] per matrix, matrices wms[s] elements apart
  int64_t wms[3];
  float* out;
  int64_t ldo;
  int accumulate;     // C += instead of C =

  struct State {
    int tt, ft;
  };
  __device__ int num_logical() const { return ntt * nft; }
  // feature tiles outermost: neighbouring work-groups share a weight tile
  __device__ bool setup_lg(int lg, State& st) const {
    if (lg >= ntt * nft) return false;
    st.ft = lg / ntt;
    st.tt = lg - st.ft * ntt;
    return true;
  }
  __device__ bool setup(int bid, State& st) const { return setup_lg(bid, st); }
  __device__ int num_ksegs() const { return nks; }
  __device__ int seg_ktiles(int s) const { return kd[s] * (int)sizeof(CT) / 128; }
  __device__ bool seg_f8(const State&, int) const { return false; }
  __device__ int tokens_valid(const State& st) const { return (int)imin64(Cfg::BT, T - (int64_t)st.tt * Cfg::BT); }
  __device__ int feats_valid(const State& st) const { return min(Cfg::BF, F - st.ft * Cfg::BF); }
  __device__ const char* x_row(const State& st, int s, int r) const {
    const int64_t t = (int64_t)st.tt * Cfg::BT + r;
    return t < T ? x[s] + t * ldx[s] * (int64_t)sizeof(CT) : nullptr;
  }
  template <int RPI = 8>
  __device__ const char* x_row_grp(const State& st, int s, int r0, int lane) const {
    return x_row(st, s, min(r0 + lane / (64 / RPI), tokens_valid(st) - 1));
  }
  // as ExpertTGradProb::w_tsrc; chunks past F read the tile's last chunk
  __device__ const char* w_tsrc(const State& st, int s, int kr, int c) const {
    const int f = min(st.ft * Cfg::BF + 8 * c, F - 8);
    const int g = f / fsplit, fl = f - g * fsplit;
    return w[s] + ((int64_t)g * wms[s] + (int64_t)kr * fsplit + fl) * (int64_t)sizeof(CT);
  }
  __device__ int64_t w_tstep(const State&, int) const { return (int64_t)64 * fsplit * sizeof(CT); }
  __device__ const char* w_row(const State&, int, int, const float**) const { return nullptr; }
  __device__ const char* w_block(const State&) const { return nullptr; }
  template <class Acc>
  __device__ __forceinline__ void epilogue(const State& st, const Acc& acc, int wf0, int wt0, int lane) const;
};

// ---------------------------------------------------------------------------
// The mainloop.
// ---------------------------------------------------------------------------
template <typename CT>
struct Frag;
template <>
struct Frag<bf16> {
  typedef bf16x8 type;  // 8 consecutive K values of one row
  static constexpr int KPM = 16;
  static constexpr int EPL = 8;
};
template <>
struct Frag<float> {
  typedef float type;
  static constexpr int KPM = 2;
  static constexpr int EPL = 1;
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 32x32x64 e4m3 x e4m3 block: lane l holds 32 codes of row (column) l % 32
// for each operand.  The E8M0 block scales of the instruction are left at
// 127 (2^0), so the products are the plain code products.
__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 8 e4m3 codes -> 8 bf16 of code * scale.
__device__ __forceinline__ uint4 widen_e4m3(uint2 q, float s) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.x, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.x, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.y, false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.y, true);
  bf16x8 o = {(bf16)(a.x * s), (bf16)(a.y * s), (bf16)(b.x * s), (bf16)(b.y * s),
              (bf16)(c.x * s), (bf16)(c.y * s), (bf16)(d.x * s), (bf16)(d.y * s)};
  return *reinterpret_cast<uint4*>(&o);
}

template <class Cfg, typename CT, class Prob>
__global__ __launch_bounds__(Cfg::NT) void gemm_kernel(const Prob p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  typename Prob::State st;
  if (!p.setup(blockIdx.x, st)) return;

  constexpr int NT = Cfg::NT, FI = Cfg::FI, TI = Cfg::TI, CW = Cfg::CW, CX = Cfg::CX;
  constexpr int ES = sizeof(CT);
  constexpr int BK = 128 / ES;
  constexpr int KPM = Frag<CT>::KPM, EPL = Frag<CT>::EPL;
  typedef typename Frag<CT>::type FT;

  char* const sW0 = smem;
  char* const sX0 = smem + 2 * Cfg::BF * kPitch;

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

  const int nks = p.num_ksegs();
  for (int s = 0; s < nks; ++s) {
    const int nkt = p.seg_ktiles(s);
    if (nkt <= 0) continue;
    const bool f8 = (ES == 2) && p.seg_f8(st, s);

    const char* wp[CW];
    const float* wsc[CW];
    const char* xp[CX];
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int c = tid + i * NT;
      wsc[i] = nullptr;
      const char* rp = p.w_row(st, s, c >> 3, &wsc[i]);
      wp[i] = rp ? rp + (c & 7) * (f8 ? 8 : 16) : nullptr;
    }
#pragma unroll
    for (int i = 0; i < CX; ++i) {
      const int c = tid + i * NT;
      const char* rp = p.x_row(st, s, c >> 3);
      xp[i] = rp ? rp + (c & 7) * 16 : nullptr;
    }

    uint4 wr[CW], xr[CX];
    float sc[CW];
    auto gload = [&](int kt) {
#pragma unroll
      for (int i = 0; i < CW; ++i) {
        if (wp[i]) {
          if (f8) {
            const uint2 q = *reinterpret_cast<const uint2*>(wp[i] + (int64_t)kt * 64);
            wr[i] = uint4{q.x, q.y, 0u, 0u};
            sc[i] = wsc[i][kt >> 1];
          } else {
            wr[i] = *reinterpret_cast<const uint4*>(wp[i] + (int64_t)kt * 128);
          }
        } else {
          wr[i] = uint4{0u, 0u, 0u, 0u};
          sc[i] = 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < CX; ++i)
        xr[i] = xp[i] ? *reinterpret_cast<const uint4*>(xp[i] + (int64_t)kt * 128) : uint4{0u, 0u, 0u, 0u};
    };
    auto lstore = [&](int buf) {
      char* sW = sW0 + buf * Cfg::BF * kPitch;
      char* sX = sX0 + buf * Cfg::BT * kPitch;
#pragma unroll
      for (int i = 0; i < CW; ++i) {
        const int c = tid + i * NT;
        uint4 v = wr[i];
        if constexpr (ES == 2) {
          if (f8) v = widen_e4m3(uint2{wr[i].x, wr[i].y}, sc[i]);
        }
        *reinterpret_cast<uint4*>(sW + (c >> 3) * kPitch + (c & 7) * 16) = v;
      }
#pragma unroll
      for (int i = 0; i < CX; ++i) {
        const int c = tid + i * NT;
        *reinterpret_cast<uint4*>(sX + (c >> 3) * kPitch + (c & 7) * 16) = xr[i];
      }
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nkt) gload(kt + 1);
      const char* sW = sW0 + cur * Cfg::BF * kPitch;
      const char* sX = sX0 + cur * Cfg::BT * kPitch;
#pragma unroll
      for (int ks = 0; ks < BK / KPM; ++ks) {
        const int kb = (ks * KPM + (lane >> 5) * EPL) * ES;
        FT a[FI], b[TI];
#pragma unroll
        for (int i = 0; i < FI; ++i)
          a[i] = *reinterpret_cast<const FT*>(sW + (wf0 + i * 32 + (lane & 31)) * kPitch + kb);
#pragma unroll
        for (int j = 0; j < TI; ++j)
          b[j] = *reinterpret_cast<const FT*>(sX + (wt0 + j * 32 + (lane & 31)) * kPitch + kb);
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
          for (int j = 0; j < TI; ++j)
            if (fea[i] && tok[j]) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
      }
      if (kt + 1 < nkt) lstore(cur ^ 1);
      __syncthreads();
    }
  }
  p.epilogue(st, acc, wf0, wt0, lane);
}

// ---------------------------------------------------------------------------
// Epilogues.  Accumulator element r of lane l in MFMA block (i, j) holds
// feature wf0 + 32i + 8(r/4) + 4(l/32) + r%4 of token wt0 + 32j + l%32.
// ---------------------------------------------------------------------------
template <class Cfg, class F>
__device__ __forceinline__ void for_acc(int wf0, int wt0, int lane, F&& f) {
#pragma unroll
  for (int i = 0; i < Cfg::FI; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TI; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) f(i, j, g, wf0 + i * 32 + g * 8 + (lane >> 5) * 4, wt0 + j * 32 + (lane & 31));
}

// GLU pairs: blocks (2q, 2q+1) hold gate and value of the same 32 units.
template <class Cfg, class F>
__device__ __forceinline__ void for_glu(int wf0, int wt0, int lane, F&& f) {
#pragma unroll
  for (int i = 0; i < Cfg::FI; i += 2)
#pragma unroll
    for (int j = 0; j < Cfg::TI; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        f(i, j, g, (wf0 + i * 32) / 2 + g * 8 + (lane >> 5) * 4, wt0 + j * 32 + (lane & 31));
}

// for_acc by pairs of accumulator groups (2h, 2h + 1) for store16_pair:
// f(i, j, h, b, tl), b the pair's first feature.
template <class Cfg, class F>
__device__ __forceinline__ void for_acc_pairs(int wf0, int wt0, int lane, F&& f) {
#pragma unroll
  for (int i = 0; i < Cfg::FI; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TI; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) f(i, j, h, wf0 + i * 32 + h * 16, wt0 + j * 32 + (lane & 31));
}

template <class Cfg, typename CT>
template <class Acc>
__device__ __forceinline__ void DenseXProb<Cfg, CT>::epilogue(const State& st, const Acc& acc, int wf0, int wt0, int lane) const {
  const NSeg& s = st.s;
  const int tv = tokens_valid(st);
  const int tt = st.tt, f0 = st.f0;
  if (s.kind == EPI_GLU) {
    for_glu<Cfg>(wf0, wt0, lane, [&](int i, int j, int g, int ul, int tl) __attribute__((always_inline)) {
      if (tl < tv) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = situ_glu(acc[i][j][4 * g + r], acc[i + 1][j][4 * g + r], cap, inv_cap);
        const int64_t t = (int64_t)tt * Cfg::BT + tl;
        CT* row = reinterpret_cast<CT*>(s.out) + t * s.ldo + s.col0;
        store4<CT>(row, f0 + ul, v, s.rows, s.vec);
      }
    });
  } else {
    for_acc<Cfg>(wf0, wt0, lane, [&](int i, int j, int g, int fl, int tl) __attribute__((always_inline)) {
      if (tl < tv) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * g + r];
        const int64_t t = (int64_t)tt * Cfg::BT + tl;
        if (s.kind == EPI_F32) {
          float* row = reinterpret_cast<float*>(s.out) + t * s.ldo + s.col0;
          store4<float>(row, f0 + fl, v, s.rows, s.vec);
        } else {
          CT* row = reinterpret_cast<CT*>(s.out) + t * s.ldo + s.col0;
          store4<CT>(row, f0 + fl, v, s.rows, s.vec);
        }
      }
    });
  }
}

template <class Cfg, typename CT>
template <class Acc>
__device__ __forceinline__ void UpProb<Cfg, CT>::epilogue(const State& st, const Acc& acc, int wf0, int wt0, int lane) const {
  const int tv = tokens_valid(st);
  const int tt = st.tt, ft = st.ft;
  if constexpr (std::is_same_v<CT, bf16>) {
    for_acc_pairs<Cfg>(wf0, wt0, lane, [&](int i, int j, int h, int fb, int tl) __attribute__((always_inline)) {
      const int f = ft * Cfg::BF + fb;
      const int64_t t = (int64_t)tt * Cfg::BT + min(tl, tv - 1);
      float va[4], vb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        va[r] = acc[i][j][8 * h + r];
        vb[r] = acc[i][j][8 * h + 4 + r];
      }
      if (addend && tl < tv) {
        // this lane's own features: f + 4 (lane / 32) + r and 8 further on
        const bf16* ar = reinterpret_cast<const bf16*>(addend) + t * N + f + (lane >> 5) * 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (f + (lane >> 5) * 4 + r < N) va[r] += to_f32(ar[r]);
          if (f + (lane >> 5) * 4 + 8 + r < N) vb[r] += to_f32(ar[8 + r]);
        }
      }
      store16_pair(reinterpret_cast<bf16*>(y) + t * N, f, pack_bf16x2(va[0], va[1]), pack_bf16x2(va[2], va[3]),
                   pack_bf16x2(vb[0], vb[1]), pack_bf16x2(vb[2], vb[3]), N, tl < tv, vec, lane);
    });
    return;
  }
  for_acc<Cfg>(wf0, wt0, lane, [&](int i, int j, int g, int fl, int tl) __attribute__((always_inline)) {
    const int f = ft * Cfg::BF + fl;
    if (tl < tv && f < N) {
      const int64_t t = (int64_t)tt * Cfg::BT + tl;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * g + r];
      if (addend) {
        const CT* ar = reinterpret_cast<const CT*>(addend) + t * N;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (f + r < N) v[r] += to_f32(ar[f + r]);
      }
      store4<CT>(reinterpret_cast<CT*>(y) + t * N, f, v, N, vec);
    }
  });
}

template <class Cfg, typename CT, int RAW>
template <class Acc>
__device__ __forceinline__ void ExpertGVProb<Cfg, CT, RAW>::epilogue(const State& st, const Acc& acc, int wf0, int wt0,
                                                                     int lane) const {
  for_glu<Cfg>(wf0, wt0, lane, [&](int i, int j, int g, int ul, int tl) __attribute__((always_inline)) {
    if (tl < st.rows) {
      if constexpr (RAW == 1) {
        float gv[4], vv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          gv[r] = acc[i][j][4 * g + r];
          vv[r] = acc[i + 1][j][4 * g + r];
        }
        const int64_t o = (int64_t)(st.m0 + tl) * I;
        store4<float>(graw + o, st.ft * (Cfg::BF / 2) + ul, gv, I, true);
        store4<float>(vraw + o, st.ft * (Cfg::BF / 2) + ul, vv, I, true);
      } else {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = situ_glu(acc[i][j][4 * g + r], acc[i + 1][j][4 * g + r], cap, inv_cap);
        typedef std::conditional_t<RAW == 2, float, CT> OT;
        OT* row = reinterpret_cast<OT*>(act) + (int64_t)(st.m0 + tl) * I;
        store4<OT>(row, st.ft * (Cfg::BF / 2) + ul, v, I, true);
      }
    }
  });
}

template <class Cfg, typename CT>
template <class Acc>
__device__ __forceinline__ void ExpertDownProb<Cfg, CT>::epilogue(const State& st, const Acc& acc, int wf0, int wt0, int lane) const {
  if constexpr (std::is_same_v<CT, bf16>) {
    for_acc_pairs<Cfg>(wf0, wt0, lane, [&](int i, int j, int h, int fb, int tl) __attribute__((always_inline)) {
      const f32x16& a = acc[i][j];
      bf16* row = reinterpret_cast<bf16*>(out) + (int64_t)(st.m0 + min(tl, st.rows - 1)) * L;
      store16_pair(row, st.ft * Cfg::BF + fb, pack_bf16x2(a[8 * h], a[8 * h + 1]), pack_bf16x2(a[8 * h + 2], a[8 * h + 3]),
                   pack_bf16x2(a[8 * h + 4], a[8 * h + 5]), pack_bf16x2(a[8 * h + 6], a[8 * h + 7]), L, tl < st.rows,
                   true, lane);
    });
    return;
  }
  for_acc<Cfg>(wf0, wt0, lane, [&](int i, int j, int g, int fl, int tl) __attribute__((always_inline)) {
    if (tl < st.rows) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * g + r];
      CT* row = reinterpret_cast<CT*>(out) + (int64_t)(st.m0 + tl) * L;
      store4<CT>(row, st.ft * Cfg::BF + fl, v, L, true);
    }
  });
}

template <class Cfg, typename CT>
template <class Acc>
__device__ __forceinline__ void ExpertTGradProb<Cfg, CT>::epilogue(const State& st, const Acc& acc, int wf0, int wt0,
                                                                   int lane) const {
  for_acc<Cfg>(wf0, wt0, lane, [&](int i, int j, int g, int fl, int tl) __attribute__((always_inline)) {
    if (tl < st.rows) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * g + r];
      store4<float>(out + (int64_t)(st.m0 + tl) * F, st.ft * Cfg::BF + fl, v, F, true);
    }
  });
}

template <class Cfg, typename CT>
template <class Acc>
__device__ __forceinline__ void DenseTProb<Cfg, CT>::epilogue(const State& st, const Acc& acc, int wf0, int wt0,
                                                              int lane) const {
  const int tv = tokens_valid(st);
  for_acc<Cfg>(wf0, wt0, lane, [&](int i, int j, int g, int fl, int tl) __attribute__((always_inline)) {
    if (tl < tv) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * g + r];
      float* row = out + ((int64_t)st.tt * Cfg::BT + tl) * ldo;
      const int f = st.ft * Cfg::BF + fl;
      if (accumulate) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (f + r < F) v[r] += row[f + r];
      }
      store4<float>(row, f, v, F, (ldo & 3) == 0);
    }
  });
}

}  // namespace lmoe
