// C ABI of the Stable Latent MoE layer: argument checks, workspace plan and
// the launch sequence of each entry point (declarations and contracts in
// include/lmoe.h).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>
#include <mutex>

#include "backward.hpp"
#include "wgrad.hpp"
#include "kernels.hpp"
#include "lmoe.h"

namespace lmoe {
namespace {

thread_local char g_err[512] = "";

lmoe_status fail(lmoe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

lmoe_status hip_fail(hipError_t e, const char* what) {
  return fail(LMOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define LMOE_HIP(call, what)                        \
  do {                                              \
    hipError_t e_ = (call);                         \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------
// Shape checks (host only).
// ---------------------------------------------------------------------------
lmoe_status check_shape(const lmoe_shape* sh) {
  if (!sh) return fail(LMOE_EINVAL, "shape is NULL");
  if (sh->T < 0) return fail(LMOE_EINVAL, "T = %lld < 0", (long long)sh->T);
  if (sh->H <= 0 || sh->L <= 0 || sh->E <= 0 || sh->k <= 0 || sh->I <= 0 || sh->S < 0)
    return fail(LMOE_EINVAL, "H, L, E, k, I must be > 0 and S >= 0");
  if (sh->S > 0 && sh->Is <= 0) return fail(LMOE_EINVAL, "Is must be > 0 when S > 0");
  if (sh->k > sh->E) return fail(LMOE_EINVAL, "k = %d > E = %d", sh->k, sh->E);
  if (!(sh->cap > 0.f)) return fail(LMOE_EINVAL, "cap must be > 0 (inf disables it)");
  if (!(sh->rms_eps >= 0.f) || isinf(sh->rms_eps)) return fail(LMOE_EINVAL, "rms_eps must be finite and >= 0");
  if (sh->act != LMOE_F32 && sh->act != LMOE_BF16)
    return fail(sh->act == LMOE_F8E4M3 ? LMOE_EUNSUPPORTED : LMOE_EINVAL, "act dtype %d not supported", sh->act);
  if (sh->w_expert < LMOE_F32 || sh->w_expert > LMOE_F8E4M3)
    return fail(LMOE_EINVAL, "w_expert dtype %d unknown", sh->w_expert);
  if (sh->act == LMOE_F32 && sh->w_expert != LMOE_F32)
    return fail(LMOE_EUNSUPPORTED, "an F32 layer needs F32 expert weights");
  if (sh->act == LMOE_BF16 && sh->w_expert == LMOE_F32)
    return fail(LMOE_EUNSUPPORTED, "a BF16 layer takes BF16 or F8E4M3 expert weights");
  const int al = sh->w_expert == LMOE_F8E4M3 ? 128 : 64;
  if (sh->H % al || sh->L % al || sh->I % al || (sh->S > 0 && sh->Is % al))
    return fail(LMOE_EUNSUPPORTED, "H, L, I, Is must be multiples of %d", al);
  if (sh->L > 8192) return fail(LMOE_EUNSUPPORTED, "L = %d > 8192", sh->L);
  if (sh->E > 1024) return fail(LMOE_EUNSUPPORTED, "E = %d > 1024", sh->E);
  if (sh->k > 64) return fail(LMOE_EUNSUPPORTED, "k = %d > 64", sh->k);
  if (sh->S > 8) return fail(LMOE_EUNSUPPORTED, "S = %d > 8", sh->S);
  if (sh->T * (int64_t)sh->k >= (int64_t(1) << 31)) return fail(LMOE_EUNSUPPORTED, "T*k must be < 2^31");
  if (sh->T >= (int64_t(1) << 31)) return fail(LMOE_EUNSUPPORTED, "T must be < 2^31");
  if (sh->a8 != 0 && sh->a8 != 1) return fail(LMOE_EINVAL, "a8 = %d is neither 0 nor 1", sh->a8);
  if (sh->a8 && !(sh->act == LMOE_BF16 && sh->w_expert == LMOE_F8E4M3))
    return fail(LMOE_EUNSUPPORTED, "W8A8 (a8 = 1) needs act BF16 and F8E4M3 expert weights");
  return LMOE_OK;
}

bool is_f8(const lmoe_shape* sh) { return sh->w_expert == LMOE_F8E4M3; }

// Which weights an entry point reads.
enum : unsigned { NEED_ROUTE = 1, NEED_EXPERT = 2, NEED_UP = 4, NEED_NORM = 8 };

// Matrices and activations move through 16-byte vector loads, DMAs and
// stores, so their base pointers must be 16-byte aligned (NULL passes).
lmoe_status check_align16(std::initializer_list<std::pair<const void*, const char*>> ptrs) {
  for (const auto& [p, name] : ptrs)
    if (reinterpret_cast<uintptr_t>(p) & 15) return fail(LMOE_EINVAL, "%s must be 16-byte aligned", name);
  return LMOE_OK;
}

lmoe_status check_weights(const lmoe_shape* sh, const lmoe_weights* w, unsigned need) {
  if (!w) return fail(LMOE_EINVAL, "weights is NULL");
  if (lmoe_status s = check_align16({{w->w_router, "w_router"}, {w->w_down, "w_down"}, {w->w_gate, "w_gate"},
                                      {w->w_value, "w_value"}, {w->w_out, "w_out"}, {w->w_up, "w_up"},
                                      {w->ws_gate, "ws_gate"}, {w->ws_value, "ws_value"}, {w->ws_out, "ws_out"}}))
    return s;
  const bool f8 = is_f8(sh);
  if (need & NEED_ROUTE) {
    if (!w->w_router || !w->b_router) return fail(LMOE_EINVAL, "w_router and b_router are required");
    if (!w->w_down && sh->L != sh->H) return fail(LMOE_EINVAL, "w_down = NULL needs L == H");
  }
  if (need & NEED_EXPERT) {
    if (w->packed) {
      if (!(sh->act == LMOE_BF16 && sh->w_expert == LMOE_BF16))
        return fail(LMOE_EUNSUPPORTED, "packed expert weights need a BF16 layer with BF16 expert weights");
      if (reinterpret_cast<uintptr_t>(w->packed) & 255) return fail(LMOE_EINVAL, "packed must be 256-byte aligned");
    } else {
      if (!w->w_gate || !w->w_value || !w->w_out) return fail(LMOE_EINVAL, "expert weights are required");
      if (f8 && (!w->s_gate || !w->s_value || !w->s_out))
        return fail(LMOE_EINVAL, "e4m3 expert scales are required");
    }
  }
  if (need & NEED_NORM) {
    if (!w->gamma) return fail(LMOE_EINVAL, "gamma is required");
  }
  if (need & NEED_UP) {
    if (!w->w_up && sh->L != sh->H) return fail(LMOE_EINVAL, "w_up = NULL needs L == H");
    if (sh->S > 0) {
      if (!w->ws_gate || !w->ws_value || !w->ws_out) return fail(LMOE_EINVAL, "shared expert weights are required");
      if (f8 && (!w->ss_gate || !w->ss_value || !w->ss_out))
        return fail(LMOE_EINVAL, "e4m3 shared expert scales are required");
    }
  }
  return LMOE_OK;
}

// ---------------------------------------------------------------------------
// Kernel choices and the workspace plan.
// ---------------------------------------------------------------------------
// Kernel choice.  bf16 layers with bf16 expert weights run the LDS-DMA
// pipeline (gemm2.hpp); fp32 layers and e4m3 weights run the register-staged
// mainloop (gemm.hpp), which widens e4m3 codes on the way into LDS.
bool use_dma(const lmoe_shape* sh) { return sh->act == LMOE_BF16 && sh->w_expert == LMOE_BF16; }
// e4m3 expert weights with bf16 activations and many rows per expert: the
// persistent LDS-DMA expert GEMMs with the codes widened at the fragment load.
bool use_dma_f8(const lmoe_shape* sh) {
  return sh->act == LMOE_BF16 && sh->w_expert == LMOE_F8E4M3 && !sh->a8 &&
         sh->T * (int64_t)sh->k >= 96 * (int64_t)sh->E;
}
// W8A8: e4m3 x e4m3 persistent expert GEMMs at every token count.
bool use_a8(const lmoe_shape* sh) { return sh->a8 != 0; }

// Experts: token tile by the mean rows per expert (T*k/E).
enum ExpertTile { ET_SMALL, ET_MID, ET_BIG };
ExpertTile expert_tile(const lmoe_shape* sh) {
  const int64_t tk = sh->T * (int64_t)sh->k;
  if (use_dma(sh)) {
    if (tk < 16 * (int64_t)sh->E) return ET_SMALL;
    if (tk < 96 * (int64_t)sh->E) return ET_MID;
    return ET_BIG;
  }
  return tk < 48 * (int64_t)sh->E ? ET_SMALL : ET_BIG;
}
int expert_bt(const lmoe_shape* sh) {
  if (use_a8(sh)) return T2ExpertGVA8::BT;
  if (use_dma_f8(sh)) return T2ExpertGVF8::BT;
  const ExpertTile t = expert_tile(sh);
  if (use_dma(sh)) return t == ET_SMALL ? T2SmallGV::BT : t == ET_MID ? T2MidGV::BT : T2ExpertGV::BT;
  return t == ET_SMALL ? CfgSmall::BT : CfgBig::BT;
}
bool dense_small(const lmoe_shape* sh) { return sh->T <= 256; }

// Upper bound of the number of token tiles over all experts.
int64_t max_tiles(const lmoe_shape* sh, int bt) {
  const int64_t tk = sh->T * sh->k;
  const int64_t busy = tk < sh->E ? tk : sh->E;
  return (tk + busy * (bt - 1)) / bt;
}

struct Plan {
  size_t logits, z, hs, n, idx, w, bcounts, offsets, sorted, pos, tiles_a, tiles_b, tcount, act, out;
  size_t zf, zq, zs_tok, zs, aq, as;  // W8A8 only: fp32 z; e4m3 z, its scales by token and in expert order;
                                      // e4m3 act, its scales
  size_t shared_bf16;              // e4m3 shared experts decoded to bf16 (gate, value, out)
  size_t total;
};

Plan plan(const lmoe_shape* sh) {
  Plan p{};
  const size_t es = sh->act == LMOE_BF16 ? 2 : 4;
  const size_t T = (size_t)sh->T, tk = T * sh->k;
  const size_t nb = (T + kPermTokens - 1) / kPermTokens;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  p.logits = take(T * sh->E * 4);
  p.z = take(T * sh->L * es);
  p.hs = take(T * (size_t)sh->S * (sh->S ? sh->Is : 0) * es);
  p.n = take(T * sh->L * es);
  p.idx = take(tk * 4);
  p.w = take(tk * 4);
  p.bcounts = take(nb * sh->E * 4);
  p.offsets = take((size_t)(sh->E + 1) * 4);
  p.sorted = take(tk * 4);
  p.pos = take(tk * 4);
  p.tiles_a = take((size_t)max_tiles(sh, expert_bt(sh)) * 16);
  p.tiles_b = take(16);
  p.tcount = take(8);
  p.act = take(tk * sh->I * (sh->a8 ? 4 : es));  // W8A8: fp32 for the quantiser
  p.out = take(tk * sh->L * es);
  if (sh->w_expert == LMOE_F8E4M3 && sh->S > 0) p.shared_bf16 = take((size_t)3 * sh->S * sh->Is * sh->H * 2);
  if (sh->a8) {
    p.zf = take(T * sh->L * 4);
    p.zq = take(T * sh->L);
    p.zs_tok = take(T * (sh->L / 128) * 4);
    p.zs = take(tk * (sh->L / 128) * 4);
    p.aq = take(tk * sh->I);
    p.as = take(tk * (sh->I / 128) * 4);
  }
  p.total = off;
  return p;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

lmoe_status check_ws(const lmoe_shape* sh, const void* ws, size_t ws_bytes) {
  const size_t need = plan(sh).total;
  if (ws_bytes < need) return fail(LMOE_EWORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  if (!ws) return fail(LMOE_EINVAL, "ws is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(LMOE_EINVAL, "ws must be 256-byte aligned");
  return LMOE_OK;
}

// ---------------------------------------------------------------------------
// GEMM launches.
// ---------------------------------------------------------------------------
// Host-side values cached per device on first use (each entry written once,
// under its own once_flag): the compute-unit count and the kernels' LDS
// attribute.  Devices past kMaxDevices are queried on every call instead.
constexpr int kMaxDevices = 64;
int current_device() {
  int d = -1;
  return hipGetDevice(&d) == hipSuccess ? d : -1;
}

int cu_count(int dev) {
  int cus = 0;
  if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

// Work-groups of a persistent GEMM: one per compute unit of the current
// device (their LDS use leaves room for one group per CU), a multiple of the
// XCD count.
int persistent_grid() {
  static std::once_flag once[kMaxDevices];
  static int n[kMaxDevices];
  const int dev = current_device();
  auto count = [](int d) { return (cu_count(d) + kXcds - 1) / kXcds * kXcds; };
  if (dev < 0 || dev >= kMaxDevices) return count(dev);
  std::call_once(once[dev], [&] { n[dev] = count(dev); });
  return n[dev];
}

template <class Cfg, typename CT, class Prob>
hipError_t launch_gemm(const Prob& p, int64_t grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  void (*kern)(const Prob);
  if constexpr (Cfg::kKind == 4) {
    kern = gemm3p_kernel<Cfg, Prob>;
    grid = persistent_grid();
  } else if constexpr (Cfg::kKind == 3) kern = gemm3_kernel<Cfg, Prob>;
  else if constexpr (Cfg::kKind == 2) kern = gemm2_kernel<Cfg, Prob>;
  else kern = gemm_kernel<Cfg, CT, Prob>;
  auto set_attr = [&] {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                               Cfg::LDS);
  };
  static std::once_flag once[kMaxDevices];
  static hipError_t attr[kMaxDevices];
  const int dev = current_device();
  hipError_t a;
  if (dev < 0 || dev >= kMaxDevices) {
    a = set_attr();
  } else {
    std::call_once(once[dev], [&] { attr[dev] = set_attr(); });
    a = attr[dev];
  }
  if (a != hipSuccess) return a;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::NT), Cfg::LDS, st, p);
  return hipGetLastError();
}

int64_t pad8(int64_t v) { return (v + kXcds - 1) / kXcds * kXcds; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Packed expert weights: gate/value blocks, then out blocks (32 KB each).
int64_t packed_gv_blocks(const lmoe_shape* sh) { return (int64_t)sh->E * cdiv(sh->I, 128) * (sh->L / 64); }
int64_t packed_dn_blocks(const lmoe_shape* sh) { return (int64_t)sh->E * cdiv(sh->L, kPackRows) * (sh->I / 64); }

struct Ctx {
  const lmoe_shape* sh;
  const lmoe_weights* w;
  hipStream_t st;
  const char* pk_gv() const { return static_cast<const char*>(w->packed); }
  const char* pk_dn() const {
    return w->packed ? static_cast<const char*>(w->packed) + packed_gv_blocks(sh) * kPackBlock : nullptr;
  }
  size_t es() const { return sh->act == LMOE_BF16 ? 2 : 4; }
  size_t wes() const { return sh->w_expert == LMOE_F8E4M3 ? 1 : es(); }
  float inv_cap() const { return isinf(sh->cap) ? 0.f : 1.f / sh->cap; }
};

// Dense GEMM launch over nft x ntt big tiles.  With the LDS-DMA 256 x 256
// tile, when the tiles make some full waves over the CUs plus a last wave
// that would leave at least half of them idle, the full waves run as they are
// and the last wave's tiles are re-cut into 2 or 4 sub-tiles each (128 x 128
// or 128 x 256), launched after them on the same stream.  Each output element
// is summed over the same k-tiles in the same order in either tile, so the
// results are bitwise those of the single launch.
typedef Tile3<128, 128, 2, 2, 0> T2DenseQuarter;
typedef Tile3<128, 256, 2, 4, 0> T2DenseHalf;

template <class To, class From>
To with_cfg(const From& f) {
  static_assert(sizeof(To) == sizeof(From), "same problem, another tile");
  To t;
  memcpy(static_cast<void*>(&t), &f, sizeof(To));
  return t;
}

// Side stream of the current device (created once, default priority): the
// route GEMM's re-cut last round runs there when all its tiles belong to the
// shared experts' segment, whose output only the up GEMM reads, so it
// overlaps top-k and the permutation instead of delaying them.
hipStream_t side_stream() {
  static std::once_flag once[kMaxDevices];
  static hipStream_t s[kMaxDevices];
  const int dev = current_device();
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(once[dev], [&] {
    if (hipStreamCreateWithFlags(&s[dev], hipStreamNonBlocking) != hipSuccess) s[dev] = nullptr;
  });
  return s[dev];
}

// One call's fork of work onto the side stream and its join back.  The
// events are the call's own, so calls on other streams do not share them;
// the destructor joins a fork that was never joined (an error path), so the
// caller's stream stays ordered after the side work.
struct TailFork {
  hipStream_t main = nullptr, side = nullptr;
  int defer_ft = 1 << 30;  // first big feature tile that may be deferred
  hipEvent_t join = nullptr;
  bool forked = false, joined = false;

  hipError_t fork(hipStream_t st) {
    hipEvent_t f = nullptr;
    hipError_t e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&join, hipEventDisableTiming)) == hipSuccess &&
        (e = hipEventRecord(f, st)) == hipSuccess && (e = hipStreamWaitEvent(side, f, 0)) == hipSuccess) {
      main = st;
      forked = true;
    }
    hipEventDestroy(f);
    return e;
  }
  hipError_t wait(hipStream_t st) {
    if (!forked || joined) return hipSuccess;
    joined = true;
    return hipStreamWaitEvent(st, join, 0);
  }
  ~TailFork() {
    if (forked && !joined) hipStreamWaitEvent(main, join, 0);
    if (join) hipEventDestroy(join);
  }
};

template <class Cfg, typename CT, template <class, typename> class Prob>
hipError_t launch_dense(Prob<Cfg, CT>& p, int nft, int ntt, hipStream_t st, TailFork* fk = nullptr) {
  const int ntiles = nft * ntt;
  p.walk = DenseWalk{nft, ntt, 0, ntiles, 1, 1};
  if constexpr (std::is_same_v<Cfg, T2Dense>) {
    const int ncu = persistent_grid();
    const int full = ntiles / ncu * ncu, tail = ntiles - full;
    if (full > 0 && tail > 0 && 2 * tail <= ncu) {
      p.walk.count = full;
      p.padded = (int)pad8(full);
      hipError_t e = launch_gemm<Cfg, CT>(p, p.padded, st);
      if (e != hipSuccess) return e;
      // a tail wholly in the deferrable segment runs on the side stream
      if (fk && fk->side) {
        bool defer = true;
        for (int b = 0; b < tail && defer; ++b) {
          int ttb, ftb, qf, qt;
          DenseWalk{nft, ntt, full, tail, 1, 1}.map(b, ttb, ftb, qf, qt);
          defer = ftb >= fk->defer_ft;
        }
        if (defer) {
          if ((e = fk->fork(st)) != hipSuccess) return e;
          st = fk->side;
        }
      }
      if (4 * tail <= ncu) {
        auto q = with_cfg<Prob<T2DenseQuarter, CT>>(p);
        q.walk = DenseWalk{nft, ntt, full, tail, 2, 2};
        q.padded = (int)pad8((int64_t)tail * 4);
        e = launch_gemm<T2DenseQuarter, CT>(q, q.padded, st);
      } else {
        auto q = with_cfg<Prob<T2DenseHalf, CT>>(p);
        q.walk = DenseWalk{nft, ntt, full, tail, 2, 1};
        q.padded = (int)pad8((int64_t)tail * 2);
        e = launch_gemm<T2DenseHalf, CT>(q, q.padded, st);
      }
      if (e == hipSuccess && fk && fk->forked) e = hipEventRecord(fk->join, fk->side);
      return e;
    }
  }
  p.padded = (int)pad8(ntiles);
  return launch_gemm<Cfg, CT>(p, p.padded, st);
}

// x-GEMM: any of router logits (fp32 [T, E]), latent z ([T, L]) and the shared
// experts' SiTU-GLU activations (hs [T, S*Is]) from one pass over x.
// z_f32: z is written in fp32 (the W8A8 quantiser's input) instead of the
// act dtype.
template <class Cfg, typename CT>
hipError_t xgemm(const Ctx& c, const void* x, float* logits, void* z, void* hs, bool z_f32 = false,
                 TailFork* fk = nullptr) {
  const lmoe_shape* sh = c.sh;
  DenseXProb<Cfg, CT> p{};
  p.x = static_cast<const char*>(x);
  p.T = sh->T;
  p.K = sh->H;
  p.cap = sh->cap;
  p.inv_cap = c.inv_cap();
  int ns = 0, ft = 0;
  if (logits) {
    NSeg& s = p.seg[ns++];
    s = NSeg{};
    s.w = static_cast<const char*>(c.w->w_router);
    s.out = reinterpret_cast<char*>(logits);
    s.ldo = sh->E;
    s.rows = sh->E;
    s.kind = EPI_F32;
    s.vec = (sh->E % 4) == 0;
    s.ft0 = ft;
    ft += (int)cdiv(sh->E, Cfg::BF);
  }
  if (z) {
    NSeg& s = p.seg[ns++];
    s = NSeg{};
    s.w = static_cast<const char*>(c.w->w_down);
    s.out = static_cast<char*>(z);
    s.ldo = sh->L;
    s.rows = sh->L;
    s.kind = z_f32 ? EPI_F32 : EPI_STORE;
    s.vec = 1;
    s.ft0 = ft;
    ft += (int)cdiv(sh->L, Cfg::BF);
  }
  if (hs) {
    // The S shared experts' gate (value) matrices are consecutive: one GLU
    // segment of S*Is units; hs column s*Is + i is unit i of expert s.
    NSeg& s = p.seg[ns++];
    s = NSeg{};
    s.w = static_cast<const char*>(c.w->ws_gate);
    s.w2 = static_cast<const char*>(c.w->ws_value);
    s.sc = c.w->ss_gate;
    s.sc2 = c.w->ss_value;
    s.f8 = is_f8(sh);
    s.out = static_cast<char*>(hs);
    s.ldo = (int64_t)sh->S * sh->Is;
    s.rows = sh->S * sh->Is;
    s.kind = EPI_GLU;
    s.vec = 1;
    s.ft0 = ft;
    if (fk) fk->defer_ft = ft;
    ft += (int)cdiv((int64_t)sh->S * sh->Is, Cfg::BF / 2);
  }
  if (ns == 0 || sh->T == 0) return hipSuccess;
  p.nseg = ns;
  return launch_dense<Cfg, CT>(p, ft, (int)cdiv(sh->T, Cfg::BT), c.st, fk);
}

// Two fp32 products of x in one pass: out_s = x . w_s^T ([T, rows_s], row
// pitch rows_s) -- the backward's shared gate and value pre-activations.
template <class Cfg, typename CT>
hipError_t xgemm_f32x2(const Ctx& c, const void* x, const void* w0, float* out0, int rows0, const void* w1, float* out1,
                       int rows1) {
  const lmoe_shape* sh = c.sh;
  DenseXProb<Cfg, CT> p{};
  p.x = static_cast<const char*>(x);
  p.T = sh->T;
  p.K = sh->H;
  p.cap = sh->cap;
  p.inv_cap = c.inv_cap();
  int ft = 0;
  const void* ws[2] = {w0, w1};
  float* os[2] = {out0, out1};
  const int rs[2] = {rows0, rows1};
  for (int i = 0; i < 2; ++i) {
    NSeg& s = p.seg[i];
    s = NSeg{};
    s.w = static_cast<const char*>(ws[i]);
    s.out = reinterpret_cast<char*>(os[i]);
    s.ldo = rs[i];
    s.rows = rs[i];
    s.kind = EPI_F32;
    s.vec = (rs[i] % 4) == 0;
    s.ft0 = ft;
    ft += (int)cdiv(rs[i], Cfg::BF);
  }
  if (sh->T == 0) return hipSuccess;
  p.nseg = 2;
  return launch_dense<Cfg, CT>(p, ft, (int)cdiv(sh->T, Cfg::BT), c.st);
}

// y = n . W_up^T + sum_s hs_s . W_so[s]^T  (n added directly when w_up is NULL).
template <class Cfg, typename CT>
hipError_t upgemm(const Ctx& c, const void* n, const void* hs, void* y) {
  const lmoe_shape* sh = c.sh;
  if (sh->T == 0) return hipSuccess;
  UpProb<Cfg, CT> p{};
  p.T = sh->T;
  p.N = sh->H;
  p.y = static_cast<char*>(y);
  p.vec = 1;
  int nk = 0;
  if (c.w->w_up) {
    KSeg& q = p.ks[nk++];
    q.x = static_cast<const char*>(n);
    q.ldx = sh->L;
    q.w = static_cast<const char*>(c.w->w_up);
    q.ldw = sh->L;
    q.nkt = (int)(sh->L * c.es() / 128);
  } else {
    p.addend = static_cast<const char*>(n);
  }
  for (int s = 0; s < sh->S; ++s) {
    KSeg& q = p.ks[nk++];
    q.x = static_cast<const char*>(hs) + (size_t)s * sh->Is * c.es();
    q.ldx = (int64_t)sh->S * sh->Is;
    q.w = static_cast<const char*>(c.w->ws_out) + (size_t)s * sh->H * sh->Is * c.wes();
    q.ldw = sh->Is;
    q.f8 = is_f8(sh);
    if (q.f8) q.sc = c.w->ss_out + (size_t)s * (sh->H / 128) * (sh->Is / 128);
    q.nkt = (int)(sh->Is * c.es() / 128);
  }
  p.nks = nk;
  return launch_dense<Cfg, CT>(p, (int)cdiv(sh->H, Cfg::BF), (int)cdiv(sh->T, Cfg::BT), c.st);
}

// xs: W8A8 row scales (z then holds e4m3 codes), [L/128, T*k] in expert
// order; act is then written in fp32.
template <class Cfg, typename CT>
hipError_t expert_gv(const Ctx& c, const void* z, const int32_t* offsets, const int32_t* sorted,
                     const int4* tiles, const int32_t* tcount, void* act, const float* xs = nullptr) {
  const lmoe_shape* sh = c.sh;
  ExpertGVProb<Cfg, CT, Cfg::XF8 ? 2 : 0> p{};
  p.et.offsets = offsets;
  p.et.tiles = tiles;
  p.et.tile_count = tcount;
  p.et.nft = (int)cdiv(sh->I, Cfg::BF / 2);
  p.z = static_cast<const char*>(z);
  p.ldz = sh->L;
  p.sorted = sorted;
  p.wg = static_cast<const char*>(c.w->w_gate);
  p.wv = static_cast<const char*>(c.w->w_value);
  p.sg = c.w->s_gate;
  p.sv = c.w->s_value;
  p.act = static_cast<char*>(act);
  if constexpr (Cfg::kDma && Cfg::BF == kPackRows) p.wpk = c.pk_gv();
  p.I = sh->I;
  p.L = sh->L;
  p.k = sh->k;
  p.f8 = is_f8(sh);
  p.a8 = xs != nullptr;
  p.xs = xs;
  p.ldxs = sh->T * sh->k;
  p.cap = sh->cap;
  p.inv_cap = c.inv_cap();
  return launch_gemm<Cfg, CT>(p, pad8(max_tiles(sh, Cfg::BT) * p.et.nft), c.st);
}

// xs: W8A8 row scales (act then holds e4m3 codes), [I/128, T*k].
template <class Cfg, typename CT>
hipError_t expert_down(const Ctx& c, const void* act, const int32_t* offsets, const int4* tiles,
                       const int32_t* tcount, void* out, const float* xs = nullptr) {
  const lmoe_shape* sh = c.sh;
  ExpertDownProb<Cfg, CT> p{};
  p.et.offsets = offsets;
  p.et.tiles = tiles;
  p.et.tile_count = tcount;
  p.et.nft = (int)cdiv(sh->L, Cfg::BF);
  p.act = static_cast<const char*>(act);
  p.wo = static_cast<const char*>(c.w->w_out);
  p.so = c.w->s_out;
  p.out = static_cast<char*>(out);
  if constexpr (Cfg::kDma && Cfg::BF == kPackRows) p.wpk = c.pk_dn();
  p.I = sh->I;
  p.L = sh->L;
  p.f8 = is_f8(sh);
  p.a8 = xs != nullptr;
  p.xs = xs;
  p.ldxs = sh->T * sh->k;
  return launch_gemm<Cfg, CT>(p, pad8(max_tiles(sh, Cfg::BT) * p.et.nft), c.st);
}

// Backward data gradients of the routed experts on the persistent engine,
// weights transposed on the way into the MFMAs: out = x0 W0[e] (+ x1 W1[e]),
// x_s [T*k, k_s] bf16 in expert order, W_s [E, k_s, F], out fp32 [T*k, F].
typedef Tile3<256, 256, 4, 4, 0, 1, 0, 3, 0, 1> T2ExpertTGrad;
hipError_t expert_tgrad(const Ctx& c, const int32_t* offsets, const int4* tiles, const int32_t* tcount, int F,
                        const void* x0, const void* w0, int k0, const void* x1, const void* w1, int k1, float* out) {
  using Cfg = T2ExpertTGrad;
  const lmoe_shape* sh = c.sh;
  ExpertTGradProb<Cfg, bf16> p{};
  p.et.offsets = offsets;
  p.et.tiles = tiles;
  p.et.tile_count = tcount;
  p.et.nft = (int)cdiv(F, Cfg::BF);
  p.x[0] = static_cast<const char*>(x0);
  p.w[0] = static_cast<const char*>(w0);
  p.kd[0] = k0;
  p.x[1] = static_cast<const char*>(x1);
  p.w[1] = static_cast<const char*>(w1);
  p.kd[1] = k1;
  p.nseg = x1 ? 2 : 1;
  p.F = F;
  p.out = out;
  return launch_gemm<Cfg, bf16>(p, pad8(max_tiles(sh, Cfg::BT) * p.et.nft), c.st);
}

// Backward data gradients of the dense projections on the persistent engine
// with transposed weight stages: out (+)= sum_s x_s . W_s, x_s bf16 [T, ldx_s]
// with K_s columns, W_s bf16 [K_s, fsplit] per stacked matrix (wms_s
// elements apart), F features, out fp32 [T, ldo].
hipError_t dense_tgrad(const Ctx& c, int nks, const void* const* x, const int64_t* ldx, const int* kd,
                       const void* const* w, const int64_t* wms, int F, int fsplit, float* out, int64_t ldo,
                       int accumulate) {
  using Cfg = T2ExpertTGrad;
  DenseTProb<Cfg, bf16> p{};
  p.T = c.sh->T;
  p.F = F;
  p.fsplit = fsplit;
  p.nks = nks;
  p.ntt = (int)cdiv(c.sh->T, Cfg::BT);
  p.nft = (int)cdiv(F, Cfg::BF);
  for (int s = 0; s < nks; ++s) {
    p.x[s] = static_cast<const char*>(x[s]);
    p.ldx[s] = ldx[s];
    p.kd[s] = kd[s];
    p.w[s] = static_cast<const char*>(w[s]);
    p.wms[s] = wms[s];
  }
  p.out = out;
  p.ldo = ldo;
  p.accumulate = accumulate;
  if (c.sh->T == 0) return hipSuccess;
  return launch_gemm<Cfg, bf16>(p, persistent_grid(), c.st);
}

template <int KR>
hipError_t launch_wgrad_kr(const Ctx& c, const WGradArgs& a) {
  using Cfg = TWGrad;
  auto kern = wgrad3p_kernel<Cfg, KR>;
  static std::once_flag once[kMaxDevices];
  static hipError_t attr[kMaxDevices];
  auto set_attr = [&] {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                               Cfg::LDS);
  };
  const int dev = current_device();
  hipError_t e;
  if (dev < 0 || dev >= kMaxDevices) {
    e = set_attr();
  } else {
    std::call_once(once[dev], [&] { attr[dev] = set_attr(); });
    e = attr[dev];
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)persistent_grid()), dim3(Cfg::NT), Cfg::LDS, c.st, a);
  return hipGetLastError();
}
// routed experts: 32-row stages; dense segments: 64-row stages
hipError_t launch_wgrad(const Ctx& c, const WGradArgs& a) {
  return a.nseg == 0 ? launch_wgrad_kr<32>(c, a) : launch_wgrad_kr<64>(c, a);
}

// Expert weight gradients on the persistent pipeline: C_e = P_e^T Q_e for
// every expert (wgrad.hpp); M and N multiples of 256.
hipError_t wgrad(const Ctx& c, const void* pm, int64_t ldp, const void* qn, int64_t ldq, const int32_t* gather, int gk,
                 float* out, int M, int N, const int32_t* offsets, const void* zero) {
  WGradArgs a{};
  a.p = static_cast<const char*>(pm);
  a.ldp = ldp;
  a.q = static_cast<const char*>(qn);
  a.ldq = ldq;
  a.gather_q = gather;
  a.gk = gk;
  a.c = out;
  a.M = M;
  a.N = N;
  a.E = c.sh->E;
  a.offsets = offsets;
  a.zero = static_cast<const char*>(zero);
  return launch_wgrad(c, a);
}

// Dense weight gradients C_s = P_s^T Q_s over all T rows, up to kWgSegs in
// one launch (wgrad.hpp); each M and N a multiple of 256.
struct WgDense {
  const void* p;
  int64_t ldp;
  const void* q;
  int64_t ldq;
  float* c;
  int M, N;
};
hipError_t wgrad_dense(const Ctx& c, const WgDense* d, int n, const void* zero) {
  if (n < 1 || n > kWgSegs) return hipErrorInvalidValue;
  WGradArgs a{};
  a.nseg = n;
  a.rows = (int)c.sh->T;
  a.zero = static_cast<const char*>(zero);
  int tiles = 0;
  for (int s = 0; s < n; ++s) {
    if (d[s].M % 8 || d[s].M <= 0 || d[s].N % 256) return hipErrorInvalidValue;
    a.seg[s] = WgSeg{static_cast<const char*>(d[s].p), static_cast<const char*>(d[s].q), d[s].c, d[s].ldp, d[s].ldq,
                     d[s].M, d[s].N, tiles};
    tiles += (int)cdiv(d[s].M, 256) * (d[s].N / 256);
  }
  a.tiles = tiles;
  return launch_wgrad(c, a);
}

// Gate and value pre-activations (fp32, assignment order) for the backward's
// recompute, with the forward's persistent bf16 expert GEMM.
hipError_t expert_gv_raw(const Ctx& c, const void* z, const int32_t* offsets, const int32_t* sorted,
                         const int4* tiles, const int32_t* tcount, float* g, float* v) {
  using Cfg = T2ExpertGV;
  const lmoe_shape* sh = c.sh;
  ExpertGVProb<Cfg, bf16, 1> p{};
  p.et.offsets = offsets;
  p.et.tiles = tiles;
  p.et.tile_count = tcount;
  p.et.nft = (int)cdiv(sh->I, Cfg::BF / 2);
  p.z = static_cast<const char*>(z);
  p.ldz = sh->L;
  p.sorted = sorted;
  p.wg = static_cast<const char*>(c.w->w_gate);
  p.wv = static_cast<const char*>(c.w->w_value);
  p.graw = g;
  p.vraw = v;
  p.wpk = c.pk_gv();
  p.I = sh->I;
  p.L = sh->L;
  p.k = sh->k;
  return launch_gemm<Cfg, bf16>(p, pad8(max_tiles(sh, Cfg::BT) * p.et.nft), c.st);
}

// W8A8 gate/value: z (or x) quantised per token -- from fp32 when z_f32 --,
// its row scales put in expert order, then the e4m3 x e4m3 GEMM with the
// SiTU-GLU epilogue writing fp32 act.
hipError_t expert_gv_a8(const Ctx& c, const Plan& pl, void* ws, const void* z, bool z_f32, const int32_t* offsets,
                        const int32_t* sorted, const int4* tiles, const int32_t* tcount, void* act) {
  const lmoe_shape* sh = c.sh;
  hipError_t e =
      launch_quant_1x128(z, z_f32, sh->T, sh->L, at<void>(ws, pl.zq), at<float>(ws, pl.zs_tok), c.st);
  if (e != hipSuccess) return e;
  e = launch_gather_scales(at<float>(ws, pl.zs_tok), sh->T, sh->L / 128, sorted, sh->k, at<float>(ws, pl.zs), c.st);
  if (e != hipSuccess) return e;
  return expert_gv<T2ExpertGVA8, bf16>(c, at<void>(ws, pl.zq), offsets, sorted, tiles, tcount, act,
                                       at<float>(ws, pl.zs));
}
// W8A8 down: the fp32 SiTU-GLU output quantised per row, then the e4m3 x
// e4m3 GEMM.
hipError_t expert_down_a8(const Ctx& c, const Plan& pl, void* ws, const void* act, const int32_t* offsets,
                          const int4* tiles, const int32_t* tcount, void* out) {
  const lmoe_shape* sh = c.sh;
  hipError_t e =
      launch_quant_1x128(act, true, sh->T * sh->k, sh->I, at<void>(ws, pl.aq), at<float>(ws, pl.as), c.st);
  if (e != hipSuccess) return e;
  return expert_down<T2ExpertDnA8, bf16>(c, at<void>(ws, pl.aq), offsets, tiles, tcount, out, at<float>(ws, pl.as));
}

// e4m3 shared experts at prefill sizes: decoded once per call to bf16 in the
// workspace, so that the route and up GEMMs (whose router, down and up
// segments are bf16) run whole on the LDS-DMA kernels.  The view describes a
// layer with bf16 expert weights for those two GEMMs only.
struct DenseView {
  lmoe_shape sh;
  lmoe_weights w;
};
bool shared_to_bf16(const lmoe_shape* sh) {
  return sh->act == LMOE_BF16 && is_f8(sh) && sh->S > 0 && !dense_small(sh);
}
hipError_t dequant_blocks(const void* q, const float* s, int64_t n, int R, int C, void* out, hipStream_t st) {
  const int64_t groups = n * R * (int64_t)(C / 8);
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_blocks_kernel, dim3((unsigned)cdiv(groups, 256)), dim3(256), 0, st,
                     static_cast<const char*>(q), s, n, R, C, static_cast<char*>(out));
  return hipGetLastError();
}
hipError_t dense_view(const Ctx& c, const Plan& pl, void* ws, DenseView& v) {
  v.sh = *c.sh;
  v.w = *c.w;
  if (!shared_to_bf16(c.sh)) return hipSuccess;
  const lmoe_shape* sh = c.sh;
  char* base = at<char>(ws, pl.shared_bf16);
  const size_t one = (size_t)sh->S * sh->Is * sh->H * 2;
  hipError_t e = dequant_blocks(c.w->ws_gate, c.w->ss_gate, sh->S, sh->Is, sh->H, base, c.st);
  if (e == hipSuccess) e = dequant_blocks(c.w->ws_value, c.w->ss_value, sh->S, sh->Is, sh->H, base + one, c.st);
  if (e == hipSuccess) e = dequant_blocks(c.w->ws_out, c.w->ss_out, sh->S, sh->H, sh->Is, base + 2 * one, c.st);
  v.sh.w_expert = LMOE_BF16;
  v.sh.a8 = 0;
  v.w.ws_gate = base;
  v.w.ws_value = base + one;
  v.w.ws_out = base + 2 * one;
  v.w.ss_gate = v.w.ss_value = v.w.ss_out = nullptr;
  return e;
}

// Dispatch on (dtype, tile).
template <typename CT>
hipError_t xgemm_any(const Ctx& c, const void* x, float* logits, void* z, void* hs, bool z_f32 = false,
                    TailFork* fk = nullptr) {
  if constexpr (sizeof(CT) == 2) {
    if (!(hs && is_f8(c.sh)))
      return dense_small(c.sh) ? xgemm<T2Thin, CT>(c, x, logits, z, hs, z_f32)
                               : xgemm<T2Dense, CT>(c, x, logits, z, hs, z_f32, fk);
  }
  return dense_small(c.sh) ? xgemm<CfgSmall, CT>(c, x, logits, z, hs, z_f32)
                           : xgemm<CfgBig, CT>(c, x, logits, z, hs, z_f32);
}
template <typename CT>
hipError_t upgemm_any(const Ctx& c, const void* n, const void* hs, void* y) {
  if constexpr (sizeof(CT) == 2) {
    if (!(c.sh->S > 0 && is_f8(c.sh)))
      return dense_small(c.sh) ? upgemm<T2Thin, CT>(c, n, hs, y) : upgemm<T2Dense, CT>(c, n, hs, y);
  }
  return dense_small(c.sh) ? upgemm<CfgSmall, CT>(c, n, hs, y) : upgemm<CfgBig, CT>(c, n, hs, y);
}

template <typename CT>
hipError_t expert_gv_any(const Ctx& c, const void* z, const int32_t* offsets, const int32_t* sorted,
                         const int4* tiles, const int32_t* tcount, void* act) {
  const ExpertTile t = expert_tile(c.sh);
  if constexpr (sizeof(CT) == 2) {
    if (use_dma_f8(c.sh)) return expert_gv<T2ExpertGVF8, CT>(c, z, offsets, sorted, tiles, tcount, act);
    if (use_dma(c.sh)) {
      if (t == ET_SMALL) return expert_gv<T2SmallGV, CT>(c, z, offsets, sorted, tiles, tcount, act);
      if (t == ET_MID) return expert_gv<T2MidGV, CT>(c, z, offsets, sorted, tiles, tcount, act);
      return expert_gv<T2ExpertGV, CT>(c, z, offsets, sorted, tiles, tcount, act);
    }
  }
  return t == ET_SMALL ? expert_gv<CfgSmall, CT>(c, z, offsets, sorted, tiles, tcount, act)
                       : expert_gv<CfgBig, CT>(c, z, offsets, sorted, tiles, tcount, act);
}
template <typename CT>
hipError_t expert_down_any(const Ctx& c, const void* act, const int32_t* offsets, const int4* tiles,
                           const int32_t* tcount, void* out) {
  const ExpertTile t = expert_tile(c.sh);
  if constexpr (sizeof(CT) == 2) {
    if (use_dma_f8(c.sh)) return expert_down<T2ExpertDnF8, CT>(c, act, offsets, tiles, tcount, out);
    if (use_dma(c.sh)) {
      if (t == ET_SMALL) return expert_down<T2SmallDn, CT>(c, act, offsets, tiles, tcount, out);
      if (t == ET_MID) return expert_down<T2MidDn, CT>(c, act, offsets, tiles, tcount, out);
      return expert_down<T2ExpertDn, CT>(c, act, offsets, tiles, tcount, out);
    }
  }
  return t == ET_SMALL ? expert_down<CfgSmall, CT>(c, act, offsets, tiles, tcount, out)
                       : expert_down<CfgBig, CT>(c, act, offsets, tiles, tcount, out);
}

// Both expert GEMMs plus the tile list they share.
template <typename CT>
hipError_t experts_any(const Ctx& c, const void* z, const int32_t* offsets, const int32_t* sorted, void* act,
                       void* out, int4* tiles, int32_t* tcount) {
  hipError_t e = launch_tiles(offsets, c.sh->E, expert_bt(c.sh), tiles, tcount, 0, nullptr, nullptr, c.st);
  if (e != hipSuccess) return e;
  if ((e = expert_gv_any<CT>(c, z, offsets, sorted, tiles, tcount, act)) != hipSuccess) return e;
  return expert_down_any<CT>(c, act, offsets, tiles, tcount, out);
}

bool bf16_act(const lmoe_shape* sh) { return sh->act == LMOE_BF16; }

lmoe_status record(void* const* ev, int i, hipStream_t st) {
  if (ev && ev[i]) LMOE_HIP(hipEventRecord(static_cast<hipEvent_t>(ev[i]), st), "hipEventRecord");
  return LMOE_OK;
}

// ---------------------------------------------------------------------------
// Backward pass: workspace plan and launch helpers.
// ---------------------------------------------------------------------------
constexpr int kBwChunks = 64;  // token chunks of the dgamma reduction

struct BPlan {
  size_t logits, z, idx, w, bcounts, offsets, sorted, pos, tiles, tcount, tiles2, tcount2;
  size_t G, V, A, dA, dG, dV, O, zr, dO, c, n, dn, dz, r, dw, dl, dl16, gs, vs, hs, dhs, dgs, dvs, dgp, zpage, total;
};

BPlan bplan(const lmoe_shape* sh) {
  BPlan p{};
  const size_t T = (size_t)sh->T, tk = T * sh->k, sis = (size_t)sh->S * (sh->S ? sh->Is : 0);
  const size_t nb = (T + kPermTokens - 1) / kPermTokens;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  p.logits = take(T * sh->E * 4);
  p.z = take(T * sh->L * 2);
  p.idx = take(tk * 4);
  p.w = take(tk * 4);
  p.bcounts = take(nb * sh->E * 4);
  p.offsets = take((size_t)(sh->E + 1) * 4);
  p.sorted = take(tk * 4);
  p.pos = take(tk * 4);
  p.tiles = take((size_t)max_tiles(sh, kBgM) * 16);
  p.tcount = take(8);
  p.tiles2 = take((size_t)max_tiles(sh, T2ExpertGV::BT) * 16);  // the persistent expert GEMMs' tiles
  p.tcount2 = take(8);
  // fp32: GEMM outputs and what elementwise gradients read; bf16: GEMM inputs
  p.G = take(tk * sh->I * 4);
  p.V = take(tk * sh->I * 4);
  p.A = take(tk * sh->I * 2);
  p.dA = take(tk * sh->I * 4);
  p.dG = take(tk * sh->I * 2);
  p.dV = take(tk * sh->I * 2);
  p.O = take(tk * sh->L * 2);
  p.zr = take(tk * sh->L * 4);
  p.dO = take(tk * sh->L * 2);
  p.c = take(T * sh->L * 4);
  p.n = take(T * sh->L * 2);
  p.dn = take(T * sh->L * 4);
  p.dz = take(T * sh->L * 2);
  p.r = take(T * 4);
  p.dw = take(tk * 4);
  p.dl = take(T * sh->E * 4);
  p.dl16 = take(T * sh->E * 2);
  p.gs = take(T * sis * 4);
  p.vs = take(T * sis * 4);
  p.hs = take(T * sis * 2);
  p.dhs = take(T * sis * 4);
  p.dgs = take(T * sis * 2);
  p.dvs = take(T * sis * 2);
  p.dgp = take((size_t)kBwChunks * sh->L * 4);
  p.zpage = take(512);  // zeros, the source of rows past an expert's last (wgrad3p_kernel)
  p.total = off;
  return p;
}

BgOp bop(const void* p, int64_t ld, int64_t gstride = 0, const int* gather = nullptr, int gk = 1, int grow = 0) {
  return BgOp{static_cast<const char*>(p), ld, gstride, gather, gk, grow};
}

template <int MODE, int ARC, int AF32, int BRC, int BF32>
hipError_t bg(BgOp a, BgOp b, void* c, int64_t ldc, int M, int N, int K, int accumulate, hipStream_t st,
              const lmoe_shape* sh, int cbf16 = 0, int64_t cgstride = 0, const int* offsets = nullptr,
              const int4* tiles = nullptr, const int* tcount = nullptr) {
  BgArgs p{a, b, static_cast<char*>(c), ldc, cgstride, M, N, K, accumulate, cbf16, offsets, tiles, tcount};
  dim3 grid((unsigned)cdiv(N, kBgN), 1, 1);
  if (MODE == BG_DENSE) grid.y = (unsigned)cdiv(M, kBgM);
  else if (MODE == BG_GROUP_M) grid.y = (unsigned)max_tiles(sh, kBgM);
  else {
    grid.y = (unsigned)cdiv(M, kBgM);
    grid.z = (unsigned)sh->E;
  }
  if (grid.x == 0 || grid.y == 0 || N <= 0) return hipSuccess;
  hipLaunchKernelGGL((bgemm_kernel<MODE, ARC, AF32, BRC, BF32>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t bw_situ(int mode, const float* g, const float* v, const float* da, void* o1, void* o2, int64_t n,
                   const lmoe_shape* sh, hipStream_t st) {
  if (n == 0) return hipSuccess;
  if (n % 4) return hipErrorInvalidValue;  // whole 4-element groups (I, Is are multiples of 64)
  const float inv = isinf(sh->cap) ? 0.f : 1.f / sh->cap;
  hipLaunchKernelGGL(bw_situ_kernel, dim3((unsigned)cdiv(n / 4, 256)), dim3(256), 0, st, mode, g, v, da,
                     static_cast<unsigned short*>(o1), static_cast<unsigned short*>(o2), n, sh->cap, inv);
  return hipGetLastError();
}

}  // namespace
}  // namespace lmoe

using namespace lmoe;

extern "C" {

const char* lmoe_status_str(lmoe_status s) {
  switch (s) {
    case LMOE_OK: return "LMOE_OK";
    case LMOE_EINVAL: return "LMOE_EINVAL";
    case LMOE_EUNSUPPORTED: return "LMOE_EUNSUPPORTED";
    case LMOE_EWORKSPACE: return "LMOE_EWORKSPACE";
    case LMOE_EHIP: return "LMOE_EHIP";
  }
  return "unknown lmoe_status";
}

const char* lmoe_last_error(void) { return g_err; }

size_t lmoe_workspace_bytes(const lmoe_shape* sh) {
  if (check_shape(sh) != LMOE_OK) return 0;
  return plan(sh).total;
}

lmoe_status lmoe_validate(const lmoe_shape* sh, const lmoe_weights* w, size_t ws_bytes) {
  g_err[0] = 0;
  if (lmoe_status s = check_shape(sh)) return s;
  if (lmoe_status s = check_weights(sh, w, NEED_ROUTE | NEED_EXPERT | NEED_UP | NEED_NORM)) return s;
  const size_t need = plan(sh).total;
  if (ws_bytes < need) return fail(LMOE_EWORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  return LMOE_OK;
}

lmoe_status lmoe_route(const lmoe_shape* sh, const lmoe_weights* w, const void* x, int32_t* topk_idx,
                       float* topk_w, void* z, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (lmoe_status s = check_shape(sh)) return s;
  if (lmoe_status s = check_weights(sh, w, NEED_ROUTE)) return s;
  if (lmoe_status s = check_ws(sh, ws, ws_bytes)) return s;
  if (sh->T == 0) return LMOE_OK;
  if (!x || !topk_idx || !topk_w || (w->w_down && !z)) return fail(LMOE_EINVAL, "x, topk_idx, topk_w, z are required");
  if (lmoe_status s = check_align16({{x, "x"}, {z, "z"}})) return s;
  const Ctx c{sh, w, static_cast<hipStream_t>(stream)};
  const Plan pl = plan(sh);
  float* logits = at<float>(ws, pl.logits);
  void* zz = w->w_down ? z : nullptr;
  LMOE_HIP(bf16_act(sh) ? xgemm_any<bf16>(c, x, logits, zz, nullptr) : xgemm_any<float>(c, x, logits, zz, nullptr),
           "router / down GEMM");
  LMOE_HIP(launch_topk(logits, w->b_router, sh->T, sh->E, sh->k, topk_idx, topk_w, c.st), "top-k");
  return LMOE_OK;
}

lmoe_status lmoe_permute(const lmoe_shape* sh, const int32_t* topk_idx, int32_t* offsets, int32_t* sorted,
                         int32_t* pos, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (lmoe_status s = check_shape(sh)) return s;
  if (lmoe_status s = check_ws(sh, ws, ws_bytes)) return s;
  if (!offsets) return fail(LMOE_EINVAL, "offsets is required");
  if (sh->T > 0 && (!topk_idx || !sorted || !pos)) return fail(LMOE_EINVAL, "topk_idx, sorted, pos are required");
  const Plan pl = plan(sh);
  LMOE_HIP(launch_permute(topk_idx, sh->T, sh->E, sh->k, at<int32_t>(ws, pl.bcounts), offsets, sorted, pos,
                          static_cast<hipStream_t>(stream)),
           "permute");
  return LMOE_OK;
}

lmoe_status lmoe_expert_gemm(const lmoe_shape* sh, const lmoe_weights* w, const void* z, const int32_t* offsets,
                             const int32_t* sorted, void* expert_out, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (lmoe_status s = check_shape(sh)) return s;
  if (lmoe_status s = check_weights(sh, w, NEED_EXPERT)) return s;
  if (lmoe_status s = check_ws(sh, ws, ws_bytes)) return s;
  if (sh->T == 0) return LMOE_OK;
  if (!z || !offsets || !sorted || !expert_out) return fail(LMOE_EINVAL, "z, offsets, sorted, expert_out are required");
  if (lmoe_status s = check_align16({{z, "z"}, {expert_out, "expert_out"}})) return s;
  const Ctx c{sh, w, static_cast<hipStream_t>(stream)};
  const Plan pl = plan(sh);
  void* act = at<void>(ws, pl.act);
  int4* tiles = at<int4>(ws, pl.tiles_a);
  int32_t* tc = at<int32_t>(ws, pl.tcount);
  if (use_a8(sh)) {
    LMOE_HIP(launch_tiles(offsets, sh->E, expert_bt(sh), tiles, tc, 0, nullptr, nullptr, c.st), "tile list");
    LMOE_HIP(expert_gv_a8(c, pl, ws, z, false, offsets, sorted, tiles, tc, act), "expert gate/value GEMM");
    LMOE_HIP(expert_down_a8(c, pl, ws, act, offsets, tiles, tc, expert_out), "expert down GEMM");
    return LMOE_OK;
  }
  LMOE_HIP(bf16_act(sh) ? experts_any<bf16>(c, z, offsets, sorted, act, expert_out, tiles, tc)
                        : experts_any<float>(c, z, offsets, sorted, act, expert_out, tiles, tc),
           "expert GEMMs");
  return LMOE_OK;
}

lmoe_status lmoe_combine_norm(const lmoe_shape* sh, const void* expert_out, const int32_t* pos, const float* topk_w,
                              const float* gamma, void* n, void* stream) {
  g_err[0] = 0;
  if (lmoe_status s = check_shape(sh)) return s;
  if (sh->T == 0) return LMOE_OK;
  if (!expert_out || !pos || !topk_w || !gamma || !n) return fail(LMOE_EINVAL, "null argument");
  if (lmoe_status s = check_align16({{expert_out, "expert_out"}, {n, "n"}})) return s;
  LMOE_HIP(launch_combine_norm(bf16_act(sh), expert_out, pos, topk_w, gamma, sh->T, sh->L, sh->k, sh->rms_eps, n,
                               static_cast<hipStream_t>(stream)),
           "combine + norm");
  return LMOE_OK;
}

lmoe_status lmoe_up(const lmoe_shape* sh, const lmoe_weights* w, const void* n, const void* x, void* y, void* ws,
                    size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (lmoe_status s = check_shape(sh)) return s;
  if (lmoe_status s = check_weights(sh, w, NEED_UP)) return s;
  if (lmoe_status s = check_ws(sh, ws, ws_bytes)) return s;
  if (sh->T == 0) return LMOE_OK;
  if (!n || !y || (sh->S > 0 && !x)) return fail(LMOE_EINVAL, "n, x, y are required");
  if (lmoe_status s = check_align16({{n, "n"}, {x, "x"}, {y, "y"}})) return s;
  const Ctx c0{sh, w, static_cast<hipStream_t>(stream)};
  const Plan pl = plan(sh);
  DenseView dv;
  LMOE_HIP(dense_view(c0, pl, ws, dv), "shared expert decode");
  const Ctx c{&dv.sh, &dv.w, c0.st};
  void* hs = at<void>(ws, pl.hs);
  if (sh->S > 0)
    LMOE_HIP(bf16_act(sh) ? xgemm_any<bf16>(c, x, nullptr, nullptr, hs) : xgemm_any<float>(c, x, nullptr, nullptr, hs),
             "shared gate/value GEMM");
  LMOE_HIP(bf16_act(sh) ? upgemm_any<bf16>(c, n, hs, y) : upgemm_any<float>(c, n, hs, y), "up GEMM");
  return LMOE_OK;
}

}  // extern "C"

namespace lmoe {
namespace {

// overlap: the route GEMM's last round may run on the side stream (not in the
// entry point that must allocate nothing, which makes no events).
lmoe_status forward_impl(const lmoe_shape* sh, const lmoe_weights* w, const void* x, void* y, int32_t* topk_idx,
                         float* topk_w, void* ws, size_t ws_bytes, void* stream, void* const* ev, bool overlap) {
  if (lmoe_status s = lmoe_validate(sh, w, ws_bytes)) return s;
  if (lmoe_status s = check_ws(sh, ws, ws_bytes)) return s;
  if (sh->T == 0) return LMOE_OK;
  if (!x || !y) return fail(LMOE_EINVAL, "x and y are required");
  if (lmoe_status s = check_align16({{x, "x"}, {y, "y"}})) return s;
  const Ctx c{sh, w, static_cast<hipStream_t>(stream)};
  const Plan pl = plan(sh);
  const bool bf = bf16_act(sh);
  float* logits = at<float>(ws, pl.logits);
  // W8A8: z goes to the quantiser in fp32
  const bool zf = use_a8(sh) && w->w_down;
  void* z = w->w_down ? at<void>(ws, zf ? pl.zf : pl.z) : nullptr;
  void* hs = sh->S > 0 ? at<void>(ws, pl.hs) : nullptr;
  void* n = at<void>(ws, pl.n);
  int32_t* idx = topk_idx ? topk_idx : at<int32_t>(ws, pl.idx);
  float* tw = topk_w ? topk_w : at<float>(ws, pl.w);
  int32_t* offsets = at<int32_t>(ws, pl.offsets);
  int32_t* sorted = at<int32_t>(ws, pl.sorted);
  int32_t* pos = at<int32_t>(ws, pl.pos);
  void* act = at<void>(ws, pl.act);
  void* out = at<void>(ws, pl.out);

  if (lmoe_status s = record(ev, 0, c.st)) return s;
  DenseView dv;
  LMOE_HIP(dense_view(c, pl, ws, dv), "shared expert decode");
  const Ctx cd{&dv.sh, &dv.w, c.st};  // route and up GEMMs
  // the side stream belongs to the current device: fork only when `stream`
  // does too
  TailFork fk;
  bool same_dev = c.st == nullptr;
  hipDevice_t sdev = -1;
  if (!same_dev && hipStreamGetDevice(c.st, &sdev) == hipSuccess) same_dev = (int)sdev == current_device();
  fk.side = overlap && hs && same_dev ? side_stream() : nullptr;
  LMOE_HIP(bf ? xgemm_any<bf16>(cd, x, logits, z, hs, zf, &fk) : xgemm_any<float>(cd, x, logits, z, hs), "route GEMM");
  if (lmoe_status s = record(ev, 1, c.st)) return s;
  LMOE_HIP(launch_topk(logits, w->b_router, sh->T, sh->E, sh->k, idx, tw, c.st), "top-k");
  if (lmoe_status s = record(ev, 2, c.st)) return s;
  if (sh->T <= kPermTokens) {
    LMOE_HIP(launch_permute_small(idx, sh->T, sh->E, sh->k, offsets, sorted, pos, expert_bt(sh),
                                  at<int4>(ws, pl.tiles_a), at<int32_t>(ws, pl.tcount), c.st),
             "permute + tile list");
  } else {
    LMOE_HIP(launch_permute(idx, sh->T, sh->E, sh->k, at<int32_t>(ws, pl.bcounts), offsets, sorted, pos, c.st),
             "permute");
    LMOE_HIP(launch_tiles(offsets, sh->E, expert_bt(sh), at<int4>(ws, pl.tiles_a), at<int32_t>(ws, pl.tcount), 0,
                          nullptr, nullptr, c.st),
             "tile list");
  }
  if (lmoe_status s = record(ev, 3, c.st)) return s;
  const void* zin = z ? z : x;
  const int4* tiles = at<int4>(ws, pl.tiles_a);
  const int32_t* tc = at<int32_t>(ws, pl.tcount);
  LMOE_HIP(use_a8(sh) ? expert_gv_a8(c, pl, ws, zin, zf, offsets, sorted, tiles, tc, act)
           : bf      ? expert_gv_any<bf16>(c, zin, offsets, sorted, tiles, tc, act)
                     : expert_gv_any<float>(c, zin, offsets, sorted, tiles, tc, act),
           "expert gate/value GEMM");
  if (lmoe_status s = record(ev, 4, c.st)) return s;
  hipError_t e = use_a8(sh) ? expert_down_a8(c, pl, ws, act, offsets, tiles, tc, out)
                 : bf       ? expert_down_any<bf16>(c, act, offsets, tiles, tc, out)
                            : expert_down_any<float>(c, act, offsets, tiles, tc, out);
  LMOE_HIP(e, "expert down GEMM");
  if (lmoe_status s = record(ev, 5, c.st)) return s;
  LMOE_HIP(launch_combine_norm(bf, out, pos, tw, w->gamma, sh->T, sh->L, sh->k, sh->rms_eps, n, c.st),
           "combine + norm");
  if (lmoe_status s = record(ev, 6, c.st)) return s;
  LMOE_HIP(fk.wait(c.st), "join of the route GEMM's last round");
  LMOE_HIP(bf ? upgemm_any<bf16>(cd, n, hs, y) : upgemm_any<float>(cd, n, hs, y), "up GEMM");
  if (lmoe_status s = record(ev, 7, c.st)) return s;
  return LMOE_OK;
}

}  // namespace
}  // namespace lmoe

// ---------------------------------------------------------------------------
// Scratch of lmoe_forward_noalloc: one array per device in the library's code
// object (device memory that exists from the code object's load on a device
// until the process ends).  Its name in host code is only a host-side
// stand-in; host code resolves each device's address once with
// hipGetSymbolAddress and passes that address to the kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[LMOE_NOALLOC_SCRATCH_BYTES];

namespace lmoe {
namespace {

// Device address of `scratch` on the current device, resolved on the first
// call made on that device (with it current) and kept for the process.
lmoe_status scratch_on_device(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices];
  const int dev = current_device();
  if (dev < 0) return fail(LMOE_EHIP, "hipGetDevice failed");
  if (dev >= kMaxDevices)
    return fail(LMOE_EUNSUPPORTED, "device %d: the no-allocation entry point serves devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    LMOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255)) return fail(LMOE_EHIP, "scratch address %p unusable", p);
    addr[dev] = p;
  }
  *out = addr[dev];
  return LMOE_OK;
}

}  // namespace
}  // namespace lmoe

extern "C" {

lmoe_status lmoe_forward(const lmoe_shape* sh, const lmoe_weights* w, const void* x, void* y, int32_t* topk_idx,
                         float* topk_w, void* ws, size_t ws_bytes, void* stream, void* const* ev) {
  g_err[0] = 0;
  return forward_impl(sh, w, x, y, topk_idx, topk_w, ws, ws_bytes, stream, ev, true);
}

lmoe_status lmoe_forward_noalloc(const lmoe_shape* sh, const lmoe_weights* w, const void* x, void* y,
                                 int32_t* topk_idx, float* topk_w, void* stream) {
  g_err[0] = 0;
  if (lmoe_status s = check_shape(sh)) return s;
  const size_t need = plan(sh).total;
  if (need > LMOE_NOALLOC_SCRATCH_BYTES)
    return fail(LMOE_EWORKSPACE,
                "this layer call needs %zu bytes of scratch; lmoe_forward_noalloc holds %zu per device "
                "(call lmoe_forward with a workspace instead)",
                need, (size_t)LMOE_NOALLOC_SCRATCH_BYTES);
  if (lmoe_status s = check_weights(sh, w, NEED_ROUTE | NEED_EXPERT | NEED_UP | NEED_NORM)) return s;
  if (sh->T == 0) return LMOE_OK;
  void* ws = nullptr;
  if (lmoe_status s = scratch_on_device(&ws)) return s;
  return forward_impl(sh, w, x, y, topk_idx, topk_w, ws, LMOE_NOALLOC_SCRATCH_BYTES, stream, nullptr, false);
}

lmoe_status lmoe_router_logits(const lmoe_shape* sh, const lmoe_weights* w, const void* x, float* logits,
                               void* stream) {
  g_err[0] = 0;
  if (lmoe_status s = check_shape(sh)) return s;
  if (!w || !w->w_router) return fail(LMOE_EINVAL, "w_router is required");
  if (sh->T == 0) return LMOE_OK;
  if (!x || !logits) return fail(LMOE_EINVAL, "x and logits are required");
  if (lmoe_status s = check_align16({{x, "x"}, {w->w_router, "w_router"}, {logits, "logits"}})) return s;
  const Ctx c{sh, w, static_cast<hipStream_t>(stream)};
  LMOE_HIP(bf16_act(sh) ? xgemm_any<bf16>(c, x, logits, nullptr, nullptr) : xgemm_any<float>(c, x, logits, nullptr,
                                                                                               nullptr),
           "router GEMM");
  return LMOE_OK;
}

lmoe_status lmoe_quantile_bias(const lmoe_shape* sh, const float* logits, float* bias, void* ws, size_t ws_bytes,
                               void* stream) {
  g_err[0] = 0;
  if (lmoe_status s = check_shape(sh)) return s;
  if (sh->T < 1) return fail(LMOE_EINVAL, "quantile thresholds need at least one token");
  if ((sh->T + 63) / 64 > 65535) return fail(LMOE_EUNSUPPORTED, "T = %lld is too large", (long long)sh->T);
  if (!logits || !bias) return fail(LMOE_EINVAL, "logits and bias are required");
  if (lmoe_status s = check_ws(sh, ws, ws_bytes)) return s;
  LMOE_HIP(launch_quantile_bias(logits, sh->T, sh->E, sh->k, at<uint32_t>(ws, plan(sh).logits), bias,
                                static_cast<hipStream_t>(stream)),
           "quantile thresholds");
  return LMOE_OK;
}

lmoe_status lmoe_quantize_1x128(const void* x, int64_t R, int32_t C, void* q, float* scales, void* stream) {
  g_err[0] = 0;
  if (R < 0) return fail(LMOE_EINVAL, "R = %lld < 0", (long long)R);
  if (C <= 0 || C % 128) return fail(LMOE_EINVAL, "C = %d is not a positive multiple of 128", C);
  if (R == 0) return LMOE_OK;
  if (!x || !q || !scales) return fail(LMOE_EINVAL, "x, q and scales are required");
  if ((reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(q) & 7) ||
      (reinterpret_cast<uintptr_t>(scales) & 3))
    return fail(LMOE_EINVAL, "x must be 16-byte, q 8-byte and scales 4-byte aligned");
  if (R * (int64_t)(C / 128) > (int64_t)INT32_MAX * 16) return fail(LMOE_EUNSUPPORTED, "too many blocks");
  LMOE_HIP(launch_quant_1x128(x, false, R, C, q, scales, static_cast<hipStream_t>(stream)), "1x128 quantisation");
  return LMOE_OK;
}

// ---------------------------------------------------------------------------
// Backward pass.
// ---------------------------------------------------------------------------
#ifndef LMOE_BW_TGRAD
#define LMOE_BW_TGRAD 1
#endif
#ifndef LMOE_BW_WGRAD
#define LMOE_BW_WGRAD 1
#endif
#ifndef LMOE_BW_DENSE_TGRAD
#define LMOE_BW_DENSE_TGRAD 1
#endif
#ifndef LMOE_BW_DENSE_WGRAD
#define LMOE_BW_DENSE_WGRAD 1
#endif
size_t lmoe_backward_workspace_bytes(const lmoe_shape* sh) {
  if (check_shape(sh) != LMOE_OK) return 0;
  return bplan(sh).total;
}

lmoe_status lmoe_backward(const lmoe_shape* sh, const lmoe_weights* w, const void* x, const void* dy,
                          int32_t* topk_idx, const lmoe_grads* gr, void* ws, size_t ws_bytes, void* stream,
                          void* const* ev) {
  g_err[0] = 0;
  if (lmoe_status s = check_shape(sh)) return s;
  if (!(sh->act == LMOE_BF16 && sh->w_expert == LMOE_BF16) || sh->a8)
    return fail(LMOE_EUNSUPPORTED, "the backward pass takes BF16 layers with BF16 expert weights (no a8)");
  if (lmoe_status s = check_weights(sh, w, NEED_ROUTE | NEED_EXPERT | NEED_UP | NEED_NORM)) return s;
  if (sh->T > 65535) return fail(LMOE_EUNSUPPORTED, "the backward pass takes at most 65535 tokens per call");
  if (!w->w_gate || !w->w_value || !w->w_out) return fail(LMOE_EINVAL, "the backward reads row-major w_gate, w_value, w_out");
  if (!gr) return fail(LMOE_EINVAL, "grads is NULL");
  if ((!gr->dx && sh->T > 0) || !gr->dw_router || !gr->dw_gate || !gr->dw_value || !gr->dw_out || !gr->dgamma ||
      (w->w_down && !gr->dw_down) || (w->w_up && !gr->dw_up) ||
      (sh->S > 0 && (!gr->dws_gate || !gr->dws_value || !gr->dws_out)))
    return fail(LMOE_EINVAL, "a gradient pointer is NULL");
  const BPlan pl = bplan(sh);
  if (ws_bytes < pl.total) return fail(LMOE_EWORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, pl.total);
  if (!ws) return fail(LMOE_EINVAL, "ws is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(LMOE_EINVAL, "ws must be 256-byte aligned");
  if (sh->T > 0 && (!x || !dy)) return fail(LMOE_EINVAL, "x and dy are required");
  if (lmoe_status s = check_align16({{x, "x"}, {dy, "dy"}, {gr->dx, "dx"}, {gr->dw_router, "dw_router"},
                                      {gr->dw_down, "dw_down"}, {gr->dw_gate, "dw_gate"}, {gr->dw_value, "dw_value"},
                                      {gr->dw_out, "dw_out"}, {gr->dw_up, "dw_up"}, {gr->dws_gate, "dws_gate"},
                                      {gr->dws_value, "dws_value"}, {gr->dws_out, "dws_out"}}))
    return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int T = (int)sh->T, H = sh->H, L = sh->L, E = sh->E, k = sh->k, I = sh->I, S = sh->S, Is = sh->Is;
  const int tk = T * k, sis = S * Is;
  float* logits = at<float>(ws, pl.logits);
  int32_t* idx = topk_idx ? topk_idx : at<int32_t>(ws, pl.idx);
  float* tw = at<float>(ws, pl.w);
  int32_t* offsets = at<int32_t>(ws, pl.offsets);
  int32_t* sorted = at<int32_t>(ws, pl.sorted);
  int32_t* pos = at<int32_t>(ws, pl.pos);
  int4* tiles = at<int4>(ws, pl.tiles);
  int32_t* tc = at<int32_t>(ws, pl.tcount);
  float *G = at<float>(ws, pl.G), *V = at<float>(ws, pl.V), *dA = at<float>(ws, pl.dA), *zr = at<float>(ws, pl.zr);
  float *c = at<float>(ws, pl.c), *dn = at<float>(ws, pl.dn), *r = at<float>(ws, pl.r), *dw = at<float>(ws, pl.dw);
  unsigned short* dl16 = at<unsigned short>(ws, pl.dl16);
  float *dl = at<float>(ws, pl.dl), *gs = at<float>(ws, pl.gs), *vs = at<float>(ws, pl.vs), *dhs = at<float>(ws, pl.dhs);
  unsigned short *A = at<unsigned short>(ws, pl.A), *dG = at<unsigned short>(ws, pl.dG), *dV = at<unsigned short>(ws, pl.dV);
  unsigned short *dO = at<unsigned short>(ws, pl.dO), *n = at<unsigned short>(ws, pl.n), *dz = at<unsigned short>(ws, pl.dz);
  unsigned short* O = at<unsigned short>(ws, pl.O);
  const Ctx cx{sh, w, st};
  unsigned short *hs = at<unsigned short>(ws, pl.hs), *dgs = at<unsigned short>(ws, pl.dgs), *dvs = at<unsigned short>(ws, pl.dvs);
  const void* zsrc = w->w_down ? at<void>(ws, pl.z) : x;

  // --- forward, keeping what the gradients need ---------------------------
  if (lmoe_status s = record(ev, 0, st)) return s;
  if (T > 0) {
    // router logits and z through the forward's route GEMM (the same kernels
    // and tiles as lmoe_forward, so the same sums)
    LMOE_HIP(xgemm_any<bf16>(cx, x, logits, w->w_down ? at<void>(ws, pl.z) : nullptr, nullptr), "router + latent down");
    LMOE_HIP(launch_topk(logits, w->b_router, sh->T, E, k, idx, tw, st), "top-k");
  }
  LMOE_HIP(launch_permute(idx, sh->T, E, k, at<int32_t>(ws, pl.bcounts), offsets, sorted, pos, st), "permute");
  int4* tiles2 = at<int4>(ws, pl.tiles2);
  int32_t* tc2 = at<int32_t>(ws, pl.tcount2);
  LMOE_HIP(launch_tiles(offsets, E, kBgM, tiles, tc, T2ExpertGV::BT, tiles2, tc2, st), "tile lists");
  // the routed experts as the forward computes them (O in bf16), keeping the
  // gate and value pre-activations
  if (T > 0) {
    LMOE_HIP(expert_gv_raw(cx, zsrc, offsets, sorted, tiles2, tc2, G, V), "expert gate/value");
    LMOE_HIP(bw_situ(0, G, V, nullptr, A, nullptr, (int64_t)tk * I, sh, st), "SiTU-GLU");
    LMOE_HIP((expert_down<T2ExpertDn, bf16>(cx, A, offsets, tiles2, tc2, O)), "expert down");
  }
  if (T > 0)
    LMOE_HIP(launch_combine_norm(true, O, pos, tw, w->gamma, T, L, k, sh->rms_eps, n, st, c, r), "combine + RMSNorm");
  LMOE_HIP(hipGetLastError(), "combine + norm");

  if (lmoe_status s = record(ev, 1, st)) return s;
  // --- up-projection ------------------------------------------------------
  // dense data gradients on the persistent engine above 256 tokens
  const bool dtg = T > 256 && LMOE_BW_DENSE_TGRAD;
  // The dense weight gradients whose matrices have whole 256-column tiles
  // (and rows in multiples of 8) are queued and run together at the end on
  // the persistent weight-gradient pipeline (their inputs all stay in the
  // workspace until then).
  WgDense dseg[kWgSegs];
  int nd = 0;
  auto add_dense = [&](const void* pp, int64_t ldp, const void* qq, int64_t ldq, float* cc, int M, int N) {
    if (!(T > 256 && LMOE_BW_DENSE_WGRAD) || M % 8 || N % 256 || nd == kWgSegs) return false;
    dseg[nd++] = WgDense{pp, ldp, qq, ldq, cc, M, N};
    return true;
  };
  if (w->w_up) {
    if (dtg) {
      const void* xs[1] = {dy};
      const int64_t lx[1] = {H};
      const int kd[1] = {H};
      const void* wsrc[1] = {w->w_up};
      const int64_t wm[1] = {0};
      LMOE_HIP(dense_tgrad(cx, 1, xs, lx, kd, wsrc, wm, L, L, dn, L, 0), "dn");
    } else {
      LMOE_HIP((bg<BG_DENSE, 0, 0, 1, 0>(bop(dy, H), bop(w->w_up, L), dn, L, T, L, H, 0, st, sh)), "dn");
    }
    if (!add_dense(dy, H, n, L, gr->dw_up, H, L))
      LMOE_HIP((bg<BG_DENSE, 1, 0, 1, 0>(bop(dy, H), bop(n, L), gr->dw_up, L, H, L, T, 0, st, sh)), "dW_up");
  } else if (T > 0) {
    hipLaunchKernelGGL(bw_widen_kernel, dim3((unsigned)cdiv((int64_t)T * L, 256)), dim3(256), 0, st,
                       static_cast<const unsigned short*>(dy), dn, (int64_t)T * L);
    LMOE_HIP(hipGetLastError(), "dn");
  }
  // --- RMSNorm and combine ------------------------------------------------
  if (T > 0) {
    if (L <= 2 * 256 * 8)
      hipLaunchKernelGGL(bw_norm_combine_grad_kernel<2>, dim3(T), dim3(256), 0, st, dn, c, r, w->gamma, O, pos, tw, L, k,
                         dO, dw);
    else
      hipLaunchKernelGGL(bw_norm_combine_grad_kernel<4>, dim3(T), dim3(256), 0, st, dn, c, r, w->gamma, O, pos, tw, L, k,
                         dO, dw);
  }
  LMOE_HIP(hipGetLastError(), "norm / combine gradient");
  {
    const int64_t chunk = cdiv(std::max<int64_t>(sh->T, 1), kBwChunks);
    const int rows = (int)cdiv(std::max<int64_t>(sh->T, 1), chunk);
    hipLaunchKernelGGL(bw_dgamma_part_kernel, dim3((unsigned)cdiv(L, 256), rows), dim3(256), 0, st, dn, c, r, sh->T, L,
                       chunk, at<float>(ws, pl.dgp));
    hipLaunchKernelGGL(bw_sum_rows_kernel, dim3((unsigned)cdiv(L, 256)), dim3(256), 0, st, at<float>(ws, pl.dgp), rows,
                       L, gr->dgamma);
    LMOE_HIP(hipGetLastError(), "dgamma");
  }
  if (lmoe_status s = record(ev, 2, st)) return s;
  // --- routed experts -----------------------------------------------------
  // The grouped data gradients run on the persistent engine with transposed
  // weight stages when its 256-row token tiles fit the batch (its tile list
  // is the forward's); the register-staged grouped GEMM otherwise.
  const bool tgrad = T > 256 && LMOE_BW_TGRAD;
  if (tgrad) {
    LMOE_HIP(expert_tgrad(cx, offsets, tiles2, tc2, I, dO, w->w_out, L, nullptr, nullptr, 0, dA), "dA");
  } else {
    LMOE_HIP((bg<BG_GROUP_M, 0, 0, 1, 0>(bop(dO, L, 0, nullptr, 1, 1), bop(w->w_out, I, (int64_t)L * I), dA, I, 0, I, L,
                                         0, st, sh, 0, 0, offsets, tiles, tc)),
             "dA");
  }
  // The weight gradients take the persistent pipeline above 256 tokens when
  // their matrices are whole 256 x 256 tiles.
  const bool wg3 = T > 256 && I % 256 == 0 && L % 256 == 0 && LMOE_BW_WGRAD;
  void* zpage = at<void>(ws, pl.zpage);
  auto zero_page = [&]() -> hipError_t {
    hipLaunchKernelGGL(zero_page_kernel, dim3(1), dim3(128), 0, st, static_cast<uint32_t*>(zpage));
    return hipGetLastError();
  };
  if (wg3) LMOE_HIP(zero_page(), "zero page");
  if (wg3) {
    LMOE_HIP(wgrad(cx, dO, L, A, I, nullptr, 1, gr->dw_out, L, I, offsets, zpage), "dW_out");
  } else {
    LMOE_HIP((bg<BG_GROUP_K, 1, 0, 1, 0>(bop(dO, L, 0, nullptr, 1, 1), bop(A, I, 0, nullptr, 1, 1), gr->dw_out, I, L, I,
                                         0, 0, st, sh, 0, (int64_t)L * I, offsets)),
             "dW_out");
  }
  LMOE_HIP(bw_situ(1, G, V, dA, dG, dV, (int64_t)tk * I, sh, st), "SiTU-GLU gradient");
  if (tgrad) {
    LMOE_HIP(expert_tgrad(cx, offsets, tiles2, tc2, L, dG, w->w_gate, I, dV, w->w_value, I, zr), "dz rows");
  } else {
    LMOE_HIP((bg<BG_GROUP_M, 0, 0, 1, 0>(bop(dG, I, 0, nullptr, 1, 1), bop(w->w_gate, L, (int64_t)I * L), zr, L, 0, L, I,
                                         0, st, sh, 0, 0, offsets, tiles, tc)),
             "dz rows (gate)");
    LMOE_HIP((bg<BG_GROUP_M, 0, 0, 1, 0>(bop(dV, I, 0, nullptr, 1, 1), bop(w->w_value, L, (int64_t)I * L), zr, L, 0, L, I,
                                         1, st, sh, 0, 0, offsets, tiles, tc)),
             "dz rows (value)");
  }
  if (wg3) {
    LMOE_HIP(wgrad(cx, dG, I, zsrc, L, sorted, k, gr->dw_gate, I, L, offsets, zpage), "dW_gate");
    LMOE_HIP(wgrad(cx, dV, I, zsrc, L, sorted, k, gr->dw_value, I, L, offsets, zpage), "dW_value");
  } else {
    LMOE_HIP((bg<BG_GROUP_K, 1, 0, 1, 0>(bop(dG, I, 0, nullptr, 1, 1), bop(zsrc, L, 0, sorted, k, 1), gr->dw_gate, L, I,
                                         L, 0, 0, st, sh, 0, (int64_t)I * L, offsets)),
             "dW_gate");
    LMOE_HIP((bg<BG_GROUP_K, 1, 0, 1, 0>(bop(dV, I, 0, nullptr, 1, 1), bop(zsrc, L, 0, sorted, k, 1), gr->dw_value, L, I,
                                         L, 0, 0, st, sh, 0, (int64_t)I * L, offsets)),
             "dW_value");
  }
  if (lmoe_status s = record(ev, 3, st)) return s;
  // --- latent projection, router and dx ----------------------------------------
  if (T > 0) {
    hipLaunchKernelGGL(bw_gather_sum_kernel, dim3((unsigned)cdiv(L, 1024), T), dim3(256), 0, st, zr, pos, L, k,
                       w->w_down ? nullptr : gr->dx, w->w_down ? dz : nullptr);
    LMOE_HIP(hipGetLastError(), "dz");
    // the router's logit gradients, fp32 and bf16 (the GEMMs below read them
    // in bf16 either way)
    hipLaunchKernelGGL(bw_route_grad_kernel, dim3(T), dim3(256), 0, st, logits, idx, dw, E, k, dl, dl16);
    LMOE_HIP(hipGetLastError(), "router gradient");
  }
  // dx = dz W_dn + dl W_r as one pass of the persistent engine when the
  // router's K (E) is whole 64-column k-tiles
  const bool rtg = dtg && E % 64 == 0;
  if (w->w_down) {
    if (dtg) {
      const void* xs[2] = {dz, dl16};
      const int64_t lx[2] = {L, E};
      const int kd[2] = {L, E};
      const void* wsrc[2] = {w->w_down, w->w_router};
      const int64_t wm[2] = {0, 0};
      LMOE_HIP(dense_tgrad(cx, rtg ? 2 : 1, xs, lx, kd, wsrc, wm, H, H, gr->dx, H, 0), "dx (latent + router)");
    } else {
      LMOE_HIP((bg<BG_DENSE, 0, 0, 1, 0>(bop(dz, L), bop(w->w_down, H), gr->dx, H, T, H, L, 0, st, sh)), "dx (latent)");
    }
    if (!add_dense(dz, L, x, H, gr->dw_down, L, H))
      LMOE_HIP((bg<BG_DENSE, 1, 0, 1, 0>(bop(dz, L), bop(x, H), gr->dw_down, H, L, H, T, 0, st, sh)), "dW_down");
  } else if (rtg) {
    const void* xs[1] = {dl16};
    const int64_t lx[1] = {E};
    const int kd[1] = {E};
    const void* wsrc[1] = {w->w_router};
    const int64_t wm[1] = {0};
    LMOE_HIP(dense_tgrad(cx, 1, xs, lx, kd, wsrc, wm, H, H, gr->dx, H, 1), "dx (router)");
  }
  if (!rtg)
    LMOE_HIP((bg<BG_DENSE, 0, 1, 1, 0>(bop(dl, E), bop(w->w_router, H), gr->dx, H, T, H, E, 1, st, sh)), "dx (router)");
  // dW_router (E rows; the last 256-row tile partial) joins the dense weight
  // gradients when E is a multiple of 8, else the register-staged GEMM
  if (!add_dense(dl16, E, x, H, gr->dw_router, E, H))
    LMOE_HIP((bg<BG_DENSE, 1, 1, 1, 0>(bop(dl, E), bop(x, H), gr->dw_router, H, E, H, T, 0, st, sh)), "dW_router");
  if (lmoe_status s = record(ev, 4, st)) return s;
  // --- shared experts ---------------------------------------------------------
  if (S > 0) {
    if (T > 256) {
      LMOE_HIP((xgemm_f32x2<T2Dense, bf16>(cx, x, w->ws_gate, gs, sis, w->ws_value, vs, sis)), "shared gate + value");
    } else {
      LMOE_HIP((bg<BG_DENSE, 0, 0, 0, 0>(bop(x, H), bop(w->ws_gate, H), gs, sis, T, sis, H, 0, st, sh)), "shared gate");
      LMOE_HIP((bg<BG_DENSE, 0, 0, 0, 0>(bop(x, H), bop(w->ws_value, H), vs, sis, T, sis, H, 0, st, sh)), "shared value");
    }
    LMOE_HIP(bw_situ(0, gs, vs, nullptr, hs, nullptr, (int64_t)T * sis, sh, st), "shared SiTU-GLU");
    // dh = dy [W_so[0] | W_so[1] ...] in one pass (a feature tile may span
    // two matrices: each 8-feature chunk finds its own)
    const bool dh1 = dtg;
    if (dh1) {
      const void* xs[1] = {dy};
      const int64_t lx[1] = {H};
      const int kd[1] = {H};
      const void* wsrc[1] = {w->ws_out};
      const int64_t wm[1] = {(int64_t)H * Is};
      LMOE_HIP(dense_tgrad(cx, 1, xs, lx, kd, wsrc, wm, sis, Is, dhs, sis, 0), "shared dh");
    }
    for (int s = 0; s < S; ++s) {
      const char* wso = static_cast<const char*>(w->ws_out) + (size_t)s * H * Is * 2;
      if (!dh1)
        LMOE_HIP((bg<BG_DENSE, 0, 0, 1, 0>(bop(dy, H), bop(wso, Is), dhs + (size_t)s * Is, sis, T, Is, H, 0, st, sh)),
                 "shared dh");
      if (!add_dense(dy, H, hs + (size_t)s * Is, sis, gr->dws_out + (size_t)s * H * Is, H, Is))
        LMOE_HIP((bg<BG_DENSE, 1, 0, 1, 0>(bop(dy, H), bop(hs + (size_t)s * Is, sis), gr->dws_out + (size_t)s * H * Is,
                                           Is, H, Is, T, 0, st, sh)),
                 "dWs_out");
    }
    LMOE_HIP(bw_situ(1, gs, vs, dhs, dgs, dvs, (int64_t)T * sis, sh, st), "shared SiTU-GLU gradient");
    if (dtg) {
      const void* xs[2] = {dgs, dvs};
      const int64_t lx[2] = {sis, sis};
      const int kd[2] = {sis, sis};
      const void* wsrc[2] = {w->ws_gate, w->ws_value};
      const int64_t wm[2] = {0, 0};
      LMOE_HIP(dense_tgrad(cx, 2, xs, lx, kd, wsrc, wm, H, H, gr->dx, H, 1), "dx (shared)");
    } else {
      LMOE_HIP((bg<BG_DENSE, 0, 0, 1, 0>(bop(dgs, sis), bop(w->ws_gate, H), gr->dx, H, T, H, sis, 1, st, sh)),
               "dx (shared gate)");
      LMOE_HIP((bg<BG_DENSE, 0, 0, 1, 0>(bop(dvs, sis), bop(w->ws_value, H), gr->dx, H, T, H, sis, 1, st, sh)),
               "dx (shared value)");
    }
    if (!add_dense(dgs, sis, x, H, gr->dws_gate, sis, H))
      LMOE_HIP((bg<BG_DENSE, 1, 0, 1, 0>(bop(dgs, sis), bop(x, H), gr->dws_gate, H, sis, H, T, 0, st, sh)), "dWs_gate");
    if (!add_dense(dvs, sis, x, H, gr->dws_value, sis, H))
      LMOE_HIP((bg<BG_DENSE, 1, 0, 1, 0>(bop(dvs, sis), bop(x, H), gr->dws_value, H, sis, H, T, 0, st, sh)), "dWs_value");
  }
  if (nd > 0) {
    if (!wg3) LMOE_HIP(zero_page(), "zero page");
    LMOE_HIP(wgrad_dense(cx, dseg, nd, zpage), "dense weight gradients");
  }
  if (lmoe_status s = record(ev, 5, st)) return s;
  return LMOE_OK;
}

size_t lmoe_packed_bytes(const lmoe_shape* sh) {
  if (check_shape(sh) != LMOE_OK) return 0;
  if (!(sh->act == LMOE_BF16 && sh->w_expert == LMOE_BF16)) return 0;
  return (size_t)(packed_gv_blocks(sh) + packed_dn_blocks(sh)) * kPackBlock;
}

lmoe_status lmoe_pack_experts(const lmoe_shape* sh, const lmoe_weights* w, void* packed, size_t bytes, void* stream) {
  g_err[0] = 0;
  if (lmoe_status s = check_shape(sh)) return s;
  if (!(sh->act == LMOE_BF16 && sh->w_expert == LMOE_BF16))
    return fail(LMOE_EUNSUPPORTED, "packed expert weights need a BF16 layer with BF16 expert weights");
  if (!w || !w->w_gate || !w->w_value || !w->w_out) return fail(LMOE_EINVAL, "w_gate, w_value and w_out are required");
  if (!packed) return fail(LMOE_EINVAL, "packed is NULL");
  if (reinterpret_cast<uintptr_t>(packed) & 255) return fail(LMOE_EINVAL, "packed must be 256-byte aligned");
  const size_t need = lmoe_packed_bytes(sh);
  if (bytes < need) return fail(LMOE_EINVAL, "packed buffer of %zu bytes, %zu needed", bytes, need);
  const int64_t blocks = packed_gv_blocks(sh) + packed_dn_blocks(sh);
  if (blocks >= (int64_t(1) << 31)) return fail(LMOE_EUNSUPPORTED, "too many packed blocks");
  hipLaunchKernelGGL(pack_experts_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const char*>(w->w_gate), static_cast<const char*>(w->w_value),
                     static_cast<const char*>(w->w_out), static_cast<char*>(packed), sh->E, sh->I, sh->L);
  LMOE_HIP(hipGetLastError(), "pack experts");
  return LMOE_OK;
}

}  // extern "C"
