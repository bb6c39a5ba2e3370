// Host entry points of libmoe (the C ABI declared in include/moe.h).
//
// Argument validation happens here, before anything is enqueued; every
// kernel launch goes to the caller's stream.  The plan is host memory owned
// by the library; every device buffer belongs to the caller.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "common.h"

namespace moe {

hipError_t launch_route(const int32_t* ids, int64_t T, int K, int E, char* ws,
                        const RouteLayout& L, hipStream_t s);
hipError_t launch_plan_decide(RouteHdr* hdr, const PlanArgs& a, hipStream_t s);
hipError_t launch_plan_rewind(RouteHdr* hdr, void* arena, hipStream_t s);
hipError_t launch_plan_enter_bwd(RouteHdr* hdr, const PlanArgs& a, hipStream_t s);
hipError_t launch_arena_reset(void* arena, hipStream_t s);
hipError_t launch_gather(const void* x, int64_t D, int es, int K, const RouteHdr* hdr,
                         const int32_t* route_to_row, void* dst, int64_t T_max, hipStream_t s);
hipError_t launch_zero_rows_f32(const RouteHdr* hdr, float* p, int64_t D, int64_t T_max,
                                hipStream_t s);
hipError_t launch_flush(void* p, int64_t bytes, uint32_t v, hipStream_t s);
hipError_t launch_fused_finish(int prec, const RouteHdr* hdr, const int32_t* route_to_row,
                               const float* scores, const float* y32, const void* addend,
                               void* y, int K, int64_t D, int64_t T_max, uint32_t* status,
                               hipStream_t s);
hipError_t launch_combine(int prec, const RouteHdr* hdr, const int32_t* route_to_row,
                          const float* scores, const void* h3, const void* addend, void* y,
                          int K, int64_t D, int64_t T_max, uint32_t* status, hipStream_t s);
hipError_t launch_combine_bwd(int prec, const RouteHdr* hdr, const int32_t* route_to_row,
                              const float* scores, const void* dy, const void* h3, void* dh3,
                              float* dscores, int K, int64_t D, int64_t T_max, hipStream_t s);
hipError_t launch_dx_reduce(int prec, const RouteHdr* hdr, const int32_t* route_to_row,
                            const float* dxr, void* dx, int K, int64_t D, int64_t T_max,
                            int accumulate, hipStream_t s);
hipError_t launch_gemm_mega(int prec, const FwdArgs& a13, const FwdArgs& a2, uint32_t* msync,
                            int look, int64_t mt_max, int cus, hipStream_t s);
hipError_t launch_gemm_fwd(int prec, int mode, const FwdArgs& a, int64_t mt_max, int cus,
                           hipStream_t s);
hipError_t launch_dgrad(int kind, const BwdArgs& a, int64_t mt_max, int cus, hipStream_t s);
hipError_t launch_prep_w(const void* w, void* q, void* s, int E, int N, int K, hipStream_t st);
hipError_t launch_rowq(const RowqArgs& a, int64_t R_max, hipStream_t st);
hipError_t launch_colq(const ColqArgs& a, int64_t Rpad_max, hipStream_t st);
hipError_t launch_mx_fwd(int mode, const MxArgs& a, int64_t mt_max, int cus, hipStream_t s);
hipError_t launch_mx_mega(const MxArgs& a13, const MxArgs& a2, uint32_t* msync, int look,
                          int64_t mt_max, int cus, hipStream_t s);
hipError_t launch_mx_dgrad(int kind, const MxArgs& a, int64_t mt_max, int cus, hipStream_t s);
hipError_t launch_mx_wgrad(int dw_f32, int tag, const MxArgs& a, int cus, hipStream_t s);
hipError_t launch_mx_bwd_mega(int kind, int dw_f32, const MxArgs& dg, const MxArgs& wg,
                              uint32_t* tickets, int cus, hipStream_t s);
hipError_t launch_wgrad(int dw_f32, int tag, const BwdArgs& a, int cus, hipStream_t s);
hipError_t launch_bwd_mega(int kind, int dw_f32, const BwdArgs& dg, const BwdArgs& wg,
                           uint32_t* tickets, uint32_t* ready, int cus, hipStream_t s);
}  // namespace moe

using namespace moe;

struct moe_plan_s {
  moe_desc d;
  int es;                 // activation element bytes
  int64_t R_max;          // t_max * K
  int64_t Rp_max;         // upper bound on rows padded to 32 per expert
  int64_t mt_max;         // upper bound on m-tiles
  bool hot;               // BF16 forward: hot experts on the 256 x 256 MFMA tiles
  int ks13, ks2;          // forward split-K factors of the W13 and W2 GEMMs (1: none)
  RouteLayout rl;
  ScratchLayout sl;
  int64_t h3_bytes;
  int64_t state_max;      // one layer's full saved state at R_max
  int64_t budget;         // arena data bytes
  int64_t arena_bytes;
  int cus;                // compute units (queried at first launch)
  struct TimerSlot {
    std::string name;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;
    double total_ms = 0.0;
    int64_t launches = 0;
  };
  bool timing = false;
  void* flush_buf = nullptr;   // benchmark: written before each timed kernel
  int64_t flush_bytes = 0;
  uint32_t flush_count = 0;
  std::vector<TimerSlot> slots;
  std::vector<hipEvent_t> pool;
};

namespace {

int64_t a256(int64_t n) { return align_up(n, 256); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

int plan_cus(moe_plan_s* p) {
  if (p->cus > 0) return p->cus;
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  p->cus = n;
  return n;
}

RouteHdr* hdr_of(void* ws) { return reinterpret_cast<RouteHdr*>(ws); }

hipEvent_t take_event(moe_plan_s* p) {
  if (!p->pool.empty()) {
    hipEvent_t e = p->pool.back();
    p->pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

moe_plan_s::TimerSlot& timer_slot(moe_plan_s* p, const char* name) {
  for (auto& sl : p->slots)
    if (sl.name == name) return sl;
  p->slots.emplace_back();
  p->slots.back().name = name;
  return p->slots.back();
}

// Runs one launcher; when timing is on, brackets it with events on stream s.
// With a flush buffer set (moe_timing_flush), each timed launch is preceded,
// outside its events, by a write of that buffer.
template <class Fn>
hipError_t timed(moe_plan_s* p, const char* name, hipStream_t s, Fn&& fn) {
  if (!p->timing) return fn();
  hipEvent_t a = take_event(p), b = take_event(p);
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t e = hipSuccess;
  if (p->flush_buf) {
    e = launch_flush(p->flush_buf, p->flush_bytes, ++p->flush_count, s);
    if (e != hipSuccess) return e;
  }
  e = hipEventRecord(a, s);
  if (e != hipSuccess) return e;
  e = fn();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, s);
  timer_slot(p, name).pending.emplace_back(a, b);
  return e;
}

template <typename T>
T* at(void* base, int64_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off);
}

// BF16 forward split (plans with hot set): cold experts stay on the
// streaming tiles, experts with many rows take the 256 x 256 MFMA tiles.
// In automatic mode the large tiles are used only when the call could give
// them at least three items per four compute units (R_max / 256 m-tiles times the GEMM's
// 256-wide n-tiles): a lone expert of 2,048 rows, such as a shared expert,
// gives the W13 GEMM 128 items and runs faster on the streaming tiles.
static void use_hot(moe_plan_s* p, void* ws, FwdArgs& a, int mode /* 0: W13, 1: W2 */) {
  if (!p->hot) return;
  const int64_t nt = mode == 0 ? p->d.f / 128 : p->d.d / 256;
  if (p->d.hot_tiles == 0 && 4 * (p->R_max / kBMH) * nt < 3 * int64_t(plan_cus(p))) return;
  a.cstoff = at<int32_t>(ws, p->rl.cstoff);
  a.ctoff = at<int32_t>(ws, p->rl.ctoff);
  a.hotoff = at<int32_t>(ws, p->rl.hotoff);
}


// BF16 weight gradients: experts with at least kHotWgRows rows take the
// 256 x 256 tiles of k_wgrad_hot unless the plan keeps every expert on the
// streaming tiles (hot_tiles = never) or no call can have such an expert
// (launch_wgrad also requires bf16 dW, no accumulation and widths that are
// multiples of 256).
static void hot_wgrad(const moe_plan_s* p, void* ws, BwdArgs& a) {
  if (p->d.prec != MOE_PREC_BF16 || p->d.hot_tiles == 2 || p->R_max < kHotWgRows) return;
  a.cst = at<int32_t>(ws, p->rl.cwoff);
  a.hot_wg = 1;
}

// MXFP8 weight gradients: the same for k_mx_wgrad_hot (launch_mx_wgrad
// also requires bf16 dW, no accumulation and widths that are multiples of
// 256), where the column bundles' exponent offsets and a tile's code offsets
// fit in 32 bits.
static void hot_wgrad_mx(const moe_plan_s* p, void* ws, MxArgs& a) {
  if (p->d.prec != MOE_PREC_MXFP8 || p->d.hot_tiles == 2 || p->R_max < kHotWgRows) return;
  const int64_t width = std::max<int64_t>(p->d.d, 2 * int64_t(p->d.f));
  if (width * (p->Rp_max / 32 + 1) >= (int64_t(1) << 31) || 256 * p->Rp_max >= (int64_t(1) << 31))
    return;
  a.cst = at<int32_t>(ws, p->rl.cwoff);
  a.hot_wg = 1;
}

// Split-K arguments of a BF16/FP32 forward GEMM launch (mode 0: W13, 1: W2).
static void set_split(const moe_plan_s* p, FwdArgs& a, int mode, char* sc) {
  a.ksplit = mode == 0 ? p->ks13 : p->ks2;
  a.part = a.ksplit > 1 ? reinterpret_cast<float*>(sc + p->sl.part) : nullptr;
  a.part_rows = p->R_max;
}

// MXFP8 forward up to h2 (after the gather): x rows -> 1x32 blocks (and the x
// column bundle in training), the W13 grouped GEMM with the SwiGLU epilogue,
// and the h2 column bundle in training.  replay_only = 1 runs the same
// launches as backward's replay predicate.
// Clamped SwiGLU limit for the kernels (+inf: the plain SwiGLU).
static float swiglu_limit(const moe_plan_s* p) {
  return p->d.swiglu_limit > 0.0f ? p->d.swiglu_limit : INFINITY;
}

// Planner arguments of a layer call: the scratch regions a replaying layer's
// state lives in (and the arena it is saved in otherwise).
PlanArgs plan_args(const moe_plan_s* p, int32_t layer, int training, void* arena, char* sc) {
  const moe_desc& d = p->d;
  const ScratchLayout& L = p->sl;
  const bool mx8 = d.prec == MOE_PREC_MXFP8;
  return PlanArgs{layer, d.max_layers, training, p->es, d.d, d.f, p->budget,
                  uint64_t(training ? arena : nullptr), uint64_t(sc + L.h1),
                  mx8 ? 1 : 0, 0,
                  {mx8 ? uint64_t(sc + L.xcq) : 0, mx8 ? uint64_t(sc + L.xcs) : 0,
                   mx8 ? uint64_t(sc + L.h2cq) : 0, mx8 ? uint64_t(sc + L.h2cs) : 0}};
}

// W2 records of expert j - kMegaLook follow the W13 records of expert j in
// the fused forward's queues (measured at T=2048, D=7168, F=2048, E=384,
// K=6: a lookahead of 1 expert leaves W2 records waiting, 6.06 ms; 2 and 4
// give 5.88 and 5.86 ms).
constexpr int kMegaLook = 4;
// Counters of the fused W2 backward: one per expert and 256-column block of F.
inline int msync_blocks(int F) { return (F + 255) / 256; }

// Arguments of the block-scaled W2 FPROP: h2 row blocks x W2 -> route slots
// h3 (or, with y32, the FUSED combine).
MxArgs mx_w2_args(moe_plan_s* p, RouteHdr* hdr, void* ws, char* sc, const moe_weights* w,
                  void* h3, const float* scores, float* y32) {
  const moe_desc& d = p->d;
  const ScratchLayout& L = p->sl;
  const int fp4 = d.prec == MOE_PREC_MXFP4;
  MxArgs a2{hdr, at<int32_t>(ws, p->rl.offsets), at<int32_t>(ws, p->rl.poffsets),
            at<int32_t>(ws, p->rl.mtoff), at<int32_t>(ws, p->rl.sorted_route),
            reinterpret_cast<const uint8_t*>(sc + L.qh2), reinterpret_cast<const uint8_t*>(sc + L.sh2),
            reinterpret_cast<const uint8_t*>(w->q2), reinterpret_cast<const uint8_t*>(w->s2),
            nullptr, nullptr, h3, nullptr, d.f, d.d, d.f, d.d / 128, d.e, 0, 0, -1, 0,
            int(p->R_max), scores, y32, d.k};
  a2.w1x32 = d.mx_w1x32 || fp4;
  a2.fp4 = fp4;
  a2.sw_rows = d.e * d.d;
  return a2;
}

// With mega (the W2 arguments) the W13 GEMM runs as the fused (Mega) launch
// together with the W2 records, msync its tickets and counters.
hipError_t mx_forward_w13(moe_plan_s* p, RouteHdr* hdr, void* ws, char* sc, const void* x,
                          const moe_weights* w, int replay_only, int cus, hipStream_t s,
                          const MxArgs* mega = nullptr, uint32_t* msync = nullptr) {
  const moe_desc& d = p->d;
  const ScratchLayout& L = p->sl;
  const int32_t* offsets = at<int32_t>(ws, p->rl.offsets);
  const int32_t* poffsets = at<int32_t>(ws, p->rl.poffsets);
  const int32_t* mtoff = at<int32_t>(ws, p->rl.mtoff);
  const int32_t* sorted_route = at<int32_t>(ws, p->rl.sorted_route);
  const char* tag = replay_only ? "replay_quant_x" : "quant_x";
  // x rows are read through the permutation (the gather happens in the loaders)
  const int fp4 = d.prec == MOE_PREC_MXFP4;
  RowqArgs rx{hdr, x, reinterpret_cast<uint8_t*>(sc + L.qx),
              reinterpret_cast<uint8_t*>(sc + L.sx), d.d, -1, -1, -1, replay_only,
              int(p->R_max), sorted_route, d.k};
  rx.fp4 = fp4;
  hipError_t e = timed(p, tag, s, [&] { return launch_rowq(rx, p->R_max, s); });
  if (e != hipSuccess) return e;
  if (d.training) {
    // A replaying layer's bundles are rebuilt in backward: the forward only
    // writes them for a layer that saves.
    ColqArgs cx{hdr, offsets, poffsets, x, nullptr, nullptr, d.d, d.e,
                -1, 0, 1, replay_only ? 1 : 2, sorted_route, d.k};
    e = timed(p, replay_only ? "replay_bundle_x" : "bundle_x", s,
              [&] { return launch_colq(cx, p->Rp_max, s); });
    if (e != hipSuccess) return e;
  }
  MxArgs a13{hdr, offsets, poffsets, mtoff, sorted_route,
             reinterpret_cast<const uint8_t*>(sc + L.qx), reinterpret_cast<const uint8_t*>(sc + L.sx),
             reinterpret_cast<const uint8_t*>(w->q13), reinterpret_cast<const uint8_t*>(w->s13),
             nullptr, nullptr, nullptr, d.training ? sc + L.h2 : nullptr, d.d, 2 * d.f, d.f,
             d.f / 64, d.e, 0, 0, -1, replay_only, int(p->R_max)};
  a13.limit = swiglu_limit(p);
  a13.w1x32 = d.mx_w1x32 || fp4;
  a13.fp4 = fp4;
  a13.sw_rows = d.e * 2 * d.f;
  if (!replay_only) {
    // h2 rows -> 1x32 blocks for the W2 GEMM, in the epilogue (bf16 h2 is
    // kept only in training, for its column bundle)
    a13.q_out = reinterpret_cast<uint8_t*>(sc + L.qh2);
    a13.s_out = reinterpret_cast<uint8_t*>(sc + L.sh2);
    a13.q_rows = int(p->R_max);
  }
  if (mega)
    e = timed(p, "mega_fwd", s, [&] {
      return launch_mx_mega(a13, *mega, msync, kMegaLook, p->mt_max, cus, s);
    });
  else
    e = timed(p, replay_only ? "replay_w13" : "w13_swiglu", s,
              [&] { return launch_mx_fwd(0, a13, p->mt_max, cus, s); });
  if (e != hipSuccess) return e;
  if (d.training) {
    ColqArgs ch{hdr, offsets, poffsets, sc + L.h2, nullptr, nullptr, d.f, d.e, -1, 2, 3,
                replay_only ? 1 : 2};
    e = timed(p, replay_only ? "replay_bundle_h2" : "bundle_h2", s,
              [&] { return launch_colq(ch, p->Rp_max, s); });
  }
  return e;
}


// MXFP8 backward after the replay gather: replay of the quantized forward
// state when needed, combine backward, both DGRADs on 1x32-quantized
// gradients with the shared 32x32 weights, both WGRADs on column bundles.
moe_status mx_backward(moe_plan_s* p, RouteHdr* hdr, void* ws, char* sc, const void* x,
                       const moe_weights* w, const float* scores, const void* dy, const void* h3,
                       void* arena, const moe_grads* g, uint32_t flags, int cus, hipStream_t s) {
  const bool mega = (flags & MOE_BWD_MEGA) != 0;
  // msync: [W2 tickets | counters | W13 tickets] (the fused launches')
  uint32_t* msync = at<uint32_t>(ws, p->rl.msync);
  uint32_t* t13 = msync + kXcds + int64_t(p->d.e) * msync_blocks(p->d.f);
  const moe_desc& d = p->d;
  const ScratchLayout& L = p->sl;
  const int32_t* offsets = at<int32_t>(ws, p->rl.offsets);
  const int32_t* poffsets = at<int32_t>(ws, p->rl.poffsets);
  const int32_t* mtoff = at<int32_t>(ws, p->rl.mtoff);
  const int32_t* sorted_route = at<int32_t>(ws, p->rl.sorted_route);
  const int32_t* route_to_row = at<int32_t>(ws, p->rl.route_to_row);
  const int dw_f32 = d.dw_dtype == MOE_DTYPE_F32;
  auto u8 = [&](int64_t off) { return reinterpret_cast<uint8_t*>(sc + off); };
  hipError_t e = mx_forward_w13(p, hdr, ws, sc, x, w, 1, cus, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = timed(p, "combine_bwd", s, [&] {
    return launch_combine_bwd(d.prec, hdr, route_to_row, scores, dy, h3, sc + L.dh3, g->dscores,
                              d.k, d.d, d.t_max, s);
  });
  if (e != hipSuccess) return MOE_ERR_HIP;
  RowqArgs r3{hdr, sc + L.dh3, u8(L.qdh3), u8(L.sdh3), d.d, -1, -1, -1, 0, int(p->R_max)};
  e = timed(p, "quant_dh3", s, [&] { return launch_rowq(r3, p->R_max, s); });
  if (e != hipSuccess) return MOE_ERR_HIP;
  ColqArgs c3{hdr, offsets, poffsets, sc + L.dh3, u8(L.dh3cq), u8(L.dh3cs), d.d, d.e, -1, -1, -1, 0};
  e = timed(p, "bundle_dh3", s, [&] { return launch_colq(c3, p->Rp_max, s); });
  if (e != hipSuccess) return MOE_ERR_HIP;
  MxArgs dg2{hdr, offsets, poffsets, mtoff, sorted_route, u8(L.qdh3), u8(L.sdh3),
             reinterpret_cast<const uint8_t*>(w->q2), reinterpret_cast<const uint8_t*>(w->s2),
             nullptr, nullptr, sc + L.dh1, nullptr, d.d, d.f, d.f, (d.f + 255) / 256, d.e, 0, 0,
             -1, 0, int(p->R_max)};
  dg2.limit = swiglu_limit(p);
  dg2.stoff = mtoff;
  MxArgs wg2{hdr, offsets, poffsets, mtoff, sorted_route, nullptr, nullptr, nullptr, nullptr,
             u8(L.dh3cq), u8(L.dh3cs), g->dw2, nullptr, 0, 0, d.f, 0, d.e, d.f, d.d, 2, 0};
  wg2.acc_dw = (flags & MOE_BWD_ACCUMULATE_DW) ? 1 : 0;
  if (mega) {
    e = timed(p, "w2_bwd_mega", s, [&] {
      return launch_mx_bwd_mega(0, dw_f32, dg2, wg2, msync, cus, s);
    });
    if (e != hipSuccess) return MOE_ERR_HIP;
  } else {
    hot_wgrad_mx(p, ws, wg2);
    e = timed(p, "w2_dgrad_swiglu", s, [&] { return launch_mx_dgrad(0, dg2, p->mt_max, cus, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
    e = timed(p, "w2_wgrad", s, [&] { return launch_mx_wgrad(dw_f32, 2, wg2, cus, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  RowqArgs r1{hdr, sc + L.dh1, u8(L.qdh1), u8(L.sdh1), 2 * d.f, -1, -1, -1, 0, int(p->R_max)};
  e = timed(p, "quant_dh1", s, [&] { return launch_rowq(r1, p->R_max, s); });
  if (e != hipSuccess) return MOE_ERR_HIP;
  ColqArgs c1{hdr, offsets, poffsets, sc + L.dh1, u8(L.dh1cq), u8(L.dh1cs), 2 * d.f, d.e,
              -1, -1, -1, 0};
  e = timed(p, "bundle_dh1", s, [&] { return launch_colq(c1, p->Rp_max, s); });
  if (e != hipSuccess) return MOE_ERR_HIP;
  MxArgs dg13{hdr, offsets, poffsets, mtoff, sorted_route, u8(L.qdh1), u8(L.sdh1),
              reinterpret_cast<const uint8_t*>(w->q13), reinterpret_cast<const uint8_t*>(w->s13),
              nullptr, nullptr, sc + L.dxr, nullptr, 2 * d.f, d.d, d.f, (d.d + 255) / 256, d.e, 0, 0,
              -1, 0, int(p->R_max)};
  dg13.stoff = mtoff;
  MxArgs wg13{hdr, offsets, poffsets, mtoff, sorted_route, nullptr, nullptr, nullptr, nullptr,
              u8(L.dh1cq), u8(L.dh1cs), g->dw13, nullptr, 0, 0, d.f, 0, d.e, d.d, 2 * d.f, 0, 0};
  wg13.acc_dw = (flags & MOE_BWD_ACCUMULATE_DW) ? 1 : 0;
  if (mega) {
    e = timed(p, "w13_bwd_mega", s, [&] {
      return launch_mx_bwd_mega(1, dw_f32, dg13, wg13, t13, cus, s);
    });
    if (e != hipSuccess) return MOE_ERR_HIP;
  } else {
    hot_wgrad_mx(p, ws, wg13);
    e = timed(p, "w13_dgrad", s, [&] { return launch_mx_dgrad(1, dg13, p->mt_max, cus, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
    e = timed(p, "w13_wgrad", s, [&] { return launch_mx_wgrad(dw_f32, 13, wg13, cus, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  e = timed(p, "dx_reduce", s, [&] {
    return launch_dx_reduce(d.prec, hdr, route_to_row, reinterpret_cast<float*>(sc + L.dxr), g->dx,
                            d.k, d.d, d.t_max, (flags & MOE_BWD_ACCUMULATE_DX) ? 1 : 0, s);
  });
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(timed(p, "rewind", s, [&] { return launch_plan_rewind(hdr, arena, s); }));
}

}  // namespace

extern "C" {

moe_status moe_plan_create(const moe_desc* desc, moe_plan_t* out) {
  if (!desc || !out) return MOE_ERR_ARG;
  *out = nullptr;
  const moe_desc& d = *desc;
  // K may exceed E: duplicate ids inside a token are independent routes.
  // D and F are bounded so that every per-row index the kernels form in 32
  // bits (row lengths, stage counts, E * 2F weight rows) stays in range.
  if (d.t_max < 0 || d.k < 1 || d.k > kMaxK || d.e < 1 || d.e > kMaxE || d.d <= 0 ||
      d.f <= 0 || d.d > kMaxWidth || d.f > kMaxWidth || d.d % 128 || d.f % 128 ||
      d.t_max * d.k > (int64_t(1) << 24))
    return MOE_ERR_SHAPE;
  if (d.prec != MOE_PREC_F32 && d.prec != MOE_PREC_BF16 && d.prec != MOE_PREC_MXFP8 &&
      d.prec != MOE_PREC_MXFP4)
    return MOE_ERR_ARG;
  if (d.prec == MOE_PREC_MXFP4 && (d.d % 256 || d.f % 256)) return MOE_ERR_SHAPE;
  if (d.prec == MOE_PREC_MXFP4 && d.training) return MOE_ERR_ARG;
  if (d.dw_dtype != MOE_DTYPE_F32 && d.dw_dtype != MOE_DTYPE_BF16) return MOE_ERR_ARG;
  if (d.prec == MOE_PREC_F32 && d.dw_dtype != MOE_DTYPE_F32) return MOE_ERR_ARG;
  if (d.max_layers < 1 || d.arena_budget < 0) return MOE_ERR_ARG;
  if (!(d.swiglu_limit >= 0.0f) || !(d.swiglu_limit < INFINITY)) return MOE_ERR_ARG;
  if (d.mx_w1x32 != 0 && (d.mx_w1x32 != 1 || d.prec != MOE_PREC_MXFP8 || d.training))
    return MOE_ERR_ARG;
  if (d.hot_tiles < 0 || d.hot_tiles > 2) return MOE_ERR_ARG;

  moe_plan_s* p = new (std::nothrow) moe_plan_s();
  if (!p) return MOE_ERR_ARG;
  p->d = d;
  p->es = d.prec == MOE_PREC_F32 ? 4 : 2;
  p->R_max = d.t_max * d.k;
  p->mt_max = std::min<int64_t>(p->R_max, (p->R_max + kBM - 1) / kBM + d.e);
  p->Rp_max = align_up(p->R_max + 31 * std::min<int64_t>(d.e, p->R_max), 32);
  {
    // the hot-expert kernel addresses an expert's weights and the token rows
    // with 32-bit byte offsets and stores 256-column W2 tiles
    const int64_t lim = int64_t(1) << 32;
    p->hot = d.prec == MOE_PREC_BF16 && d.hot_tiles != 2 && d.d % 256 == 0 &&
             int64_t(4) * d.f * d.d < lim && int64_t(2) * d.t_max * d.d < lim &&
             p->R_max * d.f * 2 < lim;
  }
  const int64_t E = d.e, D = d.d, F = d.f, R = p->R_max, es = p->es, Rp = p->Rp_max;
  const bool mx = d.prec == MOE_PREC_MXFP8;
  const bool fp4 = d.prec == MOE_PREC_MXFP4;   // inference only: no column bundles
  {
    // Split-K of the BF16/FP32 forward GEMMs ("Mixture of Experts: How
    // Routing Becomes GPU Computation", section 6): considered when even the
    // plan's upper bound on work items (m-tiles x n-tiles) gives the 256 CUs
    // of gfx950 fewer than two items each, which is decode (a handful of
    // rows, one per expert).  The streaming kernel keeps two workgroups per
    // CU, so 512 items run at once: the factor (1..8, at least 4 stages of
    // 128 bytes per part) is the one whose item count fills its last round
    // of 512 best, the smaller on ties within 2% (at one token and the
    // 7168 x 2048 layer: W13 192 items x 8 = 3 full rounds, W2 336 x 3 =
    // 1,008 of 1,024).  A plan that may put experts on the hot-expert tiles
    // does not split.
    const bool may_hot = p->hot && (d.hot_tiles == 1 || 4 * (R / kBMH) * (F / 128) >= 3 * 256 ||
                                    4 * (R / kBMH) * (D / 256) >= 3 * 256);
    auto factor = [&](int64_t items, int64_t stages) {
      constexpr int64_t kSlots = 2 * 256;
      if (mx || fp4 || may_hot || items >= kSlots || items == 0) return 1;
      int best = 1;
      double best_fill = 0.0;
      for (int ks = 1; ks <= 8 && stages / ks >= 4; ++ks) {
        const int64_t n = items * ks;
        const double fill = double(n) / double((n + kSlots - 1) / kSlots * kSlots);
        if (fill > best_fill + 0.02) {
          best = ks;
          best_fill = fill;
        }
      }
      return best;
    };
    p->ks13 = factor(p->mt_max * (F / 64), D * es / 128);
    p->ks2 = factor(p->mt_max * (D / 128), F * es / 128);
  }

  RouteLayout& L = p->rl;
  L.nchunks = (R + kRankChunk - 1) / kRankChunk;
  int64_t o = 0;
  L.hdr = o; o = a256(o + 512);
  L.counts = o; o = a256(o + 4 * E);
  L.offsets = o; o = a256(o + 4 * (E + 1));
  L.poffsets = o; o = a256(o + 4 * (E + 1));
  L.mtoff = o; o = a256(o + 4 * (E + 1));
  L.gtoff = o; o = a256(o + 4 * (E + 1));
  // cstoff, ctoff, hotoff, cwoff: one region, written by routing as split[4][E + 1]
  L.cstoff = o;
  L.ctoff = o + 4 * (E + 1);
  L.hotoff = o + 8 * (E + 1);
  L.cwoff = o + 12 * (E + 1);
  o = a256(o + 16 * (E + 1));
  L.chunk_hist = o; o = a256(o + 4 * L.nchunks * E);
  L.chunk_flags = o; o = a256(o + 4 * L.nchunks);
  L.sorted_route = o; o = a256(o + 4 * R);
  L.route_to_row = o; o = a256(o + 4 * R);
  L.msync = o; o = a256(o + 4 * (2 * kXcds + int64_t(E) * msync_blocks(d.f)));
  L.total = o;

  ScratchLayout& S = p->sl;
  {
    int64_t* all = &S.x_rows;
    for (int i = 0; i < int(sizeof(ScratchLayout) / sizeof(int64_t)); ++i) all[i] = -1;
  }
  o = 0;
  auto take = [&](int64_t& field, int64_t bytes) {
    field = o;
    o = a256(o + bytes);
  };
  take(S.h1, R * 2 * F * es);
  take(S.h2, R * F * es);
  if (p->ks13 > 1 || p->ks2 > 1)
    take(S.part, std::max<int64_t>(p->ks13 * R * 2 * F, p->ks2 * R * D) * 4);
  if (mx) {
    take(S.qx, R * D);
    take(S.sx, R * D / 32);
    take(S.qh2, R * F);
    take(S.sh2, R * F / 32);
    take(S.xcq, Rp * D);
    take(S.xcs, Rp / 32 * D);
    take(S.h2cq, Rp * F);
    take(S.h2cs, Rp / 32 * F);
  }
  if (fp4) {
    take(S.qx, R * D / 2);
    take(S.sx, R * D / 32);
    take(S.qh2, R * F / 2);
    take(S.sh2, R * F / 32);
  }
  if (d.training) {
    if (!mx) take(S.x_rows, R * D * es);   // packed x rows for the W13 weight gradient
    take(S.dh3, R * D * es);
    take(S.dh1, R * 2 * F * es);
    take(S.dxr, R * D * 4);
    if (mx) {
      take(S.qdh3, R * D);
      take(S.sdh3, R * D / 32);
      take(S.dh3cq, Rp * D);
      take(S.dh3cs, Rp / 32 * D);
      take(S.qdh1, R * 2 * F);
      take(S.sdh1, R * 2 * F / 32);
      take(S.dh1cq, Rp * 2 * F);
      take(S.dh1cs, Rp / 32 * 2 * F);
    }
  }
  S.total = std::max<int64_t>(o, 256);

  p->h3_bytes = std::max<int64_t>(a256(R * D * es), 256);
  p->state_max = mx ? align128(Rp * D) + align128(Rp / 32 * D) + align128(R * 2 * F * 2) +
                          align128(Rp * F) + align128(Rp / 32 * F)
                    : align128(R * 2 * F * es);
  p->budget = d.arena_budget > 0 ? d.arena_budget : int64_t(d.max_layers) * p->state_max;
  p->arena_bytes = d.training ? kArenaHdrBytes + a256(p->budget) : kArenaHdrBytes;
  p->cus = 0;
  *out = p;
  return MOE_OK;
}

moe_status moe_plan_sizes(moe_plan_t p, moe_sizes* s) {
  if (!p || !s) return MOE_ERR_ARG;
  std::memset(s, 0, sizeof(*s));
  s->route_ws = size_t(p->rl.total);
  s->scratch = size_t(p->sl.total);
  s->h3_slots = size_t(p->h3_bytes);
  s->arena = size_t(p->arena_bytes);
  s->layer_state_max = size_t(p->state_max);
  if (p->d.prec == MOE_PREC_MXFP8 || p->d.prec == MOE_PREC_MXFP4) {
    const int64_t E = p->d.e, D = p->d.d, F = p->d.f;
    const int64_t per_byte = p->d.prec == MOE_PREC_MXFP4 ? 2 : 1;
    const int64_t per_exp = p->d.prec == MOE_PREC_MXFP4 || p->d.mx_w1x32 ? 32 : 1024;
    // 32x32 blocks: one exponent per 1024 values; 1x32: one per 32
    s->q13 = size_t(a256(E * 2 * F * D / per_byte));
    s->s13 = size_t(a256(E * 2 * F * D / per_exp));
    s->q2 = size_t(a256(E * D * F / per_byte));
    s->s2 = size_t(a256(E * D * F / per_exp));
  }
  return MOE_OK;
}

moe_status moe_plan_explain(moe_plan_t p, char* buf, size_t cap) {
  if (!p || !buf || cap == 0) return MOE_ERR_ARG;
  const moe_desc& d = p->d;
  const char* prec = d.prec == MOE_PREC_F32    ? "f32"
                     : d.prec == MOE_PREC_BF16 ? "bf16"
                     : d.prec == MOE_PREC_MXFP8 ? "mxfp8"
                                                : "mxfp4";
  const bool mx = d.prec == MOE_PREC_MXFP8;
  auto mib = [](int64_t b) { return double(b) / (1024.0 * 1024.0); };
  std::string s;
  char line[256];
  std::snprintf(line, sizeof line,
                "moe plan: T_max=%lld D=%d F=%d E=%d K=%d prec=%s dW=%s training=%d layers=%d\n",
                (long long)d.t_max, d.d, d.f, d.e, d.k, prec,
                d.dw_dtype == MOE_DTYPE_F32 ? "f32" : "bf16", d.training, d.max_layers);
  s += line;
  if (d.swiglu_limit > 0.0f) {
    std::snprintf(line, sizeof line, "  SwiGLU clamped at L=%g (gate <= L, |up| <= L)\n",
                  double(d.swiglu_limit));
    s += line;
  }
  std::snprintf(line, sizeof line, "  routed rows R <= %lld, m-tiles <= %lld (%d rows each)\n",
                (long long)p->R_max, (long long)p->mt_max, kBM);
  s += line;
  if (p->ks13 > 1 || p->ks2 > 1) {
    std::snprintf(line, sizeof line,
                  "  forward split-K: W13 x%d, W2 x%d (fp32 partial tiles, ordered second pass)\n",
                  p->ks13, p->ks2);
    s += line;
  }
  if (d.prec == MOE_PREC_BF16) {
    static const char* kHot[] = {"automatic", "always", "never"};
    std::snprintf(line, sizeof line,
                  "  experts with >= %d rows: 256 x 256 MFMA forward tiles %s%s\n", kHotRows,
                  kHot[d.hot_tiles], p->hot ? "" : " (not with this shape)");
    s += line;
  }
  if ((d.prec == MOE_PREC_BF16 || d.prec == MOE_PREC_MXFP8) && d.training && d.hot_tiles != 2 &&
      p->R_max >= kHotWgRows) {
    std::snprintf(line, sizeof line,
                  "  experts with >= %d rows: 256 x 256 MFMA weight-gradient tiles "
                  "(bf16 dW, widths multiples of 256)\n",
                  kHotWgRows);
    s += line;
  }
  std::snprintf(line, sizeof line, "  route_ws   %10.2f MiB per layer (metadata + planner record)\n",
                mib(p->rl.total));
  s += line;
  std::snprintf(line, sizeof line, "  h3_slots   %10.2f MiB per layer [T*K, D]\n", mib(p->h3_bytes));
  s += line;
  std::snprintf(line, sizeof line,
                "  scratch    %10.2f MiB shared: h1 %.2f, h2 %.2f",
                mib(p->sl.total), mib(p->sl.h2 - p->sl.h1),
                mib((d.training ? p->sl.dh3 : p->sl.total) - p->sl.h2));
  s += line;
  if (d.training) {
    std::snprintf(line, sizeof line, ", dh3 %.2f, dh1 %.2f, dxr %.2f",
                  mib(p->sl.dh1 - p->sl.dh3), mib(p->sl.dxr - p->sl.dh1),
                  mib(p->sl.total - p->sl.dxr));
    s += line;
  }
  s += "\n";
  std::snprintf(line, sizeof line,
                "  arena      %10.2f MiB: budget %.2f MiB, full layer state %.2f MiB at R_max "
                "(%s, 128-B aligned)\n",
                mib(p->arena_bytes), mib(p->budget), mib(p->state_max),
                mx ? "x and h2 column bundles + h1" : "h1");
  s += line;
  std::snprintf(line, sizeof line,
                "  planner: a layer replays iff cursor + full_state > budget (device decision "
                "on the realized R)\n");
  s += line;
  std::strncpy(buf, s.c_str(), cap - 1);
  buf[cap - 1] = '\0';
  return MOE_OK;
}

void moe_plan_destroy(moe_plan_t p) {
  if (!p) return;
  for (auto& sl : p->slots)
    for (auto& ev : sl.pending) {
      hipEventSynchronize(ev.second);
      hipEventDestroy(ev.first);
      hipEventDestroy(ev.second);
    }
  for (hipEvent_t e : p->pool) hipEventDestroy(e);
  delete p;
}

moe_status moe_prepare_weights(moe_plan_t p, const void* w13, const void* w2, void* q13,
                               void* s13, void* q2, void* s2, hipStream_t s) {
  if (!p) return MOE_ERR_ARG;
  if (p->d.prec != MOE_PREC_MXFP8 && p->d.prec != MOE_PREC_MXFP4) return MOE_ERR_UNSUPPORTED;
  if (!w13 || !w2 || !q13 || !s13 || !q2 || !s2) return MOE_ERR_ARG;
  const moe_desc& d = p->d;
  const int fp4 = d.prec == MOE_PREC_MXFP4;
  if (d.mx_w1x32 || fp4) {
    // 1x32 blocks: the row quantizer over the weight rows [E*N, Kd], its
    // exponents grouped by stage ([Kd/128][E*N] dwords; MXFP4 [Kd/256][E*N]
    // pairs of dwords)
    auto prep = [&](const void* w, void* q, void* sc, int64_t rows, int kd) {
      RowqArgs r{nullptr, w, reinterpret_cast<uint8_t*>(q), reinterpret_cast<uint8_t*>(sc), kd,
                 -1, -1, -1, 0, int(rows), nullptr, 0, rows, fp4};
      return launch_rowq(r, rows, s);
    };
    hipError_t e = timed(p, "prep_w13", s,
                         [&] { return prep(w13, q13, s13, int64_t(d.e) * 2 * d.f, d.d); });
    if (e != hipSuccess) return MOE_ERR_HIP;
    return hip_status(
        timed(p, "prep_w2", s, [&] { return prep(w2, q2, s2, int64_t(d.e) * d.d, d.f); }));
  }
  hipError_t e = timed(p, "prep_w13", s, [&] {
    return launch_prep_w(w13, q13, s13, d.e, 2 * d.f, d.d, s);
  });
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(timed(p, "prep_w2", s, [&] {
    return launch_prep_w(w2, q2, s2, d.e, d.d, d.f, s);
  }));
}

moe_status moe_mx_quantize(moe_plan_t p, void* ws, const void* src, int32_t n, int32_t kind,
                           void* q, void* sc, hipStream_t s) {
  if (!p || !ws || !src || !q || !sc) return MOE_ERR_ARG;
  if (n <= 0 || n % 128) return MOE_ERR_SHAPE;
  RouteHdr* hdr = hdr_of(ws);
  if (kind == 0 || kind == 2) {
    RowqArgs r{hdr, src, reinterpret_cast<uint8_t*>(q), reinterpret_cast<uint8_t*>(sc), n,
               -1, -1, -1, 0};
    r.fp4 = kind == 2;
    return hip_status(launch_rowq(r, p->R_max, s));
  }
  if (kind == 1) {
    ColqArgs c{hdr, at<int32_t>(ws, p->rl.offsets), at<int32_t>(ws, p->rl.poffsets), src,
               reinterpret_cast<uint8_t*>(q), reinterpret_cast<uint8_t*>(sc), n, p->d.e,
               -1, -1, -1, 0};
    return hip_status(launch_colq(c, p->Rp_max, s));
  }
  return MOE_ERR_ARG;
}

moe_status moe_route(moe_plan_t p, int64_t T, const int32_t* ids, void* ws, hipStream_t s) {
  if (!p || !ws || T < 0 || T > p->d.t_max || (T > 0 && !ids)) return MOE_ERR_ARG;
  if (!aligned16(ws)) return MOE_ERR_ARG;
  return hip_status(timed(p, "route", s, [&] {
    return launch_route(ids, T, p->d.k, p->d.e, reinterpret_cast<char*>(ws), p->rl, s);
  }));
}

}  // extern "C"

namespace {

// Host-side checks shared by the staged and the fused (Mega) expert forward.
moe_status fwd_args_check(moe_plan_s* p, int32_t layer, void* ws, const void* x,
                          const moe_weights* w, void* h3, void* arena, void* scratch) {
  if (!p || !ws || !w || !h3 || !scratch) return MOE_ERR_ARG;
  const moe_desc& d = p->d;
  const bool mx = d.prec == MOE_PREC_MXFP8 || d.prec == MOE_PREC_MXFP4;
  if (mx ? (!w->q13 || !w->s13 || !w->q2 || !w->s2) : (!w->w13 || !w->w2)) return MOE_ERR_ARG;
  if (layer < 0 || layer >= d.max_layers) return MOE_ERR_ARG;
  if (!aligned16(x) || !aligned16(w->w13) || !aligned16(w->w2) || !aligned16(w->q13) ||
      !aligned16(w->q2) || !aligned16(h3) || !aligned16(scratch) || !aligned16(ws))
    return MOE_ERR_ARG;
  if (d.training && arena && !aligned16(arena)) return MOE_ERR_ARG;
  return MOE_OK;
}


}  // namespace

extern "C" {

moe_status moe_expert_fwd_mega(moe_plan_t p, int32_t layer, void* ws, const void* x,
                               const moe_weights* w, void* h3, void* arena, void* scratch,
                               hipStream_t s) {
  const moe_status st = fwd_args_check(p, layer, ws, x, w, h3, arena, scratch);
  if (st != MOE_OK) return st;
  const moe_desc& d = p->d;
  RouteHdr* hdr = hdr_of(ws);
  char* sc = reinterpret_cast<char*>(scratch);
  uint32_t* msync = at<uint32_t>(ws, p->rl.msync);
  PlanArgs pa = plan_args(p, layer, d.training, arena, sc);
  pa.zero = uint64_t(reinterpret_cast<uintptr_t>(msync));
  pa.zero_n = kXcds + d.e;
  hipError_t e = timed(p, "plan", s, [&] { return launch_plan_decide(hdr, pa, s); });
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (d.prec == MOE_PREC_MXFP8 || d.prec == MOE_PREC_MXFP4) {
    const MxArgs a2 = mx_w2_args(p, hdr, ws, sc, w, h3, nullptr, nullptr);
    return hip_status(mx_forward_w13(p, hdr, ws, sc, x, w, 0, plan_cus(p), s, &a2, msync));
  }
  const int32_t* offsets = at<int32_t>(ws, p->rl.offsets);
  const int32_t* mtoff = at<int32_t>(ws, p->rl.mtoff);
  const int32_t* gtoff = at<int32_t>(ws, p->rl.gtoff);
  const int32_t* sorted_route = at<int32_t>(ws, p->rl.sorted_route);
  FwdArgs a13{hdr, offsets, gtoff, sorted_route, nullptr, w->w13, nullptr, sc + p->sl.h2,
              d.d, 2 * d.f, d.f, d.f / 64, d.e, 0, x, d.k};
  a13.stoff = mtoff;
  a13.limit = swiglu_limit(p);
  FwdArgs a2{hdr, offsets, gtoff, sorted_route, sc + p->sl.h2, w->w2, h3, nullptr,
             d.f, d.d, d.f, d.d / 128, d.e, 0};
  a2.stoff = mtoff;
  return hip_status(timed(p, "mega_fwd", s, [&] {
    return launch_gemm_mega(d.prec, a13, a2, at<uint32_t>(ws, p->rl.msync), kMegaLook, p->mt_max,
                            plan_cus(p), s);
  }));
}

moe_status moe_expert_fwd(moe_plan_t p, int32_t layer, void* ws, const void* x,
                          const moe_weights* w, void* h3, void* arena, void* scratch,
                          hipStream_t s) {
  const moe_status st = fwd_args_check(p, layer, ws, x, w, h3, arena, scratch);
  if (st != MOE_OK) return st;
  const moe_desc& d = p->d;
  const bool mx8 = d.prec == MOE_PREC_MXFP8;
  const bool fp4 = d.prec == MOE_PREC_MXFP4;
  const bool mx = mx8 || fp4;
  RouteHdr* hdr = hdr_of(ws);
  char* sc = reinterpret_cast<char*>(scratch);
  const ScratchLayout& L = p->sl;
  const PlanArgs pa = plan_args(p, layer, d.training, arena, sc);
  hipError_t e = timed(p, "plan", s, [&] { return launch_plan_decide(hdr, pa, s); });
  if (e != hipSuccess) return MOE_ERR_HIP;
  const int32_t* offsets = at<int32_t>(ws, p->rl.offsets);
  const int32_t* poffsets = at<int32_t>(ws, p->rl.poffsets);
  const int32_t* mtoff = at<int32_t>(ws, p->rl.mtoff);
  const int32_t* gtoff = at<int32_t>(ws, p->rl.gtoff);  // FPROP/DGRAD m-tiles
  const int32_t* sorted_route = at<int32_t>(ws, p->rl.sorted_route);
  const int cus = plan_cus(p);
  if (!mx) {
    FwdArgs a13{hdr, offsets, gtoff, sorted_route, nullptr, w->w13, nullptr, sc + L.h2,
                d.d, 2 * d.f, d.f, d.f / 64, d.e, 0, x, d.k};
    a13.stoff = mtoff;
    set_split(p, a13, 0, sc);
    use_hot(p, ws, a13, 0);
    a13.limit = swiglu_limit(p);
    e = timed(p, "w13_swiglu", s,
              [&] { return launch_gemm_fwd(d.prec, 0, a13, p->mt_max, cus, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
    FwdArgs a2{hdr, offsets, gtoff, sorted_route, sc + L.h2, w->w2, h3, nullptr,
               d.f, d.d, d.f, d.d / 128, d.e, 0};
    a2.stoff = mtoff;
    set_split(p, a2, 1, sc);
    use_hot(p, ws, a2, 1);
    return hip_status(timed(p, "w2_scatter", s,
                            [&] { return launch_gemm_fwd(d.prec, 1, a2, p->mt_max, cus, s); }));
  }
  e = mx_forward_w13(p, hdr, ws, sc, x, w, 0, cus, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  const MxArgs a2 = mx_w2_args(p, hdr, ws, sc, w, h3, nullptr, nullptr);
  return hip_status(timed(p, "w2_scatter", s, [&] { return launch_mx_fwd(1, a2, p->mt_max, cus, s); }));
}

moe_status moe_combine(moe_plan_t p, void* ws, const float* scores, const void* h3,
                       const void* y_addend, void* y, hipStream_t s) {
  if (!p || !ws || !h3) return MOE_ERR_ARG;
  if (!aligned16(h3) || !aligned16(y) || !aligned16(y_addend))
    return MOE_ERR_ARG;
  RouteHdr* hdr = hdr_of(ws);
  return hip_status(timed(p, "combine", s, [&] {
    return launch_combine(p->d.prec, hdr, at<int32_t>(ws, p->rl.route_to_row), scores, h3,
                          y_addend, y, p->d.k, p->d.d, p->d.t_max, &hdr->status, s);
  }));
}

}  // extern "C"

namespace {

// Host-side checks of the fused inference forward (nothing enqueued).
moe_status fused_check(moe_plan_s* p, void* ws, const void* x, const moe_weights* w,
                       const void* y_addend, void* y) {
  if (!p || !ws || !w) return MOE_ERR_ARG;
  const moe_desc& d = p->d;
  if (d.training) return MOE_ERR_UNSUPPORTED;   // no route outputs are kept for a backward
  const bool mx = d.prec == MOE_PREC_MXFP8 || d.prec == MOE_PREC_MXFP4;
  if (mx ? (!w->q13 || !w->s13 || !w->q2 || !w->s2) : (!w->w13 || !w->w2)) return MOE_ERR_ARG;
  if (!aligned16(x) || !aligned16(w->w13) || !aligned16(w->w2) || !aligned16(w->q13) ||
      !aligned16(w->q2) || !aligned16(y) || !aligned16(y_addend) || !aligned16(ws))
    return MOE_ERR_ARG;
  return MOE_OK;
}

// The fused inference forward on a given scratch buffer and fp32 row buffer
// (arguments already checked).
moe_status fused_forward(moe_plan_s* p, void* ws, const void* x, const float* scores,
                         const moe_weights* w, float* y32, const void* y_addend, void* y,
                         void* scratch, hipStream_t s) {
  const moe_desc& d = p->d;
  const bool fp4 = d.prec == MOE_PREC_MXFP4;
  const bool mx = d.prec == MOE_PREC_MXFP8 || fp4;
  RouteHdr* hdr = hdr_of(ws);
  char* sc = reinterpret_cast<char*>(scratch);
  const ScratchLayout& L = p->sl;
  const PlanArgs pa = plan_args(p, 0, 0, nullptr, sc);
  hipError_t e = timed(p, "plan", s, [&] { return launch_plan_decide(hdr, pa, s); });
  if (e != hipSuccess) return MOE_ERR_HIP;
  const int32_t* offsets = at<int32_t>(ws, p->rl.offsets);
  const int32_t* poffsets = at<int32_t>(ws, p->rl.poffsets);
  const int32_t* mtoff = at<int32_t>(ws, p->rl.mtoff);
  const int32_t* gtoff = at<int32_t>(ws, p->rl.gtoff);  // FPROP/DGRAD m-tiles
  const int32_t* sorted_route = at<int32_t>(ws, p->rl.sorted_route);
  const int32_t* route_to_row = at<int32_t>(ws, p->rl.route_to_row);
  const int cus = plan_cus(p);
  if (!scores) {   // the W2 epilogue needs the scores: report, as the slot combine does
    e = launch_fused_finish(d.prec, hdr, route_to_row, nullptr, y32, y_addend, y, d.k, d.d,
                            d.t_max, &hdr->status, s);
    return hip_status(e);
  }
  e = timed(p, "zero_y32", s, [&] { return launch_zero_rows_f32(hdr, y32, d.d, d.t_max, s); });
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (!mx) {
    FwdArgs a13{hdr, offsets, gtoff, sorted_route, nullptr, w->w13, nullptr, sc + L.h2,
                d.d, 2 * d.f, d.f, d.f / 64, d.e, 0, x, d.k};
    a13.stoff = mtoff;
    set_split(p, a13, 0, sc);
    use_hot(p, ws, a13, 0);
    a13.limit = swiglu_limit(p);
    e = timed(p, "w13_swiglu", s,
              [&] { return launch_gemm_fwd(d.prec, 0, a13, p->mt_max, cus, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
    FwdArgs a2{hdr, offsets, gtoff, sorted_route, sc + L.h2, w->w2, nullptr, nullptr,
               d.f, d.d, d.f, d.d / 128, d.e, 0, nullptr, d.k, scores, y32};
    a2.stoff = mtoff;
    set_split(p, a2, 1, sc);
    use_hot(p, ws, a2, 1);
    e = timed(p, "w2_fused", s, [&] { return launch_gemm_fwd(d.prec, 1, a2, p->mt_max, cus, s); });
  } else {
    e = mx_forward_w13(p, hdr, ws, sc, x, w, 0, cus, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    const MxArgs a2 = mx_w2_args(p, hdr, ws, sc, w, nullptr, scores, y32);
    e = timed(p, "w2_fused", s, [&] { return launch_mx_fwd(1, a2, p->mt_max, cus, s); });
  }
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(timed(p, "fused_finish", s, [&] {
    return launch_fused_finish(d.prec, hdr, route_to_row, scores, y32, y_addend, y, d.k, d.d,
                               d.t_max, &hdr->status, s);
  }));
}

}  // namespace

extern "C" {

moe_status moe_expert_fwd_fused(moe_plan_t p, void* ws, const void* x, const float* scores,
                                const moe_weights* w, float* y32, const void* y_addend, void* y,
                                void* scratch, hipStream_t s) {
  if (!scratch || !y32 || !aligned16(scratch) || !aligned16(y32)) return MOE_ERR_ARG;
  const moe_status st = fused_check(p, ws, x, w, y_addend, y);
  if (st != MOE_OK) return st;
  return fused_forward(p, ws, x, scores, w, y32, y_addend, y, scratch, s);
}

moe_status moe_expert_bwd(moe_plan_t p, int32_t layer, void* ws, const void* x,
                          const float* scores, const void* dy, const moe_weights* w,
                          const void* h3, void* arena, void* scratch, const moe_grads* g,
                          uint32_t flags, hipStream_t s) {
  if (!p || !ws || !w || !g || !scratch || !h3) return MOE_ERR_ARG;
  if (flags & ~(MOE_BWD_ACCUMULATE_DX | MOE_BWD_ACCUMULATE_DW | MOE_BWD_MEGA)) return MOE_ERR_ARG;
  const moe_desc& d = p->d;
  if (!d.training || d.prec == MOE_PREC_F32) return MOE_ERR_UNSUPPORTED;
  const bool mega = (flags & MOE_BWD_MEGA) != 0;
  if (layer < 0 || layer >= d.max_layers) return MOE_ERR_ARG;
  const bool mx = d.prec == MOE_PREC_MXFP8;
  if (mx ? (!w->q13 || !w->s13 || !w->q2 || !w->s2) : (!w->w13 || !w->w2)) return MOE_ERR_ARG;
  if (!g->dw13 || !g->dw2) return MOE_ERR_ARG;
  if (!aligned16(ws) || !aligned16(x) || !aligned16(dy) || !aligned16(w->w13) ||
      !aligned16(w->w2) || !aligned16(h3) || !aligned16(scratch) || !aligned16(g->dx) ||
      !aligned16(g->dw13) || !aligned16(g->dw2) || !aligned16(arena))
    return MOE_ERR_ARG;
  RouteHdr* hdr = hdr_of(ws);
  char* sc = reinterpret_cast<char*>(scratch);
  const int32_t* offsets = at<int32_t>(ws, p->rl.offsets);
  const int32_t* mtoff = at<int32_t>(ws, p->rl.mtoff);
  const int32_t* gtoff = at<int32_t>(ws, p->rl.gtoff);  // FPROP/DGRAD m-tiles
  const int32_t* sorted_route = at<int32_t>(ws, p->rl.sorted_route);
  const int32_t* route_to_row = at<int32_t>(ws, p->rl.route_to_row);
  const int cus = plan_cus(p);
  void* dh3 = sc + p->sl.dh3;
  void* dh1 = sc + p->sl.dh1;
  float* dxr = reinterpret_cast<float*>(sc + p->sl.dxr);
  const int dw_f32 = d.dw_dtype == MOE_DTYPE_F32;
  hipError_t e;
  // A layer whose forward did not run since its routing is reported and
  // rebuilt from x like a replaying layer.
  uint32_t* msync = at<uint32_t>(ws, p->rl.msync);
  {
    PlanArgs pa = plan_args(p, layer, 1, arena, sc);
    if (mega) {   // the fused launches' tickets and counters
      pa.zero = uint64_t(reinterpret_cast<uintptr_t>(msync));
      pa.zero_n = 2 * kXcds + d.e * msync_blocks(d.f);
    }
    e = timed(p, "plan_bwd", s, [&] { return launch_plan_enter_bwd(hdr, pa, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  // Replay (device predicate): rebuild h1 in scratch from x when the forward
  // did not save it.
  if (mx) return mx_backward(p, hdr, ws, sc, x, w, scores, dy, h3, arena, g, flags, cus, s);
  FwdArgs a13{hdr, offsets, gtoff, sorted_route, nullptr, w->w13, nullptr, sc + p->sl.h2,
              d.d, 2 * d.f, d.f, d.f / 64, d.e, 1, x, d.k};
  a13.stoff = mtoff;
  set_split(p, a13, 0, sc);
  use_hot(p, ws, a13, 0);
  a13.limit = swiglu_limit(p);
  e = timed(p, "replay_w13", s, [&] { return launch_gemm_fwd(d.prec, 0, a13, p->mt_max, cus, s); });
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = timed(p, "combine_bwd", s, [&] {
    return launch_combine_bwd(d.prec, hdr, route_to_row, scores, dy, h3, dh3, g->dscores, d.k,
                              d.d, d.t_max, s);
  });
  if (e != hipSuccess) return MOE_ERR_HIP;
  void* h2 = sc + p->sl.h2;
  // BwdArgs: hdr, offsets, mtoff, W, tok, grad, arows, out, out2, Kd, N, F, D, E, NT, a_ld, b_ld
  BwdArgs b{hdr, offsets, gtoff, w->w2, dh3, nullptr, nullptr, dh1, h2,
            d.d, d.f, d.f, d.d, d.e, (d.f + 255) / 256, 0, 0, mtoff};
  b.limit = swiglu_limit(p);
  BwdArgs bw2{hdr, offsets, mtoff, nullptr, nullptr, dh3, h2, g->dw2, nullptr,
              0, 0, d.f, d.d, d.e, 0, d.f, d.d};
  bw2.acc_dw = (flags & MOE_BWD_ACCUMULATE_DW) ? 1 : 0;
  BwdArgs b13{hdr, offsets, gtoff, w->w13, dh1, nullptr, nullptr, dxr, nullptr,
              2 * d.f, d.d, d.f, d.d, d.e, (d.d + 255) / 256, 0, 0, mtoff};
  b13.row_slot = sorted_route;
  BwdArgs bw13{hdr, offsets, mtoff, nullptr, nullptr, dh1, sc + p->sl.x_rows, g->dw13, nullptr,
               0, 0, d.f, d.d, d.e, 0, d.d, 2 * d.f};
  bw13.acc_dw = (flags & MOE_BWD_ACCUMULATE_DW) ? 1 : 0;
  // dW13's A rows: a packed copy of the x rows (its loads then stream)
  auto gather = [&] {
    return timed(p, "gather", s, [&] {
      return launch_gather(x, d.d, p->es, d.k, hdr, route_to_row, sc + p->sl.x_rows, d.t_max,
                           s);
    });
  };
  if (mega) {
    // msync: [W2 tickets | one counter per expert and 256-column block of F | W13 tickets]
    uint32_t* ready = msync + kXcds;
    uint32_t* t13 = ready + int64_t(d.e) * msync_blocks(d.f);
    e = timed(p, "w2_bwd_mega", s, [&] {
      return launch_bwd_mega(0, dw_f32, b, bw2, msync, ready, cus, s);
    });
    if (e != hipSuccess) return MOE_ERR_HIP;
    e = gather();
    if (e != hipSuccess) return MOE_ERR_HIP;
    e = timed(p, "w13_bwd_mega", s, [&] {
      return launch_bwd_mega(1, dw_f32, b13, bw13, t13, nullptr, cus, s);
    });
    if (e != hipSuccess) return MOE_ERR_HIP;
  } else {
    e = timed(p, "w2_dgrad_swiglu", s, [&] { return launch_dgrad(0, b, p->mt_max, cus, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
    hot_wgrad(p, ws, bw2);
    e = timed(p, "w2_wgrad", s, [&] { return launch_wgrad(dw_f32, 2, bw2, cus, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
    e = timed(p, "w13_dgrad", s, [&] { return launch_dgrad(1, b13, p->mt_max, cus, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
    e = gather();
    if (e != hipSuccess) return MOE_ERR_HIP;
    hot_wgrad(p, ws, bw13);
    e = timed(p, "w13_wgrad", s, [&] { return launch_wgrad(dw_f32, 13, bw13, cus, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  e = timed(p, "dx_reduce", s, [&] {
    return launch_dx_reduce(d.prec, hdr, route_to_row, dxr, g->dx, d.k, d.d, d.t_max,
                            (flags & MOE_BWD_ACCUMULATE_DX) ? 1 : 0, s);
  });
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(timed(p, "rewind", s, [&] {
    return launch_plan_rewind(hdr, d.training ? arena : nullptr, s);
  }));
}

moe_status moe_read_status(void* ws, uint32_t* status, int32_t* replayed, hipStream_t s) {
  if (!ws || !status) return MOE_ERR_ARG;
  RouteHdr h;
  if (hipMemcpyAsync(&h, ws, sizeof h, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MOE_ERR_HIP;
  *status = h.status;
  if (replayed) *replayed = h.rec.replay;
  return MOE_OK;
}

moe_status moe_arena_reset(moe_plan_t p, void* arena, hipStream_t s) {
  if (!p || !arena) return MOE_ERR_ARG;
  return hip_status(launch_arena_reset(arena, s));
}

moe_status moe_route_readback(moe_plan_t p, void* ws, int32_t* counts, int32_t* offsets,
                              int32_t* poffsets, int32_t* sorted_route, int32_t* route_to_row,
                              int32_t* R_out, hipStream_t s) {
  if (!p || !ws) return MOE_ERR_ARG;
  RouteHdr h;
  if (hipMemcpyAsync(&h, ws, sizeof h, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MOE_ERR_HIP;
  const int64_t E = p->d.e;
  struct Item { void* dst; int64_t off; int64_t n; } items[] = {
      {counts, p->rl.counts, E},
      {offsets, p->rl.offsets, E + 1},
      {poffsets, p->rl.poffsets, E + 1},
      {sorted_route, p->rl.sorted_route, h.R},
      {route_to_row, p->rl.route_to_row, int64_t(h.T) * p->d.k},
  };
  for (auto& it : items) {
    if (!it.dst || it.n <= 0) continue;
    if (hipMemcpyAsync(it.dst, at<char>(ws, it.off), size_t(it.n) * 4, hipMemcpyDeviceToHost, s) !=
        hipSuccess)
      return MOE_ERR_HIP;
  }
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
  if (R_out) *R_out = h.R;
  return MOE_OK;
}

moe_status moe_saved_ptrs(moe_plan_t p, void* ws, void** x_rows, void** h1, hipStream_t s) {
  if (!p || !ws) return MOE_ERR_ARG;
  RouteHdr h;
  if (hipMemcpyAsync(&h, ws, sizeof h, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MOE_ERR_HIP;
  if (x_rows) *x_rows = reinterpret_cast<void*>(h.rec.x_rows);
  if (h1) *h1 = reinterpret_cast<void*>(h.rec.h1);
  return MOE_OK;
}

moe_status moe_timing_enable(moe_plan_t p, int32_t enable) {
  if (!p) return MOE_ERR_ARG;
  if (!enable) {
    for (auto& sl : p->slots)
      for (auto& ev : sl.pending) {
        hipEventSynchronize(ev.second);
        p->pool.push_back(ev.first);
        p->pool.push_back(ev.second);
      }
    p->slots.clear();
  }
  p->timing = enable != 0;
  return MOE_OK;
}

moe_status moe_expert_fwd_fused_noalloc(moe_plan_t p, void* ws, const void* x,
                                        const float* scores, const moe_weights* w,
                                        const void* y_addend, void* y, hipStream_t s);

moe_status moe_timing_flush(moe_plan_t p, void* buf, size_t bytes) {
  if (!p || (buf && (!aligned16(buf) || bytes < 16))) return MOE_ERR_ARG;
  p->flush_buf = buf;
  p->flush_bytes = buf ? int64_t(bytes) : 0;
  return MOE_OK;
}

moe_status moe_timing_read(moe_plan_t p, int32_t idx, char* name, size_t cap, double* total_ms,
                           int64_t* launches) {
  if (!p || idx < 0) return MOE_ERR_ARG;
  for (auto& sl : p->slots) {
    for (auto& ev : sl.pending) {
      float ms = 0.f;
      if (hipEventSynchronize(ev.second) != hipSuccess ||
          hipEventElapsedTime(&ms, ev.first, ev.second) != hipSuccess)
        return MOE_ERR_HIP;
      sl.total_ms += ms;
      sl.launches += 1;
      p->pool.push_back(ev.first);
      p->pool.push_back(ev.second);
    }
    sl.pending.clear();
  }
  if (size_t(idx) >= p->slots.size()) return MOE_ERR_ARG;
  const auto& sl = p->slots[size_t(idx)];
  if (name && cap) {
    std::strncpy(name, sl.name.c_str(), cap - 1);
    name[cap - 1] = '\0';
  }
  if (total_ms) *total_ms = sl.total_ms;
  if (launches) *launches = sl.launches;
  return MOE_OK;
}

}  // extern "C"

// ------------------------------------------------- allocation-free inference
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc):
// moe_expert_fwd_fused_noalloc keeps the fused forward's scratch and its fp32
// accumulation rows in this array instead of caller buffers.  Each GPU the
// library runs on holds its own copy until the process ends, and every call
// on that GPU shares it: calls that overlap on one GPU race.  In host code
// the name `scratch` is only a host-side stand-in; the device address comes
// from hipGetSymbolAddress, once per device, and only that address is used.
namespace {

constexpr size_t kNoAllocBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
void* g_noalloc_ptr[kMaxDevices] = {};

// This GPU's copy of `scratch` (the device of stream s; the current device
// for the null stream), looked up with that device current.
moe_status noalloc_base(hipStream_t s, char** out) {
  int dev = -1;
  if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess || dev < 0 ||
      dev >= kMaxDevices)
    return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return MOE_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return MOE_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return MOE_ERR_HIP;
    if (e != hipSuccess || !ptr) return MOE_ERR_HIP;
    g_noalloc_ptr[dev] = ptr;
  }
  *out = reinterpret_cast<char*>(g_noalloc_ptr[dev]);
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_expert_fwd_fused_noalloc(moe_plan_t p, void* ws, const void* x,
                                                   const float* scores, const moe_weights* w,
                                                   const void* y_addend, void* y,
                                                   hipStream_t s) {
  moe_status st = fused_check(p, ws, x, w, y_addend, y);
  if (st != MOE_OK) return st;
  // scratch layout of the plan, then the fp32 rows [t_max, D]
  const int64_t sc_bytes = a256(p->sl.total);
  const int64_t y32_bytes = a256(p->d.t_max * p->d.d * 4);
  if (sc_bytes + y32_bytes > int64_t(kNoAllocBytes)) return MOE_ERR_WORKSPACE;
  char* base = nullptr;
  st = noalloc_base(s, &base);
  if (st != MOE_OK) return st;
  return fused_forward(p, ws, x, scores, w, reinterpret_cast<float*>(base + sc_bytes), y_addend,
                       y, base, s);
}
