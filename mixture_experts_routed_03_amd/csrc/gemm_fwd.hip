// Grouped forward GEMMs of the expert FFN on gfx950 MFMA.
//
//   W13 pass:  h1 = A_e W13_e^T per expert (A_e = the expert's gathered rows),
//              epilogue stores h1 = [g | u] and h2 = SiLU(g) * u.
//   W2 pass:   h3 = H2_e W2_e^T, epilogue stores each row into its route slot
//              sorted_route[row] of h3_slots [T*K, D].
//
// Sources: Dist-MoE explainer section 02 (h1 = W13 x = [g; u],
// h2 = SiLU(g) * u, h3 = W2 h2) and section 05 (a persistent scheduler hands
// (expert, row tile, output tile) work to workgroups, one launch covers all
// local experts, tails are masked; the W2 epilogue writes each result to its
// return slot).  "Mixture of Experts: How Routing Becomes GPU Computation",
// section 2 (grouped GEMM over variable M_e with B stored [E, N, K]), section
// 1 (at small M_e the GEMM is bound by reading the weights) and section 6
// (column-major tile order so row tiles that share a weight block run next
// to each other).
//
// MI355X design
//  * The GEMMs are bound by streaming expert weights from HBM (~32 rows per
//    expert).  Each stage moves a 128-byte segment of 128 weight rows and of
//    the tile's <= 64 token rows with fully coalesced 16-byte loads (eight
//    consecutive lanes cover one row segment), stores them into LDS with a
//    per-row XOR swizzle of the 16-byte chunks, and the MFMA operands are
//    16-byte LDS reads.  Two further stages are in flight in registers
//    (ring of two), so ~48 KiB per workgroup is outstanding while a stage
//    computes.
//  * Workgroup tile: 128 weight rows (4 waves x 32) x 64 token rows, or x 128
//    token rows for an expert with more than 64 rows (its weight tiles are
//    then streamed once per 128 rows instead of once per 64).  Each wave
//    holds one 32x32 fp32 accumulator per 32-token block
//    (v_mfma_f32_32x32x16_bf16, or v_mfma_f32_32x32x2f32 for fp32 operands);
//    loop copies for 1, 2 and 4 blocks skip the blocks past the tile's last
//    row.  Within a stage, half h of a lane's operands covers chunks
//    [4h, 4h+4) of the row segment: a permutation of the contraction applied
//    identically to both operands.
//  * Persistent grid, XCD-aware: each XCD runs a contiguous run of work
//    items, split by token rows (xcd_first_tile), so one XCD's L2 holds an
//    expert's token rows while its n-tiles stream by; items are expert-major,
//    then n-tile, then m-tile, so m-tiles sharing a weight tile run side by
//    side.
#include <algorithm>

#include <type_traits>

#include "common.h"

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct Mma;
template <>
struct Mma<uint16_t> {
  static constexpr int kV = 1;  // u32x4 per 8-value operand
  static __device__ __forceinline__ void step(f32x16& acc, const u32x4* a, const u32x4* b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                  __builtin_bit_cast(bf16x8, b[0]), acc, 0, 0, 0);
  }
};
template <>
struct Mma<float> {
  static constexpr int kV = 2;
  static __device__ __forceinline__ void step(f32x16& acc, const u32x4* a, const u32x4* b) {
#pragma unroll
    for (int p = 0; p < 8; ++p)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[p >> 2][p & 3]),
                                                 __uint_as_float(b[p >> 2][p & 3]), acc, 0, 0, 0);
  }
};

// Stores 4 consecutive values of the accumulator as T.
template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, float a, float b, float c,
                                                 float d) {
  u32x2 v;
  v[0] = pack_bf16x2(a, b);
  v[1] = pack_bf16x2(c, d);
  *reinterpret_cast<u32x2*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// LDS byte offset of 16-byte chunk c of tile row r (128-byte rows).  Chunks
// are XOR-swizzled by (r ^ r>>3) & 7 so that both the row-wise writes (8 lanes
// per row) and the MFMA-layout reads (32 rows, one chunk) are spread over all
// banks.
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ ((r ^ (r >> 3)) & 7)) << 4); }

// Persistent grid size: a multiple of the XCD count, at most the upper bound
// on work items.
static unsigned fwd_grid(int64_t items_max, int cus, int per_cu) {
  int64_t g = std::min<int64_t>(items_max, int64_t(cus) * per_cu);
  g = (g + kXcds - 1) / kXcds * kXcds;
  return unsigned(std::max<int64_t>(g, kXcds));
}

constexpr int kFwdW = 128 * 128;          // weight stage: 128 rows x 128 B
constexpr int kFwdA = kBMX * 128;         // token stage: up to 128 rows x 128 B
constexpr int kFwdStage = kFwdW + kFwdA;
constexpr int kFwdLds = 2 * kFwdStage;    // two LDS stage buffers

// Main loop of one output tile: expert e, n-tile nt, token rows
// [row0, row0 + rows) (one of the expert's mt_e m-tiles), stages
// [s0, s0 + S) of the contraction, accumulated into acc.
// acc[b][v] is C[weight row 8*(v/4) + 4*lh + v%4][token 32*b + lr].
template <typename T, int MODE>
__device__ __forceinline__ void fwd_mainloop(const FwdArgs& a, char* lds, int e, int nt, int row0,
                                             int rows, int mt_e, int s0, int S, f32x16* acc) {
  constexpr int ES = sizeof(T);
  constexpr int kSteps = 128 / ES / 16;  // MFMA k-steps (16 values) per stage
  constexpr int kV = Mma<T>::kV;         // 16-byte chunks per 8-value operand
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;   // row inside the 32-row operand block
  const int lh = lane >> 5;   // operand half: chunks [4*lh, 4*lh + 4) of a stage row
  const int lc = tid & 7;     // loader: 16-byte chunk of a 128-byte row segment
  const int lrow = tid >> 3;  // loader: tile row (+ 32 j)
  const int64_t row_bytes = int64_t(a.Kd) * ES;
  // W13 reads the caller's x rows through the permutation (the gather is part
  // of this loader); W2 reads packed h2 rows.
  const char* Abase = reinterpret_cast<const char*>(MODE == 0 ? a.x : a.A);

  // Global sources of this thread's four weight chunks and four token
  // chunks.  Tile rows past the expert's last row re-read that row: the
  // loads are unconditional and the extra output columns are never stored.
  const char* wsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rho = lrow + 32 * j;
    const int wr = MODE == 0 ? (rho < 64 ? nt * 64 + rho : a.F + nt * 64 + rho - 64)
                             : nt * 128 + rho;
    wsrc[j] = reinterpret_cast<const char*>(a.W) + (int64_t(e) * a.N + wr) * row_bytes + lc * 16;
  }
  const char* tsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = row0 + min(lrow + 32 * j, rows - 1);
    const int64_t src = MODE == 0 ? a.sorted_route[r] / a.K : r;
    tsrc[j] = Abase + src * row_bytes + lc * 16;
  }

#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x16{};
  u32x4 R0[8], R1[8];
  // NB (a compile-time 32-row block count per loop copy: 1, 2 or 4) is the
  // number of token blocks loaded and multiplied.
  // Stages past the end (the pipeline's last two loads) are never used:
  // their weight loads read token rows, which sit in L2, instead of
  // re-reading the last weight stage (a non-temporal line that HBM would
  // have to supply again).
  auto load = [&](u32x4* R, int s, auto nb_c, auto tm_c) {
    constexpr int NB = decltype(nb_c)::value;
    constexpr bool TM = decltype(tm_c)::value;
    const bool past = s >= S;
    const int64_t off = int64_t(s0 + (past ? S - 1 : s)) * 128;
#pragma unroll
    for (int j = 0; j < 4; ++j) {   // weights: non-temporal unless TM (see below)
      const u32x4* src = reinterpret_cast<const u32x4*>((past ? tsrc[j] : wsrc[j]) + off);
      if constexpr (TM)
        R[j] = *src;
      else
        R[j] = __builtin_nontemporal_load(src);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) R[4 + j] = *reinterpret_cast<const u32x4*>(tsrc[j] + off);
  };
  auto store = [&](const u32x4* R, int buf, auto nb_c) {
    constexpr int NB = decltype(nb_c)::value;
    char* base = lds + buf * kFwdStage;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4*>(base + swz(lrow + 32 * j, lc)) = R[j];
#pragma unroll
    for (int j = 0; j < NB; ++j)
      *reinterpret_cast<u32x4*>(base + kFwdW + swz(lrow + 32 * j, lc)) = R[4 + j];
  };
  auto compute = [&](int buf, auto nb_c) {
    constexpr int NB = decltype(nb_c)::value;
    const char* wl = lds + buf * kFwdStage;
    const char* tl = wl + kFwdW;
    const int wrow = 32 * wave + lr;
#pragma unroll
    for (int q = 0; q < kSteps; ++q) {
      u32x4 av[kV], bv[NB][kV];
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        const int c = 4 * lh + q * kV + v;
        av[v] = *reinterpret_cast<const u32x4*>(wl + swz(wrow, c));
#pragma unroll
        for (int b = 0; b < NB; ++b)
          bv[b][v] = *reinterpret_cast<const u32x4*>(tl + swz(32 * b + lr, c));
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) Mma<T>::step(acc[b], av, bv[b]);
    }
  };

  // Pipeline: at the top of each pass LDS buffer 0 holds stage s, R1 stage
  // s + 1 and R0 stage s + 2.
  auto run = [&](auto nb_c, auto tm_c) {
    load(R0, 0, nb_c, tm_c);
    load(R1, 1, nb_c, tm_c);
    store(R0, 0, nb_c);
    load(R0, 2, nb_c, tm_c);
    lds_barrier();
    for (int s = 0; s + 1 < S; s += 2) {
      compute(0, nb_c);
      store(R1, 1, nb_c);
      load(R1, s + 3, nb_c, tm_c);
      lds_barrier();
      compute(1, nb_c);
      store(R0, 0, nb_c);
      load(R0, s + 4, nb_c, tm_c);
      lds_barrier();
    }
    if (S & 1) {
      compute(0, nb_c);
      lds_barrier();
    }
  };
  // An expert cut into several m-tiles re-reads its weight tiles once per
  // m-tile; those items run side by side on one XCD, so its weights are
  // loaded with the default (L2-allocating) policy to serve the sibling
  // tiles from L2.  A single-tile expert streams its weights non-temporally.
  auto go = [&](auto tm_c) {
    if (rows > 64)
      run(std::integral_constant<int, 4>{}, tm_c);
    else if (rows > 32)
      run(std::integral_constant<int, 2>{}, tm_c);
    else
      run(std::integral_constant<int, 1>{}, tm_c);
  };
  if (mt_e > 1)
    go(std::true_type{});
  else
    go(std::false_type{});
}

// Epilogue of a complete tile.  W13 (MODE 0): h1 = [g | u] rounded to T
// into out0, then SwiGLU: up waves (2,3) hand their rounded values to gate
// waves (0,1) through LDS, one 32-row block at a time, and the gate waves
// store h2 = SiLU(g) * u into out1.  W2 (MODE 1): each row to its route slot
// sorted_route[row] of out0, or score * row added into y32 (FUSED combine).
template <typename T, int MODE>
__device__ __forceinline__ void fwd_epilogue(const FwdArgs& a, char* lds, T* out0, T* out1, int nt,
                                             int row0, int rows, const f32x16* acc) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  if (MODE == 0) {
    const int F = a.F;
    const int ncol = (wave < 2 ? 0 : F) + nt * 64 + (wave & 1) * 32 + 4 * lh;
    const int jcol = nt * 64 + (wave & 1) * 32 + 4 * lh;
    const int nbk = (rows + 31) >> 5;
    float* xch = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b < nbk) {
        const int m = 32 * b + lr;
        if (m < rows) {
          T* o = out0 + int64_t(row0 + m) * (2 * F) + ncol;
#pragma unroll
          for (int g = 0; g < 4; ++g)
            store4<T>(o + 8 * g, acc[b][4 * g], acc[b][4 * g + 1], acc[b][4 * g + 2],
                      acc[b][4 * g + 3]);
        }
        if (wave >= 2) {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            xch[((wave - 2) * 16 + v) * 64 + lane] = Elem<T>::round(acc[b][v]);
        }
        lds_barrier();
        if (wave < 2 && m < rows) {
          float h[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float g = Elem<T>::round(acc[b][v]);
            const float up = xch[(wave * 16 + v) * 64 + lane];
            h[v] = silu_f(clamp_gate(g, a.limit)) * clamp_up(up, a.limit);
          }
          T* o = out1 + int64_t(row0 + m) * F + jcol;
#pragma unroll
          for (int g = 0; g < 4; ++g)
            store4<T>(o + 8 * g, h[4 * g], h[4 * g + 1], h[4 * g + 2], h[4 * g + 3]);
        }
        lds_barrier();
      }
    }
  } else {
    const int ncol = nt * 128 + wave * 32 + 4 * lh;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int m = 32 * b + lr;
      if (m < rows) {
        const int64_t slotr = a.sorted_route[row0 + m];
        if (a.y32) {
          const float sc = a.scores[slotr];
          float* o = a.y32 + (slotr / a.K) * a.N + ncol;
#pragma unroll
          for (int g = 0; g < 4; ++g)
            fused_add4(o + 8 * g, sc, Elem<T>::round(acc[b][4 * g]),
                       Elem<T>::round(acc[b][4 * g + 1]), Elem<T>::round(acc[b][4 * g + 2]),
                       Elem<T>::round(acc[b][4 * g + 3]));
        } else {
          T* o = out0 + slotr * a.N + ncol;
#pragma unroll
          for (int g = 0; g < 4; ++g)
            store4<T>(o + 8 * g, acc[b][4 * g], acc[b][4 * g + 1], acc[b][4 * g + 2],
                      acc[b][4 * g + 3]);
        }
      }
    }
  }
}

// SPLIT: the split-K instantiation (a.ksplit parts per output tile).
template <typename T, int MODE, bool SPLIT>
__global__ __launch_bounds__(256, 2) void k_gemm_fwd(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kFwdLds];
  const int tid = threadIdx.x;

  const RouteHdr* hdr = a.hdr;
  if (a.replay_only && !hdr->rec.replay) return;
  // a.mtoff is the m-tile prefix: experts with more than 64 rows are cut
  // into 128-row tiles, the others into one 64-row tile.  With split-K each
  // output tile is ks consecutive items, one per range of stages.
  const int ks = SPLIT ? a.ksplit : 1;
  const int n_items = a.mtoff[a.E] * a.NT * ks;
  if (MODE == 0 && !a.x) {  // rows to compute need x: report instead of faulting
    if (n_items > 0 && blockIdx.x == 0 && threadIdx.x == 0)
      atomicOr(const_cast<uint32_t*>(&hdr->status), MOE_STATUS_NULL_INPUT);
    return;
  }
  T* out0 = a.out0 ? reinterpret_cast<T*>(a.out0) : global_ptr<T>(hdr->rec.h1);
  T* out1 = reinterpret_cast<T*>(a.out1);
  const int ES = sizeof(T);
  const int S_all = int(int64_t(a.Kd) * ES / 128);

  const int xcd = blockIdx.x % kXcds;
  const int per = gridDim.x / kXcds;
  const int first = xcd_first_tile(a.mtoff, a.stoff, a.E, a.NT, xcd) * ks;
  const int last = xcd_first_tile(a.mtoff, a.stoff, a.E, a.NT, xcd + 1) * ks;

  // items [first, last) of this XCD come from its work queue, in order
  // (with skewed routing: when some expert spans several m-tiles; otherwise
  // dealt statically, slot, slot + per, ..., which costs no atomics)
  const bool dyn = hdr->max_count > kBMX;
  const int slot = blockIdx.x / kXcds;
  __shared__ int s_next;
  if (dyn && tid == 0) s_next = wq_take(hdr, xcd);
  lds_barrier();
  int e_prev = -1;  // expert of this workgroup's previous item
  for (int w = dyn ? first + s_next : first + slot; w < last;) {
    const int wt = ks > 1 ? w / ks : w;   // output tile
    const int kp = w - wt * ks;           // its stage range: [s0, s0 + S)
    const int s0 = int(int64_t(kp) * S_all / ks);
    const int S = int(int64_t(kp + 1) * S_all / ks) - s0;
    const int e = item_expert(a.mtoff, a.E, a.NT, wt, e_prev);
    e_prev = e;
    const int mt_e = a.mtoff[e + 1] - a.mtoff[e];
    const int u = wt - a.mtoff[e] * a.NT;
    const int nt = u / mt_e;
    const int mt = u - nt * mt_e;
    const int bm = gemm_tile_rows(a.offsets[e + 1] - a.offsets[e]);
    const int row0 = a.offsets[e] + mt * bm;
    const int rows = min(bm, a.offsets[e + 1] - row0);

    f32x16 acc[4];
    fwd_mainloop<T, MODE>(a, lds, e, nt, row0, rows, mt_e, s0, S, acc);

    // the next item, taken while this one's epilogue runs
    int taken = 0;
    if (dyn && tid == 0) taken = wq_take(hdr, xcd);

    if (SPLIT) {
      // Split-K ("Mixture of Experts: How Routing Becomes GPU Computation",
      // section 6): this part's fp32 tile, columns as the complete tile
      // would be stored; k_fwd_splitk_finish adds the parts.
      const int lane = tid & 63, wave = tid >> 6, lr = lane & 31, lh = lane >> 5;
      const int ncol = MODE == 0 ? (wave < 2 ? 0 : a.F) + nt * 64 + (wave & 1) * 32 + 4 * lh
                                 : nt * 128 + wave * 32 + 4 * lh;
      float* P = a.part + (int64_t(kp) * a.part_rows + row0) * a.N + ncol;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int m = 32 * b + lr;
        if (m < rows) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            store4<float>(P + int64_t(m) * a.N + 8 * g, acc[b][4 * g], acc[b][4 * g + 1],
                          acc[b][4 * g + 2], acc[b][4 * g + 3]);
        }
      }
    } else {
      fwd_epilogue<T, MODE>(a, lds, out0, out1, nt, row0, rows, acc);
    }
    if (dyn) {
      if (tid == 0) s_next = taken;
      lds_barrier();
      w = first + s_next;
    } else {
      w += per;
    }
  }
  if (dyn && tid == 0) wq_finish(hdr, xcd, per);
}

// Fused (Mega) forward: W13 + SwiGLU and W2 in one persistent grid
// (Dist-MoE explainer, section 05, "Kernel Pipelines: Staged and Mega": one
// grid runs both projections' work records, and counters in HBM tell a W2
// record when the h2 rows it reads are complete).
//
// MI355X design.  Each XCD has its own L2, and making a store visible to
// another XCD takes an agent-scope release (an L2 write-back) and acquire
// (an L2 invalidate) that serialize in the L2 controller; measured here at
// over a microsecond each, they would cost more than the h2 round trip this
// kernel saves.  So producer and consumer of every h2 row share one L2:
//  * each XCD owns a contiguous range of experts, split by m-tile counts
//    (xcd_first_unit over the m-tile prefix, one unit per expert), and runs
//    all their W13 and W2 records from its own ticket queue; a workgroup
//    picks the queue of the XCD it actually runs on (hw_xcd);
//  * the queue interleaves records expert by expert: W13 of expert j, then
//    W2 of expert j - look, so W2 records find their h2 rows finished or
//    nearly so;
//  * a W13 record stores h1/h2, waits until its stores are complete in L2
//    (vmcnt 0), and counts itself in ready[e]; a W2 record of expert e
//    first waits (one thread, atomic reads, bounded) until ready[e] equals
//    the expert's W13 record count.  Its h2 loads then come from the same
//    L2; no workgroup on this CU read those lines earlier in the launch.
// A W2 record only waits for records taken before it from the same queue,
// whose workgroups wait on nothing, so the wait always ends.  Tickets and
// counters (msync) are zeroed by the planner launch before each call.
constexpr int kMegaSpin = 1 << 22;   // polls (each followed by a short sleep)

template <typename T>
__global__ __launch_bounds__(256, 2) void k_gemm_mega(FwdArgs a13, FwdArgs a2, uint32_t* msync,
                                                      int look) {
  __shared__ __attribute__((aligned(16))) char lds[kFwdLds];
  __shared__ int s_t;
  const int tid = threadIdx.x;
  const RouteHdr* hdr = a13.hdr;
  const int E = a13.E;
  const int32_t* gt = a13.mtoff;   // m-tile prefix
  const int NT13 = a13.NT, NT2 = a2.NT;
  if (!a13.x) {   // rows to compute need x: report instead of faulting
    if (gt[E] > 0 && blockIdx.x == 0 && tid == 0)
      atomicOr(const_cast<uint32_t*>(&hdr->status), MOE_STATUS_NULL_INPUT);
    return;
  }
  T* h1 = a13.out0 ? reinterpret_cast<T*>(a13.out0) : global_ptr<T>(hdr->rec.h1);
  T* h2 = reinterpret_cast<T*>(a13.out1);
  T* h3 = reinterpret_cast<T*>(a2.out0);
  const int S13 = int(int64_t(a13.Kd) * sizeof(T) / 128);
  const int S2 = int(int64_t(a2.Kd) * sizeof(T) / 128);

  const int xcd = hw_xcd();
  uint32_t* ticket = msync + xcd;
  uint32_t* ready = msync + kXcds;
  const int e_lo = xcd_first_unit(gt, 0, E, 1, xcd);
  const int e_hi = xcd_first_unit(gt, 0, E, 1, xcd + 1);
  const int ne = e_hi - e_lo;
  const int g0 = gt[e_lo];
  // queue block j: W13 records of expert e_lo + j (j < ne), then W2 records
  // of expert e_lo + j - look (j >= look); start(j) = records before block j
  auto start = [&](int j) {
    const int a = min(j, ne), b = max(0, min(j - look, ne));
    return (gt[e_lo + a] - g0) * NT13 + (gt[e_lo + b] - g0) * NT2;
  };
  const int total = (gt[e_hi] - g0) * (NT13 + NT2);
  int j_lo = 0;   // tickets only grow, so blocks only move forward
  for (;;) {
    if (tid == 0) s_t = int(atomicAdd(ticket, 1u));
    lds_barrier();
    const int t = s_t;   // every record below passes a barrier before s_t is written again
    if (t >= total) break;
    int hi = ne + look;   // start(j_lo) <= t < start(hi) = total
    while (hi - j_lo > 1) {
      const int mid = (j_lo + hi) >> 1;
      if (start(mid) <= t)
        j_lo = mid;
      else
        hi = mid;
    }
    const int j = j_lo;
    int u = t - start(j);
    const int c13 = j < ne ? (gt[e_lo + j + 1] - gt[e_lo + j]) * NT13 : 0;
    const bool w13 = u < c13;
    const int e = w13 ? e_lo + j : e_lo + j - look;
    if (!w13) u -= c13;
    const int mt_e = gt[e + 1] - gt[e];
    const int nt = u / mt_e;
    const int mt = u - nt * mt_e;
    const int bm = gemm_tile_rows(a13.offsets[e + 1] - a13.offsets[e]);
    const int row0 = a13.offsets[e] + mt * bm;
    const int rows = min(bm, a13.offsets[e + 1] - row0);
    f32x16 acc[4];
    if (w13) {
      fwd_mainloop<T, 0>(a13, lds, e, nt, row0, rows, mt_e, 0, S13, acc);
      fwd_epilogue<T, 0>(a13, lds, h1, h2, nt, row0, rows, acc);
      // this record's h1/h2 stores complete in L2, then counted
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      if (tid == 0) atomicAdd(&ready[e], 1u);
    } else {
      if (tid == 0) {
        const uint32_t need = uint32_t(mt_e * NT13);
        int n = 0;
        while (atomicAdd(&ready[e], 0u) < need && ++n < kMegaSpin) __builtin_amdgcn_s_sleep(4);
        if (n >= kMegaSpin) atomicOr(const_cast<uint32_t*>(&hdr->status), MOE_STATUS_SYNC_TIMEOUT);
      }
      __syncthreads();
      fwd_mainloop<T, 1>(a2, lds, e, nt, row0, rows, mt_e, 0, S2, acc);
      fwd_epilogue<T, 1>(a2, lds, h3, nullptr, nt, row0, rows, acc);
    }
  }
}

hipError_t launch_gemm_mega(int prec, const FwdArgs& a13, const FwdArgs& a2, uint32_t* msync,
                            int look, int64_t mt_max, int cus, hipStream_t s) {
  if (mt_max == 0) return hipSuccess;
  const int64_t items = mt_max * (a13.NT + a2.NT);
  if (prec == MOE_PREC_F32) {
    hipLaunchKernelGGL(k_gemm_mega<float>, dim3(fwd_grid(items, cus, 2)), dim3(256), 0, s, a13, a2,
                       msync, look);
  } else {
    hipLaunchKernelGGL(k_gemm_mega<uint16_t>, dim3(fwd_grid(items, cus, 2)), dim3(256), 0, s, a13,
                       a2, msync, look);
  }
  return hipGetLastError();
}

// Second pass of a split-K forward GEMM ("Mixture of Experts: How Routing
// Becomes GPU Computation", section 6, Split-K: the partial results of one
// output tile are added by a separate reduction kernel).  A thread handles
// four adjacent output columns of one packed row: its loads of all parts are
// issued together, then added in order k = 0, 1, ..., so the result does not
// depend on scheduling.  The epilogue is the one of the single-pass kernel:
// W13 rounds g and u to T, stores h1 = [g | u] and h2 = SiLU(g) * u; W2
// stores the row into its route slot, or adds score * row into y32 (FUSED
// combine).
constexpr int kMaxSplit = 8;

template <typename T, int MODE>
__global__ __launch_bounds__(256) void k_fwd_splitk_finish(FwdArgs a) {
  const RouteHdr* hdr = a.hdr;
  if (a.replay_only && !hdr->rec.replay) return;
  const int ks = a.ksplit;
  const int64_t R = hdr->R;
  const int cols = (MODE == 0 ? a.F : a.N) / 4;   // 4-column groups per row
  const int64_t n = R * cols;
  const int64_t pstride = a.part_rows * a.N;
  T* h1 = MODE == 0 ? (a.out0 ? reinterpret_cast<T*>(a.out0) : global_ptr<T>(hdr->rec.h1))
                    : nullptr;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const int64_t r = i / cols;
    const int c = int(i - r * cols) * 4;
    const float* P = a.part + r * a.N + c;
    constexpr int NV = MODE == 0 ? 2 : 1;   // W13: gate and up columns
    float4 q[kMaxSplit][NV];
#pragma unroll
    for (int k = 0; k < kMaxSplit; ++k) {
      if (k < ks) {
#pragma unroll
        for (int h = 0; h < NV; ++h)
          q[k][h] = *reinterpret_cast<const float4*>(P + k * pstride + h * a.F);
      }
    }
    float v[NV][4] = {};
#pragma unroll
    for (int k = 0; k < kMaxSplit; ++k) {
      if (k < ks) {
#pragma unroll
        for (int h = 0; h < NV; ++h) {
          v[h][0] += q[k][h].x;
          v[h][1] += q[k][h].y;
          v[h][2] += q[k][h].z;
          v[h][3] += q[k][h].w;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < NV; ++h) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[h][j] = Elem<T>::round(v[h][j]);
    }
    if constexpr (MODE == 0) {
      T* o = h1 + r * (2 * a.F) + c;
      store4<T>(o, v[0][0], v[0][1], v[0][2], v[0][3]);
      store4<T>(o + a.F, v[1][0], v[1][1], v[1][2], v[1][3]);
      float hh[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        hh[j] = silu_f(clamp_gate(v[0][j], a.limit)) * clamp_up(v[1][j], a.limit);
      store4<T>(reinterpret_cast<T*>(a.out1) + r * a.F + c, hh[0], hh[1], hh[2], hh[3]);
    } else {
      const int64_t slotr = a.sorted_route[r];
      if (a.y32)
        fused_add4(a.y32 + (slotr / a.K) * a.N + c, a.scores[slotr], v[0][0], v[0][1], v[0][2],
                   v[0][3]);
      else
        store4<T>(reinterpret_cast<T*>(a.out0) + slotr * a.N + c, v[0][0], v[0][1], v[0][2],
                  v[0][3]);
    }
  }
}

template <typename T, int MODE>
static hipError_t launch_fwd_t(const FwdArgs& a, int64_t mt_max, int cus, hipStream_t s) {
  static int per_cu = 0;  // resident workgroups per CU (same on every gfx950 device)
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gemm_fwd<T, MODE, false>, 256, 0) !=
            hipSuccess ||
        n <= 0)
      n = 1;
    per_cu = n;
  }
  const int ks = a.ksplit > 1 ? a.ksplit : 1;
  const unsigned g = fwd_grid(mt_max * a.NT * ks, cus, per_cu);
  if (ks > 1) {
    if (ks > kMaxSplit) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_gemm_fwd<T, MODE, true>), dim3(g), dim3(256), 0, s, a);
    // rows <= part_rows; one thread per 4 output columns of a row
    const int64_t cols = (MODE == 0 ? a.F : a.N) / 4;
    const int64_t blocks = std::min<int64_t>((a.part_rows * cols + 255) / 256, int64_t(cus) * 8);
    hipLaunchKernelGGL((k_fwd_splitk_finish<T, MODE>), dim3(unsigned(std::max<int64_t>(blocks, 1))),
                       dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_gemm_fwd<T, MODE, false>), dim3(g), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_hot(int mode, const FwdArgs& a, int64_t items_max, int cus,
                           hipStream_t s);

// mode 0: W13 + SwiGLU (out0 = h1 or null, out1 = h2); mode 1: W2 -> slots.
// BF16 with a.hotoff: the cold experts' items (prefixes ctoff / cstoff) on
// the streaming tiles, then the hot experts' 256 x 256 tiles (k_gemm_hot;
// each hot expert has at most as many 256-row tiles as 128-row ones, so
// mt_max bounds them too).
hipError_t launch_gemm_fwd(int prec, int mode, const FwdArgs& a, int64_t mt_max, int cus,
                           hipStream_t s) {
  if (mt_max == 0) return hipSuccess;
  if (prec == MOE_PREC_F32)
    return mode == 0 ? launch_fwd_t<float, 0>(a, mt_max, cus, s)
                     : launch_fwd_t<float, 1>(a, mt_max, cus, s);
  if (a.hotoff) {
    FwdArgs c = a;
    c.ksplit = 1;   // the finish pass would cover the hot experts' rows too
    c.mtoff = a.ctoff;
    c.stoff = a.cstoff;
    const hipError_t e = mode == 0 ? launch_fwd_t<uint16_t, 0>(c, mt_max, cus, s)
                                   : launch_fwd_t<uint16_t, 1>(c, mt_max, cus, s);
    if (e != hipSuccess) return e;
    FwdArgs h = a;
    h.NT = mode == 0 ? a.F / 128 : a.N / 256;
    return launch_gemm_hot(mode, h, mt_max * h.NT, cus, s);
  }
  return mode == 0 ? launch_fwd_t<uint16_t, 0>(a, mt_max, cus, s)
                   : launch_fwd_t<uint16_t, 1>(a, mt_max, cus, s);
}

}  // namespace moe
