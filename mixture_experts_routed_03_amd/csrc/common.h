// Internal layouts and device helpers shared by the gfx950 kernels and the
// host entry points of libmoe.  Nothing here is part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---------------------------------------------------------------- constants
constexpr int kBM = 64;           // token rows per WGRAD contraction stage (and small m-tiles)
constexpr int kBMX = 128;         // token rows of an FPROP/DGRAD m-tile of an expert with > kBM rows
constexpr int kRankChunk = 256;   // routes per counting-sort chunk
constexpr int kMxBlock = 32;      // MX block length (values per E8M0 scale)
// Experts per plan.  Routing keeps one counter per expert in LDS for each
// 256-route chunk (16 KiB at 4,096) and the one-workgroup decode router holds
// E counters too; 4,096 experts is ten times the pages' largest count (384),
// and at their expert size (D = 7,168, F = 2,048) 4,096 bf16 experts would
// already need 360 GB of weights, more than one GPU's 288 GB of HBM.
constexpr int kMaxE = 4096;
constexpr int kMaxK = 16;
constexpr int kMaxWidth = 65536;  // largest D and F

__host__ __device__ inline int64_t align_up(int64_t n, int64_t a) { return (n + a - 1) / a * a; }
__host__ __device__ inline int64_t align128(int64_t n) { return align_up(n, 128); }
// Token rows per FPROP/DGRAD m-tile of an expert with c rows: a hot expert
// takes 128-row tiles, so each weight tile is streamed once per 128 rows.
__host__ __device__ inline int gemm_tile_rows(int c) { return c > kBM ? kBMX : kBM; }
// BF16 forward: an expert with at least kHotRows rows is MFMA-bound (its
// weight tiles are reused by many token rows) and runs on 256 x 256 tiles
// (k_gemm_hot); the others stream their weights on the tiles above.
constexpr int kHotRows = 256;
constexpr int kBMH = 256;         // token rows of a hot-expert m-tile
__host__ __device__ inline bool hot_expert(int c) { return c >= kHotRows; }
// BF16 weight gradients: an expert with at least kHotWgRows rows runs on
// k_wgrad_hot's 256 x 256 tiles, the others on k_gemm_wgrad's streaming
// tiles.  Measured on MI355X with three stages in flight in the large tiles:
// on ~256-row experts (8 or 9 stages of 32 rows) they took the W13 weight
// gradient from 1.40 to 1.31-1.34 ms and the W2 one from 0.70 to 0.66 ms;
// cutoffs of 384 and 512 rows measured no better on skewed routing.
constexpr int kHotWgRows = 256;
__host__ __device__ inline bool hot_wgrad_expert(int c) { return c >= kHotWgRows; }

// ------------------------------------------------- per-layer planner record
// Written on the device by the planner kernel during forward, read by every
// later kernel of that layer (forward and backward).  Pointers are device
// addresses resolved from the arena cursor or the scratch buffer.
struct LayerRec {
  int64_t start;        // arena byte offset of this layer's saved state
  int64_t bytes;        // bytes this layer keeps in the arena
  int32_t replay;       // 1: state lives in scratch; backward rebuilds it
  int32_t layer;
  int32_t done;         // forward ran
  int32_t pad0;
  uint64_t x_rows;      // gathered x rows [R, D] (act dtype)
  uint64_t h1;          // h1 [R, 2F] (act dtype)
  uint64_t aux[6];      // MXFP8 bundles
};

// Header at the start of a route workspace.
struct RouteHdr {
  int32_t T;            // tokens of the call
  int32_t R;            // valid routes = packed rows
  int32_t Rpad;         // sum over experts of counts rounded up to 32
  int32_t n_mt;         // 64-row stages over all experts (sum of ceil(count / 64))
  uint32_t status;      // MOE_STATUS_* bits
  int32_t max_count;    // largest expert row count
  // Work queues of the persistent GEMM launches: per XCD, the next item
  // ticket [0, 8) and the count of workgroups that found the queue empty
  // [8, 16).  Zeroed by routing; the last workgroup of a launch to finish
  // on an XCD zeroes that XCD's pair again for the next launch.
  uint32_t wq[16];
  LayerRec rec;
};
static_assert(sizeof(RouteHdr) <= 512, "route header must fit its slot");


struct ArenaHdr {
  int64_t cursor;       // next free byte of the data region
  int64_t pad[31];
};
constexpr int64_t kArenaHdrBytes = 4096;  // data region starts here

// Byte offsets inside a route workspace (host computed from the plan).
struct RouteLayout {
  int64_t hdr, counts, offsets, poffsets, mtoff, gtoff, chunk_hist, chunk_flags,
      sorted_route, route_to_row, total;
  // Fused (Mega) launches: kXcds work-queue tickets, completion counters
  // (forward: W13 tiles per expert; backward: W2 DGRAD tiles per expert and
  // 256-column block of F, E * ceil(F / 256) words), then kXcds tickets of the
  // fused W13 backward (uint32, zeroed before each fused call)
  int64_t msync;
  // BF16 forward split: the cold experts' 64-row stage and m-tile prefixes
  // (hot experts count 0) and the hot experts' 256-row m-tile prefix; BF16
  // WGRAD split: the 64-row stage prefix of the experts below kHotWgRows rows
  int64_t cstoff, ctoff, hotoff, cwoff;
  int64_t nchunks;
};

// Byte offsets inside the scratch buffer (regions sized for R = t_max*K and
// the padded row count Rp; -1 = region absent).
struct ScratchLayout {
  int64_t x_rows, h1, h2, dh3, dh1, dxr;
  // MXFP8: row-quantized operands (codes, exponents) and column bundles
  int64_t qx, sx, qh2, sh2, xcq, xcs, h2cq, h2cs;
  int64_t qdh3, sdh3, dh3cq, dh3cs, qdh1, sdh1, dh1cq, dh1cs;
  int64_t part;   // split-K partial tiles of the forward GEMMs (plans that split)
  int64_t total;
};

// Arguments of the grouped forward GEMM launches.
struct FwdArgs {
  const RouteHdr* hdr;
  const int32_t* offsets;
  const int32_t* mtoff;
  const int32_t* sorted_route;
  const void* A;    // token rows [R, Kd] (W2: h2); unused when x is set
  const void* W;    // [E, N, Kd]
  void* out0;       // W13: h1 [R, 2F] (null = record); W2: h3 slots [T*K, D]
  void* out1;       // W13: h2 [R, F]
  int Kd;           // contraction length (D for W13, F for W2)
  int N;            // weight rows per expert (2F or D)
  int F;
  int NT;           // n-tiles per expert
  int E;
  int replay_only;  // 1: run only when the layer's forward chose replay
  const void* x;    // W13: the caller's x [T, Kd]; packed row r reads x[sorted_route[r] / K]
  int K;
  // W2 FUSED combine: y32[t] += scores[route] * h3 (fp32 atomic add) instead
  // of the slot store (y32 null: slots)
  const float* scores;
  float* y32;
  const int32_t* stoff;  // 64-row stage prefix (XCD work split, xcd_first_tile)
  float limit;           // W13: clamped SwiGLU limit (+inf: plain)
  // BF16 only (null: every expert on the streaming tiles): the cold experts'
  // m-tile and stage prefixes and the hot experts' 256-row m-tile prefix
  const int32_t* ctoff;
  const int32_t* cstoff;
  const int32_t* hotoff;
  // Split-K (streaming tiles only; <= 1: none).  Each output tile's stage
  // loop is cut into ksplit contiguous ranges run as separate items; item k
  // stores its fp32 partial tile to part[k][row][column] (part_rows rows per
  // part, columns as in h1 / the W2 output), and a second launch adds the
  // parts in order k = 0, 1, ... before the epilogue.
  int ksplit;
  float* part;
  int64_t part_rows;
};

// Arguments of the grouped backward GEMM launches.
struct BwdArgs {
  const RouteHdr* hdr;
  const int32_t* offsets;
  const int32_t* mtoff;
  const void* W;        // DGRAD weight [E, Kd, N] (row = contraction index)
  const void* tok;      // DGRAD token operand rows [R, Kd] (dH3 or dH1)
  const void* grad;     // WGRAD gradient rows (dH3 [R, D] or dH1 [R, 2F])
  const void* arows;    // WGRAD A-operand rows (h2 [R, F] or packed x rows [R, D])
  void* out;            // dH1 [R, 2F] / dXr [R, D] fp32 / dW2 [E, D, F] / dW13 [E, 2F, D]
  void* out2;           // W2 DGRAD: h2 [R, F] rebuilt from h1 for W2 WGRAD
  int Kd;               // DGRAD contraction length
  int N;                // DGRAD output columns
  int F, D, E;
  int NT;               // DGRAD n-tiles per expert
  int a_ld, b_ld;       // WGRAD row lengths of the A rows (= dW row length) and B rows (= dW rows)
  const int32_t* stoff; // DGRAD: 64-row stage prefix (XCD work split); mtoff = the m-tile prefix
  int acc_dw;           // WGRAD: 1 = dW += result (fp32 sum, rounded once), 0 = dW = result
  float limit;          // W2 DGRAD: clamped SwiGLU limit (+inf: plain)
  const int32_t* row_slot;  // W13 DGRAD: dXr row r goes to slot row_slot[r] (the route t*K+k)
  // WGRAD with hot_wg = 1 (bf16 dW, no accumulation, a_ld and b_ld multiples
  // of 256): experts of kHotWgRows rows or more run on k_wgrad_hot's 256 x 256
  // tiles; cst = routing's 64-row stage prefix of the other experts (those
  // count 0)
  const int32_t* cst;
  int hot_wg;
};

// Arguments of the MXFP8 grouped GEMM launches.
struct MxArgs {
  const RouteHdr* hdr;
  const int32_t* offsets;
  const int32_t* poffsets;
  const int32_t* mtoff;
  const int32_t* sorted_route;
  const uint8_t* qa;    // FPROP/DGRAD: row-quantized token operand [R, Kd]; WGRAD: A column bundle
  const uint8_t* sa;    //   exponents [R, Kd/32] / A bundle exponents
  const uint8_t* qw;    // FPROP/DGRAD: E4M3 weights [E, N, Kd] (DGRAD: [E, Kd, N])
  const uint8_t* sw;    //   32x32 exponents
  const uint8_t* qb;    // WGRAD: B column bundle
  const uint8_t* sb;
  void* out0;           // h1 (null = record) / h3 slots / dH1 / dXr / dW
  void* out1;           // h2 (W13 forward)
  int Kd, N, F, NT, E;
  int a_ld, b_ld;       // WGRAD row lengths of A (= dW row length) and B (= dW rows)
  int a_slot;           // WGRAD: >= 0 takes A codes/exponents from record aux[a_slot], aux[a_slot+1]
  int replay_only;
  int sa_rows;          // FPROP/DGRAD: row stride of the stage-grouped token exponents
  const float* scores;  // W2 FUSED combine (see FwdArgs)
  float* y32;
  int K;
  const int32_t* stoff;  // DGRAD: 64-row stage prefix (XCD work split); mtoff = the m-tile prefix
  int acc_dw;            // WGRAD: 1 = dW += result (fp32 sum, rounded once), 0 = dW = result
  float limit;           // W13 FPROP / W2 DGRAD: clamped SwiGLU limit (+inf: plain)
  int w1x32;             // FPROP: weights in 1x32 blocks, exponents grouped by 128-value
                         // stage: dword (s, e*N + n) of [Kd/128][sw_rows] (see k_rowq)
  int sw_rows;           // E * N for w1x32
  int fp4;               // FPROP: E2M1 operands (two per byte) with 1x32 weight blocks;
                         // exponents grouped by 256-value stage, [Kd/256][rows][8]
  // W13 FPROP: h2 rows quantized in the epilogue (null: none), as k_rowq
  // writes them: codes [R, F] (E2M1 with fp4: [R, F/2]) and exponents grouped
  // by stage with q_rows rows (the W2 FPROP's token operand)
  uint8_t* q_out;
  uint8_t* s_out;
  int q_rows;
  // WGRAD with hot_wg = 1 (bf16 dW, no accumulation, a_ld and b_ld
  // multiples of 256): the experts of kHotWgRows rows or more run on
  // k_mx_wgrad_hot's 256 x 256 tiles; cst = routing's 64-row stage prefix of
  // the other experts (the streaming launch's XCD split)
  const int32_t* cst;
  int hot_wg;
};

// Arguments of the MXFP8 quantizer launches (pointers or layer-record slots:
// 0..5 = rec.aux[slot], 6 = rec.x_rows, 7 = rec.h1).
struct RowqArgs {
  const RouteHdr* hdr;
  const void* src;      // bf16 [R, N]
  uint8_t* q;           // [R, N]
  uint8_t* s;           // exponents, see s_rows
  int N;
  int src_slot, q_slot, s_slot;
  int replay_only;
  int s_rows;           // 0: exponents [R, N/32]; > 0: grouped by 128-column stage,
                        // [N/128][s_rows][4] (a stage's exponents of consecutive rows
                        // are consecutive dwords)
  const int32_t* gather;  // non-null: source row r is src[gather[r] / K] (src = x [T, N])
  int K;
  int64_t rows;         // > 0: rows to quantize (hdr unused); 0: the route header's R
  int fp4;              // 1: E2M1 codes, two per byte (q is [R, N/2]); grouped exponents
                        // then come per 256-column stage, [N/256][s_rows][8]
};
struct ColqArgs {
  const RouteHdr* hdr;
  const int32_t* offsets;
  const int32_t* poffsets;
  const void* src;      // bf16 [R, N]
  uint8_t* q;           // column-bundle codes (sum_e N * Mp_e bytes)
  uint8_t* s;           // column-bundle exponents (sum_e N * Mp_e / 32 bytes)
  int N, E;
  int src_slot, q_slot, s_slot;
  int replay_only;      // 0 always, 1 only if the layer replays, 2 only if it saves
  const int32_t* gather;  // non-null: source row r is src[gather[r] / K] (src = x [T, N])
  int K;
};

// Arguments of the device planner (one layer).
struct PlanArgs {
  int32_t layer, max_layers, training, es, D, F;
  int64_t budget;
  uint64_t arena;           // device base of the arena (0 when none)
  uint64_t scratch_h1;      // scratch regions used when state is not saved
  int32_t mx;               // MXFP8 layer: state = x/h2 column bundles + h1
  int32_t pad0;
  uint64_t scratch_aux[4];  // x bundle codes/exponents, h2 bundle codes/exponents
  uint64_t zero;            // words [zero, zero + 4 zero_n) set to 0 first (0: none)
  int32_t zero_n;
  int32_t pad1;
};

// ------------------------------------------------------------ device utils
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(uint32_t(h) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair, round to nearest even (one
// v_cvt_pk_bf16_f32 on gfx950).  Every bf16 value the library stores goes
// through this one conversion, so recomputed values match bit for bit.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return uint16_t(pack_bf16x2(f, 0.0f)); }

__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// SiLU(z) = z / (1 + e^-z); one definition for forward and backward replays.
__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + __expf(-z)); }

// Workgroup barrier for LDS hand-offs.  The fences cover LDS only, so the
// barrier waits for this wave's LDS operations but not for its outstanding
// global loads or stores: prefetched tiles stay in flight across it (a full
// __syncthreads() drains every outstanding global access on gfx9).
// FUSED combine: four consecutive fp32 outputs of one route, scaled by its
// score, added into the token's fp32 row with hardware float atomics (the
// summation order across routes is not fixed).
__device__ __forceinline__ void fused_add4(float* y, float s, float a, float b, float c, float d) {
  unsafeAtomicAdd(y + 0, s * a);
  unsafeAtomicAdd(y + 1, s * b);
  unsafeAtomicAdd(y + 2, s * c);
  unsafeAtomicAdd(y + 3, s * d);
}

// A device address held in memory (the layer record) as a pointer the
// compiler knows to be global: accesses through it become global rather than
// flat instructions, and flat ones also count against the LDS wait counter,
// which would make every LDS wait drain the outstanding prefetches.
template <typename T>
__device__ __forceinline__ T* global_ptr(uint64_t addr) {
  return (T*)(T __attribute__((address_space(1)))*)(addr);
}

// s_waitcnt immediate that waits for every outstanding vector memory
// operation of the wave (vmcnt 0; expcnt and lgkmcnt left at their maxima).
constexpr int kWaitVmcnt0 = 0x0F70;

// A 32-bit value in the constant address space: read-only for the whole
// kernel, so a wave-uniform load from it is a scalar (s_load) load, counted
// in lgkmcnt rather than vmcnt.
typedef const __attribute__((address_space(4))) int kconst_i32;

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Barrier of the direct-load pipelines (k_wgrad_hot, k_mx_wgrad_hot): this
// wave's LDS reads and writes have completed (lgkmcnt 0) and every wave
// has arrived.  A workgroup-scope LDS fence would also wait for all of the
// wave's direct global-to-LDS loads (they count in vmcnt), draining the
// stages in flight; the wavefront-scope fences only keep the compiler from
// moving memory accesses across the barrier.  The loads' completion is
// waited for with explicit vmcnt counts before it.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Direct global-to-LDS loads (global_load_lds_dwordx4 / _dword): lane l's
// 16 (4) bytes at g land at LDS byte address lds + 16 l (4 l), lds
// wave-uniform, in M0.  Issued from inline assembly with no output
// registers: the compiler, which does not follow across a loop which stage
// buffer such a load writes, then adds no waits of its own before the LDS
// reads of other stages (it drained every load in flight at one step in
// four).  Every wait for these loads is explicit: a vmcnt count, then a
// barrier.  The s_nop is the wait state that an M0 write needs before an
// LDS DMA.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(g), "{m0}"(lds) : "memory");
}

// Storage element traits: float (F32 plans) or bf16 bits (BF16 / MXFP8 plans).
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
  static __device__ __forceinline__ float round(float v) { return v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float to_f(uint16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ uint16_t from_f(float v) { return f32_to_bf16(v); }
  static __device__ __forceinline__ float round(float v) { return round_bf16(v); }
};

// Clamped SwiGLU (limit L; L = +inf is the plain SwiGLU): the gate is
// clamped from above and the up projection to [-L, L] before SiLU(g) * u.
// Written as comparisons, so a NaN passes through unchanged.
__device__ __forceinline__ float clamp_gate(float g, float L) { return g > L ? L : g; }
__device__ __forceinline__ float clamp_up(float u, float L) {
  return u > L ? L : (u < -L ? -L : u);
}

// Weight-gradient copy-out: four fp32 results v added to the four dW values
// at p (in-place accumulation: one rounding of old + v to the dW type).
__device__ __forceinline__ void acc_store4(float* p, const float* v) {
  typedef float f32x4_ __attribute__((ext_vector_type(4)));
  f32x4_ o = *reinterpret_cast<const f32x4_*>(p);
  o[0] += v[0];
  o[1] += v[1];
  o[2] += v[2];
  o[3] += v[3];
  __builtin_nontemporal_store(o, reinterpret_cast<f32x4_*>(p));
}
__device__ __forceinline__ void acc_store4(uint16_t* p, const float* v) {
  typedef unsigned int u32x2_ __attribute__((ext_vector_type(2)));
  u32x2_ o = *reinterpret_cast<const u32x2_*>(p);
  const float a = __uint_as_float(o[0] << 16) + v[0];
  const float b = __uint_as_float(o[0] & 0xffff0000u) + v[1];
  const float c = __uint_as_float(o[1] << 16) + v[2];
  const float d = __uint_as_float(o[1] & 0xffff0000u) + v[3];
  o[0] = pack_bf16x2(a, b);
  o[1] = pack_bf16x2(c, d);
  __builtin_nontemporal_store(o, reinterpret_cast<u32x2_*>(p));
}

// Weight-gradient tile of item i of one expert (NA column tiles x NB row
// bands of dW; the kernels pass hot only for dW13).  The items an XCD runs at once are consecutive, so their
// order decides how much operand data they share.  An expert with many rows
// (hot: its operand rows do not stay in L2 between passes over its tiles)
// takes blocks of 4 column tiles x 8 row bands: 32 concurrent items read 4
// column strips of A and 8 row bands of B instead of every column strip of
// A for one band.  Other experts keep the order that writes dW fastest: the
// row band fastest (band_fast, dW2) or the column tile fastest (dW13).
constexpr int kWgBlockA = 4, kWgBlockB = 8;
__device__ __forceinline__ void wgrad_tile(int i, int NA, int NB, bool hot, bool band_fast,
                                           int& ta, int& tb) {
  if (hot && NA % kWgBlockA == 0 && NB % kWgBlockB == 0) {
    const int blk = i / (kWgBlockA * kWgBlockB), wi = i % (kWgBlockA * kWgBlockB);
    const int nA = NA / kWgBlockA;
    ta = (blk % nA) * kWgBlockA + wi % kWgBlockA;
    tb = (blk / nA) * kWgBlockB + wi / kWgBlockA;
  } else if (band_fast) {
    tb = i % NB;
    ta = i / NB;
  } else {
    ta = i % NA;
    tb = i / NA;
  }
}

// Number of XCDs of the MI355X; workgroups are dispatched round-robin over them.
constexpr int kXcds = 8;

// The XCD (accelerator complex die) this workgroup runs on, read from the
// hardware register XCC_ID (bits [3:0]) rather than assumed from blockIdx.
__device__ __forceinline__ int hw_xcd() {
  constexpr int kXccIdReg = 20;   // HW_REG_XCC_ID
  const unsigned v = __builtin_amdgcn_s_getreg(kXccIdReg | (0 << 6) | ((4 - 1) << 11));
  return int(v % kXcds);
}

// Per-XCD work queue of a persistent GEMM launch (RouteHdr::wq): the
// workgroups of an XCD take that XCD's items in order, each the next free one
// when it is ready, so items that share a weight tile (the m-tiles of one
// expert and n-tile) run side by side even when item costs differ.  Called by
// one thread of the workgroup.
__device__ __forceinline__ int wq_take(const RouteHdr* hdr, int xcd) {
  return int(atomicAdd(const_cast<uint32_t*>(&hdr->wq[xcd]), 1u));
}
// A workgroup that found its XCD's queue empty: the last of the XCD's `per`
// workgroups re-arms the queue for the next launch.
__device__ __forceinline__ void wq_finish(const RouteHdr* hdr, int xcd, int per) {
  uint32_t* wq = const_cast<uint32_t*>(hdr->wq);
  if (atomicAdd(&wq[kXcds + xcd], 1u) == uint32_t(per - 1)) {
    atomicExch(&wq[xcd], 0u);
    atomicExch(&wq[kXcds + xcd], 0u);
  }
}

// Expert of grouped-GEMM work item w: the largest e with mtoff[e] * NT <= w
// (mtoff = the m-tile prefix, NT = n-tiles per expert).  A workgroup's items
// only move forward, so from the expert of its previous item (e_prev >= 0) a
// few steps forward usually find it; the first item (e_prev < 0), or one far
// ahead, takes a binary search.  Each step is a dependent load, so this keeps
// the chain of latencies before an item's first weight loads short.
__device__ inline int item_expert(const int32_t* __restrict__ mtoff, int E, int NT, int w,
                                  int e_prev) {
  int lo = 0;
  if (e_prev >= 0) {
    lo = e_prev;
#pragma unroll 1
    for (int k = 0; k < 4; ++k) {
      if (mtoff[lo + 1] * NT > w) return lo;
      ++lo;
    }
  }
  int hi = E;  // invariant: mtoff[lo] * NT <= w < mtoff[hi] * NT
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (mtoff[mid] * NT <= w)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// Work split over the XCDs.  Units run expert-major, per_e per expert; a
// unit of expert e costs (pre[e + 1] - pre[e]) + cw, and the XCDs receive
// runs of units of equal total cost, so one hot expert does not load a
// single XCD.  Returns the first unit of XCD x; x = kXcds gives the unit
// count.
//  * WGRAD: a unit is an output tile; pre = the 64-row stage prefix, cw = 1
//    for storing the tile (experts with no rows still store zeros).
//  * FPROP/DGRAD: a unit is a weight column (an n-tile of an expert with all
//    its m-tiles, which run side by side and share that weight tile in L2);
//    pre = the 64-row stage prefix, cw = 0.  Measured on a Zipf(1.2) load,
//    a column of a hot expert costs about its token rows: adding a per-column
//    weight cost only made the XCDs holding hot experts finish later.
__device__ inline int xcd_first_unit(const int32_t* __restrict__ pre, int cw, int E, int per_e,
                                     int x) {
  auto prefix = [&](int e) { return int64_t(pre[e]) + int64_t(cw) * e; };
  const int64_t W = int64_t(per_e) * prefix(E);
  const int64_t T = W * x / kXcds;
  int lo = 0, hi = E;  // the largest e with per_e * prefix(e) <= T
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (int64_t(per_e) * prefix(mid) <= T)
      lo = mid;
    else
      hi = mid - 1;
  }
  if (lo >= E) return E * per_e;
  const int64_t P = int64_t(per_e) * prefix(lo);
  // lo < E is the largest such e, so expert lo's units cost c >= 1 each
  const int64_t c = prefix(lo + 1) - prefix(lo);
  const int64_t i = (T - P + c - 1) / c;
  return int(min(int64_t(lo) * per_e + i, int64_t(E) * per_e));
}
__device__ inline int xcd_first_item(const int32_t* __restrict__ mtoff, int E, int per_e, int x) {
  return xcd_first_unit(mtoff, 1, E, per_e, x);
}
// First FPROP/DGRAD work item of XCD x: items run expert-major, then n-tile,
// then m-tile (gtoff = the m-tile prefix, stoff = the 64-row stage prefix);
// a weight column never straddles two XCDs.
__device__ inline int xcd_first_tile(const int32_t* __restrict__ gtoff,
                                     const int32_t* __restrict__ stoff, int E, int NT, int x) {
  const int c = xcd_first_unit(stoff, 0, E, NT, x);
  const int e = c / NT;
  if (e >= E) return gtoff[E] * NT;
  return gtoff[e] * NT + (c - e * NT) * (gtoff[e + 1] - gtoff[e]);
}

}  // namespace moe
