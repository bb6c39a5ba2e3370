// Grouped backward GEMMs of the expert FFN on gfx950 MFMA (bf16 operands,
// fp32 accumulation).
//
// For one grouped linear C_e = A_e B_e^T the input gradient is the grouped
// GEMM dA_e = dC_e B_e and the weight gradient dB_e = dC_e^T A_e, a sum over
// the expert's token rows ("Mixture of Experts: How Routing Becomes GPU
// Computation", section 2, grouped GEMM backward).  SwiGLU backward (same
// section): with s = sigmoid(g), dG = dH2 * u * s (1 + g (1 - s)) and
// dU = dH2 * SiLU(g).  Dist-MoE explainer section 05: W2 DGRAD produces the
// h2 gradient, W2 WGRAD consumes h2 rebuilt from h1, SwiGLU backward then
// gives the h1 gradient for W13 DGRAD/WGRAD; weight gradients accumulate in
// fp32 and are stored BF16 or FP32; experts with no rows get zero gradients.
//
//   k_gemm_dgrad<0>: dH2 = dH3_e W2_e (contraction over D), SwiGLU backward
//                    epilogue -> dH1 = [dG | dU] (bf16); also writes
//                    h2 = SiLU(g) * u rebuilt from h1 (the forward formula) for
//                    the W2 weight gradient.
//   k_gemm_dgrad<1>: dXr = dH1_e W13_e (contraction over 2F) -> fp32 rows,
//                    each stored at its route slot t*K + k.
//   k_gemm_wgrad:    dW_e[b][a] = sum over the expert's rows m of
//                    B[m][b] A[m][a]: dW2 = dH3^T H2 (a = F, b = D) and
//                    dW13 = dH1^T X (a = D, b = 2F).
//
// MI355X design
//  * Every global load is coalesced: consecutive lanes read whole 128- to
//    512-byte row segments.  Operands whose rows run along the contraction
//    (DGRAD weights, both WGRAD operands) are stored into LDS as they lie in
//    memory (16-byte stores, chunks XOR-swizzled per row) and read in MFMA
//    operand layout with the gfx950 transpose read ds_read_b64_tr_b16: no
//    register transpose.
//  * DGRAD: eight waves, 256 output columns x up to 128 token rows per
//    workgroup (128-row tiles for experts with more than 64 rows), 64
//    contraction values per stage, two more stages in flight in registers.
//    256 columns make the weight reads 512-byte row segments, which HBM
//    serves faster than 256-byte ones.
//  * WGRAD: eight waves, 128 dW rows x 256 dW columns of one expert per
//    work item, 64 token rows per stage; the next item's first stage is
//    loaded while the current tile is staged through LDS and stored as whole
//    512-byte (bf16) or 1 KB (fp32) row segments, the write shape HBM takes
//    fastest.  Items run expert-major.  dW13 (14 KB rows at D = 7,168) takes
//    them with the output column tile fastest, so the workgroups of one XCD
//    write long contiguous runs of dW rows; dW2, whose rows have a
//    power-of-two byte pitch at F = 1,024 ... 4,096, takes them with the
//    128-row band fastest, so the concurrent workgroups write one column
//    segment of many bands: at F = 2,048 that wrote 5.9 instead of 5.1 TB/s
//    (column-fastest reached 5.75 TB/s only at the 6 KB pitch of F = 3,072).
//    In dW13 an expert with 256 or more rows, whose operand rows do not
//    stay in L2 between passes over its tiles, takes blocks of 4 column
//    tiles x 8 row bands instead (wgrad_tile), so the items an XCD runs at
//    once share operand rows: at Zipf(1.2) the launch read 0.72 instead of
//    2.75 GB, in the same time.  (dW2 keeps its order: blocks there read
//    0.45 instead of 0.82 GB but wrote 3% slower.)
//  * Persistent, XCD-aware grids as in the forward kernels.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

__device__ __forceinline__ void mfma_bf16(f32x16& acc, u32x4 a, u32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

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

__device__ __forceinline__ void load4_bf16(const uint16_t* p, float* f) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(p);
  f[0] = __uint_as_float(v[0] << 16);
  f[1] = __uint_as_float(v[0] & 0xffff0000u);
  f[2] = __uint_as_float(v[1] << 16);
  f[3] = __uint_as_float(v[1] & 0xffff0000u);
}

// Row tile (contraction contiguous): 128-byte rows, 16-byte chunks swizzled.
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ ((r ^ (r >> 3)) & 7)) << 4); }

// ------------------------------------------------------------------ DGRAD
// Weight stage (contraction rows k, 512-byte rows of 256 output columns): the
// 16-byte chunks of row k are XOR-swizzled by 4 (k & 3), so both the
// row-wise 16-byte stores and the transpose reads (8 rows x 4 chunks per
// instruction) spread evenly over the banks.
__device__ __forceinline__ int wsw(int k, int c) { return k * 512 + ((c ^ ((k & 3) << 2)) << 4); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
// ds_read_b64_tr_b16: in each 16-lane group, lane 4j + q addresses row j,
// columns 4q..4q+3 of a 4 x 16 bf16 block; lane i receives column i, rows
// 0..3 (elements 0..3).
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) char*)p));
  return __builtin_bit_cast(u32x2, v);
}

// Eight waves: 256 output columns (32 per wave) x up to 128 token rows.  A
// 256-column tile reads 512-byte weight row segments, which HBM serves
// faster than 256-byte ones, and shares each token stage among eight waves.
constexpr int kDgW = 64 * 512;       // weight stage: 64 contraction rows x 256 columns
constexpr int kDgT = kBMX * 128;     // token stage: up to 128 rows x 64 values
constexpr int kDgStage = kDgW + kDgT;
constexpr int kDgLds = 2 * kDgStage;

// One DGRAD work item: output columns nt * 256 .. + 255 of m-tile mt of
// expert e (mt_e m-tiles).  `between` runs when the contraction is done,
// before the epilogue (a launch takes its next item there).
template <int KIND, typename Between>
__device__ __forceinline__ void dgrad_item(const BwdArgs& a, char* lds, int tid, int e, int nt,
                                           int mt, int mt_e, Between&& between) {
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int c32 = tid & 31;   // weight loader: 16-byte chunk of a 512-byte row segment
  const int kp = tid >> 5;    // weight loader: contraction rows kp + 16 i
  const int lc = tid & 7;     // token loader: 16-byte chunk of a 128-byte row segment
  const int lrow = tid >> 3;  // token loader: tile row (+ 64 j)
  // transpose reads of the weight operand: the 16-lane group (lane >> 4)
  // covers output columns 32 wave + 16 ((lane >> 4) & 1) .. + 15 and
  // contraction rows 8 lh .. 8 lh + 7 of each 16-row MFMA step
  const int tr_row = 8 * lh + ((lane & 15) >> 2);
  const int tr_chunk = 4 * wave + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_byte = 8 * (lane & 1);

  const int S = a.Kd / 64;
  const int64_t N = a.N;
  const uint16_t* h1 = global_ptr<const uint16_t>(a.hdr->rec.h1);
  const int bm = gemm_tile_rows(a.offsets[e + 1] - a.offsets[e]);
  const int row0 = a.offsets[e] + mt * bm;
  const int rows = min(bm, a.offsets[e + 1] - row0);
  // The last tile of an N that is an odd multiple of 128 has 128 columns:
  // the loads of its upper half re-read the lower half, and waves 4..7
  // multiply them but store nothing.  Every load stays unconditional, so
  // the stage loop has no branches.
  const int ncols = min(256, int(N) - nt * 256);
  const int wcol = c32 * 8 < ncols ? c32 * 8 : c32 * 8 - 128;
  const uint16_t* wsrc = reinterpret_cast<const uint16_t*>(a.W) +
                         (int64_t(e) * a.Kd + kp) * N + nt * 256 + wcol;
  // Tile rows past the expert's last row re-read that row (outputs not stored).
  const char* tsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    tsrc[j] = reinterpret_cast<const char*>(a.tok) +
              int64_t(row0 + min(lrow + 64 * j, rows - 1)) * a.Kd * 2 + lc * 16;

  f32x16 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x16{};
  u32x4 R0[6], R1[6];
  // NB: 32-token blocks multiplied (1, 2 or 4; one loop copy each, so no
  // accumulator depends on a branch inside the stage loop); the token stage
  // holds 64 rows per pass of the 512 threads (rows past the tile repeat its
  // last row).
  // W2 rows (the contraction of the W2 DGRAD) are F values apart, a
  // power-of-two byte pitch at the usual widths, and the n-tiles of one
  // expert run side by side: each starts its contraction at its own
  // offset, nt * S / NT stages, so at any moment they read different row
  // bands instead of the same one (the sum's order is fixed per item).
  const int rot = KIND == 0 ? int(int64_t(nt) * S / a.NT) : 0;
  auto load = [&](u32x4* R, int s, auto nb_c, auto tm_c) {
    constexpr int NB = decltype(nb_c)::value;
    constexpr bool TM = decltype(tm_c)::value;
    s += rot;
    if (s >= S) s -= S;
    const uint16_t* p = wsrc + int64_t(s) * 64 * N;
    // weights stream through once: non-temporal loads keep them from
    // evicting the token tiles the other n-tiles of this expert re-read
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4* src = reinterpret_cast<const u32x4*>(p + 16 * i * N);
      if constexpr (TM)
        R[i] = *src;
      else
        R[i] = __builtin_nontemporal_load(src);
    }
#pragma unroll
    for (int j = 0; j < (NB + 3) / 4 + (NB == 4); ++j)
      R[4 + j] = *reinterpret_cast<const u32x4*>(tsrc[j] + int64_t(s) * 128);
  };
  auto store = [&](const u32x4* R, int buf, auto nb_c) {
    constexpr int NB = decltype(nb_c)::value;
    char* la = lds + buf * kDgStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(la + wsw(kp + 16 * i, c32)) = R[i];
    char* lt = la + kDgW;
#pragma unroll
    for (int j = 0; j < (NB + 3) / 4 + (NB == 4); ++j)
      *reinterpret_cast<u32x4*>(lt + swz(lrow + 64 * j, lc)) = R[4 + j];
  };
  auto compute = [&](int buf, auto nb_c) {
    constexpr int NB = decltype(nb_c)::value;
    const char* la = lds + buf * kDgStage;
    const char* lt = la + kDgW;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int g = 2 * q + lh;
      const u32x2 lo = lds_read_tr16(la + wsw(16 * q + tr_row, tr_chunk) + tr_byte);
      const u32x2 hi = lds_read_tr16(la + wsw(16 * q + tr_row + 4, tr_chunk) + tr_byte);
      const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
      u32x4 bv[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) bv[b] = *reinterpret_cast<const u32x4*>(lt + swz(32 * b + lr, g));
#pragma unroll
      for (int b = 0; b < NB; ++b) mfma_bf16(acc[b], av, bv[b]);
    }
  };
  // Pipeline as in the forward kernels: LDS buffer 0 holds stage s, R1
  // stage s + 1 and R0 stage s + 2 (indices past the end repeat the last).
  auto run = [&](auto nb_c, auto tm_c) {
    load(R0, 0, nb_c, tm_c);
    load(R1, min(1, S - 1), nb_c, tm_c);
    store(R0, 0, nb_c);
    load(R0, min(2, S - 1), nb_c, tm_c);
    lds_barrier();
    for (int s = 0; s + 1 < S; s += 2) {
      compute(0, nb_c);
      store(R1, 1, nb_c);
      load(R1, min(s + 3, S - 1), nb_c, tm_c);
      lds_barrier();
      compute(1, nb_c);
      store(R0, 0, nb_c);
      load(R0, min(s + 4, S - 1), nb_c, tm_c);
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
  between();

  // acc[b][v]: output column 32*wave + 8*(v/4) + 4*lh + v%4, token 32*b + lr
  const int col = nt * 256 + 32 * wave + 4 * lh;
#pragma unroll
  for (int b = 0; b < 4 && 32 * wave < ncols; ++b) {
    const int m = 32 * b + lr;
    if (m >= rows) continue;
    const int64_t row = row0 + m;
    if (KIND == 0) {
      const int F = a.F;
      uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + row * (2 * F);
      uint16_t* h2o = reinterpret_cast<uint16_t*>(a.out2);
      const uint16_t* hr = h1 + row * (2 * F);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int j = col + 8 * g4;
        float gv[4], uv[4], dg[4], du[4], hv[4];
        load4_bf16(hr + j, gv);
        load4_bf16(hr + F + j, uv);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float dh2 = acc[b][4 * g4 + i];
          // clamped SwiGLU backward: no gradient through a clamped value
          const float L = a.limit;
          const float gc = clamp_gate(gv[i], L), uc = clamp_up(uv[i], L);
          const float sg = sigmoid_f(gc);
          const float sl = silu_f(gc);
          dg[i] = gv[i] > L ? 0.0f : dh2 * uc * (sg * (1.0f + gc * (1.0f - sg)));
          du[i] = (uv[i] > L || uv[i] < -L) ? 0.0f : dh2 * sl;
          hv[i] = sl * uc;
        }
        store4<uint16_t>(o + j, dg[0], dg[1], dg[2], dg[3]);
        store4<uint16_t>(o + F + j, du[0], du[1], du[2], du[3]);
        if (h2o) store4<uint16_t>(h2o + row * F + j, hv[0], hv[1], hv[2], hv[3]);
      }
    } else {
      // dXr rows go to their route slots, so the input-gradient sum reads
      // each token's K rows as one contiguous run
      float* o = reinterpret_cast<float*>(a.out) + int64_t(a.row_slot[row]) * N;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        store4<float>(o + col + 8 * g4, acc[b][4 * g4], acc[b][4 * g4 + 1], acc[b][4 * g4 + 2],
                      acc[b][4 * g4 + 3]);
    }
  }
}

template <int KIND>
__global__ __launch_bounds__(512, 1) void k_gemm_dgrad(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kDgLds];
  const int tid = threadIdx.x;
  const RouteHdr* hdr = a.hdr;
  const int xcd = blockIdx.x % kXcds;
  const int per = gridDim.x / kXcds;
  // a.mtoff is the m-tile prefix (128-row tiles for experts with more than
  // 64 rows); the XCDs split the items by token rows
  const int first = xcd_first_tile(a.mtoff, a.stoff, a.E, a.NT, xcd);
  const int last = xcd_first_tile(a.mtoff, a.stoff, a.E, a.NT, xcd + 1);

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
    const int e = item_expert(a.mtoff, a.E, a.NT, w, e_prev);
    e_prev = e;
    const int mt_e = a.mtoff[e + 1] - a.mtoff[e];
    const int u = w - a.mtoff[e] * a.NT;
    const int nt = u / mt_e;
    dgrad_item<KIND>(a, lds, tid, e, nt, u - nt * mt_e, mt_e, [&] {
      // the next item, taken while this one's epilogue runs (every thread
      // read s_next before this item's stage barriers)
      if (dyn && tid == 0) s_next = wq_take(hdr, xcd);
    });
    if (dyn) {
      lds_barrier();
      w = first + s_next;
    } else {
      w += per;
    }
  }
  if (dyn && tid == 0) wq_finish(hdr, xcd, per);
}

// ------------------------------------------------------------------ WGRAD
// TAG only separates the two launches in profiles (2: dW2, 13: dW13).
// Work item: 128 dW rows x 256 dW columns of one expert on eight waves,
// written as 512-byte (bf16) or 1 KB (fp32) row segments, which HBM takes
// faster than 256-byte ones; per token row the item re-reads less operand
// data than a 128 x 128 or 64 x 256 tile.  Wave w owns dW rows
// 64 (w >> 2) .. + 63 and columns 64 (w & 3) .. + 63 of the tile: 2 x 2
// accumulators of 32 x 32.  Both operand stages hold 64 token rows as they
// lie in memory (A: 256 columns, 512-byte rows; B: 128 columns, 256-byte
// rows; chunks XOR-swizzled by 4 (m & 3)) and are read with transpose reads.
__device__ __forceinline__ int bsw(int m, int c) { return m * 256 + ((c ^ ((m & 3) << 2)) << 4); }

constexpr int kWgLds = 64 * 512 + 64 * 256;   // A and B operand stages

// The WGRAD items w0, w0 + step, ... below w1 (expert-major, NA x NB tiles
// per expert), each tile's first stage loaded while the previous tile is
// stored.  With a.hot_wg the experts of kHotWgRows rows or more are skipped
// (k_wgrad_hot's).  lds: kWgLds bytes.
// ACC: in-place accumulation (dW += result): the tile is staged in fp32 and
// each copied-out value is added to the dW value it replaces, rounded once.
template <typename TW, int TAG, int ACC>
__device__ __forceinline__ void wgrad_run(const BwdArgs& a, char* lds, int tid, int w0, int w1,
                                          int step) {
  typedef typename std::conditional<ACC != 0, float, TW>::type TS;   // staging type
  constexpr int kA = 64 * 512;                         // A stage: 64 token rows x 256 columns
  constexpr int kB = 64 * 256;                         // B stage: 64 token rows x 128 columns
  constexpr int kRowB = 256 * int(sizeof(TS)) + 16;    // padded output-staging row
  constexpr int kRowsPerPass = sizeof(TS) == 4 ? 32 : 64;
  constexpr int kPasses = 128 / kRowsPerPass;
  static_assert(kRowsPerPass * kRowB <= kA + kB, "output staging reuses the operand stages");
  static_assert(kA + kB == kWgLds, "operand stages");
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wa = wave & 3;    // 64-column block of the tile
  const int wb = wave >> 2;   // 64-row block of the tile
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int c32 = tid & 31;   // A loader: 16-byte chunk of a 512-byte row segment
  const int ar = tid >> 5;    // A loader: token rows ar + 16 i
  const int c16 = tid & 15;   // B loader: 16-byte chunk of a 256-byte row segment
  const int br = tid >> 4;    // B loader: token rows br + 32 j
  // transpose reads: lane 4j + q of each 16-lane group addresses row j,
  // columns 4q .. 4q + 3 of its group's 16 columns (16 (lane >> 4 & 1) on)
  const int tr_row = 8 * lh + ((lane & 15) >> 2);
  const int tr_c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_byte = 8 * (lane & 1);

  const int a_ld = a.a_ld, b_ld = a.b_ld;
  const int NA = (a_ld + 255) / 256, NB = b_ld / 128;
  const int per_e = NA * NB;
  const int last = w1, per = step;
  const uint16_t* asrc = reinterpret_cast<const uint16_t*>(a.arows);
  const uint16_t* bsrc = reinterpret_cast<const uint16_t*>(a.grad);

  struct Item {
    int e, ta, tb, r0, Me, S, ncols;
  };
  // Work items of this workgroup: w = w0 + i * per below last.
  int wcur = w0;
  auto fill = [&](Item& t) {
    int e = 0, o0 = 0, o1 = 0;
    for (;;) {   // with hot_wg, step over the hot experts' items
      if (wcur >= last) {
        t.e = -1;
        return;
      }
      e = wcur / per_e;
      // scalar loads (constant address space): no wait behind the previous
      // tile's dW stores
      o0 = ((kconst_i32*)a.offsets)[e];
      o1 = ((kconst_i32*)a.offsets)[e + 1];
      if (!a.hot_wg || !hot_wgrad_expert(o1 - o0)) break;
      wcur += ((e + 1) * per_e - wcur + per - 1) / per * per;
    }
    const int w = wcur;
    wcur += per;
    t.e = e;
    t.r0 = o0;
    t.Me = o1 - o0;
    t.S = (t.Me + 63) / 64;
    int ta, tb;
    wgrad_tile(w - e * per_e, NA, NB, TAG == 13 && hot_expert(t.Me), TAG == 2, ta, tb);
    t.ta = ta;
    t.tb = tb;
    t.ncols = min(256, a_ld - ta * 256);
  };

  // One stage in registers.  Token rows past the expert's last row are not
  // read: their registers hold zeros, so they add nothing.  Columns past the
  // end of a 128-column half tile re-read the first half.
  u32x4 RA[4], RB[2];
  auto load = [&](const Item& t, int s) {
    const int acol = t.ta * 256 + (c32 * 8 < t.ncols ? c32 * 8 : c32 * 8 - 128);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = s * 64 + ar + 16 * i;
      RA[i] = u32x4{0u, 0u, 0u, 0u};
      if (m < t.Me) RA[i] = *reinterpret_cast<const u32x4*>(asrc + int64_t(t.r0 + m) * a_ld + acol);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = s * 64 + br + 32 * j;
      RB[j] = u32x4{0u, 0u, 0u, 0u};
      if (m < t.Me)
        RB[j] = *reinterpret_cast<const u32x4*>(bsrc + int64_t(t.r0 + m) * b_ld + t.tb * 128 +
                                                c16 * 8);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(lds + wsw(ar + 16 * i, c32)) = RA[i];
#pragma unroll
    for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4*>(lds + kA + bsw(br + 32 * j, c16)) = RB[j];
  };

  Item cur, nxt;
  fill(cur);
  if (cur.e >= 0 && cur.S > 0) load(cur, 0);
  while (cur.e >= 0) {
    fill(nxt);
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i >> 1][i & 1] = f32x16{};
    for (int s = 0; s < cur.S; ++s) {
      store();
      lds_barrier();
      if (s + 1 < cur.S)
        load(cur, s + 1);
      else if (nxt.e >= 0 && nxt.S > 0)
        load(nxt, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 av[2], bv[2];
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
          const int ch = 8 * wa + 4 * aa + tr_c;
          const u32x2 lo = lds_read_tr16(lds + wsw(16 * q + tr_row, ch) + tr_byte);
          const u32x2 hi = lds_read_tr16(lds + wsw(16 * q + tr_row + 4, ch) + tr_byte);
          av[aa] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const int ch = 8 * wb + 4 * bb + tr_c;
          const u32x2 lo = lds_read_tr16(lds + kA + bsw(16 * q + tr_row, ch) + tr_byte);
          const u32x2 hi = lds_read_tr16(lds + kA + bsw(16 * q + tr_row + 4, ch) + tr_byte);
          bv[bb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int aa = 0; aa < 2; ++aa) mfma_bf16(acc[bb][aa], av[aa], bv[bb]);
      }
      lds_barrier();
    }
    if (cur.S == 0 && nxt.e >= 0 && nxt.S > 0) load(nxt, 0);

    // acc[bb][aa][v] = dW[b = tb*128 + 64*wb + 32*bb + lr]
    //                    [a = ta*256 + 64*wa + 32*aa + 8*(v/4) + 4*lh + v%4],
    // staged through LDS (over the operand stages) in passes of
    // kRowsPerPass rows and stored as whole row segments.
    TW* o = reinterpret_cast<TW*>(a.out) + (int64_t(cur.e) * b_ld + int64_t(cur.tb) * 128) * a_ld +
            cur.ta * 256;
#pragma unroll
    for (int h = 0; h < kPasses; ++h) {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int r = 64 * wb + 32 * bb;   // first tile row of this accumulator pair
        if (r / kRowsPerPass != h) continue;
        const int rl = r + lr - h * kRowsPerPass;
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
          TS* rowp = reinterpret_cast<TS*>(lds + rl * kRowB) + 64 * wa + 32 * aa + 4 * lh;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            store4<TS>(rowp + 8 * g4, acc[bb][aa][4 * g4], acc[bb][aa][4 * g4 + 1],
                       acc[bb][aa][4 * g4 + 2], acc[bb][aa][4 * g4 + 3]);
        }
      }
      lds_barrier();
      constexpr int kChunksPerRow = 256 * int(sizeof(TS)) / 16;
      constexpr int kChunks = kRowsPerPass * kChunksPerRow;
      const int live = cur.ncols * int(sizeof(TS)) / 16;   // chunks of a row inside dW
#pragma unroll
      for (int j = 0; j < kChunks / 512; ++j) {
        const int i = tid + 512 * j;
        const int rl = i / kChunksPerRow, cc = i % kChunksPerRow;
        if (cc < live) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(lds + rl * kRowB + cc * 16);
          if (ACC) {   // four fp32 results onto the four dW values they update
            float f[4] = {__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                          __uint_as_float(v[3])};
            acc_store4(o + int64_t(rl + h * kRowsPerPass) * a_ld + cc * 4, f);
          } else {
            char* dst = reinterpret_cast<char*>(o + int64_t(rl + h * kRowsPerPass) * a_ld) + cc * 16;
            // dW is written once and not read back here: stream it past the
            // L2 so the expert's operand rows stay cached for the other tiles.
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
          }
        }
      }
      lds_barrier();
    }
    cur = nxt;
  }
}

template <typename TW, int TAG, int ACC>
__global__ __launch_bounds__(512, 1) void k_gemm_wgrad(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kWgLds];
  const int per_e = ((a.a_ld + 255) / 256) * (a.b_ld / 128);
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int per = gridDim.x / kXcds;
  // with hot_wg the experts of kHotWgRows rows or more are k_wgrad_hot's:
  // split by the other experts' stages (theirs count 0, plus 1 per item)
  const int32_t* cost = a.hot_wg ? a.cst : a.mtoff;
  const int first = xcd_first_item(cost, a.E, per_e, xcd);
  const int last = xcd_first_item(cost, a.E, per_e, xcd + 1);
  wgrad_run<TW, TAG, ACC>(a, lds, threadIdx.x, first + slot, last, per);
}

// ------------------------------------------------------------------ WGRAD, hot experts
// An expert with at least kHotWgRows rows contracts its weight gradient over
// hundreds to thousands of token rows: MFMA-bound work ("Mixture of Experts:
// How Routing Becomes GPU Computation", section 1 arithmetic intensity), for
// which the 128 x 256 streaming tile (one stage in flight, 4 MFMAs per wave
// per 16-row step) is the wrong shape.  Here a work item is a 256 x 256 dW
// tile: eight waves, wave (wa, wb) owning dW rows 128 wb .. + 127 and
// columns 64 wa .. + 63 as 4 x 2 fp32 accumulators of
// v_mfma_f32_32x32x16_bf16 (8 MFMAs per wave per 16-row step).  A stage is
// 32 token rows of both operands (256 columns each, 512-byte rows: 32 KiB),
// moved by the gfx950 direct global-to-LDS load (global_load_lds_dwordx4: a
// wave instruction fills two 512-byte LDS rows, each lane fetching the
// global chunk that the row's XOR swizzle puts at its slot).  Four stage
// buffers keep three stages (96 KiB) in flight while the fourth multiplies
// (one 64 KiB stage in flight took 1.2 times as long on 2,048-row experts;
// a fifth buffer measured no faster).  The operands are read
// in MFMA layout with ds_read_b64_tr_b16 as in k_gemm_wgrad.  Token rows past
// the expert's end are loaded clamped and their B rows zeroed in LDS before
// the last stage multiplies, so they add nothing.  The tile is staged
// through LDS in eight passes of 32 rows while the next item's first two
// stages stream in, and written as whole 512-byte row segments,
// non-temporally.  Items: the hot experts' tiles, split over the XCDs by
// their 64-row stage counts, 4 x 8 blocks of tiles where the grid allows
// (wgrad_tile); k_gemm_wgrad skips these experts (BwdArgs::hot_wg).

template <int TAG>
__global__ __launch_bounds__(512, 1) void k_wgrad_hot(BwdArgs a) {
  constexpr int kRows = 32;          // token rows per stage
  constexpr int kOp = kRows * 512;   // one operand's stage: 32 token rows x 256 columns
  constexpr int kBuf = 2 * kOp;      // a stage buffer: A then B
  constexpr int kPitch = 512 + 16;   // output-staging row (bf16), padded
  constexpr int kNb = 4;             // stage buffers: kNb - 1 stages in flight
  static_assert((kNb & (kNb - 1)) == 0, "buffer index by mask");
  __shared__ __attribute__((aligned(1024))) char lds[kNb * kBuf];   // stage s in buffer s mod kNb
  static_assert(32 * kPitch <= kBuf, "a 32-row output pass fits one buffer");
  auto buf = [&](int s) { return lds + (s & (kNb - 1)) * kBuf; };
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wa = wave & 3;    // 64-column block of the tile
  const int wb = wave >> 2;   // 128-row block of the tile
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int tr_row = 8 * lh + ((lane & 15) >> 2);
  const int tr_c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_byte = 8 * (lane & 1);

  const int a_ld = a.a_ld, b_ld = a.b_ld;
  const int NA = a_ld / 256, NB = b_ld / 256;
  const int per_e = NA * NB;
  // hot experts' 64-row stages before expert e (routing's cold prefix counts them 0)
  auto hs = [&](int e) { return a.mtoff[e] - a.cst[e]; };
  const int E = a.E;
  if (hs(E) == 0) return;
  // XCD split: units (expert-major, per_e per expert) of equal total stage cost
  auto first_unit = [&](int x) {
    const int64_t W = int64_t(per_e) * hs(E);
    const int64_t T = W * x / kXcds;
    int lo = 0, hi = E;   // the largest e with per_e * hs(e) <= T
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (int64_t(per_e) * hs(mid) <= T)
        lo = mid;
      else
        hi = mid - 1;
    }
    if (lo >= E) return E * per_e;
    const int64_t c = hs(lo + 1) - hs(lo);   // >= 1: lo is the largest such e
    const int64_t i = (T - int64_t(per_e) * hs(lo) + c - 1) / c;
    return int(min(int64_t(lo) * per_e + i, int64_t(E) * per_e));
  };
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int per = gridDim.x / kXcds;
  const int first = first_unit(xcd), last = first_unit(xcd + 1);
  const char* asrc = reinterpret_cast<const char*>(a.arows);
  const char* bsrc = reinterpret_cast<const char*>(a.grad);
  // loader roles: waves 0-3 fill the A stage, 4-7 the B stage; wave v & 3
  // covers stage rows 8 (v & 3) .. + 7, instruction i rows 2 i, 2 i + 1 of
  // those (lanes 0-31 / 32-63), lane slot chunk lane & 31
  const bool aload = wave < 4;
  const int vq = wave & 3;
  const int ldr = 8 * vq + lh;         // stage row of instruction 0 (+ 2 i)
  const int lchunk = lane & 31;

  // this workgroup's units are w0, w0 + per, ...: the first of them, from
  // w on, that belongs to a hot expert (last: none)
  auto next_hot = [&](int w) {
    while (w < last) {
      const int e = w / per_e;
      if (hot_wgrad_expert(a.offsets[e + 1] - a.offsets[e])) return w;
      // the next hot expert (the smallest e2 > e with hot stages)
      const int h1 = hs(e + 1);
      int lo = e + 1, hi = E;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (hs(mid + 1) > h1)
          hi = mid;
        else
          lo = mid + 1;
      }
      if (lo >= E) return last;
      w += (lo * per_e - w + per - 1) / per * per;
    }
    return last;
  };
  struct Item {
    int e, ta, tb, Me, S;
    const char* gbase;   // this lane's operand (A or B) at the tile's first token row
    int64_t ld2;         // its row pitch in bytes
  };
  auto decode = [&](int w, Item& t) {
    const int e = w / per_e;
    const int r0 = a.offsets[e];
    t.e = e;
    t.Me = a.offsets[e + 1] - r0;
    t.S = (t.Me + kRows - 1) / kRows;
    wgrad_tile(w - e * per_e, NA, NB, true, false, t.ta, t.tb);
    t.gbase = aload ? asrc + (int64_t(r0) * a_ld + t.ta * 256) * 2
                    : bsrc + (int64_t(r0) * b_ld + t.tb * 256) * 2;
    t.ld2 = int64_t(aload ? a_ld : b_ld) * 2;
  };
  // stage s of item t into its buffer: four 1 KiB direct loads per wave
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(lds));   // LDS byte address
  auto issue = [&](const Item& t, int s) {
    const uint32_t dst = lds0 + (s & (kNb - 1)) * kBuf + (aload ? 0 : kOp) + 8 * vq * 512;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = ldr + 2 * i;                      // stage row
      const int m = min(kRows * s + k, t.Me - 1);     // token row, clamped
      const int gc = lchunk ^ ((k & 3) << 2);          // global chunk at this slot
      dma16(t.gbase + int64_t(m) * t.ld2 + gc * 16, __builtin_amdgcn_readfirstlane(dst + i * 1024));
    }
  };

  Item cur, nxt;
  int w = next_hot(first + slot);
  int pre = 0;   // stages of cur that the previous item issued (into buffers 0, 1)
  while (w < last) {
    decode(w, cur);
    const int S = cur.S;
    const int tail = cur.Me - kRows * (S - 1);   // live rows of the last stage
    // zero the B rows of the last stage past the expert's end (after its loads landed)
    auto zero_tail = [&](char* b) {
      char* bb = b + kOp;
      for (int i = tid; i < (kRows - tail) * 32; i += 512)
        *reinterpret_cast<u32x4*>(bb + (tail + i / 32) * 512 + (i % 32) * 16) = u32x4{0u, 0u, 0u, 0u};
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    auto compute = [&](const char* b) {
      const char* la = b;
      const char* lb = b + kOp;
#pragma unroll
      for (int q = 0; q < kRows / 16; ++q) {
        u32x4 av[2], bv[4];
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
          const int ch = 8 * wa + 4 * aa + tr_c;
          const u32x2 lo = lds_read_tr16(la + wsw(16 * q + tr_row, ch) + tr_byte);
          const u32x2 hi = lds_read_tr16(la + wsw(16 * q + tr_row + 4, ch) + tr_byte);
          av[aa] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int ch = 16 * wb + 4 * bb + tr_c;
          const u32x2 lo = lds_read_tr16(lb + wsw(16 * q + tr_row, ch) + tr_byte);
          const u32x2 hi = lds_read_tr16(lb + wsw(16 * q + tr_row + 4, ch) + tr_byte);
          bv[bb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
#pragma unroll
          for (int aa = 0; aa < 2; ++aa) mfma_bf16(acc[bb][aa], av[aa], bv[bb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // Three stages in flight.  Step s waits until this wave's loads of
    // stage s have landed (vector memory loads complete in issue order, so
    // the loads of the stages behind it may stay outstanding), then for every
    // wave (which also ends every wave's reads of stage s - 1), issues stage
    // s + 3 into the buffer that stage s - 1 used, and multiplies.  Stores
    // may complete out of order with loads, so an item that follows a tile's
    // output stores first waits for everything.
    if (pre) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    for (int st = pre; st < min(kNb - 1, S); ++st) issue(cur, st);
    for (int s = 0; s < S; ++s) {
      const int after = min(S - 1 - s, kNb - 2);   // stages in flight behind stage s
      if (after >= 3)
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 | 12);
      else if (after == 2)
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 | 8);
      else if (after == 1)
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 | 4);
      else
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      stage_barrier();
      if (s + 1 == S && tail < kRows) {
        zero_tail(buf(s));
        stage_barrier();
      }
      if (s + kNb - 1 < S) issue(cur, s + kNb - 1);
      compute(buf(s));
    }
    stage_barrier();   // every wave past its last MFMAs: all four buffers free
    // the next item's first two stages stream into buffers 0 and 1 while
    // this tile is staged out through buffers 2 and 3
    const int wn = next_hot(w + per);
    pre = 0;
    if (wn < last) {
      decode(wn, nxt);
      pre = min(kNb - 2, nxt.S);
      for (int st = 0; st < pre; ++st) issue(nxt, st);
    }

    // acc[bb][aa][v] = dW[b = tb*256 + 128 wb + 32 bb + lr]
    //                    [a = ta*256 + 64 wa + 32 aa + 8 (v/4) + 4 lh + v%4],
    // staged in eight passes of 32 rows (pass h = 4 wb + bb) through buffers
    // 2 and 3 in turn; a pass's writes only start after the pass two before
    // it was read out (every wave has passed the barrier between)
    uint16_t* o = reinterpret_cast<uint16_t*>(a.out) +
                  (int64_t(cur.e) * b_ld + int64_t(cur.tb) * 256) * a_ld + cur.ta * 256;
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      char* sb = buf(kNb - 2 + (h & 1));
      if (wb == h / 4) {
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
          uint16_t* rowp = reinterpret_cast<uint16_t*>(sb + lr * kPitch) + 64 * wa + 32 * aa + 4 * lh;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            store4<uint16_t>(rowp + 8 * g4, acc[h % 4][aa][4 * g4], acc[h % 4][aa][4 * g4 + 1],
                             acc[h % 4][aa][4 * g4 + 2], acc[h % 4][aa][4 * g4 + 3]);
        }
      }
      stage_barrier();
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {   // 32 rows x 32 chunks of 16 bytes
        const int i = tid + 512 * jj;
        const int rl = i / 32, cc = i % 32;
        const u32x4 v = *reinterpret_cast<const u32x4*>(sb + rl * kPitch + cc * 16);
        __builtin_nontemporal_store(
            v, reinterpret_cast<u32x4*>(o + int64_t(rl + 32 * h) * a_ld + cc * 8));
      }
    }
    w = wn;
  }
}

// ------------------------------------------------------------------ fused (Mega) backward
// One persistent grid runs a projection's DGRAD and WGRAD work records,
// each expert's DGRAD tile range placed next to its WGRAD range (Dist-MoE
// explainer, section 05, Mega backward).  Two launches, after the combine
// backward: W2 (dH1 with the SwiGLU backward, and dW2) and W13 (dX rows and
// dW13).
//
// Unit of work: 1 / NT of an expert, NT = its DGRAD n-tiles: the DGRAD
// records of n-tile nt (one per m-tile) and dW items nt * NB .. + NB - 1 of
// the streaming WGRAD launch's order (NB = 128-row bands of dW, NT x NB
// items per expert).  For dW2 (band fastest) those are the tiles of dW
// columns nt * 256 .. + 255, which read h2 columns nt * 256 .. + 255, which
// the W2 DGRAD records of n-tile nt rebuild from h1: the unit is the unit of
// the data dependency.  W13's records read dH1 and the x rows, complete
// before the launch, and never wait; its units take the dW13 items in the
// streaming order (column tile fastest, 4 x 8 blocks for hot experts), so
// concurrent records share operand rows in L2 as there.
//
// MI355X design, as in the fused forward: an agent-scope release/acquire
// pair (an L2 write-back and invalidate) costs more than the hand-off it
// would order, so producer and consumer of every row share one L2:
//  * each XCD owns a contiguous run of units, split by the experts' 64-row
//    stages plus kMegaBwdCw per unit for its weight reads and dW writes (a
//    hot expert's blocks spread over the XCDs), and runs their records from
//    its own ticket queue (on the XCD the workgroup runs on: hw_xcd);
//  * queue block j holds the DGRAD records of unit j, then the WGRAD
//    records of unit j - look (look = the XCD's workgroup count, so a
//    unit's DGRAD records are running or done when its WGRAD records come
//    up).  A WGRAD record is about kMegaWgStages stages of work: up to
//    kMegaWgStages dW tiles of an expert with one 64-row stage, a single
//    tile of one with kMegaWgStages or more (every tile's first stage is
//    loaded while the previous one is stored).  Each workgroup first sums
//    the records per expert into LDS;
//  * W2: a DGRAD record stores, waits until its stores are in L2 (vmcnt 0)
//    and counts itself in ready[unit]; a WGRAD record first waits (one
//    thread, atomic reads, bounded) until ready[unit] equals the unit's
//    DGRAD record count.  No workgroup on that CU read those h2 lines
//    earlier in the launch;
//  * a workgroup takes its next ticket as it starts a record, so the
//    ticket's latency hides behind the record, and starts that record after
//    finishing the current one.
// Every wait ends: the smallest unfinished ticket is either running, and
// then waits only for smaller tickets (a unit's DGRAD records come before
// its WGRAD records), all finished, or it is the next ticket of a workgroup
// whose current, smaller ticket is finished.  Tickets and counters are
// zeroed by the backward's planner launch.
constexpr int kMegaWgStages = 16;    // 64-row stages per WGRAD record (at least one tile)
constexpr int kMegaBwdCw = 3;        // XCD split: a unit's fixed cost, in 64-row stages
constexpr int kMegaBwdSpin = 1 << 22;   // polls (each followed by a short sleep)

template <int KIND, typename TW, int ACC>
__global__ __launch_bounds__(512, 1) void k_bwd_mega(BwdArgs dg, BwdArgs wg, uint32_t* tickets,
                                                     uint32_t* ready, int look) {
  constexpr int TAG = KIND == 0 ? 2 : 13;
  __shared__ __attribute__((aligned(16))) char lds[kDgLds > kWgLds ? kDgLds : kWgLds];
  __shared__ int s_t;
  __shared__ int s_wp[kMaxE + 1];   // WGRAD records per unit of the experts before e (E <= kMaxE)
  __shared__ int s_part[512];
  const int tid = threadIdx.x;
  const RouteHdr* hdr = dg.hdr;
  const int E = dg.E;
  const int32_t* gt = dg.mtoff;   // DGRAD m-tile prefix
  const int NU = dg.NT;           // units per expert: 256-column weight blocks
  const int NAw = (wg.a_ld + 255) / 256, NBw = wg.b_ld / 128;
  const int per_e = NAw * NBw;    // dW tiles per expert; NBw per unit
  // dW tiles per WGRAD record of expert e, and records per unit
  auto group = [&](int e) {
    const int S = (wg.offsets[e + 1] - wg.offsets[e] + 63) / 64;
    return S <= 1 ? kMegaWgStages : max(1, kMegaWgStages / S);
  };
  auto nrec = [&](int e) {
    const int G = group(e);
    return (NBw + G - 1) / G;
  };
  {   // s_wp: exclusive prefix of nrec over the experts (each thread a run of experts)
    const int c = (E + 511) / 512;
    const int e0 = min(E, tid * c), e1 = min(E, e0 + c);
    int sum = 0;
    for (int e = e0; e < e1; ++e) sum += nrec(e);
    s_part[tid] = sum;
    lds_barrier();
    for (int off = 1; off < 512; off <<= 1) {   // inclusive scan of the run sums
      const int v = tid >= off ? s_part[tid - off] : 0;
      lds_barrier();
      s_part[tid] += v;
      lds_barrier();
    }
    int run = s_part[tid] - sum;
    for (int e = e0; e < e1; ++e) {
      s_wp[e] = run;
      run += nrec(e);
    }
    if (tid == 511) s_wp[E] = s_part[511];
    lds_barrier();
  }

  const int xcd = hw_xcd();
  uint32_t* ticket = tickets + xcd;
  const int u_lo = xcd_first_unit(wg.mtoff, kMegaBwdCw, E, NU, xcd);
  const int u_hi = xcd_first_unit(wg.mtoff, kMegaBwdCw, E, NU, xcd + 1);
  const int nu = u_hi - u_lo;
  // DGRAD records before unit u (all m-tiles of the earlier units)
  auto dpre = [&](int u) {
    const int e = u / NU, nt = u - e * NU;
    return gt[e] * NU + (e < E ? nt * (gt[e + 1] - gt[e]) : 0);
  };
  // WGRAD records before unit u
  auto wpre = [&](int u) {
    const int e = u / NU, nt = u - e * NU;
    return s_wp[e] * NU + (e < E ? nt * (s_wp[e + 1] - s_wp[e]) : 0);
  };
  const int d0 = dpre(u_lo), w0 = wpre(u_lo);
  // records before queue block j
  auto start = [&](int j) {
    return dpre(u_lo + min(j, nu)) - d0 + wpre(u_lo + max(0, min(j - look, nu))) - w0;
  };
  const int total = dpre(u_hi) - d0 + wpre(u_hi) - w0;

  if (tid == 0) s_t = int(atomicAdd(ticket, 1u));
  lds_barrier();
  // one ticket per workgroup: uniform, so everything derived from it is
  // scalar (the record's unit, tile and addresses)
  int t = __builtin_amdgcn_readfirstlane(s_t);
  int j_lo = 0;   // tickets only grow, so blocks only move forward
  while (t < total) {
    int hi = nu + look;   // start(j_lo) <= t < start(hi) = total
    while (hi - j_lo > 1) {
      const int mid = (j_lo + hi) >> 1;
      if (start(mid) <= t)
        j_lo = mid;
      else
        hi = mid;
    }
    const int j = j_lo;
    int r = t - start(j);
    const int cd = j < nu ? dpre(u_lo + j + 1) - dpre(u_lo + j) : 0;
    const bool dgr = r < cd;
    const int unit = dgr ? u_lo + j : u_lo + j - look;
    if (!dgr) r -= cd;
    const int e = unit / NU, nt = unit - e * NU;
    int nxt_t = 0;
    if (tid == 0) nxt_t = int(atomicAdd(ticket, 1u));
    // The record's lane constants (loader slots, LDS offsets) are derived
    // from this copy of the thread index, which the compiler cannot move out
    // of the loop: hoisted, the two record kinds' constants would be live at
    // once and spill.
    int rtid = tid;
    asm volatile("" : "+v"(rtid));
    if (dgr) {
      dgrad_item<KIND>(dg, lds, rtid, e, nt, r, gt[e + 1] - gt[e], [] {});
      if (KIND == 0) {   // this record's dH1/h2 stores complete in L2, then counted
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        if (tid == 0) atomicAdd(&ready[unit], 1u);
      }
    } else {
      if (KIND == 0) {
        if (tid == 0) {
          const uint32_t need = uint32_t(gt[e + 1] - gt[e]);
          int n = 0;
          while (atomicAdd(&ready[unit], 0u) < need && ++n < kMegaBwdSpin)
            __builtin_amdgcn_s_sleep(4);
          if (n >= kMegaBwdSpin)
            atomicOr(const_cast<uint32_t*>(&hdr->status), MOE_STATUS_SYNC_TIMEOUT);
        }
        __syncthreads();
      }
      // items b0 .. b1 - 1 of the unit's NBw
      const int G = group(e);
      const int b0 = r * G, b1 = min(NBw, b0 + G);
      const int w = e * per_e + nt * NBw;
      wgrad_run<TW, TAG, ACC>(wg, lds, rtid, w + b0, w + b1, 1);
    }
    if (tid == 0) s_t = nxt_t;
    lds_barrier();
    t = __builtin_amdgcn_readfirstlane(s_t);
  }
}

// ------------------------------------------------------------------ launchers
// Resident workgroups per CU of one kernel (queried once per kernel).
template <int ID, typename K>
static int occupancy(K kernel, int threads = 256) {
  static int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n <= 0)
      n = 1;
    per_cu = n;
  }
  return per_cu;
}

static unsigned persistent_grid(int per_cu, int64_t items, int cus) {
  int64_t g = std::min<int64_t>(items, int64_t(cus) * per_cu);
  g = (g + kXcds - 1) / kXcds * kXcds;
  return unsigned(std::max<int64_t>(g, kXcds));
}

// kind 0: W2 DGRAD + SwiGLU backward; 1: W13 DGRAD.
hipError_t launch_dgrad(int kind, const BwdArgs& a, int64_t mt_max, int cus, hipStream_t s) {
  if (mt_max == 0) return hipSuccess;
  if (kind == 0) {
    const unsigned g = persistent_grid(occupancy<0>(k_gemm_dgrad<0>, 512), mt_max * a.NT, cus);
    hipLaunchKernelGGL(k_gemm_dgrad<0>, dim3(g), dim3(512), 0, s, a);
  } else {
    const unsigned g = persistent_grid(occupancy<1>(k_gemm_dgrad<1>, 512), mt_max * a.NT, cus);
    hipLaunchKernelGGL(k_gemm_dgrad<1>, dim3(g), dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

// dW[e] = B_e^T A_e for every expert (a.acc_dw: dW[e] += it); dw_f32 selects
// the dW storage type; tag names the launch (2: dW2, 13: dW13).
hipError_t launch_wgrad(int dw_f32, int tag, const BwdArgs& args, int cus, hipStream_t s) {
  const int64_t items = int64_t(args.E) * ((args.a_ld + 255) / 256) * (args.b_ld / 128);
  if (items == 0) return hipSuccess;
  // the hot experts go to k_wgrad_hot only where it applies; otherwise every
  // expert stays on k_gemm_wgrad
  BwdArgs a = args;
  a.hot_wg = (args.hot_wg && args.cst && !dw_f32 && !args.acc_dw && args.a_ld % 256 == 0 &&
              args.b_ld % 256 == 0) ? 1 : 0;
#define MOE_WG(TW, TAG, ACC, ID)                                                                \
  do {                                                                                        \
    const unsigned g =                                                                        \
        persistent_grid(occupancy<ID>(k_gemm_wgrad<TW, TAG, ACC>, 512), items, cus);          \
    hipLaunchKernelGGL((k_gemm_wgrad<TW, TAG, ACC>), dim3(g), dim3(512), 0, s, a);           \
  } while (0)
  const int acc = a.acc_dw ? 1 : 0;
  if (dw_f32) {
    if (tag == 2) {
      if (acc) MOE_WG(float, 2, 1, 6); else MOE_WG(float, 2, 0, 2);
    } else {
      if (acc) MOE_WG(float, 13, 1, 7); else MOE_WG(float, 13, 0, 3);
    }
  } else {
    if (tag == 2) {
      if (acc) MOE_WG(uint16_t, 2, 1, 8); else MOE_WG(uint16_t, 2, 0, 4);
    } else {
      if (acc) MOE_WG(uint16_t, 13, 1, 9); else MOE_WG(uint16_t, 13, 0, 5);
    }
  }
#undef MOE_WG
  if (a.hot_wg) {   // the hot experts' 256 x 256 tiles
    const unsigned g = persistent_grid(1, int64_t(cus), cus);
    if (tag == 2)
      hipLaunchKernelGGL(k_wgrad_hot<2>, dim3(g), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL(k_wgrad_hot<13>, dim3(g), dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

// Fused backward of one projection: kind 0 = W2 (DGRAD + SwiGLU backward
// records with dg, dW2 records with wg; ready: one counter per expert and
// 256-column block of F), 1 = W13 (dX rows, dW13).  tickets: kXcds
// counters.  The hot experts' dW tiles stay on the streaming tiles here.
hipError_t launch_bwd_mega(int kind, int dw_f32, const BwdArgs& dg, const BwdArgs& wg,
                           uint32_t* tickets, uint32_t* ready, int cus, hipStream_t s) {
  // units: the DGRAD n-tiles are the dW column tiles (NT x NB dW items per expert)
  if (dg.NT != (wg.a_ld + 255) / 256) return hipErrorInvalidValue;
  BwdArgs w = wg;
  w.hot_wg = 0;
  const unsigned g = persistent_grid(1, int64_t(cus), cus);
  const int look = int(g / kXcds);   // the XCD's workgroups
  const int acc = w.acc_dw ? 1 : 0;
#define MOE_MB(K, TW, ACC) \
  hipLaunchKernelGGL((k_bwd_mega<K, TW, ACC>), dim3(g), dim3(512), 0, s, dg, w, tickets, ready, \
                     look)
  if (kind == 0) {
    if (dw_f32) {
      if (acc) MOE_MB(0, float, 1); else MOE_MB(0, float, 0);
    } else {
      if (acc) MOE_MB(0, uint16_t, 1); else MOE_MB(0, uint16_t, 0);
    }
  } else {
    if (dw_f32) {
      if (acc) MOE_MB(1, float, 1); else MOE_MB(1, float, 0);
    } else {
      if (acc) MOE_MB(1, uint16_t, 1); else MOE_MB(1, uint16_t, 0);
    }
  }
#undef MOE_MB
  return hipGetLastError();
}

}  // namespace moe
