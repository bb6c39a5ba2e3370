// Grouped GEMMs of the expert FFN with MXFP8 operands on gfx950
// (v_mfma_scale_f32_32x32x64_f8f6f4: E4M3 x E4M3 with one E8M0 scale per 32
// values of each operand, fp32 accumulation).
//
// Dist-MoE explainer section 02: forward GEMMs contract over features with
// 1x32 activation blocks; weights are prepared in 32x32 blocks so the forward
// and the input-gradient GEMM read the same E4M3 values with the scale matrix
// read in the other orientation; weight gradients contract over token rows
// and read column bundles (32x1 blocks down each expert's padded rows).
// "Mixture of Experts: How Routing Becomes GPU Computation", section 2: the
// grouped GEMM and its two gradients.
//
//   k_mx_fwd<0>: h1 = Xq W13q^T per expert (+ SwiGLU epilogue -> h1, h2 bf16)
//   k_mx_fwd<1>: h3 = H2q W2q^T per expert -> route slots (bf16)
//   k_mx_dgrad<0>: dH2 = dH3q W2q (contraction over D) + SwiGLU backward -> dH1
//   k_mx_dgrad<1>: dXr = dH1q W13q (contraction over 2F) -> fp32 rows at
//                  their route slots t*K + k
//   k_mx_wgrad:  dW[b][a] = sum_m B[m][b] A[m][a] from column bundles
//
// MFMA operand layout (measured on gfx950): one MFMA covers 64 contraction
// values of a row, held by lanes r and r + 32 with 32 bytes each; scale block
// b is bytes [16b, 16b + 16) of both lanes, and its E8M0 scale is the one
// supplied by lane r + 32b.  So lane (r, h) carries 16 values of each of the
// two MX blocks of the step: contraction chunks h and 2 + h (16 values each),
// and supplies the scale of block h.
//
// MI355X design: the same coalesced, XOR-swizzled LDS staging as the BF16
// kernels (128-byte row segments per stage; fp8 stages span 128 contraction
// values).  DGRAD stages the E4M3 weight tile as it lies in memory (rows along
// the contraction) and reads its MFMA operand with the gfx950 LDS transpose
// read ds_read_b64_tr_b8, so one copy of the E4M3 weights serves forward and
// backward with no register transpose.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "mxq.h"

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void mfma_mx(f32x16& acc, u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1,
                                        int sa, int sb) {
  const i32x8 a = {int(a0[0]), int(a0[1]), int(a0[2]), int(a0[3]),
                   int(a1[0]), int(a1[1]), int(a1[2]), int(a1[3])};
  const i32x8 b = {int(b0[0]), int(b0[1]), int(b0[2]), int(b0[3]),
                   int(b1[0]), int(b1[1]), int(b1[2]), int(b1[3])};
  // cbsz = blgp = 0: both operands E4M3; opsel 0: scale in byte 0.
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, sa, 0, sb);
}

// E2M1 x E2M1 (cbsz = blgp = 4): a 4-bit operand fills four registers, so
// the upper half of each 8-register operand is not read.  Lane (r, h) holds
// MX block h of the 64-value step (32 values, low nibble first) and supplies
// that block's scale (measured on gfx950).
__device__ __forceinline__ void mfma_fp4(f32x16& acc, u32x4 a0, u32x4 b0, int sa, int sb) {
  const i32x8 a = {int(a0[0]), int(a0[1]), int(a0[2]), int(a0[3]), 0, 0, 0, 0};
  const i32x8 b = {int(b0[0]), int(b0[1]), int(b0[2]), int(b0[3]), 0, 0, 0, 0};
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 4, 4, 0, sa, 0, sb);
}

__device__ __forceinline__ int byte_of(uint32_t w, int i) { return int((w >> (8 * i)) & 0xffu); }

__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ ((r ^ (r >> 3)) & 7)) << 4); }
// 64-byte rows (WGRAD): 16-byte chunk ch of row r
__device__ __forceinline__ int swz64(int r, int ch) { return r * 64 + ((ch ^ ((r >> 2) & 3)) << 4); }

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, float a, float b, float c,
                                                 float d) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
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
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = *reinterpret_cast<const u32x2*>(p);
  f[0] = __uint_as_float(v[0] << 16);
  f[1] = __uint_as_float(v[0] & 0xffff0000u);
  f[2] = __uint_as_float(v[1] << 16);
  f[3] = __uint_as_float(v[1] & 0xffff0000u);
}

// ------------------------------------------------------------------ forward
// W1: weights prepared in 1x32 blocks (inference): every weight row has its
// own exponent per 32 values, so each lane takes the exponents of its own
// row (one dword per stage, staged through LDS like the token exponents)
// instead of the wave's 32x32-block exponents.
// FP4 (needs W1): E2M1 operands, two per byte.  A stage is still 128 bytes
// of every row, now 256 values = 8 MX blocks = four MFMAs per accumulator,
// with 8 exponent bytes per row.
// MODE 2: the fused (Mega) forward: the W13 records of a and the W2 records
// of a2 from per-XCD queues with per-expert readiness counters in msync, the
// hand-off described at k_gemm_mega (gemm_fwd.hip).  Prefetch into the next
// record crosses into a W2 record only once its h2 rows are complete;
// otherwise the record waits for them before its first loads.
constexpr int kMxMegaSpin = 1 << 22;   // polls (each followed by a short sleep)

template <int MODE, int W1, int FP4, int RING = 0>
__global__ __launch_bounds__(256) void k_mx_fwd(MxArgs a, MxArgs a2, uint32_t* msync, int look) {
  static_assert(!FP4 || W1, "4-bit weights come in 1x32 blocks");
  static_assert(RING == 0 || (MODE != 2 && !W1 && RING >= 3 && RING <= 5),
                "the ring of direct loads serves the MXFP8 32x32 staged passes");
  constexpr int kW = 128 * 128;      // weight stage: 128 rows x 128 bytes
  constexpr int kA = kBM * 128;      // token stage: 64 rows x 128 bytes
  constexpr int kXb = FP4 ? 8 : 4;   // exponent bytes per row and stage
  constexpr int kSc = kBM * kXb;     // token scales of the stage
  // + the weight exponents: one dword per wave (32x32) or per weight row (1x32)
  // (the ring's weight exponents: 64 dwords, lane l's of wave l mod 4)
  constexpr int kStage = kW + kA + kSc + (RING ? 256 : W1 ? 128 * kXb : 16);
  constexpr int kNbuf = RING ? RING : 2;      // LDS stage buffers
  constexpr int kXch = 2 * 2 * 16 * 64 * 4;   // SwiGLU epilogue: up halves of two waves
  __shared__ __attribute__((aligned(16))) char lds[kNbuf * kStage + (MODE != 1 ? kXch : 0)];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int lc = tid & 7;
  const int lrow = tid >> 3;

  const RouteHdr* hdr = a.hdr;
  if (a.replay_only && !hdr->rec.replay) return;
  const int n_items = hdr->n_mt * a.NT;
  uint16_t* out0 = a.out0 ? reinterpret_cast<uint16_t*>(a.out0) : global_ptr<uint16_t>(hdr->rec.h1);
  uint16_t* out1 = reinterpret_cast<uint16_t*>(a.out1);
  const MxArgs& b2 = MODE == 2 ? a2 : a;   // the W2 records' arguments
  uint16_t* h3 = reinterpret_cast<uint16_t*>(b2.out0);
  const int Kd = a.Kd;
  const int KB = Kd / 32;           // scale bytes per row
  const int Kb = FP4 ? Kd / 2 : Kd; // code bytes per row
  const int xcd = MODE == 2 ? hw_xcd() : blockIdx.x % kXcds;
  const int per = gridDim.x / kXcds;
  const int chunk = (n_items + kXcds - 1) / kXcds;
  const int S_fix = Kb / 128;       // stages per item (MODE 0 / 1)

  // MODE 2: this XCD's experts [e_lo, e_lo + ne) and its queue: block j =
  // the W13 records of expert e_lo + j, then the W2 records of expert
  // e_lo + j - look; mstart(j) = records before block j
  const int32_t* gt = a.mtoff;
  uint32_t* ticket = msync + xcd;
  uint32_t* ready = msync + kXcds;
  int e_lo = 0, ne = 0, total = 0;
  if (MODE == 2) {
    e_lo = xcd_first_unit(gt, 0, a.E, 1, xcd);
    ne = xcd_first_unit(gt, 0, a.E, 1, xcd + 1) - e_lo;
    total = (gt[e_lo + ne] - gt[e_lo]) * (a.NT + a2.NT);
  }
  auto mstart = [&](int j) {
    const int p = min(j, ne), q = max(0, min(j - look, ne));
    return (gt[e_lo + p] - gt[e_lo]) * a.NT + (gt[e_lo + q] - gt[e_lo]) * a2.NT;
  };
  int j_lo = 0;   // tickets only grow, so blocks only move forward

  // Operand sources of one work item (an m-tile of an expert x 128 weight rows).
  struct Item {
    int md, S, e, nt, row0, rows;
    const uint8_t* w[4];     // weight rows of this thread (4 x 16 bytes per stage)
    const uint8_t* t[2];     // token rows
    const uint32_t* ws;      // weight exponents
    const uint32_t* ts;      // token exponents
  };
  int e_prev = -1;  // expert of this workgroup's previous item
  auto setup = [&](int w, Item& I) {
    int md = MODE, e, u;
    if (MODE == 2) {
      int hi = ne + look;   // mstart(j_lo) <= w < mstart(hi) = total
      while (hi - j_lo > 1) {
        const int mid = (j_lo + hi) >> 1;
        if (mstart(mid) <= w)
          j_lo = mid;
        else
          hi = mid;
      }
      u = w - mstart(j_lo);
      const int c13 = j_lo < ne ? (gt[e_lo + j_lo + 1] - gt[e_lo + j_lo]) * a.NT : 0;
      md = u < c13 ? 0 : 1;
      e = md == 0 ? e_lo + j_lo : e_lo + j_lo - look;
      if (md) u -= c13;
    } else {
      e = item_expert(a.mtoff, a.E, a.NT, w, e_prev);
      e_prev = e;
      u = w - a.mtoff[e] * a.NT;
    }
    const MxArgs& A = md == 1 ? b2 : a;
    const int Kbi = FP4 ? A.Kd / 2 : A.Kd;
    const int KBi = A.Kd / 32;
    const int mt_e = a.mtoff[e + 1] - a.mtoff[e];
    const int nt = u / mt_e;
    const int mt = u - nt * mt_e;
    const int row0 = a.offsets[e] + mt * kBM;
    const int rows = min(kBM, a.offsets[e + 1] - row0);
    I.md = md;
    I.S = MODE == 2 ? Kbi / 128 : S_fix;
    I.e = e;
    I.nt = nt;
    I.row0 = row0;
    I.rows = rows;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rho = lrow + 32 * j;
      const int wr = md == 0 ? (rho < 64 ? nt * 64 + rho : A.F + nt * 64 + rho - 64)
                             : nt * 128 + rho;
      I.w[j] = A.qw + (int64_t(e) * A.N + wr) * Kbi + lc * 16;
    }
    // the 32 weight rows of this wave form one 32-row scale block
    const int wrow0 = md == 0 ? ((wave < 2 ? 0 : A.F) + nt * 64 + (wave & 1) * 32)
                              : nt * 128 + wave * 32;
    // 1x32: thread tid < 128 fetches the exponents of tile row tid
    const int wr1 = md == 0 ? ((tid & 127) < 64 ? nt * 64 + (tid & 63)
                                                : A.F + nt * 64 + (tid & 63))
                            : nt * 128 + (tid & 127);
    I.ws = W1 ? reinterpret_cast<const uint32_t*>(A.sw) + (int64_t(e) * A.N + wr1) * (kXb / 4)
              : reinterpret_cast<const uint32_t*>(A.sw + (int64_t(e) * (A.N / 32) + wrow0 / 32) * KBi);
    // Tile rows past the expert's last row re-read that row: every load is
    // unconditional, and the extra output columns are never stored.
#pragma unroll
    for (int j = 0; j < 2; ++j)
      I.t[j] = A.qa + int64_t(row0 + min(lrow + 32 * j, rows - 1)) * Kbi + lc * 16;
    // token exponents are grouped by stage: the kXb bytes of (s, row) at
    // (s * sa_rows + row) * kXb
    I.ts = reinterpret_cast<const uint32_t*>(A.sa) + int64_t(row0 + min(tid & 63, rows - 1)) * (kXb / 4);
    if constexpr (RING > 0) {
      // Direct loads: load j of this wave fills the eight tile rows from
      // r0 = 32 wave + 8 j (weights) or 16 wave + 8 j (tokens); lane l
      // fetches the chunk of row r0 + l / 8 that the swizzle puts at slot
      // l % 8 of that row.
      const int lq = lane >> 3, ls = lane & 7;
      auto chunk = [&](int r) { return (ls ^ ((r ^ (r >> 3)) & 7)) << 4; };
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rho = 32 * wave + 8 * j + lq;
        const int wr = md == 0 ? (rho < 64 ? nt * 64 + rho : A.F + nt * 64 + rho - 64)
                               : nt * 128 + rho;
        I.w[j] = A.qw + (int64_t(e) * A.N + wr) * Kbi + chunk(rho);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 16 * wave + 8 * j + lq;
        I.t[j] = A.qa + int64_t(row0 + min(r, rows - 1)) * Kbi + chunk(r);
      }
      const int q = lane & 3;   // the wave whose block exponents this lane fetches
      const int q0 = md == 0 ? ((q < 2 ? 0 : A.F) + nt * 64 + (q & 1) * 32) : nt * 128 + q * 32;
      I.ws = reinterpret_cast<const uint32_t*>(A.sw + (int64_t(e) * (A.N / 32) + q0 / 32) * KBi);
    }
  };
  // MODE 2 (W1 weights): the exponent rows of the W13 and W2 weights differ
  auto sw_rows = [&](const Item& I) { return MODE == 2 && I.md == 1 ? b2.sw_rows : a.sw_rows; };

  u32x4 R0[6], R1[6];
  // [0..1] weight scales (of the wave, or of tile row tid with W1), [2..3]
  // token scales of row tid; the second dword of each only with FP4
  uint32_t S0[4], S1[4];
  Item cur, nxt;
  bool cross = false;   // loads past the current item's last stage fetch the next item's
  // Stage idx of the current item; idx >= S is stage idx - S of the next item
  // (without a next item: the current item's last stage, never used).
  auto load = [&](u32x4* R, uint32_t* Sc, int idx) {
    const int S = cur.S;
    const bool nx = idx >= S;
    const int st = nx ? (cross ? idx - S : S - 1) : idx;
    const bool use_n = nx && cross;
    const int64_t off = int64_t(st) * 128;
#pragma unroll
    for (int j = 0; j < 4; ++j)   // weights: non-temporal (streamed once per m-tile)
      R[j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>((use_n ? nxt.w[j] : cur.w[j]) + off));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      R[4 + j] = *reinterpret_cast<const u32x4*>((use_n ? nxt.t[j] : cur.t[j]) + off);
    const uint32_t* wsp = use_n ? nxt.ws : cur.ws;
    const uint32_t* tsp = use_n ? nxt.ts : cur.ts;
    if (FP4) {
      typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 w2 = *reinterpret_cast<const u32x2*>(wsp + int64_t(st) * sw_rows(use_n ? nxt : cur) * 2);
      const u32x2 t2 = *reinterpret_cast<const u32x2*>(tsp + int64_t(st) * a.sa_rows * 2);
      Sc[0] = w2[0];
      Sc[1] = w2[1];
      Sc[2] = t2[0];
      Sc[3] = t2[1];
    } else {
      Sc[0] = W1 ? wsp[int64_t(st) * sw_rows(use_n ? nxt : cur)] : wsp[st];
      Sc[2] = tsp[int64_t(st) * a.sa_rows];
    }
  };
  auto store = [&](const u32x4* R, const uint32_t* Sc, int buf) {
    char* base = lds + buf * kStage;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4*>(base + swz(lrow + 32 * j, lc)) = R[j];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      *reinterpret_cast<u32x4*>(base + kW + swz(lrow + 32 * j, lc)) = R[4 + j];
    uint32_t* ts = reinterpret_cast<uint32_t*>(base + kW + kA);
    uint32_t* ws = reinterpret_cast<uint32_t*>(base + kW + kA + kSc);
    if (FP4) {
      if (tid < kBM) {
        ts[2 * tid] = Sc[2];
        ts[2 * tid + 1] = Sc[3];
      }
      if (tid < 128) {
        ws[2 * tid] = Sc[0];
        ws[2 * tid + 1] = Sc[1];
      }
    } else {
      if (tid < kBM) ts[tid] = Sc[2];
      if (W1) {
        if (tid < 128) ws[tid] = Sc[0];
      } else if (lane == 0) {
        ws[wave] = Sc[0];
      }
    }
  };
  f32x16 acc0, acc1;
  // Both 32-token halves are always multiplied: no accumulator depends on
  // a branch inside the stage loop.
  auto compute = [&](int buf) {
    const char* wl = lds + buf * kStage;
    const char* tl = wl + kW;
    const uint32_t* tsc = reinterpret_cast<const uint32_t*>(tl + kA);
    const uint32_t* wscl = reinterpret_cast<const uint32_t*>(tl + kA + kSc);
    const int wrow = 32 * wave + lr;
    if (FP4) {
      // lane (r, h) multiplies 16-byte chunk 2q + h of its rows: MX block
      // 2q + h of the stage, whose exponent is byte (2q + h) of the row's 8
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 2 * q + lh;
        const int dw = q >> 1, by = c & 3;
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(wl + swz(wrow, c));
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(tl + swz(lr, c));
        const u32x4 d0 = *reinterpret_cast<const u32x4*>(tl + swz(32 + lr, c));
        const int sa = byte_of(wscl[2 * wrow + dw], by);
        mfma_fp4(acc0, a0, b0, sa, byte_of(tsc[2 * lr + dw], by));
        mfma_fp4(acc1, a0, d0, sa, byte_of(tsc[2 * (32 + lr) + dw], by));
      }
      return;
    }
    const uint32_t ts0 = tsc[lr];
    const uint32_t ts1 = tsc[32 + lr];
    const uint32_t wsc = W1 ? wscl[wrow] : wscl[wave];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int ca = 4 * q + lh, cb = 4 * q + 2 + lh;
      const int blk = 2 * q + lh;
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(wl + swz(wrow, ca));
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(wl + swz(wrow, cb));
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(tl + swz(lr, ca));
      const u32x4 b1 = *reinterpret_cast<const u32x4*>(tl + swz(lr, cb));
      const u32x4 d0 = *reinterpret_cast<const u32x4*>(tl + swz(32 + lr, ca));
      const u32x4 d1 = *reinterpret_cast<const u32x4*>(tl + swz(32 + lr, cb));
      const int sa = byte_of(wsc, blk);
      mfma_mx(acc0, a0, a1, b0, b1, sa, byte_of(ts0, blk));
      mfma_mx(acc1, a0, a1, d0, d1, sa, byte_of(ts1, blk));
    }
  };

  // Items of this XCD's chunk come from its work queue, in order, when some
  // expert spans several m-tiles (skewed routing); a workgroup then holds two
  // tickets (its current and next item) and takes the one after while an
  // item's epilogue runs.  Otherwise they are dealt statically (slot,
  // slot + per, ...), which costs no atomics.
  auto valid = [&](int it) {
    return MODE == 2 ? it < total : (it < chunk && xcd * chunk + it < n_items);
  };
  auto index = [&](int it) { return MODE == 2 ? it : xcd * chunk + it; };
  auto take = [&]() { return MODE == 2 ? int(atomicAdd(ticket, 1u)) : wq_take(hdr, xcd); };
  // MODE 2: W13 records of expert e, which its W2 records wait for
  auto need = [&](int e) { return uint32_t((gt[e + 1] - gt[e]) * a.NT); };
  // The item's epilogue (as the BF16 kernels): acc[b][v] = C[row 8*(v/4) + 4*lh + v%4][token 32*b + lr].
  auto epilogue = [&]() {
    const int nt = cur.nt, row0 = cur.row0, rows = cur.rows;
    const int md = MODE == 2 ? cur.md : MODE;
    if (md == 0) {
      const int F = a.F;
      const int ncol = (wave < 2 ? 0 : F) + nt * 64 + (wave & 1) * 32 + 4 * lh;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const f32x16& acc = b ? acc1 : acc0;
        const int m = 32 * b + lr;
        if (m < rows) {
          uint16_t* o = out0 + int64_t(row0 + m) * (2 * F) + ncol;
#pragma unroll
          for (int g = 0; g < 4; ++g)
            store4<uint16_t>(o + 8 * g, acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
        }
      }
      float* xch = reinterpret_cast<float*>(lds + kNbuf * kStage);  // not the stage buffers
      if (wave >= 2) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          xch[(((wave - 2) * 2 + 0) * 16 + v) * 64 + lane] = round_bf16(acc0[v]);
          xch[(((wave - 2) * 2 + 1) * 16 + v) * 64 + lane] = round_bf16(acc1[v]);
        }
      }
      lds_barrier();
      if (wave < 2) {
        const int jcol = nt * 64 + wave * 32 + 4 * lh;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const f32x16& acc = b ? acc1 : acc0;
          const int m = 32 * b + lr;
          if (m < rows) {
            float h[16];
#pragma unroll
            for (int v = 0; v < 16; ++v)
              h[v] = round_bf16(silu_f(clamp_gate(round_bf16(acc[v]), a.limit)) *
                                clamp_up(xch[((wave * 2 + b) * 16 + v) * 64 + lane], a.limit));
            if (out1) {
              uint16_t* o = out1 + int64_t(row0 + m) * F + jcol;
#pragma unroll
              for (int g = 0; g < 4; ++g)
                store4<uint16_t>(o + 8 * g, h[4 * g], h[4 * g + 1], h[4 * g + 2], h[4 * g + 3]);
            }
            if (a.q_out) {
              // The wave's 32 columns are one 1x32 block of the h2 row: lane
              // (r, 0) holds block values 8g + i, lane (r, 1) values 8g + 4 + i
              // (g, i < 4); amax over both, then k_rowq's encoding.
              float amax = 0.0f;
#pragma unroll
              for (int v = 0; v < 16; ++v) amax = fmaxf(amax, fabsf(h[v]));
              amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
              const int64_t row = row0 + m;
              const int c0 = nt * 64 + wave * 32;   // the block's first column
              if (FP4) {
                const int ex = e8m0_exp_fp4(amax);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                  uint32_t wv = 0;
#pragma unroll
                  for (int i = 0; i < 4; ++i) wv |= e2m1_rne(ldexp_i(h[4 * g + i], -ex)) << (4 * i);
                  *reinterpret_cast<uint16_t*>(a.q_out + row * (F / 2) + (jcol + 8 * g) / 2) =
                      uint16_t(wv);
                }
                if (lh == 0)
                  a.s_out[(int64_t(c0 / 256) * a.q_rows + row) * 8 + (c0 / 32) % 8] =
                      uint8_t(ex + 127);
              } else {
                const int ex = e8m0_exp(amax);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                  uint32_t wv = 0;
#pragma unroll
                  for (int i = 0; i < 4; ++i) wv |= e4m3_rne(ldexp_i(h[4 * g + i], -ex)) << (8 * i);
                  *reinterpret_cast<uint32_t*>(a.q_out + row * F + jcol + 8 * g) = wv;
                }
                if (lh == 0)
                  a.s_out[(int64_t(c0 / 128) * a.q_rows + row) * 4 + (c0 / 32) % 4] =
                      uint8_t(ex + 127);
              }
            }
          }
        }
      }
      lds_barrier();
      if (MODE == 2) {   // this record's stores complete in L2, then counted
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        if (tid == 0) atomicAdd(&ready[cur.e], 1u);
      }
    } else {
      const int ncol = nt * 128 + wave * 32 + 4 * lh;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const f32x16& acc = b ? acc1 : acc0;
        const int m = 32 * b + lr;
        if (m < rows) {
          const int64_t slotr = b2.sorted_route[row0 + m];
          if (b2.y32) {   // FUSED combine (h3 rounded to bf16 as the slots would hold it)
            const float sc = b2.scores[slotr];
            float* o = b2.y32 + (slotr / b2.K) * b2.N + ncol;
#pragma unroll
            for (int g = 0; g < 4; ++g)
              fused_add4(o + 8 * g, sc, round_bf16(acc[4 * g]), round_bf16(acc[4 * g + 1]),
                         round_bf16(acc[4 * g + 2]), round_bf16(acc[4 * g + 3]));
          } else {
            uint16_t* o = h3 + slotr * b2.N + ncol;
#pragma unroll
            for (int g = 0; g < 4; ++g)
              store4<uint16_t>(o + 8 * g, acc[4 * g], acc[4 * g + 1], acc[4 * g + 2],
                               acc[4 * g + 3]);
          }
        }
      }
    }
  };

  const bool dyn = MODE == 2 || hdr->max_count > kBM;
  const int slot = blockIdx.x / kXcds;
  __shared__ int s_q[2];
  __shared__ int s_ok;
  if (dyn && tid == 0) {
    s_q[0] = take();
    s_q[1] = take();
  }
  lds_barrier();
  int it = dyn ? s_q[0] : slot, itn = dyn ? s_q[1] : slot + per;
  if (valid(it)) setup(index(it), cur);
  if constexpr (RING > 0) {
    // RING stage buffers in LDS filled by direct global-to-LDS loads, RING - 1
    // stages in flight, continuing into the next item's first stages while
    // an item ends (its epilogue uses no stage buffer).  Per wave and stage:
    // four weight and two token loads of 1 KiB, then one 256-byte exponent
    // load (waves 0, 2: the token exponents; waves 1, 3: the four waves'
    // block exponents; both pairs write identical bytes).
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(lds));   // LDS byte address
    auto issue = [&](const Item& I, int st, int b) {
      const uint32_t base = lds0 + uint32_t(b) * kStage;
      const int64_t off = int64_t(st) * 128;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dma16(I.w[j] + off, __builtin_amdgcn_readfirstlane(base + (32 * wv + 8 * j) * 128));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        dma16(I.t[j] + off, __builtin_amdgcn_readfirstlane(base + kW + (16 * wv + 8 * j) * 128));
      if (wv & 1)
        dma4(I.ws + st, __builtin_amdgcn_readfirstlane(base + kW + kA + kSc));
      else
        dma4(I.ts + int64_t(st) * a.sa_rows, __builtin_amdgcn_readfirstlane(base + kW + kA));
    };
    // until this wave's loads of the stage `after` stages before the newest
    // have landed (7 per stage; loads complete in issue order)
    auto wait_behind = [&](int after) {
      if (after >= 3)
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 | (21 & 15) | ((21 >> 4) << 14));
      else if (after == 2)
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 | 14);
      else if (after == 1)
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 | 7);
      else
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    };
    int bq = 0;    // buffer of cur's stage 0
    int pre = 0;   // stages of cur that the previous item issued
    for (; valid(it);) {
      const int S = cur.S;
      const bool ahead = valid(itn) && S >= RING - 1;   // prefetch into the next item
      if (ahead) setup(index(itn), nxt);
      acc0 = f32x16{};
      acc1 = f32x16{};
      for (int st = pre; st < min(RING - 1, S); ++st) issue(cur, st, (bq + st) % RING);
      int b = bq;   // buffer of stage s
      for (int s = 0; s < S; ++s) {
        wait_behind(ahead ? RING - 2 : min(S - 1 - s, RING - 2));
        stage_barrier();   // stage s is in; every wave is done with stage s - 1
        const int t = s + RING - 1;
        const int bt = b == 0 ? RING - 1 : b - 1;   // the buffer of stage s - 1
        if (t < S)
          issue(cur, t, bt);
        else if (ahead)
          issue(nxt, t - S, bt);
        compute(b);
        b = b + 1 == RING ? 0 : b + 1;
      }
      int taken = 0;
      if (dyn && tid == 0) taken = take();
      epilogue();
      if (dyn && tid == 0) s_q[0] = taken;
      lds_barrier();
      pre = ahead ? RING - 1 : 0;
      if (ahead)
        cur = nxt;
      else if (valid(itn))
        setup(index(itn), cur);
      bq = b;
      it = itn;
      itn = dyn ? s_q[0] : itn + per;
    }
    if (dyn && tid == 0) wq_finish(hdr, xcd, per);
    return;
  }
  bool primed = false;  // buffer 0 / R1 / R0 already hold stages 0 / 1 / 2 of cur
  for (; valid(it);) {
    const int S = cur.S;
    // Prefetch across items needs three stages per item (the three stages in
    // flight at an item's end must all belong to the next item).
    cross = valid(itn) && S >= 3;
    if (cross) {
      setup(index(itn), nxt);
      if (MODE == 2) {
        cross = nxt.S >= 3;
        if (nxt.md == 1) {   // a W2 record: only with its h2 rows complete
          if (tid == 0) s_ok = atomicAdd(&ready[nxt.e], 0u) >= need(nxt.e);
          lds_barrier();
          cross = cross && s_ok;
        }
      }
    }
    acc0 = f32x16{};
    acc1 = f32x16{};

    // Pipeline: at the top of each pass LDS buffer 0 holds stage s, R1 stage
    // s + 1 and R0 stage s + 2.
    if (!primed) {
      if (MODE == 2 && cur.md == 1) {   // wait (bounded) for the h2 rows
        if (tid == 0) {
          int n = 0;
          while (atomicAdd(&ready[cur.e], 0u) < need(cur.e) && ++n < kMxMegaSpin)
            __builtin_amdgcn_s_sleep(4);
          if (n >= kMxMegaSpin)
            atomicOr(const_cast<uint32_t*>(&hdr->status), MOE_STATUS_SYNC_TIMEOUT);
        }
        lds_barrier();
      }
      load(R0, S0, 0);
      load(R1, S1, 1);
      store(R0, S0, 0);
      load(R0, S0, 2);
      lds_barrier();
    }
    for (int s = 0; s + 1 < S; s += 2) {
      compute(0);
      store(R1, S1, 1);
      load(R1, S1, s + 3);
      lds_barrier();
      compute(1);
      store(R0, S0, 0);
      load(R0, S0, s + 4);
      lds_barrier();
    }
    if (S & 1) {
      compute(0);
      lds_barrier();
      if (cross) {   // R1, R0 hold stages 0, 1 of the next item
        store(R1, S1, 0);
#pragma unroll
        for (int j = 0; j < 6; ++j) R1[j] = R0[j];
#pragma unroll
        for (int j = 0; j < 4; ++j) S1[j] = S0[j];
        load(R0, S0, S + 2);
        lds_barrier();
      }
    }
    int taken = 0;
    if (dyn && tid == 0) taken = take();
    epilogue();
    if (dyn && tid == 0) s_q[0] = taken;
    lds_barrier();
    if (!cross) {
      if (valid(itn)) setup(index(itn), cur);
      primed = false;
    } else {
      cur = nxt;
      primed = true;
    }
    it = itn;
    itn = dyn ? s_q[0] : itn + per;
  }
  if (MODE != 2 && dyn && tid == 0) wq_finish(hdr, xcd, per);
}

// ------------------------------------------------------------------ DGRAD
// ds_read_b64_tr_b8 (gfx950), as measured: within each 16-lane group, the
// lane with index 2j + hh supplies the address of row j of an 8-row block
// (8 bytes: columns 8hh .. 8hh + 7 of a 16-column slab), and lane i receives
// column i of the slab, rows 0..7 as bytes 0..7.
typedef int i32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ i32x2 lds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)((__attribute__((address_space(3))) char*)p));
}

// Weight stage of the DGRAD kernel: 128 contraction rows of 256 E4M3
// columns; the 16-byte chunks of row r are XOR-swizzled by 2 (r & 7), so the
// row-wise 16-byte stores and the transpose reads (8 + 8 rows x 2 chunks per
// instruction) both spread evenly over the banks.
__device__ __forceinline__ int wsw8(int r, int c) { return r * 256 + ((c ^ ((r & 7) << 1)) << 4); }

// Eight waves: 256 output columns (32 per wave) x up to 64 token rows.
// 256-byte weight row segments stream faster from HBM than 128-byte ones.
// (A 128-row variant, four accumulators per wave, does not fit the 256
// registers of two waves per SIMD without spilling.)
constexpr int kMxDgW = 128 * 256;      // weight stage: 128 contraction rows x 256 columns
constexpr int kMxDgT = kBM * 128;      // token stage: up to 64 rows x 128 values
constexpr int kMxDgSc = kBM * 4;       // token exponents of the stage
constexpr int kMxDgStage = kMxDgW + kMxDgT + kMxDgSc + 32;   // + weight exponents: 8 x 4 blocks
constexpr int kMxDgLds = 2 * kMxDgStage;

// One DGRAD work item: output columns nt * 256 .. + 255 of m-tile mt of
// expert e (mt_e m-tiles).  `between` runs when the contraction is done,
// before the epilogue (a launch takes its next item there).
template <int KIND, typename Between>
__device__ __forceinline__ void mx_dgrad_item(const MxArgs& a, char* lds, int tid, int e, int nt,
                                              int mt, int mt_e, Between&& between) {
  constexpr int kW = kMxDgW;
  constexpr int kT = kMxDgT;
  constexpr int kSc = kMxDgSc;
  constexpr int kStage = kMxDgStage;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int c16 = tid & 15;   // weight loader: 16-column chunk of a 256-byte row segment
  const int kq = tid >> 4;    // weight loader: rows 4kq .. 4kq+3 of the stage
  // transpose reads of the weight operand: 16-lane group G covers columns
  // 32*wave + 16*(G & 1) .. + 15 and contraction half G >> 1 (= lh)
  const int tr_chunk = 2 * wave + ((lane >> 4) & 1);
  const int tr_row = (lane & 15) >> 1;
  const int tr_byte = 8 * (lane & 1);
  const int lc = tid & 7;
  const int lrow = tid >> 3;  // token loader: tile row

  const RouteHdr* hdr = a.hdr;
  const int Kd = a.Kd;
  const int KB = Kd / 32;
  const int S = Kd / 128;
  const int64_t N = a.N;
  const int NB32 = int(N / 32);
  const uint16_t* h1 = global_ptr<const uint16_t>(hdr->rec.h1);

  {
    const int row0 = a.offsets[e] + mt * kBM;
    const int rows = min(kBM, a.offsets[e + 1] - row0);
    // The last tile of an N that is an odd multiple of 128 has 128 columns:
    // its upper half re-reads the lower half, and waves 4..7 multiply it but
    // store nothing (every load stays unconditional).
    const int ncols = min(256, int(N) - nt * 256);
    const int wcol = c16 * 16 < ncols ? c16 * 16 : c16 * 16 - 128;
    const uint8_t* wsrc = a.qw + (int64_t(e) * Kd + 4 * kq) * N + nt * 256 + wcol;
    // Weight exponents of the stage: 8 column blocks (one per wave) x 4
    // blocks along k.  Thread t loads the byte of column block (t >> 2) & 7
    // and k block t & 3; threads 0..31 put them in LDS, so wave w reads its
    // four as one dword.
    const int cb = min(nt * 8 + ((tid >> 2) & 7), NB32 - 1);
    const uint8_t* wsc_src = a.sw + int64_t(e) * KB * NB32 + (tid & 3) * NB32 + cb;
    // Tile rows past the expert's last row re-read that row (outputs not stored).
    const uint8_t* tsrc = a.qa + int64_t(row0 + min(lrow, rows - 1)) * Kd + lc * 16;
    // token exponents are grouped by stage: dword (s, row) at (s * sa_rows + row) * 4
    const uint32_t* tsc_src =
        reinterpret_cast<const uint32_t*>(a.sa) + row0 + min(tid & (kBM - 1), rows - 1);

    f32x16 acc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[b] = f32x16{};
    u32x4 R0[5], R1[5];
    uint32_t S0[2], S1[2];
    // NB: 32-token blocks multiplied (1 or 2; one loop copy each); the 512
    // threads load all 64 rows of the token stage (rows past the tile repeat
    // its last row).
    // W2 DGRAD: each n-tile starts its contraction at nt * S / NT stages, so
    // the n-tiles of an expert read different bands of W2's power-of-two
    // pitch rows at any moment (the sum's order is fixed per item).
    const int rot = KIND == 0 ? int(int64_t(nt) * S / a.NT) : 0;
    auto load = [&](u32x4* R, uint32_t* Sc, int s, auto) {
      s += rot;
      if (s >= S) s -= S;
      const uint8_t* p = wsrc + int64_t(s) * 128 * N;
#pragma unroll
      for (int i = 0; i < 4; ++i)   // weights: non-temporal (streamed once per m-tile)
        R[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + i * N));
      R[4] = *reinterpret_cast<const u32x4*>(tsrc + int64_t(s) * 128);
      Sc[0] = wsc_src[int64_t(4 * s) * NB32];
      Sc[1] = tsc_src[int64_t(s) * a.sa_rows];
    };
    auto store = [&](const u32x4* R, const uint32_t* Sc, int buf, auto) {
      char* lw = lds + buf * kStage;
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(lw + wsw8(4 * kq + i, c16)) = R[i];
      char* lt = lw + kW;
      *reinterpret_cast<u32x4*>(lt + swz(lrow, lc)) = R[4];
      if (tid < kBM) reinterpret_cast<uint32_t*>(lt + kT)[tid] = Sc[1];
      if (tid < 32) reinterpret_cast<uint8_t*>(lt + kT + kSc)[tid] = uint8_t(Sc[0]);
    };
    auto compute = [&](int buf, auto nb_c) {
      constexpr int NB = decltype(nb_c)::value;
      const char* la = lds + buf * kStage;
      const char* lt = la + kW;
      const uint32_t* tsc = reinterpret_cast<const uint32_t*>(lt + kT);
      uint32_t ts[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) ts[b] = tsc[32 * b + lr];
      const uint32_t wsc = reinterpret_cast<const uint32_t*>(lt + kT + kSc)[wave];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int ga = 4 * q + lh, gb = 4 * q + 2 + lh;
        const int blk = 2 * q + lh;
        // this lane's 32 operand bytes: contraction chunks ga and gb (16 rows
        // each) of its output column, two 8-row transpose reads per chunk
        i32x2 pc[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int row = 16 * (p < 2 ? ga : gb) + 8 * (p & 1) + tr_row;
          pc[p] = lds_read_tr8(la + wsw8(row, tr_chunk) + tr_byte);
        }
        const u32x4 a0 = {uint32_t(pc[0][0]), uint32_t(pc[0][1]), uint32_t(pc[1][0]),
                          uint32_t(pc[1][1])};
        const u32x4 a1 = {uint32_t(pc[2][0]), uint32_t(pc[2][1]), uint32_t(pc[3][0]),
                          uint32_t(pc[3][1])};
        const int sa = byte_of(wsc, blk);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const u32x4 b0 = *reinterpret_cast<const u32x4*>(lt + swz(32 * b + lr, ga));
          const u32x4 b1 = *reinterpret_cast<const u32x4*>(lt + swz(32 * b + lr, gb));
          mfma_mx(acc[b], a0, a1, b0, b1, sa, byte_of(ts[b], blk));
        }
      }
    };

    // Same pipeline as the forward kernel.
    auto run = [&](auto nb_c) {
      load(R0, S0, 0, nb_c);
      load(R1, S1, min(1, S - 1), nb_c);
      store(R0, S0, 0, nb_c);
      load(R0, S0, min(2, S - 1), nb_c);
      lds_barrier();
      for (int s = 0; s + 1 < S; s += 2) {
        compute(0, nb_c);
        store(R1, S1, 1, nb_c);
        load(R1, S1, min(s + 3, S - 1), nb_c);
        lds_barrier();
        compute(1, nb_c);
        store(R0, S0, 0, nb_c);
        load(R0, S0, min(s + 4, S - 1), nb_c);
        lds_barrier();
      }
      if (S & 1) {
        compute(0, nb_c);
        lds_barrier();
      }
    };
    if (rows > 32)
      run(std::integral_constant<int, 2>{});
    else
      run(std::integral_constant<int, 1>{});
    between();

    const int col = nt * 256 + 32 * wave + 4 * lh;
#pragma unroll
    for (int b = 0; b < 2 && 32 * wave < ncols; ++b) {
      const int m = 32 * b + lr;
      if (m >= rows) continue;
      const int64_t row = row0 + m;
      if (KIND == 0) {
        const int F = a.F;
        uint16_t* o = reinterpret_cast<uint16_t*>(a.out0) + row * (2 * F);
        const uint16_t* hr = h1 + row * (2 * F);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int j = col + 8 * g4;
          float gv[4], uv[4], dg[4], du[4];
          load4_bf16(hr + j, gv);
          load4_bf16(hr + F + j, uv);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float dh2 = acc[b][4 * g4 + i];
            // clamped SwiGLU backward: no gradient through a clamped value
            const float L = a.limit;
            const float gc = clamp_gate(gv[i], L), uc = clamp_up(uv[i], L);
            const float sg = sigmoid_f(gc);
            dg[i] = gv[i] > L ? 0.0f : dh2 * uc * (sg * (1.0f + gc * (1.0f - sg)));
            du[i] = (uv[i] > L || uv[i] < -L) ? 0.0f : dh2 * silu_f(gc);
          }
          store4<uint16_t>(o + j, dg[0], dg[1], dg[2], dg[3]);
          store4<uint16_t>(o + F + j, du[0], du[1], du[2], du[3]);
        }
      } else {
        // dXr rows go to their route slots (contiguous K rows per token)
        float* o = reinterpret_cast<float*>(a.out0) + int64_t(a.sorted_route[row]) * N;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          store4<float>(o + col + 8 * g4, acc[b][4 * g4], acc[b][4 * g4 + 1], acc[b][4 * g4 + 2],
                        acc[b][4 * g4 + 3]);
      }
    }
  }
}

template <int KIND>
__global__ __launch_bounds__(512, 1) void k_mx_dgrad(MxArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kMxDgLds];
  const int tid = threadIdx.x;
  const RouteHdr* hdr = a.hdr;
  const int xcd = blockIdx.x % kXcds;
  const int per = gridDim.x / kXcds;
  // 64-row m-tiles (a.mtoff = a.stoff); the XCDs split the items by token rows
  const int first = xcd_first_tile(a.mtoff, a.stoff, a.E, a.NT, xcd);
  const int last = xcd_first_tile(a.mtoff, a.stoff, a.E, a.NT, xcd + 1);
  // items [first, last) of this XCD come from its work queue, in order
  // (with skewed routing: when some expert spans several m-tiles; otherwise
  // dealt statically, slot, slot + per, ..., which costs no atomics)
  const bool dyn = hdr->max_count > kBM;
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
    mx_dgrad_item<KIND>(a, lds, tid, e, nt, u - nt * mt_e, mt_e, [&] {
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
// A and B are column bundles: for expert e, the codes of column c are the Mp
// bytes at base + N*poffsets[e] + c*Mp (Mp = padded rows of e), exponents at
// sbase + N*poffsets[e]/32 + c*Mp/32.
__device__ __forceinline__ uint64_t rec_ptr_m(const RouteHdr* h, int slot) {
  if (slot == 6) return h->rec.x_rows;
  if (slot == 7) return h->rec.h1;
  return h->rec.aux[slot];
}

// Work item: 128 dW rows x 256 dW columns of one expert on eight waves,
// written as 512-byte (bf16) or 1 KB (fp32) row segments, which HBM takes
// faster than 256-byte ones.  Wave w owns dW rows 64 (w >> 2) .. + 63 and
// columns 64 (w & 3) .. + 63: 2 x 2 accumulators of 32 x 32.
// ACC: in-place accumulation (dW += result): the tile is staged in fp32 and
// each copied-out value is added to the dW value it replaces, rounded once.
// operand stages + output staging (64 bf16 rows or 32 fp32 rows of 256 values, padded)
constexpr int kMxWgLds = 256 * 64 + 128 * 64 + 64 * (256 * 2 + 16);

// The WGRAD items w0, w0 + step, ... below w1 (expert-major, NA x NB tiles
// per expert), each tile's first stage loaded while the previous tile is
// stored.  lds: kMxWgLds bytes.
template <typename TW, int TAG, int ACC>
__device__ __forceinline__ void mx_wgrad_run(const MxArgs& a, char* lds, int tid, int w0, int w1,
                                             int step) {
  typedef typename std::conditional<ACC != 0, float, TW>::type TS;   // staging type
  constexpr int kOpA = 256 * 64;                       // A stage: 256 columns x 64 rows
  constexpr int kOpB = 128 * 64;                       // B stage: 128 columns x 64 rows
  constexpr int kRowB = 256 * int(sizeof(TS)) + 16;    // padded output-staging row
  constexpr int kRowsPerPass = sizeof(TS) == 4 ? 32 : 64;
  constexpr int kPasses = 128 / kRowsPerPass;
  constexpr int kOut = kRowsPerPass * kRowB;
  static_assert(kOpA + kOpB + kOut <= kMxWgLds, "operand stages and output staging");
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wa = wave & 3;     // 64-column block of the tile
  const int wb = wave >> 2;    // 64-row block of the tile
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int ch = tid & 3;      // loader: 16-byte chunk of a 64-byte column segment
  const int lcol = tid >> 2;   // loader: A columns lcol, lcol + 128; B column lcol

  const RouteHdr* hdr = a.hdr;
  const int a_ld = a.a_ld, b_ld = a.b_ld;
  const int NA = (a_ld + 255) / 256, NB = b_ld / 128;
  const int per_e = NA * NB;
  const int last = w1, per = step;
  const uint8_t* qa = a.a_slot >= 0 ? global_ptr<const uint8_t>(rec_ptr_m(hdr, a.a_slot)) : a.qa;
  const uint8_t* sa = a.a_slot >= 0 ? global_ptr<const uint8_t>(rec_ptr_m(hdr, a.a_slot + 1)) : a.sa;
  const uint8_t* qb = a.qb;
  const uint8_t* sb = a.sb;

  struct Item {
    int e, ta, tb, pb, mp, S, ncols;
  };
  // Work items of this workgroup: w = w0 + i * per below last.
  int wcur = w0;
  auto fill = [&](Item& t) {
    int e = 0, p0 = 0, p1 = 0;
    for (;;) {   // with hot_wg, step over the hot experts' items
      if (wcur >= last) {
        t.e = -1;
        return;
      }
      e = wcur / per_e;
      // scalar loads (constant address space): no wait behind the previous
      // tile's dW stores, and one round trip per item
      const int o0 = ((kconst_i32*)a.offsets)[e], o1 = ((kconst_i32*)a.offsets)[e + 1];
      p0 = ((kconst_i32*)a.poffsets)[e];
      p1 = ((kconst_i32*)a.poffsets)[e + 1];
      if (!a.hot_wg || !hot_wgrad_expert(o1 - o0)) break;
      wcur += ((e + 1) * per_e - wcur + per - 1) / per * per;
    }
    const int w = wcur;
    wcur += per;
    t.e = e;
    t.pb = p0;
    t.mp = p1 - p0;
    t.S = (t.mp + 63) / 64;
    int ta, tb;
    wgrad_tile(w - e * per_e, NA, NB, TAG == 13 && hot_expert(t.mp), TAG == 2, ta, tb);
    t.ta = ta;
    t.tb = tb;
    t.ncols = min(256, a_ld - ta * 256);
  };
  // A column of the tile, folded into the first half past a 128-column half
  // tile's end (those columns are multiplied but never stored).
  auto acol = [&](const Item& t, int c) { return t.ta * 256 + (c < t.ncols ? c : c - 128); };

  u32x4 R[3];              // codes: A columns lcol, lcol + 128; B column lcol
  uint32_t SA[2], SB[2];   // exponents of this lane's MFMA rows for the stage
  auto load = [&](const Item& t, int s) {
    const int m0 = s * 64 + ch * 16;
    const bool in = m0 < t.mp;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      R[j] = in ? *reinterpret_cast<const u32x4*>(qa + int64_t(a_ld) * t.pb +
                                                  int64_t(acol(t, lcol + 128 * j)) * t.mp + m0)
                : u32x4{0u, 0u, 0u, 0u};
    R[2] = in ? *reinterpret_cast<const u32x4*>(qb + int64_t(b_ld) * t.pb +
                                                int64_t(t.tb * 128 + lcol) * t.mp + m0)
              : u32x4{0u, 0u, 0u, 0u};
    const int mb = 2 * s + lh;   // MX block of this lane's half of the stage
    const int nmb = t.mp / 32;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      SA[i] = 127;
      SB[i] = 127;
      if (mb < nmb) {
        SA[i] = sa[int64_t(a_ld) * (t.pb / 32) + int64_t(acol(t, 64 * wa + 32 * i + lr)) * nmb + mb];
        SB[i] = sb[int64_t(b_ld) * (t.pb / 32) + int64_t(t.tb * 128 + 64 * wb + 32 * i + lr) * nmb +
                   mb];
      }
    }
  };
  uint32_t sa_cur[2] = {127, 127}, sb_cur[2] = {127, 127};
  auto store = [&]() {
#pragma unroll
    for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4*>(lds + swz64(lcol + 128 * j, ch)) = R[j];
    *reinterpret_cast<u32x4*>(lds + kOpA + swz64(lcol, ch)) = R[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      sa_cur[i] = SA[i];
      sb_cur[i] = SB[i];
    }
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
      u32x4 a0[2], a1[2];
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
        a0[aa] = *reinterpret_cast<const u32x4*>(lds + swz64(64 * wa + 32 * aa + lr, lh));
        a1[aa] = *reinterpret_cast<const u32x4*>(lds + swz64(64 * wa + 32 * aa + lr, 2 + lh));
      }
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(lds + kOpA + swz64(64 * wb + 32 * bb + lr, lh));
        const u32x4 b1 =
            *reinterpret_cast<const u32x4*>(lds + kOpA + swz64(64 * wb + 32 * bb + lr, 2 + lh));
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
          mfma_mx(acc[bb][aa], a0[aa], a1[aa], b0, b1, int(sa_cur[aa]), int(sb_cur[bb]));
      }
      lds_barrier();
    }
    if (cur.S == 0 && nxt.e >= 0 && nxt.S > 0) load(nxt, 0);

    // acc[bb][aa][v] = dW[b = tb*128 + 64*wb + 32*bb + lr]
    //                    [a = ta*256 + 64*wa + 32*aa + 8*(v/4) + 4*lh + v%4]
    TW* o = reinterpret_cast<TW*>(a.out0) + (int64_t(cur.e) * b_ld + int64_t(cur.tb) * 128) * a_ld +
            cur.ta * 256;
    char* stg = lds + kOpA + kOpB;
#pragma unroll
    for (int h = 0; h < kPasses; ++h) {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int r = 64 * wb + 32 * bb;   // first tile row of this accumulator pair
        if (r / kRowsPerPass != h) continue;
        const int rl = r + lr - h * kRowsPerPass;
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
          TS* rowp = reinterpret_cast<TS*>(stg + rl * kRowB) + 64 * wa + 32 * aa + 4 * lh;
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
          const u32x4 v = *reinterpret_cast<const u32x4*>(stg + rl * kRowB + cc * 16);
          if (ACC) {   // four fp32 results onto the four dW values they update
            float f[4] = {__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                          __uint_as_float(v[3])};
            acc_store4(o + int64_t(rl + h * kRowsPerPass) * a_ld + cc * 4, f);
          } else {
            char* dst = reinterpret_cast<char*>(o + int64_t(rl + h * kRowsPerPass) * a_ld) + cc * 16;
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
__global__ __launch_bounds__(512, 1) void k_mx_wgrad(MxArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kMxWgLds];
  const int per_e = ((a.a_ld + 255) / 256) * (a.b_ld / 128);
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int per = gridDim.x / kXcds;
  // with hot_wg the experts of kHotWgRows rows or more are k_mx_wgrad_hot's:
  // split by the other experts' stages (theirs count 0, plus 1 per item)
  const int32_t* cost = a.hot_wg ? a.cst : a.mtoff;
  const int first = xcd_first_item(cost, a.E, per_e, xcd);
  const int last = xcd_first_item(cost, a.E, per_e, xcd + 1);
  mx_wgrad_run<TW, TAG, ACC>(a, lds, threadIdx.x, first + slot, last, per);
}

// ------------------------------------------------------------------ WGRAD, hot experts
// An expert with at least kHotWgRows rows contracts its weight gradient over
// hundreds to thousands of token rows: MFMA-bound work ("Mixture of Experts:
// How Routing Becomes GPU Computation", section 1 arithmetic intensity),
// for which the streaming 128 x 256 tile with one register-staged stage in
// flight waits on every stage's loads.  As k_wgrad_hot does for BF16, a work
// item here is a 256 x 256 dW tile: eight waves, wave (wa, wb) owning dW
// rows 128 wb .. + 127 and columns 64 wa .. + 63 as 4 x 2 accumulators of
// v_mfma_scale_f32_32x32x64_f8f6f4 (one MFMA step per 64-token stage).  A
// stage holds 64 tokens of the 256 A and 256 B columns of the tile (E4M3
// codes, one 64-byte LDS row per column, chunks XOR-swizzled by
// (column >> 1) & 3) and, per column, the aligned 8-byte window of its
// exponent bytes that holds the stage's two MX blocks; both are moved by
// direct global-to-LDS loads (dma16 / dma4), three stages in flight in four
// LDS buffers.  The last stage of an expert whose padded rows end half-way
// through it loads in-range chunks in place of the missing ones and zeroes
// both operands' codes there, and blocks past the expert's end take scale
// 2^0, as the streaming tiles do: both contract the same tokens in the same
// MFMA steps, so their gradients are bit-identical.  The tile is staged
// through LDS in eight passes of 32 rows and written as whole 512-byte row
// segments, non-temporally.  Items: the hot experts' tiles, split over the
// XCDs by their 64-row stage counts, 4 x 8 blocks of tiles where the grid
// allows (wgrad_tile); k_mx_wgrad skips these experts (MxArgs::hot_wg).
template <int TAG>
__global__ __launch_bounds__(512, 1) void k_mx_wgrad_hot(MxArgs a) {
  constexpr int kSeg = 64;                   // codes per column and stage (bytes)
  constexpr int kOp = 256 * kSeg;            // one operand's codes: 256 columns x 64 bytes
  constexpr int kExp = 256 * 8;              // one operand's exponent windows
  constexpr int kBuf = 2 * kOp + 2 * kExp;   // a stage buffer: A, B codes, A, B windows
  constexpr int kNb = 4;                     // stage buffers: three stages in flight
  constexpr int kPitch = 512 + 16;           // output-staging row (bf16), padded
  static_assert((kNb & (kNb - 1)) == 0, "buffer index by mask");
  __shared__ __attribute__((aligned(1024))) char lds[kNb * kBuf];   // stage s in buffer s mod 4
  static_assert(32 * kPitch <= kBuf, "a 32-row output pass fits one buffer");
  auto buf = [&](int s) { return lds + (s & (kNb - 1)) * kBuf; };
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wa = wave & 3;    // 64-column block of the tile
  const int wb = wave >> 2;   // 128-row block of the tile
  const int lr = lane & 31;
  const int lh = lane >> 5;

  const RouteHdr* hdr = a.hdr;
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
  const uint8_t* qa = a.a_slot >= 0 ? global_ptr<const uint8_t>(rec_ptr_m(hdr, a.a_slot)) : a.qa;
  const uint8_t* sa = a.a_slot >= 0 ? global_ptr<const uint8_t>(rec_ptr_m(hdr, a.a_slot + 1)) : a.sa;
  // exponent bytes of each bundle: one per column and 32 padded rows, all
  // experts (the launcher keeps these offsets, and a tile's code offsets,
  // below 2^31)
  const uint32_t nblk = uint32_t(a.poffsets[E]) / 32;
  const uint32_t sa_end = uint32_t(a_ld) * nblk, sb_end = uint32_t(b_ld) * nblk;

  // loader roles: waves 0-3 fill the A codes and windows, 4-7 the B ones.
  // Codes: instruction i (< 4) fills columns 64 (v & 3) + 16 i + (lane >> 2),
  // LDS slot lane & 3, which holds global chunk (lane & 3) ^ ((lane >> 3) & 3)
  // (the column's swizzle).  Windows: instruction k (< 2) fills dword lane & 1
  // of column 64 (v & 3) + 32 k + (lane >> 1).
  const bool aload = wave < 4;
  const int vq = wave & 3;
  const int lcol = 64 * vq + (lane >> 2);   // + 16 i
  const int lchunk = (lane & 3) ^ ((lane >> 3) & 3);
  const int ecol = 64 * vq + (lane >> 1);   // + 32 k
  const int edw = lane & 1;
  const uint8_t* qsrc = aload ? qa : a.qb;
  const uint8_t* ssrc = aload ? sa : a.sb;
  const uint32_t s_end = aload ? sa_end : sb_end;
  const int ld = aload ? a_ld : b_ld;

  // this workgroup's units are w0, w0 + per, ...: the first of them, from
  // w on, that belongs to a hot expert (last: none)
  auto next_hot = [&](int w) {
    while (w < last) {
      const int e = w / per_e;
      if (hot_wgrad_expert(a.offsets[e + 1] - a.offsets[e])) return w;
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
    int e, ta, tb, mp, nmb, S;
    const uint8_t* qbase;   // this wave's operand codes: the tile's first column, first token
    uint32_t sbase;         // this wave's operand exponents: offset of the tile's first column
    uint32_t a_ex, b_ex;    // the same for the A and B columns the MFMAs read
  };
  auto decode = [&](int w, Item& t) {
    const int e = w / per_e;
    const int pb = a.poffsets[e];
    t.e = e;
    t.mp = a.poffsets[e + 1] - pb;
    t.nmb = t.mp / 32;
    t.S = (t.mp + 63) / 64;
    wgrad_tile(w - e * per_e, NA, NB, true, false, t.ta, t.tb);
    const int col0 = (aload ? t.ta : t.tb) * 256;
    t.qbase = qsrc + int64_t(ld) * pb + int64_t(col0) * t.mp;
    t.sbase = uint32_t(ld) * uint32_t(pb / 32) + uint32_t(col0) * uint32_t(t.nmb);
    t.a_ex = uint32_t(a_ld) * uint32_t(pb / 32) + uint32_t(t.ta * 256) * uint32_t(t.nmb);
    t.b_ex = uint32_t(b_ld) * uint32_t(pb / 32) + uint32_t(t.tb * 256) * uint32_t(t.nmb);
  };
  // exponent window of a column for stage s: the aligned 8 bytes that hold
  // its blocks 2 s and 2 s + 1, moved back to lie inside the array
  auto window = [&](uint32_t off, uint32_t end) { return min(off & ~3u, end - 8u); };
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(lds));   // LDS byte address
  // stage s of item t into its buffer: four 1 KiB code loads and two
  // 256-byte window loads per wave
  auto issue = [&](const Item& t, int s) {
    const uint32_t b0 = lds0 + (s & (kNb - 1)) * kBuf;
    const uint32_t dq = b0 + (aload ? 0 : kOp) + vq * 64 * kSeg;
    const int g = 16 * lchunk < t.mp - 64 * s ? lchunk : lchunk - 2;   // in-range chunk
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma16(t.qbase + (uint32_t(lcol + 16 * i) * uint32_t(t.mp) + uint32_t(64 * s + 16 * g)),
            __builtin_amdgcn_readfirstlane(dq + i * 1024));
    const uint32_t de = b0 + 2 * kOp + (aload ? 0 : kExp) + vq * 64 * 8;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t off = t.sbase + uint32_t(ecol + 32 * k) * uint32_t(t.nmb) + uint32_t(2 * s);
      dma4(ssrc + (window(off, s_end) + 4u * edw), __builtin_amdgcn_readfirstlane(de + k * 256));
    }
  };

  Item cur, nxt;
  int w = next_hot(first + slot);
  int pre = 0;   // stages of cur that the previous item issued (into buffers 0, 1)
  while (w < last) {
    decode(w, cur);
    const int S = cur.S;
    const bool half = cur.mp - 64 * (S - 1) == 32;   // the last stage holds 32 tokens
    // zero the codes of tokens 32..63 of both operands in the last stage
    auto zero_half = [&](char* b) {
      for (int i = tid; i < 2 * 256 * 2; i += 512) {
        const int r = i >> 1, c = 2 + (i & 1);   // code row (A then B), chunk
        *reinterpret_cast<u32x4*>(b + r * kSeg + ((c ^ ((r >> 1) & 3)) << 4)) =
            u32x4{0u, 0u, 0u, 0u};
      }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    auto compute = [&](const char* b, int s) {
      const char* la = b;
      const char* lb = b + kOp;
      const char* ea = b + 2 * kOp;
      const char* eb = ea + kExp;
      const int sw = (lr >> 1) & 3;   // the swizzle of every row this lane reads
      const bool live = 2 * s + lh < cur.nmb;   // this lane's block inside the expert
      u32x4 a0[2], a1[2];
      int xa[2];
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
        const int c = 64 * wa + 32 * aa + lr;
        a0[aa] = *reinterpret_cast<const u32x4*>(la + c * kSeg + ((lh ^ sw) << 4));
        a1[aa] = *reinterpret_cast<const u32x4*>(la + c * kSeg + (((2 + lh) ^ sw) << 4));
        const uint32_t off = cur.a_ex + uint32_t(c) * uint32_t(cur.nmb) + uint32_t(2 * s);
        const int pos = int(off - window(off, sa_end)) + lh;
        xa[aa] = live ? int(*reinterpret_cast<const uint8_t*>(ea + c * 8 + pos)) : 127;
      }
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int c = 128 * wb + 32 * bb + lr;
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(lb + c * kSeg + ((lh ^ sw) << 4));
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(lb + c * kSeg + (((2 + lh) ^ sw) << 4));
        const uint32_t off = cur.b_ex + uint32_t(c) * uint32_t(cur.nmb) + uint32_t(2 * s);
        const int pos = int(off - window(off, sb_end)) + lh;
        const int xb = live ? int(*reinterpret_cast<const uint8_t*>(eb + c * 8 + pos)) : 127;
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) mfma_mx(acc[bb][aa], a0[aa], a1[aa], b0, b1, xa[aa], xb);
        // at most two B blocks' operands live at once (register pressure)
        if (bb == 1) __builtin_amdgcn_sched_barrier(0);
      }
    };
    // Three stages in flight, as in k_wgrad_hot: step s waits until this
    // wave's loads of stage s have landed (six per wave per stage; loads
    // complete in issue order), then for every wave (which also ends every
    // wave's reads of stage s - 1), issues stage s + 3 into the buffer stage
    // s - 1 used, and multiplies.  Stores may complete out of order with
    // loads, so an item that follows a tile's stores first waits for
    // everything.
    if (pre) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    for (int st = pre; st < min(kNb - 1, S); ++st) issue(cur, st);
    for (int s = 0; s < S; ++s) {
      const int after = min(S - 1 - s, kNb - 2);   // stages in flight behind stage s
      if (after >= 2)
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 | 12);
      else if (after == 1)
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 | 6);
      else
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      stage_barrier();
      if (s + 1 == S && half) {
        zero_half(buf(s));
        stage_barrier();
      }
      if (s + kNb - 1 < S) issue(cur, s + kNb - 1);
      compute(buf(s), s);
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
    uint16_t* o = reinterpret_cast<uint16_t*>(a.out0) +
                  (int64_t(cur.e) * b_ld + int64_t(cur.tb) * 256) * a_ld + cur.ta * 256;
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      char* sbp = buf(kNb - 2 + (h & 1));
      if (wb == h / 4) {
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
          uint16_t* rowp = reinterpret_cast<uint16_t*>(sbp + lr * kPitch) + 64 * wa + 32 * aa + 4 * lh;
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
        const u32x4 v = *reinterpret_cast<const u32x4*>(sbp + rl * kPitch + cc * 16);
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
// explainer, section 05, Mega backward; section 0: the MXFP8 backward as
// two fused expert operations, W2 then W13, then the input-gradient
// reduction).  Both records of a projection read operands that exist before
// the launch (W2: the dH3 row blocks and column bundle and the saved or
// rebuilt h2 column bundle; W13: the dH1 row blocks and column bundle and
// the x column bundle), so no record waits for another.  Scheduling as in
// the BF16 fused backward: units of one 256-column weight block of an
// expert (the DGRAD records of that n-tile, one per 64-row m-tile, and
// NB dW items of the streaming WGRAD order), split over the XCDs by their
// 64-row stages + kMxMegaBwdCw, each XCD's queue holding the DGRAD records
// of unit j and the WGRAD records of unit j - look (look = the XCD's
// workgroups), a WGRAD record being about kMxWgRecordStages stages of work.
// A workgroup takes its next ticket as it starts a record.  Tickets are
// zeroed by the backward's planner launch.
constexpr int kMxWgRecordStages = 16;   // 64-row stages of work per WGRAD record (>= 1 tile)
constexpr int kMxMegaBwdCw = 3;         // XCD split: a unit's fixed cost, in 64-row stages

template <int KIND, typename TW, int ACC>
__global__ __launch_bounds__(512, 1) void k_mx_bwd_mega(MxArgs dg, MxArgs wg, uint32_t* tickets,
                                                        int look) {
  constexpr int TAG = KIND == 0 ? 2 : 13;
  __shared__ __attribute__((aligned(16))) char lds[kMxDgLds > kMxWgLds ? kMxDgLds : kMxWgLds];
  __shared__ int s_t;
  __shared__ int s_wp[kMaxE + 1];   // WGRAD records per unit of the experts before e (E <= kMaxE)
  __shared__ int s_part[512];
  const int tid = threadIdx.x;
  const int E = dg.E;
  const int32_t* gt = dg.mtoff;   // DGRAD m-tile prefix (64-row m-tiles)
  const int NU = dg.NT;           // units per expert: 256-column weight blocks
  const int NBw = wg.b_ld / 128;  // dW items per unit
  const int per_e = ((wg.a_ld + 255) / 256) * NBw;
  // dW tiles per WGRAD record of expert e, and records per unit
  auto group = [&](int e) {
    const int S = (wg.poffsets[e + 1] - wg.poffsets[e] + 63) / 64;
    return S <= 1 ? kMxWgRecordStages : max(1, kMxWgRecordStages / S);
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
  const int u_lo = xcd_first_unit(wg.mtoff, kMxMegaBwdCw, E, NU, xcd);
  const int u_hi = xcd_first_unit(wg.mtoff, kMxMegaBwdCw, E, NU, xcd + 1);
  const int nu = u_hi - u_lo;
  // DGRAD and WGRAD records before unit u
  auto dpre = [&](int u) {
    const int e = u / NU, nt = u - e * NU;
    return gt[e] * NU + (e < E ? nt * (gt[e + 1] - gt[e]) : 0);
  };
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
  // one ticket per workgroup: uniform, so everything derived from it is scalar
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
    // lane constants from an opaque copy of the thread index: hoisted out of
    // the record loop, the two record kinds' constants would be live at once
    int rtid = tid;
    asm volatile("" : "+v"(rtid));
    if (dgr) {
      mx_dgrad_item<KIND>(dg, lds, rtid, e, nt, r, gt[e + 1] - gt[e], [] {});
    } else {
      const int G = group(e);
      const int b0 = r * G;
      const int w = e * per_e + nt * NBw;
      mx_wgrad_run<TW, TAG, ACC>(wg, lds, rtid, w + b0, w + min(NBw, b0 + G), 1);
    }
    if (tid == 0) s_t = nxt_t;
    lds_barrier();
    t = __builtin_amdgcn_readfirstlane(s_t);
  }
}

// ------------------------------------------------------------------ launchers
template <int ID, typename K>
static int occupancy_m(K kernel, int threads = 256) {
  static int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n <= 0)
      n = 1;
    per_cu = n;
  }
  return per_cu;
}

static unsigned grid_m(int per_cu, int64_t items, int cus) {
  int64_t g = std::min<int64_t>(items, int64_t(cus) * per_cu);
  g = (g + kXcds - 1) / kXcds * kXcds;
  return unsigned(std::max<int64_t>(g, kXcds));
}

// Stage buffers of the MXFP8 (32x32) forward passes' direct-load ring.
constexpr int kMxRing = 4;

// mode 0: W13 (+ SwiGLU), 1: W2 -> slots
hipError_t launch_mx_fwd(int mode, const MxArgs& a, int64_t mt_max, int cus, hipStream_t s) {
  if (mt_max == 0) return hipSuccess;
#define MOE_MXF(M, W, P, R, ID)                                                                   \
  hipLaunchKernelGGL((k_mx_fwd<M, W, P, R>),                                                     \
                     dim3(grid_m(occupancy_m<ID>(k_mx_fwd<M, W, P, R>), mt_max * a.NT, cus)), \
                     dim3(256), 0, s, a, a, nullptr, 0)
  if (mode == 0) {
    if (a.fp4) MOE_MXF(0, 1, 1, 0, 14); else if (a.w1x32) MOE_MXF(0, 1, 0, 0, 12); else MOE_MXF(0, 0, 0, kMxRing, 0);
  } else {
    if (a.fp4) MOE_MXF(1, 1, 1, 0, 15); else if (a.w1x32) MOE_MXF(1, 1, 0, 0, 13); else MOE_MXF(1, 0, 0, kMxRing, 1);
  }
#undef MOE_MXF
  return hipGetLastError();
}

// Fused (Mega) MX forward: a13 = the W13 records' arguments, a2 = the W2
// records'; msync = tickets and per-expert counters, zeroed before the call.
hipError_t launch_mx_mega(const MxArgs& a13, const MxArgs& a2, uint32_t* msync, int look,
                          int64_t mt_max, int cus, hipStream_t s) {
  if (mt_max == 0) return hipSuccess;
  const int64_t items = mt_max * (a13.NT + a2.NT);
#define MOE_MXM(W, P, ID)                                                                     \
  hipLaunchKernelGGL((k_mx_fwd<2, W, P>),                                                     \
                     dim3(grid_m(occupancy_m<ID>(k_mx_fwd<2, W, P>), items, cus)),           \
                     dim3(256), 0, s, a13, a2, msync, look)
  if (a13.fp4) MOE_MXM(1, 1, 18); else if (a13.w1x32) MOE_MXM(1, 0, 17); else MOE_MXM(0, 0, 16);
#undef MOE_MXM
  return hipGetLastError();
}

// kind 0: W2 DGRAD + SwiGLU backward; 1: W13 DGRAD
hipError_t launch_mx_dgrad(int kind, const MxArgs& a, int64_t mt_max, int cus, hipStream_t s) {
  if (mt_max == 0) return hipSuccess;
  if (kind == 0) {
    hipLaunchKernelGGL(k_mx_dgrad<0>,
                       dim3(grid_m(occupancy_m<2>(k_mx_dgrad<0>, 512), mt_max * a.NT, cus)),
                       dim3(512), 0, s, a);
  } else {
    hipLaunchKernelGGL(k_mx_dgrad<1>,
                       dim3(grid_m(occupancy_m<3>(k_mx_dgrad<1>, 512), mt_max * a.NT, cus)),
                       dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

// tag 2: dW2, 13: dW13
hipError_t launch_mx_wgrad(int dw_f32, int tag, const MxArgs& args, int cus, hipStream_t s) {
  const int64_t items = int64_t(args.E) * ((args.a_ld + 255) / 256) * (args.b_ld / 128);
  if (items == 0) return hipSuccess;
  // the hot experts go to k_mx_wgrad_hot only where it applies; otherwise
  // every expert stays on k_mx_wgrad
  MxArgs a = args;
  a.hot_wg = (args.hot_wg && args.cst && !dw_f32 && !args.acc_dw && args.a_ld % 256 == 0 &&
              args.b_ld % 256 == 0) ? 1 : 0;
#define MOE_MXWG(TW, TAG, ACC, ID)                                                            \
  do {                                                                                      \
    const unsigned g = grid_m(occupancy_m<ID>(k_mx_wgrad<TW, TAG, ACC>, 512), items, cus);  \
    hipLaunchKernelGGL((k_mx_wgrad<TW, TAG, ACC>), dim3(g), dim3(512), 0, s, a);           \
  } while (0)
  const int acc = a.acc_dw ? 1 : 0;
  if (dw_f32) {
    if (tag == 2) {
      if (acc) MOE_MXWG(float, 2, 1, 8); else MOE_MXWG(float, 2, 0, 4);
    } else {
      if (acc) MOE_MXWG(float, 13, 1, 9); else MOE_MXWG(float, 13, 0, 5);
    }
  } else {
    if (tag == 2) {
      if (acc) MOE_MXWG(uint16_t, 2, 1, 10); else MOE_MXWG(uint16_t, 2, 0, 6);
    } else {
      if (acc) MOE_MXWG(uint16_t, 13, 1, 11); else MOE_MXWG(uint16_t, 13, 0, 7);
    }
  }
#undef MOE_MXWG
  if (a.hot_wg) {   // the hot experts' 256 x 256 tiles
    const unsigned g = grid_m(1, int64_t(cus), cus);
    if (tag == 2)
      hipLaunchKernelGGL(k_mx_wgrad_hot<2>, dim3(g), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL(k_mx_wgrad_hot<13>, dim3(g), dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

// Fused backward of one projection (block-scaled): kind 0 = W2 (DGRAD +
// SwiGLU backward records with dg, dW2 records with wg), 1 = W13 (dX rows,
// dW13).  tickets: kXcds counters.
hipError_t launch_mx_bwd_mega(int kind, int dw_f32, const MxArgs& dg, const MxArgs& wg,
                              uint32_t* tickets, int cus, hipStream_t s) {
  // units: the DGRAD n-tiles are the dW column tiles (NT x NB dW items per expert)
  if (dg.NT != (wg.a_ld + 255) / 256) return hipErrorInvalidValue;
  const unsigned g = grid_m(1, int64_t(cus), cus);
  const int look = int(g / kXcds);   // the XCD's workgroups
  const int acc = wg.acc_dw ? 1 : 0;
#define MOE_MXB(K, TW, ACC) \
  hipLaunchKernelGGL((k_mx_bwd_mega<K, TW, ACC>), dim3(g), dim3(512), 0, s, dg, wg, tickets, look)
  if (kind == 0) {
    if (dw_f32) {
      if (acc) MOE_MXB(0, float, 1); else MOE_MXB(0, float, 0);
    } else {
      if (acc) MOE_MXB(0, uint16_t, 1); else MOE_MXB(0, uint16_t, 0);
    }
  } else {
    if (dw_f32) {
      if (acc) MOE_MXB(1, float, 1); else MOE_MXB(1, float, 0);
    } else {
      if (acc) MOE_MXB(1, uint16_t, 1); else MOE_MXB(1, uint16_t, 0);
    }
  }
#undef MOE_MXB
  return hipGetLastError();
}

}  // namespace moe
