// MXFP8 producers: E4M3 values with one E8M0 power-of-two scale per 32
// values (Dist-MoE explainer, section 02: the producer picks the scale,
// rounds the values and publishes both; MXFP8 training quantizes BF16 rows
// after the gather; forward GEMMs take scales along the contraction (1x32
// row blocks), weight gradients take column bundles (32x1 blocks down an
// expert's token rows), static weights use 32x32 blocks).
//
//   k_prep_w : W [E, N, K] bf16 -> q [E, N, K] e4m3, s [E, N/32, K/32] e8m0
//   k_rowq   : rows [R, N] bf16 -> q [R, N], s [R, N/32]           (1x32)
//              (MXFP4: q [R, N/2], two E2M1 codes per byte)
//   k_colq   : rows [R, N] bf16 -> per expert e, q^T [N, Mp_e] and
//              s^T [N, Mp_e/32] at offsets N*poffsets[e] and N*poffsets[e]/32,
//              Mp_e = counts[e] rounded up to 32, pad rows quantized as 0.
//
// Scale rule: e = the smallest integer with amax <= 448 * 2^e, clamped to
// [-127, 127] (-127 for an all-zero block), stored as the byte e + 127.  With
// it no scaled value exceeds 448, the largest E4M3 magnitude.  E4M3 here is
// the finite-only variant (bias 7, subnormals to 2^-9); values are rounded to
// nearest, ties to even.
#include <algorithm>

#include "common.h"
#include "mxq.h"

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ weights
// One workgroup per (expert, 32-row block, 256 columns): thread = column.
__global__ __launch_bounds__(256) void k_prep_w(const uint16_t* __restrict__ w,
                                                uint8_t* __restrict__ q, uint8_t* __restrict__ s,
                                                int N, int K) {
  const int kc = blockIdx.x * 256 + threadIdx.x;     // column
  const int nb = blockIdx.y;                         // 32-row block
  const int64_t e = blockIdx.z;
  if (kc >= K) return;
  const uint16_t* src = w + (e * N + int64_t(nb) * 32) * K + kc;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    v[r] = bf16_to_f32(src[int64_t(r) * K]);
    amax = fmaxf(amax, fabsf(v[r]));
  }
  // 32x32 block = 32 consecutive columns = half a wave
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const int ex = e8m0_exp(amax);
  uint8_t* dst = q + (e * N + int64_t(nb) * 32) * K + kc;
#pragma unroll
  for (int r = 0; r < 32; ++r) dst[int64_t(r) * K] = uint8_t(e4m3_rne(ldexp_i(v[r], -ex)));
  if ((threadIdx.x & 31) == 0) s[(e * (N / 32) + nb) * (K / 32) + kc / 32] = uint8_t(ex + 127);
}

// ------------------------------------------------------------------ rows (1x32)
// Pointers may come from the layer record (slots 0..5 = aux, 6 = x rows, 7 = h1).
__device__ __forceinline__ uint64_t rec_ptr(const RouteHdr* h, int slot) {
  if (slot == 6) return h->rec.x_rows;
  if (slot == 7) return h->rec.h1;
  return h->rec.aux[slot];
}

// Lane = 8 consecutive values; 4 lanes = one block.  A wave covers 512
// values of a row per step.  FP4: E2M1 codes, value 2i in the low nibble of
// byte i (the order in which the scaled MFMA reads a 4-bit operand).
template <int FP4>
__global__ __launch_bounds__(256) void k_rowq(RowqArgs a) {
  const RouteHdr* hdr = a.hdr;
  if (a.replay_only && !hdr->rec.replay) return;
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= (a.rows > 0 ? a.rows : int64_t(hdr->R))) return;
  const uint16_t* src = a.src_slot >= 0 ? global_ptr<const uint16_t>(rec_ptr(hdr, a.src_slot))
                                         : reinterpret_cast<const uint16_t*>(a.src);
  uint8_t* q = a.q_slot >= 0 ? global_ptr<uint8_t>(rec_ptr(hdr, a.q_slot)) : a.q;
  uint8_t* s = a.s_slot >= 0 ? global_ptr<uint8_t>(rec_ptr(hdr, a.s_slot)) : a.s;
  if (!src) {  // rows to quantize need their source: report instead of faulting
    if (row == 0 && lane == 0) atomicOr(const_cast<uint32_t*>(&hdr->status), MOE_STATUS_NULL_INPUT);
    return;
  }
  const int N = a.N;
  const int64_t srow = a.gather ? a.gather[row] / a.K : row;
  for (int c0 = lane * 8; c0 < N; c0 += 512) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(src + srow * N + c0);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(raw[i] << 16);
      v[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const int ex = FP4 ? e8m0_exp_fp4(amax) : e8m0_exp(amax);
    if (FP4) {
      uint32_t wv = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) wv |= e2m1_rne(ldexp_i(v[i], -ex)) << (4 * i);
      *reinterpret_cast<uint32_t*>(q + row * (N / 2) + c0 / 2) = wv;
    } else {
      u32x2 out;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t wv = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) wv |= e4m3_rne(ldexp_i(v[4 * h + i], -ex)) << (8 * i);
        out[h] = wv;
      }
      *reinterpret_cast<u32x2*>(q + row * N + c0) = out;
    }
    if ((lane & 3) == 0) {
      constexpr int G = FP4 ? 256 : 128;     // values per stage of the grouped layout
      const int64_t si = a.s_rows ? (int64_t(c0 / G) * a.s_rows + row) * (G / 32) + (c0 / 32) % (G / 32)
                                  : row * (N / 32) + c0 / 32;
      s[si] = uint8_t(ex + 127);
    }
  }
}

// ------------------------------------------------------------------ column bundles (32x1)
// One workgroup per (32-row block of the padded row space, 1,024 columns),
// one 256-column tile at a time.  A tile's rows are loaded row-wise with
// 16-byte loads (32 lanes per 512-byte row segment) into LDS; then each
// thread takes one column, reads its 32 values from LDS, and writes 32
// contiguous code bytes and one exponent.
constexpr int kColTiles = 4;   // 256-column tiles per k_colq workgroup

__global__ __launch_bounds__(256) void k_colq(ColqArgs a) {
  constexpr int kRow = 256 + 8;              // LDS row pitch (bf16), 16-byte aligned
  __shared__ __attribute__((aligned(16))) uint16_t tile[32 * kRow];
  __shared__ int s_lo, s_e;
  const RouteHdr* hdr = a.hdr;
  // replay_only: 1 = run only when the layer replays, 2 = only when it saves
  if (a.replay_only == 1 && !hdr->rec.replay) return;
  if (a.replay_only == 2 && hdr->rec.replay) return;
  const int gb = blockIdx.x;                 // 32-row block in the padded row space
  const int key = gb * 32;
  if (key >= hdr->Rpad) return;
  const int tid = threadIdx.x;
  const int N = a.N;
  const uint16_t* src = a.src_slot >= 0 ? global_ptr<const uint16_t>(rec_ptr(hdr, a.src_slot))
                                         : reinterpret_cast<const uint16_t*>(a.src);
  uint8_t* q = a.q_slot >= 0 ? global_ptr<uint8_t>(rec_ptr(hdr, a.q_slot)) : a.q;
  uint8_t* s = a.s_slot >= 0 ? global_ptr<uint8_t>(rec_ptr(hdr, a.s_slot)) : a.s;
  if (!src) {
    if (gb == 0 && tid == 0 && blockIdx.y == 0)
      atomicOr(const_cast<uint32_t*>(&hdr->status), MOE_STATUS_NULL_INPUT);
    return;
  }
  // Expert of this block: the largest e < E with poffsets[e] <= key, found by
  // two rounds of parallel probes instead of a chain of dependent loads.
  const int E = a.E;
  const int step = (E + 255) / 256;
  if (tid == 0) {
    s_lo = 0;
    s_e = 0;
  }
  __syncthreads();
  if (tid * step < E && a.poffsets[tid * step] <= key) atomicMax(&s_lo, tid * step);
  __syncthreads();
  const int lo = s_lo;
  if (tid < step && lo + tid < E && a.poffsets[lo + tid] <= key) atomicMax(&s_e, lo + tid);
  __syncthreads();
  const int e = s_e;
  const int pbase = a.poffsets[e];
  const int mp = a.poffsets[e + 1] - pbase;
  const int mb = (key - pbase) / 32;         // block index inside the expert
  const int r0 = a.offsets[e] + mb * 32;
  const int rows = min(32, a.offsets[e + 1] - r0);

  // Column tiles of 256: this workgroup covers kColTiles of them with one
  // expert lookup; the next tile's rows are loaded while this one is
  // quantized.  Rows r = t/32 + 8j, 16-byte chunk t%32; rows past the
  // expert's end are zero.
  const int cc = tid & 31;
  u32x4 v8[4];
  auto load = [&](int c0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = (tid >> 5) + 8 * j;
      const int col = c0 + 8 * cc;
      v8[j] = u32x4{0u, 0u, 0u, 0u};
      if (r < rows && col < N) {
        const int64_t srow = a.gather ? a.gather[r0 + r] / a.K : r0 + r;
        v8[j] = *reinterpret_cast<const u32x4*>(src + srow * N + col);
      }
    }
  };
  const int cbase = blockIdx.y * (256 * kColTiles);
  load(cbase);
  for (int ct = 0; ct < kColTiles; ++ct) {
    const int c0 = cbase + 256 * ct;
    if (c0 >= N) break;   // uniform
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = (tid >> 5) + 8 * j;
      *reinterpret_cast<u32x4*>(tile + r * kRow + 8 * cc) = v8[j];
    }
    __syncthreads();
    if (ct + 1 < kColTiles && c0 + 256 < N) load(c0 + 256);
    const int col = c0 + tid;
    if (col < N) {
      float v[32];
      float amax = 0.0f;
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        v[r] = bf16_to_f32(tile[r * kRow + tid]);
        amax = fmaxf(amax, fabsf(v[r]));
      }
      const int ex = e8m0_exp(amax);
      u32x4 o0, o1;
#pragma unroll
      for (int w4 = 0; w4 < 8; ++w4) {
        uint32_t wv = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) wv |= e4m3_rne(ldexp_i(v[4 * w4 + i], -ex)) << (8 * i);
        if (w4 < 4)
          o0[w4] = wv;
        else
          o1[w4 - 4] = wv;
      }
      uint8_t* qd = q + int64_t(N) * pbase + int64_t(col) * mp + mb * 32;
      *reinterpret_cast<u32x4*>(qd) = o0;
      *reinterpret_cast<u32x4*>(qd + 16) = o1;
      s[int64_t(N) * (pbase / 32) + int64_t(col) * (mp / 32) + mb] = uint8_t(ex + 127);
    }
    __syncthreads();   // the tile is rewritten by the next column tile
  }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_prep_w(const void* w, void* q, void* s, int E, int N, int K, hipStream_t st) {
  if (E == 0) return hipSuccess;
  hipLaunchKernelGGL(k_prep_w, dim3((K + 255) / 256, N / 32, E), dim3(256), 0, st,
                     reinterpret_cast<const uint16_t*>(w), reinterpret_cast<uint8_t*>(q),
                     reinterpret_cast<uint8_t*>(s), N, K);
  return hipGetLastError();
}

hipError_t launch_rowq(const RowqArgs& a, int64_t R_max, hipStream_t st) {
  if (R_max == 0) return hipSuccess;
  if (a.fp4)
    hipLaunchKernelGGL(k_rowq<1>, dim3(unsigned((R_max + 3) / 4)), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_rowq<0>, dim3(unsigned((R_max + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_colq(const ColqArgs& a, int64_t Rpad_max, hipStream_t st) {
  if (Rpad_max == 0) return hipSuccess;
  hipLaunchKernelGGL(k_colq,
                     dim3(unsigned(Rpad_max / 32), unsigned((a.N + 256 * kColTiles - 1) / (256 * kColTiles))),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
