// Grouped forward GEMMs of hot experts on gfx950 MFMA (BF16).
//
//   W13 pass:  h1 = A_e W13_e^T, epilogue stores h1 = [g | u] and
//              h2 = SiLU(g) * u (clamped SwiGLU when a limit is set).
//   W2 pass:   h3 = H2_e W2_e^T, epilogue stores each row into its route slot
//              (or, FUSED, adds score * bf16(h3) into the token's fp32 row).
//
// Sources: Dist-MoE explainer section 02 (h1 = W13 x = [g; u],
// h2 = SiLU(g) * u, h3 = W2 h2) and section 05 (one launch covers the local
// experts, the W2 epilogue returns each result to its slot).  "Mixture of
// Experts: How Routing Becomes GPU Computation", section 1: an expert's
// GEMM does 2 M_e FLOPs per weight element, so once M_e is in the hundreds
// the work is bound by the matrix cores rather than by reading the weights.
//
// MI355X design
//  * Experts with at least kHotRows rows only (routing's hotoff prefix);
//    the others stay on the weight-streaming kernels of gemm_fwd.hip.
//  * Workgroup tile: 256 weight rows x 256 token rows, eight waves (two per
//    SIMD), each holding a 128 x 64 block as 4 x 2 fp32 accumulators of
//    v_mfma_f32_32x32x16_bf16 (128 accumulator registers).  Per 16-deep MFMA
//    step a wave reads 6 operands (16 bytes per lane) from LDS for 8 MFMAs.
//  * A stage is 128 bytes (64 values) of every tile row: 256 weight rows +
//    256 token rows = 64 KiB, moved by the gfx950 direct global-to-LDS load
//    (global_load_lds_dwordx4: a wave instruction writes 1 KiB of LDS, lane
//    l's 16 bytes at l * 16), so no registers stage it: waves 0-3 load the
//    weight rows, waves 4-7 the token rows, 8 rows per instruction with
//    eight lanes per 128-byte row segment.  Each lane fetches the chunk
//    that the XOR swizzle of the streaming kernels places at its LDS slot,
//    so the MFMA operand reads (32 rows, one chunk) are conflict-free.  The
//    next stage streams into the other of two LDS buffers (128 KiB) while
//    this one multiplies.
//  * W13 tiles hold 128 gate rows j and the 128 up rows F + j of the same j;
//    each wave owns 64 gate and the matching 64 up rows, so the SwiGLU
//    epilogue works on its own accumulators.
//  * Token rows past an expert's last row re-read that row (unconditional
//    loads); a wave whose 64 token rows are partly or wholly past the end
//    skips the MFMAs of its dead 32-row blocks (a wave-uniform branch).
//  * Persistent grid of one workgroup per CU; each XCD runs a contiguous run
//    of items ordered expert-major, then n-tile, then m-tile, so the m-tiles
//    of one expert that share a weight tile run side by side in one L2.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

__device__ __forceinline__ void st4(uint16_t* p, float a, float b, float c, float d) {
  u32x2 v;
  v[0] = pack_bf16x2(a, b);
  v[1] = pack_bf16x2(c, d);
  *reinterpret_cast<u32x2*>(p) = v;
}

}  // namespace

template <int MODE>
__global__ __launch_bounds__(512, 1) void k_gemm_hot(FwdArgs a) {
  constexpr int kHalf = 256 * 128;   // one operand's stage: 256 rows x 128 bytes
  // two stage buffers as separate objects, so the compiler can tell the
  // buffer being filled from the one being read
  __shared__ __attribute__((aligned(1024))) char lds0[2 * kHalf];
  __shared__ __attribute__((aligned(1024))) char lds1[2 * kHalf];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1;    // weight-row half of the tile
  const int wm = wave >> 1;   // token-row quarter of the tile
  const int lr = lane & 31;   // row inside a 32-row operand block
  const int lh = lane >> 5;   // operand half: chunks [4 lh, 4 lh + 4) of a stage row

  const RouteHdr* hdr = a.hdr;
  if (a.replay_only && !hdr->rec.replay) return;
  const int32_t* hot = a.hotoff;
  const int NT = a.NT;
  const int n_items = hot[a.E] * NT;
  if (n_items == 0) return;
  if (MODE == 0 && !a.x) {  // rows to compute need x: report instead of faulting
    if (blockIdx.x == 0 && threadIdx.x == 0)
      atomicOr(const_cast<uint32_t*>(&hdr->status), MOE_STATUS_NULL_INPUT);
    return;
  }
  const char* Abase = reinterpret_cast<const char*>(MODE == 0 ? a.x : a.A);
  uint16_t* out0 = a.out0 ? reinterpret_cast<uint16_t*>(a.out0) : global_ptr<uint16_t>(hdr->rec.h1);
  uint16_t* out1 = reinterpret_cast<uint16_t*>(a.out1);
  const int64_t row_bytes = int64_t(a.Kd) * 2;
  const int S = int(row_bytes / 128);

  const int xcd = blockIdx.x % kXcds;
  const int per = gridDim.x / kXcds;
  const int slot = blockIdx.x / kXcds;
  const int first = int(int64_t(n_items) * xcd / kXcds);
  const int last = int(int64_t(n_items) * (xcd + 1) / kXcds);

  // Loader lane roles: instruction i of wave v fills tile rows
  // 64 (v & 3) + 8 i + (lane >> 3) of the weights (v < 4) or of the tokens
  // (v >= 4), LDS chunk lane & 7, which holds global chunk
  // (lane & 7) ^ (lane >> 3) ^ (i & 7) of the row (the row's swizzle).
  const int lrow8 = lane >> 3;
  const int lchunk = (lane & 7) ^ lrow8;
  const bool wload = wave < 4;
  const int vq = wave & 3;
  const int vrow0 = 64 * vq + lrow8;   // first tile row of this lane (+ 8 i)
  // Operand reads: row base + lr, chunk (4 lh + q) stored at slot
  // (4 lh + q) ^ f with f = (lr & 7) ^ (lr >> 3) ^ (4 if the 32-row block
  // is odd): per-lane offsets for the 8 values of (q ^ block parity bits).
  const int fl = (lr & 7) ^ (lr >> 3);
  int rdoff[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) rdoff[v] = lr * 128 + (((4 * lh) ^ fl ^ v) << 4);

  int e_prev = -1;
  for (int w = first + slot; w < last; w += per) {
    const int e = item_expert(hot, a.E, NT, w, e_prev);
    e_prev = e;
    const int mt_e = hot[e + 1] - hot[e];
    const int u = w - hot[e] * NT;
    const int nt = u / mt_e;
    const int mt = u - nt * mt_e;
    const int row0 = a.offsets[e] + mt * kBMH;
    const int rows = min(kBMH, a.offsets[e + 1] - row0);

    // Sources: a uniform base plus a 32-bit per-lane byte offset (the
    // launcher checks that an expert's weights and the token rows span less
    // than 4 GiB).  Weight rows are linear in i within each half of the tile
    // (W13: gate rows nt*128 + rho, up rows F + nt*128 + rho - 128; W2:
    // output columns nt*256 + rho, N a multiple of 256); token rows are
    // gathered (W13) or clamped at the expert's last row.
    const char* gbase;
    uint32_t goff[8];
    if (wload) {
      gbase = reinterpret_cast<const char*>(a.W) + int64_t(e) * a.N * row_bytes;
      const int wr0 = MODE == 0 ? (vq < 2 ? nt * 128 + vrow0 : a.F + nt * 128 + vrow0 - 128)
                                : nt * 256 + vrow0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        goff[i] = uint32_t((wr0 + 8 * i) * row_bytes + ((lchunk ^ (i & 7)) << 4));
    } else {
      gbase = Abase;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = row0 + min(vrow0 + 8 * i, rows - 1);
        const int64_t src = MODE == 0 ? a.sorted_route[r] / a.K : r;
        goff[i] = uint32_t(src * row_bytes + ((lchunk ^ (i & 7)) << 4));
      }
    }
    // live 32-row token blocks of this wave's 64 rows (wave-uniform)
    const int nbl = __builtin_amdgcn_readfirstlane(min(2, max(0, (rows - wm * 64 + 31) >> 5)));

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    // stage s -> buffer: this wave's 8 instructions, 1 KiB each, at
    // operand half (waves 4-7: tokens) + rows 64 (wave & 3) + 8 i
    auto issue = [&](char* buf, int s) {
      const char* src = gbase + int64_t(s) * 128;
      char* dst = buf + (wload ? 0 : kHalf) + vq * 64 * 128;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_global_load_lds((gbl_void*)(src + goff[i]),
                                         (lds_void*)(dst + i * 1024), 16, 0, 0);
    };
    // weight row of the wave's 32-row block nb
    auto wrow = [&](int nb) {
      return MODE == 0 ? (nb < 2 ? wn * 64 + 32 * nb : 128 + wn * 64 + 32 * (nb - 2))
                       : wn * 128 + 32 * nb;
    };
    // Operands of MFMA step q are read while step q - 1 multiplies (two
    // operand sets); scheduling barriers keep the compiler from hoisting all
    // four steps' reads.
    auto compute = [&](const char* buf) {
      const char* tl = buf + kHalf;
      u32x4 av[2][4], bv[2][2];
      auto rd = [&](int q, int set) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rb = wrow(i);   // multiple of 32; bit 5 selects the swizzle's 4
          av[set][i] = *reinterpret_cast<const u32x4*>(buf + rb * 128 + rdoff[q ^ ((rb >> 3) & 4)]);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int rb = wm * 64 + 32 * j;
          bv[set][j] = *reinterpret_cast<const u32x4*>(tl + rb * 128 + rdoff[q ^ ((rb >> 3) & 4)]);
        }
      };
      rd(0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q < 3) rd(q + 1, (q + 1) & 1);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (j < nbl) {   // uniform: blocks past the expert's last row are skipped
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, av[q & 1][i]), __builtin_bit_cast(bf16x8, bv[q & 1][j]),
                  acc[i][j], 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // Pipeline: stage s multiplies from one buffer while stage s + 1 streams
    // into the other (last read by stage s - 1, before the previous barrier);
    // each pass ends when this wave's loads have landed and every wave is
    // past its MFMAs.  S = Kd / 64 is even (Kd is a multiple of 128).
    issue(lds0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    for (int s = 0; s < S; s += 2) {
      issue(lds1, s + 1);
      compute(lds0);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      if (s + 2 < S) issue(lds0, s + 2);
      compute(lds1);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
    }

    // ---------------------------------------------------------- epilogue
    // acc[i][j][v] is C[weight row wrow(i) + 8 (v / 4) + 4 lh + v % 4]
    //                  [token wm*64 + 32 j + lr].
    if (MODE == 0) {
      const int F = a.F;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int m = wm * 64 + 32 * j + lr;
        if (m < rows) {
          uint16_t* o1 = out0 + int64_t(row0 + m) * (2 * F);
          uint16_t* o2 = out1 + int64_t(row0 + m) * F;
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int jc = nt * 128 + wn * 64 + 32 * i + 4 * lh;
            float h[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const float g = round_bf16(acc[i][j][v]);
              const float up = round_bf16(acc[i + 2][j][v]);
              h[v] = silu_f(clamp_gate(g, a.limit)) * clamp_up(up, a.limit);
            }
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              st4(o1 + jc + 8 * g4, acc[i][j][4 * g4], acc[i][j][4 * g4 + 1],
                  acc[i][j][4 * g4 + 2], acc[i][j][4 * g4 + 3]);
              st4(o1 + F + jc + 8 * g4, acc[i + 2][j][4 * g4], acc[i + 2][j][4 * g4 + 1],
                  acc[i + 2][j][4 * g4 + 2], acc[i + 2][j][4 * g4 + 3]);
              st4(o2 + jc + 8 * g4, h[4 * g4], h[4 * g4 + 1], h[4 * g4 + 2], h[4 * g4 + 3]);
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int m = wm * 64 + 32 * j + lr;
        if (m < rows) {
          const int64_t slotr = a.sorted_route[row0 + m];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ncol = nt * 256 + wrow(i) + 4 * lh;
            {
              if (a.y32) {
                const float sc = a.scores[slotr];
                float* o = a.y32 + (slotr / a.K) * a.N + ncol;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
                  fused_add4(o + 8 * g4, sc, round_bf16(acc[i][j][4 * g4]),
                             round_bf16(acc[i][j][4 * g4 + 1]), round_bf16(acc[i][j][4 * g4 + 2]),
                             round_bf16(acc[i][j][4 * g4 + 3]));
              } else {
                uint16_t* o = out0 + slotr * a.N + ncol;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
                  st4(o + 8 * g4, acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2],
                      acc[i][j][4 * g4 + 3]);
              }
            }
          }
        }
      }
    }
  }
}

// One workgroup per CU (128 KiB of LDS), a multiple of the XCD count, at most the item bound.
hipError_t launch_gemm_hot(int mode, const FwdArgs& a, int64_t items_max, int cus,
                           hipStream_t s) {
  if (items_max <= 0) return hipSuccess;
  int64_t g = std::min<int64_t>(items_max, cus);
  g = std::max<int64_t>((g + kXcds - 1) / kXcds * kXcds, kXcds);
  if (mode == 0)
    hipLaunchKernelGGL(k_gemm_hot<0>, dim3(unsigned(g)), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(k_gemm_hot<1>, dim3(unsigned(g)), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
