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
//   k_gemm_dgrad<0>: dH2 = dH3_e W2_e (contraction over D) with the SwiGLU
//                    backward epilogue -> dH1 = [dG | dU] (bf16).
//   k_gemm_dgrad<1>: dXr = dH1_e W13_e (contraction over 2F) -> fp32 rows.
//   k_gemm_wgrad<2>: dW2_e  = dH3_e^T H2_e, H2 = SiLU(g) * u rebuilt from h1.
//   k_gemm_wgrad<3>: dW13_e = dH1_e^T X_e.
//
// MI355X design.  In DGRAD the weight rows run along the contraction, so the
// weight tile is transposed on its way into LDS: each thread loads the same
// 16-byte column chunk of two consecutive weight rows, interleaves them into
// eight dwords (k, k+1) and writes one dword per output column.  MFMA
// operands are then 16-byte LDS reads with the contraction contiguous.
// WGRAD contracts over token rows, so both operands take the same
// transposing path.  Work is a persistent, XCD-aware loop as in the forward
// kernels; WGRAD tiles are 128 x 128 outputs of one expert, ordered
// expert-major so the expert's operand rows stay in one XCD's L2.
#include <algorithm>

#include "common.h"

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void mfma_bf16(f32x16& acc, u32x4 a, u32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// Interleave the bf16 halves of two rows: out[q] = (lo.half[q], hi.half[q]).
__device__ __forceinline__ void interleave8(const u32x4& lo, const u32x4& hi, uint32_t* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = (lo[i] & 0xffffu) | (hi[i] << 16);
    out[2 * i + 1] = (lo[i] >> 16) | (hi[i] & 0xffff0000u);
  }
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

__device__ __forceinline__ int find_expert_b(const int32_t* __restrict__ mtoff, int E, int NT,
                                             int w) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (mtoff[mid] * NT <= w)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// ------------------------------------------------------------------ DGRAD
template <int KIND>
__global__ __launch_bounds__(256) void k_gemm_dgrad(BwdArgs a) {
  constexpr int BK = 64;                       // contraction values per stage
  constexpr int kAStrideDw = BK / 2 + 4;       // weight^T LDS row: 36 dwords (144 B)
  constexpr int kABuf = 128 * kAStrideDw * 4;  // 18432 B
  constexpr int kBStride = BK * 2 + 16;        // token LDS row: 144 B
  constexpr int kBBuf = kBM * kBStride;        // 9216 B
  __shared__ __attribute__((aligned(16))) char lds[2 * (kABuf + kBBuf)];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;
  const int lh = lane >> 5;

  const RouteHdr* hdr = a.hdr;
  const int n_items = hdr->n_mt * a.NT;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int per = gridDim.x / kXcds;
  const int chunk = (n_items + kXcds - 1) / kXcds;
  const int S = a.Kd / BK;
  const uint16_t* h1 = reinterpret_cast<const uint16_t*>(hdr->rec.h1);

  // weight^T loader: row pairs kp and kp + 16 of the stage, 8-column chunk c
  const int kp = tid & 15;
  const int c = tid >> 4;

  for (int it = slot; it < chunk; it += per) {
    const int w = xcd * chunk + it;
    if (w >= n_items) break;
    const int e = find_expert_b(a.mtoff, a.E, a.NT, w);
    const int mt_e = a.mtoff[e + 1] - a.mtoff[e];
    const int u = w - a.mtoff[e] * a.NT;
    const int nt = u / mt_e;
    const int mt = u - nt * mt_e;
    const int row0 = a.offsets[e] + mt * kBM;
    const int rows = min(kBM, a.offsets[e + 1] - row0);
    const bool two = rows > 32;

    const uint16_t* wbase = reinterpret_cast<const uint16_t*>(a.W) +
                            (int64_t(e) * a.Kd + 2 * kp) * a.N + nt * 128 + c * 8;
    const char* tbase = reinterpret_cast<const char*>(a.tok);
    const int64_t trow_bytes = int64_t(a.Kd) * 2;
    const char* tp[2];
    int toff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = tid + 256 * j;
      const int r = i >> 3, cc = i & 7;
      tp[j] = r < rows ? tbase + int64_t(row0 + r) * trow_bytes + cc * 16 : nullptr;
      toff[j] = r * kBStride + cc * 16;
    }

    f32x16 acc0 = {}, acc1 = {};
    u32x4 wr[4], tr[2];
    auto load = [&](int s) {
      const uint16_t* p = wbase + int64_t(s) * BK * a.N;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        wr[2 * pp] = *reinterpret_cast<const u32x4*>(p + int64_t(32 * pp) * a.N);
        wr[2 * pp + 1] = *reinterpret_cast<const u32x4*>(p + int64_t(32 * pp + 1) * a.N);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
        tr[j] = tp[j] ? *reinterpret_cast<const u32x4*>(tp[j] + int64_t(s) * BK * 2)
                      : u32x4{0u, 0u, 0u, 0u};
    };
    auto store = [&](int buf) {
      uint32_t* la = reinterpret_cast<uint32_t*>(lds + buf * (kABuf + kBBuf));
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        uint32_t d[8];
        interleave8(wr[2 * pp], wr[2 * pp + 1], d);
#pragma unroll
        for (int q = 0; q < 8; ++q) la[(c * 8 + q) * kAStrideDw + kp + 16 * pp] = d[q];
      }
      char* lb = lds + buf * (kABuf + kBBuf) + kABuf;
#pragma unroll
      for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4*>(lb + toff[j]) = tr[j];
    };
    auto compute = [&](int buf) {
      const char* la = lds + buf * (kABuf + kBBuf);
      const char* lb = la + kABuf;
#pragma unroll
      for (int q = 0; q < BK / 16; ++q) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(
            la + ((32 * wave + lr) * kAStrideDw + q * 8 + lh * 4) * 4);
        const u32x4 b0 =
            *reinterpret_cast<const u32x4*>(lb + lr * kBStride + (q * 16 + lh * 8) * 2);
        mfma_bf16(acc0, av, b0);
        if (two) {
          const u32x4 b1 = *reinterpret_cast<const u32x4*>(lb + (32 + lr) * kBStride +
                                                           (q * 16 + lh * 8) * 2);
          mfma_bf16(acc1, av, b1);
        }
      }
    };

    load(0);
    store(0);
    __syncthreads();
    for (int s = 0; s < S; ++s) {
      const int cur = s & 1;
      if (s + 1 < S) load(s + 1);
      compute(cur);
      if (s + 1 < S) store(cur ^ 1);
      __syncthreads();
    }

    // acc[b][v]: output column 32*wave + 8*(v/4) + 4*lh + v%4, token 32*b + lr
    const int col = nt * 128 + 32 * wave + 4 * lh;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const f32x16& acc = b ? acc1 : acc0;
      const int m = 32 * b + lr;
      if (m >= rows) continue;
      const int64_t row = row0 + m;
      if (KIND == 0) {
        const int F = a.F;
        uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + row * (2 * F);
        const uint16_t* hr = h1 + row * (2 * F);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int j = col + 8 * g4;
          float gv[4], uv[4], dg[4], du[4];
          load4_bf16(hr + j, gv);
          load4_bf16(hr + F + j, uv);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float dh2 = acc[4 * g4 + i];
            const float sg = sigmoid_f(gv[i]);
            dg[i] = dh2 * uv[i] * (sg * (1.0f + gv[i] * (1.0f - sg)));
            du[i] = dh2 * silu_f(gv[i]);
          }
          store4<uint16_t>(o + j, dg[0], dg[1], dg[2], dg[3]);
          store4<uint16_t>(o + F + j, du[0], du[1], du[2], du[3]);
        }
      } else {
        float* o = reinterpret_cast<float*>(a.out) + row * a.N;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          store4<float>(o + col + 8 * g4, acc[4 * g4], acc[4 * g4 + 1], acc[4 * g4 + 2],
                        acc[4 * g4 + 3]);
      }
    }
  }
}

// ------------------------------------------------------------------ WGRAD
template <int KIND, typename TW>
__global__ __launch_bounds__(256) void k_gemm_wgrad(BwdArgs a) {
  constexpr int BK = 32;                       // token rows per stage
  constexpr int kStrideDw = BK / 2 + 4;        // 20 dwords (80 B) per LDS row
  constexpr int kBuf = 128 * kStrideDw * 4;    // 10240 B per operand
  __shared__ __attribute__((aligned(16))) char lds[2 * 2 * kBuf];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int kp = tid & 15;   // row pair of the stage
  const int c = tid >> 4;    // 8-column chunk of the 128-wide tile

  const RouteHdr* hdr = a.hdr;
  const int F = a.F, D = a.D;
  const int per_e = a.NA * a.NB;
  const int n_items = a.E * per_e;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int per = gridDim.x / kXcds;
  const int chunk = (n_items + kXcds - 1) / kXcds;
  // A operand source (rows of the expert): KIND 2 -> h1 (H2 rebuilt), KIND 3 -> x rows.
  const uint16_t* asrc = reinterpret_cast<const uint16_t*>(KIND == 2 ? hdr->rec.h1
                                                                     : hdr->rec.x_rows);
  const int a_ld = KIND == 2 ? 2 * F : D;          // row length of the A source
  const uint16_t* bsrc = reinterpret_cast<const uint16_t*>(a.grad);
  const int b_ld = KIND == 2 ? D : 2 * F;          // row length of the B source

  for (int it = slot; it < chunk; it += per) {
    const int w = xcd * chunk + it;
    if (w >= n_items) break;
    const int e = w / per_e;
    const int rem = w - e * per_e;
    const int ta = rem / a.NB;
    const int tb = rem - ta * a.NB;
    const int r0 = a.offsets[e];
    const int Me = a.offsets[e + 1] - r0;
    const int S = (Me + BK - 1) / BK;

    const int acol = ta * 128 + c * 8;
    const int bcol = tb * 128 + c * 8;
    u32x4 ar[2], br[2];
    auto load = [&](int s) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int m = s * BK + 2 * kp + h;
        if (m < Me) {
          const int64_t row = r0 + m;
          if (KIND == 2) {
            const u32x4 gq = *reinterpret_cast<const u32x4*>(asrc + row * a_ld + acol);
            const u32x4 uq = *reinterpret_cast<const u32x4*>(asrc + row * a_ld + F + acol);
            u32x4 hq;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float g0 = __uint_as_float(gq[i] << 16), g1 = __uint_as_float(gq[i] & 0xffff0000u);
              const float u0 = __uint_as_float(uq[i] << 16), u1 = __uint_as_float(uq[i] & 0xffff0000u);
              hq[i] = pack_bf16x2(silu_f(g0) * u0, silu_f(g1) * u1);
            }
            ar[h] = hq;
          } else {
            ar[h] = *reinterpret_cast<const u32x4*>(asrc + row * a_ld + acol);
          }
          br[h] = *reinterpret_cast<const u32x4*>(bsrc + row * b_ld + bcol);
        } else {
          ar[h] = u32x4{0u, 0u, 0u, 0u};
          br[h] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    auto store = [&](int buf) {
      uint32_t* la = reinterpret_cast<uint32_t*>(lds + buf * 2 * kBuf);
      uint32_t* lb = la + kBuf / 4;
      uint32_t d[8];
      interleave8(ar[0], ar[1], d);
#pragma unroll
      for (int q = 0; q < 8; ++q) la[(c * 8 + q) * kStrideDw + kp] = d[q];
      interleave8(br[0], br[1], d);
#pragma unroll
      for (int q = 0; q < 8; ++q) lb[(c * 8 + q) * kStrideDw + kp] = d[q];
    };

    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
    if (S > 0) {
      load(0);
      store(0);
      __syncthreads();
      for (int s = 0; s < S; ++s) {
        const int cur = s & 1;
        if (s + 1 < S) load(s + 1);
        const char* la = lds + cur * 2 * kBuf;
        const char* lb = la + kBuf;
#pragma unroll
        for (int q = 0; q < BK / 16; ++q) {
          const u32x4 av = *reinterpret_cast<const u32x4*>(
              la + ((32 * wave + lr) * kStrideDw + q * 8 + lh * 4) * 4);
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const u32x4 bv = *reinterpret_cast<const u32x4*>(
                lb + ((32 * bb + lr) * kStrideDw + q * 8 + lh * 4) * 4);
            mfma_bf16(acc[bb], av, bv);
          }
        }
        if (s + 1 < S) store(cur ^ 1);
        __syncthreads();
      }
    }

    // acc[bb][v] = dW[b = tb*128 + 32*bb + lr][a = ta*128 + 32*wave + 8*(v/4) + 4*lh + v%4]
    const int64_t nb_total = KIND == 2 ? D : 2 * F;   // rows of dW per expert
    const int a_len = KIND == 2 ? F : D;               // row length of dW
    TW* o = reinterpret_cast<TW*>(a.out) + int64_t(e) * nb_total * a_len;
    const int acol0 = ta * 128 + 32 * wave + 4 * lh;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int64_t brow = tb * 128 + 32 * bb + lr;
      TW* orow = o + brow * a_len + acol0;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        store4<TW>(orow + 8 * g4, acc[bb][4 * g4], acc[bb][4 * g4 + 1], acc[bb][4 * g4 + 2],
                   acc[bb][4 * g4 + 3]);
    }
  }
}

// ------------------------------------------------------------------ launchers
// Resident workgroups per CU of one kernel (queried once per kernel).
template <int ID, typename K>
static int occupancy(K kernel) {
  static int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 256, 0) != hipSuccess || n <= 0)
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
    const unsigned g = persistent_grid(occupancy<0>(k_gemm_dgrad<0>), mt_max * a.NT, cus);
    hipLaunchKernelGGL(k_gemm_dgrad<0>, dim3(g), dim3(256), 0, s, a);
  } else {
    const unsigned g = persistent_grid(occupancy<1>(k_gemm_dgrad<1>), mt_max * a.NT, cus);
    hipLaunchKernelGGL(k_gemm_dgrad<1>, dim3(g), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// kind 2: W2 WGRAD; 3: W13 WGRAD.  dw_f32 selects the dW storage type.
hipError_t launch_wgrad(int kind, int dw_f32, const BwdArgs& a, int cus, hipStream_t s) {
  const int64_t items = int64_t(a.E) * a.NA * a.NB;
  if (items == 0) return hipSuccess;
#define MOE_WG(KD, TW)                                                                    \
  do {                                                                                    \
    const unsigned g = persistent_grid(occupancy<10 * KD + int(sizeof(TW))>(k_gemm_wgrad<KD, TW>), \
                                       items, cus);                                       \
    hipLaunchKernelGGL((k_gemm_wgrad<KD, TW>), dim3(g), dim3(256), 0, s, a);              \
  } while (0)
  if (kind == 2) {
    if (dw_f32)
      MOE_WG(2, float);
    else
      MOE_WG(2, uint16_t);
  } else {
    if (dw_f32)
      MOE_WG(3, float);
    else
      MOE_WG(3, uint16_t);
  }
#undef MOE_WG
  return hipGetLastError();
}

}  // namespace moe
