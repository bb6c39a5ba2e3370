// Bandwidth-bound row kernels: combine the K route outputs of each token,
// combine backward, the input-gradient sum, and a packed copy of the x rows
// for the backward (the forward reads x through the permutation inside the
// W13 kernel's loader).
//
// Dist-MoE explainer section 01: the expert kernel reads each route's source
// row; results return to the route's slot (t*K + k) and the token owner
// applies its scores and sums the K routes in FP32; id -1 routes are skipped
// and an all-inactive row is exact zero.  Training sends one input-gradient
// row per route back and the owner reduces the K rows.
// "Mixture of Experts: How Routing Becomes GPU Computation", section 2
// (SwiGLU backward, weighted combine): dH = p dY and dp = <H, dY>.
//
// Layout: each lane moves 16-byte chunks of a row, so a wave reads 1 KiB
// contiguous per step (fully coalesced).
#include <algorithm>

#include "common.h"

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct Vec16;  // 16 bytes of T as floats
template <>
struct Vec16<uint16_t> {
  static constexpr int n = 8;
  static __device__ __forceinline__ void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ u32x4 pack(const float* f) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return v;
  }
};
template <>
struct Vec16<float> {
  static constexpr int n = 4;
  static __device__ __forceinline__ void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
  static __device__ __forceinline__ u32x4 pack(const float* f) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
    return v;
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Grid-stride element mapping: thread g handles 16-byte chunk (row, i) for
// g = row * row_chunks + i, so every wave reads or writes 1 KiB contiguous
// per step and all chunks of all rows are in flight at once (no per-row
// serial loop); the grid is capped at a few waves per SIMD.
__device__ __forceinline__ int64_t grid_thread() {
  return int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
}
__device__ __forceinline__ int64_t grid_threads() { return int64_t(gridDim.x) * blockDim.x; }

// dst[route_to_row[t*K + k]] = x[t] for every valid route (t, k): the packed
// x rows of the backward's W13 weight gradient, whose loads then stream.
// Thread g reads 16-byte chunk i of token t once (g = t * row_chunks + i) and
// writes it to the rows of the token's valid routes; rows [0, R) are exactly
// the valid routes, so every row is written once and x is read once.
template <int KM>
__global__ __launch_bounds__(256) void k_gather(const u32x4* __restrict__ x, int64_t row_chunks,
                                                int K, const RouteHdr* __restrict__ hdr,
                                                const int32_t* __restrict__ route_to_row,
                                                u32x4* __restrict__ dst) {
  const int64_t n = int64_t(hdr->T) * row_chunks;
  if (n == 0 || hdr->R == 0) return;
  if (!x) {  // rows to copy need x: report instead of faulting
    if (grid_thread() == 0) atomicOr(const_cast<uint32_t*>(&hdr->status), MOE_STATUS_NULL_INPUT);
    return;
  }
  // with whole waves per row, a wave's token is uniform: its route reads
  // become scalar loads
  const bool wave_rows = row_chunks % 64 == 0;
  for (int64_t g = grid_thread(); g < n; g += grid_threads()) {
    int64_t t = g / row_chunks;
    if (wave_rows) t = __builtin_amdgcn_readfirstlane(int(t));
    const int64_t i = g - t * row_chunks;
    int rows[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k) rows[k] = k < K ? route_to_row[t * K + k] : -1;
    const u32x4 v = x[g];
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (rows[k] >= 0) dst[int64_t(rows[k]) * row_chunks + i] = v;
  }
}

// y[t] = sum_k valid s[t,k] h3[t*K+k] (+ addend[t]), k ascending, fp32.
// KM >= K bounds the per-thread route arrays (the launcher picks 2, 4, 8, 16).
template <typename T, int KM>
__global__ __launch_bounds__(256) void k_combine(const RouteHdr* __restrict__ hdr,
                                                 const int32_t* __restrict__ route_to_row,
                                                 const float* __restrict__ scores,
                                                 const u32x4* __restrict__ h3,
                                                 const u32x4* __restrict__ addend,
                                                 u32x4* __restrict__ y, int K, int64_t row_chunks,
                                                 uint32_t* __restrict__ status) {
  const int64_t n = int64_t(hdr->T) * row_chunks;
  if (n == 0) return;
  if (!scores || !y) {
    if (grid_thread() == 0) atomicOr(status, MOE_STATUS_NULL_INPUT);
    return;
  }
  constexpr int nv = Vec16<T>::n;
  // with whole waves per row, a wave's token is uniform: its route and score
  // reads become scalar loads
  const bool wave_rows = row_chunks % 64 == 0;
  for (int64_t g = grid_thread(); g < n; g += grid_threads()) {
    int64_t t = g / row_chunks;
    if (wave_rows) t = __builtin_amdgcn_readfirstlane(int(t));
    const int64_t i = g - t * row_chunks;
    // every slot chunk is loaded (in bounds even for padding routes, whose
    // slots are never written) and padding is dropped by a select, so the K
    // loads are independent
    u32x4 hv[KM];
    float sk[KM];
    bool valid[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (k < K) {
        hv[k] = h3[(t * K + k) * row_chunks + i];
        valid[k] = route_to_row[t * K + k] >= 0;
        sk[k] = scores[t * K + k];
      }
    }
    if (i == 0) {
      bool bad = false;
#pragma unroll
      for (int k = 0; k < KM; ++k)
        if (k < K) bad |= (!valid[k] && sk[k] != 0.0f);
      if (bad) atomicOr(status, MOE_STATUS_PAD_SCORE);
    }
    float acc[nv];
#pragma unroll
    for (int j = 0; j < nv; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (k < K && valid[k]) {
        float f[nv];
        Vec16<T>::unpack(hv[k], f);
#pragma unroll
        for (int j = 0; j < nv; ++j) acc[j] += sk[k] * f[j];
      }
    }
    if (addend) {
      float f[nv];
      Vec16<T>::unpack(addend[g], f);
#pragma unroll
      for (int j = 0; j < nv; ++j) acc[j] += f[j];
    }
    y[g] = Vec16<T>::pack(acc);
  }
}

// FUSED combine, before the W2 kernel: y32 = 0 (a fill kernel, so the call
// has no memset node when captured).
__global__ __launch_bounds__(256) void k_zero_f32(const RouteHdr* __restrict__ hdr,
                                                  float4* __restrict__ p, int64_t row4) {
  const int64_t n4 = int64_t(hdr->T) * row4;
  for (int64_t g = grid_thread(); g < n4; g += grid_threads()) p[g] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// FUSED combine, after the W2 kernel: y[t] = y32[t] (+ addend[t]) in the act
// dtype; nonzero scores on padding routes are reported as in the slot combine.
template <typename T>
__global__ __launch_bounds__(256) void k_fused_finish(const RouteHdr* __restrict__ hdr,
                                                      const int32_t* __restrict__ route_to_row,
                                                      const float* __restrict__ scores,
                                                      const float4* __restrict__ y32,
                                                      const u32x4* __restrict__ addend,
                                                      u32x4* __restrict__ y, int K,
                                                      int64_t row_chunks,
                                                      uint32_t* __restrict__ status) {
  constexpr int nv = Vec16<T>::n;   // values per 16-byte output chunk
  const int64_t n = int64_t(hdr->T) * row_chunks;
  if (n == 0) return;
  if (!scores || !y) {
    if (grid_thread() == 0) atomicOr(status, MOE_STATUS_NULL_INPUT);
    return;
  }
  for (int64_t g = grid_thread(); g < n; g += grid_threads()) {
    const int64_t t = g / row_chunks;
    const int64_t i = g - t * row_chunks;
    if (i == 0) {
      bool bad = false;
      for (int k = 0; k < K; ++k)
        bad |= route_to_row[t * K + k] < 0 && scores[t * K + k] != 0.0f;
      if (bad) atomicOr(status, MOE_STATUS_PAD_SCORE);
    }
    float acc[nv];
#pragma unroll
    for (int j = 0; j < nv / 4; ++j) {
      const float4 v = y32[g * (nv / 4) + j];
      acc[4 * j] = v.x;
      acc[4 * j + 1] = v.y;
      acc[4 * j + 2] = v.z;
      acc[4 * j + 3] = v.w;
    }
    if (addend) {
      float f[nv];
      Vec16<T>::unpack(addend[g], f);
#pragma unroll
      for (int j = 0; j < nv; ++j) acc[j] += f[j];
    }
    y[g] = Vec16<T>::pack(acc);
  }
}

// dh3[row(t,k)] = s[t,k] * dy[t];  dscores[t,k] = <h3_slot(t,k), dy[t]> (0 for padding).
// One workgroup per token at a time (grid-stride over tokens): the threads
// share the row's chunks, and the K dot products are reduced through LDS.
template <typename T, int KM>
__global__ __launch_bounds__(256) void k_combine_bwd(const RouteHdr* __restrict__ hdr,
                                                     const int32_t* __restrict__ route_to_row,
                                                     const float* __restrict__ scores,
                                                     const u32x4* __restrict__ dy,
                                                     const u32x4* __restrict__ h3,
                                                     u32x4* __restrict__ dh3,
                                                     float* __restrict__ dscores, int K,
                                                     int64_t row_chunks) {
  __shared__ float red[4][KM];
  const int n_tok = hdr->T;
  if (n_tok == 0) return;
  if (!scores || !dy) {
    if (grid_thread() == 0) atomicOr(const_cast<uint32_t*>(&hdr->status), MOE_STATUS_NULL_INPUT);
    return;
  }
  constexpr int nv = Vec16<T>::n;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int64_t t = blockIdx.x; t < n_tok; t += gridDim.x) {
    int rows[KM];
    float sk[KM], dot[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      rows[k] = k < K ? route_to_row[t * K + k] : -1;
      sk[k] = k < K ? scores[t * K + k] : 0.0f;
      dot[k] = 0.0f;
    }
    for (int64_t i = tid; i < row_chunks; i += 256) {
      float g[nv];
      Vec16<T>::unpack(dy[t * row_chunks + i], g);
      u32x4 hv[KM];
#pragma unroll
      for (int k = 0; k < KM; ++k)
        if (k < K) hv[k] = h3[(t * K + k) * row_chunks + i];
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        if (k < K && rows[k] >= 0) {
          float h[nv], o[nv];
          Vec16<T>::unpack(hv[k], h);
#pragma unroll
          for (int j = 0; j < nv; ++j) {
            dot[k] += h[j] * g[j];
            o[j] = sk[k] * g[j];
          }
          dh3[int64_t(rows[k]) * row_chunks + i] = Vec16<T>::pack(o);
        }
      }
    }
    if (dscores) {
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        if (k < K) {
          const float v = wave_sum(dot[k]);
          if (lane == 0) red[wave][k] = v;
        }
      }
      __syncthreads();
      if (tid < K) {
        const float v = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
        dscores[t * K + tid] = route_to_row[t * K + tid] >= 0 ? v : 0.0f;
      }
      __syncthreads();
    }
  }
}

// dx[t] (+)= sum over valid k, ascending, of dxr[t*K + k] (fp32) -> act dtype.
// The W13 DGRAD stores each route's fp32 row at its slot t*K + k, so a
// token's K rows are one contiguous run.  Each thread handles 4 values per
// step, so each of a wave's K row loads is 1 KiB contiguous and its store
// 512 bytes (bf16) or 1 KiB (fp32).
template <typename T>
__device__ __forceinline__ void load4(const T* p, float* f);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float* f) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  f[0] = v.x;
  f[1] = v.y;
  f[2] = v.z;
  f[3] = v.w;
}
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, float* f) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(p);
  f[0] = __uint_as_float(v[0] << 16);
  f[1] = __uint_as_float(v[0] & 0xffff0000u);
  f[2] = __uint_as_float(v[1] << 16);
  f[3] = __uint_as_float(v[1] & 0xffff0000u);
}
template <typename T>
__device__ __forceinline__ void put4(T* p, const float* f);
template <>
__device__ __forceinline__ void put4<float>(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
}
template <>
__device__ __forceinline__ void put4<uint16_t>(uint16_t* p, const float* f) {
  u32x2 v;
  v[0] = pack_bf16x2(f[0], f[1]);
  v[1] = pack_bf16x2(f[2], f[3]);
  *reinterpret_cast<u32x2*>(p) = v;
}

template <typename T, int KM>
__global__ __launch_bounds__(256) void k_dx_reduce(const RouteHdr* __restrict__ hdr,
                                                   const int32_t* __restrict__ route_to_row,
                                                   const float4* __restrict__ dxr,
                                                   T* __restrict__ dx, int K, int64_t D,
                                                   int accumulate) {
  const int n_tok = hdr->T;
  if (n_tok == 0) return;
  if (!dx) {
    if (grid_thread() == 0) atomicOr(const_cast<uint32_t*>(&hdr->status), MOE_STATUS_NULL_INPUT);
    return;
  }
  const int64_t q4 = D / 4;
  // one workgroup per token at a time: the token's route flags are uniform
  // (scalar loads) and its K slot rows stream by in 4 KiB steps
  for (int64_t t = blockIdx.x; t < n_tok; t += gridDim.x) {
    bool valid[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k) valid[k] = k < K && route_to_row[t * K + k] >= 0;
    const float4* src = dxr + t * K * q4;
    T* o = dx + t * D;
    // two chunks per thread per step, so 2K loads are in flight; the slot
    // rows are read exactly once, so the loads do not allocate in L2
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    const f32x4_t* src4 = reinterpret_cast<const f32x4_t*>(src);
    auto sum = [&](int64_t i) {
      f32x4_t v[KM];
#pragma unroll
      for (int k = 0; k < KM; ++k)
        if (k < K) v[k] = __builtin_nontemporal_load(src4 + k * q4 + i);   // padding read, not added
      return [=](float* acc) {
#pragma unroll
        for (int k = 0; k < KM; ++k) {
          if (valid[k]) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] += v[k][j];
          }
        }
      };
    };
    auto finish = [&](int64_t i, float* acc) {
      if (accumulate) {
        float f[4];
        load4<T>(o + 4 * i, f);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += f[j];
      }
      put4<T>(o + 4 * i, acc);
    };
    int64_t i = threadIdx.x;
    for (; i + 256 < q4; i += 512) {
      const auto a0 = sum(i);
      const auto a1 = sum(i + 256);
      float acc0[4] = {0.f, 0.f, 0.f, 0.f}, acc1[4] = {0.f, 0.f, 0.f, 0.f};
      a0(acc0);
      a1(acc1);
      finish(i, acc0);
      finish(i + 256, acc1);
    }
    if (i < q4) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      sum(i)(acc);
      finish(i, acc);
    }
  }
}

// ------------------------------------------------------------ launchers
// Element-mapped kernels: enough 256-thread workgroups for every chunk, capped
// at 64 per CU of a 256-CU part (grid-stride loops cover larger calls).
static inline unsigned elem_grid(int64_t chunks) {
  return unsigned(std::max<int64_t>(1, std::min<int64_t>((chunks + 255) / 256, 256 * 64)));
}
// One workgroup per token (grid-stride), capped at 8 per CU.
static inline unsigned tok_grid(int64_t T) {
  return unsigned(std::max<int64_t>(1, std::min<int64_t>(T, 256 * 8)));
}

// Route-array bound of the K-dependent kernels: 2, 4, 8 or 16.
#define MOE_DISPATCH_K(K, CALL)   \
  do {                            \
    if ((K) <= 2) {               \
      constexpr int KM = 2;       \
      CALL;                       \
    } else if ((K) <= 4) {        \
      constexpr int KM = 4;       \
      CALL;                       \
    } else if ((K) <= 8) {        \
      constexpr int KM = 8;       \
      CALL;                       \
    } else {                      \
      constexpr int KM = kMaxK;   \
      CALL;                       \
    }                             \
  } while (0)

hipError_t launch_gather(const void* x, int64_t D, int es, int K, const RouteHdr* hdr,
                         const int32_t* route_to_row, void* dst, int64_t T_max, hipStream_t s) {
  if (T_max == 0) return hipSuccess;
  const int64_t rc = D * es / 16;
  MOE_DISPATCH_K(K, hipLaunchKernelGGL((k_gather<KM>), dim3(elem_grid(T_max * rc)), dim3(256), 0,
                                       s, reinterpret_cast<const u32x4*>(x), rc, K, hdr,
                                       route_to_row, reinterpret_cast<u32x4*>(dst)));
  return hipGetLastError();
}

hipError_t launch_combine(int prec, const RouteHdr* hdr, const int32_t* route_to_row,
                          const float* scores, const void* h3, const void* addend, void* y,
                          int K, int64_t D, int64_t T_max, uint32_t* status, hipStream_t s) {
  if (T_max == 0) return hipSuccess;
  if (prec == MOE_PREC_F32)
    MOE_DISPATCH_K(K, hipLaunchKernelGGL((k_combine<float, KM>), dim3(elem_grid(T_max * (D / 4))),
                                         dim3(256), 0, s, hdr, route_to_row, scores,
                                         reinterpret_cast<const u32x4*>(h3),
                                         reinterpret_cast<const u32x4*>(addend),
                                         reinterpret_cast<u32x4*>(y), K, D / 4, status));
  else
    MOE_DISPATCH_K(K, hipLaunchKernelGGL((k_combine<uint16_t, KM>),
                                         dim3(elem_grid(T_max * (D / 8))), dim3(256), 0, s, hdr,
                                         route_to_row, scores, reinterpret_cast<const u32x4*>(h3),
                                         reinterpret_cast<const u32x4*>(addend),
                                         reinterpret_cast<u32x4*>(y), K, D / 8, status));
  return hipGetLastError();
}

// Benchmark helper: writes n16 16-byte chunks of p, so that data read next
// comes from HBM rather than from the memory-side Infinity Cache (256 MiB on
// MI355X), which a write of more than its size evicts.
__global__ __launch_bounds__(256) void k_flush(u32x4* __restrict__ p, int64_t n16, uint32_t v) {
  for (int64_t g = grid_thread(); g < n16; g += grid_threads())
    __builtin_nontemporal_store(u32x4{v, v, v, v}, p + g);
}

hipError_t launch_flush(void* p, int64_t bytes, uint32_t v, hipStream_t s) {
  if (bytes < 16) return hipSuccess;
  hipLaunchKernelGGL(k_flush, dim3(elem_grid(bytes / 16)), dim3(256), 0, s,
                     reinterpret_cast<u32x4*>(p), bytes / 16, v);
  return hipGetLastError();
}

hipError_t launch_zero_rows_f32(const RouteHdr* hdr, float* p, int64_t D, int64_t T_max,
                                hipStream_t s) {
  if (T_max == 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_f32, dim3(elem_grid(T_max * D / 4)), dim3(256), 0, s, hdr,
                     reinterpret_cast<float4*>(p), D / 4);
  return hipGetLastError();
}

hipError_t launch_fused_finish(int prec, const RouteHdr* hdr, const int32_t* route_to_row,
                               const float* scores, const float* y32, const void* addend,
                               void* y, int K, int64_t D, int64_t T_max, uint32_t* status,
                               hipStream_t s) {
  if (T_max == 0) return hipSuccess;
  if (prec == MOE_PREC_F32)
    hipLaunchKernelGGL(k_fused_finish<float>, dim3(elem_grid(T_max * (D / 4))), dim3(256), 0, s,
                       hdr, route_to_row, scores, reinterpret_cast<const float4*>(y32),
                       reinterpret_cast<const u32x4*>(addend), reinterpret_cast<u32x4*>(y), K,
                       D / 4, status);
  else
    hipLaunchKernelGGL(k_fused_finish<uint16_t>, dim3(elem_grid(T_max * (D / 8))), dim3(256), 0,
                       s, hdr, route_to_row, scores, reinterpret_cast<const float4*>(y32),
                       reinterpret_cast<const u32x4*>(addend), reinterpret_cast<u32x4*>(y), K,
                       D / 8, status);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(int prec, const RouteHdr* hdr, const int32_t* route_to_row,
                              const float* scores, const void* dy, const void* h3, void* dh3,
                              float* dscores, int K, int64_t D, int64_t T_max, hipStream_t s) {
  if (T_max == 0) return hipSuccess;
  if (prec == MOE_PREC_F32)
    MOE_DISPATCH_K(K, hipLaunchKernelGGL((k_combine_bwd<float, KM>), dim3(tok_grid(T_max)),
                                         dim3(256), 0, s, hdr, route_to_row, scores,
                                         reinterpret_cast<const u32x4*>(dy),
                                         reinterpret_cast<const u32x4*>(h3),
                                         reinterpret_cast<u32x4*>(dh3), dscores, K, D / 4));
  else
    MOE_DISPATCH_K(K, hipLaunchKernelGGL((k_combine_bwd<uint16_t, KM>), dim3(tok_grid(T_max)),
                                         dim3(256), 0, s, hdr, route_to_row, scores,
                                         reinterpret_cast<const u32x4*>(dy),
                                         reinterpret_cast<const u32x4*>(h3),
                                         reinterpret_cast<u32x4*>(dh3), dscores, K, D / 8));
  return hipGetLastError();
}

hipError_t launch_dx_reduce(int prec, const RouteHdr* hdr, const int32_t* route_to_row,
                            const float* dxr, void* dx, int K, int64_t D, int64_t T_max,
                            int accumulate, hipStream_t s) {
  if (T_max == 0) return hipSuccess;
  if (prec == MOE_PREC_F32)
    MOE_DISPATCH_K(K, hipLaunchKernelGGL((k_dx_reduce<float, KM>), dim3(tok_grid(T_max)),
                                         dim3(256), 0, s, hdr, route_to_row,
                                         reinterpret_cast<const float4*>(dxr),
                                         reinterpret_cast<float*>(dx), K, D, accumulate));
  else
    MOE_DISPATCH_K(K, hipLaunchKernelGGL((k_dx_reduce<uint16_t, KM>),
                                         dim3(tok_grid(T_max)), dim3(256), 0, s, hdr,
                                         route_to_row, reinterpret_cast<const float4*>(dxr),
                                         reinterpret_cast<uint16_t*>(dx), K, D, accumulate));
  return hipGetLastError();
}

#undef MOE_DISPATCH_K

}  // namespace moe
