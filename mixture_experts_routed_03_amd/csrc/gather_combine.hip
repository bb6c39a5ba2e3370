// Bandwidth-bound row kernels: gather x rows into expert order, combine the
// K route outputs of each token, combine backward and the input-gradient sum.
//
// Dist-MoE explainer section 01: the expert kernel reads each route's source
// row; results return to the route's slot (t*K + k) and the token owner
// applies its scores and sums the K routes in FP32; id -1 routes are skipped
// and an all-inactive row is exact zero.  Training sends one input-gradient
// row per route back and the owner reduces the K rows.
// "Mixture of Experts: How Routing Becomes GPU Computation", section 2
// (SwiGLU backward, weighted combine): dH = p dY and dp = <H, dY>.
//
// Layout: one wave per row; each lane moves 16-byte chunks, so a wave reads
// 1 KiB contiguous per step (fully coalesced).
#include "common.h"

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

// A[row] = x[sorted_route[row] / K] for row < R; destination from the
// layer's planner record (arena or scratch).
__global__ __launch_bounds__(256) void k_gather(const u32x4* __restrict__ x, int64_t row_chunks,
                                                int K, const RouteHdr* __restrict__ hdr,
                                                const int32_t* __restrict__ sorted_route,
                                                int replay_only) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (replay_only && !hdr->rec.replay) return;
  if (row >= hdr->R) return;
  if (!x) {  // T > 0 needs x: report instead of faulting
    if (row == 0 && lane == 0) atomicOr(const_cast<uint32_t*>(&hdr->status), MOE_STATUS_NULL_INPUT);
    return;
  }
  u32x4* dst = global_ptr<u32x4>(hdr->rec.x_rows) + row * row_chunks;
  const int64_t t = sorted_route[row] / K;
  const u32x4* src = x + t * row_chunks;
  for (int64_t i = lane; i < row_chunks; i += 64) dst[i] = src[i];
}

// y[t] = sum_k valid s[t,k] h3[t*K+k] (+ addend[t]), k ascending, fp32.
template <typename T>
__global__ __launch_bounds__(256) void k_combine(const RouteHdr* __restrict__ hdr,
                                                 const int32_t* __restrict__ route_to_row,
                                                 const float* __restrict__ scores,
                                                 const u32x4* __restrict__ h3,
                                                 const u32x4* __restrict__ addend,
                                                 u32x4* __restrict__ y, int K, int64_t row_chunks,
                                                 uint32_t* __restrict__ status) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= hdr->T) return;
  if (!scores || !y) {
    if (t == 0 && lane == 0) atomicOr(status, MOE_STATUS_NULL_INPUT);
    return;
  }
  float s[kMaxK];
  bool v[kMaxK];
  int bad = 0;
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    if (k < K) {
      v[k] = route_to_row[t * K + k] >= 0;
      s[k] = scores[t * K + k];
      bad |= (!v[k] && s[k] != 0.0f);
    } else {
      v[k] = false;
      s[k] = 0.0f;
    }
  }
  if (bad && lane == 0) atomicOr(status, MOE_STATUS_PAD_SCORE);
  constexpr int n = Vec16<T>::n;
  for (int64_t i = lane; i < row_chunks; i += 64) {
    float acc[n];
#pragma unroll
    for (int j = 0; j < n; ++j) acc[j] = 0.0f;
    for (int k = 0; k < K; ++k) {
      if (!v[k]) continue;
      float f[n];
      Vec16<T>::unpack(h3[(t * K + k) * row_chunks + i], f);
#pragma unroll
      for (int j = 0; j < n; ++j) acc[j] += s[k] * f[j];
    }
    if (addend) {
      float f[n];
      Vec16<T>::unpack(addend[t * row_chunks + i], f);
#pragma unroll
      for (int j = 0; j < n; ++j) acc[j] += f[j];
    }
    y[t * row_chunks + i] = Vec16<T>::pack(acc);
  }
}

// dh3[row(t,k)] = s[t,k] * dy[t];  dscores[t,k] = <h3_slot(t,k), dy[t]> (0 for padding).
template <typename T>
__global__ __launch_bounds__(256) void k_combine_bwd(const RouteHdr* __restrict__ hdr,
                                                     const int32_t* __restrict__ route_to_row,
                                                     const float* __restrict__ scores,
                                                     const u32x4* __restrict__ dy,
                                                     const u32x4* __restrict__ h3,
                                                     u32x4* __restrict__ dh3,
                                                     float* __restrict__ dscores, int K,
                                                     int64_t row_chunks) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= hdr->T) return;
  if (!scores || !dy) {
    if (t == 0 && lane == 0)
      atomicOr(const_cast<uint32_t*>(&hdr->status), MOE_STATUS_NULL_INPUT);
    return;
  }
  constexpr int n = Vec16<T>::n;
  for (int k = 0; k < K; ++k) {
    const int64_t r = t * K + k;
    const int row = route_to_row[r];
    if (row < 0) {
      if (dscores && lane == 0) dscores[r] = 0.0f;
      continue;
    }
    const float sk = scores[r];
    float dot = 0.0f;
    for (int64_t i = lane; i < row_chunks; i += 64) {
      float g[n], h[n], o[n];
      Vec16<T>::unpack(dy[t * row_chunks + i], g);
      Vec16<T>::unpack(h3[r * row_chunks + i], h);
#pragma unroll
      for (int j = 0; j < n; ++j) {
        dot += h[j] * g[j];
        o[j] = sk * g[j];
      }
      dh3[int64_t(row) * row_chunks + i] = Vec16<T>::pack(o);
    }
    dot = wave_sum(dot);
    if (dscores && lane == 0) dscores[r] = dot;
  }
}

// dx[t] (+)= sum over valid k, ascending, of dxr[row(t,k)] (fp32) -> act dtype.
template <typename T>
__global__ __launch_bounds__(256) void k_dx_reduce(const RouteHdr* __restrict__ hdr,
                                                   const int32_t* __restrict__ route_to_row,
                                                   const float4* __restrict__ dxr,
                                                   T* __restrict__ dx, int K, int64_t D,
                                                   int accumulate) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= hdr->T) return;
  if (!dx) {
    if (t == 0 && lane == 0)
      atomicOr(const_cast<uint32_t*>(&hdr->status), MOE_STATUS_NULL_INPUT);
    return;
  }
  int rows[kMaxK];
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) rows[k] = k < K ? route_to_row[t * K + k] : -1;
  const int64_t q4 = D / 4;
  for (int64_t i = lane; i < q4; i += 64) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < K; ++k) {
      if (rows[k] < 0) continue;
      const float4 v = dxr[int64_t(rows[k]) * q4 + i];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    T* o = dx + t * D + i * 4;
    if (accumulate) {
      acc.x += Elem<T>::to_f(o[0]);
      acc.y += Elem<T>::to_f(o[1]);
      acc.z += Elem<T>::to_f(o[2]);
      acc.w += Elem<T>::to_f(o[3]);
    }
    o[0] = Elem<T>::from_f(acc.x);
    o[1] = Elem<T>::from_f(acc.y);
    o[2] = Elem<T>::from_f(acc.z);
    o[3] = Elem<T>::from_f(acc.w);
  }
}

// ------------------------------------------------------------ launchers
static inline unsigned rows_grid(int64_t rows) { return unsigned((rows + 3) / 4); }

hipError_t launch_gather(const void* x, int64_t D, int es, int K, const RouteHdr* hdr,
                         const int32_t* sorted_route, int64_t R_max, int replay_only,
                         hipStream_t s) {
  if (R_max == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather, dim3(rows_grid(R_max)), dim3(256), 0, s,
                     reinterpret_cast<const u32x4*>(x), D * es / 16, K, hdr, sorted_route,
                     replay_only);
  return hipGetLastError();
}

hipError_t launch_combine(int prec, const RouteHdr* hdr, const int32_t* route_to_row,
                          const float* scores, const void* h3, const void* addend, void* y,
                          int K, int64_t D, int64_t T_max, uint32_t* status, hipStream_t s) {
  if (T_max == 0) return hipSuccess;
  if (prec == MOE_PREC_F32)
    hipLaunchKernelGGL(k_combine<float>, dim3(rows_grid(T_max)), dim3(256), 0, s, hdr,
                       route_to_row, scores, reinterpret_cast<const u32x4*>(h3),
                       reinterpret_cast<const u32x4*>(addend), reinterpret_cast<u32x4*>(y), K,
                       D / 4, status);
  else
    hipLaunchKernelGGL(k_combine<uint16_t>, dim3(rows_grid(T_max)), dim3(256), 0, s, hdr,
                       route_to_row, scores, reinterpret_cast<const u32x4*>(h3),
                       reinterpret_cast<const u32x4*>(addend), reinterpret_cast<u32x4*>(y), K,
                       D / 8, status);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(int prec, const RouteHdr* hdr, const int32_t* route_to_row,
                              const float* scores, const void* dy, const void* h3, void* dh3,
                              float* dscores, int K, int64_t D, int64_t T_max, hipStream_t s) {
  if (T_max == 0) return hipSuccess;
  if (prec == MOE_PREC_F32)
    hipLaunchKernelGGL(k_combine_bwd<float>, dim3(rows_grid(T_max)), dim3(256), 0, s, hdr,
                       route_to_row, scores, reinterpret_cast<const u32x4*>(dy),
                       reinterpret_cast<const u32x4*>(h3), reinterpret_cast<u32x4*>(dh3),
                       dscores, K, D / 4);
  else
    hipLaunchKernelGGL(k_combine_bwd<uint16_t>, dim3(rows_grid(T_max)), dim3(256), 0, s, hdr,
                       route_to_row, scores, reinterpret_cast<const u32x4*>(dy),
                       reinterpret_cast<const u32x4*>(h3), reinterpret_cast<u32x4*>(dh3),
                       dscores, K, D / 8);
  return hipGetLastError();
}

hipError_t launch_dx_reduce(int prec, const RouteHdr* hdr, const int32_t* route_to_row,
                            const float* dxr, void* dx, int K, int64_t D, int64_t T_max,
                            int accumulate, hipStream_t s) {
  if (T_max == 0) return hipSuccess;
  if (prec == MOE_PREC_F32)
    hipLaunchKernelGGL(k_dx_reduce<float>, dim3(rows_grid(T_max)), dim3(256), 0, s, hdr,
                       route_to_row, reinterpret_cast<const float4*>(dxr),
                       reinterpret_cast<float*>(dx), K, D, accumulate);
  else
    hipLaunchKernelGGL(k_dx_reduce<uint16_t>, dim3(rows_grid(T_max)), dim3(256), 0, s, hdr,
                       route_to_row, reinterpret_cast<const float4*>(dxr),
                       reinterpret_cast<uint16_t*>(dx), K, D, accumulate);
  return hipGetLastError();
}

}  // namespace moe
