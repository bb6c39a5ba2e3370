// Routing metadata on the device: per-expert histogram, prefix offsets and
// tile schedule, stable expert-major permutation and its inverse.
//
// "Mixture of Experts: How Routing Becomes GPU Computation", section 2
// ("Packing"): rows are sorted by expert with a stable sort, counts give
// exclusive prefix offsets (counts [4,3,3,2] -> [0,4,7,10,12]) and the
// inverse permutation is kept to return outputs; the page builds the tile
// schedule on the host after copying counts, and notes it could instead be
// built on the GPU - which is what happens here, with no host sync.
// Dist-MoE explainer section 01: id -1 disables a route.
//
// Deterministic counting sort.  Up to 1,024 routes (decode): one workgroup
// of one launch (k_route_small); up to 32,768 routes and 2,560 experts: one
// launch of one workgroup per 256-route chunk that needs nothing from the
// others (k_route_chunked); larger calls, three launches:
//   hist : one workgroup per chunk of 256 routes, LDS atomics -> chunk_hist[c][e]
//   scan : one workgroup; counts[e] = sum_c chunk_hist[c][e], exclusive scans
//          of counts, of counts rounded up to 32 and of m-tiles; the chunk
//          histograms become per-chunk row bases (chunk-major order)
//   rank : one workgroup per chunk; a route's row is its chunk base plus the
//          number of earlier routes of the same expert in its chunk.
// Rows are never assigned in atomic order, so the permutation is exact.
#include "common.h"

namespace moe {

__global__ __launch_bounds__(256) void k_route_hist(const int32_t* __restrict__ ids, int64_t n,
                                                    int E, int32_t* __restrict__ chunk_hist,
                                                    int32_t* __restrict__ chunk_flags) {
  extern __shared__ int32_t hist[];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int64_t r = int64_t(c) * kRankChunk + threadIdx.x;
  int bad = 0;
  if (r < n) {
    const int id = ids[r];
    if (id >= 0 && id < E)
      atomicAdd(&hist[id], 1);
    else if (id != -1)
      bad = 1;
  }
  bad = __syncthreads_or(bad);
  int32_t* out = chunk_hist + int64_t(c) * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) out[e] = hist[e];
  if (threadIdx.x == 0) chunk_flags[c] = bad ? int32_t(MOE_STATUS_BAD_ID) : 0;
}

// Inclusive scan of N ints per thread over a 1024-thread block: a shuffle
// scan inside each wave, then a scan of the 16 wave totals.
template <int N>
__device__ void block_scan(int* v /* [N] */, int* sh /* [N][16] */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int u[N];
#pragma unroll
    for (int j = 0; j < N; ++j) u[j] = __shfl_up(v[j], off, 64);
    if (lane >= off) {
#pragma unroll
      for (int j = 0; j < N; ++j) v[j] += u[j];
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int j = 0; j < N; ++j) sh[16 * j + wave] = v[j];
  }
  __syncthreads();
  int p[N] = {};
  for (int w = 0; w < wave; ++w) {
#pragma unroll
    for (int j = 0; j < N; ++j) p[j] += sh[16 * j + w];
  }
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] += p[j];
  __syncthreads();
}

// Column sums of the chunk histograms and their rewrite into row bases
// (calls above kChunkedRoutes routes): each thread reads its expert's column
// 16 chunks at a time, twice (independent loads; threads of consecutive
// experts read consecutive words).  Experts are handled in passes of 1024,
// expert e = 1024 * pass + thread, with the running totals carried between
// passes.
constexpr int kScanBatch = 16;

// The per-expert terms whose exclusive prefixes routing writes, for an
// expert with s rows: rows (offsets), rows rounded up to 32 (poffsets),
// 64-row stages (mtoff), FPROP/DGRAD m-tiles (gtoff), then the BF16 forward
// split: stages and m-tiles of cold experts (cstoff, ctoff) and 256-row
// m-tiles of hot experts (hotoff), then the BF16 WGRAD split: stages of the
// experts below kHotWgRows rows (cwoff).
constexpr int kScans = 8;
__device__ __forceinline__ void scan_terms(int s, int* v) {
  const bool hot = hot_expert(s);
  v[0] = s;
  v[1] = (s + kMxBlock - 1) / kMxBlock * kMxBlock;
  v[2] = (s + kBM - 1) / kBM;
  v[3] = (s + gemm_tile_rows(s) - 1) / gemm_tile_rows(s);
  v[4] = hot ? 0 : v[2];
  v[5] = hot ? 0 : v[3];
  v[6] = hot ? (s + kBMH - 1) / kBMH : 0;
  v[7] = hot_wgrad_expert(s) ? 0 : v[2];
}

__global__ __launch_bounds__(1024) void k_route_scan(int32_t* __restrict__ chunk_hist,
                                                     const int32_t* __restrict__ chunk_flags,
                                                     int nchunks, int E, int T,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ poffsets,
                                                     int32_t* __restrict__ mtoff,
                                                     int32_t* __restrict__ gtoff,
                                                     int32_t* __restrict__ split,
                                                     RouteHdr* __restrict__ hdr) {
  __shared__ int sh[16 * kScans];
  __shared__ int carry[kScans];
  __shared__ int red[2];
  const int tid = threadIdx.x;
  if (tid < kScans) carry[tid] = 0;
  if (tid == 0) red[0] = red[1] = 0;
  // chunk status words, loaded first so they are in flight with the columns
  int f = 0;
  for (int c = tid; c < nchunks; c += 1024) f |= chunk_flags[c];
  __syncthreads();
  int mx = 0;
  for (int e0 = 0; e0 < E; e0 += 1024) {
    const int e = e0 + tid;
    int s = 0;
    if (e < E) {
      for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
        int v[kScanBatch];
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j)
          v[j] = chunk_hist[int64_t(min(c0 + j, nchunks - 1)) * E + e];
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) s += c0 + j < nchunks ? v[j] : 0;
      }
    }
    int v[kScans];
    scan_terms(s, v);
    mx = max(mx, s);
    block_scan<kScans>(v, sh);
    int o[kScans];
    {
      int t[kScans];
      scan_terms(s, t);
#pragma unroll
      for (int j = 0; j < kScans; ++j) o[j] = carry[j] + v[j] - t[j];
    }
    const int oc = o[0];
    if (e < E) {
      counts[e] = s;
      offsets[e] = oc;
      poffsets[e] = o[1];
      mtoff[e] = o[2];
      gtoff[e] = o[3];
#pragma unroll
      for (int j = 0; j < kScans - 4; ++j) split[j * (E + 1) + e] = o[4 + j];
      // chunk histograms -> row base of each (chunk, expert)
      int run = oc;
      for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
        int v[kScanBatch];
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j)
          v[j] = chunk_hist[int64_t(min(c0 + j, nchunks - 1)) * E + e];
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) {
          if (c0 + j < nchunks) {
            chunk_hist[int64_t(c0 + j) * E + e] = run;
            run += v[j];
          }
        }
      }
    }
    __syncthreads();   // every thread has read the carries of this pass
    if (tid == 1023) {
#pragma unroll
      for (int j = 0; j < kScans; ++j) carry[j] += v[j];
    }
    __syncthreads();
  }
  // status and max count
  atomicOr(&red[0], f);
  atomicMax(&red[1], mx);
  __syncthreads();
  if (tid == 0) {
    offsets[E] = carry[0];
    poffsets[E] = carry[1];
    mtoff[E] = carry[2];
    gtoff[E] = carry[3];
#pragma unroll
    for (int j = 0; j < kScans - 4; ++j) split[j * (E + 1) + E] = carry[4 + j];
    hdr->T = T;
    hdr->R = carry[0];
    hdr->Rpad = carry[1];
    hdr->n_mt = carry[2];
    hdr->status = uint32_t(red[0]);
    hdr->max_count = red[1];
    hdr->rec.done = 0;
  }
  if (tid < 2 * kXcds) hdr->wq[tid] = 0u;
}

// Lanes of this wave below the calling lane whose key equals its key: one
// ballot per key bit keeps, in each lane's mask, the lanes that agree with
// it on that bit.  Every lane of the wave must call it (no lane masked off);
// keys are below 2^nbits.
__device__ __forceinline__ int lanes_below_equal(uint32_t key, int nbits) {
  uint64_t same = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t m = __ballot(bit);
    same &= bit ? m : ~m;
  }
  return __popcll(same & ((1ull << (threadIdx.x & 63)) - 1ull));
}

// Routes of earlier waves in sid (16-byte aligned, -1 = no route) whose
// expert is id: every lane of the wave reads the same four words per step.
__device__ __forceinline__ int earlier_waves_equal(const int32_t* sid, int id) {
  const int4* s4 = reinterpret_cast<const int4*>(sid);
  int rank = 0;
  for (int q = 0; q < (int(threadIdx.x) >> 6) * 16; ++q) {
    const int4 v = s4[q];
    rank += (v.x == id) + (v.y == id) + (v.z == id) + (v.w == id);
  }
  return rank;
}

__global__ __launch_bounds__(256) void k_route_rank(const int32_t* __restrict__ ids, int64_t n,
                                                    int E, const int32_t* __restrict__ chunk_base,
                                                    int32_t* __restrict__ sorted_route,
                                                    int32_t* __restrict__ route_to_row) {
  __shared__ __align__(16) int32_t sid[kRankChunk];
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t r = int64_t(c) * kRankChunk + tid;
  int id = r < n ? ids[r] : -1;
  const bool valid = id >= 0 && id < E;
  sid[tid] = valid ? id : -1;
  // earlier routes of the same expert inside this chunk: in this wave, then
  // in the earlier waves
  int rank = lanes_below_equal(valid ? uint32_t(id + 1) : 0u, 32 - __clz(E));
  __syncthreads();
  if (r >= n) return;
  if (!valid) {
    route_to_row[r] = -1;
    return;
  }
  rank += earlier_waves_equal(sid, id);
  const int row = chunk_base[int64_t(c) * E + id] + rank;
  sorted_route[row] = int32_t(r);
  route_to_row[r] = row;
}

// Up to kSmallRoutes routes (decode steps): the whole counting sort in one
// launch of one workgroup.  The ids sit in LDS; counts come from LDS atomics
// (their order does not matter, only their sums); offsets from the same
// block scan as k_route_scan; a route's row is its expert's offset plus the
// number of earlier routes of that expert (the stable order).  Writes the
// same outputs as the three launches (no chunk histograms).
constexpr int kSmallRoutes = 1024;

__global__ __launch_bounds__(1024) void k_route_small(const int32_t* __restrict__ ids, int n,
                                                      int E, int T,
                                                      int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ poffsets,
                                                      int32_t* __restrict__ mtoff,
                                                      int32_t* __restrict__ gtoff,
                                                      int32_t* __restrict__ split,
                                                      int32_t* __restrict__ sorted_route,
                                                      int32_t* __restrict__ route_to_row,
                                                      RouteHdr* __restrict__ hdr) {
  __shared__ __align__(16) int32_t sid[kSmallRoutes];
  __shared__ int32_t cnt[kMaxE];   // counts, then each expert's first row
  __shared__ int sh[16 * kScans];
  __shared__ int carry[kScans];
  __shared__ int s_mx;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) cnt[e] = 0;
  if (tid < kScans) carry[tid] = 0;
  if (tid == 0) s_mx = 0;
  int bad = 0;
  int id = -1;
  if (tid < n) {
    id = ids[tid];
    if (id < -1 || id >= E) {
      bad = 1;
      id = -1;
    }
  }
  sid[tid] = id;
  const int below = lanes_below_equal(uint32_t(id + 1), 32 - __clz(E));   // id -1: key 0
  __syncthreads();
  if (id >= 0) atomicAdd(&cnt[id], 1);
  bad = __syncthreads_or(bad);
  int mx = 0;
  for (int e0 = 0; e0 < E; e0 += 1024) {
    const int e = e0 + tid;
    const int s = e < E ? cnt[e] : 0;
    int v[kScans];
    scan_terms(s, v);
    mx = max(mx, s);
    block_scan<kScans>(v, sh);
    int o[kScans];
    {
      int t[kScans];
      scan_terms(s, t);
#pragma unroll
      for (int j = 0; j < kScans; ++j) o[j] = carry[j] + v[j] - t[j];
    }
    const int oc = o[0];
    if (e < E) {
      counts[e] = s;
      offsets[e] = oc;
      poffsets[e] = o[1];
      mtoff[e] = o[2];
      gtoff[e] = o[3];
#pragma unroll
      for (int j = 0; j < kScans - 4; ++j) split[j * (E + 1) + e] = o[4 + j];
      cnt[e] = oc;
    }
    __syncthreads();   // every thread has read the carries of this pass
    if (tid == 1023) {
#pragma unroll
      for (int j = 0; j < kScans; ++j) carry[j] += v[j];
    }
    __syncthreads();
  }
  if (tid < n) {
    if (id < 0) {
      route_to_row[tid] = -1;
    } else {
      // earlier routes of the same expert: in this wave, then in earlier waves
      const int row = cnt[id] + below + earlier_waves_equal(sid, id);
      sorted_route[row] = tid;
      route_to_row[tid] = row;
    }
  }
  atomicMax(&s_mx, mx);
  __syncthreads();
  if (tid == 0) {
    offsets[E] = carry[0];
    poffsets[E] = carry[1];
    mtoff[E] = carry[2];
    gtoff[E] = carry[3];
#pragma unroll
    for (int j = 0; j < kScans - 4; ++j) split[j * (E + 1) + E] = carry[4 + j];
    hdr->T = T;
    hdr->R = carry[0];
    hdr->Rpad = carry[1];
    hdr->n_mt = carry[2];
    hdr->status = bad ? uint32_t(MOE_STATUS_BAD_ID) : 0u;
    hdr->max_count = s_mx;
    hdr->rec.done = 0;
  }
  if (tid < 2 * kXcds) hdr->wq[tid] = 0u;
}

// Inclusive scan of N ints per thread over a 256-thread block (4 waves).
template <int N>
__device__ void block_scan256(int* v /* [N] */, int* sh /* [N][4] */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int u[N];
#pragma unroll
    for (int j = 0; j < N; ++j) u[j] = __shfl_up(v[j], off, 64);
    if (lane >= off) {
#pragma unroll
      for (int j = 0; j < N; ++j) v[j] += u[j];
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int j = 0; j < N; ++j) sh[4 * j + wave] = v[j];
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    if (w < wave) {
#pragma unroll
      for (int j = 0; j < N; ++j) v[j] += sh[4 * j + w];
    }
  }
  __syncthreads();
}

// Calls of kSmallRoutes + 1 .. kChunkedRoutes routes (training and prefill
// steps): the whole counting sort in one launch, one 256-thread workgroup
// per 256-route chunk, with no communication between workgroups.  Every
// workgroup reads all the ids (at most 128 KiB; after the first workgroup
// they come from L2) and counts in LDS, with integer atomics (exact in any
// order), each expert's routes in all chunks and in the chunks before its
// own.  It then scans the per-expert terms itself (each thread a run of
// consecutive experts) and ranks its own chunk's routes: a route's rank is
// the count of its expert's routes in the chunk's earlier waves (LDS
// counters) plus the earlier lanes of its own wave with that expert;
// workgroup 0 publishes counts, prefixes and the header.  Same outputs as
// the three-launch path, which stays for larger calls (each workgroup's
// read of every id would grow with the square of the call) and for more
// experts than its LDS counters fit.
constexpr int kChunkedRoutes = 32768;
constexpr int kChunkedMaxE = 2560;   // 6 E + 2 counters in LDS, within 64 KiB

__global__ __launch_bounds__(256) void k_route_chunked(const int32_t* __restrict__ ids, int n,
                                                       int E, int T,
                                                       int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ poffsets,
                                                       int32_t* __restrict__ mtoff,
                                                       int32_t* __restrict__ gtoff,
                                                       int32_t* __restrict__ split,
                                                       int32_t* __restrict__ sorted_route,
                                                       int32_t* __restrict__ route_to_row,
                                                       RouteHdr* __restrict__ hdr) {
  // [E + 1] routes per expert, [E + 1] routes before this chunk (word E of
  // each counts the invalid ids, so that every route takes an unconditional
  // atomic), then [4][E] the chunk's routes per expert in each of its four
  // waves
  extern __shared__ int32_t cnt[];
  int32_t* tot = cnt;
  int32_t* pre = cnt + E + 1;
  int32_t* wcnt = cnt + 2 * E + 2;
  __shared__ int sh[4 * kScans];
  __shared__ int s_mx;
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  for (int e = tid; e < 6 * E + 2; e += kRankChunk) cnt[e] = 0;
  if (tid == 0) s_mx = 0;
  __syncthreads();
  const int mine = c * kRankChunk + tid;   // this thread's route of the chunk
  const int before = c * kRankChunk;       // routes of the earlier chunks
  int bad = 0;
  constexpr int kBatch = 48;   // independent loads in flight per thread (12,288 routes: one batch)
  for (int r0 = 0; r0 < n; r0 += kRankChunk * kBatch) {
    int v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int r = r0 + kRankChunk * k + tid;
      v[k] = r < n ? ids[r] : -1;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int id = v[k];
      bad |= id < -1 || id >= E;
      // one LDS atomic per route: earlier chunks (a wave-uniform choice, as
      // chunks are kRankChunk-aligned) count into pre, the rest into tot,
      // and tot becomes the total below
      int32_t* const into = r0 + kRankChunk * k < before ? pre : tot;
      atomicAdd(into + (id >= 0 && id < E ? id : E), 1);
    }
  }
  int my_id = mine < n ? ids[mine] : -1;   // this thread's route of the chunk
  if (my_id < 0 || my_id >= E) my_id = -1;
  if (my_id >= 0) atomicAdd(&wcnt[(tid >> 6) * E + my_id], 1);
  bad = __syncthreads_or(bad);   // also: every count is in
  for (int e = tid; e < E; e += kRankChunk) tot[e] += pre[e];
  __syncthreads();

  // exclusive prefixes over experts; thread t owns experts [t ept, t ept + ept)
  const int ept = (E + kRankChunk - 1) / kRankChunk;
  const int e0 = tid * ept;
  int own[kScans] = {}, mx = 0;
  for (int i = 0; i < ept; ++i) {
    const int e = e0 + i;
    if (e < E) {
      int v[kScans];
      scan_terms(tot[e], v);
#pragma unroll
      for (int j = 0; j < kScans; ++j) own[j] += v[j];
      mx = max(mx, tot[e]);
    }
  }
  int run[kScans];
#pragma unroll
  for (int j = 0; j < kScans; ++j) run[j] = own[j];
  block_scan256<kScans>(run, sh);   // inclusive
#pragma unroll
  for (int j = 0; j < kScans; ++j) run[j] -= own[j];
  for (int i = 0; i < ept; ++i) {
    const int e = e0 + i;
    if (e < E) {
      const int s = tot[e];
      if (c == 0) {
        counts[e] = s;
        offsets[e] = run[0];
        poffsets[e] = run[1];
        mtoff[e] = run[2];
        gtoff[e] = run[3];
#pragma unroll
        for (int j = 0; j < kScans - 4; ++j) split[j * (E + 1) + e] = run[4 + j];
      }
      pre[e] += run[0];   // this chunk's first row of expert e
      int v[kScans];
      scan_terms(s, v);
#pragma unroll
      for (int j = 0; j < kScans; ++j) run[j] += v[j];
    }
  }
  atomicMax(&s_mx, mx);
  // earlier lanes of this wave with the same expert (key 0: no valid route)
  const int below = lanes_below_equal(mine < n ? uint32_t(my_id + 1) : 0u, 32 - __clz(E));
  __syncthreads();
  if (mine < n) {
    if (my_id < 0) {
      route_to_row[mine] = -1;
    } else {
      // earlier routes of the same expert in this chunk: those of the earlier
      // waves (counted), then the earlier lanes of this wave
      const int w = tid >> 6;
      int rank = below;
      for (int u = 0; u < w; ++u) rank += wcnt[u * E + my_id];
      const int row = pre[my_id] + rank;
      sorted_route[row] = mine;
      route_to_row[mine] = row;
    }
  }
  if (c == 0) {
    // the last thread's running prefixes are the totals
    if (tid == kRankChunk - 1) {
      offsets[E] = run[0];
      poffsets[E] = run[1];
      mtoff[E] = run[2];
      gtoff[E] = run[3];
#pragma unroll
      for (int j = 0; j < kScans - 4; ++j) split[j * (E + 1) + E] = run[4 + j];
      hdr->T = T;
      hdr->R = run[0];
      hdr->Rpad = run[1];
      hdr->n_mt = run[2];
      hdr->status = bad ? uint32_t(MOE_STATUS_BAD_ID) : 0u;
      hdr->max_count = s_mx;
      hdr->rec.done = 0;
    }
    if (tid < 2 * kXcds) hdr->wq[tid] = 0u;
  }
}

// ------------------------------------------------------------ planner
// Dist-MoE explainer section 04: before saving a layer's full state the
// planner replays instead when saved bytes + this layer's full state +
// remaining layers x replay-input bytes exceed the slot capacity; a layer
// that replays keeps only its replay input (here none: x stays with the
// caller).  Equality saves.  Layer 0 starts the step at cursor 0.
__global__ void k_plan_decide(RouteHdr* __restrict__ hdr, PlanArgs a) {
  if (a.zero) {
    uint32_t* z = reinterpret_cast<uint32_t*>(a.zero);
    for (int i = threadIdx.x; i < a.zero_n; i += blockDim.x) z[i] = 0u;
  }
  if (threadIdx.x != 0) return;
  LayerRec& rec = hdr->rec;
  const int64_t R = hdr->R;
  const int64_t Rp = hdr->Rpad;
  // Saved state of the layer.  BF16/FP32: h1 (explainer section 04 also
  // lists the gathered x rows, which on one GPU are a copy of the caller's x:
  // every kernel here reads x through the permutation instead).  MXFP8
  // (section 04, MXFP8 full-save): x and h2 column bundles (codes +
  // exponents) and dense h1.
  int64_t part[5] = {0, 0, 0, 0, 0};
  if (a.mx) {
    part[0] = align128(Rp * a.D);
    part[1] = align128(Rp / 32 * a.D);
    part[2] = align128(R * 2 * a.F * 2);
    part[3] = align128(Rp * a.F);
    part[4] = align128(Rp / 32 * a.F);
  } else {
    part[2] = align128(R * 2 * a.F * a.es);
  }
  const int64_t full = part[0] + part[1] + part[2] + part[3] + part[4];
  rec.layer = a.layer;
  rec.done = 1;
  auto to_scratch = [&]() {
    rec.x_rows = 0;
    rec.h1 = a.scratch_h1;
    for (int i = 0; i < 4; ++i) rec.aux[i] = a.scratch_aux[i];
  };
  if (!a.training || a.arena == 0) {
    rec.start = 0;
    rec.bytes = 0;
    rec.replay = a.training ? 1 : 0;
    to_scratch();
    return;
  }
  ArenaHdr* ah = reinterpret_cast<ArenaHdr*>(a.arena);
  if (a.layer == 0) ah->cursor = 0;
  const int64_t cursor = ah->cursor;
  const int64_t keep = 0;
  const int64_t remaining = int64_t(a.max_layers - 1 - a.layer);
  const bool replay = cursor + full + remaining * keep > a.budget;
  rec.start = cursor;
  rec.replay = replay ? 1 : 0;
  if (replay) {
    rec.bytes = keep;
    to_scratch();
  } else {
    rec.bytes = full;
    const uint64_t base = a.arena + uint64_t(kArenaHdrBytes) + uint64_t(cursor);
    rec.x_rows = 0;
    rec.aux[0] = base;
    rec.aux[1] = base + uint64_t(part[0]);
    rec.h1 = base + uint64_t(part[0] + part[1]);
    rec.aux[2] = rec.h1 + uint64_t(part[2]);
    rec.aux[3] = rec.aux[2] + uint64_t(part[3]);
  }
  ah->cursor = cursor + rec.bytes;
}

// First launch of a backward.  If no forward of this layer ran since its
// routing (rec.done == 0), the record's pointers are not this call's: report
// it (MOE_STATUS_ARENA) and turn the layer into a replaying one, so that the
// backward rebuilds its forward state from x in scratch, as for a layer the
// planner chose to replay, instead of reading through stale pointers.
__global__ void k_plan_enter_bwd(RouteHdr* __restrict__ hdr, PlanArgs a) {
  if (a.zero) {   // the fused backward's tickets and counters
    uint32_t* z = reinterpret_cast<uint32_t*>(a.zero);
    for (int i = threadIdx.x; i < a.zero_n; i += blockDim.x) z[i] = 0u;
  }
  if (threadIdx.x != 0) return;
  LayerRec& rec = hdr->rec;
  if (rec.done) return;
  hdr->status |= MOE_STATUS_ARENA;
  rec.start = a.arena ? reinterpret_cast<ArenaHdr*>(a.arena)->cursor : 0;
  rec.bytes = 0;
  rec.replay = 1;
  rec.layer = a.layer;
  rec.x_rows = 0;
  rec.h1 = a.scratch_h1;
  for (int i = 0; i < 4; ++i) rec.aux[i] = a.scratch_aux[i];
  rec.done = 1;
}

// Backward rewinds the cursor to the layer's start (reverse layer order).
__global__ void k_plan_rewind(RouteHdr* __restrict__ hdr, uint64_t arena) {
  if (threadIdx.x != 0) return;
  if (!hdr->rec.done) hdr->status |= MOE_STATUS_ARENA;
  if (arena) reinterpret_cast<ArenaHdr*>(arena)->cursor = hdr->rec.start;
}

__global__ void k_arena_reset(uint64_t arena) {
  if (threadIdx.x == 0) reinterpret_cast<ArenaHdr*>(arena)->cursor = 0;
}

// ------------------------------------------------------------ launchers
hipError_t launch_route(const int32_t* ids, int64_t T, int K, int E, char* ws,
                        const RouteLayout& L, hipStream_t s) {
  const int64_t n = T * K;
  if (n <= kSmallRoutes && E <= kMaxE) {
    hipLaunchKernelGGL(k_route_small, dim3(1), dim3(1024), 0, s, ids, int(n), E, int(T),
                       reinterpret_cast<int32_t*>(ws + L.counts),
                       reinterpret_cast<int32_t*>(ws + L.offsets),
                       reinterpret_cast<int32_t*>(ws + L.poffsets),
                       reinterpret_cast<int32_t*>(ws + L.mtoff),
                       reinterpret_cast<int32_t*>(ws + L.gtoff),
                       reinterpret_cast<int32_t*>(ws + L.cstoff),
                       reinterpret_cast<int32_t*>(ws + L.sorted_route),
                       reinterpret_cast<int32_t*>(ws + L.route_to_row),
                       reinterpret_cast<RouteHdr*>(ws + L.hdr));
    return hipGetLastError();
  }
  const int nchunks = int((n + kRankChunk - 1) / kRankChunk);
  if (n <= kChunkedRoutes && E <= kChunkedMaxE) {
    hipLaunchKernelGGL(k_route_chunked, dim3(nchunks), dim3(kRankChunk), (6 * E + 2) * sizeof(int32_t),
                       s, ids, int(n), E, int(T),
                       reinterpret_cast<int32_t*>(ws + L.counts),
                       reinterpret_cast<int32_t*>(ws + L.offsets),
                       reinterpret_cast<int32_t*>(ws + L.poffsets),
                       reinterpret_cast<int32_t*>(ws + L.mtoff),
                       reinterpret_cast<int32_t*>(ws + L.gtoff),
                       reinterpret_cast<int32_t*>(ws + L.cstoff),
                       reinterpret_cast<int32_t*>(ws + L.sorted_route),
                       reinterpret_cast<int32_t*>(ws + L.route_to_row),
                       reinterpret_cast<RouteHdr*>(ws + L.hdr));
    return hipGetLastError();
  }
  int32_t* hist = reinterpret_cast<int32_t*>(ws + L.chunk_hist);
  int32_t* flags = reinterpret_cast<int32_t*>(ws + L.chunk_flags);
  if (nchunks > 0)
    hipLaunchKernelGGL(k_route_hist, dim3(nchunks), dim3(256), E * sizeof(int32_t), s, ids, n, E,
                       hist, flags);
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, s, hist, flags, nchunks, E, int(T),
                     reinterpret_cast<int32_t*>(ws + L.counts),
                     reinterpret_cast<int32_t*>(ws + L.offsets),
                     reinterpret_cast<int32_t*>(ws + L.poffsets),
                     reinterpret_cast<int32_t*>(ws + L.mtoff),
                     reinterpret_cast<int32_t*>(ws + L.gtoff),
                     reinterpret_cast<int32_t*>(ws + L.cstoff),
                     reinterpret_cast<RouteHdr*>(ws + L.hdr));
  if (nchunks > 0)
    hipLaunchKernelGGL(k_route_rank, dim3(nchunks), dim3(256), 0, s, ids, n, E, hist,
                       reinterpret_cast<int32_t*>(ws + L.sorted_route),
                       reinterpret_cast<int32_t*>(ws + L.route_to_row));
  return hipGetLastError();
}

hipError_t launch_plan_decide(RouteHdr* hdr, const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_plan_decide, dim3(1), dim3(64), 0, s, hdr, a);
  return hipGetLastError();
}

hipError_t launch_plan_enter_bwd(RouteHdr* hdr, const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_plan_enter_bwd, dim3(1), dim3(64), 0, s, hdr, a);
  return hipGetLastError();
}

hipError_t launch_plan_rewind(RouteHdr* hdr, void* arena, hipStream_t s) {
  hipLaunchKernelGGL(k_plan_rewind, dim3(1), dim3(64), 0, s, hdr, uint64_t(arena));
  return hipGetLastError();
}

hipError_t launch_arena_reset(void* arena, hipStream_t s) {
  hipLaunchKernelGGL(k_arena_reset, dim3(1), dim3(64), 0, s, uint64_t(arena));
  return hipGetLastError();
}

}  // namespace moe
