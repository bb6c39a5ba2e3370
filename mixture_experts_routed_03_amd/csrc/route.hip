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
// Deterministic counting sort in three launches:
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

// Inclusive block scan of one int per thread (blockDim.x == 1024).
__device__ int block_scan_incl(int v, int* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int add = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  int res = sh[tid];
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(1024) void k_route_scan(int32_t* __restrict__ chunk_hist,
                                                     const int32_t* __restrict__ chunk_flags,
                                                     int nchunks, int E, int T,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ poffsets,
                                                     int32_t* __restrict__ mtoff,
                                                     RouteHdr* __restrict__ hdr) {
  __shared__ int sh[1024];
  __shared__ int tot[3];
  __shared__ int red[2];
  const int tid = threadIdx.x;
  // Each thread owns up to kMaxE/1024 = 4 consecutive experts.
  constexpr int per = kMaxE / 1024;
  int cnt[per];
  int sc = 0, sp = 0, sm = 0, mx = 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    int s = 0;
    if (e < E)
      for (int c = 0; c < nchunks; ++c) s += chunk_hist[int64_t(c) * E + e];
    cnt[i] = s;
    sc += s;
    sp += (s + kMxBlock - 1) / kMxBlock * kMxBlock;
    sm += (s + kBM - 1) / kBM;
    mx = max(mx, s);
  }
  const int ic = block_scan_incl(sc, sh);
  const int ip = block_scan_incl(sp, sh);
  const int im = block_scan_incl(sm, sh);
  int oc = ic - sc, op = ip - sp, om = im - sm;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < E) {
      counts[e] = cnt[i];
      offsets[e] = oc;
      poffsets[e] = op;
      mtoff[e] = om;
      // chunk histograms -> row base of each (chunk, expert)
      int run = oc;
      for (int c = 0; c < nchunks; ++c) {
        const int h = chunk_hist[int64_t(c) * E + e];
        chunk_hist[int64_t(c) * E + e] = run;
        run += h;
      }
    }
    oc += cnt[i];
    op += (cnt[i] + kMxBlock - 1) / kMxBlock * kMxBlock;
    om += (cnt[i] + kBM - 1) / kBM;
  }
  if (tid == 1023) {
    tot[0] = ic;
    tot[1] = ip;
    tot[2] = im;
  }
  // status and max count
  int f = 0;
  for (int c = tid; c < nchunks; c += 1024) f |= chunk_flags[c];
  if (tid == 0) {
    red[0] = 0;
    red[1] = 0;
  }
  __syncthreads();
  atomicOr(&red[0], f);
  atomicMax(&red[1], mx);
  __syncthreads();
  if (tid == 0) {
    offsets[E] = tot[0];
    poffsets[E] = tot[1];
    mtoff[E] = tot[2];
    hdr->T = T;
    hdr->R = tot[0];
    hdr->Rpad = tot[1];
    hdr->n_mt = tot[2];
    hdr->status = uint32_t(red[0]);
    hdr->max_count = red[1];
    hdr->rec.done = 0;
  }
}

__global__ __launch_bounds__(256) void k_route_rank(const int32_t* __restrict__ ids, int64_t n,
                                                    int E, const int32_t* __restrict__ chunk_base,
                                                    int32_t* __restrict__ sorted_route,
                                                    int32_t* __restrict__ route_to_row) {
  __shared__ int32_t sid[kRankChunk];
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t r = int64_t(c) * kRankChunk + tid;
  int id = r < n ? ids[r] : -1;
  const bool valid = id >= 0 && id < E;
  sid[tid] = valid ? id : -1;
  __syncthreads();
  if (r >= n) return;
  if (!valid) {
    route_to_row[r] = -1;
    return;
  }
  // Earlier routes of the same expert inside this chunk.  Every lane reads
  // the same LDS word per step (broadcast), so the loop is conflict-free.
  int rank = 0;
  for (int q = 0; q < tid; ++q) rank += (sid[q] == id);
  const int row = chunk_base[int64_t(c) * E + id] + rank;
  sorted_route[row] = int32_t(r);
  route_to_row[r] = row;
}

// ------------------------------------------------------------ planner
// Dist-MoE explainer section 04: before saving a layer's full state the
// planner replays instead when saved bytes + this layer's full state +
// remaining layers x replay-input bytes exceed the slot capacity; a layer
// that replays keeps only its replay input (here none: x stays with the
// caller).  Equality saves.  Layer 0 starts the step at cursor 0.
__global__ void k_plan_decide(RouteHdr* __restrict__ hdr, PlanArgs a) {
  if (threadIdx.x != 0) return;
  LayerRec& rec = hdr->rec;
  const int64_t R = hdr->R;
  const int64_t Rp = hdr->Rpad;
  // Saved state of the layer.  BF16/FP32: gathered x rows and h1.  MXFP8
  // (explainer section 04, MXFP8 full-save): x and h2 column bundles (codes +
  // exponents) and dense h1; the gathered bf16 rows stay in scratch.
  int64_t part[5] = {0, 0, 0, 0, 0};
  if (a.mx) {
    part[0] = align128(Rp * a.D);
    part[1] = align128(Rp / 32 * a.D);
    part[2] = align128(R * 2 * a.F * 2);
    part[3] = align128(Rp * a.F);
    part[4] = align128(Rp / 32 * a.F);
  } else {
    part[0] = align128(R * a.D * a.es);
    part[2] = align128(R * 2 * a.F * a.es);
  }
  const int64_t full = part[0] + part[1] + part[2] + part[3] + part[4];
  rec.layer = a.layer;
  rec.done = 1;
  auto to_scratch = [&]() {
    rec.x_rows = a.scratch_x_rows;
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
    if (a.mx) {
      rec.x_rows = a.scratch_x_rows;
      rec.aux[0] = base;
      rec.aux[1] = base + uint64_t(part[0]);
      rec.h1 = base + uint64_t(part[0] + part[1]);
      rec.aux[2] = rec.h1 + uint64_t(part[2]);
      rec.aux[3] = rec.aux[2] + uint64_t(part[3]);
    } else {
      rec.x_rows = base;
      rec.h1 = base + uint64_t(part[0]);
    }
  }
  ah->cursor = cursor + rec.bytes;
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
  const int nchunks = int((n + kRankChunk - 1) / kRankChunk);
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

hipError_t launch_plan_rewind(RouteHdr* hdr, void* arena, hipStream_t s) {
  hipLaunchKernelGGL(k_plan_rewind, dim3(1), dim3(64), 0, s, hdr, uint64_t(arena));
  return hipGetLastError();
}

hipError_t launch_arena_reset(void* arena, hipStream_t s) {
  hipLaunchKernelGGL(k_arena_reset, dim3(1), dim3(64), 0, s, uint64_t(arena));
  return hipGetLastError();
}

}  // namespace moe
