// Routing / permutation: groups the T*K (token, k) slots by expert in the
// stable token-major, k-minor order in which tpu-inference's fused_moe
// kernel (kernel.py, start_a2a_scatter) fills its per-expert buffers, and
// pads every expert's group to the GEMM row tile.
//
// Up to kRouteSingleMaxSlots slots (and kRouteSingleMaxExperts experts) one
// workgroup of 16 waves does everything in a single launch (route_single):
// every lane loads its (at most 32) ids at once, so the kernel pays one
// memory latency, and ranking, counting and the scatter work from registers.
//
// Above that, two launches, no atomics on the ordering path:
//   route_count    per workgroup, a per-expert histogram of its slot range
//                  (LDS atomics: counts do not depend on order);
//   route_scatter  every workgroup rebuilds the prefix sums it needs from the
//                  histograms (a few KB from L2), then ranks its slots with
//                  wave ballots so equal experts keep ascending slot order.
// Workgroup 0 publishes counts/offsets/num_tiles; pad rows and the
// tile->expert map are spread over the workgroups by expert.
//
// Both forms rank slots the same way: each wave owns a contiguous, ordered
// range of slots, waves are ordered by range, and inside a wave a 64-slot
// chunk is ranked by ballot with the lowest lane first.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = kRouteThreads / 64;

__global__ __launch_bounds__(kRouteThreads) void route_count(
    const int32_t* __restrict__ ids, int64_t n_slots, int32_t E, int64_t rb,
    int32_t* __restrict__ block_hist) {
  extern __shared__ int32_t hist[];  // [E]
  const int tid = threadIdx.x;
  const int64_t nblk = gridDim.x;
  for (int e = tid; e < E; e += kRouteThreads) hist[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * rb;
  for (int64_t i = tid; i < rb; i += kRouteThreads) {
    const int64_t f = base + i;
    if (f >= n_slots) break;
    const int32_t e = ids[f];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) block_hist[(int64_t)e * nblk + blockIdx.x] = hist[e];
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int32_t dpp_add_i32(int32_t v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, false);
}

// Sum over the wave (DPP moves, as group_sum in device_util.h), returned in
// every lane.
__device__ __forceinline__ int32_t wave_sum_i32(int32_t v) {
  v = dpp_add_i32<0xB1>(v);
  v = dpp_add_i32<0x4E>(v);
  v = dpp_add_i32<0x141>(v);
  v = dpp_add_i32<0x140>(v);
  v = dpp_add_i32<0x142, 0xA>(v);
  v = dpp_add_i32<0x143, 0xC>(v);
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ inline uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

constexpr int kSingleThreads = 1024;
constexpr int kSingleWaves = kSingleThreads / 64;
constexpr int kSingleChunks = (int)(kRouteSingleMaxSlots / (kSingleWaves * 64));  // per lane

__device__ inline void rank_and_scatter(const int32_t* __restrict__ ids, int64_t n_slots,
                                        int32_t E, int64_t wbase, int64_t per_wave,
                                        int32_t* myrun, int32_t* __restrict__ sorted,
                                        int32_t* __restrict__ slot_of) {
  const int lane = threadIdx.x & 63;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  for (int64_t c0 = 0; c0 < per_wave; c0 += 64) {
    const int64_t f = wbase + c0 + lane;
    const bool in = (c0 + lane < per_wave) && (f < n_slots);
    const int32_t e = in ? ids[f] : -1;
    const bool valid = in && e >= 0 && e < E;
    uint64_t mask = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = valid && ((e >> bit) & 1);
      const uint64_t bm = __ballot(set);
      mask &= set ? bm : ~bm;
    }
    if (valid) {
      const int32_t rank = __popcll(mask & lanemask_lt());
      const int32_t pos = myrun[e] + rank;
      sorted[pos] = (int32_t)f;
      slot_of[f] = pos;
      if (rank == 0) myrun[e] = pos + __popcll(mask);
    } else if (in) {
      slot_of[f] = -1;
    }
  }
}

__global__ __launch_bounds__(kRouteThreads) void route_scatter(
    const int32_t* __restrict__ ids, int64_t n_slots, int32_t E, int32_t M, int64_t rb,
    const int32_t* __restrict__ block_hist, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted, int32_t* __restrict__ slot_of,
    int32_t* __restrict__ tile_expert, int32_t* __restrict__ num_tiles) {
  // LDS: tot[E], off[E+1], pre[E], run[kWaves][E], part[kRouteThreads]
  extern __shared__ int32_t lds[];
  int32_t* tot = lds;
  int32_t* off = tot + E;
  int32_t* pre = off + E + 1;
  int32_t* run = pre + E;
  __shared__ int32_t part[kRouteThreads];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int64_t nblk = gridDim.x;
  const int64_t b = blockIdx.x;

  // 1. per expert: total count and the count in earlier workgroups. A wave
  //    takes experts wave, wave + kWaves, ... in batches of kBatch; its lanes
  //    hold the histograms of workgroups lane and lane + 64 (at most
  //    kRouteMaxBlocks = 128 of them), all loaded before the first sum.
  constexpr int kBatch = 16;
  for (int eb = wave; eb < E; eb += kWaves * kBatch) {
    int32_t h0[kBatch], h1[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int e = eb + u * kWaves;
      const int32_t* h = block_hist + (int64_t)(e < E ? e : 0) * nblk;
      h0[u] = (e < E && lane < nblk) ? h[lane] : 0;
      h1[u] = (e < E && lane + 64 < nblk) ? h[lane + 64] : 0;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int e = eb + u * kWaves;
      const int32_t s = wave_sum_i32(h0[u] + h1[u]);
      const int32_t p = wave_sum_i32((lane < b ? h0[u] : 0) + (lane + 64 < b ? h1[u] : 0));
      if (lane == 0 && e < E) {
        tot[e] = s;
        pre[e] = p;
      }
    }
  }
  for (int i = tid; i < kWaves * E; i += kRouteThreads) run[i] = 0;
  __syncthreads();

  // 2. exclusive scan over experts of the padded counts
  const int per = (E + kRouteThreads - 1) / kRouteThreads;
  const int e0 = tid * per;
  int32_t local = 0;
  for (int e = e0; e < e0 + per && e < E; ++e) local += (tot[e] + M - 1) / M * M;
  part[tid] = local;
  __syncthreads();
  for (int d = 1; d < kRouteThreads; d <<= 1) {
    const int32_t v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t acc = part[tid] - local;
  for (int e = e0; e < e0 + per && e < E; ++e) {
    off[e] = acc;
    acc += (tot[e] + M - 1) / M * M;
  }
  if (tid == kRouteThreads - 1) off[E] = part[tid];
  __syncthreads();

  // 3. metadata: workgroup 0 publishes counts/offsets; pads and the
  //    tile->expert map are shared out by expert
  if (b == 0) {
    for (int e = tid; e < E; e += kRouteThreads) counts[e] = tot[e];
    for (int e = tid; e <= E; e += kRouteThreads) offsets[e] = off[e];
    if (tid == 0) num_tiles[0] = off[E] / M;
  }
  for (int64_t e = b; e < E; e += nblk) {
    const int32_t start = off[e], padded = off[e + 1] - off[e];
    for (int32_t j = tid; j < padded / M; j += kRouteThreads) tile_expert[start / M + j] = (int32_t)e;
    for (int32_t r = tot[e] + tid; r < padded; r += kRouteThreads) sorted[start + r] = -1;
  }

  // 4. per-wave counts over this workgroup's slot range, then each wave's
  //    first row per expert
  const int64_t per_wave = rb / kWaves;
  const int64_t wbase = b * rb + wave * per_wave;
  int32_t* myrun = run + wave * E;
  for (int64_t i = lane; i < per_wave; i += 64) {
    const int64_t f = wbase + i;
    if (f >= n_slots) break;
    const int32_t e = ids[f];
    if (e >= 0 && e < E) atomicAdd(&myrun[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) {
    int32_t a = off[e] + pre[e];
    for (int w = 0; w < kWaves; ++w) {
      const int32_t c = run[w * E + e];
      run[w * E + e] = a;
      a += c;
    }
  }
  __syncthreads();

  // 5. stable scatter: chunks of 64 slots in order; rank among equal ids by
  //    ballot, lowest lane first
  rank_and_scatter(ids, n_slots, E, wbase, per_wave, myrun, sorted, slot_of);
}

__global__ __launch_bounds__(kSingleThreads) void route_single(
    const int32_t* __restrict__ ids, int64_t n_slots, int32_t E, int32_t M,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
    int32_t* __restrict__ slot_of, int32_t* __restrict__ tile_expert,
    int32_t* __restrict__ num_tiles) {
  // LDS: run[kSingleWaves][E] (per-wave counts, then each wave's first row
  // per expert), tot[E], off[E+1]
  extern __shared__ int32_t lds[];
  int32_t* run = lds;
  int32_t* tot = run + kSingleWaves * E;
  int32_t* off = tot + E;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;

  // every id of the wave's contiguous, 64-aligned slot range is loaded up
  // front (one memory latency for the whole kernel)
  const int64_t per_wave = ((n_slots + kSingleWaves - 1) / kSingleWaves + 63) / 64 * 64;
  const int64_t wbase = (int64_t)wave * per_wave;
  int32_t idr[kSingleChunks];
#pragma unroll
  for (int c = 0; c < kSingleChunks; ++c) {
    const int64_t f = wbase + c * 64 + lane;
    idr[c] = (c * 64 < per_wave && f < n_slots) ? ids[f] : -1;
  }
  for (int i = tid; i < kSingleWaves * E; i += kSingleThreads) run[i] = 0;
  __syncthreads();

  // 1. rank each chunk by ballot (lowest lane first among equal ids); the
  //    group's first lane bumps the wave's count of that expert, and the
  //    value it read is the group's start inside the wave
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  int32_t* myrun = run + wave * E;
#pragma unroll
  for (int c = 0; c < kSingleChunks; ++c) {
    if (c * 64 >= per_wave) break;  // uniform
    const int32_t e = idr[c];
    const bool valid = e >= 0 && e < E;
    uint64_t mask = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = valid && ((e >> bit) & 1);
      const uint64_t bm = __ballot(set);
      mask &= set ? bm : ~bm;
    }
    const int32_t rank = __popcll(mask & lanemask_lt());
    int32_t start = 0;
    if (valid && rank == 0) start = atomicAdd(&myrun[e], __popcll(mask));
    const int leader = valid ? __ffsll((long long)mask) - 1 : lane;
    start = __shfl(start, leader, 64);
    // keep (place in the wave, expert) in the id's register: place < 2048,
    // expert < 512
    idr[c] = valid ? ((start + rank) << 11) | e : -1;
  }
  __syncthreads();

  // 2. and 3. in wave 0: per expert the total and each wave's exclusive
  //    prefix inside the expert (the 16 per-wave counts read together), then
  //    an exclusive scan of the padded counts over experts with shuffles;
  //    lane l owns experts l*EPL .. l*EPL+EPL-1
  if (wave == 0) {
    const int epl = (E + 63) / 64;
    int32_t lane_sum = 0;
    for (int q = 0; q < epl; ++q) {
      const int e = lane * epl + q;
      if (e >= E) break;
      int32_t cw[kSingleWaves];
#pragma unroll
      for (int w = 0; w < kSingleWaves; ++w) cw[w] = run[w * E + e];
      int32_t a = 0;
#pragma unroll
      for (int w = 0; w < kSingleWaves; ++w) {
        run[w * E + e] = a;
        a += cw[w];
      }
      tot[e] = a;
      lane_sum += (a + M - 1) / M * M;
    }
    int32_t incl = lane_sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    int32_t acc = incl - lane_sum;
    for (int q = 0; q < epl; ++q) {
      const int e = lane * epl + q;
      if (e >= E) break;
      off[e] = acc;
      acc += (tot[e] + M - 1) / M * M;
    }
    if (lane == 63) off[E] = incl;
  }
  __syncthreads();

  // 4. metadata, pad rows, tile->expert map
  for (int e = tid; e < E; e += kSingleThreads) counts[e] = tot[e];
  for (int e = tid; e <= E; e += kSingleThreads) offsets[e] = off[e];
  if (tid == 0) num_tiles[0] = off[E] / M;
  for (int e = wave; e < E; e += kSingleWaves) {
    const int32_t start = off[e], padded = off[e + 1] - off[e];
    for (int32_t j = lane; j < padded / M; j += 64) tile_expert[start / M + j] = (int32_t)e;
    for (int32_t r = tot[e] + lane; r < padded; r += 64) sorted[start + r] = -1;
  }

  // 5. scatter: row = expert start + earlier waves' count + place in the wave
#pragma unroll
  for (int c = 0; c < kSingleChunks; ++c) {
    if (c * 64 >= per_wave) break;  // uniform
    const int64_t f = wbase + c * 64 + lane;
    const bool in = f < n_slots;
    const int32_t v = idr[c];
    if (in && v >= 0) {
      const int32_t e = v & 0x7ff;
      const int32_t pos = off[e] + run[wave * E + e] + (v >> 11);
      sorted[pos] = (int32_t)f;
      slot_of[f] = pos;
    } else if (in) {
      slot_of[f] = -1;
    }
  }
}

__global__ __launch_bounds__(kRouteThreads) void validate_ids(const int32_t* __restrict__ ids,
                                                             int64_t n_slots, int32_t K, int32_t E,
                                                             int32_t* __restrict__ err_flag) {
  const int64_t f = (int64_t)blockIdx.x * kRouteThreads + threadIdx.x;
  if (f >= n_slots) return;
  const int32_t e = ids[f];
  int bad = !(e >= 0 && e < E);
  for (int64_t g = f - f % K; g < f; ++g) bad |= (ids[g] == e);
  if (bad) atomicOr(err_flag, 1);
}

}  // namespace

hipError_t launch_validate_ids(const int32_t* ids, int64_t T, int64_t K, int64_t E,
                               int32_t* err_flag, hipStream_t stream) {
  const int64_t n = T * K;
  if (n == 0) return hipSuccess;
  validate_ids<<<dim3((unsigned)((n + kRouteThreads - 1) / kRouteThreads)), dim3(kRouteThreads), 0,
                 stream>>>(ids, n, (int32_t)K, (int32_t)E, err_flag);
  return hipGetLastError();
}

hipError_t launch_route(const int32_t* ids, int64_t T, int64_t K, int64_t E, int32_t m_tile,
                        int32_t* block_hist, int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* slot_of,
                        int32_t* tile_expert, int32_t* num_tiles, hipStream_t stream) {
  const int64_t n = T * K;
  if (n == 0) return hipSuccess;
  if (n <= kRouteSingleMaxSlots && E <= kRouteSingleMaxExperts) {
    const size_t lds = (size_t)(kSingleWaves * E + E + E + 1) * sizeof(int32_t);
    route_single<<<dim3(1), dim3(kSingleThreads), lds, stream>>>(
        ids, n, (int32_t)E, m_tile, counts, offsets, sorted, slot_of, tile_expert, num_tiles);
    return hipGetLastError();
  }
  const int64_t rb = route_block_slots(n);
  const int64_t nblk = route_blocks(n);
  route_count<<<dim3((unsigned)nblk), dim3(kRouteThreads), E * sizeof(int32_t), stream>>>(
      ids, n, (int32_t)E, rb, block_hist);
  hipError_t st = hipGetLastError();
  if (st != hipSuccess) return st;
  const size_t lds = (size_t)(E + E + 1 + E + kWaves * E) * sizeof(int32_t);
  route_scatter<<<dim3((unsigned)nblk), dim3(kRouteThreads), lds, stream>>>(
      ids, n, (int32_t)E, m_tile, rb, block_hist, counts, offsets, sorted, slot_of, tile_expert,
      num_tiles);
  return hipGetLastError();
}

}  // namespace moe
