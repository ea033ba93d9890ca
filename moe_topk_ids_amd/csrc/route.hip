// Routing / permutation: groups the T*K (token, k) slots by expert in the
// stable token-major, k-minor order in which tpu-inference's fused_moe
// kernel (kernel.py, start_a2a_scatter) fills its per-expert buffers, and
// pads every expert's group to the GEMM row tile.
//
// Up to kRouteOnePassMaxSlots slots (and kRouteOnePassMaxExperts experts), one
// launch (route_onepass): workgroup g ranks slots [1024 g, 1024 g + 1024),
// one 64-slot chunk per wave, and counts every other workgroup's slots
// itself, so it knows its experts' starting rows without waiting for any
// other workgroup. Every lane loads its ids (at most 16) at once: the kernel
// pays one memory latency.
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

constexpr int kOnePassThreads = 1024;
constexpr int kOnePassWaves = kOnePassThreads / 64;
constexpr int64_t kOnePassGroupSlots = kOnePassWaves * 64;  // one 64-slot chunk per wave
constexpr int kOnePassBatch = 16;  // workgroups' chunks loaded together for counting
// With at most 32 experts the counts are kept in 4 copies, lane l adding to
// copy l % 4, so that fewer lanes of one atomic instruction hit the same LDS
// word (large, E=8: 10.5 -> 8.7 us); with more experts the lanes already
// spread and the extra LDS to clear and sum cost 0.5-2 us.
__host__ __device__ inline int onepass_sub(int32_t E) { return E <= 32 ? 4 : 1; }

// Loads this wave's chunk of workgroups i0 .. i0+B-1 (those below G); -1 for
// slots past the end.
template <int B>
__device__ __forceinline__ void onepass_load(int32_t (&v)[B], const int32_t* __restrict__ ids,
                                             int64_t n_slots, int i0, int G, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < B; ++j) {
    v[j] = -1;
    if (i0 + j >= G) break;  // uniform
    const int64_t f = ((int64_t)(i0 + j) * kOnePassWaves + wave) * 64 + lane;
    if (f < n_slots) v[j] = ids[f];
  }
}

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

// Inclusive prefix sum over the wave: DPP row shifts inside each row of 16
// lanes, then row broadcasts of lanes 15 and 31 into the later rows.
__device__ __forceinline__ int32_t wave_inclusive_scan_i32(int32_t v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// One launch of G = ceil(n / 1024) workgroups. Workgroup g ranks the slots
// [1024 g, 1024 g + 1024), one 64-slot chunk per wave; it learns where its
// slots go by counting every other workgroup's slots itself (order-free LDS
// atomics over ids it loads from L2), so no workgroup waits for another. The
// counting grows as G * n over the chip, which bounds n.
__global__ __launch_bounds__(kOnePassThreads) void route_onepass(
    const int32_t* __restrict__ ids, int64_t n_slots, int32_t E, int32_t M,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
    int32_t* __restrict__ slot_of, int32_t* __restrict__ tile_expert,
    int32_t* __restrict__ num_tiles) {
  // LDS: pre[E][sub] (slots of each expert before this workgroup's range),
  // tot[E][sub] (those after it; then tot[e][0] holds the expert's total),
  // run[kOnePassWaves][E] (each wave's count in its chunk, then where the
  // wave's group starts inside the expert), off[E+1] (padded offsets)
  extern __shared__ int32_t lds[];
  const int sub = onepass_sub(E);
  int32_t* pre = lds;
  int32_t* tot = pre + sub * E;
  int32_t* run = tot + sub * E;
  int32_t* off = run + kOnePassWaves * E;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = blockIdx.x;
  const int G = gridDim.x;

  // the own chunk and the first batch of the others' loaded up front (one
  // memory latency for up to 16 workgroups)
  const int64_t own = ((int64_t)g * kOnePassWaves + wave) * 64 + lane;
  const int32_t e = own < n_slots ? ids[own] : -1;
  int32_t cur[kOnePassBatch], nxt[kOnePassBatch];
  onepass_load(cur, ids, n_slots, 0, G, wave, lane);
#pragma unroll
  for (int j = 0; j < kOnePassBatch; ++j) nxt[j] = -1;
  for (int i = tid; i < (2 * sub + kOnePassWaves) * E; i += kOnePassThreads) lds[i] = 0;
  __syncthreads();

  // 1. the other workgroups' slots, counted before / after this range; the
  //    next batch loads while this one is counted
  for (int i0 = 0; i0 < G; i0 += kOnePassBatch) {
    if (i0 + kOnePassBatch < G) onepass_load(nxt, ids, n_slots, i0 + kOnePassBatch, G, wave, lane);
#pragma unroll
    for (int j = 0; j < kOnePassBatch; ++j) {
      const int i = i0 + j;
      if (i >= G) break;  // uniform
      const int32_t x = cur[j];
      if (i != g && x >= 0 && x < E)
        atomicAdd((i < g ? pre : tot) + x * sub + (lane & (sub - 1)), 1);
    }
#pragma unroll
    for (int j = 0; j < kOnePassBatch; ++j) cur[j] = nxt[j];
  }
  // 2. the own chunk ranked by ballot (lowest lane first among equal ids);
  //    the group's first lane records the wave's count of that expert
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const bool valid = e >= 0 && e < E;
  uint64_t mask = __ballot(valid);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool set = valid && ((e >> bit) & 1);
    const uint64_t bm = __ballot(set);
    mask &= set ? bm : ~bm;
  }
  const int32_t rank = __popcll(mask & lanemask_lt());
  if (valid && rank == 0) run[wave * E + e] = __popcll(mask);
  __syncthreads();

  // 3. in wave 0: per expert the waves' starts (after the earlier
  //    workgroups' slots) and the total, then an exclusive scan of the padded
  //    totals over experts; lane l owns experts l*EPL .. l*EPL+EPL-1
  if (wave == 0) {
    const int epl = (E + 63) / 64;
    int32_t lane_sum = 0;
    for (int q = 0; q < epl; ++q) {
      const int x = lane * epl + q;
      if (x >= E) break;
      int32_t cw[kOnePassWaves];
#pragma unroll
      for (int w = 0; w < kOnePassWaves; ++w) cw[w] = run[w * E + x];
      int32_t a = 0, after = 0;
      for (int c = 0; c < sub; ++c) {
        a += pre[x * sub + c];
        after += tot[x * sub + c];
      }
#pragma unroll
      for (int w = 0; w < kOnePassWaves; ++w) {
        run[w * E + x] = a;
        a += cw[w];
      }
      a += after;
      tot[x * sub] = a;
      lane_sum += (a + M - 1) / M * M;
    }
    const int32_t incl = wave_inclusive_scan_i32(lane_sum);
    int32_t acc = incl - lane_sum;
    for (int q = 0; q < epl; ++q) {
      const int x = lane * epl + q;
      if (x >= E) break;
      off[x] = acc;
      acc += (tot[x * sub] + M - 1) / M * M;
    }
    if (lane == 63) off[E] = incl;
  }
  __syncthreads();

  // 4. metadata from workgroup 0; pad rows and the tile->expert map of
  //    expert x from workgroup x % G
  if (g == 0) {
    for (int x = tid; x < E; x += kOnePassThreads) counts[x] = tot[x * sub];
    for (int x = tid; x <= E; x += kOnePassThreads) offsets[x] = off[x];
    if (tid == 0) num_tiles[0] = off[E] / M;
  }
  for (int x = g + G * wave; x < E; x += G * kOnePassWaves) {
    const int32_t start = off[x], padded = off[x + 1] - off[x];
    for (int32_t j = lane; j < padded / M; j += 64) tile_expert[start / M + j] = (int32_t)x;
    for (int32_t r = tot[x * sub] + lane; r < padded; r += 64) sorted[start + r] = -1;
  }

  // 5. scatter: row = expert start + the wave's start + place in the chunk
  const int64_t f = ((int64_t)g * kOnePassWaves + wave) * 64 + lane;
  if (f < n_slots) {
    if (valid) {
      const int32_t pos = off[e] + run[wave * E + e] + rank;
      sorted[pos] = (int32_t)f;
      slot_of[f] = pos;
    } else {
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
  if (n <= kRouteOnePassMaxSlots && E <= kRouteOnePassMaxExperts) {
    const size_t lds =
        (size_t)((2 * onepass_sub((int32_t)E) + kOnePassWaves) * E + E + 1) * sizeof(int32_t);
    const int groups = (int)((n + kOnePassGroupSlots - 1) / kOnePassGroupSlots);
    route_onepass<<<dim3(groups), dim3(kOnePassThreads), lds, stream>>>(
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
