// C ABI of the fused MoE forward: argument validation, workspace layout and
// ownership, path choice and the launch sequence. Declarations and the
// contract of every entry point are in include/moe_topk_ids.h.
//
// Argument rules follow the ones tpu-inference's fused_moe wrapper raises
// errors for (top_k within (0, num_experts], hidden and intermediate sizes
// 128-aligned); errors are reported as codes plus a per-thread message, in
// the manner of the metrale forward_k2 dispatch refusing unsupported setups
// with a reason instead of running.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/moe_topk_ids.h"
#include "moe_internal.h"

namespace {

thread_local std::string g_last_error;

int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_error(const char* what, hipError_t st) {
  return set_error(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(st));
}

// Path choice, from a measured sweep of T = 1..512 on four expert shapes
// (H/I/E/top-k 2048/768/128/8, 2048/2048/8/2, 4096/384/128/8,
// 4096/4096/8/2) with uniform routing:
//  - per-token streaming (two kernels, no combine) is fastest while slots
//    rarely share an expert: T*K <= max(K, E/2);
//  - the per-expert small-batch path streams each routed expert once, like
//    the grouped path, but spends about 1.4e-7 us per T*K*H*I on its vector
//    dot products; it wins until that reaches the grouped path's extra cost
//    over streaming the weights (routing, sparse tiles, the slot rows):
//    about 24 us + 0.065 us per MB of routed weights with bf16 weights (the
//    sweep repeated on the current kernels put the crossovers at T ~ 28 for
//    2048/2048/8/2, ~ 56 for 2048/768/128/8, ~ 40 for 4096/384/128/8 and
//    ~ 20 for 4096/4096/8/2), and 60 us + 0.06 us per MB as first fitted
//    with FP8 weights, where the grouped path adds its widening cost;
//  - the grouped MFMA path beyond.
constexpr double kSmallBatchUsPerWork = 1.4e-7;
constexpr double kGroupedFixedUs = 24.0;
constexpr double kGroupedUsPerWeightMB = 0.065;
constexpr double kGroupedFixedUsFp8 = 60.0;
constexpr double kGroupedUsPerWeightMBFp8 = 0.06;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int check_sizes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K) {
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || K <= 0)
    return set_error(MOE_ERR_INVALID_ARG,
                     "sizes must be positive (T may be 0): T=%lld H=%lld I=%lld E=%lld K=%lld",
                     (long long)T, (long long)H, (long long)I, (long long)E, (long long)K);
  if (K > E)
    return set_error(MOE_ERR_INVALID_ARG, "top_k=%lld must not exceed num_experts=%lld",
                     (long long)K, (long long)E);
  if (E > moe::kMaxExperts)
    return set_error(MOE_ERR_UNSUPPORTED, "num_experts=%lld exceeds %d", (long long)E,
                     moe::kMaxExperts);
  if (H % 128 != 0 || I % 128 != 0)
    return set_error(MOE_ERR_UNSUPPORTED,
                     "hidden size %lld and intermediate size %lld must be multiples of 128",
                     (long long)H, (long long)I);
  if (T > (int64_t)INT32_MAX / K || T * K > (int64_t)1 << 30)
    return set_error(MOE_ERR_UNSUPPORTED, "T*K=%lld is too large", (long long)(T * K));
  // the GEMMs address the hidden states and one expert's weights through
  // 32-bit buffer offsets with bit 31 reserved for "out of range"
  if (T * H * 2 >= ((int64_t)1 << 31) || 3 * I * H * 2 >= ((int64_t)1 << 31))
    return set_error(MOE_ERR_UNSUPPORTED,
                     "hidden states (%lld bytes) and one expert's weights (%lld bytes) must each "
                     "be under 2 GiB",
                     (long long)(T * H * 2), (long long)(3 * I * H * 2));
  return MOE_OK;
}

// FP8 weights on the grouped path: either the GEMMs read code tiles and
// widen each fragment in registers, or one pass first widens every expert to
// bf16 and the bf16 GEMMs run unchanged. In-register widening is repeated by
// every row tile and wave that reads a weight tile: measured, it adds about
// 0.45 us per GFLOP with 64- and 128-row tiles and 0.19 us per GFLOP with
// 256-row tiles (more token rows per wave share each widened fragment). The
// widening pass costs about 0.55 us per million weights, for all E experts.
// So in-register widening wins with few rows per expert (many experts, few
// tokens); the pass wins for dense experts.
constexpr double kFp8InRegUsPerGflop128 = 0.45;
constexpr double kFp8InRegUsPerGflop256 = 0.19;
constexpr double kFp8WidenUsPerMWeight = 0.55;

double fp8_widen_us(int64_t H, int64_t I, int64_t E) {
  return kFp8WidenUsPerMWeight * 3.0 * (double)E * H * I * 1e-6;
}

double fp8_in_register_us(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K) {
  const int bm = moe::pick_gemm1_cfg(T, K, H, I, E).bm;
  // a widened weight fragment serves the wave's token fragments: 4 with
  // 256-row tiles, 3 with 192-row tiles (scaled from the 2 of the 128-row
  // measurement; not measured itself), 2 with the two-workgroup tiles
  const double per_gflop = bm == 256   ? kFp8InRegUsPerGflop256
                           : bm == 192 ? kFp8InRegUsPerGflop128 * 2.0 / 3.0
                                       : kFp8InRegUsPerGflop128;
  return per_gflop * 6.0 * (double)T * K * H * I * 1e-9;
}

// The grouped GEMMs can read FP8 tiles for every allowed block (a multiple
// of 128) while the tile's scales fit in LDS.
bool fp8_native_for_every_block(int64_t H, int64_t I) {
  return moe::fp8_gemm_supported(H, I, 128);
}

// Whether the grouped path widens FP8 fragments inside its GEMMs (else it
// runs the widening pass first).
bool fp8_grouped_in_gemm(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, int64_t block) {
  return moe::fp8_gemm_supported(H, I, block) &&
         fp8_in_register_us(T, H, I, E, K) < fp8_widen_us(H, I, E);
}

// Whether the grouped path needs room for the widened weights.
bool fp8_may_widen(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K) {
  return !fp8_native_for_every_block(H, I) ||
         fp8_widen_us(H, I, E) <= fp8_in_register_us(T, H, I, E, K);
}

int pick_path(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, uint32_t flags) {
  // with FP8 weights the streaming paths move half the bytes and the
  // grouped path first widens every expert's weights to bf16
  const bool fp8 = (flags & MOE_FLAG_FP8_WEIGHTS) != 0;
  const bool dec = fp8 ? moe::fp8_decode_supported(H, I, K) : moe::decode_supported(H, I, K);
  const bool sb = fp8 ? moe::fp8_small_batch_supported(T, H, I, K)
                      : moe::small_batch_supported(T, H, I, K);
  if ((flags & MOE_FLAG_FORCE_DECODE) && dec) return MOE_PATH_DECODE;
  if ((flags & MOE_FLAG_FORCE_SMALL_BATCH) && sb) return MOE_PATH_SMALL_BATCH;
  if (flags & (MOE_FLAG_FORCE_GROUPED | MOE_FLAG_FORCE_DECODE | MOE_FLAG_FORCE_SMALL_BATCH))
    return MOE_PATH_GROUPED;
  const int64_t slots = T * K;
  if (dec && slots <= std::max<int64_t>(K, E / 2)) return MOE_PATH_DECODE;
  const double routed_mb = (double)std::min<int64_t>(E, slots) * 6.0 * H * I / 1e6;
  const double sb_extra_us = kSmallBatchUsPerWork * (double)slots * H * I;
  // what FP8 weights add to the grouped path (the cheaper way of widening)
  const double dequant_us =
      !fp8 ? 0.0
           : fp8_native_for_every_block(H, I)
                 ? std::min(fp8_widen_us(H, I, E), fp8_in_register_us(T, H, I, E, K))
                 : fp8_widen_us(H, I, E);
  const double grouped_extra_us =
      fp8 ? kGroupedFixedUsFp8 + kGroupedUsPerWeightMBFp8 * routed_mb + dequant_us
          : kGroupedFixedUs + kGroupedUsPerWeightMB * routed_mb;
  if (sb && sb_extra_us <= grouped_extra_us)
    return MOE_PATH_SMALL_BATCH;
  return MOE_PATH_GROUPED;
}

// The gate/up tile the GEMM1 entry points run for routing arrays of row tile
// m_tile: the forward's own tile when m_tile is the one the forward picks for
// these sizes (so the entry point runs exactly the forward's kernel), else
// the default width for that row tile.
moe::GemmCfg gemm1_entry_cfg(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K,
                             int32_t m_tile) {
  const moe::GemmCfg fwd = moe::pick_gemm1_cfg(T, K, H, I, E);
  if (fwd.bm == m_tile) return fwd;
  return moe::GemmCfg{m_tile, m_tile == 128 ? 128 : 256};
}

// Whether the grouped path's slot rows are stored as bf16, given the
// contraction split the down projection would take with fp32 rows. The
// flags decide when set. Otherwise bf16 rows, half the bytes written by the
// down projection and read by the combine, unless the contraction is split
// (the few-token rows of the E=8 shapes, whose slot rows are small; a split
// needs fp32 partial rows summed before any rounding).
bool y_bf16_choice(int ks2, uint32_t flags) {
  if (flags & MOE_FLAG_ATOMIC_COMBINE) return false;
  if (flags & MOE_FLAG_BF16_Y) return true;
  if (flags & MOE_FLAG_FP32_Y) return false;
  return ks2 == 1;
}

bool use_decode(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, uint32_t flags) {
  return pick_path(T, H, I, E, K, flags) == MOE_PATH_DECODE;
}

// Byte offsets of every buffer inside one workspace.
struct Layout {
  int path = MOE_PATH_GROUPED;
  bool decode = false;
  moe::GemmCfg g1{}, g2{};
  int ks2 = 1;  // contraction split of the down projection
  bool y16 = false;  // slot rows stored as bf16
  bool tail = false;  // the down projection's last partial round as column halves
  int64_t cap = 0, max_tiles = 0, nblk = 0;
  bool widened = false;       // room for bf16 copies of FP8 weights (grouped path)
  size_t w1dq = 0, w2dq = 0;
  size_t err = 0, counts = 0, offsets = 0, num_tiles = 0, tile_expert = 0, sorted = 0,
         slot_of = 0, block_hist = 0, act = 0, y = 0, total = 0;
  // MOE_FLAG_DEBUG_SYNC: a guard band of kGuardBytes after every region,
  // filled before the first stage and checked after each one
  static constexpr int kMaxGuards = 16;
  int n_guards = 0;
  size_t guard[kMaxGuards] = {};
  const char* guard_after[kMaxGuards] = {};
};

constexpr size_t kGuardBytes = 256;
constexpr unsigned char kGuardByte = 0xA5;

Layout make_layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, uint32_t flags) {
  Layout L;
  const int64_t n = T * K;
  size_t p = 0;
  const bool guarded = (flags & MOE_FLAG_DEBUG_SYNC) != 0;
  auto take = [&](size_t bytes, const char* name) {
    const size_t at = p;
    p = align_up(p + bytes);
    if (guarded && L.n_guards < Layout::kMaxGuards) {
      L.guard[L.n_guards] = p;
      L.guard_after[L.n_guards++] = name;
      p += kGuardBytes;
    }
    return at;
  };
  L.err = take(sizeof(int32_t), "error flag");
  L.path = pick_path(T, H, I, E, K, flags);
  if (L.path == MOE_PATH_DECODE) {
    L.decode = true;
    L.act = take((size_t)n * I * 2, "act");
    L.total = p;
    return L;
  }
  if (L.path == MOE_PATH_SMALL_BATCH) {
    L.act = take((size_t)n * I * 2, "act");
    L.y = take((size_t)n * H * 4, "slot rows");
    L.total = p;
    return L;
  }
  L.g1 = moe::pick_gemm1_cfg(T, K, H, I, E);
  L.g2 = moe::pick_gemm2_cfg(n, H, I, E, L.g1.bm);
  // the atomic combine adds every tile's result to out: no partial sums there
  L.ks2 = (flags & MOE_FLAG_ATOMIC_COMBINE)
              ? 1
              : moe::pick_ksplit(L.g2, T, K, E, (H + L.g2.bn - 1) / L.g2.bn, I);
  L.y16 = y_bf16_choice(L.ks2, flags);
  if (L.y16) L.ks2 = 1;  // bf16 rows are whole sums, rounded once
  L.g2.ns = moe::pick_ring_stages(L.g2, T, K, E, (H + L.g2.bn - 1) / L.g2.bn * L.ks2);
  L.cap = moe::padded_capacity(n, E, L.g1.bm);
  L.max_tiles = L.cap / L.g1.bm;
  L.tail = L.ks2 == 1 && !(flags & (MOE_FLAG_NO_TAIL_SPLIT | MOE_FLAG_FP8_WEIGHTS)) &&
           moe::pick_tail_split(L.g2, T, K, E, H, I, L.max_tiles);
  L.nblk = moe::route_blocks(n);
  L.counts = take((size_t)E * 4, "counts");
  L.offsets = take((size_t)(E + 1) * 4, "offsets");
  L.num_tiles = take(4, "num_tiles");
  L.tile_expert = take((size_t)L.max_tiles * 4, "tile_expert");
  L.sorted = take((size_t)L.cap * 4, "sorted");
  L.slot_of = take((size_t)n * 4, "slot_of");
  L.block_hist = take((size_t)E * L.nblk * 4, "block histograms");
  L.act = take((size_t)L.cap * I * 2, "act");
  if (!(flags & MOE_FLAG_ATOMIC_COMBINE))
    L.y = take((size_t)L.ks2 * n * H * (L.y16 ? 2 : 4), "slot rows");
  if ((flags & MOE_FLAG_FP8_WEIGHTS) && fp8_may_widen(T, H, I, E, K)) {
    L.widened = true;
    L.w1dq = take((size_t)E * 2 * I * H * 2, "widened w1");
    L.w2dq = take((size_t)E * H * I * 2, "widened w2");
  }
  L.total = p;
  return L;
}

// ---- internal per-device workspace ----
constexpr int kMaxDevices = 64;
std::mutex g_ws_mutex;
void* g_ws_ptr[kMaxDevices] = {};
size_t g_ws_bytes[kMaxDevices] = {};

int internal_workspace(size_t need, void** out) {
  int dev = 0;
  hipError_t st = hipGetDevice(&dev);
  if (st != hipSuccess) return hip_error("hipGetDevice", st);
  if (dev < 0 || dev >= kMaxDevices) return set_error(MOE_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  if (g_ws_bytes[dev] < need) {
    if (g_ws_ptr[dev]) {
      // earlier work may still use the old buffer
      st = hipDeviceSynchronize();
      if (st != hipSuccess) return hip_error("hipDeviceSynchronize", st);
      (void)hipFree(g_ws_ptr[dev]);
      g_ws_ptr[dev] = nullptr;
      g_ws_bytes[dev] = 0;
    }
    void* p = nullptr;
    st = hipMalloc(&p, need);
    if (st != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return set_error(MOE_ERR_ALLOC, "hipMalloc(%zu) of the internal workspace failed: %s", need,
                       hipGetErrorString(st));
    }
    g_ws_ptr[dev] = p;
    g_ws_bytes[dev] = need;
  }
  *out = g_ws_ptr[dev];
  return MOE_OK;
}

// Flags of plain moe_forward, read once from the environment: MOE_COMBINE
// ("slot", the default, or "atomic") and MOE_DEBUG_SYNC (non-empty and not
// "0": synchronise after every stage and name the failing one, as the
// metrale forward_k2 dispatch does under its stage-diagnostics lever).
uint32_t env_flags() {
  static uint32_t flags = [] {
    uint32_t f = 0;
    const char* c = std::getenv("MOE_COMBINE");
    if (c && std::strcmp(c, "atomic") == 0) f |= MOE_FLAG_ATOMIC_COMBINE;
    const char* d = std::getenv("MOE_DEBUG_SYNC");
    if (d && d[0] != '\0' && std::strcmp(d, "0") != 0) f |= MOE_FLAG_DEBUG_SYNC;
    return f;
  }();
  return flags;
}

// Largest internal workspace the library may allocate, read once from the
// environment (MOE_WORKSPACE_LIMIT, bytes; unset or 0: no limit).
size_t workspace_limit() {
  static size_t limit = [] {
    const char* v = std::getenv("MOE_WORKSPACE_LIMIT");
    return v ? (size_t)std::strtoull(v, nullptr, 10) : (size_t)0;
  }();
  return limit;
}

// MOE_FLAG_DEBUG_SYNC: the guard bands of the layout (see Layout), set
// before the first stage and compared after each.
struct Guards {
  const Layout* L = nullptr;
  void* ws = nullptr;
};

int fill_guards(const Layout& L, void* ws, hipStream_t stream) {
  for (int i = 0; i < L.n_guards; ++i) {
    hipError_t st = hipMemsetAsync(static_cast<char*>(ws) + L.guard[i], kGuardByte, kGuardBytes,
                                   stream);
    if (st != hipSuccess) return hip_error("workspace guard fill", st);
  }
  return MOE_OK;
}

int check_guards(const Guards& g, const char* stage) {
  if (!g.L) return MOE_OK;
  unsigned char buf[kGuardBytes];
  for (int i = 0; i < g.L->n_guards; ++i) {
    hipError_t st = hipMemcpy(buf, static_cast<char*>(g.ws) + g.L->guard[i], kGuardBytes,
                              hipMemcpyDeviceToHost);
    if (st != hipSuccess) return hip_error("workspace guard check", st);
    for (size_t b = 0; b < kGuardBytes; ++b)
      if (buf[b] != kGuardByte)
        return set_error(MOE_ERR_WORKSPACE,
                         "stage %s wrote past the workspace region '%s' (guard byte %zu is 0x%02x)",
                         stage, g.L->guard_after[i], b, buf[b]);
  }
  return MOE_OK;
}

int stage_check(uint32_t flags, const char* stage, hipError_t launch, hipStream_t stream,
                const Guards& guards = Guards{}) {
  if (launch != hipSuccess) return hip_error(stage, launch);
  if (flags & MOE_FLAG_DEBUG_SYNC) {
    hipError_t st = hipStreamSynchronize(stream);
    if (st == hipSuccess) st = hipGetLastError();
    if (st != hipSuccess) return set_error(MOE_ERR_HIP, "stage %s failed: %s", stage, hipGetErrorString(st));
    return check_guards(guards, stage);
  }
  return MOE_OK;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

}  // namespace

namespace moe {
int set_last_error(int code, const char* msg) { return set_error(code, "%s", msg); }
}  // namespace moe

extern "C" {

const char* moe_last_error(void) { return g_last_error.c_str(); }

size_t moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, uint32_t flags) {
  if (check_sizes(T, H, I, E, K) != MOE_OK) return 0;
  if (T == 0) return 0;
  return make_layout(T, H, I, E, K, flags).total;
}

int32_t moe_m_tile(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, uint32_t flags) {
  (void)flags;
  const int rc = check_sizes(T, H, I, E, K);
  if (rc != MOE_OK) return rc;
  return moe::pick_gemm1_cfg(T, K, H, I, E).bm;
}

int moe_uses_decode_path(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, uint32_t flags) {
  const int rc = check_sizes(T, H, I, E, K);
  if (rc != MOE_OK) return rc;
  return use_decode(T, H, I, E, K, flags) ? 1 : 0;
}

int moe_path(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, uint32_t flags) {
  const int rc = check_sizes(T, H, I, E, K);
  if (rc != MOE_OK) return rc;
  return pick_path(T, H, I, E, K, flags);
}

int moe_y_bf16(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, uint32_t flags) {
  const int rc = check_sizes(T, H, I, E, K);
  if (rc != MOE_OK) return rc;
  if (T == 0) return 0;
  return make_layout(T, H, I, E, K, flags).y16 ? 1 : 0;
}

int moe_down_tail_split(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, uint32_t flags) {
  const int rc = check_sizes(T, H, I, E, K);
  if (rc != MOE_OK) return rc;
  if (T == 0) return 0;
  const Layout L = make_layout(T, H, I, E, K, flags);
  return L.path == MOE_PATH_GROUPED && L.tail ? 1 : 0;
}

}  // extern "C"

namespace {

// The whole forward; `q` non-null means FP8 weights (w1/w2 unused).
int forward_impl(const void* hidden, const void* w1, const void* w2, const moe::Fp8Weights* q,
                 const float* topk_weights, const int32_t* topk_ids, int64_t T, int64_t H,
                 int64_t I, int64_t E, int64_t K, int32_t activation, float alpha, float limit,
                 const float* b1, const float* b2, float* out, uint32_t flags, void* workspace,
                 size_t workspace_bytes, void* stream_ptr) {
  int rc = check_sizes(T, H, I, E, K);
  if (rc != MOE_OK) return rc;
  if (q) {
    flags |= MOE_FLAG_FP8_WEIGHTS;
    if (!moe::fp8_block_ok(H, I, q->block))
      return set_error(MOE_ERR_UNSUPPORTED,
                       "scale block %lld must be a multiple of 128 dividing H=%lld and I=%lld",
                       (long long)q->block, (long long)H, (long long)I);
  } else {
    flags &= ~MOE_FLAG_FP8_WEIGHTS;
  }
  if (activation < MOE_ACT_SILU || activation > MOE_ACT_GELU_ERF)
    return set_error(MOE_ERR_INVALID_ARG, "unknown activation %d", activation);
  if (activation == MOE_ACT_SWIGLUOAI && !(limit >= 0.0f && alpha == alpha))
    return set_error(MOE_ERR_INVALID_ARG, "swigluoai needs limit >= 0 and a numeric alpha");
  moe::Epilogue ep;
  ep.act = activation;
  ep.alpha = alpha;
  ep.limit = limit;
  ep.b1 = b1;
  ep.b2 = b2;
  if (T == 0) return MOE_OK;
  if (!hidden || !topk_weights || !topk_ids || !out ||
      (q ? (!q->w1q || !q->w1s || !q->w2q || !q->w2s) : (!w1 || !w2)))
    return set_error(MOE_ERR_INVALID_ARG, "null device pointer with T=%lld", (long long)T);
  const Layout L = make_layout(T, H, I, E, K, flags);
  void* ws = workspace;
  if (ws) {
    if (workspace_bytes < L.total)
      return set_error(MOE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes,
                       L.total);
    if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0)
      return set_error(MOE_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  } else {
    const size_t limit = workspace_limit();
    if (limit && L.total > limit)
      return set_error(MOE_ERR_ALLOC,
                       "the internal workspace would need %zu bytes, above MOE_WORKSPACE_LIMIT=%zu",
                       L.total, limit);
    rc = internal_workspace(L.total, &ws);
    if (rc != MOE_OK) return rc;
  }
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  Guards gd;
  if (L.n_guards) {
    if ((rc = fill_guards(L, ws, stream)) != MOE_OK) return rc;
    gd.L = &L;
    gd.ws = ws;
  }
  const auto* x = static_cast<const uint16_t*>(hidden);
  const auto* wa = static_cast<const uint16_t*>(w1);
  const auto* wb = static_cast<const uint16_t*>(w2);
  int32_t* err = at<int32_t>(ws, L.err);
  const bool validate = (flags & MOE_FLAG_VALIDATE_IDS) != 0;
  if (validate) {
    hipError_t st = hipMemsetAsync(err, 0, sizeof(int32_t), stream);
    if (st == hipSuccess) st = moe::launch_validate_ids(topk_ids, T, K, E, err, stream);
    if ((rc = stage_check(flags, "validate_ids", st, stream, gd)) != MOE_OK) return rc;
  }

  if (L.decode) {
    hipError_t st =
        q ? moe::launch_decode_fp8(x, *q, topk_weights, topk_ids, T, H, I, E, K,
                                   at<uint16_t>(ws, L.act), out, ep, stream)
          : moe::launch_decode(x, wa, wb, topk_weights, topk_ids, T, H, I, E, K,
                               at<uint16_t>(ws, L.act), out, ep, stream);
    if ((rc = stage_check(flags, "decode", st, stream, gd)) != MOE_OK) return rc;
  } else if (L.path == MOE_PATH_SMALL_BATCH) {
    float* y = at<float>(ws, L.y);
    hipError_t st =
        q ? moe::launch_small_batch_fp8(x, *q, topk_ids, T, H, I, E, K, at<uint16_t>(ws, L.act),
                                        y, ep, stream)
          : moe::launch_small_batch(x, wa, wb, topk_ids, T, H, I, E, K, at<uint16_t>(ws, L.act),
                                    y, ep, stream);
    if ((rc = stage_check(flags, "small_batch", st, stream, gd)) != MOE_OK) return rc;
    st = moe::launch_combine(y, topk_weights, nullptr, topk_ids, E, T, H, K, ep.b2, out, stream);
    if ((rc = stage_check(flags, "combine", st, stream, gd)) != MOE_OK) return rc;
  } else {
    int32_t* counts = at<int32_t>(ws, L.counts);
    int32_t* offsets = at<int32_t>(ws, L.offsets);
    int32_t* num_tiles = at<int32_t>(ws, L.num_tiles);
    int32_t* tile_expert = at<int32_t>(ws, L.tile_expert);
    int32_t* sorted = at<int32_t>(ws, L.sorted);
    int32_t* slot_of = at<int32_t>(ws, L.slot_of);
    int32_t* block_hist = at<int32_t>(ws, L.block_hist);
    uint16_t* act = at<uint16_t>(ws, L.act);
    hipError_t st = hipSuccess;
    const bool q_native = q && fp8_grouped_in_gemm(T, H, I, E, K, q->block);
    if (q && !q_native) {  // widen the FP8 weights to bf16 in the workspace
      if (!L.widened)  // cannot happen: the layout plans for every block the check allows
        return set_error(MOE_ERR_UNSUPPORTED, "no room for the widened FP8 weights");
      st = moe::launch_dequant_fp8(*q, E, H, I, at<uint16_t>(ws, L.w1dq),
                                   at<uint16_t>(ws, L.w2dq), stream);
      if ((rc = stage_check(flags, "dequant_fp8", st, stream, gd)) != MOE_OK) return rc;
      wa = at<uint16_t>(ws, L.w1dq);
      wb = at<uint16_t>(ws, L.w2dq);
    }
    st = moe::launch_route(topk_ids, T, K, E, L.g1.bm, block_hist, counts, offsets,
                                      sorted, slot_of, tile_expert, num_tiles, stream);
    if ((rc = stage_check(flags, "route", st, stream, gd)) != MOE_OK) return rc;
    st = q_native ? moe::launch_gemm1_silu_fp8(L.g1, x, q->w1q, q->w1s, q->block, sorted,
                                               tile_expert, num_tiles, T, H, I, E, K,
                                               L.max_tiles, act, ep, stream)
                  : moe::launch_gemm1_silu(L.g1, x, wa, sorted, tile_expert, num_tiles, T, H, I,
                                           E, K, L.max_tiles, act, ep, stream);
    if ((rc = stage_check(flags, "gemm1_silu", st, stream, gd)) != MOE_OK) return rc;
    if (flags & MOE_FLAG_ATOMIC_COMBINE) {
      st = moe::launch_zero(out, T * H, stream);
      if ((rc = stage_check(flags, "zero_out", st, stream, gd)) != MOE_OK) return rc;
      st = q_native ? moe::launch_gemm2_fp8(L.g2, act, q->w2q, q->w2s, q->block, sorted,
                                            tile_expert, num_tiles, topk_weights, H, I, E,
                                            K, L.max_tiles, nullptr, out, ep.b2, stream)
                    : moe::launch_gemm2(L.g2, act, wb, sorted, tile_expert, num_tiles,
                                        topk_weights, H, I, E, K, L.max_tiles, nullptr, out,
                                        ep.b2, stream, 1, 0, nullptr, L.tail);
      if ((rc = stage_check(flags, "gemm2_atomic", st, stream, gd)) != MOE_OK) return rc;
    } else {
      float* y = L.y16 ? nullptr : at<float>(ws, L.y);
      uint16_t* y16 = L.y16 ? at<uint16_t>(ws, L.y) : nullptr;
      st = q_native ? moe::launch_gemm2_fp8(L.g2, act, q->w2q, q->w2s, q->block, sorted,
                                            tile_expert, num_tiles, topk_weights, H, I, E,
                                            K, L.max_tiles, y, nullptr, nullptr, stream, L.ks2,
                                            T * K, y16)
                    : moe::launch_gemm2(L.g2, act, wb, sorted, tile_expert, num_tiles,
                                        topk_weights, H, I, E, K, L.max_tiles, y, nullptr,
                                        nullptr, stream, L.ks2, T * K, y16, L.tail);
      if ((rc = stage_check(flags, "gemm2_slot", st, stream, gd)) != MOE_OK) return rc;
      st = L.y16 ? moe::launch_combine_bf16(y16, topk_weights, slot_of, topk_ids, E, T, H, K,
                                            ep.b2, out, stream)
                 : moe::launch_combine(y, topk_weights, slot_of, topk_ids, E, T, H, K, ep.b2,
                                       out, stream, L.ks2);
      if ((rc = stage_check(flags, "combine", st, stream, gd)) != MOE_OK) return rc;
    }
  }

  if (validate) {
    int32_t host_err = 0;
    hipError_t st = hipMemcpyAsync(&host_err, err, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (st == hipSuccess) st = hipStreamSynchronize(stream);
    if (st != hipSuccess) return hip_error("validate_ids readback", st);
    if (host_err)
      return set_error(MOE_ERR_INVALID_ARG,
                       "topk_ids has an id outside [0, %lld) or a repeated id within a token",
                       (long long)E);
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_act(const void* hidden, const void* w1, const void* w2,
                    const float* topk_weights, const int32_t* topk_ids, int64_t T, int64_t H,
                    int64_t I, int64_t E, int64_t K, int32_t activation, float alpha,
                    float limit, const float* b1, const float* b2, float* out, uint32_t flags,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(hidden, w1, w2, nullptr, topk_weights, topk_ids, T, H, I, E, K,
                      activation, alpha, limit, b1, b2, out, flags, workspace, workspace_bytes,
                      stream);
}

int moe_forward_fp8(const void* hidden, const uint8_t* w1q, const float* w1_scale,
                    const uint8_t* w2q, const float* w2_scale, int64_t block,
                    const float* topk_weights, const int32_t* topk_ids, int64_t T, int64_t H,
                    int64_t I, int64_t E, int64_t K, int32_t activation, float alpha,
                    float limit, const float* b1, const float* b2, float* out, uint32_t flags,
                    void* workspace, size_t workspace_bytes, void* stream) {
  moe::Fp8Weights q;
  q.w1q = w1q;
  q.w1s = w1_scale;
  q.w2q = w2q;
  q.w2s = w2_scale;
  q.block = block;
  return forward_impl(hidden, nullptr, nullptr, &q, topk_weights, topk_ids, T, H, I, E, K,
                      activation, alpha, limit, b1, b2, out, flags, workspace, workspace_bytes,
                      stream);
}

int moe_forward_ex(const void* hidden, const void* w1, const void* w2, const float* topk_weights,
                   const int32_t* topk_ids, int64_t T, int64_t H, int64_t I, int64_t E, int64_t K,
                   float* out, uint32_t flags, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return moe_forward_act(hidden, w1, w2, topk_weights, topk_ids, T, H, I, E, K, MOE_ACT_SILU,
                         1.702f, 7.0f, nullptr, nullptr, out, flags, workspace, workspace_bytes,
                         stream);
}

int moe_forward(const void* hidden, const void* w1, const void* w2, const float* topk_weights,
                const int32_t* topk_ids, int64_t T, int64_t H, int64_t I, int64_t E, int64_t K,
                float* out, void* stream) {
  return moe_forward_ex(hidden, w1, w2, topk_weights, topk_ids, T, H, I, E, K, out, env_flags(),
                        nullptr, 0, stream);
}

size_t moe_route_scratch_bytes(int64_t T, int64_t K, int64_t E) {
  if (T < 0 || K <= 0 || E <= 0) return 0;
  return (size_t)E * moe::route_blocks(T * K) * sizeof(int32_t);
}

int moe_route(const int32_t* topk_ids, int64_t T, int64_t K, int64_t E, int32_t m_tile,
              int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* slot_of,
              int32_t* tile_expert, int32_t* num_tiles, int64_t capacity, void* scratch,
              void* stream_ptr) {
  if (T < 0 || K <= 0 || E <= 0 || K > E)
    return set_error(MOE_ERR_INVALID_ARG, "bad sizes T=%lld K=%lld E=%lld", (long long)T,
                     (long long)K, (long long)E);
  if (E > moe::kMaxExperts)
    return set_error(MOE_ERR_UNSUPPORTED, "num_experts=%lld exceeds %d", (long long)E,
                     moe::kMaxExperts);
  if (m_tile < 16 || m_tile > 256 || m_tile % 16 != 0)
    return set_error(MOE_ERR_INVALID_ARG, "m_tile=%d must be a multiple of 16 in [16, 256]", m_tile);
  if (T * K > (int64_t)1 << 30)
    return set_error(MOE_ERR_UNSUPPORTED, "T*K=%lld is too large", (long long)(T * K));
  const int64_t n = T * K;
  const int64_t live = n < E ? n : E;
  if (capacity < n + live * (m_tile - 1))
    return set_error(MOE_ERR_INVALID_ARG, "capacity %lld < %lld", (long long)capacity,
                     (long long)(n + live * (m_tile - 1)));
  if (!counts || !offsets || !num_tiles || (n > 0 && (!topk_ids || !sorted || !slot_of ||
                                                      !tile_expert || !scratch)))
    return set_error(MOE_ERR_INVALID_ARG, "null device pointer");
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  if (n == 0) {
    hipError_t st = hipMemsetAsync(counts, 0, (size_t)E * 4, stream);
    if (st == hipSuccess) st = hipMemsetAsync(offsets, 0, (size_t)(E + 1) * 4, stream);
    if (st == hipSuccess) st = hipMemsetAsync(num_tiles, 0, 4, stream);
    return st == hipSuccess ? MOE_OK : hip_error("moe_route (empty)", st);
  }
  hipError_t st = moe::launch_route(topk_ids, T, K, E, m_tile, static_cast<int32_t*>(scratch),
                                    counts, offsets, sorted, slot_of, tile_expert, num_tiles,
                                    stream);
  return st == hipSuccess ? MOE_OK : hip_error("moe_route", st);
}

int moe_gemm1_silu(const void* hidden, const void* w1, const int32_t* sorted,
                   const int32_t* tile_expert, const int32_t* num_tiles, int64_t T, int64_t H,
                   int64_t I, int64_t E, int64_t K, int32_t m_tile, int64_t max_tiles, void* act,
                   void* stream) {
  int rc = check_sizes(T, H, I, E, K);
  if (rc != MOE_OK) return rc;
  if (m_tile != 64 && m_tile != 128 && m_tile != 192 && m_tile != 256)
    return set_error(MOE_ERR_UNSUPPORTED, "m_tile=%d: the GEMM supports 64, 128, 192 and 256",
                     m_tile);
  if (max_tiles < 0 || max_tiles > INT32_MAX)
    return set_error(MOE_ERR_INVALID_ARG, "max_tiles=%lld", (long long)max_tiles);
  if (T == 0 || max_tiles == 0) return MOE_OK;
  if (!hidden || !w1 || !sorted || !tile_expert || !num_tiles || !act)
    return set_error(MOE_ERR_INVALID_ARG, "null device pointer");
  hipError_t st = moe::launch_gemm1_silu(
      gemm1_entry_cfg(T, H, I, E, K, m_tile), static_cast<const uint16_t*>(hidden),
      static_cast<const uint16_t*>(w1), sorted, tile_expert, num_tiles, T, H, I, E, K, max_tiles,
      static_cast<uint16_t*>(act), moe::Epilogue{}, static_cast<hipStream_t>(stream));
  return st == hipSuccess ? MOE_OK : hip_error("moe_gemm1_silu", st);
}

int moe_gemm1_silu_fp8(const void* hidden, const uint8_t* w1q, const float* w1_scale,
                       int64_t block, const int32_t* sorted, const int32_t* tile_expert,
                       const int32_t* num_tiles, int64_t T, int64_t H, int64_t I, int64_t E,
                       int64_t K, int32_t m_tile, int64_t max_tiles, void* act, void* stream) {
  int rc = check_sizes(T, H, I, E, K);
  if (rc != MOE_OK) return rc;
  if (m_tile != 64 && m_tile != 128 && m_tile != 192 && m_tile != 256)
    return set_error(MOE_ERR_UNSUPPORTED, "m_tile=%d: the GEMM supports 64, 128, 192 and 256",
                     m_tile);
  if (!moe::fp8_block_ok(H, I, block) || !moe::fp8_gemm_supported(H, I, block))
    return set_error(MOE_ERR_UNSUPPORTED,
                     "scale block %lld: needs a multiple of 128 dividing H=%lld and I=%lld, "
                     "with at most %d blocks per row",
                     (long long)block, (long long)H, (long long)I, moe::kMaxScaleBlocks);
  if (max_tiles < 0 || max_tiles > INT32_MAX)
    return set_error(MOE_ERR_INVALID_ARG, "max_tiles=%lld", (long long)max_tiles);
  if (T == 0 || max_tiles == 0) return MOE_OK;
  if (!hidden || !w1q || !w1_scale || !sorted || !tile_expert || !num_tiles || !act)
    return set_error(MOE_ERR_INVALID_ARG, "null device pointer");
  hipError_t st = moe::launch_gemm1_silu_fp8(
      gemm1_entry_cfg(T, H, I, E, K, m_tile), static_cast<const uint16_t*>(hidden), w1q,
      w1_scale, block, sorted, tile_expert, num_tiles, T, H, I, E, K, max_tiles,
      static_cast<uint16_t*>(act), moe::Epilogue{}, static_cast<hipStream_t>(stream));
  return st == hipSuccess ? MOE_OK : hip_error("moe_gemm1_silu_fp8", st);
}

int moe_fp8_widens_in_gemm(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K,
                           int64_t block) {
  const int rc = check_sizes(T, H, I, E, K);
  if (rc != MOE_OK) return rc;
  if (!moe::fp8_block_ok(H, I, block))
    return set_error(MOE_ERR_UNSUPPORTED, "scale block %lld", (long long)block);
  return fp8_grouped_in_gemm(T, H, I, E, K, block) ? 1 : 0;
}

int moe_topk_softmax(const float* router_logits, int64_t T, int64_t E, int64_t K,
                     int renormalize, float* topk_weights, int32_t* topk_ids, void* stream) {
  if (T < 0 || E <= 0 || K <= 0 || K > E)
    return set_error(MOE_ERR_INVALID_ARG, "bad sizes T=%lld E=%lld K=%lld", (long long)T,
                     (long long)E, (long long)K);
  if (E > moe::kMaxExperts || K > 32)
    return set_error(MOE_ERR_UNSUPPORTED, "E=%lld (max %d) K=%lld (max 32)", (long long)E,
                     moe::kMaxExperts, (long long)K);
  if (T == 0) return MOE_OK;
  if (!router_logits || !topk_weights || !topk_ids)
    return set_error(MOE_ERR_INVALID_ARG, "null device pointer");
  hipError_t st = moe::launch_topk_softmax(router_logits, T, E, K, renormalize != 0, topk_weights,
                                           topk_ids, static_cast<hipStream_t>(stream));
  return st == hipSuccess ? MOE_OK : hip_error("moe_topk_softmax", st);
}

void moe_release(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (int d = 0; d < kMaxDevices; ++d) {
    if (!g_ws_ptr[d]) continue;
    if (hipSetDevice(d) == hipSuccess) {
      (void)hipDeviceSynchronize();
      (void)hipFree(g_ws_ptr[d]);
    }
    g_ws_ptr[d] = nullptr;
    g_ws_bytes[d] = 0;
  }
  (void)hipSetDevice(cur);
}

}  // extern "C"
