// C ABI of the causal Based forward: argument validation, execution plan, workspace, launches, timing.
// The operation and the argument contract follow the page "Write a fast Based (Taylor linear attention)
// forward kernel", fields spec_md and contract_md (see include/based.h for the full contract).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "based.h"
#include "based_internal.h"

using based::Plan;
using based::Shape;

namespace {

thread_local std::string g_detail;

based_status_t fail(based_status_t s, const std::string& msg) {
  g_detail = msg;
  return s;
}

based_status_t ok() {
  g_detail.clear();
  return BASED_OK;
}

constexpr int64_t kMaxElems = int64_t(1) << 46;  // keeps every byte offset far from int64 overflow
constexpr int64_t kCUs = 256;                    // MI355X compute units
constexpr int64_t kTargetWaves = 2048;           // 256 CUs x 4 SIMDs x 2 resident waves
// Segments shorter than this are used only up to kMaxShortSegments of them: with more, the start-up reads
// of the earlier segments' sums (or a scan kernel) cost more than the shorter chains gain.
constexpr int64_t kShortSegment = 256;
constexpr int64_t kMaxShortSegments = 8;
// Shortest piece of a segment the state pass sums on its own (see make_plan).
constexpr int64_t kMinPiece = 1024;
constexpr int64_t kMaxRowRange = 0x7fffffff;     // bytes addressable through one 32-bit buffer range

based_status_t check_shape(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V) {
  if (B < 1 || T < 1 || H < 1)
    return fail(BASED_ERR_INVALID_ARGUMENT, "B, T and H must be >= 1");
  if (K != 8 && K != 16) return fail(BASED_ERR_UNSUPPORTED, "K must be 8 or 16");
  if (V < 64 || V > 512 || V % 64 != 0) return fail(BASED_ERR_UNSUPPORTED, "V must be a multiple of 64 in [64, 512]");
  if (B > kMaxElems / T || B * T > kMaxElems / H || B * T * H > kMaxElems / V)
    return fail(BASED_ERR_INVALID_ARGUMENT, "tensor too large");
  // The kernels address the rows of one (b, h) through 32-bit buffer ranges of T * H * V * 4 bytes.
  if (T * H * V * 4 > kMaxRowRange)
    return fail(BASED_ERR_UNSUPPORTED, "T * H * V * 4 must not exceed 2^31 - 1 bytes");
  return BASED_OK;
}

// Segment length for items of `item_cols` columns (see make_plan).
int64_t segment_length(const Shape& sh, int64_t item_cols, int64_t seg_override) {
  const int64_t ck = based::chunk_tokens(sh.K, item_cols);
  const int64_t t_round = (sh.T + ck - 1) / ck * ck;
  int64_t L;
  if (seg_override > 0) {
    L = (seg_override + ck - 1) / ck * ck;
  } else {
    const int64_t pairs = sh.B * sh.H * (sh.V / item_cols);
    const int64_t waves = pairs * based::waves_per_item(sh.K, item_cols);
    if (pairs >= kCUs && waves >= kTargetWaves / 2) {
      // The (b, h, columns) items alone give every CU a workgroup and every SIMD a wave: one segment, no
      // state pass (a second wave per SIMD gains less than the state pass over half the keys costs).
      L = t_round;
    } else {
      // Two waves per SIMD, except K = 8 with 128 columns, whose read-out is closest to memory-bound: one.
      const int64_t target = (sh.K == 8 && item_cols == 128) ? kTargetWaves / 2 : kTargetWaves;
      const int64_t g_target = (target + waves - 1) / waves;
      L = (sh.T + g_target - 1) / g_target;
      L = (L + ck - 1) / ck * ck;
    }
    // At least one chunk per segment for K = 8 and two for K = 16, whose segment sums are 3.3 times
    // larger, so that each further segment costs more start-up reads (measured on short sequences).
    const int64_t l_min = (sh.K == 16 ? 2 : 1) * ck;
    if (L < l_min) L = l_min;
    // Segments shorter than kShortSegment tokens only up to kMaxShortSegments of them: beyond that, the
    // shortest length that gives that many (at most kShortSegment).
    if (L < kShortSegment && (sh.T + L - 1) / L > kMaxShortSegments) {
      const int64_t l8 = (sh.T + kMaxShortSegments - 1) / kMaxShortSegments;
      L = (l8 + ck - 1) / ck * ck;
      const int64_t l_short = (kShortSegment + ck - 1) / ck * ck;
      if (L > l_short) L = l_short;
    }
  }
  return L > t_round ? t_round : L;
}

Plan make_plan(const Shape& sh, int64_t seg_override) {
  Plan pl;
  pl.item_cols = based::item_columns(sh.V);
  if (pl.item_cols == 128 && sh.K == 16 && seg_override == 0) {
    // 64-column items instead when 128-column ones leave CUs idle and 64-column ones do not, or when only
    // 64-column items avoid the state pass: the halves recompute phi and the scores, which costs less
    // (measured 3-7% faster where the state pass goes, 24-28% on short sequences; 18% slower where both
    // widths fill the CUs with the same segments).
    const int64_t p128 = sh.B * sh.H * (sh.V / 128), p64 = 2 * p128;
    const int64_t g128 = (sh.T + segment_length(sh, 128, 0) - 1) / segment_length(sh, 128, 0);
    const int64_t g64 = (sh.T + segment_length(sh, 64, 0) - 1) / segment_length(sh, 64, 0);
    if ((p128 * g128 < kCUs && p64 * g64 >= kCUs) || (g128 > 1 && g64 == 1)) pl.item_cols = 64;
  }
  pl.nvs = sh.V / pl.item_cols;
  const int64_t L = segment_length(sh, pl.item_cols, seg_override);
  pl.seg_len = L;
  pl.segments = (sh.T + L - 1) / L;
  pl.slot_floats = based::state_slot_floats(sh.K, pl.item_cols);
  // The state pass sums each segment but the last in sub pieces. Two pieces when one per segment would give
  // it at most one workgroup per CU and the halves stay long (kMinPiece tokens, whole 64-token chunks): a
  // state workgroup runs its chunks about as fast with a second one on its CU as alone, so the pass takes
  // about half the time, while each read-out adds up twice as many sums.
  pl.sub = 1;
  if (pl.segments > 1) {
    const int64_t state_items = sh.B * sh.H * pl.nvs * (pl.item_cols / 64) * (pl.segments - 1);
    if (state_items <= kCUs && pl.seg_len % 128 == 0 && pl.seg_len / 2 >= kMinPiece) pl.sub = 2;
  }
  pl.scanned = based::state_slots(pl) > based::kMaxSummedSlots;
  // XCD-affine items when the (b, columns, h) pairs split evenly over the 8 XCDs and each XCD's run of
  // heads covers whole 128-byte lines of the q and k rows (64 / K heads per line).
  const int64_t pairs = sh.B * sh.H * pl.nvs, ppx = pairs / 8, line_heads = 64 / sh.K;
  pl.affine = pairs % 8 == 0 && (ppx % sh.H == 0 || (sh.H % line_heads == 0 && ppx % line_heads == 0));
  // Output rows written whole (through LDS) rather than as 16-row tiles: measured 21% faster read-out at
  // K = 8 with 128 columns and 2-7% at K = 16 with 64 columns when segments share the CUs, 6% slower with
  // a single segment (one workgroup per CU, where the extra LDS round trip is not hidden). The K = 16,
  // 128-column read-out has no registers to spare for it and never does it.
  pl.row_stores = sh.K == 8 || (pl.item_cols == 64 && pl.segments > 1);
  return pl;
}

// The kernels number their work items in 32 bits: (b, h, columns, segment) for the read-out, up to two
// 64-column halves per state sum for the state pass.
based_status_t check_items(const Shape& sh, const Plan& pl) {
  const int64_t pairs = sh.B * sh.H * pl.nvs;
  const int64_t per_pair = 2 * std::max(pl.segments, based::state_slots(pl));
  if (pairs > based::kMaxItems / per_pair)
    return fail(BASED_ERR_UNSUPPORTED, "too many work items: B * H * (V / columns) * segments must stay below 2^30");
  return BASED_OK;
}

size_t workspace_bytes(const Shape& sh, const Plan& pl) {
  if (pl.segments <= 1) return 0;
  return static_cast<size_t>(sh.B * sh.H * pl.nvs * based::state_slots(pl) * pl.slot_floats) * sizeof(float);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

struct based_timer {
  std::vector<hipEvent_t> events;  // two per launch
  std::vector<int> kernel_ids;
  int capacity = 0;
  int used = 0;
  unsigned mask = ~0u;
};

namespace {

// Where the workspace comes from: the caller (ws, ws_bytes), stream-ordered allocation, or the library's
// static device scratch.
enum class Workspace { kCaller, kAllocate, kScratch };

based_status_t run(const void* q, const void* k, const void* v, const Shape& sh, float scale, void* out,
                   based_dtype_t out_dtype, void* ws, size_t ws_bytes, int64_t seg_override, based_timer* timer,
                   hipStream_t stream, Workspace wsk, const based::StateIO& io = based::StateIO{}) {
  const bool allocate = wsk == Workspace::kAllocate;
  if (based_status_t s = check_shape(sh.B, sh.T, sh.H, sh.K, sh.V)) return s;
  if (!q || !k || !v || !out) return fail(BASED_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (out_dtype != BASED_BF16 && out_dtype != BASED_F32)
    return fail(BASED_ERR_INVALID_ARGUMENT, "out_dtype must be BASED_BF16 or BASED_F32");
  if (std::isinf(scale)) return fail(BASED_ERR_INVALID_ARGUMENT, "scale must be finite (NaN selects K**-0.5)");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(BASED_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
  if (seg_override < 0) return fail(BASED_ERR_INVALID_ARGUMENT, "segment length override must be >= 0");
  if (timer && timer->used + 3 > timer->capacity)
    return fail(BASED_ERR_INVALID_ARGUMENT, "timer is full; reset it or create a larger one");

  const size_t qk_bytes = static_cast<size_t>(sh.B * sh.T * sh.H * sh.K) * 2;
  const size_t v_bytes = static_cast<size_t>(sh.B * sh.T * sh.H * sh.V) * 2;
  const size_t o_bytes = static_cast<size_t>(sh.B * sh.T * sh.H * sh.V) * (out_dtype == BASED_F32 ? 4 : 2);
  if (overlaps(out, o_bytes, q, qk_bytes) || overlaps(out, o_bytes, k, qk_bytes) ||
      overlaps(out, o_bytes, v, v_bytes))
    return fail(BASED_ERR_INVALID_ARGUMENT, "out overlaps an input");
  const int64_t P = 1 + sh.K + sh.K * sh.K;
  const size_t s_bytes = static_cast<size_t>(sh.B * sh.H * P * sh.V) * 4;
  const size_t z_bytes = static_cast<size_t>(sh.B * sh.H * P) * 4;
  if (!io.s_in != !io.z_in) return fail(BASED_ERR_INVALID_ARGUMENT, "state_in and norm_in must both be set or both NULL");
  if (!io.s_out != !io.z_out)
    return fail(BASED_ERR_INVALID_ARGUMENT, "state_out and norm_out must both be set or both NULL");
  if ((io.s_in && (!aligned16(io.s_in) || !aligned16(io.z_in))) ||
      (io.s_out && (!aligned16(io.s_out) || !aligned16(io.z_out))))
    return fail(BASED_ERR_INVALID_ARGUMENT, "state pointers must be 16-byte aligned");
  if (io.s_out) {
    const void* outs[2] = {io.s_out, io.z_out};
    const size_t outn[2] = {s_bytes, z_bytes};
    const void* others[6] = {q, k, v, out, io.s_in, io.z_in};
    const size_t othern[6] = {qk_bytes, qk_bytes, v_bytes, o_bytes, io.s_in ? s_bytes : 0, io.z_in ? z_bytes : 0};
    for (int i = 0; i < 2; ++i)
      for (int j = 0; j < 6; ++j)
        if (overlaps(outs[i], outn[i], others[j], othern[j]))
          return fail(BASED_ERR_INVALID_ARGUMENT, "state_out / norm_out overlap an input, out or the state input");
    if (overlaps(io.s_out, s_bytes, io.z_out, z_bytes))
      return fail(BASED_ERR_INVALID_ARGUMENT, "state_out and norm_out overlap");
  }
  if (io.s_in && (overlaps(out, o_bytes, io.s_in, s_bytes) || overlaps(out, o_bytes, io.z_in, z_bytes)))
    return fail(BASED_ERR_INVALID_ARGUMENT, "out overlaps the state input");

  const Plan pl = make_plan(sh, seg_override);
  if (based_status_t s = check_items(sh, pl)) return s;
  const size_t need = workspace_bytes(sh, pl);
  if (wsk == Workspace::kScratch) {
    if (need > based::kScratchBytes)
      return fail(BASED_ERR_UNSUPPORTED, "the plan needs " + std::to_string(need) +
                                             " bytes of workspace, more than the static scratch's " +
                                             std::to_string(based::kScratchBytes));
  } else if (!allocate) {
    if (need > 0 && !ws) return fail(BASED_ERR_WORKSPACE_TOO_SMALL, "workspace required but NULL");
    if (ws_bytes < need)
      return fail(BASED_ERR_WORKSPACE_TOO_SMALL,
                  "workspace has " + std::to_string(ws_bytes) + " bytes, needs " + std::to_string(need));
    if (need > 0 && !aligned16(ws)) return fail(BASED_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    if (overlaps(out, o_bytes, ws, need) || overlaps(ws, need, q, qk_bytes) || overlaps(ws, need, k, qk_bytes) ||
        overlaps(ws, need, v, v_bytes) || overlaps(ws, need, io.s_in, io.s_in ? s_bytes : 0) ||
        overlaps(ws, need, io.z_in, io.z_in ? z_bytes : 0) || overlaps(ws, need, io.s_out, io.s_out ? s_bytes : 0) ||
        overlaps(ws, need, io.z_out, io.z_out ? z_bytes : 0))
      return fail(BASED_ERR_INVALID_ARGUMENT, "workspace overlaps a tensor");
  }

  const float sigma = std::isnan(scale) ? static_cast<float>(1.0 / std::sqrt(static_cast<double>(sh.K))) : scale;
  const bool out_f32 = out_dtype == BASED_F32;

  float* wsf = static_cast<float*>(ws);
  if (wsk == Workspace::kScratch && need > 0) {
    void* p = nullptr;
    const hipError_t e = based::scratch_buffer(stream, &p);
    if (e != hipSuccess) return fail(BASED_ERR_HIP, std::string("static scratch: ") + hipGetErrorString(e));
    wsf = static_cast<float*>(p);
  }
  if (allocate && need > 0) {
    void* p = nullptr;
    const hipError_t e = hipMallocAsync(&p, need, stream);
    if (e != hipSuccess) return fail(BASED_ERR_OUT_OF_MEMORY, std::string("hipMallocAsync: ") + hipGetErrorString(e));
    wsf = static_cast<float*>(p);
  }

  auto launch = [&](int id) -> hipError_t {
    const bool rec = timer && ((timer->mask >> id) & 1u);
    if (rec) {
      hipError_t e = hipEventRecord(timer->events[2 * timer->used], stream);
      if (e != hipSuccess) return e;
    }
    hipError_t e = based::launch_kernel(id, q, k, v, sh, pl, sigma, wsf, out, out_f32, io, stream);
    if (e != hipSuccess) return e;
    if (rec) {
      e = hipEventRecord(timer->events[2 * timer->used + 1], stream);
      if (e != hipSuccess) return e;
      timer->kernel_ids[timer->used] = id;
      timer->used += 1;
    }
    return hipSuccess;
  };

  hipError_t e = hipSuccess;
  if (pl.segments > 1) e = launch(0);
  if (e == hipSuccess && pl.scanned) e = launch(1);
  if (e == hipSuccess) e = launch(2);
  if (allocate && need > 0) {
    const hipError_t f = hipFreeAsync(wsf, stream);
    if (e == hipSuccess) e = f;
  }
  if (e != hipSuccess) return fail(BASED_ERR_HIP, std::string("HIP: ") + hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int based_abi_version(void) { return BASED_ABI_VERSION; }

const char* based_status_string(based_status_t status) {
  switch (status) {
    case BASED_OK: return "ok";
    case BASED_ERR_INVALID_ARGUMENT: return "invalid argument";
    case BASED_ERR_UNSUPPORTED: return "unsupported shape";
    case BASED_ERR_HIP: return "HIP error";
    case BASED_ERR_OUT_OF_MEMORY: return "out of device memory";
    case BASED_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
  }
  return "unknown status";
}

const char* based_last_error_detail(void) { return g_detail.c_str(); }

size_t based_forward_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V) {
  if (check_shape(B, T, H, K, V) != BASED_OK) return 0;
  const Shape sh{B, T, H, K, V};
  return workspace_bytes(sh, make_plan(sh, 0));
}

based_status_t based_forward_plan(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                                  int64_t segment_len_override, int64_t* segments, int64_t* segment_len,
                                  size_t* ws_bytes) {
  if (based_status_t s = check_shape(B, T, H, K, V)) return s;
  if (segment_len_override < 0) return fail(BASED_ERR_INVALID_ARGUMENT, "segment length override must be >= 0");
  const Shape sh{B, T, H, K, V};
  const Plan pl = make_plan(sh, segment_len_override);
  if (based_status_t s = check_items(sh, pl)) return s;
  if (segments) *segments = pl.segments;
  if (segment_len) *segment_len = pl.seg_len;
  if (ws_bytes) *ws_bytes = workspace_bytes(sh, pl);
  return ok();
}

based_status_t based_forward(const void* q, const void* k, const void* v, int64_t B, int64_t T, int64_t H,
                             int64_t K, int64_t V, float scale, void* out, based_dtype_t out_dtype,
                             hipStream_t stream) {
  return run(q, k, v, Shape{B, T, H, K, V}, scale, out, out_dtype, nullptr, 0, 0, nullptr, stream,
             Workspace::kAllocate);
}

based_status_t based_forward_noalloc(const void* q, const void* k, const void* v, int64_t B, int64_t T, int64_t H,
                                     int64_t K, int64_t V, float scale, void* out, based_dtype_t out_dtype,
                                     hipStream_t stream) {
  return run(q, k, v, Shape{B, T, H, K, V}, scale, out, out_dtype, nullptr, 0, 0, nullptr, stream,
             Workspace::kScratch);
}

size_t based_noalloc_scratch_bytes(void) { return based::kScratchBytes; }

based_status_t based_forward_ws(const void* q, const void* k, const void* v, int64_t B, int64_t T, int64_t H,
                                int64_t K, int64_t V, float scale, void* out, based_dtype_t out_dtype,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run(q, k, v, Shape{B, T, H, K, V}, scale, out, out_dtype, workspace, workspace_bytes, 0, nullptr, stream,
             Workspace::kCaller);
}

based_status_t based_forward_ex(const void* q, const void* k, const void* v, int64_t B, int64_t T, int64_t H,
                                int64_t K, int64_t V, float scale, void* out, based_dtype_t out_dtype,
                                void* workspace, size_t workspace_bytes, int64_t segment_len_override,
                                based_timer* timer, hipStream_t stream) {
  return run(q, k, v, Shape{B, T, H, K, V}, scale, out, out_dtype, workspace, workspace_bytes, segment_len_override,
             timer, stream, Workspace::kCaller);
}

int64_t based_feature_dim(int64_t K) { return 1 + K + K * K; }

based_status_t based_forward_state(const void* q, const void* k, const void* v, int64_t B, int64_t T, int64_t H,
                                   int64_t K, int64_t V, float scale, void* out, based_dtype_t out_dtype,
                                   const float* state_in, const float* norm_in, float* state_out, float* norm_out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const based::StateIO io{state_in, norm_in, state_out, norm_out};
  return run(q, k, v, Shape{B, T, H, K, V}, scale, out, out_dtype, workspace, workspace_bytes, 0, nullptr, stream,
             workspace == nullptr ? Workspace::kAllocate : Workspace::kCaller, io);
}

based_status_t based_decode_step(const void* q, const void* k, const void* v, int64_t B, int64_t H, int64_t K,
                                 int64_t V, float scale, float* state, float* norm, void* out,
                                 based_dtype_t out_dtype, hipStream_t stream) {
  if (based_status_t s = check_shape(B, 1, H, K, V)) return s;
  if (B * H > based::kMaxItems) return fail(BASED_ERR_UNSUPPORTED, "B * H must stay below 2^31 for the decode step");
  if (!q || !k || !v || !out || !state || !norm) return fail(BASED_ERR_INVALID_ARGUMENT, "null pointer");
  if (out_dtype != BASED_BF16 && out_dtype != BASED_F32)
    return fail(BASED_ERR_INVALID_ARGUMENT, "out_dtype must be BASED_BF16 or BASED_F32");
  if (std::isinf(scale)) return fail(BASED_ERR_INVALID_ARGUMENT, "scale must be finite (NaN selects K**-0.5)");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(state) || !aligned16(norm))
    return fail(BASED_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
  const int64_t P = 1 + K + K * K;
  const size_t s_bytes = static_cast<size_t>(B * H * P * V) * 4, z_bytes = static_cast<size_t>(B * H * P) * 4;
  const size_t qk_bytes = static_cast<size_t>(B * H * K) * 2, v_bytes = static_cast<size_t>(B * H * V) * 2;
  const size_t o_bytes = static_cast<size_t>(B * H * V) * (out_dtype == BASED_F32 ? 4 : 2);
  const void* ptrs[4] = {q, k, v, out};
  const size_t sizes[4] = {qk_bytes, qk_bytes, v_bytes, o_bytes};
  for (int j = 0; j < 4; ++j)
    if (overlaps(state, s_bytes, ptrs[j], sizes[j]) || overlaps(norm, z_bytes, ptrs[j], sizes[j]))
      return fail(BASED_ERR_INVALID_ARGUMENT, "state / norm overlap an input or out");
  if (overlaps(state, s_bytes, norm, z_bytes)) return fail(BASED_ERR_INVALID_ARGUMENT, "state and norm overlap");
  if (overlaps(out, o_bytes, q, qk_bytes) || overlaps(out, o_bytes, k, qk_bytes) || overlaps(out, o_bytes, v, v_bytes))
    return fail(BASED_ERR_INVALID_ARGUMENT, "out overlaps an input");
  const float sigma = std::isnan(scale) ? static_cast<float>(1.0 / std::sqrt(static_cast<double>(K))) : scale;
  const hipError_t e =
      based::launch_decode_step(q, k, v, B, H, K, V, sigma, state, norm, out, out_dtype == BASED_F32, stream);
  if (e != hipSuccess) return fail(BASED_ERR_HIP, std::string("HIP: ") + hipGetErrorString(e));
  return ok();
}

based_status_t based_timer_create(int max_launches, based_timer** timer) {
  if (!timer || max_launches < 1 || max_launches > (1 << 20))
    return fail(BASED_ERR_INVALID_ARGUMENT, "timer: bad arguments");
  *timer = nullptr;
  based_timer* t = new based_timer;
  t->capacity = max_launches;
  t->events.assign(2 * static_cast<size_t>(max_launches), nullptr);
  t->kernel_ids.assign(static_cast<size_t>(max_launches), -1);
  for (auto& ev : t->events) {
    const hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) {
      based_timer_destroy(t);
      return fail(BASED_ERR_HIP, std::string("hipEventCreate: ") + hipGetErrorString(e));
    }
  }
  *timer = t;
  return ok();
}

void based_timer_destroy(based_timer* timer) {
  if (!timer) return;
  for (auto& ev : timer->events)
    if (ev) (void)hipEventDestroy(ev);
  delete timer;
}

void based_timer_reset(based_timer* timer) {
  if (timer) timer->used = 0;
}

void based_timer_set_kernel_mask(based_timer* timer, unsigned mask) {
  if (timer) timer->mask = mask;
}

based_status_t based_timer_read(based_timer* timer, int kernel_id, int* launches, double* total_ms) {
  if (!timer || !launches || !total_ms) return fail(BASED_ERR_INVALID_ARGUMENT, "timer: bad arguments");
  int n = 0;
  double sum = 0.0;
  for (int i = 0; i < timer->used; ++i) {
    if (timer->kernel_ids[i] != kernel_id) continue;
    hipError_t e = hipEventSynchronize(timer->events[2 * i + 1]);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, timer->events[2 * i], timer->events[2 * i + 1]);
    if (e != hipSuccess) return fail(BASED_ERR_HIP, std::string("timer: ") + hipGetErrorString(e));
    ++n;
    sum += ms;
  }
  *launches = n;
  *total_ms = sum;
  return ok();
}

based_status_t based_device_info(int device, int* compute_units, int* peak_clock_khz, int* l2_bytes) {
  const struct {
    hipDeviceAttribute_t attr;
    int* dst;
  } q[3] = {{hipDeviceAttributeMultiprocessorCount, compute_units},
            {hipDeviceAttributeClockRate, peak_clock_khz},
            {hipDeviceAttributeL2CacheSize, l2_bytes}};
  for (const auto& e : q) {
    if (!e.dst) continue;
    const hipError_t err = hipDeviceGetAttribute(e.dst, e.attr, device);
    if (err != hipSuccess) return fail(BASED_ERR_HIP, std::string("device info: ") + hipGetErrorString(err));
  }
  return ok();
}

const char* based_kernel_name(int kernel_id) {
  switch (kernel_id) {
    case 0: return "based_segment_state_kernel";
    case 1: return "based_segment_scan_kernel";
    case 2: return "based_chunk_readout_kernel";
  }
  return nullptr;
}

}  // extern "C"
