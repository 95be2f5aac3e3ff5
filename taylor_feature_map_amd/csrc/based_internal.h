// Internal declarations shared by the kernels and the C-ABI layer of the causal Based forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace based {

constexpr int kWave = 64;    // wavefront width on CDNA

struct Shape {
  int64_t B, T, H, K, V;
};

// Sequence split: `segments` pieces of `seg_len` tokens (last one possibly shorter); work items of
// `item_cols` value columns (64, or 128 when V is a multiple of 128), `nvs` of them per (b, h);
// `slot_floats` floats per stored segment state sum. With `scanned` set, the stored sums are turned into
// prefix sums by a scan kernel before the read-out; otherwise every read-out adds up the sums of its
// predecessors itself.
struct Plan {
  int64_t segments, seg_len, nvs, item_cols, slot_floats;
  int64_t sub;  // state sums per segment: the state pass splits each segment but the last into sub pieces
  bool scanned;
  bool affine;  // XCD-affine work items (every segment of a (b, h, columns) pair on one XCD)
  bool row_stores;  // bf16 output tiles staged through LDS and stored as whole rows
};

// State sums per (b, h, item columns): sub for every segment but the last.
__host__ __device__ __forceinline__ int64_t state_slots(const Plan& pl) { return (pl.segments - 1) * pl.sub; }

// Upper bound on the work items (blocks) of one launch; below it all item index arithmetic fits in 32 bits.
constexpr int64_t kMaxItems = (int64_t(1) << 31) - 8;

// Most state sums before a read-out's segment for which it adds them up itself (beyond this, the quadratic
// number of slot reads costs more than a scan kernel).
constexpr int64_t kMaxSummedSlots = 15;

template <int B, int E, typename F>
__host__ __device__ __forceinline__ void constexpr_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    constexpr_for<B + 1, E>(f);
  }
}

// Value columns per work item for V; floats per segment state sum, tokens per chunk (segment lengths are
// multiples of it) and wavefronts per work item for feature dimension K and `item_cols` columns.
int item_columns(int64_t V);
int state_slot_floats(int64_t K, int64_t item_cols);
int state_value_groups(int64_t K, int64_t item_cols);
int chunk_tokens(int64_t K, int64_t item_cols);
int waves_per_item(int64_t K, int64_t item_cols);

// Optional state in the page's layout, fp32: S of (B, H, P, V) and z of (B, H, P), P = 1 + K + K^2. The
// read-out adds s_in / z_in to its starting state and writes the state after the last token to s_out /
// z_out (either pair may be null).
struct StateIO {
  const float* s_in;
  const float* z_in;
  float* s_out;
  float* z_out;
};

// kernel_id: 0 = segment state sums, 1 = prefix over segments, 2 = chunked read-out.
hipError_t launch_kernel(int kernel_id, const void* q, const void* k, const void* v, const Shape& sh,
                         const Plan& pl, float sigma, float* ws, void* out, bool out_f32, const StateIO& io,
                         hipStream_t stream);

// One-token recurrent step on (B, H) rows of q, k (K) and v (V), state S (B, H, P, V) and z (B, H, P) updated
// in place.
hipError_t launch_decode_step(const void* q, const void* k, const void* v, int64_t B, int64_t H, int64_t K,
                              int64_t V, float sigma, float* S, float* z, void* out, bool out_f32, hipStream_t stream);

// Bytes of the static device scratch that based_forward_noalloc uses as its workspace.
constexpr size_t kScratchBytes = size_t(32) << 20;

// Device address of that scratch on the device that `stream` belongs to, looked up once per device and
// kept. No allocation is made.
hipError_t scratch_buffer(hipStream_t stream, void** ptr);

}  // namespace based
