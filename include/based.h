/*
 * based.h - C ABI of the MI355X (gfx950) causal Based forward.
 *
 * The operation is the one defined on the page "Write a fast Based (Taylor linear attention) forward
 * kernel" (KBench task spec based_forward.py), fields spec_md and contract_md: for every batch b, head h
 * and position i,
 *
 *     s[i,j] = scale * (q_i . k_j)
 *     A[i,j] = 1 + s[i,j] + s[i,j]^2 / 2        for j <= i (causal, diagonal included), else 0
 *     o_i    = ( sum_j A[i,j] v_j ) / ( sum_j A[i,j] + 1e-6 )
 *
 * evaluated as linear attention over the feature map phi(x) = [1, x, x(x)x / sqrt(2)] with an fp32 state,
 * chunked along the sequence (the page allows any chunking or algebraic rearrangement that matches).
 *
 * Layouts (all row-major, contiguous, no padding; element (b,t,h,c) of a (B,T,H,X) tensor sits at
 * ((b*T + t)*H + h)*X + c):
 *     q, k : (B, T, H, K) bfloat16, device memory, read-only
 *     v    : (B, T, H, V) bfloat16, device memory, read-only
 *     out  : (B, T, H, V) bfloat16 or float32, device memory, every element written exactly once
 *
 * Supported: K in {8, 16}; V a multiple of 64 in [64, 512]; any B, T, H >= 1 (T need not be a multiple
 * of any chunk length) with T * H * V * 4 <= 2^31 - 1 (the rows of one (b, h) are addressed through
 * 32-bit buffer ranges). Device pointers must be 16-byte aligned; out must not overlap q, k, v or the
 * workspace.
 *
 * Ownership: the caller owns q, k, v, out and any workspace; the library never frees or keeps them.
 * Execution: asynchronous on `stream` (no device synchronisation); launch errors are returned as
 * BASED_ERR_HIP, faults inside a kernel surface at the caller's next synchronisation. Argument errors
 * are detected on the host before any HIP call is made, and nothing is enqueued in that case.
 * Thread safety: all entry points are re-entrant (a timer object must not be shared between threads).
 * The only global state is based_forward_noalloc's static scratch and its per-device address, looked up
 * under a mutex. Calls that share a workspace buffer, or that use the static scratch on one device, must
 * be ordered (e.g. on one stream).
 * Determinism: for a given device and shape, the reduction order is fixed, so results are bitwise
 * repeatable.
 */
#ifndef BASED_H
#define BASED_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Raised whenever an entry point is added or changed; 3 added based_device_info, 4 based_forward_noalloc. */
#define BASED_ABI_VERSION 4

typedef enum {
    BASED_OK = 0,
    BASED_ERR_INVALID_ARGUMENT = 1,   /* null pointer, non-positive size, misalignment, overlap, inf scale */
    BASED_ERR_UNSUPPORTED = 2,        /* K or V outside the supported set, T * H * V too large, or 2^30 or more
                                         work items (B * H * column groups * segments) */
    BASED_ERR_HIP = 3,                /* a HIP runtime call or kernel launch failed */
    BASED_ERR_OUT_OF_MEMORY = 4,      /* the workspace could not be allocated */
    BASED_ERR_WORKSPACE_TOO_SMALL = 5 /* the caller's workspace is smaller than required */
} based_status_t;

typedef enum { BASED_BF16 = 0, BASED_F32 = 1 } based_dtype_t;

/* Returns BASED_ABI_VERSION of the built library. */
int based_abi_version(void);

/* Static, human-readable name of a status code. */
const char* based_status_string(based_status_t status);

/* Detail text of the last error returned on the calling thread ("" if none). Valid until the next call
 * on the same thread. */
const char* based_last_error_detail(void);

/* Bytes of device workspace `based_forward_ws` needs for this shape (0 if the sequence is processed in a
 * single segment). The sizes are validated as in based_forward; unsupported shapes return 0. */
size_t based_forward_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V);

/*
 * Causal Based forward (spec_md / contract_md of the page above).
 *   scale : the factor on the scores s = scale * (q . k); the page applies it to the query side alone.
 *           NaN stands for the page's default, (float)K**-0.5 with K the key width (V does not enter).
 *           +-inf is rejected.
 *   out_dtype : BASED_BF16 (round to nearest even) or BASED_F32.
 * Gets its workspace with hipMallocAsync / hipFreeAsync on `stream` (stream-ordered).
 */
based_status_t based_forward(const void* q, const void* k, const void* v,
                             int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                             float scale, void* out, based_dtype_t out_dtype, hipStream_t stream);

/* Same as based_forward, with a caller-provided device workspace of at least
 * based_forward_workspace_bytes(...) bytes (may be NULL when that is 0). No allocation is made and no
 * memory is cleared with a memset: the call only launches kernels on `stream`, so it can be recorded into
 * a HIP graph and replayed (the pointers are baked into the graph). */
based_status_t based_forward_ws(const void* q, const void* k, const void* v,
                                int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                                float scale, void* out, based_dtype_t out_dtype,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * based_forward for callers that cannot allocate device memory: code recorded under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same operation and arguments as based_forward;
 * no allocation of any kind is made (no hipMalloc, hipMallocAsync or library allocation). The workspace
 * is a static device array of the library, based_noalloc_scratch_bytes() bytes (32 MiB) on every device
 * the library runs on, held until the process ends; its device address is looked up on the first call on
 * a device (the device of `stream`) and kept.
 *   Errors: as based_forward; BASED_ERR_UNSUPPORTED when the shape's plan needs more workspace than the
 *   static scratch holds (no shape of the automatic plans does up to now: they need at most ~21 MiB).
 * Every call on one device shares that device's scratch (the segment state sums are fully written before
 * they are read, so nothing carries over from an earlier call): calls that overlap in time on one
 * device, such as calls on two streams without ordering between them, race and give wrong results.
 */
based_status_t based_forward_noalloc(const void* q, const void* k, const void* v,
                                     int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                                     float scale, void* out, based_dtype_t out_dtype, hipStream_t stream);

/* Bytes of the static scratch of based_forward_noalloc. */
size_t based_noalloc_scratch_bytes(void);

/* ---------------------------------------------------------------------------------------------------
 * State on either side of the forward: carried in and out, and the one-token recurrent step.
 *
 * The page's reference (field reference_src) keeps, for every (b, h), the state of the tokens processed so
 * far: S = sum_j phi(k_j) v_j^T, a P x V matrix, and z = sum_j phi(k_j), a length-P vector, with
 * phi(x) = [1, x, x (x) x / sqrt(2)] (field spec_md), P = 1 + K + K^2, k unscaled (the scale multiplies q
 * only, field contract_md). Layout, fp32, row-major, contiguous: S of (B, H, P, V), element (b, h, r, c)
 * at ((b*H + h)*P + r)*V + c; z of (B, H, P). Row 0 is the constant feature, rows 1 .. K the linear
 * block, row 1 + K + a*K + b holds x_a x_b / sqrt(2). The page grades the forward alone (field
 * contract_md excludes an initial state); these entry points are the steps on either side of it.
 * ------------------------------------------------------------------------------------------------- */

/* P = 1 + K + K^2: rows of the state for feature dimension K. */
int64_t based_feature_dim(int64_t K);

/*
 * based_forward with a state: the tokens are read out as if preceded by the tokens that produced
 * (state_in, norm_in), and the state after the last token is written to (state_out, norm_out).
 *   state_in, norm_in   : device, read-only, (B, H, P, V) and (B, H, P) fp32, or both NULL (no earlier
 *                         tokens). Only the symmetric part of the quadratic block can reach an output
 *                         (phi(q) . S weighs rows (a, b) and (b, a) alike), and only that part is read.
 *   state_out, norm_out : device, (B, H, P, V) and (B, H, P) fp32, fully written, or both NULL. The two
 *                         rows of an off-diagonal pair come out equal. Must not overlap any other argument
 *                         (in particular state_out may not alias state_in: carry state through a second
 *                         buffer).
 *   workspace           : as in based_forward_ws, or NULL to allocate it stream-ordered as based_forward does.
 * Splitting a sequence into pieces, each called with the state the previous piece returned, gives the
 * outputs and final state of one call over the whole sequence (up to rounding).
 */
based_status_t based_forward_state(const void* q, const void* k, const void* v,
                                   int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                                   float scale, void* out, based_dtype_t out_dtype,
                                   const float* state_in, const float* norm_in,
                                   float* state_out, float* norm_out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One token of the recurrence for every (b, h): the token is folded into the state first (the causal
 * sum includes the diagonal, field contract_md), then read out:
 *     S += phi(k) v^T,  z += phi(k),  o = phi(scale q) S / (phi(scale q) z + 1e-6).
 *   q, k  : device, (B, H, K) bf16 (one token; the same bytes as a (B, 1, H, K) tensor)
 *   v     : device, (B, H, V) bf16
 *   state, norm : device, (B, H, P, V) and (B, H, P) fp32, updated in place (layout above)
 *   out   : device, (B, H, V), bf16 (round to nearest even) or fp32
 * Supported K and V as for based_forward. Asynchronous on `stream`; no allocation.
 */
based_status_t based_decode_step(const void* q, const void* k, const void* v,
                                 int64_t B, int64_t H, int64_t K, int64_t V,
                                 float scale, float* state, float* norm,
                                 void* out, based_dtype_t out_dtype, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------------
 * Execution plan and instrumentation (same operation; for tests and measurement).
 * ------------------------------------------------------------------------------------------------- */

/* The sequence is split into `segments` pieces of `segment_len` tokens (the last may be shorter); each
 * piece of each (b, h, group of 64 value columns, or 128 when V is a multiple of 128) is processed by one
 * workgroup in chunks of 64 tokens (128 for 128 columns with K = 16); a first kernel sums the state of
 * every piece but the last into the workspace (each in two halves when it would otherwise run at most one
 * workgroup per compute unit and the halves are at least 1024 tokens), and the read-out of piece g starts
 * from the sum of those sums for pieces 0 .. g - 1 (with more than 15 such sums before a piece, a
 * prefix-scan kernel forms the running sums in between). Reports the plan chosen for a shape (the
 * workspace size tells the number of sums); segment_len_override > 0 forces that length (rounded up to a
 * whole number of chunks). */
based_status_t based_forward_plan(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                                  int64_t segment_len_override, int64_t* segments,
                                  int64_t* segment_len, size_t* workspace_bytes);

/* Opaque recorder of HIP events placed around the kernels launched by based_forward_ex. */
typedef struct based_timer based_timer;

/* Creates a recorder with room for `max_launches` kernel launches. */
based_status_t based_timer_create(int max_launches, based_timer** timer);
void based_timer_destroy(based_timer* timer);
/* Forgets all recorded launches (events are reused). */
void based_timer_reset(based_timer* timer);
/* Restricts recording to the kernels whose bit (1 << kernel_id) is set in `mask` (default: all). Each
 * recorded launch adds two event records to the stream. */
void based_timer_set_kernel_mask(based_timer* timer, unsigned mask);
/* Waits for the recorded events and returns, for kernel `kernel_id` (0 = segment state sums,
 * 1 = segment prefix scan, 2 = chunked read-out), the number of recorded launches and their summed
 * duration in milliseconds. */
based_status_t based_timer_read(based_timer* timer, int kernel_id, int* launches, double* total_ms);
/* Properties of HIP device `device` that measurements are reported with: compute units, peak shader
 * clock in kHz, L2 cache bytes (per device as HIP reports it). Any output pointer may be NULL.
 * Errors: BASED_ERR_HIP when the device cannot be queried. */
based_status_t based_device_info(int device, int* compute_units, int* peak_clock_khz, int* l2_bytes);
/* Static name of kernel `kernel_id` as it appears in profiler traces, or NULL. */
const char* based_kernel_name(int kernel_id);

/* based_forward_ws with an optional forced segment length (0 = automatic) and an optional timer
 * (NULL = none). */
based_status_t based_forward_ex(const void* q, const void* k, const void* v,
                                int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                                float scale, void* out, based_dtype_t out_dtype,
                                void* workspace, size_t workspace_bytes,
                                int64_t segment_len_override, based_timer* timer, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BASED_H */
