// Causal Based forward for MI355X (gfx950): chunked 2nd-order Taylor linear attention on bf16 MFMA.
//
// What is computed: the page "Write a fast Based (Taylor linear attention) forward kernel" (KBench task
// spec based_forward.py), field spec_md: o_i = sum_{j<=i} A_ij v_j / (sum_{j<=i} A_ij + 1e-6) with
// A_ij = 1 + s + s^2/2, s = scale * q_i.k_j. Per field spec_md, A_ij = phi(q_i).phi(k_j) for the feature
// map phi(x) = [1, x, x(x)x/sqrt(2)], so the sum over earlier tokens is a read-out of the running state
// S = sum phi(k_j) v_j^T and normaliser z = sum phi(k_j), and only the tokens of the current chunk need
// the direct polynomial (field reference_src; field perf_md describes the same split).
//
// Design:
//  * Work item = (batch b, head h, 64 or 128 value columns, sequence segment), run by a workgroup of W
//    wavefronts over chunks of C tokens (see Split: K = 16 with 64 columns W = 4, C = 64; with 128
//    columns W = 8, C = 128; K = 8: W = 2 or 4, C = 64). The feature tiles of the state are split between
//    the waves for the update; every wave reads out its 16-token query tile(s) of each chunk through the
//    whole state, whose bf16 copy the waves publish to LDS after each chunk.
//  * The quadratic block is used in its symmetric form: the page allows any algebraic rearrangement that
//    matches (field spec_md). Unordered feature pairs {a, b} are laid out on a 16-lane row as "cyclic
//    distance" tiles: tile d holds x_n * x_{(n-d) mod 16} in lane n, so every partner is a DPP row
//    rotation of the lane's own feature. K = 16 needs 10 tiles of 16 features (153 used of 160):
//    d = 0..7 (diagonal and 7 full distances), d = 8 (8 pairs) plus the constant feature, and the linear
//    tile. The q side carries the coefficients (s^2/2 gives 1/2 on the diagonal, 1 off it).
//  * A 16-column "ones" tile next to the 64 value columns makes z, phi(q).z and the intra-chunk row sums
//    fall out of the same MFMAs (field perf_md: no second matmul for the normaliser). S and z stay fp32
//    for the whole segment (field precision_md) and are rounded to bf16 only as MFMA operands; the
//    Taylor weights are squared in fp32 and rounded once.
//  * Per chunk: phi(Q) S for the wave's query tiles, then per 32-token key step K Q^T, the Taylor
//    weights and A V into the same fp32 tile, the fused divide and store, and S += phi(K)^T V. phi is
//    built in registers and never written to memory (field perf_md names materialising it as the waste).
//  * Global memory goes through buffer resources (32-bit per-lane offsets, the chunk advance in the
//    scalar offset, the range check covering the ragged end of the sequence). Inputs are loaded one
//    chunk ahead into registers and staged in LDS in their natural row layout (16-byte units of V
//    swizzled against bank conflicts); V and K with the token index along the contraction come from
//    ds_read_b64_tr_b16 transpose reads.
//  * Long sequences are split into segments so that all SIMDs have work (two waves per SIMD): a first
//    kernel sums phi(k)^T v per segment (every segment but the last; per half segment when one workgroup
//    per segment would leave it at most one per CU), and the read-out of segment g starts from the sum of
//    the sums before it, added in sequence order at its start. With more than 15 such sums a prefix-scan
//    kernel turns them into those starting states first.
//  * Work items are placed on the 8 XCDs so that shared q/k cache lines, and where the heads allow it all
//    segments of a (b, h) and hence the segment sums, stay in one XCD's L2 (readout_item, state_item).
//  * The one-token decode step is a separate, purely memory-bound kernel over the state in the page's
//    layout (based_decode_step_kernel).
//
// MFMA lane layouts used (v_mfma_f32_16x16x32_bf16, lane l, column c = l % 16, group g = l / 16):
//   A operand: row c, contraction slots 8g..8g+7;  B operand: column c, slots 8g..8g+7;
//   D: column c, rows 4g..4g+3.  The contraction order is free as long as A and B agree; slot e of
//   group g is token 16(e/4) + 4g + e%4 of a 32-token key step, which lets the D registers of K Q^T
//   feed the attention weights as an operand, and feature (t, 4g + e%4) of tile pair (t = 2m + e/4),
//   which lets the D registers of S feed the read-out, without any data movement. Outputs are
//   computed transposed (value column along the rows, token along the lanes) so that a lane holds four
//   adjacent output columns of one token.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "based_internal.h"

namespace based {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

constexpr unsigned kOnesBf16x2 = 0x3F803F80u;

// ------------------------------------------------------------------------------------------ helpers

__device__ __forceinline__ unsigned pack2(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2_t));  // RNE
}
__device__ __forceinline__ float lo_f(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_f(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

// DPP row rotation: lane n of each 16-lane row receives the value of lane (n - D) mod 16.
template <int D>
__device__ __forceinline__ float ror(float x) {
  if constexpr (D == 0) {
    return x;
  } else {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + D, 0xf, 0xf, true));
  }
}

__device__ __forceinline__ f32x4_t mfma32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(u32x2_t a, u32x2_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                   __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

// Transpose read: within each 16-lane group, lane 4a + c receives element c of the 4-element rows
// addressed by lanes a, a + 4, a + 8, a + 12 of that group.
__device__ __forceinline__ u32x2_t lds_tr16(const u16* p) {
  const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}

// Work item of a block: blocks are dealt to the 8 XCDs round robin, so block x runs on XCD x % 8.
// Consecutive items (neighbouring heads of one batch and segment, which share cache lines of q and k)
// are given to one XCD so that they meet in its L2.
// ------------------------------------------------------------------------- feature tiles (phi)

template <int K>
struct Feat;

// Query side, for the lane's token: u[m] = q[(4g + m) mod NQ'] (the raw values, rotated per lane group;
// NQ' = K), and for the lane's own four rows r: a[r] = scale^2 u[r], h[r] = a[r] / 2, l[r] = scale u[r].
// The scale factors sit on the lane's own row only, so a product needs one multiply.
struct QSide {
  const float* u;
  const float* a;
  const float* h;
  const float* l;
};

// K = 16. k side: lane column c holds x = k[c] for one token; tile T returns that lane's feature.
// q side: feature (T, n = 4g + R) is returned for slot R.
template <>
struct Feat<16> {
  static constexpr int NPT = 10;
  static constexpr int NQ = 16;
  template <int T>
  __device__ static __forceinline__ float kval(float x, int c) {
    if constexpr (T == 0) {
      return x * x;
    } else if constexpr (T <= 7) {
      return x * ror<T>(x);
    } else if constexpr (T == 8) {
      const float p = x * ror<8>(x);
      return c < 8 ? p : (c == 8 ? 1.0f : 0.0f);
    } else {
      return x;
    }
  }
  template <int T, int R>
  __device__ static __forceinline__ float qval(const QSide& y, int g) {
    if constexpr (T == 0) {
      return y.h[R] * y.u[R];
    } else if constexpr (T <= 7) {
      return y.a[R] * y.u[(R - T) & 15];
    } else if constexpr (T == 8) {
      const float p = y.a[R] * y.u[(R - 8) & 15];
      return g < 2 ? p : ((g == 2 && R == 0) ? 1.0f : 0.0f);
    } else if constexpr (T == 9) {
      return y.l[R];
    } else {
      return 0.0f;
    }
  }
};

// K = 8: the 16-lane row holds the 8 features twice (lane c has feature c % 8); half h = c / 8.
// Tiles: 0 = {h0: diagonal, h1: distance 1}, 1 = {h0: distance 2, h1: distance 3},
//        2 = {h0: distance 4 on features 0..3, constant on feature 4, h1: linear}; 45 of 48 used.
// q side: u[m] = q[(4 (g & 1) + m) mod 8].
template <>
struct Feat<8> {
  static constexpr int NPT = 3;
  static constexpr int NQ = 8;
  template <int T>
  __device__ static __forceinline__ float kval(float x, int c) {
    const bool h0 = c < 8;
    if constexpr (T == 0) {
      const float d1 = x * ror<1>(x);
      return h0 ? x * x : d1;
    } else if constexpr (T == 1) {
      const float d2 = x * ror<2>(x);
      const float d3 = x * ror<3>(x);
      return h0 ? d2 : d3;
    } else {
      const float d4 = x * ror<4>(x);
      const int f = c & 7;
      return h0 ? (f < 4 ? d4 : (f == 4 ? 1.0f : 0.0f)) : x;
    }
  }
  template <int T, int R>
  __device__ static __forceinline__ float qval(const QSide& y, int g) {
    const bool h0 = g < 2;
    // Both candidates of a tile are formed before the select: written as a choice between two array
    // elements, the compiler folds it into one load at an offset that depends on g and keeps the query
    // arrays in scratch memory.
    if constexpr (T == 0) {
      const float p0 = y.h[R] * y.u[R];
      const float p1 = y.a[R] * y.u[(R - 1) & 7];
      return h0 ? p0 : p1;
    } else if constexpr (T == 1) {
      const float p2 = y.a[R] * y.u[(R - 2) & 7];
      const float p3 = y.a[R] * y.u[(R - 3) & 7];
      return h0 ? p2 : p3;
    } else if constexpr (T == 2) {
      const float p = y.a[R] * y.u[(R - 4) & 7];
      return h0 ? ((g & 1) == 0 ? p : (R == 0 ? 1.0f : 0.0f)) : y.l[R];
    } else {
      return 0.0f;
    }
  }
};

// Feature (tile t, row n) of the kernels against the rows of the page's phi (field spec_md): row 0 is the
// constant, rows 1 .. K the linear block, row 1 + K + a K + b holds x_a x_b / sqrt(2). The kernels keep
// each unordered pair {a, b} once, unscaled (the query side carries the coefficients), so a state in the
// page's layout maps to them as: constant and linear rows as they are, diagonal (a, a) times sqrt(2), and
// pair {a, b} as (row (a, b) + row (b, a)) / sqrt(2); the other way round both rows of a pair get the
// kernel value / sqrt(2). Only the symmetric part of an imported quadratic block can reach an output.
enum : int { kFeatNone = 0, kFeatConst = 1, kFeatLin = 2, kFeatDiag = 3, kFeatPair = 4 };
struct FeatRows {
  int kind, a, b;
};
constexpr float kSqrt2 = 1.41421356237309515f;
constexpr float kRSqrt2 = 0.707106781186547573f;

template <int K>
__device__ __forceinline__ FeatRows feat_rows(int t, int n) {
  if constexpr (K == 16) {
    if (t == 0) return {kFeatDiag, n, n};
    if (t <= 7) return {kFeatPair, n, (n - t) & 15};
    if (t == 8) return n < 8 ? FeatRows{kFeatPair, n, n + 8} : FeatRows{n == 8 ? kFeatConst : kFeatNone, 0, 0};
    return {kFeatLin, n, n};
  } else {
    const int f = n & 7, h = n >> 3;
    if (t == 0) return h == 0 ? FeatRows{kFeatDiag, f, f} : FeatRows{kFeatPair, f, (f - 1) & 7};
    if (t == 1) return {kFeatPair, f, (f - (h == 0 ? 2 : 3)) & 7};
    if (h == 1) return {kFeatLin, f, f};
    return f < 4 ? FeatRows{kFeatPair, f, f + 4} : FeatRows{f == 4 ? kFeatConst : kFeatNone, 0, 0};
  }
}

template <int K>
__device__ __forceinline__ int quad_row(int a, int b) {
  return 1 + K + a * K + b;
}

// Kernel value of a feature from a state in the page's layout; x(row) reads the lane's entry of a row.
template <int K, typename X>
__device__ __forceinline__ float import_feature(const FeatRows& fr, X x) {
  switch (fr.kind) {
    case kFeatConst: return x(0);
    case kFeatLin: return x(1 + fr.a);
    case kFeatDiag: return kSqrt2 * x(quad_row<K>(fr.a, fr.a));
    case kFeatPair: return (x(quad_row<K>(fr.a, fr.b)) + x(quad_row<K>(fr.b, fr.a))) * kRSqrt2;
    default: return 0.0f;
  }
}

// Writes a kernel feature value into the page's layout; w(row, value) stores the lane's entry of a row.
template <int K, typename Wr>
__device__ __forceinline__ void export_feature(const FeatRows& fr, float val, Wr w) {
  switch (fr.kind) {
    case kFeatConst: w(0, val); break;
    case kFeatLin: w(1 + fr.a, val); break;
    case kFeatDiag: w(quad_row<K>(fr.a, fr.a), val * kRSqrt2); break;
    case kFeatPair:
      w(quad_row<K>(fr.a, fr.b), val * kRSqrt2);
      w(quad_row<K>(fr.b, fr.a), val * kRSqrt2);
      break;
    default: break;
  }
}

// ----------------------------------------------------------------------------- work split

#ifndef BASED_CHUNK16
#define BASED_CHUNK16 64
#endif

// Compile-time configuration of a work item: feature dimension K and VS value columns (64, or 128 when V
// is a multiple of 128), plus the ones tile that carries the normaliser: NVT = VS / 16 + 1 value tiles,
// the ones tile last.
template <int K_, int VS_>
struct Cfg {
  static constexpr int K = K_;
  static constexpr int VS = VS_;
  static constexpr int NVV = VS / 16;  // value tiles
  static constexpr int NVT = NVV + 1;  // value tiles and the ones tile
  static constexpr int ONES = NVV;     // index of the ones tile
};

// One work item (b, h, value columns, segment) runs on a workgroup of W waves over chunks of C tokens
// (NKS key steps of 32). Wave w owns the state feature tiles [T0(w), T0(w) + NT(w)) for the update and
// finishes QPW of the chunk's 16-token query tiles, Q(w, 0 .. QPW - 1). Query tile i meets i / 2 + 1 key
// steps inside the chunk, so the assignment evens out the work: the waves with more feature tiles take
// the query tiles with fewer earlier keys in the chunk.
//   K = 16, 64 columns:  W = 4, C = 64, feature tiles 3 + 3 + 2 + 2, one query tile per wave.
//   K = 16, 128 columns: W = 8, C = 128, feature tiles 2 + 2 + 1 x 6, one query tile per wave.
//   K = 8, 64 columns:   W = 2, C = 64, feature tiles 2 + 1, query tile pairs {0, 3} and {1, 2}.
//   K = 8, 128 columns:  W = 4, C = 64, feature tiles 1 + 1 + 1 + 0, one query tile per wave.
// (With C = 128 and 64 columns, K = 16 would pair {0, 5}, {1, 4} and {2, 7}, {3, 6}.) A shorter chunk
// means less causal work inside each chunk (a query meets C / 2 earlier keys of its chunk on average)
// against one more state publish per C tokens; 128 columns share phi, the scores and the ones tile
// between twice as many outputs.
template <class Cf>
struct Split {
  static constexpr int K = Cf::K;
  static constexpr bool WIDE = Cf::VS == 128;
  static constexpr int W = K == 16 ? (WIDE ? 8 : 4) : (WIDE ? 4 : 2);
  static constexpr int C = K == 16 ? (WIDE ? 128 : BASED_CHUNK16) : 64;
  static constexpr int NKS = C / 32;
  static constexpr int QPW = C / 16 / W;
  static_assert(QPW >= 1 && QPW <= 2 && QPW * 16 * W == C, "one or two query tiles per wave");
  __host__ __device__ static constexpr int T0(int w) {
    return K == 16 ? (WIDE ? (w < 2 ? 2 * w : w + 2) : (w < 2 ? 3 * w : 6 + 2 * (w - 2))) : (WIDE ? w : 2 * w);
  }
  __host__ __device__ static constexpr int NT(int w) {
    return K == 16 ? (WIDE ? (w < 2 ? 2 : 1) : (w < 2 ? 3 : 2)) : (WIDE ? (w < 3 ? 1 : 0) : (w == 0 ? 2 : 1));
  }
  __host__ __device__ static constexpr int Q(int w, int i) {
    return QPW == 1 ? w : (i == 0 ? w : (K == 16 ? (w < 2 ? 5 - w : 9 - w) : 3 - w));
  }
};

// ------------------------------------------------------------------------------ LDS staging

// One chunk of one work item, natural row layout: q[C][K], k[C][K], and v[C][VS] where the 16-byte unit
// `oct` (columns 8 oct .. 8 oct + 7) of token t is stored at position oct ^ (t % 8).
template <class Cf>
struct __align__(16) Stage {
  static constexpr int C = Split<Cf>::C;
  u16 q[C * Cf::K];
  u16 k[C * Cf::K];
  u16 v[C * Cf::VS];
};

template <int VS>
__device__ __forceinline__ int v_index(int tok, int col) {
  return tok * VS + (((col >> 3) ^ (tok & 7)) << 3) + (col & 7);
}

// The 16-byte units of one chunk: NQK q units, NQK k units, then C VS / 8 value units. Unit u lands at
// u16 offset 8 u of its LDS region. Global reads go through buffer resources whose range ends at token T,
// so units of tokens >= T read as zero; such tokens only ever meet zero Taylor weights or an update whose
// result is discarded.
template <class Cf>
struct Units {
  static constexpr int K = Cf::K;
  static constexpr int C = Split<Cf>::C;
  static constexpr int UPR = Cf::VS / 8;  // value units per token row
  static constexpr int NQK = C * K / 8;
  static constexpr int NV = C * UPR;
  static constexpr int NU = 2 * NQK + NV;
  static constexpr int PER_Q = K / 8;  // units per token row of q or k
  // Byte offset of q/k unit u relative to the chunk's first token.
  __device__ static __forceinline__ unsigned qk_off(int u, unsigned stride_bytes) {
    return (u / PER_Q) * stride_bytes + (u % PER_Q) * 16;
  }
  // Byte offset of value unit f (LDS position f % UPR of token f / UPR) relative to the chunk's first token.
  __device__ static __forceinline__ unsigned v_off(int f, unsigned stride_bytes) {
    const int tok = f / UPR, pos = f % UPR;
    return tok * stride_bytes + ((pos ^ (tok & 7)) << 4);
  }
};

// Buffer resource over the rows of one (b, h, value columns): base points at token 0, the range ends at
// token T (stride_bytes per token).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t T, int64_t stride_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(T * stride_bytes),
                                           0x00020000);
}

__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Per-item global addressing: buffer resources and row strides in bytes.
struct Rows {
  __amdgpu_buffer_rsrc_t q, k, v;
  unsigned qk_stride, v_stride;
};

// Chunk loader: the units of q (if WITH_Q), k and v spread over all threads of the workgroup, one
// chunk ahead of use, through registers. Every region is a multiple of 64 units long, so the region of
// each of wave WI's loads is known at compile time (no divergent branches around the loads).
template <class Cf, bool WITH_Q, int WI, int NW = Split<Cf>::W>
struct Prefetch {
  using U = Units<Cf>;
  static constexpr int NTH = NW * kWave;
  static constexpr int FIRST = WITH_Q ? 0 : U::NQK;  // q units are skipped without q
  static constexpr int PER = (U::NU - FIRST + NTH - 1) / NTH;
  static_assert(U::NQK % kWave == 0 && U::NV % kWave == 0, "regions must be whole waves");
  // First unit of load i of this wave, and its region: 0 = q, 1 = k, 2 = v, 3 = none.
  static constexpr int u0(int i) { return FIRST + WI * kWave + i * NTH; }
  static constexpr int region(int i) {
    return u0(i) >= U::NU ? 3 : u0(i) >= 2 * U::NQK ? 2 : u0(i) >= U::NQK ? 1 : 0;
  }
  u32x4_t r[PER];
  unsigned off[PER];
  __device__ __forceinline__ void init(const Rows& rw, int lane) {
    constexpr_for<0, PER>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int reg = region(i);
      const int u = u0(i) + lane;
      if constexpr (reg == 0) off[i] = U::qk_off(u, rw.qk_stride);
      else if constexpr (reg == 1) off[i] = U::qk_off(u - U::NQK, rw.qk_stride);
      else if constexpr (reg == 2) off[i] = U::v_off(u - 2 * U::NQK, rw.v_stride);
    });
  }
  __device__ __forceinline__ void load(const Rows& rw, int64_t t0) {
    const unsigned sqk = static_cast<unsigned>(t0) * rw.qk_stride;
    const unsigned sv = static_cast<unsigned>(t0) * rw.v_stride;
    constexpr_for<0, PER>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int reg = region(i);
      if constexpr (reg == 0) r[i] = buf_load16(rw.q, off[i], sqk);
      else if constexpr (reg == 1) r[i] = buf_load16(rw.k, off[i], sqk);
      else if constexpr (reg == 2) r[i] = buf_load16(rw.v, off[i], sv);
    });
  }
  __device__ __forceinline__ void store(Stage<Cf>& st, int lane) const {
    constexpr_for<0, PER>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int reg = region(i);
      const int u = u0(i) + lane;
      if constexpr (reg == 0) *reinterpret_cast<u32x4_t*>(st.q + u * 8) = r[i];
      else if constexpr (reg == 1) *reinterpret_cast<u32x4_t*>(st.k + (u - U::NQK) * 8) = r[i];
      else if constexpr (reg == 2) *reinterpret_cast<u32x4_t*>(st.v + (u - 2 * U::NQK) * 8) = r[i];
    });
  }
};

// B operand of value tile vt for contraction step ks (tokens 32 ks .. 32 ks + 31): column m <-> value
// column 16 vt + m; slot e <-> token 32 ks + 16(e/4) + 4g + e%4.
template <class Cf>
__device__ __forceinline__ u32x4_t value_operand(const Stage<Cf>& st, int ks, int vt, int lane) {
  const int g = lane >> 4, r = lane & 15;
  const int col = 16 * vt + 4 * (r & 3);
  const int tok = 32 * ks + 4 * g + (r >> 2);
  const u32x2_t a = lds_tr16(st.v + v_index<Cf::VS>(tok, col));
  const u32x2_t b = lds_tr16(st.v + v_index<Cf::VS>(tok + 16, col));
  return u32x4_t{a.x, a.y, b.x, b.y};
}

// Key feature c (K = 8: c % 8) of the lane's 8 token slots of contraction step ks, as floats.
template <class Cf>
__device__ __forceinline__ void key_column(const Stage<Cf>& st, int ks, int lane, float* kx) {
  constexpr int K = Cf::K;
  const int g = lane >> 4, r = lane & 15;
  const int f4 = (K == 16) ? 4 * (r & 3) : 4 * (r & 1);
  const int tok = 32 * ks + 4 * g + (r >> 2);
  const u32x2_t a = lds_tr16(st.k + tok * K + f4);
  const u32x2_t b = lds_tr16(st.k + (tok + 16) * K + f4);
  kx[0] = lo_f(a.x); kx[1] = hi_f(a.x); kx[2] = lo_f(a.y); kx[3] = hi_f(a.y);
  kx[4] = lo_f(b.x); kx[5] = hi_f(b.x); kx[6] = lo_f(b.y); kx[7] = hi_f(b.y);
}

// S[tiles T0 .. T0 + NT) (features x [VS values | ones]) += phi(K)^T [V | 1] over one 32-token step.
template <class Cf, int T0, int NT, typename SA>
__device__ __forceinline__ void state_update_step(SA& S, const float* kx, const u32x4_t (&vop)[Cf::NVT], int c) {
  constexpr int K = Cf::K;
  constexpr_for<0, NT>([&](auto lc) {
    constexpr int lt = decltype(lc)::value;
    constexpr int t = T0 + lt;
    u32x4_t a;
    a.x = pack2(Feat<K>::template kval<t>(kx[0], c), Feat<K>::template kval<t>(kx[1], c));
    a.y = pack2(Feat<K>::template kval<t>(kx[2], c), Feat<K>::template kval<t>(kx[3], c));
    a.z = pack2(Feat<K>::template kval<t>(kx[4], c), Feat<K>::template kval<t>(kx[5], c));
    a.w = pack2(Feat<K>::template kval<t>(kx[6], c), Feat<K>::template kval<t>(kx[7], c));
#pragma unroll
    for (int vt = 0; vt < Cf::NVT; ++vt) S[lt][vt] = mfma32(a, vop[vt], S[lt][vt]);
  });
}

template <class Cf>
__device__ __forceinline__ void load_value_operands(const Stage<Cf>& st, int ks, int lane, u32x4_t (&vop)[Cf::NVT]) {
#pragma unroll
  for (int vt = 0; vt < Cf::NVV; ++vt) vop[vt] = value_operand<Cf>(st, ks, vt, lane);
  vop[Cf::ONES] = u32x4_t{kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};
}

// Register-native layout of one segment state sum of a work item with VS value columns in the workspace:
// the value tiles, 4 entries (the rows r) per lane and tile, as [tile][value tile][lane][r]; then the ones
// tile (z, whose 16 columns are equal) in fp32, 16 bytes per lane group, as [tile][lane group][r]. The value
// tiles are bf16 (8 bytes per lane and tile): the read-out rounds the state to bf16 for its products every
// chunk anyway, so rounding a sum once more costs at most about one bf16 unit of it, while z keeps fp32 (its
// constant feature counts the tokens, exactly in fp32 up to 2^24, and it divides every output). The K = 16,
// 128-column read-out, at the edge of its registers, keeps fp32 value tiles (16 bytes). Offsets in bytes.
template <int K, int VS>
constexpr bool kBf16Slot = !(K == 16 && VS == 128);
template <int K, int VS>
__device__ __forceinline__ int64_t state_offset(int t, int vt, int lane) {
  return ((t * (VS / 16) + vt) * kWave + lane) * (kBf16Slot<K, VS> ? 8 : 16);
}
template <int K, int VS>
__device__ __forceinline__ int64_t ones_offset(int t, int g) {
  return Feat<K>::NPT * (VS / 16) * kWave * (kBf16Slot<K, VS> ? 8 : 16) + (t * 4 + g) * 16;
}
__device__ __forceinline__ u32x2_t to_bf16x4(const f32x4_t& x) {
  return u32x2_t{pack2(x[0], x[1]), pack2(x[2], x[3])};
}
__device__ __forceinline__ f32x4_t from_bf16x4(const u32x2_t& u) {
  return f32x4_t{lo_f(u.x), hi_f(u.x), lo_f(u.y), hi_f(u.y)};
}

struct ItemCoords {
  int64_t b, h, vs, g;
};

// Work items of a launch. Block x runs on XCD x % 8. The grid holds the items rounded up to a multiple of 8
// (fewer than 2^31, so the index arithmetic is 32-bit). By default XCD x takes the x-th eighth of the
// items, numbered (b, segment, columns, h) with h fastest, so neighbouring heads of one (b, segment), whose
// q and k rows share cache lines, meet in one L2. With pl.affine (the host sets it when the
// (b, columns, h) pairs divide evenly over the XCDs in runs of whole 128-byte q/k lines) XCD x takes a
// contiguous run of pairs with all of their segments, in the state kernel and the read-out alike, so a
// segment sum is read by the XCD that wrote it.
__device__ __forceinline__ ItemCoords decode_item(uint32_t item, uint32_t H, uint32_t NVS, uint32_t G) {
  ItemCoords ic;
  ic.h = item % H;
  uint32_t r = item / H;
  ic.vs = r % NVS;
  r /= NVS;
  ic.g = r % G;
  ic.b = r / G;
  return ic;
}

__device__ __forceinline__ uint32_t default_item() {
  const uint32_t x = blockIdx.x;
  return (x & 7) * (gridDim.x >> 3) + (x >> 3);
}

// Segment order of the read-out blocks when each work item adds up its predecessors' sums (the start-up
// of segment g reads g sums). Blocks are dealt to the CUs of an XCD in order, one per CU first, so the two
// workgroups sharing a CU are the j-th and (j + n/2)-th of the XCD's n blocks: d = n / (2 H NVS) segment
// positions apart. Positions are taken in runs of 2d as [G-1-dk .. G-d-dk, dk .. dk+d-1], which puts
// segment g next to segment G-1-g: one of the two starts computing at once while the other reads, and the
// long start-up goes to the older workgroup, which the scheduler favours. A bijection on 0 .. G-1; the
// identity when the grid does not have that shape.
__device__ __forceinline__ uint32_t paired_segment(uint32_t pos, uint32_t items, uint32_t hn, uint32_t G) {
  const uint32_t n = items >> 3;
  if ((items & 7) != 0 || n % (2 * hn) != 0) return pos;
  const uint32_t d = n / (2 * hn);
  if (G % (2 * d) != 0) return pos;
  const uint32_t k = pos / (2 * d), i = pos % (2 * d);
  return i < d ? G - 1 - d * k - i : d * k + (i - d);
}

// Read-out item of this block; false for the padding blocks past the last item.
__device__ __forceinline__ bool readout_item(const Shape& sh, const Plan& pl, ItemCoords& ic) {
  const uint32_t H = static_cast<uint32_t>(sh.H), NVS = static_cast<uint32_t>(pl.nvs);
  const uint32_t G = static_cast<uint32_t>(pl.segments);
  const uint32_t pairs = static_cast<uint32_t>(sh.B) * H * NVS;
  if (pl.affine) {  // the grid is exactly pairs * G blocks
    const uint32_t x = blockIdx.x, ppx = pairs >> 3, j = x >> 3;
    const uint32_t pair = (x & 7) * ppx + j % ppx, s = j / ppx;
    ic.h = pair % H;
    ic.vs = (pair / H) % NVS;
    ic.b = pair / (H * NVS);
    // the CU pairing of segments as in paired_segment, with runs of one
    ic.g = (!pl.scanned && (G & 1) == 0) ? (s < G / 2 ? G - 1 - s : s - G / 2) : s;
    return true;
  }
  const uint32_t item = default_item();
  if (item >= pairs * G) return false;
  ic = decode_item(item, H, NVS, G);
  if (!pl.scanned) ic.g = paired_segment(static_cast<uint32_t>(ic.g), pairs * G, H * NVS, G);
  return true;
}

// State item of this block (64-column halves: pair p of the read-out is halves p * HALVES ..; ic.g numbers
// the pieces of pl.seg_len / pl.sub tokens); false for padding blocks.
template <int HALVES>
__device__ __forceinline__ bool state_item(const Shape& sh, const Plan& pl, ItemCoords& ic) {
  const uint32_t H = static_cast<uint32_t>(sh.H), NVS = static_cast<uint32_t>(pl.nvs);
  const uint32_t G1 = static_cast<uint32_t>(state_slots(pl));
  const uint32_t pairs = static_cast<uint32_t>(sh.B) * H * NVS;
  if (pl.affine) {  // the grid is exactly pairs * HALVES * G1 blocks
    const uint32_t x = blockIdx.x, ppx = (pairs >> 3) * HALVES, j = x >> 3;
    const uint32_t p = (x & 7) * ppx + j % ppx;
    const uint32_t pr = p / HALVES;
    ic.h = pr % H;
    ic.vs = (pr / H) % NVS * HALVES + p % HALVES;
    ic.b = pr / (H * NVS);
    ic.g = j / ppx;
    return true;
  }
  const uint32_t item = default_item();
  if (item >= pairs * HALVES * G1) return false;
  ic = decode_item(item, H, NVS * HALVES, G1);
  return true;
}

// ic.vs counts work items of VS columns.
template <int K, int VS>
__device__ __forceinline__ Rows make_rows(const u16* q, const u16* k, const u16* v, const Shape& sh,
                                          const ItemCoords& ic) {
  const int64_t bh_qk = (ic.b * sh.T * sh.H + ic.h) * K;
  const int64_t bh_v = (ic.b * sh.T * sh.H + ic.h) * sh.V + ic.vs * VS;
  Rows rw;
  rw.qk_stride = static_cast<unsigned>(sh.H * K * 2);
  rw.v_stride = static_cast<unsigned>(sh.H * sh.V * 2);
  rw.q = make_rsrc(q + bh_qk, sh.T, rw.qk_stride);
  rw.k = make_rsrc(k + bh_qk, sh.T, rw.qk_stride);
  rw.v = make_rsrc(v + bh_v, sh.T, rw.v_stride);
  return rw;
}

// ------------------------------------------------------------------ kernel 0: segment state sums

// The state sum of a segment is split over the W waves of the workgroup two ways: FW groups of feature
// tiles times KW = 2 groups of key steps. Wave w owns the feature tiles of group w / KW and the key steps
// of group w % KW of every chunk, so each wave reads only its own key steps' values from LDS; the KW partial
// sums of a feature group are added at the end of the segment. The state kernel always works on 64 value
// columns (SC); with 128-column read-out items it writes each half into the item's slot. K = 16: 4 x 2
// waves, feature groups of 3, 3, 2 and 2 tiles (with 2 x 2 waves of 5 tiles, the accumulators alone took
// 100 registers and a segment item ran 4 waves, too few to keep a CU busy: 1.75 waves per SIMD on the
// benchmark shapes); K = 8: 1 x 2 waves of 3 tiles. Each wave takes half the chunk's key steps.
template <class Cf>
struct StateSplit {
  static constexpr bool K16 = Cf::K == 16;
  static constexpr int KW = 2;
  static constexpr int FW = K16 ? 4 : 1;
  static constexpr int W = FW * KW;
  __host__ __device__ static constexpr int T0(int fg) { return K16 ? (fg < 2 ? 3 * fg : 6 + 2 * (fg - 2)) : 0; }
  __host__ __device__ static constexpr int NT(int fg) { return K16 ? (fg < 2 ? 3 : 2) : 3; }
  static constexpr int NT_MAX = 3;  // the largest feature group (both splits)
  static constexpr int KS = Split<Cf>::NKS / KW;  // key steps per wave and chunk
  // Chunks loaded ahead of the one being worked on: with K = 8 there is less work per chunk to cover the
  // latency of the loads (measured: 3 sets are 18% faster than 1 at K = 8, V = 128; no change at K = 16).
  static constexpr int PREFETCH = Cf::K == 8 ? 3 : 1;
  static_assert(T0(FW - 1) + NT(FW - 1) == Feat<Cf::K>::NPT && KS * KW == Split<Cf>::NKS, "even split");
};

template <class Cf>
struct __align__(16) StateSmem {
  union {
    Stage<Cf> stage[2];
    f32x4_t red[StateSplit<Cf>::FW][StateSplit<Cf>::NT_MAX][Cf::NVT][kWave];  // partial sums of key-step group 1
  };
};

// half: which 64 columns of the slot's IVS columns this work item covers (the ones tile goes with half 0).
template <class SC, int IVS, int WI>
__device__ __forceinline__ void segment_state_body(StateSmem<SC>& sm, const Rows& rw, int64_t T, int64_t t_begin,
                                                   int64_t t_end, int half, char* __restrict__ dst) {
  using SP = Split<SC>;
  using SS = StateSplit<SC>;
  constexpr int K = SC::K;
  constexpr int FG = WI / SS::KW, KG = WI % SS::KW;
  constexpr int T0 = SS::T0(FG), NT = SS::NT(FG);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int c = lane & 15;
  f32x4_t S[NT][SC::NVT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int vt = 0; vt < SC::NVT; ++vt) S[t][vt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // The loop does little work per chunk next to the latency of a global load, so the inputs are loaded
  // D = SS::PREFETCH chunks ahead into as many register sets (two LDS stages as in the read-out): chunk
  // c + 1 is staged at the end of iteration c from the set loaded D - 1 iterations before, and that set is
  // then refilled with chunk c + 1 + D. Loads past the segment read the
  // next segment's rows (or, past the sequence, nothing) and are never used.
  constexpr int D = SS::PREFETCH;
  Prefetch<SC, false, WI, SS::W> pf[D];
  pf[0].init(rw, lane);
#pragma unroll
  for (int d = 1; d < D; ++d) pf[d] = pf[0];
  auto at = [&](int64_t t) { return t < t_end ? t : T; };  // past the sequence: no traffic
  pf[0].load(rw, t_begin);
  pf[0].store(sm.stage[0], lane);
#pragma unroll
  for (int d = 0; d < D; ++d) pf[d].load(rw, at(t_begin + (d + 1) * SP::C));
  int it = 0;
  int64_t t0 = t_begin;
  bool more = true;
  while (more) {
    constexpr_for<0, D>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      if (!more) return;
      const Stage<SC>& st = sm.stage[it & 1];
      __syncthreads();
#pragma unroll
      for (int j = 0; j < SS::KS; ++j) {
        const int ks = KG * SS::KS + j;
        u32x4_t vop[SC::NVT];
        load_value_operands<SC>(st, ks, lane, vop);
        float kx[8];
        key_column<SC>(st, ks, lane, kx);
        state_update_step<SC, T0, NT>(S, kx, vop, c);
      }
      pf[d].store(sm.stage[(it + 1) & 1], lane);  // read in iteration c - 1, finished before this iteration's barrier
      pf[d].load(rw, at(t0 + (D + 1) * SP::C));
      t0 += SP::C;
      ++it;
      more = t0 < t_end;
    });
  }
  __syncthreads();  // the stages are free: their memory holds the partial sums now
  if constexpr (KG == 1) {
#pragma unroll
    for (int lt = 0; lt < NT; ++lt)
#pragma unroll
      for (int vt = 0; vt < SC::NVT; ++vt) sm.red[FG][lt][vt][lane] = S[lt][vt];
  }
  __syncthreads();
  if constexpr (KG == 0) {
#pragma unroll
    for (int lt = 0; lt < NT; ++lt)
#pragma unroll
      for (int vt = 0; vt < SC::NVT; ++vt) S[lt][vt] += sm.red[FG][lt][vt][lane];
#pragma unroll
    for (int lt = 0; lt < NT; ++lt)
#pragma unroll
      for (int vt = 0; vt < SC::NVV; ++vt) {
        char* d = dst + state_offset<K, IVS>(T0 + lt, SC::NVV * half + vt, lane);
        if constexpr (kBf16Slot<K, IVS>)
          *reinterpret_cast<u32x2_t*>(d) = to_bf16x4(S[lt][vt]);
        else
          *reinterpret_cast<f32x4_t*>(d) = S[lt][vt];
      }
    if (half == 0 && c == 0) {
#pragma unroll
      for (int lt = 0; lt < NT; ++lt)
        *reinterpret_cast<f32x4_t*>(dst + ones_offset<K, IVS>(T0 + lt, lane >> 4)) = S[lt][SC::ONES];
    }
  }
}

// Work items of 64 columns (pl.nvs * IVS / 64 per (b, h)); the slot belongs to the read-out item of IVS columns that
// contains them.
template <int K, int IVS>
__global__ __launch_bounds__((StateSplit<Cfg<K, 64>>::W * kWave), 2) void based_segment_state_kernel(
    const u16* __restrict__ k, const u16* __restrict__ v, Shape sh, Plan pl, float* __restrict__ ws) {
  using SC = Cfg<K, 64>;
  constexpr int HALVES = IVS / 64;
  ItemCoords ic;
  if (!state_item<HALVES>(sh, pl, ic)) return;
  __shared__ StateSmem<SC> sm;
  const Rows rw = make_rows<K, 64>(k, k, v, sh, ic);
  const int64_t len = pl.seg_len / pl.sub;
  const int64_t t_begin = ic.g * len;
  const int64_t t_end = t_begin + len;  // a whole piece: only the last segment, which has none, can be short
  const int64_t bhv = (ic.b * sh.H + ic.h) * pl.nvs + ic.vs / HALVES;
  const int half = static_cast<int>(ic.vs % HALVES);
  char* dst = reinterpret_cast<char*>(ws + (bhv * state_slots(pl) + ic.g) * pl.slot_floats);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr_for<0, StateSplit<SC>::W>([&](auto wc) {
    constexpr int WI = decltype(wc)::value;
    if (w == WI) segment_state_body<SC, IVS, WI>(sm, rw, sh.T, t_begin, t_end, half, dst);
  });
}

// ------------------------------------------------------------- kernel 1: prefix over segments

// Used when there are too many state sums for each read-out to add up its predecessors' sums: in place,
// slot s of every (b, h, work item columns) becomes the sum of the state sums 0..s. One thread per group
// of four consecutive state entries: the first `bf16_groups` groups of a slot are bf16 value-tile entries (8
// bytes), the rest fp32 ones-tile entries (16 bytes); the running sum is kept in fp32 and each prefix is
// rounded once. Slots are read in batches ahead of the running sum so that the loads of a batch do not wait
// for the stores of the previous one; with up to 32 slots every load is issued before the first add.
constexpr int kScanThreads = 256;

template <typename U, typename Load, typename Store>
__device__ __forceinline__ void scan_slots(char* p, int64_t slot_bytes, int64_t slots, Load ld, Store st) {
  constexpr int kBatch = 16;
  auto at = [&](int64_t s) { return reinterpret_cast<U*>(p + s * slot_bytes); };
  // The batches stay in their stored form until they are added, so that the next batch's loads are still
  // in flight while this batch is summed and stored.
  const U zero = {};
  U cur[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) cur[j] = j < slots ? *at(j) : zero;
  f32x4_t run = {0.f, 0.f, 0.f, 0.f};
  for (int64_t s0 = 0; s0 < slots; s0 += kBatch) {
    U nxt[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) nxt[j] = s0 + kBatch + j < slots ? *at(s0 + kBatch + j) : zero;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (s0 + j < slots) {
        run += ld(cur[j]);
        *at(s0 + j) = st(run);
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) cur[j] = nxt[j];
  }
}

__global__ __launch_bounds__(kScanThreads) void based_segment_scan_kernel(float* __restrict__ ws, int64_t n_bhv,
                                                                 int64_t slots, int64_t slot_floats,
                                                                 int64_t bf16_groups) {
  const int64_t groups = bf16_groups + (slot_floats - 2 * bf16_groups) / 4;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kScanThreads + threadIdx.x;
  if (idx >= n_bhv * groups) return;
  const int64_t bhv = idx / groups;
  const int64_t e = idx - bhv * groups;
  const int64_t slot_bytes = slot_floats * 4;
  char* base = reinterpret_cast<char*>(ws + bhv * slots * slot_floats);
  if (e < bf16_groups) {
    scan_slots<u32x2_t>(base + e * 8, slot_bytes, slots, [](const u32x2_t& u) { return from_bf16x4(u); },
                        [](const f32x4_t& x) { return to_bf16x4(x); });
  } else {
    scan_slots<f32x4_t>(base + bf16_groups * 8 + (e - bf16_groups) * 16, slot_bytes, slots,
                        [](const f32x4_t& x) { return x; }, [](const f32x4_t& x) { return x; });
  }
}

// ------------------------------------------------------------------- kernel 2: chunked read-out

// With 64-column items the bf16 state is double-buffered (chunk c reads buffer c % 2, the state after
// chunk c is published into the other one), which leaves one barrier per chunk. With 128 columns one
// buffer is kept (with K = 16 a second one would not fit next to two 128-token stages) and the waves meet
// once more before the state is overwritten.
template <class Cf>
struct __align__(16) ReadoutSmem {
  static constexpr int NP = (Feat<Cf::K>::NPT + 1) / 2;  // tile pairs of the read-out contraction
  static constexpr int NSB = Cf::VS == 64 ? 2 : 1;
  Stage<Cf> stage[2];                  // chunk c in stage[c % 2]; chunk c + 1 is staged during chunk c
  u32x4_t sb[NSB][NP][Cf::NVT][kWave];  // bf16 state: buffer, tile pair m, value tile, lane (D layout)
};

// bf16 copy of this wave's state tiles into the shared tile-pair layout of buffer b.
template <class Cf, int T0, int NT, typename SA>
__device__ __forceinline__ void publish_state(ReadoutSmem<Cf>& sm, int b, const SA& S, int lane) {
#pragma unroll
  for (int lt = 0; lt < NT; ++lt) {
    const int t = T0 + lt;
#pragma unroll
    for (int vt = 0; vt < Cf::NVT; ++vt) {
      u32x2_t* d = reinterpret_cast<u32x2_t*>(&sm.sb[b][t >> 1][vt][lane]) + (t & 1);
      *d = u32x2_t{pack2(S[lt][vt][0], S[lt][vt][1]), pack2(S[lt][vt][2], S[lt][vt][3])};
    }
  }
}

// Intra-chunk contribution of key step ks (key tokens 32 ks .. 32 ks + 31) to 16-token query tile II:
// scores K Q^T on the 16x16x16 MFMA, Taylor weights, then the transposed product [V | 1]^T A^T, so
// that the output tile comes out with the token along the lanes.
template <class Cf, int II>
__device__ __forceinline__ void intra_step(const Stage<Cf>& st, int ks, const u32x4_t (&vop)[Cf::NVT],
                                           f32x4_t (&O)[Cf::NVT], float c1, float c2, int lane) {
  constexpr int K = Cf::K;
  if (2 * ks > II) return;
  const int c = lane & 15, g = lane >> 4;
  u32x2_t qb = {0u, 0u};
  if (K == 16 || g < 2) qb = *reinterpret_cast<const u32x2_t*>(st.q + (16 * II + c) * K + 4 * g);
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t d[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int jj = 2 * ks + h;
    d[h] = zero4;
    if (jj <= II) {
      u32x2_t ka = {0u, 0u};
      if (K == 16 || g < 2) ka = *reinterpret_cast<const u32x2_t*>(st.k + (16 * jj + c) * K + 4 * g);
      d[h] = mfma16(ka, qb, zero4);
    }
  }
  // B operand: slot e <-> key token 32 ks + 16(e/4) + 4g + e%4, column (query) 16 II + c.
  float w[8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int jj = 2 * ks + h;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float a = 0.0f;
      if (jj <= II) {
        const float sc = d[h][r];
        a = fmaf(sc, fmaf(sc, c2, c1), 1.0f);
        if (jj == II) a = (4 * g + r <= c) ? a : 0.0f;
      }
      w[4 * h + r] = a;
    }
  }
  const u32x4_t aop = {pack2(w[0], w[1]), pack2(w[2], w[3]), pack2(w[4], w[5]), pack2(w[6], w[7])};
#pragma unroll
  for (int vt = 0; vt < Cf::NVT; ++vt) O[vt] = mfma32(vop[vt], aop, O[vt]);
}

// o = num / (den + 1e-6) for one 16-token query tile held transposed: lane (c, g) has token c of the
// tile and value columns 16 vt + 4 g .. 16 vt + 4 g + 3, so each value tile is one 8-byte (bf16) or
// 16-byte (fp32) store per lane; the ones tile holds den in all four rows. voff is the lane's byte
// offset of (token c, column 4 g), soff the tile's first token. Rows past the end of the sequence fall
// outside the output buffer range and are dropped. A store of more than 8 bytes reads its data registers
// after it issues; the compiler keeps a later write of them far enough behind only when the store's
// scalar offset is a constant, so the 16-byte fp32 stores carry the whole offset in the vector offset.
template <class Cf, bool OUT_F32>
__device__ __forceinline__ void store_tile(__amdgpu_buffer_rsrc_t ro, unsigned voff, unsigned soff,
                                           const f32x4_t (&O)[Cf::NVT]) {
  const float inv = __builtin_amdgcn_rcpf(O[Cf::ONES][0] + 1e-6f);
#pragma unroll
  for (int vt = 0; vt < Cf::NVV; ++vt) {
    if constexpr (OUT_F32) {
      const f32x4_t o = O[vt] * inv;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, o), ro, voff + soff + 64 * vt, 0, 0);
    } else {
      const u32x2_t o = {pack2(O[vt][0] * inv, O[vt][1] * inv), pack2(O[vt][2] * inv, O[vt][3] * inv)};
      __builtin_amdgcn_raw_buffer_store_b64(o, ro, voff, soff + 32 * vt, 0);
    }
  }
}

// bf16 output tile II of wave WI written as whole rows, in two steps. The tile (16 tokens, VS columns)
// first goes into LDS, into 1 KiB blocks of the idle stage that this wave alone refills with the next
// chunk at the end of the iteration: wave WI's prefetch units WI * 64 + i * 64 W .. + 63 occupy bytes
// 1024 (WI + W i) .. + 1023 of a stage, and no wave reads that stage before the next barrier, so no barrier
// is needed (a wave's own LDS accesses are carried out in order). A block holds RB = 1024 / (2 VS) rows of
// the tile; the 16-byte unit u of tile row r sits at unit position u ^ (r % UPR), which spreads the 8-byte
// writes of one value tile over all banks (in plain row order they fell on a quarter of them, and the
// read-out was 20% slower). Later, once the registers of the chunk's contraction are free, the rows are
// read back as UPR 16-byte units each and stored with one 128-bit store per lane, so every store
// instruction covers RB whole rows of the output (32 bytes of each of 16 rows in the register layout
// otherwise).
template <class Cf, int WI, int II>
struct TileRows {
  static constexpr int W = Split<Cf>::W;
  static constexpr int VS = Cf::VS;
  static constexpr int UPR = VS / 8;          // 16-byte units per row
  static constexpr int RB = 1024 / (2 * VS);  // rows per 1 KiB block
  static constexpr int NB = 16 / RB;          // blocks per tile
  static_assert((WI + W * (NB * (II + 1) - 1)) * 64 < Units<Cf>::NU, "the tile's blocks lie inside the wave's prefetch units");
  __device__ static __forceinline__ unsigned char* block(unsigned char* idle_stage, int j) {
    return idle_stage + 1024 * (WI + W * (NB * II + j));
  }
  // o = num / (den + 1e-6) as bf16 into the blocks.
  __device__ static __forceinline__ void stage(unsigned char* idle_stage, const f32x4_t (&O)[Cf::NVT], int lane) {
    const int c = lane & 15, g = lane >> 4;
    const float inv = __builtin_amdgcn_rcpf(O[Cf::ONES][0] + 1e-6f);
    unsigned char* rowp = block(idle_stage, c / RB) + (c % RB) * (2 * VS) + 8 * (g & 1);
#pragma unroll
    for (int vt = 0; vt < Cf::NVV; ++vt) {
      const u32x2_t o = {pack2(O[vt][0] * inv, O[vt][1] * inv), pack2(O[vt][2] * inv, O[vt][3] * inv)};
      const int u = 2 * vt + (g >> 1);
      *reinterpret_cast<u32x2_t*>(rowp + 16 * (u ^ (c & (UPR - 1)))) = o;
    }
  }
  // The rows to the output; soff is the byte offset of the tile's first token. As for every store of more
  // than 8 bytes, the whole offset goes in the vector offset (the scalar offset is the constant 0).
  __device__ static __forceinline__ void store(unsigned char* idle_stage, __amdgpu_buffer_rsrc_t ro,
                                               unsigned out_stride, unsigned soff, int lane) {
    const int r = lane / UPR, p = lane % UPR;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int row = j * RB + r;
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(block(idle_stage, j) + r * (2 * VS) + 16 * (p ^ (row & (UPR - 1))));
      __builtin_amdgcn_raw_buffer_store_b128(x, ro, r * out_stride + 16 * p + soff + j * RB * out_stride, 0, 0);
    }
  }
};

// The state at the start of a segment: the sum, in segment order, of the state sums of the `n_src`
// earlier segments stored at src, src + slot_floats, ...
template <class Cf, int T0, int NT, typename SA>
__device__ __forceinline__ void initial_state(SA& S, const float* __restrict__ src, int64_t n_src, int64_t slot_floats,
                                              int lane) {
  const int g = lane >> 4;
#pragma unroll
  for (int lt = 0; lt < NT; ++lt)
#pragma unroll
    for (int vt = 0; vt < Cf::NVT; ++vt) S[lt][vt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (kBf16Slot<Cf::K, Cf::VS>) {
    // Two slots are loaded before either is added (the additions keep the segment order); the value tiles
    // stay packed bf16 until they are added.
    struct Slot {
      u32x2_t v[NT > 0 ? NT : 1][Cf::NVV];
      f32x4_t z[NT > 0 ? NT : 1];
    };
    auto load = [&](Slot& x, int64_t i) {
      const char* s = reinterpret_cast<const char*>(src + i * slot_floats);
#pragma unroll
      for (int lt = 0; lt < NT; ++lt) {
#pragma unroll
        for (int vt = 0; vt < Cf::NVV; ++vt)
          x.v[lt][vt] = *reinterpret_cast<const u32x2_t*>(s + state_offset<Cf::K, Cf::VS>(T0 + lt, vt, lane));
        x.z[lt] = *reinterpret_cast<const f32x4_t*>(s + ones_offset<Cf::K, Cf::VS>(T0 + lt, g));
      }
    };
    auto add = [&](const Slot& x) {
#pragma unroll
      for (int lt = 0; lt < NT; ++lt) {
#pragma unroll
        for (int vt = 0; vt < Cf::NVV; ++vt) S[lt][vt] += from_bf16x4(x.v[lt][vt]);
        S[lt][Cf::ONES] += x.z[lt];
      }
    };
    int64_t i = 0;
    for (; i + 1 < n_src; i += 2) {
      Slot x0, x1;
      load(x0, i);
      load(x1, i + 1);
      add(x0);
      add(x1);
    }
    if (i < n_src) {
      Slot x0;
      load(x0, i);
      add(x0);
    }
  } else {
    // fp32 slots; two are loaded before either is added (the additions keep the segment order).
    auto load = [&](f32x4_t (&x)[NT > 0 ? NT : 1][Cf::NVT], int64_t i) {
      const char* s = reinterpret_cast<const char*>(src + i * slot_floats);
#pragma unroll
      for (int lt = 0; lt < NT; ++lt) {
#pragma unroll
        for (int vt = 0; vt < Cf::NVV; ++vt)
          x[lt][vt] = *reinterpret_cast<const f32x4_t*>(s + state_offset<Cf::K, Cf::VS>(T0 + lt, vt, lane));
        x[lt][Cf::ONES] = *reinterpret_cast<const f32x4_t*>(s + ones_offset<Cf::K, Cf::VS>(T0 + lt, g));
      }
    };
    auto add = [&](const f32x4_t (&x)[NT > 0 ? NT : 1][Cf::NVT]) {
#pragma unroll
      for (int lt = 0; lt < NT; ++lt)
#pragma unroll
        for (int vt = 0; vt < Cf::NVT; ++vt) S[lt][vt] += x[lt][vt];
    };
    int64_t i = 0;
    for (; i + 1 < n_src; i += 2) {
      f32x4_t x0[NT > 0 ? NT : 1][Cf::NVT], x1[NT > 0 ? NT : 1][Cf::NVT];
      load(x0, i);
      load(x1, i + 1);
      add(x0);
      add(x1);
    }
    if (i < n_src) {
      f32x4_t x0[NT > 0 ? NT : 1][Cf::NVT];
      load(x0, i);
      add(x0);
    }
  }
}

// A state in the page's layout for one (b, h) and work item: entry (row r, item column j) of S at
// s[r * V + j], of z at z[r]. Import when s_in is set, export (of the state after the last token) when
// s_out is set; write_z selects the one work item of the (b, h) that writes z.
struct StateView {
  const float* s_in;
  const float* z_in;
  float* s_out;
  float* z_out;
  int64_t V;
  bool write_z;
};

template <class Cf, int T0, int NT, typename SA>
__device__ __forceinline__ void import_state(SA& S, const StateView& sv, int lane) {
  constexpr int K = Cf::K;
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int lt = 0; lt < NT; ++lt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const FeatRows fr = feat_rows<K>(T0 + lt, 4 * g + r);
#pragma unroll
      for (int vt = 0; vt < Cf::NVV; ++vt) {
        const float* col = sv.s_in + 16 * vt + c;
        S[lt][vt][r] += import_feature<K>(fr, [&](int row) { return col[row * sv.V]; });
      }
      S[lt][Cf::ONES][r] += import_feature<K>(fr, [&](int row) { return sv.z_in[row]; });
    }
  }
}

// The padding tokens of a ragged last chunk (k = v = 0, so phi(k) = [1, 0, ...]) added `n_pad` to the
// constant feature of z and nothing else; the exported z leaves them out.
template <class Cf, int T0, int NT, typename SA>
__device__ __forceinline__ void export_state(const SA& S, const StateView& sv, float n_pad, int lane) {
  constexpr int K = Cf::K;
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int lt = 0; lt < NT; ++lt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const FeatRows fr = feat_rows<K>(T0 + lt, 4 * g + r);
#pragma unroll
      for (int vt = 0; vt < Cf::NVV; ++vt) {
        float* col = sv.s_out + 16 * vt + c;
        export_feature<K>(fr, S[lt][vt][r], [&](int row, float x) { col[row * sv.V] = x; });
      }
      if (sv.write_z && c == 0) {
        const float zv = fr.kind == kFeatConst ? S[lt][Cf::ONES][r] - n_pad : S[lt][Cf::ONES][r];
        export_feature<K>(fr, zv, [&](int row, float x) { sv.z_out[row] = x; });
      }
    }
  }
}

template <class Cf, int WI, bool OUT_F32, bool ROWS>
__device__ __forceinline__ void readout_body(ReadoutSmem<Cf>& sm, const Rows& rw, __amdgpu_buffer_rsrc_t ro,
                                             unsigned out_stride, int64_t T, int64_t t_begin, int64_t t_end,
                                             float c1, float c2, float sigma, const float* __restrict__ src,
                                             int64_t n_src, int64_t slot_floats, const StateView& sv) {
  constexpr int K = Cf::K;
  constexpr int NVT = Cf::NVT;
  // Whole-row output stores exist for bf16 output; K = 16 with 128 columns has no registers to spare for them.
  static_assert(!ROWS || (!OUT_F32 && !(K == 16 && Cf::VS == 128)), "no whole-row stores for this read-out");
  using F = Feat<K>;
  using SP = Split<Cf>;
  constexpr int T0 = SP::T0(WI), NT = SP::NT(WI);
  constexpr int QPW = SP::QPW;  // this wave's query tiles: SP::Q(WI, 0 .. QPW - 1)
  constexpr int NP = (F::NPT + 1) / 2;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int c = lane & 15, g = lane >> 4;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const float sigma2 = 2.0f * c2;  // scale^2 (c2 = scale^2 / 2)
  constexpr unsigned kOutBytes = OUT_F32 ? 4 : 2;
  const unsigned lane_off = c * out_stride + 4 * g * kOutBytes;

  f32x4_t S[NT > 0 ? NT : 1][NVT];
  initial_state<Cf, T0, NT>(S, src, n_src, slot_floats, lane);
  if (sv.s_in) import_state<Cf, T0, NT>(S, sv, lane);
  constexpr int NSB = ReadoutSmem<Cf>::NSB;
  publish_state<Cf, T0, NT>(sm, 0, S, lane);
  if constexpr (F::NPT % 2 == 1 && T0 + NT == F::NPT && NT > 0) {
    // The last tile pair is half empty: its second half stays zero for the whole kernel.
#pragma unroll
    for (int b = 0; b < NSB; ++b)
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt)
        reinterpret_cast<u32x2_t*>(&sm.sb[b][F::NPT >> 1][vt][lane])[1] = u32x2_t{0u, 0u};
  }

  // Chunk c is read from stage[c % 2]. Chunk c + 1 is loaded into registers at the top of iteration c
  // and written to stage[(c + 1) % 2] at its end, so the loads have the whole iteration to arrive and
  // no load result is pending across the loop's back edge (which would make the memory-counter wait
  // at the top cover this chunk's output stores too). Loads past the segment read the next segment's
  // (or out-of-range, zero) rows and are never used.
  Prefetch<Cf, true, WI> pf;
  pf.init(rw, lane);
  pf.load(rw, t_begin);
  pf.store(sm.stage[0], lane);
  int it = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += SP::C, ++it) {
    // After the segment's last chunk the loads are aimed past the end of the buffer range: they return
    // zeros without touching memory.
    pf.load(rw, t0 + SP::C < t_end ? t0 + SP::C : T);
    __syncthreads();  // this chunk's inputs and the bf16 state of earlier chunks are in LDS
    const Stage<Cf>& st = sm.stage[it & 1];

    // ---- read-out of earlier tokens through the state, transposed: O^T = S^T phi(Q)^T for this wave's
    //      query tiles (the bf16 state tiles are the A operand, phi(Q) the B operand).
    f32x4_t O[QPW][NVT];
    {
      float qu[QPW][F::NQ], qa[QPW][4], qh[QPW][4], ql[QPW][4];
      u32x2_t qraw[QPW][F::NQ / 4];  // all reads first, so that their latencies overlap
      constexpr_for<0, QPW>([&](auto ic) {
        constexpr int ii = decltype(ic)::value;
        const u16* qrow = st.q + (16 * SP::Q(WI, ii) + c) * K;
#pragma unroll
        for (int kk = 0; kk < F::NQ / 4; ++kk)
          qraw[ii][kk] = *reinterpret_cast<const u32x2_t*>(qrow + 4 * ((g + kk) & (F::NQ / 4 - 1)));
      });
#pragma unroll
      for (int ii = 0; ii < QPW; ++ii) {
#pragma unroll
        for (int kk = 0; kk < F::NQ / 4; ++kk) {
          const u32x2_t w2 = qraw[ii][kk];
          qu[ii][4 * kk + 0] = lo_f(w2.x);
          qu[ii][4 * kk + 1] = hi_f(w2.x);
          qu[ii][4 * kk + 2] = lo_f(w2.y);
          qu[ii][4 * kk + 3] = hi_f(w2.y);
        }
      }
#pragma unroll
      for (int ii = 0; ii < QPW; ++ii) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          qa[ii][r] = sigma2 * qu[ii][r];
          qh[ii][r] = c2 * qu[ii][r];
          ql[ii][r] = sigma * qu[ii][r];
        }
      }
      constexpr_for<0, NP>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        constexpr int ta = 2 * m, tb = 2 * m + 1;
        u32x4_t sb[NVT];
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) sb[vt] = sm.sb[NSB == 2 ? (it & 1) : 0][m][vt][lane];
#pragma unroll
        for (int ii = 0; ii < QPW; ++ii) {
          const QSide y{qu[ii], qa[ii], qh[ii], ql[ii]};
          u32x4_t pq;
          pq.x = pack2(F::template qval<ta, 0>(y, g), F::template qval<ta, 1>(y, g));
          pq.y = pack2(F::template qval<ta, 2>(y, g), F::template qval<ta, 3>(y, g));
          pq.z = pack2(F::template qval<tb, 0>(y, g), F::template qval<tb, 1>(y, g));
          pq.w = pack2(F::template qval<tb, 2>(y, g), F::template qval<tb, 3>(y, g));
#pragma unroll
          for (int vt = 0; vt < NVT; ++vt) O[ii][vt] = mfma32(sb[vt], pq, m == 0 ? zero4 : O[ii][vt]);
        }
      });
    }

    // ---- per 32-token key step: intra-chunk term (direct polynomial) for the query tiles, then fold
    //      the step into this wave's state tiles (after the last chunk the result is unused).
    const unsigned soff_out = static_cast<unsigned>(t0) * out_stride;
    unsigned char* idle = reinterpret_cast<unsigned char*>(&sm.stage[(it + 1) & 1]);
#pragma unroll
    for (int ks = 0; ks < SP::NKS; ++ks) {
      u32x4_t vop[NVT];
      load_value_operands<Cf>(st, ks, lane, vop);
      constexpr_for<0, QPW>([&](auto ic) {
        constexpr int ii = decltype(ic)::value;
        intra_step<Cf, SP::Q(WI, ii)>(st, ks, vop, O[ii], c1, c2, lane);
        if (ks == SP::NKS - 1) {
          if constexpr (ROWS)
            TileRows<Cf, WI, ii>::stage(idle, O[ii], lane);
          else
            store_tile<Cf, OUT_F32>(ro, lane_off, soff_out + 16 * SP::Q(WI, ii) * out_stride, O[ii]);
        }
      });
      if constexpr (NT > 0) {
        float kx[8];
        key_column<Cf>(st, ks, lane, kx);
        state_update_step<Cf, T0, NT>(S, kx, vop, c);
      }
    }
    if constexpr (ROWS) {
      constexpr_for<0, QPW>([&](auto ic) {
        constexpr int ii = decltype(ic)::value;
        TileRows<Cf, WI, ii>::store(idle, ro, out_stride, soff_out + 16 * SP::Q(WI, ii) * out_stride, lane);
      });
    }
    // The state after this chunk goes into the buffer that chunk c - 1 read (every wave finished that
    // chunk before this chunk's barrier); with a single buffer the waves first wait for each other.
    if constexpr (NSB == 1) __syncthreads();
    publish_state<Cf, T0, NT>(sm, NSB == 2 ? ((it + 1) & 1) : 0, S, lane);
    pf.store(sm.stage[(it + 1) & 1], lane);  // that buffer's chunk c - 1 was finished before the last barrier
  }
  if (sv.s_out && t_end == T) {
    const int64_t n = t_end - t_begin;
    export_state<Cf, T0, NT>(S, sv, static_cast<float>((n + SP::C - 1) / SP::C * SP::C - n), lane);
  }
}


template <int K, int VS, bool OUT_F32, bool ROWS>
__global__ __launch_bounds__((Split<Cfg<K, VS>>::W * kWave)) void based_chunk_readout_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v, Shape sh, Plan pl, float c1,
    float c2, float sigma, const float* __restrict__ ws, void* __restrict__ out, StateIO io) {
  using Cf = Cfg<K, VS>;
  ItemCoords ic;
  if (!readout_item(sh, pl, ic)) return;
  __shared__ ReadoutSmem<Cf> sm;
  const Rows rw = make_rows<K, VS>(q, k, v, sh, ic);
  const int64_t bh_v = (ic.b * sh.T * sh.H + ic.h) * sh.V + ic.vs * VS;
  const unsigned out_stride = static_cast<unsigned>(sh.H * sh.V * (OUT_F32 ? 4 : 2));
  const __amdgpu_buffer_rsrc_t ro =
      make_rsrc(static_cast<char*>(out) + bh_v * (OUT_F32 ? 4 : 2), sh.T, out_stride);
  const int64_t t_begin = ic.g * pl.seg_len;
  const int64_t t_end = (t_begin + pl.seg_len < sh.T) ? t_begin + pl.seg_len : sh.T;
  // Initial state: the sum of the state sums of the pieces of segments 0 .. g - 1 (g * sub of them), or after
  // the prefix scan the single slot g * sub - 1 that already holds it.
  const int64_t bhv = (ic.b * sh.H + ic.h) * pl.nvs + ic.vs;
  const float* src = ws + bhv * state_slots(pl) * pl.slot_floats;
  int64_t n_src = ic.g * pl.sub;
  if (pl.scanned && ic.g > 0) {
    src += (ic.g * pl.sub - 1) * pl.slot_floats;
    n_src = 1;
  }
  StateView sv;
  const int64_t P = 1 + K + K * K;
  const int64_t bh = ic.b * sh.H + ic.h;
  sv.s_in = io.s_in ? io.s_in + bh * P * sh.V + ic.vs * VS : nullptr;
  sv.z_in = io.z_in ? io.z_in + bh * P : nullptr;
  sv.s_out = io.s_out ? io.s_out + bh * P * sh.V + ic.vs * VS : nullptr;
  sv.z_out = io.z_out ? io.z_out + bh * P : nullptr;
  sv.V = sh.V;
  sv.write_z = ic.vs == 0;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr_for<0, Split<Cf>::W>([&](auto wc) {
    constexpr int WI = decltype(wc)::value;
    if (w == WI)
      readout_body<Cf, WI, OUT_F32, ROWS>(sm, rw, ro, out_stride, sh.T, t_begin, t_end, c1, c2, sigma, src, n_src,
                                          pl.slot_floats, sv);
  });
}

// -------------------------------------------------------------- kernel 3: one-token recurrent step

// phi of the page (field spec_md), row r of P = 1 + K + K^2: 1, x_{r-1}, or x_a x_b / sqrt(2).
template <int K>
__device__ __forceinline__ float phi_row(const float* x, int r) {
  if (r == 0) return 1.0f;
  if (r <= K) return x[r - 1];
  const int i = r - 1 - K;
  return x[i / K] * x[i % K] * kRSqrt2;
}

// Sum of a float over the 64 lanes of a wave (every lane gets the total).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
  return x;
}

// One workgroup of NT threads per (b, h): S += phi(k) v^T and z += phi(k) in place (the page's layout,
// fp32), then o = phi(scale q) S / (phi(scale q) z + 1e-6). Memory-bound: every state entry is read and
// written once. A block of 64 value columns is 16 lanes of 16-byte accesses per state row; the NT / 16
// row groups take every (NT / 16)-th row. A workgroup's memory latencies overlap: the first block's state
// rows, its value columns and the normaliser entries are requested before anything waits, and each
// further block is requested before the barrier that ends the one before. Partial numerators meet in LDS
// (two buffers, one barrier per column block).
template <int K, int NT>
__global__ __launch_bounds__(NT) void based_decode_step_kernel(const u16* __restrict__ q, const u16* __restrict__ k,
                                                               const u16* __restrict__ v, int64_t V, float sigma,
                                                               float* __restrict__ S, float* __restrict__ z,
                                                               void* __restrict__ out, bool out_f32) {
  constexpr int P = 1 + K + K * K;
  constexpr int RG = NT / 16;             // row groups
  constexpr int NR = (P + RG - 1) / RG;   // rows per thread
  constexpr int NW = NT / kWave;
  constexpr int NZ = (P + NT - 1) / NT;   // normaliser entries per thread
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int cq = tid & 15, rg = tid >> 4;
  __shared__ float sq[K], sk[K], part_den[NW];
  __shared__ f32x4_t part[2][RG][16];
  float* Sb = S + bh * P * V;
  float* zb = z + bh * P;
  const u16* vb = v + bh * V;
  f32x4_t s[NR];
  uint2 vr;
  auto request = [&](int64_t c0) {
    const int64_t col = c0 + 4 * cq;
    vr = *reinterpret_cast<const uint2*>(vb + col);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int r = rg + RG * i;
      if (r < P) s[i] = *reinterpret_cast<const f32x4_t*>(Sb + r * V + col);
    }
  };
  request(0);
  float zr[NZ];
#pragma unroll
  for (int j = 0; j < NZ; ++j) zr[j] = tid + j * NT < P ? zb[tid + j * NT] : 0.0f;
  if (tid < K) {
    sq[tid] = sigma * lo_f(q[bh * K + tid]);
    sk[tid] = lo_f(k[bh * K + tid]);
  }
  __syncthreads();
  float dp = 0.0f;
#pragma unroll
  for (int j = 0; j < NZ; ++j) {
    const int r = tid + j * NT;
    if (r < P) {
      const float nz = zr[j] + phi_row<K>(sk, r);
      zb[r] = nz;
      dp += phi_row<K>(sq, r) * nz;
    }
  }
  dp = wave_sum(dp);
  if ((tid & (kWave - 1)) == 0) part_den[tid / kWave] = dp;
  float pk[NR], pq[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int r = rg + RG * i;
    pk[i] = r < P ? phi_row<K>(sk, r) : 0.0f;
    pq[i] = r < P ? phi_row<K>(sq, r) : 0.0f;
  }
  for (int64_t c0 = 0, blk = 0; c0 < V; c0 += 64, ++blk) {
    const int64_t col = c0 + 4 * cq;
    const float v0 = lo_f(vr.x), v1 = hi_f(vr.x), v2 = lo_f(vr.y), v3 = hi_f(vr.y);
    f32x4_t num = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int r = rg + RG * i;
      if (r < P) {
        s[i][0] += pk[i] * v0;
        s[i][1] += pk[i] * v1;
        s[i][2] += pk[i] * v2;
        s[i][3] += pk[i] * v3;
        *reinterpret_cast<f32x4_t*>(Sb + r * V + col) = s[i];
        num[0] += pq[i] * s[i][0];
        num[1] += pq[i] * s[i][1];
        num[2] += pq[i] * s[i][2];
        num[3] += pq[i] * s[i][3];
      }
    }
    part[blk & 1][rg][cq] = num;
    if (c0 + 64 < V) request(c0 + 64);
    __syncthreads();  // also publishes part_den on the first block
    if (tid < 64) {
      float n = 0.0f;
      for (int g = 0; g < RG; ++g) n += part[blk & 1][g][tid >> 2][tid & 3];
      float den = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) den += part_den[w];
      const float o = n / (den + 1e-6f);
      if (out_f32) {
        static_cast<float*>(out)[bh * V + c0 + tid] = o;
      } else {
        static_cast<u16*>(out)[bh * V + c0 + tid] = static_cast<u16>(pack2(o, 0.0f) & 0xffffu);
      }
    }
  }
}

// ------------------------------------------------------------------------------- host launchers

template <int K, int VS>
hipError_t launch_segment_state(const void* k, const void* v, const Shape& sh, const Plan& pl, float* ws,
                                hipStream_t stream) {
  const int64_t items = sh.B * sh.H * (pl.nvs * VS / 64) * state_slots(pl);
  const int64_t blocks = (items + 7) / 8 * 8;
  hipLaunchKernelGGL((based_segment_state_kernel<K, VS>), dim3(static_cast<unsigned>(blocks)),
                     dim3(StateSplit<Cfg<K, 64>>::W * kWave), 0, stream, static_cast<const u16*>(k),
                     static_cast<const u16*>(v), sh, pl, ws);
  return hipGetLastError();
}

hipError_t launch_segment_scan(const Shape& sh, const Plan& pl, float* ws, hipStream_t stream) {
  const int64_t n_bhv = sh.B * sh.H * pl.nvs;
  const int64_t bf16_groups = state_value_groups(sh.K, pl.item_cols);
  const int64_t total = n_bhv * (bf16_groups + (pl.slot_floats - 2 * bf16_groups) / 4);
  const int64_t blocks = (total + kScanThreads - 1) / kScanThreads;
  hipLaunchKernelGGL(based_segment_scan_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kScanThreads), 0, stream, ws,
                     n_bhv, state_slots(pl), pl.slot_floats, bf16_groups);
  return hipGetLastError();
}

template <int K, int VS>
hipError_t launch_chunk_readout(const void* q, const void* k, const void* v, const Shape& sh, const Plan& pl,
                                float sigma, const float* ws, void* out, bool out_f32, const StateIO& io,
                                hipStream_t stream) {
  const int64_t items = sh.B * sh.H * pl.nvs * pl.segments;
  const int64_t blocks = (items + 7) / 8 * 8;
  const float c1 = sigma;
  const float c2 = 0.5f * sigma * sigma;
  const dim3 grid(static_cast<unsigned>(blocks)), block(Split<Cfg<K, VS>>::W * kWave);
  constexpr bool kCanRows = !(K == 16 && VS == 128);
  if (out_f32) {
    hipLaunchKernelGGL((based_chunk_readout_kernel<K, VS, true, false>), grid, block, 0, stream,
                       static_cast<const u16*>(q), static_cast<const u16*>(k), static_cast<const u16*>(v), sh, pl, c1,
                       c2, sigma, ws, out, io);
  } else if (kCanRows && pl.row_stores) {
    hipLaunchKernelGGL((based_chunk_readout_kernel<K, VS, false, kCanRows>), grid, block, 0, stream,
                       static_cast<const u16*>(q), static_cast<const u16*>(k), static_cast<const u16*>(v), sh, pl, c1,
                       c2, sigma, ws, out, io);
  } else {
    hipLaunchKernelGGL((based_chunk_readout_kernel<K, VS, false, false>), grid, block, 0, stream,
                       static_cast<const u16*>(q), static_cast<const u16*>(k), static_cast<const u16*>(v), sh, pl, c1,
                       c2, sigma, ws, out, io);
  }
  return hipGetLastError();
}

hipError_t launch_decode_step(const void* q, const void* k, const void* v, int64_t B, int64_t H, int64_t K,
                              int64_t V, float sigma, float* S, float* z, void* out, bool out_f32, hipStream_t stream) {
  // 512 threads for K = 16 (273 state rows), 256 for K = 8 (73 rows): measured 19% faster than 512 at
  // B = 64, H = 16, V = 64 and 2% at B = 256, H = 32, V = 128, while K = 16 loses 4-7% at 256.
  const dim3 grid(static_cast<unsigned>(B * H));
  if (K == 16) {
    hipLaunchKernelGGL((based_decode_step_kernel<16, 512>), grid, dim3(512), 0, stream, static_cast<const u16*>(q),
                       static_cast<const u16*>(k), static_cast<const u16*>(v), V, sigma, S, z, out, out_f32);
  } else {
    hipLaunchKernelGGL((based_decode_step_kernel<8, 256>), grid, dim3(256), 0, stream, static_cast<const u16*>(q),
                       static_cast<const u16*>(k), static_cast<const u16*>(v), V, sigma, S, z, out, out_f32);
  }
  return hipGetLastError();
}

// Workspace of based_forward_noalloc, for callers that cannot allocate: one copy per device, held until
// the process ends. Host code never names it directly (in host code the name is a stand-in, not a device
// address): scratch_buffer() looks up the device address once per device and hands that out.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t scratch_buffer(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t r = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (r != hipSuccess) return r;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

int item_columns(int64_t V) { return V % 128 == 0 ? 128 : 64; }

// Groups of four bf16 value-tile entries in one segment sum (none where the slot keeps fp32 value tiles),
// and its size in 4-byte words (the value tiles, then the ones tile in fp32: 16 words per feature tile).
int state_value_groups(int64_t K, int64_t VS) {
  if (K == 16 && VS == 128) return 0;  // fp32 value tiles (kBf16Slot)
  return (K == 16 ? Feat<16>::NPT : Feat<8>::NPT) * static_cast<int>(VS / 16) * kWave;
}

int state_slot_floats(int64_t K, int64_t VS) {
  const int npt = K == 16 ? Feat<16>::NPT : Feat<8>::NPT;
  const int values = npt * static_cast<int>(VS / 16) * kWave * 4;  // value-tile entries
  return (K == 16 && VS == 128 ? values : values / 2) + npt * 16;
}

int chunk_tokens(int64_t K, int64_t VS) {
  return K == 16 ? (VS == 128 ? Split<Cfg<16, 128>>::C : Split<Cfg<16, 64>>::C)
                 : (VS == 128 ? Split<Cfg<8, 128>>::C : Split<Cfg<8, 64>>::C);
}

int waves_per_item(int64_t K, int64_t VS) {
  return K == 16 ? (VS == 128 ? Split<Cfg<16, 128>>::W : Split<Cfg<16, 64>>::W)
                 : (VS == 128 ? Split<Cfg<8, 128>>::W : Split<Cfg<8, 64>>::W);
}

hipError_t launch_kernel(int kernel_id, const void* q, const void* k, const void* v, const Shape& sh,
                         const Plan& pl, float sigma, float* ws, void* out, bool out_f32, const StateIO& io,
                         hipStream_t stream) {
  const bool wide = pl.item_cols == 128;
  switch (kernel_id) {
    case 0:
      if (sh.K == 16) return wide ? launch_segment_state<16, 128>(k, v, sh, pl, ws, stream)
                                  : launch_segment_state<16, 64>(k, v, sh, pl, ws, stream);
      return wide ? launch_segment_state<8, 128>(k, v, sh, pl, ws, stream)
                  : launch_segment_state<8, 64>(k, v, sh, pl, ws, stream);
    case 1:
      return launch_segment_scan(sh, pl, ws, stream);
    default:
      if (sh.K == 16)
        return wide ? launch_chunk_readout<16, 128>(q, k, v, sh, pl, sigma, ws, out, out_f32, io, stream)
                    : launch_chunk_readout<16, 64>(q, k, v, sh, pl, sigma, ws, out, out_f32, io, stream);
      return wide ? launch_chunk_readout<8, 128>(q, k, v, sh, pl, sigma, ws, out, out_f32, io, stream)
                  : launch_chunk_readout<8, 64>(q, k, v, sh, pl, sigma, ws, out, out_f32, io, stream);
  }
}

}  // namespace based
