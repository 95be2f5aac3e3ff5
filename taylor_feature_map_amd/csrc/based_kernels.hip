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
//  * Work item = (batch b, head h, 64-column slice of V, sequence segment), run by a workgroup of two
//    wavefronts. The feature tiles (below) are split between the two waves: each wave holds its half of
//    S in fp32 MFMA accumulators, builds only its half of phi(k) and phi(q), and the two partial
//    read-outs are added through LDS. Each wave finishes (divides and stores) one 16-token half of the
//    32-token chunk.
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
//  * Per 32-token chunk: K Q^T and the Taylor weights, the read-out phi(Q) S and the intra-chunk A V
//    accumulate into one fp32 tile; the divide and the store are fused; then S += phi(K)^T V. phi is
//    built in registers and never written to memory (field perf_md names materialising it as the waste).
//  * Inputs are prefetched one chunk ahead into registers and staged in LDS in their natural row layout
//    (16-byte units of V swizzled against bank conflicts); the transposed MFMA operands (V and K with the
//    token index along the contraction) come from ds_read_b64_tr_b16 transpose reads.
//  * Long sequences are split into segments so that all SIMDs have work: a first kernel sums
//    phi(k)^T v per segment, a second turns those sums into prefix states, and the read-out kernel
//    starts each segment from its prefix state.
//
// MFMA lane layouts used (v_mfma_f32_16x16x32_bf16, lane l, column c = l % 16, group g = l / 16):
//   A operand: row c, contraction slots 8g..8g+7;  B operand: column c, slots 8g..8g+7;
//   D: column c, rows 4g..4g+3.  The contraction order is free as long as A and B agree; slot e of
//   group g is token 16(e/4) + 4g + e%4 of the chunk, which lets the D registers of K Q^T feed A V, and
//   feature (t, 4g + e%4) of tile pair (t = 2m + e/4), which lets the D registers of S feed phi(Q) S,
//   without any data movement.

#include <hip/hip_runtime.h>
#include <stdint.h>

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
constexpr int kNW = 2;  // wavefronts per work item

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
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + D, 0xf, 0xf, false));
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
__device__ __forceinline__ int64_t item_of_block() {
  const int64_t per = gridDim.x >> 3;
  const int64_t x = blockIdx.x;
  return (x & 7) * per + (x >> 3);
}

// ------------------------------------------------------------------------- feature tiles (phi)

template <int K>
struct Feat;

// K = 16. k side: lane column c holds x = k[c] for one token; tile T returns that lane's feature.
// q side: ry[m] = y[(4g + m) mod 16] with y = scale * q (rotated per lane group), hy[r] = ry[r] / 2;
// feature (T, n = 4g + R) is returned for slot R.
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
  __device__ static __forceinline__ float qval(const float* ry, const float* hy, int g) {
    if constexpr (T == 0) {
      return ry[R] * hy[R];
    } else if constexpr (T <= 7) {
      return ry[R] * ry[(R - T) & 15];
    } else if constexpr (T == 8) {
      const float p = ry[R] * ry[(R - 8) & 15];
      return g < 2 ? p : ((g == 2 && R == 0) ? 1.0f : 0.0f);
    } else if constexpr (T == 9) {
      return ry[R];
    } else {
      return 0.0f;
    }
  }
};

// K = 8: the 16-lane row holds the 8 features twice (lane c has feature c % 8); half h = c / 8.
// Tiles: 0 = {h0: diagonal, h1: distance 1}, 1 = {h0: distance 2, h1: distance 3},
//        2 = {h0: distance 4 on features 0..3, constant on feature 4, h1: linear}; 45 of 48 used.
// q side: ry[m] = y[(4 (g & 1) + m) mod 8].
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
  __device__ static __forceinline__ float qval(const float* ry, const float* hy, int g) {
    const bool h0 = g < 2;
    if constexpr (T == 0) {
      return h0 ? ry[R] * hy[R] : ry[R] * ry[(R - 1) & 7];
    } else if constexpr (T == 1) {
      return h0 ? ry[R] * ry[(R - 2) & 7] : ry[R] * ry[(R - 3) & 7];
    } else if constexpr (T == 2) {
      const float p = ry[R] * ry[(R - 4) & 7];
      return h0 ? ((g & 1) == 0 ? p : (R == 0 ? 1.0f : 0.0f)) : ry[R];
    } else {
      return 0.0f;
    }
  }
};

// Feature tiles owned by wave W: [T0, T0 + NT). K = 16: 5 + 5; K = 8: 2 + 1.
template <int K, int W>
struct Tiles {
  static constexpr int T0 = (K == 16) ? 5 * W : 2 * W;
  static constexpr int NT = (K == 16) ? 5 : (W == 0 ? 2 : 1);
  static constexpr int NKS = (NT + 1) / 2;  // 32-deep contraction steps of the read-out
};

// ------------------------------------------------------------------------------ LDS staging

// One 32-token chunk of one (b, h, value slice), natural row layout:
//   K = 16: q[32][16], k[32][16];  K = 8: q[32][8] then k[32][8] inside `q`.
//   v: 4 blocks of 8 tokens x 64 columns; within a token row the 16-byte unit `oct` (columns
//   8 oct .. 8 oct + 7) is stored at position oct ^ (token % 8).
struct __align__(16) Stage {
  u16 q[512];
  u16 k[512];
  u16 v[2048];
};

__device__ __forceinline__ int v_index(int tok, int col) {
  return (tok >> 3) * 512 + (tok & 7) * 64 + (((col >> 3) ^ (tok & 7)) << 3) + (col & 7);
}

// Three 16-byte loads per lane per chunk. Wave W: r[0] = q (W = 0) or k (W = 1) rows for K = 16
// (K = 8: W = 0 loads q into lanes 0..31 and k into lanes 32..63, W = 1 loads none), r[1], r[2] = value
// blocks 2W and 2W + 1. Tokens >= T are clamped to T - 1: they only ever meet zero Taylor weights.
template <int K, int W, bool WITH_Q>
struct Prefetch {
  u32x4_t r[3];

  __device__ __forceinline__ void load(const u16* __restrict__ qb, const u16* __restrict__ kb,
                                       const u16* __restrict__ vb, int64_t t0, int64_t T, int64_t qk_stride,
                                       int64_t v_stride, int lane) {
    if constexpr (K == 16) {
      const u16* src = (W == 0) ? qb : kb;
      if (W == 1 || WITH_Q) {
        int64_t t = t0 + (lane >> 1);
        t = t < T ? t : T - 1;
        r[0] = *reinterpret_cast<const u32x4_t*>(src + t * qk_stride + (lane & 1) * 8);
      }
    } else if constexpr (W == 0) {
      int64_t t = t0 + (lane & 31);
      t = t < T ? t : T - 1;
      const u16* src = (lane < 32) ? qb : kb;
      if (lane >= 32 || WITH_Q) r[0] = *reinterpret_cast<const u32x4_t*>(src + t * qk_stride);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int blk = 2 * W + j;
      const int row = lane >> 3;
      int64_t t = t0 + blk * 8 + row;
      t = t < T ? t : T - 1;
      const int oct = (lane & 7) ^ row;
      r[1 + j] = *reinterpret_cast<const u32x4_t*>(vb + t * v_stride + oct * 8);
    }
  }

  __device__ __forceinline__ void store(Stage& st, int lane) const {
    if constexpr (K == 16) {
      if (W == 1 || WITH_Q) {
        u16* dst = (W == 0) ? st.q : st.k;
        *reinterpret_cast<u32x4_t*>(dst + lane * 8) = r[0];
      }
    } else if constexpr (W == 0) {
      if (lane >= 32 || WITH_Q) *reinterpret_cast<u32x4_t*>(st.q + lane * 8) = r[0];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4_t*>(st.v + (2 * W + j) * 512 + lane * 8) = r[1 + j];
  }
};

// B operand of value tile vt: column m <-> value column 16 vt + m; slot e <-> token 16(e/4) + 4g + e%4.
__device__ __forceinline__ u32x4_t value_operand(const Stage& st, int vt, int lane) {
  const int g = lane >> 4, r = lane & 15;
  const int col = 16 * vt + 4 * (r & 3);
  const u32x2_t a = lds_tr16(st.v + v_index(4 * g + (r >> 2), col));
  const u32x2_t b = lds_tr16(st.v + v_index(16 + 4 * g + (r >> 2), col));
  return u32x4_t{a.x, a.y, b.x, b.y};
}

// Key feature c (K = 8: c % 8) of the lane's 8 token slots, as floats.
template <int K>
__device__ __forceinline__ void key_column(const Stage& st, int lane, float* kx) {
  const int g = lane >> 4, r = lane & 15;
  const u16* base = (K == 16) ? st.k : st.q + 256;
  const int f4 = (K == 16) ? 4 * (r & 3) : 4 * (r & 1);
  const u32x2_t a = lds_tr16(base + (4 * g + (r >> 2)) * K + f4);
  const u32x2_t b = lds_tr16(base + (16 + 4 * g + (r >> 2)) * K + f4);
  kx[0] = lo_f(a.x); kx[1] = hi_f(a.x); kx[2] = lo_f(a.y); kx[3] = hi_f(a.y);
  kx[4] = lo_f(b.x); kx[5] = hi_f(b.x); kx[6] = lo_f(b.y); kx[7] = hi_f(b.y);
}

// S[own tiles] (features x [64 values | ones]) += phi(K_chunk)^T [V_chunk | 1].
template <int K, int W, typename SA>
__device__ __forceinline__ void state_update(SA& S, const Stage& st, const u32x4_t (&vop)[kVT], int lane) {
  using TL = Tiles<K, W>;
  const int c = lane & 15;
  float kx[8];
  key_column<K>(st, lane, kx);
  constexpr_for<0, TL::NT>([&](auto lc) {
    constexpr int lt = decltype(lc)::value;
    constexpr int t = TL::T0 + lt;
    u32x4_t a;
    a.x = pack2(Feat<K>::template kval<t>(kx[0], c), Feat<K>::template kval<t>(kx[1], c));
    a.y = pack2(Feat<K>::template kval<t>(kx[2], c), Feat<K>::template kval<t>(kx[3], c));
    a.z = pack2(Feat<K>::template kval<t>(kx[4], c), Feat<K>::template kval<t>(kx[5], c));
    a.w = pack2(Feat<K>::template kval<t>(kx[6], c), Feat<K>::template kval<t>(kx[7], c));
#pragma unroll
    for (int vt = 0; vt < kVT; ++vt) S[lt][vt] = mfma32(a, vop[vt], S[lt][vt]);
  });
}

// Register-native layout of one segment state in the workspace: [tile][value tile][row r][lane].
__device__ __forceinline__ int64_t state_offset(int t, int vt, int r, int lane) {
  return ((t * kVT + vt) * 4 + r) * kWave + lane;
}

struct ItemCoords {
  int64_t b, h, vs, g;
};

__device__ __forceinline__ ItemCoords decode_item(int64_t item, int64_t H, int64_t NVS, int64_t G) {
  ItemCoords ic;
  ic.h = item % H;
  int64_t r = item / H;
  ic.vs = r % NVS;
  r /= NVS;
  ic.g = r % G;
  ic.b = r / G;
  return ic;
}

// ------------------------------------------------------------------ kernel 0: segment state sums

struct __align__(16) StateSmem {
  Stage stage[2];
};

template <int K, int W>
__device__ __forceinline__ void segment_state_body(StateSmem& sm, const u16* __restrict__ kb,
                                                   const u16* __restrict__ vb, const Shape& sh, int64_t t_begin,
                                                   int64_t t_end, float* __restrict__ dst) {
  using TL = Tiles<K, W>;
  const int lane = threadIdx.x & 63;
  const int64_t qk_stride = sh.H * K, v_stride = sh.H * sh.V;
  f32x4_t S[TL::NT][kVT];
#pragma unroll
  for (int t = 0; t < TL::NT; ++t)
#pragma unroll
    for (int vt = 0; vt < kVT; ++vt) S[t][vt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  Prefetch<K, W, false> pf;
  pf.load(nullptr, kb, vb, t_begin, sh.T, qk_stride, v_stride, lane);
  int it = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kChunk, ++it) {
    Stage& st = sm.stage[it & 1];
    pf.store(st, lane);
    __syncthreads();
    if (t0 + kChunk < t_end) pf.load(nullptr, kb, vb, t0 + kChunk, sh.T, qk_stride, v_stride, lane);
    u32x4_t vop[kVT];
#pragma unroll
    for (int vt = 0; vt < 4; ++vt) vop[vt] = value_operand(st, vt, lane);
    vop[4] = u32x4_t{kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};
    state_update<K, W>(S, st, vop, lane);
  }
#pragma unroll
  for (int lt = 0; lt < TL::NT; ++lt)
#pragma unroll
    for (int vt = 0; vt < kVT; ++vt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[state_offset(TL::T0 + lt, vt, r, lane)] = S[lt][vt][r];
}

template <int K>
__global__ __launch_bounds__(kNW * kWave) void based_segment_state_kernel(const u16* __restrict__ k,
                                                                           const u16* __restrict__ v, Shape sh,
                                                                           Plan pl, float* __restrict__ ws) {
  const int64_t item = item_of_block();
  const int64_t items = sh.B * sh.H * pl.nvs * (pl.segments - 1);
  if (item >= items) return;
  const ItemCoords ic = decode_item(item, sh.H, pl.nvs, pl.segments - 1);
  __shared__ StateSmem sm;
  const u16* kb = k + (ic.b * sh.T * sh.H + ic.h) * K;
  const u16* vb = v + (ic.b * sh.T * sh.H + ic.h) * sh.V + ic.vs * kVSlice;
  const int64_t t_begin = ic.g * pl.seg_len;
  const int64_t t_end = t_begin + pl.seg_len;  // full segment: only the last one can be short
  const int64_t bhv = (ic.b * sh.H + ic.h) * pl.nvs + ic.vs;
  float* dst = ws + (bhv * (pl.segments - 1) + ic.g) * pl.slot_floats;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w == 0)
    segment_state_body<K, 0>(sm, kb, vb, sh, t_begin, t_end, dst);
  else
    segment_state_body<K, 1>(sm, kb, vb, sh, t_begin, t_end, dst);
}

// ------------------------------------------------------------- kernel 1: prefix over segments

// In place: slot s of every (b, h, value slice) becomes the sum of the segment sums 0..s, i.e. the
// state at the start of segment s + 1.
__global__ __launch_bounds__(256) void based_segment_scan_kernel(float* __restrict__ ws, int64_t n_bhv,
                                                                 int64_t slots, int64_t slot_floats) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= n_bhv * slot_floats) return;
  const int64_t bhv = idx / slot_floats;
  const int64_t e = idx - bhv * slot_floats;
  float* p = ws + bhv * slots * slot_floats + e;
  float run = 0.0f;
  for (int64_t s = 0; s < slots; ++s) {
    run += p[s * slot_floats];
    p[s * slot_floats] = run;
  }
}

// ------------------------------------------------------------------- kernel 2: chunked read-out

struct __align__(16) ReadoutSmem {
  Stage stage[2];
  float xch[kNW][kVT * 4][kWave];  // read-out partial of the other wave's 16-token half
};

template <int K, int W, bool OUT_F32>
__device__ __forceinline__ void readout_body(ReadoutSmem& sm, const u16* __restrict__ qb,
                                             const u16* __restrict__ kb, const u16* __restrict__ vb,
                                             const Shape& sh, int64_t t_begin, int64_t t_end, float c1, float c2,
                                             float sigma, const float* __restrict__ src, void* __restrict__ out,
                                             int64_t out_base) {
  using F = Feat<K>;
  using TL = Tiles<K, W>;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int64_t qk_stride = sh.H * K, v_stride = sh.H * sh.V;
  const int64_t out_stride = sh.H * sh.V;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  f32x4_t S[TL::NT][kVT];
  if (src) {
#pragma unroll
    for (int lt = 0; lt < TL::NT; ++lt)
#pragma unroll
      for (int vt = 0; vt < kVT; ++vt)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[lt][vt][r] = src[state_offset(TL::T0 + lt, vt, r, lane)];
  } else {
#pragma unroll
    for (int lt = 0; lt < TL::NT; ++lt)
#pragma unroll
      for (int vt = 0; vt < kVT; ++vt) S[lt][vt] = zero4;
  }

  Prefetch<K, W, true> pf;
  pf.load(qb, kb, vb, t_begin, sh.T, qk_stride, v_stride, lane);
  int it = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kChunk, ++it) {
    Stage& st = sm.stage[it & 1];
    pf.store(st, lane);
    __syncthreads();
    if (t0 + kChunk < t_end) pf.load(qb, kb, vb, t0 + kChunk, sh.T, qk_stride, v_stride, lane);

    u32x4_t vop[kVT];
#pragma unroll
    for (int vt = 0; vt < 4; ++vt) vop[vt] = value_operand(st, vt, lane);
    vop[4] = u32x4_t{kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};

    // ---- scores s' = K Q^T for this wave's 16-token half (D[j][i], lane: column i = c, rows j = 4g + r),
    //      then Taylor weights A = 1 + c1 s' + c2 s'^2 (c1 = scale, c2 = scale^2/2), causal, rounded once.
    //      A operand: slot e <-> token j = 16(e/4) + 4g + e%4, row i = 16 W + c.
    u32x4_t aop;
    {
      const u16* qarr = st.q;
      const u16* karr = (K == 16) ? st.k : st.q + 256;
      u32x2_t ka0 = {0u, 0u}, ka1 = {0u, 0u}, qbw = {0u, 0u};
      if (K == 16 || g < 2) {
        ka0 = *reinterpret_cast<const u32x2_t*>(karr + c * K + 4 * g);
        qbw = *reinterpret_cast<const u32x2_t*>(qarr + (16 * W + c) * K + 4 * g);
        if (W == 1) ka1 = *reinterpret_cast<const u32x2_t*>(karr + (16 + c) * K + 4 * g);
      }
      const f32x4_t d0 = mfma16(ka0, qbw, zero4);  // j-tile 0
      float w0[4], w1[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = fmaf(d0[r], fmaf(d0[r], c2, c1), 1.0f);
        w0[r] = (W == 1 || 4 * g + r <= c) ? a : 0.0f;
      }
      if constexpr (W == 1) {
        const f32x4_t d1 = mfma16(ka1, qbw, zero4);  // j-tile 1 (diagonal tile of the second half)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = fmaf(d1[r], fmaf(d1[r], c2, c1), 1.0f);
          w1[r] = (4 * g + r <= c) ? a : 0.0f;
        }
        aop = u32x4_t{pack2(w0[0], w0[1]), pack2(w0[2], w0[3]), pack2(w1[0], w1[1]), pack2(w1[2], w1[3])};
      } else {
        aop = u32x4_t{pack2(w0[0], w0[1]), pack2(w0[2], w0[3]), 0u, 0u};
      }
    }

    // ---- read-out of earlier tokens through this wave's half of the state, for both 16-token halves.
    f32x4_t O[2][kVT];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int vt = 0; vt < kVT; ++vt) O[ii][vt] = zero4;

    float ry[2][F::NQ], hy[2][4];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const u16* qrow = st.q + (16 * ii + c) * K;
#pragma unroll
      for (int kk = 0; kk < F::NQ / 4; ++kk) {
        const int base = 4 * ((g + kk) & (F::NQ / 4 - 1));
        const u32x2_t w2 = *reinterpret_cast<const u32x2_t*>(qrow + base);
        ry[ii][4 * kk + 0] = sigma * lo_f(w2.x);
        ry[ii][4 * kk + 1] = sigma * hi_f(w2.x);
        ry[ii][4 * kk + 2] = sigma * lo_f(w2.y);
        ry[ii][4 * kk + 3] = sigma * hi_f(w2.y);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) hy[ii][r] = 0.5f * ry[ii][r];
    }

    constexpr_for<0, TL::NKS>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int ta = TL::T0 + 2 * m, tb = TL::T0 + 2 * m + 1;
      constexpr bool has_b = (2 * m + 1) < TL::NT;
      u32x4_t pq[2];
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        pq[ii].x = pack2(F::template qval<ta, 0>(ry[ii], hy[ii], g), F::template qval<ta, 1>(ry[ii], hy[ii], g));
        pq[ii].y = pack2(F::template qval<ta, 2>(ry[ii], hy[ii], g), F::template qval<ta, 3>(ry[ii], hy[ii], g));
        if constexpr (has_b) {
          pq[ii].z = pack2(F::template qval<tb, 0>(ry[ii], hy[ii], g), F::template qval<tb, 1>(ry[ii], hy[ii], g));
          pq[ii].w = pack2(F::template qval<tb, 2>(ry[ii], hy[ii], g), F::template qval<tb, 3>(ry[ii], hy[ii], g));
        } else {
          pq[ii].z = 0u;
          pq[ii].w = 0u;
        }
      }
#pragma unroll
      for (int vt = 0; vt < kVT; ++vt) {
        u32x4_t sb;
        sb.x = pack2(S[2 * m][vt][0], S[2 * m][vt][1]);
        sb.y = pack2(S[2 * m][vt][2], S[2 * m][vt][3]);
        if constexpr (has_b) {
          sb.z = pack2(S[2 * m + 1][vt][0], S[2 * m + 1][vt][1]);
          sb.w = pack2(S[2 * m + 1][vt][2], S[2 * m + 1][vt][3]);
        } else {
          sb.z = 0u;
          sb.w = 0u;
        }
        O[0][vt] = mfma32(pq[0], sb, O[0][vt]);
        O[1][vt] = mfma32(pq[1], sb, O[1][vt]);
      }
    });

    // ---- hand the other half's partial to the other wave; add the intra-chunk term to ours.
#pragma unroll
    for (int vt = 0; vt < kVT; ++vt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.xch[W][vt * 4 + r][lane] = O[1 - W][vt][r];
#pragma unroll
    for (int vt = 0; vt < kVT; ++vt) O[W][vt] = mfma32(aop, vop[vt], O[W][vt]);
    __syncthreads();
#pragma unroll
    for (int vt = 0; vt < kVT; ++vt)
#pragma unroll
      for (int r = 0; r < 4; ++r) O[W][vt][r] += sm.xch[1 - W][vt * 4 + r][lane];

    // ---- o = num / (den + 1e-6); lane holds rows 16 W + 4g + r, columns 16 vt + c.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t tok = t0 + 16 * W + 4 * g + r;
      const float inv = __builtin_amdgcn_rcpf(O[W][4][r] + 1e-6f);
      if (tok < t_end) {
        const int64_t off = out_base + tok * out_stride + c;
#pragma unroll
        for (int vt = 0; vt < 4; ++vt) {
          const float o = O[W][vt][r] * inv;
          if constexpr (OUT_F32) {
            static_cast<float*>(out)[off + 16 * vt] = o;
          } else {
            static_cast<__bf16*>(out)[off + 16 * vt] = static_cast<__bf16>(o);
          }
        }
      }
    }

    // Unconditional: after the last chunk the state is simply not used (tokens past T were clamped to
    // finite inputs), and a conditional update would make the compiler copy S every iteration.
    state_update<K, W>(S, st, vop, lane);
  }
}

template <int K, bool OUT_F32>
__global__ __launch_bounds__(kNW * kWave) void based_chunk_readout_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v, Shape sh, Plan pl, float c1,
    float c2, float sigma, const float* __restrict__ ws, void* __restrict__ out) {
  const int64_t item = item_of_block();
  const int64_t items = sh.B * sh.H * pl.nvs * pl.segments;
  if (item >= items) return;
  const ItemCoords ic = decode_item(item, sh.H, pl.nvs, pl.segments);
  __shared__ ReadoutSmem sm;
  const int64_t bh_qk = (ic.b * sh.T * sh.H + ic.h) * K;
  const int64_t bh_v = (ic.b * sh.T * sh.H + ic.h) * sh.V + ic.vs * kVSlice;
  const int64_t t_begin = ic.g * pl.seg_len;
  const int64_t t_end = (t_begin + pl.seg_len < sh.T) ? t_begin + pl.seg_len : sh.T;
  const float* src = nullptr;
  if (ic.g > 0) {
    const int64_t bhv = (ic.b * sh.H + ic.h) * pl.nvs + ic.vs;
    src = ws + (bhv * (pl.segments - 1) + ic.g - 1) * pl.slot_floats;
  }
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w == 0)
    readout_body<K, 0, OUT_F32>(sm, q + bh_qk, k + bh_qk, v + bh_v, sh, t_begin, t_end, c1, c2, sigma, src, out,
                                bh_v);
  else
    readout_body<K, 1, OUT_F32>(sm, q + bh_qk, k + bh_qk, v + bh_v, sh, t_begin, t_end, c1, c2, sigma, src, out,
                                bh_v);
}

// ------------------------------------------------------------------------------- host launchers

template <int K>
hipError_t launch_segment_state(const void* k, const void* v, const Shape& sh, const Plan& pl, float* ws,
                                hipStream_t stream) {
  const int64_t items = sh.B * sh.H * pl.nvs * (pl.segments - 1);
  const int64_t blocks = (items + 7) / 8 * 8;
  hipLaunchKernelGGL(based_segment_state_kernel<K>, dim3(static_cast<unsigned>(blocks)), dim3(kNW * kWave), 0,
                     stream, static_cast<const u16*>(k), static_cast<const u16*>(v), sh, pl, ws);
  return hipGetLastError();
}

hipError_t launch_segment_scan(const Shape& sh, const Plan& pl, float* ws, hipStream_t stream) {
  const int64_t n_bhv = sh.B * sh.H * pl.nvs;
  const int64_t total = n_bhv * pl.slot_floats;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(based_segment_scan_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, ws,
                     n_bhv, pl.segments - 1, pl.slot_floats);
  return hipGetLastError();
}

template <int K>
hipError_t launch_chunk_readout(const void* q, const void* k, const void* v, const Shape& sh, const Plan& pl,
                                float sigma, const float* ws, void* out, bool out_f32, hipStream_t stream) {
  const int64_t items = sh.B * sh.H * pl.nvs * pl.segments;
  const int64_t blocks = (items + 7) / 8 * 8;
  const float c1 = sigma;
  const float c2 = 0.5f * sigma * sigma;
  if (out_f32) {
    hipLaunchKernelGGL((based_chunk_readout_kernel<K, true>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kNW * kWave), 0, stream, static_cast<const u16*>(q), static_cast<const u16*>(k),
                       static_cast<const u16*>(v), sh, pl, c1, c2, sigma, ws, out);
  } else {
    hipLaunchKernelGGL((based_chunk_readout_kernel<K, false>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kNW * kWave), 0, stream, static_cast<const u16*>(q), static_cast<const u16*>(k),
                       static_cast<const u16*>(v), sh, pl, c1, c2, sigma, ws, out);
  }
  return hipGetLastError();
}

int state_slot_floats(int64_t K) { return (K == 16 ? Feat<16>::NPT : Feat<8>::NPT) * kVT * 4 * kWave; }

hipError_t launch_kernel(int kernel_id, const void* q, const void* k, const void* v, const Shape& sh,
                         const Plan& pl, float sigma, float* ws, void* out, bool out_f32, hipStream_t stream) {
  switch (kernel_id) {
    case 0:
      return sh.K == 16 ? launch_segment_state<16>(k, v, sh, pl, ws, stream)
                        : launch_segment_state<8>(k, v, sh, pl, ws, stream);
    case 1:
      return launch_segment_scan(sh, pl, ws, stream);
    default:
      return sh.K == 16 ? launch_chunk_readout<16>(q, k, v, sh, pl, sigma, ws, out, out_f32, stream)
                        : launch_chunk_readout<8>(q, k, v, sh, pl, sigma, ws, out, out_f32, stream);
  }
}

}  // namespace based
