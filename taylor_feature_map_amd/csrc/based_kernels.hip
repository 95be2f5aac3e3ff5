// Causal Based forward for MI355X (gfx950): chunked 2nd-order Taylor linear attention on bf16 MFMA.
//
// What is computed: the page "Write a fast Based (Taylor linear attention) forward kernel" (KBench task
// spec based_forward.py), field spec_md: o_i = sum_{j<=i} A_ij v_j / (sum_{j<=i} A_ij + 1e-6) with
// A_ij = 1 + s + s^2/2, s = scale * q_i.k_j. Per field spec_md, A_ij = phi(q_i).phi(k_j) for the feature
// map phi(x) = [1, x, x(x)x/sqrt(2)], so the sum over earlier tokens is a read-out of the running state
// S = sum phi(k_j) v_j^T and normaliser z = sum phi(k_j), and only the tokens of the current chunk need
// the direct polynomial (field reference_src; field perf_md describes the same split).
//
// Design (one wavefront = one (batch, head, 64-column slice of V, sequence segment)):
//  * The quadratic block is used in its symmetric form: the page allows any algebraic rearrangement
//    that matches (field spec_md). Unordered feature pairs {a, b} are laid out on a 16-lane row as
//    "cyclic distance" tiles: tile d holds x_n * x_{(n-d) mod 16} in lane n, so every partner is a DPP
//    row rotation of the lane's own feature. K = 16 needs 10 tiles of 16 features (153 used of 160):
//    d = 0..7 (diagonal and 7 full distances), d = 8 (8 pairs) plus the constant feature, and the linear
//    tile. The q side carries the coefficients (s^2/2 gives 1/2 on the diagonal, 1 off it).
//  * S (features x 64 values, plus a 16-wide "ones" tile that makes z and the row sums fall out of the
//    same MFMAs, field perf_md) lives in fp32 MFMA accumulators for the whole segment (field
//    precision_md: the carry must be fp32). It is rounded to bf16 only as an MFMA operand.
//  * Per 32-token chunk: K Q^T and the Taylor weights (squared in fp32, field precision_md), the
//    read-out phi(Q) S and the intra-chunk A V accumulate into one fp32 tile; the divide and the store
//    are fused; then S += phi(K)^T V. phi is built in registers and never written to memory (field
//    perf_md names materialising it as the waste to avoid).
//  * Long sequences are split into segments so that all SIMDs have work: a first kernel sums
//    phi(k)^T v per segment, a second turns those sums into prefix states, and the read-out kernel
//    starts each segment from its prefix state.
//
// MFMA lane layouts used (v_mfma_f32_16x16x32_bf16, lane l, column c = l % 16, group g = l / 16):
//   A operand: row c, contraction slots 8g..8g+7;  B operand: column c, slots 8g..8g+7;
//   D: column c, rows 4g..4g+3.  The contraction order is free as long as A and B agree, which is used
//   to feed D registers of one product straight into the next without any data movement.

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

constexpr int kTRow = kChunk + 4;   // transposed LDS rows: 32 tokens + 8 bytes of padding
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

// ------------------------------------------------------------------------------ LDS staging

template <int K>
struct __align__(16) Smem {
  u16 q[kChunk * K];       // (token, feature)
  u16 k[kChunk * K];       // (token, feature)
  u16 kt[K * kTRow];       // (feature, token)
  u16 vt[kVSlice * kTRow]; // (value column, token)
};

struct Prefetch {
  u32x4_t q, k;
  u32x4_t v[4];
};

// Global loads of one 32-token chunk of one (b, h, value slice). Tokens >= T read as zero.
// q/k: K = 16 -> lane l loads features 8(l%2).. of token l/2; K = 8 -> lanes 0..31 load token l.
// v:   load i of lane l covers flat f = 64 i + l: token f / 8, columns 8 (f % 8) .. + 7.
template <int K, bool WITH_Q>
__device__ __forceinline__ void prefetch(Prefetch& pf, const u16* __restrict__ qb, const u16* __restrict__ kb,
                                         const u16* __restrict__ vb, int64_t t0, int64_t T, int64_t qk_stride,
                                         int64_t v_stride, int lane) {
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  int tok, col;
  if constexpr (K == 16) {
    tok = lane >> 1;
    col = (lane & 1) * 8;
  } else {
    tok = lane & 31;
    col = 0;
  }
  const bool qk_lane = (K == 16) || lane < 32;
  const bool ok = qk_lane && (t0 + tok < T);
  const int64_t off = (t0 + tok) * qk_stride + col;
  pf.k = ok ? *reinterpret_cast<const u32x4_t*>(kb + off) : zero;
  if constexpr (WITH_Q) pf.q = ok ? *reinterpret_cast<const u32x4_t*>(qb + off) : zero;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = i * 64 + lane;
    const int vtok = f >> 3;
    const bool vok = t0 + vtok < T;
    pf.v[i] = vok ? *reinterpret_cast<const u32x4_t*>(vb + (t0 + vtok) * v_stride + (f & 7) * 8) : zero;
  }
}

template <int K, bool WITH_Q>
__device__ __forceinline__ void stage(Smem<K>& sm, const Prefetch& pf, int lane) {
  int tok, col;
  if constexpr (K == 16) {
    tok = lane >> 1;
    col = (lane & 1) * 8;
  } else {
    tok = lane & 31;
    col = 0;
  }
  if ((K == 16) || lane < 32) {
    if constexpr (WITH_Q) *reinterpret_cast<u32x4_t*>(&sm.q[tok * K + col]) = pf.q;
    *reinterpret_cast<u32x4_t*>(&sm.k[tok * K + col]) = pf.k;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      sm.kt[(col + 2 * w) * kTRow + tok] = static_cast<u16>(pf.k[w]);
      sm.kt[(col + 2 * w + 1) * kTRow + tok] = static_cast<u16>(pf.k[w] >> 16);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = i * 64 + lane;
    const int vtok = f >> 3;
    const int vcol = (f & 7) * 8;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      sm.vt[(vcol + 2 * w) * kTRow + vtok] = static_cast<u16>(pf.v[i][w]);
      sm.vt[(vcol + 2 * w + 1) * kTRow + vtok] = static_cast<u16>(pf.v[i][w] >> 16);
    }
  }
}

// B operand of value tile vt (column c <-> value column 4c + vt; slot e <-> token 16(e/4) + 4g + e%4).
template <int K>
__device__ __forceinline__ u32x4_t value_operand(const Smem<K>& sm, int vt, int c, int g) {
  const u16* row = &sm.vt[(4 * c + vt) * kTRow];
  const u32x2_t a = *reinterpret_cast<const u32x2_t*>(row + 4 * g);
  const u32x2_t b = *reinterpret_cast<const u32x2_t*>(row + 16 + 4 * g);
  return u32x4_t{a.x, a.y, b.x, b.y};
}

// Key features of the lane's 8 token slots for feature c (K = 8: c % 8).
template <int K>
__device__ __forceinline__ void key_column(const Smem<K>& sm, int c, int g, float* kx) {
  const u16* row = &sm.kt[(c & (K - 1)) * kTRow];
  const u32x2_t a = *reinterpret_cast<const u32x2_t*>(row + 4 * g);
  const u32x2_t b = *reinterpret_cast<const u32x2_t*>(row + 16 + 4 * g);
  kx[0] = lo_f(a.x); kx[1] = hi_f(a.x); kx[2] = lo_f(a.y); kx[3] = hi_f(a.y);
  kx[4] = lo_f(b.x); kx[5] = hi_f(b.x); kx[6] = lo_f(b.y); kx[7] = hi_f(b.y);
}

// S (features x [64 values | ones]) += phi(K_chunk)^T [V_chunk | 1].
template <int K>
__device__ __forceinline__ void state_update(f32x4_t (&S)[Feat<K>::NPT][kVT], const Smem<K>& sm,
                                             const u32x4_t (&vop)[kVT], int c, int g) {
  float kx[8];
  key_column<K>(sm, c, g, kx);
  constexpr_for<0, Feat<K>::NPT>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    u32x4_t a;
    a.x = pack2(Feat<K>::template kval<t>(kx[0], c), Feat<K>::template kval<t>(kx[1], c));
    a.y = pack2(Feat<K>::template kval<t>(kx[2], c), Feat<K>::template kval<t>(kx[3], c));
    a.z = pack2(Feat<K>::template kval<t>(kx[4], c), Feat<K>::template kval<t>(kx[5], c));
    a.w = pack2(Feat<K>::template kval<t>(kx[6], c), Feat<K>::template kval<t>(kx[7], c));
#pragma unroll
    for (int vt = 0; vt < kVT; ++vt) S[t][vt] = mfma32(a, vop[vt], S[t][vt]);
  });
}

// Register-native layout of one segment state in the workspace: [tile][value tile][row r][lane].
template <int K>
__device__ __forceinline__ void store_state(float* __restrict__ dst, const f32x4_t (&S)[Feat<K>::NPT][kVT],
                                            int lane) {
#pragma unroll
  for (int t = 0; t < Feat<K>::NPT; ++t)
#pragma unroll
    for (int vt = 0; vt < kVT; ++vt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[((t * kVT + vt) * 4 + r) * kWave + lane] = S[t][vt][r];
}

template <int K>
__device__ __forceinline__ void load_state(const float* __restrict__ src, f32x4_t (&S)[Feat<K>::NPT][kVT],
                                           int lane) {
#pragma unroll
  for (int t = 0; t < Feat<K>::NPT; ++t)
#pragma unroll
    for (int vt = 0; vt < kVT; ++vt)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[t][vt][r] = src[((t * kVT + vt) * 4 + r) * kWave + lane];
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

template <int K>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64), amdgpu_waves_per_eu(1, 1))) void
based_segment_state_kernel(const u16* __restrict__ k, const u16* __restrict__ v, Shape sh, Plan pl,
                           float* __restrict__ ws) {
  const int64_t item = item_of_block();
  const int64_t items = sh.B * sh.H * pl.nvs * (pl.segments - 1);
  if (item >= items) return;
  const ItemCoords ic = decode_item(item, sh.H, pl.nvs, pl.segments - 1);
  const int lane = threadIdx.x;
  const int c = lane & 15, g = lane >> 4;

  __shared__ Smem<K> sm;
  const int64_t qk_stride = sh.H * K, v_stride = sh.H * sh.V;
  const u16* kb = k + (ic.b * sh.T * sh.H + ic.h) * K;
  const u16* vb = v + (ic.b * sh.T * sh.H + ic.h) * sh.V + ic.vs * kVSlice;

  f32x4_t S[Feat<K>::NPT][kVT];
#pragma unroll
  for (int t = 0; t < Feat<K>::NPT; ++t)
#pragma unroll
    for (int vt = 0; vt < kVT; ++vt) S[t][vt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t t_begin = ic.g * pl.seg_len;
  const int64_t t_end = t_begin + pl.seg_len;  // full segment: only the last one can be short
  Prefetch pf;
  prefetch<K, false>(pf, nullptr, kb, vb, t_begin, sh.T, qk_stride, v_stride, lane);
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kChunk) {
    __syncthreads();
    stage<K, false>(sm, pf, lane);
    __syncthreads();
    if (t0 + kChunk < t_end)
      prefetch<K, false>(pf, nullptr, kb, vb, t0 + kChunk, sh.T, qk_stride, v_stride, lane);
    u32x4_t vop[kVT];
#pragma unroll
    for (int vt = 0; vt < 4; ++vt) vop[vt] = value_operand<K>(sm, vt, c, g);
    vop[4] = u32x4_t{kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};
    state_update<K>(S, sm, vop, c, g);
  }
  const int64_t bhv = (ic.b * sh.H + ic.h) * pl.nvs + ic.vs;
  store_state<K>(ws + (bhv * (pl.segments - 1) + ic.g) * pl.slot_floats, S, lane);
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

template <int K, bool OUT_F32>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64), amdgpu_waves_per_eu(1, 1))) void
based_chunk_readout_kernel(const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
                           Shape sh, Plan pl, float c1, float c2, float sigma,
                           const float* __restrict__ ws, void* __restrict__ out) {
  using F = Feat<K>;
  constexpr int NPT = F::NPT;
  constexpr int NPAIR = (NPT + 1) / 2;
  const int64_t item = item_of_block();
  const int64_t items = sh.B * sh.H * pl.nvs * pl.segments;
  if (item >= items) return;
  const ItemCoords ic = decode_item(item, sh.H, pl.nvs, pl.segments);
  const int lane = threadIdx.x;
  const int c = lane & 15, g = lane >> 4;

  __shared__ Smem<K> sm;
  const int64_t qk_stride = sh.H * K, v_stride = sh.H * sh.V;
  const int64_t bh_qk = (ic.b * sh.T * sh.H + ic.h) * K;
  const int64_t bh_v = (ic.b * sh.T * sh.H + ic.h) * sh.V + ic.vs * kVSlice;
  const u16* qb = q + bh_qk;
  const u16* kb = k + bh_qk;
  const u16* vb = v + bh_v;

  f32x4_t S[NPT][kVT];
  if (ic.g > 0) {
    const int64_t bhv = (ic.b * sh.H + ic.h) * pl.nvs + ic.vs;
    load_state<K>(ws + (bhv * (pl.segments - 1) + ic.g - 1) * pl.slot_floats, S, lane);
  } else {
#pragma unroll
    for (int t = 0; t < NPT; ++t)
#pragma unroll
      for (int vt = 0; vt < kVT; ++vt) S[t][vt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int64_t t_begin = ic.g * pl.seg_len;
  const int64_t t_end = (t_begin + pl.seg_len < sh.T) ? t_begin + pl.seg_len : sh.T;
  Prefetch pf;
  prefetch<K, true>(pf, qb, kb, vb, t_begin, sh.T, qk_stride, v_stride, lane);

  for (int64_t t0 = t_begin; t0 < t_end; t0 += kChunk) {
    __syncthreads();
    stage<K, true>(sm, pf, lane);
    __syncthreads();
    if (t0 + kChunk < t_end) prefetch<K, true>(pf, qb, kb, vb, t0 + kChunk, sh.T, qk_stride, v_stride, lane);

    u32x4_t vop[kVT];
#pragma unroll
    for (int vt = 0; vt < 4; ++vt) vop[vt] = value_operand<K>(sm, vt, c, g);
    vop[4] = u32x4_t{kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};

    // ---- scores s' = K Q^T (D[j][i], lane: column i = c, rows j = 4g + r), unscaled.
    u32x2_t ka0, ka1, qb0, qb1;
    if (K == 16 || g < 2) {
      ka0 = *reinterpret_cast<const u32x2_t*>(&sm.k[c * K + 4 * g]);
      ka1 = *reinterpret_cast<const u32x2_t*>(&sm.k[(16 + c) * K + 4 * g]);
      qb0 = *reinterpret_cast<const u32x2_t*>(&sm.q[c * K + 4 * g]);
      qb1 = *reinterpret_cast<const u32x2_t*>(&sm.q[(16 + c) * K + 4 * g]);
    } else {
      ka0 = ka1 = qb0 = qb1 = u32x2_t{0u, 0u};
    }
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    const f32x4_t d00 = mfma16(ka0, qb0, zero4);  // j-tile 0, i-tile 0
    const f32x4_t d01 = mfma16(ka0, qb1, zero4);  // j-tile 0, i-tile 1
    const f32x4_t d11 = mfma16(ka1, qb1, zero4);  // j-tile 1, i-tile 1

    // ---- Taylor weights A = 1 + c1 s' + c2 s'^2 (c1 = scale, c2 = scale^2/2), causal, rounded once.
    // A operand of i-tile ii: slot e <-> token j = 16(e/4) + 4g + e%4, row i = 16 ii + c.
    u32x4_t aop[2];
    {
      float w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s = d00[r];
        const float a = fmaf(s, fmaf(s, c2, c1), 1.0f);
        w[r] = (4 * g + r <= c) ? a : 0.0f;
      }
      aop[0] = u32x4_t{pack2(w[0], w[1]), pack2(w[2], w[3]), 0u, 0u};
      float u[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s0 = d01[r];
        w[r] = fmaf(s0, fmaf(s0, c2, c1), 1.0f);
        const float s1 = d11[r];
        const float a = fmaf(s1, fmaf(s1, c2, c1), 1.0f);
        u[r] = (4 * g + r <= c) ? a : 0.0f;
      }
      aop[1] = u32x4_t{pack2(w[0], w[1]), pack2(w[2], w[3]), pack2(u[0], u[1]), pack2(u[2], u[3])};
    }

    // ---- read-out of earlier tokens through the state, plus the intra-chunk part.
    f32x4_t O[2][kVT];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int vt = 0; vt < kVT; ++vt) O[ii][vt] = zero4;

    float ry[2][F::NQ], hy[2][4];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const u16* qrow = &sm.q[(16 * ii + c) * K];
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

    constexpr_for<0, NPAIR>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int t0_ = 2 * m, t1_ = 2 * m + 1;
      u32x4_t pq[2];
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        pq[ii].x = pack2(F::template qval<t0_, 0>(ry[ii], hy[ii], g), F::template qval<t0_, 1>(ry[ii], hy[ii], g));
        pq[ii].y = pack2(F::template qval<t0_, 2>(ry[ii], hy[ii], g), F::template qval<t0_, 3>(ry[ii], hy[ii], g));
        pq[ii].z = pack2(F::template qval<t1_, 0>(ry[ii], hy[ii], g), F::template qval<t1_, 1>(ry[ii], hy[ii], g));
        pq[ii].w = pack2(F::template qval<t1_, 2>(ry[ii], hy[ii], g), F::template qval<t1_, 3>(ry[ii], hy[ii], g));
      }
#pragma unroll
      for (int vt = 0; vt < kVT; ++vt) {
        u32x4_t sb;
        sb.x = pack2(S[t0_][vt][0], S[t0_][vt][1]);
        sb.y = pack2(S[t0_][vt][2], S[t0_][vt][3]);
        if constexpr (t1_ < NPT) {
          sb.z = pack2(S[t1_][vt][0], S[t1_][vt][1]);
          sb.w = pack2(S[t1_][vt][2], S[t1_][vt][3]);
        } else {
          sb.z = 0u;
          sb.w = 0u;
        }
        O[0][vt] = mfma32(pq[0], sb, O[0][vt]);
        O[1][vt] = mfma32(pq[1], sb, O[1][vt]);
      }
    });
#pragma unroll
    for (int vt = 0; vt < kVT; ++vt) {
      O[0][vt] = mfma32(aop[0], vop[vt], O[0][vt]);
      O[1][vt] = mfma32(aop[1], vop[vt], O[1][vt]);
    }

    // ---- o = num / (den + 1e-6); lane holds rows i = 16 ii + 4g + r, columns 4c .. 4c + 3.
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t tok = t0 + 16 * ii + 4 * g + r;
        const float inv = __builtin_amdgcn_rcpf(O[ii][4][r] + 1e-6f);
        const float o0 = O[ii][0][r] * inv, o1 = O[ii][1][r] * inv;
        const float o2 = O[ii][2][r] * inv, o3 = O[ii][3][r] * inv;
        if (tok < t_end) {
          const int64_t off = ((ic.b * sh.T + tok) * sh.H + ic.h) * sh.V + ic.vs * kVSlice + 4 * c;
          if constexpr (OUT_F32) {
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + off) = f32x4_t{o0, o1, o2, o3};
          } else {
            *reinterpret_cast<u32x2_t*>(static_cast<u16*>(out) + off) = u32x2_t{pack2(o0, o1), pack2(o2, o3)};
          }
        }
      }
    }

    if (t0 + kChunk < t_end) state_update<K>(S, sm, vop, c, g);
  }
}

// ------------------------------------------------------------------------------- host launchers

template <int K>
hipError_t launch_segment_state(const void* k, const void* v, const Shape& sh, const Plan& pl, float* ws,
                                hipStream_t stream) {
  const int64_t items = sh.B * sh.H * pl.nvs * (pl.segments - 1);
  const int64_t blocks = (items + 7) / 8 * 8;
  hipLaunchKernelGGL(based_segment_state_kernel<K>, dim3(static_cast<unsigned>(blocks)), dim3(kWave), 0, stream,
                     static_cast<const u16*>(k), static_cast<const u16*>(v), sh, pl, ws);
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
    hipLaunchKernelGGL((based_chunk_readout_kernel<K, true>), dim3(static_cast<unsigned>(blocks)), dim3(kWave), 0,
                       stream, static_cast<const u16*>(q), static_cast<const u16*>(k), static_cast<const u16*>(v),
                       sh, pl, c1, c2, sigma, ws, out);
  } else {
    hipLaunchKernelGGL((based_chunk_readout_kernel<K, false>), dim3(static_cast<unsigned>(blocks)), dim3(kWave), 0,
                       stream, static_cast<const u16*>(q), static_cast<const u16*>(k), static_cast<const u16*>(v),
                       sh, pl, c1, c2, sigma, ws, out);
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
