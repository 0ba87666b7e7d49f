// Device helpers shared by the gfx950 kernels of libtopo_attn.so: bf16 unpacking, 16-byte
// chunk dot products, order-preserving integer keys for floating point values, wave and block
// reductions. Wavefronts are 64 lanes wide.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define TOPO_WAVE 64

namespace topo {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte streaming load (global_load_dwordx4 ... nt): the data is read once, so it should not
// displace reusable lines from the caches.
__device__ __forceinline__ uint4 ntload16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// bf16 pair packed in a 32-bit word: element 0 in the low half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// acc + sum of the 8 products of two 16-byte chunks of bf16 (v_dot2_f32_bf16: two products and
// an add per instruction, float32 accumulate).
__device__ __forceinline__ float dot_chunk_bf16(uint4 a, uint4 b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w), acc, false);
  return acc;
}

// acc + sum of the 4 products of two 16-byte chunks of float32 (fused multiply-adds).
__device__ __forceinline__ float dot_chunk_f32(uint4 a, uint4 b, float acc) {
  acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
  acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
  acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
  acc = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
  return acc;
}

template <bool BF16>
__device__ __forceinline__ float dot_chunk(uint4 a, uint4 b, float acc) {
  if constexpr (BF16) return dot_chunk_bf16(a, b, acc);
  else return dot_chunk_f32(a, b, acc);
}

// Order-preserving maps: a < b (as numbers, -0 == +0 excluded) <=> key(a) < key(b) (unsigned).
__device__ __forceinline__ uint32_t ord_f32(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Inverse of ord_f32 (for keys of non-NaN floats).
__device__ __forceinline__ float unord_f32(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ uint64_t ord_f64(double x) {
  x = x + 0.0;  // -0 -> +0 so that equal scores share one key
  uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

// Element t of a row stored as float32 or bf16, widened to double (exact).
template <bool BF16>
__device__ __forceinline__ double load_elem_f64(const void* row, int t) {
  if constexpr (BF16) {
    uint16_t b = ((const uint16_t*)row)[t];
    return (double)__uint_as_float((uint32_t)b << 16);
  } else {
    return (double)((const float*)row)[t];
  }
}

// Canonical score: sum over t of q_t * k_t in float64, ascending t, starting from +0.0.
// The product of two float32 (or bf16) values is exact in float64, so fma(q, k, s) rounds once,
// exactly like s + (q*k).
template <bool BF16, int D>
__device__ __forceinline__ double canonical_score(const double* qd, const void* krow) {
  double s = 0.0;
  if constexpr (BF16) {
    const uint4* p = (const uint4*)krow;
#pragma unroll 2
    for (int c = 0; c < D / 8; ++c) {
      uint4 w = p[c];
      uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s = fma(qd[c * 8 + 2 * e], (double)bf16_lo(ws[e]), s);
        s = fma(qd[c * 8 + 2 * e + 1], (double)bf16_hi(ws[e]), s);
      }
    }
  } else {
    const uint4* p = (const uint4*)krow;
#pragma unroll 2
    for (int c = 0; c < D / 4; ++c) {
      uint4 w = p[c];
      s = fma(qd[c * 4 + 0], (double)__uint_as_float(w.x), s);
      s = fma(qd[c * 4 + 1], (double)__uint_as_float(w.y), s);
      s = fma(qd[c * 4 + 2], (double)__uint_as_float(w.z), s);
      s = fma(qd[c * 4 + 3], (double)__uint_as_float(w.w), s);
    }
  }
  return s + 0.0;
}

// Same value as canonical_score, with every 16-byte chunk of the row requested before the first
// multiply-add so that the row costs one memory round trip.
// The canonical float64 score of a key row already in registers (w: its 16-byte chunks), in the
// order of canonical_score_row.
template <bool BF16, int D>
__device__ __forceinline__ double canonical_score_words(const double* qd, const uint4* w) {
  constexpr int NC = D * (BF16 ? 2 : 4) / 16;
  double s = 0.0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t ws[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (BF16) {
        s = fma(qd[c * 8 + 2 * e], (double)bf16_lo(ws[e]), s);
        s = fma(qd[c * 8 + 2 * e + 1], (double)bf16_hi(ws[e]), s);
      } else {
        s = fma(qd[c * 4 + e], (double)__uint_as_float(ws[e]), s);
      }
    }
  }
  return s + 0.0;
}

template <bool BF16, int D>
__device__ __forceinline__ double canonical_score_row(const double* qd, const void* krow) {
  constexpr int NC = D * (BF16 ? 2 : 4) / 16;
  const uint4* p = (const uint4*)krow;
  uint4 w[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) w[c] = p[c];
  return canonical_score_words<BF16, D>(qd, w);
}

__device__ __forceinline__ float wave_max_f32(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum_f32(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ double wave_max_f64(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
// Inclusive prefix sum over the lanes of a wave.
__device__ __forceinline__ int wave_incl_scan_i32(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// k-th largest value among the `n` register entries of every lane (0 = empty): the largest T
// with at least k entries >= T; 0 if fewer than k entries are non-zero.
template <int N>
__device__ __forceinline__ uint32_t wave_kth_largest(const uint32_t (&x)[N], int k) {
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int c = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) c += __popcll(__ballot(x[i] >= cand));
    if (c >= k) T = cand;
  }
  return T;
}

// A threshold T such that at least k distinct entries are >= T, computed from N register entries
// per lane (0 = empty). For k <= 64 it is the k-th largest of every lane's two largest entries,
// which is a valid bound at a fraction of the cost of the exact k-th largest; for larger k the
// exact k-th largest. 0 if fewer than k entries are non-zero.
template <int N>
__device__ __forceinline__ uint32_t wave_threshold(const uint32_t (&x)[N], int k) {
  if (k <= 64 && N > 2) {
    uint32_t m[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < N; ++i) {
      m[1] = max(m[1], min(m[0], x[i]));
      m[0] = max(m[0], x[i]);
    }
    return wave_kth_largest<2>(m, k);
  }
  return wave_kth_largest<N>(x, k);
}

// Cross-lane moves. partner<HALF> pairs every lane of a group of 2*HALF lanes with a lane of the
// other half of that group (quad permutes and row mirrors are DPP modifiers, free on the add).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int HALF>
__device__ __forceinline__ float partner(float x) {
  if constexpr (HALF == 1) return dpp_f32<0xB1>(x);        // quad_perm [1,0,3,2]
  else if constexpr (HALF == 2) return dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  else if constexpr (HALF == 4) return dpp_f32<0x141>(x);  // row_half_mirror
  else if constexpr (HALF == 8) return dpp_f32<0x140>(x);  // row_mirror
  else return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));  // xor 16
}

// Sum over aligned groups of G lanes (G = 2..32); every lane of a group gets the group's sum.
template <int G>
__device__ __forceinline__ float group_sum_f32(float x) {
#pragma unroll
  for (int hf = 1; hf < G; hf <<= 1) {
    if (hf == 1) x += partner<1>(x);
    else if (hf == 2) x += partner<2>(x);
    else if (hf == 4) x += partner<4>(x);
    else if (hf == 8) x += partner<8>(x);
    else x += partner<16>(x);
  }
  return x;
}

// One halving step of a reduce-scatter: the lanes of each half of a 2*HALF group keep their half
// of the remaining keys, summed with the partner's copy.
template <int HALF, int V, int L>
__device__ __forceinline__ void rs_step(float (&A)[V][L], bool hi) {
#pragma unroll
  for (int v = 0; v < V; ++v) {
#pragma unroll
    for (int t = 0; t < HALF; ++t) {
      const float x0 = A[v][t] + partner<HALF>(A[v][t]);
      const float x1 = A[v][t + HALF] + partner<HALF>(A[v][t + HALF]);
      A[v][t] = hi ? x1 : x0;
    }
  }
}

// A[v][m] holds this lane's partial sum of value v for key m of its L-lane group. Afterwards
// A[v][0] holds the full sum of value v for key m = (lane % L).
template <int L, int V>
__device__ __forceinline__ void reduce_scatter(float (&A)[V][L], int s) {
  if constexpr (L >= 32) rs_step<16, V, L>(A, (s & 16) != 0);
  if constexpr (L >= 16) rs_step<8, V, L>(A, (s & 8) != 0);
  rs_step<4, V, L>(A, (s & 4) != 0);
  rs_step<2, V, L>(A, (s & 2) != 0);
  rs_step<1, V, L>(A, (s & 1) != 0);
}

// Job of block `blk` among `njobs`: consecutive block indices go to different XCDs (round robin),
// so the jobs are dealt out in eight contiguous ranges, one per XCD, and neighbouring jobs (the
// rows of one head, the heads of one kv group) share one XCD's L2.
__device__ __forceinline__ int64_t xcd_job(int64_t blk, int64_t njobs) {
  return njobs % 8 == 0 ? (blk & 7) * (njobs >> 3) + (blk >> 3) : blk;
}

// Block-wide reductions through a caller-provided LDS scratch of (blockDim.x / 64) entries.
// Every thread of the block must call them; all threads get the result.
template <int NWAVES>
__device__ __forceinline__ double block_max_f64(double x, double* scratch) {
  x = wave_max_f64(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[w] = x;
  __syncthreads();
  double r = scratch[0];
#pragma unroll
  for (int i = 1; i < NWAVES; ++i) r = fmax(r, scratch[i]);
  return r;
}
template <int NWAVES>
__device__ __forceinline__ double block_sum_f64(double x, double* scratch) {
  x = wave_sum_f64(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[w] = x;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) r += scratch[i];
  return r;
}

// The value of lane (lane ^ S) for S = 1 .. 32 without an address computation: DPP quad
// permutes (1, 2), row shifts by 4 chosen by lane bit 2 (4), a row rotation by 8 (8), an LDS
// swizzle (16), and the gfx950 half-wave swap (32; its two results hold, per lane, the values of
// lanes l mod 32 and l mod 32 + 32).
template <int S>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t x) {
  // (every lane reads a lane that exists for 1, 2 and 8; for 4 each lane keeps the shift whose
  // source exists, so the zero that bound_ctrl gives a missing source is never used)
  const int v = (int)x;
  if constexpr (S == 1) return (uint32_t)__builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);
  else if constexpr (S == 2) return (uint32_t)__builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);
  else if constexpr (S == 4) {
    const int up = __builtin_amdgcn_mov_dpp(v, 0x104, 0xF, 0xF, true);  // lane + 4
    const int dn = __builtin_amdgcn_mov_dpp(v, 0x114, 0xF, 0xF, true);  // lane - 4
    return (uint32_t)((threadIdx.x & 4) ? dn : up);
  } else if constexpr (S == 8) return (uint32_t)__builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true);
  else if constexpr (S == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle(v, 0x401F);
  else {
    static_assert(S == 32, "lane_xor_u32: S in 1, 2, 4, 8, 16, 32");
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}
template <int S>
__device__ __forceinline__ float lane_xor_f32(float x) {
  return __uint_as_float(lane_xor_u32<S>(__float_as_uint(x)));
}
__device__ __forceinline__ float wave_sum_fast(float x) {
  x += lane_xor_f32<1>(x);
  x += lane_xor_f32<2>(x);
  x += lane_xor_f32<4>(x);
  x += lane_xor_f32<8>(x);
  x += lane_xor_f32<16>(x);
  x += lane_xor_f32<32>(x);
  return x;
}
__device__ __forceinline__ float wave_max_fast(float x) {
  x = fmaxf(x, lane_xor_f32<1>(x));
  x = fmaxf(x, lane_xor_f32<2>(x));
  x = fmaxf(x, lane_xor_f32<4>(x));
  x = fmaxf(x, lane_xor_f32<8>(x));
  x = fmaxf(x, lane_xor_f32<16>(x));
  x = fmaxf(x, lane_xor_f32<32>(x));
  return x;
}
template <int S>
__device__ __forceinline__ void sort_stage_u32(uint32_t& x, int size) {
  const int lane = threadIdx.x & 63;
  const uint32_t y = lane_xor_u32<S>(x);
  x = (((lane & size) == 0) == ((lane & S) == 0)) ? min(x, y) : max(x, y);
}
// Ascending bitonic sort of one value per lane across the wave, every exchange without LDS
// addresses (see lane_xor_u32).
__device__ __forceinline__ void wave_sort64_asc_u32(uint32_t& x) {
  sort_stage_u32<1>(x, 2);
  sort_stage_u32<2>(x, 4);  sort_stage_u32<1>(x, 4);
  sort_stage_u32<4>(x, 8);  sort_stage_u32<2>(x, 8);  sort_stage_u32<1>(x, 8);
  sort_stage_u32<8>(x, 16); sort_stage_u32<4>(x, 16); sort_stage_u32<2>(x, 16); sort_stage_u32<1>(x, 16);
  sort_stage_u32<16>(x, 32); sort_stage_u32<8>(x, 32); sort_stage_u32<4>(x, 32); sort_stage_u32<2>(x, 32);
  sort_stage_u32<1>(x, 32);
  sort_stage_u32<32>(x, 64); sort_stage_u32<16>(x, 64); sort_stage_u32<8>(x, 64); sort_stage_u32<4>(x, 64);
  sort_stage_u32<2>(x, 64); sort_stage_u32<1>(x, 64);
}


}  // namespace topo
