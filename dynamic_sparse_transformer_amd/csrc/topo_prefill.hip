// Many-query (prefill) path of Topological Attention on gfx950: n_q consecutive queries per
// (batch, query head), query i at position q_pos0 + i.
//
// "The Condensate Theorem: Transformers are O(n), Not O(n^2)" (gist.science explainers of
// arXiv 2602.06317): every query attends to its own condensate set, the anchor (position 0), the
// W most recent tokens and its top-k keys by Q.K^T (zh page, technical summary §3; fr page,
// technical summary §2-§3). Over a whole prompt the scores form the causal Q.K^T triangle, a dense
// contraction, so the scan runs on the matrix cores.
//
// Launches:
//   pf_norms   |q| of every query row and the largest |k| of every kv head (error bounds).
//   pf_scan    bf16 MFMA tiles: 64 query rows x 64 keys per step (4 waves, 32x32x16 MFMA each),
//              float32 scores; per row, an LDS list of the keys that may still be in its top-k,
//              pruned against the row's own k-th best lower bound whenever it fills up.
//   pf_finish  one wave per query row: float64 re-score of the row's list, exact top-k by
//              (score desc, position asc), the set, float64 softmax and V reduction. Rows whose list
//              overflowed (ties), float32 inputs and k above the scan's limit take an exact
//              float64 radix selection over all of the row's candidates instead.
#include "topo_device.h"
#include "topo_internal.h"

namespace topo {

constexpr int PF_ROWS = 64;          // query rows per scan block
constexpr int PF_KEYS = 64;          // keys per scan step
constexpr int PF_MAX_K = 96;         // largest k the MFMA scan ranks
constexpr int PF_LIST = PF_MAX_K + 96;  // per-row LDS list (room for one step after a prune)
constexpr uint32_t PF_OVERFLOW = 0xFFFFFFFFu;

// Error bound of the MFMA float32 scores: products of bf16 values are exact in float32; allowing
// every one of the d terms several roundings of the running sum (whatever the matrix unit's
// internal order and alignment) gives |s_fast - s| <= 2^-14 |q| |k| for d <= 128 with a wide margin.
constexpr float PF_EPS_COEF = 0x1p-14f;

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static int64_t pf_slot(int32_t k) { return (int64_t)k + 32; }

struct PfWs {
  float* qn;        // [B*Hq*n_q]
  uint32_t* knmax;  // [B*Hkv] float bits
  uint32_t* cnt;    // [B*Hq*n_q]
  uint2* surv;      // [B*Hq*n_q][slot]
};

size_t prefill_workspace_bytes(int32_t B, int32_t Hq, int64_t n_q, int64_t, int32_t, int32_t, int32_t k) {
  const size_t rows = (size_t)B * Hq * (size_t)n_q;
  return align256(rows * 4) + align256((size_t)B * Hq * 4) + align256(rows * 4) +
         rows * (size_t)pf_slot(k) * sizeof(uint2);
}

static PfWs pf_carve(void* ws, int32_t B, int32_t Hq, int64_t n_q) {
  const size_t rows = (size_t)B * Hq * (size_t)n_q;
  PfWs w;
  char* p = (char*)ws;
  w.qn = (float*)p;
  p += align256(rows * 4);
  w.knmax = (uint32_t*)p;
  p += align256((size_t)B * Hq * 4);
  w.cnt = (uint32_t*)p;
  p += align256(rows * 4);
  w.surv = (uint2*)p;
  return w;
}

// ---------------------------------------------------------------------------------------------
// pf_norms: one wave per row of Q (rows < nq_rows) or of K (the rest): |row|_2 in float64, rounded
// up to float32. K norms reduce to the max per kv head.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void pf_norms_kernel(const unsigned char* q, const unsigned char* k, float* qn,
                                                       uint32_t* knmax, int64_t nq_rows, int64_t nk_rows, int64_t n) {
  constexpr int RB = D * (BF16 ? 2 : 4);
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= nq_rows + nk_rows) return;
  const bool isq = row < nq_rows;
  const unsigned char* base = isq ? q + (size_t)row * RB : k + (size_t)(row - nq_rows) * RB;
  double s2 = 0.0;
  constexpr int EPL = D / 64;  // elements per lane
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const double x = load_elem_f64<BF16>(base, lane * EPL + e);
    s2 += x * x;
  }
  s2 = wave_sum_f64(s2);
  if (lane == 0) {
    const float nrm = (float)sqrt(s2) * (1.0f + 0x1p-20f);
    if (isq) qn[row] = nrm;
    else atomicMax(&knmax[(row - nq_rows) / n], __float_as_uint(nrm));
  }
}

__global__ void pf_zero_kernel(uint32_t* x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = 0u;
}

// ---------------------------------------------------------------------------------------------
struct PfArgs {
  const unsigned char* q;
  const unsigned char* k;
  const unsigned char* v;
  float* out;
  int32_t* sel_idx;
  int32_t* sel_count;
  PfWs w;
  int64_t n, n_q, q_pos0, slot, rows;
  int32_t Hq, Hkv, G, W, topk, causal, set_cap, exact_all;
  double scale;
  size_t wave_smem;  // bytes of LDS per wave in pf_finish
};

__device__ __forceinline__ bool pf_is_cand(int64_t j, int64_t p, int64_t n, int32_t W, int32_t causal) {
  const int64_t vis_hi = causal ? p : n - 1;
  const int64_t w_lo = p - W + 1 > 0 ? p - W + 1 : 0;
  return j >= 1 && j <= vis_hi && (j < w_lo || j > p);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// pf_scan: grid (ceil(n_q / 64), B*Hq), 256 threads. Wave w computes the 32x32 quadrant
// (rows 32*(w/2).., keys 32*(w%2)..) of each 64x64 score tile with v_mfma_f32_32x32x16_bf16:
// lane l supplies row / key (l % 32) and elements 8*(l/32) .. +8 of each 16-deep slice, and holds
// output (row 8*(r/4) + 4*(l/32) + r%4, key l % 32) in register r.
template <int D>
__global__ __launch_bounds__(256) void pf_scan_kernel(PfArgs a) {
  constexpr int RB = D * 2;
  constexpr int STEPS = D / 16;
  __shared__ uint2 list[PF_ROWS][PF_LIST];
  __shared__ int lcnt[PF_ROWS];
  __shared__ uint32_t lth[PF_ROWS];   // per-row threshold (order key of a lower bound)
  __shared__ float leps[PF_ROWS];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int bh = blockIdx.y;
  const int b = bh / a.Hq, h = bh - b * a.Hq, g = h / a.G;
  const int64_t i0 = (int64_t)blockIdx.x * PF_ROWS;
  const unsigned char* kb = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.n * RB;
  const float knmax = __uint_as_float(a.w.knmax[(size_t)b * a.Hkv + g]);

  if (tid < PF_ROWS) {
    lcnt[tid] = 0;
    lth[tid] = 0u;
    const int64_t i = i0 + tid;
    leps[tid] = i < a.n_q ? PF_EPS_COEF * a.w.qn[(size_t)bh * a.n_q + i] * knmax + 1e-30f : 0.f;
  }

  const int rq = wave >> 1, kq = wave & 1;
  const int m = lane & 31, half = lane >> 5;
  // A operand: this lane's query row, all K-slices.
  bf16x8_t qa[STEPS];
  {
    const int64_t i = i0 + rq * 32 + m;
    const unsigned char* qrow = a.q + ((size_t)bh * a.n_q + (i < a.n_q ? i : 0)) * RB;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const uint4 w = i < a.n_q ? *(const uint4*)(qrow + st * 32 + half * 16) : make_uint4(0u, 0u, 0u, 0u);
      qa[st] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  // Row positions held by this lane (register r): block row rq*32 + 8*(r/4) + 4*half + r%4.
  int64_t pos[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) pos[r] = a.q_pos0 + i0 + rq * 32 + 8 * (r / 4) + 4 * half + (r % 4);

  // Keys to scan: up to the last candidate of the block's last row.
  const int64_t i_last = min(i0 + PF_ROWS, a.n_q) - 1;
  const int64_t p_last = a.q_pos0 + i_last;
  const int64_t key_hi = a.causal ? p_last - a.W : a.n - 1;
  __syncthreads();

  for (int64_t kt0 = 0; kt0 <= key_hi; kt0 += PF_KEYS) {
    const int64_t j = kt0 + kq * 32 + m;  // key of this lane's B operand and output column
    f32x16_t acc = {};
    {
      const unsigned char* krow = kb + (size_t)(j < a.n ? j : a.n - 1) * RB;
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        const uint4 w = *(const uint4*)(krow + st * 32 + half * 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[st], __builtin_bit_cast(bf16x8_t, w), acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rq * 32 + 8 * (r / 4) + 4 * half + (r % 4);
      const bool ok = i0 + row < a.n_q && pf_is_cand(j, pos[r], a.n, a.W, a.causal) &&
                      ord_f32(acc[r] + leps[row]) >= lth[row];
      if (ok) {
        const int slot = atomicAdd(&lcnt[row], 1);
        if (slot < PF_LIST) list[row][slot] = make_uint2(__float_as_uint(acc[r]), (uint32_t)j);
      }
    }
    __syncthreads();
    // Prune the lists that may not hold another step: wave w takes rows w, w+4, ...
    for (int row = wave; row < PF_ROWS; row += 4) {
      const int c = lcnt[row];
      if (c <= PF_LIST - PF_KEYS) continue;
      const float eps = leps[row];
      constexpr int PER = PF_LIST / 64;
      uint2 e[PER];
      uint32_t lb[PER];
#pragma unroll
      for (int t = 0; t < PER; ++t) {
        const int idx = lane + 64 * t;
        e[t] = idx < c ? list[row][idx] : make_uint2(0u, 0u);
        lb[t] = idx < c ? ord_f32(__uint_as_float(e[t].x) - eps) : 0u;
      }
      const uint32_t T = wave_kth_largest<PER>(lb, a.topk);
      const uint32_t th = max(T, lth[row]);
      int nc = 0;
#pragma unroll
      for (int t = 0; t < PER; ++t) {
        const int idx = lane + 64 * t;
        const bool keep = idx < c && ord_f32(__uint_as_float(e[t].x) + eps) >= th;
        const uint64_t mk = __ballot(keep);
        if (keep) list[row][nc + lanes_below(mk)] = e[t];
        nc += __popcll(mk);
      }
      if (lane == 0) {
        lcnt[row] = c > PF_LIST ? (int)PF_LIST + 1 : nc;  // more than the list held: overflow
        lth[row] = th;
      }
    }
    __syncthreads();
  }

  // Final prune and hand-over: wave w writes rows w, w+4, ...
  for (int row = wave; row < PF_ROWS; row += 4) {
    const int64_t i = i0 + row;
    if (i >= a.n_q) continue;
    const size_t grow = (size_t)bh * a.n_q + i;
    const int c = lcnt[row];
    if (c > PF_LIST) {
      if (lane == 0) a.w.cnt[grow] = PF_OVERFLOW;
      continue;
    }
    const float eps = leps[row];
    constexpr int PER = PF_LIST / 64;
    uint2 e[PER];
    uint32_t lb[PER];
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      const int idx = lane + 64 * t;
      e[t] = idx < c ? list[row][idx] : make_uint2(0u, 0u);
      lb[t] = idx < c ? ord_f32(__uint_as_float(e[t].x) - eps) : 0u;
    }
    const uint32_t T = c > a.topk ? wave_kth_largest<PER>(lb, a.topk) : 0u;
    const uint32_t th = max(T, lth[row]);
    uint2* out = a.w.surv + grow * (size_t)a.slot;
    int nc = 0;
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      const int idx = lane + 64 * t;
      const bool keep = idx < c && ord_f32(__uint_as_float(e[t].x) + eps) >= th;
      const uint64_t mk = __ballot(keep);
      if (keep && nc + lanes_below(mk) < a.slot) out[nc + lanes_below(mk)] = e[t];
      nc += __popcll(mk);
    }
    if (lane == 0) a.w.cnt[grow] = nc > a.slot ? PF_OVERFLOW : (uint32_t)nc;
  }
}

// ---------------------------------------------------------------------------------------------
// pf_finish: one wave per query row (4 rows per 256-thread block), each wave with its own LDS
// region laid out by PfRowSmem::carve for the call's k and 1 + W + k.
constexpr int PF_FIN_SET = 4096;   // largest 1 + W + k served by the per-row finish
struct PfRowSmem {
  double* qd;      // [128]
  int32_t* ridx;   // [slot]
  double* rs;      // [slot]
  int32_t* tidx;   // [k]
  double* ts;      // [k]
  int32_t* cidx;   // [set_cap]
  double* cw;      // [set_cap]
  uint32_t* hist;  // [256]
  static __host__ __device__ size_t bytes(int64_t slot, int k, int set_cap) {
    const size_t kk = (size_t)(k > 0 ? k : 1);
    return 128 * 8 + (size_t)slot * 12 + kk * 12 + (size_t)set_cap * 12 + 256 * 4 + 64;
  }
  __device__ void carve(unsigned char* p, int64_t slot, int k, int set_cap) {
    const size_t kk = (size_t)(k > 0 ? k : 1);
    qd = (double*)p;
    p += 128 * 8;
    rs = (double*)p;
    p += (size_t)slot * 8;
    ts = (double*)p;
    p += kk * 8;
    cw = (double*)p;
    p += (size_t)set_cap * 8;
    ridx = (int32_t*)p;
    p += (size_t)slot * 4;
    tidx = (int32_t*)p;
    p += kk * 4;
    cidx = (int32_t*)p;
    p += (size_t)set_cap * 4;
    hist = (uint32_t*)(((uintptr_t)p + 15) & ~(uintptr_t)15);
  }
};

template <int D, bool BF16>
__device__ __forceinline__ double pf_score(const double* qd, const unsigned char* kb, int64_t j) {
  constexpr int RB = D * (BF16 ? 2 : 4);
  return canonical_score<BF16, D>(qd, kb + (size_t)j * RB);
}

// Exact top-k of one row over all of its candidates (one wave): 8-pass float64 radix select,
// then the keys above the k-th value and the lowest positions among those equal to it. Writes
// the chosen (position, score) pairs to sm->tidx / sm->ts and returns their number.
template <int D, bool BF16>
__device__ int pf_exact_row(PfRowSmem* sm, const PfArgs& a, const unsigned char* kb, int64_t p) {
  const int lane = threadIdx.x & 63;
  const int64_t vis_hi = a.causal ? p : a.n - 1;
  // candidates counted first: if at most k, take them all
  int nc = 0;
  for (int64_t j0 = 1; j0 <= vis_hi; j0 += 64) nc += __popcll(__ballot(j0 + lane <= vis_hi && pf_is_cand(j0 + lane, p, a.n, a.W, a.causal)));
  const bool take_all = nc <= a.topk;
  uint64_t prefix = 0;
  int need = a.topk;
  if (!take_all) {
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      for (int i = lane; i < 256; i += 64) sm->hist[i] = 0;
      __builtin_amdgcn_wave_barrier();
      for (int64_t j0 = 1; j0 <= vis_hi; j0 += 64) {
        const int64_t j = j0 + lane;
        if (j <= vis_hi && pf_is_cand(j, p, a.n, a.W, a.causal)) {
          const uint64_t key = ord_f64(pf_score<D, BF16>(sm->qd, kb, j));
          if (pass == 0 || (key >> (shift + 8)) == prefix) atomicAdd(&sm->hist[(key >> shift) & 255u], 1u);
        }
      }
      __builtin_amdgcn_wave_barrier();
      // bin (from the top) where the running count reaches need
      int64_t above = 0;
      int found = -1;
      for (int top = 255; top >= 0 && found < 0; top -= 64) {
        const int c = (int)sm->hist[top - lane];
        const int incl = wave_incl_scan_i32(c);
        const uint64_t hit = __ballot(above + incl >= need && c > 0);
        if (hit) {
          const int l = __builtin_ctzll(hit);
          above += __shfl(incl - c, l);
          found = top - l;
        } else {
          above += __shfl(incl, 63);
        }
      }
      prefix = (prefix << 8) | (uint64_t)(found < 0 ? 0 : found);
      need -= (int)above;
      __builtin_amdgcn_wave_barrier();
    }
  }
  int nt = 0, eq_seen = 0;
  for (int64_t j0 = 1; j0 <= vis_hi; j0 += 64) {
    const int64_t j = j0 + lane;
    const bool isc = j <= vis_hi && pf_is_cand(j, p, a.n, a.W, a.causal);
    double s = 0.0;
    bool gt = false, eq = false;
    if (isc) {
      s = pf_score<D, BF16>(sm->qd, kb, j);
      const uint64_t key = ord_f64(s);
      gt = take_all || key > prefix;
      eq = !take_all && key == prefix;
    }
    const uint64_t em = __ballot(eq);
    const bool take = gt || (eq && eq_seen + lanes_below(em) < need);
    const uint64_t tm = __ballot(take);
    if (take) {
      const int pos = nt + lanes_below(tm);
      sm->tidx[pos] = (int32_t)j;
      sm->ts[pos] = s;
    }
    nt += __popcll(tm);
    eq_seen += __popcll(em);
  }
  __builtin_amdgcn_wave_barrier();
  return nt;
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void pf_finish_kernel(PfArgs a) {
  constexpr int RB = D * (BF16 ? 2 : 4);
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  PfRowSmem smv;
  smv.carve(smem_raw + wave * a.wave_smem, a.slot, a.topk, a.set_cap);
  PfRowSmem* sm = &smv;
  const size_t grow = (size_t)blockIdx.x * 4 + wave;  // (b*Hq + h) * n_q + i
  if (grow >= (size_t)a.rows) return;
  const size_t bh = grow / (size_t)a.n_q;
  const int64_t i = (int64_t)(grow - bh * (size_t)a.n_q);
  const int b = (int)(bh / a.Hq), h = (int)(bh - (size_t)b * a.Hq), g = h / a.G;
  const unsigned char* kb = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.n * RB;
  const unsigned char* vb = a.v ? a.v + ((size_t)b * a.Hkv + g) * (size_t)a.n * RB : nullptr;
  const int64_t p = a.q_pos0 + i;
  const unsigned char* qrow = a.q + grow * RB;
  for (int t = lane; t < D; t += 64) sm->qd[t] = load_elem_f64<BF16>(qrow, t);
  __builtin_amdgcn_wave_barrier();

  // ---- the top-k part
  int nt = 0;
  if (a.topk > 0) {
    const uint32_t c = a.exact_all ? PF_OVERFLOW : a.w.cnt[grow];
    bool exact = c == PF_OVERFLOW;
    if (!exact) {
      const uint2* sv = a.w.surv + grow * (size_t)a.slot;
      for (uint32_t t = lane; t < c; t += 64) {
        const int32_t j = (int32_t)sv[t].y;
        sm->ridx[t] = j;
        sm->rs[t] = pf_score<D, BF16>(sm->qd, kb, j);
      }
      __builtin_amdgcn_wave_barrier();
      // exact rank among the list: higher score first, then lower position. The list holds
      // every key of the row's top-k (or all of its candidates when it has at most k).
      for (uint32_t t = lane; t < c; t += 64) {
        const double si = sm->rs[t];
        const int32_t ji = sm->ridx[t];
        int rank = 0;
        for (uint32_t r = 0; r < c; ++r) rank += (sm->rs[r] > si) || (sm->rs[r] == si && sm->ridx[r] < ji);
        if (rank < a.topk) {
          sm->tidx[rank] = ji;
          sm->ts[rank] = si;
        }
      }
      nt = (int)min(c, (uint32_t)a.topk);
      __builtin_amdgcn_wave_barrier();
    } else {
      nt = pf_exact_row<D, BF16>(sm, a, kb, p);
    }
  }

  // ---- set: {0} u window u T, ascending
  const int64_t w_lo = p - a.W + 1 > 0 ? p - a.W + 1 : 0;
  const int anchor = w_lo > 0 ? 1 : 0;
  const int nwin = (int)(p - w_lo + 1);
  const int count = anchor + nwin + nt;
  int tlo = 0;
  for (int t = lane; t < nt; t += 64) tlo += sm->tidx[t] < w_lo;
  tlo = wave_sum_i32(tlo);
  if (anchor && lane == 0) {
    sm->cidx[0] = 0;
    sm->cw[0] = pf_score<D, BF16>(sm->qd, kb, 0);
  }
  for (int t = lane; t < nt; t += 64) {
    const int32_t j = sm->tidx[t];
    int below = 0;
    for (int r = 0; r < nt; ++r) below += sm->tidx[r] < j;
    const int pos = anchor + below + (j > p ? nwin : 0);
    sm->cidx[pos] = j;
    sm->cw[pos] = sm->ts[t];
  }
  for (int t = lane; t < nwin; t += 64) {
    const int pos = anchor + tlo + t;
    sm->cidx[pos] = (int32_t)(w_lo + t);
    sm->cw[pos] = pf_score<D, BF16>(sm->qd, kb, w_lo + t);
  }
  __builtin_amdgcn_wave_barrier();
  if (a.sel_idx) {
    int32_t* dst = a.sel_idx + grow * (size_t)a.set_cap;
    for (int t = lane; t < a.set_cap; t += 64) dst[t] = t < count ? sm->cidx[t] : -1;
  }
  if (a.sel_count && lane == 0) a.sel_count[grow] = count;
  if (!a.out) return;

  // ---- float64 softmax over the set and the weighted V rows (lane: D/64 columns)
  double zmax = -INFINITY;
  for (int t = lane; t < count; t += 64) zmax = fmax(zmax, a.scale * sm->cw[t]);
  zmax = wave_max_f64(zmax);
  double zsum = 0.0;
  for (int t = lane; t < count; t += 64) {
    const double w = exp(a.scale * sm->cw[t] - zmax);
    sm->cw[t] = w;
    zsum += w;
  }
  zsum = wave_sum_f64(zsum);
  __builtin_amdgcn_wave_barrier();
  constexpr int CPL = D / 64;
  constexpr int BATCH = 16;
  double acc[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) acc[e] = 0.0;
  for (int t0 = 0; t0 < count; t0 += BATCH) {
    double x[BATCH][CPL];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int t = t0 + u;
#pragma unroll
      for (int e = 0; e < CPL; ++e)
        x[u][e] = t < count ? load_elem_f64<BF16>(vb + (size_t)sm->cidx[t] * RB, lane * CPL + e) : 0.0;
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int t = t0 + u;
      const double w = t < count ? sm->cw[t] : 0.0;
#pragma unroll
      for (int e = 0; e < CPL; ++e) acc[e] = fma(w, x[u][e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < CPL; ++e) a.out[grow * D + lane * CPL + e] = (float)(acc[e] / zsum);
}

// ---------------------------------------------------------------------------------------------
template <int D, bool BF16>
static hipError_t launch_pf_t(const PrefillLaunch& L, const PfArgs& pa, hipStream_t s) {
  const size_t rows = (size_t)L.B * L.Hq * (size_t)L.n_q;
  // norms and zeroed kv-head maxima
  hipLaunchKernelGGL(pf_zero_kernel, dim3((unsigned)((L.B * L.Hkv + 255) / 256)), dim3(256), 0, s, pa.w.knmax,
                     (int64_t)L.B * L.Hkv);
  const int64_t nk_rows = (int64_t)L.B * L.Hkv * L.n;
  const int64_t tot = (int64_t)rows + nk_rows;
  hipLaunchKernelGGL((pf_norms_kernel<D, BF16>), dim3((unsigned)((tot + 3) / 4)), dim3(256), 0, s,
                     (const unsigned char*)L.q, (const unsigned char*)L.k, pa.w.qn, pa.w.knmax, (int64_t)rows, nk_rows,
                     L.n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!pa.exact_all) {
    if constexpr (BF16) {
      hipLaunchKernelGGL((pf_scan_kernel<D>), dim3((unsigned)((L.n_q + PF_ROWS - 1) / PF_ROWS), (unsigned)(L.B * L.Hq)),
                         dim3(256), 0, s, pa);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  const size_t smem = 4 * pa.wave_smem;
  if (smem > 48 * 1024)
    (void)hipFuncSetAttribute((const void*)pf_finish_kernel<D, BF16>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)smem);
  hipLaunchKernelGGL((pf_finish_kernel<D, BF16>), dim3((unsigned)((rows + 3) / 4), 1), dim3(256), smem, s, pa);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillLaunch& L, hipStream_t stream) {
  if (1 + L.W + L.topk > PF_FIN_SET) return hipErrorNotSupported;
  PfArgs pa;
  pa.q = (const unsigned char*)L.q;
  pa.k = (const unsigned char*)L.k;
  pa.v = (const unsigned char*)L.v;
  pa.out = L.out;
  pa.sel_idx = L.sel_idx;
  pa.sel_count = L.sel_count;
  pa.w = pf_carve(L.ws, L.B, L.Hq, L.n_q);
  pa.n = L.n;
  pa.n_q = L.n_q;
  pa.q_pos0 = L.q_pos0;
  pa.slot = pf_slot(L.topk);
  pa.Hq = L.Hq;
  pa.Hkv = L.Hkv;
  pa.G = L.G;
  pa.W = L.W;
  pa.topk = L.topk;
  pa.causal = L.causal;
  pa.set_cap = 1 + L.W + L.topk;
  pa.exact_all = (!L.bf16 || L.topk > PF_MAX_K || (L.flags & 1)) ? 1 : 0;
  pa.scale = L.scale;
  pa.rows = (int64_t)L.B * L.Hq * L.n_q;
  pa.wave_smem = (PfRowSmem::bytes(pa.slot, L.topk, pa.set_cap) + 255) & ~(size_t)255;
  if (4 * pa.wave_smem > 160 * 1024) return hipErrorNotSupported;
  if (L.bf16) return L.d == 128 ? launch_pf_t<128, true>(L, pa, stream) : launch_pf_t<64, true>(L, pa, stream);
  return L.d == 128 ? launch_pf_t<128, false>(L, pa, stream) : launch_pf_t<64, false>(L, pa, stream);
}

}  // namespace topo
