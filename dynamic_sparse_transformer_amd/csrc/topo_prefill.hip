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
//   pf_scan    bf16 MFMA tiles, 128 query rows x 64 keys per step (8 waves, one 32x32x16 tile
//              each), float32 scores, two passes over the keys: the first bounds each row's k-th
//              best score from below, the second lists every key that may still reach it.
//   pf_window  matrix-core softmax share of every row's window (max, sum, weighted V).
//   pf_finish  one wave per query row: top-k from the list's scores with their error band,
//              float64 canonical scores where the band leaves the top-k open, the set, softmax
//              and V reduction over anchor and top-k, merged with the window's share. Rows
//              whose list overflowed (ties), float32 inputs and k above the scan's limit take
//              an exact float64 radix selection over all of the row's candidates instead.
#include "topo_device.h"
#include "topo_internal.h"

namespace topo {

constexpr int PF_ROWS = 128;         // query rows per scan block (8 waves: 4 row groups x 2 key halves)
constexpr int PF_KEYS = 64;          // keys per scan step
constexpr int PF_MAX_K = 96;         // largest k the MFMA scan ranks
constexpr uint32_t PF_OVERFLOW = 0xFFFFFFFFu;

// Error bound of the MFMA float32 scores: products of bf16 values are exact in float32; allowing
// every one of the d terms several roundings of the running sum (whatever the matrix unit's
// internal order and alignment) gives |s_fast - s| <= 2^-14 |q| |k| for d <= 128 with a wide margin.
constexpr float PF_EPS_COEF = 0x1p-14f;

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// LDS of the scan for the top-2 values of each row's lanes (phase 1), then for the waves' score
// stages (phase 2). A row's list of possible top-k keys holds k + 48 entries, at most 128 (the
// finish ranks two per lane).
constexpr int PF_LIST_BYTES = PF_ROWS * 128 * 4;
constexpr int PF_LCAP_MAX = 128;
static int64_t pf_slot(int32_t k) { return k + 48 < PF_LCAP_MAX ? k + 48 : PF_LCAP_MAX; }

struct PfWs {
  float* qn;        // [B*Hq*n_q]
  uint32_t* knmax;  // [B*Hkv] float bits
  uint32_t* cnt;    // [B*Hq*n_q]: entries of the row's list (or PF_OVERFLOW)
  uint2* surv;      // [B*Hq*n_q][list]: (float bits of the matrix-core score, key position)
  float* win_o;     // [B*Hq*n_q][d]: sum over the row's window of exp(z - m_w) v (bf16 inputs)
  float2* win_mz;   // [B*Hq*n_q]: (m_w, sum over the window of exp(z - m_w))
};

size_t prefill_workspace_bytes(int32_t B, int32_t Hq, int64_t n_q, int64_t, int32_t d, int32_t, int32_t k) {
  const size_t rows = (size_t)B * Hq * (size_t)n_q;
  return align256(rows * 4) + align256((size_t)B * Hq * 4) + align256(rows * 4) +
         align256(rows * (size_t)pf_slot(k) * sizeof(uint2)) + align256(rows * (size_t)d * 4) + rows * 8;
}

static PfWs pf_carve(void* ws, int32_t B, int32_t Hq, int64_t n_q, int32_t d, int32_t k) {
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
  p += align256(rows * (size_t)pf_slot(k) * sizeof(uint2));
  w.win_o = (float*)p;
  p += align256(rows * (size_t)d * 4);
  w.win_mz = (float2*)p;
  return w;
}

// ---------------------------------------------------------------------------------------------
// Norms of bf16 rows for the error bounds of the matrix-core scores: |q| of every query row and
// the largest |k| of every kv head. A row is LPR lanes x 16 bytes (coalesced, RPW rows per load
// instruction). The squares of bf16 values are exact in float32; their float32 sum (8 terms per
// lane, then a tree over the LPR lanes) and sqrtf carry a relative error far below the factor
// (1 + 2^-15) that rounds the norm up. Grid (blocks over the rows of a head, heads); with
// `norm` every row's norm is written, with `head_max` one atomicMax per block into its head
// (U rows per lane, large for this use: the atomics of all blocks meet on one cache line). Block
// (0, 0) also clears the `nzero` words at `zero` (the head maxima of the launch that follows).
template <int D, int U>
__global__ __launch_bounds__(256) void pf_norm_kernel(const unsigned char* x, int64_t rows_per_head, float* norm,
                                                      uint32_t* head_max, uint32_t* zero, int nzero) {
  constexpr int RB = D * 2, LPR = RB / 16, RPW = 64 / LPR;
  __shared__ float wm[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, gq = lane / LPR, cc = lane % LPR;
  const unsigned char* base = x + (size_t)blockIdx.y * (size_t)rows_per_head * RB;
  const int64_t r0 = (int64_t)blockIdx.x * (4 * U * RPW) + (int64_t)wave * U * RPW + gq;
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t row = r0 + u * RPW;
    v[u] = row < rows_per_head ? *(const uint4*)(base + (size_t)row * RB + cc * 16) : make_uint4(0u, 0u, 0u, 0u);
  }
  if (zero && blockIdx.x == 0 && blockIdx.y == 0)
    for (int t = threadIdx.x; t < nzero; t += 256) zero[t] = 0u;
  float mx = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    float s2 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = bf16_lo(w4[e]), hi = bf16_hi(w4[e]);
      s2 = fmaf(lo, lo, s2);
      s2 = fmaf(hi, hi, s2);
    }
    s2 = group_sum_f32<LPR>(s2);
    const float nrm = sqrtf(s2) * (1.0f + 0x1p-15f);
    const int64_t row = r0 + u * RPW;
    if (norm && cc == 0 && row < rows_per_head) norm[(size_t)blockIdx.y * rows_per_head + row] = nrm;
    mx = fmaxf(mx, nrm);
  }
  if (head_max) {
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) wm[wave] = mx;
    __syncthreads();
    if (threadIdx.x == 0) atomicMax(&head_max[blockIdx.y], __float_as_uint(fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]))));
  }
}

// Sum, maximum or minimum over each row of 16 lanes, in every lane of the row (DPP: quad swaps,
// half-row and row mirrors).
template <int CTRL, typename T>
__device__ __forceinline__ T pf_dpp(T y) {
  return __builtin_bit_cast(T, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, y), CTRL, 0xF, 0xF, false));
}
template <int OP, typename T>
__device__ __forceinline__ T pf_row16(T x) {
  const auto f = [](T p, T q) { return OP == 0 ? p + q : OP == 1 ? (p > q ? p : q) : (p < q ? p : q); };
  x = f(x, pf_dpp<0xB1>(x));
  x = f(x, pf_dpp<0x4E>(x));
  x = f(x, pf_dpp<0x141>(x));
  x = f(x, pf_dpp<0x140>(x));
  return x;
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
  int32_t win;  // 1: the window kernel has left (m_w, Z_w, O_w) of every row in the workspace
  float pinf;   // +inf (a run-time operand of the scan's medians)
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

// pf_scan: one block of 512 threads per (b, h, 128 consecutive query rows). Each step scores 64
// keys held in LDS (padded rows, two buffers) while the loads of the key tile two steps ahead are
// in flight and the tile one step ahead is written to the other buffer. Wave w computes the
// 32x32 quadrant (rows 32*(w/2).., keys 32*(w%2)..) with v_mfma_f32_32x32x16_bf16: lane l
// supplies row / key (l % 32) and elements 8*(l/32) .. +8 of each 16-deep slice, and holds output
// (row 8*(r/4) + 4*(l/32) + r%4, key l % 32) in register r.
// Phase 1 keeps, per lane and row, the two largest fast scores it has seen. Those 128 values per
// row belong to distinct candidate keys, so their k-th largest x_k gives the bound T = x_k - eps
// below the row's k-th largest exact score. Phase 2 scores the keys again and appends the
// position of every key whose upper bound reaches T (fast score >= x_k - 2 eps) to the row's list
// in LDS; the lists are copied out at the end, and the finish ranks them.

template <int D>
__global__ __launch_bounds__(512) void pf_scan_kernel(PfArgs a) {
  constexpr int RB = D * 2;
  constexpr int STEPS = D / 16;
  constexpr int NCH = RB / 16;            // 16-byte chunks per key row
  constexpr int STRIDE = RB + 16;         // padded LDS row
  constexpr int RPP = 512 / NCH;          // key rows staged per load pass
  constexpr int PASSES = PF_KEYS / RPP;
  constexpr int TILE_BYTES = PF_KEYS * STRIDE;
  static_assert(PASSES >= 1 && PASSES <= 2, "staging passes");
  __shared__ __align__(16) unsigned char ktiles[2 * TILE_BYTES];
  __shared__ __align__(16) unsigned char lists[PF_LIST_BYTES];
  __shared__ uint32_t lcnt[PF_ROWS];  // keys appended to each row's list
  __shared__ float lthf[PF_ROWS];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // Job of this block (the blocks of one head on one XCD). Within a head the row blocks run from
  // the last (most keys under a causal mask) to the first, so the long jobs start first.
  const int64_t nrb = (a.n_q + PF_ROWS - 1) / PF_ROWS;
  const int64_t job = xcd_job(blockIdx.x, nrb * a.Hq * (a.rows / (a.n_q * a.Hq)));
  const int bh = (int)(job / nrb);
  const int b = bh / a.Hq, h = bh - b * a.Hq, g = h / a.G;
  const int64_t i0 = (nrb - 1 - (job - (int64_t)bh * nrb)) * PF_ROWS;
  const unsigned char* kb = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.n * RB;
  const float knmax = __uint_as_float(a.w.knmax[(size_t)b * a.Hkv + g]);
  const uint32_t LCAP = (uint32_t)a.slot;
  // phase 2 stages each wave's 16 scores per lane here (where the top-2 values were): chunk q
  // (registers 4q..4q+3) of lane l at float4 index q * 64 + l of the wave's 4 KB
  float4* sst = (float4*)lists + wave * 256;
  const size_t grow0 = (size_t)bh * a.n_q + i0;  // global row of block row 0
  const int n = (int)a.n;  // the host runs this scan only when n * RB < 2^31

  const int rq = wave >> 1, kq = wave & 1;
  const int m = lane & 31, half = lane >> 5;
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
  const int row_base = rq * 32 + 4 * half;  // block row of register r: row_base + 8*(r/4) + r%4

  const int64_t i_last = min(i0 + PF_ROWS, a.n_q) - 1;
  const int64_t p_first = a.q_pos0 + i0, p_last = a.q_pos0 + i_last;
  const int64_t key_hi = a.causal ? p_last - a.W : a.n - 1;
  const int ntiles = key_hi >= 0 ? (int)(key_hi / PF_KEYS) + 1 : 0;
  // Interior tiles (every key a candidate of every row of the block): 1 <= t <= t_a (all keys
  // before every row's window) or, without the causal mask, t_b <= t <= t_c (all keys after
  // every row's position, inside the cache). Other tiles mask each register by its own test.
  const bool full_rows = i0 + PF_ROWS <= a.n_q;
  const int64_t ea = p_first - a.W - (PF_KEYS - 1);
  const int t_a = full_rows && ea >= 0 ? (int)(ea / PF_KEYS) : -1;
  const int t_b = (int)(p_last / PF_KEYS) + 1, t_c = full_rows && !a.causal ? n / PF_KEYS - 1 : -1;
#define PF_INTERIOR(t) ((t) >= 1 && ((t) <= t_a || ((t) >= t_b && (t) <= t_c)))

  // Staging of key tiles: thread tid copies 16-byte chunk (tid % NCH) of key rows
  // u * PF_KEYS + tid / NCH (+ RPP). Raw buffer loads whose range ends at the cache's last key:
  // rows past the end read as zero, so every load is issued unconditionally and no address is
  // clamped. Register set (u & 1) holds tile u from its load until its store two steps later.
  const int srow = tid / NCH, schunk = tid % NCH;
  const int voff0 = srow * RB + schunk * 16, voff1 = voff0 + RPP * RB;
  uint4 r00 = make_uint4(0u, 0u, 0u, 0u), r01 = r00, r10 = r00, r11 = r00;
#define PF_LOAD(DST0, DST1, U)                                                                     \
  {                                                                                                \
    const int kt_ = min((U) * PF_KEYS, n);                                                         \
    const __amdgpu_buffer_rsrc_t rs_ =                                                             \
        __builtin_amdgcn_make_buffer_rsrc((void*)(kb + (size_t)kt_ * RB), (short)0, (n - kt_) * RB, 0x00020000); \
    DST0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_, voff0, 0, 0));    \
    if (PASSES > 1) DST1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_, voff1, 0, 0)); \
  }
#define PF_STORE(SRC0, SRC1, U)                                                                    \
  {                                                                                                \
    unsigned char* dst = &ktiles[((U) & 1) * TILE_BYTES + srow * STRIDE + schunk * 16];            \
    *(uint4*)dst = SRC0;                                                                           \
    if (PASSES > 1) *(uint4*)(dst + RPP * STRIDE) = SRC1;                                          \
  }
// Prologue of a pass over the tiles: tiles 0 and 1 to LDS, tiles 2 and 3 in flight, scores of
// tile 0 into ACC.
#define PF_PROLOGUE(ACC)                                                                           \
  PF_LOAD(r00, r01, 0)                                                                             \
  PF_LOAD(r10, r11, 1)                                                                             \
  PF_STORE(r00, r01, 0)                                                                            \
  PF_STORE(r10, r11, 1)                                                                            \
  PF_LOAD(r00, r01, 2)                                                                             \
  PF_LOAD(r10, r11, 3)                                                                             \
  __syncthreads();                                                                                 \
  PF_MMA(ACC, 0)
// Scores of the tile in LDS buffer BUF into ACC: v_mfma_f32_32x32x16_bf16 over the D / 16 slices.
#define PF_MMA(ACC, BUF)                                                                           \
  {                                                                                                \
    const unsigned char* krow = &ktiles[(BUF) * TILE_BYTES + (kq * 32 + m) * STRIDE + half * 16]; \
    uint4 kf[STEPS];                                                                               \
    _Pragma("unroll") for (int st = 0; st < STEPS; ++st) kf[st] = *(const uint4*)(krow + st * 32); \
    ACC = f32x16_t{};                                                                              \
    _Pragma("unroll") for (int st = 0; st < STEPS; ++st)                                           \
      ACC = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[st], __builtin_bit_cast(bf16x8_t, kf[st]), ACC, 0, 0, 0); \
  }
// On a boundary tile, scores of keys that are not candidates of the register's row become -inf.
// With dr = (position of the register's row) - j, key j is a candidate of the row iff
// 1 <= j < n, the row exists, and dr >= W (j before the window) or, without the causal mask,
// dr < 0 (j after p).
  const int rows_valid = (int)min((int64_t)PF_ROWS, a.n_q - i0);
// (Positions fit in 32 bits here: the scan runs only when n * RB < 2^31. The tests combine with
// & and |, so that the 16 selects need no branches.)
  const int p_first32 = (int)p_first, rv_ = rows_valid - row_base;
  const bool ncausal_ = !a.causal;
#define PF_MASK(ACC, t)                                                                            \
  if (!PF_INTERIOR(t)) {                                                                           \
    const int j_ = (t) * PF_KEYS + kq * 32 + m;                                                    \
    const int dl = p_first32 + row_base - j_;                                                      \
    const bool jok = (j_ >= 1) & (j_ < n);                                                         \
    const int wl = a.W - dl;                                                                       \
    _Pragma("unroll") for (int r = 0; r < 16; ++r) {                                               \
      const int o = 8 * (r / 4) + (r % 4);                                                         \
      const bool cand = jok & (o < rv_) & ((o >= wl) | (ncausal_ & (o < -dl)));                    \
      ACC[r] = cand ? ACC[r] : -INFINITY;                                                          \
    }                                                                                              \
  }
// One step t of a pass: the scores of tile t are in ACC_CUR (issued a step earlier); the matrix
// cores score tile t+1 into ACC_NEXT while the vector units run the per-score work on tile t: PART
// for each register of ACC_CUR, 16 / STEPS of them after each matrix instruction, then POST. Tile
// t+2 then goes from its registers to the LDS buffer that tile t used and tile t+4 is requested.
// Scheduling fences keep that order: left to itself the compiler puts the vector work before the
// matrix instructions, and as the waves of a block meet at every barrier, the two waves of a
// SIMD would then take turns on the matrix core instead of overlapping.
#define PF_STEP(PART, POST, t, ACC_CUR, ACC_NEXT, SET0, SET1)                                      \
  PF_MASK(ACC_CUR, t)                                                                              \
  {                                                                                                \
    const unsigned char* krow = &ktiles[(((t) + 1) & 1) * TILE_BYTES + (kq * 32 + m) * STRIDE + half * 16]; \
    uint4 kf[STEPS];                                                                               \
    _Pragma("unroll") for (int st = 0; st < STEPS; ++st) kf[st] = *(const uint4*)(krow + st * 32); \
    __builtin_amdgcn_sched_barrier(0);                                                             \
    ACC_NEXT = f32x16_t{};                                                                         \
    _Pragma("unroll") for (int st = 0; st < STEPS; ++st) {                                         \
      ACC_NEXT = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[st], __builtin_bit_cast(bf16x8_t, kf[st]), ACC_NEXT, 0, 0, 0); \
      __builtin_amdgcn_sched_barrier(0);                                                           \
      _Pragma("unroll") for (int e = 0; e < 16 / STEPS; ++e) PART(ACC_CUR, st * (16 / STEPS) + e)  \
      __builtin_amdgcn_sched_barrier(0);                                                           \
    }                                                                                              \
  }                                                                                                \
  POST(ACC_CUR, t)                                                                                 \
  PF_STORE(SET0, SET1, (t) + 2)                                                                    \
  PF_LOAD(SET0, SET1, (t) + 4)                                                                     \
  __syncthreads();

  f32x16_t accA, accB;
  // ---- phase 1: per lane and row, the two largest fast scores of candidate keys. With m1 >= m2,
  // the new second best is the median of m1, m2 and the score, and the new best is the median of
  // m1, the score and +inf (a run-time operand, so that no NaN-quieting is added around a max).
  const float pinf = a.pinf;
  float m1[16], m2[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) m1[r] = m2[r] = -INFINITY;
// (The empty asm statements pin each result to its place between the matrix instructions;
// without them the compiler sinks the work of a step past the next step's boundary-tile branch.)
#define PF_PART1(ACC, r)                                                                           \
  {                                                                                                \
    m2[r] = __builtin_amdgcn_fmed3f(m1[r], m2[r], ACC[r]);                                         \
    m1[r] = __builtin_amdgcn_fmed3f(m1[r], ACC[r], pinf);                                          \
    asm volatile("" : "+v"(m1[r]), "+v"(m2[r]));                                                   \
  }
#define PF_POST1(ACC, t)
  if (ntiles > 0) {
    PF_PROLOGUE(accA)
    for (int t = 0; t < ntiles; t += 2) {
      PF_STEP(PF_PART1, PF_POST1, t, accA, accB, r00, r01)
      PF_STEP(PF_PART1, PF_POST1, t + 1, accB, accA, r10, r11)
    }
  }

  // ---- thresholds: row R's 128 values sit at tops[R][64 * kq + 2 * m + {0, 1}] (even entries:
  // the lanes' best values, 64 distinct keys; odd entries: their second best). Each row needs a
  // lower bound T of the k-th largest of its 128 values such that few values lie between: the
  // largest T = lo + c (hi - lo) / 1024, c = 0..1023, that at least k values reach (a bitwise
  // search over c, monotone in c), where hi is the largest value and lo a known lower bound of the
  // k-th largest: for k <= 64 and 64 finite best values the smallest of them, else the smallest
  // finite value (if fewer than k values are finite every candidate stays). The bound is at most
  // (hi - lo) / 1024 below the k-th largest, and it is never above it. A wave takes 16 rows in
  // four groups of four; the 16 lanes of a row hold 8 values each, counted lane by lane and
  // summed over the row with DPP moves.
  float* tops = (float*)lists;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = row_base + 8 * (r / 4) + (r % 4);
    *(float2*)&tops[row * 128 + 64 * kq + 2 * m] = make_float2(m1[r], m2[r]);
  }
  const int sub = lane & 15;
  float qn_g[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int64_t i = i0 + wave * 16 + 4 * g + (lane >> 4);
    qn_g[g] = i < a.n_q ? a.w.qn[(size_t)bh * a.n_q + i] : 0.f;
  }
  __syncthreads();
  {
    float v[4][8], lo[4], step[4];
    int c[4];
    bool ok[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float* src = &tops[(wave * 16 + 4 * g + (lane >> 4)) * 128 + 8 * sub];
      const float4 x0 = *(const float4*)src, x1 = *(const float4*)(src + 4);
      v[g][0] = x0.x; v[g][1] = x0.y; v[g][2] = x0.z; v[g][3] = x0.w;
      v[g][4] = x1.x; v[g][5] = x1.y; v[g][6] = x1.z; v[g][7] = x1.w;
      float hi = -INFINITY, lo_best = INFINITY, lo_fin = INFINITY;
      int nfin = 0, nbest = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool fin = v[g][j] > -INFINITY;
        hi = fmaxf(hi, v[g][j]);
        nfin += fin;
        lo_fin = fin ? fminf(lo_fin, v[g][j]) : lo_fin;
        if ((j & 1) == 0) {
          nbest += fin;
          lo_best = fminf(lo_best, v[g][j]);
        }
      }
      hi = pf_row16<1>(hi);
      nfin = pf_row16<0>(nfin);
      nbest = pf_row16<0>(nbest);
      lo_fin = pf_row16<2>(lo_fin);
      lo_best = pf_row16<2>(lo_best);
      ok[g] = nfin >= a.topk;
      lo[g] = a.topk <= 64 && nbest == 64 ? lo_best : lo_fin;
      step[g] = ok[g] ? (hi - lo[g]) * (1.0f / 1024.0f) : 0.f;
      lo[g] = ok[g] ? lo[g] : 0.f;
      c[g] = 0;
    }
#pragma unroll
    for (int bit = 9; bit >= 0; --bit) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int cc = c[g] | (1 << bit);
        const float cand = fmaf((float)cc, step[g], lo[g]);
        int n = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) n += v[g][j] >= cand;
        n = pf_row16<0>(n);
        c[g] = n >= a.topk ? cc : c[g];
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int row = wave * 16 + 4 * g + (lane >> 4);
      if (sub == 0) {
        const float eps = i0 + row < a.n_q ? PF_EPS_COEF * qn_g[g] * knmax + 1e-30f : 0.f;
        const float x = ok[g] ? fmaf((float)c[g], step[g], lo[g]) : -INFINITY;
        // kept finite (at least the lowest float), so that the -inf of a masked score never passes
        lthf[row] = fmaxf(x - 2.0f * eps, -0x1.fffffep+127f);
      }
    }
  }
  if (tid < PF_ROWS) lcnt[tid] = 0u;
  __syncthreads();
  float thf[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) thf[r] = lthf[row_base + 8 * (r / 4) + (r % 4)];

  // ---- phase 2: every candidate key whose upper bound reaches the row's bound goes to the row's
  // list in global memory, with its score. A lane first gathers the test results of its 16
  // registers into bit r of `fail`'s complement: the test x >= T is the sign of x - T (T finite,
  // x finite or -inf), shifted in by v_alignbit from register 15 down to 0; its 16 scores go to
  // the wave's LDS stage. Then the lane takes its set bits one at a time: a slot from the row's LDS counter, (score read back from the stage, key
  // position) into the slot. The lanes of a wave pass through that loop together as often as the
  // busiest lane needs (a step has about one passing register per four lanes). Slots past the end
  // are clamped onto the last one; a row whose count ends above LCAP takes the exact path.
  uint32_t fail = 0u;
#define PF_PART2(ACC, i)                                                                           \
  {                                                                                                \
    fail = __builtin_amdgcn_alignbit((i) == 0 ? 0u : fail, __float_as_uint(ACC[15 - (i)] - thf[15 - (i)]), 31); \
    asm volatile("" : "+v"(fail));                                                                 \
  }
#define PF_POST2(ACC, t)                                                                           \
  {                                                                                                \
    uint32_t bits = ~fail & 0xFFFFu;                                                               \
    _Pragma("unroll") for (int q4 = 0; q4 < 4; ++q4)                                               \
      sst[q4 * 64 + lane] = make_float4(ACC[4 * q4], ACC[4 * q4 + 1], ACC[4 * q4 + 2], ACC[4 * q4 + 3]); \
    const uint32_t jj = (uint32_t)((t) * PF_KEYS + kq * 32 + m);                                   \
    while (bits) {                                                                                 \
      const int r = __builtin_ctz(bits);                                                           \
      bits &= bits - 1u;                                                                           \
      const int row = row_base + r + (r & 12); /* row_base + 8 * (r / 4) + r % 4 */               \
      const uint32_t sl = min(atomicAdd(&lcnt[row], 1u), LCAP - 1u);                               \
      const float x = ((const float*)sst)[((r >> 2) * 64 + lane) * 4 + (r & 3)];                   \
      a.w.surv[(grow0 + row) * LCAP + sl] = make_uint2(__float_as_uint(x), jj);                    \
    }                                                                                              \
  }
  if (ntiles > 0) {
    PF_PROLOGUE(accA)
    for (int t = 0; t < ntiles; t += 2) {
      PF_STEP(PF_PART2, PF_POST2, t, accA, accB, r00, r01)
      PF_STEP(PF_PART2, PF_POST2, t + 1, accB, accA, r10, r11)
    }
  }

  // the counts of the lists (or the overflow mark)
  if (tid < PF_ROWS && i0 + tid < a.n_q) {
    const uint32_t c = lcnt[tid];
    a.w.cnt[grow0 + tid] = c > LCAP ? PF_OVERFLOW : c;
  }
#undef PF_INTERIOR
#undef PF_LOAD
#undef PF_STORE
#undef PF_PROLOGUE
#undef PF_MMA
#undef PF_MASK
#undef PF_STEP
#undef PF_PART1
#undef PF_POST1
#undef PF_PART2
#undef PF_POST2
}

// ---------------------------------------------------------------------------------------------
// pf_window: the window's share of the softmax of every query row (bf16 inputs), on the matrix
// cores. One block per (b, h, 64 consecutive query rows), four waves: wave w takes the 32 rows of
// row tile w / 2 and half w % 2 of the output dimensions. The window keys of the block,
// [max(0, p_first - W + 1), p_last], go in tiles of 32 keys, staged in LDS (K and V, two buffers;
// tile u+1 is loaded while tile u is used). Per tile: S' = K_tile . Q^T with
// v_mfma_f32_32x32x16_bf16 (A = key rows, B = query rows), so lane l holds query row l % 32 of
// the wave's row tile and, in register r, key 8*(r/4) + 4*(l/32) + r%4 of the tile; keys outside
// the row's window [p - W + 1, p] are masked. (The two waves of a row tile compute the same
// scores; each needs them in its registers.) The row's running maximum m, sum Z and output O
// are updated online: factor exp(m_old - m_new) on Z and O, weights w = exp(z - m_new). O += w V
// on the bf16 matrix cores: each float32 weight is split into three bf16 parts w = w1 + w2 + w3
// (w1 = w with its low 16 bits cleared, w2 the same of w - w1, w3 = the rest, at most 8
// significant bits; exact for w >= 2^-110, below which w3 may lose bits worth less than 2^-133,
// nothing next to the largest weight, 1), every product of a part and a bf16 V element is exact
// in float32, and the three products are accumulated in float32 (smallest part first). The 16
// keys of matrix instruction s are the keys of registers 8s .. 8s+7 (lane half h: keys
// 8(r/4) + 4h + r%4), in the same order in the weight (A) and V (B) operands. The output tiles'
// rows are 8*(r/4) + 4*(l/32) + r%4, so their factors are read back from LDS.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void pf_window_kernel(PfArgs a) {
  constexpr int RB = D * 2, STEPS = D / 16, NW = D / 32, NWD = NW / 2;  // dim tiles per wave
  constexpr int STR = RB + 16;         // padded LDS row (K and V)
  constexpr int CPR = RB / 16;         // 16-byte chunks per key row
  constexpr int CPT = 32 * CPR / 256;  // chunks of K (and of V) per thread and tile
  static_assert(NWD >= 1 && CPT >= 1, "window tiles");
  __shared__ __align__(16) unsigned char kt[2][32 * STR];
  __shared__ __align__(16) unsigned char vt[2][32 * STR];
  __shared__ __align__(16) float alpha[4][32];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = lane & 31, half = lane >> 5, rt = wave >> 1, dh = wave & 1;
  const int64_t nrb = (a.n_q + 63) / 64;
  const int64_t job = xcd_job(blockIdx.x, nrb * a.Hq * (a.rows / (a.n_q * a.Hq)));
  const int bh = (int)(job / nrb);
  const int64_t i0 = (job - (int64_t)bh * nrb) * 64;
  const int b = bh / a.Hq, h = bh - b * a.Hq, g = h / a.G;
  const unsigned char* kb = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.n * RB;
  const unsigned char* vb = a.v + ((size_t)b * a.Hkv + g) * (size_t)a.n * RB;

  const int64_t iw = i0 + 32 * rt + m;  // the lane's query row
  bf16x8_t qf[STEPS];
  {
    const int64_t iq = min(iw, a.n_q - 1);
    const unsigned char* qrow = a.q + ((size_t)bh * a.n_q + iq) * RB;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) qf[st] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(qrow + st * 32 + half * 16));
  }
  const int64_t key_lo = a.q_pos0 + i0 - a.W + 1 > 0 ? a.q_pos0 + i0 - a.W + 1 : 0;
  const int64_t p_last = a.q_pos0 + min(i0 + 63, a.n_q - 1);
  const int ntk = (int)((p_last - key_lo) / 32) + 1;
  // the lane's row relative to key_lo (rows past n_q get -1: no key passes)
  const int prel = iw < a.n_q ? (int)(a.q_pos0 + iw - key_lo) : -1;
  const float sc = (float)a.scale;

  // thread tid stages chunks tid and (CPT = 2) tid + 256 of the tile: key row c / CPR, chunk
  // c % CPR (scalar registers: a staging array would go to scratch memory)
  static_assert(CPT <= 2, "window staging");
  const int c0 = tid, c1 = tid + 256;
  uint4 kr0, kr1 = make_uint4(0u, 0u, 0u, 0u), vr0, vr1 = kr1;
#define PW_LOAD(u)                                                                                 \
  {                                                                                                \
    const int64_t j0 = min(key_lo + 32 * (u) + c0 / CPR, a.n - 1);                                 \
    kr0 = *(const uint4*)(kb + (size_t)j0 * RB + (c0 % CPR) * 16);                                 \
    vr0 = *(const uint4*)(vb + (size_t)j0 * RB + (c0 % CPR) * 16);                                 \
    if (CPT > 1) {                                                                                 \
      const int64_t j1 = min(key_lo + 32 * (u) + c1 / CPR, a.n - 1);                               \
      kr1 = *(const uint4*)(kb + (size_t)j1 * RB + (c1 % CPR) * 16);                               \
      vr1 = *(const uint4*)(vb + (size_t)j1 * RB + (c1 % CPR) * 16);                               \
    }                                                                                              \
  }
#define PW_STORE(buf)                                                                              \
  {                                                                                                \
    *(uint4*)&kt[buf][(c0 / CPR) * STR + (c0 % CPR) * 16] = kr0;                                   \
    *(uint4*)&vt[buf][(c0 / CPR) * STR + (c0 % CPR) * 16] = vr0;                                   \
    if (CPT > 1) {                                                                                 \
      *(uint4*)&kt[buf][(c1 / CPR) * STR + (c1 % CPR) * 16] = kr1;                                 \
      *(uint4*)&vt[buf][(c1 / CPR) * STR + (c1 % CPR) * 16] = vr1;                                 \
    }                                                                                              \
  }
  PW_LOAD(0)
  PW_STORE(0)
  __syncthreads();

  float mrun = -INFINITY, zs = 0.f;
  f32x16_t o0 = f32x16_t{}, o1 = f32x16_t{};  // output tiles t = 0, 1 (o1 unused when NWD = 1)
  for (int u = 0; u < ntk; ++u) {
    const int buf = u & 1;
    if (u + 1 < ntk) PW_LOAD(u + 1)
    f32x16_t S = f32x16_t{};
    {
      const unsigned char* krow = &kt[buf][m * STR + half * 16];
      uint4 kf[STEPS];
#pragma unroll
      for (int st = 0; st < STEPS; ++st) kf[st] = *(const uint4*)(krow + st * 32);
#pragma unroll
      for (int st = 0; st < STEPS; ++st)
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[st]), qf[st], S, 0, 0, 0);
    }
    // key (r, half) of this tile is offset 32 u + 4 half + o_r from key_lo; it is in the row's
    // window iff prel - W < offset <= prel
    const int d = prel - 32 * u - 4 * half;
    float tm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int o_r = 8 * (r / 4) + (r % 4);
      S[r] = (o_r <= d && o_r > d - a.W) ? sc * S[r] : -INFINITY;
      tm = fmaxf(tm, S[r]);
    }
    tm = fmaxf(tm, __shfl_xor(tm, 32));
    const float mnew = fmaxf(mrun, tm);
    const float al = mnew == -INFINITY ? 1.f : __expf(mrun - mnew);
    mrun = mnew;
    zs *= al;
    if (half == 0) alpha[wave][m] = al;
    __builtin_amdgcn_wave_barrier();
    const float4* a4 = (const float4*)&alpha[wave][4 * half];
    float fr[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 x = a4[2 * q4];  // rows 8 q4 + 4 half + 0..3
      fr[4 * q4] = x.x;
      fr[4 * q4 + 1] = x.y;
      fr[4 * q4 + 2] = x.z;
      fr[4 * q4 + 3] = x.w;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      o0[r] *= fr[r];
      if (NWD > 1) o1[r] *= fr[r];
    }
    float w[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      w[r] = S[r] == -INFINITY ? 0.f : __expf(S[r] - mnew);
      zs += w[r];
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      uint32_t p1[4], p2[4], p3[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t h1[2], h2[2], h3[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float x = w[8 * s2 + 2 * j + e];
          h1[e] = __float_as_uint(x) & 0xFFFF0000u;
          const float r1 = x - __uint_as_float(h1[e]);
          h2[e] = __float_as_uint(r1) & 0xFFFF0000u;
          h3[e] = __float_as_uint(r1 - __uint_as_float(h2[e]));
        }
        p1[j] = (h1[0] >> 16) | h1[1];
        p2[j] = (h2[0] >> 16) | h2[1];
        p3[j] = (h3[0] >> 16) | (h3[1] & 0xFFFF0000u);
      }
      const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, make_uint4(p1[0], p1[1], p1[2], p1[3]));
      const bf16x8_t a2 = __builtin_bit_cast(bf16x8_t, make_uint4(p2[0], p2[1], p2[2], p2[3]));
      const bf16x8_t a3 = __builtin_bit_cast(bf16x8_t, make_uint4(p3[0], p3[1], p3[2], p3[3]));
#pragma unroll
      for (int t = 0; t < NWD; ++t) {
        const unsigned char* vcol = &vt[buf][(4 * half) * STR + (32 * (dh * NWD + t) + m) * 2];
        uint32_t vb4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r0 = 8 * s2 + 2 * j;
          const uint32_t v0 = *(const uint16_t*)(vcol + (8 * (r0 / 4) + (r0 % 4)) * STR);
          const uint32_t v1 = *(const uint16_t*)(vcol + (8 * ((r0 + 1) / 4) + ((r0 + 1) % 4)) * STR);
          vb4[j] = v0 | (v1 << 16);
        }
        const bf16x8_t vbf = __builtin_bit_cast(bf16x8_t, make_uint4(vb4[0], vb4[1], vb4[2], vb4[3]));
        f32x16_t ot = t == 0 ? o0 : o1;
        ot = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3, vbf, ot, 0, 0, 0);
        ot = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, vbf, ot, 0, 0, 0);
        ot = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, vbf, ot, 0, 0, 0);
        if (t == 0) o0 = ot; else o1 = ot;
      }
    }
    if (u + 1 < ntk) PW_STORE(buf ^ 1)
    __syncthreads();
  }
  zs += __shfl_xor(zs, 32);
#undef PW_LOAD
#undef PW_STORE

  // O_w: register r of tile t holds query row 32 rt + 8*(r/4) + 4*half + r%4 of the block and
  // dimension 32 (dh NWD + t) + m
#pragma unroll
  for (int t = 0; t < NWD; ++t) {
    const int dim = 32 * (dh * NWD + t) + m;
    const f32x16_t ot = t == 0 ? o0 : o1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t i = i0 + 32 * rt + 8 * (r / 4) + 4 * half + (r % 4);
      if (i < a.n_q) a.w.win_o[((size_t)bh * a.n_q + i) * D + dim] = ot[r];
    }
  }
  if (dh == 0 && half == 0 && iw < a.n_q) a.w.win_mz[(size_t)bh * a.n_q + iw] = make_float2(mrun, zs);
}

// ---------------------------------------------------------------------------------------------
// pf_finish: one wave per query row (4 rows per 256-thread block), each wave with its own LDS
// region laid out by PfRowSmem::carve for the call's k and 1 + W + k.
constexpr int PF_FIN_SET = 4096;   // largest 1 + W + k served by the per-row finish
struct PfRowSmem {
  double* qd;      // [128]
  double* rs;      // [slot + set_cap]: float64 scores of the row's list, window and anchor keys
  double* ts;      // [k + 1]
  double* cw;      // [set_cap]
  int32_t* ridx;   // [slot + 1]: the list, then the anchor
  int32_t* tidx;   // [k + 1]
  int32_t* cidx;   // [set_cap]
  uint32_t* hist;  // [256]
  static __host__ __device__ size_t bytes(int64_t slot, int k, int set_cap) {
    const size_t kk = (size_t)k + 1;
    return 128 * 8 + ((size_t)slot + set_cap) * 8 + kk * 12 + (size_t)set_cap * 12 + ((size_t)slot + 1) * 4 + 256 * 4 + 64;
  }
  __device__ void carve(unsigned char* p, int64_t slot, int k, int set_cap) {
    const size_t kk = (size_t)k + 1;
    qd = (double*)p;
    p += 128 * 8;
    rs = (double*)p;
    p += ((size_t)slot + set_cap) * 8;
    ts = (double*)p;
    p += kk * 8;
    cw = (double*)p;
    p += (size_t)set_cap * 8;
    ridx = (int32_t*)p;
    p += ((size_t)slot + 1) * 4;
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

// Ascending bitonic sort of the 64 E values of a wave (value i = x[i / 64] of lane i % 64).
template <int E>
__device__ __forceinline__ void wave_sort_asc_u32(uint32_t (&x)[E]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64 * E; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride == 64) {  // E == 2: values lane and lane + 64, one ascending block
        const uint32_t lo = min(x[0], x[1]), hi = max(x[0], x[1]);
        x[0] = lo;
        x[1] = hi;
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = lane + 64 * e;
          const uint32_t y = (uint32_t)__shfl_xor((int)x[e], stride);
          x[e] = (((i & size) == 0) == ((i & stride) == 0)) ? min(x[e], y) : max(x[e], y);
        }
      }
    }
  }
}

// One query row of the finish, by one wave. bf16 inputs: the top-k from the scan's matrix-core
// scores of the row's list with their error band (float64 canonical scores only for entries
// inside the band), the set in ascending order, then softmax and V sum over the anchor and the
// top-k in float32, merged with the window's share from pf_window. float32 inputs: float64 canonical scores of the list, anchor and window, exact
// rank of the list, float64 softmax and V sum over the whole set.
template <int D, bool BF16>
__device__ void pf_row(const PfArgs& a, PfRowSmem* sm, size_t grow) {
  constexpr int RB = D * (BF16 ? 2 : 4);
  // a key row is LPR lanes x 16 bytes, so one load instruction covers RPI rows
  constexpr int LPR = RB / 16, RPI = 64 / LPR, EPC = BF16 ? 8 : 4;
  const int lane = threadIdx.x & 63;
  const size_t bh = grow / (size_t)a.n_q;
  const int64_t i = (int64_t)(grow - bh * (size_t)a.n_q);
  const int b = (int)(bh / a.Hq), h = (int)(bh - (size_t)b * a.Hq), g = h / a.G;
  const unsigned char* kb = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.n * RB;
  const unsigned char* vb = a.v ? a.v + ((size_t)b * a.Hkv + g) * (size_t)a.n * RB : nullptr;
  const int64_t p = a.q_pos0 + i;
  const unsigned char* qrow = a.q + grow * RB;
  const int gq = lane / LPR, cc = lane % LPR;
  // error-bound inputs, requested early: |q| of the row and the largest |k| of the kv head
  const float qn_row = a.w.qn[grow];
  const float kn_max = __uint_as_float(a.w.knmax[(size_t)b * a.Hkv + g]);
  // the float64 query (canonical scores) is filled where a path needs it: float32 inputs and
  // the exact path always, the bf16 fast path only for a band to re-score
  auto fill_qd = [&]() {
    for (int t = lane; t < D; t += 64) sm->qd[t] = load_elem_f64<BF16>(qrow, t);
    __builtin_amdgcn_wave_barrier();
  };
  // bf16: the anchor's key chunk and the row's query chunk for its float32 score, requested with
  // the list so that both cost one memory round trip
  uint4 k0v = make_uint4(0u, 0u, 0u, 0u), q0v = k0v;
  if constexpr (BF16) {
    k0v = *(const uint4*)(kb + cc * 16);
    q0v = *(const uint4*)(qrow + cc * 16);
  } else {
    fill_qd();
  }

  const int64_t w_lo = p - a.W + 1 > 0 ? p - a.W + 1 : 0;
  const int anchor = w_lo > 0 ? 1 : 0;
  const int nwin = (int)(p - w_lo + 1);

  // ---- the row's list of possible top-k keys (fast path) or the exact path
  int c = 0;
  bool exact = false;
  if (a.topk > 0) {
    // The count and the row's whole slot area (at most 128 entries, two per lane) are read
    // together, so that the list costs one memory round trip; slots at or past the count hold
    // stale entries and are ignored.
    uint32_t cr = PF_OVERFLOW;
    uint2 e0 = make_uint2(0u, 0u), e1 = e0;
    if (!a.exact_all) {
      const uint2* sv = a.w.surv + grow * (size_t)a.slot;
      cr = a.w.cnt[grow];
      if (lane < a.slot) e0 = sv[lane];
      if (lane + 64 < a.slot) e1 = sv[lane + 64];
    }
    exact = cr == PF_OVERFLOW;
    if (!exact) {
      c = (int)cr;
      // positions come from the scan and are always keys of the cache; clamping only guards
      // the reads below. With bf16 inputs the scan's matrix-core scores come along.
      if (lane < c) {
        sm->ridx[lane] = (int32_t)min(e0.y, (uint32_t)(a.n - 1));
        if constexpr (BF16) sm->rs[lane] = (double)__uint_as_float(e0.x);
      }
      if (lane + 64 < c) {
        sm->ridx[lane + 64] = (int32_t)min(e1.y, (uint32_t)(a.n - 1));
        if constexpr (BF16) sm->rs[lane + 64] = (double)__uint_as_float(e1.x);
      }
    }
  }
  __builtin_amdgcn_wave_barrier();

  // ---- scores: items [0, c) the list, c the anchor (if any), then (float32 inputs) the window;
  // with bf16 inputs the window's share of the softmax comes from pf_window
  const int wbase = c + anchor;
  const int nitems = BF16 ? wbase : wbase + nwin;
  int nt = 0;
  if constexpr (BF16) {
    // The list's scores are the scan's matrix-core float32 scores, |s_mc - s| <= eps (s the
    // exact score). The anchor gets a float32 score here (LPR lanes, a 16-byte chunk each,
    // v_dot2_f32_bf16, summed across the lanes with DPP adds); it only enters the softmax.
    if (anchor) {
      const float part = group_sum_f32<LPR>(dot_chunk_bf16(q0v, k0v, 0.0f));
      if (lane == 0) sm->rs[c] = (double)part;
    }
    __builtin_amdgcn_wave_barrier();
    const float eps = PF_EPS_COEF * qn_row * kn_max + 1e-30f;
    if (exact) {
      fill_qd();
      nt = pf_exact_row<D, BF16>(sm, a, kb, p);
    } else if (c > a.topk) {
      // x_k = k-th largest score of the list; A = entries with s_mc >= x_k - 2 eps. Every
      // entry outside A scores below all k entries with s_mc >= x_k, so the top-k lies in A, and
      // if |A| = k it is A. Otherwise an entry with s_mc > x_k + 2 eps is surely in the top-k
      // (only entries with s_mc > x_k, at most k - 1 of them, can score above it), and the rest of
      // A, the band around x_k, is ranked by float64 canonical scores, then by position; its best
      // k - (sure entries) complete the top-k.
      const float s0 = lane < c ? (float)sm->rs[lane] : 0.f;
      const float s1 = lane + 64 < c ? (float)sm->rs[lane + 64] : 0.f;
      const uint32_t key[2] = {lane < c ? ord_f32(s0) : 0u, lane + 64 < c ? ord_f32(s1) : 0u};
      const float xk = unord_f32(wave_kth_largest<2>(key, a.topk));
      const float thr = (xk - 2.0f * eps) - fabsf(xk) * 0x1p-20f;
      const bool in0 = lane < c && s0 >= thr, in1 = lane + 64 < c && s1 >= thr;
      const uint64_t m0 = __ballot(in0), m1 = __ballot(in1);
      const int na = __popcll(m0) + __popcll(m1);
      if (na == a.topk) {
        if (in0) {
          const int pos = lanes_below(m0);
          sm->tidx[pos] = sm->ridx[lane];
          sm->ts[pos] = (double)s0;
        }
        if (in1) {
          const int pos = __popcll(m0) + lanes_below(m1);
          sm->tidx[pos] = sm->ridx[lane + 64];
          sm->ts[pos] = (double)s1;
        }
        nt = a.topk;
        __builtin_amdgcn_wave_barrier();
      } else {
        const float hi = (xk + 2.0f * eps) + fabsf(xk) * 0x1p-20f;
        const bool su0 = in0 && s0 > hi, su1 = in1 && s1 > hi;
        const bool bd0 = in0 && !su0, bd1 = in1 && !su1;
        const uint64_t ms0 = __ballot(su0), ms1 = __ballot(su1), mb0 = __ballot(bd0), mb1 = __ballot(bd1);
        const int ns = __popcll(ms0) + __popcll(ms1), nb = __popcll(mb0) + __popcll(mb1);
        // sure entries to tidx / ts [0, ns); the band's positions to ridx [0, nb)
        const int32_t j0 = in0 ? sm->ridx[lane] : 0, j1 = in1 ? sm->ridx[lane + 64] : 0;
        __builtin_amdgcn_wave_barrier();
        if (su0) {
          const int pos = lanes_below(ms0);
          sm->tidx[pos] = j0;
          sm->ts[pos] = (double)s0;
        }
        if (su1) {
          const int pos = __popcll(ms0) + lanes_below(ms1);
          sm->tidx[pos] = j1;
          sm->ts[pos] = (double)s1;
        }
        if (bd0) sm->ridx[lanes_below(mb0)] = j0;
        if (bd1) sm->ridx[__popcll(mb0) + lanes_below(mb1)] = j1;
        __builtin_amdgcn_wave_barrier();
        if (nb > 0) fill_qd();
        for (int t = lane; t < nb; t += 64)
          sm->rs[t] = canonical_score_row<BF16, D>(sm->qd, kb + (size_t)sm->ridx[t] * RB);
        __builtin_amdgcn_wave_barrier();
        const int need = a.topk - ns;
        for (int t = lane; t < nb; t += 64) {
          const double si = sm->rs[t];
          const int32_t ji = sm->ridx[t];
          int rank = 0;
          for (int r = 0; r < nb; ++r) {
            const double sr = sm->rs[r];
            rank += (sr > si) || (sr == si && sm->ridx[r] < ji);
          }
          if (rank < need) {
            sm->tidx[ns + rank] = ji;
            sm->ts[ns + rank] = si;
          }
        }
        nt = a.topk;
        __builtin_amdgcn_wave_barrier();
      }
    } else if (c > 0) {
      for (int t = lane; t < c; t += 64) {
        sm->tidx[t] = sm->ridx[t];
        sm->ts[t] = sm->rs[t];
      }
      nt = c;
      __builtin_amdgcn_wave_barrier();
    }
  } else {
    // float32 inputs: float64 canonical scores throughout
    for (int t = lane; t < nitems; t += 64) {
      const int64_t j = t < c ? (int64_t)sm->ridx[t] : (t < wbase ? 0 : w_lo + (t - wbase));
      sm->rs[t] = canonical_score_row<BF16, D>(sm->qd, kb + (size_t)j * RB);
    }
    __builtin_amdgcn_wave_barrier();
    if (exact) {
      nt = pf_exact_row<D, BF16>(sm, a, kb, p);
    } else if (c > a.topk) {
      for (int t = lane; t < c; t += 64) {
        const double si = sm->rs[t];
        const int32_t ji = sm->ridx[t];
        int rank = 0;
        for (int r = 0; r < c; ++r) {
          const double sr = sm->rs[r];
          rank += (sr > si) || (sr == si && sm->ridx[r] < ji);
        }
        if (rank < a.topk) {
          sm->tidx[rank] = ji;
          sm->ts[rank] = si;
        }
      }
      nt = a.topk;
      __builtin_amdgcn_wave_barrier();
    } else if (c > 0) {
      for (int t = lane; t < c; t += 64) {
        sm->tidx[t] = sm->ridx[t];
        sm->ts[t] = sm->rs[t];
      }
      nt = c;
      __builtin_amdgcn_wave_barrier();
    }
  }

  // ---- set: {0} u window u T, ascending
  const int count = anchor + nwin + nt;
  int tlo = 0;
  for (int t = lane; t < nt; t += 64) tlo += sm->tidx[t] < w_lo;
  tlo = wave_sum_i32(tlo);
  if (anchor && lane == 0) {
    sm->cidx[0] = 0;
    if constexpr (!BF16) sm->cw[0] = sm->rs[c];
  }
  if (BF16 && nt <= 128) {
    // the top-k positions sorted (distinct keys; empty slots sort last): the t-th smallest goes
    // to slot anchor + t, after the window if it lies past p
    if (nt <= 64) {
      uint32_t x[1] = {lane < nt ? (uint32_t)sm->tidx[lane] : 0xFFFFFFFFu};
      wave_sort_asc_u32<1>(x);
      if (lane < nt) sm->cidx[anchor + lane + ((int64_t)x[0] > p ? nwin : 0)] = (int32_t)x[0];
    } else {
      uint32_t x[2] = {(uint32_t)sm->tidx[lane], lane + 64 < nt ? (uint32_t)sm->tidx[lane + 64] : 0xFFFFFFFFu};
      wave_sort_asc_u32<2>(x);
      sm->cidx[anchor + lane + ((int64_t)x[0] > p ? nwin : 0)] = (int32_t)x[0];
      if (lane + 64 < nt) sm->cidx[anchor + lane + 64 + ((int64_t)x[1] > p ? nwin : 0)] = (int32_t)x[1];
    }
  } else {
    // rank of each top-k position among the others
    for (int t = lane; t < nt; t += 64) {
      const int32_t j = sm->tidx[t];
      int below = 0;
      for (int r = 0; r < nt; ++r) below += sm->tidx[r] < j;
      const int pos = anchor + below + (j > p ? nwin : 0);
      sm->cidx[pos] = j;
      if constexpr (!BF16) sm->cw[pos] = sm->ts[t];
    }
  }
  for (int t = lane; t < nwin; t += 64) {
    const int pos = anchor + tlo + t;
    sm->cidx[pos] = (int32_t)(w_lo + t);
    if constexpr (!BF16) sm->cw[pos] = sm->rs[wbase + t];
  }
  __builtin_amdgcn_wave_barrier();
  if (a.sel_idx) {
    int32_t* dst = a.sel_idx + grow * (size_t)a.set_cap;
    for (int t = lane; t < a.set_cap; t += 64) dst[t] = t < count ? sm->cidx[t] : -1;
  }
  if (a.sel_count && lane == 0) a.sel_count[grow] = count;
  if (!a.out) return;

  // ---- softmax over the set and the weighted V rows: lane group gq takes the entries
  // t = gq (mod RPI), each lane a 16-byte chunk of the row; then the groups are summed.
  constexpr int U = BF16 ? 17 : 4;  // V rows per lane group in flight together (bf16: the whole set for k <= 67)
  if constexpr (BF16) {
    // The window's part (m_w, Z_w, O_w) comes from pf_window; here the anchor and the top-k
    // (tidx / ts [0, nt), the anchor appended at nt), then the merge of the two parts:
    // out = (f O_w + sum_e w_e v_e) / (f Z_w + sum_e w_e), w_e = exp(z_e - zmax),
    // f = exp(m_w - zmax), zmax the largest logit of the set.
    const float sc = (float)a.scale;
    const int ne = nt + anchor;
    if (anchor && lane == 0) {
      sm->tidx[nt] = 0;
      sm->ts[nt] = sm->rs[c];
    }
    __builtin_amdgcn_wave_barrier();
    // the window's part (maximum and sum, then its partial output) and the first batch of V rows
    // are requested before the weights are computed, so that their memory latency overlaps the
    // softmax
    const float2 mz = a.win ? a.w.win_mz[grow] : make_float2(-INFINITY, 0.f);
    uint4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = u * RPI + gq;
      x[u] = t < ne ? *(const uint4*)(vb + (size_t)sm->tidx[t] * RB + cc * 16) : make_uint4(0u, 0u, 0u, 0u);
    }
    float4 wo[EPC / 4];
#pragma unroll
    for (int e = 0; e < EPC / 4; ++e)
      wo[e] = a.win && gq == 0 ? ((const float4*)(a.w.win_o + grow * D + cc * EPC))[e] : make_float4(0.f, 0.f, 0.f, 0.f);
    float zmax = mz.x;
    for (int t = lane; t < ne; t += 64) zmax = fmaxf(zmax, sc * (float)sm->ts[t]);
    zmax = wave_max_f32(zmax);
    float zsum = 0.f;
    for (int t = lane; t < ne; t += 64) {
      const float w = __expf(sc * (float)sm->ts[t] - zmax);
      sm->ts[t] = (double)w;
      zsum += w;
    }
    const float fw = a.win ? __expf(mz.x - zmax) : 0.f;
    zsum = wave_sum_f32(zsum) + fw * mz.y;
    __builtin_amdgcn_wave_barrier();
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
    auto accumulate = [&](const uint4 (&x)[U], const float (&w)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t xs[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = fmaf(w[u], bf16_lo(xs[e]), acc[2 * e]);
          acc[2 * e + 1] = fmaf(w[u], bf16_hi(xs[e]), acc[2 * e + 1]);
        }
      }
    };
    for (int t0 = 0; t0 < ne; t0 += U * RPI) {
      if (t0 > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int t = t0 + u * RPI + gq;
          x[u] = t < ne ? *(const uint4*)(vb + (size_t)sm->tidx[t] * RB + cc * 16) : make_uint4(0u, 0u, 0u, 0u);
        }
      }
      float w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u * RPI + gq;
        w[u] = t < ne ? (float)sm->ts[t] : 0.f;
      }
      accumulate(x, w);
    }
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] += __shfl_xor(acc[e], o);
    if (gq == 0) {
      if (a.win) {
#pragma unroll
        for (int e = 0; e < EPC / 4; ++e) {
          const float4 o4 = wo[e];
          acc[4 * e] = fmaf(fw, o4.x, acc[4 * e]);
          acc[4 * e + 1] = fmaf(fw, o4.y, acc[4 * e + 1]);
          acc[4 * e + 2] = fmaf(fw, o4.z, acc[4 * e + 2]);
          acc[4 * e + 3] = fmaf(fw, o4.w, acc[4 * e + 3]);
        }
      }
      const float inv = 1.0f / zsum;
      float4* dst = (float4*)(a.out + grow * D + cc * EPC);
#pragma unroll
      for (int e = 0; e < EPC / 4; ++e)
        dst[e] = make_float4(acc[4 * e] * inv, acc[4 * e + 1] * inv, acc[4 * e + 2] * inv, acc[4 * e + 3] * inv);
    }
  } else {
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
    double acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
    for (int t0 = 0; t0 < count; t0 += U * RPI) {
      uint4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u * RPI + gq;
        x[u] = t < count ? *(const uint4*)(vb + (size_t)sm->cidx[t] * RB + cc * 16) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u * RPI + gq;
        const double w = t < count ? sm->cw[t] : 0.0;
        acc[0] = fma(w, (double)__uint_as_float(x[u].x), acc[0]);
        acc[1] = fma(w, (double)__uint_as_float(x[u].y), acc[1]);
        acc[2] = fma(w, (double)__uint_as_float(x[u].z), acc[2]);
        acc[3] = fma(w, (double)__uint_as_float(x[u].w), acc[3]);
      }
    }
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] += __shfl_xor(acc[e], o);
    if (gq == 0) {
      float4* dst = (float4*)(a.out + grow * D + cc * EPC);
      dst[0] = make_float4((float)(acc[0] / zsum), (float)(acc[1] / zsum), (float)(acc[2] / zsum), (float)(acc[3] / zsum));
    }
  }
}

// pf_finish: one wave per query row, 4 rows per block (consecutive rows of one head).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void pf_finish_kernel(PfArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int wave = threadIdx.x >> 6;
  PfRowSmem smv;
  smv.carve(smem_raw + wave * a.wave_smem, a.slot, a.topk, a.set_cap);
  const size_t grow = (size_t)xcd_job(blockIdx.x, gridDim.x) * 4 + wave;  // (b*Hq + h) * n_q + i
  if (grow >= (size_t)a.rows) return;
  pf_row<D, BF16>(a, &smv, grow);
}

// ---------------------------------------------------------------------------------------------
template <int D, bool BF16>
static hipError_t launch_pf_t(const PrefillLaunch& L, const PfArgs& pa, hipStream_t s) {
  const size_t rows = (size_t)L.B * L.Hq * (size_t)L.n_q;
  hipError_t e = hipSuccess;
  if constexpr (BF16) {
    if (!pa.exact_all && L.topk > 0) {
      // norms for the error bounds of the matrix-core scores (only the fast selection uses them)
      constexpr int RPW = 64 / (D * 2 / 16), QU = 4, KU = 16;  // rows per wave load; loads per lane
      hipLaunchKernelGGL((pf_norm_kernel<D, QU>), dim3((unsigned)((rows + 4 * QU * RPW - 1) / (4 * QU * RPW)), 1), dim3(256),
                         0, s, (const unsigned char*)L.q, (int64_t)rows, pa.w.qn, (uint32_t*)nullptr, pa.w.knmax,
                         L.B * L.Hkv);
      hipLaunchKernelGGL((pf_norm_kernel<D, KU>), dim3((unsigned)((L.n + 4 * KU * RPW - 1) / (4 * KU * RPW)), (unsigned)(L.B * L.Hkv)),
                         dim3(256), 0, s, (const unsigned char*)L.k, L.n, (float*)nullptr, pa.w.knmax, (uint32_t*)nullptr, 0);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (L.ev_scan_begin) (void)hipEventRecord(L.ev_scan_begin, s);
  if (!pa.exact_all && L.topk > 0) {
    if constexpr (BF16) {
      hipLaunchKernelGGL((pf_scan_kernel<D>), dim3((unsigned)((L.n_q + PF_ROWS - 1) / PF_ROWS * L.B * L.Hq)),
                         dim3(512), 0, s, pa);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (L.ev_scan_end) (void)hipEventRecord(L.ev_scan_end, s);
  if constexpr (BF16) {
    if (pa.win) {
      hipLaunchKernelGGL((pf_window_kernel<D>), dim3((unsigned)((L.n_q + 63) / 64 * L.B * L.Hq)), dim3(256), 0, s,
                         pa);
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
  pa.w = pf_carve(L.ws, L.B, L.Hq, L.n_q, L.d, L.topk);
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
  pa.win = (L.bf16 && L.W > 0 && L.out) ? 1 : 0;
  // the scan addresses a kv head's keys with 32-bit buffer offsets
  pa.exact_all = (!L.bf16 || L.topk > PF_MAX_K || (L.flags & 1) || L.n * 2 * L.d >= ((int64_t)1 << 31)) ? 1 : 0;
  static_assert(PF_MAX_K + 16 <= PF_LCAP_MAX, "list room above k");
  pa.scale = L.scale;
  pa.pinf = INFINITY;
  pa.rows = (int64_t)L.B * L.Hq * L.n_q;
  pa.wave_smem = (PfRowSmem::bytes(pa.slot, L.topk, pa.set_cap) + 255) & ~(size_t)255;
  if (4 * pa.wave_smem > 160 * 1024) return hipErrorNotSupported;
  if (L.bf16) return L.d == 128 ? launch_pf_t<128, true>(L, pa, stream) : launch_pf_t<64, true>(L, pa, stream);
  return L.d == 128 ? launch_pf_t<128, false>(L, pa, stream) : launch_pf_t<64, false>(L, pa, stream);
}

}  // namespace topo
