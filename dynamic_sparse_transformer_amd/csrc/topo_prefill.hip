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
//   pf_norms   |q| of every query row and |k| of every key (each score's own error bound).
//   pf_scan    bf16 MFMA tiles, 128 query rows x 64 keys per step (8 waves, four 16x16x32 tiles
//              each), float32 scores, two passes over the keys: the first bounds each row's k-th
//              best score from below, the second lists every key that may still reach it.
//   pf_window  matrix-core softmax share of every row's window (max, sum, weighted V).
//   pf_finish  one wave per query row: top-k from the list's scores with their error band,
//              float64 canonical scores where the band leaves the top-k open, the set, softmax
//              and V reduction over anchor and top-k, merged with the window's share. Rows
//              whose list overflowed (ties), float32 inputs and k above the scan's limit take
//              an exact float64 radix selection over all of the row's candidates instead.
#include <atomic>

#include "topo_device.h"
#include "topo_internal.h"

namespace topo {

constexpr int PF_ROWS = 128;         // query rows per scan block (8 waves: 2 row groups x 4 key quarters)
constexpr int PF_KEYS = 64;          // keys per scan step
constexpr int PF_MAX_K = 96;         // largest k the MFMA scan ranks

// Error bound of the MFMA float32 scores. Products of bf16 values are exact in float32. A float32
// sum of d <= 128 of them with round-to-nearest, in any order and grouping, is off by less than
// d 2^-24 sum_t |q_t k_t| <= 2^-17 |q| |k| (Cauchy-Schwarz). A matrix unit that instead aligns
// the 32 products of a slice to the largest of them and truncates loses less than
// 32 2^-23 max|p| <= 2^-18 sum|p| per slice, plus at most 2^-23 sum|p| for each of the d / 32
// float32 accumulations: again less than 2^-17 |q| |k|. So |s_fast - s| <= 2^-15 |q| |k| holds
// with a factor 4 to spare in either model; the spare also covers forming a bound
// s_fast -+ 2^-15 |q| |k| in float32 (half an ulp of the score, at most 2^-24 |q| |k|). The
// tests measure the largest |s_fast - s| / (|q| |k|) on the scan's lists (near 2^-23).
constexpr float PF_EPS_COEF = 0x1p-15f;
float prefill_eps_coef() { return PF_EPS_COEF; }

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// LDS of the scan for the top-2 values of each row's lanes between the two phases. A row's list
// of possible top-k keys holds k + 48 entries, at most 128 (the finish ranks two per lane).
constexpr int PF_LIST_BYTES = PF_ROWS * 136 * 4;
constexpr int PF_LCAP_MAX = 128;
static int64_t pf_slot(int32_t k) { return k + 48 < PF_LCAP_MAX ? k + 48 : PF_LCAP_MAX; }

struct PfWs {
  float* qn;        // [B*Hq*n_q]: |q| of every query row (rounded up)
  float* kn;        // [B*Hkv][n]: |k| of every key (rounded up)
  float* ktmax;     // [B*Hkv][ceil(n / 64)]: the largest |k| of each 64-key tile
  uint32_t* cnt;    // [B*Hq*n_q]: entries of the row's list, from the front of its slots (low 16 bits)
                    // and from the back (high 16 bits, 0 from this scan); more than the slots
                    // hold = overflow
  int32_t* path;    // [B*Hq*n_q]: how the finish chose the row's top-k part (PATH_*)
  uint2* surv;      // [B*Hq*n_q][list]: (float bits of the matrix-core score, key position)
  float* win_o;     // [B*Hq*n_q][d]: sum over the row's window of exp(z - m_w) v (bf16 inputs)
  float2* win_mz;   // [B*Hq*n_q]: (m_w, sum over the window of exp(z - m_w))
};

static PfWs pf_carve(void* ws, int32_t B, int32_t Hq, int32_t Hkv, int64_t n_q, int64_t n, int32_t d, int32_t k,
                     size_t* total = nullptr) {
  const size_t rows = (size_t)B * Hq * (size_t)n_q;
  PfWs w;
  char* p = (char*)ws;
  w.qn = (float*)p;
  p += align256(rows * 4);
  w.kn = (float*)p;
  p += align256((size_t)B * Hkv * (size_t)n * 4);
  w.ktmax = (float*)p;
  p += align256((size_t)B * Hkv * (size_t)((n + 63) / 64) * 4);
  w.cnt = (uint32_t*)p;
  p += align256(rows * 4);
  w.path = (int32_t*)p;
  p += align256(rows * 4);
  w.surv = (uint2*)p;
  p += align256(rows * (size_t)pf_slot(k) * sizeof(uint2));
  w.win_o = (float*)p;
  p += align256(rows * (size_t)d * 4);
  w.win_mz = (float2*)p;
  p += rows * 8;
  if (total) *total = (size_t)(p - (char*)ws);
  return w;
}

size_t prefill_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t n_q, int64_t n, int32_t d, int32_t, int32_t k) {
  size_t total = 0;
  (void)pf_carve(nullptr, B, Hq, Hkv, n_q, n, d, k, &total);
  return total;
}

PrefillView prefill_view(int32_t B, int32_t Hq, int32_t Hkv, int64_t n_q, int64_t n, int32_t d, int32_t k) {
  const PfWs w = pf_carve(nullptr, B, Hq, Hkv, n_q, n, d, k);
  PrefillView v;
  v.count = (size_t)(uintptr_t)w.cnt;
  v.entry = (size_t)(uintptr_t)w.surv;
  v.path = (size_t)(uintptr_t)w.path;
  v.slot = pf_slot(k);
  return v;
}

// ---------------------------------------------------------------------------------------------
// Norms of bf16 rows for the error bounds of the matrix-core scores: |q| of every query row and
// |k| of every key, each score's bound taking its own two norms. A row is LPR lanes x 16 bytes
// (coalesced, RPW rows per load instruction). The squares of bf16 values are exact in float32;
// their float32 sum (8 terms per lane, then a tree over the LPR lanes) and sqrtf carry a relative
// error far below the factor (1 + 2^-15) that rounds the norm up. One launch for both: blocks
// [0, qblocks) take the query rows (one run of rows), the rest the keys, kblocks per kv head;
// U rows per lane. For the keys, also the largest norm of each 64-row tile of a head (a block
// covers whole tiles: 64 or 128 rows).
template <int D, int U>
__device__ __forceinline__ void pf_norm_rows(const unsigned char* x, int64_t rows_per_head, float* norm, float* tmax,
                                             uint32_t bx, uint32_t by) {
  constexpr int RB = D * 2, LPR = RB / 16, RPW = 64 / LPR, BROWS = 4 * U * RPW;
  static_assert(BROWS % 64 == 0 && 64 % (U * RPW) == 0, "a wave's rows lie in one tile, a block covers whole tiles");
  __shared__ uint32_t tm[BROWS / 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, gq = lane / LPR, cc = lane % LPR;
  if (threadIdx.x < BROWS / 64) tm[threadIdx.x] = 0u;
  float wmax = 0.f;
  const unsigned char* base = x + (size_t)by * (size_t)rows_per_head * RB;
  const int64_t r0 = (int64_t)bx * (4 * U * RPW) + (int64_t)wave * U * RPW + gq;
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t row = r0 + u * RPW;
    v[u] = row < rows_per_head ? *(const uint4*)(base + (size_t)row * RB + cc * 16) : make_uint4(0u, 0u, 0u, 0u);
  }
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
    if (cc == 0 && row < rows_per_head) norm[(size_t)by * rows_per_head + row] = nrm;
    wmax = row < rows_per_head ? fmaxf(wmax, nrm) : wmax;
  }
  if (tmax) {
    // norms are non-negative, so their bits order like the values
    wmax = wave_max_f32(wmax);
    __syncthreads();
    if (lane == 0) atomicMax(&tm[wave * U * RPW / 64], __float_as_uint(wmax));
    __syncthreads();
    const int64_t tiles = (rows_per_head + 63) / 64, t = (int64_t)bx * (BROWS / 64) + threadIdx.x;
    if (threadIdx.x < BROWS / 64 && t < tiles) tmax[(size_t)by * tiles + t] = __uint_as_float(tm[threadIdx.x]);
  }
}
struct PfNormArgs {
  const unsigned char* q;
  int64_t q_rows;
  float* qn;
  const unsigned char* k;
  int64_t n;
  float* kn;
  float* ktmax;
  uint32_t qblocks, kblocks;  // blocks [0, qblocks) take the query rows, the rest kblocks per kv head
};
template <int D, int U>
__device__ __forceinline__ void pf_norm_block(const PfNormArgs& na, uint32_t blk) {
  if (blk < na.qblocks) {
    pf_norm_rows<D, U>(na.q, na.q_rows, na.qn, nullptr, blk, 0u);
  } else {
    const uint32_t j = blk - na.qblocks;
    pf_norm_rows<D, U>(na.k, na.n, na.kn, na.ktmax, j % na.kblocks, j / na.kblocks);
  }
}
template <int D, int U>
__global__ __launch_bounds__(256) void pf_norm_kernel(PfNormArgs na) {
  pf_norm_block<D, U>(na, blockIdx.x);
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
  int32_t B, Hq, Hkv, G, W, topk, causal, set_cap, exact_all;
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
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// pf_scan: blocks of 512 threads, each scoring one or more jobs (b, h, 128 consecutive query
// rows) in turn. Each step scores 64 keys held in LDS. Wave w = 4 rg + kg holds the 64 query rows 64 rg .. +64 as the A operands of
// four 16-row tiles and scores them against keys 16 kg .. +16 of the tile with
// v_mfma_f32_16x16x32_bf16 (one B operand read from LDS feeds four products). Lane l supplies row
// / key l % 16 and elements 8 (l / 16) .. +8 of each 32-deep slice; a slice takes, for both
// operands, the 8 consecutive dimensions starting at 32 (l / 16) + 8 s of each row, so that a
// lane's operands are one contiguous run of each row (the pairing of dimensions is the same for
// Q and K, so the sum over them is the dot product). Register e of row tile u holds the score of
// row 16 u + 4 (l / 16) + e and key l % 16.
// The key tiles rotate through 2 PF_H LDS buffers: tile t is written PF_H + 1 steps before the
// step that reads it, so that the waves meet at a barrier only every PF_H steps. The loads of the
// tiles written at steps t + 1 .. t + 4 are in flight while step t runs.
// Every score has its own error bound eps = C |q| |k| (C = PF_EPS_COEF). Phase 1 keeps, per lane
// and row, the two largest fast scores it has seen; the largest norm of the keys the block scores
// comes from the tiles' maxima. Those 128 values per row belong to distinct candidate keys, so if
// k of them reach x, k keys score at least x - C |q| max|k| exactly, and each of them has a fast
// score of at least x - 2 C |q| max|k|: phase 2 scores the keys again and lists every key whose
// fast score reaches T = x - 2 C |q| max|k| (computed with a spare far above float32 rounding) in its
// row's list in global memory, with a slot from the row's LDS counter. The finish ranks the
// lists.
constexpr int PF_H = 2;              // steps between block barriers
constexpr int PF_NBUF = 2 * PF_H;    // LDS key tile buffers

template <int D>
__global__ __launch_bounds__(512) void pf_scan_kernel(PfArgs a) {
  constexpr int RB = D * 2;
  constexpr int SL = D / 32;              // 32-deep slices of a row
  constexpr int GB = RB / 4;              // bytes of a row supplied by one lane (SL chunks of 16)
  constexpr int NCH = RB / 16;            // 16-byte chunks per key row
  constexpr int STRIDE = RB + 16;         // padded LDS row
  constexpr int RPP = 512 / NCH;          // key rows staged per load pass
  constexpr int PASSES = PF_KEYS / RPP;
  constexpr int TILE_BYTES = PF_KEYS * STRIDE;
  constexpr int SMEM = PF_NBUF * TILE_BYTES > PF_LIST_BYTES ? PF_NBUF * TILE_BYTES : PF_LIST_BYTES;
  constexpr int PER = 16 / (4 * SL);      // score registers handled after each matrix instruction
  static_assert(PASSES >= 1 && PASSES <= 2, "staging passes");
  __shared__ __align__(16) unsigned char ktiles[SMEM];  // key tiles; the thresholds' values between the phases
  __shared__ __align__(16) float sstage[8 * 64 * 16];    // phase 2: each lane's 16 scores of a step
  __shared__ float lthk[PF_ROWS];
  // the rows' list counters (see phase 2), then at +136 the byte offset of each counter's row list
  __shared__ uint32_t rowcnt[2 * 2 * 4 * 17];
  __shared__ uint32_t kmax_blk;  // float bits of the largest key norm the block has staged

  // (the wave index through readfirstlane, so that the compiler keeps what derives from it in
  // scalar registers)
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // Jobs of this block. The host launches at most as many blocks as fit on the GPU at once, so
  // the block count fixes which jobs share a compute unit instead of the dispatcher's order.
  // When the blocks and the heads both divide by eight, the jobs form eight lists, one per XCD
  // (blocks are dealt to the XCDs in turn, so block x + 8 i runs on XCD x; list x holds heads
  // x H8 .. +H8, whose keys then stay in that XCD's L2), else one list. A list runs from the
  // longest jobs to the shortest (row blocks from the last, which has the most keys under a
  // causal mask; heads interleaved), and its blocks take them in snake order: in round r, block
  // i of P takes job r P + i when r is even and r P + P - 1 - i when r is odd, so the long jobs of
  // one round pair with the short ones of the next (under a causal mask every block of a list of
  // two rounds gets the same number of key tiles).
  // (32-bit index arithmetic: the jobs, heads and row blocks fit)
  const uint32_t nrb = (uint32_t)((a.n_q + PF_ROWS - 1) / PF_ROWS);
  const uint32_t nbh = (uint32_t)(a.B * a.Hq);
  const bool xlists = gridDim.x % 8u == 0u && nbh % 8u == 0u;
  const uint32_t nlist = xlists ? 8u : 1u;
  const uint32_t lst = blockIdx.x % nlist, lb = blockIdx.x / nlist, lP = gridDim.x / nlist;
  const uint32_t lh = nbh / nlist, ljobs = lh * nrb;
  for (uint32_t round = 0;; ++round) {
  const uint32_t q_ = (round & 1u) ? (round + 1u) * lP - 1u - lb : round * lP + lb;
  if (q_ >= ljobs) break;
  const uint32_t bh = lst * lh + q_ % lh;
  const uint32_t b = bh / (uint32_t)a.Hq, h = bh - b * (uint32_t)a.Hq, g = h / (uint32_t)a.G;
  const int64_t i0 = (int64_t)(nrb - 1 - q_ / lh) * PF_ROWS;
  const unsigned char* kb = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.n * RB;
  const float* ktm = a.w.ktmax + ((size_t)b * a.Hkv + g) * (size_t)((a.n + PF_KEYS - 1) / PF_KEYS);
  const uint32_t LCAP = (uint32_t)a.slot;
  const size_t grow0 = (size_t)bh * a.n_q + i0;  // global row of block row 0
  const int n = (int)a.n;  // the host runs this scan only when n * RB < 2^31

  const int rg = wave >> 2, kg = wave & 3;
  const int m = lane & 15, grp = lane >> 4;
  const int row_base = rg * 64 + 4 * grp;  // block row of register (u, e): row_base + 16 u + e

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
  // clamped. Register set (t & 3) holds the tile that step t writes to LDS (loaded four steps
  // earlier, so that the memory latency stays hidden).
  const int srow = tid / NCH, schunk = tid % NCH;
  const int voff0 = srow * RB + schunk * 16, voff1 = voff0 + RPP * RB;
  uint4 r00 = make_uint4(0u, 0u, 0u, 0u), r01 = r00, r10 = r00, r11 = r00, r20 = r00, r21 = r00, r30 = r00,
        r31 = r00;
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
    unsigned char* dst = &ktiles[((U) % PF_NBUF) * TILE_BYTES + srow * STRIDE + schunk * 16];      \
    *(uint4*)dst = SRC0;                                                                           \
    if (PASSES > 1) *(uint4*)(dst + RPP * STRIDE) = SRC1;                                          \
  }
// Scores of the tile in LDS buffer BUF into ACC (four 16x16 tiles).
#define PF_MMA(ACC, BUF)                                                                           \
  {                                                                                                \
    const unsigned char* krow = &ktiles[(BUF) * TILE_BYTES + (kg * 16 + m) * STRIDE + grp * GB];  \
    uint4 kf[SL];                                                                                  \
    _Pragma("unroll") for (int s = 0; s < SL; ++s) kf[s] = *(const uint4*)(krow + s * 16);        \
    _Pragma("unroll") for (int u = 0; u < 4; ++u) ACC[u] = f32x4_t{};                              \
    _Pragma("unroll") for (int s = 0; s < SL; ++s)                                                 \
      _Pragma("unroll") for (int u = 0; u < 4; ++u)                                                \
        ACC[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[u][s], __builtin_bit_cast(bf16x8_t, kf[s]), ACC[u], 0, 0, 0); \
  }
// Prologue of a pass over the tiles, in two parts: the loads of tiles 0 .. PF_H (for LDS) and of
// the tiles that steps 0 .. 3 write (register sets 0 .. 3), all in flight together; then tiles
// 0 .. PF_H to LDS, scores of tile 0 into ACC, and a barrier so that no wave overwrites tile 0's
// buffer before every wave has read it.
  static_assert(PF_H == 2, "the prologue stages tiles 0 .. 2");
  uint4 p00 = r00, p01 = r00, p10 = r00, p11 = r00, p20 = r00, p21 = r00;
#define PF_PRO_ISSUE()                                                                             \
  {                                                                                                \
    PF_LOAD(p00, p01, 0)                                                                           \
    PF_LOAD(p10, p11, 1)                                                                           \
    PF_LOAD(p20, p21, 2)                                                                           \
    PF_LOAD(r00, r01, PF_H + 1)                                                                    \
    PF_LOAD(r10, r11, PF_H + 2)                                                                    \
    PF_LOAD(r20, r21, PF_H + 3)                                                                    \
    PF_LOAD(r30, r31, PF_H + 4)                                                                    \
  }
#define PF_PRO_FINISH(ACC)                                                                         \
  {                                                                                                \
    PF_STORE(p00, p01, 0)                                                                          \
    PF_STORE(p10, p11, 1)                                                                          \
    PF_STORE(p20, p21, 2)                                                                          \
    __syncthreads();                                                                               \
    PF_MMA(ACC, 0)                                                                                 \
    __syncthreads();                                                                               \
  }
// On a boundary tile, scores of keys that are not candidates of the register's row become -inf.
// With dr = (position of the register's row) - j, key j is a candidate of the row iff
// 1 <= j < n and dr >= W (j before the window) or, without the causal mask, dr < 0 (j after p).
// (Rows past the end of the queries score 0 and get the bound +inf in phase 2, so that none of
// their keys is listed.)
  const int rows_valid = (int)min((int64_t)PF_ROWS, a.n_q - i0);
// (Positions fit in 32 bits here: the scan runs only when n * RB < 2^31. The tests combine with
// & and |, so that the 16 selects need no branches.)
  const int p_first32 = (int)p_first;
  const bool ncausal_ = !a.causal;
#define PF_MASK(ACC, t)                                                                            \
  if (!PF_INTERIOR(t)) {                                                                           \
    const int j_ = (t) * PF_KEYS + kg * 16 + m;                                                    \
    const int dl = p_first32 + row_base - j_;                                                      \
    const bool jok = (j_ >= 1) & (j_ < n);                                                         \
    const int wl = a.W - dl;                                                                       \
    _Pragma("unroll") for (int u = 0; u < 4; ++u)                                                  \
      _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                              \
        const int o = 16 * u + e;                                                                  \
        const bool cand = jok & ((o >= wl) | (ncausal_ & (o < -dl)));                              \
        ACC[u][e] = cand ? ACC[u][e] : -INFINITY;                                                  \
      }                                                                                            \
  }
// One step t of a pass: the scores of tile t are in ACC_CUR (issued a step earlier); the matrix
// cores score tile t+1 into ACC_NEXT while the vector units run the per-score work on tile t:
// PART for each register of ACC_CUR, PER of them after each matrix instruction, then HOOK with
// the instruction's index (phase 2 runs the previous tile's appends there). Tile t + PF_H + 1
// then goes from its registers to its LDS buffer and tile t + PF_H + 5 is requested. Scheduling
// fences keep that order: left to itself the compiler puts the vector work before the matrix
// instructions.
  constexpr int NMMA = 4 * SL;  // matrix instructions per step
#define PF_NOHOOK(i)
#define PF_STEP(PART, HOOK, t, ACC_CUR, ACC_NEXT, SET0, SET1)                                      \
  {                                                                                                \
  PF_MASK(ACC_CUR, t)                                                                              \
  {                                                                                                \
    const unsigned char* krow = &ktiles[(((t) + 1) % PF_NBUF) * TILE_BYTES + (kg * 16 + m) * STRIDE + grp * GB]; \
    uint4 kf[SL];                                                                                  \
    _Pragma("unroll") for (int s = 0; s < SL; ++s) kf[s] = *(const uint4*)(krow + s * 16);        \
    __builtin_amdgcn_sched_barrier(0);                                                             \
    _Pragma("unroll") for (int u = 0; u < 4; ++u) ACC_NEXT[u] = f32x4_t{};                         \
    _Pragma("unroll") for (int s = 0; s < SL; ++s)                                                 \
      _Pragma("unroll") for (int u = 0; u < 4; ++u) {                                              \
        ACC_NEXT[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[u][s], __builtin_bit_cast(bf16x8_t, kf[s]), ACC_NEXT[u], 0, 0, 0); \
        __builtin_amdgcn_sched_barrier(0);                                                         \
        _Pragma("unroll") for (int e = 0; e < PER; ++e) PART(ACC_CUR, t, (s * 4 + u) * PER + e)   \
        HOOK(s * 4 + u)                                                                            \
        __builtin_amdgcn_sched_barrier(0);                                                         \
      }                                                                                            \
  }                                                                                                \
  PF_STORE(SET0, SET1, (t) + PF_H + 1)                                                             \
  PF_LOAD(SET0, SET1, (t) + PF_H + 5)                                                              \
  }

  // phase 1's first tiles are requested before the A operands, the longer wait
  if (ntiles > 0) PF_PRO_ISSUE()
  // The A operands: the block's query rows are loaded once (16-byte chunks spread over the
  // block's threads; the four waves of a row group share their rows), staged in the tile buffers,
  // which are not in use yet (rows STRIDE bytes apart, as the key tiles), and each wave reads its
  // rows' operands from there. Rows past the end of the queries load the last row (their scores
  // are never used: they get the bound +inf in phase 2).
  constexpr int QPT = PF_ROWS * NCH / 512;  // chunks per thread
  static_assert(PF_ROWS * NCH % 512 == 0 && PF_ROWS * STRIDE <= SMEM, "query staging");
  uint4 qv[QPT];
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int c = tid + 512 * j;
    const int64_t i = min(i0 + c / NCH, a.n_q - 1);
    qv[j] = *(const uint4*)(a.q + ((size_t)bh * a.n_q + i) * RB + (c % NCH) * 16);
  }
  if (tid < 2 * 4 * 17) {
    // counter rg * 68 + g * 17 + r (r < 16) is that of block row 64 rg + 4 g + 16 (r >> 2) + (r & 3)
    const uint32_t rr = (uint32_t)(tid % 17), row = (uint32_t)(tid / 68) * 64u + (uint32_t)((tid % 68) / 17) * 4u + rr + 3u * (rr & 12u);
    rowcnt[tid] = 0u;
    rowcnt[2 * 4 * 17 + tid] = rr < 16u ? row * LCAP * 8u : 0u;
  }
  if (tid == 0) kmax_blk = 0u;
  // |q| of the rows whose threshold this lane helps to find (wave w takes rows 16 w .. +16);
  // loaded unconditionally from a clamped index, so that no load waits on another
  float qn_g[4];
#pragma unroll
  for (int gq = 0; gq < 4; ++gq) {
    const int64_t i = i0 + wave * 16 + 4 * gq + (lane >> 4);
    const float qv = a.w.qn[(size_t)bh * a.n_q + min(i, a.n_q - 1)];
    qn_g[gq] = i < a.n_q ? qv : 0.f;
  }
  // the largest norm of the keys the block scores, from the tiles' maxima (after the other loads
  // are in flight: its wait covers them all)
  float knmx = 0.f;
  for (int t = tid; t < ntiles; t += 512) knmx = fmaxf(knmx, ktm[t]);
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int c = tid + 512 * j;
    *(uint4*)&ktiles[(c / NCH) * STRIDE + (c % NCH) * 16] = qv[j];
  }
  __syncthreads();
  bf16x8_t qa[4][SL];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int s = 0; s < SL; ++s)
      qa[u][s] = *(const bf16x8_t*)&ktiles[(rg * 64 + u * 16 + m) * STRIDE + grp * GB + s * 16];
  __syncthreads();  // (before the prologue writes key tiles over the staged rows)

  f32x4_t accA[4], accB[4];
  // ---- phase 1: per lane and row, the two largest fast scores of candidate keys. With m1 >= m2,
  // the new second best is the median of m1, m2 and the score, and the new best is the median of
  // m1, the score and +inf (a run-time operand, so that no NaN-quieting is added around a max).
  const float pinf = a.pinf;
  float m1[16], m2[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) m1[r] = m2[r] = -INFINITY;
// (The empty asm statements pin each result to its place between the matrix instructions;
// without them the compiler sinks the work of a step past the next step's boundary-tile branch.)
#define PF_PART1(ACC, t, r)                                                                        \
  {                                                                                                \
    const float x_ = ACC[(r) >> 2][(r) & 3];                                                       \
    m2[r] = __builtin_amdgcn_fmed3f(m1[r], m2[r], x_);                                             \
    m1[r] = __builtin_amdgcn_fmed3f(m1[r], x_, pinf);                                              \
    asm volatile("" : "+v"(m1[r]), "+v"(m2[r]));                                                   \
  }
  if (ntiles > 0) {
    PF_PRO_FINISH(accA)
    // (the norms arrived with the first tiles; taking them now keeps a wait for them out of the
    // threshold search, where the loads of phase 2's first tiles are in flight)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) asm volatile("" : "+v"(qn_g[gq]));
    // (four steps per turn, one register set each; the turn may end after its second step)
    for (int t = 0; t < ntiles; t += 2 * PF_H) {
      PF_STEP(PF_PART1, PF_NOHOOK, t, accA, accB, r00, r01)
      PF_STEP(PF_PART1, PF_NOHOOK, t + 1, accB, accA, r10, r11)
      __syncthreads();
      if (t + 2 >= ntiles) break;
      PF_STEP(PF_PART1, PF_NOHOOK, t + 2, accA, accB, r20, r21)
      PF_STEP(PF_PART1, PF_NOHOOK, t + 3, accB, accA, r30, r31)
      __syncthreads();
    }
  }

  // phase 2's first tiles are requested now, so that they arrive during the threshold search
  if (ntiles > 0) PF_PRO_ISSUE()
  // the block's largest key norm (norms are non-negative, so their bits order like the values)
  knmx = wave_max_f32(knmx);
  if (lane == 0) atomicMax(&kmax_blk, __float_as_uint(knmx));

  // ---- thresholds: row R's 128 fast scores sit at tops[136 R + 32 kg + 2 m + {0, 1}] (even
  // entries: the lanes' best values, 64 distinct keys; odd entries: their second best; rows 136
  // floats apart, so that the four lane groups' rows fall in different LDS banks). Each row
  // needs a lower bound x of the k-th largest of its 128 values such that few values lie between:
  // the largest x = lo + c (hi - lo) / 128, c = 0..127, that at least k values reach (a bitwise
  // search over c, monotone in c), where hi is the largest value and lo a known lower bound of
  // the k-th largest: for k <= 64 and 64 finite best values the smallest of them, else the
  // smallest finite value (if fewer than k values are finite every candidate stays). The bound is
  // at most (hi - lo) / 128 below the k-th largest, and it is never above it. A wave takes 16
  // rows in four groups of four; the 16 lanes of a row hold 8 values each (lane s: entries
  // 4 s .. +4 and 64 + 4 s .. +4, so that each read is conflict-free), counted lane by lane and
  // summed over the row with DPP moves.
  static_assert(PF_ROWS * 136 * 4 <= SMEM, "the thresholds' values fit in the tile buffers");
  float* tops = (float*)ktiles;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = row_base + 16 * (r >> 2) + (r & 3);
    *(float2*)&tops[row * 136 + 32 * kg + 2 * m] = make_float2(m1[r], m2[r]);
  }
  const int sub = lane & 15;
  __syncthreads();
  const float kmax = __uint_as_float(kmax_blk);
  {
    float v[4][8], lo[4], step[4];
    int c[4];
    bool ok[4];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const float* src = &tops[(wave * 16 + 4 * gq + (lane >> 4)) * 136 + 4 * sub];
      const float4 x0 = *(const float4*)src, x1 = *(const float4*)(src + 64);
      v[gq][0] = x0.x; v[gq][1] = x0.y; v[gq][2] = x0.z; v[gq][3] = x0.w;
      v[gq][4] = x1.x; v[gq][5] = x1.y; v[gq][6] = x1.z; v[gq][7] = x1.w;
      float hi = -INFINITY, lo_best = INFINITY, lo_fin = INFINITY;
      int nfin = 0, nbest = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool fin = v[gq][j] > -INFINITY;
        hi = fmaxf(hi, v[gq][j]);
        nfin += fin;
        lo_fin = fin ? fminf(lo_fin, v[gq][j]) : lo_fin;
        if ((j & 1) == 0) {
          nbest += fin;
          lo_best = fminf(lo_best, v[gq][j]);
        }
      }
      hi = pf_row16<1>(hi);
      nfin = pf_row16<0>(nfin);
      nbest = pf_row16<0>(nbest);
      lo_fin = pf_row16<2>(lo_fin);
      lo_best = pf_row16<2>(lo_best);
      ok[gq] = nfin >= a.topk;
      lo[gq] = a.topk <= 64 && nbest == 64 ? lo_best : lo_fin;
      step[gq] = ok[gq] ? (hi - lo[gq]) * (1.0f / 128.0f) : 0.f;
      lo[gq] = ok[gq] ? lo[gq] : 0.f;
      c[gq] = 0;
    }
#pragma unroll
    // (per step, the four groups' counts, at most 128 each, travel in the four bytes of one word
    // through the 16-lane sum; a lane counts the values below the candidate from the sign bits
    // of the differences)
    for (int bit = 6; bit >= 0; --bit) {
      uint32_t packed = 0u;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const float cand = fmaf((float)(c[gq] | (1 << bit)), step[gq], lo[gq]);
        uint32_t below = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) below = __builtin_amdgcn_alignbit(below, __float_as_uint(v[gq][j] - cand), 31);
        packed |= (uint32_t)(8 - __popc(below & 0xFFu)) << (8 * gq);
      }
      packed = pf_row16<0>(packed);
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int cc = c[gq] | (1 << bit);
        c[gq] = (int)((packed >> (8 * gq)) & 0xFFu) >= a.topk ? cc : c[gq];
      }
    }
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int row = wave * 16 + 4 * gq + (lane >> 4);
      if (sub == 0) {
        // T = x - 2 C |q| max|k|, one rounding (the product by a power of two is exact)
        const float x = ok[gq] ? fmaf(-2.0f * PF_EPS_COEF * qn_g[gq], kmax, fmaf((float)c[gq], step[gq], lo[gq]))
                               : -INFINITY;
        // kept finite (at least the lowest float), so that the -inf of a masked score never
        // passes; +inf for rows past the end of the queries
        lthk[row] = row < rows_valid ? fmaxf(x, -0x1.fffffep+127f) : INFINITY;
      }
    }
  }
  __syncthreads();
  float tk[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) tk[r] = lthk[row_base + 16 * (r >> 2) + (r & 3)];

  // ---- phase 2: every candidate key whose fast score reaches its row's bound goes to the row's
  // list in global memory, with its score. A lane gathers the test results of its 16 registers
  // into bit r of `fail`'s complement: the test x >= T is the sign of x - T (T finite or +inf, x
  // finite or -inf), shifted in by v_alignbit from register 15 down to 0. At the end of step t
  // every lane writes its 16 scores to its own place in LDS; the keys of its passing registers
  // are then appended one per round during step t + 1: the score read back by register index, a
  // slot from the row's LDS counter (shared by the four waves of the row group), the store. Two
  // rounds run between the matrix instructions of step t + 1 (their LDS round trips overlap the
  // matrix work); a lane with more passing registers finishes them in a loop at the end of that
  // step, before the stage is rewritten. Slots past LCAP are not written; the count then tells
  // the finish that the row overflowed.
  // (a wave's stage holds its lanes' score register r at r * 64 + lane, so that a lane finds
  // register r with one shift-add and neither the writes nor the reads conflict; the row
  // counters are kept in the order rg, g, register, padded to 17 per g, so that register r of a
  // lane finds its row's counter at cnt_l[r], its row list's byte offset at cnt_l[r + 136], and
  // the four groups' counters fall in different LDS banks)
  float* const sst_w = sstage + wave * 1024;
  uint32_t* const cnt_l = rowcnt + rg * 68 + grp * 17;
  const uint32_t kc0 = (uint32_t)(kg * 16 + m);
  uint2* const survb = a.w.surv + grow0 * LCAP;
  uint32_t fail = 0u;
  uint32_t pend = 0u, pkey = 0u;  // the staged tile's passing registers not yet appended, its key
#define PF_PART2(ACC, t, r)                                                                        \
  {                                                                                                \
    const int r_ = 15 - (r);                                                                       \
    fail = __builtin_amdgcn_alignbit((r) == 0 ? 0u : fail, __float_as_uint(ACC[r_ >> 2][r_ & 3] - tk[r_]), 31); \
    asm volatile("" : "+v"(fail));                                                                 \
  }
// one append round of the staged tile: issue (score and slot requested together), then store
#define PF_ROUND_ISSUE(X)                                                                          \
  X##_on = pend != 0u;                                                                             \
  if (X##_on) {                                                                                    \
    const uint32_t r_ = (uint32_t)__builtin_ctz(pend);                                             \
    pend &= pend - 1u;                                                                             \
    X##_x = sst_w[r_ * 64u + lane];                                                                \
    X##_slot = atomicAdd(&cnt_l[r_], 1u);                                                          \
    X##_off = cnt_l[r_ + 2 * 4 * 17];                                                              \
  }
#define PF_ROUND_STORE(X)                                                                          \
  if (X##_on && X##_slot < LCAP)                                                                   \
    *(uint2*)((char*)survb + (X##_off + X##_slot * 8u)) = make_uint2(__float_as_uint(X##_x), pkey);
  // (round A is issued after matrix instruction 1 and stored after NMMA / 2 + 1; round B after
  // NMMA / 4 and NMMA - 1 - NMMA / 8: a few matrix instructions cover each LDS round trip)
  bool ra_on = false, rb_on = false;
  float ra_x = 0.f, rb_x = 0.f;
  uint32_t ra_slot = 0u, rb_slot = 0u, ra_off = 0u, rb_off = 0u;
#define PF_HOOK2(i)                                                                                \
  if ((i) == 1) { PF_ROUND_ISSUE(ra) }                                                             \
  if ((i) == NMMA / 4) { PF_ROUND_ISSUE(rb) }                                                      \
  if ((i) == NMMA / 2 + 1) { PF_ROUND_STORE(ra) }                                                  \
  if ((i) == NMMA - 1 - NMMA / 8) { PF_ROUND_STORE(rb) }
// the rest of the staged tile's appends, one per round
#define PF_DRAIN()                                                                                 \
  if (pend) {                                                                                      \
    do {                                                                                           \
      const uint32_t r_ = (uint32_t)__builtin_ctz(pend);                                           \
      pend &= pend - 1u;                                                                           \
      const float x_ = sst_w[r_ * 64u + lane];                                                     \
      const uint32_t slot_ = atomicAdd(&cnt_l[r_], 1u);                                            \
      const uint32_t off_ = cnt_l[r_ + 2 * 4 * 17];                                                \
      if (slot_ < LCAP)                                                                            \
        *(uint2*)((char*)survb + (off_ + slot_ * 8u)) = make_uint2(__float_as_uint(x_), pkey);       \
    } while (pend);                                                                                \
  }
// end of step t: finish the previous tile's appends, then stage this tile's scores (every lane:
// with no branch around the writes the LDS waits that follow stay exact)
#define PF_POST2(ACC, t)                                                                           \
  {                                                                                                \
    PF_DRAIN()                                                                                     \
    _Pragma("unroll") for (int r = 0; r < 16; ++r) sst_w[r * 64 + lane] = ACC[r >> 2][r & 3];      \
    pend = ~fail & 0xFFFFu;                                                                        \
    pkey = kc0 + (uint32_t)(t) * PF_KEYS;                                                          \
  }
  if (ntiles > 0) {
    PF_PRO_FINISH(accA)
    for (int t = 0; t < ntiles; t += 2 * PF_H) {
      PF_STEP(PF_PART2, PF_HOOK2, t, accA, accB, r00, r01)
      PF_POST2(accA, t)
      PF_STEP(PF_PART2, PF_HOOK2, t + 1, accB, accA, r10, r11)
      PF_POST2(accB, t + 1)
      __syncthreads();
      if (t + 2 >= ntiles) break;
      PF_STEP(PF_PART2, PF_HOOK2, t + 2, accA, accB, r20, r21)
      PF_POST2(accA, t + 2)
      PF_STEP(PF_PART2, PF_HOOK2, t + 3, accB, accA, r30, r31)
      PF_POST2(accB, t + 3)
      __syncthreads();
    }
    PF_DRAIN()
  }

  // the count word: entries from the front of the row's slots in its low 16 bits, 0 in the high
  // 16 bits; a count above LCAP sends the row to the exact path. Block row R = 64 rg + 16 u + 4 g
  // + e has its counter at 68 rg + 17 g + 4 u + e.
  __syncthreads();
  if (tid < PF_ROWS && i0 + tid < a.n_q)
    a.w.cnt[grow0 + tid] = min(rowcnt[(tid >> 6) * 68 + ((tid >> 2) & 3) * 17 + ((tid >> 4) & 3) * 4 + (tid & 3)], 0xFFFFu);
  __syncthreads();  // (the next job resets the counters and overwrites the tile buffers)
  }
#undef PF_INTERIOR
#undef PF_LOAD
#undef PF_STORE
#undef PF_PRO_ISSUE
#undef PF_PRO_FINISH
#undef PF_MMA
#undef PF_MASK
#undef PF_STEP
#undef PF_PART1
#undef PF_PART2
#undef PF_POST2
#undef PF_DRAIN
#undef PF_HOOK2
#undef PF_ROUND_ISSUE
#undef PF_ROUND_STORE
#undef PF_NOHOOK
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
__device__ __forceinline__ void pf_window_block(const PfArgs& a) {
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

// One launch for the window's share and the norms: blocks [0, nwin) are window blocks, the rest
// norm blocks. Both read only the inputs, so neither waits for the other; the norm blocks fill
// the compute units that the window's last round of blocks leaves idle, and the launch and the
// separate norm pass's ramp are saved.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void pf_window_kernel(PfArgs a, PfNormArgs na,
                                                                                               uint32_t nwin) {
  if (blockIdx.x < nwin) pf_window_block<D>(a);
  else pf_norm_block<D, 4>(na, blockIdx.x - nwin);
}

// ---------------------------------------------------------------------------------------------
// pf_finish: one wave per query row (4 rows per 256-thread block), each wave with its own LDS
// region laid out by PfRowSmem::carve for the call's k and 1 + W + k.
constexpr int PF_FIN_SET = 4096;   // largest 1 + W + k served by the per-row finish
// (tidx and cw have room for the V gather's padding: the entries rounded up to a multiple of
// PF_GATHER, as positions and as float32 weights). The float64 query shares its space with cw:
// every path has read qd for the last time before it writes cw.
constexpr int PF_GATHER = 144;
// Two layouts. The general one (float32 inputs, or k > 64) keeps float64 scores and positions of
// the whole set. The compact one (bf16 inputs, k <= 64) keeps only what that path touches: the
// list and its scores, the top-k, the weights and the float64 query, none of it sized by the
// window, so its LDS does not grow with W. Its radix histogram (exact path only, where the list
// is never loaded) lies over rs[1 ..] and ridx; rs[0] keeps the anchor's score on that path.
struct PfRowSmem {
  double* qd;      // [128], in the space of cw
  double* rs;      // general: [slot + set_cap] float64 scores of the list, window and anchor keys;
                   // compact: [slot + 1] the list's scores, the anchor's, the band's float64 scores
  double* ts;      // [k + 1]
  double* cw;      // general: [max(set_cap, PF_GATHER / 2, 128)]; compact: [128]; or float32
                   // weights [round_up(k + 1, PF_GATHER)]
  int32_t* ridx;   // [slot + 1]: the list, then the anchor
  int32_t* tidx;   // [round_up(k + 1, PF_GATHER)]
  int32_t* cidx;   // general: [set_cap]; compact: none (the set goes from registers to the output)
  uint32_t* hist;  // [256]
  static __host__ __device__ bool compact(bool bf16, int k) { return bf16 && k <= 64; }
  static __host__ __device__ size_t tcap(int k) { return ((size_t)k + PF_GATHER) / PF_GATHER * PF_GATHER; }
  static __host__ __device__ size_t wcap(int k, int set_cap) {
    const size_t w = (tcap(k) + 1) / 2, s = (size_t)set_cap > 128 ? (size_t)set_cap : 128;
    return s > w ? s : w;
  }
  // compact: rs and ridx (the histogram over them), rounded to 16 bytes
  static __host__ __device__ size_t lcap(int64_t slot) {
    const size_t l = ((size_t)slot + 1) * 12, h = 8 + 256 * 4, m = l > h ? l : h;
    return (m + 15) & ~(size_t)15;
  }
  static __host__ __device__ size_t bytes(int64_t slot, int k, int set_cap, bool cmp) {
    const size_t kk = (size_t)k + 1;
    if (cmp) {
      const size_t wc = tcap(k) * 4 > 128 * 8 ? tcap(k) * 4 : 128 * 8;
      return lcap(slot) + ((kk * 8 + 15) & ~(size_t)15) + wc + tcap(k) * 4;
    }
    return ((size_t)slot + set_cap) * 8 + kk * 8 + wcap(k, set_cap) * 8 + tcap(k) * 4 +
           (size_t)set_cap * 4 + ((size_t)slot + 1) * 4 + 256 * 4 + 64;
  }
  __device__ void carve(unsigned char* p, int64_t slot, int k, int set_cap, bool cmp) {
    const size_t kk = (size_t)k + 1;
    if (cmp) {
      rs = (double*)p;
      ridx = (int32_t*)(p + ((size_t)slot + 1) * 8);
      hist = (uint32_t*)(p + 8);
      p += lcap(slot);
      ts = (double*)p;
      p += (kk * 8 + 15) & ~(size_t)15;
      cw = (double*)p;
      qd = cw;
      p += tcap(k) * 4 > 128 * 8 ? tcap(k) * 4 : 128 * 8;
      tidx = (int32_t*)p;
      cidx = nullptr;
      return;
    }
    rs = (double*)p;
    p += ((size_t)slot + set_cap) * 8;
    ts = (double*)p;
    p += kk * 8;
    cw = (double*)p;
    qd = cw;
    p += wcap(k, set_cap) * 8;
    ridx = (int32_t*)p;
    p += ((size_t)slot + 1) * 4;
    tidx = (int32_t*)p;
    p += tcap(k) * 4;
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
// OFF32: every byte offset into a kv head's rows fits in 32 bits (n * row bytes <= 2^32), so the
// gathers take a 32-bit offset from the head's base address.
template <int D, bool BF16, bool OFF32>
__device__ void pf_row(const PfArgs& a, PfRowSmem* sm, size_t grow) {
  constexpr int RB = D * (BF16 ? 2 : 4);
  // a key row is LPR lanes x 16 bytes, so one load instruction covers RPI rows
  constexpr int LPR = RB / 16, RPI = 64 / LPR, EPC = BF16 ? 8 : 4;
  const int lane = threadIdx.x & 63;
  // (32-bit divisions when the rows allow)
  size_t bh;
  int64_t i;
  if (a.rows < ((int64_t)1 << 31)) {
    const uint32_t g32 = (uint32_t)grow, nq = (uint32_t)a.n_q, bh32 = g32 / nq;
    bh = bh32;
    i = (int64_t)(g32 - bh32 * nq);
  } else {
    bh = grow / (size_t)a.n_q;
    i = (int64_t)(grow - bh * (size_t)a.n_q);
  }
  const int b = (int)((uint32_t)bh / (uint32_t)a.Hq), h = (int)((uint32_t)bh - (uint32_t)b * (uint32_t)a.Hq),
            g = (int)((uint32_t)h / (uint32_t)a.G);
  const unsigned char* kb = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.n * RB;
  const unsigned char* vb = a.v ? a.v + ((size_t)b * a.Hkv + g) * (size_t)a.n * RB : nullptr;
  const int64_t p = a.q_pos0 + i;
  const unsigned char* qrow = a.q + grow * RB;
  const int gq = lane / LPR, cc = lane % LPR;
  // error-bound inputs: |q| of the row (requested early) and |k| of each listed key
  const float qn_row = a.w.qn[grow];
  const float* knh = a.w.kn + ((size_t)b * a.Hkv + g) * (size_t)a.n;
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
  int32_t path = PATH_NONE;
  if (a.topk > 0) {
    // The count word and the row's whole slot area (at most 128 entries, two per lane) are read
    // together, so that the list costs one memory round trip. The scan filled c_f slots from the
    // front and c_b from the back; the slots between hold stale entries and are ignored.
    uint32_t cf = 0xFFFFu, cb = 0xFFFFu;
    uint2 e0 = make_uint2(0u, 0u), e1 = e0;
    const int L = (int)a.slot;
    if (!a.exact_all) {
      const uint2* sv = a.w.surv + grow * (size_t)a.slot;
      const uint32_t cr = a.w.cnt[grow];
      cf = cr & 0xFFFFu;
      cb = cr >> 16;
      if (lane < L) e0 = sv[lane];
      if (lane + 64 < L) e1 = sv[lane + 64];
    }
    exact = cf + cb > (uint32_t)L;
    if (exact) path = a.exact_all ? PATH_EXACT_ASKED : PATH_EXACT_OVERFLOW;
    if (!exact) {
      // the entries, packed: positions come from the scan and are always keys of the cache
      // (clamping only guards the reads below); with bf16 inputs the scan's matrix-core scores
      // come along
      const bool v0 = lane < L && (lane < (int)cf || lane >= L - (int)cb);
      const bool v1 = lane + 64 < L && (lane + 64 < (int)cf || lane + 64 >= L - (int)cb);
      const uint64_t b0 = __ballot(v0), b1 = __ballot(v1);
      c = (int)(cf + cb);
      if (v0) {
        const int at = lanes_below(b0);
        sm->ridx[at] = (int32_t)min(e0.y, (uint32_t)(a.n - 1));
        if constexpr (BF16) sm->rs[at] = (double)__uint_as_float(e0.x);
      }
      if (v1) {
        const int at = __popcll(b0) + lanes_below(b1);
        sm->ridx[at] = (int32_t)min(e1.y, (uint32_t)(a.n - 1));
        if constexpr (BF16) sm->rs[at] = (double)__uint_as_float(e1.x);
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
    if (exact) {
      fill_qd();
      nt = pf_exact_row<D, BF16>(sm, a, kb, p);
    } else if (c > a.topk) {
      // Each entry's bounds L = s_mc - eps_j <= s <= U = s_mc + eps_j, eps_j = C |q| |k_j|.
      // T_L = k-th largest L; A = entries with U >= T_L. Every entry outside A scores below k
      // entries, so the top-k lies in A, and if |A| = k it is A. Otherwise, with T_U the k-th
      // largest U over A, an entry with L > T_U is surely in the top-k (only entries with
      // U > T_U, at most k - 1 of them counting itself, can score above it), and the rest of A,
      // the band, is ranked by float64 canonical scores, then by position; its best
      // k - (sure entries) complete the top-k.
      const float cqr = PF_EPS_COEF * qn_row;
      const float s0 = lane < c ? (float)sm->rs[lane] : 0.f;
      const float s1 = lane + 64 < c ? (float)sm->rs[lane + 64] : 0.f;
      const float e0 = lane < c ? cqr * knh[sm->ridx[lane]] : 0.f;
      const float e1 = lane + 64 < c ? cqr * knh[sm->ridx[lane + 64]] : 0.f;
      const uint32_t lk0 = ord_f32(s0 - e0), lk1 = ord_f32(s1 - e1);
      const uint32_t uk0 = ord_f32(s0 + e0), uk1 = ord_f32(s1 + e1);
      const uint32_t key[2] = {lane < c ? lk0 : 0u, lane + 64 < c ? lk1 : 0u};
      const uint32_t TL = wave_kth_largest<2>(key, a.topk);
      const bool in0 = lane < c && uk0 >= TL, in1 = lane + 64 < c && uk1 >= TL;
      const uint64_t m0 = __ballot(in0), m1 = __ballot(in1);
      const int na = __popcll(m0) + __popcll(m1);
      path = na == a.topk ? PATH_FAST : PATH_BAND;
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
        const uint32_t ukey[2] = {in0 ? uk0 : 0u, in1 ? uk1 : 0u};
        const uint32_t TU = wave_kth_largest<2>(ukey, a.topk);
        const bool su0 = in0 && lk0 > TU, su1 = in1 && lk1 > TU;
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
          const uint64_t ki = ord_f64(si);
          const int32_t ji = sm->ridx[t];
          int rank = 0;
          for (int r = 0; r < nb; ++r) {
            const uint64_t kr = ord_f64(sm->rs[r]);
            rank += (kr > ki) || (kr == ki && sm->ridx[r] < ji);
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
      path = PATH_ALL;
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
        const uint64_t ki = ord_f64(si);
        const int32_t ji = sm->ridx[t];
        int rank = 0;
        for (int r = 0; r < c; ++r) {
          const uint64_t kr = ord_f64(sm->rs[r]);
          rank += (kr > ki) || (kr == ki && sm->ridx[r] < ji);
        }
        if (rank < a.topk) {
          sm->tidx[rank] = ji;
          sm->ts[rank] = si;
        }
      }
      nt = a.topk;
      path = PATH_FAST;
      __builtin_amdgcn_wave_barrier();
    } else if (c > 0) {
      for (int t = lane; t < c; t += 64) {
        sm->tidx[t] = sm->ridx[t];
        sm->ts[t] = sm->rs[t];
      }
      nt = c;
      path = PATH_ALL;
      __builtin_amdgcn_wave_barrier();
    }
  }

  if (lane == 0) a.w.path[grow] = path;

  // ---- set: {0} u window u T, ascending
  const int count = anchor + nwin + nt;
  if (BF16 && nt <= 64) {
    // The top-k positions sorted across the wave (distinct keys; empty slots sort last), then
    // every part of the set stored straight to the output: the t-th smallest position at slot
    // anchor + t, after the window if it lies past p; the window after the positions below it.
    uint32_t x = lane < nt ? (uint32_t)sm->tidx[lane] : 0xFFFFFFFFu;
    wave_sort64_asc_u32(x);
    const int tlo = __popcll(__ballot(lane < nt && (int64_t)x < w_lo));
    if (a.sel_idx) {
      int32_t* dst = a.sel_idx + grow * (size_t)a.set_cap;
      if (anchor && lane == 0) dst[0] = 0;
      if (lane < nt) dst[anchor + lane + ((int64_t)x > p ? nwin : 0)] = (int32_t)x;
      for (int t = lane; t < nwin; t += 64) dst[anchor + tlo + t] = (int32_t)(w_lo + t);
      for (int t = count + lane; t < a.set_cap; t += 64) dst[t] = -1;
    }
  } else {
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
    uint32_t x[2] = {(uint32_t)sm->tidx[lane], lane + 64 < nt ? (uint32_t)sm->tidx[lane + 64] : 0xFFFFFFFFu};
    wave_sort_asc_u32<2>(x);
    sm->cidx[anchor + lane + ((int64_t)x[0] > p ? nwin : 0)] = (int32_t)x[0];
    if (lane + 64 < nt) sm->cidx[anchor + lane + 64 + ((int64_t)x[1] > p ? nwin : 0)] = (int32_t)x[1];
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
  }
  if (a.sel_count && lane == 0) a.sel_count[grow] = count;
  if (!a.out) return;

  // ---- softmax over the set and the weighted V rows: lane group gq takes the entries
  // t = gq (mod RPI), each lane a 16-byte chunk of the row; then the groups are summed.
  constexpr int U = BF16 ? 6 : 4;  // V rows per lane group in flight together (bf16: 24 rows per batch at d = 128)
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
    // V row chunk of entry t. The entries are padded to a multiple of U * RPI with the first
    // entry's position (and a zero weight below), so that no load waits behind a branch and
    // every LDS index is a constant offset.
    static_assert(PF_GATHER % (U * RPI) == 0, "gather padding");
    const int npad = ne > 0 ? (ne + U * RPI - 1) / (U * RPI) * (U * RPI) : 0;
    for (int t = ne + lane; t < npad; t += 64) sm->tidx[t] = sm->tidx[0];
    __builtin_amdgcn_wave_barrier();
    auto vrow = [&](int t) -> uint4 {
      const uint32_t j = (uint32_t)sm->tidx[t];
      if constexpr (OFF32) return *(const uint4*)(vb + (j * (uint32_t)RB + (uint32_t)(cc * 16)));
      else return *(const uint4*)(vb + (size_t)j * RB + cc * 16);
    };
    uint4 x[U];
    if (ne > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = vrow(u * RPI + gq);
    }
    float4 wo[EPC / 4];
#pragma unroll
    for (int e = 0; e < EPC / 4; ++e)
      wo[e] = a.win && gq == 0 ? ((const float4*)(a.w.win_o + grow * D + cc * EPC))[e] : make_float4(0.f, 0.f, 0.f, 0.f);
    // (the weights go to the float32 array wf, which the bf16 path leaves unused otherwise)
    float* const wf = (float*)sm->cw;
    float zmax = mz.x;
    for (int t = lane; t < ne; t += 64) zmax = fmaxf(zmax, sc * (float)sm->ts[t]);
    zmax = wave_max_fast(zmax);
    float zsum = 0.f;
    for (int t = lane; t < ne; t += 64) {
      const float w = __expf(sc * (float)sm->ts[t] - zmax);
      wf[t] = w;
      zsum += w;
    }
    for (int t = ne + lane; t < npad; t += 64) wf[t] = 0.f;
    const float fw = a.win ? __expf(mz.x - zmax) : 0.f;
    zsum = wave_sum_fast(zsum) + fw * mz.y;
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
        for (int u = 0; u < U; ++u) x[u] = vrow(t0 + u * RPI + gq);
      }
      float w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) w[u] = wf[t0 + u * RPI + gq];
      accumulate(x, w);
    }
    // the lane groups' sums (groups of LPR lanes hold the same output elements)
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      if constexpr (LPR <= 8) acc[e] += lane_xor_f32<8>(acc[e]);
      if constexpr (LPR <= 16) acc[e] += lane_xor_f32<16>(acc[e]);
      acc[e] += lane_xor_f32<32>(acc[e]);
    }
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

// pf_finish: one wave per query row, 4 rows per block (consecutive rows of one head). OFF32 as in
// pf_row (chosen at launch: one row variant per kernel keeps the register count down).
template <int D, bool BF16, bool OFF32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void pf_finish_kernel(PfArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  // (the wave index through readfirstlane: the row's indices stay in scalar registers)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  PfRowSmem smv;
  smv.carve(smem_raw + wave * a.wave_smem, a.slot, a.topk, a.set_cap, PfRowSmem::compact(BF16, a.topk));
  const size_t grow = (size_t)xcd_job(blockIdx.x, gridDim.x) * 4 + wave;  // (b*Hq + h) * n_q + i
  if (grow >= (size_t)a.rows) return;
  pf_row<D, BF16, OFF32>(a, &smv, grow);
}

// ---------------------------------------------------------------------------------------------
// Blocks of pf_scan the current device holds at once (compute units times blocks per unit),
// queried once per device and kept (racing first calls store the same value).
template <int D>
static int64_t pf_scan_slots() {
  constexpr int MAX_DEV = 64;
  static std::atomic<int64_t> cache[MAX_DEV];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  if (dev >= 0 && dev < MAX_DEV) {
    const int64_t c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 256, per = 1, v = 0, nb = 0;
  if (dev >= 0 && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, pf_scan_kernel<D>, 512, 0) == hipSuccess && nb > 0) per = nb;
  const int64_t slots = (int64_t)cus * per;
  if (dev >= 0 && dev < MAX_DEV) cache[dev].store(slots, std::memory_order_relaxed);
  return slots;
}

template <int D, bool BF16>
static hipError_t launch_pf_t(const PrefillLaunch& L, const PfArgs& pa, hipStream_t s) {
  const size_t rows = (size_t)L.B * L.Hq * (size_t)L.n_q;
  hipError_t e = hipSuccess;
  if constexpr (BF16) {
    // norms for the error bounds of the matrix-core scores (only the fast selection uses them)
    // and the window's share of the softmax, in one launch when both are needed; both before the
    // scan
    constexpr int RPW = 64 / (D * 2 / 16), QU = 4;  // rows per wave load; loads per lane
    const bool norms = !pa.exact_all && L.topk > 0;
    PfNormArgs na{};
    uint64_t nnorm = 0;
    if (norms) {
      const uint64_t qblocks = (rows + 4 * QU * RPW - 1) / (4 * QU * RPW);
      const uint64_t kblocks = ((uint64_t)L.n + 4 * QU * RPW - 1) / (4 * QU * RPW);
      nnorm = qblocks + kblocks * (uint64_t)(L.B * L.Hkv);
      na = PfNormArgs{(const unsigned char*)L.q, (int64_t)rows, pa.w.qn, (const unsigned char*)L.k, L.n, pa.w.kn,
                      pa.w.ktmax, (uint32_t)qblocks, (uint32_t)kblocks};
    }
    const uint64_t nwin = pa.win ? (uint64_t)((L.n_q + 63) / 64) * (uint64_t)(L.B * L.Hq) : 0;
    if (nwin + nnorm > 0x7FFFFFFFull) return hipErrorInvalidValue;
    if (nwin + nnorm > 0) {
      if (nwin > 0)
        hipLaunchKernelGGL((pf_window_kernel<D>), dim3((unsigned)(nwin + nnorm)), dim3(256), 0, s, pa, na, (uint32_t)nwin);
      else
        hipLaunchKernelGGL((pf_norm_kernel<D, QU>), dim3((unsigned)nnorm), dim3(256), 0, s, na);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (L.ev_scan_begin) (void)hipEventRecord(L.ev_scan_begin, s);
  if (!pa.exact_all && L.topk > 0) {
    if constexpr (BF16) {
      const int64_t jobs = (L.n_q + PF_ROWS - 1) / PF_ROWS * L.B * L.Hq;
      const int64_t slots = pf_scan_slots<D>();
      hipLaunchKernelGGL((pf_scan_kernel<D>), dim3((unsigned)(jobs < slots ? jobs : slots)), dim3(512), 0, s, pa);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (L.ev_scan_end) (void)hipEventRecord(L.ev_scan_end, s);
  const size_t smem = 4 * pa.wave_smem;
  const bool off32 = (uint64_t)L.n * (uint64_t)(D * (BF16 ? 2 : 4)) <= 0xFFFFFFFFull;
  const void* fk = off32 ? (const void*)pf_finish_kernel<D, BF16, true> : (const void*)pf_finish_kernel<D, BF16, false>;
  if (smem > 48 * 1024) (void)hipFuncSetAttribute(fk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (off32)
    hipLaunchKernelGGL((pf_finish_kernel<D, BF16, true>), dim3((unsigned)((rows + 3) / 4), 1), dim3(256), smem, s, pa);
  else
    hipLaunchKernelGGL((pf_finish_kernel<D, BF16, false>), dim3((unsigned)((rows + 3) / 4), 1), dim3(256), smem, s, pa);
  return hipGetLastError();
}

// The finish gives each of its 4 waves (rows) its own LDS region; all four must fit the 160 KB of a
// compute unit.
bool prefill_fits(int32_t W, int32_t k, bool bf16) {
  const int set_cap = 1 + W + k;
  if (set_cap > PF_FIN_SET) return false;
  const size_t wave_smem =
      (PfRowSmem::bytes(pf_slot(k), k, set_cap, PfRowSmem::compact(bf16, k)) + 255) & ~(size_t)255;
  return 4 * wave_smem <= 160 * 1024;
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
  pa.w = pf_carve(L.ws, L.B, L.Hq, L.Hkv, L.n_q, L.n, L.d, L.topk);
  pa.n = L.n;
  pa.n_q = L.n_q;
  pa.q_pos0 = L.q_pos0;
  pa.slot = pf_slot(L.topk);
  pa.B = L.B;
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
  pa.wave_smem = (PfRowSmem::bytes(pa.slot, L.topk, pa.set_cap, PfRowSmem::compact(L.bf16, L.topk)) + 255) & ~(size_t)255;
  if (!prefill_fits(L.W, L.topk, L.bf16)) return hipErrorNotSupported;
  if (L.bf16) return L.d == 128 ? launch_pf_t<128, true>(L, pa, stream) : launch_pf_t<64, true>(L, pa, stream);
  return L.d == 128 ? launch_pf_t<128, false>(L, pa, stream) : launch_pf_t<64, false>(L, pa, stream);
}

}  // namespace topo
