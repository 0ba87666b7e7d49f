// Decode path of Topological Attention on gfx950: one query per (batch, query head).
//
// "The Condensate Theorem: Transformers are O(n), Not O(n^2)" (gist.science explainers of
// arXiv 2602.06317): the condensate set of a query is the anchor (position 0), the W most recent
// tokens and the top-k keys by Q.K^T, found again at every decoding step (zh page, technical
// summary §3; ko page, technical summary §3 "동적 선택"); attention is the softmax over that set
// only (fr page, technical summary §3).
//
// Three launches per call:
//   decode_window  the window's share of the softmax per (batch, query head), in parts of a few
//                  dozen rows (float64), and the clearing of the per-head scan state
//                  (decode_init clears it alone when no softmax is asked for).
//   kscan          stream K once per (batch, kv head) for all G query heads of the group
//                  (HBM bound). Fast float32 scores with a proven error bound; every wave keeps
//                  the keys that could still be in the top-k of its run of 512 keys, raises a
//                  shared per-head threshold, and appends the survivors to a per-head list.
//   decode_finish  per (batch, query head): exact k-th threshold over the survivors, float64
//                  re-scoring of the short list, exact top-k by (score desc, position asc), set
//                  assembly, float64 softmax and V reduction over the anchor and the top-k,
//                  combined with decode_window's records.
#include "topo_device.h"
#include "topo_internal.h"

// Tuning: blocks of the key scan that must fit on one CU (bounds its registers), and whether its
// loads carry the non-temporal hint.
#ifndef TOPO_KS_MIN_BLOCKS
#define TOPO_KS_MIN_BLOCKS 2
#endif
#ifndef TOPO_KS_NT
#define TOPO_KS_NT 1
#endif

namespace topo {

// ---------------------------------------------------------------------------------------------
// Error bound of the fast scores. The bf16 path sums exact products with v_dot2_f32_bf16 and the
// float32 path with fused multiply-adds, then adds the per-lane partial sums in a tree; d terms in
// all, and every term passes through at most d + 4 roundings of at most two units each, so
// |s_fast - s| <= 2 (d + 4) u sum_t |q_t k_t| <= 2 (d + 4) u |q| |k| (Cauchy-Schwarz), u = 2^-24.
// The extra 2^-20 |q| |k| covers rounding the bound itself and forming s_fast +- eps in float32.
float fast_score_eps_coef(int d) { return (float)(2.0 * (d + 4) * 0x1p-24 + 0x1p-20); }

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int64_t scan_blocks(const QueryGeom& g, int runs) {
  const int64_t span = (int64_t)KS_KEYS_PER_RUN * runs;
  return (g.scan_hi + span) / span;
}

// Runs per key-scan block: the largest count that still leaves at least two blocks per compute
// unit (fewer, longer blocks amortise each block's start and survivor merge; too few blocks
// would leave compute units idle).
static int scan_runs(const QueryGeom& g, int64_t groups) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  for (int r = KS_MAX_RUNS; r > 1; r >>= 1)
    if (scan_blocks(g, r) * groups >= 2 * (int64_t)cus) return r;
  return 1;
}
static int64_t scan_slot(int32_t k) { return k + 32 < KS_WAVE_CAP ? k + 32 : KS_WAVE_CAP; }

// Number of survivor-list levels: merge until the last level fits the finishing kernel's LDS.
static int survivor_levels(int64_t nblk0, int64_t slot, int64_t (&nblk)[MAX_LEVELS]) {
  int L = 0;
  nblk[L++] = nblk0;
  while (nblk[L - 1] * slot > SURV_LDS && L < MAX_LEVELS) {
    nblk[L] = (nblk[L - 1] + MERGE_FAN - 1) / MERGE_FAN;
    ++L;
  }
  return L;
}

// Window rows per decode_window block: four rows per group of RB / 16 lanes of its 256 threads.
static int window_rows(int32_t d, int32_t bf16) { return 4 * (256 / (d * (bf16 ? 2 : 4) / 16)); }
// decode_window blocks (records) per (batch, query head): enough for the longest window.
static int64_t window_parts(const QueryGeom& g, int32_t d, int32_t bf16) {
  const int64_t nwin = g.p - g.w_lo + 1, wr = window_rows(d, bf16);
  return nwin > 0 ? (nwin + wr - 1) / wr : 0;
}

size_t decode_workspace_bytes(int32_t B, int32_t Hq, const QueryGeom& g, int32_t k, int32_t d, int32_t bf16) {
  const size_t heads = (size_t)B * Hq;
  const int64_t slot = scan_slot(k);
  int64_t nb[MAX_LEVELS];
  // sized for one run per block: the most blocks, so any run count chosen at launch fits
  const int L = survivor_levels(scan_blocks(g, 1), slot, nb);
  size_t bytes = align256(heads * sizeof(HeadState));
  bytes += align256(heads * (size_t)window_parts(g, d, bf16) * (size_t)(d + 2) * sizeof(double));
  for (int l = 0; l < L; ++l)
    bytes += align256(heads * (size_t)nb[l] * 4) + align256(heads * (size_t)nb[l] * (size_t)slot * sizeof(uint2)) +
             align256(heads * (size_t)nb[l] * (size_t)slot * sizeof(float));
  return bytes;
}

void decode_carve(void* ws, int32_t B, int32_t Hq, const QueryGeom& g, int32_t k, DecodeLaunch& L) {
  const size_t heads = (size_t)B * Hq;
  L.slot = scan_slot(k);
  L.wstride = window_parts(g, L.d, L.bf16);
  const int GT = L.G >= 4 ? 4 : L.G;
  L.runs = scan_runs(g, (int64_t)L.B * L.Hkv * ((L.G + GT - 1) / GT));
  L.nlevels = survivor_levels(scan_blocks(g, L.runs), L.slot, L.nblk);
  char* p = (char*)ws;
  L.st = (HeadState*)p;
  p += align256(heads * sizeof(HeadState));
  L.wrec = (double*)p;
  p += align256(heads * (size_t)L.wstride * (size_t)(L.d + 2) * sizeof(double));
  for (int l = 0; l < L.nlevels; ++l) {
    L.blk_cnt[l] = (uint32_t*)p;
    p += align256(heads * (size_t)L.nblk[l] * 4);
    L.surv[l] = (uint2*)p;
    p += align256(heads * (size_t)L.nblk[l] * (size_t)L.slot * sizeof(uint2));
    L.surv_eps[l] = (float*)p;
    p += align256(heads * (size_t)L.nblk[l] * (size_t)L.slot * sizeof(float));
  }
}

DecodeView decode_view(int32_t B, int32_t Hq, int32_t Hkv, const QueryGeom& g, int32_t k, int32_t d, int32_t bf16) {
  DecodeLaunch L{};
  L.B = B;
  L.Hq = Hq;
  L.Hkv = Hkv;
  L.G = Hq / Hkv;
  L.d = d;
  L.bf16 = bf16;
  decode_carve(nullptr, B, Hq, g, k, L);
  DecodeView v;
  v.state = (size_t)(uintptr_t)L.st;
  v.count = (size_t)(uintptr_t)L.blk_cnt[0];
  v.entry = (size_t)(uintptr_t)L.surv[0];
  v.eps = (size_t)(uintptr_t)L.surv_eps[0];
  v.lists = L.nblk[0];
  v.slot = L.slot;
  return v;
}

// Geometry of batch element b's query from its position pos[b] (clamped into the cache; causal).
__device__ __forceinline__ QueryGeom ragged_geom(const int64_t* pos, int b, int64_t n, int32_t W) {
  const int64_t p = pos[b];
  return make_geom(p < 0 ? 0 : (p > n - 1 ? n - 1 : p), n, W, true);
}

__global__ void decode_init_kernel(HeadState* st, int nheads) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nheads) {
    st[i].theta = 0u;
    st[i].overflow = 0u;
  }
}

// ---------------------------------------------------------------------------------------------
// decode_window: the window's share of the softmax, before the key scan (it needs only the query
// and the cache). One block per (query head bh, part j) takes window rows [j * WR, (j + 1) * WR)
// of the head (the window is the W positions up to p; fr page, technical summary §3, the softmax
// over the set) and writes one record: O_j = sum_r exp(z_r - m_j) v_r (d values), m_j = max_r z_r
// and Z_j = sum_r exp(z_r - m_j), with z_r = scale * q.k_r in float64 (an empty part writes
// m_j = -inf, Z_j = 0, O_j = 0). The finishing kernel combines the records with the rest of the
// set. Block 0 also clears the per-head scan state, the job of decode_init when this kernel runs.
// 256 threads: groups of LPR = RB / 16 lanes hold one row each (a 16-byte chunk per lane), four
// rows per group; the K and V chunks of all of them are requested at once.
struct WindowArgs {
  const unsigned char* q;
  const unsigned char* k;
  const unsigned char* v;
  HeadState* st;
  double* rec;       // [B * Hq][rstride][D + 2]
  const int64_t* pos;  // may be null: causal query position of each batch element
  int64_t n, p, w_lo, rstride;
  int32_t Hq, Hkv, G, W, nheads;
  int32_t rstride_parts;  // blocks (parts) per head in this launch
  double scale;
};

template <int D, bool BF16>
__global__ __launch_bounds__(256) void decode_window_kernel(WindowArgs a) {
  constexpr int RB = D * (BF16 ? 2 : 4), LPR = RB / 16, RPP = 256 / LPR, U = 4, EPC = BF16 ? 8 : 4;
  constexpr int WR = U * RPP;
  __shared__ double red[4][D];
  __shared__ double scr[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (blockIdx.x == 0) {
    for (int i = tid; i < a.nheads; i += 256) {
      a.st[i].theta = 0u;
      a.st[i].overflow = 0u;
    }
  }
  // Job order: (batch, kv head, part, query head of the group), dealt to the XCDs in contiguous
  // ranges, so that the G blocks reading the same K and V rows share one XCD's L2.
  const int64_t job = xcd_job(blockIdx.x, gridDim.x);
  const int hh = (int)(job % a.G);
  const int64_t gp = job / a.G;
  const int part = (int)(gp % a.rstride_parts), bg = (int)(gp / a.rstride_parts);
  const int b = bg / a.Hkv, g = bg - b * a.Hkv, h = g * a.G + hh;
  const int bh = b * a.Hq + h;
  int64_t p = a.p, w_lo = a.w_lo;
  if (a.pos) {
    const QueryGeom gq = ragged_geom(a.pos, b, a.n, a.W);
    p = gq.p;
    w_lo = gq.w_lo;
  }
  const int nwin = (int)(p - w_lo + 1);
  const unsigned char* kb = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.n * RB;
  const unsigned char* vb = a.v + ((size_t)b * a.Hkv + g) * (size_t)a.n * RB;
  const int rsub = tid / LPR, cc = tid % LPR;
  // every load first: the query chunk, then the K and V chunks of the four rows (row indexes
  // clamped into the cache; rows past the window are ignored below)
  const uint4 qc = *(const uint4*)(a.q + (size_t)bh * RB + cc * 16);
  uint4 kx[U], vx[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int64_t j = w_lo + part * WR + u * RPP + rsub;
    j = j > a.n - 1 ? a.n - 1 : j;
    kx[u] = *(const uint4*)(kb + (size_t)j * RB + cc * 16);
    vx[u] = *(const uint4*)(vb + (size_t)j * RB + cc * 16);
  }
  double qd[EPC];
  {
    const uint32_t w4[4] = {qc.x, qc.y, qc.z, qc.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (BF16) {
        qd[2 * e] = bf16_lo(w4[e]);
        qd[2 * e + 1] = bf16_hi(w4[e]);
      } else {
        qd[e] = __uint_as_float(w4[e]);
      }
    }
  }
  // logits: float64 partial dot of the lane's chunk, summed over the LPR lanes of the row
  double z[U];
  double zm = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t w4[4] = {kx[u].x, kx[u].y, kx[u].z, kx[u].w};
    double part_s = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (BF16) {
        part_s = fma(qd[2 * e], (double)bf16_lo(w4[e]), part_s);
        part_s = fma(qd[2 * e + 1], (double)bf16_hi(w4[e]), part_s);
      } else {
        part_s = fma(qd[e], (double)__uint_as_float(w4[e]), part_s);
      }
    }
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) part_s += __shfl_xor(part_s, o);
    const bool valid = part * WR + u * RPP + rsub < nwin;
    z[u] = valid ? a.scale * part_s : -INFINITY;
    zm = fmax(zm, z[u]);
  }
  const double m = block_max_f64<4>(zm, scr);
  double wsum = 0.0;
  double acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const double w = z[u] > -INFINITY ? exp(z[u] - m) : 0.0;
    if (cc == 0) wsum += w;
    const uint32_t w4[4] = {vx[u].x, vx[u].y, vx[u].z, vx[u].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (BF16) {
        acc[2 * e] = fma(w, (double)bf16_lo(w4[e]), acc[2 * e]);
        acc[2 * e + 1] = fma(w, (double)bf16_hi(w4[e]), acc[2 * e + 1]);
      } else {
        acc[e] = fma(w, (double)__uint_as_float(w4[e]), acc[e]);
      }
    }
  }
  const double zs = block_sum_f64<4>(wsum, scr);
  // the rows of a wave that share chunk cc: lanes cc + LPR * i
#pragma unroll
  for (int e = 0; e < EPC; ++e)
    for (int o = LPR; o < 64; o <<= 1) acc[e] += __shfl_xor(acc[e], o);
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < EPC; ++e) red[wave][cc * EPC + e] = acc[e];
  }
  __syncthreads();
  double* rec = a.rec + ((size_t)bh * a.rstride + part) * (D + 2);
  if (tid < D) rec[tid] = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
  if (tid == 0) {
    rec[D] = m;
    rec[D + 1] = zs;
  }
}

// ---------------------------------------------------------------------------------------------

// ---------------------------------------------------------------------------------------------
// kscan: grid (nblk, B*Hkv, ceil(G/GT)), 256 threads = 4 waves. Block x ranks keys
// [2048 runs x, +2048 runs) for the GT query heads of its slice, in `runs` runs of 4 x 512 keys
// (wave w takes the w-th 512 keys of each run).
//
// A key row of RB bytes is spread over L = RB/16 lanes (one 16-byte chunk each), so every load
// instruction is fully coalesced and each lane keeps only its chunk of the GT queries in
// registers. Partial dot products of 64 keys are combined by a reduce-scatter over the L lanes,
// after which every lane owns one key. Each wave keeps the keys that may be in the top-k of its
// run, the block merges its four waves' survivors into one list per head, and a shared per-head
// threshold lets later blocks drop keys that can no longer be selected.
struct KscanArgs {
  const unsigned char* k;
  const unsigned char* q;
  HeadState* st;
  uint32_t* blk_cnt;
  uint2* surv;
  float* surv_eps;
  int64_t n, nblk, slot;
  int64_t p, w_lo, vis_hi, scan_hi;
  const int64_t* pos;  // may be null: causal query position of each batch element
  int32_t Hq, Hkv, G, W, topk, runs;
  int32_t group;       // 1: one selection per kv head (group score = largest of the heads' scores)
  float eps_coef;
};


// Loads of one 64-key tile. The 64 lanes form 8 groups of 8; group r handles keys 8i + r of the
// tile (i = 0..7) and lane s of a group holds 16-byte chunks c*8 + s (c < CPL) of each of them:
// every load instruction reads eight 128-byte line-aligned half rows.
template <int RB>
__device__ __forceinline__ void kscan_load(uint4 (&buf)[8][RB / 128], const unsigned char* kb, int64_t row0,
                                           int64_t last_row, int lane) {
  constexpr int CPL = RB / 128;
  const int r = lane >> 3, s = lane & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = row0 + 8 * i + r;
    const unsigned char* p = kb + (row <= last_row ? row : last_row) * RB + s * 16;
#pragma unroll
    for (int c = 0; c < CPL; ++c) buf[i][c] = TOPO_KS_NT ? ntload16(p + c * 128) : *(const uint4*)(p + c * 128);
  }
}

// RAGGED: per-sequence positions; GROUP: one shared selection per kv head (template switches, so
// the plain scan carries none of their registers).
template <int RB, int GT, bool BF16, bool RAGGED, bool GROUP>
__global__ __launch_bounds__(256, TOPO_KS_MIN_BLOCKS) void kscan_kernel(KscanArgs a) {
  constexpr int L = 8;          // lanes per key row
  constexpr int CPL = RB / 128; // 16-byte chunks of a row per lane
  __shared__ uint2 wbuf[KS_WAVES][GT][KS_WAVE_CAP];
  __shared__ float wbe[KS_WAVES][GT][KS_WAVE_CAP];  // each entry's error bound
  __shared__ int wcnt[KS_WAVES][GT];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, s = lane & 7;
  const int grp = blockIdx.y;
  const int b = grp / a.Hkv, g = grp - b * a.Hkv;
  const int slice0 = blockIdx.z * GT;
  const int h0 = g * a.G + slice0;
  const int nh = min(GT, a.G - slice0);
  // the query's geometry: the call's, or (RAGGED) that of this sequence's position
  int64_t q_p = a.p, q_wlo = a.w_lo, q_vis = a.vis_hi, q_scan = a.scan_hi;
  if constexpr (RAGGED) {
    // the grid covers the longest scan; blocks past this sequence's candidates leave empty lists
    const QueryGeom gq = ragged_geom(a.pos, b, a.n, a.W);
    q_p = gq.p;
    q_wlo = gq.w_lo;
    q_vis = gq.vis_hi;
    q_scan = gq.scan_hi;
    if ((int64_t)blockIdx.x * KS_KEYS_PER_RUN * a.runs > q_scan) {
      if (tid < nh) a.blk_cnt[((size_t)b * a.Hq + h0 + tid) * (size_t)a.nblk + blockIdx.x] = 0u;
      return;
    }
  }

  // This lane's chunks of every query of the slice, and |q_h| (float64 sum over the 8 lanes).
  uint4 qv[GT][CPL];
  float qn[GT];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    double part = 0.0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      qv[h][c] = h < nh ? *(const uint4*)(a.q + ((size_t)b * a.Hq + h0 + h) * RB + c * 128 + s * 16)
                        : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t w4[4] = {qv[h][c].x, qv[h][c].y, qv[h][c].z, qv[h][c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (BF16) {
          const double lo = bf16_lo(w4[e]), hi = bf16_hi(w4[e]);
          part += lo * lo + hi * hi;
        } else {
          const double x = __uint_as_float(w4[e]);
          part += x * x;
        }
      }
    }
    for (int o = 1; o < L; o <<= 1) part += __shfl_xor(part, o);
    qn[h] = (float)sqrt(part) * (1.0f + 0x1p-20f);
  }
  // With cq[h] = eps_coef |q_h|, a key of norm |k| has the error bound cq[h] |k| (its own).
  // Shared selection: the group score max_h s_h of a key is ranked as the scores of one head
  // (slot 0); |max_h s^_h - max_h s_h| <= max_h eps_h, so head 0 takes the largest |q_h|.
  const int nsel = GROUP ? 1 : nh;
  if constexpr (GROUP) {
#pragma unroll
    for (int h = 1; h < GT; ++h)
      if (h < nh) qn[0] = fmaxf(qn[0], qn[h]);
  }
  float cq[GT];
#pragma unroll
  for (int h = 0; h < GT; ++h) cq[h] = a.eps_coef * qn[h];

  // The block ranks a.runs runs of KS_WAVES x KS_KEYS_PER_WAVE keys; tile it of run r (KS_ROWS
  // keys) of wave w is tile (r KS_IT + it) KS_WAVES + w of the block, so that the four waves take
  // consecutive tiles and the block streams one contiguous range (a read-only probe streams
  // faster that way than with each wave on a range of its own).
  const int64_t blk_key0 = (int64_t)blockIdx.x * KS_KEYS_PER_RUN * a.runs;
  auto tile_key0 = [&](int r, int it) -> int64_t {
    return blk_key0 + ((int64_t)(r * KS_IT + it) * KS_WAVES + wave) * KS_ROWS;
  };
  const unsigned char* kb = a.k + (size_t)grp * (size_t)a.n * RB;
  const int64_t last_row = q_scan;
  const int64_t my_off = 8 * s + (lane >> 3);  // key of this lane within a tile after the reduction

  float sc[GT][KS_IT];
  float kn[KS_IT];  // norm of the lane's key of each tile of the run (rounded up)
  uint32_t vmask = 0;

  // One tile in registers. Per key group i (8 keys, one per lane group): partial dot products of
  // this lane's chunks with every query of the slice and the partial squared norm of the key;
  // right after that the registers of group i are reloaded with group i of the next tile (of
  // this run or the next), so loads stream out during the whole scan. The loads are
  // unconditional (rows past the end of the scan are clamped to its last row and never
  // selected), which keeps the wait counts exact. Then per head, and for the squared norms, a
  // reduce-scatter over the 8 lanes, and the scores and norms enter register shift queues
  // (sc[h][KS_IT-1] is the newest) so that every register index stays static. The squares of
  // bf16 values are exact in float32 and the float32 sum of the d squares carries a relative
  // error below 2^-19 (float32 data: below 2^-18), covered by the factor that rounds the norm up.
  uint4 kv[8][CPL];
  kscan_load<RB>(kv, kb, tile_key0(0, 0), last_row, lane);
  const int kr = lane >> 3;
  auto tile = [&](int64_t row0, int64_t nrow0, bool more) {
    const bool nfull = nrow0 + 63 <= last_row;
    const unsigned char* nbase = kb + (nrow0 + kr) * RB + s * 16;
    float P[GT][8];
    float N2[1][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc = dot_chunk<BF16>(kv[i][c], qv[h][c], acc);
        P[h][i] = acc;
      }
      float n2 = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) n2 = dot_chunk<BF16>(kv[i][c], kv[i][c], n2);
      N2[0][i] = n2;
      if (more) {
        const int64_t row = nrow0 + 8 * i + kr;
        const unsigned char* p = nfull ? nbase + (size_t)i * 8 * RB : kb + (row <= last_row ? row : last_row) * RB + s * 16;
#pragma unroll
        for (int c = 0; c < CPL; ++c) kv[i][c] = TOPO_KS_NT ? ntload16(p + c * 128) : *(const uint4*)(p + c * 128);
      }
    }
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      float Q1[1][8];
#pragma unroll
      for (int i = 0; i < 8; ++i) Q1[0][i] = P[h][i];
      reduce_scatter<8, 1>(Q1, s);
#pragma unroll
      for (int i = 0; i + 1 < KS_IT; ++i) sc[h][i] = sc[h][i + 1];
      sc[h][KS_IT - 1] = Q1[0][0];
    }
    reduce_scatter<8, 1>(N2, s);
#pragma unroll
    for (int i = 0; i + 1 < KS_IT; ++i) kn[i] = kn[i + 1];
    kn[KS_IT - 1] = sqrtf(N2[0][0]) * (1.0f + 0x1p-16f);
    const int64_t j = row0 + my_off;
    const bool valid = j >= 1 && j <= q_vis && (j < q_wlo || j > q_p);
    vmask = (vmask >> 1) | ((valid ? 1u : 0u) << (KS_IT - 1));
  };

  int wtotal[GT];       // survivors of each head handed to the block merge so far
  uint32_t trun[GT];    // each head's best threshold of this wave's runs so far
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    wtotal[h] = 0;
    trun[h] = 0u;
  }
#pragma unroll 1
  for (int r = 0; r < a.runs; ++r) {
    // The shared thresholds are read now, so the load overlaps the run (a stale value is still a
    // valid bound: the shared threshold only ever rises). Unconditional loads keep the wait
    // counts of the tile stream exact.
    uint32_t thp[GT];
#pragma unroll
    for (int h = 0; h < GT; ++h)
      thp[h] = __hip_atomic_load(&a.st[(size_t)b * a.Hq + h0 + (h < nh ? h : nh - 1)].theta, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll 1
    for (int it = 0; it + 1 < KS_IT; ++it) tile(tile_key0(r, it), tile_key0(r, it + 1), true);
    tile(tile_key0(r, KS_IT - 1), tile_key0(r + 1, 0), r + 1 < a.runs);
    if constexpr (GROUP) {
#pragma unroll
      for (int it = 0; it < KS_IT; ++it)
#pragma unroll
        for (int h = 1; h < GT; ++h)
          if (h < nh) sc[0][it] = fmaxf(sc[0][it], sc[h][it]);
    }
    const bool any_valid = __ballot(vmask != 0u) != 0ull;
    if (!any_valid) continue;

    // Local thresholds: k distinct keys of this run have lower bounds (score minus the key's own
    // error bound) at or above T (earlier runs' thresholds stay valid). For k <= 64 all heads
    // share one bitwise search over the k-th largest of each lane's two best lower bounds;
    // larger k take the exact k-th largest.
    if (a.topk <= 64) {
      uint32_t m0[GT], m1[GT], T[GT];
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float x0 = -INFINITY, x1 = -INFINITY;
#pragma unroll
        for (int it = 0; it < KS_IT; ++it) {
          const float x = ((vmask >> it) & 1u) ? sc[h][it] - cq[h] * kn[it] : -INFINITY;
          x1 = fmaxf(x1, fminf(x0, x));
          x0 = fmaxf(x0, x);
        }
        m0[h] = x0 == -INFINITY ? 0u : ord_f32(x0);
        m1[h] = x1 == -INFINITY ? 0u : ord_f32(x1);
        T[h] = 0u;
      }
      // The search only matters where it can beat the best known bound: fewer than k values
      // above it means this run's threshold is lower (the common case after the first run).
      bool any_search = false;
      bool search[GT];
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const uint32_t cur = max(trun[h], thp[h]);
        search[h] = h < nsel && cur < 0xFFFFFFFFu &&
                    __popcll(__ballot(m0[h] > cur)) + __popcll(__ballot(m1[h] > cur)) >= a.topk;
        any_search |= search[h];
      }
      if (any_search) {
        for (int bit = 31; bit >= 0; --bit) {
#pragma unroll
          for (int h = 0; h < GT; ++h) {
            const uint32_t cand = T[h] | (1u << bit);
            const int c = __popcll(__ballot(m0[h] >= cand)) + __popcll(__ballot(m1[h] >= cand));
            if (c >= a.topk) T[h] = cand;
          }
        }
#pragma unroll
        for (int h = 0; h < GT; ++h)
          if (search[h]) trun[h] = max(trun[h], T[h]);
      }
    } else {
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        if (h >= nsel) break;
        uint32_t lb[KS_IT];
#pragma unroll
        for (int it = 0; it < KS_IT; ++it) lb[it] = ((vmask >> it) & 1u) ? ord_f32(sc[h][it] - cq[h] * kn[it]) : 0u;
        trun[h] = max(trun[h], wave_kth_largest<KS_IT>(lb, a.topk));
      }
    }

#pragma unroll
    for (int h = 0; h < GT; ++h) {
      if (h >= nsel) break;
      const uint32_t th_g = thp[h];
      const uint32_t th = max(trun[h], th_g);
      // Hand this run's survivors (upper bound at or above the threshold) to the block merge,
      // each with its own error bound.
#pragma unroll
      for (int it = 0; it < KS_IT; ++it) {
        const float e = cq[h] * kn[it];
        const bool ok = ((vmask >> it) & 1u) && ord_f32(sc[h][it] + e) >= th;
        const uint64_t m = __ballot(ok);
        if (ok) {
          const int pos = wtotal[h] + lanes_below(m);
          if (pos < KS_WAVE_CAP) {
            wbuf[wave][h][pos] = make_uint2(__float_as_uint(sc[h][it]), (uint32_t)(tile_key0(r, it) + my_off));
            wbe[wave][h][pos] = e;
          }
        }
        wtotal[h] += __popcll(m);
      }
      // Before the next run, cut a long list to the k-th best lower bound among its entries (a
      // valid threshold: k distinct keys reach it), in place: every lane reads its entries first.
      if (r + 1 < a.runs && wtotal[h] > KS_WAVE_CAP / 2 && wtotal[h] <= KS_WAVE_CAP) {
        constexpr int PER = KS_WAVE_CAP / 64;
        uint2 e[PER];
        float ee[PER];
        uint32_t lbk[PER];
        const int c = wtotal[h];
#pragma unroll
        for (int t = 0; t < PER; ++t) {
          const int idx = lane + 64 * t;
          e[t] = idx < c ? wbuf[wave][h][idx] : make_uint2(0u, 0u);
          ee[t] = idx < c ? wbe[wave][h][idx] : 0.f;
          lbk[t] = idx < c ? ord_f32(__uint_as_float(e[t].x) - ee[t]) : 0u;
        }
        trun[h] = max(trun[h], wave_kth_largest<PER>(lbk, a.topk));
        const uint32_t thc = max(trun[h], th_g);
        __builtin_amdgcn_wave_barrier();
        int nc = 0;
#pragma unroll
        for (int t = 0; t < PER; ++t) {
          const int idx = lane + 64 * t;
          const bool keep = idx < c && ord_f32(__uint_as_float(e[t].x) + ee[t]) >= thc;
          const uint64_t m = __ballot(keep);
          if (keep) {
            wbuf[wave][h][nc + lanes_below(m)] = e[t];
            wbe[wave][h][nc + lanes_below(m)] = ee[t];
          }
          nc += __popcll(m);
        }
        wtotal[h] = nc;
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GT; ++h) wcnt[wave][h] = wtotal[h];
  }
  __syncthreads();

  // Block merge: wave h merges the four waves' survivors of query head h (shared selection: wave
  // 0 the group's, and the other heads of the slice get empty lists).
  if (wave >= nsel) {
    if (wave < nh && lane == 0) a.blk_cnt[((size_t)b * a.Hq + h0 + wave) * (size_t)a.nblk + blockIdx.x] = 0u;
    return;
  }
  const int h = wave;
  const size_t head = (size_t)b * a.Hq + h0 + h;
  HeadState* hs = a.st + head;
  const size_t bslot = head * (size_t)a.nblk + blockIdx.x;
  static_assert(KS_WAVES == 4, "the block merge below is written for four waves");
  const int c0 = wcnt[0][h], c1 = wcnt[1][h], c2 = wcnt[2][h], c3 = wcnt[3][h];
  const bool over = c0 > KS_WAVE_CAP || c1 > KS_WAVE_CAP || c2 > KS_WAVE_CAP || c3 > KS_WAVE_CAP;
  const int p1 = c0, p2 = c0 + c1, p3 = c0 + c1 + c2;
  const int total = p3 + c3;
  if (over) {
    if (lane == 0) {
      a.blk_cnt[bslot] = KS_OVERFLOW;
      hs->overflow = 1u;
    }
    return;
  }
  // Entries are read from LDS on every pass (few registers stay live).
  auto wsel = [&](int idx, int& i) -> int {
    const int w = (idx >= p1) + (idx >= p2) + (idx >= p3);
    i = idx - (w == 0 ? 0 : w == 1 ? p1 : w == 2 ? p2 : p3);
    return w;
  };
  auto lbkey = [&](int idx) -> uint32_t {
    if (idx >= total) return 0u;
    int i;
    const int w = wsel(idx, i);
    return ord_f32(__uint_as_float(wbuf[w][h][i].x) - wbe[w][h][i]);
  };
  constexpr int PER = KS_WAVES * KS_WAVE_CAP / 64;
  uint32_t T = 0;
  if (total >= a.topk) {
    if (a.topk <= 64) {
      uint32_t m[2] = {0u, 0u};
      for (int r = 0; r < PER; ++r) {
        const uint32_t x = lbkey(lane + 64 * r);
        m[1] = max(m[1], min(m[0], x));
        m[0] = max(m[0], x);
      }
      T = wave_kth_largest<2>(m, a.topk);
    } else {
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        int c = 0;
        for (int r = 0; r < PER; ++r) c += __popcll(__ballot(lbkey(lane + 64 * r) >= cand));
        if (c >= a.topk) T = cand;
      }
    }
  }
  const uint32_t th_g = *(volatile const uint32_t*)&hs->theta;
  const uint32_t th = max(T, th_g);
  uint2* out = a.surv + bslot * (size_t)a.slot;
  float* oeps = a.surv_eps + bslot * (size_t)a.slot;
  int cnt = 0;
  for (int r = 0; r < PER; ++r) {
    const int idx = lane + 64 * r;
    uint2 e = make_uint2(0u, 0u);
    float ee = 0.f;
    if (idx < total) {
      int i;
      const int w = wsel(idx, i);
      e = wbuf[w][h][i];
      ee = wbe[w][h][i];
    }
    const bool ok = idx < total && ord_f32(__uint_as_float(e.x) + ee) >= th;
    const uint64_t m = __ballot(ok);
    if (ok) {
      const int pos = cnt + lanes_below(m);
      if (pos < a.slot) {
        out[pos] = e;
        oeps[pos] = ee;
      }
    }
    cnt += __popcll(m);
  }
  if (lane == 0) {
    if (cnt > a.slot) {
      a.blk_cnt[bslot] = KS_OVERFLOW;
      hs->overflow = 1u;
    } else {
      a.blk_cnt[bslot] = (uint32_t)cnt;
    }
    if (T > th_g) atomicMax(&hs->theta, T);
  }
}

// ---------------------------------------------------------------------------------------------
// merge_lists: one wave per (group of MERGE_FAN survivor lists, head). Keeps the entries of the
// group that may still be in the top-k: the k-th best lower bound of the group (or the shared
// threshold, if higher) against every entry's upper bound, each entry with its own error bound.
// Output has the same layout, one list per group.
struct MergeArgs {
  const HeadState* st;
  HeadState* st_w;
  const uint32_t* cnt_in;
  const uint2* surv_in;
  const float* eps_in;
  uint32_t* cnt_out;
  uint2* surv_out;
  float* eps_out;
  int64_t nblk_in, nblk_out, slot;
  int32_t topk;
};

__global__ __launch_bounds__(64) void merge_lists_kernel(MergeArgs a) {
  constexpr int PER = MERGE_FAN * KS_WAVE_CAP / 64;
  const int lane = threadIdx.x;
  const size_t head = blockIdx.y;
  const int64_t g0 = (int64_t)blockIdx.x * MERGE_FAN;
  const int nin = (int)min((int64_t)MERGE_FAN, a.nblk_in - g0);
  const size_t in0 = head * (size_t)a.nblk_in + g0;
  const size_t oslot = head * (size_t)a.nblk_out + blockIdx.x;
  uint32_t c = 0;
  if (lane < nin) c = a.cnt_in[in0 + lane];
  const bool over = __ballot(c == KS_OVERFLOW) != 0ull;
  if (over) {
    if (lane == 0) {
      a.cnt_out[oslot] = KS_OVERFLOW;
      a.st_w[head].overflow = 1u;
    }
    return;
  }
  const int incl = wave_incl_scan_i32((int)c);
  const int total = __shfl(incl, 63);
  int pre[MERGE_FAN];  // start of list i in the flat order
#pragma unroll
  for (int i = 0; i < MERGE_FAN; ++i) pre[i] = i == 0 ? 0 : __shfl(incl, i - 1);
  uint2 ent[PER];
  float ee[PER];
  uint32_t lbk[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int f = lane + 64 * r;
    ent[r] = make_uint2(0u, 0u);
    ee[r] = 0.f;
    if (f < total) {
      int w = 0;
#pragma unroll
      for (int i = 1; i < MERGE_FAN; ++i) w += f >= pre[i] && i < nin;
      int base = 0;
#pragma unroll
      for (int i = 0; i < MERGE_FAN; ++i) base = i == w ? pre[i] : base;
      const size_t at = (in0 + w) * (size_t)a.slot + (f - base);
      ent[r] = a.surv_in[at];
      ee[r] = a.eps_in[at];
    }
  }
#pragma unroll
  for (int r = 0; r < PER; ++r) lbk[r] = lane + 64 * r < total ? ord_f32(__uint_as_float(ent[r].x) - ee[r]) : 0u;
  const uint32_t T = total >= a.topk ? wave_threshold<PER>(lbk, a.topk) : 0u;
  const uint32_t th = max(T, a.st[head].theta);
  uint2* out = a.surv_out + oslot * (size_t)a.slot;
  float* oeps = a.eps_out + oslot * (size_t)a.slot;
  int cnt = 0;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const bool ok = lane + 64 * r < total && ord_f32(__uint_as_float(ent[r].x) + ee[r]) >= th;
    const uint64_t m = __ballot(ok);
    if (ok) {
      const int pos = cnt + lanes_below(m);
      if (pos < a.slot) {
        out[pos] = ent[r];
        oeps[pos] = ee[r];
      }
    }
    cnt += __popcll(m);
  }
  if (lane == 0) {
    if (cnt > a.slot) {
      a.cnt_out[oslot] = KS_OVERFLOW;
      a.st_w[head].overflow = 1u;
    } else {
      a.cnt_out[oslot] = (uint32_t)cnt;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// decode_finish: one block of 512 threads per (batch, query head).
//   1. Stage the head's scan survivors in LDS (every load in flight at once), as order keys of
//      their lower and upper score bounds (each entry with its own key's error bound).
//   2. A threshold T that at least k of the survivors' lower bounds reach (distinct keys, so no
//      key whose upper bound is below T can be in the top-k): for k <= 64 a ten-step search for
//      the largest T = lo + c (hi - lo) / 1024 between the smallest of the 64 lane maxima and the
//      largest value, which lies at most (hi - lo) / 1024 below the k-th largest lower bound; for
//      larger k, or a narrower range, the exact k-th largest by a bitwise search. The short list
//      is every survivor whose upper bound reaches T (it holds the whole top-k).
//   3. Float64 canonical scores of the short list and the anchor; exact ranks by (score desc,
//      position asc).
//   4. The set {0} u window u top-k, ascending.
//   5. Float64 softmax and weighted V rows over the anchor and the top-k, merged with the
//      window's share from decode_window's records.
// Ties crowding the short list, overflowing scan blocks, k above the scan's limit and the
// TOPO_FLAG_EXACT_SELECT flag all route to an exact radix select over every candidate instead.
constexpr int FIN_THREADS = 512;
constexpr int FIN_WAVES = FIN_THREADS / 64;

struct FinishArgs {
  const unsigned char* q;
  const unsigned char* k;
  const unsigned char* v;
  float* out;
  int32_t* sel_idx;
  int32_t* sel_count;
  float* rho;
  HeadState* st;
  const uint32_t* blk_cnt;
  const uint2* surv;
  const float* surv_eps;
  int64_t n, nblk, slot;
  int64_t p, w_lo, vis_hi, scan_hi, n_cand;
  const int64_t* pos;  // may be null: causal query position of each batch element
  const double* wrec;  // the window kernel's records: [B * Hq][wstride][D + 2] (partial output, m, Z)
  int64_t wstride;
  int32_t wparts;      // records per head written by the window kernel (0: none)
  int32_t Hq, Hkv, G, W, topk, set_cap, flags;
  double scale;
  float eps_coef;
};

struct FinishSmem {
  double qd[128];
  double qg[4][128];  // shared selection: the float64 queries of the group's heads
  union {
    struct {                       // phases 1-2
      uint32_t lbk[SURV_LDS];
      uint32_t ubk[SURV_LDS];
      int32_t sidx[SURV_LDS];
    } s;
    struct {                       // phases 3-5
      int32_t tidx[MAX_SET];       // the top-k part (any order)
      double ts[MAX_SET];
      int32_t cidx[MAX_SET];       // the set, ascending
      double cw[MAX_SET];          // its scores, then its softmax weights
    } c;
  } u;
  uint32_t hist[2048];
  int32_t ridx[REFINE_CAP];
  double rs[REFINE_CAP];
  double rg[REFINE_CAP];  // shared selection: group scores of the short list
  uint64_t rkey[REFINE_CAP];  // order keys of the short list's ranking scores
  double red[FIN_WAVES * 128];
  double scratch[FIN_WAVES];
  double2 wmz[8];  // (maximum logit, sum) of the first window records
  double ascore;   // float64 score of the anchor
  int32_t ival[8];
};

// One wave finds, scanning bins from the top, the bin where the running count reaches `need`.
// Writes the bin (or -1) and the count strictly above it into sm->ival[0..1].
__device__ void find_bin_from_top(FinishSmem* sm, int nbins, int64_t need) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int64_t above = 0;
    int found = -1;
    for (int top = nbins - 1; top >= 0 && found < 0; top -= 64) {
      const int bin = top - lane;
      const int c = bin >= 0 ? (int)sm->hist[bin] : 0;
      const int incl = wave_incl_scan_i32(c);  // lane 0 = highest bin of this chunk
      const uint64_t hit = __ballot(above + incl >= need && c > 0);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        const int excl = __shfl(incl - c, l);
        found = top - l;
        above += excl;
      } else {
        above += __shfl(incl, 63);
      }
    }
    if (lane == 0) {
      sm->ival[0] = found;
      sm->ival[1] = (int)above;
    }
  }
  __syncthreads();
}

// Kept out of line: each call site then reuses one register allocation for the row and the query.
template <int D, bool BF16>
__device__ __attribute__((noinline)) double score_row(const FinishSmem* sm, const unsigned char* kb, int64_t j) {
  constexpr int RB = D * (BF16 ? 2 : 4);
  return canonical_score_row<BF16, D>(sm->qd, kb + (size_t)j * RB);
}

// Canonical score of key j for the float64 query qd (LDS).
template <int D, bool BF16>
__device__ __attribute__((noinline)) double score_row_q(const double* qd, const unsigned char* kb, int64_t j) {
  constexpr int RB = D * (BF16 ? 2 : 4);
  return canonical_score_row<BF16, D>(qd, kb + (size_t)j * RB);
}

// Group score of key j for a shared selection: the largest of the G heads' canonical scores.
template <int D, bool BF16>
__device__ double group_score_row(const FinishSmem* sm, const unsigned char* kb, int64_t j, int G) {
  double m = score_row_q<D, BF16>(sm->qg[0], kb, j);
  for (int i = 1; i < G; ++i) m = fmax(m, score_row_q<D, BF16>(sm->qg[i], kb, j));
  return m;
}

__device__ __forceinline__ bool is_candidate(const FinishArgs& a, int64_t j) {
  return j >= 1 && j <= a.vis_hi && (j < a.w_lo || j > a.p);
}

// Exact selection over every candidate by float64 radix select on the canonical scores
// (8 passes of 8 bits), then collection in ascending position so that equal scores resolve to
// the lower positions. With take_all, every candidate is collected. Returns |T| (in tidx/ts).
template <int D, bool BF16>
__device__ int exact_select(FinishSmem* sm, const FinishArgs& a, const unsigned char* kb, bool take_all) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0;
  int64_t need = a.topk;  // how many of the keys equal to the final value must be taken
  if (!take_all) {
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      for (int i = tid; i < 256; i += FIN_THREADS) sm->hist[i] = 0;
      __syncthreads();
      for (int64_t j = 1 + tid; j <= a.scan_hi; j += FIN_THREADS) {
        if (!is_candidate(a, j)) continue;
        const uint64_t key =
            ord_f64((a.flags & FLAG_GROUP_SELECT) ? group_score_row<D, BF16>(sm, kb, j, a.G) : score_row<D, BF16>(sm, kb, j));
        if (pass == 0 || (key >> (shift + 8)) == prefix) atomicAdd(&sm->hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      find_bin_from_top(sm, 256, need);
      const int digit = sm->ival[0];
      const int above = sm->ival[1];
      __syncthreads();
      prefix = (prefix << 8) | (uint64_t)(digit < 0 ? 0 : digit);
      need -= above;
    }
  }
  // prefix = order key of the k-th best score: take every key above it and the `need` lowest
  // positions among the keys equal to it.
  if (tid == 0) {
    sm->ival[2] = 0;
    sm->ival[3] = 0;  // equal keys met so far
  }
  __syncthreads();
  for (int64_t j0 = 1; j0 <= a.scan_hi; j0 += FIN_THREADS) {
    const int64_t j = j0 + tid;
    const bool is_c = j <= a.scan_hi && is_candidate(a, j);
    double s = 0.0;
    bool gt = false, eq = false;
    if (is_c) {
      s = (a.flags & FLAG_GROUP_SELECT) ? group_score_row<D, BF16>(sm, kb, j, a.G) : score_row<D, BF16>(sm, kb, j);
      if (take_all) {
        gt = true;
      } else {
        const uint64_t key = ord_f64(s);
        gt = key > prefix;
        eq = key == prefix;
      }
    }
    const uint64_t em = __ballot(eq);
    const int w = tid >> 6;
    __syncthreads();
    if ((tid & 63) == 0) sm->hist[w] = __popcll(em);
    __syncthreads();
    int before = sm->ival[3];
    for (int i = 0; i < w; ++i) before += sm->hist[i];
    const int eq_rank = before + lanes_below(em);
    if (gt || (eq && eq_rank < need)) {
      const int slot = atomicAdd(&sm->ival[2], 1);
      if (slot < MAX_SET) {
        sm->u.c.tidx[slot] = (int32_t)j;
        sm->u.c.ts[slot] = s;
      }
    }
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int i = 0; i < FIN_WAVES; ++i) tot += sm->hist[i];
      sm->ival[3] += tot;
    }
    __syncthreads();
  }
  const int nt = sm->ival[2];
  __syncthreads();
  return nt < MAX_SET ? nt : MAX_SET;
}

// Copies into LDS every survivor whose upper bound reaches `theta` (a proven bound of the head's
// k-th best score: no other entry can be selected), with its bounds as order keys. List l is
// read by `tpl` threads; each issues all of its loads of a batch before using any, and the
// count of the list is only applied afterwards, so a batch costs one memory round trip. Kept
// entries are appended in any order (one LDS atomic per wave and batch). Returns the number of
// entries, or -1 if they do not fit.
// Also requests the shared state of the head (its threshold and overflow flag, returned in
// theta_out / over_out) and the caller's query element qraw (element min(tid, qn - 1) of qrow, qb
// bytes each, raw bits) after the first batch of list loads, so that the lists, the state and the
// query share one memory round trip. sm->ival[6] must be 0 on entry.
__device__ int stage_survivors(FinishSmem* sm, const FinishArgs& a, int bh, uint32_t& theta_out, uint32_t& over_out,
                               const unsigned char* qrow, int qb, int qn, uint32_t& qraw) {
  constexpr int BATCH = 12;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t nblk = a.nblk;
  const int slot = (int)a.slot;
  const uint32_t* bc = a.blk_cnt + (size_t)bh * nblk;
  const uint2* sv = a.surv + (size_t)bh * nblk * slot;
  const float* se = a.surv_eps + (size_t)bh * nblk * slot;
  int tpl = 1;
  while (tpl < 64 && (int64_t)tpl * 2 * nblk <= FIN_THREADS) tpl *= 2;
  const int lpp = FIN_THREADS / tpl;  // lists per pass
  const int sub = tid % tpl;
  uint32_t theta = 0u, over = 0u;
  // the shared state and the query element, after the first batch (see above)
  auto request_rest = [&]() {
    theta = a.st[bh].theta;
    over = a.st[bh].overflow;
    const int qi = tid < qn ? tid : qn - 1;
    qraw = qb == 2 ? (uint32_t)((const uint16_t*)qrow)[qi] : ((const uint32_t*)qrow)[qi];
  };
  // loads of batch (l0, jb): count and BATCH entries (with their error bounds) of list
  // l0 + tid / tpl. The addresses are clamped into the arrays and every load is issued (no
  // branches, so no load waits for another); entries past the list's count, or of a list past
  // the last, are ignored.
  auto load_batch = [&](int64_t l0, int jb, uint2 (&e)[BATCH], float (&ee)[BATCH], uint32_t& c) {
    const int64_t l = l0 + tid / tpl;
    const int64_t lc = l < nblk ? l : nblk - 1;
    c = bc[lc];
    if (l >= nblk) c = 0u;
    const int j0 = jb + sub;
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int j = j0 + u * tpl;
      const size_t at = (size_t)lc * slot + (j < slot ? j : slot - 1);
      e[u] = sv[at];
      ee[u] = se[at];
    }
  };
  // keep the entries whose upper bound reaches theta: append them to the LDS arrays
  auto filter_batch = [&](int jb, const uint2 (&e)[BATCH], const float (&ee)[BATCH], uint32_t c) {
    if (c > (uint32_t)slot) c = 0u;  // overflowed list: the head is on the exact path anyway
    const int j0 = jb + sub;
    uint32_t keep = 0u;
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int j = j0 + u * tpl;
      const bool k = j < (int)c && ord_f32(__uint_as_float(e[u].x) + ee[u]) >= theta;
      keep |= (k ? 1u : 0u) << u;
    }
    const int n = __popc(keep);
    const int incl = wave_incl_scan_i32(n);
    int base = 0;
    if (lane == 63 && incl > 0) base = atomicAdd(&sm->ival[6], incl);
    base = __shfl(base, 63) + incl - n;
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if ((keep >> u) & 1u) {
        if (base < SURV_LDS) {
          const float sf = __uint_as_float(e[u].x);
          sm->u.s.lbk[base] = ord_f32(sf - ee[u]);
          sm->u.s.ubk[base] = ord_f32(sf + ee[u]);
          sm->u.s.sidx[base] = (int32_t)e[u].y;
        }
        ++base;
      }
    }
  };
  uint2 e[BATCH];
  float ee[BATCH];
  uint32_t c;
  if (nblk <= lpp && slot <= tpl * BATCH) {
    // the usual case: every list in one batch
    load_batch(0, 0, e, ee, c);
    request_rest();
    __syncthreads();  // the cleared counter
    filter_batch(0, e, ee, c);
  } else {
    request_rest();
    __syncthreads();
    for (int64_t l0 = 0; l0 < nblk; l0 += lpp) {
      for (int jb = 0; jb < slot; jb += tpl * BATCH) {  // same trip count in every lane
        load_batch(l0, jb, e, ee, c);
        filter_batch(jb, e, ee, c);
      }
    }
  }
  __syncthreads();
  theta_out = theta;
  over_out = over;
  const int M = sm->ival[6];
  return M > SURV_LDS ? -1 : M;
}

template <int D, bool BF16>
__global__ __launch_bounds__(FIN_THREADS) void decode_finish_kernel(FinishArgs args) {
  constexpr int RB = D * (BF16 ? 2 : 4);
  extern __shared__ __align__(16) unsigned char smem_raw[];
  FinishSmem* sm = (FinishSmem*)smem_raw;
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  FinishArgs a = args;
  const int b = bh / a.Hq, h = bh - b * a.Hq, g = h / a.G;
  if (a.pos) {
    const QueryGeom gq = ragged_geom(a.pos, b, a.n, a.W);
    a.p = gq.p;
    a.w_lo = gq.w_lo;
    a.vis_hi = gq.vis_hi;
    a.scan_hi = gq.scan_hi;
    a.n_cand = gq.n_cand;
  }
  const unsigned char* kb = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.n * RB;
  const unsigned char* vb = a.v + ((size_t)b * a.Hkv + g) * (size_t)a.n * RB;
  const unsigned char* qrow = a.q + (size_t)bh * RB;

  // The thread's query element (raw bits) is requested with the staging's loads when the staging
  // runs, else just before it is needed; it reaches LDS after the selection.
  uint32_t qraw = 0u;
  bool q_requested = false;
  if (tid == 0) sm->ival[6] = 0;  // survivor counter of the staging
  // The window's share of the softmax comes from decode_window as a[bh].wparts records (partial
  // output, maximum logit m_j, sum Z_j); the first WPF are requested now (partial outputs by the
  // threads t < D, one element each; (m_j, Z_j) by threads D + j) and combined after the
  // selection. Addresses are clamped so that every load is issued without a branch.
  constexpr int WPF = 8;
  const bool use_win = a.out != nullptr && a.wparts > 0;
  const double* wr = a.wrec + (size_t)bh * a.wstride * (D + 2);
  double ow[WPF];
  double2 wmz_pf = make_double2(-INFINITY, 0.0);
  if (use_win) {
    const int tc = tid < D ? tid : D - 1;
#pragma unroll
    for (int j = 0; j < WPF; ++j) ow[j] = wr[(size_t)(j < a.wparts ? j : a.wparts - 1) * (D + 2) + tc];
    const int jm = tid - D < 0 ? 0 : (tid - D < a.wparts ? tid - D : a.wparts - 1);
    wmz_pf = *(const double2*)(wr + (size_t)jm * (D + 2) + D);
  }
  // Shared selection: the group's first head holds the survivor lists and the shared state of
  // the whole group, and every head of the group ranks by the same group scores.
  const bool group = (a.flags & FLAG_GROUP_SELECT) != 0;
  const int sh = group ? b * a.Hq + g * a.G : bh;  // head whose lists and state this block reads
  if (group) {
    for (int t = tid; t < a.G * D; t += FIN_THREADS)
      sm->qg[t / D][t % D] = load_elem_f64<BF16>(a.q + (size_t)(b * a.Hq + g * a.G + t / D) * RB, t % D);
  }
  // (every path below passes a barrier before qg is used)

  const int64_t w_lo = a.w_lo, p = a.p;
  const int anchor = w_lo > 0 ? 1 : 0;
  const int nwin = (int)(p - w_lo + 1);

  // ---- the top-k part T; the short list R (fast path) is scored together with the anchor, so
  // that all float64 row scores cost one memory round trip.
  int nt = 0;
  bool fast = false;
  int nr = 0;
  bool exact = false, take_all = false;
  int32_t path = PATH_NONE;
  if (a.topk > 0 && a.n_cand > 0) {
    exact = (a.flags & 1) != 0 || a.topk > KS_MAX_K;
    take_all = a.n_cand <= a.topk;
    path = take_all ? PATH_ALL : exact ? PATH_EXACT_ASKED : PATH_FAST;
    if (!take_all && !exact) {
      uint32_t st_theta = 0u, st_over = 0u;
      const int M = stage_survivors(sm, a, sh, st_theta, st_over, qrow, BF16 ? 2 : 4, D, qraw);
      q_requested = true;
      if (st_over != 0 || M < a.topk) {
        // a scan block overflowed its slot, more survivors than LDS holds, or (impossibly) fewer
        // than k: the exact path
        exact = true;
        path = st_over != 0 ? PATH_EXACT_OVERFLOW : PATH_EXACT_CROWDED;
      } else {
        // A valid threshold: at least k of the threads' best lower bounds (distinct keys) reach
        // it. Only values at or above the shared bound st_theta matter. For k <= 64 the search
        // runs between lo, the smallest of the 64 lanes' largest values (64 distinct keys reach
        // it), and hi, the largest value: the largest T = lo + c (hi - lo) / 1024 that k values
        // reach, counted per lane and summed with DPP moves, one bit of c per step. T lies less
        // than (hi - lo) / 1024 below the k-th largest value (a few more keys for the short
        // list). For larger k, or a range under 1024, the exact k-th largest by a bitwise search
        // that starts below the leading bits the range shares.
        uint32_t m0 = 0u;
        for (int f = tid; f < M; f += FIN_THREADS) m0 = max(m0, sm->u.s.lbk[f]);
        sm->hist[tid] = m0;
        __syncthreads();
        if (tid < 64) {
          uint32_t x[FIN_THREADS / 64];
          uint32_t hi = 0u;
          int above = 0;
#pragma unroll
          for (int i = 0; i < FIN_THREADS / 64; ++i) {
            x[i] = sm->hist[tid + 64 * i];
            hi = max(hi, x[i]);
            above += __popcll(__ballot(x[i] >= st_theta));
          }
          uint32_t lmax = x[0];
#pragma unroll
          for (int i = 1; i < FIN_THREADS / 64; ++i) lmax = max(lmax, x[i]);
          uint32_t lmin = lmax;
          for (int o = 32; o > 0; o >>= 1) {
            hi = max(hi, (uint32_t)__shfl_xor((int)hi, o));
            lmin = min(lmin, (uint32_t)__shfl_xor((int)lmin, o));
          }
          uint32_t T = 0u;
          if (above >= a.topk && hi > st_theta) {
            const uint32_t lo = a.topk <= 64 && lmin > st_theta ? lmin : st_theta;
            if (lo == hi) {
              T = hi;  // the 64 lane maxima all equal hi: at least 64 >= k values reach it
            } else if (a.topk <= 64 && hi - lo >= 1024u) {
              const uint32_t step = (hi - lo) >> 10;
              uint32_t c = 0u;
              for (int bit = 9; bit >= 0; --bit) {
                const uint32_t cc = c | (1u << bit);
                const uint32_t cand = lo + cc * step;
                int n = 0;
#pragma unroll
                for (int i = 0; i < FIN_THREADS / 64; ++i) n += x[i] >= cand ? 1 : 0;
                // sum over the 16 lanes of each row (quad permutes, row half mirror, row
                // mirror), then over the four rows
                n += __builtin_amdgcn_mov_dpp(n, 0xB1, 0xF, 0xF, false);
                n += __builtin_amdgcn_mov_dpp(n, 0x4E, 0xF, 0xF, false);
                n += __builtin_amdgcn_mov_dpp(n, 0x141, 0xF, 0xF, false);
                n += __builtin_amdgcn_mov_dpp(n, 0x140, 0xF, 0xF, false);
                const int tot = __builtin_amdgcn_readlane(n, 0) + __builtin_amdgcn_readlane(n, 16) +
                                __builtin_amdgcn_readlane(n, 32) + __builtin_amdgcn_readlane(n, 48);
                if (tot >= a.topk) c = cc;
              }
              T = lo + c * step;
            } else {
              const int top = 31 - __builtin_clz(lo ^ hi);  // highest bit where they differ
              T = top == 31 ? 0u : (hi & ~((2u << top) - 1u));
              for (int bit = top; bit >= 0; --bit) {
                const uint32_t cand = T | (1u << bit);
                int c = 0;
#pragma unroll
                for (int i = 0; i < FIN_THREADS / 64; ++i) c += __popcll(__ballot(x[i] >= cand));
                if (c >= a.topk) T = cand;
              }
            }
          }
          if (tid == 0) sm->ival[5] = (int)T;
        }
        if (tid == 0) sm->ival[4] = 0;
        __syncthreads();
        const uint32_t T = (uint32_t)sm->ival[5];
        const uint32_t theta = T > st_theta ? T : st_theta;
        for (int f = tid; f < M; f += FIN_THREADS) {
          if (sm->u.s.ubk[f] >= theta) {
            const int slot = atomicAdd(&sm->ival[4], 1);
            if (slot < REFINE_CAP) sm->ridx[slot] = sm->u.s.sidx[f];
          }
        }
        __syncthreads();
        nr = sm->ival[4];
        if (nr > REFINE_CAP || nr < a.topk) {
          exact = true;
          path = PATH_EXACT_CROWDED;
        } else {
          fast = true;
        }
      }
      __syncthreads();
    }
  }
  if (tid == 0) a.st[bh].path = path;
  if (!q_requested && tid < D) qraw = BF16 ? (uint32_t)((const uint16_t*)qrow)[tid] : ((const uint32_t*)qrow)[tid];
  asm volatile("" : "+v"(qraw));  // the conversion stays here, after the staging
  if (tid < D) sm->qd[tid] = (double)__uint_as_float(BF16 ? qraw << 16 : qraw);
  if (use_win && tid >= D && tid - D < WPF && tid - D < a.wparts) sm->wmz[tid - D] = wmz_pf;
  __syncthreads();

  // Row scores: the short list (fast path) and the anchor in the canonical float64 order, one row
  // per thread (the window rows are decode_window's).
  {
    const int nc = (fast ? nr : 0) + anchor;
    for (int i = tid; i < nc; i += FIN_THREADS) {
      const int64_t j = (fast && i < nr) ? (int64_t)sm->ridx[i] : 0;
      const double sc = score_row<D, BF16>(sm, kb, j);
      if (fast && i < nr) {
        sm->rs[i] = sc;
        if (group) sm->rg[i] = group_score_row<D, BF16>(sm, kb, j, a.G);
      } else {
        sm->ascore = sc;
      }
    }
  }
  __syncthreads();
  if (fast) {
    // exact rank of each short-list entry (higher score first, then lower position; group scores
    // for a shared selection): the comparisons of entry i are split into `parts` slices over all
    // threads, summed in LDS
    // (the order keys are computed once; each slice reads them four at a time, so that four LDS
    // round trips overlap)
    const double* rk_s = group ? sm->rg : sm->rs;
    int* rank = (int*)sm->hist;
    for (int i = tid; i < nr; i += FIN_THREADS) {
      rank[i] = 0;
      sm->rkey[i] = ord_f64(rk_s[i]);
    }
    __syncthreads();
    const int parts = nr < FIN_THREADS ? FIN_THREADS / nr : 1;
    const int chunk = (nr + parts - 1) / parts;
    for (int idx = tid; idx < nr * parts; idx += FIN_THREADS) {
      const int i = idx % nr, part = idx / nr;
      const uint64_t ki = sm->rkey[i];
      const int32_t ji = sm->ridx[i];
      const int r1 = min(nr, (part + 1) * chunk);
      int cnt = 0;
      int r = part * chunk;
      for (; r + 4 <= r1; r += 4) {
        uint64_t kr[4];
        int32_t jr[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          kr[u] = sm->rkey[r + u];
          jr[u] = sm->ridx[r + u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) cnt += (kr[u] > ki) || (kr[u] == ki && jr[u] < ji);
      }
      for (; r < r1; ++r) {
        const uint64_t kr = sm->rkey[r];
        cnt += (kr > ki) || (kr == ki && sm->ridx[r] < ji);
      }
      if (cnt) atomicAdd(&rank[i], cnt);
    }
    __syncthreads();
    for (int i = tid; i < nr; i += FIN_THREADS) {
      const int rk = rank[i];
      if (rk < a.topk) {
        sm->u.c.tidx[rk] = sm->ridx[i];
        sm->u.c.ts[rk] = sm->rs[i];
      }
    }
    nt = a.topk;
  } else if (a.topk > 0 && a.n_cand > 0) {
    nt = exact_select<D, BF16>(sm, a, kb, take_all);
    if (group) {
      // the selection ranked group scores; the softmax takes this head's own scores
      for (int t = tid; t < nt; t += FIN_THREADS) sm->u.c.ts[t] = score_row<D, BF16>(sm, kb, sm->u.c.tidx[t]);
      __syncthreads();
    }
  }
  __syncthreads();

  // The first batch of V row chunks (see the weighted sum below) is requested now, so that its
  // memory latency overlaps the set assembly and the softmax; entry nt is the anchor, row 0.
  constexpr int CPR = RB / 16;             // chunks per row
  constexpr int EPC = BF16 ? 8 : 4;        // elements per chunk
  constexpr int RPP = FIN_THREADS / CPR;   // rows per pass
  constexpr int BATCH = 8;
  const int ne = nt + anchor;
  // (all the batch's indices are read first, clamped to the last entry, and the loads run under
  // a bound that is the same in every thread: no load waits behind a per-thread branch; the
  // clamped slots get weight zero below)
  const int vc = tid % CPR, vr0 = tid / CPR;
  const int nbu = a.out ? min(BATCH, (ne + RPP - 1) / RPP) : 0;
  int32_t jv[BATCH];
#pragma unroll
  for (int u = 0; u < BATCH; ++u) {
    const int ic = min(vr0 + u * RPP, ne > 0 ? ne - 1 : 0);
    jv[u] = ic < nt ? sm->u.c.tidx[ic] : 0;
  }
  uint4 chv[BATCH];
#pragma unroll
  for (int u = 0; u < BATCH; ++u)
    chv[u] = u < nbu ? *(const uint4*)(vb + (size_t)jv[u] * RB + vc * 16) : make_uint4(0u, 0u, 0u, 0u);

  // ---- set assembly: C = {0} u window u T, ascending
  const int count = anchor + nwin + nt;
  if (nt <= 64) {
    // one wave sorts the top-k positions in registers (distinct keys; empty lanes sort last):
    // the t-th smallest goes to slot anchor + t, after the window if it lies past p; the window
    // follows the positions below it
    if (tid < 64) {
      uint32_t x = tid < nt ? (uint32_t)sm->u.c.tidx[tid] : 0xFFFFFFFFu;
      wave_sort64_asc_u32(x);
      const int tlo_w = __popcll(__ballot(tid < nt && (int64_t)x < w_lo));
      if (tid < nt) sm->u.c.cidx[anchor + tid + ((int64_t)x > p ? nwin : 0)] = (int32_t)x;
      if (tid == 0) {
        sm->ival[7] = tlo_w;
        if (anchor) sm->u.c.cidx[0] = 0;
      }
    }
    __syncthreads();
    const int tlo = sm->ival[7];
    for (int i = tid; i < nwin; i += FIN_THREADS) sm->u.c.cidx[anchor + tlo + i] = (int32_t)(w_lo + i);
    __syncthreads();
  } else {
  int tlo_local = 0;
  for (int i = tid; i < nt; i += FIN_THREADS) tlo_local += sm->u.c.tidx[i] < w_lo;
  tlo_local = wave_sum_i32(tlo_local);
  if ((tid & 63) == 0) sm->hist[tid >> 6] = tlo_local;
  __syncthreads();
  int tlo = 0;
  for (int i = 0; i < FIN_WAVES; ++i) tlo += sm->hist[i];
  if (anchor && tid == 0) sm->u.c.cidx[0] = 0;
  for (int i = tid; i < nt; i += FIN_THREADS) {
    const int32_t t = sm->u.c.tidx[i];
    int below = 0;
    for (int r = 0; r < nt; ++r) below += sm->u.c.tidx[r] < t;
    sm->u.c.cidx[anchor + below + (t > p ? nwin : 0)] = t;
  }
  for (int i = tid; i < nwin; i += FIN_THREADS) sm->u.c.cidx[anchor + tlo + i] = (int32_t)(w_lo + i);
  __syncthreads();
  }

  if (a.sel_idx) {
    int32_t* dst = a.sel_idx + (size_t)bh * a.set_cap;
    for (int i = tid; i < a.set_cap; i += FIN_THREADS) dst[i] = i < count ? sm->u.c.cidx[i] : -1;
  }
  if (a.sel_count && tid == 0) a.sel_count[bh] = count;
  if (!a.out) return;

  // ---- softmax over the set (float64) and the weighted sum of the V rows. Here the anchor and
  // the top-k part (ts / tidx [0, nt), the anchor appended at nt); the window's share is the
  // combination of decode_window's records: with M_w the largest of their m_j,
  // Z_w = sum_j Z_j exp(m_j - M_w) and O_w = sum_j O_j exp(m_j - M_w); then with zmax the largest
  // logit of the set, out = (sum_e w_e v_e + f O_w) / (sum_e w_e + f Z_w), w_e = exp(z_e - zmax),
  // f = exp(M_w - zmax).
  if (anchor && tid == 0) {
    sm->u.c.tidx[nt] = 0;
    sm->u.c.ts[nt] = sm->ascore;
  }
  double Mw = -INFINITY, Zw = 0.0, Ow = 0.0;
  if (use_win) {
#pragma unroll
    for (int j = 0; j < WPF; ++j)
      if (j < a.wparts) Mw = fmax(Mw, sm->wmz[j].x);
    for (int j = WPF; j < a.wparts; ++j) Mw = fmax(Mw, wr[(size_t)j * (D + 2) + D]);
    if (Mw > -INFINITY) {
      // one exponential per record: lane j of every wave takes record j < WPF, then shuffles
      const int lw = tid & 63;
      const double mj = sm->wmz[lw < WPF ? lw : 0].x;
      const double fl = lw < WPF && lw < a.wparts && mj > -INFINITY ? exp(mj - Mw) : 0.0;
#pragma unroll
      for (int j = 0; j < WPF; ++j) {
        const double f = __shfl(fl, j);
        if (j < a.wparts) {
          Zw += f * sm->wmz[j].y;
          Ow += f * ow[j];
        }
      }
      for (int j = WPF; j < a.wparts; ++j) {
        const double2 mz = *(const double2*)(wr + (size_t)j * (D + 2) + D);
        if (mz.x > -INFINITY) {
          const double f = exp(mz.x - Mw);
          Zw += f * mz.y;
          if (tid < D) Ow += f * wr[(size_t)j * (D + 2) + tid];
        }
      }
    }
  }
  __syncthreads();
  double zmax, zsum;
  if (ne <= 128) {
    // one wave takes the largest logit, the weights and their sum (two entries per lane); the
    // other waves wait at a single barrier
    if (tid < 64) {
      const double z0 = tid < ne ? a.scale * sm->u.c.ts[tid] : -INFINITY;
      const double z1 = tid + 64 < ne ? a.scale * sm->u.c.ts[tid + 64] : -INFINITY;
      const double m = wave_max_f64(fmax(Mw, fmax(z0, z1)));
      double ws = 0.0;
      if (tid < ne) {
        const double w = exp(z0 - m);
        sm->u.c.cw[tid] = w;
        ws += w;
      }
      if (tid + 64 < ne) {
        const double w = exp(z1 - m);
        sm->u.c.cw[tid + 64] = w;
        ws += w;
      }
      ws = wave_sum_f64(ws);
      if (tid == 0) {
        sm->scratch[0] = m;
        sm->scratch[1] = ws;
      }
    }
    __syncthreads();  // (the weights are visible after it)
    zmax = sm->scratch[0];
    zsum = sm->scratch[1];
  } else {
    zmax = Mw;
    for (int i = tid; i < ne; i += FIN_THREADS) zmax = fmax(zmax, a.scale * sm->u.c.ts[i]);
    zmax = block_max_f64<FIN_WAVES>(zmax, sm->scratch);
    zsum = 0.0;
    for (int i = tid; i < ne; i += FIN_THREADS) {
      const double w = exp(a.scale * sm->u.c.ts[i] - zmax);
      sm->u.c.cw[i] = w;
      zsum += w;
    }
    zsum = block_sum_f64<FIN_WAVES>(zsum, sm->scratch);  // (contains a barrier: weights visible)
  }
  const double fw = Mw > -INFINITY ? exp(Mw - zmax) : 0.0;
  zsum += fw * Zw;
  if (a.rho) {
    // Exactness certificate: every candidate left out scores at most s_k, the lowest score of
    // the top-k part, so the left-out mass relative to the dense total is at most
    // n_omit * exp(scale * s_k - zmax) / zsum (rounded up to float32).
    double smin = INFINITY;
    for (int i = tid; i < nt; i += FIN_THREADS) smin = fmin(smin, sm->u.c.ts[i]);
    smin = -block_max_f64<FIN_WAVES>(-smin, sm->scratch);
    if (tid == 0) {
      const int64_t n_omit = a.n_cand - nt;
      double r = 0.0;
      if (n_omit > 0) r = nt == 0 ? INFINITY : (double)n_omit * exp(a.scale * smin - zmax) / zsum;
      float rf = (float)r;
      if ((double)rf < r) rf = nextafterf(rf, INFINITY);
      a.rho[bh] = rf;
    }
  }

  // Thread t reads 16-byte chunk (t % CPR) of entries t / CPR, + RPP, ...; a batch of BATCH rows
  // per thread is in flight together (one batch covers up to RPP * BATCH entries; the first was
  // requested before the set assembly).
  const int wave = tid >> 6, lane = tid & 63;
  const int c = vc, r0 = vr0;
  double acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
  for (int i0 = r0; i0 < ne; i0 += RPP * BATCH) {
    uint4 ch[BATCH];
    if (i0 == r0) {
#pragma unroll
      for (int u = 0; u < BATCH; ++u) ch[u] = chv[u];
    } else {
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int i = i0 + u * RPP;
        ch[u] = i < ne ? *(const uint4*)(vb + (size_t)sm->u.c.tidx[i] * RB + c * 16) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int i = i0 + u * RPP;
      const double w = i < ne ? sm->u.c.cw[i] : 0.0;
      const uint32_t ws[4] = {ch[u].x, ch[u].y, ch[u].z, ch[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (BF16) {
          acc[2 * e] = fma(w, (double)bf16_lo(ws[e]), acc[2 * e]);
          acc[2 * e + 1] = fma(w, (double)bf16_hi(ws[e]), acc[2 * e + 1]);
        } else {
          acc[e] = fma(w, (double)__uint_as_float(ws[e]), acc[e]);
        }
      }
    }
  }
  // lanes of a wave that share a chunk: lane % CPR
#pragma unroll
  for (int e = 0; e < EPC; ++e)
    for (int o = CPR; o < 64; o <<= 1) acc[e] += __shfl_xor(acc[e], o);
  if (lane < CPR) {
#pragma unroll
    for (int e = 0; e < EPC; ++e) sm->red[wave * D + lane * EPC + e] = acc[e];
  }
  __syncthreads();
  if (tid < D) {
    double num = fw * Ow;
    for (int w = 0; w < FIN_WAVES; ++w) num += sm->red[w * D + tid];
    a.out[(size_t)bh * D + tid] = (float)(num / zsum);
  }
}

// ---------------------------------------------------------------------------------------------
template <int RB, int GT, bool BF16>
static hipError_t launch_kscan_t(const KscanArgs& ka, dim3 grid, hipStream_t s) {
  if (ka.group) {
    if (ka.pos)
      hipLaunchKernelGGL((kscan_kernel<RB, GT, BF16, true, true>), grid, dim3(256), 0, s, ka);
    else
      hipLaunchKernelGGL((kscan_kernel<RB, GT, BF16, false, true>), grid, dim3(256), 0, s, ka);
  } else {
    if (ka.pos)
      hipLaunchKernelGGL((kscan_kernel<RB, GT, BF16, true, false>), grid, dim3(256), 0, s, ka);
    else
      hipLaunchKernelGGL((kscan_kernel<RB, GT, BF16, false, false>), grid, dim3(256), 0, s, ka);
  }
  return hipGetLastError();
}

template <int RB, bool BF16>
static hipError_t launch_kscan_g(const KscanArgs& ka, int GT, dim3 grid, hipStream_t s) {
  switch (GT) {
    case 1: return launch_kscan_t<RB, 1, BF16>(ka, grid, s);
    case 2: return launch_kscan_t<RB, 2, BF16>(ka, grid, s);
    default: return launch_kscan_t<RB, 4, BF16>(ka, grid, s);
  }
}

template <int D, bool BF16>
static hipError_t launch_finish_t(const FinishArgs& fa, int nbh, hipStream_t s) {
  const size_t smem = sizeof(FinishSmem);
  static bool attr_set = false;  // idempotent; setting it twice is harmless
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)decode_finish_kernel<D, BF16>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    attr_set = true;
  }
  hipLaunchKernelGGL((decode_finish_kernel<D, BF16>), dim3(nbh), dim3(FIN_THREADS), smem, s, fa);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream) {
  const int nbh = L.B * L.Hq;
  const QueryGeom& g = L.geom;
  // the window's share of the softmax (with the clearing of the scan state), or the clearing alone
  const int64_t wparts = L.out ? window_parts(g, L.d, L.bf16) : 0;
  if (wparts > 0) {
    WindowArgs wa;
    wa.q = (const unsigned char*)L.q;
    wa.k = (const unsigned char*)L.k;
    wa.v = (const unsigned char*)L.v;
    wa.st = L.st;
    wa.rec = L.wrec;
    wa.pos = L.pos;
    wa.n = L.n;
    wa.p = g.p;
    wa.w_lo = g.w_lo;
    wa.rstride = L.wstride;
    wa.Hq = L.Hq;
    wa.Hkv = L.Hkv;
    wa.G = L.G;
    wa.W = L.W;
    wa.nheads = nbh;
    wa.rstride_parts = (int32_t)wparts;
    wa.scale = L.scale;
    const dim3 grid((unsigned)(wparts * nbh));
    if (L.bf16) {
      if (L.d == 128) hipLaunchKernelGGL((decode_window_kernel<128, true>), grid, dim3(256), 0, stream, wa);
      else hipLaunchKernelGGL((decode_window_kernel<64, true>), grid, dim3(256), 0, stream, wa);
    } else {
      if (L.d == 128) hipLaunchKernelGGL((decode_window_kernel<128, false>), grid, dim3(256), 0, stream, wa);
      else hipLaunchKernelGGL((decode_window_kernel<64, false>), grid, dim3(256), 0, stream, wa);
    }
  } else {
    hipLaunchKernelGGL(decode_init_kernel, dim3((nbh + 255) / 256), dim3(256), 0, stream, L.st, nbh);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  if (L.ev_scan_begin) {
    e = hipEventRecord(L.ev_scan_begin, stream);
    if (e != hipSuccess) return e;
  }
  const bool need_scan = L.topk > 0 && L.topk <= KS_MAX_K && g.n_cand > L.topk && !(L.flags & 1);
  if (need_scan) {
    KscanArgs ka;
    ka.k = (const unsigned char*)L.k;
    ka.q = (const unsigned char*)L.q;
    ka.st = L.st;
    ka.blk_cnt = L.blk_cnt[0];
    ka.surv = L.surv[0];
    ka.surv_eps = L.surv_eps[0];
    ka.n = L.n;
    ka.nblk = L.nblk[0];
    ka.slot = L.slot;
    ka.p = g.p;
    ka.w_lo = g.w_lo;
    ka.vis_hi = g.vis_hi;
    ka.scan_hi = g.scan_hi;
    ka.pos = L.pos;
    ka.W = L.W;
    ka.group = (L.flags & FLAG_GROUP_SELECT) ? 1 : 0;
    ka.Hq = L.Hq;
    ka.Hkv = L.Hkv;
    ka.G = L.G;
    ka.topk = L.topk;
    ka.runs = L.runs;
    ka.eps_coef = L.eps_coef;
    const int GT = L.G >= 4 ? 4 : L.G;
    dim3 grid((unsigned)L.nblk[0], (unsigned)(L.B * L.Hkv),
              (unsigned)((L.G + GT - 1) / GT));
    const int RB = L.d * (L.bf16 ? 2 : 4);
    if (L.bf16) {
      e = RB == 256 ? launch_kscan_g<256, true>(ka, GT, grid, stream) : launch_kscan_g<128, true>(ka, GT, grid, stream);
    } else {
      e = RB == 256 ? launch_kscan_g<256, false>(ka, GT, grid, stream) : launch_kscan_g<512, false>(ka, GT, grid, stream);
    }
    if (e != hipSuccess) return e;
    if (L.ev_scan_end) {
      e = hipEventRecord(L.ev_scan_end, stream);
      if (e != hipSuccess) return e;
    }
    for (int l = 0; l + 1 < L.nlevels; ++l) {
      MergeArgs ma;
      ma.st = L.st;
      ma.st_w = L.st;
      ma.cnt_in = L.blk_cnt[l];
      ma.surv_in = L.surv[l];
      ma.eps_in = L.surv_eps[l];
      ma.cnt_out = L.blk_cnt[l + 1];
      ma.surv_out = L.surv[l + 1];
      ma.eps_out = L.surv_eps[l + 1];
      ma.nblk_in = L.nblk[l];
      ma.nblk_out = L.nblk[l + 1];
      ma.slot = L.slot;
      ma.topk = L.topk;
      hipLaunchKernelGGL(merge_lists_kernel, dim3((unsigned)L.nblk[l + 1], (unsigned)nbh), dim3(64), 0, stream, ma);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }

  if (!need_scan && L.ev_scan_end) {
    e = hipEventRecord(L.ev_scan_end, stream);
    if (e != hipSuccess) return e;
  }
  const int last = L.nlevels - 1;
  FinishArgs fa;
  fa.q = (const unsigned char*)L.q;
  fa.k = (const unsigned char*)L.k;
  fa.v = (const unsigned char*)L.v;
  fa.out = L.out;
  fa.sel_idx = L.sel_idx;
  fa.sel_count = L.sel_count;
  fa.rho = L.rho;
  fa.st = L.st;
  fa.blk_cnt = L.blk_cnt[last];
  fa.surv = L.surv[last];
  fa.surv_eps = L.surv_eps[last];
  fa.n = L.n;
  fa.nblk = L.nblk[last];
  fa.slot = L.slot;
  fa.p = g.p;
  fa.w_lo = g.w_lo;
  fa.vis_hi = g.vis_hi;
  fa.scan_hi = g.scan_hi;
  fa.n_cand = g.n_cand;
  fa.pos = L.pos;
  fa.wrec = L.wrec;
  fa.wstride = L.wstride;
  fa.wparts = (int32_t)wparts;
  fa.Hq = L.Hq;
  fa.Hkv = L.Hkv;
  fa.G = L.G;
  fa.W = L.W;
  fa.topk = L.topk;
  fa.set_cap = 1 + L.W + L.topk;
  fa.flags = L.flags;
  fa.scale = L.scale;
  fa.eps_coef = L.eps_coef;
  if (L.bf16) {
    return L.d == 128 ? launch_finish_t<128, true>(fa, nbh, stream) : launch_finish_t<64, true>(fa, nbh, stream);
  }
  return L.d == 128 ? launch_finish_t<128, false>(fa, nbh, stream) : launch_finish_t<64, false>(fa, nbh, stream);
}

// ---------------------------------------------------------------------------------------------
// KV append: block (b, g) copies the new key and value rows of batch element b, kv head g
// (row_bytes each, in 16-byte chunks) to row pos[b] of the caches; a position outside
// [0, n - 1] writes nothing.
__global__ __launch_bounds__(64) void kv_append_kernel(const uint4* k_new, const uint4* v_new, unsigned char* k_cache,
                                                       unsigned char* v_cache, const int64_t* pos, int32_t Hkv,
                                                       int64_t n, int32_t row_bytes) {
  const int grp = blockIdx.x, b = grp / Hkv;
  const int64_t p = pos[b];
  if (p < 0 || p >= n) return;
  const int nch = row_bytes / 16;
  const size_t dst = ((size_t)grp * (size_t)n + (size_t)p) * (size_t)row_bytes;
  for (int c = threadIdx.x; c < nch; c += 64) {
    *(uint4*)(k_cache + dst + (size_t)c * 16) = k_new[(size_t)grp * nch + c];
    *(uint4*)(v_cache + dst + (size_t)c * 16) = v_new[(size_t)grp * nch + c];
  }
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache, const int64_t* pos,
                            int32_t B, int32_t Hkv, int64_t n, int32_t row_bytes, hipStream_t stream) {
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)(B * Hkv)), dim3(64), 0, stream, (const uint4*)k_new,
                     (const uint4*)v_new, (unsigned char*)k_cache, (unsigned char*)v_cache, pos, Hkv, n, row_bytes);
  return hipGetLastError();
}

}  // namespace topo
