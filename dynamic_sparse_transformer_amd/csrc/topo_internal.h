// Internal interfaces between the C-ABI front end (topo_api.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace topo {

// Decode key scan geometry: a tile is 64 keys (one owned by each lane after the cross-lane
// reduction), a wave ranks KS_IT tiles per run, a block of KS_WAVES waves ranks `runs` runs of
// KS_KEYS_PER_RUN keys (chosen per call so that the grid still fills the chip) and merges the
// survivors of its waves.
constexpr int KS_ROWS = 64;
constexpr int KS_IT = 8;
constexpr int KS_WAVES = 4;
constexpr int KS_KEYS_PER_WAVE = KS_ROWS * KS_IT;
constexpr int KS_KEYS_PER_RUN = KS_KEYS_PER_WAVE * KS_WAVES;  // a block ranks 1..KS_MAX_RUNS runs
constexpr int KS_MAX_RUNS = 16;
constexpr int KS_MAX_K = 224;     // largest k the scan ranks (larger k: exact selection only)
constexpr int KS_WAVE_CAP = 256;  // survivors one wave may hand to its block merge
constexpr int MAX_SET = 4096;     // largest 1 + W + k
constexpr int REFINE_CAP = 1024;  // largest short list re-scored in float64 by the fast path
constexpr uint32_t KS_OVERFLOW = 0xFFFFFFFFu;
constexpr int MERGE_FAN = 8;      // survivor lists merged into one per merge step
constexpr int MAX_LEVELS = 8;
constexpr int SURV_LDS = 8192;    // survivors the finishing kernel stages in LDS

// Flag bits of the call (the values of TOPO_FLAG_EXACT_SELECT and TOPO_FLAG_GROUP_SELECT).
constexpr int32_t FLAG_EXACT_SELECT = 1;
constexpr int32_t FLAG_GROUP_SELECT = 4;

// Per (batch, query head) state shared by the key scan blocks, one 128-byte line per head.
struct alignas(128) HeadState {
  uint32_t theta;     // order key of a proven lower bound of the k-th best candidate score
  uint32_t overflow;  // 1 if some block had more survivors than its slot holds
  int32_t path;       // how the finish chose the top-k part (PATH_* below)
  uint32_t pad[29];
};

// Selection path of a query, left in the workspace for diagnostics (the values of TOPO_PATH_*).
constexpr int32_t PATH_NONE = 0;            // no top-k part: k = 0 or no candidate
constexpr int32_t PATH_ALL = 1;             // at most k candidates: all taken
constexpr int32_t PATH_FAST = 2;            // from the scan's lists (decode: short list re-scored in float64;
                                            // prefill: the fast scores' bounds decided every member)
constexpr int32_t PATH_BAND = 3;            // prefill: as PATH_FAST, the entries inside the band re-scored in float64
constexpr int32_t PATH_EXACT_ASKED = 4;     // exact radix selection: flag, float32 prefill inputs, or a size
                                            // above the scan's limits
constexpr int32_t PATH_EXACT_OVERFLOW = 5;  // exact radix selection: a scan list overflowed (ties)
constexpr int32_t PATH_EXACT_CROWDED = 6;   // exact radix selection: the short list was crowded (ties)

// Where one query sits and which keys are its candidates.
struct QueryGeom {
  int64_t p;        // query position
  int64_t w_lo;     // first window position: max(0, p - W + 1)
  int64_t vis_hi;   // last visible key: p (causal) or n - 1
  int64_t scan_hi;  // last key the scan must look at (candidates lie in [1, scan_hi])
  int64_t n_cand;   // number of candidates
};

__host__ __device__ inline QueryGeom make_geom(int64_t p, int64_t n, int32_t W, bool causal) {
  QueryGeom g;
  g.p = p;
  g.w_lo = p - (int64_t)W + 1 > 0 ? p - (int64_t)W + 1 : 0;
  g.vis_hi = causal ? p : n - 1;
  int64_t wlo1 = g.w_lo > 1 ? g.w_lo : 1;
  int64_t win_nonzero = p >= wlo1 ? p - wlo1 + 1 : 0;
  g.n_cand = g.vis_hi - win_nonzero;
  g.scan_hi = g.vis_hi > p ? g.vis_hi : g.w_lo - 1;
  if (g.scan_hi < 0) g.scan_hi = 0;
  return g;
}

struct DecodeLaunch {
  const void* q;
  const void* k;
  const void* v;
  float* out;          // may be null (select only)
  int32_t* sel_idx;    // may be null
  int32_t* sel_count;  // may be null
  float* rho;          // may be null: the exactness certificate per query
  HeadState* st;       // [B * Hq]
  double* wrec;        // [B * Hq][wstride][d + 2]: the window kernel's records
  int64_t wstride;
  // Survivor lists, level 0 written by the key scan and level l+1 by merging groups of
  // MERGE_FAN level-l lists:
  //   blk_cnt[l]  [B * Hq][nblk[l]]        survivors of each list (or KS_OVERFLOW)
  //   surv[l]     [B * Hq][nblk[l]][slot]  (float bits of the fast score, key index)
  //   surv_eps[l] [B * Hq][nblk[l]][slot]  error bound of that entry's fast score (its own key's)
  uint32_t* blk_cnt[MAX_LEVELS];
  uint2* surv[MAX_LEVELS];
  float* surv_eps[MAX_LEVELS];
  int64_t nblk[MAX_LEVELS];
  int nlevels;
  int64_t slot;
  int32_t runs;  // runs of KS_KEYS_PER_RUN keys per key-scan block
  int32_t B, Hq, Hkv, G, d, W, topk, bf16, flags;
  int64_t n;
  QueryGeom geom;     // the query's geometry; with pos, the geometry of position n - 1 (sizes)
  const int64_t* pos;  // may be null: per batch element b, the causal query position pos[b]
  double scale;
  float eps_coef;
  hipEvent_t ev_scan_begin;  // optional: recorded around the key-scan launch
  hipEvent_t ev_scan_end;
};

size_t decode_workspace_bytes(int32_t B, int32_t Hq, const QueryGeom& g, int32_t k, int32_t d, int32_t bf16);
// Byte offsets, within a decode workspace, of the HeadState array and of the key scan's own
// (level 0) survivor lists, with their shape, as decode_carve lays them out.
struct DecodeView {
  size_t state, count, entry, eps;
  int64_t lists, slot;
};
DecodeView decode_view(int32_t B, int32_t Hq, int32_t Hkv, const QueryGeom& g, int32_t k, int32_t d, int32_t bf16);
// Carve the workspace into the HeadState array, the window records and the survivor lists
// (L.d and L.bf16 must be set).
void decode_carve(void* ws, int32_t B, int32_t Hq, const QueryGeom& g, int32_t k, DecodeLaunch& L);
hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream);
// New key and value rows of one token per (batch, kv head) into the caches at row pos[b].
hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache, const int64_t* pos,
                            int32_t B, int32_t Hkv, int64_t n, int32_t row_bytes, hipStream_t stream);

// Float32 error-bound coefficient of the fast scores: |s_fast - s| <= coef * |q|_2 * |k|_2.
float fast_score_eps_coef(int d);

// Dense attention (pillar layer).
struct DenseLaunch {
  const void* q;
  const void* k;
  const void* v;
  float* out;
  void* ws;
  int32_t B, Hq, Hkv, G, d, bf16, causal;
  int64_t n, n_q, q_pos0;
  double scale;
  const float* gate;  // may be null; else only rows with gate[row] >= gate_min are computed
  float gate_min;
};
size_t dense_workspace_bytes(int32_t B, int32_t Hq, int64_t n_q, int64_t n, int32_t d);
hipError_t launch_dense(const DenseLaunch& L, hipStream_t stream);

// Many-query (prefill) path.
struct PrefillLaunch {
  const void* q;
  const void* k;
  const void* v;
  float* out;
  int32_t* sel_idx;
  int32_t* sel_count;
  void* ws;
  int32_t B, Hq, Hkv, G, d, W, topk, bf16, causal, flags;
  int64_t n, n_q, q_pos0;
  double scale;
  float eps_coef;
  hipEvent_t ev_scan_begin;  // optional: recorded around the key-scan launch
  hipEvent_t ev_scan_end;
};
size_t prefill_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t n_q, int64_t n, int32_t d, int32_t W, int32_t k);
// Whether the per-row finish's LDS holds a set of 1 + W + k (false: the prefill is unsupported).
bool prefill_fits(int32_t W, int32_t k, bool bf16);
// Byte offsets, within a prefill workspace, of the scan's per-row lists and the rows' paths.
struct PrefillView {
  size_t count, entry, path;
  int64_t slot;
};
PrefillView prefill_view(int32_t B, int32_t Hq, int32_t Hkv, int64_t n_q, int64_t n, int32_t d, int32_t k);
// Error-bound coefficient of the matrix-core scores: |s_fast - s| <= coef * |q|_2 * |k|_2.
float prefill_eps_coef();
hipError_t launch_prefill(const PrefillLaunch& L, hipStream_t stream);

hipError_t launch_bw_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);
// Sets bit 0 of *flag if any of the count elements (float32, or bf16 when bf16) is NaN or infinite.
hipError_t launch_check_finite(const void* buf, size_t count, int bf16, uint32_t* flag, hipStream_t stream);

}  // namespace topo
