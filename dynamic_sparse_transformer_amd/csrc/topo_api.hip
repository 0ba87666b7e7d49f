// C-ABI front end of libtopo_attn.so: argument validation, workspace sizing and carving, and the
// launch sequence of each operation. The operation and its arithmetic are described in
// include/topo_attn.h (condensate set of "The Condensate Theorem: Transformers are O(n), Not
// O(n^2)", zh page, technical summary §3; softmax over the set, fr page, technical summary §3).
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "../../include/topo_attn.h"
#include "topo_internal.h"

static_assert(TOPO_FLAG_EXACT_SELECT == topo::FLAG_EXACT_SELECT && TOPO_FLAG_GROUP_SELECT == topo::FLAG_GROUP_SELECT,
              "flag values shared with the kernels");
static_assert(TOPO_PATH_NONE == topo::PATH_NONE && TOPO_PATH_ALL == topo::PATH_ALL && TOPO_PATH_FAST == topo::PATH_FAST &&
                  TOPO_PATH_BAND == topo::PATH_BAND && TOPO_PATH_EXACT_ASKED == topo::PATH_EXACT_ASKED &&
                  TOPO_PATH_EXACT_OVERFLOW == topo::PATH_EXACT_OVERFLOW &&
                  TOPO_PATH_EXACT_CROWDED == topo::PATH_EXACT_CROWDED,
              "path codes shared with the kernels");

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape, position and scalar checks shared by every operation. Returns TOPO_OK or an error.
int check_params(const topo_params_t* p, bool need_set) {
  if (!p) return TOPO_EINVAL;
  if (p->dtype != TOPO_F32 && p->dtype != TOPO_BF16) return TOPO_EUNSUPPORTED;
  if (p->d != 64 && p->d != 128) return TOPO_EUNSUPPORTED;
  if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->Hq % p->Hkv != 0) return TOPO_EINVAL;
  if (p->n_ctx < 1 || p->n_ctx > INT32_MAX) return TOPO_EINVAL;
  if (p->n_q < 1 || p->q_pos0 < 0 || p->q_pos0 + p->n_q - 1 > p->n_ctx - 1) return TOPO_EINVAL;
  if (!(p->softmax_scale > 0.f) || !std::isfinite(p->softmax_scale)) return TOPO_EINVAL;
  if (p->causal != 0 && p->causal != 1) return TOPO_EINVAL;
  if (p->flags & ~(TOPO_FLAG_EXACT_SELECT | TOPO_FLAG_DENSE_FALLBACK | TOPO_FLAG_GROUP_SELECT)) return TOPO_EINVAL;
  if (need_set) {
    if (p->W < 0 || p->k < 0) return TOPO_EINVAL;
    if ((int64_t)p->W + p->k + 1 > TOPO_MAX_SET) return TOPO_EINVAL;
  }
  // Element counts must fit the 64-bit byte offsets used by the kernels.
  const double elems = (double)p->B * p->Hkv * (double)p->n_ctx * p->d;
  if (elems * 4.0 > 9.0e18) return TOPO_EINVAL;
  return TOPO_OK;
}

topo::QueryGeom decode_geom(const topo_params_t* p) {
  return topo::make_geom(p->q_pos0, p->n_ctx, p->W, p->causal != 0);
}

// Sizes of a call with per-sequence positions: those of a query at the cache's last row, the
// longest scan any position can need.
topo::QueryGeom ragged_sizes_geom(const topo_params_t* p) { return topo::make_geom(p->n_ctx - 1, p->n_ctx, p->W, true); }

bool aligned8(const void* p) { return ((uintptr_t)p & 7u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the certified decode: the decode's, then (with the dense fallback) the dense
// attention's partials.
size_t certified_workspace_bytes(const topo_params_t* p) {
  size_t b = align256(topo::decode_workspace_bytes(p->B, p->Hq, decode_geom(p), p->k, p->d, p->dtype == TOPO_BF16));
  if (p->flags & TOPO_FLAG_DENSE_FALLBACK) b += topo::dense_workspace_bytes(p->B, p->Hq, 1, p->n_ctx, p->d);
  return b;
}

size_t prefill_ws(const topo_params_t* p) {
  if (!topo::prefill_fits(p->W, p->k, p->dtype == TOPO_BF16)) return 0;
  return topo::prefill_workspace_bytes(p->B, p->Hq, p->Hkv, p->n_q, p->n_ctx, p->d, p->W, p->k);
}

int decode_like(const topo_params_t* p, const void* q, const void* k, const void* v, float* out,
                int32_t* sel_idx, int32_t* sel_count, void* ws, size_t ws_bytes, hipStream_t stream,
                bool softmax, hipEvent_t ev_begin = nullptr, hipEvent_t ev_end = nullptr, float* rho = nullptr,
                const int64_t* pos = nullptr) {
  int rc = check_params(p, true);
  if (rc) return rc;
  if (p->n_q != 1) return TOPO_EINVAL;
  if (pos && (p->causal != 1 || rho || !aligned8(pos))) return TOPO_EINVAL;
  if (p->flags & TOPO_FLAG_GROUP_SELECT) {
    if (rho) return TOPO_EINVAL;                        // no certificate for a shared selection
    if (p->Hq / p->Hkv > 4) return TOPO_EUNSUPPORTED;   // one key-scan slice per group
  }
  if (!rho && (p->flags & TOPO_FLAG_DENSE_FALLBACK)) return TOPO_EINVAL;
  if (rho && !aligned16(rho)) return TOPO_EINVAL;
  if (!q || !k || !aligned16(q) || !aligned16(k)) return TOPO_EINVAL;
  if (softmax && (!v || !out || !aligned16(v) || !aligned16(out))) return TOPO_EINVAL;
  if (!softmax && (!sel_idx || !sel_count)) return TOPO_EINVAL;
  if ((sel_idx && !aligned16(sel_idx)) || (sel_count && !aligned16(sel_count))) return TOPO_EINVAL;
  const topo::QueryGeom g = pos ? ragged_sizes_geom(p) : decode_geom(p);
  const size_t need = rho ? certified_workspace_bytes(p) : topo::decode_workspace_bytes(p->B, p->Hq, g, p->k, p->d, p->dtype == TOPO_BF16);
  if (!ws || ws_bytes < need || !aligned16(ws)) return TOPO_EWORKSPACE;

  topo::DecodeLaunch L{};
  L.rho = rho;
  L.q = q;
  L.k = k;
  L.v = softmax ? v : nullptr;
  L.out = softmax ? out : nullptr;
  L.sel_idx = sel_idx;
  L.sel_count = sel_count;
  L.B = p->B;
  L.Hq = p->Hq;
  L.Hkv = p->Hkv;
  L.G = p->Hq / p->Hkv;
  L.d = p->d;
  L.W = p->W;
  L.topk = p->k;
  L.bf16 = p->dtype == TOPO_BF16;
  L.flags = p->flags;
  L.n = p->n_ctx;
  L.geom = g;
  L.pos = pos;
  L.scale = (double)p->softmax_scale;
  L.eps_coef = topo::fast_score_eps_coef(p->d);
  L.ev_scan_begin = ev_begin;
  L.ev_scan_end = ev_end;
  topo::decode_carve(ws, p->B, p->Hq, g, p->k, L);
  if (topo::launch_decode(L, stream) != hipSuccess) return TOPO_EHIP;
  if (rho && (p->flags & TOPO_FLAG_DENSE_FALLBACK)) {
    // dense attention for the queries the certificate does not cover (the others skip)
    topo::DenseLaunch D{};
    D.q = q;
    D.k = k;
    D.v = v;
    D.out = out;
    D.ws = (char*)ws + align256(topo::decode_workspace_bytes(p->B, p->Hq, g, p->k, p->d, p->dtype == TOPO_BF16));
    D.B = p->B;
    D.Hq = p->Hq;
    D.Hkv = p->Hkv;
    D.G = p->Hq / p->Hkv;
    D.d = p->d;
    D.bf16 = p->dtype == TOPO_BF16;
    D.causal = p->causal;
    D.n = p->n_ctx;
    D.n_q = 1;
    D.q_pos0 = p->q_pos0;
    D.scale = (double)p->softmax_scale;
    D.gate = rho;
    D.gate_min = TOPO_CERT_RHO;
    if (topo::launch_dense(D, stream) != hipSuccess) return TOPO_EHIP;
  }
  return TOPO_OK;
}

int prefill_like(const topo_params_t* p, const void* q, const void* k, const void* v, float* out,
                 int32_t* sel_idx, int32_t* sel_count, void* ws, size_t ws_bytes, hipStream_t stream,
                 bool softmax, hipEvent_t ev_begin = nullptr, hipEvent_t ev_end = nullptr) {
  int rc = check_params(p, true);
  if (rc) return rc;
  if (p->flags & (TOPO_FLAG_DENSE_FALLBACK | TOPO_FLAG_GROUP_SELECT)) return TOPO_EINVAL;
  if (!q || !k || !aligned16(q) || !aligned16(k)) return TOPO_EINVAL;
  if (softmax && (!v || !out || !aligned16(v) || !aligned16(out))) return TOPO_EINVAL;
  if (!softmax && (!sel_idx || !sel_count)) return TOPO_EINVAL;
  if ((sel_idx && !aligned16(sel_idx)) || (sel_count && !aligned16(sel_count))) return TOPO_EINVAL;
  if (!topo::prefill_fits(p->W, p->k, p->dtype == TOPO_BF16)) return TOPO_EUNSUPPORTED;
  const size_t need = prefill_ws(p);
  if (!ws || ws_bytes < need || !aligned16(ws)) return TOPO_EWORKSPACE;
  topo::PrefillLaunch L{};
  L.q = q;
  L.k = k;
  L.v = softmax ? v : nullptr;
  L.out = softmax ? out : nullptr;
  L.sel_idx = sel_idx;
  L.sel_count = sel_count;
  L.ws = ws;
  L.B = p->B;
  L.Hq = p->Hq;
  L.Hkv = p->Hkv;
  L.G = p->Hq / p->Hkv;
  L.d = p->d;
  L.W = p->W;
  L.topk = p->k;
  L.bf16 = p->dtype == TOPO_BF16;
  L.causal = p->causal;
  L.flags = p->flags;
  L.n = p->n_ctx;
  L.n_q = p->n_q;
  L.q_pos0 = p->q_pos0;
  L.scale = (double)p->softmax_scale;
  L.eps_coef = topo::fast_score_eps_coef(p->d);
  L.ev_scan_begin = ev_begin;
  L.ev_scan_end = ev_end;
  return topo::launch_prefill(L, stream) == hipSuccess ? TOPO_OK : TOPO_EHIP;
}

}  // namespace

extern "C" {

size_t topo_workspace_bytes(const topo_params_t* p, int op) {
  const bool set = op != TOPO_OP_DENSE;
  if (check_params(p, set) != TOPO_OK) return 0;
  switch (op) {
    case TOPO_OP_DECODE:
      if (p->n_q != 1) return 0;
      return topo::decode_workspace_bytes(p->B, p->Hq, decode_geom(p), p->k, p->d, p->dtype == TOPO_BF16);
    case TOPO_OP_PREFILL:
      return prefill_ws(p);
    case TOPO_OP_SELECT:
      if (p->n_q == 1) return topo::decode_workspace_bytes(p->B, p->Hq, decode_geom(p), p->k, p->d, p->dtype == TOPO_BF16);
      return prefill_ws(p);
    case TOPO_OP_DENSE:
      return topo::dense_workspace_bytes(p->B, p->Hq, p->n_q, p->n_ctx, p->d);
    case TOPO_OP_DECODE_CERTIFIED:
      if (p->n_q != 1) return 0;
      return certified_workspace_bytes(p);
    case TOPO_OP_DECODE_RAGGED:
      if (p->n_q != 1 || p->causal != 1) return 0;
      return topo::decode_workspace_bytes(p->B, p->Hq, ragged_sizes_geom(p), p->k, p->d, p->dtype == TOPO_BF16);
    default:
      return 0;
  }
}

int topo_attn_decode(const topo_params_t* p, const void* q, const void* k, const void* v, float* out,
                     int32_t* sel_idx, int32_t* sel_count, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return decode_like(p, q, k, v, out, sel_idx, sel_count, workspace, ws_bytes, stream, true);
}

int topo_attn_decode_timed(const topo_params_t* p, const void* q, const void* k, const void* v, float* out,
                           int32_t* sel_idx, int32_t* sel_count, void* workspace, size_t ws_bytes,
                           hipStream_t stream, hipEvent_t scan_begin, hipEvent_t scan_end) {
  if (!scan_begin || !scan_end) return TOPO_EINVAL;
  return decode_like(p, q, k, v, out, sel_idx, sel_count, workspace, ws_bytes, stream, true, scan_begin, scan_end);
}

int topo_attn_decode_certified(const topo_params_t* p, const void* q, const void* k, const void* v, float* out,
                               int32_t* sel_idx, int32_t* sel_count, float* rho, void* workspace, size_t ws_bytes,
                               hipStream_t stream) {
  if (!rho) return TOPO_EINVAL;
  return decode_like(p, q, k, v, out, sel_idx, sel_count, workspace, ws_bytes, stream, true, nullptr, nullptr, rho);
}

int topo_attn_decode_ragged(const topo_params_t* p, const int64_t* pos, const void* q, const void* k, const void* v,
                            float* out, int32_t* sel_idx, int32_t* sel_count, void* workspace, size_t ws_bytes,
                            hipStream_t stream) {
  if (!pos) return TOPO_EINVAL;
  return decode_like(p, q, k, v, out, sel_idx, sel_count, workspace, ws_bytes, stream, true, nullptr, nullptr, nullptr,
                     pos);
}

int topo_kv_append(const topo_params_t* p, const int64_t* pos, const void* k_new, const void* v_new, void* k_cache,
                   void* v_cache, hipStream_t stream) {
  int rc = check_params(p, false);
  if (rc) return rc;
  if (!pos || !aligned8(pos)) return TOPO_EINVAL;
  if (!k_new || !v_new || !k_cache || !v_cache || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return TOPO_EINVAL;
  const int32_t row_bytes = p->d * (p->dtype == TOPO_BF16 ? 2 : 4);
  return topo::launch_kv_append(k_new, v_new, k_cache, v_cache, pos, p->B, p->Hkv, p->n_ctx, row_bytes, stream) ==
                 hipSuccess
             ? TOPO_OK
             : TOPO_EHIP;
}

int topo_attn_prefill(const topo_params_t* p, const void* q, const void* k, const void* v, float* out,
                      int32_t* sel_idx, int32_t* sel_count, void* workspace, size_t ws_bytes,
                      hipStream_t stream) {
  return prefill_like(p, q, k, v, out, sel_idx, sel_count, workspace, ws_bytes, stream, true);
}

int topo_attn_prefill_timed(const topo_params_t* p, const void* q, const void* k, const void* v, float* out,
                            int32_t* sel_idx, int32_t* sel_count, void* workspace, size_t ws_bytes,
                            hipStream_t stream, hipEvent_t scan_begin, hipEvent_t scan_end) {
  if (!scan_begin || !scan_end) return TOPO_EINVAL;
  return prefill_like(p, q, k, v, out, sel_idx, sel_count, workspace, ws_bytes, stream, true, scan_begin, scan_end);
}

int topo_select(const topo_params_t* p, const void* q, const void* k, int32_t* sel_idx, int32_t* sel_count,
                void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!p) return TOPO_EINVAL;
  if (p->n_q == 1)
    return decode_like(p, q, k, nullptr, nullptr, sel_idx, sel_count, workspace, ws_bytes, stream, false);
  return prefill_like(p, q, k, nullptr, nullptr, sel_idx, sel_count, workspace, ws_bytes, stream, false);
}

int topo_attn_dense(const topo_params_t* p, const void* q, const void* k, const void* v, float* out,
                    void* workspace, size_t ws_bytes, hipStream_t stream) {
  int rc = check_params(p, false);
  if (rc) return rc;
  if (p->flags & (TOPO_FLAG_DENSE_FALLBACK | TOPO_FLAG_GROUP_SELECT)) return TOPO_EINVAL;
  if (!q || !k || !v || !out || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return TOPO_EINVAL;
  const size_t need = topo::dense_workspace_bytes(p->B, p->Hq, p->n_q, p->n_ctx, p->d);
  if (!workspace || ws_bytes < need || !aligned16(workspace)) return TOPO_EWORKSPACE;
  topo::DenseLaunch L{};
  L.q = q;
  L.k = k;
  L.v = v;
  L.out = out;
  L.ws = workspace;
  L.B = p->B;
  L.Hq = p->Hq;
  L.Hkv = p->Hkv;
  L.G = p->Hq / p->Hkv;
  L.d = p->d;
  L.bf16 = p->dtype == TOPO_BF16;
  L.causal = p->causal;
  L.n = p->n_ctx;
  L.n_q = p->n_q;
  L.q_pos0 = p->q_pos0;
  L.scale = (double)p->softmax_scale;
  return topo::launch_dense(L, stream) == hipSuccess ? TOPO_OK : TOPO_EHIP;
}

size_t topo_layers_workspace_bytes(const topo_params_t* p, const topo_layer_t* layers, int32_t n_layers) {
  if (!p || !layers || n_layers < 1) return 0;
  size_t need = 16;
  for (int32_t i = 0; i < n_layers; ++i) {
    topo_params_t pl = *p;
    pl.W = layers[i].W;
    pl.k = layers[i].k;
    if (layers[i].pillar) pl.flags &= ~TOPO_FLAG_GROUP_SELECT;
    const size_t b = layers[i].pillar ? topo_workspace_bytes(&pl, TOPO_OP_DENSE) : topo_workspace_bytes(&pl, TOPO_OP_DECODE);
    if (b == 0 || layers[i].reserved != 0 || (layers[i].pillar != 0 && layers[i].pillar != 1)) return 0;
    if (b > need) need = b;
  }
  return need;
}

int topo_attn_decode_layers(const topo_params_t* p, const topo_layer_t* layers, int32_t n_layers, void* workspace,
                            size_t ws_bytes, hipStream_t stream) {
  if (!p || !layers || n_layers < 1) return TOPO_EINVAL;
  int rc = check_params(p, false);
  if (rc) return rc;
  if (p->n_q != 1 || (p->flags & TOPO_FLAG_DENSE_FALLBACK)) return TOPO_EINVAL;
  // the shared selection serves groups of up to four query heads (checked here, before any layer
  // runs, as decode_like would check it at the first condensate-set layer)
  if ((p->flags & TOPO_FLAG_GROUP_SELECT) && p->Hq / p->Hkv > 4) return TOPO_EUNSUPPORTED;
  // every layer checked before the first launch
  for (int32_t i = 0; i < n_layers; ++i) {
    const topo_layer_t& L = layers[i];
    if (L.reserved != 0 || (L.pillar != 0 && L.pillar != 1)) return TOPO_EINVAL;
    topo_params_t pl = *p;
    pl.W = L.W;
    pl.k = L.k;
    if (!L.pillar && (rc = check_params(&pl, true)) != TOPO_OK) return rc;
    if (!L.q || !L.k_cache || !L.v_cache || !L.out || !aligned16(L.q) || !aligned16(L.k_cache) ||
        !aligned16(L.v_cache) || !aligned16(L.out))
      return TOPO_EINVAL;
    if ((L.sel_idx && !aligned16(L.sel_idx)) || (L.sel_count && !aligned16(L.sel_count))) return TOPO_EINVAL;
  }
  const size_t need = topo_layers_workspace_bytes(p, layers, n_layers);
  if (need == 0) return TOPO_EINVAL;
  if (!workspace || ws_bytes < need || !aligned16(workspace)) return TOPO_EWORKSPACE;
  for (int32_t i = 0; i < n_layers; ++i) {
    const topo_layer_t& L = layers[i];
    topo_params_t pl = *p;
    pl.W = L.W;
    pl.k = L.k;
    if (L.pillar) pl.flags &= ~TOPO_FLAG_GROUP_SELECT;  // a dense layer has no selection to share
    rc = L.pillar ? topo_attn_dense(&pl, L.q, L.k_cache, L.v_cache, L.out, workspace, ws_bytes, stream)
                  : topo_attn_decode(&pl, L.q, L.k_cache, L.v_cache, L.out, L.sel_idx, L.sel_count, workspace,
                                     ws_bytes, stream);
    if (rc != TOPO_OK) return rc;
  }
  return TOPO_OK;
}

int topo_pillar_plan(int32_t n_layers, int32_t W_first, int32_t k_first, int32_t W_last, int32_t k_last,
                     topo_layer_t* layers) {
  if (!layers || n_layers < 1 || W_first < 0 || k_first < 0 || W_last < 0 || k_last < 0) return TOPO_EINVAL;
  // rint rounds halves to even (the default rounding mode)
  int32_t n_pillar = (int32_t)std::rint((double)n_layers / 16.0);
  if (n_pillar < 1) n_pillar = 1;
  for (int32_t i = 0; i < n_layers; ++i) layers[i].pillar = 0;
  for (int32_t i = 0; i < n_pillar; ++i) layers[(int64_t)i * n_layers / n_pillar].pillar = 1;
  for (int32_t i = 0; i < n_layers; ++i) {
    const double t = n_layers > 1 ? (double)i / (double)(n_layers - 1) : 0.0;
    layers[i].W = (int32_t)std::rint((double)W_first + (double)(W_last - W_first) * t);
    layers[i].k = (int32_t)std::rint((double)k_first + (double)(k_last - k_first) * t);
  }
  return TOPO_OK;
}

int topo_check_finite(const void* buf, size_t count, int32_t dtype, uint32_t* flag, hipStream_t stream) {
  if (dtype != TOPO_F32 && dtype != TOPO_BF16) return TOPO_EUNSUPPORTED;
  if (!flag || ((uintptr_t)flag & 3u) || (count > 0 && (!buf || !aligned16(buf)))) return TOPO_EINVAL;
  if (count == 0) return TOPO_OK;
  return topo::launch_check_finite(buf, count, dtype == TOPO_BF16, flag, stream) == hipSuccess ? TOPO_OK : TOPO_EHIP;
}

int topo_workspace_view(const topo_params_t* p, int op, topo_ws_view_t* view) {
  if (!view) return TOPO_EINVAL;
  int rc = check_params(p, true);
  if (rc) return rc;
  topo_ws_view_t v{};
  if (op == TOPO_OP_PREFILL || (op == TOPO_OP_SELECT && p->n_q != 1)) {
    if (!topo::prefill_fits(p->W, p->k, p->dtype == TOPO_BF16)) return TOPO_EUNSUPPORTED;
    const topo::PrefillView pv = topo::prefill_view(p->B, p->Hq, p->Hkv, p->n_q, p->n_ctx, p->d, p->k);
    v.queries = (int64_t)p->B * p->Hq * p->n_q;
    v.lists = 1;
    v.slots = pv.slot;
    v.count_offset = pv.count;
    v.entry_offset = pv.entry;
    v.eps_offset = 0;
    v.path_offset = pv.path;
    v.path_stride = sizeof(int32_t);
    v.eps_coef = topo::prefill_eps_coef();
    v.count_split = 1;
  } else if (op == TOPO_OP_DECODE || op == TOPO_OP_SELECT || op == TOPO_OP_DECODE_CERTIFIED ||
             op == TOPO_OP_DECODE_RAGGED) {
    if (p->n_q != 1) return TOPO_EINVAL;
    if (op == TOPO_OP_DECODE_RAGGED && p->causal != 1) return TOPO_EINVAL;
    const topo::QueryGeom g = op == TOPO_OP_DECODE_RAGGED ? ragged_sizes_geom(p) : decode_geom(p);
    const topo::DecodeView dv =
        topo::decode_view(p->B, p->Hq, p->Hkv, g, p->k, p->d, p->dtype == TOPO_BF16);
    const bool scan = p->k > 0 && p->k <= topo::KS_MAX_K && g.n_cand > p->k && !(p->flags & TOPO_FLAG_EXACT_SELECT);
    v.queries = (int64_t)p->B * p->Hq;
    v.lists = scan ? dv.lists : 0;
    v.slots = dv.slot;
    v.count_offset = dv.count;
    v.entry_offset = dv.entry;
    v.eps_offset = dv.eps;
    v.path_offset = dv.state + offsetof(topo::HeadState, path);
    v.path_stride = sizeof(topo::HeadState);
    v.eps_coef = topo::fast_score_eps_coef(p->d);
  } else {
    return TOPO_EINVAL;
  }
  *view = v;
  return TOPO_OK;
}

int topo_bw_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink || !aligned16(buf) || bytes == 0 || (bytes & 15u)) return TOPO_EINVAL;
  return topo::launch_bw_probe(buf, bytes, sink, stream) == hipSuccess ? TOPO_OK : TOPO_EHIP;
}

const char* topo_strerror(int status) {
  switch (status) {
    case TOPO_OK: return "ok";
    case TOPO_EINVAL: return "invalid argument (shape, position, W/k, scale, pointer or alignment)";
    case TOPO_EUNSUPPORTED: return "unsupported dtype or head dimension";
    case TOPO_EWORKSPACE: return "workspace missing or smaller than topo_workspace_bytes()";
    case TOPO_EHIP: return "HIP kernel launch failed";
    case TOPO_ESCRATCH: return "the call needs more scratch than the allocation-free entry point's static buffer holds";
    default: return "unknown status";
  }
}

}  // extern "C"
