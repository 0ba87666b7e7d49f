/*
 * topo_attn.h — C ABI of the MI355X (gfx950) Topological Attention library, libtopo_attn.so.
 *
 * The operation. "The Condensate Theorem: Transformers are O(n), Not O(n^2)" (gist.science
 * explainers of arXiv 2602.06317) defines, for every query position i, a condensate set C_i made
 * of three parts: the anchor at position 0 (the attention sink), a local window of the W most
 * recent tokens, and the k positions with the highest Q.K^T scores, found again at every step
 * (zh page, technical summary §3 "研究方法"; fr page, technical summary §2; ko page, technical
 * summary §3 "동적 선택"). Topological Attention computes the softmax only over the positions in
 * C_i and sums their V rows with those weights (fr page, technical summary §3). The method swaps
 * only the attention operation of a frozen model (plug-and-play, zh technical summary §3), so
 * this interface takes the same tensors as an attention call: Q, the K and V caches, W, k and
 * the causal mask; it returns the output and the index set it used.
 *
 * Arithmetic (where the pages are silent, this library fixes one reading):
 *   score    s_j = sum_t q_t * k_{j,t}, the exact products summed in float64 in ascending t.
 *            The library ranks with fast float32 scores and re-scores the short list of possible
 *            members this way, so the index set is the one this definition gives.
 *   window   positions max(0, p-W+1) .. p (the query's own position p included).
 *   top-k    over the candidates: visible positions outside the anchor and the window. Higher
 *            score first, on equal scores the lower position first. If there are at most k
 *            candidates, all of them are taken.
 *   softmax  float64 on z_j = softmax_scale * s_j; the output is rounded once to float32.
 *            Exception: the prefill with bfloat16 inputs computes the logits, the softmax and
 *            the V sum in float32 (products of bfloat16 values exact; the set is still the one
 *            the score definition above gives), agreeing with the float64 definition to a few
 *            float32 roundings of the output's scale.
 *   GQA      query head h reads kv head h / (Hq / Hkv) and selects its own set.
 *   visible  causal: positions 0..p; otherwise 0..n_ctx-1 (the window still ends at p).
 *
 * Layouts (row-major, contiguous, element strides implied by the shapes):
 *   q        [B, Hq, n_q, d]        dtype of the call (float32 or bfloat16)
 *   k, v     [B, Hkv, n_ctx, d]     same dtype
 *   out      [B, Hq, n_q, d]        float32
 *   sel_idx  [B, Hq, n_q, 1+W+k]    int32, the set in ascending order, padded with -1
 *   sel_count[B, Hq, n_q]           int32, |C_i| = number of valid entries of sel_idx
 * Query i of a call sits at position q_pos0 + i.
 *
 * Ownership and execution. Every pointer argument is a device pointer owned by the caller
 * (q, k, v, out, sel_idx, sel_count, workspace), 16-byte aligned. The library never allocates or
 * frees device memory, keeps no mutable global state, and is safe to call from several host
 * threads on different streams with different workspaces. Calls are asynchronous on `stream`:
 * a return of TOPO_OK means every kernel was launched; faults surface at the caller's next
 * synchronisation. Arguments are validated before anything is launched, so on an error return
 * nothing has been written. The workspace must hold topo_workspace_bytes() bytes for the same
 * parameters and operation; its contents on entry do not matter and are scratch afterwards.
 * Two calls that run concurrently must not share a workspace.
 *
 * Finite inputs. q, k and v must hold finite values (no NaN, no infinity); topo_check_finite
 * tests a buffer on the device. What a non-finite value does: the kernels rank scores by integer
 * order keys of their bit patterns (a total order: NaN above +infinity, -0 equal to +0) and
 * gather only positions of visible keys taken from their own lists, so the set output keeps its
 * form (strictly ascending positions with the anchor and the window, padded with -1), but which
 * keys fill the top-k part and sel_count are then not defined by the score rule above, and out
 * (and rho) may hold NaN or infinity.
 */
#ifndef TOPO_ATTN_H
#define TOPO_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (negative on error). */
#define TOPO_OK            0
#define TOPO_EINVAL       -1   /* bad shape, position, W, k, scale, pointer or alignment      */
#define TOPO_EUNSUPPORTED -2   /* dtype or head dimension this build has no kernels for       */
#define TOPO_EWORKSPACE   -3   /* workspace NULL or smaller than topo_workspace_bytes()       */
#define TOPO_EHIP         -4   /* a kernel launch failed (hipGetLastError after the launch)   */
#define TOPO_ESCRATCH     -5   /* topo_attn_decode_noalloc: the call needs more scratch than
                                  TOPO_NOALLOC_MAX_BYTES                                        */

/* Element type of q, k and v. The output is always float32. */
#define TOPO_F32  0
#define TOPO_BF16 1

/* Operations, for topo_workspace_bytes(). */
#define TOPO_OP_DECODE  0
#define TOPO_OP_PREFILL 1
#define TOPO_OP_SELECT  2
#define TOPO_OP_DENSE   3
#define TOPO_OP_DECODE_CERTIFIED 4  /* topo_attn_decode_certified (includes the dense fallback's
                                       scratch when TOPO_FLAG_DENSE_FALLBACK is set)            */
#define TOPO_OP_DECODE_RAGGED 5     /* topo_attn_decode_ragged (sized for the longest position) */

/* Largest condensate set (1 + W + k) a call may ask for. The prefill also needs the LDS of its
 * per-row finish to hold four rows. With bfloat16 inputs and k <= 64 that LDS does not grow with
 * the set (at most 14 KB per block), so TOPO_MAX_SET is the only limit. Otherwise (float32
 * inputs, or k > 64), with S = 1 + W + k, P = roundup(k + 1, 144) and L = min(k + 48, 128),
 * 4 * roundup256(1092 + 12 * S + 8 * max(S, P / 2, 128) + 8 * (k + 1) + 4 * P + 12 * L)
 * <= 163840 bytes (S <= 1871 at k = 64, S <= 1849 at k = 96); larger sets return
 * TOPO_EUNSUPPORTED from the prefill calls (and 0 from topo_workspace_bytes). */
#define TOPO_MAX_SET 4096

/* Flag bits of topo_params_t.flags. */
#define TOPO_FLAG_EXACT_SELECT 1  /* skip the float32 pre-ranking and select every query by the
                                     exact float64 radix path (slow; for checking)             */
#define TOPO_FLAG_DENSE_FALLBACK 2  /* topo_attn_decode_certified only: queries whose bound rho is
                                       not below TOPO_CERT_RHO get dense attention in out      */

#define TOPO_FLAG_GROUP_SELECT 4  /* decode calls (topo_attn_decode, _timed, _ragged, topo_select
                                     with n_q == 1): one condensate set per (batch, kv head),
                                     shared by the G = Hq / Hkv query heads of the group (G <= 4;
                                     TOPO_EUNSUPPORTED otherwise). A key's group score is the
                                     largest of the group's per-head scores; the top-k ranks group
                                     scores (higher first, lower position on ties); each head then
                                     takes the softmax of its own scores over the shared set, and
                                     sel_idx / sel_count repeat the set for every head of the
                                     group. The pages name GQA without fixing how it selects; this
                                     is the shared-selection variant. Not accepted by the prefill,
                                     dense and certified calls (TOPO_EINVAL).                   */

/* A query is certified when its bound on the left-out softmax mass is below the float32
 * rounding unit 2^-24: the set then carries the dense softmax to float32 precision, the
 * exactness claim of the pages (zh technical summary §2; hi technical summary §2). */
#define TOPO_CERT_RHO 0x1p-24f

typedef struct {
    int32_t B;              /* batch                                                     >= 1 */
    int32_t Hq;             /* query heads                                               >= 1 */
    int32_t Hkv;            /* kv heads; Hq % Hkv == 0                                   >= 1 */
    int32_t d;              /* head dimension: 64 or 128                                      */
    int64_t n_ctx;          /* keys per (batch, kv head), 1 .. 2^31-1                         */
    int64_t n_q;            /* queries per (batch, head): decode 1; prefill 1 .. n_ctx        */
    int64_t q_pos0;         /* position of query 0; q_pos0 + n_q - 1 <= n_ctx - 1             */
    int32_t W;              /* window length                                             >= 0 */
    int32_t k;              /* top-k size                                                >= 0 */
    int32_t causal;         /* 1: query at p sees keys 0..p; 0: it sees all n_ctx keys        */
    float   softmax_scale;  /* > 0 and finite (1/sqrt(d), or a temperature over sqrt(d))      */
    int32_t dtype;          /* TOPO_F32 or TOPO_BF16                                          */
    int32_t flags;          /* TOPO_FLAG_* bits, 0 normally                                   */
} topo_params_t;

/* Workspace bytes that the operation needs for these parameters (0 if they are invalid). */
size_t topo_workspace_bytes(const topo_params_t* p, int op);

/* Topological attention of one query per (batch, query head): n_q == 1, the query at position
 * q_pos0 (the newest token of a decode step is q_pos0 = n_ctx - 1). Writes out, and sel_idx /
 * sel_count unless they are NULL. Condensate set and softmax as above (zh technical summary §3;
 * fr technical summary §3). */
int topo_attn_decode(const topo_params_t* p, const void* q, const void* k, const void* v,
                     float* out, int32_t* sel_idx, int32_t* sel_count,
                     void* workspace, size_t ws_bytes, hipStream_t stream);

/* Allocation-free variant of topo_attn_decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and results, with the workspace in a buffer of TOPO_NOALLOC_MAX_BYTES that the library
 * holds per GPU (a static device array, allocated when the library's code is loaded on that GPU
 * and kept until the process ends) instead of a caller's. It calls no hipMalloc, hipFree or
 * allocating routine. Unlike the other calls this one has global state: every call on a GPU uses
 * that GPU's one buffer, so two calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller; calls in stream order are fine (each call
 * initialises what it reads). Returns TOPO_ESCRATCH, launching nothing, when
 * topo_workspace_bytes(p, TOPO_OP_DECODE) exceeds TOPO_NOALLOC_MAX_BYTES (e.g. 20.6 MiB for
 * B = 1, Hq = 32, Hkv = 8, d = 128, n_ctx = 2^20, W = 512, k = 64 bf16 fits); TOPO_EHIP if the
 * buffer's device address cannot be found; otherwise errors as topo_attn_decode. */
#define TOPO_NOALLOC_MAX_BYTES (32u << 20)
int topo_attn_decode_noalloc(const topo_params_t* p, const void* q, const void* k, const void* v,
                             float* out, int32_t* sel_idx, int32_t* sel_count, hipStream_t stream);

/* Measurement variant of topo_attn_decode: identical results, and additionally records the
 * caller's events scan_begin / scan_end on `stream` immediately before and after the key-scan
 * kernel (the step that streams K from HBM), so its duration can be read with
 * hipEventElapsedTime. The events must be valid hipEvent_t handles created by the caller; if no
 * scan is needed (k = 0, or at most k candidates) both are recorded back to back. */
int topo_attn_decode_timed(const topo_params_t* p, const void* q, const void* k, const void* v,
                           float* out, int32_t* sel_idx, int32_t* sel_count,
                           void* workspace, size_t ws_bytes, hipStream_t stream,
                           hipEvent_t scan_begin, hipEvent_t scan_end);

/* topo_attn_decode plus an exactness certificate per query. rho[B*Hq] (device, float32, written
 * for every query) receives an upper bound on the softmax mass of the visible keys left out of
 * the set, relative to the dense total: every left-out candidate scores at most s_k, the lowest
 * score of the top-k part, so rho = (number of left-out candidates) * exp(scale*s_k - zmax) / Z,
 * with zmax and Z the float64 softmax maximum and sum over the set (rounded up to float32; 0 if
 * no candidate is left out; +inf if candidates are left out and k = 0). With
 * TOPO_FLAG_DENSE_FALLBACK in p->flags, every query with rho >= TOPO_CERT_RHO gets the dense
 * attention output (as topo_attn_dense) in out instead; sel_idx / sel_count still describe the
 * condensate set. Workspace: topo_workspace_bytes(p, TOPO_OP_DECODE_CERTIFIED). Errors as
 * topo_attn_decode, and TOPO_EINVAL if rho is NULL or not 16-byte aligned. */
int topo_attn_decode_certified(const topo_params_t* p, const void* q, const void* k, const void* v,
                               float* out, int32_t* sel_idx, int32_t* sel_count, float* rho,
                               void* workspace, size_t ws_bytes, hipStream_t stream);

/* Decode of a batch whose sequences have different lengths, the per-token step of a generation
 * loop (the pages re-select the set at every generated token: zh technical summary §3). pos is a
 * device array of B int64 positions, 8-byte aligned: the query of batch element b sits at
 * position pos[b] of its own cache and sees keys 0 .. pos[b] (the call is causal; p->causal must
 * be 1). The caches keep their [B, Hkv, n_ctx, d] layout; rows past a sequence's position are not
 * read by its query. p->q_pos0 is not used for the positions (it is still validated). Each query's
 * set and output are those of topo_attn_decode with q_pos0 = pos[b] on that sequence. A position
 * outside [0, n_ctx - 1] is clamped into it (a caller error; no memory outside the caches is
 * read). Because the positions live in device memory, a captured HIP graph of this call serves
 * every step of a loop that advances them on the device. Workspace:
 * topo_workspace_bytes(p, TOPO_OP_DECODE_RAGGED). Errors as topo_attn_decode, and TOPO_EINVAL if
 * pos is NULL or misaligned or p->causal != 1. */
int topo_attn_decode_ragged(const topo_params_t* p, const int64_t* pos, const void* q, const void* k, const void* v,
                            float* out, int32_t* sel_idx, int32_t* sel_count,
                            void* workspace, size_t ws_bytes, hipStream_t stream);

/* KV-cache append, the step before a decode: for every (b, kv head g), the new key and value rows
 * k_new[b, g, :] and v_new[b, g, :] (layout [B, Hkv, d], the call's dtype) are copied to row
 * pos[b] of k_cache and v_cache ([B, Hkv, n_ctx, d]). pos as in topo_attn_decode_ragged (device,
 * B int64); a position outside [0, n_ctx - 1] writes nothing for that batch element. Uses B, Hkv,
 * d, n_ctx and dtype of p; no workspace. Asynchronous on stream; TOPO_EINVAL on a NULL or
 * misaligned pointer. */
int topo_kv_append(const topo_params_t* p, const int64_t* pos, const void* k_new, const void* v_new,
                   void* k_cache, void* v_cache, hipStream_t stream);

/* Topological attention of n_q consecutive queries per (batch, query head), query i at position
 * q_pos0 + i (a whole causal prompt is q_pos0 = 0, n_q = n_ctx). Same outputs as decode, one row
 * per query (zh technical summary §3). */
int topo_attn_prefill(const topo_params_t* p, const void* q, const void* k, const void* v,
                      float* out, int32_t* sel_idx, int32_t* sel_count,
                      void* workspace, size_t ws_bytes, hipStream_t stream);

/* Measurement variant of topo_attn_prefill: identical results, and additionally records the
 * caller's events scan_begin / scan_end on `stream` immediately before and after the key-scan
 * kernel (the matrix-core pass that scores every candidate key of every query row). The events
 * must be valid hipEvent_t handles created by the caller; when no scan runs (k = 0, float32
 * inputs, k above the scan's limit, or TOPO_FLAG_EXACT_SELECT) both are recorded back to back. */
int topo_attn_prefill_timed(const topo_params_t* p, const void* q, const void* k, const void* v,
                            float* out, int32_t* sel_idx, int32_t* sel_count,
                            void* workspace, size_t ws_bytes, hipStream_t stream,
                            hipEvent_t scan_begin, hipEvent_t scan_end);

/* The condensate sets only (the selection of decode or prefill, chosen by n_q == 1 or not),
 * without the softmax and V reduction. sel_idx and sel_count must not be NULL. */
int topo_select(const topo_params_t* p, const void* q, const void* k,
                int32_t* sel_idx, int32_t* sel_count,
                void* workspace, size_t ws_bytes, hipStream_t stream);

/* Dense softmax attention over every visible key (W and k are ignored): the full-attention
 * layers the zh page keeps in a few "pillar" layers (technical summary §3) and the comparator of
 * the exactness claim (technical summary §2). float32 scores and accumulation for bfloat16
 * inputs, float64 for float32 inputs. Any n_q; writes out. */
int topo_attn_dense(const topo_params_t* p, const void* q, const void* k, const void* v,
                    float* out, void* workspace, size_t ws_bytes, hipStream_t stream);

/* One attention layer of a decode step through a model's stack of layers. The pages keep a few
 * layers fully dense, the "pillar" layers (about one layer in sixteen), and size the condensate
 * set per layer: wider windows in early layers, leaner sets in later ones (zh technical summary
 * §3). Pointers are device pointers; the struct itself lives in host memory. */
typedef struct {
    const void* q;        /* [B, Hq, d] the layer's queries (dtype of the call)                  */
    const void* k_cache;  /* [B, Hkv, n_ctx, d] the layer's key cache                            */
    const void* v_cache;  /* [B, Hkv, n_ctx, d] the layer's value cache                          */
    float*      out;      /* [B, Hq, d] float32                                                  */
    int32_t*    sel_idx;  /* [B, Hq, 1 + W + k] or NULL; not written for a pillar layer          */
    int32_t*    sel_count;/* [B, Hq] or NULL; not written for a pillar layer                     */
    int32_t     W;        /* the layer's window (>= 0; unused by a pillar layer)                 */
    int32_t     k;        /* the layer's top-k (>= 0; unused by a pillar layer)                  */
    int32_t     pillar;   /* 1: dense attention over every visible key (topo_attn_dense); 0: the
                             condensate set (topo_attn_decode)                                   */
    int32_t     reserved; /* 0                                                                   */
} topo_layer_t;

/* Workspace bytes for topo_attn_decode_layers: the largest any of the layers needs (the layers
 * run one after the other on the stream and share it). 0 if a layer's parameters are invalid. */
size_t topo_layers_workspace_bytes(const topo_params_t* p, const topo_layer_t* layers, int32_t n_layers);

/* A decode step through n_layers attention layers (n_layers >= 1): layer i runs topo_attn_decode
 * with p's shapes, position, scale, dtype and flags and the layer's W and k, or topo_attn_dense
 * when it is a pillar layer, in order on `stream`. TOPO_FLAG_GROUP_SELECT in p->flags applies to
 * the condensate-set layers (pillar layers are dense and ignore it). Every layer is validated
 * before anything is launched (errors as those calls, e.g. TOPO_EUNSUPPORTED for the group flag
 * with G > 4; TOPO_EINVAL if layers is NULL, n_layers < 1 or reserved != 0). */
int topo_attn_decode_layers(const topo_params_t* p, const topo_layer_t* layers, int32_t n_layers,
                            void* workspace, size_t ws_bytes, hipStream_t stream);

/* The per-layer plan of a stack of n_layers attention layers (host only, no GPU work): the zh page
 * keeps about one layer in sixteen fully dense, the "pillar" layers, and sizes the condensate set
 * per layer, with wider windows early and leaner sets late (technical summary §3), without a
 * formula. This library's reading: max(1, round(n_layers / 16)) pillar layers (halves rounded to
 * even), layer i * n_layers / n_pillar for i = 0 .. n_pillar - 1; every layer gets
 * W = round(W_first + (W_last - W_first) * t) and k likewise, t = layer / (n_layers - 1) (0 for
 * one layer), halves rounded to even. Fills pillar, W and k of layers[0 .. n_layers - 1] (the
 * other fields are left as they are). TOPO_EINVAL if layers is NULL, n_layers < 1 or a W or k is
 * negative. */
int topo_pillar_plan(int32_t n_layers, int32_t W_first, int32_t k_first, int32_t W_last, int32_t k_last,
                     topo_layer_t* layers);

/* Finite-input check (the calls above require finite q, k and v): sets bit 0 of *flag (one uint32
 * in device memory, not cleared by this call) if any of the `count` elements of `buf` (dtype
 * TOPO_F32 or TOPO_BF16) is a NaN or an infinity. Asynchronous on `stream`; read *flag after
 * synchronising. TOPO_EINVAL on a NULL or misaligned pointer (buf 16-byte, flag 4-byte aligned),
 * TOPO_EUNSUPPORTED on another dtype. */
int topo_check_finite(const void* buf, size_t count, int32_t dtype, uint32_t* flag, hipStream_t stream);

/* Diagnostics. How a query's top-k part was chosen (TOPO_PATH_*), and where a call leaves the key
 * scan's candidate lists in its workspace, so that the fast scores can be checked against exact
 * ones and the paths counted. The layout describes the workspace of the given parameters and
 * operation; the contents are those of the last call that used the workspace, once it has
 * completed. */
#define TOPO_PATH_NONE 0            /* no top-k part (k = 0 or no candidate)                       */
#define TOPO_PATH_ALL 1             /* at most k candidates, all taken                             */
#define TOPO_PATH_FAST 2            /* from the scan's lists: decode re-scores the short list in
                                       float64; prefill: the fast scores' bounds decided it        */
#define TOPO_PATH_BAND 3            /* prefill: from the lists, entries in the band re-scored      */
#define TOPO_PATH_EXACT_ASKED 4     /* exact float64 radix selection over every candidate: flag,
                                       float32 prefill, or a size above the scan's limits          */
#define TOPO_PATH_EXACT_OVERFLOW 5  /* the same, after a scan list overflowed (tie-heavy keys)     */
#define TOPO_PATH_EXACT_CROWDED 6   /* the same, after the decode short list was crowded (ties)    */

typedef struct {
    int64_t queries;       /* query rows described: B*Hq (decode ops) or B*Hq*n_q (prefill)      */
    int64_t lists;         /* candidate lists per query row                                      */
    int64_t slots;         /* entries per list                                                   */
    size_t  count_offset;  /* uint32 [queries][lists]: entries of each list (count_split = 0:
                              the count, 0xFFFFFFFF if the list overflowed; count_split = 1: the
                              low 16 bits count entries from the front of the slots, the high 16
                              bits entries from the back, overflowed if their sum exceeds slots)  */
    size_t  entry_offset;  /* [queries][lists][slots] pairs {float fast score, int32 position}   */
    size_t  eps_offset;    /* float [queries][lists][slots]: the bound the kernels used for each
                              entry (decode); 0 when not stored (prefill: eps_coef |q| |k|)      */
    size_t  path_offset;   /* int32 TOPO_PATH_* of query i at path_offset + i * path_stride       */
    size_t  path_stride;
    float   eps_coef;      /* every fast score obeys |s_fast - s| <= eps_coef * |q|_2 * |k|_2    */
    int32_t count_split;   /* 0: decode lists; 1: prefill lists (see count_offset)              */
} topo_ws_view_t;

/* Fills *view for op TOPO_OP_DECODE, TOPO_OP_SELECT, TOPO_OP_DECODE_CERTIFIED,
 * TOPO_OP_DECODE_RAGGED or TOPO_OP_PREFILL (decode: the key scan's own lists, before any merge;
 * prefill: one list per query row). The decode layout depends on the current device's compute
 * unit count, like the calls. lists = 0 when the call runs no key scan (k = 0, at most k
 * candidates, the exact flag, or k or the shape above the scan's limits). TOPO_EINVAL for another
 * op, invalid parameters or a NULL view; TOPO_EUNSUPPORTED as the call itself. */
int topo_workspace_view(const topo_params_t* p, int op, topo_ws_view_t* view);

/* Measurement helper, not part of the method: streams `bytes` (a multiple of 16) from `buf`
 * once with the same load path as the decode key scan and reduces them into `sink`
 * (one uint32, device memory), so the achievable read bandwidth can be timed next to it. */
int topo_bw_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Static description of a status code. */
const char* topo_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* TOPO_ATTN_H */
