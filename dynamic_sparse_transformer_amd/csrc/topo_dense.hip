// Dense softmax attention over every visible key on gfx950: the full-attention "pillar" layers
// that the zh page of "The Condensate Theorem: Transformers are O(n), Not O(n^2)" keeps in a few
// layers (technical summary §3), and the comparator of the exactness claim (technical summary
// §2). Split over the keys (flash-decoding): each block folds a range of keys into a partial
// (max, sum of weights, weighted V sum) per query head with an online softmax; a second kernel
// merges the partials. K and V are each read once per (batch, kv head) for all G query heads.
// bf16 inputs use float32 scores and accumulation (dense_stream_kernel, which streams K and V
// like the decode key scan streams K); float32 inputs use float64 for both (dense_partial_kernel,
// tiles staged through LDS).
#include "topo_device.h"
#include "topo_internal.h"

namespace topo {

constexpr int DN_IT = 8;                             // 64-key tiles per wave
constexpr int DN_KEYS = 4 * DN_IT * 64;              // keys per block (4 waves)

template <int D>
struct alignas(16) DensePartial {
  double m;      // max logit of the run (-inf if the run saw no visible key)
  double z;      // sum of exp(logit - m)
  double nv[D];  // sum of exp(logit - m) * v
};

size_t dense_workspace_bytes(int32_t B, int32_t Hq, int64_t n_q, int64_t n, int32_t d) {
  const int64_t chunks = (n + DN_KEYS - 1) / DN_KEYS;
  const size_t per = d == 128 ? sizeof(DensePartial<128>) : sizeof(DensePartial<64>);
  return (size_t)B * Hq * (size_t)n_q * (size_t)chunks * per;
}

struct DenseArgs {
  const unsigned char* q;
  const unsigned char* k;
  const unsigned char* v;
  void* part;
  int64_t n, n_q, q_pos0, chunks;
  int64_t kpb;        // keys per block (the partial of block x covers keys [x * kpb, (x + 1) * kpb))
  int32_t Hq, Hkv, G, causal, nslices;
  int32_t runs;       // dense_stream_kernel: runs of DS_KEYS_PER_RUN keys per block
  double scale;
  const float* gate;  // may be null; else rows with gate[row] < gate_min are skipped
  float gate_min;
};

template <bool BF16>
__device__ __forceinline__ void unpack_chunk(uint4 w, float (&x)[BF16 ? 8 : 4]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  if constexpr (BF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_lo(ws[e]);
      x[2 * e + 1] = bf16_hi(ws[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(ws[e]);
  }
}

// grid (chunks, B*Hkv, n_q*nslices), 256 threads.
template <int D, int GT, bool BF16>
__global__ __launch_bounds__(256) void dense_partial_kernel(DenseArgs a) {
  using AccT = typename std::conditional<BF16, float, double>::type;
  constexpr int RB = D * (BF16 ? 2 : 4);
  constexpr int NCH = RB / 16;        // 16-byte chunks per row
  constexpr int EPC = BF16 ? 8 : 4;   // elements per chunk
  constexpr int RG = 64 / NCH;        // rows covered by one 64-lane load
  constexpr int STRIDE = RB + 16;
  __shared__ __align__(16) unsigned char stage[4][64 * STRIDE];
  __shared__ __align__(16) uint4 qs[GT][NCH];
  __shared__ AccT wts[4][GT][64];
  __shared__ AccT wm[4][GT], wz[4][GT];
  __shared__ AccT wn[4][GT][D];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = blockIdx.y;
  const int b = grp / a.Hkv, g = grp - b * a.Hkv;
  const int qi = blockIdx.z / a.nslices, slice = blockIdx.z - qi * a.nslices;
  const int h0 = g * a.G + slice * GT;
  const int nh = min(GT, a.G - slice * GT);
  const int64_t p = a.q_pos0 + qi;
  const int64_t vis_hi = a.causal ? p : a.n - 1;
  if (a.gate) {  // skip the block if none of its query rows is gated in
    bool any = false;
    for (int h = 0; h < nh; ++h) any |= a.gate[((size_t)b * a.Hq + h0 + h) * a.n_q + qi] >= a.gate_min;
    if (!any) return;
  }

  for (int i = tid; i < GT * NCH; i += 256) {
    const int h = i / NCH, c = i % NCH;
    const unsigned char* qrow = a.q + (((size_t)b * a.Hq + h0 + h) * a.n_q + qi) * RB;
    qs[h][c] = h < nh ? *(const uint4*)(qrow + c * 16) : make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();

  const unsigned char* kb = a.k + (size_t)grp * (size_t)a.n * RB;
  const unsigned char* vb = a.v + (size_t)grp * (size_t)a.n * RB;
  const int64_t key0 = (int64_t)blockIdx.x * DN_KEYS + (int64_t)wave * (DN_IT * 64);
  unsigned char* tile = stage[wave];

  AccT m_run[GT], z_run[GT], acc[GT][EPC];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    m_run[h] = -INFINITY;
    z_run[h] = 0;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[h][e] = 0;
  }

  for (int it = 0; it < DN_IT; ++it) {
    const int64_t row0 = key0 + (int64_t)it * 64;
    if (row0 > vis_hi) break;  // uniform across the wave
    uint4 kbuf[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ci = i * 64 + lane, r = ci / NCH, c = ci % NCH;
      const int64_t row = row0 + r;
      kbuf[i] = row <= vis_hi ? ntload16(kb + row * RB + c * 16)
                              : make_uint4(0u, 0u, 0u, 0u);
    }
    uint4 vbuf[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ci = i * 64 + lane, r = ci / NCH, c = ci % NCH;
      const int64_t row = row0 + r;
      vbuf[i] = row <= vis_hi ? ntload16(vb + row * RB + c * 16)
                              : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ci = i * 64 + lane, r = ci / NCH, c = ci % NCH;
      *(uint4*)(tile + r * STRIDE + c * 16) = kbuf[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // score of key row0 + lane for each head
    AccT z[GT];
    const unsigned char* myrow = tile + lane * STRIDE;
#pragma unroll
    for (int h = 0; h < GT; ++h) z[h] = 0;
    if constexpr (BF16) {
      float s[GT];
#pragma unroll
      for (int h = 0; h < GT; ++h) s[h] = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint4 kv = *(const uint4*)(myrow + c * 16);
#pragma unroll
        for (int h = 0; h < GT; ++h) s[h] = dot_chunk_bf16(kv, qs[h][c], s[h]);
      }
#pragma unroll
      for (int h = 0; h < GT; ++h) z[h] = (float)a.scale * s[h];
    } else {
      double s[GT];
#pragma unroll
      for (int h = 0; h < GT; ++h) s[h] = 0.0;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint4 kv = *(const uint4*)(myrow + c * 16);
        const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          const uint4 qv = qs[h][c];
          const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s[h] = fma((double)__uint_as_float(qw[e]), (double)__uint_as_float(kw[e]), s[h]);
        }
      }
#pragma unroll
      for (int h = 0; h < GT; ++h) z[h] = a.scale * s[h];
    }
    const bool vis = row0 + lane <= vis_hi;
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      AccT zt = vis ? z[h] : (AccT)(-INFINITY);
      AccT mt = zt;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mt = fmax(mt, __shfl_xor(mt, o));  // shuffle outside any branch
      const AccT m_new = m_run[h] > mt ? m_run[h] : mt;
      const AccT keep = exp(m_run[h] - m_new);  // 0 on the first visible tile
      const AccT w = vis ? (AccT)exp(zt - m_new) : (AccT)0;
      AccT ws = w;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) ws += __shfl_xor(ws, o);
      z_run[h] = z_run[h] * keep + ws;
      m_run[h] = m_new;
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[h][e] *= keep;
      wts[wave][h][lane] = w;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // weighted V rows: this lane holds chunk (lane % NCH) of rows (lane / NCH) + RG * i
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int r = (i * 64 + lane) / NCH;
      float x[EPC];
      unpack_chunk<BF16>(vbuf[i], x);
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const AccT w = wts[wave][h][r];
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] = fma(w, (AccT)x[e], acc[h][e]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // fold the row groups of the wave: lanes lane % NCH share a chunk
#pragma unroll
  for (int h = 0; h < GT; ++h)
#pragma unroll
    for (int e = 0; e < EPC; ++e)
      for (int o = NCH; o < 64; o <<= 1) acc[h][e] += __shfl_xor(acc[h][e], o);
  for (int h = 0; h < GT; ++h) {
    if (lane < NCH) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) wn[wave][h][lane * EPC + e] = acc[h][e];
    }
    if (lane == 0) {
      wm[wave][h] = m_run[h];
      wz[wave][h] = z_run[h];
    }
  }
  __syncthreads();
  // merge the 4 waves and write the block's partial
  for (int i = tid; i < nh * D; i += 256) {
    const int h = i / D, c = i - h * D;
    AccT m = wm[0][h];
    for (int w = 1; w < 4; ++w) m = m > wm[w][h] ? m : wm[w][h];
    double nv = 0.0;
    double zz = 0.0;
    if (m != (AccT)(-INFINITY)) {
      for (int w = 0; w < 4; ++w) {
        const double f = exp((double)(wm[w][h] - m));
        nv += f * (double)wn[w][h][c];
        zz += f * (double)wz[w][h];
      }
    }
    DensePartial<D>* part = (DensePartial<D>*)a.part +
                            ((((size_t)b * a.Hq + h0 + h) * a.n_q + qi) * a.chunks + blockIdx.x);
    part->nv[c] = nv;
    if (c == 0) {
      part->m = (double)m;
      part->z = zz;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dense_stream (bf16 inputs): grid (blocks over the keys, B*Hkv, n_q*nslices), 256 threads. Block x
// folds keys [x * kpb, (x + 1) * kpb) in `runs` runs of 4 waves x 512 keys, as the decode key scan
// lays out its loads: a 64-key tile is 8 groups of 8 lanes, group r holds keys 8i + r (i < 8) and
// lane s of a group the 16-byte chunks c*8 + s (c < CPL) of each, so every load instruction reads
// eight full 128-byte half rows. K and V of a tile have register sets of their own, and each key
// group's registers are reloaded with the next tile as soon as they are used (K after the partial
// dot products, V after the weighted sum), so every wave keeps about a tile of K and V (32 KB at
// d = 128) in flight; with the accumulators of four heads that takes one wave per SIMD (up to 512
// registers). A reduce-scatter over the 8 lanes of a group leaves every lane the score of key 8s + r; the
// online softmax keeps a wave-wide running maximum per head (the partial output and sums are
// rescaled when it rises); the weight of key 8i + r reaches the lanes of group r by a swizzle.
// At the end the 8 key groups and the 4 waves are folded into one partial per head.
constexpr int DS_KEYS_PER_RUN = 2048;
constexpr int DS_MAX_RUNS = 16;

// Value of lane 8 (lane / 8) + i in every lane (i < 8): within each 32-lane half, the swizzle keeps
// lane bits 3-4 (and_mask 0x18) and sets bits 0-2 to i (or_mask). i is a constant once unrolled.
__device__ __forceinline__ float group_bcast(float x, int i) {
  const int v = __float_as_int(x);
  switch (i) {
    case 0: return __int_as_float(__builtin_amdgcn_ds_swizzle(v, 0x18 | (0 << 5)));
    case 1: return __int_as_float(__builtin_amdgcn_ds_swizzle(v, 0x18 | (1 << 5)));
    case 2: return __int_as_float(__builtin_amdgcn_ds_swizzle(v, 0x18 | (2 << 5)));
    case 3: return __int_as_float(__builtin_amdgcn_ds_swizzle(v, 0x18 | (3 << 5)));
    case 4: return __int_as_float(__builtin_amdgcn_ds_swizzle(v, 0x18 | (4 << 5)));
    case 5: return __int_as_float(__builtin_amdgcn_ds_swizzle(v, 0x18 | (5 << 5)));
    case 6: return __int_as_float(__builtin_amdgcn_ds_swizzle(v, 0x18 | (6 << 5)));
    default: return __int_as_float(__builtin_amdgcn_ds_swizzle(v, 0x18 | (7 << 5)));
  }
}

template <int RB, int GT>
__global__ __launch_bounds__(256, 1) void dense_stream_kernel(DenseArgs a) {
  constexpr int D = RB / 2;       // bf16 elements per row
  constexpr int CPL = RB / 128;   // 16-byte chunks of a row per lane
  constexpr int EL = CPL * 8;     // elements of a row per lane
  __shared__ float wn[4][GT][D];
  __shared__ float wm[4][GT], wz[4][GT];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, s = lane & 7, r = lane >> 3;
  const int grp = blockIdx.y;
  const int b = grp / a.Hkv, g = grp - b * a.Hkv;
  const int qi = blockIdx.z / a.nslices, slice = blockIdx.z - qi * a.nslices;
  const int h0 = g * a.G + slice * GT;
  const int nh = min(GT, a.G - slice * GT);
  const int64_t p = a.q_pos0 + qi;
  const int64_t vis_hi = a.causal ? p : a.n - 1;
  const int64_t blk_key0 = (int64_t)blockIdx.x * a.kpb;
  if (blk_key0 > vis_hi) return;  // no visible key: the combine reads no partial of this block
  if (a.gate) {  // skip the block if none of its query rows is gated in
    bool any = false;
    for (int h = 0; h < nh; ++h) any |= a.gate[((size_t)b * a.Hq + h0 + h) * a.n_q + qi] >= a.gate_min;
    if (!any) return;
  }

  uint4 qv[GT][CPL];
#pragma unroll
  for (int h = 0; h < GT; ++h)
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      qv[h][c] = h < nh ? *(const uint4*)(a.q + (((size_t)b * a.Hq + h0 + h) * a.n_q + qi) * RB + c * 128 + s * 16)
                        : make_uint4(0u, 0u, 0u, 0u);
  const float sc = (float)a.scale;
  const unsigned char* kb = a.k + (size_t)grp * (size_t)a.n * RB;
  const unsigned char* vb = a.v + (size_t)grp * (size_t)a.n * RB;
  auto tile_key0 = [&](int t) -> int64_t {  // tile t of this wave: run t / 8, tile t % 8 of the wave's 512 keys
    return blk_key0 + (int64_t)((t >> 3) * 4 + wave) * 512 + (int64_t)(t & 7) * 64;
  };
  // loads of key group i of the tile at row0 (rows past the last visible key clamped onto it; their
  // weights are zero)
  auto load_group = [&](uint4 (&dst)[CPL], const unsigned char* base, int64_t row0, int i) {
    const int64_t row = row0 + 8 * i + r;
    const unsigned char* src = base + (row <= vis_hi ? row : vis_hi) * RB + s * 16;
#pragma unroll
    for (int c = 0; c < CPL; ++c) dst[c] = ntload16(src + c * 128);
  };

  float acc[GT][EL], m_run[GT], z_run[GT];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    m_run[h] = -INFINITY;
    z_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EL; ++e) acc[h][e] = 0.f;
  }
  uint4 kk[8][CPL], vv[8][CPL];
  const int ntiles = a.runs * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) load_group(kk[i], kb, tile_key0(0), i);
#pragma unroll
  for (int i = 0; i < 8; ++i) load_group(vv[i], vb, tile_key0(0), i);
#pragma unroll 1
  for (int t = 0; t < ntiles; ++t) {
    const int64_t row0 = tile_key0(t);
    const bool more = t + 1 < ntiles;
    const int64_t nrow0 = more ? tile_key0(t + 1) : row0;
    // K of tile t: partial dot products, then the registers take K of tile t+1
    float P[GT][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float d = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) d = dot_chunk_bf16(kk[i][c], qv[h][c], d);
        P[h][i] = d;
      }
      if (more) load_group(kk[i], kb, nrow0, i);
    }
    const bool valid = row0 + 8 * s + r <= vis_hi;
    float w[GT];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      float Q1[1][8];
#pragma unroll
      for (int i = 0; i < 8; ++i) Q1[0][i] = P[h][i];
      reduce_scatter<8, 1>(Q1, s);
      const float z = valid ? sc * Q1[0][0] : -INFINITY;
      float tm = z;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) tm = fmaxf(tm, __shfl_xor(tm, o));
      if (tm > m_run[h]) {  // wave-uniform: the running maximum rises, rescale what was summed
        const float f = __expf(m_run[h] - tm);
        z_run[h] *= f;
#pragma unroll
        for (int e = 0; e < EL; ++e) acc[h][e] *= f;
        m_run[h] = tm;
      }
      w[h] = valid ? __expf(z - m_run[h]) : 0.f;
      z_run[h] += w[h];
    }
    // V of tile t: the weighted sum, then the registers take V of tile t+1
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float wi[GT];
#pragma unroll
      for (int h = 0; h < GT; ++h)  // weight of key 8i + r, held by lane 8r + i of the group
        wi[h] = group_bcast(w[h], i);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const uint32_t ws[4] = {vv[i][c].x, vv[i][c].y, vv[i][c].z, vv[i][c].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = bf16_lo(ws[e]), hi = bf16_hi(ws[e]);
#pragma unroll
          for (int h = 0; h < GT; ++h) {
            acc[h][c * 8 + 2 * e] = fmaf(wi[h], lo, acc[h][c * 8 + 2 * e]);
            acc[h][c * 8 + 2 * e + 1] = fmaf(wi[h], hi, acc[h][c * 8 + 2 * e + 1]);
          }
        }
      }
      if (more) load_group(vv[i], vb, nrow0, i);
    }
  }

  // fold the key groups (lanes with equal s hold the same elements) and the lanes' weight sums
#pragma unroll
  for (int h = 0; h < GT; ++h) {
#pragma unroll
    for (int e = 0; e < EL; ++e)
      for (int o = 8; o < 64; o <<= 1) acc[h][e] += __shfl_xor(acc[h][e], o);
    z_run[h] = wave_sum_f32(z_run[h]);
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) wn[wave][h][(c * 8 + s) * 8 + e] = acc[h][c * 8 + e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      wm[wave][h] = m_run[h];
      wz[wave][h] = z_run[h];
    }
  }
  __syncthreads();
  for (int i = tid; i < nh * D; i += 256) {
    const int h = i / D, c = i - h * D;
    float m = wm[0][h];
    for (int w2 = 1; w2 < 4; ++w2) m = fmaxf(m, wm[w2][h]);
    double nv = 0.0, zz = 0.0;
    if (m != -INFINITY) {
      for (int w2 = 0; w2 < 4; ++w2) {
        const double f = exp((double)wm[w2][h] - (double)m);
        nv += f * (double)wn[w2][h][c];
        zz += f * (double)wz[w2][h];
      }
    }
    DensePartial<D>* part = (DensePartial<D>*)a.part +
                            ((((size_t)b * a.Hq + h0 + h) * a.n_q + qi) * a.chunks + blockIdx.x);
    part->nv[c] = nv;
    if (c == 0) {
      part->m = (double)m;
      part->z = zz;
    }
  }
}

// One wave per (batch, query head, query): merge the chunk partials. Lane c takes the maximum and
// sum of partials c, c + 64, ...; the wave reduces them and every lane keeps the weight
// exp(m_c - m) of its partials in LDS; then each lane sums its D / 64 output elements over all
// partials, eight partials' loads in flight at a time.
template <int D>
__global__ __launch_bounds__(64) void dense_combine_kernel(const void* partv, float* out, int64_t chunks, int64_t kpb,
                                                           int64_t n_q, int64_t q_pos0, int64_t n, int causal,
                                                           const float* gate, float gate_min) {
  constexpr int MAXP = 1024;  // partials merged per pass through the LDS weights
  __shared__ double fw[MAXP];
  const size_t row = blockIdx.x;  // (b*Hq + h)*n_q + qi
  if (gate && !(gate[row] >= gate_min)) return;
  const int64_t qi = (int64_t)(row % (size_t)n_q);
  const int64_t p = q_pos0 + qi;
  const int64_t vis_hi = causal ? p : n - 1;
  const int64_t used = vis_hi / kpb + 1;
  const DensePartial<D>* part = (const DensePartial<D>*)partv + row * (size_t)chunks;
  const int lane = threadIdx.x;
  double m = -INFINITY;
  for (int64_t c = lane; c < used; c += 64) m = fmax(m, part[c].m);
  m = wave_max_f64(m);
  constexpr int CPL = D / 64;
  double nv[CPL] = {};
  double z = 0.0;
  for (int64_t c0 = 0; c0 < used; c0 += MAXP) {
    const int cnt = (int)min((int64_t)MAXP, used - c0);
    for (int i = lane; i < cnt; i += 64) {
      const double mc = part[c0 + i].m;
      const double f = mc == -INFINITY ? 0.0 : exp(mc - m);
      fw[i] = f;
      z += f * part[c0 + i].z;
    }
    __syncthreads();
    int i = 0;
    for (; i + 8 <= cnt; i += 8) {
      double x[8][CPL];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < CPL; ++e) x[u][e] = part[c0 + i + u].nv[lane * CPL + e];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < CPL; ++e) nv[e] += fw[i + u] * x[u][e];
    }
    for (; i < cnt; ++i)
#pragma unroll
      for (int e = 0; e < CPL; ++e) nv[e] += fw[i] * part[c0 + i].nv[lane * CPL + e];
    __syncthreads();
  }
  z = wave_sum_f64(z);
#pragma unroll
  for (int e = 0; e < CPL; ++e) out[row * D + lane * CPL + e] = (float)(nv[e] / z);
}

template <int D, int GT, bool BF16>
static hipError_t launch_dense_t(const DenseArgs& da, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((dense_partial_kernel<D, GT, BF16>), grid, dim3(256), 0, s, da);
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t launch_dense_g(const DenseArgs& da, int GT, dim3 grid, hipStream_t s) {
  switch (GT) {
    case 1: return launch_dense_t<D, 1, BF16>(da, grid, s);
    case 2: return launch_dense_t<D, 2, BF16>(da, grid, s);
    default: return launch_dense_t<D, 4, BF16>(da, grid, s);
  }
}

template <int RB>
static hipError_t launch_stream_g(const DenseArgs& da, int GT, dim3 grid, hipStream_t s) {
  switch (GT) {
    case 1: hipLaunchKernelGGL((dense_stream_kernel<RB, 1>), grid, dim3(256), 0, s, da); break;
    case 2: hipLaunchKernelGGL((dense_stream_kernel<RB, 2>), grid, dim3(256), 0, s, da); break;
    default: hipLaunchKernelGGL((dense_stream_kernel<RB, 4>), grid, dim3(256), 0, s, da); break;
  }
  return hipGetLastError();
}

static int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  return cus;
}

hipError_t launch_dense(const DenseLaunch& L, hipStream_t stream) {
  DenseArgs da;
  da.q = (const unsigned char*)L.q;
  da.k = (const unsigned char*)L.k;
  da.v = (const unsigned char*)L.v;
  da.part = L.ws;
  da.n = L.n;
  da.n_q = L.n_q;
  da.q_pos0 = L.q_pos0;
  da.chunks = (L.n + DN_KEYS - 1) / DN_KEYS;
  da.Hq = L.Hq;
  da.Hkv = L.Hkv;
  da.G = L.G;
  da.causal = L.causal;
  da.scale = L.scale;
  da.gate = L.gate;
  da.gate_min = L.gate_min;
  // float64 accumulation (float32 inputs) needs more registers and LDS per head: fewer heads per block.
  int GT = L.G >= 4 ? 4 : L.G;
  if (!L.bf16) GT = L.d == 128 ? 1 : (L.G >= 2 ? 2 : 1);
  da.nslices = (L.G + GT - 1) / GT;
  // Only the blocks that hold visible keys of the last query are launched.
  const int64_t vis_hi_max = L.causal ? L.q_pos0 + L.n_q - 1 : L.n - 1;
  hipError_t e;
  if (L.bf16) {
    // runs per block: the largest count that still leaves two blocks per compute unit (the
    // partials fit the workspace sized for one run per block)
    const int64_t others = (int64_t)L.B * L.Hkv * L.n_q * da.nslices;
    int runs = 1;
    for (int rr = DS_MAX_RUNS; rr > 1; rr >>= 1)
      if ((vis_hi_max / (DS_KEYS_PER_RUN * (int64_t)rr) + 1) * others >= 2 * (int64_t)device_cus()) {
        runs = rr;
        break;
      }
    da.runs = runs;
    da.kpb = (int64_t)DS_KEYS_PER_RUN * runs;
    da.chunks = vis_hi_max / da.kpb + 1;
    const dim3 grid((unsigned)da.chunks, (unsigned)(L.B * L.Hkv), (unsigned)(L.n_q * da.nslices));
    e = L.d == 128 ? launch_stream_g<256>(da, GT, grid, stream) : launch_stream_g<128>(da, GT, grid, stream);
  } else {
    da.kpb = DN_KEYS;
    const dim3 grid((unsigned)(vis_hi_max / DN_KEYS + 1), (unsigned)(L.B * L.Hkv), (unsigned)(L.n_q * da.nslices));
    e = L.d == 128 ? launch_dense_g<128, false>(da, GT, grid, stream) : launch_dense_g<64, false>(da, GT, grid, stream);
  }
  if (e != hipSuccess) return e;
  const unsigned rows = (unsigned)((size_t)L.B * L.Hq * L.n_q);
  if (L.d == 128) {
    hipLaunchKernelGGL(dense_combine_kernel<128>, dim3(rows), dim3(64), 0, stream, L.ws, L.out, da.chunks, da.kpb,
                       L.n_q, L.q_pos0, L.n, L.causal, L.gate, L.gate_min);
  } else {
    hipLaunchKernelGGL(dense_combine_kernel<64>, dim3(rows), dim3(64), 0, stream, L.ws, L.out, da.chunks, da.kpb,
                       L.n_q, L.q_pos0, L.n, L.causal, L.gate, L.gate_min);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Read-bandwidth probe: every block streams 128 KiB runs with the key scan's load instruction
// (16-byte non-temporal loads, one per lane, fully coalesced) and folds them into one word. Of the
// shapes measured (8 to 32 loads per lane in flight, 1024 to 8192 blocks, grid-stride or one
// contiguous range per block), 32 loads per lane over 8192 blocks read fastest.
__global__ __launch_bounds__(256) void bw_probe_kernel(const uint4* buf, size_t n16, uint32_t* sink) {
  constexpr int U = 32;
  uint32_t x = 0;
  const size_t run = (size_t)256 * U;
  for (size_t base = (size_t)blockIdx.x * run; base < n16; base += (size_t)gridDim.x * run) {
    uint4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = base + (size_t)u * 256 + threadIdx.x;
      r[u] = i < n16 ? ntload16(buf + i) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  }
  x ^= __shfl_xor(x, 1);
  if ((threadIdx.x & 63) == 0 && x == 0x9E3779B9u) atomicXor(sink, x);  // keeps the loads live
}

hipError_t launch_bw_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  const size_t runs = (n16 + 8191) / 8192;
  const unsigned blocks = (unsigned)(runs < 8192 ? runs : 8192);
  hipLaunchKernelGGL(bw_probe_kernel, dim3(blocks), dim3(256), 0, stream, (const uint4*)buf, n16, sink);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Finite-input check: every thread tests 16-byte chunks (grid-stride) for an all-ones exponent
// field (NaN or infinity), plus the elements of a ragged tail; one atomicOr per wave that found one.
__global__ __launch_bounds__(256) void check_finite_kernel(const unsigned char* buf, size_t count, int bf16,
                                                           uint32_t* flag) {
  const size_t esize = bf16 ? 2 : 4;
  const size_t nchunk = count * esize / 16;
  bool bad = false;
  for (size_t c = (size_t)blockIdx.x * 256 + threadIdx.x; c < nchunk; c += (size_t)gridDim.x * 256) {
    const uint4 w = *(const uint4*)(buf + c * 16);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (bf16) {
        bad |= (ws[e] & 0x7F80u) == 0x7F80u;
        bad |= (ws[e] & 0x7F800000u) == 0x7F800000u;
      } else {
        bad |= (ws[e] & 0x7F800000u) == 0x7F800000u;
      }
    }
  }
  // elements past the last whole chunk
  const size_t done = nchunk * 16 / esize;
  for (size_t i = done + (size_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (size_t)gridDim.x * 256) {
    if (bf16) bad |= (((const uint16_t*)buf)[i] & 0x7F80u) == 0x7F80u;
    else bad |= (((const uint32_t*)buf)[i] & 0x7F800000u) == 0x7F800000u;
  }
  if (__ballot(bad) != 0ull && (threadIdx.x & 63) == 0) atomicOr(flag, 1u);
}

hipError_t launch_check_finite(const void* buf, size_t count, int bf16, uint32_t* flag, hipStream_t stream) {
  const size_t nchunk = count * (bf16 ? 2 : 4) / 16;
  size_t blocks = (nchunk + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(check_finite_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const unsigned char*)buf, count,
                     bf16, flag);
  return hipGetLastError();
}

}  // namespace topo
