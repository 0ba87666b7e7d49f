// Dense softmax attention over every visible key on gfx950: the full-attention "pillar" layers
// that the zh page of "The Condensate Theorem: Transformers are O(n), Not O(n^2)" keeps in a few
// layers (technical summary §3), and the comparator of the exactness claim (technical summary
// §2). Split over the keys (flash-decoding): each block folds a run of 2048 keys into a partial
// (max, sum of weights, weighted V sum) per query head with an online softmax; a second kernel
// merges the partials. K and V are each read once per (batch, kv head) for all G query heads.
// bf16 inputs use float32 scores and accumulation; float32 inputs use float64 for both.
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
  int32_t Hq, Hkv, G, causal, nslices;
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

// One wave per (batch, query head, query): merge the chunk partials.
template <int D>
__global__ __launch_bounds__(64) void dense_combine_kernel(const void* partv, float* out, int64_t chunks,
                                                           int64_t n_q, int64_t q_pos0, int64_t n, int causal,
                                                           const float* gate, float gate_min) {
  const size_t row = blockIdx.x;  // (b*Hq + h)*n_q + qi
  if (gate && !(gate[row] >= gate_min)) return;
  const int64_t qi = (int64_t)(row % (size_t)n_q);
  const int64_t p = q_pos0 + qi;
  const int64_t vis_hi = causal ? p : n - 1;
  const int64_t used = vis_hi / DN_KEYS + 1;
  const DensePartial<D>* part = (const DensePartial<D>*)partv + row * (size_t)chunks;
  const int lane = threadIdx.x;
  double m = -INFINITY;
  for (int64_t c = 0; c < used; ++c) m = fmax(m, part[c].m);
  constexpr int CPL = D / 64;
  double nv[CPL] = {};
  double z = 0.0;
  for (int64_t c = 0; c < used; ++c) {
    if (part[c].m == -INFINITY) continue;
    const double f = exp(part[c].m - m);
    z += f * part[c].z;
#pragma unroll
    for (int e = 0; e < CPL; ++e) nv[e] += f * part[c].nv[lane * CPL + e];
  }
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
  // Only the chunks that hold visible keys of the last query are launched.
  const int64_t vis_hi_max = L.causal ? L.q_pos0 + L.n_q - 1 : L.n - 1;
  dim3 grid((unsigned)(vis_hi_max / DN_KEYS + 1), (unsigned)(L.B * L.Hkv), (unsigned)(L.n_q * da.nslices));
  hipError_t e;
  if (L.bf16) {
    e = L.d == 128 ? launch_dense_g<128, true>(da, GT, grid, stream) : launch_dense_g<64, true>(da, GT, grid, stream);
  } else {
    e = L.d == 128 ? launch_dense_g<128, false>(da, GT, grid, stream) : launch_dense_g<64, false>(da, GT, grid, stream);
  }
  if (e != hipSuccess) return e;
  const unsigned rows = (unsigned)((size_t)L.B * L.Hq * L.n_q);
  if (L.d == 128) {
    hipLaunchKernelGGL(dense_combine_kernel<128>, dim3(rows), dim3(64), 0, stream, L.ws, L.out, da.chunks, L.n_q,
                       L.q_pos0, L.n, L.causal, L.gate, L.gate_min);
  } else {
    hipLaunchKernelGGL(dense_combine_kernel<64>, dim3(rows), dim3(64), 0, stream, L.ws, L.out, da.chunks, L.n_q,
                       L.q_pos0, L.n, L.causal, L.gate, L.gate_min);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Read-bandwidth probe: every block streams 64 KiB runs with the key scan's load instruction
// (16-byte non-temporal loads, one per lane, fully coalesced) and folds them into one word.
__global__ __launch_bounds__(256) void bw_probe_kernel(const uint4* buf, size_t n16, uint32_t* sink) {
  constexpr int U = 16;
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
  const size_t runs = (n16 + 4095) / 4096;
  const unsigned blocks = (unsigned)(runs < 2048 ? runs : 2048);
  hipLaunchKernelGGL(bw_probe_kernel, dim3(blocks), dim3(256), 0, stream, (const uint4*)buf, n16, sink);
  return hipGetLastError();
}

}  // namespace topo
