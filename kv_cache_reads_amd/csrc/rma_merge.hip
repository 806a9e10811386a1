// Exact branch, retrieved-token subtraction, residual estimate and single
// normalisation ("Residual-Mass Accounting for Partial-KV Decoding": §3 Eq. 3-4
// and Eq. 11 for the exact terms over anchors, retrieved and generated tokens;
// §4.2 Eq. 9 for the subtraction; §4.3 Eq. 10 for the merge; App. C.1 for the
// clamp of the residual denominator).
//
// Grid (slices, units).  The per-head list of exact-support entries is
//   [sinks | tail | generated | retrieved (idx)]  (n_a + n_gen + K entries)
// and block s handles entries [s*sl, (s+1)*sl) of every head of its unit:
//   m_s = max s_i,  N_s = sum e^{s_i - m_s} v_i,  Z_s = sum e^{s_i - m_s},
//   for retrieved entries w_i = f.Phi_K[i]:  nuK_s = sum w_i v_i, ZK_s = sum w_i.
// The last block of a unit to finish (a completion counter in the workspace)
// combines the slices with a running-max rescale, forms phi(q)^T S for all G
// heads with fp32 MFMA (v_mfma_f32_16x16x4f32), subtracts, clamps and
// normalises once.
#include "rma_device.hpp"
#include "rma_internal.hpp"

#include <math.h>

namespace rma {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ float ld_elem(const T* p, size_t i);
template <>
__device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
template <>
__device__ __forceinline__ float ld_elem<float>(const float* p, size_t i) { return p[i]; }

template <typename KT, typename PT, int D>
__global__ void __launch_bounds__(256)
merge_kernel(const float* __restrict__ q, const float* __restrict__ phi_q, int G,
             const KT* __restrict__ kb, const KT* __restrict__ vb, int64_t ustride, int L,
             int n_sink, int n_tail, int n_gen, const int32_t* __restrict__ idx,
             const float* __restrict__ sel, int K, const PT* __restrict__ phik, int m, int L_mid,
             const float* __restrict__ S, const float* __restrict__ u_, uint32_t flags,
             float* __restrict__ y, float* __restrict__ stats, float* __restrict__ part,
             uint32_t* __restrict__ counters, int n_slices, int sl, float inv_sqrt_d) {
  constexpr int E = 16, LPT = D / E, CPL = D / kWave;  // columns per lane
  const int s = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const int n_a = n_sink + n_tail;
  const int T = n_a + n_gen + K;
  const int j0 = s * sl, j1 = min(T, j0 + sl);
  const int PF = 4 + 2 * D;
  const bool sub = (flags == RMA_MERGE_SUB) && K > 0;

  __shared__ float s_sc[1024];
  __shared__ int s_pos[1024];
  __shared__ float s_f[128];
  __shared__ float s_red[4][2 * D + 4];
  __shared__ float s_mx[4];
  __shared__ int s_last;

  const KT* kunit = kb + (size_t)u * ustride;
  const KT* vunit = vb + (size_t)u * ustride;

  for (int g = 0; g < G; ++g) {
    const int ug = u * G + g;
    if (sub && tid < m) s_f[tid] = phi_q[(size_t)ug * m + tid];
    for (int j = j0 + tid; j < j1; j += 256) {
      int pos;
      float sc = 0.f;
      if (j < n_sink) pos = j;
      else if (j < n_a) pos = L - n_tail + (j - n_sink);
      else if (j < n_a + n_gen) pos = L + (j - n_a);
      else {
        const int r = j - n_a - n_gen;
        // positions come from rma_decode_topk; clamped so a bad index cannot fault
        pos = min(max(idx[(size_t)ug * K + r], n_sink), n_sink + max(L_mid, 1) - 1);
        sc = sel[(size_t)ug * K + r];
      }
      s_pos[j - j0] = pos;
      s_sc[j - j0] = sc;
    }
    __syncthreads();
    // scores of anchors and generated tokens in this slice: LPT lanes per entry
    const int jc1 = min(j1, n_a + n_gen);
    {
      const int part = lane % LPT;
      float qr[E];
      const float* qg = q + (size_t)ug * D + part * E;
#pragma unroll
      for (int e = 0; e < E; ++e) qr[e] = qg[e];
      for (int base = j0; base < jc1; base += 256 / LPT) {
        const int j = base + tid / LPT;
        float a = 0.f;
        if (j < jc1) {
          float kv[E];
          load_row_f32<E>(kunit + (size_t)s_pos[j - j0] * D + part * E, kv);
#pragma unroll
          for (int e = 0; e < E; ++e) a = __fmaf_rn(qr[e], kv[e], a);
        }
        a = lane_group_sum<LPT>(a);
        if (j < jc1 && part == 0) s_sc[j - j0] = a * inv_sqrt_d;
      }
    }
    __syncthreads();
    // slice max
    float mx = -INFINITY;
    for (int j = tid; j < j1 - j0; j += 256) mx = fmaxf(mx, s_sc[j]);
    mx = wave_max(mx);
    if (lane == 0) s_mx[wave] = mx;
    __syncthreads();
    const float ms = fmaxf(fmaxf(s_mx[0], s_mx[1]), fmaxf(s_mx[2], s_mx[3]));
    // accumulate: wave w takes entries w, w+4, ...; lane owns columns lane + 64*c
    float N[CPL], NK[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) { N[c] = 0.f; NK[c] = 0.f; }
    float Z = 0.f, ZK = 0.f;
    for (int jj = wave; jj < j1 - j0; jj += 4) {
      const int pos = s_pos[jj];
      const float ew = __expf(s_sc[jj] - ms);
      float vv[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) vv[c] = ld_elem<KT>(vunit, (size_t)pos * D + lane + kWave * c);
#pragma unroll
      for (int c = 0; c < CPL; ++c) N[c] = __fmaf_rn(ew, vv[c], N[c]);
      Z += ew;
      if (sub && j0 + jj >= n_a + n_gen) {
        const PT* prow = phik + ((size_t)u * L_mid + (pos - n_sink)) * m;
        float p = 0.f;
        for (int f = lane; f < m; f += kWave) p = __fmaf_rn(s_f[f], ld_elem<PT>(prow, f), p);
        const float w = wave_sum(p);
#pragma unroll
        for (int c = 0; c < CPL; ++c) NK[c] = __fmaf_rn(w, vv[c], NK[c]);
        ZK += w;
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      s_red[wave][lane + kWave * c] = N[c];
      s_red[wave][D + lane + kWave * c] = NK[c];
    }
    if (lane == 0) { s_red[wave][2 * D] = Z; s_red[wave][2 * D + 1] = ZK; }
    __syncthreads();
    float* pp = part + ((size_t)u * n_slices + s) * G * PF + (size_t)g * PF;
    for (int i = tid; i < 2 * D + 2; i += 256) {
      const float v = s_red[0][i] + s_red[1][i] + s_red[2][i] + s_red[3][i];
      if (i < 2 * D) pp[4 + i] = v;
      else pp[1 + (i - 2 * D)] = v;
    }
    if (tid == 0) { pp[0] = ms; pp[3] = 0.f; }
    __syncthreads();
  }

  // ---- last block of the unit combines
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&counters[u], 1u) == (uint32_t)(n_slices - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  __shared__ float s_fs[8][128];   // phi(q)^T S per head
  __shared__ float s_uf[8];
  const bool resid = flags != RMA_MERGE_NO_RESIDUAL;
  const bool whole_mid = (flags == RMA_MERGE_SUB) && K == L_mid;
  if (resid && !whole_mid) {
    // fp32 MFMA 16x16x4: rows = heads (G <= 8, zero-padded), k = features, cols = d
    const float* Su = S + (size_t)u * m * D;
    const int row = lane & 15, kq = lane >> 4;
    for (int ct = wave; ct < D / 16; ct += 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int ks = 0; ks < m / 4; ++ks) {
        const int f = 4 * ks + kq;
        const float a = row < G ? phi_q[((size_t)u * G + row) * m + f] : 0.f;
        const float b = Su[(size_t)f * D + 16 * ct + row];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * kq + r;
        if (h < G) s_fs[h][16 * ct + row] = acc[r];
      }
    }
    // u^T f per head
    for (int g = wave; g < G; g += 4) {
      float p = 0.f;
      for (int f = lane; f < m; f += kWave) p = __fmaf_rn(u_[(size_t)u * m + f], phi_q[((size_t)u * G + g) * m + f], p);
      p = wave_sum(p);
      if (lane == 0) s_uf[g] = p;
    }
  }
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int ug = u * G + g;
    const float* pb = part + (size_t)u * n_slices * G * PF + (size_t)g * PF;
    float mstar = -INFINITY;
    for (int sidx = 0; sidx < n_slices; ++sidx) mstar = fmaxf(mstar, pb[(size_t)sidx * G * PF]);
    // per column: N_E and nuK
    float ZE = 0.f, ZKt = 0.f;
    for (int sidx = 0; sidx < n_slices; ++sidx) {
      const float* ps = pb + (size_t)sidx * G * PF;
      const float sc = ps[1] > 0.f ? __expf(ps[0] - mstar) : 0.f;
      ZE = __fmaf_rn(sc, ps[1], ZE);
      ZKt += ps[2];
    }
    float zr = 0.f;
    if (resid && !whole_mid) {
      zr = s_uf[g] - (sub ? ZKt : 0.f);
      zr = fmaxf(zr, 0.f);
    }
    const float lz = zr > 0.f ? __logf(zr) : -INFINITY;
    const float M = fmaxf(mstar, lz);
    const float a = __expf(mstar - M);
    const float bres = __expf(-M);
    const float den = a * ZE + bres * zr;
    for (int c = tid; c < D; c += 256) {
      float NE = 0.f, NKc = 0.f;
      for (int sidx = 0; sidx < n_slices; ++sidx) {
        const float* ps = pb + (size_t)sidx * G * PF;
        const float sc = ps[1] > 0.f ? __expf(ps[0] - mstar) : 0.f;
        NE = __fmaf_rn(sc, ps[4 + c], NE);
        NKc += ps[4 + D + c];
      }
      float nu = 0.f;
      if (resid && !whole_mid) nu = s_fs[g][c] - (sub ? NKc : 0.f);
      y[(size_t)ug * D + c] = (a * NE + bres * nu) / den;
    }
    if (stats != nullptr && tid == 0) {
      stats[(size_t)ug * 4 + 0] = mstar;
      stats[(size_t)ug * 4 + 1] = ZE;
      stats[(size_t)ug * 4 + 2] = zr;
      stats[(size_t)ug * 4 + 3] = ZKt;
    }
  }
  if (tid == 0) counters[u] = 0u;
}

template <typename KT, typename PT, int D>
hipError_t launch_merge_t(const MergePlan& pl, const float* q, const float* phi_q, int G,
                          const rma_kv& kv, const rma_span& sp, const int32_t* idx,
                          const float* sel, int K, const void* phi_k, int m, const float* S,
                          const float* u, uint32_t flags, float* y, float* stats, uint8_t* ws,
                          hipStream_t st) {
  const int L_mid = (int)(sp.L - sp.n_sink - sp.n_tail);
  hipLaunchKernelGGL((merge_kernel<KT, PT, D>), dim3(pl.n_slices, kv.n_units), dim3(256), 0, st, q,
                     phi_q, G, static_cast<const KT*>(kv.k), static_cast<const KT*>(kv.v),
                     kv.unit_stride, (int)sp.L, sp.n_sink, sp.n_tail, (int)sp.n_gen, idx, sel, K,
                     static_cast<const PT*>(phi_k), m, L_mid, S, u, flags, y, stats,
                     reinterpret_cast<float*>(ws + pl.off_part), reinterpret_cast<uint32_t*>(ws),
                     pl.n_slices, pl.sl, 1.0f / sqrtf((float)D));
  return hipGetLastError();
}

hipError_t launch_merge(const MergePlan& pl, const float* q, const float* phi_q, int G,
                        const rma_kv& kv, const rma_span& sp, const int32_t* idx,
                        const float* sel, int K, const void* phi_k, int phi_dtype, int m,
                        const float* S, const float* u, uint32_t flags, float* y, float* stats,
                        uint8_t* ws, hipStream_t st) {
#define RMA_MERGE_DISPATCH(KT, PT)                                                             \
  return kv.d == 64 ? launch_merge_t<KT, PT, 64>(pl, q, phi_q, G, kv, sp, idx, sel, K, phi_k, m, \
                                                 S, u, flags, y, stats, ws, st)                \
                    : launch_merge_t<KT, PT, 128>(pl, q, phi_q, G, kv, sp, idx, sel, K, phi_k, \
                                                  m, S, u, flags, y, stats, ws, st);
  if (kv.dtype == RMA_BF16) {
    if (phi_dtype == RMA_BF16) { RMA_MERGE_DISPATCH(uint16_t, uint16_t) }
    RMA_MERGE_DISPATCH(uint16_t, float)
  }
  if (phi_dtype == RMA_BF16) { RMA_MERGE_DISPATCH(float, uint16_t) }
  RMA_MERGE_DISPATCH(float, float)
#undef RMA_MERGE_DISPATCH
}

}  // namespace rma
