// Exact branch, retrieved-token subtraction, residual estimate and single
// normalisation ("Residual-Mass Accounting for Partial-KV Decoding": §3 Eq. 3-4
// and Eq. 11 for the exact terms over anchors, retrieved and generated tokens;
// §4.2 Eq. 9 for the subtraction; §4.3 Eq. 10 for the merge; App. C.1 for the
// clamp of the residual denominator).
//
// One block per (unit, query head).  The head's exact-support entries
//   [sinks | tail | generated | retrieved (idx)]   (n_a + n_gen + K entries)
// are staged in LDS chunk by chunk; eight lanes share an entry (its V row, and
// for a retrieved token its phi_k row), accumulating with a running max m*:
//   N_E = sum e^{s_i - m*} v_i,  Z_E = sum e^{s_i - m*},
//   w_i = f.Phi_K[i],  nuK = sum_{K(q)} w_i v_i,  ZK = sum_{K(q)} w_i.
// phi(q)^T S comes from fp32 MFMA (v_mfma_f32_16x16x4f32) over the unit's query
// heads; then the subtraction, the clamp and one normalisation.
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

template <typename KT, typename PT, int D, int M>
__global__ void __launch_bounds__(kMergeThreads)
merge_kernel(const float* __restrict__ q, const float* __restrict__ phi_q, int G,
             const KT* __restrict__ kb, const KT* __restrict__ vb, int64_t ustride, int L,
             int n_sink, int n_tail, int n_gen, const int32_t* __restrict__ idx,
             const float* __restrict__ sel, int K, const PT* __restrict__ phik, int L_mid,
             const float* __restrict__ S, const float* __restrict__ u_, uint32_t flags,
             float* __restrict__ y, float* __restrict__ stats, float inv_sqrt_d) {
  constexpr int NT = kMergeThreads, NW = NT / kWave;
  constexpr int LPE = 8;            // lanes per entry in the accumulation
  constexpr int EPW = kWave / LPE;  // entries per wave pass
  constexpr int CPL = D / LPE;      // value columns per lane
  constexpr int FPL = M / LPE;      // phi features per lane
  constexpr int LPT = D / 16;       // lanes per anchor dot
  constexpr int CH = kMergeChunk;   // entries staged in LDS at a time
  const int ug = blockIdx.x, u = ug / G, g = ug - u * G, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int part = lane & (LPE - 1), slot = lane / LPE;
  const int n_a = n_sink + n_tail, n_ex = n_a + n_gen;
  const int T = n_ex + K;
  const bool sub = (flags == RMA_MERGE_SUB) && K > 0;

  constexpr int RW = 2 * CPL + 2;  // partial floats per lane: N, NK columns, Z, ZK
  __shared__ int s_pos[CH];
  __shared__ float s_sc[CH];
  __shared__ float s_red[NW][4][LPE][RW];
  __shared__ float s_wm[NW];
  __shared__ float s_fs[D];
  __shared__ float s_uf;

  const KT* kunit = kb + (size_t)u * ustride;
  const KT* vunit = vb + (size_t)u * ustride;
  const float* qg = q + (size_t)ug * D;
  const int32_t* ig = idx + (size_t)ug * K;
  const float* sg = sel + (size_t)ug * K;

  float fr[FPL];
#pragma unroll
  for (int i = 0; i < FPL; ++i) fr[i] = sub ? phi_q[(size_t)ug * M + part * FPL + i] : 0.f;
  float N[CPL], NK[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) { N[c] = 0.f; NK[c] = 0.f; }
  float Z = 0.f, ZK = 0.f, mrun = -INFINITY;

  // ---- phi(q)^T S and u^T f for this unit's heads (fp32 MFMA 16x16x4; rows =
  //      the G query heads zero-padded to 16, k = features, columns = d)
  const bool resid = flags != RMA_MERGE_NO_RESIDUAL;
  const bool whole_mid = (flags == RMA_MERGE_SUB) && K == L_mid;
  if (resid && !whole_mid) {
    const float* Su = S + (size_t)u * M * D;
    const int row = lane & 15, kq = lane >> 4;
    for (int ct = wave; ct < D / 16; ct += NW) {
      float av[M / 4], bv[M / 4];
#pragma unroll
      for (int ks = 0; ks < M / 4; ++ks) {
        const int f = 4 * ks + kq;
        av[ks] = row < G ? phi_q[((size_t)u * G + row) * M + f] : 0.f;
        bv[ks] = Su[(size_t)f * D + 16 * ct + row];
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < M / 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[ks], bv[ks], acc, 0, 0, 0);
      // lane holds rows 4*kq + r of column 16*ct + row; keep this block's head
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * kq + r == g) s_fs[16 * ct + row] = acc[r];
    }
    if (wave == NW - 1) {
      float p = 0.f;
      for (int f = lane; f < M; f += kWave) p = __fmaf_rn(u_[(size_t)u * M + f], phi_q[(size_t)ug * M + f], p);
      p = wave_sum_dpp(p);
      if (lane == 0) s_uf = p;
    }
  }

  // ---- exact-support entries [anchors | generated | retrieved], CH at a time
  for (int c0 = 0; c0 < T; c0 += CH) {
    const int cnt = min(CH, T - c0);
    __syncthreads();
    for (int jj = tid; jj < cnt; jj += NT) {
      const int j = c0 + jj;
      int pos;
      float sc = 0.f;
      if (j < n_sink) pos = j;
      else if (j < n_a) pos = L - n_tail + (j - n_sink);
      else if (j < n_ex) pos = L + (j - n_a);
      else {
        // positions come from rma_decode_topk; clamped so a bad index cannot fault
        pos = min(max(ig[j - n_ex], n_sink), n_sink + max(L_mid, 1) - 1);
        sc = sg[j - n_ex];
      }
      s_pos[jj] = pos;
      s_sc[jj] = sc;
    }
    __syncthreads();
    const int nc = max(0, min(c0 + cnt, n_ex) - c0);  // anchors / generated in this chunk
    if (nc > 0) {
      const int lp = lane % LPT;
      float qr[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) qr[e] = qg[lp * 16 + e];
      for (int base = 0; base < nc; base += NT / LPT) {
        const int jj = base + tid / LPT;
        float a = 0.f;
        if (jj < nc) {
          float kv[16];
          load_row_f32<16>(kunit + (size_t)s_pos[jj] * D + lp * 16, kv);
#pragma unroll
          for (int e = 0; e < 16; ++e) a = __fmaf_rn(qr[e], kv[e], a);
        }
        a = lane_group_sum<LPT>(a);
        if (jj < nc && lp == 0) s_sc[jj] = a * inv_sqrt_d;
      }
      __syncthreads();
    }
    // running max over the chunk
    float mx = -INFINITY;
    for (int jj = tid; jj < cnt; jj += NT) mx = fmaxf(mx, s_sc[jj]);
    mx = wave_max_dpp(mx);
    if (lane == 0) s_wm[wave] = mx;
    __syncthreads();
    mx = s_wm[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) mx = fmaxf(mx, s_wm[w]);
    const float mnew = fmaxf(mrun, mx);
    if (mnew > mrun) {
      const float r = __expf(mrun - mnew);   // 0 for the first chunk
#pragma unroll
      for (int c = 0; c < CPL; ++c) N[c] *= r;
      Z *= r;
      mrun = mnew;
    }
    // accumulate: 8 lanes per entry, EPW entries per wave pass
#pragma unroll 2
    for (int jb = wave * EPW; jb < cnt; jb += NW * EPW) {
      const int jj = jb + slot;
      const bool ok = jj < cnt;
      const int pos = ok ? s_pos[jj] : n_sink;
      float vv[CPL];
      if (ok) {
        load_row_f32<CPL>(vunit + (size_t)pos * D + part * CPL, vv);
      } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) vv[c] = 0.f;
      }
      const float ew = ok ? __expf(s_sc[jj] - mrun) : 0.f;
      float w = 0.f;
      if (sub && ok && c0 + jj >= n_ex) {
        float ph[FPL];
        load_row_f32<FPL>(phik + ((size_t)u * L_mid + (pos - n_sink)) * M + part * FPL, ph);
#pragma unroll
        for (int i = 0; i < FPL; ++i) w = __fmaf_rn(fr[i], ph[i], w);
      }
      w = lane_group_sum<LPE>(w);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        N[c] = __fmaf_rn(ew, vv[c], N[c]);
        NK[c] = __fmaf_rn(w, vv[c], NK[c]);
      }
      if (part == 0) { Z += ew; ZK += w; }
    }
  }
  // ---- sum the entry slots: slots 2r and 2r+1 share row r (DPP row_ror:8),
  //      then the four rows of every wave through LDS
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    N[c] += dpp_f<0x128>(N[c]);
    NK[c] += dpp_f<0x128>(NK[c]);
  }
  Z += dpp_f<0x128>(Z);
  ZK += dpp_f<0x128>(ZK);
  if ((lane & 8) == 0) {
    float* dst = s_red[wave][lane >> 4][part];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      dst[c] = N[c];
      dst[CPL + c] = NK[c];
    }
    dst[2 * CPL] = Z;
    dst[2 * CPL + 1] = ZK;
  }
  __syncthreads();
  float ZE = 0.f, ZKt = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ZE += s_red[w][r][0][2 * CPL];
      ZKt += s_red[w][r][0][2 * CPL + 1];
    }
  float zr = 0.f;
  if (resid && !whole_mid) zr = fmaxf(s_uf - (sub ? ZKt : 0.f), 0.f);
  // y = (N_E + e^{-m*} nu) / (Z_E + e^{-m*} Z_R), scaled by e^{m* - Mx} with
  // Mx = max(m*, log Z_R) so that neither term overflows
  const float lz = zr > 0.f ? __logf(zr) : -INFINITY;
  const float Mx = fmaxf(mrun, lz);
  const float a = __expf(mrun - Mx);
  const float bres = __expf(-Mx);
  const float den = a * ZE + bres * zr;
  for (int col = tid; col < D; col += NT) {
    const int pp = col / CPL, c = col - pp * CPL;
    float NE = 0.f, NKc = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        NE += s_red[w][r][pp][c];
        NKc += s_red[w][r][pp][CPL + c];
      }
    float nu = 0.f;
    if (resid && !whole_mid) nu = s_fs[col] - (sub ? NKc : 0.f);
    y[(size_t)ug * D + col] = (a * NE + bres * nu) / den;
  }
  if (stats != nullptr && tid == 0) {
    stats[(size_t)ug * 4 + 0] = mrun;
    stats[(size_t)ug * 4 + 1] = ZE;
    stats[(size_t)ug * 4 + 2] = zr;
    stats[(size_t)ug * 4 + 3] = ZKt;
  }
}

template <typename KT, typename PT, int D>
hipError_t launch_merge_t(const MergePlan& pl, const float* q, const float* phi_q, int G,
                          const rma_kv& kv, const rma_span& sp, const int32_t* idx,
                          const float* sel, int K, const void* phi_k, int m, const float* S,
                          const float* u, uint32_t flags, float* y, float* stats, uint8_t* ws,
                          hipStream_t st) {
  const int L_mid = (int)(sp.L - sp.n_sink - sp.n_tail);
  auto kern = m == 64 ? merge_kernel<KT, PT, D, 64> : merge_kernel<KT, PT, D, 128>;
  (void)pl;
  (void)ws;
  hipLaunchKernelGGL(kern, dim3(kv.n_units * G), dim3(kMergeThreads), 0, st, q, phi_q, G,
                     static_cast<const KT*>(kv.k), static_cast<const KT*>(kv.v), kv.unit_stride,
                     (int)sp.L, sp.n_sink, sp.n_tail, (int)sp.n_gen, idx, sel, K,
                     static_cast<const PT*>(phi_k), L_mid, S, u, flags, y, stats,
                     1.0f / sqrtf((float)D));
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) trace_kernel(st, "merge_kernel");
  return e;
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
