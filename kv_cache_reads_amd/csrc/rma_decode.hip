// Fused decode of one query head: the exact Top-K selection and the merge in
// one block ("Residual-Mass Accounting for Partial-KV Decoding": §1 and §3
// Eq. 3 for the exhaustive Top-K; §3 Eq. 3-4 and Eq. 11 for the exact terms
// over anchors, retrieved and generated tokens; §4.2 Eq. 9 for the
// subtraction; §4.3 Eq. 10 for the single normalisation; App. C.1 for the
// clamp of the residual denominator).
//
// rma_decode runs the scan of rma_decode_topk, then this kernel, grid U * G.
// A block first issues every load it will need before the selection's result:
// the chunk reports of its head (HeadSelect::load), then the query, the
// feature map's operands (or the given features), S and u, and the first rows
// of the anchors and generated tokens.  While the selection's reports are the
// only loads it waits for, the others arrive; then, in order:
//   1. f = phi_q(q) into LDS; phi(q)^T S per feature block and u^T f;
//   2. the exact terms of the anchors and generated tokens (eight lanes per
//      entry, a running max per 8-lane group);
//   3. the selection (rma_select.hpp): the K positions, ascending, and their
//      scaled fp32 scores into an LDS list (and to idx / sel when asked);
//   4. the retrieved tokens from that list: their V and phi_k rows are
//      gathered with every load of a batch issued before the first is used;
//      e^{s - m} v, w = f.phi_k and w v accumulate in the same groups;
//   5. the groups and waves combine with max rescaling in a fixed order, the
//      subtraction, the clamp and one normalisation.
// Steps 2 and 4 are the merge kernel's gathers; the arithmetic and its order
// within a group are the same, only the source of the retrieved entries
// differs (the LDS list instead of idx / sel in memory).
#include "rma_select.hpp"

#include <math.h>

#include <type_traits>

namespace rma {

template <typename KT, typename PT, int D, int M, int NT>
__global__ void __launch_bounds__(NT)
decode_fused_kernel(const float* __restrict__ q, int G, const KT* __restrict__ kb,
                    const KT* __restrict__ vb, int64_t ustride, int L, int n_sink, int n_tail,
                    int n_gen, int L_mid, int ch, int n_chunks, int r_cap, int K, int e_max,
                    const float4* __restrict__ hpw, const float2* __restrict__ ent,
                    const int2* __restrict__ meta, int32_t* __restrict__ idx_out,
                    float* __restrict__ sc_out, const float* __restrict__ phi_q,
                    const float* __restrict__ Wq, const float* __restrict__ bq, int P,
                    const PT* __restrict__ phik, const float* __restrict__ S,
                    const float* __restrict__ u_, uint32_t flags, float* __restrict__ y,
                    float* __restrict__ stats, float inv_sqrt_d) {
  constexpr int NW = NT / kWave;
  constexpr int LPE = 8;            // lanes per entry
  constexpr int NGR = NT / LPE;     // entry groups
  constexpr int CPL = D / LPE;      // value columns per lane
  constexpr int FPL = M / LPE;      // phi features per lane
  // retrieved entries per group whose row loads are in flight together: as in
  // the merge kernel, halved in 1024-thread blocks (128 VGPRs per lane; 128
  // groups x 4 entries already keep 512 entries in flight)
  constexpr int B0 = sizeof(KT) == 4 ? 2 : sizeof(PT) == 4 ? (D == 128 ? 2 : 4) : D == 128 ? 4 : 8;
  constexpr int B = NT == 1024 ? (B0 > 1 ? B0 / 2 : 1) : B0;
  constexpr int BX = 2;             // exactly scored entries per group per batch
  extern __shared__ __align__(16) float dyn[];
  float* es = dyn;                                        // selection: union scores
  int* ep = reinterpret_cast<int*>(dyn + e_max);          // selection: union positions
  int* lpos = reinterpret_cast<int*>(dyn + 2 * e_max);    // the K selected positions
  float* lsc = dyn + 2 * e_max + K;                       // and their scaled scores

  const int ug = blockIdx.x, u = ug / G, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int part = lane & (LPE - 1), grp = tid / LPE;
  const int n_a = n_sink + n_tail, n_ex = n_a + n_gen;
  // the subtraction runs only when part of the mid-region stays unretrieved
  const bool sub = (flags == RMA_MERGE_SUB) && K > 0 && K < L_mid;
  const bool resid = flags != RMA_MERGE_NO_RESIDUAL;
  const bool whole_mid = (flags == RMA_MERGE_SUB) && K == L_mid;
  const bool rs = resid && !whole_mid;   // phi(q)^T S and u^T f are needed

  __shared__ float s_wn[NW][D], s_wk[NW][D];
  __shared__ float s_wm[NW], s_wz[NW], s_wzk[NW];
  __shared__ float s_part[NT / D][D];
  __shared__ float s_uf;
  __shared__ float s_f[M];          // f = phi_q(q) of this head

  const KT* kunit = kb + (size_t)u * ustride;
  const KT* vunit = vb + (size_t)u * ustride;
  const float* qg = q + (size_t)ug * D;

  // ---- 1. the selection's loads (this kernel runs only with K >= 1)
  HeadSelect<KT, D, NT> sel;
  sel.ug = ug;
  sel.qg = qg;
  sel.mt = meta + (size_t)ug * n_chunks;
  sel.en = ent + (size_t)ug * n_chunks * r_cap;
  sel.kunit = kunit;
  sel.n_sink = n_sink;
  sel.L_mid = L_mid;
  sel.ch = ch;
  sel.n_chunks = n_chunks;
  sel.r_cap = r_cap;
  sel.K = K;
  sel.e_max = e_max;
  sel.inv_sqrt_d = inv_sqrt_d;
  sel.load(hpw);

  // ---- 2. the merge's loads: f's operands (or the given features), q, S, u
  constexpr int TPF = NT / M, EPT = D / TPF;     // threads per feature, elements each
  const int fi = tid / TPF, fpart = tid % TPF;
  const bool fcomp = resid && Wq != nullptr;
  float wq[EPT], xq[EPT], fb0;
  {
    const int pset = u % P;
    const float* wr = fcomp ? Wq + ((size_t)pset * M + fi) * D + fpart * EPT : qg;
    const float* qs = qg + fpart * EPT;
#pragma unroll
    for (int i = 0; i < EPT; i += 4) {
      const float4 w4 = *reinterpret_cast<const float4*>(wr + i);
      const float4 x4 = *reinterpret_cast<const float4*>(qs + i);
      wq[i] = w4.x; wq[i + 1] = w4.y; wq[i + 2] = w4.z; wq[i + 3] = w4.w;
      xq[i] = x4.x; xq[i + 1] = x4.y; xq[i + 2] = x4.z; xq[i + 3] = x4.w;
    }
    fb0 = fcomp ? bq[(size_t)pset * M + fi]
                : (resid && phi_q != nullptr ? phi_q[(size_t)ug * M + (tid % M)] : 0.f);
  }
  float qr[CPL];
#pragma unroll
  for (int i = 0; i < CPL; i += 4) {
    const float4 t = *reinterpret_cast<const float4*>(qg + part * CPL + i);
    qr[i] = t.x; qr[i + 1] = t.y; qr[i + 2] = t.z; qr[i + 3] = t.w;
  }
  // phi(q)^T S: thread (column scol, feature block fb) holds its FPB elements of
  // S (coalesced along the columns); without a residual the loads read q
  constexpr int FB = NT / D;          // feature blocks
  constexpr int FPB = M / FB;         // features per block
  static_assert(FB >= 1 && M % FB == 0, "whole feature blocks");
  const int scol = tid % D, fb = tid / D;
  float sv[FPB];
  {
    const float* Sp = rs ? S + (size_t)u * M * D + (size_t)fb * FPB * D + scol : qg;
    const size_t sst = rs ? D : 0;
#pragma unroll
    for (int i = 0; i < FPB; ++i) sv[i] = Sp[sst * i];
  }
  constexpr int UPL = (M + kWave - 1) / kWave;   // u^T f terms per lane (last wave)
  float uu[UPL];
#pragma unroll
  for (int i = 0; i < UPL; ++i) uu[i] = rs ? u_[(size_t)u * M + min(lane + kWave * i, M - 1)] : 0.f;

  // position of exactly scored entry j: sinks, tail, generated tokens
  auto ex_pos = [&](int j) {
    return j < n_sink ? j : (j < n_a ? L - n_tail + (j - n_sink) : L + (j - n_a));
  };
  // the first batch of exactly scored rows (the rest, if any, after it)
  RawPiece<KT, CPL> xv[BX], xk[BX];
  const int xlo = 0, xhi = n_ex;
  auto load_ex = [&](int jb) {
#pragma unroll
    for (int e = 0; e < BX; ++e) {
      const int jj = jb + e * NGR;
      const int pos = ex_pos(jj < xhi ? jj : xlo);
      xv[e].load(vunit + (size_t)pos * D + part * CPL);
      xk[e].load(kunit + (size_t)pos * D + part * CPL);
    }
  };
  if (n_ex > 0) load_ex(grp);

  // ---- f = phi_q(q) into LDS, then phi(q)^T S and u^T f
  if (fcomp) {
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < EPT; ++i) z = __fmaf_rn(wq[i], xq[i], z);
    z = lane_group_sum<TPF>(z);
    if (fpart == 0) s_f[fi] = phi_elu1(z + fb0);
  } else if (resid && tid < M) {
    s_f[tid] = fb0;
  }
  __syncthreads();
  if (rs) {
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < FPB; ++i) p = __fmaf_rn(s_f[fb * FPB + i], sv[i], p);
    s_part[fb][scol] = p;
    if (wave == NW - 1) {
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < UPL; ++i)
        if (lane + kWave * i < M) t = __fmaf_rn(uu[i], s_f[lane + kWave * i], t);
      t = wave_sum_dpp(t);
      if (lane == 0) s_uf = t;
    }
  }

  // the group's running sums: N = sum e^{s - m} v, Z = sum e^{s - m} over the
  // exact support; NK = sum w v, ZK = sum w over the retrieved entries (those
  // two start after the selection, so they are not live across it)
  float N[CPL], NK[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) N[c] = 0.f;
  float Z = 0.f, ZK = 0.f, mrun = -INFINITY;
  auto add_exp = [&](float s, const float (&vv)[CPL]) {
    if (s > mrun) {
      const float r = __expf(mrun - s);  // 0 while nothing is accumulated
#pragma unroll
      for (int c = 0; c < CPL; ++c) N[c] *= r;
      Z *= r;
      mrun = s;
    }
    const float ew = __expf(s - mrun);
#pragma unroll
    for (int c = 0; c < CPL; ++c) N[c] = __fmaf_rn(ew, vv[c], N[c]);
    Z += ew;
  };

  // ---- 2. exactly scored entries (anchors, generated tokens)
  for (int jb = grp; jb < n_ex; jb += NGR * BX) {
    if (jb != grp) load_ex(jb);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < BX; ++e) {
      float kv[CPL], vv[CPL];
      xk[e].unpack(kv);
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) a = __fmaf_rn(qr[i], kv[i], a);
      a = lane_group_sum<LPE>(a);
      if (jb + e * NGR < xhi) {  // uniform within the group
        xv[e].unpack(vv);
        add_exp(a * inv_sqrt_d, vv);
      }
    }
  }

  // ---- 3. the selection into the LDS list
  {
    SelOut out;
    out.lpos = lpos;
    out.lsc = lsc;
    if (idx_out != nullptr) {
      out.io = idx_out + (size_t)ug * K;
      out.so = sc_out + (size_t)ug * K;
    }
    sel.run(es, ep, out);
  }
  __syncthreads();   // the list (and s_part, s_uf) complete

  // ---- 4. retrieved entries from the list
#pragma unroll
  for (int c = 0; c < CPL; ++c) NK[c] = 0.f;
  float fr[FPL];
#pragma unroll
  for (int i = 0; i < FPL; ++i) fr[i] = sub ? s_f[part * FPL + i] : 0.f;
  for (int jb = grp; jb < K; jb += NGR * B) {
    RawPiece<KT, CPL> vr[B];
    RawPiece<PT, FPL> pr[B];
    float scs[B];
#pragma unroll
    for (int e = 0; e < B; ++e) {
      const int jj = jb + e * NGR;
      const int jc = jj < K ? jj : jb;
      const int pos = min(max(lpos[jc], n_sink), n_sink + max(L_mid, 1) - 1);
      scs[e] = lsc[jc];
      vr[e].load(vunit + (size_t)pos * D + part * CPL);
      if (sub) pr[e].load(phik + ((size_t)u * L_mid + (pos - n_sink)) * M + part * FPL);
      else pr[e].zero();
    }
    __builtin_amdgcn_sched_barrier(0);   // every load issued before any use
#pragma unroll
    for (int e = 0; e < B; ++e) {
      float ph[FPL], vv[CPL];
      pr[e].unpack(ph);
      float w = 0.f;
#pragma unroll
      for (int i = 0; i < FPL; ++i) w = __fmaf_rn(fr[i], ph[i], w);
      w = lane_group_sum<LPE>(w);
      if (jb + e * NGR < K) {  // uniform within the group
        vr[e].unpack(vv);
        add_exp(scs[e], vv);
#pragma unroll
        for (int c = 0; c < CPL; ++c) NK[c] = __fmaf_rn(w, vv[c], NK[c]);
        ZK += w;
      }
    }
  }

  // ---- 5. combine the eight groups of each wave (lanes l, l^8, l^16, l^32 hold
  //      the same columns), then the waves through LDS, rescaling to the larger max
#pragma unroll
  for (int sh = LPE; sh < kWave; sh <<= 1) {
    const float mo = __shfl_xor(mrun, sh, kWave);
    const float mn = fmaxf(mrun, mo);
    const float ra = mrun == -INFINITY ? 0.f : __expf(mrun - mn);
    const float rb = mo == -INFINITY ? 0.f : __expf(mo - mn);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      N[c] = ra * N[c] + rb * __shfl_xor(N[c], sh, kWave);
      NK[c] += __shfl_xor(NK[c], sh, kWave);
    }
    Z = ra * Z + rb * __shfl_xor(Z, sh, kWave);
    ZK += __shfl_xor(ZK, sh, kWave);
    mrun = mn;
  }
  if (lane < LPE) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      s_wn[wave][part * CPL + c] = N[c];
      s_wk[wave][part * CPL + c] = NK[c];
    }
    if (lane == 0) {
      s_wm[wave] = mrun;
      s_wz[wave] = Z;
      s_wzk[wave] = ZK;
    }
  }
  __syncthreads();
  float ms = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) ms = fmaxf(ms, s_wm[w]);
  float sw[NW];
  float ZE = 0.f, ZKt = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    sw[w] = s_wm[w] == -INFINITY ? 0.f : __expf(s_wm[w] - ms);
    ZE += sw[w] * s_wz[w];
    ZKt += s_wzk[w];
  }
  const float uf = rs ? s_uf : 0.f;
  float zr = 0.f;
  if (rs) zr = fmaxf(uf - (sub ? ZKt : 0.f), 0.f);
  // y = (N_E + e^{-m*} nu) / (Z_E + e^{-m*} Z_R), scaled by e^{m* - Mx} with
  // Mx = max(m*, log Z_R) so that neither term overflows
  const float lz = zr > 0.f ? __logf(zr) : -INFINITY;
  const float Mx = fmaxf(ms, lz);
  const float a = __expf(ms - Mx);
  const float bres = __expf(-Mx);
  const float den = a * ZE + bres * zr;
  for (int col = tid; col < D; col += NT) {
    float NE = 0.f, NKc = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      NE += sw[w] * s_wn[w][col];
      NKc += s_wk[w][col];
    }
    float nu = 0.f;
    if (rs) {
      float fs = 0.f;
#pragma unroll
      for (int k = 0; k < FB; ++k) fs += s_part[k][col];
      nu = fs - (sub ? NKc : 0.f);
    }
    y[(size_t)ug * D + col] = (a * NE + bres * nu) / den;
  }
  if (stats != nullptr && tid == 0) {
    stats[(size_t)ug * 4 + 0] = ms;
    stats[(size_t)ug * 4 + 1] = ZE;
    stats[(size_t)ug * 4 + 2] = zr;
    stats[(size_t)ug * 4 + 3] = ZKt;
  }
}

// ====================================================================== launch
namespace {

template <typename KT, typename PT, int D, int M, int NT>
hipError_t launch_fused_nt(const DecodePlan& pl, const float* q, int G, const rma_kv& kv,
                           const rma_span& sp, int K, int32_t* idx, float* sel,
                           const float* phi_q, const float* Wq, const float* bq, int P,
                           const void* phi_k, const float* S, const float* u, uint32_t flags,
                           float* y, float* stats, uint8_t* ws, hipStream_t st) {
  const TopkPlan& tp = pl.topk;
  const int L_mid = (int)(sp.L - sp.n_sink - sp.n_tail);
  auto kern = decode_fused_kernel<KT, PT, D, M, NT>;
  const size_t lds = (size_t)(2 * pl.e_max + 2 * K) * 4 + 16;
  // the plan checked the fit; a launch that would not fit is refused here too
  if (lds + kernel_static_lds<&decode_fused_kernel<KT, PT, D, M, NT>>() > device_info().lds_per_block)
    return hipErrorInvalidConfiguration;
  return launch_kernel("decode_fused_kernel", kern, dim3(kv.n_units * G), dim3(NT), (uint32_t)lds, st, q,
                       G, static_cast<const KT*>(kv.k), static_cast<const KT*>(kv.v), kv.unit_stride,
                       (int)sp.L, sp.n_sink, sp.n_tail, (int)sp.n_gen, L_mid, tp.ch, tp.n_chunks,
                       tp.r_cap, K, pl.e_max, reinterpret_cast<const float4*>(ws + tp.off_hp),
                       reinterpret_cast<const float2*>(ws + tp.off_ent),
                       reinterpret_cast<const int2*>(ws + tp.off_meta), idx, sel, phi_q, Wq, bq, P,
                       static_cast<const PT*>(phi_k), S, u, flags, y, stats, 1.0f / sqrtf((float)D));
}

template <typename KT, typename PT, int D>
hipError_t launch_fused_t(const DecodePlan& pl, const float* q, int G, const rma_kv& kv,
                          const rma_span& sp, int K, int32_t* idx, float* sel, const float* phi_q,
                          const float* Wq, const float* bq, int P, const void* phi_k, int m,
                          const float* S, const float* u, uint32_t flags, float* y, float* stats,
                          uint8_t* ws, hipStream_t st) {
#define RMA_FUSED(MM, NT)                                                                        \
  return launch_fused_nt<KT, PT, D, MM, NT>(pl, q, G, kv, sp, K, idx, sel, phi_q, Wq, bq, P, phi_k, \
                                            S, u, flags, y, stats, ws, st);
  if (pl.fused_threads == 1024) {
    if (m == 64) { RMA_FUSED(64, 1024) }
    RMA_FUSED(128, 1024)
  }
  if constexpr (D == 64) {
    if (pl.fused_threads == 256) {
      if (m == 64) { RMA_FUSED(64, 256) }
      RMA_FUSED(128, 256)
    }
  }
  if (m == 64) { RMA_FUSED(64, 512) }
  RMA_FUSED(128, 512)
#undef RMA_FUSED
}

}  // namespace

size_t fused_static_lds(int kv_dtype, int phi_dtype, int d, int m, int nt) {
#define RMA_SL(KT, PT, DD)                                                                         \
  if (nt == 1024) return m == 64 ? kernel_static_lds<&decode_fused_kernel<KT, PT, DD, 64, 1024>>()  \
                                 : kernel_static_lds<&decode_fused_kernel<KT, PT, DD, 128, 1024>>(); \
  if (nt == 512) return m == 64 ? kernel_static_lds<&decode_fused_kernel<KT, PT, DD, 64, 512>>()    \
                                : kernel_static_lds<&decode_fused_kernel<KT, PT, DD, 128, 512>>();
#define RMA_SL_D(KT, PT)                                                                           \
  if (d == 64) {                                                                                   \
    RMA_SL(KT, PT, 64)                                                                             \
    return m == 64 ? kernel_static_lds<&decode_fused_kernel<KT, PT, 64, 64, 256>>()                  \
                   : kernel_static_lds<&decode_fused_kernel<KT, PT, 64, 128, 256>>();                \
  }                                                                                                \
  RMA_SL(KT, PT, 128)                                                                              \
  return (size_t)1 << 30;   /* no such instantiation: never fits */
  if (kv_dtype == RMA_BF16) {
    if (phi_dtype == RMA_BF16) { RMA_SL_D(uint16_t, uint16_t) }
    RMA_SL_D(uint16_t, float)
  }
  if (phi_dtype == RMA_BF16) { RMA_SL_D(float, uint16_t) }
  RMA_SL_D(float, float)
#undef RMA_SL_D
#undef RMA_SL
}

hipError_t launch_decode_fused(const DecodePlan& pl, const float* q, int G, const rma_kv& kv,
                               const rma_span& sp, int K, int32_t* idx, float* sel,
                               const float* phi_q, const float* Wq, const float* bq, int P,
                               const void* phi_k, int phi_dtype, int m, const float* S,
                               const float* u, uint32_t flags, float* y, float* stats, uint8_t* ws,
                               hipStream_t st) {
#define RMA_FUSED_DISPATCH(KT, PT)                                                                 \
  return kv.d == 64 ? launch_fused_t<KT, PT, 64>(pl, q, G, kv, sp, K, idx, sel, phi_q, Wq, bq, P,  \
                                                 phi_k, m, S, u, flags, y, stats, ws, st)          \
                    : launch_fused_t<KT, PT, 128>(pl, q, G, kv, sp, K, idx, sel, phi_q, Wq, bq, P, \
                                                  phi_k, m, S, u, flags, y, stats, ws, st);
  if (kv.dtype == RMA_BF16) {
    if (phi_dtype == RMA_BF16) { RMA_FUSED_DISPATCH(uint16_t, uint16_t) }
    RMA_FUSED_DISPATCH(uint16_t, float)
  }
  if (phi_dtype == RMA_BF16) { RMA_FUSED_DISPATCH(float, uint16_t) }
  RMA_FUSED_DISPATCH(float, float)
#undef RMA_FUSED_DISPATCH
}

}  // namespace rma
