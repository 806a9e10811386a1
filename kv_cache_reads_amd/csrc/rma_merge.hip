// Exact branch, retrieved-token subtraction, residual estimate and single
// normalisation ("Residual-Mass Accounting for Partial-KV Decoding": §3 Eq. 3-4
// and Eq. 11 for the exact terms over anchors, retrieved and generated tokens;
// §4.2 Eq. 9 for the subtraction; §4.3 Eq. 10 for the merge; App. C.1 for the
// clamp of the residual denominator).
//
// One block per (unit, query head), or per (unit, query head, slice) when few
// heads would leave most of the chip idle.  The head's exact-support entries
//   [sinks | tail | generated | retrieved (idx)]   (n_a + n_gen + K entries)
// (one contiguous slice of them) are staged in LDS chunk by chunk.  Eight lanes
// share an entry; each 8-lane group takes every NGR-th entry (64 groups in 512
// threads), one kind at a time: first the anchors and generated tokens (V and K
// rows; it computes their scores), then the retrieved tokens (V and phi_k rows).
// It issues the row loads of a batch of entries (8 at d = 64 with bf16 rows,
// fewer for wider rows) before it uses any, and keeps its own running max m:
//   N = sum e^{s_i - m} v_i,  Z = sum e^{s_i - m},
//   w_i = f.Phi_K[i],  nuK = sum_{K(q)} w_i v_i,  ZK = sum_{K(q)} w_i.
// The group partials are combined with max rescaling (fixed order) into m*,
// N_E, Z_E.  phi(q)^T S is a matrix-vector product per head (fp32 VALU; its
// loads are issued before the gathers and consumed after them); then the
// subtraction, the clamp and one normalisation.  With slices, each block writes
// its partial (m, Z, sum w, N, sum w v; slice 0 also phi(q)^T S and u^T f) to the
// workspace, and a second kernel (one block per head) combines the partials in
// slice order, with max rescaling, and writes y.
#include "rma_device.hpp"
#include "rma_internal.hpp"

#include <math.h>

#include <type_traits>

namespace rma {

// RECOMP: phi_k rows are not stored; the retrieved tokens' rows are recomputed
// from their keys with the summary builder's projection (same operands, same
// MFMA order, same bf16 rounding), so the subtraction removes exactly what the
// summaries contain.  Needs bf16 keys.
template <typename KT, typename PT, int D, int M, bool RECOMP, int NTH>
__global__ void __launch_bounds__(NTH, NTH == kMergeThreads ? 1 : 2)
merge_kernel(const float* __restrict__ q, const float* __restrict__ phi_q,
             const float* __restrict__ Wq, const float* __restrict__ bq, int G,
             const KT* __restrict__ kb, const KT* __restrict__ vb, int64_t ustride, int L,
             int n_sink, int n_tail, int n_gen, const int32_t* __restrict__ idx,
             const float* __restrict__ sel, int K, const PT* __restrict__ phik, int L_mid,
             const float* __restrict__ Wk, const float* __restrict__ bk, int P,
             const float* __restrict__ S, const float* __restrict__ u_, uint32_t flags,
             float* __restrict__ y, float* __restrict__ stats, float inv_sqrt_d, int n_slices,
             int slice_len, float* __restrict__ sparts) {
  static_assert(!RECOMP || sizeof(KT) == 2, "recomputed phi rows need bf16 keys");
  static_assert(!RECOMP || NTH == kMergeThreads, "the recompute tiles assume the full block");
  constexpr int NT = NTH, NW = NT / kWave;
  constexpr int LPE = 8;            // lanes per entry
  constexpr int NGR = NT / LPE;     // entry groups
  constexpr int CPL = D / LPE;      // value columns per lane
  constexpr int FPL = M / LPE;      // phi features per lane
  constexpr int CH = kMergeChunk * NT / kMergeThreads;   // entries staged in LDS at a time
  constexpr int SPT = CH / NT;      // staged entries per thread
  // entries per group whose loads are in flight together (bounded by registers)
  constexpr int B = sizeof(KT) == 4 ? 2
                    : sizeof(PT) == 4 ? (D == 128 ? 2 : 4)
                    : D == 128 ? (RECOMP ? 3 : 4) : 8;
  const int ug = blockIdx.x / n_slices, u = ug / G, g = ug - u * G, tid = threadIdx.x;
  const int slice = blockIdx.x - ug * n_slices;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int part = lane & (LPE - 1), grp = tid / LPE;
  const int n_a = n_sink + n_tail, n_ex = n_a + n_gen;
  const int T = n_ex + K;
  const int e0 = slice * slice_len, e1 = min(T, e0 + slice_len);   // this block's entries
  // the subtraction runs only when part of the mid-region stays unretrieved:
  // with K == L_mid the residual is exactly zero and no phi_k row is read
  // (the caller may then pass neither rows nor Wk)
  const bool sub = (flags == RMA_MERGE_SUB) && K > 0 && K < L_mid;
  const bool resid = flags != RMA_MERGE_NO_RESIDUAL;
  const bool whole_mid = (flags == RMA_MERGE_SUB) && K == L_mid;

  __shared__ int s_pos[CH];
  __shared__ float s_sc[CH];
  __shared__ float s_wn[NW][D], s_wk[NW][D];
  __shared__ float s_wm[NW], s_wz[NW], s_wzk[NW];
  __shared__ float s_part[NT / D][D];
  __shared__ float s_uf;
  __shared__ float s_f[M];          // f = phi_q(q) of this head
  // recompute: key rows of a batch of retrieved tokens, per-feature-tile partial
  // weights, and the weights w_i = f.phi_k(k_i) of the chunk's retrieved entries
  constexpr int TS = D == 64 ? 512 : 256;  // tokens per recompute batch (LDS bound)
  constexpr int KROW = D + 8;       // row stride (bf16): 16 B pad
  constexpr int NFT = M / 16;       // feature tiles
  __shared__ __align__(16) uint16_t s_k[RECOMP ? TS * KROW : 8];
  __shared__ float s_wp[RECOMP ? NFT : 1][RECOMP ? TS : 1];
  __shared__ float s_w[RECOMP ? CH : 1];

  const KT* kunit = kb + (size_t)u * ustride;
  const KT* vunit = vb + (size_t)u * ustride;
  const float* qg = q + (size_t)ug * D;
  const int32_t* ig = idx + (size_t)ug * K;
  const float* sg = sel + (size_t)ug * K;

  // position and score of entry j (a retrieved position is clamped into the
  // mid-region so that a bad index cannot fault).  The index and score loads
  // are issued for all of a thread's entries before any is used.
  int spos[SPT];
  float ssc[SPT];
  auto stage_load = [&](int c0) {
    int ri[SPT];
    float rs[SPT];
    if (K > 0) {
#pragma unroll
      for (int r = 0; r < SPT; ++r) {
        const int jr = min(max(c0 + tid + NT * r - n_ex, 0), K - 1);
        ri[r] = ig[jr];
        rs[r] = sg[jr];
      }
    }
#pragma unroll
    for (int r = 0; r < SPT; ++r) {
      const int j = c0 + tid + NT * r;
      const bool ret = j >= n_ex && j < e1;
      int pos = j < n_sink ? j : (j < n_a ? L - n_tail + (j - n_sink) : L + (j - n_a));
      if (ret) pos = min(max(ri[r], n_sink), n_sink + max(L_mid, 1) - 1);
      spos[r] = j < e1 ? pos : n_sink;
      ssc[r] = ret ? rs[r] : 0.f;
    }
  };
  auto stage_store = [&]() {
#pragma unroll
    for (int r = 0; r < SPT; ++r) {
      s_pos[tid + NT * r] = spos[r];
      s_sc[tid + NT * r] = ssc[r];
    }
  };
  // f = phi_q(q): its operands are loaded first, so that computing it waits only
  // for them (loads complete in issue order); without Wq the given features are
  // read, and the loads read q instead (discarded)
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
    fb0 = fcomp ? bq[(size_t)pset * M + fi] : (resid && phi_q != nullptr ? phi_q[(size_t)ug * M + (tid % M)] : 0.f);
  }
  stage_load(e0);

  float qr[CPL], fr[FPL];
#pragma unroll
  for (int i = 0; i < CPL; i += 4) {
    const float4 t = *reinterpret_cast<const float4*>(qg + part * CPL + i);
    qr[i] = t.x; qr[i + 1] = t.y; qr[i + 2] = t.z; qr[i + 3] = t.w;
  }

  // ---- operands of phi(q)^T S and u^T f, loaded now and used after the
  //      entries, so that their latency overlaps the gathers.  For one head
  //      this is a matrix-vector product: thread (column col, feature block fb)
  //      loads its FPB elements of S once (coalesced along the columns).
  //      Without a residual the loads read q instead and are discarded.
  // (with slices, the first slice of the head forms phi(q)^T S and u^T f)
  const bool rs = resid && !whole_mid && slice == 0;
  constexpr int FB = NT / D;          // feature blocks
  constexpr int FPB = M / FB;         // features per block
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

  // recompute operands of this wave's 16-feature tile (W split into bf16 hi + lo,
  // bias), derived with the prologue loads in flight
  constexpr int RKS = RECOMP ? D / 32 : 1;
  bf16x8_t rWhi[RKS], rWlo[RKS];
  float rbf = 0.f, rfq = 0.f;
  if constexpr (RECOMP) {
    if (sub) {
      const int f = (wave % NFT) * 16 + (lane & 15), pset = u % P;
      split_w_operands<RKS>(Wk + ((size_t)pset * M + f) * D + 8 * (lane >> 4), rWhi, rWlo);
      rbf = bk[(size_t)pset * M + f];
    }
  }

  // ---- f = phi_q(q) into LDS: the given features, or elu(Wq q + bq) + 1
  //      computed here (NT/M threads per feature, fp32, fixed sum order)
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
#pragma unroll
  for (int i = 0; i < FPL; ++i) fr[i] = sub ? s_f[part * FPL + i] : 0.f;
  // bf16 phi rows: w on the bf16 dot instruction, f as packed bf16 hi / lo pairs
  // (the fused decode kernel splits the same values the same way)
  constexpr bool DOT2 = sizeof(PT) == 2 && !RECOMP;
  uint32_t fh[FPL / 2], fl[FPL / 2];
#pragma unroll
  for (int j = 0; j < FPL / 2; ++j) {
    fh[j] = 0u;
    fl[j] = 0u;
    if (DOT2 && sub) split_f_bf16x2(fr[2 * j], fr[2 * j + 1], fh[j], fl[j]);
  }
  if constexpr (RECOMP) {
    if (sub) rfq = s_f[(wave % NFT) * 16 + (lane & 15)];
  }

  // w_i of the retrieved entries [r0, cnt) of the staged chunk, into s_w
  auto recompute_w = [&](int c0, int cnt) {
    constexpr int CPR = D / 8;
    constexpr int WPT = NW / NFT;                // waves per feature tile
    const int ft = wave % NFT, th = wave / NFT;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int r0 = max(0, n_ex - c0);
    constexpr int PPT = TS * CPR / NT;             // 16-byte row pieces per thread
    static_assert(TS * CPR % NT == 0, "whole pieces per thread");
    for (int sb = r0; sb < cnt; sb += TS) {
      const int nrow = min(TS, cnt - sb);
      // key rows into LDS (rows past the batch re-read its last row); the
      // previous batch ended with a barrier, so the loads can all be issued
      // before the first store
#pragma unroll
      for (int j = 0; j < PPT; ++j) {
        const int i = tid + NT * j, row = i / CPR, cc = i - row * CPR;
        const int pos = s_pos[sb + min(row, nrow - 1)];
        *reinterpret_cast<uint4*>(s_k + row * KROW + cc * 8) =
            *reinterpret_cast<const uint4*>(kunit + (size_t)pos * D + cc * 8);
      }
      __syncthreads();
      for (int tt = th; tt < (nrow + 15) / 16; tt += WPT) {
        const f32x4 acc = proj_tile16<RKS>(s_k + (tt * 16 + l16) * KROW + 8 * g4, rWhi, rWlo);
        const uint32_t p01 = pack_bf16x2(phi_elu1(acc[0] + rbf), phi_elu1(acc[1] + rbf));
        const uint32_t p23 = pack_bf16x2(phi_elu1(acc[2] + rbf), phi_elu1(acc[3] + rbf));
        float v[4] = {rfq * bf16lo(p01), rfq * bf16hi(p01), rfq * bf16lo(p23), rfq * bf16hi(p23)};
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = lane_group_sum<16>(v[r]);
        if (l16 == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) s_wp[ft][tt * 16 + 4 * g4 + r] = v[r];
        }
      }
      __syncthreads();
      for (int i = tid; i < TS; i += NT) {
        if (sb + i < cnt) {
          float w = 0.f;
#pragma unroll
          for (int k = 0; k < NFT; ++k) w += s_wp[k][i];
          s_w[sb + i] = w;
        }
      }
      __syncthreads();  // s_k and s_wp are free again; after the last batch s_w is complete
    }
  };

  float N[CPL], NK[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) { N[c] = 0.f; NK[c] = 0.f; }
  float Z = 0.f, ZK = 0.f, mrun = -INFINITY;

  // ---- exact-support entries, CH at a time
  for (int c0 = e0; c0 < e1; c0 += CH) {
    if (c0 > e0) {
      __syncthreads();  // the previous chunk's entries are consumed
      stage_load(c0);
    }
    stage_store();
    __syncthreads();
    const int cnt = min(CH, e1 - c0);
    if constexpr (RECOMP) {
      if (sub) recompute_w(c0, cnt);
    }
    // Exactly scored entries (anchors and generated tokens: the list's first
    // n_ex) and retrieved ones in two passes.  Within a pass every entry slot
    // issues the same loads without a branch (a slot past the pass's end reads
    // the pass's first entry again and adds nothing), so all of a group's loads
    // are in flight before the first one is used.
    const int n_exc = min(max(n_ex - c0, 0), cnt);
    auto gather = [&](int lo, int hi, auto ex_tag) {
      constexpr bool EX = decltype(ex_tag)::value;
      const bool ld_phi = !EX && !RECOMP && sub;   // uniform
      for (int jb = lo + grp; jb < hi; jb += NGR * B) {
        RawPiece<KT, CPL> vr[B], kr[B];
        RawPiece<PT, FPL> pr[B];
        float scs[B];
        int jcs[B];
#pragma unroll
        for (int e = 0; e < B; ++e) {
          const int jj = jb + e * NGR;
          const int jc = jj < hi ? jj : lo;
          const int pos = s_pos[jc];
          jcs[e] = jc;
          scs[e] = s_sc[jc];
          vr[e].load(vunit + (size_t)pos * D + part * CPL);
          if constexpr (EX) kr[e].load(kunit + (size_t)pos * D + part * CPL);
          else kr[e].zero();
          if (ld_phi) pr[e].load(phik + ((size_t)u * L_mid + (pos - n_sink)) * M + part * FPL);
          else pr[e].zero();
        }
        __builtin_amdgcn_sched_barrier(0);   // every load issued before any use
#pragma unroll
        for (int e = 0; e < B; ++e) {
          // both dots on every lane (zeros where unused), so the 8-lane sums
          // never run under divergent control flow
          float kv[CPL], vv[CPL];
          kr[e].unpack(kv);
          float a = 0.f, w = 0.f;
#pragma unroll
          for (int i = 0; i < CPL; ++i) a = __fmaf_rn(qr[i], kv[i], a);
          if constexpr (DOT2) {
            w = dot_phi_bf16<FPL>(pr[e], fh, fl);
          } else {
            float ph[FPL];
            pr[e].unpack(ph);
#pragma unroll
            for (int i = 0; i < FPL; ++i) w = __fmaf_rn(fr[i], ph[i], w);
          }
          a = lane_group_sum<LPE>(a);
          w = lane_group_sum<LPE>(w);
          if constexpr (RECOMP) w = (!EX && sub) ? s_w[jcs[e]] : 0.f;
          if (jb + e * NGR < hi) {  // uniform within the group
            const float s = EX ? a * inv_sqrt_d : scs[e];
            if (s > mrun) {
              const float r = __expf(mrun - s);  // 0 while nothing is accumulated
#pragma unroll
              for (int c = 0; c < CPL; ++c) N[c] *= r;
              Z *= r;
              mrun = s;
            }
            const float ew = __expf(s - mrun);
            vr[e].unpack(vv);
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              N[c] = __fmaf_rn(ew, vv[c], N[c]);
              NK[c] = __fmaf_rn(w, vv[c], NK[c]);
            }
            Z += ew;
            ZK += w;
          }
        }
      }
    };
    gather(0, n_exc, std::true_type{});
    gather(n_exc, cnt, std::false_type{});
  }

  // ---- phi(q)^T S (per feature block) and u^T f
  if (rs) {
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < FPB; ++i) p = __fmaf_rn(s_f[fb * FPB + i], sv[i], p);  // f: LDS broadcast
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

  // ---- combine the eight groups of each wave (lanes l, l^8, l^16, l^32 hold the
  //      same columns), then the waves through LDS, rescaling to the larger max
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
  float uf = rs ? s_uf : 0.f;

  // ---- slices: this block's partial to the workspace (combined by
  //      merge_combine_kernel)
  constexpr int PFL = 4 + 3 * D;     // floats per partial
  if (n_slices > 1) {
    float* pp = sparts + ((size_t)ug * n_slices + slice) * PFL;
    if (tid == 0) {
      pp[0] = ms;
      pp[1] = ZE;
      pp[2] = ZKt;
      pp[3] = uf;
    }
    for (int col = tid; col < D; col += NT) {
      float NE = 0.f, NKc = 0.f, fs = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        NE += sw[w] * s_wn[w][col];
        NKc += s_wk[w][col];
      }
      if (rs) {
#pragma unroll
        for (int k = 0; k < FB; ++k) fs += s_part[k][col];
      }
      pp[4 + col] = NE;
      pp[4 + D + col] = NKc;
      pp[4 + 2 * D + col] = fs;
    }
    return;
  }

  float zr = 0.f;
  if (resid && !whole_mid) zr = fmaxf(uf - (sub ? ZKt : 0.f), 0.f);
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

// Combines the slice partials of each (unit, query head) in slice order: the
// running maxima are rescaled to their largest, Z, N and sum w v are summed,
// slice 0 holds phi(q)^T S and u^T f; then the subtraction, the clamp and the
// one normalisation, exactly as at the end of merge_kernel.  One thread per
// slice stages the partial headers in LDS; each column's sums over the slices
// then run with their loads in flight together.
template <int D>
__global__ void __launch_bounds__(kMergeCombineThreads)
merge_combine_kernel(const float* __restrict__ sparts, int n_slices, uint32_t flags, int K,
                     int L_mid, float* __restrict__ y, float* __restrict__ stats) {
  constexpr int PFL = 4 + 3 * D;
  __shared__ float s_m[kMergeCombineThreads], s_z[kMergeCombineThreads], s_zk[kMergeCombineThreads];
  __shared__ float s_sc[kMergeCombineThreads];
  __shared__ float s_tot[4];
  const int ug = blockIdx.x, tid = threadIdx.x;
  const bool sub = (flags == RMA_MERGE_SUB) && K > 0 && K < L_mid;
  const bool resid = flags != RMA_MERGE_NO_RESIDUAL;
  const bool whole_mid = (flags == RMA_MERGE_SUB) && K == L_mid;
  const float* pb = sparts + (size_t)ug * n_slices * PFL;
  if (tid < n_slices) {
    const float* pk = pb + (size_t)tid * PFL;
    s_m[tid] = pk[0];
    s_z[tid] = pk[1];
    s_zk[tid] = pk[2];
  }
  __syncthreads();
  float mall = -INFINITY;
  for (int k = 0; k < n_slices; ++k) mall = fmaxf(mall, s_m[k]);
  if (tid < n_slices) s_sc[tid] = s_m[tid] == -INFINITY ? 0.f : __expf(s_m[tid] - mall);
  __syncthreads();
  if (tid == 0) {
    float ZE = 0.f, ZK = 0.f;
    for (int k = 0; k < n_slices; ++k) {
      ZE += s_sc[k] * s_z[k];
      ZK += s_zk[k];
    }
    float zr = 0.f;
    if (resid && !whole_mid) zr = fmaxf(pb[3] - (sub ? ZK : 0.f), 0.f);
    s_tot[0] = ZE;
    s_tot[1] = ZK;
    s_tot[2] = zr;
    if (stats != nullptr) {
      stats[(size_t)ug * 4 + 0] = mall;
      stats[(size_t)ug * 4 + 1] = ZE;
      stats[(size_t)ug * 4 + 2] = zr;
      stats[(size_t)ug * 4 + 3] = ZK;
    }
  }
  __syncthreads();
  const float ZE = s_tot[0], zr = s_tot[2];
  const float lz = zr > 0.f ? __logf(zr) : -INFINITY;
  const float Mx = fmaxf(mall, lz);
  const float a = __expf(mall - Mx);
  const float bres = __expf(-Mx);
  const float den = a * ZE + bres * zr;
  for (int col = tid; col < D; col += kMergeCombineThreads) {
    float NE = 0.f, NK = 0.f;
#pragma unroll 8
    for (int k = 0; k < n_slices; ++k) {
      const float* pk = pb + (size_t)k * PFL;
      NE += s_sc[k] * pk[4 + col];
      NK += pk[4 + D + col];
    }
    const float nu = (resid && !whole_mid) ? pb[4 + 2 * D + col] - (sub ? NK : 0.f) : 0.f;
    y[(size_t)ug * D + col] = (a * NE + bres * nu) / den;
  }
}

template <typename KT, typename PT, int D>
hipError_t launch_merge_t(const MergePlan& pl, uint8_t* ws, const float* q, const float* phi_q,
                          const float* Wq, const float* bq, int G, const rma_kv& kv,
                          const rma_span& sp, const int32_t* idx, const float* sel, int K,
                          const void* phi_k, const float* Wk, const float* bk, int P, int m,
                          const float* S, const float* u, uint32_t flags, float* y, float* stats,
                          hipStream_t st) {
  const int L_mid = (int)(sp.L - sp.n_sink - sp.n_tail);
  const bool recomp = phi_k == nullptr && Wk != nullptr;
  // many (unit, head) blocks: 256 threads each, so that two blocks share a CU
  // and one block's prologue or combine overlaps another's gathers
  const bool small = D == 64 && !recomp && kv.n_units * G >= 2048;
  auto kern = m == 64 ? merge_kernel<KT, PT, D, 64, false, kMergeThreads>
                      : merge_kernel<KT, PT, D, 128, false, kMergeThreads>;
  if constexpr (D == 64) {  // (at d = 128 the smaller block runs out of registers)
    if (small)
      kern = m == 64 ? merge_kernel<KT, PT, D, 64, false, 256> : merge_kernel<KT, PT, D, 128, false, 256>;
  }
  if constexpr (sizeof(KT) == 2 && sizeof(PT) == 2) {
    if (recomp)
      kern = m == 64 ? merge_kernel<KT, PT, D, 64, true, kMergeThreads>
                     : merge_kernel<KT, PT, D, 128, true, kMergeThreads>;
  }
  float* part = reinterpret_cast<float*>(ws + pl.off_part);
  hipError_t e = launch_kernel("merge_kernel", kern, dim3(kv.n_units * G * pl.n_slices),
                               dim3(small ? 256 : kMergeThreads), 0, st, q, phi_q, Wq, bq, G,
                               static_cast<const KT*>(kv.k), static_cast<const KT*>(kv.v),
                               kv.unit_stride, (int)sp.L, sp.n_sink, sp.n_tail, (int)sp.n_gen, idx,
                               sel, K, static_cast<const PT*>(phi_k), L_mid, Wk, bk, P, S, u, flags,
                               y, stats, 1.0f / sqrtf((float)D), pl.n_slices, pl.sl, part);
  if (e != hipSuccess || pl.n_slices == 1) return e;
  return launch_kernel("merge_combine_kernel", merge_combine_kernel<D>, dim3(kv.n_units * G),
                       dim3(kMergeCombineThreads), 0, st, part, pl.n_slices, flags, K, L_mid, y,
                       stats);
}

hipError_t launch_merge(const MergePlan& pl, const float* q, const float* phi_q, const float* Wq,
                        const float* bq, int G,
                        const rma_kv& kv, const rma_span& sp, const int32_t* idx,
                        const float* sel, int K, const void* phi_k, int phi_dtype,
                        const float* Wk, const float* bk, int P, int m, const float* S,
                        const float* u, uint32_t flags, float* y, float* stats, uint8_t* ws,
                        hipStream_t st) {
#define RMA_MERGE_DISPATCH(KT, PT)                                                                \
  return kv.d == 64 ? launch_merge_t<KT, PT, 64>(pl, ws, q, phi_q, Wq, bq, G, kv, sp, idx, sel, K,  \
                                                 phi_k, Wk, bk, P, m, S, u, flags, y, stats, st)   \
                    : launch_merge_t<KT, PT, 128>(pl, ws, q, phi_q, Wq, bq, G, kv, sp, idx, sel, K, \
                                                  phi_k, Wk, bk, P, m, S, u, flags, y, stats, st);
  if (kv.dtype == RMA_BF16) {
    if (phi_dtype == RMA_BF16) { RMA_MERGE_DISPATCH(uint16_t, uint16_t) }
    RMA_MERGE_DISPATCH(uint16_t, float)
  }
  if (phi_dtype == RMA_BF16) { RMA_MERGE_DISPATCH(float, uint16_t) }
  RMA_MERGE_DISPATCH(float, float)
#undef RMA_MERGE_DISPATCH
}

hipError_t launch_merge_combine(const float* parts, int n_slices, int heads, int d, uint32_t flags,
                                int K, int L_mid, float* y, float* stats, hipStream_t st) {
  if (d == 64)
    return launch_kernel("merge_combine_kernel", merge_combine_kernel<64>, dim3(heads),
                         dim3(kMergeCombineThreads), 0, st, parts, n_slices, flags, K, L_mid, y, stats);
  return launch_kernel("merge_combine_kernel", merge_combine_kernel<128>, dim3(heads),
                       dim3(kMergeCombineThreads), 0, st, parts, n_slices, flags, K, L_mid, y, stats);
}

}  // namespace rma
