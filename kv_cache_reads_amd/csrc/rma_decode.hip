// Fused decode of one query head: the exact Top-K selection and the merge in
// one block ("Residual-Mass Accounting for Partial-KV Decoding": §1 and §3
// Eq. 3 for the exhaustive Top-K; §3 Eq. 3-4 and Eq. 11 for the exact terms
// over anchors, retrieved and generated tokens; §4.2 Eq. 9 for the
// subtraction; §4.3 Eq. 10 for the single normalisation; App. C.1 for the
// clamp of the residual denominator).
//
// rma_decode runs the scan of rma_decode_topk, then this kernel, grid (U, G,
// slices).  A block first issues every load it needs before the selection's
// result: its head's chunk reports and chunk table, the query, the feature
// map's operands (or the given features), S and u, and one exactly scored row
// per 8-lane group.  Then, in order (each step behind one barrier):
//   1. wave 0: each chunk's offset in the union (a wave scan of the counts)
//      and the union's scan-bin range (lowest cut, highest top bin of the
//      chunk table); everyone: f = phi_q(q) into LDS;
//   2. the reports into the union (compacted, position order), each counted
//      in the selection histogram as it is placed; phi(q)^T S per feature
//      block and u^T f; the exactly scored rows' scores and their maximum;
//   3. the selection (block_select in rma_select.hpp, the exact fallback if it
//      fails): the K positions and their scaled fp32 scores into an LDS list
//      (and, when asked, to idx / sel in ascending order);
//   4. the retrieved tokens from that list: their V and phi_k rows are
//      gathered with every load of a batch issued before the first is used;
//      e^{s - mref} v, w = f.phi_k and w v accumulate per 8-lane group, where
//      mref, the larger of the exact rows' maximum and the upper edge of the
//      union's highest scan bin, bounds every score of the exact support (no
//      running-max rescale); the exact rows' terms are added while the first
//      batch loads;
//   5. the combine: the two groups of a 16-lane row added by DPP, the pair sums
//      written into the union's LDS (free once the list is complete) and added
//      in pair order, Z and sum w per wave in row order (deterministic), m* =
//      the largest score added; then the subtraction, the clamp and one
//      normalisation.
// Every wave executes most of these steps, four waves to a SIMD: the vector
// instructions per wave, not memory, bound a block, so work each wave would
// repeat for itself is kept out of the waves (LDS atomics on order-preserving
// keys, DPP scans, 16-lane row scans in place of per-wave loops).
// The arithmetic of a term is the merge kernel's; the order of the sums
// differs (the fused kernel spreads a head's entries over more groups).
#include "rma_select.hpp"

#include <math.h>

#include <type_traits>

namespace rma {

template <typename KT, typename PT, int D, int M, int NT>
__global__ void __launch_bounds__(NT)
decode_fused_kernel(const float4* __restrict__ hpw, const int2* __restrict__ meta,
                    const float2* __restrict__ ent, const float* __restrict__ q,
                    const float* __restrict__ Wq, int G, int n_chunks, int r_cap, int P,
                    const KT* __restrict__ kb, const KT* __restrict__ vb, int64_t ustride, int L,
                    int n_sink, int n_tail, int n_gen, int L_mid, int ch, int K,
                    int32_t* __restrict__ idx_out, float* __restrict__ sc_out,
                    const float* __restrict__ phi_q, const float* __restrict__ bq,
                    const PT* __restrict__ phik, const float* __restrict__ S,
                    const float* __restrict__ u_, uint32_t flags, float* __restrict__ y,
                    float* __restrict__ stats, float inv_sqrt_d, int n_split,
                    float* __restrict__ sparts) {
  // (the first 14 argument words, hpw .. P, arrive preloaded in registers: the
  // loads of the reports, the chunk table, q and W below need no other argument)
  constexpr int NW = NT / kWave;
  constexpr int LPE = 8;            // lanes per entry
  constexpr int NGR = NT / LPE;     // entry groups
  constexpr int CPL = D / LPE;      // value columns per lane
  constexpr int FPL = M / LPE;      // phi features per lane
  constexpr int SPEC = kFusedSpec<NT>;     // report slots per thread
  // retrieved entries per group whose row loads are in flight together (the
  // merge kernel's batch, fewer in 1024-thread blocks, whose lanes have 128
  // registers: 128 groups x 4 rows at d = 64, x 3 at d = 128 with bf16 rows)
  constexpr int B = fused_gather_batch((int)sizeof(KT), (int)sizeof(PT), D, NT);
  constexpr int NV = 2 * D;         // combined vectors: N[D], sum w v [D] (Z, sum w apart)
  constexpr int NP = NT / 16;       // group pairs (two groups per 16-lane row)
  // row stride of the pair sums: = 8 (mod 64 banks), so the 8 x 8 lanes of a
  // wave that read pair pp0 + sl, value j0 + jj hit 64 different banks
  constexpr int NVS = NV + 8;
  // dynamic LDS: the union of the chunk reports (scores, positions; room for
  // n_chunks r_cap entries rounded up to whole rows of 64), at least as large as
  // the combine's pair sums, which reuse it once the list is complete; then the
  // list of the K selected (positions, scaled scores)
  extern __shared__ __align__(16) float dyn[];
  constexpr int UB = kWave;   // the union is padded to whole rows of 64 entries
  const int PS = (n_chunks * r_cap + UB - 1) / UB * UB;
  const int UR = max(2 * PS, NP * NVS);
  float* es = dyn;
  int* ep = reinterpret_cast<int*>(dyn + PS);
  int* lpos = reinterpret_cast<int*>(dyn + UR);
  float* lsc = dyn + UR + K;
  float* red = dyn;

  static_assert(kSelMaxChunks == 4 * kWave, "four chunks per lane of wave 0");
  __shared__ int s_off[kSelMaxChunks], s_bcs[kSelMaxChunks], s_nrep[kSelMaxChunks];
  __shared__ int s_nE, s_trunc;
  // ordered-integer keys (ord_f32) reduced by LDS atomics: [2] the exact rows'
  // highest score, [3] the largest score added ([0], [1] unused)
  __shared__ uint32_t s_rng[4];
  __shared__ int s_bin_lo, s_bin_hi;   // the union's scan-bin range: lowest cut, highest top
  __shared__ float s_qf[D];
  __shared__ uint32_t s_hist[kSelBins];
  __shared__ uint32_t s_coarse[kSelBins / 16];
  __shared__ __align__(16) float s_cand[kSelBandMax];
  __shared__ int s_bslot[kSelBandMax];
  __shared__ DD s_bdd[kSelBandMax];
  __shared__ int s_misc[8];
  __shared__ int s_buf[kSelThreads / kWave + 1];
  __shared__ int s_wcnt[NW];
  __shared__ float s_fin[NV + 2];   // the sums: N, sum w v, Z, sum w
  __shared__ float s_zw[NW][2];     // per wave: Z, sum w
  __shared__ float s_part[NT / D][D];
  __shared__ float s_uf;
  __shared__ float s_f[M];          // f = phi_q(q) of this head
  __shared__ uint32_t s_fhl[2][M / 2];   // f as packed bf16 hi / lo pairs (bf16 phi rows)

  // block (unit u, head g, slice rsl) of the (units, G, n_split) grid: every
  // slice's block selects, slice rsl gathers the list entries [rsl sl, (rsl + 1)
  // sl) (slice 0 also the exact rows) and writes a partial that
  // merge_combine_kernel combines.  The grid's shape gives u, g and rsl without
  // a division.  Consecutive workgroups take consecutive units and go to the 8
  // XCDs in turn, so when the unit count is a multiple of 8 a unit's heads run on
  // one XCD and share its L2 copy of S, u and the feature map's weights.
  const int rsl = blockIdx.z, u = blockIdx.x;
  const int ug = u * G + blockIdx.y, tid = threadIdx.x;
  // the head's binning parameters: a uniform load issued first, while no
  // statement with side effects precedes it (so it goes through the scalar cache)
  const f32x4 hp_in = *reinterpret_cast<const f32x4*>(hpw + ug);
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int part = lane & (LPE - 1), grp = tid / LPE;
  const float* qg = q + (size_t)ug * D;
  const int2* mt = meta + (size_t)ug * n_chunks;
  const float2* en = ent + (size_t)ug * n_chunks * r_cap;

  // ---- 1. loads.  The selection's: the chunk table and the report slots (a
  //      power-of-two group of tpc threads per chunk; thread t serves chunk
  //      t >> lg_t, its slots my_s + k tpc, so no slot index needs a division);
  //      the first SPEC tpc slots of each chunk now, the rest (only where r_cap
  //      exceeds them) in later rounds
  const int lg_c = n_chunks > 1 ? 32 - __clz(n_chunks - 1) : 0;
  const int lg_t = __builtin_ctz(NT) - lg_c, tpc = 1 << lg_t;
  const int my_c = tid >> lg_t, my_s = tid & (tpc - 1);
  const int cc = min(my_c, n_chunks - 1);
  const int2 m_mine = *off32(mt, cc);
  float2 sv2[SPEC];
#pragma unroll
  for (int k = 0; k < SPEC; ++k) sv2[k] = *off32(en, cc * r_cap + min(my_s + k * tpc, r_cap - 1));
  // the chunk table: four chunks per lane of wave 0, which computes the offsets
  int2 mc[4];
  if (wave == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) mc[k] = *off32(mt, min(lane * 4 + k, n_chunks - 1));
  }
  const float q_in = *off32(qg, min(tid, D - 1));
  // the merge's: f's operands (or the given features), q, S, u
  constexpr int TPF = NT / M, EPT = D / TPF;     // threads per feature, elements each
  const int fi = tid / TPF, fpart = tid % TPF;
  float qr[CPL];
#pragma unroll
  for (int i = 0; i < CPL; i += 4) {
    const float4 t = *reinterpret_cast<const float4*>(off32(qg, part * CPL + i));
    qr[i] = t.x; qr[i + 1] = t.y; qr[i + 2] = t.z; qr[i + 3] = t.w;
  }
  float wq[EPT], xq[EPT], fb0;
  {
    const int pset = P > 1 ? u % P : 0;
    const float* wb = Wq != nullptr ? Wq + (size_t)pset * M * D : qg;   // W of this unit's set
    const uint32_t wo = Wq != nullptr ? fi * D + fpart * EPT : 0u;
    const uint32_t qo = fpart * EPT;
#pragma unroll
    for (int i = 0; i < EPT; i += 4) {
      const float4 w4 = *reinterpret_cast<const float4*>(off32(wb, wo + i));
      wq[i] = w4.x; wq[i + 1] = w4.y; wq[i + 2] = w4.z; wq[i + 3] = w4.w;
      if constexpr (TPF != LPE) {
        const float4 x4 = *reinterpret_cast<const float4*>(off32(qg, qo + i));
        xq[i] = x4.x; xq[i + 1] = x4.y; xq[i + 2] = x4.z; xq[i + 3] = x4.w;
      }
    }
    if constexpr (TPF == LPE) {   // fpart == part, EPT == CPL: the same elements as qr
#pragma unroll
      for (int i = 0; i < EPT; ++i) xq[i] = qr[i];
    }
  }
  // every other kernel argument into registers at once (one round trip, now
  // that the first loads are in flight) rather than one per branch that needs some
  asm volatile("" ::"s"(q), "s"(G), "s"(kb), "s"(vb), "s"(ustride), "s"(L), "s"(n_sink), "s"(n_tail),
               "s"(n_gen), "s"(L_mid), "s"(ch), "s"(n_chunks), "s"(r_cap), "s"(K), "s"(hpw), "s"(ent),
               "s"(meta), "s"(idx_out), "s"(sc_out), "s"(phi_q), "s"(Wq), "s"(bq), "s"(P), "s"(phik),
               "s"(S), "s"(u_), "s"(flags), "s"(y), "s"(stats), "s"(inv_sqrt_d));
  const int n_a = n_sink + n_tail, n_ex = n_a + n_gen;
  // the subtraction runs only when part of the mid-region stays unretrieved
  const bool sub = (flags == RMA_MERGE_SUB) && K > 0 && K < L_mid;
  const bool resid = flags != RMA_MERGE_NO_RESIDUAL;
  const bool whole_mid = (flags == RMA_MERGE_SUB) && K == L_mid;
  const bool rs = resid && !whole_mid;   // phi(q)^T S and u^T f are needed

  const KT* kunit = kb + (size_t)u * ustride;
  const KT* vunit = vb + (size_t)u * ustride;
  const PT* phiu = phik + (size_t)u * L_mid * M;   // this unit's phi_k rows

  const bool fcomp = resid && Wq != nullptr;
  {
    const int pset = P > 1 ? u % P : 0;
    fb0 = fcomp ? *off32(bq + (size_t)pset * M, fi)
                : (resid && phi_q != nullptr ? *off32(phi_q + (size_t)ug * M, tid % M) : 0.f);
  }
  // phi(q)^T S: thread (column scol, feature block fb) holds its FPB elements of
  // S (coalesced along the columns); without a residual the loads read q
  constexpr int FB = NT / D;          // feature blocks
  constexpr int FPB = M / FB;         // features per block
  static_assert(FB >= 1 && M % FB == 0, "whole feature blocks");
  const int scol = tid % D, fb = tid / D;
  float sv[FPB];
  {
    const float* Sb = rs ? S + (size_t)u * M * D : qg;   // this unit's S
    const uint32_t so = rs ? fb * FPB * D + scol : 0u;
    const uint32_t sst = rs ? D : 0u;
#pragma unroll
    for (int i = 0; i < FPB; ++i) sv[i] = *off32(Sb, so + sst * i);
  }
  constexpr int UPL = (M + kWave - 1) / kWave;   // u^T f terms per lane (last wave)
  float uu[UPL];
#pragma unroll
  for (int i = 0; i < UPL; ++i) uu[i] = rs ? *off32(u_ + (size_t)u * M, min(lane + kWave * i, M - 1)) : 0.f;
  // the exactly scored rows (sinks, tail, generated tokens): group g takes rows
  // g, g + NGR, ...; the first now, scored while the retrieved rows load
  auto ex_pos = [&](int j) {
    return j < n_sink ? j : (j < n_a ? L - n_tail + (j - n_sink) : L + (j - n_a));
  };
  RawPiece<KT, CPL> xv, xk;
  {
    const int pos = ex_pos(grp < n_ex ? grp : 0);
    xv.load(off32(vunit, pos * D + part * CPL));
    xk.load(off32(kunit, pos * D + part * CPL));
  }
  const BlockSelLds wl{s_hist, s_coarse, s_cand, s_bslot, s_bdd, s_misc, s_wcnt};
  init_block_select<NT>(wl);
  if (tid < 4) s_rng[tid] = tid == 0 ? 0xffffffffu : 0u;   // the identities of min / max

  // ---- 2. wave 0: each chunk's offset in the union (a wave scan of the counts
  //      it reported, at most r_cap each), the chunk table, the scan-bin range
  //      of the union (every report lies between its chunk's cut and top bins),
  //      empty entries after the union up to a whole row of 64.  Everyone: q
  //      for the band rescoring, f = phi_q(q).
  if (wave == 0) {
    int wc4[4], ls = 0;
    uint32_t blo = 0u, bhi = 0u;   // max of ~cut (the lowest cut) and of top + 1
    bool tr = false;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = lane * 4 + k;
      wc4[k] = c < n_chunks ? min(mc[k].y, r_cap) : 0;
      tr |= c < n_chunks && mc[k].y > r_cap;   // the chunk withheld tokens
      ls += wc4[k];
      if (c < n_chunks) {
        blo = max(blo, ~(uint32_t)(mc[k].x & 0xffff));
        bhi = max(bhi, (uint32_t)(mc[k].x >> 16) + 1u);
      }
    }
    blo = ~wave_max_u32(blo);
    bhi = wave_max_u32(bhi);
    const int incl = wave_incl_scan_dpp(ls);
    int o = incl - ls;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = lane * 4 + k;
      if (c < n_chunks) {
        s_off[c] = o;
        s_bcs[c] = mc[k].x & 0xffff;
        s_nrep[c] = mc[k].y;
      }
      o += wc4[k];
    }
    const int nE = __builtin_amdgcn_readlane(incl, kWave - 1);
    const bool trunc = __ballot(tr) != 0ull;
    const int pad = (nE + UB - 1) / UB * UB;
    for (int i = nE + lane; i < pad; i += kWave) {
      es[i] = -INFINITY;
      ep[i] = 0;
    }
    if (lane == 0) {
      s_nE = nE;
      s_trunc = trunc;
      s_bin_lo = (int)blo;
      s_bin_hi = (int)bhi;   // one past the highest top bin
    }
  }
  if (tid < D) s_qf[tid] = q_in;
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

  // ---- 3. the reports into the union (chunk c's j-th at s_off[c] + j) and the
  //      histogram of their selection bins (with 16-bin sums); phi(q)^T S per
  //      feature block and u^T f
  const HeadParams hp{hp_in[0], hp_in[1], hp_in[2]};
  // the load's unused fourth word stays allocated until here, so no register of
  // the load is reused (which would make the prologue wait for it)
  asm volatile("" ::"s"(hp_in[3]));
  const SelBins sbin = sel_bins(hp, s_bin_lo, s_bin_hi);
  if (sizeof(PT) == 2 && sub && tid < M / 2)   // f as bf16 hi / lo pairs for the gather
    split_f_bf16x2(s_f[2 * tid], s_f[2 * tid + 1], s_fhl[0][tid], s_fhl[1][tid]);
  {
    if (my_c < n_chunks) {
      const int wc = min(m_mine.y, r_cap), o0 = s_off[my_c];
      for (int j0 = 0;;) {
#pragma unroll
        for (int k = 0; k < SPEC; ++k) {
          const int j = j0 + my_s + k * tpc;
          if (j < wc) {
            es[o0 + j] = sv2[k].x;
            ep[o0 + j] = __float_as_int(sv2[k].y);
            const int b = sbin(sv2[k].x);
            atomicAdd(&s_hist[b], 1u);
            atomicAdd(&s_coarse[b >> 4], 1u);
          }
        }
        j0 += SPEC * tpc;
        if (j0 >= wc) break;
#pragma unroll
        for (int k = 0; k < SPEC; ++k)
          sv2[k] = *off32(en, cc * r_cap + min(j0 + my_s + k * tpc, r_cap - 1));
      }
    }
  }
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
  // the exactly scored rows' scores q.k / sqrt(d) (eight lanes, q from LDS) and
  // their maximum; the group's first row stays loaded for its term
  auto ex_score = [&](const RawPiece<KT, CPL>& rk) {
    float kv[CPL];
    rk.unpack(kv);
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) a = __fmaf_rn(s_qf[part * CPL + i], kv[i], a);
    return lane_group_sum<LPE>(a) * inv_sqrt_d;
  };
  float a0 = -INFINITY;
  {
    float am = -INFINITY;
    if (grp < n_ex) am = a0 = ex_score(xk);
    for (int j = grp + NGR; j < n_ex; j += NGR) {   // more exact rows than groups
      RawPiece<KT, CPL> rk;
      rk.load(off32(kunit, ex_pos(j) * D + part * CPL));
      am = fmax_m3(am, ex_score(rk));
    }
    const uint32_t ka = wave_max_u32(ord_f32(am));
    if (lane == 0) atomicMax(&s_rng[2], ka);
  }
  __syncthreads();

  // ---- 4. the selection, the whole block (the exact fallback when it fails):
  //      the K selected into the LDS list (and to idx / sel when asked).  The
  //      reference for the exponentials: no score of the exact support exceeds
  //      the larger of the exact rows' maximum and the upper edge of the union's
  //      highest scan bin (the fallback's scores aside, which may pass it by an
  //      ulp)
  float mref = -INFINITY;
  {
    const float hi_edge = __fsub_rn(__fdiv_rn((float)s_bin_hi, hp.inv_w), hp.rg);
    mref = fmax_m3(unord_f32(s_rng[2]), hi_edge * inv_sqrt_d);
    SelOut io;
    if (idx_out != nullptr && rsl == 0) {
      io.io = idx_out + (size_t)ug * K;
      io.so = sc_out + (size_t)ug * K;
    }
    const bool ok = block_select<KT, D, NT>(es, ep, s_nE, sbin, s_bcs, s_nrep, n_chunks, ch, L_mid,
                                            n_sink, K, s_trunc != 0, hp, s_qf, kunit, inv_sqrt_d, wl,
                                            lpos, lsc, io);
    if (!ok) {   // uniform: a chunk withheld tokens or the band was too wide
      __syncthreads();
      SelOut out = io;
      out.lpos = lpos;
      out.lsc = lsc;
      exact_fallback<KT, D, NT>(s_qf, kunit, n_sink, L_mid, K, out, inv_sqrt_d, s_hist, s_misc, s_buf);
    }
  }
  __syncthreads();   // the list

  // the group's sums: N = sum e^{s - mref} v, Z = sum e^{s - mref} over the
  // exact support; NK = sum w v, ZK = sum w over the retrieved entries; mx =
  // the largest score added
  float N[CPL], NK[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) { N[c] = 0.f; NK[c] = 0.f; }
  float Z = 0.f, ZK = 0.f, mx = -INFINITY;
  auto add_exp = [&](float sc, const float (&vv)[CPL]) {
    const float ew = __expf(sc - mref);
#pragma unroll
    for (int c = 0; c < CPL; ++c) N[c] = __fmaf_rn(ew, vv[c], N[c]);
    Z += ew;
    mx = fmax_m3(mx, sc);
  };
  bool ex_due = grp < n_ex && rsl == 0;   // the group's first exact row (score a0, value row xv)
  // this block's slice of the list
  const int sl = n_split > 1 ? (K + n_split - 1) / n_split : K;
  const int j_lo = min(K, rsl * sl), j_hi = min(K, j_lo + sl);

  // ---- 5. retrieved entries from the list
  constexpr bool DOT2 = sizeof(PT) == 2;   // bf16 phi rows: w on the bf16 dot instruction
  float fr[DOT2 ? 1 : FPL];
  uint32_t fh[FPL / 2], fl[FPL / 2];
  if constexpr (DOT2) {
#pragma unroll
    for (int j = 0; j < FPL / 2; ++j) {
      fh[j] = sub ? s_fhl[0][part * (FPL / 2) + j] : 0u;
      fl[j] = sub ? s_fhl[1][part * (FPL / 2) + j] : 0u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < FPL; ++i) fr[i] = sub ? s_f[part * FPL + i] : 0.f;
  }
  // the first ng groups gather, entry jb + e ng in slot e, so that every slot
  // but a few of the last round holds an entry (an empty slot would still
  // issue its loads: the batch's load count is fixed)
  const int ng = min(NGR, (j_hi - j_lo + B - 1) / B);
  for (int jb = j_lo + grp; grp < ng && jb < j_hi; jb += ng * B) {
    RawPiece<KT, CPL> vr[B];
    RawPiece<PT, FPL> pr[B];
    float scs[B];
#pragma unroll
    for (int e = 0; e < B; ++e) {
      const int jj = jb + e * ng;
      const int jc = jj < j_hi ? jj : jb;
      const int pos = min(max(lpos[jc], n_sink), n_sink + max(L_mid, 1) - 1);
      scs[e] = lsc[jc];
      vr[e].load(off32(vunit, pos * D + part * CPL));
      if (sub) pr[e].load(off32(phiu, (pos - n_sink) * M + part * FPL));
      else pr[e].zero();
    }
    __builtin_amdgcn_sched_barrier(0);   // every load issued before any use
    if (ex_due) {   // uniform within the group; added while the batch loads
      float vv[CPL];
      xv.unpack(vv);
      add_exp(a0, vv);
      ex_due = false;
    }
#pragma unroll
    for (int e = 0; e < B; ++e) {
      if (jb + e * ng < j_hi) {  // uniform within the group; a wave skips its empty slots
        float vv[CPL];
        float w = 0.f;
        if constexpr (DOT2) {
          w = dot_phi_bf16<FPL>(pr[e], fh, fl);
        } else {
          float ph[FPL];
          pr[e].unpack(ph);
#pragma unroll
          for (int i = 0; i < FPL; ++i) w = __fmaf_rn(fr[i], ph[i], w);
        }
        w = lane_group_sum<LPE>(w);
        vr[e].unpack(vv);
        add_exp(scs[e], vv);
#pragma unroll
        for (int c = 0; c < CPL; ++c) NK[c] = __fmaf_rn(w, vv[c], NK[c]);
        ZK += w;
      }
    }
  }
  if (ex_due) {
    float vv[CPL];
    xv.unpack(vv);
    add_exp(a0, vv);
  }
  for (int j = grp + NGR; rsl == 0 && j < n_ex; j += NGR) {   // more exact rows than groups
    const int pos = ex_pos(j);
    xv.load(off32(vunit, pos * D + part * CPL));
    xk.load(off32(kunit, pos * D + part * CPL));
    const float sc = ex_score(xk);
    float vv[CPL];
    xv.unpack(vv);
    add_exp(sc, vv);
  }

  // ---- 6. combine: the two groups of a 16-lane row add (row rotation by 8);
  //      the pair sums go to the union's LDS (no longer read once the list is
  //      complete, so no wait for the other waves) and are added in pair order
  //      (deterministic); Z and sum w per wave (its four rows in order); the
  //      largest score added, per wave
  {
    const uint32_t km = wave_max_u32(ord_f32(mx));
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      N[c] += dpp_f<0x128>(N[c]);      // row_ror:8: the other group of the row
      NK[c] += dpp_f<0x128>(NK[c]);
    }
    Z += dpp_f<0x128>(Z);
    ZK += dpp_f<0x128>(ZK);
    // read out of lanes 0, 16, 32, 48 by the whole wave (inside a lane-0 branch
    // the compiler could leave the row additions above to lane 0 alone)
    const float zw = (readlane_f(Z, 0) + readlane_f(Z, 16)) + (readlane_f(Z, 32) + readlane_f(Z, 48));
    const float zkw = (readlane_f(ZK, 0) + readlane_f(ZK, 16)) + (readlane_f(ZK, 32) + readlane_f(ZK, 48));
    if (lane == 0) {
      atomicMax(&s_rng[3], km);
      s_zw[wave][0] = zw;
      s_zw[wave][1] = zkw;
    }
    if ((lane & 15) < LPE) {
      float* rp = red + (size_t)(wave * 4 + (lane >> 4)) * NVS;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        rp[part * CPL + c] = N[c];
        rp[D + part * CPL + c] = NK[c];
      }
    }
  }
  __syncthreads();
  for (int j0 = 0; j0 < NV; j0 += NT / 8) {
    const int j = j0 + tid / 8, sl = tid % 8;
    float acc = 0.f;
    if (j < NV) {
      for (int pp = sl; pp < NP; pp += 8) acc += red[(size_t)pp * NVS + j];
    }
    acc = lane_group_sum<8>(acc);
    if (sl == 0 && j < NV) s_fin[j] = acc;
  }
  if (wave == NW - 1) {   // Z and sum w over the waves: lanes 0.. and 16.. in a fixed butterfly
    static_assert(NW <= 16, "one wave's sums per lane of a 16-lane row");
    const int wv = lane & 15, which = lane >> 4;
    float z = (which < 2 && wv < NW) ? s_zw[wv][which] : 0.f;
    z = lane_group_sum<16>(z);
    if (lane == 0) s_fin[NV] = z;
    if (lane == 16) s_fin[NV + 1] = z;
  }
  __syncthreads();
  const float ms = unord_f32(s_rng[3]);   // m*: the largest score of the exact support
  const float ZE = s_fin[NV], ZKt = s_fin[NV + 1];
  const float uf = rs ? s_uf : 0.f;
  if (n_split > 1) {
    // this slice's partial in merge_kernel's layout (m, Z_E, sum w, u^T f, N_E,
    // sum w v, phi(q)^T S), Z_E and N_E taken relative to m = the largest score
    // this block added
    constexpr int PFL = 4 + 3 * D;
    float* pp = sparts + ((size_t)ug * n_split + rsl) * PFL;
    const float sc = ms == -INFINITY ? 0.f : __expf(mref - ms);
    if (tid == 0) {
      pp[0] = ms;
      pp[1] = ZE * sc;
      pp[2] = ZKt;
      pp[3] = uf;
    }
    for (int col = tid; col < D; col += NT) {
      float fs = 0.f;
      if (rs) {
#pragma unroll
        for (int k = 0; k < FB; ++k) fs += s_part[k][col];
      }
      pp[4 + col] = s_fin[col] * sc;
      pp[4 + D + col] = s_fin[D + col];
      pp[4 + 2 * D + col] = fs;
    }
    return;
  }
  float zr = 0.f;
  if (rs) zr = fmaxf(uf - (sub ? ZKt : 0.f), 0.f);
  // y = (N_E + e^{-mref} nu) / (Z_E + e^{-mref} Z_R) with N_E, Z_E taken
  // relative to mref, scaled by e^{mref - Mx} with Mx = max(mref, log Z_R) so
  // that neither term overflows
  const float lz = zr > 0.f ? __logf(zr) : -INFINITY;
  const float Mx = fmaxf(mref, lz);
  const float a = __expf(mref - Mx);
  const float bres = __expf(-Mx);
  const float den = a * ZE + bres * zr;
  for (int col = tid; col < D; col += NT) {
    float nu = 0.f;
    if (rs) {
      float fs = 0.f;
#pragma unroll
      for (int k = 0; k < FB; ++k) fs += s_part[k][col];
      nu = fs - (sub ? s_fin[D + col] : 0.f);
    }
    y[(size_t)ug * D + col] = (a * s_fin[col] + bres * nu) / den;
  }
  if (stats != nullptr && tid == 0) {
    stats[(size_t)ug * 4 + 0] = ms;
    stats[(size_t)ug * 4 + 1] = ZE * __expf(mref - ms);   // relative to m*
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
  const size_t lds = fused_dyn_bytes(tp.n_chunks, tp.r_cap, K, D, NT);
  // the plan checked the fit; a launch that would not fit is refused here too
  if (lds + kernel_static_lds<&decode_fused_kernel<KT, PT, D, M, NT>>() > device_info().lds_per_block)
    return hipErrorInvalidConfiguration;
  const int ns = pl.fused_split;
  float* parts = reinterpret_cast<float*>(ws + pl.off_fpart);
  const int heads = (int)(kv.n_units * G);
  hipError_t e = launch_kernel(
      "decode_fused_kernel", kern, dim3(kv.n_units, G, ns), dim3(NT), (uint32_t)lds, st,
      reinterpret_cast<const float4*>(ws + tp.off_hp), reinterpret_cast<const int2*>(ws + tp.off_meta),
      reinterpret_cast<const float2*>(ws + tp.off_ent), q, Wq, G, tp.n_chunks, tp.r_cap, P,
      static_cast<const KT*>(kv.k), static_cast<const KT*>(kv.v), kv.unit_stride, (int)sp.L, sp.n_sink,
      sp.n_tail, (int)sp.n_gen, L_mid, tp.ch, K, idx, sel, phi_q, bq,
      static_cast<const PT*>(phi_k), S, u, flags, y, stats, 1.0f / sqrtf((float)D), ns, parts);
  if (e != hipSuccess || ns == 1) return e;
  return launch_merge_combine(parts, ns, heads, D, flags, K, L_mid, y, stats, st);
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
