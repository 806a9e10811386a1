// Full exact decode attention over the whole context and the diagnostics that
// compare the method with it ("Residual-Mass Accounting for Partial-KV
// Decoding": §3 Eq. 1 for full attention, the residual definitions before
// Eq. 5 for R(q) = M minus K(q); §6 for the mid-region entropy H_mid; §7.1
// Table 3 for the relative l1 error and the residual log-partition error).
//
// full_partial  grid (chunks, units), 256 threads.  Streams the K and V rows of
//   one chunk of positions [0, L + n_gen) once for all G query heads of the
//   unit (range-checked buffer loads, two tiles in flight).  Scoring lanes:
//   16 key elements per lane, d/16 lanes per token, fp32 FMA, DPP sums; the
//   scaled scores go to LDS.  Value lanes: 8 columns per lane, d/8 lanes per
//   row; each lane keeps, per head, its own running max m and
//     Z = sum e^{s-m},  N = sum e^{s-m} v,  Z_M, T_M = sum_M e^{s-m} (s-m),
//     Z_R = sum_{M minus K(q)} e^{s-m}
//   over the rows it reads; lanes and waves are then combined with max
//   rescaling into one record per (unit, chunk, head).
// full_combine  grid (units * G), 256 threads: combines the chunk records with
//   a fixed order, writes y_full = N / Z and the diagnostics.
#include "rma_device.hpp"
#include "rma_internal.hpp"

#include <math.h>

namespace rma {

namespace {

// Running sums of one head over a set of rows, relative to the running max m.
struct Acc {
  float m, z, zm, tm, zr;
};

// Merges b into a (both relative to their own maxima).  T_M moves with the
// shift: sum e^{s-M}(s-M) = e^{m-M} (T + (m-M) Z_M).
__device__ __forceinline__ void acc_merge(Acc& a, const Acc& b, float& sa, float& sb) {
  const float M = fmaxf(a.m, b.m);
  sa = a.m == M ? 1.f : __expf(a.m - M);
  sb = b.m == M ? 1.f : __expf(b.m - M);
  const float da = a.m == -INFINITY ? 0.f : a.m - M;
  const float db = b.m == -INFINITY ? 0.f : b.m - M;
  a.tm = sa * (a.tm + da * a.zm) + sb * (b.tm + db * b.zm);
  a.z = sa * a.z + sb * b.z;
  a.zm = sa * a.zm + sb * b.zm;
  a.zr = sa * a.zr + sb * b.zr;
  a.m = M;
}

}  // namespace

template <typename KT, int D, int G, bool MEMB>
__global__ void __launch_bounds__(kFullThreads)
full_partial_kernel(const float* __restrict__ q, const KT* __restrict__ kb,
                    const KT* __restrict__ vb, int64_t ustride, int L, int n_sink, int n_tail,
                    int T_all, int ch, int n_chunks, const int32_t* __restrict__ idx, int K,
                    float* __restrict__ part, float inv_sqrt_d) {
  constexpr int NT = kFullThreads, NW = NT / kWave;
  constexpr int E = 16, LPT = D / E, TPW = kWave / LPT, TT = NW * TPW;   // scoring layout
  constexpr int CPL = 8, LPR = D / CPL, RPW = kWave / LPR, RPP = NW * RPW;  // value layout
  constexpr int VPT = TT / RPP;                          // value rows per lane per tile
  constexpr int KPC = E * (int)sizeof(KT) / 16;          // 16-byte key pieces per lane
  constexpr int VPC = CPL * (int)sizeof(KT) / 16;        // 16-byte value pieces per row
  constexpr int EPP = 16 / (int)sizeof(KT);              // elements per piece
  constexpr int WPB = kFullMaxChunk / 32;                // membership words per head
  constexpr int REC = kFullRecHead + D;
  static_assert(VPT >= 1 && TT % RPP == 0, "tile shape");

  __shared__ float s_sc[2][G][TT];
  __shared__ uint32_t s_bits[MEMB ? G : 1][MEMB ? WPB : 1];
  __shared__ int s_samp[MEMB ? G : 1][MEMB ? NT : 1];
  __shared__ int s_rng[MEMB ? G : 1][2];
  __shared__ float s_wst[NW][G][5];
  __shared__ float s_wn[NW][G][D];

  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const int kpart = lane % LPT, kslot = lane / LPT;
  const int cg = lane % LPR, rg = lane / LPR;
  const int t0 = c * ch;
  const int n = min(ch, T_all - t0);
  const int mid_lo = n_sink, mid_hi = L - n_tail;

  // range-checked views of the chunk: rows past its end load as zeros without a
  // memory access, so every pass issues the same loads
  const size_t base = (size_t)u * ustride + (size_t)t0 * D;
  const uint32_t bytes = (uint32_t)((size_t)n * D * sizeof(KT));
  const auto rk = make_rsrc(kb + base, bytes), rv = make_rsrc(vb + base, bytes);
  auto load = [&](uint4 (&kr)[KPC], uint4 (&vr)[VPT][VPC], int tok0) {
    const uint32_t ko = (uint32_t)(((tok0 + wave * TPW + kslot) * D + kpart * E) * sizeof(KT));
#pragma unroll
    for (int pc = 0; pc < KPC; ++pc) kr[pc] = buf_ld16_nt(rk, ko + 16 * pc);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const uint32_t vo =
          (uint32_t)(((tok0 + j * RPP + wave * RPW + rg) * D + cg * CPL) * sizeof(KT));
#pragma unroll
      for (int pc = 0; pc < VPC; ++pc) vr[j][pc] = buf_ld16_nt(rv, vo + 16 * pc);
    }
  };
  uint4 kA[KPC], vA[VPT][VPC], kB[KPC], vB[VPT][VPC];
  load(kA, vA, 0);
  load(kB, vB, TT);

  // query slices of every head (scoring lanes hold E elements of each)
  float qr[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float4* qp = reinterpret_cast<const float4*>(q + ((size_t)u * G + g) * D + kpart * E);
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const float4 v = qp[i];
      qr[g][4 * i] = v.x; qr[g][4 * i + 1] = v.y; qr[g][4 * i + 2] = v.z; qr[g][4 * i + 3] = v.w;
    }
  }

  // membership of K(q) inside this chunk, one bit per position and head:
  // evenly spaced samples of each (ascending) index list bracket the entries
  // that can fall in [t0, t0 + n); only those are read
  if constexpr (MEMB) {
    for (int i = tid; i < G * WPB; i += NT) (&s_bits[0][0])[i] = 0u;
#pragma unroll
    for (int g = 0; g < G; ++g)
      s_samp[g][tid] = idx[((size_t)u * G + g) * K + min(K - 1, (int)(((int64_t)tid * K) / NT))];
    __syncthreads();
    if (tid < 2 * G) {
      const int g = tid >> 1, key = (tid & 1) ? t0 + n : t0;
      int lo = 0, hi = NT;  // first sample >= key
      while (lo < hi) {
        const int mdl = (lo + hi) >> 1;
        if (s_samp[g][mdl] < key) lo = mdl + 1; else hi = mdl;
      }
      // sample i sits at index min(K-1, i*K/NT); entries before the sample
      // below t0 are below t0, entries from the sample at or past t0+n are past it
      int j;
      if (tid & 1) j = lo == NT ? K : min(K - 1, (int)(((int64_t)lo * K) / NT));
      else j = lo == 0 ? 0 : min(K - 1, (int)(((int64_t)(lo - 1) * K) / NT));
      s_rng[g][tid & 1] = j;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int32_t* ig = idx + ((size_t)u * G + g) * K;
      for (int j = s_rng[g][0] + tid; j < s_rng[g][1]; j += NT) {
        const int p = ig[j] - t0;
        if (p >= 0 && p < n) atomicOr(&s_bits[g][p >> 5], 1u << (p & 31));
      }
    }
  }
  // the first two tiles are complete before the loop, so the wait before each
  // tile in the loop covers only that tile's loads
  __syncthreads();
  __builtin_amdgcn_s_waitcnt(0x0F70);

  Acc ac[G];
  float nv[G][CPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    ac[g] = Acc{-INFINITY, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < CPL; ++e) nv[g][e] = 0.f;
  }

  auto process = [&](const uint4 (&kr)[KPC], const uint4 (&vr)[VPT][VPC], int tok0, int buf) {
    // scores of this tile -> LDS (-inf past the chunk)
    {
      float kv[E];
#pragma unroll
      for (int pc = 0; pc < KPC; ++pc) unpack_piece(kr[pc], (const KT*)nullptr, kv + pc * EPP);
      const int tl = wave * TPW + kslot;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) a = __fmaf_rn(qr[g][e], kv[e], a);
        a = lane_group_sum<LPT>(a);
        if ((g % LPT) == kpart) s_sc[buf][g][tl] = (tok0 + tl < n) ? a * inv_sqrt_d : -INFINITY;
      }
    }
    __syncthreads();
    // values: this lane's rows of the tile, every head
    float v[VPT][CPL];
    bool mid[VPT], inr[VPT];
    int rl[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
#pragma unroll
      for (int pc = 0; pc < VPC; ++pc) unpack_piece(vr[j][pc], (const KT*)nullptr, v[j] + pc * EPP);
      rl[j] = j * RPP + wave * RPW + rg;
      const int pos = t0 + tok0 + rl[j];
      inr[j] = tok0 + rl[j] < n;
      mid[j] = inr[j] && pos >= mid_lo && pos < mid_hi;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s[VPT];
      float mn = ac[g].m;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        s[j] = s_sc[buf][g][rl[j]];
        mn = fmaxf(mn, s[j]);
      }
      if (mn > ac[g].m) {
        const float r = __expf(ac[g].m - mn);  // 0 while nothing is accumulated
        ac[g].tm = ac[g].m == -INFINITY ? 0.f : r * (ac[g].tm + (ac[g].m - mn) * ac[g].zm);
        ac[g].z *= r;
        ac[g].zm *= r;
        ac[g].zr *= r;
#pragma unroll
        for (int e = 0; e < CPL; ++e) nv[g][e] *= r;
        ac[g].m = mn;
      }
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const float p = inr[j] ? __expf(s[j] - mn) : 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) nv[g][e] = __fmaf_rn(p, v[j][e], nv[g][e]);
        ac[g].z += p;
        if (mid[j]) {
          ac[g].zm += p;
          ac[g].tm = __fmaf_rn(p, s[j] - mn, ac[g].tm);
          bool ret = false;
          if constexpr (MEMB) {
            const int lp = tok0 + rl[j];
            ret = (s_bits[g][lp >> 5] >> (lp & 31)) & 1u;
          }
          if (!ret) ac[g].zr += p;
        }
      }
    }
  };

  for (int tok0 = 0; tok0 < n; tok0 += 2 * TT) {
    process(kA, vA, tok0, 0);
    load(kA, vA, tok0 + 2 * TT);
    process(kB, vB, tok0 + TT, 1);
    load(kB, vB, tok0 + 3 * TT);
  }

  // ---- lanes of a wave with the same columns hold different rows: combine them
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      Acc b;
      b.m = __shfl_xor(ac[g].m, o);
      b.z = __shfl_xor(ac[g].z, o);
      b.zm = __shfl_xor(ac[g].zm, o);
      b.tm = __shfl_xor(ac[g].tm, o);
      b.zr = __shfl_xor(ac[g].zr, o);
      float sa, sb;
      acc_merge(ac[g], b, sa, sb);
#pragma unroll
      for (int e = 0; e < CPL; ++e) nv[g][e] = sa * nv[g][e] + sb * __shfl_xor(nv[g][e], o);
    }
  }
  if (rg == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < CPL; ++e) s_wn[wave][g][cg * CPL + e] = nv[g][e];
      if (cg == 0) {
        s_wst[wave][g][0] = ac[g].m;
        s_wst[wave][g][1] = ac[g].z;
        s_wst[wave][g][2] = ac[g].zm;
        s_wst[wave][g][3] = ac[g].tm;
        s_wst[wave][g][4] = ac[g].zr;
      }
    }
  }
  __syncthreads();
  // ---- the waves, in wave order: thread (g, column) for the sums of N
  float* rec0 = part + (((size_t)u * n_chunks + c) * G) * REC;
  for (int i = tid; i < G * D; i += NT) {
    const int g = i / D, col = i - g * D;
    Acc a{s_wst[0][g][0], s_wst[0][g][1], s_wst[0][g][2], s_wst[0][g][3], s_wst[0][g][4]};
    float nn = s_wn[0][g][col];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const Acc b{s_wst[w][g][0], s_wst[w][g][1], s_wst[w][g][2], s_wst[w][g][3], s_wst[w][g][4]};
      float sa, sb;
      acc_merge(a, b, sa, sb);
      nn = sa * nn + sb * s_wn[w][g][col];
    }
    float* rec = rec0 + (size_t)g * REC;
    rec[kFullRecHead + col] = nn;
    if (col == 0) {
      rec[0] = a.m;
      rec[1] = a.z;
      rec[2] = a.zm;
      rec[3] = a.tm;
      rec[4] = a.zr;
    }
  }
}

// One block per (unit, head).  The maximum over the chunk records comes first
// (every thread a stride of chunks, then a block max), so every record's scale
// is known before its sums are read; then NT/D groups of threads take every
// (NT/D)-th chunk (record loads issued in batches of eight) and the group sums
// are added in group order.
template <int D>
__global__ void __launch_bounds__(kFullCombineThreads)
full_combine_kernel(const float* __restrict__ part, int G, int n_chunks, int L_mid, int resid_mode,
                    const float* __restrict__ y_cmp, float* __restrict__ y_full,
                    float* __restrict__ diag) {
  constexpr int NT = kFullCombineThreads, NWV = NT / kWave;
  constexpr int REC = kFullRecHead + D, CG = NT / D, BT = 8;
  __shared__ float s_red[NWV];
  __shared__ float s_nn[CG][D];
  __shared__ float s_st[CG][4];
  __shared__ float s_l1[NWV][2];
  const int ug = blockIdx.x, u = ug / G, g = ug - u * G, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const int col = tid % D, grp = tid / D;
  const float* rec0 = part + ((size_t)u * n_chunks * G + g) * REC;
  const size_t cstride = (size_t)G * REC;
  float M = -INFINITY;
  for (int c = tid; c < n_chunks; c += NT) M = fmaxf(M, rec0[(size_t)c * cstride]);
  M = wave_max_dpp(M);
  if (lane == 0) s_red[wave] = M;
  __syncthreads();
  M = s_red[0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) M = fmaxf(M, s_red[w]);
  // sums relative to M; T_M moves with each record's shift
  float z = 0.f, zm = 0.f, tm = 0.f, zr = 0.f, nn = 0.f;
  for (int c0 = grp; c0 < n_chunks; c0 += CG * BT) {
    float r[BT][5], rn[BT];
#pragma unroll
    for (int i = 0; i < BT; ++i) {
      const float* rc = rec0 + (size_t)min(c0 + i * CG, n_chunks - 1) * cstride;
#pragma unroll
      for (int j = 0; j < 5; ++j) r[i][j] = rc[j];
      rn[i] = rc[kFullRecHead + col];
    }
#pragma unroll
    for (int i = 0; i < BT; ++i) {
      if (c0 + i * CG < n_chunks) {
        const bool live = r[i][0] != -INFINITY;
        const float sc = live ? __expf(r[i][0] - M) : 0.f;
        const float dm = live ? r[i][0] - M : 0.f;
        z = __fmaf_rn(sc, r[i][1], z);
        tm = __fmaf_rn(sc, r[i][3] + dm * r[i][2], tm);
        zm = __fmaf_rn(sc, r[i][2], zm);
        zr = __fmaf_rn(sc, r[i][4], zr);
        nn = __fmaf_rn(sc, rn[i], nn);
      }
    }
  }
  s_nn[grp][col] = nn;
  if (col == 0) {
    s_st[grp][0] = z;
    s_st[grp][1] = zm;
    s_st[grp][2] = tm;
    s_st[grp][3] = zr;
  }
  __syncthreads();
  z = 0.f, zm = 0.f, tm = 0.f, zr = 0.f, nn = 0.f;
#pragma unroll
  for (int k = 0; k < CG; ++k) {
    nn += s_nn[k][col];
    z += s_st[k][0];
    zm += s_st[k][1];
    tm += s_st[k][2];
    zr += s_st[k][3];
  }
  const float yv = nn / z;
  float dl1 = 0.f, rl1 = 0.f;
  if (tid < D) {
    y_full[(size_t)ug * D + tid] = yv;
    if (y_cmp != nullptr) {
      dl1 = fabsf(y_cmp[(size_t)ug * D + tid] - yv);
      rl1 = fabsf(yv);
    }
  }
  if (diag == nullptr) return;
  dl1 = wave_sum_dpp(dl1);
  rl1 = wave_sum_dpp(rl1);
  if (lane == 0) {
    s_l1[wave][0] = dl1;
    s_l1[wave][1] = rl1;
  }
  __syncthreads();
  if (tid == 0) {
    float sd = 0.f, sr = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) { sd += s_l1[w][0]; sr += s_l1[w][1]; }
    float* dg = diag + (size_t)ug * 8;
    const float lzm = zm > 0.f ? M + logf(zm) : -INFINITY;
    dg[0] = M + logf(z);
    dg[1] = lzm;
    dg[2] = resid_mode == 0 ? NAN : (zr > 0.f ? M + logf(zr) : -INFINITY);
    dg[3] = (L_mid >= 2 && zm > 0.f) ? (logf(zm) - tm / zm) / logf((float)L_mid) : NAN;
    dg[4] = y_cmp != nullptr ? sd / sr : NAN;
    dg[5] = M;
    dg[6] = 0.f;
    dg[7] = 0.f;
  }
}

// ---------------------------------------------------------------- launcher
template <typename KT, int D>
static hipError_t launch_full_t(const FullPlan& pl, const float* q, int G, const rma_kv& kv,
                                const rma_span& sp, const int32_t* idx, int K, const float* y_cmp,
                                float* y, float* diag, uint8_t* ws, hipStream_t st) {
  const KT* kb = static_cast<const KT*>(kv.k);
  const KT* vb = static_cast<const KT*>(kv.v);
  float* part = reinterpret_cast<float*>(ws + pl.off_part);
  const float isd = 1.0f / sqrtf((float)D);
  const dim3 grid(pl.n_chunks, kv.n_units);
  const bool memb = idx != nullptr && K > 0;
  const int T_all = (int)(sp.L + sp.n_gen);
  hipError_t e = hipSuccess;
#define RMA_FP(GG)                                                                                   \
  do {                                                                                               \
    if (memb)                                                                                        \
      e = launch_kernel("full_partial_kernel", full_partial_kernel<KT, D, GG, true>, grid,           \
                        dim3(kFullThreads), 0, st, q, kb, vb, kv.unit_stride, (int)sp.L, sp.n_sink,  \
                        sp.n_tail, T_all, pl.ch, pl.n_chunks, idx, K, part, isd);                    \
    else                                                                                             \
      e = launch_kernel("full_partial_kernel", full_partial_kernel<KT, D, GG, false>, grid,          \
                        dim3(kFullThreads), 0, st, q, kb, vb, kv.unit_stride, (int)sp.L, sp.n_sink,  \
                        sp.n_tail, T_all, pl.ch, pl.n_chunks, idx, K, part, isd);                    \
  } while (0)
  switch (G) {
    case 1: RMA_FP(1); break;
    case 2: RMA_FP(2); break;
    case 3: RMA_FP(3); break;
    case 4: RMA_FP(4); break;
    case 5: RMA_FP(5); break;
    case 6: RMA_FP(6); break;
    case 7: RMA_FP(7); break;
    default: RMA_FP(8); break;
  }
#undef RMA_FP
  if (e != hipSuccess) return e;
  const int L_mid = (int)(sp.L - sp.n_sink - sp.n_tail);
  // without a retrieved set (K == 0) the residual set is the whole mid-region
  const int resid_mode = (idx != nullptr || K == 0) ? 2 : 0;
  return launch_kernel("full_combine_kernel", full_combine_kernel<D>, dim3(kv.n_units * G),
                       dim3(kFullCombineThreads), 0, st, part, G, pl.n_chunks, L_mid, resid_mode,
                       y_cmp, y, diag);
}

hipError_t launch_full(const FullPlan& pl, const float* q, int G, const rma_kv& kv,
                       const rma_span& sp, const int32_t* idx, int K, const float* y_cmp,
                       float* y, float* diag, uint8_t* ws, hipStream_t st) {
  if (kv.dtype == RMA_BF16) {
    if (kv.d == 64) return launch_full_t<uint16_t, 64>(pl, q, G, kv, sp, idx, K, y_cmp, y, diag, ws, st);
    return launch_full_t<uint16_t, 128>(pl, q, G, kv, sp, idx, K, y_cmp, y, diag, ws, st);
  }
  if (kv.d == 64) return launch_full_t<float, 64>(pl, q, G, kv, sp, idx, K, y_cmp, y, diag, ws, st);
  return launch_full_t<float, 128>(pl, q, G, kv, sp, idx, K, y_cmp, y, diag, ws, st);
}

}  // namespace rma
