// Exhaustive Top-K over the mid-region for every query head ("Residual-Mass
// Accounting for Partial-KV Decoding", §1: exhaustive Top-K is the control
// selector fixing the exact support; §3 Eq. 3: K(q) is a K-subset of M).
//
// Ranking is by the exact real value of q.k_i, ties to the lower position.
//
// Two kernels:
//  scan   grid (chunks, units).  Streams each unit's K_mid rows once for all G
//         query heads (fp32 FMA on bf16/fp32 keys, d split over 4-8 lanes and
//         summed with DPP).  Scores stay in LDS; a linear-bin histogram per head
//         picks a per-chunk threshold so that at least r_min tokens pass, and
//         the passing tokens (score, position) are written in position order.
//  select grid (units * G).  Gathers the chunk reports, radix-selects the K-th
//         largest fp32 score t, proves that no chunk withheld a token within
//         the error band, keeps every token above t + 2.5*eps, resolves the
//         band [t - 2.5*eps, t + 2.5*eps] with double-double exact scores, and
//         writes the K positions in ascending order.
//         eps bounds |fl32(q.k) - q.k| for every mid token: the fp32 dot has at
//         most 19 roundings per product path, so |err| <= gamma_19 *
//         sum|q_j k_j| <= gamma_19 * |q|_2 * kappa, kappa >= max ||k_i||_2.
//         When a check fails (a chunk withheld tokens, the band is too wide,
//         too many entries) the block falls back to an exact radix select on
//         (double-double score, -position) over the whole mid-region.
#include "rma_device.hpp"
#include "rma_internal.hpp"

#include <algorithm>
#include <math.h>

namespace rma {

struct HeadParams {
  float rg;     // score range half-width |q|_2 * kappa used for binning
  float inv_w;  // bins per score unit
  float eps;    // bound on the fp32 scoring error of any mid token
};

// Identical in every kernel: a fixed sequential order and explicit roundings,
// so the scan and the select bin a score identically.
__device__ __forceinline__ HeadParams head_params(const float* qg, int D, float kappa) {
  float n2 = 0.f;
  for (int j = 0; j < D; ++j) n2 = __fmaf_rn(qg[j], qg[j], n2);
  const float qn = __fsqrt_rn(n2);
  const float kap = (kappa > 0.f && kappa < 3.0e38f) ? kappa : 0.f;
  HeadParams h;
  h.rg = fmaxf(__fmul_rn(qn, kap), 1e-30f);
  h.inv_w = __fdiv_rn((float)kScanBins, __fmul_rn(2.f, h.rg));
  // gamma_19 < 1.14e-6; 5e-6 leaves room for the roundings of |q| and kappa
  h.eps = __fmul_rn(5e-6f, __fmul_rn(qn, kap));
  return h;
}

__device__ __forceinline__ int lin_bin(float x, const HeadParams& h) {
  const float t = __fmul_rn(__fadd_rn(x, h.rg), h.inv_w);
  return (t >= 0.f) ? (int)fminf(t, (float)(kScanBins - 1)) : 0;  // monotone in x; NaN -> 0
}

// Block-wide exclusive scan of one int per thread (256 threads); returns the
// exclusive prefix, `total` receives the sum.  Uses `buf` (>= 256 ints).
__device__ __forceinline__ int block_excl_scan256(int v, int* buf, int& total) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  if (tid < kWave) {
    int a0 = buf[4 * tid], a1 = buf[4 * tid + 1], a2 = buf[4 * tid + 2], a3 = buf[4 * tid + 3];
    int ls = a0 + a1 + a2 + a3;
    int incl = wave_incl_scan(ls);
    int ex = incl - ls;
    buf[4 * tid] = ex;
    buf[4 * tid + 1] = ex + a0;
    buf[4 * tid + 2] = ex + a0 + a1;
    buf[4 * tid + 3] = ex + a0 + a1 + a2;
    if (tid == kWave - 1) buf[256] = incl;
  }
  __syncthreads();
  int r = buf[tid];
  total = buf[256];
  __syncthreads();
  return r;
}

// ====================================================================== scan
template <typename KT, int D, int G>
__global__ void __launch_bounds__(kScanThreads)
topk_scan_kernel(const float* __restrict__ q, const KT* __restrict__ kb, int64_t ustride,
                 int n_sink, int L_mid, int ch, int n_chunks, int r_min, int r_cap,
                 const float* __restrict__ kappa, float2* __restrict__ ent,
                 int2* __restrict__ meta) {
  constexpr int E = 16;              // key elements per lane
  constexpr int LPT = D / E;         // lanes per token (4 or 8)
  constexpr int TPW = kWave / LPT;   // tokens per wave pass
  constexpr int TPP = 4 * TPW;       // tokens per block pass
  constexpr int EPP = RowPieces<KT>::kElemsPerPiece;
  constexpr int PIECES = E / EPP;    // 16-byte loads per lane per token
  constexpr int UNR = (sizeof(KT) == 2) ? 4 : 2;
  constexpr int CHMAX = (kScanScoreSlots / G) / TPP * TPP;
  constexpr int NB = kScanBins;

  __shared__ float sc[G * CHMAX];
  __shared__ uint32_t hist[G * NB];
  __shared__ int s_buf[257];
  __shared__ HeadParams s_hp[G];
  __shared__ int s_bc[G], s_nrep[G];

  const int u = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const int part = lane % LPT, slot = lane / LPT;
  const int t0 = c * ch;
  const int n = min(ch, L_mid - t0);

  float qr[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float4* qp = reinterpret_cast<const float4*>(q + ((size_t)u * G + g) * D + part * E);
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      float4 v = qp[i];
      qr[g][4 * i] = v.x; qr[g][4 * i + 1] = v.y; qr[g][4 * i + 2] = v.z; qr[g][4 * i + 3] = v.w;
    }
  }
  if (tid < G) s_hp[tid] = head_params(q + ((size_t)u * G + tid) * D, D, kappa[u]);

  const KT* kp = kb + (size_t)u * ustride + (size_t)(n_sink + t0) * D + part * E;
  for (int p0 = 0; p0 < n; p0 += TPP * UNR) {
    uint4 raw[UNR][PIECES];
#pragma unroll
    for (int i = 0; i < UNR; ++i) {
      const int t = p0 + i * TPP + wave * TPW + slot;
      if (t < n) {
        const uint4* src = reinterpret_cast<const uint4*>(kp + (size_t)t * D);
#pragma unroll
        for (int pc = 0; pc < PIECES; ++pc) raw[i][pc] = ld_stream16(src + pc);
      } else {
#pragma unroll
        for (int pc = 0; pc < PIECES; ++pc) raw[i][pc] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < UNR; ++i) {
      const int t = p0 + i * TPP + wave * TPW + slot;
      float kv[E];
#pragma unroll
      for (int pc = 0; pc < PIECES; ++pc) unpack_piece(raw[i][pc], (const KT*)nullptr, kv + pc * EPP);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) a = __fmaf_rn(qr[g][e], kv[e], a);
        a = lane_group_sum<LPT>(a);
        if (t < n && (g % LPT) == part) sc[g * CHMAX + t] = a;
      }
    }
  }
  __syncthreads();

  // ---- per-head linear-bin histogram of this chunk's scores
  for (int i = tid; i < G * NB; i += kScanThreads) hist[i] = 0u;
  __syncthreads();
  for (int i = tid; i < n; i += kScanThreads) {
#pragma unroll
    for (int g = 0; g < G; ++g) atomicAdd(&hist[g * NB + lin_bin(sc[g * CHMAX + i], s_hp[g])], 1u);
  }
  __syncthreads();

  // ---- per head: smallest bin threshold that still passes >= min(r_min, n) tokens
  for (int g = wave; g < G; g += 4) {
    const int target = min(r_min, n);
    const uint32_t* h = hist + g * NB;
    int ls = 0;
#pragma unroll
    for (int j = 0; j < NB / kWave; ++j) ls += (int)h[lane * (NB / kWave) + j];
    const int incl = wave_incl_scan(ls);
    const int total = __shfl(incl, kWave - 1, kWave);
    const int suf = total - incl + ls;  // tokens in this lane's bins and above
    const unsigned long long ball = __ballot(suf >= target);
    const int lstar = 63 - __clzll((long long)ball);
    int bc = 0, run = 0;
    if (lane == lstar) {
      run = suf - ls;
      bc = lane * (NB / kWave);
      for (int j = NB / kWave - 1; j >= 0; --j) {
        run += (int)h[lane * (NB / kWave) + j];
        if (run >= target) { bc = lane * (NB / kWave) + j; break; }
      }
    }
    bc = __shfl(bc, lstar, kWave);
    run = __shfl(run, lstar, kWave);
    // lower the threshold to just above the highest non-empty bin below it: the
    // same tokens pass, and the select's completeness test is least strict
    int hb = -1;
#pragma unroll
    for (int j = 0; j < NB / kWave; ++j) {
      const int bin = lane * (NB / kWave) + j;
      if (bin < bc && h[bin] != 0u) hb = bin;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) hb = max(hb, __shfl_xor(hb, o, kWave));
    if (lane == 0) { s_bc[g] = hb + 1; s_nrep[g] = run; }
  }
  __syncthreads();

  // ---- ordered compaction of the passing tokens (position order), per head
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
#pragma unroll 1
  for (int g = 0; g < G; ++g) {
    const HeadParams hp = s_hp[g];
    const int bc = s_bc[g];
    int cnt = 0;
    for (int i = i0; i < i1; ++i) cnt += (lin_bin(sc[g * CHMAX + i], hp) >= bc);
    int total;
    int pos = block_excl_scan256(cnt, s_buf, total);
    float2* dst = ent + ((size_t)(u * G + g) * n_chunks + c) * r_cap;
    for (int i = i0; i < i1; ++i) {
      const float s = sc[g * CHMAX + i];
      if (lin_bin(s, hp) >= bc) {
        if (pos < r_cap) dst[pos] = make_float2(s, __int_as_float(t0 + i));
        ++pos;
      }
    }
  }
  if (tid < G) meta[(size_t)(u * G + tid) * n_chunks + c] = make_int2(s_bc[tid], s_nrep[tid]);
}

// ====================================================================== select
// Exact fallback: radix select over the 160-bit key (ord(hi), ord(lo), ~pos)
// of the double-double score, recomputing keys from K on every pass.
template <typename KT, int D>
__device__ __forceinline__ void fb_key(const float* qf, const KT* kunit, int n_sink, int i,
                                       uint32_t (&w)[5], float& s32) {
  const DD dd = dd_dot<KT, D>(qf, kunit + (size_t)(n_sink + i) * D);
  const uint64_t a = ord_f64(dd.hi), b = ord_f64(dd.lo);
  w[0] = (uint32_t)(a >> 32); w[1] = (uint32_t)a;
  w[2] = (uint32_t)(b >> 32); w[3] = (uint32_t)b;
  w[4] = ~(uint32_t)i;
  s32 = (float)dd.hi;
}
__device__ __forceinline__ int fb_digit(const uint32_t (&w)[5], int p) {
  return (int)((w[p >> 2] >> (24 - 8 * (p & 3))) & 255u);
}
// compare the first nd digits of w with P: -1, 0, +1
__device__ __forceinline__ int fb_cmp(const uint32_t (&w)[5], const uint32_t (&P)[5], int nd) {
  for (int k = 0; k < 5; ++k) {
    const int left = nd - 4 * k;
    if (left <= 0) return 0;
    uint32_t msk = left >= 4 ? 0xffffffffu : ~(0xffffffffu >> (8 * left));
    uint32_t a = w[k] & msk, b = P[k] & msk;
    if (a != b) return a > b ? 1 : -1;
  }
  return 0;
}

// digit with the krem-th largest count from the top; returns (digit, count above)
__device__ __forceinline__ void find_digit(const uint32_t* hist, int krem, int* s_out) {
  const int tid = threadIdx.x;
  if (tid < kWave) {
    int c[4], ls = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) { c[j] = (int)hist[255 - 4 * tid - j]; ls += c[j]; }
    const int incl = wave_incl_scan(ls);
    const unsigned long long ball = __ballot(incl >= krem);
    const int lstar = __ffsll((long long)ball) - 1;
    if (tid == lstar) {
      int run = incl - ls;
      for (int j = 0; j < 4; ++j) {
        if (run + c[j] >= krem) { s_out[0] = 255 - 4 * tid - j; s_out[1] = run; s_out[2] = c[j]; break; }
        run += c[j];
      }
    }
  }
}

template <typename KT, int D>
__device__ void exact_fallback(const float* qf, const KT* kunit, int n_sink, int L_mid, int K,
                               int32_t* io, float* so, float inv_sqrt_d, uint32_t* hist,
                               int* s_misc, int* s_buf) {
  const int tid = threadIdx.x;
  uint32_t P[5] = {0u, 0u, 0u, 0u, 0u};
  int krem = K, nd = 0;
  for (int p = 0; p < 20; ++p) {
    hist[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < L_mid; i += 256) {
      uint32_t w[5];
      float s32;
      fb_key<KT, D>(qf, kunit, n_sink, i, w, s32);
      if (fb_cmp(w, P, p) == 0) atomicAdd(&hist[fb_digit(w, p)], 1u);
    }
    __syncthreads();
    find_digit(hist, krem, s_misc);
    __syncthreads();
    const int dig = s_misc[0], above = s_misc[1], cnt = s_misc[2];
    krem -= above;
    P[p >> 2] |= (uint32_t)dig << (24 - 8 * (p & 3));
    nd = p + 1;
    __syncthreads();
    if (cnt == krem) break;  // every key with this prefix is selected
  }
  // ordered compaction: selected iff the first nd digits are >= P
  const int per = (L_mid + 255) / 256;
  const int i0 = min(L_mid, tid * per), i1 = min(L_mid, i0 + per);
  int cnt = 0;
  for (int i = i0; i < i1; ++i) {
    uint32_t w[5];
    float s32;
    fb_key<KT, D>(qf, kunit, n_sink, i, w, s32);
    cnt += fb_cmp(w, P, nd) >= 0;
  }
  int total;
  int pos = block_excl_scan256(cnt, s_buf, total);
  for (int i = i0; i < i1; ++i) {
    uint32_t w[5];
    float s32;
    fb_key<KT, D>(qf, kunit, n_sink, i, w, s32);
    if (fb_cmp(w, P, nd) >= 0) {
      if (pos < K) { io[pos] = n_sink + i; so[pos] = s32 * inv_sqrt_d; }
      ++pos;
    }
  }
}

template <typename KT, int D>
__global__ void __launch_bounds__(256)
topk_select_kernel(const float* __restrict__ q, int G, const KT* __restrict__ kb, int64_t ustride,
                   int n_sink, int L_mid, int ch, int n_chunks, int r_cap, int K, int e_max,
                   const float* __restrict__ kappa, const float2* __restrict__ ent,
                   const int2* __restrict__ meta, int32_t* __restrict__ idx_out,
                   float* __restrict__ sc_out, float inv_sqrt_d) {
  extern __shared__ __align__(16) float es[];  // e_max fp32 scores of the union
  __shared__ int s_off[kSelMaxChunks + 1];
  __shared__ int s_bcs[kSelMaxChunks];
  __shared__ int s_nrep[kSelMaxChunks];
  __shared__ uint32_t hist[256];
  __shared__ int s_buf[257];
  __shared__ int s_misc[8];
  __shared__ DD s_bdd[kSelBandMax];
  __shared__ int s_bpos[kSelBandMax];
  __shared__ int s_bmid[kSelBandMax];
  __shared__ float s_qf[128];
  __shared__ HeadParams s_hp;

  const int ug = blockIdx.x, u = ug / G, tid = threadIdx.x;
  const float* qg = q + (size_t)ug * D;
  const int2* mt = meta + (size_t)ug * n_chunks;
  const float2* en = ent + (size_t)ug * n_chunks * r_cap;
  int32_t* io = idx_out + (size_t)ug * K;
  float* so = sc_out + (size_t)ug * K;
  const KT* kunit = kb + (size_t)u * ustride;

  if (tid == 0) s_hp = head_params(qg, D, kappa[u]);
  if (tid < D) s_qf[tid] = qg[tid];
  if (tid == 0) {
    int off = 0, trunc = 0;
    for (int c = 0; c < n_chunks; ++c) {
      const int2 mm = mt[c];
      if (mm.y > r_cap) trunc = 1;
      s_off[c] = off;
      s_bcs[c] = mm.x;
      s_nrep[c] = mm.y;
      off += min(mm.y, r_cap);
    }
    s_off[n_chunks] = off;
    s_misc[7] = trunc;
  }
  __syncthreads();
  const int nE = s_off[n_chunks];

  if (K == L_mid) {  // every mid token is selected; the chunks reported all of them in order
    for (int c = 0; c < n_chunks; ++c) {
      const int o = s_off[c], w = s_off[c + 1] - o;
      for (int j = tid; j < w; j += 256) {
        const float2 e = en[(size_t)c * r_cap + j];
        io[o + j] = n_sink + __float_as_int(e.y);
        so[o + j] = e.x * inv_sqrt_d;
      }
    }
    return;
  }

  bool fallback = s_misc[7] != 0 || nE > e_max || nE < K;
  float th_lo = 0.f, th_hi = 0.f;
  if (!fallback) {
    for (int c = 0; c < n_chunks; ++c) {
      const int o = s_off[c], w = s_off[c + 1] - o;
      for (int j = tid; j < w; j += 256) es[o + j] = en[(size_t)c * r_cap + j].x;
    }
    __syncthreads();
    // radix select of the K-th largest score (ordered 32-bit key, 8-bit digits)
    uint32_t prefix = 0u, mask = 0u;
    int krem = K;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[tid] = 0u;
      __syncthreads();
      for (int i = tid; i < nE; i += 256) {
        const uint32_t k = ord_f32(es[i]);
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      find_digit(hist, krem, s_misc);
      __syncthreads();
      krem -= s_misc[1];
      prefix |= (uint32_t)s_misc[0] << shift;
      mask |= 255u << shift;
      __syncthreads();
    }
    const float tt = unord_f32(prefix);
    const HeadParams hp = s_hp;
    th_lo = tt - 2.5f * hp.eps;
    th_hi = tt + 2.5f * hp.eps;
    // every chunk must have reported all of its tokens scoring >= th_lo
    const int blo = lin_bin(th_lo, hp);
    int bad = 0;
    for (int c = tid; c < n_chunks; c += 256) {
      const int n_c = min(ch, L_mid - c * ch);
      if (s_nrep[c] != n_c && s_bcs[c] > blo) bad = 1;
    }
    fallback = __syncthreads_or(bad) != 0;
  }
  if (!fallback) {
    if (tid == 0) { s_misc[3] = 0; s_misc[4] = 0; }
    __syncthreads();
    int nin = 0;
    for (int i = tid; i < nE; i += 256) {
      const float s = es[i];
      if (s > th_hi) {
        ++nin;
      } else if (s >= th_lo) {
        const int b = atomicAdd(&s_misc[4], 1);
        if (b < kSelBandMax) s_bpos[b] = i;
      }
    }
    atomicAdd(&s_misc[3], nin);
    __syncthreads();
    const int n_in = s_misc[3], n_band = s_misc[4];
    const int kp = K - n_in;
    if (n_band > kSelBandMax || kp < 1 || n_band < kp) {
      fallback = true;
    } else {
      // band members: mid position and (if the band must be split) exact score
      for (int b = tid; b < n_band; b += 256) {
        const int i = s_bpos[b];
        int lo = 0, hi = n_chunks - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_off[mid] <= i) lo = mid; else hi = mid - 1;
        }
        const int pos = __float_as_int(en[(size_t)lo * r_cap + (i - s_off[lo])].y);
        s_bmid[b] = pos;
        if (n_band > kp) s_bdd[b] = dd_dot<KT, D>(s_qf, kunit + (size_t)(n_sink + pos) * D);
      }
      __syncthreads();
      // rank within the band by (exact score desc, position asc); mark in es
      for (int b = tid; b < n_band; b += 256) {
        bool take = true;
        if (n_band > kp) {
          int rank = 0;
          const DD mine = s_bdd[b];
          const int mp = s_bmid[b];
          for (int b2 = 0; b2 < n_band; ++b2) rank += dd_key_greater(s_bdd[b2], s_bmid[b2], mine, mp);
          take = rank < kp;
        }
        es[s_bpos[b]] = take ? __int_as_float(0x7f800000) : __int_as_float(0xff800000);
      }
      __syncthreads();
      // ordered compaction of the selected entries (es > th_hi) in position order
      const int per = (nE + 255) / 256;
      const int i0 = min(nE, tid * per), i1 = min(nE, i0 + per);
      int cnt = 0;
      for (int i = i0; i < i1; ++i) cnt += es[i] > th_hi;
      int total;
      int pos = block_excl_scan256(cnt, s_buf, total);
      if (total != K) {
        fallback = true;  // uniform: every thread sees the same total
      } else if (i0 < i1) {
        int c = 0;
        {
          int lo = 0, hi = n_chunks - 1;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= i0) lo = mid; else hi = mid - 1;
          }
          c = lo;
        }
        for (int i = i0; i < i1; ++i) {
          while (s_off[c + 1] <= i) ++c;
          if (es[i] > th_hi) {
            const float2 e = en[(size_t)c * r_cap + (i - s_off[c])];
            io[pos] = n_sink + __float_as_int(e.y);
            so[pos] = e.x * inv_sqrt_d;
            ++pos;
          }
        }
      }
    }
  }
  if (fallback) {
    __syncthreads();
    exact_fallback<KT, D>(s_qf, kunit, n_sink, L_mid, K, io, so, inv_sqrt_d, hist, s_misc, s_buf);
  }
}

// ====================================================================== launch
namespace {

size_t g_lds_limit = 0;

template <typename KT, int D>
hipError_t launch_scan_g(int G, dim3 grid, hipStream_t st, const float* q, const KT* kb,
                         int64_t ustride, int n_sink, int L_mid, const TopkPlan& pl,
                         const float* kappa, float2* ent, int2* meta) {
#define RMA_SCAN_CASE(GG)                                                                     \
  case GG:                                                                                    \
    hipLaunchKernelGGL((topk_scan_kernel<KT, D, GG>), grid, dim3(kScanThreads), 0, st, q, kb, \
                       ustride, n_sink, L_mid, pl.ch, pl.n_chunks, pl.r_min, pl.r_cap, kappa, \
                       ent, meta);                                                            \
    break;
  switch (G) {
    RMA_SCAN_CASE(1) RMA_SCAN_CASE(2) RMA_SCAN_CASE(3) RMA_SCAN_CASE(4)
    RMA_SCAN_CASE(5) RMA_SCAN_CASE(6) RMA_SCAN_CASE(7) RMA_SCAN_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef RMA_SCAN_CASE
  return hipGetLastError();
}

template <typename KT, int D>
hipError_t launch_topk_t(const TopkPlan& pl, const float* q, int G, const rma_kv& kv,
                         const rma_span& sp, const float* kappa, int K, int32_t* idx,
                         float* sel, uint8_t* ws, hipStream_t st) {
  const int L_mid = (int)(sp.L - sp.n_sink - sp.n_tail);
  const KT* kb = static_cast<const KT*>(kv.k);
  float2* ent = reinterpret_cast<float2*>(ws + pl.off_ent);
  int2* meta = reinterpret_cast<int2*>(ws + pl.off_meta);
  hipError_t e = launch_scan_g<KT, D>(G, dim3(pl.n_chunks, kv.n_units), st, q, kb, kv.unit_stride,
                                      sp.n_sink, L_mid, pl, kappa, ent, meta);
  if (e != hipSuccess) return e;
  // dynamic LDS: the union scores, within what the device allows per block
  const size_t static_lds = 16 * 1024;
  int e_max = pl.e_max;
  if (g_lds_limit > static_lds) e_max = (int)std::min<size_t>(e_max, (g_lds_limit - static_lds) / 4);
  const size_t lds = (size_t)std::max(e_max, 1) * 4;
  hipLaunchKernelGGL((topk_select_kernel<KT, D>), dim3(kv.n_units * G), dim3(256), lds, st, q, G,
                     kb, kv.unit_stride, sp.n_sink, L_mid, pl.ch, pl.n_chunks, pl.r_cap, K, e_max,
                     kappa, ent, meta, idx, sel, 1.0f / sqrtf((float)D));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const TopkPlan& pl, const float* q, int G, const rma_kv& kv,
                       const rma_span& sp, const float* kappa, int K, int32_t* idx, float* sel,
                       uint8_t* ws, hipStream_t st) {
  if (g_lds_limit == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess)
      g_lds_limit = (size_t)v;
    else
      g_lds_limit = 64 * 1024;
  }
  if (kv.dtype == RMA_BF16) {
    if (kv.d == 64) return launch_topk_t<uint16_t, 64>(pl, q, G, kv, sp, kappa, K, idx, sel, ws, st);
    return launch_topk_t<uint16_t, 128>(pl, q, G, kv, sp, kappa, K, idx, sel, ws, st);
  }
  if (kv.d == 64) return launch_topk_t<float, 64>(pl, q, G, kv, sp, kappa, K, idx, sel, ws, st);
  return launch_topk_t<float, 128>(pl, q, G, kv, sp, kappa, K, idx, sel, ws, st);
}

}  // namespace rma
