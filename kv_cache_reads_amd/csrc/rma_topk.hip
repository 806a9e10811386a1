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

// Binning parameters of one head from its squared norm n2 (computed with a fixed
// reduction order, so every scan block of a unit gets identical bits; the
// select reads the copy the scan stores, so a score is binned identically by
// both kernels).
__device__ __forceinline__ HeadParams head_params(float n2, float kappa) {
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

// Block-wide exclusive scan of one int per thread (NT threads); returns the
// exclusive prefix, `total` receives the sum.  Uses buf[0 .. NT/64 - 1].
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* buf, int& total) {
  constexpr int NWV = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan_dpp(v);
  if (lane == kWave - 1) buf[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    const int x = buf[w];
    base += (w < wave) ? x : 0;
    tot += x;
  }
  total = tot;
  __syncthreads();
  return base + incl - v;
}
__device__ __forceinline__ int block_excl_scan256(int v, int* buf, int& total) {
  return block_excl_scan<256>(v, buf, total);
}

// The same for N independent values per thread in one pass (buf[0 .. 4N-1]):
// v[i] becomes its exclusive prefix, total[i] the sum.
template <int N>
__device__ __forceinline__ void block_excl_scan256_n(int (&v)[N], int* buf, int (&total)[N]) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  int incl[N];
#pragma unroll
  for (int i = 0; i < N; ++i) incl[i] = wave_incl_scan_dpp(v[i]);
  if (lane == kWave - 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) buf[4 * i + wave] = incl[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int w0 = buf[4 * i], w1 = buf[4 * i + 1], w2 = buf[4 * i + 2], w3 = buf[4 * i + 3];
    total[i] = w0 + w1 + w2 + w3;
    v[i] = (wave > 0 ? w0 : 0) + (wave > 1 ? w1 : 0) + (wave > 2 ? w2 : 0) + incl[i] - v[i];
  }
  __syncthreads();
}

// ====================================================================== scan
template <typename KT, int D, int G>
__global__ void __launch_bounds__(kScanThreads)
topk_scan_kernel(const float* __restrict__ q, const KT* __restrict__ kb, int64_t ustride,
                 int n_sink, int L_mid, int ch, int n_chunks, int r_min, int r_cap,
                 const float* __restrict__ kappa, float2* __restrict__ ent,
                 int2* __restrict__ meta, float4* __restrict__ hpw) {
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

  // query slices first: global loads complete in issue order, so the head
  // parameters below only wait for these, not for the key rows
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
  // histogram bins are filled while scoring
  for (int i = tid; i < G * NB; i += kScanThreads) hist[i] = 0u;

  const KT* kp = kb + (size_t)u * ustride + (size_t)(n_sink + t0) * D + part * E;
  constexpr int STEP = TPP * UNR;
  // rows past the chunk end re-read its last row (unconditional loads keep the
  // load counter exact); their scores are never stored
  auto load = [&](uint4 (&raw)[UNR][PIECES], int p0) {
#pragma unroll
    for (int i = 0; i < UNR; ++i) {
      const int t = min(p0 + i * TPP + wave * TPW + slot, n - 1);
      const uint4* src = reinterpret_cast<const uint4*>(kp + (size_t)t * D);
#pragma unroll
      for (int pc = 0; pc < PIECES; ++pc) raw[i][pc] = ld_stream16(src + pc);
    }
  };
  // two register buffers in turn, both in flight while the head parameters are derived
  uint4 ra[UNR][PIECES], rb[UNR][PIECES];
  load(ra, 0);
  if (STEP < n) load(rb, STEP);

  // every lane derives the same parameters from its query slices (the LPT lanes
  // of a token hold the whole query; fixed reduction order)
  HeadParams hp[G];
  const float kap_u = kappa[u];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float n2 = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) n2 = __fmaf_rn(qr[g][e], qr[g][e], n2);
    hp[g] = head_params(lane_group_sum<LPT>(n2), kap_u);
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
    if (tid == g) s_hp[g] = hp[g];
  __syncthreads();  // histogram cleared

  auto score = [&](const uint4 (&raw)[UNR][PIECES], int p0) {
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
        if (t < n && (g % LPT) == part) {
          sc[g * CHMAX + t] = a;
          atomicAdd(&hist[g * NB + lin_bin(a, hp[g])], 1u);
        }
      }
    }
  };
  for (int p0 = 0; p0 < n; p0 += 2 * STEP) {
    score(ra, p0);
    if (p0 + 2 * STEP < n) load(ra, p0 + 2 * STEP);
    if (p0 + STEP >= n) break;
    score(rb, p0 + STEP);
    if (p0 + 3 * STEP < n) load(rb, p0 + 3 * STEP);
  }
  __syncthreads();

  // ---- per head: smallest bin threshold that still passes >= min(r_min, n) tokens
  for (int g = wave; g < G; g += 4) {
    const int target = min(r_min, n);
    const uint32_t* h = hist + g * NB;
    int ls = 0;
#pragma unroll
    for (int j = 0; j < NB / kWave; ++j) ls += (int)h[lane * (NB / kWave) + j];
    const int incl = wave_incl_scan_dpp(ls);
    const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
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
    bc = __builtin_amdgcn_readlane(bc, lstar);
    run = __builtin_amdgcn_readlane(run, lstar);
    // lower the threshold to just above the highest non-empty bin below it: the
    // same tokens pass, and the select's completeness test is least strict
    int hb = -1;
#pragma unroll
    for (int j = 0; j < NB / kWave; ++j) {
      const int bin = lane * (NB / kWave) + j;
      if (bin < bc && h[bin] != 0u) hb = bin;
    }
    hb = (int)wave_max_dpp((float)hb);
    if (lane == 0) { s_bc[g] = hb + 1; s_nrep[g] = run; }
  }
  __syncthreads();

  // ---- ordered compaction of the passing tokens (position order), all heads
  //      with one multi-value block scan
  //      (each thread a contiguous run of at most PMAX tokens; one pass over the
  //      scores keeps a bit per passing token, the write pass visits those only)
  constexpr int PMAX = (CHMAX + kScanThreads - 1) / kScanThreads;
  static_assert(PMAX <= 32, "one 32-bit pass mask per head");
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
  int bcs[G], cnt[G], tot[G];
  uint32_t pm[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { bcs[g] = s_bc[g]; pm[g] = 0u; }
#pragma unroll
  for (int k = 0; k < PMAX; ++k) {
    if (i0 + k < i1) {
#pragma unroll
      for (int g = 0; g < G; ++g)
        pm[g] |= (lin_bin(sc[g * CHMAX + i0 + k], hp[g]) >= bcs[g]) ? (1u << k) : 0u;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) cnt[g] = __popc(pm[g]);
  block_excl_scan256_n<G>(cnt, s_buf, tot);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float2* dst = ent + ((size_t)(u * G + g) * n_chunks + c) * r_cap;
    int pos = cnt[g];
    for (uint32_t mk = pm[g]; mk != 0u; mk &= mk - 1u, ++pos) {
      const int i = i0 + __ffs(mk) - 1;
      if (pos < r_cap) dst[pos] = make_float2(sc[g * CHMAX + i], __int_as_float(t0 + i));
    }
  }
  if (tid < G) {
    meta[(size_t)(u * G + tid) * n_chunks + c] = make_int2(s_bc[tid], s_nrep[tid]);
    if (c == 0) hpw[u * G + tid] = make_float4(s_hp[tid].rg, s_hp[tid].inv_w, s_hp[tid].eps, 0.f);
  }
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
    const int incl = wave_incl_scan_dpp(ls);
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

template <typename KT, int D, int NT>
__device__ void exact_fallback(const float* qf, const KT* kunit, int n_sink, int L_mid, int K,
                               int32_t* io, float* so, float inv_sqrt_d, uint32_t* hist,
                               int* s_misc, int* s_buf) {
  const int tid = threadIdx.x;
  uint32_t P[5] = {0u, 0u, 0u, 0u, 0u};
  int krem = K, nd = 0;
  for (int p = 0; p < 20; ++p) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < L_mid; i += NT) {
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
  const int per = (L_mid + NT - 1) / NT;
  const int i0 = min(L_mid, tid * per), i1 = min(L_mid, i0 + per);
  int cnt = 0;
  for (int i = i0; i < i1; ++i) {
    uint32_t w[5];
    float s32;
    fb_key<KT, D>(qf, kunit, n_sink, i, w, s32);
    cnt += fb_cmp(w, P, nd) >= 0;
  }
  int total;
  int pos = block_excl_scan<NT>(cnt, s_buf, total);
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

// One empty statement that takes eight pairs of values loaded from LDS: the
// compiler can neither sink a read into the branch that later uses it nor wait
// for one before the next is issued.
__device__ __forceinline__ void pin_pairs8(int (&a)[8], int (&b)[8]) {
  asm volatile("" : "+v"(a[0]), "+v"(b[0]), "+v"(a[1]), "+v"(b[1]), "+v"(a[2]), "+v"(b[2]),
               "+v"(a[3]), "+v"(b[3]), "+v"(a[4]), "+v"(b[4]), "+v"(a[5]), "+v"(b[5]),
               "+v"(a[6]), "+v"(b[6]), "+v"(a[7]), "+v"(b[7]));
}

template <typename KT, int D, int NT>
__global__ void __launch_bounds__(NT)
topk_select_kernel(const float* __restrict__ q, int G, const KT* __restrict__ kb, int64_t ustride,
                   int n_sink, int L_mid, int ch, int n_chunks, int r_cap, int K, int e_max,
                   const float4* __restrict__ hpw, const float2* __restrict__ ent,
                   const int2* __restrict__ meta, int32_t* __restrict__ idx_out,
                   float* __restrict__ sc_out, float inv_sqrt_d) {
  constexpr int NBS = kSelBins;
  constexpr int NWV = NT / kWave;
  static_assert(NT >= kSelMaxChunks && NT >= 128, "one thread per chunk report and per query element");
  static_assert(NBS % NT == 0, "whole bins per thread");
  constexpr int SELF = 1 << 30;                // "selected" mark on a band member's position
  extern __shared__ __align__(16) float dyn[];
  float* es = dyn;                             // union scores (fp32, unscaled)
  int* ep = reinterpret_cast<int*>(dyn + e_max);  // union mid positions
  __shared__ int s_off[kSelMaxChunks + 1];
  __shared__ int s_bcs[kSelMaxChunks];
  __shared__ int s_nrep[kSelMaxChunks];
  __shared__ uint32_t hist[NBS];
  __shared__ float s_cand[kSelBandMax];       // scores of the K-th score's bin
  __shared__ int s_cnt;
  __shared__ uint32_t s_xlo, s_xhi;           // extent of that bin (order-preserving keys)
  __shared__ float s_t;
  __shared__ int s_buf[257];
  __shared__ int s_misc[8];
  __shared__ float s_fl[2 * NWV];
  __shared__ int s_wred[NWV];
  __shared__ DD s_bdd[kSelBandMax];
  __shared__ int s_bidx[kSelBandMax];
  __shared__ float s_qf[128];
  __shared__ float4 s_hp4;

  const int ug = blockIdx.x, u = ug / G, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const float* qg = q + (size_t)ug * D;
  const int2* mt = meta + (size_t)ug * n_chunks;
  const float2* en = ent + (size_t)ug * n_chunks * r_cap;
  int32_t* io = idx_out + (size_t)ug * K;
  float* so = sc_out + (size_t)ug * K;
  const KT* kunit = kb + (size_t)u * ustride;

  // Every input of the block is requested before any is used (one memory round
  // trip): the head's parameters, the query, the chunk counts and, when every
  // chunk's report slots fit SPEC per thread, all report slots (slot (c, j) is
  // valid for j < count_c).  The loads are unconditional (indices clamped into
  // range), so none waits inside a branch before the others are issued.
  // Slots map to threads by chunk: a power-of-two group of tpc threads per chunk
  // (thread t serves chunk t >> lg_t), so no slot index needs a division.
  const float4 hp_in = hpw[ug];  // written by the scan: identical binning and error bound
  const float q_in = qg[min(tid, D - 1)];
  constexpr int SPEC = 8;
  static_assert((NT & (NT - 1)) == 0, "power-of-two block");
  const int lg_c = n_chunks > 1 ? 32 - __clz(n_chunks - 1) : 0;   // ceil(log2(n_chunks)) <= 8
  const int lg_t = __builtin_ctz(NT) - lg_c, tpc = 1 << lg_t;
  const int my_c = tid >> lg_t, my_s = tid & (tpc - 1);
  const bool spec = r_cap <= SPEC * tpc;
  float2 sv[SPEC];
  if (spec) {
    const int cbase = min(my_c, n_chunks - 1) * r_cap;
#pragma unroll
    for (int k = 0; k < SPEC; ++k) sv[k] = en[cbase + min(my_s + k * tpc, r_cap - 1)];
  }
  const int2 mm = mt[max(0, min(tid, n_chunks - 1))];
  if (tid == 0) s_hp4 = hp_in;
  if (tid < D) s_qf[tid] = q_in;
  // chunk reports: one thread per chunk (n_chunks <= 256), offsets by a block scan
  int w_c = 0, trunc = 0;
  if (tid < n_chunks) {
    trunc = mm.y > r_cap;
    w_c = min(mm.y, r_cap);
    s_bcs[tid] = mm.x;
    s_nrep[tid] = mm.y;
  }
  int nE;
  const int off_c = block_excl_scan<NT>(w_c, s_buf, nE);
  if (tid < n_chunks) s_off[tid] = off_c;
  if (tid == 0) s_off[n_chunks] = nE;
  trunc = __syncthreads_or(trunc);
  const float4 hp4 = s_hp4;
  const HeadParams hp{hp4.x, hp4.y, hp4.z};
  int wmax = (int)wave_max_dpp((float)w_c);
  if (lane == 0) s_wred[wave] = wmax;
  __syncthreads();
  wmax = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) wmax = max(wmax, s_wred[w]);
  const FastDiv by_wmax(max(wmax, 1));

  if (K == L_mid) {  // every mid token is selected; the chunks reported all of them in order
    for (int i = tid; i < n_chunks * wmax; i += NT) {
      const int c = by_wmax.quo(i), j = i - c * wmax;
      if (j < s_off[c + 1] - s_off[c]) {
        const float2 e = en[(size_t)c * r_cap + j];
        io[s_off[c] + j] = n_sink + __float_as_int(e.y);
        so[s_off[c] + j] = e.x * inv_sqrt_d;
      }
    }
    return;
  }

  bool fallback = trunc != 0 || nE > e_max || nE < K;
  float th_lo = 0.f, th_hi = 0.f;
  int n_band = 0, kp = 0;
  if (!fallback) {
    // the union in LDS (report order = position order) and its score range
    float lo = INFINITY, hi = -INFINITY;
    if (spec) {
      // this thread's chunk: its offset and count (none for a thread past the chunks)
      const int cc = min(my_c, n_chunks - 1);
      const int o0 = s_off[cc];
      const int wc = my_c < n_chunks ? s_off[cc + 1] - o0 : 0;
#pragma unroll
      for (int k = 0; k < SPEC; ++k) {
        const int j = my_s + k * tpc;
        if (j < wc) {
          es[o0 + j] = sv[k].x;
          ep[o0 + j] = __float_as_int(sv[k].y);
          lo = fminf(lo, sv[k].x);
          hi = fmaxf(hi, sv[k].x);
        }
      }
    } else {
      // slot (chunk c, j < wmax) of the padded report layout; eight loads per
      // thread are issued before any is consumed
      const int nslots = n_chunks * wmax;
      for (int i0 = 0; i0 < nslots; i0 += 8 * NT) {
        float2 e[8];
        int dst[8], o0[8], o1[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int c = min(by_wmax.quo(i0 + k * NT + tid), n_chunks - 1);
          o0[k] = s_off[c];
          o1[k] = s_off[c + 1];
        }
        pin_pairs8(o0, o1);
        // a slot outside the reports loads a valid slot of the last chunk and
        // drops it, so no load waits inside a branch
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int i = i0 + k * NT + tid;
          const int c = min(by_wmax.quo(i), n_chunks - 1), j = i - c * wmax;
          dst[k] = ((i < nslots) & (j < o1[k] - o0[k])) ? o0[k] + j : -1;
          e[k] = en[(size_t)c * r_cap + min(j, r_cap - 1)];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (dst[k] >= 0) {
            es[dst[k]] = e[k].x;
            ep[dst[k]] = __float_as_int(e[k].y);
            lo = fminf(lo, e[k].x);
            hi = fmaxf(hi, e[k].x);
          }
        }
      }
    }
    lo = wave_min_dpp(lo);
    hi = wave_max_dpp(hi);
    if (lane == 0) { s_fl[wave] = lo; s_fl[NWV + wave] = hi; }
    for (int b = tid; b < NBS; b += NT) hist[b] = 0u;
    __syncthreads();
    lo = INFINITY;
    hi = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) { lo = fminf(lo, s_fl[w]); hi = fmaxf(hi, s_fl[NWV + w]); }
    const float inv = hi > lo ? (float)NBS / (hi - lo) : 0.f;
    auto ubin = [&](float x) {
      const float t = __fmul_rn(__fsub_rn(x, lo), inv);
      return (t >= 0.f) ? (int)fminf(t, (float)(NBS - 1)) : 0;  // monotone in x
    };
    // linear histogram over the range
    for (int i = tid; i < nE; i += NT) atomicAdd(&hist[ubin(es[i])], 1u);
    __syncthreads();
    // bin of the K-th largest score: thread t owns bins NBS-BPT*t-1 .. NBS-BPT*(t+1)
    // (descending)
    {
      constexpr int BPT = NBS / NT;
      int cb[BPT], ls = 0;
#pragma unroll
      for (int j = 0; j < BPT; ++j) { cb[j] = (int)hist[NBS - BPT * tid - 1 - j]; ls += cb[j]; }
      int tot;
      const int ex = block_excl_scan<NT>(ls, s_buf, tot);
      if (ex < K && ex + ls >= K) {
        int run = ex;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
          if (run < K && run + cb[j] >= K) {
            s_misc[0] = NBS - BPT * tid - 1 - j;
            s_misc[1] = run;  // entries in the bins above
          }
          run += cb[j];
        }
      }
      if (tid == 0) { s_cnt = 0; s_xlo = 0xffffffffu; s_xhi = 0u; }
    }
    __syncthreads();
    const int bK = s_misc[0], rK = K - s_misc[1];  // the K-th score is the rK-th largest of bin bK
    // the bin's members: their scores (up to kSelBandMax) and its exact extent
    for (int i = tid; i < nE; i += NT) {
      const float x = es[i];
      if (ubin(x) == bK) {
        const int j = atomicAdd(&s_cnt, 1);
        if (j < kSelBandMax) s_cand[j] = x;
        atomicMin(&s_xlo, ord_f32(x));
        atomicMax(&s_xhi, ord_f32(x));
      }
    }
    __syncthreads();
    const int nm = s_cnt;
    float t_lo = unord_f32(s_xlo), t_hi = unord_f32(s_xhi);
    if (nm <= kSelBandMax) {
      // t = the rK-th largest member score = the K-th largest fp32 score of the
      // union (every member holding that value writes the same bits)
      for (int j = tid; j < nm; j += NT) {
        const float x = s_cand[j];
        int gt = 0, ge = 0;
        for (int k2 = 0; k2 < nm; ++k2) {
          const float y = s_cand[k2];
          gt += y > x;
          ge += y >= x;
        }
        if (gt < rK && rK <= ge) s_t = x;
      }
      __syncthreads();
      t_lo = t_hi = s_t;
    }
    // the true K-th score lies within eps of t (or of the bin's extent when
    // the bin is too full to rank): outside +-2.5 eps the fp32 order is exact
    th_lo = t_lo - 2.5f * hp.eps;
    th_hi = t_hi + 2.5f * hp.eps;
    // every chunk must have reported all of its tokens scoring >= th_lo
    const int blo = lin_bin(th_lo, hp);
    int bad = 0;
    for (int c = tid; c < n_chunks; c += NT) {
      const int n_c = min(ch, L_mid - c * ch);
      if (s_nrep[c] != n_c && s_bcs[c] > blo) bad = 1;
    }
    if (tid == 0) { s_misc[3] = 0; s_misc[4] = 0; }
    fallback = __syncthreads_or(bad) != 0;
    if (!fallback) {
      int nin = 0;
      for (int i0 = 0; i0 < nE; i0 += NT) {
        const int i = i0 + tid;
        const float sc = i < nE ? es[i] : -INFINITY;
        nin += __popcll(__ballot(sc > th_hi));
        const bool in_band = i < nE && sc <= th_hi && sc >= th_lo;
        const uint64_t bm = __ballot(in_band);
        int base = 0;
        if (lane == 0 && bm != 0ull) base = atomicAdd(&s_misc[4], (int)__popcll(bm));
        base = __builtin_amdgcn_readlane(base, 0);
        const int b = base + lanes_below(bm);
        if (in_band && b < kSelBandMax) s_bidx[b] = i;
      }
      if (lane == 0) atomicAdd(&s_misc[3], nin);
      __syncthreads();
      n_band = s_misc[4];
      kp = K - s_misc[3];
      fallback = n_band > kSelBandMax || kp < 1 || n_band < kp;
    }
  }
  if (!fallback) {
    // band: exact double-double scores when it must be split
    for (int b = tid; b < n_band; b += NT) {
      const int i = s_bidx[b];
      s_bdd[b] = (n_band > kp) ? dd_dot<KT, D>(s_qf, kunit + (size_t)(n_sink + ep[i]) * D) : DD{0.0, 0.0};
    }
    __syncthreads();
    // rank by (exact score desc, position asc); mark the winners' positions
    for (int b = tid; b < n_band; b += NT) {
      const int i = s_bidx[b];
      bool take = true;
      if (n_band > kp) {
        int rank = 0;
        const DD mine = s_bdd[b];
        const int mp = ep[i];
        for (int b2 = 0; b2 < n_band; ++b2) rank += dd_key_greater(s_bdd[b2], ep[s_bidx[b2]], mine, mp);
        take = rank < kp;
      }
      hist[b] = take ? 1u : 0u;  // the histogram is no longer needed
    }
    __syncthreads();
    for (int b = tid; b < n_band; b += NT)
      if (hist[b] != 0u) ep[s_bidx[b]] |= SELF;
    __syncthreads();
    // ordered compaction of the selected entries in position order
    const int per = (nE + NT - 1) / NT;
    const int i0 = min(nE, tid * per), i1 = min(nE, i0 + per);
    int cnt = 0;
    for (int i = i0; i < i1; ++i) cnt += (es[i] > th_hi) | ((ep[i] & SELF) != 0);
    int total;
    int pos = block_excl_scan<NT>(cnt, s_buf, total);
    if (total != K) {
      fallback = true;  // uniform: every thread sees the same total
    } else {
      for (int i = i0; i < i1; ++i) {
        if ((es[i] > th_hi) | ((ep[i] & SELF) != 0)) {
          if (pos < K) {
            io[pos] = n_sink + (ep[i] & ~SELF);
            so[pos] = es[i] * inv_sqrt_d;
          }
          ++pos;
        }
      }
    }
  }
  if (fallback) {
    __syncthreads();
    exact_fallback<KT, D, NT>(s_qf, kunit, n_sink, L_mid, K, io, so, inv_sqrt_d, hist, s_misc, s_buf);
  }
}

// ====================================================================== launch
namespace {

size_t g_lds_limit = 0;

template <typename KT, int D>
hipError_t launch_scan_g(int G, dim3 grid, hipStream_t st, const float* q, const KT* kb,
                         int64_t ustride, int n_sink, int L_mid, const TopkPlan& pl,
                         const float* kappa, float2* ent, int2* meta, float4* hpw) {
  hipError_t e = hipSuccess;
#define RMA_SCAN_CASE(GG)                                                                            \
  case GG:                                                                                           \
    e = launch_kernel("topk_scan_kernel", topk_scan_kernel<KT, D, GG>, grid, dim3(kScanThreads), 0,  \
                      st, q, kb, ustride, n_sink, L_mid, pl.ch, pl.n_chunks, pl.r_min, pl.r_cap,     \
                      kappa, ent, meta, hpw);                                                        \
    break;
  switch (G) {
    RMA_SCAN_CASE(1) RMA_SCAN_CASE(2) RMA_SCAN_CASE(3) RMA_SCAN_CASE(4)
    RMA_SCAN_CASE(5) RMA_SCAN_CASE(6) RMA_SCAN_CASE(7) RMA_SCAN_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef RMA_SCAN_CASE
  return e;
}

template <typename KT, int D>
hipError_t launch_topk_t(const TopkPlan& pl, const float* q, int G, const rma_kv& kv,
                         const rma_span& sp, const float* kappa, int K, int32_t* idx,
                         float* sel, uint8_t* ws, hipStream_t st) {
  const int L_mid = (int)(sp.L - sp.n_sink - sp.n_tail);
  const KT* kb = static_cast<const KT*>(kv.k);
  float2* ent = reinterpret_cast<float2*>(ws + pl.off_ent);
  int2* meta = reinterpret_cast<int2*>(ws + pl.off_meta);
  float4* hpw = reinterpret_cast<float4*>(ws + pl.off_hp);
  hipError_t e = launch_scan_g<KT, D>(G, dim3(pl.n_chunks, kv.n_units), st, q, kb, kv.unit_stride,
                                      sp.n_sink, L_mid, pl, kappa, ent, meta, hpw);
  if (e != hipSuccess) return e;
  // dynamic LDS: the union (score, position) pairs, within the per-block limit
  // left by the kernel's own (static) LDS.  Many (unit, head) blocks with short
  // report lists: 256 threads each, so that several share a CU; otherwise 1024.
  const bool small = kv.n_units * G >= 1024 && (int64_t)pl.n_chunks * pl.r_cap <= 8 * 256;
  static size_t static_lds[2] = {0, 0};
  const void* kfn = small ? reinterpret_cast<const void*>(&topk_select_kernel<KT, D, 256>)
                          : reinterpret_cast<const void*>(&topk_select_kernel<KT, D, kSelThreads>);
  size_t& sl = static_lds[small ? 1 : 0];
  if (sl == 0) {
    hipFuncAttributes attr{};
    sl = hipFuncGetAttributes(&attr, kfn) == hipSuccess ? attr.sharedSizeBytes : 32 * 1024;
  }
  int e_max = pl.e_max;
  if (g_lds_limit > sl) e_max = (int)std::min<size_t>(e_max, (g_lds_limit - sl) / 8);
  const size_t lds = (size_t)std::max(e_max, 1) * 8;
  if (small)
    return launch_kernel("topk_select_kernel", topk_select_kernel<KT, D, 256>,
                         dim3(kv.n_units * G), dim3(256), lds, st, q, G, kb, kv.unit_stride,
                         sp.n_sink, L_mid, pl.ch, pl.n_chunks, pl.r_cap, K, e_max, hpw, ent, meta,
                         idx, sel, 1.0f / sqrtf((float)D));
  return launch_kernel("topk_select_kernel", topk_select_kernel<KT, D, kSelThreads>,
                       dim3(kv.n_units * G), dim3(kSelThreads), lds, st, q, G, kb, kv.unit_stride,
                       sp.n_sink, L_mid, pl.ch, pl.n_chunks, pl.r_cap, K, e_max, hpw, ent, meta,
                       idx, sel, 1.0f / sqrtf((float)D));
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
