// Exact Top-K selection of one query head from the scan's chunk reports
// ("Residual-Mass Accounting for Partial-KV Decoding", §1: exhaustive Top-K is
// the control selector fixing the exact support; §3 Eq. 3: K(q) is a K-subset
// of M).  Shared by the separate select kernel (rma_decode_topk) and the fused
// select-and-merge kernel (rma_decode).
//
// The scan leaves, per (unit, head) and chunk, every token scoring at or above
// a per-chunk threshold (score, position), the chunk's threshold bin and count,
// and the head's binning parameters.  The block gathers the reports, finds the
// K-th largest fp32 score t of their union, proves that no chunk withheld a
// token within the error band, keeps every token above t + 2.5 eps, resolves
// the band [t - 2.5 eps, t + 2.5 eps] with double-double scores and emits the K
// positions in ascending order.  eps bounds |fl32(q.k) - q.k| for every mid
// token: the fp32 dot has at most 19 roundings per product path, so
// |err| <= gamma_19 sum|q_j k_j| <= gamma_19 |q|_2 kappa, kappa >= max ||k_i||_2.
// When a check fails (a chunk withheld tokens, the band is too wide, too many
// entries) it falls back to an exact radix select on (double-double score,
// -position) over the whole mid-region.
#pragma once
#include "rma_device.hpp"
#include "rma_internal.hpp"

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
  // the fp32 dot's error is at most gamma_19 sum|q_j k_j| <= gamma_19 |q| kappa,
  // gamma_19 < 1.134e-6; |q| here is within 7e-7 of the exact norm (a fp32 sum
  // of squares and a rounded root), kappa is an upper bound and the products
  // below add two roundings, so 2e-6 covers the bound with 75% to spare
  h.eps = __fmul_rn(2e-6f, __fmul_rn(qn, kap));
  return h;
}

__device__ __forceinline__ int lin_bin(float x, const HeadParams& h) {
  const float t = __fmul_rn(__fadd_rn(x, h.rg), h.inv_w);
  // clamped to [0, kScanBins - 1] in one v_med3_f32 and truncated: monotone in x
  return (int)__builtin_amdgcn_fmed3f(t, 0.f, (float)(kScanBins - 1));
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

// Where a head's selection goes: the K positions (ascending) and their scaled
// scores s_i = fl32(q.k_i) / sqrt(d), to global memory (io, so) and/or to an
// LDS list (lpos, lsc).
struct SelOut {
  int32_t* io = nullptr;
  float* so = nullptr;
  int* lpos = nullptr;
  float* lsc = nullptr;
  __device__ __forceinline__ void put(int i, int pos, float s) const {
    if (io != nullptr) {
      io[i] = pos;
      so[i] = s;
    }
    if (lpos != nullptr) {
      lpos[i] = pos;
      lsc[i] = s;
    }
  }
};

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
                               SelOut out, float inv_sqrt_d, uint32_t* hist,
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
      if (pos < K) out.put(pos, n_sink + i, s32 * inv_sqrt_d);
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

// The selection of one (unit, head) by one block of NT threads.  load() issues
// every global load the selection needs; run() consumes them, so a caller can
// issue loads of its own in between and the selection waits only for its own.
// es, ep: e_max union slots in LDS (scores, positions).
template <typename KT, int D, int NT>
struct HeadSelect {
  static constexpr int SPEC = 8;
  // the head
  int ug;
  const float* qg;       // the head's query
  const int2* mt;        // the head's chunk metas
  const float2* en;      // the head's chunk reports
  const KT* kunit;       // the unit's keys
  int n_sink, L_mid, ch, n_chunks, r_cap, K, e_max;
  float inv_sqrt_d;
  // loaded
  f32x4 hp_in;          // the head's (rg, inv_w, eps, -) from the scan
  float q_in;
  float2 sv[SPEC];
  int2 mm;
  int lg_c, lg_t, tpc, my_c, my_s;
  bool spec;

  __device__ __forceinline__ void load(const float4* __restrict__ hpw) {
    const int tid = threadIdx.x;
    // Every input of the block is requested before any is used (one memory round
    // trip): the head's parameters, the query, the chunk counts and, when every
    // chunk's report slots fit SPEC per thread, all report slots (slot (c, j) is
    // valid for j < count_c).  The loads are unconditional (indices clamped into
    // range), so none waits inside a branch before the others are issued.
    // Slots map to threads by chunk: a power-of-two group of tpc threads per chunk
    // (thread t serves chunk t >> lg_t), so no slot index needs a division.
    hp_in = *reinterpret_cast<const f32x4*>(hpw + ug);  // written by the scan: identical binning and error bound
    q_in = qg[min(tid, D - 1)];
    static_assert((NT & (NT - 1)) == 0, "power-of-two block");
    lg_c = n_chunks > 1 ? 32 - __clz(n_chunks - 1) : 0;   // ceil(log2(n_chunks)) <= 8
    lg_t = __builtin_ctz(NT) - lg_c;
    tpc = 1 << lg_t;
    my_c = tid >> lg_t;
    my_s = tid & (tpc - 1);
    spec = r_cap <= SPEC * tpc;
    if (spec) {
      const int cbase = min(my_c, n_chunks - 1) * r_cap;
  #pragma unroll
      for (int k = 0; k < SPEC; ++k) sv[k] = en[cbase + min(my_s + k * tpc, r_cap - 1)];
    }
    mm = mt[max(0, min(tid, n_chunks - 1))];
  }

  __device__ __forceinline__ void run(float* es, int* ep, SelOut out) {
    constexpr int NBS = kSelBins;
    constexpr int NWV = NT / kWave;
    static_assert(NT >= kSelMaxChunks && NT >= 128, "one thread per chunk report and per query element");
    static_assert(NBS % NT == 0, "whole bins per thread");
    constexpr int SELF = 1 << 30;                // "selected" mark on a band member's position
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
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid >> 6;
    if (tid == 0) s_hp4 = make_float4(hp_in[0], hp_in[1], hp_in[2], hp_in[3]);
    if (tid < D) s_qf[tid] = q_in;
    // chunk reports: one thread per chunk (n_chunks <= 256), offsets by a block scan
    int w_c = 0, trunc = 0;
    if (tid < n_chunks) {
      trunc = mm.y > r_cap;
      w_c = min(mm.y, r_cap);
      s_bcs[tid] = mm.x & 0xffff;   // the cut bin (the chunk's top bin above it)
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
          out.put(s_off[c] + j, n_sink + __float_as_int(e.y), e.x * inv_sqrt_d);
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
            if (pos < K) out.put(pos, n_sink + (ep[i] & ~SELF), es[i] * inv_sqrt_d);
            ++pos;
          }
        }
      }
    }
    if (fallback) {
      __syncthreads();
      exact_fallback<KT, D, NT>(s_qf, kunit, n_sink, L_mid, K, out, inv_sqrt_d, hist, s_misc, s_buf);
    }
  }
};


// ---------------------------------------------------------------- few-barrier selection
// The exact selection of HeadSelect::run by a whole block, in as few barrier
// phases as the data dependences allow (for the fused decode kernel).  Steps
// whose input every wave can read (the K-th bin from the histogram, the rank
// of that bin's members, the chunk certificate) are computed by every wave
// redundantly instead of by one wave behind a barrier.
//
// Input: the union of the chunk reports in LDS in report order (= position
// order): score es[i] and mid position ep[i] for i < nE, followed by empty
// entries (es = -inf, ep = 0) up to a whole row of 64; the union's score range
// [lo, hi]; the chunk table (threshold bin, reported count); w.hist zeroed and
// w.misc initialised (init_block_select) behind a barrier.  The steps:
//   histogram over [lo, hi] | the bin bK of the K-th largest score, its members
//   and extent | t = the K-th largest fp32 score (rank among the members), the
//   completeness certificate of every chunk for t - 2.5 eps, the count above
//   t + 2.5 eps per wave (wave w owns a contiguous range of rows) and the band
//   [t - 2.5 eps, t + 2.5 eps] | the entries above the band into the list (wave
//   w's at the sum of the lower waves' counts, position order), the band's
//   double-double scores (one lane group per member) when it must be split |
//   rank and mark | the band's winners appended in position order.
// The list (lpos: positions, lsc: scaled scores; K entries) feeds the gather;
// its order is fixed by the data, so the sums over it are deterministic.  With
// out.io set the K indices and kept scores are also written in position order
// (one more count and barrier).
// Returns false (the same on every thread) when the block must run the exact
// fallback (a chunk withheld tokens, too few entries, band too wide).  The
// caller puts a barrier before reading the list.
// The block selection's bins: kSelBins linear bins over the scan-bin interval
// [b_lo, b_hi) that holds every report, on the scan's bin coordinate
// (x + rg) inv_w (the same two roundings as lin_bin), shifted and scaled;
// monotone in x and clamped, so any score maps to a bin
struct SelBins {
  float rg, inv_w, b_lo, scale;
  __device__ __forceinline__ int operator()(float x) const {
    const float t = __fmul_rn(__fsub_rn(__fmul_rn(__fadd_rn(x, rg), inv_w), b_lo), scale);
    return (int)__builtin_amdgcn_fmed3f(t, 0.f, (float)(kSelBins - 1));
  }
};
__device__ __forceinline__ SelBins sel_bins(const HeadParams& hp, int b_lo, int b_hi) {
  return SelBins{hp.rg, hp.inv_w, (float)b_lo, __fdiv_rn((float)kSelBins, (float)max(b_hi - b_lo, 1))};
}

struct BlockSelLds {
  uint32_t* hist;   // kSelBins
  uint32_t* coarse; // kSelBins / 16: the sums of 16 consecutive bins
  float* cand;      // kSelBandMax: scores of the K-th bin's members (16-byte aligned)
  int* bslot;       // kSelBandMax: band members' entries
  DD* bdd;          // kSelBandMax: their double-double scores
  int* misc;        // 8: [0] members, [1] / [2] ordered min / max member, [3] count above, [4] band, [5] t
  int* wcnt;        // one per wave
};

template <int NT>
__device__ __forceinline__ void init_block_select(const BlockSelLds& w) {
  for (int b = threadIdx.x; b < kSelBins; b += NT) w.hist[b] = 0u;
  for (int b = threadIdx.x; b < kSelBins / 16; b += NT) w.coarse[b] = 0u;
  if (threadIdx.x < 8) w.misc[threadIdx.x] = threadIdx.x == 1 ? (int)0xffffffffu : 0;
}

template <typename KT, int D, int NT>
__device__ bool block_select(const float* es, int* ep, int nE, const SelBins& ubin, const int* s_bcs,
                             const int* s_nrep, int n_chunks, int ch, int L_mid, int n_sink, int K,
                             bool trunc, const HeadParams& hp, const float* qf, const KT* kunit,
                             float inv_sqrt_d, const BlockSelLds& w, int* lpos, float* lsc,
                             const SelOut& out) {
  constexpr int NBS = kSelBins;
  constexpr int NW = NT / kWave;
  constexpr int BPL = NBS / kWave;             // histogram bins per lane (each wave reads them all)
  constexpr int SELF = 1 << 30;                // "taken" mark on a band member's position
  static_assert(BPL % 4 == 0, "whole 16-byte histogram reads");
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  if (trunc || nE < K) return false;
  const int rows = (nE + kWave - 1) / kWave;
  const int RW = (rows + NW - 1) / NW;   // wave w's rows [r0, r1) for the ordered steps
  const int r0 = min(rows, wave * RW), r1 = min(rows, r0 + RW);
  // the per-wave counts in w.wcnt: their sum over the lower waves and over all
  // (the first NW lanes take one each and scan inside their 16-lane row)
  auto wave_counts_prefix = [&](int& below, int& total) {
    static_assert(NW <= 16, "the counts fit one 16-lane row");
    int c = lane < NW ? w.wcnt[lane] : 0;
    c += dpp_i<0x111>(c);   // row_shr:1
    c += dpp_i<0x112>(c);   // row_shr:2
    c += dpp_i<0x114>(c);   // row_shr:4
    c += dpp_i<0x118>(c);   // row_shr:8
    total = __builtin_amdgcn_readlane(c, NW - 1);
    below = wave > 0 ? __builtin_amdgcn_readlane(c, wave - 1) : 0;
  };

  const bool whole = K == L_mid;   // every mid token is selected (the chunks reported all)
  float th_lo = -INFINITY, th_hi = -INFINITY;
  int nb = 0, kp = 0;
  if (!whole) {
    // (the caller built the histogram of the union's scores on these bins,
    // with the sums of 16 bins beside it, while placing the reports)
    // ---- every wave: the bin of the K-th largest.  Lane l owns the 16 bins
    //      NBS-16(l+1) .. NBS-16l-1 (their sum is one coarse count); a scan of
    //      the lanes' sums names the lane holding it, whose 16 bins the first 16
    //      lanes then take one each (descending) and scan again
    int bK = 0, above = 0;
    {
      static_assert(BPL == 16, "one coarse count per lane; the second scan covers one 16-lane row");
      const int ls = (int)w.coarse[NBS / BPL - 1 - lane];
      const int incl = wave_incl_scan_dpp(ls);
      const int owner = __ffsll((long long)__ballot(incl >= K)) - 1;
      const int run0 = __builtin_amdgcn_readlane(incl - ls, owner);   // entries above its bins
      const int bo = NBS - 1 - BPL * owner;
      const int c = lane < BPL ? (int)w.hist[bo - lane] : 0;
      int cum = c;                        // inclusive scan inside each 16-lane row
      cum += dpp_i<0x111>(cum);           // row_shr:1
      cum += dpp_i<0x112>(cum);           // row_shr:2
      cum += dpp_i<0x114>(cum);           // row_shr:4
      cum += dpp_i<0x118>(cum);           // row_shr:8
      const int jf = __ffsll((long long)__ballot(lane < BPL && run0 + cum >= K)) - 1;
      bK = bo - jf;
      above = __builtin_amdgcn_readlane(run0 + cum - c, jf);
    }
    const int rK = K - above;   // the K-th score is the rK-th largest member of bin bK
    // ... and its members: scores appended (order free), extent
    {
      float xlo = INFINITY, xhi = -INFINITY;
      for (int r = wave; r < rows; r += NW) {
        const float x = es[r * kWave + lane];
        const bool m = x > -INFINITY && ubin(x) == bK;
        const uint64_t bm = __ballot(m);
        if (bm != 0ull) {
          int base = 0;
          if (lane == 0) base = atomicAdd(&w.misc[0], (int)__popcll(bm));
          base = __builtin_amdgcn_readlane(base, 0);
          const int o = base + lanes_below(bm);
          if (m && o < kSelBandMax) w.cand[o] = x;
        }
        xlo = m ? fmin_m3(xlo, x) : xlo;
        xhi = m ? fmax_m3(xhi, x) : xhi;
      }
      const uint32_t klo = ~wave_max_u32(~ord_f32(xlo)), khi = wave_max_u32(ord_f32(xhi));
      if (lane == 0 && klo <= khi) {
        atomicMin(reinterpret_cast<uint32_t*>(&w.misc[1]), klo);
        atomicMax(reinterpret_cast<uint32_t*>(&w.misc[2]), khi);
      }
    }
    __syncthreads();
    const int nm = w.misc[0];
    float t_lo = unord_f32((uint32_t)w.misc[1]), t_hi = unord_f32((uint32_t)w.misc[2]);
    if (nm <= kSelBandMax) {
      // t = the rK-th largest member (every member holding that value agrees)
      float t = -INFINITY;
      if (nm <= kWave) {     // every wave ranks them (four members per 16-byte read)
        if (lane < nm) {
          const float x = w.cand[lane];
          int gt = 0, ge = 0;
          for (int k4 = 0; k4 < nm; k4 += 4) {
            const float4 y4 = *reinterpret_cast<const float4*>(w.cand + k4);
            const float y[4] = {y4.x, y4.y, y4.z, y4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bool in = k4 + i < nm;
              gt += in && y[i] > x;
              ge += in && y[i] >= x;
            }
          }
          if (gt < rK && rK <= ge) t = x;
        }
        t = wave_max_dpp(t);
      } else {               // the block ranks them
        for (int j = tid; j < nm; j += NT) {
          const float x = w.cand[j];
          int gt = 0, ge = 0;
          for (int k2 = 0; k2 < nm; ++k2) {
            const float y = w.cand[k2];
            gt += y > x;
            ge += y >= x;
          }
          if (gt < rK && rK <= ge) w.misc[5] = __float_as_int(x);
        }
        __syncthreads();
        t = __int_as_float(w.misc[5]);
      }
      t_lo = t_hi = t;
    }
    th_lo = t_lo - 2.5f * hp.eps;
    th_hi = t_hi + 2.5f * hp.eps;
    // ---- every wave: each chunk must have reported all of its tokens >= th_lo
    {
      const int blo = lin_bin(th_lo, hp);
      bool bad = false;
      for (int c = lane; c < n_chunks; c += kWave) {
        const int n_c = min(ch, L_mid - c * ch);
        bad |= s_nrep[c] != n_c && s_bcs[c] > blo;
      }
      if (__ballot(bad) != 0ull) return false;
    }
    // ---- the count above th_hi (per wave, over its row range) and the band,
    //      appended (order free)
    {
      int nin = 0;
      for (int r = r0; r < r1; ++r) {
        const float x = es[r * kWave + lane];
        nin += (int)__popcll(__ballot(x > th_hi));
        const bool inb = x > -INFINITY && x <= th_hi && x >= th_lo;
        const uint64_t bm = __ballot(inb);
        if (bm != 0ull) {
          int base = 0;
          if (lane == 0) base = atomicAdd(&w.misc[4], (int)__popcll(bm));
          base = __builtin_amdgcn_readlane(base, 0);
          const int o = base + lanes_below(bm);
          if (inb && o < kSelBandMax) w.bslot[o] = r * kWave + lane;
        }
      }
      if (lane == 0) w.wcnt[wave] = nin;
    }
    __syncthreads();
    nb = w.misc[4];
    int nin = 0, o = 0;
    wave_counts_prefix(o, nin);
    kp = K - nin;
    if (nb > kSelBandMax || kp < 1 || nb < kp) return false;
    // ---- the list, first part: the entries above th_hi in position order
    for (int r = r0; r < r1; ++r) {
      const float x = es[r * kWave + lane];
      const bool a = x > th_hi;
      const uint64_t bm = __ballot(a);
      if (a) {
        lpos[o + lanes_below(bm)] = n_sink + ep[r * kWave + lane];
        lsc[o + lanes_below(bm)] = x * inv_sqrt_d;
      }
      o += (int)__popcll(bm);
    }
    if (nb > kp) {
      // ---- the band's double-double scores, one lane group per member
      constexpr int P = DDGroup<KT, D>::P;
      for (int b = tid / P; b < nb; b += NT / P) {   // uniform within the group
        const DD d = dd_dot_group<KT, D>(qf, kunit + (size_t)(n_sink + ep[w.bslot[b]]) * D, tid % P);
        if (tid % P == 0) w.bdd[b] = d;
      }
      __syncthreads();
      // rank by (exact score desc, position asc); positions masked since marks
      // of other threads may already be set
      for (int b = tid; b < nb; b += NT) {
        const DD mine = w.bdd[b];
        const int mp = ep[w.bslot[b]] & ~SELF;
        int rank = 0;
        for (int b2 = 0; b2 < nb; ++b2) rank += dd_key_greater(w.bdd[b2], ep[w.bslot[b2]] & ~SELF, mine, mp);
        if (rank < kp) ep[w.bslot[b]] = mp | SELF;
      }
    } else {
      for (int b = tid; b < nb; b += NT) ep[w.bslot[b]] |= SELF;
    }
    __syncthreads();
    // ---- the list, second part: the band's winners in position order
    for (int b = tid; b < nb; b += NT) {
      const int e = ep[w.bslot[b]];
      if ((e & SELF) == 0) continue;
      const int mp = e & ~SELF;
      int before = 0;
      for (int b2 = 0; b2 < nb; ++b2) {
        const int e2 = ep[w.bslot[b2]];
        before += (e2 & SELF) != 0 && (e2 & ~SELF) < mp;
      }
      lpos[nin + before] = n_sink + mp;
      lsc[nin + before] = es[w.bslot[b]] * inv_sqrt_d;
    }
  } else {
    // every entry is selected: the list in position order (wave w's rows at the
    // sum of the lower waves' counts)
    int cnt = 0;
    for (int r = r0; r < r1; ++r) cnt += (int)__popcll(__ballot(es[r * kWave + lane] > -INFINITY));
    if (lane == 0) w.wcnt[wave] = cnt;
    __syncthreads();
    int o = 0, tot = 0;
    wave_counts_prefix(o, tot);
    for (int r = r0; r < r1; ++r) {
      const float x = es[r * kWave + lane];
      const bool a = x > -INFINITY;
      const uint64_t bm = __ballot(a);
      if (a) {
        lpos[o + lanes_below(bm)] = n_sink + ep[r * kWave + lane];
        lsc[o + lanes_below(bm)] = x * inv_sqrt_d;
      }
      o += (int)__popcll(bm);
    }
  }
  // ---- the indices and kept scores in position order, when asked: wave w's
  //      taken entries at the sum of the lower waves' counts
  if (out.io != nullptr) {
    auto taken = [&](float x, int e) { return x > -INFINITY && (whole || x > th_hi || (e & SELF) != 0); };
    int cnt = 0;
    for (int r = r0; r < r1; ++r)
      cnt += (int)__popcll(__ballot(taken(es[r * kWave + lane], ep[r * kWave + lane])));
    __syncthreads();   // the counts above are read
    if (lane == 0) w.wcnt[wave] = cnt;
    __syncthreads();
    int o = 0, tot = 0;
    wave_counts_prefix(o, tot);
    for (int r = r0; r < r1; ++r) {
      const float x = es[r * kWave + lane];
      const int e = ep[r * kWave + lane];
      const bool tk = taken(x, e);
      const uint64_t bm = __ballot(tk);
      if (tk && o + lanes_below(bm) < K) {
        out.io[o + lanes_below(bm)] = n_sink + (e & ~SELF);
        out.so[o + lanes_below(bm)] = x * inv_sqrt_d;
      }
      o += (int)__popcll(bm);
    }
  }
  return true;
}

}  // namespace rma
