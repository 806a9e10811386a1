// Exhaustive Top-K over the mid-region for every query head ("Residual-Mass
// Accounting for Partial-KV Decoding", §1: exhaustive Top-K is the control
// selector fixing the exact support; §3 Eq. 3: K(q) is a K-subset of M).
//
// Ranking is by the exact real value of q.k_i, ties to the lower position.
//
// Two kernels:
//  scan   grid (units, chunks).  Streams each unit's K_mid rows once for all G
//         query heads (fp32 FMA on bf16/fp32 keys, d split over 4-8 lanes and
//         summed with DPP).  Scores stay in LDS; a linear-bin histogram per head
//         picks a per-chunk threshold so that at least r_min tokens pass, and
//         the passing tokens (score, position) are written in position order;
//         the chunk's entry of the table: (cut bin | top non-empty bin << 16,
//         tokens at or above the cut).
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
#include "rma_select.hpp"

#include <algorithm>
#include <math.h>


namespace rma {

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
  constexpr int TPP = scan_tile(D);  // tokens per block pass
  static_assert(TPP == (kScanThreads / kWave) * TPW, "one token slot per lane group");
  constexpr int EPP = RowPieces<KT>::kElemsPerPiece;
  constexpr int PIECES = E / EPP;    // 16-byte loads per lane per token
  constexpr int UNR = (sizeof(KT) == 2) ? 4 : 2;
  constexpr int CHMAX = scan_chmax(D, G);
  // score rows of the G heads 8 words apart modulo the 32 banks: one store
  // instruction writes a token group's scores of every head without conflicts
  constexpr int SCS = CHMAX + 8;
  constexpr int NB = kScanBins;
  constexpr int GJ = (G + LPT - 1) / LPT;   // heads whose score a lane stores

  __shared__ float sc[G * SCS];
  __shared__ uint32_t hist[G * NB];
  __shared__ float4 s_q[G * D / 4];
  __shared__ HeadParams s_hp[G];

  // grid (units, chunks): consecutive workgroups take consecutive units and go
  // to the 8 XCDs in turn, so with a unit count that is a multiple of 8 a
  // unit's chunks, and the fused kernel's blocks that read their reports, share an XCD
  const int u = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const int part = lane % LPT, slot = lane / LPT;
  const int t0 = c * ch;
  const int n = min(ch, L_mid - t0);

  // the unit's queries (G d floats) once per block, first: global loads
  // complete in issue order, so their wait below does not wait for the keys
  static_assert(G * D / 4 <= kScanThreads, "one 16-byte query piece per thread");
  const float4 q4 = reinterpret_cast<const float4*>(q + (size_t)u * G * D)[min(tid, G * D / 4 - 1)];

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

  // histogram bins are filled while scoring
  for (int i = tid; i < G * NB; i += kScanThreads) hist[i] = 0u;
  if (tid < G * D / 4) s_q[tid] = q4;
  __syncthreads();  // histogram cleared, queries in LDS

  // every lane derives the same parameters from its query slices (the LPT lanes
  // of a token hold the whole query; fixed reduction order)
  float qr[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const float4 v = s_q[(g * D + part * E) / 4 + i];
      qr[g][4 * i] = v.x; qr[g][4 * i + 1] = v.y; qr[g][4 * i + 2] = v.z; qr[g][4 * i + 3] = v.w;
    }
  }
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
  // lane `part` of a token's lane group stores heads part, part + LPT, ...
  HeadParams hm[GJ];
#pragma unroll
  for (int j = 0; j < GJ; ++j) {
    hm[j] = hp[j * LPT];
#pragma unroll
    for (int g = j * LPT + 1; g < G && g < (j + 1) * LPT; ++g)
      if (part == g - j * LPT) hm[j] = hp[g];
  }

  auto score = [&](const uint4 (&raw)[UNR][PIECES], int p0) {
#pragma unroll
    for (int i = 0; i < UNR; ++i) {
      const int t = p0 + i * TPP + wave * TPW + slot;
      float kv[E];
#pragma unroll
      for (int pc = 0; pc < PIECES; ++pc) unpack_piece(raw[i][pc], (const KT*)nullptr, kv + pc * EPP);
      float a[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        a[g] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) a[g] = __fmaf_rn(qr[g][e], kv[e], a[g]);
        a[g] = lane_group_sum<LPT>(a[g]);   // the same bits in every lane of the group
      }
      // one score store and one histogram count per lane and owned head
#pragma unroll
      for (int j = 0; j < GJ; ++j) {
        float mine = a[j * LPT];
#pragma unroll
        for (int g = j * LPT + 1; g < G && g < (j + 1) * LPT; ++g) mine = part == g - j * LPT ? a[g] : mine;
        // materialised before the branch: the sums' last DPP steps then fold
        // into single v_add_f32_dpp instructions instead of a move and an add
        asm volatile("" : "+v"(mine));
        const int gg = j * LPT + part;
        if (t < n && gg < G) {
          sc[gg * SCS + t] = mine;
          atomicAdd(&hist[gg * NB + lin_bin(mine, hm[j])], 1u);
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

  // ---- per head, one wave: the smallest bin threshold that still passes
  //      >= min(r_min, n) tokens, then the passing tokens in position order
  //      (rows of 64 scores, appended by ballot)
  for (int g = wave; g < G; g += kScanThreads / kWave) {
    const int target = min(r_min, n);
    constexpr int BPL = NB / kWave;   // bins per lane, read once as 16-byte words
    static_assert(BPL % 4 == 0, "whole 16-byte histogram reads");
    uint32_t hb_[BPL];
    {
      const uint4* h4 = reinterpret_cast<const uint4*>(hist + g * NB + lane * BPL);
#pragma unroll
      for (int j = 0; j < BPL / 4; ++j) {
        const uint4 v = h4[j];
        hb_[4 * j] = v.x; hb_[4 * j + 1] = v.y; hb_[4 * j + 2] = v.z; hb_[4 * j + 3] = v.w;
      }
    }
    int ls = 0;
#pragma unroll
    for (int j = 0; j < BPL; ++j) ls += (int)hb_[j];
    const int incl = wave_incl_scan_dpp(ls);
    const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
    const int suf = total - incl + ls;  // tokens in this lane's bins and above
    const unsigned long long ball = __ballot(suf >= target);
    const int lstar = 63 - __clzll((long long)ball);
    // the highest bin from which the bins at and above it hold >= target
    // tokens: lane lstar's BPL bins, one per lane of the first BPL (descending),
    // scanned inside the first 16-lane row on top of the tokens above them
    static_assert(BPL <= 16, "lane lstar's bins fit one 16-lane row");
    const int above = __builtin_amdgcn_readlane(suf - ls, lstar);
    const int bt = lstar * BPL + BPL - 1;   // lane lstar's top bin
    const int cl = lane < BPL ? (int)hist[g * NB + bt - lane] : 0;
    int cum = cl;
    cum += dpp_i<0x111>(cum);   // row_shr:1
    cum += dpp_i<0x112>(cum);   // row_shr:2
    cum += dpp_i<0x114>(cum);   // row_shr:4
    cum += dpp_i<0x118>(cum);   // row_shr:8
    const int jf = __ffsll((long long)__ballot(lane < BPL && above + cum >= target)) - 1;
    const int bc = bt - jf;
    const int run = __builtin_amdgcn_readlane(above + cum, jf);
    // lower the threshold to just above the highest non-empty bin below it: the
    // same tokens pass, and the select's completeness test is least strict
    // (and the chunk's highest non-empty bin: its reports lie in [bcut, top])
    int hb = -1, tb = -1;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int bin = lane * BPL + j;
      if (hb_[j] != 0u) {
        tb = bin;
        if (bin < bc) hb = bin;
      }
    }
    const int bcut = (int)wave_max_u32((uint32_t)(hb + 1));
    const int top = (int)wave_max_u32((uint32_t)(tb + 1)) - 1;
    float2* dst = ent + ((size_t)(u * G + g) * n_chunks + c) * r_cap;
    const HeadParams hg = s_hp[g];
    constexpr int RB = 8;   // rows of 64 scores per batch: loads first, then ballots, then stores
    int base = 0;
    for (int r0 = 0; r0 < n; r0 += RB * kWave) {
      float x[RB];
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        const int i = r0 + k * kWave + lane;
        x[k] = sc[g * SCS + min(i, n - 1)];
      }
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        const int i = r0 + k * kWave + lane;
        const bool pass = i < n && lin_bin(x[k], hg) >= bcut;
        const uint64_t bm = __ballot(pass);
        const int pos = base + lanes_below(bm);
        if (pass && pos < r_cap)   // a 32-bit byte offset from the uniform base (one address operation)
          *reinterpret_cast<float2*>(reinterpret_cast<char*>(dst) + (uint32_t)pos * 8u) =
              make_float2(x[k], __int_as_float(t0 + i));
        base += (int)__popcll(bm);
      }
    }
    if (lane == 0) {
      meta[(size_t)(u * G + g) * n_chunks + c] = make_int2(bcut | (top << 16), run);
      if (c == 0) hpw[u * G + g] = make_float4(hg.rg, hg.inv_w, hg.eps, 0.f);
    }
  }
}


// ====================================================================== select
template <typename KT, int D, int NT>
__global__ void __launch_bounds__(NT)
topk_select_kernel(const float* __restrict__ q, int G, const KT* __restrict__ kb, int64_t ustride,
                   int n_sink, int L_mid, int ch, int n_chunks, int r_cap, int K, int e_max,
                   const float4* __restrict__ hpw, const float2* __restrict__ ent,
                   const int2* __restrict__ meta, int32_t* __restrict__ idx_out,
                   float* __restrict__ sc_out, float inv_sqrt_d) {
  extern __shared__ __align__(16) float dyn[];
  const int ug = blockIdx.x, u = ug / G;
  HeadSelect<KT, D, NT> sel;
  sel.ug = ug;
  sel.qg = q + (size_t)ug * D;
  sel.mt = meta + (size_t)ug * n_chunks;
  sel.en = ent + (size_t)ug * n_chunks * r_cap;
  sel.kunit = kb + (size_t)u * ustride;
  sel.n_sink = n_sink;
  sel.L_mid = L_mid;
  sel.ch = ch;
  sel.n_chunks = n_chunks;
  sel.r_cap = r_cap;
  sel.K = K;
  sel.e_max = e_max;
  sel.inv_sqrt_d = inv_sqrt_d;
  sel.load(hpw);
  SelOut out;
  out.io = idx_out + (size_t)ug * K;
  out.so = sc_out + (size_t)ug * K;
  sel.run(dyn, reinterpret_cast<int*>(dyn + e_max), out);
}

// ====================================================================== launch
namespace {

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
hipError_t launch_select_t(const TopkPlan& pl, const float* q, int G, const rma_kv& kv,
                           const rma_span& sp, int K, int32_t* idx, float* sel, uint8_t* ws,
                           hipStream_t st) {
  const int L_mid = (int)(sp.L - sp.n_sink - sp.n_tail);
  const KT* kb = static_cast<const KT*>(kv.k);
  const float2* ent = reinterpret_cast<const float2*>(ws + pl.off_ent);
  const int2* meta = reinterpret_cast<const int2*>(ws + pl.off_meta);
  const float4* hpw = reinterpret_cast<const float4*>(ws + pl.off_hp);
  // dynamic LDS: the union (score, position) pairs, within the per-block limit
  // left by the kernel's own (static) LDS.  Many (unit, head) blocks with short
  // report lists: 256 threads each, so that several share a CU; otherwise 1024.
  const bool small = kv.n_units * G >= 1024 && (int64_t)pl.n_chunks * pl.r_cap <= 8 * 256;
  const size_t sl = small ? kernel_static_lds<&topk_select_kernel<KT, D, 256>>()
                           : kernel_static_lds<&topk_select_kernel<KT, D, kSelThreads>>();
  const size_t lds_limit = device_info().lds_per_block;
  if (sl + 8 > lds_limit) return hipErrorInvalidConfiguration;
  int e_max = std::min<int>(pl.e_max, (int)((lds_limit - sl) / 8));
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

template <typename KT, int D>
hipError_t launch_scan_t(const TopkPlan& pl, const float* q, int G, const rma_kv& kv,
                         const rma_span& sp, const float* kappa, uint8_t* ws, hipStream_t st) {
  const int L_mid = (int)(sp.L - sp.n_sink - sp.n_tail);
  return launch_scan_g<KT, D>(G, dim3(kv.n_units, pl.n_chunks), st, q, static_cast<const KT*>(kv.k),
                              kv.unit_stride, sp.n_sink, L_mid, pl, kappa,
                              reinterpret_cast<float2*>(ws + pl.off_ent),
                              reinterpret_cast<int2*>(ws + pl.off_meta),
                              reinterpret_cast<float4*>(ws + pl.off_hp));
}

}  // namespace

hipError_t launch_topk_scan(const TopkPlan& pl, const float* q, int G, const rma_kv& kv,
                            const rma_span& sp, const float* kappa, uint8_t* ws, hipStream_t st) {
  if (kv.dtype == RMA_BF16) {
    if (kv.d == 64) return launch_scan_t<uint16_t, 64>(pl, q, G, kv, sp, kappa, ws, st);
    return launch_scan_t<uint16_t, 128>(pl, q, G, kv, sp, kappa, ws, st);
  }
  if (kv.d == 64) return launch_scan_t<float, 64>(pl, q, G, kv, sp, kappa, ws, st);
  return launch_scan_t<float, 128>(pl, q, G, kv, sp, kappa, ws, st);
}

hipError_t launch_topk_select(const TopkPlan& pl, const float* q, int G, const rma_kv& kv,
                              const rma_span& sp, int K, int32_t* idx, float* sel, uint8_t* ws,
                              hipStream_t st) {
  if (kv.dtype == RMA_BF16) {
    if (kv.d == 64) return launch_select_t<uint16_t, 64>(pl, q, G, kv, sp, K, idx, sel, ws, st);
    return launch_select_t<uint16_t, 128>(pl, q, G, kv, sp, K, idx, sel, ws, st);
  }
  if (kv.d == 64) return launch_select_t<float, 64>(pl, q, G, kv, sp, K, idx, sel, ws, st);
  return launch_select_t<float, 128>(pl, q, G, kv, sp, K, idx, sel, ws, st);
}

hipError_t launch_topk(const TopkPlan& pl, const float* q, int G, const rma_kv& kv,
                       const rma_span& sp, const float* kappa, int K, int32_t* idx, float* sel,
                       uint8_t* ws, hipStream_t st) {
  const hipError_t e = launch_topk_scan(pl, q, G, kv, sp, kappa, ws, st);
  if (e != hipSuccess) return e;
  return launch_topk_select(pl, q, G, kv, sp, K, idx, sel, ws, st);
}

}  // namespace rma
