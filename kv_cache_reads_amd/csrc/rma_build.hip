// Prefill summary builder and the phi feature kernel ("Residual-Mass Accounting
// for Partial-KV Decoding": §1 and §4.1, summaries S = sum phi_k(k_i) v_i^T and
// u = sum phi_k(k_i) over the mid-region; App. C.1 for the positive map).
//
// build_mfma  (bf16 K/V, bf16 phi rows, computed phi)  grid (chunks, units); with
//   STORE false the phi rows are not written (decode recomputes the retrieved
//   ones with this same instruction sequence),
//   m/16 waves (one 16-feature tile each), 64-token tiles through LDS:
//     Z = K_tile W^T        v_mfma_f32_16x16x32_bf16; W is split into bf16
//                           hi + lo parts (K is exactly bf16), so Z carries
//                           ~2^-17 relative error instead of bf16's 2^-9
//     Phi = elu(Z + b) + 1  rounded once to bf16; the rounded rows are both
//                           stored and summed, so decode subtracts exactly
//                           what the summaries contain
//     S += Phi^T V_tile     v_mfma_f32_16x16x32_bf16 with the token index as
//                           the contraction; A comes straight from the step-1
//                           accumulators, B is gathered from the V tile in LDS
//                           with the same token permutation
//     u += column sums of the rounded Phi;  kappa = max ||k_i||_2 (rounded up)
// build_valu  (every other dtype combination, or phi given as an input)
// build_reduce  sums the per-chunk partials in chunk order (deterministic).
#include "rma_device.hpp"
#include "rma_internal.hpp"

#include <math.h>

#include <type_traits>

namespace rma {


// upper bound of sqrt(x) for a sum of squares computed in fp32 over <= 128 terms (its
// rounding is below 128 * 2^-24 relative; the factor covers that and the root's)
__device__ __forceinline__ float norm_upper(float sumsq) { return sqrtf(sumsq) * (1.0f + 1e-5f); }

// ====================================================================== MFMA builder
// INJ: the Phi rows are given (read from phik) instead of computed; step 1 is
// skipped and the rows' tile is staged in LDS beside K and V.
template <int D, int M, bool STORE, bool INJ>
__global__ void __launch_bounds__(M * 4)
build_mfma_kernel(const uint16_t* __restrict__ kb, const uint16_t* __restrict__ vb, int64_t ustride,
                  int n_sink, int L_mid, int ch, int n_chunks, int m0, int len, int acc,
                  const float* __restrict__ W, const float* __restrict__ bias, int P,
                  uint16_t* __restrict__ phik, float* __restrict__ pS, float* __restrict__ pu,
                  float* __restrict__ pk) {
  constexpr int NW = M / 16;              // one 16-feature tile per wave
  constexpr int NT = NW * 64;
  constexpr int TT = 64;                  // tokens per tile
  constexpr int NTT = TT / 16;            // 16-token MFMA tiles per tile
  constexpr int KB = TT / 32;             // 32-token contraction blocks per tile
  constexpr int KS = D / 32;              // k-steps of step 1
  constexpr int CT = D / 16;              // column tiles of step 2
  constexpr int KROW = D + 8;             // Ks row stride (bf16): 16 B pad -> 4-bank shift per row
  constexpr int VROW = D + 16;            // Vs row stride (bf16): rows 32 dwords + 8 (mod 64) apart,
                                          // so the 8 rows one transposing read touches per
                                          // half-wave cover the 64 banks once
  constexpr int PROW = INJ ? M + 16        // given rows: read back transposed, as Vs
                          : M + 4;        // Phi staging row stride: 8 B pad -> the 4 lane groups
                                          // of a step-1 tile land 8 banks apart
  constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
  constexpr int LCH = TT * CPR / NT;      // 16-byte chunks per thread per tile (K or V)
  constexpr int PCH = INJ ? TT * (M / 8) / NT : 1;   // 16-byte chunks per thread of a given Phi tile
  static_assert(LCH >= 1 && TT * CPR % NT == 0, "tile shape");
  static_assert(!(INJ && STORE), "given rows are not stored");

  // two buffers of each tile: tile j is computed from buffer j % 2 while tile
  // j + 1 is staged into the other, so one barrier per tile orders both
  constexpr int KBUF = TT * KROW, VBUF = TT * VROW, PBUF = (STORE || INJ) ? TT * PROW : 4;
  __shared__ __align__(16) uint16_t Ks[2 * KBUF];
  __shared__ __align__(16) uint16_t Vs[2 * VBUF];
  __shared__ __align__(16) uint16_t Ps[2 * PBUF];
  __shared__ float s_kap[NW];

  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g4 = lane >> 4;
  const int p = u % P;
  // chunk c of the mid-region positions [m0, m0 + len)
  const int t0 = m0 + c * ch;
  const int n = min(ch, m0 + len - t0);
  const uint16_t* kp = kb + (size_t)u * ustride + (size_t)(n_sink + t0) * D;
  const uint16_t* vp = vb + (size_t)u * ustride + (size_t)(n_sink + t0) * D;
  uint16_t* php = (STORE || INJ) ? phik + ((size_t)u * L_mid + t0) * M : nullptr;
  // range-checked views of this chunk: rows past n load as zeros, Phi stores past n drop
  const auto rk = make_rsrc(kp, (uint32_t)n * D * 2), rv = make_rsrc(vp, (uint32_t)n * D * 2);
  const auto rph = make_rsrc(php, (STORE || INJ) ? (uint32_t)n * M * 2 : 0u);
  const int f = wave * 16 + l16;          // this lane's feature in step 1

  // this lane's W row piece and bias, issued ahead of the first tiles (buffer
  // loads stay in program order relative to the tile loads and the barrier)
  const auto rw = make_rsrc(W + (size_t)p * M * D, M * D * 4);
  const auto rb = make_rsrc(bias + (size_t)p * M, M * 4);
  float wv[KS][8];
  float bf = 0.f;
  if constexpr (!INJ) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t wo = (f * D + 32 * ks + 8 * g4) * 4;
      const uint4 a = buf_ld16(rw, wo), b = buf_ld16(rw, wo + 16);
      const uint32_t x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[ks][e] = __uint_as_float(x[e]);
    }
    bf = buf_ld_f32(rb, f * 4);
  }
  bf16x8_t Whi[KS], Wlo[KS];             // W (fp32) as bf16 hi + lo B-operands
  u16x8_t ones_v;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones_v[e] = 0x3F80;  // bf16 1.0: u = Phi^T 1 on the MFMA
  const bf16x8_t Bones = as_bf16x8(ones_v);

  f32x4 Sacc[CT], Uacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) Sacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float kapmax = 0.f;

  auto load_tile = [&](uint4 (&kr)[LCH], uint4 (&vr)[LCH], uint4 (&pr)[PCH], int tok0) {
#pragma unroll
    for (int j = 0; j < LCH; ++j) {
      const int chunk = tid + NT * j;
      const int row = chunk / CPR, cc = chunk % CPR;
      const uint32_t off = (uint32_t)((tok0 + row) * D + cc * 8) * 2;
      kr[j] = buf_ld16_nt(rk, off);
      vr[j] = buf_ld16_nt(rv, off);
    }
    if constexpr (INJ) {
#pragma unroll
      for (int j = 0; j < PCH; ++j) {
        const int chunk = tid + NT * j;
        const int row = chunk / (M / 8), cc = chunk % (M / 8);
        pr[j] = buf_ld16_nt(rph, (uint32_t)((tok0 + row) * M + cc * 8) * 2);
      }
    }
  };
  // K and V rows (and given Phi rows) as they are (16-byte writes)
  auto stage_tile = [&](int b, const uint4 (&kr)[LCH], const uint4 (&vr)[LCH], const uint4 (&pr)[PCH]) {
#pragma unroll
    for (int j = 0; j < LCH; ++j) {
      const int chunk = tid + NT * j;
      const int row = chunk / CPR, cc = chunk % CPR;
      *reinterpret_cast<uint4*>(Ks + b * KBUF + row * KROW + cc * 8) = kr[j];
      *reinterpret_cast<uint4*>(Vs + b * VBUF + row * VROW + cc * 8) = vr[j];
    }
    if constexpr (INJ) {
#pragma unroll
      for (int j = 0; j < PCH; ++j) {
        const int chunk = tid + NT * j;
        const int row = chunk / (M / 8), cc = chunk % (M / 8);
        *reinterpret_cast<uint4*>(Ps + b * PBUF + row * PROW + cc * 8) = pr[j];
      }
    }
  };
  // Step-2 B operand of one 16-column tile: eight tokens of one V column per lane,
  // gathered by two transposing LDS reads (ds_read_b64_tr_b16).  Within a 16-lane
  // group, lane j receives element e from the 8-byte piece that lane 4e + j/4
  // addressed, at position j%4; so lane l' points at token (l'/4) of the group's
  // 4-token block and at columns 4*(l'%4) .. +3 of the tile, and lane j gets the
  // four tokens of column j.
  const int tr_row = 4 * g4 + (l16 >> 2), tr_col = 4 * (l16 & 3);
  auto ld_tr_in = [&](const uint16_t* tile, int stride, int row, int col) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s*)(tile + row * stride + col));
    return __builtin_bit_cast(uint2, r);
  };
  auto compute_tile = [&](int tok0, auto buf_tag, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr int b = decltype(buf_tag)::value;
    const uint16_t* const Kb = Ks + b * KBUF;
    uint16_t* const Pb = Ps + b * PBUF;
    auto ld_tr = [&](int row, int col) { return ld_tr_in(Vs + b * VBUF, VROW, row, col); };
    // kappa: the largest squared key norm (NT/TT threads per token row, bf16 pair
    // dots; the root is taken once per chunk)
    {
      constexpr int TPR = NT / TT, EPT = D / TPR;
      const int row = tid / TPR, qd = tid % TPR;
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < EPT; e += 8) {
        const uint4 w = *reinterpret_cast<const uint4*>(Kb + row * KROW + qd * EPT + e);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x2_t h = __builtin_bit_cast(bf16x2_t, ws[i]);
          ss = __builtin_amdgcn_fdot2_f32_bf16(h, h, ss, false);
        }
      }
      ss = lane_group_sum<TPR>(ss);
      if (FULL || tok0 + row < n) kapmax = fmaxf(kapmax, ss);
    }
    // step 1: Z = K W^T for this wave's features, epilogue phi, bf16 pairs kept
    // (given rows: the four tokens of this lane's feature, read transposed;
    // rows past the chunk were loaded as zeros)
    uint32_t phv[NTT][2];
    if constexpr (INJ) {
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        const uint2 r = ld_tr_in(Pb, PROW, tt * 16 + tr_row, wave * 16 + tr_col);
        phv[tt][0] = r.x;
        phv[tt][1] = r.y;
      }
    }
#pragma unroll
    for (int tt = 0; tt < (INJ ? 0 : NTT); ++tt) {
      const f32x4 acc = proj_tile16<KS>(Kb + (tt * 16 + l16) * KROW + 8 * g4, Whi, Wlo);
      float ph[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = tt * 16 + 4 * g4 + r;
        ph[r] = (FULL || tok0 + row < n) ? phi_elu1(acc[r] + bf) : 0.f;  // padding rows add nothing
      }
      const uint32_t p01 = pack_bf16x2(ph[0], ph[1]), p23 = pack_bf16x2(ph[2], ph[3]);
      phv[tt][0] = p01;
      phv[tt][1] = p23;
      if constexpr (STORE) {
        const int row0 = tt * 16 + 4 * g4;
        Pb[(row0 + 0) * PROW + f] = (uint16_t)p01;
        Pb[(row0 + 1) * PROW + f] = (uint16_t)(p01 >> 16);
        Pb[(row0 + 2) * PROW + f] = (uint16_t)p23;
        Pb[(row0 + 3) * PROW + f] = (uint16_t)(p23 >> 16);
      }
    }
    // step 2: S += Phi^T V, u += Phi^T 1 over 32-token blocks.  Hardware k-slot e
    // of lane group g4 is token 32*kb + 4*g4 + e (e < 4) or 32*kb + 16 + 4*g4 +
    // (e - 4) (e >= 4): exactly where step 1 left the Phi values.
#pragma unroll
    for (int kb2 = 0; kb2 < KB; ++kb2) {
      // the packed pairs already are the operand: element e of lane group g4
      const bf16x8_t Aph = __builtin_bit_cast(
          bf16x8_t, make_uint4(phv[2 * kb2][0], phv[2 * kb2][1], phv[2 * kb2 + 1][0], phv[2 * kb2 + 1][1]));
      Uacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aph, Bones, Uacc, 0, 0, 0);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const uint2 lo4 = ld_tr(32 * kb2 + tr_row, ct * 16 + tr_col);
        const uint2 hi4 = ld_tr(32 * kb2 + 16 + tr_row, ct * 16 + tr_col);
        const bf16x8_t Bv = __builtin_bit_cast(bf16x8_t, make_uint4(lo4.x, lo4.y, hi4.x, hi4.y));
        Sacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aph, Bv, Sacc[ct], 0, 0, 0);
      }
    }
  };
  // store the Phi rows of the tile at tok0 from buffer b, after the barrier that
  // follows its computation (16-byte pieces, coalesced; rows are 8-byte aligned in
  // LDS).  tok0 = -TT, before the first tile, gives offsets that wrap past the
  // range, so those stores are dropped like the ones past the chunk.
  auto store_rows = [&](int tok0, int b) {
    constexpr int PCR = M / 8;
    static_assert(TT * PCR % NT == 0, "Phi tile store shape");
#pragma unroll
    for (int j = 0; j < TT * PCR / NT; ++j) {
      const int chunk = tid + NT * j;
      const int row = chunk / PCR, cc = chunk % PCR;
      const uint2 x = *reinterpret_cast<const uint2*>(Ps + b * PBUF + row * PROW + cc * 8);
      const uint2 y = *reinterpret_cast<const uint2*>(Ps + b * PBUF + row * PROW + cc * 8 + 4);
      buf_st16(rph, (uint32_t)((tok0 + row) * M + cc * 8) * 2, make_uint4(x.x, x.y, y.x, y.y));
    }
  };

  // Tile j: its K/V (and given Phi) registers load three tiles ahead, they are
  // staged into LDS buffer j % 2 one tile ahead, and the Phi rows it leaves in
  // that buffer are stored one tile after; one barrier closes each tile.  Two
  // register stages alternate.  Every pass issues the same memory operations
  // (tiles past the chunk load as zeros without touching memory, Phi stores
  // outside it are dropped, and a tile past an odd tile count is computed as
  // padding), so the wait before each staging step covers only the loads of the
  // tile being staged, not the stores and loads issued after them.
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  uint4 kA[LCH], vA[LCH], kB[LCH], vB[LCH], pA[PCH], pB[PCH];
  load_tile(kA, vA, pA, 0);
  load_tile(kB, vB, pB, TT);
  __syncthreads();
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): nothing in flight on entry
  if constexpr (!INJ) split_w_values<KS>(wv, Whi, Wlo);
  stage_tile(0, kA, vA, pA);
  load_tile(kA, vA, pA, 2 * TT);
  __syncthreads();
  int t_last = -TT;
  for (int tok0 = 0; tok0 < n; tok0 += 2 * TT) {
    stage_tile(1, kB, vB, pB);
    load_tile(kB, vB, pB, tok0 + 3 * TT);
    if constexpr (STORE) store_rows(tok0 - TT, 1);
    if (tok0 + TT <= n) compute_tile(tok0, B0{}, std::true_type{});
    else compute_tile(tok0, B0{}, std::false_type{});
    __syncthreads();
    stage_tile(0, kA, vA, pA);
    load_tile(kA, vA, pA, tok0 + 4 * TT);
    if constexpr (STORE) store_rows(tok0, 0);
    if (tok0 + 2 * TT <= n) compute_tile(tok0 + TT, B1{}, std::true_type{});
    else compute_tile(tok0 + TT, B1{}, std::false_type{});
    __syncthreads();
    t_last = tok0 + TT;
  }
  if constexpr (STORE) store_rows(t_last, 1);

  // ---- partials of this chunk
  float* Sp = pS + ((size_t)u * n_chunks + c) * M * D;
  const int fb = wave * 16;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // acc: the summaries already hold earlier tokens (one chunk writes them directly)
      float* dst = Sp + (size_t)(fb + 4 * g4 + r) * D + ct * 16 + l16;
      *dst = acc ? *dst + Sacc[ct][r] : Sacc[ct][r];
    }
  if (l16 == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* dst = pu + ((size_t)u * n_chunks + c) * M + fb + 4 * g4 + r;
      *dst = acc ? *dst + Uacc[r] : Uacc[r];
    }
  }
  kapmax = wave_max_dpp(kapmax);
  if (lane == 0) s_kap[wave] = kapmax;
  __syncthreads();
  if (tid == 0) {
    float mx = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, s_kap[w]);
    float* dst = pk + (size_t)u * n_chunks + c;
    *dst = acc ? fmaxf(*dst, norm_upper(mx)) : norm_upper(mx);
  }
}

// ====================================================================== VALU builder
template <typename KT, typename PT, int D, int M>
__global__ void __launch_bounds__(256)
build_valu_kernel(const KT* __restrict__ kb, const KT* __restrict__ vb, int64_t ustride, int n_sink,
                  int L_mid, int ch, int n_chunks, int m0, int len, int acc_in, const float* __restrict__ W,
                  const float* __restrict__ bias, int P, PT* __restrict__ phik,
                  float* __restrict__ pS, float* __restrict__ pu, float* __restrict__ pk) {
  constexpr int TT = 32;
  __shared__ float Kt[TT][D + 1];
  __shared__ float Vt[TT][D + 1];
  __shared__ float Pt[TT][129];
  __shared__ float s_kap[256];
  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int p = u % P;
  const int t0 = m0 + c * ch;   // chunk c of the mid-region positions [m0, m0 + len)
  const int n = min(ch, m0 + len - t0);
  const KT* kp = kb + (size_t)u * ustride + (size_t)(n_sink + t0) * D;
  const KT* vp = vb + (size_t)u * ustride + (size_t)(n_sink + t0) * D;
  PT* php = phik + ((size_t)u * L_mid + t0) * M;
  // thread -> (feature, column range) for S: M*D/256 accumulators
  constexpr int cols_per = (M * D) / 256;       // 16, 32 or 64
  const int f_s = tid / (D / cols_per);          // feature of this thread's S slice
  const int c_s = (tid % (D / cols_per)) * cols_per;
  float acc[cols_per];
#pragma unroll
  for (int i = 0; i < cols_per; ++i) acc[i] = 0.f;
  float uacc = 0.f, kap = 0.f;

  for (int tok0 = 0; tok0 < n; tok0 += TT) {
    for (int i = tid; i < TT * D; i += 256) {
      const int r = i / D, j = i % D;
      const bool ok = tok0 + r < n;
      Kt[r][j] = ok ? ld_f32(kp, (size_t)(tok0 + r) * D + j) : 0.f;
      Vt[r][j] = ok ? ld_f32(vp, (size_t)(tok0 + r) * D + j) : 0.f;
    }
    __syncthreads();
    if (tid < TT && tok0 + tid < n) {
      float ss = 0.f;
      for (int j = 0; j < D; ++j) ss = __fmaf_rn(Kt[tid][j], Kt[tid][j], ss);
      kap = fmaxf(kap, sqrtf(ss) * (1.0f + 1e-5f));
    }
    for (int i = tid; i < TT * M; i += 256) {
      const int r = i / M, f = i % M;
      float ph = 0.f;
      if (tok0 + r < n) {
        if (W != nullptr) {
          float z = bias[(size_t)p * M + f];
          const float* wr = W + ((size_t)p * M + f) * D;
          for (int j = 0; j < D; ++j) z = __fmaf_rn(wr[j], Kt[r][j], z);
          ph = st_round<PT>(phi_elu1(z));
          st_elem(php, (size_t)(tok0 + r) * M + f, ph);
        } else {
          ph = ld_f32(php, (size_t)(tok0 + r) * M + f);
        }
      }
      Pt[r][f] = ph;
    }
    __syncthreads();
    for (int r = 0; r < TT; ++r) {
      const float ph = Pt[r][f_s];
#pragma unroll
      for (int i = 0; i < cols_per; ++i) acc[i] = __fmaf_rn(ph, Vt[r][c_s + i], acc[i]);
      if (c_s == 0) uacc += ph;
    }
    __syncthreads();
  }
  float* Sp = pS + ((size_t)u * n_chunks + c) * M * D;
#pragma unroll
  for (int i = 0; i < cols_per; ++i) {
    float* dst = Sp + (size_t)f_s * D + c_s + i;
    *dst = acc_in ? *dst + acc[i] : acc[i];
  }
  if (c_s == 0) {
    float* dst = pu + ((size_t)u * n_chunks + c) * M + f_s;
    *dst = acc_in ? *dst + uacc : uacc;
  }
  s_kap[tid] = kap;
  __syncthreads();
  if (tid == 0) {
    float mx = 0.f;
    for (int i = 0; i < TT; ++i) mx = fmaxf(mx, s_kap[i]);
    float* dst = pk + (size_t)u * n_chunks + c;
    *dst = acc_in ? fmaxf(*dst, mx) : mx;
  }
}

// ====================================================================== reduce
// Sums the per-chunk partials of each unit.  A block covers 64 float4 outputs of
// one unit; wave w sums chunks [w*nq, (w+1)*nq) in order (its loads issued
// together, 16 at a time) and the four wave sums are added in wave order, so
// the result is the same on every run.
constexpr int kRedBatch = 16;
__global__ void __launch_bounds__(256)
build_reduce_kernel(const float* __restrict__ pS, const float* __restrict__ pu,
                    const float* __restrict__ pk, int n_chunks, int M, int D, int add,
                    float* __restrict__ S, float* __restrict__ u_, float* __restrict__ kappa) {
  __shared__ float4 part[4][64];
  const int u = blockIdx.y, tid = threadIdx.x, o = tid & 63, w = tid >> 6;
  const int nS4 = M * D / 4, nU4 = M / 4;
  const int e = blockIdx.x * 64 + o;               // float4 output index within the unit
  const bool live = e < nS4 + nU4;
  const float4* src = nullptr;
  size_t stride = 0;
  if (live) {
    if (e < nS4) {
      src = reinterpret_cast<const float4*>(pS + (size_t)u * n_chunks * M * D) + e;
      stride = (size_t)nS4;
    } else {
      src = reinterpret_cast<const float4*>(pu + (size_t)u * n_chunks * M) + (e - nS4);
      stride = (size_t)nU4;
    }
  }
  const int nq = (n_chunks + 3) / 4;
  const int c0 = min(n_chunks, w * nq), c1 = min(n_chunks, c0 + nq);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (live) {
    for (int cb = c0; cb < c1; cb += kRedBatch) {
      float4 t[kRedBatch];
#pragma unroll
      for (int k = 0; k < kRedBatch; ++k)
        if (cb + k < c1) t[k] = src[(size_t)(cb + k) * stride];
#pragma unroll
      for (int k = 0; k < kRedBatch; ++k)
        if (cb + k < c1) {
          acc.x += t[k].x;
          acc.y += t[k].y;
          acc.z += t[k].z;
          acc.w += t[k].w;
        }
    }
  }
  part[w][o] = acc;
  __syncthreads();
  if (w == 0 && live) {
    float4 r = part[0][o];
#pragma unroll
    for (int k = 1; k < 4; ++k) {
      r.x += part[k][o].x;
      r.y += part[k][o].y;
      r.z += part[k][o].z;
      r.w += part[k][o].w;
    }
    float4* dst = e < nS4 ? reinterpret_cast<float4*>(S + (size_t)u * M * D) + e
                          : reinterpret_cast<float4*>(u_ + (size_t)u * M) + (e - nS4);
    if (add) {  // add to the summaries of earlier tokens
      const float4 o = *dst;
      r.x = o.x + r.x;
      r.y = o.y + r.y;
      r.z = o.z + r.z;
      r.w = o.w + r.w;
    }
    *dst = r;
  }
  if (blockIdx.x == 0 && w == 1) {  // kappa: the chunk maxima spread over one wave
    float v = 0.f;
    for (int c = o; c < n_chunks; c += kWave) v = fmaxf(v, pk[(size_t)u * n_chunks + c]);
    v = wave_max_dpp(v);
    if (o == 0) kappa[u] = add ? fmaxf(kappa[u], v) : v;
  }
}

// ====================================================================== phi features
// Block = (8 rows, unit, 16 features).  A 16-lane group owns one feature: its
// lanes hold D/16 consecutive weights (coalesced 16-byte loads, issued before
// the rows arrive) and the group sums its partial dots with DPP.
template <typename XT, typename PT, int D>
__global__ void __launch_bounds__(256)
phi_kernel(const XT* __restrict__ x, int64_t xstride, int rows, const float* __restrict__ W,
           const float* __restrict__ bias, int M, int P, PT* __restrict__ phi) {
  constexpr int RB = 8, EPL = D / 16;
  __shared__ __align__(16) float xs[RB][D];
  const int r0 = blockIdx.x * RB, u = blockIdx.y, tid = threadIdx.x;
  const int f = blockIdx.z * 16 + (tid >> 4), j = tid & 15;
  const int p = u % P;
  const int nr = min(RB, rows - r0);
  float w[EPL];
  const float4* wr = reinterpret_cast<const float4*>(W + ((size_t)p * M + f) * D + j * EPL);
#pragma unroll
  for (int e = 0; e < EPL / 4; ++e) {
    const float4 t = wr[e];
    w[4 * e] = t.x;
    w[4 * e + 1] = t.y;
    w[4 * e + 2] = t.z;
    w[4 * e + 3] = t.w;
  }
  const float bf = bias[(size_t)p * M + f];
  for (int i = tid; i < nr * D; i += 256)
    xs[i / D][i % D] = ld_f32(x, (size_t)u * xstride + (size_t)(r0 + i / D) * D + i % D);
  __syncthreads();
  for (int r = 0; r < nr; ++r) {
    float z = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const float4 xv = *reinterpret_cast<const float4*>(&xs[r][j * EPL + e]);
      z = __fmaf_rn(w[e], xv.x, z);
      z = __fmaf_rn(w[e + 1], xv.y, z);
      z = __fmaf_rn(w[e + 2], xv.z, z);
      z = __fmaf_rn(w[e + 3], xv.w, z);
    }
    z = lane_group_sum<16>(z);
    if (j == 0) st_elem(phi, ((size_t)u * rows + r0 + r) * M + f, st_round<PT>(phi_elu1(z + bf)));
  }
}

// ====================================================================== launch
hipError_t launch_build(const BuildPlan& pl, const rma_kv& kv, const rma_span& sp, int m0, int len,
                        bool acc, const float* W, const float* b, int m, int P, void* phi_k,
                        int phi_dtype, float* S, float* u, float* kappa, uint8_t* ws,
                        hipStream_t st) {
  const int L_mid = (int)(sp.L - sp.n_sink - sp.n_tail);
  const int acc_direct = (acc && pl.n_chunks == 1) ? 1 : 0;   // partials never accumulate
  // one chunk per unit: the builder writes S, u and kappa itself
  const bool direct = pl.n_chunks == 1;
  float* pS = direct ? S : reinterpret_cast<float*>(ws + pl.off_S);
  float* pu = direct ? u : reinterpret_cast<float*>(ws + pl.off_u);
  float* pk = direct ? kappa : reinterpret_cast<float*>(ws + pl.off_kap);
  if (pl.n_chunks > 0) {
    const dim3 grid(pl.n_chunks, kv.n_units);
    hipError_t e = hipSuccess;
    if (pl.mfma) {
      const uint16_t* kk = static_cast<const uint16_t*>(kv.k);
      const uint16_t* vv = static_cast<const uint16_t*>(kv.v);
      uint16_t* ph = static_cast<uint16_t*>(phi_k);
#define RMA_BM1(DD, MM, STO, INJ)                                                                    \
  e = launch_kernel("build_mfma_kernel", build_mfma_kernel<DD, MM, STO, INJ>, grid, dim3(MM * 4), 0, st, \
                    kk, vv, kv.unit_stride, sp.n_sink, L_mid, pl.ch, pl.n_chunks, m0, len, acc_direct, \
                    W, b, P, ph, pS, pu, pk)
#define RMA_BM(DD, MM)                                                                               \
  do {                                                                                               \
    if (W == nullptr) RMA_BM1(DD, MM, false, true);   /* given rows */                               \
    else if (ph != nullptr) RMA_BM1(DD, MM, true, false);                                            \
    else RMA_BM1(DD, MM, false, false);                                                              \
  } while (0)
      if (kv.d == 64 && m == 64) RMA_BM(64, 64);
      else if (kv.d == 64) RMA_BM(64, 128);
      else if (m == 64) RMA_BM(128, 64);
      else RMA_BM(128, 128);
#undef RMA_BM
#undef RMA_BM1
    } else {
#define RMA_BV1(KT, PT, DD, MM)                                                                      \
  e = launch_kernel("build_valu_kernel", build_valu_kernel<KT, PT, DD, MM>, grid, dim3(256), 0, st,  \
                    static_cast<const KT*>(kv.k), static_cast<const KT*>(kv.v), kv.unit_stride,      \
                    sp.n_sink, L_mid, pl.ch, pl.n_chunks, m0, len, acc_direct, W, b, P,              \
                    static_cast<PT*>(phi_k), pS, pu, pk)
#define RMA_BV(KT, PT)                                                 \
  do {                                                                 \
    if (kv.d == 64 && m == 64) RMA_BV1(KT, PT, 64, 64);                \
    else if (kv.d == 64) RMA_BV1(KT, PT, 64, 128);                     \
    else if (m == 64) RMA_BV1(KT, PT, 128, 64);                        \
    else RMA_BV1(KT, PT, 128, 128);                                    \
  } while (0)
      if (kv.dtype == RMA_BF16) {
        if (phi_dtype == RMA_BF16) RMA_BV(uint16_t, uint16_t); else RMA_BV(uint16_t, float);
      } else {
        if (phi_dtype == RMA_BF16) RMA_BV(float, uint16_t); else RMA_BV(float, float);
      }
#undef RMA_BV1
#undef RMA_BV
    }
    if (e != hipSuccess) return e;
  }
  if (direct) return hipSuccess;
  const int blocks = (int)ceil_div((int64_t)m * kv.d / 4 + m / 4, 64);
  return launch_kernel("build_reduce_kernel", build_reduce_kernel, dim3(blocks, kv.n_units),
                       dim3(256), 0, st, pS, pu, pk, pl.n_chunks, m, kv.d, acc ? 1 : 0, S, u, kappa);
}

hipError_t launch_phi(const void* x, int x_dtype, int n_units, int64_t rows, int64_t xstride, int d,
                      const float* W, const float* b, int m, int P, void* phi, int phi_dtype,
                      hipStream_t st) {
  const dim3 grid((unsigned)ceil_div(rows, 8), n_units, m / 16);
  hipError_t e = hipSuccess;
#define RMA_PHI1(XT, PT, DD)                                                                         \
  e = launch_kernel("phi_kernel", phi_kernel<XT, PT, DD>, grid, dim3(256), 0, st,                    \
                    static_cast<const XT*>(x), xstride, (int)rows, W, b, m, P, static_cast<PT*>(phi))
#define RMA_PHI(XT, PT)                    \
  do {                                     \
    if (d == 64) RMA_PHI1(XT, PT, 64);     \
    else RMA_PHI1(XT, PT, 128);            \
  } while (0)
  if (x_dtype == RMA_F32) {
    if (phi_dtype == RMA_F32) RMA_PHI(float, float); else RMA_PHI(float, uint16_t);
  } else {
    if (phi_dtype == RMA_F32) RMA_PHI(uint16_t, float); else RMA_PHI(uint16_t, uint16_t);
  }
#undef RMA_PHI1
#undef RMA_PHI
  return e;
}

}  // namespace rma
