// The pages' feature-map family ("Residual-Mass Accounting for Partial-KV
// Decoding": §4.4, the maps are head-specific one-block ReZero MLPs; App. C.1
// "Why positivity matters", their outputs are exponentiated; §8 "Scope and
// runtime", d_phi = 64 and the parameter totals that fix width 512 and the
// biases):
//
//   h0 = W_in x + b_in,   h1 = h0 + alpha (W_2 relu(W_1 h0 + b_1) + b_2),
//   phi(x) = exp(W_o h1 + b_o)                      (width H = 512, ReLU).
//
// One block (four waves) runs all four layers for a tile of RT rows of one
// unit on the matrix cores (v_mfma_f32_16x16x32_bf16: bf16 operands, fp32
// sums).  The activations stay in LDS as bf16 (the operands of the next
// product); each wave owns a quarter of every layer's output columns and
// streams its weight rows from L2 as the B operand, several 32-wide k-steps ahead
// (the next layer's first pieces are issued before this layer's epilogue).
#include "rma_device.hpp"
#include "rma_internal.hpp"

#include <math.h>

namespace rma {

namespace {

constexpr int kMlpWaves = 4;
constexpr int kMlpThreads = kMlpWaves * 64;

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// The weight pieces of one layer in flight: a ring of DEPTH k-steps of B
// pieces.  W (N x 32*KS) is in the matrix-core tile order [k-step][column tile
// of 16][lane][8], so that one wave's pieces of a (k-step, column tile) are
// one contiguous kilobyte; the lane's piece is weight row col0 + ct*16 + l16,
// k = 32*ks + 8*g4 .. +8.
template <int NCT, int KS, int NPF>
struct WeightRing {
  static constexpr int DEPTH = NPF < KS ? NPF : KS;
  uint4 q[DEPTH][NCT];
  const uint16_t* wl;
  int n_tiles;
  __device__ __forceinline__ uint4 piece(int ks, int ct) const {
    return ldg16(wl + ((size_t)ks * n_tiles + ct) * 512);
  }
  // the first DEPTH - 1 k-steps: issued ahead (before the previous layer's
  // epilogue and barrier, which do not touch the weights)
  __device__ __forceinline__ void start(const uint16_t* W, int n_tiles_, int col0) {
    const int lane = threadIdx.x & 63;
    n_tiles = n_tiles_;
    wl = W + ((size_t)(col0 / 16) * 64 + lane) * 8;
#pragma unroll
    for (int st = 0; st < DEPTH - 1; ++st)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) q[st][ct] = piece(st, ct);
  }
};

// acc[rt][ct] = A[rt*16 .., k] * W[col0 + ct*16 .., k]^T over k in [0, 32*KS),
// A from LDS (row stride AROW bf16), the weights through a started ring.  The
// lane's A piece: row l16 of the row tile, k = 32*ks + 8*g4 .. +8.
template <int RTT, int NCT, int KS, int AROW, int NPF>
__device__ __forceinline__ void mfma_layer(const uint16_t* As, WeightRing<NCT, KS, NPF>& ring,
                                           f32x4 (&acc)[RTT][NCT]) {
  constexpr int DEPTH = WeightRing<NCT, KS, NPF>::DEPTH;
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < RTT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (ks + DEPTH - 1 < KS) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) ring.q[(ks + DEPTH - 1) % DEPTH][ct] = ring.piece(ks + DEPTH - 1, ct);
    }
    // keep the prefetch ahead of this step's products (the scheduler would
    // otherwise sink the loads next to their use to save registers)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rt = 0; rt < RTT; ++rt) {
      const bf16x8_t a = as_bf16x8(
          *reinterpret_cast<const u16x8_t*>(As + (rt * 16 + l16) * AROW + 32 * ks + 8 * g4));
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a, __builtin_bit_cast(bf16x8_t, ring.q[ks % DEPTH][ct]), acc[rt][ct], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ uint16_t bf16_bits(float v) { return (uint16_t)f32_to_bf16_bits(v); }

}  // namespace

template <typename XT, typename PT, int D, int M, int RT>
__global__ void __launch_bounds__(kMlpThreads)
phi_mlp_kernel(const XT* __restrict__ x, int64_t xstride, int rows, const uint16_t* __restrict__ Win,
               const float* __restrict__ bin, const uint16_t* __restrict__ W1,
               const float* __restrict__ b1, const uint16_t* __restrict__ W2,
               const float* __restrict__ b2, const float* __restrict__ alpha,
               const uint16_t* __restrict__ Wo, const float* __restrict__ bo, int P,
               PT* __restrict__ phi) {
  constexpr int H = kPhiMlpWidth;
  constexpr int XROW = D + 8;              // bf16; 16-byte pad between rows
  constexpr int HROW = H + 8;
  constexpr int RTT = RT / 16;             // 16-row MFMA tiles
  constexpr int CTW = H / kMlpWaves / 16;  // hidden column tiles per wave (8)
  constexpr int OTW = M / kMlpWaves / 16;  // output column tiles per wave (1 or 2)
  constexpr int NPF = RT == 16 ? 6 : 3;     // weight k-steps in flight (registers allow)
  static_assert(RT % 16 == 0 && M % (16 * kMlpWaves) == 0, "tile shape");

  __shared__ __align__(16) uint16_t Xs[RT * XROW];
  __shared__ __align__(16) uint16_t Hs[RT * HROW];
  __shared__ __align__(16) uint16_t As[RT * HROW];

  const int u = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g4 = lane >> 4;
  const int p = u % P;
  const int r0 = blockIdx.x * RT;
  const int nr = min(RT, rows - r0);

  // ---- x rows as bf16 (round to nearest even); rows past the unit's end are zero
  {
    constexpr int C8 = D / 8;
    const XT* xp = x + (size_t)u * xstride + (size_t)r0 * D;
    for (int i = tid; i < RT * C8; i += kMlpThreads) {
      const int row = i / C8, c = i - row * C8;
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (row < nr) {
        if constexpr (sizeof(XT) == 2) {
          w = ldg16(reinterpret_cast<const uint16_t*>(xp) + (size_t)row * D + 8 * c);
        } else {
          const float4 a = *reinterpret_cast<const float4*>(xp + (size_t)row * D + 8 * c);
          const float4 b = *reinterpret_cast<const float4*>(xp + (size_t)row * D + 8 * c + 4);
          w = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                         pack_bf16x2(b.z, b.w));
        }
      }
      *reinterpret_cast<uint4*>(Xs + row * XROW + 8 * c) = w;
    }
  }
  const int hc0 = wave * (H / kMlpWaves);   // this wave's hidden columns
  WeightRing<CTW, D / 32, NPF> r_in;
  r_in.start(Win + (size_t)p * H * D, H / 16, hc0);
  float bias[CTW];
#pragma unroll
  for (int ct = 0; ct < CTW; ++ct) bias[ct] = bin[(size_t)p * H + hc0 + ct * 16 + l16];
  __syncthreads();

  f32x4 acc[RTT][CTW];
  // ---- h0 = W_in x + b_in
  mfma_layer<RTT, CTW, D / 32, XROW, NPF>(Xs, r_in, acc);
  WeightRing<CTW, H / 32, NPF> r_1;
  r_1.start(W1 + (size_t)p * H * H, H / 16, hc0);
#pragma unroll
  for (int rt = 0; rt < RTT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Hs[(rt * 16 + 4 * g4 + r) * HROW + hc0 + ct * 16 + l16] = bf16_bits(acc[rt][ct][r] + bias[ct]);
#pragma unroll
  for (int ct = 0; ct < CTW; ++ct) bias[ct] = b1[(size_t)p * H + hc0 + ct * 16 + l16];
  __syncthreads();

  // ---- a = relu(W_1 h0 + b_1)
  mfma_layer<RTT, CTW, H / 32, HROW, NPF>(Hs, r_1, acc);
  WeightRing<CTW, H / 32, NPF> r_2;
  r_2.start(W2 + (size_t)p * H * H, H / 16, hc0);
#pragma unroll
  for (int rt = 0; rt < RTT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        As[(rt * 16 + 4 * g4 + r) * HROW + hc0 + ct * 16 + l16] =
            bf16_bits(fmaxf(acc[rt][ct][r] + bias[ct], 0.f));
#pragma unroll
  for (int ct = 0; ct < CTW; ++ct) bias[ct] = b2[(size_t)p * H + hc0 + ct * 16 + l16];
  const float al = alpha[p];
  __syncthreads();

  // ---- h1 = h0 + alpha (W_2 a + b_2), over h0 in place (this wave's columns)
  mfma_layer<RTT, CTW, H / 32, HROW, NPF>(As, r_2, acc);
  const int oc0 = wave * (M / kMlpWaves);   // this wave's output columns
  WeightRing<OTW, H / 32, NPF> r_o;
  r_o.start(Wo + (size_t)p * M * H, M / 16, oc0);
#pragma unroll
  for (int rt = 0; rt < RTT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint16_t& h = Hs[(rt * 16 + 4 * g4 + r) * HROW + hc0 + ct * 16 + l16];
        h = bf16_bits(bf16_to_f32(h) + al * (acc[rt][ct][r] + bias[ct]));
      }
  float obias[OTW];
#pragma unroll
  for (int ct = 0; ct < OTW; ++ct) obias[ct] = bo[(size_t)p * M + oc0 + ct * 16 + l16];
  __syncthreads();

  // ---- phi = exp(W_o h1 + b_o)
  f32x4 oacc[RTT][OTW];
  mfma_layer<RTT, OTW, H / 32, HROW, NPF>(Hs, r_o, oacc);
  PT* out = phi + ((size_t)u * rows + r0) * M;
#pragma unroll
  for (int rt = 0; rt < RTT; ++rt)
#pragma unroll
    for (int ct = 0; ct < OTW; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rt * 16 + 4 * g4 + r;
        if (row < nr) {
          const float v = expf(oacc[rt][ct][r] + obias[ct]);
          if constexpr (sizeof(PT) == 2)
            out[(size_t)row * M + oc0 + ct * 16 + l16] = bf16_bits(v);
          else
            out[(size_t)row * M + oc0 + ct * 16 + l16] = v;
        }
      }
}

hipError_t launch_phi_mlp(const void* x, int x_dtype, int n_units, int64_t rows, int64_t xstride,
                          int d, const rma_phi_mlp* w, int m, int P, void* phi, int phi_dtype,
                          hipStream_t st) {
  // one-row units (decode queries) take 16-row tiles; longer ones 64-row tiles
  const bool small = rows <= 16;
  const int rt = small ? 16 : 64;
  const dim3 grid((unsigned)ceil_div(rows, rt), (unsigned)n_units);
  hipError_t e = hipSuccess;
#define RMA_MLP1(XT, PT, DD, MM, RR)                                                                 \
  e = launch_kernel(RR == 16 ? "phi_mlp_small_kernel" : "phi_mlp_kernel",                            \
                    phi_mlp_kernel<XT, PT, DD, MM, RR>, grid, dim3(kMlpThreads), 0, st,              \
                    static_cast<const XT*>(x), xstride, (int)rows, w->W_in, w->b_in, w->W_1, w->b_1, \
                    w->W_2, w->b_2, w->alpha, w->W_o, w->b_o, P, static_cast<PT*>(phi))
#define RMA_MLP(XT, PT)                                                     \
  do {                                                                      \
    if (d == 64 && m == 64) {                                               \
      if (small) RMA_MLP1(XT, PT, 64, 64, 16); else RMA_MLP1(XT, PT, 64, 64, 64);     \
    } else if (d == 64) {                                                   \
      if (small) RMA_MLP1(XT, PT, 64, 128, 16); else RMA_MLP1(XT, PT, 64, 128, 64);   \
    } else if (m == 64) {                                                   \
      if (small) RMA_MLP1(XT, PT, 128, 64, 16); else RMA_MLP1(XT, PT, 128, 64, 64);   \
    } else {                                                                \
      if (small) RMA_MLP1(XT, PT, 128, 128, 16); else RMA_MLP1(XT, PT, 128, 128, 64); \
    }                                                                       \
  } while (0)
  if (x_dtype == RMA_BF16) {
    if (phi_dtype == RMA_BF16) RMA_MLP(uint16_t, uint16_t); else RMA_MLP(uint16_t, float);
  } else {
    if (phi_dtype == RMA_BF16) RMA_MLP(float, uint16_t); else RMA_MLP(float, float);
  }
#undef RMA_MLP
#undef RMA_MLP1
  return e;
}

}  // namespace rma
