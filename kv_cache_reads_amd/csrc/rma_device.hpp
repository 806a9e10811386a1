// Device helpers shared by the librma kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rma {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float round_bf16(float x) {
  return __uint_as_float(f32_to_bf16_bits(x) << 16);
}

// Load `n` consecutive elements (16-byte aligned) of a K/V row as fp32.
template <typename T, int N>
__device__ __forceinline__ void load_row_f32(const T* p, float (&out)[N]);

template <int N>
__device__ __forceinline__ void load_row_f32(const uint16_t* p, float (&out)[N]) {
  static_assert(N % 8 == 0, "bf16 rows load in 16-byte pieces");
  const uint4* p4 = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < N / 8; ++i) {
    uint4 w = p4[i];
    out[8 * i + 0] = bf16lo(w.x); out[8 * i + 1] = bf16hi(w.x);
    out[8 * i + 2] = bf16lo(w.y); out[8 * i + 3] = bf16hi(w.y);
    out[8 * i + 4] = bf16lo(w.z); out[8 * i + 5] = bf16hi(w.z);
    out[8 * i + 6] = bf16lo(w.w); out[8 * i + 7] = bf16hi(w.w);
  }
}

template <int N>
__device__ __forceinline__ void load_row_f32(const float* p, float (&out)[N]) {
  static_assert(N % 4 == 0, "fp32 rows load in 16-byte pieces");
  const float4* p4 = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    float4 w = p4[i];
    out[4 * i + 0] = w.x; out[4 * i + 1] = w.y; out[4 * i + 2] = w.z; out[4 * i + 3] = w.w;
  }
}

// Streaming 16-byte load (nontemporal hint: read-once data).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Buffer resource over [p, p + bytes).  The hardware range check makes a load at
// an offset at or past the end return zero and drops such a store, so tiles that
// run past a range need no branch around their memory operations (and the
// compiler's wait counts stay exact across them).  Word 3 selects 32-bit data.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
constexpr int kCpolNT = 2;  // nontemporal cache policy (read-once data)
__device__ __forceinline__ uint4 buf_ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolNT);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float buf_ld_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void buf_st16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 w) {
  const u32x4_t v = {w.x, w.y, w.z, w.w};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// Raw 16-byte pieces of a row (for double buffering of loads).
template <typename T> struct RowPieces;
template <> struct RowPieces<uint16_t> { static constexpr int kElemsPerPiece = 8; };
template <> struct RowPieces<float> { static constexpr int kElemsPerPiece = 4; };

__device__ __forceinline__ void unpack_piece(const uint4& w, const uint16_t*, float* out) {
  out[0] = bf16lo(w.x); out[1] = bf16hi(w.x); out[2] = bf16lo(w.y); out[3] = bf16hi(w.y);
  out[4] = bf16lo(w.z); out[5] = bf16hi(w.z); out[6] = bf16lo(w.w); out[7] = bf16hi(w.w);
}
__device__ __forceinline__ void unpack_piece(const uint4& w, const float*, float* out) {
  out[0] = __uint_as_float(w.x); out[1] = __uint_as_float(w.y);
  out[2] = __uint_as_float(w.z); out[3] = __uint_as_float(w.w);
}

// N elements of type T as raw 16-byte words: loaded early, unpacked at use.
template <typename T, int N>
struct RawPiece {
  static constexpr int W = N * (int)sizeof(T) / 16;
  static_assert(W >= 1 && N * (int)sizeof(T) % 16 == 0, "pieces are whole 16-byte words");
  uint4 w[W];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  __device__ __forceinline__ void load(const T* p) {
    const uint4* p4 = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = p4[i];
  }
  __device__ __forceinline__ void unpack(float (&out)[N]) const {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const uint32_t x[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          out[8 * i + 2 * k] = bf16lo(x[k]);
          out[8 * i + 2 * k + 1] = bf16hi(x[k]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) out[4 * i + k] = __uint_as_float(x[k]);
      }
    }
  }
};

// ---------------------------------------------------------------- DPP sums
// Butterfly sums inside groups of 2/4/8/16 lanes with DPP row permutations.
// After lane_group_sum<N>, every lane of an aligned N-lane group holds the sum.
__device__ __forceinline__ float dpp_add_quad_xor1(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_add_quad_xor2(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_add_half_mirror(float v) {  // lane i <-> 7-i within 8
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_add_row_mirror(float v) {  // lane i <-> 15-i within 16
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
}

template <int N>
__device__ __forceinline__ float lane_group_sum(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group size");
  if constexpr (N >= 2) v = dpp_add_quad_xor1(v);
  if constexpr (N >= 4) v = dpp_add_quad_xor2(v);
  if constexpr (N >= 8) v = dpp_add_half_mirror(v);
  if constexpr (N >= 16) v = dpp_add_row_mirror(v);
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// ---------------------------------------------------------------- DPP wave ops
// Wave-wide reductions and scans on DPP row permutations and row broadcasts
// (row_bcast:15 / row_bcast:31 exist on GFX9-family parts such as gfx950).
// They must be called by all 64 lanes of the wave.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// minimum / maximum as one v_med3_f32 against -inf / +inf: fminf / fmaxf would
// first quiet each operand (a NaN-canonicalising instruction apiece)
__device__ __forceinline__ float fmin_m3(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, -3.4028235e38f); }
__device__ __forceinline__ float fmax_m3(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, 3.4028235e38f); }
// the wave's maximum of unsigned keys: butterflies inside each 16-lane row, then
// row 0 into 1 and 2 into 3, then 1 into 2 and 3 (row broadcasts), read from
// lane 63.  Every DPP source that is absent or masked reads 0, the identity of
// the unsigned maximum, so each step is one v_max_u32 with the DPP modifier
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));    // quad xor 1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));    // quad xor 2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true));   // half-row mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true));   // row mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = lane_group_sum<16>(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
// inclusive prefix sum over the wave (lane 0 first)
__device__ __forceinline__ int wave_incl_scan_dpp(int v) {
  v += dpp_i<0x111>(v);        // row_shr:1
  v += dpp_i<0x112>(v);        // row_shr:2
  v += dpp_i<0x114>(v);        // row_shr:4
  v += dpp_i<0x118>(v);        // row_shr:8
  v += dpp_i<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_i<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}
// number of set bits of `mask` below this lane
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Full-wave reductions (ds_swizzle/bpermute based; used off the hot loops).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
// Inclusive prefix sum over the wave (lane 0 first).
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// base[i] as a wave-uniform 64-bit base plus a 32-bit unsigned byte offset: the
// global loads' SGPR-base + VGPR-offset form, one 32-bit address operation per
// load rather than a 64-bit add.  The caller guarantees i * sizeof(T) < 2^32.
template <typename T>
__device__ __forceinline__ const T* off32(const T* base, uint32_t i) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + i * (uint32_t)sizeof(T));
}

// ---------------------------------------------------------------- keys
// Monotone map fp32 -> uint32 (a < b  =>  key(a) <= key(b); -0 < +0).
__device__ __forceinline__ uint32_t ord_f32(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}
// the wave's maximum / minimum of fp32 values through their ordered keys
__device__ __forceinline__ float wave_max_dpp(float v) { return unord_f32(wave_max_u32(ord_f32(v))); }
__device__ __forceinline__ float wave_min_dpp(float v) { return unord_f32(~wave_max_u32(~ord_f32(v))); }
__device__ __forceinline__ uint64_t ord_f64(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

// ---------------------------------------------------------------- band dot
// Double-double dot product of an fp32 query with a stored key row.  Every
// product q_j*k_j is exact in fp64 (24x8 or 24x24 significand bits, exponents
// far inside fp64's range).  TwoSum keeps the rounding error of each addition
// exactly, so the only rounding is in c, the plain fp64 sum of those errors.
// Each error is a multiple of 2^E (E = the lowest last-bit exponent among the
// nonzero products) and below half an ulp of the running sum, so c is exact
// whenever the products' last bits span at most 58 - 2 log2(d) binades (46 at
// d = 64, 44 at d = 128).  Then (hi, lo) is the canonical pair of the exact
// score and comparing pairs is exact; identical keys always give identical
// pairs.  Otherwise the pair is within (d + 2) 2^-106 sum|q_j k_j| of the exact
// score, and only distinct scores closer than twice that can be misordered.
struct DD { double hi, lo; };

__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

template <typename T, int D>
__device__ DD dd_dot(const float* q, const T* krow) {
  double s = 0.0, c = 0.0;
#pragma unroll 4
  for (int j0 = 0; j0 < D; j0 += 8) {
    float kv[8];
    if constexpr (sizeof(T) == 2) {
      uint4 w = *reinterpret_cast<const uint4*>(krow + j0);
      unpack_piece(w, (const uint16_t*)nullptr, kv);
    } else {
      float4 a = *reinterpret_cast<const float4*>(krow + j0);
      float4 b = *reinterpret_cast<const float4*>(krow + j0 + 4);
      kv[0] = a.x; kv[1] = a.y; kv[2] = a.z; kv[3] = a.w;
      kv[4] = b.x; kv[5] = b.y; kv[6] = b.z; kv[7] = b.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      double p = (double)q[j0 + e] * (double)kv[e];
      double t, err;
      two_sum(s, p, t, err);
      s = t;
      c += err;
    }
  }
  DD r;
  two_sum(s, c, r.hi, r.lo);
  if (r.hi == 0.0) r.hi = 0.0;  // canonical +0
  if (r.lo == 0.0) r.lo = 0.0;
  return r;
}

// The same double-double dot by a group of P = D sizeof(T) / 16 consecutive
// lanes, each loading one 16-byte piece of the row: lane `part` sums its
// elements as above, then the partial pairs meet in a butterfly of TwoSums.  A
// lane pair computes the same TwoSum (its error term is exact in either
// argument order) and the same sum of error terms, so every lane of the group
// returns the same pair.  The exactness condition and the bound above hold
// unchanged: any order makes d - 1 additions whose running sums are bounded by
// sum|q_j k_j| and whose error terms are multiples of 2^E.
template <typename T, int D>
struct DDGroup {
  static constexpr int E = 16 / (int)sizeof(T);   // elements per lane
  static constexpr int P = D / E;                  // lanes per row
};
template <typename T, int D>
__device__ __forceinline__ DD dd_dot_group(const float* q, const T* krow, int part) {
  constexpr int E = DDGroup<T, D>::E, P = DDGroup<T, D>::P;
  static_assert(P >= 1 && (P & (P - 1)) == 0 && P <= 64, "power-of-two lane groups within a wave");
  RawPiece<T, E> w;
  w.load(krow + part * E);
  float kv[E];
  w.unpack(kv);
  double s = 0.0, c = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const double p = (double)q[part * E + e] * (double)kv[e];
    double t, err;
    two_sum(s, p, t, err);
    s = t;
    c += err;
  }
#pragma unroll
  for (int off = P / 2; off >= 1; off >>= 1) {
    const double so = __shfl_xor(s, off), co = __shfl_xor(c, off);
    double t, err;
    two_sum(s, so, t, err);
    s = t;
    c = (c + co) + err;
  }
  DD r;
  two_sum(s, c, r.hi, r.lo);
  if (r.hi == 0.0) r.hi = 0.0;  // canonical +0
  if (r.lo == 0.0) r.lo = 0.0;
  return r;
}

// a > b in the (exact score desc, position asc) order
__device__ __forceinline__ bool dd_key_greater(DD a, int ia, DD b, int ib) {
  if (a.hi != b.hi) return a.hi > b.hi;
  if (a.lo != b.lo) return a.lo > b.lo;
  return ia < ib;
}

// Scalar element access for fp32 or bf16 storage.
__device__ __forceinline__ float ld_f32(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld_f32(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
template <typename T> __device__ __forceinline__ float st_round(float x);
template <> __device__ __forceinline__ float st_round<float>(float x) { return x; }
template <> __device__ __forceinline__ float st_round<uint16_t>(float x) { return round_bf16(x); }
__device__ __forceinline__ void st_elem(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st_elem(uint16_t* p, size_t i, float v) {
  p[i] = (uint16_t)f32_to_bf16_bits(v);
}

// ---------------------------------------------------------------- misc
// Quotient by a divisor d >= 1 that is only known at run time, for 0 <= i < 2^31
// - d with a quotient below 2^22.  The compiler's integer division by a variable
// is a long sequence with a reciprocal of its own; here the float estimate
// i * (1/d) carries three roundings of relative 2^-24 each, so it is within one
// of floor(i / d), and two integer checks make it exact.
struct FastDiv {
  int d;
  float inv;
  __device__ explicit FastDiv(int d_) : d(d_), inv(1.0f / (float)d_) {}
  __device__ __forceinline__ int quo(int i) const {
    int c = (int)((float)i * inv);
    c -= (c * d > i) ? 1 : 0;
    c += ((c + 1) * d <= i) ? 1 : 0;
    return c;
  }
};

__device__ __forceinline__ float phi_elu1(float z) { return z > 0.f ? z + 1.f : __expf(z); }

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32); the
// summary builder and the decode recompute of phi_k rows both round with this
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// ---- w = f . phi over bf16 phi rows on the bf16 dot instruction.  f (fp32) is
// split into two packed bf16 pairs, hi = f rounded to bf16 and lo = the
// remainder rounded to bf16, so hi + lo = f within 2^-17 |f|; each product of
// bf16 values is exact, and v_dot2_f32_bf16 adds two of them to the fp32 sum.
// Per feature pair one instruction for hi and one for lo, where unpacking the
// row and multiplying in fp32 takes four.
__device__ __forceinline__ void split_f_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}
template <int N>
__device__ __forceinline__ float dot_phi_bf16(const RawPiece<uint16_t, N>& p, const uint32_t (&fh)[N / 2],
                                              const uint32_t (&fl)[N / 2]) {
  float w = 0.f;
#pragma unroll
  for (int i = 0; i < N / 8; ++i) {
    const uint32_t x[4] = {p.w[i].x, p.w[i].y, p.w[i].z, p.w[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bf16x2_t v = __builtin_bit_cast(bf16x2_t, x[k]);
      w = __builtin_amdgcn_fdot2_f32_bf16(v, __builtin_bit_cast(bf16x2_t, fh[4 * i + k]), w, false);
      w = __builtin_amdgcn_fdot2_f32_bf16(v, __builtin_bit_cast(bf16x2_t, fl[4 * i + k]), w, false);
    }
  }
  return w;
}

// ---- the phi projection on the MFMA, shared by the summary builder and the
// decode recompute of retrieved phi_k rows (same operands, same instruction
// order, so both produce the same bits)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8_t as_bf16x8(u16x8_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// B operands of one 16-feature tile for lane group g4: W (fp32) split into bf16
// hi + lo parts (w = hi + lo + O(2^-17 |w|)).  `wrow` points at W[feature][8*g4].
template <int KS>
__device__ __forceinline__ void split_w_values(const float (&w)[KS][8], bf16x8_t (&Whi)[KS],
                                               bf16x8_t (&Wlo)[KS]) {
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u16x8_t hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t hb = f32_to_bf16_bits(w[ks][e]);
      hi[e] = (unsigned short)hb;
      lo[e] = (unsigned short)f32_to_bf16_bits(w[ks][e] - __uint_as_float(hb << 16));
    }
    Whi[ks] = as_bf16x8(hi);
    Wlo[ks] = as_bf16x8(lo);
  }
}
template <int KS>
__device__ __forceinline__ void split_w_operands(const float* wrow, bf16x8_t (&Whi)[KS],
                                                 bf16x8_t (&Wlo)[KS]) {
  float w[KS][8];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) w[ks][e] = wrow[32 * ks + e];
  split_w_values<KS>(w, Whi, Wlo);
}

// Z = K W^T for 16 key rows x 16 features (v_mfma_f32_16x16x32_bf16).  `arow`
// points at the lane's key row (l%16 of the tile) at column 8*g4; the result
// holds rows 4*g4 .. 4*g4+3 of feature column l%16.
template <int KS>
__device__ __forceinline__ f32x4 proj_tile16(const uint16_t* arow, const bf16x8_t (&Whi)[KS],
                                             const bf16x8_t (&Wlo)[KS]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8_t A = as_bf16x8(*reinterpret_cast<const u16x8_t*>(arow + 32 * ks));
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Whi[ks], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Wlo[ks], acc, 0, 0, 0);
  }
  return acc;
}

}  // namespace rma
