// C ABI entry points of librma: argument validation, planning, workspace sizing.
// Validation runs entirely on the host before anything is enqueued.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>

#include "rma_internal.hpp"

namespace rma {
static_assert(kTraceMax == RMA_TRACE_MAX_EVENTS, "trace size");

KernelTrace& trace() {
  static thread_local KernelTrace t;
  return t;
}

namespace {

// Spans one entry point when a trace is armed: its kernels take the armed event
// pairs in launch order (launch_kernel); on exit the trace is disarmed.
struct TraceScope {
  explicit TraceScope(hipStream_t) { trace().used = 0; }
  ~TraceScope() {
    KernelTrace& t = trace();
    if (t.n_events > 0) {
      t.count = t.used / 2;
      t.n_events = 0;
      t.used = 0;
    }
  }
};

thread_local char g_last_error[512] = "";

rma_status fail(rma_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool dtype_ok(int dt) { return dt == RMA_F32 || dt == RMA_BF16; }
size_t dtype_size(int dt) { return dt == RMA_F32 ? 4 : 2; }

#define RMA_CHECK(cond, status, ...)              \
  do {                                            \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

rma_status check_kv_span(const rma_kv* kv, const rma_span* sp, bool need_v) {
  RMA_CHECK(kv != nullptr && sp != nullptr, RMA_ERR_INVALID_ARG, "kv or span is NULL");
  RMA_CHECK(dtype_ok(kv->dtype), RMA_ERR_UNSUPPORTED, "unsupported K/V dtype %d", kv->dtype);
  RMA_CHECK(kv->d == 64 || kv->d == 128, RMA_ERR_UNSUPPORTED, "head dim %d not in {64,128}", kv->d);
  RMA_CHECK(kv->n_units >= 1 && kv->n_units <= 65535, RMA_ERR_INVALID_ARG,
            "n_units must be in [1, 65535]");
  RMA_CHECK(kv->k != nullptr, RMA_ERR_INVALID_ARG, "kv->k is NULL");
  RMA_CHECK(!need_v || kv->v != nullptr, RMA_ERR_INVALID_ARG, "kv->v is NULL");
  RMA_CHECK(aligned16(kv->k) && (!need_v || aligned16(kv->v)), RMA_ERR_INVALID_ARG,
            "K/V pointers must be 16-byte aligned");
  RMA_CHECK(kv->unit_stride % 8 == 0, RMA_ERR_INVALID_ARG, "unit_stride must be a multiple of 8");
  RMA_CHECK(sp->L >= 0 && sp->n_sink >= 0 && sp->n_tail >= 0 && sp->n_gen >= 0,
            RMA_ERR_INVALID_ARG, "negative span field");
  RMA_CHECK((int64_t)sp->n_sink + sp->n_tail <= sp->L, RMA_ERR_INVALID_ARG,
            "n_sink + n_tail (%d + %d) exceeds L (%lld)", sp->n_sink, sp->n_tail,
            (long long)sp->L);
  RMA_CHECK(sp->L <= INT32_MAX / 2 && sp->n_gen <= INT32_MAX / 2, RMA_ERR_INVALID_ARG,
            "L or n_gen too large");
  RMA_CHECK(kv->t_cap >= sp->L + sp->n_gen, RMA_ERR_INVALID_ARG,
            "t_cap (%lld) < L + n_gen (%lld)", (long long)kv->t_cap,
            (long long)(sp->L + sp->n_gen));
  RMA_CHECK(kv->unit_stride >= kv->t_cap * kv->d, RMA_ERR_INVALID_ARG,
            "unit_stride < t_cap * d");
  return RMA_OK;
}

int64_t l_mid(const rma_span& sp) { return sp.L - sp.n_sink - sp.n_tail; }

// compute units of the current device
int device_cus() { return device_info().cus; }

}  // namespace

const DeviceInfo& device_info() {
  static std::once_flag once[kMaxDevices];
  static DeviceInfo info[kMaxDevices];
  static const DeviceInfo fallback{256, 64 * 1024};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return fallback;
  std::call_once(once[dev], [dev] {
    int cus = 0, lds = 0;
    info[dev].cus = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                            cus > 0
                        ? cus
                        : fallback.cus;
    info[dev].lds_per_block =
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && lds > 0
            ? (size_t)lds
            : fallback.lds_per_block;
  });
  return info[dev];
}

// ------------------------------------------------------------- static scratch
// Scratch of rma_decode_topk_static: one array per GPU (the runtime places a
// copy of every __device__ variable on each device the code object is loaded
// on).  In host code `scratch` names a host-side stand-in, not a device
// address, so it is never passed to a kernel or a copy: its address on the
// current device is obtained once per device (with that device current) and
// kept per device.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
struct StaticScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
StaticScratch g_static_scratch[kMaxDevices];
}  // namespace

hipError_t static_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  StaticScratch& s = g_static_scratch[dev];
  std::call_once(s.once, [&s] {
    void* p = nullptr;
    s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    s.ptr = s.err == hipSuccess ? p : nullptr;
  });
  *ptr = s.ptr;
  return s.err;
}

// ------------------------------------------------------------- plans
BuildPlan plan_build(const rma_kv& kv, int64_t tokens, int m, bool computed_phi, int phi_dtype) {
  BuildPlan p{};
  const int64_t Lm = tokens;
  const int64_t U = kv.n_units;
  // bf16 K/V and bf16 rows (computed, or given): the matrix-core builder
  (void)computed_phi;
  p.mfma = kv.dtype == RMA_BF16 && phi_dtype == RMA_BF16;
  const int tile = p.mfma ? 64 : 32;
  if (Lm > 0) {
    // enough blocks to cover the chip with as few per-chunk partials as possible
    int64_t nc = std::max<int64_t>(1, std::min<int64_t>(ceil_div(Lm, 256), ceil_div(512, U)));
    if (p.mfma) {
      // the MFMA builder's resident blocks (by its registers): one per CU at
      // d = 128, two at d = 64; one wave of them covers the chip
      const int64_t R = (int64_t)device_cus() * (kv.d == 128 ? 1 : 2);
      nc = std::max<int64_t>(1, std::min<int64_t>(ceil_div(Lm, 256), ceil_div(R, U)));
      // whole waves of blocks: with long chunks, a last wave that fills only
      // part of the chip leaves the rest idle for a block's whole time
      for (int64_t c = nc; c <= nc + 16 && ceil_div(Lm, c) >= 1024; ++c) {
        if ((U * c) % R == 0 || U * c >= 8 * R) {
          nc = c;
          break;
        }
      }
    }
    // chunks of at most 2^22 tokens keep the builder's 32-bit byte offsets in range
    nc = std::max<int64_t>(nc, ceil_div(Lm, int64_t(1) << 22));
    int64_t ch = ceil_div(ceil_div(Lm, nc), tile) * tile;
    p.ch = (int)ch;
    p.n_chunks = (int)ceil_div(Lm, ch);
  }
  size_t off = 0;
  const size_t nc = (size_t)std::max(p.n_chunks, 1);
  p.off_S = off;
  off = align_up(off + (size_t)U * nc * m * kv.d * 4);
  p.off_u = off;
  off = align_up(off + (size_t)U * nc * m * 4);
  p.off_kap = off;
  off = align_up(off + (size_t)U * nc * 4);
  p.total = std::max(off, kAlign);   // never 0: 0 means invalid arguments
  return p;
}

TopkPlan plan_topk(const rma_kv& kv, const rma_span& sp, int G, int K) {
  TopkPlan p{};
  const int64_t Lm = l_mid(sp);
  const int64_t U = kv.n_units;
  const int tile = scan_tile(kv.d);  // tokens per scan block pass
  const int64_t ch_max = std::max<int64_t>(tile, scan_chmax(kv.d, G));
  if (Lm > 0) {
    int64_t lo = ceil_div(Lm, ch_max);
    int64_t hi = std::min<int64_t>(kSelMaxChunks, ceil_div(Lm, tile));
    int64_t nc = std::max<int64_t>(lo, std::min<int64_t>(ceil_div(kScanBlocks, U), hi));
    int64_t ch = ceil_div(ceil_div(Lm, nc), tile) * tile;
    p.ch = (int)ch;
    p.n_chunks = (int)ceil_div(Lm, ch);
    if (K >= Lm) {
      p.r_min = p.r_cap = p.ch;
    } else {
      // a chunk holds ~Binomial(ch, K/L_mid) of the K winners (mean mu); reporting
      // mu + 4 sqrt(mu) + 4 makes an incomplete report (-> exact fallback) rare:
      // about 2e-10 per chunk at mu = 5, 1e-8 at mu = 37
      const double mu = (double)K / p.n_chunks;
      int64_t rmin = (int64_t)std::ceil(mu + 4.0 * std::sqrt(mu) + 4.0);
      rmin = std::max<int64_t>(16, (rmin + 7) / 8 * 8);
      p.r_min = (int)std::min<int64_t>(ch, rmin);
      p.r_cap = (int)std::min<int64_t>(ch, 2 * p.r_min + 32);
    }
    p.e_max = (int)std::min<int64_t>(kSelMaxEntries, (int64_t)p.n_chunks * p.r_cap);
  }
  size_t off = 0;
  p.off_ent = off;
  off = align_up(off + (size_t)U * G * std::max(p.n_chunks, 1) * std::max(p.r_cap, 1) * 8);
  p.off_meta = off;
  off = align_up(off + (size_t)U * G * std::max(p.n_chunks, 1) * 8);
  p.off_hp = off;
  off = align_up(off + (size_t)U * G * 16);
  p.total = std::max(off, kAlign);   // never 0: 0 means invalid arguments
  p.sel_lds = align_up((size_t)p.e_max * 8 + 16, 16);
  return p;
}

FullPlan plan_full(const rma_kv& kv, const rma_span& sp, int G) {
  FullPlan p{};
  const int64_t T = sp.L + sp.n_gen;
  const int64_t U = kv.n_units;
  const int tile = kv.d == 64 ? 64 : 32;  // positions per block pass
  if (T > 0) {
    int64_t nc = std::max<int64_t>(ceil_div(T, kFullMaxChunk),
                                   std::min<int64_t>(ceil_div(512, U), ceil_div(T, tile)));
    const int64_t ch = ceil_div(ceil_div(T, nc), tile) * tile;
    p.ch = (int)ch;
    p.n_chunks = (int)ceil_div(T, ch);
  }
  size_t off = 0;
  p.off_part = off;
  off = align_up(off + (size_t)U * std::max(p.n_chunks, 1) * G * (kFullRecHead + kv.d) * 4);
  p.total = std::max(off, kAlign);   // never 0: 0 means invalid arguments
  return p;
}

MergePlan plan_merge(const rma_kv& kv, const rma_span& sp, int G, int K, int m) {
  (void)m;
  MergePlan p{};
  const int64_t U = kv.n_units;
  const int64_t T = std::max<int64_t>(1, (int64_t)sp.n_sink + sp.n_tail + sp.n_gen + K);
  // One block per (unit, head) gathers its entries in rounds of `per_round`
  // (eight lanes per entry, a few entries per lane group in flight).  When the
  // heads alone leave most of the chip idle and a head needs three or more
  // rounds, its entries are split into slices of about one round each, at most
  // one block per CU in all (the merge block's registers allow one resident
  // block), and a second kernel combines the slices.  (With two rounds the
  // second kernel's launch costs about what the split saves.)
  const int64_t per_round = kv.dtype == RMA_BF16 ? (kv.d == 64 ? 512 : 256) : 128;
  const int64_t heads = U * G;
  const int64_t rounds = ceil_div(T, per_round);
  const int64_t ns = rounds < 3 ? 1
                                : std::max<int64_t>(1, std::min<int64_t>({rounds,
                                                                          (int64_t)device_cus() / heads,
                                                                          (int64_t)kMergeCombineThreads}));
  p.sl = (int)ceil_div(T, ns);
  p.n_slices = (int)ceil_div(T, p.sl);   // no empty slice
  p.part_floats = p.n_slices > 1 ? 4 + 3 * kv.d : 0;
  p.off_part = 0;
  p.total = std::max(align_up(p.off_part + (size_t)heads * p.n_slices * p.part_floats * 4), kAlign);
  return p;
}

DecodePlan plan_decode(const rma_kv& kv, const rma_span& sp, int G, int K, int m, int phi_dtype,
                       bool recompute) {
  DecodePlan p{};
  p.topk = plan_topk(kv, sp, G, K);
  p.merge = plan_merge(kv, sp, G, K, m);
  const int64_t heads = (int64_t)kv.n_units * G;
  // one 1024-thread block per head while the heads leave most of the chip free;
  // with many heads smaller blocks, several to a CU
  // (fp32 keys at d = 128 need more than the 128 registers a 1024-thread
  // block leaves each lane)
  p.fused_threads = heads < 1024 && !(kv.dtype == RMA_F32 && kv.d == 128) ? 1024
                    : (kv.d == 64 ? 256 : 512);
  // the fused kernel addresses a unit's K/V rows and phi_k rows through 32-bit
  // byte offsets: larger units take the two kernels (64-bit addressing)
  const int64_t kv_bytes = (sp.L + sp.n_gen) * kv.d * (kv.dtype == RMA_BF16 ? 2 : 4);
  const int64_t phi_bytes = l_mid(sp) * m * (phi_dtype == RMA_BF16 ? 2 : 4);
  const bool off32_fits = kv_bytes < ((int64_t)1 << 32) && phi_bytes < ((int64_t)1 << 32);
  bool fused = K > 0 && !recompute && off32_fits && p.topk.n_chunks <= kSelMaxChunks &&
               fused_slots_fit(p.topk.n_chunks, p.fused_threads);
  if (fused) {
    const size_t dyn = fused_dyn_bytes(p.topk.n_chunks, p.topk.r_cap, K, kv.d, p.fused_threads);
    fused = dyn + fused_static_lds(kv.dtype, phi_dtype, kv.d, m, p.fused_threads) <=
            device_info().lds_per_block;
  }
  p.fused = fused;
  // With few heads and a large budget the fused kernel's gather, one block per
  // head, is bound by the loads one CU keeps in flight: then each head's list
  // is split over several blocks (each selects, gathers a slice and writes a
  // partial) and merge_combine_kernel combines the slices: from four rounds on
  // (with three the second kernel costs about what the split saves), over as
  // many blocks as there are CUs, at most 16 slices per head, none empty.
  const int64_t per_round = (int64_t)(p.fused_threads / 8) *
                            fused_gather_batch(kv.dtype == RMA_BF16 ? 2 : 4, phi_dtype == RMA_BF16 ? 2 : 4,
                                               kv.d, p.fused_threads);
  const int64_t rounds = K > 0 ? ceil_div(K, per_round) : 0;
  const int64_t split_cap = heads <= 128 ? 16 : 1;
  p.fused_split = 1;
  if (fused && p.fused_threads == 1024 && rounds >= 4) {
    const int64_t ns = std::max<int64_t>(1, std::min<int64_t>(split_cap, (int64_t)device_cus() / heads));
    const int64_t sl = ceil_div(K, ns);
    p.fused_split = (int)ceil_div(K, sl);
  }
  // the separate path's regions are always reserved, so the size does not
  // depend on the device (the split partials are sized for the most slices)
  size_t off = align_up(p.topk.total);
  p.off_idx = off;
  off = align_up(off + (size_t)heads * K * 4);
  p.off_sel = off;
  off = align_up(off + (size_t)heads * K * 4);
  p.off_merge = off;
  off = align_up(off + p.merge.total);
  p.off_fpart = off;
  if (split_cap > 1) off = align_up(off + (size_t)heads * split_cap * (4 + 3 * kv.d) * 4);
  p.total = std::max(off, kAlign);
  return p;
}

}  // namespace rma

using namespace rma;

extern "C" {

const char* rma_status_string(int32_t s) {
  switch (s) {
    case RMA_OK: return "RMA_OK";
    case RMA_ERR_INVALID_ARG: return "RMA_ERR_INVALID_ARG";
    case RMA_ERR_UNSUPPORTED: return "RMA_ERR_UNSUPPORTED";
    case RMA_ERR_WORKSPACE: return "RMA_ERR_WORKSPACE";
    case RMA_ERR_HIP: return "RMA_ERR_HIP";
    default: return "RMA_ERR_UNKNOWN";
  }
}

const char* rma_last_error(void) { return g_last_error; }

int32_t rma_abi_version(void) { return RMA_ABI_VERSION; }

rma_status rma_trace_arm(void* const* events, int32_t n_events) {
  g_last_error[0] = 0;
  KernelTrace& t = trace();
  if (n_events == 0) {
    t.n_events = 0;
    t.used = 0;
    return RMA_OK;
  }
  RMA_CHECK(events != nullptr && n_events >= 2 && n_events <= kTraceMax && n_events % 2 == 0,
            RMA_ERR_INVALID_ARG, "n_events must be 0 or even in 2..%d", kTraceMax);
  for (int i = 0; i < n_events; ++i) {
    RMA_CHECK(events[i] != nullptr, RMA_ERR_INVALID_ARG, "event %d is NULL", i);
    t.ev[i] = (hipEvent_t)events[i];
  }
  t.n_events = n_events;
  t.used = 0;
  t.count = 0;
  return RMA_OK;
}

int32_t rma_trace_count(void) { return trace().count; }

const char* rma_trace_name(int32_t j) {
  const KernelTrace& t = trace();
  return (j >= 0 && j < t.count) ? t.name[j] : nullptr;
}

rma_status rma_stream_read(const void* p, int64_t bytes, int32_t blocks, uint32_t* sink, void* stream) {
  g_last_error[0] = 0;
  RMA_CHECK(p != nullptr && sink != nullptr, RMA_ERR_INVALID_ARG, "NULL pointer argument");
  RMA_CHECK(aligned16(p), RMA_ERR_INVALID_ARG, "p must be 16-byte aligned");
  RMA_CHECK(bytes > 0 && bytes % 16 == 0, RMA_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  RMA_CHECK(blocks >= 1 && blocks <= (1 << 20), RMA_ERR_INVALID_ARG, "blocks %d outside 1..2^20", blocks);
  TraceScope ts((hipStream_t)stream);
  const hipError_t e = launch_stream_read(p, bytes, blocks, sink, (hipStream_t)stream);
  RMA_CHECK(e == hipSuccess, RMA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return RMA_OK;
}

size_t rma_workspace_bytes(int32_t op, const rma_kv* kv, const rma_span* sp, int32_t G, int32_t K,
                           int32_t m) {
  if (kv == nullptr || sp == nullptr || kv->n_units < 1 || (kv->d != 64 && kv->d != 128))
    return 0;
  if (sp->L < 0 || sp->n_sink < 0 || sp->n_tail < 0 || (int64_t)sp->n_sink + sp->n_tail > sp->L)
    return 0;
  switch (op) {
    case RMA_OP_BUILD_SUMMARIES:
      if (m != 64 && m != 128) return 0;
      // the larger of the two builder layouts (MFMA tiles are coarser)
      return std::max(plan_build(*kv, l_mid(*sp), m, true, RMA_BF16).total,
                      plan_build(*kv, l_mid(*sp), m, false, RMA_F32).total);
    case RMA_OP_DECODE_TOPK:
      if (G < 1 || G > 8 || K < 0 || K > l_mid(*sp)) return 0;
      return plan_topk(*kv, *sp, G, K).total;
    case RMA_OP_DECODE_MERGE:
      if (G < 1 || G > 8 || K < 0 || K > l_mid(*sp)) return 0;
      return plan_merge(*kv, *sp, G, K, m).total;
    case RMA_OP_DECODE:
      if (G < 1 || G > 8 || K < 0 || K > l_mid(*sp) || (m != 64 && m != 128)) return 0;
      return plan_decode(*kv, *sp, G, K, m, RMA_BF16, false).total;
    case RMA_OP_DECODE_FULL:
      if (G < 1 || G > 8 || sp->n_gen < 0) return 0;
      return plan_full(*kv, *sp, G).total;
    default:
      return 0;
  }
}

rma_status rma_phi_features(const void* x, int32_t x_dtype, int32_t n_units, int64_t rows,
                            int64_t x_unit_stride, int32_t d, const float* W, const float* b,
                            int32_t m, int32_t P, void* phi, int32_t phi_dtype, void* stream) {
  g_last_error[0] = 0;
  RMA_CHECK(x && W && b && phi, RMA_ERR_INVALID_ARG, "NULL pointer argument");
  RMA_CHECK(dtype_ok(x_dtype) && dtype_ok(phi_dtype), RMA_ERR_UNSUPPORTED, "unsupported dtype");
  RMA_CHECK(d == 64 || d == 128, RMA_ERR_UNSUPPORTED, "d %d not in {64,128}", d);
  RMA_CHECK(m == 64 || m == 128, RMA_ERR_UNSUPPORTED, "m %d not in {64,128}", m);
  RMA_CHECK(n_units >= 1 && n_units <= 65535 && rows >= 0 && P >= 1, RMA_ERR_INVALID_ARG,
            "bad sizes");
  RMA_CHECK(rows <= INT32_MAX / 2, RMA_ERR_INVALID_ARG, "rows too large");
  RMA_CHECK(x_unit_stride >= rows * d && x_unit_stride % 8 == 0, RMA_ERR_INVALID_ARG,
            "x_unit_stride must be >= rows*d and a multiple of 8");
  RMA_CHECK(aligned16(x) && aligned16(W) && aligned16(b) && aligned16(phi), RMA_ERR_INVALID_ARG,
            "pointers must be 16-byte aligned");
  if (rows == 0) return RMA_OK;
  TraceScope ts((hipStream_t)stream);
  hipError_t e = launch_phi(x, x_dtype, n_units, rows, x_unit_stride, d, W, b, m, P, phi,
                            phi_dtype, (hipStream_t)stream);
  RMA_CHECK(e == hipSuccess, RMA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return RMA_OK;
}

rma_status rma_phi_mlp_features(const void* x, int32_t x_dtype, int32_t n_units, int64_t rows,
                                int64_t x_unit_stride, int32_t d, const rma_phi_mlp* w, int32_t m,
                                int32_t P, void* phi, int32_t phi_dtype, void* stream) {
  g_last_error[0] = 0;
  RMA_CHECK(x && w && phi, RMA_ERR_INVALID_ARG, "NULL pointer argument");
  RMA_CHECK(w->W_in && w->b_in && w->W_1 && w->b_1 && w->W_2 && w->b_2 && w->alpha && w->W_o &&
                w->b_o,
            RMA_ERR_INVALID_ARG, "NULL weight pointer");
  RMA_CHECK(dtype_ok(x_dtype) && dtype_ok(phi_dtype), RMA_ERR_UNSUPPORTED, "unsupported dtype");
  RMA_CHECK(d == 64 || d == 128, RMA_ERR_UNSUPPORTED, "d %d not in {64,128}", d);
  RMA_CHECK(m == 64 || m == 128, RMA_ERR_UNSUPPORTED, "m %d not in {64,128}", m);
  RMA_CHECK(n_units >= 1 && n_units <= 65535 && rows >= 0 && P >= 1, RMA_ERR_INVALID_ARG,
            "bad sizes");
  RMA_CHECK(rows <= INT32_MAX / 2, RMA_ERR_INVALID_ARG, "rows too large");
  RMA_CHECK(x_unit_stride >= rows * d && x_unit_stride % 8 == 0, RMA_ERR_INVALID_ARG,
            "x_unit_stride must be >= rows*d and a multiple of 8");
  RMA_CHECK(aligned16(x) && aligned16(phi) && aligned16(w->W_in) && aligned16(w->W_1) &&
                aligned16(w->W_2) && aligned16(w->W_o),
            RMA_ERR_INVALID_ARG, "x, phi and the weight matrices must be 16-byte aligned");
  if (rows == 0) return RMA_OK;
  TraceScope ts((hipStream_t)stream);
  hipError_t e = launch_phi_mlp(x, x_dtype, n_units, rows, x_unit_stride, d, w, m, P, phi,
                                phi_dtype, (hipStream_t)stream);
  RMA_CHECK(e == hipSuccess, RMA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return RMA_OK;
}

rma_status rma_build_summaries(const rma_kv* kv, const rma_span* sp, const float* Wk,
                               const float* bk, int32_t m, int32_t P, void* phi_k,
                               int32_t phi_dtype, float* S, float* u, float* kappa,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (kv == nullptr || sp == nullptr) {
    g_last_error[0] = 0;
    return fail(RMA_ERR_INVALID_ARG, "kv or span is NULL");
  }
  return rma_build_summaries_range(kv, sp, 0, l_mid(*sp), 0u, Wk, bk, m, P, phi_k, phi_dtype, S, u,
                                   kappa, workspace, workspace_bytes, stream);
}

rma_status rma_build_summaries_range(const rma_kv* kv, const rma_span* sp, int64_t m_begin,
                                     int64_t m_end, uint32_t flags, const float* Wk,
                                     const float* bk, int32_t m, int32_t P, void* phi_k,
                                     int32_t phi_dtype, float* S, float* u, float* kappa,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  rma_status s = check_kv_span(kv, sp, true);
  if (s != RMA_OK) return s;
  RMA_CHECK(flags == 0u || flags == RMA_BUILD_ACCUMULATE, RMA_ERR_INVALID_ARG, "unknown flags 0x%x",
            flags);
  RMA_CHECK(0 <= m_begin && m_begin <= m_end && m_end <= l_mid(*sp), RMA_ERR_INVALID_ARG,
            "token range [%lld, %lld) outside the mid-region [0, %lld)", (long long)m_begin,
            (long long)m_end, (long long)l_mid(*sp));
  RMA_CHECK(m == 64 || m == 128, RMA_ERR_UNSUPPORTED, "m %d not in {64,128}", m);
  RMA_CHECK(dtype_ok(phi_dtype), RMA_ERR_UNSUPPORTED, "unsupported phi dtype");
  RMA_CHECK(P >= 1, RMA_ERR_INVALID_ARG, "n_param_sets must be >= 1");
  RMA_CHECK(Wk == nullptr || bk != nullptr, RMA_ERR_INVALID_ARG, "bk is NULL");
  RMA_CHECK(S && u && kappa, RMA_ERR_INVALID_ARG, "NULL output pointer");
  // phi_k may be NULL only when the MFMA builder computes the features (the rows
  // are then not stored; decode recomputes the retrieved ones)
  RMA_CHECK(phi_k != nullptr || m_end == m_begin ||
                (Wk != nullptr && kv->dtype == RMA_BF16 && phi_dtype == RMA_BF16),
            RMA_ERR_INVALID_ARG, "phi_k is NULL (allowed only for bf16 keys with Wk given)");
  RMA_CHECK(aligned16(S) && aligned16(u) && aligned16(kappa) && aligned16(phi_k) &&
                aligned16(Wk) && aligned16(bk),
            RMA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  BuildPlan pl = plan_build(*kv, m_end - m_begin, m, Wk != nullptr, phi_dtype);
  RMA_CHECK(workspace != nullptr && aligned16(workspace), RMA_ERR_WORKSPACE,
            "workspace is NULL or misaligned");
  RMA_CHECK(workspace_bytes >= pl.total, RMA_ERR_WORKSPACE, "workspace %zu < required %zu",
            workspace_bytes, pl.total);
  TraceScope ts((hipStream_t)stream);
  hipError_t e = launch_build(pl, *kv, *sp, (int)m_begin, (int)(m_end - m_begin),
                              flags == RMA_BUILD_ACCUMULATE, Wk, bk, m, P, phi_k, phi_dtype, S, u,
                              kappa, (uint8_t*)workspace, (hipStream_t)stream);
  RMA_CHECK(e == hipSuccess, RMA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return RMA_OK;
}

rma_status rma_decode_topk(const float* q, int32_t G, const rma_kv* kv, const rma_span* sp,
                           const float* kappa, int32_t K, int32_t* idx, float* sel_scores,
                           void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  rma_status s = check_kv_span(kv, sp, false);
  if (s != RMA_OK) return s;
  RMA_CHECK(G >= 1 && G <= 8, RMA_ERR_UNSUPPORTED, "G %d not in 1..8", G);
  RMA_CHECK(K >= 0 && K <= l_mid(*sp), RMA_ERR_INVALID_ARG, "K %d outside [0, L_mid=%lld]", K,
            (long long)l_mid(*sp));
  if (K == 0) return RMA_OK;
  RMA_CHECK(q && kappa && idx && sel_scores, RMA_ERR_INVALID_ARG, "NULL pointer argument");
  RMA_CHECK(aligned16(q) && aligned16(kappa) && aligned16(idx) && aligned16(sel_scores),
            RMA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  TopkPlan pl = plan_topk(*kv, *sp, G, K);
  RMA_CHECK(pl.n_chunks <= kSelMaxChunks, RMA_ERR_UNSUPPORTED, "mid-region too long for G=%d", G);
  RMA_CHECK(workspace != nullptr && aligned16(workspace), RMA_ERR_WORKSPACE,
            "workspace is NULL or misaligned");
  RMA_CHECK(workspace_bytes >= pl.total, RMA_ERR_WORKSPACE, "workspace %zu < required %zu",
            workspace_bytes, pl.total);
  TraceScope ts((hipStream_t)stream);
  hipError_t e = launch_topk(pl, q, G, *kv, *sp, kappa, K, idx, sel_scores, (uint8_t*)workspace,
                             (hipStream_t)stream);
  RMA_CHECK(e == hipSuccess, RMA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return RMA_OK;
}

rma_status rma_decode_topk_static(const float* q, int32_t G, const rma_kv* kv, const rma_span* sp,
                                  const float* kappa, int32_t K, int32_t* idx, float* sel_scores,
                                  void* stream) {
  g_last_error[0] = 0;
  rma_status s = check_kv_span(kv, sp, false);
  if (s != RMA_OK) return s;
  RMA_CHECK(G >= 1 && G <= 8, RMA_ERR_UNSUPPORTED, "G %d not in 1..8", G);
  RMA_CHECK(K >= 0 && K <= l_mid(*sp), RMA_ERR_INVALID_ARG, "K %d outside [0, L_mid=%lld]", K,
            (long long)l_mid(*sp));
  if (K == 0) return RMA_OK;
  RMA_CHECK(q && kappa && idx && sel_scores, RMA_ERR_INVALID_ARG, "NULL pointer argument");
  RMA_CHECK(aligned16(q) && aligned16(kappa) && aligned16(idx) && aligned16(sel_scores),
            RMA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  TopkPlan pl = plan_topk(*kv, *sp, G, K);
  RMA_CHECK(pl.n_chunks <= kSelMaxChunks, RMA_ERR_UNSUPPORTED, "mid-region too long for G=%d", G);
  RMA_CHECK(pl.total <= kStaticScratchBytes, RMA_ERR_WORKSPACE,
            "this call needs %zu bytes of scratch, more than the library's static %zu",
            pl.total, kStaticScratchBytes);
  void* ws = nullptr;
  const hipError_t se = static_scratch(&ws);
  RMA_CHECK(se == hipSuccess && ws != nullptr, RMA_ERR_HIP,
            "address of the static scratch on this device: %s", hipGetErrorString(se));
  TraceScope ts((hipStream_t)stream);
  hipError_t e = launch_topk(pl, q, G, *kv, *sp, kappa, K, idx, sel_scores, (uint8_t*)ws,
                             (hipStream_t)stream);
  RMA_CHECK(e == hipSuccess, RMA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return RMA_OK;
}

rma_status rma_decode_merge(const float* q, const float* phi_q, const float* Wq,
                            const float* bq, int32_t G, const rma_kv* kv,
                            const rma_span* sp, const int32_t* idx, const float* sel, int32_t K,
                            const void* phi_k, int32_t phi_dtype, const float* Wk,
                            const float* bk, int32_t P, int32_t m, const float* S,
                            const float* u, uint32_t flags, float* y, float* stats,
                            void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  rma_status s = check_kv_span(kv, sp, true);
  if (s != RMA_OK) return s;
  RMA_CHECK(G >= 1 && G <= 8, RMA_ERR_UNSUPPORTED, "G %d not in 1..8", G);
  RMA_CHECK(m == 64 || m == 128, RMA_ERR_UNSUPPORTED, "m %d not in {64,128}", m);
  RMA_CHECK(dtype_ok(phi_dtype), RMA_ERR_UNSUPPORTED, "unsupported phi dtype");
  RMA_CHECK(flags == RMA_MERGE_SUB || flags == RMA_MERGE_NO_RESIDUAL ||
                flags == RMA_MERGE_NO_SUBTRACT,
            RMA_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  RMA_CHECK(K >= 0 && K <= l_mid(*sp), RMA_ERR_INVALID_ARG, "K %d outside [0, L_mid]", K);
  RMA_CHECK((int64_t)sp->n_sink + sp->n_tail + sp->n_gen + K > 0, RMA_ERR_INVALID_ARG,
            "empty exact support (no anchors, generated or retrieved tokens)");
  const bool need_res = flags != RMA_MERGE_NO_RESIDUAL;
  RMA_CHECK(q && y, RMA_ERR_INVALID_ARG, "NULL q or y");
  RMA_CHECK(K == 0 || (idx && sel), RMA_ERR_INVALID_ARG, "NULL idx or sel_scores");
  RMA_CHECK(!need_res || (S && u), RMA_ERR_INVALID_ARG, "NULL S or u");
  RMA_CHECK(!need_res || phi_q || (Wq && bq && P >= 1), RMA_ERR_INVALID_ARG,
            "NULL phi_q and no Wq/bq to compute it");
  const bool need_phik = flags == RMA_MERGE_SUB && K > 0 && K < l_mid(*sp);
  RMA_CHECK(!need_phik || phi_k != nullptr || (Wk != nullptr && bk != nullptr && P >= 1),
            RMA_ERR_INVALID_ARG, "NULL phi_k and no Wk/bk to recompute it");
  RMA_CHECK(!need_phik || phi_k != nullptr || (kv->dtype == RMA_BF16 && phi_dtype == RMA_BF16),
            RMA_ERR_UNSUPPORTED, "recomputed phi_k rows need bf16 keys and bf16 phi rounding");
  RMA_CHECK(aligned16(q) && aligned16(phi_q) && aligned16(Wq) && aligned16(bq) &&
                aligned16(idx) && aligned16(sel) &&
                aligned16(phi_k) && aligned16(Wk) && aligned16(bk) && aligned16(S) &&
                aligned16(u) && aligned16(y) && aligned16(stats),
            RMA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  MergePlan pl = plan_merge(*kv, *sp, G, K, m);
  RMA_CHECK(workspace != nullptr && aligned16(workspace), RMA_ERR_WORKSPACE,
            "workspace is NULL or misaligned");
  RMA_CHECK(workspace_bytes >= pl.total, RMA_ERR_WORKSPACE, "workspace %zu < required %zu",
            workspace_bytes, pl.total);
  TraceScope ts((hipStream_t)stream);
  // stored rows take precedence; the recompute runs only when they are absent
  hipError_t e = launch_merge(pl, q, phi_q, phi_q ? nullptr : Wq, bq, G, *kv, *sp, idx, sel, K,
                              phi_k, phi_dtype,
                              phi_k ? nullptr : Wk, bk, P, m, S, u, flags, y, stats,
                              (uint8_t*)workspace, (hipStream_t)stream);
  RMA_CHECK(e == hipSuccess, RMA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return RMA_OK;
}

rma_status rma_decode(const float* q, const float* phi_q, const float* Wq, const float* bq,
                      int32_t G, const rma_kv* kv, const rma_span* sp, const float* kappa,
                      int32_t K, const void* phi_k, int32_t phi_dtype, const float* Wk,
                      const float* bk, int32_t P, int32_t m, const float* S, const float* u,
                      uint32_t flags, int32_t* idx, float* sel, float* y, float* stats,
                      void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  rma_status s = check_kv_span(kv, sp, true);
  if (s != RMA_OK) return s;
  RMA_CHECK(G >= 1 && G <= 8, RMA_ERR_UNSUPPORTED, "G %d not in 1..8", G);
  RMA_CHECK(m == 64 || m == 128, RMA_ERR_UNSUPPORTED, "m %d not in {64,128}", m);
  RMA_CHECK(dtype_ok(phi_dtype), RMA_ERR_UNSUPPORTED, "unsupported phi dtype");
  RMA_CHECK(flags == RMA_MERGE_SUB || flags == RMA_MERGE_NO_RESIDUAL ||
                flags == RMA_MERGE_NO_SUBTRACT,
            RMA_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  RMA_CHECK(K >= 0 && K <= l_mid(*sp), RMA_ERR_INVALID_ARG, "K %d outside [0, L_mid=%lld]", K,
            (long long)l_mid(*sp));
  RMA_CHECK((int64_t)sp->n_sink + sp->n_tail + sp->n_gen + K > 0, RMA_ERR_INVALID_ARG,
            "empty exact support (no anchors, generated or retrieved tokens)");
  const bool need_res = flags != RMA_MERGE_NO_RESIDUAL;
  RMA_CHECK(q && y, RMA_ERR_INVALID_ARG, "NULL q or y");
  RMA_CHECK(K == 0 || kappa, RMA_ERR_INVALID_ARG, "NULL kappa");
  RMA_CHECK((idx == nullptr) == (sel == nullptr), RMA_ERR_INVALID_ARG,
            "idx and sel_scores must be given together");
  RMA_CHECK(!need_res || (S && u), RMA_ERR_INVALID_ARG, "NULL S or u");
  RMA_CHECK(!need_res || phi_q || (Wq && bq && P >= 1), RMA_ERR_INVALID_ARG,
            "NULL phi_q and no Wq/bq to compute it");
  const bool need_phik = flags == RMA_MERGE_SUB && K > 0 && K < l_mid(*sp);
  RMA_CHECK(!need_phik || phi_k != nullptr || (Wk != nullptr && bk != nullptr && P >= 1),
            RMA_ERR_INVALID_ARG, "NULL phi_k and no Wk/bk to recompute it");
  RMA_CHECK(!need_phik || phi_k != nullptr || (kv->dtype == RMA_BF16 && phi_dtype == RMA_BF16),
            RMA_ERR_UNSUPPORTED, "recomputed phi_k rows need bf16 keys and bf16 phi rounding");
  RMA_CHECK(aligned16(q) && aligned16(phi_q) && aligned16(Wq) && aligned16(bq) &&
                aligned16(kappa) && aligned16(idx) && aligned16(sel) && aligned16(phi_k) &&
                aligned16(Wk) && aligned16(bk) && aligned16(S) && aligned16(u) && aligned16(y) &&
                aligned16(stats),
            RMA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const bool recompute = need_phik && phi_k == nullptr;
  DecodePlan pl = plan_decode(*kv, *sp, G, K, m, phi_dtype, recompute);
  RMA_CHECK(K == 0 || pl.topk.n_chunks <= kSelMaxChunks, RMA_ERR_UNSUPPORTED,
            "mid-region too long for G=%d", G);
  RMA_CHECK(workspace != nullptr && aligned16(workspace), RMA_ERR_WORKSPACE,
            "workspace is NULL or misaligned");
  RMA_CHECK(workspace_bytes >= pl.total, RMA_ERR_WORKSPACE, "workspace %zu < required %zu",
            workspace_bytes, pl.total);
  TraceScope ts((hipStream_t)stream);
  const hipStream_t st = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  hipError_t e = hipSuccess;
  if (K > 0) e = launch_topk_scan(pl.topk, q, G, *kv, *sp, kappa, ws, st);
  if (e == hipSuccess && pl.fused) {
    e = launch_decode_fused(pl, q, G, *kv, *sp, K, idx, sel, phi_q, phi_q ? nullptr : Wq, bq, P,
                            phi_k, phi_dtype, m, S, u, flags, y, stats, ws, st);
  } else if (e == hipSuccess) {
    int32_t* ii = idx ? idx : reinterpret_cast<int32_t*>(ws + pl.off_idx);
    float* ss = sel ? sel : reinterpret_cast<float*>(ws + pl.off_sel);
    if (K > 0) e = launch_topk_select(pl.topk, q, G, *kv, *sp, K, ii, ss, ws, st);
    if (e == hipSuccess)
      e = launch_merge(pl.merge, q, phi_q, phi_q ? nullptr : Wq, bq, G, *kv, *sp, ii, ss, K, phi_k,
                       phi_dtype, phi_k ? nullptr : Wk, bk, P, m, S, u, flags, y, stats,
                       ws + pl.off_merge, st);
  }
  RMA_CHECK(e == hipSuccess, RMA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return RMA_OK;
}

rma_status rma_decode_full(const float* q, int32_t G, const rma_kv* kv, const rma_span* sp,
                           const int32_t* idx, int32_t K, const float* y_cmp, float* y_full,
                           float* diag, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  rma_status s = check_kv_span(kv, sp, true);
  if (s != RMA_OK) return s;
  RMA_CHECK(G >= 1 && G <= 8, RMA_ERR_UNSUPPORTED, "G %d not in 1..8", G);
  RMA_CHECK(sp->L + sp->n_gen > 0, RMA_ERR_INVALID_ARG, "empty context (L + n_gen == 0)");
  RMA_CHECK(K >= 0 && K <= l_mid(*sp), RMA_ERR_INVALID_ARG, "K %d outside [0, L_mid=%lld]", K,
            (long long)l_mid(*sp));
  RMA_CHECK(q && y_full, RMA_ERR_INVALID_ARG, "NULL q or y_full");
  RMA_CHECK(aligned16(q) && aligned16(idx) && aligned16(y_cmp) && aligned16(y_full) &&
                aligned16(diag),
            RMA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  FullPlan pl = plan_full(*kv, *sp, G);
  RMA_CHECK(workspace != nullptr && aligned16(workspace), RMA_ERR_WORKSPACE,
            "workspace is NULL or misaligned");
  RMA_CHECK(workspace_bytes >= pl.total, RMA_ERR_WORKSPACE, "workspace %zu < required %zu",
            workspace_bytes, pl.total);
  TraceScope ts((hipStream_t)stream);
  hipError_t e = launch_full(pl, q, G, *kv, *sp, K > 0 ? idx : nullptr, K, y_cmp, y_full, diag,
                             (uint8_t*)workspace, (hipStream_t)stream);
  RMA_CHECK(e == hipSuccess, RMA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return RMA_OK;
}

}  // extern "C"
