// Host-side planning shared by the C ABI entry points and the kernel launchers.
// A plan fixes the tiling of one call; the workspace size and every launch are
// derived from the same plan, so they cannot disagree.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <tuple>

#include "../../include/rma.h"

namespace rma {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workspaces hold per-call scratch only: every byte a kernel reads from one is
// written earlier in the same call, so a workspace needs no initialisation.

// ------------------------------------------------------------- device
// Properties of the calling thread's current HIP device, queried once per
// device (std::call_once per device id, so concurrent first calls are safe) and
// read-only afterwards.  Devices beyond kMaxDevices, or a failed query, get
// conservative defaults.
constexpr int kMaxDevices = 64;
struct DeviceInfo {
  int cus;               // compute units
  size_t lds_per_block;  // bytes of LDS one workgroup may use
};
const DeviceInfo& device_info();

// Device address of the library's static scratch on the current device
// (rma_decode_topk_static), looked up once per device.
constexpr size_t kStaticScratchBytes = RMA_STATIC_SCRATCH_BYTES;
hipError_t static_scratch(void** ptr);

// Static LDS bytes of the kernel Kern (a property of its code object, the same
// on every gfx950 device): queried on first use, a thread-safe function-local
// static per kernel.  The kernel is a template argument so that every kernel
// has its own cache (instantiations that differ only in non-type template
// parameters share one function type).  A failed query reads as "does not fit".
template <auto Kern>
size_t kernel_static_lds() {
  static const size_t bytes = [] {
    hipFuncAttributes attr{};
    return hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(Kern)) == hipSuccess
               ? (size_t)attr.sharedSizeBytes
               : (size_t)1 << 30;
  }();
  return bytes;
}

// ------------------------------------------------------------- build
struct BuildPlan {
  bool mfma;         // bf16 K/V and bf16 phi rows (computed or given) -> MFMA builder
  int n_chunks;      // token chunks per unit
  int ch;            // tokens per chunk (multiple of the tile)
  size_t off_S, off_u, off_kap, total;
};
// tokens: mid-region positions covered by one call (all of L_mid, or a range)
BuildPlan plan_build(const rma_kv& kv, int64_t tokens, int m, bool computed_phi, int phi_dtype);

// ------------------------------------------------------------- top-k
constexpr int kScanThreads = 256;
// tokens a scan block scores per pass: 64 / (d / 16) tokens per wave
constexpr int scan_tile(int d) { return (kScanThreads / 64) * (64 / (d / 16)); }
constexpr int kScanBlocks = 512;        // scan blocks aimed for when the units are few
constexpr int kScanBins = 512;          // linear score bins per head in the scan
constexpr int kScanLdsBudget = 54272;   // LDS bytes per scan block: three fit the 160 KB of a CU
// tokens per scan chunk that fit the budget: G rows of fp32 scores (8 words of
// padding each) beside the G histograms and the G queries, whole block passes
constexpr int scan_chmax(int d, int G) {
  return ((kScanLdsBudget - G * (kScanBins * 4 + d * 4) - 64) / (4 * G) - 8) / scan_tile(d) * scan_tile(d);
}
constexpr int kSelMaxChunks = 256;
constexpr int kSelBandMax = 512;        // band members resolved in LDS
constexpr int kSelMaxEntries = 16384;   // union entries held in LDS by a select block
constexpr int kSelBins = 1024;          // linear bins over the union's score range
constexpr int kSelThreads = 1024;       // select block size

struct TopkPlan {
  int n_chunks, ch, r_min, r_cap;
  int e_max;                 // entries the select block can hold
  size_t off_ent, off_meta, off_hp, total;
  size_t sel_lds;            // dynamic LDS bytes of the select kernel
};
TopkPlan plan_topk(const rma_kv& kv, const rma_span& sp, int G, int K);

// ------------------------------------------------------------- merge
constexpr int kMergeThreads = 512;    // one block per (unit, query head)
constexpr int kMergeChunk = 2048;     // exact-support entries staged in LDS at a time
constexpr int kMergeCombineThreads = 256;   // >= the most slices a head gets

struct MergePlan {
  int n_slices, sl;          // slices of the per-head entry list, entries per slice
  int part_floats;           // floats per (slice, head) partial
  size_t off_part, total;
};
MergePlan plan_merge(const rma_kv& kv, const rma_span& sp, int G, int K, int m);

// ------------------------------------------------------------- fused decode
// rma_decode: the scan of rma_decode_topk, then either the fused select-and-merge
// kernel (one block per head; when its union, list and static LDS fit) or the
// separate select and merge kernels on the same scan output.
struct DecodePlan {
  TopkPlan topk;       // the scan's chunks and reports (workspace offset 0)
  bool fused;
  int fused_threads;   // 256, 512 or 1024
  int fused_split;     // blocks per head of the fused kernel (> 1: partials + combine)
  MergePlan merge;     // the separate path
  size_t off_idx, off_sel, off_merge, off_fpart, total;
};
DecodePlan plan_decode(const rma_kv& kv, const rma_span& sp, int G, int K, int m, int phi_dtype,
                       bool recompute);
// report slots each thread of the fused kernel loads per round (a chunk's slots
// are spread over the 2^(log2 NT - ceil(log2 n_chunks)) threads it gets)
template <int NT> constexpr int kFusedSpec = 8;
// Retrieved entries each 8-lane group of the fused kernel gathers per round
// (every load of a round in flight together): as many as its registers allow
// (128 per lane in 1024-thread blocks) without spilling
constexpr int fused_gather_batch(int kt_bytes, int pt_bytes, int d, int nt) {
  const int b0 = kt_bytes == 4 ? 2 : pt_bytes == 4 ? (d == 128 ? 2 : 4) : d == 128 ? 4 : 8;
  if (nt != 1024) return b0;
  if (kt_bytes == 2 && pt_bytes == 2 && d == 128) return 3;
  return b0 > 1 ? b0 / 2 : 1;
}
inline bool fused_slots_fit(int n_chunks, int nt) { return n_chunks >= 1 && n_chunks <= nt; }
// dynamic LDS of the fused kernel: the union of the chunk reports and the
// selected list, or (reusing it) the combine's group-pair sums
inline size_t fused_dyn_bytes(int n_chunks, int r_cap, int K, int d, int nt) {
  const size_t ub = 64;   // the union padded to whole rows of 64 entries
  const size_t a = 2 * (((size_t)n_chunks * r_cap + ub - 1) / ub * ub);
  const size_t b = (size_t)(nt / 16) * (2 * d + 8);   // the combine's pair sums reuse the union
  return ((a > b ? a : b) + 2 * (size_t)K) * 4 + 16;
}
// static LDS of the fused kernel instantiation a plan would launch
size_t fused_static_lds(int kv_dtype, int phi_dtype, int d, int m, int nt);

// ------------------------------------------------------------- MLP feature map
constexpr int kPhiMlpWidth = RMA_PHI_MLP_WIDTH;

// ------------------------------------------------------------- full attention
constexpr int kFullThreads = 256;
constexpr int kFullMaxChunk = 8192;   // positions per chunk (membership bits in LDS)
constexpr int kFullRecHead = 8;       // floats before N in a chunk record
constexpr int kFullCombineThreads = 256;

struct FullPlan {
  int n_chunks, ch;
  size_t off_part, total;
};
FullPlan plan_full(const rma_kv& kv, const rma_span& sp, int G);

// ------------------------------------------------------------- kernel timing
// Benchmark instrumentation armed by rma_trace_arm: each kernel of the next call
// takes the next pair of events, stamped by its own dispatch at the start and at
// the end of its execution.  Thread-local.
constexpr int kTraceMax = 16;
struct KernelTrace {
  hipEvent_t ev[kTraceMax];
  const char* name[kTraceMax / 2];
  int n_events = 0;   // armed events (0 = off)
  int used = 0;       // events taken by the current call
  int count = 0;      // kernels timed by the last traced call
};
KernelTrace& trace();

// Enqueues kern<<<grid, block, shm, st>>>(args...).  With a trace armed and a
// pair of events left, the launch goes through hipExtLaunchKernel with that pair.
template <typename... Params, typename... Args>
hipError_t launch_kernel(const char* name, void (*kern)(Params...), dim3 grid, dim3 block,
                         uint32_t shm, hipStream_t st, Args... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "kernel argument count");
  std::tuple<Params...> vals(static_cast<Params>(args)...);
  return std::apply(
      [&](auto&... v) {
        void* argv[] = {const_cast<void*>(static_cast<const void*>(&v))..., nullptr};
        const void* fn = reinterpret_cast<const void*>(kern);
        KernelTrace& t = trace();
        if (t.n_events > 0 && t.used + 2 <= t.n_events) {
          const hipError_t e = hipExtLaunchKernel(fn, grid, block, argv, shm, st, t.ev[t.used],
                                                  t.ev[t.used + 1], 0);
          if (e == hipSuccess) {
            t.name[t.used / 2] = name;
            t.used += 2;
          }
          return e;
        }
        return hipLaunchKernel(fn, grid, block, argv, shm, st);
      },
      vals);
}

// ------------------------------------------------------------- launchers
hipError_t launch_phi(const void* x, int x_dtype, int n_units, int64_t rows, int64_t x_unit_stride,
                      int d, const float* W, const float* b, int m, int P, void* phi,
                      int phi_dtype, hipStream_t st);

hipError_t launch_stream_read(const void* p, int64_t bytes, int blocks, uint32_t* sink, hipStream_t st);

hipError_t launch_build(const BuildPlan& pl, const rma_kv& kv, const rma_span& sp, int m0, int len,
                        bool acc, const float* W, const float* b, int m, int P, void* phi_k,
                        int phi_dtype, float* S, float* u, float* kappa, uint8_t* ws,
                        hipStream_t st);

hipError_t launch_topk_scan(const TopkPlan& pl, const float* q, int G, const rma_kv& kv,
                            const rma_span& sp, const float* kappa, uint8_t* ws, hipStream_t st);
hipError_t launch_topk_select(const TopkPlan& pl, const float* q, int G, const rma_kv& kv,
                              const rma_span& sp, int K, int32_t* idx, float* sel, uint8_t* ws,
                              hipStream_t st);
hipError_t launch_topk(const TopkPlan& pl, const float* q, int G, const rma_kv& kv,
                       const rma_span& sp, const float* kappa, int K, int32_t* idx,
                       float* sel_scores, uint8_t* ws, hipStream_t st);

// combines per-slice partials (merge_kernel's layout) of `heads` query heads
hipError_t launch_merge_combine(const float* parts, int n_slices, int heads, int d, uint32_t flags,
                                int K, int L_mid, float* y, float* stats, hipStream_t st);
hipError_t launch_merge(const MergePlan& pl, const float* q, const float* phi_q, const float* Wq,
                        const float* bq, int G,
                        const rma_kv& kv, const rma_span& sp, const int32_t* idx,
                        const float* sel, int K, const void* phi_k, int phi_dtype,
                        const float* Wk, const float* bk, int P, int m, const float* S,
                        const float* u, uint32_t flags, float* y, float* stats, uint8_t* ws,
                        hipStream_t st);

hipError_t launch_decode_fused(const DecodePlan& pl, const float* q, int G, const rma_kv& kv,
                               const rma_span& sp, int K, int32_t* idx, float* sel,
                               const float* phi_q, const float* Wq, const float* bq, int P,
                               const void* phi_k, int phi_dtype, int m, const float* S,
                               const float* u, uint32_t flags, float* y, float* stats, uint8_t* ws,
                               hipStream_t st);

hipError_t launch_phi_mlp(const void* x, int x_dtype, int n_units, int64_t rows, int64_t xstride,
                          int d, const rma_phi_mlp* w, int m, int P, void* phi, int phi_dtype,
                          hipStream_t st);

hipError_t launch_full(const FullPlan& pl, const float* q, int G, const rma_kv& kv,
                       const rma_span& sp, const int32_t* idx, int K, const float* y_cmp,
                       float* y, float* diag, uint8_t* ws, hipStream_t st);

}  // namespace rma
