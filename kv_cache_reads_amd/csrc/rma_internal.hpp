// Host-side planning shared by the C ABI entry points and the kernel launchers.
// A plan fixes the tiling of one call; the workspace size and every launch are
// derived from the same plan, so they cannot disagree.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>

#include "../../include/rma.h"

namespace rma {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Completion counters (one uint32 per unit, up to the 65535-unit limit) lead
// every workspace at a fixed size, so that scratch written by one call never
// lands on counters another call (with a different unit count) relies on.
constexpr size_t kCounterBytes = 65536 * 4;
inline size_t counter_bytes(int64_t /*n_units*/) { return kCounterBytes; }

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
constexpr int kScanBins = 512;          // linear score bins per head in the scan
constexpr int kScanScoreSlots = 8192;   // fp32 LDS score slots per scan block (G * ch <= this)
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

hipError_t launch_build(const BuildPlan& pl, const rma_kv& kv, const rma_span& sp, int m0, int len,
                        bool acc, const float* W, const float* b, int m, int P, void* phi_k,
                        int phi_dtype, float* S, float* u, float* kappa, uint8_t* ws,
                        hipStream_t st);

hipError_t launch_topk(const TopkPlan& pl, const float* q, int G, const rma_kv& kv,
                       const rma_span& sp, const float* kappa, int K, int32_t* idx,
                       float* sel_scores, uint8_t* ws, hipStream_t st);

hipError_t launch_merge(const MergePlan& pl, const float* q, const float* phi_q, const float* Wq,
                        const float* bq, int G,
                        const rma_kv& kv, const rma_span& sp, const int32_t* idx,
                        const float* sel, int K, const void* phi_k, int phi_dtype,
                        const float* Wk, const float* bk, int P, int m, const float* S,
                        const float* u, uint32_t flags, float* y, float* stats, uint8_t* ws,
                        hipStream_t st);

hipError_t launch_phi_mlp(const void* x, int x_dtype, int n_units, int64_t rows, int64_t xstride,
                          int d, const rma_phi_mlp* w, int m, int P, void* phi, int phi_dtype,
                          hipStream_t st);

hipError_t launch_full(const FullPlan& pl, const float* q, int G, const rma_kv& kv,
                       const rma_span& sp, const int32_t* idx, int K, const float* y_cmp,
                       float* y, float* diag, uint8_t* ws, hipStream_t st);

}  // namespace rma
