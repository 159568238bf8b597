// Internal interface between the C-ABI host code (ssw_api.cpp) and the gfx950 kernels
// (band_attn.hip).  Not installed; the public interface is include/ssw.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace ssw {

// What a launch does with gate * Y at the output row.
//   kEpiStore:      store it in the output dtype.
//   kEpiPartial:    store it as the gated path's intermediate (SWA pass, sigma = identity only):
//                   fp32 for fp32 outputs; for bf16 outputs, fp16 bits of Y * 2^-8 in the same
//                   two bytes (8x finer than bf16, so the final result is rounded to bf16 once
//                   in effect; holds |Y| < 1.6e7).
//   kEpiAddPartial: read that intermediate, add, store in the output dtype (SA pass).
enum Epilogue { kEpiStore = 0, kEpiPartial = 1, kEpiAddPartial = 2 };

// One band-attention launch.  `perm` selects the stochastic (sigma-gathered) operator; without
// it sigma is the identity (plain SWA).
struct BandLaunch {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* sigma;  // device int32[n] when perm, else ignored
  const float* gate;     // device float32 [B, n, Hq] or nullptr
  void* out;
  int B, n, Hq, Hkv, d;
  int dtype;             // 0 = fp32, 1 = bf16
  int window;            // already clamped to [1, n]
  bool causal;
  bool perm;
  int epilogue;          // Epilogue
  // optional hipEvent_t pair attached to the kernel's dispatch: recorded when the kernel starts
  // and when it ends (no separate event packets around it)
  void* ev_start = nullptr;
  void* ev_stop = nullptr;
};

hipError_t launch_band_attn(const BandLaunch& a, hipStream_t stream);

// bits [n][ceil(n/32)] uint32, overwritten.  sigma may be nullptr (identity).
hipError_t launch_neighbor_mask(const int32_t* sigma, int n, int window, bool causal,
                                uint32_t* bits, hipStream_t stream);

}  // namespace ssw
