// Internal interface between the C-ABI host code (ssw_api.cpp) and the gfx950 kernels
// (band_attn.hip).  Not installed; the public interface is include/ssw.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace ssw {

// What a launch does with gate * Y at the output row.
//   kEpiStore:      store it in the output dtype.
//   kEpiPartial:    store it as the gated layer's intermediate (its first pass, the
//                   sigma-gathered SA pass): fp32 for fp32 outputs; for bf16 outputs, fp16 bits
//                   of Y * 2^-4 in the same two bytes (holds |Y| < 1.05e6; 3 more significand
//                   bits than bf16 for |Y| >= 2^-10, a fixed 2^-20 step below that).
//   kEpiAddPartial: read that intermediate, add, store in the output dtype (the gated layer's
//                   second pass, plain SWA with sigma = identity).
enum Epilogue { kEpiStore = 0, kEpiPartial = 1, kEpiAddPartial = 2 };

// One band-attention launch.  `perm` selects the stochastic (sigma-gathered) operator; without
// it sigma is the identity (plain SWA).
struct BandLaunch {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* sigma;  // device int32[n] when perm, else ignored
  // sigma of (batch row b, KV head g) starts at sigma + b * sig_bstride + g * sig_hstride
  int64_t sig_bstride = 0;
  int64_t sig_hstride = 0;
  const float* gate;     // device float32 [B, n, Hq] or nullptr
  void* out;
  int B, n, Hq, Hkv, d;
  int dtype;             // 0 = fp32, 1 = bf16
  int window;            // already clamped to [1, n]
  bool causal;
  bool perm;
  int epilogue;          // Epilogue
  // optional: the natural-log log-sum-exp of every row, fp32 [B, n, Hq] at original positions
  float* lse = nullptr;
  // optional hipEvent_t pair attached to the kernel's dispatch: recorded when the kernel starts
  // and when it ends (no separate event packets around it)
  void* ev_start = nullptr;
  void* ev_stop = nullptr;
};

hipError_t launch_band_attn(const BandLaunch& a, hipStream_t stream);

// The backward of one band-attention layer y = gate * A (A = the attention output), bf16 only.
// Two launches: the dQ kernel (which also stores Delta = gate * rowsum(dout * A) and, if dgate
// is set, dgate = rowsum(dout * A)), then the dK/dV kernel that reads Delta.
struct BandBwdLaunch {
  const void* q;
  const void* k;
  const void* v;
  const void* o;          // A, [B, n, Hq, d]
  const void* dout;       // dL/dy, [B, n, Hq, d]
  const float* lse;       // [B, n, Hq], natural log
  const float* gate;      // [B, n, Hq] or nullptr (gate 1)
  const int32_t* sigma;   // device int32[n] when perm
  void* dq;
  void* dk;
  void* dv;
  float* dgate;           // [B, n, Hq] or nullptr
  float* delta;           // [B, n, Hq] scratch, overwritten
  int B, n, Hq, Hkv, d;
  int window;             // already clamped to [1, n]
  bool causal;
  bool perm;
  bool accumulate;        // add into dq, dk, dv instead of overwriting them
  void* ev[4] = {nullptr, nullptr, nullptr, nullptr};  // optional dispatch events: dq start/stop,
                                                       // dk/dv start/stop
};

hipError_t launch_band_attn_bwd(const BandBwdLaunch& a, hipStream_t stream);

// The library's own Delta array for the backward entry point that allocates nothing: entries
// (B * n * Hq at most), and its device address on the current device (looked up once per device).
constexpr int64_t kBwdScratchFloats = int64_t(1) << 22;  // 16 MiB
hipError_t bwd_scratch_pointer(float** ptr);

// One decode step per batch row over a KV cache (SA and/or SWA, optionally gated).
struct DecodeLaunch {
  const void* q;          // [B, Hq, d]
  const void* k_cache;    // [B, n_max, Hkv, d]
  const void* v_cache;
  const int32_t* sigma;   // [n_max] (SA path)
  const int32_t* inv_sigma;
  const int32_t* pos;     // [B] device
  const float* gate;      // paths 1 or 2: [B, Hq] or nullptr; paths 3: [2, B, Hq]
  void* out;              // [B, Hq, d]
  int B, n_max, Hq, Hkv, d, dtype;
  int window;             // already clamped to [1, n_max]
  int paths;              // bit 0: SA, bit 1: SWA
};

hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream);

// out = g_sa * y_sa + g_swa * y_swa for bf16 rows of d elements; gates [2, rows] fp32.
hipError_t launch_gate_combine(const void* y_sa, const void* y_swa, const float* gates,
                               void* out, int64_t rows, int d, hipStream_t stream);

// bits [n][ceil(n/32)] uint32, overwritten.  sigma may be nullptr (identity).
hipError_t launch_neighbor_mask(const int32_t* sigma, int n, int window, bool causal,
                                uint32_t* bits, hipStream_t stream);

}  // namespace ssw
