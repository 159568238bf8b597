// C ABI of libssw.so (declared in include/ssw.h): argument checking, the host-side permutation
// generator and dispatch of the gfx950 kernels in band_attn.hip.
//
// Nothing here allocates device memory; forward and backward calls only enqueue kernels on the
// caller's stream.  Errors are reported as negative status codes plus a per-thread message; no C++
// exception crosses the ABI.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "../../include/ssw.h"
#include "band_attn.h"
#include "gate_proj.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// splitmix64 (Steele, Lea & Flood 2014): advance the state by the golden-ratio increment, then
// finalise it with two xor-shift/multiply rounds and a last xor-shift.
struct SplitMix64 {
  uint64_t state;
  uint64_t next() {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

// Shared checks of the three forward entry points.
int check_forward(const char* who, const void* q, const void* k, const void* v, const void* out,
                  int window, int causal, int B, int n, int Hq, int Hkv, int d, int dtype) {
  const std::string w(who);
  if (B < 0 || n < 0) return fail(SSW_EINVAL, w + ": B and n must be >= 0");
  if (window < 1) return fail(SSW_EINVAL, w + ": window must be >= 1");
  if (causal != 0 && causal != 1) return fail(SSW_EINVAL, w + ": causal must be 0 or 1");
  if (Hq < 1 || Hkv < 1) return fail(SSW_EINVAL, w + ": Hq and Hkv must be >= 1");
  if (Hq % Hkv != 0) return fail(SSW_ESHAPE, w + ": Hq must be a multiple of Hkv");
  if (dtype != SSW_F32 && dtype != SSW_BF16) return fail(SSW_EDTYPE, w + ": unsupported dtype");
  if (d != 64 && d != 128) return fail(SSW_EDTYPE, w + ": head dim d must be 64 or 128");
  // every index the kernels form must stay inside int32 where they use int32
  const int64_t G = Hq / Hkv;
  // (n * G / 128 column tiles) * B * Hkv workgroups must fit a 1-D grid
  if ((int64_t)n * G > ((int64_t)1 << 31) - 4096 || (int64_t)B * Hkv >= 65536 ||
      ((int64_t)n * G / 128 + 1) * B * Hkv >= ((int64_t)1 << 31))
    return fail(SSW_ESHAPE, w + ": n * Hq / Hkv must be <= 2^31 - 4096, B * Hkv < 65536 and "
                                "n * Hq * B / 128 < 2^31");
  // K and V rows of one (batch row, KV head) are addressed with 32-bit byte offsets below 2^31
  // (offset 2^31 is the kernels' "read zeros" marker)
  // (and row offsets are formed with 24-bit multiplies: n <= 2^24 - 64, a K/V token row < 2^24
  // bytes);
  // one batch row of out is addressed the same way
  const int64_t elem = dtype == SSW_BF16 ? 2 : 4;
  if ((int64_t)n * Hkv * d * elem > ((int64_t)1 << 31) - 4096 ||
      (int64_t)n * Hq * d * elem > ((int64_t)1 << 31) - 4096 || n > (1 << 24) - 64 ||
      (int64_t)Hkv * d * elem >= (1 << 24))
    return fail(SSW_ESHAPE, w + ": n * Hq * d * element size must be <= 2^31 - 4096 bytes and "
                                "n <= 2^24 - 64");
  if (B == 0 || n == 0) return SSW_OK;
  if (!q || !k || !v || !out) return fail(SSW_EINVAL, w + ": q, k, v and out must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(SSW_EALIGN, w + ": q, k, v and out must be 16-byte aligned");
  return SSW_OK;
}

int check_sigma_on_device(const int32_t* sigma, int n, hipStream_t stream) {
  std::vector<int32_t> host((size_t)n);
  hipError_t e = hipStreamSynchronize(stream);
  if (e == hipSuccess)
    e = hipMemcpy(host.data(), sigma, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess)
    return fail(SSW_EHIP, std::string("SSW_VALIDATE copy of sigma failed: ") + hipGetErrorString(e));
  if (ssw_check_permutation(host.data(), n) != SSW_OK)
    return fail(SSW_ENOTPERM, "sigma is not a permutation of [0, n)");
  return SSW_OK;
}

bool validate_requested() {
  const char* s = getenv("SSW_VALIDATE");
  return s && s[0] == '1';
}

int run(const char* who, const ssw::BandLaunch& a, hipStream_t stream) {
  hipError_t e = ssw::launch_band_attn(a, stream);
  if (e != hipSuccess)
    return fail(SSW_EHIP, std::string(who) + ": kernel launch failed: " + hipGetErrorString(e));
  return SSW_OK;
}

ssw::BandLaunch make_launch(const void* q, const void* k, const void* v, const int32_t* sigma,
                            int window, int causal, const float* gate, void* out, int B, int n,
                            int Hq, int Hkv, int d, int dtype) {
  ssw::BandLaunch a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.sigma = sigma;
  a.gate = gate;
  a.out = out;
  a.B = B;
  a.n = n;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.dtype = dtype;
  a.window = window < n ? window : n;  // a band of n - 1 already covers every slot
  a.causal = causal != 0;
  a.perm = sigma != nullptr;
  a.epilogue = ssw::kEpiStore;
  return a;
}

}  // namespace

extern "C" {

int ssw_sa_forward(const void* q, const void* k, const void* v, const int32_t* sigma, int window,
                   int causal, const float* gate, void* out, int B, int n, int Hq, int Hkv, int d,
                   int dtype, void* stream) {
  const char* who = "ssw_sa_forward";
  int st = check_forward(who, q, k, v, out, window, causal, B, n, Hq, Hkv, d, dtype);
  if (st != SSW_OK || B == 0 || n == 0) return st;
  if (!sigma) return fail(SSW_EINVAL, "ssw_sa_forward: sigma must be non-NULL");
  if (!aligned(sigma, 4) || (gate && !aligned(gate, 4)))
    return fail(SSW_EALIGN, "ssw_sa_forward: sigma and gate must be 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (validate_requested()) {
    st = check_sigma_on_device(sigma, n, s);
    if (st != SSW_OK) return st;
  }
  return run(who, make_launch(q, k, v, sigma, window, causal, gate, out, B, n, Hq, Hkv, d, dtype),
             s);
}

int ssw_swa_forward(const void* q, const void* k, const void* v, const int32_t* sigma, int window,
                    int causal, const float* gate, void* out, int B, int n, int Hq, int Hkv, int d,
                    int dtype, void* stream) {
  const char* who = "ssw_swa_forward";
  int st = check_forward(who, q, k, v, out, window, causal, B, n, Hq, Hkv, d, dtype);
  if (st != SSW_OK || B == 0 || n == 0) return st;
  if (sigma) return fail(SSW_EINVAL, "ssw_swa_forward: sigma must be NULL (identity)");
  if (gate && !aligned(gate, 4))
    return fail(SSW_EALIGN, "ssw_swa_forward: gate must be 4-byte aligned");
  return run(who,
             make_launch(q, k, v, nullptr, window, causal, gate, out, B, n, Hq, Hkv, d, dtype),
             (hipStream_t)stream);
}

// The gated layer's two passes (arguments already checked): the SA pass (sigma of batch row b
// and KV head g at sigma + b * sb + g * sh) leaves the intermediate, the SWA pass adds to it.
static int run_gated(const char* who, const void* q, const void* k, const void* v,
                     const int32_t* sigma, int64_t sb, int64_t sh, int window, int causal,
                     const float* gates, void* out, int B, int n, int Hq, int Hkv, int d,
                     int dtype, hipStream_t s, void* const* events) {
  const float* g_sa = gates;
  const float* g_swa = gates + (size_t)B * n * Hq;
  // Pass 1: the SA pass leaves g_sa * Y_sa in `out` as the intermediate, at the scattered rows
  // sigma[p] (fp32, or for bf16 outputs fp16 bits of the value times 2^-4, so that the sum is
  // in effect rounded to bf16 once).  sigma being a bijection means every row is written once.
  ssw::BandLaunch a1 =
      make_launch(q, k, v, sigma, window, causal, g_sa, out, B, n, Hq, Hkv, d, dtype);
  a1.epilogue = ssw::kEpiPartial;
  a1.sig_bstride = sb;
  a1.sig_hstride = sh;
  // Pass 2: the SWA pass reads the intermediate of its own (contiguous) rows, adds
  // g_swa * Y_swa and stores the result.  Stream order makes the read-modify-write race-free.
  // This order keeps the read-modify-write out of the sigma-gathered pass, which has the more
  // arithmetic per byte of the two.
  ssw::BandLaunch a2 =
      make_launch(q, k, v, nullptr, window, causal, g_swa, out, B, n, Hq, Hkv, d, dtype);
  a2.epilogue = ssw::kEpiAddPartial;
  if (events) {
    // events[0..1] bracket the SWA pass and events[2..3] the SA pass, whatever their order
    a2.ev_start = events[0];
    a2.ev_stop = events[1];
    a1.ev_start = events[2];
    a1.ev_stop = events[3];
  }
  int st = run(who, a1, s);
  if (st != SSW_OK) return st;
  return run(who, a2, s);
}


static int gated(const char* who, const void* q, const void* k, const void* v,
                 const int32_t* sigma, int window, int causal, const float* gates, void* out,
                 int B, int n, int Hq, int Hkv, int d, int dtype, void* stream,
                 void* const* events) {
  int st = check_forward(who, q, k, v, out, window, causal, B, n, Hq, Hkv, d, dtype);
  if (st != SSW_OK || B == 0 || n == 0) return st;
  if (!sigma || !gates) return fail(SSW_EINVAL, std::string(who) + ": sigma and gates must be non-NULL");
  if (!aligned(sigma, 4) || !aligned(gates, 4))
    return fail(SSW_EALIGN, std::string(who) + ": sigma and gates must be 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (validate_requested()) {
    st = check_sigma_on_device(sigma, n, s);
    if (st != SSW_OK) return st;
  }
  return run_gated(who, q, k, v, sigma, 0, 0, window, causal, gates, out, B, n, Hq, Hkv, d,
                   dtype, s, events);
}

int ssw_gated_sa_swa_forward(const void* q, const void* k, const void* v, const int32_t* sigma,
                             int window, int causal, const float* gates, void* out, int B, int n,
                             int Hq, int Hkv, int d, int dtype, void* stream) {
  return gated("ssw_gated_sa_swa_forward", q, k, v, sigma, window, causal, gates, out, B, n, Hq,
               Hkv, d, dtype, stream, nullptr);
}

int ssw_gated_sa_swa_forward_timed(const void* q, const void* k, const void* v,
                                   const int32_t* sigma, int window, int causal,
                                   const float* gates, void* out, int B, int n, int Hq, int Hkv,
                                   int d, int dtype, void* stream, void* ev_swa_start,
                                   void* ev_swa_end, void* ev_sa_start, void* ev_sa_end) {
  void* const events[4] = {ev_swa_start, ev_swa_end, ev_sa_start, ev_sa_end};
  return gated("ssw_gated_sa_swa_forward_timed", q, k, v, sigma, window, causal, gates, out, B,
               n, Hq, Hkv, d, dtype, stream, events);
}

// ---- one sigma per batch row and/or per KV head

static int check_sigma_set(const int32_t* sigma, int64_t sb, int64_t sh, int B, int n, int Hkv,
                           hipStream_t s) {
  for (int b = 0; b < (sb ? B : 1); ++b)
    for (int g = 0; g < (sh ? Hkv : 1); ++g) {
      const int st = check_sigma_on_device(sigma + b * sb + g * sh, n, s);
      if (st != SSW_OK) return st;
    }
  return SSW_OK;
}

static int forward_ex(const char* who, const void* q, const void* k, const void* v,
                      const int32_t* sigma, int64_t sb, int64_t sh, int window, int causal,
                      const float* gates, void* out, int B, int n, int Hq, int Hkv, int d,
                      int dtype, void* stream, bool gated_call) {
  int st = check_forward(who, q, k, v, out, window, causal, B, n, Hq, Hkv, d, dtype);
  if (st != SSW_OK || B == 0 || n == 0) return st;
  if (!sigma) return fail(SSW_EINVAL, std::string(who) + ": sigma must be non-NULL");
  if (gated_call && !gates) return fail(SSW_EINVAL, std::string(who) + ": gates must be non-NULL");
  if (sb < 0 || sh < 0)
    return fail(SSW_EINVAL, std::string(who) + ": sigma strides must be >= 0");
  if (!aligned(sigma, 4) || (gates && !aligned(gates, 4)))
    return fail(SSW_EALIGN, std::string(who) + ": sigma and gates must be 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (validate_requested()) {
    st = check_sigma_set(sigma, sb, sh, B, n, Hkv, s);
    if (st != SSW_OK) return st;
  }
  if (!gated_call) {
    ssw::BandLaunch a =
        make_launch(q, k, v, sigma, window, causal, gates, out, B, n, Hq, Hkv, d, dtype);
    a.sig_bstride = sb;
    a.sig_hstride = sh;
    return run(who, a, s);
  }
  return run_gated(who, q, k, v, sigma, sb, sh, window, causal, gates, out, B, n, Hq, Hkv, d,
                   dtype, s, nullptr);
}

int ssw_sa_forward_ex(const void* q, const void* k, const void* v, const int32_t* sigma,
                      int64_t sigma_batch_stride, int64_t sigma_head_stride, int window,
                      int causal, const float* gate, void* out, int B, int n, int Hq, int Hkv,
                      int d, int dtype, void* stream) {
  return forward_ex("ssw_sa_forward_ex", q, k, v, sigma, sigma_batch_stride, sigma_head_stride,
                    window, causal, gate, out, B, n, Hq, Hkv, d, dtype, stream, false);
}

int ssw_gated_sa_swa_forward_ex(const void* q, const void* k, const void* v, const int32_t* sigma,
                                int64_t sigma_batch_stride, int64_t sigma_head_stride, int window,
                                int causal, const float* gates, void* out, int B, int n, int Hq,
                                int Hkv, int d, int dtype, void* stream) {
  return forward_ex("ssw_gated_sa_swa_forward_ex", q, k, v, sigma, sigma_batch_stride,
                    sigma_head_stride, window, causal, gates, out, B, n, Hq, Hkv, d, dtype, stream,
                    true);
}

// ---- training: forward with the rows' log-sum-exp, backward, gated forward/backward

static int forward_lse(const char* who, const void* q, const void* k, const void* v,
                       const int32_t* sigma, int window, int causal, void* out, float* lse, int B,
                       int n, int Hq, int Hkv, int d, int dtype, void* stream) {
  int st = check_forward(who, q, k, v, out, window, causal, B, n, Hq, Hkv, d, dtype);
  if (st != SSW_OK || B == 0 || n == 0) return st;
  if (!lse) return fail(SSW_EINVAL, std::string(who) + ": lse must be non-NULL");
  if (!aligned(lse, 4) || (sigma && !aligned(sigma, 4)))
    return fail(SSW_EALIGN, std::string(who) + ": sigma and lse must be 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (sigma && validate_requested()) {
    st = check_sigma_on_device(sigma, n, s);
    if (st != SSW_OK) return st;
  }
  ssw::BandLaunch a =
      make_launch(q, k, v, sigma, window, causal, nullptr, out, B, n, Hq, Hkv, d, dtype);
  a.lse = lse;
  return run(who, a, s);
}

int ssw_sa_forward_lse(const void* q, const void* k, const void* v, const int32_t* sigma,
                       int window, int causal, void* out, float* lse, int B, int n, int Hq,
                       int Hkv, int d, int dtype, void* stream) {
  if (!sigma && B > 0 && n > 0) return fail(SSW_EINVAL, "ssw_sa_forward_lse: sigma must be non-NULL");
  return forward_lse("ssw_sa_forward_lse", q, k, v, sigma, window, causal, out, lse, B, n, Hq,
                     Hkv, d, dtype, stream);
}

int ssw_swa_forward_lse(const void* q, const void* k, const void* v, const int32_t* sigma,
                        int window, int causal, void* out, float* lse, int B, int n, int Hq,
                        int Hkv, int d, int dtype, void* stream) {
  if (sigma) return fail(SSW_EINVAL, "ssw_swa_forward_lse: sigma must be NULL (identity)");
  return forward_lse("ssw_swa_forward_lse", q, k, v, nullptr, window, causal, out, lse, B, n, Hq,
                     Hkv, d, dtype, stream);
}

static int check_backward(const char* who, const void* q, const void* k, const void* v,
                          const void* o, const void* dout, const float* lse, const void* dq,
                          const void* dk, const void* dv, const float* delta, int window,
                          int causal, int B, int n, int Hq, int Hkv, int d, int dtype) {
  int st = check_forward(who, q, k, v, o, window, causal, B, n, Hq, Hkv, d, dtype);
  if (st != SSW_OK) return st;
  if (dtype != SSW_BF16)
    return fail(SSW_EDTYPE, std::string(who) + ": the backward pass takes bf16 tensors only");
  if (B == 0 || n == 0) return SSW_OK;
  if (!dout || !lse || !dq || !dk || !dv || !delta)
    return fail(SSW_EINVAL, std::string(who) + ": dout, lse, dq, dk, dv and delta must be non-NULL");
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || !aligned(delta, 4))
    return fail(SSW_EALIGN, std::string(who) + ": dout, dq, dk, dv must be 16-byte aligned, lse "
                                               "and delta 4-byte aligned");
  return SSW_OK;
}

static ssw::BandBwdLaunch make_bwd(const void* q, const void* k, const void* v,
                                   const int32_t* sigma, int window, int causal, const float* gate,
                                   const void* o, const float* lse, const void* dout, void* dq,
                                   void* dk, void* dv, float* dgate, float* delta, bool accumulate,
                                   int B, int n, int Hq, int Hkv, int d) {
  ssw::BandBwdLaunch a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.gate = gate;
  a.sigma = sigma;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dgate = dgate;
  a.delta = delta;
  a.B = B;
  a.n = n;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.window = window < n ? window : n;
  a.causal = causal != 0;
  a.perm = sigma != nullptr;
  a.accumulate = accumulate;
  return a;
}

static int run_bwd(const char* who, const ssw::BandBwdLaunch& a, hipStream_t s) {
  hipError_t e = ssw::launch_band_attn_bwd(a, s);
  if (e != hipSuccess)
    return fail(SSW_EHIP, std::string(who) + ": kernel launch failed: " + hipGetErrorString(e));
  return SSW_OK;
}

static int backward(const char* who, const void* q, const void* k, const void* v,
                    const int32_t* sigma, int window, int causal, const float* gate, const void* out,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv, float* dgate,
                    float* delta, int accumulate, int B, int n, int Hq, int Hkv, int d, int dtype,
                    void* stream) {
  int st = check_backward(who, q, k, v, out, dout, lse, dq, dk, dv, delta, window, causal, B, n,
                          Hq, Hkv, d, dtype);
  if (st != SSW_OK || B == 0 || n == 0) return st;
  if (accumulate != 0 && accumulate != 1)
    return fail(SSW_EINVAL, std::string(who) + ": accumulate must be 0 or 1");
  if ((gate && !aligned(gate, 4)) || (dgate && !aligned(dgate, 4)) || (sigma && !aligned(sigma, 4)))
    return fail(SSW_EALIGN, std::string(who) + ": sigma, gate and dgate must be 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (sigma && validate_requested()) {
    st = check_sigma_on_device(sigma, n, s);
    if (st != SSW_OK) return st;
  }
  return run_bwd(who, make_bwd(q, k, v, sigma, window, causal, gate, out, lse, dout, dq, dk, dv,
                               dgate, delta, accumulate != 0, B, n, Hq, Hkv, d),
                 s);
}

int ssw_sa_backward(const void* q, const void* k, const void* v, const int32_t* sigma, int window,
                    int causal, const float* gate, const void* out, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, float* dgate, float* delta,
                    int accumulate, int B, int n, int Hq, int Hkv, int d, int dtype, void* stream) {
  if (!sigma && B > 0 && n > 0) return fail(SSW_EINVAL, "ssw_sa_backward: sigma must be non-NULL");
  return backward("ssw_sa_backward", q, k, v, sigma, window, causal, gate, out, lse, dout, dq, dk,
                  dv, dgate, delta, accumulate, B, n, Hq, Hkv, d, dtype, stream);
}

int ssw_swa_backward(const void* q, const void* k, const void* v, const int32_t* sigma,
                     int window, int causal, const float* gate, const void* out, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, float* dgate, float* delta,
                     int accumulate, int B, int n, int Hq, int Hkv, int d, int dtype,
                     void* stream) {
  if (sigma) return fail(SSW_EINVAL, "ssw_swa_backward: sigma must be NULL (identity)");
  return backward("ssw_swa_backward", q, k, v, nullptr, window, causal, gate, out, lse, dout, dq,
                  dk, dv, dgate, delta, accumulate, B, n, Hq, Hkv, d, dtype, stream);
}

int ssw_gated_sa_swa_forward_train(const void* q, const void* k, const void* v,
                                   const int32_t* sigma, int window, int causal,
                                   const float* gates, void* out, void* y_sa, float* lse_sa,
                                   void* y_swa, float* lse_swa, int B, int n, int Hq, int Hkv,
                                   int d, int dtype, void* stream) {
  const char* who = "ssw_gated_sa_swa_forward_train";
  int st = check_forward(who, q, k, v, out, window, causal, B, n, Hq, Hkv, d, dtype);
  if (st != SSW_OK) return st;
  if (dtype != SSW_BF16)
    return fail(SSW_EDTYPE, "ssw_gated_sa_swa_forward_train: bf16 tensors only");
  if (B == 0 || n == 0) return SSW_OK;
  if (!sigma || !gates || !y_sa || !lse_sa || !y_swa || !lse_swa)
    return fail(SSW_EINVAL, std::string(who) + ": sigma, gates, y_sa, lse_sa, y_swa and lse_swa "
                                               "must be non-NULL");
  if (!aligned(y_sa, 16) || !aligned(y_swa, 16) || !aligned(gates, 4) || !aligned(sigma, 4) ||
      !aligned(lse_sa, 4) || !aligned(lse_swa, 4))
    return fail(SSW_EALIGN, std::string(who) + ": y_sa and y_swa must be 16-byte aligned, sigma, "
                                               "gates and the lse buffers 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (validate_requested()) {
    st = check_sigma_on_device(sigma, n, s);
    if (st != SSW_OK) return st;
  }
  ssw::BandLaunch a1 =
      make_launch(q, k, v, nullptr, window, causal, nullptr, y_swa, B, n, Hq, Hkv, d, dtype);
  a1.lse = lse_swa;
  ssw::BandLaunch a2 =
      make_launch(q, k, v, sigma, window, causal, nullptr, y_sa, B, n, Hq, Hkv, d, dtype);
  a2.lse = lse_sa;
  if ((st = run(who, a1, s)) != SSW_OK) return st;
  if ((st = run(who, a2, s)) != SSW_OK) return st;
  hipError_t e = ssw::launch_gate_combine(y_sa, y_swa, gates, out, (int64_t)B * n * Hq, d, s);
  if (e != hipSuccess)
    return fail(SSW_EHIP, std::string(who) + ": kernel launch failed: " + hipGetErrorString(e));
  return SSW_OK;
}

// The gated layer's backward (both entry points): checks, then the SA path (writes the
// gradients) and the SWA path (adds to them); each path's Delta is consumed by its own dK/dV
// kernel before the next path overwrites it (stream order).  With delta NULL the library's own
// array is used (the entry point that allocates nothing).
static int gated_backward(const char* who, const void* q, const void* k, const void* v,
                          const int32_t* sigma, int window, int causal, const float* gates,
                          const void* y_sa, const float* lse_sa, const void* y_swa,
                          const float* lse_swa, const void* dout, void* dq, void* dk, void* dv,
                          float* dgates, float* delta, int B, int n, int Hq, int Hkv, int d,
                          int dtype, void* stream) {
  const bool own = delta == nullptr;
  if (own && B > 0 && n > 0 && (int64_t)B * n * Hq > ssw::kBwdScratchFloats)
    return fail(SSW_ESHAPE, std::string(who) + ": B * n * Hq must be <= " +
                                std::to_string(ssw::kBwdScratchFloats) +
                                " (the size of the library's Delta array)");
  // (the library's array stands in for delta in the argument checks; its device address is only
  // looked up once they have passed)
  static const float kStandIn = 0.f;
  int st = check_backward(who, q, k, v, y_sa, dout, lse_sa, dq, dk, dv, own ? &kStandIn : delta,
                          window, causal, B, n, Hq, Hkv, d, dtype);
  if (st != SSW_OK || B == 0 || n == 0) return st;
  if (!sigma || !gates || !y_swa || !lse_swa)
    return fail(SSW_EINVAL, std::string(who) + ": sigma, gates, y_swa and lse_swa must be non-NULL");
  if (!aligned(y_swa, 16) || !aligned(gates, 4) || !aligned(sigma, 4) || !aligned(lse_swa, 4) ||
      (dgates && !aligned(dgates, 4)))
    return fail(SSW_EALIGN, std::string(who) + ": y_swa must be 16-byte aligned, sigma, gates, "
                                               "lse_swa and dgates 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (validate_requested()) {
    st = check_sigma_on_device(sigma, n, s);
    if (st != SSW_OK) return st;
  }
  if (own) {
    hipError_t e = ssw::bwd_scratch_pointer(&delta);
    if (e != hipSuccess)
      return fail(SSW_EHIP, std::string(who) + ": device address of the Delta array: " +
                                hipGetErrorString(e));
  }
  const size_t plane = (size_t)B * n * Hq;
  ssw::BandBwdLaunch a1 = make_bwd(q, k, v, sigma, window, causal, gates, y_sa, lse_sa, dout, dq,
                                   dk, dv, dgates, delta, false, B, n, Hq, Hkv, d);
  ssw::BandBwdLaunch a2 =
      make_bwd(q, k, v, nullptr, window, causal, gates + plane, y_swa, lse_swa, dout, dq, dk, dv,
               dgates ? dgates + plane : nullptr, delta, true, B, n, Hq, Hkv, d);
  if ((st = run_bwd(who, a1, s)) != SSW_OK) return st;
  return run_bwd(who, a2, s);
}

int ssw_gated_sa_swa_backward(const void* q, const void* k, const void* v, const int32_t* sigma,
                              int window, int causal, const float* gates, const void* y_sa,
                              const float* lse_sa, const void* y_swa, const float* lse_swa,
                              const void* dout, void* dq, void* dk, void* dv, float* dgates,
                              float* delta, int B, int n, int Hq, int Hkv, int d, int dtype,
                              void* stream) {
  const char* who = "ssw_gated_sa_swa_backward";
  if (!delta && B > 0 && n > 0)
    return fail(SSW_EINVAL, std::string(who) + ": delta must be non-NULL");
  return gated_backward(who, q, k, v, sigma, window, causal, gates, y_sa, lse_sa, y_swa, lse_swa,
                        dout, dq, dk, dv, dgates, delta, B, n, Hq, Hkv, d, dtype, stream);
}

int ssw_gated_sa_swa_backward_noalloc(const void* q, const void* k, const void* v,
                                      const int32_t* sigma, int window, int causal,
                                      const float* gates, const void* y_sa, const float* lse_sa,
                                      const void* y_swa, const float* lse_swa, const void* dout,
                                      void* dq, void* dk, void* dv, float* dgates, int B, int n,
                                      int Hq, int Hkv, int d, int dtype, void* stream) {
  return gated_backward("ssw_gated_sa_swa_backward_noalloc", q, k, v, sigma, window, causal, gates,
                        y_sa, lse_sa, y_swa, lse_swa, dout, dq, dk, dv, dgates, nullptr, B, n, Hq,
                        Hkv, d, dtype, stream);
}

// ---- decode: one new token per batch row over a KV cache

static int decode(const char* who, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* sigma, const int32_t* inv_sigma, const int32_t* pos, int window,
                  const float* gate, void* out, int B, int n_max, int Hq, int Hkv, int d,
                  int dtype, void* stream, int paths) {
  const std::string w(who);
  if (B < 0 || n_max < 1) return fail(SSW_EINVAL, w + ": need B >= 0 and n_max >= 1");
  if (window < 1) return fail(SSW_EINVAL, w + ": window must be >= 1");
  if (Hq < 1 || Hkv < 1) return fail(SSW_EINVAL, w + ": Hq and Hkv must be >= 1");
  if (Hq % Hkv != 0) return fail(SSW_ESHAPE, w + ": Hq must be a multiple of Hkv");
  if (Hq / Hkv > 8) return fail(SSW_ESHAPE, w + ": at most 8 query heads per KV head");
  if ((int64_t)B * Hkv >= ((int64_t)1 << 31)) return fail(SSW_ESHAPE, w + ": B * Hkv too large");
  if (dtype != SSW_F32 && dtype != SSW_BF16) return fail(SSW_EDTYPE, w + ": unsupported dtype");
  if (d != 64 && d != 128) return fail(SSW_EDTYPE, w + ": head dim d must be 64 or 128");
  if (B == 0) return SSW_OK;
  if (!q || !k_cache || !v_cache || !pos || !out)
    return fail(SSW_EINVAL, w + ": q, k_cache, v_cache, pos and out must be non-NULL");
  if ((paths & 1) && (!sigma || !inv_sigma))
    return fail(SSW_EINVAL, w + ": sigma and inv_sigma must be non-NULL");
  if (paths == 3 && !gate) return fail(SSW_EINVAL, w + ": gates must be non-NULL");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return fail(SSW_EALIGN, w + ": q, k_cache, v_cache and out must be 16-byte aligned");
  if (!aligned(pos, 4) || (sigma && !aligned(sigma, 4)) || (inv_sigma && !aligned(inv_sigma, 4)) ||
      (gate && !aligned(gate, 4)))
    return fail(SSW_EALIGN, w + ": pos, sigma, inv_sigma and gate must be 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if ((paths & 1) && validate_requested()) {
    int st = check_sigma_on_device(sigma, n_max, s);
    if (st != SSW_OK) return st;
  }
  ssw::DecodeLaunch a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.sigma = sigma;
  a.inv_sigma = inv_sigma;
  a.pos = pos;
  a.gate = gate;
  a.out = out;
  a.B = B;
  a.n_max = n_max;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.dtype = dtype;
  a.window = window < n_max ? window : n_max;
  a.paths = paths;
  hipError_t e = ssw::launch_decode(a, s);
  if (e != hipSuccess) return fail(SSW_EHIP, w + ": kernel launch failed: " + hipGetErrorString(e));
  return SSW_OK;
}

int ssw_sa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* sigma,
                  const int32_t* inv_sigma, const int32_t* pos, int window, const float* gate,
                  void* out, int B, int n_max, int Hq, int Hkv, int d, int dtype, void* stream) {
  return decode("ssw_sa_decode", q, k_cache, v_cache, sigma, inv_sigma, pos, window, gate, out, B,
                n_max, Hq, Hkv, d, dtype, stream, 1);
}

int ssw_swa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* sigma,
                   const int32_t* inv_sigma, const int32_t* pos, int window, const float* gate,
                   void* out, int B, int n_max, int Hq, int Hkv, int d, int dtype, void* stream) {
  if (sigma || inv_sigma)
    return fail(SSW_EINVAL, "ssw_swa_decode: sigma and inv_sigma must be NULL (identity)");
  return decode("ssw_swa_decode", q, k_cache, v_cache, nullptr, nullptr, pos, window, gate, out,
                B, n_max, Hq, Hkv, d, dtype, stream, 2);
}

int ssw_gated_sa_swa_decode(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* sigma, const int32_t* inv_sigma, const int32_t* pos,
                            int window, const float* gates, void* out, int B, int n_max, int Hq,
                            int Hkv, int d, int dtype, void* stream) {
  return decode("ssw_gated_sa_swa_decode", q, k_cache, v_cache, sigma, inv_sigma, pos, window,
                gates, out, B, n_max, Hq, Hkv, d, dtype, stream, 3);
}

// ---- gate projections of the gated layer

int ssw_gate_projection(const void* x, const void* w_t, const float* bias, float* gates, int rows,
                        int Hm, int Hq, int dtype, void* stream) {
  const char* who = "ssw_gate_projection";
  if (rows < 0 || Hm < 1 || Hq < 1)
    return fail(SSW_EINVAL, std::string(who) + ": need rows >= 0, Hm >= 1 and Hq >= 1");
  if (dtype != SSW_BF16) return fail(SSW_EDTYPE, std::string(who) + ": bf16 x and w_t only");
  if (Hm % 16 != 0 || Hq > 64)
    return fail(SSW_ESHAPE, std::string(who) + ": Hm must be a multiple of 16 and Hq <= 64");
  if ((int64_t)rows * Hm * 2 > ((int64_t)1 << 40))
    return fail(SSW_ESHAPE, std::string(who) + ": x too large");
  if (rows == 0) return SSW_OK;
  if (!x || !w_t || !gates)
    return fail(SSW_EINVAL, std::string(who) + ": x, w_t and gates must be non-NULL");
  if (!aligned(x, 16) || !aligned(w_t, 16) || !aligned(gates, 4) || (bias && !aligned(bias, 4)))
    return fail(SSW_EALIGN, std::string(who) + ": x and w_t must be 16-byte aligned, gates and "
                                               "bias 4-byte aligned");
  hipError_t e = ssw::launch_gate_projection(x, w_t, bias, gates, rows, Hm, Hq,
                                             (hipStream_t)stream);
  if (e != hipSuccess)
    return fail(SSW_EHIP, std::string(who) + ": kernel launch failed: " + hipGetErrorString(e));
  return SSW_OK;
}

int ssw_make_permutation(uint64_t seed, int n, int32_t* sigma_out, int32_t* inv_out) {
  if (n < 0) return fail(SSW_EINVAL, "ssw_make_permutation: n must be >= 0");
  if (n > 0 && !sigma_out) return fail(SSW_EINVAL, "ssw_make_permutation: sigma_out is NULL");
  for (int i = 0; i < n; ++i) sigma_out[i] = i;
  SplitMix64 rng{seed};
  for (int i = n - 1; i >= 1; --i) {
    // Lemire's multiply-high map of a 64-bit draw onto [0, i]
    const unsigned __int128 prod = (unsigned __int128)rng.next() * (unsigned __int128)(i + 1);
    const int j = (int)(uint64_t)(prod >> 64);
    const int32_t t = sigma_out[i];
    sigma_out[i] = sigma_out[j];
    sigma_out[j] = t;
  }
  if (inv_out)
    for (int p = 0; p < n; ++p) inv_out[sigma_out[p]] = p;
  return SSW_OK;
}

int ssw_check_permutation(const int32_t* sigma, int n) {
  if (n < 0) return fail(SSW_EINVAL, "ssw_check_permutation: n must be >= 0");
  if (n == 0) return SSW_OK;
  if (!sigma) return fail(SSW_EINVAL, "ssw_check_permutation: sigma is NULL");
  std::vector<uint8_t> seen((size_t)n, 0);
  for (int p = 0; p < n; ++p) {
    const int32_t s = sigma[p];
    if (s < 0 || s >= n || seen[(size_t)s])
      return fail(SSW_ENOTPERM, "sigma is not a permutation of [0, n)");
    seen[(size_t)s] = 1;
  }
  return SSW_OK;
}

int ssw_inverse_permutation(const int32_t* sigma, int n, int32_t* inv_out) {
  const int st = ssw_check_permutation(sigma, n);
  if (st != SSW_OK) return st;
  if (n > 0 && !inv_out) return fail(SSW_EINVAL, "ssw_inverse_permutation: inv_out is NULL");
  for (int p = 0; p < n; ++p) inv_out[sigma[p]] = p;
  return SSW_OK;
}

int ssw_neighbor_mask(const int32_t* sigma, int n, int window, int causal, uint32_t* bits,
                      void* stream) {
  if (n < 0 || window < 1 || (causal != 0 && causal != 1))
    return fail(SSW_EINVAL, "ssw_neighbor_mask: need n >= 0, window >= 1, causal in {0, 1}");
  if (n > 65536) return fail(SSW_ESHAPE, "ssw_neighbor_mask: n must be <= 65536");
  if (n == 0) return SSW_OK;
  if (!bits) return fail(SSW_EINVAL, "ssw_neighbor_mask: bits is NULL");
  if (!aligned(bits, 4) || (sigma && !aligned(sigma, 4)))
    return fail(SSW_EALIGN, "ssw_neighbor_mask: sigma and bits must be 4-byte aligned");
  const int w = window < n ? window : n;
  hipError_t e = ssw::launch_neighbor_mask(sigma, n, w, causal != 0, bits, (hipStream_t)stream);
  if (e != hipSuccess)
    return fail(SSW_EHIP, std::string("ssw_neighbor_mask: launch failed: ") + hipGetErrorString(e));
  return SSW_OK;
}

// Receptive-field growth of SA / SWA / gated layers ([SA-ja] 理論的性質, 受容野の成長).
// R_0(i) = {i}; R_l(i) = union of R_{l-1}(j) over the neighbours j of i at layer l (the
// attention kernels' neighbour sets); coverage = sum |R_l(i)| / (number of pairs j <= i when
// causal, n^2 otherwise).  Bit rows of n bits, double-buffered; in causal mode row i only has
// bits <= i, so only its first i / 64 + 1 words are touched.
int ssw_receptive_field_coverage(int n, int window, int layers, const uint64_t* seeds, int mode,
                                 int causal, double* coverage_out) {
  if (n < 1 || n > 32768 || window < 1 || layers < 0 || mode < 0 || mode > 2 ||
      (causal != 0 && causal != 1))
    return fail(SSW_EINVAL, "ssw_receptive_field_coverage: need 1 <= n <= 32768, window >= 1, "
                            "layers >= 0, mode 0 (SA), 1 (SWA) or 2 (gated), causal 0 or 1");
  if (layers > 0 && (!coverage_out || (mode != 1 && !seeds)))
    return fail(SSW_EINVAL, "ssw_receptive_field_coverage: seeds and coverage_out are required");
  const size_t words = ((size_t)n + 63) / 64;
  std::vector<uint64_t> cur((size_t)n * words, 0), nxt((size_t)n * words, 0);
  for (int i = 0; i < n; ++i) cur[(size_t)i * words + i / 64] = 1ull << (i % 64);
  std::vector<int32_t> sigma((size_t)n), inv((size_t)n);
  const int w = window < n ? window : n;
  const double total = causal ? (double)n * (n + 1) / 2.0 : (double)n * n;
  for (int l = 0; l < layers; ++l) {
    if (mode != 1) ssw_make_permutation(seeds[l], n, sigma.data(), inv.data());
    std::fill(nxt.begin(), nxt.end(), 0ull);
    for (int i = 0; i < n; ++i) {
      uint64_t* dst = &nxt[(size_t)i * words];
      const size_t used = causal ? (size_t)i / 64 + 1 : words;
      auto merge = [&](int j) {
        const uint64_t* src = &cur[(size_t)j * words];
        for (size_t k = 0; k < used; ++k) dst[k] |= src[k];
      };
      if (mode != 1) {  // SA: slots within w - 1 of sigma^-1(i) (holding tokens <= i if causal)
        const int p = inv[(size_t)i];
        const int lo = p - (w - 1) > 0 ? p - (w - 1) : 0;
        const int hi = p + (w - 1) < n - 1 ? p + (w - 1) : n - 1;
        for (int q = lo; q <= hi; ++q)
          if (!causal || sigma[(size_t)q] <= i) merge(sigma[(size_t)q]);
      }
      if (mode != 0) {  // SWA: [i - w + 1, i], or |i - j| <= w - 1
        const int hi = causal ? i : (i + (w - 1) < n - 1 ? i + (w - 1) : n - 1);
        for (int j = i - (w - 1) > 0 ? i - (w - 1) : 0; j <= hi; ++j) merge(j);
      }
    }
    cur.swap(nxt);
    uint64_t bits = 0;
    for (uint64_t x : cur) bits += (uint64_t)__builtin_popcountll(x);
    coverage_out[l] = (double)bits / total;
  }
  return SSW_OK;
}

const char* ssw_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
