// One decode step of SA / SWA / the gated layer over a KV cache, on gfx950.
//
// What is computed.  The token at position t of batch row b is row t of causal SA over the
// full context n_max ([SA-ja] "技術的概要：確率的アテンション", 中核メカニズム steps 1-3 and
// 理論的性質 › 因果的制約): with one sigma per layer over n_max and p = sigma^-1(t), it attends
// to the cached tokens sigma[q] for slots |q - p| <= w - 1 with sigma[q] <= t.  The SWA step
// attends to positions [t - w + 1, t] ([HYB] ハイブリッドアーキテクチャの定義).  The gated step
// returns g_sa * SA + g_swa * SWA ([SA-ja] ゲート付き SA と SWA の組み合わせ).
//
// Mapping onto the chip.  One workgroup per (batch row, KV head): the G query heads of the KV
// head share every gathered key.  A step reads at most 2w - 1 (SA) plus w (SWA) K/V rows from
// random cache positions, so it is bound by those row reads; it runs on the vector ALUs rather
// than the matrix cores, which a handful of query rows would leave nearly idle.
//   * Candidates are taken 64 at a time, the SA path's chunks then the SWA path's as one
//     sequence: their cache rows are gathered through sigma by all 256 threads (a masked
//     candidate is redirected to row t, which is always valid, so no uninitialised cache row is
//     ever read).  The rows of chunk c + 1 are loaded into registers, and the tokens of chunk
//     c + 2 looked up, while chunk c is scored from LDS.
//   * Wave v handles query heads v, v + 4, ...; for each, lane j scores candidate j against the
//     head's query (held in LDS, read as a broadcast), the wave does the online-softmax max and
//     sum, and lane l accumulates output elements d = kDPL * l .. kDPL * l + kDPL - 1 over the
//     64 candidates, each candidate's weight broadcast from its lane by v_readlane.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "band_attn.h"

namespace ssw {
namespace dec {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kCand = 64;       // candidates per chunk, one per lane
constexpr int kMaxG = 8;        // query heads per KV head (checked at the API)
constexpr int kMaxHW = kMaxG / kWaves;

struct Params {
  const char* q;
  const char* kc;
  const char* vc;
  const int32_t* sigma;
  const int32_t* inv;
  const int32_t* pos;
  const float* gate;  // single path: [B, Hq] or nullptr; gated: [2, B, Hq]
  char* out;
  int B, n, Hq, Hkv, G, L;
  float scale_log2;
  int paths;          // bit 0: SA, bit 1: SWA
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <typename T>
__device__ __forceinline__ float to_f(T x) {
  return (float)x;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void decode_kernel(Params prm) {
  constexpr int kRowBytes = D * (int)sizeof(T);
  constexpr int kGran = kRowBytes / 16;  // 16-byte granules per row
  constexpr int kDPL = D / 64;           // output elements per lane
  constexpr int kElPerGran = 16 / (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) char k_lds[kCand * kRowBytes];
  __shared__ __attribute__((aligned(16))) char v_lds[kCand * kRowBytes];
  __shared__ __attribute__((aligned(16))) float q_lds[kMaxG * D];
  __shared__ int tok_lds[2][kCand];  // chunk c's tokens in slot c % 2
  __shared__ int ok_lds[2][kCand];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.x / prm.Hkv;
  const int g = blockIdx.x - b * prm.Hkv;
  const int n = prm.n;
  const int G = prm.G;
  const int L = prm.L;
  const int t = prm.pos[b];
  const bool t_ok = t >= 0 && t < n;
  const int tc = t_ok ? t : 0;

  // ---- the G query rows of this KV head, as fp32, in LDS
  const char* qbase = prm.q + ((int64_t)b * prm.Hq + g * G) * kRowBytes;
  for (int e = tid; e < G * D; e += kThreads) q_lds[e] = to_f(((const T*)qbase)[e]);

  const int nh = (G - wave + kWaves - 1) / kWaves;  // heads of this wave
  float y[kMaxHW][kDPL];
#pragma unroll
  for (int i = 0; i < kMaxHW; ++i)
#pragma unroll
    for (int e = 0; e < kDPL; ++e) y[i][e] = 0.f;

  const char* kcb = prm.kc + (int64_t)b * n * prm.Hkv * kRowBytes + (int64_t)g * kRowBytes;
  const char* vcb = prm.vc + (int64_t)b * n * prm.Hkv * kRowBytes + (int64_t)g * kRowBytes;
  const int64_t row_stride = (int64_t)prm.Hkv * kRowBytes;

  // ---- the candidate chunks of both paths as one sequence: SA slots [p - L, p + L] first
  // (chunks [0, nA)), then SWA positions [t - L, t] (chunks [nA, nA + nB))
  const bool do_sa = prm.paths & 1;
  // (an entry of a malformed inverse outside [0, n) is taken as slot 0: wrong, but in bounds)
  const int p_raw = do_sa ? prm.inv[tc] : 0;
  const int p_sa = (uint32_t)p_raw < (uint32_t)n ? p_raw : 0;
  const int lo_sa = max(0, p_sa - L);
  const int hi_sa = min(n - 1, p_sa + L);
  const int nA = do_sa ? (hi_sa - lo_sa) / kCand + 1 : 0;
  const int lo_w = max(0, tc - L);
  const int nB = (prm.paths & 2) ? (tc - lo_w) / kCand + 1 : 0;
  const int total = nA + nB;
  // token and validity of candidate j of chunk c (masked candidates read row t, always valid)
  auto cand = [&](int c, int j, int& tok) {
    bool ok;
    if (c < nA) {
      const int q = lo_sa + c * kCand + j;
      ok = q <= hi_sa;
      tok = ok ? prm.sigma[q] : tc;
      // unsigned: an entry of a malformed sigma below 0 is masked too, and never read
      ok = ok && (uint32_t)tok <= (uint32_t)tc;
    } else {
      const int q = lo_w + (c - nA) * kCand + j;
      ok = q <= tc;
      tok = q;
    }
    if (!ok) tok = tc;
    return ok;
  };

  // rows of the next chunk, staged in registers while the current one is scored
  constexpr int kPer = kCand * kGran / kThreads;  // granules per thread per matrix
  static_assert(kPer >= 1 && kPer * kThreads == kCand * kGran, "row split");
  u32x4 kreg[kPer], vreg[kPer];
  auto load_rows = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int gi = i * kThreads + tid;
      const int r = gi / kGran;
      const int gr = gi - r * kGran;
      const int64_t off = (int64_t)tok_lds[buf][r] * row_stride + gr * 16;
      kreg[i] = *(const u32x4*)(kcb + off);
      vreg[i] = *(const u32x4*)(vcb + off);
    }
  };
  auto store_rows = [&]() {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int gi = i * kThreads + tid;
      const int r = gi / kGran;
      const int gr = gi - r * kGran;
      // K rows swizzled by granule (lane j reads row j), V rows natural
      *(u32x4*)(k_lds + r * kRowBytes + ((gr ^ (r & (kGran - 1))) << 4)) = kreg[i];
      *(u32x4*)(v_lds + r * kRowBytes + gr * 16) = vreg[i];
    }
  };

  float m[kMaxHW], l[kMaxHW], acc[kMaxHW][kDPL];
  auto reset = [&]() {
#pragma unroll
    for (int i = 0; i < kMaxHW; ++i) {
      m[i] = -INFINITY;
      l[i] = 0.f;
#pragma unroll
      for (int e = 0; e < kDPL; ++e) acc[i][e] = 0.f;
    }
  };
  // fold a finished path into the output: y += gate * acc / l
  auto fold = [&](int path) {
#pragma unroll
    for (int i = 0; i < kMaxHW; ++i) {
      if (i >= nh) break;
      const int h = g * G + wave + kWaves * i;
      float gv = 1.f;
      if (prm.paths == 3)
        gv = prm.gate[(int64_t)path * prm.B * prm.Hq + (int64_t)b * prm.Hq + h];
      else if (prm.gate)
        gv = prm.gate[(int64_t)b * prm.Hq + h];
      const float f = gv / l[i];
#pragma unroll
      for (int e = 0; e < kDPL; ++e) y[i][e] = __builtin_fmaf(acc[i][e], f, y[i][e]);
    }
  };
  reset();

  // ---- prologue: chunk 0's tokens, chunk 1's tokens in registers, chunk 0's rows in registers
  int tok_next = tc;
  bool ok_next = false;
  if (tid < kCand) {
    int tk;
    const bool ok = cand(0, tid, tk);
    tok_lds[0][tid] = tk;
    ok_lds[0][tid] = ok;
    if (1 < total) ok_next = cand(1, tid, tok_next);
  }
  __syncthreads();
  load_rows(0);

  for (int c = 0; c < total; ++c) {
    const int cur = c & 1;
    const int nxt = cur ^ 1;
    __syncthreads();  // chunk c - 1 is scored: its rows and chunk c + 1's token slot are free
    store_rows();
    if (tid < kCand && c + 1 < total) {
      tok_lds[nxt][tid] = tok_next;
      ok_lds[nxt][tid] = ok_next;
      if (c + 2 < total) ok_next = cand(c + 2, tid, tok_next);
    }
    __syncthreads();
    if (c + 1 < total) load_rows(nxt);  // in flight while chunk c is scored

    const bool ok = ok_lds[cur][lane] != 0;
#pragma unroll
    for (int i = 0; i < kMaxHW; ++i) {
      if (i >= nh) break;
      const int hh = wave + kWaves * i;
      const float* qh = q_lds + hh * D;
      // score of candidate `lane`
      float s = 0.f;
#pragma unroll
      for (int gr = 0; gr < kGran; ++gr) {
        const u32x4 kw = *(const u32x4*)(k_lds + lane * kRowBytes +
                                         ((gr ^ (lane & (kGran - 1))) << 4));
#pragma unroll
        for (int e = 0; e < kElPerGran; ++e) {
          float kv;
          if constexpr (sizeof(T) == 2) {
            const uint32_t wd = kw[e >> 1];
            kv = __uint_as_float((e & 1) ? (wd & 0xffff0000u) : (wd << 16));
          } else {
            kv = __uint_as_float(kw[e]);
          }
          s = __builtin_fmaf(qh[gr * kElPerGran + e], kv, s);
        }
      }
      s = ok ? s * prm.scale_log2 : -INFINITY;
      const float mx = wave_max(s);
      const float m_new = fmaxf(m[i], mx);
      // the candidate at row t itself is always present, so m_new is finite after its chunk;
      // before that, with every candidate so far masked, nothing is accumulated
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[i] - m_new);
      const float pj = ok ? __builtin_amdgcn_exp2f(s - m_new) : 0.f;
      m[i] = m_new;
      l[i] = l[i] * alpha + wave_sum(pj);
#pragma unroll
      for (int e = 0; e < kDPL; ++e) acc[i][e] *= alpha;
      // candidate j's weight is broadcast from lane j (v_readlane into a scalar register)
#pragma unroll 8
      for (int j = 0; j < kCand; ++j) {
        const float pw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), j));
        if constexpr (sizeof(T) == 2) {
          if constexpr (kDPL == 2) {
            const uint32_t wd = *(const uint32_t*)(v_lds + j * kRowBytes + 4 * lane);
            acc[i][0] = __builtin_fmaf(pw, __uint_as_float(wd << 16), acc[i][0]);
            acc[i][1] = __builtin_fmaf(pw, __uint_as_float(wd & 0xffff0000u), acc[i][1]);
          } else {
            const uint32_t hw = *(const uint16_t*)(v_lds + j * kRowBytes + 2 * lane);
            acc[i][0] = __builtin_fmaf(pw, __uint_as_float(hw << 16), acc[i][0]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < kDPL; ++e)
            acc[i][e] = __builtin_fmaf(
                pw, *(const float*)(v_lds + j * kRowBytes + 4 * (kDPL * lane + e)), acc[i][e]);
        }
      }
    }
    if (c == nA - 1 || c == total - 1) {  // a path ends with this chunk
      fold(c < nA ? 0 : 1);
      reset();
    }
  }

  // ---- store; a position outside [0, n_max) gives NaN rows
#pragma unroll
  for (int i = 0; i < kMaxHW; ++i) {
    if (i >= nh) break;
    const int h = g * G + wave + kWaves * i;
    char* orow = prm.out + ((int64_t)b * prm.Hq + h) * kRowBytes;
#pragma unroll
    for (int e = 0; e < kDPL; ++e) {
      const float v = t_ok ? y[i][e] : __builtin_nanf("");
      if constexpr (sizeof(T) == 2)
        ((__bf16*)orow)[kDPL * lane + e] = (__bf16)v;
      else
        ((float*)orow)[kDPL * lane + e] = v;
    }
  }
}

}  // namespace dec

hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream) {
  dec::Params prm;
  prm.q = (const char*)a.q;
  prm.kc = (const char*)a.k_cache;
  prm.vc = (const char*)a.v_cache;
  prm.sigma = a.sigma;
  prm.inv = a.inv_sigma;
  prm.pos = a.pos;
  prm.gate = a.gate;
  prm.out = (char*)a.out;
  prm.B = a.B;
  prm.n = a.n_max;
  prm.Hq = a.Hq;
  prm.Hkv = a.Hkv;
  prm.G = a.Hq / a.Hkv;
  prm.L = a.window - 1;
  prm.scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)a.d));
  prm.paths = a.paths;
  const dim3 grid((unsigned)(a.B * a.Hkv));
  if (a.dtype == 1) {
    if (a.d == 128)
      hipLaunchKernelGGL((dec::decode_kernel<__bf16, 128>), grid, dim3(dec::kThreads), 0, stream, prm);
    else
      hipLaunchKernelGGL((dec::decode_kernel<__bf16, 64>), grid, dim3(dec::kThreads), 0, stream, prm);
  } else {
    if (a.d == 128)
      hipLaunchKernelGGL((dec::decode_kernel<float, 128>), grid, dim3(dec::kThreads), 0, stream, prm);
    else
      hipLaunchKernelGGL((dec::decode_kernel<float, 64>), grid, dim3(dec::kThreads), 0, stream, prm);
  }
  return hipGetLastError();
}

}  // namespace ssw
