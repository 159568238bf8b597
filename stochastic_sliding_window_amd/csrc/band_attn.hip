// Band attention on gfx950: the kernel behind Stochastic Attention (SA), plain SWA and both
// passes of the gated SA+SWA layer.
//
// What is computed ([SA-ja] "技術的概要：確率的アテンション", 手法 › 中核メカニズム steps 1-3 and
// 理論的性質 › 因果的制約; [HYB] ハイブリッドアーキテクチャの定義 for SWA): the query at permuted
// slot p (original token sigma[p]) attends to the keys at slots q with |p - q| <= w - 1 (keys
// left of the band edge and past the sequence end are dropped); in causal mode a key is kept only
// if sigma[q] <= sigma[p].  With sigma = identity the causal band collapses to [p - w + 1, p],
// which this kernel exploits by taking the right band extent R = 0.  The output row of slot p is
// written at original position sigma[p], optionally times a gate, optionally added to what is
// there.
//
// Mapping onto the chip.
//   * One workgroup = 8 waves = one KV head of one batch row and 256 consecutive "columns",
//     where a column is a (permuted slot, query head of the KV group) pair: column c is slot
//     c / G, head c % G (G = Hq / Hkv).  So the G query heads sharing a KV head sit side by side
//     and each K/V row staged in LDS serves all of them.
//   * Each wave owns 32 columns and computes S^T = K_chunk * Q^T with 32x32 MFMAs (rows = keys,
//     columns = the wave's 32 columns), so every lane holds whole columns: the softmax row
//     statistics of a column live in two lanes (lane l and l ^ 32) and need one cross-lane step.
//   * Keys stream through LDS in chunks of 32, double-buffered: K rows are gathered through sigma
//     straight from HBM (no permuted copy is ever written), stored in MFMA row order; V is stored
//     transposed (bf16) so the P*V MFMA reads 8 consecutive keys per lane.
//   * The MFMA row -> key map is chosen so that the registers holding P^T after the softmax are
//     already the B operand of the next MFMA (no register shuffles between the two products).
//   * Softmax is online with a lazy reference maximum (rescale only when the running max grows
//     by more than 2^8), and masks are evaluated per element only where a chunk touches the band
//     edge or when the causal rule needs sigma.
//   * Epilogue: divide by the row sum, multiply by the gate, scatter to row sigma[p] (store, or
//     read-add-store for the second gated pass).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "band_attn.h"

namespace ssw {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
#ifndef SSW_WAVES
#define SSW_WAVES 8
#endif
#ifndef SSW_XCD_REMAP
#define SSW_XCD_REMAP 1
#endif
constexpr int kWaves = SSW_WAVES;  // waves per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr int kColsWave = 32;
constexpr int kColsWG = kColsWave * kWaves;
constexpr int kChunk = 32;
constexpr float kLazy = 8.0f;  // reference max may lag the true max by up to 2^8 (log2 units)
// bf16 gated path: the SWA pass leaves g_swa * Y_swa in the output buffer as fp16 scaled by 2^-8
constexpr float kPartialScale = 1.0f / 256.0f;
constexpr float kPartialUnscale = 256.0f;

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Key membership in permuted-slot space.  The attention kernel and the neighbour-mask kernel use
// this same test.
__device__ __forceinline__ bool band_member(int p, int q, int n, int L, int R) {
  return q >= p - L && q <= p + R && q >= 0 && q < n;
}

// MFMA 32x32 output row r holds key rho(r) of the chunk; this is the inverse map (key -> row).
// rho(8a + 4h + b) = 16(a / 2) + 8h + 4(a % 2) + b makes lane half h's registers 0..7 hold keys
// 8h..8h+7 and registers 8..15 hold keys 16+8h..16+8h+7.
__device__ __forceinline__ int key_to_row(int key) {
  return 8 * (2 * (key >> 4) + ((key >> 2) & 1)) + 4 * ((key >> 3) & 1) + (key & 3);
}

template <typename T, int D>
struct Layout {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int kRowBytes = D * (int)sizeof(T);
  static constexpr int kSegs = kRowBytes / 16;                     // 16-byte pieces per row
  static constexpr int kPieces = kChunk * kSegs;                   // pieces per K (or V) chunk
  static constexpr int kPPT = (kPieces + kThreads - 1) / kThreads;  // pieces per thread
  static constexpr int kKRow = kRowBytes + 16;                     // padded K row (bytes)
  static constexpr int kKBytes = kChunk * kKRow;
  // bf16: V^T [D][32 keys] rows padded to 80 B; fp32: V [32 keys][D] rows padded by 16 B
  static constexpr int kVRow = kBf16 ? (kChunk * 2 + 16) : (kRowBytes + 16);
  static constexpr int kVBytes = kBf16 ? D * kVRow : kChunk * kVRow;
  static constexpr int kSigOff = kKBytes + kVBytes;
  static constexpr int kStage = kSigOff + kChunk * 4;
  static_assert(kPieces % kWave == 0, "staging assumes whole waves");
  static_assert(kStage % 16 == 0, "stage alignment");
};

struct Params {
  const char* q;
  const char* k;
  const char* v;
  const int32_t* sigma;
  const float* gate;
  char* out;
  int B, n, Hq, Hkv, G;
  int L, R;          // band: key slots [p - L, p + R]
  float scale_log2;  // log2(e) / sqrt(d)
  int ntiles;        // column tiles per (batch row, KV head)
  int nblocks;       // ntiles * B * Hkv
};

// The dispatcher hands consecutive workgroup ids to the 8 XCDs in turn, and each XCD has its own
// L2.  Neighbouring column tiles of one (batch row, KV head) share most of their K/V band, so the
// ids are renumbered to give every XCD a contiguous run of tiles: id i runs tile-major position
// (i % 8) * (N / 8) + i / 8 (a bijection on the first 8 * floor(N / 8) ids; the rest keep theirs).
__device__ __forceinline__ int xcd_local_order(int i, int nblocks) {
#if SSW_XCD_REMAP
  const int per = nblocks / 8;
  if (i < per * 8) return (i % 8) * per + i / 8;
#endif
  return i;
}

template <typename T, int D, bool PERM, bool SIGMASK, int EPI>
__global__ __launch_bounds__(kThreads) void band_attn_kernel(Params prm) {
  using Lay = Layout<T, D>;
  constexpr bool kBf16 = Lay::kBf16;
  __shared__ __attribute__((aligned(16))) char smem[2 * Lay::kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h32 = lane >> 5;  // lane half
  const int n = prm.n;
  const int G = prm.G;
  const int L = prm.L;
  const int R = prm.R;
  const int nG = n * G;

  const int blk = xcd_local_order(blockIdx.x, prm.nblocks);
  const int tile = blk % prm.ntiles;
  const int bg = blk / prm.ntiles;
  const int b = bg / prm.Hkv;
  const int g = bg - b * prm.Hkv;

  // ---- columns of this workgroup / wave / lane
  const int col0_wg = tile * kColsWG;
  const int col0_w = col0_wg + wave * kColsWave;
  const int mycol = col0_w + (lane & 31);
  const bool colvalid = mycol < nG;
  const int mycol_c = colvalid ? mycol : nG - 1;
  const int myslot = mycol_c / G;
  const int h = g * G + (mycol_c - myslot * G);
  const int myorig = PERM ? prm.sigma[myslot] : myslot;

  const bool wave_on = col0_w < nG;
  const int w_slo = col0_w / G;
  const int w_shi = min(col0_w + kColsWave - 1, nG - 1) / G;
  const int S_lo = col0_wg / G;
  const int S_hi = min(col0_wg + kColsWG - 1, nG - 1) / G;
  const int kbeg = max(0, S_lo - L);
  const int kend = min(n - 1, S_hi + R);
  const int nchunks = (kend - kbeg) / kChunk + 1;
  const int c_first = (max(0, w_slo - L) - kbeg) / kChunk;
  const int c_last = (min(n - 1, w_shi + R) - kbeg) / kChunk;

  // ---- Q fragment (B operand of S^T = K Q^T), kept in registers for the whole sweep
  const int64_t qrow_elems = (((int64_t)b * n + myorig) * prm.Hq + h) * D;
  constexpr int kQRegs = kBf16 ? D / 16 : D / 2;
  typedef typename std::conditional<kBf16, bf16x8, float>::type QFrag;
  QFrag qf[kQRegs];
  if constexpr (kBf16) {
    const char* qp = prm.q + (qrow_elems + 8 * h32) * 2;
#pragma unroll
    for (int kb = 0; kb < kQRegs; ++kb) {
      u32x4 raw = colvalid ? *(const u32x4*)(qp + kb * 32) : u32x4{0, 0, 0, 0};
      qf[kb] = __builtin_bit_cast(bf16x8, raw);
    }
  } else {
    const char* qp = prm.q + (qrow_elems + h32 * (D / 2)) * 4;
#pragma unroll
    for (int t4 = 0; t4 < D / 8; ++t4) {
      f32x4 v4 = colvalid ? *(const f32x4*)(qp + t4 * 16) : f32x4{0, 0, 0, 0};
      qf[4 * t4 + 0] = v4[0];
      qf[4 * t4 + 1] = v4[1];
      qf[4 * t4 + 2] = v4[2];
      qf[4 * t4 + 3] = v4[3];
    }
  }

  // ---- staging helpers: thread tid stages key r = tid & 31 (same r for all its pieces)
  const int st_r = tid & 31;
  const int64_t kv_row_stride = (int64_t)prm.Hkv * Lay::kRowBytes;
  const char* kbase = prm.k + ((int64_t)b * n * prm.Hkv + g) * Lay::kRowBytes;
  const char* vbase = prm.v + ((int64_t)b * n * prm.Hkv + g) * Lay::kRowBytes;

  auto load_sig = [&](int kc0) -> int {
    const int key = kc0 + st_r;
    if (key >= n) return -1;
    return PERM ? prm.sigma[key] : key;
  };

  u32x4 kreg[Lay::kPPT];
  u32x4 vreg[Lay::kPPT];
  auto load_kv = [&](int srcrow) {
#pragma unroll
    for (int j = 0; j < Lay::kPPT; ++j) {
      const int i = tid + j * kThreads;
      kreg[j] = u32x4{0, 0, 0, 0};
      vreg[j] = u32x4{0, 0, 0, 0};
      if (i < Lay::kPieces && srcrow >= 0) {
        const int seg = i >> 5;
        const int64_t off = (int64_t)srcrow * kv_row_stride + seg * 16;
        kreg[j] = *(const u32x4*)(kbase + off);
        vreg[j] = *(const u32x4*)(vbase + off);
      }
    }
  };

  auto store_stage = [&](int stage, int srcrow) {
    char* st = smem + stage * Lay::kStage;
    char* Kst = st;
    char* Vst = st + Lay::kKBytes;
    int* Sst = (int*)(st + Lay::kSigOff);
#pragma unroll
    for (int j = 0; j < Lay::kPPT; ++j) {
      const int i = tid + j * kThreads;
      if (i < Lay::kPieces) {
        const int seg = i >> 5;
        *(u32x4*)(Kst + key_to_row(st_r) * Lay::kKRow + seg * 16) = kreg[j];
        if constexpr (kBf16) {
          // transpose 8 d-values of keys r (even) and r+1 (odd, the neighbouring lane) into
          // V^T[8seg + e][r..r+1]: the even lane writes e = 0..3, the odd lane e = 4..7.
          const bool odd = st_r & 1;
          const u32x4 mine = vreg[j];
          const uint32_t send0 = odd ? mine[0] : mine[2];
          const uint32_t send1 = odd ? mine[1] : mine[3];
          const uint32_t got0 = __shfl_xor((int)send0, 1);
          const uint32_t got1 = __shfl_xor((int)send1, 1);
          // even lane: own = (e01, e23) of key r, other = (e01, e23) of key r+1
          // odd lane:  own = (e45, e67) of key r, other = (e45, e67) of key r-1
          const uint32_t own0 = odd ? mine[2] : mine[0];
          const uint32_t own1 = odd ? mine[3] : mine[1];
          const uint32_t lo0 = odd ? got0 : own0;  // dword holding the even key's pair
          const uint32_t hi0 = odd ? own0 : got0;  // dword holding the odd key's pair
          const uint32_t lo1 = odd ? got1 : own1;
          const uint32_t hi1 = odd ? own1 : got1;
          const int e0 = odd ? 4 : 0;
          const int kpair = st_r & ~1;
          char* vt = Vst + (8 * seg + e0) * Lay::kVRow + kpair * 2;
          *(uint32_t*)(vt + 0 * Lay::kVRow) = (lo0 & 0xffffu) | (hi0 << 16);
          *(uint32_t*)(vt + 1 * Lay::kVRow) = (lo0 >> 16) | (hi0 & 0xffff0000u);
          *(uint32_t*)(vt + 2 * Lay::kVRow) = (lo1 & 0xffffu) | (hi1 << 16);
          *(uint32_t*)(vt + 3 * Lay::kVRow) = (lo1 >> 16) | (hi1 & 0xffff0000u);
        } else {
          *(u32x4*)(Vst + st_r * Lay::kVRow + seg * 16) = vreg[j];
        }
      }
    }
    if (tid < kChunk) Sst[tid] = srcrow >= 0 ? srcrow : 0x7fffffff;
  };

  // ---- accumulators
  constexpr int kOT = D / 32;
  f32x16 o[kOT];
#pragma unroll
  for (int t = 0; t < kOT; ++t) o[t] = zero16();
  float m_ref = -INFINITY;
  float l_run = 0.f;

  // ---- prologue: chunk 0 into stage 0, sigma of chunk 1 in flight
  int sig_next = load_sig(kbeg);
  load_kv(sig_next);
  store_stage(0, sig_next);
  sig_next = nchunks > 1 ? load_sig(kbeg + kChunk) : -1;
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const int kc0 = kbeg + c * kChunk;
    const bool has_next = c + 1 < nchunks;
    const int sig_c1 = sig_next;
    if (has_next) load_kv(sig_c1);
    if (c + 2 < nchunks) sig_next = load_sig(kc0 + 2 * kChunk);

    if (wave_on && c >= c_first && c <= c_last) {
      const char* st = smem + (c & 1) * Lay::kStage;
      const char* Kst = st;
      const char* Vst = st + Lay::kKBytes;
      const int* Sst = (const int*)(st + Lay::kSigOff);

      // S^T[key rho(row)][col] = <K[key], Q[col]>
      f32x16 s = zero16();
      if constexpr (kBf16) {
        const char* kp = Kst + (lane & 31) * Lay::kKRow + h32 * 16;
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(kp + kb * 32));
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kb], s, 0, 0, 0);
        }
      } else {
        const char* kp = Kst + (lane & 31) * Lay::kKRow + h32 * (D / 2) * 4;
#pragma unroll
        for (int t4 = 0; t4 < D / 8; ++t4) {
          const f32x4 a4 = *(const f32x4*)(kp + t4 * 16);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[u], qf[4 * t4 + u], s, 0, 0, 0);
        }
      }

      // mask + scale.  Register r holds key kc0 + 16(r/8) + 8*h32 + r%8.
      const bool interior = kc0 >= w_shi - L && kc0 + kChunk - 1 <= w_slo + R &&
                            kc0 + kChunk - 1 < n;
      int sk[16];
      if constexpr (SIGMASK) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const u32x4 a = *(const u32x4*)(Sst + 16 * half + 8 * h32);
          const u32x4 bq = *(const u32x4*)(Sst + 16 * half + 8 * h32 + 4);
          sk[8 * half + 0] = a[0];
          sk[8 * half + 1] = a[1];
          sk[8 * half + 2] = a[2];
          sk[8 * half + 3] = a[3];
          sk[8 * half + 4] = bq[0];
          sk[8 * half + 5] = bq[1];
          sk[8 * half + 6] = bq[2];
          sk[8 * half + 7] = bq[3];
        }
      }
      // masked raw scores; the max is taken before scaling (the scale is positive)
      float sm[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kc0 + 16 * (r >> 3) + 8 * h32 + (r & 7);
        bool ok = interior || band_member(myslot, key, n, L, R);
        if constexpr (SIGMASK) ok = ok && sk[r] <= myorig;
        sm[r] = ok ? s[r] : -INFINITY;
      }
      float mraw = sm[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mraw = fmaxf(mraw, sm[r]);
      mraw = fmaxf(mraw, __shfl_xor(mraw, 32));
      const float mx = mraw * prm.scale_log2;  // log2 units

      const bool need = mx > m_ref + kLazy;
      const float m_new = need ? mx : m_ref;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
      m_ref = m_new;
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sm[r], prm.scale_log2, -m_use));
      if (__ballot(need)) {
#pragma unroll
        for (int t = 0; t < kOT; ++t) o[t] *= alpha;
      }

      // O^T[d][col] += V^T[d][key] P^T[key][col]
      if constexpr (kBf16) {
        bf16x8 pb0, pb1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb0[e] = (__bf16)p[e];
          pb1[e] = (__bf16)p[8 + e];
        }
        // The row sum is taken over the bf16-rounded weights that enter the P*V product, so the
        // output is an exact convex combination of V rows with (slightly perturbed) weights.
        float psum = 0.f;
        const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb0[e], pb0[e + 1]}, one2, psum, false);
          psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb1[e], pb1[e + 1]}, one2, psum, false);
        }
        l_run = l_run * alpha + psum;
        const char* vp = Vst + (lane & 31) * Lay::kVRow + h32 * 16;
#pragma unroll
        for (int t = 0; t < kOT; ++t) {
          const bf16x8 a0 = __builtin_bit_cast(bf16x8, *(const u32x4*)(vp + t * 32 * Lay::kVRow));
          const bf16x8 a1 =
              __builtin_bit_cast(bf16x8, *(const u32x4*)(vp + t * 32 * Lay::kVRow + 32));
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, pb0, o[t], 0, 0, 0);
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, pb1, o[t], 0, 0, 0);
        }
      } else {
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) psum += p[r];
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 16 * (r >> 3) + 8 * h32 + (r & 7);
          const float* vrow = (const float*)(Vst + key * Lay::kVRow) + (lane & 31);
#pragma unroll
          for (int t = 0; t < kOT; ++t)
            o[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32 * t], p[r], o[t], 0, 0, 0);
        }
      }
    }

    if (has_next) store_stage((c + 1) & 1, sig_c1);
    __syncthreads();
  }

  // ---- epilogue: normalise, gate, scatter to original row sigma[p]
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!colvalid) return;
  float f = 1.0f / l_tot;
  if (prm.gate) f *= prm.gate[((int64_t)b * n + myorig) * prm.Hq + h];
  char* orow = prm.out + qrow_elems * (int64_t)sizeof(T);
#pragma unroll
  for (int t = 0; t < kOT; ++t) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * t + 8 * a + 4 * h32;
      float y[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) y[u] = o[t][4 * a + u] * f;
      if constexpr (kBf16) {
        u32x2* dst = (u32x2*)(orow + d0 * 2);
        if constexpr (EPI == kEpiPartial) {
          // the gated intermediate: fp16 of y * 2^-8 (8x finer than bf16, range 1.6e7)
          uint32_t w[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const _Float16 lo = (_Float16)(y[2 * u] * kPartialScale);
            const _Float16 hi = (_Float16)(y[2 * u + 1] * kPartialScale);
            w[u] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
          }
          *dst = u32x2{w[0], w[1]};
        } else {
          if constexpr (EPI == kEpiAddPartial) {
            const u32x2 old = *dst;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              y[2 * u] += (float)__builtin_bit_cast(_Float16, (uint16_t)(old[u] & 0xffffu)) *
                          kPartialUnscale;
              y[2 * u + 1] += (float)__builtin_bit_cast(_Float16, (uint16_t)(old[u] >> 16)) *
                              kPartialUnscale;
            }
          }
          const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)y[0]) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)y[1]) << 16);
          const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)y[2]) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)y[3]) << 16);
          *dst = u32x2{w0, w1};
        }
      } else {
        // fp32: the gated intermediate is plain fp32
        f32x4* dst = (f32x4*)(orow + d0 * 4);
        if constexpr (EPI == kEpiAddPartial) {
          const f32x4 old = *dst;
#pragma unroll
          for (int u = 0; u < 4; ++u) y[u] += old[u];
        }
        *dst = f32x4{y[0], y[1], y[2], y[3]};
      }
    }
  }
}

// ---- neighbour bitmask (debug): same membership test as the attention kernel
__global__ void zero_words_kernel(uint32_t* p, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0u;
}

__global__ void neighbor_mask_kernel(const int32_t* sigma, int n, int L, int R, bool sigmask,
                                     uint32_t* bits, int words) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n * n) return;
  const int p = (int)(idx / n);
  const int q = (int)(idx - (int64_t)p * n);
  if (!band_member(p, q, n, L, R)) return;
  const int sp = sigma ? sigma[p] : p;
  const int sq = sigma ? sigma[q] : q;
  if (sigmask && !(sq <= sp)) return;
  atomicOr(&bits[(int64_t)sp * words + (sq >> 5)], 1u << (sq & 31));
}

// ---- host-side dispatch
template <typename T, int D, bool PERM, bool SIGMASK, int EPI>
static hipError_t launch_t(const Params& prm, int ntiles, int nbg, hipStream_t stream) {
  (void)ntiles;
  (void)nbg;
  hipLaunchKernelGGL((band_attn_kernel<T, D, PERM, SIGMASK, EPI>), dim3(prm.nblocks),
                     dim3(kThreads), 0, stream, prm);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_d(const BandLaunch& a, const Params& prm, int ntiles, int nbg,
                           hipStream_t s) {
  // The SA pass of the gated path adds to the SWA pass's intermediate; nothing else combines.
  if (a.perm) {
    const bool add = a.epilogue == kEpiAddPartial;
    if (a.causal)
      return add ? launch_t<T, D, true, true, kEpiAddPartial>(prm, ntiles, nbg, s)
                 : launch_t<T, D, true, true, kEpiStore>(prm, ntiles, nbg, s);
    return add ? launch_t<T, D, true, false, kEpiAddPartial>(prm, ntiles, nbg, s)
               : launch_t<T, D, true, false, kEpiStore>(prm, ntiles, nbg, s);
  }
  return a.epilogue == kEpiPartial ? launch_t<T, D, false, false, kEpiPartial>(prm, ntiles, nbg, s)
                                   : launch_t<T, D, false, false, kEpiStore>(prm, ntiles, nbg, s);
}

hipError_t launch_band_attn(const BandLaunch& a, hipStream_t stream) {
  Params prm;
  prm.q = (const char*)a.q;
  prm.k = (const char*)a.k;
  prm.v = (const char*)a.v;
  prm.sigma = a.sigma;
  prm.gate = a.gate;
  prm.out = (char*)a.out;
  prm.B = a.B;
  prm.n = a.n;
  prm.Hq = a.Hq;
  prm.Hkv = a.Hkv;
  prm.G = a.Hq / a.Hkv;
  prm.L = a.window - 1;
  // Causal SWA (sigma = identity): sigma[q] <= sigma[p] is q <= p, i.e. no keys right of p.
  prm.R = (!a.perm && a.causal) ? 0 : a.window - 1;
  prm.scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)a.d));
  const int64_t ncols = (int64_t)a.n * prm.G;
  const int ntiles = (int)((ncols + kColsWG - 1) / kColsWG);
  const int nbg = a.B * a.Hkv;
  prm.ntiles = ntiles;
  prm.nblocks = ntiles * nbg;
  if (a.dtype == 1) {
    return a.d == 128 ? launch_d<__bf16, 128>(a, prm, ntiles, nbg, stream)
                      : launch_d<__bf16, 64>(a, prm, ntiles, nbg, stream);
  }
  return a.d == 128 ? launch_d<float, 128>(a, prm, ntiles, nbg, stream)
                    : launch_d<float, 64>(a, prm, ntiles, nbg, stream);
}

hipError_t launch_neighbor_mask(const int32_t* sigma, int n, int window, bool causal,
                                uint32_t* bits, hipStream_t stream) {
  const int words = (n + 31) / 32;
  const int64_t count = (int64_t)n * words;
  const int L = window - 1;
  const int R = (sigma == nullptr && causal) ? 0 : window - 1;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                     stream, bits, count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t pairs = (int64_t)n * n;
  hipLaunchKernelGGL(neighbor_mask_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0,
                     stream, sigma, n, L, R, sigma != nullptr && causal, bits, words);
  return hipGetLastError();
}

}  // namespace ssw
