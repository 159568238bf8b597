// Gate projections of the gated SA + SWA layer on gfx950: gates = sigmoid(x w + b).
//
// What is computed ([SA-ja] "技術的概要：確率的アテンション", ゲート付き SA と SWA の組み合わせ: the
// gate weights come from independent sigmoid projections of the layer input): for every token
// row r of x [rows, Hm] and output column j of the projection (j < Hq: the SA gate of query head
// j; j >= Hq: the SWA gate of head j - Hq),
//     gates[j / Hq][r][j % Hq] = sigmoid(sum_k x[r][k] * w_t[j][k] + bias[j]),
// written straight into the [2, rows, Hq] layout the gated attention calls take.
//
// Mapping onto the chip: a skinny GEMM (N = 2 Hq <= 128 columns, K = Hm) bound by reading x.  A
// workgroup takes 128 rows, a wave 32 of them; each wave accumulates its 32 x N tile with bf16
// 32x32x16 MFMAs.  Its x rows are read row-contiguously in blocks of 64 k, one block ahead, and
// staged through a wave-private LDS buffer into the A-operand layout.  The matching block of the
// projection's rows w_t[j] (B operands; w_t is [N, Hm] row-major, the usual layout of a linear
// layer's weight) is read row-contiguously by the whole workgroup into a shared, double-buffered
// LDS block, so that w_t crosses the L2 once per workgroup, in whole rows.  A split of the k
// range over the waves of a workgroup (4x the waves in flight) measured slower: every workgroup
// then reads all of w_t once per wave.  The epilogue adds the bias, applies the sigmoid and
// scatters the columns to their gate plane.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gate_proj.h"

namespace ssw {
namespace gproj {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRowsWG = 128;
constexpr int kMaxTiles = 4;  // N <= 128
constexpr int kUnroll = 4;    // k steps of 16 per loop iteration
constexpr int kSub = 2;       // 64-k sub-blocks per barrier (of the shared w_t buffer)

struct Params {
  const char* x;
  const char* w_t;
  const float* bias;
  float* gates;
  int rows, Hm, Hq, N;
};

// Granule g of a 128-byte LDS row r sits at granule position g ^ swz(r).  A 16-byte read by 16
// lanes touching rows r0 .. r0 + 15 (one granule each) then covers all 64 banks: odd and even rows
// take the two halves of the banks, and the eight rows of each half get eight distinct positions.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

template <int NT>
__global__ __launch_bounds__(kThreads) void gate_proj_kernel(Params prm) {
  __shared__ __attribute__((aligned(16))) char x_lds[4][kSub][32 * 128];
  // the workgroup's block of w_t (NT * 32 rows x 64 k per sub-block), double-buffered and shared
  // by the waves
  __shared__ __attribute__((aligned(16))) char w_lds[2][kSub][NT * 32 * 128];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31;
  const int h32 = lane >> 5;
  const int row0 = blockIdx.x * kRowsWG + wave * 32;
  // waves past the last row take part in the shared loads and barriers only
  const bool wave_on = row0 < prm.rows;
  const int row0c = wave_on ? row0 : prm.rows - 1;
  const int myrow = min(row0c + r32, prm.rows - 1);
  const int64_t rb = (int64_t)prm.Hm * 2;
  const char* xrow = prm.x + (int64_t)myrow * rb + 16 * h32;
  const char* wrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    wrow[t] = prm.w_t + (int64_t)min(32 * t + r32, prm.N - 1) * rb + 16 * h32;

  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;

  // A (32 rows x 16 k): lane holds row r32, k = 8 h32 .. 8 h32 + 7; B (16 k x 32 columns): lane
  // holds column 32t + r32 at the same k
  const int steps = prm.Hm / 16;
  int s = 0;
  // Blocks of kSub * 64 k, one barrier each.  The wave's 32 x rows are read row-contiguously
  // (8 lanes cover 128 bytes of a row), one block ahead in registers, and go through a
  // wave-private LDS buffer.  The block of w_t (all N rows) is read row-contiguously by the whole
  // workgroup, one block ahead, into a shared double buffer: every wave of the workgroup takes its
  // B operands from it, so w_t crosses the L2 once per workgroup instead of once per wave, and in
  // whole rows.
  {
    const int nblk = prm.Hm / (64 * kSub);
    const char* xwave = prm.x + (int64_t)row0c * rb;
    auto load_x = [&](int kb, u32x4 (&r)[kSub][4]) {
#pragma unroll
      for (int h = 0; h < kSub; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = min(8 * i + lane / 8, prm.rows - 1 - row0c);
          r[h][i] = *(const u32x4*)(xwave + (int64_t)row * rb + (kSub * kb + h) * 128 +
                                    (lane % 8) * 16);
        }
    };
    // thread tid brings granule tid % 8 of w_t rows 32 i + tid / 8
    auto load_w = [&](int kb, u32x4 (&r)[kSub][NT]) {
#pragma unroll
      for (int h = 0; h < kSub; ++h)
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const int row = min(32 * i + tid / 8, prm.N - 1);
          r[h][i] = *(const u32x4*)(prm.w_t + (int64_t)row * rb + (kSub * kb + h) * 128 +
                                    (tid % 8) * 16);
        }
    };
    u32x4 xc[kSub][4], xn[kSub][4], wc[kSub][NT], wn[kSub][NT];
    if (nblk > 0) {
      load_x(0, xc);
      load_w(0, wc);
    }
    for (int kb = 0; kb < nblk; ++kb) {
#pragma unroll
      for (int h = 0; h < kSub; ++h) {
        char* wl = w_lds[kb & 1][h];
        char* xl = x_lds[wave][h];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const int row = 32 * i + tid / 8;
          *(u32x4*)(wl + row * 128 + (((tid % 8) ^ swz(row)) << 4)) = wc[h][i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 8 * i + lane / 8;
          *(u32x4*)(xl + row * 128 + (((lane % 8) ^ swz(row)) << 4)) = xc[h][i];
        }
      }
      // block kb of w_t is in place for every wave; every wave is done with block kb - 2, whose
      // buffer was just refilled (its reads came before the previous barrier)
      __syncthreads();
      if (kb + 1 < nblk) {
        load_x(kb + 1, xn);
        load_w(kb + 1, wn);
      }
      if (wave_on) {
#pragma unroll
        for (int h = 0; h < kSub; ++h) {
          const char* wl = w_lds[kb & 1][h];
          const char* xl = x_lds[wave][h];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int gpos = ((2 * u + h32) ^ swz(r32)) << 4;
            const u32x4 a = *(const u32x4*)(xl + r32 * 128 + gpos);
#pragma unroll
            for (int t = 0; t < NT; ++t)
              acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, a),
                  __builtin_bit_cast(bf16x8, *(const u32x4*)(wl + (32 * t + r32) * 128 + gpos)),
                  acc[t], 0, 0, 0);
          }
        }
      }
      if (kb + 1 < nblk) {
#pragma unroll
        for (int h = 0; h < kSub; ++h) {
#pragma unroll
          for (int i = 0; i < 4; ++i) xc[h][i] = xn[h][i];
#pragma unroll
          for (int i = 0; i < NT; ++i) wc[h][i] = wn[h][i];
        }
      }
    }
    s = 4 * kSub * nblk;
  }
  if (!wave_on) return;  // the remaining steps have no barrier
  for (; s + kUnroll <= steps; s += kUnroll) {
    u32x4 a[kUnroll], bw[kUnroll][NT];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      a[u] = *(const u32x4*)(xrow + 32 * (s + u));
#pragma unroll
      for (int t = 0; t < NT; ++t) bw[u][t] = *(const u32x4*)(wrow[t] + 32 * (s + u));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[u]),
                                                         __builtin_bit_cast(bf16x8, bw[u][t]),
                                                         acc[t], 0, 0, 0);
  }
  for (; s < steps; ++s) {
    const u32x4 a = *(const u32x4*)(xrow + 32 * s);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8, a),
          __builtin_bit_cast(bf16x8, *(const u32x4*)(wrow[t] + 32 * s)), acc[t], 0, 0, 0);
  }

  // ---- epilogue: output register i of tile t holds row 8(i / 4) + 4 h32 + i % 4, column
  // 32t + r32
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int j = 32 * t + r32;
    if (j >= prm.N) continue;
    const float bj = prm.bias ? prm.bias[j] : 0.f;
    const int path = j >= prm.Hq;
    const int hh = j - path * prm.Hq;
    float* plane = prm.gates + (int64_t)path * prm.rows * prm.Hq + hh;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = row0 + 8 * (i >> 2) + 4 * h32 + (i & 3);
      if (r < prm.rows) {
        const float z = acc[t][i] + bj;
        plane[(int64_t)r * prm.Hq] = 1.0f / (1.0f + __expf(-z));
      }
    }
  }
}

}  // namespace gproj

hipError_t launch_gate_projection(const void* x, const void* w_t, const float* bias,
                                  float* gates, int rows, int Hm, int Hq, hipStream_t stream) {
  gproj::Params prm;
  prm.x = (const char*)x;
  prm.w_t = (const char*)w_t;
  prm.bias = bias;
  prm.gates = gates;
  prm.rows = rows;
  prm.Hm = Hm;
  prm.Hq = Hq;
  prm.N = 2 * Hq;
  const dim3 grid((unsigned)((rows + gproj::kRowsWG - 1) / gproj::kRowsWG));
  const int nt = (prm.N + 31) / 32;
  switch (nt) {
    case 1: hipLaunchKernelGGL(gproj::gate_proj_kernel<1>, grid, dim3(gproj::kThreads), 0, stream, prm); break;
    case 2: hipLaunchKernelGGL(gproj::gate_proj_kernel<2>, grid, dim3(gproj::kThreads), 0, stream, prm); break;
    case 3: hipLaunchKernelGGL(gproj::gate_proj_kernel<3>, grid, dim3(gproj::kThreads), 0, stream, prm); break;
    default: hipLaunchKernelGGL(gproj::gate_proj_kernel<4>, grid, dim3(gproj::kThreads), 0, stream, prm); break;
  }
  return hipGetLastError();
}

}  // namespace ssw
