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
// staged through a wave-private LDS buffer into the A-operand layout; the projection's rows
// w_t[j] (B operands; w_t is [N, Hm] row-major, the usual layout of a linear layer's weight) are
// read straight from memory (they stay in the L2).  A split of the k range over the waves of a
// workgroup (4x the waves in flight) measured slower: every workgroup then reads all of w_t.  The epilogue adds the bias, applies the sigmoid and scatters the columns to their
// gate plane.
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

struct Params {
  const char* x;
  const char* w_t;
  const float* bias;
  float* gates;
  int rows, Hm, Hq, N;
};

template <int NT>
__global__ __launch_bounds__(kThreads) void gate_proj_kernel(Params prm) {
  __shared__ __attribute__((aligned(16))) char x_lds[4][32 * 128];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r32 = lane & 31;
  const int h32 = lane >> 5;
  const int row0 = blockIdx.x * kRowsWG + wave * 32;
  if (row0 >= prm.rows) return;  // wave-uniform: no barrier in this kernel
  const int myrow = min(row0 + r32, prm.rows - 1);
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
  // Blocks of 64 k: the wave's 32 x rows are read row-contiguously (8 lanes cover a row's
  // 128 bytes), one block ahead in registers, and go through a wave-private LDS buffer (granules
  // XOR-swizzled by row) from which the A operands are read.
  {
    char* xl = x_lds[wave];
    const int nblk = prm.Hm / 64;
    const char* xwave = prm.x + (int64_t)row0 * rb;
    auto load_blk = [&](int kb, u32x4 (&r)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = min(8 * i + lane / 8, prm.rows - 1 - row0);
        r[i] = *(const u32x4*)(xwave + (int64_t)row * rb + kb * 128 + (lane % 8) * 16);
      }
    };
    u32x4 cur[4], nxt[4];
    if (nblk > 0) load_blk(0, cur);
    for (int kb = 0; kb < nblk; ++kb) {
      if (kb + 1 < nblk) load_blk(kb + 1, nxt);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 8 * i + lane / 8;
        *(u32x4*)(xl + row * 128 + ((((lane % 8) ^ (row & 7))) << 4)) = cur[i];
      }
      // the wave's own LDS stores precede its reads (in-order LDS queue); nothing else shares
      // this buffer
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x4 a = *(const u32x4*)(xl + r32 * 128 + (((2 * u + h32) ^ (r32 & 7)) << 4));
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a),
              __builtin_bit_cast(bf16x8, *(const u32x4*)(wrow[t] + 32 * (4 * kb + u))), acc[t],
              0, 0, 0);
      }
      if (kb + 1 < nblk)
#pragma unroll
        for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
    }
    s = 4 * nblk;
  }
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
