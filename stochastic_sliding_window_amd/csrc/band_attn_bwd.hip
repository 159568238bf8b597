// Backward pass of band attention on gfx950 (SA, SWA and the gated layer), and the gate combine
// of the training forward.  bf16 inputs and outputs, fp32 accumulation.
//
// What is computed.  The forward is [SA-ja] "技術的概要：確率的アテンション", 中核メカニズム steps
// 1-3 with the causal rule of 理論的性質 ([HYB] ハイブリッドアーキテクチャの定義 for SWA): the query
// at permuted slot p (original token sigma[p]) attends to the keys at slots q with
// |p - q| <= w - 1, in causal mode only those with sigma[q] <= sigma[p].  A layer output is
// y = g * A with g a gate value per (token, head) (1 when absent).  Its gradient, by the chain
// rule through that definition, with P rebuilt from the forward's log-sum-exp:
//   dP = (g dy) V^T,  Delta = rowsum(g dy * A),  dS = P * (dP - Delta),
//   dQ = s dS K,  dK = s dS^T Q,  dV = P^T (g dy),  dg = rowsum(dy * A)   (s = 1/sqrt(d)).
//
// Mapping onto the chip: two kernels and no atomics, so every gradient row is written once.
//   * bwd_dq_kernel is query-major with the forward's tiling: a workgroup owns 128 (slot, head)
//     columns of one KV head, 32 per wave.  Its prologue loads the columns' Q and dy rows (MFMA
//     B operands, kept in registers), forms Delta and dg from dy and A, and stores Delta for the
//     second kernel.  Its loop streams the band's 32-key K/V chunks: S^T = K Q^T and
//     dP^T = V (dy)^T share the row-read A operands, and dQ^T += K^T dS^T takes K^T from
//     transposed LDS reads, with dS^T already in B-operand order.
//   * bwd_dkdv_kernel is key-major: a wave owns 32 key slots of one KV head (their K rows are B
//     operands in registers, their V rows sit in LDS), the workgroup 128.  Its loop streams
//     chunks of 32 query columns (Q and dy rows plus each column's log-sum-exp, Delta, gate and
//     original index): S = Q K^T and dP = dy V^T leave P and dS with one key per lane,
//     which is the B operand of dV^T += (dy)^T (g P) and dK^T += Q^T dS.
//   * Chunks are gathered through sigma by direct buffer-to-LDS loads into an LDS ring (three
//     chunks ahead in the dQ kernel, one in the dK/dV kernel).  Rows sit in MFMA row order, their
//     16-byte granules XOR-swizzled by a function of the row (Lay::swz), which keeps both the row
//     reads of the score products and the transposed reads (ds_read_b64_tr_b16) of the gradient
//     products free of bank conflicts.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "band_attn.h"
#include "lds_dma.h"

namespace ssw {
namespace bwd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
#define SSW_LDS __attribute__((address_space(3)))

constexpr int kThreads = 256;  // 4 waves
constexpr int kChunk = 32;     // keys (dq kernel) or query columns (dk/dv kernel) per chunk
constexpr int kTile = 128;     // columns (dq kernel) or key slots (dk/dv kernel) per workgroup
constexpr float kLog2e = 1.4426950408889634f;
// sigma entries held in LDS at a time: the chunk loads read a row's original index there, so a
// chunk's row loads wait for one memory latency instead of two (sigma, then the row)
constexpr int kSigCap = 2048;

// An entry of a malformed sigma (sigma is trusted unless the caller asks for validation) is
// taken as token 0: the result is wrong, but every row it selects lies inside the tensors, so it
// cannot become a memory fault.
__device__ __forceinline__ int in_range(int tok, int n) {
  return (uint32_t)tok < (uint32_t)n ? tok : 0;
}

struct Params {
  const char* q;
  const char* k;
  const char* v;
  const char* o;
  const char* dout;
  const float* lse;
  const float* gate;
  const int32_t* sigma;
  char* dq;
  char* dk;
  char* dv;
  float* dgate;
  float* delta;
  int B, n, Hq, Hkv, G;
  int L, R;          // band: key slots [p - L, p + R] of query slot p
  float scale_log2;  // log2(e) / sqrt(d)
  float scale;       // 1 / sqrt(d)
  float inv_g;       // 1 / G
  int ntiles;        // tiles per (batch row, KV head)
  int nblocks;       // ntiles * B * Hkv
  int accumulate;
};

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// lanes l and l ^ 32 hold the same column; v_permlane32_swap exchanges the halves (inline asm:
// the builtin's two results were folded into one when both inputs were the same value)
__device__ __forceinline__ float pair_sum(float x) {
  float a = x, c = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(c));
  return a + c;
}

// MFMA 32x32 row r of a chunk holds chunk entry rho(r), where rho swaps bits 2 and 3 of r: then
// output register i of lane half h holds entry 16(i / 8) + 8h + i % 8, which is the k order of
// the B operand of the next product.  rho is its own inverse.
__device__ __forceinline__ int rho(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Consecutive workgroup ids go to the 8 XCDs in turn; renumber them so each XCD (own L2) gets a
// contiguous run of tiles, whose K/V or Q/dy halos overlap.
__device__ __forceinline__ int xcd_local_order(int i, int nblocks) {
  const int per = nblocks / 8;
  if (i < per * 8) return (i % 8) * per + i / 8;
  return i;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// A wave's 32 gradient rows, from MFMA fragments to memory.  Lane l holds row l % 32; register
// 4a + u of block db holds element d = 32db + 8a + 4(l / 32) + u.  The rows are assembled in fp32
// in the wave's 32 * D * 4 bytes of LDS at `reg` (16-byte granules XOR-swizzled by row), then
// leave as whole 16-byte bf16 granules, D / 8 lanes per row, so that one store instruction writes
// complete rows.  Row r goes to base + (row offset held by lane r); lanes holding kOutOfRange
// have no row.  `accumulate` adds the stored row in fp32 and rounds once.
template <int D>
__device__ __forceinline__ void store_rows(char* reg, const f32x16* acc, float scale, char* base,
                                           uint32_t my_off, bool accumulate, int lane) {
  constexpr int kG32 = D / 4;  // 16-byte fp32 granules per row
  const int r32 = lane & 31;
  const int h32 = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int gi = (8 * db + 2 * a + h32) ^ (r32 & (kG32 - 1));
      *(f32x4*)(reg + r32 * D * 4 + 16 * gi) =
          f32x4{acc[db][4 * a] * scale, acc[db][4 * a + 1] * scale, acc[db][4 * a + 2] * scale,
                acc[db][4 * a + 3] * scale};
    }
  }
  // the rows are read back by other lanes of this wave: its LDS writes must have completed
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerRound = 64 / kLanesPerRow;
#pragma unroll
  for (int i = 0; i < 32 / kRowsPerRound; ++i) {
    const int r = i * kRowsPerRound + lane / kLanesPerRow;
    const int j = lane % kLanesPerRow;  // elements 8j .. 8j + 7
    const uint32_t roff = (uint32_t)__builtin_amdgcn_ds_bpermute(r * 4, (int)my_off);
    const char* src = reg + r * D * 4;
    const f32x4 lo = *(const f32x4*)(src + 16 * ((2 * j) ^ (r & (kG32 - 1))));
    const f32x4 hi = *(const f32x4*)(src + 16 * ((2 * j + 1) ^ (r & (kG32 - 1))));
    if (roff != lds_dma::kOutOfRange) {
      u32x4* dst = (u32x4*)(base + roff + 16 * j);
      float y[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      if (accumulate) {
        const u32x4 old = *dst;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[2 * e] += bf_lo(old[e]);
          y[2 * e + 1] += bf_hi(old[e]);
        }
      }
      *dst = u32x4{pack2(y[0], y[1]), pack2(y[2], y[3]), pack2(y[4], y[5]), pack2(y[6], y[7])};
    }
  }
  // the wave's LDS slice may be written again right after (reads done before any later write)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

template <int D>
struct Lay {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kGran = D / 8;                // 16-byte granules per row
  static constexpr int kMat = kChunk * kRowBytes;    // one 32-row matrix of a stage
  static constexpr int kPer = 2 * kChunk * kGran / kThreads;  // granules per thread per chunk
  static constexpr int kKB = D / 16;                 // k steps of the score products
  static constexpr int kDB = D / 32;                 // 32-row d blocks of a gradient accumulator
  static_assert(kPer >= 1 && 2 * kChunk * kGran == kPer * kThreads, "chunk split");
  // Granule g of MFMA row r sits at granule position g ^ swz(r) of its row.  The reads that
  // must not collide on LDS banks:
  //  * row reads (16 bytes per lane, 16 lanes per cycle): rows r .. r + 15, one granule each;
  //  * transposed reads (8 bytes per lane, 32 lanes per cycle): four rows 4a .. 4a + 3 (rows
  //    rho(e) of four consecutive entries e) times four consecutive granules 4b .. 4b + 3.
  // 256-byte rows (d = 128) span all 64 banks: swz(r) swaps the two 2-bit halves of r % 16,
  // which is one-to-one on r % 16 (row reads) and gives the rows 4a + i the values 4i + const, so
  // that g ^ swz(r) = 4(b ^ i) + (g % 4 ^ const) takes 16 distinct values (transposed reads).
  // 128-byte rows (d = 64) pair up on the banks, rows 2m and 2m + 1 side by side: swz(r) is bits
  // 1, 2, 3 of r in reverse order, one-to-one on m % 8 (row reads), and rows 4a, 4a + 2 (the
  // same bank half) differ in bit 2 of swz, which moves granules 4b .. 4b + 3 to the other four.
  static __device__ __forceinline__ int swz(int r) {
    if constexpr (kGran == 16)
      return ((r & 3) << 2) | ((r >> 2) & 3);
    else
      return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
  }
};

// LDS offset of granule `gran` of MFMA row `row` within a stage matrix
template <int D>
__device__ __forceinline__ int gran_off(int row, int gran) {
  return row * Lay<D>::kRowBytes + ((gran ^ Lay<D>::swz(row)) << 4);
}

// Per-lane LDS offsets of the transposed reads of a stage matrix.  The A operand of a gradient
// product (32 d-rows x 16 chunk entries) for k block t comes from two ds_read_b64_tr_b16: lane j
// of 16-lane group grp points at 4 d-values of chunk entry 16t + 8h + 4*hi + j/4 at
// d = 32db + 16(grp % 2) + 4(j % 4); after the read, lane l holds row d = 32db + l % 32 for
// entries 16t + 8h + [0, 8).  Entry e sits at row rho(e); adding 16t to e adds 16t to the row,
// which leaves the swizzle unchanged, so t is a constant offset.
template <int D>
__device__ __forceinline__ int tr_off(int lane, int db, int hi) {
  const int grp = lane >> 4;
  const int j = lane & 15;
  const int e = 8 * (lane >> 5) + 4 * hi + (j >> 2);
  const int row = rho(e);
  const int d = 32 * db + 16 * (grp & 1) + 4 * (j & 3);
  return row * Lay<D>::kRowBytes + (((d >> 3) ^ Lay<D>::swz(row)) << 4) + ((d & 7) << 1);
}

__device__ __forceinline__ bf16x8 tr_read(const char* lo_p, const char* hi_p) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SSW_LDS s16x4*)(const SSW_LDS char*)lo_p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SSW_LDS s16x4*)(const SSW_LDS char*)hi_p);
  // whole-vector casts only (element-wise assembly of such operands was miscompiled)
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
  const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
}

// floor(x / G) for 0 <= x < 2^12 with inv_g = 1/G in fp32: (x + 1/2) / G lies at least 1/(2G)
// from every integer, far beyond the rounding error of the product
__device__ __forceinline__ int div_small(int x, float inv_g) {
  return (int)(((float)x + 0.5f) * inv_g);
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const char* p) {
  return __builtin_bit_cast(bf16x8, *(const u32x4*)p);
}

// ------------------------------------------------------------------------------------------------
// dQ (and Delta, dg): query-major
// ------------------------------------------------------------------------------------------------
constexpr int kDqStages = 4;  // LDS ring of K/V chunks: three in flight while one is consumed

template <int D, bool PERM, bool SIGMASK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(Params prm) {
  using LY = Lay<D>;
  constexpr int kStage = 2 * LY::kMat;                // K rows, then V rows, of one chunk
  constexpr int kPF = kDqStages - 1;                  // chunks in flight
  constexpr int kSigOff = kDqStages * kStage;
  constexpr int kSegChunks = kSigCap / kChunk;        // chunks whose keys' sigma fit in LDS
  constexpr int kRowsPerDma = 1024 / LY::kRowBytes;   // rows one 64-lane 16-byte DMA covers
  constexpr int kDmaMat = LY::kMat / 1024;            // DMA instructions per matrix and chunk
  constexpr int kDW = 2 * kDmaMat / 4;                // per wave (4 waves)
  static_assert(kDW >= 1 && 2 * kDmaMat == 4 * kDW, "DMA split");
  __shared__ __attribute__((aligned(16))) char smem[kSigOff + (PERM ? kSigCap * 4 : 0)];
  int* sig_lds = (int*)(smem + kSigOff);
  const uint32_t smem_lds = lds_dma::lds_addr(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h32 = lane >> 5;
  const int r32 = lane & 31;
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

  // ---- columns: column c is (slot c / G, query head g * G + c % G)
  const int col0_wg = tile * kTile;
  const int col0_w = col0_wg + wave * 32;
  const int mycol = col0_w + r32;
  const bool colvalid = mycol < nG;
  const int mycol_c = colvalid ? mycol : nG - 1;
  const int myslot = mycol_c / G;
  const int h = g * G + (mycol_c - myslot * G);
  const int myorig = PERM ? in_range(prm.sigma[myslot], n) : myslot;
  const bool wave_on = col0_w < nG;
  const int w_slo = min(col0_w, nG - 1) / G;
  const int w_shi = min(col0_w + 31, nG - 1) / G;
  const int S_lo = col0_wg / G;
  const int S_hi = min(col0_wg + kTile - 1, nG - 1) / G;
  const int kbeg = max(0, S_lo - L);
  const int kend = min(n - 1, S_hi + R);
  const int nchunks = (kend - kbeg) / kChunk + 1;
  const int c_first = (max(0, w_slo - L) - kbeg) / kChunk;
  const int c_last = (min(n - 1, w_shi + R) - kbeg) / kChunk;

  // ---- K/V rows of this (batch row, KV head): buffer resources, rows addressed by token
  const uint32_t row_stride = (uint32_t)(prm.Hkv * LY::kRowBytes);
  const int64_t kv_base = ((int64_t)b * n * prm.Hkv + g) * LY::kRowBytes;
  const uint32_t kv_range = (uint32_t)((int64_t)(n - 1) * row_stride + LY::kRowBytes);
  const lds_dma::i32x4 rs_k = lds_dma::resource(prm.k + kv_base, kv_range);
  const lds_dma::i32x4 rs_v = lds_dma::resource(prm.v + kv_base, kv_range);
  int seg_key0 = kbeg;  // first key of the current sigma segment
  // This wave's DMA instructions of a chunk: instruction I = wave * kDW + i brings stage rows
  // kRowsPerDma m + j (m = I % kDmaMat = kDW (wave % 2) + i, j = lane / kGran) of matrix
  // I / kDmaMat; lane l writes LDS slot l % kGran of its row, which holds granule
  // (l % kGran) ^ swz(row) of that row, and row r holds chunk key rho(r).  The parts of the row
  // occupy disjoint bits and rho and swz are bit permutations, so the key is 16 (wave % 2) +
  // rho(kRowsPerDma i) + rho(j) (a wave-uniform base, an immediate and a lane constant) and the
  // granule offset a lane constant XOR an immediate; each lane reads its key's token from the
  // sigma segment itself.  Keys past the sequence end hold the token n there (or are themselves
  // >= n), whose row lies past the buffer range and reads as zeros; the band test drops them.
  static_assert(kRowsPerDma * kDW == 16 && 2 * kDW == kDmaMat, "DMA row split");
  auto dma_chunk = [&](int c) {
    const int kc0 = kbeg + c * kChunk;
    const uint32_t st_lds = smem_lds + (uint32_t)((c % kDqStages) * kStage);
    uint32_t ln = lane;  // opaque copy: the lane constants are recomputed per chunk
    asm volatile("" : "+v"(ln));
    const int j = ln / LY::kGran;
    const int gsw_l = ((ln % LY::kGran) ^ LY::swz(j)) << 4;
    const int key_l = kc0 + 16 * (wave & 1) + rho(j);
    const int* sk = sig_lds + (key_l - seg_key0);
    uint32_t voff[kDW];
#pragma unroll
    for (int i = 0; i < kDW; ++i) {
      const int tok = PERM ? sk[rho(kRowsPerDma * i)] : key_l + rho(kRowsPerDma * i);
      voff[i] = __umul24((uint32_t)tok, row_stride) +
                (uint32_t)(gsw_l ^ (LY::swz(kRowsPerDma * i) << 4));
    }
#pragma unroll
    for (int i = 0; i < kDW; ++i) {
      const int I = wave * kDW + i;
      lds_dma::load16(I < kDmaMat ? rs_k : rs_v,
                      st_lds + (I / kDmaMat) * LY::kMat + (I % kDmaMat) * 1024, voff[i]);
    }
  };
  // sigma of the keys of the segment's chunks (keys past the end hold n: no row, and every
  // causal test fails)
  auto load_sigma_seg = [&](int nkeys) {
    for (int i = tid; i < nkeys; i += kThreads) {
      const int key = seg_key0 + i;
      sig_lds[i] = key < n ? in_range(prm.sigma[key], n) : n;
    }
  };

  // ---- prologue: sigma of the first segment, two chunks in flight, the columns' O, dy and Q
  // rows, then the third chunk
  const int seg_end0 = min(nchunks, kSegChunks);
  if constexpr (PERM) {
    load_sigma_seg(seg_end0 * kChunk);
    __syncthreads();
  }
  const int npro = min(kPF, seg_end0);
  for (int c = 0; c < min(kPF - 1, npro); ++c) dma_chunk(c);

  // The rows of the wave's 32 columns arrive whole, D / 8 lanes per row (one load instruction
  // covers 64 / (D / 8) rows), pass through the wave's slice of ring stages 2 and 3 (not in use
  // until the third chunk is issued) in the stage matrices' swizzled layout, and leave it as
  // B operands: k step kb holds d = 16kb + 8h32 + [0, 8) of the lane's column.  Gathering the
  // B operands straight from memory would touch 32 rows per load instruction.
  const int64_t rowq = ((int64_t)b * n + myorig) * prm.Hq + h;
  bf16x8 qf[LY::kKB], df[LY::kKB];
  float dot = 0.f;
  {
    constexpr int kLanesPerRow = D / 8;
    constexpr int kRowsPerLd = 64 / kLanesPerRow;
    constexpr int kLd = 32 / kRowsPerLd;
    static_assert(2 * kStage >= 4 * 32 * LY::kRowBytes, "four waves' rows fit two stages");
    const int64_t qd_batch = (int64_t)b * n * prm.Hq * LY::kRowBytes;
    // byte offset of the lane's column row within batch row b (below 2^31, checked at the API)
    const uint32_t my_off = (uint32_t)(((int64_t)myorig * prm.Hq + h) * LY::kRowBytes);
    const int j = lane % kLanesPerRow;
    u32x4 ro[kLd], rd[kLd], rq[kLd];
#pragma unroll
    for (int i = 0; i < kLd; ++i) {
      const int r = i * kRowsPerLd + lane / kLanesPerRow;
      const int64_t off =
          qd_batch + (uint32_t)__builtin_amdgcn_ds_bpermute(4 * r, (int)my_off) + 16 * j;
      ro[i] = *(const u32x4*)(prm.o + off);
      rd[i] = *(const u32x4*)(prm.dout + off);
      rq[i] = *(const u32x4*)(prm.q + off);
    }
    char* reg = smem + 2 * kStage + wave * 32 * LY::kRowBytes;
    // one matrix at a time through the slice; other lanes read what a lane wrote, so each
    // matrix's writes complete before its reads, and its reads before the next one's writes
    auto through_lds = [&](const u32x4* rows, u32x4* frag) {
#pragma unroll
      for (int i = 0; i < kLd; ++i)
        *(u32x4*)(reg + gran_off<D>(i * kRowsPerLd + lane / kLanesPerRow, j)) = rows[i];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int kb = 0; kb < LY::kKB; ++kb)
        frag[kb] = *(const u32x4*)(reg + gran_off<D>(r32, 2 * kb + h32));
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };
    u32x4 aw[LY::kKB], dw[LY::kKB], qw[LY::kKB];
    through_lds(ro, aw);
    through_lds(rd, dw);
    through_lds(rq, qw);
#pragma unroll
    for (int kb = 0; kb < LY::kKB; ++kb) {
      df[kb] = __builtin_bit_cast(bf16x8, dw[kb]);
      qf[kb] = __builtin_bit_cast(bf16x8, qw[kb]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot = __builtin_fmaf(bf_lo(dw[kb][e]), bf_lo(aw[kb][e]), dot);
        dot = __builtin_fmaf(bf_hi(dw[kb][e]), bf_hi(aw[kb][e]), dot);
      }
    }
  }
  dot = pair_sum(dot);
  const float gate_v = prm.gate ? prm.gate[rowq] : 1.0f;
  const float delta = gate_v * dot;
  const float lse2 = prm.lse[rowq] * kLog2e;
  if (colvalid && h32 == 0) {
    prm.delta[rowq] = delta;
    if (prm.dgate) prm.dgate[rowq] = dot;
  }
  // Every wave is done with stages 2 and 3, which the third chunk and the loop's first DMA
  // take.  The Delta and dg stores need not complete first: the loop's vmcnt waits count them
  // as well, which only makes a wait longer, and the row loads, issued after the first two
  // chunks, have returned (in order, so those chunks have landed too).
  __syncthreads();
  if (kPF - 1 < npro) dma_chunk(kPF - 1);

  int k_off[LY::kKB];
#pragma unroll
  for (int kb = 0; kb < LY::kKB; ++kb) k_off[kb] = gran_off<D>(r32, 2 * kb + h32);
  int t_off[LY::kDB][2];
#pragma unroll
  for (int db = 0; db < LY::kDB; ++db) {
    t_off[db][0] = tr_off<D>(lane, db, 0);
    t_off[db][1] = tr_off<D>(lane, db, 1);
  }

  f32x16 acc[LY::kDB];
#pragma unroll
  for (int db = 0; db < LY::kDB; ++db) acc[db] = zero16();

  // ---- chunks, segment by segment: chunk c sits in ring stage c % kDqStages
  for (int seg_c0 = 0; seg_c0 < nchunks; seg_c0 += kSegChunks) {
    const int seg_end = min(nchunks, seg_c0 + kSegChunks);
    if (seg_c0 > 0) {
      // drain the previous segment, bring in this one's sigma, then its first chunks
      lds_dma::wait_vmcnt<0>();
      __syncthreads();
      seg_key0 = kbeg + seg_c0 * kChunk;
      if constexpr (PERM) {
        load_sigma_seg((seg_end - seg_c0) * kChunk);
        __syncthreads();
      }
      for (int c = seg_c0; c < min(seg_c0 + kPF, seg_end); ++c) dma_chunk(c);
    }
    for (int c = seg_c0; c < seg_end; ++c) {
      // chunk c has landed when at most (chunks issued after it) * kDW of this wave's DMAs are
      // outstanding: kPF - 1 chunks in steady state, fewer near the segment end
      const int after = min(kPF - 1, seg_end - 1 - c);
      if (after >= 2)
        lds_dma::wait_vmcnt<2 * kDW>();
      else if (after == 1)
        lds_dma::wait_vmcnt<kDW>();
      else
        lds_dma::wait_vmcnt<0>();
      __syncthreads();  // every wave's DMAs of chunk c landed; chunk c - 1 is consumed
      if (c + kPF < seg_end) dma_chunk(c + kPF);  // into chunk c - 1's stage
      if (!wave_on || c < c_first || c > c_last) continue;
      const char* Kst = smem + (c % kDqStages) * kStage;
      const char* Vst = Kst + LY::kMat;

      // S^T[key][col] = <K, Q>, dP^T[key][col] = <V, dy>; output register i of lane half h32
      // holds key 16(i / 8) + 8h32 + i % 8 of the chunk
      f32x16 s = zero16();
      f32x16 dp = zero16();
#pragma unroll
      for (int kb = 0; kb < LY::kKB; ++kb) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_bf16x8(Kst + k_off[kb]), qf[kb], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_bf16x8(Vst + k_off[kb]), df[kb], dp, 0, 0,
                                                     0);
      }
      const int kc0 = kbeg + c * kChunk;
      // dS of the lane's 16 scores, four keys at a time (registers 4qd .. 4qd + 3 hold keys
      // e0 .. e0 + 3): their sigma arrives as one 16-byte read and the mask is a select (exp2
      // runs for masked scores too), so that no element waits on an LDS read of its own.  In an
      // interior chunk (every key inside the band of every slot of the wave, and before the
      // sequence end) only the causal test remains.
      bf16x8 dsb[2];
      auto scores = [&](auto interior_c) {
        constexpr bool kInterior = decltype(interior_c)::value;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int e0 = 16 * (qd >> 1) + 8 * h32 + 4 * (qd & 1);
          u32x4 sg4 = {0, 0, 0, 0};
          if constexpr (SIGMASK) sg4 = *(const u32x4*)(sig_lds + (kc0 + e0 - seg_key0));
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = 4 * qd + u;
            const int key = kc0 + e0 + u;
            bool ok = true;
            if constexpr (!kInterior) ok = (key >= myslot - L) & (key <= myslot + R) & (key < n);
            if constexpr (SIGMASK) ok = ok & ((int)sg4[u] <= myorig);
            const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], prm.scale_log2, -lse2));
            const float p = ok ? x : 0.f;
            dsb[r >> 3][r & 7] = (__bf16)(p * __builtin_fmaf(gate_v, dp[r], -delta));
          }
        }
      };
      if (kc0 >= w_shi - L && kc0 + kChunk - 1 <= w_slo + R && kc0 + kChunk - 1 < n)
        scores(std::true_type{});
      else
        scores(std::false_type{});
      // dQ^T[d][col] += K^T[d][key] dS^T[key][col]
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int db = 0; db < LY::kDB; ++db) {
          const char* kt = Kst + 16 * t * LY::kRowBytes;
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              tr_read(kt + t_off[db][0], kt + t_off[db][1]), dsb[t], acc[db], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: dQ row of the column at its original token, assembled in fp32 in the ring
  // (free once every wave is past its last chunk: each wave takes 32 rows)
  __syncthreads();
  static_assert(4 * 32 * D * 4 <= kSigOff, "fp32 rows of four waves fit the ring");
  if (!wave_on) return;
  // byte offset of the column's dQ row within batch row b (below 2^31, checked at the API)
  const uint32_t my_off =
      colvalid ? (uint32_t)(((int64_t)myorig * prm.Hq + h) * LY::kRowBytes) : lds_dma::kOutOfRange;
  store_rows<D>(smem + wave * 32 * D * 4, acc, prm.scale,
                prm.dq + (int64_t)b * n * prm.Hq * LY::kRowBytes, my_off, prm.accumulate != 0,
                lane);
}

// ------------------------------------------------------------------------------------------------
// dK, dV: key-major
// ------------------------------------------------------------------------------------------------
// The V rows of the workgroup's keys sit in LDS rather than in registers: the K operand and the
// two accumulators already take 160 registers per lane at d = 128, and two waves per SIMD need
// the total to stay within 256.  At d = 64 the kernel fits 168 registers (in causal mode one
// value goes to scratch and back per chunk), which gives three waves per SIMD and three
// workgroups per CU: the 360M-shaped gated backward took 444 us against 470-474 us at two.
template <int D, bool PERM, bool SIGMASK>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2, D == 64 ? 3 : 2)))
void bwd_dkdv_kernel(Params prm) {
  using LY = Lay<D>;
  // per stage: Q rows, dy rows, then per column lse, Delta, gate (64 floats each: a 4-byte DMA
  // covers 64 lanes), then the columns' original indices (32 ints)
  constexpr int kMetaOff = 2 * LY::kMat;
  constexpr int kOrigOff = kMetaOff + 3 * 64 * 4;
  constexpr int kStage = kOrigOff + kChunk * 4;
  constexpr int kRowsPerDma = 1024 / LY::kRowBytes;
  constexpr int kDmaMat = LY::kMat / 1024;  // DMA instructions per matrix and chunk
  constexpr int kDW = 2 * kDmaMat / 4;      // per wave
  static_assert(kDW >= 1 && 2 * kDmaMat == 4 * kDW, "DMA split");
  constexpr int kVOff = 2 * kStage;                      // V rows of the 128 keys
  constexpr int kSigOff = kVOff + kTile * LY::kRowBytes;
  // The last region holds either sigma (a segment of kSigCap slots) or, when the workgroup's
  // chunks number at most kTabChunks, a table of every chunk column's row offset and (causal
  // mode) original index.
  constexpr int kTabChunks = 56;
  constexpr int kTabBytes = kTabChunks * kChunk * 4 * (SIGMASK ? 2 : 1);
  constexpr int kLastBytes = (PERM && kSigCap * 4 > kTabBytes) ? kSigCap * 4 : kTabBytes;
  static_assert(2 * (kSigOff + kLastBytes) <= 160 * 1024, "two workgroups per CU");
  __shared__ __attribute__((aligned(16))) char smem[kSigOff + kLastBytes];
  int* sig_lds = (int*)(smem + kSigOff);
  uint32_t* tab_row = (uint32_t*)(smem + kSigOff);
  int* tab_orig = (int*)(smem + kSigOff + kTabChunks * kChunk * 4);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h32 = lane >> 5;
  const int r32 = lane & 31;
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

  // ---- key slots of this workgroup / wave / lane
  const int K0 = tile * kTile;
  const int kw0 = K0 + wave * 32;
  const int myk = kw0 + r32;
  const bool keyvalid = myk < n;
  const int myk_c = keyvalid ? myk : n - 1;
  const int ktok = PERM ? in_range(prm.sigma[myk_c], n) : myk_c;
  const bool wave_on = kw0 < n;
  // key q is in the band of the query slots [q - R, q + L]
  const int khi_wg = min(K0 + kTile - 1, n - 1);
  const int col_lo = max(0, K0 - R) * G;
  const int col_hi = min(n - 1, khi_wg + L) * G + G - 1;
  // chunks lie on one grid of kChunk columns for every workgroup: chunk c holds the columns
  // col_base + c kChunk + [0, kChunk)
  const int col_base = col_lo / kChunk * kChunk;
  const int nchunks = (col_hi - col_base) / kChunk + 1;
  const int wk_lo = min(kw0, n - 1);
  const int wk_hi = min(kw0 + 31, n - 1);
  const int c_first = (max(0, wk_lo - R) * G - col_base) / kChunk;
  const int c_last = (min(n - 1, wk_hi + L) * G + G - 1 - col_base) / kChunk;
  // Visiting order.  About three neighbouring workgroups read each chunk, and in band order they
  // would reach it many chunks apart, after the L2 has cycled.  So, when every chunk's rows are
  // known from the start (the row table, or the sigma of every slot the chunks touch in one LDS
  // segment), step i takes the chunk whose index on the common grid is i modulo nchunks:
  // workgroups of equal chunk counts that start together read each chunk at the same step.
  // Otherwise the chunks go in band order and the segment moves along.
  const int last_slot_all = min(n - 1, (col_base + nchunks * kChunk - 1) / G);
  const bool use_tab = nchunks <= kTabChunks;
  const bool one_seg = !PERM || use_tab || last_slot_all - col_base / G < kSigCap;
  const int a0 = col_base / kChunk;
  const int rot = one_seg ? (nchunks - a0 % nchunks) % nchunks : 0;
  auto chunk_at = [&](int i) {
    const int c = i + rot;
    return c >= nchunks ? c - nchunks : c;
  };

  // ---- K row of the lane's key as B operands (k step kb holds d = 16kb + 8h32 + [0, 8)); its V
  // row goes to LDS in the same swizzled layout as the stage matrices (row = key within the tile)
  const int64_t krow = ((int64_t)b * n + ktok) * prm.Hkv + g;
  bf16x8 kf[LY::kKB];
  char* vrows = smem + kVOff + wave * 32 * LY::kRowBytes;
#pragma unroll
  for (int kb = 0; kb < LY::kKB; ++kb) {
    const int off = (16 * kb + 8 * h32) * 2;
    kf[kb] = ld_bf16x8(prm.k + krow * LY::kRowBytes + off);
    *(u32x4*)(vrows + gran_off<D>(r32, 2 * kb + h32)) =
        *(const u32x4*)(prm.v + krow * LY::kRowBytes + off);
  }

  // ---- sigma of the query slots [seg_s0, seg_s0 + kSigCap), in LDS (permuted operator)
  int seg_s0 = col_base / G;
  auto load_sigma_seg = [&](int s0) {
    for (int i = tid; i < kSigCap; i += kThreads) {
      const int slot = s0 + i;
      sig_lds[i] = slot < n ? in_range(prm.sigma[slot], n) : 0;
    }
  };
  auto orig_of_slot = [&](int slot) { return PERM ? sig_lds[slot - seg_s0] : slot; };

  // ---- chunk staging: direct buffer-to-LDS loads of the chunk's Q and dy rows (MFMA row order,
  // granules swizzled by row) and of its columns' lse, Delta and gate.  The columns' rows and, in
  // causal mode, original indices come from the row table when there is one; otherwise each
  // chunk's rows are looked up through the sigma segment as the chunk is issued, and the first 32
  // threads write its original indices into the stage.  One chunk is in flight while the
  // previous one is scored (two stages: the V rows of the tile take the rest of the LDS).
  const uint32_t smem_lds = lds_dma::lds_addr(smem);
  const int64_t qd_batch = (int64_t)b * n * prm.Hq;
  const uint32_t qd_range = (uint32_t)((int64_t)n * prm.Hq * LY::kRowBytes);
  const lds_dma::i32x4 rs_q = lds_dma::resource(prm.q + qd_batch * LY::kRowBytes, qd_range);
  const lds_dma::i32x4 rs_d = lds_dma::resource(prm.dout + qd_batch * LY::kRowBytes, qd_range);
  const uint32_t m_range = (uint32_t)((int64_t)n * prm.Hq * 4);
  const lds_dma::i32x4 rs_m = lds_dma::resource(
      wave == 0 ? (const void*)(prm.lse + qd_batch)
                : wave == 1 ? (const void*)(prm.delta + qd_batch)
                            : (const void*)(prm.gate ? prm.gate + qd_batch : prm.lse + qd_batch),
      m_range);
  // Table path: DMA instruction i of this wave covers stage rows kRowsPerDma m + j with
  // m = kDW (wave % 2) + i and j = lane / kGran; the three parts occupy disjoint bits, and rho and
  // swz are bit permutations, so the row's chunk entry is 16 (wave % 2) + rho(kRowsPerDma i) +
  // rho(j) (a wave-uniform base, an immediate and a lane constant) and its granule offset a lane
  // constant XOR an immediate.
  static_assert(kRowsPerDma * kDW == 16 && 2 * kDW == kDmaMat, "DMA row split");
  auto dma_chunk_tab = [&](int c, int stage) {
    const uint32_t st_lds = smem_lds + (uint32_t)(stage * kStage);
    uint32_t ln = lane;  // opaque copy: the lane constants are recomputed per chunk
    asm volatile("" : "+v"(ln));
    const int j = ln / LY::kGran;
    const int gsw_l = ((ln % LY::kGran) ^ LY::swz(j)) << 4;
    const uint32_t* tr = tab_row + c * kChunk + 16 * (wave & 1) + rho(j);
    uint32_t voff[kDW];
#pragma unroll
    for (int i = 0; i < kDW; ++i)
      voff[i] = tr[rho(kRowsPerDma * i)] + (uint32_t)(gsw_l ^ (LY::swz(kRowsPerDma * i) << 4));
#pragma unroll
    for (int i = 0; i < kDW; ++i) {
      const int I = wave * kDW + i;
      lds_dma::load16(I < kDmaMat ? rs_q : rs_d,
                      st_lds + (I / kDmaMat) * LY::kMat + (I % kDmaMat) * 1024, voff[i]);
    }
    if (wave < 3 && (wave < 2 || prm.gate)) {
      const uint32_t rb = tab_row[c * kChunk + (ln & (kChunk - 1))];
      constexpr int kSh = LY::kRowBytes == 256 ? 6 : 5;  // row bytes to 4 bytes per row
      static_assert(LY::kRowBytes == 4 << kSh, "row size");
      const uint32_t moff =
          ln < kChunk && rb != lds_dma::kOutOfRange ? rb >> kSh : lds_dma::kOutOfRange;
      lds_dma::load4(rs_m, st_lds + kMetaOff + wave * 256, moff);
    }
  };
  auto dma_chunk = [&](int c, int stage) {
    if (use_tab) {
      dma_chunk_tab(c, stage);
      return;
    }
    const int c0 = col_base + c * kChunk;
    const int slot0 = c0 / G;  // wave-uniform
    const int rem0 = c0 - slot0 * G;
    const uint32_t st_lds = smem_lds + (uint32_t)(stage * kStage);
    // Lane l finds the row of chunk entry l % 32 once (its slot, the slot's token, the query
    // head), and each row DMA takes the rows it needs from those lanes by ds_bpermute.  The lane
    // index is an opaque copy, so the lane constants below are recomputed per chunk rather than
    // held across the loop beside the accumulators.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int e_l = ln & (kChunk - 1);
    const bool ok_l = c0 + e_l < nG;  // columns past the end read as zeros; their band test fails
    const int x = rem0 + (ok_l ? e_l : nG - 1 - c0);
    const int ds = div_small(x, prm.inv_g);
    const int orig_l = orig_of_slot(slot0 + ds);
    const int row_l = orig_l * prm.Hq + g * G + (x - ds * G);  // token row * Hq + query head
    const uint32_t rb_l = ok_l ? (uint32_t)row_l * LY::kRowBytes : lds_dma::kOutOfRange;
    // DMA i covers stage rows kRowsPerDma m + j (m = I % kDmaMat, j = lane / kGran): row bits
    // below kRowsPerDma come from j alone, and rho and swz are bit permutations, so the lane's
    // entry and granule split into a lane part and a wave-uniform part joined by XOR
    const int j = ln / LY::kGran;
    const int ent_l = 4 * rho(j);                              // ds_bpermute byte address
    const int gsw_l = ((ln % LY::kGran) ^ LY::swz(j)) << 4;    // granule byte offset
    uint32_t voff[kDW];
#pragma unroll
    for (int i = 0; i < kDW; ++i) {
      const int mrow = kRowsPerDma * ((wave * kDW + i) % kDmaMat);
      const uint32_t rb =
          (uint32_t)__builtin_amdgcn_ds_bpermute(ent_l ^ (4 * rho(mrow)), (int)rb_l);
      // a row past the end stays at or above kOutOfRange, beyond the buffer's range
      voff[i] = rb + (uint32_t)(gsw_l ^ (LY::swz(mrow) << 4));
    }
#pragma unroll
    for (int i = 0; i < kDW; ++i) {
      const int I = wave * kDW + i;
      lds_dma::load16(I < kDmaMat ? rs_q : rs_d,
                      st_lds + (I / kDmaMat) * LY::kMat + (I % kDmaMat) * 1024, voff[i]);
    }
    // waves 0, 1, 2 fetch lse, Delta, gate (lanes 0..31: the chunk's columns)
    if (wave < 3 && (wave < 2 || prm.gate)) {
      const uint32_t moff = ln < kChunk && ok_l ? (uint32_t)row_l * 4u : lds_dma::kOutOfRange;
      lds_dma::load4(rs_m, st_lds + kMetaOff + wave * 256, moff);
    }
    if (SIGMASK && tid < kChunk) {
      int* mi = (int*)(smem + stage * kStage + kOrigOff);
      // the column's original index (columns past the end fail the band test)
      mi[tid] = ok_l ? orig_l : -1;
    }
  };

  f32x16 dk[LY::kDB], dv[LY::kDB];
#pragma unroll
  for (int db = 0; db < LY::kDB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }

  const int a_base = gran_off<D>(r32, h32);
  const int t_base0 = tr_off<D>(lane, 0, 0);
  const int t_base1 = tr_off<D>(lane, 0, 1);
  // The band test in column space: column col_base + x is in the band of the lane's key when
  // its slot (col_base + x) / G lies in [myk - R, myk + L] and the column exists
  // (col_base + x < nG), i.e. band_lo <= x <= band_hi.
  const int band_lo = (myk - R) * G - col_base;
  const int band_hi = min(myk + L + 1, n) * G - 1 - col_base;
  // the columns inside the band of every key of the wave
  const int wband_lo = __builtin_amdgcn_readfirstlane((wk_hi - R) * G - col_base);
  const int wband_hi = __builtin_amdgcn_readfirstlane(min(wk_lo + L + 1, n) * G - 1 - col_base);
  // Without a gate the stages' gate entries hold 1 (the gate DMA never writes them).
  if (!prm.gate && tid < 2 * kChunk)
    *(float*)(smem + (tid / kChunk) * kStage + kMetaOff + 128 * 4 + (tid % kChunk) * 4) = 1.0f;

  if (use_tab) {
    // one entry per column of the workgroup's chunks, from sigma in global memory
    for (int idx = tid; idx < nchunks * kChunk; idx += kThreads) {
      const int col = col_base + idx;
      const bool ok = col < nG;
      const int colc = ok ? col : nG - 1;
      const int slot = colc / G;
      const int orig = PERM ? in_range(prm.sigma[slot], n) : slot;
      tab_row[idx] = ok ? (uint32_t)(orig * prm.Hq + g * G + (colc - slot * G)) * LY::kRowBytes
                        : lds_dma::kOutOfRange;
      if constexpr (SIGMASK) tab_orig[idx] = ok ? orig : -1;
    }
    __syncthreads();
  } else if constexpr (PERM) {
    load_sigma_seg(seg_s0);
    __syncthreads();
  }
  dma_chunk(chunk_at(0), 0);
  for (int i = 0; i < nchunks; ++i) {
    const int c = chunk_at(i);
    const int st = i & 1;
    lds_dma::wait_vmcnt<0>();  // this wave's loads of step i (and, first time, the prologue's)
    __syncthreads();           // every wave's; step i - 1 is scored, its stage is free
    if (i + 1 < nchunks) {
      if (PERM && !one_seg) {
        // band order (c = i): move the segment when chunk c + 1 reaches past it
        const int last_slot = min(n - 1, (col_base + (c + 2) * kChunk - 1) / G);
        if (last_slot - seg_s0 >= kSigCap) {
          // every read of the current segment (chunk c's loads) was before the barrier above
          seg_s0 = (col_base + (c + 1) * kChunk) / G;
          load_sigma_seg(seg_s0);
          __syncthreads();
        }
      }
      dma_chunk(chunk_at(i + 1), st ^ 1);
    }
    if (!wave_on || c < c_first || c > c_last) continue;
    const char* Qst = smem + st * kStage;
    const char* Dst = Qst + LY::kMat;
    // Per-lane LDS offsets, from two base offsets held across the loop: the row read of k step
    // kb is a_base ^ (kb << 5) and the transposed read of d block db and half hi is
    // t_base[hi] ^ (db << 6) (the k step and the d block enter the granule index in bits the row
    // and its swizzle leave alone).  Opaque copies per chunk keep the optimiser from holding all
    // sixteen offsets in registers.
    int ab = a_base, tb0 = t_base0, tb1 = t_base1;
    asm volatile("" : "+v"(ab), "+v"(tb0), "+v"(tb1));
    int a_off[LY::kKB];
#pragma unroll
    for (int kb = 0; kb < LY::kKB; ++kb) a_off[kb] = ab ^ (kb << 5);
    int t_off[LY::kDB][2];
#pragma unroll
    for (int db = 0; db < LY::kDB; ++db) {
      t_off[db][0] = tb0 ^ (db << 6);
      t_off[db][1] = tb1 ^ (db << 6);
    }
    const float* mf = (const float*)(Qst + kMetaOff);  // lse [0, 64), Delta [64, ..), gate
    // original index of each column
    const int* mi = use_tab ? tab_orig + c * kChunk : (const int*)(Qst + kOrigOff);

    // S[col][key] = <Q, K>, dP[col][key] = <dy, V>; output register i of lane half h32 holds
    // column 16(i / 8) + 8h32 + i % 8 of the chunk, for the lane's key
    f32x16 s = zero16();
    f32x16 dp = zero16();
#pragma unroll
    for (int kb = 0; kb < LY::kKB; ++kb) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_bf16x8(Qst + a_off[kb]), kf[kb], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_bf16x8(Dst + a_off[kb]),
                                                   ld_bf16x8(vrows + a_off[kb]), dp, 0, 0, 0);
    }
    // P and dS of the lane's 16 scores, four columns at a time: registers 4qd .. 4qd + 3 hold
    // columns x = e0 + 8 h32 + u (e0 = 16 (qd / 2) + 4 (qd % 2)).  Each group's log-sum-exp,
    // Delta, gate and original indices arrive as 16-byte reads and the mask is a select (exp2
    // runs for masked scores too), so that no score waits on an LDS read of its own.  Each
    // group's reads are issued after the previous group's results (an empty asm ties their
    // address to them): all sixteen scores' values at once would not fit in the registers.
    // In an interior chunk (every column inside the band of every key of the wave) only the
    // causal test remains.
    const int lo = band_lo - c * kChunk - 8 * h32;
    const int hi = band_hi - c * kChunk - 8 * h32;
    bf16x8 pb[2], dsb[2];
    auto scores = [&](auto interior_c) {
      constexpr bool kInterior = decltype(interior_c)::value;
      int moff = 32 * h32;  // byte offset of the lane half's first column in each metadata array
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int e0 = 16 * (qd >> 1) + 4 * (qd & 1);
        const char* mq = (const char*)mf + moff + 4 * e0;
        const f32x4 lse4 = *(const f32x4*)(mq);
        const f32x4 del4 = *(const f32x4*)(mq + 64 * 4);
        const f32x4 gt4 = *(const f32x4*)(mq + 128 * 4);
        u32x4 or4 = {0, 0, 0, 0};
        if constexpr (SIGMASK) or4 = *(const u32x4*)((const char*)mi + moff + 4 * e0);
        float last = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * qd + u;
          bool ok = true;
          if constexpr (!kInterior) ok = (e0 + u >= lo) & (e0 + u <= hi);
          if constexpr (SIGMASK) ok = ok & (ktok <= (int)or4[u]);
          const float x =
              __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], prm.scale_log2, -lse4[u] * kLog2e));
          const float p = ok ? x : 0.f;
          const float pg = p * gt4[u];
          pb[r >> 3][r & 7] = (__bf16)pg;
          dsb[r >> 3][r & 7] = (__bf16)(p * __builtin_fmaf(gt4[u], dp[r], -del4[u]));
          last = pg;
        }
        asm volatile("" : "+v"(moff) : "v"(last));
      }
    };
    if (c * kChunk >= wband_lo && c * kChunk + kChunk - 1 <= wband_hi)
      scores(std::true_type{});
    else
      scores(std::false_type{});
    // dV^T[d][key] += dy^T[d][col] (g P)[col][key];  dK^T[d][key] += Q^T[d][col] dS[col][key]
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int db = 0; db < LY::kDB; ++db) {
        const char* dt = Dst + 16 * t * LY::kRowBytes;
        const char* qt = Qst + 16 * t * LY::kRowBytes;
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read(dt + t_off[db][0], dt + t_off[db][1]),
                                                         pb[t], dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read(qt + t_off[db][0], qt + t_off[db][1]),
                                                         dsb[t], dk[db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: dK, then dV, rows of the lane's key at its original token, each assembled in
  // fp32 in LDS (the stages and the V rows are free once every wave is past its last chunk)
  __syncthreads();
  static_assert(4 * 32 * D * 4 <= kSigOff, "fp32 rows of four waves fit the stages and V rows");
  if (!wave_on) return;
  // byte offset of the key's row within batch row b (below 2^31, checked at the API)
  const uint32_t my_off =
      keyvalid ? (uint32_t)(((int64_t)ktok * prm.Hkv + g) * LY::kRowBytes) : lds_dma::kOutOfRange;
  const int64_t kv_batch = (int64_t)b * n * prm.Hkv * LY::kRowBytes;
  char* reg = smem + wave * 32 * D * 4;
  store_rows<D>(reg, dk, prm.scale, prm.dk + kv_batch, my_off, prm.accumulate != 0, lane);
  store_rows<D>(reg, dv, 1.0f, prm.dv + kv_batch, my_off, prm.accumulate != 0, lane);
}

// ------------------------------------------------------------------------------------------------
// Gate combine of the training forward: out = g_sa * y_sa + g_swa * y_swa, 8 values per thread
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gate_combine_kernel(const char* y_sa, const char* y_swa,
                                                           const float* gates, char* out,
                                                           int64_t rows, int gran_per_row) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * gran_per_row) return;
  const int64_t row = i / gran_per_row;
  const float ga = gates[row];
  const float gb = gates[rows + row];
  const u32x4 a = *(const u32x4*)(y_sa + 16 * i);
  const u32x4 c = *(const u32x4*)(y_swa + 16 * i);
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = pack2(__builtin_fmaf(ga, bf_lo(a[e]), gb * bf_lo(c[e])),
                 __builtin_fmaf(ga, bf_hi(a[e]), gb * bf_hi(c[e])));
  }
  *(u32x4*)(out + 16 * i) = o;
}

// ------------------------------------------------------------------------------------------------
// host-side dispatch
// ------------------------------------------------------------------------------------------------
template <typename K>
static hipError_t launch(K kernel, int nblocks, hipStream_t s, void* e0, void* e1,
                         const Params& prm) {
  if (e0 || e1)
    hipExtLaunchKernelGGL(kernel, dim3(nblocks), dim3(kThreads), 0, s, (hipEvent_t)e0,
                          (hipEvent_t)e1, 0, prm);
  else
    hipLaunchKernelGGL(kernel, dim3(nblocks), dim3(kThreads), 0, s, prm);
  return hipGetLastError();
}

template <int D, bool PERM, bool SIGMASK>
static hipError_t launch_t(const BandBwdLaunch& a, Params prm, hipStream_t s) {
  const int64_t ncols = (int64_t)a.n * prm.G;
  prm.ntiles = (int)((ncols + kTile - 1) / kTile);
  prm.nblocks = prm.ntiles * a.B * a.Hkv;
  hipError_t e = launch(bwd_dq_kernel<D, PERM, SIGMASK>, prm.nblocks, s, a.ev[0], a.ev[1], prm);
  if (e != hipSuccess) return e;
  prm.ntiles = (a.n + kTile - 1) / kTile;
  prm.nblocks = prm.ntiles * a.B * a.Hkv;
  return launch(bwd_dkdv_kernel<D, PERM, SIGMASK>, prm.nblocks, s, a.ev[2], a.ev[3], prm);
}

template <int D>
static hipError_t launch_d(const BandBwdLaunch& a, const Params& prm, hipStream_t s) {
  if (a.perm)
    return a.causal ? launch_t<D, true, true>(a, prm, s) : launch_t<D, true, false>(a, prm, s);
  return launch_t<D, false, false>(a, prm, s);
}

}  // namespace bwd

// ---- Delta without allocation: a device array of this library (one copy per GPU, held until the
// process ends) for callers that cannot allocate memory.  Its name is a host-side stand-in for the
// array, not a device address: host code reaches the array only through the address that
// hipGetSymbolAddress returns for the current device, which is looked up on the first call on
// each device and kept.  Every call on one GPU shares the array: calls that overlap on one GPU
// race.  The dQ kernel writes every entry the dK/dV kernel reads, so nothing needs clearing.
static __device__ __align__(256) float scratch[kBwdScratchFloats];

hipError_t bwd_scratch_pointer(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    per_device[dev] = (float*)p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

hipError_t launch_band_attn_bwd(const BandBwdLaunch& a, hipStream_t stream) {
  bwd::Params prm;
  prm.q = (const char*)a.q;
  prm.k = (const char*)a.k;
  prm.v = (const char*)a.v;
  prm.o = (const char*)a.o;
  prm.dout = (const char*)a.dout;
  prm.lse = a.lse;
  prm.gate = a.gate;
  prm.sigma = a.sigma;
  prm.dq = (char*)a.dq;
  prm.dk = (char*)a.dk;
  prm.dv = (char*)a.dv;
  prm.dgate = a.dgate;
  prm.delta = a.delta;
  prm.B = a.B;
  prm.n = a.n;
  prm.Hq = a.Hq;
  prm.Hkv = a.Hkv;
  prm.G = a.Hq / a.Hkv;
  prm.L = a.window - 1;
  // causal SWA (sigma = identity): no key right of the query
  prm.R = (!a.perm && a.causal) ? 0 : a.window - 1;
  prm.scale = (float)(1.0 / __builtin_sqrt((double)a.d));
  prm.inv_g = 1.0f / (float)prm.G;
  prm.scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)a.d));
  prm.accumulate = a.accumulate ? 1 : 0;
  prm.ntiles = 0;
  prm.nblocks = 0;
  return a.d == 128 ? bwd::launch_d<128>(a, prm, stream) : bwd::launch_d<64>(a, prm, stream);
}

hipError_t launch_gate_combine(const void* y_sa, const void* y_swa, const float* gates, void* out,
                               int64_t rows, int d, hipStream_t stream) {
  const int gpr = d / 8;
  const int64_t total = rows * gpr;
  hipLaunchKernelGGL(bwd::gate_combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     stream, (const char*)y_sa, (const char*)y_swa, gates, (char*)out, rows, gpr);
  return hipGetLastError();
}

}  // namespace ssw
