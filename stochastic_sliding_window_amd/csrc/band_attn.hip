// Band attention on gfx950: the kernel behind Stochastic Attention (SA), plain SWA and both
// passes of the gated SA+SWA layer.
//
// What is computed ([SA-ja] "技術的概要：確率的アテンション", 手法 › 中核メカニズム steps 1-3 and
// 理論的性質 › 因果的制約; [HYB] ハイブリッドアーキテクチャの定義 for SWA): the query at permuted
// slot p (original token sigma[p]) attends to the keys at slots q with |p - q| <= w - 1 (keys
// left of the band edge and past the sequence end are dropped); in causal mode a key is kept only
// if sigma[q] <= sigma[p].  With sigma = identity the causal band collapses to [p - w + 1, p],
// which this kernel exploits by taking the right band extent R = 0.  The output row of slot p is
// written at original position sigma[p], optionally times a gate, optionally combined with the
// intermediate of the gated path.
//
// Mapping onto the chip.
//   * A workgroup owns one KV head of one batch row and 32 * waves consecutive "columns", where a
//     column is a (permuted slot, query head of the KV group) pair: column c is slot c / G, head
//     c % G (G = Hq / Hkv).  The G query heads sharing a KV head sit side by side, so each K/V
//     row staged in LDS serves all of them.
//   * Each wave owns 32 columns and computes S^T = K_chunk * Q^T with 32x32 MFMAs (rows = keys,
//     columns = the wave's 32 columns), so every lane holds whole columns: the softmax statistics
//     of a column live in two lanes (lane l and l ^ 32) and need one cross-lane step.
//   * Keys stream through an LDS ring of kStages chunks of 32 keys.  Rows are gathered through
//     sigma by buffer loads that write LDS directly (no registers, no permuted copy in HBM), so
//     kStages - 1 chunks are in flight while one is consumed.  Keys past the sequence end read as
//     zeros (the buffer range check).  K rows sit in MFMA row order with an XOR swizzle of their
//     16-byte granules; V rows sit in key order, swizzled, and are read transposed with
//     ds_read_b64_tr_b16 into the A operand of O^T = V^T * P^T.
//   * The MFMA row -> key map is chosen so that the registers holding P^T after the softmax are
//     already the B operand of the next MFMA (no register shuffles between the two products).
//   * Softmax is online with a lazy reference maximum (rescale only when the running max grows
//     by more than 2^8); the row sum is taken over the bf16-rounded weights the P*V product uses.
//     Masks are evaluated per element only where a chunk touches the band edge or when the causal
//     rule needs sigma.
//   * Epilogue: divide by the row sum, multiply by the gate, scatter to row sigma[p] (the gated
//     layer's SA pass stores its fp16 intermediate there; its SWA pass adds to it).
//   * Two builds of the sigma-gathered kernel (template flag W3): two waves per SIMD with a
//     4-slot ring and two chunks per loop step, and (bf16) three waves per SIMD at d = 128 (four
//     at d = 64) with a 3-slot ring and one chunk per step; the dispatcher picks the latter when a
//     workgroup's band fits its sigma segment.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "band_attn.h"

namespace ssw {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
#define SSW_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;
constexpr int kWaves = 4;  // waves per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr int kColsWave = 32;
constexpr int kColsWG = kColsWave * kWaves;
constexpr int kChunk = 32;
// The sigma-gathered kernels have two builds (template flag W3):
//   * two waves per SIMD (register allocation sized for it), a 4-stage ring (kStages - 1 chunks
//     in flight) consumed two 32-key chunks per loop step (bf16; fp32 computes the scores of
//     chunk c + 1 alongside the softmax of chunk c), and a 2048-entry sigma segment;
//   * bf16 only, three waves per SIMD at d = 128 and four at d = 64: a 3-stage ring, one chunk per
//     step and a 1024-entry sigma segment (3 x 16 KB + 4 KB of LDS per workgroup at d = 128, so
//     three workgroups fit a CU; 28 KB at d = 64, four workgroups).  The dispatcher launches it
//     when a workgroup's band fits one segment; longer bands use the two-wave build.  The causal
//     build recomputes the K/V LDS offsets at their use from one base register each and reads
//     sigma for the mask in two halves, to fit the registers of three (d = 128: 168) or four
//     (d = 64: 128) waves.
// The identity-sigma (SWA) kernels hold no sigma in LDS and fewer registers, so they run at three
// waves per SIMD (four at d = 64, which takes 106 registers) with a 3-stage ring and one chunk
// per step.
constexpr int kStages = 4;
constexpr int kWavesPerSimd = 2;
constexpr int kSigCap = 2048;      // sigma entries held in LDS at a time (two-wave build)
constexpr int kSigCapW3 = 1024;    // the same, W3 build
constexpr int kWavesPerSimdSwa = 3;
constexpr int kStagesSwa = 3;
constexpr float kLazy = 8.0f;  // reference max may lag the true max by up to 2^8 (log2 units)
// bf16 gated path: the SA pass leaves g_sa * Y_sa in the output buffer as fp16 scaled by 2^-4
// (normal fp16 for 2^-10 <= |g_sa * Y_sa| < 1.05e6; a fixed 2^-20 step below that range)
constexpr float kPartialScale = 1.0f / 16.0f;
constexpr float kPartialUnscale = 16.0f;

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{})
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// x, as a value the compiler cannot see through: a lane-derived value passed through this at its
// use is recomputed there instead of being hoisted out of the loop into a register of its own.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Lanes l and l ^ 32 hold the same column.  v_permlane32_swap exchanges the upper half of one
// register with the lower half of another in one VALU instruction; with both holding x, one ends
// up as [x_lo, x_lo] and the other as [x_hi, x_hi], and combining them gives both lanes the
// column total.  Inline asm: the compiler builtin's two results were folded into one when both
// inputs were the same value, which dropped the combine.
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float pair_max(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float pair_sum(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return a + b;
}

// Key membership in permuted-slot space.  The attention kernel and the neighbour-mask kernel use
// this same test.
__device__ __forceinline__ bool band_member(int p, int q, int n, int L, int R) {
  return q >= p - L && q <= p + R && q >= 0 && q < n;
}

// MFMA 32x32 output row r holds key rho(r) of the chunk: rho(8a + 4h + b) = 16(a / 2) + 8h +
// 4(a % 2) + b, so lane half h's registers 0..7 hold keys 8h..8h+7 and registers 8..15 hold keys
// 16+8h..16+8h+7 -- exactly the k order of the B operand of the P*V product.
__device__ __forceinline__ int row_to_key(int r) {
  const int a = r >> 3;
  return 16 * (a >> 1) + 8 * ((r >> 2) & 1) + 4 * (a & 1) + (r & 3);
}

// ---- raw buffer loads that write LDS directly (gfx950 buffer_load ... lds).  Issued as inline
// asm so that the compiler does not serialise them with s_waitcnt vmcnt(0) before every LDS read;
// the kernel waits for them itself with wait_vmcnt<N>.  Each instruction writes the 64 lanes'
// data to consecutive LDS addresses starting at M0.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));  // stride 0, no swizzle
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);                // range checked per lane
  r[3] = 0x00020000;                                                // 32-bit data format
  return r;
}
constexpr uint32_t kOutOfRange = 0x80000000u;  // any offset >= the range reads as zero

__device__ __forceinline__ i32x4 uniform4(i32x4 r) {
  i32x4 u;
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = __builtin_amdgcn_readfirstlane(r[i]);
  return u;
}
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  rsrc = uniform4(rsrc);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_addr),
               "v"(voff), "s"(rsrc)
               : "memory");
}
__device__ __forceinline__ void dma4(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  rsrc = uniform4(rsrc);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(lds_addr),
               "v"(voff), "s"(rsrc)
               : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <typename T, int D, bool PERM, bool W3 = false>
struct Layout {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int kRowBytes = D * (int)sizeof(T);
  static constexpr int kGran = kRowBytes / 16;  // 16-byte granules per row
  static constexpr int kRowsPerDma = 1024 / kRowBytes;
  static constexpr int kMatBytes = kChunk * kRowBytes;  // one K (or V) chunk
  static constexpr int kDmaK = kMatBytes / 1024;        // DMA instructions per chunk and matrix
  static constexpr int kDmaPerWave = 2 * kDmaK / kWaves;
  static constexpr int kStageBytes = 2 * kMatBytes;
  // sigma of a segment of keys (permuted operator only)
  static constexpr int kSigCapL = W3 ? kSigCapW3 : kSigCap;
  static constexpr int kSegChunks = kSigCapL / kChunk;
  static constexpr int kSigBytes = PERM ? kSigCapL * 4 : 0;
  // ring depth: the configured number of stages, or fewer if they would not fit in 160 KB of LDS
  static constexpr int kWant = W3 ? 3 : PERM ? kStages : kStagesSwa;
  static constexpr int kNS = kWant * kStageBytes + kSigBytes <= 163840
                                 ? kWant
                                 : (163840 - kSigBytes) / kStageBytes;
  static constexpr int kPF = kNS - 1;  // chunks in flight
  static constexpr int kSigOff = kNS * kStageBytes;
  static constexpr int kSmem = kSigOff + (PERM ? kSigBytes : 16);
  static_assert(kGran >= 8, "V swizzle needs 8 granules per row");
  static_assert(kNS >= 3, "the software pipeline needs at least three stages");
  static_assert((2 * kDmaK) % kWaves == 0 && kDmaK % kDmaPerWave == 0, "DMA split");
};

// K rows (in MFMA row order) XOR their granule index with the row's low bits, so the lanes of an
// A-operand read (consecutive rows, same granule) hit distinct banks.
template <int GRAN>
__device__ __forceinline__ int swz_k(int row) {
  return row & (GRAN - 1);
}
// V rows (in key order) XOR their granule index with a function of key % 4.  A transposed read
// has each 16-lane group take 2 granules of 4 consecutive keys (and two groups together take 4
// granules of the same 4 keys).  For 16-granule rows the XOR values 0, 6, 10, 12 spread both the
// 16-lane and the 32-lane footprint over distinct bank slots (their residues mod 8 are distinct
// and so are their bits 2..3); 8-granule rows use 0, 2, 4, 6.
template <int GRAN>
__device__ __forceinline__ int swz_v(int key) {
  if constexpr (GRAN >= 16)
    return (int)((0x0C0A0600u >> (8 * (key & 3))) & 0xFFu);
  else
    return 2 * (key & 3);
}

struct Params {
  const char* q;
  const char* k;
  const char* v;
  const int32_t* sigma;
  int64_t sig_bstride;  // sigma of (batch row b, KV head g) at sigma + b * sig_bstride +
  int64_t sig_hstride;  // g * sig_hstride (both 0: one sigma shared by every row and head)
  const float* gate;
  char* out;
  float* lse;        // natural-log log-sum-exp of each row [B, n, Hq], or nullptr
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
  const int per = nblocks / 8;
  if (i < per * 8) return (i % 8) * per + i / 8;
  return i;
}

template <typename T, bool PERM, int EPI, bool W3>
constexpr bool kIsW3 = W3 && PERM && sizeof(T) == 2;
template <typename T, bool PERM, int EPI, bool W3, int D>
constexpr int kWavesPerEU = kIsW3<T, PERM, EPI, W3>       ? (D == 64 ? 4 : 3)
                            : (PERM || sizeof(T) != 2) ? kWavesPerSimd
                            : D == 64                  ? 4
                                                       : kWavesPerSimdSwa;

template <typename T, int D, bool PERM, bool SIGMASK, int EPI, bool W3>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kWavesPerEU<T, PERM, EPI, W3, D>,
                                   kWavesPerEU<T, PERM, EPI, W3, D>)))
void band_attn_kernel(Params prm) {
  constexpr bool kW3 = kIsW3<T, PERM, EPI, W3>;
  using Lay = Layout<T, D, PERM, kW3>;
  constexpr int kSegChunks = Lay::kSegChunks;  // chunks per sigma segment
  constexpr bool kPipe = !kW3 && PERM;  // scores of chunk c + 1 beside the softmax of chunk c
  constexpr bool kBf16 = Lay::kBf16;
  // At three waves per SIMD (d = 128: 168 registers) or four (d = 64: 128) the causal
  // sigma-gathered kernel recomputes the K/V LDS offsets at their use (from one base register
  // each) instead of holding them across the loop, and reads sigma for the causal mask in two
  // halves.  (Held offsets spilled 11 registers at d = 64 and four waves.)
  constexpr bool kLeanAny = kW3 && SIGMASK;
  constexpr bool kLean = kLeanAny;  // K/V LDS offsets
  constexpr bool kLeanMask = kLeanAny;
  __shared__ __attribute__((aligned(16))) char smem[Lay::kSmem];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)smem;  // LDS byte address of smem
  int* sig_lds = (int*)(smem + Lay::kSigOff);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps DMA setup scalar
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

  // ---- buffer resources of this (batch row, KV head) slice of K and V, and of sigma
  const int64_t kv_row_stride = (int64_t)prm.Hkv * Lay::kRowBytes;
  const int64_t kv_base = ((int64_t)b * n * prm.Hkv + g) * Lay::kRowBytes;
  const uint32_t kv_range = (uint32_t)((int64_t)(n - 1) * kv_row_stride + Lay::kRowBytes);
  const i32x4 rs_k = make_rsrc(prm.k + kv_base, kv_range);
  const i32x4 rs_v = make_rsrc(prm.v + kv_base, kv_range);
  const int32_t* sigma = prm.sigma + (b * prm.sig_bstride + g * prm.sig_hstride);
  const i32x4 rs_sig = make_rsrc(sigma, PERM ? (uint32_t)n * 4u : 0u);

  // sigma of keys [seg_key0, seg_key0 + 32 * nseg_chunks) into LDS (permuted operator only)
  auto dma_sigma = [&](int seg_key0, int nseg_chunks) {
    const int ninstr = (nseg_chunks * kChunk + 63) / 64;
    for (int j = wave; j < ninstr; j += kWaves) {
      const int key = seg_key0 + 64 * j + lane;
      dma4(rs_sig, __builtin_amdgcn_readfirstlane(smem_lds + Lay::kSigOff + 256 * j),
           key < n ? (uint32_t)key * 4u : kOutOfRange);
    }
  };

  // this wave's share of the K and V rows of a chunk: per DMA instruction, the chunk-relative key
  // this lane fetches and the byte offset of its (swizzled) source granule
  constexpr int kDW = Lay::kDmaPerWave;
  const uint32_t row_stride32 = (uint32_t)kv_row_stride;
  // row of instruction i: kRowsPerDma * blkid + lane / kGran, source granule lane % kGran
  auto dma_key_of = [&](int i, int ln) -> int {
    const int I = wave * kDW + i;  // wave-uniform
    const bool isv = I >= Lay::kDmaK;
    const int blkid = isv ? I - Lay::kDmaK : I;
    const int row = blkid * Lay::kRowsPerDma + ln / Lay::kGran;
    return isv ? row : row_to_key(row);
  };
  auto dma_goff_of = [&](int i, int ln) -> uint32_t {
    const int I = wave * kDW + i;
    const bool isv = I >= Lay::kDmaK;
    const int blkid = isv ? I - Lay::kDmaK : I;
    const int row = blkid * Lay::kRowsPerDma + ln / Lay::kGran;
    const int gran = ln % Lay::kGran;
    return (uint32_t)((gran ^ (isv ? swz_v<Lay::kGran>(row) : swz_k<Lay::kGran>(row))) * 16);
  };
  int dma_key[kDW];
  uint32_t dma_goff[kDW];
#pragma unroll
  for (int i = 0; i < kDW; ++i) {
    dma_key[i] = dma_key_of(i, lane);
    dma_goff[i] = dma_goff_of(i, lane);
  }
  // STAGE is a compile-time ring slot, so LDS addresses fold into instruction offsets.  The sigma
  // reads for all of this wave's rows go out first (unconditionally: the segment's sigma buffer
  // covers every key of its chunks), then the loads.
  struct DmaRows {
    int row[kDW];
  };
  auto dma_prep = [&](int kc0, int seg_key0) {
    DmaRows r;
#pragma unroll
    for (int i = 0; i < kDW; ++i) {
      const int q = kc0 + dma_key[i];
      r.row[i] = PERM ? sig_lds[q - seg_key0] : q;
    }
    return r;
  };
  // Row offsets are one 24-bit multiply-add (rows <= n < 2^24 - 32 and the row stride < 2^24 are
  // checked at the API).  Keys past the sequence end need no test: their row is >= n (the key
  // itself, or the sigma entry patched to n), which lies past the buffer range and reads zeros.
  auto dma_issue = [&](int kc0, auto stage_c, const DmaRows& r) {
    constexpr int STAGE = decltype(stage_c)::value;
#pragma unroll
    for (int i = 0; i < kDW; ++i) {
      const int I = wave * kDW + i;  // wave-uniform
      const bool isv = I >= Lay::kDmaK;
      const int blkid = isv ? I - Lay::kDmaK : I;
      const uint32_t voff = __umul24((uint32_t)r.row[i], row_stride32) +
                            dma_goff[i];
      const uint32_t lds = smem_lds + STAGE * Lay::kStageBytes + (isv ? Lay::kMatBytes : 0) +
                           blkid * 1024;
      dma16(isv ? rs_v : rs_k, __builtin_amdgcn_readfirstlane(lds), voff);
    }
  };
  // Gated SA pass (bf16): the intermediate rows this wave will add to are fetched into LDS while
  // its last chunk is processed.  Only that chunk's stage is still in use then, so waves 2j and
  // 2j + 1 take the two halves of the stage STAGE + 1 + j.  Instruction i brings the rows of the
  // wave's columns i * (1024 / RB) ..., lane l granule l % kGran of column i * (1024 / RB) +
  // l / kGran; granules are XOR-swizzled by column so the epilogue's reads spread over banks.
  // bf16 with a 4-slot ring: two chunks per loop step; the prologue then fetches one step
  constexpr bool kStep2 = kPipe && kBf16 && Lay::kNS == 4;
  constexpr int kPro = kStep2 ? 2 : Lay::kPF;
  // (needs kWaves / 2 ring stages besides the last chunk's)
  constexpr bool kPrefetchPartial =
      EPI == kEpiAddPartial && kBf16 && Lay::kNS - 1 >= (kWaves + 1) / 2;
  const int64_t out_batch_bytes = (int64_t)n * prm.Hq * D * (int)sizeof(T);
  const i32x4 rs_out =
      make_rsrc(prm.out + (int64_t)b * out_batch_bytes, (uint32_t)out_batch_bytes);
  auto partial_region = [&](int last_stage) {
    return ((last_stage + 1 + wave / 2) % Lay::kNS) * Lay::kStageBytes +
           (wave % 2) * Lay::kMatBytes;
  };
  // Whole rows of the wave's 32 columns from a [B, n, Hq, D] tensor (the intermediate in `out`,
  // or Q: both have that layout, so a column's row offset is out_off for either) into the
  // wave's 8 KB region next to ring slot last_stage.
  auto dma_rows = [&](const i32x4& rsrc, int last_stage, uint32_t my_row_off) {
    const uint32_t region = smem_lds + partial_region(last_stage);
    constexpr int kColsPerDma = 1024 / Lay::kRowBytes;
#pragma unroll
    for (int i = 0; i < Lay::kDmaK; ++i) {
      const int c = i * kColsPerDma + lane / Lay::kGran;  // wave-relative column
      const uint32_t base = (uint32_t)__builtin_amdgcn_ds_bpermute(c * 4, (int)my_row_off);
      const int gran = (lane % Lay::kGran) ^ (c & (Lay::kGran - 1));
      dma16(rsrc, __builtin_amdgcn_readfirstlane(region + 1024 * i), base + 16 * gran);
    }
  };
  auto dma_partial = [&](int last_stage, uint32_t my_out_off) {
    dma_rows(rs_out, last_stage, my_out_off);
  };
  // After a sigma segment has landed (and a barrier): the entries of keys past the sequence end
  // (read as 0 by the buffer range check) become n, so their K/V rows fall outside the buffers.
  // Only a segment that crosses the end does this, with one more barrier.
  auto patch_sigma_tail = [&](int seg_key0, int nseg_chunks) {
    const int key_end = seg_key0 + nseg_chunks * kChunk;
    if (key_end > n) {
      for (int key = n + tid; key < key_end; key += kThreads) sig_lds[key - seg_key0] = n;
      __syncthreads();
    }
  };
  auto dma_chunk = [&](int kc0, auto stage_c, int seg_key0) {
    dma_issue(kc0, stage_c, dma_prep(kc0, seg_key0));
  };

  // ---- prologue: sigma of the first segment and of this lane's slot, then Q
  const int nseg = (nchunks + kSegChunks - 1) / kSegChunks;
  int myorig = myslot;
  if constexpr (PERM) {
    dma_sigma(kbeg, min(nchunks, kSegChunks));
    myorig = sigma[myslot];
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (PERM) patch_sigma_tail(kbeg, min(nchunks, kSegChunks));
  // bf16: the wave's Q rows come in as whole rows by the same LDS DMA as K and V (one
  // instruction per 1 KB of contiguous rows instead of 32-byte pieces of 32 rows), into ring
  // slots that are free until the loop starts: kQSt slots hold the workgroup's rows, in the
  // region layout the epilogue uses.  The first kProEarly chunks go in flight before Q so the
  // loads overlap; with a 3-slot ring the remaining prologue chunk follows once Q has been read.
  constexpr int kQSt = (kWaves + 1) / 2;
  constexpr bool kQDma = kBf16 && Lay::kNS - 1 >= kQSt;
  constexpr int kProEarly = kQDma ? (kPro < Lay::kNS - kQSt ? kPro : Lay::kNS - kQSt) : kPro;
  static_for<kProEarly>([&](auto pf) {
    if (pf() < min(nchunks, kSegChunks)) dma_chunk(kbeg + pf() * kChunk, pf, kbeg);
  });

  const int64_t qrow_elems = (((int64_t)b * n + myorig) * prm.Hq + h) * D;
  // the gate is fetched now, with Q, instead of in the epilogue
  // A malformed sigma (an entry outside [0, n); sigma is trusted unless the caller asks for
  // validation) must not turn into a memory fault: such a column reads no gate or Q row and
  // stores nothing.  Its K/V row loads need no test, since buffer loads past the range read
  // zeros.
  const bool rowvalid = colvalid && (uint32_t)myorig < (uint32_t)n;
  const float gate_v =
      prm.gate && rowvalid ? prm.gate[((int64_t)b * n + myorig) * prm.Hq + h] : 1.0f;
  // byte offset of this column's output row within batch row b (the out buffer holds
  // n * Hq * D elements per batch row, < 2^31 bytes as checked at the API)
  const uint32_t out_off =
      rowvalid ? (uint32_t)(((int64_t)myorig * prm.Hq + h) * (D * (int)sizeof(T))) : kOutOfRange;
  constexpr int kQRegs = kBf16 ? D / 16 : D / 2;
  typedef typename std::conditional<kBf16, bf16x8, float>::type QFrag;
  QFrag qf[kQRegs];
  if constexpr (kQDma) {
    const i32x4 rs_q = make_rsrc(prm.q + (int64_t)b * out_batch_bytes, (uint32_t)out_batch_bytes);
    dma_rows(rs_q, kProEarly - 1, out_off);
    wait_vmcnt<0>();
    // column c's granule g sits at c * kRowBytes + 16 * (g ^ (c % kGran)); the B operand of
    // the score MFMA for d block kb is granule 2 kb + h32
    const int c = lane & 31;
    const char* qreg = smem + partial_region(kProEarly - 1) + c * Lay::kRowBytes;
#pragma unroll
    for (int kb = 0; kb < kQRegs; ++kb)
      qf[kb] = __builtin_bit_cast(
          bf16x8, *(const u32x4*)(qreg + 16 * ((2 * kb + h32) ^ (c & (Lay::kGran - 1)))));
    if constexpr (kProEarly < kPro) {
      __syncthreads();  // every wave has read its Q rows before the next chunk overwrites them
      static_for<kPro - kProEarly>([&](auto pf) {
        constexpr int kC = kProEarly + decltype(pf)::value;
        if (kC < min(nchunks, kSegChunks))
          dma_chunk(kbeg + kC * kChunk, std::integral_constant<int, kC>{}, kbeg);
      });
    }
  } else if constexpr (kBf16) {
    const char* qp = prm.q + (qrow_elems + 8 * h32) * 2;
#pragma unroll
    for (int kb = 0; kb < kQRegs; ++kb) {
      u32x4 raw = rowvalid ? *(const u32x4*)(qp + kb * 32) : u32x4{0, 0, 0, 0};
      qf[kb] = __builtin_bit_cast(bf16x8, raw);
    }
  } else {
    const char* qp = prm.q + (qrow_elems + h32 * (D / 2)) * 4;
#pragma unroll
    for (int t4 = 0; t4 < D / 8; ++t4) {
      f32x4 v4 = rowvalid ? *(const f32x4*)(qp + t4 * 16) : f32x4{0, 0, 0, 0};
      qf[4 * t4 + 0] = v4[0];
      qf[4 * t4 + 1] = v4[1];
      qf[4 * t4 + 2] = v4[2];
      qf[4 * t4 + 3] = v4[3];
    }
  }

  // Q (and with it the first chunks) must have landed before the loop: waiting here, where the
  // compiler sees it, keeps it from re-waiting for Q inside the loop.
  __builtin_amdgcn_s_waitcnt(0);

  // ---- accumulators
  constexpr int kOT = D / 32;
  f32x16 o[kOT];
#pragma unroll
  for (int t = 0; t < kOT; ++t) o[t] = zero16();
  float m_ref = -INFINITY;
  float l_run = 0.f;

  // ---- per-lane LDS offsets of the MFMA operands within a stage (the same for every chunk)
  const int r32 = lane & 31;
  constexpr int kKReads = kBf16 ? D / 16 : D / 8;  // 16-byte K reads per chunk
  int k_off[kLean ? 1 : kKReads];
  if constexpr (!kLean) {
#pragma unroll
    for (int u = 0; u < kKReads; ++u) {
      const int gran = kBf16 ? 2 * u + h32 : h32 * (D / 8) + u;
      k_off[u] = r32 * Lay::kRowBytes + ((gran ^ swz_k<Lay::kGran>(r32)) << 4);
    }
  }
  // kLean: the offset of d block u is k_base ^ (u << 5) (the granule 2u + h32 is XOR-swizzled
  // with r32 % kGran, and the u part of (2u + h32) ^ (r32 % kGran) lands in bits 5.. of the
  // offset); one opaque copy of k_base per chunk keeps the eight offsets out of registers.
  const int k_base = r32 * Lay::kRowBytes + ((h32 ^ swz_k<Lay::kGran>(r32)) << 4);
  // offset of K d block u given kbv = opaque(k_base) (kLean) or anything (otherwise)
  auto k_at = [&](int kbv, int u) -> int {
    if constexpr (kLean)
      return kbv ^ (u << 5);
    else
      return k_off[u];
  };
  // bf16: transposed V reads.  Lane j of 16-lane group grp reads 4 d-values of key
  // 16t + 8*h32 + j/4 (+4 for the upper half) at d = 32db + 16(grp%2) + 4(j%4); the tr16 read then
  // hands lane i of the group column i, i.e. the A operand row d = 32db + lane%32.  Key % 4 (and
  // so the swizzle) is the same for every (t, half), which only add 16t + 4*half rows: one base
  // offset per d block, the rest are instruction offsets.
  // kLean: v_off[db] = v_off[0] ^ (db << 6) (the d block enters the granule index as 4 db)
  int v_off[kLean ? 1 : kOT];
  if constexpr (kBf16) {
    const int grp = lane >> 4;
    const int j = lane & 15;
    const int dsub = 16 * (grp & 1) + 4 * (j & 3);
    const int key = 8 * h32 + (j >> 2);
#pragma unroll
    for (int db = 0; db < (kLean ? 1 : kOT); ++db) {
      const int d = 32 * db + dsub;
      v_off[db] = Lay::kMatBytes + key * Lay::kRowBytes +
                  (((d >> 3) ^ swz_v<Lay::kGran>(key)) << 4) + ((d & 7) << 1);
    }
  }

  // ---- one chunk of keys from ring stage `stage`
  // S^T[key rho(row)][col] = <K[key], Q[col]> for the chunk in ring slot STAGE
  auto compute_s = [&](auto stage_c) {
    constexpr int STAGE = decltype(stage_c)::value;
    const char* Kst = smem + STAGE * Lay::kStageBytes;
    f32x16 s = zero16();
    if constexpr (kBf16) {
      const int kbv = kLean ? opaque(k_base) : 0;
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(Kst + k_at(kbv, kb)));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kb], s, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < D / 8; ++u) {
        const f32x4 a4 = *(const f32x4*)(Kst + k_off[u]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[e], qf[4 * u + e], s, 0, 0, 0);
      }
    }
    return s;
  };

  // A chunk is interior for this wave when every key of it lies inside the band of every one of
  // the wave's slots (and before the sequence end): then only the causal sigma test remains.
  auto is_interior = [&](int c) {
    const int kc0 = kbeg + c * kChunk;
    return kc0 >= w_shi - L && kc0 + kChunk - 1 <= w_slo + R && kc0 + kChunk - 1 < n;
  };

  // Mask, online softmax and O^T += V^T P^T for chunk c (ring slot STAGE) given its scores.
  // INTERIOR selects the mask form (is_interior(c) must agree).
  auto softmax_pv = [&](int c, auto stage_c, auto interior_c, int seg_key0, const f32x16& s) {
    constexpr int STAGE = decltype(stage_c)::value;
    constexpr bool INTERIOR = decltype(interior_c)::value;
    const int kc0 = kbeg + c * kChunk;
    const char* Kst = smem + STAGE * Lay::kStageBytes;
    const char* Vst = Kst + Lay::kMatBytes;

    // mask.  Register r holds key kc0 + 16(r/8) + 8*h32 + r%8.
    int sk[16];
    if constexpr (SIGMASK) {
      const int* sp = sig_lds + (kc0 - seg_key0);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const u32x4 a = *(const u32x4*)(sp + 16 * half + 8 * h32);
        const u32x4 bq = *(const u32x4*)(sp + 16 * half + 8 * h32 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sk[8 * half + e] = (int)a[e];
          sk[8 * half + 4 + e] = (int)bq[e];
        }
      }
    }
    // masked raw scores; the max is taken before scaling (the scale is positive).  Branch-free:
    // interior chunks need only the causal test; edge chunks also test the lane's band, held as a
    // bit mask over the chunk's 32 key offsets.
    float sm[16];
    if constexpr (INTERIOR) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        bool ok = true;
        if constexpr (SIGMASK) ok = sk[r] <= myorig;
        sm[r] = ok ? s[r] : -INFINITY;
      }
    } else {
      const int a = max(max(myslot - L, 0) - kc0, 0);         // first valid offset (may be > 31)
      const int z = min(min(myslot + R, n - 1) - kc0, 31);     // last valid offset (may be < 0)
      const uint32_t upto = z < 0 ? 0u : (0xFFFFFFFFu >> (31 - z));
      const uint32_t from = a > 31 ? 0u : (0xFFFFFFFFu << a);
      const uint32_t bm = (upto & from) >> (8 * h32);          // bit 16(r/8) + r%8 for register r
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        bool ok = (bm >> (16 * (r >> 3) + (r & 7))) & 1u;
        if constexpr (SIGMASK) ok = ok & (sk[r] <= myorig);
        sm[r] = ok ? s[r] : -INFINITY;
      }
    }
    float mraw = sm[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mraw = fmaxf(mraw, sm[r]);
    mraw = pair_max(mraw);
    const float mx = mraw * prm.scale_log2;  // log2 units

    const bool need = mx > m_ref + kLazy;
    // O is still exactly zero while the reference is -inf (every earlier key was masked), so the
    // first raise of the reference needs no rescale
    const bool rescale = need && m_ref != -INFINITY;
    const float m_new = need ? mx : m_ref;
    const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
    m_ref = m_new;
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sm[r], prm.scale_log2, -m_use));
    if (__ballot(rescale)) {
#pragma unroll
      for (int t = 0; t < kOT; ++t) o[t] *= alpha;
    }

    // O^T[d][col] += V^T[d][key] P^T[key][col]
    if constexpr (kBf16) {
      bf16x8 pb[2];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[0][e] = (__bf16)p[e];
        pb[1][e] = (__bf16)p[8 + e];
      }
      // The row sum is taken over the bf16-rounded weights that enter the P*V product, so the
      // output is an exact convex combination of V rows with (slightly perturbed) weights.
      float psum = 0.f;
      const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[0][e], pb[0][e + 1]}, one2, psum, false);
        psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[1][e], pb[1][e + 1]}, one2, psum, false);
      }
      l_run = l_run * alpha + psum;
      const SSW_LDS char* vbase = (const SSW_LDS char*)Kst;
      const int vbv = kLean ? opaque(v_off[0]) : 0;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int db = 0; db < kOT; ++db) {
          const int vo = kLean ? (vbv ^ (db << 6)) : v_off[db];
          const SSW_LDS char* vp = vbase + vo + 16 * t * Lay::kRowBytes;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SSW_LDS s16x4*)vp);
          const s16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((SSW_LDS s16x4*)(vp + 4 * Lay::kRowBytes));
          // whole-vector casts only: building the operand element by element from the 16-bit
          // lanes was miscompiled (only the first dword of each read survived)
          const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
          const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[t], o[db], 0, 0, 0);
        }
      }
    } else {
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) psum += p[r];
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 16 * (r >> 3) + 8 * h32 + (r & 7);
        const char* vrow = Vst + key * Lay::kRowBytes;
#pragma unroll
        for (int t = 0; t < kOT; ++t) {
          const int d = 32 * t + r32;
          const float vv = *(const float*)(vrow + (((d >> 2) ^ swz_v<Lay::kGran>(key)) << 4) +
                                           ((d & 3) << 2));
          o[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv, p[r], o[t], 0, 0, 0);
        }
      }
    }
  };

  // bf16: softmax and P*V of chunk c (ring slot STAGE) fused with the scores of the next chunk
  // (ring slot NEXT), which are returned.  The next chunk's MFMAs do not depend on this chunk's
  // softmax, so they are issued inside the straight-line stretch between the mask and the lazy
  // rescale branch, where the scheduler can interleave them with the column max and the first
  // half of the exponentials.  Every step's arithmetic is that of compute_s and softmax_pv.
  // The mask form is a runtime (uniform) branch that only produces sm[], so O keeps one set of
  // registers on every path.
  auto fused_step = [&](int c, auto stage_c, auto next_c, bool interior, int seg_key0,
                        const f32x16& s) {
    constexpr int STAGE = decltype(stage_c)::value;
    constexpr int NEXT = decltype(next_c)::value;
    f32x16 sn = zero16();
    if constexpr (kBf16) {
      const int kc0 = kbeg + c * kChunk;
      const char* Kst = smem + STAGE * Lay::kStageBytes;
      const char* Kn = smem + (NEXT >= 0 ? NEXT : 0) * Lay::kStageBytes;

      float sm[16];
      if constexpr (kLeanMask && SIGMASK) {
        // Register r holds key kc0 + 16(r/8) + 8*h32 + r%8.  sigma is read and applied in two
        // halves of 8 keys, with a scheduling barrier between them, so that at most 8 sigma
        // values are live; an edge chunk also tests the lane's band bits.
        const int* sp = sig_lds + (kc0 - seg_key0);
        uint32_t band16 = 0xFFFFu;
        if (!interior) {
          const int a = max(max(myslot - L, 0) - kc0, 0);
          const int z = min(min(myslot + R, n - 1) - kc0, 31);
          const uint32_t upto = z < 0 ? 0u : (0xFFFFFFFFu >> (31 - z));
          const uint32_t from = a > 31 ? 0u : (0xFFFFFFFFu << a);
          const uint32_t bm = (upto & from) >> (8 * h32);
          band16 = (bm & 0xFFu) | ((bm >> 8) & 0xFF00u);
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const u32x4 a4 = *(const u32x4*)(sp + 16 * half + 8 * h32);
          const u32x4 b4 = *(const u32x4*)(sp + 16 * half + 8 * h32 + 4);
          if (interior) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sm[8 * half + e] = (int)a4[e] <= myorig ? s[8 * half + e] : -INFINITY;
              sm[8 * half + 4 + e] = (int)b4[e] <= myorig ? s[8 * half + 4 + e] : -INFINITY;
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r0 = 8 * half + e, r1 = 8 * half + 4 + e;
              sm[r0] = ((int)a4[e] <= myorig && ((band16 >> r0) & 1u)) ? s[r0] : -INFINITY;
              sm[r1] = ((int)b4[e] <= myorig && ((band16 >> r1) & 1u)) ? s[r1] : -INFINITY;
            }
          }
          if (half == 0) __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        // mask.  Register r holds key kc0 + 16(r/8) + 8*h32 + r%8.  The causal test folds into a
        // 16-bit mask as sigma is read, so no sigma value stays live in a register.
        uint32_t cm = 0xFFFFu;
        if constexpr (SIGMASK) {
          const int* sp = sig_lds + (kc0 - seg_key0);
          cm = 0u;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const u32x4 a = *(const u32x4*)(sp + 16 * half + 8 * h32);
            const u32x4 bq = *(const u32x4*)(sp + 16 * half + 8 * h32 + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              cm |= (uint32_t)((int)a[e] <= myorig) << (8 * half + e);
              cm |= (uint32_t)((int)bq[e] <= myorig) << (8 * half + 4 + e);
            }
          }
        }
        if (interior) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sm[r] = ((cm >> r) & 1u) ? s[r] : -INFINITY;
        } else {
          const int a = max(max(myslot - L, 0) - kc0, 0);
          const int z = min(min(myslot + R, n - 1) - kc0, 31);
          const uint32_t upto = z < 0 ? 0u : (0xFFFFFFFFu >> (31 - z));
          const uint32_t from = a > 31 ? 0u : (0xFFFFFFFFu << a);
          const uint32_t bm = (upto & from) >> (8 * h32);
          // band bit of register r is bit 16(r/8) + r%8 of bm; keep both tests in one mask
          const uint32_t band16 = (bm & 0xFFu) | ((bm >> 8) & 0xFF00u);
          const uint32_t all = band16 & cm;
#pragma unroll
          for (int r = 0; r < 16; ++r) sm[r] = ((all >> r) & 1u) ? s[r] : -INFINITY;
        }
      }

      // scores of the next chunk, interleaved with the column max and the first weights
      if constexpr (NEXT >= 0) {
        const int kbv = kLean ? opaque(k_base) : 0;
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(Kn + k_at(kbv, kb)));
          sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kb], sn, 0, 0, 0);
        }
      }
      float mraw = sm[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mraw = fmaxf(mraw, sm[r]);
      mraw = pair_max(mraw);
      const float mx = mraw * prm.scale_log2;
      const bool need = mx > m_ref + kLazy;
      // O is still exactly zero while the reference is -inf (every earlier key was masked), so
      // the first raise of the reference needs no rescale
      const bool rescale = need && m_ref != -INFINITY;
      const float m_new = need ? mx : m_ref;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
      m_ref = m_new;
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sm[r], prm.scale_log2, -m_use));
      bf16x8 pb[2];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[0][e] = (__bf16)p[e];
        pb[1][e] = (__bf16)p[8 + e];
      }
      if (__ballot(rescale)) {
#pragma unroll
        for (int t = 0; t < kOT; ++t) o[t] *= alpha;
      }
      float psum = 0.f;
      const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[0][e], pb[0][e + 1]}, one2, psum, false);
        psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[1][e], pb[1][e + 1]}, one2, psum, false);
      }
      l_run = l_run * alpha + psum;
      const SSW_LDS char* vbase = (const SSW_LDS char*)Kst;
      const int vbv = kLean ? opaque(v_off[0]) : 0;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int db = 0; db < kOT; ++db) {
          const int vo = kLean ? (vbv ^ (db << 6)) : v_off[db];
          const SSW_LDS char* vp = vbase + vo + 16 * t * Lay::kRowBytes;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SSW_LDS s16x4*)vp);
          const s16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((SSW_LDS s16x4*)(vp + 4 * Lay::kRowBytes));
          const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
          const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[t], o[db], 0, 0, 0);
        }
      }
    }
    return sn;
  };


  // bf16, two chunks per step: chunks ca and ca + 1 in ring slots STA and STA + 1 (hb: the second
  // chunk exists).  Scores of both chunks (two independent MFMA chains), both masks, one column
  // max and one lazy-reference check for the 64 keys, then P*V for both.  Per chunk the arithmetic
  // is that of compute_s and softmax_pv.
  auto mask16 = [&](int c, bool interior, int seg_key0, const f32x16& s, float* sm) {
    const int kc0 = kbeg + c * kChunk;
    int sk[16];
    if constexpr (SIGMASK) {
      const int* sp = sig_lds + (kc0 - seg_key0);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const u32x4 a = *(const u32x4*)(sp + 16 * half + 8 * h32);
        const u32x4 bq = *(const u32x4*)(sp + 16 * half + 8 * h32 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sk[8 * half + e] = (int)a[e];
          sk[8 * half + 4 + e] = (int)bq[e];
        }
      }
    }
    if (interior) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        bool ok = true;
        if constexpr (SIGMASK) ok = sk[r] <= myorig;
        sm[r] = ok ? s[r] : -INFINITY;
      }
    } else {
      const int a = max(max(myslot - L, 0) - kc0, 0);
      const int z = min(min(myslot + R, n - 1) - kc0, 31);
      const uint32_t upto = z < 0 ? 0u : (0xFFFFFFFFu >> (31 - z));
      const uint32_t from = a > 31 ? 0u : (0xFFFFFFFFu << a);
      const uint32_t bm = (upto & from) >> (8 * h32);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        bool ok = (bm >> (16 * (r >> 3) + (r & 7))) & 1u;
        if constexpr (SIGMASK) ok = ok & (sk[r] <= myorig);
        sm[r] = ok ? s[r] : -INFINITY;
      }
    }
  };
  auto step2 = [&](int ca, auto sta_c, bool hb, bool int_a, bool int_b, int seg_key0) {
    constexpr int STA = decltype(sta_c)::value;
    if constexpr (kBf16) {
      const char* Ka = smem + STA * Lay::kStageBytes;
      const char* Kb = smem + (STA + 1) * Lay::kStageBytes;
      f32x16 s_a = zero16(), s_b = zero16();
      const int kbv = kLean ? opaque(k_base) : 0;
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(Ka + k_at(kbv, kb)));
        s_a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kb], s_a, 0, 0, 0);
      }
      if (hb) {
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(Kb + k_at(kbv, kb)));
          s_b = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kb], s_b, 0, 0, 0);
        }
      }
      float sm[32];
      mask16(ca, int_a, seg_key0, s_a, sm);
      if (hb) {
        mask16(ca + 1, int_b, seg_key0, s_b, sm + 16);
      } else {
#pragma unroll
        for (int r = 16; r < 32; ++r) sm[r] = -INFINITY;
      }
      float mraw = sm[0];
#pragma unroll
      for (int r = 1; r < 32; ++r) mraw = fmaxf(mraw, sm[r]);
      mraw = pair_max(mraw);
      const float mx = mraw * prm.scale_log2;
      const bool need = mx > m_ref + kLazy;
      // O is still exactly zero while the reference is -inf (every earlier key was masked), so
      // the first raise of the reference needs no rescale
      const bool rescale = need && m_ref != -INFINITY;
      const float m_new = need ? mx : m_ref;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
      m_ref = m_new;
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      bf16x8 pb[4];
#pragma unroll
      for (int r = 0; r < 32; ++r)
        pb[r >> 3][r & 7] =
            (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sm[r], prm.scale_log2, -m_use));
      if (__ballot(rescale)) {
#pragma unroll
        for (int t = 0; t < kOT; ++t) o[t] *= alpha;
      }
      // The row sum is taken over the bf16-rounded weights that enter the P*V product.
      float psum = 0.f;
      const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[t][e], pb[t][e + 1]}, one2, psum, false);
      l_run = l_run * alpha + psum;
      auto pv = [&](const char* Kst, const bf16x8* pbc) {
        const SSW_LDS char* vbase = (const SSW_LDS char*)Kst;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int db = 0; db < kOT; ++db) {
            const SSW_LDS char* vp =
                vbase + (kLean ? (opaque(v_off[0]) ^ (db << 6)) : v_off[db]) + 16 * t * Lay::kRowBytes;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SSW_LDS s16x4*)vp);
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (SSW_LDS s16x4*)(vp + 4 * Lay::kRowBytes));
            const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
            const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
            const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pbc[t], o[db], 0, 0, 0);
          }
        }
      };
      pv(Ka, pb);
      if (hb) pv(Kb, pb + 2);
    }
  };

  // ---- main loop over segments of at most kSegChunks chunks (one segment in practice)
  for (int sg = 0; sg < nseg; ++sg) {
    const int c0 = sg * kSegChunks;
    const int segc = min(kSegChunks, nchunks - c0);
    const int seg_key0 = kbeg + c0 * kChunk;
    if (sg > 0) {
      // drain the previous segment, bring in this one's sigma, then its first chunks
      wait_vmcnt<0>();
      __syncthreads();
      if constexpr (PERM) {
        dma_sigma(seg_key0, segc);
        wait_vmcnt<0>();
        __syncthreads();
        patch_sigma_tail(seg_key0, segc);
      }
      static_for<kPro>([&](auto pf) {
        if (pf() < segc) dma_chunk(seg_key0 + pf() * kChunk, pf, seg_key0);
      });
    }

    if constexpr (kStep2) {
      // Steps of two chunks: step i uses ring slots 2i % 4 and 2i % 4 + 1; after its barrier
      // (step i - 1 consumed) the next step's two chunks are fetched into step i - 1's slots.
      auto active = [&](int c) { return wave_on && c >= c_first && c <= c_last; };
      const int nsteps = (segc + 1) / 2;
      for (int st0 = 0; st0 < nsteps; st0 += 2) {
        static_for<2>([&](auto par) {
          const int st = st0 + par();
          if (st < nsteps) {
            constexpr int kSlot = 2 * par();
            constexpr int kFetchSlot = 2 * (1 - par());
            const int ca = 2 * st;
            const bool hb = ca + 1 < segc;
            const bool fetch_a = ca + 2 < segc;
            const bool fetch_b = ca + 3 < segc;
            // rows of the next step's chunks (read for a chunk inside the segment even when
            // nothing is fetched, so that the row registers need no other definition)
            const DmaRows ra = dma_prep(seg_key0 + min(ca + 2, segc - 1) * kChunk, seg_key0);
            const DmaRows rb = dma_prep(seg_key0 + min(ca + 3, segc - 1) * kChunk, seg_key0);
            wait_vmcnt<0>();  // this step's chunks (the only loads in flight)
            __syncthreads();  // and every wave's; the previous step's slots are free
            if (fetch_a)
              dma_issue(seg_key0 + (ca + 2) * kChunk, std::integral_constant<int, kFetchSlot>{}, ra);
            if (fetch_b)
              dma_issue(seg_key0 + (ca + 3) * kChunk,
                        std::integral_constant<int, kFetchSlot + 1>{}, rb);
            if constexpr (kPrefetchPartial)
              if (sg == nseg - 1 && st == nsteps - 1 && wave_on)
                dma_partial(hb ? kSlot + 1 : kSlot, out_off);
            if (active(c0 + ca) || (hb && active(c0 + ca + 1)))
              step2(c0 + ca, std::integral_constant<int, kSlot>{}, hb, is_interior(c0 + ca),
                    hb && is_interior(c0 + ca + 1), seg_key0);
          }
        });
      }
    } else if constexpr (kPipe) {
    // Software pipeline: while chunk cs is consumed (softmax + P*V from its V), the scores of
    // chunk cs + 1 are already computed from its K, so each wave has independent MFMA work to
    // overlap with the softmax VALU work.  Chunk cs + kPF is fetched meanwhile.
    auto active = [&](int c) { return wave_on && c >= c_first && c <= c_last; };
    if (Lay::kPF - 1 < segc)
      wait_vmcnt<Lay::kDmaPerWave * (Lay::kPF - 1)>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    f32x16 s_cur = zero16();
    if (active(c0)) s_cur = compute_s(std::integral_constant<int, 0>{});

    // unrolled by the ring depth so that every chunk's ring slot is a compile-time constant
    for (int cs0 = 0; cs0 < segc; cs0 += Lay::kNS) {
      static_for<Lay::kNS>([&](auto u) {
        const int cs = cs0 + u();
        if (cs < segc) {
          constexpr int kNext = (u() + 1) % Lay::kNS;
          constexpr int kFetch = (u() + Lay::kPF) % Lay::kNS;
          const bool fetch = cs + Lay::kPF < segc;
          DmaRows rows;
          if (fetch) rows = dma_prep(seg_key0 + (cs + Lay::kPF) * kChunk, seg_key0);
          // chunk cs + 1 must have landed: at most (kPF - 2) younger chunks of this wave's DMAs
          // may still be outstanding; near the end, wait for everything
          if (cs + Lay::kPF - 1 < segc)
            wait_vmcnt<Lay::kDmaPerWave * (Lay::kPF - 2)>();
          else
            wait_vmcnt<0>();
          __syncthreads();  // every wave's DMAs for chunk cs + 1 landed; chunk cs - 1 consumed
          if (fetch)
            dma_issue(seg_key0 + (cs + Lay::kPF) * kChunk, std::integral_constant<int, kFetch>{},
                      rows);
          if constexpr (kPrefetchPartial)
            if (sg == nseg - 1 && cs == segc - 1 && wave_on) dma_partial(u(), out_off);
          // bf16: one code path for every chunk a wave touches (a chunk outside the wave's band is
          // fully masked by the edge form and adds nothing; the scores computed past the last
          // chunk are discarded).  fp32: scores and softmax as separate steps.
          const bool act_cur = active(c0 + cs);
          const bool act_next = cs + 1 < segc && active(c0 + cs + 1);
          using Next = std::integral_constant<int, kNext>;
          using Edge = std::false_type;
          using Inner = std::true_type;
          f32x16 s_next = zero16();
          if constexpr (kBf16) {
            if (act_cur || act_next)
              s_next = fused_step(c0 + cs, u, Next{}, is_interior(c0 + cs), seg_key0, s_cur);
          } else {
            if (act_next) s_next = compute_s(Next{});
            if (act_cur) {
              if (is_interior(c0 + cs))
                softmax_pv(c0 + cs, u, Inner{}, seg_key0, s_cur);
              else
                softmax_pv(c0 + cs, u, Edge{}, seg_key0, s_cur);
            }
          }
          s_cur = s_next;
        }
      });
    }
    } else {
    // Chunk cs is consumed in iteration cs (scores, softmax, P*V) while chunks cs + 1 .. cs + kPF
    // are in flight; the fetch of chunk cs + kPF reuses the slot of chunk cs - 1.
    auto active = [&](int c) { return wave_on && c >= c_first && c <= c_last; };
    // unrolled by the ring depth so that every chunk's ring slot is a compile-time constant
    for (int cs0 = 0; cs0 < segc; cs0 += Lay::kNS) {
      static_for<Lay::kNS>([&](auto u) {
        const int cs = cs0 + u();
        if (cs < segc) {
          constexpr int kFetch = (u() + Lay::kPF) % Lay::kNS;
          const bool fetch = cs + Lay::kPF < segc;
          DmaRows rows;
          if (fetch) rows = dma_prep(seg_key0 + (cs + Lay::kPF) * kChunk, seg_key0);
          // chunk cs must have landed: at most kPF - 1 younger chunks of this wave's DMAs may
          // still be outstanding; near the end, wait for everything
          if (cs + Lay::kPF - 1 < segc)
            wait_vmcnt<Lay::kDmaPerWave * (Lay::kPF - 1)>();
          else
            wait_vmcnt<0>();
          __syncthreads();  // every wave's DMAs for chunk cs landed; chunk cs - 1 consumed
          if (fetch)
            dma_issue(seg_key0 + (cs + Lay::kPF) * kChunk, std::integral_constant<int, kFetch>{},
                      rows);
          if constexpr (kPrefetchPartial)
            if (sg == nseg - 1 && cs == segc - 1 && wave_on) dma_partial(u(), out_off);
          if (active(c0 + cs)) {
            const f32x16 sc = compute_s(u);
            if constexpr (kBf16) {
              fused_step(c0 + cs, u, std::integral_constant<int, -1>{}, is_interior(c0 + cs),
                         seg_key0, sc);
            } else {
              if (is_interior(c0 + cs))
                softmax_pv(c0 + cs, u, std::true_type{}, seg_key0, sc);
              else
                softmax_pv(c0 + cs, u, std::false_type{}, seg_key0, sc);
            }
          }
        }
      });
    }
    }
  }

  // ---- epilogue: normalise, gate, scatter to original row sigma[p]
  const float l_tot = pair_sum(l_run);
  if (!wave_on) return;
  // The row's log-sum-exp for a backward pass.  Every row holds its own token, so m_ref is finite
  // and l_tot >= 1 here; l_tot sums exp2 of the scaled scores minus m_ref.
  if (prm.lse && h32 == 0 && rowvalid)
    prm.lse[((int64_t)b * n + myorig) * prm.Hq + h] =
        (m_ref + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  const float f = __builtin_amdgcn_rcpf(l_tot) * gate_v;
  if constexpr (kBf16) {
    // The wave's 32 finished rows are assembled in its own 8 KB of LDS: a ring stage that the
    // last loop step does not read (the slice the gated SA pass prefetched its intermediate rows
    // into), same swizzled row layout.  Each lane turns its register fragments into 16-bit words
    // in place; the rows then leave as whole 16-byte granules, kGran lanes per row, so a store
    // instruction writes 64 / kGran complete rows instead of 16 bytes of each of 32 rows.
    const int segc_last = nchunks - (nseg - 1) * kSegChunks;
    char* reg = smem + partial_region((segc_last - 1) % Lay::kNS);
    char* rowp = reg + (lane & 31) * Lay::kRowBytes;
    if constexpr (kPrefetchPartial) wait_vmcnt<0>();
#pragma unroll
    for (int t = 0; t < kOT; ++t) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * t + 8 * a + 4 * h32;
        // granule d0 / 8 of the row, swizzled by column; bytes 8 * h32 within it
        u32x2* slot = (u32x2*)(rowp + 16 * ((d0 >> 3) ^ ((lane & 31) & (Lay::kGran - 1))) +
                               8 * h32);
        // (the intermediate's 2^-4 is a power of two: folded into the factor, it rounds the same)
        const float fs = EPI == kEpiPartial ? f * kPartialScale : f;
        f32x2 y[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) y[u] = f32x2{o[t][4 * a + 2 * u] * fs, o[t][4 * a + 2 * u + 1] * fs};
        uint32_t w[2];
        if constexpr (EPI == kEpiPartial) {
          // the gated intermediate: fp16 of y * 2^-4, one packed conversion per pair
#pragma unroll
          for (int u = 0; u < 2; ++u)
            w[u] = __builtin_bit_cast(uint32_t, __builtin_convertvector(y[u], f16x2));
        } else {
          if constexpr (EPI == kEpiAddPartial) {
            static_assert(kPrefetchPartial, "bf16 intermediate rows come through the ring");
            const u32x2 old = *slot;
            // whole-vector casts only: taking the two halves of `old` element by element
            // (then a per-element cast to fp16 pairs) was miscompiled into one 4-byte read
            const f32x4 p = __builtin_convertvector(__builtin_bit_cast(f16x4, old), f32x4);
#pragma unroll
            for (int u = 0; u < 2; ++u)
              y[u] = f32x2{__builtin_fmaf(p[2 * u], kPartialUnscale, y[u][0]),
                           __builtin_fmaf(p[2 * u + 1], kPartialUnscale, y[u][1])};
          }
#pragma unroll
          for (int u = 0; u < 2; ++u)
            w[u] = __builtin_bit_cast(uint32_t, __builtin_convertvector(y[u], bf16x2));
        }
        *slot = u32x2{w[0], w[1]};
      }
    }
    // the rows are read back by other lanes of this wave: its LDS writes must have completed
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    char* obatch = prm.out + (int64_t)b * out_batch_bytes;
    constexpr int kRowsPerStore = 64 / Lay::kGran;
    // the lane index is made opaque here so that the row indices below are recomputed: shared
    // with the identical ones of the prologue's Q row fetch, they stayed live across the loop
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
#pragma unroll
    for (int i = 0; i < 32 / kRowsPerStore; ++i) {
      const int r = i * kRowsPerStore + lane_e / Lay::kGran;  // wave-relative column
      const int gran = lane_e % Lay::kGran;
      const uint32_t roff = (uint32_t)__builtin_amdgcn_ds_bpermute(r * 4, (int)out_off);
      const u32x4 v =
          *(const u32x4*)(reg + r * Lay::kRowBytes + 16 * (gran ^ (r & (Lay::kGran - 1))));
      if (roff != kOutOfRange) *(u32x4*)(obatch + roff + 16 * gran) = v;
    }
  } else {
    if (!rowvalid) return;
    char* orow = prm.out + qrow_elems * (int64_t)sizeof(T);
#pragma unroll
    for (int t = 0; t < kOT; ++t) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * t + 8 * a + 4 * h32;
        float y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) y[u] = o[t][4 * a + u] * f;
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
template <typename T, int D, bool PERM, bool SIGMASK, int EPI, bool W3 = false>
static hipError_t launch_t(const Params& prm, hipStream_t stream, void* ev_start, void* ev_stop) {
  if (ev_start || ev_stop) {
    hipExtLaunchKernelGGL((band_attn_kernel<T, D, PERM, SIGMASK, EPI, W3>), dim3(prm.nblocks),
                          dim3(kThreads), 0, stream, (hipEvent_t)ev_start, (hipEvent_t)ev_stop, 0,
                          prm);
  } else {
    hipLaunchKernelGGL((band_attn_kernel<T, D, PERM, SIGMASK, EPI, W3>), dim3(prm.nblocks),
                       dim3(kThreads), 0, stream, prm);
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_d(const BandLaunch& a, const Params& prm, hipStream_t s) {
  void* e0 = a.ev_start;
  void* e1 = a.ev_stop;
  // The gated layer runs its SA pass first, which leaves the intermediate (kEpiPartial), and its
  // SWA pass second, which adds to it (kEpiAddPartial); everything else stores plainly.
  if (a.perm) {
    const bool part = a.epilogue == kEpiPartial;
    // The W3 build (bf16; three or four waves per SIMD) when a workgroup's band, at most
    // ceil(kColsWG / G) + 1 slots plus L + R keys, fits its 1024-entry sigma segment.
    const int64_t band = (kColsWG + prm.G - 1) / prm.G + 1 + (int64_t)prm.L + prm.R;
    if constexpr (sizeof(T) == 2) {
      if (band <= kSigCapW3) {
        if (a.causal)
          return part ? launch_t<T, D, true, true, kEpiPartial, true>(prm, s, e0, e1)
                      : launch_t<T, D, true, true, kEpiStore, true>(prm, s, e0, e1);
        return part ? launch_t<T, D, true, false, kEpiPartial, true>(prm, s, e0, e1)
                    : launch_t<T, D, true, false, kEpiStore, true>(prm, s, e0, e1);
      }
    }
    if (a.causal)
      return part ? launch_t<T, D, true, true, kEpiPartial>(prm, s, e0, e1)
                  : launch_t<T, D, true, true, kEpiStore>(prm, s, e0, e1);
    return part ? launch_t<T, D, true, false, kEpiPartial>(prm, s, e0, e1)
                : launch_t<T, D, true, false, kEpiStore>(prm, s, e0, e1);
  }
  return a.epilogue == kEpiAddPartial
             ? launch_t<T, D, false, false, kEpiAddPartial>(prm, s, e0, e1)
             : launch_t<T, D, false, false, kEpiStore>(prm, s, e0, e1);
}

hipError_t launch_band_attn(const BandLaunch& a, hipStream_t stream) {
  Params prm;
  prm.q = (const char*)a.q;
  prm.k = (const char*)a.k;
  prm.v = (const char*)a.v;
  prm.sigma = a.sigma;
  prm.sig_bstride = a.sig_bstride;
  prm.sig_hstride = a.sig_hstride;
  prm.gate = a.gate;
  prm.out = (char*)a.out;
  prm.lse = a.lse;
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
  prm.ntiles = (int)((ncols + kColsWG - 1) / kColsWG);
  prm.nblocks = prm.ntiles * a.B * a.Hkv;
  if (a.dtype == 1) {
    return a.d == 128 ? launch_d<__bf16, 128>(a, prm, stream)
                      : launch_d<__bf16, 64>(a, prm, stream);
  }
  return a.d == 128 ? launch_d<float, 128>(a, prm, stream) : launch_d<float, 64>(a, prm, stream);
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
