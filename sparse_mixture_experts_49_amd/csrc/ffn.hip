// Grouped expert FFN of the MoE layer on gfx950.
//
// Each expert is Linear(d -> d_ff) -> GELU -> Linear(d_ff -> d) (web page
// "Mixture of Experts: Scaling Parameters Without Scaling Compute", section
// "The MoE layer", the listing's expert).  After dispatch the rows of expert e
// are the contiguous segment [offsets[e], offsets[e+1]) of A, so each expert is
// one dense product out[seg] = A[seg] W_e^T (+ bias_e) with W_e stored
// [N][K] (K contiguous, like A).  Experts with no rows do no work.
//
// Three kernels, chosen on the host from a bound on rows per expert (the
// device-side counts are never read back):
//   * ffn_tiled_kernel  -- many rows per expert: 256 x 256 (or x 128) output
//     tiles for prefill, 128-row tiles from 64 rows per expert; both
//     operands loaded straight into LDS in 64-wide k-steps, bf16 MFMA 32x32x16
//     with fp32 accumulation, pipelined with one barrier per k-step, XCD-aware
//     tile order.  Each block finds its expert from `offsets`.
//   * ffn_stream_kernel -- few rows per expert (decode, many small experts):
//     each wave streams its own 16*NWN rows of W_e straight from HBM into
//     registers in the MFMA operand layout, while the block's (at most
//     16*NMT) rows of A are staged through LDS once per k-chunk and shared by
//     the four waves.  Weight bytes are read once.
//   * ffn_stream_lds_kernel -- the same blocks for bf16 layers with at most 32
//     rows per expert, both operands staged through LDS by DMA in whole 512 B
//     runs of each row, one persistent block per CU.
// The first product applies bias + exact-erf GELU in its epilogue and stores
// dtype h; the second adds its bias and stores fp32 o.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "../../include/moe_mi355x.h"

namespace moe {

// Every expert's rows cut into ceil(count/BM) m-tiles laid end to end, one
// expert per lane (E <= 64): lane e holds its rows [lo, hi), its m-tile count
// and the index of its first m-tile; `total` (uniform) counts them all.  One
// vector load per lane and a wave-wide prefix sum, not a loop of dependent
// loads over the experts.  Every lane of the wave must take part.
struct MTiles {
  int lo, hi, nt, first;   // this lane's expert (0 past E)
  int total;               // m-tiles over all experts
};

template <int BM>
__device__ __forceinline__ MTiles mtiles(const int32_t* __restrict__ offsets, int E) {
  const int lane = __lane_id();
  MTiles m;
  m.lo = lane < E ? offsets[lane] : 0;
  m.hi = lane < E ? offsets[lane + 1] : 0;
  m.nt = (m.hi - m.lo + BM - 1) / BM;
  int incl = m.nt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  m.first = incl - m.nt;
  m.total = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
  return m;
}

// The expert owning global m-tile `mt` (uniform) and the tile's rows: the lane
// whose range of m-tiles holds it.  Returns false past the last tile.
template <int BM>
__device__ __forceinline__ bool find_mtile(const MTiles& m, int mt, int& e_out, int& r0, int& r1) {
  const uint64_t own = __ballot(mt >= m.first && mt < m.first + m.nt);
  if (!own) return false;
  const int e = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)own) - 1);
  e_out = e;
  r0 = __builtin_amdgcn_readfirstlane(__shfl(m.lo + (mt - m.first) * BM, e));
  r1 = min(__builtin_amdgcn_readfirstlane(__shfl(m.hi, e)), r0 + BM);
  return true;
}

// Rows of A holding dispatched rows r[0..n): r itself, or -- when the first
// product reads the tokens straight from x -- the token of assignment
// gather[r] (gather = the dispatch's src array, gather_k = top_k).  Every
// index load is issued before any is used (one wait, not one per row; the
// null test is uniform), and the division is unsigned (indices are >= 0).
template <int n>
__device__ __forceinline__ void a_rows(const int32_t* __restrict__ gather, int gather_k, int (&r)[n]) {
  if (!gather) return;
  int32_t g[n];
#pragma unroll
  for (int i = 0; i < n; ++i) g[i] = gather[r[i]];
  const uint32_t k = (uint32_t)gather_k;
#pragma unroll
  for (int i = 0; i < n; ++i) r[i] = (int)((uint32_t)g[i] / k);
}

template <typename T, bool UP>
__device__ __forceinline__ void store_out(void* out, size_t idx, float v) {
  if constexpr (UP) {
    const float g = gelu_erf(v);
    if constexpr (sizeof(T) == 2)
      static_cast<uint16_t*>(out)[idx] = f32_to_bf16(g);
    else
      static_cast<float*>(out)[idx] = g;
  } else {
    static_cast<float*>(out)[idx] = v;
  }
}

// One finished pre-activation (bias included) of the stream path: the first
// product stores GELU of it (as dtype, or as bf16 hi + lo planes when h is
// split), the second stores it as fp32.
template <typename T, bool UP, bool SPLIT>
__device__ __forceinline__ void emit(void* out, size_t out_plane, size_t idx, float v) {
  if constexpr (UP && SPLIT) {
    const float g = gelu_erf(v);
    const uint16_t hi = f32_to_bf16(g);
    const uint16_t lo = f32_to_bf16(g - bf16_to_f32(hi));
    static_cast<uint16_t*>(out)[idx] = hi;
    static_cast<uint16_t*>(out)[out_plane + idx] = lo;
  } else {
    store_out<T, UP>(out, idx, v);
  }
}

// ---------------------------------------------------------------------------
// LDS-tiled kernel (bf16).  Block tile 256 (rows of one expert) x BN (output
// columns), k-steps of 64.  NW = 4 waves, one per SIMD, as 2 x 2; each wave
// computes 128 rows x BN/2 columns as 32x32 MFMA tiles
// (v_mfma_f32_32x32x16_bf16, 256 fp32 accumulators per lane in AGPRs).  The
// MFMA computes the transposed tile (W rows as its first operand, A rows as
// its second), so each lane holds four consecutive output columns of a row.
// One wave per SIMD keeps the matrix pipe to itself: measured on MI355X, two
// waves per SIMD lose more to arbitration and barrier skew than they hide.
//
// Memory pipeline.  Operands go from global memory straight into LDS
// (global_load_lds_dwordx4, 16 B per lane, no register staging); A has two
// LDS stages, W three, one barrier per k-step.  A wave waiting to issue a
// load cannot issue MFMAs, so each half k-step interleaves its MFMAs, the
// LDS reads of the next half's fragments and its share of the loads in a
// fixed order (see half_step).  Each row contributes a whole 128 B line per
// k-step.
//
// LDS layout per stage: rows of 128 B (64 bf16); the eight 16 B chunks of row
// r sit at chunk position (c ^ ((r >> 1) & 7)).  A load instruction writes 8
// whole rows (1 KB); a fragment read (16 consecutive rows, same chunk) touches
// all 64 banks exactly once, the rate at which the LDS serves 16-byte reads.
//
// Epilogue.  After the last k-step each wave stages its output sub-tile in
// LDS (16 B chunks XOR-swizzled by row) and writes whole row segments.
//
// Tile order.  The m-tiles of all experts are laid end to end; see the
// mapping at the top of the kernel.
// ---------------------------------------------------------------------------
constexpr int kTBM = 256, kTBK = 64, kBandM = 4, kXcds = 8;
// Weight-streaming launches aim for at least this many blocks (8 per CU on a
// 256-CU MI355X) before they split the k range.
constexpr long kStreamMinBlocks = 2048;


typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// The same load, written so that the compiler does not see an LDS write: it
// then adds no waits of its own for it (it cannot tell the stages apart and
// would wait for every load before each LDS read).  The caller waits with
// explicit s_waitcnt vmcnt before any LDS read of the loaded data.  The load
// has no register result; M0 (the LDS destination of the wave, uniform) is set
// in the same statement.
__device__ __forceinline__ void load_lds16_raw(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(lds_addr) : "memory", "m0");
}

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= vm, other counters untouched.
// The same load with a uniform 64-bit base in SGPRs and a 32-bit per-lane byte
// offset in a VGPR (global "saddr" form): no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void load_lds16_sv(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}

constexpr int waitcnt_vm(int vm) { return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kWaitLgkm0 = 0xC07F;   // lgkmcnt(0), others untouched
// vmcnt <= vm and lgkmcnt(0).
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4); }

// Which tile (and which part of its k range) block b of the tiled kernel
// computes.  Block b runs on XCD x = b % 8 (workgroups are dealt round-robin)
// and takes entry i = b / 8 of that XCD's list.  m-tiles come in groups of 32;
// in group g, XCD x owns m-tiles 32g + 4x .. +3 and walks them n-tile by
// n-tile (4 m-tiles fastest).  The 32 blocks an XCD runs at once thus cover 4
// m-tiles x 8 n-tiles (their A and W rows shared in its L2), and all XCDs
// sweep the same n-tiles at the same time, so each W slice is fetched from HBM
// once and served to the other XCDs from the last-level cache.  The m-tiles
// past the last full group are dealt round-robin over the XCDs.
//
// Tail.  An XCD's list is cut into rounds of kCusPerXcd tiles.  If the last,
// partial round has at most half a round of tiles and the k range has at
// least kSplitMinSteps steps, each of them is split into
// S = min(kMaxSplit, kCusPerXcd / tail) parts of its k range, run by S blocks
// that store fp32 partial tiles into workspace slot x * kCusPerXcd + j; the
// reduce kernel then sums the parts in order.  Otherwise the last round's
// tiles stay whole.  The split saves a share of one tile's time, which grows
// with k, and costs the partial tiles' round trip, which does not: measured
// on MI355X it pays for k = 8192 and 14336 (second products of the Switch-style
// and prefill layers, 7% and 2% of the product) and loses for k = 1024 and
// 2048 (first products of the mid-size, fine-grained and Switch-style layers,
// 1-15%).
constexpr int kCusPerXcd = 32;
constexpr int kMaxSplit = 8;
constexpr int kSplitMinSteps = 64;   // k >= 4096
constexpr int kPartialSlots = kXcds * kCusPerXcd;
constexpr size_t kPartialTileFloats = (size_t)kTBM * 256;

struct TileJob {
  int mt, nt;      // m-tile (over all experts, end to end) and n-tile
  int part, parts; // part of the k range, of `parts` (1: the whole range)
  int slot;        // partial-tile slot when parts > 1
};

__device__ __forceinline__ bool tile_job(int total_mt, int ntn, int nk, int b, TileJob& job) {
  constexpr int kGroupM = kXcds * kBandM;
  const int x = b % kXcds, i = b / kXcds;
  const int G = total_mt / kGroupM;
  const int full = G * kBandM * ntn;                 // entries from full groups, per XCD
  const int lm = total_mt - G * kGroupM;             // leftover m-tiles (< 32)
  const int left = lm * ntn;                         // leftover tiles, dealt round-robin
  const int cnt = full + (left > x ? (left - x + kXcds - 1) / kXcds : 0);
  const int rounds = cnt / kCusPerXcd, tail = cnt - rounds * kCusPerXcd;
  const int S = (tail > 0 && 2 * tail <= kCusPerXcd && nk >= kSplitMinSteps)
                    ? min(min(kMaxSplit, nk), kCusPerXcd / tail)
                    : 1;
  int entry = i;
  job.part = 0;
  job.parts = 1;
  job.slot = 0;
  if (S > 1 && i >= rounds * kCusPerXcd) {
    const int j = i - rounds * kCusPerXcd;
    if (j >= tail * S) return false;
    entry = rounds * kCusPerXcd + j / S;
    job.part = j % S;
    job.parts = S;
    job.slot = x * kCusPerXcd + j;
  }
  if (entry >= cnt) return false;
  if (entry < full) {
    const int g = entry / (kBandM * ntn), rem = entry - g * kBandM * ntn;
    job.nt = rem / kBandM;
    job.mt = g * kGroupM + x * kBandM + rem % kBandM;
  } else {
    const int u = (entry - full) * kXcds + x;
    job.nt = u / lm;
    job.mt = G * kGroupM + u % lm;
  }
  return true;
}

// First entry of XCD x's tail (its last, partial round) in tile_job's order.
__device__ __forceinline__ int tail_start(int total_mt, int ntn, int x) {
  constexpr int kGroupM = kXcds * kBandM;
  const int G = total_mt / kGroupM;
  const int left = (total_mt - G * kGroupM) * ntn;
  const int cnt = G * kBandM * ntn + (left > x ? (left - x + kXcds - 1) / kXcds : 0);
  return cnt / kCusPerXcd * kCusPerXcd;
}

// Rows staged per epilogue pass: the largest multiple of 32 dividing the wave's
// rows whose staging fits the wave's share of the LDS.
constexpr int epilogue_pass_rows(int rows, int row_bytes, int budget) {
  int best = 32;
  for (int r = 32; r <= rows; r += 32)
    if (rows % r == 0 && r * row_bytes <= budget) best = r;
  return best;
}

// Epilogue modes of the tiled kernel.
constexpr int kOutGeluBf16 = 0;    // first product: GELU, rounded to bf16
constexpr int kOutF32 = 1;         // second product, or a partial tile: fp32 as is
constexpr int kOutGeluSplit = 2;   // first product: GELU as bf16 hi + lo planes

// BM x BN output tile, 4 waves as WM (along rows) x 4/WM, WS stages of W.
// SPLIT: the first product stores h as hi + lo planes; the second reads A as
// those two planes (both in one A stage, plane 1 after plane 0) and runs one
// MFMA per plane against the same W fragment.
template <bool UP, bool SPLIT, int BM, int BN, int WM, int WS, int OCC>
__global__ __launch_bounds__(256, OCC) void ffn_tiled_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ A_lo,
    const int32_t* __restrict__ offsets, const uint16_t* __restrict__ W,
    const uint16_t* __restrict__ bias, void* __restrict__ out, size_t out_plane, int E, int N,
    int K, float* __restrict__ partial, const int32_t* __restrict__ gather, int gather_k) {
  constexpr int NW = 4;
  constexpr int kPl = (SPLIT && !UP) ? 2 : 1;   // A planes
  constexpr int kWavesN = NW / WM;
  constexpr int kWN = BN / kWavesN;       // wave tile columns
  constexpr int kNT = kWN / 32;           // 32-column subtiles per wave
  constexpr int kWM = BM / WM;            // wave tile rows
  constexpr int kMT = kWM / 32;           // 32-row subtiles per wave
  constexpr int kAPlane = BM * 128;       // bytes per A plane per stage
  constexpr int kAStage = kAPlane * kPl;
  constexpr int kBStage = BN * 128;
  constexpr int kBBase = 2 * kAStage;     // A: 2 stages, then W: WS stages
  constexpr int kLds = kBBase + WS * kBStage;
  constexpr int kAInst = BM * kPl / 8 / NW;   // 1 KB load instructions per wave per stage
  constexpr int kBInst = BN / 8 / NW;
  static_assert(kNT >= 1 && kMT >= 1 && kWM % 32 == 0, "tile shape");
  static_assert((BM * kPl) % (8 * NW) == 0 && BN % (8 * NW) == 0 && BM % 16 == 0, "load plan");
  static_assert(kLds <= 160 * 1024 && WS >= 3, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];

  // ---- which tile ----  (N need not be a multiple of BN: the last n-tile's
  // columns past N load the last W row and are not stored)
  const int ntn = (N + BN - 1) / BN;
  TileJob job;
  const MTiles mts = mtiles<BM>(offsets, E);
  if (!tile_job(mts.total, ntn, K / kTBK, blockIdx.x, job)) return;
  const int mt = job.mt, nt = job.nt;
  int e, r0, r1;
  if (!find_mtile<BM>(mts, mt, e, r0, r1)) return;
  const int n0 = nt * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS targets in SGPRs
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int fr = lane & 31, fc = lane >> 5;

  // Load plan: instruction i of wave w fills LDS rows (i*NW + w)*8 + lane/8 of
  // the stage (A: plane p's row r is LDS row p*BM + r), physical chunk lane%8,
  // i.e. logical chunk (lane%8) ^ ((row >> 1) & 7).  BM is a multiple of 16,
  // so a plane-1 row has the swizzle of its row within the plane.
  // Per-lane byte offsets (32 bits: the descriptor limits keep every operand
  // under 4 GiB) from uniform bases that advance by k.  A plane-1 row
  // (instruction i >= BM / 32 of a split A) reads from A_lo.
  uint32_t a_off[kAInst];
  uint32_t b_off[kBInst];
  const uint16_t* Wexp = W + (size_t)e * N * K;
  if constexpr (UP) {                                 // only the first product gathers
    int arow[kAInst];
#pragma unroll
    for (int i = 0; i < kAInst; ++i) arow[i] = min(r0 + ((i * NW + wave) * 8 + (lane >> 3)) % BM, r1 - 1);
    a_rows<kAInst>(gather, gather_k, arow);
#pragma unroll
    for (int i = 0; i < kAInst; ++i) {
      const int lrow = (i * NW + wave) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((lrow >> 1) & 7);
      a_off[i] = (uint32_t)(((size_t)arow[i] * K + c * 8) * 2);
    }
  } else {
#pragma unroll
    for (int i = 0; i < kAInst; ++i) {
      const int lrow = (i * NW + wave) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((lrow >> 1) & 7);
      a_off[i] = (uint32_t)(((size_t)min(r0 + lrow % BM, r1 - 1) * K + c * 8) * 2);
    }
  }
#pragma unroll
  for (int i = 0; i < kBInst; ++i) {
    const int row = (i * NW + wave) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    b_off[i] = (uint32_t)(((size_t)min(n0 + row, N - 1) * K + c * 8) * 2);
  }
  const int nk_all = K / kTBK;
  const int ks0 = (int)((long)job.part * nk_all / job.parts);
  const int nk = (int)((long)(job.part + 1) * nk_all / job.parts) - ks0;
  const uint16_t* a_base = A + ks0 * kTBK;
  const uint16_t* a_lo_base = (kPl == 2 ? A_lo : A) + ks0 * kTBK;
  const uint16_t* b_base = Wexp + ks0 * kTBK;
  auto a_plane_base = [&](int i) { return (i * NW * 8) / BM ? a_lo_base : a_base; };
  // Steps past the last are clamped to it: those loads refill a free stage and
  // are never read, which keeps the loop body branch-free.
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  auto issue_a = [&](int stage, int step) {
    const uint32_t base = lds0 + stage * kAStage;
    const int k0 = min(step, nk - 1) * kTBK;
#pragma unroll
    for (int i = 0; i < kAInst; ++i) load_lds16_sv(a_plane_base(i) + k0, a_off[i], base + (i * NW + wave) * 1024);
  };
  auto issue_b = [&](int stage, int step) {
    const uint32_t base = lds0 + kBBase + stage * kBStage;
    const int k0 = min(step, nk - 1) * kTBK;
#pragma unroll
    for (int i = 0; i < kBInst; ++i) load_lds16_sv(b_base + k0, b_off[i], base + (i * NW + wave) * 1024);
  };

  // Main loop and epilogue for a wave whose rows of the tile fill kMA of its
  // kMT 32-row subtiles.  Tiles under 256 rows instantiate it for all kMT and
  // for about half, so the padding past an expert's last row costs no MFMAs
  // when the tile is at most half full; both versions run the same barriers.
  // (The 256-row kernel keeps one version: a second one makes it spill.)
  auto body = [&](auto ma_tag) {
    constexpr int kMA = decltype(ma_tag)::value;
    constexpr int kAFa = kMA * kPl;
    f32x16 acc[kNT][kMA];
#pragma unroll
    for (int jn = 0; jn < kNT; ++jn)
#pragma unroll
      for (int im = 0; im < kMA; ++im)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[jn][im][q] = 0.f;

    // A k-step of 64 is four 16-wide MFMA slices; a half step is two slices.
    // X holds half 0 of a step, Y half 1.  Fragment r of a half (r < kReads) is
    // slice r / (kAFa + kNT) of A fragment q (q < kAFa: plane q / kMA, subtile
    // q % kMA) or of W subtile q - kAFa.
    constexpr int kReads = 2 * (kAFa + kNT);
    constexpr int kMfmas = 2 * kMA * kNT * kPl;
    static_assert(kReads % 2 == 0 && kReads / 2 <= kMfmas, "two reads per MFMA");
    static_assert(kAInst <= kMfmas && kBInst <= kMfmas, "at most one load per MFMA");
    u32x4 xa[2][kAFa], xb[2][kNT], ya[2][kAFa], yb[2][kNT];
    auto read_at = [&](u32x4 (&fa)[2][kAFa], u32x4 (&fb)[2][kNT], int sa_, int sb_, int half, int r) {
      const int sl = r / (kAFa + kNT), q = r % (kAFa + kNT);
      const int ch = (half * 2 + sl) * 2 + fc;     // 16 B chunk: 8 k of this slice
      if (q < kAFa) {
        const int row = (q / kMA) * BM + wm * kWM + (q % kMA) * 32 + fr;
        fa[sl][q] = ld16(lds + sa_ * kAStage + row * 128 + ((ch ^ ((row >> 1) & 7)) << 4));
      } else {
        const int row = wn * kWN + (q - kAFa) * 32 + fr;
        fb[sl][q - kAFa] = ld16(lds + kBBase + sb_ * kBStage + row * 128 + ((ch ^ ((row >> 1) & 7)) << 4));
      }
    };
    auto read_all = [&](u32x4 (&fa)[2][kAFa], u32x4 (&fb)[2][kNT], int sa_, int sb_, int half) {
#pragma unroll
      for (int r = 0; r < kReads; ++r) read_at(fa, fb, sa_, sb_, half, r);
    };
    // MFMA m of a half: slice m / (kPl kNT kMA), then plane, W subtile, A subtile
    // (fastest), so consecutive MFMAs update different accumulators.
    auto mfma_at = [&](const u32x4 (&fa)[2][kAFa], const u32x4 (&fb)[2][kNT], int m) {
      constexpr int kPerSlice = kPl * kNT * kMA;
      const int sl = m / kPerSlice, rem = m % kPerSlice;
      const int p = rem / (kNT * kMA), jn = (rem / kMA) % kNT, im = rem % kMA;
      acc[jn][im] = mfma32_bf16(fb[sl][jn], fa[sl][p * kMA + im], acc[jn][im]);
    };
    // One half step in a fixed instruction order: after each MFMA (whose
    // operands were read in the previous half), up to two LDS reads of the next
    // half's fragments, front-loaded so they return long before they are needed,
    // and, evenly spread, this half's L global->LDS loads.  A wave waiting to
    // issue a load cannot issue MFMAs, so loads are paced rather than burst.
    auto half_step = [&](const u32x4 (&fa)[2][kAFa], const u32x4 (&fb)[2][kNT], u32x4 (&na)[2][kAFa],
                         u32x4 (&nb)[2][kNT], int nsa, int nsb, int nhalf, auto load_fn, auto loads_tag) {
      constexpr int L = decltype(loads_tag)::value;
#pragma unroll
      for (int m = 0; m < kMfmas; ++m) {
        mfma_at(fa, fb, m);
        if (2 * m < kReads) {
          read_at(na, nb, nsa, nsb, nhalf, 2 * m);
          read_at(na, nb, nsa, nsb, nhalf, 2 * m + 1);
        }
        if ((m + 1) * L / kMfmas > m * L / kMfmas) load_fn(m * L / kMfmas);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    using LoadsA = std::integral_constant<int, kAInst>;
    using LoadsB = std::integral_constant<int, kBInst>;
    using NoLoads = std::integral_constant<int, 0>;

    // Pipeline.  Step t's A tile sits in A stage t % 2, its W tile in W stage
    // t % WS, and W runs WS - 1 steps ahead.  Per step t:
    //   X <- half 0 of step t is in registers when step t starts;
    //   first half: X MFMAs, reads of Y <- half 1 of step t, and the loads of W
    //     for step t+WS-1 into W stage (t-1) % WS, which nobody reads any more
    //     (it held step t-1, finished before the previous barrier);
    //   wait for our LDS reads and for A and W of step t+1 (only W of step
    //     t+WS-1, issued after both, may still be in flight), barrier;
    //   second half: Y MFMAs, reads of X <- half 0 of step t+1, and the loads of
    //     A for step t+2 into A stage t % 2 (every wave is done reading it).
    // Loads complete in issue order.  The prologue issues A0, A1, W0 .. W(WS-2),
    // so every wait counts whole W groups only.
    issue_a(0, 0);
    issue_a(1, 1);
#pragma unroll
    for (int d = 0; d < WS - 1; ++d) issue_b(d, d);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((WS - 2) * kBInst));   // A0, A1 and W0 landed
    __syncthreads();
    read_all(xa, xb, 0, 0, 0);
    int sa = 0, sb = 0;                                // stages of step kt
    for (int kt = 0; kt < nk - 1; ++kt) {
      const int sa1 = sa ^ 1, sb1 = sb == WS - 1 ? 0 : sb + 1, sbw = sb == 0 ? WS - 1 : sb - 1;
      const int kbw = min(kt + WS - 1, nk - 1) * kTBK, kba = min(kt + 2, nk - 1) * kTBK;
      half_step(xa, xb, ya, yb, sa, sb, 1,
                [&](int i) { load_lds16_sv(b_base + kbw, b_off[i], lds0 + kBBase + sbw * kBStage + (i * NW + wave) * 1024); },
                LoadsB{});
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kBInst));
      __syncthreads();
      half_step(ya, yb, xa, xb, sa1, sb1, 0,
                [&](int i) { load_lds16_sv(a_plane_base(i) + kba, a_off[i], lds0 + sa * kAStage + (i * NW + wave) * 1024); },
                LoadsA{});
      sa = sa1;
      sb = sb1;
    }
    half_step(xa, xb, ya, yb, sa, sb, 1, [&](int) {}, NoLoads{});
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
    for (int m = 0; m < kMfmas; ++m) mfma_at(ya, yb, m);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();                                   // LDS free for the epilogue

    // Epilogue through LDS.  Lane (fr, fc) holds, for each 32x32 subtile (jn, im)
    // and g = 0..3, row im*32 + fr and columns jn*32 + 8g + 4fc .. +3 of the
    // wave's sub-tile.  Each wave stages rows in its own LDS region with 16 B
    // chunks XOR-swizzled by row, then stores whole row segments of the rows
    // below row_lim to dst (row stride in elements).  kOutGeluBf16 stages bf16;
    // the other modes stage fp32 (kOutGeluSplit converts to hi + lo on the way
    // out, the lo plane out_plane elements after the hi plane).
    const uint16_t* bexp = bias ? bias + (size_t)e * N : nullptr;
    // The lane's bias words (four bf16 columns per (jn, g), the same in every
    // pass): loaded once per tile, all in flight before any is used -- one at a
    // time they cost a round trip each.
    uint2 braw[kNT][4];
    auto load_bias = [&](bool with_bias) {
#pragma unroll
      for (int jn = 0; jn < kNT; ++jn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = n0 + wn * kWN + jn * 32 + 8 * g + 4 * fc;
          braw[jn][g] = (with_bias && col < N) ? *reinterpret_cast<const uint2*>(bexp + col)
                                               : make_uint2(0u, 0u);
        }
    };
    auto bias4 = [&](int jn, int g, float (&bv)[4]) {
      bv[0] = __uint_as_float(braw[jn][g].x << 16);
      bv[1] = __uint_as_float(braw[jn][g].x & 0xffff0000u);
      bv[2] = __uint_as_float(braw[jn][g].y << 16);
      bv[3] = __uint_as_float(braw[jn][g].y & 0xffff0000u);
    };
    auto store_tile = [&](auto mode_tag, uint8_t* dst, size_t row_stride, int row_lim, int col_lim,
                          bool with_bias) {
      constexpr int MODE = decltype(mode_tag)::value;
      constexpr int kSElem = MODE == kOutGeluBf16 ? 2 : 4;   // staged bytes per element
      constexpr int kOElem = MODE == kOutF32 ? 4 : 2;        // stored bytes per element
      constexpr int kRowB = kWN * kSElem, kChunks = kRowB / 16;
      constexpr int kPassRows = epilogue_pass_rows(kWM, kRowB, kLds / NW);
      constexpr int kPasses = kWM / kPassRows;
      constexpr int kRowsPerInst = 64 / kChunks;
      uint8_t* my = lds + wave * (kPassRows * kRowB);
      if (with_bias) load_bias(true);
#pragma unroll
      for (int pass = 0; pass < kPasses; ++pass) {
        if (pass * kPassRows >= kMA * 32) continue;    // rows past the active subtiles
#pragma unroll
        for (int jn = 0; jn < kNT; ++jn)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if (with_bias) bias4(jn, g, bv);
#pragma unroll
            for (int imp = 0; imp < kPassRows / 32; ++imp) {
              const int im = pass * (kPassRows / 32) + imp;
              const int row = imp * 32 + fr;           // row within this pass
              if (im >= kMA) continue;                 // never active: nothing to store
              if constexpr (MODE == kOutGeluBf16) {
                const int chunk = jn * 4 + g;           // 16 B = 8 columns; fc picks the half
                uint32_t p[2];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
                  p[h2] = pack_bf16x2(gelu_erf(acc[jn][im][4 * g + 2 * h2] + bv[2 * h2]),
                                      gelu_erf(acc[jn][im][4 * g + 2 * h2 + 1] + bv[2 * h2 + 1]));
                *reinterpret_cast<uint2*>(my + row * kRowB + ((chunk ^ (row & (kChunks - 1))) << 4) + fc * 8) =
                    make_uint2(p[0], p[1]);
              } else {
                const int chunk = jn * 8 + 2 * g + fc;  // 16 B = 4 columns
                f32x4 v;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  v[q] = acc[jn][im][4 * g + q] + bv[q];
                  if constexpr (MODE == kOutGeluSplit) v[q] = gelu_erf(v[q]);
                }
                *reinterpret_cast<f32x4*>(my + row * kRowB + ((chunk ^ (row & (kChunks - 1))) << 4)) = v;
              }
            }
          }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);        // our own LDS writes are done
#pragma unroll 4
        for (int rb = 0; rb < kPassRows; rb += kRowsPerInst) {
          const int row = rb + lane / kChunks, chunk = lane % kChunks;
          const int lrow = wm * kWM + pass * kPassRows + row;
          const u32x4 v = ld16(my + row * kRowB + ((chunk ^ (row & (kChunks - 1))) << 4));
          if (lrow < row_lim && wn * kWN + chunk * (16 / kSElem) < col_lim) {
            if constexpr (MODE == kOutGeluSplit) {
              // 4 fp32 GELU values -> 4 bf16 hi (8 B) and 4 bf16 lo (8 B).
              uint32_t hi[2], lo[2];
#pragma unroll
              for (int h2 = 0; h2 < 2; ++h2) {
                const float g0 = __uint_as_float(v[2 * h2]), g1 = __uint_as_float(v[2 * h2 + 1]);
                hi[h2] = pack_bf16x2(g0, g1);
                lo[h2] = pack_bf16x2(g0 - __uint_as_float(hi[h2] << 16),
                                     g1 - __uint_as_float(hi[h2] & 0xffff0000u));
              }
              const size_t off = ((size_t)lrow * row_stride + wn * kWN) * kOElem + chunk * 8;
              *reinterpret_cast<uint2*>(dst + off) = make_uint2(hi[0], hi[1]);
              *reinterpret_cast<uint2*>(dst + out_plane * 2 + off) = make_uint2(lo[0], lo[1]);
            } else {
              st16(dst + ((size_t)lrow * row_stride + wn * kWN) * kOElem + chunk * 16, v);
            }
          }
        }
        if (kPasses > 1) __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // reads done before the next pass
      }
    };
    using ModeBf16 = std::integral_constant<int, kOutGeluBf16>;
    using ModeF32 = std::integral_constant<int, kOutF32>;
    using ModeSplit = std::integral_constant<int, kOutGeluSplit>;
    if (job.parts > 1) {
      store_tile(ModeF32{}, reinterpret_cast<uint8_t*>(partial + job.slot * kPartialTileFloats), BN,
                 r1 - r0, BN, false);
    } else if constexpr (UP) {
      using Mode = std::conditional_t<SPLIT, ModeSplit, ModeBf16>;
      store_tile(Mode{}, static_cast<uint8_t*>(out) + ((size_t)r0 * N + n0) * 2, N, r1 - r0, N - n0,
                 bexp != nullptr);
    } else {
      store_tile(ModeF32{}, static_cast<uint8_t*>(out) + ((size_t)r0 * N + n0) * 4, N, r1 - r0, N - n0,
                 bexp != nullptr);
    }
  };
  const int act = __builtin_amdgcn_readfirstlane(min(kMT, max(0, (r1 - r0 - wm * kWM + 31) / 32)));
  constexpr int kHalf = (kMT + 1) / 2;
  if constexpr (BM == 256) {
    (void)act;
    body(std::integral_constant<int, kMT>{});
  } else {
    if (act <= kHalf) body(std::integral_constant<int, kHalf>{});
    else body(std::integral_constant<int, kMT>{});
  }
}

// Finish the tiles the tiled kernel split along k: block (x = b % 8, j = b / 8)
// takes the j-th block of XCD x's tail round, i.e. part p of a split tile,
// and completes rows [p * BM / S, (p + 1) * BM / S) of it: the S partial
// tiles summed in part order, plus the bias, then the product's epilogue.
template <bool UP, bool SPLIT, int BM, int BN>
__global__ __launch_bounds__(256) void ffn_tile_reduce(
    const int32_t* __restrict__ offsets, const uint16_t* __restrict__ bias, void* __restrict__ out,
    size_t out_plane, int E, int N, int K, const float* __restrict__ partial) {
  const int ntn = (N + BN - 1) / BN, x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  TileJob job;
  const MTiles mts = mtiles<BM>(offsets, E);
  if (!tile_job(mts.total, ntn, K / kTBK, x + kXcds * (tail_start(mts.total, ntn, x) + j), job) ||
      job.parts == 1)
    return;
  int e, r0, r1;
  if (!find_mtile<BM>(mts, job.mt, e, r0, r1)) return;
  const int n0 = job.nt * BN;
  const int ra = job.part * BM / job.parts;
  const int rb = min(r1 - r0, (job.part + 1) * BM / job.parts);
  const float* p0 = partial + (size_t)(job.slot - job.part) * kPartialTileFloats;
  const uint16_t* bexp = bias ? bias + (size_t)e * N + n0 : nullptr;
  constexpr int kQuads = BN / 4;
  // kU quads per thread per pass, all of their parts loaded before any is
  // summed, so a pass keeps kU * parts loads in flight; parts add in part order.
  constexpr int kU = 4;
  const int q0 = ra * kQuads, q1 = rb * kQuads;
  for (int qb = q0 + threadIdx.x; qb < q1; qb += 256 * kU) {
    f32x4 part[kU][kMaxSplit];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int q = qb + u * 256;
      const int r = q / kQuads, c = (q % kQuads) * 4;
      if (q < q1 && n0 + c < N) {
        const float* src = p0 + (size_t)r * BN + c;
#pragma unroll
        for (int sp = 0; sp < kMaxSplit; ++sp)
          if (sp < job.parts) part[u][sp] = *reinterpret_cast<const f32x4*>(src + sp * kPartialTileFloats);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int q = qb + u * 256;
      const int r = q / kQuads, c = (q % kQuads) * 4;
      if (q >= q1 || n0 + c >= N) continue;          // past the range or the last column
      f32x4 v = part[u][0];
#pragma unroll
      for (int sp = 1; sp < kMaxSplit; ++sp)
        if (sp < job.parts) v += part[u][sp];
      if (bexp) {
        const uint2 braw = *reinterpret_cast<const uint2*>(bexp + c);
        v[0] += __uint_as_float(braw.x << 16);
        v[1] += __uint_as_float(braw.x & 0xffff0000u);
        v[2] += __uint_as_float(braw.y << 16);
        v[3] += __uint_as_float(braw.y & 0xffff0000u);
      }
      const size_t idx = (size_t)(r0 + r) * N + n0 + c;
      if constexpr (UP && SPLIT) {
#pragma unroll
        for (int w = 0; w < 4; ++w) emit<uint16_t, true, true>(out, out_plane, idx + w, v[w]);
      } else if constexpr (UP) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) =
            make_uint2(pack_bf16x2(gelu_erf(v[0]), gelu_erf(v[1])), pack_bf16x2(gelu_erf(v[2]), gelu_erf(v[3])));
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + idx) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Weight-streaming kernel.  Block = 4 waves; wave w owns the 16*NWN output
// columns n0 + w*16*NWN + [0, 16*NWN); the block owns rows
// [offsets[e] + g*16*NMT, ...) of expert e = blockIdx.y, g = blockIdx.z.
// The k range is cut into chunks; each chunk of a row is 256 B of A (two 128 B
// planes when the second product reads a split h = hi + lo).
//   - W goes straight into registers: lane l reads row (l % 16) of its n-tile
//     and pieces 4q + l / 16, q < KQ, so one load instruction reads 64
//     contiguous bytes of each of 16 rows (measured on MI355X: ~6% more HBM
//     bandwidth than KQ adjacent pieces per lane).  A ring of kDepth register
//     buffers keeps kDepth - 1 chunks of W loading while one is consumed.
//   - A goes global -> LDS by DMA (global_load_lds_dwordx4, 1 KB per wave
//     instruction) into a ring of kDepth LDS stages, kDepth - 1 chunks ahead,
//     so neither operand's load latency sits on the per-chunk path; one
//     barrier per chunk publishes a stage and frees the one consumed before.
//     Pieces of a row sit at (piece ^ swz(row)) so the fragment reads (16
//     rows, same piece) are conflict free.
//   - MFMA q of the chunk uses the lane's piece 4q + l / 16 of A (and of A's
//     low term when h is split) and of W.
// m-tiles past the block's last row issue no MFMA, so padding costs nothing.
// Long weight rows (K >= kStreamRotateK): block x walks its chunks starting
// at chunk (x % 4) * nch / 4 and wraps around, so the blocks in flight read
// four different parts of their rows instead of the same column band
// (measured on MI355X: ~3% faster weight streaming for the decode layer's
// second product; for K = 4096 it was slower).  The sum order is fixed per
// block, so results stay bitwise repeatable.
// ---------------------------------------------------------------------------
constexpr int kStreamRotateK = 8192;

template <typename T, bool UP, bool SPLIT, int NMT, int NWN>
__global__ __launch_bounds__(256) void ffn_stream_kernel(
    const T* __restrict__ A, const T* __restrict__ A_lo, const int32_t* __restrict__ offsets,
    const T* __restrict__ W, const T* __restrict__ bias, void* __restrict__ out,
    size_t out_plane, int E, int N, int K, int splits, float* __restrict__ partial, int rows_cap,
    const int32_t* __restrict__ gather, int gather_k) {
  constexpr bool kTwoA = SPLIT && !UP;             // A operand is split h
  constexpr int kQ = kTwoA ? 2 : 4;                // 16 B pieces per lane per chunk
  constexpr int kPerVec = 16 / sizeof(T);
  constexpr int kChunk = 4 * kQ * kPerVec;         // 128 bf16, 64 (split) or 64 fp32
  constexpr int kPieces = 4 * kQ;                  // pieces per row per plane
  constexpr int kRowBytes = kPieces * 16;          // 256 B, or 128 B per plane
  constexpr int kMR = 16 * NMT;
  constexpr int kPlaneBytes = kMR * kRowBytes;
  constexpr int kStageBytes = kMR * 256;           // all planes of one chunk
  constexpr int kDepth = NMT <= 4 ? 4 : 2;
  constexpr int kAInst = NMT;                      // 1 KB DMA instructions per wave per chunk
  constexpr int kWInst = NWN * kQ;                 // W load instructions per wave per chunk
  static_assert(kStageBytes == 4 * 1024 * kAInst && kPlaneBytes % 1024 == 0, "DMA plan");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kDepth * kStageBytes];
  auto swz = [](int row) { return kPieces == 16 ? (row & 15) : ((row >> 1) & 7); };

  const int e = blockIdx.y;
  const int split = blockIdx.z % splits;             // k range [c0, c1) of the chunks
  const int seg0 = offsets[e], seg1 = offsets[e + 1];
  const int r0 = seg0 + (blockIdx.z / splits) * kMR;
  if (r0 >= seg1) return;
  const int r1 = min(seg1, r0 + kMR);
  const int mt_active = (r1 - r0 + 15) >> 4;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fc = lane >> 4;
  const int n0 = blockIdx.x * (64 * NWN) + wave * 16 * NWN;

  // DMA plan: instruction i of wave w fills bytes [g*1KB, (g+1)*1KB) of a
  // stage, g = 4i + w: plane g*1KB / kPlaneBytes, rows from there on; lane L
  // writes physical piece L % kPieces of its row, i.e. logical piece
  // (L % kPieces) ^ swz(row).  Rows past the block's last are clamped (their
  // data is never used).
  const T* a_src[kAInst];
  int arow[kAInst];
#pragma unroll
  for (int i = 0; i < kAInst; ++i)
    arow[i] = min(r0 + (((i * 4 + wave) * 1024 + lane * 16) % kPlaneBytes) / kRowBytes, r1 - 1);
  if constexpr (UP) a_rows<kAInst>(gather, gather_k, arow);   // only the first product gathers
#pragma unroll
  for (int i = 0; i < kAInst; ++i) {
    const int byte = (i * 4 + wave) * 1024 + lane * 16;
    const int plane = byte / kPlaneBytes;
    const int row = (byte % kPlaneBytes) / kRowBytes;
    const int logical = ((byte % kRowBytes) / 16) ^ swz(row);
    const T* base = (kTwoA && plane) ? A_lo : A;
    a_src[i] = base + (size_t)arow[i] * K + logical * kPerVec;
  }
  // Compact plan for a block whose rows fit one m-tile (NMT > 1): the first 16
  // rows of every plane are 4 KB in all, one 1 KB instruction per wave, written
  // where the full plan puts them (plane p at p * kPlaneBytes).  Halves (or
  // better) the A loads of blocks with few rows, e.g. decode.
  constexpr int kHalfPlane = 16 * kRowBytes;
  const bool compact = NMT > 1 && mt_active == 1;
  const T* a_src1 = nullptr;
  uint32_t a_dst1 = 0;
  if (compact) {
    const int byte = wave * 1024 + lane * 16;
    const int plane = byte / kHalfPlane, rem = byte % kHalfPlane;
    const int row = rem / kRowBytes;
    int ar[1] = {min(r0 + row, r1 - 1)};
    if constexpr (UP) a_rows<1>(gather, gather_k, ar);
    const int logical = ((rem % kRowBytes) / 16) ^ swz(row);
    a_src1 = ((kTwoA && plane) ? A_lo : A) + (size_t)ar[0] * K + logical * kPerVec;
    a_dst1 = (uint32_t)(((wave * 1024) / kHalfPlane) * kPlaneBytes + (wave * 1024) % kHalfPlane);
  }
  const T* w_src[NWN];
  const T* Wexp = W + (size_t)e * N * K;
#pragma unroll
  for (int j = 0; j < NWN; ++j) w_src[j] = Wexp + (size_t)(n0 + j * 16 + fr) * K + fc * kPerVec;

  f32x4 acc[NMT][NWN];
#pragma unroll
  for (int i = 0; i < NMT; ++i)
#pragma unroll
    for (int j = 0; j < NWN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nch_all = K / kChunk;
  const int c0 = (int)((long)split * nch_all / splits);
  const int nch = (int)((long)(split + 1) * nch_all / splits) - c0;
  const int rot = K >= kStreamRotateK ? (int)((long)(blockIdx.x % 4) * nch / 4) : 0;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  u32x4 wbuf[kDepth][NWN][kQ];
  // Issue the block's chunk ch (chunk c0 + (ch + rot) mod nch of the row):
  // W into register slot `slot`, A into LDS stage `slot`.
  auto issue = [&](u32x4 (&wdst)[NWN][kQ], int slot, int ch) {
    const int cr = ch + rot < nch ? ch + rot : ch + rot - nch;
    const int k0 = (c0 + cr) * kChunk;
#pragma unroll
    for (int j = 0; j < NWN; ++j)
#pragma unroll
      for (int q = 0; q < kQ; ++q) wdst[j][q] = ld16(w_src[j] + k0 + q * 4 * kPerVec);
    if (compact) {
      load_lds16_raw(a_src1 + k0, lds0 + slot * kStageBytes + a_dst1);
    } else {
#pragma unroll
      for (int i = 0; i < kAInst; ++i)
        load_lds16_raw(a_src[i] + k0, lds0 + slot * kStageBytes + (i * 4 + wave) * 1024);
    }
  };
  auto compute = [&](const u32x4 (&wc)[NWN][kQ], int slot) {
    const uint8_t* st = lds + slot * kStageBytes;
#pragma unroll
    for (int i = 0; i < NMT; ++i) {
      if (i < mt_active) {
        const int row = i * 16 + fr;
        u32x4 af[kQ], al[kQ];
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
          const int off = row * kRowBytes + (((q * 4 + fc) ^ swz(row)) << 4);
          af[q] = ld16(st + off);
          if constexpr (kTwoA) al[q] = ld16(st + kPlaneBytes + off);
        }
#pragma unroll
        for (int j = 0; j < NWN; ++j) {
          if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int q = 0; q < kQ; ++q) {
              acc[i][j] = mfma_bf16(af[q], wc[j][q], acc[i][j]);
              if constexpr (kTwoA) acc[i][j] = mfma_bf16(al[q], wc[j][q], acc[i][j]);
            }
          } else {
#pragma unroll
            for (int q = 0; q < kQ; ++q)
#pragma unroll
              for (int u = 0; u < 4; ++u)
                acc[i][j] = mfma_f32(__uint_as_float(af[q][u]), __uint_as_float(wc[j][q][u]),
                                     acc[i][j]);
          }
        }
      }
    }
  };

  // Loads complete in issue order.  In steady state kDepth - 2 chunks' loads
  // were issued after A of the next chunk, so waiting for at most that many
  // outstanding lands it; near the end (fewer loads issued) wait for all.
  constexpr int kSteadyWait = (kDepth - 2) * (kWInst + kAInst);
  constexpr int kSteadyWait1 = (kDepth - 2) * (kWInst + 1);   // compact plan
  auto steady_wait = [&]() {
    if (compact) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kSteadyWait1));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kSteadyWait));
  };
#pragma unroll
  for (int d = 0; d < kDepth - 1; ++d)
    if (d < nch) issue(wbuf[d], d, d);
  if (nch >= kDepth - 1) steady_wait();
  else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  __syncthreads();
  for (int ch0 = 0; ch0 < nch; ch0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int ch = ch0 + d;
      if (ch < nch) {
        const int dn = (d + kDepth - 1) % kDepth;       // slot of chunk ch + kDepth - 1 (constant once unrolled)
        const bool steady = ch + kDepth - 1 < nch;
        if (steady) issue(wbuf[dn], dn, ch + kDepth - 1);
        compute(wbuf[d], d);
        if (steady) steady_wait();
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        __syncthreads();
      }
    }
  }

  // Epilogue.  Lane (fr, fc) holds column n0 + 16j + fr of rows 4fc + v.  With
  // a split k range each split stores its fp32 partial sums (split 0 adds the
  // bias) and ffn_splitk_reduce finishes the product.
  const T* bexp = bias ? bias + (size_t)e * N : nullptr;
#pragma unroll
  for (int j = 0; j < NWN; ++j) {
    const int col = n0 + j * 16 + fr;
    const float bv = (bexp && split == 0) ? Elem<T>::to_f32(bexp[col]) : 0.f;
#pragma unroll
    for (int i = 0; i < NMT; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = r0 + i * 16 + 4 * fc + v;
        if (row < r1) {
          const size_t idx = (size_t)row * N + col;
          if (splits > 1)
            partial[((size_t)split * rows_cap + row) * N + col] = acc[i][j][v] + bv;
          else
            emit<T, UP, SPLIT>(out, out_plane, idx, acc[i][j][v] + bv);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Weight-streaming kernel (bf16), both operands through LDS.  Same block shape
// as ffn_stream_kernel with NWN = 1 (4 waves, wave w owns 16 output columns of
// each 64-column block; the block owns up to 16*NMT rows of expert blockIdx.y
// at a time), but the weights go global -> LDS by DMA too, in stages of
// kLdsRun bytes of each of the block's 64 weight rows (and of its A rows, both
// planes of a split h).  One DMA instruction then reads two whole 512 B runs,
// where the register ring reads 64 B of each of 16 rows per instruction:
// measured on MI355X with the decode layer's first product, the register
// pattern streams its weights at ~5.2 TB/s whatever the A traffic (the same
// kernel without its A loads is no faster), and DMA probes of 512 B runs x 64
// rows, A rows included, at 5.7-5.8 TB/s.
//   - Stage s of the k range (kLdsStageK elements) sits in ring slot s % kLdsDepth
//     of W (64 rows) and of A (16*NMT rows per plane), rows of kLdsRun bytes
//     whose 16 B pieces sit at (piece ^ (row & 15)), so the fragment reads (16
//     rows, same piece) hit every bank once.  DMA instruction i of wave w
//     writes 1 KB of a stage part: the 1024 / kLdsRun whole rows from row
//     (1024 / kLdsRun) * g on, g = 4i + w (A: plane 0's rows, then plane 1's).
//   - Per stage: wait for its loads, barrier (the slot of stage s - 1 is then
//     free), issue stage s + kLdsDepth - 1 into that slot, then the MFMAs of
//     the active m-tiles (one per plane), lane (fr, fc) using piece 4q + fc of
//     its A row and its W row for MFMA q.
//   - Persistent over column blocks: block x streams the `cpb` column blocks
//     x*cpb .. of its expert one after the other (the host sizes the grid to
//     one block per CU), and the stage sequence runs on across their
//     boundaries, so the ring never drains and the block's set-up (offsets,
//     gathered row indices: ~2.5 us measured) is paid once, not per 64
//     columns.  Each column block keeps its own accumulators (cpb <=
//     kLdsMaxCpb) and all results are stored after the last stage: a store
//     in the loop would share the vmcnt counter with the DMA loads without
//     completing in order with them, and the loop's wait counts assume
//     loads only.
//   - Row groups: in the second product the block takes every group of 16*NMT
//     rows of its expert in turn (a new stage sequence each; between two, the
//     stores drain and the ring restarts); in the first, only group
//     blockIdx.z / splits.
//     The second product uses 16-row groups (both planes of a 32-row group and
//     three stages would not fit in the LDS), so an expert with more rows
//     streams its weights once per group.
// Rows past the group's last are clamped (their data is never used); m-tiles
// past it issue no MFMA.  Sum order is fixed per block (bitwise repeatable).
// ---------------------------------------------------------------------------
constexpr int kLdsRun = 512;                   // bytes of each row per stage
constexpr int kLdsStageK = kLdsRun / 2;        // bf16 elements per stage
constexpr int kLdsDepth = 3;
constexpr int kLdsMaxCpb = 8;                  // column blocks per block, at most

template <bool UP, bool SPLIT, int NMT>
__global__ __launch_bounds__(256) void ffn_stream_lds_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ A_lo,
    const int32_t* __restrict__ offsets, const uint16_t* __restrict__ W,
    const uint16_t* __restrict__ bias, void* __restrict__ out, size_t out_plane, int E, int N,
    int K, int splits, float* __restrict__ partial, int rows_cap,
    const int32_t* __restrict__ gather, int gather_k, int cpb, int early) {
  constexpr int kPlanes = (SPLIT && !UP) ? 2 : 1;
  constexpr bool kLoopGroups = !UP;              // the second product loops over row groups
  constexpr int kMR = 16 * NMT;
  constexpr int kWBytes = 64 * kLdsRun;          // W part of a stage: 32 KB
  constexpr int kAPlane = kMR * kLdsRun;         // A part: 8 KB per m-tile and plane
  constexpr int kABytes = kPlanes * kAPlane;
  constexpr int kWI = kWBytes / 4096;            // 1 KB DMA instructions per wave per stage
  constexpr int kAI = kABytes / 4096;
  constexpr int kPieces = kLdsRun / 16;
  static_assert(kWI * 4096 == kWBytes && kAI * 4096 == kABytes && kAPlane % 1024 == 0 &&
                kLdsRun <= 1024 && kPieces >= 16, "DMA plan");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsDepth * (kWBytes + kABytes)];

  const int e = blockIdx.y;
  const int split = blockIdx.z % splits;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fc = lane >> 4;
  const int cb0 = blockIdx.x * cpb;              // the block's first column block
  const int ncb = min(cpb, N / 64 - cb0);
  if (ncb <= 0) return;

  // DMA plan (see above): with R = 1024 / kLdsRun rows per instruction, lane L
  // of instruction i writes physical piece L % kPieces of row R*g + L / kPieces
  // of its part, i.e. loads logical piece (L % kPieces) ^ (row & 15).
  constexpr int kRowsPerInst = 1024 / kLdsRun;
  auto plan_row = [&](int i) { return kRowsPerInst * (i * 4 + wave) + lane / kPieces; };
  const int piece = lane % kPieces;
  uint32_t w_off[kWI];
#pragma unroll
  for (int i = 0; i < kWI; ++i) {
    const int row = plan_row(i);
    w_off[i] = (uint32_t)(((size_t)row * K + (piece ^ (row & 15)) * 8) * 2);
  }
  const uint16_t* w_base = W + ((size_t)e * N + (size_t)cb0 * 64) * K;

  const int nst_all = K / kLdsStageK;
  const int s0 = (int)((long)split * nst_all / splits);
  const int nst = (int)((long)(split + 1) * nst_all / splits) - s0;
  const int total = ncb * nst;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;

  // The W part of stage t of a group's sequence: column block t / nst, k stage
  // t % nst.  It depends on the block index only, so with `early` (the host
  // sets it when there are at least as many rows as experts, so few experts
  // are empty) the first group's first kLdsDepth - 1 W stages are issued
  // before the routing is read: their latency overlaps the dependent loads of
  // the offsets and gathered row indices.  A block whose expert turns out to
  // have no rows has then read those stages (at most 64 KB) for nothing, and
  // waits for them before it exits.
  auto issue_w = [&](int slot, int t) {
    const int j = t / nst, st = t - j * nst;
    const int k0 = (s0 + st) * kLdsStageK;
    const uint32_t wl = lds0 + slot * kWBytes;
    const uint16_t* wb = w_base + (size_t)j * 64 * K + k0;
#pragma unroll
    for (int i = 0; i < kWI; ++i) load_lds16_sv(wb, w_off[i], wl + (i * 4 + wave) * 1024);
  };
  if (early) {
#pragma unroll
    for (int d = 0; d < kLdsDepth - 1; ++d)
      if (d < total) issue_w(d, d);
  }

  const int seg0 = offsets[e], seg1 = offsets[e + 1];
  const int g0 = kLoopGroups ? 0 : blockIdx.z / splits;
  const int g1 = kLoopGroups ? (seg1 - seg0 + kMR - 1) / kMR : g0 + 1;
  if (seg0 + g0 * kMR >= seg1) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));   // no DMA into LDS outlives the block
    return;
  }
  constexpr int kQ = kPieces / 4;                // MFMAs per m-tile and plane per stage
  // Loads complete in issue order: in steady state kLdsDepth - 2 stages were
  // issued after stage t, so waiting for at most that many instructions lands
  // it; near the end (fewer issued after it) wait for all.
  constexpr int kSteadyWait = (kLdsDepth - 2) * (kWI + kAI);

  for (int g = g0; g < g1; ++g) {
    const int r0 = seg0 + g * kMR;
    const int r1 = min(seg1, r0 + kMR);
    const int mt_active = (r1 - r0 + 15) >> 4;
    if (g > g0) {
      // The previous group's stores drain before this group's loads are
      // counted, and every wave is past its last LDS read before the ring
      // is reused.
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
      __syncthreads();
    }
    // A plan: instruction i covers plane (row' / kMR), row row' % kMR.
    int arow[kAI];
#pragma unroll
    for (int i = 0; i < kAI; ++i) arow[i] = min(r0 + plan_row(i) % kMR, r1 - 1);
    if constexpr (UP) a_rows<kAI>(gather, gather_k, arow);
    const uint16_t* a_src[kAI];
#pragma unroll
    for (int i = 0; i < kAI; ++i) {
      const int pr = plan_row(i);
      const uint16_t* base = (kPlanes == 2 && pr >= kMR) ? A_lo : A;
      a_src[i] = base + (size_t)arow[i] * K + ((piece ^ ((pr % kMR) & 15)) * 8);
    }

    // Stage t of the group's sequence: its A part, then its W part.
    auto issue_a = [&](int slot, int t) {
      const int st = t - (t / nst) * nst;
      const int k0 = (s0 + st) * kLdsStageK;
      const uint32_t al = lds0 + kLdsDepth * kWBytes + slot * kABytes;
#pragma unroll
      for (int i = 0; i < kAI; ++i) load_lds16_raw(a_src[i] + k0, al + (i * 4 + wave) * 1024);
    };
    auto issue = [&](int slot, int t) {
      issue_a(slot, t);
      issue_w(slot, t);
    };
    // Every fragment read of the stage is issued before its MFMAs; the active
    // m-tile count picks one of two unrolled bodies (a uniform branch).
    auto compute = [&](int slot, f32x4 (&acc_j)[NMT]) {
      const uint8_t* ws = lds + slot * kWBytes;
      const uint8_t* as = lds + kLdsDepth * kWBytes + slot * kABytes;
      const int wrow = wave * 16 + fr;
      u32x4 wf[kQ];
#pragma unroll
      for (int q = 0; q < kQ; ++q) wf[q] = ld16(ws + wrow * kLdsRun + (((q * 4 + fc) ^ (wrow & 15)) << 4));
      auto tiles = [&](auto mt_c) {
        constexpr int MT = decltype(mt_c)::value;
        u32x4 af[kPlanes][MT][kQ];
#pragma unroll
        for (int p = 0; p < kPlanes; ++p)
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            const int row = i * 16 + fr;
#pragma unroll
            for (int q = 0; q < kQ; ++q)
              af[p][i][q] = ld16(as + p * kAPlane + row * kLdsRun + (((q * 4 + fc) ^ (row & 15)) << 4));
          }
#pragma unroll
        for (int q = 0; q < kQ; ++q)
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int p = 0; p < kPlanes; ++p) acc_j[i] = mfma_bf16(af[p][i][q], wf[q], acc_j[i]);
      };
      if (NMT == 1 || mt_active == 1) tiles(std::integral_constant<int, 1>{});
      else tiles(std::integral_constant<int, NMT>{});
    };

    // The column-block loop is unrolled so that each one's accumulators stay
    // in registers.
    f32x4 acc[kLdsMaxCpb][NMT];
#pragma unroll
    for (int j = 0; j < kLdsMaxCpb; ++j)
#pragma unroll
      for (int i = 0; i < NMT; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Prologue.  First group with `early`: the W parts are in flight already,
    // so the issue order is W0 W1 A0 A1 and stage 0 has landed once at most
    // A1's kAI instructions are outstanding.  Otherwise A0 W0 A1 W1, as in the
    // loop.
    const bool w_early = early && g == g0;
#pragma unroll
    for (int d = 0; d < kLdsDepth - 1; ++d) {
      if (d < total) {
        if (w_early) issue_a(d, d);
        else issue(d, d);
      }
    }
#pragma unroll
    for (int j = 0; j < kLdsMaxCpb; ++j) {
      if (j < ncb) {
        for (int st = 0; st < nst; ++st) {
          const int t = j * nst + st;
          if (t + kLdsDepth - 2 < total) {
            if (t == 0 && w_early) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((kLdsDepth - 2) * kAI));
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kSteadyWait));
          } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
          }
          __syncthreads();
          if (t + kLdsDepth - 1 < total) issue((t + kLdsDepth - 1) % kLdsDepth, t + kLdsDepth - 1);
          compute(t % kLdsDepth, acc[j]);
        }
      }
    }

    // Epilogue, as ffn_stream_kernel's, per column block: lane (fr, fc) holds
    // column 64 * (cb0 + j) + 16 * wave + fr of rows 4fc + v of each m-tile.
    // The bias words of every column block are loaded first (clamped indices,
    // one wait), not one load and wait per column block behind the stores.
    float bvs[kLdsMaxCpb];
#pragma unroll
    for (int j = 0; j < kLdsMaxCpb; ++j) bvs[j] = 0.f;
    if (bias && split == 0) {
      uint16_t braw[kLdsMaxCpb];
#pragma unroll
      for (int j = 0; j < kLdsMaxCpb; ++j)
        braw[j] = bias[(size_t)e * N + (cb0 + min(j, ncb - 1)) * 64 + wave * 16 + fr];
#pragma unroll
      for (int j = 0; j < kLdsMaxCpb; ++j) bvs[j] = bf16_to_f32(braw[j]);
    }
#pragma unroll
    for (int j = 0; j < kLdsMaxCpb; ++j) {
      if (j < ncb) {
        const int col = (cb0 + j) * 64 + wave * 16 + fr;
#pragma unroll
        for (int i = 0; i < NMT; ++i) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = r0 + i * 16 + 4 * fc + v;
            if (row < r1) {
              if (splits > 1)
                partial[((size_t)split * rows_cap + row) * N + col] = acc[j][i][v] + bvs[j];
              else
                emit<uint16_t, UP, SPLIT>(out, out_plane, (size_t)row * N + col, acc[j][i][v] + bvs[j]);
            }
          }
        }
      }
    }
  }
}

// Finish a split-k product: out[r][c] = epilogue(sum over splits s of
// partial[s][r][c]), summed in split order; rows r < offsets[E] only.  Each
// thread handles four consecutive columns.
template <typename T, bool UP, bool SPLIT>
__global__ __launch_bounds__(256) void ffn_splitk_reduce(
    const float* __restrict__ partial, const int32_t* __restrict__ offsets, int E, int N,
    int splits, int rows_cap, void* __restrict__ out, size_t out_plane) {
  const int R = offsets[E];
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;   // quad index
  const int quads = N / 4;
  const int row = (int)(q / quads), c = (int)(q % quads) * 4;
  if (row >= R) return;
  f32x4 v = *reinterpret_cast<const f32x4*>(partial + (size_t)row * N + c);
  for (int sp = 1; sp < splits; ++sp)
    v += *reinterpret_cast<const f32x4*>(partial + ((size_t)sp * rows_cap + row) * N + c);
#pragma unroll
  for (int u = 0; u < 4; ++u) emit<T, UP, SPLIT>(out, out_plane, (size_t)row * N + c + u, v[u]);
}

// Launch shape of the weight-streaming kernel, decided on the host from the
// descriptor alone (never from device data).
struct StreamShape {
  int nmt, nwn, groups, splits;
  bool lds;   // ffn_stream_lds_kernel (bf16, at most 32 rows per expert)
};
static StreamShape stream_shape(bool bf16, bool up, bool split, int E, int N, int K,
                                int max_rows_per_expert) {
  // Rows per block: 16/32/64/160, the smallest covering the host's bound on
  // any expert's rows (capped at 160); more row groups (grid z) cover the rest.
  // Empty m-tiles issue no MFMA, so a generous block costs registers only.
  StreamShape sh{};
  const int bound = max_rows_per_expert;
  sh.nmt = bound <= 16 ? 1 : bound <= 32 ? 2 : bound <= 64 ? 4 : 10;
  sh.groups = (bound + 16 * sh.nmt - 1) / (16 * sh.nmt);
  // bf16 layers with at most 32 rows per expert stream through LDS; the
  // second product there takes 16-row groups, looped inside the block.
  sh.lds = bf16 && bound <= 32 && K % kLdsStageK == 0 && N % 64 == 0;
  if (sh.lds && !up) {
    sh.nmt = 1;
    sh.groups = 1;
  }
  sh.nwn = (!sh.lds && sh.nmt < 10 && (long)E * (N / 128) >= 1024) ? 2 : 1;
  // Split the k range when the grid is too small to keep enough weight loads
  // in flight (fewer than kStreamMinBlocks / 2 blocks), up to about
  // kStreamMinBlocks blocks and keeping >= 8 chunks per split; the partial sums
  // cost rows x N x 4 B per split plus a reduce launch, which does not pay for
  // grids already above that (measured on MI355X).
  const int chunk = !bf16 ? 64 : (split && !up) ? 64 : 128;
  const long blocks = (long)(N / (64 * sh.nwn)) * E * sh.groups;
  const int max_splits = std::max(1, std::min(8, K / chunk / 8));
  sh.splits = 1;
  if (sh.lds) {
    // One persistent block per CU: split only when there are fewer column
    // blocks than CUs.
    const long cus = kXcds * kCusPerXcd;
    if (blocks < cus) sh.splits = (int)std::min<long>(max_splits, (cus + blocks - 1) / blocks);
  } else if (blocks < kStreamMinBlocks / 2) {
    while (sh.splits < max_splits && blocks * sh.splits < kStreamMinBlocks) ++sh.splits;
  }
  return sh;
}

size_t ffn_partial_bytes(int path, bool bf16, bool up, bool split, int E, int N, int K,
                         int max_rows_per_expert, int max_rows) {
  if (path == MOE_FFN_TILED) return (size_t)kPartialSlots * kPartialTileFloats * sizeof(float);
  const StreamShape sh = stream_shape(bf16, up, split, E, N, K, max_rows_per_expert);
  return sh.splits > 1 ? (size_t)sh.splits * max_rows * N * sizeof(float) : 0;
}

template <typename T, bool UP, bool SPLIT, int NMT>
static void launch_stream_nmt(const FfnArgs& a, const StreamShape& sh, hipStream_t s) {
  const T* A = static_cast<const T*>(a.a);
  const T* A_lo = SPLIT && !UP ? A + a.plane : nullptr;
  const T* W = static_cast<const T*>(a.w);
  const T* B = static_cast<const T*>(a.bias);
  const int z = sh.groups * sh.splits;
  if (sh.nwn == 2) {
    dim3 grid(a.N / 128, a.E, z);
    ffn_stream_kernel<T, UP, SPLIT, NMT, 2><<<grid, 256, 0, s>>>(
        A, A_lo, a.offsets, W, B, a.out, a.plane, a.E, a.N, a.K, sh.splits, a.partial, a.max_rows,
        a.gather, a.gather_k);
  } else {
    dim3 grid(a.N / 64, a.E, z);
    ffn_stream_kernel<T, UP, SPLIT, NMT, 1><<<grid, 256, 0, s>>>(
        A, A_lo, a.offsets, W, B, a.out, a.plane, a.E, a.N, a.K, sh.splits, a.partial, a.max_rows,
        a.gather, a.gather_k);
  }
  if (sh.splits > 1 && !(a.defer_reduce && !UP)) {
    const size_t quads = (size_t)a.max_rows * (a.N / 4);
    ffn_splitk_reduce<T, UP, SPLIT><<<(unsigned)((quads + 255) / 256), 256, 0, s>>>(
        a.partial, a.offsets, a.E, a.N, sh.splits, a.max_rows, a.out, a.plane);
  }
}

template <bool UP, bool SPLIT, int NMT>
static void launch_stream_lds(const FfnArgs& a, const StreamShape& sh, hipStream_t s) {
  // One block per CU: each block streams cpb column blocks of its expert, cpb
  // the smallest that brings the grid down to one block per CU (at most
  // kLdsMaxCpb).
  const long cbs = (long)(a.N / 64) * a.E * sh.groups * sh.splits;
  const int cpb = (int)std::min<long>(kLdsMaxCpb, std::max<long>(1, (cbs + kXcds * kCusPerXcd - 1) /
                                                                       (kXcds * kCusPerXcd)));
  const dim3 grid((a.N / 64 + cpb - 1) / cpb, a.E, sh.groups * sh.splits);
  const uint16_t* A = static_cast<const uint16_t*>(a.a);
  ffn_stream_lds_kernel<UP, SPLIT, NMT><<<grid, 256, 0, s>>>(
      A, (SPLIT && !UP) ? A + a.plane : nullptr, a.offsets, static_cast<const uint16_t*>(a.w),
      static_cast<const uint16_t*>(a.bias), a.out, a.plane, a.E, a.N, a.K, sh.splits, a.partial,
      a.max_rows, a.gather, a.gather_k, cpb, a.max_rows >= a.E ? 1 : 0);
  if (sh.splits > 1 && !(a.defer_reduce && !UP)) {
    const size_t quads = (size_t)a.max_rows * (a.N / 4);
    ffn_splitk_reduce<uint16_t, UP, SPLIT><<<(unsigned)((quads + 255) / 256), 256, 0, s>>>(
        a.partial, a.offsets, a.E, a.N, sh.splits, a.max_rows, a.out, a.plane);
  }
}

template <typename T, bool UP, bool SPLIT>
static void launch_stream(const FfnArgs& a, hipStream_t s) {
  const StreamShape sh = stream_shape(a.bf16, UP, SPLIT, a.E, a.N, a.K, a.max_rows_per_expert);
  if constexpr (std::is_same<T, uint16_t>::value) {
    if (sh.lds) {
      if constexpr (UP) {
        if (sh.nmt == 1) launch_stream_lds<UP, SPLIT, 1>(a, sh, s);
        else launch_stream_lds<UP, SPLIT, 2>(a, sh, s);
      } else {
        launch_stream_lds<UP, SPLIT, 1>(a, sh, s);
      }
      return;
    }
  }
  switch (sh.nmt) {
    case 1: launch_stream_nmt<T, UP, SPLIT, 1>(a, sh, s); break;
    case 2: launch_stream_nmt<T, UP, SPLIT, 2>(a, sh, s); break;
    case 4: launch_stream_nmt<T, UP, SPLIT, 4>(a, sh, s); break;
    default: launch_stream_nmt<T, UP, SPLIT, 10>(a, sh, s); break;
  }
}

__global__ void dense_offsets_kernel(int32_t* __restrict__ offsets, int rows) {
  if (threadIdx.x == 0) {
    offsets[0] = 0;
    offsets[1] = rows;
  }
}

hipError_t launch_dense_offsets(int32_t* offsets, int rows, hipStream_t s) {
  dense_offsets_kernel<<<1, 64, 0, s>>>(offsets, rows);
  return hipGetLastError();
}


// W stages: 3 for 256-row tiles (MFMA-bound: the loads hide behind the
// matrix work); for the smaller, weight-bound tiles as many as the LDS holds
// (at most 8), to keep more weight bytes in flight per CU.
constexpr int tile_w_stages(int bm, int bn, int planes) {
  return bm == 256 ? 3 : std::min(8, (160 * 1024 - 2 * bm * 128 * planes) / (bn * 128));
}

template <bool UP, bool SPLIT, int BM, int BN>
static void launch_tiled_t(const FfnArgs& a, hipStream_t s) {
  constexpr int WM = 2;
  // The split first product on 128 x 128 tiles runs two blocks per CU (80 KB
  // of LDS each, three W stages): one block's two-plane GELU epilogue then
  // overlaps the other's main loop.
  constexpr bool kTwoPerCu = UP && SPLIT && BM == 128 && BN == 128;
  constexpr int WS = kTwoPerCu ? 3 : tile_w_stages(BM, BN, (SPLIT && !UP) ? 2 : 1);
  constexpr int OCC = kTwoPerCu ? 2 : 1;
  // Upper bound on tiles: sum_e ceil(count_e/BM) <= ceil(R/BM) + E; the grid
  // is a multiple of the XCD count and blocks past the real tile count exit.
  // Per XCD at most ceil(max_mt * ntn / 8) entries, plus at most one round of
  // tail-split blocks; blocks without a job exit at once.
  const int max_mt = (a.max_rows + BM - 1) / BM + a.E;
  const int per_xcd = (max_mt * ((a.N + BN - 1) / BN) + kXcds - 1) / kXcds + 1 + kCusPerXcd;
  const uint16_t* A = static_cast<const uint16_t*>(a.a);
  const uint16_t* A_lo = (SPLIT && !UP) ? A + a.plane : nullptr;
  const uint16_t* W = static_cast<const uint16_t*>(a.w);
  const uint16_t* B = static_cast<const uint16_t*>(a.bias);
  ffn_tiled_kernel<UP, SPLIT, BM, BN, WM, WS, OCC><<<per_xcd * kXcds, 256, 0, s>>>(
      A, A_lo, a.offsets, W, B, a.out, a.plane, a.E, a.N, a.K, a.partial, a.gather, a.gather_k);
  // Only a k range of at least kSplitMinSteps steps is ever split (tile_job);
  // shorter ones need no reduce launch (measured: ~5 us per product).
  if (a.K / kTBK >= kSplitMinSteps)
    ffn_tile_reduce<UP, SPLIT, BM, BN><<<kPartialSlots, 256, 0, s>>>(a.offsets, B, a.out, a.plane,
                                                                     a.E, a.N, a.K, a.partial);
}

// Column tile: 256 when N >= 256, else 128.  A 256-wide tile moves half the
// A bytes per MFMA of a 128-wide one; when N is an odd multiple of 128 the
// last n-tile is half padding, which costs less than 128-wide tiles
// throughout.  The split second product (128-row tiles only) fits its two A
// planes and three W stages in the LDS at 256 columns.  The split first
// product takes 128 columns so that two blocks fit on a CU (measured faster
// than one 256-wide block).
template <bool UP, bool SPLIT, int BM>
static void launch_tiled_bm(const FfnArgs& a, hipStream_t s) {
  constexpr bool kWide = !(UP && SPLIT);
  if (kWide && a.N >= 256) launch_tiled_t<UP, SPLIT, BM, kWide ? 256 : 128>(a, s);
  else launch_tiled_t<UP, SPLIT, BM, 128>(a, s);
}

// Rows per tile (FfnArgs::tile_rows, chosen by the caller): 256 or 192 (one
// h plane only) or 128, all run as 2 x 2 waves.
template <bool UP, bool SPLIT>
static void launch_tiled(const FfnArgs& a, hipStream_t s) {
  if constexpr (!SPLIT) {
    if (a.tile_rows == 256) {
      launch_tiled_bm<UP, false, 256>(a, s);
      return;
    }
    if (a.tile_rows == 192) {
      launch_tiled_bm<UP, false, 192>(a, s);
      return;
    }
  }
  launch_tiled_bm<UP, SPLIT, 128>(a, s);
}

int ffn_k_splits(const FfnArgs& a) {
  if (a.path == MOE_FFN_TILED) return 1;
  return stream_shape(a.bf16, a.up, a.split, a.E, a.N, a.K, a.max_rows_per_expert).splits;
}

hipError_t launch_ffn(const FfnArgs& a, hipStream_t s) {
  if (a.path == MOE_FFN_TILED) {
    if (a.split) {
      if (a.up) launch_tiled<true, true>(a, s);
      else launch_tiled<false, true>(a, s);
    } else {
      if (a.up) launch_tiled<true, false>(a, s);
      else launch_tiled<false, false>(a, s);
    }
  } else if (a.bf16) {
    if (a.split) {
      if (a.up) launch_stream<uint16_t, true, true>(a, s);
      else launch_stream<uint16_t, false, true>(a, s);
    } else {
      if (a.up) launch_stream<uint16_t, true, false>(a, s);
      else launch_stream<uint16_t, false, false>(a, s);
    }
  } else {
    if (a.up) launch_stream<float, true, false>(a, s);
    else launch_stream<float, false, false>(a, s);
  }
  return hipGetLastError();
}

}  // namespace moe
