// Grouped expert FFN of the MoE layer on gfx950.
//
// Each expert is Linear(d -> d_ff) -> GELU -> Linear(d_ff -> d) (web page
// "Mixture of Experts: Scaling Parameters Without Scaling Compute", section
// "The MoE layer", the listing's expert).  After dispatch the rows of expert e
// are the contiguous segment [offsets[e], offsets[e+1]) of A, so each expert is
// one dense product out[seg] = A[seg] W_e^T (+ bias_e) with W_e stored
// [N][K] (K contiguous, like A).  Experts with no rows do no work.
//
// Two kernels, chosen on the host from a bound on rows per expert (the
// device-side counts are never read back):
//   * ffn_tiled_kernel  -- many rows per expert (prefill): 128x128 output
//     tiles, both operands staged through LDS in 64-wide k-steps, bf16 MFMA
//     16x16x32 with fp32 accumulation, double-buffered with one barrier per
//     k-step.  A 1-D grid walks (m-tile, n-tile) with the m-tiles of all
//     experts laid end to end; each block finds its expert from `offsets`.
//   * ffn_stream_kernel -- few rows per expert (decode, many small experts):
//     each wave streams its own 16*NWN rows of W_e straight from HBM into
//     registers in the MFMA operand layout, while the block's (at most
//     16*NMT) rows of A are staged through LDS once per k-chunk and shared by
//     the four waves.  Weight bytes are read once.
// The first product applies bias + exact-erf GELU in its epilogue and stores
// dtype h; the second adds its bias and stores fp32 o.
#include "device_common.h"
#include "kernels.h"
#include "../../include/moe_mi355x.h"

namespace moe {

// Find the expert owning global m-tile `mt` when every expert's rows are cut
// into ceil(count/bm) tiles laid end to end.  Returns false past the last tile.
__device__ __forceinline__ bool find_mtile(const int32_t* __restrict__ offsets, int E, int bm,
                                           int mt, int& e_out, int& r0, int& r1) {
  int cum = 0;
  int lo = offsets[0];
  for (int e = 0; e < E; ++e) {
    const int hi = offsets[e + 1];
    const int nt = (hi - lo + bm - 1) / bm;
    if (mt < cum + nt) {
      e_out = e;
      r0 = lo + (mt - cum) * bm;
      r1 = min(hi, r0 + bm);
      return true;
    }
    cum += nt;
    lo = hi;
  }
  return false;
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

// ---------------------------------------------------------------------------
// LDS-tiled kernel (bf16): 128 x 128 x 64 block tile, 4 waves as 2 x 2, each
// wave 64 x 64 = 4 x 4 MFMA tiles.
// LDS tile layout: row-major, 128 B per row (64 bf16), the eight 16-byte chunks
// of row r stored at chunk position (c ^ (r & 7)) so that both the row-wise
// stores and the MFMA fragment reads (8 rows x same chunk) are bank-conflict
// free.
// ---------------------------------------------------------------------------
constexpr int kTBM = 128, kTBN = 128, kTBK = 64;

template <bool UP>
__global__ __launch_bounds__(256, 2) void ffn_tiled_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets,
    const uint16_t* __restrict__ W, const uint16_t* __restrict__ bias, void* __restrict__ out,
    int E, int N, int K, int max_mt) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kTBM * 128];   // [stage][A|B]

  const int L = blockIdx.x;
  const int mt = L % max_mt, nt = L / max_mt;
  int e, r0, r1;
  if (!find_mtile(offsets, E, kTBM, mt, e, r0, r1)) return;
  const int n0 = nt * kTBN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 15, fc = lane >> 4;

  // Global -> LDS mapping: thread loads rows (tid/8) + 32*i, chunk tid%8.
  const int lrow = tid >> 3, lch = tid & 7;
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
  int st_off[4];
  const uint16_t* Wexp = W + (size_t)e * N * K;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = lrow + 32 * i;
    a_src[i] = A + (size_t)min(r0 + row, r1 - 1) * K + lch * 8;
    b_src[i] = Wexp + (size_t)(n0 + row) * K + lch * 8;
    st_off[i] = row * 128 + ((lch ^ (row & 7)) << 4);
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ld16(a_src[i] + k0);
      rb[i] = ld16(b_src[i] + k0);
    }
  };
  auto lstore = [&](int stage) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st16(&lds[stage][0][st_off[i]], ra[i]);
      st16(&lds[stage][1][st_off[i]], rb[i]);
    }
  };

  const int nk = K / kTBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kTBK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 64 + i * 16 + fr;
        af[i] = ld16(&lds[cur][0][row * 128 + ((((ks << 2) | fc) ^ (row & 7)) << 4)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wn * 64 + j * 16 + fr;
        bfr[j] = ld16(&lds[cur][1][row * 128 + ((((ks << 2) | fc) ^ (row & 7)) << 4)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds column fr of each 16x16 tile, rows 4*fc + v.
  const uint16_t* bexp = bias ? bias + (size_t)e * N : nullptr;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = n0 + wn * 64 + j * 16 + fr;
    const float bv = bexp ? bf16_to_f32(bexp[col]) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = r0 + wm * 64 + i * 16 + 4 * fc + v;
        if (row < r1) store_out<uint16_t, UP>(out, (size_t)row * N + col, acc[i][j][v] + bv);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Weight-streaming kernel.  Block = 4 waves; wave w owns the 16*NWN output
// columns n0 + w*16*NWN + [0, 16*NWN); the block owns rows
// [offsets[e] + g*16*NMT, ...) of expert e = blockIdx.y, g = blockIdx.z.
// Per k-chunk:
//   - the block stages its A rows into LDS (16 B per thread per m-tile); each
//     row's chunk is 256 B (two 128 B planes when the second product reads a
//     split h = hi + lo), its 16 B pieces stored at (piece ^ (row & mask)) so
//     the fragment reads (16 rows x same piece) are conflict free;
//   - each wave loads its W rows for the next chunk into registers: lane l
//     reads row (l % 16) of its n-tile and KQ consecutive 16 B pieces starting
//     at piece (l / 16) * KQ;
//   - MFMA q of the chunk uses the lane's q-th piece of A (and of A's low
//     term when h is split) and of W.
// m-tiles past the block's last row issue no MFMA, so padding costs nothing.
// ---------------------------------------------------------------------------
template <typename T, bool UP, bool SPLIT, int NMT, int NWN>
__global__ __launch_bounds__(256) void ffn_stream_kernel(
    const T* __restrict__ A, const T* __restrict__ A_lo, const int32_t* __restrict__ offsets,
    const T* __restrict__ W, const T* __restrict__ bias, void* __restrict__ out,
    size_t out_plane, int E, int N, int K) {
  constexpr bool kTwoA = SPLIT && !UP;             // A operand is split h
  constexpr int kQ = kTwoA ? 2 : 4;                // 16 B pieces per lane per chunk
  constexpr int kPerVec = 16 / sizeof(T);
  constexpr int kChunk = 4 * kQ * kPerVec;         // 128 bf16, 64 (split) or 64 fp32
  constexpr int kPieces = 4 * kQ;                  // pieces per row per plane
  constexpr int kRowBytes = kPieces * 16;
  constexpr int kMR = 16 * NMT;
  constexpr int kPlaneBytes = kMR * kRowBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kMR * 256];

  const int e = blockIdx.y;
  const int seg0 = offsets[e], seg1 = offsets[e + 1];
  const int r0 = seg0 + blockIdx.z * kMR;
  if (r0 >= seg1) return;
  const int r1 = min(seg1, r0 + kMR);
  const int mt_active = (r1 - r0 + 15) >> 4;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fc = lane >> 4;
  const int n0 = blockIdx.x * (64 * NWN) + wave * 16 * NWN;

  // A staging: vector v = tid + 256*i covers row v/16 and 16 B piece v%16
  // (plane (v%16)/8 when A is split).
  const T* a_src[NMT];
  int a_st[NMT];
  bool a_on[NMT];
#pragma unroll
  for (int i = 0; i < NMT; ++i) {
    const int v = tid + 256 * i;
    const int row = v >> 4, within = v & 15;
    const int plane = kTwoA ? (within >> 3) : 0;
    const int pc = kTwoA ? (within & 7) : within;
    const T* base = (kTwoA && plane) ? A_lo : A;
    a_src[i] = base + (size_t)min(r0 + row, r1 - 1) * K + pc * kPerVec;
    a_st[i] = plane * kPlaneBytes + row * kRowBytes + ((pc ^ (row & (kPieces - 1))) << 4);
    a_on[i] = (row >> 4) < mt_active;
  }
  const T* w_src[NWN];
  const T* Wexp = W + (size_t)e * N * K;
#pragma unroll
  for (int j = 0; j < NWN; ++j) w_src[j] = Wexp + (size_t)(n0 + j * 16 + fr) * K + fc * kQ * kPerVec;

  f32x4 acc[NMT][NWN];
#pragma unroll
  for (int i = 0; i < NMT; ++i)
#pragma unroll
    for (int j = 0; j < NWN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[NMT];
  u32x4 wcur[NWN][kQ], wnext[NWN][kQ];
  auto aload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NMT; ++i)
      if (a_on[i]) ra[i] = ld16(a_src[i] + k0);
  };
  auto astore = [&](int stage) {
#pragma unroll
    for (int i = 0; i < NMT; ++i)
      if (a_on[i]) st16(&lds[stage][a_st[i]], ra[i]);
  };
  auto wload = [&](u32x4 (&dst)[NWN][kQ], int k0) {
#pragma unroll
    for (int j = 0; j < NWN; ++j)
#pragma unroll
      for (int q = 0; q < kQ; ++q) dst[j][q] = ld16(w_src[j] + k0 + q * kPerVec);
  };

  const int nch = K / kChunk;
  aload(0);
  wload(wcur, 0);
  astore(0);
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    const int cur = ch & 1;
    const bool more = ch + 1 < nch;
    if (more) {
      aload((ch + 1) * kChunk);
      wload(wnext, (ch + 1) * kChunk);
    }
#pragma unroll
    for (int i = 0; i < NMT; ++i) {
      if (i < mt_active) {
        const int row = i * 16 + fr;
        u32x4 af[kQ], al[kQ];
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
          const int off = row * kRowBytes + ((((fc * kQ) + q) ^ (row & (kPieces - 1))) << 4);
          af[q] = ld16(&lds[cur][off]);
          if constexpr (kTwoA) al[q] = ld16(&lds[cur][kPlaneBytes + off]);
        }
#pragma unroll
        for (int j = 0; j < NWN; ++j) {
          if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int q = 0; q < kQ; ++q) {
              acc[i][j] = mfma_bf16(af[q], wcur[j][q], acc[i][j]);
              if constexpr (kTwoA) acc[i][j] = mfma_bf16(al[q], wcur[j][q], acc[i][j]);
            }
          } else {
#pragma unroll
            for (int q = 0; q < kQ; ++q)
#pragma unroll
              for (int u = 0; u < 4; ++u)
                acc[i][j] = mfma_f32(__uint_as_float(af[q][u]), __uint_as_float(wcur[j][q][u]),
                                     acc[i][j]);
          }
        }
      }
    }
    if (more) astore(cur ^ 1);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int j = 0; j < NWN; ++j)
#pragma unroll
        for (int q = 0; q < kQ; ++q) wcur[j][q] = wnext[j][q];
    }
  }

  const T* bexp = bias ? bias + (size_t)e * N : nullptr;
#pragma unroll
  for (int j = 0; j < NWN; ++j) {
    const int col = n0 + j * 16 + fr;
    const float bv = bexp ? Elem<T>::to_f32(bexp[col]) : 0.f;
#pragma unroll
    for (int i = 0; i < NMT; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = r0 + i * 16 + 4 * fc + v;
        if (row < r1) {
          const size_t idx = (size_t)row * N + col;
          if constexpr (UP && SPLIT) {
            const float g = gelu_erf(acc[i][j][v] + bv);
            const uint16_t hi = f32_to_bf16(g);
            const uint16_t lo = f32_to_bf16(g - bf16_to_f32(hi));
            static_cast<uint16_t*>(out)[idx] = hi;
            static_cast<uint16_t*>(out)[out_plane + idx] = lo;
          } else {
            store_out<T, UP>(out, idx, acc[i][j][v] + bv);
          }
        }
      }
    }
  }
}

template <typename T, bool UP, bool SPLIT, int NMT>
static void launch_stream_nwn(const FfnArgs& a, int nwn, int groups, hipStream_t s) {
  const T* A = static_cast<const T*>(a.a);
  const T* A_lo = SPLIT && !UP ? A + a.plane : nullptr;
  const T* W = static_cast<const T*>(a.w);
  const T* B = static_cast<const T*>(a.bias);
  if (nwn == 2) {
    dim3 grid(a.N / 128, a.E, groups);
    ffn_stream_kernel<T, UP, SPLIT, NMT, 2><<<grid, 256, 0, s>>>(A, A_lo, a.offsets, W, B, a.out,
                                                                 a.plane, a.E, a.N, a.K);
  } else {
    dim3 grid(a.N / 64, a.E, groups);
    ffn_stream_kernel<T, UP, SPLIT, NMT, 1><<<grid, 256, 0, s>>>(A, A_lo, a.offsets, W, B, a.out,
                                                                 a.plane, a.E, a.N, a.K);
  }
}

template <typename T, bool UP, bool SPLIT>
static void launch_stream(const FfnArgs& a, hipStream_t s) {
  // Rows per block: 16/32/64/160, the smallest covering the host's bound on
  // any expert's rows (capped at 160); more row groups (grid z) cover the rest.
  // Empty m-tiles issue no MFMA, so a generous block costs registers only.
  const int bound = a.max_rows_per_expert;
  const int nmt = bound <= 16 ? 1 : bound <= 32 ? 2 : bound <= 64 ? 4 : 10;
  const int groups = (bound + 16 * nmt - 1) / (16 * nmt);
  const int nwn = (nmt < 10 && (long)a.E * (a.N / 128) >= 1024) ? 2 : 1;
  switch (nmt) {
    case 1: launch_stream_nwn<T, UP, SPLIT, 1>(a, nwn, groups, s); break;
    case 2: launch_stream_nwn<T, UP, SPLIT, 2>(a, nwn, groups, s); break;
    case 4: launch_stream_nwn<T, UP, SPLIT, 4>(a, nwn, groups, s); break;
    default: launch_stream_nwn<T, UP, SPLIT, 10>(a, nwn, groups, s); break;
  }
}

hipError_t launch_ffn(const FfnArgs& a, hipStream_t s) {
  if (a.path == MOE_FFN_TILED) {
    const int max_mt = (a.max_rows + kTBM - 1) / kTBM + a.E;
    const int grid = max_mt * (a.N / kTBN);
    const uint16_t* A = static_cast<const uint16_t*>(a.a);
    const uint16_t* W = static_cast<const uint16_t*>(a.w);
    const uint16_t* B = static_cast<const uint16_t*>(a.bias);
    if (a.up)
      ffn_tiled_kernel<true><<<grid, 256, 0, s>>>(A, a.offsets, W, B, a.out, a.E, a.N, a.K, max_mt);
    else
      ffn_tiled_kernel<false><<<grid, 256, 0, s>>>(A, a.offsets, W, B, a.out, a.E, a.N, a.K, max_mt);
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
