// Host-side launch interface between the C ABI (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct RouterArgs {
  bool bf16;
  const void* x;
  const void* w_router;
  const float* b_router;
  const float* b_select;   // selection-only bias or null
  int T, d, E, k, renorm;
  int32_t* topk_idx;
  float* topk_w;
  double* part_psum;       // [router_blocks(T)][E]
  int32_t* part_top1;      // [router_blocks(T)][E]
  double* part_z;          // [router_blocks(T)]
  float* part_logit;       // router_small_part_bytes(): partial logit tiles of small batches
  int32_t* top1_count;     // optional
  float* prob_mean;        // optional
  float* aux;              // optional
  float* z_loss;           // optional
  int32_t* rr_rank;        // reroute policy, else null: [T][64][2], position p of token t holds
                           // {expert of rank p, bits of the weight it would get} for p < E;
                           // the partials are then reduced by launch_reroute
  int32_t* rounds_zero;    // optional: set to 0 (no reroute runs)
  // Optional dispatch layout of a small layer (T*k <= 8192, drop policy), computed by
  // the aux reduction block right after the router: counts, offsets, dest and src as
  // the permute writes them, with `capacity` (0 = none).
  bool perm;
  int capacity;
  int32_t* counts;
  int32_t* offsets;
  int32_t* dest;
  int32_t* src;
};
// Whether RouterArgs::perm may be used for T*k assignments.
bool router_can_permute(int assignments);
int router_blocks(int T);
// Bytes of RouterArgs::part_logit a router launch needs (0 when its path uses none).
size_t router_small_part_bytes(int T, int E, bool rr);
// Blocks (partial-sum rows) a router launch for T tokens and E experts uses.
int router_launch_blocks(int T, int E);
hipError_t launch_router(const RouterArgs& a, hipStream_t s);

struct RerouteArgs {
  const int32_t* rank;     // [T][64][2] from the router (RouterArgs::rr_rank)
  int T, k, E, capacity;
  int32_t* topk_idx;       // in: router choices; out: serving expert or -1 if dropped
  float* topk_w;           // out: weight of the serving expert, 0 if dropped
  int32_t* lists;          // [4][T] scratch: two lists (used in turn) of tokens with rejected
                           // slots: token ids and (cursor + 1) | pending slots << 8
  int32_t* rounds;         // optional: number of acceptance rounds
  // The router's partials (RouterArgs; nblk = router_launch_blocks) and the
  // optional aux outputs: a second block of the launch reduces them.
  const double* part_psum;
  const int32_t* part_top1;
  const double* part_z;
  int nblk;
  int32_t* top1_count;
  float* prob_mean;
  float* aux;
  float* z_loss;
};
hipError_t launch_reroute(const RerouteArgs& a, hipStream_t s);

struct PermuteArgs {
  bool bf16;
  const void* x;
  const int32_t* topk_idx;
  int T, d, E, k, capacity;
  int32_t* counts;
  int32_t* offsets;
  int32_t* dest;
  int32_t* src;
  void* x_perm;
  int32_t* blk_hist;       // [permute_blocks(T*k)][E]
  int32_t* blk_base;       // [permute_blocks(T*k)][E]
};
int permute_blocks(int assignments);
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);

struct FfnArgs {
  bool bf16;
  bool up;                 // true: GELU(A W1^T + b1) -> dtype h; false: A W2^T + b2 -> fp32 o
  const void* a;           // [rows][K] dtype
  const int32_t* offsets;  // [E+1]
  const void* w;           // [E][N][K] dtype
  const void* bias;        // [E][N] dtype or null
  void* out;               // [rows][N] dtype (up) or fp32 (down)
  int E, N, K;
  int max_rows_per_expert; // host bound on any expert's rows (no device sync)
  int max_rows;            // host bound on the total rows R
  int path;                // resolved MOE_FFN_TILED or MOE_FFN_STREAM
  int tile_rows;           // TILED: rows per tile, 256, 192 or 128 (256 and 192 need one h plane)
  bool split;              // bf16 h kept as hi + lo planes (MOE_H_SPLIT)
  size_t plane;            // elements per h plane (T*k*F) when split
  float* partial;          // workspace for split-k partial sums (ffn_partial_bytes bytes)
  const int32_t* gather;   // first product only, or null: A is x [T][K] and dispatched row r
  int gather_k;            // reads token gather[r] / gather_k (gather = src, gather_k = top_k)
  bool defer_reduce;       // second product on the stream path: leave split-k partial sums in
                           // `partial` ([splits][max_rows][N], bias in part 0) for the combine
};
hipError_t launch_ffn(const FfnArgs& a, hipStream_t s);
// k parts the product of `a` is split into: > 1 only on the stream path.
int ffn_k_splits(const FfnArgs& a);
// Writes offsets = {0, rows}: the segment table of a dense product (one
// "expert" owning every row), e.g. the shared expert over all tokens.
hipError_t launch_dense_offsets(int32_t* offsets, int rows, hipStream_t s);
// Workspace bytes the product needs for split-k partial sums on `path`
// (MOE_FFN_TILED or MOE_FFN_STREAM; 0 if it never splits).
size_t ffn_partial_bytes(int path, bool bf16, bool up, bool split, int E, int N, int K,
                         int max_rows_per_expert, int max_rows);

struct CombineArgs {
  const float* o;
  const int32_t* dest;
  const float* topk_w;
  float* y;
  int T, d, k;
  const float* shared;     // [T][d] shared expert output added after the slot sum, or null
  const float* partial;    // or null: o is not stored, row r of o is the sum over p < splits
  int splits, rows_cap;    // of partial[(p * rows_cap + r) * d + c], added in p order
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

// Streaming-read probe (measurement aid): reads `bytes` (a multiple of
// read_probe_granule()) of device memory once.
size_t read_probe_granule();
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);

}  // namespace moe
