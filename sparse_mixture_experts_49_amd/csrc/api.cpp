// C ABI of the MoE layer forward: argument validation, workspace carving and
// the launch sequence.  Kernels live in router.hip, permute.hip, ffn.hip and
// combine.hip.  No call allocates, frees or synchronises.
#include <cmath>
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <limits>
#include <mutex>

#include "../../include/moe_mi355x.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define MOE_REQUIRE_PTR(p, name)                                                       \
  do {                                                                                 \
    if (!(p)) return fail(MOE_ERR_INVALID, "%s must not be NULL", name);               \
    if (!aligned16(p)) return fail(MOE_ERR_INVALID, "%s must be 16-byte aligned", name); \
  } while (0)
#define MOE_OPTIONAL_PTR(p, name)                                                      \
  do {                                                                                 \
    if ((p) && !aligned16(p)) return fail(MOE_ERR_INVALID, "%s must be 16-byte aligned", name); \
  } while (0)

// Whether y averages over several experts or carries weight 1: top-k > 1 or a
// renormalised top-1.  A top-1 layer without renormalisation weights each
// token's one expert output by its raw probability, and capacity drops add
// zero rows, so the largest |y| error sits far above RMS(y); there bf16-rounded
// h alone misses the 2e-2 bar (0.025 and 0.041 of RMS measured on the
// switch-style layers) and h is kept as two bf16 terms.
bool renormalised_or_multi(const moe_desc* d) { return d->top_k > 1 || d->renormalize != 0; }

int validate_desc(const moe_desc* d) {
  if (!d) return fail(MOE_ERR_INVALID, "desc must not be NULL");
  if (d->tokens < 1) return fail(MOE_ERR_INVALID, "tokens must be >= 1 (got %d)", d->tokens);
  if (d->n_experts < 1) return fail(MOE_ERR_INVALID, "n_experts must be >= 1 (got %d)", d->n_experts);
  if (d->n_experts > 64)
    return fail(MOE_ERR_UNSUPPORTED, "n_experts must be <= 64 (got %d)", d->n_experts);
  if (d->top_k < 1 || d->top_k > d->n_experts)
    return fail(MOE_ERR_INVALID, "top_k must be in [1, n_experts] (got %d)", d->top_k);
  if (d->top_k > 8) return fail(MOE_ERR_UNSUPPORTED, "top_k must be <= 8 (got %d)", d->top_k);
  if (d->d_model < 1 || d->d_ff < 1)
    return fail(MOE_ERR_INVALID, "d_model and d_ff must be >= 1");
  if (d->d_model % 128 || d->d_ff % 128)
    return fail(MOE_ERR_UNSUPPORTED, "d_model (%d) and d_ff (%d) must be multiples of 128",
                d->d_model, d->d_ff);
  if (d->renormalize != 0 && d->renormalize != 1)
    return fail(MOE_ERR_INVALID, "renormalize must be 0 or 1");
  if (d->capacity < 0) return fail(MOE_ERR_INVALID, "capacity must be >= 0");
  if (d->capacity_policy != MOE_CAPACITY_DROP && d->capacity_policy != MOE_CAPACITY_REROUTE)
    return fail(MOE_ERR_INVALID, "capacity_policy must be MOE_CAPACITY_DROP or _REROUTE");
  if (d->capacity_policy == MOE_CAPACITY_REROUTE && d->capacity == 0)
    return fail(MOE_ERR_INVALID, "the reroute policy needs a capacity > 0");
  if (d->dtype != MOE_DTYPE_F32 && d->dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_INVALID, "dtype must be MOE_DTYPE_F32 or MOE_DTYPE_BF16");
  if (d->has_expert_bias != 0 && d->has_expert_bias != 1)
    return fail(MOE_ERR_INVALID, "has_expert_bias must be 0 or 1");
  if (d->ffn_path < MOE_FFN_AUTO || d->ffn_path > MOE_FFN_STREAM)
    return fail(MOE_ERR_INVALID, "ffn_path must be MOE_FFN_AUTO, _TILED or _STREAM");
  if (d->ffn_path == MOE_FFN_TILED && d->dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "the LDS-tiled expert kernel is bf16 only");
  if (d->h_mode < MOE_H_AUTO || d->h_mode > MOE_H_SPLIT)
    return fail(MOE_ERR_INVALID, "h_mode must be MOE_H_AUTO, _BF16 or _SPLIT");
  if (d->dtype == MOE_DTYPE_F32 && d->h_mode != MOE_H_AUTO)
    return fail(MOE_ERR_INVALID, "h_mode must be MOE_H_AUTO for an fp32 layer (h is fp32)");
  if (d->h_mode == MOE_H_BF16 && !renormalised_or_multi(d))
    return fail(MOE_ERR_UNSUPPORTED,
                "h_mode MOE_H_BF16 is refused for top-1 layers without renormalisation: "
                "bf16-rounded h puts y past 2e-2 of RMS(y) there (measured 0.025 and 0.041); "
                "use MOE_H_AUTO or MOE_H_SPLIT");
  const long long rows = (long long)d->tokens * d->top_k;
  const long long widest = d->d_model > d->d_ff ? d->d_model : d->d_ff;
  if (rows * widest > std::numeric_limits<int32_t>::max())
    return fail(MOE_ERR_UNSUPPORTED, "tokens * top_k * max(d_model, d_ff) exceeds int32");
  // The tiled kernel addresses one expert's weight matrix with 32-bit byte offsets.
  const long long wbytes = (long long)d->d_model * (d->d_ff > d->d_ff_shared ? d->d_ff : d->d_ff_shared) *
                           (d->dtype == MOE_DTYPE_BF16 ? 2 : 4);
  if (wbytes >= (1LL << 32))
    return fail(MOE_ERR_UNSUPPORTED, "one expert's d_model x d_ff weight matrix must be under 4 GiB");
  if (d->d_ff_shared < 0) return fail(MOE_ERR_INVALID, "d_ff_shared must be >= 0");
  if (d->d_ff_shared % 128)
    return fail(MOE_ERR_UNSUPPORTED, "d_ff_shared (%d) must be a multiple of 128", d->d_ff_shared);
  if ((long long)d->tokens * d->d_ff_shared > std::numeric_limits<int32_t>::max())
    return fail(MOE_ERR_UNSUPPORTED, "tokens * d_ff_shared exceeds int32");
  return MOE_OK;
}

int row_bound(const moe_desc* d) {
  // Any expert holds at most one row per token, and at most `capacity`.
  int b = d->tokens;
  if (d->capacity > 0 && d->capacity < b) b = d->capacity;
  return b;
}

int max_rows(const moe_desc* d) {
  // Total rows R <= T*k, and <= E*capacity under a capacity limit.
  long long r = (long long)d->tokens * d->top_k;
  if (d->capacity > 0) {
    const long long c = (long long)d->capacity * d->n_experts;
    if (c < r) r = c;
  }
  return (int)r;
}

// AUTO choices, resolved from the descriptor alone (never from device data).
struct Plan {
  int path;      // MOE_FFN_TILED or MOE_FFN_STREAM
  int h_mode;    // MOE_H_BF16 / MOE_H_SPLIT, or MOE_H_AUTO for fp32 layers
  size_t h_elem; // bytes per h element
};

// AUTO: bf16 layers averaging >= 64 rows per expert (by the host's bound) run
// the LDS-tiled kernel, the rest stream the weights.  h is one bf16 plane on
// the tiled path at >= 256 rows per expert (MFMA-bound prefill) and on the
// weight-streaming path when no expert can hold more than 32 rows (decode:
// there the second plane's DMA costs ~2% of the second product, measured on
// MI355X), and two planes in between.  Top-1 layers without renormalisation
// always keep two planes (bf16 h alone misses the bar there).
int resolve(const moe_desc* d, Plan& p) {
  const bool bf16 = d->dtype == MOE_DTYPE_BF16;
  const double avg = (double)max_rows(d) / d->n_experts;
  p.path = d->ffn_path;
  if (p.path == MOE_FFN_AUTO) p.path = (bf16 && avg >= 64.0) ? MOE_FFN_TILED : MOE_FFN_STREAM;
  if (!bf16) {
    p.h_mode = MOE_H_AUTO;
    p.h_elem = 4;
    return MOE_OK;
  }
  p.h_mode = d->h_mode;
  if (p.h_mode == MOE_H_AUTO) {
    const bool one_plane = p.path == MOE_FFN_TILED ? avg >= 256.0 : row_bound(d) <= 32;
    p.h_mode = (one_plane && renormalised_or_multi(d)) ? MOE_H_BF16 : MOE_H_SPLIT;
  }
  p.h_elem = p.h_mode == MOE_H_SPLIT ? 4 : 2;
  return MOE_OK;
}

// Rows per tile of the LDS-tiled kernel: 256 when experts average at least
// 256 rows and h is one bf16 plane (prefill, MFMA-bound), else 128.  Measured
// on MI355X for the switch-style layer (64 experts, capacity 160), 128-row
// tiles also beat 192-row ones when rerouting fills every expert to 160 rows.
// With one h plane the choice is between 256- and 192-row tiles, by the
// estimated time of the product: rounds of the 256 CUs times the tile height,
// a 192-row round costing 1.15x a 256-row one per row (measured on MI355X: the
// mid-size layer's products ran 1.11-1.16x slower per row and round).  Tiles
// per expert are estimated from the average rows per expert plus 10% for the
// uneven loads of routed experts (exact for one expert, the shared one).  Where
// the last round is partly idle or each expert's ragged last tile is a large
// share, 192-row tiles win.  Measured for the mid-size layer (16 experts,
// 460-570 rows each): first product 121 -> 105 us (3 rounds of 192 rows instead
// of 3 of 256), second 90 -> 75 us (one round of 192 tiles instead of one of
// 160); the prefill and fine-grained layers keep 256, and 128-row tiles were
// slower on both.
int tile_rows(bool split, int path_rows, int experts, int n) {
  if (split || path_rows < 256L * experts) return 128;
  const double per_expert = (double)path_rows / experts * (experts > 1 ? 1.1 : 1.0);
  const long ntn = (n + 255L) / 256;
  auto est = [&](int bm) {
    const long tiles = (long)experts * (long)std::ceil(per_expert / bm) * ntn;
    return (double)((tiles + 255) / 256) * bm * (bm == 256 ? 1.0 : 1.15);
  };
  return est(192) < est(256) ? 192 : 256;
}

// The shared expert is one dense product over all T tokens: the LDS-tiled
// kernel with bf16 h when T >= 256 rows (bf16), else weight streaming with
// split h (bf16) or fp32 h.
void resolve_shared(const moe_desc* d, Plan& p) {
  const bool bf16 = d->dtype == MOE_DTYPE_BF16;
  p.path = (bf16 && d->tokens >= 256) ? MOE_FFN_TILED : MOE_FFN_STREAM;
  p.h_mode = !bf16 ? MOE_H_AUTO : p.path == MOE_FFN_TILED ? MOE_H_BF16 : MOE_H_SPLIT;
  p.h_elem = (!bf16 || p.h_mode == MOE_H_SPLIT) ? 4 : 2;
}

int validate_weights(const moe_desc* d, const moe_weights* w, bool router, bool experts) {
  if (!w) return fail(MOE_ERR_INVALID, "weights must not be NULL");
  if (router) {
    MOE_REQUIRE_PTR(w->w_router, "w_router");
    MOE_OPTIONAL_PTR(w->b_router, "b_router");
    MOE_OPTIONAL_PTR(w->b_select, "b_select");
  }
  if (experts) {
    MOE_REQUIRE_PTR(w->w1, "w1");
    MOE_REQUIRE_PTR(w->w2, "w2");
    if (d->has_expert_bias) {
      MOE_REQUIRE_PTR(w->b1, "b1");
      MOE_REQUIRE_PTR(w->b2, "b2");
    } else if (w->b1 || w->b2) {
      return fail(MOE_ERR_INVALID, "b1/b2 given but has_expert_bias == 0");
    }
    if (d->d_ff_shared > 0) {
      MOE_REQUIRE_PTR(w->w1_shared, "w1_shared");
      MOE_REQUIRE_PTR(w->w2_shared, "w2_shared");
      if (d->has_expert_bias) {
        MOE_REQUIRE_PTR(w->b1_shared, "b1_shared");
        MOE_REQUIRE_PTR(w->b2_shared, "b2_shared");
      } else if (w->b1_shared || w->b2_shared) {
        return fail(MOE_ERR_INVALID, "b1_shared/b2_shared given but has_expert_bias == 0");
      }
    } else if (w->w1_shared || w->b1_shared || w->w2_shared || w->b2_shared) {
      return fail(MOE_ERR_INVALID, "shared expert weights given but d_ff_shared == 0");
    }
  }
  return MOE_OK;
}

size_t elem_bytes(const moe_desc* d) { return d->dtype == MOE_DTYPE_BF16 ? 2 : 4; }

// Workspace carving: every region starts on a 256-byte boundary.
struct Layout {
  size_t part_psum, part_top1, part_z, part_logit, blk_hist, blk_base;
  size_t topk_idx, topk_w, counts, offsets, dest, src, top1, prob_mean;
  size_t h, o, partial;
  size_t sh_offsets, h_sh, o_sh;   // shared expert (d_ff_shared > 0)
  size_t rr_rank, rr_list;   // reroute policy
  size_t total;
};

size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

Layout layout_of(const moe_desc* d) {
  Layout L{};
  const size_t T = d->tokens, E = d->n_experts, k = d->top_k, A = T * k;
  const size_t rb = moe::router_blocks(d->tokens), pb = moe::permute_blocks((int)A);
  size_t p = 0;
  auto take = [&](size_t bytes) { size_t at = p; p += up256(bytes); return at; };
  L.part_psum = take(rb * E * sizeof(double));
  L.part_top1 = take(rb * E * sizeof(int32_t));
  L.part_z = take(rb * sizeof(double));
  L.part_logit = take(moe::router_small_part_bytes(d->tokens, d->n_experts,
                                                   d->capacity_policy == MOE_CAPACITY_REROUTE));
  L.blk_hist = take(pb * E * sizeof(int32_t));
  L.blk_base = take(pb * E * sizeof(int32_t));
  L.topk_idx = take(A * 4);
  L.topk_w = take(A * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.dest = take(A * 4);
  L.src = take(A * 4);
  L.top1 = take(E * 4);
  L.prob_mean = take(E * 4);
  Plan plan{};
  resolve(d, plan);
  L.h = take(A * d->d_ff * plan.h_elem);
  L.o = take(A * d->d_model * sizeof(float));
  const size_t Fs = d->d_ff_shared;
  Plan sh{};
  resolve_shared(d, sh);
  if (Fs) {
    L.sh_offsets = take(2 * sizeof(int32_t));
    L.h_sh = take(T * Fs * sh.h_elem);
    L.o_sh = take(T * d->d_model * sizeof(float));
  }
  // Split-k partial sums of the expert products (one product at a time).
  size_t part = 0;
  const bool bf16 = d->dtype == MOE_DTYPE_BF16;
  for (int up = 0; up < 2; ++up) {
    size_t b = moe::ffn_partial_bytes(plan.path, bf16, up, plan.h_mode == MOE_H_SPLIT, d->n_experts,
                                      up ? d->d_ff : d->d_model, up ? d->d_model : d->d_ff,
                                      row_bound(d), max_rows(d));
    if (b > part) part = b;
    if (Fs) {
      b = moe::ffn_partial_bytes(sh.path, bf16, up, sh.h_mode == MOE_H_SPLIT, 1,
                                 up ? (int)Fs : d->d_model, up ? d->d_model : (int)Fs, d->tokens,
                                 d->tokens);
      if (b > part) part = b;
    }
  }
  L.partial = take(part);
  if (d->capacity_policy == MOE_CAPACITY_REROUTE) {
    L.rr_rank = take(T * 64 * 2 * sizeof(int32_t));
    L.rr_list = take(4 * T * sizeof(int32_t));
  }
  L.total = p;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

int check_ws(const moe_desc* d, void* ws, size_t bytes, Layout& L) {
  L = layout_of(d);
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace must not be NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", bytes, L.total);
  return MOE_OK;
}

// ---- aliasing -------------------------------------------------------------
// Outputs (the workspace included) must be disjoint from each other and from
// every input; a call that would write over its own operands is refused.

struct Span {
  const void* p;
  size_t n;
  const char* name;
};

struct Spans {
  Span s[24];
  int n = 0;
  void add(const void* p, size_t bytes, const char* name) {
    if (p && bytes && n < 24) s[n++] = Span{p, bytes, name};
  }
};

bool overlaps(const Span& a, const Span& b) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

int check_alias(const Spans& outs, const Spans& ins) {
  for (int i = 0; i < outs.n; ++i) {
    for (int j = i + 1; j < outs.n; ++j)
      if (overlaps(outs.s[i], outs.s[j]))
        return fail(MOE_ERR_INVALID, "%s overlaps %s", outs.s[i].name, outs.s[j].name);
    for (int j = 0; j < ins.n; ++j)
      if (overlaps(outs.s[i], ins.s[j]))
        return fail(MOE_ERR_INVALID, "%s overlaps %s", outs.s[i].name, ins.s[j].name);
  }
  return MOE_OK;
}

// Byte sizes of the arrays a descriptor implies.
struct Bytes {
  size_t x, w_router, b_router, w1, b1, w2, b2, w1s, b1s, w2s, b2s;
  size_t tk, e, e1, x_perm, h, o, y;
};

Bytes bytes_of(const moe_desc* d) {
  const size_t T = d->tokens, D = d->d_model, F = d->d_ff, E = d->n_experts, k = d->top_k;
  const size_t s = elem_bytes(d), Fs = d->d_ff_shared;
  Plan p{};
  resolve(d, p);
  Bytes b{};
  b.x = T * D * s;
  b.w_router = E * D * s;
  b.b_router = E * 4;
  b.w1 = E * F * D * s;
  b.b1 = E * F * s;
  b.w2 = E * D * F * s;
  b.b2 = E * D * s;
  b.w1s = Fs * D * s;
  b.b1s = Fs * s;
  b.w2s = D * Fs * s;
  b.b2s = D * s;
  b.tk = T * k * 4;
  b.e = E * 4;
  b.e1 = (E + 1) * 4;
  b.x_perm = T * k * D * s;
  b.h = T * k * F * p.h_elem;
  b.o = T * k * D * 4;
  b.y = T * D * 4;
  return b;
}

void add_weights(Spans& in, const moe_desc* d, const moe_weights* w, bool router, bool experts) {
  const Bytes b = bytes_of(d);
  if (router) {
    in.add(w->w_router, b.w_router, "w_router");
    in.add(w->b_router, b.b_router, "b_router");
    in.add(w->b_select, b.b_router, "b_select");
  }
  if (experts) {
    in.add(w->w1, b.w1, "w1");
    in.add(w->b1, b.b1, "b1");
    in.add(w->w2, b.w2, "w2");
    in.add(w->b2, b.b2, "b2");
    in.add(w->w1_shared, b.w1s, "w1_shared");
    in.add(w->b1_shared, b.b1s, "b1_shared");
    in.add(w->w2_shared, b.w2s, "w2_shared");
    in.add(w->b2_shared, b.b2s, "b2_shared");
  }
}

void add_routing_outputs(Spans& out, const moe_desc* d, const moe_routing& r) {
  const Bytes b = bytes_of(d);
  out.add(r.topk_idx, b.tk, "topk_idx");
  out.add(r.topk_w, b.tk, "topk_w");
  out.add(r.counts, b.e, "counts");
  out.add(r.offsets, b.e1, "offsets");
  out.add(r.dest, b.tk, "dest");
  out.add(r.src, b.tk, "src");
  out.add(r.top1_count, b.e, "top1_count");
  out.add(r.prob_mean, b.e, "prob_mean");
  out.add(r.z_loss, 4, "z_loss");
  out.add(r.reroute_rounds, 4, "reroute_rounds");
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Dispatch layout outputs that the router's aux reduction fills for small
// layers under the drop policy (see small_dispatch).
struct LayoutOut {
  int32_t *counts, *offsets, *dest, *src;
};

// Whether moe_forward takes the dispatch layout from the router's aux
// reduction block instead of the three permute launches: drop policy and at
// most 8192 assignments (measured: the mid-size and Switch-style layers' three
// permute kernels took ~13 us with their launch gaps).
bool small_dispatch(const moe_desc* d) {
  return d->capacity_policy == MOE_CAPACITY_DROP && moe::router_can_permute(d->tokens * d->top_k);
}

// The router, then (MOE_CAPACITY_REROUTE) the rerouting of the overflow.
// layout (small_dispatch layers only, or null): also the dispatch layout.
int launch_route(const moe_desc* d, const void* x, const moe_weights* w, int32_t* idx, float* wt,
                 int32_t* top1, float* pmean, float* aux, float* zl, int32_t* rounds,
                 const Layout& L, void* ws, hipStream_t s, const LayoutOut* layout = nullptr) {
  const bool rr = d->capacity_policy == MOE_CAPACITY_REROUTE;
  moe::RouterArgs a{};
  a.bf16 = d->dtype == MOE_DTYPE_BF16;
  a.x = x;
  a.w_router = w->w_router;
  a.b_router = w->b_router;
  a.b_select = w->b_select;
  a.T = d->tokens;
  a.d = d->d_model;
  a.E = d->n_experts;
  a.k = d->top_k;
  a.renorm = d->renormalize;
  a.topk_idx = idx;
  a.topk_w = wt;
  a.part_psum = at<double>(ws, L.part_psum);
  a.part_top1 = at<int32_t>(ws, L.part_top1);
  a.part_z = at<double>(ws, L.part_z);
  a.part_logit = at<float>(ws, L.part_logit);
  a.top1_count = top1;
  a.prob_mean = pmean;
  a.aux = aux;
  a.z_loss = zl;
  a.rr_rank = rr ? at<int32_t>(ws, L.rr_rank) : nullptr;
  a.rounds_zero = rr ? nullptr : rounds;
  if (layout) {
    a.perm = true;
    a.capacity = d->capacity;
    a.counts = layout->counts;
    a.offsets = layout->offsets;
    a.dest = layout->dest;
    a.src = layout->src;
  }
  if (int st = hip_status(moe::launch_router(a, s), "router launch")) return st;
  if (!rr) return MOE_OK;
  moe::RerouteArgs b{};
  b.rank = a.rr_rank;
  b.T = d->tokens;
  b.k = d->top_k;
  b.E = d->n_experts;
  b.capacity = d->capacity;
  b.topk_idx = idx;
  b.topk_w = wt;
  b.lists = at<int32_t>(ws, L.rr_list);
  b.rounds = rounds;
  b.part_psum = a.part_psum;
  b.part_top1 = a.part_top1;
  b.part_z = a.part_z;
  b.nblk = moe::router_launch_blocks(d->tokens, d->n_experts);
  b.top1_count = top1;
  b.prob_mean = pmean;
  b.aux = aux;
  b.z_loss = zl;
  return hip_status(moe::launch_reroute(b, s), "reroute launch");
}

int launch_perm(const moe_desc* d, const void* x, const int32_t* idx, int32_t* counts,
                int32_t* offsets, int32_t* dest, int32_t* src, void* x_perm, const Layout& L,
                void* ws, hipStream_t s) {
  moe::PermuteArgs a{};
  a.bf16 = d->dtype == MOE_DTYPE_BF16;
  a.x = x;
  a.topk_idx = idx;
  a.T = d->tokens;
  a.d = d->d_model;
  a.E = d->n_experts;
  a.k = d->top_k;
  // Under the reroute policy the router already kept every expert within capacity.
  a.capacity = d->capacity_policy == MOE_CAPACITY_DROP ? d->capacity : 0;
  a.counts = counts;
  a.offsets = offsets;
  a.dest = dest;
  a.src = src;
  a.x_perm = x_perm;
  a.blk_hist = at<int32_t>(ws, L.blk_hist);
  a.blk_base = at<int32_t>(ws, L.blk_base);
  return hip_status(moe::launch_permute(a, s), "permute launch");
}

// Split-k partial sums of the second product that the combine finishes.
struct Deferred {
  const float* partial = nullptr;
  int splits = 1, rows_cap = 0;
};

// One expert product.  gather (first product only, or null): `in` is x and
// dispatched row r reads token gather[r] / top_k (gather = the dispatch's src).
// defer (second product only, or null): if the product splits k, its partial
// sums are left for the combine and described in *defer.
int launch_one_ffn(const moe_desc* d, bool up, const void* in, const int32_t* offsets,
                   const moe_weights* w, void* out, void* ws, const Layout& L, hipStream_t s,
                   const int32_t* gather = nullptr, Deferred* defer = nullptr) {
  Plan plan{};
  if (int st = resolve(d, plan)) return st;
  moe::FfnArgs a{};
  a.split = plan.h_mode == MOE_H_SPLIT;
  a.plane = (size_t)d->tokens * d->top_k * d->d_ff;   // elements per h plane
  a.bf16 = d->dtype == MOE_DTYPE_BF16;
  a.up = up;
  a.a = in;
  a.offsets = offsets;
  a.w = up ? w->w1 : w->w2;
  a.bias = d->has_expert_bias ? (up ? w->b1 : w->b2) : nullptr;
  a.out = out;
  a.E = d->n_experts;
  a.N = up ? d->d_ff : d->d_model;
  a.K = up ? d->d_model : d->d_ff;
  a.max_rows_per_expert = row_bound(d);
  a.max_rows = max_rows(d);
  a.path = plan.path;
  a.tile_rows = tile_rows(a.split, a.max_rows, a.E, a.N);
  a.partial = at<float>(ws, L.partial);
  a.gather = gather;
  a.gather_k = d->top_k;
  if (defer && !up) {
    const int splits = moe::ffn_k_splits(a);
    a.defer_reduce = splits > 1;
    if (a.defer_reduce) {
      defer->partial = a.partial;
      defer->splits = splits;
      defer->rows_cap = a.max_rows;
    }
  }
  return hip_status(moe::launch_ffn(a, s), up ? "ffn up launch" : "ffn down launch");
}

// The shared expert: one dense product pair over all T tokens of x.
int launch_shared(const moe_desc* d, const void* x, const moe_weights* w, float* o_sh, void* ws,
                  const Layout& L, hipStream_t s) {
  Plan sh{};
  resolve_shared(d, sh);
  int32_t* offs = at<int32_t>(ws, L.sh_offsets);
  if (int st = hip_status(moe::launch_dense_offsets(offs, d->tokens, s), "shared offsets launch"))
    return st;
  moe::FfnArgs a{};
  a.split = sh.h_mode == MOE_H_SPLIT;
  a.plane = (size_t)d->tokens * d->d_ff_shared;
  a.bf16 = d->dtype == MOE_DTYPE_BF16;
  a.offsets = offs;
  a.E = 1;
  a.max_rows_per_expert = d->tokens;
  a.max_rows = d->tokens;
  a.path = sh.path;
  a.partial = at<float>(ws, L.partial);
  void* h = at<void>(ws, L.h_sh);
  a.up = true;
  a.a = x;
  a.w = w->w1_shared;
  a.bias = d->has_expert_bias ? w->b1_shared : nullptr;
  a.out = h;
  a.N = d->d_ff_shared;
  a.K = d->d_model;
  a.tile_rows = tile_rows(a.split, d->tokens, 1, a.N);
  if (int st = hip_status(moe::launch_ffn(a, s), "shared ffn up launch")) return st;
  a.up = false;
  a.a = h;
  a.w = w->w2_shared;
  a.bias = d->has_expert_bias ? w->b2_shared : nullptr;
  a.out = o_sh;
  a.N = d->d_model;
  a.K = d->d_ff_shared;
  a.tile_rows = tile_rows(a.split, d->tokens, 1, a.N);
  return hip_status(moe::launch_ffn(a, s), "shared ffn down launch");
}

int launch_comb(const moe_desc* d, const float* o, const int32_t* dest, const float* wt,
                const float* o_sh, float* y, hipStream_t s, const Deferred& part = Deferred{}) {
  moe::CombineArgs a{o,  dest, wt, y, d->tokens, d->d_model, d->top_k, o_sh, part.partial,
                     part.splits, part.rows_cap};
  return hip_status(moe::launch_combine(a, s), "combine launch");
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: outside the implemented limits";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_err; }

int moe_workspace_size(const moe_desc* desc, size_t* bytes) {
  if (int st = validate_desc(desc)) return st;
  Plan p{};
  if (int st = resolve(desc, p)) return st;
  if (!bytes) return fail(MOE_ERR_INVALID, "bytes must not be NULL");
  *bytes = layout_of(desc).total;
  return ok();
}

int moe_query_plan(const moe_desc* desc, moe_plan* plan) {
  if (int st = validate_desc(desc)) return st;
  if (!plan) return fail(MOE_ERR_INVALID, "plan must not be NULL");
  Plan p{};
  if (int st = resolve(desc, p)) return st;
  plan->ffn_path = p.path;
  plan->h_mode = p.h_mode;
  plan->h_bytes = (size_t)desc->tokens * desc->top_k * desc->d_ff * p.h_elem;
  plan->workspace_bytes = layout_of(desc).total;
  return ok();
}

int moe_route(const moe_desc* desc, const void* x, const moe_weights* w, moe_routing* out,
              float* aux, void* ws, size_t ws_bytes, void* stream) {
  if (int st = validate_desc(desc)) return st;
  MOE_REQUIRE_PTR(x, "x");
  if (int st = validate_weights(desc, w, true, false)) return st;
  if (!out) return fail(MOE_ERR_INVALID, "out must not be NULL");
  MOE_REQUIRE_PTR(out->topk_idx, "out->topk_idx");
  MOE_REQUIRE_PTR(out->topk_w, "out->topk_w");
  MOE_OPTIONAL_PTR(out->top1_count, "out->top1_count");
  MOE_OPTIONAL_PTR(out->prob_mean, "out->prob_mean");
  MOE_OPTIONAL_PTR(out->z_loss, "out->z_loss");
  MOE_OPTIONAL_PTR(out->reroute_rounds, "out->reroute_rounds");
  Layout L;
  if (int st = check_ws(desc, ws, ws_bytes, L)) return st;
  {
    const Bytes b = bytes_of(desc);
    Spans o, in;
    moe_routing r{};
    r.topk_idx = out->topk_idx;
    r.topk_w = out->topk_w;
    r.top1_count = out->top1_count;
    r.prob_mean = out->prob_mean;
    r.z_loss = out->z_loss;
    r.reroute_rounds = out->reroute_rounds;
    add_routing_outputs(o, desc, r);
    o.add(aux, 4, "aux");
    o.add(ws, ws_bytes, "workspace");
    in.add(x, b.x, "x");
    add_weights(in, desc, w, true, false);
    if (int st = check_alias(o, in)) return st;
  }
  return launch_route(desc, x, w, out->topk_idx, out->topk_w, out->top1_count, out->prob_mean,
                      aux, out->z_loss, out->reroute_rounds, L, ws,
                      static_cast<hipStream_t>(stream));
}

int moe_permute(const moe_desc* desc, const void* x, moe_routing* r, void* x_perm, void* ws,
                size_t ws_bytes, void* stream) {
  if (int st = validate_desc(desc)) return st;
  MOE_REQUIRE_PTR(x, "x");
  if (!r) return fail(MOE_ERR_INVALID, "r must not be NULL");
  MOE_REQUIRE_PTR(r->topk_idx, "r->topk_idx");
  MOE_REQUIRE_PTR(r->counts, "r->counts");
  MOE_REQUIRE_PTR(r->offsets, "r->offsets");
  MOE_REQUIRE_PTR(r->dest, "r->dest");
  MOE_REQUIRE_PTR(r->src, "r->src");
  MOE_REQUIRE_PTR(x_perm, "x_perm");
  Layout L;
  if (int st = check_ws(desc, ws, ws_bytes, L)) return st;
  {
    const Bytes b = bytes_of(desc);
    Spans o, in;
    o.add(r->counts, b.e, "counts");
    o.add(r->offsets, b.e1, "offsets");
    o.add(r->dest, b.tk, "dest");
    o.add(r->src, b.tk, "src");
    o.add(x_perm, b.x_perm, "x_perm");
    o.add(ws, ws_bytes, "workspace");
    in.add(x, b.x, "x");
    in.add(r->topk_idx, b.tk, "topk_idx");
    if (int st = check_alias(o, in)) return st;
  }
  return launch_perm(desc, x, r->topk_idx, r->counts, r->offsets, r->dest, r->src, x_perm, L, ws,
                     static_cast<hipStream_t>(stream));
}

int moe_ffn_up(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
               const moe_weights* w, void* h, void* ws, size_t ws_bytes, void* stream) {
  if (int st = validate_desc(desc)) return st;
  MOE_REQUIRE_PTR(x_perm, "x_perm");
  MOE_REQUIRE_PTR(offsets, "offsets");
  MOE_REQUIRE_PTR(h, "h");
  if (int st = validate_weights(desc, w, false, true)) return st;
  Layout L;
  if (int st = check_ws(desc, ws, ws_bytes, L)) return st;
  {
    const Bytes b = bytes_of(desc);
    Spans o, in;
    o.add(h, b.h, "h");
    o.add(ws, ws_bytes, "workspace");
    in.add(x_perm, b.x_perm, "x_perm");
    in.add(offsets, b.e1, "offsets");
    add_weights(in, desc, w, false, true);
    if (int st = check_alias(o, in)) return st;
  }
  return launch_one_ffn(desc, true, x_perm, offsets, w, h, ws, L, static_cast<hipStream_t>(stream));
}

int moe_ffn_up_gather(const moe_desc* desc, const void* x, const int32_t* src,
                      const int32_t* offsets, const moe_weights* w, void* h, void* ws,
                      size_t ws_bytes, void* stream) {
  if (int st = validate_desc(desc)) return st;
  MOE_REQUIRE_PTR(x, "x");
  MOE_REQUIRE_PTR(src, "src");
  MOE_REQUIRE_PTR(offsets, "offsets");
  MOE_REQUIRE_PTR(h, "h");
  if (int st = validate_weights(desc, w, false, true)) return st;
  Layout L;
  if (int st = check_ws(desc, ws, ws_bytes, L)) return st;
  {
    const Bytes b = bytes_of(desc);
    Spans o, in;
    o.add(h, b.h, "h");
    o.add(ws, ws_bytes, "workspace");
    in.add(x, b.x, "x");
    in.add(src, b.tk, "src");
    in.add(offsets, b.e1, "offsets");
    add_weights(in, desc, w, false, true);
    if (int st = check_alias(o, in)) return st;
  }
  return launch_one_ffn(desc, true, x, offsets, w, h, ws, L, static_cast<hipStream_t>(stream),
                        src);
}

int moe_ffn_down(const moe_desc* desc, const void* h, const int32_t* offsets,
                 const moe_weights* w, float* o, void* ws, size_t ws_bytes, void* stream) {
  if (int st = validate_desc(desc)) return st;
  MOE_REQUIRE_PTR(h, "h");
  MOE_REQUIRE_PTR(offsets, "offsets");
  MOE_REQUIRE_PTR(o, "o");
  if (int st = validate_weights(desc, w, false, true)) return st;
  Layout L;
  if (int st = check_ws(desc, ws, ws_bytes, L)) return st;
  {
    const Bytes b = bytes_of(desc);
    Spans out, in;
    out.add(o, b.o, "o");
    out.add(ws, ws_bytes, "workspace");
    in.add(h, b.h, "h");
    in.add(offsets, b.e1, "offsets");
    add_weights(in, desc, w, false, true);
    if (int st = check_alias(out, in)) return st;
  }
  return launch_one_ffn(desc, false, h, offsets, w, o, ws, L, static_cast<hipStream_t>(stream));
}

int moe_grouped_ffn(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                    const moe_weights* w, void* h, float* o, void* ws, size_t ws_bytes,
                    void* stream) {
  if (int st = validate_desc(desc)) return st;
  MOE_REQUIRE_PTR(x_perm, "x_perm");
  MOE_REQUIRE_PTR(offsets, "offsets");
  MOE_REQUIRE_PTR(h, "h");
  MOE_REQUIRE_PTR(o, "o");
  if (int st = validate_weights(desc, w, false, true)) return st;
  Layout L;
  if (int st = check_ws(desc, ws, ws_bytes, L)) return st;
  {
    const Bytes b = bytes_of(desc);
    Spans out, in;
    out.add(h, b.h, "h");
    out.add(o, b.o, "o");
    out.add(ws, ws_bytes, "workspace");
    in.add(x_perm, b.x_perm, "x_perm");
    in.add(offsets, b.e1, "offsets");
    add_weights(in, desc, w, false, true);
    if (int st = check_alias(out, in)) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (int st = launch_one_ffn(desc, true, x_perm, offsets, w, h, ws, L, s)) return st;
  return launch_one_ffn(desc, false, h, offsets, w, o, ws, L, s);
}

int moe_combine(const moe_desc* desc, const float* o, const int32_t* dest, const float* topk_w,
                const float* o_shared, float* y, void* stream) {
  if (int st = validate_desc(desc)) return st;
  MOE_REQUIRE_PTR(o, "o");
  MOE_REQUIRE_PTR(dest, "dest");
  MOE_REQUIRE_PTR(topk_w, "topk_w");
  MOE_OPTIONAL_PTR(o_shared, "o_shared");
  MOE_REQUIRE_PTR(y, "y");
  {
    const Bytes b = bytes_of(desc);
    Spans out, in;
    out.add(y, b.y, "y");
    in.add(o, b.o, "o");
    in.add(dest, b.tk, "dest");
    in.add(topk_w, b.tk, "topk_w");
    in.add(o_shared, b.y, "o_shared");
    if (int st = check_alias(out, in)) return st;
  }
  return launch_comb(desc, o, dest, topk_w, o_shared, y, static_cast<hipStream_t>(stream));
}

int moe_shared_ffn(const moe_desc* desc, const void* x, const moe_weights* w, float* o_shared,
                   void* ws, size_t ws_bytes, void* stream) {
  if (int st = validate_desc(desc)) return st;
  if (desc->d_ff_shared == 0) return fail(MOE_ERR_INVALID, "the layer has no shared expert");
  MOE_REQUIRE_PTR(x, "x");
  MOE_REQUIRE_PTR(o_shared, "o_shared");
  if (int st = validate_weights(desc, w, false, true)) return st;
  Layout L;
  if (int st = check_ws(desc, ws, ws_bytes, L)) return st;
  {
    const Bytes b = bytes_of(desc);
    Spans out, in;
    out.add(o_shared, b.y, "o_shared");
    out.add(ws, ws_bytes, "workspace");
    in.add(x, b.x, "x");
    add_weights(in, desc, w, false, true);
    if (int st = check_alias(out, in)) return st;
  }
  return launch_shared(desc, x, w, o_shared, ws, L, static_cast<hipStream_t>(stream));
}

int moe_forward(const moe_desc* desc, const void* x, const moe_weights* w, float* y, float* aux,
                moe_routing* routing, void* ws, size_t ws_bytes, void* stream) {
  if (int st = validate_desc(desc)) return st;
  MOE_REQUIRE_PTR(x, "x");
  MOE_REQUIRE_PTR(y, "y");
  if (int st = validate_weights(desc, w, true, true)) return st;
  moe_routing r{};
  if (routing) {
    r = *routing;
    MOE_OPTIONAL_PTR(r.topk_idx, "routing->topk_idx");
    MOE_OPTIONAL_PTR(r.topk_w, "routing->topk_w");
    MOE_OPTIONAL_PTR(r.counts, "routing->counts");
    MOE_OPTIONAL_PTR(r.offsets, "routing->offsets");
    MOE_OPTIONAL_PTR(r.dest, "routing->dest");
    MOE_OPTIONAL_PTR(r.src, "routing->src");
    MOE_OPTIONAL_PTR(r.top1_count, "routing->top1_count");
    MOE_OPTIONAL_PTR(r.prob_mean, "routing->prob_mean");
    MOE_OPTIONAL_PTR(r.z_loss, "routing->z_loss");
    MOE_OPTIONAL_PTR(r.reroute_rounds, "routing->reroute_rounds");
  }
  Layout L;
  if (int st = check_ws(desc, ws, ws_bytes, L)) return st;
  {
    const Bytes b = bytes_of(desc);
    Spans out, in;
    out.add(y, b.y, "y");
    out.add(aux, 4, "aux");
    add_routing_outputs(out, desc, r);
    out.add(ws, ws_bytes, "workspace");
    in.add(x, b.x, "x");
    add_weights(in, desc, w, true, true);
    if (int st = check_alias(out, in)) return st;
  }
  if (!r.topk_idx) r.topk_idx = at<int32_t>(ws, L.topk_idx);
  if (!r.topk_w) r.topk_w = at<float>(ws, L.topk_w);
  if (!r.counts) r.counts = at<int32_t>(ws, L.counts);
  if (!r.offsets) r.offsets = at<int32_t>(ws, L.offsets);
  if (!r.dest) r.dest = at<int32_t>(ws, L.dest);
  if (!r.src) r.src = at<int32_t>(ws, L.src);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* h = at<void>(ws, L.h);
  float* o = at<float>(ws, L.o);
  // The dispatch layout only: the first product reads each row's token straight
  // from x through src, so x_perm is never materialised.  Small layers get it
  // from the router's aux reduction.
  const LayoutOut layout{r.counts, r.offsets, r.dest, r.src};
  const bool small = small_dispatch(desc);
  if (int st = launch_route(desc, x, w, r.topk_idx, r.topk_w, r.top1_count, r.prob_mean, aux,
                            r.z_loss, r.reroute_rounds, L, ws, s, small ? &layout : nullptr))
    return st;
  if (!small) {
    if (int st = launch_perm(desc, x, r.topk_idx, r.counts, r.offsets, r.dest, r.src, nullptr, L,
                             ws, s))
      return st;
  }
  if (int st = launch_one_ffn(desc, true, x, r.offsets, w, h, ws, L, s, r.src)) return st;
  // The shared expert before the second routed product: both use the split-k
  // partial region, and the second product may leave its partial sums there
  // for the combine to finish (no separate reduction pass over o).
  float* o_sh = nullptr;
  if (desc->d_ff_shared > 0) {
    o_sh = at<float>(ws, L.o_sh);
    if (int st = launch_shared(desc, x, w, o_sh, ws, L, s)) return st;
  }
  Deferred part;
  if (int st = launch_one_ffn(desc, false, h, r.offsets, w, o, ws, L, s, nullptr, &part))
    return st;
  return launch_comb(desc, o, r.dest, r.topk_w, o_sh, y, s, part);
}

}  // extern "C"

extern "C" int moe_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  MOE_REQUIRE_PTR(buf, "buf");
  MOE_REQUIRE_PTR(sink, "sink");
  const size_t g = moe::read_probe_granule();
  if (bytes == 0 || bytes % g)
    return fail(MOE_ERR_INVALID, "bytes must be a positive multiple of %zu", g);
  if (bytes / g > 0x7fffffffu) return fail(MOE_ERR_UNSUPPORTED, "bytes too large");
  return hip_status(moe::launch_read_probe(buf, bytes, sink, static_cast<hipStream_t>(stream)),
                    "read probe launch");
}

// ---- the allocation-free layer call ------------------------------------------
// moe_forward_noalloc runs moe_forward on a workspace the library owns: a
// file-scope device array of kScratchBytes.  Each device holds its own copy;
// its address is looked up once per device (with that device current) and the
// kernels get that address, never the array's host-side name.  Every kernel of
// the layer writes each workspace region before reading it, so nothing needs
// clearing between calls.
namespace {
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device index %d is past the %d devices the scratch table holds",
                dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

extern "C" int moe_forward_noalloc(const moe_desc* desc, const void* x, const moe_weights* w,
                                   float* y, float* aux, moe_routing* routing, void* stream) {
  if (int st = validate_desc(desc)) return st;
  const size_t need = layout_of(desc).total;
  if (need > kScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_forward_noalloc: the layer needs %zu bytes of workspace, the library's scratch "
                "holds %zu; use moe_forward with a caller workspace",
                need, kScratchBytes);
  void* ws = nullptr;
  if (int st = scratch_of_current_device(&ws)) return st;
  return moe_forward(desc, x, w, y, aux, routing, ws, kScratchBytes, stream);
}
