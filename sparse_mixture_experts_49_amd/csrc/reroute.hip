// The reroute policy for expert overflow on gfx950.
//
// Web page "Mixture of Experts: Scaling Parameters Without Scaling Compute",
// section "The central problem: load balancing" (expert capacity: tokens past
// an expert's capacity are dropped or rerouted), and the llmdaily day-59 page,
// "Experts also have capacity limits" (overflow may be sent to other experts).
// The pages leave the rerouting rule open; the one implemented here:
//   * rounds; round 0 requests every slot's router choice;
//   * in a round, an expert accepts its requests in token order while it has
//     capacity left (a token never asks one expert twice, so token order is
//     assignment order t*k+s);
//   * a rejected slot asks, next round, for its token's best-ranked expert not
//     yet asked (ranking by the selection scores: descending, ties to the lower
//     index); a token's rejected slots take these in slot order; with none
//     left the slot is dropped;
//   * a served slot's weight is the router probability of the expert serving
//     it over the original denominator (the chosen probabilities' sum when
//     renormalising, else 1) -- the router writes that value for every expert.
//
// One block of 1024 threads runs every round, so no host synchronisation is
// needed and the number of rounds stays on the device.  Round 0 walks all
// T*k assignments; each later round walks only the ordered list of slots
// rejected in the round before (two lists, used in turn; the first 2048
// entries of a list live in LDS, the rest in the workspace).
// An entry is the token id and, packed in one word, the expert it asks, its
// token's cursor (the lowest-ranked expert the token has asked) and the slot.
//
// Acceptance walks a list in chunks of 1024 entries, in order: inside a wave,
// requests to one expert are matched with one ballot per bit of the expert
// id and the first lane of each group publishes the group's size; wave 0 then
// turns the per-wave counts into the room each expert has for each wave (its
// lane x keeps expert x's capacity left in a register across chunks).
// Rejected entries are appended to the other list in the same order, so a
// token's entries stay adjacent and in slot order.  An accepted entry needs
// no write: topk_idx already holds the expert it asked (the router's choice
// in round 0; later the next-candidate step writes it when it hands the
// expert out).  Next candidates: four lanes serve the first entry of each
// token's run; each loads 16 of the token's 64 scores and the quad hands out
// the best-ranked experts below the cursor, one per entry in slot order.  A last pass writes the
// weight of every served slot (bit-identical to the router's where its
// choice serves) and dropped slots read expert -1, weight 0.
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kRerouteThreads = 1024;
constexpr int kRerouteWaves = kRerouteThreads / 64;
constexpr int kNoExpert = 0xff;   // request or cursor field: none
constexpr int kLdsList = 2048;    // list entries kept in LDS; the rest go to the workspace

__device__ __forceinline__ int pack_req(int e, int c, int s) {
  return (e & 0xff) | ((c & 0xff) << 8) | ((s & 0xff) << 16);
}
__device__ __forceinline__ int req_expert(int r) { return r & 0xff; }
__device__ __forceinline__ int req_cursor(int r) { return (r >> 8) & 0xff; }
__device__ __forceinline__ int req_slot(int r) { return (r >> 16) & 0xff; }

// Quad-wide search: the best-ranked expert strictly below expert c (score
// cv) in the ranking of the token's scores (higher score first, equal scores
// by lower index), -1 if there is none.  Lane ql of the quad holds scores
// 16*ql .. 16*ql+15; past E they are -inf, which never beats the start of
// -inf.  The value of the winner is returned in `bv`.
__device__ __forceinline__ int quad_next_below(const float (&sc)[16], int ql, int E, int c,
                                               float cv, float& bv) {
  int best = -1;
  bv = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = 16 * ql + i;
    const float v = sc[i];
    const bool below = (v < cv) || (v == cv && e > c);
    const bool take = below && v > bv;
    best = take ? e : best;
    bv = take ? v : bv;
  }
#pragma unroll
  for (int off = 1; off <= 2; off <<= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oe = __shfl_xor(best, off);
    const bool take = oe >= 0 && (best < 0 || ov > bv || (ov == bv && oe < best));
    best = take ? oe : best;
    bv = take ? ov : bv;
  }
  return best < E ? best : -1;
}

__global__ __launch_bounds__(kRerouteThreads) void reroute_kernel(
    const float* __restrict__ score, const float* __restrict__ wt, int T, int k, int E,
    int capacity, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ lists, int32_t* __restrict__ rounds_out) {
  __shared__ int wcnt[kRerouteWaves][64];   // requests per (wave, expert) in the chunk
  __shared__ int room[kRerouteWaves][64];   // room expert x has for wave w's requests
  __shared__ int wrej[kRerouteWaves];       // rejected entries per wave in the chunk
  __shared__ int lst_a[2][kLdsList];        // list heads: token ids
  __shared__ int lst_r[2][kLdsList];        // list heads: packed requests
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int A = T * k;
  int left = capacity;                      // wave 0, lane x: capacity expert x has left
  int n = A;                                // entries of the list walked this round
  int cur = 1, nxt = 0;                     // lists read and written this round
  int rounds = 0;
  // Entry i of list l: LDS below kLdsList, workspace above (lists holds the
  // token ids of list 0, requests of list 0, token ids of list 1, requests
  // of list 1).
  auto gidx = [&](int l, int field, int i) -> size_t { return (size_t)(2 * l + field) * A + i; };
  auto get_a = [&](int l, int i) -> int { return i < kLdsList ? lst_a[l][i] : lists[gidx(l, 0, i)]; };
  auto get_r = [&](int l, int i) -> int { return i < kLdsList ? lst_r[l][i] : lists[gidx(l, 1, i)]; };
  auto put_r = [&](int l, int i, int v) {
    if (i < kLdsList) lst_r[l][i] = v;
    else lists[gidx(l, 1, i)] = v;
  };
  // Entry i of the list walked this round.  Round 0 reads the router's
  // choices (and the token's lowest-ranked one as its cursor); an id outside
  // [0, E) is dropped there.
  auto load_entry = [&](bool first, int i, int& t, int& req) {
    t = -1;
    req = pack_req(kNoExpert, kNoExpert, 0);
    if (i >= n) return;
    if (first) {
      t = i / k;
      const int e = topk_idx[i];
      const int c = topk_idx[(size_t)t * k + k - 1];
      if (e < 0 || e >= E) {
        topk_idx[i] = -1;
        topk_w[i] = 0.f;
        return;
      }
      req = pack_req(e, (c >= 0 && c < E) ? c : kNoExpert, i - t * k);
    } else {
      t = get_a(cur, i);
      req = get_r(cur, i);
    }
  };
  for (;;) {
    ++rounds;
    const bool first = rounds == 1;
    int nrej = 0;                     // rejected so far this round (same in every wave)
    int pa, pr;                       // the next chunk's entry, loaded one chunk ahead
    load_entry(first, tid, pa, pr);
    // Acceptance: requests to an expert in assignment order while capacity lasts.
    for (int base = 0; base < n; base += kRerouteThreads) {
      const int tok = pa, req = pr;
      load_entry(first, base + kRerouteThreads + tid, pa, pr);
      const int e = req_expert(req) == kNoExpert ? -1 : req_expert(req);
      int cnt;
      const int rk = wave_rank(e, lt_mask, cnt);
      wcnt[wave][lane] = 0;
      if (e >= 0 && rk == 0) wcnt[wave][e] = cnt;   // after the zero: same wave, in order
      __syncthreads();
      if (wave == 0) {
        int r = left;
#pragma unroll
        for (int w = 0; w < kRerouteWaves; ++w) {
          const int c = wcnt[w][lane];
          room[w][lane] = r;
          r -= c;
        }
        left = r;
      }
      __syncthreads();
      const bool rej = e >= 0 && rk >= room[wave][e >= 0 ? e : 0];
      const uint64_t rmask = __ballot(rej);
      if (lane == 0) wrej[wave] = __popcll(rmask);
      __syncthreads();
      // Exclusive prefix of the waves' rejections (lanes 0..15 hold one wave each).
      int before = 0, total = 0;
      {
        const int v = lane < kRerouteWaves ? wrej[lane] : 0;
        int bsum = lane < wave ? v : 0, tsum = v;
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) {
          bsum += __shfl_xor(bsum, off);
          tsum += __shfl_xor(tsum, off);
        }
        before = __builtin_amdgcn_readfirstlane(bsum);
        total = __builtin_amdgcn_readfirstlane(tsum);
      }
      if (rej) {
        const int pos = nrej + before + __popcll(rmask & lt_mask);
        if (pos < kLdsList) {
          lst_a[nxt][pos] = tok;
          lst_r[nxt][pos] = req;
        } else {
          lists[gidx(nxt, 0, pos)] = tok;
          lists[gidx(nxt, 1, pos)] = req;
        }
      }
      nrej += total;
    }
    if (wave == 0) left = max(left, 0);
    __syncthreads();
    // Next candidates.  A token's cursor advances at least once per round in
    // which it has a rejected slot, so at most E - k + 1 rounds run; past E
    // rounds every request left is dropped (unreachable).
    const bool last = rounds > E;
    int pending = 0;
    // Quad qd serves entries qd, qd + 256, ...; two per pass, with both
    // tokens' score loads in flight before either search.
    const int qd = tid >> 2, ql = tid & 3;
    constexpr int kQuads = kRerouteThreads / 4;
    for (int j0 = qd; j0 < nrej; j0 += 2 * kQuads) {
      int tt[2], tc[2];
      bool head[2];
      float tsc[2][16], tcv[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int j = j0 + b * kQuads;
        tt[b] = 0;
        tc[b] = 64;
        head[b] = false;
        if (j < nrej) {
          tt[b] = get_a(nxt, j);
          head[b] = j == 0 || get_a(nxt, j - 1) != tt[b];   // first entry of its token
          const int c = req_cursor(get_r(nxt, j));
          tc[b] = c == kNoExpert ? 64 : c;            // no cursor: nothing below
        }
        const float* row = score + (size_t)tt[b] * 64;
        tcv[b] = row[min(tc[b], 63)];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const f32x4 s4 = reinterpret_cast<const f32x4*>(row + 16 * ql)[v];
#pragma unroll
          for (int u = 0; u < 4; ++u) tsc[b][4 * v + u] = s4[u];
        }
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (!head[b]) continue;
        const int j = j0 + b * kQuads, t = tt[b];
        int c = tc[b];
        float cv = tcv[b];
        int len = 0;
#pragma unroll 1
        for (int q = 0; q < k && j + q < nrej; ++q) {
          if (get_a(nxt, j + q) != t) break;
          const int slot = req_slot(get_r(nxt, j + q));
          const size_t aq = (size_t)t * k + slot;
          float nv;
          const int nc = (last || c >= E) ? -1 : quad_next_below(tsc[b], ql, E, c, cv, nv);
          if (nc < 0) {                           // nothing left: dropped
            if (ql == 0) {
              topk_idx[aq] = -1;
              topk_w[aq] = 0.f;
            }
          } else {
            if (ql == 0) topk_idx[aq] = nc;
            c = nc;
            cv = nv;
            pending = 1;
          }
          if (ql == 0) put_r(nxt, j + q, pack_req(nc < 0 ? kNoExpert : nc, 0, slot));
          len = q + 1;
        }
        // Every entry of the token carries the token's final cursor.
        if (ql == 0)
          for (int q = 0; q < len; ++q) {
            const int r = get_r(nxt, j + q);
            put_r(nxt, j + q, pack_req(req_expert(r), c, req_slot(r)));
          }
      }
    }
    if (!__syncthreads_or(pending)) break;
    n = nrej;
    cur = nxt;
    nxt ^= 1;
  }
  // Weights of the served experts, eight loads per thread in flight at once.
  if (rounds > 1) {
    for (int b0 = 0; b0 < A; b0 += 8 * kRerouteThreads) {
      int ex[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int a = b0 + q * kRerouteThreads + tid;
        ex[q] = a < A ? topk_idx[a] : -1;
      }
      float wv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int a = b0 + q * kRerouteThreads + tid;
        wv[q] = wt[(size_t)(min(a, A - 1) / k) * E + max(ex[q], 0)];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (ex[q] >= 0) topk_w[b0 + q * kRerouteThreads + tid] = wv[q];
    }
  }
  if (tid == 0 && rounds_out) *rounds_out = rounds;
}

hipError_t launch_reroute(const RerouteArgs& a, hipStream_t s) {
  reroute_kernel<<<1, kRerouteThreads, 0, s>>>(a.score, a.wt, a.T, a.k, a.E, a.capacity,
                                               a.topk_idx, a.topk_w, a.lists, a.rounds);
  return hipGetLastError();
}

}  // namespace moe
