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
//     renormalising, else 1).
//
// The router hands over every token's experts in ranking order with the
// weight each would get.  A token asks its experts in that order, so its k
// router choices are positions 0..k-1 and its next request is the position
// after the last one it asked (its cursor): finding a candidate is one load.
//
// One block (1024 threads; 512 past two slots per token) runs every round, so
// no host synchronisation is needed and the number of rounds stays on the
// device.  A round walks a list of tokens in token order: round 0 every token,
// later rounds the tokens with a slot rejected in the round before (two lists,
// used in turn; the first kLdsList entries live in LDS, the rest in the
// workspace).  An entry is the token id and, packed in one word, its cursor + 1
// and the mask of its slots that ask this round; the i-th of those slots (in
// slot order) asks the expert at position cursor + 1 + i.
//
// Acceptance walks the list in chunks of SUB x (block size) entries; entry
// base + u * (block size) + thread belongs to group (u, wave), and the groups
// are in list order.  Inside a wave, requests to one expert are matched with
// one ballot per bit of the expert id (for each slot column, since one token's
// requests go to different experts); the lowest lane asking an expert
// publishes the group's count.  Wave 0 then turns the groups' counts into the
// room each expert has for each group (its lane x keeps expert x's capacity
// left in a register across chunks).  A request served in a later round
// writes its expert and weight at once; a rejected slot past the last
// position is dropped at once (expert -1, weight 0); a token with slots still
// asking is appended to the other list in the same order.
#include "aux_reduce.h"
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kLdsList = 4096;    // list entries kept in LDS; the rest go to the workspace

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

// Requests ev[s] (an expert id < 64, or -1) of this lane, one per slot column:
// for each, the number of requests to the same expert in the lanes below
// (`rank`) and in the whole wave (`cnt`), over all columns.
template <int KMAX>
__device__ __forceinline__ void wave_rank_cols(const int (&ev)[KMAX], uint64_t lt_mask,
                                               int (&rank)[KMAX], int (&cnt)[KMAX]) {
#pragma unroll
  for (int s = 0; s < KMAX; ++s) rank[s] = cnt[s] = 0;
#pragma unroll
  for (int col = 0; col < KMAX; ++col) {
    const int v = ev[col];
    const uint64_t valid = __ballot(v >= 0);
    uint64_t bb[6];
#pragma unroll
    for (int b = 0; b < 6; ++b) bb[b] = __ballot((v >> b) & 1);
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
      const int xv = ev[s];
      uint32_t lo = (uint32_t)valid, hi = (uint32_t)(valid >> 32);
#pragma unroll
      for (int b = 0; b < 6; ++b) {
        const uint32_t flip = ((uint32_t)(xv >> b) & 1u) - 1u;   // 0 where the bit is set
        lo &= (uint32_t)bb[b] ^ flip;
        hi &= (uint32_t)(bb[b] >> 32) ^ flip;
      }
      const uint64_t same = ((uint64_t)hi << 32) | lo;
      if (xv >= 0) {
        rank[s] += __popcll(same & lt_mask);
        cnt[s] += __popcll(same);
      }
    }
  }
}

// Block 0 reroutes; block 1 reduces the router's aux partials (aux_reduce),
// which the rerouting does not read, so the two run side by side.
template <int KMAX, int SUB, int THREADS>
__global__ __launch_bounds__(THREADS) void reroute_kernel(
    const int32_t* __restrict__ rank_rec, int T, int k, int E, int capacity,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int32_t* __restrict__ lists,
    int32_t* __restrict__ rounds_out, const double* __restrict__ part_psum,
    const int32_t* __restrict__ part_top1, const double* __restrict__ part_z, int nblk,
    int32_t* __restrict__ top1_count, float* __restrict__ prob_mean, float* __restrict__ aux,
    float* __restrict__ z_loss) {
  if (blockIdx.x == 1) {
    __shared__ AuxLds<THREADS> ared;
    aux_reduce<THREADS>(part_psum, part_top1, part_z, nblk, T, E, top1_count, prob_mean, aux,
                        z_loss, ared);
    return;
  }
  constexpr int kWaves = THREADS / 64;
  constexpr int kGroups = SUB * kWaves;             // (sub-chunk, wave) groups, list order
  constexpr int kChunk = SUB * THREADS;
  static_assert(kGroups <= 64, "one lane per group in the scans");
  __shared__ int wcnt[kGroups][64];   // requests per (group, expert) in the chunk
  __shared__ int room[kGroups][64];   // room expert x has for group g's requests
  __shared__ int wapp[kGroups];       // tokens appended per group in the chunk
  __shared__ int lst_t[2][kLdsList];  // list heads: token ids
  __shared__ int lst_m[2][kLdsList];  // list heads: words
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int left = capacity;                // wave 0, lane x: capacity expert x has left
  int n = T;                          // entries of the list walked this round
  int cur = 1, nxt = 0;               // lists read and written this round
  int rounds = 0;
  // Entry i of list l: LDS below kLdsList, workspace above (lists holds the
  // token ids of list 0, words of list 0, token ids of list 1, words of list 1).
  // Word: bits 0..7 cursor + 1, bits 8..15 the slots asking this round.
  auto gidx = [&](int l, int field, int i) -> size_t { return (size_t)(2 * l + field) * T + i; };
  auto rec = [&](int t, int pos, int field) -> int32_t {
    return rank_rec[((size_t)t * 64 + pos) * 2 + field];
  };
  for (;;) {
    ++rounds;
    const bool first = rounds == 1;
    // Positions grow by at least one per round, so past E rounds nothing is left
    // to ask (unreachable; bounds the loop).
    const bool last = rounds > E;
    int napp = 0;                     // entries appended so far this round (same in every wave)
    // Entries base + u * THREADS + tid: token, cursor, asking slots, and the
    // experts and weights the slots ask for.
    auto load_chunk = [&](int base, int (&tok)[SUB], int (&cpos)[SUB], int (&ask)[SUB],
                          int (&ev)[SUB][KMAX], float (&wv)[SUB][KMAX]) {
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        const int i = base + u * THREADS + tid;
        tok[u] = -1;
        cpos[u] = -1;
        ask[u] = 0;
#pragma unroll
        for (int s = 0; s < KMAX; ++s) {
          ev[u][s] = -1;
          wv[u][s] = 0.f;
        }
        if (i >= n) continue;
        if (first) {
          tok[u] = i;
          ask[u] = (1 << k) - 1;
#pragma unroll
          for (int s = 0; s < KMAX; ++s)
            if (s < k) ev[u][s] = topk_idx[(size_t)i * k + s];
        } else {
          int m;
          if (i < kLdsList) {
            tok[u] = lst_t[cur][i];
            m = lst_m[cur][i];
          } else {
            tok[u] = lists[gidx(cur, 0, i)];
            m = lists[gidx(cur, 1, i)];
          }
          cpos[u] = (m & 0xff) - 1;
          ask[u] = (m >> 8) & 0xff;
          int j = 0;
#pragma unroll
          for (int s = 0; s < KMAX; ++s)
            if ((ask[u] >> s) & 1) {
              ev[u][s] = rec(tok[u], cpos[u] + 1 + j, 0);
              wv[u][s] = __int_as_float(rec(tok[u], cpos[u] + 1 + j, 1));
              ++j;
            }
        }
        // An id outside [0, E) (not produced by the router) is dropped.
#pragma unroll
        for (int s = 0; s < KMAX; ++s)
          if (((ask[u] >> s) & 1) && (ev[u][s] < 0 || ev[u][s] >= E)) {
            const size_t aq = (size_t)tok[u] * k + s;
            topk_idx[aq] = -1;
            topk_w[aq] = 0.f;
            ev[u][s] = -1;
          }
      }
    };
    int tok[SUB], cpos[SUB], ask[SUB], ev[SUB][KMAX];
    float wv[SUB][KMAX];
    load_chunk(0, tok, cpos, ask, ev, wv);
    for (int base = 0; base < n; base += kChunk) {
      // The next chunk's loads go out before this chunk's decisions.
      int ntok[SUB], ncpos[SUB], nask[SUB], nev[SUB][KMAX];
      float nwv[SUB][KMAX];
      load_chunk(base + kChunk, ntok, ncpos, nask, nev, nwv);
      // Ranks inside each wave and the per-group counts.
      int rk[SUB][KMAX];
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        int cnt[KMAX];
        wave_rank_cols<KMAX>(ev[u], lt_mask, rk[u], cnt);
        const int g = u * kWaves + wave;
        wcnt[g][lane] = 0;
#pragma unroll
        for (int s = 0; s < KMAX; ++s)   // after the zero: same wave, in order
          if (ev[u][s] >= 0 && rk[u][s] == 0) wcnt[g][ev[u][s]] = cnt[s];
      }
      __syncthreads();
      if (wave == 0) {
        // Group g holds entries base + 64 g .. base + 64 g + 63, so the groups
        // with entries are a prefix.
        const int ng = min(kGroups, (n - base + 63) >> 6);
        int r = left;
#pragma unroll 4
        for (int g = 0; g < ng; ++g) {
          const int c = wcnt[g][lane];
          room[g][lane] = r;
          r -= c;
        }
        left = r;
      }
      __syncthreads();
      // Decisions, drops past the last position, and the tokens still asking.
      int word[SUB];
      uint64_t amask[SUB];
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        const int g = u * kWaves + wave;
        int rej = 0;
#pragma unroll
        for (int s = 0; s < KMAX; ++s) {
          const int e = ev[u][s];
          if (e < 0) continue;
          if (rk[u][s] < room[g][e]) {
            if (!first) {                  // served by another expert than the router's choice
              const size_t aq = (size_t)tok[u] * k + s;
              topk_idx[aq] = e;
              topk_w[aq] = wv[u][s];
            }
          } else {
            rej |= 1 << s;
          }
        }
        // Positions asked this round: the popcount of ask after cpos.
        const int cnew = cpos[u] + __popc(ask[u]);
        int keep = 0, i = 0;
#pragma unroll
        for (int s = 0; s < KMAX; ++s)
          if ((rej >> s) & 1) {
            if (!last && cnew + 1 + i < E) {
              keep |= 1 << s;
            } else {                       // nothing left to ask: dropped
              const size_t aq = (size_t)tok[u] * k + s;
              topk_idx[aq] = -1;
              topk_w[aq] = 0.f;
            }
            ++i;
          }
        word[u] = (cnew + 1) | (keep << 8);
        amask[u] = __ballot(keep != 0);
        if (lane == 0) wapp[g] = __popcll(amask[u]);
      }
      __syncthreads();
      // Exclusive prefix of the groups' appends (lane g holds group g).
      int incl = lane < kGroups ? wapp[lane] : 0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      const int total = __shfl(incl, 63);
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        const int g = u * kWaves + wave;
        const int before = __shfl(incl, g) - __popcll(amask[u]);   // every lane takes part
        if ((word[u] >> 8) == 0) continue;
        const int pos = napp + before + __popcll(amask[u] & lt_mask);
        if (pos < kLdsList) {
          lst_t[nxt][pos] = tok[u];
          lst_m[nxt][pos] = word[u];
        } else {
          lists[gidx(nxt, 0, pos)] = tok[u];
          lists[gidx(nxt, 1, pos)] = word[u];
        }
      }
      napp += total;
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        tok[u] = ntok[u];
        cpos[u] = ncpos[u];
        ask[u] = nask[u];
#pragma unroll
        for (int s = 0; s < KMAX; ++s) {
          ev[u][s] = nev[u][s];
          wv[u][s] = nwv[u][s];
        }
      }
    }
    if (wave == 0) left = max(left, 0);
    __syncthreads();
    if (napp == 0) break;
    n = napp;
    cur = nxt;
    nxt ^= 1;
  }
  if (tid == 0 && rounds_out) *rounds_out = rounds;
}

hipError_t launch_reroute(const RerouteArgs& a, hipStream_t s) {
#define MOE_REROUTE(KMAX, SUB, THREADS)                                                      \
  reroute_kernel<KMAX, SUB, THREADS><<<2, THREADS, 0, s>>>(                                    \
      a.rank, a.T, a.k, a.E, a.capacity, a.topk_idx, a.topk_w, a.lists, a.rounds, a.part_psum, \
      a.part_top1, a.part_z, a.nblk, a.top1_count, a.prob_mean, a.aux, a.z_loss)
  // Entries per thread and chunk shrink as the slots per token grow, and past
  // two slots the block halves, so that the requests stay in registers.
  if (a.k == 1)
    MOE_REROUTE(1, 4, 1024);
  else if (a.k == 2)
    MOE_REROUTE(2, 2, 1024);
  else if (a.k <= 4)
    MOE_REROUTE(4, 4, 512);
  else if (a.k <= 8)
    MOE_REROUTE(8, 2, 512);
  else
    return hipErrorInvalidValue;
#undef MOE_REROUTE
  return hipGetLastError();
}

}  // namespace moe
