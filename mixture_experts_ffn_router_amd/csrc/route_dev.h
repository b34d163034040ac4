// Per-token routing on one wavefront, shared by the routing kernel and the
// decode kernels (which recompute the routing of their few tokens in every
// block).  See route.hip for the method and its sources.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

// One token's routing on one wavefront: lane k < K ends with slot k's weight
// and expert id.  z points at the token's E logits; load_logits / route_logits
// split the load from the arithmetic so a caller can issue several tokens'
// loads at once.
// The logits a lane holds: experts lane, lane + 64, ... (0 past E), and, when
// the layer has per-expert scales, those experts' scales (loaded with the
// logits, so no load waits on the selection).
template <int VPL>
struct TokenLogits {
  float v[VPL];
  float p[VPL];
};
template <int VPL>
__device__ __forceinline__ TokenLogits<VPL> load_logits(const float* __restrict__ z, int E, int lane,
                                                        const float* __restrict__ pes = nullptr) {
  TokenLogits<VPL> r;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int idx = lane + 64 * j;
    r.v[j] = idx < E ? z[idx] : 0.f;
    r.p[j] = (pes && idx < E) ? pes[idx] : 1.f;
  }
  return r;
}

// Group-limited routing (llama.cpp MoE lesson: experts split into groups, groups
// picked first): the experts form G equal contiguous ranges; a range's score is
// its largest key (the same order as its largest logit or probability).  The KG
// best ranges are picked, ties to the lower range, and every other expert's key
// is cleared to 0, below every real key, so the top-k never takes it while K is
// at most the number of experts in the picked ranges.
template <int VPL>
__device__ __forceinline__ void mask_groups(uint32_t (&key)[VPL], int E, int G, int KG, int lane) {
  const int gsz = E / G;
  uint32_t gkey = 0u;  // lane g < G: the best key of range g
  for (int g = 0; g < G; ++g) {
    uint32_t b = 0u;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int idx = lane + 64 * j;
      if (idx < E && idx / gsz == g && key[j] > b) b = key[j];
    }
    b = wave_max_u32(b);
    if (lane == g) gkey = b;
  }
  uint64_t picked = 0;  // the same on every lane
  for (int r = 0; r < KG; ++r) {
    const bool open = lane < G && !((picked >> lane) & 1ull);
    const uint32_t c = open ? gkey : 0u;
    const uint32_t gk = wave_max_u32(c);
    const uint32_t gi = wave_min_u32(open && c == gk ? (uint32_t)lane : 0xFFFFFFFFu);
    picked |= 1ull << gi;
  }
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int idx = lane + 64 * j;
    if (idx < E && !((picked >> (idx / gsz)) & 1ull)) key[j] = 0u;
  }
}

// pes: the layer's per-expert scales (NULL: none); zl.p must hold them (load_logits
// with the same pes).
template <int VPL>
__device__ __forceinline__ void route_logits(const TokenLogits<VPL>& zl, int E, int K, const RouteOpts& o,
                                             const float* __restrict__ pes, int lane, float& w_slot,
                                             int& id_slot) {
  float v[VPL];
  uint32_t key[VPL];
  float lmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    int idx = lane + 64 * j;
    v[j] = zl.v[j];
    if (idx < E) {
      key[j] = f32_order_key(v[j]);
      lmax = fmaxf(lmax, v[j]);
    } else {
      key[j] = 0u;  // below every finite key: never selected while K <= E
    }
  }
  if (o.groups > 1) mask_groups<VPL>(key, E, o.groups, o.topk_groups, lane);
  const bool sigmoid = o.scoring == SCORE_SIGMOID;
  const float m = sigmoid ? 0.f : wave_max_f32(lmax);

  double s_all = 1.0;  // softmax without renormalisation: the sum over all E
  if (!o.renorm && !sigmoid) {
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (lane + 64 * j < E) s += (double)expf(v[j] - m);
    s_all = wave_sum_f64(s);
  }

  // Top-k by radix select on the keys: tau = the K-th largest key, found bit by
  // bit from the top (a bit stays set while at least K keys are >= the prefix);
  // every key above tau is selected, and of the keys equal to tau the lowest
  // indices (index = lane + 64 j: all j = 0 before j = 1, ...) fill the rest.
  // Counts come from ballots, so each step is a few scalar instructions.  Once
  // exactly K keys are >= the prefix they are the K largest, and the rest of the
  // bits cannot change the selection (below, every key above tau is taken and
  // the keys equal to it complete K), so the search stops there: after about
  // log2(E) informative bits when the top keys are distinct, all 32 with a tie
  // at the K-th place.
  uint32_t tau = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = tau | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < VPL; ++j) cnt += __popcll(__ballot(key[j] >= c));
    if (cnt >= K) {
      tau = c;
      if (cnt == K) break;
    }
  }
  const uint64_t lt = (1ull << lane) - 1ull;
  int need = K;  // keys equal to tau still to take
#pragma unroll
  for (int j = 0; j < VPL; ++j) need -= __popcll(__ballot(key[j] > tau));
  uint32_t sel = 0;  // bit j: this lane's value j is selected
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const uint64_t eq = __ballot(key[j] == tau);
    if (key[j] > tau || (key[j] == tau && __popcll(eq & lt) < need)) sel |= 1u << j;
    const int here = __popcll(eq);
    need -= here < need ? here : need;
  }
  // Slot order: a selected value's slot is the number of selected values with a
  // larger key, or an equal key and a lower index; the lane of that slot takes
  // its index and key.
  int my_id = 0;
  uint32_t my_key = 0;
#pragma unroll
  for (int j2 = 0; j2 < VPL; ++j2) {
    uint64_t m2 = __ballot((sel >> j2) & 1u);
    while (m2) {
      const int l2 = __builtin_ctzll(m2);
      m2 &= m2 - 1;
      const uint32_t k2 = (uint32_t)__builtin_amdgcn_readlane((int)key[j2], l2);
      const int idx2 = l2 + 64 * j2;
      int r = 0;
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const bool sj = (sel >> j) & 1u;
        r += __popcll(__ballot(sj && (key[j] > k2 || (key[j] == k2 && lane + 64 * j < idx2))));
      }
      if (lane == r) {
        my_id = idx2;
        my_key = k2;
      }
    }
  }
  // softmax: fp32 exp(z - max); sigmoid: 1 / (1 + exp(-z)) in fp64; the sum of the
  // selected terms in fp64
  double my_e = 0.0;
  if (lane < K) {
    const float zk = f32_from_order_key(my_key);
    my_e = sigmoid ? 1.0 / (1.0 + exp(-(double)zk)) : (double)expf(zk - m);
  }
  const double denom = wave_sum_f64(my_e);
  // the scale of this slot's expert, from the lane that loaded it
  float my_p = 1.f;
  if (pes) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const float pj = __shfl(zl.p[j], my_id & 63, 64);
      if ((my_id >> 6) == j) my_p = pj;
    }
  }
  w_slot = 0.f;
  id_slot = 0;
  if (lane < K) {
    const double d = o.renorm ? (denom > 0.0 ? denom : 1.0) : s_all;
    double w = my_e / d;
    if (pes) w *= (double)my_p;
    w_slot = (float)w;
    id_slot = my_id;
  }
}

}  // namespace moe
