// Routing: softmax over all experts, top-k, renormalisation, per-expert
// scale fold ("Gemma 4 26B-A4B MoE walkthrough" sections 4-5; the routing
// function of Gemma4MoE in the vLLM gemma4 API docs).
//
// One wavefront per token.  Lane l holds the logits of experts l, l+64, ...
// Selection runs K rounds of a wave-wide arg-max on the key (value desc,
// index asc): a DPP max over the order-preserving uint32 image of the value,
// then a DPP min over the indices of the lanes that hold that maximum.  The
// selected logit is recovered exactly from its key, so every lane computes the
// same exp(z - max) for it; slot k's result ends up in lane k.
//
// Renormalised weights are computed as exp(z_k - m) / sum_{selected} exp(z_j - m):
// the full softmax denominator cancels exactly (the page's own derivation of
// why softmax-all + mask + renorm equals a softmax over the selected logits),
// so only the selected terms are rounded.  Without renormalisation the weight
// is exp(z_k - m) / sum_{all E} exp(z_j - m).  The exponentials are fp32;
// the sums, the division and the scale product are carried in fp64 and
// rounded once, so a weight is within about two fp32 ulps of exact.
#include "common.h"
#include "kernels.h"

namespace moe {

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t T,
                                                    int E, int K, int renorm,
                                                    const float* __restrict__ pes,
                                                    float* __restrict__ w_out,
                                                    int32_t* __restrict__ ids_out, int out_stride,
                                                    int n_shared) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* z = logits + t * (int64_t)E;

  float v[VPL];
  uint32_t key[VPL];
  float lmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    int idx = lane + 64 * j;
    if (idx < E) {
      v[j] = z[idx];
      key[j] = f32_order_key(v[j]);
      lmax = fmaxf(lmax, v[j]);
    } else {
      v[j] = 0.f;
      key[j] = 0u;  // below every finite key: never selected while K <= E
    }
  }
  const float m = wave_max_f32(lmax);

  double s_all = 1.0;
  if (!renorm) {
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (lane + 64 * j < E) s += (double)expf(v[j] - m);
    s_all = wave_sum_f64(s);
  }

  uint32_t taken = 0;  // bit j: this lane's value j already selected
  float my_e = 0.f;
  int my_id = 0;
  double denom = 0.0;
  for (int k = 0; k < K; ++k) {
    uint32_t bk = 0, bi = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      if (!((taken >> j) & 1u) && key[j] > bk) {  // j ascending: lowest index wins ties
        bk = key[j];
        bi = (uint32_t)(lane + 64 * j);
      }
    }
    const uint32_t gk = wave_max_u32(bk);
    const uint32_t gi = wave_min_u32(bk == gk ? bi : 0xFFFFFFFFu);
    if ((int)(gi & 63u) == lane) taken |= 1u << (gi >> 6);
    const float e = expf(f32_from_order_key(gk) - m);
    denom += (double)e;  // slot order
    if (lane == k) {
      my_e = e;
      my_id = (int)gi;
    }
  }
  int64_t o = t * (int64_t)out_stride + lane;
  if (lane < K) {
    const double d = renorm ? (denom > 0.0 ? denom : 1.0) : s_all;
    double w = (double)my_e / d;
    if (pes) w *= (double)pes[my_id];
    w_out[o] = (float)w;
    ids_out[o] = my_id;
  } else if (lane < K + n_shared) {
    w_out[o] = 1.f;
    ids_out[o] = E + (lane - K);
  }
}

hipError_t launch_route(const float* logits, int64_t T, int E, int K, int renorm, const float* pes,
                        float* w_out, int32_t* ids_out, int out_stride, int n_shared,
                        hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (E <= 64)
    route_kernel<1><<<grid, block, 0, s>>>(logits, T, E, K, renorm, pes, w_out, ids_out, out_stride, n_shared);
  else if (E <= 128)
    route_kernel<2><<<grid, block, 0, s>>>(logits, T, E, K, renorm, pes, w_out, ids_out, out_stride, n_shared);
  else if (E <= 256)
    route_kernel<4><<<grid, block, 0, s>>>(logits, T, E, K, renorm, pes, w_out, ids_out, out_stride, n_shared);
  else
    route_kernel<8><<<grid, block, 0, s>>>(logits, T, E, K, renorm, pes, w_out, ids_out, out_stride, n_shared);
  return hipGetLastError();
}

}  // namespace moe
