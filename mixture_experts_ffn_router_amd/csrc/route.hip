// Routing: softmax over all experts, top-k, renormalisation, per-expert
// scale fold ("Gemma 4 26B-A4B MoE walkthrough" sections 4-5; the routing
// function of Gemma4MoE in the vLLM gemma4 API docs), with the variants of the
// llama.cpp MoE lesson: sigmoid scoring and expert groups.
//
// One wavefront per token.  Lane l holds the logits of experts l, l+64, ...
// Selection works on the order-preserving uint32 image of each logit (the key;
// value descending, index ascending on ties): a radix select finds the K-th
// largest key from ballot counts, one bit per step, the keys above it and the
// lowest-index keys equal to it are the selection, and each selected value's
// slot is its number of selected predecessors in (key desc, index asc) order,
// again from ballots.  The selected logit is recovered exactly from its key;
// slot k's result ends up in lane k.
//
// Renormalised weights are computed as exp(z_k - m) / sum_{selected} exp(z_j - m):
// the full softmax denominator cancels exactly (the page's own derivation of
// why softmax-all + mask + renorm equals a softmax over the selected logits),
// so only the selected terms are rounded.  Without renormalisation the weight
// is exp(z_k - m) / sum_{all E} exp(z_j - m).  The exponentials are fp32;
// the sums, the division and the scale product are carried in fp64 and
// rounded once, so a weight is within about two fp32 ulps of exact.
// Sigmoid scoring selects on the logits too (the sigmoid is increasing) and
// evaluates 1 / (1 + exp(-z)) of the K selected logits in fp64.  Expert groups
// clear the keys of the experts outside the picked groups before the top-k.
#include "common.h"
#include "kernels.h"
#include "route_dev.h"

namespace moe {

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t T,
                                                    int E, int K, RouteOpts ro,
                                                    const float* __restrict__ pes,
                                                    float* __restrict__ w_out,
                                                    int32_t* __restrict__ ids_out, int out_stride,
                                                    int n_shared, int nparts, int64_t part_stride,
                                                    float* __restrict__ sum_out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  // the logits of token t: partial sums of the router GEMM's reduction parts, in part order
  TokenLogits<VPL> z = load_logits<VPL>(logits + t * (int64_t)E, E, lane, pes);
  for (int q = 1; q < nparts; ++q) {
    const TokenLogits<VPL> zq = load_logits<VPL>(logits + q * part_stride + t * (int64_t)E, E, lane);
#pragma unroll
    for (int j = 0; j < VPL; ++j) z.v[j] += zq.v[j];
  }
  if (sum_out && nparts > 1) {
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (lane + 64 * j < E) sum_out[t * (int64_t)E + lane + 64 * j] = z.v[j];
  }
  float w;
  int id;
  route_logits<VPL>(z, E, K, ro, pes, lane, w, id);
  int64_t o = t * (int64_t)out_stride + lane;
  if (lane < K) {
    w_out[o] = w;
    ids_out[o] = id;
  } else if (lane < K + n_shared) {
    w_out[o] = 1.f;
    ids_out[o] = E + (lane - K);
  }
}

hipError_t launch_route(const float* logits, int64_t T, int E, int K, const RouteOpts& o, const float* pes,
                        float* w_out, int32_t* ids_out, int out_stride, int n_shared,
                        hipStream_t s, int nparts, int64_t part_stride, float* sum_out) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (E <= 64)
    route_kernel<1><<<grid, block, 0, s>>>(logits, T, E, K, o, pes, w_out, ids_out, out_stride, n_shared, nparts, part_stride, sum_out);
  else if (E <= 128)
    route_kernel<2><<<grid, block, 0, s>>>(logits, T, E, K, o, pes, w_out, ids_out, out_stride, n_shared, nparts, part_stride, sum_out);
  else if (E <= 256)
    route_kernel<4><<<grid, block, 0, s>>>(logits, T, E, K, o, pes, w_out, ids_out, out_stride, n_shared, nparts, part_stride, sum_out);
  else
    route_kernel<8><<<grid, block, 0, s>>>(logits, T, E, K, o, pes, w_out, ids_out, out_stride, n_shared, nparts, part_stride, sum_out);
  return hipGetLastError();
}

}  // namespace moe
