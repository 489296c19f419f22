// MoE routing (top-k of the router's softmax, expert-sorted dispatch order) and the gate-weighted
// combine of the experts' rows back to tokens.
//
//   moe_topk_kernel     one wave per token: the row's logits sit in registers (E/64 per lane); wave
//                       max and Σ exp give the softmax; k rounds of a wave arg-max over (logit, id)
//                       pick the experts, the larger logit first and the lower id on equal logits.
//                       The choice compares the fp32 logits themselves (softmax is monotone), so no
//                       rounding of the probabilities can reorder it.
//   moe_count_kernel    one workgroup: per-expert counts (LDS integer atomics, order-free) and their
//                       exclusive prefix, the group offsets.
//   moe_dispatch_kernel one workgroup per expert: its threads cut the tokens into contiguous blocks,
//                       count the block's rows for the expert, take an exclusive prefix over the
//                       blocks, and write the rows in token order: row_token (row -> token) and
//                       token_row ((token, j) -> row).  Integer work only: bit-exact and
//                       deterministic.
//   moe_combine_kernel  one workgroup per token: out[t] = Σ_j gate[t, j]·Z[token_row[t, j]] in fp32,
//                       j in order; 16-byte loads of the k rows (HBM-bound).  Rows outside
//                       [0, rows) contribute nothing.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace tp {

namespace {

constexpr int MOE_MAX_E = 1024;
constexpr int MOE_MAX_K = 32;

template <int EPL>
__global__ __launch_bounds__(256) void moe_topk_kernel(int tokens, int E, int k, const float* __restrict__ logits,
                                                       float* __restrict__ gates, int* __restrict__ experts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= tokens) return;                      // whole waves leave together: no block barrier below
  const float* row = logits + (long)t * E;
  float v[EPL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -INFINITY;
    m = fmaxf(m, v[i]);
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (lane + 64 * i < E) z += expf(v[i] - m);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) z += __shfl_xor(z, s, 64);
  unsigned taken = 0;                            // bit i: entry lane + 64 i already chosen
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || bi == 0x7fffffff)) {   // ascending ids: > keeps the lower
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
      const float ov = __shfl_xor(bv, s, 64);
      const int oi = __shfl_xor(bi, s, 64);
      if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == 0) {
      experts[(long)t * k + j] = bi;
      gates[(long)t * k + j] = expf(bv - m) / z;
    }
  }
}

__global__ __launch_bounds__(1024) void moe_count_kernel(int n, int E, const int* __restrict__ experts,
                                                         int* __restrict__ offsets) {
  __shared__ int cnt[MOE_MAX_E];
  for (int e = threadIdx.x; e < E; e += 1024) cnt[e] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += 1024) {
    const int e = experts[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) {
      acc += cnt[e];
      offsets[e + 1] = acc;
    }
  }
}

__global__ __launch_bounds__(256) void moe_dispatch_kernel(int tokens, int k, const int* __restrict__ experts,
                                                           const int* __restrict__ offsets,
                                                           int* __restrict__ row_token, int* __restrict__ token_row) {
  __shared__ int pre[256];
  const int e = blockIdx.x;
  const int per = (tokens + 255) / 256;
  const int t0 = min(tokens, threadIdx.x * per), t1 = min(tokens, t0 + per);
  int c = 0;
  for (int t = t0; t < t1; ++t)
    for (int j = 0; j < k; ++j) c += experts[(long)t * k + j] == e;
  pre[threadIdx.x] = c;
  __syncthreads();
  // exclusive prefix over the 256 blocks (Hillis-Steele on a copy, fixed order)
  for (int s = 1; s < 256; s <<= 1) {
    const int add = threadIdx.x >= s ? pre[threadIdx.x - s] : 0;
    __syncthreads();
    pre[threadIdx.x] += add;
    __syncthreads();
  }
  int row = offsets[e] + pre[threadIdx.x] - c;
  for (int t = t0; t < t1; ++t)
    for (int j = 0; j < k; ++j)
      if (experts[(long)t * k + j] == e) {
        row_token[row] = t;
        token_row[(long)t * k + j] = row;
        ++row;
      }
}

template <typename T, int V>
__global__ __launch_bounds__(256) void moe_combine_kernel(int k, int H, const T* __restrict__ Z,
                                                          const float* __restrict__ gates,
                                                          const int* __restrict__ token_row, int rows,
                                                          T* __restrict__ out) {
  const long t = blockIdx.x;
  for (int c = V * threadIdx.x; c < H; c += V * 256) {
    float acc[V];
#pragma unroll
    for (int q = 0; q < V; ++q) acc[q] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = token_row[t * k + j];
      if (r < 0 || r >= rows) continue;
      const float g = gates[t * k + j];
      const T* src = Z + (long)r * H + c;
      if constexpr (V == 8) {
        const bf16x8 z = *(const bf16x8*)src;
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += g * (float)z[q];
      } else if constexpr (V == 4) {
        const f32x4 z = *(const f32x4*)src;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += g * z[q];
      } else {
        acc[0] += g * to_f32(*src);
      }
    }
    T* dst = out + t * H + c;
    if constexpr (V == 8) {
      bf16x8 o;
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = (bf16)acc[q];
      *(bf16x8*)dst = o;
    } else if constexpr (V == 4) {
      *(f32x4*)dst = (f32x4){acc[0], acc[1], acc[2], acc[3]};
    } else {
      *dst = from_f32<T>(acc[0]);
    }
  }
}

template <int EPL>
hipError_t topk_t(int tokens, int E, int k, const float* logits, float* gates, int* experts, hipStream_t s) {
  moe_topk_kernel<EPL><<<(tokens + 3) / 4, 256, 0, s>>>(tokens, E, k, logits, gates, experts);
  return hipGetLastError();
}

}  // namespace

int moe_max_experts() { return MOE_MAX_E; }
int moe_max_top_k() { return MOE_MAX_K; }

hipError_t launch_moe_route(int tokens, int E, int k, const float* logits, float* gates, int* expert_idx,
                            int* group_offsets, int* row_token, int* token_row, hipStream_t s) {
  if (E < 1 || E > MOE_MAX_E || k < 1 || k > MOE_MAX_K || k > E || tokens < 0) return hipErrorInvalidValue;
  const double n = (double)tokens * k;
  if (tokens > 0) {
    ProfScope p("moe_topk", s, 4.0 * tokens * E, 4.0 * tokens * E + 8.0 * n);
    hipError_t e;
    if (E <= 64) e = topk_t<1>(tokens, E, k, logits, gates, expert_idx, s);
    else if (E <= 128) e = topk_t<2>(tokens, E, k, logits, gates, expert_idx, s);
    else if (E <= 256) e = topk_t<4>(tokens, E, k, logits, gates, expert_idx, s);
    else if (E <= 512) e = topk_t<8>(tokens, E, k, logits, gates, expert_idx, s);
    else e = topk_t<16>(tokens, E, k, logits, gates, expert_idx, s);
    if (e != hipSuccess) return e;
  }
  {
    ProfScope p("moe_count", s, 0.0, 4.0 * n + 4.0 * (E + 1));
    moe_count_kernel<<<1, 1024, 0, s>>>((int)n, E, expert_idx, group_offsets);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (tokens == 0) return hipSuccess;
  ProfScope p("moe_dispatch", s, 0.0, 4.0 * n * E + 8.0 * n);
  moe_dispatch_kernel<<<E, 256, 0, s>>>(tokens, k, expert_idx, group_offsets, row_token, token_row);
  return hipGetLastError();
}

hipError_t launch_moe_combine(int dtype, int tokens, int k, int H, const void* Z, const float* gates,
                              const int* token_row, int rows, void* out, hipStream_t s) {
  if (tokens <= 0 || H <= 0) return hipSuccess;
  const double es = dtype == DT_BF16 ? 2.0 : 4.0;
  ProfScope p("moe_combine", s, 2.0 * tokens * k * (double)H,
              es * ((double)tokens * k * H + (double)tokens * H) + 8.0 * tokens * k);
  if (dtype == DT_BF16) {
    if (H % 8 == 0) moe_combine_kernel<bf16, 8><<<tokens, 256, 0, s>>>(k, H, (const bf16*)Z, gates, token_row, rows, (bf16*)out);
    else moe_combine_kernel<bf16, 1><<<tokens, 256, 0, s>>>(k, H, (const bf16*)Z, gates, token_row, rows, (bf16*)out);
  } else {
    if (H % 4 == 0) moe_combine_kernel<float, 4><<<tokens, 256, 0, s>>>(k, H, (const float*)Z, gates, token_row, rows, (float*)out);
    else moe_combine_kernel<float, 1><<<tokens, 256, 0, s>>>(k, H, (const float*)Z, gates, token_row, rows, (float*)out);
  }
  return hipGetLastError();
}

}  // namespace tp
