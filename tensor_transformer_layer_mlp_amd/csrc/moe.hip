// MoE routing (top-k of the router's softmax, expert-sorted dispatch order) and the gate-weighted
// combine of the experts' rows back to tokens.
//
//   moe_topk_rows_kernel (E <= 256) / moe_topk_kernel: a workgroup of 16 waves owns a chunk of 64
//                       consecutive tokens, one token per 16-lane row (larger E: a wave per token,
//                       one at a time): the token's logits sit in registers (E/16 or E/64 per lane);
//                       max and Σ exp over the row (or wave) give the softmax; k rounds of an arg-max
//                       over (logit, id) (cross-lane exchanges on the VALU: DPP and permlane swaps, no
//                       LDS) pick the
//                       experts, the larger logit first and the lower id on equal logits.  The choice
//                       compares the fp32 logits themselves (softmax is monotone), so no rounding of
//                       the probabilities can reorder it.  The chunk's per-expert counts (LDS integer
//                       atomics: order-free) go to counts[chunk][e].
//   moe_scan_kernel     a workgroup per expert: the exclusive prefix of its counts over the chunks
//                       (each thread a contiguous run of chunks, then an LDS scan over the threads)
//                       and the expert's total.
//   moe_scatter_kernel  a workgroup per chunk: the exclusive prefix of the experts' totals (the group
//                       offsets, written by chunk 0); then thread i takes the chunk's i-th (token, j)
//                       entry in token order and ranks it among the earlier entries with the same
//                       expert, so rows land in (expert, token) order: row_token (row -> token) and
//                       token_row ((token, j) -> row).  Integer work only: exact and deterministic.
//   moe_combine_kernel  one workgroup per token: out[t] = Σ_j gate[t, j]·Z[token_row[t, j]] in fp32,
//                       j in order; 16-byte loads of the k rows (HBM-bound).  Rows outside
//                       [0, rows) contribute nothing.  Without gates every gate is 1 (the
//                       dispatch's backward: a token's input gradient sums its k rows').
//   moe_combine_bwd_kernel  one workgroup per token, the combine's backward: for each of its k rows
//                       dZ[r] = gate·d_out[t] and the gate gradient ⟨d_out[t], Z[r]⟩ (fp32, reduced
//                       in a fixed order); optionally also the dispatched copy X_perm[r] = X[t] (the
//                       MoE backward does not ask for it: its dW1 gathers X's rows inside its loads).
//   moe_route_bwd_kernel    one wave per token: the softmax again from the fp32 logits, then
//                       d_logits[e] = p_e·(dg(e) − Σ_j dg_j·p_{i_j}), dg(e) the gradient of the gate
//                       that chose e (0 if none did).
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace tp {

namespace {

constexpr int MOE_MAX_E = 1024;
constexpr int MOE_MAX_K = 32;

constexpr int MOE_CHUNK = 64;                   // tokens per routing chunk

constexpr int TOPK_THREADS = 1024;

// Cross-lane exchanges for wave-wide reductions without LDS traffic.  Step i hands lane l the value
// of a partner: l ^ 1 and l ^ 2 (DPP quad permutes), the mirror of l in its 8-lane half-row and in its
// 16-lane row (DPP row_half_mirror, row_mirror), then l ^ 16 and l ^ 32 (v_permlane16/32_swap).  Each
// step pairs the groups the earlier steps have combined, so after all six an associative and
// commutative operation has combined the 64 lanes in every lane.  The two swaps return {own value,
// partner's value} in an order that depends on the lane; a commutative combine of both is the same.
template <int STEP>
__device__ __forceinline__ unsigned dpp_partner(unsigned v) {
  static_assert(STEP >= 0 && STEP < 4, "DPP steps");
  constexpr int ctrl = STEP == 0 ? 0xB1 : STEP == 1 ? 0x4E : STEP == 2 ? 0x141 : 0x140;
  return (unsigned)__builtin_amdgcn_mov_dpp((int)v, ctrl, 0xF, 0xF, false);
}
__device__ __forceinline__ float wave_max(float m) {
  m = fmaxf(m, __uint_as_float(dpp_partner<0>(__float_as_uint(m))));
  m = fmaxf(m, __uint_as_float(dpp_partner<1>(__float_as_uint(m))));
  m = fmaxf(m, __uint_as_float(dpp_partner<2>(__float_as_uint(m))));
  m = fmaxf(m, __uint_as_float(dpp_partner<3>(__float_as_uint(m))));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sum(float z) {
  z += __uint_as_float(dpp_partner<0>(__float_as_uint(z)));
  z += __uint_as_float(dpp_partner<1>(__float_as_uint(z)));
  z += __uint_as_float(dpp_partner<2>(__float_as_uint(z)));
  z += __uint_as_float(dpp_partner<3>(__float_as_uint(z)));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(z), __float_as_uint(z), false, false);
  z = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(z), __float_as_uint(z), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Order key of a (logit, expert id) candidate: a larger logit, then a lower id, gives a larger key,
// so one unsigned 64-bit comparison orders candidates exactly as the fp32 comparison of the logits
// (ties to the lower id) does.  High word: the logit's bits mapped to an unsigned order (negative
// values reversed, non-negative ones above them; −0 is taken as +0, which the float comparison
// treats as equal); low word: ~id.  Key 0 lies below every candidate (a taken or absent entry).
__device__ __forceinline__ unsigned long long cand_key(float v, int e) {
  const unsigned u = v == 0.f ? 0u : __float_as_uint(v);
  const unsigned hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)hi << 32) | (unsigned)~e;
}
__device__ __forceinline__ float key_logit(unsigned long long k) {
  const unsigned hi = (unsigned)(k >> 32);
  return __uint_as_float((hi & 0x80000000u) ? (hi & 0x7fffffffu) : ~hi);
}
__device__ __forceinline__ int key_id(unsigned long long k) { return (int)~(unsigned)k; }
__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}
template <int STEP>
__device__ __forceinline__ unsigned long long key_step(unsigned long long k) {
  const unsigned lo = dpp_partner<STEP>((unsigned)k), hi = dpp_partner<STEP>((unsigned)(k >> 32));
  return umax64(k, ((unsigned long long)hi << 32) | lo);
}
// The largest key of the wave, in every lane (branch-free selects).
__device__ __forceinline__ unsigned long long wave_max_key(unsigned long long k) {
  k = key_step<0>(k);
  k = key_step<1>(k);
  k = key_step<2>(k);
  k = key_step<3>(k);
  auto rl = __builtin_amdgcn_permlane16_swap((unsigned)k, (unsigned)k, false, false);
  auto rh = __builtin_amdgcn_permlane16_swap((unsigned)(k >> 32), (unsigned)(k >> 32), false, false);
  k = umax64(((unsigned long long)rh[0] << 32) | rl[0], ((unsigned long long)rh[1] << 32) | rl[1]);
  rl = __builtin_amdgcn_permlane32_swap((unsigned)k, (unsigned)k, false, false);
  rh = __builtin_amdgcn_permlane32_swap((unsigned)(k >> 32), (unsigned)(k >> 32), false, false);
  return umax64(((unsigned long long)rh[0] << 32) | rl[0], ((unsigned long long)rh[1] << 32) | rl[1]);
}

template <int EPL>
__global__ __launch_bounds__(TOPK_THREADS) void moe_topk_kernel(int tokens, int E, int k, const float* __restrict__ logits,
                                                       float* __restrict__ gates, int* __restrict__ experts,
                                                       int* __restrict__ counts) {
  __shared__ int cnt[MOE_MAX_E];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += TOPK_THREADS) cnt[e] = 0;
  __syncthreads();
  const int c0 = blockIdx.x * MOE_CHUNK, c1 = min(tokens, c0 + MOE_CHUNK);
  for (int t = c0 + w; t < c1; t += TOPK_THREADS / 64) {
    const float* row = logits + (long)t * E;
    float v[EPL];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? row[e] : -INFINITY;
      m = fmaxf(m, v[i]);
    }
    m = wave_max(m);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + 64 * i < E) z += expf(v[i] - m);
    z = wave_sum(z);
    unsigned long long key[EPL];                 // 0: absent or already chosen
#pragma unroll
    for (int i = 0; i < EPL; ++i) key[i] = lane + 64 * i < E ? cand_key(v[i], lane + 64 * i) : 0ull;
    for (int j = 0; j < k; ++j) {
      unsigned long long best = key[0];
#pragma unroll
      for (int i = 1; i < EPL; ++i) best = umax64(best, key[i]);
      best = wave_max_key(best);
#pragma unroll
      for (int i = 0; i < EPL; ++i) key[i] = key[i] == best ? 0ull : key[i];   // ids are unique
      if (lane == 0) {
        const int bi = key_id(best);
        experts[(long)t * k + j] = bi;
        gates[(long)t * k + j] = expf(key_logit(best) - m) / z;
        atomicAdd(&cnt[bi], 1);
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += TOPK_THREADS) counts[(long)blockIdx.x * E + e] = cnt[e];
}

// The same selection with one token per 16-lane row (four tokens per wave at once), for E <= 256:
// lane i of a row holds entries i + 16j (EPR = E/16 of them), and every reduction is the four DPP
// steps that stay inside the row (quad permutes, half-row and row mirrors).  A wave's tokens are
// c0 + 4w .. c0 + 4w + 3; rows past the chunk's end compute but write nothing.
template <int EPR>
__global__ __launch_bounds__(TOPK_THREADS) void moe_topk_rows_kernel(int tokens, int E, int k,
                                                                     const float* __restrict__ logits,
                                                                     float* __restrict__ gates,
                                                                     int* __restrict__ experts,
                                                                     int* __restrict__ counts) {
  constexpr int NW = TOPK_THREADS / 64;
  static_assert(MOE_CHUNK == 4 * NW, "one token per 16-lane row of every wave");
  __shared__ int cnt[MOE_MAX_E];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, i = lane & 15;
  for (int e = threadIdx.x; e < E; e += TOPK_THREADS) cnt[e] = 0;
  __syncthreads();
  const int c0 = blockIdx.x * MOE_CHUNK, c1 = min(tokens, c0 + MOE_CHUNK);
  const int t = c0 + 4 * w + (lane >> 4);
  const bool live = t < c1;
  const float* row = logits + (long)(live ? t : c0) * E;   // c0 < tokens: a row that exists
  float v[EPR];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < EPR; ++j) {
    const int e = i + 16 * j;
    v[j] = e < E ? row[e] : -INFINITY;
    m = fmaxf(m, v[j]);
  }
  m = fmaxf(m, __uint_as_float(dpp_partner<0>(__float_as_uint(m))));
  m = fmaxf(m, __uint_as_float(dpp_partner<1>(__float_as_uint(m))));
  m = fmaxf(m, __uint_as_float(dpp_partner<2>(__float_as_uint(m))));
  m = fmaxf(m, __uint_as_float(dpp_partner<3>(__float_as_uint(m))));
  float z = 0.f;
#pragma unroll
  for (int j = 0; j < EPR; ++j)
    if (i + 16 * j < E) z += expf(v[j] - m);
  z += __uint_as_float(dpp_partner<0>(__float_as_uint(z)));
  z += __uint_as_float(dpp_partner<1>(__float_as_uint(z)));
  z += __uint_as_float(dpp_partner<2>(__float_as_uint(z)));
  z += __uint_as_float(dpp_partner<3>(__float_as_uint(z)));
  unsigned long long key[EPR];                   // 0: absent or already chosen
#pragma unroll
  for (int j = 0; j < EPR; ++j) key[j] = i + 16 * j < E ? cand_key(v[j], i + 16 * j) : 0ull;
  for (int j = 0; j < k; ++j) {
    unsigned long long best = key[0];
#pragma unroll
    for (int q = 1; q < EPR; ++q) best = umax64(best, key[q]);
    best = key_step<0>(best);
    best = key_step<1>(best);
    best = key_step<2>(best);
    best = key_step<3>(best);
#pragma unroll
    for (int q = 0; q < EPR; ++q) key[q] = key[q] == best ? 0ull : key[q];   // ids are unique
    if (i == 0 && live) {
      const int bi = key_id(best);
      experts[(long)t * k + j] = bi;
      gates[(long)t * k + j] = expf(key_logit(best) - m) / z;
      atomicAdd(&cnt[bi], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += TOPK_THREADS) counts[(long)blockIdx.x * E + e] = cnt[e];
}

// Expert blockIdx.x: base[c][e] = Σ_{c' < c} counts[c'][e] (exclusive over the chunks), total[e].
__global__ __launch_bounds__(256) void moe_scan_kernel(int chunks, int E, const int* __restrict__ counts,
                                                       int* __restrict__ base, int* __restrict__ total) {
  __shared__ int pre[256];
  const int e = blockIdx.x;
  const int per = (chunks + 255) / 256;
  const int c0 = min(chunks, threadIdx.x * per), c1 = min(chunks, c0 + per);
  int sum = 0;
  for (int c = c0; c < c1; ++c) sum += counts[(long)c * E + e];
  pre[threadIdx.x] = sum;
  __syncthreads();
  for (int s = 1; s < 256; s <<= 1) {
    const int add = threadIdx.x >= s ? pre[threadIdx.x - s] : 0;
    __syncthreads();
    pre[threadIdx.x] += add;
    __syncthreads();
  }
  int acc = pre[threadIdx.x] - sum;
  for (int c = c0; c < c1; ++c) {
    base[(long)c * E + e] = acc;
    acc += counts[(long)c * E + e];
  }
  if (threadIdx.x == 255) total[e] = pre[255];
}

__global__ __launch_bounds__(512) void moe_scatter_kernel(int tokens, int k, const int* __restrict__ experts,
                                                          const int* __restrict__ base,
                                                          const int* __restrict__ total, int E,
                                                          int* __restrict__ offsets, int* __restrict__ row_token,
                                                          int* __restrict__ token_row) {
  __shared__ int cnts[9 * MOE_MAX_E];            // per-expert counts: passes done, then 8 waves
  __shared__ int off[MOE_MAX_E];
  // the experts' offsets: exclusive prefix of the totals, two experts per thread then a thread scan
  {
    const int a = 2 * threadIdx.x, b = a + 1;
    const int va = a < E ? total[a] : 0, vb = b < E ? total[b] : 0;
    off[a] = va + vb;                              // scratch: pair sums, scanned in place below
    __syncthreads();
    int v = off[a];
    for (int s = 1; s < 512; s <<= 1) {
      const int add = threadIdx.x >= s ? off[2 * (threadIdx.x - s)] : 0;
      __syncthreads();
      v += add;
      off[a] = v;
      __syncthreads();
    }
    const int excl = v - va - vb;                  // rows before expert a
    __syncthreads();
    off[a] = excl;
    off[b] = excl + va;
    __syncthreads();
    if (blockIdx.x == 0) {
      if (a < E) offsets[a] = off[a];
      if (b < E) offsets[b] = off[b];
      if (threadIdx.x == 0) offsets[E] = off[E - 1] + total[E - 1];
    }
  }
  const int c0 = blockIdx.x * MOE_CHUNK, c1 = min(tokens, c0 + MOE_CHUNK);
  const int n = (c1 - c0) * k;                   // the chunk's entries, token-major
  const long first = (long)c0 * k;
  // An entry's rank among the chunk's earlier entries of its expert, in token order: pass p takes
  // entries [512p, 512p + 512) as eight waves of 64; within a wave each lane counts the earlier lanes
  // with its expert (readlane of every lane, no LDS), the waves' per-expert counts go to LDS (integer
  // adds: order-free), and an entry's rank is the count of earlier passes, then of earlier waves of
  // its pass, then of earlier lanes.
  int* seen = cnts;                              // per-expert count of the passes done so far
  int* wcnt = cnts + MOE_MAX_E;                  // [8 waves][E] counts of this pass
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += 512) seen[e] = 0;
  for (int p0 = 0; p0 < n; p0 += 512) {
    for (int q = threadIdx.x; q < 8 * E; q += 512) wcnt[q] = 0;
    __syncthreads();
    const int i = p0 + threadIdx.x;
    const int e = i < n ? experts[first + i] : -1;
    int lrank = 0;
    for (int q = 0; q < 64; ++q) {
      const int eq = __builtin_amdgcn_readlane(e, q);
      lrank += (q < lane && eq == e) ? 1 : 0;
    }
    if (e >= 0) atomicAdd(&wcnt[w * E + e], 1);
    __syncthreads();
    int rank = 0;
    if (e >= 0) {
      rank = seen[e] + lrank;
      for (int v = 0; v < w; ++v) rank += wcnt[v * E + e];
      const int row = off[e] + base[(long)blockIdx.x * E + e] + rank;
      row_token[row] = c0 + i / k;
      token_row[first + i] = row;
    }
    __syncthreads();
    for (int e2 = threadIdx.x; e2 < E; e2 += 512) {
      int add = 0;
      for (int v = 0; v < 8; ++v) add += wcnt[v * E + e2];
      seen[e2] += add;
    }
  }
}

__global__ __launch_bounds__(1024) void moe_zero_offsets_kernel(int E, int* __restrict__ offsets) {
  for (int e = threadIdx.x; e <= E; e += 1024) offsets[e] = 0;
}

// V consecutive elements at p as fp32 (V = 8: bf16 16-byte vector, 4: fp32 vector, 1: scalar).
template <typename T, int V>
__device__ __forceinline__ void load_v(const T* p, float (&v)[V]) {
  if constexpr (V == 8) {
    const bf16x8 x = *(const bf16x8*)p;
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = (float)x[q];
  } else if constexpr (V == 4) {
    const f32x4 x = *(const f32x4*)p;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = x[q];
  } else {
    v[0] = to_f32(*p);
  }
}

template <typename T, int V>
__device__ __forceinline__ void store_v(T* p, const float (&v)[V]) {
  if constexpr (V == 8) {
    bf16x8 x;
#pragma unroll
    for (int q = 0; q < 8; ++q) x[q] = (bf16)v[q];
    *(bf16x8*)p = x;
  } else if constexpr (V == 4) {
    *(f32x4*)p = (f32x4){v[0], v[1], v[2], v[3]};
  } else {
    *p = from_f32<T>(v[0]);
  }
}

template <typename T, int V>
// The same as a streaming store (the line is not kept for reuse).
__device__ __forceinline__ void store_v_nt(T* p, const float (&v)[V]) {
  if constexpr (V == 8) {
    bf16x8 x;
#pragma unroll
    for (int q = 0; q < 8; ++q) x[q] = (bf16)v[q];
    __builtin_nontemporal_store(x, (bf16x8*)p);
  } else if constexpr (V == 4) {
    __builtin_nontemporal_store((f32x4){v[0], v[1], v[2], v[3]}, (f32x4*)p);
  } else {
    __builtin_nontemporal_store(from_f32<T>(v[0]), p);
  }
}

// V elements at p as loaded (no conversion, so the load need not complete before the next is issued).
template <typename T, int V>
struct RawV {
  using type = typename std::conditional<V == 8, bf16x8, typename std::conditional<V == 4, f32x4, T>::type>::type;
  static __device__ __forceinline__ type load(const T* p) { return *(const type*)p; }
  // streaming load: the line is not kept for reuse
  static __device__ __forceinline__ type load_nt(const T* p) { return __builtin_nontemporal_load((const type*)p); }
  static __device__ __forceinline__ float at(const type& v, int q) {
    if constexpr (V == 1) return to_f32(v);
    else return (float)v[q];
  }
};

// Each thread keeps the loads of NB rows x CH column chunks in flight together; the rows are read and
// the output written with streaming accesses (each expert row is read exactly once, each output row
// written once): 4.6 -> 5.6 TB/s on the 128-expert shard.
template <typename T, int V>
__global__ __launch_bounds__(256) void moe_combine_kernel(int k, int H, const T* __restrict__ Z,
                                                          const float* __restrict__ gates,
                                                          const int* __restrict__ token_row, int rows,
                                                          T* __restrict__ out) {
  static_assert(V == 1 || (V == 8 && sizeof(T) == 2) || (V == 4 && sizeof(T) == 4), "vector width");
  constexpr int NB = 8;   // rows whose loads are in flight together
  constexpr int CH = 4;   // column chunks of 256·V elements per thread, loaded together
  using R = RawV<T, V>;
  const long t = blockIdx.x;
  if (rows <= 0) {   // nothing to combine: every row index is out of range
    const float zero[V] = {};
    for (int c = V * threadIdx.x; c < H; c += V * 256) store_v<T, V>(out + t * H + c, zero);
    return;
  }
  for (int c0 = V * threadIdx.x; c0 < H; c0 += V * 256 * CH) {
    float acc[CH][V];
#pragma unroll
    for (int h = 0; h < CH; ++h)
#pragma unroll
      for (int q = 0; q < V; ++q) acc[h][q] = 0.f;
    for (int j0 = 0; j0 < k; j0 += NB) {
      // the batch's loads first (a row outside [0, rows) or past k reads row 0, when there is one, and
      // is skipped; a chunk past H reloads the first), then the adds in row order: the same order of
      // addition as one row at a time
      bool ok[NB];
      float g[NB];
      long ro[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int j = j0 + i;
        const int r = j < k ? token_row[t * k + j] : -1;
        ok[i] = r >= 0 && r < rows;
        g[i] = j < k && gates ? gates[t * k + j] : 1.f;
        ro[i] = (long)(ok[i] ? r : 0) * H;   // row 0 exists (rows > 0)
      }
      typename R::type z[CH][NB];
#pragma unroll
      for (int h = 0; h < CH; ++h) {
        const int c = c0 + h * V * 256, cc = c < H ? c : c0;
#pragma unroll
        for (int i = 0; i < NB; ++i) z[h][i] = R::load_nt(Z + ro[i] + cc);
      }
#pragma unroll
      for (int h = 0; h < CH; ++h)
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          if (!ok[i]) continue;
#pragma unroll
          for (int q = 0; q < V; ++q) acc[h][q] += g[i] * R::at(z[h][i], q);
        }
    }
#pragma unroll
    for (int h = 0; h < CH; ++h) {
      const int c = c0 + h * V * 256;
      if (c < H) store_v_nt<T, V>(out + t * H + c, acc[h]);
    }
  }
}

template <typename T, int V>
__global__ __launch_bounds__(256) void moe_combine_bwd_kernel(int k, int H, const T* __restrict__ d_out,
                                                              const T* __restrict__ X, const T* __restrict__ Z,
                                                              const float* __restrict__ gates,
                                                              const int* __restrict__ token_row, int rows,
                                                              T* __restrict__ dZ, T* __restrict__ Xp,
                                                              float* __restrict__ dgates) {
  // The token's rows in batches of eight: per 16-byte piece of the row, d_out (and X) are read once
  // and the batch's Z pieces are in flight together; each row's gate-gradient partial accumulates
  // over the pieces in column order and is reduced across the workgroup once per batch, in the same
  // order as one row at a time.  A row outside [0, rows) (or past k) reads row 0, writes nothing and
  // gets a zero gate gradient.
  constexpr int NB = 8;
  using R = RawV<T, V>;
  __shared__ float red[4][NB];
  const long t = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int j0 = 0; j0 < k; j0 += NB) {
    int r[NB];
    bool ok[NB];
    float g[NB], dot[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int j = j0 + i;
      const int rr = j < k ? token_row[t * k + j] : -1;
      ok[i] = rr >= 0 && rr < rows;
      r[i] = ok[i] ? rr : 0;
      g[i] = j < k ? gates[t * k + j] : 0.f;
      dot[i] = 0.f;
    }
    if (rows > 0) {
      for (int c = V * threadIdx.x; c < H; c += V * 256) {
        float o[V], x[V];
        load_v<T, V>(d_out + t * H + c, o);
        typename R::type z[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) z[i] = R::load(Z + (long)r[i] * H + c);
        if (Xp) load_v<T, V>(X + t * H + c, x);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          if (!ok[i]) continue;
          float dz[V];
#pragma unroll
          for (int q = 0; q < V; ++q) {
            dot[i] += o[q] * R::at(z[i], q);
            dz[q] = g[i] * o[q];
          }
          store_v<T, V>(dZ + (long)r[i] * H + c, dz);
          if (Xp) store_v<T, V>(Xp + (long)r[i] * H + c, x);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int sh = 32; sh >= 1; sh >>= 1) dot[i] += __shfl_xor(dot[i], sh, 64);
    if (lane == 0)
#pragma unroll
      for (int i = 0; i < NB; ++i) red[w][i] = dot[i];
    __syncthreads();
    if (threadIdx.x < NB && j0 + (int)threadIdx.x < k) {
      const int i = threadIdx.x;
      dgates[t * k + j0 + i] = ok[i] ? ((red[0][i] + red[1][i]) + red[2][i]) + red[3][i] : 0.f;
    }
    __syncthreads();
  }
}

constexpr int RBWD_TOKENS = 16;   // tokens (waves) per workgroup of the router backward

// The MoE backward without a materialised dZ (see launch_moe_experts_bwd).  Row r's gate: the gate of
// the (t, j) whose row it is (t = row_token[r], j the choice with token_row[t, j] = r; 0 when r has no
// such choice), one thread per row; then the gate-scaled copy Yg[r] = gate·Y[r] that dW2 = Ygᵀ·d_out
// takes, one thread per 8 elements of a row (V = 8) or per element.
__global__ __launch_bounds__(256) void moe_gate_rows_kernel(int tokens, int k, int rows, const float* __restrict__ gates,
                                                            const int* __restrict__ row_token,
                                                            const int* __restrict__ token_row,
                                                            float* __restrict__ gate_row) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int t = row_token[r];
  float gt = 0.f;
  if (t >= 0 && t < tokens)
    for (int j = 0; j < k; ++j)
      if (token_row[(long)t * k + j] == r) {
        gt = gates[(long)t * k + j];
        break;
      }
  gate_row[r] = gt;
}

template <typename T, int V>
__global__ __launch_bounds__(256) void moe_scale_rows_kernel(int rows, int Fr, const float* __restrict__ gate_row,
                                                             const T* __restrict__ Y, T* __restrict__ Yg) {
  const int per = (Fr + V - 1) / V;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)rows * per) return;
  const int r = (int)(i / per), c = (int)(i % per) * V;
  const float gt = gate_row[r];
  const T* y = Y + (long)r * Fr + c;
  T* o = Yg + (long)r * Fr + c;
  if constexpr (V == 8) {
    const bf16x8 v = *(const bf16x8*)y;
    bf16x8 w;
    for (int e = 0; e < 8; ++e) w[e] = (bf16)(gt * (float)v[e]);
    *(bf16x8*)o = w;
  } else {
    for (int e = 0; e < V && c + e < Fr; ++e) o[e] = from_f32<T>(gt * to_f32(y[e]));
  }
}

// dgates[t, j] = Σ_{nt < ntiles} row_dot[nt·rows + r] in that order, r = token_row[t, j]: the gate
// gradients ⟨d_out[t], Y[r]·W2[e]⟩ from the dA1 GEMM's per-n-tile row dots.  Only rows inside the
// experts' (sanitised, non-decreasing) offsets [off[0], off[groups]) have row dots; others give 0.
__global__ __launch_bounds__(256) void moe_dgates_kernel(long n, int rows, int ntiles, const float* __restrict__ row_dot,
                                                         const int* __restrict__ token_row, const int* __restrict__ off,
                                                         int groups, float* __restrict__ dgates) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int r = token_row[i];
  float v = 0.f;
  if (r >= 0 && r < rows && r >= off[0] && r < off[groups])
    for (int nt = 0; nt < ntiles; ++nt) v += row_dot[(long)nt * rows + r];
  dgates[i] = v;
}

template <int EPL>
__global__ __launch_bounds__(64 * RBWD_TOKENS) void moe_route_bwd_kernel(int tokens, int E, int k,
                                                                         const float* __restrict__ logits,
                                                                         const int* __restrict__ experts,
                                                                         const float* __restrict__ dgates,
                                                                         float* __restrict__ d_logits) {
  const int lane = threadIdx.x & 63;
  const long t = (long)blockIdx.x * RBWD_TOKENS + (threadIdx.x >> 6);
  if (t >= tokens) return;                   // whole waves leave; no workgroup barrier follows
  const float* row = logits + t * E;
  float v[EPL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -INFINITY;
    m = fmaxf(m, v[i]);
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) m = fmaxf(m, __shfl_xor(m, sh, 64));
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    v[i] = (lane + 64 * i) < E ? expf(v[i] - m) : 0.f;
    z += v[i];
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) z += __shfl_xor(z, sh, 64);
  const float inv = 1.f / z;
  // lane j < k holds the j-th choice and its gate gradient; s = Σ_j dg_j·p_{i_j}
  const int my_e = lane < k ? experts[t * k + lane] : -1;
  const float my_g = lane < k ? dgates[t * k + lane] : 0.f;
  float sj = (my_e >= 0 && my_e < E) ? my_g * (expf(row[my_e] - m) * inv) : 0.f;
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) sj += __shfl_xor(sj, sh, 64);
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    float dg = 0.f;
    for (int j = 0; j < k; ++j) {
      const int ej = __shfl(my_e, j, 64);
      const float gj = __shfl(my_g, j, 64);
      if (ej == e) dg = gj;
    }
    if (e < E) d_logits[t * E + e] = v[i] * inv * (dg - sj);
  }
}

// The same gradient with one token per 16-lane row (four per wave), for E <= 256: entries i + 16q
// of the row in lane i, the row's max and Σ exp through the four row-local DPP steps, and every lane
// reading the token's k choices itself (the same addresses across the row).  Rows past `tokens`
// compute nothing and write nothing.
template <int EPR>
__global__ __launch_bounds__(256) void moe_route_bwd_rows_kernel(int tokens, int E, int k,
                                                                 const float* __restrict__ logits,
                                                                 const int* __restrict__ experts,
                                                                 const float* __restrict__ dgates,
                                                                 float* __restrict__ d_logits) {
  const int lane = threadIdx.x & 63, i = lane & 15;
  const long t = (long)blockIdx.x * 16 + (threadIdx.x >> 4);   // 16 tokens per 256-thread workgroup
  const bool live = t < tokens;
  const float* row = logits + (live ? t : 0) * E;               // tokens >= 1: a row that exists
  float v[EPR];
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < EPR; ++q) {
    const int e = i + 16 * q;
    v[q] = e < E ? row[e] : -INFINITY;
    m = fmaxf(m, v[q]);
  }
  m = fmaxf(m, __uint_as_float(dpp_partner<0>(__float_as_uint(m))));
  m = fmaxf(m, __uint_as_float(dpp_partner<1>(__float_as_uint(m))));
  m = fmaxf(m, __uint_as_float(dpp_partner<2>(__float_as_uint(m))));
  m = fmaxf(m, __uint_as_float(dpp_partner<3>(__float_as_uint(m))));
  float z = 0.f;
#pragma unroll
  for (int q = 0; q < EPR; ++q) {
    v[q] = (i + 16 * q) < E ? expf(v[q] - m) : 0.f;
    z += v[q];
  }
  z += __uint_as_float(dpp_partner<0>(__float_as_uint(z)));
  z += __uint_as_float(dpp_partner<1>(__float_as_uint(z)));
  z += __uint_as_float(dpp_partner<2>(__float_as_uint(z)));
  z += __uint_as_float(dpp_partner<3>(__float_as_uint(z)));
  const float inv = 1.f / z;
  if (!live) return;                           // no barrier follows
  // s = Σ_j dg_j·p_{i_j}, and each entry's own gate gradient (0 if not chosen)
  float sj = 0.f, dg[EPR];
#pragma unroll
  for (int q = 0; q < EPR; ++q) dg[q] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int ej = experts[t * k + j];
    const float gj = dgates[t * k + j];
    if (ej >= 0 && ej < E) sj += gj * (expf(row[ej] - m) * inv);
#pragma unroll
    for (int q = 0; q < EPR; ++q) dg[q] = ej == i + 16 * q ? gj : dg[q];
  }
#pragma unroll
  for (int q = 0; q < EPR; ++q) {
    const int e = i + 16 * q;
    if (e < E) d_logits[t * E + e] = v[q] * inv * (dg[q] - sj);
  }
}

template <int EPL>
hipError_t route_bwd_t(int tokens, int E, int k, const float* logits, const int* experts, const float* dgates,
                       float* d_logits, hipStream_t s) {
  const int blocks = (tokens + RBWD_TOKENS - 1) / RBWD_TOKENS;
  moe_route_bwd_kernel<EPL><<<blocks, 64 * RBWD_TOKENS, 0, s>>>(tokens, E, k, logits, experts, dgates, d_logits);
  return hipGetLastError();
}
template <int EPR>
hipError_t route_bwd_rows_t(int tokens, int E, int k, const float* logits, const int* experts, const float* dgates,
                            float* d_logits, hipStream_t s) {
  moe_route_bwd_rows_kernel<EPR><<<(tokens + 15) / 16, 256, 0, s>>>(tokens, E, k, logits, experts, dgates, d_logits);
  return hipGetLastError();
}

template <int EPL>
hipError_t topk_t(int tokens, int E, int k, const float* logits, float* gates, int* experts, int* counts,
                  hipStream_t s) {
  moe_topk_kernel<EPL><<<(tokens + MOE_CHUNK - 1) / MOE_CHUNK, TOPK_THREADS, 0, s>>>(tokens, E, k, logits, gates,
                                                                                     experts, counts);
  return hipGetLastError();
}
template <int EPR>
hipError_t topk_rows_t(int tokens, int E, int k, const float* logits, float* gates, int* experts, int* counts,
                       hipStream_t s) {
  moe_topk_rows_kernel<EPR><<<(tokens + MOE_CHUNK - 1) / MOE_CHUNK, TOPK_THREADS, 0, s>>>(tokens, E, k, logits,
                                                                                          gates, experts, counts);
  return hipGetLastError();
}

}  // namespace

int moe_max_experts() { return MOE_MAX_E; }
int moe_max_top_k() { return MOE_MAX_K; }

size_t moe_route_ws_bytes(int tokens, int E) {
  const size_t chunks = (size_t)((tokens + MOE_CHUNK - 1) / MOE_CHUNK);
  return (2 * chunks + 1) * (size_t)E * sizeof(int);
}

hipError_t launch_moe_route(int tokens, int E, int k, const float* logits, float* gates, int* expert_idx,
                            int* group_offsets, int* row_token, int* token_row, int* ws, hipStream_t s) {
  if (E < 1 || E > MOE_MAX_E || k < 1 || k > MOE_MAX_K || k > E || tokens < 0) return hipErrorInvalidValue;
  const int chunks = (tokens + MOE_CHUNK - 1) / MOE_CHUNK;
  int* counts = ws;
  int* base = ws + (size_t)chunks * E;
  int* total = base + (size_t)chunks * E;
  const double n = (double)tokens * k;
  if (tokens > 0) {
    ProfScope p("moe_topk", s, 4.0 * tokens * E, 4.0 * tokens * E + 8.0 * n + 4.0 * chunks * E);
    hipError_t e;
    if (E <= 32) e = topk_rows_t<2>(tokens, E, k, logits, gates, expert_idx, counts, s);
    else if (E <= 64) e = topk_rows_t<4>(tokens, E, k, logits, gates, expert_idx, counts, s);
    else if (E <= 128) e = topk_rows_t<8>(tokens, E, k, logits, gates, expert_idx, counts, s);
    else if (E <= 256) e = topk_rows_t<16>(tokens, E, k, logits, gates, expert_idx, counts, s);
    else if (E <= 512) e = topk_t<8>(tokens, E, k, logits, gates, expert_idx, counts, s);
    else e = topk_t<16>(tokens, E, k, logits, gates, expert_idx, counts, s);
    if (e != hipSuccess) return e;
  }
  if (tokens == 0) {                             // no chunks: every group is empty
    ProfScope p("moe_scan", s, 0.0, 4.0 * (E + 1));
    moe_zero_offsets_kernel<<<1, 1024, 0, s>>>(E, group_offsets);
    return hipGetLastError();
  }
  {
    ProfScope p("moe_scan", s, 0.0, 12.0 * chunks * E);
    moe_scan_kernel<<<E, 256, 0, s>>>(chunks, E, counts, base, total);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ProfScope p("moe_scatter", s, 0.0, 4.0 * n + 4.0 * chunks * E + 8.0 * n);
  moe_scatter_kernel<<<chunks, 512, 0, s>>>(tokens, k, expert_idx, base, total, E, group_offsets, row_token,
                                            token_row);
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

hipError_t launch_moe_combine_bwd(int dtype, int tokens, int k, int H, const void* d_out, const void* X,
                                  const void* Z, const float* gates, const int* token_row, int rows, void* dZ,
                                  void* Xp, float* dgates, hipStream_t s) {
  if (tokens <= 0) return hipSuccess;
  const double es = dtype == DT_BF16 ? 2.0 : 4.0;
  const double n = (double)tokens * k;
  ProfScope p(Xp ? "moe_combine_bwd<dispatch X>" : "moe_combine_bwd", s, 2.0 * n * H,
              es * ((double)tokens * H * (Xp ? 2.0 : 1.0) + n * H * (Xp ? 3.0 : 2.0)) + 12.0 * n);
  if (dtype == DT_BF16) {
    if (H % 8 == 0)
      moe_combine_bwd_kernel<bf16, 8><<<tokens, 256, 0, s>>>(k, H, (const bf16*)d_out, (const bf16*)X, (const bf16*)Z,
                                                              gates, token_row, rows, (bf16*)dZ, (bf16*)Xp, dgates);
    else
      moe_combine_bwd_kernel<bf16, 1><<<tokens, 256, 0, s>>>(k, H, (const bf16*)d_out, (const bf16*)X, (const bf16*)Z,
                                                              gates, token_row, rows, (bf16*)dZ, (bf16*)Xp, dgates);
  } else {
    if (H % 4 == 0)
      moe_combine_bwd_kernel<float, 4><<<tokens, 256, 0, s>>>(k, H, (const float*)d_out, (const float*)X,
                                                               (const float*)Z, gates, token_row, rows, (float*)dZ,
                                                               (float*)Xp, dgates);
    else
      moe_combine_bwd_kernel<float, 1><<<tokens, 256, 0, s>>>(k, H, (const float*)d_out, (const float*)X,
                                                               (const float*)Z, gates, token_row, rows, (float*)dZ,
                                                               (float*)Xp, dgates);
  }
  return hipGetLastError();
}

hipError_t launch_moe_route_bwd(int tokens, int E, int k, const float* logits, const int* experts,
                                const float* dgates, float* d_logits, hipStream_t s) {
  if (E < 1 || E > MOE_MAX_E || k < 1 || k > MOE_MAX_K || k > E || tokens < 0) return hipErrorInvalidValue;
  if (tokens == 0) return hipSuccess;
  ProfScope p("moe_route_bwd", s, 6.0 * tokens * E, 8.0 * tokens * E + 8.0 * tokens * k);
  if (E <= 32) return route_bwd_rows_t<2>(tokens, E, k, logits, experts, dgates, d_logits, s);
  if (E <= 64) return route_bwd_rows_t<4>(tokens, E, k, logits, experts, dgates, d_logits, s);
  if (E <= 128) return route_bwd_rows_t<8>(tokens, E, k, logits, experts, dgates, d_logits, s);
  if (E <= 256) return route_bwd_rows_t<16>(tokens, E, k, logits, experts, dgates, d_logits, s);
  if (E <= 512) return route_bwd_t<8>(tokens, E, k, logits, experts, dgates, d_logits, s);
  return route_bwd_t<16>(tokens, E, k, logits, experts, dgates, d_logits, s);
}

hipError_t launch_moe_row_gates(int dtype, int tokens, int k, int rows, int Fr, const float* gates,
                                const int* row_token, const int* token_row, const void* Y, float* gate_row, void* Yg,
                                hipStream_t s) {
  if (rows <= 0 || Fr <= 0) return hipSuccess;
  const double es = dtype == DT_BF16 ? 2.0 : 4.0;
  ProfScope p("moe_row_gates", s, (double)rows * Fr, 2.0 * es * rows * Fr + 8.0 * rows + 4.0 * rows * k);
  moe_gate_rows_kernel<<<(unsigned)((rows + 255) / 256), 256, 0, s>>>(tokens, k, rows, gates, row_token, token_row,
                                                                      gate_row);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dtype == DT_BF16 && Fr % 8 == 0 && ((((uintptr_t)Y) | ((uintptr_t)Yg)) & 15) == 0) {
    const long n = (long)rows * (Fr / 8);
    moe_scale_rows_kernel<bf16, 8><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(rows, Fr, gate_row, (const bf16*)Y,
                                                                              (bf16*)Yg);
  } else if (dtype == DT_BF16) {
    const long n = (long)rows * Fr;
    moe_scale_rows_kernel<bf16, 1><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(rows, Fr, gate_row, (const bf16*)Y,
                                                                              (bf16*)Yg);
  } else {
    const long n = (long)rows * Fr;
    moe_scale_rows_kernel<float, 1><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(rows, Fr, gate_row, (const float*)Y,
                                                                               (float*)Yg);
  }
  return hipGetLastError();
}

hipError_t launch_moe_dgates(int tokens, int k, int rows, int ntiles, const float* row_dot, const int* token_row,
                             const int* off, int groups, float* dgates, hipStream_t s) {
  const long n = (long)tokens * k;
  if (n <= 0) return hipSuccess;
  ProfScope p("moe_dgates", s, (double)n * ntiles, 4.0 * n * (ntiles + 2));
  moe_dgates_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(n, rows, ntiles, row_dot, token_row, off, groups,
                                                                dgates);
  return hipGetLastError();
}

}  // namespace tp
