// Grouped expert MLP shard: each expert's rows of the expert-sorted token matrix go through that
// expert's fc1 column shard (bias + GeLU fused) and its fc2 row shard.
//
// The row offsets live on the device (routing happened there), so the host never sees the group
// sizes.  A one-workgroup plan kernel sanitises the offsets (clamped to [0, rows], made
// non-decreasing by a running maximum, so no later access can leave the buffers) and numbers the
// row tiles of all experts for each of the two GEMMs' tile heights (prefix[e] = Σ_{j<e}
// ceil(rows_j / BM)), all with parallel scans; the
// grouped GEMM kernels launch an upper bound of ceil(rows / BM) + groups m-tiles and find their
// expert by binary search in prefix[].
#include <cstring>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace tp {

hipError_t launch_gemm_bf16_grouped(const GemmDesc& d, const int* off, const int* prefix, const int* tile_expert,
                                    int groups, long b_stride, long bias_stride, int max_mtiles, hipStream_t s);
hipError_t launch_gemm_generic_grouped(const GemmDesc& d, const int* off, const int* prefix, const int* tile_expert,
                                       int groups, long b_stride, long bias_stride, int max_mtiles, hipStream_t s);
int gemm_bf16_grouped_bm(int K);
int gemm_bf16_grouped_bn(const GemmDesc& d);
int gemm_generic_grouped_bm();
int gemm_generic_grouped_bn();
bool gemm_bf16_eligible(const GemmDesc& d);
bool gemm_bf16_grouped_k_eligible(const GemmDesc& d);
hipError_t launch_gemm_bf16_grouped_k(const GemmDesc& d, const int* off, int groups, long c_stride, hipStream_t s);
hipError_t launch_gemm_generic_grouped_k(const GemmDesc& d, const int* off, int groups, long c_stride, hipStream_t s);

namespace {

constexpr int PLAN_T = 1024;   // threads of the plan kernel: groups handled per pass

// Inclusive scan over the workgroup's threads, fixed order (Hillis-Steele in LDS).
template <typename Op>
__device__ __forceinline__ int block_scan(int v, int* sh, Op op) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int s = 1; s < PLAN_T; s <<= 1) {
    const bool has = threadIdx.x >= s;          // threads below the stride keep their value
    const int o = has ? sh[threadIdx.x - s] : 0;
    __syncthreads();
    if (has) v = op(v, o);
    sh[threadIdx.x] = v;
    __syncthreads();
  }
  return v;
}

// off_out[i] = max(off_out[i-1], min(off_in[i], rows)) with off_out[0] = clamp(off_in[0], 0, rows):
// a running maximum, so the clamped offsets come from one max-scan; the m-tile counts of the
// groups then from two sum-scans.  Groups go PLAN_T at a time, carrying the last values.  Each
// group also writes its number into tiles1 / tiles2 at its m-tiles [prefix[i], prefix[i+1]) (at
// most cap of them, cap >= ceil(rows / bm) + groups), so a GEMM workgroup finds its expert with
// one load instead of a binary search over the prefix.
__global__ __launch_bounds__(PLAN_T) void grouped_plan_kernel(const int* __restrict__ off_in, int groups,
                                                              int rows, int bm1, int bm2,
                                                              int* __restrict__ off_out,
                                                              int* __restrict__ prefix1,
                                                              int* __restrict__ prefix2,
                                                              int* __restrict__ tiles1,
                                                              int* __restrict__ tiles2, int cap) {
  __shared__ int sh[PLAN_T];
  int carry_o = min(max(off_in[0], 0), rows), carry_1 = 0, carry_2 = 0;
  if (threadIdx.x == 0) {
    off_out[0] = carry_o;
    prefix1[0] = 0;
    prefix2[0] = 0;
  }
  for (int c0 = 0; c0 < groups; c0 += PLAN_T) {
    const int i = c0 + threadIdx.x;
    const bool in = i < groups;
    const int b = in ? max(min(off_in[i + 1], rows), carry_o) : carry_o;
    const int o = block_scan(b, sh, [](int x, int y) { return max(x, y); });
    const int prev = threadIdx.x > 0 ? sh[threadIdx.x - 1] : carry_o;   // sh holds the max-scan
    __syncthreads();
    const int n = in ? o - prev : 0;
    const int p1 = block_scan((n + bm1 - 1) / bm1, sh, [](int x, int y) { return x + y; });
    const int t1 = sh[PLAN_T - 1];
    __syncthreads();
    const int p2 = block_scan((n + bm2 - 1) / bm2, sh, [](int x, int y) { return x + y; });
    const int t2 = sh[PLAN_T - 1];
    __syncthreads();
    if (in) {
      off_out[i + 1] = o;
      prefix1[i + 1] = carry_1 + p1;
      prefix2[i + 1] = carry_2 + p2;
      for (int t = carry_1 + p1 - (n + bm1 - 1) / bm1; t < min(carry_1 + p1, cap); ++t) tiles1[t] = i;
      for (int t = carry_2 + p2 - (n + bm2 - 1) / bm2; t < min(carry_2 + p2, cap); ++t) tiles2[t] = i;
    }
    carry_1 += t1;
    carry_2 += t2;
    // the last group's offset of this pass (threads past `groups` repeat it)
    sh[threadIdx.x] = o;
    __syncthreads();
    carry_o = sh[PLAN_T - 1];
    __syncthreads();
  }
}

// db[e][c] = Σ_{r in [off[e], off[e+1])} dA[r·cols + c]: a workgroup per (expert, 64 columns); four
// row phases of 64 threads each sum every fourth row (eight loads in flight per thread), then the
// four partials are added in phase order, so the result does not depend on timing.
template <typename T>
__global__ __launch_bounds__(256) void grouped_colsum_kernel(const T* __restrict__ dA, int cols,
                                                             const int* __restrict__ off, T* __restrict__ db) {
  __shared__ float part[4][64];
  const int e = blockIdx.y, lane = threadIdx.x & 63, ph = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  const int r0 = off[e], r1 = off[e + 1];
  float acc = 0.f;
  if (c < cols) {
#pragma unroll 8
    for (int r = r0 + ph; r < r1; r += 4) acc += to_f32(dA[(long)r * cols + c]);
  }
  part[ph][lane] = acc;
  __syncthreads();
  if (ph == 0 && c < cols)
    db[(long)e * cols + c] = from_f32<T>(((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane]);
}

// The same sums with 16-byte loads, for rows whose width is a multiple of the vector (V = 8 bf16 or
// 4 fp32): a workgroup of 1024 threads per (expert, 8·V columns); thread (phase ph < 128, vector
// q < 8) sums the columns of vector q over rows r0 + ph, r0 + ph + 128, ... (a few rows each, all
// loads in flight at once); then one thread per column adds the 128 phases in order, so the result
// does not depend on timing.
template <typename T, int V>
__global__ __launch_bounds__(1024) void grouped_colsum_vec_kernel(const T* __restrict__ dA, int cols,
                                                                  const int* __restrict__ off, T* __restrict__ db) {
  using Vec = typename std::conditional<V == 8, bf16x8, f32x4>::type;
  constexpr int NC = 8 * V, NP = 128;            // columns per workgroup, row phases
  __shared__ float part[NP][NC + 1];
  const int e = blockIdx.y, q = threadIdx.x & 7, ph = threadIdx.x >> 3;
  const int c = blockIdx.x * NC + q * V;
  const int r0 = off[e], r1 = off[e + 1];
  float acc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) acc[j] = 0.f;
  if (c < cols) {
#pragma unroll 8
    for (int r = r0 + ph; r < r1; r += NP) {
      const Vec x = *(const Vec*)(dA + (long)r * cols + c);
#pragma unroll
      for (int j = 0; j < V; ++j) acc[j] += (float)x[j];
    }
  }
#pragma unroll
  for (int j = 0; j < V; ++j) part[ph][q * V + j] = acc[j];
  __syncthreads();
  if (threadIdx.x < NC && blockIdx.x * NC + threadIdx.x < cols) {
    float t = part[0][threadIdx.x];
    for (int p = 1; p < NP; ++p) t += part[p][threadIdx.x];
    db[(long)e * cols + blockIdx.x * NC + threadIdx.x] = from_f32<T>(t);
  }
}

}  // namespace

// The plan: the sanitised offsets and the two m-tile prefixes ([groups + 1] each), then the two
// m-tile -> group tables (ceil(rows / 64) + groups entries each: every tile height is at least 64).
static long plan_cap(int groups, int rows) { return (long)(rows + 63) / 64 + groups; }
size_t grouped_ws_bytes(int groups, int rows) {
  return (size_t)(3 * ((long)groups + 1) + 2 * plan_cap(groups, rows)) * sizeof(int);
}

// Lays out the plan in ws and launches the plan kernel.
static hipError_t run_plan(const int* off, int groups, int rows, int bm1, int bm2, void* ws, int** off_s,
                           int** prefix1, int** prefix2, int** tiles1, int** tiles2, hipStream_t s) {
  const long cap = plan_cap(groups, rows);
  if (cap > 0x7fffffffL) return hipErrorInvalidValue;
  *off_s = (int*)ws;
  *prefix1 = *off_s + (groups + 1);    // m-tiles of the first GEMM's tile height
  *prefix2 = *prefix1 + (groups + 1);  // m-tiles of the second's
  *tiles1 = *prefix2 + (groups + 1);
  *tiles2 = *tiles1 + cap;
  ProfScope p("grouped_plan", s, 0.0, 12.0 * (groups + 1) + 4.0 * cap);
  grouped_plan_kernel<<<1, PLAN_T, 0, s>>>(off, groups, rows, bm1, bm2, *off_s, *prefix1, *prefix2, *tiles1,
                                           *tiles2, (int)cap);
  return hipGetLastError();
}

// fc1 then fc2 of the groups [0, groups) of a plan, on s.
static hipError_t grouped_pair(bool tiled, const GemmDesc& fc1, const GemmDesc& fc2, const int* off_s,
                               const int* prefix1, const int* prefix2, const int* tiles1, const int* tiles2,
                               int groups, int maxmt1, int maxmt2, double f1, double by1, double by2,
                               hipStream_t s) {
  const int H = fc1.K, Fr = fc1.N;
  const bool gather = fc1.a_rows != nullptr;
  if (tiled) {
    {
      ProfScope p(gather ? "gemm_bf16_grouped<fc1, gather, bias+gelu>" : "gemm_bf16_grouped<fc1, bias+gelu>",
                  s, f1, by1);
      hipError_t e = launch_gemm_bf16_grouped(fc1, off_s, prefix1, tiles1, groups, (long)H * Fr, Fr, maxmt1, s);
      if (e != hipSuccess) return e;
    }
    ProfScope p("gemm_bf16_grouped<fc2>", s, f1, by2);
    return launch_gemm_bf16_grouped(fc2, off_s, prefix2, tiles2, groups, (long)Fr * H, 0, maxmt2, s);
  }
  {
    ProfScope p(gather ? "gemm_generic_grouped<fc1, gather, bias+gelu>" : "gemm_generic_grouped<fc1, bias+gelu>",
                s, f1, by1);
    hipError_t e = launch_gemm_generic_grouped(fc1, off_s, prefix1, tiles1, groups, (long)H * Fr, Fr, maxmt1, s);
    if (e != hipSuccess) return e;
  }
  ProfScope p("gemm_generic_grouped<fc2>", s, f1, by2);
  return launch_gemm_generic_grouped(fc2, off_s, prefix2, tiles2, groups, (long)Fr * H, 0, maxmt2, s);
}

size_t mlp_grouped_ws_bytes(int groups, int rows, bool split) {
  const size_t one = (grouped_ws_bytes(groups, rows) + 255) & ~(size_t)255;
  return split ? 2 * one : one;
}

hipError_t launch_mlp_grouped(int dtype, int groups, const int* off, int rows, int H, int Fr,
                              const void* X, const void* W1, const void* b1, const void* W2, void* Z,
                              void* A1, void* Y, void* ws, hipStream_t s, const int* row_token, int tokens,
                              hipStream_t s2, hipEvent_t ev_plan) {
  if (rows <= 0) return hipSuccess;
  int *off_s, *prefix1, *prefix2, *tiles1, *tiles2;   // plan (fc1's tile height, then fc2's)
  const size_t es = dtype == DT_BF16 ? 2 : 4;

  GemmDesc fc1;
  memset(&fc1, 0, sizeof(fc1));
  fc1.M = rows; fc1.N = Fr; fc1.K = H;
  fc1.A = X; fc1.lda = H; fc1.a_kmajor = true;
  fc1.B = W1; fc1.ldb = Fr; fc1.b_kmajor = false;
  fc1.C = Y; fc1.ldc = Fr; fc1.C2 = A1; fc1.bias = b1; fc1.epi = EPI_BIAS_GELU; fc1.dtype = dtype;
  GemmDesc fc2 = fc1;
  fc1.a_rows = row_token;          // nullptr: X is already in expert-sorted order
  fc1.a_rows_n = tokens;
  fc2.N = H; fc2.K = Fr;
  fc2.A = Y; fc2.lda = Fr;
  fc2.B = W2; fc2.ldb = H;
  fc2.C = Z; fc2.ldc = H; fc2.C2 = nullptr; fc2.bias = nullptr; fc2.epi = EPI_STORE;

  // Each expert's slice is a plain row-major problem with the same leading dimensions, so the tiled
  // kernel's alignment rules are those of the whole matrices.
  // (the tiled gather addresses X through one 32-bit buffer range: X must stay under 2 GiB)
  const bool tiled = gemm_bf16_eligible(fc1) && gemm_bf16_eligible(fc2) &&
                     (!row_token || (long)tokens * H * 2 <= 0x7fffffffL);
  const int bm1 = tiled ? gemm_bf16_grouped_bm(fc1.K) : gemm_generic_grouped_bm();
  const int bm2 = tiled ? gemm_bf16_grouped_bm(fc2.K) : gemm_generic_grouped_bm();
  const long maxmt1 = (long)(rows + bm1 - 1) / bm1 + groups, maxmt2 = (long)(rows + bm2 - 1) / bm2 + groups;
  if (maxmt1 > 0x7fffffffL || maxmt2 > 0x7fffffffL) return hipErrorInvalidValue;
  {
    hipError_t e = run_plan(off, groups, rows, bm1, bm2, ws, &off_s, &prefix1, &prefix2, &tiles1, &tiles2, s);
    if (e != hipSuccess) return e;
  }
  const double f1 = 2.0 * rows * (double)Fr * H;
  // unique bytes: a gathered fc1 reads each of X's `tokens` rows once (its k rows per token come
  // from the same lines), not the `rows` rows of a dispatched copy
  const double by1 = es * ((double)(row_token ? tokens : rows) * H + (double)groups * H * Fr +
                           (A1 ? 2.0 : 1.0) * rows * Fr) + (row_token ? 4.0 * rows : 0.0);
  const double by2 = es * ((double)rows * Fr + (double)groups * Fr * H + (double)rows * H);
  if (s2 == nullptr || s2 == s || groups < 2)
    return grouped_pair(tiled, fc1, fc2, off_s, prefix1, prefix2, tiles1, tiles2, groups, (int)maxmt1, (int)maxmt2,
                        f1, by1, by2, s);

  // Two halves of the groups: [0, h) on s with the plan above (its first h groups and their tiles
  // are a plan of their own), [h, groups) on s2 with a second plan over the sanitised offsets from
  // h on (already clamped and non-decreasing, so that plan keeps them as they are).  The halves'
  // rows, weights and outputs are disjoint; every element is computed as in one launch.  (The
  // figures handed to the per-launch timing are split evenly; the caller does not split while it
  // is on.)
  const int h = groups / 2;
  hipError_t e = hipEventRecord(ev_plan, s);
  if (e == hipSuccess) e = hipStreamWaitEvent(s2, ev_plan, 0);
  if (e != hipSuccess) return e;
  int *off_b, *prefix1_b, *prefix2_b, *tiles1_b, *tiles2_b;
  e = run_plan(off_s + h, groups - h, rows, bm1, bm2, (char*)ws + mlp_grouped_ws_bytes(groups, rows, false),
               &off_b, &prefix1_b, &prefix2_b, &tiles1_b, &tiles2_b, s2);
  if (e != hipSuccess) return e;
  GemmDesc fc1b = fc1, fc2b = fc2;
  fc1b.B = (const char*)W1 + (size_t)h * H * Fr * es;
  fc1b.bias = (const char*)b1 + (size_t)h * Fr * es;
  fc2b.B = (const char*)W2 + (size_t)h * Fr * H * es;
  e = grouped_pair(tiled, fc1, fc2, off_s, prefix1, prefix2, tiles1, tiles2, h, (int)maxmt1, (int)maxmt2,
                   f1 / 2, by1 / 2, by2 / 2, s);
  if (e != hipSuccess) return e;
  return grouped_pair(tiled, fc1b, fc2b, off_b, prefix1_b, prefix2_b, tiles1_b, tiles2_b, groups - h, (int)maxmt1,
                      (int)maxmt2, f1 / 2, by1 / 2, by2 / 2, s2);
}

// Backward of launch_mlp_grouped on expert-sorted operands, expert by expert (rows [off[e], off[e+1])):
//   dA1 = (dZ·W2[e]ᵀ) ∘ GeLU'(A1)      grouped, rows split by expert, GeLU' in the epilogue
//   dW2[e] = Y_eᵀ·dZ_e                  grouped weight gradient, the expert's rows as k
//   db1[e] = Σ_rows dA1_e               segmented column sum
//   dW1[e] = X_eᵀ·dA1_e                 grouped weight gradient
//   dX = dA1·W1[e]ᵀ                     grouped, rows split by expert
// in that order on one stream, so dX may alias dZ (both reads of dZ come first).  An expert without
// rows gets zero weight and bias gradients.  With x_rows set, row r of the expert-sorted X is row
// x_rows[r] of the x_rows_n-row matrix at X, gathered inside dW1's operand loads.
// ws: grouped_ws_bytes(groups).
hipError_t launch_mlp_grouped_bwd(int dtype, int groups, const int* off, int rows, int H, int Fr, const void* X,
                                  const void* W1, const void* W2, const void* A1, const void* Y, const void* dZ,
                                  void* dA1, void* dX, void* dW1, void* db1, void* dW2, void* ws, hipStream_t s,
                                  const int* x_rows, int x_rows_n) {
  if (groups <= 0) return hipSuccess;
  if (groups > 65535) return hipErrorInvalidValue;   // the column sum's grid y (checked before any launch)
  int *off_s, *prefix1, *prefix2, *tiles1, *tiles2;   // plan (the dA1 GEMM's tile height, then dX's)
  const double es = dtype == DT_BF16 ? 2.0 : 4.0;

  GemmDesc ga;                                // dA1 = (dZ·W2ᵀ) ∘ GeLU'(A1)
  memset(&ga, 0, sizeof(ga));
  ga.M = rows; ga.N = Fr; ga.K = H; ga.dtype = dtype;
  ga.A = dZ; ga.lda = H; ga.a_kmajor = true;
  ga.B = W2; ga.ldb = H; ga.b_kmajor = true;
  ga.C = dA1; ga.ldc = Fr; ga.epi = EPI_DGELU; ga.aux = A1; ga.ld_aux = Fr;
  GemmDesc gx = ga;                           // dX = dA1·W1ᵀ
  gx.N = H; gx.K = Fr; gx.A = dA1; gx.lda = Fr; gx.B = W1; gx.ldb = Fr; gx.C = dX; gx.ldc = H;
  gx.epi = EPI_STORE; gx.aux = nullptr; gx.ld_aux = 0;
  GemmDesc gw2;                               // dW2[e] = Y_eᵀ·dZ_e   [Fr, H]
  memset(&gw2, 0, sizeof(gw2));
  gw2.M = Fr; gw2.N = H; gw2.dtype = dtype; gw2.epi = EPI_STORE;
  gw2.A = Y; gw2.lda = Fr; gw2.a_kmajor = false;
  gw2.B = dZ; gw2.ldb = H; gw2.b_kmajor = false;
  gw2.C = dW2; gw2.ldc = H;
  GemmDesc gw1 = gw2;                         // dW1[e] = X_eᵀ·dA1_e  [H, Fr]
  gw1.M = H; gw1.N = Fr; gw1.A = X; gw1.lda = H; gw1.B = dA1; gw1.ldb = Fr; gw1.C = dW1; gw1.ldc = Fr;
  gw1.a_rows = x_rows; gw1.a_rows_n = x_rows_n;

  const bool tiled = rows > 0 && gemm_bf16_eligible(ga) && gemm_bf16_eligible(gx);
  const int bm1 = tiled ? gemm_bf16_grouped_bm(ga.K) : gemm_generic_grouped_bm();
  const int bm2 = tiled ? gemm_bf16_grouped_bm(gx.K) : gemm_generic_grouped_bm();
  const long maxmt1 = (long)(rows + bm1 - 1) / bm1 + groups, maxmt2 = (long)(rows + bm2 - 1) / bm2 + groups;
  if (maxmt1 > 0x7fffffffL || maxmt2 > 0x7fffffffL) return hipErrorInvalidValue;
  {
    hipError_t e = run_plan(off, groups, rows, bm1, bm2, ws, &off_s, &prefix1, &prefix2, &tiles1, &tiles2, s);
    if (e != hipSuccess) return e;
  }
  const double fl = 2.0 * rows * (double)Fr * H;
  const double wts = es * (double)groups * H * Fr;
  hipError_t e;
  if (rows > 0) {
    ProfScope p(tiled ? "gemm_bf16_grouped<dZ.W2t, dgelu>" : "gemm_generic_grouped<dZ.W2t, dgelu>", s, fl,
                es * ((double)rows * H + 2.0 * rows * Fr) + wts);   // dZ and A1 read, dA1 written
    e = tiled ? launch_gemm_bf16_grouped(ga, off_s, prefix1, tiles1, groups, (long)Fr * H, 0, (int)maxmt1, s)
              : launch_gemm_generic_grouped(ga, off_s, prefix1, tiles1, groups, (long)Fr * H, 0, (int)maxmt1, s);
    if (e != hipSuccess) return e;
  }
  {
    const bool t2 = gemm_bf16_grouped_k_eligible(gw2);
    ProfScope p(t2 ? "gemm_bf16_grouped_k<Yt.dZ>" : "gemm_generic_grouped_k<Yt.dZ>", s, fl,
                es * ((double)rows * Fr + (double)rows * H) + wts);
    e = t2 ? launch_gemm_bf16_grouped_k(gw2, off_s, groups, (long)Fr * H, s)
           : launch_gemm_generic_grouped_k(gw2, off_s, groups, (long)Fr * H, s);
    if (e != hipSuccess) return e;
  }
  {
    ProfScope p("grouped_colsum", s, (double)rows * Fr, es * ((double)rows * Fr + (double)groups * Fr));
    if (dtype == DT_BF16 && Fr % 8 == 0)
      grouped_colsum_vec_kernel<bf16, 8><<<dim3((Fr + 63) / 64, groups), 1024, 0, s>>>((const bf16*)dA1, Fr, off_s,
                                                                                     (bf16*)db1);
    else if (dtype != DT_BF16 && Fr % 4 == 0)
      grouped_colsum_vec_kernel<float, 4><<<dim3((Fr + 31) / 32, groups), 1024, 0, s>>>((const float*)dA1, Fr, off_s,
                                                                                       (float*)db1);
    else if (dtype == DT_BF16)
      grouped_colsum_kernel<bf16><<<dim3((Fr + 63) / 64, groups), 256, 0, s>>>((const bf16*)dA1, Fr, off_s, (bf16*)db1);
    else
      grouped_colsum_kernel<float><<<dim3((Fr + 63) / 64, groups), 256, 0, s>>>((const float*)dA1, Fr, off_s,
                                                                                (float*)db1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const bool t1 = gemm_bf16_grouped_k_eligible(gw1);
    ProfScope p(t1 ? (x_rows ? "gemm_bf16_grouped_k<Xt.dA1, gather>" : "gemm_bf16_grouped_k<Xt.dA1>")
                   : (x_rows ? "gemm_generic_grouped_k<Xt.dA1, gather>" : "gemm_generic_grouped_k<Xt.dA1>"), s, fl,
                es * ((double)(x_rows ? x_rows_n : rows) * H + (double)rows * Fr) + wts);   // X's unique rows
    e = t1 ? launch_gemm_bf16_grouped_k(gw1, off_s, groups, (long)H * Fr, s)
           : launch_gemm_generic_grouped_k(gw1, off_s, groups, (long)H * Fr, s);
    if (e != hipSuccess) return e;
  }
  if (rows > 0) {
    ProfScope p(tiled ? "gemm_bf16_grouped<dA1.W1t>" : "gemm_generic_grouped<dA1.W1t>", s, fl,
                es * ((double)rows * Fr + (double)rows * H) + wts);
    e = tiled ? launch_gemm_bf16_grouped(gx, off_s, prefix2, tiles2, groups, (long)H * Fr, 0, (int)maxmt2, s)
              : launch_gemm_generic_grouped(gx, off_s, prefix2, tiles2, groups, (long)H * Fr, 0, (int)maxmt2, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The MoE experts' backward straight from the output gradient d_out [tokens, H] (no dZ [rows, H] in
// memory).  Row r of the expert-sorted matrix is (t, j) = (row_token[r], the choice with
// token_row[t, j] = r) with gate g_r, and dZ[r] = g_r·d_out[t]; since dZ is that row scaled, each of
// its uses takes d_out's row through the row gather and the scale where it is cheapest:
//   gate_row[r] = g_r,  Yg[r] = g_r·Y[r]                              (moe_row_gates)
//   dA1 = g_r·(d_out[t]·W2[e]ᵀ) ∘ GeLU'(A1)  and, from the same accumulators before the scale,
//   row_dot[nt, r] = Σ_{f in n-tile nt} Y[r, f]·(d_out[t]·W2[e]ᵀ)[f]   (the gated epilogue)
//   dgates[t, j] = Σ_nt row_dot[nt, r] = ⟨d_out[t], Y[r]·W2[e]⟩        (moe_dgates, fixed order)
//   dW2[e] = Σ_{r of e} Yg[r]ᵀ·d_out[t]                               (grouped over k, B's k rows gathered)
//   db1[e] = Σ_{r of e} dA1[r];  dW1[e] = Σ_{r of e} X[t]ᵀ·dA1[r];  dX_perm = dA1·W1[e]ᵀ
// The gate gradient is ⟨d_out[t], Z[r]⟩ with Z[r] = Y[r]·W2[e] not rounded to storage first.  Every
// sum has a fixed order (repeatable bit for bit).  ws: moe_experts_bwd_ws_bytes; dX_perm [rows, H].
size_t moe_experts_bwd_ws_bytes(int groups, int rows, int H, int Fr, int dtype) {
  (void)H;
  const size_t es = dtype == DT_BF16 ? 2 : 4;
  auto a256 = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t nt = (size_t)(Fr + 63) / 64;   // n-tiles of the narrowest tile (the generic kernel's)
  return a256(grouped_ws_bytes(groups, rows)) + a256((size_t)rows * Fr * es) + a256((size_t)rows * 4) +
         a256((size_t)rows * Fr * es) + a256(nt * rows * 4);
}

hipError_t launch_moe_experts_bwd(int dtype, int groups, const int* off, int tokens, int k, int rows, int H, int Fr,
                                  const void* X, const float* gates, const int* row_token, const int* token_row,
                                  const void* W1, const void* W2, const void* A1, const void* Y, const void* d_out,
                                  void* dX_perm, void* dW1, void* db1, void* dW2, float* dgates, void* ws,
                                  hipStream_t s, hipStream_t s2, hipEvent_t ev_gates, hipEvent_t ev_dA1) {
  if (groups <= 0) return hipSuccess;
  if (groups > 65535) return hipErrorInvalidValue;   // the column sum's grid y (checked before any launch)
  const bool side = s2 != s;
  const double es = dtype == DT_BF16 ? 2.0 : 4.0;
  auto a256 = [](size_t b) { return (b + 255) & ~(size_t)255; };
  char* w = (char*)ws;
  int *off_s, *prefix1, *prefix2, *tiles1, *tiles2;   // plan (the dA1 GEMM's tile height, then dX's)
  void* plan = w;
  w += a256(grouped_ws_bytes(groups, rows));
  void* dA1 = w;
  w += a256((size_t)rows * Fr * (size_t)es);
  float* gate_row = (float*)w;
  w += a256((size_t)rows * 4);
  void* Yg = w;
  w += a256((size_t)rows * Fr * (size_t)es);
  float* row_dot = (float*)w;

  GemmDesc ga;                                // dA1 = gate·(d_out[t]·W2ᵀ) ∘ GeLU'(A1), row dots with Y
  memset(&ga, 0, sizeof(ga));
  ga.M = rows; ga.N = Fr; ga.K = H; ga.dtype = dtype;
  ga.A = d_out; ga.lda = H; ga.a_kmajor = true; ga.a_rows = row_token; ga.a_rows_n = tokens;
  ga.B = W2; ga.ldb = H; ga.b_kmajor = true;
  ga.C = dA1; ga.ldc = Fr; ga.epi = EPI_DGELU_GATE; ga.aux = A1; ga.ld_aux = Fr;
  ga.aux2 = Y; ga.ld_aux2 = Fr; ga.row_scale = gate_row; ga.row_dot = row_dot; ga.rd_stride = rows;
  GemmDesc gx;                                // dX_perm = dA1·W1ᵀ
  memset(&gx, 0, sizeof(gx));
  gx.M = rows; gx.N = H; gx.K = Fr; gx.dtype = dtype; gx.epi = EPI_STORE;
  gx.A = dA1; gx.lda = Fr; gx.a_kmajor = true;
  gx.B = W1; gx.ldb = Fr; gx.b_kmajor = true;
  gx.C = dX_perm; gx.ldc = H;
  GemmDesc gw2;                               // dW2[e] = Yg_eᵀ·d_out[tokens of e]   [Fr, H]
  memset(&gw2, 0, sizeof(gw2));
  gw2.M = Fr; gw2.N = H; gw2.dtype = dtype; gw2.epi = EPI_STORE;
  gw2.A = Yg; gw2.lda = Fr; gw2.a_kmajor = false;
  gw2.B = d_out; gw2.ldb = H; gw2.b_kmajor = false; gw2.b_rows = row_token; gw2.b_rows_n = tokens;
  gw2.C = dW2; gw2.ldc = H;
  GemmDesc gw1 = gw2;                         // dW1[e] = X[tokens of e]ᵀ·dA1_e  [H, Fr]
  gw1.M = H; gw1.N = Fr; gw1.A = X; gw1.lda = H; gw1.a_rows = row_token; gw1.a_rows_n = tokens;
  gw1.B = dA1; gw1.ldb = Fr; gw1.b_rows = nullptr; gw1.b_rows_n = 0; gw1.C = dW1; gw1.ldc = Fr;

  // one 32-bit buffer range covers the gathered d_out in the tiled kernels
  const bool tiled = rows > 0 && gemm_bf16_eligible(ga) && gemm_bf16_eligible(gx) &&
                     (long)tokens * H * 2 <= 0x7fffffffL;
  const int bm1 = tiled ? gemm_bf16_grouped_bm(ga.K) : gemm_generic_grouped_bm();
  const int bm2 = tiled ? gemm_bf16_grouped_bm(gx.K) : gemm_generic_grouped_bm();
  const int bn1 = tiled ? gemm_bf16_grouped_bn(ga) : gemm_generic_grouped_bn();
  const int ntiles = (Fr + bn1 - 1) / bn1;    // <= (Fr + 63) / 64: row_dot's room
  const long maxmt1 = (long)(rows + bm1 - 1) / bm1 + groups, maxmt2 = (long)(rows + bm2 - 1) / bm2 + groups;
  if (maxmt1 > 0x7fffffffL || maxmt2 > 0x7fffffffL) return hipErrorInvalidValue;
  hipError_t e;
  e = run_plan(off, groups, rows, bm1, bm2, plan, &off_s, &prefix1, &prefix2, &tiles1, &tiles2, s);
  if (e != hipSuccess) return e;
  e = launch_moe_row_gates(dtype, tokens, k, rows, Fr, gates, row_token, token_row, Y, gate_row, Yg, s);
  if (e != hipSuccess) return e;
  const double fl = 2.0 * rows * (double)Fr * H;
  const double wts = es * (double)groups * H * Fr;
  // s: dA1, the gate gradients, db1, dX_perm;  s2 (when given): dW2 (after the plan and the row gates),
  // then dW1 (after dA1)
  if (side) {
    e = hipEventRecord(ev_gates, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(s2, ev_gates, 0);
    if (e != hipSuccess) return e;
  }
  if (rows > 0) {
    // d_out's unique rows, A1 and Y read, dA1 written, the row dots
    ProfScope p(tiled ? "gemm_bf16_grouped<dout.W2t, gather, gate+dgelu>" : "gemm_generic_grouped<dout.W2t, gather, gate+dgelu>",
                s, fl, es * ((double)tokens * H + 3.0 * rows * Fr) + wts + 4.0 * rows * (ntiles + 2));
    e = tiled ? launch_gemm_bf16_grouped(ga, off_s, prefix1, tiles1, groups, (long)Fr * H, 0, (int)maxmt1, s)
              : launch_gemm_generic_grouped(ga, off_s, prefix1, tiles1, groups, (long)Fr * H, 0, (int)maxmt1, s);
    if (e != hipSuccess) return e;
  }
  if (side) {
    e = hipEventRecord(ev_dA1, s);
    if (e != hipSuccess) return e;
  }
  {
    const bool t2 = gemm_bf16_grouped_k_eligible(gw2);
    ProfScope p(t2 ? "gemm_bf16_grouped_k<Ygt.dout, gather>" : "gemm_generic_grouped_k<Ygt.dout, gather>", s2, fl,
                es * ((double)rows * Fr + (double)tokens * H) + wts + 4.0 * rows);
    e = t2 ? launch_gemm_bf16_grouped_k(gw2, off_s, groups, (long)Fr * H, s2)
           : launch_gemm_generic_grouped_k(gw2, off_s, groups, (long)Fr * H, s2);
    if (e != hipSuccess) return e;
  }
  e = launch_moe_dgates(tokens, k, rows, ntiles, row_dot, token_row, off_s, groups, dgates, s);
  if (e != hipSuccess) return e;
  {
    ProfScope p("grouped_colsum", s, (double)rows * Fr, es * ((double)rows * Fr + (double)groups * Fr));
    if (dtype == DT_BF16 && Fr % 8 == 0)
      grouped_colsum_vec_kernel<bf16, 8><<<dim3((Fr + 63) / 64, groups), 1024, 0, s>>>((const bf16*)dA1, Fr, off_s,
                                                                                     (bf16*)db1);
    else if (dtype != DT_BF16 && Fr % 4 == 0)
      grouped_colsum_vec_kernel<float, 4><<<dim3((Fr + 31) / 32, groups), 1024, 0, s>>>((const float*)dA1, Fr, off_s,
                                                                                       (float*)db1);
    else if (dtype == DT_BF16)
      grouped_colsum_kernel<bf16><<<dim3((Fr + 63) / 64, groups), 256, 0, s>>>((const bf16*)dA1, Fr, off_s, (bf16*)db1);
    else
      grouped_colsum_kernel<float><<<dim3((Fr + 63) / 64, groups), 256, 0, s>>>((const float*)dA1, Fr, off_s,
                                                                                (float*)db1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (side) {
    e = hipStreamWaitEvent(s2, ev_dA1, 0);
    if (e != hipSuccess) return e;
  }
  {
    const bool t1 = gemm_bf16_grouped_k_eligible(gw1);
    ProfScope p(t1 ? "gemm_bf16_grouped_k<Xt.dA1, gather>" : "gemm_generic_grouped_k<Xt.dA1, gather>", s2, fl,
                es * ((double)tokens * H + (double)rows * Fr) + wts + 4.0 * rows);
    e = t1 ? launch_gemm_bf16_grouped_k(gw1, off_s, groups, (long)H * Fr, s2)
           : launch_gemm_generic_grouped_k(gw1, off_s, groups, (long)H * Fr, s2);
    if (e != hipSuccess) return e;
  }
  if (rows > 0) {
    ProfScope p(tiled ? "gemm_bf16_grouped<dA1.W1t>" : "gemm_generic_grouped<dA1.W1t>", s, fl,
                es * ((double)rows * Fr + (double)rows * H) + wts);
    e = tiled ? launch_gemm_bf16_grouped(gx, off_s, prefix2, tiles2, groups, (long)H * Fr, 0, (int)maxmt2, s)
              : launch_gemm_generic_grouped(gx, off_s, prefix2, tiles2, groups, (long)H * Fr, 0, (int)maxmt2, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tp
