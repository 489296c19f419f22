// Residual add with dropout, then LayerNorm, forward and backward — the replicated-side ops of the
// layer (or, under sequence parallelism, the same ops on a rank's row block).
//
// HBM-bound.  A workgroup of NT threads (256; 1024 when there are few rows) owns a whole row;
// thread t holds the row's elements [V·(t + NT·i), +V) for i < NV in registers (16-byte vectors: V = 8 bf16 or 4 fp32; V = 1 when
// rows are not 16-byte multiples), so every element is read from and written to HBM once.  Row sums
// go through a fixed-order wave + LDS reduction (deterministic).
//   forward : one row per workgroup; h = x + o∘keep·scale, the mean and (about a shift) the
//             variance of h in one pass and one reduction, y = (h − mean)·rstd·γ + β.
//   backward: dh and d_o one row per workgroup like the forward (two row sums, one reduction);
//             then dγ and dβ as column sums over the rows, x̂ recomputed from h and the saved
//             statistics (a second read of dy and h, 4 B per element in bf16), 64-row fp32
//             partials and a fixed-order sum of those.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace tp {

namespace {

constexpr int LN_THREADS = 256;
constexpr int LN_MAX_PER_THREAD = 96;   // elements per thread held in registers: H <= 24576

template <typename T, int V> struct Vec;
template <> struct Vec<bf16, 8> {
  typedef bf16x8 type;
  typedef unsigned long long mask;
};
template <> struct Vec<float, 4> {
  typedef f32x4 type;
  typedef unsigned mask;
};
template <typename T> struct Vec<T, 1> {
  typedef T type;
  typedef unsigned char mask;
};

template <typename T, int V>
__device__ __forceinline__ void load_vec(const T* p, float* out) {
  if constexpr (V == 1) {
    out[0] = to_f32(*p);
  } else {
    const typename Vec<T, V>::type v = *(const typename Vec<T, V>::type*)p;
#pragma unroll
    for (int j = 0; j < V; ++j) out[j] = (float)v[j];
  }
}

template <typename T, int V>
__device__ __forceinline__ void store_vec(T* p, const float* in) {
  if constexpr (V == 1) {
    *p = from_f32<T>(in[0]);
  } else {
    typename Vec<T, V>::type v;
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = from_f32<T>(in[j]);
    *(typename Vec<T, V>::type*)p = v;
  }
}

template <typename T, int V>
__device__ __forceinline__ void load_keep(const unsigned char* p, float* out) {
  const typename Vec<T, V>::mask m = *(const typename Vec<T, V>::mask*)p;
#pragma unroll
  for (int j = 0; j < V; ++j) out[j] = ((m >> (8 * j)) & 0xff) ? 1.f : 0.f;
}

// Sums of the N values v[] over the NW waves of the workgroup, the same in every thread; fixed
// order.  `red` holds NW * N floats.
template <int NW, int N>
__device__ __forceinline__ void block_sum(float* v, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1)
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] += __shfl_xor(v[k], m, 64);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int k = 0; k < N; ++k) red[w * N + k] = v[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < N; ++k) {
    float t = red[k];
#pragma unroll
    for (int q = 1; q < NW; ++q) t += red[q * N + k];
    v[k] = t;
  }
  __syncthreads();   // red may be rewritten by the next call
}

template <typename T, int NT, int V, int NV>
__global__ __launch_bounds__(NT) void ln_fwd_kernel(int H, const T* __restrict__ x, const T* __restrict__ o,
                                                    const unsigned char* __restrict__ keep, float scale,
                                                    const T* __restrict__ gamma, const T* __restrict__ beta,
                                                    float eps, T* __restrict__ h, T* __restrict__ y,
                                                    float* __restrict__ mean, float* __restrict__ rstd) {
  __shared__ float red[NT / 64 * 3];
  const long row = blockIdx.x;
  const long base = row * (long)H;
  // One pass and one reduction for both moments: mean = Σh/H, and the variance about a shift K,
  // the row's first element (computed the same way as every element): var = Σ(h−K)²/H − (Σ(h−K)/H)².
  // K lies within a few standard deviations of the mean, so the subtraction loses a bit or two.
  float K = to_f32(x[base]);
  if (o) K += to_f32(o[base]) * (keep ? (keep[base] ? scale : 0.f) : 1.f);
  K = to_f32(from_f32<T>(K));
  float v[NV][V];
  float sum[3] = {0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = V * (threadIdx.x + NT * i);
    if (c < H) {
      load_vec<T, V>(x + base + c, v[i]);
      if (o) {
        float ov[V], kv[V];
        load_vec<T, V>(o + base + c, ov);
        if (keep) {
          load_keep<T, V>(keep + base + c, kv);
#pragma unroll
          for (int j = 0; j < V; ++j) v[i][j] += ov[j] * kv[j] * scale;
        } else {
#pragma unroll
          for (int j = 0; j < V; ++j) v[i][j] += ov[j];
        }
      }
#pragma unroll
      for (int j = 0; j < V; ++j) v[i][j] = to_f32(from_f32<T>(v[i][j]));   // h as stored
      if (h) store_vec<T, V>(h + base + c, v[i]);
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const float d = v[i][j] - K;
        sum[0] += v[i][j];
        sum[1] += d;
        sum[2] += d * d;
      }
    }
  }
  block_sum<NT / 64, 3>(sum, red);
  const float mu = sum[0] / (float)H, m1 = sum[1] / (float)H;
  const float var = fmaxf(sum[2] / (float)H - m1 * m1, 0.f);
  const float rs = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = V * (threadIdx.x + NT * i);
    if (c < H) {
      float gv[V], bv[V], out[V];
      load_vec<T, V>(gamma + c, gv);
      load_vec<T, V>(beta + c, bv);
#pragma unroll
      for (int j = 0; j < V; ++j) out[j] = (v[i][j] - mu) * rs * gv[j] + bv[j];
      store_vec<T, V>(y + base + c, out);
    }
  }
  if (threadIdx.x == 0) {
    mean[row] = mu;
    rstd[row] = rs;
  }
}

template <typename T, int NT, int V, int NV>
__global__ __launch_bounds__(NT) void ln_bwd_row_kernel(int H, const T* __restrict__ dy,
                                                                const T* __restrict__ dh_in, const T* __restrict__ h,
                                                                const float* __restrict__ mean,
                                                                const float* __restrict__ rstd,
                                                                const T* __restrict__ gamma,
                                                                const unsigned char* __restrict__ keep, float scale,
                                                                T* __restrict__ dh, T* __restrict__ d_o) {
  __shared__ float red[NT / 64 * 2];
  const long row = blockIdx.x;
  const long base = row * (long)H;
  const float mu = mean[row], rs = rstd[row];
  float g[NV][V], xh[NV][V];
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = V * (threadIdx.x + NT * i);
    if (c < H) {
      float gv[V];
      load_vec<T, V>(dy + base + c, g[i]);
      load_vec<T, V>(h + base + c, xh[i]);
      load_vec<T, V>(gamma + c, gv);
#pragma unroll
      for (int j = 0; j < V; ++j) {
        xh[i][j] = (xh[i][j] - mu) * rs;
        g[i][j] *= gv[j];
        s1 += g[i][j];
        s2 += g[i][j] * xh[i][j];
      }
    }
  }
  float t[2] = {s1, s2};
  block_sum<NT / 64, 2>(t, red);
  const float m1 = t[0] / (float)H, m2 = t[1] / (float)H;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = V * (threadIdx.x + NT * i);
    if (c < H) {
      float out[V];
#pragma unroll
      for (int j = 0; j < V; ++j) out[j] = rs * (g[i][j] - m1 - xh[i][j] * m2);
      if (dh_in) {
        float a[V];
        load_vec<T, V>(dh_in + base + c, a);
#pragma unroll
        for (int j = 0; j < V; ++j) out[j] += a[j];
      }
      store_vec<T, V>(dh + base + c, out);
      if (d_o) {
        if (keep) {
          float kv[V];
          load_keep<T, V>(keep + base + c, kv);
#pragma unroll
          for (int j = 0; j < V; ++j) out[j] *= kv[j] * scale;
        }
        store_vec<T, V>(d_o + base + c, out);
      }
    }
  }
}

// dγ, dβ partials: a workgroup owns 256 columns x LP_ROWS rows; 32 column groups of 8 adjacent
// columns (16-byte loads when rows are 16-byte multiples) x 8 row groups, x̂ recomputed from h and
// the row statistics; the row groups meet in LDS in a fixed order, one fp32 partial of each per
// column and row block.
constexpr int LP_ROWS = 64;

template <typename T>
__global__ __launch_bounds__(256) void ln_param_partial_kernel(int rows, int H, const T* __restrict__ dy,
                                                               const T* __restrict__ h,
                                                               const float* __restrict__ mean,
                                                               const float* __restrict__ rstd,
                                                               float* __restrict__ ws_g, float* __restrict__ ws_b) {
  __shared__ float red[2][8][256 + 1];
  const int cg = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int c0 = blockIdx.x * 256 + 8 * cg;
  const int r0 = blockIdx.y * LP_ROWS;
  const int r1 = min(rows, r0 + LP_ROWS);
  float sg[8], sb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) sg[j] = sb[j] = 0.f;
  const bool vec = (c0 + 8 <= H) && ((H * sizeof(T)) % 16 == 0);
  if (c0 < H) {
    for (int r = r0 + rg; r < r1; r += 8) {
      const long o = (long)r * H + c0;
      const float mu = mean[r], rs = rstd[r];
      float a[8], b[8];
      if (vec) {
        if constexpr (sizeof(T) == 2) {
          load_vec<T, 8>(dy + o, a);
          load_vec<T, 8>(h + o, b);
        } else {
          load_vec<T, 4>(dy + o, a);
          load_vec<T, 4>(dy + o + 4, a + 4);
          load_vec<T, 4>(h + o, b);
          load_vec<T, 4>(h + o + 4, b + 4);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          a[j] = c0 + j < H ? to_f32(dy[o + j]) : 0.f;
          b[j] = c0 + j < H ? to_f32(h[o + j]) : mu;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sg[j] += a[j] * ((b[j] - mu) * rs);
        sb[j] += a[j];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    red[0][rg][8 * cg + j] = sg[j];
    red[1][rg][8 * cg + j] = sb[j];
  }
  __syncthreads();
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c < H) {
    float tg = 0.f, tb = 0.f;
    for (int k = 0; k < 8; ++k) {
      tg += red[0][k][threadIdx.x];
      tb += red[1][k][threadIdx.x];
    }
    ws_g[(long)blockIdx.y * H + c] = tg;
    ws_b[(long)blockIdx.y * H + c] = tb;
  }
}

int ln_param_chunks(int rows) { return rows > 0 ? (rows + LP_ROWS - 1) / LP_ROWS : 0; }

template <typename T, int NT, int V, int NV>
hipError_t ln_fwd_t(int rows, int H, const void* x, const void* o, const unsigned char* keep, float scale,
                    const void* gamma, const void* beta, float eps, void* h, void* y, float* mean,
                    float* rstd, hipStream_t s) {
  ln_fwd_kernel<T, NT, V, NV><<<rows, NT, 0, s>>>(H, (const T*)x, (const T*)o, keep, scale, (const T*)gamma,
                                                      (const T*)beta, eps, (T*)h, (T*)y, mean, rstd);
  return hipGetLastError();
}

template <typename T, int NT, int V, int NV>
hipError_t ln_bwd_t(int rows, int H, const void* dy, const void* dh_in, const void* h, const float* mean,
                    const float* rstd, const void* gamma, const unsigned char* keep, float scale, void* dh,
                    void* d_o, hipStream_t s) {
  ln_bwd_row_kernel<T, NT, V, NV><<<rows, NT, 0, s>>>(H, (const T*)dy, (const T*)dh_in, (const T*)h, mean, rstd,
                                                          (const T*)gamma, keep, scale, (T*)dh, (T*)d_o);
  return hipGetLastError();
}

template <typename T>
hipError_t ln_param_t(int rows, int H, const void* dy, const void* h, const float* mean, const float* rstd,
                      float* ws, hipStream_t s) {
  const int chunks = ln_param_chunks(rows);
  if (chunks > 0) {
    dim3 grid((H + 255) / 256, chunks);
    ln_param_partial_kernel<T><<<grid, 256, 0, s>>>(rows, H, (const T*)dy, (const T*)h, mean, rstd, ws,
                                                    ws + (size_t)chunks * H);
  }
  return hipGetLastError();
}

// Smallest register class holding ceil(H / NT) elements per thread, as NV vectors of V.  Few rows
// (a sequence-parallel block) get 1024-thread workgroups, so each row still spreads over 16 waves.
template <typename T, int V, template <typename, int, int, int> class F, typename... A>
hipError_t by_width(int rows, int H, A... a) {
  if constexpr (V > 1) {
    if (rows < 1024 && H >= 4096) {
      const int nv = ((H + 1023) / 1024 + V - 1) / V;
      if (nv <= 1) return F<T, 1024, V, 1>::run(a...);
      if (nv <= 2) return F<T, 1024, V, 2>::run(a...);
      if (nv <= 3) return F<T, 1024, V, 3>::run(a...);
      return F<T, 1024, V, LN_MAX_PER_THREAD / V / 4>::run(a...);
    }
  }
  const int per = (H + LN_THREADS - 1) / LN_THREADS;
  if constexpr (V == 1) {
    if (per <= 8) return F<T, LN_THREADS, 1, 8>::run(a...);
    if (per <= 24) return F<T, LN_THREADS, 1, 24>::run(a...);
    if (per <= 48) return F<T, LN_THREADS, 1, 48>::run(a...);
    return F<T, LN_THREADS, 1, 96>::run(a...);
  } else {
    const int nv = (per + V - 1) / V;
    if (nv <= 1) return F<T, LN_THREADS, V, 1>::run(a...);
    if (nv <= 2) return F<T, LN_THREADS, V, 2>::run(a...);
    if (nv <= 4) return F<T, LN_THREADS, V, 4>::run(a...);
    if (nv <= 6) return F<T, LN_THREADS, V, 6>::run(a...);
    if (nv <= 8) return F<T, LN_THREADS, V, 8>::run(a...);
    return F<T, LN_THREADS, V, LN_MAX_PER_THREAD / V>::run(a...);
  }
}

template <typename T, int NT, int V, int NV> struct FwdRun {
  template <typename... A> static hipError_t run(A... a) { return ln_fwd_t<T, NT, V, NV>(a...); }
};
template <typename T, int NT, int V, int NV> struct BwdRun {
  template <typename... A> static hipError_t run(A... a) { return ln_bwd_t<T, NT, V, NV>(a...); }
};

}  // namespace

int ln_max_h() { return LN_THREADS * LN_MAX_PER_THREAD; }

size_t ln_bwd_ws_bytes(int rows, int H) {
  if (rows <= 0 || H <= 0) return 0;
  return 2 * (size_t)ln_param_chunks(rows) * (size_t)H * sizeof(float);
}

hipError_t launch_ln_fwd(int dtype, int rows, int H, const void* x, const void* o, const unsigned char* keep,
                         float keep_scale, const void* gamma, const void* beta, float eps, void* h, void* y,
                         float* mean, float* rstd, hipStream_t s) {
  if (rows <= 0 || H <= 0) return hipSuccess;
  if (H > ln_max_h()) return hipErrorInvalidValue;
  const double es = dtype == DT_BF16 ? 2.0 : 4.0;
  const double n = (double)rows * H;
  const double bytes = n * es * (2.0 + (o ? 1.0 : 0.0) + (h ? 1.0 : 0.0)) + (keep ? n : 0.0) + 8.0 * rows;
  ProfScope p("ln_fwd", s, 8.0 * n, bytes);
  if (dtype == DT_BF16) {
    if (H % 8 == 0)
      return by_width<bf16, 8, FwdRun>(rows, H, rows, H, x, o, keep, keep_scale, gamma, beta, eps, h, y, mean, rstd, s);
    return by_width<bf16, 1, FwdRun>(rows, H, rows, H, x, o, keep, keep_scale, gamma, beta, eps, h, y, mean, rstd, s);
  }
  if (H % 4 == 0)
    return by_width<float, 4, FwdRun>(rows, H, rows, H, x, o, keep, keep_scale, gamma, beta, eps, h, y, mean, rstd, s);
  return by_width<float, 1, FwdRun>(rows, H, rows, H, x, o, keep, keep_scale, gamma, beta, eps, h, y, mean, rstd, s);
}

hipError_t launch_ln_bwd(int dtype, int rows, int H, const void* dy, const void* dh_in, const void* h,
                         const float* mean, const float* rstd, const void* gamma, const unsigned char* keep,
                         float keep_scale, void* dh, void* d_o, void* dgamma, void* dbeta, float* ws,
                         hipStream_t s) {
  if (H <= 0) return hipSuccess;
  if (H > ln_max_h()) return hipErrorInvalidValue;
  const double es = dtype == DT_BF16 ? 2.0 : 4.0;
  const double n = (double)rows * H;
  const int chunks = ln_param_chunks(rows);
  hipError_t e = hipSuccess;
  if (rows > 0) {
    const double bytes = n * es * (2.0 + (dh_in ? 1.0 : 0.0) + 1.0 + (d_o ? 1.0 : 0.0)) + (keep && d_o ? n : 0.0) +
                         8.0 * rows;
    ProfScope p("ln_bwd", s, 10.0 * n, bytes);
    if (dtype == DT_BF16)
      e = H % 8 == 0 ? by_width<bf16, 8, BwdRun>(rows, H, rows, H, dy, dh_in, h, mean, rstd, gamma, keep, keep_scale, dh,
                                                d_o, s)
                     : by_width<bf16, 1, BwdRun>(rows, H, rows, H, dy, dh_in, h, mean, rstd, gamma, keep, keep_scale, dh,
                                                d_o, s);
    else
      e = H % 4 == 0 ? by_width<float, 4, BwdRun>(rows, H, rows, H, dy, dh_in, h, mean, rstd, gamma, keep, keep_scale,
                                                 dh, d_o, s)
                     : by_width<float, 1, BwdRun>(rows, H, rows, H, dy, dh_in, h, mean, rstd, gamma, keep, keep_scale,
                                                 dh, d_o, s);
    if (e != hipSuccess) return e;
  }
  {
    ProfScope p("ln_bwd_params", s, 4.0 * n, n * es * 2.0 + 8.0 * rows + 16.0 * (double)chunks * H);
    if (rows > 0) {
      e = dtype == DT_BF16 ? ln_param_t<bf16>(rows, H, dy, h, mean, rstd, ws, s)
                           : ln_param_t<float>(rows, H, dy, h, mean, rstd, ws, s);
      if (e != hipSuccess) return e;
    }
    e = launch_colsum_final(dtype, ws, chunks, H, dgamma, s);
    if (e != hipSuccess) return e;
    e = launch_colsum_final(dtype, chunks > 0 ? ws + (size_t)chunks * H : ws, chunks, H, dbeta, s);
  }
  return e;
}

}  // namespace tp
