// Generic MFMA GEMM: any M, N, K, any operand layout, bf16 or fp32, all epilogues.
//
// It serves the fp32 check mode, shapes the tiled bf16 kernel does not take (ragged leading
// dimensions, tiny problems), and is the second opinion the bf16 kernel is tested against.
// 64x64 output tile, 4 waves in a 2x2 grid, each wave 32x32 = 2x2 MFMA blocks of 16x16.
// Operands are staged through LDS in a k-contiguous layout with bounds-checked loads (zero fill).
#include "common.h"
#include "kernels.h"

namespace tp {

namespace {

constexpr int GBM = 64, GBN = 64;

template <typename T> struct GenericK;
template <> struct GenericK<bf16> { static constexpr int BK = 32, PAD = 8; };
template <> struct GenericK<float> { static constexpr int BK = 16, PAD = 4; };

template <typename T, int EPI>
__device__ __forceinline__ void store_epi(const GemmDesc& d, int m, int n, float v) {
  T* C = (T*)d.C;
  long o = (long)m * d.ldc + n;
  if constexpr (EPI == EPI_STORE) {
    C[o] = from_f32<T>(v);
  } else if constexpr (EPI == EPI_BIAS) {
    C[o] = from_f32<T>(v + to_f32(((const T*)d.bias)[n]));
  } else if constexpr (EPI == EPI_BIAS_GELU) {
    float a = v + to_f32(((const T*)d.bias)[n]);
    if (d.C2) ((T*)d.C2)[o] = from_f32<T>(a);
    C[o] = from_f32<T>(act_f(a, d.act));
  } else {
    float a = to_f32(((const T*)d.aux)[(long)m * d.ld_aux + n]);
    C[o] = from_f32<T>(v * act_grad_f(a, d.act));
  }
}

template <typename T, int EPI>
__device__ __forceinline__ void generic_tile(const GemmDesc& d, int m0, int n0) {
  constexpr int BK = GenericK<T>::BK, PAD = GenericK<T>::PAD;
  __shared__ __attribute__((aligned(16))) T As[GBM][BK + PAD];
  __shared__ __attribute__((aligned(16))) T Bs[GBN][BK + PAD];
  const T* A = (const T*)d.A;
  const T* B = (const T*)d.B;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const int r16 = lane & 15, g = lane >> 4;
  f32x4 acc[2][2];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < d.K; k0 += BK) {
    for (int i = tid; i < GBM * BK; i += 256) {
      int m, k;
      if (d.a_kmajor) { m = i / BK; k = i % BK; } else { k = i / GBM; m = i % GBM; }
      const int gm = m0 + m, gk = k0 + k;
      T v = from_f32<T>(0.f);
      if (gm < d.M && gk < d.K) {
        if (d.a_rows) {          // gathered rows of the source matrix; outside [0, a_rows_n) reads zero
          const int src = d.a_rows[d.a_kmajor ? gm : gk];
          if (src >= 0 && src < d.a_rows_n) v = d.a_kmajor ? A[(long)src * d.lda + gk] : A[(long)src * d.lda + gm];
        } else {
          v = d.a_kmajor ? A[(long)gm * d.lda + gk] : A[(long)gk * d.lda + gm];
        }
      }
      As[m][k] = v;
    }
    for (int i = tid; i < GBN * BK; i += 256) {
      int n, k;
      if (d.b_kmajor) { n = i / BK; k = i % BK; } else { k = i / GBN; n = i % GBN; }
      const int gn = n0 + n, gk = k0 + k;
      T v = from_f32<T>(0.f);
      if (gn < d.N && gk < d.K) {
        if (d.b_rows) {          // gathered rows of the source matrix; outside [0, b_rows_n) reads zero
          const int src = d.b_rows[d.b_kmajor ? gn : gk];
          if (src >= 0 && src < d.b_rows_n) v = d.b_kmajor ? B[(long)src * d.ldb + gk] : B[(long)src * d.ldb + gn];
        } else {
          v = d.b_kmajor ? B[(long)gn * d.ldb + gk] : B[(long)gk * d.ldb + gn];
        }
      }
      Bs[n][k] = v;
    }
    __syncthreads();
    if constexpr (sizeof(T) == 2) {
      bf16x8 af[2], bfr[2];
      for (int i = 0; i < 2; ++i) af[i] = *(const bf16x8*)&As[wm + i * 16 + r16][8 * g];
      for (int j = 0; j < 2; ++j) bfr[j] = *(const bf16x8*)&Bs[wn + j * 16 + r16][8 * g];
      // operands swapped so that lane l holds C[m = l%16][n = 4*(l/16) + e]
      for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_16x16x32_bf16(bfr[j], af[i], acc[i][j]);
    } else {
      for (int kk = 0; kk < BK; kk += 4) {
        float af[2], bfr[2];
        for (int i = 0; i < 2; ++i) af[i] = As[wm + i * 16 + r16][kk + g];
        for (int j = 0; j < 2; ++j) bfr[j] = Bs[wn + j * 16 + r16][kk + g];
        for (int i = 0; i < 2; ++i)
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma_16x16x4_f32(bfr[j], af[i], acc[i][j]);
      }
    }
    __syncthreads();
  }
  if constexpr (EPI == EPI_DGELU_GATE) {
    // C = row_scale[m]·acc∘GeLU'(aux), and per row Σ_n aux2[m, n]·acc over this n-tile: lane-local in
    // (j, e) order, then over the four lanes of a row, then the two waves along n in LDS, in order
    __shared__ float red[2][GBM];
    float rowdot[2] = {0.f, 0.f};
    for (int i = 0; i < 2; ++i)
      for (int j = 0; j < 2; ++j)
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + wm + i * 16 + r16;
          const int n = n0 + wn + j * 16 + 4 * g + e;
          if (m < d.M && n < d.N) {
            const float v = acc[i][j][e];
            rowdot[i] = fmaf(to_f32(((const T*)d.aux2)[(long)m * d.ld_aux2 + n]), v, rowdot[i]);
            const float x = to_f32(((const T*)d.aux)[(long)m * d.ld_aux + n]);
            ((T*)d.C)[(long)m * d.ldc + n] = from_f32<T>(v * (d.row_scale[m] * act_grad_f(x, d.act)));
          }
        }
    for (int i = 0; i < 2; ++i) {
      rowdot[i] += __shfl_xor(rowdot[i], 16);
      rowdot[i] += __shfl_xor(rowdot[i], 32);
    }
    if (lane < 16)
      for (int i = 0; i < 2; ++i) red[wave & 1][wm + i * 16 + r16] = rowdot[i];
    __syncthreads();
    if ((wave & 1) == 0 && lane < 16)
      for (int i = 0; i < 2; ++i) {
        const int r = wm + i * 16 + r16;
        if (m0 + r < d.M) d.row_dot[(long)(n0 / GBN) * d.rd_stride + m0 + r] = red[0][r] + red[1][r];
      }
    return;
  }
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j)
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm + i * 16 + r16;
        const int n = n0 + wn + j * 16 + 4 * g + e;
        if (m < d.M && n < d.N) store_epi<T, EPI>(d, m, n, acc[i][j][e]);
      }
}

template <typename T, int EPI>
__global__ __launch_bounds__(256) void gemm_generic_kernel(GemmDesc d) {
  generic_tile<T, EPI>(d, blockIdx.y * GBM, blockIdx.x * GBN);
}

// Grouped form (see the tiled bf16 kernel): expert e owns rows [off[e], off[e+1]); prefix[] numbers
// the GBM-row tiles of all experts; blockIdx.y is that tile number, blockIdx.x the n-tile.
template <typename T, int EPI>
__global__ __launch_bounds__(256) void gemm_generic_grouped_kernel(GemmDesc g, const int* off,
                                                                   const int* prefix, const int* tile_expert,
                                                                   int groups, long b_stride, long bias_stride) {
  const int mt = blockIdx.y;
  if (mt >= prefix[groups]) return;
  const int e = tile_expert[mt];       // the expert whose m-tiles [prefix[e], prefix[e+1]) hold mt
  const int row0 = off[e] + (mt - prefix[e]) * GBM;
  GemmDesc d = g;
  d.M = off[e + 1] - row0;
  if (g.a_rows) d.a_rows = g.a_rows + row0;   // A stays the whole gathered-from matrix
  else d.A = (const T*)g.A + (long)row0 * g.lda;
  d.B = (const T*)g.B + (long)e * b_stride;
  d.C = (T*)g.C + (long)row0 * g.ldc;
  if (g.C2) d.C2 = (T*)g.C2 + (long)row0 * g.ldc;
  if (g.bias) d.bias = (const T*)g.bias + (long)e * bias_stride;
  if (g.aux) d.aux = (const T*)g.aux + (long)row0 * g.ld_aux;
  if constexpr (EPI == EPI_DGELU_GATE) {
    d.aux2 = (const T*)g.aux2 + (long)row0 * g.ld_aux2;
    d.row_scale = g.row_scale + row0;
    d.row_dot = g.row_dot + row0;
  }
  generic_tile<T, EPI>(d, 0, blockIdx.x * GBN);
}

// Grouped weight-gradient form (see the tiled kernel): blockIdx.z is the expert, whose rows
// [off[e], off[e+1]) of A and B form the k range; its C block sits at e·c_stride.
template <typename T>
__global__ __launch_bounds__(256) void gemm_generic_grouped_k_kernel(GemmDesc g, const int* off, long c_stride) {
  const int e = blockIdx.z;
  GemmDesc d = g;
  const int k0 = off[e];
  d.K = off[e + 1] - k0;
  if (g.a_rows) d.a_rows = g.a_rows + k0;   // A stays the whole gathered-from matrix
  else d.A = (const T*)g.A + (long)k0 * g.lda;
  if (g.b_rows) d.b_rows = g.b_rows + k0;   // B likewise
  else d.B = (const T*)g.B + (long)k0 * g.ldb;
  d.C = (T*)g.C + (long)e * c_stride;
  generic_tile<T, EPI_STORE>(d, blockIdx.y * GBM, blockIdx.x * GBN);
}

template <typename T>
hipError_t launch_generic_t(const GemmDesc& d, hipStream_t s) {
  dim3 grid((d.N + GBN - 1) / GBN, (d.M + GBM - 1) / GBM);
  switch (d.epi) {
    case EPI_STORE: gemm_generic_kernel<T, EPI_STORE><<<grid, 256, 0, s>>>(d); break;
    case EPI_BIAS: gemm_generic_kernel<T, EPI_BIAS><<<grid, 256, 0, s>>>(d); break;
    case EPI_BIAS_GELU: gemm_generic_kernel<T, EPI_BIAS_GELU><<<grid, 256, 0, s>>>(d); break;
    case EPI_DGELU: gemm_generic_kernel<T, EPI_DGELU><<<grid, 256, 0, s>>>(d); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_generic_grouped_t(const GemmDesc& d, const int* off, const int* prefix, const int* tile_expert,
                                    int groups, long b_stride, long bias_stride, int max_mtiles, hipStream_t s) {
  dim3 grid((d.N + GBN - 1) / GBN, max_mtiles);
  const int* te = tile_expert;
  if (d.epi == EPI_BIAS_GELU)
    gemm_generic_grouped_kernel<T, EPI_BIAS_GELU><<<grid, 256, 0, s>>>(d, off, prefix, te, groups, b_stride, bias_stride);
  else if (d.epi == EPI_STORE)
    gemm_generic_grouped_kernel<T, EPI_STORE><<<grid, 256, 0, s>>>(d, off, prefix, te, groups, b_stride, bias_stride);
  else if (d.epi == EPI_DGELU)
    gemm_generic_grouped_kernel<T, EPI_DGELU><<<grid, 256, 0, s>>>(d, off, prefix, te, groups, b_stride, bias_stride);
  else if (d.epi == EPI_DGELU_GATE)
    gemm_generic_grouped_kernel<T, EPI_DGELU_GATE><<<grid, 256, 0, s>>>(d, off, prefix, te, groups, b_stride,
                                                                        bias_stride);
  else
    return hipErrorNotSupported;
  return hipGetLastError();
}

}  // namespace

int gemm_generic_grouped_bm() { return GBM; }
int gemm_generic_grouped_bn() { return GBN; }

hipError_t launch_gemm_generic_grouped(const GemmDesc& d, const int* off, const int* prefix, const int* tile_expert,
                                       int groups, long b_stride, long bias_stride, int max_mtiles, hipStream_t s) {
  if (max_mtiles <= 0 || d.N <= 0) return hipSuccess;
  if (max_mtiles > 65535) return hipErrorInvalidValue;
  return d.dtype == DT_BF16
             ? launch_generic_grouped_t<bf16>(d, off, prefix, tile_expert, groups, b_stride, bias_stride,
                                              max_mtiles, s)
             : launch_generic_grouped_t<float>(d, off, prefix, tile_expert, groups, b_stride, bias_stride,
                                               max_mtiles, s);
}

hipError_t launch_gemm_generic_grouped_k(const GemmDesc& d, const int* off, int groups, long c_stride, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0 || groups <= 0) return hipSuccess;
  if ((d.M + GBM - 1) / GBM > 65535 || groups > 65535) return hipErrorInvalidValue;
  dim3 grid((d.N + GBN - 1) / GBN, (d.M + GBM - 1) / GBM, groups);
  if (d.dtype == DT_BF16) gemm_generic_grouped_k_kernel<bf16><<<grid, 256, 0, s>>>(d, off, c_stride);
  else gemm_generic_grouped_k_kernel<float><<<grid, 256, 0, s>>>(d, off, c_stride);
  return hipGetLastError();
}

hipError_t launch_gemm_generic(const GemmDesc& d, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0) return hipSuccess;
  if ((d.N + GBN - 1) / GBN > 0x7fffffff || (d.M + GBM - 1) / GBM > 65535) return hipErrorInvalidValue;
  return d.dtype == DT_BF16 ? launch_generic_t<bf16>(d, s) : launch_generic_t<float>(d, s);
}

}  // namespace tp
