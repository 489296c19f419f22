// Column sums over the token dimension (bias gradients): out[c] = Σ_r in[r, c].
//
// Deterministic two-pass reduction in fp32.  Pass 1: a workgroup owns a 256-column x 64-row block;
// its 256 threads are 32 column groups (8 adjacent columns each, 16-byte loads, so a half-wave reads
// 512 contiguous bytes of a row) x 8 row groups (rows r0 + g, r0 + g + 8, ...); the 8 row-group
// sums meet in LDS in a fixed order and one fp32 partial per column and block row is written.
// Pass 2 adds the block-row partials of each column in a fixed order.  HBM-bound: the input is read once.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace tp {

namespace {

constexpr int CS_ROWS = 64;    // rows per partial (enough workgroups to fill the chip at T = 2048)
constexpr int CS_COLS = 256;   // columns per workgroup
constexpr int CS_RG = 8;       // row groups per workgroup

template <typename T>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const T* __restrict__ in, long ld, int rows,
                                                             int cols, float* __restrict__ ws) {
  __shared__ float red[CS_RG][CS_COLS + 1];
  const int cg = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int c0 = blockIdx.x * CS_COLS + 8 * cg;
  const int r0 = blockIdx.y * CS_ROWS;
  const int r1 = min(rows, r0 + CS_ROWS);
  float s[8];
  for (int j = 0; j < 8; ++j) s[j] = 0.f;
  const bool vec = (c0 + 8 <= cols) && ((ld * sizeof(T)) % 16 == 0) && (((uintptr_t)in) % 16 == 0);
  if (c0 < cols) {
    int r = r0 + rg;
    if constexpr (sizeof(T) == 2) {
      // a whole 64-row block: all eight rows' loads issued before the adds (same order of addition)
      if (vec && r1 - r0 == CS_ROWS) {
        bf16x8 v[CS_ROWS / CS_RG];
#pragma unroll
        for (int i = 0; i < CS_ROWS / CS_RG; ++i) v[i] = *(const bf16x8*)(in + (long)(r + CS_RG * i) * ld + c0);
#pragma unroll
        for (int i = 0; i < CS_ROWS / CS_RG; ++i)
          for (int j = 0; j < 8; ++j) s[j] += (float)v[i][j];
        r = r1;
      }
    }
    for (; r < r1; r += CS_RG) {
      const T* p = in + (long)r * ld + c0;
      if (vec) {
        if constexpr (sizeof(T) == 2) {
          const bf16x8 v = *(const bf16x8*)p;
          for (int j = 0; j < 8; ++j) s[j] += (float)v[j];
        } else {
          const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
          for (int j = 0; j < 4; ++j) { s[j] += a[j]; s[4 + j] += b[j]; }
        }
      } else {
        for (int j = 0; j < 8; ++j)
          if (c0 + j < cols) s[j] += to_f32(p[j]);
      }
    }
  }
  for (int j = 0; j < 8; ++j) red[rg][8 * cg + j] = s[j];
  __syncthreads();
  const int c = blockIdx.x * CS_COLS + threadIdx.x;
  if (c < cols) {
    float t = 0.f;
    for (int g = 0; g < CS_RG; ++g) t += red[g][threadIdx.x];
    ws[(long)blockIdx.y * cols + c] = t;
  }
}

// Pass 2: 64 columns per workgroup; its four waves add every fourth partial of a column (chunks
// g, g+4, ...), and the four sums meet in LDS in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void colsum_final_kernel(const float* __restrict__ ws, int chunks,
                                                           int cols, T* __restrict__ out) {
  __shared__ float red[4][64];
  const int c = blockIdx.x * 64 + (threadIdx.x & 63), g = threadIdx.x >> 6;
  float s = 0.f;
  if (c < cols) {
    int k = g;
    // eight partials' loads at a time, added in the same order
    for (; k + 28 < chunks; k += 32) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = ws[(long)(k + 4 * i) * cols + c];
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[i];
    }
    for (; k < chunks; k += 4) s += ws[(long)k * cols + c];
  }
  red[g][threadIdx.x & 63] = s;
  __syncthreads();
  if (g == 0 && c < cols) out[c] = from_f32<T>(((red[0][threadIdx.x] + red[1][threadIdx.x]) + red[2][threadIdx.x]) + red[3][threadIdx.x]);
}

template <typename T>
hipError_t colsum_t(const void* in, long ld, int rows, int cols, float* ws, void* out, hipStream_t s) {
  const int chunks = (rows + CS_ROWS - 1) / CS_ROWS;
  if (chunks > 0) {
    dim3 grid((cols + CS_COLS - 1) / CS_COLS, chunks);
    colsum_partial_kernel<T><<<grid, 256, 0, s>>>((const T*)in, ld, rows, cols, ws);
  }
  colsum_final_kernel<T><<<(cols + 63) / 64, 256, 0, s>>>(ws, chunks, cols, (T*)out);
  return hipGetLastError();
}

// out[i] = Σ_s parts[s·n + i] in slice order, eight elements per thread.
__global__ __launch_bounds__(256) void splitk_sum_kernel(int S, long n, const float* __restrict__ parts,
                                                         bf16* __restrict__ out) {
  const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  f32x4 a = *(const f32x4*)(parts + i), b = *(const f32x4*)(parts + i + 4);
  for (int s = 1; s < S; ++s) {
    const f32x4 c = *(const f32x4*)(parts + (long)s * n + i), e = *(const f32x4*)(parts + (long)s * n + i + 4);
    a += c;
    b += e;
  }
  *(bf16x8*)(out + i) = (bf16x8){(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                                 (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
}

}  // namespace

hipError_t launch_splitk_sum(int S, long n, const float* parts, void* out, hipStream_t s) {
  if (n <= 0 || S <= 0) return hipSuccess;
  if (n % 8) return hipErrorInvalidValue;
  ProfScope p("splitk_sum", s, (double)S * n, 4.0 * S * n + 2.0 * n);
  const long blocks = (n / 8 + 255) / 256;
  splitk_sum_kernel<<<(unsigned)blocks, 256, 0, s>>>(S, n, parts, (bf16*)out);
  return hipGetLastError();
}

size_t colsum_ws_bytes(int rows, int cols) {
  const size_t chunks = (size_t)(rows + CS_ROWS - 1) / CS_ROWS;
  return chunks * (size_t)cols * sizeof(float);
}

hipError_t launch_colsum_final(int dtype, const float* ws, int chunks, int cols, void* out, hipStream_t s) {
  if (cols <= 0) return hipSuccess;
  if (dtype == DT_BF16)
    colsum_final_kernel<bf16><<<(cols + 63) / 64, 256, 0, s>>>(ws, chunks, cols, (bf16*)out);
  else
    colsum_final_kernel<float><<<(cols + 63) / 64, 256, 0, s>>>(ws, chunks, cols, (float*)out);
  return hipGetLastError();
}

hipError_t launch_colsum(int dtype, const void* in, long ld, int rows, int cols, float* ws,
                         void* out, hipStream_t s) {
  if (cols <= 0) return hipSuccess;
  const double es = dtype == DT_BF16 ? 2.0 : 4.0;
  ProfScope p("colsum", s, (double)rows * cols, es * ((double)rows * cols + cols));
  if ((rows + CS_ROWS - 1) / CS_ROWS > 65535) return hipErrorInvalidValue;
  return dtype == DT_BF16 ? colsum_t<bf16>(in, ld, rows, cols, ws, out, s)
                          : colsum_t<float>(in, ld, rows, cols, ws, out, s);
}

}  // namespace tp
