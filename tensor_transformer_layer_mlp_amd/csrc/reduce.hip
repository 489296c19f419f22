// Column sums over the token dimension (bias gradients): out[c] = Σ_r in[r, c].
// Deterministic: fixed 64-row chunks summed in order into an fp32 workspace, then the chunks in
// order.  Bandwidth-bound; each thread owns 8 adjacent columns so rows are read in 16-byte pieces
// when the layout allows.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace tp {

namespace {

constexpr int CS_ROWS = 64;   // rows per chunk
constexpr int CS_COLS = 8;    // columns per thread
constexpr int CS_THREADS = 256;

template <typename T>
__global__ __launch_bounds__(CS_THREADS) void colsum_partial_kernel(const T* in, long ld, int rows,
                                                                    int cols, float* ws) {
  const int c0 = (blockIdx.x * CS_THREADS + threadIdx.x) * CS_COLS;
  const int chunk = blockIdx.y;
  if (c0 >= cols) return;
  const int r0 = chunk * CS_ROWS, r1 = min(rows, r0 + CS_ROWS);
  float s[CS_COLS];
  for (int j = 0; j < CS_COLS; ++j) s[j] = 0.f;
  const bool full = (c0 + CS_COLS <= cols) && ((ld * sizeof(T)) % 16 == 0) &&
                    (((uintptr_t)in) % 16 == 0);
  for (int r = r0; r < r1; ++r) {
    const T* p = in + (long)r * ld + c0;
    if (full) {
      if constexpr (sizeof(T) == 2) {
        bf16x8 v = *(const bf16x8*)p;
        for (int j = 0; j < 8; ++j) s[j] += (float)v[j];
      } else {
        f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
        for (int j = 0; j < 4; ++j) { s[j] += a[j]; s[4 + j] += b[j]; }
      }
    } else {
      for (int j = 0; j < CS_COLS; ++j)
        if (c0 + j < cols) s[j] += to_f32(p[j]);
    }
  }
  for (int j = 0; j < CS_COLS; ++j)
    if (c0 + j < cols) ws[(long)chunk * cols + c0 + j] = s[j];
}

template <typename T>
__global__ __launch_bounds__(256) void colsum_final_kernel(const float* ws, int chunks, int cols,
                                                           T* out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  float s = 0.f;
  for (int k = 0; k < chunks; ++k) s += ws[(long)k * cols + c];
  out[c] = from_f32<T>(s);
}

template <typename T>
hipError_t colsum_t(const void* in, long ld, int rows, int cols, float* ws, void* out,
                    hipStream_t s) {
  const int chunks = (rows + CS_ROWS - 1) / CS_ROWS;
  if (chunks > 0) {
    dim3 grid((cols + CS_THREADS * CS_COLS - 1) / (CS_THREADS * CS_COLS), chunks);
    colsum_partial_kernel<T><<<grid, CS_THREADS, 0, s>>>((const T*)in, ld, rows, cols, ws);
  }
  colsum_final_kernel<T><<<(cols + 255) / 256, 256, 0, s>>>(ws, chunks, cols, (T*)out);
  return hipGetLastError();
}

}  // namespace

size_t colsum_ws_bytes(int rows, int cols) {
  const size_t chunks = (size_t)(rows + CS_ROWS - 1) / CS_ROWS;
  return chunks * (size_t)cols * sizeof(float);
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
