// FP8 path (OCP E4M3 for weights and activations, E5M2 for gradients): per-tensor quantisation and a
// GEMM on 8-bit codes for gfx950.
//
// Quantisation: amax = max |x| (per-workgroup maxima, then one workgroup: max is order-free, so the
// result is exact and deterministic), s = vmax / amax and descale = amax / vmax in fp32 (vmax = 448
// or 57344; 1 and 1 for an all-zero tensor), codes = nearest code of fp32(x·s), ties to the even
// mantissa, saturating at ±vmax, by exact bit arithmetic on the fp32 value (no conversion
// instruction, so the rounding is the one stated).  The transposed form writes the [cols, rows] copy a GEMM operand
// needs K-major, through 64 x 64 LDS tiles so both the reads and the writes are whole rows; one pass
// can write both layouts (16-byte pieces when rows and cols are multiples of 16).
//
// GEMM: C[M, N] = (A·Bᵀ)·descale_a·descale_b (+ bias) (-> GeLU, or ∘ GeLU'(aux)), A [M, K] and
// B [N, K] codes, each E4M3 or E5M2, both K-major; bf16 out, fp32 accumulation.  The operand formats
// are the instruction's format selectors.  v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales:
// lane l holds row (l % 16) of its 16-row operand block and the 32 bytes k = 32·(l / 16) .. +31 (the
// instruction pairs byte b of A's lane-group g with byte b of B's lane-group g).  Tiles of BM x BN
// x 128 bytes go global -> LDS directly (16-byte pieces), in rows of 128 bytes whose 16-byte chunk c
// sits at c ^ ((r >> 1) & 7); a fragment is two ds_read_b128.  The B fragment is the MFMA's first
// operand, so lane l holds C[m = l % 16][n = 4·(l / 16) + e], four consecutive columns.  Tiles are
// ordered XCD by XCD and their k loops start at rotated k-tiles, as in the bf16 kernel.
#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace tp {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr unsigned F8_OOB = 0x80000000u;

// ---- E4M3 encoding (round to nearest even, saturating) ------------------------------------------
__device__ __forceinline__ unsigned e4m3_code(float y) {
  const unsigned u = __float_as_uint(y);
  const unsigned sign = (u >> 24) & 0x80u;
  const float a = fabsf(y);
  if (a != a) return 0x7Fu;                       // NaN
  if (!(a <= 448.f)) return sign | 0x7Eu;         // saturate
  if (a < 0.015625f) {                            // below 2^-6: multiples of 2^-9 (8 -> 2^-6, normal)
    const float m = a * 512.f;                    // exact: a power-of-two scaling
    return sign | (unsigned)rintf(m);             // round to nearest even
  }
  int e = (int)((u >> 23) & 0xFFu) - 127;         // -6 .. 8
  const unsigned mant = u & 0x7FFFFFu;
  unsigned keep = mant >> 20, rest = mant & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) {
    keep = 0u;
    ++e;
  }
  if (e > 8 || (e == 8 && keep == 7u)) return sign | 0x7Eu;
  return sign | ((unsigned)(e + 7) << 3) | keep;
}

// ---- E5M2 encoding (round to nearest even, saturating at ±57344) ---------------------------------
__device__ __forceinline__ unsigned e5m2_code(float y) {
  const unsigned u = __float_as_uint(y);
  const unsigned sign = (u >> 24) & 0x80u;
  const float a = fabsf(y);
  if (a != a) return 0x7Fu;                       // NaN
  if (!(a <= 57344.f)) return sign | 0x7Bu;       // saturate
  if (a < 6.103515625e-05f) {                     // below 2^-14: multiples of 2^-16 (4 -> 2^-14, normal)
    const float m = a * 65536.f;                  // exact: a power-of-two scaling
    return sign | (unsigned)rintf(m);
  }
  int e = (int)((u >> 23) & 0xFFu) - 127;         // -14 .. 15
  const unsigned mant = u & 0x7FFFFFu;
  unsigned keep = mant >> 21, rest = mant & 0x1FFFFFu;
  if (rest > 0x100000u || (rest == 0x100000u && (keep & 1u))) ++keep;
  if (keep == 4u) {
    keep = 0u;
    ++e;
  }
  if (e > 15) return sign | 0x7Bu;
  return sign | ((unsigned)(e + 15) << 2) | keep;
}

template <int FMT>
__device__ __forceinline__ unsigned fp8_code(float y) {
  if constexpr (FMT == 0) return e4m3_code(y);
  else return e5m2_code(y);
}

// ---- amax and the scales --------------------------------------------------------------------------
constexpr int AMAX_WGS = 1024;

template <typename T>
__global__ __launch_bounds__(256) void fp8_amax_kernel(long n, const T* __restrict__ x, float* __restrict__ part) {
  __shared__ float red[4];
  float m = 0.f;
  const long stride = (long)gridDim.x * 256 * 8;
  for (long i = ((long)blockIdx.x * 256 + threadIdx.x) * 8; i < n; i += stride) {
    if (i + 8 <= n) {
      if constexpr (sizeof(T) == 2) {
        const bf16x8 v = *(const bf16x8*)(x + i);
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf((float)v[j]));
      } else {
        const f32x4 a = *(const f32x4*)(x + i), b = *(const f32x4*)(x + i + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(a[j]), fabsf(b[j])));
      }
    } else {
      for (long j = i; j < n; ++j) m = fmaxf(m, fabsf(to_f32(x[j])));
    }
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// scale = 448 / amax (the quantiser's), descale = amax / 448 (the GEMM's); 1 and 1 for amax = 0.
__global__ __launch_bounds__(256) void fp8_scale_kernel(int parts, const float* __restrict__ part, float vmax,
                                                        float* __restrict__ scale, float* __restrict__ descale) {
  __shared__ float red[4];
  float m = 0.f;
  for (int i = threadIdx.x; i < parts; i += 256) m = fmaxf(m, part[i]);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    *scale = amax > 0.f ? vmax / amax : 1.f;
    *descale = amax > 0.f ? amax / vmax : 1.f;
  }
}

template <typename T, int FMT>
__global__ __launch_bounds__(256) void fp8_quantize_kernel(long n, const T* __restrict__ x,
                                                           const float* __restrict__ scale,
                                                           unsigned char* __restrict__ q) {
  const float s = *scale;
  const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  if (i + 8 <= n) {
    float v[8];
    if constexpr (sizeof(T) == 2) {
      const bf16x8 a = *(const bf16x8*)(x + i);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (float)a[j];
    } else {
      const f32x4 a = *(const f32x4*)(x + i), b = *(const f32x4*)(x + i + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) { v[j] = a[j]; v[4 + j] = b[j]; }
    }
    unsigned long long w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= (unsigned long long)fp8_code<FMT>(v[j] * s) << (8 * j);
    *(unsigned long long*)(q + i) = w;
  } else {
    for (long j = i; j < n; ++j) q[j] = (unsigned char)fp8_code<FMT>(to_f32(x[j]) * s);
  }
}

// x [rows, cols] -> q [cols, rows], one 64 x 64 tile per workgroup.
template <typename T, int FMT>
__global__ __launch_bounds__(256) void fp8_quantize_t_kernel(int rows, int cols, const T* __restrict__ x,
                                                             const float* __restrict__ scale,
                                                             unsigned char* __restrict__ q) {
  __shared__ unsigned char t[64][64 + 4];
  const float s = *scale;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i / 64, c = i % 64;
    const int gr = r0 + r, gc = c0 + c;
    t[c][r] = (gr < rows && gc < cols) ? (unsigned char)fp8_code<FMT>(to_f32(x[(long)gr * cols + gc]) * s) : 0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int c = i / 64, r = i % 64;
    const int gr = r0 + r, gc = c0 + c;
    if (gr < rows && gc < cols) q[(long)gc * rows + gr] = t[c][r];
  }
}

// One pass writing the plain codes q [rows, cols] and / or the transposed codes qt [cols, rows] (either
// may be null), one 64 x 64 tile per workgroup, for rows and cols multiples of 16: thread i reads 16
// consecutive elements of tile row i / 4 (two or four 16-byte loads), stores their 16 codes plain with
// one 16-byte store, and leaves them in LDS; after the barrier it gathers 16 codes of one tile column
// and stores them as 16 bytes of a qt row.  Both sides are whole 16-byte pieces of rows.
template <typename T, int FMT>
__global__ __launch_bounds__(256) void fp8_quantize_2_kernel(int rows, int cols, const T* __restrict__ x,
                                                             const float* __restrict__ scale,
                                                             unsigned char* __restrict__ q,
                                                             unsigned char* __restrict__ qt) {
  __shared__ unsigned char t[64][64 + 16];
  const float s = *scale;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int r = threadIdx.x >> 2, cq = 16 * (threadIdx.x & 3);
  const int gr = r0 + r, gc = c0 + cq;
  if (gr < rows && gc < cols) {              // gc < cols implies gc + 15 < cols (cols % 16 == 0)
    float v[16];
    const T* src = x + (long)gr * cols + gc;
    if constexpr (sizeof(T) == 2) {
      const bf16x8 a = *(const bf16x8*)src, b = *(const bf16x8*)(src + 8);
#pragma unroll
      for (int j = 0; j < 8; ++j) { v[j] = (float)a[j]; v[8 + j] = (float)b[j]; }
    } else {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const f32x4 a = *(const f32x4*)(src + 4 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * h + j] = a[j];
      }
    }
    u32x4 w;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      unsigned u = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) u |= fp8_code<FMT>(v[4 * h + j] * s) << (8 * j);
      w[h] = u;
    }
    if (q) *(u32x4*)(q + (long)gr * cols + gc) = w;
    *(u32x4*)&t[r][cq] = w;
  }
  if (!qt) return;                           // uniform over the workgroup: no barrier is skipped unevenly
  __syncthreads();
  // output row c0 + oc (an input column), output columns r0 + orq .. +15 (input rows)
  const int oc = threadIdx.x >> 2, orq = 16 * (threadIdx.x & 3);
  if (c0 + oc < cols && r0 + orq < rows) {   // rows % 16 == 0: the 16 input rows all exist
    u32x4 w;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      unsigned u = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) u |= (unsigned)t[orq + 4 * h + j][oc] << (8 * j);
      w[h] = u;
    }
    *(u32x4*)(qt + (long)(c0 + oc) * rows + r0 + orq) = w;
  }
}

// ---- the GEMM -----------------------------------------------------------------------------------
template <int BM_, int BN_, int WM_, int WN_, int ST_ = 2>
struct F8Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = ST_;
  static constexpr int NW = WM * WN, NT = NW * 64;
  static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, STAGE = A_BYTES + B_BYTES;
  static constexpr int IPW_A = A_BYTES / 1024 / NW, IPW_B = B_BYTES / 1024 / NW;
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "loads must split evenly");
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(STAGES * STAGE <= 160 * 1024, "LDS holds 160 KiB");
};

template <int N>
__device__ __forceinline__ void f8_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ int f8_swz(int r) { return (r >> 1) & 7; }

// The 16-byte pieces of one operand's k-tile this lane loads: row r (of the tile) and byte column c.
template <int IPW>
__device__ __forceinline__ void f8_pieces(int wave, int lane, int (&r)[IPW], int (&c)[IPW]) {
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int o = (wave * IPW + j) * 1024 + 16 * lane;
    r[j] = o >> 7;
    c[j] = 16 * (((o >> 4) & 7) ^ f8_swz(r[j]));
  }
}

template <int W, int IPW>
__device__ __forceinline__ void f8_load(const unsigned char* p, long ld, int rows_total, int mn0, int k0, int K,
                                        TP_LDS char* dst, const int (&r)[IPW], const int (&c)[IPW], int wave) {
  const unsigned char* base = p + (long)mn0 * ld + k0;
  const unsigned span = (unsigned)((long)(W - 1) * ld + 128);
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)span, 0x00020000);
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const bool ok = (mn0 + r[j] < rows_total) && (k0 + c[j] < K);
    const unsigned off = (unsigned)((long)r[j] * ld + c[j]);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (TP_LDS void*)(dst + (wave * IPW + j) * 1024), 16,
                                             ok ? off : F8_OOB, 0, 0, 0);
  }
}

// Fragment of 16 rows x 128 k: lane l gets row mn0 + l % 16, bytes 32·(l / 16) .. +31.
__device__ __forceinline__ i32x8 f8_frag(const TP_LDS char* tile, int mn0, int lane) {
  const int r = mn0 + (lane & 15);
  const int c = 2 * (lane >> 4);
  const TP_LDS char* row = tile + r * 128;
  const u32x4 lo = *(const TP_LDS u32x4*)(row + ((c ^ f8_swz(r)) << 4));
  const u32x4 hi = *(const TP_LDS u32x4*)(row + (((c + 1) ^ f8_swz(r)) << 4));
  return (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

struct F8Desc {
  int M, N, K;
  const unsigned char* A;   // [M, K]
  const unsigned char* B;   // [N, K]
  const float* da;
  const float* db;
  const bf16* bias;         // [N] or nullptr
  bf16* C;                  // [M, N]
  bf16* C2;                 // pre-activation [M, N] (GeLU epilogues) or nullptr
  const bf16* aux;          // [M, N]: the GeLU' epilogues' A1
  int epi;                  // 0 none, 1 GeLU, 2 tanh GeLU, 3 ∘ GeLU'(aux), 4 ∘ tanh GeLU'(aux)
};

// Scale by the two descales, bias, GeLU / GeLU' epilogues, bf16 stores of the wave's FM x FN blocks at
// (wm, wn) inside the tile at (m0, n0).
template <int FM, int FN>
__device__ __forceinline__ void f8_epilogue(const F8Desc& d, int m0, int n0, int wm, int wn, int lane,
                                            const f32x4 (&acc)[FM][FN]) {
  const float sc = *d.da * *d.db;
  const int r16 = lane & 15, g4 = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm + 16 * i + r16;
    if (m >= d.M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn + 16 * j + g4;
      if (n >= d.N) continue;
      float a[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = acc[i][j][e] * sc;
      if (d.bias) {
        const bf16x4 b = *(const bf16x4*)(d.bias + n);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] += (float)b[e];
      }
      const long o = (long)m * d.N + n;
      if (d.epi == 1 || d.epi == 2) {
        if (d.C2) *(bf16x4*)(d.C2 + o) = (bf16x4){(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = act_f(a[e], d.epi - 1);
      } else if (d.epi >= 3) {
        const bf16x4 x = *(const bf16x4*)(d.aux + o);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] *= act_grad_f((float)x[e], d.epi - 3);
      }
      *(bf16x4*)(d.C + o) = (bf16x4){(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
    }
  }
}

// FA, FB: the formats of A and B (0 E4M3, 1 E5M2).  The B fragment is the instruction's first
// operand, so its format goes in the first selector.
template <class Cfg, int FA, int FB>
__global__ __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(Cfg::NW / 4, Cfg::NW / 4)))
void gemm_fp8_nt_kernel(F8Desc d, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) char smem[Cfg::STAGES * Cfg::STAGE];
  TP_LDS char* lds = (TP_LDS char*)smem;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int GROUP_M = 4;
  const int nwg = tiles_m * tiles_n;
  int wg = blockIdx.x;
  if (nwg % 8 == 0) wg = (wg % 8) * (nwg / 8) + wg / 8;
  const int per_group = GROUP_M * tiles_n;
  const int first_m = (wg / per_group) * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (wg % per_group) % gsize, tn = (wg % per_group) / gsize;
  const int m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;

  int ar[Cfg::IPW_A], ac[Cfg::IPW_A], br[Cfg::IPW_B], bc[Cfg::IPW_B];
  f8_pieces<Cfg::IPW_A>(wave, lane, ar, ac);
  f8_pieces<Cfg::IPW_B>(wave, lane, br, bc);
  const int wm = (wave / Cfg::WN) * Cfg::TM, wn = (wave % Cfg::WN) * Cfg::TN;
  f32x4 acc[Cfg::FM][Cfg::FN];
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int nk = (d.K + 127) / 128;
  const int rot = nk > 0 ? (tm + tn) % nk : 0;
  auto kpos = [&](int t) { const int i = t + rot; return (i >= nk ? i - nk : i) * 128; };
  auto load = [&](int t, int stage) {
    TP_LDS char* dst = lds + stage * Cfg::STAGE;
    const int k = kpos(t);
    f8_load<Cfg::BM, Cfg::IPW_A>(d.A, d.K, d.M, m0, k, d.K, dst, ar, ac, wave);
    f8_load<Cfg::BN, Cfg::IPW_B>(d.B, d.K, d.N, n0, k, d.K, dst + Cfg::A_BYTES, br, bc, wave);
  };
#pragma unroll
  for (int t = 0; t < Cfg::STAGES - 1; ++t)
    if (t < nk) load(t, t);
  int cur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + Cfg::STAGES - 2 < nk) f8_wait_vmcnt<(Cfg::STAGES - 2) * (Cfg::IPW_A + Cfg::IPW_B)>();
    else f8_wait_vmcnt<0>();
    __syncthreads();
    const TP_LDS char* at = lds + cur * Cfg::STAGE;
    const TP_LDS char* bt = at + Cfg::A_BYTES;
    if (kt + Cfg::STAGES - 1 < nk) {
      int ns = cur + Cfg::STAGES - 1;
      if (ns >= Cfg::STAGES) ns -= Cfg::STAGES;
      load(kt + Cfg::STAGES - 1, ns);
    }
    i32x8 af[Cfg::FM], bfr[Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) af[i] = f8_frag(at, wm + 16 * i, lane);
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) bfr[j] = f8_frag(bt, wn + 16 * j, lane);
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[j], af[i], acc[i][j], FB, FA, 0, 127, 0, 127);
    if (++cur == Cfg::STAGES) cur = 0;
  }

  f8_epilogue<Cfg::FM, Cfg::FN>(d, m0, n0, wm, wn, lane, acc);
}

// The ping-pong schedule on the 256 x 192 tile: the eight waves form two groups of four (one wave of
// each per SIMD) one phase apart; group g owns tile rows [128g, 128g + 128) as 2 x 2 waves of 64 x 96.
// Each wave alternates a memory phase (read its fragments of k-tile t from LDS, then issue its share
// of k-tile t+1's direct loads) and a compute phase (the k-tile's MFMAs), so on each SIMD one wave
// multiplies while the other reads.  Group g loads its own 128 rows of A, group 0 also loads B; each
// group waits for its loads at the end of its next compute phase (two phases for every load to land),
// and a stage is refilled only after both groups' reads of it ended.
struct F8PP {
  static constexpr int BM = 256, BN = 192, NT = 512, HALF = 128, FM = 4, FN = 6;
  static constexpr int A_HALF = HALF * 128, B_OFF = 2 * A_HALF, STAGE = B_OFF + BN * 128;
  static constexpr int IPW_A = A_HALF / 1024 / 4, IPW_B = BN * 128 / 1024 / 4;
  static_assert(2 * STAGE <= 160 * 1024 && (BN * 128) % 4096 == 0, "tile layout");
};

// Phase boundaries (the waits through the builtin, which the compiler's own wait placement counts;
// sched_barrier keeps MFMAs and memory operations inside their phase).
__device__ __forceinline__ void f8_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void f8_sync_lds() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0) alone
  f8_barrier();
}
__device__ __forceinline__ void f8_sync_vm() {
  __builtin_amdgcn_sched_barrier(0);
  f8_wait_vmcnt<0>();
  f8_barrier();
}

template <int FA, int FB>
__global__ __launch_bounds__(F8PP::NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_fp8_pp_kernel(F8Desc d, int tiles_m, int tiles_n) {
  using P = F8PP;
  __shared__ __attribute__((aligned(1024))) char smem[2 * P::STAGE];
  TP_LDS char* lds = (TP_LDS char*)smem;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 2, w4 = wave & 3;
  constexpr int GROUP_M = 4;
  const int nwg = tiles_m * tiles_n;
  int wg = blockIdx.x;
  if (nwg % 8 == 0) wg = (wg % 8) * (nwg / 8) + wg / 8;
  const int per_group = GROUP_M * tiles_n;
  const int first_m = (wg / per_group) * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (wg % per_group) % gsize, tn = (wg % per_group) / gsize;
  const int m0 = tm * P::BM, n0 = tn * P::BN;

  int ar[P::IPW_A], ac[P::IPW_A], br[P::IPW_B], bc[P::IPW_B];
  f8_pieces<P::IPW_A>(w4, lane, ar, ac);
  f8_pieces<P::IPW_B>(w4, lane, br, bc);
  const int wml = (w4 >> 1) * 64, wn = (w4 & 1) * 96;
  f32x4 acc[P::FM][P::FN];
#pragma unroll
  for (int i = 0; i < P::FM; ++i)
#pragma unroll
    for (int j = 0; j < P::FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int nk = (d.K + 127) / 128;
  const int rot = nk > 0 ? (tm + tn) % nk : 0;
  auto kpos = [&](int t) { const int i = t + rot; return (i >= nk ? i - nk : i) * 128; };
  auto issue = [&](int t, int st) {
    TP_LDS char* base = lds + st * P::STAGE;
    const int k = kpos(t);
    f8_load<P::HALF, P::IPW_A>(d.A, d.K, d.M, m0 + P::HALF * g, k, d.K, base + g * P::A_HALF, ar, ac, w4);
    if (g == 0) f8_load<P::BN, P::IPW_B>(d.B, d.K, d.N, n0, k, d.K, base + P::B_OFF, br, bc, w4);
  };

  if (nk > 0) issue(0, 0);
  f8_sync_vm();                  // k-tile 0 is in stage 0
  if (g == 1) f8_barrier();      // group 1 starts one phase behind
  for (int t = 0; t < nk; ++t) {
    const int st = t & 1;
    // memory phase: this k-tile's fragments, then the next k-tile's loads
    const TP_LDS char* at = lds + st * P::STAGE + g * P::A_HALF;
    const TP_LDS char* bt = lds + st * P::STAGE + P::B_OFF;
    i32x8 af[P::FM], bfr[P::FN];
#pragma unroll
    for (int i = 0; i < P::FM; ++i) af[i] = f8_frag(at, wml + 16 * i, lane);
#pragma unroll
    for (int j = 0; j < P::FN; ++j) bfr[j] = f8_frag(bt, wn + 16 * j, lane);
    if (t + 1 < nk) issue(t + 1, st ^ 1);
    f8_sync_lds();
    // compute phase
#pragma unroll
    for (int i = 0; i < P::FM; ++i)
#pragma unroll
      for (int j = 0; j < P::FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[j], af[i], acc[i][j], FB, FA, 0, 127, 0, 127);
    f8_sync_vm();
  }
  if (g == 0) f8_barrier();      // both groups have passed the same number of barriers

  f8_epilogue<P::FM, P::FN>(d, m0, n0, P::HALF * g + wml, wn, lane, acc);
}

using F8C0 = F8Tile<256, 256, 4, 2, 2>;   // 64 x 128 per wave
using F8C1 = F8Tile<256, 128, 4, 2, 2>;   // 64 x 64 per wave

template <class Cfg>
hipError_t f8_run(const F8Desc& d, int fa, int fb, hipStream_t s) {
  const int tm = (d.M + Cfg::BM - 1) / Cfg::BM, tn = (d.N + Cfg::BN - 1) / Cfg::BN;
  if (fa == 0 && fb == 0) gemm_fp8_nt_kernel<Cfg, 0, 0><<<tm * tn, Cfg::NT, 0, s>>>(d, tm, tn);
  else if (fa == 1 && fb == 0) gemm_fp8_nt_kernel<Cfg, 1, 0><<<tm * tn, Cfg::NT, 0, s>>>(d, tm, tn);
  else if (fa == 0 && fb == 1) gemm_fp8_nt_kernel<Cfg, 0, 1><<<tm * tn, Cfg::NT, 0, s>>>(d, tm, tn);
  else return hipErrorNotSupported;   // two E5M2 operands: not a pairing the MLP uses
  return hipGetLastError();
}

}  // namespace

size_t fp8_quantize_ws_bytes() { return (AMAX_WGS + 64) * sizeof(float); }

hipError_t launch_fp8_quantize(int dtype, int fmt, int rows, int cols, const void* x, unsigned char* q,
                               unsigned char* qt, float* descale, float* ws, hipStream_t s) {
  const long n = (long)rows * cols;
  const double es = dtype == DT_BF16 ? 2.0 : 4.0;
  float* part = ws;
  float* scale = ws + AMAX_WGS;
  const int wgs = n > 0 ? (int)std::min<long>(AMAX_WGS, (n + 2047) / 2048) : 0;
  {
    ProfScope p("fp8_amax", s, (double)n, es * n);
    if (wgs > 0) {
      if (dtype == DT_BF16) fp8_amax_kernel<bf16><<<wgs, 256, 0, s>>>(n, (const bf16*)x, part);
      else fp8_amax_kernel<float><<<wgs, 256, 0, s>>>(n, (const float*)x, part);
    }
    fp8_scale_kernel<<<1, 256, 0, s>>>(wgs, part, fmt ? 57344.f : 448.f, scale, descale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n == 0 || (!q && !qt)) return hipSuccess;
  const double outs = (q ? 1.0 : 0.0) + (qt ? 1.0 : 0.0);
  // both layouts in one pass when the 16-element pieces tile the matrix; else one kernel per layout
  const bool two = rows % 16 == 0 && cols % 16 == 0;
  ProfScope p(two && qt ? (q ? "fp8_quantize_2" : "fp8_quantize_2<t>")
                        : (q && qt ? "fp8_quantize+t" : (qt ? "fp8_quantize_t" : "fp8_quantize")),
              s, (double)n, es * n + outs * n);
  auto go = [&](auto fmt_tag) {
    constexpr int F = decltype(fmt_tag)::value;
    if (two && qt) {
      dim3 grid((cols + 63) / 64, (rows + 63) / 64);
      if (dtype == DT_BF16) fp8_quantize_2_kernel<bf16, F><<<grid, 256, 0, s>>>(rows, cols, (const bf16*)x, scale, q, qt);
      else fp8_quantize_2_kernel<float, F><<<grid, 256, 0, s>>>(rows, cols, (const float*)x, scale, q, qt);
      return;
    }
    if (qt) {
      dim3 grid((cols + 63) / 64, (rows + 63) / 64);
      if (dtype == DT_BF16) fp8_quantize_t_kernel<bf16, F><<<grid, 256, 0, s>>>(rows, cols, (const bf16*)x, scale, qt);
      else fp8_quantize_t_kernel<float, F><<<grid, 256, 0, s>>>(rows, cols, (const float*)x, scale, qt);
    }
    if (q) {
      const long blocks = (n + 2047) / 2048;
      if (dtype == DT_BF16)
        fp8_quantize_kernel<bf16, F><<<(unsigned)blocks, 256, 0, s>>>(n, (const bf16*)x, scale, q);
      else
        fp8_quantize_kernel<float, F><<<(unsigned)blocks, 256, 0, s>>>(n, (const float*)x, scale, q);
    }
  };
  if (fmt) go(std::integral_constant<int, 1>());
  else go(std::integral_constant<int, 0>());
  return hipGetLastError();
}

namespace {
hipError_t f8_run_pp(const F8Desc& d, int fa, int fb, hipStream_t s) {
  const int tm = (d.M + F8PP::BM - 1) / F8PP::BM, tn = (d.N + F8PP::BN - 1) / F8PP::BN;
  if (fa == 0 && fb == 0) gemm_fp8_pp_kernel<0, 0><<<tm * tn, F8PP::NT, 0, s>>>(d, tm, tn);
  else if (fa == 1 && fb == 0) gemm_fp8_pp_kernel<1, 0><<<tm * tn, F8PP::NT, 0, s>>>(d, tm, tn);
  else if (fa == 0 && fb == 1) gemm_fp8_pp_kernel<0, 1><<<tm * tn, F8PP::NT, 0, s>>>(d, tm, tn);
  else return hipErrorNotSupported;
  return hipGetLastError();
}
}  // namespace

hipError_t launch_fp8_gemm_nt(int M, int N, int K, const unsigned char* A, int fa, const float* da,
                              const unsigned char* B, int fb, const float* db, const void* bias, int epi,
                              const void* aux, void* C, void* C2, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  F8Desc d{M, N, K, A, B, da, db, (const bf16*)bias, (bf16*)C, (bf16*)C2, (const bf16*)aux, epi};
  const double flop = 2.0 * M * (double)N * K;
  const double outs = 1.0 + ((epi == 1 || epi == 2) && C2 ? 1.0 : 0.0) + (epi >= 3 ? 1.0 : 0.0);
  const double bytes = (double)M * K + (double)N * K + 2.0 * M * (double)N * outs;
  // tile choice: (waves of 256 tiles) x tile area / relative per-tile rate, the smallest wins; the
  // 256 x 192 tile runs on the ping-pong schedule (measured 3-6% faster than the plain one)
  const int bn[3] = {256, 192, 128};
  const double rate[3] = {1.0, 0.95, 0.8};
  int best = 0;
  double best_t = 1e300;
  for (int c = 0; c < 3; ++c) {
    const long t = (long)((M + 255) / 256) * ((N + bn[c] - 1) / bn[c]);
    const double est = (double)((t + 255) / 256) * 256.0 * bn[c] / rate[c];
    if (est < best_t * 0.999) {
      best_t = est;
      best = c;
    }
  }
  static const char* const tags[3][3] = {
      {"gemm_fp8_nt<256x256, e4m3 x e4m3>", "gemm_fp8_nt<256x256, e5m2 x e4m3>", "gemm_fp8_nt<256x256, e4m3 x e5m2>"},
      {"gemm_fp8_nt<256x192pp, e4m3 x e4m3>", "gemm_fp8_nt<256x192pp, e5m2 x e4m3>", "gemm_fp8_nt<256x192pp, e4m3 x e5m2>"},
      {"gemm_fp8_nt<256x128, e4m3 x e4m3>", "gemm_fp8_nt<256x128, e5m2 x e4m3>", "gemm_fp8_nt<256x128, e4m3 x e5m2>"}};
  const int pair = fa ? 1 : (fb ? 2 : 0);
  ProfScope p(tags[best][pair], s, flop, bytes);
  if (best == 0) return f8_run<F8C0>(d, fa, fb, s);
  if (best == 1) return f8_run_pp(d, fa, fb, s);
  return f8_run<F8C1>(d, fa, fb, s);
}

}  // namespace tp
