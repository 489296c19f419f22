// Tiled bf16 GEMM for gfx950: C = op(A)·op(B) with fp32 accumulation and a fused epilogue.
//
// Tile BM x BN x 64 per workgroup, WM x WN waves, each wave (BM/WM) x (BN/WN) built from
// v_mfma_f32_16x16x32_bf16 blocks.  Operands go global -> LDS directly (buffer_load_dwordx4 ... lds,
// no register staging) into two LDS stages: the loads of k-tile t+1 are in flight while the MFMAs
// consume k-tile t.
//
// LDS layouts (per operand, per stage):
//  * K-major operand (row m holds k contiguous: X·W's X, dY·Wᵀ's both operands): BMN rows of 128
//    bytes; the 16-byte chunk c of row r sits at chunk c ^ ((r >> 1) & 7), so the 16 rows one
//    ds_read_b128 touches land on distinct banks.
//  * MN-major operand (row k holds m or n contiguous: the [in, out] weights of the forward, both
//    operands of the weight gradients): 64 rows of 2*BMN bytes; the 32-byte chunk q of row k sits at
//    q ^ f(k), f(k) = (k & 3) | ((k >> 3) & 1) << 2.  Fragments are read with ds_read_b64_tr_b16,
//    which hands lane i of each 16-lane group column i of a 4 x 16 block: two of them give a lane the
//    8 consecutive k values of one m (or n) that the MFMA operand needs.
// Out-of-range rows, columns and k (ragged tails) are loaded as zeros: such lanes get a byte offset
// past the buffer descriptor's range.  Requires M, N, K, the leading dimensions and the base
// addresses to be multiples of 8 elements / 16 bytes (the host checks).
//
// The MFMA is issued with the B fragment as its first operand, so lane l holds
// C[m = l % 16][n = 4*(l / 16) + e], e = 0..3: four consecutive columns, stored as one 8-byte write.
#include "common.h"
#include "kernels.h"

namespace tp {

namespace {

#ifndef TP_GEMM_ROT_MIN_NK
#define TP_GEMM_ROT_MIN_NK 0      // k loops shorter than this start at k-tile 0 (tuning builds)
#endif
constexpr unsigned OOB = 0x80000000u;   // byte offset beyond any descriptor range -> loads zero

template <int BM_, int BN_, int WM_, int WN_, int ST_ = 2, int BK_ = 64, int OCC_ = 0>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = ST_, BKT = BK_;
  static constexpr int NW = WM * WN, NT = NW * 64;
  static constexpr int OCC = OCC_ ? OCC_ : NW / 4;   // waves per SIMD the registers are sized for
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 16, FN = TN / 16;
  static_assert(BKT == 32 || BKT == 64, "k per tile is 32 or 64");
  // An MN-major tile is stored as k-rows whose pitch is the tile width rounded up to a power of two
  // (the XOR swizzle needs it); columns past the width are loaded as zeros and never read.
  static constexpr int pitch(int w) { return w <= 128 ? 128 : (w <= 256 ? 256 : 512); }
  static constexpr int PM = pitch(BM), PN = pitch(BN);
  template <bool KMAJ, int W> static constexpr int bytes() { return (KMAJ ? W : pitch(W)) * BKT * 2; }
  static constexpr int STAGE = bytes<false, BM>() + bytes<false, BN>();   // room for either layout
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(BM >= 128 && BN >= 128, "MN-major swizzle needs at least 8 chunks of 32 bytes");
  static_assert(STAGES * STAGE <= 160 * 1024, "LDS holds 160 KiB");
};

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ int swz_f(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }

// K-major tile rows are 2*BKT bytes; chunk c of row r sits at c ^ ks(r), which spreads the 16 rows a
// ds_read_b128 touches over all 16 bank groups of a 256-byte window.
template <int BKT>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (BKT == 64) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}

// Byte offset inside an operand's tile of the 16-byte piece lane `lane` of load `j` carries, and the
// (row, col) of the global matrix it comes from, relative to the tile origin.  For a K-major tile the
// global piece is (mn = r, k = 8c .. 8c+7); for an MN-major one (k = r, mn = c .. c+7).
template <bool KMAJ, int BMN, int BKT>   // BMN: the LDS row pitch (elements) of an MN-major tile
__device__ __forceinline__ void piece(int o, int& r, int& c) {
  if constexpr (KMAJ) {
    r = o / (2 * BKT);
    const int p = (o >> 4) & (BKT / 8 - 1);
    c = 8 * (p ^ swz_k<BKT>(r));
  } else {
    r = o / (2 * BMN);
    const int s = (o % (2 * BMN)) >> 4;
    c = 16 * ((s >> 1) ^ swz_f(r)) + 8 * (s & 1);
  }
}

// Fragment of 16 (m or n) x 32 (k): lane l gets mn = mn0 + l % 16, k = kb + 8*(l / 16) .. +7.
template <bool KMAJ, int BMN, int BKT>
__device__ __forceinline__ bf16x8 frag(const TP_LDS char* tile, int mn0, int kb, int lane) {
  if constexpr (KMAJ) {
    const int r = mn0 + (lane & 15);
    const int c = (kb >> 3) + (lane >> 4);
    return *(const TP_LDS bf16x8*)(tile + r * (2 * BKT) + ((c ^ swz_k<BKT>(r)) << 4));
  } else {
    const int i = lane & 15;
    const int mn = mn0 + 4 * (i & 3);
    const int k1 = kb + 8 * (lane >> 4) + (i >> 2);
    const int k2 = k1 + 4;
    const int p1 = ((((mn >> 4) ^ swz_f(k1)) << 4) | (mn & 15)) * 2;
    const int p2 = ((((mn >> 4) ^ swz_f(k2)) << 4) | (mn & 15)) * 2;
    bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((TP_LDS bf16x4*)(tile + k1 * 2 * BMN + p1));
    bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((TP_LDS bf16x4*)(tile + k2 * 2 * BMN + p2));
    return (bf16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

struct Operand {
  const bf16* p;
  long ld;
  int mn_total;   // extent along m (A) or n (B)
};

// One operand's loads for one k-tile.
// BMN: rows (K-major) or the LDS pitch (MN-major); W: the tile's width along m / n.
template <bool KMAJ, int BMN, int W, int IPW, int BKT>
__device__ __forceinline__ void load_tile(const Operand& op, int mn0, int k0, int K, TP_LDS char* dst,
                                          const int (&r)[IPW], const int (&c)[IPW], int wave) {
  const bf16* base;
  unsigned span;
  if constexpr (KMAJ) {
    base = op.p + (long)mn0 * op.ld + k0;
    span = (unsigned)(((long)(W - 1) * op.ld + BKT) * 2);
  } else {
    base = op.p + (long)k0 * op.ld + mn0;
    span = (unsigned)(((long)(BKT - 1) * op.ld + W) * 2);
  }
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)span, 0x00020000);
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    bool ok;
    unsigned off;
    if constexpr (KMAJ) {
      ok = (mn0 + r[j] < op.mn_total) && (k0 + c[j] < K);
      off = (unsigned)(((long)r[j] * op.ld + c[j]) * 2);
    } else {
      ok = (k0 + r[j] < K) && (c[j] < W) && (mn0 + c[j] < op.mn_total);
      off = (unsigned)(((long)r[j] * op.ld + c[j]) * 2);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (TP_LDS void*)(dst + (wave * IPW + j) * 1024), 16,
                                             ok ? off : OOB, 0, 0, 0);
  }
}

// The K-major A operand with its rows gathered: piece j of this lane reads row ga[j] (an element
// offset into the `bytes`-byte matrix at X, or -1 for a row outside it or past the tile) at k0 + c[j].
template <int IPW>
__device__ __forceinline__ void load_tile_gather(const bf16* X, unsigned bytes, int k0, int K, TP_LDS char* dst,
                                                 const int (&ga)[IPW], const int (&c)[IPW], int wave) {
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, (int)bytes, 0x00020000);
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const bool ok = ga[j] >= 0 && k0 + c[j] < K;
    const unsigned off = ((unsigned)ga[j] + (unsigned)(k0 + c[j])) * 2u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (TP_LDS void*)(dst + (wave * IPW + j) * 1024), 16,
                                             ok ? off : OOB, 0, 0, 0);
  }
}

// The MN-major A operand with its k rows gathered (the weight gradient's Xᵀ over dispatched rows):
// piece j of this lane (k-row k0 + r[j]) reads row src[j] of the `bytes`-byte matrix at X (element
// (m, k) at X[src·lda + m], src = the index array's entry for that k, fetched one k-tile ahead), at
// columns mn0 + c[j]; k past K, an index outside the matrix, or columns past the tile or matrix
// read zeros.
template <int IPW, int W>
__device__ __forceinline__ void load_tile_gather_k(const bf16* X, unsigned bytes, int rows_n, long lda, int mn0,
                                                   int mn_total, int k0, int K, TP_LDS char* dst,
                                                   const int (&src)[IPW], const int (&r)[IPW], const int (&c)[IPW],
                                                   int wave) {
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, (int)bytes, 0x00020000);
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const bool ok = k0 + r[j] < K && src[j] >= 0 && src[j] < rows_n && c[j] < W && mn0 + c[j] < mn_total;
    const unsigned off = (unsigned)(((long)src[j] * lda + mn0 + c[j]) * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (TP_LDS void*)(dst + (wave * IPW + j) * 1024), 16,
                                             ok ? off : OOB, 0, 0, 0);
  }
}

template <int EPI>
__device__ __forceinline__ void epilogue4(const GemmDesc& d, int m, int n, f32x4 v) {
  // four consecutive columns n .. n+3 of row m (N is a multiple of 8, so all four are in range)
  const long o = (long)m * d.ldc + n;
  float a[4] = {v[0], v[1], v[2], v[3]};
  if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU) {
    const bf16x4 b = *(const bf16x4*)((const bf16*)d.bias + n);
    for (int e = 0; e < 4; ++e) a[e] += (float)b[e];
  }
  if constexpr (EPI == EPI_BIAS_GELU) {
    if (d.C2) *(bf16x4*)((bf16*)d.C2 + o) = (bf16x4){(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
    for (int e = 0; e < 4; ++e) a[e] = act_f(a[e], d.act);
  }
  if constexpr (EPI == EPI_DGELU) {
    const bf16x4 x = *(const bf16x4*)((const bf16*)d.aux + (long)m * d.ld_aux + n);
    for (int e = 0; e < 4; ++e) a[e] *= act_grad_f((float)x[e], d.act);
  }
  *(bf16x4*)((bf16*)d.C + o) = (bf16x4){(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
}

// Epilogue of a finished BM x BN tile: the wave's accumulators (wave tile at (wm, wn) inside the tile,
// FM x FN blocks of 16 x 16, lane layout as the MFMA leaves it) with bias / bias+GeLU / GeLU' applied,
// stored to C (and C2).
template <class Cfg, int EPI>
__device__ __forceinline__ void store_tile(const GemmDesc& d, int m0, int n0, TP_LDS char* lds,
                                           f32x4 (&acc)[Cfg::FM][Cfg::FN], int wm, int wn, int wave, int lane) {
  const int r16 = lane & 15, g4 = 4 * (lane >> 4);
  if constexpr (EPI == EPI_F32) {
    // fp32 partials straight from the accumulators: four consecutive columns per lane, 16 bytes
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
      const int m = m0 + wm + 16 * i + r16;
      if (m >= d.M) continue;
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j) {
        const int n = n0 + wn + 16 * j + g4;
        if (n < d.N) *(f32x4*)((float*)d.C + (long)m * d.ldc + n) = acc[i][j];
      }
    }
  } else if constexpr (Cfg::BM * Cfg::BN * 2 <= Cfg::STAGES * Cfg::STAGE) {
    // Staged epilogue: the finished tile goes through LDS (row pitch 2·BN bytes, 16-byte granule q of
    // row r at q ^ (r & XM)) so that each store instruction writes whole rows: 64 lanes x 16 bytes of
    // two to four rows instead of 16-row x 32-byte scraps.  The stores are non-temporal: on the
    // write-bound expert GEMMs (2.15 GB of output rows, read once by the combine) that took the MoE
    // block's forward from 2.17 to 2.09 ms and its backward from 3.46 to 3.40; the dense GEMMs did
    // not change.
    wait_vmcnt<0>();
    float rowdot[Cfg::FM];   // EPI_DGELU_GATE: this lane's part of Σ_n aux2[m, n]·acc[m, n]
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) rowdot[i] = 0.f;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j) {
        const int m = m0 + wm + 16 * i + r16, n = n0 + wn + 16 * j + g4;
        f32x4 a = acc[i][j];
        if constexpr (EPI == EPI_DGELU_GATE) {
          if (m < d.M && n < d.N) {
            const bf16x4 x = *(const bf16x4*)((const bf16*)d.aux + (long)m * d.ld_aux + n);
            const bf16x4 y = *(const bf16x4*)((const bf16*)d.aux2 + (long)m * d.ld_aux2 + n);
            for (int e = 0; e < 4; ++e) rowdot[i] = fmaf((float)y[e], a[e], rowdot[i]);
            const float gr = d.row_scale[m];
            for (int e = 0; e < 4; ++e) a[e] *= gr * act_grad_f((float)x[e], d.act);
          }
        }
        if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU) {
          if (n < d.N) {
            const bf16x4 b = *(const bf16x4*)((const bf16*)d.bias + n);
            for (int e = 0; e < 4; ++e) a[e] += (float)b[e];
          }
        }
        if constexpr (EPI == EPI_DGELU) {
          if (m < d.M && n < d.N) {
            const bf16x4 x = *(const bf16x4*)((const bf16*)d.aux + (long)m * d.ld_aux + n);
            for (int e = 0; e < 4; ++e) a[e] *= act_grad_f((float)x[e], d.act);
          }
        }
        acc[i][j] = a;
      }
    if constexpr (EPI == EPI_DGELU_GATE) {
      // a row's columns in this wave sit in the four lanes r16 + 16q: butterfly over them (every lane
      // ends with the same sum), then the WN waves along n meet in LDS and are added in wave order
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i) {
        rowdot[i] += __shfl_xor(rowdot[i], 16);
        rowdot[i] += __shfl_xor(rowdot[i], 32);
      }
      __syncthreads();              // the k loop is done with the LDS
      TP_LDS float* red = (TP_LDS float*)lds;   // [WN][BM]
      const int wni = wave % Cfg::WN;
      if (lane < 16) {
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i) red[wni * Cfg::BM + wm + 16 * i + r16] = rowdot[i];
      }
      __syncthreads();
      if (wni == 0 && lane < 16) {
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i) {
          const int r = wm + 16 * i + r16;
          if (m0 + r < d.M) {
            float t = red[r];
            for (int w = 1; w < Cfg::WN; ++w) t += red[w * Cfg::BM + r];
            d.row_dot[(long)(n0 / Cfg::BN) * d.rd_stride + m0 + r] = t;
          }
        }
      }
    }
    constexpr int RB = Cfg::BN * 2, NG = Cfg::BN / 8;   // row bytes, 16-byte granules per row
    // the granule swizzle stays inside a row: r & 7 when a row holds a multiple of 8 granules, r & 3
    // for the 224-wide tile's 28
    constexpr int XM = NG % 8 == 0 ? 7 : (NG % 4 == 0 ? 3 : 0);
    auto stage_out = [&](bf16* out, bool gelu) {
      __syncthreads();              // the k loop (or the previous pass) is done with the LDS
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) {
          const int r = wm + 16 * i + r16, c = wn + 16 * j + g4;
          const int ob = ((((c >> 3) ^ (r & XM)) << 4) | ((c & 7) << 1));
          f32x4 a = acc[i][j];
          if (gelu)
            for (int e = 0; e < 4; ++e) a[e] = act_f(a[e], d.act);
          *(TP_LDS bf16x4*)(lds + r * RB + ob) = (bf16x4){(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
        }
      __syncthreads();
      const int tid = wave * 64 + lane;
#pragma unroll 4
      for (int c = tid; c < Cfg::BM * NG; c += Cfg::NT) {
        const int r = c / NG, q = c % NG;
        const int m = m0 + r, n = n0 + 8 * q;
        if (m < d.M && n < d.N)   // streaming store: output tiles are written once, not re-read here
          __builtin_nontemporal_store(*(const TP_LDS bf16x8*)(lds + r * RB + ((q ^ (r & XM)) << 4)),
                                      (bf16x8*)(out + (long)m * d.ldc + n));
      }
    };
    if constexpr (EPI == EPI_BIAS_GELU) {
      if (d.C2) stage_out((bf16*)d.C2, false);
      stage_out((bf16*)d.C, true);
    } else {
      stage_out((bf16*)d.C, false);
    }
  } else {
    static_assert(EPI != EPI_DGELU_GATE, "the gated epilogue takes the LDS-staged path");
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
      const int m = m0 + wm + 16 * i + r16;
      if (m >= d.M) continue;
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j) {
        const int n = n0 + wn + 16 * j + g4;
        if (n < d.N) epilogue4<EPI>(d, m, n, acc[i][j]);
      }
    }
  }
}

// One BM x BN output tile at (m0, n0): the k loop over LDS stages and the fused epilogue.
template <class Cfg, bool AK, bool BK, int EPI, bool GATHER = false, bool GATHER_K = false, bool GATHER_KB = false>
__device__ __forceinline__ void gemm_tile(const GemmDesc& d, int m0, int n0, TP_LDS char* lds, int wave,
                                          int lane, int rot = 0) {
  static_assert(!GATHER || AK, "rows are gathered for a K-major A only");
  static_assert(!GATHER_K || (!AK && !GATHER && Cfg::STAGES == 2), "k rows are gathered for an MN-major A, 2 stages");
  static_assert(!GATHER_KB || (!BK && Cfg::STAGES == 2), "k rows are gathered for an MN-major B, 2 stages");
  constexpr int LA = AK ? Cfg::BM : Cfg::PM, LB = BK ? Cfg::BN : Cfg::PN;   // rows or pitch
  constexpr int A_BYTES = Cfg::template bytes<AK, Cfg::BM>(), B_BYTES = Cfg::template bytes<BK, Cfg::BN>();
  constexpr int IPW_A = A_BYTES / 1024 / Cfg::NW, IPW_B = B_BYTES / 1024 / Cfg::NW;   // loads per wave
  static_assert(A_BYTES % (1024 * Cfg::NW) == 0 && B_BYTES % (1024 * Cfg::NW) == 0, "loads must split evenly");
  const Operand A{(const bf16*)d.A, d.lda, d.M};
  const Operand B{(const bf16*)d.B, d.ldb, d.N};
  int ar[IPW_A], ac[IPW_A], br[IPW_B], bc[IPW_B];
#pragma unroll
  for (int j = 0; j < IPW_A; ++j) piece<AK, LA, Cfg::BKT>((wave * IPW_A + j) * 1024 + 16 * lane, ar[j], ac[j]);
#pragma unroll
  for (int j = 0; j < IPW_B; ++j) piece<BK, LB, Cfg::BKT>((wave * IPW_B + j) * 1024 + 16 * lane, br[j], bc[j]);

  int ga[IPW_A];   // gathered A: element offset of each piece's source row, -1 outside
  unsigned gbytes = 0;
  if constexpr (GATHER) {
    gbytes = (unsigned)((long)d.a_rows_n * d.lda * 2);
#pragma unroll
    for (int j = 0; j < IPW_A; ++j) {
      const int m = m0 + ar[j];
      const int src = m < d.M ? d.a_rows[m] : -1;
      ga[j] = (src >= 0 && src < d.a_rows_n) ? src * (int)d.lda : -1;
    }
  }
  // k-gathered A: the source rows of the next k-tile to load, fetched one tile ahead.  The loads are
  // unconditional (k clamped into [0, K), K >= 1 whenever a tile is loaded) and their values are
  // first used when that tile's loads are issued, so no wait is placed right after the fetch; the
  // k-range check happens there too.
  int gk[IPW_A];
  if constexpr (GATHER_K) gbytes = (unsigned)((long)d.a_rows_n * d.lda * 2);
  auto fetch_k = [&](int k) {
#pragma unroll
    for (int j = 0; j < IPW_A; ++j) gk[j] = d.a_rows[min(k + ar[j], d.K - 1)];
  };
  // k-gathered B: as for A, the source rows of the next k-tile, fetched one tile ahead
  int gkb[IPW_B];
  unsigned gbytes_b = 0;
  if constexpr (GATHER_KB) gbytes_b = (unsigned)((long)d.b_rows_n * d.ldb * 2);
  auto fetch_kb = [&](int k) {
#pragma unroll
    for (int j = 0; j < IPW_B; ++j) gkb[j] = d.b_rows[min(k + br[j], d.K - 1)];
  };
  auto load_b = [&](int k, TP_LDS char* dst) {
    if constexpr (GATHER_KB)
      load_tile_gather_k<IPW_B, Cfg::BN>((const bf16*)d.B, gbytes_b, d.b_rows_n, d.ldb, n0, d.N, k, d.K, dst, gkb,
                                         br, bc, wave);
    else load_tile<BK, LB, Cfg::BN, IPW_B, Cfg::BKT>(B, n0, k, d.K, dst, br, bc, wave);
  };
  auto load_a = [&](int k, TP_LDS char* dst) {
    if constexpr (GATHER) load_tile_gather<IPW_A>((const bf16*)d.A, gbytes, k, d.K, dst, ga, ac, wave);
    else if constexpr (GATHER_K)
      load_tile_gather_k<IPW_A, Cfg::BM>((const bf16*)d.A, gbytes, d.a_rows_n, d.lda, m0, d.M, k, d.K, dst, gk, ar,
                                         ac, wave);
    else load_tile<AK, LA, Cfg::BM, IPW_A, Cfg::BKT>(A, m0, k, d.K, dst, ar, ac, wave);
  };

  const int wm = (wave / Cfg::WN) * Cfg::TM, wn = (wave % Cfg::WN) * Cfg::TN;
  f32x4 acc[Cfg::FM][Cfg::FN];
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  constexpr int BKT = Cfg::BKT, NKK = BKT / 32;
  constexpr bool EARLY = !(AK && BK);
  const int nk = (d.K + BKT - 1) / BKT;
  // k-tiles are visited starting at tile `rot` (mod nk); the sum over k is the same, only its order
  // differs between tiles that use different starting points
  rot = (nk > 0 && nk >= TP_GEMM_ROT_MIN_NK) ? rot % nk : 0;
  auto kpos = [&](int t) { const int i = t + rot; return (i >= nk ? i - nk : i) * BKT; };
  // prologue: tiles 0 .. STAGES-2 in flight
  if constexpr (GATHER_K) {
    if (nk > 0) fetch_k(kpos(0));
  }
  if constexpr (GATHER_KB) {
    if (nk > 0) fetch_kb(kpos(0));
  }
#pragma unroll
  for (int t = 0; t < Cfg::STAGES - 1; ++t)
    if (t < nk) {
      load_a(kpos(t), lds + t * Cfg::STAGE);
      load_b(kpos(t), lds + t * Cfg::STAGE + A_BYTES);
    }
  if constexpr (GATHER_K) {
    if (nk > 1) fetch_k(kpos(1));
  }
  if constexpr (GATHER_KB) {
    if (nk > 1) fetch_kb(kpos(1));
  }
  int cur_stage = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // tile kt has landed once at most the loads of the STAGES-2 younger tiles are outstanding
    if (kt + Cfg::STAGES - 2 < nk) wait_vmcnt<(Cfg::STAGES - 2) * (IPW_A + IPW_B)>();
    else wait_vmcnt<0>();
    __syncthreads();   // every wave's part of tile kt is in LDS; the stage loaded next is free
    const TP_LDS char* at = lds + cur_stage * Cfg::STAGE;
    const TP_LDS char* bt = at + A_BYTES;
    bf16x8 af[NKK][Cfg::FM], bfr[NKK][Cfg::FN];
    // With an MN-major operand (transposed LDS reads), reading every fragment of the tile before
    // issuing the next tile's loads keeps the LDS reads off the critical path after the barrier;
    // with two K-major operands the plain order is faster (measured).
    if constexpr (EARLY) {
#pragma unroll
      for (int q = 0; q < NKK; ++q) {
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i) af[q][i] = frag<AK, LA, Cfg::BKT>(at, wm + 16 * i, 32 * q, lane);
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) bfr[q][j] = frag<BK, LB, Cfg::BKT>(bt, wn + 16 * j, 32 * q, lane);
      }
    }
    if (kt + Cfg::STAGES - 1 < nk) {
      int ns = cur_stage + Cfg::STAGES - 1;
      if (ns >= Cfg::STAGES) ns -= Cfg::STAGES;
      TP_LDS char* nxt = lds + ns * Cfg::STAGE;
      const int k1 = kpos(kt + Cfg::STAGES - 1);
      load_a(k1, nxt);
      load_b(k1, nxt + A_BYTES);
      if constexpr (GATHER_K) {
        if (kt + 2 < nk) fetch_k(kpos(kt + 2));
      }
      if constexpr (GATHER_KB) {
        if (kt + 2 < nk) fetch_kb(kpos(kt + 2));
      }
    }
#pragma unroll
    for (int q = 0; q < NKK; ++q) {
      if constexpr (!EARLY) {
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i) af[q][i] = frag<AK, LA, Cfg::BKT>(at, wm + 16 * i, 32 * q, lane);
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) bfr[q][j] = frag<BK, LB, Cfg::BKT>(bt, wn + 16 * j, 32 * q, lane);
      }
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = mfma_16x16x32_bf16(bfr[q][j], af[q][i], acc[i][j]);
    }
    if (++cur_stage == Cfg::STAGES) cur_stage = 0;
  }

  store_tile<Cfg, EPI>(d, m0, n0, lds, acc, wm, wn, wave, lane);
}

template <class Cfg, bool AK, bool BK, int EPI>
__global__ __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(Cfg::OCC, Cfg::OCC)))
void gemm_bf16_kernel(GemmDesc d, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) char smem[Cfg::STAGES * Cfg::STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS targets in SGPRs

  // Workgroups are dispatched round-robin over the 8 XCDs; renumber so that each XCD owns a
  // contiguous run of tiles, then walk that run in groups of GROUP_M tile rows x all tile columns
  // (column-major inside a group): the tiles an XCD runs at once form a compact block, so both their
  // A row panels and B column panels are shared in that XCD's L2.
  constexpr int GROUP_M = 4;
  // split-k (fp32 partials, both operands MN-major): the grid holds ksplit copies of the tile set
  const int ks = (EPI == EPI_F32 && d.ksplit > 1) ? d.ksplit : 1;
  const int tiles = tiles_m * tiles_n, nwg = tiles * ks;
  int wg = blockIdx.x;
  if (nwg % 8 == 0) wg = (wg % 8) * (nwg / 8) + wg / 8;
  const int slice = wg / tiles;
  wg -= slice * tiles;
  const int per_group = GROUP_M * tiles_n;
  const int first_m = (wg / per_group) * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (wg % per_group) % gsize, tn = (wg % per_group) / gsize;
  const int m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;
  // Tiles that run together begin their k loops at different k-tiles, so that their concurrent
  // loads of strided operand rows fall on different memory channels (measured: 2-4% per GEMM) —
  // except the whole-k Xᵀ·dY weight gradients, which measured 1-2% faster with every tile starting
  // at k-tile 0 (their k-tiles are whole 512-byte row pieces, and the tiles sharing a panel then
  // read the same k-tile at about the same time).
  if constexpr (EPI == EPI_F32) {
    static_assert(!AK && !BK, "the plain kernel's split-k takes two MN-major operands");
    GemmDesc ds = d;
    if (ks > 1) {   // slice s: k rows [s·k_per, min(K, (s+1)·k_per)) of both operands
      const int k0 = slice * d.k_per;
      ds.A = (const bf16*)d.A + (long)k0 * d.lda;
      ds.B = (const bf16*)d.B + (long)k0 * d.ldb;
      ds.K = max(0, min(d.k_per, d.K - k0));
      ds.C = (float*)d.C + slice * d.c_split;
    }
    gemm_tile<Cfg, AK, BK, EPI>(ds, m0, n0, (TP_LDS char*)smem, wave, lane, tm + tn);
  } else {
    gemm_tile<Cfg, AK, BK, EPI>(d, m0, n0, (TP_LDS char*)smem, wave, lane, (!AK && !BK) ? 0 : tm + tn);
  }
}

// Ping-pong schedule on a 256 x 192 tile (k = 64 per tile, two LDS stages, 512 threads).  The eight
// waves form two groups of four, group g = waves 4g .. 4g+3, so each SIMD holds one wave of each
// group.  Group g owns output rows [128g, 128g + 128) of the tile (a 2 x 2 arrangement of 64 x 96 wave
// tiles).  Every wave alternates a memory phase (issue its share of the next k-tile's global -> LDS
// loads, read all of its fragments of the current k-tile from LDS) and a compute phase (the k-tile's
// MFMAs), and group 1 runs one phase behind group 0: while one wave of a SIMD multiplies, the other
// reads LDS, so the matrix core is not left idle during the fragment reads.  All eight waves meet at
// every phase boundary (s_barrier), which keeps the two groups exactly one phase apart.
//
// Tile t sits in stage t & 1.  Its B part and the rows of A group 0 uses are loaded by group 0 during
// its memory phase of tile t-1 (after that phase's fragment reads); the rows group 1 uses by group 1
// during its memory phase of tile t-1.
// Each group waits for its own loads at the end of its following compute phase, so every load has two
// phases to land, and a stage is only overwritten after both groups' reads of it have completed (the
// memory phase ends with lgkmcnt(0) before its barrier).
// The tile width BN is 192 (the dense GEMMs), 160 or 224 (dense GEMMs whose n extent they cover in
// fewer or fuller rounds of 256 tiles) or 256 (the grouped expert GEMMs, whose n extent is one 256-wide
// shard): wave tiles of 64 x 96, 64 x 80, 64 x 112 or 64 x 128.
template <int BN_>
struct PPCfg {
  static constexpr int BM = 256, BN = BN_, BKT = 64, NKK = 2, NT = 512, STAGES = 2;
  static constexpr int HALF = 128;                        // A rows per group
  static constexpr int WN = 2;                            // wave columns (per group: 2 x 2 waves)
  static constexpr int OCC = 2;                           // waves per SIMD (one of each group)
  static constexpr int FM = 4, FN = BN / 32;              // 64 x BN/2 per wave
  static constexpr int A_HALF = HALF * BKT * 2;           // 16 KiB (either layout: pitch 128)
  static constexpr int B_OFF = 2 * A_HALF;
  static constexpr int STAGE = B_OFF + 256 * BKT * 2;     // B: BN rows (K-major) or pitch 256 (MN-major)
  static_assert(BN == 160 || BN == 192 || BN == 224 || BN == 256, "tile widths");
};
using PPTile = PPCfg<192>;

// Phase boundaries: every wave's LDS reads (lgkmcnt) or its global -> LDS loads (vmcnt) complete, then
// all waves of the workgroup meet.  The waits are the s_waitcnt builtin, which the compiler's own wait
// placement takes into account (a wait it cannot see makes it wait again later, on younger loads);
// sched_barrier keeps the compiler from moving MFMAs or memory operations across the boundary.
__device__ __forceinline__ void pp_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void pp_sync_lds() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0) alone
  pp_barrier();
}
__device__ __forceinline__ void pp_sync_vm() {
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<0>();
  pp_barrier();
}
__device__ __forceinline__ void pp_sync() { pp_barrier(); }

template <class P, bool AK, bool BK, int EPI, bool GATHER = false>
__device__ __forceinline__ void gemm_tile_pp(const GemmDesc& d, int m0, int n0, TP_LDS char* lds, int wave,
                                             int lane, int rot) {
  static_assert(!GATHER || AK, "rows are gathered for a K-major A only");
  constexpr int LB = BK ? P::BN : 256;                        // B rows (K-major) or pitch (MN-major)
  constexpr int B_BYTES = BK ? P::BN * P::BKT * 2 : 256 * P::BKT * 2;
  constexpr int IPW_A = P::A_HALF / 1024 / 4, IPW_B = B_BYTES / 1024 / 4;   // loads per wave of a group
  static_assert(B_BYTES % 4096 == 0 && P::STAGES * P::STAGE <= 160 * 1024, "tile layout");
  const int g = wave >> 2, w4 = wave & 3;                     // wave-uniform
  const Operand A{(const bf16*)d.A, d.lda, d.M};
  const Operand B{(const bf16*)d.B, d.ldb, d.N};
  int ar[IPW_A], ac[IPW_A], br[IPW_B], bc[IPW_B];
#pragma unroll
  for (int j = 0; j < IPW_A; ++j) piece<AK, P::HALF, P::BKT>((w4 * IPW_A + j) * 1024 + 16 * lane, ar[j], ac[j]);
#pragma unroll
  for (int j = 0; j < IPW_B; ++j) piece<BK, LB, P::BKT>((w4 * IPW_B + j) * 1024 + 16 * lane, br[j], bc[j]);
  // gathered A: element offset of each piece's source row (rows of this group's half), -1 outside
  int ga[IPW_A];
  unsigned gbytes = 0;
  if constexpr (GATHER) {
    gbytes = (unsigned)((long)d.a_rows_n * d.lda * 2);
#pragma unroll
    for (int j = 0; j < IPW_A; ++j) {
      const int m = m0 + P::HALF * g + ar[j];
      const int src = m < d.M ? d.a_rows[m] : -1;
      ga[j] = (src >= 0 && src < d.a_rows_n) ? src * (int)d.lda : -1;
    }
  }

  const int nk = (d.K + P::BKT - 1) / P::BKT;
  rot = (nk > 0 && nk >= TP_GEMM_ROT_MIN_NK) ? rot % nk : 0;
  auto kpos = [&](int t) { const int i = t + rot; return (i >= nk ? i - nk : i) * P::BKT; };
  // this wave's share of k-tile t's loads into stage st
  auto issue = [&](int t, int st) {
    TP_LDS char* base = lds + st * P::STAGE;
    const int k = kpos(t);
    if constexpr (GATHER) load_tile_gather<IPW_A>((const bf16*)d.A, gbytes, k, d.K, base + g * P::A_HALF, ga, ac, w4);
    else load_tile<AK, P::HALF, P::HALF, IPW_A, P::BKT>(A, m0 + P::HALF * g, k, d.K, base + g * P::A_HALF, ar, ac, w4);
    if (g == 0) load_tile<BK, LB, P::BN, IPW_B, P::BKT>(B, n0, k, d.K, base + P::B_OFF, br, bc, w4);
  };

  const int wml = (w4 >> 1) * 64, wn = (w4 & 1) * (P::BN / 2);   // wave tile inside the group's rows
  f32x4 acc[P::FM][P::FN];
#pragma unroll
  for (int i = 0; i < P::FM; ++i)
#pragma unroll
    for (int j = 0; j < P::FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  if (nk > 0) issue(0, 0);
  pp_sync_vm();                  // k-tile 0 is in stage 0
  if (g == 1) pp_sync();         // group 1 starts one phase behind
  for (int t = 0; t < nk; ++t) {
    const int st = t & 1;
    // memory phase: every fragment of this k-tile, then the next k-tile's loads (after the reads: the
    // compiler would otherwise wait for those loads before the transposed LDS reads, which it cannot
    // tell apart from the loads' LDS destination)
    const TP_LDS char* at = lds + st * P::STAGE + g * P::A_HALF;
    const TP_LDS char* bt = lds + st * P::STAGE + P::B_OFF;
    bf16x8 af[P::NKK][P::FM], bfr[P::NKK][P::FN];
#pragma unroll
    for (int q = 0; q < P::NKK; ++q) {
#pragma unroll
      for (int i = 0; i < P::FM; ++i) af[q][i] = frag<AK, P::HALF, P::BKT>(at, wml + 16 * i, 32 * q, lane);
#pragma unroll
      for (int j = 0; j < P::FN; ++j) bfr[q][j] = frag<BK, LB, P::BKT>(bt, wn + 16 * j, 32 * q, lane);
    }
    if (t + 1 < nk) issue(t + 1, st ^ 1);
    pp_sync_lds();
    // compute phase
#pragma unroll
    for (int q = 0; q < P::NKK; ++q)
#pragma unroll
      for (int i = 0; i < P::FM; ++i)
#pragma unroll
        for (int j = 0; j < P::FN; ++j) acc[i][j] = mfma_16x16x32_bf16(bfr[q][j], af[q][i], acc[i][j]);
    pp_sync_vm();
  }
  if (g == 0) pp_sync();         // both groups have passed the same number of barriers
  store_tile<P, EPI>(d, m0, n0, lds, acc, P::HALF * g + wml, wn, wave, lane);
}

template <int BN, bool AK, bool BK, int EPI>
__global__ __launch_bounds__(PPCfg<BN>::NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_pp_kernel(GemmDesc d, int tiles_m, int tiles_n) {
  using PPTile = PPCfg<BN>;
  __shared__ __attribute__((aligned(1024))) char smem[PPTile::STAGES * PPTile::STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup -> tile order as in gemm_bf16_kernel (contiguous runs per XCD, groups of 4 tile rows)
  constexpr int GROUP_M = 4;
  // split-k: the grid holds ksplit copies of the tile set, copy s on k-slice s (both operands K-major)
  const int ks = (EPI == EPI_F32 && d.ksplit > 1) ? d.ksplit : 1;
  const int tiles = tiles_m * tiles_n, nwg = tiles * ks;
  int wg = blockIdx.x;
  if (nwg % 8 == 0) wg = (wg % 8) * (nwg / 8) + wg / 8;
  const int slice = wg / tiles;
  wg -= slice * tiles;
  const int per_group = GROUP_M * tiles_n;
  const int first_m = (wg / per_group) * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (wg % per_group) % gsize, tn = (wg % per_group) / gsize;
  if constexpr (EPI == EPI_F32) {
    static_assert(AK && BK, "split-k takes two K-major operands");
    GemmDesc ds = d;
    if (ks > 1) {
      const int k0 = slice * d.k_per;
      ds.A = (const bf16*)d.A + k0;
      ds.B = (const bf16*)d.B + k0;
      ds.K = max(0, min(d.k_per, d.K - k0));
      ds.C = (float*)d.C + slice * d.c_split;
    }
    gemm_tile_pp<PPTile, AK, BK, EPI>(ds, tm * PPTile::BM, tn * PPTile::BN, (TP_LDS char*)smem, wave, lane, tm + tn);
  } else {
    gemm_tile_pp<PPTile, AK, BK, EPI>(d, tm * PPTile::BM, tn * PPTile::BN, (TP_LDS char*)smem, wave, lane, tm + tn);
  }
}

// Grouped GEMM: expert e owns rows [off[e], off[e+1]) of A and C and its own B (and bias), at
// b_stride (bias_stride) elements from expert e-1's.  prefix[e] = Σ_{j<e} ceil(rows_j / BM) (from
// grouped_plan_kernel) numbers the m-tiles of all experts.  The tiles are numbered expert by expert
// (expert e: slots [prefix[e]·tiles_n, prefix[e+1]·tiles_n), m-tile fastest inside it), and each XCD
// takes one contiguous eighth of that numbering: the workgroups an XCD runs together then share
// one expert's weights and a few row tiles in its L2, instead of every XCD fetching every expert.
// The 1-D grid holds 8·ceil(max_tiles / 8) workgroups; those past the real tile count return.
struct GroupedArgs {
  GemmDesc d;          // A, B, C, C2, bias, lda, ldb, ldc, N, K, epi; M unused
  const int* off;      // [groups + 1] row offsets (device)
  const int* prefix;   // [groups + 1] m-tile prefix (device workspace)
  const int* tile_expert;   // [prefix[groups]] the expert of each m-tile (device workspace)
  int groups;
  long b_stride, bias_stride;
};


template <class Cfg, int EPI, bool GATHER, bool BKM, bool PP = false>
__global__ __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(Cfg::OCC, Cfg::OCC)))
void gemm_bf16_grouped_kernel(GroupedArgs g) {
  __shared__ __attribute__((aligned(1024))) char smem[Cfg::STAGES * Cfg::STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // The plan's values are the same for every lane: readfirstlane keeps them (and the operand
  // addresses made from them) in scalar registers.  Left to the compiler, a per-lane value can
  // reach a buffer descriptor, which then costs a loop over lanes around every load.
  const auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  const int tiles_n = (g.d.N + Cfg::BN - 1) / Cfg::BN;
  const long total = (long)uni(g.prefix[g.groups]) * tiles_n;
  const long chunk = (total + 7) / 8;
  const long slot = blockIdx.x / 8;
  if (slot >= chunk) return;
  const long lin = (long)(blockIdx.x % 8) * chunk + slot;
  if (lin >= total) return;
  // expert e's slots [prefix[e]·tiles_n, prefix[e+1]·tiles_n) hold exactly the lin whose m-tile index
  // lin / tiles_n lies in [prefix[e], prefix[e+1])
  const int e = uni(g.tile_expert[lin / tiles_n]);
  const int p0 = uni(g.prefix[e]), p1 = uni(g.prefix[e + 1]);
  const int cnt = p1 - p0;                           // >= 1: lin falls inside expert e's slots
  const long local = lin - (long)p0 * tiles_n;
  const int mt = uni(p0 + (int)(local % cnt)), nt = uni((int)(local / cnt));   // (divided on the vector unit)
  const int row0 = uni(g.off[e]) + (mt - p0) * Cfg::BM;
  GemmDesc d = g.d;
  d.M = uni(g.off[e + 1]) - row0;      // rows of this expert from row0 on (>= 1)
  if constexpr (GATHER) d.a_rows = g.d.a_rows + row0;   // A stays the whole gathered-from matrix
  else d.A = (const bf16*)g.d.A + (long)row0 * g.d.lda;
  d.B = (const bf16*)g.d.B + (long)e * g.b_stride;
  d.C = (bf16*)g.d.C + (long)row0 * g.d.ldc;
  if (g.d.C2) d.C2 = (bf16*)g.d.C2 + (long)row0 * g.d.ldc;
  if (g.d.bias) d.bias = (const bf16*)g.d.bias + (long)e * g.bias_stride;
  if (g.d.aux) d.aux = (const bf16*)g.d.aux + (long)row0 * g.d.ld_aux;
  if constexpr (EPI == EPI_DGELU_GATE) {
    d.aux2 = (const bf16*)g.d.aux2 + (long)row0 * g.d.ld_aux2;
    d.row_scale = g.d.row_scale + row0;
    d.row_dot = g.d.row_dot + row0;
  }
  // k loops start at k-tile mt (mod the count): the row tiles of the same expert stream their rows
  // of A through different memory channels at the same moment (measured: fc1 2x faster)
  if constexpr (PP) gemm_tile_pp<Cfg, true, BKM, EPI, GATHER>(d, 0, nt * Cfg::BN, (TP_LDS char*)smem, wave, lane, mt);
  else gemm_tile<Cfg, true, BKM, EPI, GATHER>(d, 0, nt * Cfg::BN, (TP_LDS char*)smem, wave, lane, mt);
}

// Grouped weight-gradient GEMM: expert e's block C_e [M, N] (at e·c_stride elements) = op(A_e)·op(B_e)
// where A_e and B_e are the rows [off[e], off[e+1]) of two row-major matrices, both read MN-major
// (A element (m, k) at A[(off[e] + k)·lda + m], B element (k, n) at B[(off[e] + k)·ldb + n]): the
// experts split the k dimension, so an expert without rows gets a zero block.  The loads mask rows
// past the expert's count, so K needs no alignment.  One workgroup per (expert, m-tile, n-tile),
// numbered expert-major and handed out in contiguous runs per XCD as in the plain kernel: the
// tiles an XCD runs together share one expert's rows in its L2.
struct GroupedKArgs {
  GemmDesc d;          // A, B, C, lda, ldb, ldc, M, N; K unused
  const int* off;      // [groups + 1] sanitised row offsets (device)
  int groups;
  long c_stride;
};

template <class Cfg, bool GK, bool GKB>
__global__ __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(Cfg::OCC, Cfg::OCC)))
void gemm_bf16_grouped_k_kernel(GroupedKArgs g, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) char smem[Cfg::STAGES * Cfg::STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long per = (long)tiles_m * tiles_n, nwg = per * g.groups;
  long wg = blockIdx.x;
  if (nwg % 8 == 0) wg = (wg % 8) * (nwg / 8) + wg / 8;
  const int e = (int)(wg / per);
  const int local = (int)(wg % per);
  const int tm = local % tiles_m, tn = local / tiles_m;
  GemmDesc d = g.d;
  const int k0 = __builtin_amdgcn_readfirstlane(g.off[e]);   // uniform: scalar operand addresses
  d.K = __builtin_amdgcn_readfirstlane(g.off[e + 1]) - k0;
  if constexpr (GK) d.a_rows = g.d.a_rows + k0;   // A stays the whole gathered-from matrix
  else d.A = (const bf16*)g.d.A + (long)k0 * g.d.lda;
  if constexpr (GKB) d.b_rows = g.d.b_rows + k0;  // B likewise
  else d.B = (const bf16*)g.d.B + (long)k0 * g.d.ldb;
  d.C = (bf16*)g.d.C + (long)e * g.c_stride;
  gemm_tile<Cfg, false, false, EPI_STORE, false, GK, GKB>(d, tm * Cfg::BM, tn * Cfg::BN, (TP_LDS char*)smem, wave,
                                                           lane, tm + tn);
}

template <class Cfg, bool AK, bool BK, int EPI>
hipError_t run(const GemmDesc& d, hipStream_t s) {
  const int tiles_m = (d.M + Cfg::BM - 1) / Cfg::BM, tiles_n = (d.N + Cfg::BN - 1) / Cfg::BN;
  const int ks = (EPI == EPI_F32 && d.ksplit > 1) ? d.ksplit : 1;
  gemm_bf16_kernel<Cfg, AK, BK, EPI><<<tiles_m * tiles_n * ks, Cfg::NT, 0, s>>>(d, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int BN, bool AK, bool BK, int EPI>
hipError_t run_pp(const GemmDesc& d, hipStream_t s) {
  using PPTile = PPCfg<BN>;
  const int tiles_m = (d.M + PPTile::BM - 1) / PPTile::BM, tiles_n = (d.N + PPTile::BN - 1) / PPTile::BN;
  const int ks = (EPI == EPI_F32 && d.ksplit > 1) ? d.ksplit : 1;
  gemm_bf16_pp_kernel<BN, AK, BK, EPI><<<tiles_m * tiles_n * ks, PPTile::NT, 0, s>>>(d, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int BN>
hipError_t run_pp_cfg(const GemmDesc& d, hipStream_t s) {
  if (d.a_kmajor && !d.b_kmajor) {
    if (d.epi == EPI_BIAS) return run_pp<BN, true, false, EPI_BIAS>(d, s);
    if (d.epi == EPI_BIAS_GELU) return run_pp<BN, true, false, EPI_BIAS_GELU>(d, s);
    if (d.epi == EPI_STORE) return run_pp<BN, true, false, EPI_STORE>(d, s);
  } else if (d.a_kmajor && d.b_kmajor) {
    if (d.epi == EPI_DGELU) return run_pp<BN, true, true, EPI_DGELU>(d, s);
    if (d.epi == EPI_STORE) return run_pp<BN, true, true, EPI_STORE>(d, s);
    if constexpr (BN == 192)   // the split-k partials take the 192-wide tile only
      if (d.epi == EPI_F32) return run_pp<BN, true, true, EPI_F32>(d, s);
  }
  // Xᵀ·dY (both operands MN-major) is not taken: two operands of transposed LDS reads make the memory
  // phase longer than the compute phase (measured 15% slower than the plain 256 x 192 kernel)
  return hipErrorNotSupported;
}

template <class Cfg>
hipError_t run_cfg(const GemmDesc& d, hipStream_t s) {
  // the layouts and epilogues the shard uses: X·W (A K-major, B MN-major) with bias / bias+GeLU /
  // none; dY·Wᵀ (both K-major) with GeLU' / none; Xᵀ·dY (both MN-major) with none.
  if (d.a_kmajor && !d.b_kmajor) {
    if (d.epi == EPI_BIAS) return run<Cfg, true, false, EPI_BIAS>(d, s);
    if (d.epi == EPI_BIAS_GELU) return run<Cfg, true, false, EPI_BIAS_GELU>(d, s);
    if (d.epi == EPI_STORE) return run<Cfg, true, false, EPI_STORE>(d, s);
  } else if (d.a_kmajor && d.b_kmajor) {
    if (d.epi == EPI_DGELU) return run<Cfg, true, true, EPI_DGELU>(d, s);
    if (d.epi == EPI_STORE) return run<Cfg, true, true, EPI_STORE>(d, s);
  } else if (!d.a_kmajor && !d.b_kmajor) {
    if (d.epi == EPI_STORE) return run<Cfg, false, false, EPI_STORE>(d, s);
  }
  return hipErrorNotSupported;
}

// Tile configurations (BM, BN, waves along m, waves along n, LDS stages).  Eight waves = two per
// SIMD, so one wave's LDS reads overlap the other's MFMAs.
using C0 = Tile<256, 256, 4, 2, 2>;   // 64x128 per wave
using C1 = Tile<256, 128, 2, 4, 3>;   // 128x32 per wave
using C2 = Tile<128, 256, 4, 2, 3>;   // 32x128 per wave
using C3 = Tile<128, 128, 2, 4, 3>;   // 64x32 per wave
using C4 = Tile<256, 256, 4, 2, 3, 32>;
using C5 = Tile<256, 256, 4, 2, 4, 32>;
using C6 = Tile<256, 256, 4, 2, 5, 32>;
using C7 = Tile<256, 256, 2, 2, 2, 64>;   // 1 wave / SIMD, 128x128 per wave
using C8 = Tile<256, 192, 4, 2, 2, 64>;   // 2 waves / SIMD, 64x96 per wave
using C9 = Tile<256, 256, 4, 2, 2, 32>;   // the gathered weight gradient: k = 32 frees the registers
                                          // its row indices take (no spills; 14% faster than C0)
// 9, 10, 11: the ping-pong kernel (gemm_bf16_pp_kernel) on 256 x 192, 256 x 224 and 256 x 160 tiles
constexpr int kTileM[] = {256, 256, 128, 128, 256, 256, 256, 256, 256, 256, 256, 256};
constexpr int kTileN[] = {256, 128, 256, 128, 256, 256, 256, 256, 192, 192, 224, 160};
// relative throughput per CU of each configuration on large shapes (measured on MI355X)
constexpr double kTileRate[] = {1.0, 0.70, 0.70, 0.50, 1.0, 1.0, 1.0, 1.0, 0.95, 1.2, 1.2, 1.04};
constexpr const char* kTileName[] = {"256x256", "256x128", "128x256", "128x128", "256x256k32s3",
                                     "256x256k32s4", "256x256k32s5", "256x256w4", "256x192", "256x192pp",
                                     "256x224pp", "256x160pp"};

}  // namespace

// Whether the tiled kernel takes this GEMM (else the generic one runs).
bool gemm_bf16_eligible(const GemmDesc& d) {
  if (d.dtype != DT_BF16 || d.M <= 0 || d.N <= 0 || d.K <= 0) return false;
  if ((d.M | d.N | d.K) & 7) return false;
  if ((d.lda | d.ldb | d.ldc) & 7) return false;
  if (d.lda > (1L << 22) || d.ldb > (1L << 22)) return false;
  if ((((uintptr_t)d.A) | ((uintptr_t)d.B) | ((uintptr_t)d.C)) & 15) return false;
  if (d.epi == EPI_BIAS_GELU && d.C2 && (((uintptr_t)d.C2) & 15)) return false;
  if ((d.epi == EPI_DGELU || d.epi == EPI_DGELU_GATE) && ((d.ld_aux & 7) || (((uintptr_t)d.aux) & 15))) return false;
  if (d.epi == EPI_DGELU_GATE && ((d.ld_aux2 & 7) || (((uintptr_t)d.aux2) & 15) || !d.row_scale || !d.row_dot))
    return false;
  if (d.epi == EPI_F32)   // split-k partials: both operands K-major (the ping-pong tile) or both MN-major
    return d.a_kmajor == d.b_kmajor && ((d.ldc & 3) == 0) &&   // (the 256 x 256 tile), whole k-tiles per slice
           (d.ksplit <= 1 || (d.k_per > 0 && d.k_per % 64 == 0 && (long)d.k_per * d.ksplit >= d.K));
  const bool supported = (d.a_kmajor && !d.b_kmajor && (d.epi == EPI_BIAS || d.epi == EPI_BIAS_GELU || d.epi == EPI_STORE)) ||
                         (d.a_kmajor && d.b_kmajor && (d.epi == EPI_DGELU || d.epi == EPI_STORE || d.epi == EPI_DGELU_GATE)) ||
                         (!d.a_kmajor && !d.b_kmajor && d.epi == EPI_STORE);
  return supported;
}

// The k-split weight gradients (both operands MN-major, fp32 partials per slice): 256 x 256 (index 0,
// rate 1.1 on this layout) or 256 x 192 (index 8, rate 0.95), by rounds of 256 tiles x tile area / rate.
int gemm_bf16_wgrad_tile(int M, int N, int ks) {
  const long t0 = (long)((M + 255) / 256) * ((N + 255) / 256) * ks, t8 = (long)((M + 255) / 256) * ((N + 191) / 192) * ks;
  const double e0 = (double)((t0 + 255) / 256) * 65536 / 1.1, e8 = (double)((t8 + 255) / 256) * 49152 / 0.95;
  return e8 < e0 * 0.999 ? 8 : 0;
}

// Tile choice by a small cost model.  A build may pin one
// configuration with -DTP_GEMM_FORCE_CFG=<index> (tuning).
const char* gemm_bf16_pick(const GemmDesc& d, int* cfg) {
  if (d.epi == EPI_F32) {   // fp32 partials: the ping-pong tile (K-major operands), or for MN-major ones
    // (the k-split weight gradients) 256 x 256 or 256 x 192 by rounds x area / rate, also in tuning builds
    *cfg = d.a_kmajor ? 9 : gemm_bf16_wgrad_tile(d.M, d.N, d.ksplit > 1 ? d.ksplit : 1);
    return kTileName[*cfg];
  }
#ifdef TP_GEMM_FORCE_CFG
  *cfg = TP_GEMM_FORCE_CFG;
  return kTileName[TP_GEMM_FORCE_CFG];
#else
  // modelled time: (number of 256-CU waves of tiles) x (tile area) / (relative rate)
  int best = 0;
  double best_t = 1e300;
  // Xᵀ·dY (the weight gradients): both operands come through transposed LDS reads, and the 256 x 256
  // tile moves ≈14% fewer LDS bytes per flop than 256 x 192; on outputs of 4096 x 4096 and more its
  // rate there counts 1.1 (the GPT-3 weight gradients, 4.5 and 3.4 rounds of it, were measured faster
  // on it than on 256 x 192's 6 and 4.5 rounds: its partial last round fills with the concurrent
  // input-gradient GEMM), which still leaves 256 x 192 to an output it covers in as many rounds
  const bool tn_big = !d.a_kmajor && !d.b_kmajor && (long)d.M * d.N >= 4096L * 4096L;
  for (int c : {9, 10, 11, 0, 8, 1, 2, 3}) {
    if (c >= 9 && !d.a_kmajor) continue;   // the ping-pong tiles take X·W and dY·Wᵀ only
    // the 160-wide tile paid only on a long k loop (the GPT-3 tp=8 QKV forward, k = 12288: 246 ->
    // 237 us, 232 tiles instead of 192); at k = 1600 and 3072 it was 1% slower than 192
    if (c == 11 && d.K < 8192) continue;
    const long t = (long)((d.M + kTileM[c] - 1) / kTileM[c]) * ((d.N + kTileN[c] - 1) / kTileN[c]);
    const double rate = (tn_big && c == 0) ? 1.1 : kTileRate[c];
    const double est = (double)((t + 255) / 256) * kTileM[c] * kTileN[c] / rate;
    if (est < best_t * 0.999) { best_t = est; best = c; }
  }
  *cfg = best;
  return kTileName[best];
#endif
}

hipError_t launch_gemm_bf16(const GemmDesc& d, int cfg, hipStream_t s) {
  switch (cfg) {
    case 0:
      if (d.epi == EPI_F32 && !d.a_kmajor && !d.b_kmajor) return run<C0, false, false, EPI_F32>(d, s);
      return run_cfg<C0>(d, s);
    case 1: return run_cfg<C1>(d, s);
    case 2: return run_cfg<C2>(d, s);
    case 3: return run_cfg<C3>(d, s);
#ifdef TP_GEMM_FORCE_CFG
    // deeper-pipeline and one-wave-per-SIMD tiles: measured slower on every shard shape, compiled
    // only into tuning builds that pin a configuration
    case 4: return run_cfg<C4>(d, s);
    case 5: return run_cfg<C5>(d, s);
    case 6: return run_cfg<C6>(d, s);
    case 7: return run_cfg<C7>(d, s);
#endif
    case 9: return run_pp_cfg<192>(d, s);
    case 10: return run_pp_cfg<224>(d, s);
    case 11: return run_pp_cfg<160>(d, s);
    default:
      if (d.epi == EPI_F32 && !d.a_kmajor && !d.b_kmajor) return run<C8, false, false, EPI_F32>(d, s);
      return run_cfg<C8>(d, s);
  }
}

// Every grouped GEMM uses a 256 x 256 tile (two stages of k = 64; the ping-pong schedule for a long k
// loop over an MN-major B); the tile height is still asked per k so the plan can number m-tiles.
int gemm_bf16_grouped_bm(int) {
  static_assert(C0::BM == PPCfg<256>::BM, "the plan numbers m-tiles of one height");
  return C0::BM;
}

// The n-tile width launch_gemm_bf16_grouped takes for this GEMM (as its tile choice below).
int gemm_bf16_grouped_bn(const GemmDesc& d) { return (!d.b_kmajor && d.K >= 2048) ? PPCfg<256>::BN : C0::BN; }

template <class Cfg, bool PP = false>
static hipError_t grouped_t(const GroupedArgs& g, int max_mtiles, hipStream_t s) {
  const long tiles = (long)max_mtiles * ((g.d.N + Cfg::BN - 1) / Cfg::BN);
  if (tiles > 0x7ffffff0L) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(8 * ((tiles + 7) / 8));
  if (!g.d.a_kmajor) return hipErrorNotSupported;
  if (g.d.b_kmajor) {     // the backward's dY·Wᵀ forms: GeLU' or plain; gathered rows with the gate
    if (g.d.a_rows) {
      if (g.d.epi != EPI_DGELU_GATE || (long)g.d.a_rows_n * g.d.lda * 2 > 0x7fffffffL) return hipErrorNotSupported;
      gemm_bf16_grouped_kernel<Cfg, EPI_DGELU_GATE, true, true, PP><<<grid, Cfg::NT, 0, s>>>(g);
      return hipGetLastError();
    }
    if (g.d.epi == EPI_DGELU) gemm_bf16_grouped_kernel<Cfg, EPI_DGELU, false, true, PP><<<grid, Cfg::NT, 0, s>>>(g);
    else if (g.d.epi == EPI_STORE) gemm_bf16_grouped_kernel<Cfg, EPI_STORE, false, true, PP><<<grid, Cfg::NT, 0, s>>>(g);
    else return hipErrorNotSupported;
    return hipGetLastError();
  }
  if (g.d.a_rows) {
    if (g.d.epi != EPI_BIAS_GELU || (long)g.d.a_rows_n * g.d.lda * 2 > 0x7fffffffL) return hipErrorNotSupported;
    gemm_bf16_grouped_kernel<Cfg, EPI_BIAS_GELU, true, false, PP><<<grid, Cfg::NT, 0, s>>>(g);
  } else if (g.d.epi == EPI_BIAS_GELU) {
    gemm_bf16_grouped_kernel<Cfg, EPI_BIAS_GELU, false, false, PP><<<grid, Cfg::NT, 0, s>>>(g);
  } else if (g.d.epi == EPI_STORE) {
    gemm_bf16_grouped_kernel<Cfg, EPI_STORE, false, false, PP><<<grid, Cfg::NT, 0, s>>>(g);
  } else {
    return hipErrorNotSupported;
  }
  return hipGetLastError();
}

// prefix[] must number m-tiles of gemm_bf16_grouped_bm(d.K) rows, tile_expert[] name their experts.
hipError_t launch_gemm_bf16_grouped(const GemmDesc& d, const int* off, const int* prefix, const int* tile_expert,
                                    int groups, long b_stride, long bias_stride, int max_mtiles, hipStream_t s) {
  GroupedArgs g{d, off, prefix, tile_expert, groups, b_stride, bias_stride};
  if (max_mtiles <= 0 || d.N <= 0) return hipSuccess;
  // a long k loop takes the ping-pong schedule on a 256 x 256 tile (measured on the 128-expert shard,
  // k = 8192, gathered rows: fc1 0.30 of peak against 0.22 for four stages of k = 32 on the plain
  // tile; the backward's gated dA1 0.32 against 0.31 on the plain tile)
  if (d.K >= 2048) return grouped_t<PPCfg<256>, true>(g, max_mtiles, s);
  return grouped_t<C0>(g, max_mtiles, s);
}

// Whether the tiled grouped weight-gradient kernel takes these operands (K is free: see the kernel).
bool gemm_bf16_grouped_k_eligible(const GemmDesc& d) {
  if (d.dtype != DT_BF16 || d.M <= 0 || d.N <= 0 || d.a_kmajor || d.b_kmajor) return false;
  if ((d.M | d.N) & 7) return false;
  if ((d.lda | d.ldb | d.ldc) & 7) return false;
  if (d.lda > (1L << 22) || d.ldb > (1L << 22)) return false;
  if (d.a_rows && (long)d.a_rows_n * d.lda * 2 > 0x7fffffffL) return false;   // one buffer range over A
  if (d.b_rows && (long)d.b_rows_n * d.ldb * 2 > 0x7fffffffL) return false;   // and over B
  return ((((uintptr_t)d.A) | ((uintptr_t)d.B) | ((uintptr_t)d.C)) & 15) == 0;
}

template <class Cfg, bool GK, bool GKB>
static hipError_t grouped_k_t(const GemmDesc& d, const int* off, int groups, long c_stride, hipStream_t s) {
  const int tiles_m = (d.M + Cfg::BM - 1) / Cfg::BM, tiles_n = (d.N + Cfg::BN - 1) / Cfg::BN;
  const long nwg = (long)tiles_m * tiles_n * groups;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7fffffffL) return hipErrorInvalidValue;
  GroupedKArgs g{d, off, groups, c_stride};
  gemm_bf16_grouped_k_kernel<Cfg, GK, GKB><<<(unsigned)nwg, Cfg::NT, 0, s>>>(g, tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_grouped_k(const GemmDesc& d, const int* off, int groups, long c_stride, hipStream_t s) {
  // measured on the 128-expert weight gradients: the gathered form is 14% faster with k = 32 (C0
  // spills there), the plain form 21% slower
  // (a gathered B, the MoE backward's dW2 over the output gradient's rows, takes the same tile)
  if (d.a_rows && d.b_rows) return hipErrorNotSupported;
  if (d.a_rows) return grouped_k_t<C9, true, false>(d, off, groups, c_stride, s);
  if (d.b_rows) return grouped_k_t<C9, false, true>(d, off, groups, c_stride, s);
  return grouped_k_t<C0, false, false>(d, off, groups, c_stride, s);
}

}  // namespace tp
