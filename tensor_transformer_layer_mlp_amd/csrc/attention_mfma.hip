// Causal attention on the matrix cores (bf16 inputs, fp32 scores / softmax / accumulation).
//
// Heads are read from the head-interleaved QKV rows (q at h*3d, k at h*3d + d, v at h*3d + 2d), row
// stride 3*nh*d.  Every MFMA is v_mfma_f32_16x16x32_bf16; its result lane l holds D[4*(l/16) + e]
// [l % 16].  The kernels choose operand order so that a lane always owns one query (forward, dQ) or
// one key (dK/dV) of the result, which keeps the softmax row statistics in registers:
//
// Work split: a workgroup owns 64 queries (forward, dQ) or 64 keys (dK/dV) as two waves of 32, and
// G such wave pairs ("groups") share the other dimension's 64-wide blocks round-robin (group g takes
// blocks g, g+G, ...), each group with its own double-buffered LDS tiles.  This shortens the causal
// chain of the longest workgroups G-fold and puts 2G waves on a CU.  At the end the groups' partial
// results meet in LDS and group 0 combines them in a fixed order (deterministic).
// Forward (per wave of 32 queries): for each 64-key block of its group,
//   S = K·Qᵀ     lane: query q, keys 4g+e of each 16-key slice      (K from LDS, Q in registers)
//   online softmax in the exp2 domain: t = s·log2(e)/√d; running max m (two lane swaps give the
//   row max across the 4 lanes of a query) and per-lane partial sums l; groups merge as
//   m = max m_g, o = Σ o_g·2^(m_g − m), l = Σ l_g·2^(m_g − m)
//   Oᵀ += Vᵀ·Pᵀ  P stays in registers as the second operand; the key order of its 8 k-slots
//                (4g+e and 16+4g+e) is matched by reading V with ds_read_b64_tr_b16.
//   LSE = (m + log2 l)·ln 2.
// Backward, deterministic (no atomics), dQ first:
//   dQ      one workgroup = 64 queries, waves of 32 queries: D_i = Σ_c dO_ic·O_ic from the wave's dO
//           fragments and the same fragments of O (left in an fp32 workspace for dK/dV), then a loop
//           over the key blocks up to them: S, P = exp2(t − LSE·log2 e), dP = dO·Vᵀ, dS = P∘(dP − D)
//           in the query-owned layout, dQᵀ += Kᵀ·dSᵀ (K read transposed)
//   dK/dV   one workgroup = 64 keys, waves of 32 keys, loop over the query blocks at or after them:
//           Sᵀ, P, dPᵀ, dS as above in the key-owned layout, dVᵀ += dOᵀ·P, dKᵀ += Qᵀ·dS (dO and Q
//           read transposed from LDS).
// LDS tiles are KB rows (32 or 64) x (d padded to 32, 64 or 128) with the 32-byte chunk q of row r stored at
// q ^ sw(r), which keeps both the 16-byte row reads and the transposed 4x16 reads spread over the
// banks.  Tiles arrive by buffer_load_dwordx4 ... lds (two stages, next block in flight); rows past S
// and columns past d arrive as zeros.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace tp {

namespace {

constexpr unsigned OOB = 0x80000000u;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

template <int D>
struct AC {
  static constexpr int DP = D <= 32 ? 32 : (D <= 64 ? 64 : 128);  // d padded to the MFMA k-step
  static constexpr int PB = 2 * DP;           // LDS row pitch, bytes
  static constexpr int RS = 256 / PB;         // rows per 256-byte bank window
  static constexpr int NC32 = PB / 32;        // 32-byte chunks per row
  // 32-wide k-steps over d and 16-wide d blocks of the outputs: those that hold a column below D
  // (the tiles keep the padded pitch; the steps past D would multiply zeros: d = 96 takes 3 and 6,
  // not 4 and 8)
  static constexpr int NKK = (D + 31) / 32;
  static constexpr int NDB = (D + 15) / 16;
  template <int R> static constexpr int tile() { return R * PB; }   // R-row tile, bytes
};

template <int D>
__device__ __forceinline__ int sw(int r) { return (r / AC<D>::RS) & (AC<D>::NC32 - 1); }

// Byte address of (row r, element d) in a tile.
template <int D>
__device__ __forceinline__ int taddr(int r, int d) {
  return r * AC<D>::PB + ((((d >> 4) ^ sw<D>(r)) << 5) | ((d & 15) << 1));
}

// R rows starting at `rows` (row stride rs elements), columns [0, D) -> tile; rows >= nvalid and
// columns >= D are zero.  Two waves share the loads (1 KiB per wave-load).
template <int D, int R>
__device__ __forceinline__ void load_tile(const bf16* rows, long rs, int nvalid, TP_LDS char* dst,
                                          int wave, int lane) {
  using C = AC<D>;
  constexpr int PER = C::template tile<R>() / 1024 / 2;
  static_assert(PER >= 1, "tile smaller than two wave-loads");
  const unsigned span = (unsigned)(((R - 1L) * rs + D) * 2);
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)rows, (short)0, (int)span, 0x00020000);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int slot = wave * PER + j;
    const int o = slot * 1024 + 16 * lane;
    const int row = o / C::PB;
    const int s16 = (o % C::PB) >> 4;
    const int d = 16 * ((s16 >> 1) ^ sw<D>(row)) + 8 * (s16 & 1);
    const bool ok = row < nvalid && d < D;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (TP_LDS void*)(dst + slot * 1024), 16,
                                             ok ? (unsigned)((row * rs + d) * 2) : OOB, 0, 0, 0);
  }
}

// N (<= 64) floats from src, the first nvalid in range, into dst by one wave as a direct global -> LDS
// load: lane i (< N) writes dst[i], zero past nvalid; the lanes from N on are masked off.
template <int N>
__device__ __forceinline__ void load_floats(const float* src, int nvalid, TP_LDS float* dst, int lane) {
  static_assert(N >= 1 && N <= 64, "one wave, one float per lane");
  __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, nvalid > 0 ? nvalid * 4 : 0, 0x00020000);
  if (lane < N) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (TP_LDS void*)dst, 4, lane < nvalid ? 4u * lane : OOB, 0, 0, 0);
}

// Row fragment: lane l gets row r0 + l%16, elements d0 + 8*(l/16) .. +7 (one 16-byte read).
template <int D>
__device__ __forceinline__ bf16x8 frag_row(const TP_LDS char* t, int r0, int d0, int lane) {
  return *(const TP_LDS bf16x8*)(t + taddr<D>(r0 + (lane & 15), d0 + 8 * (lane >> 4)));
}

// Transposed fragment: lane l gets column d0 + l%16 at rows r0 + 4g + {0..3} and r0 + 16 + 4g +
// {0..3} (g = l/16) — the k-slot order of a P (or dS) fragment held in registers.
template <int D>
__device__ __forceinline__ bf16x8 frag_tr(const TP_LDS char* t, int r0, int d0, int lane) {
  const int i = lane & 15, g = lane >> 4;
  const int r1 = r0 + 4 * g + (i >> 2), r2 = r1 + 16;
  const int d = d0 + 4 * (i & 3);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((TP_LDS bf16x4*)(t + taddr<D>(r1, d)));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((TP_LDS bf16x4*)(t + taddr<D>(r2, d)));
  return (bf16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// 16 rows x 32 columns straight from global memory into a fragment (lane: row r0 + l%16, columns
// d0 + 8*(l/16) .. +7), zero outside [0, nvalid) x [0, D).
template <int D>
__device__ __forceinline__ bf16x8 frag_global(const bf16* rows, long rs, int r0, int nvalid, int d0,
                                              int lane) {
  const int r = r0 + (lane & 15), d = d0 + 8 * (lane >> 4);
  if (r < nvalid && d < D) return *(const bf16x8*)(rows + (long)r * rs + d);
  return (bf16x8){};
}

// v_permlane16_swap / v_permlane32_swap applied to two copies of v leave {v[l], v[l^16]} (resp.
// {v[l], v[l^32]}) in the two results of lane l: a cross-row exchange in one VALU op, no LDS.
__device__ __forceinline__ float pair16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// over the 4 lanes l%16 + 16g (g = 0..3) that share one query or key row
__device__ __forceinline__ float xmax4(float v) { return pair32_max(pair16_max(v)); }
__device__ __forceinline__ float xsum4(float v) { return pair32_sum(pair16_sum(v)); }

__device__ __forceinline__ bf16x8 pack8(f32x4 a, f32x4 b) {
  return (bf16x8){(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                  (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
}

__device__ __forceinline__ void store4(bf16* p, f32x4 v, float s) {
  *(bf16x4*)p = (bf16x4){(bf16)(v[0] * s), (bf16)(v[1] * s), (bf16)(v[2] * s), (bf16)(v[3] * s)};
}

// ---------------------------------------------------------------------------------------------
template <int D, int G, int KB>
__global__ __launch_bounds__(128 * G) void attn_fwd_mfma(int B, int S, int nh, int nqb,
                                                         const bf16* __restrict__ qkv,
                                                         bf16* __restrict__ ctx, float* __restrict__ lse) {
  using C = AC<D>;
  constexpr int TILE = C::template tile<KB>();
  constexpr int GST = 2 * 2 * TILE;             // per group: two stages of (K tile, V tile)
  constexpr int SLOT = 64 * (2 * C::NDB * 16 + 16);   // one wave's partial (o, m, l) for the merge
  static_assert(G == 1 || 2 * SLOT <= G * GST, "merge slots exceed the tile memory");
  __shared__ __attribute__((aligned(1024))) char smem[G * GST];
  const int lane = threadIdx.x & 63, g = lane >> 4, i16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar registers
  const int half = w & 1, grp = w >> 1;
  const int nbh = nh * B, idx = blockIdx.x;
  const int qb = nqb - 1 - idx / nbh, h = (idx % nbh) % nh, b = (idx % nbh) / nh;  // long blocks first
  const long rs = 3L * nh * D;
  const bf16* qrows = qkv + (long)b * S * rs + (long)h * 3 * D;
  const int qw = qb * 64 + 32 * half;
  const float c = LOG2E / sqrtf((float)D);

  bf16x8 qf[2][C::NKK];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) qf[qs][kk] = frag_global<D>(qrows, rs, qw + 16 * qs, S, 32 * kk, lane);
  f32x4 o[2][C::NDB];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) o[qs][db] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

  const int nkb = min((S + KB - 1) / KB, (64 * qb + 63) / KB + 1);   // key blocks up to the diagonal
  const int nit = (nkb + G - 1) / G;
  TP_LDS char* lds = (TP_LDS char*)smem + grp * GST;
  if (grp < nkb) {
    load_tile<D, KB>(qrows + (long)grp * KB * rs + D, rs, S - grp * KB, lds, half, lane);
    load_tile<D, KB>(qrows + (long)grp * KB * rs + 2 * D, rs, S - grp * KB, lds + TILE, half, lane);
  }
  for (int it = 0; it < nit; ++it) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int j = it * G + grp, jn = j + G;
    if (jn < nkb) {
      TP_LDS char* nx = lds + ((it + 1) & 1) * 2 * TILE;
      load_tile<D, KB>(qrows + (long)jn * KB * rs + D, rs, S - jn * KB, nx, half, lane);
      load_tile<D, KB>(qrows + (long)jn * KB * rs + 2 * D, rs, S - jn * KB, nx + TILE, half, lane);
    }
    const int k0 = KB * j;
    if (j >= nkb || k0 > qw + 31) continue;   // no block, or every key in the future of every query
    const TP_LDS char* kt = lds + (it & 1) * 2 * TILE;
    const TP_LDS char* vt = kt + TILE;
    f32x4 s[2][KB / 16];
#pragma unroll
    for (int kb = 0; kb < KB / 16; ++kb) {
      bf16x8 kf[C::NKK];
#pragma unroll
      for (int kk = 0; kk < C::NKK; ++kk) kf[kk] = frag_row<D>(kt, 16 * kb, 32 * kk, lane);
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        f32x4 a = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk) a = mfma_16x16x32_bf16(kf[kk], qf[qs][kk], a);
        s[qs][kb] = a;
      }
    }
    if ((k0 + KB - 1 > qw) || (k0 + KB > S)) {
      // diagonal or ragged block (wave-uniform test): hide future keys and keys past S
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int kb = 0; kb < KB / 16; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int q = qw + 16 * qs + i16, key = k0 + 16 * kb + 4 * g + e;
            if (key > q || key >= S) s[qs][kb][e] = -INFINITY;
          }
    }
    // Block max per query in the scaled log2 domain (c > 0, so max(s)·c = max(s·c)).  The reference
    // max m moves only when a block max passes it by more than 8: p = 2^(s·c − m) then stays ≤ 256
    // and most blocks skip the rescale of o and l, which always share one m, so the result is the
    // same softmax.  Every processed block holds a visible key of every query: the maxima are finite.
    float mxs[2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB / 16; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s[qs][kb][e]);
      mxs[qs] = xmax4(mx) * c;
    }
    if (__builtin_amdgcn_ballot_w64(mxs[0] > m[0] + 8.f || mxs[1] > m[1] + 8.f)) {
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        const float mn = fmaxf(m[qs], mxs[qs]);
        const float corr = __builtin_amdgcn_exp2f(m[qs] - mn);
        m[qs] = mn;
        l[qs] *= corr;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) o[qs][db] *= corr;
      }
    }
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB / 16; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[qs][kb][e], c, -m[qs]));
          s[qs][kb][e] = p;
          ls += p;
        }
      l[qs] += ls;
    }
#pragma unroll
    for (int kc = 0; kc < KB / 32; ++kc) {
      bf16x8 pf[2];
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) pf[qs] = pack8(s[qs][2 * kc], s[qs][2 * kc + 1]);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const bf16x8 vf = frag_tr<D>(vt, 32 * kc, 16 * db, lane);
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) o[qs][db] = mfma_16x16x32_bf16(vf, pf[qs], o[qs][db]);
      }
    }
  }

  if constexpr (G > 1) {
    // group gg (1..G-1) leaves (o, m, l) in LDS in lane order and group 0 folds it in, one group
    // per round, so that the merge needs two wave slots of LDS whatever G is
    __builtin_amdgcn_s_waitcnt(0);
    TP_LDS char* slot = (TP_LDS char*)smem + half * SLOT;
    for (int gg = 1; gg < G; ++gg) {
      __syncthreads();
      if (grp == gg) {
#pragma unroll
        for (int qs = 0; qs < 2; ++qs)
#pragma unroll
          for (int db = 0; db < C::NDB; ++db)
            *(TP_LDS f32x4*)(slot + ((qs * C::NDB + db) * 64 + lane) * 16) = o[qs][db];
        *(TP_LDS f32x4*)(slot + 2 * C::NDB * 64 * 16 + lane * 16) = (f32x4){m[0], m[1], l[0], l[1]};
      }
      __syncthreads();
      if (grp == 0) {
        const f32x4 ml = *(const TP_LDS f32x4*)(slot + 2 * C::NDB * 64 * 16 + lane * 16);
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
          const float mo = ml[qs], mn = fmaxf(m[qs], mo);
          if (mn == -INFINITY) continue;      // neither side has seen a key (rows past S only)
          const float ca = __builtin_amdgcn_exp2f(m[qs] - mn), cb = __builtin_amdgcn_exp2f(mo - mn);
          m[qs] = mn;
          l[qs] = l[qs] * ca + ml[2 + qs] * cb;
#pragma unroll
          for (int db = 0; db < C::NDB; ++db)
            o[qs][db] = o[qs][db] * ca + *(const TP_LDS f32x4*)(slot + ((qs * C::NDB + db) * 64 + lane) * 16) * cb;
        }
      }
    }
    if (grp > 0) return;
  }
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const float lt = xsum4(l[qs]);
    const int q = qw + 16 * qs + i16;
    if (q < S) {
      const float inv = 1.0f / lt;
      bf16* out = ctx + ((long)b * S + q) * nh * D + (long)h * D;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const int d = 16 * db + 4 * g;
        if (d < D) store4(out + d, o[qs][db], inv);
      }
      if (lse && g == 0) lse[((long)b * nh + h) * S + q] = (m[qs] + __log2f(lt)) * LN2;
    }
  }
}

// ---------------------------------------------------------------------------------------------
template <int D, int G, int KB>
__global__ __launch_bounds__(128 * G) void attn_bwd_dkv_mfma(int B, int S, int nh, int nqb,
                                                             const bf16* __restrict__ qkv,
                                                             const bf16* __restrict__ dctx,
                                                             const float* __restrict__ lse,
                                                             const float* __restrict__ Dws,
                                                             bf16* __restrict__ dqkv) {
  using C = AC<D>;
  constexpr int TILE = C::template tile<KB>();
  constexpr int STG = 2 * TILE + 8 * KB;     // Q tile, dO tile, LSE[KB], D[KB]
  constexpr int SLOT = 64 * 4 * C::NDB * 16;  // one wave's partial (dK, dV) for the merge
  static_assert(G == 1 || 2 * SLOT <= G * 2 * STG, "merge slots exceed the tile memory");
  __shared__ __attribute__((aligned(1024))) char smem[G * 2 * STG];
  const int lane = threadIdx.x & 63, g = lane >> 4, i16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar registers
  const int half = w & 1, grp = w >> 1;
  const int nbh = nh * B, idx = blockIdx.x;
  const int kb = idx / nbh, h = (idx % nbh) % nh, b = (idx % nbh) / nh;   // early keys see most queries
  const long rs = 3L * nh * D, cs = (long)nh * D;
  const bf16* rows = qkv + (long)b * S * rs + (long)h * 3 * D;
  const bf16* dorows = dctx + (long)b * S * cs + (long)h * D;
  const float* lse_bh = lse + ((long)b * nh + h) * S;
  const float* D_bh = Dws + ((long)b * nh + h) * S;
  const int kw = kb * 64 + 32 * half;
  const float c = LOG2E / sqrtf((float)D);

  bf16x8 kf[2][C::NKK], vf[2][C::NKK];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
      kf[ks][kk] = frag_global<D>(rows + D, rs, kw + 16 * ks, S, 32 * kk, lane);
      vf[ks][kk] = frag_global<D>(rows + 2 * D, rs, kw + 16 * ks, S, 32 * kk, lane);
    }
  f32x4 dk[2][C::NDB], dv[2][C::NDB];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      dk[ks][db] = (f32x4){0.f, 0.f, 0.f, 0.f};
      dv[ks][db] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }

  TP_LDS char* lds = (TP_LDS char*)smem + grp * 2 * STG;
  // the 64 threads of the group's first wave fill the LSE / D rows
  // LSE and D come straight into LDS as well: a load into registers and a store to LDS here would
  // make the compiler wait for every load in flight, the block's own tiles included.  Rows past S
  // arrive as zeros, which contribute nothing: their Q and dO rows are zero, so P = 1 and dS = 0.
  auto stage = [&](int qb, TP_LDS char* dst) {
    const int q0 = qb * KB;
    load_tile<D, KB>(rows + (long)q0 * rs, rs, S - q0, dst, half, lane);
    load_tile<D, KB>(dorows + (long)q0 * cs, cs, S - q0, dst + TILE, half, lane);
    if (half == 0) {
      load_floats<KB>(lse_bh + q0, S - q0, (TP_LDS float*)(dst + 2 * TILE), lane);
      load_floats<KB>(D_bh + q0, S - q0, (TP_LDS float*)(dst + 2 * TILE + 4 * KB), lane);
    }
  };
  const int jq0 = 64 * kb / KB;            // first query block that reaches this key block
  const int nq = (S + KB - 1) / KB - jq0;
  const int nit = (nq + G - 1) / G;
  if (grp < nq) stage(jq0 + grp, lds);
  for (int it = 0; it < nit; ++it) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int j = it * G + grp, jn = j + G;
    if (jn < nq) stage(jq0 + jn, lds + ((it + 1) & 1) * STG);
    const int q0 = (jq0 + j) * KB;
    if (j >= nq || q0 + KB - 1 < kw) continue;   // no block, or every query precedes every key here
    const TP_LDS char* qt = lds + (it & 1) * STG;
    const TP_LDS char* dt = qt + TILE;
    const TP_LDS float* Ls = (const TP_LDS float*)(qt + 2 * TILE);
    const TP_LDS float* Ds = Ls + KB;
    // P and dS for the KB queries x this wave's 32 keys; lane: key kw + 16ks + i16,
    // queries q0 + 16qsub + 4g + e.  Only blocks that reach below the diagonal need the causal mask
    // (wave-uniform choice); keys past S need none, their rows of dK and dV are never stored.
    // One 32-query chunk at a time: P and dS of its two 16-query slices are packed to bf16 right
    // away and consumed by the dV / dK MFMAs, so only one chunk's P and dS are ever live.
#pragma unroll
    for (int qc = 0; qc < KB / 32; ++qc) {
      bf16x8 pf[2], sf[2];
      auto pds = [&](auto masked) {
        f32x4 p[2][2], ds[2][2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int qsub = 2 * qc + h2;
          bf16x8 qa[C::NKK], da[C::NKK];
#pragma unroll
          for (int kk = 0; kk < C::NKK; ++kk) {
            qa[kk] = frag_row<D>(qt, 16 * qsub, 32 * kk, lane);
            da[kk] = frag_row<D>(dt, 16 * qsub, 32 * kk, lane);
          }
          const f32x4 lq = *(const TP_LDS f32x4*)(Ls + 16 * qsub + 4 * g);
          const f32x4 dq = *(const TP_LDS f32x4*)(Ds + 16 * qsub + 4 * g);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            f32x4 sa = (f32x4){0.f, 0.f, 0.f, 0.f}, pa = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < C::NKK; ++kk) {
              sa = mfma_16x16x32_bf16(qa[kk], kf[ks][kk], sa);
              pa = mfma_16x16x32_bf16(da[kk], vf[ks][kk], pa);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float pv = __builtin_amdgcn_exp2f(fmaf(sa[e], c, -lq[e] * LOG2E));
              if constexpr (decltype(masked)::value) {
                if (kw + 16 * ks + i16 > q0 + 16 * qsub + 4 * g + e) pv = 0.f;
              }
              p[h2][ks][e] = pv;
              ds[h2][ks][e] = pv * (pa[e] - dq[e]);
            }
          }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          pf[ks] = pack8(p[0][ks], p[1][ks]);
          sf[ks] = pack8(ds[0][ks], ds[1][ks]);
        }
      };
      // the causal mask only where a key of this wave can follow a query of this chunk
      if (kw + 31 > q0 + 32 * qc) pds(std::true_type{}); else pds(std::false_type{});
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const bf16x8 doT = frag_tr<D>(dt, 32 * qc, 16 * db, lane);
        const bf16x8 qT = frag_tr<D>(qt, 32 * qc, 16 * db, lane);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          dv[ks][db] = mfma_16x16x32_bf16(doT, pf[ks], dv[ks][db]);
          dk[ks][db] = mfma_16x16x32_bf16(qT, sf[ks], dk[ks][db]);
        }
      }
    }
  }

  if constexpr (G > 1) {
    // partial sums over each group's query blocks, added in group order by group 0, one group per
    // round through two wave slots of LDS
    __builtin_amdgcn_s_waitcnt(0);
    TP_LDS char* slot = (TP_LDS char*)smem + half * SLOT;
    for (int gg = 1; gg < G; ++gg) {
      __syncthreads();
      if (grp == gg) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            *(TP_LDS f32x4*)(slot + (((0 * 2 + ks) * C::NDB + db) * 64 + lane) * 16) = dk[ks][db];
            *(TP_LDS f32x4*)(slot + (((1 * 2 + ks) * C::NDB + db) * 64 + lane) * 16) = dv[ks][db];
          }
      }
      __syncthreads();
      if (grp == 0) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            dk[ks][db] += *(const TP_LDS f32x4*)(slot + (((0 * 2 + ks) * C::NDB + db) * 64 + lane) * 16);
            dv[ks][db] += *(const TP_LDS f32x4*)(slot + (((1 * 2 + ks) * C::NDB + db) * 64 + lane) * 16);
          }
      }
    }
    if (grp > 0) return;
  }
  const float scale = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int key = kw + 16 * ks + i16;
    if (key >= S) continue;
    bf16* out = dqkv + ((long)b * S + key) * rs + (long)h * 3 * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int d = 16 * db + 4 * g;
      if (d < D) {
        store4(out + D + d, dk[ks][db], scale);
        store4(out + 2 * D + d, dv[ks][db], 1.0f);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
template <int D, int G, int KB>
__global__ __launch_bounds__(128 * G) void attn_bwd_dq_mfma(int B, int S, int nh, int nqb,
                                                            const bf16* __restrict__ qkv,
                                                            const bf16* __restrict__ ctx,
                                                            const bf16* __restrict__ dctx,
                                                            const float* __restrict__ lse,
                                                            float* __restrict__ Dws,
                                                            bf16* __restrict__ dqkv) {
  using C = AC<D>;
  constexpr int TILE = C::template tile<KB>();
  constexpr int GST = 2 * 2 * TILE;          // per group: two stages of (K tile, V tile)
  constexpr int SLOT = 64 * 2 * C::NDB * 16;  // one wave's partial dQ for the merge
  static_assert(G == 1 || 2 * SLOT <= G * GST, "merge slots exceed the tile memory");
  __shared__ __attribute__((aligned(1024))) char smem[G * GST];
  const int lane = threadIdx.x & 63, g = lane >> 4, i16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar registers
  const int half = w & 1, grp = w >> 1;
  const int nbh = nh * B, idx = blockIdx.x;
  const int qb = nqb - 1 - idx / nbh, h = (idx % nbh) % nh, b = (idx % nbh) / nh;
  const long rs = 3L * nh * D, cs = (long)nh * D;
  const bf16* rows = qkv + (long)b * S * rs + (long)h * 3 * D;
  const bf16* dorows = dctx + (long)b * S * cs + (long)h * D;
  const int qw = qb * 64 + 32 * half;
  const float c = LOG2E / sqrtf((float)D);

  // D_q = Σ_c dO_qc·O_qc from this wave's dO fragments and the same fragments of O: a lane's 8·NKK
  // columns of a row, then the four lanes of the row (every lane ends with the row's sum); the waves of
  // group 0 leave it in the workspace for the dK/dV kernel, which runs after this one
  const bf16* orows = ctx + (long)b * S * cs + (long)h * D;
  bf16x8 qf[2][C::NKK], df[2][C::NKK];
  float lq[2], dq_[2];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    float dot = 0.f;
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
      qf[qs][kk] = frag_global<D>(rows, rs, qw + 16 * qs, S, 32 * kk, lane);
      df[qs][kk] = frag_global<D>(dorows, cs, qw + 16 * qs, S, 32 * kk, lane);
      const bf16x8 of = frag_global<D>(orows, cs, qw + 16 * qs, S, 32 * kk, lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf((float)df[qs][kk][e], (float)of[e], dot);
    }
    const int q = qw + 16 * qs + i16;
    lq[qs] = q < S ? lse[((long)b * nh + h) * S + q] * LOG2E : INFINITY;
    dq_[qs] = xsum4(dot);
    if (grp == 0 && g == 0 && q < S) Dws[((long)b * nh + h) * S + q] = dq_[qs];
  }
  f32x4 acc[2][C::NDB];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) acc[qs][db] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int nkb = min((S + KB - 1) / KB, (64 * qb + 63) / KB + 1);   // key blocks up to the diagonal
  const int nit = (nkb + G - 1) / G;
  TP_LDS char* lds = (TP_LDS char*)smem + grp * GST;
  if (grp < nkb) {
    load_tile<D, KB>(rows + (long)grp * KB * rs + D, rs, S - grp * KB, lds, half, lane);
    load_tile<D, KB>(rows + (long)grp * KB * rs + 2 * D, rs, S - grp * KB, lds + TILE, half, lane);
  }
  for (int it = 0; it < nit; ++it) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int j = it * G + grp, jn = j + G;
    if (jn < nkb) {
      TP_LDS char* nx = lds + ((it + 1) & 1) * 2 * TILE;
      load_tile<D, KB>(rows + (long)jn * KB * rs + D, rs, S - jn * KB, nx, half, lane);
      load_tile<D, KB>(rows + (long)jn * KB * rs + 2 * D, rs, S - jn * KB, nx + TILE, half, lane);
    }
    const int k0 = KB * j;
    if (j >= nkb || k0 > qw + 31) continue;
    const TP_LDS char* kt = lds + (it & 1) * 2 * TILE;
    const TP_LDS char* vt = kt + TILE;
    f32x4 dsv[2][KB / 16];
    // dS = P∘(dP − D) in the query-owned layout; the causal / ragged mask only on blocks that need it
    auto dsblock = [&](auto masked) {
#pragma unroll
      for (int kb = 0; kb < KB / 16; ++kb) {
        bf16x8 kfr[C::NKK], vfr[C::NKK];
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk) {
          kfr[kk] = frag_row<D>(kt, 16 * kb, 32 * kk, lane);
          vfr[kk] = frag_row<D>(vt, 16 * kb, 32 * kk, lane);
        }
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
          f32x4 sa = (f32x4){0.f, 0.f, 0.f, 0.f}, pa = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < C::NKK; ++kk) {
            sa = mfma_16x16x32_bf16(kfr[kk], qf[qs][kk], sa);
            pa = mfma_16x16x32_bf16(vfr[kk], df[qs][kk], pa);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float pv = __builtin_amdgcn_exp2f(fmaf(sa[e], c, -lq[qs]));
            if constexpr (decltype(masked)::value) {
              const int q = qw + 16 * qs + i16, key = k0 + 16 * kb + 4 * g + e;
              if (key > q || key >= S) pv = 0.f;
            }
            dsv[qs][kb][e] = pv * (pa[e] - dq_[qs]);
          }
        }
      }
    };
    if ((k0 + KB - 1 > qw) || (k0 + KB > S)) dsblock(std::true_type{}); else dsblock(std::false_type{});
#pragma unroll
    for (int kc = 0; kc < KB / 32; ++kc) {
      bf16x8 sf[2];
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) sf[qs] = pack8(dsv[qs][2 * kc], dsv[qs][2 * kc + 1]);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const bf16x8 kT = frag_tr<D>(kt, 32 * kc, 16 * db, lane);
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) acc[qs][db] = mfma_16x16x32_bf16(kT, sf[qs], acc[qs][db]);
      }
    }
  }

  if constexpr (G > 1) {
    __builtin_amdgcn_s_waitcnt(0);
    TP_LDS char* slot = (TP_LDS char*)smem + half * SLOT;
    for (int gg = 1; gg < G; ++gg) {
      __syncthreads();
      if (grp == gg) {
#pragma unroll
        for (int qs = 0; qs < 2; ++qs)
#pragma unroll
          for (int db = 0; db < C::NDB; ++db)
            *(TP_LDS f32x4*)(slot + ((qs * C::NDB + db) * 64 + lane) * 16) = acc[qs][db];
      }
      __syncthreads();
      if (grp == 0) {
#pragma unroll
        for (int qs = 0; qs < 2; ++qs)
#pragma unroll
          for (int db = 0; db < C::NDB; ++db)
            acc[qs][db] += *(const TP_LDS f32x4*)(slot + ((qs * C::NDB + db) * 64 + lane) * 16);
      }
    }
    if (grp > 0) return;
  }
  const float scale = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int q = qw + 16 * qs + i16;
    if (q >= S) continue;
    bf16* out = dqkv + ((long)b * S + q) * rs + (long)h * 3 * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int d = 16 * db + 4 * g;
      if (d < D) store4(out + d, acc[qs][db], scale);
    }
  }
}

// Launch shape: G wave-pair groups per workgroup and KB-row blocks of the looped-over dimension.
// Measured on the three GPT shards (d = 64: GPT-2 1.5B tp=2; 96: 8.3B tp=8; 128: GPT-3 tp=8):
//   d <= 64: forward G = 2, KB = 32 (32 KiB of LDS: four workgroups share a CU; 55 -> 26 us);
//            backward G = 1, KB = 64 (144 -> 87 us)
//   d = 96:  G = 2, KB = 32 both ways (23 -> 20 us, 71 -> 65 us)
//   d = 128: G = 2, KB = 64 (128 KiB of LDS, one workgroup per CU); four groups of 32 keys spill the
//            backward's accumulators and do not speed the forward
// A build may pin either kernel's shape for tuning.
#ifndef TP_ATTN_FWD_G
#define TP_ATTN_FWD_G 0
#endif
#ifndef TP_ATTN_FWD_KB
#define TP_ATTN_FWD_KB 0
#endif
#ifndef TP_ATTN_BWD_G
#define TP_ATTN_BWD_G 0
#endif
#ifndef TP_ATTN_BWD_KB
#define TP_ATTN_BWD_KB 0
#endif
template <int D>
struct AttnShape {   // backward (dK/dV and dQ)
  static constexpr int KB = TP_ATTN_BWD_KB ? TP_ATTN_BWD_KB : (D == 96 ? 32 : 64);
  static constexpr int G = TP_ATTN_BWD_G ? TP_ATTN_BWD_G : (D <= 64 ? 1 : 2);
};
template <int D>
struct AttnFwdShape {
  static constexpr int KB = TP_ATTN_FWD_KB ? TP_ATTN_FWD_KB : (D <= 96 ? 32 : 64);
  static constexpr int G = TP_ATTN_FWD_G ? TP_ATTN_FWD_G : 2;
};

template <int D>
hipError_t fwd_t(int B, int S, int nh, const void* qkv, void* ctx, float* lse, hipStream_t s) {
  constexpr int G = AttnFwdShape<D>::G, KB = AttnFwdShape<D>::KB;
  const int nqb = (S + 63) / 64;
  attn_fwd_mfma<D, G, KB><<<nqb * nh * B, 128 * G, 0, s>>>(B, S, nh, nqb, (const bf16*)qkv, (bf16*)ctx, lse);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_t(int B, int S, int nh, const void* qkv, const void* ctx, const float* lse,
                 const void* dctx, void* dqkv, float* ws, hipStream_t s) {
  constexpr int G = AttnShape<D>::G, KB = AttnShape<D>::KB;
  const int nqb = (S + 63) / 64;
  // dQ first: it takes D for its own queries from O and dO and leaves it in ws for dK/dV
  attn_bwd_dq_mfma<D, G, KB><<<nqb * nh * B, 128 * G, 0, s>>>(B, S, nh, nqb, (const bf16*)qkv, (const bf16*)ctx,
                                                              (const bf16*)dctx, lse, ws, (bf16*)dqkv);
  attn_bwd_dkv_mfma<D, G, KB><<<nqb * nh * B, 128 * G, 0, s>>>(B, S, nh, nqb, (const bf16*)qkv,
                                                               (const bf16*)dctx, lse, ws, (bf16*)dqkv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_mfma(int B, int S, int nh, int d, const void* qkv, void* ctx, float* lse,
                                hipStream_t s) {
  if (B <= 0 || S <= 0 || nh <= 0) return hipSuccess;
  switch (d) {
    case 16: return fwd_t<16>(B, S, nh, qkv, ctx, lse, s);
    case 32: return fwd_t<32>(B, S, nh, qkv, ctx, lse, s);
    case 64: return fwd_t<64>(B, S, nh, qkv, ctx, lse, s);
    case 96: return fwd_t<96>(B, S, nh, qkv, ctx, lse, s);
    case 128: return fwd_t<128>(B, S, nh, qkv, ctx, lse, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_bwd_mfma(int B, int S, int nh, int d, const void* qkv, const void* ctx,
                                const float* lse, const void* dctx, void* dqkv, float* ws,
                                hipStream_t s) {
  if (B <= 0 || S <= 0 || nh <= 0) return hipSuccess;
  switch (d) {
    case 16: return bwd_t<16>(B, S, nh, qkv, ctx, lse, dctx, dqkv, ws, s);
    case 32: return bwd_t<32>(B, S, nh, qkv, ctx, lse, dctx, dqkv, ws, s);
    case 64: return bwd_t<64>(B, S, nh, qkv, ctx, lse, dctx, dqkv, ws, s);
    case 96: return bwd_t<96>(B, S, nh, qkv, ctx, lse, dctx, dqkv, ws, s);
    case 128: return bwd_t<128>(B, S, nh, qkv, ctx, lse, dctx, dqkv, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tp
