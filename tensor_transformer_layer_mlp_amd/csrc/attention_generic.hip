// Generic causal attention (forward and backward), one thread per query (or key) row.
//
// Serves the fp32 check mode and is the second opinion for the MFMA attention kernels.  Scores,
// softmax and accumulation are fp32 with expf/logf from the device math library.  Heads are read
// from the head-interleaved QKV rows: q at h*3d, k at h*3d + d, v at h*3d + 2d.
//
// Forward: online softmax over 64-key blocks staged in LDS (m, l running max / sum per row).
// Backward (recomputing P from q, k and the saved LSE; D_i = Σ_c dO_ic·O_ic computed in place):
//   dq kernel  — one thread per query i:  dq_i = Σ_{j<=i} P_ij (dO_i·v_j − D_i) k_j / √d
//   dkv kernel — one thread per key j:    dv_j = Σ_{i>=j} P_ij dO_i ;
//                                         dk_j = Σ_{i>=j} P_ij (dO_i·v_j − D_i) q_i / √d
// No atomics: every output element is written by exactly one thread.
#include "common.h"
#include "kernels.h"

namespace tp {

namespace {

constexpr int AB = 64;   // rows per block (queries or keys)

template <typename T, int D>
__global__ __launch_bounds__(AB) void attn_fwd_generic(int S, int nh, const T* __restrict__ qkv,
                                                       T* __restrict__ ctx, float* __restrict__ lse) {
  __shared__ float Ks[AB][D + 1];
  __shared__ float Vs[AB][D + 1];
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int i = qb * AB + t;
  const long rs = 3L * nh * D;
  const T* base = qkv + (long)b * S * rs + (long)h * 3 * D;
  const float scale = 1.0f / sqrtf((float)D);
  const bool valid = i < S;
  float q[D], o[D];
  for (int c = 0; c < D; ++c) {
    q[c] = valid ? to_f32(base[(long)i * rs + c]) * scale : 0.f;
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kend = min(S, (qb + 1) * AB);
  for (int j0 = 0; j0 < kend; j0 += AB) {
    for (int idx = t; idx < AB * D; idx += AB) {
      const int jj = idx / D, c = idx % D, j = j0 + jj;
      float kv = 0.f, vv = 0.f;
      if (j < S) {
        kv = to_f32(base[(long)j * rs + D + c]);
        vv = to_f32(base[(long)j * rs + 2 * D + c]);
      }
      Ks[jj][c] = kv;
      Vs[jj][c] = vv;
    }
    __syncthreads();
    if (valid) {
      const int jmax = min(j0 + AB, i + 1);
      for (int j = j0; j < jmax; ++j) {
        float sc = 0.f;
        for (int c = 0; c < D; ++c) sc += q[c] * Ks[j - j0][c];
        const float mn = fmaxf(m, sc);
        const float corr = expf(m - mn);
        const float p = expf(sc - mn);
        l = l * corr + p;
        for (int c = 0; c < D; ++c) o[c] = o[c] * corr + p * Vs[j - j0][c];
        m = mn;
      }
    }
    __syncthreads();
  }
  if (valid) {
    T* out = ctx + ((long)b * S + i) * nh * D + (long)h * D;
    const float inv = 1.0f / l;
    for (int c = 0; c < D; ++c) out[c] = from_f32<T>(o[c] * inv);
    if (lse) lse[((long)b * nh + h) * S + i] = m + logf(l);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(AB) void attn_bwd_dq_generic(int S, int nh, const T* __restrict__ qkv,
                                                          const T* __restrict__ ctx,
                                                          const float* __restrict__ lse,
                                                          const T* __restrict__ dctx,
                                                          T* __restrict__ dqkv) {
  extern __shared__ float smem[];
  float(*Ks)[D + 1] = (float(*)[D + 1])smem;
  float(*Vs)[D + 1] = (float(*)[D + 1])(smem + AB * (D + 1));
  float(*Qs)[D + 1] = (float(*)[D + 1])(smem + 2 * AB * (D + 1));
  float(*Os)[D + 1] = (float(*)[D + 1])(smem + 3 * AB * (D + 1));
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int i = qb * AB + t;
  const long rs = 3L * nh * D, cs = (long)nh * D;
  const T* base = qkv + (long)b * S * rs + (long)h * 3 * D;
  const float scale = 1.0f / sqrtf((float)D);
  const bool valid = i < S;
  float Di = 0.f, li = 0.f;
  if (valid) {
    const T* o = ctx + ((long)b * S + i) * cs + (long)h * D;
    const T* dO = dctx + ((long)b * S + i) * cs + (long)h * D;
    for (int c = 0; c < D; ++c) {
      const float dov = to_f32(dO[c]);
      Di += dov * to_f32(o[c]);
      Qs[t][c] = to_f32(base[(long)i * rs + c]) * scale;
      Os[t][c] = dov;                        // dO row of this query
    }
    li = lse[((long)b * nh + h) * S + i];
  }
  float dq[D];
  for (int c = 0; c < D; ++c) dq[c] = 0.f;
  const int kend = min(S, (qb + 1) * AB);
  for (int j0 = 0; j0 < kend; j0 += AB) {
    __syncthreads();
    for (int idx = t; idx < AB * D; idx += AB) {
      const int jj = idx / D, c = idx % D, j = j0 + jj;
      float kv = 0.f, vv = 0.f;
      if (j < S) {
        kv = to_f32(base[(long)j * rs + D + c]);
        vv = to_f32(base[(long)j * rs + 2 * D + c]);
      }
      Ks[jj][c] = kv;
      Vs[jj][c] = vv;
    }
    __syncthreads();
    if (valid) {
      const int jmax = min(j0 + AB, i + 1);
      for (int j = j0; j < jmax; ++j) {
        float sc = 0.f, dp = 0.f;
        for (int c = 0; c < D; ++c) {
          sc += Qs[t][c] * Ks[j - j0][c];
          dp += Os[t][c] * Vs[j - j0][c];
        }
        const float p = expf(sc - li);
        const float ds = p * (dp - Di);
        for (int c = 0; c < D; ++c) dq[c] += ds * Ks[j - j0][c];
      }
    }
  }
  if (valid) {
    T* out = dqkv + ((long)b * S + i) * rs + (long)h * 3 * D;
    for (int c = 0; c < D; ++c) out[c] = from_f32<T>(dq[c] * scale);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(AB) void attn_bwd_dkv_generic(int S, int nh, const T* __restrict__ qkv,
                                                           const T* __restrict__ ctx,
                                                           const float* __restrict__ lse,
                                                           const T* __restrict__ dctx,
                                                           T* __restrict__ dqkv) {
  extern __shared__ float smem[];
  float(*Kme)[D + 1] = (float(*)[D + 1])smem;                       // this thread's key row
  float(*Vme)[D + 1] = (float(*)[D + 1])(smem + AB * (D + 1));
  float(*Qs)[D + 1] = (float(*)[D + 1])(smem + 2 * AB * (D + 1));   // query block
  float(*dOs)[D + 1] = (float(*)[D + 1])(smem + 3 * AB * (D + 1));
  float* Ls = smem + 4 * AB * (D + 1);
  float* Ds = Ls + AB;
  const int kb = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int j = kb * AB + t;
  const long rs = 3L * nh * D, cs = (long)nh * D;
  const T* base = qkv + (long)b * S * rs + (long)h * 3 * D;
  const float scale = 1.0f / sqrtf((float)D);
  const bool valid = j < S;
  for (int c = 0; c < D; ++c) {
    Kme[t][c] = valid ? to_f32(base[(long)j * rs + D + c]) : 0.f;
    Vme[t][c] = valid ? to_f32(base[(long)j * rs + 2 * D + c]) : 0.f;
  }
  float dk[D], dv[D];
  for (int c = 0; c < D; ++c) { dk[c] = 0.f; dv[c] = 0.f; }
  for (int i0 = kb * AB; i0 < S; i0 += AB) {
    __syncthreads();
    {   // stage query rows i0 .. i0+63: scaled q, dO, LSE and D_i
      const int i = i0 + t;
      float Di = 0.f, li = 0.f;
      if (i < S) {
        const T* o = ctx + ((long)b * S + i) * cs + (long)h * D;
        const T* dO = dctx + ((long)b * S + i) * cs + (long)h * D;
        for (int c = 0; c < D; ++c) {
          const float dov = to_f32(dO[c]);
          Di += dov * to_f32(o[c]);
          dOs[t][c] = dov;
          Qs[t][c] = to_f32(base[(long)i * rs + c]) * scale;
        }
        li = lse[((long)b * nh + h) * S + i];
      } else {
        for (int c = 0; c < D; ++c) { dOs[t][c] = 0.f; Qs[t][c] = 0.f; }
      }
      Ls[t] = li;
      Ds[t] = Di;
    }
    __syncthreads();
    if (valid) {
      const int iend = min(S, i0 + AB);
      for (int i = max(i0, j); i < iend; ++i) {
        const int ii = i - i0;
        float sc = 0.f, dp = 0.f;
        for (int c = 0; c < D; ++c) {
          sc += Qs[ii][c] * Kme[t][c];
          dp += dOs[ii][c] * Vme[t][c];
        }
        const float p = expf(sc - Ls[ii]);
        const float ds = p * (dp - Ds[ii]);
        for (int c = 0; c < D; ++c) {
          dv[c] += p * dOs[ii][c];
          dk[c] += ds * Qs[ii][c];       // q already carries 1/√d
        }
      }
    }
  }
  if (valid) {
    T* out = dqkv + ((long)b * S + j) * rs + (long)h * 3 * D;
    for (int c = 0; c < D; ++c) {
      out[D + c] = from_f32<T>(dk[c]);
      out[2 * D + c] = from_f32<T>(dv[c]);
    }
  }
}

template <typename T, int D>
hipError_t attn_fwd_t(int B, int S, int nh, const void* qkv, void* ctx, float* lse, hipStream_t s) {
  dim3 grid((S + AB - 1) / AB, nh, B);
  attn_fwd_generic<T, D><<<grid, AB, 0, s>>>(S, nh, (const T*)qkv, (T*)ctx, lse);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t attn_bwd_t(int B, int S, int nh, const void* qkv, const void* ctx, const float* lse,
                      const void* dctx, void* dqkv, hipStream_t s) {
  dim3 grid((S + AB - 1) / AB, nh, B);
  const size_t dq_lds = 4 * AB * (D + 1) * sizeof(float);
  const size_t dkv_lds = dq_lds + 2 * AB * sizeof(float);
  hipError_t e = hipFuncSetAttribute((const void*)attn_bwd_dq_generic<T, D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)dq_lds);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)attn_bwd_dkv_generic<T, D>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)dkv_lds);
  if (e != hipSuccess) return e;
  attn_bwd_dq_generic<T, D><<<grid, AB, dq_lds, s>>>(S, nh, (const T*)qkv, (const T*)ctx, lse,
                                                    (const T*)dctx, (T*)dqkv);
  attn_bwd_dkv_generic<T, D><<<grid, AB, dkv_lds, s>>>(S, nh, (const T*)qkv, (const T*)ctx, lse,
                                                      (const T*)dctx, (T*)dqkv);
  return hipGetLastError();
}

template <typename T>
hipError_t fwd_dispatch(int B, int S, int nh, int d, const void* qkv, void* ctx, float* lse,
                        hipStream_t s) {
  switch (d) {
    case 16: return attn_fwd_t<T, 16>(B, S, nh, qkv, ctx, lse, s);
    case 32: return attn_fwd_t<T, 32>(B, S, nh, qkv, ctx, lse, s);
    case 64: return attn_fwd_t<T, 64>(B, S, nh, qkv, ctx, lse, s);
    case 96: return attn_fwd_t<T, 96>(B, S, nh, qkv, ctx, lse, s);
    case 128: return attn_fwd_t<T, 128>(B, S, nh, qkv, ctx, lse, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t bwd_dispatch(int B, int S, int nh, int d, const void* qkv, const void* ctx,
                        const float* lse, const void* dctx, void* dqkv, hipStream_t s) {
  switch (d) {
    case 16: return attn_bwd_t<T, 16>(B, S, nh, qkv, ctx, lse, dctx, dqkv, s);
    case 32: return attn_bwd_t<T, 32>(B, S, nh, qkv, ctx, lse, dctx, dqkv, s);
    case 64: return attn_bwd_t<T, 64>(B, S, nh, qkv, ctx, lse, dctx, dqkv, s);
    case 96: return attn_bwd_t<T, 96>(B, S, nh, qkv, ctx, lse, dctx, dqkv, s);
    case 128: return attn_bwd_t<T, 128>(B, S, nh, qkv, ctx, lse, dctx, dqkv, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool attn_supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 96 || d == 128; }

hipError_t launch_attn_fwd_generic(int dtype, int B, int S, int nh, int d, const void* qkv,
                                   void* ctx, float* lse, hipStream_t s) {
  if (B <= 0 || S <= 0 || nh <= 0) return hipSuccess;
  return dtype == DT_BF16 ? fwd_dispatch<bf16>(B, S, nh, d, qkv, ctx, lse, s)
                          : fwd_dispatch<float>(B, S, nh, d, qkv, ctx, lse, s);
}

hipError_t launch_attn_bwd_generic(int dtype, int B, int S, int nh, int d, const void* qkv,
                                   const void* ctx, const float* lse, const void* dctx, void* dqkv,
                                   hipStream_t s) {
  if (B <= 0 || S <= 0 || nh <= 0) return hipSuccess;
  return dtype == DT_BF16 ? bwd_dispatch<bf16>(B, S, nh, d, qkv, ctx, lse, dctx, dqkv, s)
                          : bwd_dispatch<float>(B, S, nh, d, qkv, ctx, lse, dctx, dqkv, s);
}

}  // namespace tp
