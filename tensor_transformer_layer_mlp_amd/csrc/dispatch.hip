// Kernel selection: the tuned bf16 kernels where the shape allows, the generic ones elsewhere.
// Each launch is wrapped in a ProfScope carrying its kernel tag and algorithmic work.
#include <string>

#include "kernels.h"
#include "prof.h"

namespace tp {

hipError_t launch_gemm_generic(const GemmDesc& d, hipStream_t s);
bool gemm_bf16_eligible(const GemmDesc& d);
const char* gemm_bf16_pick(const GemmDesc& d, int* cfg);
hipError_t launch_gemm_bf16(const GemmDesc& d, int cfg, hipStream_t s);
hipError_t launch_attn_fwd_generic(int dtype, int B, int S, int nh, int d, const void* qkv,
                                   void* ctx, float* lse, hipStream_t s);
hipError_t launch_attn_bwd_generic(int dtype, int B, int S, int nh, int d, const void* qkv,
                                   const void* ctx, const float* lse, const void* dctx, void* dqkv,
                                   hipStream_t s);
hipError_t launch_attn_fwd_mfma(int B, int S, int nh, int d, const void* qkv, void* ctx, float* lse,
                                hipStream_t s);
hipError_t launch_attn_bwd_mfma(int B, int S, int nh, int d, const void* qkv, const void* ctx,
                                const float* lse, const void* dctx, void* dqkv, float* ws,
                                hipStream_t s);

namespace {

const char* tname(int dtype) { return dtype == DT_BF16 ? "__bf16" : "float"; }

// Algorithmic bytes: each operand read once, each output written once (the GeLU' epilogue also
// reads A1; a split-k launch writes one fp32 partial per slice).
double gemm_bytes(const GemmDesc& d) {
  const double es = d.dtype == DT_BF16 ? 2.0 : 4.0;
  const double mn = (double)d.M * d.N;
  const double in = es * ((double)d.M * d.K + (double)d.K * d.N);
  if (d.epi == EPI_F32) return in + 4.0 * (d.ksplit > 1 ? d.ksplit : 1) * mn;
  const double outs = 1.0 + (d.epi == EPI_BIAS_GELU && d.C2 ? 1.0 : 0.0) + (d.epi == EPI_DGELU ? 1.0 : 0.0);
  return in + es * outs * mn;
}

// Visible (query, key) pairs of a causal S x S attention: S(S+1)/2.
double causal_pairs(int S) { return 0.5 * (double)S * ((double)S + 1.0); }

}  // namespace

const char* layout_name(const GemmDesc& d) {
  return d.a_kmajor ? (d.b_kmajor ? "nt" : "nn") : (d.b_kmajor ? "tt" : "tn");
}

hipError_t launch_gemm(const GemmDesc& d, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0) return hipSuccess;
  const double flop = 2.0 * d.M * d.N * (double)d.K;
  if (gemm_bf16_eligible(d)) {
    int cfg = 0;
    const char* tile = gemm_bf16_pick(d, &cfg);
    std::string tag = std::string("gemm_bf16_kernel<") + tile + ", " + layout_name(d) + ", epi" +
                      std::to_string(d.epi) + ">";
    ProfScope p(tag.c_str(), s, flop, gemm_bytes(d));
    return launch_gemm_bf16(d, cfg, s);
  }
  std::string tag = std::string("gemm_generic_kernel<") + tname(d.dtype) + ", " + std::to_string(d.epi) + ">";
  ProfScope p(tag.c_str(), s, flop, gemm_bytes(d));
  return launch_gemm_generic(d, s);
}

hipError_t launch_attn_fwd(int dtype, int B, int S, int nh, int d, const void* qkv, void* ctx,
                           float* lse, hipStream_t s) {
  const double es = dtype == DT_BF16 ? 2.0 : 4.0;
  const double flop = 4.0 * B * nh * d * causal_pairs(S);
  const double bytes = es * (double)B * S * nh * d * 4.0 + 4.0 * B * nh * S;
  if (dtype == DT_BF16) {
    std::string tag = "attn_fwd_mfma<" + std::to_string(d) + ">";
    ProfScope p(tag.c_str(), s, flop, bytes);
    return launch_attn_fwd_mfma(B, S, nh, d, qkv, ctx, lse, s);
  }
  std::string tag = std::string("attn_fwd_generic<") + tname(dtype) + ", " + std::to_string(d) + ">";
  ProfScope p(tag.c_str(), s, flop, bytes);
  return launch_attn_fwd_generic(dtype, B, S, nh, d, qkv, ctx, lse, s);
}

size_t attn_bwd_ws_bytes(int B, int S, int nh, int d) {
  (void)d;
  return (size_t)B * (size_t)S * (size_t)nh * sizeof(float);   // D_i per (b, h, i)
}

hipError_t launch_attn_bwd(int dtype, int B, int S, int nh, int d, const void* qkv,
                           const void* ctx, const float* lse, const void* dctx, void* dqkv,
                           float* ws, hipStream_t s) {
  const double es = dtype == DT_BF16 ? 2.0 : 4.0;
  const double flop = 8.0 * B * nh * d * causal_pairs(S);
  const double bytes = es * (double)B * S * nh * d * 8.0 + 4.0 * B * nh * S;
  if (dtype == DT_BF16) {
    std::string tag = "attn_bwd_mfma<" + std::to_string(d) + ">";
    ProfScope p(tag.c_str(), s, flop, bytes);
    return launch_attn_bwd_mfma(B, S, nh, d, qkv, ctx, lse, dctx, dqkv, ws, s);
  }
  std::string tag = std::string("attn_bwd_generic<") + tname(dtype) + ", " + std::to_string(d) + ">";
  ProfScope p(tag.c_str(), s, flop, bytes);
  return launch_attn_bwd_generic(dtype, B, S, nh, d, qkv, ctx, lse, dctx, dqkv, s);
}

}  // namespace tp
