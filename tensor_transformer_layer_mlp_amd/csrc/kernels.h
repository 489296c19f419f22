// Internal host-side launch interface of libtpshard (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace tp {

enum Dtype { DT_BF16 = 0, DT_F32 = 1 };

// Epilogues fused into the GEMM's store.
enum Epi {
  EPI_STORE = 0,      // C = acc
  EPI_BIAS = 1,       // C = acc + bias[n]
  EPI_BIAS_GELU = 2,  // C2 = acc + bias[n] (if C2), C = GeLU(acc + bias[n])   (GeLU per `act`)
  EPI_DGELU = 3,      // C = acc * GeLU'(aux[m, n])
  EPI_F32 = 4,        // C (fp32) = acc: one k-slice's partial of a split-k GEMM
  EPI_DGELU_GATE = 5  // C = row_scale[m] · acc ∘ GeLU'(aux[m, n]), and row_dot[nt·rd_stride + m] =
                      // Σ_{n in n-tile nt} aux2[m, n] · acc (the MoE backward: gate and its gradient)
};

// C[M, N] = op(A)·op(B) with the epilogue applied.  Element (m, k) of A sits at A[m*lda + k] when
// a_kmajor, else at A[k*lda + m]; element (k, n) of B at B[n*ldb + k] when b_kmajor, else at
// B[k*ldb + n].  C, C2 and aux are row-major with leading dimensions ldc / ldc / ld_aux.
struct GemmDesc {
  int M, N, K;
  const void* A; long lda; bool a_kmajor;
  const void* B; long ldb; bool b_kmajor;
  void* C; long ldc;
  int epi;
  const void* bias;
  const void* aux; long ld_aux;
  void* C2;
  int dtype;
  // Row gather of a K-major A (grouped GEMMs only): when a_rows is set, row m of A is row a_rows[m]
  // of the a_rows_n-row matrix at A; indices outside [0, a_rows_n) read as zero rows.
  const int* a_rows;
  int a_rows_n;
  int act;             // the GeLU epilogues' activation: 0 exact, 1 tanh form
  // Split-k (EPI_F32, both operands K-major): ksplit slices of k_per (a multiple of 64) k each, slice s
  // writing its fp32 partial at C + s·c_split; 0 or 1 = no split
  int ksplit, k_per;
  long c_split;
  // EPI_DGELU_GATE: per-row scale (fp32 [M]), the second auxiliary matrix (storage type, leading
  // dimension ld_aux2) and the per-(n-tile, row) dots (fp32, n-tile nt at nt·rd_stride)
  const float* row_scale;
  const void* aux2; long ld_aux2;
  float* row_dot; long rd_stride;
  // Row gather of an MN-major B's k rows (grouped weight gradients only): k row k of B is row
  // b_rows[k] of the b_rows_n-row matrix at B; indices outside [0, b_rows_n) read as zero rows.
  const int* b_rows;
  int b_rows_n;
};

hipError_t launch_gemm(const GemmDesc& d, hipStream_t s);
// The tile (0: 256 x 256, 8: 256 x 192) of an Xᵀ·dY weight gradient in ks fp32 k-slices.
int gemm_bf16_wgrad_tile(int M, int N, int ks);
// Whether the tiled kernels take this GEMM (shapes, strides, alignment, layout and epilogue).
bool gemm_bf16_eligible(const GemmDesc& d);
// out[i] = Σ_{s < S} parts[s·n + i] in that order, rounded to bf16 (n a multiple of 8).
hipError_t launch_splitk_sum(int S, long n, const float* parts, void* out, hipStream_t s);

// out[c] = Σ_{r < rows} in[r*ld + c] for c < cols, deterministic (fixed chunked order, fp32).
size_t colsum_ws_bytes(int rows, int cols);
hipError_t launch_colsum(int dtype, const void* in, long ld, int rows, int cols, float* ws,
                         void* out, hipStream_t s);
// out[c] = Σ_{k < chunks} ws[k*cols + c] in that order (the second pass of launch_colsum).
hipError_t launch_colsum_final(int dtype, const float* ws, int chunks, int cols, void* out, hipStream_t s);

// Residual add with dropout, then LayerNorm over the H features of each of `rows` rows:
// h = x + o∘keep·keep_scale (o, keep nullable), y = (h − mean)·rstd·γ + β, rstd = 1/√(var + eps).
// In bf16 mode the statistics are taken over h as stored (rounded).  H <= ln_max_h().
int ln_max_h();
hipError_t launch_ln_fwd(int dtype, int rows, int H, const void* x, const void* o, const unsigned char* keep,
                         float keep_scale, const void* gamma, const void* beta, float eps, void* h, void* y,
                         float* mean, float* rstd, hipStream_t s);
// dh = dh_in + rstd·(g − mean(g) − x̂·mean(g·x̂)), g = dy∘γ, x̂ = (h − mean)·rstd; do = dh∘keep·scale;
// dγ = Σ dy∘x̂, dβ = Σ dy over the rows (fp32 partials per row block in ws, then a fixed-order sum).
size_t ln_bwd_ws_bytes(int rows, int H);
hipError_t launch_ln_bwd(int dtype, int rows, int H, const void* dy, const void* dh_in, const void* h,
                         const float* mean, const float* rstd, const void* gamma, const unsigned char* keep,
                         float keep_scale, void* dh, void* d_o, void* dgamma, void* dbeta, float* ws,
                         hipStream_t s);

// Causal attention over nh interleaved heads of width d (see the ABI header for the layout).
bool attn_supported_dim(int d);
hipError_t launch_attn_fwd(int dtype, int B, int S, int nh, int d, const void* qkv, void* ctx,
                           float* lse, hipStream_t s);
size_t attn_bwd_ws_bytes(int B, int S, int nh, int d);
hipError_t launch_attn_bwd(int dtype, int B, int S, int nh, int d, const void* qkv,
                           const void* ctx, const float* lse, const void* dctx, void* dqkv,
                           float* ws, hipStream_t s);

// Grouped expert MLP shard (rows [off[e], off[e+1]) use expert e's weights); off is device memory.
size_t grouped_ws_bytes(int groups, int rows);
// With row_token set, row r of the expert-sorted matrix is row row_token[r] of X (tokens rows),
// gathered inside fc1's operand loads.  With s2 (!= s) and two or more groups, the second half of
// the groups runs on s2 (forked off s after the plan with ev_plan; the caller joins s2 back) and ws
// holds mlp_grouped_ws_bytes(groups, rows, true) bytes, 256-byte aligned.
size_t mlp_grouped_ws_bytes(int groups, int rows, bool split);
hipError_t launch_mlp_grouped(int dtype, int groups, const int* off, int rows, int H, int Fr,
                              const void* X, const void* W1, const void* b1, const void* W2, void* Z,
                              void* A1, void* Y, void* ws, hipStream_t s, const int* row_token = nullptr,
                              int tokens = 0, hipStream_t s2 = nullptr, hipEvent_t ev_plan = nullptr);

// Backward of launch_mlp_grouped on expert-sorted operands (dX may alias dZ); dA1 [rows, Fr] is
// caller scratch; ws as for the forward.  dW1 [groups, H, Fr], db1 [groups, Fr], dW2 [groups, Fr, H].
// With x_rows set, row r of the expert-sorted X is row x_rows[r] of X (x_rows_n rows), gathered.
hipError_t launch_mlp_grouped_bwd(int dtype, int groups, const int* off, int rows, int H, int Fr, const void* X,
                                  const void* W1, const void* W2, const void* A1, const void* Y, const void* dZ,
                                  void* dA1, void* dX, void* dW1, void* db1, void* dW2, void* ws, hipStream_t s,
                                  const int* x_rows = nullptr, int x_rows_n = 0);

// FP8 (OCP E4M3) quantisation with one scale per tensor and the GEMM on codes (see fp8.hip).
size_t fp8_quantize_ws_bytes();
// fmt: 0 E4M3, 1 E5M2.
// q [rows, cols] and qt [cols, rows] codes, each nullable.
hipError_t launch_fp8_quantize(int dtype, int fmt, int rows, int cols, const void* x, unsigned char* q,
                               unsigned char* qt, float* descale, float* ws, hipStream_t s);
// fa, fb: operand formats.  epi: 0 none, 1 GeLU, 2 tanh GeLU, 3 ∘ GeLU'(aux), 4 ∘ tanh GeLU'(aux).
hipError_t launch_fp8_gemm_nt(int M, int N, int K, const unsigned char* A, int fa, const float* da,
                              const unsigned char* B, int fb, const float* db, const void* bias, int epi,
                              const void* aux, void* C, void* C2, hipStream_t s);

// MoE routing and combine (see moe.hip).
int moe_max_experts();
int moe_max_top_k();
size_t moe_route_ws_bytes(int tokens, int experts);
hipError_t launch_moe_route(int tokens, int experts, int top_k, const float* logits, float* gates, int* expert_idx,
                            int* group_offsets, int* row_token, int* token_row, int* ws, hipStream_t s);
// gates nullable: unit gates (the dispatch's backward).
hipError_t launch_moe_combine(int dtype, int tokens, int top_k, int H, const void* Z, const float* gates,
                              const int* token_row, int rows, void* out, hipStream_t s);
// The combine's backward: dZ[r] = gate·d_out[t], Xp[r] = X[t] (Xp nullable), dgates = ⟨d_out[t], Z[r]⟩.
hipError_t launch_moe_combine_bwd(int dtype, int tokens, int k, int H, const void* d_out, const void* X,
                                  const void* Z, const float* gates, const int* token_row, int rows, void* dZ,
                                  void* Xp, float* dgates, hipStream_t s);
// Row r's gate (the gate of the choice whose row r is; 0 if none) and Yg[r] = gate·Y[r].
hipError_t launch_moe_row_gates(int dtype, int tokens, int k, int rows, int Fr, const float* gates,
                                const int* row_token, const int* token_row, const void* Y, float* gate_row, void* Yg,
                                hipStream_t s);
// dgates[t, j] = Σ_{nt < ntiles} row_dot[nt·rows + token_row[t, j]] in that order (0 for a row outside
// [off[0], off[groups]), off the sanitised offsets in device memory).
hipError_t launch_moe_dgates(int tokens, int k, int rows, int ntiles, const float* row_dot, const int* token_row,
                             const int* off, int groups, float* dgates, hipStream_t s);
// The MoE experts' backward from the output gradient (no materialised dZ): see grouped.hip.
size_t moe_experts_bwd_ws_bytes(int groups, int rows, int H, int Fr, int dtype);
// With s2 != s, the weight gradients run on s2 (dW2 after ev_gates, dW1 after ev_dA1, both recorded on
// s here); the caller forks s2 off s before and joins it back after.
hipError_t launch_moe_experts_bwd(int dtype, int groups, const int* off, int tokens, int k, int rows, int H, int Fr,
                                  const void* X, const float* gates, const int* row_token, const int* token_row,
                                  const void* W1, const void* W2, const void* A1, const void* Y, const void* d_out,
                                  void* dX_perm, void* dW1, void* db1, void* dW2, float* dgates, void* ws,
                                  hipStream_t s, hipStream_t s2, hipEvent_t ev_gates, hipEvent_t ev_dA1);
hipError_t launch_moe_route_bwd(int tokens, int E, int k, const float* logits, const int* experts,
                                const float* dgates, float* d_logits, hipStream_t s);

}  // namespace tp
