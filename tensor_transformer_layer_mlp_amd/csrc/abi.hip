// C ABI of libtpshard: argument validation, shard geometry, and the launch sequence of each entry
// point.  Every check happens on the host before anything is enqueued.  See include/tpshard.h.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "tpshard.h"
#include "kernels.h"
#include "prof.h"

using namespace tp;

namespace {

thread_local char g_err[512] = "";

void set_err(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return TP_OK;
  set_err("%s: %s", where, hipGetErrorString(e));
  return TP_EHIP;
}

#define TP_TRY(call, where)                          \
  do {                                               \
    int st_ = hip_status((call), (where));           \
    if (st_ != TP_OK) return st_;                    \
  } while (0)

// The same, with the launches inside labelled by their call site for the per-launch timing.
#define TP_TRY_AT(site, call, where)                 \
  do {                                               \
    ProfSite ps_(site);                              \
    int st_ = hip_status((call), (where));           \
    if (st_ != TP_OK) return st_;                    \
  } while (0)

#define TP_CHECK(cond, code, ...)                    \
  do {                                               \
    if (!(cond)) {                                   \
      set_err(__VA_ARGS__);                          \
      return (code);                                 \
    }                                                \
  } while (0)

// A side stream per caller stream, for launches that do not depend on each other inside one call:
// the caller's stream forks onto it through an event and joins back before the call returns, so the
// caller still sees one ordered stream (and a captured graph gets two branches).  Each (device,
// caller stream) pair gets its own side stream and events, created on first use outside graph
// capture and kept until the process ends, so independent caller streams share nothing; past
// kMaxSides pairs, calls run serially on the caller's stream.  The mutex serialises the host-side
// enqueue phase of the calls that use a side stream (the events are reused from call to call).
struct Side {
  int dev = -1;
  hipStream_t caller = nullptr;
  hipStream_t s2 = nullptr;
  hipEvent_t fork = nullptr, mid = nullptr, join = nullptr;
};
constexpr int kMaxSides = 64;
std::mutex g_side_mu;
Side g_side[kMaxSides];
int g_nside = 0;

bool serial_env() {
  static const bool serial = [] {
    const char* v = getenv("TP_SERIAL");
    return v != nullptr && v[0] != '\0' && v[0] != '0';
  }();
  return serial;
}

// Call with g_side_mu held.
Side* side_stream(hipStream_t s) {
  if (serial_env() || prof_enabled()) return nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  for (int i = 0; i < g_nside; ++i)
    if (g_side[i].dev == dev && g_side[i].caller == s) return &g_side[i];
  if (g_nside == kMaxSides) return nullptr;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return nullptr;
  Side n;
  n.dev = dev;
  n.caller = s;
  if (hipStreamCreateWithFlags(&n.s2, hipStreamNonBlocking) != hipSuccess) return nullptr;
  if (hipEventCreateWithFlags(&n.fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&n.mid, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&n.join, hipEventDisableTiming) != hipSuccess) {
    for (hipEvent_t e : {n.fork, n.mid, n.join})
      if (e) (void)hipEventDestroy(e);
    (void)hipStreamDestroy(n.s2);
    return nullptr;
  }
  g_side[g_nside] = n;
  return &g_side[g_nside++];
}

// Scratch of the entry points that allocate nothing (tp_qkv_shard_bwd_noalloc): one array per
// device, held until the process ends.  Host code never passes the array's name to a kernel (in
// host code it is a stand-in, not a device address): its device address is looked up once per device
// with that device current, on the first call there, and only that address is used.
constexpr size_t kScratchBytes = (size_t)16 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[256] = {};

int scratch_address(void** out) {
  int dev = 0;
  TP_TRY(hipGetDevice(&dev), "hipGetDevice");
  TP_CHECK(dev >= 0 && dev < 256, TP_EUNSUPPORTED, "device %d outside the 256 the scratch table holds", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    TP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    TP_CHECK(p != nullptr && ((uintptr_t)p & 255u) == 0, TP_EHIP, "scratch address %p not 256-byte aligned", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TP_OK;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t esize(int dtype) { return dtype == TP_BF16 ? 2 : 4; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Balanced split, lower ranks take the remainder.
inline void shard(int n, int t, int r, int* off, int* cnt) {
  const int base = n / t, rem = n % t;
  *cnt = base + (r < rem ? 1 : 0);
  *off = r * base + (r < rem ? r : rem);
}

int check_rank_dtype(int tp_size, int rank, int dtype) {
  TP_CHECK(dtype == TP_BF16 || dtype == TP_F32, TP_EINVAL, "dtype %d is neither TP_BF16 nor TP_F32", dtype);
  TP_CHECK(tp_size >= 1, TP_EINVAL, "tp_size %d < 1", tp_size);
  TP_CHECK(rank >= 0 && rank < tp_size, TP_EINVAL, "rank %d outside [0, %d)", rank, tp_size);
  return TP_OK;
}

struct HeadGeom {
  int h0, nh, d, T, Nq;
};

int head_geom(int tp_size, int rank, int B, int S, int H, int n_heads, int dtype, HeadGeom* g) {
  int st = check_rank_dtype(tp_size, rank, dtype);
  if (st) return st;
  TP_CHECK(B >= 0 && S >= 0, TP_EINVAL, "negative batch %d or sequence %d", B, S);
  TP_CHECK(H >= 1 && n_heads >= 1, TP_EINVAL, "H %d and n_heads %d must be >= 1", H, n_heads);
  TP_CHECK(H % n_heads == 0, TP_EINVAL, "H %d is not a multiple of n_heads %d", H, n_heads);
  TP_CHECK(n_heads >= tp_size, TP_EINVAL, "n_heads %d < tp_size %d leaves a rank without heads", n_heads, tp_size);
  TP_CHECK((long)B * S <= INT_MAX / 4, TP_EINVAL, "B*S too large");
  shard(n_heads, tp_size, rank, &g->h0, &g->nh);
  g->d = H / n_heads;
  g->T = B * S;
  g->Nq = 3 * g->nh * g->d;
  return TP_OK;
}

struct MlpGeom {
  int f0, Fr;
};

int mlp_geom(int tp_size, int rank, int T, int H, int F, int dtype, MlpGeom* g) {
  int st = check_rank_dtype(tp_size, rank, dtype);
  if (st) return st;
  TP_CHECK(T >= 0 && T <= INT_MAX / 4, TP_EINVAL, "T %d out of range", T);
  TP_CHECK(H >= 1, TP_EINVAL, "H %d < 1", H);
  TP_CHECK(F >= tp_size, TP_EINVAL, "F %d < tp_size %d leaves a rank without columns", F, tp_size);
  shard(F, tp_size, rank, &g->f0, &g->Fr);
  return TP_OK;
}

// Rows a residual-LayerNorm call covers: all T, or the rank's block of them under sequence parallelism.
int ln_geom(int tp_size, int rank, int sequence_parallel, int T, int H, int dtype, int* rows) {
  int st = check_rank_dtype(tp_size, rank, dtype);
  if (st) return st;
  TP_CHECK(T >= 0 && T <= INT_MAX / 4, TP_EINVAL, "T %d out of range", T);
  TP_CHECK(H >= 1, TP_EINVAL, "H %d < 1", H);
  TP_CHECK(H <= ln_max_h(), TP_EUNSUPPORTED, "H %d above the %d features a LayerNorm row holds", H, ln_max_h());
  int off = 0;
  *rows = T;
  if (sequence_parallel) shard(T, tp_size, rank, &off, rows);
  return TP_OK;
}

// A buffer of n elements: NULL is accepted only when n == 0 (torch gives empty tensors no storage).
#define NEED(p, name, n)                                                              \
  do {                                                                                \
    TP_CHECK((p) != nullptr || (n) == 0, TP_ENULL, "%s is NULL", (name));             \
    TP_CHECK(aligned16(p), TP_EALIGN, "%s is not 16-byte aligned", (name));           \
  } while (0)
// The same for 4-byte element arrays (indices, gates, logits): 4-byte alignment.
#define NEED4(p, name, n)                                                             \
  do {                                                                                \
    TP_CHECK((p) != nullptr || (n) == 0, TP_ENULL, "%s is NULL", (name));             \
    TP_CHECK(((uintptr_t)(p) & 3u) == 0, TP_EALIGN, "%s is not 4-byte aligned", (name)); \
  } while (0)
#define MAYBE(p, name)                                                                   \
  do {                                                                                   \
    TP_CHECK((p) == nullptr || aligned16(p), TP_EALIGN, "%s is not 16-byte aligned", (name)); \
  } while (0)

// k-slices for a weight gradient C[M, N] = Aᵀ·B summed over K tokens (both operands MN-major, the
// 256 x 256 tile).  When the output has few tiles the chip runs one partial round with long k loops;
// slicing k fills more CUs at the price of fp32 partials that a bandwidth pass sums.  Model: rounds
// of 256 tiles x k per slice x 0.02 us (the tile's rate per unit of k) + 0.8 ps per partial element
// (read at about 5 TB/s); each slice at least 1024 deep.  bf16 only.
int wgrad_split(int dtype, int M, int N, int K) {
  if (dtype != DT_BF16 || M <= 0 || N <= 0 || K < 2048) return 1;
  int best = 1;
  double best_t = 1e300;
  for (int ks = 1; ks <= 4 && (long)K >= 1024L * ks; ++ks) {
    // the slices' tile (256 x 256, or 256 x 192 at 0.868 of its time per round: 3/4 of the area at
    // 0.95 / 1.1 of the rate), as the GEMM dispatch picks it for ks slices
    const bool w192 = ks > 1 && gemm_bf16_wgrad_tile(M, N, ks) == 8;
    const long tiles = (long)((M + 255) / 256) * (w192 ? (N + 191) / 192 : (N + 255) / 256);
    const long rounds = (tiles * ks + 255) / 256;
    const double t = (double)rounds * ((double)K / ks) * 0.02 * (w192 ? 0.868 : 1.0) +
                     (ks > 1 ? 0.8e-6 * ks * (double)M * N : 0.0);
    if (t < best_t * 0.97) { best_t = t; best = ks; }
  }
  return best;
}

size_t wgrad_ws(int dtype, int M, int N, int K) {
  const int ks = wgrad_split(dtype, M, N, K);
  return ks > 1 ? align256((size_t)ks * (size_t)M * (size_t)N * sizeof(float)) : 0;
}

// dA1, then the db1 and db2 column-sum partials, then the dW2 and dW1 k-slice partials (separate:
// the sums and the two weight gradients may run concurrently)
size_t mlp_bwd_ws(int T, int H, int Fr, int dtype) {
  return align256((size_t)T * Fr * esize(dtype)) + align256(colsum_ws_bytes(T, Fr)) +
         align256(colsum_ws_bytes(T, H)) + wgrad_ws(dtype, Fr, H, T) + wgrad_ws(dtype, H, Fr, T);
}

// dbqkv's column-sum partials, then dWqkv's k-slice partials (without them when split is false)
size_t qkv_bwd_ws(int T, int H, int Nq, int dtype, bool split = true) {
  return align256(colsum_ws_bytes(T, Nq)) + (split ? wgrad_ws(dtype, H, Nq, T) : 0);
}

// k-slices for the output projection's input gradient dctx = dO·Wo_rᵀ (M = T, N = nh_r·d, K = H): its
// few output tiles would leave most CUs idle, so the k dimension is split until about 256 tiles run,
// each slice at least 512 deep, partials summed afterwards (bf16 only).
int out_bwd_split(int dtype, int T, int Kr, int H) {
  if (dtype != DT_BF16 || T <= 0 || Kr <= 0) return 1;
  const long tiles = (long)((T + 255) / 256) * ((Kr + 191) / 192);
  if (tiles >= 128) return 1;
  const long s = std::min<long>(std::min<long>(4, 256 / tiles), H / 512);
  return (int)std::max<long>(s, 1);
}

size_t out_bwd_ws(int T, int H, int Kr, int dtype) {
  const int sk = out_bwd_split(dtype, T, Kr, H);
  const size_t parts = sk > 1 ? align256((size_t)sk * (size_t)T * (size_t)Kr * sizeof(float)) : 0;
  return align256(colsum_ws_bytes(T, H)) + parts + wgrad_ws(dtype, Kr, H, T);
}

GemmDesc gemm_desc(int dtype, int M, int N, int K, const void* A, long lda, bool a_kmajor,
                   const void* B, long ldb, bool b_kmajor, void* C, long ldc, int epi) {
  GemmDesc d;
  memset(&d, 0, sizeof(d));
  d.M = M; d.N = N; d.K = K;
  d.A = A; d.lda = lda; d.a_kmajor = a_kmajor;
  d.B = B; d.ldb = ldb; d.b_kmajor = b_kmajor;
  d.C = C; d.ldc = ldc; d.epi = epi; d.dtype = dtype;
  return d;
}

// Launches the weight gradient g (both operands MN-major, output bf16 at g.C) as ks k-slices of fp32
// partials in `parts` followed by their sum in slice order, or in one piece when ks <= 1 or the tiled
// kernel does not take the split form.
hipError_t launch_wgrad(const GemmDesc& g, int ks, float* parts, hipStream_t s) {
  if (ks > 1) {
    GemmDesc gs = g;
    gs.epi = EPI_F32;
    gs.C = parts;
    gs.ldc = g.N;
    gs.ksplit = ks;
    gs.k_per = ((g.K + ks - 1) / ks + 63) / 64 * 64;
    gs.c_split = (long)g.M * g.N;
    if (gemm_bf16_eligible(gs) && g.ldc == g.N && ((uintptr_t)g.C & 15) == 0 && ((long)g.M * g.N) % 8 == 0) {
      hipError_t e = launch_gemm(gs, s);
      if (e != hipSuccess) return e;
      return launch_splitk_sum(ks, (long)g.M * g.N, parts, g.C, s);
    }
  }
  return launch_gemm(g, s);
}

}  // namespace

extern "C" {

int tp_shard_range(int n, int tp_size, int rank, int* offset, int* count) {
  TP_CHECK(offset != nullptr && count != nullptr, TP_ENULL, "offset/count is NULL");
  TP_CHECK(n >= 0 && tp_size >= 1 && rank >= 0 && rank < tp_size, TP_EINVAL,
           "bad shard request n=%d tp_size=%d rank=%d", n, tp_size, rank);
  shard(n, tp_size, rank, offset, count);
  return TP_OK;
}

int tp_qkv_shard_fwd(int tp_size, int rank, int B, int S, int H, int n_heads, int dtype,
                     const void* X, const void* Wqkv_r, const void* bqkv_r, void* QKV_r,
                     void* stream) {
  HeadGeom g;
  int st = head_geom(tp_size, rank, B, S, H, n_heads, dtype, &g);
  if (st) return st;
  const long T = g.T;
  NEED(X, "X", T * H); NEED(Wqkv_r, "Wqkv_r", 1); NEED(bqkv_r, "bqkv_r", 1);
  NEED(QKV_r, "QKV_r", T * g.Nq);
  hipStream_t s = (hipStream_t)stream;
  GemmDesc d = gemm_desc(dtype, g.T, g.Nq, H, X, H, true, Wqkv_r, g.Nq, false, QKV_r, g.Nq, EPI_BIAS);
  d.bias = bqkv_r;
  TP_TRY_AT("qkv_fwd", launch_gemm(d, s), "qkv gemm");
  return TP_OK;
}

int tp_attn_heads_fwd(int tp_size, int rank, int B, int S, int H, int n_heads, int dtype,
                      const void* QKV_r, void* ctx_r, float* lse_r, void* stream) {
  HeadGeom g;
  int st = head_geom(tp_size, rank, B, S, H, n_heads, dtype, &g);
  if (st) return st;
  TP_CHECK(attn_supported_dim(g.d), TP_EUNSUPPORTED, "head_dim %d not in {16, 32, 64, 96, 128}", g.d);
  NEED(QKV_r, "QKV_r", (long)g.T); NEED(ctx_r, "ctx_r", (long)g.T); MAYBE(lse_r, "lse_r");
  TP_TRY_AT("attn_fwd", launch_attn_fwd(dtype, B, S, g.nh, g.d, QKV_r, ctx_r, lse_r, (hipStream_t)stream),
            "attention fwd");
  return TP_OK;
}

int tp_mlp_shard_fwd_act(int tp_size, int rank, int T, int H, int F, int dtype, const void* X,
                         const void* W1_r, const void* b1_r, const void* W2_r, const void* b2, void* Z_r,
                         void* A1_r, void* Y_r, int activation, void* stream) {
  TP_CHECK(activation == TP_GELU || activation == TP_GELU_TANH, TP_EINVAL, "activation %d unknown", activation);
  MlpGeom g;
  int st = mlp_geom(tp_size, rank, T, H, F, dtype, &g);
  if (st) return st;
  NEED(X, "X", (long)T); NEED(W1_r, "W1_r", 1); NEED(b1_r, "b1_r", 1); NEED(W2_r, "W2_r", 1);
  NEED(Z_r, "Z_r", (long)T); NEED(Y_r, "Y_r", (long)T); MAYBE(A1_r, "A1_r"); MAYBE(b2, "b2");
  hipStream_t s = (hipStream_t)stream;
  GemmDesc fc1 = gemm_desc(dtype, T, g.Fr, H, X, H, true, W1_r, g.Fr, false, Y_r, g.Fr, EPI_BIAS_GELU);
  fc1.bias = b1_r;
  fc1.C2 = A1_r;
  fc1.act = activation;
  TP_TRY_AT("fc1", launch_gemm(fc1, s), "fc1 gemm");
  const bool add_b2 = (rank == 0 && b2 != nullptr);
  GemmDesc fc2 = gemm_desc(dtype, T, H, g.Fr, Y_r, g.Fr, true, W2_r, H, false, Z_r, H,
                           add_b2 ? EPI_BIAS : EPI_STORE);
  fc2.bias = add_b2 ? b2 : nullptr;
  TP_TRY_AT("fc2", launch_gemm(fc2, s), "fc2 gemm");
  return TP_OK;
}

int tp_mlp_shard_fwd(int tp_size, int rank, int T, int H, int F, int dtype, const void* X,
                     const void* W1_r, const void* b1_r, const void* W2_r, const void* b2, void* Z_r,
                     void* A1_r, void* Y_r, void* stream) {
  return tp_mlp_shard_fwd_act(tp_size, rank, T, H, F, dtype, X, W1_r, b1_r, W2_r, b2, Z_r, A1_r, Y_r, TP_GELU,
                              stream);
}

int tp_mlp_shard_bwd_act(int tp_size, int rank, int T, int H, int F, int dtype, const void* X,
                         const void* W1_r, const void* W2_r, const void* A1_r, const void* Y_r,
                         const void* dZ, void* dX_r, void* dW1_r, void* db1_r, void* dW2_r, void* db2,
                         void* workspace, size_t workspace_bytes, int activation, void* stream) {
  TP_CHECK(activation == TP_GELU || activation == TP_GELU_TANH, TP_EINVAL, "activation %d unknown", activation);
  MlpGeom g;
  int st = mlp_geom(tp_size, rank, T, H, F, dtype, &g);
  if (st) return st;
  NEED(X, "X", (long)T); NEED(W1_r, "W1_r", 1); NEED(W2_r, "W2_r", 1); NEED(A1_r, "A1_r", (long)T);
  NEED(Y_r, "Y_r", (long)T); NEED(dZ, "dZ", (long)T); NEED(dX_r, "dX_r", (long)T);
  NEED(dW1_r, "dW1_r", 1); NEED(db1_r, "db1_r", 1); NEED(dW2_r, "dW2_r", 1); MAYBE(db2, "db2");
  const size_t need = mlp_bwd_ws(T, H, g.Fr, dtype);
  TP_CHECK(workspace != nullptr || need == 0, TP_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  TP_CHECK(workspace_bytes >= need, TP_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  TP_CHECK(workspace == nullptr || ((uintptr_t)workspace & 255u) == 0, TP_EALIGN, "workspace is not 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const int Fr = g.Fr;
  void* dA1 = workspace;
  float* cs1 = (float*)((char*)workspace + align256((size_t)T * Fr * esize(dtype)));
  float* cs2 = (float*)((char*)cs1 + align256(colsum_ws_bytes(T, Fr)));
  float* p2 = (float*)((char*)cs2 + align256(colsum_ws_bytes(T, H)));   // dW2's k-slice partials
  float* p1 = (float*)((char*)p2 + wgrad_ws(dtype, Fr, H, T));          // dW1's
  const int ks2 = wgrad_split(dtype, Fr, H, T), ks1 = wgrad_split(dtype, H, Fr, T);

  // dW2_r = Y_rᵀ·dZ   (M = F_r, N = H, K = T)
  GemmDesc g1 = gemm_desc(dtype, Fr, H, T, Y_r, Fr, false, dZ, H, false, dW2_r, H, EPI_STORE);
  // dA1 = (dZ·W2_rᵀ) ∘ GeLU'(A1_r)   (M = T, N = F_r, K = H)
  GemmDesc g2 = gemm_desc(dtype, T, Fr, H, dZ, H, true, W2_r, H, true, dA1, Fr, EPI_DGELU);
  g2.aux = A1_r;
  g2.ld_aux = Fr;
  g2.act = activation;
  // dW1_r = Xᵀ·dA1   (M = H, N = F_r, K = T)
  GemmDesc g3 = gemm_desc(dtype, H, Fr, T, X, H, false, dA1, Fr, false, dW1_r, Fr, EPI_STORE);
  // dX_r = dA1·W1_rᵀ   (M = T, N = H, K = F_r)
  GemmDesc g4 = gemm_desc(dtype, T, H, Fr, dA1, Fr, true, W1_r, Fr, true, dX_r, H, EPI_STORE);

  // caller's stream: dA1 -> db1, dW1;  side stream: dW2, db2, then (after dA1) dX
  std::lock_guard<std::mutex> lk(g_side_mu);
  Side* sd = side_stream(s);
  hipStream_t s2 = sd ? sd->s2 : s;
  if (sd) {
    TP_TRY(hipEventRecord(sd->fork, s), "fork");
    TP_TRY(hipStreamWaitEvent(s2, sd->fork, 0), "fork");
  }
  auto body = [&]() -> int {
    TP_TRY_AT("dA1", launch_gemm(g2, s), "dA1 gemm");
    if (sd) TP_TRY(hipEventRecord(sd->mid, s), "dA1 event");
    TP_TRY_AT("dW2", launch_wgrad(g1, ks2, p2, s2), "dW2 gemm");
    if (rank == 0 && db2 != nullptr) TP_TRY_AT("db2", launch_colsum(dtype, dZ, H, T, H, cs2, db2, s2), "db2 colsum");
    if (sd) TP_TRY(hipStreamWaitEvent(s2, sd->mid, 0), "dA1 wait");
    TP_TRY_AT("dX_mlp", launch_gemm(g4, s2), "dX gemm");
    TP_TRY_AT("db1", launch_colsum(dtype, dA1, Fr, T, Fr, cs1, db1_r, s), "db1 colsum");
    TP_TRY_AT("dW1", launch_wgrad(g3, ks1, p1, s), "dW1 gemm");
    return TP_OK;
  };
  const int rc = body();
  if (sd) {   // join even after a failed launch, so the side stream never runs ahead of the caller's
    TP_TRY(hipEventRecord(sd->join, s2), "join");
    TP_TRY(hipStreamWaitEvent(s, sd->join, 0), "join");
  }
  return rc;
}

int tp_mlp_shard_bwd(int tp_size, int rank, int T, int H, int F, int dtype, const void* X,
                     const void* W1_r, const void* W2_r, const void* A1_r, const void* Y_r,
                     const void* dZ, void* dX_r, void* dW1_r, void* db1_r, void* dW2_r, void* db2,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return tp_mlp_shard_bwd_act(tp_size, rank, T, H, F, dtype, X, W1_r, W2_r, A1_r, Y_r, dZ, dX_r, dW1_r, db1_r, dW2_r,
                              db2, workspace, workspace_bytes, TP_GELU, stream);
}

}  // extern "C"

namespace {

// The QKV shard backward's launches; `ws` holds the bias gradient's column-sum partials.  With
// use_side, dbqkv and dX run on the caller stream's side stream next to dWqkv.
int qkv_bwd_launch(int dtype, const HeadGeom& g, int H, const void* X, const void* Wqkv_r, const void* dQKV_r,
                   void* dX_r, void* dWqkv_r, void* dbqkv_r, float* ws, hipStream_t s, bool use_side,
                   bool split) {
  // dWqkv_r = Xᵀ·dQKV_r   (M = H, N = Nq, K = T)
  GemmDesc g1 = gemm_desc(dtype, H, g.Nq, g.T, X, H, false, dQKV_r, g.Nq, false, dWqkv_r, g.Nq, EPI_STORE);
  // dX_r = dQKV_r·Wqkv_rᵀ   (M = T, N = H, K = Nq)
  GemmDesc g2 = gemm_desc(dtype, g.T, H, g.Nq, dQKV_r, g.Nq, true, Wqkv_r, g.Nq, true, dX_r, H, EPI_STORE);

  // caller's stream: dWqkv;  side stream: dbqkv, dX (all three independent)
  std::unique_lock<std::mutex> lk(g_side_mu, std::defer_lock);
  Side* sd = nullptr;
  if (use_side) {
    lk.lock();
    sd = side_stream(s);
  }
  hipStream_t s2 = sd ? sd->s2 : s;
  if (sd) {
    TP_TRY(hipEventRecord(sd->fork, s), "fork");
    TP_TRY(hipStreamWaitEvent(s2, sd->fork, 0), "fork");
  }
  auto body = [&]() -> int {
    const int ks = split ? wgrad_split(dtype, H, g.Nq, g.T) : 1;
    float* parts = (float*)((char*)ws + align256(colsum_ws_bytes(g.T, g.Nq)));
    TP_TRY_AT("dWqkv", launch_wgrad(g1, ks, parts, s), "dWqkv gemm");
    TP_TRY_AT("dbqkv", launch_colsum(dtype, dQKV_r, g.Nq, g.T, g.Nq, ws, dbqkv_r, s2), "dbqkv colsum");
    TP_TRY_AT("dX_qkv", launch_gemm(g2, s2), "dX gemm");
    return TP_OK;
  };
  const int rc = body();
  if (sd) {
    TP_TRY(hipEventRecord(sd->join, s2), "join");
    TP_TRY(hipStreamWaitEvent(s, sd->join, 0), "join");
  }
  return rc;
}

int qkv_bwd_args(int tp_size, int rank, int B, int S, int H, int n_heads, int dtype, const void* X,
                 const void* Wqkv_r, const void* dQKV_r, void* dX_r, void* dWqkv_r, void* dbqkv_r, HeadGeom* g) {
  int st = head_geom(tp_size, rank, B, S, H, n_heads, dtype, g);
  if (st) return st;
  NEED(X, "X", (long)g->T); NEED(Wqkv_r, "Wqkv_r", 1); NEED(dQKV_r, "dQKV_r", (long)g->T);
  NEED(dX_r, "dX_r", (long)g->T); NEED(dWqkv_r, "dWqkv_r", 1); NEED(dbqkv_r, "dbqkv_r", 1);
  return TP_OK;
}

}  // namespace

extern "C" {

int tp_qkv_shard_bwd(int tp_size, int rank, int B, int S, int H, int n_heads, int dtype,
                     const void* X, const void* Wqkv_r, const void* dQKV_r, void* dX_r,
                     void* dWqkv_r, void* dbqkv_r, void* workspace, size_t workspace_bytes,
                     void* stream) {
  HeadGeom g;
  int st = qkv_bwd_args(tp_size, rank, B, S, H, n_heads, dtype, X, Wqkv_r, dQKV_r, dX_r, dWqkv_r, dbqkv_r, &g);
  if (st) return st;
  const size_t need = qkv_bwd_ws(g.T, H, g.Nq, dtype);
  TP_CHECK(workspace != nullptr || need == 0, TP_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  TP_CHECK(workspace_bytes >= need, TP_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  TP_CHECK(workspace == nullptr || ((uintptr_t)workspace & 255u) == 0, TP_EALIGN, "workspace is not 256-byte aligned");
  return qkv_bwd_launch(dtype, g, H, X, Wqkv_r, dQKV_r, dX_r, dWqkv_r, dbqkv_r, (float*)workspace,
                        (hipStream_t)stream, true, true);
}

size_t tp_qkv_shard_bwd_noalloc_max_scratch(void) { return kScratchBytes; }

int tp_qkv_shard_bwd_noalloc(int tp_size, int rank, int B, int S, int H, int n_heads, int dtype,
                             const void* X, const void* Wqkv_r, const void* dQKV_r, void* dX_r,
                             void* dWqkv_r, void* dbqkv_r, void* stream) {
  HeadGeom g;
  int st = qkv_bwd_args(tp_size, rank, B, S, H, n_heads, dtype, X, Wqkv_r, dQKV_r, dX_r, dWqkv_r, dbqkv_r, &g);
  if (st) return st;
  const size_t need = qkv_bwd_ws(g.T, H, g.Nq, dtype, false);
  TP_CHECK(need <= kScratchBytes, TP_EWORKSPACE,
           "scratch of %zu bytes needed, above the %zu bytes of the library's scratch array "
           "(ceil(B*S/64)*3*nh_r*d*4 bytes must stay within it)", need, kScratchBytes);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st) return st;
  // Everything on the caller's stream: no side stream or event is created here, and dWqkv is never
  // split along k (its partials would not fit the scratch).  Every partial the column sum's second
  // pass reads is written by its first pass in the same call, so the scratch needs no clearing.
  return qkv_bwd_launch(dtype, g, H, X, Wqkv_r, dQKV_r, dX_r, dWqkv_r, dbqkv_r, (float*)ws,
                        (hipStream_t)stream, false, false);
}

int tp_attn_heads_bwd(int tp_size, int rank, int B, int S, int H, int n_heads, int dtype,
                      const void* QKV_r, const void* ctx_r, const float* lse_r, const void* dctx_r,
                      void* dQKV_r, void* workspace, size_t workspace_bytes, void* stream) {
  HeadGeom g;
  int st = head_geom(tp_size, rank, B, S, H, n_heads, dtype, &g);
  if (st) return st;
  TP_CHECK(attn_supported_dim(g.d), TP_EUNSUPPORTED, "head_dim %d not in {16, 32, 64, 96, 128}", g.d);
  const long T = g.T;
  NEED(QKV_r, "QKV_r", T); NEED(ctx_r, "ctx_r", T); NEED(lse_r, "lse_r", T);
  NEED(dctx_r, "dctx_r", T); NEED(dQKV_r, "dQKV_r", T);
  const size_t need = align256(attn_bwd_ws_bytes(B, S, g.nh, g.d));
  TP_CHECK(workspace != nullptr || need == 0, TP_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  TP_CHECK(workspace_bytes >= need, TP_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  TP_CHECK(workspace == nullptr || ((uintptr_t)workspace & 255u) == 0, TP_EALIGN, "workspace is not 256-byte aligned");
  TP_TRY_AT("attn_bwd", launch_attn_bwd(dtype, B, S, g.nh, g.d, QKV_r, ctx_r, lse_r, dctx_r, dQKV_r,
                         (float*)workspace, (hipStream_t)stream), "attention bwd");
  return TP_OK;
}

int tp_attn_out_shard_fwd(int tp_size, int rank, int B, int S, int H, int n_heads, int dtype,
                          const void* ctx_r, const void* Wo_r, const void* bo, void* O_r,
                          void* stream) {
  HeadGeom g;
  int st = head_geom(tp_size, rank, B, S, H, n_heads, dtype, &g);
  if (st) return st;
  const int Kr = g.nh * g.d;
  NEED(ctx_r, "ctx_r", (long)g.T); NEED(Wo_r, "Wo_r", 1); NEED(O_r, "O_r", (long)g.T); MAYBE(bo, "bo");
  const bool add_bo = (rank == 0 && bo != nullptr);
  // O_r = ctx_r·Wo_r (+ bo)   (M = T, N = H, K = nh_r*d)
  GemmDesc d = gemm_desc(dtype, g.T, H, Kr, ctx_r, Kr, true, Wo_r, H, false, O_r, H,
                         add_bo ? EPI_BIAS : EPI_STORE);
  d.bias = add_bo ? bo : nullptr;
  TP_TRY_AT("out_fwd", launch_gemm(d, (hipStream_t)stream), "out-proj gemm");
  return TP_OK;
}

int tp_attn_out_shard_bwd(int tp_size, int rank, int B, int S, int H, int n_heads, int dtype,
                          const void* ctx_r, const void* Wo_r, const void* dO, void* dctx_r,
                          void* dWo_r, void* dbo, void* workspace, size_t workspace_bytes,
                          void* stream) {
  HeadGeom g;
  int st = head_geom(tp_size, rank, B, S, H, n_heads, dtype, &g);
  if (st) return st;
  const int Kr = g.nh * g.d;
  NEED(ctx_r, "ctx_r", (long)g.T); NEED(Wo_r, "Wo_r", 1); NEED(dO, "dO", (long)g.T);
  NEED(dctx_r, "dctx_r", (long)g.T); NEED(dWo_r, "dWo_r", 1); MAYBE(dbo, "dbo");
  const size_t need = out_bwd_ws(g.T, H, Kr, dtype);
  TP_CHECK(workspace != nullptr || need == 0, TP_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  TP_CHECK(workspace_bytes >= need, TP_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  TP_CHECK(workspace == nullptr || ((uintptr_t)workspace & 255u) == 0, TP_EALIGN, "workspace is not 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  // dWo_r = ctx_rᵀ·dO   (M = nh_r*d, N = H, K = T)
  GemmDesc g1 = gemm_desc(dtype, Kr, H, g.T, ctx_r, Kr, false, dO, H, false, dWo_r, H, EPI_STORE);
  // dctx_r = dO·Wo_rᵀ   (M = T, N = nh_r*d, K = H); with few output tiles, as k-slices into fp32
  // partials behind the column-sum workspace, then summed in slice order
  GemmDesc g2 = gemm_desc(dtype, g.T, Kr, H, dO, H, true, Wo_r, H, true, dctx_r, Kr, EPI_STORE);
  const int sk = out_bwd_split(dtype, g.T, Kr, H);
  float* parts = (float*)((char*)workspace + align256(colsum_ws_bytes(g.T, H)));
  const size_t dctx_parts = sk > 1 ? align256((size_t)sk * (size_t)g.T * (size_t)Kr * sizeof(float)) : 0;
  float* wparts = (float*)((char*)parts + dctx_parts);   // dWo's k-slice partials
  const int ksw = wgrad_split(dtype, Kr, H, g.T);
  if (sk > 1) {
    GemmDesc gs = g2;
    gs.epi = EPI_F32;
    gs.C = parts;
    gs.ksplit = sk;
    gs.k_per = ((H + sk - 1) / sk + 63) / 64 * 64;
    gs.c_split = (long)g.T * Kr;
    if (gemm_bf16_eligible(gs) && ((uintptr_t)dctx_r & 15) == 0) g2 = gs;   // the sum stores 16-byte pieces
  }

  // caller's stream: dWo;  side stream: dbo (rank 0), dctx (all independent)
  std::lock_guard<std::mutex> lk(g_side_mu);
  Side* sd = side_stream(s);
  hipStream_t s2 = sd ? sd->s2 : s;
  if (sd) {
    TP_TRY(hipEventRecord(sd->fork, s), "fork");
    TP_TRY(hipStreamWaitEvent(s2, sd->fork, 0), "fork");
  }
  auto body = [&]() -> int {
    TP_TRY_AT("dWo", launch_wgrad(g1, ksw, wparts, s), "dWo gemm");
    if (rank == 0 && dbo != nullptr)
      TP_TRY_AT("dbo", launch_colsum(dtype, dO, H, g.T, H, (float*)workspace, dbo, s2), "dbo colsum");
    TP_TRY_AT("dctx", launch_gemm(g2, s2), "dctx gemm");
    if (g2.epi == EPI_F32)
      TP_TRY_AT("dctx", launch_splitk_sum(g2.ksplit, (long)g.T * Kr, parts, dctx_r, s2), "dctx slice sum");
    return TP_OK;
  };
  const int rc = body();
  if (sd) {
    TP_TRY(hipEventRecord(sd->join, s2), "join");
    TP_TRY(hipStreamWaitEvent(s, sd->join, 0), "join");
  }
  return rc;
}

int tp_residual_ln_fwd(int tp_size, int rank, int sequence_parallel, int T, int H, int dtype,
                       const void* x, const void* o, const unsigned char* keep, float p_drop,
                       const void* gamma, const void* beta, float eps, void* h, void* y, float* mean,
                       float* rstd, void* stream) {
  int rows = 0;
  int st = ln_geom(tp_size, rank, sequence_parallel, T, H, dtype, &rows);
  if (st) return st;
  TP_CHECK(std::isfinite(p_drop) && p_drop >= 0.f && p_drop < 1.f, TP_EINVAL, "p_drop %g outside [0, 1)", p_drop);
  TP_CHECK(std::isfinite(eps) && eps >= 0.f, TP_EINVAL, "eps %g is negative or not finite", eps);
  const long n = (long)rows * H;
  NEED(x, "x", n); MAYBE(o, "o"); MAYBE(keep, "keep"); NEED(gamma, "gamma", H); NEED(beta, "beta", H);
  NEED(y, "y", n); NEED(mean, "mean", rows); NEED(rstd, "rstd", rows);
  if (o) NEED(h, "h", n); else MAYBE(h, "h");
  TP_TRY(launch_ln_fwd(dtype, rows, H, x, o, keep, (float)(1.0 / (1.0 - (double)p_drop)), gamma, beta, eps, h, y,
                       mean, rstd, (hipStream_t)stream), "residual layernorm fwd");
  return TP_OK;
}

int tp_residual_ln_bwd(int tp_size, int rank, int sequence_parallel, int T, int H, int dtype,
                       const void* dy, const void* dh_in, const void* h, const float* mean,
                       const float* rstd, const void* gamma, const unsigned char* keep, float p_drop,
                       void* dh, void* d_o, void* dgamma, void* dbeta, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int rows = 0;
  int st = ln_geom(tp_size, rank, sequence_parallel, T, H, dtype, &rows);
  if (st) return st;
  TP_CHECK(std::isfinite(p_drop) && p_drop >= 0.f && p_drop < 1.f, TP_EINVAL, "p_drop %g outside [0, 1)", p_drop);
  const long n = (long)rows * H;
  NEED(dy, "dy", n); MAYBE(dh_in, "dh_in"); NEED(h, "h", n); NEED(mean, "mean", rows); NEED(rstd, "rstd", rows);
  NEED(gamma, "gamma", H); MAYBE(keep, "keep"); NEED(dh, "dh", n); MAYBE(d_o, "d_o");
  NEED(dgamma, "dgamma", H); NEED(dbeta, "dbeta", H);
  const size_t need = align256(ln_bwd_ws_bytes(rows, H));
  TP_CHECK(workspace != nullptr || need == 0, TP_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  TP_CHECK(workspace_bytes >= need, TP_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  TP_CHECK(workspace == nullptr || ((uintptr_t)workspace & 255u) == 0, TP_EALIGN, "workspace is not 256-byte aligned");
  TP_TRY(launch_ln_bwd(dtype, rows, H, dy, dh_in, h, mean, rstd, gamma, keep, (float)(1.0 / (1.0 - (double)p_drop)),
                       dh, d_o, dgamma, dbeta, (float*)workspace, (hipStream_t)stream), "residual layernorm bwd");
  return TP_OK;
}

// Workspace of the grouped forward: room for the plans of both halves (see grouped_fwd below).
static size_t grouped_fwd_ws(int groups, int rows) { return mlp_grouped_ws_bytes(groups, rows, true); }

// The grouped expert MLP forward.  With a side stream and two or more groups, the second half of
// the groups runs there: the halves' rows, weights and outputs are disjoint, so each half's fc2
// overlaps the other's fc1 and the tail waves of each GEMM share the chip with the other half's
// tiles.  Every element's arithmetic is the same as in one launch over all groups.
static int grouped_fwd(int dtype, int groups, const int* off, int rows, int H, int Fr, const void* X,
                       const void* W1, const void* b1, const void* W2, void* Z, void* A1, void* Y, void* ws,
                       hipStream_t s, const int* row_token, int tokens) {
  std::lock_guard<std::mutex> lk(g_side_mu);
  Side* sd = groups >= 2 ? side_stream(s) : nullptr;
  const hipError_t e = launch_mlp_grouped(dtype, groups, off, rows, H, Fr, X, W1, b1, W2, Z, A1, Y, ws, s,
                                          row_token, tokens, sd ? sd->s2 : nullptr, sd ? sd->fork : nullptr);
  if (sd != nullptr) {   // joined even after a failed launch, so the side stream never outruns s
    TP_TRY(hipEventRecord(sd->join, sd->s2), "join");
    TP_TRY(hipStreamWaitEvent(s, sd->join, 0), "join");
  }
  TP_TRY(e, "grouped mlp");
  return TP_OK;
}

int tp_mlp_grouped_shard_fwd(int tp_size, int rank, int n_groups, const int* group_offsets, int rows,
                             int H, int F_group, int dtype, const void* X_perm, const void* W1_r,
                             const void* b1_r, const void* W2_r, void* Z_r, void* A1_r, void* Y_r,
                             void* workspace, size_t workspace_bytes, void* stream) {
  MlpGeom g;
  int st = mlp_geom(tp_size, rank, rows, H, F_group, dtype, &g);
  if (st) return st;
  TP_CHECK(n_groups >= 1 && n_groups <= (1 << 20), TP_EINVAL, "n_groups %d out of range", n_groups);
  TP_CHECK(group_offsets != nullptr, TP_ENULL, "group_offsets is NULL");
  TP_CHECK(((uintptr_t)group_offsets & 3u) == 0, TP_EALIGN, "group_offsets is not 4-byte aligned");
  NEED(X_perm, "X_perm", (long)rows); NEED(W1_r, "W1_r", 1); NEED(b1_r, "b1_r", 1); NEED(W2_r, "W2_r", 1);
  NEED(Z_r, "Z_r", (long)rows); NEED(Y_r, "Y_r", (long)rows); MAYBE(A1_r, "A1_r");
  const size_t need = grouped_fwd_ws(n_groups, rows);
  TP_CHECK(workspace != nullptr, TP_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  TP_CHECK(workspace_bytes >= need, TP_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  TP_CHECK(((uintptr_t)workspace & 255u) == 0, TP_EALIGN, "workspace is not 256-byte aligned");
  return grouped_fwd(dtype, n_groups, group_offsets, rows, H, g.Fr, X_perm, W1_r, b1_r, W2_r, Z_r, A1_r, Y_r,
                     workspace, (hipStream_t)stream, nullptr, 0);
}

int tp_moe_route(int tokens, int n_experts, int top_k, const float* logits, float* gates, int* expert_idx,
                 int* group_offsets, int* row_token, int* token_row, void* workspace, size_t workspace_bytes,
                 void* stream) {
  TP_CHECK(tokens >= 0, TP_EINVAL, "tokens %d < 0", tokens);
  TP_CHECK(n_experts >= 1 && n_experts <= moe_max_experts(), TP_EUNSUPPORTED, "n_experts %d outside [1, %d]",
           n_experts, moe_max_experts());
  TP_CHECK(top_k >= 1 && top_k <= n_experts && top_k <= moe_max_top_k(), TP_EINVAL,
           "top_k %d outside [1, min(n_experts, %d)]", top_k, moe_max_top_k());
  TP_CHECK((long)tokens * top_k <= INT_MAX / 4 && (long)tokens * n_experts <= INT_MAX, TP_EINVAL, "too many tokens");
  const long n = (long)tokens * top_k;
  NEED4(logits, "logits", (long)tokens * n_experts); NEED4(gates, "gates", n); NEED4(expert_idx, "expert_idx", n);
  NEED4(group_offsets, "group_offsets", n_experts + 1); NEED4(row_token, "row_token", n);
  NEED4(token_row, "token_row", n);
  const size_t need = align256(moe_route_ws_bytes(tokens, n_experts));
  TP_CHECK(workspace != nullptr || need == 0, TP_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  TP_CHECK(workspace_bytes >= need, TP_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  TP_CHECK(workspace == nullptr || ((uintptr_t)workspace & 255u) == 0, TP_EALIGN, "workspace is not 256-byte aligned");
  TP_TRY(launch_moe_route(tokens, n_experts, top_k, logits, gates, expert_idx, group_offsets, row_token, token_row,
                          (int*)workspace, (hipStream_t)stream), "moe route");
  return TP_OK;
}

int tp_moe_shard_fwd(int tp_size, int rank, int tokens, int H, int n_experts, int top_k, int F_expert, int dtype,
                     const void* X, const float* gates, const int* group_offsets, const int* row_token,
                     const int* token_row, const void* W1_r, const void* b1_r, const void* W2_r, void* out_r,
                     void* Z_r, void* A1_r, void* Y_r, void* workspace, size_t workspace_bytes, void* stream) {
  TP_CHECK(tokens >= 0 && top_k >= 1 && (long)tokens * top_k <= INT_MAX / 4, TP_EINVAL,
           "tokens %d, top_k %d out of range", tokens, top_k);
  TP_CHECK(n_experts >= 1 && n_experts <= (1 << 20), TP_EINVAL, "n_experts %d out of range", n_experts);
  TP_CHECK(top_k <= n_experts, TP_EINVAL, "top_k %d > n_experts %d", top_k, n_experts);
  const int rows = tokens * top_k;
  MlpGeom g;
  int st = mlp_geom(tp_size, rank, rows, H, F_expert, dtype, &g);
  if (st) return st;
  const long n = (long)rows;
  NEED(X, "X", (long)tokens * H); NEED4(gates, "gates", n); NEED4(group_offsets, "group_offsets", 1);
  NEED4(row_token, "row_token", n); NEED4(token_row, "token_row", n);
  NEED(W1_r, "W1_r", 1); NEED(b1_r, "b1_r", 1); NEED(W2_r, "W2_r", 1); NEED(out_r, "out_r", (long)tokens * H);
  NEED(Z_r, "Z_r", n * H); NEED(Y_r, "Y_r", n); MAYBE(A1_r, "A1_r");
  const size_t need = grouped_fwd_ws(n_experts, rows);
  TP_CHECK(workspace != nullptr, TP_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  TP_CHECK(workspace_bytes >= need, TP_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  TP_CHECK(((uintptr_t)workspace & 255u) == 0, TP_EALIGN, "workspace is not 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  st = grouped_fwd(dtype, n_experts, group_offsets, rows, H, g.Fr, X, W1_r, b1_r, W2_r, Z_r, A1_r, Y_r, workspace, s,
                   row_token, tokens);
  if (st) return st;
  TP_TRY(launch_moe_combine(dtype, tokens, top_k, H, Z_r, gates, token_row, rows, out_r, s), "moe combine");
  return TP_OK;
}

int tp_mlp_grouped_shard_bwd(int tp_size, int rank, int n_groups, const int* group_offsets, int rows, int H,
                             int F_group, int dtype, const void* X_perm, const void* W1_r, const void* W2_r,
                             const void* A1_r, const void* Y_r, const void* dZ_perm, void* dX_perm, void* dW1_r,
                             void* db1_r, void* dW2_r, void* workspace, size_t workspace_bytes, void* stream) {
  MlpGeom g;
  int st = mlp_geom(tp_size, rank, rows, H, F_group, dtype, &g);
  if (st) return st;
  TP_CHECK(n_groups >= 1 && n_groups <= 65535, TP_EINVAL, "n_groups %d out of range", n_groups);
  NEED4(group_offsets, "group_offsets", n_groups + 1);
  NEED(X_perm, "X_perm", (long)rows); NEED(W1_r, "W1_r", 1); NEED(W2_r, "W2_r", 1); NEED(A1_r, "A1_r", (long)rows);
  NEED(Y_r, "Y_r", (long)rows); NEED(dZ_perm, "dZ_perm", (long)rows); NEED(dX_perm, "dX_perm", (long)rows);
  NEED(dW1_r, "dW1_r", 1); NEED(db1_r, "db1_r", 1); NEED(dW2_r, "dW2_r", 1);
  const size_t plan = align256(grouped_ws_bytes(n_groups, rows));
  const size_t need = plan + align256((size_t)rows * g.Fr * (dtype == TP_BF16 ? 2 : 4));
  TP_CHECK(workspace != nullptr, TP_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  TP_CHECK(workspace_bytes >= need, TP_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  TP_CHECK(((uintptr_t)workspace & 255u) == 0, TP_EALIGN, "workspace is not 256-byte aligned");
  TP_TRY(launch_mlp_grouped_bwd(dtype, n_groups, group_offsets, rows, H, g.Fr, X_perm, W1_r, W2_r, A1_r, Y_r, dZ_perm,
                                (char*)workspace + plan, dX_perm, dW1_r, db1_r, dW2_r, workspace, (hipStream_t)stream),
         "grouped mlp backward");
  return TP_OK;
}

static size_t moe_bwd_ws(int rows, int H, int Fr, int E, int dtype) {
  const size_t es = dtype == TP_BF16 ? 2 : 4;
  return align256(moe_experts_bwd_ws_bytes(E, rows, H, Fr, dtype)) + align256((size_t)rows * H * es);
}

int tp_moe_shard_bwd(int tp_size, int rank, int tokens, int H, int n_experts, int top_k, int F_expert, int dtype,
                     const void* X, const float* gates, const int* group_offsets, const int* row_token,
                     const int* token_row, const void* W1_r, const void* W2_r, const void* A1_r, const void* Y_r,
                     const void* Z_r, const void* d_out, void* dX_r, float* dgates_r, void* dW1_r, void* db1_r,
                     void* dW2_r, void* workspace, size_t workspace_bytes, void* stream) {
  TP_CHECK(tokens >= 0 && top_k >= 1 && (long)tokens * top_k <= INT_MAX / 4, TP_EINVAL,
           "tokens %d, top_k %d out of range", tokens, top_k);
  TP_CHECK(n_experts >= 1 && n_experts <= 65535, TP_EINVAL, "n_experts %d out of range", n_experts);
  TP_CHECK(top_k <= n_experts, TP_EINVAL, "top_k %d > n_experts %d", top_k, n_experts);
  const int rows = tokens * top_k;
  MlpGeom g;
  int st = mlp_geom(tp_size, rank, rows, H, F_expert, dtype, &g);
  if (st) return st;
  const long n = (long)rows;
  NEED(X, "X", (long)tokens * H); NEED4(gates, "gates", n); NEED4(group_offsets, "group_offsets", n_experts + 1);
  NEED4(row_token, "row_token", n); NEED4(token_row, "token_row", n); NEED(W1_r, "W1_r", 1); NEED(W2_r, "W2_r", 1);
  NEED(A1_r, "A1_r", n);
  NEED(Y_r, "Y_r", n); MAYBE(Z_r, "Z_r"); NEED(d_out, "d_out", (long)tokens * H);
  NEED(dX_r, "dX_r", (long)tokens * H); NEED4(dgates_r, "dgates_r", n); NEED(dW1_r, "dW1_r", 1);
  NEED(db1_r, "db1_r", 1); NEED(dW2_r, "dW2_r", 1);
  const size_t need = moe_bwd_ws(rows, H, g.Fr, n_experts, dtype);
  TP_CHECK(workspace != nullptr, TP_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  TP_CHECK(workspace_bytes >= need, TP_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  TP_CHECK(((uintptr_t)workspace & 255u) == 0, TP_EALIGN, "workspace is not 256-byte aligned");
  (void)Z_r;   // the gate gradients come from Y_r and W2_r inside the dA1 GEMM
  char* experts_ws = (char*)workspace;
  char* dXp = experts_ws + align256(moe_experts_bwd_ws_bytes(n_experts, rows, H, g.Fr, dtype));
  hipStream_t s = (hipStream_t)stream;
  // the combine's backward is folded into the experts' GEMMs: d_out's rows are gathered by row_token
  // and scaled by their gates inside them, and X's rows likewise inside dW1's loads.  The two weight
  // gradients run on the side stream next to dA1, dX_perm and the dispatch's backward.
  std::lock_guard<std::mutex> lk(g_side_mu);
  Side* sd = side_stream(s);
  hipStream_t s2 = sd ? sd->s2 : s;
  auto body = [&]() -> int {
    TP_TRY(launch_moe_experts_bwd(dtype, n_experts, group_offsets, tokens, top_k, rows, H, g.Fr, X, gates, row_token,
                                  token_row, W1_r, W2_r, A1_r, Y_r, d_out, dXp, dW1_r, db1_r, dW2_r, dgates_r,
                                  experts_ws, s, s2, sd ? sd->fork : nullptr, sd ? sd->mid : nullptr),
           "moe experts backward");
    TP_TRY(launch_moe_combine(dtype, tokens, top_k, H, dXp, nullptr, token_row, rows, dX_r, s),
           "moe dispatch backward");
    return TP_OK;
  };
  const int rc = body();
  if (sd) {   // join even after a failed launch, so the side stream never runs ahead of the caller's
    TP_TRY(hipEventRecord(sd->join, s2), "join");
    TP_TRY(hipStreamWaitEvent(s, sd->join, 0), "join");
  }
  return rc;
}

int tp_moe_route_bwd(int tokens, int n_experts, int top_k, const float* logits, const int* expert_idx,
                     const float* dgates, float* d_logits, void* stream) {
  TP_CHECK(tokens >= 0, TP_EINVAL, "tokens %d < 0", tokens);
  TP_CHECK(n_experts >= 1 && n_experts <= moe_max_experts(), TP_EUNSUPPORTED, "n_experts %d outside [1, %d]",
           n_experts, moe_max_experts());
  TP_CHECK(top_k >= 1 && top_k <= n_experts && top_k <= moe_max_top_k(), TP_EINVAL,
           "top_k %d outside [1, min(n_experts, %d)]", top_k, moe_max_top_k());
  TP_CHECK((long)tokens * n_experts <= INT_MAX, TP_EINVAL, "too many tokens");
  const long n = (long)tokens * top_k;
  NEED4(logits, "logits", (long)tokens * n_experts); NEED4(expert_idx, "expert_idx", n);
  NEED4(dgates, "dgates", n); NEED4(d_logits, "d_logits", (long)tokens * n_experts);
  TP_TRY(launch_moe_route_bwd(tokens, n_experts, top_k, logits, expert_idx, dgates, d_logits, (hipStream_t)stream),
         "moe route backward");
  return TP_OK;
}

int tp_fp8_quantize(int rows, int cols, int dtype, const void* x, int format, unsigned char* q, unsigned char* q_t,
                    float* descale, void* workspace, size_t workspace_bytes, void* stream) {
  TP_CHECK(dtype == TP_BF16 || dtype == TP_F32, TP_EINVAL, "dtype %d is neither TP_BF16 nor TP_F32", dtype);
  TP_CHECK(format == TP_FP8_E4M3 || format == TP_FP8_E5M2, TP_EINVAL, "format %d is neither E4M3 nor E5M2", format);
  TP_CHECK(rows >= 0 && cols >= 0, TP_EINVAL, "negative size %d x %d", rows, cols);
  const long n = (long)rows * cols;
  TP_CHECK(q != nullptr || q_t != nullptr || n == 0, TP_ENULL, "q and q_t are both NULL");
  NEED(x, "x", n); MAYBE(q, "q"); MAYBE(q_t, "q_t"); NEED4(descale, "descale", 1);
  const size_t need = align256(fp8_quantize_ws_bytes());
  TP_CHECK(workspace != nullptr, TP_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  TP_CHECK(workspace_bytes >= need, TP_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  TP_CHECK(((uintptr_t)workspace & 255u) == 0, TP_EALIGN, "workspace is not 256-byte aligned");
  TP_TRY(launch_fp8_quantize(dtype, format, rows, cols, x, q, q_t, descale, (float*)workspace, (hipStream_t)stream),
         "fp8 quantize");
  return TP_OK;
}

int tp_fp8_gemm_nt(int M, int N, int K, const unsigned char* A, int a_format, const float* a_descale,
                   const unsigned char* B, int b_format, const float* b_descale, const void* bias, int epilogue,
                   const void* aux, void* C, void* C_pre, void* stream) {
  TP_CHECK(M >= 0 && N >= 0 && K >= 0, TP_EINVAL, "negative size %d x %d x %d", M, N, K);
  TP_CHECK((a_format == TP_FP8_E4M3 || a_format == TP_FP8_E5M2) && (b_format == TP_FP8_E4M3 || b_format == TP_FP8_E5M2),
           TP_EINVAL, "formats %d, %d are not E4M3 / E5M2", a_format, b_format);
  TP_CHECK(!(a_format == TP_FP8_E5M2 && b_format == TP_FP8_E5M2), TP_EUNSUPPORTED, "two E5M2 operands");
  TP_CHECK(epilogue >= TP_FP8_EPI_NONE && epilogue <= TP_FP8_EPI_DGELU_TANH, TP_EINVAL, "epilogue %d unknown", epilogue);
  TP_CHECK(K % 16 == 0, TP_EUNSUPPORTED, "K %d is not a multiple of 16 (rows of 16-byte pieces)", K);
  TP_CHECK(N % 8 == 0, TP_EUNSUPPORTED, "N %d is not a multiple of 8", N);
  TP_CHECK((long)M * K < 0x7fffffffL && (long)N * K < 0x7fffffffL, TP_EUNSUPPORTED, "an operand above 2 GiB");
  NEED(A, "A", (long)M * K); NEED(B, "B", (long)N * K); NEED4(a_descale, "a_descale", 1);
  NEED4(b_descale, "b_descale", 1); NEED(C, "C", (long)M * N); MAYBE(bias, "bias"); MAYBE(C_pre, "C_pre");
  const bool dg = epilogue == TP_FP8_EPI_DGELU || epilogue == TP_FP8_EPI_DGELU_TANH;
  if (dg) NEED(aux, "aux", (long)M * N); else MAYBE(aux, "aux");
  const bool g = epilogue == TP_FP8_EPI_GELU || epilogue == TP_FP8_EPI_GELU_TANH;
  TP_TRY(launch_fp8_gemm_nt(M, N, K, A, a_format, a_descale, B, b_format, b_descale, bias, epilogue,
                            dg ? aux : nullptr, C, g ? C_pre : nullptr, (hipStream_t)stream), "fp8 gemm");
  return TP_OK;
}

int tp_bias_grad(int rows, int cols, int dtype, const void* dy, void* db, void* workspace, size_t workspace_bytes,
                 void* stream) {
  TP_CHECK(dtype == TP_BF16 || dtype == TP_F32, TP_EINVAL, "dtype %d is neither TP_BF16 nor TP_F32", dtype);
  TP_CHECK(rows >= 0 && cols >= 0, TP_EINVAL, "negative size %d x %d", rows, cols);
  NEED(dy, "dy", (long)rows * cols); NEED(db, "db", cols);
  const size_t need = align256(colsum_ws_bytes(rows, cols));
  TP_CHECK(workspace != nullptr, TP_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  TP_CHECK(workspace_bytes >= need, TP_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  TP_CHECK(((uintptr_t)workspace & 255u) == 0, TP_EALIGN, "workspace is not 256-byte aligned");
  TP_TRY(launch_colsum(dtype, dy, cols, rows, cols, (float*)workspace, db, (hipStream_t)stream), "bias grad");
  return TP_OK;
}

size_t tp_workspace_bytes(const char* fn, int tp_size, int rank, int B, int S, int H, int n_heads,
                          int F, int dtype) {
  if (fn == nullptr) return 0;
  if (strcmp(fn, "tp_mlp_shard_bwd") == 0) {
    MlpGeom g;
    if (B < 0 || S < 0 || (long)B * S > INT_MAX / 4) return 0;
    if (mlp_geom(tp_size, rank, B * S, H, F, dtype, &g)) return 0;
    return mlp_bwd_ws(B * S, H, g.Fr, dtype);
  }
  HeadGeom g;
  if (strcmp(fn, "tp_qkv_shard_bwd") == 0) {
    if (head_geom(tp_size, rank, B, S, H, n_heads, dtype, &g)) return 0;
    return qkv_bwd_ws(g.T, H, g.Nq, dtype);
  }
  if (strcmp(fn, "tp_fp8_quantize") == 0) return align256(fp8_quantize_ws_bytes());
  if (strcmp(fn, "tp_bias_grad") == 0) {
    if (B < 0 || S < 0 || H < 0 || (long)B * S > INT_MAX / 4) return 0;
    return align256(colsum_ws_bytes(B * S, H));
  }
  if (strcmp(fn, "tp_moe_route") == 0) {
    if (B < 0 || S < 0 || (long)B * S > INT_MAX / 4 || n_heads < 1 || n_heads > moe_max_experts()) return 0;
    return align256(moe_route_ws_bytes(B * S, n_heads));
  }
  if (strcmp(fn, "tp_mlp_grouped_shard_bwd") == 0 || strcmp(fn, "tp_moe_shard_bwd") == 0) {
    MlpGeom mg;
    if (B < 0 || S < 0 || (long)B * S > INT_MAX / 4 || n_heads < 1 || n_heads > 65535) return 0;
    if (mlp_geom(tp_size, rank, B * S, H, F, dtype, &mg)) return 0;
    if (strcmp(fn, "tp_moe_shard_bwd") == 0) return moe_bwd_ws(B * S, H, mg.Fr, n_heads, dtype);
    return align256(grouped_ws_bytes(n_heads, B * S)) + align256((size_t)B * S * mg.Fr * (dtype == TP_BF16 ? 2 : 4));
  }
  if (strcmp(fn, "tp_mlp_grouped_shard_fwd") == 0 || strcmp(fn, "tp_moe_shard_fwd") == 0) {
    if (B < 0 || S < 0 || (long)B * S > INT_MAX / 4 || n_heads < 1 || n_heads > (1 << 20)) return 0;
    return grouped_fwd_ws(n_heads, B * S);
  }
  if (strcmp(fn, "tp_residual_ln_bwd") == 0) {
    int rows = 0;
    if (B < 0 || S < 0 || (long)B * S > INT_MAX / 4) return 0;
    if (ln_geom(tp_size, rank, 0, B * S, H, dtype, &rows)) return 0;
    return align256(ln_bwd_ws_bytes(rows, H));
  }
  if (strcmp(fn, "tp_attn_out_shard_bwd") == 0) {
    if (head_geom(tp_size, rank, B, S, H, n_heads, dtype, &g)) return 0;
    return out_bwd_ws(g.T, H, g.nh * g.d, dtype);
  }
  if (strcmp(fn, "tp_attn_heads_bwd") == 0) {
    if (head_geom(tp_size, rank, B, S, H, n_heads, dtype, &g)) return 0;
    return align256(attn_bwd_ws_bytes(B, S, g.nh, g.d));
  }
  return 0;
}

const char* tp_status_str(int status) {
  switch (status) {
    case TP_OK: return "TP_OK: success";
    case TP_EINVAL: return "TP_EINVAL: invalid size, rank, dtype or split";
    case TP_ENULL: return "TP_ENULL: a required pointer is NULL";
    case TP_EALIGN: return "TP_EALIGN: a pointer is not aligned as required";
    case TP_EUNSUPPORTED: return "TP_EUNSUPPORTED: valid request not implemented";
    case TP_EWORKSPACE: return "TP_EWORKSPACE: workspace missing or too small";
    case TP_EHIP: return "TP_EHIP: a HIP call failed";
    default: return "unknown tp_status";
  }
}

const char* tp_last_error(void) { return g_err; }

const char* tp_version(void) { return "tpshard 0.1 gfx950"; }

}  // extern "C"
