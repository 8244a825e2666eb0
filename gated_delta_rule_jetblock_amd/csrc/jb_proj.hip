// jb_proj.hip -- the block's input projections (q, k, v, the gates) and the
// kernel generator's first layer from one pass over x.
//
// The kernel generator takes the same input as the Q/K/V projection layers
// (Jet-Nemotron csdn translation, section 2.4), so the block can start from
// the layer input x instead of from q, k, v:
//     q = Wq x,  k = Wk x,  v = Wv x                          (bf16 out)
//     alpha = sigmoid(Wa x + ba),  beta = sigmoid(Wb x + bb)  (one per head)
//     taps  = W2 SiLU(W1 x + b1) + b2                          (4 per head)
// The gate projections are not described on the pages; a sigmoid keeps both
// gates in (0, 1) as the recurrence needs.
//
// The projections are plain [tokens x d_model] x [d_model x N] products and
// run as library GEMMs (hipBLASLt, bf16 operands, fp32 accumulation; q, k, v
// rounded to bf16 once, by the GEMM's output conversion).  The Q/K/V layers
// carry no bias here: the library's bias epilogue adds the bias after that
// conversion, which measured up to 3 bf16 steps off the once-rounded value
// where a bias cancels most of the product.  W1, Wa and Wb are stacked into one small
// GEMM with fp32 output; a hand-written epilogue kernel then applies SiLU and
// the 32 -> 4H second layer for the taps and the sigmoids for the gates.
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "jb_device.h"
#include "jb_internal.h"

namespace jb {

constexpr size_t kGemmWorkspace = (size_t)32 << 20;  // bytes of workspace offered to the GEMM library

size_t project_gemm_workspace_bytes() { return kGemmWorkspace; }

// ------------------------------------------------------------ GEMM

namespace {

// A GEMM plan: descriptors and the chosen algorithm for one shape, built on
// first use and kept for the life of the process (creating them per call
// cost more host time than a small GEMM takes on the GPU).
struct GemmPlan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulAlgo_t algo{};
};

struct LtState {
  std::mutex mu;
  std::map<int, hipblasLtHandle_t> handles;  // per device
  // (device, M, N, K, out f32) -> plan
  std::map<std::tuple<int, int64_t, int, int, bool>, GemmPlan> plans;
};
LtState& lt() {
  static LtState s;
  return s;
}

hipError_t make_plan(hipblasLtHandle_t handle, int64_t M, int N, int K, bool y_f32, size_t ws_bytes, GemmPlan& p) {
  const hipDataType ytype = y_f32 ? HIP_R_32F : HIP_R_16BF;
  const hipblasOperation_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
  const uint64_t wsb = ws_bytes;
  hipblasLtMatmulPreference_t pref = nullptr;
  hipError_t out = hipSuccess;
  if (hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT)) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN)) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, K, N, K) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, K, M, K) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&p.ld, ytype, N, M, N) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof(wsb)) !=
          HIPBLAS_STATUS_SUCCESS) {
    out = hipErrorInvalidValue;
  } else {
    hipblasLtMatmulHeuristicResult_t res[1];
    int n = 0;
    if (hipblasLtMatmulAlgoGetHeuristic(handle, p.desc, p.la, p.lb, p.ld, p.ld, pref, 1, res, &n) !=
            HIPBLAS_STATUS_SUCCESS ||
        n < 1)
      out = hipErrorNotSupported;
    else
      p.algo = res[0].algo;
  }
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (out != hipSuccess) {
    if (p.ld) hipblasLtMatrixLayoutDestroy(p.ld);
    if (p.lb) hipblasLtMatrixLayoutDestroy(p.lb);
    if (p.la) hipblasLtMatrixLayoutDestroy(p.la);
    if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
    p = GemmPlan{};
  }
  return out;
}

}  // namespace

// y[M][N] = x[M][K] W[N][K]^T, x and W bf16 row-major, y bf16 or fp32
// row-major.  In the library's column-major terms: D[N x M] = op_T(W) B with
// B = x^T [K x M].
hipError_t gemm_xwt(int64_t M, int N, int K, const void* x, const void* W, void* y, bool y_f32, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  LtState& s = lt();
  std::lock_guard<std::mutex> lock(s.mu);
  auto hit = s.handles.find(dev);
  if (hit == s.handles.end()) {
    hipblasLtHandle_t h = nullptr;
    if (hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS) return hipErrorInitializationError;
    hit = s.handles.emplace(dev, h).first;
  }
  const auto key = std::make_tuple(dev, M, N, K, y_f32);
  auto pit = s.plans.find(key);
  if (pit == s.plans.end()) {
    GemmPlan p;
    e = make_plan(hit->second, M, N, K, y_f32, ws_bytes, p);
    if (e != hipSuccess) return e;
    pit = s.plans.emplace(key, p).first;
  }
  const GemmPlan& p = pit->second;
  const float one = 1.f, zero = 0.f;
  if (hipblasLtMatmul(hit->second, p.desc, &one, W, p.la, x, p.lb, &zero, y, p.ld, y, p.ld, &p.algo, ws, ws_bytes,
                      stream) != HIPBLAS_STATUS_SUCCESS)
    return hipErrorLaunchFailure;
  return hipSuccess;
}

// ------------------------------------------------------------ epilogue

// 16 tokens per workgroup.  z [n][32 + 2H] holds W1 x, Wa x, Wb x in fp32.
//   taps[t][h][j] = b2[4h+j] + sum_u W2[4h+j][u] SiLU(z[t][u] + b1[u])
//   alpha[t][h] = sigmoid(z[t][32+h] + ba[h]),  beta[t][h] = sigmoid(z[t][32+H+h] + bb[h])
constexpr int EP_TOK = 16;
constexpr int EP_THR = 256;

__global__ __launch_bounds__(EP_THR) void proj_epilogue_kernel(int64_t n, int H, const float* z, const bf16_t* b1,
                                                               const bf16_t* W2, const bf16_t* b2, const bf16_t* ba,
                                                               const bf16_t* bb, float* taps, float* alpha,
                                                               float* beta) {
  __shared__ float w2s[128][33];
  __shared__ float hid[EP_TOK][33];
  const int tid = threadIdx.x;
  const int HK = 4 * H, NZ = 32 + 2 * H;
  const int64_t t0 = (int64_t)blockIdx.x * EP_TOK;
  for (int e = tid; e < HK * 32; e += EP_THR) w2s[e / 32][e % 32] = bf16_to_f32(W2[e]);
  for (int e = tid; e < EP_TOK * 32; e += EP_THR) {
    const int t = e / 32, u = e % 32;
    const int64_t tok = t0 + t;
    float hv = tok < n ? z[tok * NZ + u] : 0.f;
    if (b1) hv += bf16_to_f32(b1[u]);
    hid[t][u] = hv / (1.0f + expf(-hv));  // SiLU
  }
  for (int e = tid; e < EP_TOK * 2 * H; e += EP_THR) {
    const int t = e / (2 * H), r = e % (2 * H);
    const int64_t tok = t0 + t;
    if (tok >= n) continue;
    const bf16_t* bias = r < H ? ba : bb;
    const float zv = z[tok * NZ + 32 + r] + (bias ? bf16_to_f32(bias[r % H]) : 0.f);
    const float gv = 1.0f / (1.0f + expf(-zv));
    if (r < H) alpha[tok * H + r] = gv;
    else beta[tok * H + (r - H)] = gv;
  }
  __syncthreads();
  for (int e = tid; e < EP_TOK * HK; e += EP_THR) {
    const int t = e / HK, r = e % HK;
    const int64_t tok = t0 + t;
    if (tok >= n) continue;
    float sacc = b2 ? bf16_to_f32(b2[r]) : 0.f;
#pragma unroll 8
    for (int u = 0; u < 32; ++u) sacc += w2s[r][u] * hid[t][u];
    taps[tok * HK + r] = sacc;
  }
}

// ------------------------------------------------------------ the stage

size_t project_workspace_bytes(int64_t n, int H, int D) {
  const auto a256 = [](size_t v) { return (v + 255) & ~(size_t)255; };
  // z, the stacked [W1; Wa; Wb], the GEMM library's own
  return a256((size_t)n * (32 + 2 * H) * sizeof(float)) + a256((size_t)(32 + 2 * H) * D * 2) + kGemmWorkspace;
}

hipError_t launch_project(int64_t n, int H, int dk, int dv, int D, const void* x, const void* Wq, const void* Wk,
                          const void* Wv, const void* Wa, const void* ba, const void* Wb, const void* bb,
                          const void* W1, const void* b1,
                          const void* W2, const void* b2, void* q, void* k, void* v, float* alpha, float* beta,
                          float* taps, void* workspace, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const auto a256 = [](size_t val) { return (val + 255) & ~(size_t)255; };
  const int NZ = 32 + 2 * H;
  char* ws = static_cast<char*>(workspace);
  float* z = reinterpret_cast<float*>(ws);
  ws += a256((size_t)n * NZ * sizeof(float));
  char* wg = ws;  // [W1; Wa; Wb] stacked, bf16 [NZ][D]
  ws += a256((size_t)NZ * D * 2);
  hipError_t e = hipSuccess;
  void* gws = ws;
  const size_t rowb = (size_t)D * 2;
  e = gemm_xwt(n, H * dk, D, x, Wq, q, false, gws, kGemmWorkspace, stream);
  if (e == hipSuccess) e = gemm_xwt(n, H * dk, D, x, Wk, k, false, gws, kGemmWorkspace, stream);
  if (e == hipSuccess) e = gemm_xwt(n, H * dv, D, x, Wv, v, false, gws, kGemmWorkspace, stream);
  if (e != hipSuccess || !W1) return e;  // q, k, v only
  e = hipMemcpyAsync(wg, W1, 32 * rowb, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(wg + 32 * rowb, Wa, H * rowb, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(wg + (32 + H) * rowb, Wb, H * rowb, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess) e = gemm_xwt(n, NZ, D, x, wg, z, true, gws, kGemmWorkspace, stream);
  if (e != hipSuccess) return e;
  proj_epilogue_kernel<<<(unsigned)((n + EP_TOK - 1) / EP_TOK), EP_THR, 0, stream>>>(
      n, H, z, (const bf16_t*)b1, (const bf16_t*)W2, (const bf16_t*)b2, (const bf16_t*)ba, (const bf16_t*)bb, taps,
      alpha, beta);
  return hipGetLastError();
}

}  // namespace jb
