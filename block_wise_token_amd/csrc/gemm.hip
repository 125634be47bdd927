// libuniprefill_layer: the plain bf16 GEMMs of the layer on the surviving tokens,
// served by hipBLASLt, with the C ABI of include/uniprefill_layer.h.  Kept out of
// libuniprefill.so so that the decision path links no vendor GEMM library; the
// SwiGLU gate between the FFN's two GEMMs is libuniprefill.so's up_swiglu.
#include "uniprefill.h"
#include "uniprefill_layer.h"

#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

namespace up {

constexpr size_t kWsAlign = 256;
inline size_t align_up(size_t x, size_t a = kWsAlign) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// hipBLASLt GEMM: y[R][N] = x[R][K] w[N][K]^T (+ residual[R][N]), bf16 in and out,
// float32 accumulation.  In hipBLASLt's column-major terms y^T = op_T(w) x^T.  One
// handle per device; descriptors and the heuristic's first algorithm are cached per
// (device, R, K, N, residual, workspace bytes).
// ---------------------------------------------------------------------------
namespace {
struct GemmPlan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo;
  size_t ws_need = 0;
};
std::mutex g_blas_mu;
hipblasLtHandle_t g_blas[64] = {};
std::map<std::tuple<int, int64_t, int, int, bool, size_t>, GemmPlan> g_plans;
}  // namespace

static int linear_gemm(const void* x, const void* w, const void* residual, int64_t R, int K, int N,
                void* y, void* ws, size_t ws_bytes, hipStream_t st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  std::lock_guard<std::mutex> lk(g_blas_mu);
  if (!g_blas[dev] && hipblasLtCreate(&g_blas[dev]) != HIPBLAS_STATUS_SUCCESS) {
    g_blas[dev] = nullptr;
    return -1;
  }
  const bool res = residual != nullptr;
  const auto key = std::make_tuple(dev, R, K, N, res, ws_bytes);
  auto it = g_plans.find(key);
  if (it == g_plans.end()) {
    GemmPlan p;
    bool ok = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) ==
              HIPBLAS_STATUS_SUCCESS;
    const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta,
                                               sizeof(ta)) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb,
                                               sizeof(tb)) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, K, N, K) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, K, R, K) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&p.lc, HIP_R_16BF, N, R, N) == HIPBLAS_STATUS_SUCCESS;
    hipblasLtMatmulPreference_t pref = nullptr;
    ok = ok && hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
    uint64_t wsmax = ws_bytes;
    ok = ok && hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                     &wsmax, sizeof(wsmax)) ==
                   HIPBLAS_STATUS_SUCCESS;
    hipblasLtMatmulHeuristicResult_t hr[1];
    int n = 0;
    ok = ok && hipblasLtMatmulAlgoGetHeuristic(g_blas[dev], p.desc, p.la, p.lb, p.lc, p.lc, pref,
                                               1, hr, &n) == HIPBLAS_STATUS_SUCCESS &&
         n > 0;
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (!ok) {
      if (p.la) hipblasLtMatrixLayoutDestroy(p.la);
      if (p.lb) hipblasLtMatrixLayoutDestroy(p.lb);
      if (p.lc) hipblasLtMatrixLayoutDestroy(p.lc);
      if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
      return -2;
    }
    p.algo = hr[0].algo;
    p.ws_need = hr[0].workspaceSize;
    it = g_plans.emplace(key, p).first;
  }
  const GemmPlan& p = it->second;
  const float alpha = 1.f, beta = res ? 1.f : 0.f;
  const hipblasStatus_t s =
      hipblasLtMatmul(g_blas[dev], p.desc, &alpha, w, p.la, x, p.lb, &beta, res ? residual : y,
                      p.lc, y, p.lc, &p.algo, p.ws_need ? ws : nullptr, p.ws_need, st);
  return s == HIPBLAS_STATUS_SUCCESS ? 0 : -1;
}

}  // namespace up

namespace {
using namespace up;

// hipBLASLt workspace offered to each GEMM inside up_swiglu_ffn.
constexpr size_t kGemmWs = size_t(32) << 20;

struct FfnWs {
  size_t gu, a, gemm, total;
};
FfnWs ffn_ws_layout(int64_t R, int F) {
  FfnWs w;
  size_t o = 0;
  w.gu = o;
  o += align_up((size_t)R * 2 * F * 2);
  w.a = o;
  o += align_up((size_t)R * F * 2);
  w.gemm = o;
  o += kGemmWs;
  w.total = o;
  return w;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Largest operand (elements) a GEMM here may have.  The GEMMs have run on the device up
// to 4.03e9 elements per operand (the FFN of 131,072 rows at width 15,360); a run whose
// FFN output had 6.3e9 elements (220,884 rows x 2 x 14,336) left the GPU with a memory
// fault, and no fault of this library's own kernels at that size has been shown, so
// operands of 2^32 elements or more are refused until one is shown to be safe.
constexpr int64_t kMaxGemmElems = int64_t(1) << 32;
bool gemm_fits(int64_t R, int K, int N) {
  return R * (int64_t)K < kMaxGemmElems && R * (int64_t)N < kMaxGemmElems &&
         (int64_t)K * N < kMaxGemmElems;
}
}  // namespace

extern "C" {

int up_linear(const void* x, const void* w, const void* residual, int64_t R, int K, int N,
              void* y, void* workspace, size_t workspace_bytes, void* stream) {
  if (R < 0 || K <= 0 || N <= 0) return UP_EINVAL;
  if (R == 0) return UP_OK;
  if (!gemm_fits(R, K, N)) return UP_EUNSUPPORTED;
  if (!x || !w || !y || (workspace_bytes > 0 && !workspace)) return UP_EINVAL;
  if (workspace && !aligned(workspace, kWsAlign)) return UP_EWORKSPACE;
  const int r = linear_gemm(x, w, residual, R, K, N, y, workspace, workspace_bytes,
                            static_cast<hipStream_t>(stream));
  if (r == -1) return UP_EHIP;
  return r == -2 ? UP_EUNSUPPORTED : UP_OK;
}

size_t up_swiglu_ffn_workspace(int64_t R, int H, int F) {
  if (R < 0 || H <= 0 || F <= 0) return 0;
  return ffn_ws_layout(R, F).total;
}

int up_swiglu_ffn(const void* x, const void* w_gu, const void* w_down, const void* residual,
                  int64_t R, int H, int F, void* y, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (R < 0 || H <= 0 || F <= 0) return UP_EINVAL;
  if (F % 8 != 0) return UP_EUNSUPPORTED;
  if (R == 0) return UP_OK;
  if (!gemm_fits(R, H, 2 * F) || !gemm_fits(R, F, H)) return UP_EUNSUPPORTED;
  if (!x || !w_gu || !w_down || !y) return UP_EINVAL;
  const FfnWs L = ffn_ws_layout(R, F);
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, kWsAlign))
    return UP_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  int st = up_linear(x, w_gu, nullptr, R, H, 2 * F, ws + L.gu, ws + L.gemm, kGemmWs, stream);
  if (st != UP_OK) return st;
  st = up_swiglu(ws + L.gu, R, F, ws + L.a, stream);
  if (st != UP_OK) return st;
  return up_linear(ws + L.a, w_down, residual, R, F, H, y, ws + L.gemm, kGemmWs, stream);
}

}  // extern "C"
