// hqq_gemm.cpp -- Y = X . W^T for fp16 or bf16 matrices through hipBLASLt, the
// matrix product of the linear layer's dequantize-then-GEMM route (the layer
// computes X . W_hat^T; lnwmold.com HQQ guide, section 4.1: backends either
// fuse the dequantization into the product or dequantize first and call a
// dense GEMM).  Host code only: the product is a plain library GEMM.
//
// Row-major X [M, K], W [N, K] and Y [M, N] are, column-major, X^T (K x M),
// W^T (K x N) and Y^T (N x M); Y^T = (W^T)^T . X^T is the column-major GEMM
// with A = W^T transposed and B = X^T as is: m = N, n = M, k = K.  fp32
// accumulation and scaling, one rounding of each output to the dtype.
//
// A hipBLASLt handle per device and a plan (descriptors and the heuristic's
// first algorithm) per shape are created on first use and kept until the
// process ends; a mutex guards them and the enqueue.
#include "hqq_internal.h"

#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

namespace hqq {
namespace {

struct GemmPlan {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    size_t ws = 0;   // workspace bytes the algorithm needs
    bool ok = false;
};

using PlanKey = std::tuple<int, int64_t, int64_t, int64_t, bool, size_t>;

std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handle;
std::map<PlanKey, GemmPlan> g_plan;
// plans kept at most (M is part of the key: callers with varying row counts
// would otherwise grow the map without bound); past it the map starts over
constexpr size_t kMaxPlans = 256;

void destroy(GemmPlan &p)
{
    if (p.c)
        hipblasLtMatrixLayoutDestroy(p.c);
    if (p.b)
        hipblasLtMatrixLayoutDestroy(p.b);
    if (p.a)
        hipblasLtMatrixLayoutDestroy(p.a);
    if (p.desc)
        hipblasLtMatmulDescDestroy(p.desc);
    p = GemmPlan{};
}

bool make_plan(hipblasLtHandle_t h, int64_t M, int64_t N, int64_t K, bool bf16, size_t ws_cap, GemmPlan &p)
{
    const hipDataType dt = bf16 ? HIP_R_16BF : HIP_R_16F;
    if (hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS)
        return false;
    const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    if (hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) !=
            HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) !=
            HIPBLAS_STATUS_SUCCESS)
        return false;
    if (hipblasLtMatrixLayoutCreate(&p.a, dt, (uint64_t)K, (uint64_t)N, K) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.b, dt, (uint64_t)K, (uint64_t)M, K) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.c, dt, (uint64_t)N, (uint64_t)M, N) != HIPBLAS_STATUS_SUCCESS)
        return false;
    hipblasLtMatmulPreference_t pref = nullptr;
    if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS)
        return false;
    const uint64_t cap = ws_cap;
    bool ok = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &cap,
                                                    sizeof(cap)) == HIPBLAS_STATUS_SUCCESS;
    // room for more than one result, in case the library's result record is
    // larger than this header's
    hipblasLtMatmulHeuristicResult_t res[4];
    int found = 0;
    ok = ok && hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.a, p.b, p.c, p.c, pref, 1, res, &found) ==
                   HIPBLAS_STATUS_SUCCESS;
    hipblasLtMatmulPreferenceDestroy(pref);
    if (!ok || found < 1 || res[0].state != HIPBLAS_STATUS_SUCCESS || res[0].workspaceSize > ws_cap)
        return false;
    p.algo = res[0].algo;
    p.ws = res[0].workspaceSize;
    return true;
}

// The current device's handle and the plan of a shape, created on first use
// (g_mu held by the caller); nullptr where hipBLASLt has no algorithm.
const GemmPlan *plan_for(int64_t M, int64_t N, int64_t K, bool bf16, size_t ws_bytes, hipblasLtHandle_t &h)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return nullptr;
    auto hi = g_handle.find(dev);
    if (hi == g_handle.end()) {
        hipblasLtHandle_t nh = nullptr;
        if (hipblasLtCreate(&nh) != HIPBLAS_STATUS_SUCCESS)
            return nullptr;
        hi = g_handle.emplace(dev, nh).first;
    }
    h = hi->second;
    const PlanKey key{dev, M, N, K, bf16, ws_bytes};
    auto pi = g_plan.find(key);
    if (pi == g_plan.end()) {
        if (g_plan.size() >= kMaxPlans) {
            // every enqueued matmul has taken what it needs from its plan
            for (auto &kv : g_plan)
                destroy(kv.second);
            g_plan.clear();
        }
        GemmPlan p;
        p.ok = make_plan(h, M, N, K, bf16, ws_bytes, p);
        if (!p.ok)
            destroy(p);
        pi = g_plan.emplace(key, p).first;
    }
    return pi->second.ok ? &pi->second : nullptr;
}

}  // namespace

bool gemm_available(int64_t M, int64_t N, int64_t K, bool bf16, size_t ws_bytes)
{
    std::lock_guard<std::mutex> lock(g_mu);
    hipblasLtHandle_t h = nullptr;
    return plan_for(M, N, K, bf16, ws_bytes, h) != nullptr;
}

hipError_t gemm_xwt(const void *X, const void *W, void *Y, int64_t M, int64_t N, int64_t K, bool bf16,
                    void *ws, size_t ws_bytes, hipStream_t s)
{
    std::lock_guard<std::mutex> lock(g_mu);
    hipblasLtHandle_t h = nullptr;
    const GemmPlan *p = plan_for(M, N, K, bf16, ws_bytes, h);
    if (!p)
        return hipErrorNotSupported;
    const float alpha = 1.0f, beta = 0.0f;
    const hipblasStatus_t st = hipblasLtMatmul(h, p->desc, &alpha, W, p->a, X, p->b, &beta, Y, p->c, Y, p->c,
                                               &p->algo, p->ws ? ws : nullptr, p->ws, s);
    return st == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}

}  // namespace hqq
