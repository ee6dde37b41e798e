// Row softmax and the attention forward pass on MI355X (gfx950): the host
// side of the C ABI declared in include/attention.h (argument checks and
// launches; the kernels are in attention.hpp).
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <cmath>
#include <mutex>

#include "attention.h"
#include "attention.hpp"

namespace {

using gemm_relu::attn::AttnArgs;
using gemm_relu::attn::AttnCfg;
using gemm_relu::attn::SoftmaxArgs;

// gfx950 check, once per device id.
constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
signed char g_dev_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

int check_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GEMM_RELU_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return GEMM_RELU_EUNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_ok[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_RELU_EHIP;
        g_dev_ok[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    }
    return g_dev_ok[dev] == 1 ? GEMM_RELU_OK : GEMM_RELU_EUNSUPPORTED;
}

bool overlaps(const void* p, int64_t pbytes, const void* q, int64_t qbytes)
{
    if (pbytes <= 0 || qbytes <= 0) return false;
    const uintptr_t a0 = (uintptr_t)p, a1 = a0 + (uintptr_t)pbytes;
    const uintptr_t b0 = (uintptr_t)q, b1 = b0 + (uintptr_t)qbytes;
    return a0 < b1 && b0 < a1;
}

template <int V>
void launch_softmax_vec(const SoftmaxArgs& a, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_relu::attn::softmax_rows_vec<V>), dim3((a.rows + 3) / 4), dim3(256), 0, s, a);
}

// Waves per workgroup (32 query rows each). Two workgroups of 4 waves share
// a CU and run out of step, and under the causal mask the small workgroup
// evens out the work; without the mask at D = 128 one workgroup of 8 waves
// per CU loads each K and V tile into LDS once for 256 query rows instead of
// twice for 2 x 128, which measured 3 % faster (and 2-7 % slower for the
// causal and D = 64 cases, which keep 4).
constexpr int attn_waves(int D, int causal) { return (D == 128 && !causal) ? 8 : 4; }

template <int D, int NW>
void launch_attn(const AttnArgs& a, hipStream_t s)
{
    using T = AttnCfg<D, NW>;
    hipLaunchKernelGGL((gemm_relu::attn::attn_fwd_kernel<T>), dim3(a.BH * a.npair), dim3(T::NT), 0, s, a);
}

}  // namespace

extern "C" {

int softmax_rows_f16(int64_t rows, int64_t cols, const void* X, void* Y, void* stream)
{
    if (rows < 0 || cols < 0) return GEMM_RELU_EINVAL;
    if (rows > INT32_MAX || cols > INT32_MAX) return GEMM_RELU_EUNSUPPORTED;
    const int64_t n = rows * cols;
    if (n > 0 && (!X || !Y)) return GEMM_RELU_EINVAL;
    if ((((uintptr_t)X | (uintptr_t)Y) & 1u) != 0) return GEMM_RELU_EUNSUPPORTED;
    if (X != Y && overlaps(X, 2 * n, Y, 2 * n)) return GEMM_RELU_EINVAL;
    if (n == 0) return GEMM_RELU_OK;
    const int rc = check_device();
    if (rc != GEMM_RELU_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    SoftmaxArgs a{static_cast<const uint16_t*>(X), static_cast<uint16_t*>(Y), (int)rows, (int)cols};
    const bool vec = cols % 8 == 0 && cols <= 8192 && (((uintptr_t)X | (uintptr_t)Y) & 15u) == 0 &&
                     (rows + 3) / 4 <= INT32_MAX;
    if (vec) {
        if (cols <= 512) launch_softmax_vec<1>(a, s);
        else if (cols <= 1024) launch_softmax_vec<2>(a, s);
        else if (cols <= 2048) launch_softmax_vec<4>(a, s);
        else if (cols <= 4096) launch_softmax_vec<8>(a, s);
        else launch_softmax_vec<16>(a, s);
    } else {
        hipLaunchKernelGGL(gemm_relu::attn::softmax_rows_any, dim3((unsigned)rows), dim3(256), 0, s, a);
    }
    return hipGetLastError() == hipSuccess ? GEMM_RELU_OK : GEMM_RELU_EHIP;
}

int flash_attn_fwd_f16(int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, const void* Q, const void* K,
                       const void* V, void* O, void* lse, float scale, int causal, void* stream)
{
    if (B < 0 || H < 0 || Sq < 0 || Skv < 0 || D < 0) return GEMM_RELU_EINVAL;
    if (causal != 0 && causal != 1) return GEMM_RELU_EINVAL;
    if (!std::isfinite(scale)) return GEMM_RELU_EINVAL;
    // |scale * log2(e) * Q.K| <= 2^64 * 1.45 * 128 * 65504^2 < 2^108: finite
    // in fp32, as is the difference of two such scores
    if (std::fabs(scale) > 0x1p64f) return GEMM_RELU_EUNSUPPORTED;
    if (D != 64 && D != 128) return GEMM_RELU_EUNSUPPORTED;
    if (B > INT32_MAX || H > INT32_MAX || B * H > INT32_MAX || Sq > INT32_MAX || Skv > INT32_MAX)
        return GEMM_RELU_EUNSUPPORTED;
    // in-head offsets are 32-bit byte offsets
    if (Sq * D >= ((int64_t)1 << 30) || Skv * D >= ((int64_t)1 << 30)) return GEMM_RELU_EUNSUPPORTED;
    const int64_t BH = B * H;
    const int64_t nq = BH * Sq * D, nkv = BH * Skv * D;
    if ((nq > 0 && (!Q || !O)) || (nkv > 0 && (!K || !V))) return GEMM_RELU_EINVAL;
    if ((((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15u) != 0 || ((uintptr_t)lse & 3u) != 0)
        return GEMM_RELU_EUNSUPPORTED;
    if (overlaps(O, 2 * nq, Q, 2 * nq) || overlaps(O, 2 * nq, K, 2 * nkv) || overlaps(O, 2 * nq, V, 2 * nkv) ||
        (lse && overlaps(O, 2 * nq, lse, 4 * BH * Sq)))
        return GEMM_RELU_EINVAL;
    if (BH == 0 || Sq == 0) return GEMM_RELU_OK;
    const int64_t bm = 32 * attn_waves((int)D, causal);  // query rows per workgroup
    const int64_t nqb = (Sq + bm - 1) / bm;
    if (BH * nqb > INT32_MAX) return GEMM_RELU_EUNSUPPORTED;
    const int rc = check_device();
    if (rc != GEMM_RELU_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    AttnArgs a;
    a.Q = static_cast<const uint16_t*>(Q);
    a.K = static_cast<const uint16_t*>(K);
    a.V = static_cast<const uint16_t*>(V);
    a.O = static_cast<uint16_t*>(O);
    a.lse = static_cast<float*>(lse);
    a.BH = (int)BH;
    a.Sq = (int)Sq;
    a.Skv = (int)Skv;
    // the kernels fold the scale into their exponents and use its sign to
    // take row maxima; a zero scale (every score 0) becomes a tiny positive
    // one, which gives the same uniform weights
    a.scale_log2 = scale * gemm_relu::attn::kLog2e;
    if (a.scale_log2 == 0.0f) a.scale_log2 = 1e-30f;
    a.causal = causal;
    a.nqb = (int)nqb;
    a.paired = causal;
    a.npair = (int)(causal ? (nqb + 1) / 2 : nqb);
    if (D == 64) launch_attn<64, attn_waves(64, 0)>(a, s);
    else if (causal) launch_attn<128, attn_waves(128, 1)>(a, s);
    else launch_attn<128, attn_waves(128, 0)>(a, s);
    return hipGetLastError() == hipSuccess ? GEMM_RELU_OK : GEMM_RELU_EHIP;
}

}  // extern "C"
