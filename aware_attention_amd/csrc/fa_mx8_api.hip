// C ABI of the FP8 (MX block-scaled) forward and its quantisers:
// fa_fwd_mx8, fa_mx8_quantize_qk, fa_mx8_quantize_v, fa_mx8_tokens_padded.
// The operations are documented in include/fa.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <string>

#include "fa.h"
#include "fa_host.hpp"
#include "fa_mx8_kernel.hpp"

namespace {

using fa_host::check_device;
using fa_host::fail;

constexpr float kLog2e = 1.44269504088896340736f;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

extern "C" {

int32_t fa_mx8_tokens_padded(int32_t N) {
  if (N < 0 || N > INT32_MAX - fa::kMxTokenPad) return -1;
  return (N + fa::kMxTokenPad - 1) / fa::kMxTokenPad * fa::kMxTokenPad;
}

fa_status fa_mx8_quantize_qk(const void* x, int32_t dtype, int64_t rows, int32_t d, uint8_t* xq,
                             uint8_t* xe, void* stream) {
  fa_host::g_last_error.clear();
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
    return fail(FA_ERR_INVALID_ARGUMENT, "dtype must be FA_DTYPE_BF16 or FA_DTYPE_F16");
  if (rows < 0) return fail(FA_ERR_INVALID_ARGUMENT, "rows must be >= 0");
  if (d != fa::kMxD) return fail(FA_ERR_UNSUPPORTED, "the FP8 path serves head dimension 128");
  if (rows == 0) return FA_OK;
  if (!x || !xq || !xe) return fail(FA_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned(x, 16) || !aligned(xq, 16))
    return fail(FA_ERR_INVALID_ARGUMENT, "x and xq must be 16-byte aligned");
  const int64_t nblocks = rows * (d / fa::kMxBlock);
  const int64_t grid = (nblocks + 255) / 256;
  if (grid > INT32_MAX) return fail(FA_ERR_UNSUPPORTED, "too many blocks for one launch");
  fa_status st = check_device();
  if (st != FA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* src = static_cast<const uint16_t*>(x);
  if (dtype == FA_DTYPE_F16)
    hipLaunchKernelGGL(fa::mx8_quantize_rows_kernel<true>, dim3((uint32_t)grid), dim3(256), 0, s,
                       src, xq, xe, nblocks);
  else
    hipLaunchKernelGGL(fa::mx8_quantize_rows_kernel<false>, dim3((uint32_t)grid), dim3(256), 0, s,
                       src, xq, xe, nblocks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return FA_OK;
}

fa_status fa_mx8_quantize_v(const void* v, int32_t dtype, int32_t B, int32_t N, int32_t H,
                            int32_t d, uint8_t* vt, uint8_t* vte, void* stream) {
  fa_host::g_last_error.clear();
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
    return fail(FA_ERR_INVALID_ARGUMENT, "dtype must be FA_DTYPE_BF16 or FA_DTYPE_F16");
  if (B < 1 || N < 1 || H < 1) return fail(FA_ERR_INVALID_ARGUMENT, "B, N and H must be >= 1");
  if (d != fa::kMxD) return fail(FA_ERR_UNSUPPORTED, "the FP8 path serves head dimension 128");
  const int32_t Np = fa_mx8_tokens_padded(N);
  if (Np < 0) return fail(FA_ERR_UNSUPPORTED, "N too large");
  if (!v || !vt || !vte) return fail(FA_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned(v, 2) || !aligned(vt, 16)) return fail(FA_ERR_INVALID_ARGUMENT, "vt must be 16-byte aligned");
  const int64_t nblk = (int64_t)B * H * (Np / fa::kMxBlock) * d;
  const int64_t grid = (nblk + 255) / 256;
  if (grid > INT32_MAX) return fail(FA_ERR_UNSUPPORTED, "too many blocks for one launch");
  fa_status st = check_device();
  if (st != FA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* src = static_cast<const uint16_t*>(v);
  if (dtype == FA_DTYPE_F16)
    hipLaunchKernelGGL(fa::mx8_quantize_vt_kernel<true>, dim3((uint32_t)grid), dim3(256), 0, s, src,
                       vt, vte, B, N, H, Np);
  else
    hipLaunchKernelGGL(fa::mx8_quantize_vt_kernel<false>, dim3((uint32_t)grid), dim3(256), 0, s,
                       src, vt, vte, B, N, H, Np);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return FA_OK;
}

fa_status fa_fwd_mx8(const uint8_t* q, const uint8_t* qe, const uint8_t* k, const uint8_t* ke,
                     const uint8_t* vt, const uint8_t* vte, void* o, float* lse, int32_t B,
                     int32_t Nq, int32_t Nk, int32_t H, int32_t d, float softmax_scale,
                     int32_t causal, void* stream) {
  fa_host::g_last_error.clear();
  if (!q || !qe || !k || !ke || !vt || !vte || !o || !lse)
    return fail(FA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (B < 1 || Nq < 1 || Nk < 1 || H < 1)
    return fail(FA_ERR_INVALID_ARGUMENT, "B, Nq, Nk and H must be >= 1");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  if (causal && Nq != Nk) return fail(FA_ERR_INVALID_ARGUMENT, "causal attention needs Nq == Nk");
  if (!std::isfinite(softmax_scale)) return fail(FA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if (d != fa::kMxD) return fail(FA_ERR_UNSUPPORTED, "the FP8 path serves head dimension 128");
  if ((int64_t)Nk * H * d > (int64_t)1 << 30 || (int64_t)fa_mx8_tokens_padded(Nk) * d > (int64_t)1 << 31)
    return fail(FA_ERR_UNSUPPORTED, "sequence too long for the kernel's 32-bit tile offsets");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(vt, 16) || !aligned(vte, 16) ||
      !aligned(ke, 4) || !aligned(qe, 4) || !aligned(o, 16) || !aligned(lse, 16))
    return fail(FA_ERR_INVALID_ARGUMENT,
                "q, k, vt, vte, o, lse must be 16-byte aligned and qe, ke 4-byte aligned");
  const int64_t n_qt = (Nq + fa::kBR - 1) / fa::kBR;
  const int64_t grid = n_qt * H * (int64_t)B;
  if (grid > INT32_MAX) return fail(FA_ERR_UNSUPPORTED, "too many query tiles for one launch");
  fa_status st = check_device();
  if (st != FA_OK) return st;
  fa::Mx8Params p{};
  p.q = q;
  p.qe = qe;
  p.k = k;
  p.ke = ke;
  p.vt = vt;
  p.vte = vte;
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.Nq = Nq;
  p.Nk = Nk;
  p.Np = fa_mx8_tokens_padded(Nk);
  p.H = H;
  p.nbatch = B;
  p.n_qtiles = (int32_t)n_qt;
  p.scale_log2 = std::fabs(softmax_scale) * kLog2e;
  p.q_sign = softmax_scale < 0.f ? 0x80808080u : 0u;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (causal)
    hipLaunchKernelGGL(fa::fwd_mx8_kernel<true>, dim3((uint32_t)grid), dim3(fa::kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(fa::fwd_mx8_kernel<false>, dim3((uint32_t)grid), dim3(fa::kThreads), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return FA_OK;
}

}  // extern "C"
