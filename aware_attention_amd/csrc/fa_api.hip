// C ABI of libfa.so: argument checks, device check, launch configuration.
// The operation and the conventions are documented in include/fa.h.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

#include "fa_fwd256_kernel.hpp"
#include "fa_fwd_kernel.hpp"
#include "fa_host.hpp"

namespace fa_host {

thread_local std::string g_last_error;

fa_status fail(fa_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Per-device answer to "is this a gfx950?", looked up once per device.
struct DeviceInfo {
  bool known = false;
  bool supported = false;
  std::string arch;
};
constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
DeviceInfo g_dev[kMaxDevices];

fa_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_UNSUPPORTED, "device ordinal out of range");
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo& info = g_dev[dev];
  if (!info.known) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(FA_ERR_HIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
    info.arch = prop.gcnArchName;
    info.supported = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    info.known = true;
  }
  if (!info.supported) return fail(FA_ERR_UNSUPPORTED, "libfa runs on gfx950 only; device is " + info.arch);
  return FA_OK;
}

}  // namespace fa_host

namespace {

using fa_host::aligned16;
using fa_host::check_device;
using fa_host::fail;
using fa_host::g_last_error;

template <int D, bool CAUSAL, bool VARLEN, bool BAND, bool F16, bool KPM = false>
hipError_t launch_one(const fa::FwdParams& p, uint32_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((fa::fwd_kernel<D, CAUSAL, VARLEN, BAND, F16, KPM>), dim3(grid),
                     dim3(fa::kThreads), 0, stream, p);
  return hipGetLastError();
}

// Mask of a launch: none, causal (top-left, Nq == Nk), a band, or a key
// padding mask (dense self-attention), alone or with causal.
enum class Mask { kNone, kCausal, kBand, kPad, kPadCausal };

template <int D, bool VARLEN, bool F16>
hipError_t launch_d(const fa::FwdParams& p, Mask mask, uint32_t grid, hipStream_t stream) {
  switch (mask) {
    case Mask::kCausal: return launch_one<D, true, VARLEN, false, F16>(p, grid, stream);
    case Mask::kBand: return launch_one<D, false, VARLEN, true, F16>(p, grid, stream);
    case Mask::kPad:
    case Mask::kPadCausal:
      if constexpr (!VARLEN) {
        return mask == Mask::kPad ? launch_one<D, false, false, false, F16, true>(p, grid, stream)
                                  : launch_one<D, true, false, false, F16, true>(p, grid, stream);
      }
      return hipErrorInvalidValue;
    default: return launch_one<D, false, VARLEN, false, F16>(p, grid, stream);
  }
}

template <bool VARLEN, bool F16>
hipError_t launch_t(const fa::FwdParams& p, int d, Mask mask, uint32_t grid, hipStream_t stream) {
  switch (d) {
    case 32: return launch_d<32, VARLEN, F16>(p, mask, grid, stream);
    case 64: return launch_d<64, VARLEN, F16>(p, mask, grid, stream);
    default: return launch_d<128, VARLEN, F16>(p, mask, grid, stream);
  }
}

// Head dimension 256 (unmasked or causal): its own kernel, 128-row tiles.
template <bool VARLEN, bool F16>
hipError_t launch_256(const fa::FwdParams& p, Mask mask, uint32_t grid, hipStream_t stream) {
  const dim3 block(fa::kBwdThreads);
  switch (mask) {
    case Mask::kCausal:
      hipLaunchKernelGGL((fa::fwd256_kernel<true, VARLEN, F16>), dim3(grid), block, 0, stream, p);
      break;
    case Mask::kBand:
      hipLaunchKernelGGL((fa::fwd256_kernel<false, VARLEN, F16, true>), dim3(grid), block, 0,
                         stream, p);
      break;
    case Mask::kPad:
    case Mask::kPadCausal:
      if constexpr (!VARLEN) {   // the padding mask is dense only (checked by the caller)
        if (mask == Mask::kPad)
          hipLaunchKernelGGL((fa::fwd256_kernel<false, false, F16, false, true>), dim3(grid), block,
                             0, stream, p);
        else
          hipLaunchKernelGGL((fa::fwd256_kernel<true, false, F16, false, true>), dim3(grid), block,
                             0, stream, p);
      }
      break;
    default:
      hipLaunchKernelGGL((fa::fwd256_kernel<false, VARLEN, F16>), dim3(grid), block, 0, stream, p);
  }
  return hipGetLastError();
}

template <bool VARLEN>
hipError_t launch(const fa::FwdParams& p, int d, int32_t dtype, Mask mask, uint32_t grid,
                  hipStream_t stream) {
  if (d == 256)
    return dtype == FA_DTYPE_F16 ? launch_256<VARLEN, true>(p, mask, grid, stream)
                                 : launch_256<VARLEN, false>(p, mask, grid, stream);
  return dtype == FA_DTYPE_F16 ? launch_t<VARLEN, true>(p, d, mask, grid, stream)
                               : launch_t<VARLEN, false>(p, d, mask, grid, stream);
}

// Query rows per workgroup of the kernel that serves head dimension d.
int rows_per_workgroup(int d) { return d == 256 ? fa::kRows256 : fa::kBR; }

// Window sides: >= 0, or -1 for unbounded. A side of max(nq, nk) already
// reaches every key (left needs Nk - 1 at most, right Nq - 1), so -1 and any
// larger side are passed to the kernel as max(nq, nk); with sequences of at
// most kMaxBandLen the kernel's 32-bit band bounds (about 3 max(nq, nk)) stay
// in range.
constexpr int64_t kMaxBandLen = int64_t{1} << 29;
fa_status check_window(int32_t left, int32_t right) {
  if (left < -1 || right < -1)
    return fail(FA_ERR_INVALID_ARGUMENT, "window sides must be >= 0, or -1 for unbounded");
  return FA_OK;
}
int32_t window_side(int32_t w, int64_t nq, int64_t nk) {
  const int64_t unbounded = nq > nk ? nq : nk;
  return (int32_t)((w < 0 || w > unbounded) ? unbounded : w);
}

// The mask named by a causal flag and a window, as taken by the strided
// entry points: causal, or no mask when both sides are unbounded, else a band.
fa_status mask_of(int32_t causal, int32_t left, int32_t right, Mask* mask) {
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  const fa_status st = check_window(left, right);
  if (st != FA_OK) return st;
  const bool unbounded = left == -1 && right == -1;
  if (causal && !unbounded)
    return fail(FA_ERR_INVALID_ARGUMENT, "causal and a window are exclusive (causal is window (-1, 0))");
  *mask = causal ? Mask::kCausal : (unbounded ? Mask::kNone : Mask::kBand);
  return FA_OK;
}

// Strides of one tensor in elements (d contiguous): batch (dense only),
// token, head.
struct Strides {
  int64_t b, t, h;
};
// Token strides up to 2^24 elements keep the kernel's per-lane 32-bit byte
// offsets inside a 64-row tile in range.
constexpr int64_t kMaxTokenStride = int64_t{1} << 24;

fa_status check_strides(const Strides& s, const char* name) {
  if (s.b < 0 || s.t < 0 || s.h < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, std::string(name) + ": strides must be >= 0");
  if ((s.b | s.t | s.h) & 7)
    return fail(FA_ERR_INVALID_ARGUMENT,
                std::string(name) + ": strides must be multiples of 8 elements (16-byte aligned rows)");
  if (s.t > kMaxTokenStride)
    return fail(FA_ERR_UNSUPPORTED, std::string(name) + ": token stride above 2^24 elements");
  return FA_OK;
}

fa_status check_dtype(int32_t dtype) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
    return fail(FA_ERR_INVALID_ARGUMENT, "dtype must be FA_DTYPE_BF16 or FA_DTYPE_F16");
  return FA_OK;
}

fa_status check_common(int32_t H, int32_t d, float scale) {
  if (H < 1) return fail(FA_ERR_INVALID_ARGUMENT, "H must be >= 1");
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if (d != 32 && d != 64 && d != 128 && d != 256)
    return fail(FA_ERR_UNSUPPORTED, "head dim must be 32, 64, 128 or 256");
  return FA_OK;
}

// Head dimension 256 runs unmasked or causal only.

void set_strides(fa::FwdParams& p, const Strides st[4]) {
  p.q_bs = st[0].b; p.q_ts = st[0].t; p.q_hs = st[0].h;
  p.k_bs = st[1].b; p.k_ts = st[1].t; p.k_hs = st[1].h;
  p.v_bs = st[2].b; p.v_ts = st[2].t; p.v_hs = st[2].h;
  p.o_bs = st[3].b; p.o_ts = st[3].t; p.o_hs = st[3].h;
}

constexpr float kLog2e = 1.44269504088896340736f;
const char* const kTensorNames[4] = {"q", "k", "v", "o"};

// Equal-length batch, any strides, either element type, any mask.
fa_status dense_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                    int32_t B, int32_t Nq, int32_t Nk, int32_t H, int32_t d,
                    const Strides st[4], int32_t dtype, float softmax_scale, Mask mask,
                    int32_t win_left, int32_t win_right, void* stream,
                    const uint8_t* kpm = nullptr) {
  if (!q || !k || !v || !o || !lse) return fail(FA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (B < 1 || Nq < 1 || Nk < 1) return fail(FA_ERR_INVALID_ARGUMENT, "B, Nq and Nk must be >= 1");
  fa_status st_ = check_common(H, d, softmax_scale);
  if (st_ != FA_OK) return st_;
  st_ = check_dtype(dtype);
  if (st_ != FA_OK) return st_;
  for (int i = 0; i < 4; ++i) {
    st_ = check_strides(st[i], kTensorNames[i]);
    if (st_ != FA_OK) return st_;
  }
  if ((mask == Mask::kCausal || mask == Mask::kPadCausal) && Nq != Nk)
    return fail(FA_ERR_INVALID_ARGUMENT, "causal attention needs Nq == Nk");
  if (mask == Mask::kBand && (Nq > kMaxBandLen || Nk > kMaxBandLen))
    return fail(FA_ERR_UNSUPPORTED, "banded attention supports Nq, Nk <= 2^29");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return fail(FA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  const int64_t n_qt = (Nq + rows_per_workgroup(d) - 1) / rows_per_workgroup(d);
  const int64_t grid = n_qt * H * (int64_t)B;
  if (grid > INT32_MAX) return fail(FA_ERR_UNSUPPORTED, "too many query tiles for one launch");
  st_ = check_device();
  if (st_ != FA_OK) return st_;

  fa::FwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.cu_seqlens = nullptr;
  set_strides(p, st);
  p.lse_head_stride = Nq;
  p.lse_batch_stride = (int64_t)H * Nq;
  p.Nq = Nq;
  p.Nk = Nk;
  p.H = H;
  p.nbatch = B;
  p.n_qtiles = (int32_t)n_qt;
  p.scale_log2 = std::fabs(softmax_scale) * kLog2e;
  p.q_sign = softmax_scale < 0.f ? 0x80008000u : 0u;
  p.win_left = window_side(win_left, Nq, Nk);
  p.win_right = window_side(win_right, Nq, Nk);
  p.band_off = Nk - Nq;
  p.kpm = kpm;
  p.kpm_batch_stride = Nk;
  hipError_t e = launch<false>(p, d, dtype, mask, (uint32_t)grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return FA_OK;
}

// Packed variable-length batch, any token and head strides, either element
// type, any mask (batch strides unused).
fa_status varlen_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                     int32_t total, int32_t H, int32_t d, const Strides st[4], int32_t dtype,
                     float softmax_scale, Mask mask, int32_t win_left, int32_t win_right,
                     void* stream) {
  if (!cu_seqlens) return fail(FA_ERR_INVALID_ARGUMENT, "null cu_seqlens");
  if (num_seqs < 1) return fail(FA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 1");
  if (total < 0 || max_seqlen < 0) return fail(FA_ERR_INVALID_ARGUMENT, "total and max_seqlen must be >= 0");
  if (max_seqlen > total) return fail(FA_ERR_INVALID_ARGUMENT, "max_seqlen exceeds total");
  fa_status st_ = check_common(H, d, softmax_scale);
  if (st_ != FA_OK) return st_;
  st_ = check_dtype(dtype);
  if (st_ != FA_OK) return st_;
  for (int i = 0; i < 4; ++i) {
    st_ = check_strides(st[i], kTensorNames[i]);
    if (st_ != FA_OK) return st_;
  }
  if (mask == Mask::kBand && max_seqlen > kMaxBandLen)
    return fail(FA_ERR_UNSUPPORTED, "banded attention supports max_seqlen <= 2^29");
  if (total == 0 || max_seqlen == 0) return FA_OK;   // nothing to compute
  if (!q || !k || !v || !o || !lse) return fail(FA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
    return fail(FA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned (cu_seqlens 4-byte)");
  const int64_t n_qt = (max_seqlen + rows_per_workgroup(d) - 1) / rows_per_workgroup(d);
  const int64_t grid = n_qt * H * (int64_t)num_seqs;
  if (grid > INT32_MAX) return fail(FA_ERR_UNSUPPORTED, "too many query tiles for one launch");
  st_ = check_device();
  if (st_ != FA_OK) return st_;

  fa::FwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.cu_seqlens = cu_seqlens;
  set_strides(p, st);
  p.lse_head_stride = total;
  p.lse_batch_stride = 0;
  p.Nq = 0;
  p.Nk = 0;
  p.H = H;
  p.nbatch = num_seqs;
  p.n_qtiles = (int32_t)n_qt;
  p.scale_log2 = std::fabs(softmax_scale) * kLog2e;
  p.q_sign = softmax_scale < 0.f ? 0x80008000u : 0u;
  p.win_left = window_side(win_left, max_seqlen, max_seqlen);
  p.win_right = window_side(win_right, max_seqlen, max_seqlen);
  p.band_off = 0;
  hipError_t e = launch<true>(p, d, dtype, mask, (uint32_t)grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return FA_OK;
}

// Densely packed (B, N, H, d) tensors, or (total, H, d) with batch stride 0.
void contiguous(int64_t Nq, int64_t Nk, int32_t H, int32_t d, Strides st[4]) {
  const int64_t t = (int64_t)H * d;
  st[0] = {Nq * t, t, d};
  st[1] = {Nk * t, t, d};
  st[2] = {Nk * t, t, d};
  st[3] = {Nq * t, t, d};
}

// Strides from the caller's arrays: n entries each (3 dense, 2 varlen).
fa_status read_strides(const int64_t* const in[4], int n, Strides st[4]) {
  for (int i = 0; i < 4; ++i) {
    if (!in[i]) return fail(FA_ERR_INVALID_ARGUMENT, std::string("null stride array for ") + kTensorNames[i]);
    st[i] = n == 3 ? Strides{in[i][0], in[i][1], in[i][2]} : Strides{0, in[i][0], in[i][1]};
  }
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int32_t B, int32_t Nq, int32_t Nk, int32_t H, int32_t d,
                 float softmax_scale, int32_t causal, void* stream) {
  g_last_error.clear();
  Mask mask;
  const fa_status st_ = mask_of(causal, -1, -1, &mask);
  if (st_ != FA_OK) return st_;
  Strides st[4];
  contiguous(Nq, Nk, H, d, st);
  return dense_fwd(q, k, v, o, lse, B, Nq, Nk, H, d, st, FA_DTYPE_BF16, softmax_scale, mask,
                   -1, -1, stream);
}

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                        int32_t total, int32_t H, int32_t d, float softmax_scale,
                        int32_t causal, void* stream) {
  g_last_error.clear();
  Mask mask;
  const fa_status st_ = mask_of(causal, -1, -1, &mask);
  if (st_ != FA_OK) return st_;
  Strides st[4];
  contiguous(0, 0, H, d, st);
  return varlen_fwd(q, k, v, o, lse, cu_seqlens, num_seqs, max_seqlen, total, H, d, st,
                    FA_DTYPE_BF16, softmax_scale, mask, -1, -1, stream);
}

fa_status fa_fwd_band(const void* q, const void* k, const void* v, void* o, float* lse,
                      int32_t B, int32_t Nq, int32_t Nk, int32_t H, int32_t d,
                      float softmax_scale, int32_t window_left, int32_t window_right,
                      void* stream) {
  g_last_error.clear();
  const fa_status st_ = check_window(window_left, window_right);
  if (st_ != FA_OK) return st_;
  Strides st[4];
  contiguous(Nq, Nk, H, d, st);
  return dense_fwd(q, k, v, o, lse, B, Nq, Nk, H, d, st, FA_DTYPE_BF16, softmax_scale,
                   Mask::kBand, window_left, window_right, stream);
}

fa_status fa_fwd_varlen_band(const void* q, const void* k, const void* v, void* o, float* lse,
                             const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                             int32_t total, int32_t H, int32_t d, float softmax_scale,
                             int32_t window_left, int32_t window_right, void* stream) {
  g_last_error.clear();
  const fa_status st_ = check_window(window_left, window_right);
  if (st_ != FA_OK) return st_;
  Strides st[4];
  contiguous(0, 0, H, d, st);
  return varlen_fwd(q, k, v, o, lse, cu_seqlens, num_seqs, max_seqlen, total, H, d, st,
                    FA_DTYPE_BF16, softmax_scale, Mask::kBand, window_left, window_right, stream);
}

fa_status fa_fwd_padded(const void* q, const void* k, const void* v, void* o, float* lse,
                        const uint8_t* key_padding_mask, int32_t B, int32_t S, int32_t H,
                        int32_t d, int32_t dtype, float softmax_scale, int32_t causal,
                        void* stream) {
  g_last_error.clear();
  if (!key_padding_mask) return fail(FA_ERR_INVALID_ARGUMENT, "null key_padding_mask");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  Strides st[4];
  contiguous(S, S, H, d, st);
  return dense_fwd(q, k, v, o, lse, B, S, S, H, d, st, dtype, softmax_scale,
                   causal ? Mask::kPadCausal : Mask::kPad, -1, -1, stream, key_padding_mask);
}

fa_status fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                         int32_t B, int32_t Nq, int32_t Nk, int32_t H, int32_t d,
                         const int64_t* q_strides, const int64_t* k_strides,
                         const int64_t* v_strides, const int64_t* o_strides, int32_t dtype,
                         float softmax_scale, int32_t causal, int32_t window_left,
                         int32_t window_right, void* stream) {
  g_last_error.clear();
  Mask mask;
  fa_status st_ = mask_of(causal, window_left, window_right, &mask);
  if (st_ != FA_OK) return st_;
  const int64_t* const in[4] = {q_strides, k_strides, v_strides, o_strides};
  Strides st[4];
  st_ = read_strides(in, 3, st);
  if (st_ != FA_OK) return st_;
  return dense_fwd(q, k, v, o, lse, B, Nq, Nk, H, d, st, dtype, softmax_scale, mask,
                   window_left, window_right, stream);
}

fa_status fa_fwd_varlen_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                                int32_t total, int32_t H, int32_t d, const int64_t* q_strides,
                                const int64_t* k_strides, const int64_t* v_strides,
                                const int64_t* o_strides, int32_t dtype, float softmax_scale,
                                int32_t causal, int32_t window_left, int32_t window_right,
                                void* stream) {
  g_last_error.clear();
  Mask mask;
  fa_status st_ = mask_of(causal, window_left, window_right, &mask);
  if (st_ != FA_OK) return st_;
  const int64_t* const in[4] = {q_strides, k_strides, v_strides, o_strides};
  Strides st[4];
  st_ = read_strides(in, 2, st);
  if (st_ != FA_OK) return st_;
  return varlen_fwd(q, k, v, o, lse, cu_seqlens, num_seqs, max_seqlen, total, H, d, st, dtype,
                    softmax_scale, mask, window_left, window_right, stream);
}

const char* fa_status_string(int32_t status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported shape or device";
    case FA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

int32_t fa_abi_version(void) { return 1; }

}  // extern "C"
