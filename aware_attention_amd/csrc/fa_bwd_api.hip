// C ABI of the backward pass (fa_bwd, fa_bwd_varlen, their band,
// padding-mask and local-window forms, and the strided forms fa_bwd_strided
// and fa_bwd_varlen_strided): argument checks and the three launches. The
// operation is documented in include/fa.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <string>

#include "fa.h"
#include "fa_bwd_kernel.hpp"
#include "fa_host.hpp"

namespace {

using fa_host::aligned16;
using fa_host::check_device;
using fa_host::fail;

template <int D, bool CAUSAL, bool VARLEN, bool F16, bool BAND, bool KPM, bool LOCAL>
hipError_t launch_bwd_t(const fa::BwdParams& p, int64_t nrows, int N, uint32_t grid_k,
                        uint32_t grid_q, hipStream_t stream) {
  constexpr int kDeltaRows = fa::kDeltaThreads / (D / 8);
  hipLaunchKernelGGL((fa::delta_kernel<D, F16>),
                     dim3((uint32_t)((nrows + kDeltaRows - 1) / kDeltaRows)),
                     dim3(fa::kDeltaThreads), 0, stream, p.o, p.dout, p.delta, p.H, N, (int)nrows,
                     p.st[fa::kTO], p.st[fa::kTdO]);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // d = 256: two dK/dV workgroups per key tile, one per half of the head dimension.
  hipLaunchKernelGGL((fa::dkdv_kernel<D, CAUSAL, VARLEN, F16, BAND, KPM, LOCAL>),
                     dim3(D == 256 ? 2 * grid_k : grid_k), dim3(fa::kBwdThreads), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  fa::BwdParams pq = p;
  pq.n_tiles = (int32_t)(grid_q / (uint32_t)(p.H * p.nbatch));
  hipLaunchKernelGGL((fa::dq_kernel<D, CAUSAL, VARLEN, F16, BAND, KPM, LOCAL>), dim3(grid_q),
                     dim3(fa::kBwdThreads), 0, stream, pq);
  return hipGetLastError();
}

template <bool CAUSAL, bool VARLEN, bool F16, bool BAND, bool KPM, bool LOCAL = false>
hipError_t launch_bwd_d(const fa::BwdParams& p, int d, int64_t nrows, int N, uint32_t grid_k,
                        uint32_t grid_q, hipStream_t stream) {
  switch (d) {
    case 32:
      return launch_bwd_t<32, CAUSAL, VARLEN, F16, BAND, KPM, LOCAL>(p, nrows, N, grid_k, grid_q,
                                                                   stream);
    case 64:
      return launch_bwd_t<64, CAUSAL, VARLEN, F16, BAND, KPM, LOCAL>(p, nrows, N, grid_k, grid_q,
                                                                   stream);
    case 256:
      return launch_bwd_t<256, CAUSAL, VARLEN, F16, BAND, KPM, LOCAL>(p, nrows, N, grid_k, grid_q,
                                                                    stream);
    default:
      return launch_bwd_t<128, CAUSAL, VARLEN, F16, BAND, KPM, LOCAL>(p, nrows, N, grid_k, grid_q,
                                                                    stream);
  }
}

// Mask of a backward launch: none, causal, a band (dense or varlen), a key
// padding mask (dense) or the local window + anchor pattern (dense), the last
// two alone or with causal.
enum class BwdMask { kNone, kCausal, kBand, kPad, kPadCausal, kLocal, kLocalCausal };

template <bool VARLEN, bool F16>
hipError_t launch_bwd_m(const fa::BwdParams& p, int d, BwdMask mask, int64_t nrows, int N,
                        uint32_t grid_k, uint32_t grid_q, hipStream_t stream) {
  switch (mask) {
    case BwdMask::kCausal:
      return launch_bwd_d<true, VARLEN, F16, false, false>(p, d, nrows, N, grid_k, grid_q, stream);
    case BwdMask::kBand:
      return launch_bwd_d<false, VARLEN, F16, true, false>(p, d, nrows, N, grid_k, grid_q, stream);
    case BwdMask::kPad:
    case BwdMask::kPadCausal:
      if constexpr (!VARLEN) {
        return mask == BwdMask::kPad
                   ? launch_bwd_d<false, false, F16, false, true>(p, d, nrows, N, grid_k, grid_q, stream)
                   : launch_bwd_d<true, false, F16, false, true>(p, d, nrows, N, grid_k, grid_q, stream);
      }
      return hipErrorInvalidValue;
    case BwdMask::kLocal:
    case BwdMask::kLocalCausal:
      if constexpr (!VARLEN) {
        return mask == BwdMask::kLocal
                   ? launch_bwd_d<false, false, F16, false, false, true>(p, d, nrows, N, grid_k,
                                                                         grid_q, stream)
                   : launch_bwd_d<true, false, F16, false, false, true>(p, d, nrows, N, grid_k,
                                                                        grid_q, stream);
      }
      return hipErrorInvalidValue;
    default:
      return launch_bwd_d<false, VARLEN, F16, false, false>(p, d, nrows, N, grid_k, grid_q, stream);
  }
}

template <bool VARLEN>
hipError_t launch_bwd(const fa::BwdParams& p, int d, int32_t dtype, BwdMask mask, int64_t nrows,
                      int N, uint32_t grid_k, uint32_t grid_q, hipStream_t stream) {
  return dtype == FA_DTYPE_F16
             ? launch_bwd_m<VARLEN, true>(p, d, mask, nrows, N, grid_k, grid_q, stream)
             : launch_bwd_m<VARLEN, false>(p, d, mask, nrows, N, grid_k, grid_q, stream);
}

// Window sides: >= 0, or -1 for unbounded (passed to the kernels as
// max(nq, nk), which reaches every key); sequences up to 2^29 keep the
// kernels' 32-bit band bounds in range.
int32_t bwd_window_side(int32_t w, int64_t nq, int64_t nk) {
  const int64_t unbounded = nq > nk ? nq : nk;
  return (int32_t)((w < 0 || w > unbounded) ? unbounded : w);
}
constexpr int64_t kMaxBandLenBwd = int64_t{1} << 29;

fa_status check_bwd_common(int32_t H, int32_t d, int32_t dtype, float scale, int32_t causal) {
  if (H < 1) return fail(FA_ERR_INVALID_ARGUMENT, "H must be >= 1");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
    return fail(FA_ERR_INVALID_ARGUMENT, "dtype must be FA_DTYPE_BF16 or FA_DTYPE_F16");
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if (d != 32 && d != 64 && d != 128 && d != 256)
    return fail(FA_ERR_UNSUPPORTED, "head dim must be 32, 64, 128 or 256");
  return FA_OK;
}

bool all_aligned(const void* const* ptrs, int n) {
  for (int i = 0; i < n; ++i)
    if (!ptrs[i] || !aligned16(ptrs[i])) return false;
  return true;
}

constexpr float kLog2eHost = 1.44269504088896340736f;

using Strides = fa::BwdStrides;
const char* const kBwdNames[fa::kBwdTensors] = {"q", "k", "v", "o", "dout", "dq", "dk", "dv"};
// Token strides up to 2^24 elements keep the per-lane 32-bit byte offsets of
// the kernels' 64-row tile copies in range.
constexpr int64_t kMaxTokenStrideBwd = int64_t{1} << 24;

fa_status check_bwd_strides(const Strides st[fa::kBwdTensors]) {
  for (int i = 0; i < fa::kBwdTensors; ++i) {
    const Strides& s = st[i];
    const std::string name = kBwdNames[i];
    if (s.b < 0 || s.t < 0 || s.h < 0) return fail(FA_ERR_INVALID_ARGUMENT, name + ": strides must be >= 0");
    if ((s.b | s.t | s.h) & 7)
      return fail(FA_ERR_INVALID_ARGUMENT,
                  name + ": strides must be multiples of 8 elements (16-byte aligned rows)");
    if (s.t > kMaxTokenStrideBwd)
      return fail(FA_ERR_UNSUPPORTED, name + ": token stride above 2^24 elements");
  }
  return FA_OK;
}

// Densely packed (B, Nq|Nk, H, d) tensors (varlen: (total, H, d), the batch
// strides unused).
void contiguous_bwd(int64_t Nq, int64_t Nk, int32_t H, int32_t d, Strides st[fa::kBwdTensors]) {
  const int64_t t = (int64_t)H * d;
  const Strides sq{Nq * t, t, d}, sk{Nk * t, t, d};
  st[fa::kTQ] = st[fa::kTO] = st[fa::kTdO] = st[fa::kTdQ] = sq;
  st[fa::kTK] = st[fa::kTV] = st[fa::kTdK] = st[fa::kTdV] = sk;
}

// Strides from the caller's array: n entries per tensor (3 dense: batch,
// token, head; 2 varlen: token, head), tensors in the order of BwdTensor.
fa_status read_bwd_strides(const int64_t* in, int n, Strides st[fa::kBwdTensors]) {
  if (!in) return fail(FA_ERR_INVALID_ARGUMENT, "null stride array");
  for (int i = 0; i < fa::kBwdTensors; ++i) {
    const int64_t* x = in + n * i;
    st[i] = n == 3 ? Strides{x[0], x[1], x[2]} : Strides{0, x[0], x[1]};
  }
  return check_bwd_strides(st);
}

// Local window + anchors of fa_bwd_local (the forward's fa_fwd_local pattern).
struct LocalPattern {
  int32_t n_global, map_w, win_rows, win_cols;
};
constexpr int32_t kMaxLocalTokensBwd = 1 << 28;   // keeps the map arithmetic in int32

fa_status dense_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, float* delta, int32_t B,
                    int32_t Nq, int32_t Nk, int32_t H, int32_t d, int32_t dtype,
                    float softmax_scale, int32_t causal, BwdMask mask, int32_t win_left,
                    int32_t win_right, const uint8_t* kpm, void* stream,
                    const LocalPattern* loc = nullptr, const Strides* strides = nullptr) {
  const void* ptrs[10] = {q, k, v, o, dout, lse, dq, dk, dv, delta};
  for (const void* x : ptrs)
    if (!x) return fail(FA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (B < 1 || Nq < 1 || Nk < 1) return fail(FA_ERR_INVALID_ARGUMENT, "B, Nq and Nk must be >= 1");
  fa_status st = check_bwd_common(H, d, dtype, softmax_scale, causal);
  if (st != FA_OK) return st;
  if (causal && Nq != Nk) return fail(FA_ERR_INVALID_ARGUMENT, "causal attention needs Nq == Nk");
  if (mask == BwdMask::kBand && (Nq > kMaxBandLenBwd || Nk > kMaxBandLenBwd))
    return fail(FA_ERR_UNSUPPORTED, "banded attention supports Nq, Nk <= 2^29");
  if (loc && Nq > kMaxLocalTokensBwd)
    return fail(FA_ERR_UNSUPPORTED, "local attention supports N <= 2^28");
  if (!all_aligned(ptrs, 10)) return fail(FA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  if (!strides && (int64_t)H * d > kMaxTokenStrideBwd)
    return fail(FA_ERR_UNSUPPORTED, "H * d above 2^24");
  const int64_t units = (int64_t)H * B;
  const int64_t grid_k = (Nk + fa::kBwdRows - 1) / fa::kBwdRows * units;
  const int64_t grid_q = (Nq + fa::kBwdRows - 1) / fa::kBwdRows * units;
  const int64_t nrows = (int64_t)B * Nq * H;
  // (the D = dO . O launch numbers its rows with 32-bit integers)
  if (grid_k * (d == 256 ? 2 : 1) > INT32_MAX || grid_q > INT32_MAX || nrows > INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, "too many tiles or rows (B * N * H above 2^31 - 1) for one launch");
  st = check_device();
  if (st != FA_OK) return st;

  fa::BwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.delta = delta;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.cu_seqlens = nullptr;
  if (strides)
    std::copy(strides, strides + fa::kBwdTensors, p.st);
  else
    contiguous_bwd(Nq, Nk, H, d, p.st);
  p.lse_batch_stride = (int64_t)H * Nq;
  p.lse_head_stride = Nq;
  p.Nq = Nq;
  p.Nk = Nk;
  p.H = H;
  p.nbatch = B;
  p.n_tiles = (int32_t)(grid_k / units);
  p.scale = softmax_scale;
  p.scale_log2 = softmax_scale * kLog2eHost;
  p.win_left = bwd_window_side(win_left, Nq, Nk);
  p.win_right = bwd_window_side(win_right, Nq, Nk);
  p.band_off = Nk - Nq;
  p.kpm = kpm;
  p.kpm_batch_stride = Nk;
  if (loc) {   // sizes beyond the map's extent change nothing: clamp them (as the forward)
    const int32_t G = std::min(loc->n_global, Nq);
    const int32_t rest = Nq - G;
    const int32_t W = std::min(loc->map_w, std::max(1, rest));
    const int32_t rows = rest > 0 ? (rest + W - 1) / W : 0;
    p.n_global = G;
    p.map_w = W;
    p.loc_rows = std::min(loc->win_rows, rows);
    p.loc_cols = std::min(loc->win_cols, W);
  }
  const hipError_t e = launch_bwd<false>(p, d, dtype, mask, nrows, Nq, (uint32_t)grid_k,
                                         (uint32_t)grid_q, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return FA_OK;
}

fa_status varlen_bwd(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                     float* delta, const int32_t* cu_seqlens, int32_t num_seqs,
                     int32_t max_seqlen, int32_t total, int32_t H, int32_t d, int32_t dtype,
                     float softmax_scale, int32_t causal, BwdMask mask, int32_t win_left,
                     int32_t win_right, void* stream, const Strides* strides = nullptr) {
  if (!cu_seqlens) return fail(FA_ERR_INVALID_ARGUMENT, "null cu_seqlens");
  if (num_seqs < 1) return fail(FA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 1");
  if (total < 0 || max_seqlen < 0) return fail(FA_ERR_INVALID_ARGUMENT, "total and max_seqlen must be >= 0");
  if (max_seqlen > total) return fail(FA_ERR_INVALID_ARGUMENT, "max_seqlen exceeds total");
  fa_status st = check_bwd_common(H, d, dtype, softmax_scale, causal);
  if (st != FA_OK) return st;
  if (mask == BwdMask::kBand && max_seqlen > kMaxBandLenBwd)
    return fail(FA_ERR_UNSUPPORTED, "banded attention supports max_seqlen <= 2^29");
  if (!strides && (int64_t)H * d > kMaxTokenStrideBwd)
    return fail(FA_ERR_UNSUPPORTED, "H * d above 2^24");
  if (total == 0 || max_seqlen == 0) return FA_OK;   // nothing to compute
  const void* ptrs[10] = {q, k, v, o, dout, lse, dq, dk, dv, delta};
  for (const void* x : ptrs)
    if (!x) return fail(FA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (!all_aligned(ptrs, 10) || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
    return fail(FA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned (cu_seqlens 4-byte)");
  const int64_t units = (int64_t)H * num_seqs;
  const int64_t n_t = (max_seqlen + fa::kBwdRows - 1) / fa::kBwdRows;
  const int64_t grid = n_t * units;
  const int64_t nrows = (int64_t)total * H;
  if (grid * (d == 256 ? 2 : 1) > INT32_MAX || nrows > INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, "too many tiles or rows (B * N * H above 2^31 - 1) for one launch");
  st = check_device();
  if (st != FA_OK) return st;

  fa::BwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.delta = delta;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.cu_seqlens = cu_seqlens;
  if (strides)
    std::copy(strides, strides + fa::kBwdTensors, p.st);
  else
    contiguous_bwd(total, total, H, d, p.st);
  p.lse_batch_stride = 0;
  p.lse_head_stride = total;
  p.Nq = 0;
  p.Nk = 0;
  p.H = H;
  p.nbatch = num_seqs;
  p.n_tiles = (int32_t)n_t;
  p.scale = softmax_scale;
  p.scale_log2 = softmax_scale * kLog2eHost;
  p.win_left = bwd_window_side(win_left, max_seqlen, max_seqlen);
  p.win_right = bwd_window_side(win_right, max_seqlen, max_seqlen);
  p.band_off = 0;
  const hipError_t e = launch_bwd<true>(p, d, dtype, mask, nrows, total, (uint32_t)grid,
                                        (uint32_t)grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return FA_OK;
}

fa_status check_bwd_window(int32_t left, int32_t right) {
  if (left < -1 || right < -1)
    return fail(FA_ERR_INVALID_ARGUMENT, "window sides must be >= 0, or -1 for unbounded");
  return FA_OK;
}

// The mask named by a causal flag and a window, as taken by the strided
// entry points: causal, or no mask when both sides are unbounded, else a band.
fa_status bwd_mask_of(int32_t causal, int32_t left, int32_t right, BwdMask* mask) {
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  const fa_status st = check_bwd_window(left, right);
  if (st != FA_OK) return st;
  const bool unbounded = left == -1 && right == -1;
  if (causal && !unbounded)
    return fail(FA_ERR_INVALID_ARGUMENT, "causal and a window are exclusive (causal is window (-1, 0))");
  *mask = causal ? BwdMask::kCausal : (unbounded ? BwdMask::kNone : BwdMask::kBand);
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, float* delta, int32_t B,
                 int32_t Nq, int32_t Nk, int32_t H, int32_t d, int32_t dtype,
                 float softmax_scale, int32_t causal, void* stream) {
  fa_host::g_last_error.clear();
  return dense_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, Nq, Nk, H, d, dtype, softmax_scale,
                   causal, causal == 1 ? BwdMask::kCausal : BwdMask::kNone, -1, -1, nullptr, stream);
}

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        float* delta, const int32_t* cu_seqlens, int32_t num_seqs,
                        int32_t max_seqlen, int32_t total, int32_t H, int32_t d, int32_t dtype,
                        float softmax_scale, int32_t causal, void* stream) {
  fa_host::g_last_error.clear();
  return varlen_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, cu_seqlens, num_seqs, max_seqlen,
                    total, H, d, dtype, softmax_scale, causal,
                    causal == 1 ? BwdMask::kCausal : BwdMask::kNone, -1, -1, stream);
}

fa_status fa_bwd_band(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      float* delta, int32_t B, int32_t Nq, int32_t Nk, int32_t H, int32_t d,
                      int32_t dtype, float softmax_scale, int32_t window_left,
                      int32_t window_right, void* stream) {
  fa_host::g_last_error.clear();
  const fa_status st = check_bwd_window(window_left, window_right);
  if (st != FA_OK) return st;
  return dense_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, Nq, Nk, H, d, dtype, softmax_scale,
                   0, BwdMask::kBand, window_left, window_right, nullptr, stream);
}

fa_status fa_bwd_varlen_band(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             float* delta, const int32_t* cu_seqlens, int32_t num_seqs,
                             int32_t max_seqlen, int32_t total, int32_t H, int32_t d,
                             int32_t dtype, float softmax_scale, int32_t window_left,
                             int32_t window_right, void* stream) {
  fa_host::g_last_error.clear();
  const fa_status st = check_bwd_window(window_left, window_right);
  if (st != FA_OK) return st;
  return varlen_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, cu_seqlens, num_seqs, max_seqlen,
                    total, H, d, dtype, softmax_scale, 0, BwdMask::kBand, window_left,
                    window_right, stream);
}

fa_status fa_bwd_padded(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        float* delta, const uint8_t* key_padding_mask, int32_t B, int32_t S,
                        int32_t H, int32_t d, int32_t dtype, float softmax_scale, int32_t causal,
                        void* stream) {
  fa_host::g_last_error.clear();
  if (!key_padding_mask) return fail(FA_ERR_INVALID_ARGUMENT, "null key_padding_mask");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  return dense_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, S, S, H, d, dtype, softmax_scale,
                   causal, causal ? BwdMask::kPadCausal : BwdMask::kPad, -1, -1, key_padding_mask,
                   stream);
}

fa_status fa_bwd_local(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       float* delta, int32_t B, int32_t N, int32_t H, int32_t d, int32_t dtype,
                       float softmax_scale, int32_t causal, int32_t n_global, int32_t map_w,
                       int32_t win_rows, int32_t win_cols, void* stream) {
  fa_host::g_last_error.clear();
  if (n_global < 0 || map_w < 1 || win_rows < 0 || win_cols < 0)
    return fail(FA_ERR_INVALID_ARGUMENT,
                "need n_global >= 0, map_w >= 1, win_rows >= 0, win_cols >= 0");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  const LocalPattern loc{n_global, map_w, win_rows, win_cols};
  return dense_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, N, N, H, d, dtype, softmax_scale,
                   causal, causal ? BwdMask::kLocalCausal : BwdMask::kLocal, -1, -1, nullptr,
                   stream, &loc);
}

fa_status fa_bwd_strided(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         float* delta, int32_t B, int32_t Nq, int32_t Nk, int32_t H, int32_t d,
                         const int64_t* strides, int32_t dtype, float softmax_scale,
                         int32_t causal, int32_t window_left, int32_t window_right,
                         void* stream) {
  fa_host::g_last_error.clear();
  Strides st[fa::kBwdTensors];
  fa_status s = read_bwd_strides(strides, 3, st);
  if (s != FA_OK) return s;
  BwdMask mask;
  s = bwd_mask_of(causal, window_left, window_right, &mask);
  if (s != FA_OK) return s;
  return dense_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, Nq, Nk, H, d, dtype, softmax_scale,
                   causal, mask, window_left, window_right, nullptr, stream, nullptr, st);
}

fa_status fa_bwd_varlen_strided(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                float* delta, const int32_t* cu_seqlens, int32_t num_seqs,
                                int32_t max_seqlen, int32_t total, int32_t H, int32_t d,
                                const int64_t* strides, int32_t dtype, float softmax_scale,
                                int32_t causal, int32_t window_left, int32_t window_right,
                                void* stream) {
  fa_host::g_last_error.clear();
  Strides st[fa::kBwdTensors];
  fa_status s = read_bwd_strides(strides, 2, st);
  if (s != FA_OK) return s;
  BwdMask mask;
  s = bwd_mask_of(causal, window_left, window_right, &mask);
  if (s != FA_OK) return s;
  return varlen_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, cu_seqlens, num_seqs, max_seqlen,
                    total, H, d, dtype, softmax_scale, causal, mask, window_left, window_right,
                    stream, st);
}

}  // extern "C"
