// C ABI of the local-window + global-anchor forward (fa_fwd_local): argument
// checks, the clamping of the pattern's sizes to the map and the launch. The
// operation is documented in include/fa.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <string>

#include "fa.h"
#include "fa_host.hpp"
#include "fa_local_kernel.hpp"

namespace {

using fa_host::aligned16;
using fa_host::check_device;
using fa_host::fail;

constexpr int32_t kMaxLocalTokens = 1 << 28;   // keeps the map arithmetic in int32

template <int D, bool CAUSAL, bool F16>
hipError_t launch_local_t(const fa::LocalParams& p, uint32_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((fa::fwd_local_kernel<D, CAUSAL, F16>), dim3(grid), dim3(fa::kBwdThreads), 0,
                     stream, p);
  return hipGetLastError();
}

template <bool CAUSAL, bool F16>
hipError_t launch_local_d(const fa::LocalParams& p, int d, uint32_t grid, hipStream_t stream) {
  switch (d) {
    case 32: return launch_local_t<32, CAUSAL, F16>(p, grid, stream);
    case 64: return launch_local_t<64, CAUSAL, F16>(p, grid, stream);
    case 128: return launch_local_t<128, CAUSAL, F16>(p, grid, stream);
    default: return launch_local_t<256, CAUSAL, F16>(p, grid, stream);
  }
}

}  // namespace

extern "C" {

fa_status fa_fwd_local(const void* q, const void* k, const void* v, void* o, float* lse,
                       int32_t B, int32_t N, int32_t H, int32_t d, int32_t dtype,
                       float softmax_scale, int32_t causal, int32_t n_global, int32_t map_w,
                       int32_t win_rows, int32_t win_cols, void* stream) {
  fa_host::g_last_error.clear();
  if (!q || !k || !v || !o || !lse) return fail(FA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (B < 1 || N < 1 || H < 1) return fail(FA_ERR_INVALID_ARGUMENT, "B, N and H must be >= 1");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
    return fail(FA_ERR_INVALID_ARGUMENT, "dtype must be FA_DTYPE_BF16 or FA_DTYPE_F16");
  if (!std::isfinite(softmax_scale)) return fail(FA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if (n_global < 0 || map_w < 1 || win_rows < 0 || win_cols < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "need n_global >= 0, map_w >= 1, win_rows >= 0, win_cols >= 0");
  if (d != 32 && d != 64 && d != 128 && d != 256)
    return fail(FA_ERR_UNSUPPORTED, "head dim must be 32, 64, 128 or 256");
  if (N > kMaxLocalTokens) return fail(FA_ERR_UNSUPPORTED, "local attention supports N <= 2^28");
  if ((int64_t)H * d > (1 << 24)) return fail(FA_ERR_UNSUPPORTED, "H * d above 2^24");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return fail(FA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  // Anchor queries and map queries take separate 128-query tiles, anchors first.
  const int64_t G64 = std::min<int64_t>(n_global, N);
  const int64_t n_anchor_tiles = (G64 + fa::kLocalRows - 1) / fa::kLocalRows;
  const int64_t n_tiles = n_anchor_tiles + (N - G64 + fa::kLocalRows - 1) / fa::kLocalRows;
  const int64_t grid = n_tiles * H * B;
  if (grid > INT32_MAX) return fail(FA_ERR_UNSUPPORTED, "too many query tiles for one launch");
  fa_status st = check_device();
  if (st != FA_OK) return st;

  // Sizes beyond the map's extent change nothing; clamping them keeps the
  // kernel's index arithmetic small.
  const int32_t G = std::min(n_global, N);
  const int32_t rest = N - G;
  const int32_t W = std::min(map_w, std::max(1, rest));
  const int32_t rows = rest > 0 ? (rest + W - 1) / W : 0;
  fa::LocalParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.row_stride = (int64_t)H * d;
  p.batch_stride = (int64_t)N * H * d;
  p.N = N;
  p.H = H;
  p.B = B;
  p.n_global = G;
  p.map_w = W;
  p.win_rows = std::min(win_rows, rows);
  p.win_cols = std::min(win_cols, W);
  p.n_anchor_tiles = (int32_t)n_anchor_tiles;
  p.n_tiles = (int32_t)n_tiles;
  p.scale_log2 = softmax_scale * 1.44269504088896340736f;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f16 = dtype == FA_DTYPE_F16;
  const hipError_t e =
      causal ? (f16 ? launch_local_d<true, true>(p, d, (uint32_t)grid, s)
                    : launch_local_d<true, false>(p, d, (uint32_t)grid, s))
             : (f16 ? launch_local_d<false, true>(p, d, (uint32_t)grid, s)
                    : launch_local_d<false, false>(p, d, (uint32_t)grid, s));
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return FA_OK;
}

}  // extern "C"
