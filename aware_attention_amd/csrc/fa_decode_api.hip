// C ABI of the split-KV decode (fa_decode, fa_decode_workspace_bytes):
// argument checks, the split plan and the two launches. The operation is
// documented in include/fa.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <string>

#include "fa.h"
#include "fa_decode_kernel.hpp"
#include "fa_host.hpp"

namespace {

using fa_host::aligned16;
using fa_host::check_device;
using fa_host::fail;

// Chunks per (batch, head): enough workgroups to fill the chip (about 2048,
// eight per CU) without chunks shorter than 256 keys, and no chunk longer than
// the scores buffer of a workgroup. Chunks are multiples of 64 keys.
struct Plan {
  int splits, chunk;
};
Plan plan(int64_t B, int64_t Nk, int64_t H) {
  const int64_t units = B * H;
  int64_t splits = std::max<int64_t>(1, (2048 + units - 1) / units);
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, (Nk + 255) / 256));
  int64_t chunk = ((Nk + splits - 1) / splits + 63) / 64 * 64;
  if (chunk > fa::kDecMaxChunk) {
    chunk = fa::kDecMaxChunk;
    splits = (Nk + chunk - 1) / chunk;
  }
  return {(int)splits, (int)std::max<int64_t>(chunk, 64)};
}

template <int D, bool F16>
hipError_t launch_decode_t(const fa::DecodeParams& p, hipStream_t stream) {
  const uint32_t units = (uint32_t)(p.B * p.H);
  hipLaunchKernelGGL((fa::decode_split_kernel<D, F16>), dim3(units * (uint32_t)p.splits),
                     dim3(fa::kDecThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa::decode_merge_kernel<D, F16>), dim3(units), dim3(64), 0, stream, p);
  return hipGetLastError();
}

template <bool F16>
hipError_t launch_decode(const fa::DecodeParams& p, int d, hipStream_t stream) {
  switch (d) {
    case 32: return launch_decode_t<32, F16>(p, stream);
    case 64: return launch_decode_t<64, F16>(p, stream);
    case 128: return launch_decode_t<128, F16>(p, stream);
    default: return launch_decode_t<256, F16>(p, stream);
  }
}

// Checks shared by both decode entry points (everything but the workspace).
fa_status check_decode_args(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const int32_t* seqlens_k, int32_t B, int32_t Nk,
                            int32_t H, int32_t d, int32_t dtype, float softmax_scale) {
  if (!q || !k || !v || !o || !lse) return fail(FA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (B < 1 || Nk < 1 || H < 1) return fail(FA_ERR_INVALID_ARGUMENT, "B, Nk and H must be >= 1");
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
    return fail(FA_ERR_INVALID_ARGUMENT, "dtype must be FA_DTYPE_BF16 or FA_DTYPE_F16");
  if (!std::isfinite(softmax_scale)) return fail(FA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if (d != 32 && d != 64 && d != 128 && d != 256)
    return fail(FA_ERR_UNSUPPORTED, "head dim must be 32, 64, 128 or 256");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      (reinterpret_cast<uintptr_t>(seqlens_k) & 3u))
    return fail(FA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned (seqlens_k 4-byte)");
  const Plan s = plan(B, Nk, H);
  if ((int64_t)B * H * s.splits > INT32_MAX) return fail(FA_ERR_UNSUPPORTED, "too many chunks for one launch");
  return FA_OK;
}

// Both launches with the partial results at `workspace` (checked by the caller).
fa_status run_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                     const int32_t* seqlens_k, int32_t B, int32_t Nk, int32_t H, int32_t d,
                     int32_t dtype, float softmax_scale, void* workspace, void* stream) {
  const Plan s = plan(B, Nk, H);
  fa::DecodeParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.seqlens_k = seqlens_k;
  p.part_o = static_cast<float*>(workspace);
  p.part_l = p.part_o + (size_t)B * H * s.splits * d;
  p.kv_batch_stride = (int64_t)Nk * H * d;
  p.kv_token_stride = (int64_t)H * d;
  p.B = B;
  p.Nk = Nk;
  p.H = H;
  p.splits = s.splits;
  p.chunk = s.chunk;
  p.scale_log2 = softmax_scale * 1.44269504088896340736f;
  const hipError_t e = dtype == FA_DTYPE_F16
                           ? launch_decode<true>(p, d, static_cast<hipStream_t>(stream))
                           : launch_decode<false>(p, d, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return FA_OK;
}

// ---- the library-held scratch of fa_decode_noalloc ----
// One array per GPU, in device memory the code object reserves when it is
// loaded on that GPU (no allocation call), held until the process ends. Host
// code never uses the array's name as an address: the device address of this
// GPU's copy comes from hipGetSymbolAddress, looked up once per device (with
// that device current) and kept in g_scratch_addr.
constexpr size_t kNoAllocScratchBytes = FA_DECODE_NOALLOC_SCRATCH_BYTES;
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kScratchDevices] = {};

}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

// This device's address of `scratch` (nullptr and the error recorded on failure).
void* scratch_address(fa_status* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = fail(FA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kScratchDevices) {
    *st = fail(FA_ERR_UNSUPPORTED, "device ordinal out of range");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *st = fail(FA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                 (e != hipSuccess ? hipGetErrorString(e) : "null address"));
      return nullptr;
    }
    g_scratch_addr[dev] = ptr;
  }
  *st = FA_OK;
  return g_scratch_addr[dev];
}

}  // namespace

extern "C" {

size_t fa_decode_workspace_bytes(int32_t B, int32_t Nk, int32_t H, int32_t d) {
  if (B < 1 || Nk < 1 || H < 1 || d < 1) return 0;
  const Plan s = plan(B, Nk, H);
  return (size_t)B * H * s.splits * ((size_t)d + 1) * sizeof(float);
}

fa_status fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* seqlens_k, int32_t B, int32_t Nk, int32_t H, int32_t d,
                    int32_t dtype, float softmax_scale, void* workspace, size_t workspace_bytes,
                    void* stream) {
  fa_host::g_last_error.clear();
  if (!workspace) return fail(FA_ERR_INVALID_ARGUMENT, "null workspace pointer");
  fa_status st = check_decode_args(q, k, v, o, lse, seqlens_k, B, Nk, H, d, dtype, softmax_scale);
  if (st != FA_OK) return st;
  if (!aligned16(workspace)) return fail(FA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  if (workspace_bytes < fa_decode_workspace_bytes(B, Nk, H, d))
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace smaller than fa_decode_workspace_bytes()");
  st = check_device();
  if (st != FA_OK) return st;
  return run_decode(q, k, v, o, lse, seqlens_k, B, Nk, H, d, dtype, softmax_scale, workspace, stream);
}

fa_status fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* seqlens_k, int32_t B, int32_t Nk, int32_t H,
                            int32_t d, int32_t dtype, float softmax_scale, void* stream) {
  fa_host::g_last_error.clear();
  fa_status st = check_decode_args(q, k, v, o, lse, seqlens_k, B, Nk, H, d, dtype, softmax_scale);
  if (st != FA_OK) return st;
  const size_t need = fa_decode_workspace_bytes(B, Nk, H, d);
  if (need > kNoAllocScratchBytes)
    return fail(FA_ERR_UNSUPPORTED, "these sizes need " + std::to_string(need) +
                                        " bytes of partial results, above the " +
                                        std::to_string(kNoAllocScratchBytes) +
                                        " bytes fa_decode_noalloc holds; use fa_decode");
  st = check_device();
  if (st != FA_OK) return st;
  void* ws = scratch_address(&st);
  if (!ws) return st;
  return run_decode(q, k, v, o, lse, seqlens_k, B, Nk, H, d, dtype, softmax_scale, ws, stream);
}

}  // extern "C"
