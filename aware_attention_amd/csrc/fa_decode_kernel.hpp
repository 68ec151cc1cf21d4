// Split-KV decode for one query per (batch, head) on gfx950: device code.
//
// With a single query the scores are a matrix-vector product over the KV
// cache: the work is one pass over K and V, so the kernels are laid out for
// HBM bandwidth, not for the matrix cores. Each (batch, head) cache is cut
// into chunks handled by separate workgroups (enough of them to fill the 256
// CUs), and the partial results are merged exactly through their
// log-sum-exps ("FlashAttention/zh" (marovi.ai wiki), section
// FlashAttention 算法: the forward keeps L = m + log l per row; attention
// over a union of key sets is the L-weighted combination of the parts):
//   * split_kernel: rows of K and V are read in 16-byte chunks, D/8 lanes
//     per row (coalesced), four rows per lane in flight; each lane keeps its
//     8 elements of q (scaled by scale * log2 e) in registers, and a row's
//     partial dot products are summed across its lanes with shuffles; the
//     chunk's max and sum come from wave and LDS reductions; O_s =
//     sum_j p_j v_j / l accumulates per lane over its chunk of the rows and is
//     summed across row groups in LDS; writes O_s (fp32) and L_s = m + log2 l
//     (base 2) to the workspace;
//   * merge_kernel: L = log2 sum_s 2^{L_s}, O = sum_s 2^{L_s - L} O_s, then O
//     in the input type and L in natural-log units. A cache of length 0 (or a
//     chunk past it) contributes L_s = -inf; a row with no key gets O = 0 and
//     L = -inf.
#pragma once

#include "fa_bwd_kernel.hpp"   // half_to_float, pack2, vector types

namespace fa {

struct DecodeParams {
  const uint16_t* q;           // (B, H, d): the one query row of each (batch, head)
  const uint16_t* k;           // (B, Nk, H, d)
  const uint16_t* v;           // (B, Nk, H, d)
  uint16_t* o;                 // (B, H, d)
  float* lse;                  // (B, H)
  const int32_t* seqlens_k;    // DEVICE int32[B] or null: batch b uses keys [0, len_b)
  float* part_o;               // workspace: (B, H, splits, d) fp32
  float* part_l;               // workspace: (B, H, splits) fp32, base-2 log-sum-exp
  int64_t kv_batch_stride;     // Nk * H * d
  int64_t kv_token_stride;     // H * d
  int32_t B, Nk, H, splits, chunk;
  float scale_log2;            // softmax scale * log2(e)
};

constexpr int kDecThreads = 256;
constexpr int kDecMaxChunk = 4096;   // keys per workgroup (fp32 scores in LDS)

__device__ __forceinline__ float dec_block_reduce(float x, bool is_max, float* red, int tid) {
  for (int off = 32; off > 0; off >>= 1) {
    const float y = __shfl_xor(x, off, 64);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  __syncthreads();   // red may still be read by the previous reduction
  if ((tid & 63) == 0) red[tid >> 6] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kDecThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

template <int D, bool F16>
__global__ __attribute__((amdgpu_flat_work_group_size(kDecThreads, kDecThreads)))
void decode_split_kernel(DecodeParams p) {
  // Both passes read rows in 16-byte chunks: TPR = D/8 lanes cover one row
  // (its loads are contiguous), so a wave reads 64/TPR rows per instruction
  // and the workgroup G = 256/TPR rows per step; lane (g, c) owns chunk c of
  // rows g, g + G, ... Four rows per lane are loaded before they are used.
  constexpr int TPR = D / 8;
  constexpr int G = kDecThreads / TPR;
  constexpr int U = 4;
  __shared__ float sc[kDecMaxChunk];
  __shared__ float red[kDecThreads / 64];
  __shared__ float ored[G * D];
  const int tid = threadIdx.x;
  const int c = tid % TPR, g = tid / TPR;
  const int split = blockIdx.x % p.splits;
  const int bh = blockIdx.x / p.splits;
  const int h = bh % p.H, b = bh / p.H;
  int len = p.Nk;
  if (p.seqlens_k) len = max(0, min(p.seqlens_k[b], p.Nk));
  const int c0 = split * p.chunk;
  const int c1 = min(len, c0 + p.chunk);

  // This lane's 8 elements of q, scaled by scale * log2(e).
  float qv[8];
  {
    const u32x4 x = *reinterpret_cast<const u32x4*>(p.q + (int64_t)bh * D + 8 * c);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      qv[2 * w] = half_to_float<F16>((uint16_t)(x[w] & 0xffff)) * p.scale_log2;
      qv[2 * w + 1] = half_to_float<F16>((uint16_t)(x[w] >> 16)) * p.scale_log2;
    }
  }
  const uint16_t* kb = p.k + (int64_t)b * p.kv_batch_stride + (int64_t)h * D + 8 * c;
  const uint16_t* vb = p.v + (int64_t)b * p.kv_batch_stride + (int64_t)h * D + 8 * c;
  const int64_t ts = p.kv_token_stride;

  // Scores (base 2): partial dot products over the lane's chunk, summed over
  // the TPR lanes of the row.
  float mloc = kNegInf;
  for (int j0 = c0 + g; j0 < c1; j0 += U * G) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * G;
      x[u] = j < c1 ? *reinterpret_cast<const u32x4*>(kb + (int64_t)j * ts) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc = __builtin_fmaf(half_to_float<F16>((uint16_t)(x[u][w] & 0xffff)), qv[2 * w], acc);
        acc = __builtin_fmaf(half_to_float<F16>((uint16_t)(x[u][w] >> 16)), qv[2 * w + 1], acc);
      }
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
      const int j = j0 + u * G;
      if (j < c1) {
        if (c == 0) sc[j - c0] = acc;
        mloc = fmaxf(mloc, acc);
      }
    }
  }
  const float m = dec_block_reduce(mloc, true, red, tid);   // its barriers publish sc
  float lloc = 0.f;
  for (int j = c0 + tid; j < c1; j += kDecThreads) {
    const float pj = __builtin_amdgcn_exp2f(sc[j - c0] - m);
    sc[j - c0] = pj;
    lloc += pj;
  }
  const float l = dec_block_reduce(lloc, false, red, tid);   // its barriers publish sc

  // O_s = sum_j p_j v_j / l over the lane's chunk of the rows it owns.
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = c0 + g; j0 < c1; j0 += U * G) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * G;
      x[u] = j < c1 ? *reinterpret_cast<const u32x4*>(vb + (int64_t)j * ts) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * G;
      const float pj = j < c1 ? sc[j - c0] : 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc[2 * w] = __builtin_fmaf(pj, half_to_float<F16>((uint16_t)(x[u][w] & 0xffff)), acc[2 * w]);
        acc[2 * w + 1] = __builtin_fmaf(pj, half_to_float<F16>((uint16_t)(x[u][w] >> 16)), acc[2 * w + 1]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) ored[g * D + 8 * c + e] = acc[e];
  __syncthreads();
  const int64_t part = (int64_t)bh * p.splits + split;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  for (int e = tid; e < D; e += kDecThreads) {
    float sum = 0.f;
#pragma unroll 4
    for (int gg = 0; gg < G; ++gg) sum += ored[gg * D + e];
    p.part_o[part * D + e] = sum * inv;
  }
  if (tid == 0) p.part_l[part] = l > 0.f ? m + __builtin_amdgcn_logf(l) : kNegInf;
}

template <int D, bool F16>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64)))
void decode_merge_kernel(DecodeParams p) {
  const int bh = blockIdx.x;
  const int lane = threadIdx.x;
  const float* pl = p.part_l + (int64_t)bh * p.splits;
  float lmax = kNegInf;
  for (int s = 0; s < p.splits; ++s) lmax = fmaxf(lmax, pl[s]);
  float wsum = 0.f;
  float acc[D / 64 > 0 ? D / 64 : 1] = {};
  constexpr int PER = D / 64 > 0 ? D / 64 : 1;   // elements per lane (d >= 64)
  for (int s = 0; s < p.splits; ++s) {
    if (pl[s] == kNegInf) continue;
    const float w = __builtin_amdgcn_exp2f(pl[s] - lmax);
    wsum += w;
    const float* po = p.part_o + ((int64_t)bh * p.splits + s) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      if (e < D) acc[i] = __builtin_fmaf(w, po[e], acc[i]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    if (e < D) {
      const uint32_t h2 = pack2<F16>(acc[i] * inv, 0.f);
      p.o[(int64_t)bh * D + e] = (uint16_t)(h2 & 0xffff);
    }
  }
  if (lane == 0)
    p.lse[bh] = wsum > 0.f ? (lmax + __builtin_amdgcn_logf(wsum)) * kLn2 : kNegInf;
}

}  // namespace fa
