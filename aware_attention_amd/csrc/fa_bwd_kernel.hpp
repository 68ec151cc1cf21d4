// FlashAttention-2 backward for gfx950 (CDNA4): device code.
//
// The backward recomputes the scores S and the probabilities P from the
// saved log-sum-exp L instead of storing P ("FlashAttention/zh" (marovi.ai
// wiki), section 反向傳遞與重計算): P_ij = exp(scale q_i.k_j - L_i). With the
// incoming gradient dO, the chain rule through the softmax gives
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   D_i = dO_i . O_i,
//   dQ = scale dS K,   dK = scale dS^T Q.
// Three kernels, run in this order on one stream:
//   * delta_kernel: D_i = sum_e dO_ie O_ie in fp32, d/8 lanes per row;
//   * dkdv_kernel:  one workgroup per 128 keys of one (batch or sequence,
//     head); each lane owns one key, with its K and V rows in registers;
//     64-query tiles of Q and dO stream through LDS. Per tile: S = Q K^T and
//     dP = dO V^T on the matrix cores (keys in the accumulator columns), P and
//     dS in registers, then dV^T += dO^T P and dK^T += Q^T dS, whose A
//     operands are transposing LDS reads of the same Q and dO tiles. At
//     d = 256 two workgroups share a key tile, each accumulating dK and dV
//     for one half of the head dimension (S and dP over the full d);
//   * dq_kernel:    one workgroup per 128 queries; each lane owns one query
//     (Q and dO rows in registers, L and D lane-local); 64-key tiles of K and
//     V stream through LDS. Per tile: S^T = K Q^T and dP^T = V dO^T, dS^T in
//     registers, then dQ^T += K^T dS^T (A operand: transposing reads of K).
//     Up to d = 128 its state fits 256 registers, so two workgroups share a
//     CU (two waves per SIMD: one wave's exponentials overlap the other's
//     products); the dK/dV kernel does the same where it fits (kDkdvWaves).
//     Where a kernel runs one wave per SIMD, its LDS operands are read
//     several products ahead through a register ring.
// dQ is produced by its own pass over the keys (S and dP recomputed once more)
// instead of by atomic adds, so the library needs no accumulation buffer.
// The translation unit is compiled with MFMA results in the arch VGPRs
// (-amdgpu-mfma-vgpr-form): in the AGPR form the one-wave-per-SIMD dK/dV
// loop moved its accumulators between register files every tile.
//
// Operand layouts are those of the forward (v_mfma_f32_32x32x16, wave64):
// accumulator lane l, register r holds D[8(r/4) + 4(l/32) + r%4][l%32], and
// registers 8t..8t+7 of a 32-row block, packed to 16 bits, are the B operand
// of a 16-row k-step whose A operand comes from ds_read_b64_tr_b16 at rows
// {0..3, 8..11} + 4(l/32) of that step (the same permutation on both sides).
// LDS tiles are row-major with rows padded by 16 bytes.
#pragma once

#include "fa_fwd_kernel.hpp"

namespace fa {

// Tensors of the backward, in the order of BwdParams::st.
enum BwdTensor { kTQ, kTK, kTV, kTO, kTdO, kTdQ, kTdK, kTdV, kBwdTensors };

// Strides of one tensor in elements (the head dimension is contiguous):
// batch (dense only), token (the packed row index when varlen), head. Every
// stride is a multiple of 8 (16-byte aligned rows) and token strides are at
// most 2^24, which keeps the per-lane 32-bit byte offsets of a 64-row tile in
// range.
struct BwdStrides {
  int64_t b, t, h;
};

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;            // natural-log L from the forward
  float* delta;                // D, laid out like lse
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const int32_t* cu_seqlens;   // varlen only
  BwdStrides st[kBwdTensors];  // q, k, v, o, dout, dq, dk, dv
  int64_t lse_batch_stride;    // dense: H * Nq; varlen: 0
  int64_t lse_head_stride;     // dense: Nq; varlen: total
  int32_t Nq;                  // dense only
  int32_t Nk;                  // dense only
  int32_t H;
  int32_t nbatch;              // B or num_seqs
  int32_t n_tiles;             // 128-row tiles per unit in this launch
  float scale;                 // softmax scale
  float scale_log2;            // scale * log2(e)
  // Banded mask (BAND instances): query i sees key j iff
  // i + band_off - win_left <= j <= i + band_off + win_right.
  int32_t win_left, win_right, band_off;
  // Key padding mask (KPM instances, dense): token n of batch b is valid iff
  // kpm[b * kpm_batch_stride + n] != 0.
  const uint8_t* kpm;
  int64_t kpm_batch_stride;
  // Local window + global anchors (LOCAL instances, dense, Nq == Nk): tokens
  // [0, n_global) are anchors, the rest a row-major map of map_w tokens per
  // row; query i sees key j iff i or j is an anchor or their map positions
  // differ by at most loc_rows rows and loc_cols columns (sizes clamped to
  // the map's extent by the host).
  int32_t n_global, map_w, loc_rows, loc_cols;
};

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBwdRows = 32 * kBwdWaves;   // rows a workgroup owns
constexpr int kBwdTile = 64;               // rows of a streamed LDS tile
// Bytes of padding after each row of a streamed LDS tile: 16, and 32 at
// d = 256, where the wider padding spreads the transposing reads over the
// banks (measured at d = 256: +5 % on the backward; at d = 128 it changed
// nothing but cost the dQ kernel a small spill).
template <int D>
constexpr int kRowPad = D == 256 ? 32 : 16;
constexpr int kReadAhead = 4;              // LDS operand reads in flight ahead of the products (dQ)
constexpr float kLog2eF = 1.44269504088896340736f;
// Waves per SIMD of the dK/dV kernel: two workgroups share a CU (two waves
// per SIMD, so one wave's exponentials overlap the other's products) where
// the per-lane state fits in 256 registers without spilling: d = 32, and
// d = 64 except the local pattern. At d = 128 and 256 one wave holds its K,
// V rows and both accumulators in up to 512 registers.
template <int D, bool LOCAL>
constexpr int kDkdvWaves = (D == 32 || (D == 64 && !LOCAL)) ? 2 : 1;
// LDS operand reads the dK/dV kernel keeps in flight ahead of its products
// where it runs one wave per SIMD (nothing else there hides the LDS latency
// of each product's operand); 0: each read next to its product, where a
// second wave on the SIMD covers it and the registers are needed. Unmasked
// attention takes a deeper ring than the masked kinds, whose mask arithmetic
// needs the registers (measured at d = 128: 12 vs 8 is +5.5 % unmasked and
// -4 to -7 % causal or banded).
template <int D, bool LOCAL, bool MASKED>
constexpr int kDkdvRing = kDkdvWaves<D, LOCAL> == 1 ? (MASKED ? 8 : 12) : 0;

template <bool F16>
__device__ __forceinline__ float half_to_float(uint16_t b) {
  if constexpr (F16) return (float)__builtin_bit_cast(_Float16, b);
  else return __uint_as_float((uint32_t)b << 16);
}

// D_i = dO_i . O_i, fp32, for every row (token, head) of the launch, rows
// numbered in the contiguous layout's memory order, row = token * H + head,
// with token = b * N + n (dense) or the packed index (varlen: one batch of
// N = total rows); nrows < 2^31. A row of d values is read by D/8 consecutive
// lanes, 16 bytes each, so a wave's loads cover whole rows (coalesced, and
// consecutive rows are adjacent in memory for contiguous tensors); the lanes'
// partial sums meet in a butterfly of lane exchanges. O and dO are addressed
// through their own (batch, token, head) strides.
constexpr int kDeltaThreads = 256;

template <int D, bool F16>
__global__ __attribute__((amdgpu_flat_work_group_size(kDeltaThreads, kDeltaThreads)))
void delta_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                  float* __restrict__ delta, int H, int N, int nrows, BwdStrides so,
                  BwdStrides sd) {
  constexpr int L = D / 8;                    // lanes per row
  constexpr int R = kDeltaThreads / L;        // rows per workgroup
  const int row = (int)blockIdx.x * R + (int)threadIdx.x / L;   // token * H + head
  const int c = threadIdx.x % L;
  const uint32_t token = (uint32_t)row / (uint32_t)H;
  const int h = row - (int)token * H;
  const uint32_t b = token / (uint32_t)N;
  const int n = (int)(token - b * (uint32_t)N);
  float acc = 0.f;
  if (row < nrows) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(o + b * so.b + n * so.t + h * so.h + 8 * c);
    const u32x4 y = *reinterpret_cast<const u32x4*>(dout + b * sd.b + n * sd.t + h * sd.h + 8 * c);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = __builtin_fmaf(half_to_float<F16>((uint16_t)(x[w] & 0xffff)),
                           half_to_float<F16>((uint16_t)(y[w] & 0xffff)), acc);
      acc = __builtin_fmaf(half_to_float<F16>((uint16_t)(x[w] >> 16)),
                           half_to_float<F16>((uint16_t)(y[w] >> 16)), acc);
    }
  }
#pragma unroll
  for (int m = 1; m < L; m *= 2) acc += __shfl_xor(acc, m);
  if (row < nrows && c == 0) delta[((int64_t)b * H + h) * N + n] = acc;
}

// Row-major LDS tile of kBwdTile rows, each padded to 2 D + kRowPad<D>
// bytes, i.e. SL = D/8 + kRowPad<D>/16 slots of 16 bytes (the slots past D/8
// are padding). The tile's
// kBwdTile * SL slots are exactly SL blocks of 64 slots, so it is filled by
// SL direct HBM -> LDS copies of 64 lanes (global_load_lds_dwordx4), split
// over the workgroup's waves: lane l of copy i fills slot 64 i + l. Rows at
// or past nvalid are filled with the last valid row: the kernels give them
// P = 0, so they contribute nothing, and no read leaves the tensor. The
// copies are asynchronous; the issuing wave waits for them (s_waitcnt)
// before the barrier that publishes the tile.
template <int D>
__device__ __forceinline__ void copy_tile_async(uint32_t lds_tile, const uint16_t* g, int rs,
                                                int row0, int nvalid, int wave, int lane) {
  constexpr int SL = D / 8 + kRowPad<D> / 16;
  const uint8_t* base = reinterpret_cast<const uint8_t*>(g + (int64_t)row0 * rs);
  const int last = nvalid - 1 - row0;        // last valid row of the tile, >= 0
#pragma unroll
  for (int i = wave; i < SL; i += kBwdWaves) {
    const int slot = 64 * i + lane;
    const int row = slot / SL, ch = slot % SL;
    const int r = row < last ? row : last;
    const int c = ch < D / 8 ? ch : 0;        // padding slots re-read chunk 0
    copy16_to_lds(base, (uint32_t)(r * 2 * rs + 16 * c), lds_tile + 1024 * i);
  }
}

// Operand access of one lane into a padded tile (see the file comment).
template <int D>
struct BwdLanes {
  static constexpr int RBP = 2 * D + kRowPad<D>;
  int row_rd;        // row-major A fragment: row l%32, 16 bytes at chunk 2 ds + l/32
  int tr_rd[D / 32]; // transposed A fragment of 32-column block b
  __device__ BwdLanes(int lane) {
    const int l32 = lane & 31, hi = lane >> 5, vg16 = lane >> 4, vi = lane & 15;
    row_rd = l32 * RBP + hi * 16;
    const int v_row = 4 * hi + (vi >> 2);
#pragma unroll
    for (int b = 0; b < D / 32; ++b) tr_rd[b] = v_row * RBP + (32 * b + 16 * (vg16 & 1) + 4 * (vi & 3)) * 2;
  }
};

__device__ __forceinline__ bf16x8 lds16(const uint8_t* smem, int byte) {
  return *reinterpret_cast<const bf16x8*>(smem + byte);
}
__device__ __forceinline__ bf16x8 lds_tr8(const uint8_t* smem, int byte, int byte_up) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)((__attribute__((address_space(3))) uint8_t*)smem + byte));
  const v4i16 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)((__attribute__((address_space(3))) uint8_t*)smem + byte_up));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Map position of token t in the local pattern (tokens [0, G) are anchors,
// the rest a row-major map of W tokens per row): row and column, or the row
// kKeyAnchor for an anchor and kKeyPast for a token at or past N. Two
// positions are near iff their rows differ by at most wr and their columns by
// at most wc; the sentinels are never near anything (|sentinel| >= 2^30 and
// map rows, wr < 2^28).
constexpr int kKeyAnchor = -(1 << 30);
constexpr int kKeyPast = 1 << 30;
__device__ __forceinline__ void map_pos(int t, int G, int W, int N, int& r, int& c) {
  r = kKeyPast;
  c = 0;
  if (t < G) {
    r = kKeyAnchor;
  } else if (t < N) {
    r = (t - G) / W;
    c = (t - G) - r * W;
  }
}
__device__ __forceinline__ bool map_near(int r1, int c1, int r2, int c2, int wr, int wc) {
  return ((uint32_t)(r1 - r2 + wr) <= (uint32_t)(2 * wr)) &
         ((uint32_t)(c1 - c2 + wc) <= (uint32_t)(2 * wc));
}

// A lane's 32 keys of a 64-key tile are the 4-key groups 8 g + 4 (l/32) + 0..3
// (g = 0..7); given the tile's 64 validity bits (a ballot), gather the
// lane's bits so that key 32 kb + 8 (r/4) + 4 (l/32) + r%4 of register r in
// block kb lands at bit 16 kb + r (scalar code, once per tile).
__device__ __forceinline__ uint32_t gather_lane_bits(uint64_t kbits, int hi) {
  auto gather = [](uint64_t x) -> uint32_t {   // nibble 2n of x -> nibble n
    x &= 0x0F0F0F0F0F0F0F0Full;
    x = (x | (x >> 4)) & 0x00FF00FF00FF00FFull;
    x = (x | (x >> 8)) & 0x0000FFFF0000FFFFull;
    return (uint32_t)(x | (x >> 16));
  };
  const uint32_t even = gather(kbits), odd = gather(kbits >> 4);
  return hi ? odd : even;
}

// Work item of a workgroup: (128-row tile, head, batch or sequence) with the
// tile index taken from bid / units (bid: the workgroup's index in the grid,
// without the d-half bit of the d = 256 dK/dV launch). seq is the batch index (dense) or
// the sequence's first packed row (varlen); off(t) is the offset of tensor
// t's first row of the unit, for that head.
template <bool VARLEN>
struct BwdUnit {
  int tile, head, bidx, seq, Nq, Nk;
  int64_t l_off;
  __device__ __forceinline__ int64_t off(const BwdParams& p, int t) const {
    return (int64_t)seq * (VARLEN ? p.st[t].t : p.st[t].b) + (int64_t)head * p.st[t].h;
  }
};

template <bool VARLEN>
__device__ __forceinline__ BwdUnit<VARLEN> bwd_unit(const BwdParams& p, int bid) {
  BwdUnit<VARLEN> u;
  const int per = p.H * p.nbatch;
  u.tile = bid / per;
  const int rem = bid - u.tile * per;
  u.head = rem % p.H;
  u.bidx = rem / p.H;
  if constexpr (VARLEN) {
    const int start = p.cu_seqlens[u.bidx];
    const int len = p.cu_seqlens[u.bidx + 1] - start;
    u.seq = start;
    u.Nq = len;
    u.Nk = len;
    u.l_off = (int64_t)u.head * p.lse_head_stride + start;
  } else {
    u.seq = u.bidx;
    u.Nq = p.Nq;
    u.Nk = p.Nk;
    u.l_off = (int64_t)u.bidx * p.lse_batch_stride + (int64_t)u.head * p.lse_head_stride;
  }
  return u;
}

// Store a 32-row x D block held transposed in accumulators (lane = row,
// registers = columns 32 b + 8 g + 4 (l/32) + 0..3), times `mul`.
template <int D, bool F16>
__device__ __forceinline__ void store_rowT(uint16_t* row, const f32x16 (&acc)[D / 32], float mul,
                                           int hi) {
#pragma unroll
  for (int b = 0; b < D / 32; ++b) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint2 w = {pack2<F16>(acc[b][4 * g] * mul, acc[b][4 * g + 1] * mul),
                       pack2<F16>(acc[b][4 * g + 2] * mul, acc[b][4 * g + 3] * mul)};
      *reinterpret_cast<uint2*>(row + 32 * b + 8 * g + 4 * hi) = w;
    }
  }
}

// Span of the valid tokens of one row of a key padding mask: lo and hi are the
// first and last valid positions (lo > hi when the row has none), run says
// that every position in [lo, hi] is valid. One pass over the row by the
// whole workgroup; red is LDS for 3 ints per wave, free until the barrier
// at the end.
struct KpmSpan {
  int lo, hi;
  bool run;
};
__device__ __forceinline__ KpmSpan kpm_span(const uint8_t* row, int n, int* red, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  int lo = n, hi = -1, cnt = 0;
  for (int i = tid; i < n; i += kBwdThreads) {
    if (row[i] != 0) {
      lo = min(lo, i);
      hi = max(hi, i);
      ++cnt;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    lo = min(lo, __shfl_xor(lo, off, 64));
    hi = max(hi, __shfl_xor(hi, off, 64));
    cnt += __shfl_xor(cnt, off, 64);
  }
  if (lane == 0) {
    red[3 * wave] = lo;
    red[3 * wave + 1] = hi;
    red[3 * wave + 2] = cnt;
  }
  __syncthreads();
  lo = n;
  hi = -1;
  cnt = 0;
#pragma unroll
  for (int w = 0; w < kBwdWaves; ++w) {
    lo = min(lo, red[3 * w]);
    hi = max(hi, red[3 * w + 1]);
    cnt += red[3 * w + 2];
  }
  __syncthreads();   // red may be overwritten after this
  return {lo, hi, cnt == hi - lo + 1};
}

template <int D, bool CAUSAL, bool VARLEN, bool F16, bool BAND = false, bool KPM = false,
          bool LOCAL = false>
__global__ __attribute__((amdgpu_flat_work_group_size(kBwdThreads, kBwdThreads),
                          amdgpu_waves_per_eu(kDkdvWaves<D, LOCAL>, kDkdvWaves<D, LOCAL>)))
void dkdv_kernel(BwdParams p) {
  static_assert(!(KPM && (BAND || VARLEN)) && !(CAUSAL && BAND), "mask combination");
  static_assert(!(LOCAL && (BAND || KPM || VARLEN)), "mask combination");
  constexpr int DS = D / 16, DB = D / 32;
  constexpr int RBP = 2 * D + kRowPad<D>;
  constexpr int TB = kBwdTile * RBP;
  // [Q 0][dO 0][Q 1][dO 1][L 0][D 0][L 1][D 1]: buffer b holds the visited
  // query tiles b, b + 2, ...; L (times log2 e) and D per query of the tile.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TB + 4 * kBwdTile * 4];
  // Local pattern: map row and column of each query of the tile in buffer b.
  __shared__ __attribute__((aligned(16))) int qmap[LOCAL ? 4 * kBwdTile : 4];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  // Causal: key tiles in ascending order see the most queries first.
  // d = 256: each workgroup accumulates dK and dV for one half of the head
  // dimension (columns 128 half ..; blockIdx.x = 2 bid + half) and
  // recomputes S and dP over the full d; otherwise all of it (half = 0).
  constexpr int DV = D == 256 ? 128 : D;   // dK/dV columns of a workgroup
  constexpr int DBV = DV / 32;
  const int half = D == 256 ? (int)(blockIdx.x & 1) : 0;
  const BwdUnit<VARLEN> u = bwd_unit<VARLEN>(p, D == 256 ? (int)(blockIdx.x >> 1) : (int)blockIdx.x);
  const int k0 = u.tile * kBwdRows;
  if (k0 >= u.Nk) return;
  const uint16_t* const gq = p.q + u.off(p, kTQ);
  const uint16_t* const gdo = p.dout + u.off(p, kTdO);
  const int rs_q = (int)p.st[kTQ].t, rs_do = (int)p.st[kTdO].t;
  const int kw0 = k0 + wave * 32;
  const int krow = kw0 + l32;

  bf16x8 kr[DS], vr[DS];
  if (krow < u.Nk) {
    const u32x4* ks = reinterpret_cast<const u32x4*>(p.k + u.off(p, kTK) + krow * p.st[kTK].t);
    const u32x4* vs = reinterpret_cast<const u32x4*>(p.v + u.off(p, kTV) + krow * p.st[kTV].t);
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      kr[s] = __builtin_bit_cast(bf16x8, ks[2 * s + hi]);
      vr[s] = __builtin_bit_cast(bf16x8, vs[2 * s + hi]);
    }
  } else {
#pragma unroll
    for (int s = 0; s < DS; ++s) kr[s] = vr[s] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }
  const BwdLanes<D> ln(lane);
  f32x16 dk[DBV], dv[DBV];
#pragma unroll
  for (int b = 0; b < DBV; ++b) dk[b] = dv[b] = f32x16{};

  int n_qt = (u.Nq + kBwdTile - 1) / kBwdTile;
  int qt0 = CAUSAL ? k0 / kBwdTile : 0;
  // Band: the queries that see some key of this workgroup, i in
  // [k0 - band_hi, k0 + kBwdRows - 1 - band_lo].
  const int band_lo = BAND ? p.band_off - p.win_left : 0;
  const int band_hi = BAND ? p.band_off + p.win_right : 0;
  if constexpr (BAND) {
    const int q_lo = max(0, k0 - band_hi);
    const int q_hi = min(u.Nq - 1, min(u.Nk, k0 + kBwdRows) - 1 - band_lo);
    qt0 = q_lo / kBwdTile;
    n_qt = q_hi >= q_lo ? q_hi / kBwdTile + 1 : qt0;
  }
  // Padding mask: this lane's key takes part only if it is a valid token;
  // padding queries get L = +inf below, so their P is 0. Query tiles outside
  // the span of valid tokens hold only padding and are skipped; a workgroup
  // (or a wave) whose keys all lie outside it only writes zeros.
  const uint8_t* kpm_row = KPM ? p.kpm + (int64_t)u.bidx * p.kpm_batch_stride : nullptr;
  const bool k_valid = !KPM || (krow < u.Nk && kpm_row[krow] != 0);
  KpmSpan span{0, u.Nk - 1, true};
  if constexpr (KPM) {
    span = kpm_span(kpm_row, u.Nk, reinterpret_cast<int*>(smem), tid);   // no tile copied yet
    if (span.lo > span.hi || k0 > span.hi || k0 + kBwdRows - 1 < span.lo) {
      n_qt = qt0;
    } else {
      qt0 = max(qt0, span.lo / kBwdTile);
      n_qt = min(n_qt, span.hi / kBwdTile + 1);
    }
  }
  const bool wave_has = kw0 < u.Nk && (!KPM || (kw0 <= span.hi && kw0 + 31 >= span.lo));
  // Visited query tiles: [0, A) then [W0, W1) (without the local pattern A = 0,
  // [W0, W1) = [qt0, n_qt)). Local pattern: an anchor key is seen by every
  // query; a map key by the anchor queries (not when causal: they precede it)
  // and by the map queries within loc_rows rows. A wave skips a tile in which
  // none of its keys is seen.
  int A = 0, W0 = qt0, W1 = n_qt;
  const int G = p.n_global, MW = p.map_w, WR = p.loc_rows, WC = p.loc_cols;
  int kmr = 0, kmc = 0;                 // this lane's key on the map
  bool wave_anchor = false;             // the wave holds an anchor key
  int wqlo = 0, wqhi = u.Nq - 1;        // queries that see the wave's map keys
  if constexpr (LOCAL) {
    map_pos(krow, G, MW, u.Nk, kmr, kmc);
    const int k1 = min(u.Nk, k0 + kBwdRows);
    if (k0 >= G) {
      const int r_lo = (k0 - G) / MW, r_hi = (k1 - 1 - G) / MW;
      int qlo = G + max(0, r_lo - WR) * MW;
      const int qhi = min(u.Nq, G + (r_hi + WR + 1) * MW) - 1;
      if (CAUSAL) qlo = max(qlo, k0);
      A = CAUSAL ? 0 : min((G + kBwdTile - 1) / kBwdTile, n_qt);
      W0 = max(A, qlo / kBwdTile);
      W1 = max(W0, qhi / kBwdTile + 1);
    }
    wave_anchor = kw0 < G;
    if (wave_has && !wave_anchor) {
      const int kw1 = min(u.Nk, kw0 + 32) - 1;
      const int r_lo = (kw0 - G) / MW, r_hi = (kw1 - G) / MW;
      wqlo = G + max(0, r_lo - WR) * MW;
      wqhi = min(u.Nq, G + (r_hi + WR + 1) * MW) - 1;
    }
  }
  const int n_iter = A + max(0, W1 - W0);
  auto tile_of = [&](int it) { return it < A ? it : W0 + (it - A); };
  // Copies of query tile qt into buffer b, and its L, D values into registers
  // (threads 0..63, one query each; padding queries get L = +inf, D = 0).
  // The loads are unconditional (index clamped into the row) and their values
  // are used only in store_ld, after the tile's compute: a wait for them any
  // earlier would also wait for the tile copies issued before them.
  auto issue = [&](int qt, int b) __attribute__((always_inline)) {
    copy_tile_async<D>(smem_lds + (2 * b) * TB, gq, rs_q, qt * kBwdTile, u.Nq, wave, lane);
    copy_tile_async<D>(smem_lds + (2 * b + 1) * TB, gdo, rs_do, qt * kBwdTile, u.Nq, wave, lane);
  };
  struct Ld {
    float l, d;
    uint8_t valid;   // padding mask byte (KPM)
  };
  auto load_ld = [&](int qt, Ld& x) __attribute__((always_inline)) {
    const int qc = min(qt * kBwdTile + tid, u.Nq - 1);
    x.l = p.lse[u.l_off + qc];
    x.d = p.delta[u.l_off + qc];
    x.valid = KPM ? kpm_row[qc] : 1;
  };
  auto store_ld = [&](int b, int qt, const Ld& x) __attribute__((always_inline)) {
    const int qi = qt * kBwdTile + tid;
    // The empty asm takes the loaded values here, so that the arithmetic on
    // them (and the wait for the loads) is not hoisted up to the loads.
    float lraw = x.l, draw = x.d;
    uint32_t vraw = x.valid;
    asm volatile("" : "+v"(lraw), "+v"(draw), "+v"(vraw));
    const bool qv = qi < u.Nq && vraw != 0;
    float* ld = reinterpret_cast<float*>(smem + 4 * TB) + b * 2 * kBwdTile;
    ld[tid] = qv ? lraw * kLog2eF : __builtin_inff();
    ld[kBwdTile + tid] = qi < u.Nq ? draw : 0.f;
    if constexpr (LOCAL) {
      int r, c;
      map_pos(qt * kBwdTile + tid, G, MW, u.Nq, r, c);
      qmap[b * 2 * kBwdTile + tid] = r;
      qmap[b * 2 * kBwdTile + kBwdTile + tid] = c;
    }
  };
  if (n_iter > 0) {
    issue(tile_of(0), 0);
    if (tid < kBwdTile) {
      Ld x;
      load_ld(tile_of(0), x);
      store_ld(0, tile_of(0), x);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < n_iter; ++it) {
    const int qt = tile_of(it);
    const int qb0 = qt * kBwdTile;
    const int buf = it & 1;
    const bool more = it + 1 < n_iter;
    const int qt_next = more ? tile_of(it + 1) : 0;
    Ld nx{0.f, 0.f, 0};
    if (more) {   // the other buffer was last read before the previous barrier
      issue(qt_next, buf ^ 1);
      if (tid < kBwdTile) load_ld(qt_next, nx);
    }
    const uint8_t* q_lds = smem + (2 * buf) * TB;
    const uint8_t* do_lds = smem + (2 * buf + 1) * TB;
    const float* l_lds = reinterpret_cast<const float*>(smem + 4 * TB) + buf * 2 * kBwdTile;
    const float* d_lds = l_lds + kBwdTile;
    bool useful = wave_has && !(CAUSAL && qb0 + kBwdTile - 1 < kw0);
    if constexpr (LOCAL)
      useful = useful && (wave_anchor || (!CAUSAL && qb0 < G) ||
                          (qb0 + kBwdTile - 1 >= wqlo && qb0 <= wqhi));
    if (useful) {

    // S = Q K^T and dP = dO V^T: 64 queries x this wave's 32 keys.
    constexpr int RING = kDkdvRing<D, LOCAL, CAUSAL || BAND || KPM || LOCAL>;
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
    // L and D of the 4 queries of each (qb, t, half) group this lane needs
    // (read here, ahead of the products, when the ring is on).
    float4 L4s[8], D4s[8];
    auto ld_group = [&](int g) __attribute__((always_inline)) {
      const int q4 = 8 * g + 4 * hi;   // g = 4 qb + 2 t + half: 32 qb + 16 t + 8 half
      L4s[g] = *reinterpret_cast<const float4*>(l_lds + q4);
      D4s[g] = *reinterpret_cast<const float4*>(d_lds + q4);
    };
    if constexpr (RING > 0) {
      // Step st = 4 ds + 2 qb + (0: S from Q, 1: dP from dO); the operands
      // go through a ring of RING registers, each read issued that many
      // products ahead (sched_barrier keeps reads and products in order and
      // lets only ALU work cross).
      constexpr int NS = 4 * DS;
      auto rd = [&](int st) __attribute__((always_inline)) {
        return lds16((st & 1) ? do_lds : q_lds, ((st >> 1) & 1) * 32 * RBP + ln.row_rd + (st >> 2) * 32);
      };
      bf16x8 ra[RING];
#pragma unroll
      for (int st = 0; st < RING; ++st) ra[st] = rd(st);
#pragma unroll
      for (int g = 0; g < 8; ++g) ld_group(g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const bf16x8 a = ra[st % RING];
        if (st + RING < NS) ra[st % RING] = rd(st + RING);
        const int ds = st >> 2, qb = (st >> 1) & 1;
        if (st & 1) dp[qb] = mfma32<F16>(a, vr[ds], dp[qb]);
        else s[qb] = mfma32<F16>(a, kr[ds], s[qb]);
        __builtin_amdgcn_sched_barrier(0x7);
      }
    } else {
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int off = qb * 32 * RBP + ln.row_rd + ds * 32;
          s[qb] = mfma32<F16>(lds16(q_lds, off), kr[ds], s[qb]);
          dp[qb] = mfma32<F16>(lds16(do_lds, off), vr[ds], dp[qb]);
        }
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS: step st = 2 (DBV (2 qb + t) + b) +
    // (0: dV from dO, 1: dK from Q), A operands by transposing reads of the
    // workgroup's columns. With the ring on, its first reads are issued here,
    // so that their latency hides behind the exponentials below.
    constexpr int NP = 8 * DBV;
    constexpr int RING2 = RING > 0 ? RING : 1;
    auto rd2 = [&](int st) __attribute__((always_inline)) {
      const int which = st & 1, b = (st >> 1) % DBV, c = (st >> 1) / DBV;   // c = 2 qb + t
      const int r0 = 16 * c * RBP, tr = ln.tr_rd[b + DBV * half];
      return lds_tr8(which ? q_lds : do_lds, r0 + tr, r0 + 8 * RBP + tr);
    };
    bf16x8 rb[RING2];
    if constexpr (RING > 0) {
#pragma unroll
      for (int st = 0; st < RING; ++st) rb[st] = rd2(st);
      __builtin_amdgcn_sched_barrier(0);
    }
    // P = exp2(scale log2e S - L log2e) and dS = P (dP - D), packed as B
    // operands; masked: with the per-pair mask test, which tiles where every
    // (query, key) pair of the wave is visible skip (below the diagonal,
    // inside the band, all of the wave's keys valid; padding queries have
    // L = +inf, queries past the end a copy of the last row and L = +inf).
    bf16x8 pb[2][2], dsb[2][2];
    auto pds = [&](auto masked_tag) __attribute__((always_inline)) {
    constexpr bool masked = decltype(masked_tag)::value;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 wp, wd;
#pragma unroll
        for (int half = 0; half < 2; ++half) {   // registers 8t + 4 half + 0..3
          const int g = 4 * qb + 2 * t + half;
          const int q4 = 8 * g + 4 * hi;      // first of 4 queries
          if constexpr (RING == 0) ld_group(g);
          const float4 L4 = L4s[g], D4 = D4s[g];
          const float Lv[4] = {L4.x, L4.y, L4.z, L4.w}, Dv[4] = {D4.x, D4.y, D4.z, D4.w};
          i32x4 qmr = {0, 0, 0, 0}, qmc = {0, 0, 0, 0};
          if constexpr (LOCAL) {
            qmr = *reinterpret_cast<const i32x4*>(&qmap[buf * 2 * kBwdTile + q4]);
            qmc = *reinterpret_cast<const i32x4*>(&qmap[buf * 2 * kBwdTile + kBwdTile + q4]);
          }
          float pv[4], dsv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 8 * t + 4 * half + e;
            const int qi = qb0 + q4 + e;
            bool ok = true;
            if constexpr (masked) {
              ok = (!CAUSAL || krow <= qi) && k_valid;
              if constexpr (BAND) ok = ok && krow >= qi + band_lo && krow <= qi + band_hi;
              if constexpr (LOCAL)
                ok = ok & (map_near(qmr[e], qmc[e], kmr, kmc, WR, WC) | (qmr[e] == kKeyAnchor) |
                           (kmr == kKeyAnchor));
            }
            const float pe = ok ? __builtin_amdgcn_exp2f(s[qb][r] * p.scale_log2 - Lv[e]) : 0.f;
            pv[e] = pe;
            dsv[e] = pe * (dp[qb][r] - Dv[e]);
          }
          wp[2 * half] = pack2<F16>(pv[0], pv[1]);
          wp[2 * half + 1] = pack2<F16>(pv[2], pv[3]);
          wd[2 * half] = pack2<F16>(dsv[0], dsv[1]);
          wd[2 * half + 1] = pack2<F16>(dsv[2], dsv[3]);
        }
        pb[qb][t] = __builtin_bit_cast(bf16x8, wp);
        dsb[qb][t] = __builtin_bit_cast(bf16x8, wd);
      }
    }
    };
    // (Causal tiles keep the test: at d = 128 the two instantiations cost the
    // causal dK/dV loop more than the test itself, prefill shapes -2 to -3 %.)
    bool full = !CAUSAL;
    if constexpr (BAND) full = kw0 >= qb0 + kBwdTile - 1 + band_lo && kw0 + 31 <= qb0 + band_hi;
    if constexpr (KPM) full = full && __builtin_amdgcn_ballot_w64(k_valid) == ~0ull;
    if constexpr (LOCAL) full = false;
    if (full) pds(std::false_type{});
    else pds(std::true_type{});
    if constexpr (RING > 0) {
#pragma unroll
      for (int st = 0; st < NP; ++st) {
        const bf16x8 a = rb[st % RING];
        if (st + RING < NP) rb[st % RING] = rd2(st + RING);
        const int b = (st >> 1) % DBV, c = (st >> 1) / DBV, qb = c >> 1, t = c & 1;
        if (st & 1) dk[b] = mfma32<F16>(a, dsb[qb][t], dk[b]);
        else dv[b] = mfma32<F16>(a, pb[qb][t], dv[b]);
        __builtin_amdgcn_sched_barrier(0x7);
      }
    } else {
#pragma unroll
      for (int st = 0; st < NP; ++st) {
        const int b = (st >> 1) % DBV, c = (st >> 1) / DBV, qb = c >> 1, t = c & 1;
        if (st & 1) dk[b] = mfma32<F16>(rd2(st), dsb[qb][t], dk[b]);
        else dv[b] = mfma32<F16>(rd2(st), pb[qb][t], dv[b]);
      }
    }
    }
    if (more && tid < kBwdTile) store_ld(buf ^ 1, qt_next, nx);
    stress_pause(it);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of the next tile have landed
    __syncthreads();
  }
  if (krow < u.Nk) {
    store_rowT<DV, F16>(p.dk + u.off(p, kTdK) + krow * p.st[kTdK].t + DV * half, dk, p.scale, hi);
    store_rowT<DV, F16>(p.dv + u.off(p, kTdV) + krow * p.st[kTdV].t + DV * half, dv, 1.f, hi);
  }
}

template <int D, bool CAUSAL, bool VARLEN, bool F16, bool BAND = false, bool KPM = false,
          bool LOCAL = false>
__global__ __attribute__((amdgpu_flat_work_group_size(kBwdThreads, kBwdThreads),
                          amdgpu_waves_per_eu(D == 256 ? 1 : 2, D == 256 ? 1 : 2)))
void dq_kernel(BwdParams p) {
  static_assert(!(KPM && (BAND || VARLEN)) && !(CAUSAL && BAND), "mask combination");
  static_assert(!(LOCAL && (BAND || KPM || VARLEN)), "mask combination");
  constexpr int DS = D / 16, DB = D / 32;
  constexpr int RBP = 2 * D + kRowPad<D>;
  constexpr int TB = kBwdTile * RBP;
  // [K 0][V 0][K 1][V 1]: buffer b holds the visited key tiles b, b + 2, ...
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TB];
  // Local pattern: map row and column of each key of the tile in buffer b.
  __shared__ __attribute__((aligned(16))) int kmap[LOCAL ? 4 * kBwdTile : 4];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  BwdUnit<VARLEN> u = bwd_unit<VARLEN>(p, (int)blockIdx.x);
  if (CAUSAL) u.tile = p.n_tiles - 1 - u.tile;   // longest rows first
  const int q0 = u.tile * kBwdRows;
  if (q0 >= u.Nq) return;
  const uint16_t* const gk = p.k + u.off(p, kTK);
  const uint16_t* const gv = p.v + u.off(p, kTV);
  const int rs_k = (int)p.st[kTK].t, rs_v = (int)p.st[kTV].t;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;

  bf16x8 qr[DS], dor[DS];
  float Lq = 0.f, Dq = 0.f;
  if (qrow < u.Nq) {
    const u32x4* qs = reinterpret_cast<const u32x4*>(p.q + u.off(p, kTQ) + qrow * p.st[kTQ].t);
    const u32x4* os = reinterpret_cast<const u32x4*>(p.dout + u.off(p, kTdO) + qrow * p.st[kTdO].t);
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      qr[s] = __builtin_bit_cast(bf16x8, qs[2 * s + hi]);
      dor[s] = __builtin_bit_cast(bf16x8, os[2 * s + hi]);
    }
    // A padding query (padding mask) gets L = +inf, so its P and dQ are 0.
    const bool qv = !KPM || p.kpm[(int64_t)u.bidx * p.kpm_batch_stride + qrow] != 0;
    Lq = qv ? p.lse[u.l_off + qrow] * kLog2eF : __builtin_inff();
    Dq = p.delta[u.l_off + qrow];
  } else {
#pragma unroll
    for (int s = 0; s < DS; ++s) qr[s] = dor[s] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }
  const BwdLanes<D> ln(lane);
  f32x16 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = f32x16{};

  const int kend = CAUSAL ? min(u.Nk, q0 + kBwdRows) : u.Nk;
  const int n_kt = (kend + kBwdTile - 1) / kBwdTile;
  // Key tiles [kt_begin, kt_stop) hold a key some row of the workgroup sees.
  int kt_begin = 0, kt_stop = n_kt;
  const int band_lo = BAND ? p.band_off - p.win_left : 0;
  const int band_hi = BAND ? p.band_off + p.win_right : 0;
  if constexpr (BAND) {
    const int k_lo = max(0, q0 + band_lo);
    const int k_hi = min(u.Nk - 1, min(u.Nq, q0 + kBwdRows) - 1 + band_hi);
    kt_begin = k_lo / kBwdTile;
    kt_stop = k_hi >= k_lo ? k_hi / kBwdTile + 1 : kt_begin;
  }
  // Padding mask: key tiles outside the span of valid tokens hold only
  // padding and are skipped; a workgroup (or a wave) whose queries all lie
  // outside it only writes zeros. Inside the span, a key's validity comes from
  // the span itself when the valid tokens form one run, else from the mask.
  const uint8_t* kpm_row = KPM ? p.kpm + (int64_t)u.bidx * p.kpm_batch_stride : nullptr;
  KpmSpan span{0, u.Nk - 1, true};
  if constexpr (KPM) {
    span = kpm_span(kpm_row, u.Nk, reinterpret_cast<int*>(smem), tid);   // no tile copied yet
    if (span.lo > span.hi || q0 > span.hi || q0 + kBwdRows - 1 < span.lo) {
      kt_stop = kt_begin;
    } else {
      kt_begin = max(kt_begin, span.lo / kBwdTile);
      kt_stop = min(kt_stop, span.hi / kBwdTile + 1);
    }
  }
  const bool wave_has = qw0 < u.Nq && (!KPM || (qw0 <= span.hi && qw0 + 31 >= span.lo));
  const int wave_last_kt = CAUSAL ? (qw0 + 31) / kBwdTile : n_kt - 1;
  // Visited key tiles: [0, A) then [W0, W1) (without the local pattern A = 0,
  // [W0, W1) = [kt_begin, kt_stop)). Local pattern: an anchor query sees every
  // key; a map query sees the anchor keys and the map keys within loc_rows
  // rows. A wave skips a tile in which none of its queries sees a key.
  int A = 0, W0 = kt_begin, W1 = kt_stop;
  const int G = p.n_global, MW = p.map_w, WR = p.loc_rows, WC = p.loc_cols;
  int qmr = 0, qmc = 0;                 // this lane's query on the map
  bool wave_anchor = false;             // the wave holds an anchor query
  int wklo = 0, wkhi = u.Nk - 1;        // keys the wave's map queries see on the map
  if constexpr (LOCAL) {
    map_pos(qrow, G, MW, u.Nq, qmr, qmc);
    if (q0 >= G) {
      const int q1 = min(u.Nq, q0 + kBwdRows);
      const int r_lo = (q0 - G) / MW, r_hi = (q1 - 1 - G) / MW;
      const int klo = G + max(0, r_lo - WR) * MW;
      const int khi = min(kend, G + (r_hi + WR + 1) * MW) - 1;
      A = min((G + kBwdTile - 1) / kBwdTile, n_kt);
      W0 = max(A, klo / kBwdTile);
      W1 = max(W0, khi / kBwdTile + 1);
    }
    wave_anchor = qw0 < G;
    if (wave_has && !wave_anchor) {
      const int qw1 = min(u.Nq, qw0 + 32) - 1;
      const int r_lo = (qw0 - G) / MW, r_hi = (qw1 - G) / MW;
      wklo = G + max(0, r_lo - WR) * MW;
      wkhi = min(u.Nk, G + (r_hi + WR + 1) * MW) - 1;
    }
  }
  const int n_iter = A + max(0, W1 - W0);
  auto tile_of = [&](int it) { return it < A ? it : W0 + (it - A); };
  auto issue = [&](int kt, int b) __attribute__((always_inline)) {
    copy_tile_async<D>(smem_lds + (2 * b) * TB, gk, rs_k, kt * kBwdTile, u.Nk, wave, lane);
    copy_tile_async<D>(smem_lds + (2 * b + 1) * TB, gv, rs_v, kt * kBwdTile, u.Nk, wave,
                       lane);
    if constexpr (LOCAL) {
      if (tid < kBwdTile) {
        int r, c;
        map_pos(kt * kBwdTile + tid, G, MW, u.Nk, r, c);
        kmap[b * 2 * kBwdTile + tid] = r;
        kmap[b * 2 * kBwdTile + kBwdTile + tid] = c;
      }
    }
  };
  if (n_iter > 0) issue(tile_of(0), 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < n_iter; ++it) {
    const int kt = tile_of(it);
    const int kb0 = kt * kBwdTile;
    const int buf = it & 1;
    if (it + 1 < n_iter) issue(tile_of(it + 1), buf ^ 1);   // buffer last read before the previous barrier
    const uint8_t* k_lds = smem + (2 * buf) * TB;
    const uint8_t* v_lds = smem + (2 * buf + 1) * TB;
    bool useful = wave_has && kt <= wave_last_kt;
    if constexpr (LOCAL)
      useful = useful && (wave_anchor || kb0 < G || (kb0 + kBwdTile - 1 >= wklo && kb0 <= wkhi));
    if (useful) {
    uint32_t kvalid = ~0u;   // padding mask: validity bits of this lane's 32 keys
    if constexpr (KPM) {
      const int key = kb0 + lane;
      const bool kv = span.run ? (key >= span.lo && key <= span.hi) : (key < u.Nk && kpm_row[key] != 0);
      kvalid = gather_lane_bits(__builtin_amdgcn_ballot_w64(kv), hi);
    }

    // S^T = K Q^T and dP^T = V dO^T: this tile's 64 keys x the wave's 32
    // queries. With one wave per SIMD nothing else hides the LDS latency:
    // operands go through a ring of kReadAhead registers, each read issued
    // that many products ahead of its use (sched_barrier keeps reads and
    // products in order and lets only ALU work cross). Step
    // st = 4 ds + 2 kb + (0: S from K, 1: dP from V).
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
    {
      constexpr int NS = 4 * DS;
      auto rd = [&](int st) {
        return lds16((st & 1) ? v_lds : k_lds, ((st >> 1) & 1) * 32 * RBP + ln.row_rd + (st >> 2) * 32);
      };
      bf16x8 ra[kReadAhead];
#pragma unroll
      for (int st = 0; st < kReadAhead; ++st) ra[st] = rd(st);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const bf16x8 a = ra[st % kReadAhead];
        if (st + kReadAhead < NS) ra[st % kReadAhead] = rd(st + kReadAhead);
        const int ds = st >> 2, kb = (st >> 1) & 1;
        if (st & 1) dp[kb] = mfma32<F16>(a, dor[ds], dp[kb]);
        else s[kb] = mfma32<F16>(a, qr[ds], s[kb]);
        __builtin_amdgcn_sched_barrier(0x7);
      }
    }
    // dS^T = P^T (dP^T - D), packed as B operands; masked: with the
    // per-pair mask test, which tiles where every (query, key) pair of the
    // wave is visible skip (no key past the end, below the diagonal, inside
    // the band, all keys valid).
    bf16x8 dsb[2][2];
    auto pds = [&](auto masked_tag) __attribute__((always_inline)) {
    constexpr bool masked = decltype(masked_tag)::value;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v2[2];
          // Map positions of this pair's keys (key index 4 (r/4)-aligned group).
          const int kk = 32 * kb + 8 * ((8 * t + 2 * i) >> 2) + 4 * hi;
          i32x4 kmr = {0, 0, 0, 0}, kmc = {0, 0, 0, 0};
          if constexpr (LOCAL && masked) {
            kmr = *reinterpret_cast<const i32x4*>(&kmap[buf * 2 * kBwdTile + kk]);
            kmc = *reinterpret_cast<const i32x4*>(&kmap[buf * 2 * kBwdTile + kBwdTile + kk]);
          }
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int r = 8 * t + 2 * i + e;
            const int key = kb0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
            bool ok = true;
            if constexpr (masked) {
              ok = key < u.Nk && (!CAUSAL || key <= qrow);
              if constexpr (BAND) ok = ok && key >= qrow + band_lo && key <= qrow + band_hi;
              if constexpr (KPM) ok = ok && ((kvalid >> (16 * kb + r)) & 1);
              if constexpr (LOCAL) {
                const int j = r & 3;   // position of the key in its group of 4
                ok = ok & (map_near(qmr, qmc, kmr[j], kmc[j], WR, WC) | (qmr == kKeyAnchor) |
                           (kmr[j] == kKeyAnchor));
              }
            }
            const float pe = ok ? __builtin_amdgcn_exp2f(s[kb][r] * p.scale_log2 - Lq) : 0.f;
            v2[e] = pe * (dp[kb][r] - Dq);
          }
          w[i] = pack2<F16>(v2[0], v2[1]);
        }
        dsb[kb][t] = __builtin_bit_cast(bf16x8, w);
      }
    }
    };
    bool full = kb0 + kBwdTile <= u.Nk;
    if constexpr (CAUSAL) full = full && kb0 + kBwdTile - 1 <= qw0;
    if constexpr (BAND)
      full = full && kb0 >= qw0 + 31 + band_lo && kb0 + kBwdTile - 1 <= qw0 + band_hi;
    if constexpr (KPM) full = full && __builtin_amdgcn_ballot_w64(kvalid != ~0u) == 0;
    if constexpr (LOCAL) full = false;
    if (full) pds(std::false_type{});
    else pds(std::true_type{});
    // dQ^T += K^T dS^T, with the same read-ahead (step st = g DB + b, g = 2 kb + t).
    {
      constexpr int NP = 4 * DB;
      auto rd = [&](int st) {
        const int g = st / DB, b = st % DB;
        const int r0 = (32 * (g >> 1) + 16 * (g & 1)) * RBP;
        return lds_tr8(k_lds, r0 + ln.tr_rd[b], r0 + 8 * RBP + ln.tr_rd[b]);
      };
      bf16x8 ra[kReadAhead];
#pragma unroll
      for (int st = 0; st < kReadAhead; ++st) ra[st] = rd(st);
#pragma unroll
      for (int st = 0; st < NP; ++st) {
        const bf16x8 a = ra[st % kReadAhead];
        if (st + kReadAhead < NP) ra[st % kReadAhead] = rd(st + kReadAhead);
        const int g = st / DB;
        acc[st % DB] = mfma32<F16>(a, dsb[g >> 1][g & 1], acc[st % DB]);
        __builtin_amdgcn_sched_barrier(0x7);
      }
    }
    }
    stress_pause(it);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of the next tile have landed
    __syncthreads();
  }
  if (qrow < u.Nq)
    store_rowT<D, F16>(p.dq + u.off(p, kTdQ) + qrow * p.st[kTdQ].t, acc, p.scale, hi);
}

}  // namespace fa
