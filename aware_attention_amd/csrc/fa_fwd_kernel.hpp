// FlashAttention-2 forward for gfx950 (CDNA4): device code.
//
// What one workgroup does ("FlashAttention/zh" (marovi.ai wiki), section
// FlashAttention 算法, with the FlashAttention-2 loop order of section
// 變體與後續版本: outer loop over query blocks spread across the grid, inner
// loop over key/value blocks inside the workgroup):
//   * owns one query tile of BR = 128 rows of one (batch or sequence, head);
//     each of its 4 wavefronts owns 32 of those rows and keeps its Q rows in
//     VGPRs for the whole kernel;
//   * streams key/value tiles of BC keys through LDS, double-buffered: the
//     global loads of later tiles are in flight while the current ones are used;
//   * per tile, per wavefront: S^T = K Q^T on bf16 MFMA (fp32 accumulate),
//     online-softmax update in base 2 (running max m, running sum l, rescale
//     of the output accumulator by exp2(m_old - m_new)), then
//     O^T += V^T P^T on bf16 MFMA with P rounded to bf16;
//   * finally O = O_acc / l goes out as bf16 and L = ln2 * (m + log2 l) as fp32.
//
// Software pipeline. Keys run one tile ahead of values: while the VALU does
// the softmax of tile j, the matrix cores already compute S^T of tile j+1, so
// the exponentials overlap MFMA work inside one wavefront. K and V have their
// own pair of LDS buffers; one barrier per tile orders the buffer reuse.
//
// Deferred rescaling. The running maximum m used as the exponent offset is
// moved only when some row's tile maximum exceeds it by more than kRescaleTau
// (base-2 units); otherwise the tile is exponentiated against the stale m, so
// P~ can reach 2^kRescaleTau. In exact arithmetic the result is unchanged:
// O = sum P~ V / sum P~ and L = m + log l are invariant to the offset. This
// removes the per-tile multiply of the whole output accumulator.
//
// Layout choices (gfx950 v_mfma_f32_32x32x16_bf16, wave64):
//   MFMA A operand: lane l holds A[m = l%32][k = 8*(l/32) .. +7];
//   MFMA B operand: lane l holds B[k = 8*(l/32) .. +7][n = l%32];
//   accumulator:   lane l, register r holds D[8*(r/4) + 4*(l/32) + r%4][l%32].
// Computing the transposed products puts one query per lane (n = l%32) in
// both S^T and O^T, so the row statistics m, l and the rescale factor are
// lane-local; the only cross-lane step per tile is one max exchange between
// lane l and lane l^32. The accumulator registers of S^T feed the B operand
// of the P V product directly, with no trip through LDS: register group
// r = 8t..8t+7 of a 32-key block holds keys 16t + {0..3, 8..11} + 4*(l/32).
// V is written to LDS transposed, with the key order inside every group of 16
// keys permuted (bits 2 and 3 of the key index swapped), so the eight keys a
// lane needs for one MFMA are contiguous: one 16-byte LDS read per operand.
//
// Masking ("FlashAttention/zh", section 變體與後續版本: causal masks):
// keys past the sequence end and, when causal, keys after the query are set
// to -inf, only on the tiles that need it; tiles entirely above a wavefront's
// diagonal are skipped, and key tiles past the workgroup's last query are
// never loaded.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* cu_seqlens;   // varlen only
  int64_t q_batch_stride;      // elements between batches of q and o (dense)
  int64_t k_batch_stride;      // elements between batches of k and v (dense)
  int64_t row_stride;          // elements between consecutive tokens: H * d
  int64_t lse_batch_stride;    // dense: H * Nq
  int64_t lse_head_stride;     // dense: Nq; varlen: total
  int32_t Nq;                  // dense only
  int32_t Nk;                  // dense only
  int32_t H;
  int32_t nbatch;              // B (dense) or num_seqs (varlen)
  int32_t n_qtiles;            // query tiles per (batch or sequence, head)
  float scale_log2;            // softmax_scale * log2(e), >= 0
};

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kRescaleTau = 8.0f;

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Key order inside LDS rows of V^T: swap bits 2 and 3 of the key index.
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// LDS tile layout shared by K and V: BC rows of D bf16 (2*D bytes), no
// padding, 16-byte chunks permuted inside each row by an XOR with a
// row-dependent mask so that the MFMA operand reads hit distinct LDS banks.
template <int D>
struct TileLayout {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = D / 8;          // 16-byte chunks per row
  // K operand reads: 16 consecutive rows, one chunk each -> 16 distinct banks.
  __device__ static constexpr int k_swz(int row) {
    return D == 128 ? (row & 15) : D == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3);
  }
  // V operand reads (transposing 8-byte reads): 4 consecutive rows x 8 chunks
  // of 8 bytes per half-wave -> 32 distinct bank pairs.
  __device__ static constexpr int v_swz(int row) {
    return D == 128 ? 4 * (row & 3) : D == 64 ? 4 * ((row >> 1) & 1) : 0;
  }
};

template <int D, int BC, bool CAUSAL, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdParams p) {
  static_assert(D == 32 || D == 64 || D == 128, "head dim");
  static_assert(BC == 64, "key tile");
  using TL = TileLayout<D>;
  constexpr int RB = TL::kRowBytes;
  constexpr int TILE_BYTES = BC * RB;            // one K or V tile
  constexpr int KB = BC / 32;                    // 32-key blocks per tile
  constexpr int DS = D / 16;                     // MFMA k-steps over d
  constexpr int DB = D / 32;                     // 32-wide d blocks of O^T
  constexpr int NPW = TILE_BYTES / 1024 / kWaves;  // 1 KiB direct loads per wave per tile
  static_assert(NPW >= 1 && TILE_BYTES % (1024 * kWaves) == 0, "tile split");

  // [K buf 0][K buf 1][V buf 0][V buf 1]
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- work item: (query tile, head, batch or sequence) ----
  const int per_qt = p.H * p.nbatch;
  int qt = blockIdx.x / per_qt;
  const int rem = blockIdx.x - qt * per_qt;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;   // longest rows of the mask first
  const int head = rem % p.H;
  const int bidx = rem / p.H;

  int Nq, Nk;
  int64_t q_off, k_off, l_off;
  if (VARLEN) {
    const int start = p.cu_seqlens[bidx];
    const int len = p.cu_seqlens[bidx + 1] - start;
    Nq = len;
    Nk = len;
    q_off = (int64_t)start * p.row_stride + (int64_t)head * D;
    k_off = q_off;
    l_off = (int64_t)head * p.lse_head_stride + start;
  } else {
    Nq = p.Nq;
    Nk = p.Nk;
    q_off = (int64_t)bidx * p.q_batch_stride + (int64_t)head * D;
    k_off = (int64_t)bidx * p.k_batch_stride + (int64_t)head * D;
    l_off = (int64_t)bidx * p.lse_batch_stride + (int64_t)head * p.lse_head_stride;
  }
  const int q0 = qt * kBR;
  if (q0 >= Nq) return;   // whole workgroup: tile past this sequence's end

  const uint16_t* __restrict__ qg = p.q + q_off;
  const uint8_t* __restrict__ kg = reinterpret_cast<const uint8_t*>(p.k + k_off);
  const uint8_t* __restrict__ vg = reinterpret_cast<const uint8_t*>(p.v + k_off);
  const int rs = (int)p.row_stride;          // elements
  const int rs_bytes = 2 * rs;
  const float s2 = p.scale_log2;

  const int kend = CAUSAL ? min(Nk, q0 + kBR) : Nk;
  const int n_kt = (kend + BC - 1) / BC;

  // ---- Q rows of this lane, kept in VGPRs ----
  const int qw0 = q0 + wave * 32;        // first query row of this wavefront
  const int qrow = qw0 + l32;            // this lane's query row
  const bool wave_has_rows = qw0 < Nq;
  // Last key tile that has a visible key for some row of this wavefront.
  const int wave_last_kt = CAUSAL ? min(n_kt - 1, (qw0 + 31) / BC) : n_kt - 1;
  bf16x8 qr[DS];
  if (qrow < Nq) {
    const u32x4* src = reinterpret_cast<const u32x4*>(qg + (int64_t)qrow * rs);
#pragma unroll
    for (int s = 0; s < DS; ++s) qr[s] = __builtin_bit_cast(bf16x8, src[2 * s + hi]);
  } else {
#pragma unroll
    for (int s = 0; s < DS; ++s) qr[s] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }

  // ---- direct HBM -> LDS copies: this lane's slot in each of the wave's loads ----
  // Slot s of a tile (16 bytes at byte 16*s) holds row s / kChunks, logical
  // chunk (s % kChunks) ^ swz(row).
  int cp_row[NPW], k_src[NPW], v_src[NPW];
#pragma unroll
  for (int n = 0; n < NPW; ++n) {
    const int slot = (wave * NPW + n) * 64 + lane;
    const int row = slot / TL::kChunks;
    const int phys = slot % TL::kChunks;
    cp_row[n] = row;
    k_src[n] = row * rs_bytes + ((phys ^ TL::k_swz(row)) * 16);
    v_src[n] = row * rs_bytes + ((phys ^ TL::v_swz(row)) * 16);
  }
  auto copy_tile = [&](const uint8_t* gsrc, const int (&src)[NPW], int tile_base, int kt) {
    const int k0 = kt * BC;
    const uint8_t* g = gsrc + (int64_t)k0 * rs_bytes;
    if (k0 + BC <= Nk) {
#pragma unroll
      for (int n = 0; n < NPW; ++n)
        __builtin_amdgcn_global_load_lds(
            (__attribute__((address_space(1))) void*)(g + src[n]),
            (__attribute__((address_space(3))) void*)(smem + tile_base + (wave * NPW + n) * 1024),
            16, 0, 0);
    } else {
#pragma unroll
      for (int n = 0; n < NPW; ++n) {
        if (k0 + cp_row[n] < Nk) {
          __builtin_amdgcn_global_load_lds(
              (__attribute__((address_space(1))) void*)(g + src[n]),
              (__attribute__((address_space(3))) void*)(smem + tile_base + (wave * NPW + n) * 1024),
              16, 0, 0);
        } else {
          *reinterpret_cast<u32x4*>(smem + tile_base + (wave * NPW + n) * 1024 + 16 * lane) =
              u32x4{0, 0, 0, 0};
        }
      }
    }
  };
  auto copy_k = [&](int kt, int buf) { copy_tile(kg, k_src, buf * TILE_BYTES, kt); };
  auto copy_v = [&](int kt, int buf) { copy_tile(vg, v_src, (2 + buf) * TILE_BYTES, kt); };

  // ---- LDS operand addresses of this lane ----
  // K operand (A of S^T = K Q^T): row 32*kb + l32, logical chunk 2*ds + hi.
  int k_rd[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) k_rd[ds] = l32 * RB + (((2 * ds + hi) ^ TL::k_swz(l32)) * 16);
  // V operand (A of O^T = V^T P^T) by transposing 8-byte reads: in each group
  // of 16 lanes, lane i reads row base + 4*hi + i/4, dims 32*b + 16*half + 4*(i%4);
  // the transpose hands lane j dims 32*b + 16*half + j of four consecutive rows.
  const int vg16 = lane >> 4, vi = lane & 15;
  const int v_row = 4 * hi + (vi >> 2);
  const int v_x = 2 * (vg16 & 1) + ((vi & 3) >> 1);
  int v_rd[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
    v_rd[b] = v_row * RB + (((4 * b + v_x) ^ TL::v_swz(v_row)) * 16) + 8 * (vi & 1);

  typedef short v4i16 __attribute__((ext_vector_type(4)));
  auto lds_b128 = [&](int byte) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(smem + byte);
  };
  auto lds_tr = [&](int byte) -> v4i16 {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)((__attribute__((address_space(3))) uint8_t*)smem + byte));
  };

  // S^T of one tile for this wavefront: BC keys x 32 queries, fp32.
  auto qk = [&](f32x16 (&s)[KB], int kbuf) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const bf16x8 a = lds_b128(kbuf * TILE_BYTES + 32 * kb * RB + k_rd[ds]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr[ds], s[kb], 0, 0, 0);
      }
    }
  };

  // ---- running state (one query row per lane) ----
  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b] = f32x16{};
  float m_run = kNegInf;   // exponent offset, base-2 units of the scaled score
  float l_run = 0.f;       // running sum over this lane's half of the keys

  // Softmax pieces. need_mask: the tile holds keys past the end or, when
  // causal, keys after some query of this wavefront.
  auto need_mask = [&](int k0) { return (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > qw0); };

  // Row maximum of the tile in base-2 units, shared by the two lanes of a row.
  // The masked form scales and masks s in place.
  auto rowmax = [&](f32x16 (&s)[KB], bool masked, int k0) {
    float mt = kNegInf;
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool ok = key < Nk && (!CAUSAL || key <= qrow);
          s[kb][r] = ok ? s[kb][r] * s2 : kNegInf;
          mt = fmaxf(mt, s[kb][r]);
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) mt = fmaxf(mt, fmaxf(s[kb][r], s[kb][r + 1]));
      }
      mt *= s2;
    }
    return fmaxf(mt, xor32(mt));
  };

  // Move the exponent offset only when some row grew by more than kRescaleTau.
  auto maybe_rescale = [&](float mt) {
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleTau) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] *= alpha;
      m_run = m_new;
    }
  };

  // P~ = exp2(scaled score - m) rounded to bf16 pairs; fp32 row sums of P~.
  auto exp_pack = [&](const f32x16 (&s)[KB], bf16x8 (&pb)[KB][2], bool prescaled) {
    const float neg_m = -m_run;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 8 * t + 2 * i;
          const float x0 = prescaled ? s[kb][r] + neg_m : __builtin_fmaf(s[kb][r], s2, neg_m);
          const float x1 = prescaled ? s[kb][r + 1] + neg_m : __builtin_fmaf(s[kb][r + 1], s2, neg_m);
          const float e0 = __builtin_amdgcn_exp2f(x0);
          const float e1 = __builtin_amdgcn_exp2f(x1);
          w[i] = pack_bf16(e0, e1);
          l_run += e0 + e1;
        }
        pb[kb][t] = __builtin_bit_cast(bf16x8, w);
      }
    }
  };

  // O^T += V^T P^T for one tile.
  auto pv = [&](const bf16x8 (&pb)[KB][2], int vbuf) {
    const int base = (2 + vbuf) * TILE_BYTES;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int r0 = (32 * kb + 16 * t) * RB;
          const v4i16 lo = lds_tr(base + r0 + v_rd[b]);
          const v4i16 up = lds_tr(base + r0 + 8 * RB + v_rd[b]);
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
          o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][t], o[b], 0, 0, 0);
        }
      }
    }
  };

  // All of this thread's direct LDS copies have landed and every thread's are
  // visible: wait for the memory counters, then the workgroup barrier.
  auto tile_sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // ---- prologue: K_0 -> Kbuf0, V_0 -> Vbuf0, K_1 -> Kbuf1, S_0 ----
  copy_k(0, 0);
  copy_v(0, 0);
  if (n_kt > 1) copy_k(1, 1);
  tile_sync();
  f32x16 s_cur[KB];
  if (wave_has_rows) qk(s_cur, 0);
  __syncthreads();   // every wave is done with Kbuf0 before it is refilled

  // ---- main loop: tile j's softmax and P V, tile j+1's S ----
  for (int j = 0; j < n_kt; ++j) {
    if (j + 2 < n_kt) copy_k(j + 2, j & 1);
    if (j + 1 < n_kt) copy_v(j + 1, (j + 1) & 1);
    const bool act_j = wave_has_rows && j <= wave_last_kt;
    const bool act_j1 = wave_has_rows && j + 1 <= wave_last_kt;
    f32x16 s_next[KB];
    bf16x8 pb[KB][2];
    const int k0 = j * BC;
    const bool masked = need_mask(k0);
    if (act_j && act_j1 && !masked) {
      // Common case, one basic block: tile j+1's QK^T on the matrix cores
      // alongside tile j's exponentials, then tile j's P V.
      maybe_rescale(rowmax(s_cur, false, k0));
      qk(s_next, (j + 1) & 1);
      exp_pack(s_cur, pb, false);
      pv(pb, j & 1);
    } else {
      if (act_j1) qk(s_next, (j + 1) & 1);
      if (act_j) {
        maybe_rescale(rowmax(s_cur, masked, k0));
        exp_pack(s_cur, pb, masked);
        pv(pb, j & 1);
      }
    }
    tile_sync();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s_cur[kb] = s_next[kb];
  }

  // ---- epilogue: O = O_acc / l, L = ln2 * (m + log2 l) ----
  const float l_tot = l_run + xor32(l_run);
  if (qrow < Nq) {
    const float inv = __builtin_amdgcn_rcpf(l_tot);
    uint16_t* orow = p.o + q_off + (int64_t)qrow * rs;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) w[jj] = (__bf16)(o[b][4 * g + jj] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * b + 8 * g + 4 * hi) = w;
      }
    }
    if (hi == 0) p.lse[l_off + qrow] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

}  // namespace fa
