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
//     next tile's global loads are in flight while the current one is used;
//   * per tile, per wavefront: S^T = K Q^T on bf16 MFMA (fp32 accumulate),
//     online-softmax update in base 2 (running max m, running sum l, rescale
//     of the output accumulator by exp2(m_old - m_new)), then
//     O^T += V^T P^T on bf16 MFMA with P rounded to bf16;
//   * finally O = O_acc / l goes out as bf16 and L = ln2 * (m + log2 l) as fp32.
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

__device__ __forceinline__ float xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

// Key order inside LDS rows of V^T: swap bits 2 and 3 of the key index.
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

template <int D, int BC, bool CAUSAL, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdParams p) {
  static_assert(D == 32 || D == 64 || D == 128, "head dim");
  static_assert(BC % 32 == 0 && BC >= 32 && BC <= 128, "key tile");
  constexpr int KS = D + 8;            // LDS row stride of K (elements)
  constexpr int VS = BC + 8;           // LDS row stride of V^T (elements)
  constexpr int K_ELEMS = BC * KS;
  constexpr int V_ELEMS = D * VS;
  constexpr int BUF = K_ELEMS + V_ELEMS;
  constexpr int KB = BC / 32;          // 32-key blocks per tile
  constexpr int DS = D / 16;           // MFMA k-steps over d
  constexpr int DB = D / 32;           // 32-wide d blocks of O^T
  constexpr int KCH = BC * D / 8;      // 16-byte chunks in a K tile
  static_assert(KCH % kThreads == 0, "K tile split");
  constexpr int K_PER_T = KCH / kThreads;
  constexpr int NVB = (BC / 4) * (D / 8);   // 4-key x 8-d blocks in a V tile
  static_assert(NVB <= kThreads, "V tile split");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * BUF];

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
  const uint16_t* __restrict__ kg = p.k + k_off;
  const uint16_t* __restrict__ vg = p.v + k_off;
  const int64_t rs = p.row_stride;
  const float s2 = p.scale_log2;

  const int kend = CAUSAL ? min(Nk, q0 + kBR) : Nk;
  const int n_kt = (kend + BC - 1) / BC;

  // ---- Q rows of this lane, kept in VGPRs ----
  const int qw0 = q0 + wave * 32;        // first query row of this wavefront
  const int qrow = qw0 + l32;            // this lane's query row
  const bool wave_has_rows = qw0 < Nq;
  bf16x8 qr[DS];
  if (qrow < Nq) {
    const u32x4* src = reinterpret_cast<const u32x4*>(qg + (int64_t)qrow * rs);
#pragma unroll
    for (int s = 0; s < DS; ++s) qr[s] = __builtin_bit_cast(bf16x8, src[2 * s + hi]);
  } else {
#pragma unroll
    for (int s = 0; s < DS; ++s) qr[s] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }

  // ---- staging registers for the next K/V tile ----
  u32x4 kreg[K_PER_T];
  u32x4 vreg[4];
  const int vkq = tid % (BC / 4);        // this thread's 4-key group of V
  const int vdc = tid / (BC / 4);        // this thread's 8-wide d chunk of V

  auto load_tile = [&](int kt) {
    const int k0 = kt * BC;
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (D / 8);
      const int col = c % (D / 8);
      const int key = k0 + row;
      kreg[i] = key < Nk ? *reinterpret_cast<const u32x4*>(kg + (int64_t)key * rs + col * 8)
                         : u32x4{0, 0, 0, 0};
    }
    if (tid < NVB) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 4 * vkq + r;
        vreg[r] = key < Nk ? *reinterpret_cast<const u32x4*>(vg + (int64_t)key * rs + vdc * 8)
                           : u32x4{0, 0, 0, 0};
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* Ks = smem + buf * BUF;
    uint16_t* Vt = Ks + K_ELEMS;
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (D / 8);
      const int col = c % (D / 8);
      *reinterpret_cast<u32x4*>(Ks + row * KS + col * 8) = kreg[i];
    }
    if (tid < NVB) {
      // 4 keys x 8 dims -> 8 rows of V^T, 4 keys (8 bytes) each.
      const int pos = vt_pos(4 * vkq);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo_e = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x05040100u);
        const uint32_t hi_e = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x05040100u);
        const uint32_t lo_o = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x07060302u);
        const uint32_t hi_o = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x07060302u);
        *reinterpret_cast<u32x2*>(Vt + (vdc * 8 + 2 * w) * VS + pos) = u32x2{lo_e, hi_e};
        *reinterpret_cast<u32x2*>(Vt + (vdc * 8 + 2 * w + 1) * VS + pos) = u32x2{lo_o, hi_o};
      }
    }
  };

  // ---- running state (one query row per lane) ----
  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b] = f32x16{};
  float m_run = kNegInf;   // running max, base-2 units of the scaled score
  float l_run = 0.f;       // running sum over this lane's half of the keys

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const bool more = kt + 1 < n_kt;
    if (more) load_tile(kt + 1);
    const int k0 = kt * BC;
    const bool active = wave_has_rows && (!CAUSAL || k0 <= qw0 + 31);
    if (active) {
      const uint16_t* Ks = smem + (kt & 1) * BUF;
      const uint16_t* Vt = Ks + K_ELEMS;

      // S^T = K Q^T for BC keys x 32 queries.
      f32x16 s[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        s[kb] = f32x16{};
        const uint16_t* krow = Ks + (32 * kb + l32) * KS + 8 * hi;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 16 * ds);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr[ds], s[kb], 0, 0, 0);
        }
      }

      // Online softmax, base 2.
      const bool need_mask = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > qw0);
      float mt = kNegInf;
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool ok = key < Nk && (!CAUSAL || key <= qrow);
            const float t = s[kb][r] * s2;
            s[kb][r] = ok ? t : kNegInf;
            mt = fmaxf(mt, s[kb][r]);
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
        }
        mt *= s2;
      }
      mt = fmaxf(mt, xor32(mt));
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float rsum = 0.f;
      bf16x8 pb[KB][2];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = need_mask ? s[kb][r] - m_new : __builtin_fmaf(s[kb][r], s2, -m_new);
          const float e = __builtin_amdgcn_exp2f(x);
          rsum += e;
          pb[kb][r >> 3][r & 7] = (__bf16)e;
        }
      }
      l_run = l_run * alpha + rsum;
      m_run = m_new;
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] *= alpha;

      // O^T += V^T P^T.
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const uint16_t* vrow = Vt + (32 * b + l32) * VS + 8 * hi;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + 32 * kb + 16 * t);
            o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][t], o[b], 0, 0, 0);
          }
        }
      }
    }
    if (more) store_tile((kt + 1) & 1);
    __syncthreads();
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
        for (int j = 0; j < 4; ++j) w[j] = (__bf16)(o[b][4 * g + j] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * b + 8 * g + 4 * hi) = w;
      }
    }
    if (hi == 0) p.lse[l_off + qrow] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

}  // namespace fa
