// FP8 (MX block-scaled) attention forward for gfx950, head dimension 128,
// and the quantisers that produce its operands: device code.
//
// What is computed is the attention of "FlashAttention/zh" (marovi.ai wiki),
// section FlashAttention 算法, on block-scaled FP8 operands, the
// low-precision variant of section 變體與後續版本 (FP8 with block scaling;
// section 局限性 notes that such formats need careful scaling). The block
// format is OCP MX: 32 consecutive elements share a power-of-two E8M0 scale,
// elements are FP8 E4M3 (fn). gfx950's scaled matrix instruction
// v_mfma_scale_f32_32x32x64_f8f6f4 consumes that format directly: per lane
// 32 FP8 values and one E8M0 scale byte, 64-deep contraction. Its lane layout
// (checked on the device): lane (row m = l % 32, h = l / 32) holds k = 16 h + i
// in bytes i < 16 and k = 32 + 16 h + (i - 16) in bytes i >= 16, and supplies
// the scale of row m's block h (k in [32 h, 32 h + 32)). The accumulator
// layout is that of the 32x32 bf16 instruction.
//
// Operands and layouts (D = 128):
//   Q, K: (B, N, H, D) E4M3 codes, exponents (B, N, H, D/32): blocks along d,
//         the contraction of S = Q K^T;
//   V^T:  (B, H, D, Np) E4M3 codes, the tokens padded with zeros to Np, a
//         multiple of 64; exponents (B, H, Np/32, D): blocks of 32 tokens,
//         the contraction of P V, laid out token-block-major so that one
//         64-key tile's exponents are 2 D contiguous bytes;
//   O:    (B, Nq, H, D) bf16, L (B, H, Nq) fp32, as fa_fwd.
//
// The kernel keeps fwd_kernel's schedule (256-row query tiles, two wave
// groups in ping-pong with one barrier per 64-key tile, direct HBM -> LDS
// copies double-buffered, transposed products with one query per lane, the
// base-2 online softmax with the deferred rescale). Per tile and wave: S^T =
// K Q^T in 4 scaled MFMAs (2 key blocks x 2 d halves), P~ rounded to E4M3
// with scale 1 (P~ <= 2^8 < 448), O^T += V^T P^T in 4 scaled MFMAs (4 d
// blocks). P~ leaves the S^T accumulators with lane half h holding keys
// 8 g + 4 h + 0..3 of each 32-key block; one v_permlane32_swap per register
// pair regroups them into the instruction's order (lane half h: keys
// 16 h + 0..15 and 32 + 16 h + 0..15). The row sums stay fp32.
#pragma once

#include "fa_fwd_kernel.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kMxD = 128;                 // head dimension of the FP8 kernel
constexpr int kMxTokenPad = 64;           // token padding of V^T
constexpr int kMxBlock = 32;              // elements per E8M0 scale

struct Mx8Params {
  const uint8_t* q;      // (B, Nq, H, D) E4M3
  const uint8_t* qe;     // (B, Nq, H, D/32) E8M0
  const uint8_t* k;      // (B, Nk, H, D)
  const uint8_t* ke;     // (B, Nk, H, D/32)
  const uint8_t* vt;     // (B, H, D, Np)
  const uint8_t* vte;    // (B, H, Np/32, D)
  uint16_t* o;           // (B, Nq, H, D) bf16
  float* lse;            // (B, H, Nq)
  int32_t Nq, Nk, Np, H, nbatch, n_qtiles;
  float scale_log2;      // |softmax_scale| * log2(e)
  uint32_t q_sign;       // 0, or 0x80808080 for a negative scale (sign moved into Q)
};

// D += A B on the scaled 32x32x64 FP8 matrix instruction; SA/SB select the
// byte of the scale registers.
template <int SA, int SB>
__device__ __forceinline__ f32x16 mfma_mx8(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SA, sa, SB, sb);
}

// One 4-byte-per-lane HBM -> LDS copy (global_load_lds_dword), addressed like
// copy16_to_lds: lane l's 4 bytes from gbase + voff land at LDS lds_base + 4 l.
__device__ __forceinline__ void copy4_to_lds(const void* gbase, uint32_t voff, uint32_t lds_base) {
  const uint64_t b = reinterpret_cast<uint64_t>(gbase);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(voff), "s"(bs), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory", "m0");
}

// Swap the upper half of a with the lower half of b (v_permlane32_swap).
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

template <bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2)))
void fwd_mx8_kernel(Mx8Params p) {
  constexpr int D = kMxD;
  constexpr int BC = kBC;                    // keys per tile
  constexpr int KB = BC / 32;                // 32-key blocks per tile
  constexpr int DT = D / 64;                 // 64-deep steps over d
  constexpr int DB = D / 32;                 // 32-wide d blocks of O^T
  constexpr int KT = BC * D;                 // K tile bytes (64 rows of 128)
  constexpr int VT = D * BC;                 // V^T tile bytes (128 rows of 64)
  constexpr int KS = BC * (D / kMxBlock);    // K exponents of a tile
  constexpr int VS = (BC / kMxBlock) * D;    // V exponents of a tile
  constexpr int K0 = 0, V0 = 2 * KT, KS0 = 2 * KT + 2 * VT, VS0 = KS0 + 2 * KS;
  // Double-buffered tiles; the epilogue reuses the first kWaves * 32 * 2D
  // bytes to transpose O (store_tileT).
  constexpr int SMEM = 2 * (KT + VT + KS + VS) > kWaves * 64 * D ? 2 * (KT + VT + KS + VS)
                                                                : kWaves * 64 * D;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bool group_b = wave >= 4;
  const int gw = wave & 3;

  // ---- work item (fwd_kernel's order): causal longest tiles first, else
  // query tiles of a few (batch, head) units per XCD at a time ----
  const int units = p.H * p.nbatch;
  int qt, rem;
  if (!CAUSAL && (units & 7) == 0) {
    const int m = blockIdx.x >> 3;
    qt = m % p.n_qtiles;
    rem = (blockIdx.x & 7) + 8 * (m / p.n_qtiles);
  } else {
    qt = blockIdx.x / units;
    rem = blockIdx.x - qt * units;
  }
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;
  const int head = rem % p.H;
  const int bidx = rem / p.H;
  const int Nq = p.Nq, Nk = p.Nk;
  const int q0 = qt * kBR;
  if (q0 >= Nq) return;

  const int64_t tok = (int64_t)p.H * D;                 // token stride of Q, K (bytes)
  const int64_t tok_e = (int64_t)p.H * (D / kMxBlock);  // ... of their exponents
  const uint8_t* __restrict__ qg = p.q + (int64_t)bidx * Nq * tok + (int64_t)head * D;
  const uint8_t* __restrict__ qeg = p.qe + (int64_t)bidx * Nq * tok_e + (int64_t)head * (D / kMxBlock);
  const uint8_t* __restrict__ kg = p.k + (int64_t)bidx * Nk * tok + (int64_t)head * D;
  const uint8_t* __restrict__ keg = p.ke + (int64_t)bidx * Nk * tok_e + (int64_t)head * (D / kMxBlock);
  const int64_t unit = (int64_t)bidx * p.H + head;
  const uint8_t* __restrict__ vtg = p.vt + unit * D * p.Np;
  const uint8_t* __restrict__ vteg = p.vte + unit * (p.Np / kMxBlock) * D;
  const float s2 = p.scale_log2;

  const int kend = CAUSAL ? min(Nk, q0 + kBR) : Nk;
  const int n_kt = (kend + BC - 1) / BC;

  // ---- Q rows of this lane and their exponents ----
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  const bool wave_has_rows = qw0 < Nq;
  i32x8 qr[DT];
  uint32_t qsc = 0;
  if (qrow < Nq) {
    const u32x4* src = reinterpret_cast<const u32x4*>(qg + (int64_t)qrow * tok);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const u32x4 a = src[4 * t + hi], b = src[4 * t + 2 + hi];
      qr[t] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    }
    qsc = *reinterpret_cast<const uint32_t*>(qeg + (int64_t)qrow * tok_e) >> (8 * hi);
  } else {
#pragma unroll
    for (int t = 0; t < DT; ++t) qr[t] = i32x8{};
  }
  if (p.q_sign) {   // negative scale: scale q.k = |scale| (-q).k
#pragma unroll
    for (int t = 0; t < DT; ++t) qr[t] ^= (int)p.q_sign;
  }

  // ---- direct HBM -> LDS copies by the waves of group A ----
  // K tile: 512 16-byte slots, row s / 8, physical chunk s % 8 holding logical
  // chunk (s % 8) ^ ((row >> 1) & 7). V^T tile: 512 slots, row (d) s / 4,
  // physical chunk s % 4 holding logical chunk (s % 4) ^ ((row >> 2) & 3).
  // Both swizzles make the operand reads (16 rows x one chunk) conflict free.
  int k_row[2], k_src[2], v_src[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int slot = (gw * 2 + n) * 64 + lane;
    const int kr = slot / 8, kc = slot % 8;
    k_row[n] = kr;
    k_src[n] = kr * (int)tok + ((kc ^ ((kr >> 1) & 7)) * 16);
    const int vr = slot / 4, vc = slot % 4;
    v_src[n] = vr * p.Np + ((vc ^ ((vr >> 2) & 3)) * 16);
  }
  auto copy_k = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kt * BC;
    const int buf = kt & 1;
    const uint8_t* g = kg + (int64_t)k0 * tok;
    const uint32_t lds0 = smem_lds + K0 + buf * KT + gw * 2 * 1024;
    if (k0 + BC <= Nk) {
#pragma unroll
      for (int n = 0; n < 2; ++n) copy16_to_lds(g, (uint32_t)k_src[n], lds0 + n * 1024);
    } else {
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        if (k0 + k_row[n] < Nk)
          copy16_to_lds(g, (uint32_t)k_src[n], lds0 + n * 1024);
        else
          *reinterpret_cast<u32x4*>(smem + K0 + buf * KT + (gw * 2 + n) * 1024 + 16 * lane) =
              u32x4{0, 0, 0, 0};
      }
    }
    if (gw == 0) {   // the tile's K exponents: 4 bytes per key
      const uint32_t ldsx = smem_lds + KS0 + buf * KS;
      if (k0 + lane < Nk)
        copy4_to_lds(keg, (uint32_t)((k0 + lane) * (int)tok_e), ldsx);
      else
        *reinterpret_cast<uint32_t*>(smem + KS0 + buf * KS + 4 * lane) = 0u;
    }
  };
  auto copy_v = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kt * BC;
    const int buf = kt & 1;
    const uint8_t* g = vtg + k0;   // V^T rows are padded: always inside the tensor
    const uint32_t lds0 = smem_lds + V0 + buf * VT + gw * 2 * 1024;
#pragma unroll
    for (int n = 0; n < 2; ++n) copy16_to_lds(g, (uint32_t)v_src[n], lds0 + n * 1024);
    if (gw == 1 && lane < VS / 16)   // the tile's V exponents: 2 D contiguous bytes
      copy16_to_lds(vteg + (int64_t)(k0 / kMxBlock) * D, (uint32_t)(16 * lane),
                    smem_lds + VS0 + buf * VS);
  };

  // ---- LDS operand addresses of this lane ----
  int k_rd[DT][2];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      k_rd[t][j] = l32 * D + (((4 * t + 2 * j + hi) ^ ((l32 >> 1) & 7)) * 16);
  int v_rd[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) v_rd[j] = l32 * BC + (((2 * j + hi) ^ ((l32 >> 2) & 3)) * 16);

  auto lds16 = [&](int byte) __attribute__((always_inline)) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(smem + byte);
  };
  auto frag = [&](int b0, int b1) __attribute__((always_inline)) -> i32x8 {
    const u32x4 a = lds16(b0), b = lds16(b1);
    return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
  };

  // ---- running state ----
  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b] = f32x16{};
  float m_run = kNegInf;
  float l_run = 0.f;
  f32x16 s[KB];
  i32x8 pb = {};                 // P~ of the previous tile, E4M3, as the B operand
  constexpr int kPScale = 127;   // E8M0 1.0

  // M phase: S^T of tile kt (4 MFMAs) and/or O^T += V^T P^T of tile kt-1
  // (4 MFMAs), operands read from LDS four MFMAs ahead. QK and PV are
  // compile-time flags so that every register index is static.
  auto qk_pv = [&](auto qk_tag, auto pv_tag, int kt) __attribute__((always_inline)) {
    constexpr bool QK = decltype(qk_tag)::value, PV = decltype(pv_tag)::value;
    const int kb_ = K0 + (kt & 1) * KT;
    const int vb_ = V0 + ((kt - 1) & 1) * VT;
    uint32_t ksc[KB] = {};
    if constexpr (QK) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        ksc[kb] = *reinterpret_cast<const uint32_t*>(smem + KS0 + (kt & 1) * KS + 4 * (32 * kb + l32)) >> (8 * hi);
    }
    int vsc[DB] = {};
    if constexpr (PV) {
#pragma unroll
      for (int b = 0; b < DB; ++b) vsc[b] = smem[VS0 + ((kt - 1) & 1) * VS + hi * D + 32 * b + l32];
    }
    constexpr int NQ = DT * KB, NP = DB;
    constexpr int FIRST = QK ? 0 : NQ, LAST = PV ? NQ + NP : NQ, R = 4;
    // Fragment f: QK steps (t = f / KB, kb = f % KB) first, then PV steps (b = f - NQ).
    auto load = [&](int f) __attribute__((always_inline)) -> i32x8 {
      if (f < NQ) {
        const int t = f / KB, kb = f % KB;
        return frag(kb_ + 32 * kb * D + k_rd[t][0], kb_ + 32 * kb * D + k_rd[t][1]);
      }
      const int b = f - NQ;
      return frag(vb_ + 32 * b * BC + v_rd[0], vb_ + 32 * b * BC + v_rd[1]);
    };
    i32x8 ring[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (FIRST + i < LAST) ring[i] = load(FIRST + i);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (QK) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = FIRST; f < LAST; ++f) {
      const int slot = (f - FIRST) % R;
      if (f < NQ) {
        const int t = f / KB, kb = f % KB;
        if (t == 0)
          s[kb] = mfma_mx8<0, 0>(ring[slot], qr[0], s[kb], (int)ksc[kb], (int)qsc);
        else
          s[kb] = mfma_mx8<2, 2>(ring[slot], qr[1], s[kb], (int)ksc[kb], (int)qsc);
      } else {
        const int b = f - NQ;
        o[b] = mfma_mx8<0, 0>(ring[slot], pb, o[b], vsc[b], kPScale);
      }
      if (f + R < LAST) ring[slot] = load(f + R);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto mfma_phase = [&](bool do_qk, bool do_pv, int kt) __attribute__((always_inline)) {
    if (do_qk && do_pv) qk_pv(std::true_type{}, std::true_type{}, kt);
    else if (do_qk) qk_pv(std::true_type{}, std::false_type{}, kt);
    else if (do_pv) qk_pv(std::false_type{}, std::true_type{}, kt);
  };

  // P~ = exp2(x - m) of one tile, rounded to E4M3 and regrouped across the
  // lane halves into the B operand pb; returns this lane's sum of P~ (x =
  // S^T scale_log2, or the already scaled, masked s).
  auto exps = [&](auto masked_tag, float neg_m) __attribute__((always_inline)) -> float {
    constexpr bool masked = decltype(masked_tag)::value;
    float sum = 0.f;
    uint32_t w[KB][4];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * g + j;
          e[j] = __builtin_amdgcn_exp2f(masked ? s[kb][r] + neg_m : __builtin_fmaf(s[kb][r], s2, neg_m));
        }
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
        x = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], x, true);
        w[kb][g] = (uint32_t)x;
        sum += (e[0] + e[1]) + (e[2] + e[3]);
      }
      // lane half h then holds keys 16 h + 0..15 of the block, in order
      swap32(w[kb][0], w[kb][2]);
      swap32(w[kb][1], w[kb][3]);
    }
    pb = i32x8{(int)w[0][0], (int)w[0][2], (int)w[0][1], (int)w[0][3],
               (int)w[1][0], (int)w[1][2], (int)w[1][1], (int)w[1][3]};
    return sum;
  };

  // Online softmax of one tile (fwd_kernel's, with P~ rounded to E4M3 and
  // regrouped across the lane halves for the B operand).
  auto softmax_tile = [&](auto masked_tag, int k0) __attribute__((always_inline)) {
    constexpr bool masked = decltype(masked_tag)::value;
    float mt = kNegInf;
    if constexpr (masked) {
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
        for (int r = 0; r < 16; r += 2) mt = max3(mt, s[kb][r], s[kb][r + 1]);
      }
      mt *= s2;
    }
    mt = max_xor32(mt);
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleTau) != 0) {
      asm volatile("" ::: "memory");   // a real branch, taken rarely
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] *= alpha;
      m_run = m_new;
    }
    l_run += exps(masked_tag, -m_run);
  };

  // Softmax of a full unmasked tile in the steady loop, without the row
  // maximum (fwd_kernel's): exponentials against the current offset first;
  // the lane's sum of P~ bounds each of its terms, so only a sum above
  // 2^kRescaleTau (or not a number) makes the wave take the maximum, the
  // rescale and the exponentials again. P~ <= 2^kRescaleTau stays below
  // E4M3's largest finite value either way.
  auto softmax_lazy = [&]() __attribute__((always_inline)) {
    // A wave whose rows have no offset yet (their first tile) goes straight
    // to the full path.
    float tsum = 0.f;
    bool full = true;
    if (__builtin_amdgcn_ballot_w64(m_run == kNegInf) == 0) {
      tsum = exps(std::false_type{}, -m_run);
      full = __builtin_amdgcn_ballot_w64(!(tsum <= (float)(1 << (int)kRescaleTau))) != 0;
    }
    if (full) {
      asm volatile("" : "+v"(m_run) : : "memory");   // a real branch; no reuse of the above
      float mt = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) mt = max3(mt, s[kb][r], s[kb][r + 1]);
      }
      mt = max_xor32(mt * s2);
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] *= alpha;
      m_run = m_new;
      tsum = exps(std::false_type{}, -m_run);
    }
    l_run += tsum;
  };
  auto softmax = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kt * BC;
    if ((k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > qw0))
      softmax_tile(std::true_type{}, k0);
    else
      softmax_tile(std::false_type{}, k0);
  };
  auto active = [&](int kt) __attribute__((always_inline)) {
    return wave_has_rows && (!CAUSAL || kt <= min(n_kt - 1, (qw0 + 31) / BC));
  };

  // ---- schedule: fwd_kernel's periods (group A copies K(j+1), V(j) and
  // runs M_j then the softmax of tile j; group B the softmax of tile j-1
  // then M_j; one barrier per period) ----
  auto period = [&](int j) __attribute__((always_inline)) {
    const bool do_qk = j < n_kt && active(j);
    const bool do_pv = j > 0 && active(j - 1);
    stress_pause(4 * j);
    if (!group_b) {
      if (j < n_kt) {
        if (j + 1 < n_kt) copy_k(j + 1);
        copy_v(j);
      }
      mfma_phase(do_qk, do_pv, j);
      stress_pause(4 * j + 1);
      if (j < n_kt && active(j)) softmax(j);
      stress_pause(4 * j + 2);
      __builtin_amdgcn_s_waitcnt(0);
    } else {
      if (j > 0 && active(j - 1)) softmax(j - 1);
      stress_pause(4 * j + 1);
      mfma_phase(do_qk, do_pv, j);
    }
    stress_pause(4 * j + 3);
    barrier_nofence();
  };
  const int full_kt = Nk / BC;
  const int unmasked_kt = CAUSAL ? min(full_kt, q0 / BC) : full_kt;
  const int js0 = 1;
  const int js1 = (q0 + kBR <= Nq) ? max(1, min(unmasked_kt, full_kt - 1)) : 1;
  if (!group_b) copy_k(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int j = 0; j < js0; ++j) period(j);
  for (int j = js0; j < js1; ++j) {   // steady: full, unmasked, active tiles for every wave
    stress_pause(4 * j);
    if (!group_b) {
      copy_k(j + 1);
      copy_v(j);
      qk_pv(std::true_type{}, std::true_type{}, j);
      stress_pause(4 * j + 1);
      softmax_lazy();
      stress_pause(4 * j + 2);
      __builtin_amdgcn_s_waitcnt(0);
    } else {
      softmax_lazy();
      stress_pause(4 * j + 1);
      qk_pv(std::true_type{}, std::true_type{}, j);
    }
    stress_pause(4 * j + 3);
    barrier_nofence();
  }
  for (int j = js1; j <= n_kt; ++j) period(j);

  // ---- epilogue: O = O_acc / l, L = ln2 (m + log2 l) ----
  // O goes out through LDS (store_tileT), each wave using its own 32 * 2D
  // bytes, free once every wave has crossed the last barrier.
  const float l_tot = l_run + xor32(l_run);
  if (qw0 < Nq)
    store_tileT<D, false>(p.o + ((int64_t)bidx * Nq + qw0) * tok + (int64_t)head * D, tok,
                          min(32, Nq - qw0), o, __builtin_amdgcn_rcpf(l_tot),
                          smem + wave * 64 * D, lane);
  if (qrow < Nq && hi == 0)
    p.lse[((int64_t)bidx * p.H + head) * Nq + qrow] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

// ---- quantisers (HBM-bound, one thread per 32-element block) ----

// E8M0 exponent of a block with absolute maximum amax: floor(log2 amax) - 8,
// clamped to [-127, 127]; -127 for an all-zero block. A block holding an
// infinity or a NaN takes the NaN scale (byte 0xFF, exponent 128 here) and
// stores zeros, as the MX format defines.
constexpr int kMxNanExp = 128;
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.f)) return -127;
  const int e = __builtin_amdgcn_frexp_expf(amax) - 1 - 8;   // amax = m 2^(e+9), m in [0.5, 1)
  return min(127, max(-127, e));
}

// x 2^-e rounded to E4M3 (nearest even), saturated to +-448: four values per
// 32-bit word, low byte first.
__device__ __forceinline__ uint32_t mx_pack4(float a, float b, float c, float d, int e) {
  auto q = [&](float x) __attribute__((always_inline)) {
    return __builtin_amdgcn_fmed3f(__builtin_ldexpf(x, -e), -448.f, 448.f);
  };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q(a), q(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q(c), q(d), w, true);
  return (uint32_t)w;
}

// Quantise one block of 32 values into two 16-byte words of E4M3 codes;
// returns the exponent.
__device__ __forceinline__ int mx_block(const float (&v)[kMxBlock], u32x4 (&out)[2]) {
  float amax = 0.f;
  bool finite = true;
#pragma unroll
  for (int i = 0; i < kMxBlock; ++i) {
    const float a = fabsf(v[i]);
    finite = finite && (a <= 3.40282347e38f);   // false for inf and NaN
    amax = fmaxf(amax, a);
  }
  if (!finite) {
    out[0] = out[1] = u32x4{0, 0, 0, 0};
    return kMxNanExp;
  }
  const int e = mx_exponent(amax);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    out[i / 4][i % 4] = mx_pack4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3], e);
  return e;
}

template <bool F16>
__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  if constexpr (F16) return (float)__builtin_bit_cast(_Float16, h);
  else return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// Rows of 32 d-blocks: x (rows, D) 16-bit, densely packed -> codes (rows, D),
// exponents (rows, D / 32).
template <bool F16>
__global__ void mx8_quantize_rows_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ xq,
                                         uint8_t* __restrict__ xe, int64_t nblocks) {
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= nblocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + blk * kMxBlock);
  float v[kMxBlock];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 w = src[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * c + 2 * i] = half_bits_to_float<F16>((uint16_t)(w[i] & 0xffff));
      v[8 * c + 2 * i + 1] = half_bits_to_float<F16>((uint16_t)(w[i] >> 16));
    }
  }
  u32x4 out[2];
  const int e = mx_block(v, out);
  u32x4* dst = reinterpret_cast<u32x4*>(xq + blk * kMxBlock);
  dst[0] = out[0];
  dst[1] = out[1];
  xe[blk] = (uint8_t)(e + 127);
}

// V (B, N, H, D) 16-bit -> V^T codes (B, H, D, Np) and exponents
// (B, H, Np / 32, D): one thread per (batch, head, 32-token block, d); the
// tokens past N are zeros.
template <bool F16>
__global__ void mx8_quantize_vt_kernel(const uint16_t* __restrict__ v, uint8_t* __restrict__ vt,
                                       uint8_t* __restrict__ vte, int32_t B, int32_t N, int32_t H,
                                       int32_t Np) {
  constexpr int D = kMxD;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nblk = (int64_t)B * H * (Np / kMxBlock) * D;
  if (idx >= nblk) return;
  const int dd = (int)(idx % D);
  const int64_t r = idx / D;
  const int tb = (int)(r % (Np / kMxBlock));
  const int64_t bh = r / (Np / kMxBlock);
  const int h = (int)(bh % H);
  const int b = (int)(bh / H);
  float x[kMxBlock];
#pragma unroll
  for (int i = 0; i < kMxBlock; ++i) {
    const int n = tb * kMxBlock + i;
    x[i] = n < N ? half_bits_to_float<F16>(v[(((int64_t)b * N + n) * H + h) * D + dd]) : 0.f;
  }
  u32x4 out[2];
  const int e = mx_block(x, out);
  u32x4* dst = reinterpret_cast<u32x4*>(vt + (bh * D + dd) * (int64_t)Np + tb * kMxBlock);
  dst[0] = out[0];
  dst[1] = out[1];
  vte[(bh * (Np / kMxBlock) + tb) * D + dd] = (uint8_t)(e + 127);
}

}  // namespace fa
