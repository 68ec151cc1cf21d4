// FlashAttention-2 forward for head dimension 256 on gfx950: device code.
//
// The same computation as fwd_kernel ("FlashAttention/zh" (marovi.ai wiki),
// sections FlashAttention 算法 and 變體與後續版本; the page notes the fused
// kernel reaches head dimensions up to about 256, section 局限性), with a
// layout that fits d = 256. fwd_kernel keeps one wave's 32 Q rows (64 VGPRs
// at d = 256) and its O accumulator (128 VGPRs) in registers with two waves
// per SIMD, which does not fit here; this kernel runs one wave per SIMD
// (four per workgroup, 128 query rows) with the full register file:
//   * each lane owns one query: its Q row slices (B operands of S^T = K Q^T)
//     and its column of O^T stay in registers; m and l are lane-local;
//   * 64-key tiles of K and V stream through LDS in padded rows, double
//     buffered: direct global_load_lds_dwordx4 copies of the next tile are
//     issued before the current one is used (one barrier per tile);
//   * per tile: S^T on the matrix cores, the online softmax in base 2 with the
//     deferred rescale of fwd_kernel (the offset moves only when a row max
//     grows by more than kRescaleTau), P rounded to 16 bits in registers as
//     the B operand of O^T += V^T P^T, whose A operand comes from transposing
//     LDS reads of the V tile.
// Masks: causal (tiles above a wave's diagonal skipped) and the sequence tail.
#pragma once

#include "fa_bwd_kernel.hpp"   // padded LDS tiles, async tile copies, operand lanes

namespace fa {

constexpr int kRows256 = kBwdRows;   // query rows per workgroup (4 waves x 32)

template <bool CAUSAL, bool VARLEN, bool F16>
__global__ __attribute__((amdgpu_flat_work_group_size(kBwdThreads, kBwdThreads),
                          amdgpu_waves_per_eu(1, 1)))
void fwd256_kernel(FwdParams p) {
  constexpr int D = 256, DS = D / 16, DB = D / 32, BC = kBwdTile;
  constexpr int RBP = 2 * D + 16;
  constexpr int TB = BC * RBP;
  // [K 0][V 0][K 1][V 1]: buffer b holds key tile 2 m + b.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TB];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int per = p.H * p.nbatch;
  int qt = blockIdx.x / per;
  const int rem = blockIdx.x - qt * per;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;   // longest rows of the mask first
  const int head = rem % p.H;
  const int bidx = rem / p.H;

  int Nq, Nk;
  int64_t q_off, k_off, v_off, o_off, l_off;
  if (VARLEN) {
    const int start = p.cu_seqlens[bidx];
    const int len = p.cu_seqlens[bidx + 1] - start;
    Nq = len;
    Nk = len;
    q_off = (int64_t)start * p.q_ts + (int64_t)head * p.q_hs;
    k_off = (int64_t)start * p.k_ts + (int64_t)head * p.k_hs;
    v_off = (int64_t)start * p.v_ts + (int64_t)head * p.v_hs;
    o_off = (int64_t)start * p.o_ts + (int64_t)head * p.o_hs;
    l_off = (int64_t)head * p.lse_head_stride + start;
  } else {
    Nq = p.Nq;
    Nk = p.Nk;
    q_off = (int64_t)bidx * p.q_bs + (int64_t)head * p.q_hs;
    k_off = (int64_t)bidx * p.k_bs + (int64_t)head * p.k_hs;
    v_off = (int64_t)bidx * p.v_bs + (int64_t)head * p.v_hs;
    o_off = (int64_t)bidx * p.o_bs + (int64_t)head * p.o_hs;
    l_off = (int64_t)bidx * p.lse_batch_stride + (int64_t)head * p.lse_head_stride;
  }
  const int q0 = qt * kRows256;
  if (q0 >= Nq) return;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  const float s2 = p.scale_log2;

  bf16x8 qr[DS];
  if (qrow < Nq) {
    const u32x4* src = reinterpret_cast<const u32x4*>(p.q + q_off + (int64_t)qrow * p.q_ts);
#pragma unroll
    for (int s = 0; s < DS; ++s) qr[s] = __builtin_bit_cast(bf16x8, src[2 * s + hi]);
  } else {
#pragma unroll
    for (int s = 0; s < DS; ++s) qr[s] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }
  const BwdLanes<D> ln(lane);
  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b] = f32x16{};
  float m_run = kNegInf;   // exponent offset (base 2, scaled scores)
  float l_run = 0.f;       // running sum over this lane's half of the keys

  const int kend = CAUSAL ? min(Nk, q0 + kRows256) : Nk;
  const int n_kt = (kend + BC - 1) / BC;
  const bool wave_has = qw0 < Nq;
  const int wave_last_kt = CAUSAL ? min(n_kt - 1, (qw0 + 31) / BC) : n_kt - 1;
  auto issue = [&](int kt, int b) __attribute__((always_inline)) {
    copy_tile_async<D>(smem_lds + (2 * b) * TB, p.k + k_off, (int)p.k_ts, kt * BC, Nk, wave, lane);
    copy_tile_async<D>(smem_lds + (2 * b + 1) * TB, p.v + v_off, (int)p.v_ts, kt * BC, Nk, wave,
                       lane);
  };
  if (n_kt > 0) issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * BC;
    const int buf = kt & 1;
    if (kt + 1 < n_kt) issue(kt + 1, buf ^ 1);   // buffer last read before the previous barrier
    const uint8_t* k_lds = smem + (2 * buf) * TB;
    const uint8_t* v_lds = smem + (2 * buf + 1) * TB;
    if (wave_has && kt <= wave_last_kt) {
      // S^T = K Q^T: 64 keys x the wave's 32 queries, keys in accumulator rows.
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          s[kb] = mfma32<F16>(lds16(k_lds, kb * 32 * RBP + ln.row_rd + ds * 32), qr[ds], s[kb]);
      }
      // Online softmax (base 2); masked keys (past the end, or after the
      // query when causal) get -inf, only on the tiles that can hold them.
      const bool masked = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > qw0);
      float mt = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool ok = !masked || (key < Nk && (!CAUSAL || key <= qrow));
          s[kb][r] = ok ? s[kb][r] * s2 : kNegInf;
          mt = fmaxf(mt, s[kb][r]);
        }
      }
      mt = max_xor32(mt);
      if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleTau) != 0) {
        asm volatile("" ::: "memory");   // keep the rescale a real branch
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < DB; ++b) o[b] *= alpha;
        m_run = m_new;
      }
      bf16x8 pb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          u32x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 8 * t + 2 * i;
            const float e0 = __builtin_amdgcn_exp2f(s[kb][r] - m_run);
            const float e1 = __builtin_amdgcn_exp2f(s[kb][r + 1] - m_run);
            w[i] = pack2<F16>(e0, e1);
            l_run += e0 + e1;
          }
          pb[kb][t] = __builtin_bit_cast(bf16x8, w);
        }
      }
      // O^T += V^T P^T.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int r0 = (32 * kb + 16 * t) * RBP;
#pragma unroll
          for (int b = 0; b < DB; ++b)
            o[b] = mfma32<F16>(lds_tr8(v_lds, r0 + ln.tr_rd[b], r0 + 8 * RBP + ln.tr_rd[b]), pb[kb][t], o[b]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of the next tile have landed
    __syncthreads();
  }
  // Epilogue: O = O_acc / l, L = ln2 (m + log2 l).
  const float l_tot = l_run + xor32(l_run);
  if (qrow < Nq) {
    store_rowT<D, F16>(p.o + o_off + (int64_t)qrow * p.o_ts, o, __builtin_amdgcn_rcpf(l_tot), hi);
    if (hi == 0) p.lse[l_off + qrow] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

}  // namespace fa
