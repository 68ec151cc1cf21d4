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
// Masks: causal (tiles above a wave's diagonal skipped), the sequence tail,
// the banded mask of fwd_kernel (BAND: query i sees key j iff
// i + band_off - win_left <= j <= i + band_off + win_right; key tiles outside
// the workgroup's band are not visited, a wave skips tiles outside its own)
// and the key padding mask (KPM, dense: one pass over the batch row's mask
// gives the span of valid tokens, tiles outside it are not visited, key
// validity per tile comes from a ballot of the mask, or from the span when
// the valid tokens form one run; padding queries get O = 0, L = -inf). A row
// that sees no key gets O = 0 and L = -inf.
#pragma once

#include "fa_bwd_kernel.hpp"   // padded LDS tiles, async tile copies, operand lanes

namespace fa {

constexpr int kRows256 = kBwdRows;   // query rows per workgroup (4 waves x 32)

template <bool CAUSAL, bool VARLEN, bool F16, bool BAND = false, bool KPM = false>
__global__ __attribute__((amdgpu_flat_work_group_size(kBwdThreads, kBwdThreads),
                          amdgpu_waves_per_eu(1, 1)))
void fwd256_kernel(FwdParams p) {
  static_assert(!(KPM && (BAND || VARLEN)) && !(CAUSAL && BAND), "mask combination");
  constexpr bool EMPTY_ROWS = BAND || KPM;
  constexpr int D = 256, DS = D / 16, DB = D / 32, BC = kBwdTile;
  constexpr int RBP = 2 * D + kRowPad<D>;
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
  if (p.q_sign) {   // negative scale: scale q.k = |scale| (-q).k
#pragma unroll
    for (int s = 0; s < DS; ++s) qr[s] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qr[s]) ^ p.q_sign);
  }
  const BwdLanes<D> ln(lane);
  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b] = f32x16{};
  float m_run = kNegInf;   // exponent offset (base 2, scaled scores)
  float l_run = 0.f;       // running sum over this lane's half of the keys

  const int kend = CAUSAL ? min(Nk, q0 + kRows256) : Nk;
  // Key tiles [kt_begin, kt_stop) hold a key some row of the workgroup sees.
  int kt_begin = 0, kt_stop = (kend + BC - 1) / BC;
  const int band_lo = BAND ? p.band_off - p.win_left : 0;
  const int band_hi = BAND ? p.band_off + p.win_right : 0;
  const int qw1 = min(Nq, qw0 + 32) - 1;   // last row of this wave
  if constexpr (BAND) {
    const int k_lo = max(0, q0 + band_lo);
    const int k_hi = min(Nk - 1, min(Nq, q0 + kRows256) - 1 + band_hi);
    kt_begin = k_lo / BC;
    kt_stop = k_hi >= k_lo ? k_hi / BC + 1 : kt_begin;
  }
  const uint8_t* kpm_row = KPM ? p.kpm + (int64_t)bidx * p.kpm_batch_stride : nullptr;
  KpmSpan span{0, Nk - 1, true};
  if constexpr (KPM) {
    span = kpm_span(kpm_row, Nk, reinterpret_cast<int*>(smem), tid);   // no tile copied yet
    if (span.lo > span.hi || q0 > span.hi || q0 + kRows256 - 1 < span.lo) {
      kt_stop = kt_begin;   // no valid key, or only padding queries
    } else {
      kt_begin = max(kt_begin, span.lo / BC);
      kt_stop = min(kt_stop, span.hi / BC + 1);
    }
  }
  const bool wave_has = qw0 < Nq && (!KPM || (qw0 <= span.hi && qw1 >= span.lo));
  // This wave's last tile (causal) and, with a band, its first and last.
  int wave_first_kt = kt_begin, wave_last_kt = kt_stop - 1;
  if (CAUSAL) wave_last_kt = min(wave_last_kt, qw1 / BC);
  if constexpr (BAND) {
    wave_first_kt = max(wave_first_kt, max(0, qw0 + band_lo) / BC);
    wave_last_kt = min(wave_last_kt, (qw1 + band_hi) / BC);
  }
  auto issue = [&](int kt, int b) __attribute__((always_inline)) {
    copy_tile_async<D>(smem_lds + (2 * b) * TB, p.k + k_off, (int)p.k_ts, kt * BC, Nk, wave, lane);
    copy_tile_async<D>(smem_lds + (2 * b + 1) * TB, p.v + v_off, (int)p.v_ts, kt * BC, Nk, wave,
                       lane);
  };
  if (kt_begin < kt_stop) issue(kt_begin, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = kt_begin; kt < kt_stop; ++kt) {
    const int k0 = kt * BC;
    const int buf = (kt - kt_begin) & 1;
    if (kt + 1 < kt_stop) issue(kt + 1, buf ^ 1);   // buffer last read before the previous barrier
    const uint8_t* k_lds = smem + (2 * buf) * TB;
    const uint8_t* v_lds = smem + (2 * buf + 1) * TB;
    if (wave_has && kt >= wave_first_kt && kt <= wave_last_kt) {
      uint32_t kvalid = ~0u;   // padding mask: validity bits of this lane's 32 keys
      bool kall = true;        // ... and whether all 64 keys of the tile are valid
      if constexpr (KPM) {
        const int key = k0 + lane;
        const bool kv = span.run ? (key >= span.lo && key <= span.hi)
                                 : (key < Nk && kpm_row[key] != 0);
        const uint64_t kbits = __builtin_amdgcn_ballot_w64(kv);
        kvalid = gather_lane_bits(kbits, hi);
        kall = kbits == ~0ull;
      }
      // S^T = K Q^T: 64 keys x the wave's 32 queries, keys in accumulator rows.
      // With one wave per SIMD nothing else hides the LDS latency: the K
      // operands go through a ring of RA registers, each read issued RA
      // products ahead of its use (sched_barrier keeps the reads and products
      // in that order, letting only ALU work move across), instead of a read,
      // a wait and a product in turn.
      constexpr int RA = 4, NS = 2 * DS;   // steps st = (ds, kb) = (st / 2, st % 2)
      auto k_off = [&](int st) { return (st & 1) * 32 * RBP + ln.row_rd + (st >> 1) * 32; };
      f32x16 s[2] = {f32x16{}, f32x16{}};
      bf16x8 ka[RA];
#pragma unroll
      for (int st = 0; st < RA; ++st) ka[st] = lds16(k_lds, k_off(st));
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const bf16x8 a = ka[st % RA];
        if (st + RA < NS) ka[st % RA] = lds16(k_lds, k_off(st + RA));
        s[st & 1] = mfma32<F16>(a, qr[st >> 1], s[st & 1]);
        __builtin_amdgcn_sched_barrier(0x7);   // only ALU work may cross
      }
      // Online softmax (base 2); masked keys (past the end, after the query
      // when causal, outside the band, padding) get -inf, only on the tiles
      // that can hold them.
      // Masked: some (row, key) pair of the wave's rows and the tile's keys is
      // hidden (past the end, after the query, outside the band, padding).
      const bool masked = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > qw0) ||
                          (BAND && (k0 < qw1 + band_lo || k0 + BC - 1 > qw0 + band_hi)) ||
                          (KPM && !kall);
      bf16x8 pb[2][2];
      // P~ = exp2(x - m) into the MFMA operands pb; returns the lane's sum.
      // x = S^T scale_log2, or the already scaled and masked s.
      auto exps = [&](auto scaled_tag, float neg_m) __attribute__((always_inline)) -> float {
        constexpr bool scaled = decltype(scaled_tag)::value;
        float sum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            u32x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 8 * t + 2 * i;
              const float x0 = scaled ? s[kb][r] + neg_m : __builtin_fmaf(s[kb][r], s2, neg_m);
              const float x1 = scaled ? s[kb][r + 1] + neg_m : __builtin_fmaf(s[kb][r + 1], s2, neg_m);
              const float e0 = __builtin_amdgcn_exp2f(x0);
              const float e1 = __builtin_amdgcn_exp2f(x1);
              w[i] = pack2<F16>(e0, e1);
              sum += e0 + e1;
            }
            pb[kb][t] = __builtin_bit_cast(bf16x8, w);
          }
        }
        return sum;
      };
      // Unmasked tile: exponentials against the current offset first; the
      // lane's sum bounds each of its P~, so the row maximum and the rescale
      // below are needed only when some lane's sum exceeds 2^kRescaleTau (or
      // is not a number). Masked tiles, and a wave with a row that has no
      // offset yet (its first visible tile), take that path always.
      float tsum = 0.f;
      bool full = true;
      if (!masked && __builtin_amdgcn_ballot_w64(m_run == kNegInf) == 0) {
        tsum = exps(std::false_type{}, -m_run);
        full = __builtin_amdgcn_ballot_w64(!(tsum <= (float)(1 << (int)kRescaleTau))) != 0;
      }
      if (full) {
        // A real branch, and m_run opaque, so the exponentials above are
        // not kept alive for reuse.
        asm volatile("" : "+v"(m_run) : : "memory");
        float mt = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
            bool ok = (key < Nk) & (!CAUSAL | (key <= qrow));
            if constexpr (BAND) ok = ok & (key >= qrow + band_lo) & (key <= qrow + band_hi);
            if constexpr (KPM) ok = ok & (((kvalid >> (16 * kb + r)) & 1u) != 0);
            ok = ok | !masked;
            s[kb][r] = ok ? s[kb][r] * s2 : kNegInf;
            mt = fmaxf(mt, s[kb][r]);
          }
        }
        mt = max_xor32(mt);
        if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleTau) != 0) {
          asm volatile("" ::: "memory");   // keep the rescale a real branch
          const float m_new = fmaxf(m_run, mt);
          // A row that has seen no key yet keeps m = -inf (no NaN from -inf - -inf).
          const float alpha = (EMPTY_ROWS && m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int b = 0; b < DB; ++b) o[b] *= alpha;
          m_run = m_new;
        }
        const float m_use = (EMPTY_ROWS && m_run == kNegInf) ? 0.f : m_run;   // no key yet: p = 0
        tsum = exps(std::true_type{}, -m_use);
      }
      l_run += tsum;
      // O^T += V^T P^T, with the same read-ahead for the transposed V
      // operands (steps st = (16-key group g = st / DB, column block st % DB)).
      constexpr int NP = 4 * DB;
      auto v_op = [&](int st) {
        const int g = st / DB, b = st % DB;
        const int r0 = (32 * (g >> 1) + 16 * (g & 1)) * RBP;
        return lds_tr8(v_lds, r0 + ln.tr_rd[b], r0 + 8 * RBP + ln.tr_rd[b]);
      };
      bf16x8 va[RA];
#pragma unroll
      for (int st = 0; st < RA; ++st) va[st] = v_op(st);
#pragma unroll
      for (int st = 0; st < NP; ++st) {
        const bf16x8 a = va[st % RA];
        if (st + RA < NP) va[st % RA] = v_op(st + RA);
        const int g = st / DB;
        o[st % DB] = mfma32<F16>(a, pb[g >> 1][g & 1], o[st % DB]);
        __builtin_amdgcn_sched_barrier(0x7);   // only ALU work may cross
      }
    }
    stress_pause(kt);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of the next tile have landed
    __syncthreads();
  }
  // Epilogue: O = O_acc / l, L = ln2 (m + log2 l); a row that saw no key
  // (band) or a padding query: O = 0, L = -inf.
  const float l_tot = l_run + xor32(l_run);
  if (qrow < Nq) {
    bool empty = EMPTY_ROWS && !(l_tot > 0.f);
    if constexpr (KPM) empty = empty || kpm_row[qrow] == 0;
    store_rowT<D, F16>(p.o + o_off + (int64_t)qrow * p.o_ts, o,
                       empty ? 0.f : __builtin_amdgcn_rcpf(l_tot), hi);
    if (hi == 0) p.lse[l_off + qrow] = empty ? kNegInf : (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

}  // namespace fa
