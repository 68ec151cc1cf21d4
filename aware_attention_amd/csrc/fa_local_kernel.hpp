// Attention with a local window on a token map plus global anchor tokens, on
// gfx950: device code.
//
// The pattern is that of the detector page ("YOLOv12官版镜像集成Flash
// Attention v2，提速原理浅析", section 4.2, dynamic sparse attention): each
// token attends its neighbourhood on the feature map (a 5 x 5 window in the
// page's example) plus a few global anchors, the window restricting the
// range of key blocks that are visited, the anchors' K and V loaded on their
// own. Layout of the tokens: the first n_global are the anchors, the rest a
// row-major map of map_w tokens per row. Query i sees key j iff i or j is an
// anchor, or their map positions differ by at most win_rows rows and
// win_cols columns; causal adds j <= i.
//
// Kernel: one workgroup of four waves per 128 queries of one (batch, head);
// each lane owns one query (its Q row slices in registers as the B operand of
// S^T = K Q^T, its column of O^T in accumulators), as in the head-dimension-
// 256 forward. The anchor queries get workgroups of their own (dispatched
// first: they visit every key tile, with no map test); a map workgroup holds
// 128 map queries and visits the anchor key tiles, then the key tiles of the
// map rows its queries reach; a wave skips a visited tile in which none of
// its queries sees a key. Tiles of 64 keys stream through a ring of R LDS slots
// (R = 4 for d <= 64, 2 above, so that two workgroups fit a CU): the direct
// global_load_lds_dwordx4 copies of tile it + R - 1 are issued before tile
// it is used, and each wave waits only for the copies of the next tile
// (s_waitcnt vmcnt with the later tiles' copies still in flight) before the
// one barrier per tile. With each tile, 64 threads write the map row and
// column of its keys to LDS (integer division once per key and tile), so
// that the per-score visibility test is a few integer compares. The online
// softmax (base 2, deferred rescale) and P V follow the forward kernels; a
// row that has not seen a key yet keeps m = -inf without producing NaN.
#pragma once

#include "fa_bwd_kernel.hpp"   // padded LDS tiles, async tile copies, operand lanes

namespace fa {

struct LocalParams {
  const uint16_t* q;          // (B, N, H, d)
  const uint16_t* k;          // (B, N, H, d)
  const uint16_t* v;          // (B, N, H, d)
  uint16_t* o;                // (B, N, H, d)
  float* lse;                 // (B, H, N), natural log
  int64_t row_stride;         // H * d
  int64_t batch_stride;       // N * H * d
  int32_t N, H, B;
  int32_t n_global;           // anchors: tokens [0, n_global), n_global <= N
  int32_t map_w;              // map tokens per row, 1 <= map_w <= max(1, N - n_global)
  int32_t win_rows, win_cols; // window half-sizes, clamped to the map's extent
  int32_t n_anchor_tiles;     // 128-query tiles of anchor queries per (batch, head)
  int32_t n_tiles;            // all 128-query tiles per (batch, head), anchor ones first
  float scale_log2;           // softmax scale * log2(e)
};

constexpr int kLocalRows = kBwdRows;            // queries per workgroup
template <int D> constexpr int kLocalRing = D <= 64 ? 4 : 2;   // LDS tile slots

// s_waitcnt: at most n vector memory operations of this wave still in flight
// and none of its LDS operations (expcnt unconstrained).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));
}

// Wait until at most `newer` tiles' copies, issued after the tile that is
// needed next, remain in flight. Each wave issues at least D/16 copies per
// tile (K and V, kBwdWaves waves sharing D/8 + kRowPad<D>/16 slots per row), so allowing
// newer * D/16 outstanding never lets the needed tile's copies through
// unfinished.
template <int D, int R>
__device__ __forceinline__ void wait_tile(int newer) {
  constexpr int C = D / 16;
  if constexpr (R > 3) {
    if (newer >= 3) { wait_vmcnt<3 * C < 64 ? 3 * C : 0>(); return; }
  }
  if constexpr (R > 2) {
    if (newer >= 2) { wait_vmcnt<2 * C < 64 ? 2 * C : 0>(); return; }
    if (newer == 1) { wait_vmcnt<C < 64 ? C : 0>(); return; }
  }
  wait_vmcnt<0>();
}

template <int D, bool CAUSAL, bool F16>
__global__ __attribute__((amdgpu_flat_work_group_size(kBwdThreads, kBwdThreads),
                          amdgpu_waves_per_eu(D == 256 ? 1 : 2, D == 256 ? 1 : 8)))
void fwd_local_kernel(LocalParams p) {
  constexpr int DS = D / 16, DB = D / 32, BC = kBwdTile, R = kLocalRing<D>;
  constexpr int RBP = 2 * D + kRowPad<D>;
  constexpr int TB = BC * RBP;
  // [K 0][V 0][K 1][V 1]...: slot b holds visited tiles b, b + R, b + 2R, ...
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * R * TB];
  // Map row and column of each key of the tile in slot b.
  __shared__ __attribute__((aligned(16))) int kmrow[R][BC];
  __shared__ __attribute__((aligned(16))) int kmcol[R][BC];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int per = p.H * p.B;
  const int qt = blockIdx.x / per;
  const int rem = blockIdx.x - qt * per;
  const int head = rem % p.H;
  const int bidx = rem / p.H;
  const int N = p.N, G = p.n_global, W = p.map_w, WR = p.win_rows, WC = p.win_cols;
  const int64_t base = (int64_t)bidx * p.batch_stride + (int64_t)head * D;
  const int64_t l_off = ((int64_t)bidx * p.H + head) * N;
  const int rs = (int)p.row_stride;

  // Queries [q0, q1): anchors [0, G) in the first n_anchor_tiles tiles, then
  // the map tokens from G on.
  const bool anchor_wg = qt < p.n_anchor_tiles;
  const int q0 = anchor_wg ? qt * kLocalRows : G + (qt - p.n_anchor_tiles) * kLocalRows;
  const int q1 = min(anchor_wg ? G : N, q0 + kLocalRows);
  if (q0 >= q1) return;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  const float s2 = p.scale_log2;

  // Key tiles the workgroup visits: [0, A) (the anchors' tiles; every tile
  // up to the causal limit when the workgroup holds an anchor query), then
  // [W0, W1) (the map rows within win_rows of its queries' rows).
  const int kend = CAUSAL ? q1 : N;
  const int n_kt_all = (kend + BC - 1) / BC;
  int A, W0, W1;
  if (anchor_wg) {
    A = n_kt_all;
    W0 = W1 = A;
  } else {
    A = min((G + BC - 1) / BC, n_kt_all);
    const int r_lo = (q0 - G) / W, r_hi = (q1 - 1 - G) / W;
    const int klo = G + max(0, r_lo - WR) * W;
    const int khi = min(kend, G + (r_hi + WR + 1) * W) - 1;
    W0 = max(A, klo / BC);
    W1 = max(W0, khi / BC + 1);
  }
  const int n_iter = A + (W1 - W0);

  // This wave's queries: which tiles hold a key one of them sees.
  const bool wave_has = qw0 < q1;
  const int qw1 = min(q1, qw0 + 32) - 1;
  int wklo = 0, wkhi = N - 1;
  if (wave_has && !anchor_wg) {
    const int rlo = (qw0 - G) / W, rhi = (qw1 - G) / W;
    wklo = G + max(0, rlo - WR) * W;
    wkhi = min(N, G + (rhi + WR + 1) * W) - 1;
  }
  // This lane's query on the map (unused in an anchor workgroup).
  const bool q_valid = qrow < q1;
  int ir = 0, ic = 0;
  if (!anchor_wg && q_valid) {
    ir = (qrow - G) / W;
    ic = (qrow - G) - ir * W;
  }

  bf16x8 qr[DS];
  if (q_valid) {
    const u32x4* src = reinterpret_cast<const u32x4*>(p.q + base + (int64_t)qrow * rs);
#pragma unroll
    for (int s = 0; s < DS; ++s) qr[s] = __builtin_bit_cast(bf16x8, src[2 * s + hi]);
  } else {
#pragma unroll
    for (int s = 0; s < DS; ++s) qr[s] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }
  // The Q rows land before the first tile copy is issued, so that no wait
  // for them inside the loop holds back the copies in flight.
  __builtin_amdgcn_s_waitcnt(0);
  const BwdLanes<D> ln(lane);
  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b] = f32x16{};
  float m_run = kNegInf;   // exponent offset (base 2, scaled scores)
  float l_run = 0.f;       // running sum over this lane's half of the keys

  auto tile_of = [&](int it) { return it < A ? it : W0 + (it - A); };
  auto issue = [&](int kt, int b) __attribute__((always_inline)) {
    copy_tile_async<D>(smem_lds + (2 * b) * TB, p.k + base, rs, kt * BC, N, wave, lane);
    copy_tile_async<D>(smem_lds + (2 * b + 1) * TB, p.v + base, rs, kt * BC, N, wave, lane);
    if (!anchor_wg && tid < BC) {
      int r, c;
      map_pos(kt * BC + tid, G, W, N, r, c);
      kmrow[b][tid] = r;
      kmcol[b][tid] = c;
    }
  };
  // The copies are asynchronous writes into LDS that the compiler does not
  // see. Before the one barrier per tile (without a fence) every wave waits
  // for its copies of the next tile (wait_tile) and for all of its LDS
  // operations: its reads of the slot the next copy overwrites, and wave 0's
  // key coordinates. sched_barrier keeps the tile's LDS reads and their uses
  // ahead of that wait.
  auto publish = [&](int newer) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    stress_pause(newer);
    wait_tile<D, R>(newer);
    barrier_nofence();
  };
  for (int j = 0; j < R - 1 && j < n_iter; ++j) issue(tile_of(j), j);
  if (n_iter > 0) publish(min(R - 2, n_iter - 1));
  for (int it = 0; it < n_iter; ++it) {
    const int kt = tile_of(it);
    const int k0 = kt * BC;
    const int buf = it % R;
    // Slot (it + R - 1) % R was last read in tile it - 1, before its barrier.
    if (it + R - 1 < n_iter) issue(tile_of(it + R - 1), (it + R - 1) % R);
    const uint8_t* k_lds = smem + (2 * buf) * TB;
    const uint8_t* v_lds = smem + (2 * buf + 1) * TB;
    const bool useful = wave_has && (!CAUSAL || k0 <= qw1) &&
                        (anchor_wg || k0 < G || (k0 + BC - 1 >= wklo && k0 <= wkhi));
    if (useful) {
      // S^T = K Q^T: 64 keys x the wave's 32 queries, keys in accumulator rows.
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          s[kb] = mfma32<F16>(lds16(k_lds, kb * 32 * RBP + ln.row_rd + ds * 32), qr[ds], s[kb]);
      }
      // P~ = exp2(x - m) into the MFMA operands pb; returns the lane's sum.
      // x = S^T scale_log2, or the already scaled and masked s.
      bf16x8 pb[2][2];
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
      // An anchor query sees every key of a tile inside the sequence (when
      // causal, of a tile left of the wave's first row): no mask. Such a tile
      // is exponentiated against the current offset first; the lane's sum of
      // P~ bounds each term, so the row maximum and the rescale are needed
      // only when some lane's sum exceeds 2^kRescaleTau (or is not a number),
      // or while a row has no offset yet.
      const bool open_tile = anchor_wg && k0 + BC <= N && (!CAUSAL || k0 + BC - 1 <= qw0);
      float tsum = 0.f;
      bool full = true;
      if (open_tile && __builtin_amdgcn_ballot_w64(m_run == kNegInf) == 0) {
        tsum = exps(std::false_type{}, -m_run);
        full = __builtin_amdgcn_ballot_w64(!(tsum <= (float)(1 << (int)kRescaleTau))) != 0;
      }
      if (full) {
        // A real branch, and m_run opaque, so the exponentials above are not
        // kept alive for reuse.
        asm volatile("" : "+v"(m_run) : : "memory");
        // Visibility of each score: an anchor query sees every key (up to
        // itself when causal); a map query decides from the keys' map positions.
        float mt = kNegInf;
        if (anchor_wg) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
              const bool vis = (key < N) & (!CAUSAL | (key <= qrow));
              s[kb][r] = vis ? s[kb][r] * s2 : kNegInf;
              mt = fmaxf(mt, s[kb][r]);
            }
          }
        } else {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int kk = 32 * kb + 8 * g + 4 * hi;   // first of this lane's 4 keys
              const i32x4 kr = *reinterpret_cast<const i32x4*>(&kmrow[buf][kk]);
              const i32x4 kc = *reinterpret_cast<const i32x4*>(&kmcol[buf][kk]);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * g + e;
                // Bitwise, not short-circuit, operators: one select per score
                // instead of divergent branches.
                bool vis = map_near(kr[e], kc[e], ir, ic, WR, WC) | (kr[e] == kKeyAnchor);
                if (CAUSAL) vis = vis & (k0 + kk + e <= qrow);
                s[kb][r] = vis ? s[kb][r] * s2 : kNegInf;
                mt = fmaxf(mt, s[kb][r]);
              }
            }
          }
        }
        mt = max_xor32(mt);
        if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleTau) != 0) {
          asm volatile("" ::: "memory");   // keep the rescale a real branch
          const float m_new = fmaxf(m_run, mt);
          const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int b = 0; b < DB; ++b) o[b] *= alpha;
          m_run = m_new;
        }
        const float m_use = m_run == kNegInf ? 0.f : m_run;   // no key seen yet: every p is 0
        tsum = exps(std::true_type{}, -m_use);
      }
      l_run += tsum;
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
    if (it + 1 < n_iter) publish(min(R - 2, n_iter - 2 - it));   // tile it + 1 is next
  }
  // Epilogue: O = O_acc / l, L = ln2 (m + log2 l). Every query sees itself,
  // so l > 0; the guard only keeps a degenerate row finite.
  const float l_tot = l_run + xor32(l_run);
  if (q_valid) {
    const bool empty = !(l_tot > 0.f);
    store_rowT<D, F16>(p.o + base + (int64_t)qrow * rs, o, empty ? 0.f : __builtin_amdgcn_rcpf(l_tot), hi);
    if (hi == 0) p.lse[l_off + qrow] = empty ? kNegInf : (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

}  // namespace fa
