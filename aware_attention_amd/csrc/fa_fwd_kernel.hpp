// FlashAttention-2 forward for gfx950 (CDNA4): device code.
//
// What one workgroup does ("FlashAttention/zh" (marovi.ai wiki), section
// FlashAttention 算法, with the FlashAttention-2 loop order of section
// 變體與後續版本: outer loop over query blocks spread across the grid, inner
// loop over key/value blocks inside the workgroup):
//   * owns one query tile of BR = 256 rows of one (batch or sequence, head);
//     each of its 8 wavefronts owns 32 of those rows and keeps its Q rows in
//     VGPRs for the whole kernel;
//   * streams key/value tiles of BC = 64 keys through LDS, double-buffered,
//     copied straight from HBM into LDS (global_load_lds_dwordx4);
//   * per tile, per wavefront: S^T = K Q^T on bf16 MFMA (fp32 accumulate),
//     online-softmax update in base 2 (running max m, running sum l, rescale
//     of the output accumulator by exp2(m_old - m_new)), then
//     O^T += V^T P^T on bf16 MFMA with P rounded to bf16;
//   * finally O = O_acc / l goes out as bf16 and L = ln2 * (m + log2 l) as fp32.
//
// Two wave groups in ping-pong. Waves 0-3 (group A, rows 0-127) and waves 4-7
// (group B, rows 128-255) share the four SIMDs of a CU, one wave of each
// group per SIMD. Each key tile j is one period between workgroup barriers,
// made of an M block (matrix cores: S^T of tile j, and O^T += V^T P^T of
// tile j-1) and a V block (vector ALU: the online softmax of a tile):
//   group A runs M_j, then the softmax of tile j;
//   group B runs the softmax of tile j-1, then M_j.
// So on every SIMD one wave issues MFMAs while the other does exponentials,
// then they swap. There is no barrier between the two blocks: measured on
// gfx950, a barrier at each block change restarts both waves of a SIMD in
// step and serialises them, while free-running waves overlap their MFMA and
// VALU work.
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
// lane l and lane l^32 (v_permlane32_swap). The accumulator registers of S^T
// feed the B operand of the P V product directly, with no trip through LDS:
// register group r = 8t..8t+7 of a 32-key block holds keys
// 16t + {0..3, 8..11} + 4*(l/32). K and V sit in LDS row-major; the V^T
// operand comes from transposing 8-byte reads (ds_read_b64_tr_b16),
// addressed so the transpose hands each lane the keys in exactly that order.
//
// Masking ("FlashAttention/zh", section 變體與後續版本: causal masks):
// keys past the sequence end and, when causal, keys after the query are set
// to -inf, only on the tiles that need it; tiles entirely above a wavefront's
// diagonal are skipped, and key tiles past the workgroup's last query are
// never loaded. A banded mask (same section: the fused kernel composes with
// banded masks) likewise loads only the key tiles inside some row's band.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

// Operand registers are typed bf16x8 whatever the element type; for fp16
// inputs the same bits hold fp16 values and are reinterpreted at the MFMA.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* cu_seqlens;   // varlen only
  // Strides in elements of q, k, v and o (d is contiguous): between batches
  // (dense only), consecutive tokens and heads. Token strides are at most
  // 2^24 and every stride is a multiple of 8 (16-byte aligned rows).
  int64_t q_bs, q_ts, q_hs;
  int64_t k_bs, k_ts, k_hs;
  int64_t v_bs, v_ts, v_hs;
  int64_t o_bs, o_ts, o_hs;
  int64_t lse_batch_stride;    // dense: H * Nq
  int64_t lse_head_stride;     // dense: Nq; varlen: total
  int32_t Nq;                  // dense only
  int32_t Nk;                  // dense only
  int32_t H;
  int32_t nbatch;              // B (dense) or num_seqs (varlen)
  int32_t n_qtiles;            // query tiles per (batch or sequence, head)
  float scale_log2;            // |softmax_scale| * log2(e)
  // 0, or 0x80008000 for a negative softmax_scale: the sign is moved into Q
  // (every 16-bit element of the Q registers negated, which is exact), so the
  // kernel always works with the non-negative |scale| above.
  uint32_t q_sign;
  // Band (BAND instances only): query i sees key j iff
  // i + band_off - win_left <= j <= i + band_off + win_right.
  int32_t win_left;            // >= 0; an unbounded side is passed as max(Nq, Nk)
  int32_t win_right;           // >= 0; likewise (varlen: max_seqlen)
  int32_t band_off;            // Nk - Nq (dense), 0 (varlen)
  // Key padding mask (KPM instances only, dense self-attention): token n of
  // batch b is valid iff kpm[b * kpm_batch_stride + n] != 0.
  const uint8_t* kpm;
  int64_t kpm_batch_stride;
};

constexpr int kWaves = 8;                 // two groups of four
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;          // query rows per workgroup
constexpr int kBC = 64;                   // keys per LDS tile
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kRescaleTau = 8.0f;
constexpr int kPrefetch = 8;              // MFMA-phase operand fragments in flight

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// max(x[l], x[l ^ 32]) in every lane l with one v_permlane32_swap, a VALU
// op: it swaps the upper half of one copy of x with the lower half of
// another, so each lane then holds x from both halves of the wave, whichever
// half is swapped with which. Unlike a ds_bpermute it does not queue behind
// the other wave group's LDS operand reads. Written as inline asm (the s_nop
// covers the VALU-write-then-permlane-read hazard, which the compiler does
// not see inside asm); the builtin was folded incorrectly by the compiler
// when both operands were the same value.
__device__ __forceinline__ float max_xor32(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

// max(a, b, c) in one v_max3_f32. Written as inline asm: the generic fmaxf
// route quiets each MFMA result with an extra v_max before comparing, which
// doubles the cost of the row maximum. NaN scores still reach the output:
// they are dropped from the maximum but not from exp2(score - m).
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Two floats rounded (to nearest even) to the 16-bit element type, packed
// low then high: one v_cvt_pk_bf16_f32 or v_cvt_pk_f16_f32.
template <bool F16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (F16) {
    const f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
}

// D += A B on the 32x32x16 matrix core in the element type (fp32 accumulate).
template <bool F16>
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Timing-perturbed build (compiled with -DFA_STRESS into a library of its own
// for the race tests): a wave-uniform pseudo-random pause of 0..7 x 64 cycles
// at the points where waves hand LDS buffers to one another, so that a
// missing wait or barrier shows as a wrong result instead of staying hidden
// by the usual timing. Compiles to nothing otherwise.
__device__ __forceinline__ void stress_pause(int salt) {
#ifdef FA_STRESS
  uint32_t h = ((uint32_t)blockIdx.x * 0x9E3779B1u) ^ ((uint32_t)(threadIdx.x >> 6) * 0x85EBCA77u) ^
               ((uint32_t)salt * 0xC2B2AE3Du);
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  const int n = __builtin_amdgcn_readfirstlane((int)(h & 7u));
  for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(1);
#else
  (void)salt;
#endif
}

// Workgroup barrier without a memory fence: LDS operand reads of the current
// tiles may stay in flight across it (they are read-only). The copies into
// LDS are made visible explicitly (s_waitcnt by the issuing waves before the
// barrier that publishes them).
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// One 16-byte-per-lane HBM -> LDS copy (global_load_lds_dwordx4): lane l's
// 16 bytes from gbase + voff land at LDS byte lds_base + 16*l. gbase and
// lds_base must be the same in every lane of the wave (they go to SGPRs and
// M0); voff is the lane's unsigned 32-bit byte offset, so the per-lane
// address needs no 64-bit arithmetic. Issued as inline asm on purpose: the
// compiler would otherwise treat every later LDS read as a possible reader
// of this asynchronous write and wait for the copy to land before it, even
// when (as here, by construction) the reads target another buffer. The
// instruction has no register outputs; the kernel itself waits for the
// copies (s_waitcnt vmcnt) before the barrier that publishes them.
__device__ __forceinline__ void copy16_to_lds(const void* gbase, uint32_t voff, uint32_t lds_base) {
  // readfirstlane returns a signed int: widen through uint32_t, or a low
  // word with bit 31 set would be sign-extended over the high word.
  const uint64_t b = reinterpret_cast<uint64_t>(gbase);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(bs), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory", "m0");
}

// Store a wave's 32 x D block of rows held transposed in MFMA accumulators
// (lane l owns row l % 32; register group b, g holds columns
// 32 b + 8 g + 4 (l / 32) + 0..3), each row times its lane's `mul`, rounded to
// the 16-bit element type. Stored directly, that is 16 eight-byte stores per
// lane with every instruction touching 32 rows. Instead the block goes
// through `wtile`, 32 * 2D bytes of LDS that this wave alone uses at this
// point: the pieces are written with the 16-byte chunks of each row
// XOR-swizzled by the row's position in the 64 LDS banks (so the writes and
// the reads spread over the banks), read back in row order and stored as
// whole rows, D/8 lanes per row and 16 bytes per lane. Rows r >= nrows are
// not stored; row r goes to row0 + r * rstride (elements).
template <int D, bool F16>
__device__ __forceinline__ void store_tileT(uint16_t* row0, int64_t rstride, int nrows,
                                            const f32x16 (&acc)[D / 32], float mul,
                                            uint8_t* wtile, int lane) {
  constexpr int RB = 2 * D, CPR = D / 8, RPI = 64 / CPR;
  constexpr int RPB = RB < 256 ? 256 / RB : 1;        // rows per 256 bytes (64 banks)
  constexpr int SW = CPR < 16 ? CPR : 16;
  auto swz = [](int r) { return (r / RPB) % SW; };
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int b = 0; b < D / 32; ++b) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint2 w = {pack2<F16>(acc[b][4 * g] * mul, acc[b][4 * g + 1] * mul),
                       pack2<F16>(acc[b][4 * g + 2] * mul, acc[b][4 * g + 3] * mul)};
      const int c = 4 * b + g;                        // chunk of columns 8c .. 8c + 7
      *reinterpret_cast<uint2*>(wtile + l32 * RB + ((c ^ swz(l32)) * 16) + 8 * hi) = w;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the block is in LDS
  const int rsub = lane / CPR, ch = lane % CPR;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + rsub;
    const u32x4 val = *reinterpret_cast<const u32x4*>(wtile + r * RB + ((ch ^ swz(r)) * 16));
    if (r < nrows) *reinterpret_cast<u32x4*>(row0 + (int64_t)r * rstride + 8 * ch) = val;
  }
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

// Occupancy: two waves per SIMD (one workgroup per CU) at d = 64 and 128,
// where the per-lane state needs up to 256 VGPRs. At d = 32 the state fits
// in 128 VGPRs, so two workgroups share a CU (four waves per SIMD): the
// softmax dominates there, and the extra waves hide its latency.
// BAND selects the banded mask (FlashAttention composes with banded masks:
// "FlashAttention/zh", section 變體與後續版本; each token attends a local
// window and window attention skips the key blocks outside it: "YOLOv12官版
// 镜像集成Flash Attention v2，提速原理浅析", section 4.2). A row that sees no
// key gets O = 0 and L = -inf.
// Dispatch rank r (0 = first) -> query tile for a band, longest rows first.
// Tile t (q0 = t kBR) holds min(Nk, q0 + kBR + band_hi) - max(0, q0 + band_lo)
// key columns: a concave function of q0 with slopes +1 and -1, largest
// around q0 = c = (Nk - kBR - band_hi - band_lo) / 2. Tiles are taken by
// distance from c, alternating sides (tile floor(c / kBR), the one after
// it, the one before, ...), then the longer side's remainder; a causal-like
// band (left side unbounded) gives the descending order of causal
// attention. Returns a permutation of [0, n) over r in [0, n).
__device__ inline int band_tile_of_rank(int r, int n, int Nk, int band_lo, int band_hi) {
  const int64_t c2 = (int64_t)Nk - kBR - band_hi - band_lo;     // 2c
  const int tc = c2 < 0 ? 0 : (int)min<int64_t>(c2 / (2 * kBR), n - 1);
  const int left = tc + 1, right = n - 1 - tc;                  // tiles on each side
  const int m = min(left, right);
  if (r < 2 * m) return (r & 1) ? tc + 1 + (r >> 1) : tc - (r >> 1);
  const int rest = r - 2 * m;
  return left > right ? tc - m - rest : tc + 1 + m + rest;
}

template <int D, bool CAUSAL, bool VARLEN, bool BAND, bool F16, bool KPM>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(D == 32 ? 4 : 2, D == 32 ? 4 : 2)))
void fwd_kernel(FwdParams p) {
  static_assert(D == 32 || D == 64 || D == 128, "head dim");
  static_assert(!(CAUSAL && BAND), "causal is the band (unbounded, 0)");
  static_assert(!(KPM && (BAND || VARLEN)), "the key padding mask is for dense batches");
  // A row can see no key at all (a band, or a padding mask).
  constexpr bool EMPTY_ROWS = BAND || KPM;
  constexpr int BC = kBC;
  using TL = TileLayout<D>;
  constexpr int RB = TL::kRowBytes;
  constexpr int TILE_BYTES = BC * RB;            // one K or V tile
  constexpr int KB = BC / 32;                    // 32-key blocks per tile
  constexpr int DS = D / 16;                     // MFMA k-steps over d
  constexpr int DB = D / 32;                     // 32-wide d blocks of O^T
  constexpr int NCP = TILE_BYTES / 1024;         // 1 KiB direct copies per tile
  constexpr int NPW = NCP / 4;                   // ... per wave of group A
  static_assert(NCP % 4 == 0 && NPW >= 1, "tile split");

  // [K buf 0][K buf 1][V buf 0][V buf 1]
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TILE_BYTES];

  // LDS byte address of smem (the low 32 bits of its flat address).
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bool group_b = wave >= 4;
  const int gw = wave & 3;               // wave index inside its group

  // ---- work item: (query tile, head, batch or sequence) ----
  // A unit is one (batch or sequence, head): all its query tiles read the
  // same K and V. Workgroups go to the 8 XCDs round-robin by blockIdx.x, and
  // each XCD has its own L2.
  //  * Unmasked attention, unit count a multiple of 8: blockIdx.x = 8m + x
  //    maps XCD x's m-th workgroup to unit x + 8 * (m / n_qtiles), query tile
  //    m % n_qtiles, so an XCD works through the query tiles of a few units
  //    at a time and they share K/V tiles in its L2 (ViT-shaped batch: HBM
  //    reads 2.3 GB -> 0.64 GB per launch, +15 %).
  //  * Otherwise, and always for causal and banded attention, tile-major:
  //    blockIdx.x = rank * units + unit. With a unit count that is a
  //    multiple of 8 each XCD still sees only units congruent to its index;
  //    causal and banded ranks run the query tiles with the most key tiles
  //    first, across all units, which balances the CUs (unit-grouped causal
  //    order measured 2-12 % slower).
  const int per_qt = p.H * p.nbatch;   // units
  int qt, rem;
  if (!CAUSAL && !BAND && (per_qt & 7) == 0) {
    const int m = blockIdx.x >> 3;
    qt = m % p.n_qtiles;
    rem = (blockIdx.x & 7) + 8 * (m / p.n_qtiles);
  } else {
    qt = blockIdx.x / per_qt;
    rem = blockIdx.x - qt * per_qt;
  }
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;
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
  int band_lo = 0, band_hi = 0;
  if constexpr (BAND) {
    band_lo = p.band_off - p.win_left;
    band_hi = p.band_off + p.win_right;
    const int n_seq = (Nq + kBR - 1) / kBR;   // this sequence's query tiles
    if (qt < n_seq) qt = band_tile_of_rank(qt, n_seq, Nk, band_lo, band_hi);
  }
  const int q0 = qt * kBR;
  if (q0 >= Nq) return;   // whole workgroup: tile past this sequence's end

  const uint16_t* __restrict__ qg = p.q + q_off;
  const uint8_t* __restrict__ kg = reinterpret_cast<const uint8_t*>(p.k + k_off);
  const uint8_t* __restrict__ vg = reinterpret_cast<const uint8_t*>(p.v + v_off);
  const int q_ts = (int)p.q_ts;              // token strides: elements
  const int o_ts = (int)p.o_ts;
  const int k_tb = 2 * (int)p.k_ts;          // ... and bytes
  const int v_tb = 2 * (int)p.v_ts;
  const float s2 = p.scale_log2;

  const int kend = CAUSAL ? min(Nk, q0 + kBR) : Nk;
  const int n_kt = (kend + BC - 1) / BC;
  // Key tiles [kt0, kt_end) hold a visible key for some row of the
  // workgroup; with a band, keys j visible from row i satisfy
  // i + band_lo <= j <= i + band_hi, and the range may be empty.
  int kt0 = 0, kt_end = n_kt;
  if constexpr (BAND) {
    const int k_lo = max(0, q0 + band_lo);
    const int k_hi = min(Nk - 1, min(Nq, q0 + kBR) - 1 + band_hi);
    kt0 = k_lo / BC;
    kt_end = k_hi >= k_lo ? k_hi / BC + 1 : kt0;
  }
  // Key padding mask: the valid tokens of this batch row lie in [kv_lo,
  // kv_hi] (one pass over the row's mask by the whole workgroup). Key tiles
  // outside that span hold only padding and are skipped; a query tile outside
  // it holds only padding rows and does no work at all.
  // kv_run: the valid tokens form one run (no padding inside the span).
  const uint8_t* kpm_row = nullptr;
  int kv_lo = 0, kv_hi = Nk - 1;
  bool kv_run = true;
  if constexpr (KPM) {
    kpm_row = p.kpm + (int64_t)bidx * p.kpm_batch_stride;
    int lo = Nk, hi_ = -1, cnt = 0;
    for (int i = tid; i < Nk; i += kThreads) {
      if (kpm_row[i] != 0) {
        lo = min(lo, i);
        hi_ = max(hi_, i);
        ++cnt;
      }
    }
    for (int off = 32; off > 0; off >>= 1) {
      lo = min(lo, __shfl_xor(lo, off, 64));
      hi_ = max(hi_, __shfl_xor(hi_, off, 64));
      cnt += __shfl_xor(cnt, off, 64);
    }
    int* red = reinterpret_cast<int*>(smem);   // no tile has been copied yet
    if (lane == 0) {
      red[3 * wave] = lo;
      red[3 * wave + 1] = hi_;
      red[3 * wave + 2] = cnt;
    }
    __syncthreads();
    lo = Nk;
    hi_ = -1;
    cnt = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      lo = min(lo, red[3 * w]);
      hi_ = max(hi_, red[3 * w + 1]);
      cnt += red[3 * w + 2];
    }
    __syncthreads();   // before the tile copies reuse the LDS
    kv_lo = lo;
    kv_hi = hi_;
    kv_run = cnt == hi_ - lo + 1;
    if (hi_ < lo || q0 > hi_ || q0 + kBR - 1 < lo) {
      kt_end = kt0;    // no valid key, or no valid query in this tile
    } else {
      kt0 = max(kt0, lo / BC);
      kt_end = min(kt_end, hi_ / BC + 1);
    }
  }

  // ---- Q rows of this lane, kept in VGPRs ----
  const int qw0 = q0 + wave * 32;        // first query row of this wavefront
  const int qrow = qw0 + l32;            // this lane's query row
  // (With a padding mask, a wave whose rows all lie outside the valid span
  // has only padding rows: it skips the work and writes zeros.)
  const bool wave_has_rows = qw0 < Nq && (!KPM || (qw0 <= kv_hi && qw0 + 31 >= kv_lo));
  // First and last key tiles with a visible key for some row of this wavefront.
  int wave_first_kt = 0;
  int wave_last_kt = CAUSAL ? min(n_kt - 1, (qw0 + 31) / BC) : n_kt - 1;
  if constexpr (BAND) {
    const int w_lo = max(0, qw0 + band_lo);
    const int w_hi = min(Nk - 1, min(Nq - 1, qw0 + 31) + band_hi);
    wave_first_kt = w_lo / BC;
    wave_last_kt = w_hi >= w_lo ? w_hi / BC : -1;
  }
  // Key padding mask: this batch's row of the mask, and whether this lane's
  // query is a valid token (padding queries write O = 0, L = -inf).
  bool q_valid = true;
  if constexpr (KPM) q_valid = qrow < Nq && kpm_row[qrow] != 0;
  bf16x8 qr[DS];
  if (qrow < Nq) {
    const u32x4* src = reinterpret_cast<const u32x4*>(qg + (int64_t)qrow * q_ts);
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

  // ---- direct HBM -> LDS copies, issued by the waves of group A ----
  // Slot s of a tile (16 bytes at byte 16*s) holds row s / kChunks, logical
  // chunk (s % kChunks) ^ swz(row).
  int cp_row[NPW], k_src[NPW], v_src[NPW];
#pragma unroll
  for (int n = 0; n < NPW; ++n) {
    const int slot = (gw * NPW + n) * 64 + lane;
    const int row = slot / TL::kChunks;
    const int phys = slot % TL::kChunks;
    cp_row[n] = row;
    k_src[n] = row * k_tb + ((phys ^ TL::k_swz(row)) * 16);
    v_src[n] = row * v_tb + ((phys ^ TL::v_swz(row)) * 16);
  }
  auto copy_tile = [&](const uint8_t* gsrc, int tb, const int (&src)[NPW], int tile_base, int kt) __attribute__((always_inline)) {
    const int k0 = kt * BC;
    const uint8_t* g = gsrc + (int64_t)k0 * tb;
    const uint32_t lds0 = smem_lds + tile_base + gw * NPW * 1024;
    if (k0 + BC <= Nk) {
#pragma unroll
      for (int n = 0; n < NPW; ++n) copy16_to_lds(g, (uint32_t)src[n], lds0 + n * 1024);
    } else {
#pragma unroll
      for (int n = 0; n < NPW; ++n) {
        if (k0 + cp_row[n] < Nk) {
          copy16_to_lds(g, (uint32_t)src[n], lds0 + n * 1024);
        } else {
          *reinterpret_cast<u32x4*>(smem + tile_base + (gw * NPW + n) * 1024 + 16 * lane) =
              u32x4{0, 0, 0, 0};
        }
      }
    }
  };
  auto copy_k = [&](int kt) __attribute__((always_inline)) { copy_tile(kg, k_tb, k_src, (kt & 1) * TILE_BYTES, kt); };
  auto copy_v = [&](int kt) __attribute__((always_inline)) { copy_tile(vg, v_tb, v_src, (2 + (kt & 1)) * TILE_BYTES, kt); };

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

  auto lds_b128 = [&](int byte) __attribute__((always_inline)) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(smem + byte);
  };
  auto lds_tr = [&](int byte) __attribute__((always_inline)) -> v4i16 {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)((__attribute__((address_space(3))) uint8_t*)smem + byte));
  };

  // ---- running state (one query row per lane) ----
  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b] = f32x16{};
  float m_run = kNegInf;   // exponent offset, base-2 units of the scaled score
  float l_run = 0.f;       // running sum over this lane's half of the keys
  f32x16 s[KB];            // S^T of the current tile
  bf16x8 pb[KB][2];        // P~ of the previous tile, as MFMA B operands

  // S^T = K Q^T for one tile (BC keys x 32 queries).
  auto qk = [&](int kt) __attribute__((always_inline)) {
    const int base = (kt & 1) * TILE_BYTES;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {   // alternate accumulators
        const bf16x8 a = lds_b128(base + 32 * kb * RB + k_rd[ds]);
        s[kb] = mfma32<F16>(a, qr[ds], s[kb]);
      }
    }
  };
  // O^T += V^T P^T for one tile.
  auto pv = [&](int kt) __attribute__((always_inline)) {
    const int base = (2 + (kt & 1)) * TILE_BYTES;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int b = 0; b < DB; ++b) {   // alternate accumulators
          const int r0 = (32 * kb + 16 * t) * RB;
          const v4i16 lo = lds_tr(base + r0 + v_rd[b]);
          const v4i16 up = lds_tr(base + r0 + 8 * RB + v_rd[b]);
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
          o[b] = mfma32<F16>(a, pb[kb][t], o[b]);
        }
      }
    }
  };

  // M phase with both products: the KB*DS QK^T MFMAs of tile kt, then the
  // DB*KB*2 P V MFMAs of tile kt-1. Each product walks its accumulators in
  // turn (S^T: KB blocks, O^T: DB blocks), so consecutive MFMAs never depend
  // on each other. One register ring of kPrefetch operand fragments runs
  // over both products, read from LDS that many MFMAs ahead, and
  // sched_barrier keeps that order, so the MFMAs issue back to back instead
  // of each waiting for its LDS read. (Measured on gfx950: this order with an
  // 8-deep ring beats alternating QK and PV MFMAs with two 4-deep rings, at
  // the same register count.) `between` runs after the ring's first reads
  // are issued and before the first MFMA (group A issues its HBM -> LDS
  // copies there, which hides the first reads' latency behind them).
  auto qk_pv = [&](int kt, auto&& between) __attribute__((always_inline)) {
    constexpr int N = KB * DS;                   // MFMAs per product
    static_assert(N == DB * KB * 2, "both products have the same length");
    // Causal d = 128 has registers to spare (221 of 256 with 8): a 16-deep
    // ring there (253, no spills) measured +1.9 % on the causal prefill shape.
    constexpr int PF = CAUSAL && D == 128 ? 2 * kPrefetch : kPrefetch;
    constexpr int R = 2 * N < PF ? 2 * N : PF;
    const int kbase = (kt & 1) * TILE_BYTES;
    const int vbase = (2 + ((kt - 1) & 1)) * TILE_BYTES;
    auto frag = [&](int i) __attribute__((always_inline)) -> bf16x8 {
      if (i < N) {   // K fragment of QK^T step i
        const int ds = i / KB, kb = i % KB;
        return lds_b128(kbase + 32 * kb * RB + k_rd[ds]);
      }
      const int ii = i - N, b = ii % DB, c = ii / DB, kb2 = c / 2, t = c % 2;
      const int r0 = (32 * kb2 + 16 * t) * RB;   // V^T fragment of PV step ii
      const v4i16 lo = lds_tr(vbase + r0 + v_rd[b]);
      const v4i16 up = lds_tr(vbase + r0 + 8 * RB + v_rd[b]);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 ring[R];
#pragma unroll
    for (int i = 0; i < R; ++i) ring[i] = frag(i);
    __builtin_amdgcn_sched_barrier(0);
    between();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2 * N; ++i) {
      if (i < N) {
        const int ds = i / KB, kb = i % KB;
        s[kb] = mfma32<F16>(ring[i % R], qr[ds], s[kb]);
      } else {
        const int ii = i - N, b = ii % DB, c = ii / DB, kb2 = c / 2, t = c % 2;
        o[b] = mfma32<F16>(ring[i % R], pb[kb2][t], o[b]);
      }
      if (i + R < 2 * N) ring[i % R] = frag(i + R);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // P~ = exp2(S^T scale_log2 - m) of one tile into the MFMA operands pb,
  // returning this lane's sum of P~ (masked tiles: s already scaled, masked
  // scores -inf).
  auto exps = [&](auto masked_tag, float neg_m) __attribute__((always_inline)) -> float {
    constexpr bool masked = decltype(masked_tag)::value;
    float sum = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 8 * t + 2 * i;
          float x0, x1;
          if constexpr (masked) {
            x0 = s[kb][r] + neg_m;
            x1 = s[kb][r + 1] + neg_m;
          } else {
            x0 = __builtin_fmaf(s[kb][r], s2, neg_m);
            x1 = __builtin_fmaf(s[kb][r + 1], s2, neg_m);
          }
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

  // Online softmax of one tile: s -> pb, updating m_run, l_run and (rarely) o.
  // Instantiated separately for tiles that need the mask and tiles that do
  // not, so the common path carries no per-element selects.
  auto softmax_tile = [&](auto masked_tag, int k0, uint32_t kvalid) __attribute__((always_inline)) {
    constexpr bool masked = decltype(masked_tag)::value;
    float mt = kNegInf;
    if constexpr (masked) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          bool ok = key < Nk && (!CAUSAL || key <= qrow);
          if constexpr (BAND) ok = ok && key >= qrow + band_lo && key <= qrow + band_hi;
          if constexpr (KPM) ok = ok && ((kvalid >> (16 * kb + r)) & 1);
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
      // Keep this a real (wave-uniform) branch: if the compiler speculates
      // it into selects, every tile pays the multiply of the accumulator.
      asm volatile("" ::: "memory");
      const float m_new = fmaxf(m_run, mt);
      // A band row that still sees no key has m_run = m_new = -inf; its
      // state is all zeros and stays so (alpha 1 instead of exp2(NaN)).
      const float alpha = (EMPTY_ROWS && m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] *= alpha;
      m_run = m_new;
    }
    // A row that has seen no key yet (band only) keeps m = -inf; its
    // exponentials are of -inf and must come out 0, not NaN.
    const float neg_m = (EMPTY_ROWS && m_run == kNegInf) ? 0.f : -m_run;
    l_run += exps(masked_tag, neg_m);
  };

  // Softmax of a full unmasked tile in the steady loop, without the row
  // maximum. The exponentials are taken against the current offset m_run
  // straight away; the lane's sum of the tile's P~ then bounds every one of
  // its terms (they are non-negative), so a sum of at most 2^kRescaleTau
  // proves that no P~ of the lane exceeds 2^kRescaleTau, which is all the
  // deferred rescale guarantees. Only when some lane's sum is larger (or not
  // a number) does the wave take the full path above: the row maximum, the
  // rescale if the maximum moved by more than kRescaleTau, and the
  // exponentials again. Once a row's offset is set this happens on a
  // vanishing fraction of tiles, and the common tile saves the maximum's
  // 16 v_max3, the exchange and the compare.
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
      // A real branch, not selects; m_run made opaque, or the compiler keeps
      // the exponentials above alive to reuse them below.
      asm volatile("" : "+v"(m_run) : : "memory");
      float mt = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) mt = max3(mt, s[kb][r], s[kb][r + 1]);
      }
      mt = max_xor32(mt * s2);
      // The offset moves to the row maximum (alpha = 1 if it did not grow).
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

  // Key padding mask of a tile: lane l reads the byte of key 64 kt + l, and a
  // ballot gives the wave the tile's 64 validity bits. The byte of the wave's
  // next tile is loaded one softmax ahead, so its latency hides behind a tile.
  int kpm_kt = -1;
  bool kpm_next = false;
  auto kpm_byte = [&](int kt) __attribute__((always_inline)) -> bool {
    const int key = kt * BC + lane;
    return key < Nk && kpm_row[key] != 0;
  };
  // The 32 keys of a lane are the 4-key groups 8 g + 4 (l/32) + 0..3 of the
  // tile (g = 0..7); their validity bits are gathered once per tile from the
  // wave's 64 bits (scalar code), key 32 kb + 8 (r/4) + 4 (l/32) + r%4 of
  // register r in block kb landing at bit 16 kb + r.
  auto lane_bits = [&](uint64_t kbits) __attribute__((always_inline)) -> uint32_t {
    auto gather = [](uint64_t x) -> uint32_t {   // nibble 2n of x -> nibble n
      x &= 0x0F0F0F0F0F0F0F0Full;
      x = (x | (x >> 4)) & 0x00FF00FF00FF00FFull;
      x = (x | (x >> 8)) & 0x0000FFFF0000FFFFull;
      return (uint32_t)(x | (x >> 16));
    };
    const uint32_t even = gather(kbits), odd = gather(kbits >> 4);
    return hi ? odd : even;
  };
  auto softmax = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kt * BC;
    uint64_t kbits = ~0ull;
    if constexpr (KPM) {
      const bool cur = kpm_kt == kt ? kpm_next : kpm_byte(kt);
      kpm_next = kpm_byte(kt + 1);
      kpm_kt = kt + 1;
      kbits = __builtin_amdgcn_ballot_w64(cur);
    }
    if ((k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > qw0) ||
        (BAND && (k0 < qw0 + 31 + band_lo || k0 + BC - 1 > qw0 + band_hi)) ||
        (KPM && kbits != ~0ull))
      softmax_tile(std::true_type{}, k0, KPM ? lane_bits(kbits) : 0u);
    else
      softmax_tile(std::false_type{}, k0, 0u);
  };

  auto active = [&](int kt) __attribute__((always_inline)) {
    return wave_has_rows && kt <= wave_last_kt && (!BAND || kt >= wave_first_kt);
  };

  // ---- schedule ----
  // One workgroup barrier per key tile. In period j (between barriers j-1
  // and j):
  //   group A: copies K(j+1), V(j); M_j = [S^T_j, O^T += V^T_{j-1} P_{j-1}];
  //            V_j = softmax of tile j; waits for its copies;
  //   group B: V_{j-1} = softmax of tile j-1; M_j.
  // On every SIMD one wave starts with MFMAs while the other starts with
  // exponentials, and the two then swap, with no barrier in between.
  // LDS buffers: K_t in K buf t&1, V_t in V buf t&1. The buffers written in
  // period j held K_{j-1} and V_{j-2}, last read in period j-1; the copies
  // land (s_waitcnt by the issuing waves) before barrier j, ahead of their
  // first readers in period j+1.
  auto mfma_phase = [&](int j) __attribute__((always_inline)) {
    const bool do_qk = j < kt_end && active(j);
    const bool do_pv = j > kt0 && active(j - 1);
    if (do_qk && do_pv) {
      qk_pv(j, [] {});
    } else {
      if (do_qk) qk(j);
      if (do_pv) pv(j - 1);
    }
  };
  // Steady periods: j in [1, j_steady) where, for every wavefront of the
  // workgroup, tiles j-1 and j are full, unmasked and active, and K(j+1) is a
  // full tile. They run without any of the per-tile tests. The bound is the
  // same in every wave, so all waves cross the same barriers.
  const int full_kt = Nk / BC;                         // tiles with BC keys
  const int unmasked_kt = CAUSAL ? min(full_kt, q0 / BC) : full_kt;
  // Steady periods are [js0, js1); the first tile's period and the ones
  // after js1 take the general path.
  int js0 = 1;
  int js1 = (q0 + kBR <= Nq) ? max(1, min(unmasked_kt, full_kt - 1)) : 1;
  if constexpr (BAND) {
    // Tiles every row of the workgroup sees in full: keys from the last
    // row's lower bound to the first row's upper bound.
    js0 = kt0 + 1;
    js1 = js0;
    if (q0 + kBR <= Nq) {
      const int t_a = (max(0, q0 + kBR - 1 + band_lo) + BC - 1) / BC;
      const int t_b = (q0 + band_hi + 1) / BC - 1;
      js0 = max(js0, t_a + 1);
      js1 = max(js0, min(min(t_b, full_kt - 2), kt_end - 2) + 1);
    }
  }
  if constexpr (KPM) {
    // Steady periods only when the valid tokens form one run and this query
    // tile lies inside it (every wave active): then tiles whose keys all lie
    // in the run need no mask. Otherwise every period takes the general path.
    js0 = kt0 + 1;
    js1 = js0;
    if (kv_run && q0 >= kv_lo && q0 + kBR - 1 <= kv_hi) {
      const int t_a = (kv_lo + BC - 1) / BC;   // first tile with all keys valid
      const int t_b = (kv_hi + 1) / BC - 1;    // last one
      js0 = max(js0, t_a + 1);
      js1 = max(js0, min(min(t_b, unmasked_kt - 1), min(full_kt - 2, kt_end - 2)) + 1);
    }
  }
  auto period = [&](int j) __attribute__((always_inline)) {
    stress_pause(4 * j);
    if (!group_b) {
      if (j < kt_end) {
        if (j + 1 < kt_end) copy_k(j + 1);
        copy_v(j);
      }
      mfma_phase(j);
      stress_pause(4 * j + 1);
      if (j < kt_end && active(j)) softmax(j);
      stress_pause(4 * j + 2);
      __builtin_amdgcn_s_waitcnt(0);   // this period's copies have landed
    } else {
      if (j > kt0 && active(j - 1)) softmax(j - 1);
      stress_pause(4 * j + 1);
      mfma_phase(j);
    }
    stress_pause(4 * j + 3);
    barrier_nofence();
  };
  if (kt0 < kt_end) {   // a band can leave a workgroup without any key
    if (!group_b) copy_k(kt0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int j = kt0; j < js0; ++j) period(j);
    for (int j = js0; j < js1; ++j) {
      stress_pause(4 * j);
      if (!group_b) {
        const uint8_t* gk = kg + (int64_t)((j + 1) * BC) * k_tb;
        const uint8_t* gv = vg + (int64_t)(j * BC) * v_tb;
        const uint32_t lk = smem_lds + ((j + 1) & 1) * TILE_BYTES + gw * NPW * 1024;
        const uint32_t lv = smem_lds + (2 + (j & 1)) * TILE_BYTES + gw * NPW * 1024;
        qk_pv(j, [&]() __attribute__((always_inline)) {
#pragma unroll
          for (int n = 0; n < NPW; ++n) copy16_to_lds(gk, (uint32_t)k_src[n], lk + n * 1024);
#pragma unroll
          for (int n = 0; n < NPW; ++n) copy16_to_lds(gv, (uint32_t)v_src[n], lv + n * 1024);
        });
        stress_pause(4 * j + 1);
        softmax_lazy();
        stress_pause(4 * j + 2);
        __builtin_amdgcn_s_waitcnt(0);   // this period's copies have landed
      } else {
        softmax_lazy();
        stress_pause(4 * j + 1);
        qk_pv(j, [] {});
      }
      stress_pause(4 * j + 3);
      barrier_nofence();
    }
    for (int j = js1; j <= kt_end; ++j) period(j);
  }

  // ---- epilogue: O = O_acc / l, L = ln2 * (m + log2 l) ----
  // O goes out through LDS (store_tileT), each wave using its own 32 * 2D
  // bytes of the K/V buffers, free once every wave has crossed the last
  // barrier (a workgroup without key tiles never wrote them).
  const float l_tot = l_run + xor32(l_run);
  const bool empty = (EMPTY_ROWS && l_tot == 0.f) || !q_valid;
  const float inv = empty ? 0.f : __builtin_amdgcn_rcpf(l_tot);
  store_tileT<D, F16>(p.o + o_off + (int64_t)qw0 * o_ts, o_ts, min(32, Nq - qw0), o, inv,
                      smem + wave * 64 * D, lane);
  if (qrow < Nq && hi == 0)
    p.lse[l_off + qrow] = empty ? kNegInf : (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

}  // namespace fa
