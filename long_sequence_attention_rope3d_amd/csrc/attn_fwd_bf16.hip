// attn_fwd_bf16.hip — blockwise joint-sequence attention on gfx950 bf16 MFMA.
//
// Computes, per (b, h, query row), softmax(scale * q K^T) V over all Skv keys,
// non-causal ("Context Parallelism in vLLM Omni Neuron", §Self-Attention:
// _nf_attend(query, key, value, scale); §Overview: full attention is kept
// while the sequence is split).  Keys are visited in chunks of kv_chunk keys,
// the single-device form of ring attention's one-K/V-shard-per-round loop
// (§Ring attention):
//   * inside a chunk: online softmax over 32-key steps (running max m,
//     running sum l, accumulator acc rescaled by 2^(m_old - m_new));
//   * across chunks, the log-sum-exp merge of the chunk partial
//     (O_c, lse_c) = (acc_c / l_c, m_c + log2 l_c) into the running result
//       L' = log2(2^L + 2^lse_c),  O' = O 2^(L - L') + O_c 2^(lse_c - L'),
//     done in the accumulator itself: at a chunk end acc is normalised to
//     (O, L) = (acc / l, m + log2 l) and the next chunk starts from acc = O,
//     m = L, l = 1, i.e. the running result enters as value O at weight 2^L.
//     The chunk's online rescale then produces exactly O' and L' (the
//     formula above with both weights over the common normaliser), without a
//     second 64-register accumulator.  Nothing partial is written to memory
//     (§Memory and Compute Benefits: the split keeps full attention quality).
// The softmax runs in the log2 domain: logits are multiplied by
// c = |scale| * log2(e) inside one FMA, so p = 2^(s*c - m).
// A launch whose last round of blocks would leave many CUs idle can also
// split the keys of that round's query tiles into ranges of whole chunks run
// by separate blocks; each then writes its fp32 partial (O, lse) and the
// ranges are combined by the same log-sum-exp merge in a second kernel
// (lse_merge.hip) -- ring attention's per-shard partials, with the shards as
// blocks of one launch.
//
// Mapping onto CDNA4
// ------------------
// * Block = 12 waves = 384 query rows (32 per wave), one block per CU, i.e.
//   three waves per SIMD: while one wave of a SIMD runs its softmax on the
//   VALU or waits on LDS, the others keep the matrix core busy.  That caps a
//   wave at 168 registers (the kernel needs 160 and spills nothing).  384
//   also divides the 52608-token workload exactly, and 137 query tiles per
//   head keep the last round of blocks on the CUs nearly full.  A grid of
//   few query tiles (fewer than the CUs) may instead take blocks of 8 waves =
//   256 rows, two waves per SIMD (up to 256 registers): 10% slower per CU,
//   but more of the CUs busy (the same kernel, instantiated for 8 waves).
// * Grid = one block per query tile (B*H*ceil(Sq/384) tiles), plus n_split
//   blocks per tile of a split last round in place of one; re-numbered so
//   consecutive query tiles over the same keys land on the same XCD
//   (hardware hands block i to XCD i % 8): the CUs of an XCD stream the same
//   K/V and share it in that XCD's L2.
// * K/V tiles of kBN = 128 keys are copied global -> LDS by DMA
//   (global_load_lds_dwordx4) into two stage buffers, row-major [key][d],
//   with the 16-byte chunks of every row XOR-swizzled so that the operand
//   reads served in one LDS cycle (16 lanes x 16 B for K, a 16-lane
//   transpose group for V) fall into distinct banks (choices measured with
//   the LDS bank-conflict counter).
// * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K rows (ds_read_b128),
//   B = Q^T (kept in VGPRs for the whole block).  The accumulator holds, in
//   lane l, 16 keys of query column l%32, so each lane owns one query row:
//   the row max needs one v_permlane32_swap, the row sum none until the end
//   of a chunk.
// * K rows are fed to the MFMA in the permuted order pi (bits 2 and 3 of the
//   row index swapped) so accumulator element i of lane-half hf holds key
//   16*(i/8) + 8*hf + i%8: eight consecutive keys per half — exactly the
//   B-operand fragment of the PV product, so P goes from the S^T accumulator
//   to the PV MFMA in registers (packed fp32 -> bf16 convert).
// * O^T = V^T P^T: A = V^T, read from the row-major V tile with
//   ds_read_b64_tr_b16 (in each 16-lane group, lane i receives element i%4
//   of the rows addressed by lanes 4k + i/4, k = 0..3 — a 4x16 transpose of
//   b16 values), two reads per 8-key fragment.  The O^T accumulator again
//   holds one query per lane, so rescales and the chunk merge are per-lane
//   scalars.
// * Rescale only on a new maximum: when the row max is formed, the reference
//   moves to it as soon as a step's max exceeds it (no lazy margin), so a
//   row's largest logit gets p = 2^0 = 1 (2^-off with an offset), exact in bf16, and a row dominated by one
//   key carries no rounding of that key's weight; steps whose max does not
//   exceed the reference skip the 64-register rescale of acc.  (A lazy
//   threshold of 8 was no faster and doubled the worst output error on rows
//   dominated by one outlier key.)
// * Bound-gated max: the row max itself is only formed while some row of the
//   wave has a Cauchy-Schwarz logit bound more than the head's slack above
//   its reference (see the kernel's comment); on typical inputs that is the
//   first step, and later steps spend no VALU work on the max at all.
// * The row sum l adds the fp32 p before their bf16 rounding for the PV
//   product, so lse keeps fp32 accuracy.
// * Issue priority: every wave keeps the default priority.  Raising it
//   while a wave issues its MFMAs once paid 1%, but with the VALU trimmed as
//   it is now it costs 0.5% (52k and long-video alike).
#include <algorithm>
#include <type_traits>

#include "launch.h"

namespace r3d {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Block shape: kWaves waves of 32 query rows; kStages K/V stage buffers in
// LDS (prefetch distance kStages - 1 tiles).
#ifndef R3D_ATTN_WAVES
#define R3D_ATTN_WAVES 12
#endif
#ifndef R3D_ATTN_STAGES
#define R3D_ATTN_STAGES 2
#endif
constexpr int kWaves = R3D_ATTN_WAVES;  // the block of every launch but small grids'
constexpr int kWavesSmall = 8;          // the block a grid of few query tiles may take instead
constexpr int kStages = R3D_ATTN_STAGES;
// Block of W waves: 64 W threads, 32 W query rows, W / 4 waves per SIMD (one
// block per CU).
template <int W>
struct Blk {
  static_assert(W % 4 == 0, "whole waves per SIMD");
  static constexpr int kThreads = 64 * W;
  static constexpr int kBM = 32 * W;  // query rows per block
  static constexpr int kWavesPerSimd = W / 4;
};
static_assert(kAttnMaxSeq + Blk<kWaves>::kBM <= INT32_MAX, "query rows fit in 32 bits");
static_assert(kAttnMaxSeq + Blk<kWavesSmall>::kBM <= INT32_MAX, "query rows fit in 32 bits");
static_assert(kStages == 2 || kStages == 3, "2 or 3 stages");
#ifndef R3D_ATTN_BN
#define R3D_ATTN_BN 128
#endif
constexpr int kBN = R3D_ATTN_BN;  // keys per LDS tile (a multiple of 32)
static_assert(kAttnMaxSeq + kBN <= INT32_MAX, "key cursor fits in 32 bits");
constexpr int kSub = kBN / 32;   // 32-key softmax steps per tile
constexpr int kXcds = 8;
constexpr int kSlackMax = 32;     // largest bound slack under which the row max is skipped, log2 units

template <int D, int W>
struct Geom {
  static constexpr int kSteps = D / 16;               // MFMA k-steps of Q K^T
  static constexpr int kDBlk = D / 32;                // 32-wide d blocks of O^T
  static constexpr int kCpr = D / 8;                  // 16-byte chunks per K/V row
  static constexpr int kTile = kBN * D;               // elements of one K or V tile
  static constexpr int kDma = kBN * kCpr / 64;         // 1 KB DMA instructions per tensor per tile
  static constexpr int kDmaPerWave = (kDma + W - 1) / W;  // the last may be partial
  static_assert(kDma >= W, "every wave copies");
  // With a tile left in flight across the barrier (3 stages) every wave must
  // issue the same number of copies for its vmcnt wait to cover the older tile.
  static_assert(kStages == 2 || kDma % W == 0, "uneven copy split needs 2 stages");
};

// Per-row XOR swizzles of the 16-byte chunk index (see the bank notes above).
template <int D>
constexpr __device__ __host__ int swz_k(int r) {
  // ds_read_b128 is served 16 lanes (256 bytes) per LDS cycle; the 16 lanes of
  // a group read 16 different rows at the same logical chunk.
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
constexpr __device__ __host__ int swz_v(int r) {
  // ds_read_b64_tr_b16: a 16-lane group reads 4 consecutive rows x 32 bytes.
  return D == 128 ? 4 * (r & 3) : 2 * (r & 3);
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_u32(const uint16_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// True if the swizzle of row r equals that of row r + step for every row of a tile.
template <int D, bool IS_V>
constexpr bool swz_periodic(int step) {
  for (int r = 0; r < 256; ++r)
    if ((IS_V ? swz_v<D>(r) : swz_k<D>(r)) != (IS_V ? swz_v<D>(r + step) : swz_k<D>(r + step))) return false;
  return true;
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 (a in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Maximum that propagates NaN (IEEE 754-2019 maximum): one v_maximum3_f32
// per two new operands, with no quieting of the inputs first (fmaxf's
// maxNum needs a canonicalising v_max x, x per operand).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// x of this lane combined with x of lane l^32.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// MFMA row m of the S^T product reads tile key pi(m): bits 2 and 3 swapped.
__device__ __forceinline__ int key_of_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Walks the key tiles in order: tiles of kBN keys inside chunks of `chunk`
// keys (the last tile of a chunk may be short), advanced by additions only.
// Key indices are 32-bit (the host keeps Sq and Skv within kAttnMaxSeq): the
// tile bookkeeping then stays on the scalar unit, where 64-bit compares
// would each cost vector instructions (gfx9 has no scalar 64-bit less-than),
// and the cursor never overflows (every sum below is bounded by Skv + kBN).
struct TileCursor {
  int kv0;   // first key of the tile
  int cend;  // end of the tile's chunk
  __device__ __forceinline__ int n() const { return (cend - kv0 > kBN) ? kBN : cend - kv0; }
  __device__ __forceinline__ void advance(int chunk, int Skv) {
    kv0 += kBN;
    if (kv0 >= cend) {
      kv0 = cend;
      cend = (Skv - cend > chunk) ? cend + chunk : Skv;
    }
  }
};

// Direct global -> LDS copy of one K or V tile into the LDS bytes at
// lds_tile, as kDma wave-instructions of 64 x 16 bytes; `src` points at the
// tile's first key row and n of its rows are valid.  global_load_lds_dwordx4
// writes lane L's 16 bytes to (M0 + 16*L), so the swizzle is realised by
// choosing, per lane, which global chunk lands in its slot: slot s = 64*m + L
// holds row s / kCpr, logical chunk (s % kCpr) ^ swz(row).  Rows past n
// re-read the last valid row (in bounds); their logits are masked and their
// p is exactly zero.  kFull: n == kBN, no clamp.  The global address is the
// wave-uniform tile base (SGPRs) plus a 32-bit per-lane byte offset.
//
// The copy is issued from inline assembly on purpose: the compiler's own
// wait-count insertion cannot prove that the LDS reads of the stage being
// consumed are independent of the copy in flight into another stage, and
// puts a full vmcnt(0) wait after every prefetch, exposing the whole copy
// latency on each tile.  Hidden from it, the copies are ordered only by the
// explicit waits in wait_vm_barrier (every read of a stage follows the wait
// + barrier that retire that stage's copies).  The compiler's own vmcnt waits
// (the Q loads) only become stricter by the extra operations in the counter.
// One wait state separates the M0 write from the DMA.
template <int D, int W, bool IS_V, bool kFull>
__device__ __forceinline__ void dma_tile(uint32_t lds_tile, const uint16_t* src, int n, int wave, int lane) {
  using G = Geom<D, W>;
  // Instruction i of a wave covers slots 64*(wave + W*i) + [0, 64): rows
  // r0 + kRowStep*i.  The swizzles depend on row bits that kRowStep leaves
  // unchanged, so the chunk (and for full tiles the whole per-lane offset) is
  // the same for every i; instruction i adds kRowStep rows (8 KB) to the
  // wave-uniform global base and to M0.
  constexpr int kRowStep = 64 * W / G::kCpr;
  static_assert(swz_periodic<D, IS_V>(kRowStep), "swizzle must be invariant under a step of kRowStep rows");
  const int r0 = (64 * wave + lane) / G::kCpr;
  const int cl = (lane % G::kCpr) ^ (IS_V ? swz_v<D>(r0) : swz_k<D>(r0));
#pragma unroll
  for (int i = 0; i < G::kDmaPerWave; ++i) {
    if (G::kDma % W != 0 && wave + W * i >= G::kDma) break;  // wave-uniform
    // Full tile: base advanced by i*kRowStep rows, offset of row r0.  Short
    // tile: base at the tile, offset of the clamped absolute row.  Either way
    // the unsigned 32-bit offset is the in-bounds row's distance from base.
    const int r = r0 + kRowStep * i;
    const int row = kFull ? r0 : (r < n ? r : n - 1);
    const uint32_t off = (uint32_t)(row * D + cl * 8) * 2u;
    const uint16_t* const src_i = kFull ? src + (int64_t)kRowStep * i * D : src;
    // Both are wave-uniform; readfirstlane pins them to SGPRs, which the
    // asm operands require (the compiler would otherwise hand over a VGPR).
    const uint64_t b64 = reinterpret_cast<uint64_t>(src_i);
    // (readfirstlane returns int: go through uint32_t so nothing sign-extends.)
    const uint32_t b_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b64);
    const uint32_t b_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b64 >> 32));
    const uint64_t base = (uint64_t)b_lo | ((uint64_t)b_hi << 32);
    const uint32_t lds =
        (uint32_t)__builtin_amdgcn_readfirstlane((int)(lds_tile + (uint32_t)((wave + W * i) * 64 * 16)));
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
  }
}

// Wait until at most N of this wave's vector-memory operations (here: LDS
// DMAs) are outstanding and all of its LDS reads have returned, then meet the
// other waves at the barrier.  The empty asm with a memory clobber keeps
// memory accesses from being moved across the barrier.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  // s_waitcnt immediate: vmcnt[3:0] in bits 3:0, expcnt (7 = no wait) in
  // 6:4, lgkmcnt (0) in 11:8, vmcnt[5:4] in 15:14.
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Both variants read the head statistics of the pre-pass: max_j |k_j|^2,
// which gives each row the Cauchy-Schwarz bound bnd = c |q_i| max_j |k_j| >=
// every logit of the row (log2 units), and max_j |v_j| over all elements.
//
// Online (kConstMax false): the reference m is an attained value -- a step's
// row max (plus the offset below), or a chunk's log-sum-exp after the merge --
// as in the plain online softmax, but the 16-element row max is only formed
// while bnd > m + slack for some row of the wave.  Once m is within `slack`
// of the bound, no later logit can exceed it by more than that, so
// p = 2^(s c - m) <= 2^slack without looking at the step's values; only rows
// whose bound is loose (or the first step, m = -inf) pay for the max.
// The slack is per head: the accumulator sums up to chunk + 1 terms of
// p |v| (the chunk's keys and the carried result), so the slack is capped
// at E = 126 - ceil(log2(chunk + 1)) - floor(log2(max |v|)), which keeps
// |acc| below 2^127 (fp32 ends at 2^128): min(32, E).  Where even p <= 1
// would not (E < 0: |v| near the top of bf16's range), the reference is held
// `off` = -E above the row's max -- a moved reference is max + off, a carried
// chunk result enters at weight 2^-off -- so every p <= 2^E.  For ordinary
// inputs E >= 32 and off = 0.  Either way the reference only sets the scale
// of acc and l: the result is the online softmax's for every finite input up
// to the bf16 rounding of p (a key above a skipped max enters with p > 1,
// rounded like any p, where the online softmax gives it exactly 1), without
// its overflow for very large V.
//
// kConstMax: the reference is the bound itself, fixed before any key is read:
// no max reduction, no rescale, and chunk partials simply add.  Exact as long
// as the bound exceeds the row's true max by less than fp32's exponent range
// (about 87 in natural-log units); each wave flags, per block tile, rows whose
// row sum fell below 2^-100 or whose output is not finite, and a second
// launch of the online kernel (fix_flags) recomputes exactly those tiles.
template <int D, bool kConstMax, int W>
__global__ __launch_bounds__(Blk<W>::kThreads, Blk<W>::kWavesPerSimd) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    void* __restrict__ out, float* __restrict__ lse, int64_t H, int64_t Sq, int64_t Skv, float c,
    uint32_t qsign, int64_t chunk, int n_qt, int n_tiles, int n_bulk, int out_bshd, const float* __restrict__ stats,
    int n_split, int64_t split_len, float* __restrict__ o_parts, float* __restrict__ l_parts, int64_t tail_row0,
    int chunk_bits, int* __restrict__ flags_out, const int* __restrict__ fix_flags) {
  using G = Geom<D, W>;
  constexpr int kBM = Blk<W>::kBM;
  // K/V stage buffers (the third only with kStages == 3).
  // K/V stage buffers in one array, K stages first: [K_0 .. K_{kStages-1} | V_0 .. V_{kStages-1}].
  // A DS instruction's immediate offset has 16 bits, so every operand read
  // must reach its byte with a constant below 64 KB: K reads add at most
  // (kStages-1) tiles + 3 steps to their lane offset, and V reads carry the V
  // region's start inside their per-lane base registers (see v_base), so
  // neither needs an address instruction per read.
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * kStages * G::kTile];
  static_assert((kStages - 1) * G::kTile * 2 + kBN * G::kCpr * 16 <= 65536, "K reads within the DS offset");

  // Block -> work.  Query tiles are numbered head-major (logical tile =
  // bh * n_qt + qt).  Blocks [0, n_bulk) run tiles [0, n_bulk) over all keys;
  // the blocks after them run each remaining tile n_split times, once per
  // key range (split), as pieces whose fp32 partials an lse_merge combines.
  // Within each group, XCD x runs indices [x*per + min(x, rem), ...), so that
  // consecutive indices -- consecutive query tiles over the same keys -- share
  // an XCD's L2 (hardware hands block i to XCD i % 8).
  const int bid = blockIdx.x;
  const bool piece = bid >= n_bulk;
  const int n_tail = n_tiles - n_bulk;
  const int nb = piece ? n_tail * n_split : n_bulk;
  const int b0 = piece ? bid - n_bulk : bid;
  const int per = nb / kXcds, rem = nb % kXcds;
  const int xcd = b0 % kXcds, slot = b0 / kXcds;
  const int idx = xcd * per + (xcd < rem ? xcd : rem) + slot;
  const int split = piece ? idx / n_tail : -1;
  const int logical = piece ? n_bulk + (idx - split * n_tail) : idx;
  const int64_t bh = logical / n_qt;
  const int qt = logical - (int)bh * n_qt;
  // This block's keys: [kv_begin, kv_end), the whole sequence or one range
  // of split_len keys (a whole number of chunks, or with one chunk of tiles).
  const int skv = (int)Skv;
  const int chunk32 = (int)(chunk < Skv ? chunk : Skv);
  const int kv_begin = piece ? split * (int)split_len : 0;
  const int kv_end = (piece && skv - kv_begin > (int)split_len) ? kv_begin + (int)split_len : skv;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int r32 = lane & 31, hf = lane >> 5;
  // Recompute pass after the constant-max kernel: only tiles that some wave
  // flagged.  Every wave reads the same flags, so the whole block leaves
  // together, before its first barrier.
  if (!kConstMax && fix_flags) {
    const int f = lane < W ? fix_flags[(int64_t)logical * W + lane] : 0;
    if (__ballot(f != 0) == 0) return;
  }
  const int qrow = qt * kBM + wave * 32 + r32;  // < Sq + kBM <= 2^31
  const int sq = (int)Sq;
  const uint16_t* kb = k + bh * Skv * D;
  const uint16_t* vb = v + bh * Skv * D;

  // Q^T fragments (B operand): query qrow, d = 16*s + 8*hf + [0, 8).  A
  // negative scale is folded into Q by flipping sign bits (exact), so c >= 0.
  bf16x8 qf[G::kSteps];
#pragma unroll
  for (int s = 0; s < G::kSteps; ++s) {
    u32x4 x = u32x4{0, 0, 0, 0};
    if (qrow < sq) x = *reinterpret_cast<const u32x4*>(q + (bh * Sq + qrow) * D + 16 * s + 8 * hf) ^ qsign;
    qf[s] = __builtin_bit_cast(bf16x8, x);
  }

  // Per-lane byte offsets of the MFMA operand reads inside a tile; every
  // other term of the address is a compile-time immediate.
  //  K: row 32*h2 + pi(r32), chunk 2*s + hf (swizzled); the 32-row half h2 adds
  //     32*kCpr*16 bytes (the swizzle of row and row+32 is the same).
  //  V: row 16*sg + 4*rd + 8*hf + (lane&15)/4 (row terms other than the last
  //     two are immediates; the swizzle depends on row&3 only), elements
  //     32*b + 16*((lane>>4)&1) + 4*(lane&3) .. +3.
  int k_base[G::kSteps];
  {
    const int row = key_of_row(r32);
#pragma unroll
    for (int s = 0; s < G::kSteps; ++s) k_base[s] = (row * G::kCpr + ((2 * s + hf) ^ swz_k<D>(row))) * 16;
  }
  int v_base[G::kDBlk];
  {
    const int row = 8 * hf + ((lane & 15) >> 2);
    const int d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int b = 0; b < G::kDBlk; ++b)
    {
      int vb = kStages * G::kTile * 2 + (row * G::kCpr + (((32 * b + d) >> 3) ^ swz_v<D>(row))) * 16 + (d & 7) * 2;
      asm volatile("" : "+v"(vb));  // keep the V region's start in the register, out of the offsets
      v_base[b] = vb;
    }
  }

  f32x16 oacc[G::kDBlk];
#pragma unroll
  for (int b = 0; b < G::kDBlk; ++b) oacc[b] = f32x16{};
  // Running state: acc (oacc), reference m and per-lane partial sum l, log2
  // domain; thr = (m - off) / c, the raw logit above which the reference
  // must move while the row max is being formed (a moved reference is
  // max + off: the reference moves on every new maximum).
  float m_run = -INFINITY, l_run = 0.f, thr = -INFINITY;
  const float inv_c = 1.0f / c;
  // Head statistics: the pre-pass left kStatParts (= 64, one per lane)
  // partial maxima of |k_j|^2 and of |v| per head; a butterfly gives every
  // lane the maxima, made wave-uniform.
  float kmax2, vabs_max;
  {
    static_assert(kStatParts == 64, "one partial per lane");
    float a = stats[bh * kStatParts + lane];
    float b = stats[((int64_t)(n_tiles / n_qt) + bh) * kStatParts + lane];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      a = fmaxf(a, __shfl_xor(a, o));
      b = fmaxf(b, __shfl_xor(b, o));
    }
    kmax2 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a)));
    vabs_max = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(b)));
  }
  // Per-head slack and reference offset (see the kernel's comment):
  // E = 126 - chunk_bits - floor(log2 max|v|), slack = min(32, E),
  // off = max(0, -E); a non-finite V (exponent field 255) keeps the plain
  // online softmax's p <= 1.
  float slack, off, carry;
  {
    const int ex = (int)((__float_as_uint(vabs_max) >> 23) & 0xff);
    int e_max = 126 - chunk_bits - (ex == 0 ? -127 : ex - 127);
    if (ex == 255) e_max = 0;
    slack = (float)(e_max < kSlackMax ? e_max : kSlackMax);
    const int off_i = e_max < 0 ? -e_max : 0;  // <= 128 + 31 - 126 = 33: 2^-off is a normal float
    off = (float)off_i;
    carry = __int_as_float((127 - off_i) << 23);  // 2^-off exactly
  }
  // The row's logit bound: |q_i|^2 from the Q fragments (each lane half holds
  // half of the row) times max_j |k_j|^2.
  float bnd;
  {
    float qq = 0.f;
#pragma unroll
    for (int s = 0; s < G::kSteps; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)qf[s][e];
        qq = fmaf(x, x, qq);
      }
    qq = sum_halves(qq);
    bnd = c * sqrtf(qq * kmax2);
  }
  if constexpr (kConstMax) m_run = bnd;  // the fixed reference
  // Wave-uniform: some row of the wave still needs its row max formed.
  bool need_max = true;
  auto update_need_max = [&]() { need_max = __ballot(bnd > m_run + slack) != 0; };

  const int first_cend = (kv_end - kv_begin > chunk32) ? kv_begin + chunk32 : kv_end;
  // pf: the next tile to prefetch.  Prologue: tiles 0 and 1 in flight, wait for tile 0.
  TileCursor pf{kv_begin, first_cend};
  // Copy tile pf into stage P (K and V), then advance pf.
  auto copy = [&](auto stage) {
    constexpr int P = decltype(stage)::value;
    const int n = pf.n();
    const uint32_t lk = lds_u32(lds + P * G::kTile);
    const uint32_t lv = lds_u32(lds + (kStages + P) * G::kTile);
    const uint16_t* ks = kb + (int64_t)pf.kv0 * D;
    const uint16_t* vs = vb + (int64_t)pf.kv0 * D;
    if (n == kBN) {
      dma_tile<D, W, false, true>(lk, ks, n, wave, lane);
      dma_tile<D, W, true, true>(lv, vs, n, wave, lane);
    } else {
      dma_tile<D, W, false, false>(lk, ks, n, wave, lane);
      dma_tile<D, W, true, false>(lv, vs, n, wave, lane);
    }
    pf.advance(chunk32, kv_end);
  };
  copy(std::integral_constant<int, 0>{});
  if (kStages == 3 && pf.kv0 < kv_end) copy(std::integral_constant<int, 1>{});
  // The prologue tiles target different LDS objects, so their DMAs may be
  // issued in either order: wait for all of them once.
  wait_vm_barrier<0>();

  // One tile of n keys in stage S: prefetch the tile after next into stage
  // (S+2)%3, consume stage S, then wait for the next tile (this wave's part of
  // it) and meet at the barrier.
  TileCursor cur{kv_begin, first_cend};  // the tile being consumed
  auto step = [&](auto stage) {
    constexpr int S = decltype(stage)::value;
    const int n = cur.n();
    const bool chunk_done = cur.kv0 + n == cur.cend;
    const bool issue = pf.kv0 < kv_end;
    if (issue) copy(std::integral_constant<int, (S + kStages - 1) % kStages>{});  // the tile kStages-1 ahead

    const char* kt = reinterpret_cast<const char*>(lds + S * G::kTile);
    char* vt = reinterpret_cast<char*>(lds) + S * G::kTile * 2;  // v_base holds the V region's start
    // 32-key steps, software-pipelined inside the tile: step h's S^T = K Q^T
    // is issued before step h-1's PV product, so the matrix core runs that PV
    // while the same wave computes step h's softmax on the VALU.  In a short
    // tile, steps wholly past n still run: their keys are copies of the last
    // valid key (the DMA clamps the row), which cannot raise the max, and all
    // their p are zeroed.
    u32x4 pw[2];  // P of the step whose PV is pending, as bf16 pairs
#pragma unroll
    for (int h2 = 0; h2 <= kSub; ++h2) {
      f32x16 sacc = f32x16{};
      if (h2 < kSub) {
        // ---- S^T = K Q^T for keys [32*h2, 32*h2 + 32) ----
#pragma unroll
        for (int s = 0; s < G::kSteps; ++s)
          sacc = mfma(*reinterpret_cast<const bf16x8*>(kt + k_base[s] + h2 * 32 * G::kCpr * 16), qf[s], sacc);
      }
      if (h2 > 0) {
        // ---- O^T += V^T P^T for step h2-1: two 16-key steps ----
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          const bf16x8 pf = __builtin_bit_cast(bf16x8, pw[sl]);
          const int sg = 2 * (h2 - 1) + sl;
#pragma unroll
          for (int b = 0; b < G::kDBlk; ++b) {
            char* vp = vt + v_base[b] + 16 * sg * G::kCpr * 16;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp);
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 4 * G::kCpr * 16));
            const s16x4 a4[2] = {lo, hi};
            oacc[b] = mfma(__builtin_bit_cast(bf16x8, a4), pf, oacc[b]);
          }
        }
      }
      if (h2 == kSub) break;

      // ---- online softmax, log2 domain; element i is key 32*h2 + 16*(i/8) + 8*hf + i%8 ----
      // The row max is compared in raw logit units against thr, so the
      // common step (no row moves) spends one compare; only a step in which
      // some row's max exceeds its threshold forms the new reference.
      // A moved reference takes effect at once (m_run is updated here, the
      // factor alpha for acc and l kept for the rescale below), so the common
      // step reads m_run itself and needs no copy of it.
      bool moved = false;  // wave-uniform
      float alpha;  // set (and read) only when the reference moved
      if (!kConstMax && need_max) {
        // This lane's 16 keys first: a half-row above the threshold means its
        // row is above it too, so the cross-half maximum is only formed in
        // the rare step in which some row moves.
        float mx = sacc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = vmax(mx, sacc[i]);
        if (__builtin_expect(__ballot(mx > thr) != 0, 0)) {
          mx = max_halves(mx);
          const bool up = mx > thr;
          const float m_new = up ? fmaf(mx, c, off) : m_run;
          alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 1 where the row kept it, 0 from m = -inf
          m_run = m_new;
          moved = true;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = __builtin_amdgcn_exp2f(fmaf(sacc[i], c, -m_run));
      // Row sum from the unrounded fp32 p (keeps lse at fp32 accuracy).
      float ps = sacc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) ps += sacc[i];
#pragma unroll
      for (int w = 0; w < 8; ++w) pw[w >> 2][w & 3] = pack_bf16(sacc[2 * w], sacc[2 * w + 1]);
      if (n < 32 * (h2 + 1)) {
        // Short tile (rare; kept out of the common block): keys past its end
        // get p = 0 exactly; redo the sum and the packing.
        const int lim = n - 32 * h2 - 8 * hf;  // element i is a real key iff 16*(i/8) + i%8 < lim
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (16 * (i / 8) + (i % 8) >= lim) sacc[i] = 0.f;
        ps = sacc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) ps += sacc[i];
#pragma unroll
        for (int w = 0; w < 8; ++w) pw[w >> 2][w & 3] = pack_bf16(sacc[2 * w], sacc[2 * w + 1]);
      }
      // Rescale last, and only when some row's reference moved (alpha is 0 on
      // a chunk's first step): acc already holds step h2-1's PV (issued above),
      // and step h2's PV comes after.
      if (!kConstMax && moved) {
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < G::kDBlk; ++b) oacc[b] *= alpha;
        thr = (m_run - off) * inv_c;
        update_need_max();
      }
      l_run += ps;
    }

    if (kStages == 3 && issue)
      wait_vm_barrier<2 * G::kDmaPerWave>();  // the tile just issued may stay in flight
    else
      wait_vm_barrier<0>();

    // ---- end of a chunk: log-sum-exp merge ----
    // (acc, m, l) now describe the running result merged with this chunk:
    // normalise to (O, L) = (acc / l, m + log2 l), and let the next chunk
    // start from acc = O, m = L, l = 1 -- value O at weight 2^L.  The next
    // chunk's online rescale then forms exactly O 2^(L - L') + O_c 2^(lse_c - L').
    // (With a reference offset the carried result enters as acc = O 2^-off,
    // l = 2^-off, m = L + off: the same weight 2^L.  The last chunk keeps O, L.)
    if (!kConstMax && chunk_done) {
      const bool last = cur.kv0 + n >= kv_end;
      const float w_carry = last ? 1.0f : carry;
      const float l_tot = sum_halves(l_run);
      const float inv = w_carry / l_tot;
#pragma unroll
      for (int b = 0; b < G::kDBlk; ++b) oacc[b] *= inv;
      m_run += log2f(l_tot);
      if (!last) m_run += off;
      thr = (m_run - off) * inv_c;
      update_need_max();
      l_run = hf == 0 ? w_carry : 0.0f;  // the weight counts once per row (halves are summed)
    }
    cur.advance(chunk32, kv_end);
  };

  // Tiles run through the stages in a straight line; a chunk's last tile ends
  // with the merge.  The first chunk starts from m = -inf: its first step's
  // alpha = 0 clears acc and l.
  for (;;) {
    step(std::integral_constant<int, 0>{});
    if (cur.kv0 >= kv_end) break;
    step(std::integral_constant<int, 1>{});
    if (cur.kv0 >= kv_end) break;
    if constexpr (kStages == 3) {
      step(std::integral_constant<int, 2>{});
      if (cur.kv0 >= kv_end) break;
    }
  }

  if constexpr (kConstMax) {  // one sum over all keys: normalise now
    const float l_tot = sum_halves(l_run);
    const float inv = 1.0f / l_tot;
    // A row whose sum underflowed (the bound far above its true maximum) or
    // whose output is not finite is recomputed by the online kernel: the
    // wave flags its block's tile.  Padding rows (past Sq) have q = 0, p = 1.
    bool bad = !(l_tot >= 0x1p-100f);
#pragma unroll
    for (int b = 0; b < G::kDBlk; ++b) {
      oacc[b] *= inv;
#pragma unroll
      for (int i = 0; i < 16; ++i) bad |= !(fabsf(oacc[b][i]) <= 3.40282347e38f);
    }
    m_run += log2f(l_tot);
    const bool any_bad = __ballot(bad) != 0;
    if (__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) == 0)
      flags_out[(int64_t)logical * W + wave] = any_bad ? 1 : 0;
  }

  // ---- epilogue: out (bf16, RNE; or an fp32 partial for a piece) and lse (natural log) ----
  // The last tile closed a chunk, so acc = O and m = L (log2).
  // oacc[b][i] of lane (r32, hf) is d = 32*b + 8*(i/4) + 4*hf + i%4 of query qrow.
  // The lane's row and half are formed again here from the hardware lane
  // count (v_mbcnt), which the compiler cannot identify with the thread-id
  // arithmetic above: no per-lane value of the prologue (or 64-bit form of
  // one) stays live across the key loop, where every register is taken.
  const int e_lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int e_hf = e_lane >> 5;
  const int e_qrow = qt * kBM + wave * 32 + (e_lane & 31);
  if (e_qrow < sq) {
    if (piece) {
      // Partial of a piece: [n_split, rows, D] and lse [n_split, rows], rows
      // counted from the first row of the split tiles (tail_row0 of [B*H*Sq]).
      const int64_t n_rows = (int64_t)(n_tiles / n_qt) * Sq - tail_row0;
      const int64_t prow = (int64_t)split * n_rows + (bh * Sq + e_qrow - tail_row0);
      float* op = o_parts + prow * D;
#pragma unroll
      for (int b = 0; b < G::kDBlk; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(op + 32 * b + 8 * g + 4 * e_hf) =
              make_float4(oacc[b][4 * g], oacc[b][4 * g + 1], oacc[b][4 * g + 2], oacc[b][4 * g + 3]);
      if (e_hf == 0) l_parts[prow] = m_run * 0.69314718055994530942f;
    } else {
      // Row of (b, h, qrow): [B, H, Sq, D], or [B, Sq, H, D] (token-major).
      const int64_t b = bh / H;
      const int64_t prow = bh * Sq + e_qrow;
      const int64_t orow = out_bshd ? (b * Sq + e_qrow) * H + (bh - b * H) : prow;
      uint16_t* op = static_cast<uint16_t*>(out) + orow * D;
#pragma unroll
      for (int b = 0; b < G::kDBlk; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 w = u32x2{pack_bf16(oacc[b][4 * g], oacc[b][4 * g + 1]),
                                pack_bf16(oacc[b][4 * g + 2], oacc[b][4 * g + 3])};
          *reinterpret_cast<u32x2*>(op + 32 * b + 8 * g + 4 * e_hf) = w;
        }
      if (lse && e_hf == 0) lse[prow] = m_run * 0.69314718055994530942f;
    }
  }
}

// Head statistics for the bound-gated max: per head, kStatParts partial
// maxima of |k_j|^2 (stats[0 .. B*H*kStatParts)) and of |v| over every
// element (the next B*H*kStatParts floats).  Grid (B*H) x kStatParts blocks;
// block (bh, part) scans rows part*kRows + r, stepping kStatParts*kRows;
// kCpr consecutive lanes hold one row's 16-byte chunks.  Every partial is
// written (no atomics, nothing to clear first).
constexpr int kNormThreads = 256;
template <int D>
__global__ __launch_bounds__(kNormThreads) void head_stats_kernel(const uint16_t* __restrict__ k,
                                                                  const uint16_t* __restrict__ v,
                                                                  float* __restrict__ stats, int64_t Skv,
                                                                  int64_t nbh) {
  constexpr int kCpr = D / 8;
  constexpr int kRows = kNormThreads / kCpr;  // rows per block pass
  const int64_t bh = blockIdx.x / kStatParts;
  const int part = blockIdx.x % kStatParts;
  const int t = threadIdx.x, r = t / kCpr, ci = t % kCpr;
  const uint16_t* kb = k + bh * Skv * D;
  const uint16_t* vb = v + bh * Skv * D;
  float best = 0.f;
  uint32_t vbest = 0;  // largest |v| as a bf16 bit pattern (magnitudes order like integers)
  for (int64_t j = (int64_t)part * kRows + r; j < Skv; j += (int64_t)kStatParts * kRows) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(kb + j * D + ci * 8);
    const u32x4 y = *reinterpret_cast<const u32x4*>(vb + j * D + ci * 8);
    float ss = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = __uint_as_float(x[w] << 16), b = __uint_as_float(x[w] & 0xffff0000u);
      ss = fmaf(a, a, fmaf(b, b, ss));
      vbest = max(vbest, max(y[w] & 0x7fffu, (y[w] >> 16) & 0x7fffu));
    }
#pragma unroll
    for (int o = kCpr / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    best = fmaxf(best, ss);
  }
  __shared__ float red[kNormThreads];
  __shared__ uint32_t vred[kNormThreads];
  red[t] = best;
  vred[t] = vbest;
  __syncthreads();
  for (int sz = kNormThreads / 2; sz > 0; sz >>= 1) {
    if (t < sz) {
      red[t] = fmaxf(red[t], red[t + sz]);
      vred[t] = max(vred[t], vred[t + sz]);
    }
    __syncthreads();
  }
  if (t == 0) {
    stats[bh * kStatParts + part] = red[0];
    stats[(nbh + bh) * kStatParts + part] = __uint_as_float(vred[0] << 16);
  }
}

// Smallest b with 2^b >= n + 1 (n >= 0): the bit count of the accumulation
// length bound used for the per-head slack.
int bits_for(int64_t n) {
  int b = 0;
  while (b < 62 && (int64_t(1) << b) < n + 1) ++b;
  return b;
}

// The head statistics pre-pass (reads K and V once) into stats.
hipError_t launch_head_stats(const uint16_t* kp, const uint16_t* vp, float* stats, int64_t B, int64_t H,
                             int64_t Skv, int64_t D, hipStream_t stream) {
  const int64_t nbh = B * H;
  if (D == 64)
    head_stats_kernel<64><<<(unsigned)(nbh * kStatParts), kNormThreads, 0, stream>>>(kp, vp, stats, Skv, nbh);
  else
    head_stats_kernel<128><<<(unsigned)(nbh * kStatParts), kNormThreads, 0, stream>>>(kp, vp, stats, Skv, nbh);
  return hipGetLastError();
}

template <bool kConstMax, int W>
hipError_t launch_attn_kernel_w(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B,
                                int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale, int64_t kv_chunk,
                                bool out_bshd, const float* stats, const KeySplit& ks, float* o_parts,
                                float* l_parts, int* flags_out, const int* fix_flags, hipStream_t stream) {
  constexpr int kBM = Blk<W>::kBM;
  const int n_qt = (int)((Sq + kBM - 1) / kBM);
  const int n_tiles = (int)(B * H * n_qt);
  const int n_split = ks.n_split > 1 ? ks.n_split : 1;
  const int n_bulk = n_split > 1 ? (int)ks.n_bulk : n_tiles;
  const int n_blocks = n_bulk + (n_tiles - n_bulk) * n_split;
  const int64_t tail_row0 = attn_bf16_split_first_row(n_bulk, Sq, W);
  const float c = fabsf(scale) * 1.44269504088896340736f;  // |scale| * log2(e)
  const uint32_t qsign = scale < 0.f ? 0x80008000u : 0u;
  // Longest run of keys accumulated without a merge: a chunk (within a key
  // range when every tile is split).
  int64_t run = std::min(kv_chunk, Skv);
  if (n_split > 1 && n_bulk == 0) run = std::min(run, ks.split_len);
  const int chunk_bits = bits_for(run);
  const auto* qp = static_cast<const uint16_t*>(q);
  const auto* kp = static_cast<const uint16_t*>(k);
  const auto* vp = static_cast<const uint16_t*>(v);
  if (D == 64)
    attn_bf16_kernel<64, kConstMax, W><<<n_blocks, Blk<W>::kThreads, 0, stream>>>(
        qp, kp, vp, out, lse, H, Sq, Skv, c, qsign, kv_chunk, n_qt, n_tiles, n_bulk, out_bshd ? 1 : 0, stats,
        n_split, ks.split_len, o_parts, l_parts, tail_row0, chunk_bits, flags_out, fix_flags);
  else
    attn_bf16_kernel<128, kConstMax, W><<<n_blocks, Blk<W>::kThreads, 0, stream>>>(
        qp, kp, vp, out, lse, H, Sq, Skv, c, qsign, kv_chunk, n_qt, n_tiles, n_bulk, out_bshd ? 1 : 0, stats,
        n_split, ks.split_len, o_parts, l_parts, tail_row0, chunk_bits, flags_out, fix_flags);
  return hipGetLastError();
}

template <bool kConstMax>
hipError_t launch_attn_kernel(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B,
                              int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale, int64_t kv_chunk,
                              bool out_bshd, const float* stats, const KeySplit& ks, float* o_parts,
                              float* l_parts, int* flags_out, const int* fix_flags, hipStream_t stream) {
  if (!kConstMax && ks.waves == kWavesSmall)
    return launch_attn_kernel_w<kConstMax, kWavesSmall>(q, k, v, out, lse, B, H, Sq, Skv, D, scale, kv_chunk,
                                                        out_bshd, stats, ks, o_parts, l_parts, flags_out,
                                                        fix_flags, stream);
  return launch_attn_kernel_w<kConstMax, kWaves>(q, k, v, out, lse, B, H, Sq, Skv, D, scale, kv_chunk, out_bshd,
                                                 stats, ks, o_parts, l_parts, flags_out, fix_flags, stream);
}

}  // namespace

bool attn_bf16_launches_fit(int64_t B, int64_t H, int64_t Sq) {
  auto fits = [](int64_t blocks, int64_t threads) {
    return blocks > 0 && blocks <= (int64_t(1) << 31) - 1 && blocks * threads < (int64_t(1) << 32);
  };
  const int64_t nbh = B * H;
  return fits(nbh * kStatParts, kNormThreads) &&
         fits(nbh * ((Sq + Blk<kWaves>::kBM - 1) / Blk<kWaves>::kBM), Blk<kWaves>::kThreads);
}

int64_t attn_bf16_query_tiles(int64_t Sq, int waves) {
  const int64_t bm = 32 * (int64_t)waves;
  return (Sq + bm - 1) / bm;
}

int64_t attn_bf16_split_first_row(int64_t n_bulk, int64_t Sq, int waves) {
  const int64_t bm = 32 * (int64_t)waves;
  const int64_t n_qt = (Sq + bm - 1) / bm;
  return (n_bulk / n_qt) * Sq + (n_bulk % n_qt) * bm;
}

namespace {
// The best key split for blocks of `waves` waves, and its modelled time in
// seconds.  Cost model fitted to timings of forced splits on the MI355X
// (shard shapes, image and long-video workloads): a round of blocks that
// fills a share f of the CUs costs 0.83 + 0.17 f of a full one (the chip is
// power-limited and clocks up when fewer CUs run, but not by much); a piece
// of len keys costs like len + 700 keys (prologue, pipeline fill, partial
// write); the partials' write and merge stream at ~5 TB/s; a split must gain
// 2%.  A block of 12 waves works at ~1250 TFLOP/s over the chip; one of 8
// waves at 0.9 of that rate per CU (two waves per SIMD hide less).
KeySplit plan_waves(int waves, int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, int64_t kv_chunk,
                    int n_cus, double* seconds) {
  const int64_t bm = 32 * (int64_t)waves;
  const int64_t tiles = B * H * attn_bf16_query_tiles(Sq, waves);
  const double eff = waves == kWaves ? 1.0 : 0.9;
  const double tile_s = 4.0 * bm * (double)Skv * (double)D / (1250e12 / n_cus) / eff;  // one tile, all keys
  auto round_cost = [](double f) { return 0.83 + 0.17 * f; };
  auto rounds = [&](int64_t nb, double len) {  // nb blocks of relative length len
    const int64_t r = nb / n_cus, f = nb % n_cus;
    return len * ((double)r + (f ? round_cost((double)f / n_cus) : 0.0));
  };
  KeySplit best;
  best.waves = waves;
  best.n_bulk = tiles;
  best.n_split = 1;
  best.split_len = Skv;
  const int64_t tail = tiles % n_cus;  // tiles of the last, partly filled round
  const int64_t full = tiles / n_cus;
  const double base = ((double)full + (tail ? round_cost((double)tail / n_cus) : 0.0)) * tile_s;
  *seconds = base;
  if (tail == 0) return best;
  const double tail_rows = (double)(B * H * Sq - attn_bf16_split_first_row(tiles - tail, Sq, waves));
  const int64_t unit = kv_chunk < Skv ? kv_chunk : kBN;  // ranges hold whole chunks, else whole tiles
  const int64_t n_units = (Skv + unit - 1) / unit;
  for (int s = 2; s <= kMaxKeySplit; ++s) {
    const int64_t len = ((n_units + s - 1) / s) * unit;
    if (len < kMinSplitKeys) break;
    const int64_t n = (Skv + len - 1) / len;  // ranges actually made
    if (n < 2) continue;
    const double merge_s = ((double)n * tail_rows * (D + 1) * 4.0 * 2.0 + tail_rows * D * 2.0) / 5e12 + 10e-6;
    const double cost =
        ((double)full + rounds(tail * n, (double)(len + 700) / (double)Skv)) * tile_s + merge_s;
    if (cost < base * 0.98 && cost < *seconds) {
      best.n_bulk = tiles - tail;
      best.n_split = (int)n;
      best.split_len = len;
      *seconds = cost;
    }
  }
  return best;
}
}  // namespace

KeySplit attn_bf16_key_split(int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, int64_t kv_chunk,
                             int n_cus) {
  KeySplit none;
  none.waves = kWaves;
  none.n_bulk = B * H * attn_bf16_query_tiles(Sq, kWaves);
  none.n_split = 1;
  none.split_len = Skv;
  if (n_cus <= 0) return none;
  double t_big = 0.0, t_small = 0.0;
  const KeySplit big = plan_waves(kWaves, B, H, Sq, Skv, D, kv_chunk, n_cus, &t_big);
  if (D != 128) return big;  // the 8-wave block's rate was measured at D = 128
  const KeySplit small = plan_waves(kWavesSmall, B, H, Sq, Skv, D, kv_chunk, n_cus, &t_small);
  // The smaller block only for grids it clearly serves better (few query
  // tiles: the larger block leaves CUs idle).
  return t_small < 0.98 * t_big ? small : big;
}

int attn_bf16_waves() { return kWaves; }

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* out, float* lse, float* stats,
                            int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale,
                            int64_t kv_chunk, bool out_bshd, const KeySplit& ks, float* o_parts, float* l_parts,
                            hipStream_t stream) {
  hipError_t e = launch_head_stats(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), stats, B, H,
                                   Skv, D, stream);
  if (e != hipSuccess) return e;
  e = launch_attn_kernel<false>(q, k, v, out, lse, B, H, Sq, Skv, D, scale, kv_chunk, out_bshd, stats, ks, o_parts,
                                l_parts, nullptr, nullptr, stream);
  if (e != hipSuccess || ks.n_split <= 1) return e;
  // Merge the pieces' partials into the rows of the split tiles (token-major
  // rows for a [B, Sq, H, D] output).
  const int64_t row0 = attn_bf16_split_first_row(ks.n_bulk, Sq, ks.waves);
  TokenMajor tm;
  if (out_bshd) {
    tm.row0 = row0;
    tm.H = H;
    tm.Sq = Sq;
  }
  return launch_lse_merge(o_parts, l_parts, ks.n_split, false,
                          static_cast<uint16_t*>(out) + (out_bshd ? 0 : row0 * D), lse ? lse + row0 : nullptr, true,
                          B * H * Sq - row0, D, stream, tm);
}

hipError_t launch_attn_bf16_constmax(const void* q, const void* k, const void* v, void* out, float* lse,
                                     float* stats, int* flags, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                                     int64_t D, float scale, hipStream_t stream) {
  hipError_t e = launch_head_stats(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), stats, B, H,
                                   Skv, D, stream);
  if (e != hipSuccess) return e;
  KeySplit whole;
  whole.waves = kWaves;
  whole.n_bulk = B * H * attn_bf16_query_tiles(Sq, kWaves);
  whole.n_split = 1;
  whole.split_len = Skv;
  e = launch_attn_kernel<true>(q, k, v, out, lse, B, H, Sq, Skv, D, scale, Skv, false, stats, whole, nullptr,
                               nullptr, flags, nullptr, stream);
  if (e != hipSuccess) return e;
  // Recompute the flagged tiles with the online reference (one chunk: the
  // same function; blocks of clean tiles return at once).
  return launch_attn_kernel<false>(q, k, v, out, lse, B, H, Sq, Skv, D, scale, Skv, false, stats, whole, nullptr,
                                   nullptr, nullptr, flags, stream);
}

}  // namespace r3d
