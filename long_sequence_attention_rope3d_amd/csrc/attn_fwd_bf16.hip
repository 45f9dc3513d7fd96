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
//   * at the end of a chunk: O_c = acc / l, lse_c = m + log2 l is merged into
//     the running result (O, L) by the explicit log-sum-exp rule
//       L' = log2(2^L + 2^lse_c),  O = O 2^(L - L') + O_c 2^(lse_c - L'),
//     in registers; nothing partial is written to memory (§Memory and Compute
//     Benefits: the split keeps full attention quality).
// The softmax runs in the log2 domain: logits are multiplied by
// c = |scale| * log2(e) inside one FMA, so p = 2^(s*c - m).
//
// Mapping onto CDNA4
// ------------------
// * Block = 8 waves = 256 query rows (32 per wave), i.e. two waves per SIMD:
//   while one wave of a SIMD runs its softmax on the VALU the other keeps the
//   matrix core busy (a single wave per SIMD issues VALU at half rate and
//   stalls on its own MFMA chains).  That caps a wave at 256 registers.
// * Grid = B*H*ceil(Sq/256) blocks, re-numbered so consecutive query tiles of
//   one head land on the same XCD (hardware hands block i to XCD i % 8): the
//   CUs of an XCD stream the same K/V and share it in that XCD's L2.
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
// * Lazy rescale: the running max is only raised when a step's max exceeds
//   it by more than kTau (log2 units); otherwise p = 2^(s*c - m) <= 2^kTau and
//   acc keeps its scale.  The result is unchanged (the same m scales both
//   acc and l); most steps skip the 64-register rescale of acc.
// * The row sum l adds the fp32 p before their bf16 rounding for the PV
//   product, so lse keeps fp32 accuracy.
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
#define R3D_ATTN_WAVES 8
#endif
#ifndef R3D_ATTN_STAGES
#define R3D_ATTN_STAGES 2
#endif
constexpr int kWaves = R3D_ATTN_WAVES;
constexpr int kStages = R3D_ATTN_STAGES;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per block
constexpr int kWavesPerSimd = 2;  // two waves per SIMD: from one block (8 waves) or two (4 waves)
static_assert(kStages == 2 || kStages == 3, "2 or 3 stages");
#ifndef R3D_ATTN_BN
#define R3D_ATTN_BN 128
#endif
constexpr int kBN = R3D_ATTN_BN;  // keys per LDS tile (a multiple of 32)
constexpr int kXcds = 8;
constexpr float kTau = 8.0f;      // lazy-rescale threshold, log2 units

template <int D>
struct Geom {
  static constexpr int kSteps = D / 16;               // MFMA k-steps of Q K^T
  static constexpr int kDBlk = D / 32;                // 32-wide d blocks of O^T
  static constexpr int kCpr = D / 8;                  // 16-byte chunks per K/V row
  static constexpr int kTile = kBN * D;               // elements of one K or V tile
  static constexpr int kDma = kBN * kCpr / 64;         // 1 KB DMA instructions per tensor per tile
  static constexpr int kDmaPerWave = kDma / kWaves;
  static_assert(kDmaPerWave >= 1 && kDma % kWaves == 0, "tile/waves mismatch");
};

// Per-row XOR swizzles of the 16-byte chunk index (see the bank notes above).
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  // ds_read_b128 is served 16 lanes (256 bytes) per LDS cycle; the 16 lanes of
  // a group read 16 different rows at the same logical chunk.
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  // ds_read_b64_tr_b16: a 16-lane group reads 4 consecutive rows x 32 bytes.
  return D == 128 ? 4 * (r & 3) : 2 * (r & 3);
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

// x of this lane combined with x of lane l^32.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// MFMA row m of the S^T product reads tile key pi(m): bits 2 and 3 swapped.
__device__ __forceinline__ int key_of_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Walks the key tiles in order: tiles of kBN keys inside chunks of `chunk`
// keys (the last tile of a chunk may be short), advanced by additions only.
struct TileCursor {
  int64_t kv0;   // first key of the tile
  int64_t cend;  // end of the tile's chunk
  __device__ __forceinline__ int n() const { return (int)((kv0 + kBN < cend) ? kBN : cend - kv0); }
  __device__ __forceinline__ void advance(int64_t chunk, int64_t Skv) {
    kv0 += kBN;
    if (kv0 >= cend) {
      kv0 = cend;
      cend = (cend + chunk < Skv) ? cend + chunk : Skv;
    }
  }
};

// Direct global -> LDS copy of one K or V tile (n valid keys from kv0) into
// `tile`, as kDma wave-instructions of 64 x 16 bytes.  global_load_lds_dwordx4
// writes lane L's 16 bytes to (M0 + 16*L), so the swizzle is realised by
// choosing, per lane, which global chunk lands in its slot: slot s = 64*m + L
// holds row s / kCpr, logical chunk (s % kCpr) ^ swz(row).  Rows past n
// re-read the last valid row (in bounds); their logits are masked and their p
// is exactly zero.
//
// The copy is issued from inline assembly on purpose: the compiler's own
// wait-count insertion cannot prove that the LDS reads of the stage being
// consumed are independent of the copy in flight into another stage, and
// puts a full vmcnt(0) wait after every prefetch, exposing the whole copy
// latency on each tile.  Hidden from it, the copies are ordered only by the
// explicit waits in wait_vm_barrier (every read of a stage follows the wait
// + barrier that retire that stage's copies).  The compiler's own vmcnt
// waits (the Q loads) only become stricter by the extra operations in the
// counter.  One wait state separates the M0 write from the DMA.
template <int D, bool IS_V>
__device__ __forceinline__ void dma_tile(uint16_t* tile, const uint16_t* __restrict__ src, int64_t kv0, int n,
                                         int wave, int lane) {
  using G = Geom<D>;
#pragma unroll
  for (int i = 0; i < G::kDmaPerWave; ++i) {
    const int m = wave + kWaves * i;
    const int slot = 64 * m + lane;
    const int r = slot / G::kCpr;
    const int cl = (slot % G::kCpr) ^ (IS_V ? swz_v<D>(r) : swz_k<D>(r));
    const int64_t row = kv0 + (r < n ? r : n - 1);
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(tile + m * 64 * 8));
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src + row * D + cl * 8),
                 "s"(lds)
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

template <int D>
__global__ __launch_bounds__(kThreads, kWavesPerSimd) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ out, float* __restrict__ lse, int64_t Sq, int64_t Skv, float c, uint32_t qsign,
    int64_t chunk, int n_qt, int n_blocks) {
  using G = Geom<D>;
  // K/V stage buffers (the third only with kStages == 3).
  __shared__ __attribute__((aligned(1024))) uint16_t st0_k[G::kTile], st0_v[G::kTile];
  __shared__ __attribute__((aligned(1024))) uint16_t st1_k[G::kTile], st1_v[G::kTile];
  __shared__ __attribute__((aligned(1024))) uint16_t st2_k[G::kTile], st2_v[G::kTile];

  // Block -> (head, query tile): XCD x runs logical tiles [x*per + min(x, rem), ...).
  const int bid = blockIdx.x;
  const int per = n_blocks / kXcds, rem = n_blocks % kXcds;
  const int xcd = bid % kXcds, slot = bid / kXcds;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + slot;
  const int64_t bh = logical / n_qt;
  const int qt = logical - (int)bh * n_qt;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, hf = lane >> 5;
  const int64_t qrow = (int64_t)qt * kBM + wave * 32 + r32;
  const uint16_t* kb = k + bh * Skv * D;
  const uint16_t* vb = v + bh * Skv * D;

  // Q^T fragments (B operand): query qrow, d = 16*s + 8*hf + [0, 8).  A
  // negative scale is folded into Q by flipping sign bits (exact), so c >= 0.
  bf16x8 qf[G::kSteps];
#pragma unroll
  for (int s = 0; s < G::kSteps; ++s) {
    u32x4 x = u32x4{0, 0, 0, 0};
    if (qrow < Sq) x = *reinterpret_cast<const u32x4*>(q + (bh * Sq + qrow) * D + 16 * s + 8 * hf) ^ qsign;
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
      v_base[b] = (row * G::kCpr + (((32 * b + d) >> 3) ^ swz_v<D>(row))) * 16 + (d & 7) * 2;
  }

  f32x16 oacc[G::kDBlk], orun[G::kDBlk];
#pragma unroll
  for (int b = 0; b < G::kDBlk; ++b) {
    oacc[b] = f32x16{};
    orun[b] = f32x16{};
  }
  float m_run = -INFINITY, l_run = 0.f, L = -INFINITY;

  const int64_t first_cend = chunk < Skv ? chunk : Skv;
  // pf: the next tile to prefetch.  Prologue: tiles 0 and 1 in flight, wait for tile 0.
  TileCursor pf{0, first_cend};
  dma_tile<D, false>(st0_k, kb, pf.kv0, pf.n(), wave, lane);
  dma_tile<D, true>(st0_v, vb, pf.kv0, pf.n(), wave, lane);
  pf.advance(chunk, Skv);
  if (kStages == 3 && pf.kv0 < Skv) {
    dma_tile<D, false>(st1_k, kb, pf.kv0, pf.n(), wave, lane);
    dma_tile<D, true>(st1_v, vb, pf.kv0, pf.n(), wave, lane);
    pf.advance(chunk, Skv);
  }
  // The prologue tiles target different LDS objects, so their DMAs may be
  // issued in either order: wait for all of them once.
  wait_vm_barrier<0>();

  // One tile of n keys in stage S: prefetch the tile after next into stage
  // (S+2)%3, consume stage S, then wait for the next tile (this wave's part of
  // it) and meet at the barrier.
  TileCursor cur{0, first_cend};  // the tile being consumed
  auto step = [&](auto stage) {
    constexpr int S = decltype(stage)::value;
    const int n = cur.n();
    const bool chunk_done = cur.kv0 + n == cur.cend;
    const bool issue = pf.kv0 < Skv;
    if (issue) {
      constexpr int P = (S + kStages - 1) % kStages;  // stage of the tile kStages-1 ahead
      dma_tile<D, false>(P == 0 ? st0_k : P == 1 ? st1_k : st2_k, kb, pf.kv0, pf.n(), wave, lane);
      dma_tile<D, true>(P == 0 ? st0_v : P == 1 ? st1_v : st2_v, vb, pf.kv0, pf.n(), wave, lane);
      pf.advance(chunk, Skv);
    }

    const char* kt = reinterpret_cast<const char*>(S == 0 ? st0_k : S == 1 ? st1_k : st2_k);
    char* vt = reinterpret_cast<char*>(S == 0 ? st0_v : S == 1 ? st1_v : st2_v);
#pragma unroll
    for (int h2 = 0; h2 < kBN / 32; ++h2) {  // 32-key softmax steps of the tile
      if (32 * h2 >= n) break;        // wholly past the end of the chunk
      // ---- S^T = K Q^T for 32 keys ----
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int s = 0; s < G::kSteps; ++s)
        sacc = mfma(*reinterpret_cast<const bf16x8*>(kt + k_base[s] + h2 * 32 * G::kCpr * 16), qf[s], sacc);

      // ---- online softmax, log2 domain; element i is key 32*h2 + 16*(i/8) + 8*hf + i%8 ----
      // Keys past the end of a short tile hold copies of its last valid key
      // (the DMA clamps the row), so they cannot raise the max; only their p
      // is zeroed below.
      float mx = sacc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
      mx = max_halves(mx);
      const float cand = mx * c;
      const float m_use = (cand > m_run + kTau) ? cand : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);  // 1 if kept, 0 on a chunk's first step
      if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int b = 0; b < G::kDBlk; ++b) oacc[b] *= alpha;
      }
      m_run = m_use;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = __builtin_amdgcn_exp2f(fmaf(sacc[i], c, -m_use));
      if (n < 32 * (h2 + 1)) {  // short tile: keys past its end get p = 0 exactly
        const int lim = n - 32 * h2 - 8 * hf;  // element i is a real key iff 16*(i/8) + i%8 < lim
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (16 * (i / 8) + (i % 8) >= lim) sacc[i] = 0.f;
      }
      // Row sum from the unrounded fp32 p (keeps lse at fp32 accuracy).
      float ps = l_run * alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) ps += sacc[i];
      u32x4 pw[2];
#pragma unroll
      for (int w = 0; w < 8; ++w) pw[w >> 2][w & 3] = pack_bf16(sacc[2 * w], sacc[2 * w + 1]);
      l_run = ps;

      // ---- O^T += V^T P^T: two 16-key steps ----
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const bf16x8 pf = __builtin_bit_cast(bf16x8, pw[sl]);
        const int sg = 2 * h2 + sl;
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


    if (kStages == 3 && issue)
      wait_vm_barrier<2 * G::kDmaPerWave>();  // the tile just issued may stay in flight
    else
      wait_vm_barrier<0>();

    // ---- end of a chunk: explicit log-sum-exp merge into (orun, L) ----
    if (chunk_done) {
      const float l_tot = sum_halves(l_run);
      const float lse_c = m_run + log2f(l_tot);
      const float hi = fmaxf(L, lse_c);
      const float Ln = hi + log2f(exp2f(L - hi) + exp2f(lse_c - hi));
      const float wa = exp2f(L - Ln);
      const float wb = exp2f(lse_c - Ln) / l_tot;
#pragma unroll
      for (int b = 0; b < G::kDBlk; ++b) orun[b] = orun[b] * wa + oacc[b] * wb;
      L = Ln;
      m_run = -INFINITY;  // the next chunk starts afresh: its first alpha is 0
    }
    cur.advance(chunk, Skv);
  };

  // Tiles run through stages 0, 1, 2, 0, ... in a straight line; a chunk's
  // last tile ends with the explicit merge of its partial (O_c = acc/l,
  // lse_c = m + log2 l) into (orun, L).  Inside a chunk the online softmax
  // starts from m = -inf: the first step's alpha = 0 clears acc and l.  With
  // L = -inf initially the first merge gives orun weight 0.
  for (;;) {
    step(std::integral_constant<int, 0>{});
    if (cur.kv0 >= Skv) break;
    step(std::integral_constant<int, 1>{});
    if (cur.kv0 >= Skv) break;
    if constexpr (kStages == 3) {
      step(std::integral_constant<int, 2>{});
      if (cur.kv0 >= Skv) break;
    }
  }

  // ---- epilogue: out (bf16, RNE) and lse (natural log) ----
  // orun[b][i] of lane (r32, hf) is d = 32*b + 8*(i/4) + 4*hf + i%4 of query qrow.
  if (qrow < Sq) {
    uint16_t* op = out + (bh * Sq + qrow) * D;
#pragma unroll
    for (int b = 0; b < G::kDBlk; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 w = u32x2{pack_bf16(orun[b][4 * g], orun[b][4 * g + 1]),
                              pack_bf16(orun[b][4 * g + 2], orun[b][4 * g + 3])};
        *reinterpret_cast<u32x2*>(op + 32 * b + 8 * g + 4 * hf) = w;
      }
    if (lse && hf == 0) lse[bh * Sq + qrow] = L * 0.69314718055994530942f;
  }
}

}  // namespace

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B,
                            int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale, int64_t kv_chunk,
                            hipStream_t stream) {
  const int n_qt = (int)((Sq + kBM - 1) / kBM);
  const int n_blocks = (int)(B * H * n_qt);
  const float c = fabsf(scale) * 1.44269504088896340736f;  // |scale| * log2(e)
  const uint32_t qsign = scale < 0.f ? 0x80008000u : 0u;
  const auto* qp = static_cast<const uint16_t*>(q);
  const auto* kp = static_cast<const uint16_t*>(k);
  const auto* vp = static_cast<const uint16_t*>(v);
  auto* op = static_cast<uint16_t*>(out);
  if (D == 64)
    attn_bf16_kernel<64><<<n_blocks, kThreads, 0, stream>>>(qp, kp, vp, op, lse, Sq, Skv, c, qsign, kv_chunk, n_qt,
                                                             n_blocks);
  else
    attn_bf16_kernel<128><<<n_blocks, kThreads, 0, stream>>>(qp, kp, vp, op, lse, Sq, Skv, c, qsign, kv_chunk,
                                                              n_qt, n_blocks);
  return hipGetLastError();
}

}  // namespace r3d
