// attn_fwd_bf16.hip — blockwise joint-sequence attention on gfx950 bf16 MFMA.
//
// Computes, per (b, h, query row), softmax(scale * q K^T) V over all Skv keys,
// non-causal ("Context Parallelism in vLLM Omni Neuron", §Self-Attention:
// _nf_attend(query, key, value, scale); §Overview: full attention is kept
// while the sequence is split).  Keys are visited in chunks of kv_chunk keys,
// the single-device form of ring attention's one-K/V-shard-per-round loop
// (§Ring attention):
//   * inside a chunk: online softmax over key tiles of kBN keys (running max
//     m, running sum l, accumulator acc rescaled by 2^(m_old - m_new));
//   * at the end of a chunk: O_c = acc / l, lse_c = m + log2 l is merged into
//     the running result (O, L) by the explicit log-sum-exp rule
//       L' = log2(2^L + 2^lse_c),  O = O 2^(L - L') + O_c 2^(lse_c - L'),
//     in registers; nothing partial is written to memory (§Memory and Compute
//     Benefits: the split keeps full attention quality).
// The softmax runs in the log2 domain: logits are pre-multiplied by
// c = scale * log2(e) inside one FMA, so p = 2^(s*c - m).
//
// Mapping onto CDNA4
// ------------------
// * Block = 4 waves, 128 query rows (32 per wave); grid = B*H*ceil(Sq/128)
//   blocks, re-numbered so that consecutive tiles of one head land on the
//   same XCD (hardware hands block i to XCD i % 8), so the 32 CUs of an XCD
//   stream the same K/V and share it through that XCD's L2.
// * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K rows (from LDS), B = Q^T
//   (kept in VGPRs for the whole block).  The 32x32 accumulator then holds,
//   in lane l, 16 keys of query column l%32 — so each lane owns one query row
//   and the row max / row sum need only in-lane work plus one exchange with
//   lane l^32.
// * K rows are fed to the MFMA in the permuted order pi (bits 2 and 3 of the
//   row index swapped) so that accumulator element i of lane-half hf holds
//   tile key 16*(i/8) + 8*hf + i%8: eight consecutive keys per half, exactly
//   the B-operand fragment of the PV product.  P therefore goes from the
//   S^T accumulator to the PV MFMA in registers (fp32 -> bf16 packed
//   convert), with no LDS round trip.
// * O^T = V^T P^T with the same MFMA: A = V^T (V stored transposed in LDS,
//   so a lane's 8 keys are one 16-byte read), B = P^T.  The O^T accumulator
//   again holds one query per lane, so the per-row rescale and the chunk
//   merge are per-lane scalars.
// * K and V^T tiles are double-buffered in LDS; the next tile's global loads
//   are issued before the current tile's MFMAs and written to the other LDS
//   buffer afterwards (one barrier per tile).  Rows are padded by 16 bytes so
//   the 16-byte MFMA operand reads of a wave spread over all LDS banks.
#include "launch.h"

namespace r3d {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per block
constexpr int kBN = 64;           // keys per tile
constexpr int kXcds = 8;

template <int D>
struct Geom {
  static constexpr int kSteps = D / 16;                 // MFMA k-steps of Q K^T
  static constexpr int kDBlk = D / 32;                  // 32-wide d blocks of O^T
  static constexpr int kKRow = D + 8;                   // K tile row, elements (padded)
  static constexpr int kVRow = kBN + 8;                 // V^T tile row, elements (padded)
  static constexpr int kKElems = kBN * kKRow;
  static constexpr int kVElems = D * kVRow;
  static constexpr int kCpr = D / 8;                    // 16-byte chunks per K/V row
  static constexpr int kKLoads = kBN * kCpr / kThreads; // 16-byte K loads per thread
  static constexpr int kVItems = (kBN / 4) * (D / 8);   // 4-key x 8-d V items per tile
};

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// MFMA row m of the S^T product reads tile key pi(m): bits 2 and 3 swapped.
__device__ __forceinline__ int key_of_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <int D>
struct Stage {
  u32x4 k[Geom<D>::kKLoads];
  u32x4 v[4];
};

// Global -> registers for the tile of n (<= kBN) keys starting at kv0.
// Rows past n are zero (their logits are masked; zero V keeps 0 * V finite).
template <int D>
__device__ __forceinline__ void load_tile(Stage<D>& st, const uint16_t* __restrict__ kb,
                                          const uint16_t* __restrict__ vb, int64_t kv0, int n, int tid) {
  using G = Geom<D>;
#pragma unroll
  for (int r = 0; r < G::kKLoads; ++r) {
    const int idx = tid + r * kThreads;
    const int row = idx / G::kCpr, ch = idx % G::kCpr;
    st.k[r] = row < n ? *reinterpret_cast<const u32x4*>(kb + (kv0 + row) * D + ch * 8) : u32x4{0, 0, 0, 0};
  }
  if (tid < G::kVItems) {
    const int kg = tid / G::kCpr, dc = tid % G::kCpr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = 4 * kg + j;
      st.v[j] = key < n ? *reinterpret_cast<const u32x4*>(vb + (kv0 + key) * D + dc * 8) : u32x4{0, 0, 0, 0};
    }
  }
}

// Registers -> LDS: K row-major [key][d]; V transposed [d][key] (4 keys x 8 d
// per thread, written as eight 8-byte rows of 4 keys).
template <int D>
__device__ __forceinline__ void store_tile(const Stage<D>& st, uint16_t* ks, uint16_t* vts, int tid) {
  using G = Geom<D>;
#pragma unroll
  for (int r = 0; r < G::kKLoads; ++r) {
    const int idx = tid + r * kThreads;
    const int row = idx / G::kCpr, ch = idx % G::kCpr;
    *reinterpret_cast<u32x4*>(ks + row * G::kKRow + ch * 8) = st.k[r];
  }
  if (tid < G::kVItems) {
    const int kg = tid / G::kCpr, dc = tid % G::kCpr;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int w = i >> 1;
      const int sh = (i & 1) * 16;
      const uint32_t e0 = (st.v[0][w] >> sh) & 0xffffu, e1 = (st.v[1][w] >> sh) & 0xffffu;
      const uint32_t e2 = (st.v[2][w] >> sh) & 0xffffu, e3 = (st.v[3][w] >> sh) & 0xffffu;
      *reinterpret_cast<u32x2*>(vts + (dc * 8 + i) * G::kVRow + 4 * kg) = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ out, float* __restrict__ lse, int64_t Sq, int64_t Skv, float c, uint32_t qsign,
    int64_t chunk, int n_qt, int n_blocks) {
  using G = Geom<D>;
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][G::kKElems];
  __shared__ __attribute__((aligned(16))) uint16_t vts[2][G::kVElems];

  // Block -> (head, query tile): XCD x runs logical tiles [x*q + min(x, r), ...).
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

  f32x16 oacc[G::kDBlk], orun[G::kDBlk];
#pragma unroll
  for (int b = 0; b < G::kDBlk; ++b) {
    oacc[b] = f32x16{};
    orun[b] = f32x16{};
  }
  float m_run = -INFINITY, l_run = 0.f, L = -INFINITY;
  bool first_chunk = true;

  const int krow0 = key_of_row(r32);
  int64_t kv = 0;
  int64_t chunk_end = chunk < Skv ? chunk : Skv;
  Stage<D> st;
  load_tile<D>(st, kb, vb, 0, (int)((chunk_end < kBN) ? chunk_end : kBN), tid);
  store_tile<D>(st, ks[0], vts[0], tid);
  __syncthreads();
  int buf = 0;

  while (true) {
    const int64_t tile_end = (kv + kBN < chunk_end) ? kv + kBN : chunk_end;
    const int n = (int)(tile_end - kv);
    int64_t nkv = tile_end, nchunk_end = chunk_end;
    if (nkv == chunk_end) nchunk_end = (chunk_end + chunk < Skv) ? chunk_end + chunk : Skv;
    const bool has_next = nkv < Skv;
    if (has_next) {
      const int64_t ne = (nkv + kBN < nchunk_end) ? nkv + kBN : nchunk_end;
      load_tile<D>(st, kb, vb, nkv, (int)(ne - nkv), tid);
    }

    // ---- S^T = K Q^T over the tile (two 32-key blocks) ----
    const uint16_t* kt = ks[buf];
    f32x16 sacc[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      sacc[kb2] = f32x16{};
      const uint16_t* kp = kt + (32 * kb2 + krow0) * G::kKRow + 8 * hf;
#pragma unroll
      for (int s = 0; s < G::kSteps; ++s)
        sacc[kb2] = mfma(*reinterpret_cast<const bf16x8*>(kp + 16 * s), qf[s], sacc[kb2]);
    }

    // ---- online softmax (log2 domain), one query row per lane ----
    // element i of sacc[kb2] is tile key 32*kb2 + 16*(i/8) + 8*hf + i%8
    if (n < kBN) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * kb2 + 16 * (i / 8) + 8 * hf + (i % 8) >= n) sacc[kb2][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb2][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on a chunk's first tile
    float psum = 0.f;
    float p[2][16];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[kb2][i] = __builtin_amdgcn_exp2f(fmaf(sacc[kb2][i], c, -m_new));
        psum += p[kb2][i];
      }
    if (n < kBN) {  // masked keys: exactly zero, also when c == 0
      psum = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (32 * kb2 + 16 * (i / 8) + 8 * hf + (i % 8) >= n) p[kb2][i] = 0.f;
          psum += p[kb2][i];
        }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int b = 0; b < G::kDBlk; ++b) oacc[b] *= alpha;
    }

    // ---- O^T += V^T P^T: four 16-key steps ----
    const uint16_t* vt = vts[buf];
#pragma unroll
    for (int sg = 0; sg < 4; ++sg) {
      const int kb2 = sg >> 1, base = 8 * (sg & 1);
      u32x4 pw;
#pragma unroll
      for (int w = 0; w < 4; ++w) pw[w] = pack_bf16(p[kb2][base + 2 * w], p[kb2][base + 2 * w + 1]);
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int b = 0; b < G::kDBlk; ++b)
        oacc[b] = mfma(*reinterpret_cast<const bf16x8*>(vt + (32 * b + r32) * G::kVRow + 16 * sg + 8 * hf), pf,
                       oacc[b]);
    }

    if (has_next) store_tile<D>(st, ks[buf ^ 1], vts[buf ^ 1], tid);
    __syncthreads();

    // ---- end of a chunk: explicit log-sum-exp merge into (orun, L) ----
    if (tile_end == chunk_end) {
      const float l_tot = l_run + __shfl_xor(l_run, 32);
      const float lse_c = m_run + log2f(l_tot);
      if (first_chunk) {
        const float inv = 1.0f / l_tot;
#pragma unroll
        for (int b = 0; b < G::kDBlk; ++b) orun[b] = oacc[b] * inv;
        L = lse_c;
        first_chunk = false;
      } else {
        const float hi = fmaxf(L, lse_c);
        const float Ln = hi + log2f(exp2f(L - hi) + exp2f(lse_c - hi));
        const float wa = exp2f(L - Ln);
        const float wb = exp2f(lse_c - Ln) / l_tot;
#pragma unroll
        for (int b = 0; b < G::kDBlk; ++b) orun[b] = orun[b] * wa + oacc[b] * wb;
        L = Ln;
      }
#pragma unroll
      for (int b = 0; b < G::kDBlk; ++b) oacc[b] = f32x16{};
      m_run = -INFINITY;
      l_run = 0.f;
    }
    if (!has_next) break;
    kv = nkv;
    chunk_end = nchunk_end;
    buf ^= 1;
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
