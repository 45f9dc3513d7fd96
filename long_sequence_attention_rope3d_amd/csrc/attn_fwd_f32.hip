// attn_fwd_f32.hip — the all-fp32 attention path (fp32 storage, fp32 math).
//
// Same blockwise algorithm as the bf16 MFMA path, in plain fp32 VALU code:
// keys are visited chunk by chunk; inside a chunk an online softmax keeps a
// running max m, sum l and accumulator acc (rescaled per 64-key block); at
// the end of every chunk (O_c = acc/l, lse_c = m + ln l) is merged into the
// running result by the log-sum-exp rule
//   L' = ln(e^L + e^lse_c),  O = O e^(L - L') + O_c e^(lse_c - L').
// ("Context Parallelism in vLLM Omni Neuron", §Self-Attention, §Ring
// attention, §Memory and Compute Benefits.)
//
// One wave per query row, four rows of one head per block; the block stages
// 64-key tiles of K and V in LDS.  For a tile, lane j forms key j's logit
// against the row's query (read from LDS as a broadcast), the wave reduces
// the tile's max and sum, writes the tile's p to LDS, and lane l accumulates
// d = l (and l + 64 for D = 128) of P V in four interleaved chains.  K rows
// are padded to D + 4 floats so that the 16-byte reads of 16 lanes (16
// different rows, same columns) fall into distinct banks; V rows are read
// along d, conflict-free.  The next tile's K and V are loaded into registers
// while the current one is computed, so only the first tile's load latency
// is exposed.
#include "launch.h"

namespace r3d {
namespace {

constexpr int kRowsF32 = 4;          // query rows (waves) per block
constexpr int kBNF32 = 64;           // keys per tile: one per lane
constexpr int kThreadsF32 = 64 * kRowsF32;

// Wave-wide max and sum (the result wave-uniform).  DPP row rotations
// (row_ror 8, 4, 2, 1 within each row of 16 lanes: register reads, no LDS
// round trip) leave every lane of a row with its row's result; lanes 0, 16,
// 32 and 48 are then read into scalars and combined.
template <int kRor>
__device__ __forceinline__ float row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + kRor, 0xf, 0xf, false));
}
__device__ __forceinline__ float rows_of(float x, float (*op)(float, float)) {
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return op(op(r0, r1), op(r2, r3));
}
__device__ __forceinline__ float max2(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ float add2(float a, float b) { return a + b; }
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, row_ror<8>(x));
  x = fmaxf(x, row_ror<4>(x));
  x = fmaxf(x, row_ror<2>(x));
  x = fmaxf(x, row_ror<1>(x));
  return rows_of(x, max2);
}
__device__ __forceinline__ float wave_sum(float x) {
  x += row_ror<8>(x);
  x += row_ror<4>(x);
  x += row_ror<2>(x);
  x += row_ror<1>(x);
  return rows_of(x, add2);
}

template <int D>
__global__ __launch_bounds__(kThreadsF32) void attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                               const float* __restrict__ v, float* __restrict__ out,
                                                               float* __restrict__ lse, int64_t H, int64_t Sq,
                                                               int64_t Skv, float scale, int64_t chunk, int64_t n_qt,
                                                               int out_bshd) {
  constexpr int E = D / 64;    // d values per lane
  constexpr int KP = D + 4;    // padded K row (floats)
  __shared__ __attribute__((aligned(16))) float ks[kBNF32][KP];
  __shared__ __attribute__((aligned(16))) float vs[kBNF32][D];
  __shared__ __attribute__((aligned(16))) float qs[kRowsF32][D];
  __shared__ __attribute__((aligned(16))) float ps[kRowsF32][kBNF32];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t bh = (int64_t)blockIdx.x / n_qt;
  const int64_t qi = ((int64_t)blockIdx.x - bh * n_qt) * kRowsF32 + w;
  const bool valid = qi < Sq;
  const float* kb = k + bh * Skv * D;
  const float* vb = v + bh * Skv * D;
#pragma unroll
  for (int e = 0; e < E; ++e) qs[w][lane + 64 * e] = valid ? q[(bh * Sq + qi) * D + lane + 64 * e] : 0.f;

  // The thread's share of a tile: kLd 16-byte pieces of K and of V, zero past
  // the tile's n keys.
  constexpr int kLd = kBNF32 * (D / 4) / kThreadsF32;
  float4 kn[kLd], vn[kLd];
  auto fetch = [&](int64_t t0, int n) {
#pragma unroll
    for (int r = 0; r < kLd; ++r) {
      const int i = tid + r * kThreadsF32;
      const int j = i / (D / 4), d4 = (i - j * (D / 4)) * 4;
      kn[r] = vn[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j < n) {
        kn[r] = *reinterpret_cast<const float4*>(kb + (t0 + j) * D + d4);
        vn[r] = *reinterpret_cast<const float4*>(vb + (t0 + j) * D + d4);
      }
    }
  };

  // The running result's log-sum-exp L and each chunk's lse_c are kept in
  // fp64 (by additions only): their difference sets the merge weights, and
  // in fp32 a value near ln Skv would carry ~1e-6 absolute error into every
  // merge.  The transcendental steps stay in fp32 on small arguments: ln of
  // l's mantissa (in [0.5, 1)), and e^-|L - lse_c| with its log1p.
  double L = -INFINITY;
  float o[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  // Tiles run chunk by chunk: [t0, t0 + n) inside the chunk that ends at c1
  // (chunk >= 1; the last chunk ends at Skv).
  int64_t t0 = 0, c1 = chunk < Skv ? chunk : Skv;
  fetch(0, (int)(c1 < kBNF32 ? c1 : kBNF32));
  for (;;) {
    const int n = (int)((c1 - t0 < kBNF32) ? (c1 - t0) : kBNF32);
    __syncthreads();  // the previous tile's readers are done (and qs is written)
#pragma unroll
    for (int r = 0; r < kLd; ++r) {
      const int i = tid + r * kThreadsF32;
      const int j = i / (D / 4), d4 = (i - j * (D / 4)) * 4;
      *reinterpret_cast<float4*>(&ks[j][d4]) = kn[r];
      *reinterpret_cast<float4*>(&vs[j][d4]) = vn[r];
    }
    __syncthreads();
    const int64_t nt0 = t0 + n;
    const bool chunk_end = nt0 >= c1;
    const int64_t nc1 = chunk_end ? ((Skv - c1 < chunk) ? Skv : c1 + chunk) : c1;
    const bool more = nt0 < Skv;
    if (more) fetch(nt0, (int)((nc1 - nt0 < kBNF32) ? (nc1 - nt0) : kBNF32));

    // Logit of key `lane` (four partial sums: independent FMA chains).
    float p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      const float4 kx = *reinterpret_cast<const float4*>(&ks[lane][d]);
      const float4 qx = *reinterpret_cast<const float4*>(&qs[w][d]);
      p4[0] = fmaf(qx.x, kx.x, p4[0]);
      p4[1] = fmaf(qx.y, kx.y, p4[1]);
      p4[2] = fmaf(qx.z, kx.z, p4[2]);
      p4[3] = fmaf(qx.w, kx.w, p4[3]);
    }
    const float s = lane < n ? ((p4[0] + p4[1]) + (p4[2] + p4[3])) * scale : -INFINITY;
    const float mn = fmaxf(m, wave_max(s));
    const float alpha = expf(m - mn);  // m = -inf on the chunk's first tile: alpha = 0
    const float p = lane < n ? expf(s - mn) : 0.f;
    l = l * alpha + wave_sum(p);
    m = mn;
    ps[w][lane] = p;
    __builtin_amdgcn_wave_barrier();  // the wave's own p are written before it reads them
    // P V over all 64 keys of the tile: keys past n have p = 0 and zero V rows.
    float a4[E][4];
#pragma unroll
    for (int e = 0; e < E; ++e) a4[e][0] = a4[e][1] = a4[e][2] = a4[e][3] = 0.f;
#pragma unroll
    for (int j = 0; j < kBNF32; j += 4) {
      const float4 pj = *reinterpret_cast<const float4*>(&ps[w][j]);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        a4[e][0] = fmaf(pj.x, vs[j][lane + 64 * e], a4[e][0]);
        a4[e][1] = fmaf(pj.y, vs[j + 1][lane + 64 * e], a4[e][1]);
        a4[e][2] = fmaf(pj.z, vs[j + 2][lane + 64 * e], a4[e][2]);
        a4[e][3] = fmaf(pj.w, vs[j + 3][lane + 64 * e], a4[e][3]);
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(acc[e], alpha, (a4[e][0] + a4[e][1]) + (a4[e][2] + a4[e][3]));

    if (chunk_end) {
      // explicit log-sum-exp merge of this chunk into the running result
      int le;
      const float lm = frexpf(l, &le);  // l = lm 2^le (l >= 1: the row max's p is 1)
      const double lse_c = (double)m + (double)le * 0.69314718055994530942 + (double)logf(lm);
      // L' = max + ln(1 + t), t = e^-|L - lse_c|; the weights of the two
      // results are 1 / (1 + t) and t / (1 + t) (wb also divides by l).
      double Ln;
      float wa, wb;
      if (L == -INFINITY) {
        Ln = lse_c;
        wa = 0.f;
        wb = 1.0f / l;
      } else {
        const double d = L - lse_c;
        const float t = expf(-(float)fabs(d));
        const float r = 1.0f / (1.0f + t);
        Ln = fmax(L, lse_c) + (double)log1pf(t);
        const bool keep = d >= 0.0;  // the running result is the larger
        wa = keep ? r : t * r;
        wb = (keep ? t * r : r) / l;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        o[e] = o[e] * wa + acc[e] * wb;
        acc[e] = 0.f;
      }
      L = Ln;
      m = -INFINITY;
      l = 0.f;
    }
    if (!more) break;
    t0 = nt0;
    c1 = nc1;
  }
  if (valid) {
    // out row of (b, h, qi): [B, H, Sq, D], or [B, Sq, H, D] (token-major).
    const int64_t b = bh / H;
    const int64_t orow = out_bshd ? (b * Sq + qi) * H + (bh - b * H) : bh * Sq + qi;
#pragma unroll
    for (int e = 0; e < E; ++e) out[orow * D + lane + 64 * e] = o[e];
    if (lse && lane == 0) lse[bh * Sq + qi] = (float)L;
  }
}

}  // namespace

int64_t attn_f32_blocks(int64_t B, int64_t H, int64_t Sq) { return B * H * ((Sq + kRowsF32 - 1) / kRowsF32); }
int attn_f32_threads() { return kThreadsF32; }

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* out, float* lse, int64_t B,
                           int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale, int64_t kv_chunk,
                           bool out_bshd, hipStream_t stream) {
  const int64_t n_qt = (Sq + kRowsF32 - 1) / kRowsF32;
  const unsigned grid = (unsigned)(n_qt * B * H);
  if (D == 64)
    attn_f32_kernel<64><<<grid, kThreadsF32, 0, stream>>>(q, k, v, out, lse, H, Sq, Skv, scale, kv_chunk, n_qt,
                                                          out_bshd ? 1 : 0);
  else
    attn_f32_kernel<128><<<grid, kThreadsF32, 0, stream>>>(q, k, v, out, lse, H, Sq, Skv, scale, kv_chunk, n_qt,
                                                           out_bshd ? 1 : 0);
  return hipGetLastError();
}

}  // namespace r3d
