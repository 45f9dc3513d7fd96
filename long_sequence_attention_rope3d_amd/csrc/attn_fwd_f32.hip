// attn_fwd_f32.hip — the all-fp32 attention path (fp32 storage, fp32 math).
//
// Same blockwise algorithm as the bf16 MFMA path, in plain fp32 VALU code:
// keys are visited chunk by chunk; inside a chunk an online softmax keeps a
// running max m, sum l and accumulator acc (rescaled per key tile); at the end
// of every chunk (O_c = acc/l, lse_c = m + ln l) is merged into the running
// result by the log-sum-exp rule
//   L' = ln(e^L + e^lse_c),  O = O e^(L - L') + O_c e^(lse_c - L').
// ("Context Parallelism in vLLM Omni Neuron", §Self-Attention, §Ring
// attention, §Memory and Compute Benefits.)
//
// One thread per query row, 64 rows per block; key/value tiles of kBN rows are
// staged in LDS and read by every thread with broadcast (same-address) loads.
// The merged result O lives in LDS (one padded row per thread), the chunk
// accumulator in registers.
#include "launch.h"

namespace r3d {
namespace {

constexpr int kRows = 64;
constexpr int kBN = 16;

template <int D>
__global__ __launch_bounds__(kRows) void attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                         const float* __restrict__ v, float* __restrict__ out,
                                                         float* __restrict__ lse, int64_t H, int64_t Sq,
                                                         int64_t Skv, float scale, int64_t chunk, int64_t n_qt,
                                                         int out_bshd) {
  __shared__ float ks[kBN][D];
  __shared__ float vs[kBN][D];
  __shared__ float orun[kRows][D + 1];
  const int t = threadIdx.x;
  const int64_t bh = (int64_t)blockIdx.x / n_qt;
  const int64_t qi = ((int64_t)blockIdx.x - bh * n_qt) * kRows + t;
  const bool valid = qi < Sq;
  const float* kb = k + bh * Skv * D;
  const float* vb = v + bh * Skv * D;

  float qr[D];
#pragma unroll
  for (int d = 0; d < D; ++d) qr[d] = valid ? q[(bh * Sq + qi) * D + d] : 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) orun[t][d] = 0.f;

  float L = -INFINITY;
  float acc[D];
  for (int64_t c0 = 0; c0 < Skv; c0 += chunk) {
    const int64_t c1 = (Skv - c0 < chunk) ? Skv : c0 + chunk;
    float m = -INFINITY, l = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = 0.f;
    for (int64_t t0 = c0; t0 < c1; t0 += kBN) {
      const int n = (int)((c1 - t0 < kBN) ? (c1 - t0) : kBN);
      __syncthreads();
      for (int e = t; e < kBN * D; e += kRows) {
        const int j = e / D, d = e - j * D;
        ks[j][d] = j < n ? kb[(t0 + j) * D + d] : 0.f;
        vs[j][d] = j < n ? vb[(t0 + j) * D + d] : 0.f;
      }
      __syncthreads();
      float s[kBN];
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < kBN; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) dot = fmaf(qr[d], ks[j][d], dot);
        s[j] = dot * scale;
        if (j < n) tmax = fmaxf(tmax, s[j]);
      }
      const float mn = fmaxf(m, tmax);
      const float alpha = expf(m - mn);  // m = -inf on the first tile: alpha = 0
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
      for (int j = 0; j < kBN; ++j) {
        const float p = j < n ? expf(s[j] - mn) : 0.f;
        l += p;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[j][d], acc[d]);
      }
      m = mn;
    }
    // explicit log-sum-exp merge of this chunk into the running result
    const float lse_c = m + logf(l);
    const float hi = fmaxf(L, lse_c);
    const float Ln = (L == -INFINITY) ? lse_c : hi + logf(expf(L - hi) + expf(lse_c - hi));
    const float wa = expf(L - Ln);
    const float wb = expf(lse_c - Ln) / l;
#pragma unroll
    for (int d = 0; d < D; ++d) orun[t][d] = orun[t][d] * wa + acc[d] * wb;
    L = Ln;
  }
  if (valid) {
    // out row of (b, h, qi): [B, H, Sq, D], or [B, Sq, H, D] (token-major).
    const int64_t b = bh / H;
    const int64_t orow = out_bshd ? (b * Sq + qi) * H + (bh - b * H) : bh * Sq + qi;
#pragma unroll
    for (int d = 0; d < D; ++d) out[orow * D + d] = orun[t][d];
    if (lse) lse[bh * Sq + qi] = L;
  }
}

}  // namespace

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* out, float* lse, int64_t B,
                           int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale, int64_t kv_chunk,
                           bool out_bshd, hipStream_t stream) {
  const int64_t n_qt = (Sq + kRows - 1) / kRows;
  const unsigned grid = (unsigned)(n_qt * B * H);
  if (D == 64)
    attn_f32_kernel<64><<<grid, kRows, 0, stream>>>(q, k, v, out, lse, H, Sq, Skv, scale, kv_chunk, n_qt,
                                                    out_bshd ? 1 : 0);
  else
    attn_f32_kernel<128><<<grid, kRows, 0, stream>>>(q, k, v, out, lse, H, Sq, Skv, scale, kv_chunk, n_qt,
                                                     out_bshd ? 1 : 0);
  return hipGetLastError();
}

}  // namespace r3d
