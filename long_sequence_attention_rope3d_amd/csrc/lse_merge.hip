// lse_merge.hip — n-way log-sum-exp merge of partial attention results.
//
// The ring-attention combine: each ring step attends the local queries to one
// K/V shard, and the partial (O_i, lse_i) of the steps are merged into the
// full-attention result ("Context Parallelism in vLLM Omni Neuron",
// §Ring attention and §Memory and Compute Benefits; xDiT PR "Adds support for
// KV-cache and joint tensors to USP method", ring_attn):
//   L = ln sum_i e^(lse_i),   out = sum_i e^(lse_i - L) O_i.
// A part with lse = -inf has weight 0; a row whose parts are all -inf has no
// keys, and gets out = 0, L = -inf.
//
// HBM-bound: each thread owns 8 consecutive elements of one output row and
// streams the n parts of them (16 or 32 bytes per part, consecutive threads on
// consecutive addresses).  The n weights of a row are recomputed by each of
// its D/8 threads from the (cached) lse values — n exps per thread, far below
// the memory time.  The parts are read with ordinary loads: the non-temporal
// hint measured 11% slower on this 13-stream read pattern.
#include "launch.h"

namespace r3d {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool PBF16>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&x)[8]) {
  if constexpr (PBF16) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + elem);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[2 * w] = __uint_as_float(v[w] << 16);
      x[2 * w + 1] = __uint_as_float(v[w] & 0xffff0000u);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + elem);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
}

template <bool PBF16, bool OBF16>
__global__ __launch_bounds__(256) void lse_merge_kernel(const void* __restrict__ parts,
                                                        const float* __restrict__ lse_parts, int n,
                                                        void* __restrict__ out, float* __restrict__ lse_out,
                                                        int64_t rows, int D, TokenMajor tm) {
  const int cpr = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / cpr;
  const int c = (int)(gid - row * cpr);
  if (row >= rows) return;

  // The first kHeld parts' lse values are loaded together and kept in
  // registers (indices are compile-time, predicated on n, which is uniform);
  // parts beyond them (n > kHeld) are read again as needed.
  // Data loads go out in groups of kG parts: all 16 held parts at once for
  // fp32 parts (4.4% faster than groups of 4 on 13 parts, at 154 VGPRs), 4 for
  // bf16 parts (16 at once was 33% slower there: the occupancy).
  constexpr int kHeld = 16, kG = PBF16 ? 4 : 16;
  float lv[kHeld];
#pragma unroll
  for (int j = 0; j < kHeld; ++j) lv[j] = j < n ? lse_parts[(int64_t)j * rows + row] : -INFINITY;
  float hi = -INFINITY;
#pragma unroll
  for (int j = 0; j < kHeld; ++j) hi = fmaxf(hi, lv[j]);
  for (int i = kHeld; i < n; ++i) hi = fmaxf(hi, lse_parts[(int64_t)i * rows + row]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = -INFINITY;
  if (hi != -INFINITY) {
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < kHeld; ++j)
      if (j < n) sum += expf(lv[j] - hi);
    for (int i = kHeld; i < n; ++i) sum += expf(lse_parts[(int64_t)i * rows + row] - hi);
    L = hi + logf(sum);
    // Data in groups of kG parts: a group's loads are all issued before any
    // is used, so several parts are in flight per thread.
#pragma unroll
    for (int g = 0; g < kHeld; g += kG) {
      if (g < n) {
        float x[kG][8];
#pragma unroll
        for (int j = 0; j < kG; ++j)
          if (g + j < n) load8<PBF16>(parts, ((int64_t)(g + j) * rows + row) * D + c * 8, x[j]);
#pragma unroll
        for (int j = 0; j < kG; ++j) {
          if (g + j < n) {
            const float w = expf(lv[g + j] - L);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, x[j][e], acc[e]);
          }
        }
      }
    }
    for (int i = kHeld; i < n; ++i) {
      const float w = expf(lse_parts[(int64_t)i * rows + row] - L);
      float x[8];
      load8<PBF16>(parts, ((int64_t)i * rows + row) * D + c * 8, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, x[e], acc[e]);
    }
  }
  int64_t orow = row;
  if (tm.H > 0) {  // token-major output: row g = (b*H + h)*Sq + s -> (b*Sq + s)*H + h
    const int64_t g = tm.row0 + row, bh = g / tm.Sq, s = g - bh * tm.Sq, b = bh / tm.H;
    orow = (b * tm.Sq + s) * tm.H + (bh - b * tm.H);
  }
  const int64_t o = orow * D + c * 8;
  if constexpr (OBF16) {
    u32x4 v;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const __bf16 a = (__bf16)acc[2 * w], b = (__bf16)acc[2 * w + 1];
      v[w] = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
    }
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + o) = v;
  } else {
    f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(out) + o);
    p[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    p[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
  if (lse_out && c == 0) lse_out[row] = L;
}

}  // namespace

hipError_t launch_lse_merge(const void* parts, const float* lse_parts, int32_t n, bool parts_bf16, void* out,
                            float* lse_out, bool out_bf16, int64_t rows, int64_t D, hipStream_t stream,
                            const TokenMajor& tm) {
  const int64_t threads = rows * (D / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (parts_bf16 && out_bf16)
    lse_merge_kernel<true, true><<<blocks, 256, 0, stream>>>(parts, lse_parts, n, out, lse_out, rows, (int)D, tm);
  else if (parts_bf16)
    lse_merge_kernel<true, false><<<blocks, 256, 0, stream>>>(parts, lse_parts, n, out, lse_out, rows, (int)D, tm);
  else if (out_bf16)
    lse_merge_kernel<false, true><<<blocks, 256, 0, stream>>>(parts, lse_parts, n, out, lse_out, rows, (int)D, tm);
  else
    lse_merge_kernel<false, false><<<blocks, 256, 0, stream>>>(parts, lse_parts, n, out, lse_out, rows, (int)D, tm);
  return hipGetLastError();
}

}  // namespace r3d
