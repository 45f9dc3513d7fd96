// rope_permute.hip — 3-D rotary embedding and the joint concat +
// sequence->head re-layout, as one HBM-bound kernel body.
//
// Operations ("Context Parallelism in vLLM Omni Neuron", §Self-Attention
// with Context Parallelism: RoPE on query/key in [B, S, N, D], then
// transpose(1, 2) to [B, N, S, D]; xDiT PR "Adds support for KV-cache and
// joint tensors to USP method": joint tensors join the sequence inside
// attention; the Ulysses input all-to-all is the multi-device form of the
// re-layout):
//   rope3d_apply         : [B, Nv, H, D] -> [B, Nv, H, D], video tokens rotated
//   joint_concat_permute : segments [B, S_i, H, D] -> [B, H, S, D], optionally
//                          rotating segment 0 (video) on the way through, and
//                          optionally RMS-normalising each token's H*D values
//                          first (QK-norm: norm_q / norm_k act on the projected
//                          q, k before they are split into heads and before
//                          RoPE, same page, §Self-Attention with Context
//                          Parallelism; each of those ops yields a tensor in
//                          the model dtype, so the norm's output is rounded to
//                          the storage type before it is rotated, as a stored
//                          value would be).
//
// Layout of the work.  A block owns kTok (with the QK-norm kTokNorm)
// consecutive tokens of one batch row and all H heads of them.  Per token, the cos/sin of its D/2 pair angles are
// computed once into LDS and reused by all H heads (angles depend only on
// the token).  Each thread then moves 16-byte chunks: a thread keeps one
// (token, chunk) slot and walks the heads, so for a fixed head the block
// reads one contiguous 256-byte row per token and writes that many contiguous
// rows of the [B, H, S, D] output — both sides are full-line, coalesced
// accesses, and no LDS transpose is needed (the re-layout moves whole
// D-rows).  Copies are bit-exact.  Angles, sin/cos and the rotation are
// fp64 — the cos/sin table is per token and shared by all heads, so its cost
// is small — followed by one round-to-nearest-even to the storage type: the
// result is the correctly rounded rotation, also where x0 c - x1 s cancels
// to a value far below |x| (an fp32 rotation is off by several bf16 ulps
// there).
#include "launch.h"

namespace r3d {
namespace {

// Copy: 512-thread blocks of 4 tokens, so that each thread moves only a few
// chunks (3 for 24 heads of 128 bf16) and many blocks are in flight:
// measured 12% faster than 256-thread blocks of 8 tokens whose threads
// walked 12 heads each (a plain 16-byte-per-thread copy of the same bytes
// peaks at about 6.5 TB/s on the MI355X).  The re-layout with RoPE:
// 256-thread blocks of 4 tokens, 6 chunks per thread all loaded before the
// cos/sin table is formed (111.0 vs 116.4 us for 2 tokens and 3 chunks at
// 52k, bit-identical); rope3d_apply keeps 2 tokens and 3 chunks per thread
// (102 vs 106 us the other way round).
constexpr int kThreads = kPermuteThreads;
constexpr int kTok = kPermuteTok;
// With the QK-norm a block is 256 threads over 4 tokens, so that each thread
// holds only a few of its token's chunks (kHold) through the norm's
// reduction: the kernel then fits 6 waves per SIMD instead of 4, and the
// latency of the load -> reduce -> store sequence is hidden by more blocks in
// flight.
constexpr int kThreadsNorm = kPermuteThreadsNorm;
constexpr int kTokNorm = kPermuteTokNorm;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Correctly rounded binary64 -> bfloat16 (round to nearest, ties to even).
// bfloat16 keeps 8 significant bits, so for |y| >= 2^-126 the binary64
// significand is rounded at bit 45 by integer arithmetic; below 2^-126 the
// spacing is fixed at 2^-133 and rint() on the scaled value rounds.  The
// rounded value is exactly representable in binary32, whose upper half is
// the bfloat16 pattern.
__device__ __forceinline__ uint32_t f64_to_bf16(double y) {
  uint64_t u = (uint64_t)__double_as_longlong(y);
  const uint64_t a = u & 0x7fffffffffffffffull;
  double r;
  if (a >= 0x7ff0000000000000ull) {
    r = y;  // inf / nan
  } else if (a >= 0x3810000000000000ull) {  // |y| >= 2^-126
    u += 0x00000fffffffffffull + ((u >> 45) & 1u);
    r = __longlong_as_double((long long)(u & ~0x00001fffffffffffull));
  } else {
    r = rint(y * 0x1p133) * 0x1p-133;
  }
  const uint32_t f = __float_as_uint((float)r);  // exact, or +-inf past the bf16 range
  return ((f & 0x7fffffffu) > 0x7f800000u) ? 0x7fc0u : (f >> 16);
}

// Zero or subnormal binary32: one v_cmp_class_f32 (classes -denorm, -0, +0,
// +denorm), the same set whether or not the mode flushes subnormals.
__device__ __forceinline__ bool zero_or_subnormal(float f) { return __builtin_amdgcn_classf(f, 0xf0); }

// Two binary64 values -> two bfloat16 (y0 in the low half), each rounded
// to nearest-even exactly as f64_to_bf16 does, mostly in hardware: RNE to
// binary32 (v_cvt_f32_f64), then the packed binary32 -> bfloat16 RNE
// (v_cvt_pk_bf16_f32).  bfloat16 midpoints are binary32 values and rounding
// is monotonic, so the first rounding keeps y on its side of every midpoint;
// the pair of roundings can differ from one rounding only when the first
// lands exactly on a midpoint (low 16 bits 0x8000) without being exact --
// or in the binary32 subnormal range.  Lanes meeting either case take
// f64_to_bf16 (rare; a branch per call).
__device__ __forceinline__ uint32_t f64x2_to_bf16x2(double y0, double y1) {
  const float f0 = (float)y0, f1 = (float)y1;
  const uint32_t u0 = __float_as_uint(f0), u1 = __float_as_uint(f1);
  const bool slow = ((u0 & 0xffffu) == 0x8000u) | ((u1 & 0xffffu) == 0x8000u) | zero_or_subnormal(f0) |
                    zero_or_subnormal(f1);
  if (__builtin_expect(slow, 0)) return f64_to_bf16(y0) | (f64_to_bf16(y1) << 16);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{f0, f1}, bf16x2_t));
}

// Rotates the pairs held in one 16-byte chunk.  Pair p of the row is
// (x[2p], x[2p+1]); its (cos, sin) is cs[p].  The rotation is done in fp64
// and rounded once to the storage type.
template <bool BF16>
__device__ __forceinline__ u32x4 rotate_chunk(u32x4 v, const double2* cs, int chunk) {
  if constexpr (BF16) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const double2 c = cs[chunk * 4 + w];
      const double x0 = (double)__uint_as_float(v[w] << 16);
      const double x1 = (double)__uint_as_float(v[w] & 0xffff0000u);
      v[w] = f64x2_to_bf16x2(x0 * c.x - x1 * c.y, x0 * c.y + x1 * c.x);
    }
  } else {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const double2 c = cs[chunk * 2 + p];
      const double x0 = (double)__uint_as_float(v[2 * p]), x1 = (double)__uint_as_float(v[2 * p + 1]);
      v[2 * p] = __float_as_uint((float)(x0 * c.x - x1 * c.y));
      v[2 * p + 1] = __float_as_uint((float)(x0 * c.y + x1 * c.x));
    }
  }
  return v;
}

// QK-norm of one 16-byte chunk: every element x becomes x * r * w (r =
// 1/sqrt(mean square + eps) of its token, w its channel's weight: wa, wb hold
// the chunk's channels 0..7, fp32 rows use wa only), correctly rounded to the
// storage type -- the norm's stored output, which a rotation then reads like
// any stored value.  bfloat16: y32 = x * r32 * w in fp32 (r32 = (float)r;
// three roundings, so |y32 - x r w| <= 3 * 2^-24 |y32| <= 3 ulps of y32), then
// RNE to bfloat16 by v_cvt_pk_bf16_f32.  That is the correctly rounded value
// unless x r w sits within those 3 ulps of a bfloat16 midpoint (a binary32
// value with low half 0x8000): lanes whose y32 is within 4 ulps of one, or
// subnormal, recompute x r w in fp64 and round it exactly (rare: about 9 in
// 65536 values).  binary32 storage: fp64 arithmetic and one rounding.
template <bool BF16>
__device__ __forceinline__ u32x4 norm_chunk(u32x4 v, double r, float4 wa, float4 wb) {
  const float w[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
  if constexpr (BF16) {
    const float r32 = (float)r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float x0 = __uint_as_float(v[q] << 16), x1 = __uint_as_float(v[q] & 0xffff0000u);
      const float y0 = x0 * r32 * w[2 * q], y1 = x1 * r32 * w[2 * q + 1];
      const uint32_t u0 = __float_as_uint(y0), u1 = __float_as_uint(y1);
      const bool slow = (((u0 - 0x7ffcu) & 0xffffu) <= 8u) | (((u1 - 0x7ffcu) & 0xffffu) <= 8u) |
                        zero_or_subnormal(y0) | zero_or_subnormal(y1);
      if (__builtin_expect(slow, 0))
        v[q] = f64_to_bf16((double)x0 * r * (double)w[2 * q]) |
               (f64_to_bf16((double)x1 * r * (double)w[2 * q + 1]) << 16);
      else
        v[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{y0, y1}, bf16x2_t));
    }
  } else {
#pragma unroll
    for (int p = 0; p < 4; ++p)
      v[p] = __float_as_uint((float)((double)__uint_as_float(v[p]) * r * (double)w[p]));
  }
  return v;
}

// Sum of squares of the values in one 16-byte chunk, in fp64 (each square of
// a bfloat16 or binary32 value is exact there; the sums round at 2^-53).
template <bool BF16>
__device__ __forceinline__ double chunk_sumsq(u32x4 v) {
  double s = 0.0;
  if constexpr (BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double x0 = (double)__uint_as_float(v[q] << 16), x1 = (double)__uint_as_float(v[q] & 0xffff0000u);
      s = fma(x0, x0, s);
      s = fma(x1, x1, s);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double x = (double)__uint_as_float(v[q]);
      s = fma(x, x, s);
    }
  }
  return s;
}

// PERMUTE = false: rope3d_apply layout (src and dst both [B, S, H, D], one
//                  segment, every token rotated).
// PERMUTE = true : joint concat into [B, H, S, D]; ROPE rotates segment 0.
// NORM (with PERMUTE, D in {64, 128}): segments with a weight vector get the
// RMS QK-norm before the rotation.
// Block shape of each path: tokens per block and threads per block.
template <bool PERMUTE, bool ROPE, bool NORM>
constexpr int tok_per_block() {
  return NORM ? kTokNorm : !PERMUTE ? kRopeApplyTok : ROPE ? kPermuteTokRope : kTok;
}
template <bool PERMUTE, bool ROPE, bool NORM>
constexpr int threads_per_block() {
  return NORM ? kThreadsNorm : !PERMUTE ? kRopeApplyThreads : ROPE ? kPermuteThreadsRope : kThreads;
}
// 16-byte chunks each thread loads up front and keeps in registers.
template <bool PERMUTE, bool ROPE, bool NORM>
constexpr int chunks_held() { return (NORM || (PERMUTE && ROPE)) ? 6 : 3; }

template <bool BF16, bool PERMUTE, bool ROPE, bool NORM>
__global__ __launch_bounds__((threads_per_block<PERMUTE, ROPE, NORM>())) void rope_permute_kernel(
    SegArgs segs, void* out, int H, int D, int64_t n_tb, RopeArgs rope) {
  constexpr int kT = tok_per_block<PERMUTE, ROPE, NORM>();       // tokens per block
  constexpr int kNT = threads_per_block<PERMUTE, ROPE, NORM>();  // threads per block
  __shared__ double2 cs[kT][kMaxPairs];
  // Norm partial sums, one per (head group, token): hstep * kT = kNT / cpr
  // of them, and cpr >= 8 for the row widths the norm accepts.
  __shared__ double red[NORM ? kNT / 8 : 1];
  const int64_t b = (int64_t)blockIdx.x / n_tb;
  const int64_t tok0 = ((int64_t)blockIdx.x - b * n_tb) * kT;
  const int64_t S = segs.S;
  const int npairs = D / 2;
  const int cpr = D * (BF16 ? 2 : 4) / 16;  // 16-byte chunks per row

  // cos/sin of the block's token angles into LDS, one table entry (token tl,
  // pair p) per thread.  The angle is formed first -- its frequency and axis
  // come from the argument block by a per-thread index, i.e. by vector-memory
  // loads -- and the fp64 sincos and the LDS write only after the thread has
  // issued its chunk loads, so the sincos latency overlaps them instead of
  // waiting for them.  The table is read after the next barrier.
  static_assert(kT * kMaxPairs <= kNT, "one table entry per thread");
  double angle = 0.0;
  const int e_tl = threadIdx.x / npairs, e_p = threadIdx.x - e_tl * npairs;
  const bool has_entry = ROPE && threadIdx.x < kT * npairs;
  if (has_entry) {
    // Token n of the video segment sits at (t, h, w), n = (t*gh + h)*gw + w;
    // other tokens keep angle 0 (cos 1, sin 0).
    const int64_t s = tok0 + e_tl;
    if (s < segs.len[0]) {
      const int64_t w = s % rope.grid_w;
      const int64_t hw = s / rope.grid_w;
      const int64_t h = hw % rope.grid_h;
      const int64_t t = hw / rope.grid_h;
      const int ax = rope.axis[e_p];
      angle = (double)(ax == 0 ? t : (ax == 1 ? h : w)) * rope.omega[e_p];
    }
  }
  auto build_table = [&]() {
    if (has_entry) {
      double sn, c;
      sincos(angle, &sn, &c);
      cs[e_tl][e_p] = make_double2(c, sn);
    }
  };

  const int per_h = kT * cpr;
  // (The host allows NORM only for D in {64, 128}, which always takes this branch.)
  if (NORM || (per_h <= kNT && kNT % per_h == 0)) {
    // Each thread keeps one (token, chunk) slot and walks the heads.
    const int slot = threadIdx.x % per_h;
    const int tl = slot / cpr, chunk = slot - tl * cpr;
    const int hstep = kNT / per_h;
    const int64_t s = tok0 + tl;
    const bool valid = s < S;  // every thread reaches the barrier below
    // A slot past the last token (last block only) loads token S-1 instead,
    // in bounds, so that every thread issues the same loads without a branch;
    // it stores nothing.
    const int64_t sc = valid ? s : S - 1;
    int seg = 0;
    if constexpr (PERMUTE) {
      while (seg + 1 < segs.n && sc >= segs.off[seg + 1]) ++seg;
    }
    const int64_t ls = sc - segs.off[seg];
    const u32x4* src = reinterpret_cast<const u32x4*>(segs.src[seg]) + ((b * segs.len[seg] + ls) * H) * cpr + chunk;
    u32x4* dst = reinterpret_cast<u32x4*>(out);
    const bool rot = ROPE && seg == 0;
    const int epc = 16 / (BF16 ? 2 : 4);  // elements per 16-byte chunk
    const float* wn = nullptr;
    double r = 1.0;
    const int h0 = threadIdx.x / per_h;
    // The thread's first kHold chunks (heads h0, h0 + hstep, ...) are loaded
    // first, all in flight together, and kept in registers for the
    // normalise / rotate / store pass (with a norm they are also summed);
    // heads beyond them (only for H > kHold * hstep) are read afterwards.
    // The loads take no branch (a slot past the thread's last head re-reads
    // head H-1 of the same token, in bounds, and is not used): with a branch
    // around them the compiler copied the loaded registers at the join, i.e.
    // waited for the loads before the table below.
    constexpr int kHold = chunks_held<PERMUTE, ROPE, NORM>();  // all of them for bf16, D = 128, H <= 24
    u32x4 held[kHold];
    const int nh = (valid && H > h0) ? (H - h0 + hstep - 1) / hstep : 0;  // this thread's heads
    auto ld = [&](int h) {
      return NORM ? src[(int64_t)h * cpr] : __builtin_nontemporal_load(src + (int64_t)h * cpr);
    };
#pragma unroll
    for (int i = 0; i < kHold; ++i) held[i] = ld(min(h0 + i * hstep, H - 1));
    build_table();
    if constexpr (NORM) {
      // Pass 1: the token's sum of squares over all H*D values.  The cpr
      // threads of token tl in each of the hstep head groups are consecutive
      // lanes of one wave: they reduce by butterfly shuffles, and the group
      // partials meet in LDS behind one barrier; every thread then forms its
      // token's r itself.
      wn = valid ? segs.norm_w[seg] : nullptr;
      double ss = 0.0;
      if (wn) {
#pragma unroll
        for (int i = 0; i < kHold; ++i)
          if (i < nh) ss += chunk_sumsq<BF16>(held[i]);
        for (int h = h0 + kHold * hstep; h < H; h += hstep) ss += chunk_sumsq<BF16>(src[(int64_t)h * cpr]);
      }
      for (int m = cpr / 2; m > 0; m >>= 1) ss += __shfl_xor(ss, m, cpr);
      if (chunk == 0) red[h0 * kT + tl] = ss;
      __syncthreads();  // also publishes the cos/sin table
      if (!valid) return;
      double t = 0.0;
      for (int g = 0; g < hstep; ++g) t += red[g * kT + tl];
      r = 1.0 / sqrt(t / (double)((int64_t)H * D) + segs.norm_eps);
    }
    if constexpr (!NORM) {
      if constexpr (ROPE) __syncthreads();  // the cos/sin table
      if (!valid) return;
    }
    auto store = [&](int h, u32x4 v) {
      const int64_t o = PERMUTE ? (((b * H + h) * S + s) * cpr + chunk) : (((b * S + s) * H + h) * cpr + chunk);
      __builtin_nontemporal_store(v, dst + o);
    };
    if (NORM && wn) {
      // Pass 2 with a norm: from the registers, then the re-read tail.  The
      // chunk's weights (epc fp32 values, 16-byte aligned) are loaded one
      // head ahead, before the previous head's store, so their L2 latency
      // overlaps the arithmetic.
      auto wload = [&](int h, float4& a, float4& c) {
        const float4* wp = reinterpret_cast<const float4*>(wn + (int64_t)h * D + chunk * epc);
        a = wp[0];
        c = BF16 ? wp[1] : a;
      };
      float4 wa = {}, wb = {};
      if (nh > 0) wload(h0, wa, wb);
#pragma unroll
      for (int i = 0; i < kHold; ++i) {
        if (i < nh) {
          const int h = h0 + i * hstep;
          float4 na = wa, nb = wb;
          if (i + 1 < nh) wload(h + hstep, na, nb);
          u32x4 y = norm_chunk<BF16>(held[i], r, wa, wb);
          if (rot) y = rotate_chunk<BF16>(y, cs[tl], chunk);
          store(h, y);
          wa = na;
          wb = nb;
        }
      }
      for (int h = h0 + kHold * hstep; h < H; h += hstep) {
        wload(h, wa, wb);
        u32x4 y = norm_chunk<BF16>(src[(int64_t)h * cpr], r, wa, wb);
        if (rot) y = rotate_chunk<BF16>(y, cs[tl], chunk);
        store(h, y);
      }
    } else {
      // Copy / rotate: the held chunks, then any remaining heads.
#pragma unroll
      for (int i = 0; i < kHold; ++i) {
        if (i < nh) {
          u32x4 v = held[i];
          if (rot) v = rotate_chunk<BF16>(v, cs[tl], chunk);
          store(h0 + i * hstep, v);
        }
      }
      for (int h = h0 + kHold * hstep; h < H; h += hstep) {
        u32x4 v = ld(h);
        if (rot) v = rotate_chunk<BF16>(v, cs[tl], chunk);
        store(h, v);
      }
    }
  } else {
    // Generic row widths (no RoPE: any D whose row is a multiple of 16 bytes).
    build_table();
    if constexpr (ROPE) __syncthreads();
    const int64_t items = (int64_t)per_h * H;
    for (int64_t idx = threadIdx.x; idx < items; idx += kNT) {
      const int h = (int)(idx / per_h);
      const int slot = (int)(idx - (int64_t)h * per_h);
      const int tl = slot / cpr, chunk = slot - tl * cpr;
      const int64_t s = tok0 + tl;
      if (s >= S) continue;
      int seg = 0;
      if constexpr (PERMUTE) {
        while (seg + 1 < segs.n && s >= segs.off[seg + 1]) ++seg;
      }
      const int64_t ls = s - segs.off[seg];
      u32x4 v = reinterpret_cast<const u32x4*>(segs.src[seg])[((b * segs.len[seg] + ls) * H + h) * cpr + chunk];
      if (ROPE && seg == 0) v = rotate_chunk<BF16>(v, cs[tl], chunk);
      const int64_t o = PERMUTE ? (((b * H + h) * S + s) * cpr + chunk) : (((b * S + s) * H + h) * cpr + chunk);
      reinterpret_cast<u32x4*>(out)[o] = v;
    }
  }
}

template <bool PERMUTE, bool ROPE, bool NORM = false>
hipError_t launch_typed(bool bf16, const SegArgs& segs, void* out, int64_t B, int64_t H, int64_t D,
                        const RopeArgs& rope, hipStream_t stream) {
  constexpr int kT = tok_per_block<PERMUTE, ROPE, NORM>();
  constexpr int kNT = threads_per_block<PERMUTE, ROPE, NORM>();
  const int64_t n_tb = (segs.S + kT - 1) / kT;  // token blocks per batch row
  const unsigned grid = (unsigned)(n_tb * B);
  if (bf16)
    rope_permute_kernel<true, PERMUTE, ROPE, NORM><<<grid, kNT, 0, stream>>>(segs, out, (int)H, (int)D, n_tb, rope);
  else
    rope_permute_kernel<false, PERMUTE, ROPE, NORM><<<grid, kNT, 0, stream>>>(segs, out, (int)H, (int)D, n_tb, rope);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope3d(const void* x, void* y, bool bf16, int64_t B, int64_t Nv, int64_t H, int64_t D,
                         const RopeArgs& rope, hipStream_t stream) {
  SegArgs segs{};
  segs.src[0] = x;
  segs.len[0] = Nv;
  segs.off[0] = 0;
  segs.n = 1;
  segs.S = Nv;
  return launch_typed<false, true>(bf16, segs, y, B, H, D, rope, stream);
}

hipError_t launch_permute(const SegArgs& segs, void* out, bool bf16, int64_t B, int64_t H, int64_t D,
                          const RopeArgs& rope, hipStream_t stream) {
  if (segs.norm) {
    if (rope.enabled) return launch_typed<true, true, true>(bf16, segs, out, B, H, D, rope, stream);
    return launch_typed<true, false, true>(bf16, segs, out, B, H, D, rope, stream);
  }
  if (rope.enabled) return launch_typed<true, true>(bf16, segs, out, B, H, D, rope, stream);
  return launch_typed<true, false>(bf16, segs, out, B, H, D, rope, stream);
}

}  // namespace r3d
