// Internal launcher interface between the C-ABI layer (capi.cpp) and the HIP
// kernel files.  Not installed; every argument here has already been checked
// by capi.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace r3d {

constexpr int kMaxSegs = 8;

// Largest Sq and Skv of a bf16 attention call: the kernel keeps query and key
// indices in 32 bits, with a margin for one query tile and one key tile past
// the end.
constexpr int64_t kAttnMaxSeq = (int64_t(1) << 31) - 1024;
constexpr int kMaxPairs = 64;  // D/2 for D = 128

// rope_permute launches, per path (the host's launch-size checks use these):
// plain copy, blocks of kPermuteThreads threads over kPermuteTok consecutive
// tokens; the re-layout with RoPE, kPermuteThreadsRope over kPermuteTokRope;
// rope3d_apply (no re-layout), kRopeApplyThreads over kRopeApplyTok; with the
// QK-norm, kPermuteThreadsNorm over kPermuteTokNorm.
constexpr int kPermuteThreads = 512;
constexpr int kPermuteTok = 4;
constexpr int kPermuteThreadsRope = 256;
constexpr int kPermuteTokRope = 4;
constexpr int kRopeApplyThreads = 256;
constexpr int kRopeApplyTok = 2;
constexpr int kPermuteThreadsNorm = 256;
constexpr int kPermuteTokNorm = 4;

// Rotary tables built on the host: per rotated pair p (0 .. D/2-1) its
// frequency theta^(-2j/d_axis) (double) and its grid axis.
struct RopeArgs {
  double omega[kMaxPairs];
  int8_t axis[kMaxPairs];  // 0 = t, 1 = h, 2 = w
  int64_t grid_h, grid_w;
  int32_t enabled;
};

struct SegArgs {
  const void* src[kMaxSegs];
  int64_t len[kMaxSegs];
  int64_t off[kMaxSegs];
  int32_t n;
  int64_t S;  // sum of len
  // QK-norm: per segment NULL (no norm) or an fp32 weight vector [H*D]; the
  // RMS statistic is over each token's H*D values.
  const float* norm_w[kMaxSegs];
  double norm_eps;
  int32_t norm;  // any norm_w non-NULL
};

// rope3d_apply: [B, Nv, H, D] -> [B, Nv, H, D] (may be in place).
hipError_t launch_rope3d(const void* x, void* y, bool bf16, int64_t B, int64_t Nv, int64_t H,
                         int64_t D, const RopeArgs& rope, hipStream_t stream);

// joint_concat_permute: segments [B, S_i, H, D] -> [B, H, S, D]; rope.enabled
// rotates segment 0; segs.norm applies the per-segment RMS QK-norm first.
hipError_t launch_permute(const SegArgs& segs, void* out, bool bf16, int64_t B, int64_t H,
                          int64_t D, const RopeArgs& rope, hipStream_t stream);

// Head statistics of the bf16 attention path: kStatParts partial maxima per
// head of |k_j|^2 and of |v| (2 * B*H*kStatParts floats of workspace).
constexpr int kStatParts = 64;
inline int64_t attn_stats_floats(int64_t B, int64_t H) { return 2 * B * H * kStatParts; }

// Key split of a bf16 attention launch.  Query tiles are numbered head-major;
// the first n_bulk run over all keys and write out / lse directly.  With
// n_split > 1 each remaining tile runs n_split times, once per range of
// split_len keys (a multiple of kv_chunk, or of the 128-key tile when
// kv_chunk >= Skv), writing fp32 partials that an lse_merge combines into the
// rows of those tiles.
struct KeySplit {
  int waves = 12;  // waves per block: 32 * waves query rows per tile (12, or 8 for grids of few tiles)
  int64_t n_bulk = 0;
  int n_split = 1;
  int64_t split_len = 0;
};
constexpr int kMaxKeySplit = 16;
constexpr int64_t kMinSplitKeys = 512;

// The block shape and split for a launch on a device with n_cus compute
// units: the tiles of the last, partly filled round of blocks are split when
// a cost model of the rounds (and of the partial writes and merge) says that
// is faster, and a grid of few query tiles may take 8-wave blocks.
KeySplit attn_bf16_key_split(int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, int64_t kv_chunk,
                             int n_cus);
// First row (of the [B*H*Sq] rows) of query tile n_bulk for blocks of
// `waves` waves: the split tiles' partials and merged rows start there.
int64_t attn_bf16_split_first_row(int64_t n_bulk, int64_t Sq, int waves);

// attn_fwd, bf16 MFMA path (D = 64 or 128).  out_bshd: out is [B, Sq, H, D]
// instead of [B, H, Sq, D] (a key split's merge writes it token-major too).  stats is a device workspace
// of attn_stats_floats(B, H) floats, written by a pre-pass and read by the
// attention kernel on `stream`.  With ks.n_split > 1, o_parts / l_parts hold
// the pieces' partials [n_split, rows, D] / [n_split, rows] (rows = B*H*Sq -
// attn_bf16_split_first_row(ks.n_bulk, Sq, ks.waves)) and the call ends with their merge.
hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                            float* stats, int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                            float scale, int64_t kv_chunk, bool out_bshd, const KeySplit& ks, float* o_parts,
                            float* l_parts, hipStream_t stream);

// Query tiles per head for blocks of `waves` waves, and the waves per block
// of every launch but small grids' (the constant-max variant always uses it;
// its flags take query_tiles * waves ints per head).
int64_t attn_bf16_query_tiles(int64_t Sq, int waves);
int attn_bf16_waves();

// True when the launches of one bf16 attn_fwd call without a key split (the
// statistics pre-pass and the attention grid) each stay within a 1-D grid's
// 2^31 - 1 blocks and 2^32 work-items.  (A split adds fewer than
// kMaxKeySplit blocks per CU.)
bool attn_bf16_launches_fit(int64_t B, int64_t H, int64_t Sq);

// attn_fwd with a constant per-row softmax reference (the Cauchy-Schwarz
// bound from the head's largest key norm).  stats as above; flags is a
// device workspace of B*H*attn_bf16_query_tiles(Sq)*attn_bf16_waves() ints,
// written by the constant-max kernel (per wave: some row underflowed or is
// not finite) and read by a second launch of the online kernel that
// recomputes the flagged tiles.
hipError_t launch_attn_bf16_constmax(const void* q, const void* k, const void* v, void* out, float* lse,
                                     float* stats, int* flags, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                                     int64_t D, float scale, hipStream_t stream);

// attn_fwd, fp32 path (D = 64 or 128); out_bshd as above.  One wave per
// query row: attn_f32_blocks(B, H, Sq) blocks of attn_f32_threads() threads.
int64_t attn_f32_blocks(int64_t B, int64_t H, int64_t Sq);
int attn_f32_threads();
hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* out, float* lse,
                           int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale,
                           int64_t kv_chunk, bool out_bshd, hipStream_t stream);

// lse_merge: parts [n, rows, D] + lse [n, rows] -> out [rows, D] (+ lse_out).
// With a token-major map (tm.H > 0) merged row r is row g = tm.row0 + r of
// [B*H*Sq] order, (b, h, s), and goes to row (b*Sq + s)*H + h of out
// ([B, Sq, H, D]); lse_out stays indexed by r.
struct TokenMajor {
  int64_t row0 = 0, H = 0, Sq = 0;
};
hipError_t launch_lse_merge(const void* parts, const float* lse_parts, int32_t n, bool parts_bf16,
                            void* out, float* lse_out, bool out_bf16, int64_t rows, int64_t D,
                            hipStream_t stream, const TokenMajor& tm = TokenMajor{});

}  // namespace r3d
