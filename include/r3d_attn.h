/*
 * r3d_attn.h — C ABI of librope3d_attn.so: joint-sequence attention with 3-D
 * rotary embeddings for video(+audio) diffusion transformers, on one AMD
 * MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Buffers are DEVICE pointers owned by the caller, contiguous (row-major)
 *    in the layout stated per call, 16-byte aligned.  The library allocates
 *    no device memory at run time (the one fixed array of r3d_attn_fwd_noalloc
 *    is part of the loaded library), keeps no pointer to caller memory after
 *    it returns, and creates no stream.
 *    Calls that need device scratch memory take a caller-owned `workspace`
 *    of at least the size their *_workspace_size query reports; its contents
 *    on entry and on return mean nothing to the caller, and it is used in
 *    stream order on `stream` (do not hand it to other work until the call's
 *    work on that stream has finished).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    null stream).  A return of R3D_OK means the work was enqueued; errors of
 *    the kernels themselves surface on the stream like any HIP error.
 *  - Arguments are validated on the host before anything is enqueued.  On
 *    failure nothing is launched, the return is a negative r3d_status, and
 *    r3d_last_error() describes it.  No C++ exception crosses the ABI.
 *  - Outputs must not alias inputs unless a call says otherwise.
 *  - Thread safety: calls may be made from several host threads; the error
 *    message is per thread.
 */
#ifndef R3D_ATTN_H
#define R3D_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define R3D_API __attribute__((visibility("default")))
#else
#define R3D_API
#endif

typedef enum {
  R3D_OK = 0,
  R3D_EINVAL = -1,        /* bad argument: NULL/misaligned pointer, size, split, aliasing */
  R3D_EUNSUPPORTED = -2,  /* valid request that this library has no kernel for (D, dtype) */
  R3D_EHIP = -3           /* the HIP runtime reported an error at launch */
} r3d_status;

typedef enum {
  R3D_F32 = 0,   /* IEEE binary32 */
  R3D_BF16 = 1   /* bfloat16, stored as the upper 16 bits of binary32 */
} r3d_dtype;

/*
 * 3-D rotary embedding of the video tokens.  The pages apply
 * apply_rotary_emb_wan(query/key, freqs_cos, freqs_sin) to Q and K (never V)
 * before the transpose to [B, N, S, D], with rotary tables indexed by
 * sequence position ("Context Parallelism in vLLM Omni Neuron",
 * §Self-Attention with Context Parallelism, §Positional Embedding Handling).
 * The formula itself is not printed there; this library's definition:
 *  - video token n of a segment sits at grid position (t, h, w) with
 *    n = (t*grid_h + h)*grid_w + w (row-major latent grid, §Problem);
 *  - the head dimension is split into contiguous [d_t | d_h | d_w];
 *  - in the segment of axis a, pair (off_a + 2j, off_a + 2j + 1) turns by
 *    angle p_a * theta^(-2j/d_a), i.e. (x0, x1) -> (x0 c - x1 s, x0 s + x1 c);
 *  - d_a may be 0 (2-D RoPE on an image uses d_t = 0).
 * Angles, sin/cos and the rotation are computed in fp64 and the result is
 * rounded once to the storage dtype (round-to-nearest-even).
 */
typedef struct {
  int64_t grid_t, grid_h, grid_w;  /* video tokens = grid_t*grid_h*grid_w       */
  int32_t d_t, d_h, d_w;           /* even, >= 0, d_t + d_h + d_w == D          */
  double theta;                    /* base, finite and > 0 (10000 here)         */
} r3d_rope_desc;

/*
 * r3d_rope3d_apply — rotate the video tokens of Q or K.
 *   x, y : [B, Nv, H, D] in `dtype`; y == x (in place) is allowed, any other
 *          overlap is rejected.  Nv must equal the grid product of `rope`.
 *   D    : 64 or 128.
 * Errors: R3D_EINVAL (NULL/misaligned, sizes <= 0, split/grid mismatch,
 * partial overlap), R3D_EUNSUPPORTED (D or dtype), R3D_EHIP.
 */
R3D_API int r3d_rope3d_apply(const void* x, void* y, int32_t dtype, int64_t B, int64_t Nv,
                             int64_t H, int64_t D, const r3d_rope_desc* rope, void* stream);

/*
 * r3d_joint_concat_permute — joint concat + sequence->head re-layout.
 * The single-device form of the Ulysses input all-to-all followed by
 * .transpose(1, 2) ("Context Parallelism in vLLM Omni Neuron",
 * §Self-Attention with Context Parallelism; xDiT PR "Adds support for
 * KV-cache and joint tensors to USP method": joint tensors are concatenated
 * to the visual sequence inside attention):
 *     out[b, h, off_i + s, :] = segs[i][b, s, h, :],  off_i = sum_{j<i} seg_len[j]
 *   segs    : HOST array of n_segs DEVICE pointers, segment i is [B, seg_len[i], H, D]
 *             (video first, then audio, then text); a segment of length 0 may be NULL.
 *   seg_len : HOST array of n_segs lengths >= 0, sum S > 0.  1 <= n_segs <= 8.
 *   out     : [B, H, S, D] in `dtype`; must not overlap any segment.
 *   rope_seg0 : NULL -> a pure copy, bit-exact.  Otherwise segment 0 (the video
 *             tokens, seg_len[0] == grid product) is rotated as r3d_rope3d_apply
 *             would while it is copied (one HBM round trip instead of two);
 *             the other segments are copied bit-exactly (joint tokens carry no
 *             position).
 * Errors: R3D_EINVAL, R3D_EUNSUPPORTED (D not 64/128 with RoPE, dtype), R3D_EHIP.
 * Without RoPE any D >= 1 whose row is a multiple of 16 bytes is accepted.
 */
R3D_API int r3d_joint_concat_permute(const void* const* segs, const int64_t* seg_len,
                                     int32_t n_segs, void* out, int32_t dtype, int64_t B,
                                     int64_t H, int64_t D, const r3d_rope_desc* rope_seg0,
                                     void* stream);

/*
 * r3d_joint_concat_permute_qknorm — r3d_joint_concat_permute with the QK-norm
 * fused in front of the rotation ("Context Parallelism in vLLM Omni Neuron",
 * §Self-Attention with Context Parallelism: norm_q / norm_k act on the
 * projected q, k — one token's H*D values before .unflatten into heads — and
 * then the rotary embedding is applied; §Distributed Normalization: the
 * statistic is the sum of squares over that hidden dimension):
 *     x <- x / sqrt(mean(x^2 over the token's H*D values) + eps) * w
 * for every token of segment i when norm_w[i] != NULL, then RoPE on segment 0
 * when rope_seg0 != NULL, then the re-layout.  Norm, rotation and rounding
 * are fp64 with one round-to-nearest-even store (the composition is rounded
 * once, not after each step).
 *   norm_w : HOST array of n_segs pointers, each NULL (segment copied, or only
 *            rotated) or a DEVICE fp32 vector of H*D weights, 16-byte aligned.
 *   eps    : finite, >= 0 (the pages give no value; 1e-6 is a common choice).
 *   D      : 64 or 128 when any weight vector is given.
 *   Other arguments as r3d_joint_concat_permute.
 * Errors: as r3d_joint_concat_permute, plus R3D_EINVAL for a NULL norm_w
 * array, misaligned weights, bad eps or out overlapping weights.
 */
R3D_API int r3d_joint_concat_permute_qknorm(const void* const* segs, const int64_t* seg_len,
                                            int32_t n_segs, const float* const* norm_w, double eps,
                                            void* out, int32_t dtype, int64_t B, int64_t H, int64_t D,
                                            const r3d_rope_desc* rope_seg0, void* stream);

/*
 * r3d_attn_fwd — full non-causal multi-head attention, blockwise.
 * ("Context Parallelism in vLLM Omni Neuron", §Self-Attention:
 * _nf_attend(query, key, value, scale) on [B, N, S, D]; §Ring attention and
 * §Full K/V AllGather: local Q attends the full K/V, one K/V chunk at a time;
 * xDiT PR #586: _attention(query, key, value, dropout_p, is_causal) with no
 * dropout and is_causal false for DiT self-attention.)
 *   q   : [B, H, Sq, D];  k, v : [B, H, Skv, D];  all in `dtype`.
 *   out : [B, H, Sq, D] in `dtype` (bf16 rounded to nearest-even from fp32).
 *   lse : [B, H, Sq] fp32 natural-log log-sum-exp of the scaled logits, or NULL.
 *   scale : logit multiplier (finite; 1/sqrt(D) in every workload here).
 *   kv_chunk : keys are processed in chunks [c*kv_chunk, (c+1)*kv_chunk); inside a
 *           chunk the softmax is online (running max / sum, rescaled per key tile);
 *           each finished chunk (O_c = acc/l, lse_c = m + ln l) is combined into the
 *           running result by an explicit log-sum-exp merge
 *             L' = ln(e^L + e^lse_c), O = O e^(L-L') + O_c e^(lse_c-L'),
 *           in registers, with no partials written to memory.  0 or >= Skv means one
 *           chunk.  The result equals softmax(q k^T scale) v for every kv_chunk (up to
 *           rounding).
 *   D   : 64 or 128.  dtype R3D_BF16 runs on bf16 MFMA with fp32 accumulation and an
 *         fp32 softmax (P rounded to bf16 for the PV product); R3D_F32 is an all-fp32
 *         path.
 *   workspace, workspace_bytes : device scratch of at least
 *         r3d_attn_fwd_workspace_size(...) bytes (0 for R3D_F32, where workspace may be
 *         NULL), 16-byte aligned, overlapping no tensor of the call.  The R3D_BF16 path
 *         keeps there per-head statistics of K and V (2*B*H*64 floats: partial maxima of
 *         |k_j|^2 for a Cauchy-Schwarz bound on every row's logits, and of |v|) and, for
 *         a key-split launch, the fp32 partials (below).
 * Block shape and key split (R3D_BF16): the query tiles (384 rows of one
 *   head each; for D = 128 a grid of few tiles may use 256-row tiles instead)
 *   run one block per tile, a round of blocks per round of the GPU's compute
 *   units.  When the last round would leave many units idle, the tiles of
 *   that round instead run as up to 16 blocks each over ranges of whole
 *   chunks (whole 128-key tiles with one chunk, at least 512 keys), and the
 *   ranges' fp32 partials (O, lse) are merged by the lse_merge kernel into
 *   those tiles' rows -- the ring's per-shard partial + merge, on one device.
 *   A cost model of the rounds picks the tile height and the split (either
 *   must gain 2%).  The result equals that of any other choice up to
 *   rounding.  r3d_attn_fwd_bshd plans the same way (its merge writes token-major rows).
 * Errors: R3D_EINVAL (NULL/misaligned, sizes <= 0, kv_chunk < 0, non-finite scale,
 * out/lse overlapping an input, a workspace that is NULL, too small, misaligned or
 * overlapping a tensor), R3D_EUNSUPPORTED (D, dtype, or for R3D_BF16 an Sq or Skv
 * above 2^31 - 1024: that kernel indexes rows in 32 bits), R3D_EHIP.
 */
R3D_API int r3d_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                         int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale,
                         int64_t kv_chunk, int32_t dtype, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * r3d_attn_fwd_workspace_size — bytes of workspace r3d_attn_fwd needs for these
 * arguments on the CURRENT device (the key-split decision depends on its number of
 * compute units); r3d_attn_fwd_bshd needs the same.  Writes *bytes; performs
 * no device work and allocates nothing.
 * Errors: R3D_EINVAL (sizes <= 0, kv_chunk < 0, NULL bytes, overflow),
 * R3D_EUNSUPPORTED (dtype).
 */
R3D_API int r3d_attn_fwd_workspace_size(int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                                        int64_t kv_chunk, int32_t dtype, size_t* bytes);

/*
 * r3d_attn_fwd_plan — the launch plan r3d_attn_fwd (and r3d_attn_fwd_bshd) would use for
 * R3D_BF16 arguments on a device with n_cus compute units (0: unknown, which plans no key
 * split): the tile height and the key split described under r3d_attn_fwd (the ring's
 * per-shard partials and their log-sum-exp merge, "Context Parallelism in vLLM Omni
 * Neuron", §Ring attention).  A host query: performs no device work, allocates nothing.
 *   plan->waves           waves per block; a query tile is 32 * waves rows of one head
 *   plan->n_tiles         query tiles, B * H * ceil(Sq / (32 * waves)), head-major
 *   plan->n_bulk          tiles [0, n_bulk) run over all keys in one block each
 *   plan->n_split         tiles [n_bulk, n_tiles) run as n_split blocks over key ranges
 *                         of split_len keys (1: no split, n_bulk = n_tiles)
 *   plan->split_len       keys per range (a whole number of kv_chunk chunks)
 *   plan->workspace_bytes r3d_attn_fwd's workspace for this plan
 * Errors: R3D_EINVAL (NULL plan, sizes <= 0, kv_chunk or n_cus < 0, sizes too large),
 * R3D_EUNSUPPORTED (D, or Sq or Skv above 2^31 - 1024).
 */
typedef struct r3d_attn_plan {
  int32_t waves;
  int32_t n_split;
  int64_t n_tiles;
  int64_t n_bulk;
  int64_t split_len;
  int64_t workspace_bytes;
} r3d_attn_plan;
R3D_API int r3d_attn_fwd_plan(int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, int64_t kv_chunk,
                              int32_t n_cus, r3d_attn_plan* plan);

/*
 * r3d_attn_fwd_noalloc — r3d_attn_fwd without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Its scratch is a
 * fixed 16 MiB device array inside the library, one per GPU, held until the process
 * ends; its address is looked up once per device on the first call.
 *   Limit: the R3D_BF16 path needs 512 * B * H bytes of per-head statistics, so B*H
 *   above 32768 is rejected (R3D_EINVAL).  A launch that r3d_attn_fwd would key-split
 *   runs unsplit when the split's fp32 partials do not fit beside them (the result
 *   then differs from r3d_attn_fwd's only by rounding).  R3D_F32 uses no scratch.
 *   Concurrency: every call on one GPU shares that GPU's array, so calls whose work
 *   overlaps on one GPU (different streams, or threads without ordering) race; calls
 *   in order on one stream are safe.  Nothing in the array needs clearing between
 *   calls (each call writes all it reads).
 *   Other arguments, output and errors as r3d_attn_fwd.
 */
R3D_API int r3d_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                                 int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale,
                                 int64_t kv_chunk, int32_t dtype, void* stream);

/*
 * r3d_attn_fwd_bshd — r3d_attn_fwd with the output written token-major:
 *   out : [B, Sq, H, D] (everything else, lse and workspace included, as in
 *         r3d_attn_fwd).
 * This is the inverse of the [B, S, H, D] -> [B, H, S, D] re-layout done by
 * r3d_joint_concat_permute, i.e. the local form of the Ulysses output
 * all-to-all that returns the head-sharded result to sequence order (xDiT PR
 * #586, USP: _ft_c_output_all_to_all(out)), and the token-major form that the
 * output projection consumes ("Context Parallelism in vLLM Omni Neuron",
 * §Self-Attention: o_proj after _nf_attend).  Same arithmetic as
 * r3d_attn_fwd: the values are identical, only their placement differs.
 * Errors: as r3d_attn_fwd.
 */
R3D_API int r3d_attn_fwd_bshd(const void* q, const void* k, const void* v, void* out, float* lse,
                              int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale,
                              int64_t kv_chunk, int32_t dtype, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * r3d_attn_fwd_constmax — r3d_attn_fwd (bf16, out [B, H, Sq, D], one chunk) whose
 * softmax reference is a per-row bound fixed before any key is read instead of
 * the running max: the kernel of "Context Parallelism in vLLM Omni Neuron",
 * §Related information (ring_attention_const_max_fwd: "softmax max is a
 * runtime bound"), where a known bound lets K/V chunks be consumed in any
 * order with no rescaling — chunk partials simply add, no log-sum-exp merge.
 * The bound is Cauchy-Schwarz:  m_i = |scale| |q_i| max_j |k_j|  >=  every
 * logit of row i; p = e^(s - m_i) <= 1, out = sum p v / sum p,
 * lse = m_i + ln(sum p).  Where the bound exceeds a row's true maximum by more
 * than fp32's exponent range can carry (the row sum falls below 2^-100, or the
 * output is not finite), the block tile holding that row is recomputed inside
 * the same call with the running-max reference, so every row gets
 * r3d_attn_fwd's result: no row comes back silently underflowed.
 *   workspace, workspace_bytes : device scratch of at least
 *             r3d_attn_fwd_constmax_workspace_size(...) bytes, 16-byte aligned,
 *             overlapping no tensor of the call (per-head statistics of K and V,
 *             and one flag per wave of every block tile).
 *   dtype   : R3D_BF16 only.  Other arguments as r3d_attn_fwd (no kv_chunk:
 *             with a fixed reference the chunking does not change the result).
 * Errors: as r3d_attn_fwd, and R3D_EUNSUPPORTED for fp32.
 */
R3D_API int r3d_attn_fwd_constmax(const void* q, const void* k, const void* v, void* out, float* lse,
                                  int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale,
                                  int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/* r3d_attn_fwd_constmax_workspace_size — bytes of workspace r3d_attn_fwd_constmax
 * needs for these sizes (writes *bytes; no device work).  Errors as
 * r3d_attn_fwd_workspace_size, and R3D_EUNSUPPORTED for fp32. */
R3D_API int r3d_attn_fwd_constmax_workspace_size(int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                                                 int32_t dtype, size_t* bytes);

/*
 * r3d_lse_merge — combine n partial attention results of the same queries
 * against disjoint key sets (the ring-attention combine: each ring step
 * attends one K/V shard, "Context Parallelism in vLLM Omni Neuron",
 * §Ring attention; xDiT PR #586, ring_attn):
 *     L = ln sum_i e^(lse_i),   out = sum_i e^(lse_i - L) o_i
 *   o_parts   : [n_parts, B, H, S, D] in parts_dtype (F32 or BF16).
 *   lse_parts : [n_parts, B, H, S] fp32, natural log; -inf marks an empty part
 *               (weight 0).  A row whose parts are all -inf gets out = 0, L = -inf.
 *   out       : [B, H, S, D] in out_dtype;  lse_out : [B, H, S] fp32 or NULL.
 *   1 <= n_parts <= 64; D a multiple of 8, <= 256.
 * Errors: R3D_EINVAL, R3D_EUNSUPPORTED, R3D_EHIP.
 */
R3D_API int r3d_lse_merge(const void* o_parts, const float* lse_parts, int32_t n_parts,
                          int32_t parts_dtype, void* out, float* lse_out, int32_t out_dtype,
                          int64_t B, int64_t H, int64_t S, int64_t D, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
R3D_API const char* r3d_last_error(void);

/* Library version string, e.g. "0.1.0 gfx950". */
R3D_API const char* r3d_version(void);

#ifdef __cplusplus
}
#endif

#endif /* R3D_ATTN_H */
