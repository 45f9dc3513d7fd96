// capi.cpp — the C ABI of librope3d_attn.so (declared in include/r3d_attn.h).
//
// Every argument is validated here, on the host, before anything is
// enqueued; the kernels assume what is checked here (sizes, alignment,
// supported head dims, non-overlap).  No exception crosses the ABI.
#include "r3d_attn.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return R3D_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(R3D_EHIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a*b*... with overflow detection; sizes must be positive.
bool mul_ok(int64_t& acc, int64_t x) {
  int64_t r;
  if (x < 0 || __builtin_mul_overflow(acc, x, &r)) return false;
  acc = r;
  return true;
}

bool product(int64_t& out, std::initializer_list<int64_t> xs) {
  int64_t acc = 1;
  for (int64_t x : xs)
    if (!mul_ok(acc, x)) return false;
  out = acc;
  return true;
}

// Byte ranges [a, a+na) and [b, b+nb) overlap?
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

int elt_size(int32_t dt) { return dt == R3D_F32 ? 4 : dt == R3D_BF16 ? 2 : 0; }

constexpr int64_t kMaxElems = int64_t(1) << 40;  // 1 Ti elements per tensor

// A 1-D launch of `blocks` blocks of `threads` work-items must stay below
// 2^32 work-items in total.
bool launch_fits(int64_t blocks, int64_t threads) {
  return blocks > 0 && blocks <= (int64_t(1) << 31) - 1 && blocks * threads < (int64_t(1) << 32);
}

// Builds the per-pair frequency/axis table of a rotary descriptor for head
// dim D and checks it against the video token count Nv.
int build_rope(const r3d_rope_desc* rope, int64_t D, int64_t Nv, r3d::RopeArgs& out) {
  if (!rope) return fail(R3D_EINVAL, "rope descriptor is NULL");
  if (rope->grid_t < 1 || rope->grid_h < 1 || rope->grid_w < 1)
    return fail(R3D_EINVAL, "rope grid (%lld,%lld,%lld) must be >= 1 on every axis",
                (long long)rope->grid_t, (long long)rope->grid_h, (long long)rope->grid_w);
  int64_t n;
  if (!product(n, {rope->grid_t, rope->grid_h, rope->grid_w}) || n != Nv)
    return fail(R3D_EINVAL, "video token count %lld != grid product %lld*%lld*%lld", (long long)Nv,
                (long long)rope->grid_t, (long long)rope->grid_h, (long long)rope->grid_w);
  const int32_t d[3] = {rope->d_t, rope->d_h, rope->d_w};
  for (int a = 0; a < 3; ++a)
    if (d[a] < 0 || (d[a] & 1))
      return fail(R3D_EINVAL, "rope split (%d,%d,%d): every part must be even and >= 0", d[0], d[1], d[2]);
  if ((int64_t)d[0] + d[1] + d[2] != D)
    return fail(R3D_EINVAL, "rope split (%d,%d,%d) does not sum to D=%lld", d[0], d[1], d[2], (long long)D);
  if (!(std::isfinite(rope->theta) && rope->theta > 0.0))
    return fail(R3D_EINVAL, "rope theta must be finite and > 0");
  if (D / 2 > r3d::kMaxPairs) return fail(R3D_EUNSUPPORTED, "RoPE supports D <= %d", 2 * r3d::kMaxPairs);
  int p = 0;
  for (int a = 0; a < 3; ++a)
    for (int j = 0; j < d[a] / 2; ++j, ++p) {
      out.omega[p] = std::pow(rope->theta, -2.0 * (double)j / (double)d[a]);
      out.axis[p] = (int8_t)a;
    }
  for (; p < r3d::kMaxPairs; ++p) {
    out.omega[p] = 0.0;
    out.axis[p] = 0;
  }
  out.grid_h = rope->grid_h;
  out.grid_w = rope->grid_w;
  out.enabled = 1;
  return R3D_OK;
}

}  // namespace

extern "C" {

R3D_API const char* r3d_last_error(void) { return g_last_error.c_str(); }

R3D_API const char* r3d_version(void) { return "0.1.0 gfx950"; }

R3D_API int r3d_rope3d_apply(const void* x, void* y, int32_t dtype, int64_t B, int64_t Nv,
                             int64_t H, int64_t D, const r3d_rope_desc* rope, void* stream) {
  const int es = elt_size(dtype);
  if (!es) return fail(R3D_EUNSUPPORTED, "rope3d_apply: unknown dtype %d", dtype);
  if (!x || !y) return fail(R3D_EINVAL, "rope3d_apply: NULL tensor pointer");
  if (!aligned16(x) || !aligned16(y)) return fail(R3D_EINVAL, "rope3d_apply: pointers must be 16-byte aligned");
  if (B <= 0 || Nv <= 0 || H <= 0 || D <= 0)
    return fail(R3D_EINVAL, "rope3d_apply: B, Nv, H, D must be > 0");
  if (D != 64 && D != 128) return fail(R3D_EUNSUPPORTED, "rope3d_apply: D=%lld (supported: 64, 128)", (long long)D);
  int64_t n;
  if (!product(n, {B, Nv, H, D}) || n > kMaxElems) return fail(R3D_EINVAL, "rope3d_apply: tensor too large");
  if (x != y && overlap(x, n * es, y, n * es))
    return fail(R3D_EINVAL, "rope3d_apply: x and y overlap without being identical");
  if (!launch_fits(((Nv + r3d::kRopeApplyTok - 1) / r3d::kRopeApplyTok) * B, r3d::kRopeApplyThreads))
    return fail(R3D_EINVAL, "rope3d_apply: B*Nv too large for one launch");
  r3d::RopeArgs ra{};
  int st = build_rope(rope, D, Nv, ra);
  if (st != R3D_OK) return st;
  return hip_status(r3d::launch_rope3d(x, y, dtype == R3D_BF16, B, Nv, H, D, ra, (hipStream_t)stream),
                    "rope3d_apply");
}

namespace {
// Shared by the plain and the QK-norm entry points (norm_w == NULL: no norm).
int permute_impl(const void* const* segs, const int64_t* seg_len, int32_t n_segs, const float* const* norm_w,
                 double eps, void* out, int32_t dtype, int64_t B, int64_t H, int64_t D,
                 const r3d_rope_desc* rope_seg0, void* stream) {
  const int es = elt_size(dtype);
  if (!es) return fail(R3D_EUNSUPPORTED, "joint_concat_permute: unknown dtype %d", dtype);
  if (!segs || !seg_len) return fail(R3D_EINVAL, "joint_concat_permute: NULL segment arrays");
  if (n_segs < 1 || n_segs > r3d::kMaxSegs)
    return fail(R3D_EINVAL, "joint_concat_permute: n_segs=%d (1..%d)", n_segs, r3d::kMaxSegs);
  if (!out || !aligned16(out)) return fail(R3D_EINVAL, "joint_concat_permute: out NULL or not 16-byte aligned");
  if (B <= 0 || H <= 0 || D <= 0) return fail(R3D_EINVAL, "joint_concat_permute: B, H, D must be > 0");
  if ((D * es) % 16 != 0)
    return fail(R3D_EUNSUPPORTED, "joint_concat_permute: a row of D=%lld elements must be a multiple of 16 bytes",
                (long long)D);
  r3d::SegArgs sa{};
  int64_t S = 0;
  for (int i = 0; i < n_segs; ++i) {
    if (seg_len[i] < 0) return fail(R3D_EINVAL, "joint_concat_permute: seg_len[%d] < 0", i);
    if (seg_len[i] > 0 && (!segs[i] || !aligned16(segs[i])))
      return fail(R3D_EINVAL, "joint_concat_permute: segment %d NULL or not 16-byte aligned", i);
    sa.src[i] = segs[i];
    sa.len[i] = seg_len[i];
    sa.off[i] = S;
    if (__builtin_add_overflow(S, seg_len[i], &S)) return fail(R3D_EINVAL, "joint_concat_permute: S overflows");
  }
  sa.n = n_segs;
  sa.S = S;
  if (S <= 0) return fail(R3D_EINVAL, "joint_concat_permute: total sequence length is 0");
  int64_t n_out;
  if (!product(n_out, {B, H, S, D}) || n_out > kMaxElems)
    return fail(R3D_EINVAL, "joint_concat_permute: output too large");
  for (int i = 0; i < n_segs; ++i) {
    int64_t ni;
    product(ni, {B, seg_len[i], H, D});
    if (overlap(segs[i], ni * es, out, n_out * es))
      return fail(R3D_EINVAL, "joint_concat_permute: out overlaps segment %d", i);
  }
  r3d::RopeArgs ra{};
  if (rope_seg0) {
    if (D != 64 && D != 128)
      return fail(R3D_EUNSUPPORTED, "joint_concat_permute: RoPE needs D in {64, 128}, got %lld", (long long)D);
    int st = build_rope(rope_seg0, D, seg_len[0], ra);
    if (st != R3D_OK) return st;
  }
  if (norm_w) {
    if (!std::isfinite(eps) || eps < 0.0)
      return fail(R3D_EINVAL, "joint_concat_permute: norm eps must be finite and >= 0");
    int64_t nw;
    if (!product(nw, {H, D}) || nw > kMaxElems) return fail(R3D_EINVAL, "joint_concat_permute: H*D too large");
    for (int i = 0; i < n_segs; ++i) {
      if (!norm_w[i]) continue;
      if (D != 64 && D != 128)
        return fail(R3D_EUNSUPPORTED, "joint_concat_permute: QK-norm needs D in {64, 128}, got %lld", (long long)D);
      if (!aligned16(norm_w[i]))
        return fail(R3D_EINVAL, "joint_concat_permute: norm weights %d not 16-byte aligned", i);
      if (overlap(norm_w[i], nw * 4, out, n_out * es))
        return fail(R3D_EINVAL, "joint_concat_permute: out overlaps the norm weights of segment %d", i);
      if (seg_len[i] > 0) sa.norm = 1;
      sa.norm_w[i] = norm_w[i];
    }
    sa.norm_eps = eps;
  }
  // tokens and threads per block of the path launch_permute takes
  const bool rot = rope_seg0 != nullptr;
  const int64_t tok = sa.norm ? r3d::kPermuteTokNorm : rot ? r3d::kPermuteTokRope : r3d::kPermuteTok;
  const int64_t threads = sa.norm ? r3d::kPermuteThreadsNorm : rot ? r3d::kPermuteThreadsRope : r3d::kPermuteThreads;
  if (!launch_fits(((S + tok - 1) / tok) * B, threads))
    return fail(R3D_EINVAL, "joint_concat_permute: B*S too large for one launch");
  return hip_status(r3d::launch_permute(sa, out, dtype == R3D_BF16, B, H, D, ra, (hipStream_t)stream),
                    "joint_concat_permute");
}
}  // namespace

R3D_API int r3d_joint_concat_permute(const void* const* segs, const int64_t* seg_len,
                                     int32_t n_segs, void* out, int32_t dtype, int64_t B,
                                     int64_t H, int64_t D, const r3d_rope_desc* rope_seg0,
                                     void* stream) {
  return permute_impl(segs, seg_len, n_segs, nullptr, 0.0, out, dtype, B, H, D, rope_seg0, stream);
}

R3D_API int r3d_joint_concat_permute_qknorm(const void* const* segs, const int64_t* seg_len,
                                            int32_t n_segs, const float* const* norm_w, double eps,
                                            void* out, int32_t dtype, int64_t B, int64_t H, int64_t D,
                                            const r3d_rope_desc* rope_seg0, void* stream) {
  if (!norm_w) return fail(R3D_EINVAL, "joint_concat_permute: NULL norm weight array");
  return permute_impl(segs, seg_len, n_segs, norm_w, eps, out, dtype, B, H, D, rope_seg0, stream);
}

namespace {
// Compute units of the current device (cached per device; 0 if unknown).
int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cus;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cus.find(dev);
  if (it != cus.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
  cus[dev] = n;
  return n;
}

// Device scratch of r3d_attn_fwd_noalloc, for callers that cannot allocate:
// one fixed array per GPU, held until the process ends.  Host code never
// uses the name itself (on the host it is a stand-in, not a device
// address): scratch_ptr() returns the array's address on the current device,
// taken with hipGetSymbolAddress once per device.
constexpr int64_t kScratchBytes = int64_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Address of `scratch` on the current device (NULL and *err set on failure).
void* scratch_ptr(hipError_t* err) {
  static std::mutex mu;
  static std::map<int, void*> addr;
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it != addr.end()) return it->second;
  void* p = nullptr;
  *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (*err != hipSuccess || !p) return nullptr;
  addr[dev] = p;
  return p;
}

constexpr int64_t kWsAlign = 256;  // each workspace region starts on a 256-byte boundary
int64_t ws_round(int64_t bytes) { return (bytes + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Validation shared by every attention entry point (q, k, v, out, lse and the
// sizes); the workspace is checked by the caller of this.
int check_attn_args(const char* what, const void* q, const void* k, const void* v, const void* out,
                    const float* lse, int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale,
                    int32_t dtype, int64_t& nq, int64_t& nk, int64_t& bhq) {
  const int es = elt_size(dtype);
  if (!es) return fail(R3D_EUNSUPPORTED, "%s: unknown dtype %d", what, dtype);
  if (!q || !k || !v || !out) return fail(R3D_EINVAL, "%s: NULL tensor pointer", what);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || (lse && !aligned16(lse)))
    return fail(R3D_EINVAL, "%s: pointers must be 16-byte aligned", what);
  if (B <= 0 || H <= 0 || Sq <= 0 || Skv <= 0 || D <= 0)
    return fail(R3D_EINVAL, "%s: B, H, Sq, Skv, D must be > 0", what);
  if (!std::isfinite(scale)) return fail(R3D_EINVAL, "%s: scale must be finite", what);
  if (D != 64 && D != 128) return fail(R3D_EUNSUPPORTED, "%s: D=%lld (supported: 64, 128)", what, (long long)D);
  if (dtype == R3D_BF16 && (Sq > r3d::kAttnMaxSeq || Skv > r3d::kAttnMaxSeq))
    return fail(R3D_EUNSUPPORTED, "%s: Sq=%lld, Skv=%lld (bf16: at most %lld each)", what, (long long)Sq,
                (long long)Skv, (long long)r3d::kAttnMaxSeq);
  if (!product(nq, {B, H, Sq, D}) || !product(nk, {B, H, Skv, D}) || nq > kMaxElems || nk > kMaxElems)
    return fail(R3D_EINVAL, "%s: tensor too large", what);
  product(bhq, {B, H, Sq});
  if (dtype == R3D_BF16 ? !r3d::attn_bf16_launches_fit(B, H, Sq)
                        : !launch_fits(r3d::attn_f32_blocks(B, H, Sq), r3d::attn_f32_threads()))
    return fail(R3D_EINVAL, "%s: B*H*Sq too large for one launch", what);
  const void* ins[3] = {q, k, v};
  const int64_t in_bytes[3] = {nq * es, nk * es, nk * es};
  for (int i = 0; i < 3; ++i) {
    if (overlap(out, nq * es, ins[i], in_bytes[i])) return fail(R3D_EINVAL, "%s: out overlaps an input", what);
    if (lse && overlap(lse, bhq * 4, ins[i], in_bytes[i])) return fail(R3D_EINVAL, "%s: lse overlaps an input", what);
  }
  if (lse && overlap(lse, bhq * 4, out, nq * es)) return fail(R3D_EINVAL, "%s: lse overlaps out", what);
  return R3D_OK;
}

// The workspace must hold `need` bytes, be 16-byte aligned and overlap no
// tensor of the call.
int check_workspace(const char* what, const void* ws, size_t ws_bytes, int64_t need, const void* q,
                    const void* k, const void* v, const void* out, const float* lse, int64_t nq, int64_t nk,
                    int64_t bhq, int es) {
  if (need == 0) return R3D_OK;
  if (!ws) return fail(R3D_EINVAL, "%s: NULL workspace (this call needs %lld bytes)", what, (long long)need);
  if (!aligned16(ws)) return fail(R3D_EINVAL, "%s: workspace must be 16-byte aligned", what);
  if (ws_bytes < (size_t)need)
    return fail(R3D_EINVAL, "%s: workspace of %llu bytes, this call needs %lld", what,
                (unsigned long long)ws_bytes, (long long)need);
  const void* ts[5] = {q, k, v, out, lse};
  const int64_t tb[5] = {nq * es, nk * es, nk * es, nq * es, lse ? bhq * 4 : 0};
  for (int i = 0; i < 5; ++i)
    if (overlap(ws, need, ts[i], tb[i])) return fail(R3D_EINVAL, "%s: workspace overlaps a tensor", what);
  return R3D_OK;
}

// Workspace plan of a bf16 attn_fwd call: the head statistics, then (for a
// key-split launch) the fp32 partials n_split x rows x (D + 1) of the split
// tiles' rows.
struct AttnPlan {
  r3d::KeySplit ks;
  int64_t stats_bytes = 0, parts_bytes = 0, part_rows = 0;
  int64_t total() const { return stats_bytes + parts_bytes; }
  void unsplit(int64_t B, int64_t H, int64_t Sq, int64_t Skv) {
    ks.waves = r3d::attn_bf16_waves();
    ks.n_bulk = B * H * r3d::attn_bf16_query_tiles(Sq, ks.waves);
    ks.n_split = 1;
    ks.split_len = Skv;
    parts_bytes = part_rows = 0;
  }
};

// n_cus: compute units of the device the call runs on (0: unknown, no key split).
AttnPlan plan_attn(int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, int64_t kv_chunk, int32_t dtype,
                   int n_cus) {
  AttnPlan p;
  p.unsplit(B, H, Sq, Skv);
  if (dtype != R3D_BF16) return p;  // the fp32 kernel needs no workspace
  const int64_t chunk = (kv_chunk == 0 || kv_chunk >= Skv) ? Skv : kv_chunk;
  p.stats_bytes = ws_round(r3d::attn_stats_floats(B, H) * 4);
  p.ks = r3d::attn_bf16_key_split(B, H, Sq, Skv, D, chunk, n_cus);
  {  // the planned grid must still fit a 1-D launch
    const int64_t tiles = B * H * r3d::attn_bf16_query_tiles(Sq, p.ks.waves);
    const int64_t blocks = p.ks.n_split > 1 ? p.ks.n_bulk + (tiles - p.ks.n_bulk) * p.ks.n_split : tiles;
    if (blocks > (int64_t(1) << 31) - 1 || blocks * 64 * p.ks.waves >= (int64_t(1) << 32)) p.unsplit(B, H, Sq, Skv);
  }
  if (p.ks.n_split > 1) {
    p.part_rows = B * H * Sq - r3d::attn_bf16_split_first_row(p.ks.n_bulk, Sq, p.ks.waves);
    p.parts_bytes = ws_round(p.ks.n_split * p.part_rows * (D + 1) * 4);
  }
  return p;
}

int64_t constmax_flags_ints(int64_t B, int64_t H, int64_t Sq) {
  return B * H * r3d::attn_bf16_query_tiles(Sq, r3d::attn_bf16_waves()) * r3d::attn_bf16_waves();
}

// Shared by both output layouts: the validation is identical (out has the
// same number of elements either way).
// scratch_limit >= 0: the call of r3d_attn_fwd_noalloc, whose workspace is
// the fixed scratch array of that many bytes (a key split whose partials do
// not fit runs unsplit; statistics that do not fit are rejected).
int attn_fwd_impl(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B, int64_t H,
                  int64_t Sq, int64_t Skv, int64_t D, float scale, int64_t kv_chunk, int32_t dtype,
                  void* workspace, size_t workspace_bytes, bool out_bshd, void* stream,
                  int64_t scratch_limit = -1) {
  const char* what = scratch_limit >= 0 ? "attn_fwd_noalloc" : "attn_fwd";
  int64_t nq, nk, bhq;
  int st = check_attn_args(what, q, k, v, out, lse, B, H, Sq, Skv, D, scale, dtype, nq, nk, bhq);
  if (st != R3D_OK) return st;
  if (kv_chunk < 0) return fail(R3D_EINVAL, "%s: kv_chunk=%lld < 0", what, (long long)kv_chunk);
  AttnPlan plan = plan_attn(B, H, Sq, Skv, D, kv_chunk, dtype, device_cus());
  if (scratch_limit >= 0 && plan.total() > 0) {
    if (plan.stats_bytes > scratch_limit)
      return fail(R3D_EINVAL, "%s: B*H=%lld needs %lld bytes of scratch, more than the %lld available", what,
                  (long long)(B * H), (long long)plan.stats_bytes, (long long)scratch_limit);
    if (plan.total() > scratch_limit) plan.unsplit(B, H, Sq, Skv);  // partials do not fit: no key split
    hipError_t e = hipSuccess;
    workspace = scratch_ptr(&e);
    if (!workspace) return hip_status(e == hipSuccess ? hipErrorInvalidSymbol : e, what);
    workspace_bytes = (size_t)scratch_limit;
  }
  st = check_workspace(what, workspace, workspace_bytes, plan.total(), q, k, v, out, lse, nq, nk, bhq,
                       elt_size(dtype));
  if (st != R3D_OK) return st;
  const int64_t chunk = (kv_chunk == 0 || kv_chunk >= Skv) ? Skv : kv_chunk;
  const hipStream_t strm = (hipStream_t)stream;
  hipError_t e;
  if (dtype == R3D_BF16) {
    float* stats = static_cast<float*>(workspace);
    // A key split (the last round's tiles run as pieces over key ranges):
    // their fp32 partials follow the statistics.
    float* o_parts = nullptr;
    float* l_parts = nullptr;
    if (plan.ks.n_split > 1) {
      o_parts = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.stats_bytes);
      l_parts = o_parts + plan.ks.n_split * plan.part_rows * D;
    }
    e = r3d::launch_attn_bf16(q, k, v, out, lse, stats, B, H, Sq, Skv, D, scale, chunk, out_bshd, plan.ks, o_parts,
                              l_parts, strm);
  } else
    e = r3d::launch_attn_f32((const float*)q, (const float*)k, (const float*)v, (float*)out, lse, B, H, Sq, Skv,
                             D, scale, chunk, out_bshd, strm);
  return hip_status(e, what);
}

int ws_size_out(const char* what, int64_t need, size_t* bytes) {
  if (!bytes) return fail(R3D_EINVAL, "%s: NULL result pointer", what);
  *bytes = (size_t)need;
  return ok();
}
}  // namespace

R3D_API int r3d_attn_fwd_workspace_size(int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, int64_t kv_chunk,
                                        int32_t dtype, size_t* bytes) {
  const int es = elt_size(dtype);
  if (!es) return fail(R3D_EUNSUPPORTED, "attn_fwd_workspace_size: unknown dtype %d", dtype);
  if (B <= 0 || H <= 0 || Sq <= 0 || Skv <= 0 || D <= 0 || kv_chunk < 0)
    return fail(R3D_EINVAL, "attn_fwd_workspace_size: B, H, Sq, Skv, D must be > 0 and kv_chunk >= 0");
  int64_t bhq;
  if (!product(bhq, {B, H, Sq, D + 1}) || bhq > kMaxElems)
    return fail(R3D_EINVAL, "attn_fwd_workspace_size: sizes too large");
  return ws_size_out("attn_fwd_workspace_size", plan_attn(B, H, Sq, Skv, D, kv_chunk, dtype, device_cus()).total(),
                     bytes);
}

R3D_API int r3d_attn_fwd_plan(int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, int64_t kv_chunk,
                              int32_t n_cus, r3d_attn_plan* plan) {
  if (!plan) return fail(R3D_EINVAL, "attn_fwd_plan: NULL result pointer");
  if (B <= 0 || H <= 0 || Sq <= 0 || Skv <= 0 || D <= 0 || kv_chunk < 0 || n_cus < 0)
    return fail(R3D_EINVAL, "attn_fwd_plan: B, H, Sq, Skv, D must be > 0, kv_chunk and n_cus >= 0");
  if (D != 64 && D != 128) return fail(R3D_EUNSUPPORTED, "attn_fwd_plan: D=%lld (supported: 64, 128)", (long long)D);
  if (Sq > r3d::kAttnMaxSeq || Skv > r3d::kAttnMaxSeq)
    return fail(R3D_EUNSUPPORTED, "attn_fwd_plan: Sq=%lld, Skv=%lld (at most %lld each)", (long long)Sq,
                (long long)Skv, (long long)r3d::kAttnMaxSeq);
  int64_t bhq;
  if (!product(bhq, {B, H, Sq, D + 1}) || bhq > kMaxElems || !r3d::attn_bf16_launches_fit(B, H, Sq))
    return fail(R3D_EINVAL, "attn_fwd_plan: sizes too large");
  const AttnPlan p = plan_attn(B, H, Sq, Skv, D, kv_chunk, R3D_BF16, n_cus);
  plan->waves = p.ks.waves;
  plan->n_split = p.ks.n_split;
  plan->n_tiles = B * H * r3d::attn_bf16_query_tiles(Sq, p.ks.waves);
  plan->n_bulk = p.ks.n_bulk;
  plan->split_len = p.ks.split_len;
  plan->workspace_bytes = p.total();
  return ok();
}

R3D_API int r3d_attn_fwd_constmax_workspace_size(int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                                                 int32_t dtype, size_t* bytes) {
  if (dtype != R3D_BF16) return fail(R3D_EUNSUPPORTED, "attn_fwd_constmax_workspace_size: bf16 only");
  if (B <= 0 || H <= 0 || Sq <= 0 || Skv <= 0 || D <= 0)
    return fail(R3D_EINVAL, "attn_fwd_constmax_workspace_size: B, H, Sq, Skv, D must be > 0");
  int64_t bhq;
  if (!product(bhq, {B, H, Sq}) || bhq > kMaxElems)
    return fail(R3D_EINVAL, "attn_fwd_constmax_workspace_size: sizes too large");
  return ws_size_out("attn_fwd_constmax_workspace_size",
                     ws_round(r3d::attn_stats_floats(B, H) * 4) + ws_round(constmax_flags_ints(B, H, Sq) * 4), bytes);
}

R3D_API int r3d_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                         int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale,
                         int64_t kv_chunk, int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return attn_fwd_impl(q, k, v, out, lse, B, H, Sq, Skv, D, scale, kv_chunk, dtype, workspace, workspace_bytes,
                       false, stream);
}

R3D_API int r3d_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                                 int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale,
                                 int64_t kv_chunk, int32_t dtype, void* stream) {
  return attn_fwd_impl(q, k, v, out, lse, B, H, Sq, Skv, D, scale, kv_chunk, dtype, nullptr, 0, false, stream,
                       kScratchBytes);
}

R3D_API int r3d_attn_fwd_bshd(const void* q, const void* k, const void* v, void* out, float* lse,
                              int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale,
                              int64_t kv_chunk, int32_t dtype, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return attn_fwd_impl(q, k, v, out, lse, B, H, Sq, Skv, D, scale, kv_chunk, dtype, workspace, workspace_bytes,
                       true, stream);
}

R3D_API int r3d_attn_fwd_constmax(const void* q, const void* k, const void* v, void* out, float* lse,
                                  int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale,
                                  int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != R3D_BF16) return fail(R3D_EUNSUPPORTED, "attn_fwd_constmax: bf16 only");
  int64_t nq, nk, bhq;
  int st = check_attn_args("attn_fwd_constmax", q, k, v, out, lse, B, H, Sq, Skv, D, scale, dtype, nq, nk, bhq);
  if (st != R3D_OK) return st;
  const int64_t stats_bytes = ws_round(r3d::attn_stats_floats(B, H) * 4);
  const int64_t need = stats_bytes + ws_round(constmax_flags_ints(B, H, Sq) * 4);
  st = check_workspace("attn_fwd_constmax", workspace, workspace_bytes, need, q, k, v, out, lse, nq, nk, bhq, 2);
  if (st != R3D_OK) return st;
  float* stats = static_cast<float*>(workspace);
  int* flags = reinterpret_cast<int*>(static_cast<char*>(workspace) + stats_bytes);
  return hip_status(r3d::launch_attn_bf16_constmax(q, k, v, out, lse, stats, flags, B, H, Sq, Skv, D, scale,
                                                   (hipStream_t)stream),
                    "attn_fwd_constmax");
}

R3D_API int r3d_lse_merge(const void* o_parts, const float* lse_parts, int32_t n_parts,
                          int32_t parts_dtype, void* out, float* lse_out, int32_t out_dtype,
                          int64_t B, int64_t H, int64_t S, int64_t D, void* stream) {
  const int pes = elt_size(parts_dtype), oes = elt_size(out_dtype);
  if (!pes || !oes) return fail(R3D_EUNSUPPORTED, "lse_merge: unknown dtype");
  if (!o_parts || !lse_parts || !out) return fail(R3D_EINVAL, "lse_merge: NULL tensor pointer");
  if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(out) || (lse_out && !aligned16(lse_out)))
    return fail(R3D_EINVAL, "lse_merge: pointers must be 16-byte aligned");
  if (n_parts < 1 || n_parts > 64) return fail(R3D_EINVAL, "lse_merge: n_parts=%d (1..64)", n_parts);
  if (B <= 0 || H <= 0 || S <= 0 || D <= 0) return fail(R3D_EINVAL, "lse_merge: B, H, S, D must be > 0");
  if (D % 8 != 0 || D > 256) return fail(R3D_EUNSUPPORTED, "lse_merge: D=%lld (multiple of 8, <= 256)", (long long)D);
  int64_t rows, n_o, n_p;
  if (!product(rows, {B, H, S}) || !product(n_o, {rows, D}) || !product(n_p, {n_o, (int64_t)n_parts}) ||
      n_p > kMaxElems)
    return fail(R3D_EINVAL, "lse_merge: tensor too large");
  if (!launch_fits((rows * (D / 8) + 255) / 256, 256)) return fail(R3D_EINVAL, "lse_merge: too many rows for one launch");
  if (overlap(out, n_o * oes, o_parts, n_p * pes) || overlap(out, n_o * oes, lse_parts, rows * n_parts * 4) ||
      (lse_out && (overlap(lse_out, rows * 4, o_parts, n_p * pes) ||
                   overlap(lse_out, rows * 4, lse_parts, rows * n_parts * 4) ||
                   overlap(lse_out, rows * 4, out, n_o * oes))))
    return fail(R3D_EINVAL, "lse_merge: an output overlaps an input or the other output");
  return hip_status(r3d::launch_lse_merge(o_parts, lse_parts, n_parts, parts_dtype == R3D_BF16, out, lse_out,
                                          out_dtype == R3D_BF16, rows, D, (hipStream_t)stream),
                    "lse_merge");
}

}  // extern "C"
