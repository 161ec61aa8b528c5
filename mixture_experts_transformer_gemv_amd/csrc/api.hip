// C ABI of the Grok-1 MoE layer library (declarations and contracts in include/grok_moe.h).
//
// Host side only: argument validation, workspace layout, choice of kernel family, and the launches on the
// caller's stream.  Nothing here allocates memory or synchronises.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "../../include/grok_moe.h"
#include "launch.h"

namespace {

constexpr int64_t kMaxTokens = int64_t(1) << 24;
// At most this many tokens: few rows per expert -> weight-streaming kernels (16 or 32 rows per pass over the
// weights), else the LDS-tiled kernels.  Measured on MI355X at the Grok-1 shape: bf16 streams win up to T = 96
// (T = 96: 1.50 against 1.64 ms per layer) and lose at T = 128 (two passes for most experts: 2.46 against 1.66);
// int8 tiles spend their MFMA time on padding rows at small T, and the int8 streams win up to T = 128 (grouped
// scales, T = 128: 1.51 against 2.08 ms; one scale group: even at T = 128, slower from T = 160).
constexpr int kStreamMaxTokensBf16 = 96;
constexpr int kStreamMaxTokensInt8 = 128;
int stream_max_tokens(int dtype) {
  return dtype == GROK_MOE_W8 ? kStreamMaxTokensInt8 : kStreamMaxTokensBf16;
}

struct Plan {
  int64_t slots;
  bool stream;  // streaming kernels (else LDS-tiled grouped GEMM or the fp32 kernels)
  int mt;       // 16-row MFMA tiles per pass of the streaming kernels
  int mt_oi;    // the same for the [out, in] streaming kernels
  int splits;   // partial sums of the down-projection
  size_t o_idx, o_p, o_counts, o_offsets, o_perm, o_inv, o_h, o_y, total;
  size_t o_xn, total_block;  // the block form adds the normed input [T, d]
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

int check_shape(int64_t T, int64_t d, int64_t f, int E, int k, int dtype) {
  if (dtype != GROK_MOE_F32 && dtype != GROK_MOE_BF16 && dtype != GROK_MOE_W8) return GROK_MOE_EINVAL;
  if (T < 0 || d <= 0 || f <= 0) return GROK_MOE_EINVAL;
  if (k != 2 || E < 2 || E > 64) return GROK_MOE_EUNSUPPORTED;
  if (T > kMaxTokens || d > (int64_t(1) << 20) || f > (int64_t(1) << 20)) return GROK_MOE_EUNSUPPORTED;
  const int64_t g = dtype == GROK_MOE_F32 ? 64 : 256;
  if (d % g != 0 || f % g != 0) return GROK_MOE_EUNSUPPORTED;
  if (d * f >= (int64_t(1) << 31)) return GROK_MOE_EUNSUPPORTED;  // one expert matrix < 2^32 bytes (32-bit offsets)
  return GROK_MOE_OK;
}

// Tokens of one pass of the layer.  The LDS-tiled kernels of the bf16 and int8 layers (direct-to-LDS copies)
// address x [T, d] and h [2 T, f], both bf16, with 32-bit byte offsets below 2^31; longer batches run as several
// passes over consecutive token ranges (the layer treats tokens independently; only the expert counts are
// summed).  The fp32 kernels address with 64-bit offsets.
int64_t max_pass_tokens(int64_t d, int64_t f, int dtype) {
  if (dtype == GROK_MOE_F32) return kMaxTokens;
  const int64_t lim = (int64_t(1) << 31) - 1;
  return std::max<int64_t>(stream_max_tokens(dtype) + 1, std::min(lim / (2 * d), lim / (4 * f)));
}

// T tokens as n passes of near-equal size: the first `rem` passes take base + 1 tokens, the others base.
struct Passes {
  int64_t n, base, rem;
  int64_t start(int64_t i) const { return i * base + std::min(i, rem); }
  int64_t size(int64_t i) const { return base + (i < rem ? 1 : 0); }
};
Passes passes(int64_t T, int64_t d, int64_t f, int dtype) {
  const int64_t m = max_pass_tokens(d, f, dtype);
  const int64_t n = std::max<int64_t>(1, (T + m - 1) / m);
  return Passes{n, T / n, T % n};
}

int down_splits(int64_t T, int64_t f, int E, int dtype) {
  // LDS-tiled bf16 down-projection: K split in two, so that its tiles fill the chip in more, shorter rounds
  if (dtype == GROK_MOE_BF16 && T > stream_max_tokens(dtype)) return 2;
  // fp32 layer: a small batch gives few tiles, each a long chain of 16-deep K steps: for T <= 256 split K into
  // up to 8 parts of at least 128 k (partial sums added by the combine)
  if (dtype == GROK_MOE_F32) {
    int s = 1;
    while (T <= 256 && s < 8 && f / (2 * s) >= 128 && (f / (2 * s)) % 16 == 0) s *= 2;
    return s;
  }
  if (T > stream_max_tokens(dtype)) return 1;
  // near-equal chunks of at least 2048 rows of W2 with boundaries on multiples of 128 rows: at most 5 (measured
  // against 3, 4, 6, 8 and 16 chunks), or 2 for bf16 16-row token tiles with at least as many tokens as experts
  // (every expert likely hit: fewer, longer weight streams read faster there; measured on MI355X at Grok-1 shape,
  // down-projection ms with 5 -> 2 chunks: T = 8 0.465 -> 0.452, T = 16 0.470 -> 0.456, but T = 4 0.329 -> 0.350,
  // T = 64 0.484 -> 0.496, int8 with grouped scales 0.292 -> 0.389)
  if (f % 128 != 0) return 1;
  const int64_t most = (dtype == GROK_MOE_BF16 && T <= 16 && T >= E) ? 2 : 5;
  return int(std::min<int64_t>(most, std::max<int64_t>(1, f / 2048)));
}

Plan make_plan(int64_t T, int64_t d, int64_t f, int E, int dtype) {
  Plan p;
  p.slots = 2 * T;
  p.stream = dtype != GROK_MOE_F32 && T <= stream_max_tokens(dtype);
  p.mt = T <= 16 ? 1 : 2;
  p.mt_oi = T <= 16 ? 1 : 2;  // (4 tiles measured slower at T = 64: the token tile outgrows the weight tile)
  p.splits = down_splits(T, f, E, dtype);
  size_t o = 0;
  p.o_idx = o; o = align256(o + size_t(p.slots) * 4);
  p.o_p = o; o = align256(o + size_t(p.slots) * 4);
  p.o_counts = o; o = align256(o + size_t(E) * 4);
  p.o_offsets = o; o = align256(o + size_t(E + 1) * 4);
  p.o_perm = o; o = align256(o + size_t(p.slots) * 4);
  p.o_inv = o; o = align256(o + size_t(p.slots) * 4);
  p.o_h = o; o = align256(o + size_t(p.slots) * f * (dtype == GROK_MOE_F32 ? 4 : 2));
  p.o_y = o; o = align256(o + size_t(p.splits) * p.slots * d * 4);
  p.total = o;
  p.o_xn = o; o = align256(o + size_t(T) * d * (dtype == GROK_MOE_F32 ? 4 : 2));
  p.total_block = o;
  return p;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
inline bool ok_opt(const void* p) { return p == nullptr || aligned16(p); }

int check_scales(int dtype, const void* s1, const void* sv, const void* s2) {
  if (dtype == GROK_MOE_W8) return (ok_ptr(s1) && ok_ptr(sv) && ok_ptr(s2)) ? GROK_MOE_OK : GROK_MOE_EINVAL;
  return (s1 == nullptr && sv == nullptr && s2 == nullptr) ? GROK_MOE_OK : GROK_MOE_EINVAL;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? GROK_MOE_OK : GROK_MOE_EHIP; }

// Weight storage ([E, in, out] or [E, out, in]) and int8 scale tensors [scale_experts, groups, out]; the default
// is [E, in, out] with per-expert scales of one group.
struct ScaleSpec {
  int experts;  // 1 (shared by all experts) or E
  int g_up;     // groups along d of W1 / Wv
  int g_down;   // groups along f of W2
  bool outin = false;  // weights stored [E, out, in]
};

inline bool ok_layout(int weight_layout) {
  return weight_layout == GROK_MOE_IN_OUT || weight_layout == GROK_MOE_OUT_IN;
}

int check_groups(const ScaleSpec& sp, int64_t d, int64_t f, int E) {
  if ((sp.experts != 1 && sp.experts != E) || sp.g_up < 1 || sp.g_down < 1) return GROK_MOE_EINVAL;
  if (d % sp.g_up != 0 || (d / sp.g_up) % 64 != 0) return GROK_MOE_EUNSUPPORTED;
  if (f % sp.g_down != 0 || (f / sp.g_down) % 64 != 0) return GROK_MOE_EUNSUPPORTED;
  return GROK_MOE_OK;
}

inline gm::ScaleLayout up_layout(const ScaleSpec& sp, int64_t d, int64_t f) {
  return gm::ScaleLayout{sp.experts == 1 ? 0 : int64_t(sp.g_up) * f, int(d / sp.g_up)};
}
inline gm::ScaleLayout down_layout(const ScaleSpec& sp, int64_t d, int64_t f) {
  return gm::ScaleLayout{sp.experts == 1 ? 0 : int64_t(sp.g_down) * d, int(f / sp.g_down)};
}

// ---- the steps, without argument checks (callers have validated)
hipError_t do_up(const void* x, const void* w1, const void* wv, const void* s1, const void* sv, const ScaleSpec& sp,
                 const int32_t* counts, const int32_t* offsets, const int32_t* perm, const Plan& p, int64_t d,
                 int64_t f, int E, int dtype, void* h, hipStream_t s) {
  if (dtype == GROK_MOE_F32)
    return gm::launch_up_f32(static_cast<const float*>(x), static_cast<const float*>(w1),
                             static_cast<const float*>(wv), sp.outin, counts, offsets, perm, int(d), int(f), E,
                             int(p.slots), static_cast<float*>(h), s);
  const bool i8 = dtype == GROK_MOE_W8;
  if (p.stream && sp.outin && gm::oi_stream_fits(int(d), i8, up_layout(sp, d, f), int(d)))
    return gm::launch_up_stream_oi(static_cast<const uint16_t*>(x), w1, wv, static_cast<const uint16_t*>(s1),
                                   static_cast<const uint16_t*>(sv), up_layout(sp, d, f), counts, offsets, perm,
                                   int(d), int(f), E, int(p.slots), i8, p.mt_oi, static_cast<uint16_t*>(h), s);
  if (p.stream)
    return gm::launch_up_stream(static_cast<const uint16_t*>(x), w1, wv, static_cast<const uint16_t*>(s1),
                                static_cast<const uint16_t*>(sv), up_layout(sp, d, f), sp.outin, counts, offsets,
                                perm, int(d), int(f), E, int(p.slots), i8, p.mt, static_cast<uint16_t*>(h), s);
  return gm::launch_up_tiled(static_cast<const uint16_t*>(x), w1, wv, static_cast<const uint16_t*>(s1),
                             static_cast<const uint16_t*>(sv), up_layout(sp, d, f), sp.outin, counts, offsets, perm,
                             int(d), int(f), E, int(p.slots), i8, static_cast<uint16_t*>(h), s);
}

hipError_t do_down(const void* h, const void* w2, const void* s2, const ScaleSpec& sp, const int32_t* counts,
                   const int32_t* offsets, const Plan& p, int64_t d, int64_t f, int E, int dtype, float* y,
                   hipStream_t s) {
  if (dtype == GROK_MOE_F32)
    return gm::launch_down_f32(static_cast<const float*>(h), static_cast<const float*>(w2), sp.outin, counts,
                               offsets, int(d), int(f), E, int(p.slots), p.splits, y, s);
  const bool i8 = dtype == GROK_MOE_W8;
  if (p.stream && sp.outin && gm::oi_stream_fits(int(f), i8, down_layout(sp, d, f), int(f)))
    return gm::launch_down_stream_oi(static_cast<const uint16_t*>(h), w2, static_cast<const uint16_t*>(s2),
                                     down_layout(sp, d, f), counts, offsets, int(d), int(f), E, int(p.slots),
                                     p.splits, i8, p.mt_oi, y, s);
  if (p.stream)
    return gm::launch_down_stream(static_cast<const uint16_t*>(h), w2, static_cast<const uint16_t*>(s2),
                                  down_layout(sp, d, f), sp.outin, counts, offsets, int(d), int(f), E, int(p.slots),
                                  p.splits, i8, p.mt, y, s);
  return gm::launch_down_tiled(static_cast<const uint16_t*>(h), w2, static_cast<const uint16_t*>(s2),
                               down_layout(sp, d, f), sp.outin, counts, offsets, int(d), int(f), E, int(p.slots),
                               p.splits, i8, y, s);
}

// Workspace of the whole layer: the larger of the two pass sizes (block: with the normed input).
size_t workspace_need(int64_t T, int64_t d, int64_t f, int E, int dtype, bool block) {
  const Passes ps = passes(T, d, f, dtype);
  size_t need = 0;
  for (int64_t n : {ps.base + (ps.rem ? 1 : 0), ps.base}) {
    if (n <= 0) continue;
    const Plan p = make_plan(n, d, f, E, dtype);
    need = std::max(need, block ? p.total_block : p.total);
  }
  return need;
}

// One pass of the layer over T tokens, its workspace at ws; the block form if pre_scale is given.  The counts of
// the pass are written to expert_counts, or added to it if add_counts.
hipError_t run_pass(const void* x, const void* pre_scale, const void* post_scale, double eps, const void* router_w,
                    const void* w1, const void* wv, const void* w2, const void* s1, const void* sv, const void* s2,
                    const ScaleSpec& sp, int64_t T, int64_t d, int64_t f, int E, int dtype, float* out,
                    const float* router_bias, int32_t* topk_idx, float* topk_p, int32_t* expert_counts,
                    bool add_counts, char* ws, hipStream_t s) {
  const Plan p = make_plan(T, d, f, E, dtype);
  const bool bf = dtype != GROK_MOE_F32, block = pre_scale != nullptr;
  int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(ws + p.o_idx);
  float* pr = topk_p ? topk_p : reinterpret_cast<float*>(ws + p.o_p);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + p.o_counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + p.o_offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(ws + p.o_perm);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + p.o_inv);
  void* h = ws + p.o_h;
  float* y = reinterpret_cast<float*>(ws + p.o_y);
  const void* xe = block ? ws + p.o_xn : x;  // the experts' input

  hipError_t e = block ? gm::launch_router_norm(x, pre_scale, eps, router_w, router_bias, int(T), int(d), E, bf,
                                                ws + p.o_xn, idx, pr, s)
                       : gm::launch_router(x, router_w, router_bias, int(T), int(d), E, bf, idx, pr, s);
  if (e == hipSuccess) e = gm::launch_bin(idx, int(T), E, counts, offsets, perm, inv, s);
  if (e == hipSuccess) e = do_up(xe, w1, wv, s1, sv, sp, counts, offsets, perm, p, d, f, E, dtype, h, s);
  if (e == hipSuccess) e = do_down(h, w2, s2, sp, counts, offsets, p, d, f, E, dtype, y, s);
  if (e == hipSuccess)
    e = block ? gm::launch_combine_norm(y, p.splits, pr, inv, int(T), int(d), x, bf, post_scale, eps, out, s)
              : gm::launch_combine(y, p.splits, pr, inv, int(T), int(d), out, s);
  if (e == hipSuccess && expert_counts) e = gm::launch_counts_out(expert_counts, counts, E, add_counts, s);
  return e;
}

// The whole layer (grok_moe_forward, grok_moe_block_forward and their forms) as passes over consecutive token
// ranges; arguments validated by the caller.
int run_layer(const void* x, const void* pre_scale, const void* post_scale, double eps, const void* router_w,
              const void* w1, const void* wv, const void* w2, const void* s1, const void* sv, const void* s2,
              const ScaleSpec& sp, int64_t T, int64_t d, int64_t f, int E, int dtype, float* out,
              const float* router_bias, int32_t* topk_idx, float* topk_p, int32_t* expert_counts, void* workspace,
              size_t workspace_bytes, hipStream_t stream) {
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return GROK_MOE_EINVAL;
  if (workspace_bytes < workspace_need(T, d, f, E, dtype, pre_scale != nullptr)) return GROK_MOE_EWORKSPACE;
  const Passes ps = passes(T, d, f, dtype);
  const size_t xrow = size_t(d) * (dtype == GROK_MOE_F32 ? 4 : 2);  // bytes per token of x
  hipError_t e = hipSuccess;
  for (int64_t i = 0; i < ps.n && e == hipSuccess; ++i) {
    const int64_t t0 = ps.start(i);
    e = run_pass(static_cast<const char*>(x) + t0 * xrow, pre_scale, post_scale, eps, router_w, w1, wv, w2, s1, sv,
                 s2, sp, ps.size(i), d, f, E, dtype, out + t0 * d, router_bias,
                 topk_idx ? topk_idx + 2 * t0 : nullptr, topk_p ? topk_p + 2 * t0 : nullptr, expert_counts, i > 0,
                 static_cast<char*>(workspace), stream);
  }
  return hip_status(e);
}

// ---- argument checks shared by the entry points

// Scale spec of an entry point's (weight_layout, scale_experts, groups) arguments; GROK_MOE_OK or a status.
int make_spec(grok_moe_layout weight_layout, int scale_experts, int groups_up, int groups_down, int64_t d,
              int64_t f, int E, grok_moe_dtype dtype, ScaleSpec* sp) {
  if (!ok_layout(weight_layout)) return GROK_MOE_EINVAL;
  *sp = ScaleSpec{E, 1, 1, weight_layout == GROK_MOE_OUT_IN};
  if (dtype != GROK_MOE_W8) return GROK_MOE_OK;
  sp->experts = scale_experts;
  sp->g_up = groups_up;
  sp->g_down = groups_down;
  return check_groups(*sp, d, f, E);
}

// The whole layer (or the block if pre_scale != NULL): shape, pointer and scale checks, then the passes.
int layer_entry(const void* x, const void* pre_scale, const void* post_scale, double eps, const void* router_w,
                const void* w1, const void* wv, const void* w2, const void* s1, const void* sv, const void* s2,
                grok_moe_layout weight_layout, int scale_experts, int groups_up, int groups_down, int64_t T,
                int64_t d, int64_t f, int E, int k, grok_moe_dtype dtype, float* out, const float* router_bias,
                int32_t* topk_idx, float* topk_p, int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  int st = check_shape(T, d, f, E, k, dtype);
  if (st != GROK_MOE_OK) return st;
  const bool block = pre_scale != nullptr || post_scale != nullptr;
  if (block && !(eps >= 0.0)) return GROK_MOE_EINVAL;
  ScaleSpec sp;
  if ((st = make_spec(weight_layout, scale_experts, groups_up, groups_down, d, f, E, dtype, &sp)) != GROK_MOE_OK)
    return st;
  if (T == 0) return GROK_MOE_OK;
  if (!ok_ptr(x) || !ok_ptr(router_w) || !ok_ptr(w1) || !ok_ptr(wv) || !ok_ptr(w2) || !ok_ptr(out))
    return GROK_MOE_EINVAL;
  if (block && (!ok_ptr(pre_scale) || !ok_ptr(post_scale))) return GROK_MOE_EINVAL;
  if (!ok_opt(router_bias) || !ok_opt(topk_idx) || !ok_opt(topk_p) || !ok_opt(expert_counts)) return GROK_MOE_EINVAL;
  if ((st = check_scales(dtype, s1, sv, s2)) != GROK_MOE_OK) return st;
  return run_layer(x, pre_scale, post_scale, eps, router_w, w1, wv, w2, s1, sv, s2, sp, T, d, f, E, dtype, out,
                   router_bias, topk_idx, topk_p, expert_counts, workspace, workspace_bytes, stream);
}

// ---- the scratch memory of grok_moe_forward_noalloc: one static device array, a copy on every GPU.  In host code
// `scratch` is only a host-side stand-in for the symbol; its device address on each GPU comes from
// hipGetSymbolAddress with that GPU current, looked up once per device and kept here.
constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch_slots[kMaxDevices];

}  // namespace

static __device__ __align__(256) unsigned char scratch[GROK_MOE_SCRATCH_BYTES];

namespace {

// Device address of the current device's scratch array (resolved on the first call with that device current).
hipError_t current_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ScratchSlot& slot = g_scratch_slots[dev];
  std::call_once(slot.once, [&slot] { slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch)); });
  if (slot.err != hipSuccess) return slot.err;
  if (slot.ptr == nullptr || (reinterpret_cast<uintptr_t>(slot.ptr) & 255) != 0) return hipErrorInvalidSymbol;
  *out = slot.ptr;
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* grok_moe_strerror(int status) {
  switch (status) {
    case GROK_MOE_OK: return "ok";
    case GROK_MOE_EINVAL: return "invalid argument (NULL or misaligned pointer, negative size, unknown dtype or "
                                 "layout)";
    case GROK_MOE_EUNSUPPORTED: return "unsupported shape (needs k == 2, 2 <= E <= 64, d and f multiples of 256 "
                                       "for bf16/int8 or of 64 for fp32, d * f < 2^31; the expert step entry "
                                       "points take at most one pass of tokens)";
    case GROK_MOE_EWORKSPACE: return "workspace too small";
    case GROK_MOE_EHIP: return "HIP kernel launch failed";
    case GROK_MOE_ESCRATCH: return "the batch needs more workspace than the static scratch array of "
                                   "grok_moe_forward_noalloc holds (GROK_MOE_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

size_t grok_moe_workspace_size(int64_t T, int64_t d, int64_t f, int E, int k, grok_moe_dtype dtype) {
  if (check_shape(T, d, f, E, k, dtype) != GROK_MOE_OK || T == 0) return 0;
  return workspace_need(T, d, f, E, dtype, false);
}

int grok_moe_down_splits(int64_t T, int64_t d, int64_t f, int E, int k, grok_moe_dtype dtype) {
  if (check_shape(T, d, f, E, k, dtype) != GROK_MOE_OK) return 1;
  return make_plan(passes(T, d, f, dtype).size(0), d, f, E, dtype).splits;
}

int grok_moe_forward_ex(const void* x, const void* router_w, const void* w1, const void* wv, const void* w2,
                        const void* s1, const void* sv, const void* s2, grok_moe_layout weight_layout,
                        int scale_experts, int groups_up, int groups_down, int64_t T, int64_t d, int64_t f, int E,
                        int k, grok_moe_dtype dtype, float* out, const float* router_bias, int32_t* topk_idx,
                        float* topk_p, int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  return layer_entry(x, nullptr, nullptr, 0.0, router_w, w1, wv, w2, s1, sv, s2, weight_layout, scale_experts,
                     groups_up, groups_down, T, d, f, E, k, dtype, out, router_bias, topk_idx, topk_p, expert_counts,
                     workspace, workspace_bytes, stream);
}

int grok_moe_forward(const void* x, const void* router_w, const void* w1, const void* wv, const void* w2,
                     const void* s1, const void* sv, const void* s2, int64_t T, int64_t d, int64_t f, int E, int k,
                     grok_moe_dtype dtype, float* out, const float* router_bias, int32_t* topk_idx, float* topk_p,
                     int32_t* expert_counts, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return layer_entry(x, nullptr, nullptr, 0.0, router_w, w1, wv, w2, s1, sv, s2, GROK_MOE_IN_OUT, E, 1, 1, T, d, f,
                     E, k, dtype, out, router_bias, topk_idx, topk_p, expert_counts, workspace, workspace_bytes,
                     stream);
}

int grok_moe_route(const void* x, const void* router_w, const float* router_bias, int64_t T, int64_t d, int E, int k,
                   grok_moe_dtype dtype, int32_t* topk_idx, float* topk_p, hipStream_t stream) {
  int st = check_shape(T, d, dtype == GROK_MOE_F32 ? 64 : 256, E, k, dtype);
  if (st != GROK_MOE_OK) return st;
  if (T == 0) return GROK_MOE_OK;
  if (!ok_ptr(x) || !ok_ptr(router_w) || !ok_ptr(topk_idx) || !ok_ptr(topk_p) || !ok_opt(router_bias))
    return GROK_MOE_EINVAL;
  return hip_status(gm::launch_router(x, router_w, router_bias, int(T), int(d), E, dtype != GROK_MOE_F32, topk_idx,
                                      topk_p, stream));
}

int grok_moe_bin(const int32_t* topk_idx, int64_t T, int E, int k, int32_t* counts, int32_t* offsets, int32_t* perm,
                 int32_t* inv, hipStream_t stream) {
  if (T < 0) return GROK_MOE_EINVAL;
  if (k != 2 || E < 2 || E > 64 || T > kMaxTokens) return GROK_MOE_EUNSUPPORTED;
  if (!ok_ptr(counts) || !ok_ptr(offsets)) return GROK_MOE_EINVAL;
  if (T > 0 && (!ok_ptr(topk_idx) || !ok_ptr(perm) || !ok_ptr(inv))) return GROK_MOE_EINVAL;
  return hip_status(gm::launch_bin(topk_idx, int(T), E, counts, offsets, perm, inv, stream));
}

int grok_moe_expert_up(const void* x, const void* w1, const void* wv, const void* s1, const void* sv,
                       grok_moe_layout weight_layout, int scale_experts, int groups_up, const int32_t* counts,
                       const int32_t* offsets, const int32_t* perm, int64_t T, int64_t d, int64_t f, int E, int k,
                       grok_moe_dtype dtype, void* h, hipStream_t stream) {
  int st = check_shape(T, d, f, E, k, dtype);
  if (st != GROK_MOE_OK) return st;
  if (T > max_pass_tokens(d, f, dtype)) return GROK_MOE_EUNSUPPORTED;  // one pass only (32-bit offsets)
  ScaleSpec sp;
  if ((st = make_spec(weight_layout, scale_experts, groups_up, 1, d, f, E, dtype, &sp)) != GROK_MOE_OK) return st;
  if (T == 0) return GROK_MOE_OK;
  if (!ok_ptr(x) || !ok_ptr(w1) || !ok_ptr(wv) || !ok_ptr(counts) || !ok_ptr(offsets) || !ok_ptr(perm) || !ok_ptr(h))
    return GROK_MOE_EINVAL;
  if ((st = check_scales(dtype, s1, sv, dtype == GROK_MOE_W8 ? s1 : nullptr)) != GROK_MOE_OK) return st;
  const Plan p = make_plan(T, d, f, E, dtype);
  return hip_status(do_up(x, w1, wv, s1, sv, sp, counts, offsets, perm, p, d, f, E, dtype, h, stream));
}

int grok_moe_expert_down(const void* h, const void* w2, const void* s2, grok_moe_layout weight_layout,
                         int scale_experts, int groups_down, const int32_t* counts, const int32_t* offsets,
                         int64_t T, int64_t d, int64_t f, int E, int k, grok_moe_dtype dtype, int splits, float* y,
                         hipStream_t stream) {
  int st = check_shape(T, d, f, E, k, dtype);
  if (st != GROK_MOE_OK) return st;
  if (T > max_pass_tokens(d, f, dtype)) return GROK_MOE_EUNSUPPORTED;  // one pass only (32-bit offsets)
  ScaleSpec sp;
  if ((st = make_spec(weight_layout, scale_experts, 1, groups_down, d, f, E, dtype, &sp)) != GROK_MOE_OK) return st;
  const Plan p = make_plan(T, d, f, E, dtype);
  if (splits != p.splits) return GROK_MOE_EINVAL;
  if (T == 0) return GROK_MOE_OK;
  if (!ok_ptr(h) || !ok_ptr(w2) || !ok_ptr(counts) || !ok_ptr(offsets) || !ok_ptr(y)) return GROK_MOE_EINVAL;
  if (dtype == GROK_MOE_W8 ? !ok_ptr(s2) : s2 != nullptr) return GROK_MOE_EINVAL;
  return hip_status(do_down(h, w2, s2, sp, counts, offsets, p, d, f, E, dtype, y, stream));
}

int grok_moe_combine(const float* y, int splits, const float* topk_p, const int32_t* inv, int64_t T, int64_t d, int k,
                     float* out, hipStream_t stream) {
  if (T < 0 || d <= 0 || splits < 1 || splits > 64) return GROK_MOE_EINVAL;
  if (k != 2 || T > kMaxTokens || d % 4 != 0) return GROK_MOE_EUNSUPPORTED;
  if (T == 0) return GROK_MOE_OK;
  if (!ok_ptr(y) || !ok_ptr(topk_p) || !ok_ptr(inv) || !ok_ptr(out)) return GROK_MOE_EINVAL;
  return hip_status(gm::launch_combine(y, splits, topk_p, inv, int(T), int(d), out, stream));
}

size_t grok_moe_block_workspace_size(int64_t T, int64_t d, int64_t f, int E, int k, grok_moe_dtype dtype) {
  if (check_shape(T, d, f, E, k, dtype) != GROK_MOE_OK || T == 0) return 0;
  return workspace_need(T, d, f, E, dtype, true);
}

int grok_moe_block_forward(const void* x, const void* pre_scale, const void* post_scale, double eps,
                           const void* router_w, const void* w1, const void* wv, const void* w2, const void* s1,
                           const void* sv, const void* s2, grok_moe_layout weight_layout, int scale_experts,
                           int groups_up, int groups_down, int64_t T, int64_t d, int64_t f, int E, int k,
                           grok_moe_dtype dtype, float* out, const float* router_bias, int32_t* topk_idx,
                           float* topk_p, int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  if (pre_scale == nullptr || post_scale == nullptr) return GROK_MOE_EINVAL;
  return layer_entry(x, pre_scale, post_scale, eps, router_w, w1, wv, w2, s1, sv, s2, weight_layout, scale_experts,
                     groups_up, groups_down, T, d, f, E, k, dtype, out, router_bias, topk_idx, topk_p, expert_counts,
                     workspace, workspace_bytes, stream);
}

int grok_moe_route_norm(const void* x, const void* pre_scale, double eps, const void* router_w,
                        const float* router_bias, int64_t T, int64_t d, int E, int k, grok_moe_dtype dtype, void* xn,
                        int32_t* topk_idx, float* topk_p, hipStream_t stream) {
  int st = check_shape(T, d, dtype == GROK_MOE_F32 ? 64 : 256, E, k, dtype);
  if (st != GROK_MOE_OK) return st;
  if (!(eps >= 0.0)) return GROK_MOE_EINVAL;
  if (T == 0) return GROK_MOE_OK;
  if (!ok_ptr(x) || !ok_ptr(pre_scale) || !ok_ptr(router_w) || !ok_ptr(xn) || !ok_ptr(topk_idx) || !ok_ptr(topk_p) ||
      !ok_opt(router_bias))
    return GROK_MOE_EINVAL;
  return hip_status(gm::launch_router_norm(x, pre_scale, eps, router_w, router_bias, int(T), int(d), E,
                                           dtype != GROK_MOE_F32, xn, topk_idx, topk_p, stream));
}

int grok_moe_combine_norm(const float* y, int splits, const float* topk_p, const int32_t* inv, const void* x,
                          const void* post_scale, double eps, int64_t T, int64_t d, int k, grok_moe_dtype dtype,
                          float* out, hipStream_t stream) {
  if (T < 0 || d <= 0 || splits < 1 || splits > 64 || !(eps >= 0.0)) return GROK_MOE_EINVAL;
  if (dtype != GROK_MOE_F32 && dtype != GROK_MOE_BF16 && dtype != GROK_MOE_W8) return GROK_MOE_EINVAL;
  if (k != 2 || T > kMaxTokens || d % 4 != 0) return GROK_MOE_EUNSUPPORTED;
  if (T == 0) return GROK_MOE_OK;
  if (!ok_ptr(y) || !ok_ptr(topk_p) || !ok_ptr(inv) || !ok_ptr(x) || !ok_ptr(post_scale) || !ok_ptr(out))
    return GROK_MOE_EINVAL;
  return hip_status(gm::launch_combine_norm(y, splits, topk_p, inv, int(T), int(d), x, dtype != GROK_MOE_F32,
                                            post_scale, eps, out, stream));
}

int grok_moe_forward_noalloc(const void* x, const void* router_w, const void* w1, const void* wv, const void* w2,
                             const void* s1, const void* sv, const void* s2, int64_t T, int64_t d, int64_t f, int E,
                             int k, grok_moe_dtype dtype, float* out, const float* router_bias, int32_t* topk_idx,
                             float* topk_p, int32_t* expert_counts, hipStream_t stream) {
  const int st = check_shape(T, d, f, E, k, dtype);
  if (st != GROK_MOE_OK) return st;
  if (T > 0 && workspace_need(T, d, f, E, dtype, false) > GROK_MOE_SCRATCH_BYTES) return GROK_MOE_ESCRATCH;
  void* ws = nullptr;
  if (T > 0 && current_scratch(&ws) != hipSuccess) return GROK_MOE_EHIP;
  return layer_entry(x, nullptr, nullptr, 0.0, router_w, w1, wv, w2, s1, sv, s2, GROK_MOE_IN_OUT, E, 1, 1, T, d, f,
                     E, k, dtype, out, router_bias, topk_idx, topk_p, expert_counts, ws, GROK_MOE_SCRATCH_BYTES,
                     stream);
}

}  // extern "C"
