// C ABI of the MoE block: argument validation, workspace carving and launch
// sequencing.  Declarations and the contract of every entry point are in
// include/beam_moe.h.
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "../../include/beam_moe.h"
#include "../../include/beam_moe_debug.h"
#include "common.h"
#include "kernels.h"

namespace {

using namespace beam;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Weight layouts an entry point accepts (bit i = layout i).
constexpr int kBf16Layouts = (1 << MOE_LAYOUT_ROW_MAJOR) | (1 << MOE_LAYOUT_PACKED);
constexpr int kFp8Layouts = 1 << MOE_LAYOUT_FP8_PACKED;
constexpr int kAnyLayout = kBf16Layouts | kFp8Layouts;

int validate(const moe_config_t* c, int layouts = kBf16Layouts) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->num_tokens < 0 || c->hidden <= 0 || c->intermediate <= 0 || c->num_experts <= 0 ||
      c->num_groups <= 0 || c->topk_groups <= 0 || c->topk <= 0)
    return MOE_ERR_INVALID_ARG;
  if (c->renormalize != 0 && c->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(c->routed_scaling)) return MOE_ERR_INVALID_ARG;
  if (c->num_experts % c->num_groups != 0) return MOE_ERR_INVALID_ARG;
  if (c->weight_layout < 0 || c->weight_layout > 2 || !((layouts >> c->weight_layout) & 1))
    return MOE_ERR_INVALID_ARG;
  if (c->topk_groups > c->num_groups) return MOE_ERR_INVALID_ARG;
  if ((int64_t)c->topk > (int64_t)c->topk_groups * (c->num_experts / c->num_groups))
    return MOE_ERR_INVALID_ARG;
  // shapes the gfx950 kernels are built for
  if (c->num_experts != 256) return MOE_ERR_UNSUPPORTED;
  if (c->num_groups > 64 || (c->num_groups & (c->num_groups - 1)) != 0) return MOE_ERR_UNSUPPORTED;
  if (c->topk > 8) return MOE_ERR_UNSUPPORTED;
  if (c->hidden % 256 != 0 || c->intermediate % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (c->num_tokens * (int64_t)c->topk >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int64_t pairs(const moe_config_t* c) { return c->num_tokens * (int64_t)c->topk; }

int mb_for(const moe_config_t* c) { return ffn_choose_mb(pairs(c), c->num_experts); }
int mb_for_fp8(const moe_config_t* c) { return ffn_fp8_choose_mb(pairs(c), c->num_experts); }

// Upper bound on the m-tiles of either weight format's plan (one workspace
// size serves the bf16 and the fp8 entry points).
int64_t max_tiles_for(const moe_config_t* c) {
  const int64_t n = pairs(c);
  int64_t bmax = ffn_rows_per_tile(mb_for(c));
  const int64_t b8 = ffn_rows_per_tile(mb_for_fp8(c));
  if (b8 < bmax) bmax = b8;
  return n / bmax + (n < c->num_experts ? n : c->num_experts) + 1;
}

size_t route_ws(const moe_config_t* c) {
  return align_up((size_t)router_splits(c->num_tokens, c->hidden) * c->num_tokens *
                  c->num_experts * sizeof(float));
}
size_t permute_ws(const moe_config_t* c) {
  const int64_t nchunks = (pairs(c) + kChunk - 1) / kChunk;
  return align_up((size_t)(nchunks > 0 ? nchunks : 1) * c->num_experts * sizeof(int32_t));
}
size_t plan_bytes(const moe_config_t* c) {
  return align_up((size_t)plan_ints(max_tiles_for(c)) * sizeof(int32_t));
}
size_t ffn_ws(const moe_config_t* c) {
  return plan_bytes(c) + align_up((size_t)pairs(c) * c->intermediate * sizeof(uint16_t));
}
// LoRA intermediates t_gate_up and t_down [pairs, rank] bf16, sized for the
// largest supported rank
constexpr int kMaxLoraRank = 64;
size_t lora_t_bytes(const moe_config_t* c) {
  return align_up((size_t)pairs(c) * kMaxLoraRank * sizeof(uint16_t));
}
size_t ffn_lora_ws(const moe_config_t* c) { return ffn_ws(c) + 2 * lora_t_bytes(c); }

struct LayerLayout {
  size_t ids, w, counts, offsets, psrc, pdst, y, scratch, total;
};

LayerLayout layer_layout(const moe_config_t* c, bool lora = false) {
  LayerLayout L{};
  const size_t n = (size_t)pairs(c);
  size_t o = 0;
  L.ids = o;      o += align_up(n * sizeof(int32_t));
  L.w = o;        o += align_up(n * sizeof(float));
  L.counts = o;   o += align_up((size_t)c->num_experts * sizeof(int32_t));
  L.offsets = o;  o += align_up((size_t)(c->num_experts + 1) * sizeof(int32_t));
  L.psrc = o;     o += align_up(n * sizeof(int32_t));
  L.pdst = o;     o += align_up(n * sizeof(int32_t));
  L.y = o;        o += align_up(n * (size_t)c->hidden * sizeof(uint16_t));
  L.scratch = o;
  size_t s = route_ws(c);
  if (permute_ws(c) > s) s = permute_ws(c);
  const size_t f = lora ? ffn_lora_ws(c) : ffn_ws(c);
  if (f > s) s = f;
  o += s;
  L.total = o;
  return L;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return MOE_OK;
  if (!ws || have < need) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

int device_ready() {
  int dev = -1;
  return hipGetDevice(&dev) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// ---- internal steps (arguments already validated) ----
int do_route(const moe_config_t* c, const uint16_t* x, const float* wr, const float* bias,
             int32_t* ids, float* w, void* scratch, hipStream_t s) {
  const int T = (int)c->num_tokens;
  float* part = static_cast<float*>(scratch);
  const int splits = router_splits(T, c->hidden);
  int st = hip_status(launch_router_logits(x, wr, part, T, c->hidden, splits, s));
  if (st) return st;
  return hip_status(launch_select(part, splits, bias, ids, w, T, c->num_groups, c->topk_groups,
                                  c->topk, c->renormalize, s));
}

int do_permute(const moe_config_t* c, const int32_t* ids, int32_t* counts, int32_t* offsets,
               int32_t* psrc, int32_t* pdst, void* scratch, hipStream_t s) {
  return hip_status(launch_permute(ids, pairs(c), c->num_experts, counts, offsets, psrc, pdst,
                                   static_cast<int32_t*>(scratch), s));
}

int do_plan(const moe_config_t* c, const int32_t* offsets, int32_t* plan, int mb, hipStream_t s) {
  return hip_status(launch_tile_plan(offsets, c->num_experts, ffn_rows_per_tile(mb), plan,
                                     (int)max_tiles_for(c), ffn_blocked_order(mb), s));
}

// the sizes the checked build verifies the GEMMs' indices against: permuted
// rows, rows of A (tokens for gate/up, permuted rows for down), experts
GemmBounds bounds_of(const moe_config_t* c, bool gate_up) {
  GemmBounds b;
  b.n_rows = pairs(c);
  b.n_src = gate_up ? c->num_tokens : pairs(c);
  b.n_experts = c->num_experts;
  return b;
}

int do_gate_up(const moe_config_t* c, const uint16_t* x, const int32_t* psrc,
               const int32_t* plan, const uint16_t* wgu, uint16_t* h, hipStream_t s,
               const LoraArgs& lora = LoraArgs{}) {
  const int64_t max_tiles = max_tiles_for(c);
  const int H = c->hidden, I = c->intermediate;
  return hip_status(launch_grouped_gemm(mb_for(c), true, x, psrc, c->topk, wgu,
                                        (int64_t)2 * I * H, h, plan, (int)max_tiles, H, I, I,
                                        c->weight_layout, lora,
                                        max_tiles * (I / ffn_out_cols_per_item(true)), s,
                                        ffn_stream_weights(pairs(c), c->num_experts),
                                        bounds_of(c, true)));
}

int do_down(const moe_config_t* c, const uint16_t* h, const int32_t* plan, const uint16_t* wd,
            uint16_t* y, hipStream_t s, const LoraArgs& lora = LoraArgs{}) {
  const int64_t max_tiles = max_tiles_for(c);
  const int H = c->hidden, I = c->intermediate;
  return hip_status(launch_grouped_gemm(mb_for(c), false, h, nullptr, c->topk, wd,
                                        (int64_t)H * I, y, plan, (int)max_tiles, I, H, 0,
                                        c->weight_layout, lora,
                                        max_tiles * (H / ffn_out_cols_per_item(false)), s,
                                        ffn_stream_weights(pairs(c), c->num_experts),
                                        bounds_of(c, false)));
}

int do_ffn(const moe_config_t* c, const uint16_t* x, const int32_t* psrc, const int32_t* offsets,
           const uint16_t* wgu, const uint16_t* wd, uint16_t* y, void* scratch, hipStream_t s) {
  int32_t* plan = static_cast<int32_t*>(scratch);
  uint16_t* h = reinterpret_cast<uint16_t*>(static_cast<char*>(scratch) + plan_bytes(c));
  int st = do_plan(c, offsets, plan, mb_for(c), s);
  if (st) return st;
  if ((st = do_gate_up(c, x, psrc, plan, wgu, h, s))) return st;
  return do_down(c, h, plan, wd, y, s);
}

// ---- expert LoRA on the bf16 expert weights ----
bool lora_ok(const moe_lora_t* l) {
  if (!l) return false;
  if (l->rank != 16 && l->rank != 32 && l->rank != 48 && l->rank != 64) return false;
  if (!std::isfinite(l->scale)) return false;
  return l->a_gate_up && l->b_gate_up && l->a_down && l->b_down && aligned16(l->a_gate_up) &&
         aligned16(l->b_gate_up) && aligned16(l->a_down) && aligned16(l->b_down);
}

// plan, t_gate_up = s x A_gu^T, gate/up (+ t_gate_up B_gu^T), t_down = s h A_d^T,
// down (+ t_down B_d^T)
int do_ffn_lora(const moe_config_t* c, const uint16_t* x, const int32_t* psrc,
                const int32_t* offsets, const uint16_t* wgu, const uint16_t* wd,
                const moe_lora_t* l, uint16_t* y, void* scratch, hipStream_t s) {
  char* base = static_cast<char*>(scratch);
  int32_t* plan = reinterpret_cast<int32_t*>(base);
  uint16_t* h = reinterpret_cast<uint16_t*>(base + plan_bytes(c));
  uint16_t* t_gu = reinterpret_cast<uint16_t*>(base + ffn_ws(c));
  uint16_t* t_d = reinterpret_cast<uint16_t*>(base + ffn_ws(c) + lora_t_bytes(c));
  const int H = c->hidden, I = c->intermediate, R = l->rank;
  const int max_tiles = (int)max_tiles_for(c);
  int st = do_plan(c, offsets, plan, mb_for(c), s);
  if (st) return st;
  if ((st = hip_status(launch_lora_a(x, psrc, c->topk, l->a_gate_up, H, R, l->scale, t_gu, plan,
                                     max_tiles, s))))
    return st;
  LoraArgs lg;
  lg.t = t_gu; lg.b = l->b_gate_up; lg.b_stride = (int64_t)2 * I * R; lg.rank = R;
  if ((st = do_gate_up(c, x, psrc, plan, wgu, h, s, lg))) return st;
  if ((st = hip_status(launch_lora_a(h, nullptr, c->topk, l->a_down, I, R, l->scale, t_d, plan,
                                     max_tiles, s))))
    return st;
  LoraArgs ld;
  ld.t = t_d; ld.b = l->b_down; ld.b_stride = (int64_t)H * R; ld.rank = R;
  return do_down(c, h, plan, wd, y, s, ld);
}

// ---- fp8 expert weights ----
struct Fp8Weights {
  const uint8_t* q_gate_up;
  const float* s_gate_up;
  const uint8_t* q_down;
  const float* s_down;
};

int do_gate_up_fp8(const moe_config_t* c, const uint16_t* x, const int32_t* psrc,
                   const int32_t* plan, const uint8_t* q, const float* sc, uint16_t* h,
                   hipStream_t s) {
  const int64_t max_tiles = max_tiles_for(c);
  const int H = c->hidden, I = c->intermediate;
  return hip_status(launch_grouped_gemm_fp8(mb_for_fp8(c), true, x, psrc, c->topk, q, sc,
                                            (int64_t)2 * I * H, 2 * I, h, plan, (int)max_tiles, H,
                                            I, I, max_tiles * (I / ffn_out_cols_per_item(true)),
                                            s, bounds_of(c, true)));
}

int do_down_fp8(const moe_config_t* c, const uint16_t* h, const int32_t* plan, const uint8_t* q,
                const float* sc, uint16_t* y, hipStream_t s) {
  const int64_t max_tiles = max_tiles_for(c);
  const int H = c->hidden, I = c->intermediate;
  return hip_status(launch_grouped_gemm_fp8(mb_for_fp8(c), false, h, nullptr, c->topk, q, sc,
                                            (int64_t)H * I, H, y, plan, (int)max_tiles, I, H, 0,
                                            max_tiles * (H / ffn_out_cols_per_item(false)), s,
                                            bounds_of(c, false)));
}

int do_ffn_fp8(const moe_config_t* c, const uint16_t* x, const int32_t* psrc,
               const int32_t* offsets, const Fp8Weights& w, uint16_t* y, void* scratch,
               hipStream_t s) {
  int32_t* plan = static_cast<int32_t*>(scratch);
  uint16_t* h = reinterpret_cast<uint16_t*>(static_cast<char*>(scratch) + plan_bytes(c));
  int st = do_plan(c, offsets, plan, mb_for_fp8(c), s);
  if (st) return st;
  if ((st = do_gate_up_fp8(c, x, psrc, plan, w.q_gate_up, w.s_gate_up, h, s))) return st;
  return do_down_fp8(c, h, plan, w.q_down, w.s_down, y, s);
}

bool fp8_weights_ok(const uint8_t* q, const float* sc) {
  return q && sc && aligned16(q) && aligned4(sc);
}

// The whole block around an expert-MLP step `ffn(x, psrc, offsets, y, scratch)`.
template <class Ffn>
int layer_common(const moe_config_t* cfg, const uint16_t* x, const float* w_router,
                 const float* sel_bias, uint16_t* out, int32_t* topk_ids_out, float* topk_w_out,
                 void* workspace, size_t workspace_bytes, hipStream_t s, Ffn ffn,
                 bool lora = false) {
  const LayerLayout L = layer_layout(cfg, lora);
  int st = check_ws(workspace, workspace_bytes, L.total);
  if (st) return st;
  if (cfg->num_tokens == 0) return MOE_OK;
  if ((st = device_ready())) return st;
  char* ws = static_cast<char*>(workspace);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(ws + L.w);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* psrc = reinterpret_cast<int32_t*>(ws + L.psrc);
  int32_t* pdst = reinterpret_cast<int32_t*>(ws + L.pdst);
  uint16_t* y = reinterpret_cast<uint16_t*>(ws + L.y);
  void* scratch = ws + L.scratch;
  if ((st = do_route(cfg, x, w_router, sel_bias, ids, w, scratch, s))) return st;
  if ((st = do_permute(cfg, ids, counts, offsets, psrc, pdst, scratch, s))) return st;
  if ((st = ffn(psrc, offsets, y, scratch))) return st;
  return hip_status(launch_combine(y, pdst, w, out, (int)cfg->num_tokens, cfg->hidden, cfg->topk,
                                   cfg->routed_scaling, s));
}

bool layer_args_ok(const moe_config_t* cfg, const uint16_t* x, const float* w_router,
                   const float* sel_bias, uint16_t* out, int32_t* topk_ids_out,
                   float* topk_w_out) {
  (void)cfg;
  if (!x || !w_router || !out) return false;
  return aligned16(x) && aligned16(w_router) && aligned16(out) &&
         (!sel_bias || aligned4(sel_bias)) && (!topk_ids_out || aligned4(topk_ids_out)) &&
         (!topk_w_out || aligned4(topk_w_out));
}

// ---- scratch for moe_layer_forward_noalloc ----
// The one scratch buffer of the library that no caller provides: a static
// device array, one copy per GPU the library runs on, held until the process
// ends.  Host code never uses the array's name as an address (on the host it
// is only a stand-in for the symbol); it reads the device address once per
// device with hipGetSymbolAddress and passes that on.
constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device (with it current) and kept.
int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK: success";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape not supported by the gfx950 kernels";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime error";
    case MOE_ERR_TOO_LARGE:
      return "MOE_ERR_TOO_LARGE: the call needs more scratch than the library's static 128 MiB";
    default: return "unknown moe status";
  }
}

int moe_workspace_bytes(const moe_config_t* cfg, int entry, size_t* bytes) {
  int st = validate(cfg, kAnyLayout);
  if (st) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  switch (entry) {
    case MOE_ENTRY_ROUTE: *bytes = route_ws(cfg); break;
    case MOE_ENTRY_PERMUTE: *bytes = permute_ws(cfg); break;
    case MOE_ENTRY_EXPERT_FFN: *bytes = ffn_ws(cfg); break;
    case MOE_ENTRY_LAYER: *bytes = layer_layout(cfg).total; break;
    case MOE_ENTRY_EXPERT_STAGE: *bytes = plan_bytes(cfg); break;
    case MOE_ENTRY_EXPERT_FFN_LORA: *bytes = ffn_lora_ws(cfg); break;
    case MOE_ENTRY_LAYER_LORA: *bytes = layer_layout(cfg, true).total; break;
    default: return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

int moe_route(const moe_config_t* cfg, const uint16_t* x, const float* w_router,
              const float* sel_bias, int32_t* topk_ids, float* topk_w, void* workspace,
              size_t workspace_bytes, void* stream) {
  int st = validate(cfg, kAnyLayout);
  if (st) return st;
  if (!x || !w_router || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned4(topk_ids) || !aligned4(topk_w) ||
      (sel_bias && !aligned4(sel_bias)))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(workspace, workspace_bytes, route_ws(cfg)))) return st;
  if (cfg->num_tokens == 0) return MOE_OK;
  if ((st = device_ready())) return st;
  return do_route(cfg, x, w_router, sel_bias, topk_ids, topk_w, workspace,
                  static_cast<hipStream_t>(stream));
}

int moe_route_replay(const moe_config_t* cfg, const uint16_t* x, const float* w_router,
                     const int32_t* topk_ids, float* topk_w, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = validate(cfg, kAnyLayout);
  if (st) return st;
  if (!x || !w_router || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned4(topk_ids) || !aligned4(topk_w))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(workspace, workspace_bytes, route_ws(cfg)))) return st;
  if (cfg->num_tokens == 0) return MOE_OK;
  if ((st = device_ready())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(workspace);
  const int T = (int)cfg->num_tokens;
  const int splits = router_splits(T, cfg->hidden);
  st = hip_status(launch_router_logits(x, w_router, part, T, cfg->hidden, splits, s));
  if (st) return st;
  return hip_status(launch_replay(part, splits, topk_ids, topk_w, T, cfg->num_experts, cfg->topk,
                                  cfg->renormalize, s));
}

int moe_permute(const moe_config_t* cfg, const int32_t* topk_ids, int32_t* counts,
                int32_t* offsets, int32_t* perm_src, int32_t* perm_dst, void* workspace,
                size_t workspace_bytes, void* stream) {
  int st = validate(cfg, kAnyLayout);
  if (st) return st;
  if (!topk_ids || !counts || !offsets || !perm_src || !perm_dst) return MOE_ERR_INVALID_ARG;
  if (!aligned4(topk_ids) || !aligned4(counts) || !aligned4(offsets) || !aligned4(perm_src) ||
      !aligned4(perm_dst))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(workspace, workspace_bytes, permute_ws(cfg)))) return st;
  if (cfg->num_tokens == 0) return MOE_OK;
  if ((st = device_ready())) return st;
  return do_permute(cfg, topk_ids, counts, offsets, perm_src, perm_dst, workspace,
                    static_cast<hipStream_t>(stream));
}

int moe_expert_ffn(const moe_config_t* cfg, const uint16_t* x, const int32_t* perm_src,
                   const int32_t* offsets, const uint16_t* w_gate_up, const uint16_t* w_down,
                   uint16_t* y_perm, void* workspace, size_t workspace_bytes, void* stream) {
  int st = validate(cfg);
  if (st) return st;
  if (!x || !perm_src || !offsets || !w_gate_up || !w_down || !y_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(y_perm) ||
      !aligned4(perm_src) || !aligned4(offsets))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(workspace, workspace_bytes, ffn_ws(cfg)))) return st;
  if (cfg->num_tokens == 0) return MOE_OK;
  if ((st = device_ready())) return st;
  return do_ffn(cfg, x, perm_src, offsets, w_gate_up, w_down, y_perm, workspace,
                static_cast<hipStream_t>(stream));
}

int moe_expert_gate_up(const moe_config_t* cfg, const uint16_t* x, const int32_t* perm_src,
                       const int32_t* offsets, const uint16_t* w_gate_up, uint16_t* h,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int st = validate(cfg);
  if (st) return st;
  if (!x || !perm_src || !offsets || !w_gate_up || !h) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(h) || !aligned4(perm_src) ||
      !aligned4(offsets))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(workspace, workspace_bytes, plan_bytes(cfg)))) return st;
  if (cfg->num_tokens == 0) return MOE_OK;
  if ((st = device_ready())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* plan = static_cast<int32_t*>(workspace);
  if ((st = do_plan(cfg, offsets, plan, mb_for(cfg), s))) return st;
  return do_gate_up(cfg, x, perm_src, plan, w_gate_up, h, s);
}

int moe_expert_down(const moe_config_t* cfg, const uint16_t* h, const int32_t* offsets,
                    const uint16_t* w_down, uint16_t* y_perm, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int st = validate(cfg);
  if (st) return st;
  if (!h || !offsets || !w_down || !y_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w_down) || !aligned16(y_perm) || !aligned4(offsets))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(workspace, workspace_bytes, plan_bytes(cfg)))) return st;
  if (cfg->num_tokens == 0) return MOE_OK;
  if ((st = device_ready())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* plan = static_cast<int32_t*>(workspace);
  if ((st = do_plan(cfg, offsets, plan, mb_for(cfg), s))) return st;
  return do_down(cfg, h, plan, w_down, y_perm, s);
}

int moe_pack_weights(const moe_config_t* cfg, const uint16_t* w_gate_up, const uint16_t* w_down,
                     uint16_t* packed_gate_up, uint16_t* packed_down, void* stream) {
  moe_config_t c = cfg ? *cfg : moe_config_t{};
  c.num_tokens = 0;
  c.weight_layout = MOE_LAYOUT_ROW_MAJOR;  // not read here
  int st = validate(cfg ? &c : nullptr);
  if (st) return st;
  if ((w_gate_up == nullptr) != (packed_gate_up == nullptr) ||
      (w_down == nullptr) != (packed_down == nullptr))
    return MOE_ERR_INVALID_ARG;
  if ((w_gate_up && (!aligned16(w_gate_up) || !aligned16(packed_gate_up))) ||
      (w_down && (!aligned16(w_down) || !aligned16(packed_down))))
    return MOE_ERR_INVALID_ARG;
  const int64_t E = c.num_experts, H = c.hidden, I = c.intermediate;
  auto overlap = [](const void* a, const void* b, int64_t n) {
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(b);
    return x < y + n && y < x + n;
  };
  if (w_gate_up && overlap(w_gate_up, packed_gate_up, E * 2 * I * H * 2)) return MOE_ERR_INVALID_ARG;
  if (w_down && overlap(w_down, packed_down, E * H * I * 2)) return MOE_ERR_INVALID_ARG;
  if (!w_gate_up && !w_down) return MOE_OK;
  if ((st = device_ready())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w_gate_up &&
      (st = hip_status(launch_pack_weights(w_gate_up, packed_gate_up, (int)E, (int)(2 * I), (int)H, s))))
    return st;
  if (w_down && (st = hip_status(launch_pack_weights(w_down, packed_down, (int)E, (int)H, (int)I, s))))
    return st;
  return MOE_OK;
}

int moe_combine(const moe_config_t* cfg, const uint16_t* y_perm, const int32_t* perm_dst,
                const float* topk_w, uint16_t* out, void* stream) {
  int st = validate(cfg, kAnyLayout);
  if (st) return st;
  if (!y_perm || !perm_dst || !topk_w || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y_perm) || !aligned16(out) || !aligned4(perm_dst) || !aligned4(topk_w))
    return MOE_ERR_INVALID_ARG;
  if (cfg->num_tokens == 0) return MOE_OK;
  if ((st = device_ready())) return st;
  return hip_status(launch_combine(y_perm, perm_dst, topk_w, out, (int)cfg->num_tokens,
                                   cfg->hidden, cfg->topk, cfg->routed_scaling,
                                   static_cast<hipStream_t>(stream)));
}

int moe_layer_forward(const moe_config_t* cfg, const uint16_t* x, const float* w_router,
                      const float* sel_bias, const uint16_t* w_gate_up, const uint16_t* w_down,
                      uint16_t* out, int32_t* topk_ids_out, float* topk_w_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st = validate(cfg);
  if (st) return st;
  if (!layer_args_ok(cfg, x, w_router, sel_bias, out, topk_ids_out, topk_w_out) || !w_gate_up ||
      !w_down || !aligned16(w_gate_up) || !aligned16(w_down))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return layer_common(cfg, x, w_router, sel_bias, out, topk_ids_out, topk_w_out, workspace,
                      workspace_bytes, s,
                      [&](const int32_t* psrc, const int32_t* offsets, uint16_t* y, void* scratch) {
                        return do_ffn(cfg, x, psrc, offsets, w_gate_up, w_down, y, scratch, s);
                      });
}

int moe_debug_check_flags(uint32_t* flags) {
  if (!flags) return MOE_ERR_INVALID_ARG;
  *flags = 0;
#if BEAM_MOE_CHECKED
  if (device_ready()) return MOE_ERR_HIP;
  if (hipDeviceSynchronize() != hipSuccess) return MOE_ERR_HIP;
  *flags = check_flags_permute() | check_flags_ffn() | check_flags_combine();
  return MOE_OK;
#else
  return MOE_ERR_UNSUPPORTED;
#endif
}

int moe_layer_forward_noalloc(const moe_config_t* cfg, const uint16_t* x, const float* w_router,
                              const float* sel_bias, const uint16_t* w_gate_up,
                              const uint16_t* w_down, uint16_t* out, int32_t* topk_ids_out,
                              float* topk_w_out, void* stream) {
  int st = validate(cfg);
  if (st) return st;
  if (!layer_args_ok(cfg, x, w_router, sel_bias, out, topk_ids_out, topk_w_out) || !w_gate_up ||
      !w_down || !aligned16(w_gate_up) || !aligned16(w_down))
    return MOE_ERR_INVALID_ARG;
  if (layer_layout(cfg).total > kNoAllocScratchBytes) return MOE_ERR_TOO_LARGE;
  if (cfg->num_tokens == 0) return MOE_OK;
  void* ws = nullptr;
  if ((st = noalloc_scratch(&ws))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return layer_common(cfg, x, w_router, sel_bias, out, topk_ids_out, topk_w_out, ws,
                      kNoAllocScratchBytes, s,
                      [&](const int32_t* psrc, const int32_t* offsets, uint16_t* y, void* sc) {
                        return do_ffn(cfg, x, psrc, offsets, w_gate_up, w_down, y, sc, s);
                      });
}

int moe_quantize_fp8(const moe_config_t* cfg, const uint16_t* w_gate_up, const uint16_t* w_down,
                     uint8_t* q_gate_up, float* s_gate_up, uint8_t* q_down, float* s_down,
                     void* stream) {
  moe_config_t c = cfg ? *cfg : moe_config_t{};
  c.num_tokens = 0;
  c.weight_layout = MOE_LAYOUT_ROW_MAJOR;  // not read here
  int st = validate(cfg ? &c : nullptr);
  if (st) return st;
  const bool gu = w_gate_up || q_gate_up || s_gate_up;
  const bool dn = w_down || q_down || s_down;
  if (gu && (!w_gate_up || !q_gate_up || !s_gate_up)) return MOE_ERR_INVALID_ARG;
  if (dn && (!w_down || !q_down || !s_down)) return MOE_ERR_INVALID_ARG;
  if ((gu && (!aligned16(w_gate_up) || !aligned16(q_gate_up) || !aligned4(s_gate_up))) ||
      (dn && (!aligned16(w_down) || !aligned16(q_down) || !aligned4(s_down))))
    return MOE_ERR_INVALID_ARG;
  const int64_t E = c.num_experts, H = c.hidden, I = c.intermediate;
  auto overlap = [](const void* a, int64_t na, const void* b, int64_t nb) {
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(b);
    return x < y + nb && y < x + na;
  };
  const int64_t ngu = E * 2 * I * H, ndn = E * H * I;
  if (gu && (overlap(w_gate_up, 2 * ngu, q_gate_up, ngu) ||
             overlap(w_gate_up, 2 * ngu, s_gate_up, 4 * E * 2 * I) ||
             overlap(q_gate_up, ngu, s_gate_up, 4 * E * 2 * I)))
    return MOE_ERR_INVALID_ARG;
  if (dn && (overlap(w_down, 2 * ndn, q_down, ndn) || overlap(w_down, 2 * ndn, s_down, 4 * E * H) ||
             overlap(q_down, ndn, s_down, 4 * E * H)))
    return MOE_ERR_INVALID_ARG;
  if (!gu && !dn) return MOE_OK;
  if ((st = device_ready())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (gu && (st = hip_status(launch_quantize_fp8(w_gate_up, q_gate_up, s_gate_up, (int)E,
                                                 (int)(2 * I), (int)H, s))))
    return st;
  if (dn && (st = hip_status(launch_quantize_fp8(w_down, q_down, s_down, (int)E, (int)H, (int)I, s))))
    return st;
  return MOE_OK;
}

int moe_expert_ffn_fp8(const moe_config_t* cfg, const uint16_t* x, const int32_t* perm_src,
                       const int32_t* offsets, const uint8_t* q_gate_up, const float* s_gate_up,
                       const uint8_t* q_down, const float* s_down, uint16_t* y_perm,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int st = validate(cfg, kFp8Layouts);
  if (st) return st;
  if (!x || !perm_src || !offsets || !y_perm || !fp8_weights_ok(q_gate_up, s_gate_up) ||
      !fp8_weights_ok(q_down, s_down))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y_perm) || !aligned4(perm_src) || !aligned4(offsets))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(workspace, workspace_bytes, ffn_ws(cfg)))) return st;
  if (cfg->num_tokens == 0) return MOE_OK;
  if ((st = device_ready())) return st;
  return do_ffn_fp8(cfg, x, perm_src, offsets, Fp8Weights{q_gate_up, s_gate_up, q_down, s_down},
                    y_perm, workspace, static_cast<hipStream_t>(stream));
}

int moe_expert_gate_up_fp8(const moe_config_t* cfg, const uint16_t* x, const int32_t* perm_src,
                           const int32_t* offsets, const uint8_t* q_gate_up,
                           const float* s_gate_up, uint16_t* h, void* workspace,
                           size_t workspace_bytes, void* stream) {
  int st = validate(cfg, kFp8Layouts);
  if (st) return st;
  if (!x || !perm_src || !offsets || !h || !fp8_weights_ok(q_gate_up, s_gate_up))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(h) || !aligned4(perm_src) || !aligned4(offsets))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(workspace, workspace_bytes, plan_bytes(cfg)))) return st;
  if (cfg->num_tokens == 0) return MOE_OK;
  if ((st = device_ready())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* plan = static_cast<int32_t*>(workspace);
  if ((st = do_plan(cfg, offsets, plan, mb_for_fp8(cfg), s))) return st;
  return do_gate_up_fp8(cfg, x, perm_src, plan, q_gate_up, s_gate_up, h, s);
}

int moe_expert_down_fp8(const moe_config_t* cfg, const uint16_t* h, const int32_t* offsets,
                        const uint8_t* q_down, const float* s_down, uint16_t* y_perm,
                        void* workspace, size_t workspace_bytes, void* stream) {
  int st = validate(cfg, kFp8Layouts);
  if (st) return st;
  if (!h || !offsets || !y_perm || !fp8_weights_ok(q_down, s_down)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(y_perm) || !aligned4(offsets)) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(workspace, workspace_bytes, plan_bytes(cfg)))) return st;
  if (cfg->num_tokens == 0) return MOE_OK;
  if ((st = device_ready())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* plan = static_cast<int32_t*>(workspace);
  if ((st = do_plan(cfg, offsets, plan, mb_for_fp8(cfg), s))) return st;
  return do_down_fp8(cfg, h, plan, q_down, s_down, y_perm, s);
}

int moe_layer_forward_fp8(const moe_config_t* cfg, const uint16_t* x, const float* w_router,
                          const float* sel_bias, const uint8_t* q_gate_up, const float* s_gate_up,
                          const uint8_t* q_down, const float* s_down, uint16_t* out,
                          int32_t* topk_ids_out, float* topk_w_out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int st = validate(cfg, kFp8Layouts);
  if (st) return st;
  if (!layer_args_ok(cfg, x, w_router, sel_bias, out, topk_ids_out, topk_w_out) ||
      !fp8_weights_ok(q_gate_up, s_gate_up) || !fp8_weights_ok(q_down, s_down))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Fp8Weights w{q_gate_up, s_gate_up, q_down, s_down};
  return layer_common(cfg, x, w_router, sel_bias, out, topk_ids_out, topk_w_out, workspace,
                      workspace_bytes, s,
                      [&](const int32_t* psrc, const int32_t* offsets, uint16_t* y, void* scratch) {
                        return do_ffn_fp8(cfg, x, psrc, offsets, w, y, scratch, s);
                      });
}

int moe_expert_ffn_lora(const moe_config_t* cfg, const uint16_t* x, const int32_t* perm_src,
                        const int32_t* offsets, const uint16_t* w_gate_up, const uint16_t* w_down,
                        const moe_lora_t* lora, uint16_t* y_perm, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int st = validate(cfg);
  if (st) return st;
  if (!x || !perm_src || !offsets || !w_gate_up || !w_down || !y_perm || !lora_ok(lora))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(y_perm) ||
      !aligned4(perm_src) || !aligned4(offsets))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(workspace, workspace_bytes, ffn_lora_ws(cfg)))) return st;
  if (cfg->num_tokens == 0) return MOE_OK;
  if ((st = device_ready())) return st;
  return do_ffn_lora(cfg, x, perm_src, offsets, w_gate_up, w_down, lora, y_perm, workspace,
                     static_cast<hipStream_t>(stream));
}

int moe_layer_forward_lora(const moe_config_t* cfg, const uint16_t* x, const float* w_router,
                           const float* sel_bias, const uint16_t* w_gate_up,
                           const uint16_t* w_down, const moe_lora_t* lora, uint16_t* out,
                           int32_t* topk_ids_out, float* topk_w_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  int st = validate(cfg);
  if (st) return st;
  if (!layer_args_ok(cfg, x, w_router, sel_bias, out, topk_ids_out, topk_w_out) || !w_gate_up ||
      !w_down || !aligned16(w_gate_up) || !aligned16(w_down) || !lora_ok(lora))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return layer_common(
      cfg, x, w_router, sel_bias, out, topk_ids_out, topk_w_out, workspace, workspace_bytes, s,
      [&](const int32_t* psrc, const int32_t* offsets, uint16_t* y, void* scratch) {
        return do_ffn_lora(cfg, x, psrc, offsets, w_gate_up, w_down, lora, y, scratch, s);
      },
      true);
}

}  // extern "C"
