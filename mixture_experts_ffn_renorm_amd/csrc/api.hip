// C ABI of the MoE layer forward: argument checks, workspace carve-up,
// kernel choice and launches.  Declarations and the contract of every call
// are in include/moe_mi355x.h.
#include <algorithm>

#include "moe_common.h"
#include "moe_mi355x.h"

using namespace moe_host;

namespace {

constexpr size_t kAlign = 256;
constexpr long long kMaxPairs = 1LL << 24;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

long long max_blocks(long long P, int E, int B) {
  return (P + B - 1) / B + std::min<long long>(E, P);
}
long long sorted_capacity(long long P, int E, int B) {
  return P + std::min<long long>(E, P) * (B - 1);
}

// Workspace regions of moe_forward for one (M, E, top_k, H, I, block_m).
// Only the arrival counter of the fused top-k + align launch needs clearing
// (done by the router-logits kernel).  partial holds GEMM 2's pair-order
// rows: fp32 weighted (streaming) or bf16 (tiled).
struct Layout {
  size_t arrive, ids, wts, logits, sorted, eids, boff, counts, align_scratch, act, partial;
  size_t total;
};

Layout forward_layout(int M, int E, int top_k, int H, int I, int B) {
  const long long P = (long long)M * top_k;
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.arrive = take(4);
  L.partial = take((size_t)P * H * 4);
  L.ids = take((size_t)P * 4);
  L.wts = take((size_t)P * 4);
  L.logits = take((size_t)M * E * 4);
  L.sorted = take((size_t)sorted_capacity(P, E, B) * 4);
  L.eids = take((size_t)max_blocks(P, E, B) * 4);
  L.boff = take((size_t)(E + 1) * 4);
  L.counts = take((size_t)E * 4);
  L.align_scratch = take(align_scratch_bytes((int)P, E));
  L.act = take((size_t)P * I * 2);
  L.total = off;
  return L;
}

int check_sizes(int M, int E, int top_k, int H, int I) {
  if (M < 0 || E <= 0 || top_k <= 0 || H <= 0 || I <= 0) return MOE_ERR_INVALID_ARG;
  if (top_k > E) return MOE_ERR_INVALID_ARG;
  if (E > 512 || top_k > 32) return MOE_ERR_UNSUPPORTED;
  if (H % 8 != 0 || I % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if ((long long)M * top_k >= kMaxPairs) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Block sizes the GEMM calls accept (1: per-pair GEMVs; 16: weight-streaming
// kernels; the others: tiled kernels).
constexpr int kBlockSizes[] = {1, 16, 64, 128, 256};
bool gemm_block_ok(int B) {
  for (int b : kBlockSizes)
    if (B == b) return true;
  return false;
}

// The kernels copy 16-byte pieces of every tensor.
bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Small batches run the top-k and the index lists in one launch.
bool fused_route(int M, int top_k) { return align_segments(M * top_k) == 1; }

// Very small batches skip the sort (page "Mixture of Experts in vLLM ...",
// sub-section "Small batches skip the sort"): when M*top_k*4 <= E every pair
// is its own product, run as per-pair GEMVs (block_m 1); moe_forward then
// builds no index lists and the GEMVs read topk_ids directly.
bool per_pair_gemv(int M, int top_k, int E) {
  return M >= 1 && (long long)M * top_k * 4 <= E;
}

// Kernels queued by one GEMM 2 call: the GEMM and the per-token weighted sum.
constexpr int kGemm2Launches = 2;

// Kernels queued by moe_forward's per-pair path: router logits, top-k,
// GEMV 1, GEMV 2 with the weighted sum.
constexpr int kPairGemvForwardLaunches = 4;

void fill_info(moe_dispatch_info* info, int B, int H, int I, int launches, int sorted = 1) {
  if (info == nullptr) return;
  info->sorted = sorted;
  info->block_m = B;
  if (B == 1) {
    info->variant = MOE_VARIANT_PAIR_GEMV;
    info->block_n = kPairGemvFeatures;
    info->block_k = kPairGemvK;
  } else {
    const bool stream = B == 16;
    info->variant = stream ? MOE_VARIANT_STREAM : MOE_VARIANT_TILED;
    info->block_n = stream ? kStreamG1Features : kTiledG1Features;
    info->block_k = stream ? kStreamBK : kTiledBK;
  }
  info->k_tail = (H % info->block_k != 0 || I % info->block_k != 0) ? 1 : 0;
  info->launches = launches;
}

#define MOE_TRY_HIP(expr)                            \
  do {                                               \
    if ((expr) != hipSuccess) return MOE_ERR_HIP;    \
  } while (0)

GemmArgs gemm_args(int M, int top_k, int E, int H, int I, int B) {
  GemmArgs g{};
  g.M = M;
  g.top_k = top_k;
  g.E = E;
  g.H = H;
  g.I = I;
  g.block_m = B;
  g.max_blocks = (int)max_blocks((long long)M * top_k, E, B);
  return g;
}

// block_m 1: the per-pair GEMVs in index-list order (one pair per block).
PairGemvArgs pair_args(const GemmArgs& g) {
  PairGemvArgs a{};
  a.M = g.M;
  a.top_k = g.top_k;
  a.H = g.H;
  a.I = g.I;
  a.sorted = g.sorted_token_ids;
  a.expert_ids = g.expert_ids;
  a.topk_weights = g.topk_weights;
  return a;
}

int run_gemm1(GemmArgs g, hipStream_t s) {
  if (g.block_m == 1) {
    PairGemvArgs a = pair_args(g);
    a.x = g.a_src;
    a.w13 = g.w;
    a.act = g.out;
    MOE_TRY_HIP(launch_pair_gemv1(a, s));
    return MOE_OK;
  }
  MOE_TRY_HIP(g.block_m == 16 ? launch_gemm1_stream(g, s) : launch_gemm1_tiled(g, s));
  return MOE_OK;
}

int run_gemm2(GemmArgs g, hipStream_t s) {
  if (g.block_m == 1) {
    PairGemvArgs a = pair_args(g);
    a.act = const_cast<uint16_t*>(g.a_src);
    a.w2 = g.w;
    a.out = g.out;
    a.partial = g.partial;
    MOE_TRY_HIP(launch_pair_gemv2(a, s));
    return MOE_OK;
  }
  MOE_TRY_HIP(g.block_m == 16 ? launch_gemm2_stream(g, s) : launch_gemm2_tiled(g, s));
  return MOE_OK;
}

}  // namespace

namespace moe_host {

int device_cu_count() {
  static int cached[64] = {0};   // benign race: every writer stores the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace moe_host

extern "C" {

size_t moe_workspace_size(int M_max, int E, int top_k, int H, int I) {
  if (check_sizes(M_max, E, top_k, H, I) != MOE_OK) return 0;
  size_t best = 0;
  for (int B : kBlockSizes) best = std::max(best, forward_layout(M_max, E, top_k, H, I, B).total);
  return std::max<size_t>(best, kAlign);
}

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported size or option";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int moe_pick_block_m(int M, int E, int top_k) {
  if (E <= 0) return 16;
  if (per_pair_gemv(M, top_k, E)) return 1;
  const double per_expert = (double)M * top_k / E;
  if (per_expert <= 8.0) return 16;
  if (per_expert <= 48.0) return 64;
  // Measured on the copy-wave tiles: 128-pair blocks up to 128 pairs per
  // expert; 256 where a 128-pair expert would end in a second, nearly empty
  // block that streams its weights again (Qwen1.5 shape, 136 per expert);
  // 128 again from 192 on, where 256-pair blocks leave more pad quarters.
  if (per_expert < 128.0) return 128;
  if (per_expert < 192.0) return 256;
  return 128;
}

int moe_forward_list_offsets(int M, int E, int top_k, int H, int I, moe_forward_lists* out) {
  const int st = check_sizes(M, E, top_k, H, I);
  if (st != MOE_OK) return st;
  if (out == nullptr) return MOE_ERR_INVALID_ARG;
  const int B = moe_pick_block_m(M, E, top_k);
  const Layout L = forward_layout(M, E, top_k, H, I, B);
  out->block_m = B;
  out->sorted = (M > 0 && !per_pair_gemv(M, top_k, E)) ? 1 : 0;
  out->sorted_token_ids = L.sorted;
  out->expert_ids = L.eids;
  out->expert_block_offsets = L.boff;
  out->expert_counts = L.counts;
  return MOE_OK;
}

int moe_route(const uint16_t* x, const uint16_t* w_router, const float* logit_bias, int M,
              int H, int E, int top_k, int renormalize, int32_t* topk_ids,
              float* topk_weights, float* logits_out, void* workspace, size_t ws_bytes,
              void* stream) {
  int st = check_sizes(M, E, top_k, H, 8);
  if (st != MOE_OK) return st;
  if (renormalize != 0 && renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (M == 0) return MOE_OK;
  if (!x || !w_router || !topk_ids || !topk_weights) return MOE_ERR_INVALID_ARG;
  float* logits = logits_out;
  if (logits == nullptr) {
    if (workspace == nullptr || ws_bytes < (size_t)M * E * 4) return MOE_ERR_WORKSPACE;
    logits = static_cast<float*>(workspace);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  RouteArgs a{x, w_router, logit_bias, M, H, E, top_k, renormalize, logits, topk_ids,
              topk_weights, nullptr, 0};
  MOE_TRY_HIP(launch_route_logits(a, s));
  MOE_TRY_HIP(launch_route_topk(a, s));
  return MOE_OK;
}

size_t moe_align_workspace_size(int M, int top_k, int E) {
  if (check_sizes(M, E, top_k, 8, 8) != MOE_OK) return 0;
  return align_scratch_bytes(M * top_k, E);
}

int moe_align(const int32_t* topk_ids, int M, int top_k, int E, int block_m,
              int32_t* sorted_token_ids, int32_t* expert_ids, int32_t* expert_block_offsets,
              int32_t* expert_counts, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_sizes(M, E, top_k, 8, 8);
  if (st != MOE_OK) return st;
  if (block_m < 1 || block_m > 256) return MOE_ERR_UNSUPPORTED;
  if (M == 0) return MOE_OK;
  if (!topk_ids || !sorted_token_ids || !expert_ids || !expert_block_offsets)
    return MOE_ERR_INVALID_ARG;
  const size_t need = align_scratch_bytes(M * top_k, E);
  if (need > 0 && (workspace == nullptr || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  AlignArgs a{topk_ids, M * top_k, E, block_m, sorted_token_ids, expert_ids,
              expert_block_offsets, expert_counts, static_cast<int32_t*>(workspace)};
  MOE_TRY_HIP(launch_align(a, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

int moe_grouped_gemm_w13_act(const uint16_t* x, const uint16_t* w13,
                             const int32_t* sorted_token_ids, const int32_t* expert_ids,
                             const int32_t* expert_block_offsets, int M, int top_k, int E,
                             int H, int I, int block_m, uint16_t* act,
                             moe_dispatch_info* info, void* stream) {
  int st = check_sizes(M, E, top_k, H, I);
  if (st != MOE_OK) return st;
  if (!gemm_block_ok(block_m)) return MOE_ERR_UNSUPPORTED;
  fill_info(info, block_m, H, I, M == 0 ? 0 : 1);
  if (M == 0) return MOE_OK;
  if (!x || !w13 || !sorted_token_ids || !expert_ids || !expert_block_offsets || !act)
    return MOE_ERR_INVALID_ARG;
  if (!a16(x) || !a16(w13) || !a16(sorted_token_ids) || !a16(act)) return MOE_ERR_INVALID_ARG;
  GemmArgs g = gemm_args(M, top_k, E, H, I, block_m);
  g.a_src = x;
  g.w = w13;
  g.sorted_token_ids = sorted_token_ids;
  g.expert_ids = expert_ids;
  g.expert_block_offsets = expert_block_offsets;
  g.out = act;
  return run_gemm1(g, static_cast<hipStream_t>(stream));
}

int moe_grouped_gemm_w2_combine(const uint16_t* act, const uint16_t* w2,
                                const float* topk_weights, const int32_t* sorted_token_ids,
                                const int32_t* expert_ids, const int32_t* expert_block_offsets,
                                int M, int top_k, int E, int H, int I, int block_m,
                                uint16_t* out, void* workspace, size_t ws_bytes,
                                moe_dispatch_info* info, void* stream) {
  int st = check_sizes(M, E, top_k, H, I);
  if (st != MOE_OK) return st;
  if (!gemm_block_ok(block_m)) return MOE_ERR_UNSUPPORTED;
  fill_info(info, block_m, H, I, M == 0 ? 0 : kGemm2Launches);
  if (M == 0) return MOE_OK;
  if (!act || !w2 || !topk_weights || !sorted_token_ids || !expert_ids ||
      !expert_block_offsets || !out)
    return MOE_ERR_INVALID_ARG;
  if (!a16(act) || !a16(w2) || !a16(sorted_token_ids) || !a16(out) || !a16(workspace))
    return MOE_ERR_INVALID_ARG;
  const Layout L = forward_layout(M, E, top_k, H, I, block_m);
  const size_t need = L.partial + (size_t)M * top_k * H * 4;
  if (workspace == nullptr || ws_bytes < need) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  GemmArgs g = gemm_args(M, top_k, E, H, I, block_m);
  g.a_src = act;
  g.w = w2;
  g.topk_weights = topk_weights;
  g.sorted_token_ids = sorted_token_ids;
  g.expert_ids = expert_ids;
  g.expert_block_offsets = expert_block_offsets;
  g.out = out;
  g.partial = reinterpret_cast<float*>(ws + L.partial);
  return run_gemm2(g, s);
}

int moe_forward(const uint16_t* x, const uint16_t* w_router, const float* logit_bias,
                const uint16_t* w13, const uint16_t* w2, int M, int E, int top_k, int H, int I,
                int renormalize, uint16_t* out, int32_t* topk_ids_out, float* topk_weights_out,
                void* workspace, size_t ws_bytes, moe_dispatch_info* info, void* stream) {
  int st = check_sizes(M, E, top_k, H, I);
  if (st != MOE_OK) return st;
  if (renormalize != 0 && renormalize != 1) return MOE_ERR_INVALID_ARG;
  const int B = moe_pick_block_m(M, E, top_k);
  const int route_launches = fused_route(M, top_k) ? 2 : 2 + (align_segments(M * top_k) > 1 ? 2 : 1);
  const bool per_pair = B == 1;
  if (per_pair)
    fill_info(info, B, H, I, kPairGemvForwardLaunches, 0);
  else
    fill_info(info, B, H, I, M == 0 ? 0 : route_launches + 1 + kGemm2Launches);
  if (M == 0) return MOE_OK;
  if (!x || !w_router || !w13 || !w2 || !out) return MOE_ERR_INVALID_ARG;
  if (!a16(x) || !a16(w_router) || !a16(w13) || !a16(w2) || !a16(out) || !a16(workspace))
    return MOE_ERR_INVALID_ARG;
  const Layout L = forward_layout(M, E, top_k, H, I, B);
  if (workspace == nullptr || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* wts = topk_weights_out ? topk_weights_out : reinterpret_cast<float*>(ws + L.wts);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* eids = reinterpret_cast<int32_t*>(ws + L.eids);
  int32_t* boff = reinterpret_cast<int32_t*>(ws + L.boff);
  uint16_t* act = reinterpret_cast<uint16_t*>(ws + L.act);

  // the router-logits kernel clears the arrival counter
  RouteArgs ra{x, w_router, logit_bias, M, H, E, top_k, renormalize,
               reinterpret_cast<float*>(ws + L.logits), ids, wts,
               reinterpret_cast<float*>(ws + L.arrive), 1};
  AlignArgs aa{ids, M * top_k, E, B, sorted, eids, boff,
               reinterpret_cast<int32_t*>(ws + L.counts),
               reinterpret_cast<int32_t*>(ws + L.align_scratch)};
  MOE_TRY_HIP(launch_route_logits(ra, s));
  if (per_pair) {
    PairGemvArgs pg{x, w13, w2, ids, wts, M, top_k, H, I, act, out, nullptr, nullptr, nullptr};
    MOE_TRY_HIP(launch_route_topk(ra, s));
    MOE_TRY_HIP(launch_pair_gemv1(pg, s));
    MOE_TRY_HIP(launch_pair_gemv2(pg, s));
    return MOE_OK;
  }
  if (fused_route(M, top_k)) {
    MOE_TRY_HIP(launch_route_topk_align(ra, aa, reinterpret_cast<int32_t*>(ws + L.arrive), s));
  } else {
    MOE_TRY_HIP(launch_route_topk(ra, s));
    MOE_TRY_HIP(launch_align(aa, s));
  }
  GemmArgs g = gemm_args(M, top_k, E, H, I, B);
  g.sorted_token_ids = sorted;
  g.expert_ids = eids;
  g.expert_block_offsets = boff;
  g.a_src = x;
  g.w = w13;
  g.out = act;
  st = run_gemm1(g, s);
  if (st != MOE_OK) return st;
  g.a_src = act;
  g.w = w2;
  g.topk_weights = wts;
  g.out = out;
  g.partial = reinterpret_cast<float*>(ws + L.partial);
  return run_gemm2(g, s);
}

int moe_forward_quantized(const uint16_t* x, const uint16_t* w_router, const float* logit_bias,
                          const moe_quantized_weights* qw, int M, int E, int top_k, int H, int I,
                          int renormalize, uint16_t* out, int32_t* topk_ids_out,
                          float* topk_weights_out, void* workspace, size_t ws_bytes,
                          moe_dispatch_info* info, void* stream) {
  int st = check_sizes(M, E, top_k, H, I);
  if (st != MOE_OK) return st;
  if (renormalize != 0 && renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (qw == nullptr) return MOE_ERR_INVALID_ARG;
  if ((qw->bits != 4 && qw->bits != 8) || qw->group_size != 64) return MOE_ERR_UNSUPPORTED;
  if (H % 64 != 0 || I % 64 != 0) return MOE_ERR_UNSUPPORTED;
  // per-pair GEMVs up to E/2 pairs, weight-streaming GEMMs over block_m 16
  // index lists (per-pair GEMVs instead for shapes the streaming kernels do
  // not take), the copy-wave tiles with the codes widened in LDS over
  // block_m 128 lists where the bf16 layer runs tiles (more than 8 pairs per
  // expert).  Measured on the Qwen3 shape (E = 128, top_k = 8; us, 4 / 8
  // bits): 8 tokens 63 / 71 per-pair against 69 / 81 streaming, 16 tokens
  // 103 / 129 against 84 / 102; 128 tokens 102 / 126 streaming against
  // 132 / 145 tiled, 256 tokens 155 / 191 against 152 / 158, 512 tokens
  // 245 / 318 against 198 / 209.
  int B = 1;
  if ((long long)M * top_k * 2 > E) {
    if (moe_pick_block_m(M, E, top_k) >= 64) B = 128;
    else if (qgemm_stream_shapes_ok(H, I)) B = 16;
  }
  const bool per_pair = B == 1;
  const int route_launches = fused_route(M, top_k) ? 2 : 2 + (align_segments(M * top_k) > 1 ? 2 : 1);
  if (per_pair) {
    fill_info(info, 1, H, I, M == 0 ? 0 : kPairGemvForwardLaunches, 0);
    if (info != nullptr) info->variant = MOE_VARIANT_PAIR_GEMV_QUANT;
  } else {
    fill_info(info, B, H, I, M == 0 ? 0 : route_launches + 1 + kGemm2Launches);
    if (info != nullptr) {
      info->variant = B == 16 ? MOE_VARIANT_STREAM_QUANT : MOE_VARIANT_TILED_QUANT;
      info->block_k = B == 16 ? 256 : kTiledBK;
      info->k_tail = H % info->block_k != 0 ? 1 : 0;
    }
  }
  if (M == 0) return MOE_OK;
  if (!x || !w_router || !out || !qw->w13_q || !qw->w13_scales || !qw->w13_biases ||
      !qw->w2_q || !qw->w2_scales || !qw->w2_biases)
    return MOE_ERR_INVALID_ARG;
  if (!a16(x) || !a16(w_router) || !a16(out) || !a16(workspace) || !a16(qw->w13_q) ||
      !a16(qw->w2_q) || !a16(qw->w13_scales) || !a16(qw->w13_biases) || !a16(qw->w2_scales) ||
      !a16(qw->w2_biases))
    return MOE_ERR_INVALID_ARG;
  const Layout L = forward_layout(M, E, top_k, H, I, B);
  if (workspace == nullptr || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* wts = topk_weights_out ? topk_weights_out : reinterpret_cast<float*>(ws + L.wts);
  uint16_t* act = reinterpret_cast<uint16_t*>(ws + L.act);
  RouteArgs ra{x, w_router, logit_bias, M, H, E, top_k, renormalize,
               reinterpret_cast<float*>(ws + L.logits), ids, wts,
               per_pair ? nullptr : reinterpret_cast<float*>(ws + L.arrive), per_pair ? 0u : 1u};
  MOE_TRY_HIP(launch_route_logits(ra, s));
  if (per_pair) {
    QPairGemvArgs q{x, qw->w13_q, qw->w13_scales, qw->w13_biases, qw->w2_q, qw->w2_scales,
                    qw->w2_biases, ids, wts, M, top_k, H, I, qw->bits, act, out};
    MOE_TRY_HIP(launch_route_topk(ra, s));
    MOE_TRY_HIP(launch_qpair_gemv1(q, s));
    MOE_TRY_HIP(launch_qpair_gemv2(q, s));
    return MOE_OK;
  }
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* eids = reinterpret_cast<int32_t*>(ws + L.eids);
  int32_t* boff = reinterpret_cast<int32_t*>(ws + L.boff);
  AlignArgs aa{ids, M * top_k, E, B, sorted, eids, boff,
               reinterpret_cast<int32_t*>(ws + L.counts),
               reinterpret_cast<int32_t*>(ws + L.align_scratch)};
  if (fused_route(M, top_k)) {
    MOE_TRY_HIP(launch_route_topk_align(ra, aa, reinterpret_cast<int32_t*>(ws + L.arrive), s));
  } else {
    MOE_TRY_HIP(launch_route_topk(ra, s));
    MOE_TRY_HIP(launch_align(aa, s));
  }
  QGemmArgs g{x, qw->w13_q, qw->w13_scales, qw->w13_biases, qw->w2_q, qw->w2_scales,
              qw->w2_biases, sorted, eids, boff, wts, M, top_k, E, H, I, qw->bits,
              (int)max_blocks((long long)M * top_k, E, B), act,
              reinterpret_cast<float*>(ws + L.partial), out};
  if (B == 16) {
    MOE_TRY_HIP(launch_qgemm1_stream(g, s));
    MOE_TRY_HIP(launch_qgemm2_stream(g, s));
  } else {
    MOE_TRY_HIP(launch_qgemm1_tiled(g, s));
    MOE_TRY_HIP(launch_qgemm2_tiled(g, s));
  }
  return MOE_OK;
}

}  // extern "C"

// ---- MXFP8 layer ----

namespace {

struct MxLayout {
  Layout base;
  size_t qx, sx, qact, sact, total;
};

// the tile table's block size (1: per-pair MXFP8 GEMVs, no index lists)
int mx_block_m(int M, int E, int top_k) { return moe_pick_block_m(M, E, top_k); }

MxLayout mx_layout(int M, int E, int top_k, int H, int I, int B) {
  MxLayout L;
  L.base = forward_layout(M, E, top_k, H, I, B);
  const size_t P = (size_t)M * top_k;
  size_t off = L.base.total;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.qx = take((size_t)M * H);
  L.sx = take((size_t)M * H / 32);
  L.qact = take(P * I);
  L.sact = take(P * I / 32);
  L.total = off;
  return L;
}

bool mx_sizes_ok(int H, int I) { return H % 128 == 0 && I % 128 == 0; }

}  // namespace

extern "C" {

int moe_mx_quantize(const uint16_t* src, int rows, int K, uint8_t* codes, uint8_t* scales,
                    void* stream) {
  if (rows < 0 || K <= 0) return MOE_ERR_INVALID_ARG;
  if (K % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!src || !codes || !scales || !a16(src) || !a16(codes)) return MOE_ERR_INVALID_ARG;
  MOE_TRY_HIP(launch_mx_quantize(src, rows, K, codes, scales, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

size_t moe_mx_workspace_size(int M_max, int E, int top_k, int H, int I) {
  if (check_sizes(M_max, E, top_k, H, I) != MOE_OK || !mx_sizes_ok(H, I)) return 0;
  size_t best = 0;
  for (int B : kBlockSizes) best = std::max(best, mx_layout(M_max, E, top_k, H, I, B).total);
  return std::max<size_t>(best, kAlign);
}

int moe_forward_mxfp8(const uint16_t* x, const uint16_t* w_router, const float* logit_bias,
                      const moe_mx_weights* w, int M, int E, int top_k, int H, int I,
                      int renormalize, uint16_t* out, int32_t* topk_ids_out,
                      float* topk_weights_out, void* workspace, size_t ws_bytes,
                      moe_dispatch_info* info, void* stream) {
  int st = check_sizes(M, E, top_k, H, I);
  if (st != MOE_OK) return st;
  if (renormalize != 0 && renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (w == nullptr) return MOE_ERR_INVALID_ARG;
  if (!mx_sizes_ok(H, I)) return MOE_ERR_UNSUPPORTED;
  const int B = mx_block_m(M, E, top_k);
  const bool per_pair = B == 1;
  const int route_launches = fused_route(M, top_k) ? 2 : 2 + (align_segments(M * top_k) > 1 ? 2 : 1);
  if (per_pair) {
    // router logits, top-k (+ x quantized), GEMV 1, GEMV 2 with the sum
    fill_info(info, B, H, I, M == 0 ? 0 : kPairGemvForwardLaunches, 0);
    if (info != nullptr) info->variant = MOE_VARIANT_PAIR_GEMV_MXFP8;
  } else {
    // GEMM 1, quantize act (in GEMM 1's epilogue at block_m 16), then GEMM 2
    // and its per-token sum (x is quantized by the top-k launch)
    fill_info(info, B, H, I, M == 0 ? 0 : route_launches + (B == 16 ? 1 : 2) + kGemm2Launches);
    if (info != nullptr)
      info->variant = B == 16 ? MOE_VARIANT_STREAM_MXFP8 : MOE_VARIANT_TILED_MXFP8;
  }
  if (M == 0) return MOE_OK;
  if (!x || !w_router || !out || !w->w13_codes || !w->w13_scales || !w->w2_codes ||
      !w->w2_scales)
    return MOE_ERR_INVALID_ARG;
  if (!a16(x) || !a16(w_router) || !a16(out) || !a16(workspace) || !a16(w->w13_codes) ||
      !a16(w->w2_codes) || !a16(w->w13_scales) || !a16(w->w2_scales))
    return MOE_ERR_INVALID_ARG;
  const MxLayout X = mx_layout(M, E, top_k, H, I, B);
  const Layout& L = X.base;
  if (workspace == nullptr || ws_bytes < X.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* wts = topk_weights_out ? topk_weights_out : reinterpret_cast<float*>(ws + L.wts);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* eids = reinterpret_cast<int32_t*>(ws + L.eids);
  int32_t* boff = reinterpret_cast<int32_t*>(ws + L.boff);
  uint16_t* act = reinterpret_cast<uint16_t*>(ws + L.act);
  uint8_t* qx = reinterpret_cast<uint8_t*>(ws + X.qx);
  uint8_t* sx = reinterpret_cast<uint8_t*>(ws + X.sx);
  uint8_t* qact = reinterpret_cast<uint8_t*>(ws + X.qact);
  uint8_t* sact = reinterpret_cast<uint8_t*>(ws + X.sact);

  RouteArgs ra{x, w_router, logit_bias, M, H, E, top_k, renormalize,
               reinterpret_cast<float*>(ws + L.logits), ids, wts,
               reinterpret_cast<float*>(ws + L.arrive), 1};
  AlignArgs aa{ids, M * top_k, E, B, sorted, eids, boff,
               reinterpret_cast<int32_t*>(ws + L.counts),
               reinterpret_cast<int32_t*>(ws + L.align_scratch)};
  MOE_TRY_HIP(launch_route_logits(ra, s));
  if (per_pair) {
    // Small batches skip the sort: the top-k launch also quantizes x, and
    // each pair runs as its own GEMV against its expert's MXFP8 rows.
    ra.qx_codes = qx;
    ra.qx_scales = sx;
    MOE_TRY_HIP(launch_route_topk(ra, s));
    MxPairGemvArgs pg{qx, sx, w->w13_codes, w->w13_scales, w->w2_codes, w->w2_scales, ids, wts,
                      M, top_k, H, I, act, out};
    MOE_TRY_HIP(launch_mx_pair_gemv1(pg, s));
    MOE_TRY_HIP(launch_mx_pair_gemv2(pg, s));
    return MOE_OK;
  }
  // the top-k launch also quantizes x
  ra.qx_codes = qx;
  ra.qx_scales = sx;
  if (fused_route(M, top_k)) {
    MOE_TRY_HIP(launch_route_topk_align(ra, aa, reinterpret_cast<int32_t*>(ws + L.arrive), s));
  } else {
    MOE_TRY_HIP(launch_route_topk(ra, s));
    MOE_TRY_HIP(launch_align(aa, s));
  }
  GemmArgs g = gemm_args(M, top_k, E, H, I, B);
  g.sorted_token_ids = sorted;
  g.expert_ids = eids;
  g.expert_block_offsets = boff;
  g.mx = 1;
  g.a_src = reinterpret_cast<const uint16_t*>(qx);
  g.a_scales = sx;
  g.w = reinterpret_cast<const uint16_t*>(w->w13_codes);
  g.w_scales = w->w13_scales;
  g.out = act;
  if (B == 16) {
    // the streaming GEMM 1 quantizes act in its epilogue
    MOE_TRY_HIP(launch_gemm1_stream_mx_quantize(g, qact, sact, s));
  } else {
    MOE_TRY_HIP(launch_gemm1_tiled(g, s));
    MOE_TRY_HIP(launch_mx_quantize(act, M * top_k, I, qact, sact, s));
  }
  g.a_src = reinterpret_cast<const uint16_t*>(qact);
  g.a_scales = sact;
  g.w = reinterpret_cast<const uint16_t*>(w->w2_codes);
  g.w_scales = w->w2_scales;
  g.topk_weights = wts;
  g.out = out;
  g.partial = reinterpret_cast<float*>(ws + L.partial);
  MOE_TRY_HIP(B == 16 ? launch_gemm2_stream(g, s) : launch_gemm2_tiled(g, s));
  return MOE_OK;
}

}  // extern "C"
