// C ABI of libmoe.so: host-side validation, workspace layout and the order
// of kernel launches.  Declarations and the meaning of every argument are
// in include/moe.h.
#include <cmath>
#include <mutex>

#include "../../include/moe.h"
#include "ffn_common.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
constexpr int kPlanCounters = kCtrSets * kXcds;  // GEMM work counters after the tile plan

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

moe_status check_desc(const moe_desc* d) {
  if (!d) return MOE_ERR_NULL;
  if (d->T < 0 || d->d <= 0 || d->F <= 0 || d->E <= 0 || d->S < 0 || d->k <= 0)
    return MOE_ERR_SHAPE;
  if (d->act != MOE_F32 && d->act != MOE_BF16) return MOE_ERR_DTYPE;
  const bool fp4 = d->act == MOE_BF16 && d->weight == MOE_MXFP4;
  if (d->weight != d->act && !fp4) return MOE_ERR_DTYPE;
  if (d->gate_norm != MOE_GATE_RATIO && d->gate_norm != MOE_GATE_LOGSUMEXP) return MOE_ERR_SHAPE;
  if (!(d->gate_scale > 0.0f) || !(d->gate_scale < INFINITY)) return MOE_ERR_SHAPE;
  if (!(d->capacity_factor >= 0.0f) || !(d->capacity_factor < INFINITY)) return MOE_ERR_SHAPE;
  if ((d->E != 64 && d->E != 128 && d->E != 256) || d->S > 2 || d->k != 6)
    return MOE_ERR_UNSUPPORTED;
  if (d->d % 32 != 0) return MOE_ERR_UNSUPPORTED;
  const long long T = d->T;
  if (T * d->k >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  const long long wide = d->d > d->F ? d->d : d->F;
  if (T * (d->k + d->S) * wide >= (1LL << 40)) return MOE_ERR_UNSUPPORTED;
  // FP4 routed weights: decode batches (the 32-row GEMM path) only
  if (fp4 && T * d->k >= 48LL * d->E) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The expert GEMMs' tiles need d % 256 == 0 and F % 128 == 0 (the router,
// dispatch, combine and bias update only d % 32 == 0).
moe_status check_ffn_desc(const moe_desc* d) {
  const moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->d % 256 != 0 || d->F % 128 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

Shape to_shape(const moe_desc* d) {
  Shape s;
  s.T = d->T;
  s.d = d->d;
  s.F = d->F;
  s.E = d->E;
  s.S = d->S;
  s.k = d->k;
  s.bf16 = d->act == MOE_BF16;
  s.w_fp4 = d->weight == MOE_MXFP4;
  s.gate_logsumexp = d->gate_norm == MOE_GATE_LOGSUMEXP;
  s.gate_scale = d->gate_scale;
  s.capacity = INT32_MAX;
  if (d->capacity_factor > 0.0f) {
    const double c = std::ceil(static_cast<double>(d->capacity_factor) *
                               static_cast<double>(static_cast<long long>(d->k) * d->T) /
                               static_cast<double>(d->E));
    s.capacity = c < static_cast<double>(INT32_MAX) ? static_cast<int>(c) : INT32_MAX;
  }
  return s;
}

size_t esize(const Shape& s) { return s.bf16 ? 2 : 4; }

// Workspace carving: a bump allocator over the caller's buffer.
struct Carver {
  char* base;
  size_t used = 0;
  template <typename T> T* take(size_t count) {
    T* p = reinterpret_cast<T*>(base ? base + used : nullptr);
    used = align_up(used + count * sizeof(T));
    return p;
  }
};

struct RouterWs { bf16_t* planes; double* partial; int32_t* refine; };
RouterWs carve_router(Carver& c, const Shape& s) {
  RouterWs r;
  const size_t npad = router_cols_padded(s);
  r.planes = c.take<bf16_t>(3 * npad * s.d);
  r.partial = c.take<double>(static_cast<size_t>(router_ksplits(s)) * s.T * npad);
  r.refine = c.take<int32_t>(router_refine_ints(s));
  return r;
}
int32_t* carve_dispatch(Carver& c, const Shape& s) {
  return c.take<int32_t>(static_cast<size_t>(dispatch_segments(s)) * s.E + 1);
}
int32_t* carve_plan(Carver& c, const Shape& s) {
  const int small = s.E + s.S + 1 + kPlanCounters;
  const int big = big_plan_ints(s.E + s.S);
  return c.take<int32_t>(small > big ? small : big);
}
float* carve_part(Carver& c, const Shape& s) { return c.take<float>(shared_partial_floats(s)); }
void* carve_h(Carver& c, const Shape& s) {
  return c.take<char>(static_cast<size_t>(s.k + s.S) * s.T * s.F * esize(s));
}

struct FwdWs {
  int32_t* topk;
  float* gates;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_pair;
  int32_t* pair_pos;
  RouterWs router;
  int32_t* seg;
  int32_t* plan;
  void* h;
  void* y_routed;
  void* y_shared;
  float* part;
};
FwdWs carve_forward(Carver& c, const Shape& s) {
  FwdWs w;
  const size_t kT = static_cast<size_t>(s.k) * s.T;
  w.topk = c.take<int32_t>(kT);
  w.gates = c.take<float>(static_cast<size_t>(s.k + s.S) * s.T);
  w.counts = c.take<int32_t>(s.E);
  w.offsets = c.take<int32_t>(s.E + 1);
  w.sorted_pair = c.take<int32_t>(kT);
  w.pair_pos = c.take<int32_t>(kT);
  w.router = carve_router(c, s);
  w.seg = carve_dispatch(c, s);
  w.plan = carve_plan(c, s);
  w.h = carve_h(c, s);
  w.y_routed = c.take<char>(kT * s.d * esize(s));
  w.y_shared = c.take<char>(static_cast<size_t>(s.S) * s.T * s.d * esize(s));
  w.part = carve_part(c, s);
  return w;
}

size_t ws_bytes_for(const Shape& s, moe_call call) {
  Carver c{nullptr};
  switch (call) {
    case MOE_CALL_ROUTER: carve_router(c, s); break;
    case MOE_CALL_DISPATCH: carve_dispatch(c, s); break;
    case MOE_CALL_GATE_UP:
    case MOE_CALL_DOWN: carve_plan(c, s); carve_part(c, s); break;
    case MOE_CALL_EXPERT_FFN: carve_plan(c, s); carve_h(c, s); carve_part(c, s); break;
    case MOE_CALL_FORWARD: carve_forward(c, s); break;
    default: break;
  }
  return c.used;
}

moe_status check_ws(const Shape& s, moe_call call, const void* ws, size_t ws_bytes) {
  const size_t need = ws_bytes_for(s, call);
  if (need == 0) return MOE_OK;
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

bool weights_ok(const moe_weights* w, const Shape& s) {
  if (!(w && w->w_gate && w->w_up && w->w_down)) return false;
  if (s.S > 0 && !(w->ws_gate && w->ws_up && w->ws_down)) return false;
  return !s.w_fp4 || (w->sc_gate && w->sc_up && w->sc_down);
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "invalid size, gamma, gate normalisation or capacity factor";
    case MOE_ERR_DTYPE:
      return "unsupported dtype (act and weight both f32, both bf16, or bf16 with MXFP4 weights)";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_UNSUPPORTED: return "shape outside the supported limits";
    case MOE_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

moe_status moe_workspace_size(const moe_desc* desc, moe_call call, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  if (call < MOE_CALL_ROUTER || call > MOE_CALL_FORWARD) return desc ? MOE_ERR_SHAPE : MOE_ERR_NULL;
  const bool ffn = call == MOE_CALL_GATE_UP || call == MOE_CALL_DOWN ||
                   call == MOE_CALL_EXPERT_FFN || call == MOE_CALL_FORWARD;
  const moe_status st = ffn ? check_ffn_desc(desc) : check_desc(desc);
  if (st != MOE_OK) return st;
  *bytes = ws_bytes_for(to_shape(desc), call);
  return MOE_OK;
}

moe_status moe_router(const moe_desc* desc, const void* x, const float* w_router,
                      const float* bias, int32_t* topk_idx, float* gates,
                      float* margin_or_null, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  const Shape s = to_shape(desc);
  if (s.T > 0 && (!x || !w_router || !bias || !topk_idx || !gates)) return MOE_ERR_NULL;
  if ((st = check_ws(s, MOE_CALL_ROUTER, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  const RouterWs r = carve_router(c, s);
  return hip_status(launch_router(s, x, w_router, nullptr, bias, topk_idx, gates,
                                  margin_or_null, r.planes, r.partial, r.refine, stream));
}

moe_status moe_router_planes_size(const moe_desc* desc, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  const moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  const Shape s = to_shape(desc);
  *bytes = 3 * static_cast<size_t>(router_cols_padded(s)) * s.d * sizeof(bf16_t);
  return MOE_OK;
}

moe_status moe_router_prepare(const moe_desc* desc, const float* w_router, uint16_t* planes,
                              hipStream_t stream) {
  const moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (!w_router || !planes) return MOE_ERR_NULL;
  return hip_status(launch_router_planes(to_shape(desc), w_router, planes, stream));
}

moe_status moe_dispatch(const moe_desc* desc, const int32_t* topk_idx, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  const Shape s = to_shape(desc);
  if (!counts || !offsets) return MOE_ERR_NULL;
  if (s.T > 0 && (!topk_idx || !sorted_pair || !pair_pos)) return MOE_ERR_NULL;
  if ((st = check_ws(s, MOE_CALL_DISPATCH, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  int32_t* seg = carve_dispatch(c, s);
  return hip_status(
      launch_dispatch(s, topk_idx, counts, offsets, sorted_pair, pair_pos, seg, stream));
}

moe_status moe_expert_gate_up(const moe_desc* desc, const void* x, const moe_weights* w,
                              const int32_t* offsets, const int32_t* sorted_pair, void* h,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_ffn_desc(desc);
  if (st != MOE_OK) return st;
  const Shape s = to_shape(desc);
  if (!weights_ok(w, s) || !offsets) return MOE_ERR_NULL;
  if (s.T > 0 && (!x || !sorted_pair || !h)) return MOE_ERR_NULL;
  if ((st = check_ws(s, MOE_CALL_GATE_UP, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  int32_t* plan = carve_plan(c, s);
  float* part = carve_part(c, s);
  const int mt = ffn_row_tile(s);
  hipError_t e = launch_tile_plan(s, offsets, mt, plan, stream);
  if (e == hipSuccess)
    e = launch_gate_up(s, x, w->w_gate, w->w_up, w->ws_gate, w->ws_up, w->sc_gate, w->sc_up,
                       offsets, sorted_pair, plan, mt, h, part, nullptr, stream);
  return hip_status(e);
}

moe_status moe_expert_down(const moe_desc* desc, const moe_weights* w, const int32_t* offsets,
                           const void* h, void* y_routed, void* y_shared, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_ffn_desc(desc);
  if (st != MOE_OK) return st;
  const Shape s = to_shape(desc);
  if (!weights_ok(w, s) || !offsets) return MOE_ERR_NULL;
  if (s.T > 0 && (!h || !y_routed || (s.S > 0 && !y_shared))) return MOE_ERR_NULL;
  if ((st = check_ws(s, MOE_CALL_DOWN, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  int32_t* plan = carve_plan(c, s);
  float* part = carve_part(c, s);
  const int mt = ffn_row_tile(s);
  hipError_t e = launch_tile_plan(s, offsets, mt, plan, stream);
  if (e == hipSuccess)
    e = launch_down(s, w->w_down, w->ws_down, w->sc_down, offsets, plan, mt, h, y_routed,
                    y_shared, part, nullptr, stream);
  return hip_status(e);
}

moe_status moe_expert_gate_up_marked(const moe_desc* desc, const void* x, const moe_weights* w,
                                     const int32_t* offsets, const int32_t* sorted_pair, void* h,
                                     void* ws, size_t ws_bytes, hipEvent_t* marks,
                                     hipStream_t stream) {
  moe_status st = check_ffn_desc(desc);
  if (st != MOE_OK) return st;
  const Shape s = to_shape(desc);
  if (!weights_ok(w, s) || !offsets || !marks || !marks[0] || !marks[1])
    return MOE_ERR_NULL;
  if (s.T > 0 && (!x || !sorted_pair || !h)) return MOE_ERR_NULL;
  if ((st = check_ws(s, MOE_CALL_GATE_UP, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  int32_t* plan = carve_plan(c, s);
  float* part = carve_part(c, s);
  const int mt = ffn_row_tile(s);
  hipError_t e = launch_tile_plan(s, offsets, mt, plan, stream);
  if (e == hipSuccess) e = hipEventRecord(marks[0], stream);
  if (e == hipSuccess)
    e = launch_gate_up(s, x, w->w_gate, w->w_up, w->ws_gate, w->ws_up, w->sc_gate, w->sc_up,
                       offsets, sorted_pair, plan, mt, h, part, marks + 1, stream);
  return hip_status(e);
}

moe_status moe_expert_down_marked(const moe_desc* desc, const moe_weights* w,
                                  const int32_t* offsets, const void* h, void* y_routed,
                                  void* y_shared, void* ws, size_t ws_bytes, hipEvent_t* marks,
                                  hipStream_t stream) {
  moe_status st = check_ffn_desc(desc);
  if (st != MOE_OK) return st;
  const Shape s = to_shape(desc);
  if (!weights_ok(w, s) || !offsets || !marks || !marks[0] || !marks[1])
    return MOE_ERR_NULL;
  if (s.T > 0 && (!h || !y_routed || (s.S > 0 && !y_shared))) return MOE_ERR_NULL;
  if ((st = check_ws(s, MOE_CALL_DOWN, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  int32_t* plan = carve_plan(c, s);
  float* part = carve_part(c, s);
  const int mt = ffn_row_tile(s);
  hipError_t e = launch_tile_plan(s, offsets, mt, plan, stream);
  if (e == hipSuccess) e = hipEventRecord(marks[0], stream);
  if (e == hipSuccess)
    e = launch_down(s, w->w_down, w->ws_down, w->sc_down, offsets, plan, mt, h, y_routed,
                    y_shared, part, marks + 1, stream);
  return hip_status(e);
}

moe_status moe_expert_ffn(const moe_desc* desc, const void* x, const moe_weights* w,
                          const int32_t* offsets, const int32_t* sorted_pair, void* y_routed,
                          void* y_shared, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_ffn_desc(desc);
  if (st != MOE_OK) return st;
  const Shape s = to_shape(desc);
  if (!weights_ok(w, s) || !offsets) return MOE_ERR_NULL;
  if (s.T > 0 && (!x || !sorted_pair || !y_routed || (s.S > 0 && !y_shared)))
    return MOE_ERR_NULL;
  if ((st = check_ws(s, MOE_CALL_EXPERT_FFN, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  int32_t* plan = carve_plan(c, s);
  void* h = carve_h(c, s);
  float* part = carve_part(c, s);
  const int mt = ffn_row_tile(s);
  hipError_t e = launch_tile_plan(s, offsets, mt, plan, stream);
  if (e == hipSuccess)
    e = launch_gate_up(s, x, w->w_gate, w->w_up, w->ws_gate, w->ws_up, w->sc_gate, w->sc_up,
                       offsets, sorted_pair, plan, mt, h, part, nullptr, stream);
  if (e == hipSuccess)
    e = launch_down(s, w->w_down, w->ws_down, w->sc_down, offsets, plan, mt, h, y_routed,
                    y_shared, part, nullptr, stream);
  return hip_status(e);
}

moe_status moe_combine(const moe_desc* desc, const void* y_routed, const void* y_shared,
                       const float* gates, const int32_t* pair_pos, void* y,
                       hipStream_t stream) {
  const moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  const Shape s = to_shape(desc);
  if (s.T > 0 && (!y_routed || (s.S > 0 && !y_shared) || !gates || !pair_pos || !y))
    return MOE_ERR_NULL;
  return hip_status(launch_combine(s, y_routed, y_shared, gates, pair_pos, y, stream));
}

moe_status moe_bias_update(const moe_desc* desc, const int32_t* counts, float gamma,
                           float* bias, hipStream_t stream) {
  const moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (!counts || !bias) return MOE_ERR_NULL;
  if (!std::isfinite(gamma)) return MOE_ERR_SHAPE;
  return hip_status(launch_bias_update(to_shape(desc), counts, gamma, bias, stream));
}

moe_status moe_quantize_mxfp4(int32_t E, int32_t N, int32_t K, const void* w, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream) {
  if (E < 0 || N <= 0 || K <= 0 || K % 128 != 0) return MOE_ERR_SHAPE;
  if (E == 0) return MOE_OK;
  if (!w || !codes || !scales) return MOE_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(w) % 16 != 0 || reinterpret_cast<uintptr_t>(codes) % 16 != 0)
    return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_quantize_mxfp4(E, N, K, w, codes, scales, stream));
}

}  // extern "C"

namespace {

// moe_forward's launches; marks (7 events, or NULL) are recorded after the
// router, the dispatch, the tile plan, the gate/up GEMM, the down GEMM, the
// combine and the bias update.  Small batches with 32-row tiles make the
// tile plan and the bias update in the dispatch launch (their marks then
// follow the dispatch and the combine).  With the fused shared-expert down + combine
// (large batches with shared experts) the down mark follows the routed
// experts' down GEMM and the combine mark the fused launch.
moe_status forward_impl(const moe_desc* desc, const void* x, const moe_weights* w, float* bias,
                        float gamma, void* y, const moe_routing* routing, void* ws,
                        size_t ws_bytes, hipEvent_t* marks, hipStream_t stream) {
  moe_status st = check_ffn_desc(desc);
  if (st != MOE_OK) return st;
  const Shape s = to_shape(desc);
  if (!weights_ok(w, s) || !w->w_router || !bias) return MOE_ERR_NULL;
  if (s.T > 0 && (!x || !y)) return MOE_ERR_NULL;
  if (!std::isfinite(gamma)) return MOE_ERR_SHAPE;
  if (marks)
    for (int i = 0; i < 7; ++i)
      if (!marks[i]) return MOE_ERR_NULL;
  if ((st = check_ws(s, MOE_CALL_FORWARD, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  FwdWs f = carve_forward(c, s);
  float* margin = nullptr;
  if (routing) {
    if (routing->topk_idx) f.topk = routing->topk_idx;
    if (routing->gates) f.gates = routing->gates;
    if (routing->counts) f.counts = routing->counts;
    if (routing->offsets) f.offsets = routing->offsets;
    if (routing->sorted_pair) f.sorted_pair = routing->sorted_pair;
    if (routing->pair_pos) f.pair_pos = routing->pair_pos;
    margin = routing->margin;
  }
  auto mark = [&](int i, hipError_t e) {
    return (e == hipSuccess && marks) ? hipEventRecord(marks[i], stream) : e;
  };
  const int mt = ffn_row_tile(s);
  hipError_t e = launch_router(s, x, w->w_router, w->w_router_planes, bias, f.topk, f.gates,
                               margin, f.router.planes, f.router.partial, f.router.refine,
                               stream);
  e = mark(0, e);
  // small batches with 32-row tiles: dispatch, tile plan and bias update in
  // one launch (the bias has been read by the router)
  const bool small = mt == 32 && dispatch_is_small(s);
  if (e == hipSuccess) {
    if (small)
      e = launch_dispatch_small(s, f.topk, f.counts, f.offsets, f.sorted_pair, f.pair_pos, mt,
                                f.plan, gamma, bias, stream);
    else
      e = launch_dispatch(s, f.topk, f.counts, f.offsets, f.sorted_pair, f.pair_pos, f.seg,
                          stream);
  }
  e = mark(1, e);
  if (e == hipSuccess && !small) e = launch_tile_plan(s, f.offsets, mt, f.plan, stream);
  e = mark(2, e);
  // Large batches (256-row tiles) with shared experts: the shared experts'
  // down GEMM runs after the routed one, fused with the combine (their rows
  // of h carry their gates), so Y_s never goes through HBM.  With 128-row
  // tiles (~100 rows per expert) the fused launch has about one tile per CU
  // and its combine epilogue runs alone, slower than the combine kernel.
  const bool fused = s.bf16 && s.S > 0 && mt == BigCfgRows;
  if (e == hipSuccess)
    e = launch_gate_up(s, x, w->w_gate, w->w_up, w->ws_gate, w->ws_up, w->sc_gate, w->sc_up,
                       f.offsets, f.sorted_pair, f.plan, mt, f.h, f.part,
                       marks ? marks + 3 : nullptr, stream, fused ? f.gates : nullptr);
  // FP4 routed weights with shared experts: the combine sums the shared
  // experts' K-slice partials itself
  const bool fp4_part = s.w_fp4 && s.bf16 && s.S > 0 && mt == 32;
  if (e == hipSuccess)
    e = launch_down(s, w->w_down, w->ws_down, w->sc_down, f.offsets, f.plan, mt, f.h, f.y_routed,
                    f.y_shared, f.part, marks ? marks + 4 : nullptr, stream, fused, fp4_part);
  if (e == hipSuccess) {
    if (fused)
      e = launch_shared_combine(s, w->ws_down, f.plan, mt, f.h, f.y_routed, f.gates,
                                f.pair_pos, y, stream);
    else if (fp4_part)
      e = launch_combine_part(s, f.y_routed, f.part, fp4_shared_slices(s.F), f.gates,
                              f.pair_pos, y, stream);
    else
      e = launch_combine(s, f.y_routed, f.y_shared, f.gates, f.pair_pos, y, stream);
  }
  e = mark(5, e);
  if (e == hipSuccess && !small && gamma != 0.0f)
    e = launch_bias_update(s, f.counts, gamma, bias, stream);
  e = mark(6, e);
  return hip_status(e);
}

}  // namespace

extern "C" {

moe_status moe_forward(const moe_desc* desc, const void* x, const moe_weights* w, float* bias,
                       float gamma, void* y, const moe_routing* routing, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  return forward_impl(desc, x, w, bias, gamma, y, routing, ws, ws_bytes, nullptr, stream);
}

moe_status moe_forward_marked(const moe_desc* desc, const void* x, const moe_weights* w,
                              float* bias, float gamma, void* y, const moe_routing* routing,
                              void* ws, size_t ws_bytes, hipEvent_t* marks, hipStream_t stream) {
  if (!marks) return MOE_ERR_NULL;
  return forward_impl(desc, x, w, bias, gamma, y, routing, ws, ws_bytes, marks, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- no-alloc

// Scratch of moe_dispatch_noalloc: the dispatch's per-segment expert counts
// (dispatch_segments(s) * E + 1 ints), in an array the library owns instead
// of a caller workspace.  Each GPU holds its own copy for the life of the
// process.  Host code never passes this name to a kernel: it takes the
// device address from hipGetSymbolAddress once per device (scratch_on).
constexpr size_t kNoAllocScratchInts = size_t(1) << 18;  // 1 MiB
static __device__ __align__(256) int32_t scratch[kNoAllocScratchInts];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept; nullptr on a HIP error.
int32_t* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" moe_status moe_dispatch_noalloc(const moe_desc* desc, const int32_t* topk_idx,
                                           int32_t* counts, int32_t* offsets,
                                           int32_t* sorted_pair, int32_t* pair_pos,
                                           hipStream_t stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  const Shape s = to_shape(desc);
  if (!counts || !offsets) return MOE_ERR_NULL;
  if (s.T > 0 && (!topk_idx || !sorted_pair || !pair_pos)) return MOE_ERR_NULL;
  const size_t need = static_cast<size_t>(dispatch_segments(s)) * s.E + 1;
  if (need > kNoAllocScratchInts) return MOE_ERR_UNSUPPORTED;
  int32_t* seg = scratch_on_current_device();
  if (!seg) return MOE_ERR_HIP;
  return hip_status(
      launch_dispatch(s, topk_idx, counts, offsets, sorted_pair, pair_pos, seg, stream));
}
