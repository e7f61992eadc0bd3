// C ABI of the MoE layer (declared in include/moe.h): argument checks,
// workspace sizing and launch sequencing.  Every check runs on the host
// before anything is enqueued; no call allocates, frees or synchronises.
#include "moe.h"

#include <new>

#include "moe_internal.h"

namespace {

using moe::Shape;

bool supported_pair(int act, int weight) {
  return (act == MOE_F32 && weight == MOE_F32) || (act == MOE_BF16 && weight == MOE_BF16) ||
         (act == MOE_BF16 && weight == MOE_FP8_E4M3) || (act == MOE_BF16 && weight == MOE_MXFP4);
}

// Shape checks shared by every call.  Returns MOE_OK and fills `s` on success.
moe_status_t check_problem(const moe_problem_t* p, Shape* s) {
  if (p == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (p->T < 0 || p->d <= 0 || p->E <= 0 || p->F <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (p->k < 1 || p->k > p->E) return MOE_ERR_INVALID_ARGUMENT;
  if (p->expert_begin < 0 || p->num_local < 1) return MOE_ERR_INVALID_ARGUMENT;
  if ((long long)p->expert_begin + p->num_local > p->E) return MOE_ERR_INVALID_ARGUMENT;
  if (p->d % 128 != 0 || p->F % 128 != 0) return MOE_ERR_INVALID_ARGUMENT;
  if (p->act < MOE_F32 || p->act > MOE_MXFP4 || p->weight < MOE_F32 || p->weight > MOE_MXFP4)
    return MOE_ERR_INVALID_ARGUMENT;
  if (p->weight_layout != MOE_LAYOUT_ROWS && p->weight_layout != MOE_LAYOUT_BLOCKED)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!supported_pair(p->act, p->weight)) return MOE_ERR_UNSUPPORTED;
  if (p->weight_layout == MOE_LAYOUT_BLOCKED && p->weight == MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (p->E > moe::kMaxExperts || p->d > 65536 || p->F > 65536) return MOE_ERR_UNSUPPORTED;
  const long long S = (long long)p->T * p->k;
  if (S >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  // the expert GEMMs address x and one expert's weight matrix with 32-bit
  // offsets
  const long long ab = p->act == MOE_F32 ? 4 : 2;
  const long long wbits = p->weight == MOE_F32 ? 32 : p->weight == MOE_BF16 ? 16
                        : p->weight == MOE_FP8_E4M3 ? 8 : 4;
  if ((long long)p->T * p->d * ab >= (1LL << 32) || (long long)p->F * p->d * wbits / 8 >= (1LL << 32))
    return MOE_ERR_UNSUPPORTED;
  s->T = p->T;
  s->d = p->d;
  s->E = p->E;
  s->k = p->k;
  s->F = p->F;
  s->e0 = p->expert_begin;
  s->El = p->num_local;
  s->act = p->act;
  s->weight = p->weight;
  s->blocked = p->weight_layout == MOE_LAYOUT_BLOCKED;
  s->S = S;
  return MOE_OK;
}

moe_status_t from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Device-memory layout of the moe_forward workspace.
struct ForwardLayout {
  size_t logits, idx, w, counts, offsets, sorted, pos, y, router, permute, ffn, total;
};

ForwardLayout forward_layout(const Shape& s) {
  ForwardLayout L{};
  size_t o = 0;
  auto take = [&o](size_t bytes) {
    const size_t at = o;
    o += moe::align_up(bytes);
    return at;
  };
  L.logits = take((size_t)s.T * s.E * sizeof(float));
  L.idx = take((size_t)s.S * sizeof(int32_t));
  L.w = take((size_t)s.S * sizeof(float));
  L.counts = take((size_t)s.El * sizeof(int32_t));
  L.offsets = take((size_t)(s.El + 1) * sizeof(int32_t));
  L.sorted = take((size_t)s.S * sizeof(int32_t));
  L.pos = take((size_t)s.S * sizeof(int32_t));
  L.y = take((size_t)s.S * s.d * moe::act_bytes(s));
  L.router = take(moe::route_ws_bytes(s));
  L.permute = take(moe::permute_ws_bytes(s));
  L.ffn = take(moe::ffn_ws_bytes(s));
  L.total = o;
  return L;
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_problem_t* p, int32_t call) {
  Shape s;
  if (check_problem(p, &s) != MOE_OK) return 0;
  switch (call) {
    case MOE_CALL_PERMUTE:
      return moe::permute_ws_bytes(s);
    case MOE_CALL_EXPERT_FFN:
      return moe::ffn_ws_bytes(s);
    case MOE_CALL_FORWARD:
      return forward_layout(s).total;
    case MOE_CALL_ROUTE:
      return moe::route_ws_bytes(s);
    default:
      return 0;
  }
}

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK:
      return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT:
      return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED:
      return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL:
      return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP:
      return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

moe_status_t moe_route(const moe_problem_t* p, const void* x, const void* w_router,
                       const float* router_bias, float* logits, int32_t* topk_idx,
                       float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  moe_status_t st = check_problem(p, &s);
  if (st != MOE_OK) return st;
  if (topk_idx == nullptr || topk_w == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (w_router != nullptr && x == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (logits == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (w_router != nullptr) {
    const size_t need = moe::route_ws_bytes(s);
    if (need > 0 && ws == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  }
  if (s.T == 0) return MOE_OK;
  const float* lin = w_router == nullptr ? logits : nullptr;
  return from_hip(moe::route(s, x, w_router, router_bias, lin, logits, topk_idx, topk_w, ws,
                             static_cast<hipStream_t>(stream)));
}

moe_status_t moe_permute(const moe_problem_t* p, const int32_t* topk_idx, int32_t* counts,
                         int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos, void* ws,
                         size_t ws_bytes, void* stream) {
  Shape s;
  moe_status_t st = check_problem(p, &s);
  if (st != MOE_OK) return st;
  if (topk_idx == nullptr || counts == nullptr || offsets == nullptr || sorted_slot == nullptr ||
      slot_pos == nullptr)
    return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = moe::permute_ws_bytes(s);
  if (need > 0 && ws == nullptr) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (s.T == 0) return MOE_OK;
  return from_hip(moe::permute(s, topk_idx, counts, offsets, sorted_slot, slot_pos, ws,
                               static_cast<hipStream_t>(stream)));
}

moe_status_t moe_expert_ffn(const moe_problem_t* p, const void* x, const int32_t* sorted_slot,
                            const int32_t* offsets, const void* w_gate, const void* w_up,
                            const void* w_down, const void* s_gate, const void* s_up,
                            const void* s_down, const float* topk_w, void* y, void* ws,
                            size_t ws_bytes, void* stream) {
  Shape s;
  moe_status_t st = check_problem(p, &s);
  if (st != MOE_OK) return st;
  if (x == nullptr || sorted_slot == nullptr || offsets == nullptr || w_gate == nullptr ||
      w_up == nullptr || w_down == nullptr || y == nullptr)
    return MOE_ERR_INVALID_ARGUMENT;
  if ((s.weight == MOE_FP8_E4M3 || s.weight == MOE_MXFP4) &&
      (s_gate == nullptr || s_up == nullptr || s_down == nullptr))
    return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = moe::ffn_ws_bytes(s);
  if (ws == nullptr || ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (s.T == 0) return MOE_OK;
  return from_hip(moe::expert_ffn(s, x, sorted_slot, offsets, w_gate, w_up, w_down, s_gate, s_up,
                                  s_down, topk_w, y, ws, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_combine(const moe_problem_t* p, const void* y, const int32_t* slot_pos,
                         const float* topk_w, void* out, void* stream) {
  Shape s;
  moe_status_t st = check_problem(p, &s);
  if (st != MOE_OK) return st;
  if (y == nullptr || slot_pos == nullptr || out == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (s.T == 0) return MOE_OK;
  return from_hip(moe::combine(s, y, slot_pos, topk_w, out, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_forward(const moe_problem_t* p, const moe_forward_args_t* a, void* ws,
                         size_t ws_bytes, void* stream) {
  Shape s;
  moe_status_t st = check_problem(p, &s);
  if (st != MOE_OK) return st;
  if (a == nullptr || a->x == nullptr || a->w_gate == nullptr || a->w_up == nullptr ||
      a->w_down == nullptr || a->out == nullptr)
    return MOE_ERR_INVALID_ARGUMENT;
  if (a->w_router == nullptr && a->logits == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if ((s.weight == MOE_FP8_E4M3 || s.weight == MOE_MXFP4) &&
      (a->s_gate == nullptr || a->s_up == nullptr || a->s_down == nullptr))
    return MOE_ERR_INVALID_ARGUMENT;
  const ForwardLayout L = forward_layout(s);
  if (ws == nullptr || ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (s.T == 0) return MOE_OK;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  unsigned char* base = static_cast<unsigned char*>(ws);
  auto pick = [base](void* user, size_t off) { return user ? user : static_cast<void*>(base + off); };
  float* logits = static_cast<float*>(pick(a->logits, L.logits));
  int32_t* idx = static_cast<int32_t*>(pick(a->topk_idx, L.idx));
  float* gw = static_cast<float*>(pick(a->topk_w, L.w));
  int32_t* counts = static_cast<int32_t*>(pick(a->counts, L.counts));
  int32_t* offsets = static_cast<int32_t*>(pick(a->offsets, L.offsets));
  int32_t* sorted = static_cast<int32_t*>(pick(a->sorted_slot, L.sorted));
  int32_t* pos = static_cast<int32_t*>(pick(a->slot_pos, L.pos));
  void* y = base + L.y;

  const float* lin = a->w_router == nullptr ? a->logits : nullptr;
  float* lout = a->w_router == nullptr ? nullptr : logits;
  hipEvent_t ev[MOE_FORWARD_EVENTS];
  if (a->events)
    for (int i = 0; i < MOE_FORWARD_EVENTS; ++i) ev[i] = static_cast<hipEvent_t>(a->events[i]);
  auto mark = [&](int i) { return a->events ? hipEventRecord(ev[i], strm) : hipSuccess; };
  hipError_t e = mark(0);
  if (e == hipSuccess)
    e = moe::route(s, a->x, a->w_router, a->router_bias, lin, lout, idx, gw, base + L.router,
                   strm);
  if (e == hipSuccess) e = mark(1);
  const moe::FfnSchedule sched = moe::ffn_schedule_view(s, base + L.ffn);
  bool sched_ready = false;
  if (e == hipSuccess)
    e = moe::permute(s, idx, counts, offsets, sorted, pos, base + L.permute, strm, &sched,
                     &sched_ready);
  if (e == hipSuccess) e = mark(2);
  if (e == hipSuccess)
    e = moe::expert_ffn(s, a->x, sorted, offsets, a->w_gate, a->w_up, a->w_down, a->s_gate,
                        a->s_up, a->s_down, gw, y, base + L.ffn, strm, sched_ready,
                        a->events ? ev + 3 : nullptr);
  if (e == hipSuccess) e = moe::combine(s, y, pos, nullptr, a->out, strm);
  if (e == hipSuccess) e = mark(6);
  return from_hip(e);
}

moe_status_t moe_pack_weights(const moe_problem_t* p, int32_t which, const void* src, void* dst,
                              void* stream) {
  Shape s;
  moe_status_t st = check_problem(p, &s);
  if (st != MOE_OK) return st;
  if (which != 0 && which != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (s.weight == MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (src == nullptr || dst == nullptr || src == dst) return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(moe::pack_weights(s, which, src, dst, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_eplb_plan(const int64_t* load, int32_t E, int32_t G, int32_t R,
                           int32_t* replicas, int32_t* phys_to_log, int32_t* log_to_phys,
                           double* rank_load) {
  if (load == nullptr || replicas == nullptr || phys_to_log == nullptr || log_to_phys == nullptr)
    return MOE_ERR_INVALID_ARGUMENT;
  if (E < 1 || G < 1 || R < 0 || (long long)R > (long long)E * (G - 1))
    return MOE_ERR_INVALID_ARGUMENT;
  if (((long long)E + R) % G != 0) return MOE_ERR_INVALID_ARGUMENT;
  if ((long long)E + R > moe::kMaxExperts) return MOE_ERR_UNSUPPORTED;
  for (int e = 0; e < E; ++e)
    if (load[e] < 0 || load[e] >= (1LL << 40)) return MOE_ERR_INVALID_ARGUMENT;
  try {
    moe::eplb_plan(load, E, G, R, replicas, phys_to_log, log_to_phys, rank_load);
  } catch (const std::bad_alloc&) {
    return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

moe_status_t moe_eplb_remap(int32_t T, int32_t k, int32_t E, int32_t G, const int32_t* topk_idx,
                            const int32_t* replicas, const int32_t* log_to_phys,
                            int32_t* topk_phys, void* stream) {
  if (T < 0 || k < 1 || E < 1 || G < 1) return MOE_ERR_INVALID_ARGUMENT;
  if ((long long)T * k >= (1LL << 31) || (long long)E * G >= (1LL << 31))
    return MOE_ERR_UNSUPPORTED;
  if (topk_idx == nullptr || replicas == nullptr || log_to_phys == nullptr || topk_phys == nullptr)
    return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  return from_hip(moe::eplb_remap(T, k, E, G, topk_idx, replicas, log_to_phys, topk_phys,
                                  static_cast<hipStream_t>(stream)));
}

}  // extern "C"
