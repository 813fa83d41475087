// Compute entry points: validate, plan on the host, upload the work list into the
// caller's workspace through a pinned staging ring, launch the kernels.
//
// Decode tokens go to MBGMV (page-gathered GEMV groups), prefill segments to SGMV
// (MFMA tiles), per the split between the memory-bound decode phase and the
// parallel, compute-heavy prefill phase ("vLLM ile cikarimi olceklemek", the
// prefill / decode paragraphs).
#include <string.h>

#include <map>
#include <mutex>

#include "internal.h"

using namespace slora;

namespace {

// Pinned staging ring for work lists. A slot is reused only after the copy that
// last read it has completed (its event), so the host never overwrites a buffer a
// pending hipMemcpyAsync still reads.
struct StagingSlot {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};
constexpr int kSlots = 8;
struct Ring {
  StagingSlot slot[kSlots];
  int next = 0;
};
std::mutex g_ring_mu;
std::map<int, Ring> g_rings;  // per device

int upload(const void* src, size_t n, void* dst, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_ring_mu);
  Ring& ring = g_rings[dev];
  StagingSlot& s = ring.slot[ring.next];
  ring.next = (ring.next + 1) % kSlots;
  if (s.pending) {
    e = hipEventSynchronize(s.ev);
    if (e != hipSuccess) return hip_fail(e, "staging: hipEventSynchronize");
    s.pending = false;
  }
  if (!s.ev) {
    e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming);
    if (e != hipSuccess) { s.ev = nullptr; return hip_fail(e, "staging: hipEventCreate"); }
  }
  if (s.cap < n) {
    if (s.host) (void)hipHostFree(s.host);
    s.host = nullptr;
    s.cap = 0;
    size_t cap = 1 << 16;
    while (cap < n) cap <<= 1;
    e = hipHostMalloc(&s.host, cap, hipHostMallocDefault);
    if (e != hipSuccess) { s.host = nullptr; return hip_fail(e, "staging: hipHostMalloc"); }
    s.cap = cap;
  }
  memcpy(s.host, src, n);
  e = hipMemcpyAsync(dst, s.host, n, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "staging: hipMemcpyAsync");
  e = hipEventRecord(s.ev, stream);
  if (e != hipSuccess) return hip_fail(e, "staging: hipEventRecord");
  s.pending = true;
  return SLORA_OK;
}

enum Mode { kShrink = 1, kExpand = 2, kApply = 3 };

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

int run(const slora_lora* L, const slora_routing* R, const void* x, float* v_out,
        const float* v_in, void* y, void* ws, int64_t ws_bytes, void* stream, int mode) {
  clear_error();
  Plan plan;
  int rc = validate_and_plan(L, R, &plan);
  if (rc) return rc;
  if ((mode & kShrink) && (!x || misaligned(x, 16)))
    return fail(SLORA_E_INVALID, "x must be a 16-byte aligned device pointer");
  if ((mode & kExpand) && (!y || misaligned(y, 16)))
    return fail(SLORA_E_INVALID, "y must be a 16-byte aligned device pointer");
  if (mode == kShrink && (!v_out || misaligned(v_out, 16)))
    return fail(SLORA_E_INVALID, "v must be a 16-byte aligned device pointer");
  if (mode == kExpand && (!v_in || misaligned(v_in, 16)))
    return fail(SLORA_E_INVALID, "v must be a 16-byte aligned device pointer");
  const PlanLayout lay = layout_plan(L, R, plan);
  if (!ws || misaligned(ws, 256)) return fail(SLORA_E_INVALID, "ws must be 256-byte aligned");
  if (ws_bytes < lay.total)
    return fail(SLORA_E_INVALID, "workspace of %lld bytes is smaller than the %lld needed",
                (long long)ws_bytes, (long long)lay.total);
  if (plan.n_routed == 0) return SLORA_OK;

  std::vector<uint8_t> blob((size_t)lay.blob_bytes, 0);
  auto put = [&](int64_t off, const void* src, size_t n) {
    if (n) memcpy(blob.data() + (off - lay.blob_off), src, n);
  };
  put(lay.tok_off, plan.tok.data(), plan.tok.size() * 4);
  put(lay.mbg_off, plan.mb_groups.data(), plan.mb_groups.size() * sizeof(GroupDesc));
  put(lay.mbs_off, plan.mb_shrink.data(), plan.mb_shrink.size() * sizeof(Item));
  put(lay.sgt_off, plan.sg_tiles.data(), plan.sg_tiles.size() * sizeof(GroupDesc));
  hipStream_t s = (hipStream_t)stream;
  uint8_t* wsb = (uint8_t*)ws;
  rc = upload(blob.data(), blob.size(), wsb + lay.blob_off, s);
  if (rc) return rc;

  Geom g;
  g.pool = (const uint16_t*)L->pool;
  g.n_pages = L->n_pages;
  g.P = L->page_elems;
  g.dtype = L->dtype;
  g.d_in = L->d_in;
  g.d_out = L->d_out;
  g.cA = (L->d_in + g.P - 1) / g.P;
  g.cB = (L->d_out + g.P - 1) / g.P;
  g.pt = L->page_table;
  g.r_max = L->r_max;
  const int32_t* tok = (const int32_t*)(wsb + lay.tok_off);
  const GroupDesc* mbg = (const GroupDesc*)(wsb + lay.mbg_off);
  const Item* mbs = (const Item*)(wsb + lay.mbs_off);
  const GroupDesc* sgt = (const GroupDesc*)(wsb + lay.sgt_off);
  float* v = mode == kApply ? (float*)(wsb + lay.v_off) : (mode == kShrink ? v_out : nullptr);
  const float* vr = mode == kApply ? v : v_in;
  const int32_t n_mbg = (int32_t)plan.mb_groups.size(), n_mbs = (int32_t)plan.mb_shrink.size();
  const int32_t n_sgt = (int32_t)plan.sg_tiles.size();
  hipError_t e;
  if (mode & kShrink) {
    if (n_sgt) {
      e = launch_sgmv_shrink(g, tok, sgt, n_sgt, x, v, s);
      if (e != hipSuccess) return hip_fail(e, "sgmv_shrink launch");
    }
    if (n_mbs) {
      e = launch_mbgmv_shrink(g, tok, mbg, mbs, n_mbs, x, v, s);
      if (e != hipSuccess) return hip_fail(e, "mbgmv_shrink launch");
    }
  }
  if (mode & kExpand) {
    if (n_sgt) {
      e = launch_sgmv_expand(g, tok, sgt, n_sgt, vr, y, s);
      if (e != hipSuccess) return hip_fail(e, "sgmv_expand launch");
    }
    if (n_mbg) {
      e = launch_mbgmv_expand(g, tok, mbg, n_mbg, vr, y, s);
      if (e != hipSuccess) return hip_fail(e, "mbgmv_expand launch");
    }
  }
  return SLORA_OK;
}

}  // namespace

extern "C" {

int slora_workspace_size(const slora_lora* lora, const slora_routing* routing, int64_t* bytes) {
  clear_error();
  if (!lora || !routing || !bytes) return fail(SLORA_E_INVALID, "workspace_size: NULL argument");
  *bytes = workspace_bound(lora, routing);
  return SLORA_OK;
}

int slora_shrink(const slora_lora* lora, const slora_routing* routing, const void* x, float* v,
                 void* ws, int64_t ws_bytes, void* stream) {
  return run(lora, routing, x, v, nullptr, nullptr, ws, ws_bytes, stream, kShrink);
}

int slora_expand(const slora_lora* lora, const slora_routing* routing, const float* v, void* y,
                 void* ws, int64_t ws_bytes, void* stream) {
  return run(lora, routing, nullptr, nullptr, v, y, ws, ws_bytes, stream, kExpand);
}

int slora_plan_inspect(const slora_lora* lora, const slora_routing* routing, int32_t* n_groups,
                       int32_t* info, int32_t info_cap, int32_t* tokens) {
  clear_error();
  if (!n_groups) return fail(SLORA_E_INVALID, "plan_inspect: n_groups is NULL");
  Plan plan;
  int rc = validate_and_plan(lora, routing, &plan);
  if (rc) return rc;
  const int32_t n = (int32_t)(plan.mb_groups.size() + plan.sg_tiles.size());
  *n_groups = n;
  if (n > info_cap || !info) return fail(SLORA_E_INVALID, "plan_inspect: %d groups > cap %d", n, info_cap);
  int32_t at = 0;
  for (int fam = 0; fam < 2; ++fam) {
    const std::vector<GroupDesc>& gs = fam == 0 ? plan.mb_groups : plan.sg_tiles;
    for (const GroupDesc& g : gs) {
      info[5 * at + 0] = fam;
      info[5 * at + 1] = g.tok_begin;
      info[5 * at + 2] = g.n_tok;
      info[5 * at + 3] = g.pt_base;
      info[5 * at + 4] = g.rank;
      ++at;
    }
  }
  if (tokens && !plan.tok.empty()) memcpy(tokens, plan.tok.data(), plan.tok.size() * 4);
  return SLORA_OK;
}

int slora_apply(const slora_lora* lora, const slora_routing* routing, const void* x, void* y,
                void* ws, int64_t ws_bytes, void* stream) {
  return run(lora, routing, x, nullptr, nullptr, y, ws, ws_bytes, stream, kApply);
}

}  // extern "C"
