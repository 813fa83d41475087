// Compute entry points: validate and plan on the host straight into a pinned
// staging buffer, then launch the kernels, which read the work list from that
// buffer over the bus (no separate upload, no device staging).
//
// Decode tokens go to MBGMV (page-gathered GEMV groups, shrink and expand in one
// launch), prefill segments to SGMV (MFMA tiles), following the split between the
// memory-bound decode phase and the parallel, compute-heavy prefill phase ("vLLM
// ile cikarimi olceklemek", the prefill / decode paragraphs).
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>

#include "guard.h"
#include "internal.h"

using namespace slora;

namespace {

// Pinned staging ring. The host writes a slot only after the kernels that read its
// previous plan have finished. Slots are guarded in groups of kGroup consecutive
// calls: one event, recorded after the group's last call, covers the group when all
// its calls went to one stream (an event per call puts a marker packet behind every
// launch, ~3 us of GPU time per decode call). A group whose calls went to more than
// one stream, or one of whose calls failed after taking its slot, is waited for with
// a device synchronization when its slots come round again.
//
// Every slot (kSlotBytes of pinned memory) and every group event is created with the
// ring, on a device's first compute call, so steady-state calls allocate nothing; a
// slot grows (a new pinned buffer) only for a plan larger than it has held before.
struct StagingSlot {
  void* host = nullptr;
  size_t cap = 0;
};
constexpr int kSlots = 16;
constexpr int kGroup = 8;
constexpr size_t kSlotBytes = size_t(1) << 20;
struct SlotGroup {
  hipEvent_t ev = nullptr;
  bool pending = false;    // ev recorded and not yet waited for
  bool unguarded = false;  // no single event covers the group's calls
  hipStream_t stream = nullptr;
};
struct Ring {
  StagingSlot slot[kSlots];
  SlotGroup grp[kSlots / kGroup];
  int next = 0;
  bool ready = false;
  // Fused decode launches wait across workgroups of one launch; two of them resident at
  // once could each hold slots the other's shrinks need, so the library orders them:
  // a fused launch on another stream than the previous one first waits for everything
  // queued on that stream so far (one event, recorded only when the stream changes).
  hipStream_t fused_stream = nullptr;
  hipEvent_t fused_ev = nullptr;
  // Allocation-free calls share the device's static scratch, so each of them is ordered
  // after the previous one the same way, whatever kernels it runs.
  hipStream_t shared_stream = nullptr;
  hipEvent_t shared_ev = nullptr;
};
std::mutex g_mu;  // guards the rings, the epoch map and the timing state
int32_t g_spin_limit = kDefaultSpinLimit;  // decode expand waves' bounded wait
std::map<int, Ring> g_rings;                 // per device
std::map<const void*, uint32_t> g_ws_tag;  // last tag a fused call used, per workspace
thread_local PlanScratch t_scratch;

struct SlotRef {
  Ring* ring = nullptr;
  int index = 0;
  void* host() const { return ring->slot[index].host; }
};

int grow_slot(StagingSlot& s, size_t n) {
  if (s.host) (void)hipHostFree(s.host);
  s.host = nullptr;
  s.cap = 0;
  size_t cap = kSlotBytes;
  while (cap < n) cap <<= 1;
  const hipError_t e = hipHostMalloc(&s.host, cap, hipHostMallocDefault);
  if (e != hipSuccess) {
    s.host = nullptr;
    return hip_fail(e, "staging: hipHostMalloc");
  }
  // touch every page now: the first write to each page of a new host mapping faults,
  // which would otherwise cost the first planned call of each slot ~20 us
  memset(s.host, 0, cap);
  s.cap = cap;
  return SLORA_OK;
}

// All slots and events of a device's ring, once.
int ring_init(Ring& ring) {
  if (ring.ready) return SLORA_OK;
  for (StagingSlot& s : ring.slot)
    if (!s.host) {
      const int rc = grow_slot(s, kSlotBytes);
      if (rc) return rc;
    }
  for (SlotGroup& g : ring.grp)
    if (!g.ev) {
      const hipError_t e = hipEventCreateWithFlags(&g.ev, hipEventDisableTiming);
      if (e != hipSuccess) { g.ev = nullptr; return hip_fail(e, "staging: hipEventCreate"); }
    }
  for (hipEvent_t* ev : {&ring.fused_ev, &ring.shared_ev})
    if (!*ev) {
      const hipError_t e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
      if (e != hipSuccess) { *ev = nullptr; return hip_fail(e, "hipEventCreate"); }
    }
  ring.ready = true;
  return SLORA_OK;
}

// may_grow = false (allocation-free calls): a plan larger than the slot is an error
// raised before the slot is taken.
int acquire_slot(size_t n, hipStream_t stream, bool may_grow, SlotRef* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  Ring& ring = g_rings[dev];
  int rc = ring_init(ring);
  if (rc) return rc;
  const int i = ring.next;
  if (!may_grow && ring.slot[i].cap < n)
    return fail(SLORA_E_INVALID, "work list of %zu bytes exceeds the %zu-byte staging slot an "
                "allocation-free call may use", n, ring.slot[i].cap);
  SlotGroup& grp = ring.grp[i / kGroup];
  if (i % kGroup == 0) {  // the group comes round again: its previous calls must be done
    if (grp.pending) {
      e = hipEventSynchronize(grp.ev);
      if (e != hipSuccess) return hip_fail(e, "staging: hipEventSynchronize");
      grp.pending = false;
    }
    if (grp.unguarded) {
      e = hipDeviceSynchronize();
      if (e != hipSuccess) return hip_fail(e, "staging: hipDeviceSynchronize");
      grp.unguarded = false;
    }
    grp.stream = stream;
  } else if (stream != grp.stream) {
    grp.unguarded = true;
  }
  ring.next = (i + 1) % kSlots;
  StagingSlot& s = ring.slot[i];
  if (s.cap < n) {
    rc = grow_slot(s, n);
    if (rc) {
      grp.unguarded = true;
      return rc;
    }
  }
  out->ring = &ring;
  out->index = i;
  return SLORA_OK;
}

// Orders work about to go to `s` after everything queued so far on `*last` (the stream
// of the previous launch of its kind on this device) when that is another stream.
int order_after(hipStream_t* last, hipEvent_t ev, hipStream_t s) {
  if (*last != nullptr && *last != s) {
    hipError_t e = hipEventRecord(ev, *last);
    if (e == hipSuccess) {
      e = hipStreamWaitEvent(s, ev, 0);
      if (e != hipSuccess) return hip_fail(e, "launch ordering: hipStreamWaitEvent");
    } else {  // that stream was destroyed since: wait for all work on the device instead
      (void)hipGetLastError();
      e = hipDeviceSynchronize();
      if (e != hipSuccess) return hip_fail(e, "launch ordering: hipDeviceSynchronize");
    }
  }
  *last = s;
  return SLORA_OK;
}
int order_fused(Ring& ring, hipStream_t s) { return order_after(&ring.fused_stream, ring.fused_ev, s); }

// After a call's launches (ok) or a failure after acquire_slot (!ok): the group's last
// call records the group's event.
int release_slot(const SlotRef& r, hipStream_t stream, bool ok) {
  SlotGroup& grp = r.ring->grp[r.index / kGroup];
  if (!ok) {
    grp.unguarded = true;
    return SLORA_OK;
  }
  if (r.index % kGroup == kGroup - 1 && !grp.unguarded) {
    const hipError_t e = hipEventRecord(grp.ev, stream);
    if (e != hipSuccess) {
      grp.unguarded = true;
      return hip_fail(e, "staging: hipEventRecord");
    }
    grp.pending = true;
  }
  return SLORA_OK;
}

// Kernel timing while enabled (benchmarks only): each timed launch is given an event
// pair that the launch itself records at the kernel's start and end.
struct TimedLaunch {
  int kernel;
  hipEvent_t start, stop;
};
bool g_timing_on = false;
std::vector<TimedLaunch> g_timed;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_spare_events;
constexpr size_t kTimingEvents = 512;  // event pairs created when timing is enabled

hipError_t new_event_pair(std::pair<hipEvent_t, hipEvent_t>* ev) {
  hipError_t e = hipEventCreate(&ev->first);
  if (e != hipSuccess) return e;
  e = hipEventCreate(&ev->second);
  if (e != hipSuccess) (void)hipEventDestroy(ev->first);
  return e;
}

template <typename F>
hipError_t timed_launch(int kernel, hipStream_t s, F&& launch) {
  if (!g_timing_on) return launch(LaunchEvents());
  std::pair<hipEvent_t, hipEvent_t> ev{nullptr, nullptr};
  if (!g_spare_events.empty()) {
    ev = g_spare_events.back();
    g_spare_events.pop_back();
  } else {  // more timed launches than were prepared for
    const hipError_t e = new_event_pair(&ev);
    if (e != hipSuccess) return e;
  }
  LaunchEvents le;
  le.start = ev.first;
  le.stop = ev.second;
  const hipError_t e = launch(le);
  if (e != hipSuccess) {
    g_spare_events.push_back(ev);
    return e;
  }
  g_timed.push_back({kernel, ev.first, ev.second});
  return hipSuccess;
}

enum Mode { kShrink = 1, kExpand = 2, kApply = 3 };

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

int launch_plan(const slora_lora* L, const slora_routing* R, const PlanView& pv, const void* x,
                float* v_out, const float* v_in, void* y, void* ws, int64_t ws_bytes,
                const WsLayout& lay, hipStream_t s, int mode, Ring* ring);

// shared: ws is the device's static scratch (allocation-free calls): the call is
// ordered after the previous such call and allocates nothing.
int run(const slora_lora* L, const slora_routing* R, const void* x, float* v_out,
        const float* v_in, void* y, void* ws, int64_t ws_bytes, void* stream, int mode,
        bool shared = false) {
  clear_error();
  PlanView pv;
  const int64_t bytes = plan_bytes(L, R, &t_scratch, &pv);
  if (bytes < 0) return (int)bytes;
  if ((mode & kShrink) && (!x || misaligned(x, 16)))
    return fail(SLORA_E_INVALID, "x must be a 16-byte aligned device pointer");
  if ((mode & kExpand) && (!y || misaligned(y, 16)))
    return fail(SLORA_E_INVALID, "y must be a 16-byte aligned device pointer");
  if (mode == kShrink && (!v_out || misaligned(v_out, 16)))
    return fail(SLORA_E_INVALID, "v must be a 16-byte aligned device pointer");
  if (mode == kExpand && (!v_in || misaligned(v_in, 16)))
    return fail(SLORA_E_INVALID, "v must be a 16-byte aligned device pointer");
  const WsLayout lay = ws_layout(L, R);
  if (!ws || misaligned(ws, 256)) return fail(SLORA_E_INVALID, "ws must be 256-byte aligned");
  if (ws_bytes < lay.total)
    return fail(SLORA_E_INVALID, "workspace of %lld bytes is smaller than the %lld needed",
                (long long)ws_bytes, (long long)lay.total);
  if (pv.n_routed == 0) return SLORA_OK;

  std::lock_guard<std::mutex> lk(g_mu);
  hipStream_t s = (hipStream_t)stream;
  SlotRef slot;
  int rc = acquire_slot((size_t)bytes, s, !shared, &slot);
  if (rc) return rc;
  if (shared) {
    rc = order_after(&slot.ring->shared_stream, slot.ring->shared_ev, s);
    if (rc) {
      (void)release_slot(slot, s, false);
      return rc;
    }
  }
  plan_write(L, R, &t_scratch, slot.host(), &pv);  // kernels read this host buffer directly
  rc = launch_plan(L, R, pv, x, v_out, v_in, y, ws, ws_bytes, lay, s, mode, slot.ring);
  const int rc2 = release_slot(slot, s, rc == SLORA_OK);
  return rc ? rc : rc2;
}

// The launches of one planned call (the work list is in a pinned staging slot).
int launch_plan(const slora_lora* L, const slora_routing* R, const PlanView& pv, const void* x,
                float* v_out, const float* v_in, void* y, void* ws, int64_t ws_bytes,
                const WsLayout& lay, hipStream_t s, int mode, Ring* ring) {
  uint8_t* wsb = (uint8_t*)ws;
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
  unsigned long long* err = (unsigned long long*)wsb;
  float* v = mode == kApply ? (float*)(wsb + lay.v_off) : (mode == kShrink ? v_out : nullptr);
  const float* vr = mode == kApply ? v : v_in;
  hipError_t e = hipSuccess;
  uint32_t tag = 0;
  bool mb_done = false;  // the decode groups ran in the segments' launch
  if (mode == kApply && (pv.n_mb || pv.n_sg)) {
    // A fresh tag per fused call on this workspace; before a tag could repeat, the
    // workspace past its header is cleared so no stale word can carry it (the header
    // keeps any give-up until slora_workspace_status reads it).
    uint32_t& last = g_ws_tag[ws];
    if (last == 0xFFFFFFFFu) {
      e = launch_zero(wsb + kHeaderBytes, (ws_bytes & ~(int64_t)255) - kHeaderBytes, s);
      if (e != hipSuccess) return hip_fail(e, "workspace clear");
      last = 0;
    }
    tag = ++last;
    const int rc = order_fused(*ring, s);  // both families' fused launches wait within a launch
    if (rc) return rc;
  }
  if (pv.n_sg) {
    // apply: k-range partials in the workspace; shrink / expand only: one range,
    // straight into / out of the caller's v
    int32_t v_stride = sg_v_stride(L->r_max);
    SgSplit sp = sg_split(L->d_in, pv.n_sg, sgmv_shrink_resident(pv.sg_max_rank, L->dtype));
    float* vpart = (float*)(wsb + lay.sg_off);
    if (mode != kApply) {
      sp.ksplit = 1;
      sp.kc = (L->d_in + 127) / 128 * 128;
      vpart = mode == kShrink ? v_out : const_cast<float*>(v_in);
      v_stride = L->r_max;
    }
    const int64_t stride = (int64_t)R->n_tokens * v_stride;
    // Tiles come in descending rank. Ranks above 64 need the widest kernels, which keep
    // fewer waves per SIMD. With enough tiles of both kinds, each kind gets its own
    // launch, timed as one interval (the first launch records the start, the second
    // the stop); with few tiles on one side the second launch costs more than the
    // narrower kernels save.
    int32_t hi = 0;
    while (hi < pv.n_sg && pv.sg[hi].rank > 64) ++hi;
    const bool split = hi >= kSgSplitTiles && pv.n_sg - hi >= kSgSplitTiles;
    auto by_rank = [&](const LaunchEvents& le, auto&& one) -> hipError_t {
      if (!split) return one(0, pv.n_sg, pv.sg_max_rank, le);
      LaunchEvents first = le, second = le;
      first.stop = nullptr;
      second.start = nullptr;
      const hipError_t e1 = one(0, hi, pv.sg_max_rank, first);
      if (e1 != hipSuccess) return e1;
      return one(hi, pv.n_sg - hi, pv.sg[hi].rank, second);
    };
    if (mode == kApply) {
      uint32_t* flags = (uint32_t*)(wsb + lay.flg_off);
      // decode groups too, and the segments in one launch: both families in that launch
      mb_done = pv.n_mb > 0 && !split;
      e = timed_launch(mb_done ? SLORA_K_MIXED_FUSED : SLORA_K_SGMV_FUSED, s, [&](const LaunchEvents& le) {
        if (mb_done)
          return launch_sgmv_fused(g, pv.tok, pv.sg, pv.n_sg, pv.sg_max_rank, sp.ksplit, sp.kc, x,
                                   vpart, v_stride, stride, flags, tag, g_spin_limit, err, y, s, le,
                                   pv.mb, pv.n_mb, pv.n_mb_shrink, pv.mb_max_tok, v);
        return by_rank(le, [&](int32_t t0, int32_t nt, int32_t mr, const LaunchEvents& l) {
          // up to 2 * ksplit flags per tile (tiles of rank above 64 are shrunk in two
          // row blocks), so each launch's flags start past every flag the tiles before
          // it could use: a launch must never find the call's tag left by another
          return launch_sgmv_fused(g, pv.tok, pv.sg + t0, nt, mr, sp.ksplit, sp.kc, x, vpart,
                                   v_stride, stride, flags + 2 * (int64_t)t0 * sp.ksplit, tag,
                                   g_spin_limit, err, y, s, l);
        });
      });
      if (e != hipSuccess) return hip_fail(e, "sgmv_fused launch");
    } else if (mode & kShrink) {
      e = timed_launch(SLORA_K_SGMV_SHRINK, s, [&](const LaunchEvents& le) {
        return by_rank(le, [&](int32_t t0, int32_t nt, int32_t mr, const LaunchEvents& l) {
          return launch_sgmv_shrink(g, pv.tok, pv.sg + t0, nt, mr, sp.ksplit, sp.kc, x, vpart,
                                    v_stride, stride, s, l);
        });
      });
      if (e != hipSuccess) return hip_fail(e, "sgmv_shrink launch");
    }
    if (mode == kExpand) {
      e = timed_launch(SLORA_K_SGMV_EXPAND, s, [&](const LaunchEvents& le) {
        return by_rank(le, [&](int32_t t0, int32_t nt, int32_t mr, const LaunchEvents& l) {
          return launch_sgmv_expand(g, pv.tok, pv.sg + t0, nt, mr, sp.ksplit, vpart, v_stride,
                                    stride, y, s, l);
        });
      });
      if (e != hipSuccess) return hip_fail(e, "sgmv_expand launch");
    }
  }
  if (pv.n_mb && !mb_done) {
    const bool has_expand = pv.n_mb > pv.n_mb_shrink;
    if (mode == kApply) {
      e = timed_launch(SLORA_K_MBGMV_FUSED, s, [&](const LaunchEvents& le) {
        return launch_mbgmv(g, pv.mb, pv.n_mb, pv.n_mb_shrink > 0, has_expand, pv.mb_max_tok, x,
                            v, y, tag, err, g_spin_limit, s, le);
      });
    } else if (mode == kShrink) {
      e = timed_launch(SLORA_K_MBGMV_SHRINK, s, [&](const LaunchEvents& le) {
        return launch_mbgmv(g, pv.mb, pv.n_mb_shrink, true, false, pv.mb_max_tok, x, v, nullptr, 0,
                            err, g_spin_limit, s, le);
      });
    } else {
      e = timed_launch(SLORA_K_MBGMV_EXPAND, s, [&](const LaunchEvents& le) {
        return launch_mbgmv(g, pv.mb + pv.n_mb_shrink, pv.n_mb - pv.n_mb_shrink, false, true,
                            pv.mb_max_tok, nullptr, const_cast<float*>(vr), y, 0, err, g_spin_limit,
                            s, le);
      });
    }
    if (e != hipSuccess) return hip_fail(e, "mbgmv launch");
  }
  return SLORA_OK;
}

// ---------------------------------------------------------------- several projections
// Projections that can share one plan: the same pool, geometry and adapters, with the
// same page-table layout (base, rank and scale arrays equal; each its own table).
int same_layout(const slora_lora* a, const slora_lora* b, int32_t p) {
  if (b->pool != a->pool || b->n_pages != a->n_pages || b->page_elems != a->page_elems ||
      b->dtype != a->dtype || b->d_in != a->d_in || b->d_out != a->d_out ||
      b->n_adapters != a->n_adapters || b->r_max != a->r_max ||
      b->page_table_len != a->page_table_len || (b->page_table_len > 0 && !b->page_table))
    return fail(SLORA_E_INVALID, "apply_multi: projection %d differs from projection 0 in pool, "
                "geometry or adapters", p);
  const size_t n = (size_t)std::max<int32_t>(a->n_adapters, 0);
  if (n && (!b->base || !b->rank || !b->scale || memcmp(a->base, b->base, n * sizeof *a->base) ||
            memcmp(a->rank, b->rank, n * sizeof *a->rank) || memcmp(a->scale, b->scale, n * sizeof *a->scale)))
    return fail(SLORA_E_INVALID, "apply_multi: projection %d's base / rank / scale differ from "
                "projection 0's", p);
  return SLORA_OK;
}

int64_t multi_region(const slora_lora* L, const slora_routing* R) {
  return (ws_layout(L, R).total + 255) / 256 * 256;
}

// The launches of a planned call over n projections; projection p's workspace region
// starts at ws + p * region.
int launch_multi(int32_t n, const slora_lora* Ls, const slora_routing* R, const PlanView& pv,
                 const void* const* xs, void* const* ys, void* ws, int64_t region,
                 const WsLayout& lay, hipStream_t s, Ring* ring) {
  const slora_lora* L = &Ls[0];
  uint8_t* wsb = (uint8_t*)ws;
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
  unsigned long long* err = (unsigned long long*)wsb;
  uint32_t& last = g_ws_tag[ws];
  if (last == 0xFFFFFFFFu) {  // as in launch_plan, over every projection's region
    const hipError_t e = launch_zero(wsb + kHeaderBytes, n * region - kHeaderBytes, s);
    if (e != hipSuccess) return hip_fail(e, "workspace clear");
    last = 0;
  }
  const uint32_t tag = ++last;
  int rc = order_fused(*ring, s);
  if (rc) return rc;
  const int32_t v_stride = sg_v_stride(L->r_max);
  const SgSplit sp = pv.n_sg ? sg_split(L->d_in, pv.n_sg, sgmv_shrink_resident(pv.sg_max_rank, L->dtype), n)
                             : SgSplit{};
  const int64_t part_stride = (int64_t)R->n_tokens * v_stride;
  ProjIO io[kMaxProj], io2[kMaxProj];
  int32_t hi = 0;
  while (hi < pv.n_sg && pv.sg[hi].rank > 64) ++hi;
  const bool split = hi >= kSgSplitTiles && pv.n_sg - hi >= kSgSplitTiles;
  for (int32_t p = 0; p < n; ++p) {
    uint8_t* r = wsb + p * region;
    io[p] = ProjIO{Ls[p].page_table, xs[p], ys[p], r + lay.v_off, (float*)(r + lay.sg_off),
                   (uint32_t*)(r + lay.flg_off)};
    io2[p] = io[p];
    io2[p].flags += 2 * (int64_t)hi * sp.ksplit;  // past every flag the wide tiles can use
  }
  const hipError_t e = timed_launch(SLORA_K_MULTI_FUSED, s, [&](const LaunchEvents& le) {
    if (!split)
      return launch_multi_fused(g, pv.tok, pv.sg, pv.n_sg, pv.sg_max_rank, sp.ksplit, sp.kc, v_stride,
                                part_stride, io, n, tag, g_spin_limit, err, s, le, pv.mb, pv.n_mb,
                                pv.n_mb_shrink, pv.mb_max_tok);
    // the rank classes in two launches (as launch_plan does), the decode groups with the
    // narrower one; timed as one interval
    LaunchEvents first = le, second = le;
    first.stop = nullptr;
    second.start = nullptr;
    const hipError_t e1 = launch_multi_fused(g, pv.tok, pv.sg, hi, pv.sg_max_rank, sp.ksplit, sp.kc,
                                             v_stride, part_stride, io, n, tag, g_spin_limit, err, s,
                                             first, nullptr, 0, 0, 0);
    if (e1 != hipSuccess) return e1;
    return launch_multi_fused(g, pv.tok, pv.sg + hi, pv.n_sg - hi, pv.sg[hi].rank, sp.ksplit, sp.kc,
                              v_stride, part_stride, io2, n, tag, g_spin_limit, err, s, second, pv.mb,
                              pv.n_mb, pv.n_mb_shrink, pv.mb_max_tok);
  });
  return e != hipSuccess ? hip_fail(e, "multi-projection launch") : SLORA_OK;
}

int run_multi(int32_t n, const slora_lora* Ls, const slora_routing* R, const void* const* xs,
              void* const* ys, void* ws, int64_t ws_bytes, void* stream) {
  clear_error();
  if (n < 1 || n > kMaxProj) return fail(SLORA_E_INVALID, "apply_multi: %d projections (1..%d)", n, kMaxProj);
  if (!Ls || !xs || !ys) return fail(SLORA_E_INVALID, "apply_multi: NULL argument");
  PlanView pv;
  const int64_t bytes = plan_bytes(&Ls[0], R, &t_scratch, &pv);
  if (bytes < 0) return (int)bytes;
  for (int32_t p = 1; p < n; ++p) {
    const int rc = same_layout(&Ls[0], &Ls[p], p);
    if (rc) return rc;
  }
  for (int32_t p = 0; p < n; ++p)
    if (!xs[p] || !ys[p] || misaligned(xs[p], 16) || misaligned(ys[p], 16))
      return fail(SLORA_E_INVALID, "apply_multi: x / y of projection %d must be 16-byte aligned device pointers", p);
  const WsLayout lay = ws_layout(&Ls[0], R);
  const int64_t region = multi_region(&Ls[0], R);
  if (!ws || misaligned(ws, 256)) return fail(SLORA_E_INVALID, "ws must be 256-byte aligned");
  if (ws_bytes < n * region)
    return fail(SLORA_E_INVALID, "workspace of %lld bytes is smaller than the %lld needed",
                (long long)ws_bytes, (long long)(n * region));
  if (pv.n_routed == 0) return SLORA_OK;
  std::lock_guard<std::mutex> lk(g_mu);
  hipStream_t s = (hipStream_t)stream;
  SlotRef slot;
  int rc = acquire_slot((size_t)bytes, s, true, &slot);
  if (rc) return rc;
  plan_write(&Ls[0], R, &t_scratch, slot.host(), &pv);
  rc = launch_multi(n, Ls, R, pv, xs, ys, ws, region, lay, s, slot.ring);
  const int rc2 = release_slot(slot, s, rc == SLORA_OK);
  return rc ? rc : rc2;
}

}  // namespace

namespace {

// ---------------------------------------------------------------- gathered baseline
// A synthetic call over the rank-padded copies: adapter q of the copy is request q.
struct Gathered {
  std::vector<int64_t> base;
  std::vector<int32_t> rank, seg_off, seg_ad;
  std::vector<float> scale;
  std::vector<GatherReq> reqs;
  slora_lora L{};
  slora_routing R{};
  int32_t r_pad = 0;
  int64_t copy_pages = 0;
  int64_t pages_off = 0, pt_off = 0, sg_off = 0, total = 0;  // workspace layout
};
thread_local Gathered t_gathered;

int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

// Validates the call like slora_apply, then lays out requests, copies and workspace.
int gathered_build(const slora_lora* L, const slora_routing* R, Gathered* g) {
  PlanView pv;
  const int64_t bytes = plan_bytes(L, R, &t_scratch, &pv);  // the same validation
  if (bytes < 0) return (int)bytes;
  const int32_t cA = (L->d_in + L->page_elems - 1) / L->page_elems;
  const int32_t cB = (L->d_out + L->page_elems - 1) / L->page_elems;
  g->base.clear();
  g->rank.clear();
  g->scale.clear();
  g->reqs.clear();
  g->seg_off.assign(1, 0);
  g->seg_ad.clear();
  g->r_pad = 0;
  auto add = [&](int32_t a, int32_t len) {  // one synthetic segment of len tokens
    const bool lora = a >= 0 && L->rank[a] > 0;
    g->seg_ad.push_back(lora ? (int32_t)g->reqs.size() : -1);
    g->seg_off.push_back(g->seg_off.back() + len);
    if (lora) {
      g->reqs.push_back(GatherReq{(int32_t)L->base[a], L->rank[a]});
      g->scale.push_back(L->scale[a]);
      g->r_pad = std::max(g->r_pad, L->rank[a]);
    }
  };
  const int32_t S = R->n_segments;
  for (int32_t s = 0; s < S; ++s) add(R->seg_adapter[s], R->seg_offsets[s + 1] - R->seg_offsets[s]);
  const int32_t seg_end = S > 0 ? R->seg_offsets[S] : 0;
  for (int32_t t = seg_end; t < R->n_tokens; ++t) add(R->token_adapter[t - seg_end], 1);
  const int32_t n_req = (int32_t)g->reqs.size();
  const int32_t r_pad = std::max(g->r_pad, 1);
  g->copy_pages = (int64_t)n_req * r_pad * (cA + cB);
  if (g->copy_pages > INT32_MAX)
    return fail(SLORA_E_INVALID, "gathered: %lld copy pages", (long long)g->copy_pages);
  for (int32_t q = 0; q < n_req; ++q) {
    g->base.push_back((int64_t)q * r_pad * (cA + cB));
    g->rank.push_back(r_pad);
  }
  g->L = *L;
  g->L.n_pages = std::max<int64_t>(g->copy_pages, 1);
  g->L.page_table_len = g->copy_pages;
  g->L.n_adapters = n_req;
  g->L.base = g->base.data();
  g->L.rank = g->rank.data();
  g->L.scale = g->scale.data();
  g->L.r_max = r_pad;
  g->R.n_tokens = R->n_tokens;
  g->R.n_segments = (int32_t)g->seg_ad.size();
  g->R.seg_offsets = g->seg_off.data();
  g->R.seg_adapter = g->seg_ad.data();
  g->R.token_adapter = nullptr;
  g->R.policy = SLORA_POLICY_SGMV;
  // The apply's own workspace comes first, so its header (the give-up word) is the
  // header of the caller's workspace; the copies and their page table follow it.
  g->sg_off = 0;
  g->pages_off = align256(ws_layout(&g->L, &g->R).total);
  g->pt_off = g->pages_off + align256(g->copy_pages * L->page_elems * 2);
  g->total = g->pt_off + align256(g->copy_pages * 4);
  return SLORA_OK;
}

int run_gathered(const slora_lora* L, const slora_routing* R, const void* x, void* y, void* ws,
                 int64_t ws_bytes, void* stream) {
  clear_error();
  Gathered& g = t_gathered;
  int rc = gathered_build(L, R, &g);
  if (rc) return rc;
  if (!x || !y || misaligned(x, 16) || misaligned(y, 16))
    return fail(SLORA_E_INVALID, "x / y must be 16-byte aligned device pointers");
  if (!ws || misaligned(ws, 256)) return fail(SLORA_E_INVALID, "ws must be 256-byte aligned");
  if (ws_bytes < g.total)
    return fail(SLORA_E_INVALID, "workspace of %lld bytes is smaller than the %lld needed",
                (long long)ws_bytes, (long long)g.total);
  if (g.reqs.empty()) return SLORA_OK;
  uint8_t* wsb = (uint8_t*)ws;
  g.L.pool = wsb + g.pages_off;
  g.L.page_table = (const int32_t*)(wsb + g.pt_off);
  PlanView pv;
  const int64_t plan = plan_bytes(&g.L, &g.R, &t_scratch, &pv);
  if (plan < 0) return (int)plan;
  const int64_t req_bytes = align256((int64_t)g.reqs.size() * (int64_t)sizeof(GatherReq));

  std::lock_guard<std::mutex> lk(g_mu);
  hipStream_t s = (hipStream_t)stream;
  SlotRef slot;
  rc = acquire_slot((size_t)(req_bytes + plan), s, true, &slot);
  if (rc) return rc;
  uint8_t* host = (uint8_t*)slot.host();
  memcpy(host, g.reqs.data(), g.reqs.size() * sizeof(GatherReq));
  plan_write(&g.L, &g.R, &t_scratch, host + req_bytes, &pv);
  Geom src;
  src.pool = (const uint16_t*)L->pool;
  src.n_pages = L->n_pages;
  src.P = L->page_elems;
  src.dtype = L->dtype;
  src.d_in = L->d_in;
  src.d_out = L->d_out;
  src.cA = (L->d_in + src.P - 1) / src.P;
  src.cB = (L->d_out + src.P - 1) / src.P;
  src.pt = L->page_table;
  src.r_max = L->r_max;
  const hipError_t e = timed_launch(SLORA_K_GATHER, s, [&](const LaunchEvents& le) {
    return launch_gather(src, (const GatherReq*)host, (int32_t)g.reqs.size(), std::max(g.r_pad, 1),
                         wsb + g.pages_off, (int32_t*)(wsb + g.pt_off), s, le);
  });
  if (e != hipSuccess) rc = hip_fail(e, "gather launch");
  if (!rc)
    rc = launch_plan(&g.L, &g.R, pv, x, nullptr, nullptr, y, wsb + g.sg_off, g.pages_off - g.sg_off,
                     ws_layout(&g.L, &g.R), s, kApply, slot.ring);
  const int rc2 = release_slot(slot, s, rc == SLORA_OK);
  return rc ? rc : rc2;
}

}  // namespace

namespace slora {
hipError_t timed_fetch(const FetchPage* pages, int64_t n, uint16_t* pool, int32_t page_elems,
                       hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  return timed_launch(SLORA_K_FETCH, s, [&](const LaunchEvents& le) {
    return launch_fetch(pages, n, pool, page_elems, s, le);
  });
}

int apply_shared(const slora_lora* L, const slora_routing* R, const void* x, void* y, void* ws,
                 int64_t ws_bytes, void* stream) {
  return run(L, R, x, nullptr, nullptr, y, ws, ws_bytes, stream, kApply, true);
}
}  // namespace slora

extern "C" {

static int impl_slora_timing_enable(int32_t on) {
  clear_error();
  std::lock_guard<std::mutex> lk(g_mu);
  // the event pairs timed launches take are created here, not inside compute calls
  while (on && g_spare_events.size() + g_timed.size() < kTimingEvents) {
    std::pair<hipEvent_t, hipEvent_t> ev;
    const hipError_t e = new_event_pair(&ev);
    if (e != hipSuccess) return hip_fail(e, "timing_enable: hipEventCreate");
    g_spare_events.push_back(ev);
  }
  g_timing_on = on != 0;
  return SLORA_OK;
}

static int impl_slora_set_wait_limit(int32_t polls) {
  clear_error();
  if (polls < 0) return fail(SLORA_E_INVALID, "set_wait_limit: polls %d < 0", polls);
  std::lock_guard<std::mutex> lk(g_mu);
  g_spin_limit = polls == 0 ? kDefaultSpinLimit : polls;
  return SLORA_OK;
}

static int impl_slora_timing_read(int32_t n_kernels, int64_t* launches, double* total_ms) {
  clear_error();
  if (n_kernels < 0 || n_kernels > SLORA_K_COUNT || (n_kernels > 0 && (!launches || !total_ms)))
    return fail(SLORA_E_INVALID, "timing_read: bad arguments");
  std::lock_guard<std::mutex> lk(g_mu);
  for (int32_t k = 0; k < n_kernels; ++k) { launches[k] = 0; total_ms[k] = 0.0; }
  int rc = SLORA_OK;
  for (auto& t : g_timed) {
    hipError_t e = hipEventSynchronize(t.stop);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.start, t.stop);
    if (e != hipSuccess && rc == SLORA_OK) rc = hip_fail(e, "timing_read");
    if (t.kernel < n_kernels) {
      launches[t.kernel] += 1;
      total_ms[t.kernel] += ms;
    }
    g_spare_events.push_back({t.start, t.stop});
  }
  g_timed.clear();
  return rc;
}

static int impl_slora_timing_read_all(int64_t cap, int32_t* kernel, double* ms, int64_t* n) {
  clear_error();
  if (!n || cap < 0 || (cap > 0 && (!kernel || !ms)))
    return fail(SLORA_E_INVALID, "timing_read_all: bad arguments");
  std::lock_guard<std::mutex> lk(g_mu);
  *n = (int64_t)g_timed.size();
  if (*n > cap)
    return fail(SLORA_E_INVALID, "timing_read_all: %lld launches recorded, room for %lld",
                (long long)*n, (long long)cap);
  int rc = SLORA_OK;
  int64_t i = 0;
  for (auto& t : g_timed) {
    hipError_t e = hipEventSynchronize(t.stop);
    float f = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&f, t.start, t.stop);
    if (e != hipSuccess && rc == SLORA_OK) rc = hip_fail(e, "timing_read_all");
    kernel[i] = t.kernel;
    ms[i] = f;
    ++i;
    g_spare_events.push_back({t.start, t.stop});
  }
  g_timed.clear();
  return rc;
}

static int impl_slora_workspace_size(const slora_lora* lora, const slora_routing* routing, int64_t* bytes) {
  clear_error();
  if (!lora || !routing || !bytes) return fail(SLORA_E_INVALID, "workspace_size: NULL argument");
  *bytes = ws_layout(lora, routing).total;
  return SLORA_OK;
}

static int impl_slora_workspace_size_multi(int32_t n, const slora_lora* loras,
                                           const slora_routing* routing, int64_t* bytes) {
  clear_error();
  if (!loras || !routing || !bytes) return fail(SLORA_E_INVALID, "workspace_size_multi: NULL argument");
  if (n < 1 || n > kMaxProj) return fail(SLORA_E_INVALID, "workspace_size_multi: %d projections (1..%d)", n, kMaxProj);
  *bytes = n * multi_region(&loras[0], routing);
  return SLORA_OK;
}

static int impl_slora_workspace_status(void* ws, void* stream, int32_t* status) {
  clear_error();
  if (!status) return fail(SLORA_E_INVALID, "workspace_status: status is NULL");
  if (!ws) {  // the current device's static scratch (allocation-free calls)
    const int rc = shared_scratch(&ws, nullptr);
    if (rc) return rc;
    if (!ws) {  // no allocation-free call has set it up on this device: nothing to report
      *status = 0;
      return SLORA_OK;
    }
  }
  unsigned long long flag = 0;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(&flag, ws, sizeof flag, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess && flag != 0) {  // report once: the word is cleared for the next calls
    e = hipMemsetAsync(ws, 0, sizeof flag, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
  }
  if (e != hipSuccess) return hip_fail(e, "workspace_status");
  *status = flag != 0 ? 1 : 0;
  return SLORA_OK;
}

static int impl_slora_shrink(const slora_lora* lora, const slora_routing* routing, const void* x, float* v,
                 void* ws, int64_t ws_bytes, void* stream) {
  return run(lora, routing, x, v, nullptr, nullptr, ws, ws_bytes, stream, kShrink);
}

static int impl_slora_expand(const slora_lora* lora, const slora_routing* routing, const float* v, void* y,
                 void* ws, int64_t ws_bytes, void* stream) {
  return run(lora, routing, nullptr, nullptr, v, y, ws, ws_bytes, stream, kExpand);
}

static int impl_slora_apply(const slora_lora* lora, const slora_routing* routing, const void* x, void* y,
                void* ws, int64_t ws_bytes, void* stream) {
  return run(lora, routing, x, nullptr, nullptr, y, ws, ws_bytes, stream, kApply);
}

static int impl_slora_plan_inspect(const slora_lora* lora, const slora_routing* routing, int32_t* n_groups,
                       int32_t* info, int32_t info_cap, int32_t* tokens) {
  clear_error();
  if (!n_groups) return fail(SLORA_E_INVALID, "plan_inspect: n_groups is NULL");
  PlanScratch sc;
  PlanView pv;
  const int64_t bytes = plan_bytes(lora, routing, &sc, &pv);
  if (bytes < 0) return (int)bytes;
  std::vector<uint8_t> buf((size_t)bytes + 64);
  void* aligned = (void*)(((uintptr_t)buf.data() + 63) & ~(uintptr_t)63);
  plan_write(lora, routing, &sc, aligned, &pv);
  const int32_t n = pv.n_groups + pv.n_sg;
  *n_groups = n;
  if (n > info_cap || !info) return fail(SLORA_E_INVALID, "plan_inspect: %d groups > cap %d", n, info_cap);
  // MBGMV groups from their first shrink item each, in dispatch order
  int32_t at = 0, slot = 0;
  for (int32_t i = 0; i < pv.n_mb_shrink; ++i) {
    const MbItem& it = pv.mb[i];
    if (it.part != 0) continue;
    info[5 * at + 0] = 0;
    info[5 * at + 1] = slot;
    info[5 * at + 2] = it.n_tok();
    info[5 * at + 3] = it.pt_base;
    info[5 * at + 4] = it.rank;
    if (tokens)
      for (int32_t t = 0; t < it.n_tok(); ++t) tokens[slot + t] = it.tok[t];
    slot += it.n_tok();
    ++at;
  }
  for (int32_t i = 0; i < pv.n_sg; ++i) {
    const SgTile& t = pv.sg[i];
    info[5 * at + 0] = 1;
    info[5 * at + 1] = slot;
    info[5 * at + 2] = t.n_tok;
    info[5 * at + 3] = t.pt_base;
    info[5 * at + 4] = t.rank;
    if (tokens)
      for (int32_t q = 0; q < t.n_tok; ++q)
        tokens[slot + q] = t.first_tok >= 0 ? t.first_tok + q : pv.tok[t.tok_begin + q];
    slot += t.n_tok;
    ++at;
  }
  return SLORA_OK;
}

}  // extern "C"

// Entry points: every C++ exception (host memory exhausted included) becomes an
// error code here, so none crosses the C ABI.
extern "C" {

int slora_timing_enable(int32_t on) {
  return slora::guarded(__func__, [&] { return impl_slora_timing_enable(on); });
}

int slora_timing_read(int32_t n_kernels, int64_t* launches, double* total_ms) {
  return slora::guarded(__func__, [&] { return impl_slora_timing_read(n_kernels, launches, total_ms); });
}

int slora_workspace_size(const slora_lora* lora, const slora_routing* routing, int64_t* bytes) {
  return slora::guarded(__func__, [&] { return impl_slora_workspace_size(lora, routing, bytes); });
}

int slora_workspace_status(void* ws, void* stream, int32_t* status) {
  return slora::guarded(__func__, [&] { return impl_slora_workspace_status(ws, stream, status); });
}

int slora_gathered_workspace_size(const slora_lora* lora, const slora_routing* routing, int64_t* bytes) {
  return slora::guarded(__func__, [&] {
    clear_error();
    if (!bytes) return fail(SLORA_E_INVALID, "gathered_workspace_size: bytes is NULL");
    const int rc = gathered_build(lora, routing, &t_gathered);
    if (rc) return rc;
    *bytes = t_gathered.total;
    return SLORA_OK;
  });
}

int slora_apply_gathered(const slora_lora* lora, const slora_routing* routing, const void* x, void* y,
                         void* ws, int64_t ws_bytes, void* stream) {
  return slora::guarded(__func__, [&] { return run_gathered(lora, routing, x, y, ws, ws_bytes, stream); });
}

int slora_set_wait_limit(int32_t polls) {
  return slora::guarded(__func__, [&] { return impl_slora_set_wait_limit(polls); });
}

int slora_timing_read_all(int64_t cap, int32_t* kernel, double* ms, int64_t* n) {
  return slora::guarded(__func__, [&] { return impl_slora_timing_read_all(cap, kernel, ms, n); });
}

int slora_shrink(const slora_lora* lora, const slora_routing* routing, const void* x, float* v,
                 void* ws, int64_t ws_bytes, void* stream) {
  return slora::guarded(__func__, [&] { return impl_slora_shrink(lora, routing, x, v, ws, ws_bytes, stream); });
}

int slora_expand(const slora_lora* lora, const slora_routing* routing, const float* v, void* y,
                 void* ws, int64_t ws_bytes, void* stream) {
  return slora::guarded(__func__, [&] { return impl_slora_expand(lora, routing, v, y, ws, ws_bytes, stream); });
}

int slora_apply(const slora_lora* lora, const slora_routing* routing, const void* x, void* y,
                void* ws, int64_t ws_bytes, void* stream) {
  return slora::guarded(__func__, [&] { return impl_slora_apply(lora, routing, x, y, ws, ws_bytes, stream); });
}

int slora_workspace_size_multi(int32_t n_proj, const slora_lora* loras, const slora_routing* routing,
                               int64_t* bytes) {
  return slora::guarded(__func__, [&] { return impl_slora_workspace_size_multi(n_proj, loras, routing, bytes); });
}

int slora_apply_multi(int32_t n_proj, const slora_lora* loras, const slora_routing* routing,
                      const void* const* xs, void* const* ys, void* ws, int64_t ws_bytes,
                      void* stream) {
  return slora::guarded(__func__, [&] { return run_multi(n_proj, loras, routing, xs, ys, ws, ws_bytes, stream); });
}

int slora_plan_inspect(const slora_lora* lora, const slora_routing* routing, int32_t* n_groups,
                       int32_t* info, int32_t info_cap, int32_t* tokens) {
  return slora::guarded(__func__, [&] { return impl_slora_plan_inspect(lora, routing, n_groups, info, info_cap, tokens); });
}

}  // extern "C"
