// Routing validation and work-list planning (host, integer only).
//
// Every token picks its adapter: by segment for a request's contiguous prefill
// tokens, or by its own id for decode tokens ("Makale Bulteni - S-LoRA", section
// "Iddia ve Gerceklik": each token of a batch may use a different adapter; the
// S-LoRA overview, section "2. Heterogeneous Batching": adapters of different
// ranks are batched together). The planner groups tokens that share an adapter so
// that each group reads the adapter's pages once:
//   * MBGMV groups: decode tokens bucketed by adapter (stable), split evenly into
//     groups of at most kMbGroup tokens;
//   * SGMV tiles: a segment (or a bucket of ids) split evenly into tiles of at
//     most kSgTile tokens.
// Groups are ordered by descending rank so that the costliest work items are
// dispatched first. The order only decides scheduling: every token's result is
// computed by the same fixed sequence of operations wherever it lands.
#include <algorithm>
#include <cmath>

#include "internal.h"

namespace slora {

namespace {

int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

struct Pair {
  int32_t adapter;
  int32_t token;
};

// Append groups of at most `cap` tokens, sizes as even as possible, for one run
// of tokens that share `adapter`.
void split_run(const int32_t* toks, int32_t n, int32_t adapter, int32_t cap,
               const slora_lora* L, std::vector<std::pair<GroupDesc, std::vector<int32_t>>>* out) {
  if (n <= 0) return;
  const int32_t g = (n + cap - 1) / cap;
  const int32_t base = n / g, extra = n % g;
  int32_t at = 0;
  for (int32_t i = 0; i < g; ++i) {
    const int32_t m = base + (i < extra ? 1 : 0);
    GroupDesc d{};
    d.n_tok = m;
    d.pt_base = (int32_t)L->base[adapter];
    d.rank = L->rank[adapter];
    d.scale = L->scale[adapter];
    out->emplace_back(d, std::vector<int32_t>(toks + at, toks + at + m));
    at += m;
  }
}

}  // namespace

int validate_and_plan(const slora_lora* L, const slora_routing* R, Plan* plan) {
  if (!L || !R) return fail(SLORA_E_INVALID, "lora / routing is NULL");
  if (!L->pool || (reinterpret_cast<uintptr_t>(L->pool) & 15))
    return fail(SLORA_E_INVALID, "lora.pool must be a 16-byte aligned device pointer");
  if (L->dtype != SLORA_F16 && L->dtype != SLORA_BF16)
    return fail(SLORA_E_INVALID, "lora.dtype %d unknown", L->dtype);
  if (L->page_elems <= 0 || L->page_elems % 8)
    return fail(SLORA_E_INVALID, "lora.page_elems %d must be a positive multiple of 8", L->page_elems);
  if (L->n_pages <= 0 || L->n_pages > INT32_MAX)
    return fail(SLORA_E_INVALID, "lora.n_pages %lld out of range", (long long)L->n_pages);
  if (L->d_in <= 0 || L->d_out <= 0 || L->d_in % 8 || L->d_out % 8)
    return fail(SLORA_E_INVALID, "lora.d_in / d_out (%d, %d) must be positive multiples of 8",
                L->d_in, L->d_out);
  if (L->r_max < 0 || L->r_max > kMaxRank)
    return fail(SLORA_E_INVALID, "lora.r_max %d outside [0, %d]", L->r_max, kMaxRank);
  if (L->n_adapters < 0 || (L->n_adapters > 0 && (!L->base || !L->rank || !L->scale)))
    return fail(SLORA_E_INVALID, "lora.base / rank / scale missing");
  if (L->page_table_len < 0) return fail(SLORA_E_INVALID, "lora.page_table_len < 0");
  if (R->n_tokens < 0 || R->n_segments < 0)
    return fail(SLORA_E_INVALID, "routing.n_tokens / n_segments < 0");
  if (R->policy < SLORA_POLICY_AUTO || R->policy > SLORA_POLICY_SGMV)
    return fail(SLORA_E_INVALID, "routing.policy %d unknown", R->policy);
  const int32_t S = R->n_segments;
  int32_t seg_end = 0;
  if (S > 0) {
    if (!R->seg_offsets || !R->seg_adapter)
      return fail(SLORA_E_INVALID, "routing.seg_offsets / seg_adapter is NULL");
    if (R->seg_offsets[0] != 0) return fail(SLORA_E_INVALID, "routing.seg_offsets[0] != 0");
    for (int32_t s = 0; s < S; ++s)
      if (R->seg_offsets[s + 1] < R->seg_offsets[s])
        return fail(SLORA_E_INVALID, "routing.seg_offsets decreases at %d", s);
    seg_end = R->seg_offsets[S];
    if (seg_end > R->n_tokens)
      return fail(SLORA_E_INVALID, "routing.seg_offsets[S] = %d > n_tokens %d", seg_end, R->n_tokens);
  } else if (R->seg_offsets && R->seg_offsets[0] != 0) {
    return fail(SLORA_E_INVALID, "routing.seg_offsets[0] != 0");
  }
  const int32_t n_dec = R->n_tokens - seg_end;
  if (n_dec > 0 && !R->token_adapter) return fail(SLORA_E_INVALID, "routing.token_adapter is NULL");

  const int32_t P = L->page_elems;
  const int32_t cA = (L->d_in + P - 1) / P, cB = (L->d_out + P - 1) / P;

  // Check one adapter id; returns 1 if the token does LoRA work, 0 if not, < 0 on error.
  auto check = [&](int32_t a) -> int {
    if (a < -1 || a >= L->n_adapters)
      return fail(SLORA_E_INVALID, "adapter id %d outside [-1, %d)", a, L->n_adapters);
    if (a < 0) return 0;
    const int32_t r = L->rank[a];
    if (r < 0 || r > kMaxRank) return fail(SLORA_E_INVALID, "adapter %d rank %d invalid", a, r);
    if (r == 0) return 0;
    if (r > L->r_max)
      return fail(SLORA_E_INVALID, "adapter %d rank %d > r_max %d", a, r, L->r_max);
    const int64_t b = L->base[a];
    if (b < 0) return fail(SLORA_E_STATE, "adapter %d is not resident", a);
    const int64_t end = b + (int64_t)r * (cA + cB);
    if (end > L->page_table_len || end > INT32_MAX)
      return fail(SLORA_E_INVALID, "adapter %d page-table entries [%lld, %lld) exceed length %lld", a,
                  (long long)b, (long long)end, (long long)L->page_table_len);
    if (!L->page_table) return fail(SLORA_E_INVALID, "lora.page_table is NULL");
    if (!std::isfinite(L->scale[a])) return fail(SLORA_E_INVALID, "adapter %d scale not finite", a);
    return 1;
  };

  std::vector<Pair> mb;  // tokens for MBGMV
  std::vector<std::pair<GroupDesc, std::vector<int32_t>>> sg, mbg;
  std::vector<Pair> sg_ids;  // per-token ids bucketed into SGMV tiles (policy SGMV)
  for (int32_t s = 0; s < S; ++s) {
    const int32_t b = R->seg_offsets[s], e = R->seg_offsets[s + 1];
    if (e == b) {
      int rc = check(R->seg_adapter[s]);  // ids of empty segments must still be valid
      if (rc < 0) return rc;
      continue;
    }
    const int32_t a = R->seg_adapter[s];
    int rc = check(a);
    if (rc < 0) return rc;
    if (rc == 0) continue;
    if (R->policy == SLORA_POLICY_MBGMV) {
      for (int32_t t = b; t < e; ++t) mb.push_back({a, t});
    } else {
      std::vector<int32_t> toks((size_t)(e - b));
      for (int32_t t = b; t < e; ++t) toks[(size_t)(t - b)] = t;
      split_run(toks.data(), e - b, a, kSgTile, L, &sg);
    }
  }
  for (int32_t q = 0; q < n_dec; ++q) {
    const int32_t a = R->token_adapter[q];
    int rc = check(a);
    if (rc < 0) return rc;
    if (rc == 0) continue;
    if (R->policy == SLORA_POLICY_SGMV) sg_ids.push_back({a, seg_end + q});
    else mb.push_back({a, seg_end + q});
  }
  auto by_adapter = [](const Pair& x, const Pair& y) { return x.adapter < y.adapter; };
  std::stable_sort(mb.begin(), mb.end(), by_adapter);
  std::stable_sort(sg_ids.begin(), sg_ids.end(), by_adapter);
  auto bucket = [&](const std::vector<Pair>& v, int32_t cap,
                    std::vector<std::pair<GroupDesc, std::vector<int32_t>>>* out) {
    std::vector<int32_t> toks;
    for (size_t i = 0; i < v.size();) {
      size_t j = i;
      toks.clear();
      while (j < v.size() && v[j].adapter == v[i].adapter) toks.push_back(v[j++].token);
      split_run(toks.data(), (int32_t)toks.size(), v[i].adapter, cap, L, out);
      i = j;
    }
  };
  bucket(mb, kMbGroup, &mbg);
  bucket(sg_ids, kSgTile, &sg);

  auto by_rank_desc = [](const std::pair<GroupDesc, std::vector<int32_t>>& x,
                         const std::pair<GroupDesc, std::vector<int32_t>>& y) {
    return x.first.rank > y.first.rank;
  };
  std::stable_sort(mbg.begin(), mbg.end(), by_rank_desc);
  std::stable_sort(sg.begin(), sg.end(), by_rank_desc);

  plan->tok.clear();
  plan->mb_groups.clear();
  plan->mb_shrink.clear();
  plan->sg_tiles.clear();
  for (auto& g : mbg) {
    g.first.tok_begin = (int32_t)plan->tok.size();
    plan->tok.insert(plan->tok.end(), g.second.begin(), g.second.end());
    const int32_t gi = (int32_t)plan->mb_groups.size();
    plan->mb_groups.push_back(g.first);
    const int32_t nb = (g.first.rank + kMbShrinkRows - 1) / kMbShrinkRows;
    for (int32_t blk = 0; blk < nb; ++blk) plan->mb_shrink.push_back({gi, blk});
  }
  for (auto& g : sg) {
    g.first.tok_begin = (int32_t)plan->tok.size();
    plan->tok.insert(plan->tok.end(), g.second.begin(), g.second.end());
    plan->sg_tiles.push_back(g.first);
  }
  plan->n_routed = (int32_t)plan->tok.size();
  return SLORA_OK;
}

int64_t workspace_bound(const slora_lora* L, const slora_routing* R) {
  const int64_t T = std::max<int32_t>(R->n_tokens, 0);
  const int64_t rm = std::max<int32_t>(L->r_max, 0);
  int64_t b = align_up(T * rm * 4, 256);                                     // v
  b += align_up(T * 4, 256);                                                 // tokens
  b += align_up(T * (int64_t)sizeof(GroupDesc), 256);                        // MBGMV groups
  b += align_up(T * ((rm + kMbShrinkRows - 1) / kMbShrinkRows) * (int64_t)sizeof(Item), 256);
  b += align_up(T * (int64_t)sizeof(GroupDesc), 256);                        // SGMV tiles
  return std::max<int64_t>(b, 256);
}

PlanLayout layout_plan(const slora_lora* L, const slora_routing* R, const Plan& p) {
  PlanLayout o{};
  o.v_off = 0;
  o.v_bytes = align_up((int64_t)std::max<int32_t>(R->n_tokens, 0) * std::max<int32_t>(L->r_max, 0) * 4, 256);
  int64_t at = o.v_bytes;
  o.blob_off = at;
  o.tok_off = at;
  at += align_up((int64_t)p.tok.size() * 4, 256);
  o.mbg_off = at;
  at += align_up((int64_t)p.mb_groups.size() * (int64_t)sizeof(GroupDesc), 256);
  o.mbs_off = at;
  at += align_up((int64_t)p.mb_shrink.size() * (int64_t)sizeof(Item), 256);
  o.sgt_off = at;
  at += align_up((int64_t)p.sg_tiles.size() * (int64_t)sizeof(GroupDesc), 256);
  o.blob_bytes = at - o.blob_off;
  o.total = std::max<int64_t>(at, 256);
  return o;
}

}  // namespace slora
