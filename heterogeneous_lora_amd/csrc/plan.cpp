// Routing validation and work-list planning (host, integer only).
//
// Every token picks its adapter: by segment for a request's contiguous prefill
// tokens, or by its own id for decode tokens ("Makale Bulteni - S-LoRA", section
// "Iddia ve Gerceklik": each token of a batch may use a different adapter; the
// S-LoRA overview, section "2. Heterogeneous Batching": adapters of different
// ranks are batched together). The planner groups tokens that share an adapter so
// that each group reads the adapter's pages once:
//   * MBGMV groups: decode tokens bucketed by adapter (token order kept), split
//     evenly into groups of at most kMbGroup tokens; each group becomes
//     ceil(rank / 8) shrink items and, per pair of its tokens, one expand item per
//     column tile;
//   * SGMV tiles: a segment (or a bucket of ids) split evenly into tiles of at
//     most kSgTile tokens.
// Groups are ordered by descending rank so that the costliest work items are
// dispatched first. The order only decides scheduling: every token's result is
// computed by the same fixed sequence of operations wherever it lands.
//
// The plan is written straight into a pinned staging buffer that the kernels read
// over the bus, so planning allocates nothing per call (scratch vectors are reused).
#include <algorithm>
#include <cmath>
#include <cstring>

#include "internal.h"

namespace slora {

namespace {

int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

int validate(const slora_lora* L, const slora_routing* R, int32_t* seg_end_out) {
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
  if ((L->d_in + L->page_elems - 1) / L->page_elems > 32)  // a wave holds 2 rows' page ids
    return fail(SLORA_E_INVALID, "d_in %d spans more than 32 pages of %d", L->d_in, L->page_elems);
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
  if (R->n_tokens - seg_end > 0 && !R->token_adapter)
    return fail(SLORA_E_INVALID, "routing.token_adapter is NULL");
  *seg_end_out = seg_end;
  return SLORA_OK;
}

// 1 if a token with adapter a does LoRA work, 0 if not, < 0 on an invalid id.
int check_adapter(const slora_lora* L, int32_t a, int32_t cA, int32_t cB) {
  if (a < -1 || a >= L->n_adapters)
    return fail(SLORA_E_INVALID, "adapter id %d outside [-1, %d)", a, L->n_adapters);
  if (a < 0) return 0;
  const int32_t r = L->rank[a];
  if (r < 0 || r > kMaxRank) return fail(SLORA_E_INVALID, "adapter %d rank %d invalid", a, r);
  if (r == 0) return 0;
  if (r > L->r_max) return fail(SLORA_E_INVALID, "adapter %d rank %d > r_max %d", a, r, L->r_max);
  const int64_t b = L->base[a];
  if (b < 0) return fail(SLORA_E_STATE, "adapter %d is not resident", a);
  const int64_t end = b + (int64_t)r * (cA + cB);
  if (end > L->page_table_len || end > INT32_MAX)
    return fail(SLORA_E_INVALID, "adapter %d page-table entries [%lld, %lld) exceed length %lld", a,
                (long long)b, (long long)end, (long long)L->page_table_len);
  if (!L->page_table) return fail(SLORA_E_INVALID, "lora.page_table is NULL");
  if (!std::isfinite(L->scale[a])) return fail(SLORA_E_INVALID, "adapter %d scale not finite", a);
  return 1;
}

// Even split of n tokens into ceil(n / cap) parts: part i has base + (i < extra).
struct Split {
  int32_t parts, base, extra;
  Split(int32_t n, int32_t cap) : parts((n + cap - 1) / cap), base(0), extra(0) {
    if (parts) { base = n / parts; extra = n % parts; }
  }
  int32_t size(int32_t i) const { return base + (i < extra ? 1 : 0); }
};

int32_t n_ctile(const slora_lora* L, int32_t rank) {
  const int32_t cols = 4 / mb_split(rank) * kMbWaveCols;
  return (L->d_out + cols - 1) / cols;
}

}  // namespace

int64_t plan_bytes(const slora_lora* L, const slora_routing* R, PlanScratch* sc, PlanView* v) {
  int32_t seg_end = 0;
  int rc = validate(L, R, &seg_end);
  if (rc) return rc;
  const int32_t P = L->page_elems;
  const int32_t cA = (L->d_in + P - 1) / P, cB = (L->d_out + P - 1) / P;
  sc->mb_keys.clear();
  sc->sg_keys.clear();
  sc->grp.clear();
  sc->tiles.clear();
  *v = PlanView{};
  const int32_t S = R->n_segments;
  for (int32_t s = 0; s < S; ++s) {
    const int32_t b = R->seg_offsets[s], e = R->seg_offsets[s + 1], a = R->seg_adapter[s];
    if (e == b) {  // an empty segment does no work; its id must still be in range
      if (a < -1 || a >= L->n_adapters)
        return fail(SLORA_E_INVALID, "adapter id %d outside [-1, %d)", a, L->n_adapters);
      continue;
    }
    rc = check_adapter(L, a, cA, cB);
    if (rc < 0) return rc;
    if (rc == 0) continue;
    if (R->policy == SLORA_POLICY_MBGMV) {
      for (int32_t t = b; t < e; ++t) sc->mb_keys.push_back(((uint64_t)a << 32) | (uint32_t)t);
    } else {  // a segment's tokens are contiguous: tiles straight from the offsets
      const Split sp(e - b, kSgTile);
      int32_t at = b;
      for (int32_t i = 0; i < sp.parts; ++i) {
        sc->tiles.insert(sc->tiles.end(), {at, sp.size(i), a, 0});
        at += sp.size(i);
      }
    }
  }
  const int32_t n_dec = R->n_tokens - seg_end;
  for (int32_t q = 0; q < n_dec; ++q) {
    const int32_t a = R->token_adapter[q];
    rc = check_adapter(L, a, cA, cB);
    if (rc < 0) return rc;
    if (rc == 0) continue;
    const uint64_t key = ((uint64_t)a << 32) | (uint32_t)(seg_end + q);
    (R->policy == SLORA_POLICY_SGMV ? sc->sg_keys : sc->mb_keys).push_back(key);
  }
  // (adapter, token) keys sort adapter-major with tokens ascending: a stable bucket
  std::sort(sc->mb_keys.begin(), sc->mb_keys.end());
  std::sort(sc->sg_keys.begin(), sc->sg_keys.end());
  auto runs = [](const std::vector<uint64_t>& keys, int32_t cap, std::vector<int32_t>* out,
                 int32_t width) {
    for (size_t i = 0; i < keys.size();) {
      size_t j = i;
      const uint32_t a = (uint32_t)(keys[i] >> 32);
      while (j < keys.size() && (uint32_t)(keys[j] >> 32) == a) ++j;
      const Split sp((int32_t)(j - i), cap);
      int32_t at = (int32_t)i;
      for (int32_t p = 0; p < sp.parts; ++p) {
        out->push_back(at);
        out->push_back(sp.size(p));
        out->push_back((int32_t)a);
        if (width == 4) out->push_back(1);  // tile whose tokens come from the keys
        at += sp.size(p);
      }
      i = j;
    }
  };
  runs(sc->mb_keys, kMbGroup, &sc->grp, 3);
  runs(sc->sg_keys, kSgTile, &sc->tiles, 4);

  // MBGMV groups by descending rank (stable)
  const int32_t n_groups = (int32_t)(sc->grp.size() / 3);
  sc->order.resize((size_t)n_groups);
  for (int32_t gi = 0; gi < n_groups; ++gi) sc->order[(size_t)gi] = gi;
  std::stable_sort(sc->order.begin(), sc->order.end(), [&](int32_t x, int32_t y) {
    return L->rank[sc->grp[3 * (size_t)x + 2]] > L->rank[sc->grp[3 * (size_t)y + 2]];
  });
  // SGMV tiles by descending rank too (stable: segments first, then bucketed ids)
  {
    const size_t nt = sc->tiles.size() / 4;
    std::vector<int32_t>& idx = sc->tile_order;
    idx.resize(nt);
    for (size_t i = 0; i < nt; ++i) idx[i] = (int32_t)i;
    std::stable_sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) {
      return L->rank[sc->tiles[4 * (size_t)x + 2]] > L->rank[sc->tiles[4 * (size_t)y + 2]];
    });
    sc->tiles_sorted.resize(sc->tiles.size());
    for (size_t i = 0; i < nt; ++i)
      for (int j = 0; j < 4; ++j) sc->tiles_sorted[4 * i + j] = sc->tiles[4 * (size_t)idx[i] + j];
    sc->tiles.swap(sc->tiles_sorted);
  }
  int64_t n_shrink = 0, n_expand = 0;
  int32_t max_tok = 0;
  for (int32_t gi = 0; gi < n_groups; ++gi) {
    const int32_t n = sc->grp[3 * (size_t)gi + 1], r = L->rank[sc->grp[3 * (size_t)gi + 2]];
    n_shrink += (r + kMbShrinkRows - 1) / kMbShrinkRows;
    n_expand += (int64_t)((n + kMbExpandTok - 1) / kMbExpandTok) * n_ctile(L, r);
    max_tok = std::max(max_tok, n);
  }
  if (n_shrink + n_expand > INT32_MAX / 2) return fail(SLORA_E_INVALID, "batch too large");
  v->n_mb = (int32_t)(n_shrink + n_expand);
  v->n_mb_shrink = (int32_t)n_shrink;
  v->n_groups = n_groups;
  v->mb_max_tok = max_tok;
  v->n_sg = (int32_t)(sc->tiles.size() / 4);
  int32_t sg_tok = 0;
  for (int32_t t = 0; t < v->n_sg; ++t) sg_tok += sc->tiles[4 * (size_t)t + 1];
  v->n_tok = sg_tok;
  v->n_routed = (int32_t)sc->mb_keys.size() + sg_tok;
  return align_up((int64_t)v->n_mb * (int64_t)sizeof(MbItem), 64) +
         align_up((int64_t)v->n_sg * (int64_t)sizeof(SgTile), 64) +
         align_up((int64_t)sg_tok * 4, 64);
}

void plan_write(const slora_lora* L, const slora_routing* R, PlanScratch* sc, void* buf,
                PlanView* v) {
  (void)R;
  uint8_t* p = (uint8_t*)buf;
  v->mb = (MbItem*)p;
  p += align_up((int64_t)v->n_mb * (int64_t)sizeof(MbItem), 64);
  v->sg = (SgTile*)p;
  p += align_up((int64_t)v->n_sg * (int64_t)sizeof(SgTile), 64);
  v->tok = (int32_t*)p;

  auto base_item = [&](int32_t gi) {
    const int32_t k0 = sc->grp[3 * (size_t)gi], n = sc->grp[3 * (size_t)gi + 1];
    const int32_t a = sc->grp[3 * (size_t)gi + 2];
    MbItem it;
    memset(&it, 0, sizeof it);
    for (int32_t t = 0; t < n; ++t) it.tok[t] = (int32_t)(uint32_t)sc->mb_keys[(size_t)(k0 + t)];
    it.n_tok = n;
    it.pt_base = (int32_t)L->base[a];
    it.rank = L->rank[a];
    it.scale = L->scale[a];
    return it;
  };
  MbItem* out = v->mb;
  for (int32_t s = 0; s < v->n_groups; ++s) {  // shrink items, groups in dispatch order
    const int32_t gi = sc->order[(size_t)s];
    MbItem it = base_item(gi);
    it.role = 0;
    const int32_t nb = (it.rank + kMbShrinkRows - 1) / kMbShrinkRows;
    for (int32_t b = 0; b < nb; ++b) {
      it.part = b;
      *out++ = it;
    }
  }
  for (int32_t s = 0; s < v->n_groups; ++s) {  // expand items
    const int32_t gi = sc->order[(size_t)s];
    const MbItem g = base_item(gi);
    const int32_t nct = n_ctile(L, g.rank);
    for (int32_t t0 = 0; t0 < g.n_tok; t0 += kMbExpandTok) {
      MbItem it = g;
      it.n_tok = std::min(kMbExpandTok, g.n_tok - t0);
      for (int32_t t = 0; t < kMbGroup; ++t) it.tok[t] = t < it.n_tok ? g.tok[t0 + t] : 0;
      it.role = 1;
      it.split = mb_split(g.rank);
      for (int32_t ct = 0; ct < nct; ++ct) {
        it.part = ct;
        *out++ = it;
      }
    }
  }
  int32_t at = 0;
  for (int32_t t = 0; t < v->n_sg; ++t) {
    const int32_t first = sc->tiles[4 * (size_t)t], n = sc->tiles[4 * (size_t)t + 1];
    const int32_t a = sc->tiles[4 * (size_t)t + 2], from_keys = sc->tiles[4 * (size_t)t + 3];
    SgTile tile;
    memset(&tile, 0, sizeof tile);
    tile.tok_begin = at;
    tile.n_tok = n;
    tile.pt_base = (int32_t)L->base[a];
    tile.rank = L->rank[a];
    tile.scale = L->scale[a];
    tile.first_tok = from_keys ? -1 : first;
    v->sg[t] = tile;
    v->sg_max_rank = std::max(v->sg_max_rank, tile.rank);
    for (int32_t q = 0; q < n; ++q)
      v->tok[at + q] = from_keys ? (int32_t)(uint32_t)sc->sg_keys[(size_t)(first + q)] : first + q;
    at += n;
  }
}

WsLayout ws_layout(const slora_lora* L, const slora_routing* R) {
  WsLayout o{};
  const int64_t T = std::max<int32_t>(R->n_tokens, 0);
  const int64_t rows = T * std::max<int32_t>(L->r_max, 0);
  o.v_off = kHeaderBytes;
  o.sg_off = o.v_off + align_up(rows * 8, 256);
  const int64_t sg_rows = T * sg_v_stride(std::max<int32_t>(L->r_max, 0));
  o.total = o.sg_off + align_up((int64_t)sg_max_split(std::max<int32_t>(L->d_in, 0)) * sg_rows * 4, 256);
  return o;
}

}  // namespace slora
