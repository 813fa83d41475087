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

// Per-adapter counts of the call's kept tokens live in sc->cnt (all zero between calls).
void clear_counts(PlanScratch* sc) {
  for (int32_t a : sc->mb_ad) sc->cnt[(size_t)a] = 0;
  for (int32_t a : sc->sg_ad) sc->cnt[(size_t)a] = 0;
  for (int32_t a : sc->seen) sc->cnt[(size_t)a] = 0;
}

void count_pair(PlanScratch* sc, std::vector<int32_t>* ad, std::vector<int32_t>* in, int32_t a,
                int32_t t) {
  ad->push_back(a);
  in->push_back(t);
  ++sc->cnt[(size_t)a];
}

// Counting sort of (adapter, token) pairs by adapter id, tokens kept in input order;
// appends one record (first, count, adapter[, 1]) per part of at most `cap` tokens
// (an even split of each adapter's tokens). Leaves the counts of these adapters zero.
void bucket(PlanScratch* sc, const std::vector<int32_t>& ad, const std::vector<int32_t>& in,
            std::vector<int32_t>* out_tok, int32_t cap, std::vector<int32_t>* recs, int width) {
  std::vector<int32_t>& used = sc->used;
  used.clear();
  for (int32_t a : ad)
    if (sc->cnt[(size_t)a] > 0) {
      used.push_back(a);
      sc->cnt[(size_t)a] = -sc->cnt[(size_t)a];  // mark as listed
    }
  const size_t words = (sc->cnt.size() + 63) / 64;
  if (used.size() * 16 < words) {
    std::sort(used.begin(), used.end());
  } else {  // ascending ids from a bitmap when it is short next to the list
    sc->bits.assign(words, 0);
    for (int32_t a : used) sc->bits[(size_t)a >> 6] |= 1ull << (a & 63);
    used.clear();
    for (size_t w = 0; w < words; ++w)
      for (uint64_t b = sc->bits[w]; b; b &= b - 1)
        used.push_back((int32_t)(w * 64 + (size_t)__builtin_ctzll(b)));
  }
  int32_t at = 0;
  for (int32_t a : used) {
    const int32_t n = -sc->cnt[(size_t)a];
    sc->cnt[(size_t)a] = at;  // now the write cursor of a's tokens
    const Split sp(n, cap);
    int32_t f = at;
    for (int32_t p = 0; p < sp.parts; ++p) {
      recs->push_back(f);
      recs->push_back(sp.size(p));
      recs->push_back(a);
      if (width == 4) recs->push_back(1);  // tile whose tokens come from the list
      f += sp.size(p);
    }
    at += n;
  }
  out_tok->resize((size_t)at);
  for (size_t i = 0; i < ad.size(); ++i) (*out_tok)[(size_t)sc->cnt[(size_t)ad[i]]++] = in[i];
  for (int32_t a : used) sc->cnt[(size_t)a] = 0;
}

// Stable order of records (width ints, adapter at index 2) by descending rank.
void rank_order(const slora_lora* L, const std::vector<int32_t>& recs, int width,
                std::vector<int32_t>* order, std::vector<int32_t>* hist) {
  const int32_t n = (int32_t)(recs.size() / (size_t)width);
  hist->assign(kMaxRank + 2, 0);
  for (int32_t i = 0; i < n; ++i) ++(*hist)[(size_t)(kMaxRank - L->rank[recs[(size_t)i * width + 2]] + 1)];
  for (int32_t b = 1; b <= kMaxRank + 1; ++b) (*hist)[(size_t)b] += (*hist)[(size_t)b - 1];
  order->resize((size_t)n);
  for (int32_t i = 0; i < n; ++i)
    (*order)[(size_t)(*hist)[(size_t)(kMaxRank - L->rank[recs[(size_t)i * width + 2]])]++] = i;
}

}  // namespace

int64_t plan_bytes(const slora_lora* L, const slora_routing* R, PlanScratch* sc, PlanView* v) {
  int32_t seg_end = 0;
  int rc = validate(L, R, &seg_end);
  if (rc) return rc;
  const int32_t P = L->page_elems;
  const int32_t cA = (L->d_in + P - 1) / P, cB = (L->d_out + P - 1) / P;
  sc->mb_ad.clear();
  sc->mb_in.clear();
  sc->seen.clear();
  sc->sg_ad.clear();
  sc->sg_in.clear();
  sc->grp.clear();
  sc->tiles.clear();
  if ((int64_t)sc->cnt.size() < (int64_t)L->n_adapters) sc->cnt.assign((size_t)L->n_adapters, 0);
  *v = PlanView{};
  // an adapter is checked when first met in a call (cnt[a] == 0 until a token of it is kept)
  auto admit = [&](int32_t a) -> int {
    if (a < -1 || a >= L->n_adapters) {
      clear_counts(sc);
      return fail(SLORA_E_INVALID, "adapter id %d outside [-1, %d)", a, L->n_adapters);
    }
    if (a < 0) return 0;
    if (sc->cnt[(size_t)a] > 0) return 1;
    const int rc = check_adapter(L, a, cA, cB);
    if (rc < 0) clear_counts(sc);
    return rc;
  };
  const int32_t S = R->n_segments;
  for (int32_t s = 0; s < S; ++s) {
    const int32_t b = R->seg_offsets[s], e = R->seg_offsets[s + 1], a = R->seg_adapter[s];
    if (e == b) {  // an empty segment does no work; its id must still be in range
      if (a < -1 || a >= L->n_adapters) {
        clear_counts(sc);
        return fail(SLORA_E_INVALID, "adapter id %d outside [-1, %d)", a, L->n_adapters);
      }
      continue;
    }
    rc = admit(a);
    if (rc < 0) return rc;
    if (rc == 0) continue;
    if (R->policy == SLORA_POLICY_MBGMV) {
      for (int32_t t = b; t < e; ++t) count_pair(sc, &sc->mb_ad, &sc->mb_in, a, t);
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
  if (R->policy == SLORA_POLICY_AUTO) {
    // Per-token ids of an adapter with at least kAutoSgmvTok tokens in the call go to
    // SGMV tiles (its weights are then read once per 64 tokens instead of once per 4)
    // when SGMV runs anyway (segments) or when they are numerous enough to pay for its
    // launches (kAutoSgmvBatch tokens, and at least a 1 / (1 + kAutoSgmvShare) share of
    // the ids: a small share saves less than the launches cost); the rest to MBGMV,
    // unless SGMV runs and fewer
    // than kAutoMbgmvMin tokens would be left: then a launch of its own for them costs
    // more than the tiles they add, and every id goes to SGMV.
    for (int32_t q = 0; q < n_dec; ++q) {
      const int32_t a = R->token_adapter[q];
      rc = admit(a);
      if (rc < 0) return rc;
      if (rc == 0) continue;
      if (sc->cnt[(size_t)a]++ == 0) sc->seen.push_back(a);
    }
    int64_t hot = 0, cold = 0;
    for (int32_t a : sc->seen)
      (sc->cnt[(size_t)a] >= kAutoSgmvTok ? hot : cold) += sc->cnt[(size_t)a];
    const bool sg_runs =
        !sc->tiles.empty() || (hot >= kAutoSgmvBatch && hot * kAutoSgmvShare >= cold);
    const bool sg_hot = hot > 0 && sg_runs;
    const int64_t left = sg_hot ? cold : cold + hot;  // ids MBGMV would get
    const bool sg_all = sg_runs && left > 0 && left < kAutoMbgmvMin;
    for (int32_t q = 0; q < n_dec; ++q) {
      const int32_t a = R->token_adapter[q];
      if (a < 0 || sc->cnt[(size_t)a] == 0) continue;  // no adapter, or rank 0
      const bool to_sg = sg_all || (sg_hot && sc->cnt[(size_t)a] >= kAutoSgmvTok);
      (to_sg ? sc->sg_ad : sc->mb_ad).push_back(a);
      (to_sg ? sc->sg_in : sc->mb_in).push_back(seg_end + q);
    }
  } else {
    for (int32_t q = 0; q < n_dec; ++q) {
      const int32_t a = R->token_adapter[q];
      rc = admit(a);
      if (rc < 0) return rc;
      if (rc == 0) continue;
      if (R->policy == SLORA_POLICY_SGMV) count_pair(sc, &sc->sg_ad, &sc->sg_in, a, seg_end + q);
      else count_pair(sc, &sc->mb_ad, &sc->mb_in, a, seg_end + q);
    }
  }
  // tokens bucketed by adapter (ascending id, tokens in ascending order): groups of <= 4
  // for MBGMV, tiles of <= 64 for SGMV
  bucket(sc, sc->mb_ad, sc->mb_in, &sc->mb_tok, kMbGroup, &sc->grp, 3);
  bucket(sc, sc->sg_ad, sc->sg_in, &sc->sg_tok, kSgTile, &sc->tiles, 4);

  // groups and tiles by descending rank (stable), the costliest work first
  const int32_t n_groups = (int32_t)(sc->grp.size() / 3);
  rank_order(L, sc->grp, 3, &sc->order, &sc->hist);
  {
    rank_order(L, sc->tiles, 4, &sc->tile_order, &sc->hist);
    const size_t nt = sc->tiles.size() / 4;
    sc->tiles_sorted.resize(sc->tiles.size());
    for (size_t i = 0; i < nt; ++i)
      for (int j = 0; j < 4; ++j)
        sc->tiles_sorted[4 * i + j] = sc->tiles[4 * (size_t)sc->tile_order[i] + j];
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
  v->n_tok = (int32_t)sc->sg_tok.size();  // listed tokens: those of bucketed tiles only
  v->n_routed = (int32_t)sc->mb_tok.size() + sg_tok;
  return align_up((int64_t)v->n_mb * (int64_t)sizeof(MbItem), 64) +
         align_up((int64_t)v->n_sg * (int64_t)sizeof(SgTile), 64) +
         align_up((int64_t)v->n_tok * 4, 64);
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

  // one template per group; items are 32-byte copies of it with `part` (and the token
  // pair of expand items) filled in
  MbItem* out = v->mb;
  MbItem* out_e = v->mb + v->n_mb_shrink;
  for (int32_t s = 0; s < v->n_groups; ++s) {
    const int32_t gi = sc->order[(size_t)s];
    const int32_t k0 = sc->grp[3 * (size_t)gi], n = sc->grp[3 * (size_t)gi + 1];
    const int32_t a = sc->grp[3 * (size_t)gi + 2];
    const int32_t* tk = sc->mb_tok.data() + k0;
    const int32_t r = L->rank[a];
    alignas(32) MbItem it;
    memset(&it, 0, sizeof it);
    for (int32_t t = 0; t < n; ++t) it.tok[t] = tk[t];
    it.pt_base = (int32_t)L->base[a];
    it.rank = (uint8_t)r;
    it.scale = L->scale[a];
    it.info = MbItem::pack_info(n, 0, 0);
    const int32_t nb = (r + kMbShrinkRows - 1) / kMbShrinkRows;
    for (int32_t b = 0; b < nb; ++b, ++out) {  // shrink: role 0, part = row block
      memcpy(out, &it, sizeof it);
      out->part = (int16_t)b;
    }
    const int32_t nct = n_ctile(L, r);
    for (int32_t t0 = 0; t0 < n; t0 += kMbExpandTok) {  // expand: a token pair, part = column tile
      const int32_t m = std::min(kMbExpandTok, n - t0);
      it.info = MbItem::pack_info(m, 1, mb_split(r));
      for (int32_t t = 0; t < kMbGroup; ++t) it.tok[t] = t < m ? tk[t0 + t] : 0;
      for (int32_t ct = 0; ct < nct; ++ct, ++out_e) {
        memcpy(out_e, &it, sizeof it);
        out_e->part = (int16_t)ct;
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
    if (from_keys) {  // segment tiles name their tokens by first_tok
      for (int32_t q = 0; q < n; ++q) v->tok[at + q] = sc->sg_tok[(size_t)(first + q)];
      at += n;
    }
  }
}

WsLayout ws_layout(const slora_lora* L, const slora_routing* R) {
  WsLayout o{};
  const int64_t T = std::max<int32_t>(R->n_tokens, 0);
  const int64_t rows = T * std::max<int32_t>(L->r_max, 0);
  o.v_off = kHeaderBytes;
  o.sg_off = o.v_off + align_up(rows * 8, 256);
  const int64_t sg_rows = T * sg_v_stride(std::max<int32_t>(L->r_max, 0));
  o.flg_off = o.sg_off + align_up((int64_t)sg_max_split(std::max<int32_t>(L->d_in, 0)) * sg_rows * 4, 256);
  o.total = o.flg_off + align_up(T * 2 * kSgMaxSplit * 4, 256);
  return o;
}

}  // namespace slora
