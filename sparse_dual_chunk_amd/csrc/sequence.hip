// Whole-prompt chunked prefill: the equal-time chunk schedule (chunk sizing
// by the attention cost, as dynamic chunked pipeline parallelism does on the
// paper-review page, section 4, "Pipeline parallelism", Figure 9) and the
// driver that runs the chunks, with each chunk's index build one chunk ahead
// on a second stream.  Declared in include/dcasparse.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <vector>

#include "../../include/dcasparse.h"
#include "entry.h"

namespace {

constexpr int QB = 64;

// Chunk costs over 64-row blocks in O(1) per chunk from prefix sums of the
// blocks' pair counts.
struct CostTable {
  const dca_chunk_cost* m;
  int n = 0, nb = 0;
  std::vector<double> pairs;   // pairs[b] = sum over blocks < b of r * cover(i0 + r)

  CostTable(int n_tokens, const dca_chunk_cost* cost) : m(cost), n(n_tokens) {
    nb = (n + QB - 1) / QB;
    pairs.assign(nb + 1, 0.0);
    for (int b = 0; b < nb; ++b) {
      const long long i0 = (long long)b * QB, r = std::min<long long>(QB, n - i0);
      // dense: the causal extent E; sparse: the expected union of cap keys'
      // worth of 64-key footprints scattered over E, E (1 - exp(-cap / E))
      double ext = (double)(i0 + r);
      if (m->cover_cap > 0) ext = ext * -std::expm1(-(double)m->cover_cap / ext);
      pairs[b + 1] = pairs[b] + (double)r * ext;
    }
  }
  int row(int b) const { return b < nb ? b * QB : n; }
  int rows(int a, int b) const { return row(b) - row(a); }
  // chunk of blocks [a, b)
  double cost(int a, int b) const {
    return m->per_call + m->per_row * rows(a, b) + m->per_index_key * row(b) + m->per_pair * (pairs[b] - pairs[a]);
  }
};

// Greedy packing under a cost limit: each chunk takes blocks while its cost
// stays within T and its rows within max_rows.  Returns the chunk count, or
// INT32_MAX when a single block already exceeds T.  Optionally records the
// block boundaries.
int pack(const CostTable& t, int max_blocks, double T, std::vector<int>* cuts) {
  if (cuts) { cuts->clear(); cuts->push_back(0); }
  int a = 0, count = 0;
  while (a < t.nb) {
    if (t.cost(a, a + 1) > T) return INT32_MAX;
    int b = a + 1;
    while (b < t.nb && b + 1 - a <= max_blocks && t.cost(a, b + 1) <= T) ++b;
    ++count;
    if (cuts) cuts->push_back(b);
    a = b;
  }
  return count;
}

}  // namespace

extern "C" {

int dca_chunk_cost_default(const dca_cfg* cfg, int32_t sparse, dca_chunk_cost* cost) {
  if (!cfg || !cost) return DCA_EINVAL;
  if (cfg->h_q < 1 || cfg->h_kv < 1 || cfg->h_q % cfg->h_kv) return DCA_EINVAL;
  if (cfg->vs_k_vertical < 0 || cfg->vs_k_slash < 0) return DCA_EINVAL;
  if (sparse != 0 && sparse != 1) return DCA_EINVAL;
  const double h = cfg->h_q;
  // least-squares fit to the chunk times of a 256K-token, 40-head prompt in
  // eight 32K-row chunks on MI355X (the fit reproduces them within 3%):
  // 0.55 ns per modelled (row, key, head) pair, 3.8 ns per (row, head),
  // 0.62 ns per (prefix key, head) of index build, 0.4 ms per chunk
  cost->per_call = 400.0;
  cost->per_row = 3.8e-3 * h;
  cost->per_pair = 5.5e-7 * h;
  cost->per_index_key = sparse ? 6.2e-4 * h : 0.0;
  cost->cover_cap = sparse ? 64LL * cfg->vs_k_slash + cfg->vs_k_vertical : 0;
  return DCA_OK;
}

int dca_chunk_schedule(int32_t n_tokens, int32_t n_chunks, int32_t max_rows, const dca_chunk_cost* cost,
                       int32_t* bounds, int32_t* n_out, double* max_cost) {
  if (!cost || !bounds || !n_out) return DCA_EINVAL;
  if (n_tokens < 1 || n_chunks < 1 || max_rows < QB) return DCA_EINVAL;
  const double coef[4] = {cost->per_call, cost->per_row, cost->per_index_key, cost->per_pair};
  for (double c : coef)
    if (!(c >= 0.0) || !std::isfinite(c)) return DCA_EINVAL;
  const CostTable t(n_tokens, cost);
  const int max_blocks = max_rows / QB;
  // chunks of max_blocks blocks are the fewest possible
  if ((t.nb + max_blocks - 1) / max_blocks > n_chunks) return DCA_EINVAL;
  const int want = std::min(n_chunks, t.nb);
  // bisection on the cost limit: pack(T) <= want iff T >= the optimum
  double lo = 0.0, hi = 0.0;
  for (int a = 0; a < t.nb; a += max_blocks) hi = std::max(hi, t.cost(a, std::min(t.nb, a + max_blocks)));
  if (pack(t, max_blocks, lo, nullptr) <= want) hi = lo;
  for (int it = 0; it < 200 && hi - lo > 1e-13 * hi; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (pack(t, max_blocks, mid, nullptr) <= want) hi = mid; else lo = mid;
  }
  std::vector<int> cuts;
  pack(t, max_blocks, hi, &cuts);
  // fewer chunks than asked: split the costliest divisible chunk at its best
  // point until the count is reached (a split never raises the largest cost)
  while ((int)cuts.size() - 1 < want) {
    int pick = -1;
    double pc = -1.0;
    for (size_t c = 0; c + 1 < cuts.size(); ++c)
      if (cuts[c + 1] - cuts[c] >= 2 && t.cost(cuts[c], cuts[c + 1]) > pc) { pc = t.cost(cuts[c], cuts[c + 1]); pick = (int)c; }
    if (pick < 0) break;
    const int a = cuts[pick], b = cuts[pick + 1];
    int best = a + 1;
    double bv = 1e300;
    for (int s = a + 1; s < b; ++s) {
      const double v = std::max(t.cost(a, s), t.cost(s, b));
      if (v < bv) { bv = v; best = s; }
    }
    cuts.insert(cuts.begin() + pick + 1, best);
  }
  double mx = 0.0;
  for (size_t c = 0; c < cuts.size(); ++c) {
    bounds[c] = t.row(cuts[c]);
    if (c + 1 < cuts.size()) mx = std::max(mx, t.cost(cuts[c], cuts[c + 1]));
  }
  *n_out = (int32_t)cuts.size() - 1;
  if (max_cost) *max_cost = mx;
  return DCA_OK;
}

}  // extern "C"

namespace {

// Per-chunk configuration derived from the whole-prompt one.
dca_cfg chunk_cfg(const dca_cfg* cfg, int b0, int b1) {
  dca_cfg c = *cfg;
  c.n_q = b1 - b0;
  c.n_k = b1;
  c.v_idx = nullptr;
  c.s_off = nullptr;
  c.lse_out = nullptr;
  c.cover_pairs = nullptr;
  c.attended_pairs = nullptr;
  c.status = nullptr;
  c.stage_events = nullptr;
  c.workspace = nullptr;
  c.workspace_bytes = 0;
  return c;
}

bool chunk_sparse(const dca_cfg* cfg, const dca_sequence_plan* plan, int n_k) {
  if (!plan->sparse) return false;
  if (cfg->vs_k_per_head) return true;
  // every offset 0 .. n_k - 1 selected: the cover is the dense causal set
  return n_k > cfg->vs_k_slash;
}

struct SeqLayout {
  size_t slot_bytes = 0, ws_bytes = 0, vidx_off = 0, soff_off = 0, lse_off = 0, total = 0;
  int slots = 1;
};

inline size_t up256(size_t x) { return (x + 255) / 256 * 256; }

int seq_layout(const dca_cfg* cfg, const dca_sequence_plan* plan, SeqLayout* L, bool paged = false) {
  if (!cfg || !plan || !plan->bounds) return DCA_EINVAL;
  if (plan->n_chunks < 1 || (plan->sparse != 0 && plan->sparse != 1)) return DCA_EINVAL;
  if (cfg->n_q != cfg->n_k) return DCA_EINVAL;
  const int32_t* b = plan->bounds;
  if (b[0] != 0 || b[plan->n_chunks] != cfg->n_k) return DCA_EINVAL;
  size_t ws = 0;
  int max_rows = 0;
  for (int c = 0; c < plan->n_chunks; ++c) {
    if (!(b[c] < b[c + 1])) return DCA_EINVAL;
    if (b[c] % QB) return DCA_EUNSUPPORTED;
    const dca_cfg cc = chunk_cfg(cfg, b[c], b[c + 1]);
    size_t w = 0;
    const int rc = paged ? dca::paged_prefill_bytes(&cc, &w) : dca_workspace_size(&cc, &w);
    if (rc != DCA_OK) return rc;
    ws = std::max(ws, w);
    max_rows = std::max(max_rows, b[c + 1] - b[c]);
  }
  L->ws_bytes = up256(ws);
  size_t cur = L->ws_bytes;
  L->vidx_off = cur; cur += up256((size_t)cfg->h_q * std::max(cfg->vs_k_vertical, 1) * 4);
  L->soff_off = cur; cur += up256((size_t)cfg->h_q * std::max(cfg->vs_k_slash, 1) * 4);
  L->lse_off = cur; cur += up256((size_t)cfg->h_q * max_rows * 4);
  L->slot_bytes = cur;
  L->slots = plan->index_stream ? 2 : 1;
  L->total = L->slot_bytes * L->slots;
  return DCA_OK;
}

struct Events {
  std::vector<hipEvent_t> ev;
  ~Events() {
    // an event whose recorded work is still pending is released once it completes
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  }
  hipEvent_t make() {
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return nullptr;
    ev.push_back(e);
    return e;
  }
};

void record_opt(void** events, int i, hipStream_t st) {
  if (events && events[i]) (void)hipEventRecord((hipEvent_t)events[i], st);
}

}  // namespace

extern "C" {

int dca_prefill_sequence_workspace_size(const dca_cfg* cfg, const dca_sequence_plan* plan, size_t* bytes) {
  if (!bytes) return DCA_EINVAL;
  SeqLayout L;
  const int rc = seq_layout(cfg, plan, &L);
  if (rc != DCA_OK) return rc;
  *bytes = L.total;
  return DCA_OK;
}

// The whole-prompt driver over a contiguous key cache (values in v) or a paged
// pool (paged: keys and values appended into their pages).
static int sequence_impl(const dca_bf16* q, const dca_bf16* k, const dca_bf16* v, const dca_sequence_plan* plan,
                  const dca_cfg* cfg, const dca_key_cache* cache, const dca_paged_kv* paged, dca_bf16* out) {
  if (!q || !k || !v || !out || !(cache || paged) || !cfg) return DCA_EINVAL;
  if (cfg->v_idx || cfg->s_off || cfg->cover_pairs || cfg->attended_pairs || cfg->stage_events) return DCA_EINVAL;
  SeqLayout L;
  int rc = seq_layout(cfg, plan, &L, paged != nullptr);
  if (rc != DCA_OK) return rc;
  if (!cfg->workspace || cfg->workspace_bytes < L.total || ((uintptr_t)cfg->workspace) % 256) return DCA_EWORKSPACE;
  if (cache && (!cache->k_hi || !cache->k_lo || !cache->k_flags || cache->capacity < cfg->n_k)) return DCA_EINVAL;
  if (paged) {
    rc = dca::paged_valid(paged, cfg->h_kv, cfg->head_dim);
    if (rc != DCA_OK) return rc;
    if ((long long)paged->n_table * paged->page_keys < cfg->n_k) return DCA_EINVAL;
  }
  const int n_chunks = plan->n_chunks, h_q = cfg->h_q, D = cfg->head_dim;
  const int32_t* b = plan->bounds;
  // validate every chunk call before anything is enqueued
  for (int c = 0; c < n_chunks; ++c) {
    const dca_cfg cc = chunk_cfg(cfg, b[c], b[c + 1]);
    size_t w = 0;
    rc = paged ? dca::paged_prefill_bytes(&cc, &w) : dca_workspace_size(&cc, &w);
    if (rc != DCA_OK) return rc;
  }
  hipStream_t st = (hipStream_t)cfg->stream;
  hipStream_t ist = plan->index_stream ? (hipStream_t)plan->index_stream : st;
  const bool overlap = ist != st;
  Events E;
  std::vector<hipEvent_t> idx_done(n_chunks, nullptr), chunk_done(n_chunks, nullptr);
  hipEvent_t start = nullptr;
  if (overlap) {
    start = E.make();
    if (!start) return DCA_EHIP;
    for (int c = 0; c < n_chunks; ++c) {
      idx_done[c] = E.make();
      chunk_done[c] = E.make();
      if (!idx_done[c] || !chunk_done[c]) return DCA_EHIP;
    }
    // the index stream starts after the work already queued on cfg->stream (the inputs)
    if (hipEventRecord(start, st) != hipSuccess || hipStreamWaitEvent(ist, start, 0) != hipSuccess) return DCA_EHIP;
  }
  char* base = (char*)cfg->workspace;
  auto slot = [&](int c) { return base + (size_t)(c % L.slots) * L.slot_bytes; };
  // the index build of chunk c, into its slot
  auto run_index = [&](int c) -> int {
    const int n_k = b[c + 1];
    const bool sparse = chunk_sparse(cfg, plan, n_k);
    // the slot's previous user (chunk c - 2) must have finished its attention
    if (sparse && overlap && c >= L.slots && hipStreamWaitEvent(ist, chunk_done[c - L.slots], 0) != hipSuccess)
      return DCA_EHIP;
    record_opt(plan->index_events, 2 * c, ist);
    if (sparse) {
      dca_cfg cc = chunk_cfg(cfg, b[c], n_k);
      cc.workspace = slot(c);
      cc.workspace_bytes = L.ws_bytes;
      cc.stream = ist;
      // the chunk's positions are b_c .. b_{c+1}-1 by construction (implied, not checked)
      const int r = dca::index_impl(q + (size_t)b[c] * h_q * D, k, nullptr, &cc, (int32_t*)(slot(c) + L.vidx_off),
                                    (int32_t*)(slot(c) + L.soff_off));
      if (r != DCA_OK) return r;
    }
    record_opt(plan->index_events, 2 * c + 1, ist);
    if (overlap && hipEventRecord(idx_done[c], ist) != hipSuccess) return DCA_EHIP;
    return DCA_OK;
  };
  if (overlap) {
    rc = run_index(0);
    if (rc != DCA_OK) return rc;
  }
  for (int c = 0; c < n_chunks; ++c) {
    // index builds run one chunk ahead on their own stream
    if (overlap && c + 1 < n_chunks) {
      rc = run_index(c + 1);
      if (rc != DCA_OK) return rc;
    }
    if (!overlap) {
      rc = run_index(c);
      if (rc != DCA_OK) return rc;
    }
    const int n_k = b[c + 1], n_q = b[c + 1] - b[c];
    const bool sparse = chunk_sparse(cfg, plan, n_k);
    dca_cfg cc = chunk_cfg(cfg, b[c], n_k);
    cc.workspace = slot(c);
    cc.workspace_bytes = L.ws_bytes;
    cc.stream = st;
    if (sparse) {
      cc.v_idx = (const int32_t*)(slot(c) + L.vidx_off);
      cc.s_off = (const int32_t*)(slot(c) + L.soff_off);
    }
    cc.lse_out = cfg->lse_out ? (float*)(slot(c) + L.lse_off) : nullptr;
    cc.cover_pairs = plan->cover_pairs ? plan->cover_pairs + c : nullptr;
    record_opt(plan->chunk_events, 2 * c, st);
    if (overlap && hipStreamWaitEvent(st, idx_done[c], 0) != hipSuccess) return DCA_EHIP;
    const size_t kv0 = (size_t)b[c] * cfg->h_kv * D;
    rc = paged ? dca_paged_append(k + kv0, v + kv0, b[c], n_q, &cc, paged)
               : dca_key_cache_append(k + kv0, b[c], n_q, &cc, cache);
    if (rc != DCA_OK) return rc;
    rc = dca::prefill_impl(q + (size_t)b[c] * h_q * D, nullptr, cache, paged, paged ? nullptr : v, nullptr, &cc,
                           out + (size_t)b[c] * h_q * D);
    if (rc != DCA_OK) return rc;
    if (cfg->lse_out) {
      // the chunk's [h_q][n_q] block into columns b_c .. b_{c+1}-1 of [h_q][n]
      if (hipMemcpy2DAsync(cfg->lse_out + b[c], (size_t)cfg->n_k * 4, cc.lse_out, (size_t)n_q * 4, (size_t)n_q * 4,
                           h_q, hipMemcpyDeviceToDevice, st) != hipSuccess)
        return DCA_EHIP;
    }
    record_opt(plan->chunk_events, 2 * c + 1, st);
    if (overlap && hipEventRecord(chunk_done[c], st) != hipSuccess) return DCA_EHIP;
  }
  return DCA_OK;
}

int dca_prefill_sequence(const dca_bf16* q, const dca_bf16* k, const dca_bf16* v, const dca_sequence_plan* plan,
                         const dca_cfg* cfg, const dca_key_cache* cache, dca_bf16* out) {
  if (!cache) return DCA_EINVAL;
  return sequence_impl(q, k, v, plan, cfg, cache, nullptr, out);
}

int dca_prefill_sequence_paged_workspace_size(const dca_cfg* cfg, const dca_sequence_plan* plan, size_t* bytes) {
  if (!bytes) return DCA_EINVAL;
  SeqLayout L;
  const int rc = seq_layout(cfg, plan, &L, true);
  if (rc != DCA_OK) return rc;
  *bytes = L.total;
  return DCA_OK;
}

int dca_prefill_sequence_paged(const dca_bf16* q, const dca_bf16* k, const dca_bf16* v, const dca_sequence_plan* plan,
                               const dca_cfg* cfg, const dca_paged_kv* cache, dca_bf16* out) {
  if (!cache) return DCA_EINVAL;
  return sequence_impl(q, k, v, plan, cfg, nullptr, cache, out);
}

}  // extern "C"
