// C ABI of the DCA sparse prefill library: validation, workspace layout and
// launch sequences.  Declared in include/dcasparse.h.
#include <cmath>
#include <algorithm>
#include <cstring>
#include <mutex>

#include "../../include/dcasparse.h"
#include "entry.h"
#include "args.h"
#include "common.h"

namespace dca {

hipError_t launch_rotate_keys(const uint16_t* k, uint16_t* khi, uint16_t* klo, uint32_t* kbits,
                              const Freqs& f, int j0, int n, int h_kv, int S, float thr2, int kbits_words,
                              bool clear_all, hipStream_t stream);
hipError_t launch_hn_next(const uint32_t* kbits, uint8_t* hn, int n_pad, int h_kv, int kbits_words,
                          hipStream_t stream);
hipError_t launch_paged_gather(const uint16_t* khi_p, const uint16_t* klo_p, const uint16_t* v_p,
                               const uint32_t* flags_p, const int32_t* ptab, int page_keys, int n_pages, int n_table,
                               int n_k, int h_kv, int kbits_words, uint16_t* khi, uint16_t* klo, uint16_t* vd,
                               uint32_t* kbits, hipStream_t stream);
hipError_t launch_hn_list(const uint32_t* kbits, int kbits_words, int n_k, int h_kv, int32_t* hnl_n, int32_t* hnall,
                          hipStream_t stream);
hipError_t launch_rotate_queries(const uint16_t* q, uint16_t* qhi, uint16_t* qlo, const double* inv_freq,
                                 int n_q, int h_q, int p0, int S, int W, float qscale, hipStream_t stream);
hipError_t launch_attn(const AttnArgs& A, hipStream_t stream);
hipError_t launch_lse_merge(const uint16_t* part_o, const float* part_lse, uint16_t* out, float* lse_out,
                            int P, int n_q, int h_q, const int32_t* bad, hipStream_t stream);
hipError_t launch_vs_score(const VsArgs& A, const uint16_t* q, int n_q, hipStream_t stream);
hipError_t launch_select(const SelArgs& A, hipStream_t stream);
hipError_t launch_plan(const PlanArgs& A, hipStream_t stream);
hipError_t launch_decode_attn(const DecArgs& A, hipStream_t stream);
hipError_t launch_rotate_keys_paged(const uint16_t* k, const uint16_t* v, uint16_t* khi, uint16_t* klo,
                                    uint16_t* vpool, uint32_t* kflags, const int32_t* ptab, int page_keys,
                                    int n_pages, const Freqs& f, int j0, int n, int h_kv, int S, float thr2,
                                    hipStream_t stream);
hipError_t launch_decode_merge(const DecArgs& A, uint16_t* out, float* lse_out, hipStream_t stream);

}  // namespace dca

namespace {

using namespace dca;

__global__ void write_freqs_kernel(Freqs f, double* dst) { dst[threadIdx.x] = f.v[threadIdx.x]; }

// Dense calls: the cover and attended pair counts, known on the host.
__global__ void write_pairs_kernel(long long* cover, long long cover_v, long long* att, long long att_v,
                                   const int32_t* bad) {
  if (bad && *bad) return;
  if (cover) *cover = cover_v;
  if (att) *att = att_v;
}

// The device check of a call's positions: every entry must be p0 + i.  One
// workgroup; *bad (workspace) is rewritten by every checked call, and read by
// each kernel that writes a caller-visible output.
__global__ void __launch_bounds__(256) positions_check_kernel(const int32_t* pos, int n_q, int p0, int32_t* bad,
                                                              int32_t* status) {
  int wrong = 0;
  for (int i = threadIdx.x; i < n_q; i += blockDim.x) wrong |= (pos[i] != p0 + i);
  wrong = __syncthreads_or(wrong);
  if (threadIdx.x == 0) {
    *bad = wrong;
    if (status) *status = wrong ? DCA_EINVAL : DCA_OK;
  }
}

constexpr size_t ALIGN = 256;
inline size_t up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Region { size_t off = 0, bytes = 0; };

// words per (head, block) of the extra-vertical lists: E entries (the vertical
// columns the ranges miss, and up to HN_MOVE_CAP covered high-norm keys); with
// exact diagonals also a two-word row mask per entry after them (3E words)
int ext_stride(const dca_cfg* c) {
  const int e = (c->vs_k_vertical > 0 ? c->vs_k_vertical : 1) + HN_MOVE_CAP;
  return c->slash_exact ? 3 * e : e;
}

// Workspace layouts of the two entry points (regions are 256-byte aligned).
struct Layout {
  // shared
  Region freqs, flag;
  // prefill
  Region hnl_n, hnall, hnt, cov_pre;
  Region khi, klo, kbits, hn, qhi, qlo, iv, iv_pre, n_iv, cov, ext, n_ext, tiles, n_tiles, t_first, part_o, part_lse;
  Region dbits, vbits, smask;
  Region vg;             // values gathered from a paged pool
  int dbits_words = 0, vbits_words = 0;
  // index
  Region qs, part_ms, lse, vert, slash, edge, logits, trig, hist, prefix, krem, bcount;
  size_t prefill_bytes = 0, index_bytes = 0;
  int hnt_words = 0;
  int split = 1, nb = 0, n_ranges = 0, range_keys = 0, cov_words = 0, max_blocks = 0, kbits_words = 0, hn_pad = 0,
      tile_stride = 0;
};

inline void place(Region& r, size_t& cur, size_t bytes) { r.off = cur; r.bytes = bytes; cur += up(bytes); }

// Host checks of a call.  The positions array lives in device memory and is
// checked by positions_check_kernel; the host checks p0 = n_k - n_q.
int validate(const dca_cfg* c) {
  if (!c) return DCA_EINVAL;
  if (c->n_q < 1 || c->n_k < 1 || c->h_q < 1 || c->h_kv < 1) return DCA_EINVAL;
  if (c->h_q % c->h_kv != 0) return DCA_EINVAL;
  if (c->n_k < c->n_q) return DCA_EINVAL;
  if (c->head_dim != 128) return DCA_EUNSUPPORTED;
  if (c->dca_chunk < 64 || c->dca_chunk % 64 != 0) return DCA_EUNSUPPORTED;
  if (c->dca_local < 1 || c->dca_local > c->dca_chunk) return DCA_EUNSUPPORTED;
  if (!(c->rope_base > 1.0) || !std::isfinite(c->rope_base)) return DCA_EINVAL;
  if (!(c->yarn_s > 0.0) || !std::isfinite(c->yarn_s)) return DCA_EINVAL;
  if (c->vs_k_vertical < 0 || c->vs_k_slash < 0) return DCA_EINVAL;
  if (c->vs_last_q < 1 || c->vs_last_q > 64) return DCA_EUNSUPPORTED;
  if (c->split_k < 0 || c->split_k > 256) return DCA_EINVAL;
  if (!std::isfinite(c->precise_norm)) return DCA_EINVAL;
  if (c->slash_exact != 0 && c->slash_exact != 1) return DCA_EINVAL;
  // the chunk of rows must be the tail of the prefix, starting on a 64 boundary
  const long long p0 = (long long)c->n_k - c->n_q;
  if (p0 % 64 != 0) return DCA_EUNSUPPORTED;
  // int32 key and offset arithmetic inside the kernels
  if ((long long)c->n_k + 2LL * c->dca_chunk + 128 > (1LL << 30)) return DCA_EUNSUPPORTED;
  // K / V rows of one KV head are addressed by 32-bit byte offsets
  if ((long long)c->n_k * c->h_kv * c->head_dim * 2 >= (1LL << 32)) return DCA_EUNSUPPORTED;
  return DCA_OK;
}

Layout make_layout(const dca_cfg* c, bool paged = false) {
  Layout L;
  const int n_q = c->n_q, n_k = c->n_k, h_q = c->h_q, h_kv = c->h_kv;
  const int p_last = n_k - 1;
  L.nb = (n_q + 63) / 64;
  const int units = h_q * L.nb;
  if (c->split_k > 0) {
    L.split = c->split_k;
  } else {
    // enough independent work items to fill 256 compute units several times
    // over, and key shares of about 16K keys: the attention workgroups run
    // split part by split part, so the keys read by the work in flight stay
    // within one share (16K keys of K and V per KV head: 8 MiB) and are
    // served from the dies' caches rather than memory (from 64K keys on;
    // below that the keys fit the caches whole)
    L.split = 1;
    while (units * L.split < 2048 && L.split < 16) L.split *= 2;
    const int by_keys = n_k < 65536 ? 1 : (int)std::min<long long>(64, ((long long)n_k + 16383) / 16384);
    L.split = std::max(L.split, by_keys);
    const int tiles = (n_k + 63) / 64;
    while (L.split > 1 && L.split > tiles) L.split /= 2;
  }
  size_t cur = 0;
  place(L.freqs, cur, HALF * sizeof(double));
  place(L.flag, cur, sizeof(int32_t));
  const size_t base = cur;
  // --- prefill
  place(L.khi, cur, (size_t)n_k * h_kv * D * 2);
  place(L.klo, cur, (size_t)n_k * h_kv * D * 2);
  L.kbits_words = (n_k + 31) / 32 + 4;   // guard words: a tile reads the two words of each run
  place(L.kbits, cur, (size_t)h_kv * L.kbits_words * 4);
  L.hn_pad = (n_k + 128 + 3) / 4 * 4;   // runs may start up to 95 keys past n_k - 1
  place(L.hn, cur, (size_t)h_kv * L.hn_pad);
  place(L.hnl_n, cur, (size_t)h_kv * 4);
  place(L.hnall, cur, (size_t)h_kv * HN_MOVE_CAP * 4);
  place(L.qhi, cur, (size_t)3 * n_q * h_q * D * 2);
  place(L.qlo, cur, (size_t)3 * n_q * h_q * D * 2);
  place(L.iv, cur, (size_t)h_q * (c->vs_k_slash + 1) * 2 * 4);
  place(L.iv_pre, cur, (size_t)h_q * (c->vs_k_slash + 2) * 4);
  place(L.n_iv, cur, (size_t)h_q * 4);
  L.cov_words = (p_last + 64 + 31) / 32;
  place(L.cov, cur, (size_t)h_q * L.cov_words * 4);
  place(L.cov_pre, cur, (size_t)h_q * L.cov_words * 4);
  place(L.ext, cur, (size_t)h_q * L.nb * (size_t)ext_stride(c) * 4);
  place(L.n_ext, cur, (size_t)h_q * L.nb * 4);
  // range tiles of 32 covered offsets: every merged interval is at least 64 long
  L.tile_stride = 2 * (c->vs_k_slash + 1) + 1;
  place(L.tiles, cur, (size_t)h_q * L.tile_stride * 16);
  // bitmaps over a block's range tiles (one word past the last: the walk reads a tile ahead)
  L.hnt_words = (L.tile_stride + 31) / 32 + 1;
  place(L.hnt, cur, (size_t)h_q * L.nb * L.hnt_words * 4);
  place(L.n_tiles, cur, (size_t)h_q * 4);
  place(L.t_first, cur, (size_t)h_q * L.nb * 4);
  if (c->slash_exact) {
    // windows of up to 8 words start between bit 34 and bit p_last + 160
    L.dbits_words = (p_last + 160) / 32 + 9;
    // 2-word windows start at key bit a + 128, a <= n_k + 95
    L.vbits_words = (n_k + 254) / 32 + 3;
    place(L.dbits, cur, (size_t)h_q * L.dbits_words * 4);
    place(L.vbits, cur, (size_t)h_q * L.vbits_words * 4);
    place(L.smask, cur, (size_t)h_q * L.tile_stride * 64 * 4);
  }
  if (L.split > 1) {
    place(L.part_o, cur, (size_t)L.split * n_q * h_q * D * 2);
    place(L.part_lse, cur, (size_t)L.split * h_q * n_q * 4);
  }
  if (paged) place(L.vg, cur, (size_t)n_k * h_kv * D * 2);
  L.prefill_bytes = cur;
  // --- index (reuses the space after the frequencies)
  cur = base;
  long long target = 2048;
  long long rk = ((long long)n_k * h_q) / target;
  rk = (rk + 31) / 32 * 32;
  if (rk < 64) rk = 64;
  if (rk > 2048) rk = 2048;
  L.range_keys = (int)rk;
  L.n_ranges = (int)((n_k + rk - 1) / rk);
  place(L.qs, cur, (size_t)2 * h_q * 64 * D * 8);
  place(L.part_ms, cur, (size_t)h_q * L.n_ranges * 64 * 2 * 8);
  place(L.lse, cur, (size_t)h_q * 64 * 8);
  place(L.vert, cur, (size_t)h_q * n_k * 8);
  place(L.slash, cur, (size_t)h_q * (p_last + 1) * 8);
  place(L.edge, cur, (size_t)h_q * L.n_ranges * 2 * 64 * 2 * 8);
  place(L.logits, cur, (size_t)h_q * 64 * n_k * 8);
  place(L.trig, cur, (size_t)(c->dca_chunk / 8) * HALF * 16);
  place(L.hist, cur, (size_t)2 * h_q * 256 * 4);
  place(L.prefix, cur, (size_t)2 * h_q * 8);
  place(L.krem, cur, (size_t)2 * h_q * 4);
  L.max_blocks = (n_k + 8191) / 8192;
  place(L.bcount, cur, (size_t)2 * h_q * L.max_blocks * 2 * 4);
  L.index_bytes = cur;
  return L;
}

// ---- generation step (decode)
int validate_decode(const dca_cfg* c) {
  if (!c) return DCA_EINVAL;
  if (c->n_q < 1 || c->n_k < c->n_q || c->h_q < 1 || c->h_kv < 1) return DCA_EINVAL;
  if (c->h_q % c->h_kv != 0) return DCA_EINVAL;
  if (c->n_q > 64) return DCA_EUNSUPPORTED;
  if (c->head_dim != 128) return DCA_EUNSUPPORTED;
  if (c->dca_chunk < 64 || c->dca_chunk % 64 != 0) return DCA_EUNSUPPORTED;
  if (c->dca_local < 1 || c->dca_local > c->dca_chunk) return DCA_EUNSUPPORTED;
  if (!(c->rope_base > 1.0) || !std::isfinite(c->rope_base)) return DCA_EINVAL;
  if (!(c->yarn_s > 0.0) || !std::isfinite(c->yarn_s)) return DCA_EINVAL;
  if (c->v_idx || c->s_off) return DCA_EINVAL;
  if (c->split_k < 0 || c->split_k > 4096) return DCA_EINVAL;
  if ((long long)c->n_k + 2LL * c->dca_chunk + 128 > (1LL << 30)) return DCA_EUNSUPPORTED;
  if ((long long)c->n_k * c->h_kv * c->head_dim * 2 >= (1LL << 32)) return DCA_EUNSUPPORTED;
  return DCA_OK;
}

struct DecLayout {
  Region freqs, qhi, qlo, part_o, part_lse;
  int n_cb = 1, part_keys = 32, n_parts = 1;
  size_t bytes = 0;
};

DecLayout make_dec_layout(const dca_cfg* c) {
  DecLayout L;
  const int G = c->h_q / c->h_kv;
  L.n_cb = (c->n_q * G + 31) / 32;
  long long pk;
  if (c->split_k > 0) {
    pk = ((long long)c->n_k + c->split_k - 1) / c->split_k;
  } else {
    // about 2048 one-wave workgroups: two per SIMD of the 256 compute units
    pk = ((long long)c->n_k * c->h_kv * L.n_cb + 2047) / 2048;
    pk = std::max(pk, 256LL);
  }
  pk = (pk + 31) / 32 * 32;
  L.part_keys = (int)pk;
  L.n_parts = (int)((c->n_k + pk - 1) / pk);
  size_t cur = 0;
  place(L.freqs, cur, HALF * sizeof(double));
  place(L.qhi, cur, (size_t)3 * c->n_q * c->h_q * D * 2);
  place(L.qlo, cur, (size_t)3 * c->n_q * c->h_q * D * 2);
  place(L.part_o, cur, (size_t)L.n_parts * c->n_q * c->h_q * D * 4);
  place(L.part_lse, cur, (size_t)L.n_parts * c->h_q * c->n_q * 4);
  L.bytes = cur;
  return L;
}

template <class T>
T* at(const dca_cfg* c, const Region& r) { return (T*)((char*)c->workspace + r.off); }

int check_workspace(const dca_cfg* c, size_t need) {
  if (!c->workspace) return DCA_EWORKSPACE;
  if (c->workspace_bytes < need) return DCA_EWORKSPACE;
  if (((uintptr_t)c->workspace) % ALIGN != 0) return DCA_EWORKSPACE;
  return DCA_OK;
}

Freqs make_freqs(double base) {
  Freqs f;
  for (int k = 0; k < HALF; ++k) f.v[k] = std::pow(base, -(2.0 * k) / (double)D);
  return f;
}

double yarn_factor(double s) {
  if (s <= 1.0) return 1.0;
  const double r = 0.1 * std::log(s) + 1.0;
  return r * r;
}

void record(const dca_cfg* c, int stage, int which) {
  if (!c->stage_events) return;
  hipEvent_t ev = (hipEvent_t)c->stage_events[2 * stage + which];
  if (ev) (void)hipEventRecord(ev, (hipStream_t)c->stream);
}

}  // namespace

extern "C" {

int dca_workspace_size(const dca_cfg* cfg, size_t* bytes) {
  if (!bytes) return DCA_EINVAL;
  const int rc = validate(cfg);
  if (rc != DCA_OK) return rc;
  const Layout L = make_layout(cfg);
  *bytes = L.prefill_bytes > L.index_bytes ? L.prefill_bytes : L.index_bytes;
  return DCA_OK;
}

int vs_index_build(const dca_bf16* q, const dca_bf16* k, const int32_t* positions, const dca_cfg* cfg,
                   int32_t* v_idx, int32_t* s_off) {
  if (!positions) return DCA_EINVAL;
  return dca::index_impl(q, k, positions, cfg, v_idx, s_off);
}

}  // extern "C"

namespace dca {

// The index build of one chunk; positions == nullptr: implied (p0 + i), not checked.
int index_impl(const dca_bf16* q, const dca_bf16* k, const int32_t* positions, const dca_cfg* cfg,
               int32_t* v_idx, int32_t* s_off) {
  int rc = validate(cfg);
  if (rc != DCA_OK) return rc;
  if (!q || !k) return DCA_EINVAL;
  if ((cfg->vs_k_vertical > 0 && !v_idx) || (cfg->vs_k_slash > 0 && !s_off)) return DCA_EINVAL;
  const Layout L = make_layout(cfg);
  rc = check_workspace(cfg, L.index_bytes);
  if (rc != DCA_OK) return rc;
  hipStream_t st = (hipStream_t)cfg->stream;
  const int n_q = cfg->n_q, n_k = cfg->n_k, h_q = cfg->h_q;
  const int p_last = n_k - 1;
  const int n_s = cfg->vs_last_q < n_q ? cfg->vs_last_q : n_q;
  int32_t* bad = nullptr;
  if (positions) {
    bad = at<int32_t>(cfg, L.flag);
    hipLaunchKernelGGL(positions_check_kernel, dim3(1), dim3(256), 0, st, positions, n_q, n_k - n_q, bad,
                       cfg->status);
  }

  hipLaunchKernelGGL(write_freqs_kernel, dim3(1), dim3(HALF), 0, st, make_freqs(cfg->rope_base),
                     at<double>(cfg, L.freqs));
  VsArgs V;
  V.k = k;
  V.qs = at<double>(cfg, L.qs);
  V.inv_freq = at<double>(cfg, L.freqs);
  V.part_ms = at<double>(cfg, L.part_ms);
  V.lse = at<double>(cfg, L.lse);
  V.vert = at<double>(cfg, L.vert);
  V.slash = at<double>(cfg, L.slash);
  V.edge = at<double>(cfg, L.edge);
  V.logits = at<double>(cfg, L.logits);
  V.trig = at<double2>(cfg, L.trig);
  V.n_k = n_k; V.h_q = h_q; V.h_kv = cfg->h_kv; V.S = cfg->dca_chunk; V.n_s = n_s;
  V.p_first = p_last - n_s + 1; V.range_keys = L.range_keys; V.n_ranges = L.n_ranges; V.n_off = p_last + 1;
  V.scale = yarn_factor(cfg->yarn_s) / std::sqrt((double)D);
  if (launch_vs_score(V, q, n_q, st) != hipSuccess) return DCA_EHIP;

  SelArgs S;
  S.vert = V.vert; S.slash = V.slash;
  S.v_out = v_idx; S.s_out = s_off;
  S.h_q = h_q; S.n_v = n_k; S.n_sl = p_last + 1; S.k_v = cfg->vs_k_vertical; S.k_s = cfg->vs_k_slash;
  S.hist = at<uint32_t>(cfg, L.hist);
  S.prefix = at<uint64_t>(cfg, L.prefix);
  S.krem = at<int32_t>(cfg, L.krem);
  S.bcount = at<uint32_t>(cfg, L.bcount);
  S.max_blocks = L.max_blocks;
  S.k_head = cfg->vs_k_per_head;
  S.bad = bad;
  if (launch_select(S, st) != hipSuccess) return DCA_EHIP;
  return DCA_OK;
}

}  // namespace dca

namespace {
int paged_check(const dca_paged_kv* c, int h_kv, int head_dim);
}  // namespace

namespace dca {

int paged_valid(const dca_paged_kv* cache, int h_kv, int head_dim) { return paged_check(cache, h_kv, head_dim); }

int paged_prefill_bytes(const dca_cfg* cfg, size_t* bytes) {
  if (!bytes) return DCA_EINVAL;
  const int rc = validate(cfg);
  if (rc != DCA_OK) return rc;
  const Layout L = make_layout(cfg, true);
  *bytes = L.prefill_bytes > L.index_bytes ? L.prefill_bytes : L.index_bytes;
  return DCA_OK;
}

// The prefill of one chunk.  Keys come raw (k: rotated here into the
// workspace), from a rotated key cache (cache: rotated when they entered it)
// or from a paged pool (paged: its keys, values and flags are gathered into
// the workspace first, a coalesced copy of the sequence's pages).
// positions == nullptr: implied (p0 + i), not checked.
int prefill_impl(const dca_bf16* q, const dca_bf16* k, const dca_key_cache* cache, const dca_paged_kv* paged,
                 const dca_bf16* v, const int32_t* positions, const dca_cfg* cfg, dca_bf16* out) {
  int rc = validate(cfg);
  if (rc != DCA_OK) return rc;
  if (!q || !(k || cache || paged) || !(v || paged) || !out) return DCA_EINVAL;
  if (cache) {
    if (!cache->k_hi || !cache->k_lo || !cache->k_flags || cache->capacity < cfg->n_k) return DCA_EINVAL;
    if ((long long)cache->capacity * cfg->h_kv * cfg->head_dim * 2 >= (1LL << 32)) return DCA_EUNSUPPORTED;
  }
  if (paged) {
    rc = paged_check(paged, cfg->h_kv, cfg->head_dim);
    if (rc != DCA_OK) return rc;
    if ((long long)paged->n_table * paged->page_keys < cfg->n_k) return DCA_EINVAL;
  }
  const bool sparse = cfg->v_idx || cfg->s_off;
  if (sparse && ((cfg->vs_k_vertical > 0 && !cfg->v_idx) || (cfg->vs_k_slash > 0 && !cfg->s_off)))
    return DCA_EINVAL;
  const Layout L = make_layout(cfg, paged != nullptr);
  rc = check_workspace(cfg, L.prefill_bytes);
  if (rc != DCA_OK) return rc;
  hipStream_t st = (hipStream_t)cfg->stream;
  const int n_q = cfg->n_q, n_k = cfg->n_k, h_q = cfg->h_q, h_kv = cfg->h_kv;
  const int p0 = n_k - n_q;
  const int p_last = n_k - 1;

  int32_t* bad = nullptr;
  if (positions) {
    bad = at<int32_t>(cfg, L.flag);
    hipLaunchKernelGGL(positions_check_kernel, dim3(1), dim3(256), 0, st, positions, n_q, p0, bad, cfg->status);
  }
  hipLaunchKernelGGL(write_freqs_kernel, dim3(1), dim3(HALF), 0, st, make_freqs(cfg->rope_base),
                     at<double>(cfg, L.freqs));
  // rotated keys and their high-norm bits: this call's own rotation, or the cache's
  const uint16_t* khi = cache ? cache->k_hi : at<uint16_t>(cfg, L.khi);
  const uint16_t* klo = cache ? cache->k_lo : at<uint16_t>(cfg, L.klo);
  const uint32_t* kbits = cache ? cache->k_flags : at<uint32_t>(cfg, L.kbits);
  const int kbits_words = cache ? (cache->capacity + 31) / 32 : L.kbits_words;
  // stage 0: chunk-local key rotation (or the gather from the pages), query rotations of the three DCA modes
  record(cfg, 0, 0);
  if (paged) {
    if (launch_paged_gather(paged->k_hi, paged->k_lo, paged->v, paged->k_flags, paged->page_table,
                            paged->page_keys, paged->n_pages, paged->n_table, n_k, h_kv, L.kbits_words,
                            at<uint16_t>(cfg, L.khi), at<uint16_t>(cfg, L.klo), at<uint16_t>(cfg, L.vg),
                            at<uint32_t>(cfg, L.kbits), st) != hipSuccess)
      return DCA_EHIP;
    v = at<uint16_t>(cfg, L.vg);
  } else if (!cache) {
    float thr = cfg->precise_norm == 0.f ? 2.f * std::sqrt((float)D) : cfg->precise_norm;
    const float thr2 = thr < 0.f ? -1.f : thr * thr;
    if (launch_rotate_keys(k, at<uint16_t>(cfg, L.khi), at<uint16_t>(cfg, L.klo), at<uint32_t>(cfg, L.kbits),
                           make_freqs(cfg->rope_base), 0, n_k, h_kv, cfg->dca_chunk, thr2, L.kbits_words, true,
                           st) != hipSuccess)
      return DCA_EHIP;
  }
  if (launch_hn_next(kbits, at<uint8_t>(cfg, L.hn), L.hn_pad, h_kv, kbits_words, st) != hipSuccess)
    return DCA_EHIP;
  if (launch_hn_list(kbits, kbits_words, n_k, h_kv, at<int32_t>(cfg, L.hnl_n), at<int32_t>(cfg, L.hnall), st) !=
      hipSuccess)
    return DCA_EHIP;
  // softmax scale sqrt(1/t)^2 / sqrt(d) and log2(e) (the kernel works in base 2)
  const float qscale = (float)(yarn_factor(cfg->yarn_s) / std::sqrt((double)D) * 1.4426950408889634);
  if (launch_rotate_queries(q, at<uint16_t>(cfg, L.qhi), at<uint16_t>(cfg, L.qlo), at<double>(cfg, L.freqs), n_q,
                            h_q, p0, cfg->dca_chunk, cfg->dca_local, qscale, st) != hipSuccess)
    return DCA_EHIP;
  record(cfg, 0, 1);
  // stage 1: sparse plan
  record(cfg, 1, 0);
  if (sparse) {
    PlanArgs P;
    P.v_idx = cfg->v_idx; P.s_off = cfg->s_off;
    P.iv = at<int32_t>(cfg, L.iv); P.iv_pre = at<int32_t>(cfg, L.iv_pre); P.n_iv = at<int32_t>(cfg, L.n_iv);
    P.cover_pairs = (long long*)cfg->cover_pairs;
    P.cov = at<uint32_t>(cfg, L.cov); P.cov_pre = at<int32_t>(cfg, L.cov_pre);
    P.ext = at<int32_t>(cfg, L.ext); P.n_ext = at<int32_t>(cfg, L.n_ext);
    P.h_q = h_q; P.k_v = cfg->vs_k_vertical; P.k_s = cfg->vs_k_slash; P.p_last = p_last; P.p0 = p0;
    P.n_q = n_q; P.nb = L.nb; P.iv_stride = cfg->vs_k_slash + 1;
    P.ext_stride = ext_stride(cfg); P.cov_words = L.cov_words;
    P.tiles = at<int4>(cfg, L.tiles); P.n_tiles = at<int32_t>(cfg, L.n_tiles); P.t_first = at<int32_t>(cfg, L.t_first);
    P.kbits = kbits; P.h_kv = h_kv; P.tile_stride = L.tile_stride;
    P.kbits_words = kbits_words;
    P.dbits = cfg->slash_exact ? at<uint32_t>(cfg, L.dbits) : nullptr;
    P.vbits = cfg->slash_exact ? at<uint32_t>(cfg, L.vbits) : nullptr;
    P.smask = cfg->slash_exact ? at<uint32_t>(cfg, L.smask) : nullptr;
    P.dbits_words = L.dbits_words; P.vbits_words = L.vbits_words;
    P.attended = (long long*)cfg->attended_pairs;
    P.bad = bad;
    P.hnl_n = at<int32_t>(cfg, L.hnl_n); P.hnall = at<int32_t>(cfg, L.hnall);
    P.hnt = at<uint32_t>(cfg, L.hnt); P.hnt_words = L.hnt_words;
    P.S = cfg->dca_chunk;
    if (launch_plan(P, st) != hipSuccess) return DCA_EHIP;
  } else if (cfg->cover_pairs || cfg->attended_pairs) {
    // dense: every block covers its whole causal extent [0, i0 + rows); row i attends p_i + 1 keys
    long long pairs = 0;
    for (int b = 0; b < L.nb; ++b) {
      const long long rows = std::min(64, n_q - 64 * b);
      pairs += rows * (long long)(p0 + 64 * b + rows);
    }
    const long long att = ((long long)n_k * (n_k + 1) / 2 - (long long)p0 * (p0 + 1) / 2) * h_q;
    hipLaunchKernelGGL(write_pairs_kernel, dim3(1), dim3(1), 0, st, (long long*)cfg->cover_pairs, pairs * h_q,
                       (long long*)cfg->attended_pairs, att, bad);
  }
  record(cfg, 1, 1);
  // stage 2: attention
  record(cfg, 2, 0);
  AttnArgs A;
  A.qhi = at<uint16_t>(cfg, L.qhi); A.qlo = at<uint16_t>(cfg, L.qlo);
  A.khi = khi; A.klo = klo; A.v = v;
  A.kbits = kbits; A.hn = at<uint8_t>(cfg, L.hn); A.hn_pad = L.hn_pad;
  A.out = out; A.lse_out = cfg->lse_out;
  A.part_o = L.split > 1 ? at<uint16_t>(cfg, L.part_o) : nullptr;
  A.part_lse = L.split > 1 ? at<float>(cfg, L.part_lse) : nullptr;
  A.tiles = at<int4>(cfg, L.tiles); A.n_tiles = at<int32_t>(cfg, L.n_tiles); A.t_first = at<int32_t>(cfg, L.t_first);
  A.ext = at<int32_t>(cfg, L.ext); A.n_ext = at<int32_t>(cfg, L.n_ext);
  A.n_q = n_q; A.n_k = n_k; A.h_q = h_q; A.h_kv = h_kv; A.p0 = p0; A.S = cfg->dca_chunk; A.W = cfg->dca_local;
  A.nb = L.nb; A.tile_stride = L.tile_stride; A.kbits_words = kbits_words;
  A.ext_stride = ext_stride(cfg);
  A.split = L.split; A.dense = sparse ? 0 : 1;
  A.exact = (sparse && cfg->slash_exact) ? 1 : 0;
  A.dbits = A.exact ? at<uint32_t>(cfg, L.dbits) : nullptr;
  A.vbits = A.exact ? at<uint32_t>(cfg, L.vbits) : nullptr;
  A.smask = A.exact ? at<uint32_t>(cfg, L.smask) : nullptr;
  A.dbits_words = L.dbits_words; A.vbits_words = L.vbits_words;
  A.bad = bad;
  A.hnl_n = at<int32_t>(cfg, L.hnl_n);
  A.hnt = sparse ? at<uint32_t>(cfg, L.hnt) : nullptr; A.hnt_words = L.hnt_words;
  if (launch_attn(A, st) != hipSuccess) return DCA_EHIP;
  record(cfg, 2, 1);
  // stage 3: LSE merge of the split partials
  record(cfg, 3, 0);
  if (L.split > 1) {
    if (launch_lse_merge(A.part_o, A.part_lse, out, cfg->lse_out, L.split, n_q, h_q, bad, st) != hipSuccess)
      return DCA_EHIP;
  }
  record(cfg, 3, 1);
  return DCA_OK;
}

}  // namespace dca

extern "C" {

int dca_sparse_prefill(const dca_bf16* q, const dca_bf16* k, const dca_bf16* v, const int32_t* positions,
                       const dca_cfg* cfg, dca_bf16* out) {
  if (!k || !positions) return DCA_EINVAL;
  return dca::prefill_impl(q, k, nullptr, nullptr, v, positions, cfg, out);
}

}  // extern "C"

// Scratch of the allocation-free prefill: one array per GPU (each device that
// runs the library holds its own copy until the process ends).  Host code never
// passes the array's name to a kernel: its device address is taken once per
// device with hipGetSymbolAddress and kept below.
static __device__ __align__(256) unsigned char scratch[DCA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// device address of the current device's scratch array
int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DCA_EHIP;
  if (dev < 0 || dev >= MAX_DEVICES) return DCA_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DCA_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DCA_OK;
}

}  // namespace

extern "C" {

int dca_sparse_prefill_noalloc(const dca_bf16* q, const dca_bf16* k, const dca_bf16* v, const int32_t* positions,
                               const dca_cfg* cfg, dca_bf16* out) {
  if (!cfg || !k || !positions) return DCA_EINVAL;
  int rc = validate(cfg);
  if (rc != DCA_OK) return rc;
  if (make_layout(cfg).prefill_bytes > (size_t)DCA_STATIC_SCRATCH_BYTES) return DCA_ESCRATCH;
  void* ws = nullptr;
  rc = static_scratch(&ws);
  if (rc != DCA_OK) return rc;
  dca_cfg c = *cfg;
  c.workspace = ws;
  c.workspace_bytes = DCA_STATIC_SCRATCH_BYTES;
  return dca::prefill_impl(q, k, nullptr, nullptr, v, positions, &c, out);
}

int dca_sparse_prefill_cached(const dca_bf16* q, const dca_key_cache* cache, const dca_bf16* v,
                              const int32_t* positions, const dca_cfg* cfg, dca_bf16* out) {
  if (!cache || !positions) return DCA_EINVAL;
  return dca::prefill_impl(q, nullptr, cache, nullptr, v, positions, cfg, out);
}

int dca_paged_prefill_workspace_size(const dca_cfg* cfg, size_t* bytes) { return dca::paged_prefill_bytes(cfg, bytes); }

int dca_sparse_prefill_paged(const dca_bf16* q, const dca_paged_kv* cache, const int32_t* positions, const dca_cfg* cfg,
                             dca_bf16* out) {
  if (!cache || !positions) return DCA_EINVAL;
  return dca::prefill_impl(q, nullptr, nullptr, cache, nullptr, positions, cfg, out);
}

int dca_key_cache_append(const dca_bf16* k, int32_t j0, int32_t n, const dca_cfg* cfg, const dca_key_cache* cache) {
  if (!cfg || !cache || !k) return DCA_EINVAL;
  if (!cache->k_hi || !cache->k_lo || !cache->k_flags || cache->capacity < 1) return DCA_EINVAL;
  if (cfg->h_kv < 1) return DCA_EINVAL;
  if (cfg->head_dim != 128) return DCA_EUNSUPPORTED;
  if (cfg->dca_chunk < 64 || cfg->dca_chunk % 64 != 0) return DCA_EUNSUPPORTED;
  if (!(cfg->rope_base > 1.0) || !std::isfinite(cfg->rope_base)) return DCA_EINVAL;
  if (!std::isfinite(cfg->precise_norm)) return DCA_EINVAL;
  if (j0 < 0 || n < 1 || (long long)j0 + n > cache->capacity) return DCA_EINVAL;
  if ((long long)cache->capacity + 2LL * cfg->dca_chunk + 128 > (1LL << 30)) return DCA_EUNSUPPORTED;
  if ((long long)cache->capacity * cfg->h_kv * cfg->head_dim * 2 >= (1LL << 32)) return DCA_EUNSUPPORTED;
  const float thr = cfg->precise_norm == 0.f ? 2.f * std::sqrt((float)D) : cfg->precise_norm;
  const float thr2 = thr < 0.f ? -1.f : thr * thr;
  const int words = (cache->capacity + 31) / 32;
  if (launch_rotate_keys(k, cache->k_hi, cache->k_lo, cache->k_flags, make_freqs(cfg->rope_base), j0, n, cfg->h_kv,
                         cfg->dca_chunk, thr2, words, false, (hipStream_t)cfg->stream) != hipSuccess)
    return DCA_EHIP;
  return DCA_OK;
}

int dca_decode_workspace_size(const dca_cfg* cfg, size_t* bytes) {
  if (!bytes) return DCA_EINVAL;
  const int rc = validate_decode(cfg);
  if (rc != DCA_OK) return rc;
  *bytes = make_dec_layout(cfg).bytes;
  return DCA_OK;
}

}  // extern "C"

namespace {

int paged_check(const dca_paged_kv* c, int h_kv, int head_dim) {
  if (!c || !c->k_hi || !c->k_lo || !c->v || !c->k_flags || !c->page_table) return DCA_EINVAL;
  if (c->n_pages < 1 || c->n_table < 1) return DCA_EINVAL;
  if (c->page_keys < 32 || c->page_keys % 32) return DCA_EUNSUPPORTED;
  if ((long long)c->n_pages * c->page_keys * h_kv * head_dim * 2 >= (1LL << 32)) return DCA_EUNSUPPORTED;
  if ((long long)c->n_table * c->page_keys >= (1LL << 30)) return DCA_EUNSUPPORTED;
  return DCA_OK;
}

// The generation step over a contiguous cache (paged == nullptr) or a paged pool.
int decode_impl(const dca_bf16* q, const dca_key_cache* cache, const dca_paged_kv* paged, const dca_bf16* v,
                const dca_cfg* cfg, dca_bf16* out) {
  int rc = validate_decode(cfg);
  if (rc != DCA_OK) return rc;
  if (!q || !out) return DCA_EINVAL;
  if (paged) {
    rc = paged_check(paged, cfg->h_kv, cfg->head_dim);
    if (rc != DCA_OK) return rc;
    if ((long long)paged->n_table * paged->page_keys < cfg->n_k) return DCA_EINVAL;
  } else {
    if (!cache || !v) return DCA_EINVAL;
    if (!cache->k_hi || !cache->k_lo || !cache->k_flags || cache->capacity < cfg->n_k) return DCA_EINVAL;
    if ((long long)cache->capacity * cfg->h_kv * cfg->head_dim * 2 >= (1LL << 32)) return DCA_EUNSUPPORTED;
  }
  const DecLayout L = make_dec_layout(cfg);
  rc = check_workspace(cfg, L.bytes);
  if (rc != DCA_OK) return rc;
  hipStream_t st = (hipStream_t)cfg->stream;
  const int n_t = cfg->n_q, n_k = cfg->n_k, h_q = cfg->h_q;
  record(cfg, 0, 0);
  hipLaunchKernelGGL(write_freqs_kernel, dim3(1), dim3(HALF), 0, st, make_freqs(cfg->rope_base),
                     at<double>(cfg, L.freqs));
  const float qscale = (float)(yarn_factor(cfg->yarn_s) / std::sqrt((double)D) * 1.4426950408889634);
  if (launch_rotate_queries(q, at<uint16_t>(cfg, L.qhi), at<uint16_t>(cfg, L.qlo), at<double>(cfg, L.freqs), n_t,
                            h_q, n_k - n_t, cfg->dca_chunk, cfg->dca_local, qscale, st) != hipSuccess)
    return DCA_EHIP;
  record(cfg, 0, 1);
  record(cfg, 1, 0);
  record(cfg, 1, 1);
  DecArgs A;
  A.qhi = at<uint16_t>(cfg, L.qhi); A.qlo = at<uint16_t>(cfg, L.qlo);
  if (paged) {
    A.khi = paged->k_hi; A.klo = paged->k_lo; A.kflags = paged->k_flags; A.v = paged->v;
    A.ptab = paged->page_table; A.page_keys = paged->page_keys; A.n_pages = paged->n_pages;
    A.kflag_words = 0;
  } else {
    A.khi = cache->k_hi; A.klo = cache->k_lo; A.kflags = cache->k_flags; A.v = v;
    A.ptab = nullptr; A.page_keys = 32; A.n_pages = 1;
    A.kflag_words = (cache->capacity + 31) / 32;
  }
  A.part_o = at<float>(cfg, L.part_o); A.part_lse = at<float>(cfg, L.part_lse);
  A.n_t = n_t; A.n_k = n_k; A.h_q = h_q; A.h_kv = cfg->h_kv; A.S = cfg->dca_chunk;
  A.part_keys = L.part_keys; A.n_parts = L.n_parts; A.n_cb = L.n_cb;
  record(cfg, 2, 0);
  if (launch_decode_attn(A, st) != hipSuccess) return DCA_EHIP;
  record(cfg, 2, 1);
  record(cfg, 3, 0);
  if (launch_decode_merge(A, out, cfg->lse_out, st) != hipSuccess) return DCA_EHIP;
  record(cfg, 3, 1);
  return DCA_OK;
}

}  // namespace

extern "C" {

int dca_decode(const dca_bf16* q, const dca_key_cache* cache, const dca_bf16* v, const dca_cfg* cfg, dca_bf16* out) {
  if (!cache) return DCA_EINVAL;
  return decode_impl(q, cache, nullptr, v, cfg, out);
}

int dca_decode_paged(const dca_bf16* q, const dca_paged_kv* cache, const dca_cfg* cfg, dca_bf16* out) {
  if (!cache) return DCA_EINVAL;
  return decode_impl(q, nullptr, cache, nullptr, cfg, out);
}

int dca_paged_append(const dca_bf16* k, const dca_bf16* v, int32_t j0, int32_t n, const dca_cfg* cfg,
                     const dca_paged_kv* cache) {
  if (!cfg || !cache || !k || !v) return DCA_EINVAL;
  if (cfg->h_kv < 1) return DCA_EINVAL;
  if (cfg->head_dim != 128) return DCA_EUNSUPPORTED;
  if (cfg->dca_chunk < 64 || cfg->dca_chunk % 64 != 0) return DCA_EUNSUPPORTED;
  if (!(cfg->rope_base > 1.0) || !std::isfinite(cfg->rope_base)) return DCA_EINVAL;
  if (!std::isfinite(cfg->precise_norm)) return DCA_EINVAL;
  int rc = paged_check(cache, cfg->h_kv, cfg->head_dim);
  if (rc != DCA_OK) return rc;
  if (j0 < 0 || n < 1 || (long long)j0 + n > (long long)cache->n_table * cache->page_keys) return DCA_EINVAL;
  const float thr = cfg->precise_norm == 0.f ? 2.f * std::sqrt((float)D) : cfg->precise_norm;
  const float thr2 = thr < 0.f ? -1.f : thr * thr;
  if (launch_rotate_keys_paged(k, v, cache->k_hi, cache->k_lo, cache->v, cache->k_flags, cache->page_table,
                               cache->page_keys, cache->n_pages, make_freqs(cfg->rope_base), j0, n, cfg->h_kv,
                               cfg->dca_chunk, thr2, (hipStream_t)cfg->stream) != hipSuccess)
    return DCA_EHIP;
  return DCA_OK;
}

const char* dca_strerror(int code) {
  switch (code) {
    case DCA_OK: return "ok";
    case DCA_EINVAL: return "invalid argument (null pointer, inconsistent sizes or positions)";
    case DCA_EUNSUPPORTED: return "unsupported configuration (head_dim, chunk, window, alignment or size)";
    case DCA_EWORKSPACE: return "workspace missing, misaligned or smaller than dca_workspace_size";
    case DCA_EHIP: return "HIP launch or runtime error";
    case DCA_ESCRATCH: return "the call needs more scratch than the allocation-free entry point holds";
    default: return "unknown error code";
  }
}

}  // extern "C"
