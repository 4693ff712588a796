// Top-k selection of vertical columns and slash offsets, and the sparse plan.
//
// Selection: the k best scores of each list by (score desc, index asc),
// emitted in ascending index order and padded with -1.  Scores are
// non-negative doubles, so their bit patterns order like the values; the k-th
// largest bit pattern T is found by an 8-pass radix select (8 bits per pass,
// integer histograms: deterministic), then every score above T and the
// lowest-index scores equal to T are compacted in index order.  Slash offset 0
// is forced in by ranking it as +inf.
//
// Plan: per query head, the selected offsets (plus 0) become disjoint key
// ranges in offset space, [-delta, -delta+64) merged when they touch; per
// query block, the vertical columns those ranges do not already cover are
// listed for the attention kernel.
#include "common.h"
#include "args.h"

namespace dca {

constexpr int SEL_CHUNK = 8192;           // list elements per histogram / compaction block
constexpr uint64_t FORCED_KEY = 0x7FF0000000000000ull;   // +inf


// List `list` (2h: vertical scores of head h, 2h+1: slash scores): scores s[n],
// output row out of length kcap, and the number k of picks (the head's own
// budget when per-head budgets are given, at most kcap).
__device__ __forceinline__ void sel_list(const SelArgs& A, int list, const double*& s, int32_t*& out, int& n,
                                         int& k, int& forced0, int& kcap) {
  const int h = list >> 1;
  if ((list & 1) == 0) {
    s = A.vert + (long long)h * A.n_v; out = A.v_out + (long long)h * A.k_v; n = A.n_v; kcap = A.k_v; forced0 = 0;
  } else {
    s = A.slash + (long long)h * A.n_sl; out = A.s_out + (long long)h * A.k_s; n = A.n_sl; kcap = A.k_s; forced0 = 1;
  }
  k = kcap;
  if (A.k_head) k = min(max(A.k_head[2 * h + (list & 1)], 0), kcap);
}
__device__ __forceinline__ void sel_list(const SelArgs& A, int list, const double*& s, int32_t*& out, int& n,
                                         int& k, int& forced0) {
  int kcap;
  sel_list(A, list, s, out, n, k, forced0, kcap);
}

__device__ __forceinline__ uint64_t sel_key(const double* s, int i, int forced0) {
  if (forced0 && i == 0) return FORCED_KEY;
  return (uint64_t)__double_as_longlong(s[i]);
}

__global__ void sel_init_kernel(SelArgs A) {
  const int list = blockIdx.x;
  const double* s; int32_t* out; int n, k, f;
  sel_list(A, list, s, out, n, k, f);
  A.hist[list * 256 + threadIdx.x] = 0;
  if (threadIdx.x == 0) { A.prefix[list] = 0; A.krem[list] = k; }
}

// Histogram of the byte at `shift` among elements whose higher bytes equal the prefix.
__global__ void __launch_bounds__(256) sel_hist_kernel(SelArgs A, int shift) {
  __shared__ uint32_t lh[256];
  const int list = blockIdx.y;
  const double* s; int32_t* out; int n, k, f;
  sel_list(A, list, s, out, n, k, f);
  lh[threadIdx.x] = 0;
  __syncthreads();
  const int beg = blockIdx.x * SEL_CHUNK;
  if (k > 0 && k < n && beg < n) {
    const uint64_t pre = A.prefix[list];
    const uint64_t mask = (shift >= 56) ? 0ull : (~0ull << (shift + 8));
    const int end = min(n, beg + SEL_CHUNK);
    for (int i = beg + threadIdx.x; i < end; i += 256) {
      const uint64_t key = sel_key(s, i, f);
      if ((key & mask) == pre) atomicAdd(&lh[(key >> shift) & 0xFF], 1u);
    }
  }
  __syncthreads();
  const uint32_t c = lh[threadIdx.x];
  if (c) atomicAdd(&A.hist[list * 256 + threadIdx.x], c);
}

// Pick the byte holding the k_rem-th largest key; clear the histogram for the next pass.
__global__ void sel_pick_kernel(SelArgs A, int shift) {
  __shared__ uint32_t hs[256];
  const int list = blockIdx.x;
  hs[threadIdx.x] = A.hist[list * 256 + threadIdx.x];
  A.hist[list * 256 + threadIdx.x] = 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double* s; int32_t* out; int n, k, f;
    sel_list(A, list, s, out, n, k, f);
    if (k > 0 && k < n) {
      int rem = A.krem[list];
      uint32_t above = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (above + hs[d] >= (uint32_t)rem) break;
        above += hs[d];
      }
      A.prefix[list] |= ((uint64_t)d) << shift;
      A.krem[list] = rem - (int)above;
    }
  }
}

// Per-block counts of keys above T and equal to T.
__global__ void __launch_bounds__(256) sel_count_kernel(SelArgs A) {
  __shared__ uint32_t cg[256], ce[256];
  const int list = blockIdx.y;
  const double* s; int32_t* out; int n, k, f;
  sel_list(A, list, s, out, n, k, f);
  const int beg = blockIdx.x * SEL_CHUNK;
  uint32_t ng = 0, ne = 0;
  if (beg < n) {
    const int end = min(n, beg + SEL_CHUNK);
    const uint64_t T = A.prefix[list];
    const bool all = (k >= n);
    for (int i = beg + threadIdx.x; i < end; i += 256) {
      const uint64_t key = sel_key(s, i, f);
      if (all || key > T) ++ng; else if (key == T) ++ne;
    }
  }
  cg[threadIdx.x] = ng; ce[threadIdx.x] = ne;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) { cg[threadIdx.x] += cg[threadIdx.x + off]; ce[threadIdx.x] += ce[threadIdx.x + off]; }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    uint32_t* dst = A.bcount + ((long long)list * A.max_blocks + blockIdx.x) * 2;
    dst[0] = cg[0]; dst[1] = ce[0];
  }
}

// Exclusive scan of the block counts (one thread per list; block counts are few).
__global__ void sel_scan_kernel(SelArgs A) {
  const int list = blockIdx.x * blockDim.x + threadIdx.x;
  if (list >= 2 * A.h_q) return;
  const double* s; int32_t* out; int n, k, f;
  sel_list(A, list, s, out, n, k, f);
  const int nb = (n + SEL_CHUNK - 1) / SEL_CHUNK;
  uint32_t g = 0, e = 0;
  for (int b = 0; b < nb; ++b) {
    uint32_t* p = A.bcount + ((long long)list * A.max_blocks + b) * 2;
    const uint32_t tg = p[0], te = p[1];
    p[0] = g; p[1] = e;
    g += tg; e += te;
  }
}

// Write selected indices in ascending order; the first block of each list pads with -1.
// Each wave owns a contiguous quarter of the block's elements and walks it 64
// at a time (coalesced reads); ballots give every lane the number of selected
// elements before it.  A pass of counts first gives each wave its start.
__global__ void __launch_bounds__(256) sel_write_kernel(SelArgs A) {
  __shared__ uint32_t wcg[4], wce[4];
  const int list = blockIdx.y;
  const double* s; int32_t* out; int n, k, f, kcap;
  sel_list(A, list, s, out, n, k, f, kcap);
  if (A.bad && *A.bad) return;   // positions check failed: v_idx / s_off keep their contents
  if (blockIdx.x == 0) {
    for (int i = min(k, n) + threadIdx.x; i < kcap; i += 256) out[i] = -1;
  }
  if (k <= 0) return;
  const int beg = blockIdx.x * SEL_CHUNK;
  const bool all = (k >= n);
  const uint64_t T = A.prefix[list];
  const uint32_t need_eq = all ? 0u : (uint32_t)A.krem[list];
  if (beg >= n) return;
  const int end = min(n, beg + SEL_CHUNK);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int w0 = beg + w * (SEL_CHUNK / 4);
  const int w1 = min(end, w0 + SEL_CHUNK / 4);
  const uint64_t below = (1ull << lane) - 1ull;
  auto classify = [&](int i, bool& g, bool& e) __attribute__((always_inline)) {
    g = false; e = false;
    if (i < w1) {
      const uint64_t key = sel_key(s, i, f);
      g = all || key > T;
      e = !g && key == T;
    }
  };
  uint32_t cg = 0, ce = 0;
  for (int i0 = w0; i0 < w1; i0 += 64) {
    bool g, e;
    classify(i0 + lane, g, e);
    cg += (uint32_t)__popcll(__ballot(g));
    ce += (uint32_t)__popcll(__ballot(e));
  }
  if (lane == 0) { wcg[w] = cg; wce[w] = ce; }
  __syncthreads();
  const uint32_t* bc = A.bcount + ((long long)list * A.max_blocks + blockIdx.x) * 2;
  uint32_t gb = bc[0], eb = bc[1];
  for (int u = 0; u < w; ++u) { gb += wcg[u]; eb += wce[u]; }
  for (int i0 = w0; i0 < w1; i0 += 64) {
    bool g, e;
    const int i = i0 + lane;
    classify(i, g, e);
    const uint64_t bg = __ballot(g), be = __ballot(e);
    const uint32_t g_before = gb + (uint32_t)__popcll(bg & below);
    const uint32_t e_before = eb + (uint32_t)__popcll(be & below);
    if (g) out[g_before + min(e_before, need_eq)] = i;
    else if (e && e_before < need_eq) out[g_before + e_before] = i;
    gb += (uint32_t)__popcll(bg);
    eb += (uint32_t)__popcll(be);
  }
}

hipError_t launch_select(const SelArgs& A, hipStream_t stream) {
  const int lists = 2 * A.h_q;
  const int nblk = (max(A.n_v, A.n_sl) + SEL_CHUNK - 1) / SEL_CHUNK;
  hipLaunchKernelGGL(sel_init_kernel, dim3(lists), dim3(256), 0, stream, A);
  for (int shift = 56; shift >= 0; shift -= 8) {
    hipLaunchKernelGGL(sel_hist_kernel, dim3(nblk, lists), dim3(256), 0, stream, A, shift);
    hipLaunchKernelGGL(sel_pick_kernel, dim3(lists), dim3(256), 0, stream, A, shift);
  }
  hipLaunchKernelGGL(sel_count_kernel, dim3(nblk, lists), dim3(256), 0, stream, A);
  hipLaunchKernelGGL(sel_scan_kernel, dim3((lists + 63) / 64), dim3(64), 0, stream, A);
  hipLaunchKernelGGL(sel_write_kernel, dim3(nblk, lists), dim3(256), 0, stream, A);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Sparse plan
// ---------------------------------------------------------------------------

// One workgroup (1024 threads) per head.  The selected offsets in descending
// order (ascending key offset -delta) with the forced 0 appended; out-of-range
// entries (padding -1, delta > p_last) are skipped.  An offset is kept when it
// lies strictly below the previous valid one (this drops duplicates and a
// forced 0 the list already held); a kept offset opens a new interval when
// the previous valid offset lies more than 64 above it, else it extends the
// current one.  Interval k is [-first kept, -last kept + 64).  Every quantity
// is a prefix scan over the list (1024 entries per pass, carries between
// passes); the covered-offset prefix iv_pre is a scan over the intervals.
__device__ __forceinline__ int scan1024_max(int x, int* wred) {   // inclusive max-scan over the block
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x = max(x, y);
  }
  if (lane == 63) wred[w] = x;
  __syncthreads();
  int pre = -1;
  for (int u = 0; u < w; ++u) pre = max(pre, wred[u]);
  __syncthreads();
  return max(x, pre);
}
__device__ __forceinline__ int scan1024_sum(int x, int* wred) {   // inclusive sum-scan over the block
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wred[w] = x;
  __syncthreads();
  int pre = 0;
  for (int u = 0; u < w; ++u) pre += wred[u];
  __syncthreads();
  return x + pre;
}

__global__ void __launch_bounds__(1024) plan_intervals_kernel(PlanArgs A) {
  __shared__ int32_t sd[1024];      // offsets of this pass (-1: skipped)
  __shared__ int32_t sx[1024];      // inclusive scan results, read back at tid - 1
  __shared__ int32_t wred[16];
  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const int32_t* so = A.s_off + (long long)h * A.k_s;
  int32_t* ivh = A.iv + (long long)h * A.iv_stride * 2;
  const int total = A.k_s + 1;
  int carry_valid = -1;   // last valid offset of the earlier passes
  int carry_kept = -1;    // last kept offset of the earlier passes
  int carry_count = 0;    // intervals opened in the earlier passes
  for (int base = 0; base < total; base += 1024) {
    const int t = base + tid;
    int d = -1;
    if (t < A.k_s) d = so[A.k_s - 1 - t];
    else if (t == A.k_s) d = 0;
    if (d < 0 || d > A.p_last) d = -1;
    sd[tid] = d;
    // previous valid offset
    const int vi = scan1024_max(d >= 0 ? tid : -1, wred);
    sx[tid] = vi;
    __syncthreads();
    const int pv_i = tid > 0 ? sx[tid - 1] : -1;
    const int prev = pv_i >= 0 ? sd[pv_i] : carry_valid;
    const bool keep = d >= 0 && (prev < 0 || d < prev);
    const bool start = keep && (prev < 0 || prev - d > 64);
    __syncthreads();
    // previous kept offset
    const int ki = scan1024_max(keep ? tid : -1, wred);
    sx[tid] = ki;
    __syncthreads();
    const int pk_i = tid > 0 ? sx[tid - 1] : -1;
    const int prev_kept = pk_i >= 0 ? sd[pk_i] : carry_kept;
    // interval ids
    const int n_start = scan1024_sum(start ? 1 : 0, wred);
    if (start) {
      const int id = carry_count + n_start - 1;
      ivh[2 * id] = -d;
      if (id > 0) ivh[2 * (id - 1) + 1] = -prev_kept + 64;   // close the interval before it
    }
    // carries (thread 1023 holds the pass totals)
    if (tid == 1023) {
      sx[0] = vi >= 0 ? sd[vi] : carry_valid;
      sx[1] = ki >= 0 ? sd[ki] : carry_kept;
      sx[2] = carry_count + n_start;
    }
    __syncthreads();
    carry_valid = sx[0]; carry_kept = sx[1]; carry_count = sx[2];
    __syncthreads();
  }
  if (tid == 0) {
    if (carry_count > 0) ivh[2 * (carry_count - 1) + 1] = -carry_kept + 64;
    A.n_iv[h] = carry_count;
    if (h == 0 && !(A.bad && *A.bad)) {
      if (A.cover_pairs) *A.cover_pairs = 0;
      if (A.attended) *A.attended = 0;
    }
  }
  __syncthreads();   // the interval ends are written (global memory, same workgroup)
  __threadfence_block();
  // iv_pre[u] = covered offsets of intervals 0..u-1
  int32_t* pre = A.iv_pre + (long long)h * (A.iv_stride + 1);
  int acc = 0;
  for (int base = 0; base < carry_count; base += 1024) {
    const int u = base + tid;
    const int len = u < carry_count ? ivh[2 * u + 1] - ivh[2 * u] : 0;
    const int inc = scan1024_sum(len, wred);
    if (u < carry_count) pre[u] = acc + inc - len;
    if (tid == 1023) sx[0] = inc;
    __syncthreads();
    acc += sx[0];
    __syncthreads();
  }
  if (tid == 0) pre[carry_count] = acc;
}

__global__ void plan_cov_clear_kernel(PlanArgs A) {
  const long long n = (long long)A.h_q * A.cov_words;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    A.cov[i] = 0u;
}

// Set the coverage bits of every merged interval (offset o -> bit o + p_last).
__global__ void plan_cov_kernel(PlanArgs A) {
  const int h = blockIdx.y;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= A.n_iv[h]) return;
  const int32_t* ivh = A.iv + (long long)h * A.iv_stride * 2;
  uint32_t* cv = A.cov + (long long)h * A.cov_words;
  const int b0 = max(ivh[2 * t], -A.p_last) + A.p_last;
  const int b1 = min(ivh[2 * t + 1], 64) + A.p_last;   // exclusive
  for (int bit = b0; bit < b1;) {
    const int w = bit >> 5;
    const int lo = bit & 31;
    const int hi = min(32, lo + (b1 - bit));
    const uint32_t m = (hi == 32 ? 0xFFFFFFFFu : ((1u << hi) - 1u)) & ~((1u << lo) - 1u);
    atomicOr(&cv[w], m);
    bit += hi - lo;
  }
}

// Exclusive prefix counts of the coverage bitmap's words, one workgroup per head.
__global__ void __launch_bounds__(1024) plan_cov_scan_kernel(PlanArgs A) {
  __shared__ int32_t wred[16];
  __shared__ int32_t tot;
  const int h = blockIdx.x, tid = threadIdx.x;
  const uint32_t* cv = A.cov + (long long)h * A.cov_words;
  int32_t* pc = A.cov_pre + (long long)h * A.cov_words;
  int acc = 0;
  for (int base = 0; base < A.cov_words; base += 1024) {
    const int w = base + tid;
    const int c = w < A.cov_words ? __popc(cv[w]) : 0;
    const int inc = scan1024_sum(c, wred);
    if (w < A.cov_words) pc[w] = acc + inc - c;
    if (tid == 1023) tot = inc;
    __syncthreads();
    acc += tot;
    __syncthreads();
  }
}

// Covered offsets of head h below x: the whole intervals before the one that
// holds x, plus the part of that one below x.
__device__ inline long long covered_below(const int32_t* ivh, const int32_t* pre, int n_iv, int x) {
  int a = 0, z = n_iv;
  while (a < z) { const int mid = (a + z) >> 1; if (ivh[2 * mid + 1] > x) z = mid; else a = mid + 1; }
  long long c = pre[a];
  if (a < n_iv && x > ivh[2 * a]) c += x - ivh[2 * a];
  return c;
}

// One wave per (head, query block): vertical columns inside the block's causal
// extent that the block's ranges miss, ascending, duplicates dropped; bit 30
// of an entry marks a high-norm key.  When the KV head has at most
// HN_MOVE_CAP high-norm keys, the list also takes the high-norm keys of the
// block's causal extent that the ranges cover, marked by bit 29 (the attention
// walk masks them in the range tiles; with exact diagonals it tests each
// row's offset to them): the list is then ordered by DCA mode (inter-chunk,
// successive, intra-chunk), each mode's columns first, then its high-norm
// keys, so every 32 entries still hold each mode's keys in one run of slots,
// and the keys at or above the block's first row, all intra-chunk, are the
// list's ascending tail.
// Also the block's first range tile (the one holding its lowest in-range
// offset) and its cover size.
__global__ void __launch_bounds__(256) plan_ext_kernel(PlanArgs A) {
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (unit >= A.h_q * A.nb) return;
  const int h = unit / A.nb;
  const int b = unit % A.nb;
  const int g = h / (A.h_q / A.h_kv);
  const int i0 = A.p0 + 64 * b;
  const int hi_key = i0 + min(64, A.n_q - 64 * b);
  const int32_t* vi = A.v_idx + (long long)h * A.k_v;
  const uint32_t* cv = A.cov + (long long)h * A.cov_words;
  const uint32_t* kb = A.kbits + (long long)g * A.kbits_words;
  int32_t* dst = A.ext + ((long long)h * A.nb + b) * A.ext_stride;
  const int m_blk = i0 / A.S;
  const int segA = max(0, (m_blk - 1) * A.S);    // DCA modes: [0, segA), [segA, segB), [segB, ..)
  const int segB = max(0, m_blk * A.S);
  // covered high-norm keys of the block's causal extent, per mode (ascending in the list)
  const int n_mv = (A.hnl_n[g] <= HN_MOVE_CAP) ? A.hnl_n[g] : 0;
  const int32_t* hall = A.hnall + (long long)g * HN_MOVE_CAP;
  // listed high-norm key t of the KV head, if covered inside the block's causal extent
  auto covered_hn = [&](int t, int& j) -> bool {
    if (t >= min(A.hnl_n[g], HN_MOVE_CAP)) return false;
    j = hall[t];
    if (j >= hi_key) return false;
    const int bit = j - i0 + A.p_last;
    return (cv[bit >> 5] >> (bit & 31)) & 1u;
  };
  auto moved = [&](int t, int& j) -> bool { return t < n_mv && covered_hn(t, j); };
  int mb0 = 0, mb1 = 0, mbn = 0;   // moved keys below segA, below segB, in all
  for (int base = 0; base < n_mv; base += 64) {
    int j = 0;
    const bool mk = moved(base + lane, j);
    mb0 += __popcll(__ballot(mk && j < segA));
    mb1 += __popcll(__ballot(mk && j < segB));
    mbn += __popcll(__ballot(mk));
  }
  // Exact diagonals, KV heads with at most HN_MOVE_CAP high-norm keys: the
  // vertical columns the ranges cover (other than the listed high-norm keys)
  // are listed too, after each mode's high-norm keys (bit 29, with a row mask
  // of the rows whose diagonal does not already reach them in the range
  // tiles), so the range tiles need no vertical-column test.
  const bool list_cv = A.dbits && A.hnl_n[g] <= HN_MOVE_CAP;
  auto covered_col = [&](int t, int& j) -> bool {
    j = -1;
    if (!list_cv || t >= A.k_v) return false;
    j = vi[t];
    const int prev = (t > 0) ? vi[t - 1] : -1;
    if (j < 0 || j >= hi_key || j == prev) return false;
    const int bit = j - i0 + A.p_last;
    return ((cv[bit >> 5] >> (bit & 31)) & 1u) && !((kb[j >> 5] >> (j & 31)) & 1u);
  };
  int vb0 = 0, vb1 = 0, vbn = 0;   // listed covered columns below segA, below segB, in all
  if (list_cv) {
    for (int base = 0; base < A.k_v; base += 64) {
      int j;
      const bool ck = covered_col(base + lane, j);
      vb0 += __popcll(__ballot(ck && j < segA));
      vb1 += __popcll(__ballot(ck && j < segB));
      vbn += __popcll(__ballot(ck));
    }
  }
  int cnt = 0, ca0 = 0, ca1 = 0;   // columns in all, below segA, below segB
  for (int base = 0; base < A.k_v; base += 64) {
    const int t = base + lane;
    bool keep = false;
    int j = -1;
    if (t < A.k_v) {
      j = vi[t];
      const int prev = (t > 0) ? vi[t - 1] : -1;
      if (j >= 0 && j < hi_key && j != prev) {
        const int bit = j - i0 + A.p_last;
        keep = !((cv[bit >> 5] >> (bit & 31)) & 1u);
      }
    }
    const unsigned long long bal = __ballot(keep);
    if (keep) {
      const int pos = __popcll(bal & ((1ull << lane) - 1ull));
      const int flagged = (kb[j >> 5] >> (j & 31)) & 1u;
      // after the moved keys and listed covered columns of the earlier modes
      dst[cnt + pos + (j < segA ? 0 : (j < segB ? mb0 + vb0 : mb1 + vb1))] = j | (flagged << 30);
    }
    cnt += __popcll(bal);
    ca0 += __popcll(__ballot(keep && j < segA));
    ca1 += __popcll(__ballot(keep && j < segB));
  }
  // the moved keys, each after the columns of its mode and the earlier modes
  for (int base = 0, k0 = 0; base < n_mv; base += 64) {
    int j = 0;
    const bool mk = moved(base + lane, j);
    const unsigned long long bal = __ballot(mk);
    if (mk) {
      const int pos = k0 + __popcll(bal & ((1ull << lane) - 1ull));
      const int at = pos + (j < segA ? ca0 : (j < segB ? ca1 + vb0 : cnt + vb1));
      dst[at] = j | (3 << 29);
      if (A.dbits) {
        // exact diagonals: the block rows r that attend key j, whose offset
        // i0 + r - j is selected (bits i0 - j + 128 .. + 63 of the offset
        // bitmap; negative offsets read its leading zero bits) or for which j
        // is a selected vertical column not above the row
        const uint32_t* db = A.dbits + (long long)h * A.dbits_words;
        const int b0 = i0 - j + 128;   // >= 65: j < i0 + 64
        const int w = b0 >> 5, sh = b0 & 31;
        const uint64_t x01 = (uint64_t)db[w] | ((uint64_t)db[w + 1] << 32);
        const uint64_t x12 = (uint64_t)db[w + 1] | ((uint64_t)db[w + 2] << 32);
        uint64_t rm = (uint64_t)(uint32_t)(x01 >> sh) | ((uint64_t)(uint32_t)(x12 >> sh) << 32);
        const int vb = j + 128;
        if ((A.vbits[(long long)h * A.vbits_words + (vb >> 5)] >> (vb & 31)) & 1u)
          rm |= j <= i0 ? ~0ull : (~0ull << (j - i0));
        const int E = A.ext_stride / 3;
        dst[E + 2 * at] = (int32_t)(uint32_t)rm;
        dst[E + 2 * at + 1] = (int32_t)(uint32_t)(rm >> 32);
      }
    }
    k0 += __popcll(bal);
  }
  // the listed covered columns, each after its mode's columns and moved keys:
  // row mask = the rows not above the column whose offset to it is not selected
  if (list_cv) {
    const uint32_t* db = A.dbits + (long long)h * A.dbits_words;
    const int E = A.ext_stride / 3;
    for (int base = 0, k0 = 0; base < A.k_v; base += 64) {
      int j;
      const bool ck = covered_col(base + lane, j);
      const unsigned long long bal = __ballot(ck);
      if (ck) {
        const int pos = k0 + __popcll(bal & ((1ull << lane) - 1ull));
        const int at = pos + (j < segA ? ca0 + mb0 : (j < segB ? ca1 + mb1 : cnt + mbn));
        dst[at] = j | (1 << 29);
        const int b0 = i0 - j + 128;   // >= 65: j < i0 + 64
        const int w = b0 >> 5, sh = b0 & 31;
        const uint64_t x01 = (uint64_t)db[w] | ((uint64_t)db[w + 1] << 32);
        const uint64_t x12 = (uint64_t)db[w + 1] | ((uint64_t)db[w + 2] << 32);
        const uint64_t slash = (uint64_t)(uint32_t)(x01 >> sh) | ((uint64_t)(uint32_t)(x12 >> sh) << 32);
        const uint64_t rm = (j <= i0 ? ~0ull : (~0ull << (j - i0))) & ~slash;
        dst[E + 2 * at] = (int32_t)(uint32_t)rm;
        dst[E + 2 * at + 1] = (int32_t)(uint32_t)(rm >> 32);
      }
      k0 += __popcll(bal);
    }
  }
  const int32_t* ivh = A.iv + (long long)h * A.iv_stride * 2;
  const int32_t* pre = A.iv_pre + (long long)h * (A.iv_stride + 1);
  const int n_iv = A.n_iv[h];
  const int tf = (int)(covered_below(ivh, pre, n_iv, -i0) / 32);   // the block's first range tile
  // the range tiles (from the block's first) holding a listed high-norm key,
  // as a bitmap the attention walk reads a word per tile
  if (A.hnl_n[g] <= HN_MOVE_CAP) {
    // the walk reads the words of its tiles and of up to two tiles past them
    uint32_t* bm = A.hnt + (long long)unit * A.hnt_words;
    const int n_range = (pre[n_iv] + 31) / 32 - tf;
    const int nw = min(A.hnt_words, (n_range + 2) / 32 + 1);
    for (int w = lane; w < nw; w += 64) bm[w] = 0u;
    __threadfence();
    const int32_t* pc = A.cov_pre + (long long)h * A.cov_words;
    const int n_hn = A.hnl_n[g];
    for (int base = 0; base < n_hn; base += 64) {
      int j = 0;
      if (covered_hn(base + lane, j)) {
        // covered offsets below j - i0: set bits of the coverage bitmap below its bit
        const int bit = j - i0 + A.p_last;
        const int below = pc[bit >> 5] + __popc(cv[bit >> 5] & ((1u << (bit & 31)) - 1u));
        const int rel = below / 32 - tf;
        atomicOr(&bm[rel >> 5], 1u << (rel & 31));
      }
    }
  }
  if (lane == 0) {
    A.n_ext[unit] = cnt + mbn + vbn;
    const int rows = hi_key - i0;
    long long below[2];
    below[0] = covered_below(ivh, pre, n_iv, -i0);
    below[1] = covered_below(ivh, pre, n_iv, rows);
    A.t_first[unit] = tf;
    const long long cover = (below[1] - below[0]) + cnt;
    if (!(A.bad && *A.bad)) {
      if (A.cover_pairs) atomicAdd((unsigned long long*)A.cover_pairs, (unsigned long long)(cover * rows));
      // block cover: the block's own keys [i0, i0 + rows) are always covered and
      // nothing above them, so row r attends |cover| - rows + r + 1 keys
      if (A.attended && !A.dbits) {
        const long long att = (long long)rows * (cover - rows) + (long long)rows * (rows + 1) / 2;
        atomicAdd((unsigned long long*)A.attended, (unsigned long long)att);
      }
    }
  }
}

// Range tiles of one head in offset space: tile t holds covered offsets of
// ranks [32t, 32t+32) of the merged intervals, as at most two runs (every
// interval is at least 64 long).  One thread per tile.
__global__ void __launch_bounds__(256) plan_tiles_kernel(PlanArgs A) {
  const int h = blockIdx.y;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int n_iv = A.n_iv[h];
  const int32_t* ivh = A.iv + (long long)h * A.iv_stride * 2;
  const int32_t* pre = A.iv_pre + (long long)h * (A.iv_stride + 1);
  const int total = pre[n_iv];
  const int n_t = (total + 31) / 32;
  if (t == 0) {
    A.n_tiles[h] = n_t;
  }
  if (t >= n_t) return;
  const int r0 = 32 * t;
  int a = 0, z = n_iv;   // last interval with pre <= r0
  while (z - a > 1) { const int mid = (a + z) >> 1; if (pre[mid] <= r0) a = mid; else z = mid; }
  const int len_a = ivh[2 * a + 1] - ivh[2 * a];
  const int off = r0 - pre[a];
  const int want = min(32, total - r0);
  const int len1 = min(want, len_a - off);
  int o2 = 0, len2 = 0;
  if (len1 < want && a + 1 < n_iv) {
    o2 = ivh[2 * (a + 1)];
    len2 = min(want - len1, ivh[2 * (a + 1) + 1] - o2);
  }
  A.tiles[(long long)h * A.tile_stride + t] = make_int4(ivh[2 * a] + off, o2, len1 | (len2 << 8), 0);
}

// Exact-diagonal semantics: the selected offsets (and 0) and vertical columns
// of each head as bitmaps, bit delta + 128 and bit j + 128 (the 128 leading
// zero bits let a window start below 0).
__global__ void plan_bits_clear_kernel(PlanArgs A) {
  const long long nd = (long long)A.h_q * A.dbits_words, nv = (long long)A.h_q * A.vbits_words;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < nd + nv; i += (long long)gridDim.x * blockDim.x) {
    if (i < nd) A.dbits[i] = 0u;
    else A.vbits[i - nd] = 0u;
  }
}

__global__ void plan_bits_kernel(PlanArgs A) {
  const int h = blockIdx.y;
  uint32_t* db = A.dbits + (long long)h * A.dbits_words;
  uint32_t* vb = A.vbits + (long long)h * A.vbits_words;
  const int n = A.k_s + A.k_v + 1;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    if (i < A.k_s) {
      const int d = A.s_off[(long long)h * A.k_s + i];
      if (d >= 0 && d <= A.p_last) atomicOr(&db[(d + 128) >> 5], 1u << ((d + 128) & 31));
    } else if (i < A.k_s + A.k_v) {
      const int c = A.v_idx[(long long)h * A.k_v + (i - A.k_s)];
      if (c >= 0 && c <= A.p_last) atomicOr(&vb[(c + 128) >> 5], 1u << ((c + 128) & 31));
    } else {
      atomicOr(&db[128 >> 5], 1u);   // offset 0
    }
  }
}

// Exact diagonals: the slash part of every row's mask, per range tile of a
// head and row r of a 64-row block.  Slot x of a run that starts d keys after
// the block's first row holds offset r - d - x from row r, whatever the block
// (the tiles are shared by the head's blocks), so one table serves them all:
// bit s is set when the offset of slot s is selected (or 0).  Four tiles of
// 64 rows per workgroup; slots past the tile's runs stay clear.
__global__ void __launch_bounds__(256) plan_smask_kernel(PlanArgs A) {
  const int h = blockIdx.y;
  const int t = 4 * blockIdx.x + (threadIdx.x >> 6);
  const int r = threadIdx.x & 63;
  if (t >= A.tile_stride) return;
  uint32_t m = 0u;
  if (t < A.n_tiles[h]) {
    const int4 d = A.tiles[(long long)h * A.tile_stride + t];
    const uint32_t* db = A.dbits + (long long)h * A.dbits_words;
    const int len1 = d.z & 0xFF, len2 = (d.z >> 8) & 0xFF;
    auto bit = [&](int off) -> uint32_t {   // off > -128 always (r >= 0, d < 64, x < 32)
      const int b = off + 128;
      return (db[b >> 5] >> (b & 31)) & 1u;
    };
    for (int x = 0; x < len1; ++x) m |= bit(r - d.x - x) << x;
    for (int x = 0; x < len2; ++x) m |= bit(r - d.y - x) << (len1 + x);
  }
  A.smask[((long long)h * A.tile_stride + t) * 64 + r] = m;
}

// Exact diagonals: the (row, key) pairs of one head, sum over rows i of
// |{delta selected (or 0) : delta <= p_i}| + |{j selected : j <= p_i}| minus the
// keys that are both, i.e. the pairs (column j, offset delta) with
// p0 <= j + delta <= p_last.  Workgroups (head, slice) over the two bitmaps.
__global__ void __launch_bounds__(1024) plan_attended_exact_kernel(PlanArgs A) {
  __shared__ unsigned long long red[16];
  if (A.bad && *A.bad) return;
  const int h = blockIdx.x;
  const uint32_t* db = A.dbits + (long long)h * A.dbits_words;
  const uint32_t* vb = A.vbits + (long long)h * A.vbits_words;
  const int p_last = A.p_last;
  const int p0 = A.p0;
  // rows whose position is at least x
  auto rows_from = [&](int x) -> long long { return x > p_last ? 0 : (long long)(p_last - max(x, p0) + 1); };
  // set bits of db in offsets [lo, hi] (bit delta + 128)
  auto dcount = [&](int lo, int hi) -> long long {
    lo = max(lo, 0);
    if (hi < lo) return 0;
    const int b0 = lo + 128, b1 = hi + 128;   // inclusive
    const int w0 = b0 >> 5, w1 = b1 >> 5;
    long long c = 0;
    for (int w = w0; w <= w1; ++w) {
      uint32_t m = db[w];
      if (w == w0) m &= ~0u << (b0 & 31);
      if (w == w1 && (b1 & 31) != 31) m &= (1u << ((b1 & 31) + 1)) - 1u;
      c += __popc(m);
    }
    return c;
  };
  long long acc = 0;
  const int nbits = p_last + 1;
  for (int x = blockIdx.y * blockDim.x + threadIdx.x; x < nbits; x += gridDim.y * blockDim.x) {
    const int bit = x + 128;
    if ((db[bit >> 5] >> (bit & 31)) & 1u) acc += rows_from(x);
    if ((vb[bit >> 5] >> (bit & 31)) & 1u) acc += rows_from(x) - dcount(p0 - x, p_last - x);
  }
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = (unsigned long long)acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long t = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
    atomicAdd((unsigned long long*)A.attended, t);
  }
}

hipError_t launch_plan(const PlanArgs& A, hipStream_t stream) {
  if (A.dbits) {
    hipLaunchKernelGGL(plan_bits_clear_kernel, dim3(256), dim3(256), 0, stream, A);
    const int n = A.k_s + A.k_v + 1;
    hipLaunchKernelGGL(plan_bits_kernel, dim3((n + 255) / 256, A.h_q), dim3(256), 0, stream, A);
  }
  hipLaunchKernelGGL(plan_intervals_kernel, dim3(A.h_q), dim3(1024), 0, stream, A);
  hipLaunchKernelGGL(plan_cov_clear_kernel, dim3(256), dim3(256), 0, stream, A);
  const int ivb = (A.iv_stride + 255) / 256;
  hipLaunchKernelGGL(plan_cov_kernel, dim3(ivb, A.h_q), dim3(256), 0, stream, A);
  hipLaunchKernelGGL(plan_cov_scan_kernel, dim3(A.h_q), dim3(1024), 0, stream, A);
  const int units = A.h_q * A.nb;
  hipLaunchKernelGGL(plan_ext_kernel, dim3((units + 3) / 4), dim3(256), 0, stream, A);
  hipLaunchKernelGGL(plan_tiles_kernel, dim3((A.tile_stride + 255) / 256, A.h_q), dim3(256), 0, stream, A);
  if (A.smask)
    hipLaunchKernelGGL(plan_smask_kernel, dim3((A.tile_stride + 3) / 4, A.h_q), dim3(256), 0, stream, A);
  if (A.dbits && A.attended)
    hipLaunchKernelGGL(plan_attended_exact_kernel, dim3(A.h_q, min(64, (A.p_last + 1024) / 1024)), dim3(1024), 0,
                       stream, A);
  return hipGetLastError();
}

}  // namespace dca
