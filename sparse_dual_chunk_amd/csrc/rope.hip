// Rotary embeddings of the attention kernel's operands under Dual Chunk
// Attention (paper-review page, section 4, Figure 2).
//
// Keys: every key takes the position of its offset inside its own chunk
// (r_j = j mod S), so a key is rotated once and the three query rotations
// carry the DCA mode.  The rotated key is stored as a
// bf16 pair (hi, lo) with hi + lo within 2^-16 relative of the fp32 rotation;
// the attention kernel adds the lo half only for tiles holding a key flagged as
// high-norm (L2 norm above a threshold), whose logits would otherwise carry
// bf16 rounding errors large enough to move the output (attention sinks).
#include <algorithm>

#include "common.h"
#include "args.h"

namespace dca {

__global__ void kbits_clear_kernel(uint32_t* __restrict__ kbits, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    kbits[i] = 0u;
}

// Destination rows of key j: the contiguous cache (row j), or a paged pool
// (logical page j / page_keys of the sequence is pool page ptab[..]; keys of
// a page whose entry lies outside [0, n_pages) are not written).
struct PageMap {
  const int32_t* ptab;
  int page_keys, n_pages;
};

// destination row (in rows of head_dim elements) of key j, KV head g:
// contiguous [capacity][h_kv] rows, or a pool page laid out head-major,
// [h_kv][page_keys] rows; -1 when the page entry is out of range
__device__ inline long long out_row(const PageMap& pm, int j, int g, int h_kv) {
  if (!pm.ptab) return (long long)j * h_kv + g;
  const int pg = pm.ptab[j / pm.page_keys];
  if (pg < 0 || pg >= pm.n_pages) return -1;
  return ((long long)pg * h_kv + g) * pm.page_keys + j % pm.page_keys;
}

// index of the flag word holding key j of KV head g (contiguous: [h_kv][words];
// paged: [n_pages][h_kv][page_keys / 32]), or -1
__device__ inline long long flag_index(const PageMap& pm, int g, int j, int kbits_words, int h_kv) {
  if (!pm.ptab) return (long long)g * kbits_words + (j >> 5);
  const int pg = pm.ptab[j / pm.page_keys];
  if (pg < 0 || pg >= pm.n_pages) return -1;
  return ((long long)pg * h_kv + g) * (pm.page_keys / 32) + (j % pm.page_keys) / 32;
}

// One 16-lane group per (key, kv head) row; lane c16 owns pairs 4*c16 .. 4*c16+3.
// Keys j0 .. j0+n-1: k (and v, when given) point at key j0, the outputs and
// bits are indexed by the absolute key through the page map.
__global__ void __launch_bounds__(256) rotate_keys_kernel(
    const uint16_t* __restrict__ k, uint16_t* __restrict__ khi, uint16_t* __restrict__ klo,
    uint32_t* __restrict__ kbits, Freqs fq, int j0,
    int n, int h_kv, int S, float thr2, int kbits_words, PageMap pm,
    const uint16_t* __restrict__ v_src, uint16_t* __restrict__ v_dst) {
  const int lane16 = threadIdx.x & 15;
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const long long n_rows = (long long)n * h_kv;
  const bool active = row < n_rows;
  const long long rrow = active ? row : 0;
  const int j = j0 + (int)(rrow / h_kv);
  const int g = (int)(rrow % h_kv);
  const double pos = (double)(j % S);
  const uint16_t* src = k + rrow * D;
  const long long orow = out_row(pm, j, g, h_kv);
  // two 8-byte loads: dims 4c..4c+3 and 64+4c..64+4c+3
  uint2 a = *(const uint2*)(src + 4 * lane16);
  uint2 b = *(const uint2*)(src + HALF + 4 * lane16);
  uint16_t xa[4] = {(uint16_t)(a.x & 0xFFFF), (uint16_t)(a.x >> 16), (uint16_t)(a.y & 0xFFFF), (uint16_t)(a.y >> 16)};
  uint16_t xb[4] = {(uint16_t)(b.x & 0xFFFF), (uint16_t)(b.x >> 16), (uint16_t)(b.y & 0xFFFF), (uint16_t)(b.y >> 16)};
  uint16_t ha[4], hb[4], la[4], lb[4];
  float ss = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int c = 4 * lane16 + t;
    float sn, cs;
    sincosf(reduce_angle(pos, fq.v[c]), &sn, &cs);
    const float x = bf16_bits_to_f32(xa[t]);
    const float y = bf16_bits_to_f32(xb[t]);
    ss += x * x + y * y;
    const float xr = x * cs - y * sn;
    const float yr = x * sn + y * cs;
    ha[t] = f32_to_bf16_bits(xr);
    hb[t] = f32_to_bf16_bits(yr);
    la[t] = f32_to_bf16_bits(xr - bf16_bits_to_f32(ha[t]));
    lb[t] = f32_to_bf16_bits(yr - bf16_bits_to_f32(hb[t]));
  }
  // squared norm of the raw key row over its 16 lanes
  ss += __shfl_xor(ss, 8, 16);
  ss += __shfl_xor(ss, 4, 16);
  ss += __shfl_xor(ss, 2, 16);
  ss += __shfl_xor(ss, 1, 16);
  if (!active || orow < 0) return;
  uint2 oa, ob, pa, pb;
  oa.x = ha[0] | ((uint32_t)ha[1] << 16); oa.y = ha[2] | ((uint32_t)ha[3] << 16);
  ob.x = hb[0] | ((uint32_t)hb[1] << 16); ob.y = hb[2] | ((uint32_t)hb[3] << 16);
  pa.x = la[0] | ((uint32_t)la[1] << 16); pa.y = la[2] | ((uint32_t)la[3] << 16);
  pb.x = lb[0] | ((uint32_t)lb[1] << 16); pb.y = lb[2] | ((uint32_t)lb[3] << 16);
  *(uint2*)(khi + orow * D + 4 * lane16) = oa;
  *(uint2*)(khi + orow * D + HALF + 4 * lane16) = ob;
  *(uint2*)(klo + orow * D + 4 * lane16) = pa;
  *(uint2*)(klo + orow * D + HALF + 4 * lane16) = pb;
  if (v_src) {
    // the value row is copied as is: 16 bytes per lane
    *(uint4*)(v_dst + orow * D + 8 * lane16) = *(const uint4*)(v_src + rrow * D + 8 * lane16);
  }
  // high-norm keys: one bit per key, OR-ed in (order-independent)
  if (lane16 == 0 && thr2 >= 0.f && ss > thr2)
    atomicOr(&kbits[flag_index(pm, g, j, kbits_words, h_kv)], 1u << (j & 31));
}

// Queries: one rotation per DCA mode the row takes part in, at the mode's query
// position: intra-chunk r_i, successive-chunk min(S + r_i, S + W - 1),
// inter-chunk S + W - 1 (W: local window).  A row of chunk c meets keys of mode
// m only when c >= 2 - m; the other entries are left unwritten and never read.
// The rotated row times the softmax scale (log2 units) is stored as bf16 hi
// plus bf16 lo residual in [3 modes][n_q][h_q][128].  Angles are reduced in
// fp64 to a fraction of a turn, then evaluated with the hardware sine / cosine
// of that fraction.  One 16-lane group per (row, head), as for the keys.
__global__ void __launch_bounds__(256) rotate_queries_kernel(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ qhi, uint16_t* __restrict__ qlo,
    const double* __restrict__ inv_freq, int n_q, int h_q, int p0, int S, int W, float qscale) {
  const int lane16 = threadIdx.x & 15;
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= (long long)n_q * h_q) return;
  const int i = (int)(row / h_q);
  const int pos = p0 + i;
  const int chunk = pos / S;
  const int r = pos % S;
  const uint16_t* src = q + row * D;
  uint2 a = *(const uint2*)(src + 4 * lane16);
  uint2 b = *(const uint2*)(src + HALF + 4 * lane16);
  const uint16_t xa[4] = {(uint16_t)(a.x & 0xFFFF), (uint16_t)(a.x >> 16), (uint16_t)(a.y & 0xFFFF), (uint16_t)(a.y >> 16)};
  const uint16_t xb[4] = {(uint16_t)(b.x & 0xFFFF), (uint16_t)(b.x >> 16), (uint16_t)(b.y & 0xFFFF), (uint16_t)(b.y >> 16)};
  for (int mode = 2 - min(chunk, 2); mode <= 2; ++mode) {
    const double qpos = mode == 2 ? (double)r : (mode == 1 ? (double)min(S + r, S + W - 1) : (double)(S + W - 1));
    uint16_t ha[4], hb[4], la[4], lb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = 4 * lane16 + t;
      const double turns = qpos * inv_freq[c] * INV_TWO_PI;
      const float f = (float)(turns - rint(turns));
      const float sn = __builtin_amdgcn_sinf(f);
      const float cs = __builtin_amdgcn_cosf(f);
      const float x = bf16_bits_to_f32(xa[t]);
      const float y = bf16_bits_to_f32(xb[t]);
      const float xr = (x * cs - y * sn) * qscale;
      const float yr = (x * sn + y * cs) * qscale;
      ha[t] = f32_to_bf16_bits(xr);
      hb[t] = f32_to_bf16_bits(yr);
      la[t] = f32_to_bf16_bits(xr - bf16_bits_to_f32(ha[t]));
      lb[t] = f32_to_bf16_bits(yr - bf16_bits_to_f32(hb[t]));
    }
    const long long o = ((long long)mode * n_q * h_q + row) * D;
    uint2 oa, ob, pa, pb;
    oa.x = ha[0] | ((uint32_t)ha[1] << 16); oa.y = ha[2] | ((uint32_t)ha[3] << 16);
    ob.x = hb[0] | ((uint32_t)hb[1] << 16); ob.y = hb[2] | ((uint32_t)hb[3] << 16);
    pa.x = la[0] | ((uint32_t)la[1] << 16); pa.y = la[2] | ((uint32_t)la[3] << 16);
    pb.x = lb[0] | ((uint32_t)lb[1] << 16); pb.y = lb[2] | ((uint32_t)lb[3] << 16);
    *(uint2*)(qhi + o + 4 * lane16) = oa;
    *(uint2*)(qhi + o + HALF + 4 * lane16) = ob;
    *(uint2*)(qlo + o + 4 * lane16) = pa;
    *(uint2*)(qlo + o + HALF + 4 * lane16) = pb;
  }
}

hipError_t launch_rotate_queries(const uint16_t* q, uint16_t* qhi, uint16_t* qlo, const double* inv_freq,
                                 int n_q, int h_q, int p0, int S, int W, float qscale, hipStream_t stream) {
  const long long rows = (long long)n_q * h_q;
  const int blocks = (int)((rows + 15) / 16);
  hipLaunchKernelGGL(rotate_queries_kernel, dim3(blocks), dim3(256), 0, stream, q, qhi, qlo, inv_freq,
                     n_q, h_q, p0, S, W, qscale);
  return hipGetLastError();
}

// hn[g][j] = distance from key j to the next high-norm key of KV head g,
// capped at 64 (a run [a, a+len) of len <= 32 holds one iff hn[a] < len).
// Entries j < n_pad (n_pad = the padded row count, a multiple of 4); the
// bitmap has guard words past n_k, so the three words read stay inside.
__global__ void __launch_bounds__(256) hn_next_kernel(const uint32_t* __restrict__ kbits, uint8_t* __restrict__ hn,
                                                      int n_pad, int h_kv, int kbits_words) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (long long)h_kv * n_pad) return;
  const int g = (int)(e / n_pad);
  const int j = (int)(e % n_pad);
  const uint32_t* kb = kbits + (long long)g * kbits_words;
  const int w = j >> 5;
  int d = 64;
  if (w < kbits_words) {
    // bits j .. j+63 of the bitmap, as a 96-bit window starting at word w
    const uint64_t lo = (uint64_t)kb[w] | ((uint64_t)(w + 1 < kbits_words ? kb[w + 1] : 0u) << 32);
    const uint32_t hi = w + 2 < kbits_words ? kb[w + 2] : 0u;
    const int sh = j & 31;
    const uint64_t win = (lo >> sh) | (sh ? ((uint64_t)hi << (64 - sh)) : 0ull);
    if (win) d = min(64, __builtin_ctzll(win));
  }
  hn[e] = (uint8_t)d;
}

hipError_t launch_hn_next(const uint32_t* kbits, uint8_t* hn, int n_pad, int h_kv, int kbits_words,
                          hipStream_t stream) {
  const long long n = (long long)h_kv * n_pad;
  hipLaunchKernelGGL(hn_next_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, kbits, hn, n_pad, h_kv,
                     kbits_words);
  return hipGetLastError();
}

// Keys and values 0 .. n_k-1 of a sequence in a paged pool, gathered into the
// contiguous rows the prefill attention reads ([n_k][h_kv][128] hi, lo and
// value rows), and the sequence's high-norm flag words into a contiguous
// [h_kv][kbits_words] bitmap (words past the page table read as zero).  Page
// entries outside [0, n_pages) are clamped.  One 16-lane group per (key, KV
// head) row, 16 bytes per lane of each tensor; the flag words follow in a
// grid-stride loop.
__global__ void __launch_bounds__(256) paged_gather_kernel(const uint16_t* __restrict__ khi_p,
                                                           const uint16_t* __restrict__ klo_p,
                                                           const uint16_t* __restrict__ v_p,
                                                           const uint32_t* __restrict__ flags_p, PageMap pm,
                                                           int n_table, int n_k, int h_kv, int kbits_words,
                                                           uint16_t* __restrict__ khi, uint16_t* __restrict__ klo,
                                                           uint16_t* __restrict__ vd, uint32_t* __restrict__ kbits) {
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int lane16 = threadIdx.x & 15;
  if (row < (long long)n_k * h_kv) {
    const int j = (int)(row / h_kv), g = (int)(row % h_kv);
    const int pg = min(max(pm.ptab[j / pm.page_keys], 0), pm.n_pages - 1);
    const long long src = (((long long)pg * h_kv + g) * pm.page_keys + j % pm.page_keys) * D + 8 * lane16;
    const long long dst = row * D + 8 * lane16;
    *(uint4*)(khi + dst) = *(const uint4*)(khi_p + src);
    *(uint4*)(klo + dst) = *(const uint4*)(klo_p + src);
    *(uint4*)(vd + dst) = *(const uint4*)(v_p + src);
  }
  const int wpp = pm.page_keys / 32;   // flag words per page and head
  const long long nwords = (long long)h_kv * kbits_words;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < nwords;
       i += (long long)gridDim.x * blockDim.x) {
    const int g = (int)(i / kbits_words), w = (int)(i % kbits_words);
    const int key0 = 32 * w;
    const int lp = key0 / pm.page_keys;
    uint32_t word = 0u;
    if (lp < n_table) {
      const int pg = min(max(pm.ptab[lp], 0), pm.n_pages - 1);
      word = flags_p[((long long)pg * h_kv + g) * wpp + (key0 % pm.page_keys) / 32];
    }
    kbits[i] = word;
  }
}

hipError_t launch_paged_gather(const uint16_t* khi_p, const uint16_t* klo_p, const uint16_t* v_p,
                               const uint32_t* flags_p, const int32_t* ptab, int page_keys, int n_pages, int n_table,
                               int n_k, int h_kv, int kbits_words, uint16_t* khi, uint16_t* klo, uint16_t* vd,
                               uint32_t* kbits, hipStream_t stream) {
  const long long rows = (long long)n_k * h_kv;
  const int blocks = (int)std::max<long long>((rows + 15) / 16, 1);
  const PageMap pm = {ptab, page_keys, n_pages};
  hipLaunchKernelGGL(paged_gather_kernel, dim3(blocks), dim3(256), 0, stream, khi_p, klo_p, v_p, flags_p, pm,
                     n_table, n_k, h_kv, kbits_words, khi, klo, vd, kbits);
  return hipGetLastError();
}

// The first HN_MOVE_CAP high-norm keys j < n_k of each KV head, ascending, and
// how many there are in all (counting stops once it exceeds HN_MOVE_CAP).  One
// workgroup of 1024 threads per KV head: each round scans 1024 flag words,
// places every word's keys after an exclusive prefix sum of the words' counts.
__global__ void __launch_bounds__(1024) hn_list_kernel(const uint32_t* __restrict__ kbits, int kbits_words, int n_k,
                                                       int32_t* __restrict__ hnl_n, int32_t* __restrict__ hnall) {
  __shared__ int wave_tot[16];
  __shared__ int base_s;
  const int g = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint32_t* kb = kbits + (long long)g * kbits_words;
  const int nw = (n_k + 31) / 32;
  if (tid == 0) base_s = 0;
  __syncthreads();
  for (int w0 = 0; w0 < nw; w0 += 1024) {
    const int w = w0 + tid;
    uint32_t word = w < nw ? kb[w] : 0u;
    if (w == nw - 1 && (n_k & 31)) word &= (1u << (n_k & 31)) - 1u;
    const int c = __popc(word);
    int incl = c;   // inclusive prefix within the wave
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d);
      if (lane >= d) incl += t;
    }
    if (lane == 63) wave_tot[wv] = incl;
    __syncthreads();
    int before = base_s;
    for (int i = 0; i < wv; ++i) before += wave_tot[i];
    int pos = before + incl - c;
    while (word) {
      if (pos < HN_MOVE_CAP) hnall[g * HN_MOVE_CAP + pos] = 32 * w + __builtin_ctz(word);
      ++pos;
      word &= word - 1u;
    }
    __syncthreads();
    if (tid == 0) {
      int t = base_s;
      for (int i = 0; i < 16; ++i) t += wave_tot[i];
      base_s = t;
    }
    __syncthreads();
    if (base_s > HN_MOVE_CAP) break;
  }
  if (tid == 0) hnl_n[g] = base_s;
}

hipError_t launch_hn_list(const uint32_t* kbits, int kbits_words, int n_k, int h_kv, int32_t* hnl_n,
                          int32_t* hnall, hipStream_t stream) {
  hipLaunchKernelGGL(hn_list_kernel, dim3(h_kv), dim3(1024), 0, stream, kbits, kbits_words, n_k, hnl_n, hnall);
  return hipGetLastError();
}

// Clear the bits of keys [j0, j0 + n) of every KV head (partial words keep
// their other bits); a word never straddles a page (page_keys % 32 == 0).
__global__ void kbits_clear_range_kernel(uint32_t* __restrict__ kbits, int kbits_words, int h_kv, int j0, int n,
                                         PageMap pm) {
  const int w0 = j0 >> 5, w1 = (j0 + n - 1) >> 5;
  const long long nw = (long long)(w1 - w0 + 1) * h_kv;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < nw; i += (long long)gridDim.x * blockDim.x) {
    const int g = (int)(i / (w1 - w0 + 1));
    const int w = w0 + (int)(i % (w1 - w0 + 1));
    const int lo = max(j0, 32 * w) - 32 * w;             // first bit of the range in this word
    const int hi = min(j0 + n, 32 * w + 32) - 32 * w;    // one past the last
    const uint32_t m = (hi - lo == 32) ? 0xFFFFFFFFu : (((1u << (hi - lo)) - 1u) << lo);
    const long long fi = flag_index(pm, g, 32 * w, kbits_words, h_kv);
    if (fi >= 0) atomicAnd(&kbits[fi], ~m);
  }
}

// Rotates keys [j0, j0 + n) (k points at key j0).  clear_all: the whole bitmap
// is cleared first (a fresh prefix), else only the bits of the range.
hipError_t launch_rotate_keys(const uint16_t* k, uint16_t* khi, uint16_t* klo, uint32_t* kbits,
                              const Freqs& f, int j0, int n, int h_kv, int S, float thr2, int kbits_words,
                              bool clear_all, hipStream_t stream) {
  const long long rows = (long long)n * h_kv;
  const int blocks = (int)((rows + 15) / 16);
  const PageMap none = {nullptr, 0, 0};
  if (clear_all)
    hipLaunchKernelGGL(kbits_clear_kernel, dim3(256), dim3(256), 0, stream, kbits, (long long)h_kv * kbits_words);
  else
    hipLaunchKernelGGL(kbits_clear_range_kernel, dim3(64), dim3(256), 0, stream, kbits, kbits_words, h_kv, j0, n,
                       none);
  hipLaunchKernelGGL(rotate_keys_kernel, dim3(blocks), dim3(256), 0, stream,
                     k, khi, klo, kbits, f, j0, n, h_kv, S, thr2, kbits_words, none, (const uint16_t*)nullptr,
                     (uint16_t*)nullptr);
  return hipGetLastError();
}

// Paged append: keys [j0, j0 + n) rotated into the pool pages of the page
// table, their values copied, their flag bits rewritten.
hipError_t launch_rotate_keys_paged(const uint16_t* k, const uint16_t* v, uint16_t* khi, uint16_t* klo,
                                    uint16_t* vpool, uint32_t* kflags, const int32_t* ptab, int page_keys,
                                    int n_pages, const Freqs& f, int j0, int n, int h_kv, int S, float thr2,
                                    hipStream_t stream) {
  const long long rows = (long long)n * h_kv;
  const int blocks = (int)((rows + 15) / 16);
  const PageMap pm = {ptab, page_keys, n_pages};
  hipLaunchKernelGGL(kbits_clear_range_kernel, dim3(64), dim3(256), 0, stream, kflags, 0, h_kv, j0, n, pm);
  hipLaunchKernelGGL(rotate_keys_kernel, dim3(blocks), dim3(256), 0, stream,
                     k, khi, klo, kflags, f, j0, n, h_kv, S, thr2, 0, pm, v, vpool);
  return hipGetLastError();
}

}  // namespace dca
