// Generation-step (decode) DCA attention over a rotated key cache, gfx950.
//
// The newest n_t tokens (positions n_k - n_t .. n_k - 1) attend every cached
// key up to their own position, densely, with the positions of Dual Chunk
// Attention (paper-review page, section 4, Figure 2): a key sits at
// r_j = j mod S, so it is rotated once, when it enters the cache; the query of
// a token in chunk m is rotated to r (keys of chunk m), min(S + r, S + W - 1)
// (keys of chunk m - 1) or S + W - 1 (earlier chunks).
//
// The step is bound by memory bandwidth: every cached key and value row of a
// KV head is read once.  One wave per (key part, KV head, block of 32 query
// columns), where the columns are the (token, query head) pairs of the KV
// head, so one 32-key tile of K and V staged in LDS serves every query head
// of the group (GQA).  Scores are computed transposed (S^T = K Q^T,
// v_mfma_f32_32x32x16_bf16) with one query column per lane, then the same
// online softmax and O^T += V^T P^T as the prefill kernel.  Each part writes
// its normalised partial (O, lse) per column; a second kernel merges the
// parts by log-sum-exp.
#include "common.h"
#include "args.h"
#include "attn_tile.h"

namespace dca {

// PAGED: keys, values and flags live in pages of a pool (a tile of 32 keys
// never straddles a page); the tile at logical key kt0 starts at pool row
// tile_row(kt0).  Otherwise the pool is the contiguous cache (pool row = key).
template <bool PAGED>
__global__ void __launch_bounds__(64) dca_decode_kernel(DecArgs A) {
  // two stages of K and V: four LDS objects, so that the compiler tells the
  // reads of one stage from the direct loads in flight into the other
  __shared__ __align__(16) uint8_t kst0[TILEB];
  __shared__ __align__(16) uint8_t vst0[TILEB];
  __shared__ __align__(16) uint8_t kst1[TILEB];
  __shared__ __align__(16) uint8_t vst1[TILEB];
  const int lane = threadIdx.x;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int grp = l32 >> 4;
  const int s16 = lane & 15;

  // ---- work item and this lane's query column
  const int per_part = A.h_kv * A.n_cb;
  const int part = blockIdx.x / per_part;
  const int g = (blockIdx.x % per_part) / A.n_cb;
  const int cb = blockIdx.x % A.n_cb;
  const int G = A.h_q / A.h_kv;
  const int f = 32 * cb + l32;
  const bool col_ok = f < A.n_t * G;
  const int fc = col_ok ? f : 32 * cb;          // padding columns repeat the block's first column
  const int t = fc / G;                         // token
  const int h = g * G + fc % G;                 // query head
  const int p_t = A.n_k - A.n_t + t;            // the token's position
  const int m_t = p_t / A.S;                    // its DCA chunk
  const int p_min = A.n_k - A.n_t;

  const int k0 = part * A.part_keys;            // a multiple of 32
  const int t_beg = k0 / BN;
  const int t_end = (min(A.n_k, k0 + A.part_keys) + BN - 1) / BN;

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m_run = 0.f;         // reference max (log2 domain) of this column
  f32x16 negm = {};          // -m_run: the S^T MFMAs start from it
  bool started = false;
  float l_run = 0.f;

  // rotated query column for one DCA mode (2 intra, 1 successive, 0 inter);
  // the lo half is read back from memory by high-norm tiles only
  bf16x8 qh[8];
  const uint16_t* ql_row = A.qlo;
  int q_mode = -1;
  auto load_q = [&](int mode) __attribute__((always_inline)) {
    const long long qo = (((long long)mode * A.n_t + t) * A.h_q + h) * D + 8 * half;
    ql_row = A.qlo + qo;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qh[kk] = *(const bf16x8*)(A.qhi + qo + 16 * kk);
    // a mode change is rare: wait here, so that no wait for these loads is
    // left on the tile path (where it would also wait for the staged loads)
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    q_mode = mode;
  };

  // ---- staged loads: 8 direct loads per tensor and tile, load j filling rows
  // 4j .. 4j+3 (lane: row lane >> 4, chunk (lane & 15) ^ 5(lane >> 4)); rows
  // past the last key read the last key (masked later)
  // contiguous cache: rows [key][h_kv] from this head's column; paged pool:
  // pages [h_kv][page_keys], so a tile of one head is 32 consecutive rows
  const __amdgpu_buffer_rsrc_t rs_k =
      __builtin_amdgcn_make_buffer_rsrc((void*)(PAGED ? A.khi : A.khi + g * D), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_v =
      __builtin_amdgcn_make_buffer_rsrc((void*)(PAGED ? A.v : A.v + g * D), (short)0, -1, 0x00020000);
  const unsigned rowb = (unsigned)((PAGED ? 1 : A.h_kv) * D * 2);
  const int lrow = lane >> 4;
  const unsigned lchunk = 16u * (unsigned)((lane & 15) ^ (5 * lrow));
  // pool page of the tile at logical key kt0 (wave-uniform; a scalar load,
  // so its wait never drains the vector loads in flight)
  typedef __attribute__((address_space(4))) const int32_t ci32;
  auto tile_page = [&](int kt0) __attribute__((always_inline)) -> int {
    const int pg = ((ci32*)A.ptab)[kt0 / A.page_keys];
    return min(max(pg, 0), A.n_pages - 1);
  };
  // row (in units of rowb) of the tile's first key
  auto tile_row = [&](int kt0) __attribute__((always_inline)) -> int {
    return PAGED ? (tile_page(kt0) * A.h_kv + g) * A.page_keys + kt0 % A.page_keys : kt0;
  };
  auto issue = [&](__amdgpu_buffer_rsrc_t rs, uint8_t* stage, int kt0, int row0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = min(kt0 + 4 * j + lrow, A.n_k - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(stage + j * GRPB), 16,
                                               (int)((unsigned)(row0 + key - kt0) * rowb + lchunk), 0, 0, 0);
    }
  };
  typedef __attribute__((address_space(4))) const uint32_t cu32;
  cu32* kf = (cu32*)(A.kflags + (long long)g * A.kflag_words);
  const int pwords = A.page_keys / 32;
  // the high-norm flag word of the tile at kt0
  auto flag_word = [&](int kt0) __attribute__((always_inline)) -> uint32_t {
    if (PAGED)
      return ((cu32*)A.kflags)[((long long)tile_page(kt0) * A.h_kv + g) * pwords + (kt0 % A.page_keys) / 32];
    return kf[kt0 >> 5];
  };

  // S^T of the staged tile for one mode's query rotation, plus the lo terms
  // when the tile holds a high-norm key
  const uint16_t* kl_base = PAGED ? A.klo : A.klo + g * D;
  const long long kstride = (long long)(PAGED ? 1 : A.h_kv) * D;
  auto qk = [&](const uint8_t* kt, int mode, int kt0, int row0, bool precise) __attribute__((always_inline)) -> f32x16 {
    if (mode != q_mode) load_q(mode);
    f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(kt + tile_off(l32, half)), qh[0],
                                                       negm, 0, 0, 0);
#pragma unroll
    for (int kk = 1; kk < 8; ++kk) {
      const bf16x8 a = *(const bf16x8*)(kt + tile_off(l32, 2 * kk + half));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qh[kk], s, 0, 0, 0);
    }
    if (precise) {
      const uint16_t* klrow = kl_base + (long long)(row0 + min(kt0 + l32, A.n_k - 1) - kt0) * kstride;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 alo = *(const bf16x8*)(klrow + 16 * kk + 8 * half);
        const bf16x8 ahi = *(const bf16x8*)(kt + tile_off(l32, 2 * kk + half));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, qh[kk], s, 0, 0, 0);
        const bf16x8 qlo = *(const bf16x8*)(ql_row + 16 * kk);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, qlo, s, 0, 0, 0);
      }
    }
    return s;
  };

  // one tile: S^T per mode present among the columns (merged column by
  // column), the causal mask, online softmax, O^T += V^T P^T
  auto compute_tile = [&](const uint8_t* kt, const uint8_t* vt, int kt0) __attribute__((always_inline)) {
    const int m_k = kt0 / A.S;                 // a tile lies inside one DCA chunk
    const int mode = m_k == m_t ? 2 : (m_k + 1 == m_t ? 1 : 0);
    const bool precise = flag_word(kt0) != 0u;
    const int row0 = PAGED && precise ? tile_row(kt0) : kt0;
    const bool has0 = __any(col_ok && mode == 0);
    const bool has1 = __any(col_ok && mode == 1);
    const int first = has0 ? 0 : (has1 ? 1 : 2);
    f32x16 s = qk(kt, first, kt0, row0, precise);
    // the columns' tokens span at most a few chunks: later modes are spelled
    // out (a loop here would make the compiler wait for the staged loads)
    auto merge_mode = [&](int m) __attribute__((always_inline)) {
      const f32x16 s2 = qk(kt, m, kt0, row0, precise);
#pragma unroll
      for (int vv = 0; vv < 16; ++vv)
        if (mode == m) s[vv] = s2[vv];
    };
    if (first < 1 && has1) merge_mode(1);
    if (first < 2 && __any(col_ok && mode == 2)) merge_mode(2);
    if (kt0 + BN - 1 > p_min) {
      // keys past the column's token (and past the last key) are masked
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int key = kt0 + 8 * (vv >> 2) + (vv & 3) + 4 * half;
        if (key > p_t) s[vv] = -INFINITY;
      }
    }
    // online softmax (log2 domain; s holds score - m_run): the reference max
    // moves only when a score exceeds it by more than 8, or at the first keys
    float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
    for (int vv = 3; vv < 15; vv += 2) mx = fmaxf(fmaxf(mx, s[vv]), s[vv + 1]);
    mx = fmaxf(mx, s[15]);
    mx = pair_max(mx);
    const bool need = (mx > 8.f) || (!started && mx != -INFINITY);
    if (__any(need)) {
      const float shift = need ? mx : 0.f;
      const float alpha = started ? fast_exp2(-shift) : 0.f;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) o[i][vv] *= alpha;
      m_run += shift;
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        s[vv] -= shift;
        negm[vv] = -m_run;
      }
    }
    started = started || (mx != -INFINITY);
    bf16x8 pf[2];
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) pf[vv >> 3][vv & 7] = (__bf16)fast_exp2(s[vv]);
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int G2 = 0; G2 < 2; ++G2) {
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[G2], pf[G2], 0, 1), ones, l_run, false);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[G2], pf[G2], 2, 3), ones, l_run, false);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[G2], pf[G2], 4, 5), ones, l_run, false);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[G2], pf[G2], 6, 7), ones, l_run, false);
    }
    // O^T += V^T P^T, V^T read transposed from the row-major V tile
#pragma unroll
    for (int G2 = 0; G2 < 2; ++G2) {
      const int r1 = 16 * G2 + 4 * half + (s16 >> 2);
      const int r2 = r1 + 8;
      bf16x8 a[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int c = 4 * db + 2 * grp + ((s16 & 3) >> 1);
        const int bo = 8 * (s16 & 1);
        const bf16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, vt + tile_off(r1, c) + bo));
        const bf16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, vt + tile_off(r2, c) + bo));
        a[db] = __builtin_shufflevector(t1, t2, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[db], pf[G2], o[db], 0, 0, 0);
    }
  };

  // ---- the part's tiles, two stages: tile ti+2 is loaded into the stage of
  // tile ti once ti is computed.  Every step issues its 16 loads (8 K, 8 V),
  // past the part's end as repeats of its last tile (served by the L2), so
  // the number of loads issued after any tile is fixed: a tile has landed
  // when at most 16 of this wave's vector loads are outstanding (other loads
  // in between only make that wait longer).
  const int t_last = t_end - 1;
  {
    const int k0 = BN * t_beg, k1 = BN * min(t_beg + 1, t_last);
    const int r0 = tile_row(k0), r1 = tile_row(k1);
    issue(rs_k, kst0, k0, r0);
    issue(rs_v, vst0, k0, r0);
    issue(rs_k, kst1, k1, r1);
    issue(rs_v, vst1, k1, r1);
  }
  auto step = [&](uint8_t* kc, uint8_t* vc, int ti) __attribute__((always_inline)) {
    const int kn = BN * min(ti + 2, t_last);
    const int rn = tile_row(kn);            // scalar page-table load, waited for with the LDS reads below
    __builtin_amdgcn_s_waitcnt(0x4F70);   // vmcnt(16): tile ti landed, tile ti+1 may be in flight
    asm volatile("" ::: "memory");
    compute_tile(kc, vc, BN * ti);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this stage's reads are done
    asm volatile("" ::: "memory");
    issue(rs_k, kc, kn, rn);
    issue(rs_v, vc, kn, rn);
  };
  for (int ti = t_beg; ti < t_end; ti += 2) {
    step(kst0, vst0, ti);
    if (ti + 1 < t_end) step(kst1, vst1, ti + 1);
  }
  // the repeats land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // ---- the part's partial of this column: O normalised, natural-log lse
  const float l_tot = pair_sum(l_run);
  const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  if (!col_ok) return;
  float* dst = A.part_o + (((long long)part * A.n_t + t) * A.h_q + h) * D;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int d0 = 32 * db + 8 * qd + 4 * half;
      float4 v4;
      v4.x = o[db][4 * qd + 0] * inv_l; v4.y = o[db][4 * qd + 1] * inv_l;
      v4.z = o[db][4 * qd + 2] * inv_l; v4.w = o[db][4 * qd + 3] * inv_l;
      *(float4*)(dst + d0) = v4;
    }
  }
  if (half == 0) A.part_lse[((long long)part * A.h_q + h) * A.n_t + t] = lse;
}

// LSE merge of the parts of one (token, head): m = max_p lse_p,
// O = sum_p e^{lse_p - m} O_p / sum_p e^{lse_p - m}.  32 groups of 32 lanes
// take every 32nd part (lane: 4 dims); the groups' sums are combined in order.
constexpr int MERGE_GROUPS = 32;
__global__ void __launch_bounds__(1024) dca_decode_merge_kernel(const float* __restrict__ part_o,
                                                                const float* __restrict__ part_lse,
                                                                uint16_t* __restrict__ out, float* __restrict__ lse_out,
                                                                int P, int n_t, int h_q) {
  __shared__ float sm_m[MERGE_GROUPS], sm_w[MERGE_GROUPS];
  __shared__ float4 sm_acc[MERGE_GROUPS][32];
  const int t = blockIdx.x / h_q;
  const int h = blockIdx.x % h_q;
  const int sg = threadIdx.x >> 5;
  const int l = threadIdx.x & 31;
  float m = -INFINITY;
  for (int p = sg; p < P; p += MERGE_GROUPS) m = fmaxf(m, part_lse[((long long)p * h_q + h) * n_t + t]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float w = 0.f;
  if (m != -INFINITY) {
    for (int p = sg; p < P; p += MERGE_GROUPS) {
      const float lp = part_lse[((long long)p * h_q + h) * n_t + t];
      const float wt = (lp == -INFINITY) ? 0.f : __expf(lp - m);
      const float4 x = *(const float4*)(part_o + (((long long)p * n_t + t) * h_q + h) * D + 4 * l);
      acc.x += wt * x.x; acc.y += wt * x.y; acc.z += wt * x.z; acc.w += wt * x.w;
      w += wt;
    }
  }
  sm_acc[sg][l] = acc;
  if (l == 0) { sm_m[sg] = m; sm_w[sg] = w; }
  __syncthreads();
  if (sg != 0) return;
  float M = -INFINITY;
  for (int u = 0; u < MERGE_GROUPS; ++u) M = fmaxf(M, sm_m[u]);
  float4 tot = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int u = 0; u < MERGE_GROUPS; ++u) {
      const float e = (sm_m[u] == -INFINITY) ? 0.f : __expf(sm_m[u] - M);
      const float4 a = sm_acc[u][l];
      tot.x += e * a.x; tot.y += e * a.y; tot.z += e * a.z; tot.w += e * a.w;
      wsum += e * sm_w[u];
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  uint2 pk;
  pk.x = f32_to_bf16_bits(tot.x * inv) | ((uint32_t)f32_to_bf16_bits(tot.y * inv) << 16);
  pk.y = f32_to_bf16_bits(tot.z * inv) | ((uint32_t)f32_to_bf16_bits(tot.w * inv) << 16);
  *(uint2*)(out + ((long long)t * h_q + h) * D + 4 * l) = pk;
  if (lse_out && l == 0) lse_out[(long long)h * n_t + t] = (wsum > 0.f) ? M + __logf(wsum) : -INFINITY;
}

hipError_t launch_decode_attn(const DecArgs& A, hipStream_t stream) {
  const long long wgs = (long long)A.n_parts * A.h_kv * A.n_cb;
  if (A.ptab)
    hipLaunchKernelGGL(dca_decode_kernel<true>, dim3((unsigned)wgs), dim3(64), 0, stream, A);
  else
    hipLaunchKernelGGL(dca_decode_kernel<false>, dim3((unsigned)wgs), dim3(64), 0, stream, A);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecArgs& A, uint16_t* out, float* lse_out, hipStream_t stream) {
  hipLaunchKernelGGL(dca_decode_merge_kernel, dim3((unsigned)(A.n_t * A.h_q)), dim3(1024), 0, stream, A.part_o,
                     A.part_lse, out, lse_out, A.n_parts, A.n_t, A.h_q);
  return hipGetLastError();
}

}  // namespace dca
