// Block-sparse DCA flash attention for gfx950 (bf16 MFMA, fp32 accumulation).
//
// One work item is one query block (64 rows) of one query head, or a key
// range of it when the item is split.  Its keys are walked in DCA-mode order
// (inter-chunk, successive chunk, intra-chunk: paper-review page, section 4,
// Figure 2), each mode with its own query rotation, so one online softmax
// over all tiles equals the log-sum-exp merge of the three modes' partials.
// Within a mode the covered keys are enumerated in ascending order: first the
// merged slash ranges (vertical-slash sparsity, Figure 4 of the same page),
// then the vertical columns that no range covers.  Every 64 enumerated keys
// form one tile; tiles that hold a high-norm key add the lo halves of the
// rotated q and k to their logits (three MFMA passes) to keep the bf16 error
// of those logits small.
//
// Wave w of a 2-wave workgroup owns rows 32w..32w+31.  Scores are computed
// transposed (S^T = K Q^T) with v_mfma_f32_32x32x16_bf16 so that each lane
// holds one query row: the row max and sum need one cross-half exchange.
#include "common.h"
#include "args.h"

namespace dca {


// LDS row pitches (bf16 elements).  K rows: 136 (68 dwords) keeps the 16-byte
// operand reads of 16 consecutive rows on distinct banks.  V rows: 144
// (72 dwords) keeps the transposed 8-byte reads of 4 consecutive rows apart.
constexpr int KP = 136;
constexpr int VP = 144;

struct __align__(16) AttnSmem {
  uint16_t k[64 * KP];
  uint16_t v[64 * VP];
  uint16_t kl[64 * KP];
  uint16_t ql[2][8 * 64 * 8];  // per wave: q lo fragments [kk][lane][8]
  int32_t keys[64];
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Rotate this lane's query fragment for one DCA mode.  Lane (row = l%32,
// half = l/32) holds dims {16kk + 8half + e}: pairs (c, c+64) sit in slots kk
// and kk+4 of the same lane.
__device__ __forceinline__ void rotate_q(const AttnArgs& A, int h, int row, bool row_ok, int half,
                                         double qpos, bf16x8 (&qh)[8], uint16_t* ql_w, int lane) {
  const uint16_t* src = A.q + ((long long)row * A.h_q + h) * D;
  uint4 raw[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    if (row_ok) raw[kk] = *(const uint4*)(src + 16 * kk + 8 * half);
    else raw[kk] = make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const uint16_t* xa = (const uint16_t*)&raw[kk];
    const uint16_t* xb = (const uint16_t*)&raw[kk + 4];
    uint16_t hi_a[8], hi_b[8], lo_a[8], lo_b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = 16 * kk + 8 * half + e;
      float sn, cs;
      sincosf(reduce_angle(qpos, A.inv_freq[c]), &sn, &cs);
      const float x = bf16_bits_to_f32(xa[e]);
      const float y = bf16_bits_to_f32(xb[e]);
      const float xr = (x * cs - y * sn) * A.qscale;
      const float yr = (x * sn + y * cs) * A.qscale;
      hi_a[e] = f32_to_bf16_bits(xr);
      hi_b[e] = f32_to_bf16_bits(yr);
      lo_a[e] = f32_to_bf16_bits(xr - bf16_bits_to_f32(hi_a[e]));
      lo_b[e] = f32_to_bf16_bits(yr - bf16_bits_to_f32(hi_b[e]));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qh[kk][e] = bits_as_bf16(hi_a[e]);
      qh[kk + 4][e] = bits_as_bf16(hi_b[e]);
      ql_w[(kk * 64 + lane) * 8 + e] = lo_a[e];
      ql_w[((kk + 4) * 64 + lane) * 8 + e] = lo_b[e];
    }
  }
}

__global__ void __launch_bounds__(128, 2) dca_attn_kernel(AttnArgs A) {
  __shared__ AttnSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // ---- work item.  Workgroups reach the dies round-robin (j -> die j % 8) and
  // each die starts its share in order, so die x is given query-block rows
  // x, x+8, ... in descending block order (heavy first, dies balanced), and
  // all heads (and split parts) of one block row back to back: the 7 or 5 query
  // heads of a KV group then stream the same keys through that die's L2.
  const int C = A.h_q * A.split;
  const int die = blockIdx.x % NXCD;
  const int local = blockIdx.x / NXCD;
  const int c = NXCD * (local / C) + die;
  if (c >= A.nb) return;
  const int w = local % C;
  const int b = A.nb - 1 - c;
  const int h = w / A.split;
  const int part = w % A.split;
  const int g = h / (A.h_q / A.h_kv);

  const int i0 = A.p0 + QB * b;                  // absolute position of the block's first row
  const int rows = min(QB, A.n_q - QB * b);
  const int hi_key = i0 + rows;                  // keys [0, hi_key): the block's causal extent
  const int m_blk = i0 / A.S;
  const int rloc = 32 * wave + l32;              // row inside the block owned by this lane
  const bool row_ok = rloc < rows;
  const int qrow = QB * b + (row_ok ? rloc : 0);
  const int prow = i0 + rloc;                    // absolute position of this lane's row

  // key range of this split part (64-aligned)
  int k_beg = 0, k_end = hi_key;
  if (A.split > 1) {
    const int tiles = (hi_key + 63) / 64;
    k_beg = min(hi_key, (int)(((long long)tiles * part / A.split) * 64));
    k_end = min(hi_key, (int)(((long long)tiles * (part + 1) / A.split) * 64));
  }

  // mode segments: inter [0, A), successive [A, B), intra [B, hi_key)
  const int segA = min(hi_key, max(0, (m_blk - 1) * A.S));
  const int segB = min(hi_key, max(0, m_blk * A.S));
  const int seg_lo[3] = {0, segA, segB};
  const int seg_hi[3] = {segA, segB, hi_key};

  const int32_t* ivh = A.iv + (long long)h * A.iv_stride * 2;
  const int n_ivh = A.dense ? 0 : A.n_iv[h];
  const int32_t* exth = A.ext + ((long long)h * A.nb + b) * A.ext_stride;
  const int n_exth = A.dense ? 0 : A.n_ext[h * A.nb + b];

  const uint16_t* kh_base = A.khi + (long long)g * D;
  const uint16_t* kl_base = A.klo + (long long)g * D;
  const uint16_t* v_base = A.v + (long long)g * D;
  const long long kstride = (long long)A.h_kv * D;
  const uint8_t* flag_base = A.kflag + (long long)g * A.n_k;

  uint16_t* ql_w = sm.ql[wave];   // [kk][lane][8]: each lane reads back only its own slots

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m_run = -INFINITY;   // running max, log2 domain, shared by the two lanes of a row
  float l_run = 0.f;         // this lane's partial row sum

  bf16x8 qh[8];

  for (int seg = 0; seg < 3; ++seg) {
    const int lo = max(seg_lo[seg], k_beg);
    const int hi = min(seg_hi[seg], k_end);
    if (lo >= hi) continue;
    // ---- rotate the query fragment for this mode
    {
      const int r = prow % A.S;
      double qpos;
      if (seg == 2) qpos = r;
      else if (seg == 1) qpos = min(A.S + r, A.S + A.W - 1);
      else qpos = A.S + A.W - 1;
      rotate_q(A, h, qrow, row_ok, half, qpos, qh, ql_w, lane);
    }

    // ---- enumerate the covered keys of [lo, hi): range keys, then extra verticals
    // range cursor (sparse): interval index and current offset
    int cur_k = 0, cur_o = 0;
    if (!A.dense) {
      const int olo = lo - i0;
      // first interval with hi > olo (intervals ascending and disjoint)
      int a = 0, z = n_ivh;
      while (a < z) {
        int mid = (a + z) >> 1;
        if (ivh[2 * mid + 1] > olo) z = mid; else a = mid + 1;
      }
      cur_k = a;
      cur_o = (cur_k < n_ivh) ? max(olo, ivh[2 * cur_k]) : 0;
    }
    int dense_next = lo;
    // extra verticals inside [lo, hi)
    int e_beg = 0, e_end = 0;
    if (!A.dense) {
      int a = 0, z = n_exth;
      while (a < z) { int mid = (a + z) >> 1; if (exth[mid] >= lo) z = mid; else a = mid + 1; }
      e_beg = a;
      z = n_exth;
      while (a < z) { int mid = (a + z) >> 1; if (exth[mid] >= hi) z = mid; else a = mid + 1; }
      e_end = a;
    }
    bool ranges_done = false;
    int e_next = e_beg;
    const int ohi = hi - i0;

    while (true) {
      // ---- build this tile's key list (every lane computes all 64 keys: lane l -> key l)
      int key = -1;
      int count = 0;
      if (!ranges_done) {
        if (A.dense) {
          count = min(64, hi - dense_next);
          if (count > 0) { key = (lane < count) ? dense_next + lane : -1; dense_next += count; }
          if (dense_next >= hi) ranges_done = true;
        } else {
          if (cur_k < n_ivh && ivh[2 * cur_k] < ohi) {
            const int end1 = min(ivh[2 * cur_k + 1], ohi);
            const int run1 = min(64, end1 - cur_o);
            int run2 = 0, o2 = 0;
            int nk = cur_k, no = cur_o + run1;
            if (no >= end1) {
              nk = cur_k + 1;
              if (nk < n_ivh && ivh[2 * nk] < ohi) {
                o2 = ivh[2 * nk];
                const int end2 = min(ivh[2 * nk + 1], ohi);
                run2 = min(64 - run1, end2 - o2);
                no = o2 + run2;
                if (no >= end2) { nk = nk + 1; no = (nk < n_ivh) ? ivh[2 * nk] : 0; }
              } else {
                no = (nk < n_ivh) ? ivh[2 * nk] : 0;
              }
            }
            count = run1 + run2;
            if (lane < run1) key = i0 + cur_o + lane;
            else if (lane < count) key = i0 + o2 + (lane - run1);
            cur_k = nk;
            cur_o = no;
          }
          if (count == 0) ranges_done = true;
        }
      }
      if (count == 0) {
        if (e_next >= e_end) break;
        count = min(64, e_end - e_next);
        key = (lane < count) ? exth[e_next + lane] : -1;
        e_next += count;
      }
      if (count <= 0) break;
      key = (key >= 0 && key < A.n_k) ? key : -1;
      const bool precise = __any(key >= 0 && flag_base[key >= 0 ? key : 0] != 0);
      const bool need_mask = (count < 64) || __any(key >= i0) || __any(key < 0);

      // ---- stage K (hi, and lo when precise) and V rows in LDS
      __syncthreads();   // previous tile's LDS reads are done
      if (wave == 0) sm.keys[lane] = key;
      {
        const int c16 = tid & 15;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = (tid >> 4) + 8 * i;
          int kr = __shfl(key, r);
          kr = kr < 0 ? 0 : kr;
          const long long off = (long long)kr * kstride + 8 * c16;
          uint4 kv = *(const uint4*)(kh_base + off);
          uint4 vv = *(const uint4*)(v_base + off);
          *(uint4*)&sm.k[r * KP + 8 * c16] = kv;
          *(uint4*)&sm.v[r * VP + 8 * c16] = vv;
          if (precise) {
            uint4 kl = *(const uint4*)(kl_base + off);
            *(uint4*)&sm.kl[r * KP + 8 * c16] = kl;
          }
        }
      }
      __syncthreads();

      // ---- S^T = K Q^T for the 64 keys x 32 rows of this wave
      f32x16 s[2];
#pragma unroll
      for (int nbk = 0; nbk < 2; ++nbk) {
        s[nbk] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const bf16x8 a = *(const bf16x8*)&sm.k[(32 * nbk + l32) * KP + 16 * kk + 8 * half];
          s[nbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qh[kk], s[nbk], 0, 0, 0);
        }
      }
      if (precise) {
#pragma unroll
        for (int nbk = 0; nbk < 2; ++nbk) {
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) {
            const bf16x8 ahi = *(const bf16x8*)&sm.k[(32 * nbk + l32) * KP + 16 * kk + 8 * half];
            const bf16x8 alo = *(const bf16x8*)&sm.kl[(32 * nbk + l32) * KP + 16 * kk + 8 * half];
            const bf16x8 qlo = *(const bf16x8*)&ql_w[(kk * 64 + lane) * 8];
            s[nbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, qh[kk], s[nbk], 0, 0, 0);
            s[nbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, qlo, s[nbk], 0, 0, 0);
          }
        }
      }

      // ---- mask: absent keys and keys after the row's position
      if (need_mask) {
#pragma unroll
        for (int nbk = 0; nbk < 2; ++nbk) {
#pragma unroll
          for (int vv = 0; vv < 16; ++vv) {
            const int t = 32 * nbk + 8 * (vv >> 2) + 4 * half + (vv & 3);
            const int kj = sm.keys[t];
            if (kj < 0 || kj > prow || !row_ok) s[nbk][vv] = -INFINITY;
          }
        }
      }

      // ---- online softmax (log2 domain), lazy rescaling
      float mx = -INFINITY;
#pragma unroll
      for (int nbk = 0; nbk < 2; ++nbk)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) mx = fmaxf(mx, s[nbk][vv]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool grow = mx > m_run + 8.f;
      if (__any(grow)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int vv = 0; vv < 16; ++vv) o[i][vv] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      bf16x8 pf[4];
#pragma unroll
      for (int nbk = 0; nbk < 2; ++nbk) {
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
          const float p = fast_exp2(s[nbk][vv] - m_use);
          l_run += p;
          pf[2 * nbk + (vv >> 3)][vv & 7] = (__bf16)p;
        }
      }

      // ---- O^T += V^T P^T: A operand read transposed from the row-major V tile
      const int grp = l32 >> 4;       // which 16-wide d slice of the 32-d block
      const int s16 = lane & 15;
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        const int r1 = 16 * G + 4 * half + (s16 >> 2);
        const int r2 = r1 + 8;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int col = 32 * db + 16 * grp + 4 * (s16 & 3);
          const bf16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, &sm.v[r1 * VP + col]));
          const bf16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, &sm.v[r2 * VP + col]));
          const bf16x8 a = __builtin_shufflevector(t1, t2, 0, 1, 2, 3, 4, 5, 6, 7);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[G], o[db], 0, 0, 0);
        }
      }
    }
  }

  // ---- finish: row sum over both halves, normalise, write
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse2 = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
  const float lse = lse2 * 0.69314718055994531f;
  if (!row_ok) return;
  if (A.split == 1) {
    uint16_t* dst = A.out + ((long long)qrow * A.h_q + h) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d0 = 32 * db + 8 * qd + 4 * half;
        uint2 pk;
        pk.x = f32_to_bf16_bits(o[db][4 * qd + 0] * inv_l) | ((uint32_t)f32_to_bf16_bits(o[db][4 * qd + 1] * inv_l) << 16);
        pk.y = f32_to_bf16_bits(o[db][4 * qd + 2] * inv_l) | ((uint32_t)f32_to_bf16_bits(o[db][4 * qd + 3] * inv_l) << 16);
        *(uint2*)(dst + d0) = pk;
      }
    }
    if (A.lse_out && half == 0) A.lse_out[(long long)h * A.n_q + qrow] = lse;
  } else {
    float* dst = A.part_o + (((long long)part * A.n_q + qrow) * A.h_q + h) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d0 = 32 * db + 8 * qd + 4 * half;
        float4 f;
        f.x = o[db][4 * qd + 0] * inv_l; f.y = o[db][4 * qd + 1] * inv_l;
        f.z = o[db][4 * qd + 2] * inv_l; f.w = o[db][4 * qd + 3] * inv_l;
        *(float4*)(dst + d0) = f;
      }
    }
    if (half == 0) A.part_lse[((long long)part * A.h_q + h) * A.n_q + qrow] = lse;
  }
}

// LSE merge of split partials: m = max lse_p, O = sum e^{lse_p-m} O_p / sum e^{lse_p-m}.
__global__ void __launch_bounds__(256) lse_merge_kernel(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_lse,
                                                        uint16_t* __restrict__ out, float* __restrict__ lse_out,
                                                        int P, int n_q, int h_q) {
  // one 32-lane group per (row, head); lane owns 4 dims
  const long long item = (long long)blockIdx.x * 8 + (threadIdx.x >> 5);
  const int l = threadIdx.x & 31;
  if (item >= (long long)n_q * h_q) return;
  const int row = (int)(item / h_q);
  const int h = (int)(item % h_q);
  float m = -INFINITY;
  for (int p = 0; p < P; ++p) m = fmaxf(m, part_lse[((long long)p * h_q + h) * n_q + row]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int p = 0; p < P; ++p) {
      const float lp = part_lse[((long long)p * h_q + h) * n_q + row];
      const float w = (lp == -INFINITY) ? 0.f : __expf(lp - m);
      const float4 x = *(const float4*)(part_o + (((long long)p * n_q + row) * h_q + h) * D + 4 * l);
      acc.x += w * x.x; acc.y += w * x.y; acc.z += w * x.z; acc.w += w * x.w;
      wsum += w;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  uint2 pk;
  pk.x = f32_to_bf16_bits(acc.x * inv) | ((uint32_t)f32_to_bf16_bits(acc.y * inv) << 16);
  pk.y = f32_to_bf16_bits(acc.z * inv) | ((uint32_t)f32_to_bf16_bits(acc.w * inv) << 16);
  *(uint2*)(out + ((long long)row * h_q + h) * D + 4 * l) = pk;
  if (lse_out && l == 0) lse_out[(long long)h * n_q + row] = (wsum > 0.f) ? m + __logf(wsum) : -INFINITY;
}

hipError_t launch_attn(const AttnArgs& A, hipStream_t stream) {
  const int C = A.h_q * A.split;
  const int blocks = NXCD * ((A.nb + NXCD - 1) / NXCD) * C;
  hipLaunchKernelGGL(dca_attn_kernel, dim3(blocks), dim3(128), 0, stream, A);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const float* part_o, const float* part_lse, uint16_t* out, float* lse_out,
                            int P, int n_q, int h_q, hipStream_t stream) {
  const long long items = (long long)n_q * h_q;
  const int blocks = (int)((items + 7) / 8);
  hipLaunchKernelGGL(lse_merge_kernel, dim3(blocks), dim3(256), 0, stream, part_o, part_lse, out, lse_out,
                     P, n_q, h_q);
  return hipGetLastError();
}

}  // namespace dca
