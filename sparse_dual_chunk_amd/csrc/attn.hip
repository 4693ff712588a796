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


// Tiles of 32 keys staged in LDS by direct global->LDS loads, two stages.
// A tile of one tensor is 8 groups of 4 key rows; a group is stored
// chunk-major ([16-byte chunk][row], 1 KiB) followed by 64 bytes of padding.
// Each direct load instruction fills one group (lane l: chunk l/4, row l%4).
// With the padding, the K operand reads (16 rows, one chunk) and the
// transposed V reads (4 rows, two chunks) of a 16-lane group fall on distinct
// banks, and every read address is a per-lane base plus an immediate offset.
constexpr int BN = 32;
constexpr int GRPB = 1024 + 64;                // bytes per 4-row group
constexpr int TILEB = 8 * GRPB;                // one tensor of one tile
constexpr int STAGEB = 2 * TILEB;              // K then V

// byte offset of (row, 16-byte chunk) inside a tensor tile
__device__ __forceinline__ int tile_off(int row, int chunk) { return (row >> 2) * GRPB + chunk * 64 + (row & 3) * 16; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of a value with the one held by lane ^ 32 (the other half of the row)
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One tile of the walk, wave-uniform: range tiles hold two runs of keys
// [a1, a1+len1) ++ [a2, a2+len2) (absolute; a1 < 0 possible in the first tile
// of a block); extra tiles (cnt > 0) hold entries [eoff, eoff+cnt) of the
// block's extra-vertical list.
struct Tile {
  int a1, a2, len1, len2, eoff, cnt;
};

__device__ __forceinline__ int tile_count(const Tile& T) { return T.cnt ? T.cnt : T.len1 + T.len2; }

// key of slot t (0..31) of a range tile, or -1 outside the tile
__device__ __forceinline__ int range_key(const Tile& T, int t) {
  return t < T.len1 ? T.a1 + t : (t < T.len1 + T.len2 ? T.a2 + (t - T.len1) : -1);
}

__global__ void __launch_bounds__(128, 2) dca_attn_kernel(AttnArgs A) {
  __shared__ __align__(16) uint8_t stage0[STAGEB];
  __shared__ __align__(16) uint8_t stage1[STAGEB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS bases stay scalar
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // ---- work item.  Workgroups reach the dies round-robin (j -> die j % 8) and
  // each die starts its share in order.  Split parts are outermost in every
  // die's sequence, so the workgroups in flight all read the same share of
  // their key ranges.  Where the KV groups divide the dies evenly, a die serves
  // one KV group per part (the group advancing with the part, which evens out
  // the per-group work), else all heads.  Within a part a die takes one query
  // head at a time, its block rows in descending order (longest causal extent
  // first): the rows of one head share one cover pattern shifted by 64 keys a
  // row, so the workgroups in flight do near-equal work, start and end
  // together and walk the same keys at the same time through the die's L2.
  const int die = blockIdx.x % NXCD;
  const int local = blockIdx.x / NXCD;
  const int hpg = A.h_q / A.h_kv;
  int b, h, part;
  if (NXCD % A.h_kv == 0) {
    const int dpg = NXCD / A.h_kv;                 // dies per KV group
    const int rows = (A.nb + dpg - 1) / dpg;       // block rows of this die
    part = local / (rows * hpg);
    const int rem = local % (rows * hpg);
    const int cidx = dpg * (rem % rows) + die / A.h_kv;
    if (cidx >= A.nb) return;
    b = A.nb - 1 - cidx;
    h = ((die + part) % A.h_kv) * hpg + rem / rows;
  } else {
    const int rows = (A.nb + NXCD - 1) / NXCD;
    part = local / (rows * A.h_q);
    const int rem = local % (rows * A.h_q);
    const int cidx = NXCD * (rem % rows) + die;
    if (cidx >= A.nb) return;
    b = A.nb - 1 - cidx;
    h = rem / rows;
  }
  const int g = h / (A.h_q / A.h_kv);

  const int i0 = A.p0 + QB * b;                  // absolute position of the block's first row
  const int rows = min(QB, A.n_q - QB * b);
  const int hi_key = i0 + rows;                  // keys [0, hi_key): the block's causal extent
  const int m_blk = i0 / A.S;
  const int rloc = 32 * wave + l32;              // row inside the block owned by this lane
  const bool row_ok = rloc < rows;
  const int qrow = QB * b + (row_ok ? rloc : 0);
  const int prow = i0 + rloc;                    // absolute position of this lane's row
  // DCA mode of a key: 2 intra-chunk [segB, ..), 1 successive [segA, segB), 0 inter-chunk [0, segA)
  const int segA = max(0, (m_blk - 1) * A.S);
  const int segB = max(0, m_blk * A.S);

  const int unit = h * A.nb + b;
  const int* tl_h = (const int*)(A.tiles + (long long)h * A.tile_stride);
  const int t_first = A.dense ? 0 : A.t_first[unit];
  const int n_range = A.dense ? (hi_key + BN - 1) / BN : A.n_tiles[h] - t_first;
  const int32_t* ext_h = A.ext + (long long)unit * A.ext_stride;
  const int n_ext = A.dense ? 0 : A.n_ext[unit];
  const int n_all = n_range + (n_ext + BN - 1) / BN;
  const int t_beg = (int)((long long)n_all * part / A.split);
  const int t_end = (int)((long long)n_all * (part + 1) / A.split);

  const int kstride = A.h_kv * D;
  const uint16_t* kh_base = A.khi + g * D;
  const uint16_t* kl_base = A.klo + g * D;
  const uint16_t* v_base = A.v + g * D;
  const uint32_t* kb = A.kbits + (long long)g * A.kbits_words;
  const int grp = l32 >> 4;       // which 16-wide d slice of a 32-d block (transposed V reads)
  const int s16 = lane & 15;

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m_run = 0.f;         // reference max (log2 domain) of this row
  bool started = false;      // the row has met a key
  float l_run = 0.f;         // this lane's partial row sum
  // rotated query row of this lane for the current DCA mode: the hi half is
  // held in registers (qh[kk]: dims 16kk + 8half .. +7), the lo half is read
  // back from global memory by high-norm tiles only
  bf16x8 qh[8];
  const uint16_t* ql_row = A.qlo;
  int q_mode = -1;

  // ---- tile metadata.  A range tile's descriptor is read by lanes 0..3 (one
  // int each, a vector load) two tiles ahead; the slot key (lane & 31) and the
  // high-norm flag of a tile are loaded one tile ahead, before the tile's
  // direct-to-LDS loads are issued, so no wait on them stalls those loads.
  auto desc_load = [&](int idx) -> int {   // per-lane part of the descriptor of tile idx
    if (A.dense || idx >= n_range || idx >= t_end) return 0;
    return tl_h[4 * (t_first + idx) + (lane & 3)];
  };
  auto make_tile = [&](int idx, int dv) -> Tile {
    Tile T;
    T.a2 = 0; T.len2 = 0; T.eoff = 0; T.cnt = 0;
    if (idx < n_range) {
      if (A.dense) {
        T.a1 = BN * idx;
        T.len1 = min(BN, hi_key - T.a1);
      } else {
        const int d0 = __builtin_amdgcn_readlane(dv, 0);
        const int d1 = __builtin_amdgcn_readlane(dv, 1);
        const int d2 = __builtin_amdgcn_readlane(dv, 2);
        T.a1 = i0 + d0;
        T.a2 = i0 + d1;
        T.len1 = d2 & 0xFF;
        T.len2 = (d2 >> 8) & 0xFF;
      }
    } else {
      T.a1 = 0; T.len1 = 0;
      T.eoff = BN * (idx - n_range);
      T.cnt = min(BN, n_ext - T.eoff);
    }
    return T;
  };
  // slot key of this lane (slot lane & 31): an extra-vertical entry (bit 30
  // marks a high-norm key) or a range key; -1 for an empty slot
  auto slot_key = [&](const Tile& T) -> int {
    if (T.cnt) return (l32 < T.cnt) ? ext_h[T.eoff + l32] : -1;
    const int key = range_key(T, l32);
    return (key < 0 || key >= A.n_k) ? -1 : key;
  };
  // the bitmap word holding a range slot key's high-norm bit (read one tile ahead)
  auto flag_word = [&](int key) -> uint32_t { return key >= 0 ? kb[key >> 5] : 0u; };
  // K and V rows of this KV head through buffer resources: one 32-bit byte
  // offset per row serves both tensors (the host bounds n_k * h_kv * 256 < 2^32)
  const __amdgpu_buffer_rsrc_t rs_k = __builtin_amdgcn_make_buffer_rsrc((void*)kh_base, (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_v = __builtin_amdgcn_make_buffer_rsrc((void*)v_base, (short)0, -1, 0x00020000);
  const int rowb = kstride * 2;
  auto issue_tile = [&](uint8_t* stage, const Tile& T, int skey) {
    // all row offsets first, then the loads: no wait lands between two loads
    int voff[4];
    const int choff = 16 * (lane >> 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * (2 * j + wave) + (lane & 3);
      int key;
      if (T.cnt) key = __shfl(skey, r) & 0x3FFFFFFF;
      else key = (r < T.len1 ? T.a1 : T.a2 - T.len1) + r;   // slots past the count are masked later
      key = min(max(key, 0), A.n_k - 1);
      voff[j] = __umul24((unsigned)key, (unsigned)rowb) + choff;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int grp4 = 2 * j + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_k, (__attribute__((address_space(3))) void*)(stage + grp4 * GRPB),
                                               16, voff[j], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs_v, (__attribute__((address_space(3))) void*)(stage + TILEB + grp4 * GRPB), 16, voff[j], 0, 0, 0);
    }
  };

  auto compute_tile = [&](const uint8_t* kt, const uint8_t* vt, const Tile& T, int skey, uint32_t fword) {
    const int count = tile_count(T);
    const bool flagged = T.cnt ? (skey >= 0 && ((skey >> 30) & 1)) : (skey >= 0 && ((fword >> (skey & 31)) & 1u));
    const bool precise = __any(flagged);
    const int key_first = T.cnt ? (__builtin_amdgcn_readlane(skey, 0) & 0x3FFFFFFF) : T.a1;
    const int key_last = T.cnt ? (__builtin_amdgcn_readlane(skey, count - 1) & 0x3FFFFFFF)
                               : (T.len2 ? T.a2 + T.len2 - 1 : T.a1 + T.len1 - 1);
    const int mode_first = key_first >= segB ? 2 : (key_first >= segA ? 1 : 0);
    const int mode_last = key_last >= segB ? 2 : (key_last >= segA ? 1 : 0);
    const bool edge = (count < BN) || (key_first < 0) || (key_last >= i0);

    for (int mode = mode_first; mode <= mode_last; ++mode) {
      // ---- query rotation for this DCA mode
      if (mode != q_mode) {
        const long long qo = (((long long)mode * A.n_q + qrow) * A.h_q + h) * D + 8 * half;
        const uint16_t* qh_row = A.qhi + qo;
        ql_row = A.qlo + qo;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qh[kk] = row_ok ? *(const bf16x8*)(qh_row + 16 * kk) : bf16x8{};
        q_mode = mode;
      }
      // ---- S^T = K Q^T: 32 keys x 32 rows of this wave (scores in log2 units)
      f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(kt + tile_off(l32, half)), qh[0],
                                                         f32x16{}, 0, 0, 0);
#pragma unroll
      for (int kk = 1; kk < 8; ++kk) {
        const bf16x8 a = *(const bf16x8*)(kt + tile_off(l32, 2 * kk + half));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qh[kk], s, 0, 0, 0);
      }
      if (precise) {
        // + K_lo Q_hi + K_hi Q_lo; K_lo rows come straight from global memory
        int kr = __shfl(skey, l32);
        kr = (kr < 0) ? 0 : min(kr & 0x3FFFFFFF, A.n_k - 1);
        const uint16_t* klrow = kl_base + kr * kstride;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const bf16x8 alo = *(const bf16x8*)(klrow + 16 * kk + 8 * half);
          const bf16x8 ahi = *(const bf16x8*)(kt + tile_off(l32, 2 * kk + half));
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, qh[kk], s, 0, 0, 0);
          const bf16x8 qlo = row_ok ? *(const bf16x8*)(ql_row + 16 * kk) : bf16x8{};
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, qlo, s, 0, 0, 0);
        }
      }
      // ---- masks: absent slots, keys outside [0, p_row], keys of another DCA mode
      if (edge || mode_first != mode_last) {
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
          const int t = 8 * (vv >> 2) + 4 * half + (vv & 3);
          int kj;
          if (T.cnt) {
            kj = __shfl(skey, t);
            kj = kj < 0 ? -1 : (kj & 0x3FFFFFFF);
          } else {
            kj = range_key(T, t);
          }
          const int km = kj >= segB ? 2 : (kj >= segA ? 1 : 0);
          if (kj < 0 || kj > prow || km != mode) s[vv] = -INFINITY;
        }
      }
      // ---- online softmax (log2 domain).  The reference max moves only when a
      // score exceeds it by more than 8 (so p <= 2^8), or at the row's first keys.
      float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
      for (int vv = 3; vv < 15; vv += 2) mx = fmaxf(fmaxf(mx, s[vv]), s[vv + 1]);
      mx = fmaxf(mx, s[15]);
      mx = pair_max(mx);
      const bool need = (mx > m_run + 8.f) || (!started && mx != -INFINITY);
      if (__any(need)) {
        const float m_new = need ? mx : m_run;
        const float alpha = started ? fast_exp2(m_run - m_new) : 0.f;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int vv = 0; vv < 16; ++vv) o[i][vv] *= alpha;
        m_run = m_new;
      }
      started = started || (mx != -INFINITY);
      bf16x8 pf[2];
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const float p = fast_exp2(s[vv] - m_run);
        l_run += p;
        pf[vv >> 3][vv & 7] = (__bf16)p;
      }
      // ---- O^T += V^T P^T, V^T operand read transposed from the row-major V tile
#pragma unroll
      for (int G = 0; G < 2; ++G) {
        const int r1 = 16 * G + 4 * half + (s16 >> 2);
        const int r2 = r1 + 8;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int c = 4 * db + 2 * grp + ((s16 & 3) >> 1);     // 16-byte chunk of the 4 columns read
          const int bo = 8 * (s16 & 1);                           // byte offset inside the chunk
          const bf16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, vt + tile_off(r1, c) + bo));
          const bf16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, vt + tile_off(r2, c) + bo));
          const bf16x8 a = __builtin_shufflevector(t1, t2, 0, 1, 2, 3, 4, 5, 6, 7);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[G], o[db], 0, 0, 0);
        }
      }
    }
  };

  // ---- prologue: tile t_beg staged, descriptor of t_beg+1 in flight
  int dv_cur = desc_load(t_beg);
  Tile T_cur = make_tile(t_beg, dv_cur);
  int sk_cur = -1;
  uint32_t fw_cur = 0;
  if (t_beg < t_end) {
    sk_cur = slot_key(T_cur);
    fw_cur = T_cur.cnt ? 0u : flag_word(sk_cur);
    issue_tile(stage0, T_cur, sk_cur);
  }
  int dv_nxt = desc_load(t_beg + 1);
  __syncthreads();

  // One step: prefetch tile ti+1 into the other stage, then compute tile ti.
  // The other stage was last read before the previous barrier.  Range tiles
  // issue their loads before any metadata read they would wait for; an
  // extra-vertical tile needs its keys first (these tiles are few).
  auto step = [&](const uint8_t* cur, uint8_t* nxt, int ti) {
    Tile T_n;
    int sk_n = -1;
    uint32_t fw_n = 0;
    const bool more = ti + 1 < t_end;
    if (more) {
      T_n = make_tile(ti + 1, dv_nxt);
      if (T_n.cnt) {
        sk_n = slot_key(T_n);
        issue_tile(nxt, T_n, sk_n);
      } else {
        issue_tile(nxt, T_n, 0);
        sk_n = slot_key(T_n);
        fw_n = flag_word(sk_n);
      }
      dv_nxt = desc_load(ti + 2);
    }
    compute_tile(cur, cur + TILEB, T_cur, sk_cur, fw_cur);
    __syncthreads();   // the prefetched stage has landed; this stage may be overwritten next
    if (more) { T_cur = T_n; sk_cur = sk_n; fw_cur = fw_n; }
  };
  for (int ti = t_beg; ti < t_end; ti += 2) {
    step(stage0, stage1, ti);
    if (ti + 1 < t_end) step(stage1, stage0, ti + 1);
  }

  // ---- finish: row sum over both halves, normalise, write
  const float l_tot = pair_sum(l_run);
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
  // every die runs split * (its block rows) * (heads per row) workgroups
  const int blocks = NXCD % A.h_kv == 0
      ? NXCD * A.split * ((A.nb + NXCD / A.h_kv - 1) / (NXCD / A.h_kv)) * (A.h_q / A.h_kv)
      : NXCD * A.split * ((A.nb + NXCD - 1) / NXCD) * A.h_q;
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
