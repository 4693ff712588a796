// Block-sparse DCA flash attention for gfx950: a software-pipelined tile walk
// whose common step carries almost no per-tile bookkeeping.
//
// Computes what the paper-review page's sparse prefill computes (section 4,
// Figure 4: vertical-slash sparsity under chunked prefill; Figure 2: the three
// DCA modes, each with its own query rotation): for one query block of one
// head (or a key-range part of it), the covered keys are walked as tiles of
// 32, S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16, with an
// online softmax in base 2.
//
// A workgroup is two waves, wave w holding rows 32w..32w+31 of the block; both
// read the K and V tiles that they stage together in LDS by direct
// global->LDS loads (two stages per tensor).  Step x of the walk:
//   A: the S^T MFMAs of tile x+1 (K fragments read two MFMAs ahead), each
//      followed by one exp2 pair of tile x's weights;
//   B: O += P V(x), the V fragments read two MFMAs ahead.
// Two barriers per step: before A (K(x+1) staged by both waves; both have
// read V(x-1), so V(x+1) may take its stage) and before B (V(x) staged; both
// have read K(x+1), so K(x+3) may take its stage).  Every step issues the same
// number of vector loads per wave, so each wait is a fixed count.
//
// Events.  Almost every tile is plain: 32 keys in [0, first row], one DCA
// mode (the one whose query rotation sits in registers) and no high-norm key.
// The few that are not (the walk's start and wrap, the tiles past the block's
// first row, the tiles where a later DCA mode begins, the tiles holding a
// high-norm key) are listed once per block as walk positions: the plan gives
// the mode and high-norm tiles of sparse calls, dense calls derive them from
// the key positions.  An event tile is loaded with clamped keys and scored on
// the general path (masks, several modes, split-precision logits); after it,
// the registers take the rotation of its last key's mode.  Everything else
// takes the short path.  When a head has more high-norm keys than the list
// holds, every tile is an event.
//
// Softmax: the S^T MFMAs start from -m_run; the reference m_run moves only
// when a half-row sum of this tile's weights exceeds 256 (every weight then
// stays <= 256) or while a row has not met a key; O's factor is applied once,
// before the next O += P V.  The row sums add the bf16 weights that enter P V.
#include <climits>

#include "common.h"
#include "args.h"
#include "attn_tile.h"

namespace dca {

namespace {

// s_waitcnt encodings: at most N vector-memory operations outstanding; all
// LDS operations of this wave retired
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void lgkm_wait0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void wg_barrier() {
  lgkm_wait0();                 // this wave's LDS reads are done
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// exp2 of two scores, rounded to a packed bf16 pair.  Written out so that the
// compiler keeps each pair where it is placed between the MFMAs (it would
// otherwise gather the exponentials of a tile in one place); the
// transcendental results are read one wait state later, as the ISA requires.
__device__ __forceinline__ uint32_t exp2_pk_bf16(float a, float b) {
  uint32_t r;
  float t0, t1;
  asm volatile("v_exp_f32 %1, %3\n\tv_exp_f32 %2, %4\n\ts_nop 0\n\tv_cvt_pk_bf16_f32 %0, %1, %2"
               : "=v"(r), "=&v"(t0), "=&v"(t1)
               : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float dot_ones(uint32_t pr, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pr), ones, acc, false);
}

// smallest value of v over the wave
__device__ __forceinline__ int wave_min(int v) {
  for (int d = 32; d >= 1; d >>= 1) v = min(v, __shfl_xor(v, d));
  return __builtin_amdgcn_readfirstlane(v);
}

// One tile of a walk, wave-uniform: runs [a1, a1 + len1) ++ [a2, a2 + len2) of
// absolute keys; ev: an event tile (clamped loads, general path).
struct TM {
  int a1, a2, len1, len2, ev;
};

}  // namespace

template <bool DENSE>
__device__ __forceinline__ void attn_pipe_body(const AttnArgs& A) {
  __shared__ __align__(16) uint8_t kst0[TILEB];
  __shared__ __align__(16) uint8_t kst1[TILEB];
  __shared__ __align__(16) uint8_t vst0[TILEB];
  __shared__ __align__(16) uint8_t vst1[TILEB];
  if (A.bad && *A.bad) return;   // positions check failed: no output is written
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // ---- work item: (query head, block, key part).  Workgroups reach the dies
  // round-robin (j -> die j % 8).  Where the KV groups divide the dies, a die
  // serves one KV group per part (the group advancing with the part); within a
  // part a die takes one head at a time, block rows in descending order, and
  // split calls give each die a contiguous half of the rows, so the blocks in
  // flight on a die read close keys through its L2.
  const int die = blockIdx.x % NXCD;
  const int local = blockIdx.x / NXCD;
  const int hpg = A.h_q / A.h_kv;
  const int NBW = A.nb;
  int b, h, part;
  int mpos = 0;              // the block's place in its die's row sequence (split calls)
  if (NXCD % A.h_kv == 0) {
    const int dpg = NXCD / A.h_kv;
    const int rws = (NBW + dpg - 1) / dpg;
    part = local / (rws * hpg);
    const int rem = local % (rws * hpg);
    const int sub = die / A.h_kv;
    const int cidx = A.split > 1 ? ((sub + part) % dpg) * rws + rem % rws : dpg * (rem % rws) + sub;
    if (cidx >= NBW) return;
    b = NBW - 1 - cidx;
    mpos = A.split > 1 ? rem % rws : 0;
    h = ((die + part) % A.h_kv) * hpg + rem / rws;
  } else {
    const int rws = (NBW + NXCD - 1) / NXCD;
    part = local / (rws * A.h_q);
    const int rem = local % (rws * A.h_q);
    const int cidx = NXCD * (rem % rws) + die;
    if (cidx >= NBW) return;
    b = NBW - 1 - cidx;
    h = rem / rws;
  }
  const int g = h / hpg;
  const int i0 = A.p0 + 64 * b;                  // absolute position of the block's first row
  const int rows = min(64, A.n_q - 64 * b);
  const int hi_key = i0 + rows;                  // keys [0, hi_key): the block's causal extent
  const int m_blk = i0 / A.S;
  // DCA mode of a key: 2 intra-chunk [segB, ..), 1 successive [segA, segB), 0 inter-chunk [0, segA)
  const int segA = max(0, (m_blk - 1) * A.S);
  const int segB = max(0, m_blk * A.S);
  auto key_mode = [&](int key) __attribute__((always_inline)) -> int {
    return (int)((unsigned)(segA - 1 - key) >> 31) + (int)((unsigned)(segB - 1 - key) >> 31);
  };
  const int rloc = 32 * wave + l32;              // this lane's row inside the block
  const bool row_ok = rloc < rows;
  const int qrow = 64 * b + (row_ok ? rloc : rows - 1);
  const int prow = i0 + rloc;                    // absolute position of this lane's row

  // ---- the part's tiles
  const int unit = h * A.nb + b;
  const int t_first = DENSE ? 0 : A.t_first[unit];
  const int n_range = DENSE ? (hi_key + BN - 1) / BN : A.n_tiles[h] - t_first;
  const int n_ext = DENSE ? 0 : A.n_ext[unit];
  const int n_all = n_range + (n_ext + BN - 1) / BN;
  const int t_beg = (int)((long long)n_all * part / A.split);
  const int t_end = (int)((long long)n_all * (part + 1) / A.split);
  const int r_end = min(t_end, n_range);
  const int nw = max(r_end - t_beg, 0);          // range tiles walked by this part
  // Staggered start: the range tiles of a sparse part are walked from a
  // rotated start.  A block's tiles are offsets from its first row, so blocks
  // b and b+1 read the same key about two tiles apart; with the start shifted
  // by twice the block's mean tiles per 64 keys per place on its die, the
  // blocks in flight on a die read close keys at the same time (L2 reuse).
  const int shift = (DENSE || nw == 0) ? 0 : (int)(((long long)mpos * n_range * 128 / max(hi_key, 1)) % nw);
  auto tile_index = [&](int x) __attribute__((always_inline)) -> int {
    int p = x + shift;
    if (p >= nw) p -= nw;
    return t_beg + p;
  };

  // ---- events: walk positions of the tiles that take the general path, one
  // candidate per lane (INT_MAX: none), consumed in increasing order
  int evx = INT_MAX;
  bool all_ev = false;
  {
    int ti = -1;
    if (DENSE) {
      const int n_hn = A.hnl_n[g];
      all_ev = n_hn > EV_PREC;
      if (lane < min(n_hn, EV_PREC)) {
        const int j = A.hnl[g * HN_CAP + lane];
        if (j < hi_key) ti = j >> 5;
      }
      if (lane == EV_PREC) ti = segA > 0 ? segA >> 5 : -1;
      if (lane == EV_PREC + 1) ti = segB > 0 ? segB >> 5 : -1;
      if (lane >= 33 && lane < 37) ti = (i0 >> 5) + (lane - 33);
    } else {
      const int32_t* rec = A.ev + (long long)unit * EV_REC;
      const int n_prec = rec[2];
      all_ev = n_prec < 0;
      if (lane < EV_PREC && lane < n_prec) ti = rec[3 + lane];
      if (lane == EV_PREC) ti = rec[0];
      if (lane == EV_PREC + 1) ti = rec[1];
      if (lane >= 33 && lane < 37) ti = A.npe[h] - t_first + (lane - 33);
    }
    if (lane == 31) ti = t_beg;                  // the wrap of the rotated walk
    if (lane == 32) ti = t_beg + shift;          // its start
    if (ti >= t_beg && ti < r_end) {
      int xe = ti - t_beg - shift;
      if (xe < 0) xe += nw;
      evx = xe;
    }
  }
  auto next_event = [&](int after) __attribute__((always_inline)) -> int {
    return wave_min(evx > after ? evx : INT_MAX);
  };
  int evk = next_event(-1);                      // next event at or after the next K load

  const int* tl_g = (const int*)(A.tiles + (long long)h * A.tile_stride) + 4 * t_first;
  const uint32_t* hn_g = (const uint32_t*)(A.hn + (long long)g * A.hn_pad);
  // tile of walk position y from its descriptor (lanes 0..2 of dv); y outside
  // the walk: rows 0..31 (clamped), which keeps the loads per step fixed
  auto make_tm = [&](int y, int dv) __attribute__((always_inline)) -> TM {
    TM T;
    if (y < 0 || y >= nw) {
      T.a1 = 0; T.a2 = 0; T.len1 = BN; T.len2 = 0; T.ev = 1;
      return T;
    }
    if (DENSE) {
      T.a1 = BN * (t_beg + y);
      T.len1 = min(BN, hi_key - T.a1);
      T.a2 = T.a1 + T.len1; T.len2 = 0;
    } else {
      const int dx = __builtin_amdgcn_readlane(dv, 0);
      const int dy = __builtin_amdgcn_readlane(dv, 1);
      const int dz = __builtin_amdgcn_readlane(dv, 2);
      T.a1 = i0 + dx;
      T.a2 = i0 + dy;
      T.len1 = dz & 0xFF;
      T.len2 = (dz >> 8) & 0xFF;
    }
    // a tile off the event list that is not plain would break the fast loads'
    // bounds: it is taken as an event all the same
    const int a_last = T.len2 ? T.a2 + T.len2 - 1 : T.a1 + T.len1 - 1;
    const bool plain = (T.len1 + T.len2 == BN) && T.a1 >= 0 && a_last <= i0;
    T.ev = all_ev || y == evk || !plain;
    if (y == evk) evk = next_event(y);
    return T;
  };
  // descriptor dwords of walk position y in lanes 0..3 (a per-lane vector load)
  auto desc_issue = [&](int y) __attribute__((always_inline)) -> int {
    if (DENSE) return 0;
    const int tix = (y < 0 || y >= nw) ? 0 : tile_index(y);
    return tl_g[4 * tix + (lane & 3)];
  };

  // ---- loads.  K and V rows of this KV head through buffer resources; one
  // 32-bit byte offset per row serves both tensors (the host bounds
  // n_k * h_kv * 256 < 2^32).  Load j of wave w fills group 2j + w of a tile
  // (rows 4(2j+w)..+3): lane -> row 4(2j+w) + (lane >> 4), 16-byte chunk
  // (lane & 15) ^ 5(lane >> 4).
  const __amdgpu_buffer_rsrc_t rs_k = __builtin_amdgcn_make_buffer_rsrc((void*)(A.khi + g * D), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_v = __builtin_amdgcn_make_buffer_rsrc((void*)(A.v + g * D), (short)0, -1, 0x00020000);
  const int rowb = A.h_kv * D * 2;
  const int lrow = lane >> 4;
  const unsigned lchunk = 16u * (unsigned)((lane & 15) ^ (5 * lrow));
  unsigned roff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) roff[j] = (unsigned)((4 * (2 * j + wave) + lrow) * rowb) + lchunk;
  // this wave's 4 direct loads of one tensor of tile T into a stage
  auto issue = [&](__amdgpu_buffer_rsrc_t rs, uint8_t* stage, const TM& T) __attribute__((always_inline)) {
    if (!T.ev) {
      // keys a1 + r (one run) or two runs, all inside [0, i0]: the first key's
      // row offset goes in the scalar offset, rows of the second run add the gap
      const int soff = (int)((unsigned)T.a1 * (unsigned)rowb);
      const unsigned gap = (unsigned)(T.a2 - T.a1 - T.len1) * (unsigned)rowb;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned vo = roff[j] + (lrow >= T.len1 - 4 * (2 * j + wave) ? gap : 0u);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(stage + (2 * j + wave) * GRPB),
                                                 16, vo, soff, 0, 0);
      }
    } else {
      // event tiles: negative keys, keys past the count (the keys after the
      // last run) or past n_k are clamped into [0, n_k); those slots are masked
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * (2 * j + wave) + lrow;
        int key = r < T.len1 ? T.a1 + r : T.a2 - T.len1 + r;
        key = min(max(key, 0), A.n_k - 1);
        const unsigned vo = (unsigned)key * (unsigned)rowb + lchunk;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(stage + (2 * j + wave) * GRPB),
                                                 16, vo, 0, 0, 0);
      }
    }
  };

  // ---- LDS reads: K fragments (A operand of S^T) and transposed V fragments
  // (A operand of O^T); per-lane byte offsets inside a tile
  unsigned kaddr[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) kaddr[kk] = (unsigned)tile_off(l32, 2 * kk + half);
  const int s16 = lane & 15;
  const int grp = l32 >> 4;
  unsigned vaddr[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int r1 = 4 * half + (s16 >> 2);
    const int c = 4 * db + 2 * grp + ((s16 & 3) >> 1);
    vaddr[db] = (unsigned)(tile_off(r1, c) + 8 * (s16 & 1));
  }
  // V fragment f (k-step G = f >> 2, d-block db = f & 3)
  auto read_v = [&](const uint8_t* vt, int f) __attribute__((always_inline)) -> bf16x8 {
    const int G = f >> 2, db = f & 3;
    const bf16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, vt + vaddr[db] + 4 * G * GRPB));
    const bf16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, vt + vaddr[db] + (4 * G + 2) * GRPB));
    return __builtin_shufflevector(t1, t2, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  // ---- state of this lane's row
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float m_run = 0.f;         // reference (log2 domain)
  float l_run = 0.f;         // this lane's partial row sum
  f32x16 negm = {};          // -m_run in every entry: the S^T MFMAs start from it
  bool started = false;      // the row has met a key
  bool all_started = false;  // wave-uniform: every row of the wave has

  // rotated query row of this lane for the current DCA mode (hi half; the lo
  // half is read from global memory by high-norm tiles only)
  bf16x8 qh[8];
  int q_mode = -1;
  auto q_off = [&](int mode) __attribute__((always_inline)) -> long long {
    return (((long long)mode * A.n_q + qrow) * A.h_q + h) * D + 8 * half;
  };
  // The rotation for another mode overwrites qh in place: the loads name the
  // registers qh already holds (and complete inside the statement), which
  // keeps this rare reload from splitting qh's registers in the walk loop.
  auto load_q = [&](int mode) __attribute__((always_inline)) {
    const uint16_t* qp = A.qhi + q_off(mode);
    asm volatile(
        "global_load_dwordx4 %0, %8, off\n\t"
        "global_load_dwordx4 %1, %8, off offset:32\n\t"
        "global_load_dwordx4 %2, %8, off offset:64\n\t"
        "global_load_dwordx4 %3, %8, off offset:96\n\t"
        "global_load_dwordx4 %4, %8, off offset:128\n\t"
        "global_load_dwordx4 %5, %8, off offset:160\n\t"
        "global_load_dwordx4 %6, %8, off offset:192\n\t"
        "global_load_dwordx4 %7, %8, off offset:224\n\t"
        "s_waitcnt vmcnt(0)"
        : "+v"(qh[0]), "+v"(qh[1]), "+v"(qh[2]), "+v"(qh[3]), "+v"(qh[4]), "+v"(qh[5]), "+v"(qh[6]), "+v"(qh[7])
        : "v"(qp)
        : "memory");
    q_mode = mode;
  };
  // S^T of a staged tile for one DCA mode's query rotation (+ the lo terms of
  // a high-norm tile: the slot keys' K_lo rows and the rotated query's lo
  // half, from global memory).  The rotation held in registers serves its
  // mode; another mode's rotation is read from global memory.  The K
  // fragments are read from LDS per pass, and the lo terms are taken in two
  // halves, which bounds the registers this rare path holds at once
  // (compiler barriers keep the passes apart).
  auto qk_mode = [&](f32x16& s, const uint8_t* kt, int mode, bool precise, int slot_key)
      __attribute__((always_inline)) {
    const bool held = mode == q_mode;
    const uint16_t* qhp = A.qhi + q_off(mode);
    asm volatile("" ::: "memory");
    s = negm;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8 qv = held ? qh[kk] : *(const bf16x8*)(qhp + 16 * kk);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(kt + kaddr[kk]), qv, s, 0, 0, 0);
    }
    if (precise) {
      const int kr = min(max(slot_key, 0), A.n_k - 1);
      const uint16_t* klrow = A.klo + (long long)kr * (A.h_kv * D) + g * D + 8 * half;
      const uint16_t* qlp = A.qlo + q_off(mode);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int kk = 4 * hf; kk < 4 * hf + 4; ++kk) {
          const bf16x8 alo = *(const bf16x8*)(klrow + 16 * kk);
          const bf16x8 qlo = *(const bf16x8*)(qlp + 16 * kk);
          const bf16x8 qv = held ? qh[kk] : *(const bf16x8*)(qhp + 16 * kk);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, qv, s, 0, 0, 0);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(kt + kaddr[kk]), qlo, s, 0, 0, 0);
        }
      }
    }
  };
  // a run [a, a + len) holds a high-norm key: the distance from its first
  // non-negative key to the next high-norm key is below its remaining length
  auto run_flagged = [&](uint32_t w, int a, int len) __attribute__((always_inline)) -> bool {
    const int ac = max(a, 0);
    const int lc = len - (ac - a);
    if (lc <= 0) return false;
    return (int)((w >> (8 * (ac & 3))) & 0xFFu) < lc;
  };
  // General scores of a tile: every DCA mode it holds (merged slot by slot,
  // keys ascend with the slot), split precision for high-norm keys, edge
  // masks.  For extra-vertical tiles skey is the lane's slot key (bit 30:
  // high-norm) and cnt the tile's count; range tiles have cnt = 0 and look
  // their high-norm keys up in the distance table.  Returns the DCA mode of
  // the tile's last key.
  auto qk_general = [&](f32x16& s, const uint8_t* kt, const TM& T, int cnt, int skey)
      __attribute__((always_inline)) -> int {
    int key_first, key_last, count;
    bool precise;
    if (cnt) {
      count = cnt;
      key_first = __builtin_amdgcn_readlane(skey, 0) & 0x3FFFFFFF;
      key_last = __builtin_amdgcn_readlane(skey, cnt - 1) & 0x3FFFFFFF;
      precise = __any(skey >= 0 && ((skey >> 30) & 1));
    } else {
      count = T.len1 + T.len2;
      key_first = T.a1;
      key_last = T.len2 ? T.a2 + T.len2 - 1 : T.a1 + T.len1 - 1;
      const uint32_t hv = hn_g[max((lane & 1) && T.len2 ? T.a2 : T.a1, 0) >> 2];
      precise = run_flagged(__builtin_amdgcn_readlane(hv, 0), T.a1, T.len1) ||
                run_flagged(__builtin_amdgcn_readlane(hv, 1), T.a2, T.len2);
    }
    const int slot_key = cnt ? (skey & 0x3FFFFFFF)
                             : (l32 < T.len1 ? T.a1 + l32 : (l32 < count ? T.a2 + (l32 - T.len1) : -1));
    const int mode_first = key_mode(max(key_first, 0));   // negative keys are masked
    const int mode_last = key_mode(key_last);
    // number of the tile's keys below x
    auto below = [&](int x) __attribute__((always_inline)) -> int {
      if (cnt) {
        const int kj = skey & 0x3FFFFFFF;
        return __builtin_popcountll(__ballot(l32 < cnt && half == 0 && kj < x));
      }
      return min(max(x - T.a1, 0), T.len1) + min(max(x - T.a2, 0), T.len2);
    };
    qk_mode(s, kt, mode_first, precise, slot_key);
    // slots from the first key of mode m on take that mode's scores (the
    // later modes are spelled out, as in key order)
    auto merge_mode = [&](int m) __attribute__((always_inline)) {
      f32x16 s2;
      qk_mode(s2, kt, m, precise, slot_key);
      const int base = below(m == 2 ? segB : segA) - 4 * half;
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int c = 8 * (vv >> 2) + (vv & 3);
        if (c >= base) s[vv] = s2[vv];
      }
    };
    if (mode_first + 1 <= mode_last) merge_mode(mode_first + 1);
    if (mode_first + 2 <= mode_last) merge_mode(mode_first + 2);
    if (count < BN || key_first < 0 || key_last > i0) {
      // extra-vertical keys all lie below the block (its own keys are range-covered)
      const int t_lo = cnt ? 0 : below(0);
      const int t_hi = cnt ? count : below(prow + 1);
      const int base = t_lo - 4 * half;
      const unsigned span = (unsigned)max(t_hi - t_lo, 0);
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int c = 8 * (vv >> 2) + (vv & 3);
        if ((unsigned)(c - base) >= span) s[vv] = -INFINITY;
      }
    }
    return mode_last;
  };

  // ---- softmax of one tile's scores: P as packed bf16 pairs (pw[G] holds the
  // B operand of k-step G of O += P V) and the tile's half-row sum of them
  u32x4 pw[2];
  float tsum = 0.f;
  auto exp_tile = [&](const f32x16& s) __attribute__((always_inline)) {
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      pw[q >> 2][q & 3] = exp2_pk_bf16(s[2 * q], s[2 * q + 1]);
      t = dot_ones(pw[q >> 2][q & 3], t);
    }
    tsum = t;
  };
  // the reference must move: a half-row sum above 256 (or not finite), or a
  // row of the wave has not met a key yet (wave-uniform)
  auto must_move = [&]() __attribute__((always_inline)) -> bool {
    return !all_started || __any(!(tsum <= 256.f));
  };
  // The reference moves to the tile's row max (rows whose max is above it,
  // and rows meeting their first keys); l and the scores follow at once, the
  // weights are taken again, and O's factor is gathered in alpha and applied
  // once, just before the next O += P V.
  float alpha = 1.f;
  bool rescale = false;      // wave-uniform: alpha must be applied
  auto move_reference = [&](f32x16& s, f32x16& s_nx, bool have_next) __attribute__((always_inline)) {
    float mx = s[0];
#pragma unroll
    for (int vv = 1; vv < 16; ++vv) mx = fmaxf(mx, s[vv]);
    mx = pair_max(mx);
    const bool mv = (mx > 0.f) || (!started && mx != -INFINITY);
    const float shift_m = mv ? mx : 0.f;
    const float a = mv ? (started ? fast_exp2(-mx) : 0.f) : 1.f;
    alpha *= a;
    l_run *= a;
    m_run += shift_m;
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) {
      s[vv] -= shift_m;
      negm[vv] = -m_run;
    }
    if (have_next) {
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) s_nx[vv] -= shift_m;
    }
    started = started || (mx != -INFINITY);
    all_started = !__any(!started);
    rescale = true;
    exp_tile(s);
  };
  auto apply_rescale = [&]() __attribute__((always_inline)) {
    if (rescale) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) o[db][vv] *= alpha;
      alpha = 1.f;
      rescale = false;
    }
  };
  // O^T += V^T P^T of a staged V tile, the V fragments read two MFMAs ahead
  auto pv = [&](const uint8_t* vt) __attribute__((always_inline)) {
    bf16x8 va[3];
    va[0] = read_v(vt, 0);
    va[1] = read_v(vt, 1);
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f + 2 < 8) va[(f + 2) % 3] = read_v(vt, f + 2);
      o[f & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[f % 3], __builtin_bit_cast(bf16x8, pw[f >> 2]), o[f & 3],
                                                         0, 0, 0);
    }
  };

  // ---- the pipelined walk over the part's range tiles.  Tile x is staged in
  // K stage x & 1 and V stage x & 1.  Step x = -2 .. nw-1 (steps before 0 only
  // fill the pipeline):
  //   (wait: own K(x+1) loads) barrier A; V(x+1) loads; A: scores of tile
  //   x+1 under tile x's weights;
  //   (wait: own V(x) loads) barrier B; K(x+3) loads, descriptor of x+5;
  //   B: O += P V(x).
  // Each wave issues exactly NL vector loads per step (tiles outside the walk
  // load clamped rows), so "own K(x+1) landed" at A and "own V(x) landed" at
  // B are both "at most NL loads outstanding" (loads of the general path only
  // make these waits stricter); a descriptor loaded at step x is read at step
  // x+2 behind the same waits.
  constexpr int NL = DENSE ? 8 : 9;
  f32x16 s_cur = {}, s_nx = {};
  auto step = [&](int x, TM& T1, TM& T2, int& dA, int& dB, uint8_t* kst_n, uint8_t* vst_c, uint8_t* vst_n)
      __attribute__((always_inline)) {
    // T1, T2: tiles x+1, x+2; dA, dB: the descriptors of tiles x+3, x+4.
    // kst_n, vst_n: stages of tile x+1 (and of tile x+3); vst_c: V stage of tile x.
    const bool have_cur = x >= 0;
    const bool have_next = x + 1 >= 0 && x + 1 < nw;
    vm_wait<NL>();
    wg_barrier();                // A
    issue(rs_v, vst_n, T1);      // V(x+1)
    // ---- A: tile x+1's scores under tile x's weights
    if (have_cur && have_next && !T1.ev) {
      // each S^T MFMA is followed by one pair of tile x's weights
      bf16x8 kb[3];
      kb[0] = *(const bf16x8*)(kst_n + kaddr[0]);
      kb[1] = *(const bf16x8*)(kst_n + kaddr[1]);
      float t = 0.f;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        if (kk + 2 < 8) kb[(kk + 2) % 3] = *(const bf16x8*)(kst_n + kaddr[kk + 2]);
        s_nx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[kk % 3], qh[kk], kk ? s_nx : negm, 0, 0, 0);
        pw[kk >> 2][kk & 3] = exp2_pk_bf16(s_cur[2 * kk], s_cur[2 * kk + 1]);
        if (kk >= 1) t = dot_ones(pw[(kk - 1) >> 2][(kk - 1) & 3], t);
        __builtin_amdgcn_sched_barrier(0);
      }
      tsum = dot_ones(pw[1][3], t);
      if (must_move()) move_reference(s_cur, s_nx, true);
      l_run += tsum;
    } else {
      // tile x's weights first (a moved reference then holds for tile x+1's scores)
      if (have_cur) {
        exp_tile(s_cur);
        if (must_move()) move_reference(s_cur, s_nx, false);
        l_run += tsum;
      }
      if (have_next) {
        const int ml = qk_general(s_nx, kst_n, T1, 0, -1);
        // the tiles after an event hold keys of its last key's mode
        if (ml != q_mode) load_q(ml);
      }
    }
    vm_wait<NL>();
    wg_barrier();                // B
    // tile x+3 from its descriptor: its K loads; the descriptor of x+5
    const TM T3 = make_tm(x + 3, dA);
    issue(rs_k, kst_n, T3);      // K(x+3)
    const int dC = desc_issue(x + 5);
    // ---- B: O += P V(x)
    if (have_cur) {
      apply_rescale();
      pv(vst_c);
    }
    s_cur = s_nx;
    T1 = T2; T2 = T3;
    dA = dB; dB = dC;
  };
  if (nw > 0) {
    // descriptors of tiles 0, 1, 2; then tile 0's K loads
    const int d0 = desc_issue(0);
    int dA = desc_issue(1), dB = desc_issue(2);
    vm_wait<0>();
    TM T1 = make_tm(-1, 0);
    TM T2 = make_tm(0, d0);
    issue(rs_k, kst0, T2);
    for (int x = -2; x < nw; x += 2) {
      step(x, T1, T2, dA, dB, kst1, vst0, vst1);
      if (x + 1 < nw) step(x + 1, T1, T2, dA, dB, kst0, vst1, vst0);
    }
  }
  // the clamped loads past the walk land before the stages are reused
  vm_wait<0>();
  wg_barrier();

  // ---- extra-vertical tiles (a few per block, after the range tiles): keys,
  // then K and V (both waves), then the tile, one at a time
  const int32_t* ext_h = A.ext + (long long)unit * A.ext_stride;
  for (int ti = max(t_beg, n_range); ti < t_end; ++ti) {
    const int eoff = BN * (ti - n_range);
    const int cnt = min(BN, n_ext - eoff);
    const int sk = (l32 < cnt) ? ext_h[eoff + l32] : -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int key = __shfl(sk, 4 * (2 * j + wave) + lrow) & 0x3FFFFFFF;
      key = min(max(key, 0), A.n_k - 1);
      const unsigned vo = (unsigned)key * (unsigned)rowb + lchunk;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_k, (__attribute__((address_space(3))) void*)(kst0 + (2 * j + wave) * GRPB),
                                               16, vo, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_v, (__attribute__((address_space(3))) void*)(vst0 + (2 * j + wave) * GRPB),
                                               16, vo, 0, 0, 0);
    }
    vm_wait<0>();
    wg_barrier();
    TM Tx;
    Tx.a1 = Tx.a2 = Tx.len1 = Tx.len2 = Tx.ev = 0;
    f32x16 sx, dummy;
    qk_general(sx, kst0, Tx, cnt, sk);
    exp_tile(sx);
    if (must_move()) move_reference(sx, dummy, false);
    l_run += tsum;
    apply_rescale();
    pv(vst0);
    wg_barrier();                // the stage is read; the next tile may overwrite it
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
    // the normalised partial in fp16 (values within max |v|), half the bytes the merge reads
    uint16_t* dst = A.part_o + (((long long)qrow * A.h_q + h) * A.split + part) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d0 = 32 * db + 8 * qd + 4 * half;
        uint2 pk;
        pk.x = f32_to_f16_bits(o[db][4 * qd + 0] * inv_l) | ((uint32_t)f32_to_f16_bits(o[db][4 * qd + 1] * inv_l) << 16);
        pk.y = f32_to_f16_bits(o[db][4 * qd + 2] * inv_l) | ((uint32_t)f32_to_f16_bits(o[db][4 * qd + 3] * inv_l) << 16);
        *(uint2*)(dst + d0) = pk;
      }
    }
    if (half == 0) A.part_lse[((long long)h * A.n_q + qrow) * A.split + part] = lse;
  }
}

__global__ void __launch_bounds__(128, 2) dca_attn_pipe_kernel(AttnArgs A) { attn_pipe_body<false>(A); }
__global__ void __launch_bounds__(128, 2) dca_attn_pipe_dense_kernel(AttnArgs A) { attn_pipe_body<true>(A); }

hipError_t launch_attn_pipe(const AttnArgs& A, hipStream_t stream) {
  // every die runs split * (its block rows) * (heads per row) two-wave workgroups
  const int blocks = NXCD % A.h_kv == 0
      ? NXCD * A.split * ((A.nb + NXCD / A.h_kv - 1) / (NXCD / A.h_kv)) * (A.h_q / A.h_kv)
      : NXCD * A.split * ((A.nb + NXCD - 1) / NXCD) * A.h_q;
  if (A.dense) hipLaunchKernelGGL(dca_attn_pipe_dense_kernel, dim3(blocks), dim3(128), 0, stream, A);
  else hipLaunchKernelGGL(dca_attn_pipe_kernel, dim3(blocks), dim3(128), 0, stream, A);
  return hipGetLastError();
}

}  // namespace dca
