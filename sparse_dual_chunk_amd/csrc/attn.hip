// Block-sparse DCA flash attention for gfx950 (bf16 MFMA, fp32 accumulation).
//
// One work item is one query block (64 rows) of one query head, or a key
// range of it when the item is split.  Its keys are walked in DCA-mode order
// (inter-chunk, successive chunk, intra-chunk: paper-review page, section 4,
// Figure 2), each mode with its own query rotation, so one online softmax
// over all tiles equals the log-sum-exp merge of the three modes' partials.
// Within a mode the covered keys are enumerated in ascending order: first the
// merged slash ranges (vertical-slash sparsity, Figure 4 of the same page),
// then the vertical columns that no range covers.  Every 32 enumerated keys
// form one tile; tiles that hold a high-norm key add the lo halves of the
// rotated q and k to their logits (three MFMA passes) to keep the bf16 error
// of those logits small.
//
// Wave w of a 2-wave workgroup owns rows 32w..32w+31.  Scores are computed
// transposed (S^T = K Q^T) with v_mfma_f32_32x32x16_bf16 so that each lane
// holds one query row: the row max and sum need one cross-half exchange.
#include "common.h"
#include "args.h"
#include "attn_tile.h"

#include <algorithm>

namespace dca {


// One tile of the walk, wave-uniform: range tiles hold two runs of keys
// [a1, a1+len1) ++ [a2, a2+len2) (absolute; a1 < 0 possible in the first tile
// of a block); extra tiles (cnt > 0) hold entries [eoff, eoff+cnt) of the
// block's extra-vertical list.
struct Tile {
  int a1, a2, len1, len2, eoff, cnt;
};

__device__ __forceinline__ int tile_count(Tile T) { return T.cnt ? T.cnt : T.len1 + T.len2; }

// key of slot t (0..31) of a range tile, or -1 outside the tile
__device__ __forceinline__ int range_key(Tile T, int t) {
  return t < T.len1 ? T.a1 + t : (t < T.len1 + T.len2 ? T.a2 + (t - T.len1) : -1);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes): raw dwords, no stride.
__device__ __forceinline__ i32x4 raw_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r.z = (int)bytes;
  r.w = 0x00020000;
  return r;
}

// Direct loads into LDS: lane l's 16 (4) bytes at byte offset voff of the
// buffer land at lds + 16 l (4 l).  They are issued where the compiler does
// not see them, so it places no wait of its own for them (it cannot tell the
// stages of consecutive loop iterations apart and would wait for the loads of
// the next tile before reading the current one): every read of their data is
// ordered by the walk's own vmcnt waits and barriers.  M0 takes the LDS
// address one instruction before the load.
__device__ __forceinline__ void dma_b128(i32x4 rs, uint32_t lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rs) : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(i32x4 rs, uint32_t lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rs) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}


// NW waves of 32 rows per workgroup: 2 (one 64-row block) for every call; 4
// (two adjacent blocks, 128 rows, sharing every staged K / V tile) for dense
// calls whose pairs of blocks lie inside one DCA chunk: their key ranges
// differ only by the 64 keys of the second block, so the pair walks its
// union at no extra work and loads half the bytes per MFMA.  The DCA mode
// boundaries are per workgroup, hence the one-chunk condition.
//
// HP (dense calls, NW = 4): the four waves serve one 64-row block of two query
// heads of one KV group (waves 0-1 and 2-3), which walk the same keys; with an
// odd number of heads per group the last pair has one head and its second pair
// of waves only keeps its place in the loads and barriers.
//
// HNF (sparse calls): the work items of KV heads with at most HN_MOVE_CAP
// high-norm keys, for which the plan marks the range tiles holding one.  For
// block-cover calls it also lists those keys with the extra keys, so a range
// tile masks its high-norm slots and needs no split-precision pass; with
// exact diagonals the marked tiles take the passes.  The instance without
// HNF takes the other heads and tests each tile's runs.
//
// wg: the work item's index in the launch order (the workgroup index, or the
// grid-stride position of the instance that serves few work items).
template <bool DENSE, bool EXACT, int NW = 2, bool HP = false, bool HNF = false>
__device__ __forceinline__ void attn_body(const AttnArgs& A, int wg) {
  static_assert(NW == 2 || (NW == 4 && DENSE), "four-wave workgroups serve dense calls");
  static_assert(!HP || NW == 4, "head pairs take four waves");
  constexpr int NR = HP ? 2 : NW;  // waves per row block
  constexpr int RB = 32 * NR;      // rows per block
  constexpr int LPW = 8 / NW;      // direct loads per wave and tensor of a tile
  constexpr int XL = EXACT ? 1 : 0;  // mask-word loads per lane and tile (exact diagonals)
  // K and V of the two stages are four LDS objects: the compiler then tells
  // the reads of one stage from the direct loads in flight into the other
  // and places no wait for those loads inside the tile's computation
  __shared__ __align__(16) uint8_t kst0[TILEB];
  __shared__ __align__(16) uint8_t vst0[TILEB];
  __shared__ __align__(16) uint8_t kst1[TILEB];
  __shared__ __align__(16) uint8_t vst1[TILEB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS bases stay scalar
  const int wrow = HP ? (wave & 1) : wave;   // the wave's rows in its block: 32 wrow ..
  const int hsub = HP ? (wave >> 1) : 0;     // its head in the pair
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
  if (A.bad && *A.bad) return;   // positions check failed: no output is written
  const int die = wg % NXCD;   // wg and the workgroup index agree modulo 8: same die
  const int local = wg / NXCD;
  const int hpg = A.h_q / A.h_kv;
  const int NBW = (A.nb + NR / 2 - 1) / (NR / 2);   // row groups of RB rows
  const int hpw = HP ? (hpg + 1) / 2 : hpg;          // work items per KV group and row
  int b, h, part;
  int mpos = 0;              // the block's place in its die's row sequence (split calls)
  bool idle = false;         // the absent second head of a pair (HP)
  if (NXCD % A.h_kv == 0) {
    const int dpg = NXCD / A.h_kv;                 // dies per KV group
    const int rows = (NBW + dpg - 1) / dpg;        // block rows of this die
    part = local / (rows * hpw);
    const int rem = local % (rows * hpw);
    // split calls: each die takes a contiguous half of the block rows (the
    // halves swap with the part), so the rows in flight on a die are adjacent
    // and read nearly the same keys; one part: rows interleave (balance)
    const int sub = die / A.h_kv;
    const int cidx = A.split > 1 ? ((sub + part) % dpg) * rows + rem % rows : dpg * (rem % rows) + sub;
    if (cidx >= NBW) return;
    b = NBW - 1 - cidx;
    mpos = A.split > 1 ? rem % rows : 0;
    h = ((die + part) % A.h_kv) * hpg + (HP ? 2 * (rem / rows) + hsub : rem / rows);
    idle = HP && 2 * (rem / rows) + hsub >= hpg;
  } else {
    const int rows = (NBW + NXCD - 1) / NXCD;
    part = local / (rows * A.h_kv * hpw);
    const int rem = local % (rows * A.h_kv * hpw);
    const int cidx = NXCD * (rem % rows) + die;
    if (cidx >= NBW) return;
    b = NBW - 1 - cidx;
    const int item = rem / rows;
    h = HP ? (item / hpw) * hpg + 2 * (item % hpw) + hsub : item;
    idle = HP && 2 * (item % hpw) + hsub >= hpg;
  }
  if (idle) h -= 1;   // a valid head for the addresses; nothing is computed or written
  const int g = h / (A.h_q / A.h_kv);
  if (!DENSE && HNF != (A.hnl_n[g] <= HN_MOVE_CAP)) return;   // the other instance's item

  const int i0 = A.p0 + RB * b;                  // absolute position of the block's first row
  const int rows = min(RB, A.n_q - RB * b);
  const int hi_key = i0 + rows;                  // keys [0, hi_key): the block's causal extent
  const int m_blk = i0 / A.S;
  const int rloc = 32 * wrow + l32;              // row inside the block owned by this lane
  const bool row_ok = rloc < rows;
  const int qrow = RB * b + (row_ok ? rloc : 0);
  const int prow = i0 + rloc;                    // absolute position of this lane's row
  // DCA mode of a key: 2 intra-chunk [segB, ..), 1 successive [segA, segB), 0 inter-chunk [0, segA)
  const int segA = max(0, (m_blk - 1) * A.S);
  const int segB = max(0, m_blk * A.S);

  const int unit = h * A.nb + b;
  const int* tl_h = (const int*)(A.tiles + (long long)h * A.tile_stride);
  const int t_first = DENSE ? 0 : A.t_first[unit];
  const int n_range = DENSE ? (hi_key + BN - 1) / BN : A.n_tiles[h] - t_first;
  const int32_t* ext_h = A.ext + (long long)unit * A.ext_stride;
  const int n_ext = DENSE ? 0 : A.n_ext[unit];
  const int n_all = n_range + (n_ext + BN - 1) / BN;
  const int t_beg = (int)((long long)n_all * part / A.split);
  const int t_end = (int)((long long)n_all * (part + 1) / A.split);

  const int kstride = A.h_kv * D;
  const uint16_t* kh_base = A.khi + g * D;
  const uint16_t* kl_base = A.klo + g * D;
  const uint16_t* v_base = A.v + g * D;
  const int grp = l32 >> 4;       // which 16-wide d slice of a 32-d block (transposed V reads)
  const int s16 = lane & 15;

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m_run = 0.f;         // reference max (log2 domain) of this row
  f32x16 negm = {};          // -m_run in every entry: the S^T MFMAs start from it, so the
                             // scores come out already shifted by the reference max
  bool started = false;      // the row has met a key
  float l_run = 0.f;         // this lane's partial row sum
  // rotated query row of this lane for the current DCA mode: the hi half is
  // held in registers (qh[kk]: dims 16kk + 8half .. +7), the lo half is read
  // back from global memory by high-norm tiles only.  Rows past the block's
  // end read row qrow (clamped) and are never written.
  bf16x8 qh[8];
  const uint16_t* ql_row = A.qlo;
  int q_mode = -1;
  auto load_q = [&](int mode) __attribute__((always_inline)) {
    const long long qo = (((long long)mode * A.n_q + qrow) * A.h_q + h) * D + 8 * half;
    const uint16_t* qh_row = A.qhi + qo;
    ql_row = A.qlo + qo;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qh[kk] = *(const bf16x8*)(qh_row + 16 * kk);
    // a mode change is rare: wait here, so that no wait for these loads is
    // left on the common path (where it would also drain the tile loads)
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    q_mode = mode;
  };

  // ---- tile metadata.  Range tiles: descriptor and high-norm bitmap words
  // through scalar loads (their waits do not hold the vector-memory queue of
  // the staged K / V loads); an extra-vertical tile's keys (one per slot,
  // lane & 31) with a vector load.
  typedef __attribute__((address_space(4))) const int ci32;
  typedef __attribute__((address_space(4))) const uint32_t cu32;
  ci32* tl4 = (ci32*)(A.tiles + (long long)h * A.tile_stride);
  auto desc_load = [&](int idx) __attribute__((always_inline)) -> int4 {
    if (DENSE || idx >= n_range || idx >= t_end) return make_int4(0, 0, 0, 0);
    ci32* d = tl4 + 4 * (t_first + idx);
    return make_int4(d[0], d[1], d[2], d[3]);
  };
  auto range_tile = [&](int idx, int4 d) __attribute__((always_inline)) -> Tile {
    Tile T;
    T.eoff = 0; T.cnt = 0;
    if (DENSE) {
      T.a1 = BN * idx;
      T.len1 = min(BN, hi_key - T.a1);
      T.a2 = 0; T.len2 = 0;
    } else {
      T.a1 = i0 + d.x;
      T.a2 = i0 + d.y;
      T.len1 = d.z & 0xFF;
      T.len2 = (d.z >> 8) & 0xFF;
    }
    return T;
  };
  auto ext_tile = [&](int idx) __attribute__((always_inline)) -> Tile {
    Tile T;
    T.a1 = 0; T.a2 = 0; T.len1 = 0; T.len2 = 0;
    T.eoff = BN * (idx - n_range);
    T.cnt = min(BN, n_ext - T.eoff);
    return T;
  };
  // a run [a, a + len) holds a high-norm key: the distance from its first
  // (non-negative) key to the next high-norm key is below its length (one
  // byte of the distance table, read through the scalar cache as its dword)
  cu32* hn4 = (cu32*)(A.hn + (long long)g * A.hn_pad);
  auto run_flagged = [&](int a, int len) __attribute__((always_inline)) -> bool {
    const int ac = max(a, 0);
    const int lc = len - (ac - a);
    if (lc <= 0) return false;
    const int d = (int)((hn4[ac >> 2] >> (8 * (ac & 3))) & 0xFFu);
    return d < lc;
  };
  auto range_precise = [&](Tile T) __attribute__((always_inline)) -> bool {
    return run_flagged(T.a1, T.len1) || run_flagged(T.a2, T.len2);
  };
  // HNF, block cover: the plan lists the covered high-norm keys with the
  // block's extra keys, so a range tile masks its high-norm slots, found in the
  // flag bitmap (two words per run; indexes clamped into it: the slots of keys
  // past n_k are masked anyway).
  cu32* kb4 = (cu32*)(A.kbits + (long long)g * A.kbits_words);
  auto run_hn = [&](int a, int len) __attribute__((always_inline)) -> uint32_t {   // bit t: key a + t high-norm
    const int ac = max(a, 0);
    const int sh = ac - a;
    if (sh >= len) return 0u;
    const int w = ac >> 5;
    const uint32_t w0 = kb4[min(w, A.kbits_words - 1)], w1 = kb4[min(w + 1, A.kbits_words - 1)];
    uint32_t v = (uint32_t)((((uint64_t)w1 << 32) | w0) >> (ac & 31));
    const int n = len - sh;
    if (n < 32) v &= (1u << n) - 1u;
    return v << sh;
  };
  // HNF: which range tiles hold a covered high-norm key, one bitmap word per
  // 32 tiles of the walk, read a step ahead of its use (its address depends on
  // the walk position only).  Dense tiles hold keys 32 t .. 32 t + 31: the
  // word of the flag bitmap with those keys, read a step ahead the same way.
  // Otherwise a test of the tile's runs.
  cu32* hbm4 = (cu32*)(HNF ? A.hnt + (long long)unit * A.hnt_words : A.hnt);
  auto flag_word = [&](int px) __attribute__((always_inline)) -> uint32_t {
    return HNF ? hbm4[px >> 5] : (DENSE ? kb4[min(px, A.kbits_words - 1)] : 0u);
  };
  auto tile_flagged = [&](Tile T, int px, uint32_t fw) __attribute__((always_inline)) -> bool {
    return HNF ? ((fw >> (px & 31)) & 1u) != 0u : (DENSE ? fw != 0u : range_precise(T));
  };
  // the slots to mask (HNF) and whether the split-precision passes are needed
  auto hn_split = [&](Tile T, bool flagged, uint32_t& mv) __attribute__((always_inline)) -> bool {
    mv = 0u;
    if (!flagged) return false;
    if (!HNF) return true;
    mv = run_hn(T.a1, T.len1) | (T.len1 < 32 ? run_hn(T.a2, T.len2) << T.len1 : 0u);
    return false;
  };
  // Exact-diagonal semantics: the slots of a range tile that this lane's row
  // attends are the tile's slash slots for the row (its offset prow - key is
  // selected, or 0) and the slots holding selected vertical columns.  The
  // slash slots depend on the row's place in the block only (the tile's keys
  // are offsets from the block's first row): the plan tabulates them per
  // (tile, row) and each lane loads its word two tiles ahead.  The vertical
  // bits of a run are the same for every row (scalar loads).
  typedef __attribute__((address_space(4))) const uint32_t cu32b;
  cu32b* vb4 = (cu32b*)(A.vbits + (long long)h * A.vbits_words);
  // mask words: a ring of 4 tiles x 64 lanes per wave, filled by direct loads
  // (lanes l and l + 32 load their row's word twice) two tiles ahead
  __shared__ __align__(16) uint32_t msk_[EXACT ? NW * 4 * 64 : 1];
  uint32_t* msk = msk_ + (EXACT ? wave * 4 * 64 : 0);
  const i32x4 rs_m = EXACT ? raw_rsrc(A.smask + (long long)h * A.tile_stride * 64, (uint32_t)A.tile_stride * 256u)
                           : i32x4{0, 0, 0, 0};
  auto mask_issue = [&](int idx, int slot) __attribute__((always_inline)) {   // tile idx of the walk (phys)
    if (!EXACT) return;
    const int t = min(t_first + idx, A.tile_stride - 1);   // tiles past the walk: any word (unused)
    dma_b32(rs_m, lds_addr(msk + 64 * (slot & 3)), (t * 64 + rloc) * 4);
  };
  auto mask_read = [&](int slot) __attribute__((always_inline)) -> uint32_t {
    return EXACT ? msk[64 * (slot & 3) + lane] : 0u;
  };
  // the vertical bits of both runs of a range tile at their slots; the four
  // words are loaded whatever the run lengths, so that one wait covers them.
  // A run starts below n_k + 96; one far below key 0 (the tail of an interval
  // in a block's first tile, all of its keys negative and masked) reads the
  // bitmap's first words instead.
  // The words are requested a step before the tile is computed (vert_words),
  // so no wait for them falls on the walk.
  struct VW { uint32_t w10, w11, w20, w21; };
  auto vert_words = [&](Tile T) __attribute__((always_inline)) -> VW {
    VW w = {0u, 0u, 0u, 0u};
    if (!EXACT || HNF) return w;   // HNF: the plan lists the covered columns with the extra keys
    const int b1 = max(T.a1 + 128, 0), b2 = max(T.a2 + 128, 0);
    w.w10 = vb4[b1 >> 5]; w.w11 = vb4[(b1 >> 5) + 1];
    w.w20 = vb4[b2 >> 5]; w.w21 = vb4[(b2 >> 5) + 1];
    return w;
  };
  auto vert_bits = [&](Tile T, VW w) __attribute__((always_inline)) -> uint32_t {
    const int b1 = max(T.a1 + 128, 0), b2 = max(T.a2 + 128, 0);
    const uint32_t v1 = (uint32_t)((((uint64_t)w.w11 << 32) | w.w10) >> (b1 & 31));
    const uint32_t v2 = (uint32_t)((((uint64_t)w.w21 << 32) | w.w20) >> (b2 & 31));
    const uint32_t m1 = T.len1 >= 32 ? 0xFFFFFFFFu : ((1u << T.len1) - 1u);
    const uint32_t m2 = T.len2 >= 32 ? 0xFFFFFFFFu : ((1u << T.len2) - 1u);
    return (v1 & m1) | (T.len1 < 32 ? (v2 & m2) << T.len1 : 0u);
  };
  // slot key of an extra-vertical tile (bit 30 marks a high-norm key), -1 past the count
  auto ext_key = [&](Tile T) __attribute__((always_inline)) -> int { return (l32 < T.cnt) ? ext_h[T.eoff + l32] : -1; };
  // K and V rows of this KV head through buffer resources: one 32-bit byte
  // offset per row serves both tensors (the host bounds n_k * h_kv * 256 < 2^32)
  const i32x4 rs_k = raw_rsrc(kh_base, 0xFFFFFFFFu);
  const i32x4 rs_v = raw_rsrc(v_base, 0xFFFFFFFFu);
  const int rowb = kstride * 2;
  const int lrow = lane >> 4;                       // row of a load's group this lane fills
  const int lchunk = 16 * ((lane & 15) ^ (5 * lrow));  // byte offset of the chunk it reads
  // byte offset of load j's row inside a tile of consecutive keys, plus the lane's chunk
  unsigned roff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) roff[j] = (unsigned)((4 * (NW * j + wave) + lrow) * rowb + lchunk);
  // Row offsets of a tile's direct loads: load j of wave w fills rows
  // 4(2j + w) .. +3 of the tile (lane: row lane >> 4, chunk (lane & 15) ^ 5(lane >> 4)).
  struct Offs { int v[4]; };
  // Rows past a tile's count read the keys after its last run; together with
  // negative keys (only in a block's first range tile) they can leave
  // [0, n_k) only in the prologue's tiles, in the block's first range tile and
  // in blocks within 95 keys of the end: there, and for extra-vertical tiles,
  // keys are clamped.
  const bool clamp_all = RB * b + RB + 31 >= A.n_q;
  auto tile_offsets = [&](Tile T, int skey, bool clamp) __attribute__((always_inline)) -> Offs {
    Offs f;
    if (clamp || T.cnt) {
#pragma unroll
      for (int j = 0; j < LPW; ++j) {
        const int r = 4 * (NW * j + wave) + lrow;
        int key;
        if (T.cnt) key = __shfl(skey, r) & 0x1FFFFFFF;
        else key = (r < T.len1 ? T.a1 : T.a2 - T.len1) + r;   // slots past the count are masked later
        key = min(max(key, 0), A.n_k - 1);
        f.v[j] = __umul24((unsigned)key, (unsigned)rowb) + lchunk;
      }
    } else if (T.len2 == 0) {
      const unsigned base = (unsigned)T.a1 * (unsigned)rowb;
#pragma unroll
      for (int j = 0; j < LPW; ++j) f.v[j] = (int)(base + roff[j]);
    } else {
      // rows from slot len1 on belong to run 2, a gap of a2 - a1 - len1 keys later
      const unsigned base = (unsigned)T.a1 * (unsigned)rowb;
      const unsigned gap = (unsigned)(T.a2 - T.a1 - T.len1) * (unsigned)rowb;
#pragma unroll
      for (int j = 0; j < LPW; ++j)
        f.v[j] = (int)(base + roff[j] + (lrow >= T.len1 - 4 * (NW * j + wave) ? gap : 0u));
    }
    return f;
  };
  // the 4 direct loads of one tensor of a tile into a stage
  auto issue = [&](i32x4 rs, uint8_t* stage, Offs f) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) dma_b128(rs, lds_addr(stage + (NW * j + wave) * GRPB), f.v[j]);
  };

  // ---- pipeline.  The K and V stages are released separately: step t
  //   B1: own loads of K(t) landed, barrier; then V(t+1) is issued into the V
  //       stage that V(t-1) held;
  //   S^T = K Q^T of tile t;
  //   B2: barrier (both waves are done with K(t)); then K(t+2) is issued into
  //       K(t)'s stage, with the metadata reads of the tiles after it;
  //   softmax;
  //   B3: own loads of V(t) landed, barrier; then O += P V.
  // So K is read about 1.5 steps and V about 2 steps after its loads were
  // issued.  A wave issues 4 direct loads per tile and tensor, also for tiles
  // past the end (clamped rows, never read), so the number of these loads
  // issued after any given one is fixed and the waits below count them (reads
  // of metadata in between only make a wait longer).  Barriers carry no memory
  // fence (a fence would wait for every load in flight).
  auto vm_wait = [&](int n) __attribute__((always_inline)) {   // at most n vector-memory ops outstanding
    if (n >= 14) __builtin_amdgcn_s_waitcnt(0x0F7E);
    else if (n >= 12) __builtin_amdgcn_s_waitcnt(0x0F7C);
    else if (n >= 9) __builtin_amdgcn_s_waitcnt(0x0F79);
    else if (n >= 8) __builtin_amdgcn_s_waitcnt(0x0F78);
    else if (n >= 6) __builtin_amdgcn_s_waitcnt(0x0F76);
    else if (n >= 4) __builtin_amdgcn_s_waitcnt(0x0F74);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
  };
  auto wg_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS reads are done
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // DCA mode of a key: 2 intra-chunk [segB, ..), 1 successive [segA, segB),
  // 0 inter-chunk [0, segA); sign-bit arithmetic keeps it scalar
  auto key_mode = [&](int key) __attribute__((always_inline)) -> int {
    return (int)((unsigned)(segA - 1 - key) >> 31) + (int)((unsigned)(segB - 1 - key) >> 31);
  };

  // One DCA mode's pass over the staged tile: S^T = K Q^T (+ the lo terms of a
  // high-norm tile), the masks (masked passes only), the online softmax and
  // O^T += V^T P^T.
  // S^T = K Q^T of the staged tile for one DCA mode's query rotation (+ the
  // lo terms of a high-norm tile)
  auto qk = [&](const uint8_t* kt, Tile T, int skey, int mode, bool precise) __attribute__((always_inline))
      -> f32x16 {
    if (mode != q_mode) load_q(mode);
    // 32 keys x 32 rows of this wave (scores in log2 units)
    f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(kt + tile_off(l32, half)), qh[0],
                                                       negm, 0, 0, 0);
#pragma unroll
    for (int kk = 1; kk < 8; ++kk) {
      const bf16x8 a = *(const bf16x8*)(kt + tile_off(l32, 2 * kk + half));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qh[kk], s, 0, 0, 0);
    }
    if (precise) {
      // + K_lo Q_hi + K_hi Q_lo; K_lo rows come straight from global memory
      int kr = T.cnt ? (skey & 0x1FFFFFFF) : range_key(T, l32);
      kr = min(max(kr, 0), A.n_k - 1);
      const uint16_t* klrow = kl_base + kr * kstride;
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

  // A tile.  Its keys ascend with the slot, so each DCA mode's keys fill one
  // interval of slots, and so do the keys inside [0, row].  S^T is computed
  // once per mode the tile holds and merged slot by slot; slots outside
  // [0, row] or past the count are masked (only tiles at the block's edges
  // have such slots).  Then one online softmax and one O += P V.  after_qk
  // runs once S^T is done (B2 and the K issue), B3 before the V reads.
  auto compute_tile = [&](const uint8_t* kt, const uint8_t* vt, Tile T, int skey, bool precise, uint32_t smk,
                          uint32_t mv, VW vw, auto&& after_qk) __attribute__((always_inline)) {
    const int count = tile_count(T);
    int key_first, key_last;
    if (T.cnt) {
      key_first = __builtin_amdgcn_readlane(skey, 0) & 0x1FFFFFFF;
      key_last = __builtin_amdgcn_readlane(skey, count - 1) & 0x1FFFFFFF;
    } else {
      key_first = T.a1;
      key_last = T.len2 ? T.a2 + T.len2 - 1 : T.a1 + T.len1 - 1;
    }
    const int mode_first = key_mode(max(key_first, 0));   // negative keys are masked
    const int mode_last = key_mode(key_last);
    // number of the tile's keys below x
    auto below = [&](int x) __attribute__((always_inline)) -> int {
      if (T.cnt) {
        const int kj = skey & 0x1FFFFFFF;
        return __builtin_popcountll(__ballot(l32 < T.cnt && half == 0 && kj < x));
      }
      return min(max(x - T.a1, 0), T.len1) + min(max(x - T.a2, 0), T.len2);
    };
    // keep s[vv] where its slot (c + 4 half) lies in [t_lo, t_hi), else take alt
    auto select_slots = [&](f32x16& s, int t_lo, int t_hi, float alt) __attribute__((always_inline)) {
      const int base = t_lo - 4 * half;
      const unsigned span = (unsigned)max(t_hi - t_lo, 0);
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int c = 8 * (vv >> 2) + (vv & 3);
        if ((unsigned)(c - base) >= span) s[vv] = alt;
      }
    };
    // Exact diagonals: the rows' masks first.  A tile none of the wave's rows
    // attends costs no MFMA, softmax or P V: the wave only keeps its place in
    // the step's loads and barriers.
    uint32_t xm = 0u;
    bool skip = HP && idle;
    if (EXACT && !T.cnt) {
      // the listed high-norm keys are attended in the extra tiles
      xm = (smk | (HNF ? 0u : vert_bits(T, vw))) & ~mv;
      skip = !__any(xm != 0u);
    }
    f32x16 s = {};
    bf16x8 pf[2] = {};
    if (!skip) {
    s = qk(kt, T, skey, mode_first, precise);
    // slots from the first key of mode m on take that mode's scores (the
    // modes after the first are spelled out: a loop here would make the
    // compiler wait for the staged loads in flight before every S^T)
    auto merge_mode = [&](int m) __attribute__((always_inline)) {
      const int tb = below(m == 2 ? segB : segA);
      const f32x16 s2 = qk(kt, T, skey, m, precise);
      const int base = tb - 4 * half;
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int c = 8 * (vv >> 2) + (vv & 3);
        if (c >= base) s[vv] = s2[vv];
      }
    };
    if (mode_first + 1 <= mode_last) merge_mode(mode_first + 1);
    if (mode_first + 2 <= mode_last) merge_mode(mode_first + 2);
    if (!(EXACT && HNF && T.cnt) && (count < BN || key_first < 0 || key_last > i0)) {
      // the keys of an extra tile at or above the block's first row (listed
      // high-norm keys) are its ascending last slots: the row keeps the slots
      // of the tile's keys up to its own position, counted slot by slot
      // (below() counts for wave-uniform bounds only)
      const int t_lo = T.cnt ? 0 : below(0);
      int t_hi;
      if (T.cnt) {
        t_hi = 0;
        for (int t = 0; t < count; ++t) t_hi += (__builtin_amdgcn_readlane(skey, t) & 0x1FFFFFFF) <= prow;
      } else {
        t_hi = below(prow + 1);
      }
      select_slots(s, t_lo, t_hi, -INFINITY);
    }
    if (HNF && !EXACT && mv) {
      // high-norm keys taken by the extra list: slot c + 4 half is bit c of xh
      const uint32_t xh = mv >> (4 * half);
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int c = 8 * (vv >> 2) + (vv & 3);
        if ((xh >> c) & 1u) s[vv] = -INFINITY;
      }
    }
    if (EXACT && T.cnt && HNF) {
      // extra tiles: an entry with bit 29 (a covered high-norm key or a
      // covered vertical column) is attended by the rows of its row mask,
      // which the plan stores after the block's list (two words per entry:
      // rows 0-31, 32-63; causal included); the other entries are vertical
      // columns the ranges miss, attended by every row they do not follow.
      // The entries of a mode are not in key order, so each slot is tested.
      const int E = A.ext_stride / 3;
      uint32_t xh = 0u;
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int c = 8 * (vv >> 2) + (vv & 3);
        const int slot = c + 4 * half;
        const int e = __shfl(skey, slot);
        const int idx = min(T.eoff + slot, E - 1);
        const uint32_t w = (uint32_t)ext_h[E + 2 * idx + wrow];
        const bool keep = slot < count && (((e >> 29) & 1) ? ((w >> l32) & 1u) != 0u : (e & 0x1FFFFFFF) <= prow);
        xh |= (uint32_t)keep << c;
      }
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int c = 8 * (vv >> 2) + (vv & 3);
        if (!((xh >> c) & 1u)) s[vv] = -INFINITY;
      }
    }
    if (EXACT && !T.cnt) {
      // bit c of xh is slot c + 4 half; each score keeps s - m_run where its
      // bit is set (a sign-extended 1-bit field selects it), else -inf
      const uint32_t xh = xm >> (4 * half);
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int c = 8 * (vv >> 2) + (vv & 3);
        const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)xh, c, 1);
        s[vv] = __uint_as_float((__float_as_uint(s[vv]) & sel) | (0xFF800000u & ~sel));
      }
    }
    }
    after_qk();
    if (!skip) {
    // ---- online softmax (log2 domain; s already holds score - m_run).  The
    // reference max moves only when a score exceeds it by more than 8 (so
    // p <= 2^8), or at the row's first keys.
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
        negm[vv] -= shift;   // = -m_run exactly, updated in place
      }
    }
    started = started || (mx != -INFINITY);
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) pf[vv >> 3][vv & 7] = (__bf16)fast_exp2(s[vv]);
    // row sum of the bf16 weights that enter P V (pairs summed by dot products)
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int G = 0; G < 2; ++G) {
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[G], pf[G], 0, 1), ones, l_run, false);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[G], pf[G], 2, 3), ones, l_run, false);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[G], pf[G], 4, 5), ones, l_run, false);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[G], pf[G], 6, 7), ones, l_run, false);
    }
    }
    // B3: this wave's loads of V(t) landed (issued after them: K(t+1), V(t+1)
    // and K(t+2), and in the exact walk the mask words of t+1 and t+2); barrier
    vm_wait(3 * LPW + 2 * XL);
    wg_barrier();
    if (skip) return;
    // ---- O^T += V^T P^T, V^T operand read transposed from the row-major V tile.
    // All 8 reads of a 16-key half are issued before its 4 MFMAs, so their
    // latency overlaps instead of stalling every MFMA.
#pragma unroll
    for (int G = 0; G < 2; ++G) {
      const int r1 = 16 * G + 4 * half + (s16 >> 2);
      const int r2 = r1 + 8;
      bf16x8 a[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int c = 4 * db + 2 * grp + ((s16 & 3) >> 1);     // 16-byte chunk of the 4 columns read
        const int bo = 8 * (s16 & 1);                           // byte offset inside the chunk
        const bf16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, vt + tile_off(r1, c) + bo));
        const bf16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, vt + tile_off(r2, c) + bo));
        a[db] = __builtin_shufflevector(t1, t2, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[db], pf[G], o[db], 0, 0, 0);
    }
  };

  const Tile T_dummy = {0, 0, BN, 0, 0, 0};   // rows 0..31, for loads past the last tile

  // ---- range tiles [t_beg, r_end), pipelined.  Prologue: K(t0), V(t0),
  // K(t0+1) in flight, the descriptor of t0+2 requested.
  const int r_end = min(t_end, n_range);
  const int t0 = t_beg;
  // Staggered start.  The range tiles of a part are walked from a rotated
  // start, tile t_beg + shift, wrapping at r_end.  A block's tiles are offsets
  // relative to its first row, so blocks b and b+1 read the same key about
  // two tiles apart in their walks (64 keys, at the covered density); with
  // the shift growing with the block's place on its die, the blocks in flight
  // on a die read close keys at the same time and their loads are served by
  // the die's L2 (at 1M: 2.07 -> 0.22 TB fetched per launch).  The shift is
  // twice the block's mean tiles per 64 keys per place (measured best at 128K
  // and 1M), modulo the part's length; dense tiles are absolute and keep the
  // order.
  const int n_part = max(r_end - t_beg, 1);
  const int shift = DENSE ? 0 : (int)(((long long)mpos * n_range * 128 / max(hi_key, 1)) % n_part);
  auto phys = [&](int x) __attribute__((always_inline)) -> int {
    if (x >= r_end) return x;   // past the walk: dummy tiles
    const int p = x + shift;
    return p < r_end ? p : p - n_part;
  };
  Tile T_c = range_tile(phys(t0), desc_load(phys(t0)));
  const Offs f_c = tile_offsets(t0 < r_end ? T_c : T_dummy, -1, true);
  mask_issue(phys(t0), t0);
  issue(rs_k, kst0, f_c);
  issue(rs_v, vst0, f_c);
  uint32_t mv_c = 0u;
  bool p_c = t0 < r_end && hn_split(T_c, tile_flagged(T_c, phys(t0), flag_word(phys(t0))), mv_c);
  Tile T_n = range_tile(phys(t0 + 1), desc_load(phys(t0 + 1)));
  Offs f_n = tile_offsets(t0 + 1 < r_end ? T_n : T_dummy, -1, true);
  mask_issue(phys(t0 + 1), t0 + 1);
  issue(rs_k, kst1, f_n);
  uint32_t mv_n = 0u;
  bool p_n = t0 + 1 < r_end && hn_split(T_n, tile_flagged(T_n, phys(t0 + 1), flag_word(phys(t0 + 1))), mv_n);
  uint32_t fw_2 = flag_word(phys(t0 + 2));   // the flag word of the next step's third tile
  VW vw_c = vert_words(T_c), vw_n = {0u, 0u, 0u, 0u};
  int4 d_2 = desc_load(phys(t0 + 2));

  // One step on range tile ti: its stages kc / vc, and vn, the V stage of tile ti+1.
  auto step = [&](uint8_t* kc, const uint8_t* vc, uint8_t* vn, int ti) __attribute__((always_inline)) {
    // K(ti) (and its mask words) landed: V(ti), K(ti+1) (and the mask words
    // of ti+1) were issued after it
    vm_wait(2 * LPW + XL);
    wg_barrier();          // B1: K(ti) visible; V(ti-1)'s stage is free
    issue(rs_v, vn, f_n);
    bool p_2 = false;
    uint32_t mv_2 = 0u;
    Offs f_2;
    Tile T_2 = T_dummy;
    auto after_qk = [&]() __attribute__((always_inline)) {
      wg_barrier();        // B2: both waves are done with K(ti)
      const int px = phys(ti + 2);
      T_2 = range_tile(px, d_2);
      // the block's first range tile (negative keys) may now come after the prologue
      f_2 = tile_offsets(ti + 2 < r_end ? T_2 : T_dummy, -1, clamp_all || px == 0);
      mask_issue(px, ti + 2);
      issue(rs_k, kc, f_2);
      p_2 = ti + 2 < r_end && hn_split(T_2, tile_flagged(T_2, px, fw_2), mv_2);
      fw_2 = flag_word(phys(ti + 3));
      vw_n = vert_words(T_n);
      d_2 = desc_load(phys(ti + 3));
    };
    compute_tile(kc, vc, T_c, -1, p_c, mask_read(ti), mv_c, vw_c, after_qk);
    T_c = T_n; p_c = p_n; mv_c = mv_n; vw_c = vw_n;
    T_n = T_2; p_n = p_2; mv_n = mv_2; f_n = f_2;
  };
  for (int ti = t_beg; ti < r_end; ti += 2) {
    step(kst0, vst0, vst1, ti);
    if (ti + 1 < r_end) step(kst1, vst1, vst0, ti + 1);
  }
  // the clamped loads past the last range tile land before the stages are reused
  vm_wait(0);
  wg_barrier();

  // ---- extra-vertical tiles (a few per block, after the range tiles): keys,
  // then K and V, then the tile, one at a time
  for (int ti = max(t_beg, n_range); ti < t_end; ++ti) {
    const Tile T = ext_tile(ti);
    const int sk = ext_key(T);
    const bool prec = __any(sk >= 0 && ((sk >> 30) & 1));
    const Offs f = tile_offsets(T, sk, true);
    issue(rs_k, kst0, f);
    issue(rs_v, vst0, f);
    vm_wait(0);
    wg_barrier();
    compute_tile(kst0, vst0, T, sk, prec, 0u, 0u, VW{0u, 0u, 0u, 0u}, [] {});
    wg_barrier();          // the stage is read; the next tile may overwrite it
  }

  // ---- finish: row sum over both halves, normalise, write
  const float l_tot = pair_sum(l_run);
  const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse2 = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
  const float lse = lse2 * 0.69314718055994531f;
  if (!row_ok || idle) return;
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
    // the normalised partial in fp16 (values within max |v|; 2^-11 relative,
    // well below the bf16 rounding of the merged output), half the bytes the
    // merge reads
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

// sparse (vertical-slash) calls, sparse calls with exact diagonals, and dense
// calls: one body, the variant known at compile time (the exact masks cost
// registers the other two do not pay for)
__global__ void __launch_bounds__(128, 2) dca_attn_kernel(AttnArgs A) { attn_body<false, false, 2, false, true>(A, blockIdx.x); }
__global__ void __launch_bounds__(128, 2) dca_attn_exact_kernel(AttnArgs A) { attn_body<false, true, 2, false, true>(A, blockIdx.x); }
// KV heads with many high-norm keys are rare: these instances walk the work
// items grid-stride over a bounded grid (a multiple of 8 workgroups, so an
// item stays on its die), which costs little when none of the items is theirs
__device__ __forceinline__ bool some_head_has_many_high_norm_keys(const AttnArgs& A) {
  bool many = false;
  for (int g = 0; g < A.h_kv; ++g) many = many || A.hnl_n[g] > HN_MOVE_CAP;
  return many;
}
__global__ void __launch_bounds__(128, 2) dca_attn_hn_kernel(AttnArgs A, int items) {
  if (!some_head_has_many_high_norm_keys(A)) return;
  for (int w = blockIdx.x; w < items; w += gridDim.x) attn_body<false, false>(A, w);
}
__global__ void __launch_bounds__(128, 2) dca_attn_exact_hn_kernel(AttnArgs A, int items) {
  if (!some_head_has_many_high_norm_keys(A)) return;
  for (int w = blockIdx.x; w < items; w += gridDim.x) attn_body<false, true>(A, w);
}
__global__ void __launch_bounds__(128, 2) dca_attn_dense_kernel(AttnArgs A) { attn_body<true, false>(A, blockIdx.x); }
__global__ void __launch_bounds__(256, 2) dca_attn_dense4_kernel(AttnArgs A) { attn_body<true, false, 4>(A, blockIdx.x); }
__global__ void __launch_bounds__(256, 2) dca_attn_dense_hp_kernel(AttnArgs A) { attn_body<true, false, 4, true>(A, blockIdx.x); }

// LSE merge of the key parts of one (row, head): m = max_p lse_p,
// O = sum_p e^{lse_p - m} O_p / sum_p e^{lse_p - m}.  One wave per (row, head):
// the row's parts are contiguous (P x 128 halves), lane l takes dims
// 8 (l % 16) .. + 7 of parts l / 16, l / 16 + 4, ..., so each load
// instruction reads 1 KB; the four part groups are combined by shuffles.
__global__ void __launch_bounds__(256) lse_merge_kernel(const uint16_t* __restrict__ part_o,
                                                        const float* __restrict__ part_lse,
                                                        uint16_t* __restrict__ out, float* __restrict__ lse_out,
                                                        int P, int n_q, int h_q, const int32_t* bad) {
  if (bad && *bad) return;   // positions check failed: no output is written
  const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (item >= (long long)n_q * h_q) return;
  const int row = (int)(item / h_q);
  const int h = (int)(item % h_q);
  const int pg = lane >> 4;        // part group
  const int dc = lane & 15;        // dims 8 dc .. 8 dc + 7
  const float* lse_row = part_lse + ((long long)h * n_q + row) * P;
  const uint16_t* o_row = part_o + ((long long)row * h_q + h) * P * D + 8 * dc;
  float m = -INFINITY;
  for (int p = pg; p < P; p += 4) m = fmaxf(m, lse_row[p]);
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (m != -INFINITY) {
#pragma unroll 4
    for (int p = pg; p < P; p += 4) {
      const float lp = lse_row[p];
      const float w = (lp == -INFINITY) ? 0.f : __expf(lp - m);
      const uint4 hx = *(const uint4*)(o_row + (long long)p * D);
      const uint32_t wd[4] = {hx.x, hx.y, hx.z, hx.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += w * f16_bits_to_f32(wd[i] & 0xFFFFu);
        acc[2 * i + 1] += w * f16_bits_to_f32(wd[i] >> 16);
      }
      wsum += w;
    }
  }
  // combine the four part groups (lanes dc, dc + 16, dc + 32, dc + 48), in a fixed order
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc[i] += __shfl_xor(acc[i], 16);
    acc[i] += __shfl_xor(acc[i], 32);
  }
  wsum += __shfl_xor(wsum, 16);
  wsum += __shfl_xor(wsum, 32);
  if (pg != 0) return;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  uint4 pk;
  pk.x = f32_to_bf16_bits(acc[0] * inv) | ((uint32_t)f32_to_bf16_bits(acc[1] * inv) << 16);
  pk.y = f32_to_bf16_bits(acc[2] * inv) | ((uint32_t)f32_to_bf16_bits(acc[3] * inv) << 16);
  pk.z = f32_to_bf16_bits(acc[4] * inv) | ((uint32_t)f32_to_bf16_bits(acc[5] * inv) << 16);
  pk.w = f32_to_bf16_bits(acc[6] * inv) | ((uint32_t)f32_to_bf16_bits(acc[7] * inv) << 16);
  *(uint4*)(out + ((long long)row * h_q + h) * D + 8 * dc) = pk;
  if (lse_out && dc == 0) lse_out[(long long)h * n_q + row] = (wsum > 0.f) ? m + __logf(wsum) : -INFINITY;
}

hipError_t launch_attn(const AttnArgs& A, hipStream_t stream) {
  // every die runs split * (its block rows) * (heads per row) workgroups
  // dense calls: workgroups of two blocks (128 rows) when no pair can straddle
  // a DCA chunk boundary (the workgroup's rows must share one chunk), i.e. S
  // and p0 multiples of 128; else one block per workgroup
  // dense calls whose block pairs may straddle a chunk, with an even number of
  // query heads per KV group: workgroups of two heads of one block instead
  // (the same sharing of each staged tile; with an odd number per group the
  // idle half of the last pair costs more than the sharing gains)
  const int hpg = A.h_q / A.h_kv;
  const bool pairs = A.dense && A.S % 128 == 0 && A.p0 % 128 == 0;
  if (A.dense && !pairs && hpg % 2 == 0) {
    const int hpw = hpg / 2;
    const int blocks = NXCD % A.h_kv == 0 ? NXCD * A.split * ((A.nb + NXCD / A.h_kv - 1) / (NXCD / A.h_kv)) * hpw
                                          : NXCD * A.split * ((A.nb + NXCD - 1) / NXCD) * A.h_kv * hpw;
    hipLaunchKernelGGL(dca_attn_dense_hp_kernel, dim3(blocks), dim3(256), 0, stream, A);
    return hipGetLastError();
  }
  const int nbw = pairs ? (A.nb + 1) / 2 : A.nb;
  const int blocks = NXCD % A.h_kv == 0
      ? NXCD * A.split * ((nbw + NXCD / A.h_kv - 1) / (NXCD / A.h_kv)) * (A.h_q / A.h_kv)
      : NXCD * A.split * ((nbw + NXCD - 1) / NXCD) * A.h_q;
  if (pairs) {
    hipLaunchKernelGGL(dca_attn_dense4_kernel, dim3(blocks), dim3(256), 0, stream, A);
  } else if (A.dense) {
    hipLaunchKernelGGL(dca_attn_dense_kernel, dim3(blocks), dim3(128), 0, stream, A);
  } else {
    // KV heads with few high-norm keys, then the others (each launch leaves the
    // other's work items alone; blocks is a multiple of 8)
    const int hn_grid = std::min(blocks, 2048);
    if (A.exact) {
      hipLaunchKernelGGL(dca_attn_exact_kernel, dim3(blocks), dim3(128), 0, stream, A);
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
      hipLaunchKernelGGL(dca_attn_exact_hn_kernel, dim3(hn_grid), dim3(128), 0, stream, A, blocks);
    } else {
      hipLaunchKernelGGL(dca_attn_kernel, dim3(blocks), dim3(128), 0, stream, A);
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
      hipLaunchKernelGGL(dca_attn_hn_kernel, dim3(hn_grid), dim3(128), 0, stream, A, blocks);
    }
  }
  return hipGetLastError();
}

hipError_t launch_lse_merge(const uint16_t* part_o, const float* part_lse, uint16_t* out, float* lse_out,
                            int P, int n_q, int h_q, const int32_t* bad, hipStream_t stream) {
  const long long items = (long long)n_q * h_q;
  const int blocks = (int)((items + 3) / 4);      // one wave per (row, head), four per workgroup
  hipLaunchKernelGGL(lse_merge_kernel, dim3(blocks), dim3(256), 0, stream, part_o, part_lse, out, lse_out,
                     P, n_q, h_q, bad);
  return hipGetLastError();
}

}  // namespace dca
