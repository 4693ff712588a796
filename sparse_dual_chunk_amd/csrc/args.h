// Argument blocks of the kernels, shared by the kernels and the host entry points.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dca {

// A sparse call whose KV head has at most HN_MOVE_CAP high-norm keys takes the
// covered ones out of a block's range tiles (there they are masked, so those
// tiles need one MFMA pass) and lists them with the block's extra-vertical keys
// (split-precision logits; with exact diagonals each with a mask of the block
// rows that attend it).
constexpr int HN_MOVE_CAP = 1024;

struct AttnArgs {
  const uint16_t* qhi;      // [3 modes][n_q][h_q][128] rotated query * scale * log2(e), bf16 hi
  const uint16_t* qlo;      // same, lo residual
  const uint16_t* khi;      // [n_k][h_kv][128] rotated, bf16 hi
  const uint16_t* klo;      // same, lo residual
  const uint16_t* v;        // [n_k][h_kv][128]
  const uint32_t* kbits;    // [h_kv][kbits_words] bit j: key j is high-norm (split-precision logits)
  const uint8_t* hn;        // [h_kv][hn_pad] distance from key j to the next high-norm key, capped at 64
  uint16_t* out;            // [n_q][h_q][128]
  float* lse_out;           // [h_q][n_q] or null
  uint16_t* part_o;         // [n_q][h_q][P][128] fp16 normalised partials (P > 1)
  float* part_lse;          // [h_q][n_q][P]      (P > 1)
  const int4* tiles;        // [h_q][tile_stride] range tiles in offset space: {o1, o2, len1 | len2 << 8, 0}
  const int32_t* n_tiles;   // [h_q]
  const int32_t* t_first;   // [h_q][nb] first range tile of each query block
  const int32_t* ext;       // [h_q][nb][ext_stride] vertical keys outside the ranges and, with few high-norm
                            // keys, the covered high-norm keys of the block's extent (bit 30: high-norm,
                            // bit 29: a covered key taken from the range tiles), ordered by DCA mode; with
                            // exact diagonals ext_stride = 3E: E entries, then a row mask (2 words) per entry
  const int32_t* n_ext;     // [h_q][nb]
  const uint32_t* dbits;    // exact diagonals: [h_q][dbits_words] bit delta + 128 = selected offset (and 0)
  const uint32_t* vbits;    // exact diagonals: [h_q][vbits_words] bit j + 128 = selected vertical column
  const uint32_t* smask;    // exact diagonals: [h_q][tile_stride][64] slots of range tile t whose offset
                            // from block row r is selected (or 0); the same for every block of the head
  int n_q, n_k, h_q, h_kv, p0, S, W, nb, tile_stride, ext_stride, split, dense, kbits_words, hn_pad;
  int exact, dbits_words, vbits_words;
  const int32_t* bad;       // device flag set by the positions check: write no output when nonzero (or null)
  const int32_t* hnl_n;     // [h_kv] how many high-norm keys the head has (counting stops past HN_MOVE_CAP)
  const uint32_t* hnt;      // [h_q][nb][hnt_words] bit i: range tile i of the block (from its first) holds a
                            // listed high-norm key (KV heads with at most HN_MOVE_CAP of them)
  int hnt_words;
};

struct DecArgs {
  const uint16_t* qhi;      // [3 modes][n_t][h_q][128] rotated token rows * scale * log2(e), bf16 hi
  const uint16_t* qlo;      // same, lo residual
  const uint16_t* khi;      // key cache [capacity][h_kv][128] rotated, bf16 hi
  const uint16_t* klo;      // same, lo residual
  const uint32_t* kflags;   // [h_kv][kflag_words] bit j: key j is high-norm
  const uint16_t* v;        // [capacity][h_kv][128]
  float* part_o;            // [P][n_t][h_q][128] normalised partial outputs
  float* part_lse;          // [P][h_q][n_t] natural-log partial LSE
  int n_t, n_k, h_q, h_kv, S, kflag_words, part_keys, n_parts, n_cb;
  // paged cache: khi / klo / v are pools of n_pages pages of page_keys rows,
  // kflags is [n_pages][h_kv][page_keys / 32], logical page p of the sequence
  // is pool page ptab[p] (clamped into [0, n_pages))
  const int32_t* ptab;
  int page_keys, n_pages;
};

struct VsArgs {
  const uint16_t* k;         // raw keys [n_k][h_kv][128]
  const double* qs;          // [2][h_q][64][128] scoring rows rotated at r_i ([0]) and S + r_i ([1])
  const double* inv_freq;    // [64]
  double* part_ms;           // [h_q][n_ranges][64][2] pass-1 (max, sum) per row and range
  const double* lse;         // [h_q][64]
  double* vert;              // [h_q][n_k]
  double* slash;             // [h_q][n_off], n_off = p_last + 1
  double* edge;              // [h_q][n_ranges][2][64][2] double-double partial diagonals at range edges
  double* logits;            // [h_q][64][n_k] scaled logits of pass 1 (read back by pass 2)
  double2* trig;             // [S / 8][64] (cos, sin) of the key positions 8a, a < S / 8
  int n_k, h_q, h_kv, S, n_s, p_first, range_keys, n_ranges, n_off;
  double scale;
};

struct SelArgs {
  const double* vert;      // [h_q][n_v]
  const double* slash;     // [h_q][n_s]
  int32_t* v_out;          // [h_q][k_v]
  int32_t* s_out;          // [h_q][k_s]
  int h_q, n_v, n_sl, k_v, k_s;
  uint32_t* hist;          // [2*h_q][256]
  uint64_t* prefix;        // [2*h_q]
  int32_t* krem;           // [2*h_q]
  uint32_t* bcount;        // [2*h_q][max_blocks][2] (gt, eq)
  int max_blocks;
  const int32_t* k_head;   // optional [h_q][2] per-head (k_v, k_s), clamped to [0, k_v / k_s]
  const int32_t* bad;      // device flag set by the positions check: write no output when nonzero (or null)
};

struct PlanArgs {
  const int32_t* v_idx;    // [h_q][k_v]
  const int32_t* s_off;    // [h_q][k_s]
  int32_t* iv;             // [h_q][iv_stride][2]
  int32_t* iv_pre;         // [h_q][iv_stride + 1] covered offsets before interval k
  int32_t* n_iv;           // [h_q]
  uint32_t* cov;           // [h_q][cov_words] bitmap over offsets o in [-p_last, 64)
  int32_t* cov_pre;        // [h_q][cov_words] set bits of cov before each word
  int32_t* ext;            // [h_q][nb][ext_stride]
  int32_t* n_ext;          // [h_q][nb]
  int4* tiles;             // [h_q][tile_stride]
  int32_t* n_tiles;        // [h_q]
  int32_t* t_first;        // [h_q][nb]
  const uint32_t* kbits;   // [h_kv][kbits_words]
  long long* cover_pairs;  // optional: sum of rows * |cover| over all (head, block)
  long long* attended;     // optional: sum over heads and rows of the attended (row, key) pairs
  const int32_t* bad;      // device flag set by the positions check: write no output when nonzero (or null)
  const int32_t* hnl_n;    // [h_kv] how many high-norm keys the head has (counting stops past HN_MOVE_CAP)
  const int32_t* hnall;    // [h_kv][HN_MOVE_CAP] the first high-norm keys of each KV head, ascending
  uint32_t* hnt;           // [h_q][nb][hnt_words] range tiles holding a listed high-norm key
  int hnt_words;
  int S;                   // DCA chunk size
  uint32_t* dbits;         // exact diagonals (or null): [h_q][dbits_words], bit delta + 128
  uint32_t* vbits;         // exact diagonals (or null): [h_q][vbits_words], bit j + 128
  uint32_t* smask;         // exact diagonals (or null): [h_q][tile_stride][64] slash slots of (tile, block row)
  int h_q, h_kv, k_v, k_s, p_last, p0, n_q, nb, iv_stride, ext_stride, cov_words, tile_stride, kbits_words;
  int dbits_words, vbits_words;
};

}  // namespace dca
