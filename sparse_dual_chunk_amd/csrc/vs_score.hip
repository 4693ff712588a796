// Vertical-slash scoring in float64 (v_mfma_f64_16x16x4f64) for the index builder.
//
// The sparse attention of the paper-review page (section 4, Figure 4) picks
// key columns ("vertical") and diagonals ("slash") per head and per prefill
// chunk, restoring continuous relative positions while it picks.  The last
// scoring rows of the chunk (at most 64) are scored against every causal key:
// query position r_i for keys of the row's own DCA chunk, S + r_i for keys of
// any earlier chunk, key position r_j.  Pass 1 gives each row's log-sum-exp;
// pass 2 turns logits into probabilities and sums them by column and by
// diagonal (offset delta = p_i - j).  Sums are double-double, so that equal
// multisets of terms give bitwise equal sums however the key range was split.
//
// Grid: one workgroup per (key range, query head); wave w holds scoring rows
// 16w..16w+15 as the A operand, the 32-key sub-tile of rotated keys sits in
// LDS as fp64 and feeds the B operand.
#include <type_traits>

#include "common.h"
#include "args.h"

namespace dca {

constexpr int SUB = 32;    // keys per sub-tile
constexpr int KPD = 130;   // LDS pitch of fp64 key rows (260 dwords: 16 rows x 2 dims per half-wave on distinct banks)
constexpr int APD = 33;    // LDS pitch of the probability tile (doubles)
constexpr int RING = 128;  // diagonal accumulators kept alive across sub-tiles


// Rotated scoring rows in fp64: position r_i (variant 0) and S + r_i (variant 1).
__global__ void __launch_bounds__(256) vs_prep_q_kernel(const uint16_t* __restrict__ q, double* __restrict__ qs,
                                                        const double* __restrict__ inv_freq,
                                                        int n_q, int h_q, int S, int n_s, int p_first) {
  const int h = blockIdx.x;
  for (int idx = threadIdx.x; idx < 64 * HALF; idx += blockDim.x) {
    const int t = idx / HALF;      // scoring row
    const int c = idx % HALF;      // pair
    double x = 0.0, y = 0.0;
    const int p = p_first + t;
    if (t < n_s) {
      const int row = n_q - n_s + t;
      const uint16_t* src = q + ((long long)row * h_q + h) * D;
      x = (double)bf16_bits_to_f32(src[c]);
      y = (double)bf16_bits_to_f32(src[c + HALF]);
    }
    const int r = (t < n_s) ? p % S : 0;
#pragma unroll
    for (int var = 0; var < 2; ++var) {
      const double pos = (double)(var == 0 ? r : S + r);
      double sn, cs;
      sincos(pos * inv_freq[c], &sn, &cs);
      double* dst = qs + (((long long)var * h_q + h) * 64 + t) * D;
      dst[c] = x * cs - y * sn;
      dst[c + HALF] = x * sn + y * cs;
    }
  }
}

// Anchor rotations of the key positions that are multiples of 8:
// trig[p / 8][c] = (cos, sin)(p * inv_freq[c]) for p in [0, S).  A key row is
// rotated from its anchor by at most 7 steps of angle addition.
__global__ void __launch_bounds__(256) vs_trig_kernel(const double* __restrict__ inv_freq, double2* __restrict__ trig,
                                                      int n_anchor) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)n_anchor * HALF) return;
  const int a = (int)(i / HALF);
  const int c = (int)(i % HALF);
  double sn, cs;
  sincos((double)(8 * a) * inv_freq[c], &sn, &cs);
  trig[i] = make_double2(cs, sn);
}

struct __align__(16) VsSmem {
  double kt[SUB * KPD];          // rotated keys of the sub-tile, [key][dim]
};
// pass 2 holds no keys: a third of the LDS, so more workgroups share a CU
struct __align__(16) VsSmem2 {
  double at[64 * APD];           // probabilities [row][key]
  double ring_hi[RING], ring_lo[RING];
};

template <int PASS>
__global__ void __launch_bounds__(256, 3) vs_pass_kernel(VsArgs A) {
  __shared__ typename std::conditional<PASS == 1, VsSmem, VsSmem2>::type sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // die-aware mapping: die x takes ranges x, x+8, ... with every head back to back
  const int die = blockIdx.x % NXCD;
  const int local = blockIdx.x / NXCD;
  const int r = NXCD * (local / A.h_q) + die;
  if (r >= A.n_ranges) return;
  const int h = local % A.h_q;
  const int g = h / (A.h_q / A.h_kv);
  const int kr0 = r * A.range_keys;
  const int kr1 = min(A.n_k, kr0 + A.range_keys);

  // rows of this lane as A operand (i = lane%16) and as C rows ((lane/16) + 4v)
  const int arow = 16 * wave + (lane & 15);
  const int kd = lane >> 4;
  const int p_arow = A.p_first + arow;
  const int m_arow = p_arow / A.S;

  // key-rotation role: pair c, keys 8*kg .. 8*kg+7 of each sub-tile
  const int c = tid & 63;
  const int kg = tid >> 6;
  double ct, st;
  sincos(A.inv_freq[c], &st, &ct);
  const uint16_t* kbase = A.k + (long long)g * D;
  const long long kstride = (long long)A.h_kv * D;

  double qa[32];
  int cur_var = -1;

  // raw key values (x | y << 16) of this thread's pair for keys 8kg .. 8kg+7
  // of a sub-tile and the anchor rotation of the first, loaded a sub-tile ahead
  uint32_t kraw[8];
  double2 anc;
  auto load_raw = [&](int t0) __attribute__((always_inline)) {
    const int j0 = t0 + 8 * kg;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint16_t* p = kbase + (long long)min(j0 + u, A.n_k - 1) * kstride + c;
      kraw[u] = (uint32_t)p[0] | ((uint32_t)p[HALF] << 16);
    }
    anc = A.trig[(long long)((j0 % A.S) >> 3) * HALF + c];
  };
  if (PASS == 1) load_raw(kr0);
  // pass 2: the scaled logits of a sub-tile (16 lanes read 128 contiguous bytes), loaded a sub-tile ahead
  double lg[2][4];
  auto load_lg = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int j = min(t0 + 16 * nb + (lane & 15), A.n_k - 1);
#pragma unroll
      for (int v = 0; v < 4; ++v) lg[nb][v] = A.logits[((long long)h * 64 + 16 * wave + kd + 4 * v) * A.n_k + j];
    }
  };
  if (PASS == 2) load_lg(kr0);

  double row_m[4], row_s[4], lse_v[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    row_m[v] = -INFINITY; row_s[v] = 0.0;
    const int crow = 16 * wave + kd + 4 * v;
    lse_v[v] = (PASS == 2) ? A.lse[h * 64 + crow] : 0.0;
  }
  if constexpr (PASS == 2) {
    for (int i = tid; i < RING; i += 256) { sm.ring_hi[i] = 0.0; sm.ring_lo[i] = 0.0; }
  }

  for (int t0 = kr0; t0 < kr1; t0 += SUB) {
    f64x4 acc[2];
    if constexpr (PASS == 1) {
    // ---- rotate 32 keys into LDS (fp64): the anchor rotation of each 8 keys
    // (exact), then angle addition
    {
      const int j0 = t0 + 8 * kg;
      double cs = anc.x, sn = anc.y;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        double x = 0.0, y = 0.0;
        if (j < A.n_k) {
          x = (double)bf16_bits_to_f32((uint16_t)(kraw[u] & 0xFFFFu));
          y = (double)bf16_bits_to_f32((uint16_t)(kraw[u] >> 16));
        }
        sm.kt[(8 * kg + u) * KPD + c] = x * cs - y * sn;
        sm.kt[(8 * kg + u) * KPD + c + HALF] = x * sn + y * cs;
        const double cs2 = cs * ct - sn * st;
        const double sn2 = sn * ct + cs * st;
        cs = cs2; sn = sn2;
      }
    }
    if (t0 + SUB < kr1) load_raw(t0 + SUB);   // lands while this sub-tile's MFMAs run
    // ---- query variant for this sub-tile (keys of one DCA chunk)
    const int m_key = t0 / A.S;
    const int need_var = (m_key == m_arow) ? 0 : 1;
    if (__any(need_var != cur_var)) {
      const double* src = A.qs + (((long long)need_var * A.h_q + h) * 64 + arow) * D + kd;
#pragma unroll
      for (int ks = 0; ks < 32; ++ks) qa[ks] = src[4 * ks];
      // a variant change is rare: wait here, so that no wait for these loads is
      // left in the MFMA loop (where it would also wait for the logit stores)
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
      cur_var = need_var;
    }
    __syncthreads();

    // ---- logits for 16 rows x 32 keys per wave
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      acc[nb] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int ks = 0; ks < 32; ++ks) {
        const double bop = sm.kt[(16 * nb + (lane & 15)) * KPD + 4 * ks + kd];
        acc[nb] = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[ks], bop, acc[nb], 0, 0, 0);
      }
    }
    } else {
      // pass 2 reads the scaled logits pass 1 stored
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[nb][v] = lg[nb][v];
      if (t0 + SUB < kr1) load_lg(t0 + SUB);
    }

    if constexpr (PASS == 1) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int j = t0 + 16 * nb + (lane & 15);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int crow = 16 * wave + kd + 4 * v;
          const int p = A.p_first + crow;
          const double l = A.scale * acc[nb][v];
          if (j < A.n_k) A.logits[((long long)h * 64 + crow) * A.n_k + j] = l;
          if (crow < A.n_s && j <= p && j < A.n_k) {
            if (l > row_m[v] + 200.0) {
              row_s[v] = (row_m[v] == -INFINITY) ? 0.0 : row_s[v] * exp(row_m[v] - l);
              row_m[v] = l;
            }
            row_s[v] += exp(l - row_m[v]);
          }
        }
      }
    } else {
      // probabilities into LDS [row][key]
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int jj = 16 * nb + (lane & 15);
        const int j = t0 + jj;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int crow = 16 * wave + kd + 4 * v;
          const int p = A.p_first + crow;
          double a = 0.0;
          if (crow < A.n_s && j <= p && j < A.n_k) a = exp(acc[nb][v] - lse_v[v]);
          sm.at[crow * APD + jj] = a;
        }
      }
      __syncthreads();
      // vertical: column tid / 8 summed over rows 8 (tid % 8) .. +7 by each of
      // eight consecutive lanes, the partial sums combined across the lanes
      {
        const int jj = tid >> 3, part = tid & 7;
        double hi = 0.0, lo = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) dd_add(hi, lo, sm.at[(8 * part + i) * APD + jj]);
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) {
          const double oh = __shfl_xor(hi, off), ol = __shfl_xor(lo, off);
          dd_add_dd(hi, lo, oh, ol);
        }
        const int j = t0 + jj;
        if (part == 0 && j < kr1) A.vert[(long long)h * A.n_k + j] = dd_round(hi, lo);
      }
      // slash: diagonal e = key of row 0 (delta = p_first - e), active e in
      // [t0-63, t0+31]; two lanes take the two halves of its rows inside the
      // sub-tile, the first adds both to the diagonal's running sum
      if (tid < 2 * (SUB + 63)) {
        const int d = tid >> 1, hf = tid & 1;
        const int e = t0 - 63 + d;
        // rows i of the diagonal inside the sub-tile: 0 <= e + i - t0 < SUB
        const int i_lo = max(0, t0 - e), i_hi = min(64, t0 + SUB - e);
        const int mid = (i_lo + i_hi) >> 1;
        const int r0 = hf ? mid : i_lo, r1 = hf ? i_hi : mid;
        double ph = 0.0, pl = 0.0;
        for (int i = r0; i < r1; ++i) dd_add(ph, pl, sm.at[i * APD + (e + i - t0)]);
        const double oh = __shfl_xor(ph, 1), ol = __shfl_xor(pl, 1);
        if (hf == 0 && e <= A.p_first) {
          dd_add_dd(ph, pl, oh, ol);
          const int slot = (e + (1 << 30)) & (RING - 1);
          double hi = sm.ring_hi[slot], lo = sm.ring_lo[slot];
          dd_add_dd(hi, lo, ph, pl);
          const bool last_sub = (t0 + SUB >= kr1);
          const bool complete = (e + 63 < t0 + SUB) || (last_sub && kr1 == A.n_k);
          const bool started_here = (e >= kr0) || (kr0 == 0);
          if (complete || last_sub) {
            const int delta = A.p_first - e;
            if (complete && started_here) {
              if (delta >= 0 && delta < A.n_off) A.slash[(long long)h * A.n_off + delta] = dd_round(hi, lo);
            } else {
              // partial at a range edge: side 0 = started before kr0, side 1 = continues past kr1
              const int side = started_here ? 1 : 0;
              const int idx = side ? e - (kr1 - 63) : e - (kr0 - 63);
              double* dst = A.edge + ((((long long)h * A.n_ranges + r) * 2 + side) * 64 + idx) * 2;
              dst[0] = hi; dst[1] = lo;
            }
            hi = 0.0; lo = 0.0;
          }
          sm.ring_hi[slot] = hi; sm.ring_lo[slot] = lo;
        }
      }
    }
    __syncthreads();
  }

  if (PASS == 1) {
    // combine (max, sum) over the 16 lanes that share kd (keys lane%16)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      double m = row_m[v], s = row_s[v];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const double mo = __shfl_xor(m, off, 16);
        const double so = __shfl_xor(s, off, 16);
        const double mn = fmax(m, mo);
        const double a = (m == -INFINITY) ? 0.0 : s * exp(m - mn);
        const double bb = (mo == -INFINITY) ? 0.0 : so * exp(mo - mn);
        m = mn; s = a + bb;
      }
      if ((lane & 15) == 0) {
        const int crow = 16 * wave + kd + 4 * v;
        double* dst = A.part_ms + (((long long)h * A.n_ranges + r) * 64 + crow) * 2;
        dst[0] = m; dst[1] = s;
      }
    }
  }
}

// Row log-sum-exp from the per-range partials, combined in range order.
__global__ void vs_lse_kernel(const double* __restrict__ part_ms, double* __restrict__ lse, int h_q, int n_ranges) {
  const int h = blockIdx.x;
  const int row = threadIdx.x;   // 64 threads
  double m = -INFINITY, s = 0.0;
  for (int r = 0; r < n_ranges; ++r) {
    const double* p = part_ms + (((long long)h * n_ranges + r) * 64 + row) * 2;
    const double mo = p[0], so = p[1];
    const double mn = fmax(m, mo);
    if (mn == -INFINITY) continue;
    const double a = (m == -INFINITY) ? 0.0 : s * exp(m - mn);
    const double bb = (mo == -INFINITY) ? 0.0 : so * exp(mo - mn);
    m = mn; s = a + bb;
  }
  lse[h * 64 + row] = (m == -INFINITY) ? 0.0 : m + log(s);
}

// Diagonals that cross a range boundary B: high-edge partial of the range below
// plus low-edge partial of the range above.
__global__ void vs_edge_kernel(const double* __restrict__ edge, double* __restrict__ slash,
                               int h_q, int n_ranges, int range_keys, int p_first, int n_off) {
  const int h = blockIdx.y;
  const int r = blockIdx.x + 1;    // boundary B = r * range_keys, between ranges r-1 and r
  const int idx = threadIdx.x;     // 0..62
  if (r >= n_ranges || idx >= 63) return;
  const int B = r * range_keys;
  const int e = B - 63 + idx;
  if (e > p_first) return;
  const double* below = edge + ((((long long)h * n_ranges + (r - 1)) * 2 + 1) * 64 + idx) * 2;
  const double* above = edge + ((((long long)h * n_ranges + r) * 2 + 0) * 64 + idx) * 2;
  double hi = below[0], lo = below[1];
  dd_add_dd(hi, lo, above[0], above[1]);
  const int delta = p_first - e;
  if (delta >= 0 && delta < n_off) slash[(long long)h * n_off + delta] = dd_round(hi, lo);
}

hipError_t launch_vs_score(const VsArgs& A, const uint16_t* q, int n_q, hipStream_t stream) {
  const long long n_trig = (long long)(A.S / 8) * HALF;
  hipLaunchKernelGGL(vs_trig_kernel, dim3((unsigned)((n_trig + 255) / 256)), dim3(256), 0, stream, A.inv_freq,
                     A.trig, A.S / 8);
  hipLaunchKernelGGL(vs_prep_q_kernel, dim3(A.h_q), dim3(256), 0, stream, q, (double*)A.qs, A.inv_freq, n_q,
                     A.h_q, A.S, A.n_s, A.p_first);
  const int blocks = NXCD * ((A.n_ranges + NXCD - 1) / NXCD) * A.h_q;
  hipLaunchKernelGGL(vs_pass_kernel<1>, dim3(blocks), dim3(256), 0, stream, A);
  hipLaunchKernelGGL(vs_lse_kernel, dim3(A.h_q), dim3(64), 0, stream, A.part_ms, (double*)A.lse, A.h_q,
                     A.n_ranges);
  hipLaunchKernelGGL(vs_pass_kernel<2>, dim3(blocks), dim3(256), 0, stream, A);
  if (A.n_ranges > 1)
    hipLaunchKernelGGL(vs_edge_kernel, dim3(A.n_ranges - 1, A.h_q), dim3(64), 0, stream, A.edge, A.slash,
                       A.h_q, A.n_ranges, A.range_keys, A.p_first, A.n_off);
  return hipGetLastError();
}

}  // namespace dca
