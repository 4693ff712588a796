// Fused mixture-of-experts layer for small token batches (declared in
// include/moe.h).  At generation batch sizes an expert receives a few tokens,
// so the layer is bound by streaming the routed experts' weights from HBM
// (paper-review page, section 4, "MoE kernel optimisation", Figure 8).
//
// Kernels, in launch order:
//   moe_sort_kernel      slots (token, k) grouped by expert, in slot order
//   moe_mma_kernel<1>    gate and up products of every routed expert, SwiGLU,
//                        bf16 activations per slot
//   moe_swiglu_kernel    (k-split gate/up only) SwiGLU of the summed k parts
//   moe_mma_kernel<0>    down product, scaled by the slot's routing weight
//   moe_sum_kernel       out_t = sum over the token's slots (and k parts), in order
//
// The two products use v_mfma_f32_32x32x16_bf16 with the weights as the A
// operand (32 weight rows per wave) and up to 64 of the expert's tokens as B.
// A product only needs A and B to agree on which k each element stands for,
// so in a step of 64 k lane half h takes k = 32 h .. 32 h + 31 and MFMA j of
// the step uses elements 8 j .. 8 j + 7 of them, in both operands.  The
// weights are stored in that order (moe_pack_weights), so a wave streams its
// 32 rows as one contiguous region, 1 KB per load instruction: whole DRAM
// pages rather than 128-byte pieces of rows 7 KB apart.  The activation rows
// (B) are read from the caches.  Loads run ahead of the MFMAs by STG - 1 steps.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "../../include/moe.h"
#include "common.h"

namespace {

constexpr int KSTEP = 64;     // k per pipeline step (4 MFMAs of k 16)

struct MoeArgs {
  const uint16_t* x;          // [T][d_model]
  const int32_t* ids;         // [T * top_k]
  const float* wts;           // [T * top_k]
  const uint16_t* w13;        // [E][2 d_ff][d_model]
  const uint16_t* w2;         // [E][d_model][d_ff]
  const int32_t* offsets;     // [E + 1] first sorted slot of each expert
  const int32_t* sorted;      // [N] slot ids grouped by expert, slot order inside
  uint16_t* act;              // [N][d_ff] bf16 SwiGLU activations, sorted order
  float* ys;                  // [ks_dn][N][d_model] weighted expert outputs (per k part), slot order
  float* part;                // [ks_gu][N][2][d_ff] fp32 gate / up sums per k part (ks_gu > 1 only)
  int n_slots, n_experts, top_k, d_model, d_ff;
  int ks_gu, ks_dn;           // k parts of the gate/up and down products
};

__device__ inline uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// One workgroup of 1024 threads, one slot per thread and round of 1024 slots:
//   counts per expert (LDS atomics), an exclusive scan over the experts (the
//   offsets), then stable placement: a slot's place is its expert's running
//   position plus the number of earlier slots of the same expert in its
//   round, counted from the round's ids in LDS (16-byte broadcast reads).
// Every index stays inside its array: an expert's places run from its offset
// to its offset + count - 1 < n_slots; ids outside [0, E) are never placed.
__global__ __launch_bounds__(1024) void moe_sort_kernel(MoeArgs A) {
  __shared__ int4 s_ids4[256];
  __shared__ int s_run[1024];
  __shared__ int s_scan[1024];
  int* s_ids = (int*)s_ids4;
  const int tid = threadIdx.x;
  const int N = A.n_slots, E = A.n_experts;
  s_run[tid] = 0;
  __syncthreads();
  for (int i = tid; i < N; i += 1024) {
    const int id = A.ids[i];
    if (id >= 0 && id < E) atomicAdd(&s_run[id], 1);
  }
  __syncthreads();
  const int cnt = tid < E ? s_run[tid] : 0;
  s_scan[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += add;
    __syncthreads();
  }
  const int excl = s_scan[tid] - cnt;
  if (tid < E) ((int32_t*)A.offsets)[tid] = excl;
  if (tid == E - 1) ((int32_t*)A.offsets)[E] = s_scan[tid];
  __syncthreads();
  if (tid < E) s_run[tid] = excl;
  __syncthreads();
  for (int base = 0; base < N; base += 1024) {
    const int i = base + tid;
    const int id = i < N ? A.ids[i] : -1;
    s_ids[tid] = id;
    __syncthreads();
    const bool valid = id >= 0 && id < E;
    if (valid) {
      int rank = 0;
      const int full = tid >> 2;
#pragma unroll 8
      for (int w = 0; w < full; ++w) {
        const int4 v = s_ids4[w];
        rank += (v.x == id) + (v.y == id) + (v.z == id) + (v.w == id);
      }
      for (int j = 4 * full; j < tid; ++j) rank += s_ids[j] == id;
      ((int32_t*)A.sorted)[s_run[id] + rank] = i;
    }
    __syncthreads();
    if (valid) atomicAdd(&s_run[id], 1);
    __syncthreads();
  }
}

// Operands of one pipeline step: NW weight row sets (gate and up, or down)
// and NT token tiles of 32.
template <int NW, int NT>
struct Step {
  bf16x8 a[NW][4];
  bf16x8 b[NT][4];
};

constexpr int TILE_ELEMS = 32 * KSTEP;   // one packed 32 x 64 tile

template <int NW, int NT>
__device__ inline void load_step(Step<NW, NT>& s, const uint16_t* const (&wp)[NW], const uint16_t* const (&bp)[NT],
                                 int ks) {
  const int o = ks * KSTEP;
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      s.a[w][j] = __builtin_nontemporal_load((const bf16x8*)(wp[w] + (size_t)ks * TILE_ELEMS + 512 * j));
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) s.b[t][j] = *(const bf16x8*)(bp[t] + o + 8 * j);
}

template <int NW, int NT>
__device__ inline void mma_step(const Step<NW, NT>& s, f32x16 (&c)[NW][NT]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int t = 0; t < NT; ++t) c[w][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(s.a[w][j], s.b[t][j], c[w][t], 0, 0, 0);
}

// C[w][t] += W_w (32 rows x K) * B_t^T over nks steps, STG steps in flight.
template <int NW, int NT, int STG>
__device__ inline void mma_pass(const uint16_t* const (&wp)[NW], const uint16_t* const (&bp)[NT], int nks,
                                f32x16 (&c)[NW][NT]) {
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) c[w][t][i] = 0.f;
  // Every iteration issues its loads unconditionally (steps past the end
  // repeat the last one, which the caches serve), so the wait before each
  // step's MFMAs is always "the later STG - 1 steps' loads may be pending".
  // Ring invariant at the top of an iteration: s[i] holds step ks0 + i for
  // i < STG - 1 and s[STG - 1] is free.
  Step<NW, NT> s[STG];
  const int last = nks - 1;
#pragma unroll
  for (int i = 0; i < STG - 1; ++i) load_step(s[i], wp, bp, i < last ? i : last);
  __builtin_amdgcn_sched_barrier(0);
  int ks0 = 0;
  for (; ks0 + STG <= nks; ks0 += STG) {
#pragma unroll
    for (int i = 0; i < STG; ++i) {
      const int ahead = ks0 + i + STG - 1;
      load_step(s[(i + STG - 1) % STG], wp, bp, ahead < last ? ahead : last);
      // keep the loads of a step ahead of its MFMAs in issue order
      __builtin_amdgcn_sched_barrier(0);
      mma_step(s[i], c);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // fewer than STG steps remain, all already loaded
#pragma unroll
  for (int i = 0; i < STG - 1; ++i)
    if (ks0 + i < nks) mma_step(s[i], c);
}

// Rows of the C fragment held by this lane: r(i) = 8 (i / 4) + 4 half + i % 4,
// column = lane % 32.
template <bool GATE_UP, int NT>
__device__ inline void expert_pass(const MoeArgs& A, int e, int beg, int m, int t0, int r0, int l32, int half,
                                   int ks, int k0, int nks) {
  const int d = A.d_model, dff = A.d_ff;
  const int KS = GATE_UP ? A.ks_gu : A.ks_dn;
  constexpr int NW = GATE_UP ? 2 : 1;
  // packed tiles: tile row r0 / 32 of the expert's matrix, this lane's piece
  const uint16_t* wp[NW];
  const int lane = 32 * half + l32;
  if (GATE_UP) {
    const uint16_t* g = A.w13 + (size_t)e * 2 * dff * d + ((size_t)(r0 / 32) * (d / KSTEP) + k0) * TILE_ELEMS + 8 * lane;
    wp[0] = g;
    wp[NW - 1] = g + (size_t)dff * d;
  } else {
    wp[0] = A.w2 + (size_t)e * d * dff + ((size_t)(r0 / 32) * (dff / KSTEP) + k0) * TILE_ELEMS + 8 * lane;
  }
  // token columns: lanes past the expert's last slot read its first slot's row
  // (finite values) and their columns are not stored
  const uint16_t* bp[NT];
  int slot[NT];
  bool ok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int idx = t0 + 32 * t + l32;
    ok[t] = idx < m;
    const int j = beg + (ok[t] ? idx : 0);
    slot[t] = A.sorted[j];
    bp[t] = (GATE_UP ? A.x + (size_t)(slot[t] / A.top_k) * d : A.act + (size_t)j * dff) + KSTEP * k0 + 32 * half;
  }
  f32x16 c[NW][NT];
  constexpr int STG = (NW * 16 + NT * 16) <= 48 ? 3 : 2;
  mma_pass<NW, NT, STG>(wp, bp, nks, c);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (!ok[t]) continue;
    const int idx = t0 + 32 * t + l32;
    if (GATE_UP && KS > 1) {
      // this k part's gate and up sums; moe_swiglu_kernel adds the parts
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        float* dst = A.part + (((size_t)ks * A.n_slots + beg + idx) * 2 + w) * dff + r0 + 4 * half;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(float4*)(dst + 8 * q) = make_float4(c[w][t][4 * q], c[w][t][4 * q + 1], c[w][t][4 * q + 2],
                                                c[w][t][4 * q + 3]);
      }
    } else if (GATE_UP) {
      uint16_t* dst = A.act + (size_t)(beg + idx) * dff + r0 + 4 * half;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint16_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = c[0][t][4 * q + i], u = c[NW - 1][t][4 * q + i];
          v[i] = f2bf(g / (1.f + __expf(-g)) * u);
        }
        uint2 p;
        p.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
        p.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
        *(uint2*)(dst + 8 * q) = p;
      }
    } else {
      const float wt = A.wts[slot[t]];
      float* dst = A.ys + ((size_t)ks * A.n_slots + slot[t]) * d + r0 + 4 * half;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 p;
        p.x = wt * c[0][t][4 * q + 0];
        p.y = wt * c[0][t][4 * q + 1];
        p.z = wt * c[0][t][4 * q + 2];
        p.w = wt * c[0][t][4 * q + 3];
        *(float4*)(dst + 8 * q) = p;
      }
    }
  }
}

// Workgroup (expert e, 32 * WAVES output rows): WAVES waves of 32 rows;
// passes of up to 64 of the expert's slots.  Experts without slots return at
// once, so only routed experts' weights are read.  WAVES = 4 in general; 1
// when few experts can be routed (a token or two), so that their rows spread
// over every compute unit.
template <bool GATE_UP, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 2) void moe_mma_kernel(MoeArgs A) {
  constexpr int ROWS = 32 * WAVES;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l32 = lane & 31, half = lane >> 5;
  const int tiles = (GATE_UP ? A.d_ff : A.d_model) / ROWS;
  // blockIdx = (k part, expert, row tile); the k parts split the product's
  // 64-wide k steps evenly
  const int per = A.n_experts * tiles;
  const int ks = blockIdx.x / per, rem = blockIdx.x - ks * per;
  const int e = rem / tiles, rt = rem - e * tiles;
  const int KS = GATE_UP ? A.ks_gu : A.ks_dn;
  const int steps = (GATE_UP ? A.d_model : A.d_ff) / KSTEP;
  const int k0 = (int)((long long)steps * ks / KS), k1 = (int)((long long)steps * (ks + 1) / KS);
  const int beg = A.offsets[e], m = A.offsets[e + 1] - beg;
  if (m <= 0) return;
  const int r0 = rt * ROWS + 32 * wave;
  for (int t0 = 0; t0 < m; t0 += 64) {
    if (m - t0 > 32)
      expert_pass<GATE_UP, 2>(A, e, beg, m, t0, r0, l32, half, ks, k0, k1 - k0);
    else
      expert_pass<GATE_UP, 1>(A, e, beg, m, t0, r0, l32, half, ks, k0, k1 - k0);
  }
}

// Packed layout of n_mats matrices [R][C]: thread = one 16-byte piece
// (matrix, tile row t, tile column s, MFMA step j, lane l) <- 8 elements of
// row 32 t + l % 32 from column 64 s + 32 (l / 32) + 8 j.
__global__ __launch_bounds__(256) void moe_pack_kernel(const uint16_t* src, uint16_t* dst, int n_mats, int R, int C) {
  const long long pieces = (long long)n_mats * R * C / 8;
  const long long g = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= pieces) return;
  const int l = (int)(g & 63);
  const int j = (int)((g >> 6) & 3);
  const long long tile = g >> 8;                   // (matrix, t, s) in storage order
  const int tiles_per_row = C / KSTEP;
  const long long tiles_per_mat = (long long)(R / 32) * tiles_per_row;
  const long long mat = tile / tiles_per_mat;
  const long long rem = tile - mat * tiles_per_mat;
  const int t = (int)(rem / tiles_per_row), s = (int)(rem - (long long)t * tiles_per_row);
  const size_t from = (size_t)mat * R * C + (size_t)(32 * t + (l & 31)) * C + KSTEP * s + 32 * (l >> 5) + 8 * j;
  *(uint4*)(dst + 8 * g) = *(const uint4*)(src + from);
}

// out[t][c .. c+3] = bf16(sum over the token's valid slots, in slot order)
// SwiGLU of the gate / up sums written in k parts: thread = 4 activations of
// one sorted slot; the parts are added in order.  Slots past the placed ones
// (dropped ids) are skipped.
__global__ __launch_bounds__(256) void moe_swiglu_kernel(MoeArgs A) {
  const int q = A.d_ff / 4;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)A.n_slots * q) return;
  const int j = (int)(gid / q), r = 4 * (int)(gid - (long long)j * q);
  if (j >= A.offsets[A.n_experts]) return;
  float g[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
  for (int ks = 0; ks < A.ks_gu; ++ks) {
    const float* p = A.part + ((size_t)ks * A.n_slots + j) * 2 * A.d_ff + r;
    const float4 a = *(const float4*)p, b = *(const float4*)(p + A.d_ff);
    g[0] += a.x; g[1] += a.y; g[2] += a.z; g[3] += a.w;
    u[0] += b.x; u[1] += b.y; u[2] += b.z; u[3] += b.w;
  }
  uint16_t v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = f2bf(g[i] / (1.f + __expf(-g[i])) * u[i]);
  uint2 p;
  p.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
  p.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
  *(uint2*)(A.act + (size_t)j * A.d_ff + r) = p;
}

__global__ __launch_bounds__(256) void moe_sum_kernel(MoeArgs A, uint16_t* out, int n_tokens) {
  const int q = A.d_model / 4;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)n_tokens * q) return;
  const int t = (int)(gid / q), c = 4 * (int)(gid - (long long)t * q);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < A.top_k; ++s) {
    const int slot = t * A.top_k + s;
    const int id = A.ids[slot];
    if (id < 0 || id >= A.n_experts) continue;
    for (int ks = 0; ks < A.ks_dn; ++ks) {
      const float4 y = *(const float4*)(A.ys + ((size_t)ks * A.n_slots + slot) * A.d_model + c);
      acc.x += y.x; acc.y += y.y; acc.z += y.z; acc.w += y.w;
    }
  }
  uint2 p;
  p.x = (uint32_t)f2bf(acc.x) | ((uint32_t)f2bf(acc.y) << 16);
  p.y = (uint32_t)f2bf(acc.z) | ((uint32_t)f2bf(acc.w) << 16);
  *(uint2*)(out + (size_t)t * A.d_model + c) = p;
}

struct MoeLayout {
  size_t offsets = 0, sorted = 0, act = 0, ys = 0, part = 0, total = 0;
};

// Launch shape.  At most min(E, slots) experts are routed: with fewer than
// two 4-wave workgroups per compute unit for them, one-wave workgroups fill
// the GPU (narrow).  When those waves make a single pass (at most 64 slots)
// and are still few, each one's k range is split into parts so that about
// KSPLIT_WAVES waves stream the weights: more loads in flight and an even
// spread over the compute units.
constexpr long long KSPLIT_WAVES = 3072;
struct MoeShape {
  bool narrow = false;
  int ks_gu = 1, ks_dn = 1;
};

MoeShape moe_shape(const moe_cfg* c) {
  MoeShape S;
  const long long N = (long long)c->n_tokens * c->top_k;
  const long long routed = std::min<long long>(c->n_experts, N);
  S.narrow = routed * (c->d_ff / 128) < 512;
  if (S.narrow && N <= 64) {
    S.ks_gu = (int)std::clamp<long long>(KSPLIT_WAVES / (routed * (c->d_ff / 32)), 1,
                                         std::min(8, c->d_model / KSTEP));
    S.ks_dn = (int)std::clamp<long long>(KSPLIT_WAVES / (routed * (c->d_model / 32)), 1,
                                         std::min(8, c->d_ff / KSTEP));
  }
  return S;
}

inline size_t up256(size_t x) { return (x + 255) / 256 * 256; }

int moe_validate(const moe_cfg* c) {
  if (!c) return DCA_EINVAL;
  if (c->n_tokens < 1 || c->n_experts < 1 || c->top_k < 1) return DCA_EINVAL;
  if (c->n_experts > 1023 || c->top_k > c->n_experts) return DCA_EUNSUPPORTED;
  if (c->d_model < 128 || c->d_model % 128 || c->d_ff < 128 || c->d_ff % 128) return DCA_EUNSUPPORTED;
  // slot ids and activation rows are int32; expert tiles fit a 1-D grid
  if ((long long)c->n_tokens * c->top_k >= (1LL << 30)) return DCA_EUNSUPPORTED;
  return DCA_OK;
}

MoeLayout moe_layout(const moe_cfg* c) {
  MoeLayout L;
  const size_t N = (size_t)c->n_tokens * c->top_k;
  size_t cur = 0;
  L.offsets = cur; cur += up256((size_t)(c->n_experts + 1) * 4);
  L.sorted = cur; cur += up256(N * 4);
  const MoeShape S = moe_shape(c);
  L.act = cur; cur += up256(N * c->d_ff * 2);
  L.ys = cur; cur += up256((size_t)S.ks_dn * N * c->d_model * 4);
  L.part = cur; cur += S.ks_gu > 1 ? up256((size_t)S.ks_gu * N * 2 * c->d_ff * 4) : 0;
  L.total = cur;
  return L;
}

void moe_record(const moe_cfg* c, int stage, int which) {
  if (!c->stage_events) return;
  hipEvent_t ev = (hipEvent_t)c->stage_events[2 * stage + which];
  if (ev) (void)hipEventRecord(ev, (hipStream_t)c->stream);
}

}  // namespace

extern "C" {

int moe_workspace_size(const moe_cfg* cfg, size_t* bytes) {
  if (!bytes) return DCA_EINVAL;
  const int rc = moe_validate(cfg);
  if (rc != DCA_OK) return rc;
  *bytes = moe_layout(cfg).total;
  return DCA_OK;
}

int moe_pack_weights(const dca_bf16* w13, const dca_bf16* w2, const moe_cfg* cfg, dca_bf16* w13_packed,
                     dca_bf16* w2_packed) {
  if (!cfg || !w13 || !w2 || !w13_packed || !w2_packed) return DCA_EINVAL;
  if (cfg->n_experts < 1) return DCA_EINVAL;
  if (cfg->n_experts > 1023) return DCA_EUNSUPPORTED;
  if (cfg->d_model < 128 || cfg->d_model % 128 || cfg->d_ff < 128 || cfg->d_ff % 128) return DCA_EUNSUPPORTED;
  const size_t n13 = (size_t)cfg->n_experts * 2 * cfg->d_ff * cfg->d_model;
  const size_t n2 = (size_t)cfg->n_experts * cfg->d_model * cfg->d_ff;
  // the packed copies must not overlap their sources
  auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    const char* x = (const char*)a;
    const char* y = (const char*)b;
    return x < y + nb && y < x + na;
  };
  if (overlap(w13, 2 * n13, w13_packed, 2 * n13) || overlap(w2, 2 * n2, w2_packed, 2 * n2)) return DCA_EINVAL;
  hipStream_t st = (hipStream_t)cfg->stream;
  const unsigned b13 = (unsigned)((n13 / 8 + 255) / 256), b2 = (unsigned)((n2 / 8 + 255) / 256);
  hipLaunchKernelGGL(moe_pack_kernel, dim3(b13), dim3(256), 0, st, w13, w13_packed, cfg->n_experts, 2 * cfg->d_ff,
                     cfg->d_model);
  if (hipGetLastError() != hipSuccess) return DCA_EHIP;
  hipLaunchKernelGGL(moe_pack_kernel, dim3(b2), dim3(256), 0, st, w2, w2_packed, cfg->n_experts, cfg->d_model,
                     cfg->d_ff);
  if (hipGetLastError() != hipSuccess) return DCA_EHIP;
  return DCA_OK;
}

int moe_forward(const dca_bf16* x, const int32_t* topk_ids, const float* topk_weights, const dca_bf16* w13,
                const dca_bf16* w2, const moe_cfg* cfg, dca_bf16* out) {
  int rc = moe_validate(cfg);
  if (rc != DCA_OK) return rc;
  if (!x || !topk_ids || !topk_weights || !w13 || !w2 || !out) return DCA_EINVAL;
  const MoeLayout L = moe_layout(cfg);
  if (!cfg->workspace || cfg->workspace_bytes < L.total || ((uintptr_t)cfg->workspace) % 256) return DCA_EWORKSPACE;
  hipStream_t st = (hipStream_t)cfg->stream;
  char* ws = (char*)cfg->workspace;
  MoeArgs A;
  A.x = x; A.ids = topk_ids; A.wts = topk_weights; A.w13 = w13; A.w2 = w2;
  A.offsets = (const int32_t*)(ws + L.offsets);
  A.sorted = (const int32_t*)(ws + L.sorted);
  A.act = (uint16_t*)(ws + L.act);
  A.ys = (float*)(ws + L.ys);
  A.part = (float*)(ws + L.part);
  const MoeShape S = moe_shape(cfg);
  A.ks_gu = S.ks_gu;
  A.ks_dn = S.ks_dn;
  A.n_slots = cfg->n_tokens * cfg->top_k;
  A.n_experts = cfg->n_experts; A.top_k = cfg->top_k; A.d_model = cfg->d_model; A.d_ff = cfg->d_ff;
  moe_record(cfg, 0, 0);
  hipLaunchKernelGGL(moe_sort_kernel, dim3(1), dim3(1024), 0, st, A);
  if (hipGetLastError() != hipSuccess) return DCA_EHIP;
  moe_record(cfg, 0, 1);
  const bool narrow = S.narrow;
  moe_record(cfg, 1, 0);
  if (narrow)
    hipLaunchKernelGGL((moe_mma_kernel<true, 1>), dim3(cfg->n_experts * (cfg->d_ff / 32) * S.ks_gu), dim3(64), 0,
                       st, A);
  else
    hipLaunchKernelGGL((moe_mma_kernel<true, 4>), dim3(cfg->n_experts * (cfg->d_ff / 128)), dim3(256), 0, st, A);
  if (hipGetLastError() != hipSuccess) return DCA_EHIP;
  if (S.ks_gu > 1) {
    const long long items = (long long)A.n_slots * (cfg->d_ff / 4);
    hipLaunchKernelGGL(moe_swiglu_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, st, A);
    if (hipGetLastError() != hipSuccess) return DCA_EHIP;
  }
  moe_record(cfg, 1, 1);
  moe_record(cfg, 2, 0);
  if (narrow)
    hipLaunchKernelGGL((moe_mma_kernel<false, 1>), dim3(cfg->n_experts * (cfg->d_model / 32) * S.ks_dn), dim3(64),
                       0, st, A);
  else
    hipLaunchKernelGGL((moe_mma_kernel<false, 4>), dim3(cfg->n_experts * (cfg->d_model / 128)), dim3(256), 0, st, A);
  if (hipGetLastError() != hipSuccess) return DCA_EHIP;
  moe_record(cfg, 2, 1);
  moe_record(cfg, 3, 0);
  const long long items = (long long)cfg->n_tokens * (cfg->d_model / 4);
  hipLaunchKernelGGL(moe_sum_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, st, A, out, cfg->n_tokens);
  if (hipGetLastError() != hipSuccess) return DCA_EHIP;
  moe_record(cfg, 3, 1);
  return DCA_OK;
}

}  // extern "C"
