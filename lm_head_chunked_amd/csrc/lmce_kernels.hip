// Device kernels of the fused LM-head + cross-entropy loss for gfx950 (CDNA4).
//
// Page: TRL docs "Training Beyond 1M Tokens", sections "The loss is the
// first thing to break" (logits = h W^T, cross entropy against the labels)
// and "The massive logits matrix: chunk it" (rows split cleanly: each row's
// softmax runs over its own vocabulary, so per-row pieces add up).
//
// Every logit tile z[128 x 128] is produced by bf16 MFMA (32x32x16) from
// h and W staged through LDS, and is consumed in registers:
//   k_fwd          folds it into per-lane online (max, sum-exp) states and
//                  picks out the label logit;
//   k_fwd_rows     merges the per-segment states into lse and nll per row
//                  and a fixed-order block sum of nll;
//   k_fwd_loss     sums the block sums in a fixed order and divides by N;
//   k_bwd_dh       recomputes z, forms G = g/N (softmax - onehot) in bf16
//                  and contracts it with W over the vocabulary (row-owned dh);
//   k_bwd_dW       recomputes z, forms G and contracts it with h over the
//                  rows (vocabulary-tile-owned dW, no atomics).
// No kernel writes a logit (or a G) tile to global memory.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lmce_internal.h"

namespace lmce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16;

constexpr int NT = 256;                 // threads per workgroup: 4 waves of 64
constexpr int TILE = 128;               // rows of each operand in a logit tile
constexpr int BK = 64;                  // K (hidden) elements per pipeline stage
constexpr int LDS_K = BK + 8;           // padded LDS row stride of a stage (u16)
constexpr int LDS_T = TILE + 8;         // padded LDS row stride of a 128-wide tile (u16)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_BIG = -1.0e30f;     // "no value yet" for running maxima

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void zero(f32x16& x) {
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = 0.f;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// (m, s) <- merge of two partial log-sum-exp states, s measured relative to m.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  float M = fmaxf(m, m2);
  s = s * fast_exp2((m - M) * LOG2E) + s2 * fast_exp2((m2 - M) * LOG2E);
  m = M;
}

// Row position, inside a 32x32 accumulator block, of register `reg` of lane
// `lane` (v_mfma_f32_32x32x16: column = lane % 32).
__device__ __forceinline__ int acc_row(int reg, int lane) {
  return ((reg >> 2) << 3) + ((lane >> 5) << 2) + (reg & 3);
}

// Two-stage LDS buffers of the logit-tile main loop.
struct StageLds {
  u16 a[2][TILE * LDS_K];
  u16 b[2][TILE * LDS_K];
};

// Loads this thread's four 16-byte chunks of a 128 x 64 slice
// [row0, row0+128) x [k0, k0+64) of a row-major matrix with `nrows` rows and
// leading dimension ld.  Rows past the end are clamped to the last row (their
// results are masked by the caller).
__device__ __forceinline__ void stage_load(const u16* __restrict__ base, int64_t row0, int64_t nrows,
                                           int64_t ld, int64_t k0, u32x4 (&r)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int c = threadIdx.x + NT * i;
    int64_t row = row0 + (c >> 3);
    row = row < nrows ? row : nrows - 1;
    r[i] = *(const u32x4*)(base + row * ld + k0 + (c & 7) * 8);
  }
}

__device__ __forceinline__ void stage_store(u16* lds, const u32x4 (&r)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int c = threadIdx.x + NT * i;
    *(u32x4*)(lds + (c >> 3) * LDS_K + (c & 7) * 8) = r[i];
  }
}

// Logit tile: acc[mb][nb] (wave (wm, wn) of a 2x2 wave grid) receives
//   D[m][n] = sum_k A[a0 + m][k] * B[b0 + n][k],  m, n in [0, 128), k in [0, K)
// where m = wm*64 + mb*32 + acc_row(reg, lane) and n = wn*64 + nb*32 + lane%32.
// A and B are row-major bf16 with K contiguous (h rows or W rows).
__device__ void logit_tile(const u16* __restrict__ A, int64_t a0, int64_t nA,
                           const u16* __restrict__ B, int64_t b0, int64_t nB, int64_t K,
                           StageLds& s, f32x16 (&acc)[2][2]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) zero(acc[i][j]);

  u32x4 ra[4], rb[4];
  const int nk = (int)(K / BK);
  stage_load(A, a0, nA, K, 0, ra);
  stage_load(B, b0, nB, K, 0, rb);
  stage_store(s.a[0], ra);
  stage_store(s.b[0], rb);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      stage_load(A, a0, nA, K, (int64_t)(kt + 1) * BK, ra);
      stage_load(B, b0, nB, K, (int64_t)(kt + 1) * BK, rb);
    }
    const u16* la = s.a[cur];
    const u16* lb = s.b[cur];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kk = ks * 16 + (lane >> 5) * 8;
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        fa[mb] = *(const bf16x8*)(la + (wm * 64 + mb * 32 + (lane & 31)) * LDS_K + kk);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        fb[nb] = *(const bf16x8*)(lb + (wn * 64 + nb * 32 + (lane & 31)) * LDS_K + kk);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32x32x16(fa[mb], fb[nb], acc[mb][nb]);
    }
    if (kt + 1 < nk) {
      stage_store(s.a[cur ^ 1], ra);
      stage_store(s.b[cur ^ 1], rb);
    }
    __syncthreads();
  }
}

// Copies rows [row0, row0 + nrows_tile) x cols [col0, col0 + 128) of a
// row-major bf16 matrix (leading dimension ld) into LDS with stride LDS_T.
// The source is a zero-padded transposed copy, so every read is in bounds.
template <int NROWS>
__device__ __forceinline__ void tile_to_lds(const u16* __restrict__ src, int64_t row0, int64_t ld, int64_t col0,
                                            u16* lds) {
  constexpr int CHUNKS = NROWS * (TILE / 8);
#pragma unroll
  for (int i = 0; i < CHUNKS / NT; ++i) {
    int c = threadIdx.x + NT * i;
    int r = c >> 4, k = (c & 15) * 8;
    *(u32x4*)(lds + r * LDS_T + k) = *(const u32x4*)(src + (row0 + r) * ld + col0 + k);
  }
}

// acc[mb][nb] += sum_{k<128} A[m][k] B[n][k] for A, B in LDS (stride LDS_T),
// m = mrow0 + mb*32 + ..., n = nrow0 + nb*32 + lane%32.
template <int MB, int NB>
__device__ __forceinline__ void lds_mma(const u16* la, int mrow0, const u16* lb, int nrow0, f32x16 (&acc)[MB][NB]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int ks = 0; ks < TILE / 16; ++ks) {
    const int kk = ks * 16 + (lane >> 5) * 8;
    bf16x8 fa[MB], fb[NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) fa[mb] = *(const bf16x8*)(la + (mrow0 + mb * 32 + (lane & 31)) * LDS_T + kk);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) fb[nb] = *(const bf16x8*)(lb + (nrow0 + nb * 32 + (lane & 31)) * LDS_T + kk);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma32x32x16(fa[mb], fb[nb], acc[mb][nb]);
  }
}

__device__ __forceinline__ float pick16(const f32x16& x, int reg) {
  float v = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q) v = (q == reg) ? x[q] : v;
  return v;
}

// Packs 4 floats to bf16 (round to nearest even) and stores 8 bytes to LDS.
__device__ __forceinline__ void store_bf16x4(u16* dst, float a, float b, float c, float d) {
  bf16x4 v = __builtin_convertvector((f32x4){a, b, c, d}, bf16x4);
  *(bf16x4*)dst = v;
}

// ---------------------------------------------------------------- K0: labels

// Counts rows whose label is not ignore_index and checks the others lie in
// [0, V).  One workgroup; fixed-order reduction.
__global__ __launch_bounds__(1024) void k_count_labels(const int64_t* __restrict__ labels, int64_t L, int64_t V,
                                                       int64_t ignore_index, WsHeader* __restrict__ hdr) {
  __shared__ int s_cnt[1024];
  __shared__ int s_bad[1024];
  int cnt = 0, bad = 0;
  for (int64_t i = threadIdx.x; i < L; i += 1024) {
    int64_t y = labels[i];
    if (y != ignore_index) {
      if (y < 0 || y >= V) bad = 1;
      else ++cnt;
    }
  }
  s_cnt[threadIdx.x] = cnt;
  s_bad[threadIdx.x] = bad;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      s_cnt[threadIdx.x] += s_cnt[threadIdx.x + w];
      s_bad[threadIdx.x] |= s_bad[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    hdr->n_valid = s_cnt[0];
    hdr->status = s_bad[0] ? kStatusLabel : 0;
  }
}

// ---------------------------------------------------------------- forward

// Grid: one workgroup per (row tile, vocabulary segment).  The workgroup
// sweeps the 128-wide vocabulary tiles of its segment; each lane keeps an
// online (max, sum-exp) state for its two rows over the logits it holds.
__global__ __launch_bounds__(NT) void k_fwd(FwdArgs p) {
  __shared__ StageLds s;
  __shared__ float red_m[128], red_s[128];

  const int seg = blockIdx.x % p.segments;
  const int tile = blockIdx.x / p.segments;
  const int64_t chunk = tile / p.tiles_per_chunk;
  const int64_t cbeg = chunk * p.chunk_rows;
  const int64_t cend = min(cbeg + (int64_t)p.chunk_rows, p.L);
  const int64_t r0 = cbeg + (int64_t)(tile % p.tiles_per_chunk) * TILE;
  if (r0 >= cend) return;  // uniform across the workgroup
  const int64_t rend = min(r0 + TILE, cend);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int64_t tok[2];
  int64_t lab[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    tok[nb] = r0 + wn * 64 + nb * 32 + (lane & 31);
    lab[nb] = tok[nb] < rend ? p.labels[tok[nb]] : p.ignore_index;
  }
  float m[2] = {NEG_BIG, NEG_BIG}, sum[2] = {0.f, 0.f};

  const int vt0 = seg * p.vtiles_per_seg;
  const int vt1 = min(vt0 + p.vtiles_per_seg, p.vtiles);
  for (int vt = vt0; vt < vt1; ++vt) {
    const int64_t v0 = (int64_t)vt * TILE;
    f32x16 acc[2][2];
    // A = W rows (vocabulary on the MFMA M side), B = h rows (tokens on N):
    // a token's logits sit in one lane's registers.
    logit_tile(p.W, v0, p.V, p.h, r0, rend, p.H, s, acc);

    const int64_t vw = v0 + wm * 64;  // first vocabulary index of this wave
    if (v0 + TILE > p.V) {            // ragged last tile: mask v >= V
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (vw + mb * 32 + acc_row(r, lane) >= p.V) {
            acc[mb][0][r] = -INFINITY;
            acc[mb][1][r] = -INFINITY;
          }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float mt = fmaxf(acc[0][nb][0], acc[1][nb][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, fmaxf(acc[0][nb][r], acc[1][nb][r]));
      const float mn = fmaxf(m[nb], mt);
      const float off = -mn * LOG2E;
      float add = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) add += fast_exp2(__builtin_fmaf(acc[mb][nb][r], LOG2E, off));
      sum[nb] = sum[nb] * fast_exp2((m[nb] - mn) * LOG2E) + add;
      m[nb] = mn;

      const int64_t d = lab[nb] - vw;
      if (lab[nb] != p.ignore_index && d >= 0 && d < 64) {
        const int mb = (int)(d >> 5), i = (int)(d & 31);
        if (((i >> 2) & 1) == (lane >> 5)) {
          const int reg = ((i >> 3) << 2) | (i & 3);
          const float zl = mb ? pick16(acc[1][nb], reg) : pick16(acc[0][nb], reg);
          if (tok[nb] < rend) p.zlabel[tok[nb]] = zl;
        }
      }
    }
  }

  // Merge lane halves (same tokens, other vocabulary rows), then the two
  // waves that share tokens; write one (max, sum) pair per token and segment.
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float m2 = __shfl_xor(m[nb], 32);
    float s2 = __shfl_xor(sum[nb], 32);
    lse_merge(m[nb], sum[nb], m2, s2);
  }
  if (wm == 1 && lane < 32) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      red_m[wn * 64 + nb * 32 + lane] = m[nb];
      red_s[wn * 64 + nb * 32 + lane] = sum[nb];
    }
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      lse_merge(m[nb], sum[nb], red_m[wn * 64 + nb * 32 + lane], red_s[wn * 64 + nb * 32 + lane]);
      if (tok[nb] < rend) {
        p.part_m[(int64_t)seg * p.L + tok[nb]] = m[nb];
        p.part_s[(int64_t)seg * p.L + tok[nb]] = sum[nb];
      }
    }
  }
}

// Per row: merge the segment states in segment order into lse, form nll;
// per workgroup: fixed-order tree sum of nll into block_sum[blockIdx.x].
__global__ __launch_bounds__(256) void k_fwd_rows(FwdArgs p, float* __restrict__ lse_out) {
  __shared__ float red[256];
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float nll = 0.f;
  if (r < p.L) {
    float m = NEG_BIG, s = 0.f;
    for (int seg = 0; seg < p.segments; ++seg)
      lse_merge(m, s, p.part_m[(int64_t)seg * p.L + r], p.part_s[(int64_t)seg * p.L + r]);
    const float lse = m + logf(s);
    lse_out[r] = lse;
    const int64_t y = p.labels[r];
    if (y != p.ignore_index && y >= 0 && y < p.V) nll = lse - p.zlabel[r];
  }
  red[threadIdx.x] = nll;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.block_sum[blockIdx.x] = red[0];
}

// loss = (sum of block sums, fixed order) / N; NaN if N == 0 or a label was bad.
__global__ __launch_bounds__(256) void k_fwd_loss(FwdArgs p, int nblocks, float* __restrict__ loss_out) {
  __shared__ float red[256];
  float acc = 0.f;
  for (int i = threadIdx.x; i < nblocks; i += 256) acc += p.block_sum[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int n = p.hdr->n_valid;
    float loss = (n > 0) ? red[0] / (float)n : __builtin_nanf("");
    if (p.hdr->status != 0) loss = __builtin_nanf("");
    *loss_out = loss;
  }
}

// ---------------------------------------------------------------- transposes

// out[c][r] = in[r][c] for r < R, 0 for R <= r < Rpad.  in is [R x C]
// row-major, out is [C x Rpad].  64x64 tiles through LDS; C % 64 == 0.
__global__ __launch_bounds__(256) void k_transpose(const u16* __restrict__ in, int64_t R, int64_t C,
                                                   u16* __restrict__ out, int64_t Rpad) {
  __shared__ u16 t[64][66];
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int64_t c0 = (int64_t)blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int rr = i >> 6, cc = i & 63;
    const int64_t r = r0 + rr;
    t[rr][cc] = (r < R) ? in[r * C + c0 + cc] : (u16)0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int cc = i >> 6, rr = i & 63;
    out[(c0 + cc) * Rpad + r0 + rr] = t[rr][cc];
  }
}

// ---------------------------------------------------------------- backward

// dh pass.  Workgroup = (128-row tile, H slice of HS columns).  For every
// vocabulary tile: recompute z^T (vocabulary on M, tokens on N), form
// G[r][v] = scale_r * (exp(z - lse_r) - [v == y_r]) in bf16 into LDS, stage
// W^T[slice][tile] into LDS, and accumulate dh[r][slice] += G W.
template <int HS>
__global__ __launch_bounds__(NT) void k_bwd_dh(BwdArgs p) {
  constexpr int NB = HS / 64;  // 32-wide column blocks per wave (waves: 2 rows x 2 cols)
  __shared__ StageLds s;
  __shared__ u16 g_lds[TILE * LDS_T];
  u16* wt_lds = &s.a[0][0];  // reused after each logit tile: HS x 128 bf16
  static_assert(HS * LDS_T <= 2 * 2 * TILE * LDS_K, "W^T tile must fit in the stage buffers");

  const int64_t r0 = (int64_t)blockIdx.x * TILE;
  const int64_t c0 = (int64_t)blockIdx.y * HS;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t rend = min(r0 + TILE, p.L);

  const int n_valid = p.hdr->n_valid;
  const float g = *p.grad_loss;
  float lse2[2], scale[2];
  int64_t lab[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int64_t t = r0 + wn * 64 + nb * 32 + (lane & 31);
    const int64_t y = t < rend ? p.labels[t] : p.ignore_index;
    const bool valid = (t < rend) && y != p.ignore_index && y >= 0 && y < p.V;
    lab[nb] = valid ? y : -1;
    scale[nb] = valid ? g / (float)n_valid : 0.f;
    lse2[nb] = (t < rend) ? p.lse[t] * LOG2E : INFINITY;  // rows past L: probability 0
  }

  f32x16 dacc[2][NB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) zero(dacc[i][j]);

  for (int vt = 0; vt < p.vtiles; ++vt) {
    const int64_t v0 = (int64_t)vt * TILE;
    f32x16 acc[2][2];
    logit_tile(p.W, v0, p.V, p.h, r0, rend, p.H, s, acc);
    // G into LDS as g_lds[token][v] (token-major, v contiguous)
    const int64_t vw = v0 + wm * 64;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int tl = wn * 64 + nb * 32 + (lane & 31);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float gv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int reg = q * 4 + e;
            const int64_t v = vw + mb * 32 + acc_row(reg, lane);
            float pr = fast_exp2(__builtin_fmaf(acc[mb][nb][reg], LOG2E, -lse2[nb]));
            pr = (v == lab[nb]) ? pr - 1.f : pr;
            gv[e] = (v < p.V) ? pr * scale[nb] : 0.f;
          }
          const int vl = wm * 64 + mb * 32 + acc_row(q * 4, lane);
          store_bf16x4(g_lds + tl * LDS_T + vl, gv[0], gv[1], gv[2], gv[3]);
        }
      }
    }
    // W^T[c0 .. c0+HS][v0 .. v0+128] (zero-padded past V) into LDS
    tile_to_lds<HS>(p.WT, c0, p.Vpad, v0, wt_lds);
    __syncthreads();
    // dh[r][c] += sum_v G[r][v] W^T[c][v]; waves: 2 (rows) x 2 (columns)
    lds_mma<2, NB>(g_lds, wm * 64, wt_lds, wn * (HS / 2), dacc);
    __syncthreads();
  }

#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int reg = 0; reg < 16; ++reg) {
        const int64_t r = r0 + wm * 64 + mb * 32 + acc_row(reg, lane);
        const int64_t c = c0 + wn * (HS / 2) + nb * 32 + (lane & 31);
        if (r < p.L) p.dh[r * p.H + c] = dacc[mb][nb][reg];
      }
}

// dW pass.  Workgroup = (128-wide vocabulary tile, H slice of HS columns).
// For every 128-row tile: recompute z (tokens on M, vocabulary on N), form
// G^T[v][r] in bf16 into LDS, stage h^T[slice][rows] into LDS, and
// accumulate dW[v][slice] += G^T h.
template <int HS>
__global__ __launch_bounds__(NT) void k_bwd_dW(BwdArgs p) {
  constexpr int NB = HS / 64;
  __shared__ StageLds s;
  __shared__ u16 g_lds[TILE * LDS_T];
  __shared__ float row_lse2[TILE], row_scale[TILE];
  __shared__ int64_t row_lab[TILE];
  u16* ht_lds = &s.a[0][0];
  static_assert(HS * LDS_T <= 2 * 2 * TILE * LDS_K, "h^T tile must fit in the stage buffers");

  const int64_t v0 = (int64_t)blockIdx.x * TILE;
  const int64_t c0 = (int64_t)blockIdx.y * HS;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int n_valid = p.hdr->n_valid;
  const float g = *p.grad_loss;

  f32x16 dacc[2][NB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) zero(dacc[i][j]);

  const int ntiles = (int)((p.L + TILE - 1) / TILE);
  for (int rt = 0; rt < ntiles; ++rt) {
    const int64_t r0 = (int64_t)rt * TILE;
    const int64_t rend = min(r0 + TILE, p.L);
    if (threadIdx.x < TILE) {
      const int64_t t = r0 + threadIdx.x;
      const int64_t y = t < rend ? p.labels[t] : p.ignore_index;
      const bool valid = (t < rend) && y != p.ignore_index && y >= 0 && y < p.V;
      row_lab[threadIdx.x] = valid ? y : -1;
      row_scale[threadIdx.x] = valid ? g / (float)n_valid : 0.f;
      row_lse2[threadIdx.x] = (t < rend) ? p.lse[t] * LOG2E : INFINITY;  // rows past L: probability 0
    }
    f32x16 acc[2][2];
    // logit_tile's first barrier orders the row_* writes before their use.
    logit_tile(p.h, r0, rend, p.W, v0, p.V, p.H, s, acc);
    // G^T into LDS as g_lds[v][token] (v-major, tokens contiguous)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int vl = wn * 64 + nb * 32 + (lane & 31);
      const int64_t v = v0 + vl;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float gv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tl = wm * 64 + mb * 32 + acc_row(q * 4 + e, lane);
            float pr = fast_exp2(__builtin_fmaf(acc[mb][nb][q * 4 + e], LOG2E, -row_lse2[tl]));
            pr = (v == row_lab[tl]) ? pr - 1.f : pr;
            gv[e] = (v < p.V) ? pr * row_scale[tl] : 0.f;
          }
          const int tl0 = wm * 64 + mb * 32 + acc_row(q * 4, lane);
          store_bf16x4(g_lds + vl * LDS_T + tl0, gv[0], gv[1], gv[2], gv[3]);
        }
      }
    }
    // h^T[c0 .. c0+HS][r0 .. r0+128] (zero-padded past L) into LDS
    tile_to_lds<HS>(p.hT, c0, p.Lpad, r0, ht_lds);
    __syncthreads();
    // dW[v][c] += sum_r G^T[v][r] h^T[c][r]; waves: 2 (vocabulary) x 2 (columns)
    lds_mma<2, NB>(g_lds, wm * 64, ht_lds, wn * (HS / 2), dacc);
    __syncthreads();
  }

#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int reg = 0; reg < 16; ++reg) {
        const int64_t v = v0 + wm * 64 + mb * 32 + acc_row(reg, lane);
        const int64_t c = c0 + wn * (HS / 2) + nb * 32 + (lane & 31);
        if (v < p.V) p.dW[v * p.H + c] = dacc[mb][nb][reg];
      }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_count_labels(const int64_t* labels, int64_t L, int64_t V, int64_t ignore_index, WsHeader* hdr,
                               hipStream_t st) {
  hipLaunchKernelGGL(k_count_labels, dim3(1), dim3(1024), 0, st, labels, L, V, ignore_index, hdr);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, float* loss_out, float* lse_out, hipStream_t st) {
  const int ntiles = a.n_chunks * a.tiles_per_chunk;
  hipLaunchKernelGGL(k_fwd, dim3((unsigned)(ntiles * a.segments)), dim3(NT), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nblocks = (int)((a.L + 255) / 256);
  hipLaunchKernelGGL(k_fwd_rows, dim3(nblocks), dim3(256), 0, st, a, lse_out);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_fwd_loss, dim3(1), dim3(256), 0, st, a, nblocks, loss_out);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* in, int64_t R, int64_t C, void* out, int64_t Rpad, hipStream_t st) {
  dim3 grid((unsigned)(Rpad / 64), (unsigned)(C / 64));
  hipLaunchKernelGGL(k_transpose, grid, dim3(256), 0, st, (const u16*)in, R, C, (u16*)out, Rpad);
  return hipGetLastError();
}

hipError_t launch_bwd_dh(const BwdArgs& a, int hs, hipStream_t st) {
  const dim3 grid((unsigned)((a.L + TILE - 1) / TILE), (unsigned)(a.H / hs));
  if (hs == 256) hipLaunchKernelGGL(k_bwd_dh<256>, grid, dim3(NT), 0, st, a);
  else if (hs == 128) hipLaunchKernelGGL(k_bwd_dh<128>, grid, dim3(NT), 0, st, a);
  else hipLaunchKernelGGL(k_bwd_dh<64>, grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dW(const BwdArgs& a, int hs, hipStream_t st) {
  const dim3 grid((unsigned)a.vtiles, (unsigned)(a.H / hs));
  if (hs == 256) hipLaunchKernelGGL(k_bwd_dW<256>, grid, dim3(NT), 0, st, a);
  else if (hs == 128) hipLaunchKernelGGL(k_bwd_dW<128>, grid, dim3(NT), 0, st, a);
  else hipLaunchKernelGGL(k_bwd_dW<64>, grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace lmce
