// Forward kernels of the fused LM-head + cross-entropy loss (gfx950).
//
// Page: TRL docs "Training Beyond 1M Tokens", sections "The loss is the
// first thing to break" (logits = h W^T, cross entropy against the target
// labels) and "The massive logits matrix: chunk it" (each row's softmax runs
// over its own vocabulary, so per-row pieces combine exactly).
//
// k_fwd computes 256 (vocabulary) x BN (token) logit tiles with bf16 MFMA,
// K = H, and folds each tile in registers into per-lane online
// (max, sum of exp) states of the lane's tokens.  No logit leaves the
// registers.  k_fwd_rows merges the per-segment states of every row into its
// log-sum-exp, takes the label logit as one H-long dot product per row and
// forms nll; k_fwd_loss sums nll in a fixed order.

#include "lmce_device.h"
#include "lmce_internal.h"

namespace lmce {

// Counts rows whose label is not ignore_index and checks that the others lie
// in [0, V).  One workgroup; fixed-order reduction.  It is the first kernel of
// every entry point: it clears the call's own flags, ORs a label error into
// them and into the accumulated status (which only lmce_read_status clears),
// and initialises the header of a workspace this library has not used yet.
// `saved` >= 0 is written to the header's training-forward tag.
__global__ __launch_bounds__(1024) void k_count_labels(const int64_t* __restrict__ labels, int64_t L, int64_t V,
                                                       int64_t ignore_index, WsHeader* __restrict__ hdr, int saved) {
  __shared__ int s_cnt[1024];
  __shared__ int s_bad[1024];
  int cnt = 0, bad = 0;
  for (int64_t i = threadIdx.x; i < L; i += 1024) {
    const int64_t y = labels[i];
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
    if (hdr->tag != kHdrTag) {  // a fresh workspace: no earlier status, no saved forward
      hdr->status = 0;
      hdr->saved = 0;
      hdr->tag = kHdrTag;
    }
    const int flags = s_bad[0] ? kStatusLabel : 0;
    hdr->n_valid = s_cnt[0];
    hdr->call_flags = flags;
    hdr->status |= flags;
    if (saved >= 0) hdr->saved = saved;
  }
}

// Work item -> (row tile, vocabulary segment).  With 8 segments and a
// multiple of 32 row tiles, the 32 items that run together on one XCD cover
// 4 row tiles x 8 segments, so each h tile is shared by 8 and each W tile
// by 4 concurrent workgroups through that XCD's L2.
__device__ __forceinline__ void fwd_item(int i, const FwdArgs& p, int& tile, int& seg) {
  if (p.xcd_map) {
    const int x = i & 7, j = i >> 3;
    const int round = j >> 5, jj = j & 31;
    seg = jj & 7;
    tile = ((round * 8 + x) << 2) + (jj >> 3);
  } else {
    seg = i % p.segments;
    tile = i / p.segments;
  }
}

// Folds one logit tile into the lane's running (max, sum) states.  Lane l
// holds, for each of its NB tokens, MB*16 logits (MB blocks x 16 rows).
// MASK: rows at or past `valid_rows` (counted from this wave's first
// vocabulary row) lie beyond V and are skipped.
template <int MB, int NB, bool MASK>
__device__ __forceinline__ void fold_tile(const f32x16 (&acc)[MB][NB], float (&m)[NB], float (&sum)[NB],
                                          int valid_rows, int lane) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float mt = kNegBig;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool in = !MASK || (mb * 32 + acc_row(r, lane) < valid_rows);
        mt = in ? fmaxf(mt, acc[mb][nb][r]) : mt;
      }
    const float mn = fmaxf(m[nb], mt);
    const float off = -mn * kLog2e;
    float add = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2_fast(__builtin_fmaf(acc[mb][nb][r], kLog2e, off));
        const bool in = !MASK || (mb * 32 + acc_row(r, lane) < valid_rows);
        add += in ? e : 0.f;
      }
    sum[nb] = sum[nb] * exp2_fast((m[nb] - mn) * kLog2e) + add;
    m[nb] = mn;
    __builtin_amdgcn_sched_barrier(0);  // one token block at a time: bounded register use
  }
}

// 8 waves (2 per SIMD) in a 4 (vocabulary) x 2 (token) grid over a 256 x BN
// logit tile: each wave holds 64 vocabulary rows of BN/2 tokens.
constexpr int kFwdWM = 4, kFwdWN = 2, kFwdThreads = 64 * kFwdWM * kFwdWN;

template <int BN>
__global__ __launch_bounds__(kFwdThreads) void k_fwd(FwdArgs p) {
  using G = TileGemm<256, BN, kFwdWM, kFwdWN, 0, 0, 0, true>;
  constexpr int MB = G::MB, NB = G::NB;
  __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES];
  __shared__ float red_m[kFwdWM - 1][BN], red_s[kFwdWM - 1][BN];

  int tile, seg;
  fwd_item(blockIdx.x, p, tile, seg);
  const int64_t chunk = tile / p.tiles_per_chunk;
  const int64_t cbeg = chunk * p.chunk_rows;
  const int64_t cend = min(cbeg + (int64_t)p.chunk_rows, p.L);
  const int64_t r0 = cbeg + (int64_t)(tile % p.tiles_per_chunk) * BN;
  if (r0 >= cend) return;  // uniform across the workgroup
  const int64_t rend = min(r0 + BN, cend);

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave / kFwdWN, wn = wave % kFwdWN;
  const int64_t H = p.H, V = p.V;

  int64_t tok[NB];
  float m[NB], sum[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    tok[nb] = r0 + wn * (BN / 2) + nb * 32 + (lane & 31);
    m[nb] = kNegBig;
    sum[nb] = 0.f;
  }
  const Operand ob = linear_operand(p.h + r0 * H, (uint64_t)(rend - r0) * H * 2, (uint32_t)(H * 2));

  const int vt0 = seg * p.vtiles_per_seg;
  const int vt1 = min(vt0 + p.vtiles_per_seg, p.vtiles);
  for (int vt = vt0; vt < vt1; ++vt) {
    const int64_t v0 = (int64_t)vt * 256;
    // A = W rows (vocabulary on the MFMA M side), B = h rows (tokens on N):
    // every logit of a token sits in the registers of one lane pair per wave.
    const Operand oa = linear_operand(p.W + v0 * H, (uint64_t)(V - v0) * H * 2, (uint32_t)(H * 2));
    f32x16 acc[MB][NB];
    zero_acc(acc);
    G::run(oa, ob, (int)H, lds, acc);
    if (v0 + 256 <= V) fold_tile<MB, NB, false>(acc, m, sum, 0, lane);
    else fold_tile<MB, NB, true>(acc, m, sum, (int)(V - (v0 + wm * 64)), lane);  // ragged last tile
  }

  // Merge the two lane halves (same tokens, other vocabulary rows), then the
  // four waves that share tokens, in wave order; one (max, sum) pair per
  // token and segment.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float m2 = __shfl_xor(m[nb], 32);
    const float s2 = __shfl_xor(sum[nb], 32);
    lse_merge(m[nb], sum[nb], m2, s2);
  }
  if (wm > 0 && lane < 32) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      red_m[wm - 1][wn * (BN / 2) + nb * 32 + lane] = m[nb];
      red_s[wm - 1][wn * (BN / 2) + nb * 32 + lane] = sum[nb];
    }
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int t = wn * (BN / 2) + nb * 32 + lane;
#pragma unroll
      for (int w = 0; w < kFwdWM - 1; ++w) lse_merge(m[nb], sum[nb], red_m[w][t], red_s[w][t]);
      if (tok[nb] < rend) {
        p.part_m[(int64_t)seg * p.L + tok[nb]] = m[nb];
        p.part_s[(int64_t)seg * p.L + tok[nb]] = sum[nb];
      }
    }
  }
}

// Per row (one wave each, 16 rows per wave, 64 rows per workgroup): merge
// the segment states in segment order into lse; the label logit
// z_{i, y_i} = h_i . W_{y_i} is a fp32 dot product over H; nll = lse - z.
// Per workgroup: fixed-order sum of its 64 nll values into block_sum.
__global__ __launch_bounds__(256) void k_fwd_rows(FwdArgs p, float* __restrict__ lse_out) {
  __shared__ float red[64];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int64_t H = p.H;
  for (int i = 0; i < 16; ++i) {
    const int local = wave * 16 + i;
    const int64_t r = (int64_t)blockIdx.x * 64 + local;
    float nll = 0.f;
    if (r < p.L) {
      const int64_t y = p.labels[r];
      const bool valid = y != p.ignore_index && y >= 0 && y < p.V;
      float dot = 0.f;
      if (valid) {
        const u16* hr = p.h + r * H;
        const u16* wr = p.W + y * H;
        for (int64_t k = lane * 8; k < H; k += 512) {
          const bf16x8 a = *(const bf16x8*)(hr + k);
          const bf16x8 b = *(const bf16x8*)(wr + k);
#pragma unroll
          for (int e = 0; e < 8; ++e) dot = __builtin_fmaf((float)a[e], (float)b[e], dot);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
      }
      if (lane == 0) {
        // the training forward may have run the rows in a labelled-first order
        const int64_t pos = (p.finv != nullptr && p.hdr->fcompact) ? (int64_t)p.finv[r] : r;
        float m = kNegBig, s = 0.f;
        for (int seg = 0; seg < p.segments; ++seg)
          lse_merge(m, s, p.part_m[(int64_t)seg * p.L + pos], p.part_s[(int64_t)seg * p.L + pos]);
        const float lse = m + logf(s);
        lse_out[r] = lse;
        nll = valid ? lse - dot : 0.f;
      }
    }
    if (lane == 0) red[local] = nll;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float acc = 0.f;
    for (int i = 0; i < 64; ++i) acc += red[i];
    p.block_sum[blockIdx.x] = acc;
  }
}

// loss = (sum of block sums, fixed order) / N; NaN if N == 0, or if this call
// saw a bad label or a group wait that gave up.  train: the last kernel of the
// training forward, which marks the workspace as holding a complete O only
// when none of its group waits gave up.
__global__ __launch_bounds__(256) void k_fwd_loss(FwdArgs p, int nblocks, float* __restrict__ loss_out, int train,
                                                  const float* o_buf) {
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
    const int flags = __hip_atomic_load(&p.hdr->call_flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float loss = (n > 0) ? red[0] / (float)n : __builtin_nanf("");
    if (flags != 0) loss = __builtin_nanf("");
    *loss_out = loss;
    if (train) {
      p.hdr->o_addr = (unsigned long long)(uintptr_t)o_buf;
      p.hdr->saved = (flags & kStatusSync) ? 0 : kSavedTag;
    }
  }
}

hipError_t launch_count_labels(const int64_t* labels, int64_t L, int64_t V, int64_t ignore_index, WsHeader* hdr,
                               int saved, hipStream_t st) {
  hipLaunchKernelGGL(k_count_labels, dim3(1), dim3(1024), 0, st, labels, L, V, ignore_index, hdr, saved);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, float* loss_out, float* lse_out, hipStream_t st) {
  const unsigned items = (unsigned)(a.ntiles * a.segments);
  if (a.tile_rows == 256) hipLaunchKernelGGL(k_fwd<256>, dim3(items), dim3(kFwdThreads), 0, st, a);
  else hipLaunchKernelGGL(k_fwd<128>, dim3(items), dim3(kFwdThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_fwd_rows(a, loss_out, lse_out, st);
}

// Merges the per-segment (max, sum) partials of every row into lse, forms
// nll and the loss.
hipError_t launch_fwd_rows(const FwdArgs& a, float* loss_out, float* lse_out, hipStream_t st, bool train,
                           const float* o_buf) {
  hipError_t e;
  const int nblocks = (int)((a.L + 63) / 64);
  hipLaunchKernelGGL(k_fwd_rows, dim3(nblocks), dim3(256), 0, st, a, lse_out);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_fwd_loss, dim3(1), dim3(256), 0, st, a, nblocks, loss_out, train ? 1 : 0, o_buf);
  return hipGetLastError();
}

}  // namespace lmce
