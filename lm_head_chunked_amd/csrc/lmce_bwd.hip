// Backward kernels of the fused LM-head + cross-entropy loss (gfx950).
//
// Page: TRL docs "Training Beyond 1M Tokens", section "The massive logits
// matrix: chunk it" (per-row pieces); the gradient of the mean NLL is
// G = g/N * valid * (softmax - onehot), dh = G W and dW = G^T h.
//
// dh and dW are H wide: a 256 x H fp32 accumulator (4 MiB at H = 4096) does
// not fit in one compute unit, so each pass runs as groups of s = H / HS
// workgroups, workgroup j of a group owning an HS-wide slice of the
// accumulator (HS = 128 in registers, or 256 parked in the workspace between
// rounds).  In every round each member recomputes R = round_tiles(HS) full-H
// 256 x 256 logit tiles with MFMA (two with 256-wide slices, one with
// 128-wide), turns each into bf16 G' = valid * (softmax - onehot) (or P) in
// registers and writes it to the group's exchange slot; after a group barrier
// every member contracts all R x s tiles of the round into its own slice.
// The factor g/N of G = g/N * G' multiplies the fp32 slice when it is stored:
// folded into G before the bf16 rounding, its own rounding error (up to 2^-9
// relative, the same for every term) would scale the whole result.  Each
// logit is thus recomputed exactly once per pass and no logit or G tile
// exists for more than one round (the exchange holds 2 x R x s tiles per
// group).  Two tiles
// per round halve the group barriers and the parked accumulator's round
// trips; four were slower (the exchange then outgrows what the last-level
// cache keeps).
//
//   k_bwd_dh : group = 256 rows of h; rounds sweep the vocabulary, 256 per
//              member; dh[rows][slice] += G W   (row-owned, no atomics)
//   k_bwd_dW : group = 256 vocabulary rows; rounds sweep the tokens, 256 per
//              member; dW[rows][slice] += G^T h (vocabulary-owned, no atomics)
//              over the labelled rows only when that saves a block
//              (k_compact_rows), the leftover vocabulary blocks split over
//              all groups and summed by k_dw_tail
//   k_fwd_dh : the training forward, the groups and rounds of k_bwd_dh with
//              an online softmax: lse of every row and O = sum_v softmax W_v
//
// The groups run as one cooperative launch (all workgroups resident), placed
// on the XCDs as the host chooses (xcd_tiled).  The exchange uses
// device-coherent (sc1) stores and loads and a per-group arrival counter;
// every wait is bounded and reports a sync error instead of hanging.

#include "lmce_device.h"
#include "lmce_internal.h"

namespace lmce {

// ------------------------------------------------ labelled-row compaction
// Rows without a label (ignore_index) carry no gradient: their G row is 0 and
// they add nothing to dW.  When dropping them saves at least one 256-row
// block, the dW pass sweeps only the labelled rows, in their original order
// (a stable compaction, so the results are repeatable).

// Labelled rows of each 1024-row chunk.
__global__ __launch_bounds__(256) void k_count_chunks(const int64_t* __restrict__ labels, int64_t L, int64_t V,
                                                      int64_t ignore_index, int* __restrict__ cnt) {
  __shared__ int red[256];
  const int64_t base = (int64_t)blockIdx.x * 1024;
  int c = 0;
  for (int i = threadIdx.x; i < 1024; i += 256) {
    const int64_t r = base + i;
    if (r < L) {
      const int64_t y = labels[r];
      c += (y != ignore_index && y >= 0 && y < V) ? 1 : 0;
    }
  }
  red[threadIdx.x] = c;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) cnt[blockIdx.x] = red[0];
}

// Decides the compaction (every block reaches the same decision from the
// same counts) and writes, for the labelled rows of its chunk in order, their
// index, label and lse.  ch_rows: rows the gathered-rows area can hold.
__global__ __launch_bounds__(1024) void k_compact_rows(const int64_t* __restrict__ labels, const float* __restrict__ lse,
                                                       int64_t L, int64_t V, int64_t ignore_index, int64_t ch_rows,
                                                       const int* __restrict__ cnt, int nchunks, WsHeader* hdr,
                                                       int* __restrict__ crow, int64_t* __restrict__ clab,
                                                       float* __restrict__ clse) {
  __shared__ int scan[1024];
  __shared__ int s_before, s_total;
  if (threadIdx.x == 0) {
    int before = 0, total = 0;
    for (int b = 0; b < nchunks; ++b) {
      if (b < (int)blockIdx.x) before += cnt[b];
      total += cnt[b];
    }
    s_before = before;
    s_total = total;
  }
  __syncthreads();
  const int64_t n = s_total;
  const bool compact = (n + 255) / 256 < (L + 255) / 256 && n <= ch_rows;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    hdr->compact = compact ? 1 : 0;
    hdr->n_compact = compact ? (int)n : 0;
  }
  if (!compact) return;
  const int64_t r = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  int64_t y = ignore_index;
  if (r < L) y = labels[r];
  const int f = (r < L && y != ignore_index && y >= 0 && y < V) ? 1 : 0;
  scan[threadIdx.x] = f;
  __syncthreads();
  // inclusive scan over the block (Hillis-Steele)
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = (int)threadIdx.x >= d ? scan[threadIdx.x - d] : 0;
    __syncthreads();
    scan[threadIdx.x] += v;
    __syncthreads();
  }
  if (f) {
    const int64_t pos = s_before + scan[threadIdx.x] - 1;
    crow[pos] = (int)r;
    clab[pos] = y;
    clse[pos] = lse[r];
  }
}

// Training forward: when it saves at least one 256-row block, a stable
// labelled-first order of the rows (labelled rows at positions 0 .. n-1 in
// their order, the others after them in theirs): fperm[position] = row,
// finv[row] = position.  Row blocks made only of unlabelled rows then compute
// lse alone, without the O contraction.
__global__ __launch_bounds__(1024) void k_permute_rows(const int64_t* __restrict__ labels, int64_t L, int64_t V,
                                                       int64_t ignore_index, const int* __restrict__ cnt, int nchunks,
                                                       int* flags, int* __restrict__ fperm, int* __restrict__ finv) {
  __shared__ int scan[1024];
  __shared__ int s_before, s_total;
  if (threadIdx.x == 0) {
    int before = 0, total = 0;
    for (int b = 0; b < nchunks; ++b) {
      if (b < (int)blockIdx.x) before += cnt[b];
      total += cnt[b];
    }
    s_before = before;
    s_total = total;
  }
  __syncthreads();
  const int64_t n = s_total;
  const bool compact = (n + 255) / 256 < (L + 255) / 256;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    flags[0] = compact ? 1 : 0;
    flags[1] = compact ? (int)n : 0;
  }
  if (!compact) return;
  const int64_t r = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  int f = 0;
  if (r < L) {
    const int64_t y = labels[r];
    f = (y != ignore_index && y >= 0 && y < V) ? 1 : 0;
  }
  scan[threadIdx.x] = f;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = (int)threadIdx.x >= d ? scan[threadIdx.x - d] : 0;
    __syncthreads();
    scan[threadIdx.x] += v;
    __syncthreads();
  }
  if (r < L) {
    const int64_t lab_before = s_before + scan[threadIdx.x] - f;  // labelled rows before r
    const int64_t pos = f ? lab_before : n + (r - lab_before);
    fperm[pos] = (int)r;
    if (finv) finv[r] = (int)pos;
  }
}

// h rows in the labelled-first order (one row per block), when in use.
__global__ __launch_bounds__(256) void k_gather_perm(const u16* __restrict__ h, int64_t H, const int* flags,
                                                     const int* __restrict__ fperm, u16* __restrict__ hp) {
  if (flags[0] == 0) return;
  const int64_t src = fperm[blockIdx.x];
  const uint4* in = reinterpret_cast<const uint4*>(h + src * H);
  uint4* out = reinterpret_cast<uint4*>(hp + (int64_t)blockIdx.x * H);
  for (int64_t c = threadIdx.x; c < H / 8; c += 256) out[c] = in[c];
}

// h rows of the labelled rows, in order, into the rows area (one row per
// block; rows past the compaction's own count exit).
__global__ __launch_bounds__(256) void k_gather_rows(const u16* __restrict__ h, int64_t H, const WsHeader* hdr,
                                                     const int* __restrict__ crow, u16* __restrict__ ch) {
  if (hdr->compact == 0 || (int)blockIdx.x >= hdr->n_compact) return;
  const int64_t src = crow[blockIdx.x];
  const uint4* in = reinterpret_cast<const uint4*>(h + src * H);
  uint4* out = reinterpret_cast<uint4*>(ch + (int64_t)blockIdx.x * H);
  for (int64_t c = threadIdx.x; c < H / 8; c += 256) out[c] = in[c];
}

// dW rows of the leftover blocks of the dW pass: block t of them was swept by
// groups t * gpb .. t * gpb + gpb - 1, member j's partial 256 x HS slice of
// group q at dw_part + (q * s + j) * 256 * HS; they are added in group order.
// One workgroup per (block, member).
__global__ __launch_bounds__(256) void k_dw_tail(const float* __restrict__ part, float* __restrict__ dW, int64_t V,
                                                 int64_t H, int hs, int s, int gpb, int64_t v_first) {
  const int t = blockIdx.x / s, j = blockIdx.x % s;
  const int64_t v0 = v_first + (int64_t)t * 256;
  for (int e = threadIdx.x * 4; e < 256 * hs; e += 1024) {
    const int r = e / hs, c = e % hs;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int q = 0; q < gpb; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(part + ((int64_t)(t * gpb + q) * s + j) * 256 * hs + e);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    if (v0 + r < V) *reinterpret_cast<float4*>(dW + (v0 + r) * H + (int64_t)j * hs + c) = acc;
  }
}

// dW *= g/N after a dW pass with 128-wide slices (which stores G'^T h).
__global__ __launch_bounds__(256) void k_dw_scale(float* __restrict__ dW, int64_t n4,
                                                  const float* __restrict__ grad_loss, const WsHeader* __restrict__ hdr) {
  const int n = hdr->n_valid;
  const float f = *grad_loss / (float)(n > 0 ? n : 1);
  float4* d = reinterpret_cast<float4*>(dW);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    float4 v = d[i];
    v.x *= f;
    v.y *= f;
    v.z *= f;
    v.w *= f;
    d[i] = v;
  }
}

__global__ void k_zero_u32(unsigned* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Position of workgroup b in XCD-major order (workgroups are dispatched to
// the 8 XCDs round-robin), so that the members of a group share an L2: the
// dW pass's order when xcd_tiled does not apply.
__device__ __forceinline__ int xcd_major(int b, int nwg) {
  if (nwg % 8 != 0) return b;
  return (b & 7) * (nwg >> 3) + (b >> 3);
}

// Position of workgroup b with the members of each group spread over the
// XCDs: b = g * s + j, so member j of every group sits on XCD (g * s + j) % 8,
// which is j % 8 for all groups when s is a multiple of 8.  The order of the
// passes whose groups own row blocks when xcd_tiled does not apply: in a
// round, member j of every group loads the same vocabulary tile of W (and the
// same H columns of the round's W rows), so groups that share an XCD read it
// through one L2.
// The exchange then crosses XCDs, which its device-coherent stores and loads
// allow.
__device__ __forceinline__ int member_spread(int b) { return b; }

// Position of workgroup b when every XCD hosts `a` members of each of
// nwg / 8 / a groups: a group spans s / a XCDs, and in a round the workgroups
// of one XCD read a distinct member operands and nwg / 8 / a distinct group
// operands, each through one L2 (XCD x, index i on it: group
// (x / (s/a)) * (nwg/8/a) + i / a, member (x % (s/a)) * a + i % a).  The host
// passes a > 0 only when nwg % 8 == 0, s % a == 0, 8 % (s / a) == 0 and
// (nwg / 8) % a == 0; the map is then a bijection of [0, nwg).
__device__ __forceinline__ int xcd_tiled(int b, int nwg, int s, int a) {
  const int x = b & 7, i = b >> 3;
  const int per = s / a;
  const int bg = (nwg >> 3) / a;
  return ((x / per) * bg + i / a) * s + (x % per) * a + i % a;
}

// All s members of group g have written round `epoch`; bounded wait.
// Returns false (and records kStatusSync) if the group did not arrive.
__device__ __forceinline__ bool group_arrive_wait(unsigned* ctr, unsigned target, int spin_limit, WsHeader* hdr,
                                                  int* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's exchange stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int n = 0, ok = 1;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++n > spin_limit) {
        ok = 0;
        break;
      }
    }
    if (!ok) {
      __hip_atomic_fetch_or(&hdr->status, kStatusSync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_or(&hdr->call_flags, kStatusSync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    *s_flag = ok;
  }
  __syncthreads();
  return *s_flag != 0;
}

// Producer and consumer tiles.  Eight waves (two per SIMD) in a 4 x 2 grid;
// the producer's 256 x 256 logit tile gives each wave 64 x 128 logits (128
// accumulator registers).  HS is the H slice one member owns:
//   HS = 128: the 256 x 128 accumulator slice (64 registers per lane) stays
//             in registers across the rounds of a block, beside the logit tile;
//   HS = 256: the 256 x 256 slice (128 registers) does not fit beside the
//             logit tile, so between two contractions it is parked in the
//             workgroup's own workspace area (256 KiB out and back per round)
//             and both GEMMs run on square 256 x 256 tiles.
constexpr int kBwdThreads = 512;

template <int HS>
struct BwdCfg {
  static constexpr bool kPark = HS == 256;
  // producers: the logit tile; h's rows are the B operand (row-block passes) or the A operand (dW
  // pass), read in place (P, PA) or through the row order or selection (gathered form: PG, PAG, a
  // separate instantiation so that the in-order case keeps its registers)
  using P = TileGemm<256, 256, 4, 2, 0, 0, 0, kPark>;
  using PG = TileGemm<256, 256, 4, 2, 0, 0, 3, kPark>;
  using PA = TileGemm<256, 256, 4, 2, 0, 0, 0, kPark>;
  using PAG = TileGemm<256, 256, 4, 2, 0, 3, 0, kPark>;
  // consumers: the exchange slot against W's rows (row-block passes) or h's rows (dW pass), read MN-major;
  // the dW pass's through the row selection (gathered form) with 256-wide slices only: the three-stage
  // schedule of 128-wide slices would wait for its index loads, so with those the selected rows come
  // from a gathered copy (the host plans one)
  using C = TileGemm<256, HS, 4, 2, kAuxSc1, 1, 2, true>;
  using CH = TileGemm<256, HS, 4, 2, kAuxSc1, 1, HS == 256 ? 4 : 2, true>;
  static constexpr int kLds = P::LDS_BYTES > C::LDS_BYTES ? P::LDS_BYTES : C::LDS_BYTES;
  static_assert(PG::LDS_BYTES == P::LDS_BYTES && PAG::LDS_BYTES == P::LDS_BYTES && CH::LDS_BYTES == C::LDS_BYTES,
                "same stages");
};

// Parking area of one workgroup: accumulator register r of lane l of wave w
// at float index (w * R + r) * 64 + l (R registers per lane), moved with
// 4-byte buffer accesses: the lane part is one vector offset, the register
// part an immediate offset, the block of 16 registers the scalar offset, so
// no address register stays live across the transfers and they pipeline.
template <int MB, int NB>
__device__ __forceinline__ void park_acc(const f32x16 (&acc)[MB][NB], rsrc_t rs, int wave, int lane) {
  // (a fresh value at every call: otherwise the compiler hoists the 16
  // offsets voff + 256 e out of the round loop as registers of their own,
  // instead of immediate offsets, and spills them)
  uint32_t voff = (uint32_t)lane * 4u;
  asm volatile("" : "+v"(voff));
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        store_b32(rs, voff + (uint32_t)e * 256u, (uint32_t)((wave * MB * NB + mb * NB + nb) * 4096), acc[mb][nb][e]);
}

template <int MB, int NB>
__device__ __forceinline__ void unpark_acc(f32x16 (&acc)[MB][NB], rsrc_t rs, int wave, int lane) {
  uint32_t voff = (uint32_t)lane * 4u;  // (fresh at every call, as in park_acc)
  asm volatile("" : "+v"(voff));
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        acc[mb][nb][e] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rs, voff + (uint32_t)e * 256u,
                                                        (uint32_t)((wave * MB * NB + mb * NB + nb) * 4096), 0));
}

// A member's G tile is staged in LDS as [256 rows][256 K] bf16 (512 bytes
// per row), the 16-byte chunk c of row r at chunk c ^ (r % 32): 32 lanes that
// write the same chunk of 32 consecutive rows, or read the 32 chunks of one
// row, hit distinct banks.  Byte offset of K elements k .. k+3 (k % 4 == 0).
__device__ __forceinline__ uint32_t gstage_offset(int row, int k) {
  return (uint32_t)(row * 512 + ((((k >> 3) ^ (row & 31)) << 4) | ((k & 4) << 1)));
}

__device__ __forceinline__ void gstage_put(char* lds, int row, int k, uint64_t v) {
  *reinterpret_cast<__attribute__((address_space(3))) uint64_t*>(
      (__attribute__((address_space(3))) char*)lds + gstage_offset(row, k)) = v;
}

// Copies the staged tile into the member's two K-tiles (2j, 2j+1) of the
// round's slot, a sequence of [256][128] bf16 K-tiles: each half-wave writes
// one 256-byte row segment per instruction.
__device__ __forceinline__ void gstage_flush(const char* lds, rsrc_t rslot, int j) {
  const int t = threadIdx.x;
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int idx = i * 512 + t;   // 16-byte chunk of the tile
    const int row = idx >> 5, c = idx & 31;
    const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
        (const __attribute__((address_space(3))) char*)lds + row * 512 + ((c ^ (row & 31)) << 4));
    const uint32_t voff = (uint32_t)(((c >> 4) * 256 * 128 + row * 128 + (c & 15) * 8) * 2);
    store_sc1_b128(rslot, voff + (uint32_t)j * 2u * 256u * 128u * 2u, v);
  }
}

// g/N, the factor of G = g/N * G' that the passes apply to their fp32
// results.  Read where a result is stored (relaxed atomic loads, which the
// compiler does not hoist), so that it is not held in a register across the
// rounds.
__device__ __forceinline__ float grad_factor(const BwdArgs& p) {
  const int n = __hip_atomic_load(&p.hdr->n_valid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float g = __hip_atomic_load(p.grad_loss, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return g / (float)(n > 0 ? n : 1);
}

// ---------------------------------------------------------------- dh pass
// Group = 256 rows of h.  Round k: member j recomputes the logit tiles of
// vocabulary rows [((k*R + e)*s + j)*256, +256), e < R = round_tiles(HS),
// against the group's rows (A = W, B = h, so the tile is z^T: vocabulary on
// M, tokens on N), forms G[token][v] and stores each as two K-tiles
// (2(e*s + j), +1) of the round's slot [256 tokens][K].  Then every member
// accumulates
//   dh[rows][c0 .. c0+HS] += slot[256][K] * W[round's vocabulary][c0 .. c0+HS]
// with K = 128 * (K-tiles in the round), W's rows read MN-major (no copy).
// Writes an accumulator tile of TileGemm's layout (rows row0 + ..., columns
// col0 + ...) whose tile rows are positions pos0 + ... of a row order:
// position pos goes to dh row perm[pos], columns c0 + ...; positions at or
// past L are skipped.  ZERO writes zeros instead (acc is not read).
template <int MB, int NB, bool ZERO>
__device__ __forceinline__ void store_rows_perm(float* dh, const int* perm, int64_t pos0, int64_t L, int64_t H,
                                                int64_t c0, const f32x16 (&acc)[MB][NB], int row0, int col0, int lane,
                                                float f = 1.f) {
  const int lrow = (lane >> 5) << 2;  // row offset of this lane half
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int reg = 0; reg < 16; ++reg) {
      const int64_t pos = pos0 + row0 + mb * 32 + ((reg >> 2) << 3) + (reg & 3) + lrow;
      if (pos < L) {
        float* d = dh + (int64_t)perm[pos] * H + c0 + col0 + (lane & 31);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) d[nb * 32] = ZERO ? 0.f : acc[mb][nb][reg] * f;
      }
    }
}

template <int HS>
__global__ __launch_bounds__(kBwdThreads) void k_bwd_dh(BwdArgs p) {
  using P = typename BwdCfg<HS>::P;
  using PG = typename BwdCfg<HS>::PG;
  using C = typename BwdCfg<HS>::C;
  constexpr bool kPark = BwdCfg<HS>::kPark;
  __shared__ __attribute__((aligned(16))) char lds[BwdCfg<HS>::kLds];
  __shared__ int s_flag;

  const int s = p.group_size;
  const int q = p.xcd_members > 0 ? xcd_tiled(blockIdx.x, gridDim.x, s, p.xcd_members) : member_spread(blockIdx.x);
  const int g = q / s, j = q % s;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t H = p.H, V = p.V, L = p.L;
  const int64_t c0 = (int64_t)j * HS;
  const rsrc_t park = make_rsrc(p.park + (int64_t)blockIdx.x * (kParkPerWG / 4), kPark ? kParkPerWG : 0);  // this workgroup's parking area
  constexpr int R = round_tiles(HS);
  const int64_t slot_elems = (int64_t)R * s * 256 * 256;  // 2Rs K-tiles of [256][128]
  const int vt256 = (int)((V + 255) / 256);
  const int vt128 = (int)((V + 127) / 128);
  const int rounds = (vt256 + R * s - 1) / (R * s);
  const int nrb = (int)((L + 255) / 256);
  // Rows in this pass's labelled-first order when it saves a block
  // (crow[position] = row, h rows in hp): blocks past the labelled rows only
  // write their zero dh rows, and every row is read and written through the
  // order.  Each row's products and their order stay the same.
  const bool reordered = p.hdr->dcompact != 0;
  const int64_t n_lab = reordered ? (int64_t)p.hdr->d_n : L;
  // h rows in the pass's order: through the order itself, or (when 32-bit
  // offsets cannot reach all of h) from the gathered copy
  const bool by_index = reordered && !p.gather_copy;
  const u16* const hrows = reordered && p.gather_copy ? p.hp : p.h;
  unsigned epoch = 0;

  for (int rb = g; rb < nrb; rb += p.n_groups) {
    const int64_t r0 = (int64_t)rb * 256;
    const int64_t rend = min(r0 + 256, L);
    if (r0 >= n_lab) {  // (the whole group skips the block: the same rb for every member)
      f32x16 none[C::MB][C::NB];
      store_rows_perm<C::MB, C::NB, true>(p.dh, p.crow, r0, L, H, c0, none, wm * 64, wn * (HS / 2), lane);
      continue;
    }
    // producer wave (wm: vocabulary quarter, wn: token half); lane's 4 tokens
    float lse2[4], keep[4];
    int lab[4];  // label, or -2^30 for rows that take no gradient
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int64_t t = r0 + wn * 128 + nb * 32 + (lane & 31);
      const int64_t src = t < rend ? (reordered ? (int64_t)p.crow[t] : t) : 0;
      const int64_t y = t < rend ? p.labels[src] : p.ignore_index;
      const bool valid = t < rend && y != p.ignore_index && y >= 0 && y < V;
      lab[nb] = valid ? (int)y : -(1 << 30);
      keep[nb] = valid ? 1.f : 0.f;
      lse2[nb] = t < rend ? p.lse[src] * kLog2e : INFINITY;  // rows past L: probability 0
    }
    const Operand oh = by_index ? gathered_operand(p.h, (uint64_t)L * H * 2, (uint32_t)(H * 2), p.crow + r0,
                                                   (int)(rend - r0))
                                : gathered_operand(hrows + r0 * H, (uint64_t)(rend - r0) * H * 2, (uint32_t)(H * 2),
                                                   nullptr, (int)(rend - r0));

    f32x16 dacc[C::MB][C::NB];
    if constexpr (!kPark) zero_acc(dacc);
    for (int k = 0; k < rounds; ++k, ++epoch) {
      u16* slot = p.xbuf + ((int64_t)g * 2 + (epoch & 1)) * slot_elems;
      const rsrc_t rslot = make_rsrc(slot, (uint64_t)slot_elems * 2);
      for (int e = 0; e < R; ++e) {
        const int vt = (k * R + e) * s + j;
        if (vt < vt256) {
          const int v0 = vt * 256;
          f32x16 z[P::MB][P::NB];
          zero_acc(z);
          const Operand ow = linear_operand(p.W + (int64_t)v0 * H, (uint64_t)(V - v0) * H * 2, (uint32_t)(H * 2));
          if (by_index) PG::run(ow, oh, (int)H, lds, z);
          else P::run(ow, oh, (int)H, lds, z);
          // G'[token][v] = valid * (exp(z - lse) - [v == y]), staged in LDS as
          // [token][v], 4 consecutive v per write (G = g/N * G': the factor is
          // applied to the fp32 dh, so that its bf16 rounding does not scale
          // every term alike).  Tile-local coordinates: vl = v - v0, the
          // label at lab - v0.
          const int vlim = min((int)(V - v0), 256);
          raw_barrier();  // every wave is done with the GEMM's last LDS stage
  #pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int yl = lab[nb] - v0;  // outside [0, 256) if the label is not in this tile
  #pragma unroll
            for (int mb = 0; mb < 2; ++mb)
  #pragma unroll
              for (int qq = 0; qq < 4; ++qq) {
                float gv[4];
                const int vl0 = wm * 64 + mb * 32 + acc_row(qq * 4, lane);
  #pragma unroll
                for (int e = 0; e < 4; ++e) {
                  float pr = exp2_fast(__builtin_fmaf(z[mb][nb][qq * 4 + e], kLog2e, -lse2[nb]));
                  pr = (vl0 + e == yl) ? pr - 1.f : pr;
                  gv[e] = pr * ((vl0 + e < vlim) ? keep[nb] : 0.f);
                }
                gstage_put(lds, wn * 128 + nb * 32 + (lane & 31), vl0, pack_bf16x4(gv[0], gv[1], gv[2], gv[3]));
              }
            __builtin_amdgcn_sched_barrier(0);
          }
          __syncthreads();
          gstage_flush(lds, rslot, e * s + j);
        }
      }
      if constexpr (kPark) {
        if (k == 0) zero_acc(dacc);
        else unpark_acc(dacc, park, wave, lane);
      }
      if (!group_arrive_wait(p.sync + g * kSyncStride, (unsigned)s * (epoch + 1), p.spin_limit, p.hdr, &s_flag))
        return;
      const int ntl = min(2 * R * s, vt128 - k * 2 * R * s);
      const int64_t vbase = (int64_t)k * R * s * 256;
      // A: the slot's K-tiles [256][128]; B: the round's W rows (K = vocabulary),
      // columns c0 .. c0+HS, read MN-major (rows past V read as zero)
      const int64_t krows = min<int64_t>((int64_t)ntl * 128, V - vbase);
      C::run(tiled_operand(slot, (uint64_t)slot_elems * 2, 256, 256 * 128 * 2),
             linear_operand(p.W + vbase * H, (uint64_t)krows * H * 2, (uint32_t)(H * 2), (uint32_t)(c0 * 2)),
             ntl * 128, lds, dacc);
      if constexpr (kPark) park_acc(dacc, park, wave, lane);  // also after the last round: dacc is dead at the back edge
    }
    // dh[r][c] = g/N * (G' W)[r][c] for r < L (waves: wm token quarter, wn column half)
    if constexpr (kPark) {
      f32x16 fin[C::MB][C::NB];
      unpark_acc(fin, park, wave, lane);
      if (reordered)
        store_rows_perm<C::MB, C::NB, false>(p.dh, p.crow, r0, L, H, c0, fin, wm * 64, wn * (HS / 2), lane,
                                             grad_factor(p));
      else store_tile_f32(p.dh + r0 * H + c0, L - r0, H, H - c0, fin, wm * 64, wn * (HS / 2), lane, grad_factor(p));
    } else {
      if (reordered)
        store_rows_perm<C::MB, C::NB, false>(p.dh, p.crow, r0, L, H, c0, dacc, wm * 64, wn * (HS / 2), lane,
                                             grad_factor(p));
      else store_tile_f32(p.dh + r0 * H + c0, L - r0, H, H - c0, dacc, wm * 64, wn * (HS / 2), lane, grad_factor(p));
    }
  }
}

// ---------------------------------------------------------------- dW pass
// Group = 256 vocabulary rows.  Round k: member j recomputes the logit tiles
// of tokens [((k*R + e)*s + j)*256, +256), e < R = round_tiles(HS), against the
// group's vocabulary rows (A = h, B = W: tokens on M, vocabulary on N), forms
// G'^T[v][token] and stores each as two K-tiles (2(e*s + j), +1) of the
// round's slot [256 v][K].  Then
//   dW[v rows][c0 .. c0+HS] += slot[256][K] * h[round's tokens][c0 .. c0+HS],
// h's rows read MN-major (no copy), and the slice is stored times g/N.
template <int HS>
__global__ __launch_bounds__(kBwdThreads) void k_bwd_dW(BwdArgs p) {
  using P = typename BwdCfg<HS>::PA;
  using PAG = typename BwdCfg<HS>::PAG;
  using C = typename BwdCfg<HS>::CH;
  constexpr bool kPark = BwdCfg<HS>::kPark;
  __shared__ __attribute__((aligned(16))) char lds[BwdCfg<HS>::kLds];
  __shared__ float row_lse2[256], row_keep[256];  // lse * log2(e); 1 for rows that take a gradient, else 0
  __shared__ int row_lab[256];  // label - v0 of the group's vocabulary block, or -1
  __shared__ int s_flag;

  const int s = p.group_size;
  const int q = p.xcd_members > 0 ? xcd_tiled(blockIdx.x, gridDim.x, s, p.xcd_members) : xcd_major(blockIdx.x, gridDim.x);
  const int g = q / s, j = q % s;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t H = p.H, V = p.V, L_all = p.L;
  const int64_t c0 = (int64_t)j * HS;
  const rsrc_t park = make_rsrc(p.park + (int64_t)blockIdx.x * (kParkPerWG / 4), kPark ? kParkPerWG : 0);  // this workgroup's parking area
  constexpr int R = round_tiles(HS);
  const int64_t slot_elems = (int64_t)R * s * 256 * 256;
  // the rows swept: the compacted labelled rows when hdr->compact, else all
  const bool compact = p.hdr->compact != 0;
  const int64_t L = compact ? (int64_t)p.hdr->n_compact : L_all;
  // h rows of the swept positions: through the selection itself, or (when
  // 32-bit offsets cannot reach all of h) from the gathered copy
  const bool by_index = compact && !p.gather_copy;  // (never with 128-wide slices: the host sees to that)
  const u16* const hrows = compact && p.gather_copy ? p.ch : p.h;
  const int64_t* const labels = compact ? p.clab : p.labels;
  const float* const lse = compact ? p.clse : p.lse;
  const int rt256 = (int)((L + 255) / 256);
  const int rt128 = (int)((L + 127) / 128);
  const int rounds = (rt256 + R * s - 1) / (R * s);
  const int nvb = (int)((V + 255) / 256);
  unsigned epoch = 0;

  // Blocks g, g + n_groups, ... in lockstep with the other groups (member j of
  // every group reads the same token block in the same round).  The blocks
  // left over after the last whole wave are shared by all groups instead of
  // keeping a few busy while the rest idle: n_groups / tail_blocks groups
  // sweep consecutive round ranges of each, write partial slices, and
  // k_dw_tail adds them up in a fixed order.
  const int full_waves = nvb / p.n_groups;
  const int tail_blocks = nvb - full_waves * p.n_groups;
  const int gpb = tail_blocks > 0 ? p.n_groups / tail_blocks : 1;  // groups per leftover block
  const int nwork = full_waves + ((tail_blocks > 0 && g < gpb * tail_blocks) ? 1 : 0);
  for (int w = 0; w < nwork; ++w) {
    const bool tail = w == full_waves;
    const int vb = tail ? full_waves * p.n_groups + g / gpb : g + w * p.n_groups;
    const int k_begin = tail ? (g % gpb) * rounds / gpb : 0;
    const int k_end = tail ? (g % gpb + 1) * rounds / gpb : rounds;
    const bool to_part = tail && gpb > 1;  // a partial slice, summed by k_dw_tail
    const int64_t v0 = (int64_t)vb * 256;
    const Operand ow = linear_operand(p.W + v0 * H, (uint64_t)(V - v0) * H * 2, (uint32_t)(H * 2));
    f32x16 dacc[C::MB][C::NB];
    if constexpr (!kPark) zero_acc(dacc);
    for (int k = k_begin; k < k_end; ++k, ++epoch) {
      u16* slot = p.xbuf + ((int64_t)g * 2 + (epoch & 1)) * slot_elems;
      const rsrc_t rslot = make_rsrc(slot, (uint64_t)slot_elems * 2);
      for (int e = 0; e < R; ++e) {
        const int rt = (k * R + e) * s + j;
        if (rt < rt256) {
          const int64_t r0 = (int64_t)rt * 256;
          const int64_t rend = min(r0 + 256, L);
          if (threadIdx.x < 256) {
            const int64_t t = r0 + threadIdx.x;
            const int64_t y = t < rend ? labels[t] : p.ignore_index;
            const bool valid = t < rend && y != p.ignore_index && y >= 0 && y < V;
            row_lab[threadIdx.x] = (valid && y >= v0 && y < v0 + 256) ? (int)(y - v0) : -1;
            row_keep[threadIdx.x] = valid ? 1.f : 0.f;
            row_lse2[threadIdx.x] = t < rend ? lse[t] * kLog2e : INFINITY;
          }
          f32x16 z[P::MB][P::NB];
          zero_acc(z);
          // (the GEMM's first barrier orders the row_* writes before their use)
          const Operand oh = by_index ? gathered_operand(p.h, (uint64_t)L_all * H * 2, (uint32_t)(H * 2), p.crow + r0,
                                                         (int)(rend - r0))
                                      : gathered_operand(hrows + r0 * H, (uint64_t)(rend - r0) * H * 2,
                                                         (uint32_t)(H * 2), nullptr, (int)(rend - r0));
          if (by_index) PAG::run(oh, ow, (int)H, lds, z);
          else P::run(oh, ow, (int)H, lds, z);
          // G'^T[v][token]: lane = v (column), 4 consecutive tokens per store.
          // Token data is read once per 4-token group and reused for the
          // lane's 4 vocabulary columns; columns past V get a zero factor.
          const int vlim = (int)min<int64_t>(V - v0, 256);
          raw_barrier();  // every wave is done with the GEMM's last LDS stage
          float vmask[4];
  #pragma unroll
          for (int nb = 0; nb < 4; ++nb) vmask[nb] = (wn * 128 + nb * 32 + (lane & 31) < vlim) ? 1.f : 0.f;
  #pragma unroll
          for (int mb = 0; mb < 2; ++mb)
  #pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const int tl0 = wm * 64 + mb * 32 + acc_row(qq * 4, lane);
              float tlse[4], tkeep[4];
              int tlab[4];
  #pragma unroll
              for (int e = 0; e < 4; ++e) {
                tlse[e] = row_lse2[tl0 + e];
                tkeep[e] = row_keep[tl0 + e];
                tlab[e] = row_lab[tl0 + e];
              }
  #pragma unroll
              for (int nb = 0; nb < 4; ++nb) {
                const int vl = wn * 128 + nb * 32 + (lane & 31);
                float gv[4];
  #pragma unroll
                for (int e = 0; e < 4; ++e) {
                  float pr = exp2_fast(__builtin_fmaf(z[mb][nb][qq * 4 + e], kLog2e, -tlse[e]));
                  pr = (vl == tlab[e]) ? pr - 1.f : pr;
                  gv[e] = pr * (tkeep[e] * vmask[nb]);
                }
                gstage_put(lds, vl, tl0, pack_bf16x4(gv[0], gv[1], gv[2], gv[3]));
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          __syncthreads();
          gstage_flush(lds, rslot, e * s + j);
        }
      }
      if constexpr (kPark) {
        if (k == k_begin) zero_acc(dacc);
        else unpark_acc(dacc, park, wave, lane);
      }
      if (!group_arrive_wait(p.sync + g * kSyncStride, (unsigned)s * (epoch + 1), p.spin_limit, p.hdr, &s_flag))
        return;
      const int ntl = min(2 * R * s, rt128 - k * 2 * R * s);
      const int64_t rbase = (int64_t)k * R * s * 256;
      // B: the round's h rows (K = tokens), columns c0 .. c0+HS, read MN-major
      // (rows past the swept ones read as zero)
      const int64_t krows = min<int64_t>((int64_t)ntl * 128, L - rbase);
      const Operand ohk =
          by_index ? gathered_operand(p.h, (uint64_t)L_all * H * 2, (uint32_t)(H * 2), p.crow + rbase, (int)krows,
                                      (uint32_t)(c0 * 2))
                   : gathered_operand(hrows + rbase * H, (uint64_t)krows * H * 2, (uint32_t)(H * 2), nullptr,
                                      (int)krows, (uint32_t)(c0 * 2));
      C::run(tiled_operand(slot, (uint64_t)slot_elems * 2, 256, 256 * 128 * 2), ohk, ntl * 128, lds, dacc);
      if constexpr (kPark) park_acc(dacc, park, wave, lane);  // also after the last round: dacc is dead at the back edge
    }
    // (an empty round range, e.g. no labelled rows at all, leaves 0)
    f32x16 fin[C::MB][C::NB];
    if constexpr (kPark) {
      if (k_end > k_begin) unpark_acc(fin, park, wave, lane);
      else zero_acc(fin);
    } else {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) fin[mb][nb] = dacc[mb][nb];
    }
    // dW = g/N * (G'^T h): the factor in fp32, as in the dh pass.  With
    // 128-wide slices (accumulators held in registers across the rounds) a
    // product here makes the compiler spill the accumulators in every round,
    // so that variant stores G'^T h and k_dw_scale applies the factor after
    // the pass.
    const float f = HS == 256 ? grad_factor(p) : 1.f;
    if (to_part)
      store_tile_f32(p.dw_part + ((int64_t)g * s + j) * 256 * HS, 256, HS, HS, fin, wm * 64, wn * (HS / 2), lane,
                     f);
    else
      store_tile_f32(p.dW + v0 * H + c0, V - v0, H, H - c0, fin, wm * 64, wn * (HS / 2), lane, f);
  }
}

// ----------------------------------------------------- fused training forward
// Maximum and sum of one value per group member (member i's value at byte
// offset base + i * 1024 + voff of the statistics exchange).  Eight loads are
// issued before any is used, so a round waits for s / 8 device-coherent
// round trips instead of s.  The sum adds the members in index order.
__device__ __forceinline__ float group_max(rsrc_t rs, int s, uint32_t voff, uint32_t base) {
  float mx = -INFINITY;
  for (int i0 = 0; i0 < s; i0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = i0 + u < s ? load_sc1_b32(rs, voff, base + (uint32_t)(i0 + u) * 1024u) : -INFINITY;
#pragma unroll
    for (int u = 0; u < 8; ++u) mx = fmaxf(mx, v[u]);
  }
  return mx;
}
__device__ __forceinline__ float group_sum(rsrc_t rs, int s, uint32_t voff, uint32_t base) {
  float sum = 0.f;
  for (int i0 = 0; i0 < s; i0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = i0 + u < s ? load_sc1_b32(rs, voff, base + (uint32_t)(i0 + u) * 1024u) : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += v[u];
  }
  return sum;
}

// Copies the staged tile like gstage_flush, scaling row r by fac[r] on the way.
__device__ __forceinline__ void gstage_flush_scaled(const char* lds, const float* fac, rsrc_t rslot, int j) {
  const int t = threadIdx.x;
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int idx = i * 512 + t;
    const int row = idx >> 5, c = idx & 31;
    const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
        (const __attribute__((address_space(3))) char*)lds + row * 512 + ((c ^ (row & 31)) << 4));
    const bf16x8 x = __builtin_bit_cast(bf16x8, v);
    const float f = fac[row];
    const f32x4 lo = {(float)x[0] * f, (float)x[1] * f, (float)x[2] * f, (float)x[3] * f};
    const f32x4 hi = {(float)x[4] * f, (float)x[5] * f, (float)x[6] * f, (float)x[7] * f};
    const bf16x4 blo = __builtin_convertvector(lo, bf16x4), bhi = __builtin_convertvector(hi, bf16x4);
    const u32x4 w = {__builtin_bit_cast(u32x2, blo)[0], __builtin_bit_cast(u32x2, blo)[1],
                     __builtin_bit_cast(u32x2, bhi)[0], __builtin_bit_cast(u32x2, bhi)[1]};
    const uint32_t voff = (uint32_t)(((c >> 4) * 256 * 128 + row * 128 + (c & 15) * 8) * 2);
    store_sc1_b128(rslot, voff + (uint32_t)j * 2u * 256u * 128u * 2u, w);
  }
}

// Slack of the training forward's reference: a tile's P is taken against the
// running maximum while its own maximum exceeds that by at most this much
// (P <= e^16, well inside bf16 and fp32 range), else against its own maximum.
constexpr float kRefSlack = 16.f;

// Multiplies the rows of the member's tile at slot position j (two K-tiles
// written by gstage_flush from this same thread's chunks, long completed) by
// fac[row], skipping the rows whose factor is exactly 1.
__device__ __forceinline__ void gslot_rescale(rsrc_t rslot, const float* fac, int j) {
  const int t = threadIdx.x;
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int idx = i * 512 + t;
    const int row = idx >> 5, c = idx & 31;
    const float f = fac[row];
    if (f != 1.f) {
      const uint32_t voff = (uint32_t)(((c >> 4) * 256 * 128 + row * 128 + (c & 15) * 8) * 2) +
                            (uint32_t)j * 2u * 256u * 128u * 2u;
      const bf16x8 x = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rslot, voff, 0, kAuxSc1));
      const f32x4 lo = {(float)x[0] * f, (float)x[1] * f, (float)x[2] * f, (float)x[3] * f};
      const f32x4 hi = {(float)x[4] * f, (float)x[5] * f, (float)x[6] * f, (float)x[7] * f};
      const bf16x4 blo = __builtin_convertvector(lo, bf16x4), bhi = __builtin_convertvector(hi, bf16x4);
      const u32x4 w = {__builtin_bit_cast(u32x2, blo)[0], __builtin_bit_cast(u32x2, blo)[1],
                       __builtin_bit_cast(u32x2, bhi)[0], __builtin_bit_cast(u32x2, bhi)[1]};
      store_sc1_b128(rslot, voff, w);
    }
  }
}

// One vocabulary sweep per 256-row block yields both the log-sum-exp of every
// row and O = sum_v softmax(z)_v W_v, so that dh = g/N * (O - W_y) needs no
// second sweep (the gradient of the mean NLL, the definition on the pages
// above).  The structure is that of k_bwd_dh, with the softmax reference
// taken on the fly as in an online softmax.  In round k each member computes
// its logit tile, the tile's per-token maximum m_j, P_j = exp(z - m_j)
// (staged in LDS as bf16) and the lane's sums of P_j; after a group barrier
// all members read the s maxima and agree on the running maximum M_k of each
// token; each member writes its P_j scaled by exp(m_j - M_k) to the exchange
// and rescales its row sums; the contraction rescales its O slice by
// exp(M_{k-1} - M_k) and adds the round's P W.  After the last round the row
// sums are exchanged once more, O is divided by them and stored, and
// (max, sum) go out as a one-segment log-sum-exp partial of every row.
template <int HS>
__global__ __launch_bounds__(kBwdThreads) void k_fwd_dh(BwdArgs p) {
  using P = typename BwdCfg<HS>::P;
  using PG = typename BwdCfg<HS>::PG;
  using C = typename BwdCfg<HS>::C;
  constexpr bool kPark = BwdCfg<HS>::kPark;
  constexpr int R = round_tiles(HS);
  __shared__ __attribute__((aligned(16))) char lds[BwdCfg<HS>::kLds];
  __shared__ float red[4][256];     // per-wave partial (max or sum) of each token
  __shared__ float row_m[256];      // the group's running maximum M of each token (the reference)
  __shared__ float row_a[256];      // exp(M_old - M_new) (last: 1 / sum)
  __shared__ float row_s[256];      // sum of exp(z - M) over the tiles so far (this member's)
  __shared__ float row_mx[256];     // this member's maximum over the round's tiles
  __shared__ float row_r[R][256];   // reference r_u of tile u's P = exp(z - r_u)
  __shared__ float row_ps[R][256];  // sum of tile u's P per token
  __shared__ float row_f[R][256];   // exp(r_u - M_new): tile u's factor into the new reference
  __shared__ int s_flag;

  const int s = p.group_size;
  const int q = p.xcd_members > 0 ? xcd_tiled(blockIdx.x, gridDim.x, s, p.xcd_members) : member_spread(blockIdx.x);
  const int g = q / s, j = q % s;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int t = threadIdx.x;  // token of the per-token steps (t < 256)
  const int64_t H = p.H, V = p.V, L = p.L;
  const int64_t c0 = (int64_t)j * HS;
  const rsrc_t park = make_rsrc(p.park + (int64_t)blockIdx.x * (kParkPerWG / 4), kPark ? kParkPerWG : 0);
  const int64_t slot_elems = (int64_t)R * s * 256 * 256;
  // this group's statistics exchange: [2][s][256] round maxima, [s][256] sums
  const rsrc_t rstat = make_rsrc(p.xstat + (int64_t)g * 3 * s * 256, (uint64_t)3 * s * 256 * 4);
  const int vt256 = (int)((V + 255) / 256);
  const int vt128 = (int)((V + 127) / 128);
  const int rounds = (vt256 + R * s - 1) / (R * s);
  const int nrb = (int)((L + 255) / 256);
  // rows in the labelled-first order when the host-side plan found it worth
  // a block (every output of this kernel is then indexed by position)
  const bool reordered = p.hdr->fcompact != 0;
  const int64_t n_lab = reordered ? (int64_t)p.hdr->f_n : L;
  const bool by_index = reordered && !p.gather_copy;  // as in the dh pass
  const u16* const hrows = reordered && p.gather_copy ? p.hp : p.h;
  unsigned epoch = 0, nbar = 0;

  for (int rb = g; rb < nrb; rb += p.n_groups) {
    const int64_t r0 = (int64_t)rb * 256;
    const int64_t rend = min(r0 + 256, L);
    // a block with no labelled row needs lse only: no P exchange, no O
    const bool o_block = r0 < n_lab;
    const Operand oh = by_index ? gathered_operand(p.h, (uint64_t)L * H * 2, (uint32_t)(H * 2), p.fperm + r0,
                                                   (int)(rend - r0))
                                : gathered_operand(hrows + r0 * H, (uint64_t)(rend - r0) * H * 2, (uint32_t)(H * 2),
                                                   nullptr, (int)(rend - r0));
    if (t < 256) {  // ordered by the barriers below
      row_m[t] = -INFINITY;
      row_s[t] = 0.f;
    }
    f32x16 dacc[C::MB][C::NB];
    if constexpr (!kPark) zero_acc(dacc);
    for (int k = 0; k < rounds; ++k, ++epoch) {
      u16* slot = p.xbuf + ((int64_t)g * 2 + (epoch & 1)) * slot_elems;
      const rsrc_t rslot = make_rsrc(slot, (uint64_t)slot_elems * 2);
      const uint32_t xm = (uint32_t)((k & 1) * s * 256 * 4);  // this round's maxima slot (bytes)
      if (t < 256) row_mx[t] = -INFINITY;
      // The member's tiles u = 0 .. R-1 of the round.  Tile u's P is taken
      // against r_u = the running reference M (the group's maximum before
      // this round) when the tile's row maximum m_u stays within kRefSlack of
      // it, else against m_u: P <= exp(kRefSlack) either way.  Every tile but
      // the last goes to the slot at once (the next tile's GEMM needs the
      // LDS); the last stays staged.  Once the group's new maximum M' is
      // known each tile is brought to it with the factor exp(r_u - M'), which
      // is exactly 1 for the rows whose reference did not move.
#pragma unroll 1
      for (int u = 0; u < R; ++u) {
        const int vt = (k * R + u) * s + j;
        if (vt >= vt256) {
          if (t < 256) {
            row_r[u][t] = -INFINITY;
            row_ps[u][t] = 0.f;
          }
          continue;
        }
        const int v0 = vt * 256;
        const int vlim = min((int)(V - v0), 256);
        f32x16 z[P::MB][P::NB];
        zero_acc(z);
        const Operand ow = linear_operand(p.W + (int64_t)v0 * H, (uint64_t)(V - v0) * H * 2, (uint32_t)(H * 2));
        if (by_index) PG::run(ow, oh, (int)H, lds, z);
        else P::run(ow, oh, (int)H, lds, z);
        // per-token maximum of the tile: the lane's 32 values, the other lane
        // half, then the 4 waves that share the token
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          float mx = -INFINITY;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const int vl0 = wm * 64 + mb * 32 + acc_row(qq * 4, lane);
#pragma unroll
              for (int e = 0; e < 4; ++e) mx = (vl0 + e < vlim) ? fmaxf(mx, z[mb][nb][qq * 4 + e]) : mx;
            }
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          if (lane < 32) red[wm][wn * 128 + nb * 32 + lane] = mx;
        }
        __syncthreads();  // also: every wave is done with the GEMM's LDS stages
        if (t < 256) {
          const float m = fmaxf(fmaxf(red[0][t], red[1][t]), fmaxf(red[2][t], red[3][t]));
          const float ref = row_m[t];
          row_r[u][t] = m <= ref + kRefSlack ? ref : m;
          row_mx[t] = fmaxf(row_mx[t], m);
        }
        __syncthreads();
        // P_u = exp(z - r_u), staged in LDS as [token][v]; columns past V are 0
        float psum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const float ml = row_r[u][wn * 128 + nb * 32 + (lane & 31)] * kLog2e;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              float gv[4];
              const int vl0 = wm * 64 + mb * 32 + acc_row(qq * 4, lane);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float pr = exp2_fast(__builtin_fmaf(z[mb][nb][qq * 4 + e], kLog2e, -ml));
                gv[e] = (vl0 + e < vlim) ? pr : 0.f;
                psum[nb] += gv[e];
              }
              gstage_put(lds, wn * 128 + nb * 32 + (lane & 31), vl0, pack_bf16x4(gv[0], gv[1], gv[2], gv[3]));
            }
          __builtin_amdgcn_sched_barrier(0);
        }
        // the tile's sum per token: lane halves, then the 4 waves
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const float v = psum[nb] + __shfl_xor(psum[nb], 32);
          if (lane < 32) red[wm][wn * 128 + nb * 32 + lane] = v;
        }
        __syncthreads();  // also: the staged tile is complete
        if (t < 256) row_ps[u][t] = (red[0][t] + red[1][t]) + (red[2][t] + red[3][t]);
        if (u < R - 1 && o_block) gstage_flush(lds, rslot, u * s + j);
      }
      if (t < 256) store_sc1_b32(rstat, (uint32_t)t * 4u, xm + (uint32_t)j * 1024u, row_mx[t]);
      if (!group_arrive_wait(p.sync + g * kSyncStride, (unsigned)s * (++nbar), p.spin_limit, p.hdr, &s_flag)) return;
      if (t < 256) {
        const float old = row_m[t];
        const float mx = fmaxf(old, group_max(rstat, s, (uint32_t)t * 4u, xm));
        const float a = (old == -INFINITY) ? 0.f : (old == mx ? 1.f : exp2_fast((old - mx) * kLog2e));
        float sum = row_s[t] * a;
#pragma unroll
        for (int u = 0; u < R; ++u) {
          const float r = row_r[u][t];
          const float f = (r == -INFINITY) ? 0.f : (r == mx ? 1.f : exp2_fast((r - mx) * kLog2e));
          row_f[u][t] = f;
          sum = __builtin_fmaf(row_ps[u][t], f, sum);
        }
        row_a[t] = a;
        row_s[t] = sum;
        row_m[t] = mx;
      }
      __syncthreads();
      if (!o_block) continue;  // (uniform over the group: every member takes the same block)
      // the last tile from LDS with its factor; the earlier ones in the slot,
      // only the rows whose factor is not 1
      if ((k * R + R - 1) * s + j < vt256) gstage_flush_scaled(lds, row_f[R - 1], rslot, (R - 1) * s + j);
#pragma unroll 1
      for (int u = 0; u < R - 1; ++u)
        if ((k * R + u) * s + j < vt256) gslot_rescale(rslot, row_f[u], u * s + j);
      if constexpr (kPark) {
        if (k == 0) zero_acc(dacc);
        else unpark_acc(dacc, park, wave, lane);
      }
      if (k > 0) {
        // O rows (tokens) follow the new maximum
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int reg = 0; reg < 16; ++reg) {
            const float a = row_a[wm * 64 + mb * 32 + acc_row(reg, lane)];
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) dacc[mb][nb][reg] *= a;
          }
      }
      if (!group_arrive_wait(p.sync + g * kSyncStride, (unsigned)s * (++nbar), p.spin_limit, p.hdr, &s_flag)) return;
      const int ntl = min(2 * R * s, vt128 - k * 2 * R * s);
      const int64_t vbase = (int64_t)k * R * s * 256;
      const int64_t krows = min<int64_t>((int64_t)ntl * 128, V - vbase);
      C::run(tiled_operand(slot, (uint64_t)slot_elems * 2, 256, 256 * 128 * 2),
             linear_operand(p.W + vbase * H, (uint64_t)krows * H * 2, (uint32_t)(H * 2), (uint32_t)(c0 * 2)),
             ntl * 128, lds, dacc);
      if constexpr (kPark) park_acc(dacc, park, wave, lane);  // also after the last round: dacc is dead at the back edge
    }
    // row sums of the s members
    if (t < 256) store_sc1_b32(rstat, (uint32_t)t * 4u, (uint32_t)(2 * s * 1024 + j * 1024), row_s[t]);
    if (!group_arrive_wait(p.sync + g * kSyncStride, (unsigned)s * (++nbar), p.spin_limit, p.hdr, &s_flag)) return;
    if (t < 256) {
      const float sum = group_sum(rstat, s, (uint32_t)t * 4u, (uint32_t)(2 * s * 1024));
      row_a[t] = 1.f / sum;
      if (j == 0 && r0 + t < L) {
        p.part_m[r0 + t] = row_m[t];
        p.part_s[r0 + t] = sum;
      }
    }
    __syncthreads();
    if (!o_block) continue;
    f32x16 fin[C::MB][C::NB];
    if constexpr (kPark) unpark_acc(fin, park, wave, lane);
    else {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) fin[mb][nb] = dacc[mb][nb];
    }
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int reg = 0; reg < 16; ++reg) {
        const float a = row_a[wm * 64 + mb * 32 + acc_row(reg, lane)];
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) fin[mb][nb][reg] *= a;
      }
    // O rows go to their row of the caller's buffer (through the order, if any)
    if (reordered) store_rows_perm<C::MB, C::NB, false>(p.O, p.fperm, r0, L, H, c0, fin, wm * 64, wn * (HS / 2), lane);
    else store_tile_f32(p.O + r0 * H + c0, L - r0, H, H - c0, fin, wm * 64, wn * (HS / 2), lane);
  }
}

// dh = g/N * (O - W_y) for rows with a label, 0 for the others, in place in
// the buffer that holds O (row r of O is row r of dh: each element is read,
// then overwritten by the same thread); NaN (and the state flag) if that
// buffer does not hold a complete training forward's O (none ran, another
// forward ran since, one of its group waits gave up, or the forward wrote O
// into another buffer).
__global__ __launch_bounds__(256) void k_dh_finish(BwdArgs p) {
  const int64_t r = blockIdx.x;
  const int64_t H = p.H;
  const int64_t y = p.labels[r];
  const bool valid = y != p.ignore_index && y >= 0 && y < p.V;
  const bool ok = p.hdr->saved == kSavedTag && p.hdr->o_addr == (unsigned long long)(uintptr_t)p.dh;
  const int n = p.hdr->n_valid;
  const float scale = *p.grad_loss / (float)(n > 0 ? n : 1);
  if (!ok && r == 0 && threadIdx.x == 0)
    __hip_atomic_fetch_or(&p.hdr->status, kStatusState, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const u16* w = p.W + (valid ? y : 0) * H;
  float4* d = reinterpret_cast<float4*>(p.dh + r * H);
  for (int64_t c = threadIdx.x; c < H / 4; c += 256) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!ok) {
      v = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
    } else if (valid) {
      const float4 ov = d[c];
      const bf16x4 wv = *reinterpret_cast<const bf16x4*>(w + c * 4);
      v = make_float4(scale * (ov.x - (float)wv[0]), scale * (ov.y - (float)wv[1]), scale * (ov.z - (float)wv[2]),
                      scale * (ov.w - (float)wv[3]));
    }
    d[c] = v;
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_compact(const BwdArgs& a, int* cnt, int64_t ch_rows, hipStream_t st) {
  const int nchunks = (int)((a.L + 1023) / 1024);
  hipLaunchKernelGGL(k_count_chunks, dim3((unsigned)nchunks), dim3(256), 0, st, a.labels, a.L, a.V, a.ignore_index, cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_compact_rows, dim3((unsigned)nchunks), dim3(1024), 0, st, a.labels, a.lse, a.L, a.V,
                     a.ignore_index, ch_rows, (const int*)cnt, nchunks, a.hdr, a.crow, a.clab, a.clse);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!a.gather_copy) return hipSuccess;  // the dW pass reads h through crow
  hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)a.L), dim3(256), 0, st, a.h, a.H, (const WsHeader*)a.hdr,
                     (const int*)a.crow, a.ch);
  return hipGetLastError();
}

hipError_t launch_permute(const BwdArgs& a, int* cnt, int* flags, int* perm, int* inv, hipStream_t st) {
  const int nchunks = (int)((a.L + 1023) / 1024);
  hipLaunchKernelGGL(k_count_chunks, dim3((unsigned)nchunks), dim3(256), 0, st, a.labels, a.L, a.V, a.ignore_index, cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_permute_rows, dim3((unsigned)nchunks), dim3(1024), 0, st, a.labels, a.L, a.V, a.ignore_index,
                     (const int*)cnt, nchunks, flags, perm, inv);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!a.gather_copy) return hipSuccess;  // the pass reads h through perm
  hipLaunchKernelGGL(k_gather_perm, dim3((unsigned)a.L), dim3(256), 0, st, a.h, a.H, (const int*)flags,
                     (const int*)perm, a.hp);
  return hipGetLastError();
}


hipError_t launch_dw_tail(const BwdArgs& a, int hs, hipStream_t st) {
  const int nvb = (int)((a.V + 255) / 256);
  const int full_waves = nvb / a.n_groups;
  const int tail_blocks = nvb - full_waves * a.n_groups;
  if (tail_blocks == 0) return hipSuccess;
  const int gpb = a.n_groups / tail_blocks;
  if (gpb < 2) return hipSuccess;  // each leftover block went whole to one group
  hipLaunchKernelGGL(k_dw_tail, dim3((unsigned)(tail_blocks * a.group_size)), dim3(256), 0, st, (const float*)a.dw_part,
                     a.dW, a.V, a.H, hs, a.group_size, gpb, (int64_t)full_waves * a.n_groups * 256);
  return hipGetLastError();
}

hipError_t launch_dw_scale(const BwdArgs& a, int hs, hipStream_t st) {
  if (hs == 256) return hipSuccess;  // the 256-wide pass applied the factor itself
  const int64_t n4 = a.V * a.H / 4;  // H is a multiple of 128
  const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 8192);
  hipLaunchKernelGGL(k_dw_scale, dim3((unsigned)blocks), dim3(256), 0, st, a.dW, n4, a.grad_loss, a.hdr);
  return hipGetLastError();
}

hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t st) {
  hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

const void* bwd_kernel(int pass, int hs) {
  if (hs == 256) {
    if (pass == kPassDh) return reinterpret_cast<const void*>(&k_bwd_dh<256>);
    if (pass == kPassFwdDh) return reinterpret_cast<const void*>(&k_fwd_dh<256>);
    return reinterpret_cast<const void*>(&k_bwd_dW<256>);
  }
  if (pass == kPassDh) return reinterpret_cast<const void*>(&k_bwd_dh<128>);
  if (pass == kPassDw) return reinterpret_cast<const void*>(&k_bwd_dW<128>);
  return reinterpret_cast<const void*>(&k_fwd_dh<128>);
}

hipError_t bwd_resident_wgs(int pass, int hs, int* wgs) {
  int dev = 0, cus = 0, per = 0, coop = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
  if (e != hipSuccess) return e;
  if (!coop) return hipErrorNotSupported;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, bwd_kernel(pass, hs), kBwdThreads, 0);
  if (e != hipSuccess) return e;
  *wgs = cus * per;
  return hipSuccess;
}

hipError_t launch_bwd_group(int pass, const BwdArgs& a, int hs, int n_wgs, hipStream_t st) {
  BwdArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchCooperativeKernel(bwd_kernel(pass, hs), dim3((unsigned)n_wgs), dim3(kBwdThreads), args, 0, st);
}

hipError_t launch_dh_finish(const BwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_dh_finish, dim3((unsigned)a.L), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lmce
