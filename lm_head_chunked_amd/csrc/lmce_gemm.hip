// General bf16 GEMM on the library's tile engine (gfx950), with fused
// epilogues.  Used by the row-chunked paths that materialise one chunk of
// rows at a time: the pages' own chunked loss (TRL docs "Training Beyond 1M
// Tokens", section "The massive logits matrix: chunk it": each chunk's
// logits are formed, its loss taken and the pieces summed) and the sequence-
// tiled MLP (same page, section "One GPU is not enough: split the sequence
// across many": down_proj(act_fn(gate_proj(x)) * up_proj(x)) with its wide
// intermediates built for a block of rows at a time).
//
// One workgroup of 8 waves computes one 256 x 256 output tile with
// v_mfma_f32_32x32x16_bf16 through TileGemm (LDS-DMA stages, interleaved
// schedule); grid.x walks the tiles in patches that keep the 32 workgroups
// of one XCD on neighbouring tiles, so they share their operand rows in that
// XCD's L2; grid.y splits K.

#include "lmce_device.h"
#include "lmce_internal.h"

namespace lmce {

constexpr int kGemmThreads = 512;
constexpr uint32_t kDrop = 0xfffffff0u;  // a buffer offset past every resource end: the access is dropped

// Tile (tm, tn) of workgroup b.  patch_m > 0: the tiles are ordered
// patch-major (patches of patch_m x (32 / patch_m) tiles, row-major over the
// patches and within each patch; a partial patch at the grid's edge keeps
// only its tiles inside the grid), and XCD x (workgroups are dispatched to
// the 8 XCDs round-robin, so b % 8 is the XCD) takes the x-th of eight equal
// consecutive shares of that order.  The 32 workgroups an XCD runs at once
// then cover a compact block of tiles that share operand rows in its L2, and
// every XCD gets the same number of tiles.  patch_m == 0: row-major order
// (for grids with fewer tiles than CUs).  False for the grid's padding.
__device__ __forceinline__ bool gemm_tile(int b, const GemmArgs& p, int& tm, int& tn) {
  const int mt = (int)((p.M + 255) / 256), nt = (int)((p.N + 255) / 256);
  if (p.patch_m == 0) {
    tm = b / nt;
    tn = b % nt;
    return tm < mt;
  }
  const int total = mt * nt;
  const int share = (total + 7) / 8;
  const int t = (b & 7) * share + (b >> 3);  // position in the patch-major order
  if ((b >> 3) >= share || t >= total) return false;
  const int pm = p.patch_m, pn = 32 / pm;
  // patches of full height come first in each band of pm tile rows; the
  // band's width is nt, its last patch may be narrower
  const int band = t / (pm * nt);             // band of pm tile rows
  const int rows = min(pm, mt - band * pm);   // tile rows in this band
  const int in_band = t - band * pm * nt;
  const int patch = in_band / (rows * pn);    // full-width patches of this band
  const int pw = min(pn, nt - patch * pn);    // width of this patch
  const int w = in_band - patch * rows * pn;  // position in the patch
  tm = band * pm + w / pw;
  tn = patch * pn + w % pw;
  return true;
}

// Operand of the tile whose first row is r0, for the K piece starting at k0.
template <int FORM>
__device__ __forceinline__ Operand gemm_operand(const void* base, uint64_t bytes, uint32_t ld, int64_t r0, int64_t k0) {
  const char* b = static_cast<const char*>(base);
  if constexpr (FORM == 0) {
    const uint64_t off = (uint64_t)r0 * ld;
    return linear_operand(b + off, bytes > off ? bytes - off : 0, ld, (uint32_t)(k0 * 2));
  } else {
    const uint64_t off = (uint64_t)k0 * ld;
    return linear_operand(b + off, bytes > off ? bytes - off : 0, ld, (uint32_t)(r0 * 2));
  }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __builtin_bit_cast(float, (uint32_t)v << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);  // round to nearest even
}

__device__ __forceinline__ float load_f32(rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
}
__device__ __forceinline__ void store_f32(rsrc_t rs, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, off, 0, 0);
}
__device__ __forceinline__ float load_bf16(rsrc_t rs, uint32_t off) {
  return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0));
}
__device__ __forceinline__ void store_bf16(rsrc_t rs, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), rs, off, 0, 0);
}
__device__ __forceinline__ void store_b64(rsrc_t rs, uint32_t off, uint64_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rs, off, 0, 0);
}
// 16-byte accesses; the scalar offset stays the constant 0 (see store_sc1_b128)
__device__ __forceinline__ void store_b128(rsrc_t rs, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 0);
}
__device__ __forceinline__ u32x4 load_b128(rsrc_t rs, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
}

typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef short v4i16 __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// alpha * registers base .. base + 7 of an accumulator block as 8 bf16 (round to nearest even)
__device__ __forceinline__ u32x4 pack_bf16x8(const f32x16& v, int base, float alpha) {
  const f32x8 t = {alpha * v[base + 0], alpha * v[base + 1], alpha * v[base + 2], alpha * v[base + 3],
                   alpha * v[base + 4], alpha * v[base + 5], alpha * v[base + 6], alpha * v[base + 7]};
  return __builtin_bit_cast(u32x4, __builtin_convertvector(t, bf16x8));
}

// Register `reg` (0 .. 15) of a fragment-order block held as two 16-byte words.
__device__ __forceinline__ float frag_bf16(const u32x4 (&w)[2], int reg) {
  const uint32_t x = w[reg >> 3][(reg & 7) >> 1];
  return __builtin_bit_cast(float, (reg & 1) ? (x & 0xffff0000u) : (x << 16));
}

// Accumulator element (mb, nb, reg) of lane `lane` in wave (wm, wn) sits at
// tile row wm*64 + mb*32 + acc_row(reg, lane), tile column wn*128 + nb*32 + lane%32.
// One output tile: workgroup b of the problem's grid, K piece kz, stages in lds.
template <int FA, int FB>
__device__ __forceinline__ void gemm_block(const GemmArgs& p, int b, int kz, char* lds) {
  using G = TileGemm<256, 256, 4, 2, 0, FA, FB, true>;
  int tm, tn;
  if (!gemm_tile(b, p, tm, tn)) return;  // uniform across the workgroup
  const int64_t m0 = (int64_t)tm * 256, n0 = (int64_t)tn * 256;
  const int64_t k0 = (int64_t)kz * p.kchunk;
  const Operand oa = gemm_operand<FA>(p.A, p.a_bytes, p.a_ld, m0, k0);
  const Operand ob = gemm_operand<FB>(p.B, p.b_bytes, p.b_ld, n0, k0);
  f32x16 acc[2][4];
  zero_acc(acc);
  G::run(oa, ob, (int)p.kchunk, lds, acc);

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int rl = (int)min<int64_t>(256, p.M - m0);  // rows and columns of the tile inside C
  const int cl = (int)min<int64_t>(256, p.N - n0);
  const int ldc = (int)p.ldc;
  const float alpha = p.alpha;

  if (p.epi == kEpiStoreF32 || p.epi == kEpiAccF32) {
    float* base = static_cast<float*>(p.C) + (int64_t)kz * p.c_split + m0 * p.ldc + n0;
    const rsrc_t rs = make_rsrc(base, (uint64_t)((int64_t)(rl - 1) * ldc + cl) * 4);
    const bool accum = p.epi == kEpiAccF32;
    // The accumulate loads the 16 old values of a 32x32 block before its
    // first store: a load may not pass an earlier store to a possibly equal
    // address, so interleaved load-add-store pairs would wait for one L2
    // round trip each.
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int c = wn * 128 + nb * 32 + (lane & 31);
        float old[16];
#pragma unroll
        for (int reg = 0; reg < 16; ++reg) {
          const int r = wm * 64 + mb * 32 + acc_row(reg, lane);
          old[reg] = accum ? load_f32(rs, (r < rl && c < cl) ? (uint32_t)(r * ldc + c) * 4u : kDrop) : 0.f;
        }
#pragma unroll
        for (int reg = 0; reg < 16; ++reg) {
          const int r = wm * 64 + mb * 32 + acc_row(reg, lane);
          const uint32_t off = (r < rl && c < cl) ? (uint32_t)(r * ldc + c) * 4u : kDrop;
          store_f32(rs, off, old[reg] + alpha * acc[mb][nb][reg]);
        }
      }
  } else if (p.epi == kEpiStoreFrag) {
    // each lane's 16 registers of a 32 x 32 block as 32 contiguous bytes: a
    // consumer with the same tile and lane layout reads them back whole
    const int64_t ntn = (p.N + 255) / 256;
    const rsrc_t rs = make_rsrc(static_cast<uint16_t*>(p.C) + ((int64_t)tm * ntn + tn) * 65536, 131072);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const uint32_t off = ((uint32_t)(wave * 8 + mb * 4 + nb) * 1024u + (uint32_t)lane * 16u) * 2u;
        store_b128(rs, off, pack_bf16x8(acc[mb][nb], 0, alpha));
        store_b128(rs, off + 16u, pack_bf16x8(acc[mb][nb], 8, alpha));
      }
  } else if (p.epi == kEpiSwigluFwd) {
    // tile columns 64q + j (gate) and 64q + 32 + j (up) are unit i = 32q + j
    const int64_t ni = p.N / 2;
    const int64_t i0 = n0 / 2 + wn * 64;  // first unit of this wave
    uint16_t* base = static_cast<uint16_t*>(p.C) + m0 * p.ldc;
    const rsrc_t rs = make_rsrc(base, (uint64_t)((int64_t)(rl - 1) * ldc + ni) * 2);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int reg = 0; reg < 16; ++reg) {
        const int r = wm * 64 + mb * 32 + acc_row(reg, lane);
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int64_t i = i0 + pp * 32 + (lane & 31);
          const float g = alpha * acc[mb][2 * pp][reg], u = alpha * acc[mb][2 * pp + 1][reg];
          const float silu = g / (1.f + exp2_fast(-g * kLog2e));
          store_bf16(rs, (r < rl && i < ni) ? (uint32_t)(r * ldc + i) * 2u : kDrop, silu * u);
        }
      }
  } else if (p.epi == kEpiSwigluBwd) {
    // acc = d(act) at unit i = column.  The gate and up values of unit i sit at columns
    // 64 (i / 32) + i % 32 and + 32 of the gate/up GEMM, which stored them in fragment order:
    // this lane's are in that GEMM's tile (tm, 2 tn + wn), wave 2 wm + nb / 2, blocks
    // mb * 4 + 2 (nb % 2) (gate) and + 1 (up), at the same lane and registers.
    // Outputs, row-major: d(gate/up) at C, interleaved like the gate/up columns, and
    // p = silu(g) * u at aux.  They pass through LDS one 32-unit column block nb at a time
    // (64 units of the tile): 192 columns (d(gate), d(up) of the two wave columns, then p) of
    // 256 rows in 8-byte units of four rows, unit (col, rq) at col * 64 + (rq ^ 2 (col % 16)),
    // written by the lanes as they hold them and read back row-wise with transposing reads.
    const int64_t n2 = 2 * p.N;
    const int64_t ntg = (n2 + 255) / 256;  // tiles per tile row of the gate/up GEMM
    const int64_t gtile = 2 * (int64_t)tn + wn;
    const rsrc_t rgu = make_rsrc(p.gu + ((int64_t)tm * ntg + gtile) * 65536, gtile < ntg ? 131072 : 0);
    const rsrc_t rdg = make_rsrc(static_cast<uint16_t*>(p.C) + m0 * n2, (uint64_t)rl * n2 * 2);
    const rsrc_t rpa = make_rsrc(p.aux + m0 * p.N, (uint64_t)rl * p.N * 2);
    uint64_t* st = reinterpret_cast<uint64_t*>(lds);
    auto unit = [](int col, int rq) { return col * 64 + (rq ^ (2 * (col & 15))); };
    // [mb][0..1] gate registers 0..7, 8..15; [mb][2..3] up
    u32x4 gu[2][2][4];
    auto load_gu = [&](int nb, u32x4 (&d)[2][4]) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const uint32_t off = ((uint32_t)((wm * 2 + (nb >> 1)) * 8 + mb * 4 + 2 * (nb & 1)) * 1024u +
                              (uint32_t)lane * 16u) * 2u;
        d[mb][0] = load_b128(rgu, off);
        d[mb][1] = load_b128(rgu, off + 16u);
        d[mb][2] = load_b128(rgu, off + 2048u);
        d[mb][3] = load_b128(rgu, off + 2064u);
      }
    };
    load_gu(0, gu[0]);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      u32x4 (&cur)[2][4] = gu[nb & 1];
      // every wave is past its last read of the LDS (the GEMM's stages, or the previous block)
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      raw_barrier();
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const u32x4 gw[2] = {cur[mb][0], cur[mb][1]}, uw[2] = {cur[mb][2], cur[mb][3]};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float dg[4], du[4], pa[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int reg = 4 * q + e;
            const float g = frag_bf16(gw, reg), u = frag_bf16(uw, reg);
            const float d = alpha * acc[mb][nb][reg];
            const float sg = 1.f / (1.f + exp2_fast(-g * kLog2e));
            const float silu = g * sg;
            dg[e] = d * u * sg * (1.f + g * (1.f - sg));
            du[e] = d * silu;
            pa[e] = silu * u;
          }
          const int rq = wm * 16 + mb * 8 + 2 * q + (lane >> 5);  // rows 4 rq .. 4 rq + 3
          const int c = lane & 31;
          st[unit(wn * 64 + c, rq)] = pack_bf16x4(dg[0], dg[1], dg[2], dg[3]);
          st[unit(wn * 64 + 32 + c, rq)] = pack_bf16x4(du[0], du[1], du[2], du[3]);
          st[unit(128 + wn * 32 + c, rq)] = pack_bf16x4(pa[0], pa[1], pa[2], pa[3]);
        }
      }
      if (nb + 1 < 4) load_gu(nb + 1, gu[(nb + 1) & 1]);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      raw_barrier();
      // Row-wise read-out with ds_read_b64_tr_b16.  In a group of 16 lanes, lane k reads rows
      // 4 (rq0 + k % 4) .. + 3 of column c0 + k / 4; lane i then holds columns c0 .. c0 + 3 of
      // row 4 rq0 + i.  Task t: rows 16 (t % 16) .., columns 32 (t / 16) ..; group g of the
      // wave takes 8 of those columns (two reads), so each row gets 64 contiguous bytes.
      // Column blocks 0 .. 3 are d(gate/up), 4 and 5 are p.
#pragma unroll
      for (int s = 0; s < 12; ++s) {
        const int t = s * 8 + wave;
        const int rb = t & 15, cb = t >> 4;
        const int k = lane & 15, g = lane >> 4;
        const int c0 = 32 * cb + 8 * g + (k >> 2);
        const int rq = 4 * rb + (k & 3);
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(st + unit(c0, rq)));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(st + unit(c0 + 4, rq)));
        const int r = 16 * rb + k;
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 v = {l2[0], l2[1], h2[0], h2[1]};
        if (s < 8) {
          const int cc = 32 * cb + 8 * g;
          const int64_t gcol = 512 * (int64_t)tn + 256 * (cc >> 6) + 64 * nb + (cc & 63);
          store_b128(rdg, (r < rl && gcol < n2) ? (uint32_t)((r * n2 + gcol) * 2) : kDrop, v);
        } else {
          const int64_t i = 256 * (int64_t)tn + 128 * (cb - 4) + 32 * nb + 8 * g;
          store_b128(rpa, (r < rl && i < p.N) ? (uint32_t)((r * p.N + i) * 2) : kDrop, v);
        }
      }
    }
  } else if (p.epi == kEpiAccF32Gu) {
    // tile rows wm*64 + [0, 32) are gate rows, wm*64 + [32, 64) up rows, of
    // units (m0 + wm*64)/2 + [0, 32); old values loaded before any store, as above
    const int64_t units = p.M / 2;
    const int64_t u0 = m0 / 2;
    const int ul = (int)min<int64_t>(128, units - u0);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      float* base = static_cast<float*>(mb == 0 ? p.C : p.C2) + u0 * p.ldc + n0;
      const rsrc_t rs = make_rsrc(base, (uint64_t)((int64_t)(ul - 1) * ldc + cl) * 4);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int c = wn * 128 + nb * 32 + (lane & 31);
        float old[16];
#pragma unroll
        for (int reg = 0; reg < 16; ++reg) {
          const int ur = wm * 32 + acc_row(reg, lane);
          old[reg] = load_f32(rs, (ur < ul && c < cl) ? (uint32_t)(ur * ldc + c) * 4u : kDrop);
        }
#pragma unroll
        for (int reg = 0; reg < 16; ++reg) {
          const int ur = wm * 32 + acc_row(reg, lane);
          const uint32_t off = (ur < ul && c < cl) ? (uint32_t)(ur * ldc + c) * 4u : kDrop;
          store_f32(rs, off, old[reg] + alpha * acc[mb][nb][reg]);
        }
      }
    }
  }
}

constexpr int kGemmLds = TileGemm<256, 256, 4, 2, 0, 0, 0, true>::LDS_BYTES;
static_assert(TileGemm<256, 256, 4, 2, 0, 0, 2, true>::LDS_BYTES == kGemmLds &&
                  TileGemm<256, 256, 4, 2, 0, 2, 2, true>::LDS_BYTES == kGemmLds,
              "one LDS size for every operand form");

template <int FA, int FB>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
  gemm_block<FA, FB>(p, blockIdx.x, blockIdx.y, lds);
}

// Several independent GEMMs (no K split) in one grid: workgroups
// start[i] .. start[i+1] - 1 are problem i's grid (each start a multiple of 8,
// so that a workgroup's XCD is the same in both numberings).  Workgroups are
// dispatched in index order as CUs free up, so the problems' tiles pack the
// chip instead of each problem's last partial wave idling part of it.
__global__ __launch_bounds__(kGemmThreads) void k_gemm_group(GemmGroup q) {
  __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
  int i = 0;
  while (i + 1 < q.n && (int)blockIdx.x >= q.start[i + 1]) ++i;
  const GemmArgs& p = q.g[i];
  const int b = (int)blockIdx.x - q.start[i];
  if (p.a_form == 0 && p.b_form == 0) gemm_block<0, 0>(p, b, 0, lds);
  else if (p.a_form == 0 && p.b_form == 2) gemm_block<0, 2>(p, b, 0, lds);
  else gemm_block<2, 2>(p, b, 0, lds);
}

hipError_t launch_gemm_group(const GemmArgs* g, int n, hipStream_t st) {
  if (n < 1 || n > kGemmGroupMax) return hipErrorInvalidValue;
  GemmGroup q = {};
  q.n = 0;
  int64_t blocks = 0;
  for (int i = 0; i < n; ++i) {
    const GemmArgs& a = g[i];
    if (a.M <= 0 || a.N <= 0) continue;
    if (a.ksplit != 1 || a.kchunk % 64 != 0) return hipErrorInvalidValue;
    const bool known = (a.a_form == 0 && (a.b_form == 0 || a.b_form == 2)) || (a.a_form == 2 && a.b_form == 2);
    if (!known) return hipErrorInvalidValue;
    q.g[q.n] = a;
    q.start[q.n] = (int)blocks;
    int64_t b = ((a.M + 255) / 256) * ((a.N + 255) / 256);
    b = (b + 7) / 8 * 8;  // a multiple of 8 (XCD shares when patch_m > 0, alignment of the next start)
    blocks += b;
    ++q.n;
  }
  if (q.n == 0) return hipSuccess;
  q.start[q.n] = (int)blocks;
  hipLaunchKernelGGL(k_gemm_group, dim3((unsigned)blocks), dim3(kGemmThreads), 0, st, q);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0 || a.ksplit <= 0) return hipSuccess;
  const int64_t mt = (a.M + 255) / 256, nt = (a.N + 255) / 256;
  int64_t blocks = mt * nt;
  if (a.patch_m > 0) blocks = (blocks + 7) / 8 * 8;  // eight equal shares, one per XCD
  const dim3 grid((unsigned)blocks, (unsigned)a.ksplit);
  if (a.kchunk % 64 != 0) return hipErrorInvalidValue;
  if (a.a_form == 0 && a.b_form == 0) hipLaunchKernelGGL((k_gemm<0, 0>), grid, dim3(kGemmThreads), 0, st, a);
  else if (a.a_form == 0 && a.b_form == 2) hipLaunchKernelGGL((k_gemm<0, 2>), grid, dim3(kGemmThreads), 0, st, a);
  else if (a.a_form == 2 && a.b_form == 2) hipLaunchKernelGGL((k_gemm<2, 2>), grid, dim3(kGemmThreads), 0, st, a);
  else return hipErrorInvalidValue;  // no other pairing is instantiated
  return hipGetLastError();
}

}  // namespace lmce
