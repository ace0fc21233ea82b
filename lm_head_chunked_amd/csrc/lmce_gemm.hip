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
template <int KT>
__device__ __forceinline__ Operand gemm_operand(const void* base, uint64_t bytes, uint32_t ld, uint32_t tstride,
                                                int64_t r0, int64_t k0) {
  const char* b = static_cast<const char*>(base);
  if constexpr (KT == 0) {
    const uint64_t off = (uint64_t)r0 * ld;
    return linear_operand(b + off, bytes > off ? bytes - off : 0, ld, (uint32_t)(k0 * 2));
  } else {
    const uint64_t off = (uint64_t)(k0 / 128) * tstride + (uint64_t)r0 * ld;
    return tiled_operand(b + off, bytes > off ? bytes - off : 0, ld, tstride);
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

// Accumulator element (mb, nb, reg) of lane `lane` in wave (wm, wn) sits at
// tile row wm*64 + mb*32 + acc_row(reg, lane), tile column wn*128 + nb*32 + lane%32.
template <int KTA, int KTB>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(GemmArgs p) {
  using G = TileGemm<256, 256, 4, 2, 0, KTA, KTB, true>;
  __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES];
  int tm, tn;
  if (!gemm_tile(blockIdx.x, p, tm, tn)) return;  // uniform across the workgroup
  const int64_t m0 = (int64_t)tm * 256, n0 = (int64_t)tn * 256;
  const int64_t k0 = (int64_t)blockIdx.y * p.kchunk;
  const Operand oa = gemm_operand<KTA>(p.A, p.a_bytes, p.a_ld, p.a_tstride, m0, k0);
  const Operand ob = gemm_operand<KTB>(p.B, p.b_bytes, p.b_ld, p.b_tstride, n0, k0);
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
    float* base = static_cast<float*>(p.C) + (int64_t)blockIdx.y * p.c_split + m0 * p.ldc + n0;
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
  } else if (p.epi == kEpiStoreBf16) {
    uint16_t* base = static_cast<uint16_t*>(p.C) + (int64_t)blockIdx.y * p.c_split + m0 * p.ldc + n0;
    const rsrc_t rs = make_rsrc(base, (uint64_t)((int64_t)(rl - 1) * ldc + cl) * 2);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int reg = 0; reg < 16; ++reg) {
        const int r = wm * 64 + mb * 32 + acc_row(reg, lane);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int c = wn * 128 + nb * 32 + (lane & 31);
          store_bf16(rs, (r < rl && c < cl) ? (uint32_t)(r * ldc + c) * 2u : kDrop, alpha * acc[mb][nb][reg]);
        }
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
    // acc = d(act) at unit i = column; gate/up of unit i at 64 (i / 32) + i % 32 (+ 32) of the
    // row.  Outputs: d(gate/up) row-major at C (the dx GEMM's A operand), and K-tiled
    // transposes of d(gate/up) at gT and of silu(g) * u at aux (the weight-gradient GEMMs'
    // operands over the chunk's rows, [t_rows / 128][columns][128]): the lane's registers
    // 4q .. 4q + 3 are four consecutive rows of one column, i.e. 8 contiguous bytes there.
    // Rows from M up to t_rows come out as zeros (their acc and gate/up values read as 0).
    const int64_t n2 = 2 * p.N;
    const int tl = (int)min<int64_t>(256, p.t_rows - m0);  // rows of this tile in the K-tiled outputs
    const rsrc_t rgu = make_rsrc(p.gu + m0 * n2, (uint64_t)rl * n2 * 2);
    const rsrc_t rdg = make_rsrc(static_cast<uint16_t*>(p.C) + m0 * n2, (uint64_t)rl * n2 * 2);
    const rsrc_t rgT = make_rsrc(p.gT + (m0 / 128) * n2 * 128, (uint64_t)((tl + 127) / 128) * n2 * 128 * 2);
    const rsrc_t raT = make_rsrc(p.aux + (m0 / 128) * p.N * 128, (uint64_t)((tl + 127) / 128) * p.N * 128 * 2);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int64_t i = n0 + wn * 128 + nb * 32 + (lane & 31);
        const uint32_t gcol = (uint32_t)((i >> 5) * 64 + (i & 31));
        float g[16], u[16];
#pragma unroll
        for (int reg = 0; reg < 16; ++reg) {  // every load of the block first
          const int r = wm * 64 + mb * 32 + acc_row(reg, lane);
          const uint32_t og = (r < rl && i < p.N) ? ((uint32_t)r * (uint32_t)n2 + gcol) * 2u : kDrop;
          g[reg] = load_bf16(rgu, og);
          u[reg] = load_bf16(rgu, og == kDrop ? kDrop : og + 64u);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float dg[4], du[4], pa[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int reg = 4 * q + e;
            const float d = alpha * acc[mb][nb][reg];
            const float sg = 1.f / (1.f + exp2_fast(-g[reg] * kLog2e));
            const float silu = g[reg] * sg;
            dg[e] = d * u[reg] * sg * (1.f + g[reg] * (1.f - sg));
            du[e] = d * silu;
            pa[e] = silu * u[reg];
            const int r = wm * 64 + mb * 32 + acc_row(reg, lane);
            const uint32_t og = (r < rl && i < p.N) ? ((uint32_t)r * (uint32_t)n2 + gcol) * 2u : kDrop;
            store_bf16(rdg, og, dg[e]);
            store_bf16(rdg, og == kDrop ? kDrop : og + 64u, du[e]);
          }
          const int r4 = wm * 64 + mb * 32 + acc_row(4 * q, lane);  // first of the four rows
          const bool tin = r4 < tl && i < p.N;
          const uint32_t blk = (uint32_t)(r4 >> 7), within = (uint32_t)(r4 & 127);
          const uint32_t ogT = tin ? ((blk * (uint32_t)n2 + gcol) * 128u + within) * 2u : kDrop;
          const uint32_t oaT = tin ? ((blk * (uint32_t)p.N + (uint32_t)i) * 128u + within) * 2u : kDrop;
          store_b64(rgT, ogT, pack_bf16x4(dg[0], dg[1], dg[2], dg[3]));
          store_b64(rgT, tin ? ogT + 32u * 128u * 2u : kDrop, pack_bf16x4(du[0], du[1], du[2], du[3]));
          store_b64(raT, oaT, pack_bf16x4(pa[0], pa[1], pa[2], pa[3]));
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

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0 || a.ksplit <= 0) return hipSuccess;
  const int64_t mt = (a.M + 255) / 256, nt = (a.N + 255) / 256;
  int64_t blocks = mt * nt;
  if (a.patch_m > 0) blocks = (blocks + 7) / 8 * 8;  // eight equal shares, one per XCD
  const dim3 grid((unsigned)blocks, (unsigned)a.ksplit);
  if (a.a_tiled && a.b_tiled) hipLaunchKernelGGL((k_gemm<1, 1>), grid, dim3(kGemmThreads), 0, st, a);
  else if (a.a_tiled) hipLaunchKernelGGL((k_gemm<1, 0>), grid, dim3(kGemmThreads), 0, st, a);
  else if (a.b_tiled) hipLaunchKernelGGL((k_gemm<0, 1>), grid, dim3(kGemmThreads), 0, st, a);
  else hipLaunchKernelGGL((k_gemm<0, 0>), grid, dim3(kGemmThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace lmce
