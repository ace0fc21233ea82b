// Device-side building blocks for gfx950 (CDNA4): vector types, the bf16
// MFMA, buffer resources, the swizzled LDS stage layout and the pipelined
// MFMA tile GEMM shared by every kernel of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

#define LMCE_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kThreads = 256;                    // 4 waves of 64 lanes
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;              // running max before any value
constexpr int kAuxSc1 = 16;                      // cache policy: coherent at device scope

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void zero(f32x16& x) {
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = 0.f;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// The wave index within the workgroup, known to the compiler as uniform
// (scalar register), so that addresses built from it stay scalar.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// A wave-uniform value hidden from loop-invariant code motion (kept in a
// scalar register): expressions built from it are recomputed where used.
__device__ __forceinline__ int opaque_s(int x) {
  asm volatile("" : "+s"(x));
  return x;
}

// The lane index, hidden from loop-invariant code motion: addresses derived
// from it are recomputed where they are used instead of being hoisted out of
// the long loops and kept live in registers.
__device__ __forceinline__ int lane_id() {
  int l = threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  return l;
}

// v_mfma_f32_32x32x16 result layout: lane l holds column l % 32 of the
// 32x32 block; its register r holds this row.
__device__ __forceinline__ int acc_row(int reg, int lane) { return ((reg >> 2) << 3) + ((lane >> 5) << 2) + (reg & 3); }

// (m, s) <- merge of two partial log-sum-exp states (s relative to m).
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  s = s * exp2_fast((m - M) * kLog2e) + s2 * exp2_fast((m2 - M) * kLog2e);
  m = M;
}

// Buffer resource over [base, base + bytes): loads past the end return 0,
// stores past the end are dropped.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const int n = bytes > 0x7ffff000ull ? 0x7ffff000 : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left alone).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Barrier across the workgroup without the memory fence of __syncthreads():
// outstanding LDS-DMA loads of the pipeline stay in flight.
__device__ __forceinline__ void raw_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ stages
// A pipeline stage holds ROWS rows x 64 bf16 (128 bytes = eight 16-byte
// chunks per row, one whole cache line).  Logical chunk c of row r sits in
// physical slot c ^ swz(r).  Over every 8 consecutive rows that start at a
// multiple of 8, swz is a permutation of 0..7, and so it is over the even and
// over the odd rows of every 16 such rows: the rows that a ds_read_b128
// serves together (one chunk of consecutive rows) hit distinct banks with
// either a 32- or a 64-bank LDS.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// One wave-level LDS-DMA load moves 1 KiB: lane i lands at lds_base + 16*i,
// i.e. rows r0 .. r0+7, physical slot i % 8, so the eight lanes of a row
// read its whole 128-byte line (TileGemm::dma_one).

// Fragment read from a stage through inline asm: the compiler's LDS-DMA
// bookkeeping would otherwise put a full vmcnt(0) wait in front of every LDS
// read and serialise the prefetch pipeline.  The caller waits for the reads
// with lds_wait() before using the fragments.
__device__ __forceinline__ bf16x8 stage_frag(const char* region, int row, int chunk) {
  const char* p = region + (row * 8 + (chunk ^ swz(row))) * 16;
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
  bf16x8 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(a));
  return v;
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ MN-major stages
// An operand stored MN-major (element (k, r) at k * ld + col + 2 r: consecutive
// rows r of one K index are contiguous) fills a stage as 64 K rows of R bf16
// (2R bytes), 16-byte chunk c of K row kr in physical slot c ^ mn_swz(kr).
// One LDS-DMA instruction moves 1 KiB, 1024 / 2R whole K rows, each lane one
// chunk.  A fragment (the 32 x 16 K-major block the MFMA takes) is read with
// two ds_read_b64_tr_b16: in a group of 16 lanes, lane k reads 4 consecutive
// rows of one K row (8 bytes), and lane i of the group then holds 4
// consecutive K values of one row.  With mn_swz, the 16 lanes of a read hit
// distinct banks.
__device__ __forceinline__ int mn_swz(int kr) { return (2 * (kr & 3)) ^ (8 * ((kr >> 3) & 1)); }

// MFMA operand fragments.  K-major stages (forms 0, 1, 3) give one
// ds_read_b128; MN-major stages (forms 2, 4) two transposing 8-byte reads.
template <int KT>
struct Frag {
  static constexpr int kReads = 1;
  bf16x8 v;
};
struct FragMN {
  static constexpr int kReads = 2;
  u32x2 lo, hi;
};
template <>
struct Frag<2> : FragMN {};
template <>
struct Frag<4> : FragMN {};

template <int KT>
__device__ __forceinline__ bf16x8 frag_value(const Frag<KT>& f) {
  if constexpr (KT == 2 || KT == 4) {
    const u32x4 v = {f.lo[0], f.lo[1], f.hi[0], f.hi[1]};
    return __builtin_bit_cast(bf16x8, v);
  } else {
    return f.v;
  }
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// The fragment of rows rbase .. rbase + 31 (lane % 32) and K columns
// 16 ks + 8 (lane / 32) .. + 7 of the stage part at `region` (R rows).
template <int R, int KT>
__device__ __forceinline__ void frag_read(Frag<KT>& f, const char* region, int rbase, int ks, int lane) {
  if constexpr (KT == 2 || KT == 4) {
    const int g = lane >> 4, i = lane & 15;
    const int kr = 16 * ks + 8 * (g >> 1) + (i >> 2);
    const int r = rbase + 16 * (g & 1) + 4 * (i & 3);
    const char* p0 = region + kr * (2 * R) + (((r >> 3) ^ mn_swz(kr)) << 4) + ((r & 7) << 1);
    const char* p1 = region + (kr + 4) * (2 * R) + (((r >> 3) ^ mn_swz(kr + 4)) << 4) + ((r & 7) << 1);
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(f.lo) : "v"(lds_addr(p0)));
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(f.hi) : "v"(lds_addr(p1)));
  } else {
    f.v = stage_frag(region, rbase + (lane & 31), 2 * ks + (lane >> 5));
  }
}

template <int KT>
__device__ __forceinline__ void frag_tie(Frag<KT>& f) {
  if constexpr (KT == 2 || KT == 4) asm volatile("" : "+v"(f.lo), "+v"(f.hi));
  else asm volatile("" : "+v"(f.v));
}

// s_waitcnt lgkmcnt(N), then every fragment register is tied to a point after
// the wait (volatile asm statements keep their order), so that no use of a
// fragment is scheduled before its read has landed.
template <int N, class FA, int MB, class FB, int NB>
__device__ __forceinline__ void lds_wait(FA (&fa)[MB], FB (&fb)[NB]) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
#pragma unroll
  for (int i = 0; i < MB; ++i) frag_tie(fa[i]);
#pragma unroll
  for (int i = 0; i < NB; ++i) frag_tie(fb[i]);
}

// ------------------------------------------------------------------ GEMM
// acc[mb][nb] += sum_k A[m][k] * B[n][k] over a BM x BN tile, WM x WN waves,
// each wave (wm, wn) owning rows wm*BM/WM + mb*32 + acc_row(.) and columns
// wn*BN/WN + nb*32 + lane%32.  A and B are bf16 with K contiguous,
// reached through buffer resources.  K % 64 == 0.  LDS-DMA loads keep the
// next stages in flight (two 64 KiB stages of a 256 x 256 tile, three 48 KiB
// stages of a 256 x 128 one); one barrier per 64-wide K step.  Whole-line
// (128-byte) row segments per stage matter on gfx950: with 64-byte segments
// the same tiles ran 10 % (256 x 256) and 25 % (256 x 128) slower.  Two-stage
// tiles with fragment prefetch place every fragment read and DMA instruction
// between two MFMAs and pass the K-step barrier before the last sub-step's
// MFMAs (run_interleaved): 6 to 7 % faster in both passes of the training
// pair than issuing them in bursts after the barrier (run_staged).
//
// Operand addressing (bytes from the resource base): row r, K index k is at
//   linear   (KT == 0):  r * ld + col + 2k
//   K-tiled  (KT == 1):  (k / 128) * tstride + r * ld + 2 (k % 128)
//   MN-major (KT == 2):  k * ld + col + 2r  (r counted from the tile's first row)
//   gathered linear   (KT == 3):  idx[r] * ld + col + 2k
//   gathered MN-major (KT == 4):  idx[k] * ld + col + 2r
// The K-tiled form reads matrices stored as consecutive [rows][128] blocks; the
// MN-major form reads a matrix whose rows are the K index (a row-major [K][M]
// matrix used as the transposed operand) without any copy.  The gathered forms
// read the rows of a matrix through an index (a row order or a selection of
// rows) instead of a gathered copy; their offsets idx * ld must stay below
// 2^31 (the buffer range), and rows at or past nrows read as zero.
struct Operand {
  rsrc_t rs;
  uint32_t ld;       // bytes between rows (MN-major: between K rows)
  uint32_t col;      // linear: byte offset of the first K column; MN-major: of the first row
  uint32_t tstride;  // K-tiled: bytes between 128-wide K blocks
  const int* idx;    // gathered forms: row index of each operand row (form 3) or K row (form 4), null for
                     // the identity
  int nrows;         // gathered forms: rows (form 3) or K rows (form 4) that exist; the rest read as zero
  uint32_t roff[4];  // form 3: byte offsets of this lane's DMA rows (the same in every K step)
  int kidx;          // form 4: lane l holds idx of K row 8 wave + l % 8 of the K step whose DMA is issued next
};

template <int KT>
__device__ __forceinline__ uint32_t k_offset(const Operand& o, int kt) {
  if constexpr (KT == 0) return o.col + (uint32_t)kt * 128u;
  else return (uint32_t)(kt >> 1) * o.tstride + (uint32_t)(kt & 1) * 128u;
}

template <int BM, int BN, int WM, int WN, int AUXA = 0, int KTA = 0, int KTB = 0, bool PF = false>
struct TileGemm {
  static constexpr int NW = WM * WN;             // waves
  static constexpr int NT = 64 * NW;             // threads
  static constexpr int BK = 64;
  static constexpr int NKS = BK / 16;            // MFMA K sub-steps per stage
  static constexpr int STAGES = BM + BN <= 384 ? 3 : 2;
  static constexpr int MB = BM / WM / 32;        // 32-row blocks per wave
  static constexpr int NB = BN / WN / 32;        // 32-column blocks per wave
  static constexpr int LOADS = (BM + BN) / 8 / NW;  // DMA instructions per wave per stage
  static constexpr int STAGE_BYTES = (BM + BN) * 128;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static_assert(LDS_BYTES <= 144 * 1024, "leave LDS for the kernels' own arrays");
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "rows per stage must split evenly over the waves");
  static_assert(((KTA != 2 && KTA != 4) || BM == 128 || BM == 256) &&
                    ((KTB != 2 && KTB != 4) || BN == 128 || BN == 256),
                "MN-major operands of 128 or 256 rows");
  using FA = Frag<KTA>;
  using FB = Frag<KTB>;

  // DMA instruction q (of R / 8 / NW per wave) of one operand's part of a stage.
  template <int R, int KT, int AUX>
  __device__ __forceinline__ static void dma_one(const Operand& o, int kt, int q, char* region, int wave, int lane) {
    if constexpr (KT == 2 || KT == 4) {
      // MN-major: instruction qq moves K rows qq * 1024 / 2R .. of the stage, lane by lane in 16-byte chunks
      constexpr int kRowsPer = 1024 / (2 * R);
      const int qq = wave * (R / 8 / NW) + q;
      const int kr = qq * kRowsPer + lane / (R / 8);
      const int c = (lane % (R / 8)) ^ mn_swz(kr);
      uint32_t row;
      if constexpr (KT == 2) {
        row = (uint32_t)(kt * 64 + kr) * o.ld;
      } else {
        // this lane's K row among the wave's 8 of the step: q * kRowsPer + lane / (R / 8); its index is
        // read from the lane of the wave that loaded it
        const int sel = lane / (R / 8);
        int cand[kRowsPer];  // read every candidate first, so that the selection stays branch-free
#pragma unroll
        for (int e = 0; e < kRowsPer; ++e) cand[e] = __builtin_amdgcn_readlane(o.kidx, q * kRowsPer + e);
        int v = cand[0];
#pragma unroll
        for (int e = 1; e < kRowsPer; ++e) v = sel == e ? cand[e] : v;
        const int krg = kt * 64 + wave * 8 + q * kRowsPer + sel;  // the K row, counted from the operand's first
        if (o.idx == nullptr) v = krg;
        row = krg < o.nrows ? (uint32_t)v * o.ld : kNoRow;
      }
      const uint32_t voff = row + o.col + (uint32_t)c * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(o.rs, LMCE_LDS_PTR(region + qq * 1024), 16, voff, 0, 0, AUX);
    } else if constexpr (KT == 3) {
      const int r0 = (wave * (R / 8 / NW) + q) * 8;
      const int r = r0 + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      const uint32_t voff = o.roff[q] + o.col + (uint32_t)kt * 128u + (uint32_t)c * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(o.rs, LMCE_LDS_PTR(region + r0 * 128), 16, voff, 0, 0, AUX);
    } else {
      const int r0 = (wave * (R / 8 / NW) + q) * 8;
      const int r = r0 + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      const uint32_t voff = (uint32_t)r * o.ld + k_offset<KT>(o, kt) + (uint32_t)c * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(o.rs, LMCE_LDS_PTR(region + r0 * 128), 16, voff, 0, 0, AUX);
    }
  }

  static constexpr uint32_t kNoRow = 0x80000000u;  // a row offset past every buffer range: reads zero



  // Form 3: byte offsets of the rows this lane's DMA instructions move (the
  // same rows in every K step), from the index with vector loads.
  template <int R, int KT>
  __device__ __forceinline__ static void gather_rows(Operand& o, int wave, int lane) {
    if constexpr (KT == 3) {
      static_assert(R / 8 / NW <= 4, "row offsets per lane");
#pragma unroll
      for (int q = 0; q < R / 8 / NW; ++q) {
        const int r = (wave * (R / 8 / NW) + q) * 8 + (lane >> 3);
        o.roff[q] = r < o.nrows ? (uint32_t)(o.idx ? o.idx[r] : r) * o.ld : kNoRow;
      }
    }
  }
  // Form 4: idx of the 8 consecutive K rows that the wave's DMA instructions
  // move in K step kt, one per lane (lane l: K row 8 wave + l % 8), with a
  // vector load whose range ends at nrows (past it: zero, unused).  Loaded
  // ahead of the DMA; the DMA picks its rows with v_readlane after the
  // stage's own vmcnt wait, so nothing waits for this load elsewhere.
  template <int R, int KT>
  __device__ __forceinline__ static void load_krows(Operand& o, int kt, int wave, int lane) {
    if constexpr (KT == 4) {
      static_assert((R / 8 / NW) * (1024 / (2 * R)) == 8 && R / 8 / NW <= 4, "8 K rows per wave and step");
      if (o.idx != nullptr) {
        const rsrc_t ri = make_rsrc(o.idx, (uint64_t)(o.nrows > 0 ? o.nrows : 0) * 4);
        o.kidx = (int)__builtin_amdgcn_raw_buffer_load_b32(ri, (uint32_t)((kt * 64 + wave * 8 + (lane & 7)) * 4), 0, 0);
      }
    }
  }

  __device__ __forceinline__ static void issue(int kt, const Operand& a, const Operand& b, char* lds, int wave,
                                               int lane) {
    char* st = lds + (kt % STAGES) * STAGE_BYTES;
#pragma unroll
    for (int q = 0; q < BM / 8 / NW; ++q) dma_one<BM, KTA, AUXA>(a, kt, q, st, wave, lane);
#pragma unroll
    for (int q = 0; q < BN / 8 / NW; ++q) dma_one<BN, KTB, 0>(b, kt, q, st + BM * 128, wave, lane);
  }

  __device__ __forceinline__ static void run(const Operand& a, const Operand& b, int K, char* lds,
                                             f32x16 (&acc)[MB][NB]) {
    if constexpr (PF && STAGES == 2) run_interleaved(a, b, K, lds, acc);
    else run_staged(a, b, K, lds, acc);
  }

  // Fragments of sub-step ks (K columns 16 ks .. 16 ks + 15 of the stage at st).
  __device__ __forceinline__ static void read_a(FA& f, const char* st, int mb, int ks, int wm, int lane) {
    frag_read<BM>(f, st, wm * (BM / WM) + mb * 32, ks, lane);
  }
  __device__ __forceinline__ static void read_b(FB& f, const char* st, int nb, int ks, int wn, int lane) {
    frag_read<BN>(f, st + BM * 128, wn * (BN / WN) + nb * 32, ks, lane);
  }

  __device__ __forceinline__ static void run_staged(const Operand& a, const Operand& b, int K, char* lds,
                                                    f32x16 (&acc)[MB][NB]) {
    const int lane = lane_id();
    const int wave = wave_id();
    const int wm = wave / WN, wn = wave % WN;
    const int nk = K / BK;
    // Every earlier reader of this LDS is past this barrier, and every
    // earlier LDS write of the workgroup has landed (an earlier GEMM's DMA
    // was waited for in its own last step).  Earlier stores of the wave (an
    // exchange tile, a parked accumulator) may still be in flight: they count
    // in vmcnt ahead of the stage loads, so the stage waits below cover them
    // too (loads complete in order, stores only ever add to the count), and
    // they drain while the first stages load instead of before.
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    raw_barrier();
    Operand aa = a, bb = b;  // gathered forms: this lane's row offsets
    gather_rows<BM, KTA>(aa, wave, lane);
    gather_rows<BN, KTB>(bb, wave, lane);
    // gathered MN-major forms: each stage's K rows are loaded one DMA ahead,
    // before the DMA issued in between, so the stage waits below cover them
    Operand an = aa, bn = bb;  // the next stage's
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < nk) {
        load_krows<BM, KTA>(aa, s, wave, lane);
        load_krows<BN, KTB>(bb, s, wave, lane);
        issue(s, aa, bb, lds, wave, lane);
      }
    load_krows<BM, KTA>(an, STAGES - 1, wave, lane);
    load_krows<BN, KTB>(bn, STAGES - 1, wave, lane);
    for (int kt = 0; kt < nk; ++kt) {
      // stage kt has landed (with three stages, kt + 1 may still be in flight)
      if constexpr (STAGES == 3) {
        if (kt + 1 < nk) wait_vmcnt<LOADS>();
        else wait_vmcnt<0>();
      } else {
        wait_vmcnt<0>();
      }
      raw_barrier();
      // the stage refilled here was last read in step kt - 1, whose reads
      // every wave completed before the barrier
      if (kt + STAGES - 1 < nk) {
        aa = an;
        bb = bn;
        load_krows<BM, KTA>(an, kt + STAGES, wave, lane);  // for the next step's DMA, before this one
        load_krows<BN, KTB>(bn, kt + STAGES, wave, lane);
        issue(kt + STAGES - 1, aa, bb, lds, wave, lane);
      }
      const char* st = lds + (kt % STAGES) * STAGE_BYTES;
      if constexpr (PF) {
        // the next sub-step's fragments are read while this one's MFMAs run
        FA fa[2][MB];
        FB fb[2][NB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) read_a(fa[0][mb], st, mb, 0, wm, lane);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) read_b(fb[0][nb], st, nb, 0, wn, lane);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const int cur = ks & 1;
          if (ks + 1 < NKS) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) read_a(fa[cur ^ 1][mb], st, mb, ks + 1, wm, lane);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) read_b(fb[cur ^ 1][nb], st, nb, ks + 1, wn, lane);
            lds_wait<MB * FA::kReads + NB * FB::kReads>(fa[cur], fb[cur]);
          } else {
            lds_wait<0>(fa[cur], fb[cur]);
          }
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              acc[mb][nb] = mfma32(frag_value(fa[cur][mb]), frag_value(fb[cur][nb]), acc[mb][nb]);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          FA fa[MB];
          FB fb[NB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) read_a(fa[mb], st, mb, ks, wm, lane);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) read_b(fb[nb], st, nb, ks, wn, lane);
          lds_wait<0>(fa, fb);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma32(frag_value(fa[mb]), frag_value(fb[nb]), acc[mb][nb]);
        }
      }
    }
  }
  // ---- interleaved schedule (two stages, fragment prefetch)
  static constexpr int LA = BM / 8 / NW, LB = BN / 8 / NW;  // DMA instructions per wave: A part, B part

  // One LDS-DMA instruction of stage kt: idx < LA is one of the A part's, else one of the B part's (the
  // same addresses and slots as issue()).
  __device__ __forceinline__ static void issue_one(int kt, int idx, const Operand& a, const Operand& b, char* lds,
                                                   int wave, int lane) {
    char* st = lds + (kt % STAGES) * STAGE_BYTES;
    if (idx < LA) dma_one<BM, KTA, AUXA>(a, kt, idx, st, wave, lane);
    else dma_one<BN, KTB, 0>(b, kt, idx - LA, st + BM * 128, wave, lane);
  }

  // Fragment j of sub-step ks of a stage: j < MB is A block j, else B block j - MB.
  __device__ __forceinline__ static void read_j(FA (&fa)[MB], FB (&fb)[NB], int j, const char* st, int ks, int wm,
                                                int wn, int lane) {
    if (j < MB) read_a(fa[j], st, j, ks, wm, lane);
    else read_b(fb[j - MB], st, j - MB, ks, wn, lane);
  }

  // One K step over stage kt.  On entry the fragments of sub-step 0 are in
  // flight into set 0.  Each sub-step waits for its own fragments, then issues
  // its MFMAs one at a time with one other instruction after each (scheduling
  // barriers keep that order): the next sub-step's fragment reads, and in the
  // last sub-step the first fragments of stage kt+1 and the DMA of stage kt+2.
  // Before the last sub-step's MFMAs the wave has read all of stage kt, waits
  // for its own part of stage kt+1 and passes the workgroup barrier, after
  // which stage kt+1 is complete and stage kt's buffer can be refilled.
  template <bool NEXT, bool DMA>
  __device__ __forceinline__ static void step_interleaved(int kt, Operand& a, Operand& b, char* lds, int wave,
                                                          int lane, int wm, int wn, FA (&fa)[2][MB], FB (&fb)[2][NB],
                                                          f32x16 (&acc)[MB][NB]) {
    const char* st = lds + (kt % STAGES) * STAGE_BYTES;
    const char* nx = lds + ((kt + 1) % STAGES) * STAGE_BYTES;
    if (DMA) {  // gathered MN-major forms: the K rows of stage kt + 2, read during this step
      load_krows<BM, KTA>(a, kt + 2, wave, lane);
      load_krows<BN, KTB>(b, kt + 2, wave, lane);
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int cur = ks & 1;
      lds_wait<0>(fa[cur], fb[cur]);
      if (NEXT && ks == NKS - 1) {
        wait_vmcnt<0>();
        raw_barrier();
      }
#pragma unroll
      for (int i = 0; i < MB * NB; ++i) {
        acc[i / NB][i % NB] =
            mfma32(frag_value(fa[cur][i / NB]), frag_value(fb[cur][i % NB]), acc[i / NB][i % NB]);
        __builtin_amdgcn_sched_barrier(0);
        if (ks + 1 < NKS) {
          if (i < MB + NB) read_j(fa[cur ^ 1], fb[cur ^ 1], i, st, ks + 1, wm, wn, lane);
        } else if (NEXT) {
          if (i < MB + NB) read_j(fa[cur ^ 1], fb[cur ^ 1], i, nx, 0, wm, wn, lane);
          if (DMA && i < LA + LB) issue_one(kt + 2, i, a, b, lds, wave, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Two stages in LDS; stage kt+2 is loaded while stage kt+1 waits and stage
  // kt is multiplied, and no wave waits for LDS reads with its MFMA queue
  // empty at a stage boundary.  Same products in the same order as
  // run_staged(), so the results are bitwise identical.
  __device__ __forceinline__ static void run_interleaved(const Operand& a, const Operand& b, int K, char* lds,
                                                         f32x16 (&acc)[MB][NB]) {
    static_assert(STAGES == 2 && NKS % 2 == 0 && MB * NB >= MB + NB && MB * NB >= LA + LB,
                  "every fragment read and DMA instruction needs an MFMA slot");
    const int lane = lane_id(), wave = wave_id();
    const int wm = wave / WN, wn = wave % WN;
    const int nk = K / BK;
    // as in run_staged(): earlier readers of this LDS are past the barrier,
    // earlier stores may still drain
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    raw_barrier();
    if (nk <= 0) return;
    Operand aa = a, bb = b;  // gathered forms: this lane's row offsets
    gather_rows<BM, KTA>(aa, wave, lane);
    gather_rows<BN, KTB>(bb, wave, lane);
    load_krows<BM, KTA>(aa, 0, wave, lane);
    load_krows<BN, KTB>(bb, 0, wave, lane);
    issue(0, aa, bb, lds, wave, lane);
    if (nk > 1) {
      load_krows<BM, KTA>(aa, 1, wave, lane);
      load_krows<BN, KTB>(bb, 1, wave, lane);
      issue(1, aa, bb, lds, wave, lane);
      wait_vmcnt<LOADS>();
    } else {
      wait_vmcnt<0>();
    }
    raw_barrier();
    FA fa[2][MB];
    FB fb[2][NB];
#pragma unroll
    for (int j = 0; j < MB + NB; ++j) read_j(fa[0], fb[0], j, lds, 0, wm, wn, lane);
    int kt = 0;
    for (; kt + 2 < nk; ++kt) step_interleaved<true, true>(kt, aa, bb, lds, wave, lane, wm, wn, fa, fb, acc);
    if (kt + 1 < nk) step_interleaved<true, false>(kt++, aa, bb, lds, wave, lane, wm, wn, fa, fb, acc);
    step_interleaved<false, false>(kt, aa, bb, lds, wave, lane, wm, wn, fa, fb, acc);
  }
};

__device__ __forceinline__ Operand linear_operand(const void* base, uint64_t bytes, uint32_t ld, uint32_t col = 0) {
  Operand o;
  o.rs = make_rsrc(base, bytes);
  o.ld = ld;
  o.col = col;
  o.tstride = 0;
  o.idx = nullptr;
  o.nrows = 0;
  return o;
}

// Rows of `base` (ld bytes apart) through idx (null: rows 0, 1, ...); rows at
// or past nrows read as zero.  For the gathered forms 3 and 4.
__device__ __forceinline__ Operand gathered_operand(const void* base, uint64_t bytes, uint32_t ld, const int* idx,
                                                    int nrows, uint32_t col = 0) {
  Operand o = linear_operand(base, bytes, ld, col);
  o.idx = idx;
  o.nrows = nrows;
  return o;
}

__device__ __forceinline__ Operand tiled_operand(const void* base, uint64_t bytes, uint32_t ld, uint32_t tstride) {
  Operand o;
  o.rs = make_rsrc(base, bytes);
  o.ld = ld;
  o.col = 0;
  o.tstride = tstride;
  o.idx = nullptr;
  o.nrows = 0;
  return o;
}

template <int MB, int NB>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[MB][NB]) {
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) zero(acc[i][j]);
}

__device__ __forceinline__ float pick16(const f32x16& x, int reg) {
  float v = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q) v = (q == reg) ? x[q] : v;
  return v;
}

__device__ __forceinline__ uint64_t pack_bf16x4(float a, float b, float c, float d) {
  bf16x4 v = __builtin_convertvector((f32x4){a, b, c, d}, bf16x4);
  return __builtin_bit_cast(uint64_t, v);
}

// 8-byte buffer store, coherent at device scope (seen by sc1 loads of other
// workgroups once the storing wave has waited for it).  voff is per lane,
// soff wave-uniform (kept in a scalar register).
__device__ __forceinline__ void store_sc1_b64(rsrc_t rs, uint32_t voff, uint32_t soff, uint64_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rs, voff, soff, kAuxSc1);
}

// 16-byte buffer store, coherent at device scope.  The whole offset goes in
// the vector offset and the scalar offset is the constant 0: for a buffer
// store of more than 8 bytes whose scalar offset is an SGPR, the compiler
// puts no wait state between the store and a VALU write of its data
// registers, and on gfx950 such a write can reach the data before the store
// has read it (a training-forward build that reused the registers at once
// wrote wrong exchange tiles from run to run).  With a constant scalar
// offset the compiler separates the two itself.
__device__ __forceinline__ void store_sc1_b128(rsrc_t rs, uint32_t voff, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, voff, 0, kAuxSc1);
}

// 4-byte buffer store and load, coherent at device scope.
__device__ __forceinline__ void store_sc1_b32(rsrc_t rs, uint32_t voff, uint32_t soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, voff, soff, kAuxSc1);
}
__device__ __forceinline__ float load_sc1_b32(rsrc_t rs, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, kAuxSc1));
}

// 4-byte buffer store (stores past the resource end are dropped).
__device__ __forceinline__ void store_b32(rsrc_t rs, uint32_t voff, uint32_t soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, voff, soff, 0);
}

// Writes a BM x BN fp32 accumulator tile (the layout of TileGemm) to a
// row-major matrix whose element (0, 0) is at `base`; rows at or past
// `rows_left` are skipped.  Address parts that are the same for the whole
// wave go in the scalar offset; a skipped row gets a vector offset past the
// resource end (the range check applies to the vector offset), so its store
// is dropped.  Each value is stored times f.
template <int MB, int NB>
__device__ __forceinline__ void store_tile_f32(float* base, int64_t rows_left, int64_t ld, int64_t cols_left,
                                               const f32x16 (&acc)[MB][NB], int row0, int col0, int lane,
                                               float f = 1.f) {
  const rsrc_t rs = make_rsrc(base, (uint64_t)((rows_left - 1) * ld + cols_left) * 4);
  lane = lane_id();
  row0 = opaque_s(row0);
  const int lrow = (lane >> 5) << 2;  // row offset of this lane half
  const uint32_t voff = (uint32_t)((lrow * ld + (lane & 31)) * 4);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int reg = 0; reg < 16; ++reg) {
        const int rr = row0 + mb * 32 + ((reg >> 2) << 3) + (reg & 3);
        const uint32_t soff = (uint32_t)(((int64_t)rr * ld + col0 + nb * 32) * 4);
        const uint32_t v = (rr + lrow < rows_left) ? voff : 0xfffffff0u;
        store_b32(rs, v, soff, acc[mb][nb][reg] * f);
      }
}

}  // namespace lmce
