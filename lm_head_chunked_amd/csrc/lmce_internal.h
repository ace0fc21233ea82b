// Internal declarations shared by the host planner (lmce_api.hip) and the
// device kernels (lmce_fwd.hip, lmce_bwd.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmce {

constexpr int kStatusLabel = 1;     // asynchronous flag: a label was out of range
constexpr int kStatusSync = 2;      // asynchronous flag: a group wait timed out
constexpr int kStatusState = 4;     // asynchronous flag: a training backward without its training forward
constexpr int kSavedTag = 0x6c6d6365;  // header tag: the workspace holds a training forward's O
constexpr int kHdrTag = 0x6c6d6831;    // header tag: status and saved were initialised by this library
constexpr int kStageK = 128;        // hidden-size granularity (the backward slices H by 128)
constexpr int kVTile = 256;         // vocabulary rows per forward logit tile
constexpr int kSyncStride = 64;     // u32 words between two groups' counters (256 bytes)
constexpr int kMaxBwdWGs = 256;     // upper bound of a backward cooperative grid
// Logit tiles each member of a group produces per round: two with 256-wide
// H slices (half the group barriers and parked-accumulator round trips), one
// with 128-wide slices (whose kernels have no registers to spare for it).
constexpr int round_tiles(int hs) { return hs == 256 ? 2 : 1; }
constexpr int kXbufPerTile = 2 * 256 * 256 * 2;  // exchange bytes per workgroup and tile of a round (2 slots)
constexpr int kParkPerWG = 256 * 256 * 4;      // parked 256 x 256 fp32 accumulator slice per backward workgroup
constexpr int kXstatPerWG = 3 * 256 * 4;       // fused forward: per-member round maxima (2 slots) and final sums

// First 256 bytes of the workspace.
struct WsHeader {
  int n_valid;   // rows whose label is not ignore_index (and is in range)
  int status;    // flags of every call since lmce_read_status last cleared them: kStatusLabel | kStatusSync | kStatusState
  int saved;     // kSavedTag once a training forward has filled O without a failed group wait, else 0
  int compact;   // 1 while the dW pass runs on the compacted labelled rows (set by k_compact_rows)
  int n_compact; // rows written by that compaction (its own count of labelled rows)
  int fcompact;  // 1 when the training forward runs on the rows reordered labelled-first (k_permute_rows)
  int f_n;       // labelled rows of that order (the first f_n positions)
  int dcompact;  // 1 when the dh pass of lmce_bwd / lmce_bwd_dh runs on its own labelled-first order
  int d_n;       // labelled rows of that order
  int tag;       // kHdrTag once k_count_labels has initialised status and saved
  int call_flags;  // flags raised by the current entry point only (cleared when it starts)
  int pad0;
  unsigned long long o_addr;  // device address of the buffer the training forward wrote O into
  int pad[50];
};
static_assert(sizeof(WsHeader) == 256, "the header is the first 256 bytes of the workspace");

struct FwdArgs {
  const uint16_t* h;
  const uint16_t* W;
  const int64_t* labels;
  int64_t L, H, V, ignore_index;
  int chunk_rows;       // rows per schedule chunk
  int tile_rows;        // tokens per workgroup tile (128 or 256)
  int tiles_per_chunk;  // ceil(chunk_rows / tile_rows)
  int ntiles;           // row tiles over all chunks
  int segments;         // vocabulary segments swept by separate workgroups
  int vtiles;           // ceil(V / 256)
  int vtiles_per_seg;   // vocabulary tiles per segment
  int xcd_map;          // 1: XCD-aware item order (8 segments, ntiles % 32 == 0)
  WsHeader* hdr;
  float* part_m;        // [segments][L] running max per row and segment
  float* part_s;        // [segments][L] sum of exp(z - max) per row and segment
  float* block_sum;     // [ceil(L/64)] per-block nll sums
  const int* finv;      // training forward: position of row r in the reordered rows (hdr->fcompact), or null
};

struct BwdArgs {
  const uint16_t* h;
  const uint16_t* W;
  const int64_t* labels;
  const float* lse;
  const float* grad_loss;
  int64_t L, H, V, ignore_index;
  int group_size;       // workgroups per group = H / HS (HS = 256 if H % 256 == 0 and H >= 1024, else 128)
  int n_groups;
  int xcd_members;      // > 0: members of one group per XCD (xcd_tiled order); 0: the pass's default order
  int spin_limit;       // bound of every group wait
  unsigned* sync;       // [n_groups * kSyncStride] arrival counters, zeroed before the launch
  uint16_t* xbuf;       // [n_groups][2][2 * R * group_size][256][128] exchange slots, R = round_tiles(HS)
  float* park;          // [workgroups][256 x 256] parked accumulators (HS = 256 only)
  float* xstat;         // [n_groups][3][group_size][256] round maxima (2 slots) and final sums, fused forward
  float* O;             // [L][H] normalised sum_v softmax(z)_v W_v by row: the fused forward's output, written into
                        // the caller's dh buffer
  float* part_m;        // [L] row max, fused forward output
  float* part_s;        // [L] row sum of exp(z - max), fused forward output
  WsHeader* hdr;
  // The labelled rows in order (written by k_compact_rows when hdr->compact):
  // their index, label and lse, and their h rows in the workspace's rows
  // area; the dW pass then sweeps hdr->n_valid rows.  Before
  // that, crow holds the dh pass's labelled-first order when hdr->dcompact
  // (crow[position] = row, h rows in hp).
  int* crow;
  int64_t* clab;
  float* clse;
  uint16_t* ch;
  float* dw_part;       // [group][member][256][HS] partial dW slices of the dW pass's leftover blocks
  // Training forward on the rows reordered labelled-first (when hdr->fcompact):
  // fperm[position] = row, finv[row] = position, hp the reordered h rows (in
  // the rows area, free during the forward); blocks of unlabelled rows compute
  // lse only, and O, part_m, part_s are indexed by position.
  int* fperm;
  int* finv;
  uint16_t* hp;
  // 1: the reordered or compacted h rows are gathered into the rows area (hp,
  // ch) and read from there; 0: they are read from h through the order or
  // selection (when L * H * 2 bytes fit 32-bit buffer offsets) and hp, ch are
  // unused
  int gather_copy;
  float* dh;
  float* dW;
};

// ------------------------------------------------------------------ GEMM
// C = alpha * A B^T on the tile engine: A has M rows, B has N rows, both bf16,
// each read in place either K-major (row r, K index k at r * ld + 2k bytes)
// or MN-major (at k * ld + 2r: a row-major [K][rows] matrix used as the
// transposed operand).  256 x 256 output tiles; grid.y splits K into ksplit
// pieces of kchunk (a multiple of 64), piece z writing at C + z * c_split
// (elements).  Rows past M or N read as zero and are not written; K past an
// operand's end reads as zero.
enum GemmEpi {
  kEpiStoreF32 = 0,   // C fp32 [M][ldc] = alpha * acc
  kEpiAccF32 = 1,     // C fp32 [M][ldc] += alpha * acc
  kEpiStoreFrag = 2,  // C bf16 = alpha * acc in fragment order: per 256 x 256 tile (tm, tn), tile index
                      // tm * ceil(N / 256) + tn, 64 blocks (wave, mb, nb) of 64 lanes x 16 accumulator registers
  kEpiSwigluFwd = 3,  // acc = gate/up pairs (32-column blocks interleaved): C bf16 [M][ldc] = silu(g) * u at column i
  kEpiSwigluBwd = 4,  // acc = d(act) [M][N]: reads the gate/up values gu [M][2N] (interleaved) in fragment order;
                      // C bf16 [M][2N] = d(gate/up) interleaved, aux bf16 [M][N] = silu(g) * u
  kEpiAccF32Gu = 5,   // C (gate rows) and C2 (up rows) fp32 [M/2][ldc] += alpha * acc, A rows interleaved
};

// Largest byte range one buffer resource addresses exactly (make_rsrc clamps
// to it); an operand whose offsets may go past it is read another way.
constexpr uint64_t kMaxBufferBytes = 0x7ffff000ull;

struct GemmArgs {
  // Operand forms: 0 K-major (row r, K index k at r * ld + 2k), 2 MN-major
  // (k * ld + 2r: a row-major [K][rows] matrix read transposed, in place).
  const void* A;
  uint64_t a_bytes;     // bytes readable from A
  uint32_t a_ld;
  int a_form;
  const void* B;
  uint64_t b_bytes;
  uint32_t b_ld;
  int b_form;
  int64_t M, N;
  int64_t kchunk;       // K of one split piece (a multiple of 64)
  int ksplit;
  int epi;
  float alpha;
  void* C;
  void* C2;
  int64_t ldc, c_split;
  const uint16_t* gu;   // kEpiSwigluBwd: gate/up values (fragment order)
  uint16_t* aux;        // kEpiSwigluBwd: silu(g) * u, row-major [M][N]
  int patch_m;          // tile order: patches of patch_m (1, 2, 4, 8) x (32 / patch_m) tiles, one patch per XCD
                        // at a time; 0: row-major
};

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);

// Up to kGemmGroupMax independent GEMMs (ksplit 1, any instantiated operand
// forms and epilogues) in one launch, their tiles packed onto the chip in the
// order given (put the problems with the longest K first).
constexpr int kGemmGroupMax = 3;
struct GemmGroup {
  GemmArgs g[kGemmGroupMax];
  int start[kGemmGroupMax + 1];
  int n;
};
hipError_t launch_gemm_group(const GemmArgs* g, int n, hipStream_t st);

hipError_t launch_count_labels(const int64_t* labels, int64_t L, int64_t V, int64_t ignore_index, WsHeader* hdr,
                               int saved, hipStream_t st);
hipError_t launch_fwd(const FwdArgs& a, float* loss_out, float* lse_out, hipStream_t st);
// train: the training forward, whose last kernel sets the saved tag when its
// group waits all succeeded.
hipError_t launch_fwd_rows(const FwdArgs& a, float* loss_out, float* lse_out, hipStream_t st, bool train = false,
                           const float* o_buf = nullptr);
// Compaction of the labelled rows for the dW pass (cnt: ceil(L / 1024) ints)
// and their h rows gathered into a.ch.
hipError_t launch_compact(const BwdArgs& a, int* cnt, int64_t ch_rows, hipStream_t st);
// Labelled-first order of the rows, if it saves a 256-row block: flags[0] = 1
// and flags[1] = labelled rows (else 0, 0), perm[position] = row, inv[row] =
// position (inv may be null), and the reordered h rows in a.hp.  Used by the
// training forward (fperm, finv, hdr->fcompact) and by the dh pass (crow,
// hdr->dcompact).
hipError_t launch_permute(const BwdArgs& a, int* cnt, int* flags, int* perm, int* inv, hipStream_t st);
hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t st);
// Group-scheduled kernels: the two backward passes and the fused training forward.
constexpr int kPassDh = 0, kPassDw = 1, kPassFwdDh = 2;
hipError_t bwd_resident_wgs(int pass, int hs, int* wgs);
hipError_t launch_bwd_group(int pass, const BwdArgs& a, int hs, int n_wgs, hipStream_t st);
hipError_t launch_dh_finish(const BwdArgs& a, hipStream_t st);
// Sums the dW pass's partial slices of its leftover blocks (no-op when none).
hipError_t launch_dw_tail(const BwdArgs& a, int hs, hipStream_t st);
// dW *= g/N after a dW pass with 128-wide slices (no-op for 256-wide ones,
// which apply the factor when they store).
hipError_t launch_dw_scale(const BwdArgs& a, int hs, hipStream_t st);

}  // namespace lmce
