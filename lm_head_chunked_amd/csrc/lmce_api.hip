// Host side of the C ABI declared in include/lmce.h: argument checks,
// schedule and workspace planning, and kernel launches on the caller's
// stream.  The library never allocates device memory and never synchronises
// outside lmce_read_status.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "lmce.h"
#include "lmce_internal.h"

namespace lmce {
namespace {

constexpr int64_t kMaxRows = int64_t(1) << 21;   // L and V limits (32-bit buffer offsets stay exact)
constexpr int64_t kMaxHidden = 16384;
constexpr int kSpinLimit = 1 << 21;                // bound of every group wait (about a second)

// Bound of every group wait.  LMCE_SPIN_LIMIT (a non-negative integer) lowers
// it, so that tests can make the waits give up and check how that failure is
// reported while every kernel still exits normally.
int spin_limit() {
  const char* e = getenv("LMCE_SPIN_LIMIT");
  if (e == nullptr || *e == '\0') return kSpinLimit;
  char* end = nullptr;
  const long v = strtol(e, &end, 10);
  if (end == e || *end != '\0' || v < 0 || v > kSpinLimit) return kSpinLimit;
  return (int)v;
}

struct Plan {
  int64_t L, H, V;
  int chunk_rows, tile_rows, tiles_per_chunk, n_chunks, ntiles, segments, vtiles, vtiles_per_seg, xcd_map;
  int hs, xbuf_wgs, gather_copy;
  size_t off_pm, off_ps, off_bsum, off_rows, off_sync, off_xbuf, off_park, off_xstat, off_cnt, off_crow,
      off_clab, off_clse, off_part, off_fperm, off_finv, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int check_shape(int64_t L, int64_t H, int64_t V, int64_t chunk_rows) {
  if (L < 1 || L > kMaxRows || V < 1 || V > kMaxRows || H < 1 || H > kMaxHidden) return LMCE_ERR_SHAPE;
  if (H % kStageK != 0) return LMCE_ERR_UNSUPPORTED;
  if (chunk_rows < 32 || chunk_rows > 1024 || chunk_rows % 32 != 0) return LMCE_ERR_UNSUPPORTED;
  return LMCE_OK;
}

int make_plan(int64_t L, int64_t H, int64_t V, int64_t chunk_rows, Plan* p) {
  int st = check_shape(L, H, V, chunk_rows);
  if (st != LMCE_OK) return st;
  p->L = L;
  p->H = H;
  p->V = V;
  p->chunk_rows = (int)chunk_rows;
  // Forward row tiles: 256 tokens when chunks are whole multiples of 256,
  // else 128.  Per-row arithmetic does not depend on the tile height.
  p->tile_rows = (chunk_rows % 256 == 0) ? 256 : 128;
  p->tiles_per_chunk = (int)((chunk_rows + p->tile_rows - 1) / p->tile_rows);
  p->n_chunks = (int)((L + chunk_rows - 1) / chunk_rows);
  p->ntiles = p->n_chunks * p->tiles_per_chunk;
  p->vtiles = (int)((V + kVTile - 1) / kVTile);
  // Vocabulary segments: a function of V only, so that results never depend
  // on chunk_rows.  Eight segments (one per XCD position) when V allows.
  int seg = p->vtiles >= 32 ? 8 : (p->vtiles / 4 > 0 ? p->vtiles / 4 : 1);
  p->vtiles_per_seg = (p->vtiles + seg - 1) / seg;
  p->segments = (p->vtiles + p->vtiles_per_seg - 1) / p->vtiles_per_seg;
  p->xcd_map = (p->segments == 8 && p->ntiles % 32 == 0) ? 1 : 0;
  // Widest H slice of one backward workgroup.  A 256-wide slice parks its
  // accumulator (256 KiB out and back per round of two logit tiles per
  // member); the round's work grows with H, and from H = 1024 up the square
  // tiles and the second tile per round win (Qwen3-4B head, H = 2560:
  // training pair 507.5 against 454.0 ms; Qwen3-0.6B head, H = 1024: 11.25
  // against 10.8 ms, same box).
  p->hs = (H % 256 == 0 && H >= 1024) ? 256 : 128;

  size_t off = align256(sizeof(WsHeader));
  p->off_pm = off;
  off = align256(off + sizeof(float) * (size_t)L * (size_t)p->segments);
  p->off_ps = off;
  off = align256(off + sizeof(float) * (size_t)L * (size_t)p->segments);
  p->off_bsum = off;
  off = align256(off + sizeof(float) * (size_t)((L + 63) / 64));
  // The group passes read h's rows in a labelled-first order or only the
  // labelled ones through an index, with 32-bit buffer offsets from h.  Past
  // 2^31 bytes of h they read a gathered copy instead (the labelled-first
  // rows of the training forward or of the dh pass, or the dW pass's
  // compacted rows, one at a time).
  // Also with 128-wide slices (see k_bwd_dW's consumer).
  p->gather_copy = ((uint64_t)L * (uint64_t)H * 2 > kMaxBufferBytes || p->hs == 128) ? 1 : 0;
  p->off_rows = off;
  if (p->gather_copy) off = align256(off + sizeof(uint16_t) * (size_t)H * (size_t)L);
  p->off_sync = off;
  off = align256(off + sizeof(unsigned) * (size_t)kMaxBwdWGs * kSyncStride);
  p->off_xbuf = off;
  // Exchange slots for as many backward workgroups as can be useful (at most
  // one group per row block or vocabulary block, at most kMaxBwdWGs).
  const int64_t items = (L + 255) / 256 > (V + 255) / 256 ? (L + 255) / 256 : (V + 255) / 256;
  int64_t wgs = items * (H / 128);  // enough for either slice width
  if (wgs > kMaxBwdWGs) wgs = kMaxBwdWGs;
  p->xbuf_wgs = (int)wgs;
  off = align256(off + (size_t)wgs * kXbufPerTile * round_tiles(p->hs));
  p->off_park = off;
  if (p->hs == 256) off = align256(off + (size_t)wgs * kParkPerWG);
  p->off_xstat = off;
  off = align256(off + (size_t)wgs * kXstatPerWG);
  // dW pass on the labelled rows only: per-chunk counts, then their index,
  // label and lse (their h rows go to the rows area)
  p->off_cnt = off;
  off = align256(off + sizeof(int) * (size_t)((L + 1023) / 1024));
  p->off_crow = off;
  off = align256(off + sizeof(int) * (size_t)L);
  p->off_clab = off;
  off = align256(off + sizeof(int64_t) * (size_t)L);
  p->off_clse = off;
  off = align256(off + sizeof(float) * (size_t)L);
  // dW pass: partial slices of its leftover vocabulary blocks (one 256 x HS
  // fp32 slice per workgroup at most)
  p->off_part = off;
  off = align256(off + (size_t)wgs * kParkPerWG);
  // training forward: labelled-first order of the rows and its inverse (the
  // reordered h rows go to the rows area)
  p->off_fperm = off;
  off = align256(off + sizeof(int) * (size_t)L);
  p->off_finv = off;
  off = align256(off + sizeof(int) * (size_t)L);
  p->total = off;
  return LMCE_OK;
}

bool aligned(const void* ptr, uintptr_t a) { return ptr != nullptr && (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

}  // namespace
}  // namespace lmce

using namespace lmce;

extern "C" int lmce_version(void) { return 100; }

extern "C" const char* lmce_strerror(int status) {
  switch (status) {
    case LMCE_OK: return "ok";
    case LMCE_ERR_NULL: return "a required pointer is NULL or misaligned";
    case LMCE_ERR_SHAPE: return "L, H or V out of range";
    case LMCE_ERR_UNSUPPORTED: return "unsupported shape: H must be a multiple of 128, chunk_rows a multiple of 32 in [32, 1024]";
    case LMCE_ERR_WORKSPACE: return "workspace smaller than lmce_workspace_size()";
    case LMCE_ERR_HIP: return "HIP runtime error";
    case LMCE_ERR_LABEL: return "a label is outside [0, V) and is not ignore_index";
    case LMCE_ERR_STATE: return "lmce_bwd_train without a preceding lmce_fwd_train on this workspace";
    case LMCE_ERR_SCRATCH: return "the shape needs more than the fixed no-allocation area holds (L up to 2^20 rows)";
    default: return "unknown status";
  }
}

extern "C" int lmce_workspace_size(int64_t L, int64_t H, int64_t V, int64_t chunk_rows, size_t* bytes) {
  if (bytes == nullptr) return LMCE_ERR_NULL;
  Plan p;
  int st = make_plan(L, H, V, chunk_rows, &p);
  if (st != LMCE_OK) return st;
  *bytes = p.total;
  return LMCE_OK;
}

namespace lmce {
namespace {

// The plain forward on a prepared area: the header at `hdr` and the
// per-segment partials and block sums at the plan's offsets from `base`
// (the first p.off_rows bytes of a workspace layout).
int fwd_launch(const Plan& p, const void* h, const void* W, const int64_t* labels, int64_t ignore_index,
               float* loss_out, float* lse_out, void* base, hipStream_t s) {
  WsHeader* hdr = at<WsHeader>(base, 0);
  if (launch_count_labels(labels, p.L, p.V, ignore_index, hdr, 0, s) != hipSuccess) return LMCE_ERR_HIP;
  FwdArgs a = {};
  a.finv = nullptr;  // the plain forward keeps the rows in their order
  a.h = static_cast<const uint16_t*>(h);
  a.W = static_cast<const uint16_t*>(W);
  a.labels = labels;
  a.L = p.L;
  a.H = p.H;
  a.V = p.V;
  a.ignore_index = ignore_index;
  a.chunk_rows = p.chunk_rows;
  a.tile_rows = p.tile_rows;
  a.tiles_per_chunk = p.tiles_per_chunk;
  a.ntiles = p.ntiles;
  a.segments = p.segments;
  a.vtiles = p.vtiles;
  a.vtiles_per_seg = p.vtiles_per_seg;
  a.xcd_map = p.xcd_map;
  a.hdr = hdr;
  a.part_m = at<float>(base, p.off_pm);
  a.part_s = at<float>(base, p.off_ps);
  a.block_sum = at<float>(base, p.off_bsum);
  if (launch_fwd(a, loss_out, lse_out, s) != hipSuccess) return LMCE_ERR_HIP;
  return LMCE_OK;
}

}  // namespace
}  // namespace lmce

extern "C" int lmce_fwd(const void* h, const void* W, const int64_t* labels, int64_t L, int64_t H, int64_t V,
                        int64_t ignore_index, int64_t chunk_rows, float* loss_out, float* lse_out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  Plan p;
  int st = make_plan(L, H, V, chunk_rows, &p);
  if (st != LMCE_OK) return st;
  if (!aligned(h, 16) || !aligned(W, 16) || !aligned(labels, 8) || !aligned(loss_out, 4) || !aligned(lse_out, 4) ||
      !aligned(workspace, 256))
    return LMCE_ERR_NULL;
  if (workspace_bytes < p.total) return LMCE_ERR_WORKSPACE;
  return fwd_launch(p, h, W, labels, ignore_index, loss_out, lse_out, workspace, static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------ no-allocation forward
// lmce_fwd_noalloc runs the plain forward's kernels on a fixed area of device
// memory that the library itself holds, `scratch`, instead of a workspace
// the caller allocates.  The area has room for the forward's part of the
// workspace layout (header, per-row partials of the vocabulary segments,
// block sums: about 64 bytes per row), which covers L up to 2^20 rows.  Each
// device the library runs on holds its own copy until the process ends.
namespace lmce {
namespace {

constexpr size_t kScratchBytes = size_t(65) << 20;
constexpr int64_t kScratchMaxRows = int64_t(1) << 20;  // the forward layout of 2^20 rows (8 segments) needs 64.06 MiB
constexpr int kMaxScratchDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device (in host code the array's name is only a host-side stand-in).
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LMCE_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return LMCE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return LMCE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LMCE_OK;
}

}  // namespace
}  // namespace lmce

extern "C" int lmce_fwd_noalloc(const void* h, const void* W, const int64_t* labels, int64_t L, int64_t H,
                                int64_t V, int64_t ignore_index, int64_t chunk_rows, float* loss_out, float* lse_out,
                                void* stream) {
  Plan p;
  int st = make_plan(L, H, V, chunk_rows, &p);
  if (st != LMCE_OK) return st;
  if (!aligned(h, 16) || !aligned(W, 16) || !aligned(labels, 8) || !aligned(loss_out, 4) || !aligned(lse_out, 4))
    return LMCE_ERR_NULL;
  if (L > kScratchMaxRows || p.off_rows > kScratchBytes) return LMCE_ERR_SCRATCH;  // the forward's part of the layout
  void* base = nullptr;
  st = scratch_on_current_device(&base);
  if (st != LMCE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The area keeps the previous call's contents: clear the header (with a
  // fill kernel, which graph capture records as an ordinary node), so that
  // this call's status starts empty; every other part is written before it
  // is read.
  if (launch_zero_u32(static_cast<unsigned*>(base), (int)(sizeof(WsHeader) / sizeof(unsigned)), s) != hipSuccess)
    return LMCE_ERR_HIP;
  return fwd_launch(p, h, W, labels, ignore_index, loss_out, lse_out, base, s);
}

namespace {

// Members of one group per XCD (xcd_tiled order), or 0 for the pass's
// default order.  In a round, every member reads two operands of its own
// (the producer's 256 x H tile, and the consumer's HS columns of W^T or h^T
// over the round's 256 s vocabulary or token rows: 512 H bytes each, shared
// with the same member of the other groups) and two of its group (the
// producer's other 256 x H tile and the exchange slot of s 256 x 256 bf16
// tiles).  The workgroups of one XCD that
// host a members of each of b = nwg / 8 / a groups read about
// 1024 H a + (512 H + 131072 s) b bytes per round through their L2, that is
// 2a + 2b tile-sized units for 256-wide slices and 2a + 3b for 128-wide ones;
// the valid a with the smallest cost is taken.  Ties are broken as measured
// on the Qwen3-8B head shape with 131072 rows (H = 4096, V = 151936; A/B runs
// of both builds on one GPU, 256-wide slices, a = 4 or 8): the dW
// pass takes the larger a (a = 8 against whole groups per XCD cut it from
// 305.6 to 296.9 ms), the passes whose groups own row blocks the smaller one
// (the training forward ran 299.9 ms with a = 4 against 308.7 with a = 8).
int group_xcd_members(int pass, int hs, int s, int nwg) {
  if (nwg % 8 != 0) return 0;
  const int c = hs == 256 ? 2 : 3;
  const bool larger = pass == kPassDw;
  int best = 0, cost = 1 << 30;
  for (int i = 1; i <= s; ++i) {
    const int a = larger ? s + 1 - i : i;
    if (s % a != 0 || 8 % (s / a) != 0 || (nwg / 8) % a != 0) continue;
    const int k = 2 * a + c * ((nwg / 8) / a);
    if (k < cost) {
      cost = k;
      best = a;
    }
  }
  return best;
}

// One group-scheduled pass over `items` blocks (row blocks or vocabulary
// blocks): picks the H slice width, sizes the cooperative grid to the
// resident workgroups, resets the group counters and launches.
int launch_group_pass(int pass, BwdArgs& a, const Plan& p, int64_t items, hipStream_t s) {
  int hs = p.hs;
  int resident = 0;
  if (bwd_resident_wgs(pass, hs, &resident) != hipSuccess) return LMCE_ERR_HIP;
  if (resident > p.xbuf_wgs) resident = p.xbuf_wgs;
  // 256-wide slices run both GEMMs on square tiles, but a group then holds
  // half as many workgroups: with fewer blocks than groups, half the chip
  // would idle, so such a pass takes 128-wide slices.
  // (Not the dW pass without a gathered copy: with 128-wide slices it reads
  // the selected rows from that copy.)
  if (hs == 256 && items < resident / (p.H / 256) && (pass != kPassDw || p.gather_copy)) {
    hs = 128;
    if (bwd_resident_wgs(pass, hs, &resident) != hipSuccess) return LMCE_ERR_HIP;
    if (resident > p.xbuf_wgs) resident = p.xbuf_wgs;
  }
  const int group_size = (int)(p.H / hs);
  int64_t groups = resident / group_size;
  if (groups > items) groups = items;
  if (groups < 1) return LMCE_ERR_UNSUPPORTED;
  a.group_size = group_size;
  a.n_groups = (int)groups;
  a.xcd_members = group_xcd_members(pass, hs, group_size, (int)groups * group_size);
  if (launch_zero_u32(a.sync, (int)groups * kSyncStride, s) != hipSuccess) return LMCE_ERR_HIP;
  if (launch_bwd_group(pass, a, hs, (int)groups * group_size, s) != hipSuccess) return LMCE_ERR_HIP;
  if (pass == kPassDw && (launch_dw_tail(a, hs, s) != hipSuccess || launch_dw_scale(a, hs, s) != hipSuccess))
    return LMCE_ERR_HIP;
  return LMCE_OK;
}

// Arguments shared by the group-scheduled kernels (pointers into the workspace).
BwdArgs group_args(const Plan& p, const void* h, const void* W, const int64_t* labels, int64_t ignore_index,
                   void* workspace) {
  BwdArgs a = {};
  a.h = static_cast<const uint16_t*>(h);
  a.W = static_cast<const uint16_t*>(W);
  a.labels = labels;
  a.L = p.L;
  a.H = p.H;
  a.V = p.V;
  a.ignore_index = ignore_index;
  a.spin_limit = spin_limit();
  a.sync = at<unsigned>(workspace, p.off_sync);
  a.xbuf = at<uint16_t>(workspace, p.off_xbuf);
  a.park = at<float>(workspace, p.off_park);
  a.xstat = at<float>(workspace, p.off_xstat);
  a.part_m = at<float>(workspace, p.off_pm);
  a.part_s = at<float>(workspace, p.off_ps);
  a.hdr = at<WsHeader>(workspace, 0);
  a.crow = at<int>(workspace, p.off_crow);
  a.clab = at<int64_t>(workspace, p.off_clab);
  a.clse = at<float>(workspace, p.off_clse);
  a.ch = at<uint16_t>(workspace, p.off_rows);
  a.dw_part = at<float>(workspace, p.off_part);
  a.fperm = at<int>(workspace, p.off_fperm);
  a.finv = at<int>(workspace, p.off_finv);
  a.hp = at<uint16_t>(workspace, p.off_rows);
  a.gather_copy = p.gather_copy;
  return a;
}

// Runs the dW pass: compacts the labelled rows (if that saves a 256-row
// block; their h rows overwrite the rows area, so it comes after every pass
// that reads the dh pass's reordered rows), then the group pass.
int dw_pass(BwdArgs& a, const Plan& p, void* workspace, hipStream_t s) {
  if (launch_compact(a, at<int>(workspace, p.off_cnt), p.L, s) != hipSuccess) return LMCE_ERR_HIP;
  return launch_group_pass(kPassDw, a, p, (p.V + 255) / 256, s);
}

// Shared by lmce_bwd, lmce_bwd_dh and lmce_bwd_dW: which = 1 (dh), 2 (dW), 3 (both).
int bwd_common(int which, const void* h, const void* W, const int64_t* labels, const float* lse, int64_t L,
               int64_t H, int64_t V, int64_t ignore_index, int64_t chunk_rows, const float* grad_loss, float* dh_out,
               float* dW_out, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  int st = make_plan(L, H, V, chunk_rows, &p);
  if (st != LMCE_OK) return st;
  if (!aligned(h, 16) || !aligned(W, 16) || !aligned(labels, 8) || !aligned(lse, 4) || !aligned(grad_loss, 4) ||
      ((which & 1) && !aligned(dh_out, 16)) || ((which & 2) && !aligned(dW_out, 16)) || !aligned(workspace, 256))
    return LMCE_ERR_NULL;
  if (workspace_bytes < p.total) return LMCE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);

  WsHeader* hdr = at<WsHeader>(workspace, 0);
  if (launch_count_labels(labels, L, V, ignore_index, hdr, -1, s) != hipSuccess) return LMCE_ERR_HIP;
  BwdArgs a = group_args(p, h, W, labels, ignore_index, workspace);
  a.lse = lse;
  a.grad_loss = grad_loss;
  a.dh = dh_out;
  a.dW = dW_out;
  if (which & 1) {
    // the dh pass's own labelled-first order, in the compaction's row array
    // and the rows area (the dW pass rewrites both afterwards)
    if (launch_permute(a, at<int>(workspace, p.off_cnt), &hdr->dcompact, a.crow, nullptr, s) != hipSuccess)
      return LMCE_ERR_HIP;
    st = launch_group_pass(kPassDh, a, p, (L + 255) / 256, s);
    if (st != LMCE_OK) return st;
  }
  if (which & 2) {
    st = dw_pass(a, p, workspace, s);
    if (st != LMCE_OK) return st;
  }
  return LMCE_OK;
}

}  // namespace

extern "C" int lmce_bwd(const void* h, const void* W, const int64_t* labels, const float* lse, int64_t L, int64_t H,
                        int64_t V, int64_t ignore_index, int64_t chunk_rows, const float* grad_loss, float* dh_out,
                        float* dW_out, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_common(3, h, W, labels, lse, L, H, V, ignore_index, chunk_rows, grad_loss, dh_out, dW_out, workspace,
                    workspace_bytes, stream);
}

extern "C" int lmce_bwd_dh(const void* h, const void* W, const int64_t* labels, const float* lse, int64_t L,
                           int64_t H, int64_t V, int64_t ignore_index, int64_t chunk_rows, const float* grad_loss,
                           float* dh_out, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_common(1, h, W, labels, lse, L, H, V, ignore_index, chunk_rows, grad_loss, dh_out, nullptr, workspace,
                    workspace_bytes, stream);
}

extern "C" int lmce_bwd_dW(const void* h, const void* W, const int64_t* labels, const float* lse, int64_t L,
                           int64_t H, int64_t V, int64_t ignore_index, int64_t chunk_rows, const float* grad_loss,
                           float* dW_out, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_common(2, h, W, labels, lse, L, H, V, ignore_index, chunk_rows, grad_loss, nullptr, dW_out, workspace,
                    workspace_bytes, stream);
}

extern "C" int lmce_fwd_train(const void* h, const void* W, const int64_t* labels, int64_t L, int64_t H, int64_t V,
                              int64_t ignore_index, int64_t chunk_rows, float* loss_out, float* lse_out,
                              float* dh_out, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  int st = make_plan(L, H, V, chunk_rows, &p);
  if (st != LMCE_OK) return st;
  if (!aligned(h, 16) || !aligned(W, 16) || !aligned(labels, 8) || !aligned(loss_out, 4) || !aligned(lse_out, 4) ||
      !aligned(dh_out, 16) || !aligned(workspace, 256))
    return LMCE_ERR_NULL;
  if (workspace_bytes < p.total) return LMCE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);

  // the saved tag is cleared now and set by the forward's last kernel only
  // if every group wait of k_fwd_dh succeeded
  WsHeader* hdr = at<WsHeader>(workspace, 0);
  if (launch_count_labels(labels, L, V, ignore_index, hdr, 0, s) != hipSuccess) return LMCE_ERR_HIP;
  BwdArgs a = group_args(p, h, W, labels, ignore_index, workspace);
  a.O = dh_out;  // O rows live in the caller's dh buffer until lmce_bwd_train turns them into dh
  if (launch_permute(a, at<int>(workspace, p.off_cnt), &hdr->fcompact, a.fperm, a.finv, s) != hipSuccess)
    return LMCE_ERR_HIP;
  st = launch_group_pass(kPassFwdDh, a, p, (L + 255) / 256, s);
  if (st != LMCE_OK) return st;
  // (max, sum) of every row came out as one log-sum-exp segment
  FwdArgs f = {};
  f.h = a.h;
  f.W = a.W;
  f.labels = labels;
  f.L = L;
  f.H = H;
  f.V = V;
  f.ignore_index = ignore_index;
  f.chunk_rows = p.chunk_rows;
  f.segments = 1;
  f.hdr = hdr;
  f.part_m = a.part_m;
  f.part_s = a.part_s;
  f.block_sum = at<float>(workspace, p.off_bsum);
  f.finv = a.finv;
  if (launch_fwd_rows(f, loss_out, lse_out, s, true, dh_out) != hipSuccess) return LMCE_ERR_HIP;
  return LMCE_OK;
}

extern "C" int lmce_bwd_train(const void* h, const void* W, const int64_t* labels, const float* lse, int64_t L,
                              int64_t H, int64_t V, int64_t ignore_index, int64_t chunk_rows, const float* grad_loss,
                              float* dh_out, float* dW_out, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  int st = make_plan(L, H, V, chunk_rows, &p);
  if (st != LMCE_OK) return st;
  if (!aligned(h, 16) || !aligned(W, 16) || !aligned(labels, 8) || !aligned(lse, 4) || !aligned(grad_loss, 4) ||
      !aligned(dh_out, 16) || !aligned(dW_out, 16) || !aligned(workspace, 256))
    return LMCE_ERR_NULL;
  if (workspace_bytes < p.total) return LMCE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);

  // N from these labels: a plain backward with other labels may have run on
  // the workspace since the training forward (the forward's tag stays)
  if (launch_count_labels(labels, L, V, ignore_index, at<WsHeader>(workspace, 0), -1, s) != hipSuccess)
    return LMCE_ERR_HIP;
  BwdArgs a = group_args(p, h, W, labels, ignore_index, workspace);
  a.lse = lse;
  a.grad_loss = grad_loss;
  a.dh = dh_out;
  a.dW = dW_out;
  if (launch_dh_finish(a, s) != hipSuccess) return LMCE_ERR_HIP;
  return dw_pass(a, p, workspace, s);
}

extern "C" int lmce_read_status(void* workspace, void* stream) {
  if (!aligned(workspace, 256)) return LMCE_ERR_NULL;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return LMCE_ERR_HIP;
  WsHeader hdr;
  if (hipMemcpy(&hdr, workspace, sizeof(hdr), hipMemcpyDeviceToHost) != hipSuccess) return LMCE_ERR_HIP;
  if (hdr.tag != kHdrTag) return LMCE_OK;  // no call has run on this workspace yet
  if (hdr.status != 0) {
    // the flags accumulate over calls until read here; clear them
    const int zero = 0;
    if (hipMemcpy(&at<WsHeader>(workspace, 0)->status, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess)
      return LMCE_ERR_HIP;
  }
  if (hdr.status & kStatusLabel) return LMCE_ERR_LABEL;
  if (hdr.status & kStatusSync) return LMCE_ERR_HIP;
  if (hdr.status & kStatusState) return LMCE_ERR_STATE;
  return LMCE_OK;
}
