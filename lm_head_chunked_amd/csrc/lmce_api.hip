// Host side of the C ABI declared in include/lmce.h: argument checks,
// schedule and workspace planning, and kernel launches on the caller's
// stream.  The library never allocates device memory and never synchronises
// outside lmce_read_status.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "lmce.h"
#include "lmce_internal.h"

namespace lmce {
namespace {

constexpr int64_t kMaxRows = int64_t(1) << 24;   // L and V limits (int32 grid math stays exact)
constexpr int64_t kMaxHidden = 16384;

struct Plan {
  int64_t L, H, V;
  int chunk_rows, tiles_per_chunk, n_chunks, segments, vtiles, vtiles_per_seg;
  int64_t Lpad, Vpad;
  int hs;
  size_t off_zlabel, off_pm, off_ps, off_bsum, off_hT, off_WT, total;
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
  p->tiles_per_chunk = (int)((chunk_rows + kTile - 1) / kTile);
  p->n_chunks = (int)((L + chunk_rows - 1) / chunk_rows);
  p->vtiles = (int)((V + kTile - 1) / kTile);
  // Vocabulary segments: enough workgroups to fill the chip when L is small.
  // Depends on L and V only, so that results never depend on chunk_rows.
  const int64_t row_tiles = (L + kTile - 1) / kTile;
  int64_t seg = (1024 + row_tiles - 1) / row_tiles;
  int64_t seg_cap = p->vtiles / 4 > 0 ? p->vtiles / 4 : 1;
  if (seg > seg_cap) seg = seg_cap;
  if (seg < 1) seg = 1;
  p->vtiles_per_seg = (int)((p->vtiles + seg - 1) / seg);
  p->segments = (p->vtiles + p->vtiles_per_seg - 1) / p->vtiles_per_seg;
  p->Lpad = (L + kTile - 1) / kTile * kTile;
  p->Vpad = (V + kTile - 1) / kTile * kTile;
  p->hs = (H % 256 == 0) ? 256 : (H % 128 == 0) ? 128 : 64;

  size_t off = align256(sizeof(WsHeader));
  p->off_zlabel = off;
  off = align256(off + sizeof(float) * (size_t)L);
  p->off_pm = off;
  off = align256(off + sizeof(float) * (size_t)L * (size_t)p->segments);
  p->off_ps = off;
  off = align256(off + sizeof(float) * (size_t)L * (size_t)p->segments);
  p->off_bsum = off;
  off = align256(off + sizeof(float) * (size_t)((L + 255) / 256));
  p->off_hT = off;
  off = align256(off + sizeof(uint16_t) * (size_t)H * (size_t)p->Lpad);
  p->off_WT = off;
  off = align256(off + sizeof(uint16_t) * (size_t)H * (size_t)p->Vpad);
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
    case LMCE_ERR_UNSUPPORTED: return "unsupported shape: H must be a multiple of 64, chunk_rows a multiple of 32 in [32, 1024]";
    case LMCE_ERR_WORKSPACE: return "workspace smaller than lmce_workspace_size()";
    case LMCE_ERR_HIP: return "HIP runtime error";
    case LMCE_ERR_LABEL: return "a label is outside [0, V) and is not ignore_index";
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
  hipStream_t s = static_cast<hipStream_t>(stream);

  WsHeader* hdr = at<WsHeader>(workspace, 0);
  if (launch_count_labels(labels, L, V, ignore_index, hdr, s) != hipSuccess) return LMCE_ERR_HIP;
  FwdArgs a;
  a.h = static_cast<const uint16_t*>(h);
  a.W = static_cast<const uint16_t*>(W);
  a.labels = labels;
  a.L = L;
  a.H = H;
  a.V = V;
  a.ignore_index = ignore_index;
  a.chunk_rows = p.chunk_rows;
  a.tiles_per_chunk = p.tiles_per_chunk;
  a.n_chunks = p.n_chunks;
  a.segments = p.segments;
  a.vtiles = p.vtiles;
  a.vtiles_per_seg = p.vtiles_per_seg;
  a.hdr = hdr;
  a.zlabel = at<float>(workspace, p.off_zlabel);
  a.part_m = at<float>(workspace, p.off_pm);
  a.part_s = at<float>(workspace, p.off_ps);
  a.block_sum = at<float>(workspace, p.off_bsum);
  if (launch_fwd(a, loss_out, lse_out, s) != hipSuccess) return LMCE_ERR_HIP;
  return LMCE_OK;
}

namespace {

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
  if (launch_count_labels(labels, L, V, ignore_index, hdr, s) != hipSuccess) return LMCE_ERR_HIP;
  uint16_t* hT = at<uint16_t>(workspace, p.off_hT);
  uint16_t* WT = at<uint16_t>(workspace, p.off_WT);
  if ((which & 2) && launch_transpose(h, L, H, hT, p.Lpad, s) != hipSuccess) return LMCE_ERR_HIP;
  if ((which & 1) && launch_transpose(W, V, H, WT, p.Vpad, s) != hipSuccess) return LMCE_ERR_HIP;
  BwdArgs a;
  a.h = static_cast<const uint16_t*>(h);
  a.W = static_cast<const uint16_t*>(W);
  a.labels = labels;
  a.lse = lse;
  a.grad_loss = grad_loss;
  a.hT = hT;
  a.WT = WT;
  a.L = L;
  a.H = H;
  a.V = V;
  a.ignore_index = ignore_index;
  a.Lpad = p.Lpad;
  a.Vpad = p.Vpad;
  a.vtiles = p.vtiles;
  a.hdr = hdr;
  a.dh = dh_out;
  a.dW = dW_out;
  if ((which & 1) && launch_bwd_dh(a, p.hs, s) != hipSuccess) return LMCE_ERR_HIP;
  if ((which & 2) && launch_bwd_dW(a, p.hs, s) != hipSuccess) return LMCE_ERR_HIP;
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

extern "C" int lmce_read_status(const void* workspace, void* stream) {
  if (!aligned(workspace, 256)) return LMCE_ERR_NULL;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return LMCE_ERR_HIP;
  WsHeader hdr;
  if (hipMemcpy(&hdr, workspace, sizeof(hdr), hipMemcpyDeviceToHost) != hipSuccess) return LMCE_ERR_HIP;
  return hdr.status == 0 ? LMCE_OK : LMCE_ERR_LABEL;
}
